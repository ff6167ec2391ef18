"""Shared GPU-test case builders: seeded inputs -> device path through the C ABI,
and the fp64 oracle on the same logical inputs.

Nothing here feeds a value computed by the HIP path into the oracle: the oracle
sees only the generator's logical q/k/v, lengths, positions and block tables.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field

import numpy as np
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
import oracle

DEV = "cuda"


def announce(msg: str):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------------------
# tolerance gates
# ---------------------------------------------------------------------------

GATE_LOG = os.environ.get("CP_GATE_LOG")  # optional JSONL file of every gate's margin


def _record(name, kind, dmax, scale, used):
    """Print (and optionally log) a gate's achieved error: max|d|, max|d| / max|ref|
    and the largest fraction of the element-wise bound used."""
    ratio = dmax / scale if scale > 0 else 0.0
    print(f"[gate] {kind} {name}: max|d| = {dmax:.3e}, max|d|/max|ref| = {ratio:.3e}, "
          f"bound used {used:.3f}", flush=True)
    if GATE_LOG:
        with open(GATE_LOG, "a") as f:
            f.write(json.dumps({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0],
                                "gate": name, "kind": kind, "max_abs": dmax,
                                "max_rel_to_max_ref": ratio, "bound_used": used}) + "\n")


def _same_nonfinite(got, ref, name):
    """Non-finite values must sit exactly where the oracle's are: -inf where the
    oracle has -inf (empty key sets), NaN where it has NaN, and a finite value
    everywhere else."""
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{name}: -inf pattern differs"
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{name}: NaN pattern differs"
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all(), f"{name}: non-finite values where the oracle is finite"
    return fin


FP32_FLOOR = 1e-6


def gate_f32(got, ref, name):
    """fp32 configs: |d| <= 1e-5 |ref| + 1e-6 max|ref| element-wise, after the
    non-finite patterns agree.

    1e-5 relative is the stated fp32 tolerance.  A relative bound is undefined at
    cancellation points (an output element that is a near-zero weighted sum of
    O(1) values), so the gate adds an absolute floor at the rounding level of the
    whole tensor.  The kernels' fp32 results are weighted sums o = sum_t w_t v_t
    (sum_t w_t = 1) whose longest chain of dependent roundings has k <= ~50 steps
    (a 32-key chunk per lane, then at most ~8 split parts and N shard parts); in
    the probabilistic rounding model the error is ~ sqrt(k) * 2^-24 * sum_t w_t |v_t|,
    about 4e-7 * max|v|, and max|v| is at most ~3 max|ref| for these inputs.  The
    floor 1e-6 max|ref| sits a few standard deviations of that model above it;
    each gate prints the achieved max|d| / max|ref| so the margin is visible."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = _same_nonfinite(got, ref, name)
    scale = np.abs(ref[fin]).max(initial=0.0)
    d = np.abs(got[fin] - ref[fin])
    bound = 1e-5 * np.abs(ref[fin]) + FP32_FLOOR * scale
    bad = d > bound
    _record(name, "f32", float(d.max(initial=0.0)), float(scale),
            float((d / np.maximum(bound, 1e-300)).max(initial=0.0)))
    assert not bad.any(), (f"{name}: {bad.sum()} elements beyond fp32 gate, max |d| = {d.max():.3e}"
                           f", max|ref| = {scale:.3e}")


def gate_lowp(got, ref, name, atol, norm=1e-2):
    """bf16 / fp8 configs: |d| <= atol element-wise and max|d| <= norm * max|ref|,
    after the non-finite patterns agree."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = _same_nonfinite(got, ref, name)
    d = np.abs(got[fin] - ref[fin])
    scale = np.abs(ref[fin]).max(initial=0.0)
    dmax = float(d.max(initial=0.0))
    bound = atol if norm is None or scale == 0 else min(atol, norm * scale)
    _record(name, "lowp", dmax, float(scale), dmax / bound if bound > 0 else 0.0)
    assert dmax <= atol, f"{name}: max |d| = {dmax:.3e} > {atol}"
    if norm is not None and scale > 0:
        assert dmax <= norm * scale, (
            f"{name}: max |d| = {dmax:.3e} > {norm} x max|ref| = {norm * scale:.3e}")


def lowp_gate_passes(got, ref, atol, norm=1e-2):
    try:
        gate_lowp(got, ref, "probe", atol, norm)
        return True
    except AssertionError:
        return False


# ---------------------------------------------------------------------------
# sharded decode case (GQA or MLA)
# ---------------------------------------------------------------------------

@dataclass
class DecodeCase:
    w: ci.Workload
    seq: np.ndarray                 # [B] context lengths
    offs: np.ndarray                # [B+1] ragged offsets into the logical rows
    q: torch.Tensor                 # device [B][Hq][D]
    k: torch.Tensor                 # device logical rows [sumL][Hkv][D] (MLA: [sumL][1][Dk])
    v: torch.Tensor | None          # device [sumL][Hkv][D] (None for MLA)
    kv_scale: float
    shards: list                    # per rank: dict(bt, bt_dev, pool, kc, vc, ll, ll_dev, slots)
    host: dict = field(default_factory=dict)  # request b -> its logical rows on the host


def build_decode_case(w: ci.Workload, *, seq=None, pool_factor=2.0, check_slots=True,
                      check_cache=True) -> DecodeCase:
    """Generate inputs, fill N shard caches through cp_slot_map + cp_cache_write."""
    mla = w.kind == "mla_decode"
    if seq is None:
        seq = ci.uniform_lengths(w.B, w.ctx[0], w.ctx[1], w.seed)
    seq = np.asarray(seq, dtype=np.int32)
    offs = np.concatenate([[0], np.cumsum(seq)]).astype(np.int64)
    total = int(offs[-1])
    q = ci.to_storage(ci.normal((w.B, w.Hq, w.D), w.seed + 1, DEV, w.q_std), w.q_dtype)
    kv_scale = 1.0
    if mla:
        lat = ci.normal((total, 1, w.D), w.seed + 2, DEV, w.kv_std)
        if w.kv_dtype == "fp8_e4m3fn":
            k, kv_scale = ci.fp8_quantize(lat)
        else:
            k = ci.to_storage(lat, w.kv_dtype)
        del lat
        v = None
    else:
        k = ci.to_storage(ci.normal((total, w.Hkv, w.D), w.seed + 2, DEV, w.kv_std), w.kv_dtype)
        v = ci.to_storage(ci.normal((total, w.Hkv, w.D), w.seed + 3, DEV, w.kv_std), w.kv_dtype)
    req = torch.from_numpy(np.repeat(np.arange(w.B, dtype=np.int32), seq)).to(DEV)
    pos = torch.from_numpy(np.concatenate([np.arange(L, dtype=np.int32) for L in seq])
                           if total else np.zeros(0, np.int32)).to(DEV)
    shards = []
    for r in range(w.N):
        ll = oracle.local_lens(seq, r, w.N, w.I)
        needed = (ll.astype(np.int64) + w.bs - 1) // w.bs
        bt, pool = ci.block_tables(needed, w.seed + 100 + r, pool_factor)
        bt_dev = torch.from_numpy(bt).to(DEV)
        tdt = ci.TORCH_DTYPE[w.kv_dtype]
        if mla:
            kc = ci.nan_fill_(torch.empty(pool, w.bs, w.D, dtype=tdt, device=DEV), w.kv_dtype)
            vc = None
        else:
            kc = ci.nan_fill_(torch.empty(pool, w.Hkv, w.bs, w.D, dtype=tdt, device=DEV),
                              w.kv_dtype)
            vc = ci.nan_fill_(torch.empty_like(kc), w.kv_dtype)
        seq_dev = torch.from_numpy(seq).to(DEV)
        ll_dev = cp.cp_local_seq_lens(seq_dev, r, w.N, w.I)
        slots = cp.cp_slot_map(req, pos, bt_dev, r, w.N, w.I, w.bs)
        if mla:
            cp.cp_cache_write(slots, k.view(total, w.D), None, kc, None, w.bs)
        else:
            cp.cp_cache_write(slots, k, v, kc, vc, w.bs)
        torch.cuda.synchronize()
        assert np.array_equal(ll_dev.cpu().numpy(), ll), f"local lengths differ on rank {r}"
        if check_slots:
            ref_slots = oracle.slot_map(req.cpu().numpy(), pos.cpu().numpy(), bt, r, w.N, w.I,
                                        w.bs)
            assert np.array_equal(slots.cpu().numpy(), ref_slots), f"slot map differs, rank {r}"
        if check_cache:
            _check_cache_bytes(w, slots, k, v, kc, vc)
        shards.append(dict(bt=bt, bt_dev=bt_dev, pool=pool, kc=kc, vc=vc, ll=ll, ll_dev=ll_dev,
                           slots=slots if check_slots else None))
    return DecodeCase(w, seq, offs, q, k, v, kv_scale, shards)


def _bits(t):
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t.view(torch.uint8)


def _check_cache_bytes(w, slots, k, v, kc, vc):
    """Every owned token's rows sit bit-exactly at its slot; every other cache
    row still holds the NaN poison."""
    own = slots >= 0
    s = slots[own]
    blk, off = s // w.bs, s % w.bs
    if vc is None:
        got = _bits(kc)[blk, off]
        assert torch.equal(got, _bits(k.view(k.shape[0], -1))[own]), "latent rows differ"
        written = torch.zeros(kc.shape[0], kc.shape[1], dtype=torch.bool, device=DEV)
        written[blk, off] = True
        rest = _bits(kc)[~written]
    else:
        assert torch.equal(_bits(kc)[blk, :, off], _bits(k)[own]), "K rows differ"
        assert torch.equal(_bits(vc)[blk, :, off], _bits(v)[own]), "V rows differ"
        written = torch.zeros(kc.shape[0], kc.shape[2], dtype=torch.bool, device=DEV)
        written[blk, off] = True
        rest = _bits(kc).permute(0, 2, 1, 3)[~written]
    nan = ci.NAN_BITS[w.kv_dtype]
    if rest.dtype == torch.int16:
        nan = nan - (1 << 16) if nan >= (1 << 15) else nan
    assert bool((rest == nan).all()), "a cache row outside the owned slots was written"


def run_partials(case: DecodeCase):
    """Shard partials through the C ABI, stacked as [N][B][H][Dv] / [N][B][H]."""
    w = case.w
    mla = w.kind == "mla_decode"
    outs, lses = [], []
    for sh in case.shards:
        if mla:
            o, l = cp.cp_decode_attn_partial_mla(case.q, sh["kc"], sh["bt_dev"], sh["ll_dev"],
                                                 w.scale, Dv=w.Dv, kv_scale=case.kv_scale)
        else:
            o, l = cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], sh["bt_dev"],
                                                 sh["ll_dev"], w.scale)
        outs.append(o)
        lses.append(l)
    return torch.stack(outs), torch.stack(lses)


def oracle_request(case: DecodeCase, b: int, shard=None, heads=None):
    """fp64 oracle for request b (all heads or ``heads``), over the whole context
    or one shard's owned positions."""
    w = case.w
    lo, hi = int(case.offs[b]), int(case.offs[b + 1])
    q = ci.bits(case.q[b:b + 1].cpu())
    if b not in case.host:
        case.host.clear()  # keep one request's rows (a 1M-token request is 600 MB)
        if w.kind == "mla_decode":
            lat = ci.bits(case.k[lo:hi].cpu())
            case.host[b] = (lat, lat)
        else:
            case.host[b] = (ci.bits(case.k[lo:hi].cpu()), ci.bits(case.v[lo:hi].cpu()))
    k, v = case.host[b]
    dv = w.Dv if w.kind == "mla_decode" else None
    out, lse = oracle.attention(q, k, v, key_begin=0, key_end=hi - lo, scale=w.scale,
                                q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, Dv=dv,
                                kv_scale=case.kv_scale, shard=shard, heads=heads)
    return out[0], lse[0]


def miswritten_shard(case: DecodeCase, r: int, I_bad: int, pool_factor=1.25):
    """Shard r's cache as a rank would hold it had it written the context with
    interleave I_bad instead of the case's I (stale cache metadata, "Where It
    Breaks" in the code-reading page): (cache, v cache or None, block table,
    local lengths), all on the device."""
    w = case.w
    mla = w.kind == "mla_decode"
    seq = case.seq
    total = int(case.offs[-1])
    req = torch.from_numpy(np.repeat(np.arange(w.B, dtype=np.int32), seq)).to(DEV)
    pos = torch.from_numpy(np.concatenate([np.arange(L, dtype=np.int32) for L in seq])).to(DEV)
    ll = oracle.local_lens(seq, r, w.N, I_bad)
    bt, pool = ci.block_tables((ll.astype(np.int64) + w.bs - 1) // w.bs, w.seed + 900 + r,
                               pool_factor)
    bt_dev = torch.from_numpy(bt).to(DEV)
    tdt = ci.TORCH_DTYPE[w.kv_dtype]
    if mla:
        kc = ci.nan_fill_(torch.empty(pool, w.bs, w.D, dtype=tdt, device=DEV), w.kv_dtype)
        vc = None
    else:
        kc = ci.nan_fill_(torch.empty(pool, w.Hkv, w.bs, w.D, dtype=tdt, device=DEV), w.kv_dtype)
        vc = ci.nan_fill_(torch.empty_like(kc), w.kv_dtype)
    slots = cp.cp_slot_map(req, pos, bt_dev, r, w.N, I_bad, w.bs)
    if mla:
        cp.cp_cache_write(slots, case.k.view(total, w.D), None, kc, None, w.bs)
    else:
        cp.cp_cache_write(slots, case.k, case.v, kc, vc, w.bs)
    torch.cuda.synchronize()
    return kc, vc, bt_dev, torch.from_numpy(ll).to(DEV)
