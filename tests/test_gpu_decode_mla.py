"""GPU parity: absorbed-MLA decode partials (bf16 and fp8 E4M3 latent) and their
exact merge against the fp64 oracle -- ragged small cases element by element,
the full 64-request / 64K-context bf16 and 4-request / 1M-context fp8 workloads
on sampled requests and heads, the unit-variance ("peaked") twin whose softmax
is far from uniform, and a negative control."""
import numpy as np
import pytest
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
from _cases import (announce, build_decode_case, gate_lowp, lowp_gate_passes, miswritten_shard,
                    oracle_request, run_partials)

pytestmark = pytest.mark.gpu

ATOL_OUT, ATOL_LSE = 2e-2, 1e-3


def _check(case, requests, shards, heads=None, merged=True):
    w = case.w
    po, pl = run_partials(case)
    mo, ml = cp.cp_lse_merge(po, pl)
    torch.cuda.synchronize()
    po, pl, mo, ml = po.cpu().numpy(), pl.cpu().numpy(), mo.cpu().numpy(), ml.cpu().numpy()
    hs = np.arange(w.Hq) if heads is None else np.asarray(heads)
    for b in requests:
        for r in shards:
            ro, rl = oracle_request(case, b, shard=(w.N, w.I, r), heads=heads)
            gate_lowp(po[r, b][hs], ro, f"partial out r{r} b{b}", ATOL_OUT)
            gate_lowp(pl[r, b][hs], rl, f"partial lse r{r} b{b}", ATOL_LSE, norm=None)
        if merged:
            ro, rl = oracle_request(case, b, heads=heads)
            gate_lowp(mo[b][hs], ro, f"merged out b{b}", ATOL_OUT)
            gate_lowp(ml[b][hs], rl, f"merged lse b{b}", ATOL_LSE, norm=None)


@pytest.mark.parametrize("H,bs,N,I", [(128, 64, 2, 1), (16, 16, 4, 16), (32, 64, 3, 5),
                                      (128, 32, 8, 1)])
def test_mla_bf16_ragged(H, bs, N, I):
    # peaked values (unit variance) so that outputs and LSEs carry information
    w = ci.scaled(ci.WORKLOADS["mla_decode_bf16_peaked"], B=4, Hq=H, N=N, I=I, bs=bs,
                  seed=3100 + H + bs + N)
    announce(f"mla bf16 ragged H={H} bs={bs} N={N} I={I}")
    case = build_decode_case(w, seq=[0, 5, 1000, 2999])
    _check(case, range(4), range(N))


@pytest.mark.parametrize("fp8", [False, True])
def test_mla_sharp_softmax_rescales(fp8):
    """Scores with a standard deviation of ~6 (scale 1/4 on unit-variance data):
    the running maximum jumps by more than the kernel's lazy-rescale margin
    many times within a segment, so the rescale path is exercised."""
    base = ci.WORKLOADS["mla_decode_fp8" if fp8 else "mla_decode_bf16_peaked"]
    w = ci.scaled(base, B=3, Hq=48, N=2, I=1, bs=64, scale=0.25, seed=3400 + fp8)
    announce(f"mla sharp softmax fp8={fp8}")
    case = build_decode_case(w, seq=[2500, 77, 4096])
    _check(case, range(3), range(2))


@pytest.mark.parametrize("seq", [[37, 1500], [64, 4097]])
def test_mla_fp8_ragged(seq):
    w = ci.scaled(ci.WORKLOADS["mla_decode_fp8"], B=len(seq), N=2, seed=3200 + seq[0])
    announce(f"mla fp8 ragged seq={seq}")
    case = build_decode_case(w, seq=seq)
    _check(case, range(len(seq)), range(2))


def test_mla_bf16_full_workload_sampled():
    w = ci.WORKLOADS["mla_decode_bf16"]
    announce(f"{w.name} full size, seed={w.seed}")
    case = build_decode_case(w, pool_factor=1.25, check_cache=False)
    _check(case, [0, 63], [0, 5], heads=[0, 1, 64, 127])


def test_mla_bf16_peaked_full_size_sampled_and_negative_control():
    w = ci.WORKLOADS["mla_decode_bf16_peaked"]
    announce(f"{w.name} full size, seed={w.seed}")
    case = build_decode_case(w, pool_factor=1.25, check_cache=False, check_slots=False)
    _check(case, [7], [3], heads=[2, 100])
    # corrupt one block-table entry of request 7 on shard 3: the gate must fail
    sh = case.shards[3]
    bt = sh["bt_dev"].clone()
    bt[7, 0] = bt[8, 0]
    o, _ = cp.cp_decode_attn_partial_mla(case.q, sh["kc"], bt, sh["ll_dev"], w.scale, Dv=w.Dv)
    ro, _ = oracle_request(case, 7, shard=(w.N, w.I, 3), heads=[2, 100])
    assert not lowp_gate_passes(o[7].cpu().numpy()[[2, 100]], ro, ATOL_OUT)


def test_mla_fp8_full_workload_sampled():
    """The 4-request, 1M-token fp8 workload: every shard's partial of one request
    and their 8-way merge against unsharded attention over all 1,048,576 keys,
    on four heads; then stale cache metadata that the gate must catch."""
    w = ci.WORKLOADS["mla_decode_fp8"]
    announce(f"{w.name} full size (1M-token contexts), seed={w.seed}")
    case = build_decode_case(w, pool_factor=1.25)
    heads = [0, 31, 64, 127]
    _check(case, [2], range(w.N), heads=heads, merged=True)
    # stale metadata on shard 6: (i) sixteen block-table entries of request 2
    # (1,024 of its 131,072 keys) pointing at request 3's blocks -- a single
    # 64-key block moves the outputs by only ~4e-3 max|ref| at this length,
    # below what the 1e-2 max|ref| gate can see; (ii) the shard's cache written
    # with interleave I + 1
    r, b = 6, 2
    sh = case.shards[r]
    ro, _ = oracle_request(case, b, shard=(w.N, w.I, r), heads=heads)
    bt = sh["bt_dev"].clone()
    bt[b, 100:116] = bt[b + 1, 100:116]
    o, _ = cp.cp_decode_attn_partial_mla(case.q, sh["kc"], bt, sh["ll_dev"], w.scale, Dv=w.Dv,
                                         kv_scale=case.kv_scale)
    assert not lowp_gate_passes(o[b].cpu().numpy()[heads], ro, ATOL_OUT), "block-table control"
    kc, _, bt_bad, ll_bad = miswritten_shard(case, r, w.I + 1)
    o, _ = cp.cp_decode_attn_partial_mla(case.q, kc, bt_bad, ll_bad, w.scale, Dv=w.Dv,
                                         kv_scale=case.kv_scale)
    assert not lowp_gate_passes(o[b].cpu().numpy()[heads], ro, ATOL_OUT), "interleave control"


def test_mla_bf16_peaked_interleave_control():
    """Stale metadata on the peaked MLA twin: a shard whose cache was written
    with interleave I + 1 must fail the gate."""
    w = ci.scaled(ci.WORKLOADS["mla_decode_bf16_peaked"], B=4, seed=3500)
    case = build_decode_case(w, seq=[9000, 12000, 4000, 8192], check_cache=False)
    heads = [5, 77]
    _check(case, [1], [2], heads=heads, merged=False)
    kc, _, bt_bad, ll_bad = miswritten_shard(case, 2, w.I + 1)
    o, _ = cp.cp_decode_attn_partial_mla(case.q, kc, bt_bad, ll_bad, w.scale, Dv=w.Dv)
    ro, _ = oracle_request(case, 1, shard=(w.N, w.I, 2), heads=heads)
    assert not lowp_gate_passes(o[1].cpu().numpy()[heads], ro, ATOL_OUT)


def test_mla_unsupported_shapes():
    w = ci.scaled(ci.WORKLOADS["mla_decode_bf16"], B=1, Hq=24, seed=3300)
    case = build_decode_case(w, seq=[100], check_cache=False)
    sh = case.shards[0]
    with pytest.raises(cp.CpError, match="CP_E_UNSUPPORTED"):
        cp.cp_decode_attn_partial_mla(case.q, sh["kc"], sh["bt_dev"], sh["ll_dev"], w.scale)
