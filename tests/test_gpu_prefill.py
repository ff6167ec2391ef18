"""GPU parity: PCP causal prefill -- each rank's two pieces against the chunk's
own keys (causal), against every DCP shard of the cached prefix (paged), and the
exact merge of the 1 + N partials -- compared with the fp64 oracle, which
selects the rank's query rows with its own head-tail piece rule."""
import math

import numpy as np
import pytest
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
import oracle
from _cases import announce, build_decode_case, gate_lowp, lowp_gate_passes, miswritten_shard

pytestmark = pytest.mark.gpu
ATOL_OUT, ATOL_LSE = 2e-2, 1e-3


def _setup(C, P, N, Hq, Hkv, N_dcp, I, bs, seed):
    """Chunk q/k/v (device, bf16) and the prefix held in N_dcp paged shards."""
    D = 128
    scale = 1 / math.sqrt(D)
    q = ci.to_storage(ci.normal((C, Hq, D), seed + 1, "cuda"), "bf16")
    k = ci.to_storage(ci.normal((C, Hkv, D), seed + 2, "cuda"), "bf16")
    v = ci.to_storage(ci.normal((C, Hkv, D), seed + 3, "cuda"), "bf16")
    wp = ci.Workload("prefix", "gqa_decode", B=1, Hq=Hq, Hkv=Hkv, D=D, Dv=D, N=N_dcp, I=I, bs=bs,
                     q_dtype="bf16", kv_dtype="bf16", scale=scale, seed=seed + 50)
    prefix = build_decode_case(wp, seq=[P], check_cache=P < 100000)
    return q, k, v, prefix, scale


def _rank_partials(q, k, v, prefix, P, r, N, scale):
    """Causal partial + one partial per prefix shard, stacked [1 + N_dcp][2c][Hq][D]."""
    outs, lses = [], []
    o, l = cp.pcp_prefill_attn_causal(q, P, r, N, scale, k=k, v=v)
    outs.append(o)
    lses.append(l)
    for sh in prefix.shards:
        o, l = cp.pcp_prefill_attn_causal(q, P, r, N, scale, k_cache=sh["kc"], v_cache=sh["vc"],
                                          block_table=sh["bt_dev"][0].contiguous(),
                                          local_len=int(sh["ll"][0]))
        outs.append(o)
        lses.append(l)
    po = torch.stack([x.reshape(-1, x.shape[-2], x.shape[-1]) for x in outs])
    pl = torch.stack([x.reshape(-1, x.shape[-1]) for x in lses])
    return po, pl


_HOST = {}


@pytest.fixture(autouse=True)
def _fresh_host_rows():
    _HOST.clear()  # ids of a finished test's tensors may be reused
    yield
    _HOST.clear()


def _oracle_rows(q, k, v, prefix, P, rows, scale, key_begin=None, key_end=None, shard=None,
                 heads=None):
    """fp64 oracle for chunk rows `rows` over the logical [prefix; chunk] keys."""
    key = (id(prefix), id(q), id(k), id(v))
    if _HOST.get("key") != key:  # one case's logical rows on the host at a time
        _HOST.clear()
        _HOST.update(key=key, q=ci.bits(q.cpu()),
                     k=np.concatenate([ci.bits(prefix.k.cpu()), ci.bits(k.cpu())]),
                     v=np.concatenate([ci.bits(prefix.v.cpu()), ci.bits(v.cpu())]))
    kall, vall = _HOST["k"], _HOST["v"]
    qb = _HOST["q"][rows]
    kb = P + rows if key_begin is None else key_begin
    ke = P + rows + 1 if key_end is None else key_end
    return oracle.attention(qb, kall, vall, key_begin=kb, key_end=ke, scale=scale, q_dtype="bf16",
                            kv_dtype="bf16", shard=shard, heads=heads)


@pytest.mark.parametrize("C,P,N,Hq,Hkv,N_dcp", [(256, 200, 2, 32, 8, 3), (384, 0, 3, 8, 8, 1),
                                                 (512, 777, 4, 16, 8, 2), (256, 64, 2, 8, 1, 2),
                                                 # pieces that are not whole 32-row blocks:
                                                 # the pages' PCP2 example (L = 8, pieces of 2),
                                                 # PCP3 (six pieces of 10), and 125-row pieces
                                                 (8, 0, 2, 8, 2, 1), (8, 40, 2, 8, 2, 2),
                                                 (60, 37, 3, 16, 8, 2), (2000, 1000, 8, 32, 8, 8),
                                                 (96, 50, 1, 16, 2, 3)])
def test_prefill_small(C, P, N, Hq, Hkv, N_dcp):
    announce(f"prefill C={C} P={P} N={N} Hq={Hq} Hkv={Hkv} N_dcp={N_dcp}")
    q, k, v, prefix, scale = _setup(C, max(P, 1), N, Hq, Hkv, N_dcp, 16, 16, 4000 + C + P)
    if P == 0:
        # an empty prefix: shards hold nothing; keep one real key out of the way
        prefix.shards = []
    Pk = prefix.k.shape[0] if P > 0 else 0
    for r in range(N):
        rows = oracle.pcp_rank_positions(C, N, r)
        po, pl = _rank_partials(q, k, v, prefix, Pk, r, N, scale)
        mo, ml = cp.cp_lse_merge(po, pl)
        torch.cuda.synchronize()
        po, pl, mo, ml = po.cpu().numpy(), pl.cpu().numpy(), mo.cpu().numpy(), ml.cpu().numpy()
        if P == 0:
            kall = ci.bits(k.cpu())
            vall = ci.bits(v.cpu())
            ro, rl = oracle.attention(ci.bits(q.cpu())[rows], kall, vall, key_begin=0,
                                      key_end=rows + 1, scale=scale, q_dtype="bf16",
                                      kv_dtype="bf16")
            gate_lowp(po[0], ro, f"causal r{r}", ATOL_OUT)
            gate_lowp(pl[0], rl, f"causal lse r{r}", ATOL_LSE, norm=None)
            continue
        ro, rl = _oracle_rows(q, k, v, prefix, Pk, rows, scale, key_begin=Pk + 0 * rows)
        gate_lowp(po[0], ro, f"causal r{r}", ATOL_OUT)
        gate_lowp(pl[0], rl, f"causal lse r{r}", ATOL_LSE, norm=None)
        for s in range(N_dcp):
            ro, rl = _oracle_rows(q, k, v, prefix, Pk, rows, scale, key_begin=0, key_end=Pk,
                                  shard=(N_dcp, 16, s))
            gate_lowp(po[1 + s], ro, f"prefix shard {s} r{r}", ATOL_OUT)
            gate_lowp(pl[1 + s], rl, f"prefix lse shard {s} r{r}", ATOL_LSE, norm=None)
        ro, rl = _oracle_rows(q, k, v, prefix, Pk, rows, scale, key_begin=0)
        gate_lowp(mo, ro, f"merged r{r}", ATOL_OUT)
        gate_lowp(ml, rl, f"merged lse r{r}", ATOL_LSE, norm=None)


def test_prefill_full_workload_sampled():
    """The 32K-chunk / 64K-prefix workload on every PCP rank: the causal part,
    each of the 8 prefix-shard partials and the 9-way merge, on the first and
    last row of both pieces plus random rows, for three heads."""
    w = ci.WORKLOADS["pcp_prefill_bf16"]
    announce(f"{w.name}: C={w.C} P={w.P} N={w.N}, sampled rows")
    q, k, v, prefix, scale = _setup(w.C, w.P, w.N, w.Hq, w.Hkv, w.N, w.I, w.bs, w.seed)
    rng = np.random.default_rng(w.seed)
    c = w.C // (2 * w.N)
    heads = [0, 13, 31]
    for r in range(w.N):
        rows = oracle.pcp_rank_positions(w.C, w.N, r)
        po, pl = _rank_partials(q, k, v, prefix, w.P, r, w.N, scale)
        mo, ml = cp.cp_lse_merge(po, pl)
        torch.cuda.synchronize()
        po, pl = po.cpu().numpy(), pl.cpu().numpy()
        pick = np.unique(np.concatenate([[0, c - 1, c, 2 * c - 1], rng.integers(0, 2 * c, 4)]))
        ro, rl = _oracle_rows(q, k, v, prefix, w.P, rows[pick], scale, key_begin=0, heads=heads)
        gate_lowp(mo.cpu().numpy()[pick][:, heads], ro, f"merged r{r}", ATOL_OUT)
        gate_lowp(ml.cpu().numpy()[pick][:, heads], rl, f"merged lse r{r}", ATOL_LSE, norm=None)
        ro, rl = _oracle_rows(q, k, v, prefix, w.P, rows[pick], scale, key_begin=w.P, heads=heads)
        gate_lowp(po[0][pick][:, heads], ro, f"causal r{r}", ATOL_OUT)
        gate_lowp(pl[0][pick][:, heads], rl, f"causal lse r{r}", ATOL_LSE, norm=None)
        for s in range(w.N):
            ro, rl = _oracle_rows(q, k, v, prefix, w.P, rows[pick], scale, key_begin=0,
                                  key_end=w.P, shard=(w.N, w.I, s), heads=heads)
            gate_lowp(po[1 + s][pick][:, heads], ro, f"prefix shard {s} r{r}", ATOL_OUT)
            gate_lowp(pl[1 + s][pick][:, heads], rl, f"prefix lse shard {s} r{r}", ATOL_LSE,
                      norm=None)
    # stale cache metadata on prefix shard 3, rank 5's pieces: (i) the block
    # table naming blocks 44-47 twice (the 64 keys of blocks 40-43 lost, those
    # of 44-47 counted twice, 0.8% of the shard's 8,192 keys), (ii) the shard's
    # prefix written with interleave I + 1
    r, s = 5, 3
    rows = oracle.pcp_rank_positions(w.C, w.N, r)
    pick = np.array([0, 1, c, 2 * c - 1])
    ro, _ = _oracle_rows(q, k, v, prefix, w.P, rows[pick], scale, key_begin=0, key_end=w.P,
                         shard=(w.N, w.I, s), heads=heads)
    sh = prefix.shards[s]
    bt = sh["bt_dev"][0].clone()
    bt[40:44] = bt[44:48]
    o, _ = cp.pcp_prefill_attn_causal(q, w.P, r, w.N, scale, k_cache=sh["kc"], v_cache=sh["vc"],
                                      block_table=bt, local_len=int(sh["ll"][0]))
    got = o.reshape(-1, w.Hq, w.D).cpu().numpy()[pick][:, heads]
    assert not lowp_gate_passes(got, ro, ATOL_OUT), "block-table control"
    kc, vc, bt_bad, ll_bad = miswritten_shard(prefix, s, w.I + 1)
    o, _ = cp.pcp_prefill_attn_causal(q, w.P, r, w.N, scale, k_cache=kc, v_cache=vc,
                                      block_table=bt_bad[0].contiguous(),
                                      local_len=int(ll_bad[0]))
    got = o.reshape(-1, w.Hq, w.D).cpu().numpy()[pick][:, heads]
    assert not lowp_gate_passes(got, ro, ATOL_OUT), "interleave control"


def test_prefill_negative_control_and_validation():
    C, P, N = 256, 300, 2
    q, k, v, prefix, scale = _setup(C, P, N, 32, 8, 2, 16, 16, 4500)
    rows = oracle.pcp_rank_positions(C, N, 1)
    # the wrong rank's pieces must not pass for rank 1
    o, _ = cp.pcp_prefill_attn_causal(q, P, 0, N, scale, k=k, v=v)
    ro, _ = _oracle_rows(q, k, v, prefix, P, rows, scale, key_begin=P)
    assert not lowp_gate_passes(o.reshape(-1, 32, 128).cpu().numpy(), ro, ATOL_OUT)
    o, _ = cp.pcp_prefill_attn_causal(q, P, 1, N, scale, k=k, v=v)
    assert lowp_gate_passes(o.reshape(-1, 32, 128).cpu().numpy(), ro, ATOL_OUT)
    # a chunk not aligned to 2N is rejected: by the binding, and by the library
    # itself when called through the C ABI
    q2, k2, v2 = q[:250].contiguous(), k[:250].contiguous(), v[:250].contiguous()
    with pytest.raises(ValueError, match="multiple of 2 x pcp_size"):
        cp.pcp_prefill_attn_causal(q2, P, 0, N, scale, k=k2, v=v2)
    o = torch.empty(2, 62, 32, 128, device="cuda")
    l = torch.empty(2, 62, 32, device="cuda")
    a = cp._lib.CpPrefillArgs(q=cp._ptr(q2), C=250, P=P, pcp_rank=0, pcp_size=N, Hq=32, Hkv=8,
                              D=128, scale=scale, kv_source=cp.CP_KV_DENSE, k=cp._ptr(k2),
                              v=cp._ptr(v2), out=cp._ptr(o), lse=cp._ptr(l))
    import ctypes
    assert cp._lib.load().pcp_prefill_attn_causal(ctypes.byref(a), None, 0,
                                                  cp._stream()) == cp.CP_E_INVALID


def _dcp_setup(C, P, Hq, Hkv, N_dcp, I, bs, seed, check_cache=True):
    """Chunk queries plus the logical [prefix; chunk] K/V held, all of it,
    interleaved in N_dcp paged shards."""
    D = 128
    scale = 1 / math.sqrt(D)
    q = ci.to_storage(ci.normal((C, Hq, D), seed + 1, "cuda"), "bf16")
    wp = ci.Workload("dcp", "gqa_decode", B=1, Hq=Hq, Hkv=Hkv, D=D, Dv=D, N=N_dcp, I=I, bs=bs,
                     q_dtype="bf16", kv_dtype="bf16", scale=scale, seed=seed + 50)
    allkv = build_decode_case(wp, seq=[P + C], check_cache=check_cache)
    return q, allkv, scale


def _dcp_partials(q, allkv, P, r, N, N_dcp, I, scale):
    outs, lses = [], []
    for s, sh in enumerate(allkv.shards):
        o, l = cp.pcp_prefill_attn_causal(q, P, r, N, scale, k_cache=sh["kc"], v_cache=sh["vc"],
                                          block_table=sh["bt_dev"][0].contiguous(),
                                          local_len=int(sh["ll"][0]), dcp=(s, N_dcp, I))
        outs.append(o.reshape(-1, o.shape[-2], o.shape[-1]))
        lses.append(l.reshape(-1, l.shape[-1]))
    return torch.stack(outs), torch.stack(lses)


@pytest.mark.parametrize("C,P,N,Hq,Hkv,N_dcp,I", [(256, 200, 2, 32, 8, 3, 16),
                                                   (384, 0, 3, 8, 8, 4, 64),
                                                   (512, 777, 4, 16, 8, 2, 5),
                                                   (256, 64, 2, 8, 1, 8, 1),
                                                   (2000, 300, 8, 32, 8, 4, 16),
                                                   (60, 0, 3, 8, 8, 3, 4)])
def test_prefill_dcp_causal_shards(C, P, N, Hq, Hkv, N_dcp, I):
    """DCP-sharded causal prefill: every shard holds prefix and chunk keys
    interleaved; each shard's partial is the attention over its keys at
    positions <= the query's, and their merge is causal attention over prefix
    and chunk.  (P = 0 with I = 64: early rows see no key of shards 1..3.)"""
    announce(f"dcp causal prefill C={C} P={P} N={N} Hq={Hq} Hkv={Hkv} N_dcp={N_dcp} I={I}")
    q, allkv, scale = _dcp_setup(C, P, Hq, Hkv, N_dcp, I, 16, 4700 + C + P + I)
    kall, vall = ci.bits(allkv.k.cpu()), ci.bits(allkv.v.cpu())
    qb = ci.bits(q.cpu())
    for r in range(N):
        rows = oracle.pcp_rank_positions(C, N, r)
        po, pl = _dcp_partials(q, allkv, P, r, N, N_dcp, I, scale)
        mo, ml = cp.cp_lse_merge(po, pl)
        torch.cuda.synchronize()
        po, pl, mo, ml = po.cpu().numpy(), pl.cpu().numpy(), mo.cpu().numpy(), ml.cpu().numpy()
        for s in range(N_dcp):
            ro, rl = oracle.attention(qb[rows], kall, vall, key_begin=0, key_end=P + rows + 1,
                                      scale=scale, q_dtype="bf16", kv_dtype="bf16",
                                      shard=(N_dcp, I, s))
            gate_lowp(po[s], ro, f"shard {s} r{r}", ATOL_OUT)
            gate_lowp(pl[s], rl, f"shard lse {s} r{r}", ATOL_LSE, norm=None)
        ro, rl = oracle.attention(qb[rows], kall, vall, key_begin=0, key_end=P + rows + 1,
                                  scale=scale, q_dtype="bf16", kv_dtype="bf16")
        gate_lowp(mo, ro, f"merged r{r}", ATOL_OUT)
        gate_lowp(ml, rl, f"merged lse r{r}", ATOL_LSE, norm=None)


def test_prefill_dcp_causal_full_workload_sampled():
    w = ci.WORKLOADS["dcp_prefill_bf16"]
    announce(f"{w.name}: C={w.C} P={w.P} N={w.N} sampled rows")
    q, allkv, scale = _dcp_setup(w.C, w.P, w.Hq, w.Hkv, w.N, w.I, w.bs, w.seed, check_cache=False)
    kall, vall = ci.bits(allkv.k.cpu()), ci.bits(allkv.v.cpu())
    qb = ci.bits(q.cpu())
    rng = np.random.default_rng(w.seed)
    c = w.C // (2 * w.N)
    heads = [0, 17, 31]
    for r in [0, 6]:
        rows = oracle.pcp_rank_positions(w.C, w.N, r)
        po, pl = _dcp_partials(q, allkv, w.P, r, w.N, w.N, w.I, scale)
        mo, ml = cp.cp_lse_merge(po, pl)
        torch.cuda.synchronize()
        pick = np.unique(np.concatenate([[0, c - 1, c, 2 * c - 1], rng.integers(0, 2 * c, 3)]))
        ro, rl = oracle.attention(qb[rows[pick]], kall, vall, key_begin=0,
                                  key_end=w.P + rows[pick] + 1, scale=scale, q_dtype="bf16",
                                  kv_dtype="bf16", heads=heads)
        gate_lowp(mo.cpu().numpy()[pick][:, heads], ro, f"merged r{r}", ATOL_OUT)
        gate_lowp(ml.cpu().numpy()[pick][:, heads], rl, f"merged lse r{r}", ATOL_LSE, norm=None)
        s = 5
        ro, rl = oracle.attention(qb[rows[pick]], kall, vall, key_begin=0,
                                  key_end=w.P + rows[pick] + 1, scale=scale, q_dtype="bf16",
                                  kv_dtype="bf16", heads=heads, shard=(w.N, w.I, s))
        gate_lowp(po[s].cpu().numpy()[pick][:, heads], ro, f"shard {s} r{r}", ATOL_OUT)
