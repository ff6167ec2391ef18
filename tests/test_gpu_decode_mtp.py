"""GPU parity: multi-token decode queries (the last T positions of each
request, causal on the shard's interleaved positions) against the fp64
oracle -- per shard, and the exact merge of all shards against unsharded
causal attention."""
import numpy as np
import pytest
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
import oracle
from _cases import DEV, announce, build_decode_case, gate_f32, gate_lowp

pytestmark = pytest.mark.gpu


def _mtp_case(w, T, seq, seed):
    case = build_decode_case(w, seq=seq, check_cache=False, check_slots=False)
    q = ci.to_storage(ci.normal((w.B, T, w.Hq, w.D), seed, DEV, w.q_std), w.q_dtype)
    return case, q


def _run(case, q, T):
    w = case.w
    seq_dev = torch.from_numpy(case.seq).to(DEV)
    outs, lses = [], []
    for r, sh in enumerate(case.shards):
        o, l = cp.cp_decode_attn_partial_gqa_mtp(q, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"],
                                                 seq_dev, w.scale, r, w.N, w.I)
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    return torch.stack(outs), torch.stack(lses)   # [N][B][T][Hq][D], [N][B][T][Hq]


def _oracle(case, q, b, shard=None):
    w = case.w
    lo, hi = int(case.offs[b]), int(case.offs[b + 1])
    return oracle.decode_mtp(ci.bits(q[b].cpu()), ci.bits(case.k[lo:hi].cpu()),
                             ci.bits(case.v[lo:hi].cpu()), L=hi - lo, scale=w.scale,
                             q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, shard=shard)


def _check(case, q, T, o, l, reqs):
    w = case.w
    lowp = w.kv_dtype != "f32"
    mo, ml = cp.cp_lse_merge(o.reshape(w.N, -1, w.D), l.reshape(w.N, -1))
    mo = mo.reshape(w.B, T, w.Hq, w.D)
    ml = ml.reshape(w.B, T, w.Hq)
    torch.cuda.synchronize()
    for b in reqs:
        announce(f"mtp {w.name} T={T} request {b} (L={case.seq[b]})")
        for r in sorted({0, w.N // 2, w.N - 1}):
            ro, rl = _oracle(case, q, b, shard=(w.N, w.I, r))
            if lowp:
                gate_lowp(o[r, b].cpu().numpy(), ro, f"shard {r} out", atol=2e-2)
                gate_lowp(l[r, b].cpu().numpy(), rl, f"shard {r} lse", atol=1e-3, norm=None)
            else:
                gate_f32(o[r, b].cpu().numpy(), ro, f"shard {r} out")
                gate_f32(l[r, b].cpu().numpy(), rl, f"shard {r} lse")
        ro, rl = _oracle(case, q, b)
        if lowp:
            gate_lowp(mo[b].cpu().numpy(), ro, "merged out", atol=2e-2)
            gate_lowp(ml[b].cpu().numpy(), rl, "merged lse", atol=1e-3, norm=None)
        else:
            gate_f32(mo[b].cpu().numpy(), ro, "merged out")
            gate_f32(ml[b].cpu().numpy(), rl, "merged lse")


# f32 head dim 64 (group 4, 2 tokens = 8 rows per KV head); bf16 head dim 128
# with group 4 x 2 tokens, group 1 x 8 tokens, group 2 x 4 tokens; requests as
# short as the token count (shards without a visible key for early tokens),
# ragged lengths around tile and interleave boundaries.  Past 8 rows per KV
# head the tokens go in several launches: group 4 x 3 tokens (2 + 1), group
# 4 x 4 (2 + 2), group 8 x 2 (1 + 1), group 2 x 5 (4 + 1), group 1 x 11
# (8 + 2 + 1), f32 group 4 x 3.
@pytest.mark.parametrize("name,T,Hq,Hkv,seq", [
    ("gqa_tiny_f32", 2, 8, 2, [1000, 33, 2, 517]),
    ("gqa_decode_bf16", 2, 32, 8, [4097, 2, 130, 9000]),
    ("gqa_decode_bf16", 8, 8, 8, [8, 300, 2049]),
    ("gqa_decode_bf16", 4, 16, 8, [5000, 4, 777]),
    ("gqa_decode_bf16", 3, 32, 8, [3, 4097, 531]),
    ("gqa_decode_bf16", 4, 32, 8, [100, 200, 6000]),
    ("gqa_decode_bf16", 2, 64, 8, [2, 2500, 129]),
    ("gqa_decode_bf16", 5, 16, 8, [5, 1030, 3333]),
    ("gqa_decode_bf16", 11, 8, 8, [11, 700, 4100]),
    ("gqa_decode_bf16", 3, 16, 8, [3, 1500, 2047]),
    ("gqa_decode_bf16", 7, 8, 8, [7, 64, 3001]),
    ("gqa_decode_bf16", 6, 8, 8, [900, 6, 33]),
    ("gqa_tiny_f32", 3, 8, 2, [1000, 3, 260]),
])
def test_mtp_against_oracle(name, T, Hq, Hkv, seq):
    base = ci.WORKLOADS[name]
    w = ci.scaled(base, B=len(seq), Hq=Hq, Hkv=Hkv, seed=6100 + T)
    case, q = _mtp_case(w, T, seq, 6200 + T)
    o, l = _run(case, q, T)
    _check(case, q, T, o, l, range(len(seq)))


def test_mtp_one_token_is_plain_decode():
    """q_len 1 gives the single-token entry's results (up to fp32 rounding: the
    two entries are separately compiled kernels)."""
    w = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=3, seed=6300)
    case, q = _mtp_case(w, 1, [3000, 17, 9001], 6301)
    o, l = _run(case, q, 1)
    for r, sh in enumerate(case.shards):
        o1, l1 = cp.cp_decode_attn_partial_gqa(q[:, 0].contiguous(), sh["kc"], sh["vc"],
                                               sh["bt_dev"], sh["ll_dev"], w.scale)
        # outputs are sums of bf16-rounded probabilities times bf16 values:
        # separately compiled code may round an O(0.1) element 1e-5 apart
        assert torch.allclose(o1, o[r, :, 0], rtol=0, atol=1e-4)
        assert torch.allclose(l1, l[r, :, 0], rtol=0, atol=1e-5)


def test_mtp_full_size_sampled():
    """The bench's shape (32 requests, 4K..32K tokens, 2 query tokens): every
    shard's partial of three requests and their merge."""
    w = ci.WORKLOADS["gqa_decode_bf16"]
    T = 2
    case, q = _mtp_case(w, T, None, 6400)
    o, l = _run(case, q, T)
    _check(case, q, T, o, l, [0, w.B // 2, w.B - 1])


def test_mtp_rejects_unsupported_and_invalid():
    # a group of 16 query heads per KV head is not a row-kernel shape
    w16 = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=2, Hq=16, Hkv=1, seed=6502)
    case16, q16 = _mtp_case(w16, 2, [100, 200], 6503)
    sh = case16.shards[0]
    with pytest.raises(cp.CpError) as e:
        cp.cp_decode_attn_partial_gqa_mtp(q16, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"],
                                          torch.from_numpy(case16.seq).to(DEV), w16.scale, 0,
                                          w16.N, w16.I)
    assert e.value.status == cp.CP_E_UNSUPPORTED
    w = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=2, seed=6500)
    case, q = _mtp_case(w, 4, [100, 200], 6501)
    sh = case.shards[0]
    seq_dev = torch.from_numpy(case.seq).to(DEV)
    with pytest.raises(cp.CpError):
        cp.cp_decode_attn_partial_gqa_mtp(q[:, :2].contiguous(), sh["kc"], sh["vc"],
                                          sh["bt_dev"], sh["ll_dev"], seq_dev, w.scale, w.N,
                                          w.N, w.I)   # rank outside the group
    # a request shorter than its query tokens is flagged NaN, the other is not
    short = torch.tensor([1, 200], dtype=torch.int32, device=DEV)
    o, l = cp.cp_decode_attn_partial_gqa_mtp(q[:, :2].contiguous(), sh["kc"], sh["vc"],
                                             sh["bt_dev"], sh["ll_dev"], short, w.scale, 0, w.N,
                                             w.I)
    torch.cuda.synchronize()
    assert torch.isnan(l[0]).all() and not torch.isnan(l[1]).any()
    # the same over two launches of two tokens (4 tokens x group 4): every
    # token of the short request is NaN, whichever launch takes it
    short = torch.tensor([3, 200], dtype=torch.int32, device=DEV)
    o, l = cp.cp_decode_attn_partial_gqa_mtp(q, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"],
                                             short, w.scale, 0, w.N, w.I)
    torch.cuda.synchronize()
    assert torch.isnan(l[0]).all() and not torch.isnan(l[1]).any()
