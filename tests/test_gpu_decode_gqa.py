"""GPU parity: slot mapping, cache write, GQA decode partials and the exact LSE
merge against the fp64 oracle (element by element), on the tiny fp32 workload,
ragged multi-request cases, and the full 32-request bf16 workload (sampled
requests), plus negative controls that the gates must catch."""
import math

import numpy as np
import pytest
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
import oracle
from _cases import (announce, build_decode_case, gate_f32, gate_lowp, lowp_gate_passes,
                    oracle_request, run_partials)

pytestmark = pytest.mark.gpu


def _check_case(case, requests, lowp):
    w = case.w
    po, pl = run_partials(case)
    mo, ml = cp.cp_lse_merge(po, pl)
    torch.cuda.synchronize()
    po, pl, mo, ml = po.cpu().numpy(), pl.cpu().numpy(), mo.cpu().numpy(), ml.cpu().numpy()
    for b in requests:
        for r in range(w.N):
            ro, rl = oracle_request(case, b, shard=(w.N, w.I, r))
            if lowp:
                gate_lowp(po[r, b], ro, f"partial out r{r} b{b}", 2e-2)
                gate_lowp(pl[r, b], rl, f"partial lse r{r} b{b}", 1e-3, norm=None)
            else:
                gate_f32(po[r, b], ro, f"partial out r{r} b{b}")
                gate_f32(pl[r, b], rl, f"partial lse r{r} b{b}")
        ro, rl = oracle_request(case, b)
        if lowp:
            gate_lowp(mo[b], ro, f"merged out b{b}", 2e-2)
            gate_lowp(ml[b], rl, f"merged lse b{b}", 1e-3, norm=None)
        else:
            gate_f32(mo[b], ro, f"merged out b{b}")
            gate_f32(ml[b], rl, f"merged lse b{b}")


def test_gqa_tiny_f32():
    w = ci.WORKLOADS["gqa_tiny_f32"]
    announce(f"{w.name} seed={w.seed}")
    case = build_decode_case(w)
    assert [int(s["ll"][0]) for s in case.shards] == [252, 252, 248, 248]
    _check_case(case, [0], lowp=False)


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 8, 2), (128, 8, 8), (128, 16, 8), (64, 16, 2),
                                      (128, 16, 4)])
def test_gqa_f32_ragged(D, Hq, Hkv):
    # lengths 0 and 3 leave shards empty; others end mid-block and mid-group
    w = ci.scaled(ci.WORKLOADS["gqa_tiny_f32"], B=6, Hq=Hq, Hkv=Hkv, D=D, Dv=D, N=4, I=4,
                  scale=1 / math.sqrt(D), seed=2100 + D + Hq)
    announce(f"f32 ragged D={D} Hq={Hq} Hkv={Hkv}")
    case = build_decode_case(w, seq=[0, 3, 17, 1000, 5003, 257])
    _check_case(case, range(6), lowp=False)


@pytest.mark.parametrize("N,I,bs", [(8, 16, 16), (8, 1, 64), (4, 16, 32), (2, 64, 16)])
def test_gqa_bf16_ragged(N, I, bs):
    w = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=5, N=N, I=I, bs=bs, seed=2200 + N + I + bs)
    announce(f"bf16 ragged N={N} I={I} bs={bs}")
    case = build_decode_case(w, seq=[1, 100, 2049, 7777, 33])
    _check_case(case, range(5), lowp=True)


@pytest.mark.parametrize("B", [63, 64, 97])
def test_gqa_bf16_many_requests(B):
    """Below 64 requests each wave scans the chunk counts itself and finds a
    chunk's request by one ballot; from 64 on the kernel takes the
    workgroup-wide scan and a binary search.  Ragged lengths with empty
    requests (zero) between long ones, every request checked."""
    rng = np.random.default_rng(2600 + B)
    seq = [int(x) for x in rng.integers(0, 3000, size=B)]
    seq[0], seq[B // 2], seq[-1] = 0, 1, 0
    w = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=B, seed=2600 + B)
    announce(f"bf16 B={B} ragged")
    case = build_decode_case(w, seq=seq, check_cache=False, check_slots=False)
    _check_case(case, range(B), lowp=True)


def test_gqa_bf16_full_workload_sampled():
    w = ci.WORKLOADS["gqa_decode_bf16"]
    announce(f"{w.name} full size, seed={w.seed}")
    case = build_decode_case(w, pool_factor=1.25)
    _check_case(case, [0, 13, 31], lowp=True)


def test_gqa_f32_wide_group_is_rejected():
    # fp32, 8 query heads per KV head, head dim 128: the query no longer fits the
    # register budget; the call reports CP_E_UNSUPPORTED instead of spilling
    w = ci.scaled(ci.WORKLOADS["gqa_tiny_f32"], B=1, Hq=16, Hkv=2, D=128, Dv=128, seed=2150)
    case = build_decode_case(w, seq=[40], check_cache=False)
    sh = case.shards[0]
    with pytest.raises(cp.CpError, match="CP_E_UNSUPPORTED"):
        cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"],
                                      w.scale)


def test_gqa_deterministic_and_workspace():
    w = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=3, seed=2300)
    case = build_decode_case(w, seq=[5000, 9000, 20000], check_cache=False)
    a1 = run_partials(case)
    for _ in range(8):  # the split combine sums the partials in slot order
        a2 = run_partials(case)
        assert torch.equal(a1[0], a2[0]) and torch.equal(a1[1], a2[1])
    sh = case.shards[0]
    out = torch.empty(3, w.Hq, w.D, device="cuda")
    lse = torch.empty(3, w.Hq, device="cuda")
    args = cp.gqa_args(case.q, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"], w.scale, out, lse)
    need = cp.cp_workspace_bytes(cp.CP_OP_DECODE_GQA, args)
    assert need > 0
    # the workspace need not be initialised: random bytes, all ones, all zeros
    g = torch.Generator(device="cuda").manual_seed(7)
    fills = [torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g),
             torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda"),
             torch.zeros(need, dtype=torch.uint8, device="cuda")]
    ref = cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"],
                                        w.scale)
    for ws in fills:
        o, l = cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], sh["bt_dev"],
                                             sh["ll_dev"], w.scale, workspace=ws)
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1])
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cp.CpError):
        # an explicit workspace that is too small is rejected before launch
        cp._check(cp._lib.load().cp_decode_attn_partial_gqa(
            __import__("ctypes").byref(args), cp._ptr(small), 16, cp._stream()), "gqa")


def test_gqa_negative_controls():
    """Corrupted metadata must fail the gates (or be flagged NaN)."""
    w = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=4, seed=2400)
    case = build_decode_case(w, seq=[3000, 4100, 6000, 8000])
    sh = case.shards[0]
    ro, rl = oracle_request(case, 2, shard=(w.N, w.I, 0))
    o, l = cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"],
                                         w.scale)
    assert lowp_gate_passes(o[2].cpu().numpy(), ro, 2e-2)
    # point one block-table entry of request 2 at a block holding request 1's keys
    # (swapping two entries of one request would only permute its key set, which
    # attention does not see)
    bt = sh["bt_dev"].clone()
    bt[2, 0] = bt[1, 0]
    o, l = cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], bt, sh["ll_dev"], w.scale)
    assert not lowp_gate_passes(o[2].cpu().numpy(), ro, 2e-2)
    # write the shard with the interleave shifted by one: the stored rows are the
    # wrong positions for this rank
    kc, vc = torch.full_like(sh["kc"], 0.0), torch.full_like(sh["vc"], 0.0)
    total = int(case.offs[-1])
    req = torch.from_numpy(np.repeat(np.arange(w.B, dtype=np.int32), case.seq)).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(L, dtype=np.int32)
                                           for L in case.seq])).cuda()
    slots = cp.cp_slot_map(req, pos, sh["bt_dev"], 0, w.N, w.I + 1, w.bs)
    cp.cp_cache_write(slots, case.k, case.v, kc, vc, w.bs)
    o, l = cp.cp_decode_attn_partial_gqa(case.q, kc, vc, sh["bt_dev"], sh["ll_dev"], w.scale)
    assert total > 0 and not lowp_gate_passes(o[2].cpu().numpy(), ro, 2e-2)
    # out-of-range block id: that request becomes NaN, the others stay exact
    bt = sh["bt_dev"].clone()
    bt[1, 0] = sh["pool"] + 5
    o, l = cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], bt, sh["ll_dev"], w.scale)
    o, l = o.cpu(), l.cpu()
    assert torch.isnan(o[1]).all() and torch.isnan(l[1]).all()
    assert lowp_gate_passes(o[2].numpy(), ro, 2e-2)
    # local length beyond the block table's capacity: NaN as well
    ll = sh["ll_dev"].clone()
    ll[3] = sh["bt"].shape[1] * w.bs + 1
    o, l = cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], sh["bt_dev"], ll, w.scale)
    assert torch.isnan(o[3].cpu()).all()


# (parts, rows, Dv): the lane-parallel merge (few parts, rows up to 1024 wide,
# part counts not a multiple of its batch of 8) and the block merge (many
# parts, or wider rows)
@pytest.mark.parametrize("n,rows,Dv", [(9, 5000, 128), (3, 2700, 512), (1, 140000, 4), (13, 2600, 1024),
                                       (100, 520, 128), (5, 530, 2048)])
def test_lse_merge_against_oracle(n, rows, Dv):
    g = torch.Generator().manual_seed(77 + n + Dv)
    po = torch.randn(n, rows, Dv, generator=g)
    pl = 5 * torch.randn(n, rows, generator=g)
    pl[n // 2, :100] = float("-inf")     # empty parts
    po[n // 2, :100] = float("nan")      # their outputs must not be read
    pl[:, rows - 3] = float("-inf")      # a row with every part empty
    announce(f"lse merge n={n} rows={rows} Dv={Dv}")
    mo, ml = cp.cp_lse_merge(po.cuda(), pl.cuda())
    mb, _ = cp.cp_lse_merge(po.cuda(), pl.cuda(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(po.double().numpy(), pl.double().numpy())
    gate_f32(mo.cpu().numpy(), ro, "merge out")
    gate_f32(ml.cpu().numpy(), rl, "merge lse")
    assert (mo[rows - 3] == 0).all() and torch.isneginf(ml[rows - 3])
    # bf16 output: exactly the round-to-nearest-even of the same kernel's fp32
    # result (the fp32 result is gated against the oracle above; near-zero
    # outputs of cancelling sums keep only the fp32 gate's absolute accuracy,
    # so a one-ulp check against the exact value would not hold there)
    assert torch.equal(mb.cpu(), mo.cpu().to(torch.bfloat16))
    # NaN LSE propagates to its row only
    pl2 = pl.clone()
    pl2[n - 1, 7] = float("nan")
    mo2, ml2 = cp.cp_lse_merge(po.cuda(), pl2.cuda())
    assert torch.isnan(mo2[7].cpu()).all() and torch.isnan(ml2[7].cpu())
    assert torch.equal(mo2[8], mo[8])


def test_gqa_one_workspace_many_calls_and_long_request():
    """One workspace reused across calls of different shapes, an empty request,
    and a single long request whose (request, KV head) rows are split over
    hundreds of waves (hundreds of partials in one exact merge)."""
    w = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=1, seed=2500)
    long_case = build_decode_case(w, seq=[300000], check_cache=False, check_slots=False)
    w2 = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=5, seed=2501)
    short_case = build_decode_case(w2, seq=[17, 40, 4000, 0, 9000], check_cache=False)
    need = 0
    for case in (long_case, short_case):
        sh = case.shards[0]
        a = cp.gqa_args(case.q, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"], case.w.scale,
                        torch.empty(case.w.B, case.w.Hq, case.w.D, device="cuda"),
                        torch.empty(case.w.B, case.w.Hq, device="cuda"))
        need = max(need, cp.cp_workspace_bytes(cp.CP_OP_DECODE_GQA, a))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ref = {}
    for rep in range(3):
        for name, case in (("long", long_case), ("short", short_case)):
            sh = case.shards[0]
            o, l = cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], sh["bt_dev"],
                                                 sh["ll_dev"], case.w.scale, workspace=ws)
            torch.cuda.synchronize()
            if rep == 0:
                ref[name] = (o.clone(), l.clone())
            else:
                assert torch.equal(o, ref[name][0]) and torch.equal(l, ref[name][1]), name
    for name, case in (("long", long_case), ("short", short_case)):
        o, l = ref[name]
        for b in range(case.w.B):
            ro, rl = oracle_request(case, b, shard=(case.w.N, case.w.I, 0))
            gate_lowp(o[b].cpu().numpy(), ro, f"{name} out b{b}", 2e-2)
            gate_lowp(l[b].cpu().numpy(), rl, f"{name} lse b{b}", 1e-3, norm=None)
