"""GPU parity: the per-rank kernels around the head-scattered output exchanges
(AG+RS correction, all-to-all packing, packed merge) against the fp64 oracle,
on seeded partials and on real shard partials of the decode kernels."""
import numpy as np
import pytest
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
import oracle
from _cases import announce, build_decode_case, gate_f32, gate_lowp, oracle_request, run_partials

pytestmark = pytest.mark.gpu


def _partials(n, rows, Dv, seed):
    g = torch.Generator().manual_seed(seed)
    po = torch.randn(n, rows, Dv, generator=g)
    pl = 5 * torch.randn(n, rows, generator=g)
    pl[n // 2, :100] = float("-inf")     # empty parts
    po[n // 2, :100] = float("nan")      # their outputs must not be read
    pl[:, rows - 3] = float("-inf")      # a row with every part empty
    return po, pl


# (parts, rows, Dv): lane groups of 8 (Dv 20: five float4 columns, ragged), 32,
# 64 with two and four columns per lane; part counts below, at and above the
# lane group, so a lane reads several LSEs
@pytest.mark.parametrize("n,rows,Dv", [(8, 3000, 20), (3, 2700, 128), (100, 1500, 512),
                                       (64, 700, 1024), (1, 4100, 4)])
def test_lse_correct_against_oracle(n, rows, Dv):
    po, pl = _partials(n, rows, Dv, 300 + n + Dv)
    total = torch.zeros(rows, Dv, dtype=torch.float64)
    ranks = sorted({0, n // 2, n - 1})
    for r in range(n):
        announce(f"lse correct n={n} rows={rows} Dv={Dv} rank={r}") if r in ranks else None
        co, L = cp.cp_lse_correct(po[r].cuda(), pl.cuda(), r)
        torch.cuda.synchronize()
        if r in ranks:
            rc, rL = oracle.lse_correct(po[r].double().numpy(), pl.double().numpy(), r)
            gate_f32(co.cpu().numpy(), rc, f"corrected rank {r}")
            gate_f32(L.cpu().numpy(), rL, "L")
            assert (co[rows - 3] == 0).all() and torch.isneginf(L[rows - 3])
        total += co.cpu().double()
    if n * rows * Dv <= 2e7:
        # the reduce-scatter's sum of all ranks' corrections is the exact merge
        ro, _ = oracle.lse_merge(po.double().numpy(), pl.double().numpy())
        d = np.abs(total.numpy() - ro)
        assert d.max() <= 1e-5 * np.abs(ro).max() * max(1.0, np.sqrt(n) / 4)
    # a NaN LSE poisons its row only
    pl2 = pl.clone()
    pl2[n - 1, 7] = float("nan")
    co2, L2 = cp.cp_lse_correct(po[0].cuda(), pl2.cuda(), 0)
    co1, _ = cp.cp_lse_correct(po[0].cuda(), pl.cuda(), 0)
    assert torch.isnan(co2[7].cpu()).all() and torch.isnan(L2[7].cpu())
    assert torch.equal(co2[8], co1[8])


@pytest.mark.parametrize("B,H,Dv,N", [(5, 16, 512, 8), (3, 16, 128, 4), (7, 8, 4, 8),
                                      (64, 128, 512, 8), (1, 6, 36, 3), (2, 4, 16, 1)])
def test_a2a_pack_bit_exact(B, H, Dv, N):
    g = torch.Generator().manual_seed(400 + B + H + Dv)
    out = torch.randn(B, H, Dv, generator=g)
    lse = 3 * torch.randn(B, H, generator=g)
    lse[0, 0] = float("-inf")
    announce(f"a2a pack B={B} H={H} Dv={Dv} N={N}")
    buf = torch.full((N, B, H // N, Dv + 4), float("nan"), device="cuda")
    cp.cp_a2a_pack(out.cuda(), lse.cuda(), N, buf=buf)
    torch.cuda.synchronize()
    ref = oracle.a2a_pack(out.numpy(), lse.numpy(), N)
    assert np.array_equal(buf.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def _send_buffers(o, l, N):
    """Stacked send buffers of the N ranks: [src][dst][B][H/N][Dv+4]."""
    return torch.stack([cp.cp_a2a_pack(o[r], l[r], N) for r in range(o.shape[0])])


@pytest.mark.parametrize("N,B,H,Dv", [(8, 5, 16, 512), (4, 33, 8, 128), (8, 64, 128, 512),
                                      (2, 300, 64, 64)])
def test_lse_merge_packed_after_exchange(N, B, H, Dv):
    g = torch.Generator().manual_seed(500 + N + B)
    o = torch.randn(N, B, H, Dv, generator=g)
    l = 4 * torch.randn(N, B, H, generator=g)
    l[N - 1, :2] = float("-inf")
    l[:, B - 1, 0] = float("-inf")
    o[N - 1, :2] = float("nan")
    send = _send_buffers(o.cuda(), l.cuda(), N)
    ref_send = np.stack([oracle.a2a_pack(o[r].numpy(), l[r].numpy(), N) for r in range(N)])
    assert np.array_equal(send.cpu().numpy().view(np.uint32), ref_send.view(np.uint32))
    recv = oracle.all_to_all(ref_send)  # the oracle's own exchange of its own packing
    hs = H // N
    for d in range(N):
        announce(f"merge packed N={N} B={B} H={H} Dv={Dv} dest={d}")
        mo, ml = cp.cp_lse_merge_packed(send[:, d], Dv)     # strided view: no exchange copy
        mb, _ = cp.cp_lse_merge_packed(send[:, d], Dv, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        ro, rl = oracle.lse_merge_packed(recv[d], Dv)
        gate_f32(mo.cpu().numpy(), ro, f"packed merge dest {d}")
        gate_f32(ml.cpu().numpy(), rl, "packed merge lse")
        assert torch.equal(mb.cpu(), mo.cpu().to(torch.bfloat16))
        # the same numbers cp_lse_merge gives on that head slice
        so = o[:, :, d * hs:(d + 1) * hs].contiguous().cuda()
        sl = l[:, :, d * hs:(d + 1) * hs].contiguous().cuda()
        uo, ul = cp.cp_lse_merge(so, sl)
        assert torch.equal(uo, mo) and torch.equal(ul, ml)


@pytest.mark.parametrize("name", ["mla_decode_bf16", "gqa_decode_bf16"])
def test_decode_partials_through_both_exchanges(name):
    """Shard partials of the decode kernels, then (a) AG+RS: each rank's
    corrected output, summed over ranks, and (b) all-to-all: pack, exchange,
    packed merge per destination head slice -- each against the fp64 oracle's
    attention over the whole context."""
    w = ci.scaled(ci.WORKLOADS[name], B=3, seed=4100)
    case = build_decode_case(w, seq=[700, 1, 2500], check_cache=False, check_slots=False)
    N = w.N
    o, l = run_partials(case)
    H, Dv = o.shape[2], o.shape[3]
    hs = H // N
    # (a) AG+RS
    acc = torch.zeros(w.B, H, Dv, device="cuda")
    for r in range(N):
        c, L = cp.cp_lse_correct(o[r], l, r)
        acc += c
    # (b) all-to-all
    send = _send_buffers(o, l, N)
    slices = [cp.cp_lse_merge_packed(send[:, d], Dv) for d in range(N)]
    a2a_o = torch.cat([s[0] for s in slices], dim=1)
    a2a_l = torch.cat([s[1] for s in slices], dim=1)
    torch.cuda.synchronize()
    for b in range(w.B):
        announce(f"{name} exchanges request {b} (L={case.seq[b]})")
        ro, rl = oracle_request(case, b)
        gate_lowp(acc[b].cpu().numpy(), ro, "AG+RS sum", atol=2e-2)
        gate_lowp(a2a_o[b].cpu().numpy(), ro, "A2A merge", atol=2e-2)
        gate_lowp(a2a_l[b].cpu().numpy(), rl, "A2A lse", atol=1e-3, norm=None)
        gate_lowp(L[b].cpu().numpy(), rl, "AG+RS L", atol=1e-3, norm=None)
        # rank d keeps heads d*hs .. (d+1)*hs - 1
        assert torch.equal(a2a_o[b, hs:2 * hs], slices[1][0][b])
