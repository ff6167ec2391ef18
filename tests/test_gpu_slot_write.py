"""GPU: cp_slot_map_cache_write (both steps in one launch) gives exactly the
slots and cache bytes of cp_slot_map followed by cp_cache_write, for GQA rows
and MLA latent rows, every rank, with invalid requests / positions, local
blocks past the table and block ids past the pool among the tokens."""
import pytest
import torch

import kv_context_parallelism_amd as cp
from _cases import announce

pytestmark = pytest.mark.gpu


def _tokens(lens, g):
    req = torch.cat([torch.full((L,), b, dtype=torch.int32) for b, L in enumerate(lens)])
    pos = torch.cat([torch.arange(L, dtype=torch.int32) for L in lens])
    # invalid entries: request -1 and B, a negative position
    req = torch.cat([req, torch.tensor([-1, len(lens), 0], dtype=torch.int32)])
    pos = torch.cat([pos, torch.tensor([3, 3, -5], dtype=torch.int32)])
    perm = torch.randperm(req.numel(), generator=g)
    return req[perm].contiguous(), pos[perm].contiguous()


@pytest.mark.parametrize("mla,N,I,bs,Hkv,D,dtype", [
    (False, 8, 16, 16, 8, 128, torch.bfloat16),
    (False, 4, 4, 16, 2, 64, torch.float32),
    (True, 8, 1, 64, 1, 576, torch.bfloat16),
    (False, 3, 5, 24, 2, 128, torch.bfloat16),   # block size not a power of two
])
def test_fused_equals_two_calls(mla, N, I, bs, Hkv, D, dtype):
    g = torch.Generator().manual_seed(6100 + N + D)
    lens = [700, 1, 2500]
    req, pos = _tokens(lens, g)
    T = req.numel()
    rows = torch.randn(T, Hkv, D, generator=g).to(dtype)
    k = rows[:, 0, :].contiguous() if mla else rows
    v = None if mla else torch.randn(T, Hkv, D, generator=g).to(dtype)
    per_rank = [-(-L // (N * I)) * I for L in lens]
    width = max(-(-p // bs) for p in per_rank)
    nblk = 3 * width + 4
    for r in range(N):
        announce(f"fused slot map + cache write mla={mla} N={N} I={I} bs={bs} rank={r}")
        bt = torch.randperm(nblk, generator=g)[:3 * width].view(3, width).to(torch.int32)
        bt[1, 0] = nblk + 7  # a block id past the pool: its token is skipped
        bt_d = bt.cuda()
        shape = (nblk, bs, D) if mla else (nblk, Hkv, bs, D)
        kc_a = torch.full(shape, float("nan"), dtype=dtype, device="cuda")
        kc_b, kc_c = kc_a.clone(), kc_a.clone()
        vc_a = None if mla else kc_a.clone()
        vc_b = None if mla else kc_a.clone()
        vc_c = None if mla else kc_a.clone()
        kd, vd = k.cuda(), (None if mla else v.cuda())
        rq, ps = req.cuda(), pos.cuda()
        mb = width - 1  # the last column is past max_blocks: slot -2 for its tokens
        slots_a = cp.cp_slot_map(rq, ps, bt_d, r, N, I, bs, max_blocks=mb)
        cp.cp_cache_write(slots_a, kd, vd, kc_a, vc_a, bs)
        slots_b = torch.full((T,), 12345, dtype=torch.int64, device="cuda")
        cp.cp_slot_map_cache_write(rq, ps, bt_d, r, N, I, bs, kd, vd, kc_b, vc_b, max_blocks=mb,
                                   slot_out=slots_b)
        cp.cp_slot_map_cache_write(rq, ps, bt_d, r, N, I, bs, kd, vd, kc_c, vc_c, max_blocks=mb)
        torch.cuda.synchronize()
        assert torch.equal(slots_a, slots_b)
        assert (slots_a == -1).any() and (slots_a == -2).any() and (slots_a >= 0).any()
        for a, b in [(kc_a, kc_b), (kc_a, kc_c)] + ([] if mla else [(vc_a, vc_b), (vc_a, vc_c)]):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
