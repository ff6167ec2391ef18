"""GPU parity: cp_kv_gather -- the inverse of the interleaved placement -- bit for
bit against the fp64 oracle's gather and against the logical KV it must
reproduce.  Shard caches are written on the host (numpy, through the oracle's
slot map) with poisoned unused slots, so no input comes from the HIP path."""
import numpy as np
import pytest
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
import oracle
from _cases import announce

pytestmark = pytest.mark.gpu

_RAW = {torch.bfloat16: (np.uint16, torch.int16), torch.float32: (np.uint32, torch.int32),
        torch.float8_e4m3fn: (np.uint8, torch.uint8)}


def _shards(L, N, I, bs, Hkv, D, dtype, seed, latent=False, pool_extra=3):
    """Logical KV (raw bits) per request and N shard caches + block tables."""
    npdt, _ = _RAW[dtype]
    rng = np.random.default_rng(seed)
    hi = np.iinfo(npdt).max
    kv = rng.integers(0, hi, size=(int(sum(L)), Hkv, D), dtype=npdt, endpoint=True)
    if npdt == np.uint16:       # keep bf16 patterns finite (not needed for a copy, but tidy)
        kv &= np.uint16(0xBFFF)
    offs = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    B = len(L)
    caches, bts = [], []
    for r in range(N):
        ll = oracle.local_lens(np.asarray(L), r, N, I)
        need = (ll.astype(np.int64) + bs - 1) // bs
        stride = int(need.max()) + 1
        nblk = int(need.sum()) + pool_extra
        perm = rng.permutation(nblk)
        bt = np.full((B, stride), -1, dtype=np.int32)
        k = 0
        for b in range(B):
            bt[b, :need[b]] = perm[k:k + need[b]]
            k += need[b]
        cache = np.full((nblk, Hkv, bs, D), hi, dtype=npdt)  # poison: all-ones bytes
        req = np.repeat(np.arange(B, dtype=np.int32), L)
        pos = np.concatenate([np.arange(l, dtype=np.int32) for l in L]) if sum(L) else \
            np.zeros(0, np.int32)
        sl = oracle.slot_map(req, pos, bt, r, N, I, bs)
        mine = np.nonzero(sl >= 0)[0]
        cache[sl[mine] // bs, :, sl[mine] % bs, :] = kv[offs[req[mine]] + pos[mine]]
        caches.append(cache[:, 0] if latent else cache)
        bts.append(bt)
    return kv, offs, caches, bts


def _dev(a, dtype):
    npdt, tdt = _RAW[dtype]
    return torch.from_numpy(a.view(np.int16) if npdt == np.uint16 else
                            (a.view(np.int32) if npdt == np.uint32 else a)).cuda().view(dtype)


def _bits(t):
    npdt, tdt = _RAW[t.dtype]
    return t.view(tdt).cpu().numpy().view(npdt)


def _run(L, N, I, bs, Hkv, D, dtype, seed, windows, latent=False, with_v=True, corrupt=None):
    kv, offs, caches, bts = _shards(L, N, I, bs, Hkv, D, dtype, seed, latent)
    vcaches = [c ^ 0x5A for c in caches]  # distinct V bits, same placement
    if corrupt is not None:
        r, b, j = corrupt
        bts[r][b, j] = 10 ** 7
    kc = [_dev(c, dtype) for c in caches]
    vc = [_dev(c, dtype) for c in vcaches] if with_v else None
    btd = [torch.from_numpy(bt).cuda() for bt in bts]
    seq = torch.tensor(L, dtype=torch.int32, device="cuda")
    for t0, W in windows:
        announce(f"kv gather N={N} I={I} bs={bs} Hkv={Hkv} D={D} {dtype} t0={t0} W={W}")
        ko, vo = cp.cp_kv_gather(kc, vc, btd, seq, N, I, bs, t0, W)
        torch.cuda.synchronize()
        ref = oracle.kv_gather(caches, bts, L, N, I, bs, t0, W)
        got = _bits(ko)
        assert np.array_equal(got.reshape(ref.shape), ref), "K differs from the oracle gather"
        if with_v:
            vref = oracle.kv_gather(vcaches, bts, L, N, I, bs, t0, W)
            assert np.array_equal(_bits(vo).reshape(vref.shape), vref), "V differs"
        else:
            assert vo is None
        if corrupt is None:  # the gather reproduces the logical KV (zeros past each end)
            for b, l in enumerate(L):
                n = max(0, min(W, l - t0))
                assert np.array_equal(got[b, :n].reshape(n, Hkv, D),
                                      kv[offs[b] + t0:offs[b] + t0 + n])
                assert (got[b, n:] == 0).all()


def test_kv_gather_gqa_bf16_ragged_windows():
    _run([200, 37, 0, 130, 1, 4000], 3, 5, 16, 8, 128, torch.bfloat16, 7100,
         [(0, 4000), (100, 77), (3990, 40), (5000, 10), (0, 1)])


def test_kv_gather_latent_fp8_and_bf16():
    # latent caches [nblk][bs][576]: 36 (fp8) and 72 (bf16) chunks per token row
    _run([700, 64, 1000], 8, 1, 64, 1, 576, torch.float8_e4m3fn, 7200, [(0, 1000), (63, 129)],
         latent=True, with_v=False)
    _run([700, 64, 1000], 4, 2, 32, 1, 576, torch.bfloat16, 7201, [(0, 1000)], latent=True,
         with_v=False)


def test_kv_gather_f32_rows_and_bad_block_ids():
    _run([300, 1, 77], 4, 4, 16, 2, 64, torch.float32, 7300, [(0, 300)])
    # token rows of 256 chunks (8 heads x 128 fp32): the kernel's row-at-a-time path
    _run([150, 9], 2, 3, 16, 8, 128, torch.float32, 7302, [(0, 150), (140, 20)])
    # rank 1's local block 2 of request 0 names a block outside the pool:
    # exactly the positions it holds come back as 0xFF bytes
    _run([300, 1, 77], 4, 4, 16, 2, 64, torch.float32, 7301, [(0, 300), (40, 100)],
         corrupt=(1, 0, 2))


def test_kv_gather_full_prefix_workload():
    """The prefill workload's cached prefix: 64K positions in 8 DCP shards
    (I 16, bs 16), 8 KV heads x 128, bf16, K and V, gathered whole: compared
    with the logical prefix on the device, and with the oracle on a window."""
    w = ci.WORKLOADS["kv_gather_bf16"]
    P = w.P
    announce(f"{w.name}: P={P} N={w.N} I={w.I} bs={w.bs}")
    kv, offs, caches, bts = _shards([P], w.N, w.I, w.bs, w.Hkv, w.D, torch.bfloat16, w.seed)
    kc = [_dev(c, torch.bfloat16) for c in caches]
    vc = [_dev(c ^ 0x5A, torch.bfloat16) for c in caches]
    btd = [torch.from_numpy(bt).cuda() for bt in bts]
    seq = torch.tensor([P], dtype=torch.int32, device="cuda")
    ko, vo = cp.cp_kv_gather(kc, vc, btd, seq, w.N, w.I, w.bs, 0, P)
    logical = _dev(kv, torch.bfloat16).reshape(1, P, w.Hkv, w.D)
    torch.cuda.synchronize()
    assert torch.equal(ko.view(torch.int16), logical.view(torch.int16))
    assert torch.equal(vo.view(torch.int16), logical.view(torch.int16) ^ 0x5A)
    ref = oracle.kv_gather(caches, bts, [P], w.N, w.I, w.bs, 30000, 700)
    assert np.array_equal(_bits(ko)[:, 30000:30700], ref)
