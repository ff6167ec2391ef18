"""fp64 CPU oracle for the context-parallel attention path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``kv_context_parallelism_amd``) never does, and nothing here imports it.

Thin numpy/ctypes glue over ``oracle.c`` (plain fp64 loops), plus the
piece bookkeeping of PCP's head-tail split, which is small enough to state
directly in Python.

Pages followed (cited by title and section):
  [P1] "Breaking the Long-Sequence Inference Bottleneck: A Deep Dive into
       vLLM's Distributed Context Parallelism Architecture"
  [P3] "vLLM DCP and PCP: Decode and Prefill Context Parallelism"

Every function is pinned by tests/test_oracle_pins.py; none is "parity
unpinned" except where that file says so.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "bf16": 1, "fp8_e4m3fn": 2}
_RAW = {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3fn": np.uint8}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "oracle.c")
    if (not os.path.exists(_LIB_PATH)
            or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src)):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32p, i64p, dp = (ctypes.c_int64, ctypes.POINTER(ctypes.c_int32),
                           ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double))
    vp = ctypes.c_void_p
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_e4m3fn.restype = ctypes.c_double
    lib.oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
    lib.oracle_owner.restype = i64
    lib.oracle_owner.argtypes = [i64, i64, i64]
    lib.oracle_local_lens.restype = None
    lib.oracle_local_lens.argtypes = [i64, i32p, i64, i64, i64, i32p]
    lib.oracle_slot_map.restype = None
    lib.oracle_slot_map.argtypes = [i64, i32p, i32p, i32p, i64, i64, i64, i64, i64, i64, i64p]
    lib.oracle_attention.restype = None
    lib.oracle_attention.argtypes = [
        i64, i64, i64, i64, i64,            # n_q Hq Hkv Dk Dv
        i32p, i64,                          # heads n_heads
        vp, ctypes.c_int, i64, i64,         # q
        vp, ctypes.c_int, i64, i64, ctypes.c_double,   # k
        vp, ctypes.c_int, i64, i64, ctypes.c_double,   # v
        i64p, i64p,                         # key_begin key_end
        i64, i64, i64,                      # shard N I r
        ctypes.c_double, dp, dp]
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_lse_merge.restype = None
    lib.oracle_lse_merge.argtypes = [i64, i64, i64, dp, dp, dp, dp]
    _lib = lib
    return lib


def set_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (timing only: the
    results are the same for every thread count)."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# --------------------------------------------------------------------------
# element decoding
# --------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 values (upper half of a binary32)."""
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_decode_bf16(int(b)) for b in flat]).reshape(np.shape(bits))


def decode_e4m3fn(bits: np.ndarray) -> np.ndarray:
    """OCP fp8 E4M3 (finite-only) bit patterns -> fp64 values."""
    lib = _load()
    flat = np.ascontiguousarray(bits, dtype=np.uint8).ravel()
    return np.array([lib.oracle_decode_e4m3fn(int(b)) for b in flat]).reshape(np.shape(bits))


# --------------------------------------------------------------------------
# ownership, local lengths, slot mapping   ([P1] section 2, [P3] Deep Dive 5)
# --------------------------------------------------------------------------

def owner(t: int, N: int, I: int) -> int:
    """Rank that stores position t: floor(t / I) mod N ([P1] section 2)."""
    return int(_load().oracle_owner(int(t), int(N), int(I)))


def local_lens(seq_lens, rank: int, N: int, I: int) -> np.ndarray:
    """Per-request count of positions in [0, L) owned by ``rank``."""
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.zeros(sl.shape[0], dtype=np.int32)
    _load().oracle_local_lens(sl.shape[0], _ptr(sl, ctypes.c_int32), rank, N, I,
                              _ptr(out, ctypes.c_int32))
    return out


def slot_map(req, pos, block_table: np.ndarray, rank: int, N: int, I: int, bs: int,
             max_blocks: int | None = None) -> np.ndarray:
    """Physical cache slot of each token on ``rank``; -1 where another rank owns
    it, -2 where its local block index is past the block table's width."""
    req = np.ascontiguousarray(req, dtype=np.int32)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    stride = bt.shape[1]
    mb = stride if max_blocks is None else max_blocks
    out = np.empty(req.shape[0], dtype=np.int64)
    _load().oracle_slot_map(req.shape[0], _ptr(req, ctypes.c_int32), _ptr(pos, ctypes.c_int32),
                            _ptr(bt, ctypes.c_int32), stride, mb, rank, N, I, bs,
                            _ptr(out, ctypes.c_int64))
    return out


# --------------------------------------------------------------------------
# attention and merge   ([P3] Deep Dive 6)
# --------------------------------------------------------------------------

def attention(q, k, v, *, key_begin, key_end, scale: float, q_dtype: str, kv_dtype: str,
              Dv: int | None = None, kv_scale: float = 1.0, shard=None, heads=None):
    """Exact softmax attention in fp64.

    q: raw array [n_q, Hq, Dk]; k: raw array [n_k, Hkv, Dk]; v: raw array
    [n_k, Hkv, Dv_total] of which the first ``Dv`` columns are the values
    (for an absorbed-MLA latent, pass the latent as both k and v).
    Raw arrays hold storage bits: float32 for "f32", uint16 for "bf16",
    uint8 for "fp8_e4m3fn" (decoded value times ``kv_scale``).
    Query row i attends to keys t with key_begin[i] <= t < key_end[i] and,
    if ``shard=(N, I, r)``, owner(t) == r.
    Returns (out [n_q, n_heads, Dv] fp64, lse [n_q, n_heads] fp64).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=_RAW[q_dtype])
    k = np.ascontiguousarray(k, dtype=_RAW[kv_dtype])
    v = np.ascontiguousarray(v, dtype=_RAW[kv_dtype])
    assert q.ndim == 3 and k.ndim == 3 and v.ndim == 3
    n_q, Hq, Dk = q.shape
    n_k, Hkv, Dk2 = k.shape
    assert Dk2 == Dk and v.shape[0] == n_k and v.shape[1] == Hkv
    Dv = v.shape[2] if Dv is None else Dv
    assert Dv <= v.shape[2]
    kb = np.ascontiguousarray(np.broadcast_to(key_begin, (n_q,)), dtype=np.int64)
    ke = np.ascontiguousarray(np.broadcast_to(key_end, (n_q,)), dtype=np.int64)
    assert kb.min(initial=0) >= 0 and ke.max(initial=0) <= n_k
    if heads is None:
        hp, nh = None, Hq
    else:
        hs = np.ascontiguousarray(heads, dtype=np.int32)
        hp, nh = _ptr(hs, ctypes.c_int32), hs.shape[0]
    sN, sI, sr = (0, 1, 0) if shard is None else shard
    out = np.zeros((n_q, nh, Dv), dtype=np.float64)
    lse = np.zeros((n_q, nh), dtype=np.float64)
    lib.oracle_attention(
        n_q, Hq, Hkv, Dk, Dv, hp, nh,
        q.ctypes.data, DTYPES[q_dtype], Hq * Dk, Dk,
        k.ctypes.data, DTYPES[kv_dtype], Hkv * Dk, Dk, float(kv_scale),
        v.ctypes.data, DTYPES[kv_dtype], Hkv * v.shape[2], v.shape[2], float(kv_scale),
        _ptr(kb, ctypes.c_int64), _ptr(ke, ctypes.c_int64), sN, sI, sr,
        float(scale), _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return out, lse


def decode_mtp(q, k, v, *, L: int, scale: float, q_dtype: str, kv_dtype: str, shard=None):
    """Multi-token decode of one request ([P1] "Inapplicable scenarios and known
    limitations" and [P4] "Future Roadmap": DCP combined with MTP / speculative
    decoding; [P1] section 4: a token sees itself and earlier positions).

    q: raw [T, Hq, D], the request's last T positions L-T .. L-1; k, v: raw
    [L, Hkv, D], the whole sequence.  Token t attends positions 0 .. L-T+t
    (and, with ``shard=(N, I, r)``, only those rank r owns).  Returns
    (out [T, Hq, D], lse [T, Hq]) in fp64; a token with no visible key gets
    zeros and -inf.
    """
    T = q.shape[0]
    assert 1 <= T <= L
    key_end = np.arange(L - T + 1, L + 1, dtype=np.int64)
    return attention(q, k, v, key_begin=0, key_end=key_end, scale=scale, q_dtype=q_dtype,
                     kv_dtype=kv_dtype, shard=shard)


def lse_merge(part_out, part_lse):
    """Exact merge of partial attention results ([P3] Deep Dive 6).

    part_out [n, rows, Dv], part_lse [n, rows] -> (out [rows, Dv], lse [rows])."""
    po = np.ascontiguousarray(part_out, dtype=np.float64)
    pl = np.ascontiguousarray(part_lse, dtype=np.float64)
    n, rows, Dv = po.shape
    assert pl.shape == (n, rows)
    out = np.zeros((rows, Dv), dtype=np.float64)
    lse = np.zeros(rows, dtype=np.float64)
    _load().oracle_lse_merge(n, rows, Dv, _ptr(po, ctypes.c_double), _ptr(pl, ctypes.c_double),
                             _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return out, lse


# --------------------------------------------------------------------------
# Head-scattered exchanges around the merge   ([P3] Deep Dive 6: AG+RS, AG+AR
# and the all-to-all path)
# --------------------------------------------------------------------------

def lse_correct(part_out_i, part_lse, rank: int):
    """AG+RS correction of rank ``rank``'s partial ([P3] Deep Dive 6): after the
    LSE all-gather every rank knows L = log sum_i exp(L_i) per row and scales
    its own normalised output by exp(L_rank - L); the reduce-scatter then adds
    the corrected outputs of all ranks.  A part with L_i = -inf gets factor 0;
    a row whose parts are all -inf gets zeros and L = -inf.

    part_out_i [rows, Dv], part_lse [n, rows] -> (corrected [rows, Dv], L [rows])."""
    po = np.asarray(part_out_i, dtype=np.float64)
    pl = np.asarray(part_lse, dtype=np.float64)
    n, rows = pl.shape
    assert po.shape[0] == rows and 0 <= rank < n
    out = np.zeros_like(po)
    L = np.full(rows, -np.inf)
    for r in range(rows):
        l = pl[:, r].max()
        if l == -np.inf:
            continue
        L[r] = l + np.log(sum(np.exp(x - l) for x in pl[:, r] if x != -np.inf))
        if pl[rank, r] != -np.inf:
            out[r] = po[r] * np.exp(pl[rank, r] - L[r])
    return out, L


def a2a_pack(out, lse, N: int):
    """All-to-all send buffer of one rank ([P3] Deep Dive 6: each partial output
    travels with its fp32 LSE in one buffer, and destination d is sent the
    d-th of N equal head partitions).  out [B, H, Dv], lse [B, H] ->
    [N, B, H/N, Dv + 4] float32: the Dv outputs, the LSE, three zeros."""
    out = np.asarray(out, dtype=np.float32)
    lse = np.asarray(lse, dtype=np.float32)
    B, H, Dv = out.shape
    assert lse.shape == (B, H) and H % N == 0
    hs = H // N
    buf = np.zeros((N, B, hs, Dv + 4), dtype=np.float32)
    for d in range(N):
        for b in range(B):
            for j in range(hs):
                buf[d, b, j, :Dv] = out[b, d * hs + j]
                buf[d, b, j, Dv] = lse[b, d * hs + j]
    return buf


def all_to_all(send):
    """The exchange itself, on stacked per-rank send buffers: rank d receives,
    in source order, what every rank s put in its slot d.
    send [N_src, N_dst, ...] -> recv [N_dst, N_src, ...]."""
    send = np.asarray(send)
    return np.ascontiguousarray(np.swapaxes(send, 0, 1))


def lse_merge_packed(recv, Dv: int):
    """Exact merge of packed partials ([P3] Deep Dive 6, the LSE-weighted
    reduction after the all-to-all): recv [n, ..., Dv + 4] holds each part's
    outputs followed by its LSE.  Returns (out [..., Dv], lse [...])."""
    recv = np.asarray(recv)
    n = recv.shape[0]
    lead = recv.shape[1:-1]
    rows = int(np.prod(lead)) if lead else 1
    flat = recv.reshape(n, rows, recv.shape[-1])
    o, l = lse_merge(flat[:, :, :Dv], flat[:, :, Dv])
    return o.reshape(*lead, Dv), l.reshape(lead)


# --------------------------------------------------------------------------
# PCP head-tail split   ([P1] section 4; [P3] Deep Dive 3)
# --------------------------------------------------------------------------

def pcp_pieces(N: int, r: int):
    """The sequence is cut into 2N equal pieces; rank r computes piece r (head)
    and piece 2N-1-r (tail), in that order ([P1] section 4, "Head-tail
    concatenation strategy")."""
    assert 0 <= r < N
    return (r, 2 * N - 1 - r)


def pcp_rank_positions(C: int, N: int, r: int, P: int = 0) -> np.ndarray:
    """Global positions of rank r's query rows, head piece first, for a chunk of
    C new tokens that starts at position P.  C must be a multiple of 2N
    ([P1] section 4, "Minimal state progression": alignment to 2 x PCP size)."""
    assert C % (2 * N) == 0
    c = C // (2 * N)
    return np.concatenate([P + p * c + np.arange(c) for p in pcp_pieces(N, r)]).astype(np.int64)


# --------------------------------------------------------------------------
# KV gather   ([P1] section 3 "MLA path": the gathered KV of all ranks is put
# back into each request's own order; section 2: the placement it inverts)
# --------------------------------------------------------------------------

def kv_gather(caches, block_tables, seq_lens, N: int, I: int, bs: int, t0: int, W: int):
    """Rows t0 .. t0+W-1 of every request's KV, read back from N shard caches.

    caches[r]: raw element array [nblk][Hkv][bs][D] (or [nblk][bs][D] for a
    latent cache) of rank r; block_tables[r]: [B][stride] int32.  Row (b, i) is
    position t = t0 + i of request b: for t < L_b it is the cache row of rank
    owner(t) at the slot ``slot_map`` gives t on that rank (head h at
    [slot // bs][h][slot % bs]); for t >= L_b it is zero; where the slot map
    reports a block index past the table (-2) or the block id lies outside the
    cache, every byte is 0xFF.  Returns [B][W][Hkv][D] of the caches' dtype.
    """
    caches = [np.asarray(c) for c in caches]
    latent = caches[0].ndim == 3
    cs = [c[:, None, :, :] if latent else c for c in caches]  # [nblk][Hkv][bs][D]
    Hkv, D = cs[0].shape[1], cs[0].shape[3]
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = seq_lens.shape[0]
    out = np.zeros((B, W, Hkv, D), dtype=caches[0].dtype)
    out_bytes = out.view(np.uint8).reshape(B, W, -1)
    for b in range(B):
        n = int(max(0, min(W, seq_lens[b] - t0)))
        if n == 0:
            continue
        pos = np.arange(t0, t0 + n, dtype=np.int32)
        req = np.full(n, b, dtype=np.int32)
        for r in range(N):
            slots = slot_map(req, pos, block_tables[r], r, N, I, bs)
            for i in np.nonzero(slots != -1)[0]:
                s = int(slots[i])
                blk = s // bs if s >= 0 else -1
                if s == -2 or blk < 0 or blk >= cs[r].shape[0]:
                    out_bytes[b, i, :] = 0xFF
                else:
                    out[b, i] = cs[r][blk, :, s % bs, :]
    return out
