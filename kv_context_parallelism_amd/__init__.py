"""libcpattn Python binding: the single-GPU hot path of decode / prefill context
parallelism on MI355X, as thin argument marshalling over the C ABI
(include/cpattn.h).

Every function takes torch tensors that live on the GPU (torch supplies the
device memory and the current HIP stream; all computation runs in the HIP
kernels of libcpattn.so).  Errors raise ``CpError`` carrying the library's
status and message.  There is no fallback: if libcpattn.so is missing the
first call raises ImportError.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (CP_BF16, CP_E_HIP, CP_E_INVALID, CP_E_UNSUPPORTED, CP_E_WORKSPACE, CP_F32,
                   CP_FP8_E4M3FN, CP_KV_DENSE, CP_KV_PAGED, CP_KV_PAGED_CAUSAL, CP_OK,
                   CP_OP_DECODE_GQA, CP_OP_DECODE_GQA_MTP,
                   CP_OP_DECODE_MLA, CP_OP_PREFILL, CP_SLOT_INVALID, CP_SLOT_NOT_MINE, CP_MAX_SHARDS)

__all__ = [
    "CpError", "cp_local_seq_lens", "cp_slot_map", "cp_cache_write", "cp_decode_attn_partial_gqa",
    "cp_decode_attn_partial_gqa_mtp", "gqa_mtp_args", "cp_decode_attn_partial_gqa_noalloc",
    "cp_decode_attn_partial_mla", "cp_lse_merge", "cp_lse_correct", "cp_a2a_pack",
    "cp_lse_merge_packed", "pcp_prefill_attn_causal", "cp_workspace_bytes",
    "gqa_args", "mla_args", "prefill_args", "library_path", "cp_kv_gather", "kv_gather_args",
]

_DT = {torch.float32: CP_F32, torch.bfloat16: CP_BF16, torch.float8_e4m3fn: CP_FP8_E4M3FN}


class CpError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        self.status = status
        msg = lib.cp_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.cp_status_str(status).decode()}: {msg}")


def library_path() -> str:
    return _lib.LIB_PATH


def _check(st: int, where: str):
    if st != CP_OK:
        raise CpError(st, where)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libcpattn takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libcpattn takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def _i32(t, name):
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32")
    return _ptr(t)


# Shape and dtype checks of the binding.  The kernels trust the sizes they are
# given (a cache's block dimension, a buffer's row count), so a tensor whose
# shape disagrees with them would be read or written out of bounds: every
# wrapper checks its tensors here, before any pointer is taken.

def _shape(t, shape, name, dtype=None):
    """t must have exactly ``shape`` (None entries match any size) and, if given,
    ``dtype``."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dim() != len(shape) or any(s is not None and t.shape[i] != s
                                    for i, s in enumerate(shape)):
        want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _count(t, n, name, dtype=torch.int32):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} elements, expected {n}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _block_table(bt, B, name="block_table"):
    """A 2-D int32 table with a row for each of the B requests."""
    if bt is None or bt.dim() != 2 or bt.dtype != torch.int32:
        raise ValueError(f"{name} must be a 2-D int32 tensor")
    if bt.shape[0] < B or bt.shape[1] < 1:
        raise ValueError(f"{name} has shape {list(bt.shape)}: needs {B} rows of at least one "
                         "block")


def _rows_and_caches(T, k, v, k_cache, v_cache, bs):
    """Token rows and paged caches of a cache write: GQA k, v [T][Hkv][D] into
    caches [num_blocks][Hkv][bs][D]; MLA k [T][Dk] (or [T][1][Dk]) into a
    latent cache [num_blocks][bs][Dk].  Returns (heads, row elements)."""
    if (v is None) != (v_cache is None):
        raise ValueError("v and v_cache must both be given (GQA) or both be None (MLA)")
    if v is None:
        if k_cache.dim() != 3:
            raise ValueError(f"latent cache has shape {list(k_cache.shape)}, expected "
                             "[num_blocks, bs, Dk]")
        row = k_cache.shape[2]
        if k.dim() == 3:
            _shape(k, (T, 1, row), "k")
        else:
            _shape(k, (T, row), "k")
        _shape(k_cache, (None, bs, row), "k_cache", k.dtype)
        return 1, row
    _shape(k, (T, None, None), "k")
    heads, row = k.shape[1], k.shape[2]
    _shape(v, tuple(k.shape), "v", k.dtype)
    _shape(k_cache, (None, heads, bs, row), "k_cache", k.dtype)
    _shape(v_cache, tuple(k_cache.shape), "v_cache", k.dtype)
    return heads, row


# ---------------------------------------------------------------------------
# ownership and paging
# ---------------------------------------------------------------------------

def cp_local_seq_lens(seq_lens, rank: int, N: int, I: int, out=None, stream=None):
    """Local KV length of each request on ``rank`` (int32 [B])."""
    lib = _lib.load()
    B = seq_lens.numel()
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=seq_lens.device)
    _count(out, B, "out")
    _check(lib.cp_local_seq_lens(B, _i32(seq_lens, "seq_lens"), rank, N, I, _i32(out, "out"),
                                 _stream(stream)), "cp_local_seq_lens")
    return out


def cp_slot_map(req, pos, block_table, rank: int, N: int, I: int, bs: int, max_blocks=None,
                out=None, stream=None):
    """Slot of every token on ``rank`` (int64 [T]; -1 not mine, -2 invalid)."""
    lib = _lib.load()
    T = req.numel()
    _count(pos, T, "pos")
    _block_table(block_table, 1)
    B, stride = block_table.shape
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=req.device)
    _count(out, T, "out", torch.int64)
    mb = stride if max_blocks is None else max_blocks
    _check(lib.cp_slot_map(T, _i32(req, "req"), _i32(pos, "pos"),
                           _i32(block_table, "block_table"), B, stride, mb, rank, N, I, bs,
                           _ptr(out), _stream(stream)), "cp_slot_map")
    return out


def cp_cache_write(slot, k, v, k_cache, v_cache, bs: int, stream=None):
    """Scatter token rows to their slots.  GQA: k, v [T][Hkv][D] into caches
    [num_blocks][Hkv][bs][D].  MLA: k [T][Dk] latent rows, v = v_cache = None,
    cache [num_blocks][bs][Dk]."""
    lib = _lib.load()
    T = slot.numel()
    if slot.dtype != torch.int64:
        raise ValueError("slot must be int64")
    heads, row = _rows_and_caches(T, k, v, k_cache, v_cache, bs)
    num_blocks = k_cache.shape[0]
    _check(lib.cp_cache_write(T, _ptr(slot), _ptr(k), _ptr(v), heads, row, _dt(k), _ptr(k_cache),
                              _ptr(v_cache), num_blocks, bs, _stream(stream)), "cp_cache_write")


def cp_slot_map_cache_write(req, pos, block_table, rank: int, N: int, I: int, bs: int, k, v,
                            k_cache, v_cache, max_blocks=None, slot_out=None, stream=None):
    """cp_slot_map then cp_cache_write in one launch (same results); the slots
    go to ``slot_out`` (int64 [T]) when it is given."""
    lib = _lib.load()
    T = req.numel()
    _count(pos, T, "pos")
    _block_table(block_table, 1)
    B, stride = block_table.shape
    mb = stride if max_blocks is None else max_blocks
    heads, row = _rows_and_caches(T, k, v, k_cache, v_cache, bs)
    if slot_out is not None:
        _count(slot_out, T, "slot_out", torch.int64)
    _check(lib.cp_slot_map_cache_write(T, _i32(req, "req"), _i32(pos, "pos"),
                                       _i32(block_table, "block_table"), B, stride, mb, rank, N, I,
                                       bs, _ptr(slot_out), _ptr(k), _ptr(v), heads, row, _dt(k),
                                       _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
                                       _stream(stream)), "cp_slot_map_cache_write")
    return slot_out


# ---------------------------------------------------------------------------
# decode partials
# ---------------------------------------------------------------------------

def _gqa_common(q, k_cache, v_cache, block_table, local_len, B, Hq, D):
    if k_cache is None or k_cache.dim() != 4:
        raise ValueError("k_cache must be [num_blocks, Hkv, bs, D]")
    _shape(k_cache, (None, None, None, D), "k_cache", q.dtype)
    _shape(v_cache, tuple(k_cache.shape), "v_cache", q.dtype)
    _block_table(block_table, B)
    _count(local_len, B, "local_len")
    return k_cache.shape


def gqa_args(q, k_cache, v_cache, block_table, local_len, scale, out, lse):
    if q.dim() != 3:
        raise ValueError(f"q has shape {list(q.shape)}, expected [B, Hq, D]")
    B, Hq, D = q.shape
    nb, Hkv, bs, _ = _gqa_common(q, k_cache, v_cache, block_table, local_len, B, Hq, D)
    _shape(out, (B, Hq, D), "out", torch.float32)
    _shape(lse, (B, Hq), "lse", torch.float32)
    return _lib.CpGqaArgs(q=_ptr(q), k_cache=_ptr(k_cache), v_cache=_ptr(v_cache),
                          block_table=_i32(block_table, "block_table"),
                          local_len=_i32(local_len, "local_len"), B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                          bt_stride=block_table.shape[1], num_blocks=nb, scale=scale, dt=_dt(q),
                          out=_ptr(out), lse=_ptr(lse))


def mla_args(q, kv_cache, block_table, local_len, scale, out, lse, Dv=512, kv_scale=1.0):
    if q.dim() != 3:
        raise ValueError(f"q has shape {list(q.shape)}, expected [B, H, Dk]")
    if q.dtype != torch.bfloat16:
        raise ValueError(f"q has dtype {q.dtype}, expected torch.bfloat16")
    B, H, Dk = q.shape
    if kv_cache is None or kv_cache.dim() != 3:
        raise ValueError("kv_cache must be [num_blocks, bs, Dk]")
    _shape(kv_cache, (None, None, Dk), "kv_cache")
    if kv_cache.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
        raise ValueError(f"kv_cache has dtype {kv_cache.dtype}, expected bf16 or fp8 e4m3fn")
    nb, bs, _ = kv_cache.shape
    _block_table(block_table, B)
    _count(local_len, B, "local_len")
    _shape(out, (B, H, Dv), "out", torch.float32)
    _shape(lse, (B, H), "lse", torch.float32)
    return _lib.CpMlaArgs(q=_ptr(q), kv_cache=_ptr(kv_cache),
                          block_table=_i32(block_table, "block_table"),
                          local_len=_i32(local_len, "local_len"), B=B, H=H, Dk=Dk, Dv=Dv, bs=bs,
                          bt_stride=block_table.shape[1], num_blocks=nb, scale=scale,
                          kv_dt=_dt(kv_cache), kv_scale=kv_scale, out=_ptr(out), lse=_ptr(lse))


def cp_workspace_bytes(op: int, args) -> int:
    n = _lib.load().cp_workspace_bytes(op, ctypes.byref(args))
    if n == ctypes.c_size_t(-1).value:
        raise CpError(CP_E_INVALID, "cp_workspace_bytes")
    return int(n)


def _workspace(op, args, device, workspace):
    need = cp_workspace_bytes(op, args)
    if need == 0:
        return None, 0
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def cp_decode_attn_partial_gqa(q, k_cache, v_cache, block_table, local_len, scale, out=None,
                               lse=None, workspace=None, stream=None):
    """Partial attention of q [B][Hq][D] over one shard's paged KV; returns
    (out fp32 [B][Hq][D], lse fp32 [B][Hq])."""
    lib = _lib.load()
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    a = gqa_args(q, k_cache, v_cache, block_table, local_len, scale, out, lse)
    ws, nws = _workspace(CP_OP_DECODE_GQA, a, q.device, workspace)
    _check(lib.cp_decode_attn_partial_gqa(ctypes.byref(a), _ptr(ws), nws, _stream(stream)),
           "cp_decode_attn_partial_gqa")
    return out, lse


def cp_decode_attn_partial_gqa_noalloc(q, k_cache, v_cache, block_table, local_len, scale, out,
                                       lse, stream=None):
    """cp_decode_attn_partial_gqa without a workspace: the split partials use the
    library's per-device scratch, so nothing is allocated -- the caller passes
    out (fp32 [B][Hq][D]) and lse (fp32 [B][Hq]).  Calls that overlap on one
    device race on that scratch."""
    lib = _lib.load()
    a = gqa_args(q, k_cache, v_cache, block_table, local_len, scale, out, lse)
    _check(lib.cp_decode_attn_partial_gqa_noalloc(ctypes.byref(a), _stream(stream)),
           "cp_decode_attn_partial_gqa_noalloc")
    return out, lse


def gqa_mtp_args(q, k_cache, v_cache, block_table, local_len, seq_len, scale, out, lse, rank, N,
                 I):
    """Arguments of the multi-token entry; q [B][T][Hq][D], out [B][T][Hq][D],
    lse [B][T][Hq]."""
    if q.dim() != 4:
        raise ValueError(f"q has shape {list(q.shape)}, expected [B, T, Hq, D]")
    B, T, Hq, D = q.shape
    nb, Hkv, bs, _ = _gqa_common(q, k_cache, v_cache, block_table, local_len, B, Hq, D)
    _count(seq_len, B, "seq_len")
    _shape(out, (B, T, Hq, D), "out", torch.float32)
    _shape(lse, (B, T, Hq), "lse", torch.float32)
    base = _lib.CpGqaArgs(q=_ptr(q), k_cache=_ptr(k_cache), v_cache=_ptr(v_cache),
                          block_table=_i32(block_table, "block_table"),
                          local_len=_i32(local_len, "local_len"), B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                          bt_stride=block_table.shape[1], num_blocks=nb, scale=scale, dt=_dt(q),
                          out=_ptr(out), lse=_ptr(lse))
    return _lib.CpGqaMtpArgs(base=base, q_len=T, dcp_rank=int(rank), dcp_size=int(N),
                             interleave=int(I), seq_len=_i32(seq_len, "seq_len"))


def cp_decode_attn_partial_gqa_mtp(q, k_cache, v_cache, block_table, local_len, seq_len, scale,
                                   rank, N, I, out=None, lse=None, workspace=None, stream=None):
    """Partial attention of T query tokens per request, q [B][T][Hq][D] (the
    last T positions of each request, causal on the shard's interleaved
    positions), over one shard's paged KV; returns (out fp32 [B][T][Hq][D],
    lse fp32 [B][T][Hq])."""
    lib = _lib.load()
    B, T, Hq, D = q.shape
    if out is None:
        out = torch.empty(B, T, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, T, Hq, dtype=torch.float32, device=q.device)
    a = gqa_mtp_args(q, k_cache, v_cache, block_table, local_len, seq_len, scale, out, lse, rank,
                     N, I)
    ws, nws = _workspace(CP_OP_DECODE_GQA_MTP, a, q.device, workspace)
    _check(lib.cp_decode_attn_partial_gqa_mtp(ctypes.byref(a), _ptr(ws), nws, _stream(stream)),
           "cp_decode_attn_partial_gqa_mtp")
    return out, lse


def cp_decode_attn_partial_mla(q, kv_cache, block_table, local_len, scale, Dv=512, kv_scale=1.0,
                               out=None, lse=None, workspace=None, stream=None):
    """Absorbed-MLA partial attention of q [B][H][Dk] (bf16) over one shard's
    latent cache [num_blocks][bs][Dk]; returns (out fp32 [B][H][Dv], lse [B][H])."""
    lib = _lib.load()
    B, H, _ = q.shape
    if out is None:
        out = torch.empty(B, H, Dv, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
    a = mla_args(q, kv_cache, block_table, local_len, scale, out, lse, Dv=Dv, kv_scale=kv_scale)
    ws, nws = _workspace(CP_OP_DECODE_MLA, a, q.device, workspace)
    _check(lib.cp_decode_attn_partial_mla(ctypes.byref(a), _ptr(ws), nws, _stream(stream)),
           "cp_decode_attn_partial_mla")
    return out, lse


# ---------------------------------------------------------------------------
# merge
# ---------------------------------------------------------------------------

def cp_lse_merge(part_out, part_lse, out=None, lse_out=None, out_dtype=torch.float32,
                 stream=None):
    """Exact merge of part_out [n][rows...][Dv] with part_lse [n][rows...]."""
    lib = _lib.load()
    n = part_out.shape[0]
    Dv = part_out.shape[-1]
    rows = part_lse[0].numel()
    if part_out.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise ValueError("partials must be fp32")
    if part_out.numel() != n * rows * Dv:
        raise ValueError("part_out / part_lse shape mismatch")
    if out is None:
        out = torch.empty(part_out.shape[1:], dtype=out_dtype, device=part_out.device)
    if lse_out is None:
        lse_out = torch.empty(part_lse.shape[1:], dtype=torch.float32, device=part_out.device)
    if out.numel() != rows * Dv or out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out must hold rows x Dv = {rows * Dv} fp32 or bf16 elements")
    _count(lse_out, rows, "lse_out", torch.float32)
    _check(lib.cp_lse_merge(n, rows, Dv, _ptr(part_out), _ptr(part_lse), _ptr(out), _dt(out),
                            _ptr(lse_out), _stream(stream)), "cp_lse_merge")
    return out, lse_out


def cp_lse_correct(part_out_i, part_lse, rank, corrected=None, lse_out=None, stream=None):
    """AG+RS correction of one rank's partial part_out_i [rows...][Dv] given
    every rank's LSE part_lse [n][rows...]: part_out_i * exp(L_rank - L)."""
    lib = _lib.load()
    n = part_lse.shape[0]
    Dv = part_out_i.shape[-1]
    rows = part_lse[0].numel()
    if part_out_i.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise ValueError("partials must be fp32")
    if part_out_i.numel() != rows * Dv:
        raise ValueError("part_out_i / part_lse shape mismatch")
    if corrected is None:
        corrected = torch.empty_like(part_out_i)
    if lse_out is None:
        lse_out = torch.empty(part_lse.shape[1:], dtype=torch.float32, device=part_lse.device)
    _count(corrected, rows * Dv, "corrected", torch.float32)
    _count(lse_out, rows, "lse_out", torch.float32)
    _check(lib.cp_lse_correct(n, rows, Dv, int(rank), _ptr(part_out_i), _ptr(part_lse),
                              _ptr(corrected), _ptr(lse_out), _stream(stream)), "cp_lse_correct")
    return corrected, lse_out


def cp_a2a_pack(out, lse, N, buf=None, stream=None):
    """All-to-all send buffer [N][B][H/N][Dv+4] of one rank's out [B][H][Dv]
    and lse [B][H] (fp32)."""
    lib = _lib.load()
    B, H, Dv = out.shape
    if out.dtype != torch.float32 or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H):
        raise ValueError("out [B][H][Dv] and lse [B][H] must be fp32")
    if H % N:
        raise ValueError(f"H={H} is not a multiple of N={N}")
    if buf is None:
        buf = torch.empty((N, B, H // N, Dv + 4), dtype=torch.float32, device=out.device)
    _shape(buf, (N, B, H // N, Dv + 4), "buf", torch.float32)
    _check(lib.cp_a2a_pack(B, H, Dv, N, _ptr(out), _ptr(lse), _ptr(buf), _stream(stream)),
           "cp_a2a_pack")
    return buf


def cp_lse_merge_packed(packed, Dv, out=None, lse_out=None, out_dtype=torch.float32,
                        stream=None):
    """Exact merge of packed partials: packed [n][rows...][Dv+4] (any strides
    between parts, rows contiguous inside a part)."""
    lib = _lib.load()
    n = packed.shape[0]
    lead = tuple(packed.shape[1:-1])
    rows = 1
    for x in lead:
        rows *= x
    if packed.dtype != torch.float32 or packed.shape[-1] != Dv + 4:
        raise ValueError("packed must be fp32 with rows of Dv + 4")
    if not packed[0].is_contiguous():
        raise ValueError("rows of one part must be contiguous")
    if not packed.is_cuda:
        raise ValueError("libcpattn takes device tensors")
    stride = packed.stride(0) if n > 1 else rows * (Dv + 4)
    if out is None:
        out = torch.empty(lead + (Dv,), dtype=out_dtype, device=packed.device)
    if lse_out is None:
        lse_out = torch.empty(lead, dtype=torch.float32, device=packed.device)
    if out.numel() != rows * Dv or out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out must hold rows x Dv = {rows * Dv} fp32 or bf16 elements")
    _count(lse_out, rows, "lse_out", torch.float32)
    _check(lib.cp_lse_merge_packed(n, rows, Dv, ctypes.c_void_p(packed.data_ptr()), stride, _ptr(out), _dt(out),
                                   _ptr(lse_out), _stream(stream)), "cp_lse_merge_packed")
    return out, lse_out


# ---------------------------------------------------------------------------
# PCP causal prefill
# ---------------------------------------------------------------------------

def prefill_args(q, P, pcp_rank, pcp_size, scale, out, lse, *, k=None, v=None, k_cache=None,
                 v_cache=None, block_table=None, local_len=0, dcp=None):
    """``dcp=(rank, size, interleave)`` selects the causal paged source (a DCP
    shard holding prefix and chunk keys)."""
    if q.dim() != 3 or q.dtype != torch.bfloat16:
        raise ValueError(f"q must be bf16 [C, Hq, D], got {q.dtype} {list(q.shape)}")
    C, Hq, D = q.shape
    dr, ds, di = dcp if dcp is not None else (0, 1, 1)
    if (k is None) == (k_cache is None):
        raise ValueError("give either the chunk's k, v (dense) or a paged k_cache, v_cache")
    if k is not None:
        if k_cache is not None or v_cache is not None or block_table is not None or dcp:
            raise ValueError("the dense source takes no paged arguments")
        _shape(k, (C, None, D), "k", torch.bfloat16)
        _shape(v, tuple(k.shape), "v", torch.bfloat16)
        src, Hkv = CP_KV_DENSE, k.shape[1]
        nb, bs, stride = 0, 16, 1
    else:
        if k is not None or v is not None:
            raise ValueError("the paged source takes no dense k, v")
        if k_cache.dim() != 4:
            raise ValueError("k_cache must be [num_blocks, Hkv, bs, D]")
        _shape(k_cache, (None, None, None, D), "k_cache", torch.bfloat16)
        _shape(v_cache, tuple(k_cache.shape), "v_cache", torch.bfloat16)
        if block_table is None or block_table.dim() != 1 or block_table.dtype != torch.int32:
            raise ValueError("block_table must be a 1-D int32 tensor (the shard's blocks)")
        src, Hkv = (CP_KV_PAGED if dcp is None else CP_KV_PAGED_CAUSAL), k_cache.shape[1]
        nb, bs, stride = k_cache.shape[0], k_cache.shape[2], block_table.numel()
    if pcp_size < 1 or C % (2 * pcp_size):
        raise ValueError(f"C={C} must be a multiple of 2 x pcp_size={pcp_size}")
    c = C // (2 * pcp_size)
    _shape(out, (2, c, Hq, D), "out", torch.float32)
    _shape(lse, (2, c, Hq), "lse", torch.float32)
    return _lib.CpPrefillArgs(
        q=_ptr(q), C=C, P=P, pcp_rank=pcp_rank, pcp_size=pcp_size, Hq=Hq, Hkv=Hkv, D=D,
        scale=scale, kv_source=src, k=_ptr(k), v=_ptr(v), k_cache=_ptr(k_cache),
        v_cache=_ptr(v_cache), block_table=None if block_table is None else _i32(block_table, "bt"),
        local_len=int(local_len), bs=bs, bt_stride=stride, num_blocks=nb, out=_ptr(out),
        lse=_ptr(lse), dcp_rank=dr, dcp_size=ds, dcp_interleave=di)


def pcp_prefill_attn_causal(q, P, pcp_rank, pcp_size, scale, *, k=None, v=None, k_cache=None,
                            v_cache=None, block_table=None, local_len=0, dcp=None, out=None,
                            lse=None, stream=None):
    """Rank ``pcp_rank``'s two pieces of the chunk q [C][Hq][D] (bf16) against
    the chunk's own keys (k, v: causal), one DCP shard of the prefix
    (k_cache, v_cache, block_table, local_len), or -- with
    ``dcp=(rank, size, interleave)`` -- one DCP shard holding prefix and chunk
    keys, causal on their interleaved positions.  Returns (out fp32
    [2][C/2N][Hq][D], lse fp32 [2][C/2N][Hq])."""
    lib = _lib.load()
    C, Hq, D = q.shape
    c = C // (2 * pcp_size) if pcp_size >= 1 else 0
    if out is None:
        out = torch.empty(2, c, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(2, c, Hq, dtype=torch.float32, device=q.device)
    a = prefill_args(q, P, pcp_rank, pcp_size, scale, out, lse, k=k, v=v, k_cache=k_cache,
                     v_cache=v_cache, block_table=block_table, local_len=local_len, dcp=dcp)
    _check(lib.pcp_prefill_attn_causal(ctypes.byref(a), None, 0, _stream(stream)),
           "pcp_prefill_attn_causal")
    return out, lse


# ---------------------------------------------------------------------------
# KV gather (the inverse of the interleaved placement)
# ---------------------------------------------------------------------------

def kv_gather_args(k_caches, v_caches, block_tables, seq_len, N: int, I: int, bs: int, t0: int,
                   W: int, k_out, v_out):
    """The argument struct plus the host pointer arrays it refers to (keep the
    returned tuple alive for the duration of the call)."""
    if len(k_caches) != N or len(block_tables) != N or (v_caches is not None and len(v_caches) != N):
        raise ValueError("one cache and one block table per shard")
    kc0 = k_caches[0]
    if kc0.dim() not in (3, 4):
        raise ValueError("caches must be [num_blocks, Hkv, bs, D] or [num_blocks, bs, D]")
    Hkv, D = (kc0.shape[1], kc0.shape[3]) if kc0.dim() == 4 else (1, kc0.shape[2])
    B = int(seq_len.shape[0])
    row = (None, Hkv, bs, D) if kc0.dim() == 4 else (None, bs, D)
    for r in range(N):
        _shape(k_caches[r], row, f"k_caches[{r}]", kc0.dtype)
        if v_caches is not None:
            _shape(v_caches[r], tuple(k_caches[r].shape), f"v_caches[{r}]", kc0.dtype)
        _block_table(block_tables[r], B, f"block_tables[{r}]")
        if block_tables[r].shape[1] != block_tables[0].shape[1]:
            raise ValueError("every shard's block table must have the same width")
    _count(seq_len, B, "seq_len")
    _shape(k_out, (B, W, Hkv, D), "k_out", kc0.dtype)
    if (v_out is None) != (v_caches is None):
        raise ValueError("v_out must be given exactly when v_caches is")
    if v_out is not None:
        _shape(v_out, (B, W, Hkv, D), "v_out", kc0.dtype)
    arr = ctypes.c_void_p * N
    kp = arr(*[_ptr(c).value for c in k_caches])
    vp = arr(*[_ptr(c).value for c in v_caches]) if v_caches is not None else None
    for bt in block_tables:
        _i32(bt, "block_table")
    bp = arr(*[_ptr(bt).value for bt in block_tables])
    nb = (ctypes.c_int64 * N)(*[int(c.shape[0]) for c in k_caches])
    a = _lib.CpKvGatherArgs(N=N, I=I, bs=bs, B=int(seq_len.shape[0]), Hkv=Hkv, D=D, dt=_dt(kc0),
                            k_caches=ctypes.cast(kp, ctypes.c_void_p),
                            v_caches=ctypes.cast(vp, ctypes.c_void_p) if vp is not None else None,
                            block_tables=ctypes.cast(bp, ctypes.c_void_p),
                            num_blocks=ctypes.cast(nb, ctypes.c_void_p),
                            bt_stride=int(block_tables[0].shape[1]), t0=t0, W=W,
                            seq_len=_i32(seq_len, "seq_len"), k_out=_ptr(k_out), v_out=_ptr(v_out))
    return a, (kp, vp, bp, nb)


def cp_kv_gather(k_caches, v_caches, block_tables, seq_len, N: int, I: int, bs: int, t0: int,
                 W: int, k_out=None, v_out=None, stream=None):
    """Window [t0, t0 + W) of every request's KV, gathered from the N shard
    caches (each [num_blocks][Hkv][bs][D], or [num_blocks][bs][D] for a latent
    cache) through their block tables ([B][bt_stride] int32 each).  Returns
    (k_out, v_out) of shape [B][W][Hkv][D] (v_out None without v_caches)."""
    lib = _lib.load()
    kc0 = k_caches[0]
    Hkv, D = (kc0.shape[1], kc0.shape[3]) if kc0.dim() == 4 else (1, kc0.shape[2])
    B = int(seq_len.shape[0])
    if k_out is None:
        k_out = torch.empty(B, W, Hkv, D, dtype=kc0.dtype, device=kc0.device)
    if v_out is None and v_caches is not None:
        v_out = torch.empty(B, W, Hkv, D, dtype=kc0.dtype, device=kc0.device)
    a, keep = kv_gather_args(k_caches, v_caches, block_tables, seq_len, N, I, bs, t0, W, k_out,
                             v_out)
    _check(lib.cp_kv_gather(ctypes.byref(a), _stream(stream)), "cp_kv_gather")
    del keep
    return k_out, v_out
