"""CPU checks of the C ABI: the built library loads, exports every function
include/cpattn.h declares, its argument structs have the layout the Python
binding assumes (checked against gcc's own offsetof), and host-side argument
validation rejects bad calls before any launch (no GPU needed for those)."""
import ctypes
import os
import re
import subprocess

import pytest

from kv_context_parallelism_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_six_calls():
    names = _declared_functions()
    for n in ["cp_slot_map", "cp_cache_write", "cp_decode_attn_partial_gqa",
              "cp_decode_attn_partial_mla", "cp_lse_merge", "pcp_prefill_attn_causal",
              "cp_kv_gather"]:
        assert n in names


def test_library_exports_every_declared_function():
    lib = _lib.load()
    declared = _declared_functions()
    assert set(declared) == set(_lib.SIGNATURES), "binding and header disagree"
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared) <= exported


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.cp_abi_version() == 1
    assert lib.cp_status_str(0) == b"CP_OK"
    assert lib.cp_status_str(3) == b"CP_E_WORKSPACE"


_LAYOUT_C = r"""
#include <stddef.h>
#include <stdio.h>
#include "cpattn.h"
#define F(T, f) printf(#T " " #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("cp_gqa_args sizeof %zu\n", sizeof(cp_gqa_args));
  printf("cp_mla_args sizeof %zu\n", sizeof(cp_mla_args));
  printf("cp_prefill_args sizeof %zu\n", sizeof(cp_prefill_args));
  printf("cp_kv_gather_args sizeof %zu\n", sizeof(cp_kv_gather_args));
  printf("cp_gqa_mtp_args sizeof %zu\n", sizeof(cp_gqa_mtp_args));
  %FIELDS%
  return 0;
}
"""


@pytest.mark.parametrize("cname,pytype", [("cp_gqa_args", _lib.CpGqaArgs),
                                          ("cp_mla_args", _lib.CpMlaArgs),
                                          ("cp_prefill_args", _lib.CpPrefillArgs),
                                          ("cp_kv_gather_args", _lib.CpKvGatherArgs),
                                          ("cp_gqa_mtp_args", _lib.CpGqaMtpArgs)])
def test_struct_layout_matches_c(tmp_path, cname, pytype):
    fields = "\n".join(f"F({cname}, {f})" for f, _ in pytype._fields_)
    src = tmp_path / "layout.c"
    src.write_text(_LAYOUT_C.replace("%FIELDS%", fields))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.dirname(HEADER),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {}
    for ln in lines.splitlines():
        t, f, v = ln.split()
        got[(t, f)] = int(v)
    assert got[(cname, "sizeof")] == ctypes.sizeof(pytype)
    for f, _ in pytype._fields_:
        assert got[(cname, f)] == getattr(pytype, f).offset, f


def test_host_validation_rejects_bad_arguments():
    lib = _lib.load()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    # rank outside [0, N)
    assert lib.cp_slot_map(4, fake, fake, fake, 1, 4, 4, 4, 4, 4, 16, fake, None) == 1
    # interleave 0
    assert lib.cp_local_seq_lens(4, fake, 0, 4, 0, fake, None) == 1
    # merge: Dv not a multiple of 4 -> unsupported; zero parts -> invalid
    assert lib.cp_lse_merge(2, 10, 6, fake, fake, fake, 0, fake, None) == 2
    assert lib.cp_lse_merge(0, 10, 8, fake, fake, fake, 0, fake, None) == 1
    # cache write with v but no v_cache
    assert lib.cp_cache_write(4, fake, fake, fake, 1, 64, 1, fake, None, 8, 16, None) == 1
    # GQA: Hq not a multiple of Hkv; unsupported head dim; workspace missing
    a = _lib.CpGqaArgs(q=16, k_cache=16, v_cache=16, block_table=16, local_len=16, B=2, Hq=6,
                       Hkv=4, D=128, bs=16, bt_stride=8, num_blocks=64, scale=0.1, dt=1, out=16,
                       lse=16)
    assert lib.cp_decode_attn_partial_gqa(ctypes.byref(a), None, 0, None) == 1
    a.Hq, a.D = 8, 96
    assert lib.cp_decode_attn_partial_gqa(ctypes.byref(a), None, 0, None) == 2
    a.D, a.bs = 128, 24
    assert lib.cp_decode_attn_partial_gqa(ctypes.byref(a), None, 0, None) == 2
    a.bs, a.bt_stride = 16, 4096
    need = lib.cp_workspace_bytes(1, ctypes.byref(a))
    assert need > 0
    assert lib.cp_decode_attn_partial_gqa(ctypes.byref(a), None, 0, None) == 3
    assert b"workspace" in lib.cp_last_error()
    # prefill: chunk not aligned to 2N
    p = _lib.CpPrefillArgs(q=16, C=100, P=0, pcp_rank=0, pcp_size=8, Hq=32, Hkv=8, D=128,
                           scale=0.1, kv_source=0, k=16, v=16, out=16, lse=16)
    assert lib.pcp_prefill_attn_causal(ctypes.byref(p), None, 0, None) in (1, 2)
    # prefill: the softmax scale must be positive and finite
    p.C, p.pcp_size = 128, 2
    for bad_scale in (0.0, -0.1, float("inf"), float("nan")):
        p.scale = bad_scale
        assert lib.pcp_prefill_attn_causal(ctypes.byref(p), None, 0, None) == 1
        assert b"scale" in lib.cp_last_error()


def test_fused_slot_map_cache_write_validation():
    """The fused call rejects what either of its two steps rejects."""
    lib = _lib.load()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    args = [4, fake, fake, fake, 1, 4, 4, 0, 4, 4, 16, None, fake, fake, 2, 64, 1, fake, fake, 8,
            None]
    bad = list(args)
    bad[7] = 4  # rank outside [0, N)
    assert lib.cp_slot_map_cache_write(*bad) == 1
    bad = list(args)
    bad[6] = 5  # max_blocks past the block-table width
    assert lib.cp_slot_map_cache_write(*bad) == 1
    bad = list(args)
    bad[18] = None  # v without v_cache
    assert lib.cp_slot_map_cache_write(*bad) == 1
    bad = list(args)
    bad[15] = 4  # a 4-element bf16 row is 8 bytes, not a multiple of 16
    assert lib.cp_slot_map_cache_write(*bad) == 2
    bad = list(args)
    bad[1] = None  # req missing
    assert lib.cp_slot_map_cache_write(*bad) == 1
    bad = list(args)
    bad[0] = 0  # nothing to do
    assert lib.cp_slot_map_cache_write(*bad) == 0


def test_mla_validation_rejects_unsupported_head_counts():
    """The MLA kernel covers up to 128 heads (four waves of 32) in multiples of
    16; other head counts are refused on the host, before any device call."""
    lib = _lib.load()
    a = _lib.CpMlaArgs(q=16, kv_cache=16, block_table=16, local_len=16, B=2, H=128, Dk=576,
                       Dv=512, bs=64, bt_stride=8, num_blocks=64, scale=0.1, kv_dt=1, kv_scale=1.0,
                       out=16, lse=16)
    for bad_h in (144, 256, 24, 8):
        a.H = bad_h
        assert lib.cp_decode_attn_partial_mla(ctypes.byref(a), None, 0, None) == 2
        assert b"H=" in lib.cp_last_error()
    a.H, a.Dk = 128, 512
    assert lib.cp_decode_attn_partial_mla(ctypes.byref(a), None, 0, None) == 2
    a.Dk, a.bs = 576, 24
    assert lib.cp_decode_attn_partial_mla(ctypes.byref(a), None, 0, None) == 2


def test_kv_gather_validation():
    """cp_kv_gather refuses bad shard counts, windows, pointer pairings and row
    shapes on the host (the host pointer arrays are never dereferenced first)."""
    lib = _lib.load()
    arr = (ctypes.c_void_p * 2)(16, 32)
    nb = (ctypes.c_int64 * 2)(4, 4)
    a = _lib.CpKvGatherArgs(N=2, I=4, bs=16, B=1, Hkv=8, D=128, dt=1,
                            k_caches=ctypes.cast(arr, ctypes.c_void_p), v_caches=None,
                            block_tables=ctypes.cast(arr, ctypes.c_void_p),
                            num_blocks=ctypes.cast(nb, ctypes.c_void_p), bt_stride=4, t0=0, W=64,
                            seq_len=16, k_out=16, v_out=None)
    for field, bad in [("N", 0), ("N", 17), ("I", 0), ("bs", 0), ("W", -1), ("t0", -5)]:
        old = getattr(a, field)
        setattr(a, field, bad)
        assert lib.cp_kv_gather(ctypes.byref(a), None) == 1, field
        setattr(a, field, old)
    a.v_out = 16  # v_out without v_caches
    assert lib.cp_kv_gather(ctypes.byref(a), None) == 1
    assert b"v_caches" in lib.cp_last_error()
    a.v_out = None
    a.D = 100  # 200-byte rows are not whole 16-byte chunks
    assert lib.cp_kv_gather(ctypes.byref(a), None) == 2
    a.D, a.Hkv = 128, 6  # Hkv > 1 must be a power of two
    assert lib.cp_kv_gather(ctypes.byref(a), None) == 2
    a.Hkv, a.dt = 8, 9
    assert lib.cp_kv_gather(ctypes.byref(a), None) == 1


def test_prefill_dcp_causal_validation():
    """The causal paged source checks its DCP placement and that the shard
    holds every key the chunk's last position sees, before any launch."""
    lib = _lib.load()
    p = _lib.CpPrefillArgs(q=16, C=128, P=100, pcp_rank=0, pcp_size=2, Hq=32, Hkv=8, D=128,
                           scale=0.1, kv_source=2, k_cache=16, v_cache=16, block_table=16,
                           local_len=57, bs=16, bt_stride=8, num_blocks=64, out=16, lse=16,
                           dcp_rank=1, dcp_size=4, dcp_interleave=16)
    # positions below P + C = 228 owned by rank 1 of 4 with I = 16: 3 rounds of
    # 64 give 48, the partial round [192, 228) overlaps [208, 224) in 16: 64
    assert lib.pcp_prefill_attn_causal(ctypes.byref(p), None, 0, None) == 1
    assert b"need 64" in lib.cp_last_error()
    for field, bad in [("dcp_rank", 4), ("dcp_rank", -1), ("dcp_size", 0), ("dcp_interleave", 0)]:
        p.local_len = 64
        old = getattr(p, field)
        setattr(p, field, bad)
        assert lib.pcp_prefill_attn_causal(ctypes.byref(p), None, 0, None) == 1, field
        setattr(p, field, old)


def test_head_scatter_validation():
    """cp_lse_correct, cp_a2a_pack and cp_lse_merge_packed check sizes,
    ranks, head partitions, strides and alignment on the host."""
    lib = _lib.load()
    # rank outside [0, n_parts), Dv not a multiple of 4, misaligned output
    assert lib.cp_lse_correct(4, 8, 16, 4, 16, 16, 16, None, None) == 1
    assert lib.cp_lse_correct(4, 8, 16, -1, 16, 16, 16, None, None) == 1
    assert lib.cp_lse_correct(4, 8, 18, 0, 16, 16, 16, None, None) == 2
    assert lib.cp_lse_correct(4, 8, 16, 0, 16, 16, 20, None, None) == 1
    assert lib.cp_lse_correct(4, 0, 16, 0, None, None, None, None, None) == 0
    # H not a multiple of N; Dv % 4; NULL buffer
    assert lib.cp_a2a_pack(2, 12, 16, 8, 16, 16, 16, None) == 1
    assert lib.cp_a2a_pack(2, 16, 6, 8, 16, 16, 16, None) == 2
    assert lib.cp_a2a_pack(2, 16, 16, 8, 16, 16, None, None) == 1
    assert lib.cp_a2a_pack(0, 16, 16, 8, None, None, None, None) == 0
    # part_stride below rows * (Dv + 4), or not a multiple of 4; bad dtype
    assert lib.cp_lse_merge_packed(4, 10, 16, 16, 199, 16, 0, None, None) == 1
    assert lib.cp_lse_merge_packed(4, 10, 16, 16, 202, 16, 0, None, None) == 1
    assert b"part_stride" in lib.cp_last_error()
    assert lib.cp_lse_merge_packed(4, 10, 16, 16, 200, 16, 2, None, None) == 2
    assert lib.cp_lse_merge_packed(4, 10, 16, 24, 200, 16, 0, None, None) == 1


def test_gqa_mtp_validation():
    """The multi-token entry checks q_len, the DCP rank and interleave, the
    sequence lengths and the supported row count on the host."""
    lib = _lib.load()
    base = _lib.CpGqaArgs(q=16, k_cache=16, v_cache=16, block_table=16, local_len=16, B=2, Hq=8,
                          Hkv=2, D=128, bs=16, bt_stride=4, num_blocks=8, scale=0.1,
                          dt=_lib.CP_BF16, out=16, lse=16)
    good = dict(q_len=2, dcp_rank=1, dcp_size=4, interleave=16, seq_len=16)
    for field, bad, code in [("q_len", 0, 1), ("dcp_rank", 4, 1), ("dcp_rank", -1, 1),
                             ("dcp_size", 0, 1), ("interleave", 0, 1), ("seq_len", None, 1)]:
        kw = dict(good)
        kw[field] = bad
        m = _lib.CpGqaMtpArgs(base=base, **kw)
        assert lib.cp_decode_attn_partial_gqa_mtp(ctypes.byref(m), None, 0, None) == code, (field, bad)
    # group 4: q_len 2 is 8 rows per KV head (one launch); q_len 3, 4 and 7 are
    # taken in launches of at most 2 tokens.  All supported, so only the
    # workspace is missing -- and it is sized for one launch of 2 tokens.
    sizes = {}
    for q_len in (1, 2, 3, 4, 7):
        m = _lib.CpGqaMtpArgs(base=base, **dict(good, q_len=q_len))
        assert lib.cp_decode_attn_partial_gqa_mtp(ctypes.byref(m), None, 0, None) == 3, q_len
        sizes[q_len] = lib.cp_workspace_bytes(_lib.CP_OP_DECODE_GQA_MTP, ctypes.byref(m))
    assert 0 < sizes[1] < sizes[2] == sizes[3] == sizes[4] == sizes[7]
    # groups 2 and 1: q_len 3, 5, 6 and 7 are not powers of two and exceed no
    # limit; they run as launches of 4, 2 and 1 tokens (at most 8 rows each)
    for hq, hkv in ((8, 4), (2, 2)):
        b2 = _lib.CpGqaArgs(**{f: getattr(base, f) for f, _ in base._fields_})
        b2.Hq, b2.Hkv = hq, hkv
        for q_len in (3, 5, 6, 7):
            m = _lib.CpGqaMtpArgs(base=b2, **dict(good, q_len=q_len))
            assert lib.cp_decode_attn_partial_gqa_mtp(ctypes.byref(m), None, 0, None) == 3, (hq, hkv, q_len)
            assert lib.cp_workspace_bytes(_lib.CP_OP_DECODE_GQA_MTP, ctypes.byref(m)) > 0
    # groups the row kernel does not take: 16 heads per KV head, or D 64 in bf16
    for over in (dict(Hq=32, Hkv=2), dict(D=64)):
        b2 = _lib.CpGqaArgs(**{f: getattr(base, f) for f, _ in base._fields_})
        for f, v in over.items():
            setattr(b2, f, v)
        m = _lib.CpGqaMtpArgs(base=b2, **good)
        assert lib.cp_decode_attn_partial_gqa_mtp(ctypes.byref(m), None, 0, None) == 2, over
