"""CPU checks of the binding's shape and dtype validation: a tensor whose shape
disagrees with the sizes the kernels are given (a cache's block dimension, a
buffer's row count, a request count) must raise ValueError before any pointer
is taken.  With CPU tensors a well-formed call gets past every check and stops
at the device-tensor check, which shows that the checks accept it."""
import pytest
import torch

import kv_context_parallelism_amd as cp

BF, F32, I32, I64 = torch.bfloat16, torch.float32, torch.int32, torch.int64
DEVICE_MSG = "device tensors"


def _gqa(B=3, Hq=8, Hkv=2, D=64, nb=10, bs=16, width=4, dt=F32):
    return dict(q=torch.zeros(B, Hq, D, dtype=dt),
                k_cache=torch.zeros(nb, Hkv, bs, D, dtype=dt),
                v_cache=torch.zeros(nb, Hkv, bs, D, dtype=dt),
                block_table=torch.zeros(B, width, dtype=I32),
                local_len=torch.zeros(B, dtype=I32),
                out=torch.zeros(B, Hq, D, dtype=F32), lse=torch.zeros(B, Hq, dtype=F32))


def _call_gqa(a):
    return cp.cp_decode_attn_partial_gqa(a["q"], a["k_cache"], a["v_cache"], a["block_table"],
                                         a["local_len"], 0.125, out=a["out"], lse=a["lse"])


def test_gqa_well_formed_reaches_device_check():
    with pytest.raises(ValueError, match=DEVICE_MSG):
        _call_gqa(_gqa())


@pytest.mark.parametrize("field,bad,msg", [
    ("v_cache", torch.zeros(10, 2, 8, 64), "v_cache has shape"),
    ("k_cache", torch.zeros(10, 2, 16, 32), "k_cache has shape"),
    ("k_cache", torch.zeros(10, 2, 16, 64, dtype=BF), "k_cache has dtype"),
    ("out", torch.zeros(3, 8, 64, dtype=BF), "out has dtype"),
    ("out", torch.zeros(2, 8, 64), "out has shape"),
    ("lse", torch.zeros(3, 4), "lse has shape"),
    ("local_len", torch.zeros(2, dtype=I32), "local_len has 2 elements"),
    ("block_table", torch.zeros(2, 4, dtype=I32), "needs 3 rows"),
    ("block_table", torch.zeros(3, 4, dtype=I64), "2-D int32"),
])
def test_gqa_mismatch_raises(field, bad, msg):
    a = _gqa()
    a[field] = bad
    with pytest.raises(ValueError, match=msg):
        _call_gqa(a)


def test_gqa_mtp_mismatch_raises():
    B, T, Hq, Hkv, D = 2, 2, 8, 2, 64
    args = dict(q=torch.zeros(B, T, Hq, D), k_cache=torch.zeros(4, Hkv, 16, D),
                v_cache=torch.zeros(4, Hkv, 16, D), block_table=torch.zeros(B, 2, dtype=I32),
                local_len=torch.zeros(B, dtype=I32), seq_len=torch.zeros(B, dtype=I32))
    call = lambda **kw: cp.cp_decode_attn_partial_gqa_mtp(  # noqa: E731
        args["q"], args["k_cache"], args["v_cache"], args["block_table"], args["local_len"],
        kw.get("seq_len", args["seq_len"]), 0.125, 0, 2, 16, out=kw.get("out"), lse=kw.get("lse"))
    with pytest.raises(ValueError, match=DEVICE_MSG):
        call()
    with pytest.raises(ValueError, match="seq_len has 1 elements"):
        call(seq_len=torch.zeros(1, dtype=I32))
    with pytest.raises(ValueError, match="out has shape"):
        call(out=torch.zeros(B, 1, Hq, D))
    with pytest.raises(ValueError, match="lse has shape"):
        call(lse=torch.zeros(B, T, Hq + 1))


def _mla(B=2, H=16, nb=6, bs=64, dt=BF):
    return dict(q=torch.zeros(B, H, 576, dtype=BF), kv_cache=torch.zeros(nb, bs, 576, dtype=dt),
                block_table=torch.zeros(B, 3, dtype=I32), local_len=torch.zeros(B, dtype=I32),
                out=torch.zeros(B, H, 512), lse=torch.zeros(B, H))


def _call_mla(a):
    return cp.cp_decode_attn_partial_mla(a["q"], a["kv_cache"], a["block_table"], a["local_len"],
                                         1 / 24, out=a["out"], lse=a["lse"])


def test_mla_well_formed_reaches_device_check():
    with pytest.raises(ValueError, match=DEVICE_MSG):
        _call_mla(_mla())
    with pytest.raises(ValueError, match=DEVICE_MSG):
        _call_mla(_mla(dt=torch.float8_e4m3fn))


@pytest.mark.parametrize("field,bad,msg", [
    ("q", torch.zeros(2, 16, 576), "expected torch.bfloat16"),
    ("kv_cache", torch.zeros(6, 64, 512, dtype=BF), "kv_cache has shape"),
    ("kv_cache", torch.zeros(6, 64, 576), "bf16 or fp8"),
    ("out", torch.zeros(2, 16, 576), "out has shape"),
    ("lse", torch.zeros(2, 16, dtype=BF), "lse has dtype"),
    ("local_len", torch.zeros(3, dtype=I32), "local_len has 3 elements"),
    ("block_table", torch.zeros(1, 3, dtype=I32), "needs 2 rows"),
])
def test_mla_mismatch_raises(field, bad, msg):
    a = _mla()
    a[field] = bad
    with pytest.raises(ValueError, match=msg):
        _call_mla(a)


def test_cache_write_gqa_shapes():
    T, Hkv, D, bs = 5, 2, 64, 16
    slot = torch.zeros(T, dtype=I64)
    k, v = torch.zeros(T, Hkv, D), torch.zeros(T, Hkv, D)
    kc, vc = torch.zeros(4, Hkv, bs, D), torch.zeros(4, Hkv, bs, D)
    with pytest.raises(ValueError, match=DEVICE_MSG):
        cp.cp_cache_write(slot, k, v, kc, vc, bs)
    # a block size larger than the cache's block dimension would write past it
    with pytest.raises(ValueError, match="k_cache has shape"):
        cp.cp_cache_write(slot, k, v, kc, vc, 32)
    with pytest.raises(ValueError, match="k_cache has shape"):
        cp.cp_cache_write(slot, k, v, torch.zeros(4, Hkv + 1, bs, D), vc, bs)
    with pytest.raises(ValueError, match="v_cache has shape"):
        cp.cp_cache_write(slot, k, v, kc, torch.zeros(3, Hkv, bs, D), bs)
    with pytest.raises(ValueError, match="k has shape"):
        cp.cp_cache_write(slot, k[:4], v, kc, vc, bs)
    with pytest.raises(ValueError, match="v has shape"):
        cp.cp_cache_write(slot, k, v[:, :1], kc, vc, bs)
    with pytest.raises(ValueError, match="both be given"):
        cp.cp_cache_write(slot, k, None, kc, vc, bs)


def test_cache_write_latent_shapes():
    T, Dk, bs = 3, 576, 64
    slot = torch.zeros(T, dtype=I64)
    lat = torch.zeros(T, Dk, dtype=BF)
    kc = torch.zeros(5, bs, Dk, dtype=BF)
    with pytest.raises(ValueError, match=DEVICE_MSG):
        cp.cp_cache_write(slot, lat, None, kc, None, bs)
    with pytest.raises(ValueError, match="k_cache has shape"):
        cp.cp_cache_write(slot, lat, None, kc, None, 128)
    with pytest.raises(ValueError, match="k_cache has dtype"):
        cp.cp_cache_write(slot, lat, None, kc.float(), None, bs)
    with pytest.raises(ValueError, match="k has shape"):
        cp.cp_cache_write(slot, lat[:, :512], None, kc, None, bs)


def test_slot_map_and_fused_write_shapes():
    T, Hkv, D, bs = 6, 2, 64, 16
    req, pos = torch.zeros(T, dtype=I32), torch.zeros(T, dtype=I32)
    bt = torch.zeros(2, 3, dtype=I32)
    k, v = torch.zeros(T, Hkv, D), torch.zeros(T, Hkv, D)
    kc, vc = torch.zeros(4, Hkv, bs, D), torch.zeros(4, Hkv, bs, D)
    with pytest.raises(ValueError, match=DEVICE_MSG):
        cp.cp_slot_map(req, pos, bt, 0, 2, 4, bs)
    with pytest.raises(ValueError, match="pos has 5 elements"):
        cp.cp_slot_map(req, pos[:5], bt, 0, 2, 4, bs)
    with pytest.raises(ValueError, match="out has 3 elements"):
        cp.cp_slot_map(req, pos, bt, 0, 2, 4, bs, out=torch.zeros(3, dtype=I64))
    with pytest.raises(ValueError, match="2-D int32"):
        cp.cp_slot_map(req, pos, bt[0], 0, 2, 4, bs)
    with pytest.raises(ValueError, match=DEVICE_MSG):
        cp.cp_slot_map_cache_write(req, pos, bt, 0, 2, 4, bs, k, v, kc, vc)
    with pytest.raises(ValueError, match="k_cache has shape"):
        cp.cp_slot_map_cache_write(req, pos, bt, 0, 2, 4, 8, k, v, kc, vc)
    with pytest.raises(ValueError, match="k has shape"):
        cp.cp_slot_map_cache_write(req, pos, bt, 0, 2, 4, bs, k[:2], v[:2], kc, vc)
    with pytest.raises(ValueError, match="slot_out has 2 elements"):
        cp.cp_slot_map_cache_write(req, pos, bt, 0, 2, 4, bs, k, v, kc, vc,
                                   slot_out=torch.zeros(2, dtype=I64))


def test_merge_and_exchange_output_shapes():
    po, pl = torch.zeros(3, 4, 8, 64), torch.zeros(3, 4, 8)
    with pytest.raises(ValueError, match=DEVICE_MSG):
        cp.cp_lse_merge(po, pl)
    with pytest.raises(ValueError, match="rows x Dv"):
        cp.cp_lse_merge(po, pl, out=torch.zeros(4, 8, 32))
    with pytest.raises(ValueError, match="lse_out has 16 elements"):
        cp.cp_lse_merge(po, pl, lse_out=torch.zeros(4, 4))
    with pytest.raises(ValueError, match="corrected has"):
        cp.cp_lse_correct(po[0], pl, 0, corrected=torch.zeros(4, 8, 32))
    with pytest.raises(ValueError, match="buf has shape"):
        cp.cp_a2a_pack(torch.zeros(2, 8, 64), torch.zeros(2, 8), 4, buf=torch.zeros(4, 2, 2, 64))


def test_prefill_shapes():
    C, Hq, Hkv, D, N = 64, 8, 2, 128, 2
    q = torch.zeros(C, Hq, D, dtype=BF)
    k, v = torch.zeros(C, Hkv, D, dtype=BF), torch.zeros(C, Hkv, D, dtype=BF)
    kc, vc = torch.zeros(6, Hkv, 16, D, dtype=BF), torch.zeros(6, Hkv, 16, D, dtype=BF)
    bt = torch.zeros(6, dtype=I32)
    with pytest.raises(ValueError, match=DEVICE_MSG):
        cp.pcp_prefill_attn_causal(q, 0, 0, N, 0.1, k=k, v=v)
    with pytest.raises(ValueError, match=DEVICE_MSG):
        cp.pcp_prefill_attn_causal(q, 100, 0, N, 0.1, k_cache=kc, v_cache=vc, block_table=bt,
                                   local_len=50)
    with pytest.raises(ValueError, match="k has shape"):
        cp.pcp_prefill_attn_causal(q, 0, 0, N, 0.1, k=k[:32], v=v[:32])
    with pytest.raises(ValueError, match="v_cache has shape"):
        cp.pcp_prefill_attn_causal(q, 0, 0, N, 0.1, k_cache=kc, v_cache=vc[:5], block_table=bt,
                                   local_len=50)
    with pytest.raises(ValueError, match="1-D int32"):
        cp.pcp_prefill_attn_causal(q, 0, 0, N, 0.1, k_cache=kc, v_cache=vc,
                                   block_table=bt.view(2, 3), local_len=50)
    with pytest.raises(ValueError, match="out has shape"):
        cp.pcp_prefill_attn_causal(q, 0, 0, N, 0.1, k=k, v=v, out=torch.zeros(2, 8, Hq, D))
    with pytest.raises(ValueError, match="either"):
        cp.pcp_prefill_attn_causal(q, 0, 0, N, 0.1)
    with pytest.raises(ValueError, match="multiple of 2 x pcp_size"):
        cp.pcp_prefill_attn_causal(q[:62], 0, 0, N, 0.1, k=k[:62], v=v[:62])


def test_kv_gather_shapes():
    N, B, W, Hkv, D, bs = 2, 2, 8, 2, 64, 16
    kcs = [torch.zeros(4, Hkv, bs, D) for _ in range(N)]
    bts = [torch.zeros(B, 2, dtype=I32) for _ in range(N)]
    seq = torch.zeros(B, dtype=I32)
    with pytest.raises(ValueError, match=DEVICE_MSG):
        cp.cp_kv_gather(kcs, None, bts, seq, N, 4, bs, 0, W)
    with pytest.raises(ValueError, match=r"k_caches\[1\] has shape"):
        cp.cp_kv_gather([kcs[0], torch.zeros(4, Hkv, 8, D)], None, bts, seq, N, 4, bs, 0, W)
    with pytest.raises(ValueError, match=r"k_caches\[0\] has shape"):
        cp.cp_kv_gather(kcs, None, bts, seq, N, 4, 32, 0, W)
    with pytest.raises(ValueError, match="same width"):
        cp.cp_kv_gather(kcs, None, [bts[0], torch.zeros(B, 3, dtype=I32)], seq, N, 4, bs, 0, W)
    with pytest.raises(ValueError, match="k_out has shape"):
        cp.cp_kv_gather(kcs, None, bts, seq, N, 4, bs, 0, W, k_out=torch.zeros(B, W - 1, Hkv, D))
