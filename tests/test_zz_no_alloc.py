"""GPU check of the allocation-free GQA decode entry: through the C ABI it must
give exactly the bytes of cp_decode_attn_partial_gqa with a workspace, on two
calls in a row (the second with a smaller input, so the shared scratch holds
the first call's partials when it starts), and reject a call whose split
partials do not fit the scratch."""
import ctypes

import pytest
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
from _cases import announce, build_decode_case, gate_f32, gate_lowp, oracle_request

pytestmark = pytest.mark.gpu


def _both(case, shard, B=None):
    """(workspace entry, no-alloc entry) outputs for shard `shard`, first B requests."""
    w = case.w
    sh = case.shards[shard]
    B = w.B if B is None else B
    q = case.q[:B].contiguous()
    bt, ll = sh["bt_dev"][:B].contiguous(), sh["ll_dev"][:B].contiguous()
    ref = cp.cp_decode_attn_partial_gqa(q, sh["kc"], sh["vc"], bt, ll, w.scale)
    out = torch.full((B, w.Hq, w.D), float("nan"), device="cuda")
    lse = torch.full((B, w.Hq), float("nan"), device="cuda")
    a = cp.gqa_args(q, sh["kc"], sh["vc"], bt, ll, w.scale, out, lse)
    st = cp._lib.load().cp_decode_attn_partial_gqa_noalloc(ctypes.byref(a), cp._stream())
    assert st == cp.CP_OK, cp._lib.load().cp_last_error()
    torch.cuda.synchronize()
    return ref, (out, lse)


@pytest.mark.parametrize("name", ["gqa_decode_bf16", "gqa_tiny_f32"])
def test_noalloc_matches_workspace_entry_twice(name):
    base = ci.WORKLOADS[name]
    if name == "gqa_decode_bf16":
        w = ci.scaled(base, B=12, seed=7100)
        seq = [4096, 32768, 17, 9000, 0, 20000, 30001, 5000, 12345, 64, 8192, 27000]
    else:
        w = ci.scaled(base, B=5, seed=7200)
        seq = [1000, 3, 2500, 0, 777]
    announce(f"no-alloc entry {name} B={w.B}")
    case = build_decode_case(w, seq=seq, check_cache=False)
    for B in (w.B, 3):  # the second call is smaller: the scratch keeps the first call's data
        (ro, rl), (o, l) = _both(case, shard=1, B=B)
        assert torch.equal(ro, o) and torch.equal(rl, l), f"B={B}: differs from the workspace entry"
        # and both are the oracle's result for one request of the call
        b = 1 if B > 1 else 0
        xo, xl = oracle_request(case, b, shard=(w.N, w.I, 1))
        if w.kv_dtype == "bf16":
            gate_lowp(o[b].cpu().numpy(), xo, f"no-alloc out b{b}", 2e-2)
            gate_lowp(l[b].cpu().numpy(), xl, f"no-alloc lse b{b}", 1e-3, norm=None)
        else:
            gate_f32(o[b].cpu().numpy(), xo, f"no-alloc out b{b}")
            gate_f32(l[b].cpu().numpy(), xl, f"no-alloc lse b{b}")


def test_noalloc_rejects_calls_beyond_the_scratch():
    lib = cp._lib.load()
    cap = lib.cp_noalloc_scratch_bytes()
    assert cap == 16 << 20
    B, Hq, Hkv, D = 8192, 32, 8, 128   # 65,536 (request, KV head) pairs of split partials
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(1, Hkv, 16, D, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    ll = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    a = cp.gqa_args(q, kc, kc, bt, ll, 0.1, out, lse)
    assert cp.cp_workspace_bytes(cp.CP_OP_DECODE_GQA, a) > cap
    st = lib.cp_decode_attn_partial_gqa_noalloc(ctypes.byref(a), cp._stream())
    assert st == cp.CP_E_WORKSPACE and b"scratch" in lib.cp_last_error()
