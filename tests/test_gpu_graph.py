"""GPU: a step (every shard's partial, then the merge) captured as a HIP graph
replays to the eager step's exact bytes -- three replays, each after an eager
step and a synchronisation, with every output poisoned before the replay.
Decode steps (GQA, MLA bf16, MLA fp8), a multi-token decode step whose entry
runs two launches per shard, and a PCP prefill step (one rank's causal part,
its prefix-shard partials and their merge).  (bench.py times its step rate by
replaying its whole step as one graph, and checks the last replay against the
eager step.)"""
import pytest
import torch

import cp_inputs as ci
import kv_context_parallelism_amd as cp
from _cases import announce, build_decode_case, run_partials

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("name", ["gqa_decode_bf16", "mla_decode_bf16", "mla_decode_fp8"])
def test_decode_step_graph_replays_match_eager(name):
    w = ci.scaled(ci.WORKLOADS[name], B=3, seed=4200)
    case = build_decode_case(w, seq=[700, 1, 2500], check_cache=False, check_slots=False)
    mla = w.kind == "mla_decode"
    po, pl = run_partials(case)
    out = torch.empty(po.shape[1:], dtype=torch.float32, device="cuda")
    lse = torch.empty(pl.shape[1:], dtype=torch.float32, device="cuda")

    def step():
        for r, sh in enumerate(case.shards):
            if mla:
                cp.cp_decode_attn_partial_mla(case.q, sh["kc"], sh["bt_dev"], sh["ll_dev"], w.scale,
                                              Dv=w.Dv, kv_scale=case.kv_scale, out=po[r], lse=pl[r])
            else:
                cp.cp_decode_attn_partial_gqa(case.q, sh["kc"], sh["vc"], sh["bt_dev"],
                                              sh["ll_dev"], w.scale, out=po[r], lse=pl[r])
        cp.cp_lse_merge(po, pl, out=out, lse_out=lse)

    _replays_match(step, (po, pl, out, lse), name)


def _replays_match(step, outs, name):
    announce(f"graph capture of a {name} step")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        step()  # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(_bytes(a), _bytes(b)), "eager steps differ"
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"{name} graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(_bytes(a), _bytes(b)), f"replay {rep} differs from the eager step"


def test_mtp_step_graph_replays_match_eager():
    """Four query tokens x group 4 = 16 rows per KV head: two launches (and two
    split combines) per shard call, captured and replayed."""
    w = ci.scaled(ci.WORKLOADS["gqa_decode_bf16"], B=3, seed=4300)
    T = 4
    case = build_decode_case(w, seq=[700, 4, 2500], check_cache=False, check_slots=False)
    q = ci.to_storage(ci.normal((w.B, T, w.Hq, w.D), 4301, "cuda", w.q_std), w.q_dtype)
    seq_dev = torch.from_numpy(case.seq).to("cuda")
    po = torch.empty(w.N, w.B, T, w.Hq, w.D, dtype=torch.float32, device="cuda")
    pl = torch.empty(w.N, w.B, T, w.Hq, dtype=torch.float32, device="cuda")
    out = torch.empty(w.B * T * w.Hq, w.D, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.B * T * w.Hq, dtype=torch.float32, device="cuda")

    def step():
        for r, sh in enumerate(case.shards):
            cp.cp_decode_attn_partial_gqa_mtp(q, sh["kc"], sh["vc"], sh["bt_dev"], sh["ll_dev"],
                                              seq_dev, w.scale, r, w.N, w.I, out=po[r], lse=pl[r])
        cp.cp_lse_merge(po.view(w.N, -1, w.D), pl.view(w.N, -1), out=out, lse_out=lse)

    _replays_match(step, (po, pl, out, lse), "multi-token decode")


def test_prefill_step_graph_replays_match_eager():
    """PCP rank 1 of 2: the causal call, three prefix-shard calls and the merge
    of the four partials."""
    from test_gpu_prefill import _setup
    C, P, N, Hq, Hkv, N_dcp = 256, 200, 2, 32, 8, 3
    q, k, v, prefix, scale = _setup(C, P, N, Hq, Hkv, N_dcp, 16, 16, 4400)
    c = C // (2 * N)
    po = torch.empty(1 + N_dcp, 2, c, Hq, 128, dtype=torch.float32, device="cuda")
    pl = torch.empty(1 + N_dcp, 2, c, Hq, dtype=torch.float32, device="cuda")
    out = torch.empty(2 * c * Hq, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(2 * c * Hq, dtype=torch.float32, device="cuda")
    Pk = prefix.k.shape[0]

    def step():
        cp.pcp_prefill_attn_causal(q, Pk, 1, N, scale, k=k, v=v, out=po[0], lse=pl[0])
        for s, sh in enumerate(prefix.shards):
            cp.pcp_prefill_attn_causal(q, Pk, 1, N, scale, k_cache=sh["kc"], v_cache=sh["vc"],
                                       block_table=sh["bt_dev"][0].contiguous(),
                                       local_len=int(sh["ll"][0]), out=po[1 + s], lse=pl[1 + s])
        cp.cp_lse_merge(po.view(1 + N_dcp, -1, 128), pl.view(1 + N_dcp, -1), out=out, lse_out=lse)

    _replays_match(step, (po, pl, out, lse), "PCP prefill")
