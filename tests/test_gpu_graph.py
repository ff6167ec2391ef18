"""GPU: a decode step (every shard's partial, then the merge) captured as a
HIP graph replays to the eager step's exact bytes -- three replays, each after
an eager step and a synchronisation, with every output poisoned before the
replay.  (bench.py times its step rate by replaying its whole step -- slot map
and cache write, every shard's partial, the merge -- as one graph, and checks
the last replay against the eager step.)"""
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

    announce(f"graph capture of a {name} step")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (po, pl, out, lse)]
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
        for a, b in zip(ref, (po, pl, out, lse)):
            assert torch.equal(_bytes(a), _bytes(b)), "eager steps differ"
        for t in (po, pl, out, lse):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"{name} graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (po, pl, out, lse)):
            assert torch.equal(_bytes(a), _bytes(b)), f"replay {rep} differs from the eager step"
