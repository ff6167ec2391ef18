#!/usr/bin/env python3
"""Benchmark of the context-parallel attention hot path on one MI355X.

Default workload: one DCP decode step of a GQA model, bf16, 32 requests with
contexts uniform in [4K, 32K], 32 query / 8 KV heads, head dim 128, KV sharded
over 8 simulated DCP ranks (interleave 16, block size 16).  One step =
  for every rank r: cp_slot_map + cp_cache_write of the step's new tokens,
  for every rank r: cp_decode_attn_partial_gqa over shard r,
  then cp_lse_merge of the 8 partials.
Inputs are synthetic (seeded), resident in HBM before timing starts.

Prints ONE JSON line: metric, value (KV GB/s over the whole step), roofline of
the dominant kernel (the shard decode partial; HIP events around each launch in
the timed region) and the fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "shard decode attn KV GB/s (% HBM peak); MLA/prefill TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def _cpu_cores() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit():
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
# GQA decode step
# ---------------------------------------------------------------------------

class GqaDecodeBench:
    def __init__(self, w, dev="cuda"):
        import numpy as np
        import torch

        import cp_inputs as ci
        import kv_context_parallelism_amd as cp

        self.w, self.dev, self.cp, self.torch = w, dev, cp, torch
        seq = ci.uniform_lengths(w.B, w.ctx[0], w.ctx[1], w.seed)
        self.seq = seq
        offs = np.concatenate([[0], np.cumsum(seq)]).astype(np.int64)
        total = int(offs[-1])
        self.q = ci.to_storage(ci.normal((w.B, w.Hq, w.D), w.seed + 1, dev), w.q_dtype)
        self.k = ci.to_storage(ci.normal((total, w.Hkv, w.D), w.seed + 2, dev), w.kv_dtype)
        self.v = ci.to_storage(ci.normal((total, w.Hkv, w.D), w.seed + 3, dev), w.kv_dtype)
        self.offs = offs
        seq_d = torch.from_numpy(seq).to(dev)
        # context written before the step: every position but each request's last
        req_ctx = torch.from_numpy(np.repeat(np.arange(w.B, dtype=np.int32), seq - 1)).to(dev)
        pos_ctx = torch.from_numpy(np.concatenate([np.arange(L - 1, dtype=np.int32)
                                                   for L in seq])).to(dev)
        keep = torch.ones(total, dtype=torch.bool, device=dev)
        keep[torch.from_numpy(offs[1:] - 1).to(dev)] = False
        k_ctx, v_ctx = self.k[keep].contiguous(), self.v[keep].contiguous()
        # the step's new tokens: position L_b - 1 of every request
        last = torch.from_numpy(offs[1:] - 1).to(dev)
        self.k_new = self.k[last].contiguous()
        self.v_new = self.v[last].contiguous()
        self.req_new = torch.arange(w.B, dtype=torch.int32, device=dev)
        self.pos_new = torch.from_numpy(seq - 1).to(dev)
        self.shards = []
        for r in range(w.N):
            ll_d = cp.cp_local_seq_lens(seq_d, r, w.N, w.I)
            ll = ll_d.cpu().numpy()
            bt, pool = ci.block_tables((ll.astype(np.int64) + w.bs - 1) // w.bs, w.seed + 100 + r,
                                       1.25)
            bt_d = torch.from_numpy(bt).to(dev)
            kc = torch.empty(pool, w.Hkv, w.bs, w.D, dtype=self.q.dtype, device=dev)
            vc = torch.empty_like(kc)
            ci.nan_fill_(kc, w.kv_dtype)
            ci.nan_fill_(vc, w.kv_dtype)
            slots = cp.cp_slot_map(req_ctx, pos_ctx, bt_d, r, w.N, w.I, w.bs)
            cp.cp_cache_write(slots, k_ctx, v_ctx, kc, vc, w.bs)
            out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
            lse = torch.empty(w.B, w.Hq, dtype=torch.float32, device=dev)
            args = cp.gqa_args(self.q, kc, vc, bt_d, ll_d, w.scale, out, lse)
            ws = torch.empty(max(cp.cp_workspace_bytes(cp.CP_OP_DECODE_GQA, args), 16),
                             dtype=torch.uint8, device=dev)
            self.shards.append(dict(ll=ll, ll_d=ll_d, bt_d=bt_d, kc=kc, vc=vc, ws=ws,
                                    slots=torch.empty(w.B, dtype=torch.int64, device=dev)))
        del k_ctx, v_ctx, req_ctx, pos_ctx, keep
        self.part_out = torch.empty(w.N, w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
        self.part_lse = torch.empty(w.N, w.B, w.Hq, dtype=torch.float32, device=dev)
        self.out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
        self.lse = torch.empty(w.B, w.Hq, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        kv_tok = w.Hkv * w.D * self.q.element_size() * 2
        self.kv_bytes_step = int(seq.sum()) * kv_tok
        self.per_launch_bytes = []  # algorithmic bytes of each shard partial
        for sh in self.shards:
            self.per_launch_bytes.append(int(sh["ll"].sum()) * kv_tok
                                         + self.q.numel() * self.q.element_size()
                                         + w.B * w.Hq * (w.D + 1) * 4)
        self.events = None

    def step(self, ev=None):
        cp, w = self.cp, self.w
        for r, sh in enumerate(self.shards):
            cp.cp_slot_map(self.req_new, self.pos_new, sh["bt_d"], r, w.N, w.I, w.bs,
                           out=sh["slots"])
            cp.cp_cache_write(sh["slots"], self.k_new, self.v_new, sh["kc"], sh["vc"], w.bs)
        for r, sh in enumerate(self.shards):
            if ev is not None:
                ev[r][0].record()
            cp.cp_decode_attn_partial_gqa(self.q, sh["kc"], sh["vc"], sh["bt_d"], sh["ll_d"],
                                          w.scale, out=self.part_out[r], lse=self.part_lse[r],
                                          workspace=sh["ws"])
            if ev is not None:
                ev[r][1].record()
        cp.cp_lse_merge(self.part_out, self.part_lse, out=self.out, lse_out=self.lse)

    def cpu_baseline(self, budget_s=15.0):
        """The fp64 oracle on the same workload: all shard partials of whole
        requests plus their merge, request by request until the time budget is
        spent.  Returns (KV GB/s, sample description)."""
        import numpy as np

        import cp_inputs as ci
        import oracle

        w = self.w
        done, kv_bytes, t0 = 0, 0, time.perf_counter()
        q = ci.bits(self.q.cpu())
        for b in range(w.B):
            lo, hi = int(self.offs[b]), int(self.offs[b + 1])
            k = ci.bits(self.k[lo:hi].cpu())
            v = ci.bits(self.v[lo:hi].cpu())
            po, pl = [], []
            for r in range(w.N):
                o, l = oracle.attention(q[b:b + 1], k, v, key_begin=0, key_end=hi - lo,
                                        scale=w.scale, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                                        shard=(w.N, w.I, r))
                po.append(o[0])
                pl.append(l[0])
            oracle.lse_merge(np.stack(po), np.stack(pl))
            done += 1
            kv_bytes += (hi - lo) * w.Hkv * w.D * 2 * 2
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return kv_bytes / dt / 1e9, f"{done} of {w.B} requests (all {w.N} shard partials + merge)"

    def config(self):
        w = self.w
        return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                "head_dim": w.D, "context": f"uniform[{w.ctx[0]},{w.ctx[1]}]",
                "total_context_tokens": int(self.seq.sum()), "dcp_shards": w.N,
                "interleave": w.I, "block_size": w.bs}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_decode_bf16", choices=["gqa_decode_bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the N shards are simulated as separate buffers on a "
              "single MI355X, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import cp_inputs as ci

    torch.cuda.set_device(0)
    w = ci.WORKLOADS[args.workload]
    print(f"[bench] setting up {w.name}", file=sys.stderr, flush=True)
    bench = GqaDecodeBench(w)
    for _ in range(args.warmup):
        bench.step()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(w.N)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        bench.step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    launch_ms = [e[0].elapsed_time(e[1]) for step in ev for e in step]
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    avg_bytes = sum(bench.per_launch_bytes) / len(bench.per_launch_bytes)
    achieved = avg_bytes / avg_launch_s / 1e9
    value = bench.kv_bytes_step / (ms_step / 1e3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": bench.config(),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "cp_decode_attn_partial_gqa (attention + split combine)",
                     "avg_launch_us": round(avg_launch_s * 1e6, 2),
                     "algorithmic_bytes_per_launch": int(avg_bytes)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a bounded sample", file=sys.stderr, flush=True)
        v, sample = bench.cpu_baseline()
        line["cpu_baseline"] = {"value": round(v, 4), "unit": "GB/s", "cores": _cpu_cores(),
                                "kind": "oracle", "sample": sample}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
