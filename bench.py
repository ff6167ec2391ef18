#!/usr/bin/env python3
"""Benchmark of the context-parallel attention hot path on one MI355X.

Default workload (--workload gqa_decode_bf16): one DCP decode step of a GQA
model, bf16, 32 requests with contexts uniform in [4K, 32K], 32 query / 8 KV
heads, head dim 128, KV sharded over 8 simulated DCP ranks (interleave 16,
block size 16).  One step =
  for every rank r: the slot map and cache write of the step's new tokens
                   (cp_slot_map_cache_write: both in one launch),
  for every rank r: cp_decode_attn_partial_gqa over shard r,
  then cp_lse_merge of the 8 partials.
value = KV bytes the step reads / step time (GB/s).

Other workloads, same step structure:
  mla_decode_bf16   absorbed MLA, 64 requests x 64K context, 128 heads, latent
                    576 / value 512, 8 shards (interleave 1, block 64)
  mla_decode_fp8    the same with an fp8 E4M3 latent cache, 4 requests x 1M
  pcp_prefill_bf16  a 32K chunk over a 64K prefix in 8 DCP shards; per PCP rank
                    the causal call over the chunk, one call per prefix shard
                    and the merge; the chunk's K/V is first written to the shards
value = algorithmic FLOP (unmasked score + PV products) / step time (TFLOP/s).
  dcp_prefill_bf16     the same chunk with its K/V interleaved into the 8 DCP
                       shards: per PCP rank one causal call per shard + merge
  gqa_decode_mtp_bf16  the GQA step with 2 query tokens per request
  kv_gather_bf16       every request's 64K-token window gathered from the 8
                       shard caches into token order
  head_scatter_mla     16 layers of the head-scattered output exchange
                       (correct, pack, packed merge) of an MLA step
(GB/s for the last three.)

Inputs are synthetic (seeded), resident in HBM before timing starts.  Prints
ONE JSON line: metric, value, the roofline of the dominant kernel (HIP events
around its launches in the timed region, on the stream it runs on), the step
rate from a HIP-graph replay, and the fp64 CPU oracle timed on a bounded
sample of the same workload.  The default run adds a `workloads` block with
the small fp32 latency case and every other workload above.
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


def _counted_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy of known
    size), or None when there is none or the kernel's sources have changed
    since the counters were taken."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    m_f = re.search(r"^kernel_sources: (.+)$", text, re.M)
    m_h = re.search(r"^kernel_sources_sha256_16: ([0-9a-f]+)$", text, re.M)
    if not (m_t and m_f and m_h):
        return None
    h = hashlib.sha256()
    for f in sorted(m_f.group(1).split()):
        h.update(f.encode())
        with open(os.path.join(ROOT, "kv_context_parallelism_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return int(m_t.group(1)) if h.hexdigest()[:16] == m_h.group(1) else None


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
    metric_unit = "GB/s"

    def __init__(self, w, dev="cuda"):
        import numpy as np
        import torch

        import cp_inputs as ci
        import kv_context_parallelism_amd as cp

        self.w, self.dev, self.cp, self.torch = w, dev, cp, torch
        T = self.T = w.q_len  # query tokens per request: its last T positions
        seq = ci.uniform_lengths(w.B, w.ctx[0], w.ctx[1], w.seed)
        self.seq = seq
        offs = np.concatenate([[0], np.cumsum(seq)]).astype(np.int64)
        total = int(offs[-1])
        qshape = (w.B, w.Hq, w.D) if T == 1 else (w.B, T, w.Hq, w.D)
        self.q = ci.to_storage(ci.normal(qshape, w.seed + 1, dev), w.q_dtype)
        self.k = ci.to_storage(ci.normal((total, w.Hkv, w.D), w.seed + 2, dev), w.kv_dtype)
        self.v = ci.to_storage(ci.normal((total, w.Hkv, w.D), w.seed + 3, dev), w.kv_dtype)
        self.offs = offs
        seq_d = torch.from_numpy(seq).to(dev)
        self.seq_d = seq_d
        # context written before the step: every position but each request's last T
        req_ctx = torch.from_numpy(np.repeat(np.arange(w.B, dtype=np.int32), seq - T)).to(dev)
        pos_ctx = torch.from_numpy(np.concatenate([np.arange(L - T, dtype=np.int32)
                                                   for L in seq])).to(dev)
        new_rows = (offs[1:, None] - T + np.arange(T)[None, :]).reshape(-1)
        keep = torch.ones(total, dtype=torch.bool, device=dev)
        keep[torch.from_numpy(new_rows).to(dev)] = False
        k_ctx, v_ctx = self.k[keep].contiguous(), self.v[keep].contiguous()
        # the step's new tokens: positions L_b - T .. L_b - 1 of every request
        last = torch.from_numpy(new_rows).to(dev)
        self.k_new = self.k[last].contiguous()
        self.v_new = self.v[last].contiguous()
        self.req_new = torch.from_numpy(np.repeat(np.arange(w.B, dtype=np.int32), T)).to(dev)
        self.pos_new = torch.from_numpy((seq[:, None] - T + np.arange(T)[None, :])
                                        .reshape(-1).astype(np.int32)).to(dev)
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
            out = torch.empty(qshape, dtype=torch.float32, device=dev)
            lse = torch.empty(qshape[:-1], dtype=torch.float32, device=dev)
            if T == 1:
                args, op = cp.gqa_args(self.q, kc, vc, bt_d, ll_d, w.scale, out, lse), \
                    cp.CP_OP_DECODE_GQA
            else:
                args = cp.gqa_mtp_args(self.q, kc, vc, bt_d, ll_d, seq_d, w.scale, out, lse, r,
                                       w.N, w.I)
                op = cp.CP_OP_DECODE_GQA_MTP
            ws = torch.empty(max(cp.cp_workspace_bytes(op, args), 16), dtype=torch.uint8,
                             device=dev)
            self.shards.append(dict(ll=ll, ll_d=ll_d, bt_d=bt_d, kc=kc, vc=vc, ws=ws,
                                    slots=torch.empty(w.B * T, dtype=torch.int64, device=dev)))
        del k_ctx, v_ctx, req_ctx, pos_ctx, keep
        self.part_out = torch.empty((w.N,) + qshape, dtype=torch.float32, device=dev)
        self.part_lse = torch.empty((w.N,) + qshape[:-1], dtype=torch.float32, device=dev)
        self.out = torch.empty(qshape, dtype=torch.float32, device=dev)
        self.lse = torch.empty(qshape[:-1], dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        kv_tok = w.Hkv * w.D * self.q.element_size() * 2
        self.kv_bytes_step = int(seq.sum()) * kv_tok
        self.per_launch_bytes = []  # algorithmic bytes of each shard partial
        for sh in self.shards:
            self.per_launch_bytes.append(int(sh["ll"].sum()) * kv_tok
                                         + self.q.numel() * self.q.element_size()
                                         + w.B * T * w.Hq * (w.D + 1) * 4)
        self.work_step = self.kv_bytes_step
        self.tokens_step = w.B * T  # query tokens decoded per step (one layer, all shards)
        self.per_launch_work = self.per_launch_bytes
        # one event pair around the N shard calls back to back, one around the merge
        self.launches_per_step = 2
        self.launches_per_event = w.N
        self.dominant = [0]
        self.merge_idx = 1
        self.merge_bytes = (w.N + 1) * w.B * T * w.Hq * (w.D + 1) * 4
        self.kernel_name = ("cp_decode_attn_partial_gqa (attention + split combine)" if T == 1 else
                            f"cp_decode_attn_partial_gqa_mtp ({T} query tokens; attention + split "
                            "combine)")
        self.dtype = w.kv_dtype

    def step(self, ev=None):
        cp, w = self.cp, self.w
        for r, sh in enumerate(self.shards):
            cp.cp_slot_map_cache_write(self.req_new, self.pos_new, sh["bt_d"], r, w.N, w.I, w.bs,
                                       self.k_new, self.v_new, sh["kc"], sh["vc"],
                                       slot_out=sh["slots"])
        if ev is not None:
            ev[0][0].record()
        for r, sh in enumerate(self.shards):
            if self.T == 1:
                cp.cp_decode_attn_partial_gqa(self.q, sh["kc"], sh["vc"], sh["bt_d"], sh["ll_d"],
                                              w.scale, out=self.part_out[r], lse=self.part_lse[r],
                                              workspace=sh["ws"])
            else:
                cp.cp_decode_attn_partial_gqa_mtp(self.q, sh["kc"], sh["vc"], sh["bt_d"],
                                                  sh["ll_d"], self.seq_d, w.scale, r, w.N, w.I,
                                                  out=self.part_out[r], lse=self.part_lse[r],
                                                  workspace=sh["ws"])
        if ev is not None:
            ev[0][1].record()
            ev[1][0].record()
        cp.cp_lse_merge(self.part_out, self.part_lse, out=self.out, lse_out=self.lse)
        if ev is not None:
            ev[1][1].record()

    def cpu_baseline(self, budget_s=15.0, min_s=1.0):
        """The fp64 oracle on the same workload: all shard partials of whole
        requests plus their merge, request after request (cycling through the
        batch again while less than ``min_s`` has passed) until the time budget
        is spent.  Returns (KV GB/s, sample description)."""
        import numpy as np

        import cp_inputs as ci
        import oracle

        w = self.w
        done, kv_bytes, passes, t0 = 0, 0, 0, time.perf_counter()
        q = ci.bits(self.q.cpu())
        host = {}
        over = False
        while not over:
            for b in range(w.B):
                lo, hi = int(self.offs[b]), int(self.offs[b + 1])
                if b not in host:
                    host[b] = (ci.bits(self.k[lo:hi].cpu()), ci.bits(self.v[lo:hi].cpu()))
                k, v = host[b]
                po, pl = [], []
                for r in range(w.N):
                    if self.T == 1:
                        o, l = oracle.attention(q[b:b + 1], k, v, key_begin=0, key_end=hi - lo,
                                                scale=w.scale, q_dtype=w.q_dtype,
                                                kv_dtype=w.kv_dtype, shard=(w.N, w.I, r))
                    else:
                        o, l = oracle.decode_mtp(q[b], k, v, L=hi - lo, scale=w.scale,
                                                 q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                                                 shard=(w.N, w.I, r))
                    po.append(o.reshape(-1, w.D))
                    pl.append(l.reshape(-1))
                oracle.lse_merge(np.stack(po), np.stack(pl))
                done += 1
                kv_bytes += (hi - lo) * w.Hkv * w.D * self.q.element_size() * 2
                if time.perf_counter() - t0 > budget_s:
                    over = True
                    break
            else:
                passes += 1
                over = over or time.perf_counter() - t0 >= min_s
        dt = time.perf_counter() - t0
        self.cpu_step_s = dt / done * w.B  # one whole step of the batch
        return kv_bytes / dt / 1e9, (f"{done} request partial sets ({passes} whole passes over "
                                     f"the {w.B} requests; each: all {w.N} shard partials + "
                                     "merge)")

    def config(self):
        w = self.w
        return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                "head_dim": w.D, "context": f"uniform[{w.ctx[0]},{w.ctx[1]}]",
                "total_context_tokens": int(self.seq.sum()), "dcp_shards": w.N,
                "interleave": w.I, "block_size": w.bs, "query_tokens": self.T}



# ---------------------------------------------------------------------------
# MLA decode step (absorbed latent, bf16 or fp8 E4M3 cache)
# ---------------------------------------------------------------------------

class MlaDecodeBench:
    metric_unit = "TFLOP/s"

    def __init__(self, w, dev="cuda"):
        import numpy as np
        import torch

        import cp_inputs as ci
        import kv_context_parallelism_amd as cp

        self.w, self.cp = w, cp
        seq = np.full(w.B, w.ctx[0], dtype=np.int32)
        self.seq = seq
        total = int(seq.sum())
        self.q = ci.to_storage(ci.normal((w.B, w.Hq, w.D), w.seed + 1, dev, w.q_std), w.q_dtype)
        lat = ci.normal((total, w.D), w.seed + 2, dev, w.kv_std)
        if w.kv_dtype == "fp8_e4m3fn":
            self.lat, self.kv_scale = ci.fp8_quantize(lat)
        else:
            self.lat, self.kv_scale = ci.to_storage(lat, w.kv_dtype), 1.0
        del lat
        offs = np.concatenate([[0], np.cumsum(seq)]).astype(np.int64)
        self.offs = offs
        seq_d = torch.from_numpy(seq).to(dev)
        req_ctx = torch.from_numpy(np.repeat(np.arange(w.B, dtype=np.int32), seq - 1)).to(dev)
        pos_ctx = torch.arange(int(seq[0]) - 1, dtype=torch.int32, device=dev).repeat(w.B)
        keep = torch.ones(total, dtype=torch.bool, device=dev)
        last = torch.from_numpy(offs[1:] - 1).to(dev)
        keep[last] = False
        lat_ctx = self.lat[keep].contiguous()
        self.lat_new = self.lat[last].contiguous()
        self.req_new = torch.arange(w.B, dtype=torch.int32, device=dev)
        self.pos_new = torch.from_numpy(seq - 1).to(dev)
        self.shards = []
        for r in range(w.N):
            ll_d = cp.cp_local_seq_lens(seq_d, r, w.N, w.I)
            ll = ll_d.cpu().numpy()
            bt, pool = ci.block_tables((ll.astype(np.int64) + w.bs - 1) // w.bs, w.seed + 100 + r,
                                       1.25)
            bt_d = torch.from_numpy(bt).to(dev)
            kc = torch.empty(pool, w.bs, w.D, dtype=self.lat.dtype, device=dev)
            ci.nan_fill_(kc, w.kv_dtype)
            slots = cp.cp_slot_map(req_ctx, pos_ctx, bt_d, r, w.N, w.I, w.bs)
            cp.cp_cache_write(slots, lat_ctx, None, kc, None, w.bs)
            out = torch.empty(w.B, w.Hq, w.Dv, dtype=torch.float32, device=dev)
            lse = torch.empty(w.B, w.Hq, dtype=torch.float32, device=dev)
            args = cp.mla_args(self.q, kc, bt_d, ll_d, w.scale, out, lse, Dv=w.Dv,
                               kv_scale=self.kv_scale)
            ws = torch.empty(cp.cp_workspace_bytes(cp.CP_OP_DECODE_MLA, args), dtype=torch.uint8,
                             device=dev)
            self.shards.append(dict(ll=ll, ll_d=ll_d, bt_d=bt_d, kc=kc, ws=ws,
                                    slots=torch.empty(w.B, dtype=torch.int64, device=dev)))
            del slots
        del lat_ctx, req_ctx, pos_ctx, keep
        self.part_out = torch.empty(w.N, w.B, w.Hq, w.Dv, dtype=torch.float32, device=dev)
        self.part_lse = torch.empty(w.N, w.B, w.Hq, dtype=torch.float32, device=dev)
        self.out = torch.empty(w.B, w.Hq, w.Dv, dtype=torch.float32, device=dev)
        self.lse = torch.empty(w.B, w.Hq, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        flop_tok = w.Hq * (w.D + w.Dv) * 2
        self.work_step = int(seq.sum()) * flop_tok
        self.tokens_step = w.B  # decode tokens per step (one layer, all shards)
        self.per_launch_work = [int(sh["ll"].sum()) * flop_tok for sh in self.shards]
        eb = self.lat.element_size()
        self.per_launch_bytes = [int(sh["ll"].sum()) * w.D * eb + self.q.numel() * 2
                                 + w.B * w.Hq * (w.Dv + 1) * 4 for sh in self.shards]
        # one event pair around the N shard calls back to back, one around the merge
        self.launches_per_step = 2
        self.launches_per_event = w.N
        self.dominant = [0]
        self.merge_idx = 1
        self.merge_bytes = (w.N + 1) * w.B * w.Hq * (w.Dv + 1) * 4
        self.kernel_name = "cp_decode_attn_partial_mla (attention + split combine)"
        self.dtype = "bf16"

    def step(self, ev=None):
        cp, w = self.cp, self.w
        for r, sh in enumerate(self.shards):
            cp.cp_slot_map_cache_write(self.req_new, self.pos_new, sh["bt_d"], r, w.N, w.I, w.bs,
                                       self.lat_new, None, sh["kc"], None, slot_out=sh["slots"])
        if ev is not None:
            ev[0][0].record()
        for r, sh in enumerate(self.shards):
            cp.cp_decode_attn_partial_mla(self.q, sh["kc"], sh["bt_d"], sh["ll_d"], w.scale,
                                          Dv=w.Dv, kv_scale=self.kv_scale, out=self.part_out[r],
                                          lse=self.part_lse[r], workspace=sh["ws"])
        if ev is not None:
            ev[0][1].record()
            ev[1][0].record()
        cp.cp_lse_merge(self.part_out, self.part_lse, out=self.out, lse_out=self.lse)
        if ev is not None:
            ev[1][1].record()

    def cpu_baseline(self, budget_s=15.0):
        """The fp64 oracle on the same workload: shard partials of request 0,
        sixteen heads at a time, shard after shard, until the budget is spent."""
        import cp_inputs as ci
        import oracle

        w = self.w
        L = int(self.seq[0])
        lat = ci.bits(self.lat[:L].cpu()).reshape(L, 1, w.D)
        q = ci.bits(self.q[:1].cpu())
        work, parts, t0 = 0, 0, time.perf_counter()
        for r in range(w.N):
            n_own = int(self.shards[r]["ll"][0])
            for h0 in range(0, w.Hq, 16):
                oracle.attention(q, lat, lat, key_begin=0, key_end=L, Dv=w.Dv, scale=w.scale,
                                 q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, kv_scale=self.kv_scale,
                                 shard=(w.N, w.I, r), heads=list(range(h0, h0 + 16)))
                work += n_own * 16 * (w.D + w.Dv) * 2
                parts += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return work / dt / 1e12, (f"request 0: {parts} shard-partial x 16-head blocks "
                                  f"({parts * 16} of {w.N * w.Hq} shard-heads)")

    def config(self):
        w = self.w
        return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "latent": w.D,
                "value_dim": w.Dv, "context": int(self.seq[0]), "kv_dtype": w.kv_dtype,
                "dcp_shards": w.N, "interleave": w.I, "block_size": w.bs}


# ---------------------------------------------------------------------------
# PCP prefill step: every rank's causal part + its prefix partials + merge
# ---------------------------------------------------------------------------

class PrefillBench:
    metric_unit = "TFLOP/s"

    def __init__(self, w, dev="cuda"):
        import numpy as np
        import torch

        import cp_inputs as ci
        import kv_context_parallelism_amd as cp

        self.w, self.cp = w, cp
        C, P = w.C, w.P
        self.q = ci.to_storage(ci.normal((C, w.Hq, w.D), w.seed + 1, dev), "bf16")
        self.k = ci.to_storage(ci.normal((C, w.Hkv, w.D), w.seed + 2, dev), "bf16")
        self.v = ci.to_storage(ci.normal((C, w.Hkv, w.D), w.seed + 3, dev), "bf16")
        pk = ci.to_storage(ci.normal((P, w.Hkv, w.D), w.seed + 52, dev), "bf16")
        pv = ci.to_storage(ci.normal((P, w.Hkv, w.D), w.seed + 53, dev), "bf16")
        self.pk, self.pv = pk, pv
        tot = torch.tensor([P + C], dtype=torch.int32, device=dev)
        pre = torch.tensor([P], dtype=torch.int32, device=dev)
        req_p = torch.zeros(P, dtype=torch.int32, device=dev)
        pos_p = torch.arange(P, dtype=torch.int32, device=dev)
        self.req_c = torch.zeros(C, dtype=torch.int32, device=dev)
        self.pos_c = torch.arange(P, P + C, dtype=torch.int32, device=dev)
        self.shards = []
        for s in range(w.N):
            cap = cp.cp_local_seq_lens(tot, s, w.N, w.I).cpu().numpy()
            ll = int(cp.cp_local_seq_lens(pre, s, w.N, w.I).cpu()[0])
            bt, pool = ci.block_tables((cap.astype(np.int64) + w.bs - 1) // w.bs, w.seed + 100 + s,
                                       1.25)
            bt_d = torch.from_numpy(bt).to(dev)
            kc = ci.nan_fill_(torch.empty(pool, w.Hkv, w.bs, w.D, dtype=torch.bfloat16,
                                          device=dev), "bf16")
            vc = ci.nan_fill_(torch.empty_like(kc), "bf16")
            slots = cp.cp_slot_map(req_p, pos_p, bt_d, s, w.N, w.I, w.bs)
            cp.cp_cache_write(slots, pk, pv, kc, vc, w.bs)
            self.shards.append(dict(ll=ll, bt_d=bt_d, bt_row=bt_d[0].contiguous(), kc=kc, vc=vc,
                                    slots=torch.empty(C, dtype=torch.int64, device=dev)))
        c = C // (2 * w.N)
        # per rank: the two pieces [2][c] of its causal-chunk and prefix-shard partials
        self.part_out = torch.empty(w.N + 1, 2, c, w.Hq, w.D, dtype=torch.float32, device=dev)
        self.part_lse = torch.empty(w.N + 1, 2, c, w.Hq, dtype=torch.float32, device=dev)
        self.out = torch.empty(w.N, 2, c, w.Hq, w.D, dtype=torch.float32, device=dev)
        self.lse = torch.empty(w.N, 2, c, w.Hq, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        causal = C * (C + 1) // 2
        self.work_causal = causal * w.Hq * 4 * w.D
        self.work_prefix = C * P * w.Hq * 4 * w.D
        self.work_step = self.work_causal + self.work_prefix
        self.tokens_step = w.C  # prefill tokens per step (one layer, all PCP ranks)
        # events bracket every launch: per rank one causal-chunk call, then one
        # call per prefix shard; the prefix calls carry 80% of the work
        # per query rank: one event pair around the causal call, one around
        # its N prefix-shard calls back to back
        self.launches_per_step = 2 * w.N
        self.launches_per_event = w.N
        self.dominant = [2 * r + 1 for r in range(w.N)]
        self.secondary = [2 * r for r in range(w.N)]
        self.per_launch_work = [self.work_prefix / (w.N * w.N)]
        self.secondary_work = self.work_causal / w.N
        kv_tok = w.Hkv * w.D * 2 * 2
        self.per_launch_bytes = [sum(sh["ll"] for sh in self.shards) * kv_tok / w.N / w.N
                                 + (2 * C // (2 * w.N)) * w.Hq * w.D * (2 + 4)]
        self.kernel_name = "pcp_prefill_attn_causal over one paged DCP prefix shard"
        self.dtype = "bf16"

    def step(self, ev=None):
        cp, w = self.cp, self.w
        # the chunk's new K/V into the DCP shards (positions P .. P+C-1)
        for s, sh in enumerate(self.shards):
            cp.cp_slot_map_cache_write(self.req_c, self.pos_c, sh["bt_d"], s, w.N, w.I, w.bs,
                                       self.k, self.v, sh["kc"], sh["vc"], slot_out=sh["slots"])
        for r in range(w.N):
            if ev is not None:
                ev[2 * r][0].record()
            cp.pcp_prefill_attn_causal(self.q, w.P, r, w.N, w.scale, k=self.k, v=self.v,
                                       out=self.part_out[0], lse=self.part_lse[0])
            if ev is not None:
                ev[2 * r][1].record()
                ev[2 * r + 1][0].record()
            for s, sh in enumerate(self.shards):
                cp.pcp_prefill_attn_causal(self.q, w.P, r, w.N, w.scale, k_cache=sh["kc"],
                                           v_cache=sh["vc"], block_table=sh["bt_row"],
                                           local_len=sh["ll"], out=self.part_out[1 + s],
                                           lse=self.part_lse[1 + s])
            if ev is not None:
                ev[2 * r + 1][1].record()
            cp.cp_lse_merge(self.part_out, self.part_lse, out=self.out[r], lse_out=self.lse[r])

    def cpu_baseline(self, budget_s=15.0):
        import numpy as np

        import cp_inputs as ci
        import oracle

        w = self.w
        kall = np.concatenate([ci.bits(self.pk.cpu()), ci.bits(self.k.cpu())])
        vall = np.concatenate([ci.bits(self.pv.cpu()), ci.bits(self.v.cpu())])
        q = ci.bits(self.q.cpu())
        rows = oracle.pcp_rank_positions(w.C, w.N, w.N - 1)
        done, work, t0 = 0, 0, time.perf_counter()
        for i in rows[::max(1, len(rows) // 64)]:
            oracle.attention(q[i:i + 1], kall, vall, key_begin=0, key_end=w.P + i + 1,
                             scale=w.scale, q_dtype="bf16", kv_dtype="bf16")
            work += (w.P + int(i) + 1) * w.Hq * 4 * w.D
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return work / dt / 1e12, f"{done} query rows of rank {w.N - 1} (all {w.Hq} heads, full causal + prefix)"

    def config(self):
        w = self.w
        return {"workload": w.name, "chunk": w.C, "prefix": w.P, "pcp_ranks": w.N,
                "dcp_shards": w.N, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
                "interleave": w.I, "block_size": w.bs}


# ---------------------------------------------------------------------------
# DCP-sharded causal prefill: the new chunk's KV interleaved like the prefix's
# ---------------------------------------------------------------------------

class DcpPrefillBench:
    metric_unit = "TFLOP/s"

    def __init__(self, w, dev="cuda"):
        import numpy as np
        import torch

        import cp_inputs as ci
        import kv_context_parallelism_amd as cp

        self.w, self.cp = w, cp
        C, P = w.C, w.P
        self.q = ci.to_storage(ci.normal((C, w.Hq, w.D), w.seed + 1, dev), "bf16")
        self.k = ci.to_storage(ci.normal((P + C, w.Hkv, w.D), w.seed + 2, dev), "bf16")
        self.v = ci.to_storage(ci.normal((P + C, w.Hkv, w.D), w.seed + 3, dev), "bf16")
        tot = torch.tensor([P + C], dtype=torch.int32, device=dev)
        req_p = torch.zeros(P, dtype=torch.int32, device=dev)
        pos_p = torch.arange(P, dtype=torch.int32, device=dev)
        self.req_c = torch.zeros(C, dtype=torch.int32, device=dev)
        self.pos_c = torch.arange(P, P + C, dtype=torch.int32, device=dev)
        self.k_c, self.v_c = self.k[P:].contiguous(), self.v[P:].contiguous()
        self.shards = []
        for s in range(w.N):
            ll = int(cp.cp_local_seq_lens(tot, s, w.N, w.I).cpu()[0])
            bt, pool = ci.block_tables(np.array([(ll + w.bs - 1) // w.bs]), w.seed + 100 + s, 1.25)
            bt_d = torch.from_numpy(bt).to(dev)
            kc = ci.nan_fill_(torch.empty(pool, w.Hkv, w.bs, w.D, dtype=torch.bfloat16,
                                          device=dev), "bf16")
            vc = ci.nan_fill_(torch.empty_like(kc), "bf16")
            slots = cp.cp_slot_map(req_p, pos_p, bt_d, s, w.N, w.I, w.bs)
            cp.cp_cache_write(slots, self.k[:P].contiguous(), self.v[:P].contiguous(), kc, vc,
                              w.bs)
            self.shards.append(dict(ll=ll, bt_d=bt_d, bt_row=bt_d[0].contiguous(), kc=kc, vc=vc,
                                    slots=torch.empty(C, dtype=torch.int64, device=dev)))
        c = C // (2 * w.N)
        self.part_out = torch.empty(w.N, 2, c, w.Hq, w.D, dtype=torch.float32, device=dev)
        self.part_lse = torch.empty(w.N, 2, c, w.Hq, dtype=torch.float32, device=dev)
        self.out = torch.empty(w.N, 2, c, w.Hq, w.D, dtype=torch.float32, device=dev)
        self.lse = torch.empty(w.N, 2, c, w.Hq, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        causal = C * (C + 1) // 2
        # every (query, key) pair with key position <= query position, once
        self.work_step = (causal + C * P) * w.Hq * 4 * w.D
        self.tokens_step = C  # prefill tokens per step (one layer, all ranks)
        # events bracket every shard call: per PCP rank one call per DCP shard
        # per query rank: one event pair around its N shard calls back to back
        self.launches_per_step = w.N
        self.launches_per_event = w.N
        self.dominant = list(range(w.N))
        self.per_launch_work = [self.work_step / (w.N * w.N)]
        kv_tok = w.Hkv * w.D * 2 * 2
        self.per_launch_bytes = [sum(sh["ll"] for sh in self.shards) * kv_tok / w.N / w.N
                                 + (2 * c) * w.Hq * w.D * (2 + 4)]
        self.kernel_name = ("pcp_prefill_attn_causal over one DCP shard of prefix and chunk "
                            "(causal on interleaved positions), average call")
        self.dtype = "bf16"

    def step(self, ev=None):
        cp, w = self.cp, self.w
        # the chunk's K/V into the DCP shards (positions P .. P+C-1), interleaved
        for s, sh in enumerate(self.shards):
            cp.cp_slot_map_cache_write(self.req_c, self.pos_c, sh["bt_d"], s, w.N, w.I, w.bs,
                                       self.k_c, self.v_c, sh["kc"], sh["vc"], slot_out=sh["slots"])
        for r in range(w.N):
            if ev is not None:
                ev[r][0].record()
            for s, sh in enumerate(self.shards):
                cp.pcp_prefill_attn_causal(self.q, w.P, r, w.N, w.scale, k_cache=sh["kc"],
                                           v_cache=sh["vc"], block_table=sh["bt_row"],
                                           local_len=sh["ll"], dcp=(s, w.N, w.I),
                                           out=self.part_out[s], lse=self.part_lse[s])
            if ev is not None:
                ev[r][1].record()
            cp.cp_lse_merge(self.part_out, self.part_lse, out=self.out[r], lse_out=self.lse[r])

    def cpu_baseline(self, budget_s=15.0):
        import numpy as np

        import cp_inputs as ci
        import oracle

        w = self.w
        kall, vall = ci.bits(self.k.cpu()), ci.bits(self.v.cpu())
        q = ci.bits(self.q.cpu())
        rows = oracle.pcp_rank_positions(w.C, w.N, w.N - 1)
        done, work, t0 = 0, 0, time.perf_counter()
        for i in rows[::max(1, len(rows) // 64)]:
            po, pl = [], []
            for s in range(w.N):
                o, l = oracle.attention(q[i:i + 1], kall, vall, key_begin=0, key_end=w.P + i + 1,
                                        scale=w.scale, q_dtype="bf16", kv_dtype="bf16",
                                        shard=(w.N, w.I, s))
                po.append(o.reshape(-1, w.D))
                pl.append(l.reshape(-1))
            oracle.lse_merge(np.stack(po), np.stack(pl))
            work += (w.P + int(i) + 1) * w.Hq * 4 * w.D
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return work / dt / 1e12, (f"{done} query rows of rank {w.N - 1} (all {w.Hq} heads, "
                                  f"{w.N} causal shard partials + merge)")

    def config(self):
        w = self.w
        return {"workload": w.name, "new_tokens": w.C, "prefix_tokens": w.P, "q_heads": w.Hq,
                "kv_heads": w.Hkv, "head_dim": w.D, "pcp_size": w.N, "dcp_shards": w.N,
                "interleave": w.I, "block_size": w.bs}


# ---------------------------------------------------------------------------
# KV gather: a cached prefix reassembled from its DCP shards in position order
# ---------------------------------------------------------------------------

class KvGatherBench:
    metric_unit = "GB/s"

    def __init__(self, w, dev="cuda"):
        import numpy as np
        import torch

        import cp_inputs as ci
        import kv_context_parallelism_amd as cp

        self.w, self.cp = w, cp
        P = w.P
        self.k = ci.to_storage(ci.normal((P, w.Hkv, w.D), w.seed + 2, dev), w.kv_dtype)
        self.v = ci.to_storage(ci.normal((P, w.Hkv, w.D), w.seed + 3, dev), w.kv_dtype)
        self.seq = torch.tensor([P], dtype=torch.int32, device=dev)
        req = torch.zeros(P, dtype=torch.int32, device=dev)
        pos = torch.arange(P, dtype=torch.int32, device=dev)
        self.kc, self.vc, self.bt = [], [], []
        for r in range(w.N):
            ll = cp.cp_local_seq_lens(self.seq, r, w.N, w.I).cpu().numpy()
            bt, pool = ci.block_tables((ll.astype(np.int64) + w.bs - 1) // w.bs, w.seed + 100 + r,
                                       1.25)
            bt_d = torch.from_numpy(bt).to(dev)
            kc = ci.nan_fill_(torch.empty(pool, w.Hkv, w.bs, w.D, dtype=self.k.dtype, device=dev),
                              w.kv_dtype)
            vc = ci.nan_fill_(torch.empty_like(kc), w.kv_dtype)
            slots = cp.cp_slot_map(req, pos, bt_d, r, w.N, w.I, w.bs)
            cp.cp_cache_write(slots, self.k, self.v, kc, vc, w.bs)
            self.kc.append(kc)
            self.vc.append(vc)
            self.bt.append(bt_d)
        self.k_out = torch.empty(1, P, w.Hkv, w.D, dtype=self.k.dtype, device=dev)
        self.v_out = torch.empty_like(self.k_out)
        torch.cuda.synchronize()
        row = w.Hkv * w.D * self.k.element_size()
        # K and V: every row read from its shard once and written once
        self.work_step = 2 * 2 * P * row
        self.tokens_step = P  # tokens gathered per step
        self.per_launch_work = [self.work_step]
        self.per_launch_bytes = [self.work_step]
        self.launches_per_step = 1
        self.launches_per_event = 4
        self.dominant = [0]
        self.kernel_name = "cp_kv_gather (K and V, whole prefix)"
        self.dtype = w.kv_dtype

    def step(self, ev=None):
        w = self.w
        if ev is None:
            self.cp.cp_kv_gather(self.kc, self.vc, self.bt, self.seq, w.N, w.I, w.bs, 0, w.P,
                                 k_out=self.k_out, v_out=self.v_out)
            return
        # the timed launches: the gather repeated back to back between one
        # event pair (an event pair around a single ~90 us launch adds its own
        # few-us gap to it)
        ev[0][0].record()
        for _ in range(self.launches_per_event):
            self.cp.cp_kv_gather(self.kc, self.vc, self.bt, self.seq, w.N, w.I, w.bs, 0, w.P,
                                 k_out=self.k_out, v_out=self.v_out)
        ev[0][1].record()

    def cpu_baseline(self, budget_s=15.0):
        """The oracle's gather (numpy over the oracle's slot map) on windows of
        4,096 positions of the same shard caches, until the budget is spent."""
        import oracle

        import cp_inputs as ci

        w = self.w
        caches = [ci.bits(c.cpu()) for c in self.kc] + [ci.bits(c.cpu()) for c in self.vc]
        bts = [bt.cpu().numpy() for bt in self.bt]
        row = w.Hkv * w.D * self.k.element_size()
        done, t0 = 0, time.perf_counter()
        W = 4096
        while done + W <= w.P:
            oracle.kv_gather(caches[:w.N], bts, [w.P], w.N, w.I, w.bs, done, W)
            oracle.kv_gather(caches[w.N:], bts, [w.P], w.N, w.I, w.bs, done, W)
            done += W
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return 2 * 2 * done * row / dt / 1e9, f"positions 0..{done - 1} of {w.P} (K and V)"

    def config(self):
        w = self.w
        return {"workload": w.name, "prefix_tokens": w.P, "kv_heads": w.Hkv, "head_dim": w.D,
                "dcp_shards": w.N, "interleave": w.I, "block_size": w.bs,
                "window": [0, w.P]}


# ---------------------------------------------------------------------------
# Head-scattered output exchanges: the per-rank kernels of AG+RS and all-to-all
# ---------------------------------------------------------------------------

class HeadScatterBench:
    """One rank's share of both exchange paths at the MLA decode shape, for
    every layer of a decode step: the AG+RS correction of its [B][H][Dv]
    partial (given all N ranks' LSEs), the all-to-all packing of the same
    partial, and the exact merge of the N packed partials of its H/N-head slice
    into the bf16 output.  Each layer has its own buffers (over 1 GB in all, so
    that nothing is served from the last-level cache between layers); each
    kernel runs for all layers back to back between one pair of events."""
    metric_unit = "GB/s"
    layers = 16

    def __init__(self, w, dev="cuda"):
        import torch

        import cp_inputs as ci
        import kv_context_parallelism_amd as cp

        self.w, self.cp = w, cp
        B, H, Dv, N = w.B, w.Hq, w.Dv, w.N
        hs = H // N
        self.o, self.l, self.recv = [], [], []
        for j in range(self.layers):
            o = ci.normal((N, B, H, Dv), w.seed + 10 * j + 1, dev)
            l = 4 * ci.normal((N, B, H), w.seed + 10 * j + 2, dev)
            # what rank 0 receives: slot 0 of every rank's send buffer
            self.recv.append(torch.stack([cp.cp_a2a_pack(o[r], l[r], N)[0] for r in range(N)]))
            self.o.append(o[0].clone())
            self.l.append(l)
            del o
        self.buf = [torch.empty(N, B, hs, Dv + 4, device=dev) for _ in range(self.layers)]
        self.corr = [torch.empty(B, H, Dv, device=dev) for _ in range(self.layers)]
        self.L = [torch.empty(B, H, device=dev) for _ in range(self.layers)]
        self.out = [torch.empty(B, hs, Dv, dtype=torch.bfloat16, device=dev)
                    for _ in range(self.layers)]
        self.lse = [torch.empty(B, hs, device=dev) for _ in range(self.layers)]
        torch.cuda.synchronize()
        rows = B * H
        # algorithmic bytes: each element read once, written once (the pack
        # writes the padding of its packed rows; the merge does not read it)
        self.work_correct = rows * (Dv * 4 + N * 4) + rows * (Dv + 1) * 4
        self.work_pack = rows * (Dv + 1) * 4 + rows * (Dv + 4) * 4
        self.work_merge = (rows // N) * (N * (Dv + 1) * 4 + Dv * 2 + 4)
        self.work_step = self.layers * (self.work_correct + self.work_pack + self.work_merge)
        self.tokens_step = None  # no token count: three exchange kernels of one rank
        self.per_launch_work = [self.work_pack]
        self.per_launch_bytes = [self.work_pack]
        self.launches_per_step = 3
        self.launches_per_event = self.layers
        self.dominant = [1]
        self.kernel_name = "cp_a2a_pack (one rank's partial, 8 head partitions)"
        self.secondaries = [("cp_lse_correct (AG+RS, one rank's partial)", [0], self.work_correct),
                            ("cp_lse_merge_packed (8 parts of a 16-head slice, bf16 out)", [2],
                             self.work_merge)]
        self.dtype = "f32"

    def step(self, ev=None):
        cp, N, Dv = self.cp, self.w.N, self.w.Dv
        for k in range(3):
            if ev is not None:
                ev[k][0].record()
            for j in range(self.layers):
                if k == 0:
                    cp.cp_lse_correct(self.o[j], self.l[j], 0, corrected=self.corr[j],
                                      lse_out=self.L[j])
                elif k == 1:
                    cp.cp_a2a_pack(self.o[j], self.l[j][0], N, buf=self.buf[j])
                else:
                    cp.cp_lse_merge_packed(self.recv[j], Dv, out=self.out[j], lse_out=self.lse[j])
            if ev is not None:
                ev[k][1].record()

    def cpu_baseline(self, budget_s=15.0):
        """The oracle's correction, packing and packed merge of layer 0's
        partials, over blocks of requests until the budget is spent."""
        import oracle

        w = self.w
        o = self.o[0].cpu().numpy()
        l = self.l[0].cpu().numpy()
        recv = self.recv[0].cpu().numpy()
        per_req = self.work_step / self.layers / w.B
        done, t0 = 0, time.perf_counter()
        blk = 4
        while done + blk <= w.B:
            sl = slice(done, done + blk)
            oracle.lse_correct(o[sl].reshape(-1, w.Dv), l[:, sl].reshape(w.N, -1), 0)
            oracle.a2a_pack(o[sl], l[0, sl], w.N)
            oracle.lse_merge_packed(recv[:, sl], w.Dv)
            done += blk
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return done * per_req / dt / 1e9, f"requests 0..{done - 1} of {w.B} of one layer, all three steps"

    def config(self):
        w = self.w
        return {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "value_dim": w.Dv,
                "cp_ranks": w.N, "heads_per_rank": w.Hq // w.N, "layers": self.layers,
                "partials": "fp32 out + fp32 LSE", "merged_out": "bf16"}


BENCHES = {"gqa_decode": GqaDecodeBench, "mla_decode": MlaDecodeBench,
           "pcp_prefill": PrefillBench, "dcp_prefill": DcpPrefillBench,
           "kv_gather": KvGatherBench, "head_scatter": HeadScatterBench}
BENCH_WORKLOADS = ["gqa_decode_bf16", "gqa_decode_mtp_bf16", "mla_decode_bf16", "mla_decode_fp8",
                   "pcp_prefill_bf16", "dcp_prefill_bf16", "kv_gather_bf16", "head_scatter_mla"]


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def _step_outputs(bench) -> list:
    """The tensors a step writes last (the merged output and LSE)."""
    ts = []
    for t in (getattr(bench, "out", None), getattr(bench, "lse", None)):
        if isinstance(t, (list, tuple)):
            ts.extend(t)
        elif t is not None:
            ts.append(t)
    return ts


def time_graph(bench, steps: int, warmup: int):
    """The step captured once as a HIP graph (every launch of the step, the same
    work as the eager step) and replayed: ``warmup`` untimed replays, then
    exactly ``steps`` timed ones between synchronisations.  The outputs of the
    last replay must equal the eager step's byte for byte.  Returns
    (ms per step, median ms per step from events around each replay)."""
    import torch

    bench.step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in _step_outputs(bench)]
    side = torch.cuda.Stream()  # capture needs the step warmed on a side stream
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bench.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bench.step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    for t in _step_outputs(bench):
        t.fill_(float("nan"))
    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))  # noqa
    sev = [mk() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sev[i][0].record()
        g.replay()
        sev[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for a, b in zip(ref, _step_outputs(bench)):
        if not torch.equal(a.view(torch.uint8), b.view(torch.uint8)):
            raise RuntimeError("graph replay of the step differs from the eager step")
    del g
    return elapsed * 1e3 / steps, _median([a.elapsed_time(b) for a, b in sev])


def _spin_cycles(bench) -> int:
    """Clock cycles of a GPU spin that outlasts the host's issue of one step
    (three times the measured issue time, at least 2 ms)."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cyc = 1 << 20
    torch.cuda.synchronize()
    a.record()
    torch.cuda._sleep(cyc)
    b.record()
    torch.cuda.synchronize()
    ms_per_cyc = max(a.elapsed_time(b), 1e-3) / cyc
    t0 = time.perf_counter()
    bench.step()
    issue_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    return int(min(max(3 * issue_ms, 2.0), 200.0) / ms_per_cyc)


def measure(bench, steps: int, warmup: int, graph: bool = True) -> dict:
    """Warm up, then time exactly ``steps`` steps of ``bench`` with HIP events
    around every launch of interest and around every step (the launches'
    roofline), and exactly ``steps`` replays of the step captured as a HIP
    graph (the step rate); returns the fields of a bench line (value, step
    times, the dominant kernel's roofline, the final merge)."""
    import torch

    w = bench.w
    for _ in range(warmup):
        bench.step()
    torch.cuda.synchronize()
    n_ev = bench.launches_per_step
    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))  # noqa
    ev = [[mk() for _ in range(n_ev)] for _ in range(steps)]
    sev = [mk() for _ in range(steps)]
    print(f"[bench] {w.name}: timing {steps} steps", file=sys.stderr, flush=True)
    # eager steps as the host issues them (launch gaps included)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sev[i][0].record()
        bench.step()
        sev[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    eager_ms_step = elapsed * 1e3 / steps
    eager_step_ms = [a.elapsed_time(b) for a, b in sev]
    # the launches of interest, each step queued behind a GPU spin that outlasts
    # the host's issue of the step, so the events time the kernels back to back
    # (as a kernel trace does) and not the host's launch rate
    spin = _spin_cycles(bench)
    torch.cuda.synchronize()
    for i in range(steps):
        torch.cuda._sleep(spin)
        bench.step(ev[i])
    torch.cuda.synchronize()
    per_event = getattr(bench, "launches_per_event", 1)  # launches between one event pair
    launch_ms = [step[k][0].elapsed_time(step[k][1]) / per_event for step in ev
                 for k in bench.dominant]
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    med_launch_s = _median(launch_ms) / 1e3
    unit = bench.metric_unit
    if unit == "GB/s":
        scale_v, peak, bound = 1e9, HBM_PEAK_GBS, "hbm"
    else:
        scale_v, peak, bound = 1e12, BF16_PEAK_TFLOPS, "mfma"
    avg_work = sum(bench.per_launch_work) / len(bench.per_launch_work)
    achieved = avg_work / avg_launch_s / scale_v
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": _counted_traffic(w.name),
            "kernel": bench.kernel_name,
            "avg_launch_us": round(avg_launch_s * 1e6, 2),
            "median_launch_us": round(med_launch_s * 1e6, 2),
            "launches_timed": len(launch_ms) * per_event,
            ("algorithmic_bytes_per_launch" if unit == "GB/s" else "algorithmic_flop_per_launch"):
                int(avg_work)}
    if unit != "GB/s":
        avg_bytes = sum(bench.per_launch_bytes) / len(bench.per_launch_bytes)
        roof["hbm_gbs"] = round(avg_bytes / avg_launch_s / 1e9, 2) if avg_bytes else None
    if getattr(bench, "secondary", None):
        sec_ms = [step[k][0].elapsed_time(step[k][1]) for step in ev for k in bench.secondary]
        sec_s = sum(sec_ms) / len(sec_ms) / 1e3
        roof["secondary"] = {"kernel": "pcp_prefill_attn_causal over the chunk's own keys",
                             "avg_launch_us": round(sec_s * 1e6, 2),
                             "median_launch_us": round(_median(sec_ms) * 1e3, 2),
                             "achieved": round(bench.secondary_work / sec_s / scale_v, 2),
                             "frac": round(bench.secondary_work / sec_s / scale_v / peak, 4)}
    if getattr(bench, "secondaries", None):
        roof["secondary"] = []
        for name, idx, work in bench.secondaries:
            sec_ms = [step[k][0].elapsed_time(step[k][1]) / per_event for step in ev for k in idx]
            sec_s = sum(sec_ms) / len(sec_ms) / 1e3
            roof["secondary"].append({"kernel": name, "avg_launch_us": round(sec_s * 1e6, 2),
                                      "median_launch_us": round(_median(sec_ms) * 1e3, 2),
                                      "achieved": round(work / sec_s / scale_v, 2),
                                      "frac": round(work / sec_s / scale_v / peak, 4)})
    # the step rate: the step replayed as one HIP graph (no launch gaps)
    if graph:
        print(f"[bench] {w.name}: timing {steps} graph replays of the step", file=sys.stderr,
              flush=True)
        ms_step, med_step = time_graph(bench, steps, warmup)
    else:
        ms_step, med_step = eager_ms_step, _median(eager_step_ms)
    out = {"value": round(bench.work_step / (ms_step / 1e3) / scale_v, 2), "unit": unit,
           "ms_per_step": round(ms_step, 4), "median_step_ms": round(med_step, 4),
           "timing": "HIP graph replay of the whole step" if graph else "eager launches",
           "eager": {"ms_per_step": round(eager_ms_step, 4),
                     "median_step_ms": round(_median(eager_step_ms), 4),
                     "value": round(bench.work_step / (eager_ms_step / 1e3) / scale_v, 2)},
           "roofline": roof}
    if getattr(bench, "merge_idx", None) is not None:
        m_ms = [step[bench.merge_idx][0].elapsed_time(step[bench.merge_idx][1]) for step in ev]
        m_s = sum(m_ms) / len(m_ms) / 1e3
        out["merge"] = {"kernel": "cp_lse_merge of the N shard partials",
                        "avg_launch_us": round(m_s * 1e6, 2),
                        "median_launch_us": round(_median(m_ms) * 1e3, 2),
                        "gbs": round(bench.merge_bytes / m_s / 1e9, 2)}
    if getattr(bench, "tokens_step", None):
        # tokens of one layer of the whole (simulated) CP group per second: the
        # N ranks' calls run one after another on this GPU
        out["tokens_per_s"] = round(bench.tokens_step / (ms_step / 1e3), 1)
    return out


def cpu_leg(bench, budget_s: float, one_thread: bool = False) -> dict:
    """The untuned fp64 oracle on a bounded sample of the same workload, on
    every host core this process may use (and, if asked, on one thread)."""
    import oracle

    cores = _cpu_cores()
    oracle.set_threads(cores)
    v, sample = bench.cpu_baseline(budget_s)
    leg = {"value": round(v, 6), "unit": bench.metric_unit, "cores": cores, "kind": "oracle",
           "sample": sample}
    if hasattr(bench, "cpu_step_s"):
        leg["step_ms"] = round(bench.cpu_step_s * 1e3, 3)
    if one_thread:
        oracle.set_threads(1)
        v1, sample1 = bench.cpu_baseline(budget_s)
        leg["one_thread"] = {"value": round(v1, 6), "unit": bench.metric_unit, "cores": 1,
                             "sample": sample1}
        if hasattr(bench, "cpu_step_s"):
            leg["one_thread"]["step_ms"] = round(bench.cpu_step_s * 1e3, 3)
        oracle.set_threads(cores)
    return leg


# The default run adds these to the headline line: the small fp32 case as a
# latency, and the MLA (bf16, fp8) and prefill workloads with their own roofline
# (TFLOP/s against the bf16 MFMA peak) and oracle timings.
EXTRA_WORKLOADS = ["gqa_tiny_f32", "mla_decode_bf16", "mla_decode_fp8", "pcp_prefill_bf16",
                   "dcp_prefill_bf16", "gqa_decode_mtp_bf16", "kv_gather_bf16", "head_scatter_mla"]


def extra_block(name: str, steps: int, warmup: int, cpu: bool, budget_s: float) -> dict:
    import torch

    import cp_inputs as ci

    w = ci.WORKLOADS[name]
    print(f"[bench] setting up {w.name}", file=sys.stderr, flush=True)
    bench = BENCHES[w.kind](w)
    m = measure(bench, steps, warmup)
    if name == "gqa_tiny_f32":
        # a latency case: one decode step of 4 shards of a 1,000-token request
        # (slot map + cache write, 4 shard partials, merge) in microseconds
        block = {"metric": "step latency", "unit": "us", "higher_is_better": False,
                 "latency_us_median": round(m["median_step_ms"] * 1e3, 2),
                 "latency_us_mean": round(m["ms_per_step"] * 1e3, 2),
                 "timing": m["timing"],
                 "eager_latency_us_median": round(m["eager"]["median_step_ms"] * 1e3, 2),
                 "dtype": bench.dtype, "config": bench.config(),
                 "shard_partial_median_us": m["roofline"]["median_launch_us"]}
        if "merge" in m:
            block["merge_median_us"] = m["merge"]["median_launch_us"]
    else:
        block = dict(m)
        block["dtype"] = bench.dtype
        block["config"] = bench.config()
    if cpu:
        print(f"[bench] {w.name}: timing the fp64 oracle", file=sys.stderr, flush=True)
        leg = cpu_leg(bench, budget_s, one_thread=(name == "gqa_tiny_f32"))
        if name == "gqa_tiny_f32":
            leg = {"step_us": round(bench.cpu_step_s * 1e6, 1), "unit": "us", "cores": leg["cores"],
                   "kind": "oracle", "sample": leg["sample"],
                   "one_thread": {"step_us": round(leg["one_thread"]["step_ms"] * 1e3, 1),
                                  "unit": "us", "cores": 1}}
        block["cpu_baseline"] = leg
    del bench
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return block


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_decode_bf16", choices=BENCH_WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (for profiler counter passes)")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the selected workload (the default run also measures "
                         + ", ".join(EXTRA_WORKLOADS) + ")")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of a workload, run a plain device copy of MIB MiB (the "
                         "known-size reference that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the N shards are simulated as separate buffers on a "
              "single MI355X, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import cp_inputs as ci

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": args.steps}), flush=True)
        return
    w = ci.WORKLOADS[args.workload]
    print(f"[bench] setting up {w.name}", file=sys.stderr, flush=True)
    bench = BENCHES[w.kind](w)
    m = measure(bench, args.steps, args.warmup, graph=not args.no_graph)
    line = {
        "metric": METRIC, "value": m["value"], "unit": m["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": m["ms_per_step"],
        "median_step_ms": m["median_step_ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": bench.dtype, "data": "synthetic", "config": bench.config(),
        "roofline": m["roofline"],
    }
    for key in ("timing", "eager", "merge", "tokens_per_s"):
        if key in m:
            line[key] = m[key]
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_leg(bench, 15.0,
                                       one_thread=args.workload == "gqa_decode_bf16")
    del bench
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if args.workload == "gqa_decode_bf16" and not args.no_extra:
        line["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            line["workloads"][name] = extra_block(name, args.steps, args.warmup,
                                                  not args.no_cpu_baseline, 10.0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
