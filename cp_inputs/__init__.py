"""Seeded synthetic inputs for the context-parallel attention workloads.

Shared by both sides of every parity check: the fp64 oracle (test
infrastructure) and the HIP library.  This module holds none of the method's
arithmetic -- no ownership rule, no slot formula, no attention, no merge.  It
only draws numbers:

  * normal(shape, seed, device, std): i.i.d. N(0, std^2) float32 from a torch
    generator seeded with ``seed`` (on ``device``; a given seed reproduces the
    same values on the same device type);
  * to_storage(x, dtype): the storage form of x -- float32, bfloat16 by
    round-to-nearest-even, or OCP fp8 E4M3 (finite) after clamping to +-448;
  * fp8_quantize(x): per-tensor scale amax/448, then to_storage(x/scale);
  * uniform_lengths(...): integer context lengths, inclusive bounds;
  * block_tables(needed, ...): a random permutation of a block pool handed out
    in request order, padded with -1 (the caller says how many blocks each
    request needs);
  * bits(t): the storage bits of a CPU tensor as a numpy array.

WORKLOADS lists the shapes, sizes and distributions of the workloads the
pages describe (decode over sharded paged KV for GQA and absorbed-MLA models,
and a PCP prefill over a DCP-sharded prefix).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

FP8_MAX = 448.0
NAN_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0, "fp8_e4m3fn": 0x7F}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3fn": torch.float8_e4m3fn}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                      # "gqa_decode" | "mla_decode" | "pcp_prefill" | "dcp_prefill"
                                   # | "kv_gather" | "head_scatter"
    B: int = 1
    Hq: int = 1
    Hkv: int = 1
    D: int = 128                   # key width (GQA head dim, MLA latent width)
    Dv: int = 128                  # value width
    ctx: tuple = (1000, 1000)      # inclusive range of context lengths (decode)
    N: int = 1                     # shards
    I: int = 1                     # interleave size
    bs: int = 16                   # block size
    q_dtype: str = "f32"
    kv_dtype: str = "f32"
    q_std: float = 1.0
    kv_std: float = 1.0
    scale: float = 1.0
    C: int = 0                     # prefill: new-chunk length
    P: int = 0                     # prefill: cached-prefix length
    seed: int = 1000
    q_len: int = 1                 # decode: query tokens per request (the last q_len positions)
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # tiny fp32 GQA decode: the oracle finishes it in milliseconds
    "gqa_tiny_f32": Workload("gqa_tiny_f32", "gqa_decode", B=1, Hq=8, Hkv=2, D=64, Dv=64,
                             ctx=(1000, 1000), N=4, I=4, bs=16, q_dtype="f32", kv_dtype="f32",
                             scale=1 / 8, seed=1001),
    # bf16 GQA decode: 32 requests, 32/8 heads, contexts uniform in [4K, 32K], 8 shards
    "gqa_decode_bf16": Workload("gqa_decode_bf16", "gqa_decode", B=32, Hq=32, Hkv=8, D=128,
                                Dv=128, ctx=(4096, 32768), N=8, I=16, bs=16, q_dtype="bf16",
                                kv_dtype="bf16", scale=1 / math.sqrt(128), seed=1002),
    # the same decode step with two query tokens per request (one speculative
    # token verified with the current one), causal on the interleaved positions
    "gqa_decode_mtp_bf16": Workload("gqa_decode_mtp_bf16", "gqa_decode", B=32, Hq=32, Hkv=8, D=128,
                                Dv=128, ctx=(4096, 32768), N=8, I=16, bs=16, q_dtype="bf16",
                                kv_dtype="bf16", scale=1 / math.sqrt(128), seed=1009, q_len=2),
    # absorbed MLA decode, bf16 latent 576 (512 + 64 rope), value width 512
    "mla_decode_bf16": Workload("mla_decode_bf16", "mla_decode", B=64, Hq=128, Hkv=1, D=576,
                                Dv=512, ctx=(65536, 65536), N=8, I=1, bs=64, q_dtype="bf16",
                                kv_dtype="bf16", q_std=1 / 24, kv_std=1 / 24, scale=1 / 24,
                                seed=1003),
    # same shapes with unit-variance q and latent, so scores are peaked and the
    # softmax is far from uniform (discriminates outputs and LSE)
    "mla_decode_bf16_peaked": Workload("mla_decode_bf16_peaked", "mla_decode", B=64, Hq=128,
                                       Hkv=1, D=576, Dv=512, ctx=(65536, 65536), N=8, I=1,
                                       bs=64, q_dtype="bf16", kv_dtype="bf16", scale=1 / 24,
                                       seed=1013),
    # absorbed MLA decode, 1M-token contexts, fp8 E4M3 latent with a per-tensor scale
    "mla_decode_fp8": Workload("mla_decode_fp8", "mla_decode", B=4, Hq=128, Hkv=1, D=576,
                               Dv=512, ctx=(1 << 20, 1 << 20), N=8, I=1, bs=64, q_dtype="bf16",
                               kv_dtype="fp8_e4m3fn", scale=1 / 24, seed=1004),
    # PCP causal prefill: a 32K new chunk over a 64K prefix held in 8 DCP shards
    "pcp_prefill_bf16": Workload("pcp_prefill_bf16", "pcp_prefill", B=1, Hq=32, Hkv=8, D=128,
                                 Dv=128, N=8, I=16, bs=16, q_dtype="bf16", kv_dtype="bf16",
                                 scale=1 / math.sqrt(128), C=32768, P=65536, seed=1005),
    # DCP-sharded causal prefill: the prefill workload with the new chunk's KV
    # also interleaved over the 8 DCP shards (prefix and chunk: 98,304 positions)
    "dcp_prefill_bf16": Workload("dcp_prefill_bf16", "dcp_prefill", B=1, Hq=32, Hkv=8, D=128,
                                 Dv=128, N=8, I=16, bs=16, q_dtype="bf16", kv_dtype="bf16",
                                 scale=1 / math.sqrt(128), C=32768, P=65536, seed=1007),
    # KV gather: the prefill workload's 64K-token prefix, held in 8 DCP shards
    # (I 16, bs 16, 8 KV heads x 128, bf16 K and V), reassembled in position order
    "kv_gather_bf16": Workload("kv_gather_bf16", "kv_gather", B=1, Hkv=8, D=128, Dv=128, N=8,
                               I=16, bs=16, kv_dtype="bf16", P=65536, seed=1006),
    # Head-scattered output exchanges at the MLA decode shape: one rank's
    # partials for 64 requests x 128 heads x 512 (fp32 outputs and LSEs) and
    # the 8 packed partials of its 16-head slice that the all-to-all delivers
    "head_scatter_mla": Workload("head_scatter_mla", "head_scatter", B=64, Hq=128, Dv=512, N=8,
                                 seed=1008),
}


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    x = torch.randn(tuple(shape), generator=generator(seed, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def to_storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x.to(torch.float32)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "fp8_e4m3fn":
        # torch's cast does not saturate: clamp first, then round to nearest even
        return x.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    raise ValueError(dtype)


def fp8_scale(amax: float) -> float:
    return float(amax) / FP8_MAX if amax > 0 else 1.0


def fp8_quantize(x: torch.Tensor):
    s = fp8_scale(float(x.abs().max()))
    return to_storage(x / s, "fp8_e4m3fn"), s


def uniform_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def block_tables(needed, seed: int, pool_factor: float = 2.0):
    """needed[b] blocks for request b; returns (table [B][width] int32 padded with
    -1, pool size).  Block ids are a seeded random permutation of the pool."""
    needed = np.asarray(needed, dtype=np.int64)
    total = int(needed.sum())
    pool = max(int(math.ceil(total * pool_factor)), 1)
    width = max(int(needed.max(initial=0)), 1)
    perm = np.random.default_rng(seed).permutation(pool).astype(np.int32)
    bt = np.full((len(needed), width), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(needed):
        bt[b, :n] = perm[off:off + n]
        off += int(n)
    return bt, pool


def bits(t: torch.Tensor) -> np.ndarray:
    """Storage bits of a CPU tensor as numpy (float32 / uint16 / uint8)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise ValueError(t.dtype)


def nan_fill_(t: torch.Tensor, dtype: str) -> torch.Tensor:
    """Fill a storage tensor with the dtype's quiet-NaN bit pattern."""
    if dtype == "f32":
        t.view(torch.int32).fill_(NAN_BITS["f32"])
    elif dtype == "bf16":
        t.view(torch.int16).fill_(NAN_BITS["bf16"])
    else:
        t.view(torch.uint8).fill_(NAN_BITS["fp8_e4m3fn"])
    return t


def scaled(w: Workload, **kw) -> Workload:
    """A copy of workload w with some fields replaced (smaller parity cases)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)
