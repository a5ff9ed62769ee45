"""Seeded synthetic jagged-attention workloads.

This module only draws inputs: sequence lengths, offsets and random values.
It contains none of the attention arithmetic, so the CPU oracle tests and the
HIP path can both be fed from it.

The five workloads below stand in for the production ads traffic of the web
page piletech.kr/articles/112134 (section 상세 정리 / Detailed notes, item on
the jagged-input problem: every ad request carries a user history of a
different length, and padding those to a common length wastes up to half of
the compute).  The production data is private, so lengths are drawn from
parametric distributions with the stated medians, maxima and tails.

Draw order for one (workload, seed): lengths (query lengths first, then key
lengths when they differ), then Q, K, V and dO as float32 standard normals
times the workload's std, each in that order, then bf16 rounding
(round-to-nearest-even) for bf16 workloads.
"""

import math
from dataclasses import dataclass

import numpy as np

# sigma of the log-normal length laws: with mu = ln(median) and
# sigma = sqrt(2 ln 2) the unclipped mean exp(mu + sigma^2/2) is 2 * median,
# i.e. max/2 for max = 4 * median -- the "about 50% padding waste" shape.
LOGNORMAL_SIGMA = math.sqrt(2.0 * math.log(2.0))


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    dtype: str            # "bf16" or "fp32"
    std: float            # value scale of Q, K, V and dO
    causal: bool
    activation: str       # "softmax" or "silu"
    q_law: tuple          # length law of the query side
    kv_law: tuple | None  # length law of the key side (None: same lengths as q)
    backward: bool        # whether the workload runs the backward pass
    description: str
    block: int = 0        # > 0: BlockAttention, attention within runs of `block` tokens
    rope_base: float = 0.0  # > 0: BlockAttention's fused rotary embedding of that base
    n_seeds: int = 0      # > 0: pooled attention, n_seeds shared queries per sequence (q_law unused)
    mx: bool = False      # MXFP8 (E4M3 operands, E8M0 block scales; bf16 in and out)


WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", 8, 2, 32, "fp32", 1.0, False, "softmax",
        ("uniform", 1, 64), None, True,
        "tiny jagged self-attention, batch 8, lengths U{1..64}, 2 heads, d 32, fp32"),
    "selfattn_causal": Workload(
        "selfattn_causal", 256, 4, 128, "bf16", 1.0, True, "softmax",
        ("lognormal", 256, 1024), None, True,
        "jagged causal self-attention, batch 256, log-normal lengths "
        "(median 256, max 1024), 4 heads, d 128, bf16"),
    "cross_asym": Workload(
        "cross_asym", 512, 8, 64, "bf16", 1.0, False, "softmax",
        ("uniform", 1, 64), ("lognormal", 1024, 4096), False,
        "asymmetric jagged cross-attention, batch 512, query lengths U{1..64} "
        "(candidate ads), key lengths log-normal (median 1024, max 4096) "
        "(user history), 8 heads, d 64, bf16, forward only"),
    "gdpa_silu": Workload(
        "gdpa_silu", 256, 4, 128, "bf16", 0.5, True, "silu",
        ("lognormal", 512, 2048), None, True,
        "GDPA causal self-attention with silu(s*qk)/L_kv, batch 256, "
        "log-normal lengths (median 512, max 2048), 4 heads, d 128, bf16, std 0.5"),
    "pareto_train": Workload(
        "pareto_train", 1024, 4, 128, "bf16", 1.0, True, "softmax",
        ("pareto", 16, 2048, 1.5), None, True,
        "training-scale jagged causal self-attention, batch 1024, Pareto(1.5) "
        "lengths clipped to [16, 2048], random order, 4 heads, d 128, bf16"),
}

# Workload order as listed above; index 1 is the headline workload.
# BlockAttention (piletech.kr/articles/112134, Detailed notes, BlockAttention
# item: fixed 64-token blocks) on the lengths of the causal self-attention
# workload; not one of the five configurations, measured beside them.
WORKLOADS["block_attn"] = Workload(
    "block_attn", 256, 4, 128, "bf16", 1.0, True, "softmax",
    ("lognormal", 256, 1024), None, True,
    "BlockAttention (causal within fixed 64-token blocks), batch 256, log-normal lengths "
    "(median 256, max 1024), 4 heads, d 128, bf16", block=64)

# The same with the rotary embedding the BlockAttention item fuses in (base
# 10000, rotate-half pairs; positions from each block's first token).
WORKLOADS["block_rope"] = Workload(
    "block_rope", 256, 4, 128, "bf16", 1.0, True, "softmax",
    ("lognormal", 256, 1024), None, True,
    "BlockAttention with fused rotary embedding (base 10000), causal within fixed 64-token blocks, batch 256, "
    "log-normal lengths (median 256, max 1024), 4 heads, d 128, bf16", block=64, rope_base=10000.0)

# Pooled multi-head attention (Detailed notes, jagged-input item): 4 seed
# queries shared by every sequence pool the user histories of the
# cross-attention workload; forward and backward.
WORKLOADS["pooled_hist"] = Workload(
    "pooled_hist", 512, 8, 64, "bf16", 1.0, False, "softmax",
    ("fixed", 4), ("lognormal", 1024, 4096), True,
    "pooled multi-head attention, 4 seed queries shared by 512 sequences, key lengths log-normal (median 1024, "
    "max 4096), 8 heads, d 64, bf16", n_seeds=4)

# MXFP8 forward (Key points, MXFP8 bullet; Detailed notes, MXFP8 item) on the
# shapes of the causal self-attention and cross-attention workloads, beside
# the bf16 forward on the same batch.
WORKLOADS["mx_selfattn_causal"] = Workload(
    "mx_selfattn_causal", 256, 4, 128, "bf16", 1.0, True, "softmax",
    ("lognormal", 256, 1024), None, True,
    "MXFP8 (E4M3, E8M0 block scales) jagged causal self-attention forward and backward, batch 256, log-normal "
    "lengths (median 256, max 1024), 4 heads, d 128, bf16 in and out", mx=True)
WORKLOADS["mx_cross_asym"] = Workload(
    "mx_cross_asym", 512, 8, 64, "bf16", 1.0, False, "softmax",
    ("uniform", 1, 64), ("lognormal", 1024, 4096), False,
    "MXFP8 (E4M3, E8M0 block scales) asymmetric jagged cross-attention forward, batch 512, query lengths "
    "U{1..64}, key lengths log-normal (median 1024, max 4096), 8 heads, d 64, bf16 in and out", mx=True)

ORDER = ["tiny_fp32", "selfattn_causal", "cross_asym", "gdpa_silu", "pareto_train"]


def draw_lengths(rng, law, n):
    """n sequence lengths from a length law; see the module docstring."""
    kind = law[0]
    if kind == "uniform":                       # integers in [lo, hi], both ends
        return rng.integers(law[1], law[2] + 1, size=n).astype(np.int64)
    if kind == "lognormal":                     # median, max; clipped to [1, max]
        median, hi = law[1], law[2]
        x = np.exp(math.log(median) + LOGNORMAL_SIGMA * rng.standard_normal(n))
        return np.clip(np.rint(x), 1, hi).astype(np.int64)
    if kind == "fixed":                         # every length equal
        return np.full(n, law[1], dtype=np.int64)
    if kind == "pareto":                        # Pareto type I, x_m, max, alpha
        xm, hi, alpha = law[1], law[2], law[3]
        u = 1.0 - rng.random(n)                 # uniform on (0, 1]
        return np.minimum(hi, np.floor(xm * u ** (-1.0 / alpha))).astype(np.int64)
    raise ValueError("unknown length law %r" % (kind,))


def offsets_from_lengths(lengths):
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits):
    """bf16 bit patterns -> exact float64 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclass
class Batch:
    """One drawn batch. Values are held twice: as the storage the GPU gets
    (bf16 bit patterns as uint16, or float32) and as exact float64 copies."""
    workload: Workload
    seed: int
    q_lengths: np.ndarray
    kv_lengths: np.ndarray
    q_offsets: np.ndarray   # int64 [B+1]
    kv_offsets: np.ndarray  # int64 [B+1]
    q: np.ndarray           # storage dtype, [T_q, H, d]
    k: np.ndarray
    v: np.ndarray
    dout: np.ndarray | None

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.workload.head_dim)

    def f64(self, name):
        arr = getattr(self, name)
        if self.workload.dtype == "bf16":
            return bf16_bits_to_f64(arr)
        return arr.astype(np.float64)


def _values(rng, n_rows, heads, d, std, dtype):
    x = rng.standard_normal((n_rows, heads, d), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_bits(x) if dtype == "bf16" else x


def make_batch(workload, seed, batch=None, q_lengths=None, kv_lengths=None, with_dout=None):
    """Draw one batch of a workload.

    ``batch`` overrides the number of sequences (reduced-size parity runs);
    explicit ``q_lengths`` / ``kv_lengths`` override the length laws (edge
    cases); ``with_dout`` defaults to whether the workload has a backward.
    """
    if isinstance(workload, str):
        workload = WORKLOADS[workload]
    rng = np.random.default_rng(seed)
    n = workload.batch if batch is None else batch
    if q_lengths is None:
        q_lengths = draw_lengths(rng, workload.q_law, n)
    else:
        q_lengths = np.asarray(q_lengths, dtype=np.int64)
    if kv_lengths is None:
        if workload.kv_law is None:
            kv_lengths = q_lengths.copy()
        else:
            kv_lengths = draw_lengths(rng, workload.kv_law, len(q_lengths))
    else:
        kv_lengths = np.asarray(kv_lengths, dtype=np.int64)
    qo, ko = offsets_from_lengths(q_lengths), offsets_from_lengths(kv_lengths)
    H, d, dt, std = workload.heads, workload.head_dim, workload.dtype, workload.std
    # pooled attention: q holds the n_seeds shared queries; the query offsets
    # (b * n_seeds) describe the pooled output rows
    q = _values(rng, workload.n_seeds if workload.n_seeds else int(qo[-1]), H, d, std, dt)
    k = _values(rng, int(ko[-1]), H, d, std, dt)
    v = _values(rng, int(ko[-1]), H, d, std, dt)
    if with_dout is None:
        with_dout = workload.backward
    dout = _values(rng, int(qo[-1]), H, d, 1.0, dt) if with_dout else None
    return Batch(workload, seed, q_lengths, kv_lengths, qo, ko, q, k, v, dout)
