#!/usr/bin/env python3
"""Throughput of jagged attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: the forward call
(work-list build + attention kernel) and the backward call (work-list
builds, softmax row statistics, dK/dV kernel -- which also stores the dS
blocks, and writes the dQ of sequences of at most 64 tokens -- and dQ
kernel).  Inputs are generated on the host, copied to HBM before timing,
and stay resident.

Timing: W untimed warm-up steps, then K timed steps (default 10 and 50).
Before each timed step a 512 MiB buffer is overwritten, which evicts L2 and
the last-level cache; each step is timed by its own HIP events (the flush
excluded) and the headline is the median step, with p10 and p90.  The same
K steps back to back (warm caches) are reported beside it, labelled.

Prints one JSON line: useful TFLOPS counted on the visible (query, key)
pairs of the real, unpadded tokens -- 4*d FLOPs per pair forward, 10*d
backward -- the forward and backward passes against their targets,
per-kernel durations (from untimed steps with an event between every two
launches), the roofline position of the dominant kernel (its algorithmic
bytes: the method's own tensors, each once; timed by two events inside the
timed steps), the mean over further seeds, and the CPU oracle timed on the
host's cores.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "useful TFLOPS (unpadded tokens) fwd/bwd + % of bf16 MFMA peak, 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS   # dense fp8 (and MX fp8) products: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# Device sources each kernel of a step is built from (beside the shared
# headers): stored counters stay valid while these are unchanged.
COMMON_SRC = ("jfa_common.hpp", "jfa_internal.h")
KERNEL_SRC = {"sched_q": ("sched.hip", "blocks.hip", "pooled.hip"), "fwd": ("fwd.hip",),
              "bwd_sched": ("sched.hip", "bwd_stats.hpp", "pooled.hip"), "bwd_stats": ("bwd.hip", "bwd_stats.hpp"),
              "bwd_dkdv": ("bwd.hip",), "bwd_dq": ("bwd.hip", "pooled.hip"), "mx_quant": ("mx.hip",),
              "mx_fwd": ("mx.hip", "mx_common.hpp"), "mx_bwd_dkdv": ("mx_bwd.hip", "mx_common.hpp"),
              "mx_bwd_dq": ("mx_bwd.hip", "mx_common.hpp")}


def kernel_source_digest(kernel=None):
    """Digest of the device sources of `kernel` (a key of KERNEL_SRC) and
    the shared headers, or of every device source (None): tells whether
    stored counters still apply (the host-side C ABI layer is left out)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "jagged_attention_ads_amd", "csrc")
    names = sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".hpp", ".h")))
    if kernel is not None:
        names = sorted(set(COMMON_SRC) | set(KERNEL_SRC[kernel]))
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """Minimal hipEvent_t wrapper over the HIP runtime (timing only)."""

    def __init__(self):
        # the HIP runtime already in the process (torch's), never a second copy
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("no HIP runtime loaded")
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h.value
        return arr

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def destroy(self, arr):
        for h in arr:
            self.lib.hipEventDestroy(h)


def block_runs(lengths, block):
    """Lengths of the `block`-token runs of every sequence, in order
    (BlockAttention: each run attends within itself)."""
    out = []
    for n in np.asarray(lengths, dtype=np.int64):
        out += [block] * int(n // block) + ([int(n % block)] if n % block else [])
    return np.asarray(out, dtype=np.int64)


def visible_pairs(q_lengths, kv_lengths, causal):
    """Per sequence, the number of (query, key) pairs that are visible."""
    lq = np.asarray(q_lengths, dtype=np.int64)
    lk = np.asarray(kv_lengths, dtype=np.int64)
    if not causal:
        return lq * lk
    out = np.zeros_like(lq)
    for b in range(len(lq)):
        i = np.arange(lq[b])
        out[b] = np.clip(i + lk[b] - lq[b] + 1, 0, lk[b]).sum()
    return out


def ds_blocks(q_lengths, kv_lengths, causal, blk=32):
    """Number of 32 x 32 dS blocks that hold a visible pair (the blocks the
    dK/dV pass stores and the dQ pass reads), over all sequences, per head."""
    n = 0
    for lq, lk in zip(np.asarray(q_lengths, np.int64), np.asarray(kv_lengths, np.int64)):
        if lq <= 0 or lk <= 0:
            continue
        last = np.minimum(np.arange(blk, lq + blk, blk), lq) - 1   # last row of each query block
        kv_end = np.minimum(lk, last + (lk - lq) + 1) if causal else np.full(len(last), lk)
        n += int(np.sum(-(-np.maximum(kv_end, 0) // blk)))
    return n


def short_split(q_lengths, kv_lengths, causal):
    """(query rows, key rows, visible pairs, dS blocks) of the short
    sequences -- at most 64 queries and 1 .. 64 keys -- whose dQ the dK/dV
    pass writes itself, so that the dQ pass skips them."""
    lq = np.asarray(q_lengths, dtype=np.int64)
    lk = np.asarray(kv_lengths, dtype=np.int64)
    m = (lq <= 64) & (lk >= 1) & (lk <= 64)
    return (int(lq[m].sum()), int(lk[m].sum()), int(visible_pairs(lq[m], lk[m], causal).sum()),
            ds_blocks(lq[m], lk[m], causal))


def kernel_accounting(wl, T_q, T_k, pairs_total, n_ds_blocks, ds_path, short=(0, 0, 0, 0)):
    """Algorithmic FLOPs (the products each kernel must execute per visible
    pair) and algorithmic bytes per launch: the method's own tensors the
    kernel's step touches, each once -- Q, K, V, O, dO, dQ, dK, dV, lse and
    delta.  Re-reads and the library's own intermediates are not algorithmic:
    the dS blocks that the dK/dV pass stores and the dQ pass reads back are
    reported apart, as `ds_store_bytes` (workspace traffic, once each way).
    `short` is short_split of the sequences whose dQ the dK/dV pass forms
    (all zeros when it forms none): their dS stays on chip, and the dQ pass
    does not touch them."""
    H, d = wl.heads, wl.head_dim
    es = 2 if wl.dtype == "bf16" else 4
    sq, sk, sp, sb = short
    q_bytes, k_bytes = T_q * H * d * es, T_k * H * d * es
    lq_bytes, lk_bytes = (T_q - sq) * H * d * es, (T_k - sk) * H * d * es   # sequences the dQ pass takes
    row_f32 = T_q * H * 4
    soft = wl.activation == "softmax"
    ds_bytes = (n_ds_blocks - sb) * H * 32 * 32 * es if ds_path else 0
    acc = {
        # reads Q, K, V; writes O (and lse)
        "fwd": dict(flops=4 * d * H * pairs_total,
                    bytes=q_bytes + 2 * k_bytes + q_bytes + (row_f32 if soft else 0)),
        # reads Q, dO, K, V (and lse, delta); writes dK, dV and the short
        # sequences' dQ
        "bwd_dkdv": dict(flops=8 * d * H * pairs_total + 2 * d * H * sp,
                         bytes=2 * q_bytes + 2 * k_bytes + (2 * row_f32 if soft else 0) + 2 * k_bytes
                         + sq * H * d * es,
                         ds_store_bytes=ds_bytes),
    }
    if ds_path:   # dQ = scale * dS K: reads K, writes dQ (plus the dS blocks: workspace)
        acc["bwd_dq"] = dict(flops=2 * d * H * (pairs_total - sp), bytes=lk_bytes + lq_bytes,
                             ds_store_bytes=ds_bytes)
    else:         # recomputes S, P, dP, dS: reads Q, dO, K, V, lse, delta, writes dQ
        acc["bwd_dq"] = dict(flops=6 * d * H * (pairs_total - sp),
                             bytes=3 * lq_bytes + 2 * lk_bytes + (2 * (T_q - sq) * H * 4 if soft else 0))
    if soft:      # reads O, dO and lse, writes delta (and lse in log2 units)
        acc["bwd_stats"] = dict(flops=2 * d * H * T_q, bytes=2 * q_bytes + 3 * row_f32)
    if wl.mx:
        # MXFP8: the quantisation reads Q, K, V (bf16) and writes their images
        # (a byte per element plus a scale byte per 32); the attention reads
        # the images and writes O (bf16) and lse.  The backward's images:
        # Q, dO along the head dimension and along queries, K along the head
        # dimension and along keys, V along the head dimension (its
        # quantisation reads Q, K, V, dO in bf16 and writes the seven); the
        # dK/dV pass reads the Q and dO images of both kinds, the K and V
        # rows, lse and delta and writes dK, dV; the dQ pass reads the Q and
        # dO rows, the three K and V images, lse and delta and writes dQ
        img = lambda rows: rows * H * d * (1 + 1.0 / 32)   # noqa: E731
        acc = {"mx_quant": dict(flops=0, bytes=(T_q + 2 * T_k) * H * d * 2 + img(T_q) + 2 * img(T_k)),
               "fwd": dict(flops=4 * d * H * pairs_total, bytes=img(T_q) + 2 * img(T_k) + T_q * H * d * 2 + row_f32),
               "mx_quant_bwd": dict(flops=0, bytes=(2 * T_q + 2 * T_k) * H * d * 2 + 4 * img(T_q) + 3 * img(T_k)),
               "bwd_sched": dict(flops=2 * d * H * T_q, bytes=2 * q_bytes + 3 * row_f32),
               "bwd_dkdv": dict(flops=8 * d * H * pairs_total, bytes=4 * img(T_q) + 2 * img(T_k) + 2 * row_f32
                                + 2 * k_bytes),
               "bwd_dq": dict(flops=6 * d * H * pairs_total, bytes=2 * img(T_q) + 3 * img(T_k) + 2 * row_f32 + q_bytes)}
    return acc


def stored_traffic(kernel, digest, workload):
    """HBM bytes per launch of `kernel` on `workload` from the stored counter
    runs (profiles/traffic.json), or None when none were taken with the
    current device sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get("workloads", {}).get(workload, {}).get(kernel)
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers():
    """Worker processes of the CPU baseline: every core this process may run
    on, at most 16 (a GPU's share of the host on the boxes this runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# The batch the CPU-baseline workers read: set in the parent before the pool
# forks, so that every worker sees it without a copy.
_CPU_BATCH = {}


def _cpu_worker_init():
    # single-threaded BLAS in every worker: the pool provides the parallelism
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _cpu_unit(arg):
    """One (sequence, head) unit of the oracle: forward, or forward and
    backward; returns its useful FLOPs."""
    import oracle
    b, h, with_bwd = arg
    c = _CPU_BATCH
    qo, ko, blk = c["qo"], c["ko"], c["block"]
    sq, sk = slice(qo[b], qo[b + 1]), slice(ko[b], ko[b + 1])
    one_q, one_k = np.array([0, qo[b + 1] - qo[b]]), np.array([0, ko[b + 1] - ko[b]])
    hs = slice(h, h + 1)
    if c["pooled"]:   # the shared seeds against sequence b's keys
        k, v = c["k"][sk, hs], c["v"][sk, hs]
        oracle.pooled_fwd(c["q"][:, hs], k, v, one_k, c["scale"], c["act"])
        if with_bwd:
            oracle.pooled_bwd(c["q"][:, hs], k, v, c["do"][sq, hs], one_k, c["scale"], c["act"])
        return (14 if with_bwd else 4) * c["d"] * c["pairs"][b]
    q, k, v = c["q"][sq, hs], c["k"][sk, hs], c["v"][sk, hs]
    if c["mx"]:   # MXFP8 (its column blocks start at each sequence: one sequence alone is the same)
        out, lse = oracle.mx_attention_fwd(q, k, v, one_q, one_k, c["scale"], c["causal"])
        if with_bwd:
            oracle.mx_attention_bwd(q, k, v, out, c["do"][sq, hs], lse, one_q, one_k, c["scale"], c["causal"])
        return (14 if with_bwd else 4) * c["d"] * c["pairs"][b]
    oracle.attention_fwd(q, k, v, one_q, one_k, c["scale"], c["act"], c["causal"], block=blk, rope_base=c["rope"])
    if with_bwd:
        oracle.attention_bwd(q, k, v, c["do"][sq, hs], one_q, one_k, c["scale"], c["act"], c["causal"], block=blk,
                             rope_base=c["rope"])
    return (14 if with_bwd else 4) * c["d"] * c["pairs"][b]


def cpu_baseline(batch, budget_s):
    """The CPU oracle, as it is, on the host: worker processes with
    single-threaded BLAS over (sequence, head) units handed out longest
    first, forward alone and forward + backward timed separately, plus the
    same on one core.  The sample is every s-th sequence of the batch, s
    chosen from a one-core calibration so that the pool runs about
    `budget_s` seconds; useful TFLOPS under the GPU's accounting.  Runs
    before anything touches the GPU (the pool forks this process)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits
    wl = batch.workload
    qo, ko = np.asarray(batch.q_offsets), np.asarray(batch.kv_offsets)
    blk = wl.block
    if blk:
        pairs = np.array([visible_pairs(block_runs([n], blk), block_runs([n], blk), wl.causal).sum()
                          for n in batch.q_lengths])
    else:
        pairs = visible_pairs(batch.q_lengths, batch.kv_lengths, wl.causal)
    _CPU_BATCH.update(q=batch.f64("q"), k=batch.f64("k"), v=batch.f64("v"),
                      do=batch.f64("dout") if batch.dout is not None else None, qo=qo, ko=ko, block=blk,
                      scale=1.0 / math.sqrt(wl.head_dim), act=wl.activation, causal=wl.causal, d=wl.head_dim,
                      pairs=pairs, rope=wl.rope_base or None, pooled=bool(wl.n_seeds), mx=wl.mx)
    B, H = len(pairs), wl.heads
    with_bwd = bool(wl.backward and batch.dout is not None)
    dense = (np.diff(qo) * np.diff(ko)).astype(np.float64)   # the oracle's work follows Lq * Lk
    order = np.argsort(-dense, kind="stable")
    workers = cpu_workers()

    def one_core(seqs, bwd):
        t0, f = time.perf_counter(), 0.0
        with threadpool_limits(1):
            for b in seqs:
                for h in range(H):
                    f += _cpu_unit((b, h, bwd))
        return f, time.perf_counter() - t0

    # one-core calibration on a spread of sequences (median-ish first)
    calib = [int(b) for b in order[len(order) // 2::max(1, B // 8)]][:8]
    _, t1 = one_core(calib, with_bwd)
    rate = dense[calib].sum() * H / max(t1, 1e-9)   # dense pairs per second on one core
    total_s = dense.sum() * H / rate / workers        # the whole batch on the pool
    stride = max(1, int(math.ceil(total_s / (0.45 * budget_s))))
    sample = [b for b in order if b % stride == 0]
    ctx = mp.get_context("fork")
    res = {}
    for name, bwd in (("fwd", False), ("fwd_bwd", True)):
        if bwd and not with_bwd:
            continue
        units = [(int(b), h, bwd) for b in sample for h in range(H)]   # longest first
        with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
            t0 = time.perf_counter()
            flops = float(sum(pool.imap_unordered(_cpu_unit, units, chunksize=1)))
            el = time.perf_counter() - t0
        res[name] = (flops, el)
    # one core, on a sub-sample of the sample sized to about 0.15 * budget_s
    # (fwd + bwd where it runs)
    one_core_s = dense[sample].sum() * H / rate
    sub = sample[::max(1, int(math.ceil(one_core_s / (0.15 * budget_s))))] or sample[:1]
    fo, to = one_core(sub, with_bwd)
    key = "fwd_bwd" if with_bwd else "fwd"
    flops, el = res[key]
    _CPU_BATCH.clear()
    return {
        "value": flops / el / 1e12, "unit": "TFLOPS", "cores": workers, "kind": "oracle",
        "sample": "fp64 NumPy oracle%s, %s, every %d-th sequence of the same batch (%d of %d sequences x %d heads, "
                  "%.3g useful GFLOP, %.1f s); %d worker processes with single-threaded BLAS, (sequence, head) "
                  "units longest first" % (" (MXFP8)" if wl.mx else "", "fwd+bwd" if with_bwd else "fwd", stride, len(sample), B, H,
                                           flops / 1e9, el, workers),
        "cpu_model": cpu_model(),
        "fwd_tflops": res["fwd"][0] / res["fwd"][1] / 1e12,
        "fwd_bwd_tflops": (res["fwd_bwd"][0] / res["fwd_bwd"][1] / 1e12) if with_bwd else None,
        "one_core_tflops": fo / to / 1e12,
        "one_core_sample": "%s on %d sequences x %d heads (%.1f s)" % ("fwd+bwd" if with_bwd else "fwd", len(sub),
                                                                       H, to),
    }


COPY_BYTES = 256 << 20


def calibrate_copy():
    """One elementwise kernel per dispatch that reads and writes COPY_BYTES:
    what a perfect kernel's FETCH_SIZE / WRITE_SIZE read for that traffic."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "dispatches": 3}))


def pctl(xs, p):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), p))


class Runner:
    """One batch on the device with its outputs, workspaces and the two
    library calls of a step (through the C ABI's profiled entry points, which
    record caller events between launches)."""

    def __init__(self, wl, batch, dev, mx_mode="attend"):
        import torch
        from jagged_attention_ads_amd import jfa
        self.torch, self.jfa = torch, jfa
        self.wl, self.batch = wl, batch
        T_q, T_k, H, D = int(batch.q_offsets[-1]), int(batch.kv_offsets[-1]), wl.heads, wl.head_dim
        self.T_q, self.T_k, self.H, self.D = T_q, T_k, H, D

        def to_dev(a):
            if wl.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)
        self.q, self.k, self.v, self.do = (to_dev(x) for x in (batch.q, batch.k, batch.v, batch.dout))
        qo = torch.from_numpy(batch.q_offsets.astype(np.int32)).to(dev)
        ko = torch.from_numpy(batch.kv_offsets.astype(np.int32)).to(dev)
        mq, mk = int(batch.q_lengths.max()), int(batch.kv_lengths.max())
        self.scale = 1.0 / math.sqrt(D)
        # pooled attention: q holds the shared seeds; the output has a row
        # per (sequence, seed)
        self.out = torch.empty((T_q, H, D), dtype=self.q.dtype, device=dev)
        self.lse = torch.empty((H, T_q), dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        B = len(batch.q_lengths)
        L = self.L = jfa.lib()
        P = self.P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.derive = None
        self.q_lens, self.kv_lens = batch.q_lengths, batch.kv_lengths
        self.seq_off, self.n_seq = qo, B
        if wl.block and wl.rope_base:
            # BlockAttention with the fused rotary embedding: the block calls
            # derive the runs' offsets themselves (between events 0 and 1)
            self.q_lens = self.kv_lens = block_runs(batch.q_lengths, wl.block)
        elif wl.block:
            # BlockAttention: the runs of wl.block tokens as sequences, derived
            # on the device from the sequences' offsets in every step
            seq_off, n_seq = qo, B
            n_runs = L.jfa_block_offsets_count(n_seq, T_q, wl.block)
            runs = torch.empty(n_runs, dtype=torch.int32, device=dev)

            def derive():
                st = L.jfa_block_offsets(P(seq_off), n_seq, T_q, wl.block, P(runs), n_runs, self.stream)
                if st != 0:
                    raise jfa.JfaError(st, L.jfa_last_error().decode())
            self.derive = derive
            qo = ko = runs
            B = n_runs - 1
            mq = mk = min(wl.block, mq)
            self.q_lens = self.kv_lens = block_runs(batch.q_lengths, wl.block)
        self.qo, self.ko, self.B, self.mq, self.mk = qo, ko, B, mq, mk
        # the forward call's event slots: its kernels between consecutive
        # slots, its end at the last
        # MXFP8: "attend" takes the operands as MX images, resident like
        # any input (the pages fuse the quantisation into the producing
        # norm / projection kernels); "forward" takes bf16 and quantises
        # them first (jfa_mx_forward)
        self.mx_mode = mx_mode if wl.mx else None
        self.fwd_slots = {"sched_q": (0, 1), "fwd": (1, 2)}
        if self.mx_mode == "forward":
            self.fwd_slots = {"mx_quant": (0, 1), "sched_q": (1, 2), "fwd": (2, 3)}
        self.nf = max(b for _, b in self.fwd_slots.values()) + 1
        self.fwd_end = self.nf - 1
        # the backward call's event slots likewise (the list launch forms the
        # row statistics: "bwd_stats" is empty unless a kernel of its own runs)
        self.bwd_slots = {"bwd_sched": (0, 1), "bwd_stats": (1, 2), "bwd_dkdv": (2, 3), "bwd_dq": (3, 4)}
        if self.mx_mode == "attend":
            self.bwd_slots = {"bwd_sched": (0, 1), "bwd_dkdv": (1, 2), "bwd_dq": (2, 3)}
        elif self.mx_mode == "forward":
            self.bwd_slots = {"mx_quant_bwd": (0, 1), "bwd_sched": (1, 2), "bwd_dkdv": (2, 3), "bwd_dq": (3, 4)}
        self.nb = max(b for _, b in self.bwd_slots.values()) + 1
        self.bwd_end = self.nb - 1
        if wl.mx:
            self.ws_f = torch.empty(max(L.jfa_mx_workspace_size(B, H, D, T_q, T_k, int(mx_mode == "forward")), 1),
                                    dtype=torch.uint8, device=dev)
            self.ws_b = torch.empty(max(L.jfa_mx_backward_workspace_size(B, H, D, T_q, T_k,
                                                                         int(mx_mode == "forward")), 1),
                                    dtype=torch.uint8, device=dev)
            if mx_mode == "attend":
                # the operands as their producers would hand them over: the
                # forward's Q, K rows and V columns; the backward's seven
                self.images = [jfa.mx_quantize(t, o, lay) for t, o, lay in
                               ((self.q, qo, "rows"), (self.k, ko, "rows"), (self.v, ko, "keys"))]
                src = {"q": (self.q, qo), "k": (self.k, ko), "v": (self.v, ko), "dout": (self.do, qo)}
                self.bwd_images = [self.images[0] if (t, lay) == ("q", "rows") else
                                   self.images[1] if (t, lay) == ("k", "rows") else
                                   jfa.mx_quantize(src[t][0], src[t][1], lay) for t, lay in jfa.MX_BACKWARD_IMAGES]
                self.bwd_image_ptrs = (ctypes.c_void_p * len(self.bwd_images))(
                    *[x.data_ptr() for x in self.bwd_images])
                torch.cuda.synchronize()
        elif wl.n_seeds:
            dtc = jfa.DTYPES[self.q.dtype]
            self.ws_f = torch.empty(L.jfa_pooled_workspace_size(B, wl.n_seeds, H, D, T_k, mk, dtc, 0),
                                    dtype=torch.uint8, device=dev)
            self.ws_b = torch.empty(L.jfa_pooled_workspace_size(B, wl.n_seeds, H, D, T_k, mk, dtc, 1),
                                    dtype=torch.uint8, device=dev)
        elif wl.block and wl.rope_base:
            dtc = jfa.DTYPES[self.q.dtype]
            self.ws_f = torch.empty(L.jfa_block_workspace_size(B, H, D, T_q, wl.block, dtc, 0), dtype=torch.uint8,
                                    device=dev)
            self.ws_b = torch.empty(L.jfa_block_workspace_size(B, H, D, T_q, wl.block, dtc, 1), dtype=torch.uint8,
                                    device=dev)
            self.B = int(L.jfa_block_offsets_count(B, T_q, wl.block)) - 1   # the runs, for reporting
        else:
            self.ws_f = jfa.workspace(B, H, D, T_q, T_k, mk, self.q.dtype, False, dev)
            self.ws_b = jfa.workspace(B, H, D, T_q, T_k, mk, self.q.dtype, True, dev)
        # the dK/dV pass stores dS and the dQ pass reads it, unless switched
        # off or the store was left out of the workspace
        self.ds_path = (not wl.rope_base and not wl.n_seeds and not wl.mx and L.jfa_get_option(1) != 0
                        and self.ws_b.numel() > jfa.jfa_workspace_size(B, H, D, T_q, T_k, mk, self.q.dtype, 2))
        # the dK/dV pass writes the dQ of short sequences (bf16, d 64 or 128:
        # where its LDS has room) when every sequence is short, or always with
        # the option bwd_short_dq on; never with it off
        fuse_opt = L.jfa_get_option(2)
        self.fuse_short = (wl.dtype == "bf16" and D in (64, 128)
                           and (bool(wl.rope_base) or (fuse_opt != 0 and (fuse_opt == 1 or max(mq, mk) <= 64))))
        self.act = jfa.ACTIVATIONS[wl.activation]
        self.dt = jfa.DTYPES[self.q.dtype]
        self.lse_arg = self.lse if wl.activation == "softmax" else None
        self.run_bwd = wl.backward

    def slots(self, name):
        """(side, first event, second event) around kernel `name`."""
        if name in self.fwd_slots:
            return (0,) + self.fwd_slots[name]
        return (1,) + self.bwd_slots[name]

    def fwd(self, events):
        ev = ctypes.cast(events, ctypes.c_void_p) if events is not None else None
        if self.mx_mode == "attend":
            qi, ki, vi = self.images
            st = self.L.jfa_mx_attend(
                self.P(qi), self.P(ki), self.P(vi), self.P(self.qo), self.P(self.ko), self.B, self.H,
                self.D, self.T_q, self.T_k, self.mq, self.mk, self.scale, int(self.wl.causal), self.P(self.out),
                self.P(self.lse), self.P(self.ws_f), self.ws_f.numel(), self.stream, ev)
            if st != 0:
                raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())
            return
        if self.mx_mode == "forward":
            st = self.L.jfa_mx_forward(
                self.P(self.q), self.P(self.k), self.P(self.v), self.P(self.qo), self.P(self.ko), self.B, self.H,
                self.D, self.T_q, self.T_k, self.mq, self.mk, self.scale, int(self.wl.causal), self.P(self.out),
                self.P(self.lse), self.P(self.ws_f), self.ws_f.numel(), self.stream, ev)
            if st != 0:
                raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())
            return
        if self.wl.n_seeds:
            st = self.L.jfa_pooled_forward(
                self.P(self.q), self.P(self.k), self.P(self.v), self.P(self.ko), self.B, self.wl.n_seeds, self.H,
                self.D, self.T_k, self.mk, self.scale, self.act, self.dt, self.P(self.out), self.P(self.lse_arg),
                self.P(self.ws_f), self.ws_f.numel(), self.stream, ev)
            if st != 0:
                raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())
            return
        if self.wl.rope_base:
            st = self.L.jfa_block_forward(
                self.P(self.q), self.P(self.k), self.P(self.v), self.P(self.seq_off), self.n_seq, self.H, self.D,
                self.T_q, int(self.batch.q_lengths.max()), self.wl.block, self.scale, self.act, int(self.wl.causal),
                self.dt, self.wl.rope_base, self.P(self.out), self.P(self.lse_arg), self.P(self.ws_f),
                self.ws_f.numel(), self.stream, ev)
            if st != 0:
                raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())
            return
        st = self.L.jfa_forward_profiled(
            self.P(self.q), self.P(self.k), self.P(self.v), self.P(self.qo), self.P(self.ko), self.B, self.H,
            self.D, self.T_q, self.T_k, self.mq, self.mk, self.scale, self.act, int(self.wl.causal), self.dt,
            self.P(self.out), self.P(self.lse_arg), self.P(self.ws_f), self.ws_f.numel(), self.stream,
            ctypes.cast(events, ctypes.c_void_p) if events is not None else None)
        if st != 0:
            raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())

    def bwd(self, events):
        ev = ctypes.cast(events, ctypes.c_void_p) if events is not None else None
        if self.mx_mode == "attend":
            st = self.L.jfa_mx_backward_images(
                self.bwd_image_ptrs, self.P(self.out), self.P(self.do), self.P(self.lse), self.P(self.qo),
                self.P(self.ko), self.B, self.H, self.D, self.T_q, self.T_k, self.mq, self.mk, self.scale,
                int(self.wl.causal), self.P(self.dq), self.P(self.dk), self.P(self.dv), self.P(self.ws_b),
                self.ws_b.numel(), self.stream, ev)
            if st != 0:
                raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())
            return
        if self.mx_mode == "forward":
            st = self.L.jfa_mx_backward(
                self.P(self.q), self.P(self.k), self.P(self.v), self.P(self.out), self.P(self.do), self.P(self.lse),
                self.P(self.qo), self.P(self.ko), self.B, self.H, self.D, self.T_q, self.T_k, self.mq, self.mk,
                self.scale, int(self.wl.causal), self.P(self.dq), self.P(self.dk), self.P(self.dv), self.P(self.ws_b),
                self.ws_b.numel(), self.stream, ev)
            if st != 0:
                raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())
            return
        if self.wl.n_seeds:
            st = self.L.jfa_pooled_backward(
                self.P(self.q), self.P(self.k), self.P(self.v), self.P(self.out), self.P(self.do),
                self.P(self.lse_arg), self.P(self.ko), self.B, self.wl.n_seeds, self.H, self.D, self.T_k, self.mk,
                self.scale, self.act, self.dt, self.P(self.dq), self.P(self.dk), self.P(self.dv), self.P(self.ws_b),
                self.ws_b.numel(), self.stream, ev)
            if st != 0:
                raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())
            return
        if self.wl.rope_base:
            st = self.L.jfa_block_backward(
                self.P(self.q), self.P(self.k), self.P(self.v), self.P(self.out), self.P(self.do),
                self.P(self.lse_arg), self.P(self.seq_off), self.n_seq, self.H, self.D, self.T_q,
                int(self.batch.q_lengths.max()), self.wl.block, self.scale, self.act, int(self.wl.causal), self.dt,
                self.wl.rope_base, self.P(self.dq), self.P(self.dk), self.P(self.dv), self.P(self.ws_b),
                self.ws_b.numel(), self.stream, ev)
            if st != 0:
                raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())
            return
        st = self.L.jfa_backward_profiled(
            self.P(self.q), self.P(self.k), self.P(self.v), self.P(self.out), self.P(self.do),
            self.P(self.lse_arg), self.P(self.qo), self.P(self.ko), self.B, self.H, self.D, self.T_q, self.T_k,
            self.mq, self.mk, self.scale, self.act, int(self.wl.causal), self.dt, self.P(self.dq), self.P(self.dk),
            self.P(self.dv), self.P(self.ws_b), self.ws_b.numel(), self.stream,
            ctypes.cast(events, ctypes.c_void_p) if events is not None else None)
        if st != 0:
            raise self.jfa.JfaError(st, self.L.jfa_last_error().decode())

    def step(self, ef=None, eb=None):
        if self.derive:
            self.derive()
        self.fwd(ef)
        if self.run_bwd:
            self.bwd(eb)

    def pairs(self):
        return int(visible_pairs(self.q_lens, self.kv_lens, self.wl.causal).sum())


def timed_steps(r, ev, K, flush_buf, dom=None):
    """K steps, each timed by its own events (with flush_buf, the buffer is
    overwritten before each step, outside its events), bracketed by a
    synchronisation on both sides.  Events per step: the forward's start,
    the backward's start, the backward's end (the forward's end for a
    forward-only workload); `dom` = (side, i0, i1) adds the two events around
    that kernel (side 0: the forward's event slots, 1: the backward's).
    Returns per-step lists of milliseconds: step, fwd, bwd, dominant kernel,
    and the whole timed region."""
    nf, nb = r.nf, r.nb
    evs = []
    for _ in range(K):
        ef, eb = (ctypes.c_void_p * nf)(), (ctypes.c_void_p * nb)()
        made = ev.create(5)
        ef[0] = made[0]
        if r.run_bwd:
            eb[0], eb[r.bwd_end] = made[1], made[2]
        else:
            ef[r.fwd_end] = made[2]
        if dom is not None:
            arr = ef if dom[0] == 0 else eb
            # the two slots may coincide with the step events (e.g. forward-only)
            arr[dom[1]] = arr[dom[1]] or made[3]
            arr[dom[2]] = arr[dom[2]] or made[4]
        evs.append((ef, eb, made))
    edge = ev.create(2)
    r.torch.cuda.synchronize()
    ev.lib.hipEventRecord(edge[0], r.stream)
    for i in range(K):
        if flush_buf is not None:
            flush_buf.fill_(i & 0xff)
        ef, eb, _ = evs[i]
        r.step(ef, eb if r.run_bwd else None)
    ev.lib.hipEventRecord(edge[1], r.stream)
    r.torch.cuda.synchronize()
    out = {"step": [], "fwd": [], "bwd": [], "dom": [], "region": ev.ms(edge[0], edge[1])}
    for ef, eb, made in evs:
        end = eb[r.bwd_end] if r.run_bwd else ef[r.fwd_end]
        out["step"].append(ev.ms(ef[0], end))
        if r.run_bwd:
            out["fwd"].append(ev.ms(ef[0], eb[0]))
            out["bwd"].append(ev.ms(eb[0], eb[r.bwd_end]))
        else:
            out["fwd"].append(ev.ms(ef[0], ef[r.fwd_end]))
        if dom is not None:
            arr = ef if dom[0] == 0 else eb
            out["dom"].append(ev.ms(arr[dom[1]], arr[dom[2]]))
        ev.destroy(made)
    ev.destroy(edge)
    return out


def kernel_breakdown(r, ev, K, flush_buf):
    """Mean per-kernel milliseconds from K steps with an event between every
    two launches (each event adds a few microseconds between launches, so
    these steps are not the timed ones)."""
    ef = [ev.create(r.nf) for _ in range(K)]
    eb = [ev.create(r.nb) for _ in range(K)] if r.run_bwd else []
    r.torch.cuda.synchronize()
    for i in range(K):
        if flush_buf is not None:
            flush_buf.fill_(i & 0xff)
        r.step(ef[i], eb[i] if r.run_bwd else None)
    r.torch.cuda.synchronize()

    def avg(lst, a, b):
        return float(np.mean([ev.ms(e[a], e[b]) for e in lst])) if lst else 0.0
    kern = {n: avg(ef, a, b) for n, (a, b) in r.fwd_slots.items()}
    if r.run_bwd:
        kern.update({n: avg(eb, a, b) for n, (a, b) in r.bwd_slots.items()})
    for e in ef + eb:
        ev.destroy(e)
    return kern


def bbs_study(args):
    """Base Batch Shuffling against plain consecutive batches, one GPU
    standing in for R ranks.  The samples of each rank's pool are drawn from
    the workload's length law; a rank's step takes two base batches of 128
    samples: the next two in order (plain), or the rank's BBS merged batch
    (jfa_bbs_plan over its own pool: no exchange between ranks).  Every
    merged batch's forward + backward is timed on the GPU (median of its
    flushed repetitions); a synchronous step lasts as long as its slowest
    rank.  Prints one JSON line."""
    import torch
    from jagged_attention_ads_amd import jfa
    from jagged_attention_ads_amd.workloads import WORKLOADS, draw_lengths
    wl = WORKLOADS[args.workload]
    R, S, base = args.ranks, args.bbs_steps, 128
    rng = np.random.default_rng(args.seed)
    pools = [draw_lengths(rng, wl.q_law, S * 2 * base).astype(np.int32) for _ in range(R)]
    plans = {"plain": [], "bbs": []}
    t0 = time.perf_counter()
    for pool in pools:
        perm, start = jfa.jfa_bbs_plan(pool, base, args.bbs_cost)
        plans["bbs"].append([pool[perm[start[i]:start[i + 1]]] for i in range(len(start) - 1)])
        plans["plain"].append([pool[2 * base * i:2 * base * (i + 1)] for i in range(S)])
    plan_us = (time.perf_counter() - t0) / R * 1e6
    dev = torch.device("cuda:0")
    H, D = wl.heads, wl.head_dim
    t_max = max(int(b.sum()) for p in plans.values() for rk in p for b in rk)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q, k, v, do = (torch.randn((t_max, H, D), device=dev).to(dt) * wl.std for _ in range(4))
    ev = HipEvents()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = jfa.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731

    def time_batch(lengths):
        T = int(lengths.sum())
        off = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).to(dev)
        B, mq = len(lengths), int(lengths.max())
        qs, ks, vs, dos = q[:T], k[:T], v[:T], do[:T]
        out, dq, dk, dv = (torch.empty_like(qs) for _ in range(4))
        lse = torch.empty((H, T), dtype=torch.float32, device=dev)
        wf = jfa.workspace(B, H, D, T, T, mq, dt, False, dev)
        wb = jfa.workspace(B, H, D, T, T, mq, dt, True, dev)
        act, sc = jfa.ACTIVATIONS[wl.activation], 1.0 / math.sqrt(D)
        lse_arg = lse if wl.activation == "softmax" else None

        def step():
            st = L.jfa_forward(P(qs), P(ks), P(vs), P(off), P(off), B, H, D, T, T, mq, mq, sc, act, int(wl.causal),
                               jfa.DTYPES[dt], P(out), P(lse_arg), P(wf), wf.numel(), stream)
            st |= L.jfa_backward(P(qs), P(ks), P(vs), P(out), P(dos), P(lse_arg), P(off), P(off), B, H, D, T, T, mq,
                                 mq, sc, act, int(wl.causal), jfa.DTYPES[dt], P(dq), P(dk), P(dv), P(wb),
                                 wb.numel(), stream)
            if st != 0:
                raise jfa.JfaError(st, L.jfa_last_error().decode())
        step()
        e = ev.create(2 * args.bbs_reps)
        for i in range(args.bbs_reps):
            flush.fill_(i & 0xff)
            ev.lib.hipEventRecord(e[2 * i], stream)
            step()
            ev.lib.hipEventRecord(e[2 * i + 1], stream)
        torch.cuda.synchronize()
        ms = float(np.median([ev.ms(e[2 * i], e[2 * i + 1]) for i in range(args.bbs_reps)]))
        ev.destroy(e)
        return ms

    res = {"study": "base batch shuffling", "workload": wl.description, "ranks": R, "steps": S,
           "base_batch": base, "cost": args.bbs_cost, "seed": args.seed, "plan_us_per_rank_pool": plan_us,
           "timing": "per merged batch: forward + backward, median of %d flushed repetitions" % args.bbs_reps}
    for name, plan in plans.items():
        t = np.array([[time_batch(plan[r][s]) for s in range(S)] for r in range(R)])   # [rank, step]
        work = np.array([[int((plan[r][s].astype(np.int64) ** 2).sum()) for s in range(S)] for r in range(R)])
        step = t.max(axis=0)
        res[name] = {"sync_step_ms_mean": float(step.mean()), "rank_ms_mean": float(t.mean()),
                     "spread_across_ranks": float(np.mean((t.max(0) - t.min(0)) / t.mean(0))),
                     "idle_frac": float(np.mean(1.0 - t.mean(0) / step)),
                     "work_spread_across_ranks": float(np.mean((work.max(0) - work.min(0)) / work.mean(0)))}
    res["sync_step_speedup"] = res["plain"]["sync_step_ms_mean"] / res["bbs"]["sync_step_ms_mean"]
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="selfattn_causal")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--seed-mean", default="11-15",
                    help="seeds a-b of the same workload whose flushed median steps are averaged ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true",
                    help="headline from warm steps (no flush before each step); the default flushes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain elementwise copy of known size (256 MiB read + 256 MiB written per "
                         "dispatch, 3 dispatches), to scale the HBM byte counters")
    ap.add_argument("--study", choices=["bbs"], default=None,
                    help="bbs: Base Batch Shuffling against plain batches (its own JSON line, not the headline)")
    ap.add_argument("--ranks", type=int, default=8)
    ap.add_argument("--bbs-steps", type=int, default=6)
    ap.add_argument("--bbs-reps", type=int, default=5)
    ap.add_argument("--bbs-cost", choices=["tokens", "pairs"], default="tokens")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.study == "bbs":
        bbs_study(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences are independent; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch
    wl = WORKLOADS[args.workload]
    batch = make_batch(wl, args.seed, with_dout=True)
    # the CPU oracle first: its worker pool forks this process, which must
    # not have touched the GPU yet
    cpu = None if args.no_cpu_baseline else cpu_baseline(batch, args.cpu_seconds)

    import torch
    dev = torch.device("cuda:0")
    r = Runner(wl, batch, dev)
    ev = HipEvents()
    flush_buf = None if args.warm else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    warm_buf = None
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()
    K = args.steps

    # per-kernel breakdown (untimed steps, flushed like the headline)
    kern_ms = kernel_breakdown(r, ev, K, flush_buf)
    pairs = r.pairs()
    n_blk = ds_blocks(r.q_lens, r.kv_lens, wl.causal) if r.run_bwd else 0
    short = short_split(r.q_lens, r.kv_lens, wl.causal) if r.run_bwd and r.fuse_short else (0, 0, 0, 0)
    acct = kernel_accounting(wl, r.T_q, r.T_k, pairs, n_blk, r.ds_path, short)
    name = max((n for n in acct if n in kern_ms), key=lambda n: kern_ms[n])   # the dominant kernel

    # the timed steps: headline (flushed unless --warm), then the same warm
    t = timed_steps(r, ev, K, flush_buf, r.slots(name))
    t_warm = timed_steps(r, ev, K, warm_buf) if flush_buf is not None else None
    ms_step = float(np.median(t["step"]))
    D, H = r.D, r.H
    useful_fwd = 4.0 * D * H * pairs
    useful_bwd = 10.0 * D * H * pairs if r.run_bwd else 0.0
    tf = lambda flops, ms: flops / (ms * 1e-3) / 1e12  # noqa: E731
    value = tf(useful_fwd + useful_bwd, ms_step)
    fwd_ms, bwd_ms = float(np.median(t["fwd"])), (float(np.median(t["bwd"])) if r.run_bwd else None)
    dom_ms = float(np.mean(t["dom"]))

    # roofline of the dominant kernel, timed inside the timed steps
    t_s = dom_ms * 1e-3
    a = acct[name]
    ai = a["flops"] / a["bytes"]
    mx_kernel = wl.mx and name in ("fwd", "bwd_dkdv", "bwd_dq")
    src_key = "mx_" + name if mx_kernel else name
    digest = kernel_source_digest(src_key)
    # the MXFP8 attention's products run at the fp8 rate
    peak_mfma = PEAK_FP8_TFLOPS if mx_kernel else PEAK_BF16_TFLOPS
    if ai < peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": a["bytes"] / t_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": a["flops"] / t_s / 1e12, "peak": peak_mfma, "unit": "TFLOP/s",
                "peak_dtype": "fp8 (MX E4M3)" if peak_mfma == PEAK_FP8_TFLOPS else "bf16"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(name, digest, wl.name)
    roof.update({
        "traffic_from": ("rocprofv3 FETCH_SIZE + WRITE_SIZE per dispatch, copy-scaled, stored in "
                         "profiles/traffic.json for these device sources (digest %s)" % digest)
                        if roof["traffic"] is not None else "no counters for the current device sources",
        "kernel": name, "avg_launch_us": dom_ms * 1e3,
        "algorithmic_bytes": a["bytes"], "algorithmic_flops": a["flops"], "arith_intensity": ai,
        "workspace_ds_bytes": a.get("ds_store_bytes", 0),
        "mfma_frac": a["flops"] / t_s / 1e12 / peak_mfma})

    def pass_summary(useful, ms, target):
        if ms is None:
            return None
        v = tf(useful, ms)
        return {"tflops": v, "pct_of_peak": 100.0 * v / PEAK_BF16_TFLOPS, "target_pct": target,
                "median_us": ms * 1e3}
    res = {
        "metric": METRIC, "value": value, "unit": "TFLOPS", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("mxfp8 (E4M3 operands, E8M0 block scales, fp32 accumulation; bf16 in and out)" if wl.mx
                  else wl.dtype),
        "data": "synthetic (seeded; lengths and values drawn per the workload recipe)",
        "config": {"workload": wl.description, "name": wl.name, "batch": r.B, "heads": H, "head_dim": D,
                   "causal": wl.causal, "activation": wl.activation, "seed": args.seed, "total_q_tokens": r.T_q,
                   "total_kv_tokens": r.T_k, "visible_pairs_per_head": pairs, "block": wl.block,
                   "bwd_dq_from_stored_ds": bool(r.run_bwd and r.ds_path),
                   "bwd_short_seqs_dq_in_dkdv": bool(r.run_bwd and r.fuse_short),
                   "useful_gflop_per_step": (useful_fwd + useful_bwd) / 1e9},
        "timing": ("median over %d steps, each flushed first (512 MiB written, evicting L2 and the last-level "
                   "cache), timed by its own HIP events" % K) if flush_buf is not None else
                  ("median over %d warm steps, each timed by its own HIP events" % K),
        "ms_p10": pctl(t["step"], 10), "ms_p90": pctl(t["step"], 90), "timed_region_ms": t["region"],
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "fwd": pass_summary(useful_fwd, fwd_ms, 40.0),
        "bwd": pass_summary(useful_bwd, bwd_ms, 30.0) if r.run_bwd else None,
        "kernel_us": {k_: v_ * 1e3 for k_, v_ in kern_ms.items()},
        "kernel_us_from": "mean of %d %s steps with an event between every two launches" % (
            K, "flushed" if flush_buf is not None else "warm"),
        "kernel_source_digest": digest, "kernel_sources": list(COMMON_SRC) + list(KERNEL_SRC[src_key]),
        "roofline": roof,
    }
    if wl.mx:
        # the bf16 path on the same batch, and the MXFP8 path from bf16
        # inputs (quantisation included), timed the same way: the pages quote
        # MXFP8's forward and backward gains over the 16-bit kernels
        res["fwd"]["pct_of_fp8_peak"] = 100.0 * res["fwd"]["tflops"] / PEAK_FP8_TFLOPS
        if r.run_bwd:
            res["bwd"]["pct_of_fp8_peak"] = 100.0 * res["bwd"]["tflops"] / PEAK_FP8_TFLOPS
        import dataclasses
        rb = Runner(dataclasses.replace(wl, mx=False), batch, dev)
        for _ in range(3):
            rb.step()
        tb = timed_steps(rb, ev, K, flush_buf)
        bf = float(np.median(tb["fwd"]))
        kb = kernel_breakdown(rb, ev, K, flush_buf)
        base = {"fwd_us": bf * 1e3, "fwd_tflops": tf(useful_fwd, bf), "mx_fwd_speedup": bf / fwd_ms,
                "mx_fwd_kernel_speedup": kb["fwd"] / kern_ms["fwd"],
                "kernel_us": {k_: v_ * 1e3 for k_, v_ in kb.items()}}
        if r.run_bwd:
            bb, bs = float(np.median(tb["bwd"])), float(np.median(tb["step"]))
            base.update({"bwd_us": bb * 1e3, "bwd_tflops": tf(useful_bwd, bb), "step_us": bs * 1e3,
                         "mx_bwd_speedup": bb / bwd_ms, "mx_step_speedup": bs / ms_step,
                         "mx_bwd_kernels_speedup": (kb["bwd_dkdv"] + kb["bwd_dq"])
                         / (kern_ms["bwd_dkdv"] + kern_ms["bwd_dq"])})
        base["timing"] = "the same batch through jfa_forward / jfa_backward (bf16), timed as the headline"
        res["bf16_path"] = base
        del rb
        rq = Runner(wl, batch, dev, mx_mode="forward")
        for _ in range(3):
            rq.step()
        tq = timed_steps(rq, ev, K, flush_buf)
        qf = float(np.median(tq["fwd"]))
        kq = kernel_breakdown(rq, ev, K, flush_buf)
        qa = acct["mx_quant"]
        fb = {"fwd_us": qf * 1e3, "fwd_tflops": tf(useful_fwd, qf), "fwd_vs_bf16": bf / qf,
              "kernel_us": {k_: v_ * 1e3 for k_, v_ in kq.items()},
              "mx_quant_hbm_frac": qa["bytes"] / (kq["mx_quant"] * 1e-3) / 1e9 / PEAK_HBM_GBS}
        if r.run_bwd:
            qb, qs_ = float(np.median(tq["bwd"])), float(np.median(tq["step"]))
            qq = acct["mx_quant_bwd"]
            fb.update({"bwd_us": qb * 1e3, "bwd_tflops": tf(useful_bwd, qb), "bwd_vs_bf16": bb / qb,
                       "step_us": qs_ * 1e3, "step_vs_bf16": bs / qs_,
                       "mx_quant_bwd_hbm_frac": qq["bytes"] / (kq["mx_quant_bwd"] * 1e-3) / 1e9 / PEAK_HBM_GBS})
        fb["timing"] = ("jfa_mx_forward / jfa_mx_backward (bf16 q, k, v, dO quantised by the library, then the "
                        "attention), timed as the headline")
        res["mx_from_bf16"] = fb
        del rq
    if t_warm is not None:
        wms = float(np.median(t_warm["step"]))
        res["warm"] = {"value": tf(useful_fwd + useful_bwd, wms), "ms_per_step": wms,
                       "ms_p10": pctl(t_warm["step"], 10), "ms_p90": pctl(t_warm["step"], 90),
                       "fwd_tflops": tf(useful_fwd, float(np.median(t_warm["fwd"]))),
                       "bwd_tflops": tf(useful_bwd, float(np.median(t_warm["bwd"]))) if r.run_bwd else None,
                       "timing": "median over %d warm steps (back to back, no flush)" % K}
    # the same workload at other seeds: flushed median step of each
    if args.seed_mean:
        lo, hi = (int(x) for x in args.seed_mean.split("-"))
        vals = []
        del r
        torch.cuda.empty_cache()
        for sd in range(lo, hi + 1):
            rs = Runner(wl, make_batch(wl, sd, with_dout=True), dev)
            for _ in range(3):
                rs.step()
            ts = timed_steps(rs, ev, min(K, 20), flush_buf)
            p = rs.pairs()
            vals.append(tf((4.0 + (10.0 if rs.run_bwd else 0.0)) * D * H * p, float(np.median(ts["step"]))))
            del rs
            torch.cuda.empty_cache()
        res["seed_mean"] = {"seeds": list(range(lo, hi + 1)), "values": vals, "mean": float(np.mean(vals)),
                            "timing": "median of %d steps per seed, as the headline" % min(K, 20)}
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
