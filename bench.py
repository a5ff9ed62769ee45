#!/usr/bin/env python3
"""Throughput of jagged attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: the forward call
(work-list build + attention kernel) and the backward call (work-list
builds, softmax row statistics, dK/dV kernel -- which also stores the dS
blocks, and writes the dQ of sequences of at most 64 tokens -- and dQ
kernel).  Inputs are generated on
the host, copied to HBM before timing, and stay resident.  Prints one JSON
line: useful TFLOPS counted on the visible (query, key) pairs of the real,
unpadded tokens -- 4*d FLOPs per pair forward, 10*d backward -- the split
into forward and backward, the share of the bf16 MFMA peak, per-kernel
durations from HIP events recorded between the library's launches (in an
untimed pass: each event adds a few microseconds between launches), the
roofline position of the dominant kernel (timed by the only two events
inside the timed steps), and the CPU oracle timed on a bounded sample of
the same batch.
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
PEAK_HBM_GBS = 8000.0
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_digest():
    """Digest of the device sources (kernels and the headers they include;
    not the host-side C ABI layer), to tell whether stored counters still
    apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "jagged_attention_ads_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".hpp", ".h")):
            continue
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
    pair) and bytes (every tensor the kernel must touch, once) per launch.
    `short` is short_split of the sequences whose dQ the dK/dV pass forms
    (all zeros when it forms none): their dS stays on chip, and the dQ pass
    does not touch them."""
    H, d = wl.heads, wl.head_dim
    es = 2 if wl.dtype == "bf16" else 4
    sq, sk, sp, sb = short
    q_bytes, k_bytes = T_q * H * d * es, T_k * H * d * es
    lq_bytes, lk_bytes = (T_q - sq) * H * d * es, (T_k - sk) * H * d * es   # sequences the dQ pass takes
    row_f32 = T_q * H * 4
    ds_bytes = (n_ds_blocks - sb) * H * 32 * 32 * es if ds_path else 0
    soft = wl.activation == "softmax"
    acc = {
        "fwd": dict(flops=4 * d * H * pairs_total,
                    bytes=q_bytes + 2 * k_bytes + q_bytes + (row_f32 if soft else 0)),
        # reads Q, dO, K, V (and lse2, delta); writes dK, dV, the dS blocks
        # and the short sequences' dQ
        "bwd_dkdv": dict(flops=8 * d * H * pairs_total + 2 * d * H * sp,
                         bytes=2 * q_bytes + 2 * k_bytes + (2 * row_f32 if soft else 0) + 2 * k_bytes + ds_bytes
                         + sq * H * d * es),
    }
    if ds_path:   # dQ = scale * dS K: reads the dS blocks and K, writes dQ
        acc["bwd_dq"] = dict(flops=2 * d * H * (pairs_total - sp), bytes=ds_bytes + lk_bytes + lq_bytes)
    else:         # recomputes S, P, dP, dS: reads Q, dO, K, V, lse2, delta, writes dQ
        acc["bwd_dq"] = dict(flops=6 * d * H * (pairs_total - sp),
                             bytes=3 * lq_bytes + 2 * lk_bytes + (2 * (T_q - sq) * H * 4 if soft else 0))
    if soft:      # reads O, dO and lse, writes lse2 and delta
        acc["bwd_stats"] = dict(flops=2 * d * H * T_q, bytes=2 * q_bytes + 3 * row_f32)
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


def cpu_baseline(batch, budget_s):
    """The CPU oracle, as it is, on the first sequences of the same batch
    until about `budget_s` seconds of work; useful TFLOPS under the same
    accounting."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    wl = batch.workload
    s = 1.0 / math.sqrt(wl.head_dim)
    q, k, v = batch.f64("q"), batch.f64("k"), batch.f64("v")
    do = batch.f64("dout") if batch.dout is not None else None
    qo, ko = batch.q_offsets, batch.kv_offsets
    blk = wl.block
    if blk:
        pairs = np.array([visible_pairs(block_runs([n], blk), block_runs([n], blk), wl.causal).sum()
                          for n in batch.q_lengths])
    else:
        pairs = visible_pairs(batch.q_lengths, batch.kv_lengths, wl.causal)
    done, flops, t0 = 0, 0.0, time.perf_counter()
    while done < len(pairs) and time.perf_counter() - t0 < budget_s:
        b = done
        sl_q, sl_k = slice(qo[b], qo[b + 1]), slice(ko[b], ko[b + 1])
        one_q = np.array([0, qo[b + 1] - qo[b]])
        one_k = np.array([0, ko[b + 1] - ko[b]])
        oracle.attention_fwd(q[sl_q], k[sl_k], v[sl_k], one_q, one_k, s, wl.activation, wl.causal, block=blk)
        if wl.backward and do is not None:
            oracle.attention_bwd(q[sl_q], k[sl_k], v[sl_k], do[sl_q], one_q, one_k, s, wl.activation, wl.causal,
                                 block=blk)
        flops += (14 if wl.backward else 4) * wl.head_dim * wl.heads * pairs[b]
        done += 1
    el = time.perf_counter() - t0
    return {
        "value": flops / el / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
        "sample": "fp64 NumPy oracle, %s on the first %d of %d sequences of the same batch (%.1f s, %.3g useful GFLOP)"
                  % ("fwd+bwd" if wl.backward else "fwd", done, len(pairs), el, flops / 1e9),
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="selfattn_causal")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", action="store_true",
                    help="before each step, overwrite a 512 MiB buffer (evicting the last-level cache and L2), "
                         "and time each step by its own events, flush excluded")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain elementwise copy of known size (256 MiB read + 256 MiB written per "
                         "dispatch, 3 dispatches), to scale the HBM byte counters")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences are independent; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from jagged_attention_ads_amd import jfa
    from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    batch = make_batch(wl, args.seed, with_dout=True)
    T_q, T_k, H, D = int(batch.q_offsets[-1]), int(batch.kv_offsets[-1]), wl.heads, wl.head_dim

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    q, k, v, do = (to_dev(x) for x in (batch.q, batch.k, batch.v, batch.dout))
    qo = torch.from_numpy(batch.q_offsets.astype(np.int32)).to(dev)
    ko = torch.from_numpy(batch.kv_offsets.astype(np.int32)).to(dev)
    mq, mk = int(batch.q_lengths.max()), int(batch.kv_lengths.max())
    scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q)
    lse = torch.empty((H, T_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B = len(batch.q_lengths)
    L = jfa.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    derive = None
    q_lens, kv_lens = batch.q_lengths, batch.kv_lengths
    if wl.block:
        # BlockAttention: the runs of wl.block tokens as sequences, derived on
        # the device from the sequences' offsets in every step
        seq_off, n_seq = qo, B
        n_runs = L.jfa_block_offsets_count(n_seq, T_q, wl.block)
        runs = torch.empty(n_runs, dtype=torch.int32, device=dev)

        def derive():
            st = L.jfa_block_offsets(P(seq_off), n_seq, T_q, wl.block, P(runs), n_runs, stream)
            if st != 0:
                raise jfa.JfaError(st, L.jfa_last_error().decode())
        qo = ko = runs
        B = n_runs - 1
        mq = mk = min(wl.block, mq)
        q_lens = kv_lens = block_runs(batch.q_lengths, wl.block)
    ws_f = jfa.workspace(B, H, D, T_q, T_k, mk, q.dtype, False, dev)
    ws_b = jfa.workspace(B, H, D, T_q, T_k, mk, q.dtype, True, dev)
    # the dK/dV pass stores dS and the dQ pass reads it, unless switched off
    # or the store was left out of the workspace
    ds_path = (os.environ.get("JFA_BWD_DS") != "0"
               and ws_b.numel() > jfa.jfa_workspace_size(B, H, D, T_q, T_k, mk, q.dtype, 2))
    # the dK/dV pass writes the dQ of short sequences (bf16, d 64 or 128: where
    # its LDS has room) when every sequence is short, or always with
    # JFA_BWD_FUSE_SHORT=2; never with 0
    fuse_mode = os.environ.get("JFA_BWD_FUSE_SHORT", "1")
    fuse_short = (fuse_mode != "0" and wl.dtype == "bf16" and D in (64, 128)
                  and (fuse_mode == "2" or max(mq, mk) <= 64))
    act = jfa.ACTIVATIONS[wl.activation]
    dt = jfa.DTYPES[q.dtype]
    soft = wl.activation == "softmax"
    lse_arg = lse if soft else None

    def evp(events):
        return ctypes.cast(events, ctypes.c_void_p) if events is not None else None

    def fwd(events):
        st = L.jfa_forward_profiled(P(q), P(k), P(v), P(qo), P(ko), B, H, D, T_q, T_k, mq, mk, scale, act,
                                    int(wl.causal), dt, P(out), P(lse_arg), P(ws_f), ws_f.numel(), stream, evp(events))
        if st != 0:
            raise jfa.JfaError(st, L.jfa_last_error().decode())

    def bwd(events):
        st = L.jfa_backward_profiled(P(q), P(k), P(v), P(out), P(do), P(lse_arg), P(qo), P(ko), B, H, D, T_q, T_k,
                                     mq, mk, scale, act, int(wl.causal), dt, P(dq), P(dk), P(dv), P(ws_b),
                                     ws_b.numel(), stream, evp(events))
        if st != 0:
            raise jfa.JfaError(st, L.jfa_last_error().decode())


    torch.cuda.synchronize()
    ev = HipEvents()
    run_bwd = wl.backward
    for _ in range(args.warmup):
        if derive:
            derive()
        fwd(None)
        if run_bwd:
            bwd(None)
    torch.cuda.synchronize()

    K = args.steps
    # Per-kernel breakdown: an untimed pass of K steps with an event between
    # every two launches.  Each recorded event adds a few microseconds
    # between launches, so the timed pass below records only the two around
    # the dominant kernel.
    ef = [ev.create(3) for _ in range(K)]
    eb = [ev.create(5) for _ in range(K)] if run_bwd else []
    for i in range(K):
        if derive:
            derive()
        fwd(ef[i])
        if run_bwd:
            bwd(eb[i])
    torch.cuda.synchronize()

    def avg(lst, a, b):
        return float(np.mean([ev.ms(e[a], e[b]) for e in lst])) if lst else 0.0
    kern_ms = {"sched_q": avg(ef, 0, 1), "fwd": avg(ef, 1, 2)}
    fwd_ms = avg(ef, 0, 2)
    bwd_ms = 0.0
    if run_bwd:
        kern_ms.update({"bwd_sched": avg(eb, 0, 1), "bwd_stats": avg(eb, 1, 2), "bwd_dkdv": avg(eb, 2, 3),
                        "bwd_dq": avg(eb, 3, 4)})
        bwd_ms = avg(eb, 0, 4)

    pairs = int(visible_pairs(q_lens, kv_lens, wl.causal).sum())
    n_blk = ds_blocks(q_lens, kv_lens, wl.causal) if run_bwd else 0
    short = short_split(q_lens, kv_lens, wl.causal) if run_bwd and fuse_short else (0, 0, 0, 0)
    acct = kernel_accounting(wl, T_q, T_k, pairs, n_blk, ds_path, short)
    name = max((n for n in acct if n in kern_ms), key=lambda n: kern_ms[n])   # the dominant kernel
    side, i0, i1 = {"sched_q": (0, 0, 1), "fwd": (0, 1, 2), "bwd_sched": (1, 0, 1), "bwd_stats": (1, 1, 2),
                    "bwd_dkdv": (1, 2, 3), "bwd_dq": (1, 3, 4)}[name]

    # Timed pass: exactly K steps between two events and synchronisations;
    # inside them only the events around the dominant kernel (and with
    # --flush, each step's start and end)
    dom_a, dom_b = ev.create(K), ev.create(K)
    tev = []
    for i in range(K):
        arr = (ctypes.c_void_p * (3 if side == 0 else 5))()
        arr[i0], arr[i1] = dom_a[i], dom_b[i]
        tev.append(arr)
    st_a, st_b = (ev.create(K), ev.create(K)) if args.flush else (None, None)
    edge = ev.create(2)
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.flush else None
    torch.cuda.synchronize()
    ev.lib.hipEventRecord(edge[0], stream)
    for i in range(K):
        if flush_buf is not None:
            flush_buf.fill_(i & 0xff)
        if derive:
            derive()
        if st_a is not None:
            ev.lib.hipEventRecord(st_a[i], stream)
        fwd(tev[i] if side == 0 else None)
        if run_bwd:
            bwd(tev[i] if side == 1 else None)
        if st_b is not None:
            ev.lib.hipEventRecord(st_b[i], stream)
    ev.lib.hipEventRecord(edge[1], stream)
    torch.cuda.synchronize()
    total_ms = ev.ms(edge[0], edge[1])
    ms_step = total_ms / K
    if st_a is not None:   # each step from its start to its end, without the flush
        ms_step = float(np.mean([ev.ms(st_a[i], st_b[i]) for i in range(K)]))
    dom_ms = float(np.mean([ev.ms(dom_a[i], dom_b[i]) for i in range(K)]))

    useful_fwd = 4.0 * D * H * pairs
    useful_bwd = 10.0 * D * H * pairs if run_bwd else 0.0
    value = (useful_fwd + useful_bwd) / (ms_step * 1e-3) / 1e12
    fwd_tf = useful_fwd / (fwd_ms * 1e-3) / 1e12
    bwd_tf = useful_bwd / (bwd_ms * 1e-3) / 1e12 if run_bwd else None

    # roofline of the dominant kernel, timed inside the timed pass
    t_s = dom_ms * 1e-3
    ai = acct[name]["flops"] / acct[name]["bytes"]
    digest = kernel_source_digest()
    if ai < RIDGE:
        roof = {"bound": "hbm", "achieved": acct[name]["bytes"] / t_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": acct[name]["flops"] / t_s / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(name, digest, wl.name)
    roof.update({"kernel": name, "avg_launch_us": dom_ms * 1e3,
                 "algorithmic_bytes": acct[name]["bytes"], "algorithmic_flops": acct[name]["flops"],
                 "arith_intensity": ai, "mfma_frac": acct[name]["flops"] / t_s / 1e12 / PEAK_BF16_TFLOPS})

    res = {
        "metric": METRIC, "value": value, "unit": "TFLOPS", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded; lengths and values drawn per the workload recipe)",
        "config": {"workload": wl.description, "name": wl.name, "batch": B, "heads": H, "head_dim": D,
                   "causal": wl.causal, "activation": wl.activation, "seed": args.seed, "total_q_tokens": T_q,
                   "total_kv_tokens": T_k, "visible_pairs_per_head": pairs, "block": wl.block,
                   "bwd_dq_from_stored_ds": bool(run_bwd and ds_path),
                   "bwd_short_seqs_dq_in_dkdv": bool(run_bwd and fuse_short),
                   "useful_gflop_per_step": (useful_fwd + useful_bwd) / 1e9},
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "fwd_tflops": fwd_tf, "fwd_pct_peak": 100.0 * fwd_tf / PEAK_BF16_TFLOPS,
        "bwd_tflops": bwd_tf, "bwd_pct_peak": (100.0 * bwd_tf / PEAK_BF16_TFLOPS) if bwd_tf else None,
        "kernel_us": {k_: v_ * 1e3 for k_, v_ in kern_ms.items()},
        "kernel_us_from": "an untimed pass of the same steps with an event between every two launches",
        "cache": "flushed before each step (512 MiB written)" if args.flush else "warm (steps back to back)",
        "kernel_source_digest": digest,
        "roofline": roof,
    }
    for lst in ef + eb + [edge, dom_a, dom_b] + ([st_a, st_b] if st_a is not None else []):
        ev.destroy(lst)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
