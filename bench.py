"""Benchmark: LSH-attention forward tokens/s on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload text_64k]

A step is one full forward pass (hash -> sort -> chunk attention -> combine and
un-sort) of the workload through ``reformer_lsh_attention`` on inputs already
resident in HBM.  The default workload is the 64K-token long-text shape
(batch 1, 8 heads, L = 65536, d = 128, 1024 buckets, chunks of 64, 4 rounds,
causal, bf16).  Rank 0 prints one JSON line.

Besides the end-to-end rate the script times every stage entry point on the
same stream with HIP events, reports the dominant kernel against its roofline
(algorithmic bytes or flops per launch / average launch time), and times the
CPU oracle on a bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
MFMA_FP6_PEAK_TFLOPS = 10100.0  # dense fp6 / fp4 MFMA
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="text_64k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8, help="heads of the workload the oracle runs for cpu_baseline")
    ap.add_argument("--quiet", action="store_true", help="only print the JSON line")
    ap.add_argument("--accuracy-sweep", action="store_true",
                    help="print the error of LSH attention against full shared-QK attention for several "
                         "round and bucket counts (instead of the timing line)")
    ap.add_argument("--local", action="store_true",
                    help="time local (sliding-chunk) attention on the workload's shape instead (separate q, k, v; "
                         "--local-chunk, --local-before, --local-after)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (gradients wrt qk and v for the forward's sorted order) instead")
    ap.add_argument("--ff", action="store_true",
                    help="time the chunked feed-forward layer (65536 positions, d_model 1024, d_ff 4096) instead")
    ap.add_argument("--ff-chunk", type=int, default=8192)
    ap.add_argument("--local-chunk", type=int, default=64)
    ap.add_argument("--local-before", type=int, default=1)
    ap.add_argument("--local-after", type=int, default=0)
    ap.add_argument("--profile-stage", choices=["full", "hash", "sort", "attend", "combine", "copy"],
                    help="profiling mode: run the prerequisite stages once, then only this stage --steps times "
                         "(copy = a plain 256 MiB device copy for counter calibration); prints its timing")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


class Stages:
    """Preallocated buffers and direct C-ABI calls for each stage (marshalling only)."""

    def __init__(self, nat, w, qk, v, rot):
        import torch

        self.nat, self.w, self.qk, self.v, self.rot = nat, w, qk, v, rot
        self.lib = nat.lib()
        B, H, L, d, r, nb = w.batch, w.heads, w.seq_len, w.d_head, w.n_rounds, w.n_buckets
        dev = qk.device
        self.dtype = nat._dtype_code(qk)
        self.buckets = torch.empty((B, H, r, L), dtype=torch.int32, device=dev)
        self.perm = torch.empty_like(self.buckets)
        self.o = torch.empty((B, H, r, L, d), dtype=torch.float32, device=dev)
        self.z = torch.empty((B, H, r, L), dtype=torch.float32, device=dev)
        self.out = torch.empty_like(v)
        self.hash_ws_n = max(1, nat.hash_workspace_bytes(B, H, L, d, r, nb))
        self.sort_ws_n = max(1, nat.sort_workspace_bytes(B, H, L, r, nb))
        self.full_ws_n = nat.workspace_bytes(B, H, L, d, r, nb, w.chunk_len, self.dtype)
        self.hash_ws = torch.empty(self.hash_ws_n, dtype=torch.uint8, device=dev)
        self.sort_ws = torch.empty(self.sort_ws_n, dtype=torch.uint8, device=dev)
        self.full_ws = torch.empty(self.full_ws_n, dtype=torch.uint8, device=dev)
        self.shape = (B, H, L, d, r, nb)

    def _ok(self, st, name):
        self.nat._check(st, name)

    def stream(self):
        import torch

        return torch.cuda.current_stream().cuda_stream

    def full(self):
        B, H, L, d, r, nb = self.shape
        w = self.w
        self._ok(self.lib.reformer_lsh_attention(self.qk.data_ptr(), self.v.data_ptr(), self.rot.data_ptr(), self.dtype,
                                                 B, H, L, d, r, nb, w.chunk_len, int(w.causal), self.out.data_ptr(),
                                                 self.full_ws.data_ptr(), self.full_ws_n, self.stream()),
                 "reformer_lsh_attention")

    def full_timed(self, events):
        """The pipeline with events at its kernel boundaries (reformer_lsh_attention_timed)."""
        import ctypes

        B, H, L, d, r, nb = self.shape
        w = self.w
        arr = (ctypes.c_void_p * len(events))(*[ev.cuda_event for ev in events])
        self._ok(self.lib.reformer_lsh_attention_timed(self.qk.data_ptr(), self.v.data_ptr(), self.rot.data_ptr(),
                                                       self.dtype, B, H, L, d, r, nb, w.chunk_len, int(w.causal),
                                                       self.out.data_ptr(), self.full_ws.data_ptr(), self.full_ws_n,
                                                       arr, len(events), self.stream()),
                 "reformer_lsh_attention_timed")

    def hash(self):
        B, H, L, d, r, nb = self.shape
        self._ok(self.lib.reformer_lsh_hash(self.qk.data_ptr(), self.dtype, self.rot.data_ptr(), B, H, L, d, r, nb,
                                            self.buckets.data_ptr(), None, self.hash_ws.data_ptr(), self.hash_ws_n,
                                            self.stream()), "reformer_lsh_hash")

    def sort(self):
        B, H, L, d, r, nb = self.shape
        self._ok(self.lib.reformer_lsh_sort(self.buckets.data_ptr(), B, H, L, r, nb, self.perm.data_ptr(), None,
                                            self.sort_ws.data_ptr(), self.sort_ws_n, self.stream()),
                 "reformer_lsh_sort")

    def attend(self):
        B, H, L, d, r, nb = self.shape
        w = self.w
        self._ok(self.lib.reformer_lsh_chunk_attend(self.qk.data_ptr(), self.v.data_ptr(), self.dtype,
                                                    self.perm.data_ptr(), B, H, L, d, r, w.chunk_len, int(w.causal),
                                                    self.o.data_ptr(), self.z.data_ptr(), self.stream()),
                 "reformer_lsh_chunk_attend")

    def combine(self):
        B, H, L, d, r, nb = self.shape
        self._ok(self.lib.reformer_lsh_combine(self.o.data_ptr(), self.z.data_ptr(), self.v.data_ptr(), self.dtype,
                                               B, H, L, d, r, self.out.data_ptr(), self.stream()),
                 "reformer_lsh_combine")


def time_calls(fn, steps, warmup):
    """Average GPU milliseconds per call, measured with events on the launch stream."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def compact_rounds(w) -> bool:
    """bf16 inputs with 64-slot chunks keep per-round results as float16 + (z, k) pairs."""
    return w.dtype == "bf16" and min(w.chunk_len, w.seq_len) == 64 and w.seq_len % 64 == 0


def stage_work(w):
    """Algorithmic work per launch of each pipeline kernel (formulas in the design notes).

    Per head-token (N = batch * heads * seq_len) and round r: the hash projects
    onto b/2 rotation columns (2 d b/2 flops); chunk attention gathers one qk and
    one v row plus the permutation entry and writes one o row plus its
    normaliser; the combine reads the r rows and writes the output row.  In the
    compact bf16 pipeline the last round's attention launch does the combine
    itself: "attend" then covers rounds 0..r-2 and "combine" the last round
    (gather, no o written) plus the reads of the earlier rounds and the output.
    """
    N = w.batch * w.heads * w.seq_len
    r, d, b = w.n_rounds, w.d_head, w.n_buckets
    e = 2 if w.dtype == "bf16" else 4
    window = min(2 * w.chunk_len, w.seq_len)
    gather = 2 * d * e + 4
    if compact_rounds(w):
        o_row = 2 * d + 8
        attend = {"bytes": N * (r - 1) * (gather + o_row), "flops": N * (r - 1) * 4 * window * d}
        combine = {"bytes": N * (gather + (r - 1) * o_row + d * e), "flops": N * 4 * window * d}
    else:
        o_row = 4 * d + 4
        attend = {"bytes": N * r * (gather + o_row), "flops": N * r * 4 * window * d}
        combine = {"bytes": N * (r * o_row + d * e)}
    return {
        "hash": {"flops": N * r * d * b, "bytes": N * (d * e + 4 * r)},
        "sort": {"bytes": N * r * 12},   # bucket ids read by histogram and scatter, perm written
        "attend": attend,
        "combine": combine,
    }


def kernel_of_stage(w):
    fast = w.dtype == "bf16" and min(w.chunk_len, w.seq_len) == 64
    if compact_rounds(w):
        attend, combine = "chunk_attend64_kernel<compact>", "chunk_attend64_kernel<final>"
    else:
        attend, combine = ("chunk_attend64_kernel" if fast else "chunk_attend_kernel"), "combine_kernel"
    hash_k = "hash_mfma_kernel" if w.dtype == "bf16" else "hash_fma_kernel"
    return {
        "hash": (hash_k, "efficient_long_sequence_lsh_amd/csrc/hash.hip"),
        "sort": ("sort_hist_kernel+sort_scan_kernel+sort_scatter_kernel", "efficient_long_sequence_lsh_amd/csrc/sort.hip"),
        "attend": (attend, "efficient_long_sequence_lsh_amd/csrc/attend.hip"),
        "combine": (combine, "efficient_long_sequence_lsh_amd/csrc/attend.hip" if compact_rounds(w)
                    else "efficient_long_sequence_lsh_amd/csrc/combine.hip"),
    }


def roofline_for(stage, ms, w):
    work = stage_work(w)[stage]
    kernel, src = kernel_of_stage(w)[stage]
    secs = ms / 1e3
    if stage == "hash":
        ach = work["flops"] / secs / 1e12
        rf = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
              "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
              # float32-accurate projections: x.R_hi on bf16 MFMA plus x.R_lo on fp6 MFMA,
              # each as many flops as the algorithm, priced at its own dense peak
              "executed_mfma_frac": round(ach / MFMA_BF16_PEAK_TFLOPS + ach / MFMA_FP6_PEAK_TFLOPS, 4)}
    else:
        ach = work["bytes"] / secs / 1e9
        rf = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": round(ach / HBM_PEAK_GBS, 4)}
    rf["kernel"] = kernel
    rf["traffic"] = measured_traffic(kernel, src, w)
    return rf


def measured_traffic(kernel, src, w):
    """HBM bytes per launch from rocprofv3 counters, if taken on the current kernel source."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(w.name, {}).get(kernel)
    if not ent or ent.get("source_sha256_16") != source_digest(os.path.join(ROOT, src)):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, inp, heads):
    """The float64 oracle on `heads` (batch, head) slices of the same workload."""
    import numpy as np

    import oracle

    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)][:heads]
    t0 = time.perf_counter()
    for b, h in pairs:
        oracle.lsh_attention_head(inp.qk[b, h].astype(np.float64), inp.v[b, h].astype(np.float64), inp.rotations,
                                  w.n_buckets, w.chunk_len, w.causal)
    dt = time.perf_counter() - t0
    frac = len(pairs) / (w.batch * w.heads)       # share of one forward pass the sample covers
    value = w.tokens * frac / dt
    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = len(os.sched_getaffinity(0))
    return {"value": round(value, 1), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(pairs)} of {w.batch * w.heads} (batch, head) slices, full length {w.seq_len}, "
                      f"all {w.n_rounds} rounds; {dt:.1f} s wall; value = covered share of one forward's "
                      f"{w.tokens} tokens / wall time"}


def profile_stage(args, st, w):
    """Run one stage repeatedly (for rocprofv3 kernel traces and counters)."""
    import torch

    name = args.profile_stage
    if name == "copy":
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)  # noqa: E731
        work = {"bytes": 2 * n}
    else:
        if name in ("sort", "attend", "combine"):
            st.hash()
        if name in ("attend", "combine"):
            st.sort()
        if name == "combine":
            st.attend()
        fn = getattr(st, name)
        work = stage_work(w).get(name, {})
    ms = time_calls(fn, args.steps, args.warmup)
    print(json.dumps({"profile_stage": name, "workload": w.name, "ms_per_launch": round(ms, 4),
                      "algorithmic": work}), flush=True)


def accuracy_sweep(args):
    """Error of LSH attention against full attention as rounds and buckets vary.

    Both sides run in this library on the GPU: full shared-QK attention is the
    same pipeline with one bucket and one chunk spanning the sequence (every
    key visible, self masked unless it is the only key), whose agreement with
    the float64 oracle the parity tests check.  Inputs: the small causal shape
    (batch 2, 4 heads, L = 4096, d = 64, chunks of 64, float32) with iid normal
    and with clustered (mixture) shared vectors, the latter also scaled by 3
    (peaked attention); v iid normal.  Reported: the relative Frobenius error
    ||out - full|| / ||full|| over all heads.  Diffuse full attention averages
    thousands of rows of v, so its norm is small and the relative error of any
    128-key window exceeds 1 there.
    """
    import dataclasses

    import numpy as np
    import torch

    from efficient_long_sequence_lsh_amd import _native as nat
    from efficient_long_sequence_lsh_amd import workloads as W

    if not os.path.exists(nat.LIB_PATH):
        from efficient_long_sequence_lsh_amd import build

        build.build()
    base = W.WORKLOADS["small_4k_f32"]
    rounds, buckets = [1, 2, 4, 8], [8, 16, 32, 64, 128]
    rows = []
    # (label, generator kind, factor on qk): the mixture scaled by 3 makes the
    # attention peaked (same-centre scores ~ 81/sqrt(d)) instead of diffuse.
    for label, kind, qk_scale in (("normal", "normal", 1.0), ("mixture", "mixture", 1.0),
                                  ("mixture_x3", "mixture", 3.0)):
        w0 = dataclasses.replace(base, qk_kind=kind, name=f"sweep_{kind}")
        ref_in = W.make_inputs(dataclasses.replace(w0, n_buckets=1, n_rounds=1))
        qk = torch.from_numpy((ref_in.qk * np.float32(qk_scale)).astype(np.float32)).cuda()
        v = torch.from_numpy(ref_in.v).cuda()
        full = nat.attention(qk, v, None, 1, w0.seq_len, w0.causal, n_rounds=1).double()
        fnorm = float(torch.linalg.vector_norm(full))
        for b in buckets:
            for r in rounds:
                inp = W.make_inputs(dataclasses.replace(w0, n_buckets=b, n_rounds=r))   # same qk, v; own R
                rot = torch.from_numpy(inp.rotations).cuda()
                out = nat.attention(qk, v, rot, b, w0.chunk_len, w0.causal, n_rounds=r).double()
                err = float(torch.linalg.vector_norm(out - full)) / fnorm
                rows.append({"qk": label, "n_buckets": b, "n_rounds": r, "rel_err": round(err, 5)})
                log(args, f"[sweep] {label:10s} b={b:4d} r={r}: {err:.4f}")
    print(json.dumps({"accuracy_sweep": rows, "shape": {"batch": base.batch, "heads": base.heads,
                      "seq_len": base.seq_len, "d_head": base.d_head, "chunk_len": base.chunk_len,
                      "causal": base.causal, "dtype": "f32"},
                      "reference": "full shared-QK attention (one bucket, one chunk) in the same library"}),
          flush=True)


def local_bench(args):
    """Local (sliding-chunk) attention on the workload's shape: separate q, k, v
    drawn iid normal, one JSON line with tokens/s and the HBM roofline.

    Algorithmic bytes per token: one row each of q, k and v read and one output
    row written (4 d e); the kernel reloads a key tile for every query tile
    whose window covers it, which the roofline fraction then exposes.
    """
    import numpy as np
    import torch

    from efficient_long_sequence_lsh_amd import _native as nat
    from efficient_long_sequence_lsh_amd import workloads as W

    if not os.path.exists(nat.LIB_PATH):
        from efficient_long_sequence_lsh_amd import build

        build.build()
    w = W.WORKLOADS[args.workload]
    B, H, L, d = w.batch, w.heads, w.seq_len, w.d_head
    g = np.random.default_rng(np.random.SeedSequence([20200104, 900 + w.index]))
    tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(g.standard_normal((B, H, L, d), dtype=np.float32)).to(tdtype).cuda() for _ in range(3))
    out = torch.empty_like(v)
    m, nb, na = args.local_chunk, args.local_before, args.local_after
    fn = lambda: nat.local_attention(q, k, v, m, nb, na, w.causal, out=out)  # noqa: E731
    ms = time_calls(fn, args.steps, args.warmup)
    e = 2 if w.dtype == "bf16" else 4
    N = B * H * L
    bytes_ = N * 4 * d * e
    mm = min(m, L)
    window = min(L, (nb + 1 + na) * mm)
    ach = bytes_ / (ms / 1e3) / 1e9
    line = {
        "metric": "local attention fwd tokens/sec",
        "value": round(N / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded iid normal q, k, v)",
        "config": {"workload": f"local_{w.name}", "batch": B, "heads": H, "seq_len": L, "d_head": d, "chunk_len": m,
                   "n_before": nb, "n_after": na, "causal": w.causal},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "kernel": "local_ring_kernel", "traffic": None},
        "flops_per_token": 4 * window * d,
    }
    print(json.dumps(line), flush=True)


MFMA_F32_PEAK_TFLOPS = 157.3


def backward_bench(args):
    """Backward pass on the workload: perm from the library's hash and sort,
    out from its forward, dout iid normal; times reformer_lsh_attend_backward.

    The forward runs as reformer_lsh_attend_lse, and the timed backward takes
    its log normaliser (the way a training step uses them); the backward that
    recomputes the normalisers is timed too and reported on stderr.

    Work per head-token and round (bf16 MFMA for bf16 inputs, float32 MFMA
    for float32 inputs): the key role S, dP, dV and dK for the 2m queries that
    see a key (4 * 2 * 2m * d), the query role S, dP and dQ over the window
    (3 * 2 * 2m * d); recomputing the normalisers adds S over the window
    (2 * 2m * d).
    """
    import numpy as np
    import torch

    from efficient_long_sequence_lsh_amd import _native as nat
    from efficient_long_sequence_lsh_amd import workloads as W

    if not os.path.exists(nat.LIB_PATH):
        from efficient_long_sequence_lsh_amd import build

        build.build()
    w = W.WORKLOADS[args.workload]
    inp = W.make_inputs(w)
    if inp.qk_bits is not None:
        qk = torch.from_numpy(inp.qk_bits.view(np.int16)).view(torch.bfloat16).cuda()
        v = torch.from_numpy(inp.v_bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        qk = torch.from_numpy(inp.qk).cuda()
        v = torch.from_numpy(inp.v).cuda()
    rot = torch.from_numpy(inp.rotations).cuda()
    perm, _ = nat.lsh_sort(nat.lsh_hash(qk, rot, w.n_buckets), w.n_buckets, inverse=False)
    out, lse = nat.attend(qk, v, perm, w.chunk_len, w.causal, return_lse=True)
    g = np.random.default_rng(np.random.SeedSequence([20200104, 950 + w.index]))
    dout = torch.from_numpy(g.standard_normal(tuple(v.shape), dtype=np.float32)).to(v.dtype).cuda()
    fn = lambda: nat.attend_backward(qk, v, perm, w.chunk_len, w.causal, out, dout, lse=lse)  # noqa: E731
    ms = time_calls(fn, args.steps, args.warmup)
    ms_recompute = time_calls(lambda: nat.attend_backward(qk, v, perm, w.chunk_len, w.causal, out, dout),
                              args.steps, args.warmup)
    print(f"[bench] backward with the forward's normaliser {ms:.3f} ms; recomputing it {ms_recompute:.3f} ms",
          file=sys.stderr, flush=True)
    N = w.batch * w.heads * w.seq_len
    win = min(2 * w.chunk_len, w.seq_len)
    flops = N * w.n_rounds * (4 + 3) * 2 * win * w.d_head
    ach = flops / (ms / 1e3) / 1e12
    # bf16 inputs run every contraction on the bf16 MFMA, float32 inputs on the float32 MFMA
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    line = {
        "metric": "LSH-attention backward tokens/sec (grads wrt qk and v)",
        "value": round(w.tokens / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded)",
        "config": {"workload": f"backward_{w.name}", "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "d_head": w.d_head, "n_buckets": w.n_buckets, "chunk_len": w.chunk_len, "n_rounds": w.n_rounds,
                   "causal": w.causal, "normaliser": "saved by the forward (lse)"},
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(ach / peak, 4), "kernel": "bwd_*_kernel (whole pass)", "traffic": None},
    }
    print(json.dumps(line), flush=True)


def ff_bench(args):
    """Chunked feed-forward relu(x W1^T + b1) W2^T + b2 on 65536 positions
    (the 64K text sequence at batch 1), d_model 1024, d_ff 4096, bf16, in
    chunks of --ff-chunk positions; 4 n d f flops per call against the bf16
    MFMA peak.  The whole-sequence call is timed too (same result bit for bit)."""
    import numpy as np
    import torch

    from efficient_long_sequence_lsh_amd import _native as nat

    if not os.path.exists(nat.LIB_PATH):
        from efficient_long_sequence_lsh_amd import build

        build.build()
    n, d, f = 65536, 1024, 4096
    g = np.random.default_rng(np.random.SeedSequence([20200104, 970]))
    x = torch.from_numpy(g.standard_normal((n, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    w1 = torch.from_numpy(g.standard_normal((f, d), dtype=np.float32) / 32.0).to(torch.bfloat16).cuda()
    w2 = torch.from_numpy(g.standard_normal((d, f), dtype=np.float32) / 64.0).to(torch.bfloat16).cuda()
    b1 = torch.from_numpy(0.1 * g.standard_normal(f, dtype=np.float32)).cuda()
    b2 = torch.from_numpy(0.1 * g.standard_normal(d, dtype=np.float32)).cuda()
    out = torch.empty_like(x)
    flops = 4.0 * n * d * f
    res = {}
    for label, chunk in (("chunked", args.ff_chunk), ("whole", 0)):
        ms = time_calls(lambda: nat.feed_forward(x, w1, b1, w2, b2, chunk_tokens=chunk, out=out),  # noqa: B023
                        args.steps, args.warmup)
        res[label] = {"ms": round(ms, 4), "tflops": round(flops / (ms / 1e3) / 1e12, 1),
                      "hidden_bytes": int(nat.lib().reformer_lsh_feed_forward_workspace_bytes(n, d, f, chunk))}
    ms = res["chunked"]["ms"]
    ach = flops / (ms / 1e3) / 1e12
    line = {
        "metric": "chunked feed-forward tokens/sec", "value": round(n / (ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded)",
        "config": {"workload": "feed_forward_64k", "n_tokens": n, "d_model": d, "d_ff": f, "chunk_tokens": args.ff_chunk},
        "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "kernel": "linear_kernel", "traffic": None},
        "whole_sequence": res["whole"], "chunked": res["chunked"],
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.accuracy_sweep:
        accuracy_sweep(args)
        return
    if args.local:
        local_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.ff:
        ff_bench(args)
        return

    import numpy as np
    import torch

    from efficient_long_sequence_lsh_amd import _native as nat
    from efficient_long_sequence_lsh_amd import workloads as W

    if not os.path.exists(nat.LIB_PATH):
        from efficient_long_sequence_lsh_amd import build

        build.build()
    w = W.WORKLOADS[args.workload]
    log(args, f"[bench] generating {w.name}")
    inp = W.make_inputs(w)
    if inp.qk_bits is not None:
        qk = torch.from_numpy(inp.qk_bits.view(np.int16)).view(torch.bfloat16).cuda()
        v = torch.from_numpy(inp.v_bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        qk = torch.from_numpy(inp.qk).cuda()
        v = torch.from_numpy(inp.v).cuda()
    rot = torch.from_numpy(inp.rotations).cuda()
    st = Stages(nat, w, qk, v, rot)
    if args.profile_stage:
        profile_stage(args, st, w)
        return

    log(args, f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    for _ in range(args.warmup):
        st.full()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(args.steps):
        st.full()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    value = w.tokens / (ms / 1e3)
    log(args, f"[bench] {ms:.3f} ms/step, {value:.4g} tokens/s")

    # Per-kernel durations of the pipeline's own launches: HIP events recorded
    # by the library at its kernel boundaries on this stream, every timed step.
    events = [torch.cuda.Event(enable_timing=True) for _ in range(nat.TIMED_EVENTS)]
    for ev in events:
        ev.record()                       # creates the underlying hipEvent_t
    torch.cuda.synchronize()
    spans = {"hash_setup": (0, 1), "hash": (1, 2), "hash_fixup": (2, 3), "sort": (3, 4), "attend": (4, 5),
             "combine": (5, 6)}
    acc = {k: 0.0 for k in spans}
    for _ in range(args.steps):
        st.full_timed(events)
        torch.cuda.synchronize()
        for k, (a, b) in spans.items():
            acc[k] += events[a].elapsed_time(events[b])
    stage_ms = {k: v / args.steps for k, v in acc.items()}
    for k, v in stage_ms.items():
        log(args, f"[bench] {k}: {v:.4f} ms")
    main = ["hash", "sort", "attend", "combine"]
    dominant = max(main, key=lambda k: stage_ms[k])
    roof = roofline_for(dominant, stage_ms[dominant], w)
    stages = {}
    for name in main:
        r = roofline_for(name, stage_ms[name], w)
        stages[name] = {"ms": round(stage_ms[name], 4), "kernel": r["kernel"], "achieved": r["achieved"],
                        "unit": r["unit"], "frac": r["frac"]}
    stages["hash_setup"] = {"ms": round(stage_ms["hash_setup"], 4)}
    stages["hash_fixup"] = {"ms": round(stage_ms["hash_fixup"], 4)}

    cpu = None
    if not args.no_cpu_baseline:
        log(args, f"[bench] cpu baseline: oracle on {args.cpu_heads} slices")
        cpu = cpu_baseline(w, inp, args.cpu_heads)

    line = {
        "metric": "LSH-attention fwd tokens/sec at L=64K, 4 rounds; % of HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes and structure of the workload, no dataset)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len, "d_head": w.d_head,
                   "n_buckets": w.n_buckets, "chunk_len": w.chunk_len, "n_rounds": w.n_rounds, "causal": w.causal,
                   "qk": w.qk_kind},
        "roofline": roof,
        "stages": stages,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
