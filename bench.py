"""Benchmark: LSH-attention forward tokens/s on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 200] [--workload text_64k]

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
MFMA_F32_PEAK_TFLOPS = 157.3    # dense float32 MFMA
FP32_VECTOR_PEAK_TFLOPS = 157.3  # float32 vector FMA (256 CUs x 128 lanes x 2 flops x 2.4 GHz)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The first few hundred milliseconds of back-to-back forwards on a fresh
    # process run 5-7 % slower (clocks and memory ramp up), so the default
    # warm-up reaches the steady state before the timed steps.
    ap.add_argument("--warmup", type=int, default=200)
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
    ap.add_argument("--ingest-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="read rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv output of --profile-stage full and of "
                         "--profile-stage copy for --workload, and record calibrated HBM bytes per launch of each "
                         "kernel (with its source digest) in profiles/traffic.json")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="time a large bf16 GEMM (torch.matmul, hipBLASLt) on random and on constant operands: "
                         "the matrix-core rate the chip sustains under its power limit, beside the dense peak")
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

    def hash(self, ties=None):
        B, H, L, d, r, nb = self.shape
        self._ok(self.lib.reformer_lsh_hash(self.qk.data_ptr(), self.dtype, self.rot.data_ptr(), B, H, L, d, r, nb,
                                            self.buckets.data_ptr(), None if ties is None else ties.data_ptr(),
                                            self.hash_ws.data_ptr(), self.hash_ws_n, self.stream()),
                 "reformer_lsh_hash")

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
    (gather, no o written) plus the reads of the earlier rounds and the output;
    its rows (12-bit block floating point at d = 128, float16 at d = 64) carry
    their normaliser in their own bits.
    """
    N = w.batch * w.heads * w.seq_len
    r, d, b = w.n_rounds, w.d_head, w.n_buckets
    e = 2 if w.dtype == "bf16" else 4
    window = min(2 * w.chunk_len, w.seq_len)
    gather = 2 * d * e + 4
    if compact_rounds(w):
        # compact row: 12-bit block floating point at d = 128, float16 at d = 64;
        # z and the scale exponent ride in the values' lowest bits
        o_row = 3 * d // 2 if d == 128 else 2 * d
        attend = {"bytes": N * (r - 1) * (gather + o_row), "flops": N * (r - 1) * 4 * window * d}
        combine = {"bytes": N * (gather + (r - 1) * o_row + d * e), "flops": N * 4 * window * d}
    else:
        o_row = 4 * d + 4
        attend = {"bytes": N * r * (gather + o_row), "flops": N * r * 4 * window * d}
        combine = {"bytes": N * (r * o_row + d * e)}
    return {
        "hash": {"flops": N * r * d * b, "bytes": N * (d * e + 4 * r)},
        "sort": {"bytes": N * r * SORT_BYTES[sort_path(w)]},
        "attend": attend,
        "combine": combine,
    }


SORT_KERNELS = {"block": "sort_block_kernel",
                "tiles": "sort_hist_kernel+sort_scan_kernel+sort_scatter_kernel",
                "two_pass": "sort_hist_kernel+sort_scan_kernel+sort_scatter_kernel+sort_block_kernel"}
# Bytes per (position, round) each sort path moves by its design: bucket ids
# read once (block) or twice (tiles: histogram and scatter) and the
# permutation written; two passes add the 4-byte entries written and read back.
SORT_BYTES = {"block": 8, "tiles": 12, "two_pass": 20}


def sort_path(w):
    """Which sort the library runs for this shape (the rule of its sort shape)."""
    kb = max(0, (w.n_buckets - 1).bit_length())
    if kb <= 8 and w.seq_len <= 12288:
        return "block"
    if kb > 6 and (kb > 10 or w.seq_len > 131072):
        return "two_pass"
    return "tiles"


def kernel_of_stage(w):
    fast = w.dtype == "bf16" and min(w.chunk_len, w.seq_len) == 64
    if compact_rounds(w):
        attend, combine = "chunk_attend64_kernel<compact>", "chunk_attend64_kernel<final>"
    else:
        attend, combine = ("chunk_attend64_kernel" if fast else "chunk_attend_kernel"), "combine_kernel"
    hash_k = "hash_mfma_kernel" if w.dtype == "bf16" else "hash_fma_kernel"
    return {
        "hash": (hash_k, "efficient_long_sequence_lsh_amd/csrc/hash.hip"),
        "sort": (SORT_KERNELS[sort_path(w)], "efficient_long_sequence_lsh_amd/csrc/sort.hip"),
        "attend": (attend, "efficient_long_sequence_lsh_amd/csrc/attend.hip"),
        "combine": (combine, "efficient_long_sequence_lsh_amd/csrc/attend.hip" if compact_rounds(w)
                    else "efficient_long_sequence_lsh_amd/csrc/combine.hip"),
    }


def roofline_for(stage, ms, w):
    work = stage_work(w)[stage]
    kernel, src = kernel_of_stage(w)[stage]
    secs = ms / 1e3
    if stage == "hash" and w.dtype != "bf16":   # float32 inputs: the FMA kernel on the vector ALU
        ach = work["flops"] / secs / 1e12
        rf = {"bound": "alu", "achieved": round(ach, 2), "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
              "frac": round(ach / FP32_VECTOR_PEAK_TFLOPS, 4)}
    elif stage == "hash":
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


def other_resource(stage, ms, w):
    """The stage's rate against the resource that does not bind it: the hash's
    algorithmic bytes (x read once, ids written) against HBM, and chunk
    attention's algorithmic matrix work (S = K Q^T and O = V P^T over each
    chunk's window) against the dense MFMA peak of its operand type."""
    work = stage_work(w)[stage]
    secs = ms / 1e3
    if stage == "hash":
        ach = work["bytes"] / secs / 1e9
        return {"hbm": {"achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4)}}
    if stage in ("attend", "combine") and "flops" in work:
        peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
        ach = work["flops"] / secs / 1e12
        return {"mfma": {"achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4)}}
    return {}


def path_roofline(ms, w):
    """The whole forward against its floor: each stage's algorithmic work at its
    own peak (the hash's projections on the dense bf16 MFMA, or the float32
    vector ALU for float32 inputs; sort, attention and combine at HBM's 8 TB/s
    for the bytes the algorithm must move), summed, over the measured time."""
    work = stage_work(w)
    hash_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_VECTOR_PEAK_TFLOPS
    floor = {"hash": work["hash"]["flops"] / (hash_peak * 1e12) * 1e3}
    for name in ("sort", "attend", "combine"):
        floor[name] = work[name]["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e3
    t_roof = sum(floor.values())
    return {"t_roof_ms": round(t_roof, 4), "frac": round(t_roof / ms, 4),
            "stage_floor_ms": {k: round(v, 4) for k, v in floor.items()},
            "basis": "hash flops at the dense bf16 MFMA peak (float32 vector peak for float32 inputs); "
                     "sort, attention and combine algorithmic bytes at 8 TB/s; set-up kernel excluded"}


def occupancy(st, w):
    """Bucket occupancy of the library's ids for the workload (hashed once more
    after the timing): largest and mean bucket size over all (batch, head,
    round) segments, and the mean number of empty buckets per segment."""
    import numpy as np
    import torch

    st.hash()
    torch.cuda.synchronize()
    ids = st.buckets.cpu().numpy().reshape(-1, w.seq_len)
    counts = np.stack([np.bincount(row, minlength=w.n_buckets) for row in ids])
    return {"max_bucket": int(counts.max()), "mean_bucket": round(w.seq_len / w.n_buckets, 2),
            "empty_buckets_per_round": round(float((counts == 0).sum(axis=1).mean()), 1)}


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


KERNEL_SOURCES = {"hash_": "hash.hip", "sort_": "sort.hip", "chunk_attend": "attend.hip", "combine_": "combine.hip"}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_KIB = 262144   # --profile-stage copy moves 256 MiB each way


def _kernel_key(name: str) -> str:
    """Kernel key as the bench names it, from a demangled rocprofv3 kernel name."""
    base = name.replace("(anonymous namespace)", "").split("(")[0]
    ident = base.split("<")[0].split("::")[-1].strip()
    if ident == "chunk_attend64_kernel" and "<" in base:
        mode = int(base.split("<", 1)[1].rstrip(">").split(",")[-1])
        return ident + ("" if mode == 0 else "<compact>" if mode == 1 else "<final>")
    return ident


def _counter_means(folder: str, counter: str) -> dict:
    """Mean counter value per dispatch of each kernel in a rocprofv3 csv run."""
    import csv
    import glob

    sums, counts = {}, {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {folder}")
    for path in files:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                k = row["Kernel_Name"]
                sums[k] = sums.get(k, 0.0) + float(row["Counter_Value"])
                counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def ingest_traffic(args):
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.ingest_traffic
    cf = _counter_means(cfetch_dir, "FETCH_SIZE")
    cw = _counter_means(cwrite_dir, "WRITE_SIZE")
    copy_f = [v for k, v in cf.items() if COPY_KERNEL in k]
    copy_w = [v for k, v in cw.items() if COPY_KERNEL in k]
    if not copy_f or not copy_w:
        raise SystemExit(f"no {COPY_KERNEL} dispatches in the calibration runs")
    ff, wf = COPY_KIB / copy_f[0], COPY_KIB / copy_w[0]
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    entries = {}
    for name, fk in fetch.items():
        key = _kernel_key(name)
        src = next((v for p, v in KERNEL_SOURCES.items() if key.startswith(p)), None)
        wk = next((v for n, v in write.items() if _kernel_key(n) == key), None)
        if src is None or wk is None:
            continue
        entries[key] = {"bytes_per_launch": int(round((fk * ff + wk * wf) * 1024)), "fetch_factor": round(ff, 4),
                        "fetch_kib": round(fk, 1), "source": src,
                        "source_sha256_16": source_digest(os.path.join(ROOT, "efficient_long_sequence_lsh_amd",
                                                                       "csrc", src)),
                        "write_factor": round(wf, 4), "write_kib": round(wk, 1)}
    try:
        with open(PROFILE_TRAFFIC) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data.setdefault(args.workload, {}).update(entries)
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({"workload": args.workload, "fetch_factor": ff, "write_factor": wf, "kernels": entries}, indent=1))


def cpu_baseline(w, inp, heads):
    """The float64 oracle on `heads` (batch, head) slices of the same workload.

    Returns the baseline record and the oracle's results per slice (bucket
    ids, margins, permutation and output), which the parity check compares
    with the GPU's."""
    import numpy as np

    import oracle

    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)][:heads]
    results = {}
    t0 = time.perf_counter()
    for b, h in pairs:
        results[(b, h)] = oracle.lsh_attention_head(inp.qk[b, h].astype(np.float64), inp.v[b, h].astype(np.float64),
                                                    inp.rotations, w.n_buckets, w.chunk_len, w.causal)
    dt = time.perf_counter() - t0
    frac = len(pairs) / (w.batch * w.heads)       # share of one forward pass the sample covers
    value = w.tokens * frac / dt
    affinity = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl

        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = affinity
    return {"value": round(value, 1), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "host": {"cpu_count": os.cpu_count(), "affinity": affinity, "blas_threads": int(cores)},
            "sample": f"{len(pairs)} of {w.batch * w.heads} (batch, head) slices, full length {w.seq_len}, "
                      f"all {w.n_rounds} rounds; {dt:.1f} s wall; value = covered share of one forward's "
                      f"{w.tokens} tokens / wall time"}, results


NEAR_TIE = 1e-5
TOL = {"f32": 1e-4, "bf16": 2e-2}


def parity_vs_oracle(st, w, results):
    """The GPU's bucket ids, permutation and output against the oracle's on the
    slices the CPU baseline ran (every position, every round of each slice).

    bucket_flips counts differing ids; near_ties_lt_1e-5 the (position, round)
    pairs whose exact top-two gap is below 1e-5 (where a flip is allowed);
    flips_at_margin_ge_1e-5 must be 0.  redecided is the GPU's own count of
    float64 re-decisions over the whole workload.  perm_exact compares the
    GPU's sort with the oracle's; max_abs_err the pipeline's output with the
    oracle's (both only meaningful without flips, else they are taken against
    the oracle's sort of the GPU ids and reported as null respectively)."""
    import numpy as np
    import torch

    import oracle

    ties = torch.zeros(1, dtype=torch.int32, device=st.qk.device)
    st.hash(ties)
    st.sort()
    st.full()
    torch.cuda.synchronize()
    gb = st.buckets.cpu().numpy()
    gp = st.perm.cpu().numpy()
    out = st.out.float().cpu().numpy()
    n_ids = flips = near = bad = 0
    perm_ok = True
    err = 0.0
    for (b, h), res in results.items():
        ob, om = res["buckets"], res["margin"]
        mism = gb[b, h] != ob
        n_ids += mism.size
        flips += int(mism.sum())
        near += int((om < NEAR_TIE).sum())
        bad += int((mism & (om >= NEAR_TIE)).sum())
        want_p = res["perm"] if not mism.any() else oracle.lsh_sort(gb[b, h])[0]
        perm_ok &= bool(np.array_equal(gp[b, h], want_p))
        if not mism.any():
            err = max(err, float(np.abs(out[b, h] - res["out"]).max()))
    return {"slices": len(results), "bucket_ids": n_ids, "bucket_flips": flips, "near_ties_lt_1e-5": near,
            "flips_at_margin_ge_1e-5": bad, "redecided": int(ties.item()), "perm_exact": perm_ok,
            "max_abs_err": round(err, 6) if flips == 0 else None, "tol": TOL[w.dtype],
            "pass": bad == 0 and perm_ok and (flips > 0 or err <= TOL[w.dtype])}


def peak_memory(nat, w, qk, v, rot):
    """Device memory of one forward pass: inputs resident, then the output and
    the workspace allocated and the pipeline run (torch's allocator counts
    every device allocation the pass makes)."""
    import torch

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws_n = nat.workspace_bytes(w.batch, w.heads, w.seq_len, w.d_head, w.n_rounds, w.n_buckets, w.chunk_len,
                               nat._dtype_code(qk))
    nat.attention(qk, v, rot, w.n_buckets, w.chunk_len, w.causal)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    return {"peak_allocated_bytes": int(peak), "inputs_bytes": int(base), "workspace_bytes": int(ws_n),
            "out_bytes": int(v.numel() * v.element_size()), "peak_gib": round(peak / 2 ** 30, 3)}


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
    """Error and cost of LSH attention against full attention as rounds and
    buckets vary ("Reformer: The Efficient Transformer", Key points, Number of
    hash rounds bullet: more rounds come closer to full attention and cost
    more).

    Error: both sides run in this library on the GPU; full shared-QK attention
    is the same pipeline with one bucket and one chunk spanning the sequence
    (every key visible, self masked unless it is the only key), which the GPU
    tests check against the float64 oracle at this very shape.  Inputs: the
    small causal shape (batch 2, 4 heads, L = 4096, d = 64, chunks of 64,
    float32) with iid normal, clustered (mixture) and position-smooth (AR(1),
    rho = 0.9) shared vectors, the mixture also scaled by 3 (peaked
    attention); v iid normal.  Reported: the relative Frobenius error
    ||out - full|| / ||full|| over all heads, and the GPU time per forward at
    that shape.  Diffuse full attention averages thousands of rows of v, so
    its norm is small and the relative error of any 128-key window exceeds 1.

    Cost: milliseconds per forward for every (rounds, buckets) cell at the
    64K-token text shape (batch 1, 8 heads, d = 128, chunks of 64, causal,
    bf16, mixture input), where the work is large enough to show it.
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
                                  ("mixture_x3", "mixture", 3.0), ("ar1", "ar1", 1.0)):
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
                ws = torch.empty(nat.workspace_bytes(base.batch, base.heads, base.seq_len, base.d_head, r, b,
                                                     base.chunk_len, torch.float32), dtype=torch.uint8, device="cuda")
                o = torch.empty_like(v)
                ms = time_calls(lambda: nat.attention(qk, v, rot, b, w0.chunk_len, w0.causal, n_rounds=r,  # noqa: B023
                                                      workspace=ws, out=o), 10, 2)
                rows.append({"qk": label, "n_buckets": b, "n_rounds": r, "rel_err": round(err, 5), "ms": round(ms, 4)})
                log(args, f"[sweep] {label:10s} b={b:4d} r={r}: {err:.4f}  {ms:.3f} ms")
    # cost at the 64K-token text shape
    text = W.WORKLOADS["text_64k"]
    t_in = W.make_inputs(text)
    qk = torch.from_numpy(t_in.qk_bits.view(np.int16)).view(torch.bfloat16).cuda()
    v = torch.from_numpy(t_in.v_bits.view(np.int16)).view(torch.bfloat16).cuda()
    cost = []
    for b in [64, 256, 1024, 4096]:
        for r in rounds:
            g = np.random.default_rng(np.random.SeedSequence([20200104, 990, b, r]))
            rot = torch.from_numpy(g.standard_normal((r, text.d_head, b // 2), dtype=np.float32)).cuda()
            ws = torch.empty(nat.workspace_bytes(text.batch, text.heads, text.seq_len, text.d_head, r, b,
                                                 text.chunk_len, torch.bfloat16), dtype=torch.uint8, device="cuda")
            o = torch.empty_like(v)
            ms = time_calls(lambda: nat.attention(qk, v, rot, b, text.chunk_len, text.causal, n_rounds=r,  # noqa: B023
                                                  workspace=ws, out=o), 10, 3)
            cost.append({"n_buckets": b, "n_rounds": r, "ms": round(ms, 4)})
            log(args, f"[sweep-cost] text_64k b={b:5d} r={r}: {ms:.3f} ms")
            del ws, o
    print(json.dumps({"accuracy_sweep": rows, "shape": {"batch": base.batch, "heads": base.heads,
                      "seq_len": base.seq_len, "d_head": base.d_head, "chunk_len": base.chunk_len,
                      "causal": base.causal, "dtype": "f32"},
                      "reference": "full shared-QK attention (one bucket, one chunk) in the same library",
                      "cost_text_64k": cost}), flush=True)


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
        # tokens as in the main metric (batch x positions); head-tokens beside them
        "value": round(B * L / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded iid normal q, k, v)",
        "config": {"workload": f"local_{w.name}", "batch": B, "heads": H, "seq_len": L, "d_head": d, "chunk_len": m,
                   "n_before": nb, "n_after": na, "causal": w.causal},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "kernel": "local_ring_kernel", "traffic": None},
        "flops_per_token": 4 * window * d,
        "head_tokens_per_s": round(N / (ms / 1e3), 1),
    }
    print(json.dumps(line), flush=True)



def backward_work(w):
    """Algorithmic flops and HBM bytes of one backward with the forward's normaliser.

    Flops per head-token and round: the key role S, dP, dV and dK for the 2m
    queries that see a key (4 * 2 * 2m * d), the query role S, dP and dQ over
    the window (3 * 2 * 2m * d).  Bytes per head-token: the stats pass reads
    out and dout and the saved normaliser and writes Z and D; each round
    gathers the qk, v and dout rows once and reads the perm entry, Z and D;
    the float32 dqk and dv rows are written in round 0 and read and written in
    every later round."""
    N = w.batch * w.heads * w.seq_len
    win = min(2 * w.chunk_len, w.seq_len)
    d, r = w.d_head, w.n_rounds
    e = 2 if w.dtype == "bf16" else 4
    flops = N * r * (4 + 3) * 2 * win * d
    stats = 2 * d * e + 4 + 8
    gather = 3 * d * e + 4 + 8
    grads = 2 * 4 * d + (r - 1) * 2 * (2 * 4 * d)
    return flops, N * (stats + r * gather + grads)


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
    (2 * 2m * d).  The pass is bound by its bytes (counted below), so the
    roofline is HBM's, with the matrix-core fraction beside it.
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
    flops, hbm_bytes = backward_work(w)
    ach = flops / (ms / 1e3) / 1e12
    # bf16 inputs run every contraction on the bf16 MFMA, float32 inputs on the float32 MFMA
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    gbs = hbm_bytes / (ms / 1e3) / 1e9
    line = {
        "metric": "LSH-attention backward tokens/sec (grads wrt qk and v)",
        "value": round(w.tokens / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded)",
        "config": {"workload": f"backward_{w.name}", "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "d_head": w.d_head, "n_buckets": w.n_buckets, "chunk_len": w.chunk_len, "n_rounds": w.n_rounds,
                   "causal": w.causal, "normaliser": "saved by the forward (lse)"},
        # the bytes bind: at the MFMA peak the contractions would take a fraction of the time HBM needs
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "bwd_*_kernel (whole pass)", "traffic": None,
                     "algorithmic_bytes": int(hbm_bytes),
                     "mfma": {"achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4)}},
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


def gemm_context(ach_tflops):
    """What the vendor bf16 GEMM sustains on this machine with iid normal operands
    (8192 x 8192 x 8192, the practical matrix-core ceiling under the power
    limit), next to the hash's executed matrix work: its bf16 pass at the
    algorithmic rate plus the fp6 correction pass, which costs a quarter of
    the bf16 time per flop."""
    import torch

    n = 8192
    g = torch.Generator(device="cuda").manual_seed(1234)
    a = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16).t().contiguous()
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    ms = time_calls(lambda: torch.matmul(a, b, out=c), 50, 50)
    del a, b, c
    gemm = 2.0 * n ** 3 / (ms / 1e3) / 1e12
    executed = ach_tflops * (1.0 + MFMA_BF16_PEAK_TFLOPS / MFMA_FP6_PEAK_TFLOPS)
    return {"vendor_bf16_gemm_tflops": round(gemm, 1), "gemm": f"{n}x{n}x{n} torch.matmul, iid normal operands",
            "hash_executed_tflops": round(executed, 1), "hash_executed_vs_gemm": round(executed / gemm, 4)}


def mfma_ceiling(args):
    """Sustained bf16 matrix-core rate of the chip, measured with the vendor
    GEMM (8192 x 8192 x 8192, bf16 in, float32 accumulate) on iid normal
    operands, on constant operands and on zeros.  The dense peak assumes the
    full clock; with operands whose bits toggle the chip reaches its power
    limit and lowers the clock, so the random-operand rate is the practical
    ceiling for a kernel that keeps the matrix cores busy on real data."""
    import torch

    n = 8192
    g = torch.Generator(device="cuda").manual_seed(1234)
    res = {}
    for label in ("random", "constant", "zeros"):
        if label == "random":
            a = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
            b = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16).t().contiguous()
        elif label == "constant":
            a = torch.full((n, n), 0.5, device="cuda", dtype=torch.bfloat16)
            b = torch.full((n, n), 0.25, device="cuda", dtype=torch.bfloat16)
        else:
            a = torch.zeros((n, n), device="cuda", dtype=torch.bfloat16)
            b = torch.zeros((n, n), device="cuda", dtype=torch.bfloat16)
        c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
        ms = time_calls(lambda: torch.matmul(a, b, out=c), max(args.steps, 10), max(args.warmup, 3))  # noqa: B023
        tf = 2.0 * n ** 3 / (ms / 1e3) / 1e12
        res[label] = {"ms": round(ms, 3), "tflops": round(tf, 1), "frac_of_dense_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        log(args, f"[mfma-ceiling] {label}: {ms:.3f} ms, {tf:.0f} TFLOP/s")
        del a, b, c
    # The unfused alternative to the hash at this workload's shape: the vendor
    # GEMM forming every projection x . R (bf16 out), without the argmax.
    from efficient_long_sequence_lsh_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    N, d, cols = w.batch * w.heads * w.seq_len, w.d_head, w.n_rounds * (w.n_buckets // 2)
    unfused = None
    if cols > 0 and N * cols * 2 <= (8 << 30):
        x = torch.randn((N, d), device="cuda", generator=g).to(torch.bfloat16)
        rr = torch.randn((d, cols), device="cuda", generator=g).to(torch.bfloat16)
        p = torch.empty((N, cols), device="cuda", dtype=torch.bfloat16)
        ms = time_calls(lambda: torch.matmul(x, rr, out=p), max(args.steps, 10), max(args.warmup, 3))
        tf = 2.0 * N * d * cols / (ms / 1e3) / 1e12
        unfused = {"shape": f"{N}x{d} . {d}x{cols}", "ms": round(ms, 3), "tflops": round(tf, 1)}
        log(args, f"[mfma-ceiling] projections of {w.name} as one bf16 GEMM: {ms:.3f} ms, {tf:.0f} TFLOP/s")
        del x, rr, p
    print(json.dumps({"mfma_ceiling": res, "gemm": f"{n}x{n}x{n} bf16 torch.matmul",
                      "dense_peak_tflops": MFMA_BF16_PEAK_TFLOPS, "unfused_projection_gemm": unfused}),
          flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.ingest_traffic:
        ingest_traffic(args)
        return
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
    if args.mfma_ceiling:
        mfma_ceiling(args)
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
    memory = None if args.profile_stage else peak_memory(nat, w, qk, v, rot)
    st = Stages(nat, w, qk, v, rot)
    if args.profile_stage:
        profile_stage(args, st, w)
        return

    log(args, f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    for _ in range(args.warmup):
        st.full()
    torch.cuda.synchronize()
    # one event between consecutive steps on the launch stream: the total
    # over the K steps gives ms_per_step, the per-step spans the spread
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(args.steps):
        st.full()
        marks[i + 1].record()
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[-1]) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    value = w.tokens / (ms / 1e3)

    def pct(q):
        return round(per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))], 4)

    spread = {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9), "min": round(per_step[0], 4),
              "max": round(per_step[-1], 4)}
    log(args, f"[bench] {ms:.3f} ms/step (median {spread['median']}, p10 {spread['p10']}, p90 {spread['p90']}), "
              f"{value:.4g} tokens/s")

    # Per-kernel durations of the pipeline's own launches: HIP events recorded
    # by the library at its kernel boundaries on this stream, every timed step.
    events = [torch.cuda.Event(enable_timing=True) for _ in range(nat.TIMED_EVENTS)]
    for ev in events:
        ev.record()                       # creates the underlying hipEvent_t
    torch.cuda.synchronize()
    # the hashing kernel re-decides its own near-ties: "hash" spans events 1..3
    spans = {"hash_setup": (0, 1), "hash": (1, 3), "sort": (3, 4), "attend": (4, 5), "combine": (5, 6)}
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
                        "unit": r["unit"], "frac": r["frac"], **other_resource(name, stage_ms[name], w)}
    stages["hash_setup"] = {"ms": round(stage_ms["hash_setup"], 4)}
    path = path_roofline(ms, w)
    occ = occupancy(st, w)
    mfma_ctx = gemm_context(stages["hash"]["achieved"]) if w.dtype == "bf16" else None

    cpu = parity = None
    if not args.no_cpu_baseline:
        log(args, f"[bench] cpu baseline: oracle on {args.cpu_heads} slices")
        cpu, results = cpu_baseline(w, inp, args.cpu_heads)
        parity = parity_vs_oracle(st, w, results)
        log(args, f"[bench] parity: {parity}")

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
        "head_tokens_per_s": round(w.batch * w.heads * w.seq_len / (ms / 1e3), 1),
        "path_roofline": path,
        "mfma_context": mfma_ctx,
        "occupancy": occ,
        "ms_per_step_spread": spread,
        "memory": memory,
        "stages": stages,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
