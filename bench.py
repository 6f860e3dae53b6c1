"""Benchmark of the DSA draft-and-verify hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  indexer scores (draft step 1) -> top-k -> sparse attention for the G = 7
  draft steps reusing the step-1 indices (IndexShare) -> rejection-sampling
  verification of the drafted chains over the vocabulary.

Default workload (the largest single-GPU configuration): batched decode of 16
sequences with contexts uniform in [16,384, 65,536] (seeded), K/V and index
keys paged in 64-token blocks from one shuffled physical pool; indexer 64
heads x 128 bf16 with one shared index key per position; top-k 2048;
attention 64 heads x 128 bf16 per-head KV; 7 draft steps; verification of
each sequence's 7 drafts + bonus over a 151,552-token vocabulary (target
logits N(0, 2^2), draft = target + N(0, 1)).  Inputs are seeded synthetic
data already resident in HBM.  --workload decode_32k runs the single-sequence
32K step instead.

Prints one JSON line: value = G * sum(context) / step time (draft-step
sparse-attention context tokens/s), verified positions/s, a roofline object
for the dominant kernel (sparse attention, HBM-bound) with its cache-flushed
fraction, per-kernel side measurements on every configuration (warm and
cache-flushed), and the CPU oracle timed on the host cores per configuration.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0              # MI355X datasheet
BF16_MFMA_PEAK_TFLOPS = 2500.0     # MI355X datasheet, dense
FLUSH_BYTES = 1 << 30              # read-modify-write before each cache-flushed launch
METRIC = "draft-step sparse-attn context tokens/s + verified positions/s; % of HBM roofline"
WORKLOADS = ("batched_16x16k_64k", "decode_32k")
# positions with a launch of their own in the library's early-exit verify
# schedules (rejection sampling, greedy); the rest is read in one launch
VERIFY_PHASED_POSITIONS = 4
GREEDY_PHASED_POSITIONS = 2
EXTRA_GROUPS = ("peaks", "decode_32k", "verify", "indexer_1m", "long_1m", "cross_layer", "verify_pass", "topk")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOADS[0], choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the oracle on the headline workload")
    ap.add_argument("--no-extras", action="store_true", help="skip the side measurements")
    ap.add_argument("--extras-only", action="store_true",
                    help="only the side measurements (for profiling them on their own)")
    ap.add_argument("--extras-reps", type=int, default=20, help="graph replays per side measurement")
    ap.add_argument("--extras", default=",".join(EXTRA_GROUPS),
                    help="comma-separated side measurement groups: " + ", ".join(EXTRA_GROUPS))
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy (HBM counter calibration)")
    return ap.parse_args()


def calibrate_copy():
    import torch
    n = 256 * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 5}), flush=True)


# ----------------------------------------------------------------------------
# traffic counters (committed rocprofv3 summary, valid for one kernel source)
# ----------------------------------------------------------------------------
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "mha_attn_batched_16x16k_64k_hbm_traffic.txt")
ATTN_SOURCE = os.path.join(ROOT, "dsa_sparse_attention_lightning_amd", "csrc", "sparse_attn.hip")
TRAFFIC_KERNELS = ("void mha_attn_kernel", "void combine_kernel<128")


def measured_traffic():
    """HBM bytes per attention call (every kernel of the call) from the
    committed rocprofv3 counter summary, or None when the kernel source has
    changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    src = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()[:16]
    if f"sha256[:16] at measurement time: {src}" not in text:
        return None
    total = 0.0
    for line in text.splitlines():
        if line.startswith(TRAFFIC_KERNELS):
            total += float(line.split()[-1]) * 1e6
    return total or None


def progress(msg):
    """One line per finished piece of work, on stderr (stdout carries only
    the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# timing helpers
# ----------------------------------------------------------------------------
_FLUSH = None


def _flush(clean=True):
    """Evicts the L2 caches and the 256 MiB last-level cache: a 1 GiB
    read-modify-write, enqueued eagerly on the current stream.  clean=True
    then reads another 1 GiB, so the last-level cache holds clean unrelated
    lines (the timed call pays no write-back of the flush's dirty lines)."""
    import torch
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = (torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0"),
                  torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0"),
                  torch.zeros(1, dtype=torch.int64, device="cuda:0"))
    rmw, sweep, acc = _FLUSH
    rmw.add_(1)
    if clean:
        torch.sum(sweep, dim=(0,), dtype=torch.int64, out=acc[0])


def _capture(fn, inner=1):
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for _ in range(inner):
            fn()
    return g


def _warm(g, warm_s=0.05):
    import torch
    t_end, n = time.perf_counter() + warm_s, 0
    while n < 3 or time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
        n += 1


def time_warm(fn, reps=20, inner=8):
    """Average duration (us) of one call of `fn` with its inputs warm in the
    caches: `inner` calls captured back to back in one HIP graph, replayed
    `reps` times and timed with events on the launch stream, after at least
    50 ms of untimed replays (a cold start measured 2-3 % slow)."""
    import torch
    g = _capture(fn, inner)
    _warm(g)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (reps * inner)


def time_flushed(fn, reps=20, clean=True):
    """Average duration (us) of one call of `fn` after a cache flush: each
    repetition enqueues the flush eagerly, then one eager call bracketed by
    events on the launch stream.  The figure includes one launch's latency
    (EVENT_OVERHEAD_US measures it for an empty call)."""
    import torch
    fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = []
    for _ in range(reps):
        _flush(clean)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return 1e3 * sum(a.elapsed_time(b) for a, b in evs) / reps


def launch_overhead_us(reps=20):
    """time_flushed of a one-element kernel: the latency a single timed
    launch carries beyond its own work."""
    import torch
    x = torch.zeros(1, device="cuda:0")
    return time_flushed(lambda: x.add_(1), reps)


def hbm_entry(nbytes, us_warm, us_cold, peaks):
    out = {"algorithmic_bytes": nbytes, "us_warm": us_warm, "us_flushed": us_cold,
           "GBps_warm": nbytes / us_warm / 1e3, "GBps_flushed": nbytes / us_cold / 1e3,
           "frac_hbm_warm": nbytes / us_warm / 1e3 / HBM_PEAK_GBS,
           "frac_hbm_flushed": nbytes / us_cold / 1e3 / HBM_PEAK_GBS}
    if peaks.get("read_GBps"):
        out["frac_measured_read_flushed"] = nbytes / us_cold / 1e3 / peaks["read_GBps"]
    return out


def mfma_entry(flops, us_warm, us_cold, peaks):
    out = {"flops": flops, "us_warm": us_warm, "us_flushed": us_cold,
           "TFLOPs_warm": flops / us_warm / 1e6, "TFLOPs_flushed": flops / us_cold / 1e6,
           "frac_mfma_warm": flops / us_warm / 1e6 / BF16_MFMA_PEAK_TFLOPS,
           "frac_mfma_flushed": flops / us_cold / 1e6 / BF16_MFMA_PEAK_TFLOPS}
    if peaks.get("mfma_bf16_TFLOPs"):
        out["frac_measured_mfma_flushed"] = flops / us_cold / 1e6 / peaks["mfma_bf16_TFLOPs"]
    return out


# ----------------------------------------------------------------------------
# measured peaks
# ----------------------------------------------------------------------------
def measure_peaks(reps=10):
    """Measured peaks on this GPU (libdsa_bench.so): the HBM read stream and
    copy bandwidth of 2 GiB with 16-byte non-temporal accesses (each
    workgroup its own contiguous chunk; copy counts bytes read + written),
    and the dense bf16 MFMA rate of a register-only loop."""
    import torch
    path = os.path.join(ROOT, "dsa_sparse_attention_lightning_amd", "libdsa_bench.so")
    if not os.path.exists(path):
        return {}
    lib = ctypes.CDLL(path)
    for fn in (lib.dsa_bench_mfma_peak, lib.dsa_bench_mfma16_peak):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.dsa_bench_stream.restype = ctypes.c_int
    lib.dsa_bench_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                                     ctypes.c_int, ctypes.c_void_p]
    cur = lambda: torch.cuda.current_stream().cuda_stream
    n = 2 << 30
    blocks = 256 * 8
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")

    def read():
        assert lib.dsa_bench_stream(src.data_ptr(), None, out.data_ptr(), n, blocks, cur()) == 0

    def copy():
        assert lib.dsa_bench_stream(src.data_ptr(), dst.data_ptr(), out.data_ptr(), n, blocks, cur()) == 0

    peaks = {"read_GBps": n / time_warm(read, reps=reps, inner=2) / 1e3,
             "copy_GBps": 2 * n / time_warm(copy, reps=reps, inner=2) / 1e3, "stream_bytes": n}
    del src, dst, out
    blocks, iters = 256 * 8, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")

    def mfma32():
        assert lib.dsa_bench_mfma_peak(out.data_ptr(), blocks, iters, cur()) == 0

    blocks16, iters16 = 256, 1024   # 512-thread workgroups, one per CU

    def mfma16():
        assert lib.dsa_bench_mfma16_peak(out.data_ptr(), blocks16, iters16, cur()) == 0

    flops = blocks * 4 * iters * 4 * 2 * 32 * 32 * 16
    flops16 = blocks16 * 8 * iters16 * 32 * 2 * 16 * 16 * 32
    peaks["mfma_bf16_32x32x16_TFLOPs"] = flops / time_warm(mfma32, reps=reps, inner=1) / 1e6
    peaks["mfma_bf16_16x16x32_TFLOPs"] = flops16 / time_warm(mfma16, reps=reps, inner=1) / 1e6
    peaks["mfma_bf16_TFLOPs"] = max(peaks["mfma_bf16_32x32x16_TFLOPs"], peaks["mfma_bf16_16x16x32_TFLOPs"])
    peaks["probes"] = ("libdsa_bench.so: 2 GiB stream, 16-byte non-temporal loads (copy: and stores), 2048 "
                       "workgroups each on a contiguous chunk; register-only v_mfma_f32_32x32x16_bf16 and "
                       "v_mfma_f32_16x16x32_bf16 loops on pseudo-random full-mantissa bf16 operands, 4 chains "
                       "per wave, 8 waves per CU, accumulators in AGPRs and in ArchVGPRs respectively "
                       "(mfma_bf16_TFLOPs: the higher of the two)")
    torch.cuda.empty_cache()
    return peaks


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
def build_workload(name):
    import dsa_inputs as I
    from dsa_inputs import device as DI
    if name == "batched_16x16k_64k":
        d = DI.draft_inputs(2, I.batched_lens(2), H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048,
                            G=7, shuffle_pages=True)
        v = DI.verify_inputs(102, d.B, 7, 151552, 2.0)
        desc = ("batched_16x16k_64k: 16 sequences, contexts uniform in [16384, 65536] (seeded), K/V and index "
                "keys paged 64 from one shuffled pool, indexer 64x128, top-k 2048, MHA 64x128, 7 draft steps "
                "(IndexShare), verify 7+1 x vocab 151552 per sequence")
    elif name == "decode_32k":
        d = DI.draft_inputs(1, [32768], H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048, G=7)
        v = DI.verify_inputs(101, 1, 7, 151552, 2.0)
        desc = ("decode_32k: 1 sequence, context 32768, indexer 64x128, top-k 2048, MHA 64x128 paged 64, "
                "7 draft steps (IndexShare), verify 7+1 x vocab 151552")
    else:
        raise ValueError(name)
    return d, v, desc


def attn_bytes(d):
    """Algorithmic bytes of one sparse-attention call: the selected K and V
    rows of every KV head, plus q, idx, out and lse."""
    n_sel = sum(min(d.k, L) for L in d.lens)
    return (n_sel * d.H_kv * (d.D_qk + d.D_v) * 2 + d.B * d.H_q * d.D_qk * 2 + d.B * d.k * 4
            + d.B * d.H_q * d.D_v * 4 + d.B * d.H_q * 4)


class Path:
    """Persistent outputs and workspaces of one workload, and the phase
    callables (no allocation inside them)."""

    def __init__(self, dsa, d, v):
        import torch
        dev = "cuda:0"
        self.dsa, self.d, self.v = dsa, d, v
        B, k = d.B, d.k
        self.scores = torch.empty((B, 1, d.ld), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
        self.topk_ws = torch.empty(max(1, dsa.topk_workspace_size(B, 1, d.ld, k)), dtype=torch.uint8, device=dev)
        self.outs = torch.empty((d.G, B, 1, d.H_q, d.D_v), dtype=torch.float32, device=dev)
        self.lses = torch.empty((d.G, B, 1, d.H_q), dtype=torch.float32, device=dev)
        self.attn_ws = torch.zeros(max(1, dsa.sparse_attn_workspace_size(B, 1, d.H_q, d.H_kv, d.D_qk, d.D_v, k)),
                                   dtype=torch.uint8, device=dev)
        Bv, Gv, V = v.draft_logits.shape
        self.acc_len = torch.empty(Bv, dtype=torch.int32, device=dev)
        self.emitted = torch.empty((Bv, Gv + 1), dtype=torch.int32, device=dev)
        self.ver_ws = torch.empty(max(1, dsa.spec_verify_workspace_size(Bv, Gv, V)), dtype=torch.uint8, device=dev)

    def indexer(self):
        d = self.d
        self.dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, d.row_len, page=d.page, out=self.scores)

    def select(self):
        self.dsa.topk(self.scores, self.d.row_len, self.d.k, out=self.idx, workspace=self.topk_ws)

    def attend_one(self, j=0):
        d = self.d
        self.dsa.sparse_attn(d.q[j][:, None], d.k_cache, d.v_cache, d.block_table, self.idx[:, 0], page=d.page,
                             D_v=d.D_v, sm_scale=d.sm_scale, out=self.outs[j], lse=self.lses[j],
                             workspace=self.attn_ws)

    def attend(self):
        for j in range(self.d.G):
            self.attend_one(j)

    def verify(self):
        v = self.v
        self.dsa.spec_verify(v.target_logits, v.draft_logits, v.drafts, seed=v.seed, offset=v.offset,
                             accepted_len=self.acc_len, emitted=self.emitted, workspace=self.ver_ws)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch
    import dsa_sparse_attention_lightning_amd as dsa
    torch.cuda.set_device(0)
    if args.extras_only:
        print(json.dumps({"extras": extra_measurements(dsa, args.extras_reps, args.extras.split(","), {})}),
              flush=True)
        return
    import numpy as np

    d, v, desc = build_workload(args.workload)
    p = Path(dsa, d, v)
    G = d.G

    # The step is one HIP graph (indexer, top-k, G attention launches,
    # verify); per-phase graphs give the breakdown.
    phases = [("indexer", p.indexer), ("topk", p.select), ("attn", p.attend), ("verify", p.verify)]
    for _, fn in phases:          # eager warm-up (loads code objects, checks arguments)
        fn()
    torch.cuda.synchronize()
    g_step = _capture(lambda: [fn() for _, fn in phases])
    g_block = _capture(lambda: [fn() for n, fn in phases if n != "verify"])
    g_phase = {n: _capture(fn) for n, fn in phases}
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()

    # timed region: K whole-step replays, bracketed by synchronisation
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        g_step.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gpu_ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # per-phase replays timed with events on the launch stream; the attention
    # graph holds the G sparse-attention launches of one step
    names = [n for n, _ in phases] + ["draft_block"]
    graphs = dict(g_phase, draft_block=g_block)
    per = {n: [] for n in names}
    for _ in range(args.steps):
        for n in names:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graphs[n].replay()
            b.record(stream)
            per[n].append((a, b))
    torch.cuda.synchronize()
    phase_us = {n: 1e3 * float(np.mean([a.elapsed_time(b) for a, b in per[n]])) for n in names}
    attn_us = phase_us["attn"] / G
    acc = p.acc_len.cpu().numpy()
    progress(f"{args.workload}: {args.steps} timed steps, {ms_per_step:.3f} ms/step")

    # the dominant kernel after a cache flush (one call per flush)
    peaks = measure_peaks() if (not args.no_extras and "peaks" in args.extras.split(",")) else {}
    attn_us_cold = time_flushed(lambda: p.attend_one(0), reps=args.extras_reps)
    attn_us_dirty = time_flushed(lambda: p.attend_one(0), reps=args.extras_reps, clean=False)
    overhead_us = launch_overhead_us()

    L_total = sum(d.lens)
    abytes = attn_bytes(d)
    achieved = abytes / (attn_us * 1e-6) / 1e9
    idx_bytes = L_total * d.D_I * 2 + L_total * 4 + d.B * d.H_I * (d.D_I * 2 + 4)
    topk_bytes = L_total * 4 + d.B * d.k * 4
    Bv, Gv, V = v.draft_logits.shape
    ver_bytes = Bv * (2 * Gv + 1) * V * 4
    value = G * L_total / (ms_per_step * 1e-3)
    split = dsa.sparse_attn_workspace_size(d.B, 1, d.H_q, d.H_kv, d.D_qk, d.D_v, d.k) > 0
    roofline = {
        "bound": "hbm",
        "kernel": "dsa_sparse_attn call (mha_attn_kernel" + (" + split-k combine_kernel)" if split else ")"),
        "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
        "traffic": measured_traffic(),
        "traffic_source": os.path.relpath(TRAFFIC_PROFILE, ROOT) + " (FETCH_SIZE x2.0 + WRITE_SIZE x1.0 per call, "
                          "copy-calibrated; null when the attention source differs from the measured one)",
        "bytes_per_launch": abytes, "avg_launch_us": attn_us,
        "timing": "HIP events on the launch stream around replays of a graph of one step's G attention calls, "
                  "divided by G (steps 2..G re-read the rows step 1 gathered: IndexShare)",
        "flushed": {"avg_launch_us": attn_us_cold, "achieved": abytes / attn_us_cold / 1e3,
                    "frac": abytes / attn_us_cold / 1e3 / HBM_PEAK_GBS,
                    "avg_launch_us_dirty": attn_us_dirty,
                    "frac_dirty": abytes / attn_us_dirty / 1e3 / HBM_PEAK_GBS,
                    "launch_overhead_us": overhead_us,
                    "timing": "one eager call between events after a 1 GiB read-modify-write and a 1 GiB read "
                              "(the last-level cache then holds clean unrelated lines); _dirty: after the "
                              "read-modify-write only; launch_overhead_us: the same for an empty call"},
    }
    if peaks.get("read_GBps"):
        roofline["measured_read_GBps"] = peaks["read_GBps"]
        roofline["frac_of_measured_read"] = achieved / peaks["read_GBps"]
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": gpu_ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the pages' decode workloads)",
        "config": {"workload": desc, "global_batch": d.B, "context_total": int(L_total), "draft_steps": G,
                   "parallelism": "none (1 GPU)"},
        "verified_positions_per_s": Bv * (Gv + 1) / (ms_per_step * 1e-3),
        "draft_block_context_tokens_per_s": G * L_total / (phase_us["draft_block"] * 1e-6),
        "roofline": roofline,
        "phases_us": phase_us,
        "phases_roofline": {
            "indexer": {"bytes": idx_bytes, "GBps": idx_bytes / phase_us["indexer"] / 1e3,
                        "frac_hbm": idx_bytes / phase_us["indexer"] / 1e3 / HBM_PEAK_GBS},
            "topk": {"bytes": topk_bytes, "GBps": topk_bytes / phase_us["topk"] / 1e3},
            "verify": {"bytes": ver_bytes, "GBps": ver_bytes / phase_us["verify"] / 1e3,
                       "frac_hbm": ver_bytes / phase_us["verify"] / 1e3 / HBM_PEAK_GBS},
        },
        "graph": "each timed step is one replay of a HIP graph holding the whole step",
        "mean_accepted_len": float(acc.mean()),
    }
    if peaks:
        result["measured_peaks"] = peaks
    headline_cpu = None
    if not args.no_cpu_baseline:
        headline_cpu = cpu_baseline_draft(d, v, p.idx, args.cpu_seconds)
        result["cpu_baseline"] = headline_cpu
        progress(f"cpu baseline: {headline_cpu['sample']}")
    del p, d, v, g_step, g_block, g_phase
    torch.cuda.empty_cache()
    if not args.no_extras:
        result["extras"] = extra_measurements(dsa, args.extras_reps, args.extras.split(","), peaks,
                                              cpu=not args.no_cpu_baseline)
    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------------------
# side measurements (other configurations; not the headline)
# ----------------------------------------------------------------------------
def extra_measurements(dsa, reps=20, groups=EXTRA_GROUPS, peaks=None, cpu=False):
    """Per-kernel measurements on every configuration, warm (inputs resident
    in the caches, as IndexShare re-reads them) and cache-flushed (one call
    after a 1 GiB read-modify-write):
      peaks       measured copy bandwidth and bf16 MFMA rate;
      decode_32k  the single-sequence 32K draft block and its kernels;
      verify      spec_verify on 256 x 8 x 151,552 at logit scales 0.5, 2, 6
                  (mean accepted length next to its closed form), and greedy;
      indexer_1m  the indexer at 2^20 positions, R = 1 (HBM) and R = 8 (MFMA);
      long_1m     the 1M-context latent-MQA draft block;
      cross_layer a 4-layer cross-layer IndexShare block at 32K;
      verify_pass the 8-row verify-pass DSA step at 32K;
      topk        single-row top-k at 32K and 2^20."""
    peaks = dict(peaks or {})
    out = {}
    if "peaks" in groups and not peaks:
        peaks = measure_peaks()
        out["measured_peaks"] = peaks
    for g in groups:
        if g == "peaks":
            continue
        t0 = time.perf_counter()
        out.update(_EXTRAS[g](dsa, reps, peaks, cpu))
        progress(f"side measurement {g} done in {time.perf_counter() - t0:.1f} s")
    return out


def _extra_decode_32k(dsa, reps, peaks, cpu):
    import torch
    d, v, _ = build_workload("decode_32k")
    p = Path(dsa, d, v)
    p.indexer(), p.select()
    us_block = time_warm(lambda: (p.indexer(), p.select(), p.attend()), reps, inner=2)
    L = d.lens[0]
    ab = attn_bytes(d)
    ib = L * d.D_I * 2 + L * 4
    res = {"decode_32k": {
        "us_draft_block": us_block, "context_tokens_per_s": d.G * L / (us_block * 1e-6),
        "attention_call": hbm_entry(ab, time_warm(p.attend_one, reps), time_flushed(p.attend_one, reps), peaks),
        "indexer": hbm_entry(ib, time_warm(p.indexer, reps), time_flushed(p.indexer, reps), peaks),
        "topk_us_warm": time_warm(p.select, reps), "topk_us_flushed": time_flushed(p.select, reps),
        "verify_1seq_us": time_warm(p.verify, reps)}}
    if cpu:
        res["decode_32k"]["cpu_oracle"] = cpu_baseline_draft(d, v, p.idx, 3.0)
    del p, d, v
    torch.cuda.empty_cache()
    return res


def _closed_form_mean_accepted(v):
    """E[n] = sum_m prod_{j<=m} alpha_j per sequence, alpha_j = sum_x
    min(p_j, q_j) (closed form of the chain length), averaged over the batch;
    computed with torch on the device as a diagnostic, row by row."""
    import torch
    B, G, V = v.draft_logits.shape
    alpha = torch.empty((B, G), dtype=torch.float64, device=v.draft_logits.device)
    for j in range(G):
        pj = torch.softmax(v.target_logits[:, j].double(), dim=-1)
        qj = torch.softmax(v.draft_logits[:, j].double(), dim=-1)
        alpha[:, j] = torch.minimum(pj, qj).sum(-1)
        del pj, qj
    return float(torch.cumprod(alpha, dim=1).sum(dim=1).mean())


class _schedule:
    """Sets DSA_VERIFY_SCHEDULE (the library reads it per call) for a block,
    then restores what was there."""

    def __init__(self, name):
        self.name, self.old = name, None

    def __enter__(self):
        self.old = os.environ.get("DSA_VERIFY_SCHEDULE")
        os.environ["DSA_VERIFY_SCHEDULE"] = self.name

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("DSA_VERIFY_SCHEDULE", None)
        else:
            os.environ["DSA_VERIFY_SCHEDULE"] = self.old
        return False


def _extra_verify(dsa, reps, peaks, cpu):
    import torch
    from dsa_inputs import device as DI
    out = {}
    B, G, V = 256, 7, 151552
    n = torch.empty(B, dtype=torch.int32, device="cuda:0")
    em = torch.empty((B, G + 1), dtype=torch.int32, device="cuda:0")
    ws = torch.empty(dsa.spec_verify_workspace_size(B, G, V), dtype=torch.uint8, device="cuda:0")
    vbytes = B * (2 * G + 1) * V * 4
    for std, seed in ((0.5, 4), (2.0, 5), (6.0, 6)):
        v = DI.verify_inputs(seed, B, G, V, std, offset=11)

        def call():
            dsa.spec_verify(v.target_logits, v.draft_logits, v.drafts, seed=v.seed, offset=v.offset,
                            accepted_len=n, emitted=em, workspace=ws)

        # default schedule (early exit at this size): bytes it reads, from the
        # accepted lengths.  Positions 0..P-1 have a launch each (both rows of
        # a position are read while the chain is accepted); a chain that
        # reaches P reads all its remaining rows in one launch; then the
        # sampled rows are read once more for the draw.
        us_w, us_c = time_warm(call, reps, inner=2), time_flushed(call, max(5, reps // 2))
        nn = n.cpu().long()
        P = min(VERIFY_PHASED_POSITIONS, G)
        redraw = torch.where(nn < G, 2, 1)
        rows = torch.where(nn < P, 2 * (nn + 1), 2 * G + 1) + redraw
        e = hbm_entry(int(rows.sum()) * V * 4, us_w, us_c, peaks)
        e["schedule"] = "early exit (rows past each chain's first rejection are not read)"
        e["all_rows_bytes"] = vbytes
        e["all_rows_GBps_flushed"] = vbytes / us_c / 1e3   # rate at which the batch's logits are consumed
        # the one-pass schedule on the same batch: every row read once (the
        # stats pass), the bandwidth figure of a full read
        with _schedule("onepass"):
            e["onepass"] = hbm_entry(vbytes, time_warm(call, reps, inner=2), time_flushed(call, max(5, reps // 2)),
                                     peaks)
        e.update({"verified_positions_per_s_flushed": B * (G + 1) / (us_c * 1e-6),
                  "verified_positions_per_s_warm": B * (G + 1) / (us_w * 1e-6),
                  "mean_accepted_len": float(n.float().mean()),
                  "mean_accepted_len_std_err": float(n.float().std() / B ** 0.5),
                  "mean_accepted_len_closed_form": _closed_form_mean_accepted(v)})
        if cpu:
            e["cpu_oracle"] = cpu_baseline_verify(v)
        out[f"verify_256x8x151552_s{std}"] = e
        if std == 2.0:
            # greedy verification of the same batch (greedy drafts: the draft
            # model's argmax); reads only the target rows
            gdr = v.draft_logits.argmax(dim=-1).to(torch.int32)
            gws = torch.empty(dsa.spec_verify_greedy_workspace_size(B, G, V), dtype=torch.uint8, device="cuda:0")

            def gcall():
                dsa.spec_verify_greedy(v.target_logits, gdr, accepted_len=n, emitted=em, workspace=gws)

            # default schedule (early exit): target rows 0..accepted length, or
            # all G+1 once a chain reaches the one-pass tail
            gbytes = B * (G + 1) * V * 4
            us_gw, us_gc = time_warm(gcall, reps, inner=2), time_flushed(gcall, max(5, reps // 2))
            nn = n.cpu().long()
            Pg = min(GREEDY_PHASED_POSITIONS, G)
            e = hbm_entry(int(torch.where(nn < Pg, nn + 1, G + 1).sum()) * V * 4, us_gw, us_gc, peaks)
            e["schedule"] = "early exit (rows past each chain's first mismatch are not read)"
            e["all_rows_bytes"] = gbytes
            e["all_rows_GBps_flushed"] = gbytes / us_gc / 1e3
            with _schedule("onepass"):
                e["onepass"] = hbm_entry(gbytes, time_warm(gcall, reps, inner=2),
                                         time_flushed(gcall, max(5, reps // 2)), peaks)
            e["verified_positions_per_s_flushed"] = B * (G + 1) / (us_gc * 1e-6)
            e["mean_accepted_len"] = float(n.float().mean())
            out["greedy_verify_256x8x151552_s2.0"] = e
            del gdr, gws
        del v
        torch.cuda.empty_cache()
    return out


def _extra_indexer_1m(dsa, reps, peaks, cpu):
    import torch
    from dsa_inputs import device as DI
    out = {}
    L = 1 << 20
    for R in (1, 8):
        d = DI.draft_inputs(3, [L], H_I=64, D_I=128, H_q=64, D_qk=576, D_v=512, k=2048, G=0, R=R, latent=True)
        sc = torch.empty((1, R, d.ld), dtype=torch.float32, device="cuda:0")

        def call():
            dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, d.row_len, page=d.page, out=sc)

        us_w, us_c = time_warm(call, reps), time_flushed(call, reps)
        flops = 2.0 * R * L * d.H_I * d.D_I
        kbytes = L * d.D_I * 2 + R * L * 4
        e = {"hbm": hbm_entry(kbytes, us_w, us_c, peaks), "mfma": mfma_entry(flops, us_w, us_c, peaks)}
        if cpu and R == 8:
            e["cpu_oracle"] = cpu_baseline_indexer(d, R)
        out[f"indexer_1m_R{R}"] = e
        del d, sc
    torch.cuda.empty_cache()
    return out


def _extra_long_1m(dsa, reps, peaks, cpu):
    """The 1M-context draft block (latent MQA): indexer (R = 1) and top-k over
    2^20 positions once, then 7 latent sparse-attention steps reusing the
    indices; phases timed separately and as one graph."""
    import torch
    from dsa_inputs import device as DI
    d = DI.draft_inputs(3, [1 << 20], H_I=64, D_I=128, H_q=64, D_qk=576, D_v=512, k=2048, G=7, latent=True)
    sc = torch.empty((1, 1, d.ld), dtype=torch.float32, device="cuda:0")
    ix = torch.empty((1, 1, d.k), dtype=torch.int32, device="cuda:0")
    tws = torch.empty(max(1, dsa.topk_workspace_size(1, 1, d.ld, d.k)), dtype=torch.uint8, device="cuda:0")
    o = torch.empty((d.G, 1, 1, d.H_q, d.D_v), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((d.G, 1, 1, d.H_q), dtype=torch.float32, device="cuda:0")
    aws = torch.zeros(max(1, dsa.sparse_attn_workspace_size(1, 1, d.H_q, 1, d.D_qk, d.D_v, d.k)), dtype=torch.uint8,
                      device="cuda:0")

    def indexer():
        dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, d.row_len, page=d.page, out=sc)

    def select():
        dsa.topk(sc, d.row_len, d.k, out=ix, workspace=tws)

    def attend_one(j=0):
        dsa.sparse_attn(d.q[j][:, None], d.k_cache, d.v_cache, d.block_table, ix[:, 0], page=d.page,
                        D_v=d.D_v, sm_scale=d.sm_scale, out=o[j], lse=lse[j], workspace=aws)

    def block():
        indexer()
        select()
        for j in range(d.G):
            attend_one(j)

    us_block = time_warm(block, reps, inner=2)
    res = {"us_per_block": us_block, "context_tokens_per_s": d.G * (1 << 20) / (us_block * 1e-6),
           "us_indexer_warm": time_warm(indexer, reps), "us_indexer_flushed": time_flushed(indexer, reps),
           "us_topk_warm": time_warm(select, reps), "us_topk_flushed": time_flushed(select, reps),
           "us_attention_per_step_warm": time_warm(attend_one, reps),
           "us_attention_per_step_flushed": time_flushed(attend_one, reps)}
    if cpu:
        res["cpu_oracle"] = cpu_baseline_latent(d, ix)
    del d, sc, ix, tws, o, lse, aws
    torch.cuda.empty_cache()
    return {"long_1m_latent_draft_block": res}


def _extra_cross_layer(dsa, reps, peaks, cpu):
    import torch
    from dsa_inputs import device as DI
    # cross-layer IndexShare at context 32K: one indexer + top-k serves a block
    # of 4 layers (each with its own queries and KV), against an indexer per layer
    layers = [DI.draft_inputs(40 + l, [32768], H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048, G=1)
              for l in range(4)]
    d0 = layers[0]
    sc = torch.empty((1, 1, d0.ld), dtype=torch.float32, device="cuda:0")
    ix = torch.empty((1, 1, d0.k), dtype=torch.int32, device="cuda:0")
    o = torch.empty((1, 1, d0.H_q, d0.D_v), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((1, 1, d0.H_q), dtype=torch.float32, device="cuda:0")
    aws = torch.zeros(max(1, dsa.sparse_attn_workspace_size(1, 1, 64, 64, 128, 128, 2048)), dtype=torch.uint8,
                      device="cuda:0")

    def select(l):
        dsa.index_scores(l.q_index, l.w, l.kidx, l.block_table, l.row_len, page=l.page, out=sc)
        dsa.topk(sc, l.row_len, l.k, out=ix)

    def attend(l):
        dsa.sparse_attn(l.q[0][:, None], l.k_cache, l.v_cache, l.block_table, ix[:, 0], page=l.page,
                        sm_scale=l.sm_scale, out=o, lse=lse, workspace=aws)

    def shared():
        select(d0)
        for l in layers:
            attend(l)

    def per_layer():
        for l in layers:
            select(l)
            attend(l)

    us_shared = time_warm(shared, reps, inner=4)
    us_per = time_warm(per_layer, reps, inner=4)
    del layers, d0, sc, ix, o, lse, aws
    torch.cuda.empty_cache()
    return {"cross_layer_indexshare_32k_4layers": {
        "us_per_block_shared": us_shared, "us_per_block_indexer_each_layer": us_per, "speedup": us_per / us_shared}}


def _extra_verify_pass(dsa, reps, peaks, cpu):
    import torch
    from dsa_inputs import device as DI
    # verify-pass DSA at context 32K: 8 chained rows (7 drafts + bonus), row r
    # sees [0, L + r + 1); indexer at R = 8, per-row top-k, 8-row attention
    # with per-row index sets
    L, R = 32768, 8
    d = DI.draft_inputs(45, [L], H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048, G=R, R=R)
    rl = torch.arange(L + 1, L + R + 1, dtype=torch.int32, device="cuda:0")[None].contiguous()
    sc = torch.empty((1, R, L + R), dtype=torch.float32, device="cuda:0")
    ix = torch.empty((1, R, d.k), dtype=torch.int32, device="cuda:0")
    qv = d.q[:, 0][None].contiguous()                                   # [1, R, H, D]
    o = torch.empty((1, R, d.H_q, d.D_v), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((1, R, d.H_q), dtype=torch.float32, device="cuda:0")
    aws = torch.zeros(max(1, dsa.sparse_attn_workspace_size(1, R, 64, 64, 128, 128, d.k)), dtype=torch.uint8,
                      device="cuda:0")
    tws = torch.empty(max(1, dsa.topk_workspace_size(1, R, L + R, d.k)), dtype=torch.uint8, device="cuda:0")

    def verify_pass():
        dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, rl, page=d.page, out=sc)
        dsa.topk(sc, rl, d.k, out=ix, workspace=tws)
        dsa.sparse_attn(qv, d.k_cache, d.v_cache, d.block_table, ix, page=d.page, sm_scale=d.sm_scale, out=o,
                        lse=lse, workspace=aws)

    us = time_warm(verify_pass, reps)
    del d, rl, sc, ix, qv, o, lse, aws, tws
    torch.cuda.empty_cache()
    return {"verify_pass_dsa_32k_8rows": {"us_per_call": us, "rows_per_s": R / (us * 1e-6),
                                          "context_tokens_per_s": R * L / (us * 1e-6)}}


def _extra_topk(dsa, reps, peaks, cpu):
    import torch
    out = {}
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(77)
    for L in (32768, 1 << 20):
        sc = torch.randn((1, 1, L), generator=gen, device="cuda:0")
        rl = torch.full((1, 1), L, dtype=torch.int32, device="cuda:0")
        ix = torch.empty((1, 1, 2048), dtype=torch.int32, device="cuda:0")
        ws = torch.empty(max(1, dsa.topk_workspace_size(1, 1, L, 2048)), dtype=torch.uint8, device="cuda:0")

        def call():
            dsa.topk(sc, rl, 2048, out=ix, workspace=ws)

        us_w, us_c = time_warm(call, reps), time_flushed(call, reps)
        out[f"topk_1x{L}_k2048"] = {"us_warm": us_w, "us_flushed": us_c, "GBps_flushed": (L + 2048) * 4 / us_c / 1e3}
    return out


_EXTRAS = {"decode_32k": _extra_decode_32k, "verify": _extra_verify, "indexer_1m": _extra_indexer_1m,
           "long_1m": _extra_long_1m, "cross_layer": _extra_cross_layer, "verify_pass": _extra_verify_pass,
           "topk": _extra_topk}


# ----------------------------------------------------------------------------
# the CPU oracle, timed on the host cores
# ----------------------------------------------------------------------------
def _cpu_threads():
    """Threads the oracle may use: the CPUs this process may run on, capped
    by OMP_NUM_THREADS when set (the host's share for this GPU)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def _blas_limits():
    from threadpoolctl import threadpool_limits
    n = _cpu_threads()
    return n, threadpool_limits(limits=n, user_api="blas")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _f64(t):
    import numpy as np
    return t.float().cpu().numpy().astype(np.float64)


def cpu_baseline_draft(d, v, idx, budget_s):
    """The float64 oracle on full steps of a per-head-KV workload (every
    sequence: indexer over its context, top-k, G attention steps, verification
    of its chain), repeated until the time budget is spent; same unit as the
    GPU value.  The selected K/V rows are handed to the oracle already
    gathered (a float64 copy of the whole cache does not fit the host), so
    its attention does the same work over the same k rows."""
    import numpy as np
    import torch
    import dsa_inputs as I
    from oracle import dsa_oracle as O

    t_prep = time.perf_counter()
    seqs = []
    for b, L in enumerate(d.lens):
        n_pages = (L + d.page - 1) // d.page
        pages = d.block_table[b, :n_pages].long()
        keys = _f64(d.kidx[pages].reshape(-1, d.D_I)[:L])
        sel = idx[b, 0]
        pos = sel[sel >= 0].long()
        phys = d.block_table[b][pos // d.page].long()
        K = _f64(d.k_cache[phys, pos % d.page])
        V = _f64(d.v_cache[phys, pos % d.page])
        seqs.append(dict(L=L, keys=keys, K=K, V=V, local=np.arange(len(pos)), q_idx=_f64(d.q_index[b, 0]),
                         w=d.w[b, 0].double().cpu().numpy(), q=_f64(d.q[:, b]),
                         tl=v.target_logits[b].cpu().numpy(), dl=v.draft_logits[b].cpu().numpy(),
                         dr=v.drafts[b].cpu().numpy()))
    ua, us = I.verify_uniforms(v.seed, v.offset, d.B, d.G)
    prep = time.perf_counter() - t_prep
    threads, limiter = _blas_limits()
    per_op = {"index_scores": 0.0, "topk": 0.0, f"sparse_attn_x{d.G}": 0.0, "spec_verify": 0.0}
    reps, spent = 0, 0.0
    with limiter:
        while reps < 1 or (spent < budget_s and reps < 200):
            for b, s in enumerate(seqs):
                t0 = time.perf_counter()
                row = O.index_scores(s["q_idx"][None], s["w"][None], s["keys"], [s["L"]])[0]
                t1 = time.perf_counter()
                O.topk(row, s["L"], d.k)
                t2 = time.perf_counter()
                for j in range(d.G):
                    O.sparse_attn(s["q"][j], s["K"], s["V"], s["local"], d.sm_scale)
                t3 = time.perf_counter()
                O.spec_verify_seq(s["tl"], s["dl"], s["dr"], ua[b], us[b])
                t4 = time.perf_counter()
                for key, dt in zip(per_op, (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
                    per_op[key] += dt
                spent += t4 - t0
            reps += 1
    per_step = spent / reps
    del seqs
    torch.cuda.empty_cache()
    return {"value": d.G * sum(d.lens) / per_step, "unit": "context tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full step(s) of the same workload ({d.B} sequence(s), contexts {min(d.lens)}.."
                      f"{max(d.lens)}: indexer, top-k, {d.G} attention steps, verification over vocab "
                      f"{v.draft_logits.shape[-1]}); float64 NumPy, {per_step:.3f} s/step; input conversion "
                      f"{prep:.1f} s not timed",
            "seconds_per_op_per_step": {key: val / reps for key, val in per_op.items()},
            "verified_positions_per_s": d.B * (d.G + 1) / per_step,
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}


def cpu_baseline_verify(v):
    """The oracle's verification of every sequence of a batch, timed."""
    import dsa_inputs as I
    from oracle import dsa_oracle as O
    B, G, V = v.draft_logits.shape
    tl, dl, dr = v.target_logits.cpu().numpy(), v.draft_logits.cpu().numpy(), v.drafts.cpu().numpy()
    ua, us = I.verify_uniforms(v.seed, v.offset, B, G)
    threads, limiter = _blas_limits()
    with limiter:
        t0 = time.perf_counter()
        O.spec_verify(tl, dl, dr, ua, us)
        dt = time.perf_counter() - t0
    return {"value": B * (G + 1) / dt, "unit": "verified positions/s", "cores": threads, "kind": "oracle",
            "sample": f"all {B} sequences x {G + 1} positions, vocab {V}; {dt:.2f} s"}


def cpu_baseline_indexer(d, R, n_pos=1 << 17):
    """The oracle's indexer at R rows over a contiguous sample of positions,
    scaled to FLOP/s (the whole 2^20-position call takes minutes in float64)."""
    from oracle import dsa_oracle as O
    keys = _f64(d.kidx.reshape(-1, d.D_I)[:n_pos])
    q, w = _f64(d.q_index[0]), d.w[0].double().cpu().numpy()
    threads, limiter = _blas_limits()
    with limiter:
        t0 = time.perf_counter()
        O.index_scores(q, w, keys, [n_pos] * R)
        dt = time.perf_counter() - t0
    flops = 2.0 * R * n_pos * d.H_I * d.D_I
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{R} rows x {n_pos} positions (of 2^20), 64 heads x 128; {dt:.2f} s"}


def cpu_baseline_latent(d, idx):
    """The oracle's 1M-context latent draft block: indexer over 2^20
    positions, top-k, 7 latent attention steps over the selected rows."""
    import numpy as np
    from oracle import dsa_oracle as O
    L = d.lens[0]
    keys = _f64(d.kidx.reshape(-1, d.D_I)[:L])
    sel = idx[0, 0]
    pos = sel[sel >= 0].long()
    rows = _f64(d.k_cache.reshape(-1, d.D_qk)[pos])                 # identity table: logical == physical
    K, V = rows[:, None, :], rows[:, None, : d.D_v]
    q_idx, w, q = _f64(d.q_index[0, 0]), d.w[0, 0].double().cpu().numpy(), _f64(d.q[:, 0])
    threads, limiter = _blas_limits()
    with limiter:
        t0 = time.perf_counter()
        row = O.index_scores(q_idx[None], w[None], keys, [L])[0]
        t1 = time.perf_counter()
        O.topk(row, L, d.k)
        t2 = time.perf_counter()
        for j in range(d.G):
            O.sparse_attn(q[j], K, V, np.arange(len(pos)), d.sm_scale)
        t3 = time.perf_counter()
    dt = t3 - t0
    return {"value": d.G * L / dt, "unit": "context tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one 1M latent draft block: indexer {t1 - t0:.2f} s, top-k {t2 - t1:.2f} s, "
                      f"{d.G} attention steps {t3 - t2:.2f} s"}


if __name__ == "__main__":
    main()
