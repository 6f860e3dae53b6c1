"""Benchmark of the DSA draft-and-verify hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  indexer scores (draft step 1) -> top-k -> sparse attention for the G = 7
  draft steps reusing the step-1 indices (IndexShare) -> rejection-sampling
  verification of the drafted chain over the vocabulary.

Default workload: single-sequence decode at context 32,768 (indexer 64 heads
x 128 bf16, one shared index key per position; top-k 2048; attention 64
heads x 128 bf16 per-head KV; 7 draft steps; verification of 7 drafts + bonus
over a 151,552-token vocabulary with target logits N(0, 2^2) and draft =
target + N(0, 1)).  Inputs are seeded synthetic data already resident in HBM.

Prints one JSON line: value = draft-step sparse-attention context tokens/s
(G * context / step time), plus a roofline object for the dominant kernel
(sparse attention, HBM-bound) and the CPU oracle timed on the host cores.
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

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_32k", choices=["decode_32k"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the verify-batch and 1M-indexer side measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--extras-only", action="store_true",
                    help="only the side measurements (for profiling them on their own)")
    ap.add_argument("--extras-reps", type=int, default=20,
                    help="graph replays per side measurement")
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


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "mha_attn_decode32k_hbm_traffic.txt")
ATTN_SOURCE = os.path.join(ROOT, "dsa_sparse_attention_lightning_amd", "csrc", "sparse_attn.hip")


def measured_traffic():
    """HBM bytes per attention call (gather + combine) from the committed
    rocprofv3 counter summary, or None when the kernel source has changed
    since the counters were taken."""
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
        if line.startswith("void mha_attn_kernel") or line.startswith("void combine_kernel<128"):
            total += float(line.split()[-1]) * 1e6
    return total or None


def build_workload(name):
    from dsa_inputs import device as DI
    if name == "decode_32k":
        d = DI.draft_inputs(1, [32768], H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048, G=7)
        v = DI.verify_inputs(101, 1, 7, 151552, 2.0)
        return d, v
    raise ValueError(name)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.extras_only:
        import dsa_sparse_attention_lightning_amd as dsa
        print(json.dumps({"extras": extra_measurements(dsa, args.extras_reps, args.extras.split(","))}), flush=True)
        return
    import numpy as np
    import torch

    import dsa_sparse_attention_lightning_amd as dsa

    dev = "cuda:0"
    torch.cuda.set_device(0)
    d, v = build_workload(args.workload)
    B, G, k = d.B, d.G, d.k
    stream = torch.cuda.current_stream()

    # persistent outputs and workspaces (no allocation inside the timed loop)
    scores = torch.empty((B, 1, d.ld), dtype=torch.float32, device=dev)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    topk_ws = torch.empty(max(1, dsa.topk_workspace_size(B, 1, d.ld, k)), dtype=torch.uint8, device=dev)
    outs = torch.empty((G, B, 1, d.H_q, d.D_v), dtype=torch.float32, device=dev)
    lses = torch.empty((G, B, 1, d.H_q), dtype=torch.float32, device=dev)
    attn_ws = torch.zeros(max(1, dsa.sparse_attn_workspace_size(B, 1, d.H_q, d.H_kv, d.D_qk, d.D_v, k)),
                          dtype=torch.uint8, device=dev)
    Bv, Gv, V = v.draft_logits.shape
    acc_len = torch.empty(Bv, dtype=torch.int32, device=dev)
    emitted = torch.empty((Bv, Gv + 1), dtype=torch.int32, device=dev)
    ver_ws = torch.empty(max(1, dsa.spec_verify_workspace_size(Bv, Gv, V)), dtype=torch.uint8, device=dev)

    # The step is captured as three HIP graphs replayed back to back:
    #   draft_first = indexer + top-k (draft step 1), attn = the G sparse-
    #   attention launches (IndexShare), verify = rejection sampling.
    # Events between the replays time each phase on the launch stream.
    def draft_first():
        dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, d.row_len, page=d.page, out=scores)
        dsa.topk(scores, d.row_len, k, out=idx, workspace=topk_ws)

    def attn_steps():
        for j in range(G):
            dsa.sparse_attn(d.q[j][:, None], d.k_cache, d.v_cache, d.block_table, idx[:, 0], page=d.page,
                            D_v=d.D_v, sm_scale=d.sm_scale, out=outs[j], lse=lses[j], workspace=attn_ws)

    def verify():
        dsa.spec_verify(v.target_logits, v.draft_logits, v.drafts, seed=v.seed, offset=v.offset,
                        accepted_len=acc_len, emitted=emitted, workspace=ver_ws)

    phases = [("draft_first", draft_first), ("attn", attn_steps), ("verify", verify)]
    for _, fn in phases:          # eager warm-up (loads code objects, checks arguments)
        fn()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()

    def capture(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for fn in fns:
                fn()
        return g

    g_step = capture([fn for _, fn in phases])            # the whole step, one launch
    g_phase = {n: capture([fn]) for n, fn in phases}      # per-phase graphs for the breakdown
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
    names = [n for n, _ in phases]
    per = {n: [] for n in names}
    for _ in range(args.steps):
        for n in names:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g_phase[n].replay()
            b.record(stream)
            per[n].append((a, b))
    torch.cuda.synchronize()
    kern_us = {n: 1e3 * float(np.mean([a.elapsed_time(b) for a, b in per[n]])) for n in names}
    attn_us = kern_us["attn"] / G

    L_total = sum(d.lens)
    n_sel = sum(min(k, L) for L in d.lens)
    # algorithmic bytes per launch
    attn_bytes = (n_sel * d.H_kv * (d.D_qk + d.D_v) * 2 + B * d.H_q * d.D_qk * 2 + B * k * 4
                  + B * d.H_q * d.D_v * 4 + B * d.H_q * 4)
    idx_bytes = L_total * d.D_I * 2 + L_total * 4 + B * d.H_I * (d.D_I * 2 + 4)
    idx_flops = 2.0 * L_total * d.H_I * d.D_I
    topk_bytes = L_total * 4 + B * k * 4
    ver_bytes = Bv * (2 * Gv + 1) * V * 4
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9

    value = G * L_total / (ms_per_step * 1e-3)
    result = {
        "metric": "draft-step sparse-attn context tokens/s + verified positions/s; % of HBM roofline",
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
        "data": "synthetic",
        "config": {"workload": "decode_32k: 1 sequence, context 32768, indexer 64x128, top-k 2048, "
                               "MHA 64x128 paged 64, 7 draft steps (IndexShare), verify 7+1 x vocab 151552",
                   "global_batch": B, "seq_len": L_total, "parallelism": "none (1 GPU)"},
        "verified_positions_per_s": Bv * (Gv + 1) / (ms_per_step * 1e-3),
        "roofline": {"bound": "hbm", "kernel": "mha_attn_kernel (dsa_sparse_attn)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "traffic_source": "profiles/mha_attn_decode32k_hbm_traffic.txt (FETCH_SIZE x2.0 + "
                                       "WRITE_SIZE x1.0 per call, copy-calibrated)",
                     "bytes_per_launch": attn_bytes, "avg_launch_us": attn_us,
                     "timing": "HIP events around replays of a graph of one step's G attention launches, "
                               "divided by G (includes the split-k combine kernel)"},
        "phases_us": kern_us,
        "phases_roofline": {
            "draft_first (indexer + top-k)": {"bytes": idx_bytes + topk_bytes,
                                              "GBps": (idx_bytes + topk_bytes) / kern_us["draft_first"] / 1e3},
            "verify": {"bytes": ver_bytes, "GBps": ver_bytes / kern_us["verify"] / 1e3},
        },
        "graph": "each timed step is one replay of a HIP graph holding the whole step",
        "accepted_len": acc_len.cpu().tolist(),
    }
    if not args.no_extras:
        result["extras"] = extra_measurements(dsa, args.extras_reps, args.extras.split(","))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(d, v, scores, idx, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _time_graph(fn, reps=20, inner=8, warm_s=0.05):
    """Average duration (us) of one call of `fn`: `inner` calls captured
    back to back in one HIP graph (so the per-replay launch gap is spread
    over them), replayed `reps` times and timed with events on the launch
    stream.  At least 3 untimed replays and `warm_s` seconds of them come
    first (a cold start measured 2-3 % slower)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for _ in range(inner):
            fn()
    t_end, n = time.perf_counter() + warm_s, 0
    while n < 3 or time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (reps * inner)


EXTRA_GROUPS = ("verify", "attn_batched", "cross_layer", "verify_pass", "indexer_1m", "long_1m")


def extra_measurements(dsa, reps=20, groups=EXTRA_GROUPS):
    """Side measurements on the other workload shapes (not the headline), by
    group: verify = spec_verify and greedy verification on the 256 x 8 x
    151,552 verification batch; attn_batched = sparse attention on the
    16-sequence batched configuration; cross_layer = a 4-layer IndexShare
    block at 32K; verify_pass = the 8-row verify-pass DSA step at 32K;
    indexer_1m = the indexer at 1M context for one row (draft step 1,
    HBM-bound) and eight rows (verify-pass shape, MFMA-bound); long_1m = the
    whole 1M-context latent-MQA draft block."""
    out = {}
    for g in groups:
        out.update(_EXTRAS[g](dsa, reps))
    return out


def _extra_verify(dsa, reps):
    import torch
    from dsa_inputs import device as DI
    out = {}
    B, G, V = 256, 7, 151552
    v = DI.verify_inputs(5, B, G, V, 2.0, offset=11)
    n = torch.empty(B, dtype=torch.int32, device="cuda:0")
    em = torch.empty((B, G + 1), dtype=torch.int32, device="cuda:0")
    ws = torch.empty(dsa.spec_verify_workspace_size(B, G, V), dtype=torch.uint8, device="cuda:0")
    us = _time_graph(lambda: dsa.spec_verify(v.target_logits, v.draft_logits, v.drafts, seed=v.seed,
                                             offset=v.offset, accepted_len=n, emitted=em, workspace=ws), reps)
    vbytes = B * (2 * G + 1) * V * 4
    out["verify_256x8x151552"] = {
        "us_per_call": us, "verified_positions_per_s": B * (G + 1) / (us * 1e-6),
        "algorithmic_bytes": vbytes, "GBps": vbytes / us / 1e3, "frac_hbm": vbytes / us / 1e3 / HBM_PEAK_GBS,
        "mean_accepted": float(n.float().mean()), "logit_std": 2.0}
    # greedy verification of the same batch (greedy drafts: the draft model's
    # argmax); reads only the target rows
    gdr = v.draft_logits.argmax(dim=-1).to(torch.int32)
    gws = torch.empty(dsa.spec_verify_greedy_workspace_size(B, G, V), dtype=torch.uint8, device="cuda:0")
    us = _time_graph(lambda: dsa.spec_verify_greedy(v.target_logits, gdr, accepted_len=n, emitted=em,
                                                    workspace=gws), reps)
    gbytes = B * (G + 1) * V * 4
    out["greedy_verify_256x8x151552"] = {
        "us_per_call": us, "verified_positions_per_s": B * (G + 1) / (us * 1e-6), "algorithmic_bytes": gbytes,
        "GBps": gbytes / us / 1e3, "frac_hbm": gbytes / us / 1e3 / HBM_PEAK_GBS,
        "mean_accepted": float(n.float().mean())}
    del v, ws, gws, gdr
    return out


def _extra_attn_batched(dsa, reps):
    import torch
    from dsa_inputs import device as DI
    out = {}
    # sparse attention on the batched configuration: 16 sequences with context
    # uniform in [16K, 64K], paged KV from one shuffled pool (about 1 GiB of
    # gathered K/V per call, more than the last-level cache holds)
    import dsa_inputs as I
    d = DI.draft_inputs(2, I.batched_lens(2), H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048,
                        G=1, shuffle_pages=True)
    sc = dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, d.row_len, page=d.page, ld=d.ld)
    idx = dsa.topk(sc, d.row_len, d.k)
    # the indexer (one row per sequence, draft step 1) and the top-k on the same batch
    us_ix = _time_graph(lambda: dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, d.row_len, page=d.page,
                                                 out=sc), reps)
    tws = torch.empty(max(1, dsa.topk_workspace_size(d.B, 1, d.ld, d.k)), dtype=torch.uint8, device="cuda:0")
    us_tk = _time_graph(lambda: dsa.topk(sc, d.row_len, d.k, out=idx, workspace=tws), reps)
    L_total = sum(d.lens)
    ibytes = L_total * d.D_I * 2 + L_total * 4
    out["indexer_batched_16x16k_64k"] = {"us_per_call": us_ix, "algorithmic_bytes": ibytes,
                                         "GBps": ibytes / us_ix / 1e3, "frac_hbm": ibytes / us_ix / 1e3 / HBM_PEAK_GBS}
    out["topk_batched_16x16k_64k"] = {"us_per_call": us_tk, "rows": d.B}
    del sc, tws
    o = torch.empty((d.B, 1, d.H_q, d.D_v), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((d.B, 1, d.H_q), dtype=torch.float32, device="cuda:0")
    aws = torch.zeros(max(1, dsa.sparse_attn_workspace_size(d.B, 1, d.H_q, d.H_kv, d.D_qk, d.D_v, d.k)),
                      dtype=torch.uint8, device="cuda:0")
    us = _time_graph(lambda: dsa.sparse_attn(d.q[0][:, None], d.k_cache, d.v_cache, d.block_table, idx[:, 0],
                                             page=d.page, D_v=d.D_v, sm_scale=d.sm_scale, out=o, lse=lse,
                                             workspace=aws), reps)
    n_sel = sum(min(d.k, L) for L in d.lens)
    abytes = (n_sel * d.H_kv * (d.D_qk + d.D_v) * 2 + d.B * d.H_q * d.D_qk * 2 + d.B * d.k * 4
              + d.B * d.H_q * d.D_v * 4 + d.B * d.H_q * 4)
    out["attn_batched_16x16k_64k"] = {
        "us_per_call": us, "algorithmic_bytes": abytes, "GBps": abytes / us / 1e3,
        "frac_hbm": abytes / us / 1e3 / HBM_PEAK_GBS, "context_tokens_per_s": sum(d.lens) / (us * 1e-6)}
    del d, idx, o, lse, aws
    return out


def _extra_cross_layer(dsa, reps):
    import torch
    from dsa_inputs import device as DI
    out = {}
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

    us_shared = _time_graph(shared, reps, inner=4)
    us_per = _time_graph(per_layer, reps, inner=4)
    out["cross_layer_indexshare_32k_4layers"] = {
        "us_per_block_shared": us_shared, "us_per_block_indexer_each_layer": us_per,
        "speedup": us_per / us_shared}
    del layers, d0, sc, ix, o, lse, aws
    return out


def _extra_verify_pass(dsa, reps):
    import torch
    from dsa_inputs import device as DI
    out = {}
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

    us = _time_graph(verify_pass, reps)
    out["verify_pass_dsa_32k_8rows"] = {"us_per_call": us, "rows_per_s": R / (us * 1e-6),
                                        "context_tokens_per_s": R * L / (us * 1e-6)}
    del d, rl, sc, ix, qv, o, lse, aws, tws
    return out


def _extra_indexer_1m(dsa, reps):
    import torch
    from dsa_inputs import device as DI
    out = {}
    L = 1 << 20
    for R in (1, 8):
        d = DI.draft_inputs(3, [L], H_I=64, D_I=128, H_q=64, D_qk=576, D_v=512, k=2048, G=0, R=R,
                            latent=True)
        sc = torch.empty((1, R, d.ld), dtype=torch.float32, device="cuda:0")
        us = _time_graph(lambda: dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, d.row_len,
                                                  page=d.page, out=sc), reps)
        flops = 2.0 * R * L * d.H_I * d.D_I
        kbytes = L * d.D_I * 2 + R * L * 4
        out[f"indexer_1m_R{R}"] = {
            "us_per_call": us, "TFLOPs": flops / us / 1e6, "frac_mfma": flops / us / 1e6 / BF16_MFMA_PEAK_TFLOPS,
            "GBps": kbytes / us / 1e3, "frac_hbm": kbytes / us / 1e3 / HBM_PEAK_GBS}
        del d, sc
    return out


def _extra_long_1m(dsa, reps):
    """The 1M-context draft block (latent MQA): indexer (R = 1) and top-k over
    2^20 positions once, then 7 latent sparse-attention steps reusing the
    indices; phases timed separately and as one graph."""
    import torch
    from dsa_inputs import device as DI
    out = {}
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

    def attend():
        for j in range(d.G):
            dsa.sparse_attn(d.q[j][:, None], d.k_cache, d.v_cache, d.block_table, ix[:, 0], page=d.page,
                            D_v=d.D_v, sm_scale=d.sm_scale, out=o[j], lse=lse[j], workspace=aws)

    def block():
        indexer()
        select()
        attend()

    us_block = _time_graph(block, reps, inner=2)
    out["long_1m_latent_draft_block"] = {
        "us_per_block": us_block, "context_tokens_per_s": d.G * (1 << 20) / (us_block * 1e-6),
        "us_indexer": _time_graph(indexer, reps), "us_topk": _time_graph(select, reps),
        "us_attention_per_step": _time_graph(attend, reps, inner=2) / d.G}
    return out


_EXTRAS = {"verify": _extra_verify, "attn_batched": _extra_attn_batched, "cross_layer": _extra_cross_layer,
           "verify_pass": _extra_verify_pass, "indexer_1m": _extra_indexer_1m, "long_1m": _extra_long_1m}


def cpu_baseline(d, v, scores, idx, budget_s):
    """Times the float64 CPU oracle on one full step of the same workload
    (draft block + verification of the same sequence), repeated until the
    time budget is spent; same unit as the GPU value."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import dsa_oracle as O
    import dsa_inputs as I

    def f64(t):
        return t.float().cpu().numpy().astype(np.float64)

    L = d.lens[0]
    t_prep = time.perf_counter()
    pages = d.block_table[0].cpu().numpy()
    order = pages[: (L + d.G + d.page - 1) // d.page]
    keys = f64(d.kidx[order].reshape(-1, d.D_I))
    K = f64(d.k_cache[order].reshape(-1, d.H_kv, d.D_qk))
    V = f64(d.v_cache[order].reshape(-1, d.H_kv, d.D_v))
    q_idx = f64(d.q_index[0, 0])
    w = d.w[0, 0].double().cpu().numpy()
    q = f64(d.q[:, 0])
    tl = v.target_logits[0].cpu().numpy()
    dl = v.draft_logits[0].cpu().numpy()
    dr = v.drafts[0].cpu().numpy()
    ua, us = I.verify_uniforms(v.seed, v.offset, 1, d.G)
    prep = time.perf_counter() - t_prep

    threads = sum(p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas") or 1
    reps, spent = 0, 0.0
    per_op = {"index_scores": 0.0, "topk": 0.0, "sparse_attn_x7": 0.0, "spec_verify": 0.0}
    while spent < budget_s and reps < 200:
        t0 = time.perf_counter()
        s_row = O.index_scores(q_idx[None], w[None], keys, [L])[0]
        t1 = time.perf_counter()
        sel = O.topk(s_row, L, d.k)
        t2 = time.perf_counter()
        for j in range(d.G):
            O.sparse_attn(q[j], K, V, sel, d.sm_scale)
        t3 = time.perf_counter()
        O.spec_verify_seq(tl, dl, dr, ua[0], us[0])
        t4 = time.perf_counter()
        for key, dt in zip(per_op, (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
            per_op[key] += dt
        spent += t4 - t0
        reps += 1
    per_step = spent / reps
    return {"value": d.G * L / per_step, "unit": "context tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full steps of the same workload (1 sequence, context {L}: indexer, top-k, "
                      f"{d.G} attention steps, verify over vocab {v.draft_logits.shape[-1]}); "
                      f"float64 NumPy, {per_step:.3f} s/step, input conversion {prep:.1f} s not timed",
            "seconds_per_op": {key: v / reps for key, v in per_op.items()},
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
