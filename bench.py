"""Benchmark: ragged, batched, masked GQA attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config k|name] [--split S]
                    [--no-cpu-baseline] [--copy-calibration]

A step is one pass of the whole hot path over one batch of synthetic input:
one launch of the attention kernel (work partition, Q load + RoPE, K/V gather
+ RoPE, QK^T, mask, online softmax, PV, epilogue all run inside it). Inputs
are resident in HBM before the timed region. Default workload: the batched
tree-attention configuration (16 trees of 64 nodes, h_q 32 / h_kv 8, d 128,
fp16, inline RoPE theta 1e4). Other workloads (--config 0..4) print the same
line for that workload; `--config paged_decode` times the split-KV entry point
(ra_paged_attn_split, one step = the attention kernel + the merge kernel) on a
decode batch, `--split S` picks its split count (0: chosen by the library,
-1: the unsplit entry point); `--config ragged_left_padded` times
ra_ragged_prefill on left-padded causal prompts.

Prints ONE JSON line on stdout. value = TFLOP/s counted on unmasked
(query row, head, key) pairs only, 4*d flops each (QK^T and PV); also
tokens/s and the fractions of the MFMA (2.5 PFLOP/s fp16/bf16 dense) and HBM
(8 TB/s) peaks. The K timed steps are launched as replays of a HIP graph
that holds --graph-launches launches (the launch path is the same C ABI call;
the graph only removes the per-call host cost, which for small workloads is
comparable to the kernel itself); the duration per step comes from HIP events
recorded around the replays on the stream the kernels run on. The same
number of eager launches is timed first and reported as
timing.eager_ms_per_step. ``roofline.traffic`` is the HBM traffic per
launch measured by rocprofv3 counters (profiles/<kernel>_<workload>_pmc.md),
reported only while the kernel source is unchanged since that measurement.
``cpu_baseline`` times the CPU oracle on a bounded sample of the workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "masked-attention TFLOP/s (unmasked pairs) + tokens/s, % of MFMA/HBM roofline"
PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense fp16/bf16
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
KERNEL_SOURCE = os.path.join(ROOT, "attention_ragged_gqa_amd", "csrc", "attn_fwd.hip")
KERNEL_NAME = "attn_fwd_kernel"
DEFAULT_CONFIG = 1


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# work accounting (closed forms from the workload's structure)
# ---------------------------------------------------------------------------

def chunk_lengths(w) -> np.ndarray:
    """KV columns of each sequence's chunk."""
    if w.kind in ("tree", "ragged"):
        return np.diff(w.kv_indptr).astype(np.int64)
    stored = np.diff(w.kv_store_indptr).astype(np.int64)
    if not w.sliding_window:
        return stored
    li = np.asarray(w.length_info)
    return stored - li[1].astype(np.int64) + li[2].astype(np.int64)


def visible_pairs(w) -> int:
    """Unmasked (query row, query head, key) triples. Trees: a node sees its
    depth+1 ancestors-or-self plus the whole prefix; causal: row t of qo sees
    min(L, L - qo + t + 1) columns of an L-column chunk; padded batches
    restrict rows and columns to the valid prefix (right) or suffix (left)."""
    L = chunk_lengths(w)
    qo = np.diff(w.q_indptr).astype(np.int64)
    total = 0
    for b in range(w.batch):
        if qo[b] == 0:
            continue
        if w.kind == "ragged" and w.pad_mode != 0:
            v = int(w.valid_len[b])
            if w.pad_mode == 1:
                total += max(0, min(v, qo[b])) * max(0, min(v, L[b]))
            else:
                vq, vk = max(0, min(v, qo[b])), max(0, min(v, L[b]))
                t = np.arange(qo[b] - vq, qo[b])
                total += int(np.sum(np.clip(np.minimum(L[b], L[b] - qo[b] + t + 1) - (L[b] - vk), 0, None)))
            continue
        if w.kind == "tree" or w.tree_order is not None:
            depth = np.asarray(w.depths[b], np.int64)
            prefix = L[b] - len(depth)
            total += int(np.sum(depth + 1 + prefix))
        elif w.causal:
            t = np.arange(qo[b])
            total += int(np.sum(np.clip(np.minimum(L[b], L[b] - qo[b] + t + 1), 0, None)))
        else:
            total += int(qo[b] * L[b])
    return total * w.h_q


def algorithmic_bytes(w) -> int:
    """Q and out (dtype) + every visible K/V row read once (dtype) + lse (fp32)
    + index arrays (indptrs, tree intervals, page table entries, positions)."""
    esz = 2
    total_q = w.total_q
    qo = np.diff(w.q_indptr).astype(np.int64)
    L = chunk_lengths(w)
    kv_rows = int(np.sum(np.where(qo > 0, L, 0)))
    if w.kind == "ragged" and w.pad_mode != 0:   # only the valid rows are read
        v = np.asarray(w.valid_len, np.int64)
        kv_rows = int(np.sum(np.where(np.minimum(v, qo) > 0, np.clip(np.minimum(v, L), 0, None), 0)))
    nbytes = 2 * total_q * w.h_q * w.d * esz + total_q * w.h_q * 4
    nbytes += kv_rows * w.h_kv * w.d * 2 * esz
    nbytes += 4 * (w.batch + 1) * 2                       # q_indptr + kv/page indptr
    if w.kind == "tree":
        nbytes += 4 * (w.batch + 1) + 8 * len(w.tree_mask)
    elif w.kind == "ragged":
        nbytes += 4 * w.batch if w.pad_mode != 0 else 0
    else:
        nbytes += 4 * int(np.sum((L + 15) // 16)) + 4 * np.asarray(w.length_info).size
        if w.tree_order is not None:
            nbytes += 4 * (w.batch + 1) + 8 * len(w.tree_order)
    if w.rotary_mode == 1:
        nbytes += 4 * total_q
    return int(nbytes)


def config_summary(w) -> dict:
    qo = np.diff(w.q_indptr)
    c = {"workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.d,
         "total_q": w.total_q, "qo_len_range": [int(qo.min()), int(qo.max())],
         "kv_layout": "contiguous" if w.kind in ("tree", "ragged") else "paged16",
         "mask": {1: "right-padded", 2: "left-padded causal"}[w.pad_mode]
                 if (w.kind == "ragged" and w.pad_mode) else
                 "tree" if (w.kind == "tree" or w.tree_order is not None) else
                 ("sliding+causal" if w.sliding_window else ("causal" if w.causal else "none")),
         "rope": ("inline q/k theta=%g" % w.rope_theta) if (w.kind == "tree" and w.rotary_mode)
                 else ("inline q theta=%g" % w.rope_theta if w.rotary_mode else "none"),
         "sm_scale": w.sm_scale}
    if w.kind == "ragged" and w.pad_mode:
        c["valid_len_range"] = [int(np.min(w.valid_len)), int(np.max(w.valid_len))]
    if w.kind == "paged":
        c["kv_chunk_range"] = [int(chunk_lengths(w).min()), int(chunk_lengths(w).max())]
        c["num_pages"] = w.num_pages
    return c


# ---------------------------------------------------------------------------
# rocprofv3 counter summary (traffic)
# ---------------------------------------------------------------------------

def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("attn_fwd.hip", "device_common.h", "ra_internal.h"):
        with open(os.path.join(ROOT, "attention_ragged_gqa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "%s_%s_pmc.md" % (KERNEL_NAME, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return int(m_bytes.group(1))


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(w, pairs_per_pass: int, budget_s: float = 12.0) -> dict:
    from tests.parity import run_oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    if w.total_q * w.h_q <= 64 * 1024:
        # small workload: whole passes until the budget is spent
        n, t0 = 0, time.perf_counter()
        while True:
            run_oracle(w)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 50:
                break
        pairs, sample = pairs_per_pass * n, "%d full passes of the workload" % n
    else:
        # large workload: the first query token of each sequence, then more
        # tokens per sequence until the budget is spent; pairs are counted on
        # the sampled rows only
        from tests.parity import sample_rows
        rows = sample_rows(w, per_seq=2, seed=0)
        frac = len(rows) / max(w.total_q, 1)
        t0 = time.perf_counter()
        run_oracle(w, rows=rows)
        el = time.perf_counter() - t0
        pairs = int(pairs_per_pass * frac)
        sample = "%d sampled query tokens (all heads), %.3f%% of the rows; pairs scaled by the row fraction" % (
            len(rows), 100 * frac)
    tflops = 4.0 * w.d * pairs / el / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(el, 3),
            "cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------

def copy_calibration(steps: int):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = 256 * 1024 * 1024
    src = torch.ones(n // 2, dtype=torch.float16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default=str(DEFAULT_CONFIG),
                    help="0..4, or an extra workload name (paged_decode, ragged_left_padded)")
    ap.add_argument("--split", type=int, default=None,
                    help="split-KV count for paged workloads (0: auto, -1: unsplit entry point); "
                         "default: auto for paged_decode, unsplit otherwise")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--graph-launches", type=int, default=100,
                    help="kernel launches captured per HIP graph (0: time eager launches)")
    ap.add_argument("--eager-steps", type=int, default=None,
                    help="eager launches timed for the host-issue comparison (default: --steps)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    import attention_ragged_gqa_amd as ra
    import attention_ragged_gqa_amd as ra
    from workloads import EXTRA_NAMES, make_config, make_extra
    from workloads.device import DeviceInputs

    ra.library()
    t_gen = time.perf_counter()
    w = make_extra(args.config) if args.config in EXTRA_NAMES else make_config(int(args.config))
    split = args.split
    if split is None:
        split = 0 if args.config == "paged_decode" else -1
    if split >= 0 and w.kind != "paged":
        split = -1
    launch_kw = {} if split < 0 else {"num_kv_splits": split}
    log("[bench] generated %s in %.1fs" % (w.name, time.perf_counter() - t_gen))
    di = DeviceInputs(w, "cuda:0")
    torch.cuda.synchronize()
    log("[bench] inputs resident on cuda:0")

    for _ in range(args.warmup):
        di.launch(**launch_kw)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()       # the stream the kernel is launched on
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    # Eager launches, one Python call each: for small workloads the host
    # issue rate (ctypes + hipLaunchKernel) can be the bound, so this is
    # reported alongside and the steps are timed as HIP graph replays.
    eager_steps = args.steps if args.eager_steps is None else args.eager_steps
    ms_eager = None
    if eager_steps > 0:
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(eager_steps):
            di.launch(**launch_kw)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_eager = ev0.elapsed_time(ev1) / eager_steps

    use_graph = args.graph_launches > 0
    per_graph = max(1, min(args.steps, args.graph_launches)) if use_graph else 0
    reps, rem = divmod(args.steps, per_graph) if use_graph else (0, 0)

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                di.launch(**launch_kw)
        return g

    if use_graph:
        g_main = capture(per_graph)
        g_rem = capture(rem) if rem else None
        g_main.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if use_graph:
        for _ in range(reps):
            g_main.replay()
        if g_rem is not None:
            g_rem.replay()
    else:   # eager launches only (--graph-launches 0)
        for _ in range(args.steps):
            di.launch(**launch_kw)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    log("[bench] %d steps as graph replays (%d launches per graph): %.3f ms (events), %.3f s wall;"
        " eager %s ms/step" % (args.steps, per_graph, ms_total, wall,
                               "%.5f" % ms_eager if ms_eager is not None else "-"))

    pairs = visible_pairs(w)
    flops = 4.0 * w.d * pairs
    nbytes = algorithmic_bytes(w)
    t_s = ms_step / 1e3
    tflops = flops / t_s / 1e12
    gbs = nbytes / t_s / 1e9
    tokens_s = w.total_q / t_s
    hbm_frac = gbs / PEAK_HBM_GBS
    mfma_frac = tflops / PEAK_MFMA_TFLOPS
    ai = flops / nbytes
    bound = "mfma" if ai > PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(hbm_frac, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(mfma_frac, 4)}
    roof["traffic"] = measured_traffic(w.name)
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops
    roof["kernel"] = KERNEL_NAME

    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.dtype == "f16" else "bf16", "data": "synthetic",
        "config": dict(config_summary(w), **({"kv_splits": "auto" if split == 0 else split}
                                               if split >= 0 else {})),
        "tokens_per_s": round(tokens_s, 1),
        "fractions": {"mfma": round(mfma_frac, 4), "hbm": round(hbm_frac, 4)},
        "unmasked_pairs": pairs, "roofline": roof,
        "timing": {"mode": "hip_graph_replay" if use_graph else "eager", "launches_per_graph": per_graph,
                   "eager_ms_per_step": round(ms_eager, 6) if ms_eager is not None else None,
                   # the attention kernel's workgroup shape (split-KV launches: four)
                   "workgroup_waves": ra.ra_attn_workgroup_waves(
                       w.total_q, w.h_q, w.h_kv, split if split > 1 else (2 if split == 0 else 1))},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(w, pairs)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
