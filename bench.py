"""Benchmark: ragged, batched, masked GQA attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config k|name] [--split S]
                    [--copies N] [--no-per-config] [--no-extra] [--no-cpu-baseline]
                    [--copy-calibration]

A step is one pass of the whole hot path over one batch of synthetic input:
one launch of the attention kernel (work partition, Q load + RoPE, K/V gather
+ RoPE, QK^T, mask, online softmax, PV, epilogue all run inside it). Inputs
are resident in HBM before the timed region.

Default workload (the headline): the largest single-GPU configuration, the
speculative-decode tree over a paged prefix (128 sequences, 4096-token
prefix + 256-node tree, h_q 64 / h_kv 8, d 128, bf16, q RoPE inline at
prefix + depth, theta 5e5). The same JSON line carries a ``per_config``
block timing the other four configurations (tree_tiny, tree_batched,
paged_causal, paged_sliding) in the same run. ``--config 0..4`` puts another
configuration in the headline; ``--config paged_decode`` times the split-KV
entry point (ra_paged_attn_split, one step = the attention kernel + the
merge kernel) on a decode batch, ``--split S`` picks its split count (0:
chosen by the library, -1: the unsplit entry point); ``--config
ragged_left_padded`` times ra_ragged_prefill on left-padded causal prompts,
``--config mla_prefill`` ra_mla_paged_prefill on the latent-attention
prefill. Those three follow-on workloads are also timed in an
``extra_workloads`` block of the default line (decode split with the
library's count; ``--no-extra`` skips it), and so is the step before the
path, ``kv_append``: ra_paged_kv_append writing the headline's 32,768 new
tree tokens (K rotated at prefix + depth) into its paged cache, HBM-bound,
counted as each new K/V row read once and written once (``--config
kv_append`` prints a line of its own in GB/s).

Prints ONE JSON line on stdout. value = TFLOP/s counted on unmasked
(query row, head, key) pairs only, 4*d flops each (QK^T and PV); also
tokens/s and the fractions of the MFMA (2.5 PFLOP/s fp16/bf16 dense) and HBM
(8 TB/s) peaks. The K timed steps are launched as replays of a HIP graph
that holds --graph-launches launches (the launch path is the same C ABI call;
the graph only removes the per-call host cost, which for small workloads is
comparable to the kernel itself); the duration per step comes from HIP events
recorded around the replays on the stream the kernels run on. The same
number of eager launches is timed first and reported as
timing.eager_ms_per_step.

HBM-bound workloads (flop/byte below the ridge point) are timed cold: the
graph cycles through enough separate copies of the inputs (--copies, default
enough for 512 MiB, twice the 256 MB Infinity Cache) that every launch reads
its bytes from HBM; the same launch on one resident copy is reported as
``warm``. ``roofline.traffic`` is the HBM traffic per launch measured by
rocprofv3 counters (profiles/<kernel>_<workload>_pmc.md), reported only while
the kernel's code (comments aside) is unchanged since that measurement. ``cpu_baseline`` times
the CPU oracle on a bounded sample of the headline workload: whole passes of
a small workload, else whole sequences (every row and head of each), with the
unmasked pairs of exactly those sequences counted.
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
DEFAULT_CONFIG = 4                 # spec_tree_paged, the largest configuration
COLD_FOOTPRINT = 512 << 20         # bytes of distinct inputs cycled per graph (HBM-bound)
INFINITY_CACHE = 256 << 20         # MI355X's last-level (MALL) cache
# steps per configuration in the per_config block (about 25-100 ms of GPU time each)
PER_CONFIG_STEPS = {0: 2000, 1: 2000, 2: 200, 3: 200, 4: 20}
# the follow-on workloads (split-KV decode, padded batches, latent attention),
# timed in the same run unless --no-extra: steps each (paged_decode is split
# with the automatic count, as its own bench line runs it)
EXTRA_STEPS = {"paged_decode": 100, "ragged_left_padded": 100, "mla_prefill": 50}
# the step before the path: appending the headline's new tokens (its tree
# nodes, K rotated at their cache positions) into its paged cache
APPEND_NAME = "kv_append"
APPEND_SOURCE = DEFAULT_CONFIG
APPEND_STEPS = 100


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


def visible_pairs(w, seqs=None) -> int:
    """Unmasked (query row, query head, key) triples (of the sequences in
    ``seqs`` only, when given). Trees: a node sees its depth+1
    ancestors-or-self plus the whole prefix; causal: row t of qo sees
    min(L, L - qo + t + 1) columns of an L-column chunk; padded batches
    restrict rows and columns to the valid prefix (right) or suffix (left)."""
    L = chunk_lengths(w)
    qo = np.diff(w.q_indptr).astype(np.int64)
    total = 0
    for b in (range(w.batch) if seqs is None else seqs):
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


def rows_with_keys(w, seqs=None) -> int:
    """Query tokens with at least one visible key (of the sequences in
    ``seqs`` only, when given), by the same row limits as visible_pairs:
    the rows whose Q the kernels read. The others (padding, or causal rows
    past a shorter chunk) are masked everywhere; only their zero output and
    -inf lse are written."""
    L = chunk_lengths(w)
    qo = np.diff(w.q_indptr).astype(np.int64)
    total = 0
    for b in (range(w.batch) if seqs is None else seqs):
        if qo[b] == 0:
            continue
        if w.kind == "ragged" and w.pad_mode != 0:
            v = int(w.valid_len[b])
            if w.pad_mode == 1:
                total += max(0, min(v, qo[b])) if min(v, L[b]) > 0 else 0
            else:
                vq, vk = max(0, min(v, qo[b])), max(0, min(v, L[b]))
                t = np.arange(qo[b] - vq, qo[b])
                total += int(np.sum(np.minimum(L[b], L[b] - qo[b] + t + 1) - (L[b] - vk) > 0))
            continue
        if w.causal and not (w.kind == "tree" or w.tree_order is not None):
            t = np.arange(qo[b])
            total += int(np.sum(np.minimum(L[b], L[b] - qo[b] + t + 1) > 0))
        else:   # trees (a node sees itself) and unmasked rows
            total += int(qo[b]) if L[b] > 0 else 0
    return total


def flops_per_pair(w) -> float:
    """2 d_qk for the score and 2 d_v for the PV product of one unmasked
    (row, head, key) pair: 4 d, or 2 (576 + 512) for latent attention."""
    d_v = w.d_latent if w.kind == "mla" else w.d
    return 2.0 * (w.d + d_v)


def algorithmic_bytes(w) -> int:
    """Q of the rows that see a key (rows_with_keys) and out of every row
    (dtype) + every visible K/V row read once (dtype) + lse (fp32) + index
    arrays (indptrs, tree intervals, page table entries, positions)."""
    esz = 2
    total_q = w.total_q
    q_rows = rows_with_keys(w)
    qo = np.diff(w.q_indptr).astype(np.int64)
    L = chunk_lengths(w)
    kv_rows = int(np.sum(np.where(qo > 0, L, 0)))
    if w.kind == "ragged" and w.pad_mode != 0:   # only the valid rows are read
        v = np.asarray(w.valid_len, np.int64)
        kv_rows = int(np.sum(np.where(np.minimum(v, qo) > 0, np.clip(np.minimum(v, L), 0, None), 0)))
    if w.kind == "mla":   # q + out (latent width) + lse, one shared latent row per key
        nbytes = (q_rows * w.d + total_q * w.d_latent) * w.h_q * esz + total_q * w.h_q * 4
        nbytes += kv_rows * w.d * esz
        nbytes += 4 * (w.batch + 1) * 2 + 4 * int(np.sum((L + 15) // 16)) + 4 * w.batch
        return int(nbytes)
    nbytes = (q_rows + total_q) * w.h_q * w.d * esz + total_q * w.h_q * 4
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


def append_bytes(ai) -> int:
    """Algorithmic bytes of one append (AppendInputs ai): every new token's K
    and V rows read once and written once into their page slots (dtype), its
    cache position (int32), the append indptr and starts and the page indptr
    (int32), and the page-table entries the new tokens land on."""
    w = ai.w
    row = w.h_kv * w.d * 2
    n = ai.n_tokens
    pages = sum(int((s0 + n0 - 1) // 16 - s0 // 16 + 1) for s0, n0 in zip(ai.new_start, ai.new_len) if n0 > 0)
    return int(2 * 2 * n * row + 4 * n + 4 * (w.batch + 1) + 4 * w.batch + 4 * (w.batch + 1) + 4 * pages)


def append_summary(ai) -> dict:
    w = ai.w
    starts = np.asarray(ai.new_start)
    pos = np.asarray(w.store_rope_position)
    return {"workload": APPEND_NAME, "source": "%s (the new tokens of each sequence)" % w.name,
            "batch": w.batch, "tokens": ai.n_tokens, "h_kv": w.h_kv, "head_dim": w.d,
            "kv_layout": "paged16", "num_pages": w.num_pages,
            "rope": "K rotated on the way in, theta=%g" % w.rope_theta,
            "positions_range": [int(pos.min()), int(pos.max())] if pos.size else [0, 0],
            "mid_page_starts": int(np.sum(starts % 16 != 0))}


def measure_append(w, steps, warmup, graph_launches, copies=None):
    """Time the append step of w like the HBM-bound attention workloads:
    cold, cycling through `copies` input copies (default COLD_FOOTPRINT worth),
    and warm on one. Returns (result dict, copies used, AppendInputs)."""
    from workloads.device import AppendInputs
    ai = AppendInputs(w, "cuda:0")
    nbytes = append_bytes(ai)
    if copies is None:
        copies = max(1, min(64, -(-COLD_FOOTPRINT // nbytes)))

    def rate(ms):
        t = ms / 1e3
        gbs = nbytes / t / 1e9
        return {"ms_per_step": round(ms, 6), "gbs": round(gbs, 2), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "tokens_per_s": round(ai.n_tokens / t, 1), "bytes": nbytes}

    ms_warm, ms_eager, per_graph = time_steps([ai], steps, warmup, graph_launches, {}, 0)
    res = {"bound": "hbm", "copies": copies, "eager_ms_per_step": ms_eager, "launches_per_graph": per_graph}
    if copies > 1:
        ais = [ai] + [AppendInputs(w, "cuda:0") for _ in range(copies - 1)]
        ms_cold, _, per_graph = time_steps(ais, steps, warmup, graph_launches, {}, 0)
        res.update(rate(ms_cold))
        res["warm"] = rate(ms_warm)
        del ais
    else:
        res.update(rate(ms_warm))
    res["frac"] = res["hbm_frac"]
    return res, copies, ai


def append_entry(ai, r) -> dict:
    e = {"workload": APPEND_NAME, "source": ai.w.name, "dtype": ai.w.dtype, "bound": "hbm",
         "frac": r["frac"], "ms_per_step": r["ms_per_step"], "gbs": r["gbs"], "tokens_per_s": r["tokens_per_s"],
         "hbm_frac": r["hbm_frac"], "timing": timing_label(r), "kernel": kernel_name(APPEND_NAME)}
    if "warm" in r:
        e["warm"] = {k: r["warm"][k] for k in ("ms_per_step", "gbs", "hbm_frac")}
    return e


def append_main(args):
    """bench.py --config kv_append: one JSON line for the append step alone."""
    import torch
    from workloads import make_config
    w = make_config(APPEND_SOURCE)
    r, copies, ai = measure_append(w, args.steps, args.warmup, args.graph_launches, args.copies)
    torch.cuda.synchronize()
    log("[bench] %s: %d steps, %.5f ms/step" % (APPEND_NAME, args.steps, r["ms_per_step"]))
    line = {
        "metric": "paged KV append GB/s (new K/V rows read and written once)", "value": r["gbs"],
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.dtype == "f16" else "bf16", "data": "synthetic", "config": append_summary(ai),
        "tokens_per_s": r["tokens_per_s"],
        "roofline": {"bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": r["hbm_frac"], "traffic": measured_traffic(APPEND_NAME),
                     "algorithmic_bytes": r["bytes"], "algorithmic_flops": 0,
                     "kernel": kernel_name(APPEND_NAME)},
        "timing": {"mode": "hip_graph_replay" if args.graph_launches > 0 else "eager",
                   "launches_per_graph": r["launches_per_graph"], "input_copies": copies,
                   "inputs": timing_label(r)},
        "cpu_baseline": None,
    }
    if "warm" in r:
        line["warm"] = r["warm"]
    print(json.dumps(line), flush=True)


def config_summary(w) -> dict:
    qo = np.diff(w.q_indptr)
    c = {"workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.d,
         "total_q": w.total_q, "qo_len_range": [int(qo.min()), int(qo.max())],
         "kv_layout": "contiguous" if w.kind in ("tree", "ragged") else
                      ("paged16 latent (%d + %d)" % (w.d_latent, w.d - w.d_latent) if w.kind == "mla" else "paged16"),
         "mask": {1: "right-padded", 2: "left-padded causal"}[w.pad_mode]
                 if (w.kind == "ragged" and w.pad_mode) else
                 "tree" if (w.kind == "tree" or w.tree_order is not None) else
                 ("sliding+causal" if w.sliding_window else ("causal" if w.causal else "none")),
         "rope": ("inline q/k theta=%g" % w.rope_theta) if (w.kind == "tree" and w.rotary_mode)
                 else ("inline q theta=%g" % w.rope_theta if w.rotary_mode else "none"),
         "sm_scale": w.sm_scale}
    if w.kind == "ragged" and w.pad_mode:
        c["valid_len_range"] = [int(np.min(w.valid_len)), int(np.max(w.valid_len))]
    if w.kind in ("paged", "mla"):
        c["kv_chunk_range"] = [int(chunk_lengths(w).min()), int(chunk_lengths(w).max())]
        c["num_pages"] = w.num_pages
    return c


# ---------------------------------------------------------------------------
# rocprofv3 counter summary (traffic)
# ---------------------------------------------------------------------------

def kernel_name(workload: str) -> str:
    """The dominant kernel of a workload's step."""
    if workload == APPEND_NAME:
        return "kv_append_kernel"
    return "mla_fwd_kernel" if workload.startswith("mla") else KERNEL_NAME


def source_code_text(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed (string
    and character literals kept), so that a comment or layout edit leaves
    the kernel hash unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(kernel: str = KERNEL_NAME) -> str:
    """Hash of the kernel's code (comments and layout excluded): a counter
    summary in profiles/ applies while it matches."""
    src = {"mla_fwd_kernel": "mla_fwd.hip", "kv_append_kernel": "kv_append.hip"}.get(kernel, "attn_fwd.hip")
    h = hashlib.sha256()
    for name in (src, "device_common.h", "ra_internal.h"):
        with open(os.path.join(ROOT, "attention_ragged_gqa_amd", "csrc", name), encoding="utf-8") as f:
            h.update(source_code_text(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    kernel = kernel_name(workload)
    path = os.path.join(ROOT, "profiles", "%s_%s_pmc.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(kernel):
        return None
    return int(m_bytes.group(1))


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(w, pairs_per_pass: int, budget_s: float = 12.0) -> dict:
    """The CPU oracle as it stands, timed on this host: whole passes of a
    small workload, or whole sequences of a large one (in order, until the
    budget is spent), each with the unmasked pairs it actually computes. The
    page pool the oracle reads is built before the clock starts."""
    from tests.parity import run_oracle
    from workloads import pages_from_logical
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    from workloads import mla_pages_from_logical
    pool = pages_from_logical(w) if w.kind == "paged" else (mla_pages_from_logical(w) if w.kind == "mla" else None)
    if w.total_q * w.h_q <= 64 * 1024:
        n, t0 = 0, time.perf_counter()
        while True:
            run_oracle(w, pool=pool, spread=False)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 50:
                break
        pairs, sample = pairs_per_pass * n, "%d full passes of the workload" % n
    else:
        el, pairs, done = 0.0, 0, 0
        for b in range(w.batch):
            rows = np.arange(int(w.q_indptr[b]), int(w.q_indptr[b + 1]))
            if len(rows) == 0:
                continue
            t0 = time.perf_counter()
            run_oracle(w, rows=rows, pool=pool, spread=False)
            el += time.perf_counter() - t0
            pairs += visible_pairs(w, seqs=[b])
            done += 1
            if el >= budget_s:
                break
        sample = ("sequences 0..%d of %d (every query row and head of each, %.2f%% of the "
                  "workload's unmasked pairs), pairs counted exactly" % (done - 1, w.batch,
                                                                        100.0 * pairs / pairs_per_pass))
    tflops = flops_per_pair(w) * pairs / el / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(el, 3), "estimated": False,
            "cpu": _cpu_model(), "host_cpus": os.cpu_count()}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# timing
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


def bound_of(w) -> str:
    """'mfma' when the workload's flop/byte ratio is above the ridge point."""
    ai = flops_per_pair(w) * visible_pairs(w) / algorithmic_bytes(w)
    return "mfma" if ai > PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"


def time_steps(dis, steps: int, warmup: int, graph_launches: int, launch_kw: dict,
               eager_steps: int):
    """Warm up, time `eager_steps` eager launches, then time exactly `steps`
    launches as HIP-graph replays (graph_launches per graph; 0: eager). Launch
    i uses dis[i % len(dis)]. Returns (ms per step, eager ms per step or None,
    launches per graph)."""
    import torch
    n = len(dis)
    for i in range(warmup):
        dis[i % n].launch(**launch_kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()       # the stream the kernels are launched on
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ms_eager = None
    if eager_steps > 0:
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(eager_steps):
            dis[i % n].launch(**launch_kw)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_eager = ev0.elapsed_time(ev1) / eager_steps

    use_graph = graph_launches > 0
    per_graph = max(1, min(steps, graph_launches)) if use_graph else 0
    reps, rem = divmod(steps, per_graph) if use_graph else (0, 0)

    def capture(count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                dis[i % n].launch(**launch_kw)
        return g

    if use_graph:
        g_main = capture(per_graph)
        g_rem = capture(rem) if rem else None
        g_main.replay()
        torch.cuda.synchronize()
    ev0.record(stream)
    if use_graph:
        for _ in range(reps):
            g_main.replay()
        if g_rem is not None:
            g_rem.replay()
    else:
        for i in range(steps):
            dis[i % n].launch(**launch_kw)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, ms_eager, per_graph


def rates(w, ms_step: float) -> dict:
    """Throughput and roofline fractions of one step of w taking ms_step."""
    pairs = visible_pairs(w)
    flops = flops_per_pair(w) * pairs
    nbytes = algorithmic_bytes(w)
    t_s = ms_step / 1e3
    tflops = flops / t_s / 1e12
    gbs = nbytes / t_s / 1e9
    return {"ms_per_step": round(ms_step, 6), "tflops": round(tflops, 3),
            "tokens_per_s": round(w.total_q / t_s, 1), "gbs": round(gbs, 2),
            "mfma_frac": round(tflops / PEAK_MFMA_TFLOPS, 4), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "pairs": pairs, "flops": flops, "bytes": nbytes}


def measure(w, steps, warmup, graph_launches, launch_kw, eager_steps, copies=None):
    """Time w. HBM-bound workloads are timed cold, cycling through `copies`
    (default: COLD_FOOTPRINT worth) separate input copies, and warm on one
    copy; others warm only. Returns (result dict, copies used)."""
    from workloads.device import DeviceInputs
    bound = bound_of(w)
    di = DeviceInputs(w, "cuda:0")
    if copies is None:
        copies = 1 if bound == "mfma" else max(1, min(64, -(-COLD_FOOTPRINT // algorithmic_bytes(w))))
    ms_warm, ms_eager, per_graph = time_steps([di], steps, warmup, graph_launches, launch_kw, eager_steps)
    res = {"bound": bound, "copies": copies, "eager_ms_per_step": ms_eager, "launches_per_graph": per_graph}
    if copies > 1:
        dis = [di] + [DeviceInputs(w, "cuda:0") for _ in range(copies - 1)]
        ms_cold, _, per_graph = time_steps(dis, steps, warmup, graph_launches, launch_kw, 0)
        res.update(rates(w, ms_cold))
        res["warm"] = rates(w, ms_warm)
        del dis
    else:
        res.update(rates(w, ms_warm))
    res["frac"] = res["mfma_frac"] if bound == "mfma" else res["hbm_frac"]
    return res, copies


def timing_label(r) -> str:
    """How the inputs of a timed run relate to the 256 MB Infinity Cache."""
    if r["copies"] > 1:
        return "cold (%d input copies cycled)" % r["copies"]
    if r["bytes"] > INFINITY_CACHE:
        return "one copy of %d MB, larger than the 256 MB Infinity Cache" % (r["bytes"] >> 20)
    return "warm"


def per_config_entry(w, r) -> dict:
    e = {"workload": w.name, "dtype": w.dtype, "bound": r["bound"], "frac": r["frac"],
         "ms_per_step": r["ms_per_step"], "tflops": r["tflops"], "tokens_per_s": r["tokens_per_s"],
         "mfma_frac": r["mfma_frac"], "hbm_frac": r["hbm_frac"], "timing": timing_label(r)}
    if "warm" in r:
        e["warm"] = {k: r["warm"][k] for k in ("ms_per_step", "tflops", "hbm_frac", "mfma_frac")}
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=str(DEFAULT_CONFIG),
                    help="0..4, or an extra workload name (paged_decode, ragged_left_padded, "
                         "mla_prefill, kv_append)")
    ap.add_argument("--split", type=int, default=None,
                    help="split-KV count for paged workloads (0: auto, -1: unsplit entry point); "
                         "default: auto for paged_decode, unsplit otherwise")
    ap.add_argument("--copies", type=int, default=None,
                    help="input copies cycled per graph (default: 1 for MFMA-bound workloads, "
                         "512 MiB worth for HBM-bound ones)")
    ap.add_argument("--waves", type=int, default=None,
                    help="force the attention workgroup shape: 4 or 8 waves of 32 query rows "
                         "(default: chosen per launch)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra_workloads block (decode, padded batches, latent attention)")
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
    from workloads import CONFIG_NAMES, EXTRA_NAMES, make_config, make_extra

    ra.library()
    if args.config == APPEND_NAME:
        append_main(args)
        return
    if args.waves is not None:
        ra.ra_set_workgroup_waves(args.waves)
    t_gen = time.perf_counter()
    w = make_extra(args.config) if args.config in EXTRA_NAMES else make_config(int(args.config))
    split = args.split
    if split is None:
        split = 0 if args.config == "paged_decode" else -1
    if split >= 0 and w.kind != "paged":
        split = -1
    launch_kw = {} if split < 0 else {"num_kv_splits": split}
    log("[bench] generated %s in %.1fs" % (w.name, time.perf_counter() - t_gen))
    eager_steps = args.steps if args.eager_steps is None else args.eager_steps
    r, copies = measure(w, args.steps, args.warmup, args.graph_launches, launch_kw, eager_steps,
                        args.copies)
    torch.cuda.synchronize()
    log("[bench] %s: %d steps, %.5f ms/step (%s)" % (w.name, args.steps, r["ms_per_step"],
                                                     "cold, %d copies" % copies if copies > 1 else "warm"))

    bound = r["bound"]
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": r["hbm_frac"]}
    else:
        roof = {"bound": "mfma", "achieved": r["tflops"], "peak": PEAK_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": r["mfma_frac"]}
    roof["traffic"] = measured_traffic(w.name)
    roof["algorithmic_bytes"] = r["bytes"]
    roof["algorithmic_flops"] = r["flops"]
    roof["kernel"] = kernel_name(w.name)

    line = {
        "metric": METRIC, "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.dtype == "f16" else "bf16", "data": "synthetic",
        "config": dict(config_summary(w), **({"kv_splits": "auto" if split == 0 else split}
                                               if split >= 0 else {})),
        "tokens_per_s": r["tokens_per_s"],
        "fractions": {"mfma": r["mfma_frac"], "hbm": r["hbm_frac"]},
        "unmasked_pairs": r["pairs"], "roofline": roof,
        "timing": {"mode": "hip_graph_replay" if args.graph_launches > 0 else "eager",
                   "launches_per_graph": r["launches_per_graph"],
                   "input_copies": copies,
                   "inputs": timing_label(r),
                   "eager_ms_per_step": round(r["eager_ms_per_step"], 6) if r["eager_ms_per_step"] is not None else None,
                   # the attention kernel's workgroup shape (split-KV launches: four)
                   "workgroup_waves": ra.ra_attn_workgroup_waves(
                       w.total_q, w.h_q, w.h_kv, split if split > 1 else (2 if split == 0 else 1))
                       if w.kind != "mla" else 4},
    }
    if "warm" in r:
        line["warm"] = r["warm"]

    if not args.no_per_config:
        per = [per_config_entry(w, r)] if args.config in [str(k) for k in range(len(CONFIG_NAMES))] else []
        for k in range(len(CONFIG_NAMES)):
            if str(k) == args.config:
                continue
            t0 = time.perf_counter()
            wk = make_config(k)
            rk, _ = measure(wk, PER_CONFIG_STEPS[k], 5, args.graph_launches, {}, 0)
            per.append(per_config_entry(wk, rk))
            log("[bench] per-config %s: %.5f ms/step, %s frac %.4f (%.1fs)"
                % (wk.name, rk["ms_per_step"], rk["bound"], rk["frac"], time.perf_counter() - t0))
            del wk
            torch.cuda.empty_cache()
        per.sort(key=lambda e: CONFIG_NAMES.index(e["workload"]) if e["workload"] in CONFIG_NAMES else 99)
        line["per_config"] = per

    if not args.no_extra and not args.no_per_config:
        extra = []
        for name, steps in EXTRA_STEPS.items():
            if name == args.config:
                continue
            t0 = time.perf_counter()
            we = make_extra(name)
            kw = {"num_kv_splits": 0} if name == "paged_decode" else {}
            re_, _ = measure(we, steps, 5, args.graph_launches, kw, 0)
            e = dict(per_config_entry(we, re_), kernel=kernel_name(name))
            if kw:
                e["kv_splits"] = "auto"
            extra.append(e)
            log("[bench] extra %s: %.5f ms/step, %s frac %.4f (%.1fs)"
                % (we.name, re_["ms_per_step"], re_["bound"], re_["frac"], time.perf_counter() - t0))
            del we
            torch.cuda.empty_cache()
        t0 = time.perf_counter()
        wa = make_config(APPEND_SOURCE) if str(APPEND_SOURCE) != args.config else w
        ra_, _, ai = measure_append(wa, APPEND_STEPS, 5, args.graph_launches)
        extra.append(append_entry(ai, ra_))
        log("[bench] extra %s: %.5f ms/step, hbm frac %.4f (%.1fs)"
            % (APPEND_NAME, ra_["ms_per_step"], ra_["frac"], time.perf_counter() - t0))
        del ai
        torch.cuda.empty_cache()
        line["extra_workloads"] = extra

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(w, r["pairs"])
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
