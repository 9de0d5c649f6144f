"""Seeded generators for the five attention workloads and for custom test shapes.

Everything here is input construction: lengths, trees, DFS intervals, page
tables and N(0,1) values rounded (round-to-nearest-even) to fp16 or bf16. No
attention arithmetic lives here.

Random draws use ``numpy.random.Generator(PCG64(seed))``. Structure is drawn
first (lengths, trees, page permutation), then q, k, v in that order, so a
workload is a pure function of its seed.

Layouts follow the tree-attention page (tree_attn.py, kernel signatures):
  q / out            [total_q, h_q, d]
  k / v (contiguous) [total_kv, h_kv, d]
  tree mask          [n, 2] int32 rows (enter, exit)
  pages              [num_pages, 2, h_kv, 16, d]  (slot 0 = K, slot 1 = V)
  length_info        [b] last_page_len, or [3, b] (last_page_len,
                     sliding-window offset, sink size)
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

PAGE_SIZE = 16

CONFIG_NAMES = (
    "tree_tiny",        # batch 2, trees of 7 and 15 nodes, h 4/2, d 64, fp16
    "tree_batched",     # batch 16, 64-node trees, h 32/8, d 128, fp16, inline RoPE
    "paged_causal",     # batch 8, causal prefill over paged KV, h 32/8, bf16
    "paged_sliding",    # batch 4, sink 4 + window 4096 of 32768, h 64/8, bf16
    "spec_tree_paged",  # batch 128, 256-node trees over a 4096 prefix, h 64/8
)

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    """N(0,1) drawn in fp32, rounded to the storage dtype (RNE)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(TORCH_DTYPES[dtype])


def random_tree(rng: np.random.Generator, n: int, max_children: Optional[int] = None,
                max_depth: Optional[int] = None):
    """Random rooted tree on nodes 0..n-1 in generation order (parent[i] < i).

    Node i >= 1 picks its parent uniformly among earlier nodes that still have
    fewer than ``max_children`` children and depth below ``max_depth``.
    Returns (parent, depth) int32 arrays, parent[0] = -1, depth[0] = 0.
    """
    parent = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    children = np.zeros(n, dtype=np.int32)
    for i in range(1, n):
        ok = np.ones(i, dtype=bool)
        if max_children is not None:
            ok &= children[:i] < max_children
        if max_depth is not None:
            ok &= depth[:i] < max_depth
        cand = np.flatnonzero(ok)
        if cand.size == 0:
            raise ValueError("tree constraints leave no parent for node %d" % i)
        p = int(cand[rng.integers(cand.size)])
        parent[i] = p
        depth[i] = depth[p] + 1
        children[p] += 1
    return parent, depth


def dfs_intervals(parent: np.ndarray) -> np.ndarray:
    """(enter, exit) per node from a pre-order DFS rooted at node 0.

    Children are visited in increasing index order; enter is the pre-order
    index and exit = enter + subtree size (half-open), so node p is an
    ancestor-or-self of node c exactly when enter[p] <= enter[c] < exit[p].
    """
    n = len(parent)
    kids = [[] for _ in range(n)]
    for i in range(1, n):
        kids[int(parent[i])].append(i)
    enter = np.zeros(n, dtype=np.int32)
    exit_ = np.zeros(n, dtype=np.int32)
    counter = 0
    stack = [(0, False)]
    while stack:
        node, done = stack.pop()
        if done:
            exit_[node] = counter
            continue
        enter[node] = counter
        counter += 1
        stack.append((node, True))
        for c in reversed(kids[node]):
            stack.append((c, False))
    return np.stack([enter, exit_], axis=1).astype(np.int32)


def _indptr(lengths) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


@dataclass
class Workload:
    """One batch of attention inputs (CPU tensors / numpy arrays)."""

    name: str
    kind: str                      # "tree" / "ragged" (contiguous KV) or "paged"
    dtype: str                     # "f16" or "bf16"
    batch: int
    h_q: int
    h_kv: int
    d: int
    sm_scale: float
    rotary_mode: int = 0
    rope_theta: float = 1e4
    rope_scale: float = 1.0
    q: torch.Tensor = None         # [total_q, h_q, d]
    q_indptr: np.ndarray = None    # [b+1]
    q_rope_position: Optional[np.ndarray] = None   # [total_q]
    # contiguous tree attention
    k: Optional[torch.Tensor] = None               # [total_kv, h_kv, d]
    v: Optional[torch.Tensor] = None
    kv_indptr: Optional[np.ndarray] = None
    mn_indptr: Optional[np.ndarray] = None
    tree_mask: Optional[np.ndarray] = None         # [n, 2]
    parents: list = field(default_factory=list)    # per-sequence parent arrays
    depths: list = field(default_factory=list)
    # paged attention
    causal: int = 0
    sliding_window: int = 0
    page_indptr: Optional[np.ndarray] = None
    page_values: Optional[np.ndarray] = None
    length_info: Optional[np.ndarray] = None       # [b] or [3, b]
    num_pages: int = 0
    tree_order_indptr: Optional[np.ndarray] = None
    tree_order: Optional[np.ndarray] = None
    k_rope_pos_offset: Optional[np.ndarray] = None  # [b], in-kernel K rotation
    # Tokens as stored in the cache, in sequence order: token t of sequence b
    # sits at storage offset t. These are the values written into the pages.
    kv_store_indptr: Optional[np.ndarray] = None
    k_store: Optional[torch.Tensor] = None          # [sum stored, h_kv, d]
    v_store: Optional[torch.Tensor] = None
    # Position at which each stored K token is rotated before caching (the
    # "normal" RoPE mode of the KV cache); None when K is stored unrotated.
    store_rope_position: Optional[np.ndarray] = None
    # ragged prefill over contiguous K/V (kind "ragged"): padded-batch masks
    pad_mode: int = 0
    valid_len: Optional[np.ndarray] = None          # [b]
    # multi-head latent attention (kind "mla"): one latent row of d (= d_qk)
    # values per stored token in k_store, shared by every query head; V is
    # its first d_latent values. Pages [num_pages, 16, d].
    d_latent: int = 0

    @property
    def total_q(self) -> int:
        return int(self.q_indptr[-1])

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    def qo_lens(self) -> np.ndarray:
        return np.diff(self.q_indptr)


def mla_pages_from_logical(w: Workload) -> torch.Tensor:
    """Latent page pool [num_pages, 16, d_qk]: stored token t of sequence b in
    page page_values[page_indptr[b] + t // 16], slot t % 16; other slots zero."""
    pool = torch.zeros((w.num_pages, PAGE_SIZE, w.d), dtype=TORCH_DTYPES[w.dtype])
    for b in range(w.batch):
        s0, s1 = int(w.kv_store_indptr[b]), int(w.kv_store_indptr[b + 1])
        if s1 == s0:
            continue
        t = np.arange(s1 - s0)
        pg = torch.from_numpy(w.page_values[w.page_indptr[b] + t // PAGE_SIZE].astype(np.int64))
        pool[pg, torch.from_numpy(t % PAGE_SIZE)] = w.k_store[s0:s1]
    return pool


def pages_from_logical(w: Workload) -> torch.Tensor:
    """Scatter the stored tokens into a page pool [num_pages, 2, h_kv, 16, d].

    Token t of sequence b goes to page page_values[page_indptr[b] + t // 16],
    slot t % 16. Slots past a sequence's stored length stay zero.
    """
    pool = torch.zeros((w.num_pages, 2, w.h_kv, PAGE_SIZE, w.d), dtype=TORCH_DTYPES[w.dtype])
    for b in range(w.batch):
        s0, s1 = int(w.kv_store_indptr[b]), int(w.kv_store_indptr[b + 1])
        n = s1 - s0
        if n == 0:
            continue
        npg = (n + PAGE_SIZE - 1) // PAGE_SIZE
        pg = torch.from_numpy(w.page_values[w.page_indptr[b]:w.page_indptr[b] + npg].astype(np.int64))
        pad = npg * PAGE_SIZE - n
        for src, slot in ((w.k_store, 0), (w.v_store, 1)):
            x = src[s0:s1]
            if pad:
                x = torch.cat([x, torch.zeros((pad,) + tuple(x.shape[1:]), dtype=x.dtype)])
            # [npg, 16, h_kv, d] -> [npg, h_kv, 16, d]
            pool[pg, slot] = x.view(npg, PAGE_SIZE, w.h_kv, w.d).transpose(1, 2)
    return pool


# ----------------------------------------------------------------------------
# builders
# ----------------------------------------------------------------------------

def make_custom_tree(seed: int, tree_sizes, h_q: int, h_kv: int, d: int, dtype: str,
                     rotary_mode: int = 0, rope_theta: float = 1e4, rope_scale: float = 1.0,
                     max_children: Optional[int] = None, max_depth: Optional[int] = None,
                     sm_scale: Optional[float] = None, name: str = "custom_tree",
                     position_offset: int = 0) -> Workload:
    """Contiguous tree attention: each sequence is one tree, kv_indptr = q_indptr."""
    rng = _rng(seed)
    parents, depths, masks = [], [], []
    for n in tree_sizes:
        if n == 0:
            parents.append(np.zeros(0, np.int32))
            depths.append(np.zeros(0, np.int32))
            masks.append(np.zeros((0, 2), np.int32))
            continue
        p, dep = random_tree(rng, n, max_children, max_depth)
        parents.append(p)
        depths.append(dep)
        masks.append(dfs_intervals(p))
    indptr = _indptr(tree_sizes)
    total = int(indptr[-1])
    q = _normal(rng, (total, h_q, d), dtype)
    k = _normal(rng, (total, h_kv, d), dtype)
    v = _normal(rng, (total, h_kv, d), dtype)
    pos = (np.concatenate(depths) if total else np.zeros(0, np.int64)).astype(np.int32)
    return Workload(
        name=name, kind="tree", dtype=dtype, batch=len(tree_sizes), h_q=h_q, h_kv=h_kv, d=d,
        sm_scale=(1.0 / math.sqrt(d)) if sm_scale is None else sm_scale,
        rotary_mode=rotary_mode, rope_theta=rope_theta, rope_scale=rope_scale,
        q=q, q_indptr=indptr, q_rope_position=pos + np.int32(position_offset),
        k=k, v=v, kv_indptr=indptr.copy(), mn_indptr=indptr.copy(),
        tree_mask=np.concatenate(masks).astype(np.int32) if total else np.zeros((0, 2), np.int32),
        parents=parents, depths=depths)


def make_custom_paged(seed: int, qo_lens, stored_lens, h_q: int, h_kv: int, d: int, dtype: str,
                      causal: int = 1, sliding=None, tree: bool = False,
                      tree_max_children: Optional[int] = None, tree_max_depth: Optional[int] = None,
                      store_rope: Optional[str] = None, rotary_mode: int = 0,
                      k_rope_pos_offset=None, rope_theta: float = 1e4, rope_scale: float = 1.0,
                      permute_pages: bool = True, extra_pages: int = 0,
                      sm_scale: Optional[float] = None, name: str = "custom_paged",
                      rng: Optional[np.random.Generator] = None) -> Workload:
    """Paged-KV workload.

    qo_lens[b] query tokens attend to sequence b's KV chunk. stored_lens[b]
    tokens are stored in pages of 16.

    sliding: None, or (window_offset[b], sink[b]) giving the [3, b] length_info.
    tree: if True, the last qo_lens[b] stored tokens of each sequence form a
      random tree (generation order) and the queries are its nodes; everything
      before them is a fully visible prefix.
    store_rope: None (K stored as drawn), "linear" (K rotated before caching at
      its storage offset) or "tree" (prefix offset p at p, tree node i at
      prefix_len + depth(i)); q_rope_position is prefix_len + depth for trees,
      and the storage offset of the query token otherwise.
    rng: continue an existing stream (seed is then ignored).
    """
    rng = _rng(seed) if rng is None else rng
    b = len(qo_lens)
    qo_lens = [int(x) for x in qo_lens]
    stored_lens = [int(x) for x in stored_lens]
    # ---- structure ----
    parents, depths, masks = [], [], []
    if tree:
        for n in qo_lens:
            if n == 0:
                parents.append(np.zeros(0, np.int32))
                depths.append(np.zeros(0, np.int32))
                masks.append(np.zeros((0, 2), np.int32))
                continue
            p, dep = random_tree(rng, n, tree_max_children, tree_max_depth)
            parents.append(p)
            depths.append(dep)
            masks.append(dfs_intervals(p))
    npages = [(s + PAGE_SIZE - 1) // PAGE_SIZE for s in stored_lens]
    num_pages = int(sum(npages)) + int(extra_pages)
    perm = rng.permutation(num_pages).astype(np.int32) if permute_pages else np.arange(num_pages, dtype=np.int32)
    page_indptr = _indptr(npages)
    page_values = perm[: int(page_indptr[-1])].copy()
    last = np.array([s - PAGE_SIZE * (n - 1) if n > 0 else 0 for s, n in zip(stored_lens, npages)], np.int32)
    if sliding is None:
        length_info = last
        sliding_window = 0
    else:
        off, sink = sliding
        length_info = np.stack([last, np.asarray(off, np.int32), np.asarray(sink, np.int32)]).astype(np.int32)
        sliding_window = 1
    q_indptr = _indptr(qo_lens)
    kv_store_indptr = _indptr(stored_lens)
    # ---- values ----
    q = _normal(rng, (int(q_indptr[-1]), h_q, d), dtype)
    k_store = _normal(rng, (int(kv_store_indptr[-1]), h_kv, d), dtype)
    v_store = _normal(rng, (int(kv_store_indptr[-1]), h_kv, d), dtype)
    # ---- positions ----
    q_pos = np.zeros(int(q_indptr[-1]), np.int32)
    store_pos = None
    if store_rope is not None or rotary_mode:
        store_pos = np.zeros(int(kv_store_indptr[-1]), np.int32)
        for i in range(b):
            s0 = int(kv_store_indptr[i])
            n_st = stored_lens[i]
            lin = np.arange(n_st, dtype=np.int32)
            if tree and store_rope == "tree":
                pre = n_st - qo_lens[i]
                lin[pre:] = pre + depths[i]
            store_pos[s0:s0 + n_st] = lin
            q0 = int(q_indptr[i])
            if tree:
                q_pos[q0:q0 + qo_lens[i]] = (n_st - qo_lens[i]) + depths[i]
            else:
                q_pos[q0:q0 + qo_lens[i]] = np.arange(n_st - qo_lens[i], n_st, dtype=np.int32)
        if store_rope is None:
            store_pos = None
    w = Workload(
        name=name, kind="paged", dtype=dtype, batch=b, h_q=h_q, h_kv=h_kv, d=d,
        sm_scale=(1.0 / math.sqrt(d)) if sm_scale is None else sm_scale,
        rotary_mode=rotary_mode, rope_theta=rope_theta, rope_scale=rope_scale,
        q=q, q_indptr=q_indptr, q_rope_position=q_pos,
        causal=int(causal), sliding_window=sliding_window, page_indptr=page_indptr,
        page_values=page_values, length_info=length_info, num_pages=num_pages,
        kv_store_indptr=kv_store_indptr, k_store=k_store, v_store=v_store,
        store_rope_position=store_pos, parents=parents, depths=depths)
    if k_rope_pos_offset is not None:
        w.k_rope_pos_offset = np.asarray(k_rope_pos_offset, np.int32)
    if tree:
        w.tree_order_indptr = _indptr(qo_lens)
        w.tree_order = (np.concatenate(masks) if masks and int(q_indptr[-1]) else np.zeros((0, 2), np.int32)).astype(np.int32)
    return w


def make_custom_ragged(seed: int, qo_lens, kv_lens, h_q: int, h_kv: int, d: int, dtype: str,
                       causal: int = 1, pad_mode: int = 0, valid_lens=None,
                       sm_scale: Optional[float] = None, name: str = "custom_ragged",
                       rng: Optional[np.random.Generator] = None) -> Workload:
    """Ragged prefill over contiguous K/V: sequence b has qo_lens[b] queries
    and kv_lens[b] keys (q_indptr / kv_indptr); pad_mode / valid_lens select
    the padded-batch masks (1: right padding, 2: left padding, causal)."""
    rng = _rng(seed) if rng is None else rng
    qo = [int(x) for x in qo_lens]
    kv = [int(x) for x in kv_lens]
    q_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    kv_indptr = np.concatenate([[0], np.cumsum(kv)]).astype(np.int32)
    q = _normal(rng, (int(q_indptr[-1]), h_q, d), dtype)
    k = _normal(rng, (int(kv_indptr[-1]), h_kv, d), dtype)
    v = _normal(rng, (int(kv_indptr[-1]), h_kv, d), dtype)
    return Workload(name=name, kind="ragged", dtype=dtype, batch=len(qo), h_q=h_q, h_kv=h_kv, d=d,
                    sm_scale=(1.0 / math.sqrt(d)) if sm_scale is None else sm_scale,
                    q=q, q_indptr=q_indptr, k=k, v=v, kv_indptr=kv_indptr, causal=int(causal),
                    pad_mode=int(pad_mode),
                    valid_len=None if valid_lens is None else np.asarray(valid_lens, np.int32))


def make_custom_mla(seed: int, qo_lens, stored_lens, h_q: int, d_qk: int, d_latent: int, dtype: str,
                    causal: int = 1, permute_pages: bool = True, extra_pages: int = 0,
                    sm_scale: Optional[float] = None, name: str = "custom_mla",
                    rng: Optional[np.random.Generator] = None) -> Workload:
    """Latent-cache workload: qo_lens[b] query tokens (h_q heads of d_qk)
    attend to sequence b's stored_lens[b] latent rows (d_qk values each) in
    pages of 16; the queries are the last qo_lens[b] stored tokens."""
    rng = _rng(seed) if rng is None else rng
    b = len(qo_lens)
    qo_lens = [int(x) for x in qo_lens]
    stored_lens = [int(x) for x in stored_lens]
    npages = [(s + PAGE_SIZE - 1) // PAGE_SIZE for s in stored_lens]
    num_pages = int(sum(npages)) + int(extra_pages)
    perm = rng.permutation(num_pages).astype(np.int32) if permute_pages else np.arange(num_pages, dtype=np.int32)
    page_indptr = _indptr(npages)
    page_values = perm[: int(page_indptr[-1])].copy()
    last = np.array([s - PAGE_SIZE * (n - 1) if n > 0 else 0 for s, n in zip(stored_lens, npages)], np.int32)
    q_indptr = _indptr(qo_lens)
    kv_store_indptr = _indptr(stored_lens)
    q = _normal(rng, (int(q_indptr[-1]), h_q, d_qk), dtype)
    kv = _normal(rng, (int(kv_store_indptr[-1]), d_qk), dtype)
    return Workload(name=name, kind="mla", dtype=dtype, batch=b, h_q=h_q, h_kv=1, d=d_qk,
                    sm_scale=(1.0 / math.sqrt(d_qk)) if sm_scale is None else sm_scale,
                    q=q, q_indptr=q_indptr, causal=int(causal), page_indptr=page_indptr,
                    page_values=page_values, length_info=last, num_pages=num_pages,
                    kv_store_indptr=kv_store_indptr, k_store=kv, d_latent=int(d_latent))


# Workloads beyond the five configurations, for entry points adjacent to
# the main path (split-KV decode, padded batches, latent attention).
EXTRA_NAMES = ("paged_decode", "ragged_left_padded", "mla_prefill")


def make_extra(name: str, seed: Optional[int] = None) -> Workload:
    """paged_decode: 16 sequences decoding one token each over 8K-24K cached
    tokens (K rotated when cached, pages permuted), h_q 32 / h_kv 8, d 128,
    bf16, causal. Seed 2000."""
    if name == "ragged_left_padded":
        # 8 prompts left-padded to 2048 tokens (valid 512..2048), causal
        # prefill over their own keys, h 32/8, d 128, bf16. Seed 2001.
        seed = 2001 if seed is None else seed
        rng = _rng(seed)
        valid = rng.integers(512, 2049, size=8)
        return make_custom_ragged(seed, [2048] * 8, [2048] * 8, h_q=32, h_kv=8, d=128, dtype="bf16",
                                  causal=1, pad_mode=2, valid_lens=valid, name=name, rng=rng)
    if name == "mla_prefill":
        # 8 sequences, qo ~ U[512, 2048] new tokens after a cached prefix
        # ~ U[0, 2048], 16 query heads (a 128-head model's share at 8-way
        # head sharding) over a latent cache of 512 + 64 values per token,
        # bf16, causal; sm_scale 1/sqrt(192) as for 128 + 64-dim heads
        # before absorption. Seed 2002.
        seed = 2002 if seed is None else seed
        rng = _rng(seed)
        qo = rng.integers(512, 2049, size=8)
        prefix = rng.integers(0, 2049, size=8)
        return make_custom_mla(seed, qo, prefix + qo, h_q=16, d_qk=576, d_latent=512, dtype="bf16",
                               causal=1, sm_scale=1.0 / math.sqrt(192.0), name=name, rng=rng)
    if name != "paged_decode":
        raise KeyError(name)
    seed = 2000 if seed is None else seed
    rng = _rng(seed)
    b = 16
    stored = rng.integers(8192, 24577, size=b)
    return make_custom_paged(seed, [1] * b, stored, h_q=32, h_kv=8, d=128, dtype="bf16",
                             causal=1, store_rope="linear", rotary_mode=0, rope_theta=1e4,
                             name=name, rng=rng)


def make_config(k: int, seed: Optional[int] = None) -> Workload:
    """The five workloads, by 0-based index into CONFIG_NAMES. Seed 1000 + k."""
    name = CONFIG_NAMES[k]
    seed = 1000 + k if seed is None else seed
    if k == 0:
        return make_custom_tree(seed, [7, 15], h_q=4, h_kv=2, d=64, dtype="f16",
                                rotary_mode=0, name=name)
    if k == 1:
        return make_custom_tree(seed, [64] * 16, h_q=32, h_kv=8, d=128, dtype="f16",
                                rotary_mode=1, rope_theta=1e4, rope_scale=1.0,
                                max_children=4, name=name)
    if k == 2:
        rng = _rng(seed)
        qo = rng.integers(512, 2049, size=8)
        prefix = rng.integers(0, 2049, size=8)
        return make_custom_paged(seed, qo, prefix + qo, h_q=32, h_kv=8, d=128,
                                 dtype="bf16", causal=1, store_rope="linear", rotary_mode=0,
                                 rope_theta=1e4, name=name, rng=rng)
    if k == 3:
        b, stored, window, sink = 4, 32768, 4096, 4
        return make_custom_paged(seed, [1024] * b, [stored] * b, h_q=64, h_kv=8, d=128,
                                 dtype="bf16", causal=1,
                                 sliding=([stored - window] * b, [sink] * b), name=name)
    if k == 4:
        b, prefix, n = 128, 4096, 256
        return make_custom_paged(seed, [n] * b, [prefix + n] * b, h_q=64, h_kv=8, d=128,
                                 dtype="bf16", causal=0, tree=True, tree_max_children=4,
                                 tree_max_depth=16, store_rope="tree", rotary_mode=1,
                                 rope_theta=5e5, name=name)
    raise IndexError(k)
