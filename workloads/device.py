"""Stage a workload on the GPU and launch it through the library's Python
binding (used by the tests, the smoke test and the benchmark).

Paged workloads whose K is rotated before caching get their page pool from
the library's append kernel (ra_paged_kv_append), which rotates K on the way
in; the others copy the generator's pages. Nothing here computes attention.
"""

from __future__ import annotations

import numpy as np
import torch

from .generators import mla_pages_from_logical, pages_from_logical


def _i32(a, dev):
    return None if a is None else torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32, device=dev)


def append_range(pool, w, starts, lens, dev):
    """Append tokens [starts[b], starts[b] + lens[b]) of each sequence's
    stored tokens into ``pool`` with the library's append kernel, at storage
    offsets starts[b] (any offset: mid-page starts are the normal case),
    rotating K at the workload's cache positions."""
    import attention_ragged_gqa_amd as ra
    starts = np.asarray(starts, np.int64)
    lens = np.asarray(lens, np.int64)
    idx = np.concatenate([np.arange(int(w.kv_store_indptr[b]) + starts[b],
                                    int(w.kv_store_indptr[b]) + starts[b] + lens[b])
                          for b in range(w.batch)]).astype(np.int64) if w.batch else np.zeros(0, np.int64)
    sel = torch.from_numpy(idx)
    indptr = np.zeros(w.batch + 1, np.int64)
    indptr[1:] = np.cumsum(lens)
    ra.ra_paged_kv_append(w.k_store[sel].to(dev), w.v_store[sel].to(dev), _i32(indptr, dev),
                          _i32(starts, dev), _i32(np.asarray(w.store_rope_position)[idx], dev),
                          _i32(w.page_indptr, dev), _i32(w.page_values, dev), pool,
                          rope_scale=w.rope_scale, rope_theta=w.rope_theta)


def gpu_pages(w, dev):
    """Page pool on the device. K rotated before caching is written by the
    library's append kernel in two calls, as a cache is filled in use: each
    sequence's cached prefix at storage offset 0, then its new tokens (the
    last qo_len stored tokens, the ones the queries belong to) appended
    after it, usually starting mid-page. Otherwise the generator's pages are
    copied."""
    if w.store_rope_position is None:
        return pages_from_logical(w).to(dev)
    pool = torch.zeros((w.num_pages, 2, w.h_kv, 16, w.d), dtype=w.q.dtype, device=dev)
    stored = np.diff(w.kv_store_indptr).astype(np.int64)
    new = np.minimum(np.diff(w.q_indptr).astype(np.int64), stored)
    old = stored - new
    append_range(pool, w, np.zeros(w.batch, np.int64), old, dev)
    append_range(pool, w, old, new, dev)
    return pool


class DeviceInputs:
    """All device tensors of one workload, built once, so the same launch can
    be repeated (tests, bench)."""

    def __init__(self, w, dev="cuda:0"):
        self.w = w
        self.dev = torch.device(dev)
        d = self.dev
        self.q = w.q.to(d)
        self.q_indptr = _i32(w.q_indptr, d)
        self.q_rope_position = _i32(w.q_rope_position, d) if w.rotary_mode == 1 else None
        # poisoned: a row the kernels never write stays NaN
        out_d = w.d_latent if w.kind == "mla" else w.d
        self.out = torch.full((w.total_q, w.h_q, out_d), float("nan"), dtype=w.q.dtype, device=d)
        self.lse = torch.full((w.total_q, w.h_q), float("nan"), dtype=torch.float32, device=d)
        if w.kind == "tree":
            self.k = w.k.to(d)
            self.v = w.v.to(d)
            self.kv_indptr = _i32(w.kv_indptr, d)
            self.mn_indptr = _i32(w.mn_indptr, d)
            self.tree_mask = _i32(w.tree_mask.reshape(-1, 2), d)
        elif w.kind == "mla":
            self.pages = mla_pages_from_logical(w).to(d)
            self.page_indptr = _i32(w.page_indptr, d)
            self.page_values = _i32(w.page_values, d)
            self.length_info = _i32(w.length_info, d)
        elif w.kind == "ragged":
            self.k = w.k.to(d)
            self.v = w.v.to(d)
            self.kv_indptr = _i32(w.kv_indptr, d)
            self.valid_len = _i32(w.valid_len, d)
        else:
            self.pages = gpu_pages(w, d)
            self.page_indptr = _i32(w.page_indptr, d)
            self.page_values = _i32(w.page_values, d)
            self.length_info = _i32(w.length_info, d)
            self.k_rope_pos_offset = _i32(w.k_rope_pos_offset, d)
            self.tree_order_indptr = _i32(w.tree_order_indptr, d)
            self.tree_order = _i32(None if w.tree_order is None else w.tree_order.reshape(-1, 2), d)

    def poison(self):
        """Fill out and lse with NaN, so that rows a launch leaves unwritten
        are caught by the finiteness checks."""
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))

    def launch(self, stream=None, num_kv_splits=None):
        """One launch; num_kv_splits (paged only) selects the split-KV entry
        point (0: the library chooses the count)."""
        import attention_ragged_gqa_amd as ra
        w = self.w
        if num_kv_splits is not None:
            if w.kind != "paged":
                raise ValueError("split-KV is a paged entry point")
            if getattr(self, "workspace", None) is None:
                n = ra.ra_paged_attn_split_workspace(w.total_q, w.h_q, w.d, 64)
                self.workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=self.dev)
            return ra.ra_paged_attn_split(
                self.q, self.q_indptr, self.pages, self.page_indptr, self.page_values,
                self.length_info, sliding_window=w.sliding_window,
                k_rope_pos_offset=self.k_rope_pos_offset, q_rope_position=self.q_rope_position,
                tree_order_indptr=self.tree_order_indptr, tree_order=self.tree_order,
                causal=w.causal, out=self.out, lse=self.lse, rotary_mode=w.rotary_mode,
                rope_scale=w.rope_scale, rope_theta=w.rope_theta, sm_scale=w.sm_scale,
                num_kv_splits=num_kv_splits, workspace=self.workspace, stream=stream)
        if w.kind == "mla":
            return ra.ra_mla_paged_prefill(self.q, self.q_indptr, self.pages, self.page_indptr,
                                           self.page_values, self.length_info, causal=w.causal,
                                           d_latent=w.d_latent, out=self.out, lse=self.lse,
                                           sm_scale=w.sm_scale, stream=stream)
        if w.kind == "ragged":
            return ra.ra_ragged_prefill(self.q, self.q_indptr, self.k, self.v, self.kv_indptr,
                                        valid_len=self.valid_len, pad_mode=w.pad_mode,
                                        causal=w.causal, out=self.out, lse=self.lse,
                                        sm_scale=w.sm_scale, stream=stream)
        if w.kind == "tree":
            return ra.ra_tree_attn(self.q, self.q_indptr, self.k, self.v, self.kv_indptr,
                                   self.q_rope_position, self.mn_indptr, self.tree_mask,
                                   out=self.out, lse=self.lse, rotary_mode=w.rotary_mode,
                                   rope_scale=w.rope_scale, rope_theta=w.rope_theta,
                                   sm_scale=w.sm_scale, stream=stream)
        return ra.ra_paged_attn(self.q, self.q_indptr, self.pages, self.page_indptr,
                                self.page_values, self.length_info,
                                sliding_window=w.sliding_window,
                                k_rope_pos_offset=self.k_rope_pos_offset,
                                q_rope_position=self.q_rope_position,
                                tree_order_indptr=self.tree_order_indptr,
                                tree_order=self.tree_order, causal=w.causal, out=self.out,
                                lse=self.lse, rotary_mode=w.rotary_mode, rope_scale=w.rope_scale,
                                rope_theta=w.rope_theta, sm_scale=w.sm_scale, stream=stream)


class AppendInputs:
    """The append step of a paged workload whose K is rotated before caching:
    the new tokens of every sequence (its last qo_len stored tokens, K, V and
    their cache positions, on the device) and the page pool. launch() appends
    the new tokens at their storage offsets (after each sequence's cached
    prefix, mid-page where the prefix ends mid-page), rotating K; repeated
    launches rewrite the same values. The append never reads the pool, so
    the prefix slots are left zero (staging them would run the same kernel
    on 16 times the tokens of the measured step)."""

    def __init__(self, w, dev="cuda:0"):
        if w.kind != "paged" or w.store_rope_position is None:
            raise ValueError("the append step needs a paged workload with K rotated before caching")
        self.w = w
        self.dev = torch.device(dev)
        d = self.dev
        stored = np.diff(w.kv_store_indptr).astype(np.int64)
        new = np.minimum(np.diff(w.q_indptr).astype(np.int64), stored)
        old = stored - new
        self.n_tokens = int(new.sum())
        self.pool = torch.zeros((w.num_pages, 2, w.h_kv, 16, w.d), dtype=w.q.dtype, device=d)
        idx = np.concatenate([np.arange(int(w.kv_store_indptr[b]) + old[b], int(w.kv_store_indptr[b + 1]))
                              for b in range(w.batch)]).astype(np.int64)
        sel = torch.from_numpy(idx)
        self.k = w.k_store[sel].to(d)
        self.v = w.v_store[sel].to(d)
        indptr = np.zeros(w.batch + 1, np.int64)
        indptr[1:] = np.cumsum(new)
        self.append_indptr = _i32(indptr, d)
        self.append_start = _i32(old, d)
        self.rope_position = _i32(np.asarray(w.store_rope_position)[idx], d)
        self.page_indptr = _i32(w.page_indptr, d)
        self.page_values = _i32(w.page_values, d)
        self.new_start = old
        self.new_len = new

    def launch(self, stream=None):
        import attention_ragged_gqa_amd as ra
        w = self.w
        return ra.ra_paged_kv_append(self.k, self.v, self.append_indptr, self.append_start,
                                     self.rope_position, self.page_indptr, self.page_values, self.pool,
                                     rope_scale=w.rope_scale, rope_theta=w.rope_theta, stream=stream)
