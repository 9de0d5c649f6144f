"""Vectorised float64 CPU oracle (test infrastructure; see the package docstring).

Definitions followed, by page and section:

* Scores. "_kernel_common.py" page, macro ``compute_s_gemm``: s = sm_scale *
  sum_t q[t] k[t] accumulated from the dtype values. The kernels carry the
  scores pre-multiplied by log2(e) and use exp2; that is the same softmax.
* Softmax state and epilogue. Same page, macros ``softmax_update_causal`` and
  ``paged_store_output_lse``: out = sum_j softmax(s)_j v_j over visible keys,
  lse = m + log2(d) in the log2 domain, i.e. lse = log2(sum_j exp(s_j)).
  The online (tiled) update is a reordering of this sum, so the oracle uses
  the two-pass definition.
* Causal mask. Same page, ``_causal_mask``: column j is visible to query row
  i iff j < kv_len - qo_len + i + 1 (bottom-right aligned), else j < kv_len.
* Tree mask. "tree_attn.py" page, ``_check_tree_order``: with tree_len nodes
  at the end of the KV, tree_start = kv_len - tree_len; column j is visible
  iff j < kv_len and (j < tree_start or enter[c] in [enter[p], exit[p])),
  c = i + tree_len - qo_len, p = j - tree_start.
* Paged KV. "_kernel_common.py" page, ``_get_kv_chunk_len`` and
  ``_get_seq_offset``, with the page gather of the paged tree kernel on the
  "tree_attn.py" page: chunk length (np-1)*16 + last_page_len (minus the
  window offset plus the sink when the sliding window is on); chunk position
  j maps to storage offset j, or j - sink + window_offset past the sink;
  offset o lives in page page_values[page_indptr[b] + o // 16], slot o % 16.
* Rotary embedding. "_kernel_common.py" page, ``_rope``: rotate-half over
  rotary_dim = head_dim, evaluated in float32 and cast to the storage dtype.
  The frequency function it calls is not on the pages; the plain unscaled
  reading is used: dims t and t + D/2 share inv_freq = theta^(-2k/D) with
  k = t mod D/2, angle = float32(pos * scale) * inv_freq.

Every entry point takes an optional ``spread`` array shaped like ``out``:
when given, it is filled with the standard deviation of v under each row's
attention weights (``attend``). That statistic is not part of the operation;
the parity tests use it to bound how far rounding the weights to the MFMA
input type can move an output.

Readings where the pages are silent (also listed in the design notes):
  * A row with no visible key yields out = 0 and lse = -inf.
  * A tree row whose node index c falls outside [0, tree_len) sees only the
    prefix columns.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

LN2 = math.log(2.0)
PAGE_SIZE = 16

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _round_f32_to(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (RNE), returned as float64."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(_TORCH[dtype]).to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# rotary embedding ("_kernel_common.py" page, _rope)
# ----------------------------------------------------------------------------

def _rope_angles(pos: np.ndarray, d: int, theta: float, scale: float) -> np.ndarray:
    """Angles [n, d/2] in float64: float32(pos * scale) * theta^(-2k/d)."""
    pos_f32 = (np.asarray(pos).astype(np.float32) * np.float32(scale)).astype(np.float64)
    k = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * k / d)
    return pos_f32[:, None] * inv_freq[None, :]


def rope_exact(x: np.ndarray, pos: np.ndarray, theta: float, scale: float) -> np.ndarray:
    """Rotate-half RoPE in float64 without rounding. x [n, H, D], pos [n]."""
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    ang = _rope_angles(pos, d, theta, scale)[:, None, :]          # [n, 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope(x, pos: np.ndarray, theta: float, scale: float, dtype: str) -> np.ndarray:
    """Rotate-half RoPE as the pages evaluate it: float32 cos/sin and products,
    y[t] = cos*x[t] + sin*(t < D/2 ? -x[t+D/2] : x[t-D/2]), cast to dtype.
    x [n, H, D] (dtype values), pos [n]. Returns float64 values of dtype."""
    x32 = _f64(x).astype(np.float32)
    d = x32.shape[-1]
    half = d // 2
    ang = _rope_angles(pos, d, theta, scale)
    cos32 = np.cos(ang).astype(np.float32)[:, None, :]
    sin32 = np.sin(ang).astype(np.float32)[:, None, :]
    cos_full = np.concatenate([cos32, cos32], axis=-1)
    sin_full = np.concatenate([sin32, sin32], axis=-1)
    partner = np.concatenate([-x32[..., half:], x32[..., :half]], axis=-1)
    y32 = (cos_full * x32).astype(np.float32) + (sin_full * partner).astype(np.float32)
    return _round_f32_to(y32.astype(np.float32), dtype)


# ----------------------------------------------------------------------------
# masks
# ----------------------------------------------------------------------------

def causal_visible(rows: np.ndarray, kv_len: int, qo_len: int, causal: int = 1) -> np.ndarray:
    """[len(rows), kv_len] visibility ("_kernel_common.py" page, _causal_mask)."""
    cols = np.arange(kv_len)[None, :]
    rows = np.asarray(rows)[:, None]
    if causal > 0:
        return cols < (kv_len - qo_len + rows + 1)
    return np.broadcast_to(cols < kv_len, (rows.shape[0], kv_len)).copy()


def tree_visible(order: np.ndarray, rows: np.ndarray, kv_len: int, qo_len: int) -> np.ndarray:
    """[len(rows), kv_len] visibility ("tree_attn.py" page, _check_tree_order).

    order: this sequence's [tree_len, 2] (enter, exit) rows."""
    order = np.asarray(order).reshape(-1, 2)
    tree_len = order.shape[0]
    tree_start = kv_len - tree_len
    rows = np.asarray(rows)
    cols = np.arange(kv_len)
    c = rows + tree_len - qo_len                        # query's node index
    vis = np.zeros((rows.shape[0], kv_len), dtype=bool)
    vis[:, : max(tree_start, 0)] = True                 # prefix columns
    if tree_len == 0:
        return vis
    p = cols[max(tree_start, 0):] - tree_start          # key node indices
    ok_c = (c >= 0) & (c < tree_len)
    cc = np.clip(c, 0, tree_len - 1)
    enter_c = order[cc, 0][:, None]
    in_tree = (enter_c >= order[p, 0][None, :]) & (enter_c < order[p, 1][None, :])
    vis[:, max(tree_start, 0):] = in_tree & ok_c[:, None]
    return vis


# ----------------------------------------------------------------------------
# paged KV helpers ("_kernel_common.py" page)
# ----------------------------------------------------------------------------

def kv_chunk_len(b: int, page_indptr, length_info, sliding_window: int) -> int:
    """_get_kv_chunk_len, with 0 for a sequence that owns no pages."""
    npg = int(page_indptr[b + 1]) - int(page_indptr[b])
    if npg == 0:
        return 0
    li = np.asarray(length_info)
    if not sliding_window:
        return (npg - 1) * PAGE_SIZE + int(li[b])
    return (npg - 1) * PAGE_SIZE + int(li[0, b]) - int(li[1, b]) + int(li[2, b])


def seq_offset(j: np.ndarray, b: int, length_info, sliding_window: int) -> np.ndarray:
    """_get_seq_offset: chunk position -> storage offset in the sequence."""
    j = np.asarray(j)
    if not sliding_window:
        return j
    li = np.asarray(length_info)
    sink, off = int(li[2, b]), int(li[1, b])
    return np.where(j < sink, j, j - sink + off)


# ----------------------------------------------------------------------------
# the attention definition
# ----------------------------------------------------------------------------

def attend(qr: np.ndarray, kr: np.ndarray, vr: np.ndarray, vis: np.ndarray, sm_scale: float,
           spread: bool = False):
    """out = softmax(sm_scale * q k^T | visible) v and lse = log2 sum exp.

    qr [R, D], kr [L, D], vr [L, Dv] float64 (Dv = D, or the latent width
    for multi-head latent attention); vis [R, L] bool.
    Rows with no visible key: out = 0, lse = -inf.
    spread: also return the standard deviation of v under each row's
    attention weights, sqrt(sum_j w_j v_j^2 - out^2) per column (0 for rows
    with no visible key). It is not part of the operation: parity tests use
    it to bound the effect of rounding the weights (see tests/parity.py)."""
    R = qr.shape[0]
    out = np.zeros((R, vr.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    sd = np.zeros((R, vr.shape[1]), dtype=np.float64)
    if kr.shape[0] == 0 or R == 0:
        return (out, lse, sd) if spread else (out, lse)
    s = sm_scale * (qr @ kr.T)
    s = np.where(vis, s, -np.inf)
    has = vis.any(axis=1)
    if not has.any():
        return (out, lse, sd) if spread else (out, lse)
    m = np.max(s[has], axis=1, keepdims=True)
    p = np.exp(s[has] - m)
    denom = p.sum(axis=1, keepdims=True)
    out[has] = (p @ vr) / denom
    lse[has] = (m[:, 0] + np.log(denom[:, 0])) / LN2
    if spread:
        second = (p @ (vr * vr)) / denom
        sd[has] = np.sqrt(np.maximum(second - out[has] ** 2, 0.0))
        return out, lse, sd
    return out, lse


def merge_states(part_out: np.ndarray, part_lse: np.ndarray):
    """Combine attention states over disjoint key sets.

    part_out [S, R, D] (each row normalised over its own key set), part_lse
    [S, R] base-2 log-sum-exp (-inf for an empty set). Since each part is
    out_s = sum_{j in K_s} e^{s_j} v_j / sum_{j in K_s} e^{s_j} with
    sum_{j in K_s} e^{s_j} = 2^{lse_s}, the union gives
    lse = log2 sum_s 2^{lse_s} and out = sum_s 2^{lse_s - lse} out_s
    (the online-softmax update of the "_kernel_common.py" page applied to
    whole key sets). Rows empty in every part: out 0, lse -inf."""
    part_out = np.asarray(part_out, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    S, R, D = part_out.shape
    out = np.zeros((R, D), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    has = np.isfinite(part_lse).any(axis=0)
    if not has.any():
        return out, lse
    m = np.max(np.where(np.isfinite(part_lse[:, has]), part_lse[:, has], -np.inf), axis=0)
    w = np.exp2(part_lse[:, has] - m)                      # [S, R'] (0 for empty parts)
    tot = w.sum(axis=0)
    lse[has] = m + np.log2(tot)
    out[has] = np.einsum("sr,srd->rd", w / tot, part_out[:, has, :])
    return out, lse


def _select_tokens(q_indptr, rows: Optional[np.ndarray], b: int) -> np.ndarray:
    """Query indices (within sequence b) to evaluate."""
    q0, q1 = int(q_indptr[b]), int(q_indptr[b + 1])
    if rows is None:
        return np.arange(q1 - q0)
    r = np.asarray(rows)
    return np.sort(r[(r >= q0) & (r < q1)] - q0)


def _extra(spread):
    """Trailing argument of _attend_sequence: the spread array when requested."""
    return () if spread is None else (spread,)


def _attend_sequence(qb, tok_global, qi, kseq, vseq, vis, h_q, h_kv, sm_scale, out, lse, spread=None):
    """qb [n, h_q, d] rows of this sequence; writes out/lse (and, when given,
    spread) at tok_global. Query head h reads KV head h // (h_q / h_kv)."""
    g = h_q // h_kv
    for kvh in range(h_kv):
        heads = slice(kvh * g, (kvh + 1) * g)
        qr = qb[:, heads, :].reshape(len(qi) * g, -1)
        vis_r = np.repeat(vis, g, axis=0)
        if spread is None:
            res = attend(qr, kseq[:, kvh, :], vseq[:, kvh, :], vis_r, sm_scale)
        else:
            res = attend(qr, kseq[:, kvh, :], vseq[:, kvh, :], vis_r, sm_scale, spread=True)
        out[tok_global, heads, :] = res[0].reshape(len(qi), g, -1)
        lse[tok_global, heads] = res[1].reshape(len(qi), g)
        if spread is not None:
            spread[tok_global, heads, :] = res[2].reshape(len(qi), g, -1)


def tree_attn(q, q_indptr, k, v, kv_indptr, q_rope_position, mn_indptr, tree_mask,
              rotary_mode: int, rope_scale: float, rope_theta: float, sm_scale: float,
              dtype: str, rows: Optional[np.ndarray] = None, spread: Optional[np.ndarray] = None):
    """Batched tree attention over contiguous KV ("tree_attn.py" page, the
    tree_attn operator and its CPU kernel).

    q [total_q, h_q, d]; k, v [total_kv, h_kv, d] (dtype values as torch or
    numpy); index arrays int32. With rotary_mode == 1, q row r is rotated at
    q_rope_position[r] and K row kv_indptr[b] + j at q_rope_position of that
    same index, as the page's kernels do.
    rows: optional global query indices to evaluate (others stay NaN).
    Returns (out [total_q, h_q, d], lse [total_q, h_q]) float64."""
    total_q, h_q, d = q.shape
    h_kv = k.shape[1]
    out = np.full((total_q, h_q, d), np.nan)
    lse = np.full((total_q, h_q), np.nan)
    q_indptr = np.asarray(q_indptr)
    kv_indptr = np.asarray(kv_indptr)
    mn_indptr = np.asarray(mn_indptr)
    tree_mask = np.asarray(tree_mask).reshape(-1, 2)
    pos = None if q_rope_position is None else np.asarray(q_rope_position)
    batch = len(q_indptr) - 1
    for b in range(batch):
        qi = _select_tokens(q_indptr, rows, b)
        if len(qi) == 0:
            continue
        q0 = int(q_indptr[b])
        qo_len = int(q_indptr[b + 1]) - q0
        k0, k1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
        kv_len = k1 - k0
        tok = q0 + qi
        qb = _f64(q[tok])
        kb = _f64(k[k0:k1])
        if rotary_mode == 1:
            qb = rope(qb, pos[tok], rope_theta, rope_scale, dtype)
            kb = rope(kb, pos[k0:k1], rope_theta, rope_scale, dtype)
        order = tree_mask[int(mn_indptr[b]):int(mn_indptr[b + 1])]
        vis = tree_visible(order, qi, kv_len, qo_len)
        _attend_sequence(qb, tok, qi, kb, _f64(v[k0:k1]), vis, h_q, h_kv, sm_scale, out, lse, *_extra(spread))
    return out, lse


def paged_attn(q, q_indptr, pages, page_indptr, page_values, length_info, sliding_window: int,
               causal: int, sm_scale: float, dtype: str, *, tree_order_indptr=None,
               tree_order=None, q_rope_position=None, k_rope_pos_offset=None,
               rotary_mode: int = 0, rope_scale: float = 1.0, rope_theta: float = 1e4,
               cache_rope_position=None, cache_rope_indptr=None,
               rows: Optional[np.ndarray] = None, spread: Optional[np.ndarray] = None):
    """Ragged prefill / tree attention over a paged KV cache.

    pages [num_pages, 2, h_kv, 16, d]. The mask is the tree test when tree
    arrays are given ("tree_attn.py" page, paged tree kernel), else the causal
    test with the ``causal`` flag ("_kernel_common.py" page, _causal_mask).
    With rotary_mode == 1, q is rotated at q_rope_position[row]; K is rotated
    at k_rope_pos_offset[b] + j (chunk position j) when k_rope_pos_offset is
    given, and taken as stored otherwise.
    cache_rope_position / cache_rope_indptr: the K values in ``pages`` are
    the unrotated values of a cache whose K was rotated before caching at
    position cache_rope_position[cache_rope_indptr[b] + storage offset]; the
    oracle applies that rotation after the gather.
    Returns (out [total_q, h_q, d], lse [total_q, h_q]) float64."""
    total_q, h_q, d = q.shape
    h_kv = pages.shape[2]
    out = np.full((total_q, h_q, d), np.nan)
    lse = np.full((total_q, h_q), np.nan)
    q_indptr = np.asarray(q_indptr)
    page_indptr = np.asarray(page_indptr)
    page_values = np.asarray(page_values)
    batch = len(q_indptr) - 1
    for b in range(batch):
        qi = _select_tokens(q_indptr, rows, b)
        if len(qi) == 0:
            continue
        q0 = int(q_indptr[b])
        qo_len = int(q_indptr[b + 1]) - q0
        L = kv_chunk_len(b, page_indptr, length_info, sliding_window)
        tok = q0 + qi
        j = np.arange(L)
        off = seq_offset(j, b, length_info, sliding_window)
        page = page_values[int(page_indptr[b]) + off // PAGE_SIZE] if L else np.zeros(0, np.int64)
        slot = off % PAGE_SIZE
        pg_t = torch.from_numpy(np.asarray(page, dtype=np.int64))
        sl_t = torch.from_numpy(np.asarray(slot, dtype=np.int64))
        kb = _f64(pages[pg_t, 0, :, sl_t, :]) if L else np.zeros((0, h_kv, d))   # [L, h_kv, d]
        vb = _f64(pages[pg_t, 1, :, sl_t, :]) if L else np.zeros((0, h_kv, d))
        if cache_rope_position is not None and L:
            cpos = np.asarray(cache_rope_position)[int(cache_rope_indptr[b]) + off]
            kb = rope(kb, cpos, rope_theta, rope_scale, dtype)
        qb = _f64(q[tok])
        if rotary_mode == 1:
            qb = rope(qb, np.asarray(q_rope_position)[tok], rope_theta, rope_scale, dtype)
            if k_rope_pos_offset is not None and L:
                kb = rope(kb, int(np.asarray(k_rope_pos_offset)[b]) + j, rope_theta, rope_scale, dtype)
        if tree_order is not None:
            toi = np.asarray(tree_order_indptr)
            order = np.asarray(tree_order).reshape(-1, 2)[int(toi[b]):int(toi[b + 1])]
            vis = tree_visible(order, qi, L, qo_len)
        else:
            vis = causal_visible(qi, L, qo_len, causal)
        _attend_sequence(qb, tok, qi, kb, vb, vis, h_q, h_kv, sm_scale, out, lse, *_extra(spread))
    return out, lse


# ----------------------------------------------------------------------------
# ragged prefill over contiguous K/V, with the padded-batch masks
# ----------------------------------------------------------------------------

def padded_visible(rows: np.ndarray, kv_len: int, qo_len: int, valid: int, pad_mode: int,
                   causal: int) -> np.ndarray:
    """Visibility [len(rows), kv_len] for query rows of one sequence.

    pad_mode 0: the causal test (_causal_mask, "_kernel_common.py" page).
    pad_mode 1: right padding, macro softmax_update_valid_length on the same
      page: row < qo_len, row < valid and col < valid.
    pad_mode 2: left padding with causal alignment, macro
      softmax_update_causal_padded_left: row in [qo_len - valid, qo_len),
      col in [kv_len - valid, kv_len - qo_len + row + 1)."""
    rows = np.asarray(rows)
    col = np.arange(kv_len)[None, :]
    r = rows[:, None]
    if pad_mode == 0:
        return causal_visible(rows, kv_len, qo_len, causal)
    if pad_mode == 1:
        return (r < qo_len) & (r < valid) & (col < valid)
    if pad_mode == 2:
        pad_q, pad_kv = qo_len - valid, kv_len - valid
        return (r < qo_len) & (r >= pad_q) & (col >= pad_kv) & (col < kv_len - qo_len + r + 1)
    raise ValueError(pad_mode)


def ragged_prefill(q, q_indptr, k, v, kv_indptr, valid_len, pad_mode: int, causal: int,
                   sm_scale: float, rows: Optional[np.ndarray] = None,
                   spread: Optional[np.ndarray] = None):
    """Ragged prefill: sequence b's queries q[q_indptr[b]:q_indptr[b+1]]
    attend to k/v[kv_indptr[b]:kv_indptr[b+1]] under padded_visible.
    Returns (out [total_q, h_q, d], lse [total_q, h_q]) float64."""
    total_q, h_q, d = q.shape
    h_kv = k.shape[1]
    out = np.full((total_q, h_q, d), np.nan)
    lse = np.full((total_q, h_q), np.nan)
    q_indptr = np.asarray(q_indptr)
    kv_indptr = np.asarray(kv_indptr)
    for b in range(len(q_indptr) - 1):
        qi = _select_tokens(q_indptr, rows, b)
        if len(qi) == 0:
            continue
        q0 = int(q_indptr[b])
        qo_len = int(q_indptr[b + 1]) - q0
        k0, k1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
        L = k1 - k0
        valid = 0 if valid_len is None else int(np.asarray(valid_len)[b])
        vis = padded_visible(qi, L, qo_len, valid, pad_mode, causal)
        tok = q0 + qi
        _attend_sequence(_f64(q[tok]), tok, qi, _f64(k[k0:k1]), _f64(v[k0:k1]), vis, h_q, h_kv,
                         sm_scale, out, lse, *_extra(spread))
    return out, lse


# ----------------------------------------------------------------------------
# multi-head latent attention over a paged latent cache
# ----------------------------------------------------------------------------

def mla_paged_attn(q, q_indptr, pages, page_indptr, page_values, last_page_len, causal: int,
                   sm_scale: float, d_latent: int, rows: Optional[np.ndarray] = None,
                   spread: Optional[np.ndarray] = None):
    """Multi-head latent attention prefill ("_kernel_common.py" page: AttnKind
    MLA, and _alloc_mla_qkvo_buffers, whose one combined KV tile serves as K
    over all d_qk columns and as V over the first d_latent columns; the
    epilogue paged_store_output_lse with every query head in one group).

    q [total_q, h_q, d_qk]; pages [num_pages, 16, d_qk] hold one latent row
    per token (no K/V split, no KV heads); sequence b's rows are at storage
    offsets 0..kv_len-1, kv_len = (np - 1) * 16 + last_page_len[b] for its
    np pages (0 with no pages), offset o in page page_values[page_indptr[b]
    + o // 16], slot o % 16. For query token i of sequence b and head h:
      s_j = sm_scale * sum_{t < d_qk} q[i, h, t] kv_j[t]
      out[i, h, :] = sum_j softmax(s)_j kv_j[:d_latent]
      lse[i, h] = log2 sum_j exp(s_j)
    over the keys the causal test (_causal_mask) leaves visible.
    Returns (out [total_q, h_q, d_latent], lse [total_q, h_q]) float64."""
    total_q, h_q, d_qk = q.shape
    out = np.full((total_q, h_q, d_latent), np.nan)
    lse = np.full((total_q, h_q), np.nan)
    q_indptr = np.asarray(q_indptr)
    page_indptr = np.asarray(page_indptr)
    page_values = np.asarray(page_values)
    for b in range(len(q_indptr) - 1):
        qi = _select_tokens(q_indptr, rows, b)
        if len(qi) == 0:
            continue
        q0 = int(q_indptr[b])
        qo_len = int(q_indptr[b + 1]) - q0
        L = kv_chunk_len(b, page_indptr, last_page_len, 0)
        j = np.arange(L)
        page = page_values[int(page_indptr[b]) + j // PAGE_SIZE] if L else np.zeros(0, np.int64)
        pg_t = torch.from_numpy(np.asarray(page, dtype=np.int64))
        sl_t = torch.from_numpy(np.asarray(j % PAGE_SIZE, dtype=np.int64))
        kv = _f64(pages[pg_t, sl_t, :]) if L else np.zeros((0, d_qk))       # [L, d_qk]
        vis = causal_visible(qi, L, qo_len, causal)
        tok = q0 + qi
        qb = _f64(q[tok])                                                    # [n, h_q, d_qk]
        qr = qb.reshape(len(qi) * h_q, d_qk)
        vis_r = np.repeat(vis, h_q, axis=0)
        if spread is None:
            res = attend(qr, kv, kv[:, :d_latent], vis_r, sm_scale)
        else:
            res = attend(qr, kv, kv[:, :d_latent], vis_r, sm_scale, spread=True)
        out[tok] = res[0].reshape(len(qi), h_q, d_latent)
        lse[tok] = res[1].reshape(len(qi), h_q)
        if spread is not None:
            spread[tok] = res[2].reshape(len(qi), h_q, d_latent)
    return out, lse
