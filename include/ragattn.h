/*
 * ragattn: ragged, batched, masked grouped-query attention for MI355X (gfx950).
 *
 * C ABI of libragattn.so. Every entry point launches asynchronously on the
 * caller's HIP stream, never synchronises, allocates no device memory and
 * keeps no state between calls (apart from the process-wide workgroup shape
 * that ra_set_workgroup_waves may fix, and the per-GPU scratch array of
 * ra_paged_attn_split_noalloc). Pointers are caller-owned device memory
 * unless stated otherwise; inputs are read-only. Index arrays are int32.
 *
 * Operation defined by the TVM pages (cited by page and section):
 *   page "relax/frontend/nn/llm/_kernel_common.py": _rope, _causal_mask,
 *     _get_kv_chunk_len, _get_seq_offset and the prefill macros
 *     (compute_s_gemm, softmax_update_causal, compute_o_gemm,
 *     paged_store_output_lse);
 *   page "relax/frontend/nn/llm/tree_attn.py": _check_tree_order, the
 *     tree_attn operator (contiguous KV) and tree_attn_with_paged_kv_cache.
 *
 * For every query token i of sequence b and query head h (KV head
 * h / (h_q / h_kv)) over the visible KV columns j of that sequence:
 *   s_j = sm_scale * sum_t q[i,h,t] * k[j,kvh,t]
 *   out[i,h,:] = sum_j softmax(s)_j * v[j,kvh,:]          (stored in dtype)
 *   lse[i,h]   = log2(sum_j exp(s_j))                      (float32, base 2)
 * A row with no visible column gets out = 0 and lse = -inf.
 *
 * Layouts (row-major):
 *   q, out     [total_q, h_q, head_dim]    fp16 or bf16
 *   lse        [total_q, h_q]              float32
 *   k, v       [total_kv, h_kv, head_dim]  (contiguous KV)
 *   pages      [num_pages, 2, h_kv, page_size, head_dim], slot 0 = K, 1 = V
 *   tree masks [n, 2] rows of (enter, exit): DFS pre-order index and
 *              pre-order index + subtree size of each tree node.
 *
 * Size limits of the attention entry points (RA_EUNSUPPORTED beyond them):
 * total_q * h_q < 2^31, total_q < 2^29, tree_size < 2^28, nnz_pages < 2^27.
 *
 * Index arrays must be consistent with the sizes passed (indptr arrays
 * non-decreasing, entries inside their arrays). The kernels bound every
 * access they derive from them by the sizes given: a row, page or tree entry
 * outside its array is read as zero / not visible rather than dereferenced.
 */
#ifndef RAGATTN_H
#define RAGATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_EINVAL = -1,        /* bad argument: null pointer, negative size, h_q % h_kv != 0, ... */
  RA_EUNSUPPORTED = -2,  /* valid but not built: head_dim, dtype, page_size, combination */
  RA_EHIP = -3           /* a HIP launch error (message from hipGetErrorString) */
} ra_status;

/* Storage type of q, k, v, out and the caches. A caller may pass any 32-bit
 * value: others are rejected with RA_EUNSUPPORTED. In C++ the enum has a fixed
 * int32_t underlying type, so every such value is a valid ra_dtype there too
 * (without one, values outside 0..1 would be out of the enum's range). */
#ifdef __cplusplus
typedef enum : int32_t { RA_F16 = 0, RA_BF16 = 1 } ra_dtype;
#else
typedef enum { RA_F16 = 0, RA_BF16 = 1 } ra_dtype;
#endif

/*
 * Batched tree attention over contiguous KV ("tree_attn.py" page: tree_attn,
 * the batch_tree_attn kernel and _check_tree_order).
 *
 * Sequence b owns query rows [q_indptr[b], q_indptr[b+1]) and KV rows
 * [kv_indptr[b], kv_indptr[b+1]); its tree occupies mask rows
 * [mn_indptr[b], mn_indptr[b+1]) and its nodes are the last
 * tree_len = mn_indptr[b+1] - mn_indptr[b] KV columns. Column j is visible to
 * query row i iff j < kv_len and (j < kv_len - tree_len, or with
 * c = i + tree_len - qo_len and p = j - (kv_len - tree_len):
 * tree_mask[c].enter in [tree_mask[p].enter, tree_mask[p].exit)).
 *
 * rotary_mode: 0 = no rotation; 1 = rotate-half RoPE inside the kernel, q row
 *   r at position q_rope_position[r] and K row r at q_rope_position[r] (the
 *   page's kernels index K positions with the same array; KV rows and query
 *   rows coincide in this operator). Angles: float32(pos * rope_scale) *
 *   rope_theta^(-2k/head_dim) for dims k and k + head_dim/2 (the product in
 *   float64); cos and sin are their float32 values (rounded once from a
 *   float64 evaluation), and a rotated value is the float32 sum of two
 *   float32 products, cos*x -/+ sin*partner (no fused multiply-add),
 *   rounded to dtype (to nearest, ties to even).
 * q_rope_position may be NULL when rotary_mode == 0.
 * tree_size = mn_indptr[batch] (rows of tree_mask); total_kv = kv_indptr[batch].
 * Supported: head_dim 64 or 128, dtype fp16/bf16, any h_q divisible by h_kv.
 */
ra_status ra_tree_attn(const void* q, const int32_t* q_indptr, const void* k, const void* v,
                       const int32_t* kv_indptr, const int32_t* q_rope_position,
                       const int32_t* mn_indptr, const int32_t* tree_mask, void* out, float* lse,
                       int32_t batch, int32_t total_q, int32_t total_kv, int32_t tree_size,
                       int32_t h_q, int32_t h_kv, int32_t head_dim, ra_dtype dtype,
                       int32_t rotary_mode, float rope_scale, float rope_theta, float sm_scale,
                       hipStream_t stream);

/*
 * Ragged prefill or tree attention over a paged KV cache (the paged_prefill_attn
 * operation). Page gather and lengths follow "_kernel_common.py" page,
 * _get_kv_chunk_len / _get_seq_offset, and the paged tree kernel on the
 * "tree_attn.py" page:
 *   sequence b owns pages page_values[page_indptr[b] .. page_indptr[b+1]);
 *   with np pages its KV chunk holds
 *     kv_len = (np-1)*page_size + last_page_len                (no window)
 *     kv_len = (np-1)*page_size + last_page_len - offset + sink (window)
 *   (kv_len = 0 when np == 0); chunk position j lives at storage offset
 *   o = j, or o = (j < sink ? j : j - sink + offset) with the window, i.e.
 *   in page page_values[page_indptr[b] + o / page_size], slot o % page_size.
 * length_info: [batch] last_page_len when sliding_window == 0, else
 *   [3, batch] rows (last_page_len, window offset, sink size).
 * Mask: when tree_order is given, the tree test of ra_tree_attn with the tree
 *   being the last tree_order_indptr[b+1] - tree_order_indptr[b] chunk
 *   columns (everything before it is a fully visible prefix); otherwise
 *   _causal_mask: causal != 0 -> j < kv_len - qo_len + i + 1, else j < kv_len.
 * rotary_mode: 0 = none; 1 = q row r rotated at q_rope_position[r], and K at
 *   chunk position j rotated at k_rope_pos_offset[b] + j when
 *   k_rope_pos_offset is non-NULL (when it is NULL, K is used as stored:
 *   the cache's K was rotated before caching, see ra_paged_kv_append).
 * nnz_pages = page_indptr[batch]; tree_size = tree_order_indptr[batch] (0 when
 *   no tree). page_size must be 16. A sliding window combined with a tree
 *   mask is RA_EUNSUPPORTED (the page's paged tree kernel disables it).
 */
ra_status ra_paged_attn(const void* q, const int32_t* q_indptr, const void* pages,
                        const int32_t* page_indptr, const int32_t* page_values,
                        const int32_t* length_info, int32_t sliding_window,
                        const int32_t* k_rope_pos_offset, const int32_t* q_rope_position,
                        const int32_t* tree_order_indptr, const int32_t* tree_order,
                        int32_t causal, void* out, float* lse, int32_t batch, int32_t total_q,
                        int32_t num_pages, int32_t nnz_pages, int32_t tree_size,
                        int32_t page_size, int32_t h_q, int32_t h_kv, int32_t head_dim,
                        ra_dtype dtype, int32_t rotary_mode, float rope_scale, float rope_theta,
                        float sm_scale, hipStream_t stream);

/*
 * Ragged prefill over contiguous K/V, optionally with padded batches.
 * Sequence b's queries are q rows [q_indptr[b], q_indptr[b+1]) and its keys
 * k/v rows [kv_indptr[b], kv_indptr[b+1]) (layouts as ra_tree_attn); query
 * row t of the sequence sees key j under:
 *   pad_mode 0: causal ? j < kv_len - qo_len + t + 1 : all keys
 *               (_causal_mask on the "_kernel_common.py" page);
 *   pad_mode 1: right padding (causal must be 0): t < valid_len[b] and
 *               j < valid_len[b] (softmax_update_valid_length, same page);
 *   pad_mode 2: left padding, causal (causal must be 1): the real queries are
 *               [qo_len - valid, qo_len), the real keys [kv_len - valid,
 *               kv_len), and j < kv_len - qo_len + t + 1
 *               (softmax_update_causal_padded_left, same page).
 * valid_len: [batch] int32 device array (NULL when pad_mode is 0); values are
 * clamped to [0, qo_len] / [0, kv_len]. Rows with no visible key (padding
 * rows) get out = 0, lse = -inf. No RoPE (rotate before calling).
 * Errors: RA_EINVAL (NULL pointers, pad_mode not 0..2, pad_mode 1 with causal,
 * pad_mode 2 without causal, sizes, sm_scale), RA_EUNSUPPORTED (head_dim,
 * dtype), RA_EHIP (launch).
 */
ra_status ra_ragged_prefill(const void* q, const int32_t* q_indptr, const void* k, const void* v,
                            const int32_t* kv_indptr, const int32_t* valid_len, int32_t pad_mode,
                            int32_t causal, void* out, float* lse, int32_t batch,
                            int32_t total_q, int32_t total_kv, int32_t h_q, int32_t h_kv,
                            int32_t head_dim, ra_dtype dtype, float sm_scale, hipStream_t stream);

/*
 * Split-KV form of ra_paged_attn, for few query rows over long KV (decode).
 * Same arguments and result as ra_paged_attn, plus:
 *   num_kv_splits   1..64: each work item's KV tiles are cut into this many
 *                   contiguous ranges, processed by separate workgroups;
 *                   0: chosen by the library (about four work items per
 *                   compute unit, at least two 64-key tiles per range on the
 *                   mean sequence, limited by the workspace); 1: no split.
 *   workspace       caller-owned device memory for the partial states,
 *                   at least ra_paged_attn_split_workspace(...) bytes for the
 *                   split count used (may be NULL when that is 0).
 * Each range writes its normalised output (fp32) and base-2 lse; a second
 * kernel merges them (see ra_merge_states). The merge is the online-softmax
 * update of the "_kernel_common.py" page applied to whole ranges; the base-2
 * lse that the page's epilogue stores is what makes the ranges combinable.
 * Errors as ra_paged_attn, and RA_EINVAL for num_kv_splits outside [0, 64]
 * or a workspace smaller than the explicit split count needs. Both kernels
 * run on `stream`; the workspace must stay valid until they finish. With
 * more than one split every row of out/lse is written by the merge, so
 * q_indptr[batch] must equal total_q (rows outside every sequence would get
 * unspecified values).
 */
ra_status ra_paged_attn_split(const void* q, const int32_t* q_indptr, const void* pages,
                              const int32_t* page_indptr, const int32_t* page_values,
                              const int32_t* length_info, int32_t sliding_window,
                              const int32_t* k_rope_pos_offset, const int32_t* q_rope_position,
                              const int32_t* tree_order_indptr, const int32_t* tree_order,
                              int32_t causal, void* out, float* lse, int32_t batch,
                              int32_t total_q, int32_t num_pages, int32_t nnz_pages,
                              int32_t tree_size, int32_t page_size, int32_t h_q, int32_t h_kv,
                              int32_t head_dim, ra_dtype dtype, int32_t rotary_mode,
                              float rope_scale, float rope_theta, float sm_scale,
                              int32_t num_kv_splits, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * ra_paged_attn_split without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments and result as
 * ra_paged_attn_split minus the workspace: the partial states go to a
 * 32 MiB (33554432-byte) array of device memory that the library holds, one
 * copy per GPU, from the first call on that GPU until the process ends. The
 * call allocates nothing. num_kv_splits 0 picks the split count as
 * ra_paged_attn_split does, limited to what fits the array (falling back to
 * the unsplit kernel); an explicit count whose partial states need more
 * than 32 MiB (see ra_paged_attn_split_workspace) returns RA_EINVAL. Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (different streams, or host threads) race and give wrong results;
 * calls ordered on one stream are safe. Errors as ra_paged_attn_split, and
 * RA_EHIP when the array's device address cannot be obtained.
 */
ra_status ra_paged_attn_split_noalloc(const void* q, const int32_t* q_indptr, const void* pages,
                                      const int32_t* page_indptr, const int32_t* page_values,
                                      const int32_t* length_info, int32_t sliding_window,
                                      const int32_t* k_rope_pos_offset,
                                      const int32_t* q_rope_position,
                                      const int32_t* tree_order_indptr, const int32_t* tree_order,
                                      int32_t causal, void* out, float* lse, int32_t batch,
                                      int32_t total_q, int32_t num_pages, int32_t nnz_pages,
                                      int32_t tree_size, int32_t page_size, int32_t h_q,
                                      int32_t h_kv, int32_t head_dim, ra_dtype dtype,
                                      int32_t rotary_mode, float rope_scale, float rope_theta,
                                      float sm_scale, int32_t num_kv_splits, hipStream_t stream);

/* Bytes of workspace ra_paged_attn_split needs for num_kv_splits ranges
 * (0 when num_kv_splits <= 1): num_kv_splits * total_q * h_q * (head_dim + 1)
 * floats, the output part rounded up to 256 bytes. */
size_t ra_paged_attn_split_workspace(int32_t total_q, int32_t h_q, int32_t head_dim,
                                     int32_t num_kv_splits);

/*
 * Merge partial attention states over disjoint KV ranges:
 *   part_out [num_splits, rows, head_dim] fp32, each row normalised over its
 *   range; part_lse [num_splits, rows] fp32 base-2 lse of the range (-inf for
 *   a range with no visible key).
 * Writes lse[r] = log2 sum_s 2^part_lse[s][r] and
 * out[r] = sum_s 2^(part_lse[s][r] - lse[r]) * part_out[s][r] in `dtype`
 * (rows with no visible key anywhere: out 0, lse -inf). rows = tokens * heads
 * of a [tokens, heads, head_dim] output. Errors: RA_EINVAL (num_splits not in
 * [1, 64], negative rows, NULL pointers), RA_EUNSUPPORTED (head_dim, dtype).
 */
ra_status ra_merge_states(const float* part_out, const float* part_lse, int32_t num_splits,
                          int32_t rows, int32_t head_dim, ra_dtype dtype, void* out, float* lse,
                          hipStream_t stream);

/*
 * Multi-head latent attention prefill over a paged latent cache
 * ("_kernel_common.py" page: AttnKind MLA; _alloc_mla_qkvo_buffers, whose
 * single KV tile of d_qk columns serves as K over all of them and as V over
 * the first d_latent; paged_store_output_lse with every query head in one
 * group; _causal_mask).
 *
 * Every token of a sequence has one cached row of d_qk values shared by all
 * h_q query heads (a compressed latent vector of d_latent values followed by
 * its rotary part). For query token i of sequence b and head h:
 *   s_j = sm_scale * sum_{t < d_qk} q[i,h,t] * kv_j[t]
 *   out[i,h,:] = sum_j softmax(s)_j * kv_j[0 : d_latent]     (stored in dtype)
 *   lse[i,h]   = log2(sum_j exp(s_j))                        (float32)
 * over the keys j < kv_len - qo_len + i + 1 (causal != 0) or j < kv_len.
 * Layouts (row-major): q [total_q, h_q, d_qk]; out [total_q, h_q, d_latent];
 * lse [total_q, h_q]; pages [num_pages, page_size, d_qk]. Sequence b owns
 * pages page_values[page_indptr[b] .. page_indptr[b+1]); with np pages its
 * chunk holds kv_len = (np-1)*page_size + last_page_len[b] rows (0 when
 * np == 0), row o in page page_values[page_indptr[b] + o / page_size], slot
 * o % page_size. Any RoPE on q and on the cached rotary part is applied by
 * the caller. A row with no visible key gets out = 0 and lse = -inf.
 * Supported: d_qk = 576 and d_latent = 512 (RA_EUNSUPPORTED otherwise),
 * page_size 16, fp16/bf16, any h_q. nnz_pages = page_indptr[batch].
 * Errors: RA_EINVAL (NULL pointers, negative sizes, sm_scale), RA_EUNSUPPORTED,
 * RA_EHIP (launch).
 */
ra_status ra_mla_paged_prefill(const void* q, const int32_t* q_indptr, const void* pages,
                               const int32_t* page_indptr, const int32_t* page_values,
                               const int32_t* last_page_len, int32_t causal, void* out, float* lse,
                               int32_t batch, int32_t total_q, int32_t num_pages,
                               int32_t nnz_pages, int32_t page_size, int32_t h_q, int32_t d_qk,
                               int32_t d_latent, ra_dtype dtype, float sm_scale,
                               hipStream_t stream);

/*
 * Append new K/V tokens into the paged cache, rotating K first when
 * rope_position is non-NULL (the "normal" RoPE mode of the KV cache on the
 * "_kernel_common.py" page, RopeMode: RoPE applied to k before adding it to
 * the cache).
 *
 * k, v [n_tokens, h_kv, head_dim]; tokens [append_indptr[b], append_indptr[b+1])
 * belong to sequence b and go to storage offsets append_start[b] + 0, 1, ...
 * i.e. page page_values[page_indptr[b] + o / page_size], slot o % page_size,
 * of pages [num_pages, 2, h_kv, page_size, head_dim]. K is rotated at
 * rope_position[token] with the angles of ra_tree_attn. A token whose page
 * index falls outside page_values or the pool is skipped.
 * Errors: RA_EINVAL (negative sizes, tokens without sequences, NULL
 * pointers, non-finite rope_theta/rope_scale with rotation), RA_EUNSUPPORTED
 * (head_dim not 64/128, dtype, page size not 16, n_tokens > 2^30 or
 * h_kv > 2^16), RA_EHIP (launch error).
 */
ra_status ra_paged_kv_append(const void* k, const void* v, const int32_t* append_indptr,
                             const int32_t* append_start, const int32_t* rope_position,
                             const int32_t* page_indptr, const int32_t* page_values, void* pages,
                             int32_t batch, int32_t n_tokens, int32_t num_pages,
                             int32_t nnz_pages, int32_t page_size, int32_t h_kv,
                             int32_t head_dim, ra_dtype dtype, float rope_scale,
                             float rope_theta, hipStream_t stream);

/*
 * Workgroup shape of the attention kernels (a tuning override; results do not
 * depend on it beyond rounding order, which it leaves unchanged): waves = 4
 * or 8 fixes 4 or 8 waves of 64 per workgroup, i.e. 128 or 256 packed query
 * rows (token, head of the group) per work item, for every later
 * ra_tree_attn, ra_paged_attn and ra_ragged_prefill launch in the process;
 * waves = 0 (the default) lets each launch choose: 8 when its 256-row work
 * items cover the current device's compute units (256 on a whole MI355X)
 * at least twice, else 4. Eight
 * waves share each K/V tile between twice the rows (half the K/V loads per
 * row) at one workgroup per compute unit. Split-KV launches always use 4.
 * Errors: RA_EINVAL for any other value (the setting is then unchanged).
 */
ra_status ra_set_workgroup_waves(int32_t waves);

/*
 * Waves per workgroup (4 or 8) that an attention launch of these sizes uses
 * under the current ra_set_workgroup_waves setting; num_kv_splits is the
 * launch's split count (0 or 1: not split). Returns 0 for sizes the entry
 * points reject (total_q < 0, h_q or h_kv not positive, h_q not a multiple
 * of h_kv). Launches nothing.
 */
int32_t ra_attn_workgroup_waves(int32_t total_q, int32_t h_q, int32_t h_kv, int32_t num_kv_splits);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RAGATTN_H */
