// Internal interface between the C ABI (capi.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Keys per KV tile, and packed query rows per work item of a four-wave
// workgroup (4 waves x 32 rows; the split-KV launches use four waves, other
// launches the count waves_per_item picks).
constexpr int kBN = 64;
constexpr int kBM = 128;

enum KvLayout { kContiguous = 0, kPaged = 1 };
enum MaskKind { kMaskCausal = 0, kMaskTree = 1 };  // kMaskCausal also covers "no mask"

// One kernel launch. All pointers are device pointers.
struct AttnParams {
  const uint16_t* q;
  const int32_t* q_indptr;
  void* out;
  float* lse;
  // contiguous KV
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_indptr;
  // paged KV
  const uint16_t* pages;
  const int32_t* page_indptr;
  const int32_t* page_values;
  const int32_t* length_info;
  const int32_t* k_rope_pos_offset;
  // tree mask (mn_indptr / tree_mask, or tree_order_indptr / tree_order)
  const int32_t* tree_indptr;
  const int32_t* tree_order;
  const int32_t* q_rope_position;
  int32_t batch, total_q, total_kv, tree_size;
  int32_t h_q, h_kv, group;
  int32_t num_pages, nnz_pages;
  int32_t sliding, causal;
  int32_t rope_q, rope_k;  // 0/1
  float rope_scale;
  float sm_scale_log2;     // sm_scale * log2(e)
  // padded batches (causal-or-none masks only): pad_mode 1 = right padding,
  // query row t and key j visible iff t < valid_len[b] and j < valid_len[b];
  // pad_mode 2 = left padding with causal alignment, queries
  // [qo_len - valid, qo_len) and keys [kv_len - valid, kv_len) are real
  const int32_t* valid_len;
  int32_t pad_mode;
  // split-KV: num_splits > 1 splits each item's KV tiles into num_splits
  // contiguous ranges; range s writes its normalised partial output (fp32)
  // and lse to part_out / part_lse at [s][row] instead of out / lse.
  int32_t num_splits;
  float* part_out;         // [num_splits, total_q * h_q, head_dim]
  float* part_lse;         // [num_splits, total_q * h_q]
  double inv_freq[64];     // RoPE: theta^(-2k/head_dim), k < head_dim / 2
};

// Merge of split-KV partial states into out (dtype) and lse.
struct MergeParams {
  const float* part_out;   // [num_splits, rows, head_dim]
  const float* part_lse;   // [num_splits, rows]
  void* out;               // [rows, head_dim] fp16/bf16
  float* lse;              // [rows]
  int32_t num_splits, rows;
};

struct AppendParams {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* append_indptr;
  const int32_t* append_start;
  const int32_t* rope_position;
  const int32_t* page_indptr;
  const int32_t* page_values;
  uint16_t* pages;
  int32_t batch, n_tokens, num_pages, nnz_pages, h_kv;
  float rope_scale;
  double inv_freq[64];     // RoPE: theta^(-2k/head_dim), k < head_dim / 2
};

// Multi-head latent attention prefill over a paged latent cache
// (mla_fwd.hip): one KV row of d_qk = 512 + 64 values per token, read as K
// over all of them and as V over the first 512.
struct MlaParams {
  const uint16_t* q;             // [total_q, h_q, 576]
  const int32_t* q_indptr;
  const uint16_t* pages;         // [num_pages, 16, 576]
  const int32_t* page_indptr;
  const int32_t* page_values;
  const int32_t* last_page_len;  // [batch]
  void* out;                     // [total_q, h_q, 512]
  float* lse;                    // [total_q, h_q]
  int32_t batch, total_q, h_q, num_pages, nnz_pages, causal;
  float sm_scale_log2;           // sm_scale * log2(e)
};

// Launchers (attn_fwd.hip / kv_append.hip). Return the hipError_t of the launch.
// Waves per workgroup (4 or 8) that launch_attn uses for p: the work item is
// 32 packed query rows per wave. set_waves_override(0 | 4 | 8) fixes it for
// every later launch without split-KV (0: chosen per launch).
int waves_per_item(const AttnParams& p);
void set_waves_override(int waves);
hipError_t launch_attn(const AttnParams& p, int is_bf16, int head_dim, KvLayout layout,
                       MaskKind mask, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, int is_bf16, int head_dim, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, int is_bf16, int head_dim, hipStream_t stream);
hipError_t launch_mla(const MlaParams& p, int is_bf16, hipStream_t stream);

}  // namespace ra
