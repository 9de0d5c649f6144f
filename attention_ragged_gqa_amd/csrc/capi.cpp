// C ABI of libragattn.so: argument validation, error reporting and dispatch.
// Nothing here touches device memory; every call launches at most one kernel
// on the caller's stream and returns without synchronising.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "ra_internal.h"
#include "../../include/ragattn.h"

namespace {

thread_local char g_err[512] = "";

ra_status fail(ra_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ra_status ok() {
  g_err[0] = '\0';
  return RA_OK;
}

ra_status check_common(const void* q, const void* q_indptr, const void* out, const void* lse,
                       int32_t batch, int32_t total_q, int32_t h_q, int32_t h_kv,
                       int32_t head_dim, ra_dtype dtype, int32_t rotary_mode, float sm_scale) {
  if (batch < 0 || total_q < 0) return fail(RA_EINVAL, "negative batch (%d) or total_q (%d)", batch, total_q);
  if (batch > 0 && q_indptr == nullptr) return fail(RA_EINVAL, "q_indptr is NULL");
  if (total_q > 0 && (q == nullptr || out == nullptr || lse == nullptr))
    return fail(RA_EINVAL, "q, out and lse must be non-NULL");
  if (h_q <= 0 || h_kv <= 0) return fail(RA_EINVAL, "h_q (%d) and h_kv (%d) must be positive", h_q, h_kv);
  if (h_q % h_kv != 0) return fail(RA_EINVAL, "h_q (%d) is not a multiple of h_kv (%d)", h_q, h_kv);
  if (rotary_mode != 0 && rotary_mode != 1) return fail(RA_EINVAL, "rotary_mode must be 0 or 1, got %d", rotary_mode);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(RA_EINVAL, "sm_scale must be finite and > 0");
  if (dtype != RA_F16 && dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "dtype %d not supported (fp16=0, bf16=1)", (int)dtype);
  if (head_dim != 64 && head_dim != 128) return fail(RA_EUNSUPPORTED, "head_dim %d not supported (64, 128)", head_dim);
  return RA_OK;
}

// Size limits of the attention kernels: (token, head) row indices are 32-bit,
// and the index arrays read through bounds-checked buffer loads address at
// most 2^31 - 1 bytes (positions and page numbers 4 bytes each, tree entries
// 8); a sequence's chunk length, up to 16 * its page count, is 32-bit too.
ra_status check_limits(int32_t total_q, int32_t h_q, int32_t tree_size, int32_t nnz_pages) {
  if (static_cast<int64_t>(total_q) * h_q > INT32_MAX)
    return fail(RA_EUNSUPPORTED, "total_q * h_q = %lld exceeds 2^31 - 1",
                static_cast<long long>(total_q) * h_q);
  if (total_q >= (1 << 29)) return fail(RA_EUNSUPPORTED, "total_q %d exceeds 2^29 - 1", total_q);
  if (tree_size >= (1 << 28)) return fail(RA_EUNSUPPORTED, "tree_size %d exceeds 2^28 - 1", tree_size);
  if (nnz_pages >= (1 << 27)) return fail(RA_EUNSUPPORTED, "nnz_pages %d exceeds 2^27 - 1", nnz_pages);
  return RA_OK;
}

ra_status check_rope(int32_t rotary_mode, float rope_scale, float rope_theta) {
  if (rotary_mode == 1 && (!(rope_theta > 0.f) || !std::isfinite(rope_theta) || !std::isfinite(rope_scale)))
    return fail(RA_EINVAL, "rope_theta must be finite and > 0, rope_scale finite");
  return RA_OK;
}

// RoPE frequencies theta^(-2k/head_dim), k < head_dim / 2, in float64 (the
// rotate-half convention of the "_kernel_common.py" page, _rope).
void fill_inv_freq(double* inv_freq, bool rope, float theta, int32_t head_dim) {
  for (int k = 0; k < 64; ++k)
    inv_freq[k] = (rope && 2 * k < head_dim)
                      ? std::pow(static_cast<double>(theta), -2.0 * k / static_cast<double>(head_dim))
                      : 0.0;
}

ra_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(RA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* ra_last_error(void) { return g_err; }

ra_status ra_set_workgroup_waves(int32_t waves) {
  if (waves != 0 && waves != 4 && waves != 8)
    return fail(RA_EINVAL, "waves must be 0 (per launch), 4 or 8, got %d", waves);
  ra::set_waves_override(waves);
  return ok();
}

int32_t ra_attn_workgroup_waves(int32_t total_q, int32_t h_q, int32_t h_kv, int32_t num_kv_splits) {
  if (total_q < 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0) return 0;
  ra::AttnParams p{};
  p.total_q = total_q;
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.group = h_q / h_kv;
  p.num_splits = num_kv_splits > 1 ? num_kv_splits : 0;
  return ra::waves_per_item(p);
}

ra_status ra_tree_attn(const void* q, const int32_t* q_indptr, const void* k, const void* v,
                       const int32_t* kv_indptr, const int32_t* q_rope_position,
                       const int32_t* mn_indptr, const int32_t* tree_mask, void* out, float* lse,
                       int32_t batch, int32_t total_q, int32_t total_kv, int32_t tree_size,
                       int32_t h_q, int32_t h_kv, int32_t head_dim, ra_dtype dtype,
                       int32_t rotary_mode, float rope_scale, float rope_theta, float sm_scale,
                       hipStream_t stream) {
  ra_status st = check_common(q, q_indptr, out, lse, batch, total_q, h_q, h_kv, head_dim, dtype,
                              rotary_mode, sm_scale);
  if (st != RA_OK) return st;
  if ((st = check_rope(rotary_mode, rope_scale, rope_theta)) != RA_OK) return st;
  if (total_kv < 0 || tree_size < 0) return fail(RA_EINVAL, "negative total_kv or tree_size");
  if ((st = check_limits(total_q, h_q, tree_size, 0)) != RA_OK) return st;
  if (batch > 0 && (kv_indptr == nullptr || mn_indptr == nullptr))
    return fail(RA_EINVAL, "kv_indptr and mn_indptr must be non-NULL");
  if (total_kv > 0 && (k == nullptr || v == nullptr)) return fail(RA_EINVAL, "k and v must be non-NULL");
  if (tree_size > 0 && tree_mask == nullptr) return fail(RA_EINVAL, "tree_mask is NULL");
  if (rotary_mode == 1 && (total_q > 0 || total_kv > 0) && q_rope_position == nullptr)
    return fail(RA_EINVAL, "rotary_mode 1 needs q_rope_position");
  if (rotary_mode == 1 && total_kv > total_q)
    return fail(RA_EINVAL, "rotary_mode 1 rotates K row r at q_rope_position[r]: total_kv (%d) must not exceed total_q (%d)",
                total_kv, total_q);
  if (batch == 0 || total_q == 0) return ok();

  ra::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_indptr = q_indptr;
  p.out = out;
  p.lse = lse;
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.kv_indptr = kv_indptr;
  p.tree_indptr = mn_indptr;
  p.tree_order = tree_mask;
  p.q_rope_position = q_rope_position;
  p.batch = batch;
  p.total_q = total_q;
  p.total_kv = total_kv;
  p.tree_size = tree_size;
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.group = h_q / h_kv;
  p.rope_q = rotary_mode == 1;
  p.rope_k = rotary_mode == 1;
  p.rope_scale = rope_scale;
  fill_inv_freq(p.inv_freq, rotary_mode == 1, rope_theta, head_dim);
  p.sm_scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  return launched(ra::launch_attn(p, dtype == RA_BF16, head_dim, ra::kContiguous, ra::kMaskTree, stream));
}

}  // extern "C"

namespace {

// ---- split-KV ------------------------------------------------------------
constexpr int32_t kMaxSplits = 64;

size_t part_out_bytes(size_t rows, int32_t head_dim, int32_t splits) {
  const size_t b = static_cast<size_t>(splits) * rows * head_dim * sizeof(float);
  return (b + 255) / 256 * 256;
}

size_t split_workspace_bytes(int32_t total_q, int32_t h_q, int32_t head_dim, int32_t splits) {
  if (splits <= 1 || total_q <= 0 || h_q <= 0) return 0;
  const size_t rows = static_cast<size_t>(total_q) * h_q;
  return part_out_bytes(rows, head_dim, splits) + static_cast<size_t>(splits) * rows * sizeof(float);
}

// Splits so that about four workgroups per CU (1024) have work, with at
// least two 64-key tiles per split on the average sequence (KV lengths are
// on the device; the page count gives their mean).
int32_t auto_splits(int32_t batch, int32_t total_q, int32_t group, int32_t h_kv, int32_t nnz_pages) {
  const long items = std::max<long>((static_cast<long>(total_q) * group + ra::kBM - 1) / ra::kBM,
                                    batch) * h_kv;
  const long tiles = static_cast<long>(nnz_pages) * 16 / std::max(batch, 1) / ra::kBN;
  long s = (1024 + items - 1) / std::max(items, 1L);
  s = std::min(s, tiles / 2);
  return static_cast<int32_t>(std::max(1L, std::min<long>(s, kMaxSplits)));
}

}  // namespace

static ra_status paged_attn_impl(const void* q, const int32_t* q_indptr, const void* pages,
                        const int32_t* page_indptr, const int32_t* page_values,
                        const int32_t* length_info, int32_t sliding_window,
                        const int32_t* k_rope_pos_offset, const int32_t* q_rope_position,
                        const int32_t* tree_order_indptr, const int32_t* tree_order,
                        int32_t causal, void* out, float* lse, int32_t batch, int32_t total_q,
                        int32_t num_pages, int32_t nnz_pages, int32_t tree_size,
                        int32_t page_size, int32_t h_q, int32_t h_kv, int32_t head_dim,
                        ra_dtype dtype, int32_t rotary_mode, float rope_scale, float rope_theta,
                        float sm_scale, int32_t num_kv_splits, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  ra_status st = check_common(q, q_indptr, out, lse, batch, total_q, h_q, h_kv, head_dim, dtype,
                              rotary_mode, sm_scale);
  if (st != RA_OK) return st;
  if ((st = check_rope(rotary_mode, rope_scale, rope_theta)) != RA_OK) return st;
  if (page_size != 16) return fail(RA_EUNSUPPORTED, "page_size %d not supported (16)", page_size);
  if (num_pages < 0 || nnz_pages < 0 || tree_size < 0) return fail(RA_EINVAL, "negative num_pages, nnz_pages or tree_size");
  if ((st = check_limits(total_q, h_q, tree_size, nnz_pages)) != RA_OK) return st;
  if (sliding_window != 0 && sliding_window != 1) return fail(RA_EINVAL, "sliding_window must be 0 or 1");
  if (batch > 0 && (page_indptr == nullptr || length_info == nullptr))
    return fail(RA_EINVAL, "page_indptr and length_info must be non-NULL");
  if (nnz_pages > 0 && page_values == nullptr) return fail(RA_EINVAL, "page_values is NULL");
  if (num_pages > 0 && pages == nullptr) return fail(RA_EINVAL, "pages is NULL");
  const bool tree = tree_order != nullptr || tree_order_indptr != nullptr;
  if (tree && tree_order_indptr == nullptr) return fail(RA_EINVAL, "tree_order given without tree_order_indptr");
  if (tree && tree_size > 0 && tree_order == nullptr) return fail(RA_EINVAL, "tree_order is NULL");
  if (tree && sliding_window) return fail(RA_EUNSUPPORTED, "sliding window with a tree mask is not supported");
  if (rotary_mode == 1 && total_q > 0 && q_rope_position == nullptr)
    return fail(RA_EINVAL, "rotary_mode 1 needs q_rope_position");
  if (batch == 0 || total_q == 0) return ok();

  ra::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_indptr = q_indptr;
  p.out = out;
  p.lse = lse;
  p.pages = static_cast<const uint16_t*>(pages);
  p.page_indptr = page_indptr;
  p.page_values = page_values;
  p.length_info = length_info;
  p.k_rope_pos_offset = k_rope_pos_offset;
  p.tree_indptr = tree_order_indptr;
  p.tree_order = tree_order;
  p.q_rope_position = q_rope_position;
  p.batch = batch;
  p.total_q = total_q;
  p.tree_size = tree ? tree_size : 0;
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.group = h_q / h_kv;
  p.num_pages = num_pages;
  p.nnz_pages = nnz_pages;
  p.sliding = sliding_window;
  p.causal = causal != 0;
  p.rope_q = rotary_mode == 1;
  p.rope_k = rotary_mode == 1 && k_rope_pos_offset != nullptr;
  p.rope_scale = rope_scale;
  fill_inv_freq(p.inv_freq, rotary_mode == 1, rope_theta, head_dim);
  p.sm_scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  const ra::MaskKind mask = tree ? ra::kMaskTree : ra::kMaskCausal;
  int32_t splits = num_kv_splits;
  if (splits < 0 || splits > kMaxSplits) return fail(RA_EINVAL, "num_kv_splits must be in [0, %d]", kMaxSplits);
  if (splits == 0) {
    splits = auto_splits(batch, total_q, p.group, h_kv, nnz_pages);
    while (splits > 1 && split_workspace_bytes(total_q, h_q, head_dim, splits) > workspace_bytes) --splits;
  } else if (splits > 1 && split_workspace_bytes(total_q, h_q, head_dim, splits) > workspace_bytes) {
    return fail(RA_EINVAL, "workspace of %zu bytes is smaller than the %zu needed for %d splits",
                workspace_bytes, split_workspace_bytes(total_q, h_q, head_dim, splits), splits);
  }
  if (splits > 1 && workspace == nullptr) return fail(RA_EINVAL, "workspace is NULL");
  if (splits <= 1) return launched(ra::launch_attn(p, dtype == RA_BF16, head_dim, ra::kPaged, mask, stream));
  const size_t rows = static_cast<size_t>(total_q) * h_q;
  p.num_splits = splits;
  p.part_out = static_cast<float*>(workspace);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + part_out_bytes(rows, head_dim, splits));
  hipError_t e = ra::launch_attn(p, dtype == RA_BF16, head_dim, ra::kPaged, mask, stream);
  if (e != hipSuccess) return launched(e);
  ra::MergeParams mp{};
  mp.part_out = p.part_out;
  mp.part_lse = p.part_lse;
  mp.out = out;
  mp.lse = lse;
  mp.num_splits = splits;
  mp.rows = static_cast<int32_t>(rows);
  return launched(ra::launch_merge(mp, dtype == RA_BF16, head_dim, stream));
}


extern "C" {

ra_status ra_paged_attn(const void* q, const int32_t* q_indptr, const void* pages,
                        const int32_t* page_indptr, const int32_t* page_values,
                        const int32_t* length_info, int32_t sliding_window,
                        const int32_t* k_rope_pos_offset, const int32_t* q_rope_position,
                        const int32_t* tree_order_indptr, const int32_t* tree_order,
                        int32_t causal, void* out, float* lse, int32_t batch, int32_t total_q,
                        int32_t num_pages, int32_t nnz_pages, int32_t tree_size,
                        int32_t page_size, int32_t h_q, int32_t h_kv, int32_t head_dim,
                        ra_dtype dtype, int32_t rotary_mode, float rope_scale, float rope_theta,
                        float sm_scale, hipStream_t stream) {
  return paged_attn_impl(q, q_indptr, pages, page_indptr, page_values, length_info,
                         sliding_window, k_rope_pos_offset, q_rope_position, tree_order_indptr,
                         tree_order, causal, out, lse, batch, total_q, num_pages, nnz_pages,
                         tree_size, page_size, h_q, h_kv, head_dim, dtype, rotary_mode,
                         rope_scale, rope_theta, sm_scale, 1, nullptr, 0, stream);
}

ra_status ra_ragged_prefill(const void* q, const int32_t* q_indptr, const void* k, const void* v,
                            const int32_t* kv_indptr, const int32_t* valid_len, int32_t pad_mode,
                            int32_t causal, void* out, float* lse, int32_t batch,
                            int32_t total_q, int32_t total_kv, int32_t h_q, int32_t h_kv,
                            int32_t head_dim, ra_dtype dtype, float sm_scale,
                            hipStream_t stream) {
  ra_status st = check_common(q, q_indptr, out, lse, batch, total_q, h_q, h_kv, head_dim, dtype, 0,
                              sm_scale);
  if (st != RA_OK) return st;
  if (total_kv < 0) return fail(RA_EINVAL, "negative total_kv");
  if ((st = check_limits(total_q, h_q, 0, 0)) != RA_OK) return st;
  if (batch > 0 && kv_indptr == nullptr) return fail(RA_EINVAL, "kv_indptr is NULL");
  if (total_kv > 0 && (k == nullptr || v == nullptr)) return fail(RA_EINVAL, "k and v must be non-NULL");
  if (pad_mode < 0 || pad_mode > 2) return fail(RA_EINVAL, "pad_mode must be 0, 1 or 2, got %d", pad_mode);
  if (pad_mode != 0 && batch > 0 && valid_len == nullptr) return fail(RA_EINVAL, "valid_len is NULL");
  if (pad_mode == 1 && causal != 0) return fail(RA_EINVAL, "pad_mode 1 (right padding) is not causal");
  if (pad_mode == 2 && causal == 0) return fail(RA_EINVAL, "pad_mode 2 (left padding) is causal");
  if (batch == 0 || total_q == 0) return ok();
  ra::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_indptr = q_indptr;
  p.out = out;
  p.lse = lse;
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.kv_indptr = kv_indptr;
  p.batch = batch;
  p.total_q = total_q;
  p.total_kv = total_kv;
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.group = h_q / h_kv;
  p.causal = causal != 0;
  p.valid_len = valid_len;
  p.pad_mode = pad_mode;
  p.sm_scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  return launched(ra::launch_attn(p, dtype == RA_BF16, head_dim, ra::kContiguous, ra::kMaskCausal,
                                  stream));
}

size_t ra_paged_attn_split_workspace(int32_t total_q, int32_t h_q, int32_t head_dim,
                                     int32_t num_kv_splits) {
  return split_workspace_bytes(total_q, h_q, head_dim, std::min(num_kv_splits, kMaxSplits));
}

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
                              hipStream_t stream) {
  return paged_attn_impl(q, q_indptr, pages, page_indptr, page_values, length_info,
                         sliding_window, k_rope_pos_offset, q_rope_position, tree_order_indptr,
                         tree_order, causal, out, lse, batch, total_q, num_pages, nnz_pages,
                         tree_size, page_size, h_q, h_kv, head_dim, dtype, rotary_mode,
                         rope_scale, rope_theta, sm_scale, num_kv_splits, workspace,
                         workspace_bytes, stream);
}

}  // extern "C"

// ---- split-KV without a caller workspace ---------------------------------
// The partial states live in a file-scope device array, one copy per GPU,
// held until the process ends. `scratch` names the host-side shadow of that
// array: host code never passes it to a kernel, it passes the device address
// hipGetSymbolAddress returns for the GPU the launch runs on (kept per
// device below). Nothing in it has to start at zero: every (split, row)
// partial the merge reads is written by the attention kernel of the same
// call first.
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of this GPU's scratch array, looked up once per device with
// that device current. dev: the device the caller's stream belongs to.
ra_status scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return fail(RA_EHIP, "hipGetDevice failed");
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    const hipError_t e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return fail(RA_EHIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    dev = static_cast<int>(d);
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(RA_EUNSUPPORTED, "device %d beyond %d", dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return fail(RA_EHIP, "hipSetDevice(%d) failed", dev);
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
      return fail(RA_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
}

}  // namespace

extern "C" {

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
                                      float sm_scale, int32_t num_kv_splits, hipStream_t stream) {
  // explicit split counts whose partial states exceed the array are refused
  // before anything else (the automatic count is chosen to fit)
  if (num_kv_splits > 1 && num_kv_splits <= kMaxSplits &&
      split_workspace_bytes(total_q, h_q, head_dim, num_kv_splits) > kScratchBytes)
    return fail(RA_EINVAL, "%d splits need %zu bytes of partial states, beyond the %zu-byte scratch array",
                num_kv_splits, split_workspace_bytes(total_q, h_q, head_dim, num_kv_splits), kScratchBytes);
  void* ws = nullptr;
  if (num_kv_splits != 1 && total_q > 0 && batch > 0) {
    const ra_status st = scratch_address(stream, &ws);
    if (st != RA_OK) return st;
  }
  return paged_attn_impl(q, q_indptr, pages, page_indptr, page_values, length_info,
                         sliding_window, k_rope_pos_offset, q_rope_position, tree_order_indptr,
                         tree_order, causal, out, lse, batch, total_q, num_pages, nnz_pages,
                         tree_size, page_size, h_q, h_kv, head_dim, dtype, rotary_mode,
                         rope_scale, rope_theta, sm_scale, num_kv_splits, ws,
                         ws != nullptr ? kScratchBytes : 0, stream);
}

ra_status ra_mla_paged_prefill(const void* q, const int32_t* q_indptr, const void* pages,
                               const int32_t* page_indptr, const int32_t* page_values,
                               const int32_t* last_page_len, int32_t causal, void* out, float* lse,
                               int32_t batch, int32_t total_q, int32_t num_pages,
                               int32_t nnz_pages, int32_t page_size, int32_t h_q, int32_t d_qk,
                               int32_t d_latent, ra_dtype dtype, float sm_scale,
                               hipStream_t stream) {
  if (batch < 0 || total_q < 0 || num_pages < 0 || nnz_pages < 0)
    return fail(RA_EINVAL, "negative batch, total_q, num_pages or nnz_pages");
  if (h_q <= 0) return fail(RA_EINVAL, "h_q must be positive, got %d", h_q);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(RA_EINVAL, "sm_scale must be finite and > 0");
  if (dtype != RA_F16 && dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "dtype %d not supported (fp16=0, bf16=1)", (int)dtype);
  if (d_latent != 512 || d_qk != 576)
    return fail(RA_EUNSUPPORTED, "latent widths (d_qk %d, d_latent %d) not supported (576, 512)", d_qk, d_latent);
  if (page_size != 16) return fail(RA_EUNSUPPORTED, "page_size %d not supported (16)", page_size);
  ra_status st = check_limits(total_q, h_q, 0, nnz_pages);
  if (st != RA_OK) return st;
  if (batch > 0 && (q_indptr == nullptr || page_indptr == nullptr || last_page_len == nullptr))
    return fail(RA_EINVAL, "q_indptr, page_indptr and last_page_len must be non-NULL");
  if (total_q > 0 && (q == nullptr || out == nullptr || lse == nullptr))
    return fail(RA_EINVAL, "q, out and lse must be non-NULL");
  if (nnz_pages > 0 && page_values == nullptr) return fail(RA_EINVAL, "page_values is NULL");
  if (num_pages > 0 && pages == nullptr) return fail(RA_EINVAL, "pages is NULL");
  if (batch == 0 || total_q == 0) return ok();
  ra::MlaParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_indptr = q_indptr;
  p.pages = static_cast<const uint16_t*>(pages);
  p.page_indptr = page_indptr;
  p.page_values = page_values;
  p.last_page_len = last_page_len;
  p.out = out;
  p.lse = lse;
  p.batch = batch;
  p.total_q = total_q;
  p.h_q = h_q;
  p.num_pages = num_pages;
  p.nnz_pages = nnz_pages;
  p.causal = causal != 0;
  p.sm_scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  return launched(ra::launch_mla(p, dtype == RA_BF16, stream));
}

ra_status ra_merge_states(const float* part_out, const float* part_lse, int32_t num_splits,
                          int32_t rows, int32_t head_dim, ra_dtype dtype, void* out, float* lse,
                          hipStream_t stream) {
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(RA_EINVAL, "num_splits must be in [1, %d]", kMaxSplits);
  if (rows < 0) return fail(RA_EINVAL, "negative rows");
  if (dtype != RA_F16 && dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "dtype %d not supported", (int)dtype);
  if (head_dim != 64 && head_dim != 128) return fail(RA_EUNSUPPORTED, "head_dim %d not supported (64, 128)", head_dim);
  if (rows == 0) return ok();
  if (part_out == nullptr || part_lse == nullptr || out == nullptr || lse == nullptr)
    return fail(RA_EINVAL, "a required pointer is NULL");
  ra::MergeParams mp{};
  mp.part_out = part_out;
  mp.part_lse = part_lse;
  mp.out = out;
  mp.lse = lse;
  mp.num_splits = num_splits;
  mp.rows = rows;
  return launched(ra::launch_merge(mp, dtype == RA_BF16, head_dim, stream));
}

ra_status ra_paged_kv_append(const void* k, const void* v, const int32_t* append_indptr,
                             const int32_t* append_start, const int32_t* rope_position,
                             const int32_t* page_indptr, const int32_t* page_values, void* pages,
                             int32_t batch, int32_t n_tokens, int32_t num_pages,
                             int32_t nnz_pages, int32_t page_size, int32_t h_kv,
                             int32_t head_dim, ra_dtype dtype, float rope_scale,
                             float rope_theta, hipStream_t stream) {
  if (batch < 0 || n_tokens < 0 || num_pages < 0 || nnz_pages < 0)
    return fail(RA_EINVAL, "negative size argument");
  if (n_tokens > 0 && batch == 0) return fail(RA_EINVAL, "n_tokens > 0 needs batch > 0");
  if (h_kv <= 0) return fail(RA_EINVAL, "h_kv must be positive");
  if (dtype != RA_F16 && dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "dtype %d not supported", (int)dtype);
  if (head_dim != 64 && head_dim != 128) return fail(RA_EUNSUPPORTED, "head_dim %d not supported (64, 128)", head_dim);
  if (page_size != 16) return fail(RA_EUNSUPPORTED, "page_size %d not supported (16)", page_size);
  // the kernel's token and chunk indices are 32-bit
  if (n_tokens > (1 << 30) || h_kv > (1 << 16))
    return fail(RA_EUNSUPPORTED, "n_tokens %d or h_kv %d past the kernel's limits (2^30, 2^16)", n_tokens, h_kv);
  if (n_tokens == 0) return ok();
  if (k == nullptr || v == nullptr || append_indptr == nullptr || append_start == nullptr ||
      page_indptr == nullptr || pages == nullptr || (nnz_pages > 0 && page_values == nullptr))
    return fail(RA_EINVAL, "a required pointer is NULL");
  if (rope_position != nullptr && (!(rope_theta > 0.f) || !std::isfinite(rope_theta) || !std::isfinite(rope_scale)))
    return fail(RA_EINVAL, "rope_theta must be finite and > 0, rope_scale finite");

  ra::AppendParams p{};
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.append_indptr = append_indptr;
  p.append_start = append_start;
  p.rope_position = rope_position;
  p.page_indptr = page_indptr;
  p.page_values = page_values;
  p.pages = static_cast<uint16_t*>(pages);
  p.batch = batch;
  p.n_tokens = n_tokens;
  p.num_pages = num_pages;
  p.nnz_pages = nnz_pages;
  p.h_kv = h_kv;
  p.rope_scale = rope_scale;
  fill_inv_freq(p.inv_freq, rope_position != nullptr, rope_theta, head_dim);
  return launched(ra::launch_append(p, dtype == RA_BF16, head_dim, stream));
}

}  // extern "C"
