// Checks of the C ABI layer (capi.cpp) on the CPU, built against the
// recording launchers of launch_stubs.cpp and run under host sanitizers
// (AddressSanitizer + UndefinedBehaviorSanitizer in one build,
// ThreadSanitizer in another). Device pointers are never dereferenced by the
// layer, so distinct fake addresses stand in for them and the checks read
// back what reached each launcher: the kernel chosen, the parameters, the
// split-KV workspace layout; plus every error path's status and message and
// the per-thread error text under concurrent calls.
//
// Prints "host checks: N passed, M failed" and exits non-zero on a failure.

#include <atomic>
#include <cinttypes>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "launch_stubs.h"
#include "ragattn.h"

namespace {

std::atomic<int> g_checks{0}, g_failed{0};

#define CHECK(cond)                                                              \
  do {                                                                           \
    g_checks.fetch_add(1, std::memory_order_relaxed);                           \
    if (!(cond)) {                                                               \
      g_failed.fetch_add(1, std::memory_order_relaxed);                         \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
    }                                                                            \
  } while (0)

// Distinct fake device addresses (256-byte aligned, never dereferenced).
template <typename T = void>
T* fake(uintptr_t n) { return reinterpret_cast<T*>(uintptr_t(0x7f0000000000) + n * 0x100000); }

bool err_has(const char* needle) { return std::strstr(ra_last_error(), needle) != nullptr; }
bool err_empty() { return ra_last_error()[0] == '\0'; }
bool close_rel(double a, double b, double rel) { return std::fabs(a - b) <= rel * std::fabs(b); }

const double kLog2e = 1.4426950408889634;

// ---- argument bundles, valid by default ----
struct Tree {
  const void* q = fake(1); const int32_t* q_indptr = fake<int32_t>(2); const void* k = fake(3);
  const void* v = fake(4); const int32_t* kv_indptr = fake<int32_t>(5); const int32_t* pos = fake<int32_t>(6);
  const int32_t* mn_indptr = fake<int32_t>(7); const int32_t* tree_mask = fake<int32_t>(8);
  void* out = fake(9); float* lse = fake<float>(10);
  int32_t batch = 16, total_q = 1024, total_kv = 1024, tree_size = 1024, h_q = 32, h_kv = 8, head_dim = 128;
  ra_dtype dtype = RA_F16; int32_t rotary_mode = 1;
  float rope_scale = 1.f, rope_theta = 1e4f, sm_scale = 0.08838835f;
  ra_status call() const {
    return ra_tree_attn(q, q_indptr, k, v, kv_indptr, pos, mn_indptr, tree_mask, out, lse, batch, total_q,
                        total_kv, tree_size, h_q, h_kv, head_dim, dtype, rotary_mode, rope_scale, rope_theta,
                        sm_scale, nullptr);
  }
};

enum PagedEntry { kPlain, kSplit, kNoAlloc };

struct Paged {
  const void* q = fake(11); const int32_t* q_indptr = fake<int32_t>(12); const void* pages = fake(13);
  const int32_t* page_indptr = fake<int32_t>(14); const int32_t* page_values = fake<int32_t>(15);
  const int32_t* length_info = fake<int32_t>(16); int32_t sliding = 0;
  const int32_t* k_rope_pos_offset = nullptr; const int32_t* q_rope_position = nullptr;
  const int32_t* tree_order_indptr = nullptr; const int32_t* tree_order = nullptr;
  int32_t causal = 1; void* out = fake(17); float* lse = fake<float>(18);
  int32_t batch = 8, total_q = 11414, num_pages = 30000, nnz_pages = 20000, tree_size = 0, page_size = 16;
  int32_t h_q = 64, h_kv = 8, head_dim = 128; ra_dtype dtype = RA_BF16; int32_t rotary_mode = 0;
  float rope_scale = 1.f, rope_theta = 1e4f, sm_scale = 0.08838835f;
  int32_t splits = 0; void* workspace = nullptr; size_t ws_bytes = 0;
  ra_status call(PagedEntry e = kPlain) const {
    if (e == kPlain)
      return ra_paged_attn(q, q_indptr, pages, page_indptr, page_values, length_info, sliding, k_rope_pos_offset,
                           q_rope_position, tree_order_indptr, tree_order, causal, out, lse, batch, total_q,
                           num_pages, nnz_pages, tree_size, page_size, h_q, h_kv, head_dim, dtype, rotary_mode,
                           rope_scale, rope_theta, sm_scale, nullptr);
    if (e == kSplit)
      return ra_paged_attn_split(q, q_indptr, pages, page_indptr, page_values, length_info, sliding,
                                 k_rope_pos_offset, q_rope_position, tree_order_indptr, tree_order, causal, out,
                                 lse, batch, total_q, num_pages, nnz_pages, tree_size, page_size, h_q, h_kv,
                                 head_dim, dtype, rotary_mode, rope_scale, rope_theta, sm_scale, splits,
                                 workspace, ws_bytes, nullptr);
    return ra_paged_attn_split_noalloc(q, q_indptr, pages, page_indptr, page_values, length_info, sliding,
                                       k_rope_pos_offset, q_rope_position, tree_order_indptr, tree_order, causal,
                                       out, lse, batch, total_q, num_pages, nnz_pages, tree_size, page_size, h_q,
                                       h_kv, head_dim, dtype, rotary_mode, rope_scale, rope_theta, sm_scale,
                                       splits, nullptr);
  }
};

// decode shape: 16 sequences of one query token over 1024 pages each
Paged decode_shape() {
  Paged a;
  a.batch = 16; a.total_q = 16; a.h_q = 32; a.h_kv = 8; a.nnz_pages = 16 * 1024; a.num_pages = 16 * 1024;
  return a;
}

struct Ragged {
  const void* q = fake(21); const int32_t* q_indptr = fake<int32_t>(22); const void* k = fake(23);
  const void* v = fake(24); const int32_t* kv_indptr = fake<int32_t>(25); const int32_t* valid_len = nullptr;
  int32_t pad_mode = 0, causal = 1; void* out = fake(26); float* lse = fake<float>(27);
  int32_t batch = 4, total_q = 300, total_kv = 500, h_q = 16, h_kv = 4, head_dim = 64;
  ra_dtype dtype = RA_F16; float sm_scale = 0.125f;
  ra_status call() const {
    return ra_ragged_prefill(q, q_indptr, k, v, kv_indptr, valid_len, pad_mode, causal, out, lse, batch, total_q,
                             total_kv, h_q, h_kv, head_dim, dtype, sm_scale, nullptr);
  }
};

struct Mla {
  const void* q = fake(31); const int32_t* q_indptr = fake<int32_t>(32); const void* pages = fake(33);
  const int32_t* page_indptr = fake<int32_t>(34); const int32_t* page_values = fake<int32_t>(35);
  const int32_t* last_page_len = fake<int32_t>(36); int32_t causal = 1; void* out = fake(37);
  float* lse = fake<float>(38);
  int32_t batch = 4, total_q = 2048, num_pages = 600, nnz_pages = 512, page_size = 16, h_q = 16, d_qk = 576,
          d_latent = 512;
  ra_dtype dtype = RA_BF16; float sm_scale = 0.0416667f;
  ra_status call() const {
    return ra_mla_paged_prefill(q, q_indptr, pages, page_indptr, page_values, last_page_len, causal, out, lse,
                                batch, total_q, num_pages, nnz_pages, page_size, h_q, d_qk, d_latent, dtype,
                                sm_scale, nullptr);
  }
};

struct Merge {
  const float* part_out = fake<float>(41); const float* part_lse = fake<float>(42);
  int32_t num_splits = 4, rows = 512, head_dim = 128; ra_dtype dtype = RA_F16;
  void* out = fake(43); float* lse = fake<float>(44);
  ra_status call() const {
    return ra_merge_states(part_out, part_lse, num_splits, rows, head_dim, dtype, out, lse, nullptr);
  }
};

struct Append {
  const void* k = fake(51); const void* v = fake(52); const int32_t* append_indptr = fake<int32_t>(53);
  const int32_t* append_start = fake<int32_t>(54); const int32_t* rope_position = fake<int32_t>(55);
  const int32_t* page_indptr = fake<int32_t>(56); const int32_t* page_values = fake<int32_t>(57);
  void* pages = fake(58);
  int32_t batch = 4, n_tokens = 100, num_pages = 64, nnz_pages = 40, page_size = 16, h_kv = 8, head_dim = 128;
  ra_dtype dtype = RA_BF16; float rope_scale = 1.f, rope_theta = 5e5f;
  ra_status call() const {
    return ra_paged_kv_append(k, v, append_indptr, append_start, rope_position, page_indptr, page_values, pages,
                              batch, n_tokens, num_pages, nnz_pages, page_size, h_kv, head_dim, dtype, rope_scale,
                              rope_theta, nullptr);
  }
};

// inv_freq[k] = theta^(-2k/d) for k < d/2, zero beyond: checked through
// values that follow from the definition (k = 0 gives 1, k = d/4 gives
// theta^(-1/2), a constant ratio theta^(-2/d) between neighbours).
void check_inv_freq(const double* f, double theta, int d) {
  CHECK(f[0] == 1.0);
  CHECK(close_rel(f[d / 4], 1.0 / std::sqrt(theta), 1e-14));
  const double ratio = std::exp(-2.0 / d * std::log(theta));
  bool ok = true;
  for (int k = 0; k + 1 < d / 2; ++k) ok = ok && close_rel(f[k + 1] / f[k], ratio, 1e-12);
  CHECK(ok);
  bool zero = true;
  for (int k = d / 2; k < 64; ++k) zero = zero && f[k] == 0.0;
  CHECK(zero);
}

void check_zero_freq(const double* f) {
  bool zero = true;
  for (int k = 0; k < 64; ++k) zero = zero && f[k] == 0.0;
  CHECK(zero);
}

// ---- ra_tree_attn ----
void tree_checks() {
  stub_reset();
  Tree a;
  CHECK(a.call() == RA_OK && err_empty());
  StubRecord r = stub_record();
  CHECK(r.attn_calls == 1 && r.merge_calls == 0);
  CHECK(r.attn_layout == ra::kContiguous && r.attn_mask == ra::kMaskTree);
  CHECK(r.attn_bf16 == 0 && r.attn_head_dim == 128);
  CHECK(r.attn.q == a.q && r.attn.k == a.k && r.attn.v == a.v && r.attn.out == a.out && r.attn.lse == a.lse);
  CHECK(r.attn.q_indptr == a.q_indptr && r.attn.kv_indptr == a.kv_indptr);
  CHECK(r.attn.tree_indptr == a.mn_indptr && r.attn.tree_order == a.tree_mask && r.attn.q_rope_position == a.pos);
  CHECK(r.attn.batch == 16 && r.attn.total_q == 1024 && r.attn.total_kv == 1024 && r.attn.tree_size == 1024);
  CHECK(r.attn.h_q == 32 && r.attn.h_kv == 8 && r.attn.group == 4 && r.attn.num_splits == 0);
  CHECK(r.attn.rope_q == 1 && r.attn.rope_k == 1 && r.attn.rope_scale == 1.f);
  CHECK(close_rel(r.attn.sm_scale_log2, a.sm_scale * kLog2e, 1e-7));
  check_inv_freq(r.attn.inv_freq, 1e4, 128);

  // head_dim 64, bf16, no rotation
  stub_reset();
  a.head_dim = 64; a.dtype = RA_BF16; a.rotary_mode = 0; a.pos = nullptr;
  CHECK(a.call() == RA_OK);
  r = stub_record();
  CHECK(r.attn_calls == 1 && r.attn_bf16 == 1 && r.attn_head_dim == 64 && r.attn.rope_q == 0 && r.attn.rope_k == 0);
  check_zero_freq(r.attn.inv_freq);
  a.rotary_mode = 1; a.pos = fake<int32_t>(6); a.rope_theta = 5e5f;
  stub_reset();
  CHECK(a.call() == RA_OK);
  r = stub_record();
  check_inv_freq(r.attn.inv_freq, 5e5, 64);

  // nothing to do: no launch, status OK, message cleared
  for (int which = 0; which < 2; ++which) {
    stub_reset();
    Tree e;
    Tree bad;
    bad.h_q = 3;
    (void)bad.call();   // leaves a message behind
    CHECK(!err_empty());
    if (which == 0) {
      e.batch = 0;
    } else {
      e.total_q = 0;
      e.total_kv = 0;   // K rows take the query rows' positions: none without queries
    }
    CHECK(e.call() == RA_OK && err_empty() && stub_record().attn_calls == 0);
  }

  // argument errors: status, a message, no launch
  struct Case { const char* what; Tree t; ra_status st; const char* msg; };
  std::vector<Case> cases;
  { Tree t; t.q_indptr = nullptr; cases.push_back({"q_indptr", t, RA_EINVAL, "q_indptr"}); }
  { Tree t; t.out = nullptr; cases.push_back({"out", t, RA_EINVAL, "non-NULL"}); }
  { Tree t; t.h_q = 30; cases.push_back({"h_q % h_kv", t, RA_EINVAL, "multiple"}); }
  { Tree t; t.h_kv = 0; cases.push_back({"h_kv", t, RA_EINVAL, "positive"}); }
  { Tree t; t.rotary_mode = 2; cases.push_back({"rotary_mode", t, RA_EINVAL, "got 2"}); }
  { Tree t; t.sm_scale = 0.f; cases.push_back({"sm_scale 0", t, RA_EINVAL, "sm_scale"}); }
  { Tree t; t.sm_scale = NAN; cases.push_back({"sm_scale nan", t, RA_EINVAL, "sm_scale"}); }
  { Tree t; t.rope_theta = -1.f; cases.push_back({"rope_theta", t, RA_EINVAL, "rope_theta"}); }
  { Tree t; t.rope_scale = INFINITY; cases.push_back({"rope_scale", t, RA_EINVAL, "rope_scale"}); }
  { Tree t; t.dtype = static_cast<ra_dtype>(7); cases.push_back({"dtype", t, RA_EUNSUPPORTED, "dtype 7"}); }
  { Tree t; t.head_dim = 96; cases.push_back({"head_dim", t, RA_EUNSUPPORTED, "head_dim 96"}); }
  { Tree t; t.total_kv = -1; cases.push_back({"total_kv", t, RA_EINVAL, "negative"}); }
  { Tree t; t.kv_indptr = nullptr; cases.push_back({"kv_indptr", t, RA_EINVAL, "kv_indptr"}); }
  { Tree t; t.k = nullptr; cases.push_back({"k", t, RA_EINVAL, "k and v"}); }
  { Tree t; t.tree_mask = nullptr; cases.push_back({"tree_mask", t, RA_EINVAL, "tree_mask"}); }
  { Tree t; t.pos = nullptr; cases.push_back({"positions", t, RA_EINVAL, "q_rope_position"}); }
  { Tree t; t.total_kv = 1025; cases.push_back({"total_kv > total_q", t, RA_EINVAL, "must not exceed"}); }
  { Tree t; t.total_q = 1 << 27; t.total_kv = 1024; cases.push_back({"rows", t, RA_EUNSUPPORTED, "2^31"}); }
  { Tree t; t.tree_size = 1 << 28; cases.push_back({"tree_size", t, RA_EUNSUPPORTED, "tree_size"}); }
  for (const Case& c : cases) {
    stub_reset();
    const ra_status st = c.t.call();
    const bool good = st == c.st && err_has(c.msg) && stub_record().attn_calls == 0;
    if (!good) std::fprintf(stderr, "  tree case '%s': status %d, message '%s'\n", c.what, st, ra_last_error());
    CHECK(good);
  }

  // a failed launch is reported with the HIP error text
  stub_reset();
  stub_set_status(hipErrorInvalidValue);
  CHECK(Tree{}.call() == RA_EHIP && err_has("kernel launch failed"));
  stub_reset();
}

// ---- ra_paged_attn and its split forms ----
void paged_checks() {
  stub_reset();
  Paged a;
  a.causal = 7;
  CHECK(a.call() == RA_OK && err_empty());
  StubRecord r = stub_record();
  CHECK(r.attn_calls == 1 && r.merge_calls == 0 && r.attn.num_splits == 0);
  CHECK(r.attn_layout == ra::kPaged && r.attn_mask == ra::kMaskCausal && r.attn_bf16 == 1);
  CHECK(r.attn.causal == 1 && r.attn.sliding == 0 && r.attn.tree_size == 0 && r.attn.group == 8);
  CHECK(r.attn.pages == a.pages && r.attn.page_indptr == a.page_indptr && r.attn.page_values == a.page_values);
  CHECK(r.attn.length_info == a.length_info && r.attn.num_pages == 30000 && r.attn.nnz_pages == 20000);
  CHECK(r.attn.rope_q == 0 && r.attn.rope_k == 0);
  check_zero_freq(r.attn.inv_freq);

  // a tree mask: the tree kernel, its size passed on; without one, size 0
  stub_reset();
  Paged t = a;
  t.tree_order_indptr = fake<int32_t>(19); t.tree_order = fake<int32_t>(20); t.tree_size = 777; t.causal = 0;
  CHECK(t.call() == RA_OK);
  r = stub_record();
  CHECK(r.attn_mask == ra::kMaskTree && r.attn.tree_size == 777 && r.attn.tree_order == t.tree_order);
  stub_reset();
  Paged nt = a;
  nt.tree_size = 5;
  CHECK(nt.call() == RA_OK && stub_record().attn.tree_size == 0);

  // RoPE: q always when rotary_mode 1, K only with k_rope_pos_offset
  stub_reset();
  Paged rq = a;
  rq.rotary_mode = 1; rq.q_rope_position = fake<int32_t>(21); rq.rope_scale = 0.5f;
  CHECK(rq.call() == RA_OK);
  r = stub_record();
  CHECK(r.attn.rope_q == 1 && r.attn.rope_k == 0 && r.attn.rope_scale == 0.5f);
  check_inv_freq(r.attn.inv_freq, 1e4, 128);
  stub_reset();
  rq.k_rope_pos_offset = fake<int32_t>(22);
  CHECK(rq.call() == RA_OK && stub_record().attn.rope_k == 1 && stub_record().attn.k_rope_pos_offset == rq.k_rope_pos_offset);

  // sliding window
  stub_reset();
  Paged sw = a;
  sw.sliding = 1;
  CHECK(sw.call() == RA_OK && stub_record().attn.sliding == 1);

  struct Case { const char* what; Paged p; ra_status st; const char* msg; };
  std::vector<Case> cases;
  { Paged p; p.page_size = 32; cases.push_back({"page_size", p, RA_EUNSUPPORTED, "page_size 32"}); }
  { Paged p; p.sliding = 2; cases.push_back({"sliding", p, RA_EINVAL, "sliding_window"}); }
  { Paged p; p.length_info = nullptr; cases.push_back({"length_info", p, RA_EINVAL, "length_info"}); }
  { Paged p; p.page_values = nullptr; cases.push_back({"page_values", p, RA_EINVAL, "page_values"}); }
  { Paged p; p.pages = nullptr; cases.push_back({"pages", p, RA_EINVAL, "pages is NULL"}); }
  { Paged p; p.tree_order = fake<int32_t>(20); cases.push_back({"tree without indptr", p, RA_EINVAL, "tree_order_indptr"}); }
  { Paged p; p.tree_order_indptr = fake<int32_t>(19); p.tree_size = 4; cases.push_back({"tree_order", p, RA_EINVAL, "tree_order is NULL"}); }
  { Paged p; p.tree_order_indptr = fake<int32_t>(19); p.sliding = 1; cases.push_back({"tree + window", p, RA_EUNSUPPORTED, "sliding window"}); }
  { Paged p; p.rotary_mode = 1; cases.push_back({"positions", p, RA_EINVAL, "q_rope_position"}); }
  { Paged p; p.num_pages = -1; cases.push_back({"num_pages", p, RA_EINVAL, "negative"}); }
  { Paged p; p.nnz_pages = 1 << 27; cases.push_back({"nnz_pages", p, RA_EUNSUPPORTED, "nnz_pages"}); }
  for (const Case& c : cases) {
    stub_reset();
    const ra_status st = c.p.call();
    const bool good = st == c.st && err_has(c.msg) && stub_record().attn_calls == 0;
    if (!good) std::fprintf(stderr, "  paged case '%s': status %d, message '%s'\n", c.what, st, ra_last_error());
    CHECK(good);
  }
}

void split_checks() {
  // workspace size: 0 without a split, partials (256-byte rounded) + lse
  const size_t rows = 16 * 32;
  CHECK(ra_paged_attn_split_workspace(16, 32, 128, 0) == 0);
  CHECK(ra_paged_attn_split_workspace(16, 32, 128, 1) == 0);
  CHECK(ra_paged_attn_split_workspace(0, 32, 128, 4) == 0);
  const size_t po4 = (4 * rows * 128 * 4 + 255) / 256 * 256;
  CHECK(ra_paged_attn_split_workspace(16, 32, 128, 4) == po4 + 4 * rows * 4);
  CHECK(ra_paged_attn_split_workspace(16, 32, 128, 2) < ra_paged_attn_split_workspace(16, 32, 128, 3));
  CHECK(ra_paged_attn_split_workspace(16, 32, 128, 100) == ra_paged_attn_split_workspace(16, 32, 128, 64));
  // the largest accepted problem (total_q * h_q = 2^31 - 32) does not wrap
  {
    const int32_t tq = (1 << 26) - 1, hq = 32;
    const unsigned __int128 r = static_cast<unsigned __int128>(tq) * hq;
    const unsigned __int128 po = (64 * r * 128 * 4 + 255) / 256 * 256;
    CHECK(static_cast<unsigned __int128>(ra_paged_attn_split_workspace(tq, hq, 128, 64)) == po + 64 * r * 4);
  }

  // explicit split count with an exact workspace: attention writes the
  // partials, the merge reads them back into the caller's out and lse
  stub_reset();
  Paged a = decode_shape();
  const size_t need = ra_paged_attn_split_workspace(a.total_q, a.h_q, a.head_dim, 4);
  char* ws = fake<char>(60);
  a.splits = 4; a.workspace = ws; a.ws_bytes = need;
  CHECK(a.call(kSplit) == RA_OK && err_empty());
  StubRecord r = stub_record();
  CHECK(r.attn_calls == 1 && r.merge_calls == 1 && r.attn.num_splits == 4);
  CHECK(reinterpret_cast<char*>(r.attn.part_out) == ws);
  const char* lse_at = reinterpret_cast<const char*>(r.attn.part_lse);
  CHECK(lse_at >= ws + 4 * rows * 128 * 4 && (reinterpret_cast<uintptr_t>(lse_at) & 255) == 0);
  CHECK(lse_at + 4 * rows * 4 <= ws + need);
  CHECK(r.merge.part_out == r.attn.part_out && r.merge.part_lse == r.attn.part_lse);
  CHECK(r.merge.out == a.out && r.merge.lse == a.lse && r.merge.num_splits == 4);
  CHECK(r.merge.rows == static_cast<int32_t>(rows) && r.merge_bf16 == 1 && r.merge_head_dim == 128);

  // one byte short: refused before any launch
  stub_reset();
  a.ws_bytes = need - 1;
  CHECK(a.call(kSplit) == RA_EINVAL && err_has("smaller than") && stub_record().attn_calls == 0);
  // no workspace for an explicit split
  stub_reset();
  a.ws_bytes = need; a.workspace = nullptr;
  CHECK(a.call(kSplit) == RA_EINVAL && err_has("workspace is NULL") && stub_record().attn_calls == 0);
  // split counts outside [0, 64]
  for (int s : {-1, 65}) {
    stub_reset();
    Paged b = decode_shape();
    b.splits = s; b.workspace = ws; b.ws_bytes = size_t(1) << 40;
    CHECK(b.call(kSplit) == RA_EINVAL && err_has("num_kv_splits") && stub_record().attn_calls == 0);
  }
  // split count 1: the plain kernel alone
  stub_reset();
  Paged one = decode_shape();
  one.splits = 1;
  CHECK(one.call(kSplit) == RA_OK && stub_record().attn_calls == 1 && stub_record().merge_calls == 0);

  // automatic count: more than one range on the decode shape, within
  // [2, 64] and the workspace given; none without a workspace
  stub_reset();
  Paged au = decode_shape();
  au.splits = 0; au.workspace = ws; au.ws_bytes = size_t(1) << 40;
  CHECK(au.call(kSplit) == RA_OK);
  r = stub_record();
  const int auto_s = r.attn.num_splits;
  CHECK(auto_s >= 2 && auto_s <= 64 && r.merge_calls == 1 && r.merge.num_splits == auto_s);
  stub_reset();
  au.ws_bytes = ra_paged_attn_split_workspace(au.total_q, au.h_q, au.head_dim, 3);
  CHECK(au.call(kSplit) == RA_OK);
  r = stub_record();
  CHECK(r.attn.num_splits == std::min(auto_s, 3) && r.merge_calls == (std::min(auto_s, 3) > 1 ? 1 : 0));
  stub_reset();
  au.ws_bytes = 0; au.workspace = nullptr;
  CHECK(au.call(kSplit) == RA_OK);
  r = stub_record();
  CHECK(r.attn_calls == 1 && r.merge_calls == 0 && r.attn.num_splits <= 1);
  // prefill-sized problem: enough work items already, so no split
  stub_reset();
  Paged big;
  big.splits = 0; big.workspace = ws; big.ws_bytes = size_t(1) << 40;
  CHECK(big.call(kSplit) == RA_OK && stub_record().merge_calls == 0);

  // the attention launch failing: no merge launched after it
  stub_reset();
  stub_set_status(hipErrorLaunchFailure);
  Paged f = decode_shape();
  f.splits = 4; f.workspace = ws; f.ws_bytes = need;
  CHECK(f.call(kSplit) == RA_EHIP && err_has("kernel launch failed"));
  r = stub_record();
  CHECK(r.attn_calls == 1 && r.merge_calls == 0);
  stub_reset();
}

void noalloc_checks() {
  // an explicit split count whose partial states exceed the library's
  // array is refused before anything else, with the array size named
  stub_reset();
  Paged a;
  a.total_q = 4096; a.splits = 64;
  CHECK(a.call(kNoAlloc) == RA_EINVAL && err_has("33554432") && stub_record().attn_calls == 0);
  // no split: no device lookup at all, one launch
  stub_reset();
  Paged one = decode_shape();
  one.splits = 1;
  CHECK(one.call(kNoAlloc) == RA_OK && stub_record().attn_calls == 1 && stub_record().merge_calls == 0);
  // a split needs the array's device address: on a host without a GPU the
  // lookup fails and nothing launches; with one, the split runs in it
  stub_reset();
  Paged s = decode_shape();
  s.splits = 4;
  const ra_status st = s.call(kNoAlloc);
  const StubRecord r = stub_record();
  if (st == RA_OK) {
    CHECK(r.attn_calls == 1 && r.merge_calls == 1 && r.attn.num_splits == 4 && r.attn.part_out != nullptr);
  } else {
    CHECK(st == RA_EHIP && !err_empty() && r.attn_calls == 0);
  }
  stub_reset();
}

// ---- ra_ragged_prefill ----
void ragged_checks() {
  stub_reset();
  Ragged a;
  CHECK(a.call() == RA_OK);
  StubRecord r = stub_record();
  CHECK(r.attn_calls == 1 && r.attn_layout == ra::kContiguous && r.attn_mask == ra::kMaskCausal);
  CHECK(r.attn.causal == 1 && r.attn.pad_mode == 0 && r.attn.group == 4 && r.attn_head_dim == 64);
  CHECK(r.attn.k == a.k && r.attn.v == a.v && r.attn.kv_indptr == a.kv_indptr && r.attn.total_kv == 500);
  CHECK(r.attn.rope_q == 0 && r.attn.rope_k == 0 && r.attn.tree_size == 0);
  CHECK(close_rel(r.attn.sm_scale_log2, 0.125 * kLog2e, 1e-7));
  // right padding (not causal) and left padding (causal) with their lengths
  stub_reset();
  Ragged rp = a;
  rp.pad_mode = 1; rp.causal = 0; rp.valid_len = fake<int32_t>(28);
  CHECK(rp.call() == RA_OK && stub_record().attn.pad_mode == 1 && stub_record().attn.valid_len == rp.valid_len);
  stub_reset();
  Ragged lp = a;
  lp.pad_mode = 2; lp.valid_len = fake<int32_t>(28);
  CHECK(lp.call() == RA_OK && stub_record().attn.pad_mode == 2 && stub_record().attn.causal == 1);

  struct Case { const char* what; Ragged g; ra_status st; const char* msg; };
  std::vector<Case> cases;
  { Ragged g; g.pad_mode = 3; cases.push_back({"pad_mode", g, RA_EINVAL, "pad_mode"}); }
  { Ragged g; g.pad_mode = 1; g.valid_len = fake<int32_t>(28); cases.push_back({"right + causal", g, RA_EINVAL, "not causal"}); }
  { Ragged g; g.pad_mode = 2; g.causal = 0; g.valid_len = fake<int32_t>(28); cases.push_back({"left, not causal", g, RA_EINVAL, "is causal"}); }
  { Ragged g; g.pad_mode = 2; cases.push_back({"valid_len", g, RA_EINVAL, "valid_len"}); }
  { Ragged g; g.total_kv = -5; cases.push_back({"total_kv", g, RA_EINVAL, "negative"}); }
  { Ragged g; g.v = nullptr; cases.push_back({"v", g, RA_EINVAL, "k and v"}); }
  { Ragged g; g.kv_indptr = nullptr; cases.push_back({"kv_indptr", g, RA_EINVAL, "kv_indptr"}); }
  { Ragged g; g.head_dim = 256; cases.push_back({"head_dim", g, RA_EUNSUPPORTED, "head_dim 256"}); }
  for (const Case& c : cases) {
    stub_reset();
    const ra_status st = c.g.call();
    const bool good = st == c.st && err_has(c.msg) && stub_record().attn_calls == 0;
    if (!good) std::fprintf(stderr, "  ragged case '%s': status %d, message '%s'\n", c.what, st, ra_last_error());
    CHECK(good);
  }
}

// ---- ra_mla_paged_prefill ----
void mla_checks() {
  stub_reset();
  Mla a;
  a.causal = 3;
  CHECK(a.call() == RA_OK);
  StubRecord r = stub_record();
  CHECK(r.mla_calls == 1 && r.attn_calls == 0 && r.mla_bf16 == 1);
  CHECK(r.mla.q == a.q && r.mla.pages == a.pages && r.mla.last_page_len == a.last_page_len && r.mla.out == a.out);
  CHECK(r.mla.batch == 4 && r.mla.total_q == 2048 && r.mla.h_q == 16 && r.mla.causal == 1);
  CHECK(r.mla.num_pages == 600 && r.mla.nnz_pages == 512);
  CHECK(close_rel(r.mla.sm_scale_log2, a.sm_scale * kLog2e, 1e-7));
  stub_reset();
  Mla e;
  e.total_q = 0;
  CHECK(e.call() == RA_OK && stub_record().mla_calls == 0);

  struct Case { const char* what; Mla m; ra_status st; const char* msg; };
  std::vector<Case> cases;
  { Mla m; m.d_latent = 256; cases.push_back({"d_latent", m, RA_EUNSUPPORTED, "latent widths"}); }
  { Mla m; m.d_qk = 512; cases.push_back({"d_qk", m, RA_EUNSUPPORTED, "latent widths"}); }
  { Mla m; m.page_size = 8; cases.push_back({"page_size", m, RA_EUNSUPPORTED, "page_size 8"}); }
  { Mla m; m.h_q = 0; cases.push_back({"h_q", m, RA_EINVAL, "h_q"}); }
  { Mla m; m.last_page_len = nullptr; cases.push_back({"last_page_len", m, RA_EINVAL, "last_page_len"}); }
  { Mla m; m.lse = nullptr; cases.push_back({"lse", m, RA_EINVAL, "non-NULL"}); }
  { Mla m; m.sm_scale = -1.f; cases.push_back({"sm_scale", m, RA_EINVAL, "sm_scale"}); }
  { Mla m; m.total_q = 1 << 27; cases.push_back({"rows", m, RA_EUNSUPPORTED, "2^31"}); }
  for (const Case& c : cases) {
    stub_reset();
    const ra_status st = c.m.call();
    const bool good = st == c.st && err_has(c.msg) && stub_record().mla_calls == 0;
    if (!good) std::fprintf(stderr, "  latent case '%s': status %d, message '%s'\n", c.what, st, ra_last_error());
    CHECK(good);
  }
}

// ---- ra_merge_states ----
void merge_checks() {
  stub_reset();
  Merge a;
  CHECK(a.call() == RA_OK);
  StubRecord r = stub_record();
  CHECK(r.merge_calls == 1 && r.merge.num_splits == 4 && r.merge.rows == 512 && r.merge_head_dim == 128);
  CHECK(r.merge.part_out == a.part_out && r.merge.part_lse == a.part_lse && r.merge.out == a.out && r.merge.lse == a.lse);
  stub_reset();
  Merge z;
  z.rows = 0; z.out = nullptr;
  CHECK(z.call() == RA_OK && stub_record().merge_calls == 0);
  Merge s1;
  s1.num_splits = 1;
  stub_reset();
  CHECK(s1.call() == RA_OK && stub_record().merge.num_splits == 1);
  for (int bad : {0, 65}) {
    Merge m;
    m.num_splits = bad;
    stub_reset();
    CHECK(m.call() == RA_EINVAL && err_has("num_splits") && stub_record().merge_calls == 0);
  }
  Merge np;
  np.part_lse = nullptr;
  stub_reset();
  CHECK(np.call() == RA_EINVAL && stub_record().merge_calls == 0);
  Merge hd;
  hd.head_dim = 32;
  stub_reset();
  CHECK(hd.call() == RA_EUNSUPPORTED && stub_record().merge_calls == 0);
}

// ---- ra_paged_kv_append ----
void append_checks() {
  stub_reset();
  Append a;
  CHECK(a.call() == RA_OK);
  StubRecord r = stub_record();
  CHECK(r.append_calls == 1 && r.append_bf16 == 1 && r.append_head_dim == 128);
  CHECK(r.append.k == a.k && r.append.pages == a.pages && r.append.append_start == a.append_start);
  CHECK(r.append.batch == 4 && r.append.n_tokens == 100 && r.append.h_kv == 8 && r.append.nnz_pages == 40);
  check_inv_freq(r.append.inv_freq, 5e5, 128);
  // without positions nothing rotates and the RoPE scalars are not read
  stub_reset();
  Append nr = a;
  nr.rope_position = nullptr; nr.rope_theta = NAN;
  CHECK(nr.call() == RA_OK);
  check_zero_freq(stub_record().append.inv_freq);

  struct Case { const char* what; Append p; ra_status st; };
  std::vector<Case> cases;
  { Append p; p.rope_theta = NAN; cases.push_back({"rope_theta", p, RA_EINVAL}); }
  { Append p; p.batch = 0; cases.push_back({"tokens without sequences", p, RA_EINVAL}); }
  { Append p; p.page_values = nullptr; cases.push_back({"page_values", p, RA_EINVAL}); }
  { Append p; p.append_start = nullptr; cases.push_back({"append_start", p, RA_EINVAL}); }
  { Append p; p.page_size = 64; cases.push_back({"page_size", p, RA_EUNSUPPORTED}); }
  { Append p; p.h_kv = -2; cases.push_back({"h_kv", p, RA_EINVAL}); }
  { Append p; p.n_tokens = -1; cases.push_back({"n_tokens", p, RA_EINVAL}); }
  { Append p; p.n_tokens = (1 << 30) + 1; cases.push_back({"n_tokens limit", p, RA_EUNSUPPORTED}); }
  { Append p; p.h_kv = (1 << 16) + 1; cases.push_back({"h_kv limit", p, RA_EUNSUPPORTED}); }
  for (const Case& c : cases) {
    stub_reset();
    const ra_status st = c.p.call();
    const bool good = st == c.st && !err_empty() && stub_record().append_calls == 0;
    if (!good) std::fprintf(stderr, "  append case '%s': status %d, message '%s'\n", c.what, st, ra_last_error());
    CHECK(good);
  }
  stub_reset();
  Append none = a;
  none.n_tokens = 0; none.k = nullptr;
  CHECK(none.call() == RA_OK && stub_record().append_calls == 0);
}

// ---- workgroup shape override, and message length ----
void misc_checks() {
  stub_reset();
  CHECK(ra_set_workgroup_waves(3) == RA_EINVAL && err_has("got 3"));
  CHECK(ra_set_workgroup_waves(8) == RA_OK && stub_record().waves_override == 8);
  CHECK(ra_attn_workgroup_waves(1024, 32, 8, 0) == 8);
  CHECK(ra_set_workgroup_waves(0) == RA_OK && stub_record().waves_override == 0);
  CHECK(ra_attn_workgroup_waves(-1, 32, 8, 0) == 0);
  CHECK(ra_attn_workgroup_waves(16, 30, 8, 0) == 0);
  CHECK(ra_attn_workgroup_waves(16, 32, 8, 4) == 4);
  // the longest messages (two sizes and a count) fit the error buffer
  Paged a = decode_shape();
  a.total_q = (1 << 26) - 1; a.h_q = 32; a.h_kv = 32; a.splits = 64; a.workspace = fake(60); a.ws_bytes = 1;
  CHECK(a.call(kSplit) == RA_EINVAL);
  const size_t n = std::strlen(ra_last_error());
  CHECK(n > 0 && n < 512 && err_has("smaller than"));
  stub_reset();
}

// ---- the error text is per thread ----
// Threads interleave failing calls, each with a value of its own in the
// message, and successful ones (which clear it), and check after every call
// that they see their own text.
void thread_checks() {
  constexpr int kThreads = 8, kIters = 2000;
  std::atomic<int> mismatches{0};
  std::vector<std::thread> pool;
  for (int t = 0; t < kThreads; ++t) {
    pool.emplace_back([t, &mismatches] {
      const std::string mine = "got " + std::to_string(100 + t);
      for (int i = 0; i < kIters; ++i) {
        if (i % 2 == 0) {
          Tree bad;
          bad.rotary_mode = 100 + t;
          if (bad.call() != RA_EINVAL || std::strstr(ra_last_error(), mine.c_str()) == nullptr) ++mismatches;
        } else {
          Merge good;
          good.rows = 64 + t;
          if (good.call() != RA_OK || ra_last_error()[0] != '\0') ++mismatches;
        }
      }
    });
  }
  for (std::thread& th : pool) th.join();
  CHECK(mismatches.load() == 0);
  CHECK(stub_record().merge_calls == kThreads * kIters / 2);
}

}  // namespace

int main(int argc, char** argv) {
  const bool threads_only = argc > 1 && std::strcmp(argv[1], "threads") == 0;
  if (!threads_only) {
    tree_checks();
    paged_checks();
    split_checks();
    noalloc_checks();
    ragged_checks();
    mla_checks();
    merge_checks();
    append_checks();
    misc_checks();
  }
  stub_reset();
  thread_checks();
  std::printf("host checks: %d passed, %d failed\n", g_checks.load() - g_failed.load(), g_failed.load());
  return g_failed.load() == 0 ? 0 : 1;
}
