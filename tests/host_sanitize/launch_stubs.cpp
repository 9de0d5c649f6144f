// Recording stand-ins for the launchers of attn_fwd.hip, merge.hip,
// mla_fwd.hip and kv_append.hip (see launch_stubs.h). No device code and no
// HIP calls: the C ABI layer built against these runs on the CPU alone.

#include "launch_stubs.h"

#include <mutex>

namespace {
std::mutex g_mu;
StubRecord g_rec;
hipError_t g_status = hipSuccess;
}  // namespace

void stub_reset() {
  std::lock_guard<std::mutex> lock(g_mu);
  g_rec = StubRecord{};
  g_status = hipSuccess;
}

void stub_set_status(hipError_t e) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_status = e;
}

StubRecord stub_record() {
  std::lock_guard<std::mutex> lock(g_mu);
  return g_rec;
}

namespace ra {

// The real policy reads the device's compute-unit count; here a fixed shape
// (the override when set) is enough for the layer above.
int waves_per_item(const AttnParams& p) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (p.num_splits > 1) return 4;
  return g_rec.waves_override != 0 ? g_rec.waves_override : 4;
}

void set_waves_override(int waves) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_rec.waves_override = waves;
}

hipError_t launch_attn(const AttnParams& p, int is_bf16, int head_dim, KvLayout layout, MaskKind mask,
                       hipStream_t) {
  std::lock_guard<std::mutex> lock(g_mu);
  ++g_rec.attn_calls;
  g_rec.attn = p;
  g_rec.attn_bf16 = is_bf16;
  g_rec.attn_head_dim = head_dim;
  g_rec.attn_layout = layout;
  g_rec.attn_mask = mask;
  return g_status;
}

hipError_t launch_merge(const MergeParams& p, int is_bf16, int head_dim, hipStream_t) {
  std::lock_guard<std::mutex> lock(g_mu);
  ++g_rec.merge_calls;
  g_rec.merge = p;
  g_rec.merge_bf16 = is_bf16;
  g_rec.merge_head_dim = head_dim;
  return g_status;
}

hipError_t launch_mla(const MlaParams& p, int is_bf16, hipStream_t) {
  std::lock_guard<std::mutex> lock(g_mu);
  ++g_rec.mla_calls;
  g_rec.mla = p;
  g_rec.mla_bf16 = is_bf16;
  return g_status;
}

hipError_t launch_append(const AppendParams& p, int is_bf16, int head_dim, hipStream_t) {
  std::lock_guard<std::mutex> lock(g_mu);
  ++g_rec.append_calls;
  g_rec.append = p;
  g_rec.append_bf16 = is_bf16;
  g_rec.append_head_dim = head_dim;
  return g_status;
}

}  // namespace ra
