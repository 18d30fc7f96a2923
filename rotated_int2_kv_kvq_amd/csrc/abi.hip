// extern "C" entry points of libkvq: host-side validation, workspace sizing and
// kernel launches.  No allocation, no synchronisation, no global state.
#include <stdint.h>

#include <mutex>

#include "kvq.h"
#include "kvq_common.h"

#include "kvq_launch.h"

#define KVQ_API extern "C" __attribute__((visibility("default")))

namespace {
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool valid_geometry(int32_t head_dim, int32_t group) {
  return head_dim > 0 && (group == 64 || group == 128) && head_dim % group == 0;
}
}  // namespace

KVQ_API const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration (head_dim must be 128)";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP runtime error at launch";
    case KVQ_ERR_SCRATCH:
      return "decode needs more than the library's static scratch (KVQ_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

KVQ_API size_t kvq_page_bytes(int32_t head_dim, int32_t group) {
  if (head_dim != kvq::kHeadDim || !valid_geometry(head_dim, group)) return 0;
  return static_cast<size_t>(kvq::page_bytes_for_groups(head_dim / group));
}

namespace {
// Host-side checks of kvq_append's arguments (num_new tokens); KVQ_OK when the
// call may proceed (batch or num_new zero included).
int check_append(const void* pages, int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                 int32_t group, const int32_t* block_table, int32_t max_blocks_per_seq,
                 const int32_t* start_pos, int32_t batch, int32_t num_new, const void* k,
                 const void* v, int32_t kv_dtype, const float* mu, const float* rot_k,
                 const float* rot_v, float clip_k, float clip_v) {
  if (!valid_geometry(head_dim, group)) return KVQ_ERR_INVALID_ARG;
  if (head_dim != kvq::kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (batch < 0 || num_new < 0 || num_kv_heads < 1 || num_blocks < 1 || max_blocks_per_seq < 1)
    return KVQ_ERR_INVALID_ARG;
  if (num_kv_heads > 65535 || batch > 65535) return KVQ_ERR_INVALID_ARG;
  if (kv_dtype != KVQ_F32 && kv_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if (!(clip_k > 0.f && clip_k <= 1.f) || !(clip_v > 0.f && clip_v <= 1.f))
    return KVQ_ERR_INVALID_ARG;
  if (batch == 0 || num_new == 0) return KVQ_OK;
  // rot_v may be null: the value rotation is folded into the caller's weights;
  // rot_k may be null: keys are centred but not rotated
  if (!pages || !block_table || !start_pos || !k || !v || !mu) return KVQ_ERR_INVALID_ARG;
  if (!aligned(pages, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(mu, 16) ||
      (rot_k && !aligned(rot_k, 16)) || (rot_v && !aligned(rot_v, 16)))
    return KVQ_ERR_INVALID_ARG;
  if (!aligned(block_table, 4) || !aligned(start_pos, 4)) return KVQ_ERR_INVALID_ARG;
  return KVQ_OK;
}
}  // namespace

KVQ_API int kvq_append(void* pages, int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                       int32_t group, const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* start_pos, int32_t batch, int32_t num_new, const void* k,
                       const void* v, int32_t kv_dtype, const float* mu, const float* rot_k,
                       const float* rot_v, float clip_k, float clip_v, void* stream) {
  const int st = check_append(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                              max_blocks_per_seq, start_pos, batch, num_new, k, v, kv_dtype, mu,
                              rot_k, rot_v, clip_k, clip_v);
  if (st != KVQ_OK || batch == 0 || num_new == 0) return st;
  const int rc = kvq::launch_append(static_cast<uint8_t*>(pages), num_blocks, num_kv_heads,
                                    head_dim / group, block_table, max_blocks_per_seq, start_pos,
                                    batch, num_new, k, v, kv_dtype == KVQ_BF16, mu, rot_k, rot_v,
                                    clip_k, clip_v, static_cast<hipStream_t>(stream));
  return rc == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

namespace {
bool valid_decode_shape(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t max_ctx_len, int32_t split_pages) {
  if (batch < 0 || batch > 65535 || num_kv_heads < 1 || num_q_heads < num_kv_heads) return false;
  if (num_q_heads % num_kv_heads != 0 || max_ctx_len < 0) return false;
  if (split_pages < 0 || split_pages % 8 != 0 || split_pages > 512) return false;
  const int qg = (num_q_heads / num_kv_heads + 3) / 4;
  if (static_cast<int64_t>(num_kv_heads) * qg > 65535) return false;
  return true;
}
}  // namespace

KVQ_API size_t kvq_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_ctx_len, int32_t split_pages) {
  if (head_dim != kvq::kHeadDim) return 0;
  if (!valid_decode_shape(batch, num_q_heads, num_kv_heads, max_ctx_len, split_pages)) return 0;
  return kvq::make_plan(batch, num_q_heads, num_kv_heads, max_ctx_len, split_pages).total;
}

KVQ_API int kvq_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_ctx_len, int32_t split_pages,
                            int32_t* num_splits, int32_t* split_pages_out,
                            int32_t* operand_in_scan) {
  if (head_dim != kvq::kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (!valid_decode_shape(batch, num_q_heads, num_kv_heads, max_ctx_len, split_pages))
    return KVQ_ERR_INVALID_ARG;
  const kvq::DecodePlan p = kvq::make_plan(batch, num_q_heads, num_kv_heads, max_ctx_len,
                                           split_pages);
  if (num_splits) *num_splits = p.S;
  if (split_pages_out) *split_pages_out = p.spw;
  if (operand_in_scan)
    *operand_in_scan = p.S > 0 && kvq::operand_in_scan(p, num_kv_heads, batch, KVQ_STAGE_ALL);
  return KVQ_OK;
}

namespace {
// Host-side checks of the decode arguments; on KVQ_OK with batch > 0, *plan
// is the workspace carve-up.
int check_decode(const void* pages, int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                 int32_t group, const int32_t* block_table, int32_t max_blocks_per_seq,
                 const int32_t* ctx_len, int32_t max_ctx_len, int32_t batch, int32_t num_q_heads,
                 const void* q, int32_t q_dtype, const float* rot_k, const float* rot_v,
                 float sm_scale, const float* out, const void* workspace, size_t workspace_bytes,
                 int32_t split_pages, kvq::DecodePlan* plan, bool own_workspace = true) {
  if (!valid_geometry(head_dim, group)) return KVQ_ERR_INVALID_ARG;
  if (head_dim != kvq::kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (!valid_decode_shape(batch, num_q_heads, num_kv_heads, max_ctx_len, split_pages))
    return KVQ_ERR_INVALID_ARG;
  if (num_blocks < 1 || max_blocks_per_seq < 1) return KVQ_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_ctx_len) > static_cast<int64_t>(max_blocks_per_seq) * kvq::kBlock)
    return KVQ_ERR_INVALID_ARG;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale) || sm_scale == 1.0f / 0.0f || sm_scale == -1.0f / 0.0f)
    return KVQ_ERR_INVALID_ARG;
  if (batch == 0) return KVQ_OK;
  // rot_v may be null: the output stays in the rotated value basis; rot_k may
  // be null: the keys were encoded unrotated and the query is not rotated
  if (!pages || !block_table || !ctx_len || !q || !out) return KVQ_ERR_INVALID_ARG;
  // q is read as 32- and 64-bit words and out written as 32-bit words: both
  // must be 16-byte aligned (as every tensor allocation is)
  if (!aligned(pages, 16) || (rot_k && !aligned(rot_k, 16)) || (rot_v && !aligned(rot_v, 16)) ||
      !aligned(q, 16) || !aligned(out, 16) || !aligned(block_table, 4) || !aligned(ctx_len, 4))
    return KVQ_ERR_INVALID_ARG;
  *plan = kvq::make_plan(batch, num_q_heads, num_kv_heads, max_ctx_len, split_pages);
  if (!own_workspace) return KVQ_OK;  // the library's static scratch; its size is checked apart
  if (!workspace || workspace_bytes < plan->total || !aligned(workspace, 256))
    return KVQ_ERR_WORKSPACE;
  return KVQ_OK;
}
}  // namespace

KVQ_API int kvq_decode_attn_staged(const void* pages, int64_t num_blocks, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t group, const int32_t* block_table,
                                   int32_t max_blocks_per_seq, const int32_t* ctx_len,
                                   int32_t max_ctx_len, int32_t batch, int32_t num_q_heads,
                                   const void* q, int32_t q_dtype, const float* rot_k,
                                   const float* rot_v, float sm_scale, float* out,
                                   void* workspace, size_t workspace_bytes, int32_t split_pages,
                                   int32_t stages, void* stream) {
  if (stages < 1 || stages > KVQ_STAGE_ALL) return KVQ_ERR_INVALID_ARG;
  kvq::DecodePlan plan{};
  const int st = check_decode(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                              max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q,
                              q_dtype, rot_k, rot_v, sm_scale, out, workspace, workspace_bytes,
                              split_pages, &plan);
  if (st != KVQ_OK || batch == 0) return st;
  const int rc = kvq::launch_decode(
      static_cast<const uint8_t*>(pages), num_blocks, num_kv_heads, head_dim / group, block_table,
      max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q, q_dtype == KVQ_BF16, rot_k,
      rot_v, sm_scale, out, workspace, plan, stages, static_cast<hipStream_t>(stream));
  return rc == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

KVQ_API int kvq_decode_attn(const void* pages, int64_t num_blocks, int32_t num_kv_heads,
                            int32_t head_dim, int32_t group, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* ctx_len,
                            int32_t max_ctx_len, int32_t batch, int32_t num_q_heads,
                            const void* q, int32_t q_dtype, const float* rot_k,
                            const float* rot_v, float sm_scale, float* out, void* workspace,
                            size_t workspace_bytes, int32_t split_pages, void* stream) {
  return kvq_decode_attn_staged(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                                max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q,
                                q_dtype, rot_k, rot_v, sm_scale, out, workspace, workspace_bytes,
                                split_pages, KVQ_STAGE_ALL, stream);
}

KVQ_API int kvq_append_decode(void* pages, int64_t num_blocks, int32_t num_kv_heads,
                              int32_t head_dim, int32_t group, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* start_pos,
                              const int32_t* ctx_len, int32_t max_ctx_len, int32_t batch,
                              const void* k, const void* v, int32_t kv_dtype, const float* mu,
                              float clip_k, float clip_v, int32_t num_q_heads, const void* q,
                              int32_t q_dtype, const float* rot_k, const float* rot_v,
                              float sm_scale, float* out, void* workspace,
                              size_t workspace_bytes, int32_t split_pages, void* stream) {
  int st = check_append(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                        max_blocks_per_seq, start_pos, batch, 1, k, v, kv_dtype, mu, rot_k, rot_v,
                        clip_k, clip_v);
  if (st != KVQ_OK) return st;
  kvq::DecodePlan plan{};
  st = check_decode(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                    max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q, q_dtype,
                    rot_k, rot_v, sm_scale, out, workspace, workspace_bytes, split_pages, &plan);
  if (st != KVQ_OK || batch == 0) return st;
  const int rc = kvq::launch_append_decode(
      static_cast<uint8_t*>(pages), num_blocks, num_kv_heads, head_dim / group, block_table,
      max_blocks_per_seq, start_pos, k, v, kv_dtype == KVQ_BF16, mu, clip_k, clip_v, ctx_len,
      max_ctx_len, batch, num_q_heads, q, q_dtype == KVQ_BF16, rot_k, rot_v, sm_scale, out,
      workspace, plan, static_cast<hipStream_t>(stream));
  return rc == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

// ----------------------------------------------------------------- BF16 windows
KVQ_API size_t kvq_window_bytes(int32_t batch, int32_t num_kv_heads, int32_t head_dim) {
  if (head_dim != kvq::kHeadDim || batch < 0 || num_kv_heads < 1) return 0;
  return static_cast<size_t>(batch) * num_kv_heads * 2 * kvq::kWindow * kvq::kHeadDim * 2;
}

KVQ_API int kvq_window_write(void* window, int32_t num_kv_heads, int32_t head_dim,
                             int32_t batch, const int32_t* start_pos, int32_t num_new,
                             const void* k, const void* v, int32_t kv_dtype, void* stream) {
  if (head_dim != kvq::kHeadDim) return head_dim > 0 ? KVQ_ERR_UNSUPPORTED : KVQ_ERR_INVALID_ARG;
  if (batch < 0 || batch > 65535 || num_new < 0 || num_kv_heads < 1 || num_kv_heads > 65535)
    return KVQ_ERR_INVALID_ARG;
  if (kv_dtype != KVQ_F32 && kv_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if (batch == 0 || num_new == 0) return KVQ_OK;
  if (!window || !start_pos || !k || !v) return KVQ_ERR_INVALID_ARG;
  if (!aligned(window, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(start_pos, 4))
    return KVQ_ERR_INVALID_ARG;
  const int rc = kvq::launch_window_write(static_cast<uint16_t*>(window), num_kv_heads, batch,
                                          start_pos, num_new, k, v, kv_dtype == KVQ_BF16,
                                          static_cast<hipStream_t>(stream));
  return rc == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

KVQ_API int kvq_decode_attn_window(const void* pages, int64_t num_blocks, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t group, const int32_t* block_table,
                                   int32_t max_blocks_per_seq, const void* window,
                                   const float* mu, const int32_t* ctx_len, int32_t max_ctx_len,
                                   int32_t batch, int32_t num_q_heads, const void* q,
                                   int32_t q_dtype, const float* rot_k, const float* rot_v,
                                   float sm_scale, float* out, void* workspace,
                                   size_t workspace_bytes, int32_t split_pages, void* stream) {
  kvq::DecodePlan plan{};
  const int st = check_decode(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                              max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q,
                              q_dtype, rot_k, rot_v, sm_scale, out, workspace, workspace_bytes,
                              split_pages, &plan);
  if (st != KVQ_OK || batch == 0) return st;
  if (!window || !mu || !aligned(window, 16) || !aligned(mu, 16)) return KVQ_ERR_INVALID_ARG;
  plan = kvq::make_window_plan(batch, num_q_heads, num_kv_heads, max_ctx_len, split_pages);
  const int rc = kvq::launch_decode(
      static_cast<const uint8_t*>(pages), num_blocks, num_kv_heads, head_dim / group, block_table,
      max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q, q_dtype == KVQ_BF16, rot_k,
      rot_v, sm_scale, out, workspace, plan, KVQ_STAGE_ALL, static_cast<hipStream_t>(stream),
      static_cast<const uint16_t*>(window), mu);
  return rc == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

KVQ_API int kvq_append_decode_window(void* pages, int64_t num_blocks, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t group, const int32_t* block_table,
                                     int32_t max_blocks_per_seq, void* window,
                                     const int32_t* start_pos, const int32_t* ctx_len,
                                     int32_t max_ctx_len, int32_t batch, const void* k,
                                     const void* v, int32_t kv_dtype, const float* mu,
                                     float clip_k, float clip_v, int32_t num_q_heads,
                                     const void* q, int32_t q_dtype, const float* rot_k,
                                     const float* rot_v, float sm_scale, float* out,
                                     void* workspace, size_t workspace_bytes, int32_t split_pages,
                                     void* stream) {
  int st = check_append(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                        max_blocks_per_seq, start_pos, batch, 1, k, v, kv_dtype, mu, rot_k, rot_v,
                        clip_k, clip_v);
  if (st != KVQ_OK) return st;
  kvq::DecodePlan plan{};
  st = check_decode(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                    max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q, q_dtype,
                    rot_k, rot_v, sm_scale, out, workspace, workspace_bytes, split_pages, &plan);
  if (st != KVQ_OK || batch == 0) return st;
  if (!window || !aligned(window, 16)) return KVQ_ERR_INVALID_ARG;
  plan = kvq::make_window_plan(batch, num_q_heads, num_kv_heads, max_ctx_len, split_pages);
  const int rc = kvq::launch_append_decode(
      static_cast<uint8_t*>(pages), num_blocks, num_kv_heads, head_dim / group, block_table,
      max_blocks_per_seq, start_pos, k, v, kv_dtype == KVQ_BF16, mu, clip_k, clip_v, ctx_len,
      max_ctx_len, batch, num_q_heads, q, q_dtype == KVQ_BF16, rot_k, rot_v, sm_scale, out,
      workspace, plan, static_cast<hipStream_t>(stream), static_cast<uint16_t*>(window));
  return rc == 0 ? KVQ_OK : KVQ_ERR_HIP;
}

// ----------------------------------------------------------------- no allocation
// The decode's workspace (query operands, split partials) in a file-scope
// device array, for callers that cannot allocate.  In host code `scratch` is
// only a stand-in symbol: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and that address, never the
// symbol, is what the kernels get.  Every call on a GPU shares that GPU's
// array; it keeps the last call's contents, and nothing in it needs to start
// at zero (each call writes every entry it later reads).
namespace {
__device__ __align__(256) uint8_t scratch[KVQ_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch array, or null on a HIP error.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}
}  // namespace

KVQ_API int kvq_decode_attn_noalloc(const void* pages, int64_t num_blocks, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t group, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, const int32_t* ctx_len,
                                    int32_t max_ctx_len, int32_t batch, int32_t num_q_heads,
                                    const void* q, int32_t q_dtype, const float* rot_k,
                                    const float* rot_v, float sm_scale, float* out,
                                    int32_t split_pages, void* stream) {
  kvq::DecodePlan plan{};
  const int st = check_decode(pages, num_blocks, num_kv_heads, head_dim, group, block_table,
                              max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q,
                              q_dtype, rot_k, rot_v, sm_scale, out, nullptr, 0, split_pages, &plan,
                              /*own_workspace=*/false);
  if (st != KVQ_OK || batch == 0) return st;
  if (plan.total > static_cast<size_t>(KVQ_SCRATCH_BYTES)) return KVQ_ERR_SCRATCH;
  void* ws = scratch_address();
  if (!ws) return KVQ_ERR_HIP;
  const int rc = kvq::launch_decode(
      static_cast<const uint8_t*>(pages), num_blocks, num_kv_heads, head_dim / group, block_table,
      max_blocks_per_seq, ctx_len, max_ctx_len, batch, num_q_heads, q, q_dtype == KVQ_BF16, rot_k,
      rot_v, sm_scale, out, ws, plan, KVQ_STAGE_ALL, static_cast<hipStream_t>(stream));
  return rc == 0 ? KVQ_OK : KVQ_ERR_HIP;
}
