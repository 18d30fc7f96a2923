// Host-side launchers shared between the entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

int launch_append(uint8_t* pages, int64_t num_blocks, int Hkv, int G, const int* block_table,
                  int max_blocks, const int* start_pos, int B, int T, const void* k,
                  const void* v, bool bf16, const float* mu, const float* rot_k,
                  const float* rot_v, float clip_k, float clip_v, hipStream_t stream);

// Workspace carve-up of one decode call.
struct DecodePlan {
  int QG;    // query-head tiles of 4 per KV head
  int spw;   // pages per workgroup split
  int S;     // splits for the longest context
  size_t qa_off, qf_off, part_off, wpart_off, deq_off, qr_off, total;
};

DecodePlan make_plan(int B, int Hq, int Hkv, int max_ctx, int split_pages);

// The plan of a call with BF16 windows (split_pages 0: a split size that
// keeps the scan launch within one round of workgroups where it can).
DecodePlan make_window_plan(int B, int Hq, int Hkv, int max_ctx, int split_pages);

// Whether a call launching the PREPARE and SPLITS stages together builds the
// query operand inside the split workgroups (no prologue launch).
bool operand_in_scan(const DecodePlan& p, int Hkv, int B, int stages);

int launch_decode(const uint8_t* pages, int64_t num_blocks, int Hkv, int G,
                  const int* block_table, int max_blocks, const int* ctx_len, int max_ctx, int B,
                  int Hq, const void* q, bool q_bf16, const float* rot_k, const float* rot_v,
                  float sm_scale, float* out, void* workspace, const DecodePlan& p, int stages,
                  hipStream_t stream, const uint16_t* win = nullptr, const float* mu = nullptr);

// The single-token append of one decode step fused with the first decode
// stage, then the scan and the merge.
int launch_append_decode(uint8_t* pages, int64_t num_blocks, int Hkv, int G,
                         const int* block_table, int max_blocks, const int* start_pos,
                         const void* k, const void* v, bool kv_bf16, const float* mu,
                         float clip_k, float clip_v, const int* ctx_len, int max_ctx, int B,
                         int Hq, const void* q, bool q_bf16, const float* rot_k,
                         const float* rot_v, float sm_scale, float* out, void* workspace,
                         const DecodePlan& p, hipStream_t stream, uint16_t* win = nullptr);

// Copy tokens (rounded to bfloat16) into the BF16 window store.
int launch_window_write(uint16_t* win, int Hkv, int B, const int* start_pos, int T, const void* k,
                        const void* v, bool bf16, hipStream_t stream);

}  // namespace kvq
