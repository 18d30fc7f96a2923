// Device-side constants and helpers shared by the append and decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kBlock = 16;          // tokens per page
constexpr int kKCodeOff = 0;        // 16 rows x 32 bytes
constexpr int kVCodeOff = 512;      // 128 32-bit words, one per channel
constexpr int kSzOff = 1024;        // K (scale, zero) pairs, then V pairs
constexpr float kF16Max = 65504.0f;

__host__ __device__ constexpr int page_bytes_for_groups(int G) { return 1024 + 128 * G; }

// BF16 windows: the first kSink tokens of a sequence and its last kRecent
// tokens, kept as given (rounded to bfloat16) beside the INT2 body.  Window
// store of one layer: bfloat16 [batch][Hkv][2: K, V][kWindow][head_dim]; the
// slot of position p is p for a sink, else a ring slot.
constexpr int kSink = 64;
constexpr int kRecent = 256;
constexpr int kWindow = kSink + kRecent;
__host__ __device__ constexpr int window_slot(int p) {
  return p < kSink ? p : kSink + (p - kSink) % kRecent;
}
// First sink-free token of the body and the body's end for a context of n.
__host__ __device__ constexpr int body_end(int n) { return n - kRecent > kSink ? n - kRecent : kSink; }

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// fp16 of x, round to nearest even, saturating at +-65504.
__device__ __forceinline__ _Float16 f16_sat(float x) {
  return static_cast<_Float16>(fminf(fmaxf(x, -kF16Max), kF16Max));
}

__device__ __forceinline__ uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

__device__ __forceinline__ float f16_lo_to_f32(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi_to_f32(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// bfloat16 of x, round to nearest even (finite x).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, 64);
}

// Reductions over the 16 lanes of a DPP row:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true));
}
// The maximum with a DPP source operand: one v_max_f32 per step (fmaxf would
// add a NaN-quieting max before each; these values are never NaN).  The nop
// gives the two wait states a DPP read of a just-written VGPR needs.
#define KVQ_MAX_DPP(v, ctrl)                                                            \
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf bound_ctrl:1" \
      : "=v"(v)                                                                         \
      : "v"(v))
__device__ __forceinline__ float row16_max(float v) {
  KVQ_MAX_DPP(v, "quad_perm:[1,0,3,2]");
  KVQ_MAX_DPP(v, "quad_perm:[2,3,0,1]");
  KVQ_MAX_DPP(v, "row_half_mirror");
  KVQ_MAX_DPP(v, "row_mirror");
  return v;
}
#undef KVQ_MAX_DPP
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xb1>(v);
  v += dpp<0x4e>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

// Reductions over the whole wave, the same value in every lane: the rows by
// DPP, then the four row results read as scalars.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float row16_min(float v) {
  asm("s_nop 1\n\tv_min_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\tv_min_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\tv_min_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\tv_min_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=&v"(v)
      : "v"(v));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
  v = row16_min(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fminf(fminf(r0, r1), fminf(r2, r3));
}

}  // namespace kvq
