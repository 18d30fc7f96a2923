// Single-token decode attention over the paged INT2 cache.
//
// Method: "Output-Aware Rotation for INT2 KV-Cache Quantization" (Pith review
// of arXiv 2608.02691), "What carries the argument" (attention over
// dequantised rotated keys and values, then the inverse rotation) and the
// abstract (the paged cache is read directly).  The softmax is the standard
// scaled dot product; the context is split across workgroups and merged by
// log-sum-exp.
//
// Three launches on the caller's stream:
//   1. prologue: q_r = q * R_K[h], scaled by sm_scale*log2(e) and a power of
//      two, split into fp16 hi + 2^11*lo parts laid out as the A operand of the
//      q.K MFMA (rows = 4 query heads x {hi, lo} x {channel half}).
//   2. scan: each wave streams 2-page chunks of one (sequence, KV head) through
//      an LDS ring filled by global->LDS DMA; q.K and P.V both run on 16x16x32
//      f16 MFMAs.  Cached 2-bit codes become MFMA operands through the packed
//      FP6 (e2m3) to f16 conversion, 32 values per instruction: masking a
//      32-bit word of 16 codes with 0xC30C30C3, 0x30C30C30 and 0x0C30C30C gives
//      three dwords of a packed FP6 block in which every 6-bit field holds one
//      code in its low bits, a subnormal that decodes to exactly code/8, a
//      normal fp16 value; field k of the block is code (3k mod 16) of word
//      k/16.  (fp16 subnormal operands are not an option: MFMA products with
//      them accumulate at roughly 2^-16 of the magnitude sum, normal ones at
//      2^-24.)  The four waves of a workgroup
//      interleave chunks and combine their (max, sum, output) in LDS; each
//      workgroup writes one partial per query head.
//   3. merge: log-sum-exp merge of the partials and the inverse value
//      rotation o = o_r * R_V^T.  (A separate launch: merging inside the scan
//      through a last-workgroup counter needs device-scope release/acquire,
//      i.e. an L2 writeback and invalidate per workgroup on this multi-XCD
//      part, which costs far more than the launch.)
#include "kvq_common.h"
#include "kvq_launch.h"

namespace kvq {

constexpr int kHT = 4;          // query heads per MFMA row tile
constexpr int kPartStride = 132;  // floats per partial: [0] = lse2, [4..131] = o
constexpr float kLog2e = 1.4426950408889634f;
// fp16 "lo" parts are stored scaled by 2^11 (their own MFMA rows) so that they
// stay clear of the fp16 subnormal range; the row sums are unscaled by 2^-11.
constexpr float kLoScale = 2048.0f;
constexpr float kLoUnscale = 1.0f / 2048.0f;

// --------------------------------------------------------------------------- prologue
// grid (Hkv * QG, B), block 256: wave w handles query head 4*qg + w of KV head h.
template <bool kBf16>
__global__ __launch_bounds__(256) void prologue_kernel(const void* __restrict__ q,
                                                       const float* __restrict__ rot_k, int Hq,
                                                       int Hkv, int QG, float qscale,
                                                       uint4* __restrict__ qa,
                                                       float4* __restrict__ qf) {
  __shared__ float qin[kHT][kHeadDim];
  __shared__ float qsc[kHT][kHeadDim];
  const int h = blockIdx.x / QG;
  const int qg = blockIdx.x % QG;
  const int b = blockIdx.y;
  const int Hg = Hq / Hkv;
  const int lane = threadIdx.x & 63;
  const int hl = threadIdx.x >> 6;
  const int hloc = qg * kHT + hl;
  const bool valid = hloc < Hg;

  const size_t qrow = (static_cast<size_t>(b) * Hq + h * Hg + hloc) * kHeadDim;
  float q0 = 0.f, q1 = 0.f;
  if (valid) {
    if constexpr (kBf16) {
      const uint16_t* qq = static_cast<const uint16_t*>(q) + qrow;
      q0 = bf16_to_f32(qq[lane]);
      q1 = bf16_to_f32(qq[lane + 64]);
    } else {
      const float* qq = static_cast<const float*>(q) + qrow;
      q0 = qq[lane];
      q1 = qq[lane + 64];
    }
  }
  qin[hl][lane] = q0;
  qin[hl][lane + 64] = q1;
  __syncthreads();

  // q_r[j] = sum_i q[i] R_K[i][j]; lane computes j = lane and j = lane + 64.
  const float* R = rot_k + static_cast<size_t>(h) * kHeadDim * kHeadDim;
  float r0 = 0.f, r1 = 0.f;
  if (valid) {
#pragma unroll 16
    for (int i = 0; i < kHeadDim; ++i) {
      const float qi = qin[hl][i];
      r0 = fmaf(qi, R[i * kHeadDim + lane], r0);
      r1 = fmaf(qi, R[i * kHeadDim + lane + 64], r1);
    }
  }
  r0 *= qscale;  // logits in log2 units
  r1 *= qscale;
  float amax = fmaxf(fabsf(r0), fabsf(r1));
  float s0 = r0, s1 = r1;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    amax = fmaxf(amax, shfl_xor(amax, m));
    s0 += shfl_xor(s0, m);
    s1 += shfl_xor(s1, m);
  }
  // Scale by 2^E so that max|q| * 2^E is in [2^14, 2^15): fp16 range.
  int E = 0;
  if (amax > 0.f) E = min(max(14 - ilogbf(amax), -100), 100);
  qsc[hl][lane] = ldexpf(r0, E);
  qsc[hl][lane + 64] = ldexpf(r1, E);
  if (lane == 0) {
    // the code operand holds code/8, so sum(q*code) = 2^(3-E) * D
    const size_t fi = ((static_cast<size_t>(b) * Hkv + h) * QG + qg) * kHT + hl;
    qf[fi] = make_float4(ldexpf(1.0f, 3 - E), s0, s1, 0.f);
  }
  __syncthreads();

  // A operand: lane L (row m = L%16 -> head m/4, half (m/2)%2, part m%2;
  // k-group kg = L/16) for MFMA j, element e holds channel
  // 32kg + 16(j/2) + (3*(8(j%2) + e) mod 16), matching codes_fp6.
  const int tid = threadIdx.x;
  const int L = tid >> 2;
  const int j = tid & 3;
  const int m = L & 15;
  const int rh = m >> 2, rgam = (m >> 1) & 1, rpart = m & 1;
  const int kg = L >> 4;
  uint32_t packed[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint32_t word = 0;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int e = 2 * e2 + hb;
      const int ch = 32 * kg + 16 * (j >> 1) + ((3 * (8 * (j & 1) + e)) & 15);
      const float x = (rgam == (kg >> 1)) ? qsc[rh][ch] : 0.f;
      const _Float16 hi = static_cast<_Float16>(x);
      const _Float16 lo = static_cast<_Float16>((x - static_cast<float>(hi)) * kLoScale);
      word |= static_cast<uint32_t>(f16_bits(rpart ? lo : hi)) << (16 * hb);
    }
    packed[e2] = word;
  }
  const size_t qi = (((static_cast<size_t>(b) * Hkv + h) * QG + qg) * 64 + L) * 4 + j;
  qa[qi] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
}

// --------------------------------------------------------------------------- split
// Code operands: two 32-bit code words (u = 0..15 at bits 2u) -> 32 fp16
// values code/8; value k = code (3*(k%16) mod 16) of word k/16.  The four
// 8-value slices are the B operands of four MFMAs.
typedef unsigned u32x6_t __attribute__((ext_vector_type(6)));
typedef _Float16 half32 __attribute__((ext_vector_type(32)));

__device__ __forceinline__ half32 codes_fp6(uint32_t w0, uint32_t w1) {
  const u32x6_t f = {w0 & 0xC30C30C3u, w0 & 0x30C30C30u, w0 & 0x0C30C30Cu,
                     w1 & 0xC30C30C3u, w1 & 0x30C30C30u, w1 & 0x0C30C30Cu};
  return __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(f, 1.0f);
}
template <int kS>
__device__ __forceinline__ half8 slice8(const half32& v) {
  return __builtin_shufflevector(v, v, 8 * kS, 8 * kS + 1, 8 * kS + 2, 8 * kS + 3, 8 * kS + 4,
                                 8 * kS + 5, 8 * kS + 6, 8 * kS + 7);
}

struct Chunk {
  uint2 kc0, kc1;  // K codes, pages 0/1: token t, bytes 8kg..8kg+7
  uint4 vc;        // V codes of page kg/2, token half kg%2, channel lane n
  uint2 szk0, szk1, szv0, szv1;  // (scale, zero) of token t; .y = group 1 if G == 2
  int pg0;
};

// ---- LDS ring: each wave keeps kDepth 2-page chunks in flight, loaded with
// global->LDS DMA (no VGPRs held while in flight).  A slot holds the two page
// images exactly as laid out in the cache: codes [0, 1024) and (scale, zero)
// pairs [1024, 1024 + 128G).  One chunk is kDmaPerChunk DMA instructions.
// Two chunks in flight per wave keep the workgroup's LDS under 40 KB, so four
// workgroups (four waves per SIMD) fit on a CU alongside the register cap.
constexpr int kDepth = 2;
constexpr int kRing = kDepth + 1;
constexpr int kDmaPerChunk = 4;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const uint8_t* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_base, 4, 0, 0);
}

// The compiler does not track when an LDS DMA lands: waits are explicit, and
// the memory clobber keeps LDS reads and DMA issues on their side of them.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int G>
__device__ __forceinline__ void issue_chunk(uint8_t* slot, const uint8_t* __restrict__ pages,
                                            int64_t num_blocks, int Hkv, int h,
                                            const int* __restrict__ row, int pg0, int p_end,
                                            int lane) {
  constexpr int PB = page_bytes_for_groups(G);
  int b0 = row[pg0];
  int b1 = (pg0 + 1 < p_end) ? row[pg0 + 1] : b0;
  b0 = static_cast<int>(min(static_cast<int64_t>(static_cast<uint32_t>(b0)), num_blocks - 1));
  b1 = static_cast<int>(min(static_cast<int64_t>(static_cast<uint32_t>(b1)), num_blocks - 1));
  const uint8_t* p0 = pages + (static_cast<int64_t>(b0) * Hkv + h) * PB;
  const uint8_t* p1 = pages + (static_cast<int64_t>(b1) * Hkv + h) * PB;
  dma16(p0 + 16 * lane, slot);
  dma16(p1 + 16 * lane, slot + PB);
  if (G == 2 || lane < 32) {
    dma4(p0 + kSzOff + 4 * lane, slot + kSzOff);
    dma4(p1 + kSzOff + 4 * lane, slot + PB + kSzOff);
  }
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)p));
}

// Read this lane's share of one ring slot.  The reads are inline assembly so
// that the compiler's wait insertion, which cannot tell ring slots apart and
// would drain every pending DMA before any LDS read, does not see them; the
// caller has already waited for this slot's DMAs, and the block ends with
// lgkmcnt(0) so its results are complete when it returns.
template <int G>
__device__ __forceinline__ void read_chunk(Chunk& c, const uint8_t* slot, int pg0, int lane) {
  constexpr int PB = page_bytes_for_groups(G);
  const int t = lane & 15, kg = lane >> 4;
  const uint32_t ak = lds_addr(slot + kKCodeOff + 32 * t + 8 * kg);
  const uint32_t av = lds_addr(slot + (kg >> 1) * PB + kVCodeOff + 256 * (kg & 1) + 16 * t);
  const uint32_t as = lds_addr(slot + kSzOff + t * 4 * G);
  u32x2 k0, k1;
  u32x4 v;
  if constexpr (G == 2) {
    u32x2 s0, s1, s2, s3;
    asm volatile(
        "ds_read_b64 %0, %7\n"
        "ds_read_b64 %1, %7 offset:%10\n"
        "ds_read_b128 %2, %8\n"
        "ds_read_b64 %3, %9\n"
        "ds_read_b64 %4, %9 offset:%10\n"
        "ds_read_b64 %5, %9 offset:%11\n"
        "ds_read_b64 %6, %9 offset:%12\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0), "=&v"(k1), "=&v"(v), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
        : "v"(ak), "v"(av), "v"(as), "i"(PB), "i"(64 * G), "i"(PB + 64 * G)
        : "memory");
    c.szk0 = make_uint2(s0.x, s0.y);
    c.szk1 = make_uint2(s1.x, s1.y);
    c.szv0 = make_uint2(s2.x, s2.y);
    c.szv1 = make_uint2(s3.x, s3.y);
  } else {
    uint32_t s0, s1, s2, s3;
    asm volatile(
        "ds_read_b64 %0, %7\n"
        "ds_read_b64 %1, %7 offset:%10\n"
        "ds_read_b128 %2, %8\n"
        "ds_read_b32 %3, %9\n"
        "ds_read_b32 %4, %9 offset:%10\n"
        "ds_read_b32 %5, %9 offset:%11\n"
        "ds_read_b32 %6, %9 offset:%12\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0), "=&v"(k1), "=&v"(v), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
        : "v"(ak), "v"(av), "v"(as), "i"(PB), "i"(64 * G), "i"(PB + 64 * G)
        : "memory");
    c.szk0 = make_uint2(s0, s0);
    c.szk1 = make_uint2(s1, s1);
    c.szv0 = make_uint2(s2, s2);
    c.szv1 = make_uint2(s3, s3);
  }
  c.kc0 = make_uint2(k0.x, k0.y);
  c.kc1 = make_uint2(k1.x, k1.y);
  c.vc = make_uint4(v.x, v.y, v.z, v.w);
  c.pg0 = pg0;
}

struct SoftmaxState {
  float m, l, zs0, zs1;
  floatx4 acc[8];
};

// Reductions over the 16 lanes of a DPP row (all lanes of one query head):
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xb1>(v));
  v = fmaxf(v, dpp<0x4e>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xb1>(v);
  v += dpp<0x4e>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

// 2^x on the hardware exp unit; arguments here are <= 0 (or -inf -> 0)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int G>
__device__ __forceinline__ void compute_chunk(const Chunk& c, SoftmaxState& st,
                                              const half8 (&qA)[4], float fac, float sq0,
                                              float sq1, int ctx, int p_end, int lane,
                                              _Float16* __restrict__ atile) {
  const int t = lane & 15;
  // ---- q.K: D[m = 4*hl + 2*gamma + part][token t]; one FP6 conversion per
  // page gives the four B operands (channels 32kg + 16(j/2) + ...)
  floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
  {
    const half32 k0 = codes_fp6(c.kc0.x, c.kc0.y);
    const half32 k1 = codes_fp6(c.kc1.x, c.kc1.y);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[0], slice8<0>(k0), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[0], slice8<0>(k1), d1, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[1], slice8<1>(k0), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[1], slice8<1>(k1), d1, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[2], slice8<2>(k0), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[2], slice8<2>(k1), d1, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[3], slice8<3>(k0), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[3], slice8<3>(k1), d1, 0, 0, 0);
  }

  const int pos0 = c.pg0 * kBlock + t;
  const bool v0 = pos0 < ctx;
  const bool v1 = (c.pg0 + 1 < p_end) && (pos0 + kBlock < ctx);
  float l0 = fac * (f16_lo_to_f32(c.szk0.x) * fmaf(d0[1], kLoUnscale, d0[0]) +
                    f16_lo_to_f32(c.szk0.y) * fmaf(d0[3], kLoUnscale, d0[2])) +
             f16_hi_to_f32(c.szk0.x) * sq0 + f16_hi_to_f32(c.szk0.y) * sq1;
  float l1 = fac * (f16_lo_to_f32(c.szk1.x) * fmaf(d1[1], kLoUnscale, d1[0]) +
                    f16_lo_to_f32(c.szk1.y) * fmaf(d1[3], kLoUnscale, d1[2])) +
             f16_hi_to_f32(c.szk1.x) * sq0 + f16_hi_to_f32(c.szk1.y) * sq1;
  l0 = v0 ? l0 : -INFINITY;
  l1 = v1 ? l1 : -INFINITY;

  // ---- online softmax (base 2), lazy rescale
  const float mc = row16_max(fmaxf(l0, l1));
  const float mnew = fmaxf(st.m, mc);
  if (__any(mnew > st.m)) {
    const float alpha = exp2_hw(st.m - mnew);
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] *= alpha;
    st.l *= alpha;
    st.zs0 *= alpha;
    st.zs1 *= alpha;
    st.m = mnew;
  }
  const float p0 = v0 ? exp2_hw(l0 - st.m) : 0.f;
  const float p1 = v1 ? exp2_hw(l1 - st.m) : 0.f;
  st.l += p0 + p1;
  const float sv00 = f16_lo_to_f32(c.szv0.x), zv00 = f16_hi_to_f32(c.szv0.x);
  const float sv01 = f16_lo_to_f32(c.szv0.y), zv01 = f16_hi_to_f32(c.szv0.y);
  const float sv10 = f16_lo_to_f32(c.szv1.x), zv10 = f16_hi_to_f32(c.szv1.x);
  const float sv11 = f16_lo_to_f32(c.szv1.y), zv11 = f16_hi_to_f32(c.szv1.y);
  st.zs0 += (v0 ? p0 * zv00 : 0.f) + (v1 ? p1 * zv10 : 0.f);
  st.zs1 += (v0 ? p0 * zv01 : 0.f) + (v1 ? p1 * zv11 : 0.f);

  // ---- P into the A tile of the P.V MFMA: row 4*hl + 2*gamma + part; token
  // t of page p sits at k = 16p + t (the V-code word layout puts token e of a
  // channel tile at conversion slot e).
  const int hl = lane >> 4;
  const int kk = t;
  const float w[2][2] = {{v0 ? p0 * sv00 : 0.f, v0 ? p0 * sv01 : 0.f},
                         {v1 ? p1 * sv10 : 0.f, v1 ? p1 * sv11 : 0.f}};
  uint32_t hv[2][2], lv[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const _Float16 hi = static_cast<_Float16>(w[p][g]);
      const _Float16 lo = static_cast<_Float16>((w[p][g] - static_cast<float>(hi)) * kLoScale);
      hv[p][g] = f16_bits(hi);
      lv[p][g] = f16_bits(lo);
    }
  }
  // Tile rows are 64 bytes (32 k slots); row 4hl + 2g + part, column 16p + kk.
  // Inline assembly keeps the compiler from draining the ring DMAs before
  // these accesses; LDS operations of one wave execute in order, so the read
  // sees the writes.
  const uint32_t wa = lds_addr(reinterpret_cast<const uint8_t*>(atile)) + 256 * hl + 2 * kk;
  asm volatile(
      "ds_write_b16 %0, %1\n"
      "ds_write_b16 %0, %2 offset:64\n"
      "ds_write_b16 %0, %3 offset:128\n"
      "ds_write_b16 %0, %4 offset:192\n"
      "ds_write_b16 %0, %5 offset:32\n"
      "ds_write_b16 %0, %6 offset:96\n"
      "ds_write_b16 %0, %7 offset:160\n"
      "ds_write_b16 %0, %8 offset:224"
      :
      : "v"(wa), "v"(hv[0][0]), "v"(lv[0][0]), "v"(hv[0][1]), "v"(lv[0][1]), "v"(hv[1][0]),
        "v"(lv[1][0]), "v"(hv[1][1]), "v"(lv[1][1])
      : "memory");
  const uint32_t ra =
      lds_addr(reinterpret_cast<const uint8_t*>(atile)) + 64 * (lane & 15) + 16 * (lane >> 4);
  u32x4 awv;
  asm volatile(
      "ds_read_b128 %0, %1\n"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(awv)
      : "v"(ra)
      : "memory");
  const half8 aw = __builtin_bit_cast(half8, awv);

  // ---- P.V: D[m][channel 16j + n]; dwords (0, 1) of this lane's V codes
  // convert to the B operands of channel tiles 0-3, dwords (2, 3) to 4-7
  {
    const half32 va = codes_fp6(c.vc.x, c.vc.y);
    st.acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, slice8<0>(va), st.acc[0], 0, 0, 0);
    st.acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, slice8<1>(va), st.acc[1], 0, 0, 0);
    st.acc[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, slice8<2>(va), st.acc[2], 0, 0, 0);
    st.acc[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, slice8<3>(va), st.acc[3], 0, 0, 0);
    const half32 vb = codes_fp6(c.vc.z, c.vc.w);
    st.acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, slice8<0>(vb), st.acc[4], 0, 0, 0);
    st.acc[5] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, slice8<1>(vb), st.acc[5], 0, 0, 0);
    st.acc[6] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, slice8<2>(vb), st.acc[6], 0, 0, 0);
    st.acc[7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, slice8<3>(vb), st.acc[7], 0, 0, 0);
  }
}

// ---- merge: log-sum-exp merge of the ns partials of the nh query heads of
// one head tile, then o = o_r * R_V[h]^T.  grid (Hkv * QG, B), block 256.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part,
                                                    const int* __restrict__ ctx_len, int max_ctx,
                                                    int Hq, int Hkv, int QG, int spw, int S,
                                                    const float* __restrict__ rot_v,
                                                    float* __restrict__ out) {
  __shared__ float orow[kHT * kHeadDim];
  const int h = blockIdx.x / QG;
  const int qg = blockIdx.x % QG;
  const int b = blockIdx.y;
  const int Hg = Hq / Hkv;
  const int nh = min(kHT, Hg - qg * kHT);
  const int ctx = min(max(ctx_len[b], 0), max_ctx);
  const int ns = ((ctx + kBlock - 1) / kBlock + spw - 1) / spw;
  const int u = threadIdx.x >> 6;
  const int c = threadIdx.x & 63;
  if (ns == 0) {  // empty context: zero output
    if (u < nh) {
      float* o = out + (static_cast<size_t>(b) * Hq + h * Hg + qg * kHT + u) * kHeadDim;
      o[c] = 0.f;
      o[c + 64] = 0.f;
    }
    return;
  }
  if (u < nh) {
    const float* p = part + (static_cast<size_t>(b) * Hq + h * Hg + qg * kHT + u) * S * kPartStride;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p[s * kPartStride]);
    float W = 0.f, a0 = 0.f, a1 = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float a = exp2_hw(p[s * kPartStride] - M);
      W += a;
      a0 = fmaf(a, p[s * kPartStride + 4 + c], a0);
      a1 = fmaf(a, p[s * kPartStride + 4 + c + 64], a1);
    }
    const float inv = 1.0f / W;
    orow[u * kHeadDim + c] = a0 * inv;
    orow[u * kHeadDim + c + 64] = a1 * inv;
  }
  __syncthreads();
  // thread -> (output channel j = tid/2, half of the input channels)
  const int j = threadIdx.x >> 1;
  const int half = threadIdx.x & 1;
  const float4* R = reinterpret_cast<const float4*>(
      rot_v + static_cast<size_t>(h) * kHeadDim * kHeadDim + j * kHeadDim + 64 * half);
  float o[kHT] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i4 = 0; i4 < 16; ++i4) {
    const float4 r = R[i4];
    const int i = 64 * half + 4 * i4;
#pragma unroll
    for (int uu = 0; uu < kHT; ++uu) {
      const float* orr = orow + uu * kHeadDim + i;
      o[uu] = fmaf(orr[0], r.x, fmaf(orr[1], r.y, fmaf(orr[2], r.z, fmaf(orr[3], r.w, o[uu]))));
    }
  }
#pragma unroll
  for (int uu = 0; uu < kHT; ++uu) {
    const float tot = o[uu] + __shfl_xor(o[uu], 1, 64);
    if (half == 0 && uu < nh)
      out[(static_cast<size_t>(b) * Hq + h * Hg + qg * kHT + uu) * kHeadDim + j] = tot;
  }
}

// grid (S, Hkv * QG, B), block 256: workgroup x covers pages [x*spw, (x+1)*spw).
// Capped at 128 VGPRs so that four waves share each SIMD: the scan is bound by
// the latency of its per-chunk dependency chain more than by issue slots.
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void split_kernel(
    const uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ ctx_len,
    int max_ctx, int Hq, int QG, int spw, const uint4* __restrict__ qa,
    const float4* __restrict__ qf, float* __restrict__ part, int S) {
  constexpr int kSlot = 2 * page_bytes_for_groups(G);
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][kRing][kSlot];
  __shared__ __attribute__((aligned(16))) _Float16 atile[4][16 * 32];
  __shared__ float cm[4][kHT], cl[4][kHT];

  const int h = blockIdx.y / QG;
  const int qg = blockIdx.y % QG;
  const int b = blockIdx.z;
  const int wgs = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ctx = min(max(ctx_len[b], 0), max_ctx);
  const int n_pages = (ctx + kBlock - 1) / kBlock;
  const int p_begin = wgs * spw;
  if (p_begin >= n_pages) return;
  const int p_end = min(p_begin + spw, n_pages);
  const int n_chunks = (p_end - p_begin + 1) >> 1;
  const int* row = block_table + static_cast<size_t>(b) * max_blocks;
  // this wave's chunks: c_i = wave + 4i
  const int nc = wave < n_chunks ? (n_chunks - wave + 3) / 4 : 0;
  // query operand first: waiting for it must not drain the ring's DMAs
  const size_t hgi = (static_cast<size_t>(b) * Hkv + h) * QG + qg;
  const uint4* qap = qa + (hgi * 64 + lane) * 4;
  half8 qA[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qA[j] = __builtin_bit_cast(half8, qap[j]);
  const int hl = lane >> 4;
  const float4 fq = qf[hgi * kHT + hl];
  // consume them here, so the wait for these loads is placed before the DMAs
  asm volatile("" ::"v"(qA[0]), "v"(qA[1]), "v"(qA[2]), "v"(qA[3]), "v"(fq.x), "v"(fq.y),
               "v"(fq.z));

  uint8_t* myring = &ring[wave][0][0];
  for (int i = 0; i < kDepth && i < nc; ++i)
    issue_chunk<G>(myring + i * kSlot, pages, num_blocks, Hkv, h, row,
                   p_begin + 2 * (wave + 4 * i), p_end, lane);

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.zs0 = 0.f;
  st.zs1 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < nc; ++i) {
    if (i + kDepth < nc)
      issue_chunk<G>(myring + ((i + kDepth) % kRing) * kSlot, pages, num_blocks, Hkv, h, row,
                     p_begin + 2 * (wave + 4 * (i + kDepth)), p_end, lane);
    // chunk i has landed once at most the DMAs of the chunks behind it are pending
    const int behind = min(kDepth, nc - 1 - i);
    if (behind == 2)
      wait_vmem<2 * kDmaPerChunk>();
    else if (behind == 1)
      wait_vmem<kDmaPerChunk>();
    else
      wait_vmem<0>();
    Chunk c;
    read_chunk<G>(c, myring + (i % kRing) * kSlot, p_begin + 2 * (wave + 4 * i), lane);
    compute_chunk<G>(c, st, qA, fq.x, fq.y, fq.z, ctx, p_end, lane, atile[wave]);
  }

  // ---- per-wave finish: reduce row sums, form unnormalised outputs
  const float l = row16_sum(st.l);
  const float zs0 = row16_sum(st.zs0);
  const float zs1 = row16_sum(st.zs1);
  const int n = lane & 15;
  __syncthreads();  // every wave is done with its ring; reuse it for the combine
  float(*co)[kHT][kHeadDim] = reinterpret_cast<float(*)[kHT][kHeadDim]>(&ring[0][0][0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int g = j >> 2;
    // code operand = code/8: sum(w * code) = 8 * D
    const float val = 8.0f * fmaf(st.acc[j][2 * g + 1], kLoUnscale, st.acc[j][2 * g]) +
                      (g ? zs1 : zs0);
    co[wave][hl][16 * j + n] = val;
  }
  if (n == 0) {
    cm[wave][hl] = st.m;
    cl[wave][hl] = l;
  }
  __syncthreads();

  // ---- combine the 4 waves: thread -> (head tid/64, channels c, c + 64)
  const int ch = threadIdx.x >> 6;
  const int cc = threadIdx.x & 63;
  const int hloc = qg * kHT + ch;
  const int Hg = Hq / Hkv;
  const int nh = min(kHT, Hg - qg * kHT);
  if (ch < nh) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, cm[w][ch]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = (cm[w][ch] == -INFINITY) ? 0.f : exp2_hw(cm[w][ch] - M);
      L += a * cl[w][ch];
      o0 += a * co[w][ch][cc];
      o1 += a * co[w][ch][cc + 64];
    }
    const int hq = h * Hg + hloc;
    float* dst = part + ((static_cast<size_t>(b) * Hq + hq) * S + wgs) * kPartStride;
    const float inv = 1.0f / L;
    dst[4 + cc] = o0 * inv;
    dst[4 + cc + 64] = o1 * inv;
    if (cc == 0) dst[0] = M + __log2f(L);
  }
}
// --------------------------------------------------------------------------- host side


static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int choose_split_pages(int B, int Hkv, int QG, int max_ctx) {
  const int64_t max_pages = (static_cast<int64_t>(max_ctx) + kBlock - 1) / kBlock;
  const int64_t total = static_cast<int64_t>(B) * Hkv * QG * max_pages;
  const int64_t target_wgs = 1024;  // 4 waves each: 16 waves per CU on 256 CUs
  int64_t spw = (total + target_wgs - 1) / target_wgs;
  spw = (spw + 7) / 8 * 8;
  if (spw < 8) spw = 8;
  if (spw > 256) spw = 256;
  return static_cast<int>(spw);
}

DecodePlan make_plan(int B, int Hq, int Hkv, int max_ctx, int split_pages) {
  DecodePlan p{};
  const int Hg = Hq / Hkv;
  p.QG = (Hg + kHT - 1) / kHT;
  p.spw = split_pages > 0 ? split_pages : choose_split_pages(B, Hkv, p.QG, max_ctx);
  const int64_t max_pages = (static_cast<int64_t>(max_ctx) + kBlock - 1) / kBlock;
  p.S = static_cast<int>((max_pages + p.spw - 1) / p.spw);
  const size_t hg = static_cast<size_t>(B) * Hkv * p.QG;
  p.qa_off = 0;
  p.qf_off = align256(hg * 64 * 64);
  p.part_off = p.qf_off + align256(hg * kHT * 16);
  p.total = p.part_off + align256(static_cast<size_t>(B) * Hq * (p.S ? p.S : 1) * kPartStride * 4);
  return p;
}

int launch_decode(const uint8_t* pages, int64_t num_blocks, int Hkv, int G,
                  const int* block_table, int max_blocks, const int* ctx_len, int max_ctx, int B,
                  int Hq, const void* q, bool q_bf16, const float* rot_k, const float* rot_v,
                  float sm_scale, float* out, void* workspace, const DecodePlan& p, int stages,
                  hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint4* qa = reinterpret_cast<uint4*>(ws + p.qa_off);
  float4* qf = reinterpret_cast<float4*>(ws + p.qf_off);
  float* part = reinterpret_cast<float*>(ws + p.part_off);
  const float qscale = sm_scale * kLog2e;
  if (p.S > 0 && (stages & 1)) {
    const dim3 g1(Hkv * p.QG, B);
    if (q_bf16)
      hipLaunchKernelGGL(prologue_kernel<true>, g1, dim3(256), 0, stream, q, rot_k, Hq, Hkv, p.QG,
                         qscale, qa, qf);
    else
      hipLaunchKernelGGL(prologue_kernel<false>, g1, dim3(256), 0, stream, q, rot_k, Hq, Hkv,
                         p.QG, qscale, qa, qf);
  }
  if (p.S > 0 && (stages & 2)) {
    const dim3 g2(p.S, Hkv * p.QG, B);
    if (G == 2)
      hipLaunchKernelGGL(split_kernel<2>, g2, dim3(256), 0, stream, pages, num_blocks, Hkv,
                         block_table, max_blocks, ctx_len, max_ctx, Hq, p.QG, p.spw, qa, qf, part,
                         p.S);
    else
      hipLaunchKernelGGL(split_kernel<1>, g2, dim3(256), 0, stream, pages, num_blocks, Hkv,
                         block_table, max_blocks, ctx_len, max_ctx, Hq, p.QG, p.spw, qa, qf, part,
                         p.S);
  }
  if (stages & 4)
    hipLaunchKernelGGL(merge_kernel, dim3(Hkv * p.QG, B), dim3(256), 0, stream, part, ctx_len,
                       max_ctx, Hq, Hkv, p.QG, p.spw, p.S ? p.S : 1, rot_v, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvq
