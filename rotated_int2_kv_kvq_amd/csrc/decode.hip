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
//   2. split: each wave streams 2-page chunks of one (sequence, KV head);
//      q.K and P.V both run on 16x16x32 f16 MFMAs.  Cached 2-bit codes become
//      MFMA operands through the FP4 (e2m1) to f16 conversion: masking a code
//      word with 0x33333333 leaves one code in the low bits of every nibble,
//      and such a nibble decodes to exactly code/2, a normal fp16 value.
//      (fp16 subnormal operands are not an option: MFMA products with them
//      accumulate at roughly 2^-16 of the magnitude sum, normal ones at 2^-24.)
//      The four waves of a workgroup interleave chunks and combine their
//      (max, sum, output) in LDS, so each workgroup writes one partial per
//      query head.
//   3. merge: log-sum-exp merge of the partials, then o = o_r * R_V^T.
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
    // the code operand holds code/2, so sum(q*code) = 2^(1-E) * D
    const size_t fi = ((static_cast<size_t>(b) * Hkv + h) * QG + qg) * kHT + hl;
    qf[fi] = make_float4(ldexpf(1.0f, 1 - E), s0, s1, 0.f);
  }
  __syncthreads();

  // A operand: lane L (row m = L%16 -> head m/4, half (m/2)%2, part m%2;
  // k-group kg = L/16) for MFMA j, element e holds channel
  // 32kg + 16(j/2) + 8(j%2) + 4(e/4) + (e/2)%2 + 2(e%2), matching codes_b.
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
      const int ch = 32 * kg + 16 * (j >> 1) + 8 * (j & 1) + 4 * (e >> 2) + ((e >> 1) & 1) +
                     2 * (e & 1);
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
// Code operands.  m0 = w & 0x33333333 holds codes u = 4b, 4b+2 in the two
// nibbles of byte b, m1 = (w >> 2) & 0x33333333 codes u = 4b+1, 4b+3; each
// FP4 conversion turns one byte into two fp16 values code/2.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <int kByte>
__device__ __forceinline__ half2v fp4x2(uint32_t m) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 1.0f, kByte);
}

// B operand from bytes kB and kB+1 of (m0, m1): element e = 2*dd + h holds
// code u = 4*(kB + dd/2) + dd%2 + 2h, i.e. with u0 = 4*kB:
// u0 + 4(e/4) + (e/2)%2 + 2(e%2).
template <int kB>
__device__ __forceinline__ half8 codes_b(uint32_t m0, uint32_t m1) {
  const half2v d0 = fp4x2<kB>(m0), d1 = fp4x2<kB>(m1);
  const half2v d2 = fp4x2<kB + 1>(m0), d3 = fp4x2<kB + 1>(m1);
  return half8{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

struct Chunk {
  uint2 kc0, kc1;  // K codes, pages 0/1: token t, bytes 8kg..8kg+7
  uint4 vc;        // V codes of page kg/2, token half kg%2, channel lane n
  uint2 szk0, szk1, szv0, szv1;  // (scale, zero) of token t; .y = group 1 if G == 2
  int pg0;
};

template <int G>
__device__ __forceinline__ uint2 load_sz(const uint8_t* p) {
  if constexpr (G == 2) {
    return *reinterpret_cast<const uint2*>(p);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    return make_uint2(w, w);
  }
}

template <int G>
__device__ __forceinline__ void load_chunk(Chunk& c, const uint8_t* __restrict__ pages,
                                           int64_t num_blocks, int Hkv, int h,
                                           const int* __restrict__ row, int pg0, int p_end,
                                           int lane) {
  constexpr int PB = page_bytes_for_groups(G);
  const int t = lane & 15, kg = lane >> 4;
  int b0 = row[pg0];
  int b1 = (pg0 + 1 < p_end) ? row[pg0 + 1] : b0;
  b0 = static_cast<int>(min(static_cast<int64_t>(static_cast<uint32_t>(b0)), num_blocks - 1));
  b1 = static_cast<int>(min(static_cast<int64_t>(static_cast<uint32_t>(b1)), num_blocks - 1));
  const uint8_t* p0 = pages + (static_cast<int64_t>(b0) * Hkv + h) * PB;
  const uint8_t* p1 = pages + (static_cast<int64_t>(b1) * Hkv + h) * PB;
  c.kc0 = *reinterpret_cast<const uint2*>(p0 + kKCodeOff + 32 * t + 8 * kg);
  c.kc1 = *reinterpret_cast<const uint2*>(p1 + kKCodeOff + 32 * t + 8 * kg);
  const uint8_t* pv = (kg >> 1) ? p1 : p0;
  c.vc = *reinterpret_cast<const uint4*>(pv + kVCodeOff + 256 * (kg & 1) + 16 * t);
  c.szk0 = load_sz<G>(p0 + kSzOff + t * 4 * G);
  c.szk1 = load_sz<G>(p1 + kSzOff + t * 4 * G);
  c.szv0 = load_sz<G>(p0 + kSzOff + 64 * G + t * 4 * G);
  c.szv1 = load_sz<G>(p1 + kSzOff + 64 * G + t * 4 * G);
  c.pg0 = pg0;
}

struct SoftmaxState {
  float m, l, zs0, zs1;
  floatx4 acc[8];
};

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, shfl_xor(v, 1));
  v = fmaxf(v, shfl_xor(v, 2));
  v = fmaxf(v, shfl_xor(v, 4));
  v = fmaxf(v, shfl_xor(v, 8));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += shfl_xor(v, 1);
  v += shfl_xor(v, 2);
  v += shfl_xor(v, 4);
  v += shfl_xor(v, 8);
  return v;
}

template <int G>
__device__ __forceinline__ void compute_chunk(const Chunk& c, SoftmaxState& st,
                                              const half8 (&qA)[4], float fac, float sq0,
                                              float sq1, int ctx, int p_end, int lane,
                                              _Float16* __restrict__ atile) {
  const int t = lane & 15;
  // ---- q.K: D[m = 4*hl + 2*gamma + part][token t]; MFMA j takes word j/2,
  // bytes 2(j%2), 2(j%2)+1 (channels 32kg + 16(j/2) + 8(j%2) + ...)
  floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
  {
    const uint32_t a0 = c.kc0.x & 0x33333333u, a1 = (c.kc0.x >> 2) & 0x33333333u;
    const uint32_t b0 = c.kc1.x & 0x33333333u, b1 = (c.kc1.x >> 2) & 0x33333333u;
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[0], codes_b<0>(a0, a1), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[0], codes_b<0>(b0, b1), d1, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[1], codes_b<2>(a0, a1), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[1], codes_b<2>(b0, b1), d1, 0, 0, 0);
  }
  {
    const uint32_t a0 = c.kc0.y & 0x33333333u, a1 = (c.kc0.y >> 2) & 0x33333333u;
    const uint32_t b0 = c.kc1.y & 0x33333333u, b1 = (c.kc1.y >> 2) & 0x33333333u;
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[2], codes_b<0>(a0, a1), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[2], codes_b<0>(b0, b1), d1, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[3], codes_b<2>(a0, a1), d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[3], codes_b<2>(b0, b1), d1, 0, 0, 0);
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
    const float alpha = exp2f(st.m - mnew);
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] *= alpha;
    st.l *= alpha;
    st.zs0 *= alpha;
    st.zs1 *= alpha;
    st.m = mnew;
  }
  const float p0 = v0 ? exp2f(l0 - st.m) : 0.f;
  const float p1 = v1 ? exp2f(l1 - st.m) : 0.f;
  st.l += p0 + p1;
  const float sv00 = f16_lo_to_f32(c.szv0.x), zv00 = f16_hi_to_f32(c.szv0.x);
  const float sv01 = f16_lo_to_f32(c.szv0.y), zv01 = f16_hi_to_f32(c.szv0.y);
  const float sv10 = f16_lo_to_f32(c.szv1.x), zv10 = f16_hi_to_f32(c.szv1.x);
  const float sv11 = f16_lo_to_f32(c.szv1.y), zv11 = f16_hi_to_f32(c.szv1.y);
  st.zs0 += (v0 ? p0 * zv00 : 0.f) + (v1 ? p1 * zv10 : 0.f);
  st.zs1 += (v0 ? p0 * zv01 : 0.f) + (v1 ? p1 * zv11 : 0.f);

  // ---- P into the A tile of the P.V MFMA: row 4*hl + 2*gamma + part; token
  // t = 8*th + e of page p sits at k = 16p + 8th + 4(e/4) + 2(e%2) + (e/2)%2,
  // the slot whose V code codes_b places there.
  const int hl = lane >> 4;
  const int e = t & 7;
  const int kk = 8 * (t >> 3) + 4 * (e >> 2) + 2 * (e & 1) + ((e >> 1) & 1);
  const float w[2][2] = {{v0 ? p0 * sv00 : 0.f, v0 ? p0 * sv01 : 0.f},
                         {v1 ? p1 * sv10 : 0.f, v1 ? p1 * sv11 : 0.f}};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const _Float16 hi = static_cast<_Float16>(w[p][g]);
      const _Float16 lo = static_cast<_Float16>((w[p][g] - static_cast<float>(hi)) * kLoScale);
      const int row = 4 * hl + 2 * g;
      atile[row * 32 + 16 * p + kk] = hi;
      atile[(row + 1) * 32 + 16 * p + kk] = lo;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const half8 aw = *reinterpret_cast<const half8*>(atile + (lane & 15) * 32 + 8 * (lane >> 4));

  // ---- P.V: D[m][channel 16j + n]; dword j/2 holds the chunks of MFMAs j
  // (bytes 0-1) and j+1 (bytes 2-3), token e of a chunk at bits 2e.
  const uint32_t vw[4] = {c.vc.x, c.vc.y, c.vc.z, c.vc.w};
#pragma unroll
  for (int q2 = 0; q2 < 4; ++q2) {
    const uint32_t m0 = vw[q2] & 0x33333333u, m1 = (vw[q2] >> 2) & 0x33333333u;
    st.acc[2 * q2] =
        __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, codes_b<0>(m0, m1), st.acc[2 * q2], 0, 0, 0);
    st.acc[2 * q2 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, codes_b<2>(m0, m1),
                                                                st.acc[2 * q2 + 1], 0, 0, 0);
  }
}

// grid (S, Hkv * QG, B), block 256: workgroup x covers pages [x*spw, (x+1)*spw).
template <int G>
__global__ __launch_bounds__(256) void split_kernel(
    const uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ ctx_len,
    int max_ctx, int Hq, int QG, int spw, const uint4* __restrict__ qa,
    const float4* __restrict__ qf, float* __restrict__ part, int S) {
  __shared__ __attribute__((aligned(16))) _Float16 atile[4][2][16 * 32];
  __shared__ float cm[4][kHT], cl[4][kHT];
  __shared__ float co[4][kHT][kHeadDim];

  const int h = blockIdx.y / QG;
  const int qg = blockIdx.y % QG;
  const int b = blockIdx.z;
  const int wgs = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ctx = min(max(ctx_len[b], 0), max_ctx);
  const int n_pages = (ctx + kBlock - 1) / kBlock;
  const int p_begin = wgs * spw;
  if (p_begin >= n_pages) return;
  const int p_end = min(p_begin + spw, n_pages);
  const int n_chunks = (p_end - p_begin + 1) >> 1;
  const int* row = block_table + static_cast<size_t>(b) * max_blocks;

  const size_t hgi = (static_cast<size_t>(b) * Hkv + h) * QG + qg;
  const uint4* qap = qa + (hgi * 64 + lane) * 4;
  half8 qA[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qA[j] = __builtin_bit_cast(half8, qap[j]);
  const int hl = lane >> 4;
  const float4 fq = qf[hgi * kHT + hl];

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.zs0 = 0.f;
  st.zs1 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  Chunk ca, cb;
  int c = wave;
  if (c < n_chunks)
    load_chunk<G>(ca, pages, num_blocks, Hkv, h, row, p_begin + 2 * c, p_end, lane);
  while (c < n_chunks) {
    if (c + 4 < n_chunks)
      load_chunk<G>(cb, pages, num_blocks, Hkv, h, row, p_begin + 2 * (c + 4), p_end, lane);
    compute_chunk<G>(ca, st, qA, fq.x, fq.y, fq.z, ctx, p_end, lane, atile[wave][0]);
    c += 4;
    if (c >= n_chunks) break;
    if (c + 4 < n_chunks)
      load_chunk<G>(ca, pages, num_blocks, Hkv, h, row, p_begin + 2 * (c + 4), p_end, lane);
    compute_chunk<G>(cb, st, qA, fq.x, fq.y, fq.z, ctx, p_end, lane, atile[wave][1]);
    c += 4;
  }

  // ---- per-wave finish: reduce row sums, form unnormalised outputs
  const float l = row16_sum(st.l);
  const float zs0 = row16_sum(st.zs0);
  const float zs1 = row16_sum(st.zs1);
  const int n = lane & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int g = j >> 2;
    // code operand = code/2: sum(w * code) = 2 * D
    const float val = 2.0f * fmaf(st.acc[j][2 * g + 1], kLoUnscale, st.acc[j][2 * g]) +
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
  if (hloc < Hg) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, cm[w][ch]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = (cm[w][ch] == -INFINITY) ? 0.f : exp2f(cm[w][ch] - M);
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

// --------------------------------------------------------------------------- merge
// grid (Hkv, B), block 128: thread j = output channel.
constexpr int kMergeHeads = 8;
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part,
                                                    const int* __restrict__ ctx_len, int max_ctx,
                                                    int Hq, int Hkv, int spw, int S,
                                                    const float* __restrict__ rot_v,
                                                    float* __restrict__ out) {
  __shared__ float orow[kMergeHeads][kHeadDim];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int j = threadIdx.x;
  const int Hg = Hq / Hkv;
  const int ctx = min(max(ctx_len[b], 0), max_ctx);
  const int n_pages = (ctx + kBlock - 1) / kBlock;
  const int ns = (n_pages + spw - 1) / spw;
  const float* R = rot_v + static_cast<size_t>(h) * kHeadDim * kHeadDim + j * kHeadDim;
  for (int h0 = 0; h0 < Hg; h0 += kMergeHeads) {
    const int nh = min(kMergeHeads, Hg - h0);
    for (int u = 0; u < nh; ++u) {
      const int hq = h * Hg + h0 + u;
      const float* p = part + (static_cast<size_t>(b) * Hq + hq) * S * kPartStride;
      float M = -INFINITY;
      for (int s = 0; s < ns; ++s) M = fmaxf(M, p[s * kPartStride]);
      float W = 0.f, acc = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float a = exp2f(p[s * kPartStride] - M);
        W += a;
        acc = fmaf(a, p[s * kPartStride + 4 + j], acc);
      }
      orow[u][j] = ns ? acc / W : 0.f;
    }
    __syncthreads();
    // o[j] = sum_i o_r[i] * R_V[j][i]
    float o[kMergeHeads];
#pragma unroll
    for (int u = 0; u < kMergeHeads; ++u) o[u] = 0.f;
    for (int i = 0; i < kHeadDim; i += 4) {
      const float4 r = *reinterpret_cast<const float4*>(R + i);
#pragma unroll
      for (int u = 0; u < kMergeHeads; ++u) {
        if (u < nh) {
          o[u] = fmaf(orow[u][i], r.x, o[u]);
          o[u] = fmaf(orow[u][i + 1], r.y, o[u]);
          o[u] = fmaf(orow[u][i + 2], r.z, o[u]);
          o[u] = fmaf(orow[u][i + 3], r.w, o[u]);
        }
      }
    }
    for (int u = 0; u < nh; ++u)
      out[(static_cast<size_t>(b) * Hq + h * Hg + h0 + u) * kHeadDim + j] = o[u];
    __syncthreads();
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
    hipLaunchKernelGGL(merge_kernel, dim3(Hkv, B), dim3(128), 0, stream, part, ctx_len, max_ctx,
                       Hq, Hkv, p.spw, p.S ? p.S : 1, rot_v, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvq
