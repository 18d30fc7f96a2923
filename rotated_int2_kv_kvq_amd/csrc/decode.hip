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
//   1. prologue: q_r = q * R_K, scaled by sm_scale*log2(e), written as the A
//      operands of the q.K products: each query head's |q_r| is fixed-point
//      with 32 fraction bits under a per-head power of two, and its 4-bit
//      digits are MFMA rows (rows = 4 heads x 4 digits per operand), each
//      digit an FP6 value b/8 with the sign of q_r, each row weighted by its
//      own E8M0 block scale.
//   2. scan: each wave streams its 8-page (128-token) blocks of one
//      (sequence, KV head) through an LDS ring filled by global->LDS DMA.
//      Cached 2-bit codes are MFMA operands as they stand: masking a 32-bit
//      word of 16 codes with 0xC30C30C3, 0x30C30C30 and 0x0C30C30C gives three
//      dwords of a packed FP6 block whose 6-bit fields hold one code each in
//      their low bits, i.e. the FP6 subnormal code/8 (field k = code 3k mod 16
//      of the word).  q.K runs as 16x16x128 FP6 x FP6 MFMAs per page (two
//      digit operands, three for group 64); P.V as two 16x16x128 FP8 x FP6
//      MFMAs per 16 output channels and block, with the softmax weights p*s_V
//      again fixed-point (24 bits under a per-head, per-block power of two)
//      split into six 4-bit digits, each digit b an FP8 byte worth b*2^-9.
//      Digits and codes are short enough that the MFMA sums are exact before
//      the fp32 accumulation.
//      The four waves of a split combine their (max, sum, output) in LDS;
//      each split writes one partial per query head.
//   3. merge: log-sum-exp merge of the partials and the inverse value
//      rotation o = o_r * R_V^T.  (A separate launch: merging inside the scan
//      through a last-workgroup counter needs device-scope release/acquire,
//      i.e. an L2 writeback and invalidate per workgroup on this multi-XCD
//      part, which costs far more than the launch.)
#include <stddef.h>

#include <algorithm>

#include "append_one.h"
#include "kvq_common.h"
#include "kvq_launch.h"


namespace kvq {

constexpr int kHT = 4;            // query heads per MFMA row tile (x 4 digit rows)
constexpr int kPartStride = 132;  // floats per partial: [0] = lse2, [4..131] = o
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so exp2(l - m) is 0, not NaN
constexpr float kLazy = 8.0f;        // log2 headroom before the running maximum is raised
// Per lane of the q.K A operands: [0, 6) and [6, 12) and (group 64) [12, 18)
// three FP6 operands, [28] and [29] the E8M0 row scales of the high- and
// low-digit operands.
constexpr int kQaDwords = 32;
constexpr int kQaScale = 28;
// The same operand in LDS (built by a split workgroup itself): 20 dwords per
// lane, the row scales at 18 and 19.
constexpr int kQaLds = 20;
constexpr int kQaLdsScale = 18;
constexpr int kFmtFp8 = 0;           // f8f6f4 MFMA operand formats
constexpr int kFmtFp6 = 2;
constexpr int kScaleOne = 127;  // E8M0 2^0

typedef int v8i __attribute__((ext_vector_type(8)));

// A compile-time value passed to a generic lambda.
template <typename T, T V>
struct Const {
  static constexpr T value = V;
};
// f(Const<int, I>{}) for I = I0 .. N-1, in order.
template <int I0, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(Const<int, I0>{});
    static_for<I0 + 1, N>(f);
  }
}

// 16x16x128 MFMA, D = A*B + C with per-lane E8M0 scales (A scale = this lane's
// row; every lane of a row passes the same value).
template <int FA, int FB>
__device__ __forceinline__ floatx4 mfma128(const v8i& a, const v8i& b, const floatx4& c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, kScaleOne);
}

// FP6 operand from two code words (16 codes each, code u at bits 2u): field j
// of the 32 holds code (3*(j%16)) mod 16 of word j/16, as the value code/8.
// An FP6 operand is six dwords; the MFMA never reads the last two of the
// eight-register tuple, so they are left undefined (no moves to fill them).
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v8i fp6_codes(uint32_t w0, uint32_t w1) {
  const v4i a = {static_cast<int>(w0 & 0xC30C30C3u), static_cast<int>(w0 & 0x30C30C30u),
                 static_cast<int>(w0 & 0x0C30C30Cu), static_cast<int>(w1 & 0xC30C30C3u)};
  const v4i c = {static_cast<int>(w1 & 0x30C30C30u), static_cast<int>(w1 & 0x0C30C30Cu), 0, 0};
  return __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, -1, -1);
}

// 2^x on the hardware exp unit
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// exponent e with |x| < 2^e <= 2|x| (0 for x == 0)
__device__ __forceinline__ int exp_above(float x) { return __builtin_amdgcn_frexp_expf(x); }

// Splits of a context of n_pages pages: round(n_pages / spw) of them (at least
// one for a non-empty context), spw pages each except the last, which takes
// the rest (between spw/2 and 3spw/2 pages), so that a context a few pages
// past a multiple of spw does not start a nearly empty workgroup after all
// the others.
__host__ __device__ inline int num_splits(int n_pages, int spw) {
  if (n_pages <= 0) return 0;
  return max(1, (n_pages + spw / 2) / spw);
}

// Division by a divisor fixed for the launch as a multiply and a shift
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994): for 1 <= d <= 2^31 take l = ceil(log2 d),
// s = 31 + l and m = ceil(2^s / d), which lies in [2^31, 2^32).  With
// e = m d - 2^s in [0, d), n m / 2^s = n / d + n e / (d 2^s), and for
// 0 <= n < 2^31 the second term is below 1/d, so the floor is n / d.  The
// host computes (m, s); in a kernel the quotient of a uniform n is three
// scalar instructions instead of the integer division's reciprocal sequence,
// whose vector-to-scalar round trips make up much of a workgroup's start.
struct FastDiv {
  uint32_t m, s;
  __device__ __forceinline__ int div(int n) const {
    return static_cast<int>((static_cast<uint64_t>(static_cast<uint32_t>(n)) * m) >> s);
  }
};
inline FastDiv fast_div(int d) {
  uint32_t l = 0;
  while ((1ull << l) < static_cast<uint64_t>(d)) ++l;
  const uint64_t sh = 31 + l;
  return FastDiv{static_cast<uint32_t>(((1ull << sh) + d - 1) / static_cast<uint64_t>(d)),
                 static_cast<uint32_t>(sh)};
}
// num_splits of a non-negative page count with spw as a FastDiv
__device__ __forceinline__ int num_splits_fd(int n_pages, int spw, FastDiv fspw) {
  if (n_pages <= 0) return 0;
  return max(1, fspw.div(n_pages + spw / 2));
}

// --------------------------------------------------------------------------- prologue
// grid (Hkv * QG, B), block 512: eight waves form q.R_K of query tile qg of
// KV head h (a quarter of R_K's rows and half its columns each), four turn
// the four heads into digits, then 64 threads per operand pack the A
// operands lane by lane.
//
// |x| is fixed-point with 32 fraction bits under 2^e: eight 4-bit digits,
// digit d (0 = most significant) worth b * 2^(e - 4 - 4d), as the FP6 value
// b/8 under the row scale 2^(e + 2 - 4d): the extra 8 cancels the code
// operand's code/8, so the MFMA rows sum to x . code.  In an A operand, lane
// L has row r = L%16 and lane group g = L/16; FP6 field j (k = 32g + j) is
// channel 32g + 16(j/16) + (3(j%16) mod 16), the channel order fp6_codes
// gives the key code words.
//   group 128: operand 0 rows (head r/4, digit r%4), operand 1 rows
//              (head r/4, digit 4 + r%4);
//   group 64:  operand 0 and 1 rows (head r/4, digit r%4) over the channels
//              of group 0 and 1 (zero in the other lanes), operand 2 rows
//              (head r/4, group (r/2)%2, digit 4 + r%2) over that group's
//              channels: 24 bits.

// Wave hl of the first 256 threads: the digits of query head hl of the tile
// into dig, its exponent into qe and its per-group sums into qf.
template <int G>
__device__ __forceinline__ void prologue_digits(float qscale,
                                                const float (&red)[4][kHT][kHeadDim],
                                                uint8_t (&dig)[kHT][kHeadDim][8],
                                                int (&qe)[kHT], float4* __restrict__ qf_tile,
                                                float* __restrict__ qr_tile) {
  const int lane = threadIdx.x & 63;
  const int wv = (threadIdx.x >> 6) & 3;
  // wave hl: x = qscale * q_r of head hl, channels lane and lane + 64
  const int hl = wv;
  float r0 = ((red[0][hl][lane] + red[1][hl][lane]) + (red[2][hl][lane] + red[3][hl][lane]));
  float r1 = ((red[0][hl][lane + 64] + red[1][hl][lane + 64]) +
              (red[2][hl][lane + 64] + red[3][hl][lane + 64]));
  r0 *= qscale;  // logits in log2 units
  r1 *= qscale;
  if (qr_tile) {  // the rotated, scaled query in float32 (the decode step's new token)
    qr_tile[hl * kHeadDim + lane] = r0;
    qr_tile[hl * kHeadDim + lane + 64] = r1;
  }
  const float amax = wave_max(fmaxf(fabsf(r0), fabsf(r1)));
  const float s0 = wave_sum(r0), s1 = wave_sum(r1);
  // |x| < 2^e: |x| / 2^e to 32 fraction bits, rounded to nearest; digit d
  // (0 = most significant) as the FP6 field sign | nibble, the eight fields
  // of a channel as bytes d = 0..7.  Within a register: the four nibbles of
  // each half of W spread to the four bytes (lowest nibble to byte 0), the
  // bytes reversed (digit 0 is the top nibble), and a nonzero byte b (b + 15
  // reaches bit 4, b <= 15 carries no further) given the sign bit 0x20.
  const int e = min(max(exp_above(amax), -100), 100);
  auto digits = [&](float x, int ch) {
    const uint32_t W =
        static_cast<uint32_t>(fminf(rintf(ldexpf(fabsf(x), 32 - e)), 4294967040.0f));
    const uint32_t sg = x < 0.f ? ~0u : 0u;
    auto fields4 = [&](uint32_t t) {  // t: 16 bits, digits 4k..4k+3 from the top
      uint32_t v = (t | (t << 8)) & 0x00FF00FFu;
      v = __builtin_bswap32((v | (v << 4)) & 0x0F0F0F0Fu);
      return v | ((((v + 0x0F0F0F0Fu) & 0x10101010u) << 1) & sg);
    };
    *reinterpret_cast<uint2*>(&dig[hl][ch][0]) =
        make_uint2(fields4(W >> 16), fields4(W & 0xffffu));
  };
  digits(r0, lane);
  digits(r1, lane + 64);
  if (lane == 0) {
    qe[hl] = e;
    // per-group sums of x for the zero-point term (channels < 64, >= 64)
    qf_tile[hl] = make_float4(0.f, s0, s1, 0.f);
  }
}

// The A operands, one thread per (operand, lane).
template <int G>
__device__ __forceinline__ void prologue_pack(const uint8_t (&dig)[kHT][kHeadDim][8],
                                              const int (&qe)[kHT], uint32_t* __restrict__ qa_tile,
                                              int lane_stride, int scale_off) {
  const int lane = threadIdx.x & 63;
  const int wv = (threadIdx.x >> 6) & 3;
  // thread (operand, lane L): FP6 field j of lane L (row r = L%16, lane group
  // g = L/16) holds the digit of channel 32g + 16(j/16) + (3(j%16) mod 16)
  constexpr int kOps = G == 1 ? 2 : 3;
  const int op = wv;
  if (op < kOps) {
    const int L = lane;
    const int r = L & 15, g = L >> 4;
    const int head = r >> 2;
    int digit;
    bool use = true;
    if (op == 0) {
      digit = r & 3;
      if (G == 2) use = g < 2;
    } else if (op == 1 && G == 1) {
      digit = 4 + (r & 3);
    } else if (op == 1) {
      digit = r & 3;
      use = g >= 2;
    } else {
      digit = 4 + (r & 1);
      use = (g >> 1) == ((r >> 1) & 1);
    }
    // field j at bits 6j.. of the operand's six dwords (little-endian)
    uint32_t bits[6] = {0, 0, 0, 0, 0, 0};
    if (use) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int ch = 32 * g + 16 * (j >> 4) + ((3 * (j & 15)) & 15);
        const uint32_t field = dig[head][ch][digit];
        const int bit = 6 * j;
        bits[bit >> 5] |= field << (bit & 31);
        if ((bit & 31) > 26) bits[(bit >> 5) + 1] |= field >> (32 - (bit & 31));
      }
    }
    uint32_t* dst = qa_tile + L * lane_stride;
#pragma unroll
    for (int d = 0; d < 6; ++d) dst[6 * op + d] = bits[d];
    if (op == 0)
      dst[scale_off] =
          static_cast<uint32_t>(min(max(kScaleOne + qe[head] + 2 - 4 * (r & 3), 1), 254));
    if (op == kOps - 1) {
      // low-digit operand: digit 4 + r%4 (group 128) or 4 + r%2 (group 64)
      const int dlo = G == 1 ? 4 + (r & 3) : 4 + (r & 1);
      dst[scale_off + 1] =
          static_cast<uint32_t>(min(max(kScaleOne + qe[head] + 2 - 4 * dlo, 1), 254));
    }
  }
}

// ---- BF16 windows ([OptR] "Assumptions & free parameters": 64 sink and 256
// recent tokens kept in BF16 beside the INT2 body).  Workgroups of the scan
// launch, dispatched ahead of its split workgroups, score the window tokens
// of one (sequence, query tile) against the unrotated query, subtracting
// q . mu as the centred body keys do (the same shift for every logit of the
// context), and write one partial (lse2, o) per query head in the unrotated
// basis; the merge folds it in after the inverse value rotation.  The window
// store already holds every token of the context when the scan runs.
//
// By the first 256 threads (further threads of a larger workgroup only pass
// the barriers).  Logits: one thread per window token, its key row read once for
// the four heads.  Softmax: one wave per head.  P.V: four groups of 64
// threads take every fourth token (a group's loads in flight together), a
// lane two channels of all four heads; the groups' sums meet in LDS.  lds:
// kWinLds floats of scratch; qin: the tile's raw query rows (zero past nh).
constexpr int kWinLds = kHT * kWindow + 4 * kHT * kHeadDim + 3 * kHT;
__device__ __forceinline__ void window_block(const uint16_t* __restrict__ win,
                                             const float* __restrict__ mu, int n, int b, int h,
                                             int qg, int nh, int Hq, int Hkv, float qscale,
                                             const float (*qin)[kHeadDim], float* lds,
                                             float* __restrict__ wpart) {
  float(*lg)[kWindow] = reinterpret_cast<float(*)[kWindow]>(lds);  // logits, then weights
  float(*acc)[kHT][kHeadDim] = reinterpret_cast<float(*)[kHT][kHeadDim]>(lds + kHT * kWindow);
  float(*hs)[kHT] = reinterpret_cast<float(*)[kHT]>(lds + kHT * kWindow + 4 * kHT * kHeadDim);
  const int tid = threadIdx.x;
  const bool act = tid < 256;
  const int lane = tid & 63;
  const int wv = (tid >> 6) & 3;
  const uint16_t* wk = win + (static_cast<size_t>(b) * Hkv + h) * 2 * kWindow * kHeadDim;
  const uint16_t* wvs = wk + kWindow * kHeadDim;
  const int nsk = min(kSink, n);
  const int rlo = max(kSink, n - kRecent);
  const int nw = nsk + max(0, n - rlo);
  auto slot_of = [&](int i) { return window_slot(i < nsk ? i : rlo + (i - nsk)); };

  if (act) {  // q . mu per head (wave wv)
    const float* muh = mu + static_cast<size_t>(h) * kHeadDim;
    float qm = qin[wv][lane] * muh[lane] + qin[wv][lane + 64] * muh[lane + 64];
    qm = wave_sum(qm);
    if (lane == 0) hs[0][wv] = qm;
  }
  __syncthreads();
  for (int i = tid; act && i < nw; i += 256) {
    // the query values are re-read from LDS for every token rather than held
    // in registers across the loop (512 of them)
    asm volatile("" ::: "memory");
    const uint4* kr = reinterpret_cast<const uint4*>(wk + slot_of(i) * kHeadDim);
    float dot[kHT] = {0.f, 0.f, 0.f, 0.f};
    // the key row in two halves of 64 channels
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint4 kw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kw[e] = kr[8 * half + e];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int c8 = 8 * half + c;
        const uint32_t w4[4] = {kw[c].x, kw[c].y, kw[c].z, kw[c].w};
        float kf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = __uint_as_float(w4[e] << 16);
          kf[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
        }
#pragma unroll
        for (int u = 0; u < kHT; ++u) {
          const float4 qa4 = *reinterpret_cast<const float4*>(&qin[u][8 * c8]);
          const float4 qb4 = *reinterpret_cast<const float4*>(&qin[u][8 * c8 + 4]);
          dot[u] = fmaf(qa4.x, kf[0], dot[u]);
          dot[u] = fmaf(qa4.y, kf[1], dot[u]);
          dot[u] = fmaf(qa4.z, kf[2], dot[u]);
          dot[u] = fmaf(qa4.w, kf[3], dot[u]);
          dot[u] = fmaf(qb4.x, kf[4], dot[u]);
          dot[u] = fmaf(qb4.y, kf[5], dot[u]);
          dot[u] = fmaf(qb4.z, kf[6], dot[u]);
          dot[u] = fmaf(qb4.w, kf[7], dot[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kHT; ++u) lg[u][i] = qscale * (dot[u] - hs[0][u]);
  }
  __syncthreads();
  if (act) {  // softmax of head wv
    float m = -INFINITY;
    for (int i = lane; i < nw; i += 64) m = fmaxf(m, lg[wv][i]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < nw; i += 64) {
      const float pi = exp2_hw(lg[wv][i] - m);
      lg[wv][i] = pi;
      l += pi;
    }
    l = wave_sum(l);
    if (lane == 0) {
      hs[1][wv] = m;
      hs[2][wv] = l;
    }
  }
  __syncthreads();
  if (act) {  // P.V: group wv takes tokens wv, wv + 4, ... (80 at most), 20 loads at a time
    constexpr int kChunk = 20;
    float a[kHT][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
    for (int i0 = wv; i0 < nw; i0 += 4 * kChunk) {
      uint32_t w2[kChunk];
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        const int i = min(i0 + 4 * r, nw - 1);
        w2[r] = reinterpret_cast<const uint32_t*>(wvs + slot_of(i) * kHeadDim)[lane];
      }
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        const int i = i0 + 4 * r;
        if (i < nw) {
          const float v0 = __uint_as_float(w2[r] << 16);
          const float v1 = __uint_as_float(w2[r] & 0xffff0000u);
#pragma unroll
          for (int u = 0; u < kHT; ++u) {
            a[u][0] = fmaf(lg[u][i], v0, a[u][0]);
            a[u][1] = fmaf(lg[u][i], v1, a[u][1]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kHT; ++u) {
      acc[wv][u][2 * lane] = a[u][0];
      acc[wv][u][2 * lane + 1] = a[u][1];
    }
  }
  __syncthreads();
  if (act && wv < nh) {  // head wv: the four groups' sums, normalised
    const int hq = h * (Hq / Hkv) + qg * kHT + wv;
    float* dst = wpart + (static_cast<size_t>(b) * Hq + hq) * kPartStride;
    const float inv = nw > 0 ? 1.0f / hs[2][wv] : 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = lane + 64 * e;
      dst[4 + c] = ((acc[0][wv][c] + acc[1][wv][c]) + (acc[2][wv][c] + acc[3][wv][c])) * inv;
    }
    if (lane == 0) dst[0] = nw > 0 ? hs[1][wv] + __log2f(hs[2][wv]) : kNegBig;
  }
}

// LDS the query-operand computation works in.
struct QScratch {
  float qin[kHT][kHeadDim];       // the tile's query rows
  float red[4][kHT][kHeadDim];    // split-K partial products
  uint8_t dig[kHT][kHeadDim][8];  // FP6 digit fields (sign | nibble)
  int qe[kHT];                    // per-head exponents
};

// What a thread of the operand computation loads: R_K rows [32 wv, 32 wv + 32)
// at columns 2 lane and 2 lane + 1 (one 8-byte load per row), and two
// channels of one query row.  Split from the arithmetic so that a split
// workgroup can issue these loads ahead of its cache DMAs (a wave's loads
// complete in order).
struct QLoads {
  float2 r[32];
  float v0, v1;
};

// The loads of query tile (h, qg) of sequence b (threads 0-255, with kEight
// threads 0-511 for R_K; further threads load nothing).  rot_k null: the
// keys were not rotated, q_r = q.
// kEight: a workgroup of eight or more waves splits the products over eight
// of them: wave w takes rows 32 (w % 4).. of R_K at the one column
// 64 (w / 4) + lane (in L.r[i].x), so each wave loads and multiplies half as
// much; the sums are the same, in the same order.
template <int G, bool kEight = false>
__device__ __forceinline__ void prologue_load(int h, int qg, int b, const void* __restrict__ q,
                                              bool q_bf16, const float* __restrict__ rot_k, int Hq,
                                              int Hg, QLoads& L) {
  const int tid = threadIdx.x;
  const bool act = tid < 256;
  const int lane = tid & 63;
  const int wv = (tid >> 6) & 3;
  const int nh = min(kHT, Hg - qg * kHT);
  if constexpr (kEight) {
    if (tid < 512 && rot_k != nullptr) {
      const float* R = rot_k + static_cast<size_t>(h) * kHeadDim * kHeadDim +
                       32 * wv * kHeadDim + 64 * ((tid >> 8) & 1) + lane;
#pragma unroll
      for (int i = 0; i < 32; ++i) L.r[i].x = R[i * kHeadDim];
    }
  } else if (act && rot_k != nullptr) {
    const float2* R = reinterpret_cast<const float2*>(
        rot_k + static_cast<size_t>(h) * kHeadDim * kHeadDim + 32 * wv * kHeadDim + 2 * lane);
#pragma unroll
    for (int i = 0; i < 32; ++i) L.r[i] = R[i * (kHeadDim / 2)];
  }
  // the tile's query rows (zero for rows past the KV head's query heads)
  L.v0 = 0.f;
  L.v1 = 0.f;
  const int hh = tid >> 6, c = (tid & 63) * 2;
  if (act && hh < nh) {
    const size_t qrow = (static_cast<size_t>(b) * Hq + h * Hg + qg * kHT + hh) * kHeadDim + c;
    if (q_bf16) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(q) + qrow);
      L.v0 = bf16_to_f32(static_cast<uint16_t>(u & 0xffffu));
      L.v1 = bf16_to_f32(static_cast<uint16_t>(u >> 16));
    } else {
      const float2 f = *reinterpret_cast<const float2*>(static_cast<const float*>(q) + qrow);
      L.v0 = f.x;
      L.v1 = f.y;
    }
  }
}

// The operand from the loads: threads 0-255 do the work (with kEight, the
// products: threads 0-511); further threads of a larger workgroup only pass
// the barriers (the fused decode step runs it in 1024-thread workgroups).
// q.R_K as a split-K product (quarter wv of the input channels, output
// channels 2 lane and 2 lane + 1, or with kEight channel 64 (w / 4) + lane,
// the four heads in one pass).  The A operands of lane L go to qa_tile + L * lane_stride (dwords
// 0-17, row scales at scale_off and scale_off + 1), the per-head group sums
// to qf_tile[0..3].
template <int G, bool kEight = false>
__device__ __forceinline__ void prologue_finish(const QLoads& L, bool ident, float qscale,
                                                QScratch& ls, uint32_t* qa_tile, int lane_stride,
                                                int scale_off, float4* qf_tile,
                                                float* qr_tile = nullptr) {
  const int tid = threadIdx.x;
  const bool act = tid < 256;
  const int lane = tid & 63;
  const int wv = (tid >> 6) & 3;
  if (act) {
    const int hh = tid >> 6, c = (tid & 63) * 2;
    ls.qin[hh][c] = L.v0;
    ls.qin[hh][c + 1] = L.v1;
  }
  __syncthreads();
  if (act && ident) {
    // quarter wv of the split-K sum holds channels 32wv..32wv+31 of q
#pragma unroll
    for (int hh = 0; hh < kHT; ++hh) {
      ls.red[wv][hh][lane] = (lane >> 5) == wv ? ls.qin[hh][lane] : 0.f;
      ls.red[wv][hh][lane + 64] = ((lane + 64) >> 5) == wv ? ls.qin[hh][lane + 64] : 0.f;
    }
  } else if (kEight && !ident && tid < 512) {
    const int c = 64 * ((tid >> 8) & 1) + lane;
#pragma unroll
    for (int hh = 0; hh < kHT; ++hh) {
      float a0 = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) a0 = fmaf(ls.qin[hh][32 * wv + i], L.r[i].x, a0);
      ls.red[wv][hh][c] = a0;
    }
  } else if (act) {
#pragma unroll
    for (int hh = 0; hh < kHT; ++hh) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float qi = ls.qin[hh][32 * wv + i];
        a0 = fmaf(qi, L.r[i].x, a0);
        a1 = fmaf(qi, L.r[i].y, a1);
      }
      ls.red[wv][hh][2 * lane] = a0;
      ls.red[wv][hh][2 * lane + 1] = a1;
    }
  }
  __syncthreads();
  if (act) prologue_digits<G>(qscale, ls.red, ls.dig, ls.qe, qf_tile, qr_tile);
  __syncthreads();
  if (act) prologue_pack<G>(ls.dig, ls.qe, qa_tile, lane_stride, scale_off);
}

// Both parts back to back (the products on eight waves: every workgroup
// that runs this has at least 512 threads).
template <int G>
__device__ __forceinline__ void prologue_compute(int h, int qg, int b, const void* __restrict__ q,
                                                 bool q_bf16, const float* __restrict__ rot_k,
                                                 int Hq, int Hkv, float qscale, QScratch& ls,
                                                 uint32_t* qa_tile, int lane_stride,
                                                 int scale_off, float4* qf_tile) {
  QLoads L;
  prologue_load<G, true>(h, qg, b, q, q_bf16, rot_k, Hq, Hq / Hkv, L);
  prologue_finish<G, true>(L, rot_k == nullptr, qscale, ls, qa_tile, lane_stride, scale_off,
                           qf_tile);
}

// The prologue kernel's view: its own LDS, the operand to the workspace.
template <bool kBf16, int G>
__device__ __forceinline__ void prologue_body(int hx, int b, const void* __restrict__ q,
                                              const float* __restrict__ rot_k, int Hq, int Hkv,
                                              int QG, float qscale, uint32_t* __restrict__ qa,
                                              float4* __restrict__ qf) {
  __shared__ __attribute__((aligned(16))) QScratch ls;
  const size_t tile = (static_cast<size_t>(b) * Hkv + hx / QG) * QG + hx % QG;
  prologue_compute<G>(hx / QG, hx % QG, b, q, kBf16, rot_k, Hq, Hkv, qscale, ls,
                      qa + tile * 64 * kQaDwords, kQaDwords, kQaScale, qf + tile * kHT);
}

template <bool kBf16, int G>
__global__ __launch_bounds__(512) void prologue_kernel(const void* __restrict__ q,
                                                       const float* __restrict__ rot_k, int Hq,
                                                       int Hkv, int QG, float qscale,
                                                       uint32_t* __restrict__ qa,
                                                       float4* __restrict__ qf) {
  prologue_body<kBf16, G>(blockIdx.x, blockIdx.y, q, rot_k, Hq, Hkv, QG, qscale, qa, qf);
}

// --------------------------------------------------------------------------- decode step
// The single-token append and the query rotation in one launch (both read
// R_K of the KV head; neither depends on the other).  grid (Hkv * (1 + QG),
// B), block 1024: x < Hkv appends the new token of KV head x, the others
// prepare query tile x - Hkv.
//
// kWin (BF16 windows): the append role first encodes the token that the new
// one displaces from the recent window (position p - 256, from its window
// copy) into the INT2 body, then writes the new token into the window.
template <bool kKvBf16, bool kQBf16, int G, bool kWin>
__global__ __launch_bounds__(1024) void step_prep_kernel(
    uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv, const int* __restrict__ block_table,
    int max_blocks, const int* __restrict__ start_pos, const void* __restrict__ k,
    const void* __restrict__ v, const float* __restrict__ mu, const float* __restrict__ rot_k,
    const float* __restrict__ rot_v, float clip_k, float clip_v, const void* __restrict__ q,
    int Hq, int QG, float qscale, uint32_t* __restrict__ qa, float4* __restrict__ qf,
    uint16_t* __restrict__ win) {
  const int b = blockIdx.y;
  if (static_cast<int>(blockIdx.x) < Hkv) {
    const int h = blockIdx.x;
    if constexpr (!kWin) {
      append_one_body<kKvBf16>(h, b, pages, num_blocks, Hkv, G, block_table, max_blocks,
                               start_pos, 0, token_row<kKvBf16>(k, b, h, Hkv),
                               token_row<kKvBf16>(v, b, h, Hkv), mu, rot_k, rot_v, clip_k,
                               clip_v);
    } else {
      const int p = start_pos[b];
      if (p < 0) return;
      uint16_t* wk = win + (static_cast<size_t>(b) * Hkv + h) * 2 * kWindow * kHeadDim;
      uint16_t* wv = wk + kWindow * kHeadDim;
      const int slot = window_slot(p);
      if (p >= kWindow)  // position p - 256 leaves the recent window for the body
        append_one_body<true>(h, b, pages, num_blocks, Hkv, G, block_table, max_blocks,
                              start_pos, -kRecent, wk + slot * kHeadDim, wv + slot * kHeadDim,
                              mu, rot_k, rot_v, clip_k, clip_v);
      __syncthreads();  // the displaced token has been read
      const int tid = threadIdx.x;
      if (tid < 2 * kHeadDim) {
        const int m = tid >> 7, c = tid & 127;
        const void* src = token_row<kKvBf16>(m ? v : k, b, h, Hkv);
        const uint16_t x = kKvBf16 ? static_cast<const uint16_t*>(src)[c]
                                   : f32_to_bf16(static_cast<const float*>(src)[c]);
        (m ? wv : wk)[slot * kHeadDim + c] = x;
      }
    }
  } else {
    prologue_body<kQBf16, G>(blockIdx.x - Hkv, b, q, rot_k, Hq, Hkv, QG, qscale, qa, qf);
  }
}

// --------------------------------------------------------------------------- scan
// ---- LDS ring: each wave keeps kDepth 2-page slices in flight, loaded with
// global->LDS DMA (no VGPRs held while in flight).  A slot holds a slice's two
// pages as [codes of page 0 (1024 B)][codes of page 1][(scale, zero) pairs of
// page 0 (128G B)][pairs of page 1], each part as laid out in the cache, so
// that for group 128 one 64-lane DMA fetches both pages' pairs: a slice is
// dma_per_slice<G>() DMA instructions, with no lane-dependent branch for the
// compiler to duplicate (the waits count them exactly).  Four slots, one per
// slice of an 8-page block, so that every slot address is a compile-time
// offset.  A slot is free once its slice has been read into registers, so
// three slices are in flight per wave: slice s of a block issues the slice
// three ahead into the slot read one slice before.  The P tile lives in the
// slot of the block's last slice, whose next DMA is issued by the next
// block's first slice, after the P.V products.
constexpr int kDepth = 3;
constexpr int kRing = 4;
constexpr int kSlotCodes1 = 1024;  // codes of a slot's second page
constexpr int kSlotPairs = 2048;   // (scale, zero) pairs of its first page
template <int G>
__host__ __device__ constexpr int dma_per_slice() {
  return G == 1 ? 3 : 4;
}
// Pages one workgroup may take: splits of at most 512 pages, the last split
// of a context taking up to half a split more.
constexpr int kMaxSplitPages = 768;
// P tile: 16 rows (4 heads x 4 digits) x 8 pages x 16 tokens of FP8 digit
// bytes, stored by token column (16 bytes per column: 8 rows of each half of
// the heads).  It lives in the ring slot of the block's last slice, which is
// free from the moment that slice is read until the next slice's DMA is
// issued.
constexpr int kPTile = 2048;

typedef __attribute__((address_space(3))) void lds_void_t;

// The compiler does not track when an LDS DMA lands: waits are explicit, and
// the memory clobber keeps LDS reads and DMA issues on their side of them.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)p));
}

// One slice into a ring slot (wide form): each page is a buffer resource
// built in scalar registers (base = the page, 1 record per byte up to the page
// size); the per-lane offsets are fixed.  Group 128 fetches each page's 32
// pair words with lanes 0-31 (the DMA writes lane L's word at slot base + 4L).
constexpr int kBufferWord3 = 0x00020000;  // raw byte buffer, gfx9 family

template <int G>
__device__ __forceinline__ void dma_slice(const uint8_t* page0, const uint8_t* page1,
                                          uint8_t* slot, uint32_t off16, uint32_t off4,
                                          bool lo_lane) {
  constexpr int PB = page_bytes_for_groups(G);
  const __amdgpu_buffer_rsrc_t r0 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(page0), 0, PB, kBufferWord3);
  const __amdgpu_buffer_rsrc_t r1 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(page1), 0, PB, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, (lds_void_t*)slot, 16, off16, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (lds_void_t*)(slot + kSlotCodes1), 16, off16, 0, 0,
                                           0);
  if (G == 2 || lo_lane) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, (lds_void_t*)(slot + kSlotPairs), 4, off4, 0, 0,
                                             0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (lds_void_t*)(slot + kSlotPairs + 128 * G), 4,
                                             off4, 0, 0, 0);
  }
}

// The same through one buffer resource over the whole cache (when it spans
// less than 4 GiB): a page is the scalar offset o0 or o1.  Group 128: lanes
// 0-31 fetch page 0's pair words and lanes 32-63 page 1's in one DMA
// (off4 = this lane's word offset inside a page).
template <int G>
__device__ __forceinline__ void dma_slice_at(__amdgpu_buffer_rsrc_t r, uint32_t o0, uint32_t o1,
                                             uint8_t* slot, uint32_t off16, uint32_t off4,
                                             bool lo_lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)slot, 16, off16, o0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(slot + kSlotCodes1), 16, off16, o1, 0,
                                           0);
  if constexpr (G == 2) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(slot + kSlotPairs), 4, off4, o0, 0,
                                             0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(slot + kSlotPairs + 256), 4, off4,
                                             o1, 0, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(slot + kSlotPairs), 4,
                                             off4 + (lo_lane ? o0 : o1), 0, 0, 0);
  }
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// This lane's share of one ring slot for the q.K products and the softmax:
// key codes of token t, channels 32kg..32kg+31, of both pages, and the (scale,
// zero) words of token t (K then V, each for both pages; .y = group 1).
// Inline assembly keeps the compiler's wait insertion, which cannot tell
// ring slots apart and would drain every pending DMA, out of the way; the
// caller has waited for this slot, and the block ends with lgkmcnt(0).
struct Slice {
  u32x2 kc0, kc1;
  uint2 szk0, szk1, szv0, szv1;
};

template <int G, int kOff>
__device__ __forceinline__ void read_slice(Slice& c, uint32_t ak, uint32_t as) {
  if constexpr (G == 2) {
    u32x2 s0, s1, s2, s3;
    asm volatile(
        "ds_read_b64 %0, %6 offset:%8\n"
        "ds_read_b64 %1, %6 offset:%9\n"
        "ds_read_b64 %2, %7 offset:%8\n"
        "ds_read_b64 %3, %7 offset:%10\n"
        "ds_read_b64 %4, %7 offset:%11\n"
        "ds_read_b64 %5, %7 offset:%12\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c.kc0), "=&v"(c.kc1), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
        : "v"(ak), "v"(as), "i"(kOff), "i"(kOff + kSlotCodes1), "i"(kOff + 128 * G),
          "i"(kOff + 64 * G), "i"(kOff + 192 * G)
        : "memory");
    c.szk0 = make_uint2(s0.x, s0.y);
    c.szk1 = make_uint2(s1.x, s1.y);
    c.szv0 = make_uint2(s2.x, s2.y);
    c.szv1 = make_uint2(s3.x, s3.y);
  } else {
    uint32_t s0, s1, s2, s3;
    asm volatile(
        "ds_read_b64 %0, %6 offset:%8\n"
        "ds_read_b64 %1, %6 offset:%9\n"
        "ds_read_b32 %2, %7 offset:%8\n"
        "ds_read_b32 %3, %7 offset:%10\n"
        "ds_read_b32 %4, %7 offset:%11\n"
        "ds_read_b32 %5, %7 offset:%12\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c.kc0), "=&v"(c.kc1), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
        : "v"(ak), "v"(as), "i"(kOff), "i"(kOff + kSlotCodes1), "i"(kOff + 128 * G),
          "i"(kOff + 64 * G), "i"(kOff + 192 * G)
        : "memory");
    c.szk0 = make_uint2(s0, s0);
    c.szk1 = make_uint2(s1, s1);
    c.szv0 = make_uint2(s2, s2);
    c.szv1 = make_uint2(s3, s3);
  }
}

// read_slice and read_ids8 under one wait (slice 0 of a block whose
// successor exists).
template <int G, int kOff>
__device__ __forceinline__ void read_slice_ids(Slice& c, uint32_t ak, uint32_t as, uint32_t ai,
                                               int (&id)[8]) {
  u32x4 x, y;
  if constexpr (G == 2) {
    u32x2 s0, s1, s2, s3;
    asm volatile(
        "ds_read_b64 %0, %8 offset:%11\n"
        "ds_read_b64 %1, %8 offset:%12\n"
        "ds_read_b64 %2, %9 offset:%11\n"
        "ds_read_b64 %3, %9 offset:%13\n"
        "ds_read_b64 %4, %9 offset:%14\n"
        "ds_read_b64 %5, %9 offset:%15\n"
        "ds_read_b128 %6, %10\n"
        "ds_read_b128 %7, %10 offset:16\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c.kc0), "=&v"(c.kc1), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3), "=&v"(x),
          "=&v"(y)
        : "v"(ak), "v"(as), "v"(ai), "i"(kOff), "i"(kOff + kSlotCodes1), "i"(kOff + 128 * G),
          "i"(kOff + 64 * G), "i"(kOff + 192 * G)
        : "memory");
    c.szk0 = make_uint2(s0.x, s0.y);
    c.szk1 = make_uint2(s1.x, s1.y);
    c.szv0 = make_uint2(s2.x, s2.y);
    c.szv1 = make_uint2(s3.x, s3.y);
  } else {
    uint32_t s0, s1, s2, s3;
    asm volatile(
        "ds_read_b64 %0, %8 offset:%11\n"
        "ds_read_b64 %1, %8 offset:%12\n"
        "ds_read_b32 %2, %9 offset:%11\n"
        "ds_read_b32 %3, %9 offset:%13\n"
        "ds_read_b32 %4, %9 offset:%14\n"
        "ds_read_b32 %5, %9 offset:%15\n"
        "ds_read_b128 %6, %10\n"
        "ds_read_b128 %7, %10 offset:16\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c.kc0), "=&v"(c.kc1), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3), "=&v"(x),
          "=&v"(y)
        : "v"(ak), "v"(as), "v"(ai), "i"(kOff), "i"(kOff + kSlotCodes1), "i"(kOff + 128 * G),
          "i"(kOff + 64 * G), "i"(kOff + 192 * G)
        : "memory");
    c.szk0 = make_uint2(s0, s0);
    c.szk1 = make_uint2(s1, s1);
    c.szv0 = make_uint2(s2, s2);
    c.szv1 = make_uint2(s3, s3);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    id[k] = __builtin_amdgcn_readfirstlane(static_cast<int>(x[k]));
    id[4 + k] = __builtin_amdgcn_readfirstlane(static_cast<int>(y[k]));
  }
}

// Eight block ids (one 8-page block of the workgroup's id table) into scalar
// registers; `ai` is the same LDS address in every lane.
__device__ __forceinline__ void read_ids8(uint32_t ai, int (&id)[8]) {
  u32x4 x, y;
  asm volatile(
      "ds_read_b128 %0, %2\n"
      "ds_read_b128 %1, %2 offset:16\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x), "=&v"(y)
      : "v"(ai)
      : "memory");
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    id[k] = __builtin_amdgcn_readfirstlane(static_cast<int>(x[k]));
    id[4 + k] = __builtin_amdgcn_readfirstlane(static_cast<int>(y[k]));
  }
}

// Value code words of channel 16*tau + n (tau = 0..7) of both pages of a slot:
// word position 8n + tau, i.e. 32 contiguous bytes per page.
template <int kOff>
__device__ __forceinline__ void read_vwords(u32x4 (&vw)[4], uint32_t av) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n"
      "ds_read_b128 %1, %4 offset:%6\n"
      "ds_read_b128 %2, %4 offset:%7\n"
      "ds_read_b128 %3, %4 offset:%8\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vw[0]), "=&v"(vw[1]), "=&v"(vw[2]), "=&v"(vw[3])
      : "v"(av), "i"(kOff), "i"(kOff + 16), "i"(kOff + kSlotCodes1), "i"(kOff + kSlotCodes1 + 16)
      : "memory");
}

// A lane's P-tile store for page kJ: the four digit bytes of its head, or
// the low two.
template <int kJ>
__device__ __forceinline__ void put_p32(uint32_t wbase, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(wbase), "v"(v), "i"(256 * kJ) : "memory");
}
template <int kJ>
__device__ __forceinline__ void put_p16(uint32_t wbase, uint32_t v) {
  asm volatile("ds_write_b16 %0, %1 offset:%2" ::"v"(wbase), "v"(v), "i"(256 * kJ) : "memory");
}

struct ScanState {
  float m, l, zs0, zs1;
  floatx4 acc[8];
};

// The P.V products of one 128-token block for output channel tiles
// [kT0, kT1).  w = p * s_V is fixed-point with 24 fraction bits under 2^e
// (per head and block, rounded to nearest), six 4-bit digits D0 (most
// significant) .. D5, an FP8 byte b being worth b * 2^-9.  The P tile holds,
// for each token column c (16 page + token) and half h of the heads, the
// eight bytes of rows 8h .. 8h + 7 (row 4 * head + k), 16 bytes per column:
// a lane writes its token's four digit bytes of one head with one 32-bit
// store, and each A operand (row r = lane%16; lane group g = lane/16 takes
// pages g and g + 4) comes back with four 8-byte transposing reads, which
// hand lane r byte r%8 of eight column chunks.  Row 4 * head + k holds D(3-k)
// in the first pass (row scale 2^(e - 4 + 4k), which also cancels the code
// operand's code/8) and D(5-k) for k < 2 in the second (2^(e - 12 + 4k));
// rows k = 2, 3 then still hold D1, D0, scaled by 2^-127 to nothing.  Two
// MFMAs per 16 output channels on one code operand.
template <int kT0, int kT1>
__device__ __forceinline__ void block_pv(ScanState& st, const float (&p)[8],
                                         const uint32_t (&szv)[8], uint8_t* ptile, int* pexp,
                                         const u32x4 (&vw)[4], int lane) {
  const int t = lane & 15, hl = lane >> 4;
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = p[j] * f16_lo_to_f32(szv[j]);
  float wmax = w[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) wmax = fmaxf(wmax, w[j]);
  wmax = row16_max(wmax);
  // w < 2^(e-1): w * 2^(24 - e) + 1/2 < 2^23, so rounding never carries out
  const int e = exp_above(wmax) + 1;
  const float sc = ldexpf(1.0f, 24 - e);
  uint32_t W[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) W[j] = static_cast<uint32_t>(fmaf(w[j], sc, 0.5f));
  // kept opaque: computed here, not held across the scan loop.  This lane's
  // dword of page 0: column t, half hl/2, bytes 4(hl%2) ..; page j at + 256 j
  uint32_t wbase = lds_addr(ptile) + 16 * t + 4 * hl;
  uint32_t hdr = lds_addr(reinterpret_cast<const uint8_t*>(pexp));
  asm volatile("" : "+v"(wbase), "+v"(hdr));
  if (t == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(hdr + 4 * hl), "v"(e) : "memory");
  const int r = lane & 15, g = lane >> 4;
  // transposing reads: lane (r, g) addresses the chunk of column 16g + r/2
  // (+ 8, + 64, + 72 for the other three), half r%2
  uint32_t ra = lds_addr(ptile) + 16 * (16 * g + (r >> 1)) + 8 * (r & 1);
  asm volatile("" : "+v"(ra));
  u32x2 h0, h1, h2, h3, l0, l1, l2, l3;
  int er;
  static_for<0, 8>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    // bytes [D3, D2, D1, D0]: the two upper bytes of W spread to nibbles
    const uint32_t t1 = __builtin_amdgcn_perm(W[j], W[j], 0x0C020C01u);
    const uint32_t hi = (t1 & 0x000F000Fu) | ((t1 << 4) & 0x0F000F00u);
    put_p32<j>(wbase, hi);
  });
  asm volatile(
      "ds_read_b64_tr_b8 %0, %4\n"
      "ds_read_b64_tr_b8 %1, %4 offset:128\n"
      "ds_read_b64_tr_b8 %2, %4 offset:1024\n"
      "ds_read_b64_tr_b8 %3, %4 offset:1152\n"
      "ds_read_b32 %5, %6\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3), "+v"(ra), "=&v"(er)
      : "v"(hdr + 4 * (r >> 2))
      : "memory");
  static_for<0, 8>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    // bytes [D5, D4] over the first pass's [D3, D2]
    const uint32_t lo = (W[j] & 0x0Fu) | ((W[j] << 4) & 0x0F00u);
    put_p16<j>(wbase, lo);
  });
  asm volatile(
      "ds_read_b64_tr_b8 %0, %4\n"
      "ds_read_b64_tr_b8 %1, %4 offset:128\n"
      "ds_read_b64_tr_b8 %2, %4 offset:1024\n"
      "ds_read_b64_tr_b8 %3, %4 offset:1152\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l0), "=&v"(l1), "=&v"(l2), "=&v"(l3), "+v"(ra)
      :
      : "memory");
  const int k = r & 3;
  const int sa_hi = min(max(kScaleOne + er - 4 + 4 * k, 1), 254);
  // rows k = 2, 3 of a head still hold D1, D0: the smallest E8M0 scale
  // (2^-127) takes their products below every accumulated value
  const int sa_lo = k < 2 ? min(max(kScaleOne + er - 12 + 4 * k, 1), 254) : 0;
  const v8i Ahi = {static_cast<int>(h0.x), static_cast<int>(h0.y), static_cast<int>(h1.x),
                   static_cast<int>(h1.y), static_cast<int>(h2.x), static_cast<int>(h2.y),
                   static_cast<int>(h3.x), static_cast<int>(h3.y)};
  const v8i Alo = {static_cast<int>(l0.x), static_cast<int>(l0.y), static_cast<int>(l1.x),
                   static_cast<int>(l1.y), static_cast<int>(l2.x), static_cast<int>(l2.y),
                   static_cast<int>(l3.x), static_cast<int>(l3.y)};
  // value words: vw[0..1] = page 2g, tiles 0-7; vw[2..3] = page 2g + 1
  const uint32_t p0[8] = {vw[0].x, vw[0].y, vw[0].z, vw[0].w, vw[1].x, vw[1].y, vw[1].z, vw[1].w};
  const uint32_t p1[8] = {vw[2].x, vw[2].y, vw[2].z, vw[2].w, vw[3].x, vw[3].y, vw[3].z, vw[3].w};
#pragma unroll
  for (int tau = kT0; tau < kT1; ++tau) {
    const v8i B = fp6_codes(p0[tau], p1[tau]);
    st.acc[tau] = mfma128<kFmtFp8, kFmtFp6>(Ahi, B, st.acc[tau], sa_hi);
    st.acc[tau] = mfma128<kFmtFp8, kFmtFp6>(Alo, B, st.acc[tau], sa_lo);
  }
}

// 1-D grid of n_win + S * Hkv * QG * B workgroups of 256 threads (or, where a
// workgroup takes two splits, see split_waves, ceil(S / 2) * Hkv * QG * B of
// 512), then the decode step's append workgroups.  With BF16 windows (kWin;
// n_win = 0 otherwise) the first n_win = Hkv * QG * B workgroups each score
// the window of one (query tile, sequence) and write its partial to wpart (q:
// the raw queries, bf16 when q_bf16); they are dispatched first and run beside
// the splits.  The rest are the splits: split x of a query tile covers body
// pages [x*spw, (x+1)*spw) (after the sink pages with windows), cut into
// 8-page blocks dealt to the split's four waves in turn.  Group 128 fits in
// 128 VGPRs (four waves per SIMD); group 64, with a third q.K operand and a
// second value group, gets up to 168 (three waves per SIMD) rather than spill
// inside the loop (a spill reload waits for every outstanding DMA).  kWide
// builds a buffer descriptor per page for caches of 4 GiB and more.
//
// kSelfQ: every split workgroup builds its query operand itself (from q and
// rot_k, with the prologue's arithmetic, so bit for bit the same operand)
// while its first slices are in flight, in ring slots the loop has not
// reached yet (2-3, or 3 with eight waves); otherwise the operand comes from
// qa/qf, written by the prologue (or the fused step's preparation) launch.
// The decode step's single-token append run in the scan launch (see
// split_kernel): the new tokens, and where the scan leaves what the merge
// needs to add them.  n_app == 0: no step.
struct StepTail {
  uint8_t* pages;        // the cache, written by the append workgroups
  const int* start_pos;  // [B] positions of the new tokens
  const void* k;         // [B][1][Hkv][128]
  const void* v;
  int kv_bf16;
  const float* mu;
  const float* rot_v;
  float clip_k, clip_v;
  float* deq;            // [B][Hkv][kDeqStride]: K, V dequantised (rotated), valid flag
  float* qr;             // [B][Hkv][4][128] rotated query x sm_scale x log2(e)
  int n_app;             // append workgroups at the end of the grid
};
constexpr int kDeqStride = 2 * kHeadDim + 4;

// Waves per split workgroup.  A workgroup that builds its query operand
// itself (group 128, no windows) takes two consecutive splits of its query
// tile, four waves each, and builds the operand once for both: half the
// workgroups load R_K (64 KB each, the largest read of the operand; every
// workgroup of a CU loads it at the same moment, ahead of its cache slices).
// Otherwise a workgroup is one split.
__host__ __device__ constexpr int split_waves(int G, bool win, bool self_q) {
  return (self_q && !win && G == 1) ? 8 : 4;
}

// The scan launch's divisors: y = Hkv * QG (query tiles of a sequence), sp
// (split workgroups of a tile), qg = QG, hkv = Hkv, spw; hg = Hq / Hkv.
struct ScanDivs {
  FastDiv y, sp, qg, hkv, spw;
  int hg;
};

// The merge launch's divisors: qg = QG, spw; hg = Hq / Hkv.  (The per-head
// merge keeps its one division: there the compiler fetched such constants
// with a second kernel-argument load behind a branch, a round trip longer
// than the division.)
struct MergeDivs {
  FastDiv qg, spw;
  int hg;
};

template <int G, bool kWide, bool kWin, bool kSelfQ>
__global__ __launch_bounds__(64 * split_waves(G, kWin, kSelfQ))
__attribute__((amdgpu_waves_per_eu(G == 1 ? 4 : 3, 4))) void
split_kernel(const uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv,
             const int* __restrict__ block_table, int max_blocks, const int* __restrict__ ctx_len,
             int max_ctx, int Hq, int QG, int spw, const uint32_t* __restrict__ qa,
             const float4* __restrict__ qf, float* __restrict__ part, int S,
             const uint16_t* __restrict__ wstore, int n_win, const void* __restrict__ q,
             int q_bf16, const float* __restrict__ mu, float qscale, float* __restrict__ wpart,
             const float* __restrict__ rot_k, StepTail step, ScanDivs dv) {
  constexpr int PB = page_bytes_for_groups(G);
  constexpr int kSlot = 2 * PB;
  constexpr int kW = split_waves(G, kWin, kSelfQ);  // waves
  constexpr int kPair = kW / 4;                     // splits
  // slot s of wave w at ring[s][w]: the slots 2-3 of all the waves are one
  // contiguous region, free from the start until the first block's loop
  constexpr int kSlotStride = kW * kSlot;
  static_assert(kPTile <= kSlot, "the P tile must fit in a ring slot");
  static_assert(kRing == 4 && kDepth == 3, "slots are the slices of a block; three in flight");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][kW][kSlot];
  // block ids of each split's pages
  __shared__ __attribute__((aligned(16))) int wids[kPair][kMaxSplitPages];
  __shared__ int pexp[kW][kHT];  // per-head digit exponents of the P tile
  __shared__ float cm[kW][kHT], cl[kW][kHT];
  const int Y = Hkv * QG;

  if (kWin && static_cast<int>(blockIdx.x) < n_win) {  // a window workgroup
    static_assert(sizeof(ring) >= (kHT * kHeadDim + kWinLds) * sizeof(float),
                  "window scratch lives in the ring");
    float(*qin)[kHeadDim] = reinterpret_cast<float(*)[kHeadDim]>(&ring[0][0][0]);
    const int b = dv.y.div(blockIdx.x), hy = blockIdx.x - b * Y;
    const int h = dv.qg.div(hy), qg = hy - h * QG;
    const int Hg = dv.hg;
    const int nh = min(kHT, Hg - qg * kHT);
    const int u = threadIdx.x >> 6, c = threadIdx.x & 63;
    const size_t qrow =
        (static_cast<size_t>(b) * Hq + h * Hg + qg * kHT + min(u, nh - 1)) * kHeadDim;
    float x0, x1;
    if (q_bf16) {
      const uint16_t* qp = static_cast<const uint16_t*>(q) + qrow;
      x0 = bf16_to_f32(qp[c]);
      x1 = bf16_to_f32(qp[c + 64]);
    } else {
      const float* qp = static_cast<const float*>(q) + qrow;
      x0 = qp[c];
      x1 = qp[c + 64];
    }
    qin[u][c] = u < nh ? x0 : 0.f;
    qin[u][c + 64] = u < nh ? x1 : 0.f;
    const int n = min(max(ctx_len[b], 0), max_ctx);
    __syncthreads();
    window_block(wstore, mu, n, b, h, qg, nh, Hq, Hkv, qscale, qin, &qin[kHT][0], wpart);
    return;
  }

  // Workgroups go to the eight XCDs round-robin in launch order, and each XCD
  // has its own L2.  Where the scan builds its operand, renumber the splits so
  // that every XCD takes one contiguous run of (query group, split) pairs: the
  // splits of a query tile then share one L2 copy of its R_K and query rows
  // instead of fetching them once per XCD.  Where the operand comes from the
  // workspace the splits keep launch order (the ragged group-64 batch of 64:
  // 188 -> 179 us): neighbouring workgroups, on neighbouring XCDs, then start
  // on the same sequence's pages together.  Consecutive jobs run over the KV
  // heads and query groups of one split first, so the KV heads of a sequence
  // read neighbouring slices of each block.
  // The decode step's appends (kSelfQ without windows: the scan builds its own
  // operand and needs no earlier launch) are the last n_app workgroups, one
  // per (sequence, KV head).  Dispatched after every split, they start as the
  // first splits finish, and the scan leaves the new tokens' slots out, so
  // they run in the launch's tail.  A split may read a page while its new
  // token's bytes change: it masks that slot, and the other codes in the
  // bytes it shares are rewritten as they were.
  const int n_app = (kSelfQ && !kWin) ? step.n_app : 0;
  const int n_wg = static_cast<int>(gridDim.x) - n_win - n_app;
  const int lin = static_cast<int>(blockIdx.x) - n_win;
  if constexpr (kSelfQ && !kWin) {
    if (lin >= n_wg) {
      const int a = lin - n_wg, hb = dv.hkv.div(a), ha = a - hb * Hkv;
      float* scratch = reinterpret_cast<float*>(&ring[0][0][0]);
      float* dq = step.deq + (static_cast<size_t>(hb) * Hkv + ha) * kDeqStride;
      const int pos = step.start_pos[hb];
      if (step.kv_bf16)
        append_one_256<true>(ha, hb, step.pages, num_blocks, Hkv, G, block_table, max_blocks, pos,
                             token_row<true>(step.k, hb, ha, Hkv),
                             token_row<true>(step.v, hb, ha, Hkv), step.mu, rot_k, step.rot_v,
                             step.clip_k, step.clip_v, scratch, dq);
      else
        append_one_256<false>(ha, hb, step.pages, num_blocks, Hkv, G, block_table, max_blocks,
                              pos, token_row<false>(step.k, hb, ha, Hkv),
                              token_row<false>(step.v, hb, ha, Hkv), step.mu, rot_k, step.rot_v,
                              step.clip_k, step.clip_v, scratch, dq);
      // whether the token was stored (a position outside the table or a
      // block id outside the cache stores nothing, and the merge skips it)
      if (threadIdx.x == 0) {
        const int bi = pos >= 0 && pos / kBlock < max_blocks
                           ? block_table[static_cast<size_t>(hb) * max_blocks + pos / kBlock]
                           : -1;
        dq[2 * kHeadDim] = (bi >= 0 && bi < num_blocks) ? 1.f : 0.f;
      }
      return;
    }
  }
  const int xcd = lin & 7;
  const int job = kSelfQ ? xcd * (n_wg >> 3) + min(xcd, n_wg & 7) + (lin >> 3) : lin;
  const int SP = (S + kPair - 1) / kPair;  // workgroups per query tile
  const int jy = dv.y.div(job);
  const int hy = job - jy * Y;
  const int b = dv.sp.div(jy);
  const int wgp = jy - b * SP;
  const int h = dv.qg.div(hy);
  const int qg = hy - h * QG;
  const int Hg = dv.hg;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this wave's split of the workgroup, and its place among the split's four
  const int half = kPair > 1 ? wave >> 2 : 0;
  const int lw = kPair > 1 ? wave & 3 : wave;
  const int ht = kPair > 1 ? threadIdx.x & 255 : threadIdx.x;
  const int wgs = kPair * wgp + half;  // the split (may be past the last one)
  // with BF16 windows the body starts after the sinks (a whole number of pages)
  constexpr bool win = kWin;
  const int lo_pages = win ? kSink / kBlock : 0;
  const int p_begin = lo_pages + wgs * spw;
  const int* row = block_table + static_cast<size_t>(b) * max_blocks;

  // Block ids, clamped into the cache (block ids past INT32_MAX cannot be
  // addressed by the table anyway).  They are loaded before the context
  // length is known, with indices clamped into the table row rather than
  // branched on, so that every load issues at once (entries past the range
  // are never used unmasked): lanes 0-7 take the wave's first block, whose
  // DMAs then wait for nothing else, and every thread up to three entries of
  // the range's id table, which goes to LDS.
  const int ctx_in = ctx_len[b];
  const int max_block = static_cast<int>(min(num_blocks, static_cast<int64_t>(0x7fffffff)) - 1);
  auto clamp_id = [&](int id) {
    return static_cast<int>(min(static_cast<uint32_t>(id), static_cast<uint32_t>(max_block)));
  };
  const int id_lane = row[min(p_begin + 8 * lw + (lane & 7), max_blocks - 1)];
  static_assert(kMaxSplitPages == 3 * 256, "three table entries per thread of a split");
  int idv[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) idv[k] = row[min(p_begin + ht + 256 * k, max_blocks - 1)];

  // The query operand is loaded next, and the ring's first slices are issued
  // once the context length is known; the operand is then waited for on each
  // path separately, so the wait counts only the loads ahead of the slices
  // (they complete in order and the slices stay in flight) and the loop never
  // waits on it again.
  const size_t hgi = (static_cast<size_t>(b) * Hkv + h) * QG + qg;
  const int t = lane & 15;
  const int hl = lane >> 4;
  uint4 q0 = make_uint4(0u, 0u, 0u, 0u), q1 = q0, q2 = q0, q3 = q0, q4 = q0, qsv = q0;
  float4 fq = make_float4(0.f, 0.f, 0.f, 0.f);
  // kSelfQ: R_K and the query rows for the operand, loaded here so that they
  // land ahead of the cache DMAs issued below (with the wide descriptor or the
  // window role the registers are short: loaded after the DMAs)
  constexpr bool kEarlyQ = kSelfQ && !kWide && !kWin;
  QLoads qload;
  if constexpr (kEarlyQ)
    prologue_load<G, (kPair > 1)>(h, qg, b, q, q_bf16 != 0, rot_k, Hq, Hg, qload);
  if constexpr (!kSelfQ) {
    const uint4* qap = reinterpret_cast<const uint4*>(qa + (hgi * 64 + lane) * kQaDwords);
    q0 = qap[0];
    q1 = qap[1];
    q2 = qap[2];
    if (G == 2) {
      q3 = qap[3];
      q4 = qap[4];
    }
    qsv = qap[kQaScale / 4];
    fq = qf[hgi * kHT + hl];
  }

  const int ctx = min(max(ctx_in, 0), max_ctx);
  const int hi_tok = win ? body_end(ctx) : ctx;  // tokens scanned: [lo_pages * 16, hi_tok)
  // with the step's appends in this launch the new token's slot is left out
  // (the merge adds the token) and the block holding it takes the masked path
  const int pex = n_app > 0 ? step.start_pos[b] : -1;
  const int n_pages = (hi_tok + kBlock - 1) / kBlock;
  const int ns_b = num_splits_fd(n_pages - lo_pages, spw, dv.spw);
  // a split past the tile's count, or starting past the context, has no pages
  // (the splits of a workgroup are consecutive: if its first has none, neither
  // has the second)
  if (kPair * wgp >= ns_b || lo_pages + kPair * wgp * spw >= n_pages) return;
  const bool has = kPair == 1 || (wgs < ns_b && p_begin < n_pages);
  const int p_end = !has ? p_begin : (wgs == ns_b - 1) ? n_pages : p_begin + spw;
  const int np = p_end - p_begin;  // at most kMaxSplitPages - 1 (split_pages <= 512)
  // 8-page blocks of this range; this wave's are lw, lw + 4, ...  Only the
  // range's last block can be short; its slices past the range are skipped.
  const int nblk = (np + 7) >> 3;
  const int nbw = lw < nblk ? (nblk - lw + 3) >> 2 : 0;
  const bool owns_last = nbw > 0 && ((nblk - 1 - lw) & 3) == 0;
  const int ns_last = owns_last ? min(4, (np - 8 * (nblk - 1) + 1) >> 1) : 4;
  const int nsl = nbw > 0 ? 4 * (nbw - 1) + ns_last : 0;
  // the table, padded with block 0 to whole 8-page blocks (padding pages are
  // masked out)
  const int np8 = (np + 7) & ~7;
  int idc[8];                             // ids of the current block's pages
  int idn[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // of the next block's
#pragma unroll
  for (int k = 0; k < 8; ++k) idc[k] = clamp_id(__builtin_amdgcn_readlane(id_lane, k));
  auto fill_table = [&]() {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int lp = ht + 256 * k;
      if (lp < np8) wids[half][lp] = lp < np ? clamp_id(idv[k]) : 0;
    }
  };

  uint8_t* myring = &ring[0][wave][0];
  // DMA lane offsets: 16 code bytes per lane; one (scale, zero) word per lane
  // (group 128: lanes 0-31 and 32-63 take the same words of the two pages)
  const uint32_t off16 = 16u * lane;
  const uint32_t off4 = kSzOff + 4u * static_cast<uint32_t>(G == 2 ? lane : (lane & 31));
  const bool lo_lane = lane < 32;
  // one descriptor over the whole cache (narrow form): page = scalar offset
  const uint32_t pstride = static_cast<uint32_t>(Hkv) * PB, hoff = static_cast<uint32_t>(h) * PB;
  const uint32_t cache_bytes =
      kWide ? 0u : static_cast<uint32_t>(static_cast<uint64_t>(num_blocks) * pstride);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(pages), 0, static_cast<int>(cache_bytes), kBufferWord3);
  auto issue = [&](uint8_t* slot, int b0, int b1) {
    if constexpr (kWide)
      dma_slice<G>(pages + (static_cast<int64_t>(b0) * Hkv + h) * PB,
                   pages + (static_cast<int64_t>(b1) * Hkv + h) * PB, slot, off16, off4, lo_lane);
    else
      dma_slice_at<G>(rsrc, static_cast<uint32_t>(b0) * pstride + hoff,
                      static_cast<uint32_t>(b1) * pstride + hoff, slot, off16, off4, lo_lane);
  };
  // LDS address of the ids of this wave's block m (the same in every lane)
  const uint32_t ids_base = lds_addr(reinterpret_cast<const uint8_t*>(&wids[half][0]));
  auto ids_addr = [&](int m) { return ids_base + 32u * static_cast<uint32_t>(lw + 4 * m); };

  // The operand passes through an empty asm on each path: the compiler waits
  // for it there, and afterwards sees it as defined by the asm, not by a
  // pending load.  Distinct texts keep the three from being merged.
  u32x4 qv0 = __builtin_bit_cast(u32x4, q0), qv1 = __builtin_bit_cast(u32x4, q1);
  u32x4 qv2 = __builtin_bit_cast(u32x4, q2), qv3 = __builtin_bit_cast(u32x4, q3);
  u32x4 qv4 = __builtin_bit_cast(u32x4, q4), qvs = __builtin_bit_cast(u32x4, qsv);
  float fqy = fq.y, fqz = fq.z;
#define KVQ_HOLD_Q(tag)                                                                        \
  asm volatile("; q operand " tag                                                              \
               : "+v"(qv0), "+v"(qv1), "+v"(qv2), "+v"(qv3), "+v"(qv4), "+v"(qvs), "+v"(fqy),  \
                 "+v"(fqz))
  // A workgroup of two splits builds its operand in slot 3 of its eight waves
  // (enough room), so a wave with more than one block sends slice 2 out with
  // the first two (with one block, whose slices all land at the start, that
  // was slower: batch 4 8K 12.7 against 12.1 us); otherwise the operand takes
  // slots 2-3 and slice 2 waits for it.
  constexpr bool kSlice2First = kSelfQ && kPair > 1;
  const bool early2 = kSlice2First && nsl > 4;
  if (early2) {
    issue(myring, idc[0], idc[1]);
    issue(myring + kSlotStride, idc[2], idc[3]);
    issue(myring + 2 * kSlotStride, idc[4], idc[5]);
    fill_table();
    KVQ_HOLD_Q("after three slices");
  } else if (nsl >= 2) {
    issue(myring, idc[0], idc[1]);
    issue(myring + kSlotStride, idc[2], idc[3]);
    fill_table();
    KVQ_HOLD_Q("after two slices");
  } else if (nsl == 1) {
    issue(myring, idc[0], idc[1]);
    fill_table();
    KVQ_HOLD_Q("after one slice");
  } else {
    fill_table();
    KVQ_HOLD_Q("alone");
  }
#undef KVQ_HOLD_Q
  if constexpr (kSelfQ) {
    // slots 2-3 (slot 3 with two splits) of every wave: the prologue's
    // scratch, then the operand of lane L at dwords 20L.. (over the partial
    // products, dead by then), the per-head group sums after the scratch
    uint8_t* free_lds = &ring[kSlice2First ? 3 : 2][0][0];
    static_assert(sizeof(QScratch) + kHT * sizeof(float4) <=
                      (kSlice2First ? 1 : 2) * kSlotStride,
                  "the operand's scratch fits in the free slots");
    static_assert(offsetof(QScratch, red) + 64 * kQaLds * 4 <= offsetof(QScratch, dig),
                  "the operand overwrites only the partial products");
    QScratch& ls = *reinterpret_cast<QScratch*>(free_lds);
    uint32_t* qa_s = reinterpret_cast<uint32_t*>(free_lds + offsetof(QScratch, red));
    float4* qf_s = reinterpret_cast<float4*>(free_lds + sizeof(QScratch));
    if constexpr (!kEarlyQ)
      prologue_load<G, (kPair > 1)>(h, qg, b, q, q_bf16 != 0, rot_k, Hq, Hg, qload);
    prologue_finish<G, (kPair > 1)>(
        qload, rot_k == nullptr, qscale, ls, qa_s, kQaLds, kQaLdsScale, qf_s,
        (n_app > 0 && wgp == 0) ? step.qr + hgi * kHT * kHeadDim : nullptr);
    __syncthreads();  // the operand is packed
    const uint32_t* mine = qa_s + lane * kQaLds;
    qv0 = u32x4{mine[0], mine[1], mine[2], mine[3]};
    qv1 = u32x4{mine[4], mine[5], mine[6], mine[7]};
    qv2 = u32x4{mine[8], mine[9], mine[10], mine[11]};
    if (G == 2) {
      qv3 = u32x4{mine[12], mine[13], mine[14], mine[15]};
      qv4 = u32x4{mine[16], mine[17], 0u, 0u};
    }
    qvs = u32x4{mine[kQaLdsScale], mine[kQaLdsScale + 1], 0u, 0u};
    fqy = qf_s[hl].y;
    fqz = qf_s[hl].z;
  }
  // the id table is complete (and the operand read before its slots refill)
  __syncthreads();
  if (!early2 && nsl >= 3) issue(myring + 2 * kSlotStride, idc[4], idc[5]);

  auto op6 = [](uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t e, uint32_t f) {
    return v8i{static_cast<int>(a), static_cast<int>(b), static_cast<int>(c), static_cast<int>(d),
               static_cast<int>(e), static_cast<int>(f), 0, 0};
  };
  const v8i qA0 = op6(qv0.x, qv0.y, qv0.z, qv0.w, qv1.x, qv1.y);
  const v8i qA1 = op6(qv1.z, qv1.w, qv2.x, qv2.y, qv2.z, qv2.w);
  const v8i qA2 = op6(qv3.x, qv3.y, qv3.z, qv3.w, qv4.x, qv4.y);
  const int qsc_hi = static_cast<int>(qvs.x);
  const int qsc_lo = static_cast<int>(qvs.y);
  const float sq0 = G == 1 ? fqy + fqz : fqy;
  const float sq1 = fqz;

  ScanState st;
  st.m = kNegBig;
  st.l = 0.f;
  st.zs0 = 0.f;
  st.zs1 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  u32x4 vw[4] = {};
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // this lane's LDS read addresses in slot 0 (other slots: immediate offsets)
  const uint32_t ring0 = lds_addr(myring);
  const uint32_t ak = ring0 + kKCodeOff + 32 * t + 8 * hl;
  const uint32_t as = ring0 + kSlotPairs + 4 * G * t;
  const uint32_t av = ring0 + kVCodeOff + 32 * t;

  // One 8-page block.  kFast: a block whose four slices all exist, each with
  // its successor two slices ahead to issue, and whose pages are all full (it
  // is neither the range's last block nor holds the context's last page):
  // no per-slice conditions.
  auto run_block = [&](auto fast, int bi) {
    constexpr bool kFast = decltype(fast)::value;
    const int pblk = p_begin + 8 * (lw + 4 * bi);
    float lg[8];
    uint2 szv[8];
    auto slice = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const int i = 4 * bi + s;
      if (kFast || i < nsl) {
        // slice i + 3: slice 3 of this block, then 0-2 of the next (into the
        // slot that slice i - 1 was read from)
        static_assert(kDepth == 3, "the slot schedule assumes three slices in flight");
        if (kFast || i + kDepth < nsl) {
          if constexpr (s == 0)
            issue(myring + 3 * kSlotStride, idc[6], idc[7]);
          else
            issue(myring + (s - 1) * kSlotStride, idn[2 * s - 2], idn[2 * s - 1]);
        }
        // slice i has landed once at most the DMAs of the slices behind it are pending
        if (kFast || i + 3 < nsl)
          wait_vmem<3 * dma_per_slice<G>()>();
        else if (i + 2 < nsl)
          wait_vmem<2 * dma_per_slice<G>()>();
        else if (i + 1 < nsl)
          wait_vmem<dma_per_slice<G>()>();
        else
          wait_vmem<0>();
        Slice c;
        // the next block's ids (two slices before its first DMA) with slice 0
        if constexpr (kFast && s == 0)
          read_slice_ids<G, s * kSlotStride>(c, ak, as, ids_addr(bi + 1), idn);
        else
          read_slice<G, s * kSlotStride>(c, ak, as);
        if (hl == s) read_vwords<s * kSlotStride>(vw, av);
        if (!kFast && s == 0 && bi + 1 < nbw) read_ids8(ids_addr(bi + 1), idn);

        // q.K: D[4*head + digit][token t]; the digit rows add up in-lane
        const v8i k0 = fp6_codes(c.kc0.x, c.kc0.y);
        const v8i k1 = fp6_codes(c.kc1.x, c.kc1.y);
        float l0, l1;
        if constexpr (G == 1) {
          // high digits, then low digits accumulated onto them
          floatx4 d0 = mfma128<kFmtFp6, kFmtFp6>(qA0, k0, zero4, qsc_hi);
          floatx4 d1 = mfma128<kFmtFp6, kFmtFp6>(qA0, k1, zero4, qsc_hi);
          d0 = mfma128<kFmtFp6, kFmtFp6>(qA1, k0, d0, qsc_lo);
          d1 = mfma128<kFmtFp6, kFmtFp6>(qA1, k1, d1, qsc_lo);
          const float D0 = (d0[0] + d0[1]) + (d0[2] + d0[3]);
          const float D1 = (d1[0] + d1[1]) + (d1[2] + d1[3]);
          // logit = s_K sum(x code) + z_K sum(x)
          l0 = fmaf(f16_lo_to_f32(c.szk0.x), D0, f16_hi_to_f32(c.szk0.x) * sq0);
          l1 = fmaf(f16_lo_to_f32(c.szk1.x), D1, f16_hi_to_f32(c.szk1.x) * sq0);
        } else {
          // group 0: high rows of qA0 plus low rows 0-1 of qA2; group 1: qA1
          // plus qA2 rows 2-3.  Page by page, to keep few results live.
          auto logit2 = [&](const v8i& kb, uint2 szk) {
            const floatx4 a = mfma128<kFmtFp6, kFmtFp6>(qA0, kb, zero4, qsc_hi);
            const floatx4 bb = mfma128<kFmtFp6, kFmtFp6>(qA1, kb, zero4, qsc_hi);
            const floatx4 cc = mfma128<kFmtFp6, kFmtFp6>(qA2, kb, zero4, qsc_lo);
            const float D = ((a[0] + a[1]) + (a[2] + a[3])) + (cc[0] + cc[1]);
            const float E = ((bb[0] + bb[1]) + (bb[2] + bb[3])) + (cc[2] + cc[3]);
            return fmaf(f16_lo_to_f32(szk.x), D, f16_hi_to_f32(szk.x) * sq0) +
                   fmaf(f16_lo_to_f32(szk.y), E, f16_hi_to_f32(szk.y) * sq1);
          };
          l0 = logit2(k0, c.szk0);
          l1 = logit2(k1, c.szk1);
        }
        // the logits are complete before the next slice's reads: otherwise the
        // compiler sinks the q.K products to the softmax, holding every
        // slice's code operands at once
        asm volatile("" : "+v"(l0), "+v"(l1));
        if constexpr (kFast) {
          lg[2 * s] = l0;
          lg[2 * s + 1] = l1;
          szv[2 * s] = c.szv0;
          szv[2 * s + 1] = c.szv1;
        } else {
          const int pg = pblk + 2 * s;
          const int pos = pg * kBlock + t;
          const bool v0 = pos < hi_tok && pos != pex;
          const bool v1 = pg + 1 < p_end && pos + kBlock < hi_tok && pos + kBlock != pex;
          lg[2 * s] = v0 ? l0 : -INFINITY;
          lg[2 * s + 1] = v1 ? l1 : -INFINITY;
          // slots past the context hold arbitrary bytes (possibly NaN as fp16):
          // their value scale and zero are replaced, not multiplied by p = 0
          szv[2 * s] = v0 ? c.szv0 : make_uint2(0u, 0u);
          szv[2 * s + 1] = v1 ? c.szv1 : make_uint2(0u, 0u);
        }
      } else {
        lg[2 * s] = -INFINITY;
        lg[2 * s + 1] = -INFINITY;
        szv[2 * s] = make_uint2(0u, 0u);
        szv[2 * s + 1] = make_uint2(0u, 0u);
      }
    };
    // the scheduler keeps each slice's work between its reads and the next
    // slice's (interleaving slices only raises register pressure)
    slice(Const<int, 0>{});
    __builtin_amdgcn_sched_barrier(0);
    slice(Const<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    slice(Const<int, 2>{});
    __builtin_amdgcn_sched_barrier(0);
    slice(Const<int, 3>{});
    __builtin_amdgcn_sched_barrier(0);

    // ---- online softmax over the block (base 2).  The running maximum is
    // raised only when the block's exceeds it by more than 2^kLazy: weights up
    // to 2^kLazy are exact in the fixed-point P digits and harmless in fp32,
    // and the accumulators are rescaled far less often.
    float mb = lg[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mb = fmaxf(mb, lg[j]);
    mb = row16_max(mb);
    if (__any(mb > st.m + kLazy)) {
      const float mnew = fmaxf(st.m, mb);
      const float alpha = exp2_hw(st.m - mnew);
#pragma unroll
      for (int j = 0; j < 8; ++j) st.acc[j] *= alpha;
      st.l *= alpha;
      st.zs0 *= alpha;
      st.zs1 *= alpha;
      st.m = mnew;
    }
    float p[8];
    uint32_t sz0[8], sz1[8];
    float lsum = 0.f, z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = exp2_hw(lg[j] - st.m);
      lsum += p[j];
      sz0[j] = szv[j].x;
      sz1[j] = szv[j].y;
      z0 = fmaf(p[j], f16_hi_to_f32(sz0[j]), z0);
      if constexpr (G == 2) z1 = fmaf(p[j], f16_hi_to_f32(sz1[j]), z1);
    }
    st.l += lsum;
    st.zs0 += z0;
    st.zs1 += z1;
    // slot 3: read above; the DMAs in flight target slots 0-2
    uint8_t* ptile = myring + 3 * kSlotStride;
    if constexpr (G == 1) {
      block_pv<0, 8>(st, p, sz0, ptile, pexp[wave], vw, lane);
    } else {
      block_pv<0, 4>(st, p, sz0, ptile, pexp[wave], vw, lane);
      block_pv<4, 8>(st, p, sz1, ptile, pexp[wave], vw, lane);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) idc[k] = idn[k];
  };
  int nfast = nsl >= 4 + kDepth ? (nsl - 4 - kDepth) / 4 + 1 : 0;
  if (pex >= 0) {
    const int rel = pex / kBlock - p_begin;  // page of the new token in this range
    if (rel >= 0 && rel < np && ((rel >> 3) & 3) == lw) nfast = min(nfast, (rel >> 3) >> 2);
  }
  int bi = 0;
  for (; bi < nfast; ++bi) run_block(Const<bool, true>{}, bi);
  for (; bi < nbw; ++bi) run_block(Const<bool, false>{}, bi);

  // ---- per-wave finish: reduce row sums, form unnormalised outputs
  const float l = row16_sum(st.l);
  const float zs0 = row16_sum(st.zs0);
  const float zs1 = G == 2 ? row16_sum(st.zs1) : zs0;
  const int n = lane & 15;
  __syncthreads();  // every wave is done with its ring; reuse it for the combine
  float(*co)[kHT][kHeadDim] = reinterpret_cast<float(*)[kHT][kHeadDim]>(&ring[0][0][0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // digit rows add up to sum(w code)
    const floatx4 a = st.acc[j];
    co[wave][hl][16 * j + n] = ((a[0] + a[1]) + (a[2] + a[3])) + (j < 4 ? zs0 : zs1);
  }
  if (n == 0) {
    cm[wave][hl] = st.m;
    cl[wave][hl] = l;
  }
  __syncthreads();

  // ---- combine each split's 4 waves: thread -> (split tid/256, head
  // (tid/64)%4, channels c, c + 64)
  const int ch = (threadIdx.x >> 6) & 3;
  const int cc = threadIdx.x & 63;
  const int w0 = 4 * half;
  const int hloc = qg * kHT + ch;
  const int nh = min(kHT, Hg - qg * kHT);
  if (has && ch < nh) {
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, cm[w0 + w][ch]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = exp2_hw(cm[w0 + w][ch] - M);  // 0 for a wave that saw no token
      L += a * cl[w0 + w][ch];
      o0 += a * co[w0 + w][ch][cc];
      o1 += a * co[w0 + w][ch][cc + 64];
    }
    const int hq = h * Hg + hloc;
    float* dst = part + ((static_cast<size_t>(b) * Hq + hq) * S + wgs) * kPartStride;
    // a split whose only token is the step's new one saw nothing
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    dst[4 + cc] = o0 * inv;
    dst[4 + cc + 64] = o1 * inv;
    if (cc == 0) dst[0] = L > 0.f ? M + __log2f(L) : kNegBig;
  }
}

// ---- merge: log-sum-exp merge of the ns partials of the nh query heads of
// one head tile, then o = o_r * R_V[h]^T.  grid (Hkv * QG, B), block 1024.
// Latency-bound, so every load is issued before the first one is used:
//   - thread (j = tid/8, part = tid%8) loads its sixteen entries of row j of
//     R_V for the rotation;
//   - thread (head u = tid/256, half = lane/32, channel c = 32 ((tid/64)%4) +
//     lane%32) loads channel c of splits half, half + 2, ... (kMS of them
//     per round, below; the first two rounds at once), and lane l of each
//     wave the lse of split l.
// Each wave of head u then reduces the head's maximum lse and weight sum over
// the splits itself; lane l's term of the sum, the weight of split l, is what
// the wave's other lanes read from it for that split (one exponential per
// lane, not one per split).  The two halves of a channel meet by a lane swap,
// so one barrier (the channel sums into LDS) separates the merge from the
// rotation.
// kMS: splits per thread and round (two halves: 2 kMS per round): 16, or 4
// where a tile has at most 16 splits (the first two rounds' loads are issued
// together, and the smaller register count lets two workgroups share a CU),
// so that a thread issues few loads that only repeat the last split's (the
// loads are unconditional, the split index clamped).  The sums are the same
// either way (each half's splits in order).
constexpr int kMergeSplits = 16;

// kStep: the decode step's new token of (sequence, KV head), left out by the
// scan and appended in its launch (one query tile per KV head), joins as one
// more partial: its logit is the scan's float32 rotated query (qr) against the
// dequantised new key (each wave forms it: channels lane and lane + 64, two
// wave sums), its output the dequantised new value (deq).
template <bool kStep, int kMS>
__global__ __launch_bounds__(1024) void merge_kernel(const float* __restrict__ part,
                                                     const int* __restrict__ ctx_len, int max_ctx,
                                                     int Hq, int Hkv, int QG, int spw, int S,
                                                     const float* __restrict__ rot_v,
                                                     float* __restrict__ out,
                                                     const float* __restrict__ wpart,
                                                     const int* __restrict__ new_pos,
                                                     const float* __restrict__ deq,
                                                     const float* __restrict__ qr,
                                                     MergeDivs md) {
  __shared__ __attribute__((aligned(16))) float osum[kHT][kHeadDim];  // both halves
  __shared__ float hinv[kHT];  // 1 / (weight sum) per head
  __shared__ float hwin[kHT];  // the window partial's share of each head's output
  const int h = md.qg.div(blockIdx.x);
  const int qg = blockIdx.x - h * QG;
  const int b = blockIdx.y;
  const int Hg = md.hg;
  const int nh = min(kHT, Hg - qg * kHT);
  const int tid = threadIdx.x;
  const int j = tid >> 3, part8 = tid & 7;
  // input channels 4 part + 32 i4 + (0..3): eight lanes read 128 contiguous bytes
  // rot_v null: the value rotation is folded into the caller's weights and
  // the output stays in the rotated basis
  const bool rotate_out = rot_v != nullptr;
  float4 rr[4] = {};
  if (rotate_out) {
    const float4* R = reinterpret_cast<const float4*>(
        rot_v + (static_cast<size_t>(h) * kHeadDim + j) * kHeadDim + 4 * part8);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) rr[i4] = R[8 * i4];
  }
  const int u = tid >> 8, lane = tid & 63, half = lane >> 5;
  const int c = 32 * ((tid >> 6) & 3) + (lane & 31);
  const size_t row0 = static_cast<size_t>(b) * Hq + h * Hg + qg * kHT;
  const float* p = part + (row0 + min(u, nh - 1)) * S * kPartStride;
  const int ctx_in = ctx_len[b];
  float dk0 = 0.f, dk1 = 0.f, q0 = 0.f, q1 = 0.f, dv = 0.f, dflag = 0.f;
  int pn = -1;
  if constexpr (kStep) {
    const float* dq = deq + (static_cast<size_t>(b) * Hkv + h) * kDeqStride;
    const float* qq = qr + ((static_cast<size_t>(b) * Hkv + h) * kHT + u) * kHeadDim;
    dk0 = dq[lane];
    dk1 = dq[lane + 64];
    q0 = qq[lane];
    q1 = qq[lane + 64];
    dv = dq[kHeadDim + c];
    dflag = dq[2 * kHeadDim];
    pn = new_pos[b];
  }
  // Loaded before the context length (and so the split count) is known, for
  // the S allocated splits; entries of splits past the count are never used.
  const float lse_l = p[min(lane, S - 1) * kPartStride];
  float xv[kMS], xw[kMS], lv[kMS];
  // unconditional loads with the split index clamped (a guarded load becomes a
  // branch whose result copy waits for it, serialising the round)
  auto load_x = [&](int r, float(&x)[kMS]) {
#pragma unroll
    for (int k = 0; k < kMS; ++k)
      x[k] = p[min(2 * (kMS * r + k) + half, S - 1) * kPartStride + 4 + c];
  };
  load_x(0, xv);
  if (S > 2 * kMS) load_x(1, xw);  // S: the same in every thread
  const int ctx = min(max(ctx_in, 0), max_ctx);
  // kStep: head u's new-token logit (log2 units); kNegBig: not attended
  float lse_n = kNegBig;
  if constexpr (kStep) {
    const float x0 = wave_sum(q0 * dk0);
    const float x1 = wave_sum(q1 * dk1);
    if (pn >= 0 && pn < ctx && dflag != 0.f) lse_n = x0 + x1;
  }
  // the window partial's lse, and the window output this thread adds
  const float lse_w = wpart ? wpart[(row0 + min(u, nh - 1)) * kPartStride] : kNegBig;
  const float wv = wpart ? wpart[(row0 + min(part8 & 3, nh - 1)) * kPartStride + 4 + j] : 0.f;
  // with BF16 windows (wpart != null) the splits cover the body only
  const int lo_pages = wpart ? kSink / kBlock : 0;
  const int hi_tok = wpart ? body_end(ctx) : ctx;
  const int ns = num_splits_fd((hi_tok + kBlock - 1) / kBlock - lo_pages, spw, md.spw);
  if (ns == 0) {  // no body: the window's output, or zero for an empty context
    if (half == 0 && u < nh) {
      const size_t row = row0 + u;
      out[row * kHeadDim + c] = wpart ? wpart[row * kPartStride + 4 + c] : 0.f;
    }
    return;
  }

  // head u's maximum lse and weight sum over the ns splits (every wave of the
  // head computes them), with the window partial's
  float M = lane < ns ? lse_l : -INFINITY;
  for (int s = lane + 64; s < ns; s += 64) M = fmaxf(M, p[s * kPartStride]);
  M = wave_max(M);
  M = fmaxf(M, lse_w);
  M = fmaxf(M, lse_n);
  const float wl = lane < ns ? exp2_hw(lse_l - M) : 0.f;  // the weight of split `lane`
  float W = wl;
  for (int s = lane + 64; s < ns; s += 64) W += exp2_hw(p[s * kPartStride] - M);
  W = wave_sum(W);
  const float a_w = exp2_hw(lse_w - M);  // 0 without windows
  W += a_w;
  const float a_n = (kStep && lse_n > kNegBig) ? exp2_hw(lse_n - M) : 0.f;
  W += a_n;

  // channel c over this half's splits, a round at a time (one round covers
  // 32 splits); a split past the count contributes nothing (its stale values
  // are never multiplied).  The weight of split s < 64 is lane s's wl.
  float acc = 0.f;
  auto wgt_of = [&](int s) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s));
  };
  const int nr = (ns + 2 * kMS - 1) / (2 * kMS);
#pragma unroll
  for (int k = 0; k < kMS; ++k) {
    // the two halves of the wave take splits 2k and 2k + 1
    const int s0 = 2 * k;
    const float w0 = wgt_of(s0), w1 = wgt_of(s0 + 1);
    const int s = s0 + half;
    if (s < ns) acc = fmaf(half ? w1 : w0, xv[k], acc);
  }
  if (nr > 1) {
#pragma unroll
    for (int k = 0; k < kMS; ++k) {
      const int s0 = 2 * (kMS + k);
      const float w0 = wgt_of(s0), w1 = wgt_of(s0 + 1);
      const int s = s0 + half;
      if (s < ns) acc = fmaf(half ? w1 : w0, xw[k], acc);
    }
  }
  for (int r = 2; r < nr; ++r) {
    load_x(r, xv);
#pragma unroll
    for (int k = 0; k < kMS; ++k)
      lv[k] = p[min(2 * (kMS * r + k) + half, S - 1) * kPartStride];
#pragma unroll
    for (int k = 0; k < kMS; ++k) {
      const int s = 2 * (kMS * r + k) + half;
      if (s < ns) acc = fmaf(exp2_hw(lv[k] - M), xv[k], acc);
    }
  }
  if (kStep && half == 0 && a_n > 0.f) acc = fmaf(a_n, dv, acc);
  // the two halves of channel c: lanes l and l + 32 (the even splits' sum first)
  const float other = shfl_xor(acc, 32);
  if (half == 0) osum[u][c] = acc + other;
  if ((tid & 255) == 0) {
    const float inv = 1.0f / W;
    hinv[u] = inv;
    hwin[u] = a_w * inv;
  }
  __syncthreads();

  if (!rotate_out) {
    // thread (j, part) with part = head < nh writes channel j of that head
    if (part8 < nh) {
      const size_t row = row0 + part8;
      out[row * kHeadDim + j] = fmaf(hwin[part8], wv, osum[part8][j] * hinv[part8]);
    }
    return;
  }
  // o * R_V^T: thread (j, part) over input channels 4 part + 32 i4 + (0..3)
  // for the four heads, then a sum over the eight parts (eight adjacent lanes)
  float o[kHT] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 r = rr[i4];
    const int i = 4 * part8 + 32 * i4;
#pragma unroll
    for (int uu = 0; uu < kHT; ++uu) {
      const float4 x = *reinterpret_cast<const float4*>(&osum[uu][i]);
      o[uu] = fmaf(x.x, r.x, fmaf(x.y, r.y, fmaf(x.z, r.z, fmaf(x.w, r.w, o[uu]))));
    }
  }
  // quad_perm [1,0,3,2], [2,3,0,1], then row_half_mirror (lane i and 7 - i
  // of each eight hold the two quads' sums)
#pragma unroll
  for (int uu = 0; uu < kHT; ++uu) {
    o[uu] += dpp<0xb1>(o[uu]);
    o[uu] += dpp<0x4e>(o[uu]);
    o[uu] += dpp<0x141>(o[uu]);
  }
#pragma unroll
  for (int uu = 0; uu < kHT; ++uu) {
    if (part8 == uu && uu < nh) {
      const size_t row = row0 + uu;
      out[row * kHeadDim + j] = fmaf(hwin[uu], wv, o[uu] * hinv[uu]);
    }
  }
}

// ---- merge of one query head per workgroup, for small grids without windows
// (batch-1 long contexts, where one workgroup per KV head would leave most
// CUs idle).  grid (Hq, B), block 256.  Lane l of every wave loads the lse of
// split l (more in a loop), so every wave forms the head's maximum and weight
// sum (lane l's term, the weight of split l, is read from it for that split);
// wave w adds up splits w, w + 4, ... for channels lane and lane + 64,
// all of its loads issued at once, and the four waves meet in LDS.  Then
// thread (row j = tid / 2, half) takes 64 columns of R_V row j, loaded at the
// start, and the two halves add by a DPP step.
// kHMS: splits per wave and round: 16, or 4 where a head has at most 16
// splits (no loads that only repeat the last split's), or 32 where it has
// 65-128: then every load, the second 64 splits' lse included, is issued
// before the context length is known.
constexpr int kHeadMergeSplits = 16;

template <int kHMS>
__global__ __launch_bounds__(256) void merge_head_kernel(const float* __restrict__ part,
                                                         const int* __restrict__ ctx_len,
                                                         int max_ctx, int Hq, int Hkv, int spw,
                                                         int S, const float* __restrict__ rot_v,
                                                         float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float osum[4][kHeadDim];
  __shared__ __attribute__((aligned(16))) float ofin[kHeadDim];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int h = hq / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = tid >> 1, half = tid & 1;
  const bool rotate_out = rot_v != nullptr;
  float4 rr[16] = {};
  if (rotate_out) {
    const float4* R = reinterpret_cast<const float4*>(
        rot_v + (static_cast<size_t>(h) * kHeadDim + j) * kHeadDim + 64 * half);
#pragma unroll
    for (int m = 0; m < 16; ++m) rr[m] = R[m];
  }
  const size_t row = static_cast<size_t>(b) * Hq + hq;
  const float* p = part + row * S * kPartStride;
  const int ctx_in = ctx_len[b];
  const float lse_l = p[min(lane, S - 1) * kPartStride];
  constexpr bool kLse2 = kHMS == 32;  // lane l also holds split l + 64's lse
  const float lse_h = kLse2 ? p[min(lane + 64, S - 1) * kPartStride] : 0.f;
  float x0[kHMS], x1[kHMS];
  auto load_round = [&](int r) {
#pragma unroll
    for (int k = 0; k < kHMS; ++k) {
      const float* e = p + min(4 * (kHMS * r + k) + w, S - 1) * kPartStride;
      x0[k] = e[4 + lane];
      x1[k] = e[4 + lane + 64];
    }
  };
  load_round(0);
  const int ctx = min(max(ctx_in, 0), max_ctx);
  const int ns = num_splits((ctx + kBlock - 1) / kBlock, spw);
  if (ns == 0) {
    if (tid < kHeadDim) out[row * kHeadDim + tid] = 0.f;
    return;
  }
  float M = lane < ns ? lse_l : -INFINITY;
  if (kLse2 && lane + 64 < ns) M = fmaxf(M, lse_h);
  for (int s = lane + (kLse2 ? 128 : 64); s < ns; s += 64) M = fmaxf(M, p[s * kPartStride]);
  M = wave_max(M);
  const float wl = lane < ns ? exp2_hw(lse_l - M) : 0.f;  // the weight of split `lane`
  const float wh = kLse2 && lane + 64 < ns ? exp2_hw(lse_h - M) : 0.f;  // of split lane + 64
  float W = wl + wh;
  for (int s = lane + (kLse2 ? 128 : 64); s < ns; s += 64) W += exp2_hw(p[s * kPartStride] - M);
  W = wave_sum(W);
  // this wave's splits; the weight of split s < 64 is lane s's wl (s < 128:
  // lane s - 64's wh)
  auto wgt_of = [&](int s) {
    if (s < 64)
      return __builtin_bit_cast(float,
                                __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s));
    if (kLse2 && s < 128)
      return __builtin_bit_cast(float,
                                __builtin_amdgcn_readlane(__builtin_bit_cast(int, wh), s - 64));
    return exp2_hw(p[s * kPartStride] - M);
  };
  float a0 = 0.f, a1 = 0.f;
  const int nr = (ns + 4 * kHMS - 1) / (4 * kHMS);
  for (int r = 0; r < nr; ++r) {
    if (r > 0) load_round(r);
#pragma unroll
    for (int k = 0; k < kHMS; ++k) {
      const int s = 4 * (kHMS * r + k) + w;
      if (s < ns) {
        const float wgt = wgt_of(s);
        a0 = fmaf(wgt, x0[k], a0);
        a1 = fmaf(wgt, x1[k], a1);
      }
    }
  }
  osum[w][lane] = a0;
  osum[w][lane + 64] = a1;
  __syncthreads();
  const float inv = 1.0f / W;
  if (!rotate_out) {
    if (tid < kHeadDim)
      out[row * kHeadDim + tid] =
          (((osum[0][tid] + osum[1][tid]) + osum[2][tid]) + osum[3][tid]) * inv;
    return;
  }
  if (tid < kHeadDim)
    ofin[tid] = (((osum[0][tid] + osum[1][tid]) + osum[2][tid]) + osum[3][tid]) * inv;
  __syncthreads();
  // out_j = sum_i o_i R_V[j][i]: columns 64 half + 4 m + (0..3)
  float o = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const float4 x = *reinterpret_cast<const float4*>(&ofin[64 * half + 4 * m]);
    const float4 r = rr[m];
    o = fmaf(x.x, r.x, fmaf(x.y, r.y, fmaf(x.z, r.z, fmaf(x.w, r.w, o))));
  }
  o += dpp<0xb1>(o);  // quad_perm [1,0,3,2]: the other half of row j
  if (half == 0) out[row * kHeadDim + j] = o;
}

// --------------------------------------------------------------------------- host side
static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Pages per split, from the longest context (the lengths themselves stay on
// the device).  A large grid takes at least 128 pages per split (four 8-page
// blocks per wave), below which per-workgroup start-up and the merge of many
// partials cost more than the extra workgroups bring; above that, about 5120
// workgroups for the longest context in every sequence, in whole 32-page
// steps, so that a ragged batch (whose actual work may be half of that) still
// leaves the dispatcher many short workgroups to balance; at most 512 pages.
// A small grid lowers the floor toward 32 pages (one block per wave) so that
// the launch still has about 512 workgroups: 128 splits of 128 pages would
// leave half of the 256 CUs idle.  Measured cold on MI355X: 128K context
// batch 1 and 16K batch 16 are fastest at 128 pages; a batch of 64 with
// contexts of 1K-32K (group 64) at 192 pages: whole call 183.9-194.1 us,
// against 191.1-194.0 at 160, 193.1 at 224, 202.5-206.5 at 128 and 207.7 at
// 256.
int choose_split_pages(int B, int Hkv, int QG, int max_ctx) {
  const int64_t max_pages = (static_cast<int64_t>(max_ctx) + kBlock - 1) / kBlock;
  const int64_t total = static_cast<int64_t>(B) * Hkv * QG * max_pages;
  const int64_t floor = std::min<int64_t>(128, std::max<int64_t>(32, total / 512 / 8 * 8));
  int64_t spw = (total / 5120 + 16) / 32 * 32;
  if (spw < floor) spw = floor;
  if (spw > 512) spw = 512;
  return static_cast<int>(spw);
}

// With BF16 windows the scan launch has B * Hkv * QG window workgroups
// beside the splits, four-wave workgroups four to a CU (one round of the
// MI355X's 256 CUs holds 1024).  An automatic split size is raised, by up to
// half, to the first multiple of 8 pages that brings the launch within one
// round: the last splits would otherwise start only as the window
// workgroups end (16K batch 16: 8 splits of 128 pages, 1152 workgroups, a
// windowed step of 1.733-1.734 ms; 7 of 144, 1024 workgroups, 1.696-1.698).
// The split count only falls, so the plain call's workspace still suffices.
constexpr int kWindowScanSlots = 4 * 256;
DecodePlan make_window_plan(int B, int Hq, int Hkv, int max_ctx, int split_pages) {
  if (split_pages > 0) return make_plan(B, Hq, Hkv, max_ctx, split_pages);
  const int QG = (Hq / Hkv + kHT - 1) / kHT;
  const int64_t tiles = static_cast<int64_t>(B) * Hkv * QG;
  const int base = choose_split_pages(B, Hkv, QG, max_ctx);
  const int max_pages = static_cast<int>((static_cast<int64_t>(max_ctx) + kBlock - 1) / kBlock);
  for (int spw = base; spw <= std::min(512, base + base / 2); spw += 8)
    if (tiles + tiles * num_splits(max_pages, spw) <= kWindowScanSlots)
      return make_plan(B, Hq, Hkv, max_ctx, spw);
  return make_plan(B, Hq, Hkv, max_ctx, 0);
}

DecodePlan make_plan(int B, int Hq, int Hkv, int max_ctx, int split_pages) {
  DecodePlan p{};
  const int Hg = Hq / Hkv;
  p.QG = (Hg + kHT - 1) / kHT;
  p.spw = split_pages > 0 ? split_pages : choose_split_pages(B, Hkv, p.QG, max_ctx);
  const int64_t max_pages = (static_cast<int64_t>(max_ctx) + kBlock - 1) / kBlock;
  p.S = num_splits(static_cast<int>(max_pages), p.spw);
  const size_t hg = static_cast<size_t>(B) * Hkv * p.QG;
  p.qa_off = 0;
  p.qf_off = align256(hg * 64 * kQaDwords * 4);
  p.part_off = p.qf_off + align256(hg * kHT * 16);
  p.wpart_off =
      p.part_off + align256(static_cast<size_t>(B) * Hq * (p.S ? p.S : 1) * kPartStride * 4);
  p.deq_off = p.wpart_off + align256(static_cast<size_t>(B) * Hq * kPartStride * 4);
  p.qr_off = p.deq_off + align256(static_cast<size_t>(B) * Hkv * kDeqStride * 4);
  p.total = p.qr_off + align256(hg * kHT * kHeadDim * 4);
  return p;
}

// A call that launches the PREPARE and SPLITS stages together builds the
// query operand inside the split workgroups, with no prologue launch, when
// the grid is one round of workgroups (at most 1024): the CUs have time to
// spare while the first slices land (16K batch 16: 46.5 -> 42.9 us per call;
// 128K batch 1: 31.1 -> 29.7 us).  On larger grids every workgroup repeating
// the rotation costs more than the launch (the ragged batch of 64: 231 -> 256
// us).  A PREPARE-only call still writes the operand to the workspace for a
// later SPLITS-only call.
bool operand_in_scan(const DecodePlan& p, int Hkv, int B, int stages) {
  return (stages & 3) == 3 && static_cast<int64_t>(p.S) * Hkv * p.QG * B <= 1024;
}

// The decode launches.  tail (the decode step with the operand built in the
// scan, one query tile per KV head, no windows): the scan also appends the
// new tokens in workgroups of its own, leaving their slots out, and the merge
// adds them.
static int launch_decode_impl(const uint8_t* pages, int64_t num_blocks, int Hkv, int G,
                              const int* block_table, int max_blocks, const int* ctx_len,
                              int max_ctx, int B, int Hq, const void* q, bool q_bf16,
                              const float* rot_k, const float* rot_v, float sm_scale, float* out,
                              void* workspace, const DecodePlan& p, int stages,
                              hipStream_t stream, const uint16_t* win, const float* mu,
                              const StepTail* tail) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* qa = reinterpret_cast<uint32_t*>(ws + p.qa_off);
  float4* qf = reinterpret_cast<float4*>(ws + p.qf_off);
  float* part = reinterpret_cast<float*>(ws + p.part_off);
  float* wpart = win ? reinterpret_cast<float*>(ws + p.wpart_off) : nullptr;
  const float qscale = sm_scale * kLog2e;
  const bool self_q = operand_in_scan(p, Hkv, B, stages);
  if (p.S > 0 && (stages & 1) && !self_q) {
    const dim3 g1(Hkv * p.QG, B);
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, g1, dim3(512), 0, stream, q, rot_k, Hq, Hkv, p.QG, qscale, qa,
                         qf);
    };
    if (q_bf16)
      G == 2 ? go(prologue_kernel<true, 2>) : go(prologue_kernel<true, 1>);
    else
      G == 2 ? go(prologue_kernel<false, 2>) : go(prologue_kernel<false, 1>);
  }
  const int n_win = win ? B * Hkv * p.QG : 0;
  StepTail st{};
  if (tail) {
    st = *tail;
    st.deq = reinterpret_cast<float*>(ws + p.deq_off);
    st.qr = reinterpret_cast<float*>(ws + p.qr_off);
    st.n_app = B * Hkv;
  }
  if ((p.S > 0 || win) && (stages & 2)) {
    const int nw = split_waves(G, win != nullptr, self_q);
    const int sp = (p.S + nw / 4 - 1) / (nw / 4);  // split workgroups per query tile
    const ScanDivs dv{fast_div(Hkv * p.QG), fast_div(std::max(sp, 1)), fast_div(p.QG),
                      fast_div(Hkv), fast_div(std::max(p.spw, 1)), Hq / Hkv};
    const dim3 g2(n_win + sp * Hkv * p.QG * B + st.n_app);
    // one buffer descriptor spans the cache when its byte size fits 32 bits
    const bool wide = static_cast<uint64_t>(num_blocks) * Hkv * page_bytes_for_groups(G) >
                      0xFFFFFFFFull;
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, g2, dim3(64 * nw), 0, stream, pages, num_blocks, Hkv,
                         block_table, max_blocks, ctx_len, max_ctx, Hq, p.QG, p.spw, qa, qf, part,
                         p.S, win, n_win, q, q_bf16 ? 1 : 0, mu, qscale, wpart, rot_k, st, dv);
    };
    auto pick = [&](auto g, auto wd) {
      constexpr int GG = decltype(g)::value;
      constexpr bool WD = decltype(wd)::value;
      if (win)
        self_q ? go(split_kernel<GG, WD, true, true>) : go(split_kernel<GG, WD, true, false>);
      else
        self_q ? go(split_kernel<GG, WD, false, true>) : go(split_kernel<GG, WD, false, false>);
    };
    auto pick_w = [&](auto g) {
      wide ? pick(g, Const<bool, true>{}) : pick(g, Const<bool, false>{});
    };
    G == 2 ? pick_w(Const<int, 2>{}) : pick_w(Const<int, 1>{});
  }
  const MergeDivs mdv{fast_div(std::max(p.QG, 1)), fast_div(std::max(p.spw, 1)), Hq / Hkv};
  // fewer than 64 query tiles without windows: a workgroup per query head
  const bool per_head = !win && !tail && static_cast<int64_t>(B) * Hkv * p.QG < 64;
  if ((stages & 4) && per_head) {
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(Hq, B), dim3(256), 0, stream, part, ctx_len, max_ctx, Hq,
                         Hkv, p.spw, p.S ? p.S : 1, rot_v, out);
    };
    if (p.S <= 16)
      go(merge_head_kernel<4>);
    else if (p.S <= 64 || p.S > 128)
      go(merge_head_kernel<kHeadMergeSplits>);
    else
      go(merge_head_kernel<32>);
  } else if (stages & 4) {
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(Hkv * p.QG, B), dim3(1024), 0, stream, part, ctx_len,
                         max_ctx, Hq, Hkv, p.QG, p.spw, p.S ? p.S : 1, rot_v, out,
                         static_cast<const float*>(wpart), st.start_pos,
                         static_cast<const float*>(st.deq), static_cast<const float*>(st.qr), mdv);
    };
    if (p.S <= 16)
      tail ? go(merge_kernel<true, 4>) : go(merge_kernel<false, 4>);
    else
      tail ? go(merge_kernel<true, kMergeSplits>) : go(merge_kernel<false, kMergeSplits>);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_decode(const uint8_t* pages, int64_t num_blocks, int Hkv, int G,
                  const int* block_table, int max_blocks, const int* ctx_len, int max_ctx, int B,
                  int Hq, const void* q, bool q_bf16, const float* rot_k, const float* rot_v,
                  float sm_scale, float* out, void* workspace, const DecodePlan& p, int stages,
                  hipStream_t stream, const uint16_t* win, const float* mu) {
  return launch_decode_impl(pages, num_blocks, Hkv, G, block_table, max_blocks, ctx_len, max_ctx,
                            B, Hq, q, q_bf16, rot_k, rot_v, sm_scale, out, workspace, p, stages,
                            stream, win, mu, nullptr);
}

int launch_append_decode(uint8_t* pages, int64_t num_blocks, int Hkv, int G,
                         const int* block_table, int max_blocks, const int* start_pos,
                         const void* k, const void* v, bool kv_bf16, const float* mu,
                         float clip_k, float clip_v, const int* ctx_len, int max_ctx, int B,
                         int Hq, const void* q, bool q_bf16, const float* rot_k,
                         const float* rot_v, float sm_scale, float* out, void* workspace,
                         const DecodePlan& p, hipStream_t stream, uint16_t* win) {
  // Two launches when the scan builds its own query operand (one round of
  // workgroups), with one query tile per KV head and no windows: the appends
  // run in the scan's launch (its tail) and the merge adds the new tokens.
  // Otherwise three: the append and the query rotation share the first.
  if (!win && p.QG == 1 && p.S > 0 && operand_in_scan(p, Hkv, B, 7)) {
    const StepTail tail{pages, start_pos, k, v, kv_bf16 ? 1 : 0, mu, rot_v, clip_k, clip_v,
                        nullptr, nullptr, 0};
    return launch_decode_impl(pages, num_blocks, Hkv, G, block_table, max_blocks, ctx_len,
                              max_ctx, B, Hq, q, q_bf16, rot_k, rot_v, sm_scale, out, workspace,
                              p, 7, stream, nullptr, mu, &tail);
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* qa = reinterpret_cast<uint32_t*>(ws + p.qa_off);
  float4* qf = reinterpret_cast<float4*>(ws + p.qf_off);
  const float qscale = sm_scale * kLog2e;
  const dim3 grid(Hkv * (1 + p.QG), B);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(1024), 0, stream, pages, num_blocks, Hkv, block_table,
                       max_blocks, start_pos, k, v, mu, rot_k, rot_v, clip_k, clip_v, q, Hq,
                       p.QG, qscale, qa, qf, win);
  };
  // (kv dtype, q dtype, group, windows) -> one instantiation
  auto pick = [&](auto kvb, auto qb, auto g) {
    constexpr bool KV = decltype(kvb)::value, QB = decltype(qb)::value;
    constexpr int GG = decltype(g)::value;
    win ? go(step_prep_kernel<KV, QB, GG, true>) : go(step_prep_kernel<KV, QB, GG, false>);
  };
  auto pick_g = [&](auto kvb, auto qb) {
    G == 2 ? pick(kvb, qb, Const<int, 2>{}) : pick(kvb, qb, Const<int, 1>{});
  };
  auto pick_q = [&](auto kvb) {
    q_bf16 ? pick_g(kvb, Const<bool, true>{}) : pick_g(kvb, Const<bool, false>{});
  };
  kv_bf16 ? pick_q(Const<bool, true>{}) : pick_q(Const<bool, false>{});
  if (hipGetLastError() != hipSuccess) return -1;
  return launch_decode(pages, num_blocks, Hkv, G, block_table, max_blocks, ctx_len, max_ctx, B,
                       Hq, q, q_bf16, rot_k, rot_v, sm_scale, out, workspace, p, 2 | 4, stream,
                       win, mu);
}

}  // namespace kvq
