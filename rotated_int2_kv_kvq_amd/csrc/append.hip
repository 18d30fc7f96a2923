// Cache-append quantiser: centre, rotate, clip, group INT2 round-to-nearest
// with fp16 scale/zero, pack into the paged cache.
//
// Method: "Output-Aware Rotation for INT2 KV-Cache Quantization" (Pith review
// of arXiv 2608.02691), "What carries the argument" (key centring before
// rotation; rotation, clipping, grouping, rounding) and "Core claim" (one
// orthogonal rotation per KV head and layer).
//
// Work decomposition.  One workgroup (8 waves, two per SIMD) owns one
// (sequence, KV head) and a run of consecutive pages touched by this call; it
// stages R_K and R_V in LDS once (transposed, columns permuted so that each
// lane ends up holding 8 consecutive rotated channels; 135 KB, so one
// workgroup per CU), then waves 0-3 encode keys and waves 4-7 values, each
// taking every fourth page, with the next page's token rows loaded while the
// current page is rotated.  A wave encodes one 16-token page at a time:
// the 16 x 128 x 128 rotation is 256 fp32 MFMAs (16x16x4), whose output
// gives lane l tokens 4*(l/16)..+3 and channels 8*(l%16)..+7; group min/max
// is a 16-lane (or 8-lane) butterfly; codes are packed in registers and
// written to the page.  Because a page is owned by one wave for the whole
// call, partially filled V-code words are updated read-modify-write without
// races.
#include <algorithm>

#include "append_one.h"
#include "kvq_common.h"
#include "kvq_launch.h"

namespace kvq {

constexpr int kRStride = 132;  // LDS row stride (floats) of a staged rotation

// One lane's 32 input channels of a token row as loaded (bf16: four 16-byte
// loads; fp32: eight), kept raw while in flight.
template <bool kBf16>
struct RawRow {
  uint4 u[kBf16 ? 4 : 8];
};

template <bool kBf16>
__device__ __forceinline__ void load_raw32(const void* src, size_t elem_off, RawRow<kBf16>& r) {
  if constexpr (kBf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + elem_off);
#pragma unroll
    for (int q = 0; q < 4; ++q) r.u[q] = p[q];
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(src) + elem_off);
#pragma unroll
    for (int q = 0; q < 8; ++q) r.u[q] = p[q];
  }
}

template <bool kBf16>
__device__ __forceinline__ void raw_to_f32(const RawRow<kBf16>& r, float (&a)[32]) {
  if constexpr (kBf16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w[4] = {r.u[q].x, r.u[q].y, r.u[q].z, r.u[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
        a[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      a[4 * q] = __uint_as_float(r.u[q].x);
      a[4 * q + 1] = __uint_as_float(r.u[q].y);
      a[4 * q + 2] = __uint_as_float(r.u[q].z);
      a[4 * q + 3] = __uint_as_float(r.u[q].w);
    }
  }
}

// Minimum and maximum over the 16 lanes of a DPP row (kHalfRow: over each
// 8-lane half row), the same in every lane: quad_perm [1,0,3,2],
// [2,3,0,1], row_half_mirror, row_mirror, one min and one max per step (the
// values are finite, so no NaN quieting is needed).  The nop gives the two
// wait states a DPP read of a just-written VGPR needs.
#define KVQ_MINMAX_DPP(ctrl)                                                                \
  asm("s_nop 1\n\t"                                                                         \
      "v_min_f32_dpp %0, %2, %2 " ctrl " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"         \
      "v_max_f32_dpp %1, %3, %3 " ctrl " row_mask:0xf bank_mask:0xf bound_ctrl:1"            \
      : "=&v"(a), "=&v"(b)                                                                  \
      : "v"(mn), "v"(mx));                                                                  \
  mn = a;                                                                                   \
  mx = b
template <bool kHalfRow>
__device__ __forceinline__ void row_minmax(float& mn, float& mx) {
  float a, b;
  KVQ_MINMAX_DPP("quad_perm:[1,0,3,2]");
  KVQ_MINMAX_DPP("quad_perm:[2,3,0,1]");
  KVQ_MINMAX_DPP("row_half_mirror");
  if constexpr (!kHalfRow) {
    KVQ_MINMAX_DPP("row_mirror");
  }
}
#undef KVQ_MINMAX_DPP

template <bool kBf16>
__global__ __launch_bounds__(512) void append_kernel(
    uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv, int G,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ start_pos,
    int T, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ mu, const float* __restrict__ rot_k,
    const float* __restrict__ rot_v, float clip_k, float clip_v, int pages_per_wg) {
  __shared__ float Bt[2][kHeadDim * kRStride];

  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int s0 = start_pos[b];
  if (s0 < 0) return;
  const int first_page = s0 / kBlock;
  const int last_page = (s0 + T - 1) / kBlock;
  const int wg_first = first_page + blockIdx.x * pages_per_wg;
  if (wg_first > last_page) return;
  const int wg_last = min(last_page, wg_first + pages_per_wg - 1);

  // rot_v null: the value rotation is folded into the caller's weights and
  // values are encoded as given (no products for them); rot_k null: keys are
  // centred but not rotated (plain INT2 of the centred key).
  const bool v_ident = rot_v == nullptr;
  const bool k_ident = rot_k == nullptr;
  // Stage R_K and R_V: LDS row r = 16*(c%8) + c/8 holds column c of R, so the
  // MFMA output column (tile nt, lane n) is rotated channel 8*n + nt.
  for (int mat = 0; mat < 2; ++mat) {
    if (mat ? v_ident : k_ident) continue;
    const float* R = (mat ? rot_v : rot_k) + static_cast<size_t>(h) * kHeadDim * kHeadDim;
    for (int idx = tid; idx < kHeadDim * kHeadDim / 4; idx += 512) {
      const int krow = idx >> 5;
      const int c4 = (idx & 31) * 4;
      const float4 r = *reinterpret_cast<const float4*>(R + krow * kHeadDim + c4);
      const float rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c4 + u;
        Bt[mat][((c & 7) * 16 + (c >> 3)) * kRStride + krow] = rv[u];
      }
    }
  }
  __syncthreads();

  const int mat = wave >> 2;  // 0 = keys, 1 = values
  const int w4 = wave & 3;    // pages wg_first + w4, + 4, ...
  const float clip = mat ? clip_v : clip_k;
  const void* src = mat ? v : k;
  const int PB = page_bytes_for_groups(G);
  const int n = lane & 15;   // B/D column lane: channels 8n..8n+7
  const int kg = lane >> 4;  // A/B k-group: input channels 32kg..32kg+31
  const int t = lane & 15;   // A row: token slot in the page
  const int r4 = lane >> 4;  // D rows: tokens 4*r4..4*r4+3

  // the key mean of this lane's 32 input channels (keys only)
  float mr[32];
#pragma unroll
  for (int s = 0; s < 32; ++s) mr[s] = 0.f;
  if (mat == 0 && !k_ident) {
    const float4* m4 = reinterpret_cast<const float4*>(mu + h * kHeadDim + 32 * kg);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 m = m4[q];
      mr[4 * q] = m.x;
      mr[4 * q + 1] = m.y;
      mr[4 * q + 2] = m.z;
      mr[4 * q + 3] = m.w;
    }
  }
  // Token row t of page pg (input channels 32kg..32kg+31) if that token is
  // one this call writes; false (nothing loaded) otherwise.
  // Unrotated rows are read in the output layout below instead.
  const bool direct = mat == 1 ? v_ident : k_ident;
  auto fetch = [&](int pg, RawRow<kBf16>& r) {
    const int pos = pg * kBlock + t;
    const bool row_new = !direct && pg <= wg_last && pos >= s0 && pos < s0 + T;
    if (row_new)
      load_raw32<kBf16>(src,
                        (static_cast<size_t>(b) * T + (pos - s0)) * Hkv * kHeadDim +
                            static_cast<size_t>(h) * kHeadDim + 32 * kg,
                        r);
    return row_new;
  };
  RawRow<kBf16> raw;
  bool cur_new = fetch(wg_first + w4, raw);
  // unrotated keys: the mean of this lane's output channels 8n..8n+7
  float m8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m8[e] = (direct && mat == 0) ? mu[h * kHeadDim + 8 * n + e] : 0.f;

  for (int pg = wg_first + w4; pg <= wg_last; pg += 4) {
    if (pg >= max_blocks) break;
    // A operand: this lane's token row (centred keys); zero for old tokens
    float a[32];
    raw_to_f32<kBf16>(raw, a);
#pragma unroll
    for (int s = 0; s < 32; ++s) a[s] = cur_new ? a[s] - mr[s] : 0.f;
    // the next page's rows are in flight during this page's products
    RawRow<kBf16> nraw;
    const bool nxt_new = fetch(pg + 4, nraw);
    const int blk = block_table[static_cast<size_t>(b) * max_blocks + pg];
    raw = nraw;
    cur_new = nxt_new;
    if (blk < 0 || blk >= num_blocks) continue;
    uint8_t* page = pages + (static_cast<int64_t>(blk) * Hkv + h) * PB;

    floatx4 acc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (direct) {
      // lane holds tokens 4*r4 + i, channels 8n..8n+7 of the value as given
      // (of the key less its mean)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tpos = pg * kBlock + 4 * r4 + i;
        if (tpos >= s0 && tpos < s0 + T) {
          const size_t off = (static_cast<size_t>(b) * T + (tpos - s0)) * Hkv * kHeadDim +
                             static_cast<size_t>(h) * kHeadDim + 8 * n;
          float x8[8];
          if constexpr (kBf16) {
            const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + off);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x8[2 * e] = __uint_as_float(w[e] << 16);
              x8[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
          } else {
            const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
            const float4 f0 = f[0], f1 = f[1];
            x8[0] = f0.x; x8[1] = f0.y; x8[2] = f0.z; x8[3] = f0.w;
            x8[4] = f1.x; x8[5] = f1.y; x8[6] = f1.z; x8[7] = f1.w;
          }
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) acc[nt][i] = x8[nt] - m8[nt];
        }
      }
    } else {
      const float* Bm = Bt[mat];
#pragma unroll
      for (int sb = 0; sb < 8; ++sb) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const float4 bv =
              *reinterpret_cast<const float4*>(Bm + (nt * 16 + n) * kRStride + 32 * kg + 4 * sb);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * sb + 0], bv.x, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * sb + 1], bv.y, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * sb + 2], bv.z, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * sb + 3], bv.w, acc[nt], 0, 0, 0);
        }
      }
    }

    // Quantise: lane holds tokens 4*r4 + i, channels 8n + nt.
    uint32_t code_bits[4];  // per token: 16 bits, channel 8n+e at bits 2e
    const int gl = (G == 2) ? 8 : 16;  // lanes per group
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mn = acc[0][i], mx = acc[0][i];
#pragma unroll
      for (int nt = 1; nt < 8; ++nt) {
        mn = fminf(mn, acc[nt][i]);
        mx = fmaxf(mx, acc[nt][i]);
      }
      // over the group's lanes: a DPP row (group 128) or half row (group 64)
      if (G == 2)
        row_minmax<true>(mn, mx);
      else
        row_minmax<false>(mn, mx);
      const float lo = clip * mn;
      const float hi = clip * mx;
      const _Float16 s16 = f16_sat((hi - lo) / 3.0f);
      const _Float16 z16 = f16_sat(lo);
      const float sf = static_cast<float>(s16);
      const float zf = static_cast<float>(z16);
      uint32_t bits = 0;
      if (sf != 0.f && !direct) {
        // rotated values: one division per group; the product differs from
        // the quotient by about an ulp, which moves a code only within the
        // rounding-boundary tolerance the codes are held to
        const float inv = 1.0f / sf;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          float qv = rintf((acc[nt][i] - zf) * inv);
          qv = fminf(fmaxf(qv, 0.f), 3.f);
          bits |= static_cast<uint32_t>(qv) << (2 * nt);
        }
      } else if (sf != 0.f) {
        // unrotated values (bfloat16 ones often lie exactly on a rounding
        // boundary): the correctly rounded quotient breaks ties to even
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          float qv = rintf((acc[nt][i] - zf) / sf);
          qv = fminf(fmaxf(qv, 0.f), 3.f);
          bits |= static_cast<uint32_t>(qv) << (2 * nt);
        }
      }
      code_bits[i] = bits;
      const int tq = 4 * r4 + i;
      const int tpos = pg * kBlock + tq;
      if (tpos >= s0 && tpos < s0 + T) {
        if (mat == 0) {
          *reinterpret_cast<uint16_t*>(page + kKCodeOff + 32 * tq + 2 * n) =
              static_cast<uint16_t>(bits);
        }
        if ((n & (gl - 1)) == 0) {
          const int gidx = n / gl;
          const uint32_t sz = static_cast<uint32_t>(f16_bits(s16)) |
                              (static_cast<uint32_t>(f16_bits(z16)) << 16);
          *reinterpret_cast<uint32_t*>(page + kSzOff + mat * 64 * G + (tq * G + gidx) * 4) = sz;
        }
      }
    }

    if (mat == 1) {
      // V words: one per channel c at word 8*(c % 16) + c / 16 of the value
      // block, token tq at code position (3*tq) mod 16.  This lane holds
      // tokens 4*r4 + i of channels 8n + e; lanes ^16 and ^32 hold the other
      // tokens of the same channels, so the four quarters are combined and
      // each of the four lanes writes two of the eight words.
      uint32_t newq = 0;  // which of this lane's tokens are new
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tpos = pg * kBlock + 4 * r4 + i;
        if (tpos >= s0 && tpos < s0 + T) newq |= 1u << i;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t word = 0, mask = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int u = (3 * (4 * r4 + i)) & 15;
          word |= ((code_bits[i] >> (2 * e)) & 3u) << (2 * u);
          if (newq & (1u << i)) mask |= 3u << (2 * u);
        }
        word |= shfl_xor(word, 16);
        mask |= shfl_xor(mask, 16);
        word |= shfl_xor(word, 32);
        mask |= shfl_xor(mask, 32);
        if (r4 == (e & 3) && mask != 0) {
          uint32_t* dst = reinterpret_cast<uint32_t*>(page + kVCodeOff +
                                                      4 * (64 * (n & 1) + 8 * e + (n >> 1)));
          *dst = (mask == 0xffffffffu) ? word : ((*dst & ~mask) | (word & mask));
        }
      }
    }
  }
}

// One new token per sequence: one workgroup of 1024 threads per (KV head,
// sequence), grid (Hkv, B).
template <bool kBf16>
__global__ __launch_bounds__(1024) void append_one_kernel(
    uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv, int G,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ start_pos,
    const void* __restrict__ k, const void* __restrict__ v, const float* __restrict__ mu,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v, float clip_k,
    float clip_v) {
  const int h = blockIdx.x, b = blockIdx.y;
  append_one_body<kBf16>(h, b, pages, num_blocks, Hkv, G, block_table, max_blocks, start_pos, 0,
                         token_row<kBf16>(k, b, h, Hkv), token_row<kBf16>(v, b, h, Hkv), mu,
                         rot_k, rot_v, clip_k, clip_v);
}

// ---------------------------------------------------------------------------
// BF16 window store writes ([OptR] "Assumptions & free parameters": sink and
// recent tokens kept in BF16).  grid (T, Hkv, B), 256 threads: thread
// m*128 + c copies element c of the key (m = 0) or value (m = 1) row of token
// tau, rounded to bfloat16, into the slot of its position.  A ring slot that a
// later token of the same call also takes keeps the later one (the earlier
// write is skipped, so the result does not depend on write order).
template <bool kBf16>
__global__ __launch_bounds__(256) void window_write_kernel(uint16_t* __restrict__ win, int Hkv,
                                                           const int* __restrict__ start_pos,
                                                           int T, const void* __restrict__ k,
                                                           const void* __restrict__ v) {
  const int tau = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int p0 = start_pos[b];
  const int p = p0 + tau;
  if (p0 < 0) return;
  if (p >= kSink && p + kRecent < p0 + T) return;
  const int m = threadIdx.x >> 7, c = threadIdx.x & 127;
  const size_t off = ((static_cast<size_t>(b) * T + tau) * Hkv + h) * kHeadDim + c;
  const void* src = m ? v : k;
  const uint16_t x = kBf16 ? static_cast<const uint16_t*>(src)[off]
                           : f32_to_bf16(static_cast<const float*>(src)[off]);
  win[((static_cast<size_t>(b) * Hkv + h) * 2 + m) * kWindow * kHeadDim +
      static_cast<size_t>(window_slot(p)) * kHeadDim + c] = x;
}

int launch_window_write(uint16_t* win, int Hkv, int B, const int* start_pos, int T, const void* k,
                        const void* v, bool bf16, hipStream_t stream) {
  const dim3 grid(T, Hkv, B);
  if (bf16)
    hipLaunchKernelGGL(window_write_kernel<true>, grid, dim3(256), 0, stream, win, Hkv, start_pos,
                       T, k, v);
  else
    hipLaunchKernelGGL(window_write_kernel<false>, grid, dim3(256), 0, stream, win, Hkv,
                       start_pos, T, k, v);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_append(uint8_t* pages, int64_t num_blocks, int Hkv, int G, const int* block_table,
                  int max_blocks, const int* start_pos, int B, int T, const void* k,
                  const void* v, bool bf16, const float* mu, const float* rot_k,
                  const float* rot_v, float clip_k, float clip_v, hipStream_t stream) {
  if (T == 1) {
    const dim3 grid(Hkv, B);
    if (bf16)
      hipLaunchKernelGGL(append_one_kernel<true>, grid, dim3(1024), 0, stream, pages, num_blocks,
                         Hkv, G, block_table, max_blocks, start_pos, k, v, mu, rot_k, rot_v,
                         clip_k, clip_v);
    else
      hipLaunchKernelGGL(append_one_kernel<false>, grid, dim3(1024), 0, stream, pages, num_blocks,
                         Hkv, G, block_table, max_blocks, start_pos, k, v, mu, rot_k, rot_v,
                         clip_k, clip_v);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  // Pages per workgroup: each stages 128 KB of rotations, so large appends
  // take up to 64 pages (16 per wave), keeping about 2048 workgroups (eight
  // per CU over the launch) when there are fewer pages; at least 8.
  const int max_pages = (T + kBlock - 1) / kBlock + 1;
  const int64_t total = static_cast<int64_t>(B) * Hkv * max_pages;
  const int ppw = static_cast<int>(std::min<int64_t>(64, std::max<int64_t>(8, (total / 2048 + 3) / 4 * 4)));
  const dim3 grid((max_pages + ppw - 1) / ppw, Hkv, B);
  if (bf16)
    hipLaunchKernelGGL(append_kernel<true>, grid, dim3(512), 0, stream, pages, num_blocks, Hkv, G,
                       block_table, max_blocks, start_pos, T, k, v, mu, rot_k, rot_v, clip_k,
                       clip_v, ppw);
  else
    hipLaunchKernelGGL(append_kernel<false>, grid, dim3(512), 0, stream, pages, num_blocks, Hkv,
                       G, block_table, max_blocks, start_pos, T, k, v, mu, rot_k, rot_v, clip_k,
                       clip_v, ppw);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvq
