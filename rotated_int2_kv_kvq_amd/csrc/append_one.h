// Single-token append (one new token per sequence), shared by the append
// entry point and the decode step.
//
// Method: "Output-Aware Rotation for INT2 KV-Cache Quantization" (Pith review
// of arXiv 2608.02691), "What carries the argument" (key centring before
// rotation; rotation, clipping, grouping, rounding).
#pragma once

#include "kvq_common.h"

namespace kvq {

// ---------------------------------------------------------------------------
// One new token per sequence (the decode-step append), one workgroup per (KV
// head, sequence).  Rotated channel j of the key (mat 0) or value (mat 1) is
// sum_i a_i R[i][j] over the 128 input channels a (the centred key, or the
// value), taken as four quarter sums of 32 rows (four interleaved
// accumulators each), then (q0 + q1) + (q2 + q3).  Threads 0-255 then own
// one rotated channel each (0-127 keys, 128-255 values), reduce group min/max
// across the channel's group (one wave for group 64, two waves through LDS
// for group 128), round and write: key codes are gathered four to a byte by
// lane shuffles; each value code goes to a byte of the value block that no
// other thread of the call touches, updated read-modify-write.
//
// Two forms with the same arithmetic (so the same bytes): append_one_body for
// 1024-thread workgroups, the four quarters in parallel (thread (mat,
// quarter, j) loads its 32 rows of column j, all in flight at once, and the
// partials meet in LDS); append_one_256 for 256-thread workgroups, a thread
// per rotated channel taking the quarters in turn.  k_row, v_row are the
// token's 128 key and value elements (kBf16: bfloat16, else float32).

// The destination of the token (a position outside the table, or a block id
// outside the cache, writes nothing) and the value byte thread (mat 1, j)
// updates (only it writes it): word 8*(j % 16) + j / 16, code position 3t
// mod 16.
struct OneDst {
  uint8_t* page;
  uint8_t* vdst;
  uint32_t vold;
  int t;
  bool valid;
};

__device__ __forceinline__ void append_one_locate(int h, int b, uint8_t* __restrict__ pages,
                                                  int64_t num_blocks, int Hkv, int G,
                                                  const int* __restrict__ block_table,
                                                  int max_blocks, int pos, OneDst& D) {
  const int tid = threadIdx.x;
  int blk = -1;
  if (pos >= 0 && pos / kBlock < max_blocks)
    blk = block_table[static_cast<size_t>(b) * max_blocks + pos / kBlock];
  D.valid = blk >= 0 && blk < num_blocks;
  D.page = pages + (static_cast<int64_t>(D.valid ? blk : 0) * Hkv + h) * page_bytes_for_groups(G);
  D.t = (pos >= 0 ? pos : 0) % kBlock;
  const int j = tid & 127;
  const int u = (3 * D.t) & 15;
  D.vdst = D.page + kVCodeOff + 4 * (8 * (j & 15) + (j >> 4)) + (u >> 2);
  const bool own_v = tid < 256 && D.valid && ((tid >> 7) & 1);
  D.vold = own_v ? *D.vdst : 0u;
}

// The token's element of input channel jc of mat (keys centred).
template <bool kBf16>
__device__ __forceinline__ float append_one_input(int h, int pm, int jc,
                                                  const void* __restrict__ k_row,
                                                  const void* __restrict__ v_row,
                                                  const float* __restrict__ mu) {
  float x;
  if constexpr (kBf16)
    x = bf16_to_f32((pm ? static_cast<const uint16_t*>(v_row)
                        : static_cast<const uint16_t*>(k_row))[jc]);
  else
    x = (pm ? static_cast<const float*>(v_row) : static_cast<const float*>(k_row))[jc];
  if (pm == 0) x -= mu[h * kHeadDim + jc];
  return x;
}

// One quarter of the rotation: a[0..31] against rows 32 kq .. 32 kq + 31 of
// the column.
__device__ __forceinline__ float rot_quarter(const float* __restrict__ a,
                                             const float (&rcol)[32]) {
  float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    x0 = fmaf(a[i], rcol[i], x0);
    x1 = fmaf(a[i + 1], rcol[i + 1], x1);
    x2 = fmaf(a[i + 2], rcol[i + 2], x2);
    x3 = fmaf(a[i + 3], rcol[i + 3], x3);
  }
  return (x0 + x1) + (x2 + x3);
}

// Threads 0-255 hold rotated channel x of (mat tid/128, j tid%128); every
// thread of the workgroup calls this (it has a barrier for group 128).  red:
// 8 floats of LDS.  deq (optional, [K, V][128]) receives the token's
// dequantised key and value in the rotated basis.
__device__ __forceinline__ void append_one_store(float x, const OneDst& D, int G, float clip_k,
                                                 float clip_v, float* red,
                                                 float* __restrict__ deq) {
  const int tid = threadIdx.x;
  const bool own = tid < 256 && D.valid;
  const int mat = (tid >> 7) & 1;
  const int j = tid & 127;
  const int wave = (tid >> 6) & 3;
  float mn = wave_min(x), mx = wave_max(x);
  if (G == 1) {  // group of 128 channels spans this thread's two waves
    if (own && (tid & 63) == 0) {
      red[2 * wave] = mn;
      red[2 * wave + 1] = mx;
    }
    __syncthreads();
    const int w0 = wave & ~1;
    mn = fminf(red[2 * w0], red[2 * w0 + 2]);
    mx = fmaxf(red[2 * w0 + 1], red[2 * w0 + 3]);
  }
  if (!own) return;
  const float clip = mat ? clip_v : clip_k;
  const float lo = clip * mn;
  const float hi = clip * mx;
  const _Float16 s16 = f16_sat((hi - lo) / 3.0f);
  const _Float16 z16 = f16_sat(lo);
  const float sf = static_cast<float>(s16);
  const float zf = static_cast<float>(z16);
  uint32_t code = 0;
  if (sf != 0.f) code = static_cast<uint32_t>(fminf(fmaxf(rintf((x - zf) / sf), 0.f), 3.f));
  if (deq) deq[mat * kHeadDim + j] = fmaf(sf, static_cast<float>(code), zf);

  const int t = D.t;
  if (mat == 0) {
    uint32_t byte = code << (2 * (j & 3));
    byte |= shfl_xor(byte, 1);
    byte |= shfl_xor(byte, 2);
    if ((j & 3) == 0) D.page[kKCodeOff + 32 * t + (j >> 2)] = static_cast<uint8_t>(byte);
  } else {
    const int u = (3 * t) & 15;
    const int sh = 2 * (u & 3);
    *D.vdst = static_cast<uint8_t>((D.vold & ~(3u << sh)) | (code << sh));
  }
  const int gl = G == 2 ? 64 : 128;
  if ((j & (gl - 1)) == 0) {
    const uint32_t sz = static_cast<uint32_t>(f16_bits(s16)) |
                        (static_cast<uint32_t>(f16_bits(z16)) << 16);
    *reinterpret_cast<uint32_t*>(D.page + kSzOff + mat * 64 * G + (t * G + j / gl) * 4) = sz;
  }
}

// 1024 threads: the quarters in parallel; the token goes to position
// start_pos[b] + pos_delta.  rot_v null (value rotation folded into the
// caller's weights): the value is encoded as given; rot_k null: the centred
// key is encoded unrotated.
template <bool kBf16>
__device__ __forceinline__ void append_one_body(
    int h, int b, uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv, int G,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ start_pos,
    int pos_delta, const void* __restrict__ k_row, const void* __restrict__ v_row,
    const float* __restrict__ mu, const float* __restrict__ rot_k,
    const float* __restrict__ rot_v, float clip_k, float clip_v) {
  __shared__ float a_s[2][kHeadDim];
  __shared__ float part[2][4][kHeadDim];
  __shared__ float red[8];
  const int tid = threadIdx.x;

  // Destination page first: its chain of loads (start position, block id,
  // the value byte this thread updates) overlaps the rotation's.
  OneDst D;
  append_one_locate(h, b, pages, num_blocks, Hkv, G, block_table, max_blocks,
                    start_pos[b] + pos_delta, D);
  {
    const int pm = tid >> 9, kq = (tid >> 7) & 3, jc = tid & 127;
    const float* Rm = pm ? rot_v : rot_k;
    const bool ident = Rm == nullptr;
    float rcol[32];
    if (!ident) {
      const float* R = Rm + static_cast<size_t>(h) * kHeadDim * kHeadDim + 32 * kq * kHeadDim + jc;
#pragma unroll
      for (int i = 0; i < 32; ++i) rcol[i] = R[i * kHeadDim];
    }
    if (kq == 0) a_s[pm][jc] = append_one_input<kBf16>(h, pm, jc, k_row, v_row, mu);
    __syncthreads();
    if (ident)
      part[pm][kq][jc] = kq == 0 ? a_s[pm][jc] : 0.f;
    else
      part[pm][kq][jc] = rot_quarter(a_s[pm] + 32 * kq, rcol);
  }
  __syncthreads();
  const int mat = (tid >> 7) & 1;
  const int j = tid & 127;
  const float x = (part[mat][0][j] + part[mat][1][j]) + (part[mat][2][j] + part[mat][3][j]);
  append_one_store(x, D, G, clip_k, clip_v, red, nullptr);
}

// 256 threads (a thread per rotated channel, the quarters in turn, the next
// quarter's column loads in flight while one is summed); the token goes to
// position pos.  Threads 256 and up of a larger workgroup write the first
// 256's inputs again (the same values to the same LDS words), skip the
// rotation's loads, pass the barriers and store nothing.  scratch: 264 floats of LDS that the caller lends (the
// token's inputs and the group reduction).  deq as for append_one_store.
template <bool kBf16>
__device__ __forceinline__ void append_one_256(
    int h, int b, uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv, int G,
    const int* __restrict__ block_table, int max_blocks, int pos, const void* __restrict__ k_row,
    const void* __restrict__ v_row, const float* __restrict__ mu, const float* __restrict__ rot_k,
    const float* __restrict__ rot_v, float clip_k, float clip_v, float* scratch,
    float* __restrict__ deq) {
  const int tid = threadIdx.x;
  const int mat = (tid >> 7) & 1, j = tid & 127;
  float* a_s = scratch;                 // [2][128]
  float* red = scratch + 2 * kHeadDim;  // [8]
  OneDst D;
  append_one_locate(h, b, pages, num_blocks, Hkv, G, block_table, max_blocks, pos, D);
  const float* Rm = mat ? rot_v : rot_k;
  const bool ident = Rm == nullptr || tid >= 256;  // (per wave)
  const float* R = ident ? nullptr : Rm + static_cast<size_t>(h) * kHeadDim * kHeadDim + j;
  float rc[2][32];
  if (!ident) {
#pragma unroll
    for (int i = 0; i < 32; ++i) rc[0][i] = R[i * kHeadDim];
  }
  a_s[mat * kHeadDim + j] = append_one_input<kBf16>(h, mat, j, k_row, v_row, mu);
  __syncthreads();
  float x;
  if (ident) {
    // as the 1024-thread form adds its zero quarters
    x = (a_s[mat * kHeadDim + j] + 0.f) + (0.f + 0.f);
  } else {
    float q[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      if (kq < 3) {
#pragma unroll
        for (int i = 0; i < 32; ++i) rc[(kq + 1) & 1][i] = R[(32 * (kq + 1) + i) * kHeadDim];
      }
      q[kq] = rot_quarter(a_s + mat * kHeadDim + 32 * kq, rc[kq & 1]);
    }
    x = (q[0] + q[1]) + (q[2] + q[3]);
  }
  append_one_store(x, D, G, clip_k, clip_v, red, deq);
}

// Row pointer of sequence b, KV head h in a [B][1][Hkv][128] token tensor.
template <bool kBf16>
__device__ __forceinline__ const void* token_row(const void* x, int b, int h, int Hkv) {
  const size_t off = (static_cast<size_t>(b) * Hkv + h) * kHeadDim;
  if constexpr (kBf16)
    return static_cast<const uint16_t*>(x) + off;
  else
    return static_cast<const float*>(x) + off;
}

}  // namespace kvq
