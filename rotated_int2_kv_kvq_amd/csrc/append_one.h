// Single-token append (one new token per sequence), shared by the append
// entry point and the fused decode step.
//
// Method: "Output-Aware Rotation for INT2 KV-Cache Quantization" (Pith review
// of arXiv 2608.02691), "What carries the argument" (key centring before
// rotation; rotation, clipping, grouping, rounding).
#pragma once

#include "kvq_common.h"

namespace kvq {

// ---------------------------------------------------------------------------
// One new token per sequence (the decode-step append).  Workgroup = (KV head,
// sequence), 1024 threads.  The two 128 x 128 rotations are split four ways
// along the input channel: thread (mat, quarter, j) loads its 32 rows of
// column j of R_K or R_V (all loads in flight at once, coalesced across j)
// and forms a partial dot product; the partials meet in LDS.  Threads 0-255
// then own one rotated channel each (0-127 keys, 128-255 values), reduce group
// min/max across the channel's group (one wave for group 64, two waves
// through LDS for group 128), round and write: key codes are gathered four to
// a byte by lane shuffles; each value code goes to a byte of the value block
// that no other thread of the call touches, updated read-modify-write.
//
// The body is a device function of (KV head h, sequence b) so that a decode
// step can run it in the same launch as the query rotation.  It needs all
// 1024 threads of the workgroup.  k_row, v_row are the token's 128 key and
// value elements (kBf16: bfloat16, else float32); it goes to position
// start_pos[b] + pos_delta.
template <bool kBf16>
__device__ __forceinline__ void append_one_body(
    int h, int b, uint8_t* __restrict__ pages, int64_t num_blocks, int Hkv, int G,
    const int* __restrict__ block_table, int max_blocks, const int* __restrict__ start_pos,
    int pos_delta, const void* __restrict__ k_row, const void* __restrict__ v_row,
    const float* __restrict__ mu, const float* __restrict__ rot_k,
    const float* __restrict__ rot_v, float clip_k, float clip_v) {
  __shared__ float a_s[2][kHeadDim];
  __shared__ float part[2][4][kHeadDim];
  __shared__ float red[4][2];
  const int tid = threadIdx.x;

  // Destination page first (a position outside the table, or a block id
  // outside the cache, writes nothing): its chain of loads (start position,
  // block id, the value byte this thread updates) overlaps the rotation's.
  const int pos = start_pos[b] + pos_delta;
  int blk = -1;
  if (pos >= 0 && pos / kBlock < max_blocks)
    blk = block_table[static_cast<size_t>(b) * max_blocks + pos / kBlock];
  const bool valid = blk >= 0 && blk < num_blocks;
  const int PB = page_bytes_for_groups(G);
  uint8_t* page = pages + (static_cast<int64_t>(valid ? blk : 0) * Hkv + h) * PB;
  const int t = (pos >= 0 ? pos : 0) % kBlock;
  const bool own = tid < 256 && valid;  // threads 0-255 own one rotated channel each
  const int mat = (tid >> 7) & 1;
  const int j = tid & 127;
  const int wave = (tid >> 6) & 3;
  // the value byte this thread will update (only this thread writes it):
  // word 8*(j % 16) + j / 16, code position 3t mod 16
  const int u = (3 * t) & 15;
  uint8_t* vdst = page + kVCodeOff + 4 * (8 * (j & 15) + (j >> 4)) + (u >> 2);
  const uint32_t vold = (own && mat) ? *vdst : 0u;

  // split-K partial products: thread -> (mat, quarter kq, column jc).  The
  // rotation loads go out first: nothing they need depends on another load.
  // rot_v null (value rotation folded into the caller's weights): the value
  // is encoded as given; rot_k null: the centred key is encoded unrotated.
  {
    const int pm = tid >> 9, kq = (tid >> 7) & 3, jc = tid & 127;
    const bool ident = (pm ? rot_v : rot_k) == nullptr;
    float rcol[32];
    if (!ident) {
      const float* R = (pm ? rot_v : rot_k) + static_cast<size_t>(h) * kHeadDim * kHeadDim +
                       32 * kq * kHeadDim + jc;
#pragma unroll
      for (int i = 0; i < 32; ++i) rcol[i] = R[i * kHeadDim];
    }
    if (kq == 0) {
      float x;
      if constexpr (kBf16)
        x = bf16_to_f32((pm ? static_cast<const uint16_t*>(v_row)
                            : static_cast<const uint16_t*>(k_row))[jc]);
      else
        x = (pm ? static_cast<const float*>(v_row) : static_cast<const float*>(k_row))[jc];
      if (pm == 0) x -= mu[h * kHeadDim + jc];
      a_s[pm][jc] = x;
    }
    __syncthreads();
    if (ident) {
      part[pm][kq][jc] = kq == 0 ? a_s[pm][jc] : 0.f;
    } else {
      const float* a = a_s[pm] + 32 * kq;
      float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        x0 = fmaf(a[i], rcol[i], x0);
        x1 = fmaf(a[i + 1], rcol[i + 1], x1);
        x2 = fmaf(a[i + 2], rcol[i + 2], x2);
        x3 = fmaf(a[i + 3], rcol[i + 3], x3);
      }
      part[pm][kq][jc] = (x0 + x1) + (x2 + x3);
    }
  }
  __syncthreads();

  const float x = (part[mat][0][j] + part[mat][1][j]) + (part[mat][2][j] + part[mat][3][j]);

  float mn = wave_min(x), mx = wave_max(x);
  if (G == 1) {  // group of 128 channels spans this thread's two waves
    if (own && (tid & 63) == 0) {
      red[wave][0] = mn;
      red[wave][1] = mx;
    }
    __syncthreads();
    const int w0 = wave & ~1;
    mn = fminf(red[w0][0], red[w0 + 1][0]);
    mx = fmaxf(red[w0][1], red[w0 + 1][1]);
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

  if (mat == 0) {
    uint32_t byte = code << (2 * (j & 3));
    byte |= shfl_xor(byte, 1);
    byte |= shfl_xor(byte, 2);
    if ((j & 3) == 0) page[kKCodeOff + 32 * t + (j >> 2)] = static_cast<uint8_t>(byte);
  } else {
    const int sh = 2 * (u & 3);
    *vdst = static_cast<uint8_t>((vold & ~(3u << sh)) | (code << sh));
  }
  const int gl = G == 2 ? 64 : 128;
  if ((j & (gl - 1)) == 0) {
    const uint32_t sz = static_cast<uint32_t>(f16_bits(s16)) |
                        (static_cast<uint32_t>(f16_bits(z16)) << 16);
    *reinterpret_cast<uint32_t*>(page + kSzOff + mat * 64 * G + (t * G + j / gl) * 4) = sz;
  }
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
