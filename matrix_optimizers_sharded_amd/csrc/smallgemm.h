// The three Newton-Schulz products for matrices with m = min(rows, cols) <= 256:
// one wave per 32 x 32 output block, operands read straight from the workspace
// (which stays in L2 at these sizes), no LDS ring, and no padding beyond the next
// multiple of 32.
//
// On 256 x 256 tiles such a matrix is one tile per product, on one CU, with its m
// padded to 256 (a 256 x 128 matrix: four times the useful work); here its products
// spread over 10-64 waves.  The choice depends on the matrix alone, so its result
// never depends on the rest of the batch.  Same workspace layout, same products,
// same rounding points as k_ns_gemm (gemm.h): A and B' written exactly symmetric
// from their upper blocks, a added on B's diagonal for rows < m, the first products
// taking the Frobenius factor.  Blocks reach into the zero padding of the workspace
// only up to the next multiple of 32 (rows) and of the k step (the reduction), where
// every operand is zero, so those products are exact zeros; nothing reads further.
#pragma once

#include "common.h"
#include "gemm.h"

namespace mo {

constexpr int SB = 32;            // output block

// per-matrix item counts of the small kinds
__host__ __device__ inline int64_t small_upper_items(int m) {
  const int64_t t = (m + SB - 1) / SB;
  return t * (t + 1) / 2;
}
__host__ __device__ inline int64_t small_rect_items(int m, int n) {
  return static_cast<int64_t>((m + SB - 1) / SB) * ((n + SB - 1) / SB);
}

// upper block (bi <= bj) number `local` of a t x t block grid, row by row
__device__ inline void small_upper(int64_t local, int t, int& bi, int& bj) {
  int r = 0;
  while (local >= t - r) {
    local -= t - r;
    ++r;
  }
  bi = r;
  bj = r + static_cast<int>(local);
}

// One 32 x 32 block per 256-thread block: each of its 4 waves (one per SIMD) takes a
// quarter of the k steps, waves 1-3 leave their partial sums in LDS, and wave 0 adds
// them in wave order and writes the block.  (With one block per wave, the whole k
// range was one chain of dependent MFMAs on one SIMD.)
//   SYRK   C = alpha X X^T (upper blocks, mirrored), K = n
//   POLY   C = aI + b A + c A A (upper blocks, mirrored), K = m
//   APPLY  X' = alpha B' X (all blocks), K = m; the last one writes U or W - lr U
template <typename T, int MODE, typename TO>
__global__ __launch_bounds__(256) void k_ns_small(const MatDesc* __restrict__ descs, int count, int64_t total,
                                                  int parity, float ca, float cb, float cc,
                                                  const float* __restrict__ first) {
  constexpr bool SYM = MODE == GM_SYRK || MODE == GM_POLY;
  constexpr int kind = SYM ? KIND_SMALL_UPPER : KIND_SMALL_RECT;
  constexpr int KB = ROW_BYTES / static_cast<int>(sizeof(T));   // elements per k-block
  constexpr int KSTEP = sizeof(T) == 2 ? 16 : 8;                 // k per MFMA step (both lane halves)
  __shared__ float partial[3][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t item = blockIdx.x;
  if (item >= total) return;   // the whole block (the grid holds `total` blocks)
  const int di = find_desc(descs, count, kind, item);
  const MatDesc& d = descs[di];
  const int64_t local = item - d.begin[kind];
  int bi, bj;
  if (SYM) {
    small_upper(local, (d.m + SB - 1) / SB, bi, bj);
  } else {
    const int tn = (d.n + SB - 1) / SB;
    bi = static_cast<int>(local / tn);
    bj = static_cast<int>(local % tn);
  }
  const int i0 = bi * SB, j0 = bj * SB;
  const int l32 = lane & 31, half = lane >> 5;
  const unsigned char* P;
  const unsigned char* Q;
  uint32_t pP, pQ;
  int K;
  if (MODE == GM_SYRK) {
    P = Q = static_cast<const unsigned char*>(d.X[parity]);
    pP = pQ = d.pX;
    K = d.n;
  } else if (MODE == GM_POLY) {
    P = Q = static_cast<const unsigned char*>(d.A);
    pP = pQ = d.pM;
    K = d.m;
  } else {
    P = static_cast<const unsigned char*>(d.B);
    Q = static_cast<const unsigned char*>(d.X[parity]);
    pP = d.pM;
    pQ = d.pX;
    K = d.m;
  }
  const int steps = (K + KSTEP - 1) / KSTEP;
  // this wave's quarter of the k steps
  const int s_begin = steps * wave / 4, s_end = steps * (wave + 1) / 4;
  typedef typename Mfma<T>::frag frag_t;
  // first operand: row i0 + l32, the 16 bytes of k at chunk c = 2 (s % 4) + half of
  // k-block s / 4 (the fragment layout of gemm.h, read from the workspace directly)
  auto frag_rows = [&](const unsigned char* base, uint32_t pitch, int row, int s) {
    const uint32_t o = static_cast<uint32_t>(s / 4) * pitch + static_cast<uint32_t>(row) * ROW_BYTES +
                       static_cast<uint32_t>(2 * (s % 4) + half) * 16;
    return *reinterpret_cast<gptr<const frag_t>>(global(base) + o);
  };
  // APPLY's second operand: X[k][j0 + l32] for the same k as the first operand's
  // chunk, one element at a time (X is k-blocked along its columns j)
  auto frag_cols = [&](int s) {
    frag_t f;
    const int j = j0 + l32;
    constexpr int E = 16 / sizeof(T);
    const int kbase = s * KSTEP + half * E;
    const uint32_t col = static_cast<uint32_t>(j / KB) * pQ + static_cast<uint32_t>(j % KB) * sizeof(T);
#pragma unroll
    for (int e = 0; e < E; ++e)
      f[e] = *reinterpret_cast<gptr<const T>>(global(Q) + col + static_cast<uint32_t>(kbase + e) * ROW_BYTES);
    return f;
  };
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // steps whose loads go out together: 16 took APPLY on a 256 x 128 fp32 matrix
  // from 17.9 to 9.8 us per launch against 4 (its second operand arrives element by
  // element); SYRK and POLY, whose operands are 16-byte loads, did not change
  constexpr int U = 16;
  int s = s_begin;
  for (; s + U <= s_end; s += U) {
    frag_t a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = frag_rows(P, pP, i0 + l32, s + u);
      b[u] = SYM ? frag_rows(Q, pQ, j0 + l32, s + u) : frag_cols(s + u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) Mfma<T>::mma(acc, a[u], b[u]);
  }
  for (; s < s_end; ++s) {
    const frag_t a = frag_rows(P, pP, i0 + l32, s);
    const frag_t b = SYM ? frag_rows(Q, pQ, j0 + l32, s) : frag_cols(s);
    Mfma<T>::mma(acc, a, b);
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) partial[wave - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += partial[w][r][lane];

  float alpha = 1.f;
  if (MODE != GM_POLY && first != nullptr) {
    const float f = first[d.scale_slot];
    alpha = MODE == GM_SYRK ? f * f : f;
  }
  // accumulator layout of a 32x32 block: register r of lane l holds row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
  const int j = j0 + l32;
  if (SYM) {
    T* C = static_cast<T*>(MODE == GM_SYRK ? d.A : d.B);
    const gptr<const T> Ain = global(static_cast<const T*>(d.A));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + 8 * (r / 4) + 4 * half + r % 4;
      if (i > j) continue;   // the upper triangle, then its mirror
      float v = acc[r] * alpha;
      if (MODE == GM_POLY) {
        v = cb * to_f32(*at<const T>(Ain, kb_off<T>(i, j, d.pM))) + cc * v;
        if (i == j && j < d.m) v += ca;
      }
      const T x = from_f32<T>(v);
      *at<T>(global(C), kb_off<T>(i, j, d.pM)) = x;
      if (i < j) *at<T>(global(C), kb_off<T>(j, i, d.pM)) = x;
    }
  } else if (MODE == GM_APPLY) {
    T* Xn = static_cast<T*>(d.X[parity ^ 1]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + 8 * (r / 4) + 4 * half + r % 4;
      *at<T>(global(Xn), kb_off<T>(i, j, d.pX)) = from_f32<T>(acc[r] * alpha);
    }
  } else {
    const gptr<TO> out = global(static_cast<TO*>(d.out));
    const int m = d.m, n = d.n;
    if (j < n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r / 4) + 4 * half + r % 4;
        if (i >= m) continue;
        const float u = acc[r] * alpha;
        const gptr<TO> o = d.transposed ? out + static_cast<int64_t>(j) * m + i : out + static_cast<int64_t>(i) * n + j;
        *o = from_f32<TO>(MODE == GM_APPLY_WEIGHT ? to_f32(*o) - ca * u : u);
      }
    }
  }
}

}  // namespace mo
