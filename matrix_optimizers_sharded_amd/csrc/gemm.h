// The three Newton-Schulz products as one MFMA GEMM core with three epilogues.
//
// Every product is C[i][j] = sum_k P[i][k] * Q[j][k] with both operands read along
// k-contiguous rows:
//   SYRK   A  = X X^T         P = Q = X (rows of X, k over n); upper tiles only,
//                             each off-diagonal tile also stored mirrored
//   POLY   B  = bA + c A A    P = Q = A (A symmetric, so A A = A A^T); upper tiles,
//                             mirrored; b*A in the epilogue reads the same rounded A
//   APPLY  X' = aX + B X      P = B, Q = X^T (the kernel keeps X^T as a second
//                             copy so this is k-contiguous too); the epilogue
//                             reads X, writes X' in place and X'^T to the other
//                             ping-pong buffer, or the final U to the caller.
// All workspace dims are multiples of 256, zero-padded, so the main loop needs no
// bounds checks; only the final write to the caller's buffer is clipped.
//
// Tiling (gfx950, wave64): 256x256 block tile, 4 waves in 2x2, each wave owns a
// 128x128 sub-tile = 4x4 MFMA 32x32 blocks (256 fp32 accumulators per lane, held in
// AGPRs).  The k-loop streams 128-byte row slabs (64 bf16 or 32 fp32 of k) of both
// operands straight from HBM/L2 into LDS with 16-byte buffer loads that write LDS
// directly (no register staging), through a 2-stage ring: the loads of slab t+1
// are in flight while slab t is multiplied.  LDS rows are 128 bytes with the 16-byte
// chunk index XOR-swizzled by (r ^ r>>1) & 7, so the fragment reads of 8 or 16
// consecutive rows hit distinct banks.
#pragma once

#include "common.h"

namespace mo {

enum GemmMode { GM_SYRK = 0, GM_POLY = 1, GM_APPLY = 2, GM_APPLY_FINAL = 3 };

constexpr int GT = GEMM_TILE;          // 256
constexpr int ROW_BYTES = 128;         // one k-slab row of an operand tile
constexpr int OPERAND_BYTES = GT * ROW_BYTES;          // 32768
constexpr int STAGE_BYTES = 2 * OPERAND_BYTES;         // P and Q
constexpr int GEMM_LDS_BYTES = 2 * STAGE_BYTES;        // 2 stages = 131072

// raw-buffer resource word 3 for gfx9-family: 32-bit data format, no swizzle
constexpr int RSRC_FLAGS = 0x00020000;

__device__ inline int swz(int r) { return (r ^ (r >> 1)) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
  typedef bf16x8_t frag;
  static __device__ inline void mma(f32x16_t& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  typedef f32x4_t frag;
  // a 16-byte chunk holds 4 consecutive k per lane; four k=2 MFMAs consume it.  P
  // and Q use the same k order, so the contraction is exact regardless of it.
  static __device__ inline void mma(f32x16_t& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], acc, 0, 0, 0);
  }
};

// local upper-triangle index -> (ti, tj), ti <= tj, row-major over the triangle
__device__ inline void upper_tile(int64_t local, int T, int& ti, int& tj) {
  int r = 0;
  int64_t L = local;
  while (L >= T - r) { L -= T - r; ++r; }
  ti = r;
  tj = r + static_cast<int>(L);
}

template <typename T>
__device__ inline void store4(T* p, float v0, float v1, float v2, float v3);
template <> __device__ inline void store4<bf16_t>(bf16_t* p, float v0, float v1, float v2, float v3) {
  bf16x4_t v = {static_cast<bf16_t>(v0), static_cast<bf16_t>(v1), static_cast<bf16_t>(v2),
                static_cast<bf16_t>(v3)};
  *reinterpret_cast<bf16x4_t*>(p) = v;
}
template <> __device__ inline void store4<float>(float* p, float v0, float v1, float v2, float v3) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v0, v1, v2, v3};
}

template <typename T, int MODE, typename TO>
__global__ __launch_bounds__(256, 1) void k_ns_gemm(const MatDesc* __restrict__ descs, int count,
                                                    int parity, float ca, float cb, float cc) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[GEMM_LDS_BYTES];
  constexpr int kind = (MODE == GM_SYRK) ? KIND_SYRK : (MODE == GM_POLY) ? KIND_POLY : KIND_APPLY;
  const int64_t item = blockIdx.x;
  const MatDesc& d = descs[find_desc(descs, count, kind, item)];
  const int64_t local = item - d.begin[kind];

  int ti, tj;
  const T* P;
  const T* Q;
  int64_t ldp, ldq;
  int K;
  if (MODE == GM_SYRK) {
    upper_tile(local, d.mp / GT, ti, tj);
    P = Q = static_cast<const T*>(d.X);
    ldp = ldq = d.np;
    K = d.np;
  } else if (MODE == GM_POLY) {
    upper_tile(local, d.mp / GT, ti, tj);
    P = Q = static_cast<const T*>(d.A);
    ldp = ldq = d.mp;
    K = d.mp;
  } else {
    const int tn = d.np / GT;
    ti = static_cast<int>(local / tn);
    tj = static_cast<int>(local % tn);
    P = static_cast<const T*>(d.B);
    Q = static_cast<const T*>(d.XT[parity]);
    ldp = ldq = d.mp;
    K = d.mp;
  }
  const int i0 = ti * GT, j0 = tj * GT;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;

  // Direct-to-LDS loads: wave w, instruction q fills rows 8*(4q+w) .. +7 of an
  // operand slab (1 KiB contiguous in LDS: lane l -> row 8*(4q+w) + l/8, physical
  // chunk l%8).  The lane fetches the logical chunk that the swizzle stores there.
  const uint32_t esz = sizeof(T);
  const uint32_t rowsP = d.mp;   // X, A and B all have mp rows
  const uint32_t rowsQ = (MODE == GM_APPLY || MODE == GM_APPLY_FINAL) ? d.np : d.mp;
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(P), 0, static_cast<int>(rowsP * static_cast<uint32_t>(ldp) * esz), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(Q), 0, static_cast<int>(rowsQ * static_cast<uint32_t>(ldq) * esz), RSRC_FLAGS);
  uint32_t vP[8], vQ[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = 8 * (4 * q + wave) + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    vP[q] = static_cast<uint32_t>(i0 + row) * static_cast<uint32_t>(ldp) * esz + c * 16;
    vQ[q] = static_cast<uint32_t>(j0 + row) * static_cast<uint32_t>(ldq) * esz + c * 16;
  }
  auto issue = [&](int kt, int stage) {
    const int soff = kt * ROW_BYTES;
    unsigned char* base = smem + stage * STAGE_BYTES + wave * 1024;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (lds_ptr_t)(base + q * 4096), 16, vP[q], soff, 0, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (lds_ptr_t)(base + OPERAND_BYTES + q * 4096), 16, vQ[q],
                                               soff, 0, 0);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // fragment read offsets (row part), per sub-block
  int rowA[4], rowB[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    rowA[a] = wm + a * 32 + l32;
    rowB[a] = wn + a * 32 + l32;
  }

  typedef typename Mfma<T>::frag frag_t;
  const int KE = ROW_BYTES / sizeof(T);
  const int nk = K / KE;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
    const unsigned char* sP = smem + (kt & 1) * STAGE_BYTES;
    const unsigned char* sQ = sP + OPERAND_BYTES;
    // fragments double-buffered across the four k16 steps of the slab: the reads of
    // step kk+1 are issued between the MFMAs of step kk
    frag_t fa[2][4], fb[2][4];
    auto read_frags = [&](int kk, frag_t* A, frag_t* B) {
      const int c = 2 * kk + half;
#pragma unroll
      for (int a = 0; a < 4; ++a)
        A[a] = *reinterpret_cast<const frag_t*>(sP + rowA[a] * ROW_BYTES + ((c ^ swz(rowA[a])) << 4));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        B[b] = *reinterpret_cast<const frag_t*>(sQ + rowB[b] * ROW_BYTES + ((c ^ swz(rowB[b])) << 4));
    };
    read_frags(0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      if (kk < 3) read_frags(kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) Mfma<T>::mma(acc[a][b], fa[cur][a], fb[cur][b]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue.  Accumulator layout of a 32x32 MFMA block: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  if (MODE == GM_SYRK || MODE == GM_POLY) {
    T* C = static_cast<T*>(MODE == GM_SYRK ? d.A : d.B);
    const T* Ain = static_cast<const T*>(d.A);
    const int64_t ld = d.mp;
    const bool diag = (ti == tj);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ib = i0 + wm + a * 32 + 8 * g + 4 * half;
          const int j = j0 + wn + b * 32 + l32;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[t] = acc[a][b][4 * g + t];
            if (MODE == GM_POLY) v[t] = cb * to_f32(Ain[(ib + t) * ld + j]) + cc * v[t];
          }
          if (!diag) {
#pragma unroll
            for (int t = 0; t < 4; ++t) C[(ib + t) * ld + j] = from_f32<T>(v[t]);
            store4<T>(C + static_cast<int64_t>(j) * ld + ib, v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int i = ib + t;
              if (i <= j) {
                const T x = from_f32<T>(v[t]);
                C[static_cast<int64_t>(i) * ld + j] = x;
                C[static_cast<int64_t>(j) * ld + i] = x;
              }
            }
          }
        }
  } else {
    T* X = static_cast<T*>(d.X);
    T* XTn = static_cast<T*>(d.XT[parity ^ 1]);
    const int64_t ldx = d.np, ldt = d.mp;
    TO* out = static_cast<TO*>(d.out);
    const int m = d.m, n = d.n;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ib = i0 + wm + a * 32 + 8 * g + 4 * half;
          const int j = j0 + wn + b * 32 + l32;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            v[t] = ca * to_f32(X[static_cast<int64_t>(ib + t) * ldx + j]) + acc[a][b][4 * g + t];
          if (MODE == GM_APPLY) {
#pragma unroll
            for (int t = 0; t < 4; ++t) X[static_cast<int64_t>(ib + t) * ldx + j] = from_f32<T>(v[t]);
            store4<T>(XTn + static_cast<int64_t>(j) * ldt + ib, v[0], v[1], v[2], v[3]);
          } else if (j < n) {
            if (!d.transposed) {
              // out is m x n row-major
#pragma unroll
              for (int t = 0; t < 4; ++t)
                if (ib + t < m) out[static_cast<int64_t>(ib + t) * n + j] = from_f32<TO>(v[t]);
            } else {
              // out is n x m row-major: out[j][i]
              TO* o = out + static_cast<int64_t>(j) * m + ib;
              if (d.vec_ok && ib + 4 <= m) {
                store4<TO>(o, v[0], v[1], v[2], v[3]);
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  if (ib + t < m) o[t] = from_f32<TO>(v[t]);
              }
            }
          }
        }
  }
}

}  // namespace mo
