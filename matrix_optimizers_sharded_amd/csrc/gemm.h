// The three Newton-Schulz products as one MFMA GEMM core with three epilogues.
//
// Every product is C[i][j] = sum_k P[i][k] * Q[j][k] with both operands read along
// k-contiguous rows:
//   SYRK   A  = X X^T         P = Q = X (rows of X, k over n); upper tiles only,
//                             each off-diagonal tile also stored mirrored
//   POLY   B' = aI + bA + c A A   P = Q = A (A symmetric, so A A = A A^T); upper
//                             tiles, mirrored; b*A in the epilogue reads the same
//                             rounded A, and a is added on the diagonal (rows < m)
//   APPLY  X' = B' X = aX + (bA + cA^2) X   P = B', Q = X^T (the kernel keeps X^T
//                             as a second copy so this is k-contiguous too); the
//                             epilogue only stores: X' in place and X'^T to the
//                             other ping-pong buffer, or the final U to the caller.
// Folding a into B' removes every epilogue read from the largest product; it
// rounds a + B_ii to the compute dtype once instead of rounding B_ii.
// All workspace dims are multiples of 256, zero-padded, so the main loop needs no
// bounds checks; only the final write to the caller's buffer is clipped.
//
// Tiling (gfx950, wave64): 256x256 block tile; NWAVES = 8 waves in a 2 x 4 grid,
// each owning a 128 x 64 sub-tile = 4 x 2 MFMA 32x32 blocks (128 fp32 accumulators
// per lane), two waves per SIMD so that twice as many operand loads are in flight
// as with 4 waves of 128 x 128 (the operand stream into LDS, not the MFMA rate, is
// what bounds this kernel).  The k-loop streams 128-byte row slabs (64 bf16 or 32 fp32 of k) of both
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

// k-slab geometry: each operand row of a slab is ROW_BYTES (128: 64 bf16 / 32 fp32 of
// k), and NSTAGE slabs are in flight in an LDS ring, so the loads of slab t+NSTAGE-1
// overlap the MFMAs of slabs t .. t+NSTAGE-2.
#ifndef MO_GEMM_SLAB_BYTES
#define MO_GEMM_SLAB_BYTES 128
#endif
#ifndef MO_GEMM_STAGES
#define MO_GEMM_STAGES 2
#endif
constexpr int ROW_BYTES = MO_GEMM_SLAB_BYTES;
constexpr int CHUNKS = ROW_BYTES / 16;                 // 16-byte chunks per row
constexpr int KSTEPS = CHUNKS / 2;                     // k16 MFMA steps per slab
constexpr int NSTAGE = MO_GEMM_STAGES;
constexpr int OPERAND_BYTES = GT * ROW_BYTES;
constexpr int STAGE_BYTES = 2 * OPERAND_BYTES;         // P and Q
constexpr int GEMM_LDS_BYTES = NSTAGE * STAGE_BYTES;
#ifndef MO_GEMM_WAVES
#define MO_GEMM_WAVES 8
#endif
constexpr int NWAVES = MO_GEMM_WAVES;                  // 8 (4 builds and is slower)
constexpr int NTHREADS = 64 * NWAVES;
constexpr int WAVES_N = NWAVES / 2;                    // wave grid: 2 x WAVES_N
constexpr int WAVE_N = GT / WAVES_N;                   // columns per wave: 128 or 64
constexpr int NB = WAVE_N / 32;                        // 32-column MFMA blocks per wave
constexpr int ROWS_PER_INST = 1024 / ROW_BYTES;        // rows one 1 KiB wave load fills
constexpr int INST_PER_OPERAND = OPERAND_BYTES / 1024 / NWAVES;  // per wave, per slab
constexpr int INST_PER_SLAB = 2 * INST_PER_OPERAND;
static_assert(GEMM_LDS_BYTES <= 160 * 1024, "LDS ring exceeds 160 KiB");
static_assert(NSTAGE * (ROW_BYTES / 2) <= 256, "the ring must not be deeper than the shortest K (256)");
static_assert(INST_PER_SLAB * (NSTAGE - 1) < 64, "vmcnt is a 6-bit field");

// raw-buffer resource word 3 for gfx9-family: 32-bit data format, no swizzle
constexpr int RSRC_FLAGS = 0x00020000;

// 16-byte chunk swizzle inside a row, chosen so that the fragment reads of 8
// consecutive rows (32 banks x 4 B) and of 16 consecutive rows (64 banks) fall in
// distinct banks.
__device__ inline int swz(int r) {
  if (CHUNKS == 8) return (r ^ (r >> 1)) & 7;
  return ((r >> 1) ^ (r >> 3)) & 3;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt immediate (gfx9 encoding): vmcnt = N (bits 3:0 and 15:14), expcnt = 7
// (no wait), lgkmcnt = 0
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }

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

// Tile order inside one matrix: rows of tiles are cut into bands of BAND rows; a
// band is walked column by column, top to bottom within a column.  Consecutive
// items (which run at the same time on one XCD) then form a BAND x 8 block whose
// operand row-panels are shared through that XCD's L2.
#ifndef MO_GEMM_BAND
#define MO_GEMM_BAND 4
#endif
#ifndef MO_GEMM_XCD_REMAP
#define MO_GEMM_XCD_REMAP 1
#endif
constexpr int BAND = MO_GEMM_BAND;

__device__ inline void rect_tile(int64_t local, int tm, int tn, int& ti, int& tj) {
  const int64_t per_band = static_cast<int64_t>(BAND) * tn;
  const int b = static_cast<int>(local / per_band);
  const int r = static_cast<int>(local - b * per_band);
  const int h = min(BAND, tm - b * BAND);
  tj = r / h;
  ti = b * BAND + r % h;
}

// Upper triangle (ti <= tj) of a T x T tile grid in the same banded order.
__device__ inline void upper_tile(int64_t local, int T, int& ti, int& tj) {
  int b = 0;
  for (;; ++b) {
    const int h = min(BAND, T - b * BAND);
    const int64_t n = static_cast<int64_t>(h) * (h + 1) / 2 + static_cast<int64_t>(T - b * BAND - h) * h;
    if (local < n) break;
    local -= n;
  }
  const int r0 = b * BAND, h = min(BAND, T - r0);
  // first h columns of the band hold 1, 2, ..., h tiles; the rest hold h
  int c = 0;
  for (; c < h; ++c) {
    if (local < c + 1) break;
    local -= c + 1;
  }
  if (c < h) {
    ti = r0 + static_cast<int>(local);
    tj = r0 + c;
  } else {
    tj = r0 + h + static_cast<int>(local / h);
    ti = r0 + static_cast<int>(local % h);
  }
}

// Blocks are dealt to the 8 XCDs round-robin (block b -> XCD b % 8).  Remap so that
// XCD x receives runs of XCD_CHUNK consecutive work items (chunks dealt round-robin
// over the XCDs): the blocks one XCD runs at a time are neighbours in the work
// list and share operand panels in that XCD's L2, while all XCDs still progress
// through the list together (equal load).
#ifndef MO_GEMM_XCD_CHUNK
#define MO_GEMM_XCD_CHUNK 32
#endif
__device__ inline int64_t xcd_remap(int64_t b, int64_t total) {
  constexpr int64_t G = MO_GEMM_XCD_CHUNK;
  const int64_t full = total / (8 * G) * (8 * G);   // blocks in complete rounds
  if (b >= full) return b;                          // ragged tail: identity
  const int64_t x = b % 8, k = b / 8;               // k-th block of XCD x
  return (k / G) * (8 * G) + x * G + (k % G);
}

template <typename T> struct Vec4;
template <> struct Vec4<bf16_t> { typedef bf16x4_t type; };
template <> struct Vec4<float> { typedef f32x4_t type; };

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
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(NWAVES / 4, NWAVES / 4)))
void k_ns_gemm(const MatDesc* __restrict__ descs, int count,
                                                    int parity, float ca, float cb, float cc) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[GEMM_LDS_BYTES];
  constexpr int kind = (MODE == GM_SYRK) ? KIND_SYRK : (MODE == GM_POLY) ? KIND_POLY : KIND_APPLY;
  const int64_t item = MO_GEMM_XCD_REMAP ? xcd_remap(blockIdx.x, gridDim.x) : static_cast<int64_t>(blockIdx.x);
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
    ldp = ldq = d.ldx;
    K = d.np;
  } else if (MODE == GM_POLY) {
    upper_tile(local, d.mp / GT, ti, tj);
    P = Q = static_cast<const T*>(d.A);
    ldp = ldq = d.ldm;
    K = d.mp;
  } else {
    rect_tile(local, d.mp / GT, d.np / GT, ti, tj);
    P = static_cast<const T*>(d.B);
    Q = static_cast<const T*>(d.XT[parity]);
    ldp = ldq = d.ldm;
    K = d.mp;
  }
  const int i0 = ti * GT, j0 = tj * GT;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = (wave / WAVES_N) * 128, wn = (wave % WAVES_N) * WAVE_N;

  // Direct-to-LDS loads: wave w, instruction q fills ROWS_PER_INST rows starting at
  // ROWS_PER_INST*(NWAVES*q+w) of an operand slab, 1 KiB contiguous in LDS (lane l ->
  // row + l/CHUNKS, physical chunk l%CHUNKS); the lane fetches the logical chunk
  // that the swizzle stores there.
  const uint32_t esz = sizeof(T);
  const uint32_t rowsP = d.mp;   // X, A and B all have mp rows
  const uint32_t rowsQ = (MODE == GM_APPLY || MODE == GM_APPLY_FINAL) ? d.np : d.mp;
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(P), 0, static_cast<int>(rowsP * static_cast<uint32_t>(ldp) * esz), RSRC_FLAGS);
  const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(Q), 0, static_cast<int>(rowsQ * static_cast<uint32_t>(ldq) * esz), RSRC_FLAGS);
  // Rows advance by ROWS_PER_INST * NWAVES between a wave's instructions, a multiple
  // of 16, which leaves the swizzle unchanged: one base offset per operand plus a
  // uniform stride per instruction.
  const int row0 = ROWS_PER_INST * wave + lane / CHUNKS;
  const uint32_t vP0 = static_cast<uint32_t>(i0 + row0) * static_cast<uint32_t>(ldp) * esz +
                       (((lane % CHUNKS) ^ swz(row0)) << 4);
  const uint32_t vQ0 = static_cast<uint32_t>(j0 + row0) * static_cast<uint32_t>(ldq) * esz +
                       (((lane % CHUNKS) ^ swz(row0)) << 4);
  const uint32_t vPs = static_cast<uint32_t>(ROWS_PER_INST * NWAVES) * static_cast<uint32_t>(ldp) * esz;
  const uint32_t vQs = static_cast<uint32_t>(ROWS_PER_INST * NWAVES) * static_cast<uint32_t>(ldq) * esz;
  auto issue = [&](int kt, int stage) {
    const int soff = kt * ROW_BYTES;
    unsigned char* base = smem + stage * STAGE_BYTES + wave * 1024;
#pragma unroll
    for (int q = 0; q < INST_PER_OPERAND; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (lds_ptr_t)(base + q * NWAVES * 1024), 16, vP0 + q * vPs,
                                               soff, 0, 0);
#pragma unroll
    for (int q = 0; q < INST_PER_OPERAND; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (lds_ptr_t)(base + OPERAND_BYTES + q * NWAVES * 1024), 16,
                                               vQ0 + q * vQs, soff, 0, 0);
  };

  f32x16_t acc[4][NB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // fragment read offsets (row part), per sub-block
  int rowA[4], rowB[NB];
#pragma unroll
  for (int a = 0; a < 4; ++a) rowA[a] = wm + a * 32 + l32;
#pragma unroll
  for (int b = 0; b < NB; ++b) rowB[b] = wn + b * 32 + l32;

  typedef typename Mfma<T>::frag frag_t;
  const int KE = ROW_BYTES / sizeof(T);
  const int nk = K / KE;   // >= NSTAGE: K >= 256, KE <= 64 and NSTAGE <= 4 for 128-byte rows

  // Pipeline per slab kt (stage kt % NSTAGE), fragments double-buffered over the
  // k16 steps: steps 0..KSTEPS-2 read the next step's fragments, then run 16 MFMAs;
  // then wait for this wave's loads of slab kt+1 and its own LDS reads, one barrier
  // (slab kt+1 is in LDS for everyone, and nobody reads slab kt any more), start the
  // loads of slab kt+NSTAGE into slab kt's stage, read slab kt+1's first fragments;
  // the last step's 16 MFMAs hide that barrier and those reads.  A slab's loads
  // have NSTAGE-1 slabs of MFMA work to land.
  frag_t fa[2][4], fb[2][NB];
  auto read_frags = [&](const unsigned char* sP, int kk, frag_t* A, frag_t* B) {
    const unsigned char* sQ = sP + OPERAND_BYTES;
    const int c = 2 * kk + half;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      A[a] = *reinterpret_cast<const frag_t*>(sP + rowA[a] * ROW_BYTES + ((c ^ swz(rowA[a])) << 4));
#pragma unroll
    for (int b = 0; b < NB; ++b)
      B[b] = *reinterpret_cast<const frag_t*>(sQ + rowB[b] * ROW_BYTES + ((c ^ swz(rowB[b])) << 4));
  };
  auto mfma_step = [&](const frag_t* A, const frag_t* B) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) Mfma<T>::mma(acc[a][b], A[a], B[b]);
  };
#pragma unroll
  for (int sidx = 0; sidx < NSTAGE; ++sidx) issue(sidx, sidx);   // nk >= NSTAGE
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(INST_PER_SLAB * (NSTAGE - 1)));
  __syncthreads();
  read_frags(smem, 0, fa[0], fb[0]);
  int stage = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const unsigned char* sP = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < KSTEPS - 1; ++kk) {
      read_frags(sP, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(fa[kk & 1], fb[kk & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int next = (stage + 1 == NSTAGE) ? 0 : stage + 1;
    // The block below runs on every slab, the last one included (where it reads
    // stale, unused fragments), so that the wait counters the last step's MFMAs
    // see do not depend on the path taken.  Slab kt+1 must have landed; slabs
    // kt+2 .. kt+NSTAGE-1 may still be in flight.
    if (kt + NSTAGE - 1 < nk)
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(INST_PER_SLAB * (NSTAGE - 2)));
    else
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    __syncthreads();
    if (kt + NSTAGE < nk) issue(kt + NSTAGE, stage);
    read_frags(smem + next * STAGE_BYTES, 0, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(fa[(KSTEPS - 1) & 1], fb[(KSTEPS - 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    stage = next;
  }

  // Epilogue.  Accumulator layout of a 32x32 MFMA block: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32, so each lane owns 4 consecutive rows
  // ib..ib+3 of one column j per register group g.  Values the epilogue needs at
  // [ib..ib+3][j] are read as one vector from a transposed copy: A[j][ib..] (A is
  // symmetric) for POLY and X^T[j][ib..] for APPLY.  Loads are issued a whole
  // sub-block row (16 vectors) at a time before any of them is used.
  typedef typename Vec4<T>::type v4_t;
  const int64_t ldt = d.ldm;
  if (MODE == GM_SYRK || MODE == GM_POLY) {
    T* C = static_cast<T*>(MODE == GM_SYRK ? d.A : d.B);
    const T* Ain = static_cast<const T*>(d.A);
    const bool diag = (ti == tj);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      v4_t e[NB][4];
      if (MODE == GM_POLY) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int ib = i0 + wm + a * 32 + 8 * g + 4 * half;
            const int j = j0 + wn + b * 32 + l32;
            e[b][g] = *reinterpret_cast<const v4_t*>(Ain + static_cast<int64_t>(j) * ldt + ib);
          }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ib = i0 + wm + a * 32 + 8 * g + 4 * half;
          const int j = j0 + wn + b * 32 + l32;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[t] = acc[a][b][4 * g + t];
            if (MODE == GM_POLY) {
              v[t] = cb * to_f32(e[b][g][t]) + cc * v[t];
              if (diag && ib + t == j && j < d.m) v[t] += ca;
            }
          }
          if (!diag) {
#pragma unroll
            for (int t = 0; t < 4; ++t) C[static_cast<int64_t>(ib + t) * ldt + j] = from_f32<T>(v[t]);
            store4<T>(C + static_cast<int64_t>(j) * ldt + ib, v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int i = ib + t;
              if (i <= j) {
                const T x = from_f32<T>(v[t]);
                C[static_cast<int64_t>(i) * ldt + j] = x;
                C[static_cast<int64_t>(j) * ldt + i] = x;
              }
            }
          }
        }
    }
  } else {
    T* X = static_cast<T*>(d.X);
    T* XTn = static_cast<T*>(d.XT[parity ^ 1]);
    const int64_t ldx = d.ldx;
    TO* out = static_cast<TO*>(d.out);
    const int m = d.m, n = d.n;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ib = i0 + wm + a * 32 + 8 * g + 4 * half;
          const int j = j0 + wn + b * 32 + l32;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = acc[a][b][4 * g + t];
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
}

}  // namespace mo
