// HBM-streaming kernels: the fused momentum + operand pass (and the momentum +
// sum-of-squares pass of the iters == 0 path), the per-matrix scale, the scaled
// operand writer for out-of-range norms, and the sign pack / vote.
#pragma once

#include <type_traits>

#include "common.h"

namespace mo {

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Fixed-order block sum for 256 threads (4 waves); result valid in thread 0.
template <typename T>
__device__ inline T block_sum_256(T v) {
  __shared__ T part[4];
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = 0;
  if (threadIdx.x == 0) r = ((part[0] + part[1]) + part[2]) + part[3];
  return r;
}

template <typename T> __device__ inline f32x4_t load4_f32(const T* p);
template <> __device__ inline f32x4_t load4_f32<float>(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}
template <> __device__ inline f32x4_t load4_f32<bf16_t>(const bf16_t* p) {
  bf16x4_t v = *reinterpret_cast<const bf16x4_t*>(p);
  return f32x4_t{static_cast<float>(v[0]), static_cast<float>(v[1]),
                 static_cast<float>(v[2]), static_cast<float>(v[3])};
}

// Non-temporal forms of load4_f32 (whole-line reads of data used once).
template <typename T> __device__ inline f32x4_t load4_f32_nt(const T* p);
template <> __device__ inline f32x4_t load4_f32_nt<float>(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
}
template <> __device__ inline f32x4_t load4_f32_nt<bf16_t>(const bf16_t* p) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return f32x4_t{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                 __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
}

// Pass 1, one 4096-element chunk per block.  With MOMENTUM: M <- fma(beta, M, G)
// in place, and the chunk's sum of M^2 goes to partial[item].  Without: the sum of
// squares of the input only.  The squares are summed in fp64: exact products, and
// no overflow for any finite fp32 value (fp32 squares overflow from |M| ~ 1.8e19);
// the kernel is bound by HBM, so the fp64 arithmetic costs nothing.
template <typename TG, bool MOMENTUM>
__global__ __launch_bounds__(256) void k_momentum_sumsq(const MatDesc* __restrict__ descs,
                                                        int count, float beta,
                                                        double* __restrict__ partial) {
  const int64_t item = blockIdx.x;
  const MatDesc& d = descs[find_desc(descs, count, KIND_CHUNK, item)];
  const int64_t e0 = (item - d.begin[KIND_CHUNK]) * CHUNK;
  const int64_t numel = d.numel;
  const TG* __restrict__ g = static_cast<const TG*>(d.grad);
  float* __restrict__ m = d.mom;
  double ss = 0.0;
  if (d.vec_ok && e0 + CHUNK <= numel) {
    f32x4_t gv[4], mv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) gv[q] = load4_f32<TG>(g + e0 + q * 1024 + threadIdx.x * 4);
    if (MOMENTUM) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        mv[q] = *reinterpret_cast<const f32x4_t*>(m + e0 + q * 1024 + threadIdx.x * 4);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4_t v = gv[q];
      if (MOMENTUM) {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(beta, mv[q][t], gv[q][t]);
        *reinterpret_cast<f32x4_t*>(m + e0 + q * 1024 + threadIdx.x * 4) = v;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) ss = __builtin_fma(static_cast<double>(v[t]), static_cast<double>(v[t]), ss);
    }
  } else {
    const int64_t e1 = (e0 + CHUNK < numel) ? e0 + CHUNK : numel;
    for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) {
      float v = static_cast<float>(g[e]);
      if (MOMENTUM) {
        v = __builtin_fmaf(beta, m[e], v);
        m[e] = v;
      }
      ss = __builtin_fma(static_cast<double>(v), static_cast<double>(v), ss);
    }
  }
  ss = block_sum_256(ss);
  if (threadIdx.x == 0) partial[item] = ss;
}

// Norms inside [2^-20, 2^40] leave the unscaled operand safe for the first products:
// every |A_ij| <= ||M||_F^2 <= 2^80 accumulates in fp32 without overflow, and the
// typical element (at least ||M||_F / 2^13 for up to 2^26 elements) squares to well
// above fp32's smallest normal.
constexpr double DEFER_NORM_LO = 0x1p-20, DEFER_NORM_HI = 0x1p40;

// One block per matrix: scale = 1 / (sqrt(sum of partials) + eps), summed in fp64
// in a fixed order over the matrix's work items of launch kind `kind`.  With
// `first` (the fused momentum + operand pass wrote X unscaled): first[slot] is the
// factor the first NS products apply instead (scale, or 1 where the norm lies
// outside the deferral range), and redo[slot] = 1 marks the matrices whose operand
// k_prep_redo rewrites scaled.
__global__ __launch_bounds__(256) void k_norm_scale(const MatDesc* __restrict__ descs,
                                                    const double* __restrict__ partial, int kind,
                                                    float eps, float* __restrict__ scale,
                                                    float* __restrict__ first, int* __restrict__ redo) {
  const MatDesc& d = descs[blockIdx.x];
  double s = 0.0;
  const double* p = partial + d.begin[kind];
  for (int64_t c = threadIdx.x; c < d.items[kind]; c += 256) s += p[c];
  s = block_sum_256(s);
  if (threadIdx.x == 0) {
    const double norm = sqrt(s);
    const float sc = static_cast<float>(1.0 / (norm + static_cast<double>(eps)));
    scale[d.scale_slot] = sc;
    if (first) {
      const bool defer = norm >= DEFER_NORM_LO && norm <= DEFER_NORM_HI;
      first[d.scale_slot] = defer ? sc : 1.f;
      redo[d.scale_slot] = defer ? 0 : 1;
    }
  }
}

// The operand writers below fill X (mp x np, compute dtype, zero outside the m x n
// corner) one 64x64 tile per block.  Eight consecutive values go out with 16-byte
// stores (the address is 16-byte aligned: workspace rows are multiples of 128 bytes
// and b is a multiple of 8).
template <typename T>
__device__ inline void store8(gptr<T> p, const float (&v)[8]);
// The bf16 form stores non-temporally: X is written once per pass and the NS
// products read it back from HBM (an owner set's operands exceed the caches).
template <>
__device__ inline void store8<bf16_t>(gptr<bf16_t> p, const float (&v)[8]) {
  bf16x8_t x;
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = static_cast<bf16_t>(v[k]);
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, x), reinterpret_cast<gptr<u32x4_t>>(p));
}
template <>
__device__ inline void store8<float>(gptr<float> p, const float (&v)[8]) {
  reinterpret_cast<gptr<f32x4_t>>(p)[0] = f32x4_t{v[0], v[1], v[2], v[3]};
  reinterpret_cast<gptr<f32x4_t>>(p)[1] = f32x4_t{v[4], v[5], v[6], v[7]};
}

// Writes X[i0 + a][j0 + b] for a 64 x 64 tile from tile[][] (source orientation):
// eight consecutive outputs per thread and store, a row piece X[i0 + a][j0 + b ..]
// (a column piece of the tile when the source is transposed; the padded tile, +1
// column, keeps those reads free of bank conflicts).  X is k-blocked along its
// columns, and eight consecutive columns from a multiple of 8 never straddle a
// k-block.
template <typename TC>
__device__ inline void write_operand_tile(const MatDesc& d, int i0, int j0,
                                          const float (&tile)[PREP_TILE][PREP_TILE + 1]) {
  const int t = threadIdx.x;
  unsigned char* const X = static_cast<unsigned char*>(d.X[0]);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int a = (t >> 3) + 32 * q, b = (t & 7) * 8;
    float vx[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) vx[k] = d.transposed ? tile[b + k][a] : tile[a][b + k];
    store8<TC>(global(reinterpret_cast<TC*>(X + kb_off<TC>(i0 + a, j0 + b, d.pX))), vx);
  }
}

// The fused first pass of a step with at least one NS iteration, MP_TPB = 4 64x64
// tiles of the padded oriented operand per block (256 threads; the item count of
// every matrix is a multiple of 16 and its tile grid a multiple of 4 in each
// direction, so a block's tiles never leave their matrix): with MOMENTUM,
// M <- fma(beta, M, G) in place over the tiles' source elements; X = M (or the
// input), unscaled, in the compute dtype, zero outside the m x n corner; and the
// block's fp64 sum of squares to partial[first item] (0 to the others).  One HBM
// sweep: G and M read once, M and X written once.  The Frobenius scale s comes
// afterwards, applied by the first NS products (s^2 on X X^T, s on the first B X),
// which in exact arithmetic is the same as scaling X first: (sX)(sX)^T = s^2 X X^T
// and B'(sX) = s B'X.
// Four tiles per block (2 blocks per CU by LDS) measured fastest: 5.1-5.7 TB/s
// against 4.7-5.3 TB/s with one tile per block at the 7B-class owner set, as more
// of each thread's loads are in flight before its first store.  Every access of the
// whole-tile path covers whole 128-byte lines per instruction, and all of them are
// non-temporal (G, M read once; M, X written once and not read again in this pass):
// 12.3-13.2 ms per pass at the 7B-class set against 14.0-15.2 ms with ordinary
// accesses (two boxes, three rounds each); non-temporal loads alone gave 12.8-14.9.
constexpr int MP_TPB = 4;
template <typename TG, typename TC, bool MOMENTUM>
__global__ __launch_bounds__(256) void k_momentum_prep(const MatDesc* __restrict__ descs, int count,
                                                       float beta, double* __restrict__ partial) {
  __shared__ float tile[MP_TPB][PREP_TILE][PREP_TILE + 1];
  const int64_t item = static_cast<int64_t>(blockIdx.x) * MP_TPB;
  const MatDesc& d = descs[find_desc(descs, count, KIND_PREP, item)];
  const int64_t local = item - d.begin[KIND_PREP];
  // Tile arrangement (MP_TPB = 4 tiles per block, consecutive blocks next to each
  // other along the source's rows):
  //   X = S^T (rows of X are columns of S): tiles u at X rows ib + 64u, so each row
  //     of S is read in 1 KiB runs and 256 consecutive rows of one k-block of X are
  //     written; against tiles along X columns 14.7-15.8 -> 13.4-13.7 ms per pass at
  //     the 7B-class set (its transposed matrices hold 22% of the elements).
  //   X = S: a 2 x 2 group (128 x 128 of X): 512-byte runs of S's rows, and 128
  //     consecutive rows in each of two k-blocks of X; against 1 x 4 tiles along X
  //     columns (1 KiB runs, four k-blocks) 14.5-15.4 -> 13.3-13.6 ms, one box.
  const bool along_rows = d.transposed;
  const int tn = d.np / PREP_TILE, tmr = d.mp / PREP_TILE;   // multiples of 4
  const int64_t grp = local / 4;                               // 2 x 2 groups over (tmr/2) x (tn/2)
  const int ib = along_rows ? static_cast<int>(local % tmr) * PREP_TILE
                            : static_cast<int>(grp / (tn / 2)) * 2 * PREP_TILE;
  const int jb = along_rows ? static_cast<int>(local / tmr) * PREP_TILE
                            : static_cast<int>(grp % (tn / 2)) * 2 * PREP_TILE;
  auto tile_i0 = [&](int u) { return along_rows ? ib + PREP_TILE * u : ib + PREP_TILE * (u >> 1); };  // rows of X
  auto tile_j0 = [&](int u) { return along_rows ? jb : jb + PREP_TILE * (u & 1); };                 // cols of X
  const int t = threadIdx.x;
  const int64_t ld = d.cols;
  const int64_t rlim = d.rows, clim = d.cols;
  const TG* __restrict__ g = static_cast<const TG*>(d.grad);
  float* __restrict__ m = d.mom;
  // source rows/cols of tile u: X[i][j] = S[i][j] (not transposed) or S[j][i]
  auto src_r0 = [&](int u) { return d.transposed ? tile_j0(u) : tile_i0(u); };
  auto src_c0 = [&](int u) { return d.transposed ? tile_i0(u) : tile_j0(u); };
  bool inside = d.vec_ok;
#pragma unroll
  for (int u = 0; u < MP_TPB; ++u)
    inside = inside && src_r0(u) + PREP_TILE <= rlim && src_c0(u) + PREP_TILE <= clim;
  double ss = 0.0;
  if (inside) {
    // whole tiles inside the source: four consecutive elements per thread and load,
    // all loads of the thread issued before the first store
    f32x4_t gv[MP_TPB][4], mv[MP_TPB][4];
#pragma unroll
    for (int u = 0; u < MP_TPB; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int a = (t >> 4) + 16 * q, b = (t & 15) * 4;
        const int64_t e = (src_r0(u) + a) * ld + src_c0(u) + b;
        gv[u][q] = load4_f32_nt<TG>(g + e);
        if (MOMENTUM) mv[u][q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(m + e));
      }
#pragma unroll
    for (int u = 0; u < MP_TPB; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int a = (t >> 4) + 16 * q, b = (t & 15) * 4;
        f32x4_t v = gv[u][q];
        if (MOMENTUM) {
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = __builtin_fmaf(beta, mv[u][q][k], gv[u][q][k]);
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(m + (src_r0(u) + a) * ld + src_c0(u) + b));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ss = __builtin_fma(static_cast<double>(v[k]), static_cast<double>(v[k]), ss);
          tile[u][a][b + k] = v[k];
        }
      }
  } else {
    const int tx = t & 63, ty = t >> 6;
    for (int u = 0; u < MP_TPB; ++u) {
      const int r0 = src_r0(u), c0 = src_c0(u);
#pragma unroll 4
      for (int q = 0; q < 16; ++q) {
        const int a = ty + 4 * q;
        const int64_t r = r0 + a, c = c0 + tx;
        float v = 0.f;
        if (r < rlim && c < clim) {
          v = static_cast<float>(g[r * ld + c]);
          if (MOMENTUM) {
            v = __builtin_fmaf(beta, m[r * ld + c], v);
            m[r * ld + c] = v;
          }
        }
        ss = __builtin_fma(static_cast<double>(v), static_cast<double>(v), ss);
        tile[u][a][tx] = v;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < MP_TPB; ++u) write_operand_tile<TC>(d, tile_i0(u), tile_j0(u), tile[u]);
  ss = block_sum_256(ss);
  if (t < MP_TPB) partial[item + t] = t == 0 ? ss : 0.0;
}

// X = S * scale for the matrices flagged in redo[] (their norm lies outside the range
// where the first products may take the scale, see k_norm_scale): S is the updated
// momentum or the input, X the padded oriented operand in the compute dtype.  The
// grid strides over each flagged matrix's 64x64 tiles; a block first checks 256
// flags at a time, so with nothing flagged the launch costs a few microseconds.  The
// source tile is read along its contiguous dimension and X is written along its own,
// through an LDS tile (the source is the transpose of X when rows > cols).
template <typename TS, typename TC>
__global__ __launch_bounds__(256) void k_prep_redo(const MatDesc* __restrict__ descs, int count,
                                                   const float* __restrict__ scale,
                                                   const int* __restrict__ redo, int from_momentum) {
  __shared__ float tile[PREP_TILE][PREP_TILE + 1];
  const int t = threadIdx.x;
  for (int c0 = 0; c0 < count; c0 += 256) {
    const int c = c0 + t;
    if (!__syncthreads_or(c < count && redo[descs[c].scale_slot])) continue;
    const int c1 = c0 + 256 < count ? c0 + 256 : count;
    for (int k = c0; k < c1; ++k) {
      const MatDesc& d = descs[k];
      if (!redo[d.scale_slot]) continue;
      const float s = scale[d.scale_slot];
      const int tn = d.np / PREP_TILE;
      const int64_t ld = d.cols, rlim = d.rows, clim = d.cols;
      const float* sm = d.mom;
      const TS* sx = static_cast<const TS*>(d.grad);
      for (int64_t local = blockIdx.x; local < d.items[KIND_PREP]; local += gridDim.x) {
        const int i0 = static_cast<int>(local / tn) * PREP_TILE;
        const int j0 = static_cast<int>(local % tn) * PREP_TILE;
        const int r0 = d.transposed ? j0 : i0, cc0 = d.transposed ? i0 : j0;
        const int tx = t & 63, ty = t >> 6;
        for (int q = 0; q < 16; ++q) {
          const int a = ty + 4 * q;
          const int64_t r = r0 + a, cc = cc0 + tx;
          float v = 0.f;
          if (r < rlim && cc < clim) v = from_momentum ? sm[r * ld + cc] : static_cast<float>(sx[r * ld + cc]);
          tile[a][tx] = v * s;
        }
        __syncthreads();
        write_operand_tile<TC>(d, i0, j0, tile);
        __syncthreads();   // the next tile overwrites tile[][]
      }
    }
  }
}

// iters == 0: out = S * scale in the caller's orientation and out dtype, or, when
// applying to a weight, out <- out - lr * S * scale.
template <typename TS, typename TO>
__global__ __launch_bounds__(256) void k_scaled_copy(const MatDesc* __restrict__ descs, int count,
                                                     const float* __restrict__ scale,
                                                     int from_momentum, int apply, float lr) {
  const int64_t item = blockIdx.x;
  const MatDesc& d = descs[find_desc(descs, count, KIND_CHUNK, item)];
  const int64_t e0 = (item - d.begin[KIND_CHUNK]) * CHUNK;
  const int64_t e1 = (e0 + CHUNK < d.numel) ? e0 + CHUNK : d.numel;
  const float s = scale[d.scale_slot];
  TO* out = static_cast<TO*>(d.out);
  const TS* sx = static_cast<const TS*>(d.grad);
  for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) {
    const float v = (from_momentum ? d.mom[e] : static_cast<float>(sx[e])) * s;
    out[e] = from_f32<TO>(apply ? to_f32(out[e]) - lr * v : v);
  }
}

// ---------------------------------------------------------------------------
// Sign-Muon tail.

// 16-byte pieces per lane (see below).  Measured at 2^28 elements, each kernel
// timed right after the others in a pack/vote/unpack/apply loop, three rounds on
// one box: sign_unpack (bf16 out) 1 piece 7.09-7.19 TB/s, 2 pieces 5.97-6.09,
// 4 pieces 5.92-6.05, 8 pieces 5.63-5.73; sign_apply (fp32 weight) 1 piece
// 6.49-6.54, 2 pieces 6.18-6.22, 4 pieces 6.13-6.17.  sign_pack (below) wants 2
// loads per lane: 6.45-6.52 TB/s against 5.19-5.21 with 1.
constexpr int UNPACK_PIECES = 1;
constexpr int SAPPLY_PIECES = 1;

// sign_pack: each lane of a wave reads PACK_LOADS 16-byte pieces (4 fp32 or 8 bf16
// elements each), the 64 lanes of one load on 64 consecutive pieces, so that every
// load instruction reads 1 KiB of whole cache lines.  The loads are non-temporal:
// with ordinary loads the pack ran at 6.3 TB/s on its own but 4.7 TB/s right after a
// kernel that had written 1 GiB (the tail of an optimizer step), against 6.4 and
// 6.1 TB/s non-temporal (2^28 fp32 elements).  Non-temporal loads of pieces that do
// not cover whole lines per instruction were slower than ordinary ones.
constexpr int PACK_LOADS = 2;

// Sign bits of the 16 / sizeof(T) elements of one 16-byte piece as loaded (bit k =
// element k >= 0; a bf16 value widens to fp32 exactly by moving it to the high half).
template <typename T>
__device__ inline uint32_t piece_bits(const u32x4_t v) {
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (sizeof(T) == 4) {
      bits |= static_cast<uint32_t>(__uint_as_float(v[q]) >= 0.f) << q;
    } else {
      bits |= static_cast<uint32_t>(__uint_as_float(v[q] << 16) >= 0.f) << (2 * q);
      bits |= static_cast<uint32_t>(__uint_as_float(v[q] & 0xFFFF0000u) >= 0.f) << (2 * q + 1);
    }
  }
  return bits;
}

// Element i -> bit i % 32 of word i / 32, bit = (u >= 0): the G = 32 / EPL lanes
// whose pieces make up one word OR their bits together.  Row y of the grid packs
// worker y: its numel values start at u + y * u_stride and its words at packed + y *
// nwords (the [M][nwords] stack a vote reads), so M workers take one launch.  A
// piece that runs past numel, or any piece when the rows are not 16-byte aligned,
// is read element by element; bits past numel stay 0.
template <typename T>
__global__ __launch_bounds__(256) void k_sign_pack(const T* __restrict__ u, int64_t u_stride, int64_t numel,
                                                   uint32_t* __restrict__ packed, int vec_ok) {
  constexpr int EPL = 16 / static_cast<int>(sizeof(T));   // elements per piece
  constexpr int G = 32 / EPL;                              // lanes per word
  const int lane = threadIdx.x & 63;
  const int64_t nwords = (numel + 31) >> 5;
  u += static_cast<int64_t>(blockIdx.y) * u_stride;
  packed += static_cast<int64_t>(blockIdx.y) * nwords;
  const int64_t load0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * PACK_LOADS;
  u32x4_t v[PACK_LOADS];
  bool full[PACK_LOADS];
#pragma unroll
  for (int h = 0; h < PACK_LOADS; ++h) {
    const int64_t e0 = ((load0 + h) * 64 + lane) * EPL;
    full[h] = vec_ok && e0 + EPL <= numel;
    if (full[h]) v[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(u + e0));
  }
#pragma unroll
  for (int h = 0; h < PACK_LOADS; ++h) {
    const int64_t e0 = ((load0 + h) * 64 + lane) * EPL;
    uint32_t bits = 0;
    if (full[h]) {
      bits = piece_bits<T>(v[h]);
    } else {
      for (int k = 0; k < EPL; ++k)
        if (e0 + k < numel) bits |= static_cast<uint32_t>(static_cast<float>(u[e0 + k]) >= 0.f) << k;
    }
    uint32_t w = bits << (EPL * (lane % G));
#pragma unroll
    for (int x = 1; x < G; x <<= 1) w |= __shfl_xor(w, x, 64);
    const int64_t word = e0 >> 5;
    if (lane % G == 0 && word < nwords) packed[word] = w;
  }
}

__device__ inline uint32_t lane_word(uint32_t v, int) { return v; }
__device__ inline uint32_t lane_word(const u32x4_t& v, int q) { return v[q]; }

// Loads of the vote: the four-word path reads 1 KiB of whole lines per instruction
// and loads non-temporally (as sign_pack does); the one-word path reads 256 bytes
// per instruction and loads normally.
__device__ inline uint32_t vote_load(const uint32_t* p) { return *p; }
__device__ inline u32x4_t vote_load(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

// Vote of one group of W (1 or 4) consecutive words: a bit-sliced counter of LV bit
// planes (2^LV > M) adds the M workers' words (all 32 bit positions of every word at
// once), and a bit-sliced compare gives count >= ceil(M/2), which is
// 2*count - M >= 0 (ties -> +1).  Loads are issued 8 workers at a time ahead of the
// additions.  V is uint32_t or a 4-vector of them.
template <typename V, int LV, int NG>
__device__ inline void vote_groups(const V* __restrict__ src, int64_t gstep, int64_t stride, int M,
                                   V (&cnt)[NG][LV], V (&res)[NG]) {
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int l = 0; l < LV; ++l) cnt[g][l] = V{} ^ V{};
  auto add = [&](V (&c)[LV], V carry) {
#pragma unroll
    for (int l = 0; l < LV; ++l) {
      const V o = c[l];
      c[l] = o ^ carry;
      carry = o & carry;
    }
  };
  int k = 0;
  for (; k + 8 <= M; k += 8) {
    V x[8][NG];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int g = 0; g < NG; ++g) x[u][g] = vote_load(src + g * gstep + static_cast<int64_t>(k + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int g = 0; g < NG; ++g) add(cnt[g], x[u][g]);
  }
  for (; k < M; ++k)
#pragma unroll
    for (int g = 0; g < NG; ++g) add(cnt[g], vote_load(src + g * gstep + static_cast<int64_t>(k) * stride));
  // count >= T with T = ceil(M/2) <=> carry out of count + (2^LV - T)
  const uint32_t addend = (1u << LV) - static_cast<uint32_t>((M + 1) >> 1);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    V carry = V{} ^ V{};
#pragma unroll
    for (int l = 0; l < LV; ++l) {
      const V kbits = V{} ^ V{} ^ (((addend >> l) & 1u) ? 0xFFFFFFFFu : 0u);
      carry = (cnt[g][l] & kbits) | ((cnt[g][l] ^ kbits) & carry);
    }
    res[g] = carry;
  }
}

// int8 sums 2*count - M of the n (<= 32) elements of one word, word q of the group,
// from the counter's bit planes.
template <typename V, int LV>
__device__ inline void vote_sums(const V (&cnt)[LV], int q, int M, int n, int8_t* dst) {
  uint32_t planes[LV];
#pragma unroll
  for (int l = 0; l < LV; ++l) planes[l] = lane_word(cnt[l], q);
  for (int b = 0; b < n; ++b) {
    int c = 0;
#pragma unroll
    for (int l = 0; l < LV; ++l) c |= static_cast<int>((planes[l] >> b) & 1u) << l;
    dst[b] = static_cast<int8_t>(2 * c - M);
  }
}

// quad = 0: a thread votes one word.  quad = 1 (the buffers allow 16-byte loads): a
// thread votes one group of 4 words, a block 256 groups.  quad = 2: two groups 256
// apart, a block 512 groups, with twice the loads in flight per thread; 4% more
// bandwidth at 2^28 elements (5.8 against 5.6 TB/s), but 1 us slower at 2^24, where
// the vote is latency-bound and wants more blocks.  Pad bits of the last word are
// cleared.  LV bit planes count up to 2^LV - 1 workers; SUMS also writes the int8
// sums.
constexpr int64_t VOTE_PAIR_GROUPS = int64_t(1) << 20;
template <int LV, bool SUMS>
__global__ __launch_bounds__(256) void k_sign_vote(const uint32_t* __restrict__ packed, int M, int64_t numel,
                                                   int64_t nwords, uint32_t* __restrict__ out,
                                                   int8_t* __restrict__ out_sum, int quad) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  auto finish = [&](int64_t w, uint32_t word) {
    const int64_t tail = numel - w * 32;
    out[w] = tail < 32 ? word & ((1u << tail) - 1u) : word;
  };
  if (quad) {
    // nwords % 4 == 0: groups (four whole words) b * per + tid and, for quad = 2,
    // b * per + 256 + tid of block b, both in one pass where both exist
    const int64_t nq = nwords / 4;
    const int64_t qa = static_cast<int64_t>(blockIdx.x) * (quad == 2 ? 512 : 256) + threadIdx.x;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(packed);
    auto emit = [&](int64_t q4, const u32x4_t& v, const u32x4_t (&cnt)[LV]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        finish(q4 * 4 + q, v[q]);
        if (SUMS) {
          const int64_t tail = numel - (q4 * 4 + q) * 32;
          vote_sums<u32x4_t, LV>(cnt, q, M, tail < 32 ? static_cast<int>(tail) : 32, out_sum + (q4 * 4 + q) * 32);
        }
      }
    };
    if (quad == 2 && qa + 256 < nq) {
      u32x4_t cnt[2][LV], v[2];
      vote_groups<u32x4_t, LV, 2>(src + qa, 256, nq, M, cnt, v);
      emit(qa, v[0], cnt[0]);
      emit(qa + 256, v[1], cnt[1]);
    } else if (qa < nq) {
      u32x4_t cnt[1][LV], v[1];
      vote_groups<u32x4_t, LV, 1>(src + qa, 0, nq, M, cnt, v);
      emit(qa, v[0], cnt[0]);
    }
  } else {
    if (t >= nwords) return;
    uint32_t cnt[1][LV], v[1];
    vote_groups<uint32_t, LV, 1>(packed + t, 0, nwords, M, cnt, v);
    finish(t, v[0]);
    if (SUMS) {
      const int64_t tail = numel - t * 32;
      vote_sums<uint32_t, LV>(cnt[0], 0, M, tail < 32 ? static_cast<int>(tail) : 32, out_sum + t * 32);
    }
  }
}

// sign_unpack and sign_apply: each lane handles *_PIECES 16-byte pieces of the
// output (4 fp32 or 8 bf16 elements each), the 64 lanes of one access on 64
// consecutive pieces, so that each load and store instruction covers 1 KiB of whole
// lines; the lanes of one word read it together.  Output stores, and sign_apply's
// loads of the weight, are non-temporal.
template <typename T> __device__ inline uint32_t bits_of(T v) {
  if constexpr (sizeof(T) == 4) return __float_as_uint(v);
  else return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, v));
}
// element k of a 16-byte piece as fp32, and the piece with element k replaced
template <typename T> __device__ inline float piece_get(const u32x4_t& v, int k) {
  if constexpr (sizeof(T) == 4) return __uint_as_float(v[k]);
  else return __uint_as_float((k & 1) ? (v[k >> 1] & 0xFFFF0000u) : (v[k >> 1] << 16));
}
template <typename T> __device__ inline void piece_set(u32x4_t& v, int k, float x) {
  if constexpr (sizeof(T) == 4) {
    v[k] = __float_as_uint(x);
  } else {
    const uint32_t h = bits_of(static_cast<bf16_t>(x));
    v[k >> 1] = (k & 1) ? ((v[k >> 1] & 0xFFFFu) | (h << 16)) : ((v[k >> 1] & 0xFFFF0000u) | h);
  }
}

// The inverse of the packing, for the local polar step on the voted signs: element
// i <- +1 where bit i is set, else -1.
template <typename T>
__global__ __launch_bounds__(256) void k_sign_unpack(const uint32_t* __restrict__ packed, int64_t numel,
                                                     T* __restrict__ out, int vec_ok) {
  constexpr int EPL = 16 / static_cast<int>(sizeof(T));
  const int lane = threadIdx.x & 63;
  const int64_t load0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * UNPACK_PIECES;
  uint32_t words[UNPACK_PIECES];
#pragma unroll
  for (int h = 0; h < UNPACK_PIECES; ++h) {
    const int64_t e0 = ((load0 + h) * 64 + lane) * EPL;
    words[h] = e0 < numel ? packed[e0 >> 5] : 0u;
  }
#pragma unroll
  for (int h = 0; h < UNPACK_PIECES; ++h) {
    const int64_t e0 = ((load0 + h) * 64 + lane) * EPL;
    if (e0 >= numel) continue;
    const uint32_t bits = words[h] >> (e0 & 31);
    if (vec_ok && e0 + EPL <= numel) {
      u32x4_t v = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < EPL; ++k) piece_set<T>(v, k, ((bits >> k) & 1u) ? 1.f : -1.f);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + e0));
    } else {
      for (int k = 0; k < EPL && e0 + k < numel; ++k) out[e0 + k] = from_f32<T>(((bits >> k) & 1u) ? 1.f : -1.f);
    }
  }
}

// Sign-Muon parameter update W <- W - lr * S with S = +1 where bit i is set, else
// -1: the difference is formed in fp32 and stored in W's dtype.
template <typename T>
__global__ __launch_bounds__(256) void k_sign_apply(const uint32_t* __restrict__ packed, int64_t numel,
                                                    T* __restrict__ w, float lr, int vec_ok) {
  constexpr int EPL = 16 / static_cast<int>(sizeof(T));
  const int lane = threadIdx.x & 63;
  const int64_t load0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * SAPPLY_PIECES;
  uint32_t words[SAPPLY_PIECES];
  u32x4_t x[SAPPLY_PIECES];
  bool full[SAPPLY_PIECES];
#pragma unroll
  for (int h = 0; h < SAPPLY_PIECES; ++h) {
    const int64_t e0 = ((load0 + h) * 64 + lane) * EPL;
    words[h] = e0 < numel ? packed[e0 >> 5] : 0u;
    full[h] = vec_ok && e0 + EPL <= numel;
    if (full[h]) x[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(w + e0));
  }
#pragma unroll
  for (int h = 0; h < SAPPLY_PIECES; ++h) {
    const int64_t e0 = ((load0 + h) * 64 + lane) * EPL;
    if (e0 >= numel) continue;
    const uint32_t bits = words[h] >> (e0 & 31);
    if (full[h]) {
      u32x4_t y = x[h];
#pragma unroll
      for (int k = 0; k < EPL; ++k) piece_set<T>(y, k, piece_get<T>(x[h], k) - (((bits >> k) & 1u) ? lr : -lr));
      __builtin_nontemporal_store(y, reinterpret_cast<u32x4_t*>(w + e0));
    } else {
      for (int k = 0; k < EPL && e0 + k < numel; ++k)
        w[e0 + k] = from_f32<T>(to_f32(w[e0 + k]) - (((bits >> k) & 1u) ? lr : -lr));
    }
  }
}

}  // namespace mo
