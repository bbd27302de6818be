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
template <>
__device__ inline void store8<bf16_t>(gptr<bf16_t> p, const float (&v)[8]) {
  bf16x8_t x;
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = static_cast<bf16_t>(v[k]);
  *reinterpret_cast<gptr<bf16x8_t>>(p) = x;
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
// of each thread's loads are in flight before its first store.
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
        gv[u][q] = load4_f32<TG>(g + e);
        if (MOMENTUM) mv[u][q] = *reinterpret_cast<const f32x4_t*>(m + e);
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
          *reinterpret_cast<f32x4_t*>(m + (src_r0(u) + a) * ld + src_c0(u) + b) = v;
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

// The sign kernels work in units of 256 threads x 8 elements (one packed byte per
// thread); a block covers *_UNITS consecutive units, and each thread issues the
// loads of all its units before it stores anything.  Measured at 2^28 elements
// (fp32 pack input, bf16 unpack output), one box, three rounds each:
//   sign_pack    1 unit 4.73 TB/s; 2 units 4.50; 4 units 4.40
//   sign_unpack  1 unit 4.65 TB/s; 2 units 5.27; 4 units 5.46
//   sign_apply   1 unit 5.75 TB/s; 2 units 5.54; 4 units 5.33 (fp32 weight)
constexpr int PACK_UNITS = 1;
constexpr int UNPACK_UNITS = 4;
constexpr int SAPPLY_UNITS = 1;

// The byte of the 8 consecutive elements from e0 (bit k = (u[e0 + k] >= 0)).
template <typename T>
__device__ inline uint32_t sign_byte(const T* __restrict__ u, int64_t e0, int64_t numel, int vec_ok) {
  uint32_t byte = 0;
  if (vec_ok && e0 + 8 <= numel) {
    if (sizeof(T) == 4) {
      const f32x4_t* p = reinterpret_cast<const f32x4_t*>(u + e0);
      const f32x4_t x0 = p[0], x1 = p[1];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        byte |= static_cast<uint32_t>(x0[k] >= 0.f) << k;
        byte |= static_cast<uint32_t>(x1[k] >= 0.f) << (k + 4);
      }
    } else {
      const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(u + e0);
#pragma unroll
      for (int k = 0; k < 8; ++k) byte |= static_cast<uint32_t>(static_cast<float>(x[k]) >= 0.f) << k;
    }
  } else {
    for (int k = 0; k < 8; ++k) {
      const int64_t e = e0 + k;
      if (e < numel) byte |= static_cast<uint32_t>(static_cast<float>(u[e]) >= 0.f) << k;
    }
  }
  return byte;
}

// One thread per 8 consecutive elements of each unit -> one byte; 4 lanes OR their
// bytes into a 32-bit word (element i -> bit i % 32 of word i / 32).  bit = (u >= 0).
// Row y of the grid packs worker y: its numel values start at u + y * u_stride and
// its words at packed + y * nwords (the [M][nwords] stack a vote reads), so M
// workers take one launch.  (A grid of a few blocks per CU looping over the bytes,
// four per thread per round, was slower at 2^28 elements: 3.98 against 4.71 TB/s.)
template <typename T>
__global__ __launch_bounds__(256) void k_sign_pack(const T* __restrict__ u, int64_t u_stride, int64_t numel,
                                                   uint32_t* __restrict__ packed, int vec_ok) {
  const int lane = threadIdx.x & 63;
  const int64_t nwords = (numel + 31) >> 5;
  u += static_cast<int64_t>(blockIdx.y) * u_stride;
  packed += static_cast<int64_t>(blockIdx.y) * nwords;
  uint32_t bytes[PACK_UNITS];
#pragma unroll
  for (int s = 0; s < PACK_UNITS; ++s) {
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * PACK_UNITS + s) * 256 + threadIdx.x;
    bytes[s] = sign_byte(u, t * 8, numel, vec_ok);
  }
#pragma unroll
  for (int s = 0; s < PACK_UNITS; ++s) {
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * PACK_UNITS + s) * 256 + threadIdx.x;
    uint32_t w = bytes[s] << (8 * (lane & 3));
    w |= __shfl_xor(w, 1, 64);
    w |= __shfl_xor(w, 2, 64);
    if ((lane & 3) == 0 && (t >> 2) < nwords) packed[t >> 2] = w;
  }
}

__device__ inline uint32_t lane_word(uint32_t v, int) { return v; }
__device__ inline uint32_t lane_word(const u32x4_t& v, int q) { return v[q]; }

// Vote of one group of W (1 or 4) consecutive words: a bit-sliced counter of LV bit
// planes (2^LV > M) adds the M workers' words (all 32 bit positions of every word at
// once), and a bit-sliced compare gives count >= ceil(M/2), which is
// 2*count - M >= 0 (ties -> +1).  Loads are issued 8 workers at a time ahead of the
// additions.  V is uint32_t or a 4-vector of them.
template <typename V, int LV>
__device__ inline V vote_group(const V* __restrict__ src, int64_t stride, int M, V (&cnt)[LV]) {
#pragma unroll
  for (int l = 0; l < LV; ++l) cnt[l] = V{} ^ V{};
  auto add = [&](V carry) {
#pragma unroll
    for (int l = 0; l < LV; ++l) {
      const V c = cnt[l];
      cnt[l] = c ^ carry;
      carry = c & carry;
    }
  };
  int k = 0;
  for (; k + 8 <= M; k += 8) {
    V x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = src[static_cast<int64_t>(k + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) add(x[u]);
  }
  for (; k < M; ++k) add(src[static_cast<int64_t>(k) * stride]);
  // count >= T with T = ceil(M/2) <=> carry out of count + (2^LV - T)
  const uint32_t addend = (1u << LV) - static_cast<uint32_t>((M + 1) >> 1);
  V carry = V{} ^ V{};
#pragma unroll
  for (int l = 0; l < LV; ++l) {
    const V kbits = V{} ^ V{} ^ (((addend >> l) & 1u) ? 0xFFFFFFFFu : 0u);
    carry = (cnt[l] & kbits) | ((cnt[l] ^ kbits) & carry);
  }
  return carry;
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

// One thread per 4 packed words (16-byte loads) when the buffers allow it, else one
// per word.  Pad bits of the last word are cleared.  LV bit planes count up to
// 2^LV - 1 workers; SUMS also writes the int8 sums.
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
    // nwords % 4 == 0: every thread below nwords / 4 owns four whole words
    const int64_t w0 = t * 4;
    if (w0 >= nwords) return;
    u32x4_t cnt[LV];
    const u32x4_t v = vote_group<u32x4_t, LV>(reinterpret_cast<const u32x4_t*>(packed + w0), nwords / 4, M, cnt);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      finish(w0 + q, v[q]);
      if (SUMS) {
        const int64_t tail = numel - (w0 + q) * 32;
        vote_sums<u32x4_t, LV>(cnt, q, M, tail < 32 ? static_cast<int>(tail) : 32, out_sum + (w0 + q) * 32);
      }
    }
  } else {
    if (t >= nwords) return;
    uint32_t cnt[LV];
    finish(t, vote_group<uint32_t, LV>(packed + t, nwords, M, cnt));
    if (SUMS) {
      const int64_t tail = numel - t * 32;
      vote_sums<uint32_t, LV>(cnt, 0, M, tail < 32 ? static_cast<int>(tail) : 32, out_sum + t * 32);
    }
  }
}

// The inverse of the packing, for the local polar step on the voted signs: element
// i <- +1 where bit i is set, else -1.  One thread per 8 elements (one byte).
template <typename T>
__global__ __launch_bounds__(256) void k_sign_unpack(const uint32_t* __restrict__ packed, int64_t numel,
                                                     T* __restrict__ out, int vec_ok) {
  uint32_t words[UNPACK_UNITS];
#pragma unroll
  for (int s = 0; s < UNPACK_UNITS; ++s) {
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * UNPACK_UNITS + s) * 256 + threadIdx.x;
    words[s] = t * 8 < numel ? packed[t >> 2] : 0u;
  }
#pragma unroll
  for (int s = 0; s < UNPACK_UNITS; ++s) {
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * UNPACK_UNITS + s) * 256 + threadIdx.x;
    const int64_t e0 = t * 8;
    if (e0 >= numel) continue;
    const uint32_t byte = (words[s] >> (8 * (t & 3))) & 0xFFu;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ((byte >> k) & 1u) ? 1.f : -1.f;
    if (vec_ok && e0 + 8 <= numel) {
      if (sizeof(T) == 4) {
        f32x4_t* p = reinterpret_cast<f32x4_t*>(out + e0);
        p[0] = f32x4_t{v[0], v[1], v[2], v[3]};
        p[1] = f32x4_t{v[4], v[5], v[6], v[7]};
      } else {
        bf16x8_t x;
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = static_cast<bf16_t>(v[k]);
        *reinterpret_cast<bf16x8_t*>(out + e0) = x;
      }
    } else {
      for (int k = 0; k < 8 && e0 + k < numel; ++k) out[e0 + k] = from_f32<T>(v[k]);
    }
  }
}

// Sign-Muon parameter update W <- W - lr * S with S = +1 where bit i is set, else
// -1: the difference is formed in fp32 and stored in W's dtype.  One thread per 8
// elements of each unit.
template <typename T>
__global__ __launch_bounds__(256) void k_sign_apply(const uint32_t* __restrict__ packed, int64_t numel,
                                                    T* __restrict__ w, float lr, int vec_ok) {
  typedef typename std::conditional<sizeof(T) == 4, f32x4_t, bf16x8_t>::type v_t;   // 16 bytes
  constexpr int NV = sizeof(T) == 4 ? 2 : 1;                                        // per 8 elements
  uint32_t words[SAPPLY_UNITS];
  v_t x[SAPPLY_UNITS][NV];
#pragma unroll
  for (int s = 0; s < SAPPLY_UNITS; ++s) {
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * SAPPLY_UNITS + s) * 256 + threadIdx.x;
    const int64_t e0 = t * 8;
    words[s] = e0 < numel ? packed[t >> 2] : 0u;
    if (vec_ok && e0 + 8 <= numel) {
#pragma unroll
      for (int h = 0; h < NV; ++h) x[s][h] = reinterpret_cast<const v_t*>(w + e0)[h];
    }
  }
#pragma unroll
  for (int s = 0; s < SAPPLY_UNITS; ++s) {
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * SAPPLY_UNITS + s) * 256 + threadIdx.x;
    const int64_t e0 = t * 8;
    if (e0 >= numel) continue;
    const uint32_t byte = (words[s] >> (8 * (t & 3))) & 0xFFu;
    if (vec_ok && e0 + 8 <= numel) {
#pragma unroll
      for (int h = 0; h < NV; ++h) {
        v_t y = x[s][h];
        constexpr int PER = 8 / NV;
#pragma unroll
        for (int k = 0; k < PER; ++k)
          y[k] = from_f32<T>(to_f32(y[k]) - (((byte >> (h * PER + k)) & 1u) ? lr : -lr));
        reinterpret_cast<v_t*>(w + e0)[h] = y;
      }
    } else {
      for (int k = 0; k < 8 && e0 + k < numel; ++k)
        w[e0 + k] = from_f32<T>(to_f32(w[e0 + k]) - (((byte >> k) & 1u) ? lr : -lr));
    }
  }
}

}  // namespace mo
