// Shared device types and the per-matrix descriptor of one batched call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

namespace mo {

// Work decomposition of each batched launch kind.  Every kernel finds its matrix
// by a binary search of `begin[kind]` over the descriptor table.
enum Kind {
  KIND_SYRK = 0,   // upper-triangle 256x256 tiles of A = X X^T
  KIND_POLY = 1,   // upper-triangle 256x256 tiles of B = bA + cA^2
  KIND_APPLY = 2,  // 256x256 tiles of X <- aX + BX
  KIND_PREP = 3,   // 64x64 tiles of the padded oriented X0 (and X0^T)
  KIND_CHUNK = 4,  // 4096-element chunks of the caller's matrix (momentum, norm)
  KIND_SMALL_UPPER = 5,   // upper-triangle 32x32 blocks of A or B (calls on the small path)
  KIND_SMALL_RECT = 6,    // 32x32 blocks of X (small path)
  NKIND = 7
};

constexpr int GEMM_TILE = 256;   // workspace dims are padded to multiples of this
constexpr int PREP_TILE = 64;
constexpr int CHUNK = 4096;      // elements per momentum / sum-of-squares block
// Workspace operands (X, A, B) are k-blocked: a buffer of R rows and K columns (K,
// the reduction index of the GEMM that reads it) is stored as K / kb blocks of R
// rows x KB_BYTES, one after another.  Element (r, k) then sits at byte
//   (k / kb) * pitch + r * KB_BYTES + (k % kb) * es,   kb = KB_BYTES / es elements,
// pitch = R * KB_BYTES.  The k-slab of 256 rows that one GEMM step consumes is one
// contiguous 32 KiB run instead of 256 row pieces spread over megabytes: 2-3% less
// GEMM time than row-major operands with a padded pitch.  (64-byte blocks, which
// leave room for a four-slab LDS ring of whole lines, measured no faster.)
constexpr int KB_BYTES = 128;

// Byte offset of element (r, k) of a k-blocked buffer whose k-blocks are `pitch`
// bytes apart.  Workspace buffers stay below 2 GiB, so 32 bits hold every offset.
template <typename T>
__host__ __device__ inline uint32_t kb_off(uint32_t r, uint32_t k, uint32_t pitch) {
  constexpr uint32_t kb = KB_BYTES / sizeof(T);
  return (k / kb) * pitch + r * KB_BYTES + (k % kb) * static_cast<uint32_t>(sizeof(T));
}

struct MatDesc {
  // caller buffers
  const void* grad;   // gradient (momentum step) or input x (orthogonalise only)
  float* mom;         // fp32 momentum, null for orthogonalise only
  void* out;          // U in the caller's orientation
  int64_t rows, cols, numel;
  // oriented problem: X is m x n with m = min(rows, cols), n = max(rows, cols)
  int32_t m, n, mp, np;   // mp, np: m and n rounded up to GEMM_TILE
  uint32_t pX, pM;        // k-block pitch (bytes) of X and of A, B (mp rows each)
  int32_t transposed;     // 1 if rows > cols (X = M^T)
  int32_t vec_ok;         // 1 if grad/mom/out allow 16-byte vector access
  // workspace buffers, compute dtype, k-blocked (see kb_off), zero outside the m x n
  // corner: the first pass writes all of X; the products write their padding as
  // exact zeros, on the 256-tile path up to mp / np and on the small path up to the
  // next multiple of 32, which is as far as that path reads
  void* X[2];             // mp x np (k = column), ping-pong: iteration t reads X[t % 2]
                          // (SYRK's operands, APPLY's second operand) and APPLY writes
                          // X[(t + 1) % 2]
  void* A;                // mp x mp, symmetric
  void* B;                // mp x mp, symmetric
  int64_t begin[NKIND];   // first work item of this matrix per launch kind
  int64_t items[NKIND];   // work items of this matrix per launch kind
  int32_t scale_slot;     // index into the per-matrix scale array
  int32_t pad_[3];
};

// Global-address-space view of a device pointer.  Accesses through it compile to
// global_* instructions, which count only against vmcnt; through a generic pointer
// the compiler emits flat_* instructions, which count against lgkmcnt as well, so
// the next wait for an LDS read would also wait for every one of them to finish.
template <typename T> using gptr = __attribute__((address_space(1))) T*;
template <typename T> __device__ inline gptr<T> global(T* p) { return (gptr<T>)p; }

__device__ inline int find_desc(const MatDesc* __restrict__ d, int count, int kind, int64_t item) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (d[mid].begin[kind] <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline float bf16_to_f32(bf16_t v) { return static_cast<float>(v); }

template <typename T> __device__ inline T from_f32(float v);
template <> __device__ inline float from_f32<float>(float v) { return v; }
template <> __device__ inline bf16_t from_f32<bf16_t>(float v) { return static_cast<bf16_t>(v); }

template <typename T> __device__ inline float to_f32(T v) { return static_cast<float>(v); }

}  // namespace mo
