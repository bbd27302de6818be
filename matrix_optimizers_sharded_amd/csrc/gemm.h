// The three Newton-Schulz products as one MFMA GEMM core with three epilogues.
//
// Every product is C[i][j] = sum_k P[i][k] * Q(k, j), P read along k-contiguous rows:
//   SYRK   A  = X X^T         P = Q = X (rows of X, k over n), Q(k, j) = X[j][k];
//                             upper tiles only, each off-diagonal tile also
//                             stored mirrored
//   POLY   B' = aI + bA + c A A   P = Q = A (A symmetric, so A A = A A^T); upper
//                             tiles, mirrored; b*A in the epilogue reads the same
//                             rounded A, and a is added on the diagonal (rows < m)
//   APPLY  X' = B' X = aX + (bA + cA^2) X   P = B', Q(k, j) = X[k][j]: X itself,
//                             whose slab (rows k, the tile's columns j) gfx950's
//                             transposing LDS reads turn into k-contiguous MFMA
//                             operands; the epilogue only stores X' into the other
//                             ping-pong buffer, or the final U to the caller.
// Folding a into B' removes every epilogue read from the largest product; it
// rounds a + B_ii to the compute dtype once instead of rounding B_ii.
// All workspace dims are multiples of 256, zero-padded, so the main loop needs no
// bounds checks; only the final write to the caller's buffer is clipped.
//
// Tiling (gfx950, wave64): 256x256 block tile; NWAVES = 8 waves in a 2 x 4 grid,
// each owning a 128 x 64 sub-tile = 4 x 2 MFMA 32x32 blocks (128 fp32 accumulators
// per lane), two waves per SIMD: with bf16 operands one of them issues the slab
// loads for both while the other keeps the SIMD's matrix core busy (see the loader
// waves below).  The k-loop streams slabs of 256 rows x 128 bytes (64 bf16 or 32
// fp32 of k) of both operands, each one contiguous k-block of the workspace layout,
// straight from HBM/L2 into LDS with 16-byte buffer loads that write LDS directly
// (no register staging), through a 2-stage ring: the loads of slab t+2 are issued
// early in slab t+1 and land while it is multiplied.  LDS rows are 128 bytes with
// the 16-byte chunk index XOR-swizzled by (r ^ r>>1) & 7, so the fragment reads of
// 8 or 16 consecutive rows hit distinct banks.
#pragma once

#include <type_traits>

#include "common.h"

namespace mo {

// GM_APPLY_FINAL writes U to the caller's buffer; GM_APPLY_WEIGHT instead updates the
// caller's weight in place, W <- W - lr * U, with lr passed as `ca`.
enum GemmMode { GM_SYRK = 0, GM_POLY = 1, GM_APPLY = 2, GM_APPLY_FINAL = 3, GM_APPLY_WEIGHT = 4 };

constexpr int GT = GEMM_TILE;          // 256

// k-slab geometry: each operand row of a slab is ROW_BYTES, one k-block of the
// workspace layout (128: 64 bf16 / 32 fp32 of k), and NSTAGE = 2 slabs are in flight
// in an LDS ring (2 x 64 KiB, with the 32 KiB epilogue staging the whole 160 KiB),
// so the loads of slab t+1 overlap the MFMAs of slab t.  (A four-stage ring of
// 64-byte slabs, three slabs of load cover instead of one, with this kernel: 8%
// slower at the 7B-class owner set, SYRK 15%; 3-4% faster at the 1B- and
// 125M-class sets, APPLY 9% there.)
// The epilogue's stores into the workspace are non-temporal: they are read again
// only by the next launch, so they need not displace the operand panels that the
// other blocks of an XCD are sharing in L2.  Measured: -0.5% time for the staged
// whole-line transposed copies, a further -1.1% for the row-major results.
template <typename V>
__device__ inline void store_ws(gptr<V> p, const V& v) {
  __builtin_nontemporal_store(v, p);
}
constexpr int ROW_BYTES = KB_BYTES;
constexpr int CHUNKS = ROW_BYTES / 16;                 // 16-byte chunks per row
constexpr int KSTEPS = CHUNKS / 2;                     // k16 MFMA steps per slab
constexpr int NSTAGE = 2;
constexpr int OPERAND_BYTES = GT * ROW_BYTES;
constexpr int STAGE_BYTES = 2 * OPERAND_BYTES;         // P and Q
constexpr int GEMM_LDS_BYTES = NSTAGE * STAGE_BYTES;
// 8 waves, two per SIMD.  APPLY's transposed slab layout needs a multiple of the 8
// row groups of a bf16 k-block (a 4-wave grid of 128 x 128 sub-tiles measured 2.7%
// slower before that layout existed).
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int WAVES_N = NWAVES / 2;                    // wave grid: 2 x WAVES_N
constexpr int WAVE_N = GT / WAVES_N;                   // columns per wave: 64
constexpr int NB = WAVE_N / 32;                        // 32-column MFMA blocks per wave
constexpr int ROWS_PER_INST = 1024 / ROW_BYTES;        // rows one 1 KiB wave load fills
constexpr int INST_PER_OPERAND = OPERAND_BYTES / 1024 / NWAVES;  // per wave, per slab
constexpr int INST_PER_SLAB = 2 * INST_PER_OPERAND;
static_assert(GEMM_LDS_BYTES + NWAVES * 4096 <= 160 * 1024, "LDS ring and staging exceed 160 KiB");
// the shortest K is 256: a tile has at least 512 / ROW_BYTES slabs (bf16), and the
// ring, which starts the next tile's loads during this tile's last NSTAGE slabs,
// needs at least NSTAGE of them
static_assert(512 / ROW_BYTES >= NSTAGE, "ring too deep for K = 256");
static_assert(INST_PER_SLAB * 3 < 64, "vmcnt is a 6-bit field");

// raw-buffer resource word 3 for gfx9-family: 32-bit data format, no swizzle
constexpr int RSRC_FLAGS = 0x00020000;

// 16-byte chunk swizzle inside a row, chosen so that the fragment reads of 8
// consecutive rows (32 banks x 4 B) and of 16 consecutive rows (64 banks) fall in
// distinct banks.
__device__ inline int swz(int r) { return (r ^ (r >> 1)) & 7; }

// Swizzle of the [k][n] slabs of APPLY's second operand (rows k of 128 bytes of n):
// a transposing read by 32 lanes covers 64 bytes of each of 4 consecutive rows, and
// rows k and k + 2 share banks unless their halves are swapped.
__device__ inline int swz_tr(int k) { return ((k >> 1) & 1) << 2; }

// Transposing LDS read of gfx950 (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives in slot e the 16-bit element at (the address that lane
// 4e + i/4 supplied) + (i % 4) elements.  So if lane 16g + 4e + q points at row
// r0 + e, columns c0 + 4q .. c0 + 4q + 3 of a row-major 16-bit tile, lane 16g + i
// receives rows r0 .. r0 + 3 of column c0 + i.
__device__ inline bf16x4_t lds_read_tr16(const unsigned char* p) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)(p));
  return __builtin_bit_cast(bf16x4_t, v);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource (gfx9 layout): 48-bit base, stride 0, size in bytes, flags.
__device__ inline i32x4_t buffer_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4_t r;
  r[0] = static_cast<int>(static_cast<uint32_t>(a));
  r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r[2] = static_cast<int>(bytes);
  r[3] = RSRC_FLAGS;
  return r;
}

// Four 16-byte-per-lane loads from one buffer straight into LDS: load q writes
// lds[q] + 16 * lane from byte voff[q] + soff of the buffer.  Written as inline asm
// so that the compiler's wait-count pass does not track them: that pass cannot tell
// which ring stage they write and would otherwise wait for them before every LDS
// read.  The ring's own explicit waits cover these loads.  M0 (the LDS base of a
// load) is saved and restored, so the compiler's view of it stays valid; every
// operand is made uniform first so that it is an SGPR.
__device__ inline void load_lds16x4(i32x4_t rsrc, const uint32_t (&lds)[4], const uint32_t (&voff)[4],
                                    uint32_t soff) {
  i32x4_t r;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = __builtin_amdgcn_readfirstlane(rsrc[c]);
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds[0]), l1 = __builtin_amdgcn_readfirstlane(lds[1]);
  const uint32_t l2 = __builtin_amdgcn_readfirstlane(lds[2]), l3 = __builtin_amdgcn_readfirstlane(lds[3]);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %5, %9, %10 offen lds\n\t"
      "s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %6, %9, %10 offen lds\n\t"
      "s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %7, %9, %10 offen lds\n\t"
      "s_mov_b32 m0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %8, %9, %10 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(l0), "s"(l1), "s"(l2), "s"(l3), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(r),
        "s"(so)
      : "memory");
}
__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

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
constexpr int BAND = 4;

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
// XCD x receives runs of G = 32 consecutive work items (chunks dealt round-robin
// over the XCDs): the blocks one XCD runs at a time are neighbours in the work
// list and share operand panels in that XCD's L2, while all XCDs still progress
// through the list together (equal load).
__device__ inline int64_t xcd_remap(int64_t b, int64_t total) {
  constexpr int64_t G = 32;
  const int64_t full = total / (8 * G) * (8 * G);   // blocks in complete rounds
  if (b >= full) return b;                          // ragged tail: identity
  const int64_t x = b % 8, k = b / 8;               // k-th block of XCD x
  return (k / G) * (8 * G) + x * G + (k % G);
}

// element at a byte offset from a global base pointer
template <typename V, typename T>
__device__ inline gptr<V> at(gptr<T> base, uint32_t byte_off) {
  typedef __attribute__((address_space(1))) unsigned char* bytes_t;
  return (gptr<V>)((bytes_t)base + byte_off);
}

template <typename T> struct Vec4;
template <> struct Vec4<bf16_t> { typedef bf16x4_t type; };
template <> struct Vec4<float> { typedef f32x4_t type; };

template <typename T>
__device__ inline void store4(gptr<T> p, float v0, float v1, float v2, float v3) {
  typedef typename Vec4<T>::type v4_t;
  const v4_t v = {from_f32<T>(v0), from_f32<T>(v1), from_f32<T>(v2), from_f32<T>(v3)};
  *reinterpret_cast<gptr<v4_t>>(p) = v;
}

// Stores rows ib..ib+3 of column j (v[0..3], this lane's share of an MFMA result
// block) into a k-blocked buffer as 2-column pieces instead of single elements:
// lanes l and l ^ 1 hold columns j and j ^ 1 of the same rows, so one lane-pair
// exchange (DPP quad permutation 1,0,3,2) gives the even lane rows ib, ib+1 of
// columns j, j+1 and the odd lane rows ib+2, ib+3 of columns j-1, j.  Half as many
// store instructions, each still covering 64 contiguous bytes per row.  Used for
// POLY's off-diagonal tiles: -2.5% POLY time; the same stores made APPLY 1% slower
// and left SYRK unchanged (A/B on one box, three rounds each).
__device__ inline uint32_t dpp_swap_pair(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0xB1, 0xF, 0xF, false));
}
template <typename T>
__device__ inline void store_pairs(gptr<T> C, uint32_t pitch, int lane, int ib, int j, const float (&v)[4]) {
  const bool odd = lane & 1;
  const int row = odd ? ib + 2 : ib, col = odd ? j - 1 : j;
  const uint32_t o = kb_off<T>(row, col, pitch);
  if constexpr (sizeof(T) == 2) {
    auto bits = [](float f) { return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<bf16_t>(f))); };
    const uint32_t p01 = bits(v[0]) | (bits(v[1]) << 16), p23 = bits(v[2]) | (bits(v[3]) << 16);
    const uint32_t r = dpp_swap_pair(odd ? p01 : p23);   // the partner's rows this lane stores
    const uint32_t own = odd ? p23 : p01;
    uint32_t w0, w1;
    if (!odd) {
      w0 = (own & 0xffffu) | (r << 16);
      w1 = (own >> 16) | (r & 0xffff0000u);
    } else {
      w0 = (r & 0xffffu) | (own << 16);
      w1 = (r >> 16) | (own & 0xffff0000u);
    }
    store_ws(at<uint32_t>(C, o), w0);
    store_ws(at<uint32_t>(C, o + ROW_BYTES), w1);
  } else {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    const float s0 = odd ? v[0] : v[2], s1 = odd ? v[1] : v[3];
    const float r0 = __builtin_bit_cast(float, dpp_swap_pair(__builtin_bit_cast(uint32_t, s0)));
    const float r1 = __builtin_bit_cast(float, dpp_swap_pair(__builtin_bit_cast(uint32_t, s1)));
    const f2_t w0 = odd ? f2_t{r0, v[2]} : f2_t{v[0], r0};
    const f2_t w1 = odd ? f2_t{r1, v[3]} : f2_t{v[1], r1};
    store_ws(at<f2_t>(C, o), w0);
    store_ws(at<f2_t>(C, o + ROW_BYTES), w1);
  }
}

// Wave placement and diagonal tiles.  A wave owns the 128 x WAVE_N sub-tile at block
// row wrow (of 2) and block column wcol (of WAVES_N), 4 x NB MFMA blocks of 32x32.
// SYRK and POLY store only the upper triangle of A and B', so on a diagonal tile
// (ti == tj) the MFMA block (a, b) of a wave is needed only when it reaches the
// diagonal, a - b <= D with D = NB * wcol - 4 * wrow (in 32-row blocks); the rest of
// the tile is skipped.  Waves w and w + 4 share a SIMD, so SYRK and POLY place the
// first row's waves at block columns 2, 3, 1, 0: on a diagonal tile the two waves of
// each SIMD then hold 8 + 0, 8 + 0, 7 + 3 and 3 + 7 of the 36 blocks on or above the
// diagonal, and the tile takes 10 block-times instead of 16.  (In the natural order
// the SIMDs would hold 3, 7, 11 and 15 blocks: almost no saving.)  Both operands
// are still loaded: loading only P for a diagonal tile, whose second operand is
// the same rows, measured 6% slower for SYRK at the 7B-class set.
constexpr int sym_col(int w) { return w < 4 ? (w == 0 ? 2 : w == 1 ? 3 : w == 2 ? 1 : 0) : w - 4; }
constexpr int wave_d(int w) { return NB * sym_col(w) - 4 * (w / WAVES_N); }
// the k-loop is instantiated for D = 3 (every block), 2, 0 and -NB (no block)
constexpr int d_class(int d) { return d >= 3 ? 3 : d == 2 ? 2 : d == 0 ? 0 : d <= -NB ? -NB : 99; }
static_assert(NWAVES == 8 && WAVES_N == 4 && NB == 2, "diagonal-tile placement assumes a 2 x 4 grid of 4 x 2 blocks");
static_assert(d_class(wave_d(0)) != 99 && d_class(wave_d(1)) != 99 && d_class(wave_d(2)) != 99 &&
                  d_class(wave_d(3)) != 99 && d_class(wave_d(4)) != 99 && d_class(wave_d(5)) != 99 &&
                  d_class(wave_d(6)) != 99 && d_class(wave_d(7)) != 99,
              "every wave's diagonal class has a k-loop instantiation");
// blocks, first-operand fragments (a < A) and second-operand fragments (b >= B0) of a
// wave with diagonal class D
constexpr int n_active(int d) {
  int n = 0;
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < NB; ++b) n += (a - b <= d) ? 1 : 0;
  return n;
}
constexpr int a_needed(int d) { return d + NB < 0 ? 0 : (d + NB > 4 ? 4 : d + NB); }
constexpr int b_first(int d) { return d >= 0 ? 0 : (-d > NB ? NB : -d); }
template <int V> using IC = std::integral_constant<int, V>;

// One tile's operand stream: buffer resources over P and Q and this lane's byte
// offsets of its first rows, plus where the tile sits.
struct TileRef {
  int di, ti, tj, nk;   // descriptor index, tile row and column, k slabs
  int diag;             // SYRK/POLY diagonal tile: only blocks on or above the diagonal are computed
  i32x4_t rP, rQ;
  uint32_t vP0, vQ0;    // this lane's byte offsets of its first load of slab 0 of P and Q
  uint32_t kP, kQ;      // byte step from one slab to the next, in P and in Q
  uint32_t qQ;          // byte step from one of a wave's Q loads to the next
};

// Persistent kernel: the grid holds at most one block per CU, and block b walks the
// work items b, b + G, b + 2G, ... of the remapped order (G = gridDim.x, a multiple
// of 8 whenever a block gets more than one item, so a block keeps to its XCD's share
// of that order).  The operand ring runs across tile boundaries: the last NSTAGE
// slabs of a tile start the loads of the next tile's first slabs, so those land while
// this tile finishes and writes its epilogue, and no tile pays a cold start.  (A
// shared work queue fed by an atomic counter measured about 1% slower.)
// SMALLK (bf16 operands only) is chosen by the host for SYRK / POLY launches whose
// matrices all have m <= 1024: at most 4 x 4 tiles per matrix, two fifths or more of
// the upper ones diagonal, and POLY tiles of at most 16 k-slabs.  A diagonal tile,
// whose two operands are the same row panel, loads that panel once and reads both
// operands' fragments from it.  That was measured slower at the 1B- and 7B-class
// sets (m = 2048 and 4096), which keep the plain kernel.
constexpr int SMALLK_MAX_M = 1024;
template <typename T, int MODE, typename TO, bool SMALLK = false>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(NWAVES / 4, NWAVES / 4)))
void k_ns_gemm(const MatDesc* __restrict__ descs, int count, int64_t total, int parity, float ca, float cb,
               float cc, const float* __restrict__ first) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[GEMM_LDS_BYTES];
  // per-wave 4 KiB epilogue staging slabs
  __shared__ __attribute__((aligned(16))) unsigned char staging[NWAVES * 4096];
  constexpr int kind = (MODE == GM_SYRK) ? KIND_SYRK : (MODE == GM_POLY) ? KIND_POLY : KIND_APPLY;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  constexpr bool SYM = MODE == GM_SYRK || MODE == GM_POLY;
  const int wcol = SYM ? sym_col(wave) : wave % WAVES_N;
  const int wm = (wave / WAVES_N) * 128, wn = wcol * WAVE_N;
  const int wdc = d_class(wave_d(wave));   // this wave's diagonal class

  // Direct-to-LDS loads: wave w, instruction q fills ROWS_PER_INST rows starting at
  // ROWS_PER_INST*(NWAVES*q+w) of an operand slab, 1 KiB contiguous in LDS (lane l ->
  // row + l/CHUNKS, physical chunk l%CHUNKS); the lane fetches the logical chunk
  // that the swizzle stores there.  Rows advance by ROWS_PER_INST * NWAVES between a
  // wave's instructions, a multiple of 16, which leaves the swizzle unchanged: one
  // base offset per operand plus a uniform stride per instruction.
  const int row0 = ROWS_PER_INST * wave + lane / CHUNKS;
  const uint32_t lane_chunk = ((lane % CHUNKS) ^ swz(row0)) << 4;
  // rows advance by ROWS_PER_INST * NWAVES from one of a wave's loads to the next
  constexpr uint32_t VSTEP = ROWS_PER_INST * NWAVES * ROW_BYTES;

  // APPLY's second operand is X itself: X'[i][j] = sum_k B'[i][k] X[k][j].  Its slab
  // is rows k of the slab's k range and the tile's 256 columns j, which in X's
  // k-blocked layout are JB = 256 / KB k-blocks, each holding the KR = KB rows as one
  // contiguous run of KR x 128 bytes.  LDS keeps them as [JB][KR][128 bytes] (16-byte
  // chunks swizzled by swz_tr(k)), and the MFMA's second operand, 8 consecutive k of
  // one column per lane, comes out of transposing reads.  Wave w's load q covers 8
  // rows of k-block (NWAVES q + w) / RG, from row ((NWAVES q + w) % RG) * 8.
  constexpr bool QT = MODE == GM_APPLY || MODE == GM_APPLY_FINAL || MODE == GM_APPLY_WEIGHT;
  constexpr bool EARLY_P = MODE == GM_POLY;   // POLY: P loads before the last step's MFMAs
  static_assert(!SMALLK || sizeof(T) == 2, "the SMALLK kernel is for bf16 operands");
  constexpr bool ONE_PANEL = SMALLK && SYM;    // diagonal tiles load P only
  constexpr int KB = ROW_BYTES / static_cast<int>(sizeof(T));   // elements per k-block
  constexpr int KR = KB;                                         // k rows per slab
  constexpr int JB = GT / KB;                                    // k-blocks per tile width
  constexpr int RG = KR / 8;                                     // 8-row groups per k-block
  static_assert(ROW_BYTES == 128 && NWAVES % RG == 0,
                "transposed slab layout: 128-byte k-blocks, waves a multiple of the row groups");
  const int qrow = (wave % RG) * 8 + lane / 8;   // k row of this lane's loads within the slab
  const uint32_t qlane = static_cast<uint32_t>(qrow) * ROW_BYTES + (((lane % 8) ^ swz_tr(qrow)) << 4);

  auto setup = [&](int64_t v, TileRef& t) {
    const int64_t item = xcd_remap(v, total);
    const int di = __builtin_amdgcn_readfirstlane(find_desc(descs, count, kind, item));
    const MatDesc* d = descs + di;
    const int64_t local = item - d->begin[kind];
    const T* P;
    const T* Q;
    uint32_t kP, kQ;   // k-block pitches
    int K;
    if (MODE == GM_SYRK) {
      upper_tile(local, d->mp / GT, t.ti, t.tj);
      P = Q = static_cast<const T*>(d->X[parity]);
      kP = kQ = d->pX;
      K = d->np;
    } else if (MODE == GM_POLY) {
      upper_tile(local, d->mp / GT, t.ti, t.tj);
      P = Q = static_cast<const T*>(d->A);
      kP = kQ = d->pM;
      K = d->mp;
    } else {
      rect_tile(local, d->mp / GT, d->np / GT, t.ti, t.tj);
      P = static_cast<const T*>(d->B);
      Q = static_cast<const T*>(d->X[parity]);
      kP = d->pM;
      kQ = d->pX;
      K = d->mp;
    }
    t.di = di;
    t.diag = SYM && t.ti == t.tj;
    t.nk = K / KB;   // >= 512 / ROW_BYTES >= NSTAGE: K >= 256
    t.rP = buffer_rsrc(P, t.nk * kP);
    t.vP0 = static_cast<uint32_t>(t.ti * GT + row0) * ROW_BYTES + lane_chunk;
    t.kP = kP;
    if (QT) {
      // the tile's columns j are the JB k-blocks tj * JB .. of X; the slab's k range
      // is rows kt * KR .. of each
      t.rQ = buffer_rsrc(Q, static_cast<uint32_t>(d->np / KB) * kQ);
      t.vQ0 = static_cast<uint32_t>(t.tj * JB + wave / RG) * kQ + qlane;
      t.kQ = KR * ROW_BYTES;
      t.qQ = (NWAVES / RG) * kQ;
    } else {
      t.rQ = buffer_rsrc(Q, t.nk * kQ);
      t.vQ0 = static_cast<uint32_t>(t.tj * GT + row0) * ROW_BYTES + lane_chunk;
      t.kQ = kQ;
      t.qQ = VSTEP;
    }
  };
  static_assert(INST_PER_OPERAND % 4 == 0, "loads per operand per wave: a multiple of 4");
  // Loader waves.  With bf16 operands only the first LOADERS waves (one per SIMD for
  // 4) issue the slab loads, each also issuing those of waves w + LOADERS,
  // w + 2 LOADERS, ...: the slab's rows of wave w + i LOADERS are 8 i LOADERS rows
  // further, i LOADERS KiB on in the operand and in LDS, and a multiple of 16 rows
  // leaves both swizzles unchanged.  The other wave on each SIMD then never stalls
  // at load issue, and keeps the SIMD's matrix core busy while its partner waits on
  // a full texture-address FIFO.  Measured at the 7B-class set: 4 loaders -4% per
  // step against 8 (APPLY -5.5%, SYRK -3%, POLY unchanged).  fp32 operands keep all
  // 8 waves loading (their APPLY slab maps wave w + 4 to another k-block).
  constexpr int LOADERS = sizeof(T) == 2 ? 4 : NWAVES;
  static_assert(NWAVES % LOADERS == 0 && (LOADERS == NWAVES || sizeof(T) == 2), "loader waves");
  // this wave's loads of k-block kt of one operand (h = 0: P, h = 1: Q) into a stage
  auto issue_op = [&](const TileRef& t, int kt, int stage, int h) {
    if (wave >= LOADERS) return;
#pragma unroll
    for (int vw = 0; vw < NWAVES / LOADERS; ++vw) {
      const uint32_t shift = vw * LOADERS * 1024;   // bytes, in the operand and in LDS
      const uint32_t base = lds_addr(smem) + stage * STAGE_BYTES + wave * 1024 + (h ? OPERAND_BYTES : 0) + shift;
#pragma unroll
      for (int q0 = 0; q0 < INST_PER_OPERAND; q0 += 4) {
        uint32_t l[4], vo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          l[q] = base + (q0 + q) * NWAVES * 1024;
          vo[q] = (h ? t.vQ0 + (q0 + q) * t.qQ : t.vP0 + (q0 + q) * VSTEP) + shift;
        }
        load_lds16x4(h ? t.rQ : t.rP, l, vo, kt * (h ? t.kQ : t.kP));
      }
    }
  };
  auto issue = [&](const TileRef& t, int kt, int stage) {
    issue_op(t, kt, stage, 0);
    if (!(ONE_PANEL && t.diag)) issue_op(t, kt, stage, 1);
  };
  // where the second operand sits in a stage: P's own half for a diagonal tile
  // that loads one panel
  auto q_off = [&](const TileRef& t) {
    return (ONE_PANEL && t.diag) ? 0u : static_cast<uint32_t>(OPERAND_BYTES);
  };

  f32x16_t acc[4][NB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  };

  // fragment read offsets (row part), per sub-block
  int rowA[4], rowB[NB];
#pragma unroll
  for (int a = 0; a < 4; ++a) rowA[a] = wm + a * 32 + l32;
#pragma unroll
  for (int b = 0; b < NB; ++b) rowB[b] = wn + b * 32 + l32;

  typedef typename Mfma<T>::frag frag_t;
  // Pipeline per slab kt (stage kt % NSTAGE), fragments double-buffered over the
  // k16 steps: steps 0..KSTEPS-2 read the next step's fragments, then run 8 MFMAs;
  // then wait until this wave's loads of slab kt+1 have landed (later slabs may stay
  // in flight) and its own LDS reads are done, one barrier (slab kt+1 is in LDS for
  // everyone, and nobody reads slab kt any more), read slab kt+1's first fragments
  // beside the last step's 8 MFMAs, and only then start the loads of slab kt+NSTAGE
  // (of this tile or the next) into slab kt's stage.  Right after the barrier all
  // eight waves would otherwise issue their 64 direct-to-LDS loads at once: the
  // texture-address command FIFO fills (rocprofv3 SQ_VMEM_TA_CMD_FIFO_FULL), waves
  // stall at issue, and their MFMAs wait behind the loads.  With the MFMAs issued
  // first the matrix cores stay busy while the loads drain.  Measured against loads
  // first, on two boxes: APPLY and SYRK -5%; POLY -1% with all loads after, -4% with
  // its P loads before and Q loads after the MFMAs (EARLY_P).
  // The waits count loads only: buffer loads complete in issue order, so "at most
  // n outstanding", with n the loads issued after slab kt+1's, means slab kt+1 is
  // in, whatever stores or atomics are also in flight.
  // Within a k16 step the next step's fragment reads are interleaved one to one
  // with this step's MFMAs (then the remaining MFMAs), so the LDS and the matrix
  // cores work side by side instead of in turns.
  // LDS reads and MFMAs per k16 step: one 16-byte read per first-operand fragment;
  // per second-operand fragment one 16-byte read, or (QT) two transposing 8-byte
  // reads for bf16 and four 4-byte reads for fp32; one MFMA per active fragment pair
  // for bf16, four for fp32.  Within a step the next step's fragment reads are
  // interleaved one to one with this step's MFMAs (then the rest), so the LDS and
  // the matrix cores work side by side instead of in turns (+1.4%, and 3% over
  // grouped reads on the final kernel).
  constexpr int READS_PER_B = QT ? (sizeof(T) == 2 ? 2 : 4) : 1;
  constexpr int MMA_PER_PAIR = sizeof(T) == 2 ? 1 : 4;
  auto interleave = [&](auto nr_tag, auto nm_tag) {
    constexpr int NR = decltype(nr_tag)::value, NM = decltype(nm_tag)::value;
    constexpr int NP = NR < NM ? NR : NM;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    }
    if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
    if constexpr (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
  };
  frag_t fa[2][4], fb[2][NB];
  // QT, bf16: lane 16g + 4e + q addresses row 8 (g / 2) + e (plus 16 per k16 step)
  // and columns 16 (g % 2) + 4q .. + 3 of a 32-column block, so that two
  // transposing reads (rows +0..3, +4..7) give it 8 consecutive k of column l % 32
  const int trow = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // the fragments of k16 step kk of the stage at sP that a wave of diagonal class D
  // uses (every fragment for D = 3)
  auto read_frags = [&](auto dtag, const unsigned char* sP, uint32_t qoff, int kk, frag_t* A, frag_t* B) {
    constexpr int D = decltype(dtag)::value;
    constexpr int NA = a_needed(D), B0 = b_first(D);
    const unsigned char* sQ = sP + (ONE_PANEL ? qoff : static_cast<uint32_t>(OPERAND_BYTES));
    const int c = 2 * kk + half;
#pragma unroll
    for (int a = 0; a < NA; ++a)
      A[a] = *reinterpret_cast<const frag_t*>(sP + rowA[a] * ROW_BYTES + ((c ^ swz(rowA[a])) << 4));
    if constexpr (!QT) {
#pragma unroll
      for (int b = B0; b < NB; ++b)
        B[b] = *reinterpret_cast<const frag_t*>(sQ + rowB[b] * ROW_BYTES + ((c ^ swz(rowB[b])) << 4));
    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int n = wn + 32 * b + tcol;                  // column j - j0 of the tile
        const int nb = (n % KB) * 2, k = 16 * kk + trow;   // byte in the k-block row; k row
        const unsigned char* q =
            sQ + (n / KB) * (KR * ROW_BYTES) + k * ROW_BYTES + ((((nb >> 4) ^ swz_tr(k)) << 4) | (nb & 15));
        const bf16x4_t lo = lds_read_tr16(q), hi = lds_read_tr16(q + 4 * ROW_BYTES);   // swz_tr(k + 4) == swz_tr(k)
        B[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    } else {
      // fp32: lane l needs rows 4c .. 4c + 3 (the k of its first-operand chunk) of
      // column l % 32, four 4-byte reads
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int n = wn + 32 * b + l32, nb = (n % KB) * 4;
        const unsigned char* col = sQ + (n / KB) * (KR * ROW_BYTES);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * c + e;
          B[b][e] = *reinterpret_cast<const float*>(col + k * ROW_BYTES + ((((nb >> 4) ^ swz_tr(k)) << 4) | (nb & 15)));
        }
      }
    }
  };
  auto mfma_step = [&](auto dtag, const frag_t* A, const frag_t* B) {
    constexpr int D = decltype(dtag)::value;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (a - b <= D) Mfma<T>::mma(acc[a][b], A[a], B[b]);
  };

  static_assert(NSTAGE >= 2 && NSTAGE <= 5, "ring depth 2..5");
  // at most n slabs' loads of one wave still in flight, counted as n * INST_PER_SLAB
  // (callers pass n <= NSTAGE - 1; more than 3 is waited for as 3); a loader wave
  // issues NWAVES / LOADERS times that per slab, so for it the wait is stricter than
  // n slabs, never looser: loads complete in issue order
  auto wait_loads = [&](int n) {
    if (n >= 3)
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(3 * INST_PER_SLAB));
    else if (n == 2)
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * INST_PER_SLAB));
    else if (n == 1)
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(INST_PER_SLAB));
    else
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  };

  const int64_t G = gridDim.x;
  int64_t v = blockIdx.x;   // < total: the grid never exceeds the item count
  TileRef cur, nxt;
  setup(v, cur);
  bool has_next = v + G < total;
  if (has_next) setup(v + G, nxt);

  // prologue: slabs 0..NSTAGE-1 of the first tile (every tile has more slabs)
#pragma unroll
  for (int sidx = 0; sidx < NSTAGE; ++sidx) issue(cur, sidx, sidx);
  // slab 0 landed: one slab's loads may still be in flight, unless a diagonal first
  // tile loaded one panel, where that count would also cover slab 0's
  if (ONE_PANEL && cur.diag)
    wait_loads(0);
  else
    wait_loads(NSTAGE - 1);
  __syncthreads();
  read_frags(IC<3>{}, smem, q_off(cur), 0, fa[0], fb[0]);
  int stage = 0;
  // The k-loop of one tile for a wave of diagonal class D (3 off the diagonal).
  auto kloop = [&](auto dtag) {
    constexpr int D = decltype(dtag)::value;
    constexpr int NM = n_active(D) * MMA_PER_PAIR;
    constexpr int NR_IN = a_needed(D) + (NB - b_first(D)) * READS_PER_B;   // reads inside the slab
    constexpr int NR_NEXT = 4 + NB * READS_PER_B;   // the next slab's first reads: every fragment
    for (int kt = 0; kt < cur.nk; ++kt) {
      const unsigned char* sP = smem + stage * STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk < KSTEPS - 1; ++kk) {
        read_frags(dtag, sP, q_off(cur), kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
        mfma_step(dtag, fa[kk & 1], fb[kk & 1]);
        interleave(IC<NR_IN>{}, IC<NM>{});
        __builtin_amdgcn_sched_barrier(0);
      }
      const int next = (stage + 1 == NSTAGE) ? 0 : stage + 1;
      // loads issued after slab kt+1's: slabs kt+2 .. kt+NSTAGE-1, those past this
      // tile only if there is a next one.  On the block's very last slab the reads
      // below fetch stale, unused fragments.
      wait_loads(has_next ? NSTAGE - 2 : min(NSTAGE - 2, cur.nk - kt - 2));
      __syncthreads();
      // slab kt + NSTAGE (of this tile or the next) goes into slab kt's stage; one
      // issue site per operand for both cases (see load_lds16x4)
      const int ks = kt + NSTAGE;
      const bool own = ks < cur.nk;
      const bool load = own || has_next;
      const TileRef& lt = own ? cur : nxt;
      const int lk = own ? ks : ks - cur.nk;
      if (EARLY_P && load) issue_op(lt, lk, stage, 0);
      // the next slab's first fragments, of this tile or (last slab) the next one:
      // all of them, whatever the next tile's class
      read_frags(IC<3>{}, smem + next * STAGE_BYTES, q_off(kt + 1 < cur.nk ? cur : nxt), 0, fa[0], fb[0]);
      mfma_step(dtag, fa[(KSTEPS - 1) & 1], fb[(KSTEPS - 1) & 1]);
      interleave(IC<NR_NEXT>{}, IC<NM>{});
      __builtin_amdgcn_sched_barrier(0);
      if (load) {
        if (!EARLY_P) issue_op(lt, lk, stage, 0);
        if (!(ONE_PANEL && lt.diag)) issue_op(lt, lk, stage, 1);
      }
      stage = next;
    }
  };
  for (;;) {
    zero_acc();
    if constexpr (SYM) {
      const int dc = cur.diag ? wdc : 3;
      if (dc == 3)
        kloop(IC<3>{});
      else if (dc == 2)
        kloop(IC<2>{});
      else if (dc == 0)
        kloop(IC<0>{});
      else
        kloop(IC<-NB>{});
    } else {
      kloop(IC<3>{});
    }

    {
      // a uniform index, so the descriptor comes in through scalar loads, which no
      // vmcnt wait covers (a vector load here would wait for the ring's loads too)
      const MatDesc& d = descs[__builtin_amdgcn_readfirstlane(cur.di)];
      const int ti = cur.ti, tj = cur.tj;
      const int i0 = ti * GT, j0 = tj * GT;
      // The first iteration's operand X is the unscaled momentum when `first` is
      // given: SYRK then scales its products by f^2 and APPLY by f, the matrix's
      // Frobenius factor (f = 1 where X was written scaled).  Otherwise alpha = 1,
      // and acc * 1 is acc exactly.
      float alpha = 1.f;
      if (MODE != GM_POLY && first != nullptr) {
        const float f = first[d.scale_slot];
        alpha = MODE == GM_SYRK ? f * f : f;
      }
      // Epilogue.  Accumulator layout of a 32x32 MFMA block: lane l, register r holds
      // row 8*(r/4) + 4*(l/32) + r%4, column l%32, so each lane owns 4 consecutive rows
      // ib..ib+3 of one column j per register group g.
      //
      // Both destinations are k-blocked along their columns (a 128-byte k-block row is
      // one line).  Row-major results straight from the registers take one instruction
      // per 64 contiguous bytes of each of 2 rows; with bf16 operands, APPLY's X' and
      // SYRK's off-diagonal A go through the staging slab below and leave as whole
      // lines instead (POLY has no registers to spare for that and stores its B'
      // tile's rows as 2-column pieces).  The
      // mirror tile of C (SYRK and POLY) would leave the registers as 8 or 16 bytes per
      // row per instruction, i.e. 8 partial writes per line, and L2 write traffic of
      // that shape slows everyone's operand loads.  It goes through this wave's 4 KiB
      // LDS staging slab instead: a round puts 32 columns j x 128 bytes of
      // rows i there in [j][i] order (16-byte chunks XOR-swizzled by j & 7) and sends
      // them out as whole 128-byte lines, 8 rows per instruction.  POLY needs b*A at
      // [ib..ib+3][j].
      typedef typename Vec4<T>::type v4_t;
      if (MODE != GM_APPLY_FINAL && MODE != GM_APPLY_WEIGHT) {
        constexpr int AP = 128 / (32 * static_cast<int>(sizeof(T)));   // MFMA row blocks per 128 bytes of k
        // row-major and transposed destinations (C[i][j] and C^T[j][i], both k-blocked
        // along their columns) and their k-block pitches
        gptr<T> Cr, Ct;
        uint32_t pr, pt;
        if (MODE == GM_APPLY) {
          // X' into the other ping-pong buffer (other tiles still read X); no
          // transposed copy
          Cr = Ct = global(static_cast<T*>(d.X[parity ^ 1]));
          pr = pt = d.pX;
        } else {
          Cr = Ct = global(static_cast<T*>(MODE == GM_SYRK ? d.A : d.B));
          pr = pt = d.pM;
        }
        const gptr<const T> Ain = global(static_cast<const T*>(d.A));
        const bool diag = MODE != GM_APPLY && ti == tj;
        // Every workspace buffer is below 2 GiB: element addresses are a uniform base
        // plus a 32-bit byte offset, one VGPR per address.
        constexpr uint32_t ES = sizeof(T);
        // the four results of register group (a, b, g): rows ib..ib+3 of column j
        auto values = [&](int a, int b, int g, int ib, int j, const v4_t& e, float (&v)[4]) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[t] = acc[a][b][4 * g + t] * alpha;
            if (MODE == GM_POLY) {
              v[t] = cb * to_f32(e[t]) + cc * v[t];
              if (diag && ib + t == j && j < d.m) v[t] += ca;
            }
          }
        };
        // A[ib..ib+3][j] for bA, read by rows: A is stored exactly symmetric, and with
        // consecutive lanes on consecutive j each element load covers 64 contiguous
        // bytes of each of 2 rows.  (The one vector load of A[j][ib..ib+3] per lane it
        // replaces touched 32 rows per instruction; POLY -0.8%.)
        auto load_e = [&](int ib, int j) {
          v4_t e;
#pragma unroll
          for (int t = 0; t < 4; ++t) e[t] = *at<const T>(Ain, kb_off<T>(ib + t, j, d.pM));
          return e;
        };
        unsigned char* stg = staging + wave * 4096;
        // One row block (32 rows) of row-major results through the staging slab: the
        // wave's 64 columns are one 128-byte k-block row, so the block goes out as 4
        // stores of 8 whole rows (1 KiB contiguous) each, not 64 stores of 128 bytes
        // (bf16 only: a row of 64 fp32 values spans two k-blocks).  Used for APPLY's
        // X' and for SYRK's A off the diagonal (whose rows are stored whole).
        auto stage_rows = [&](int a) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int r = 8 * g + 4 * half + t;        // row within the block
                const int off = (b * 32 + l32) * 2;        // byte within the row
                *reinterpret_cast<T*>(stg + r * 128 + ((((off >> 4) ^ (r & 7)) << 4) | (off & 15))) =
                    from_f32<T>(acc[a][b][4 * g + t] * alpha);
              }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = (lane >> 3) + 8 * q, c = lane & 7;
            const u32x4_t w = *reinterpret_cast<const u32x4_t*>(stg + r * 128 + ((c ^ (r & 7)) << 4));
            store_ws(at<u32x4_t>(Cr, kb_off<T>(i0 + wm + a * 32 + r, j0 + wn + c * 8, pr)), w);
          }
          __builtin_amdgcn_sched_barrier(0);   // blocks one after another
        };
        const bool staged_rows = MODE == GM_SYRK && sizeof(T) == 2 && !diag;
        if constexpr (sizeof(T) == 2 && MODE == GM_APPLY) {
#pragma unroll
          for (int a = 0; a < 4; ++a) stage_rows(a);
        } else
#pragma unroll
        for (int p = 0; p < 4 / AP; ++p) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const int j = j0 + wn + b * 32 + l32;
            v4_t e[AP][4];
            if (MODE == GM_POLY) {
#pragma unroll
              for (int ap = 0; ap < AP; ++ap)
#pragma unroll
                for (int g = 0; g < 4; ++g) e[ap][g] = load_e(i0 + wm + (AP * p + ap) * 32 + 8 * g + 4 * half, j);
            }
#pragma unroll
            for (int ap = 0; ap < AP; ++ap)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const int a = AP * p + ap;
                const int ib = i0 + wm + a * 32 + 8 * g + 4 * half;
                float v[4];
                values(a, b, g, ib, j, e[ap][g], v);
                // rows ib..ib+3 of column j: consecutive rows of one k-block are
                // ROW_BYTES apart, and a half-wave writes 64 contiguous bytes per row
                if (staged_rows) {
                  // stored whole after this pair of row blocks' mirror rounds
                } else if (MODE == GM_POLY && !diag) {
                  store_pairs<T>(Cr, pr, lane, ib, j, v);
                } else {
                  const uint32_t o = kb_off<T>(ib, j, pr);
#pragma unroll
                  for (int t = 0; t < 4; ++t)
                    if (!diag || ib + t <= j) store_ws(at<T>(Cr, o + t * ROW_BYTES), from_f32<T>(v[t]));
                }
                if (MODE == GM_APPLY) continue;
                const v4_t w = {from_f32<T>(v[0]), from_f32<T>(v[1]), from_f32<T>(v[2]), from_f32<T>(v[3])};
                const int off = (32 * ap + 8 * g + 4 * half) * static_cast<int>(ES);   // within the staged row
                *reinterpret_cast<v4_t*>(stg + l32 * 128 + ((((off >> 4) ^ (l32 & 7)) << 4) | (off & 15))) = w;
              }
            // the wave's own LDS accesses execute in order: these reads see the writes
            // above, and the next round's writes come after them
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (MODE == GM_APPLY) break;
              const int jr = (lane >> 3) + 8 * r, c = lane & 7;
              const u32x4_t w = *reinterpret_cast<const u32x4_t*>(stg + jr * 128 + ((c ^ (jr & 7)) << 4));
              // 16 bytes of row j of C^T, from column i0 + wm + 32 AP p + c (16 / es)
              // on; the 8 lanes of row j fill one whole k-block row (with 64-byte
              // k-blocks, rows j and j + 1, j even, share the line)
              const uint32_t jrow = static_cast<uint32_t>(j0 + wn + b * 32 + jr);
              const uint32_t icol = static_cast<uint32_t>(i0 + wm + 32 * AP * p) + c * (16 / sizeof(T));
              constexpr uint32_t EPV = 16 / sizeof(T);   // elements per 16-byte piece
              if (!diag || icol + EPV <= jrow) {
                store_ws(at<u32x4_t>(Ct, kb_off<T>(jrow, icol, pt)), w);
              } else if (icol < jrow) {
                // the piece that straddles the diagonal: only the mirrors of upper
                // elements (i < j), one by one
                T x[EPV];
                __builtin_memcpy(x, &w, 16);
#pragma unroll
                for (uint32_t e = 0; e < EPV; ++e)
                  if (icol + e < jrow) store_ws(at<T>(Ct, kb_off<T>(jrow, icol + e, pt)), x[e]);
              }
            }
            __builtin_amdgcn_sched_barrier(0);   // rounds one after another: bounded live ranges
          }
          if constexpr (MODE == GM_SYRK && sizeof(T) == 2) if (staged_rows) {
#pragma unroll
            for (int ap = 0; ap < AP; ++ap) stage_rows(AP * p + ap);
          }
        }
      } else {
        const gptr<TO> out = global(static_cast<TO*>(d.out));
        const int m = d.m, n = d.n;
        // register group (a, b, g): rows ib..ib+3 of column j, element by element
        // (or 4 at a time along a transposed output's row)
        auto plain_group = [&](int a, int b, int g) {
          const int ib = i0 + wm + a * 32 + 8 * g + 4 * half;
          const int j = j0 + wn + b * 32 + l32;
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = acc[a][b][4 * g + t] * alpha;
          // the value stored at o: U itself, or W - lr * U
          auto result = [&](gptr<TO> o, float u) {
            return from_f32<TO>(MODE == GM_APPLY_WEIGHT ? to_f32(*o) - ca * u : u);
          };
          if (j < n) {
            if (!d.transposed) {
              // out is m x n row-major
#pragma unroll
              for (int t = 0; t < 4; ++t)
                if (ib + t < m) {
                  const gptr<TO> o = out + static_cast<int64_t>(ib + t) * n + j;
                  *o = result(o, v[t]);
                }
            } else {
              // out is n x m row-major: out[j][i]
              const gptr<TO> o = out + static_cast<int64_t>(j) * m + ib;
              if (d.vec_ok && ib + 4 <= m) {
                if (MODE == GM_APPLY_WEIGHT) {
                  typedef typename Vec4<TO>::type w4_t;
                  const w4_t w = *reinterpret_cast<gptr<const w4_t>>(o);
#pragma unroll
                  for (int t = 0; t < 4; ++t) v[t] = to_f32(w[t]) - ca * v[t];
                }
                store4<TO>(o, v[0], v[1], v[2], v[3]);
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  if (ib + t < m) o[t] = result(o + t, v[t]);
              }
            }
          }
        };
        // U with bf16 elements through the staging slab, for blocks wholly inside the
        // matrix: whole 128-byte pieces of U's rows (64 elements) instead of 2-byte
        // stores (U as stored) or 8-byte pieces spread over 64 rows (U transposed).
        // Needs 16-byte aligned rows: the output base (vec_ok) and the row pitch.
        unsigned char* stg = staging + wave * 4096;
        const bool stage_out = MODE == GM_APPLY_FINAL && sizeof(TO) == 2 && d.vec_ok &&
                               (static_cast<int64_t>(d.transposed ? m : n) * 2) % 16 == 0;
        if (!d.transposed) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int r0 = i0 + wm + a * 32;
            if (sizeof(TO) == 2 && stage_out && r0 + 32 <= m && j0 + wn + 64 <= n) {
              // rows r0..r0+31, columns j0+wn..+63: [row][column] in the slab
#pragma unroll
              for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                  for (int t = 0; t < 4; ++t) {
                    const int r = 8 * g + 4 * half + t;
                    const int off = (b * 32 + l32) * 2;
                    *reinterpret_cast<TO*>(stg + r * 128 + ((((off >> 4) ^ (r & 7)) << 4) | (off & 15))) =
                        from_f32<TO>(acc[a][b][4 * g + t] * alpha);
                  }
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int r = (lane >> 3) + 8 * q, c = lane & 7;
                const u32x4_t w = *reinterpret_cast<const u32x4_t*>(stg + r * 128 + ((c ^ (r & 7)) << 4));
                *reinterpret_cast<gptr<u32x4_t>>(out + static_cast<int64_t>(r0 + r) * n + j0 + wn + c * 8) = w;
              }
            } else {
#pragma unroll
              for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g) plain_group(a, b, g);
            }
            __builtin_amdgcn_sched_barrier(0);   // blocks one after another
          }
        } else {
#pragma unroll
          for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const int ir = i0 + wm + 64 * p, jc = j0 + wn + b * 32;
              if (sizeof(TO) == 2 && stage_out && ir + 64 <= m && jc + 32 <= n) {
                // columns jc..jc+31 as rows of U, rows ir..ir+63 of X' along them:
                // [j][i] in the slab
                typedef typename Vec4<TO>::type o4_t;
#pragma unroll
                for (int ap = 0; ap < 2; ++ap)
#pragma unroll
                  for (int g = 0; g < 4; ++g) {
                    const int a = 2 * p + ap;
                    const o4_t w = {from_f32<TO>(acc[a][b][4 * g] * alpha), from_f32<TO>(acc[a][b][4 * g + 1] * alpha),
                                    from_f32<TO>(acc[a][b][4 * g + 2] * alpha),
                                    from_f32<TO>(acc[a][b][4 * g + 3] * alpha)};
                    const int off = (32 * ap + 8 * g + 4 * half) * 2;
                    *reinterpret_cast<o4_t*>(stg + l32 * 128 + ((((off >> 4) ^ (l32 & 7)) << 4) | (off & 15))) = w;
                  }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const int jr = (lane >> 3) + 8 * r, c = lane & 7;
                  const u32x4_t w = *reinterpret_cast<const u32x4_t*>(stg + jr * 128 + ((c ^ (jr & 7)) << 4));
                  *reinterpret_cast<gptr<u32x4_t>>(out + static_cast<int64_t>(jc + jr) * m + ir + c * 8) = w;
                }
              } else {
#pragma unroll
                for (int ap = 0; ap < 2; ++ap)
#pragma unroll
                  for (int g = 0; g < 4; ++g) plain_group(2 * p + ap, b, g);
              }
              __builtin_amdgcn_sched_barrier(0);   // rounds one after another
            }
        }
      }
    }
    if (!has_next) break;
    cur = nxt;
    v += G;
    has_next = v + G < total;
    if (has_next) setup(v + G, nxt);
  }
}

}  // namespace mo
