// libmatopt: host side of the C ABI declared in include/matopt.h.
//
// One batched call = one descriptor table (written to the head of the caller's
// workspace by copy kernels that take it as kernel arguments) + a fixed launch
// sequence on the caller's stream:
//   k_momentum_prep    momentum fma in place, the unscaled oriented operand X,
//                      per-tile sum of squares                          (HBM)
//   k_norm_scale       per-matrix s = 1 / (||M||_F + eps)                (tiny)
//   k_prep_redo        X = s M for norms outside the deferral range     (usually idle)
//   iters x { k_ns_gemm<SYRK>, k_ns_gemm<POLY>, k_ns_gemm<APPLY> }       (MFMA)
//             A = X X^T,  B' = aI + bA + cA^2,  X <- B' X
//             (the first SYRK and APPLY take the factor s^2 and s)
// With iters == 0 the sequence is k_momentum_sumsq (momentum + per-chunk sum of
// squares), k_norm_scale and k_scaled_copy (U = s M).
// Each launch covers every matrix of the batch (grouped launch); blocks find their
// matrix by binary search over the table, which is sorted by decreasing size so
// the longest tiles start first.  The GEMM launches are persistent: one block per
// CU, each walking a strided share of the tile list.  When those launches hold only
// a few rounds of tiles, the batch is cut into two halves whose products run on the
// caller's stream and on a second stream of the library's own (split_wanted).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <mutex>
#include <numeric>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/matopt.h"
#include "common.h"
#include "elementwise.h"
#include "gemm.h"
#include "smallgemm.h"
#include "planner.h"

using namespace mo;

// Scratch of the allocation-free entry point (muon_step_batched_noalloc): the
// descriptor table, scalars, partial sums and X/A/B operands live here instead of
// in a caller workspace.  Each GPU the library is loaded on holds its own copy for
// the life of the process.  Host code never uses this name as an address: the
// per-device address comes from hipGetSymbolAddress (scratch_base below).
static __device__ __attribute__((aligned(256))) unsigned char scratch[MO_NOALLOC_SCRATCH_BYTES];

namespace {

// Descriptor upload through kernel arguments, DESC_ARG descriptors per launch of a
// copy kernel into the head of the workspace: the runtime copies the argument block
// into its own kernel-argument memory, so the upload needs no pinned staging
// buffer, no host wait and no allocation, and stays in stream order.  (It replaced a
// pinned staging ring with hipMemcpyAsync, which allocated on first use and made the
// host wait once four calls were in flight; step times are unchanged.)
constexpr int DESC_ARG = 16;
struct DescArg {
  MatDesc d[DESC_ARG];
};
static_assert(sizeof(DescArg) <= 4000, "kernel argument block too large");
static_assert(sizeof(MatDesc) % 4 == 0, "descriptors are copied as 32-bit words");

__global__ __launch_bounds__(256) void k_store_descs(DescArg a, int n, MatDesc* __restrict__ dst) {
  const uint32_t* src = reinterpret_cast<const uint32_t*>(&a.d[0]);
  uint32_t* out = reinterpret_cast<uint32_t*>(dst);
  const int words = n * static_cast<int>(sizeof(MatDesc) / 4);
  for (int i = threadIdx.x; i < words; i += blockDim.x) out[i] = src[i];
}

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

constexpr int64_t MAX_DIM = int64_t(1) << 24;
constexpr size_t ALIGN = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
size_t dtype_size(int dt) { return dt == MO_F32 ? 4 : 2; }
bool valid_dtype(int dt) { return dt == MO_F32 || dt == MO_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
  std::vector<MatDesc> descs;
  int64_t total[NKIND] = {};
  size_t off_desc = 0, off_scale = 0, off_partial = 0, bytes = 0;
  // Split plans (see split_wanted): descriptors [0, split_at) are half A, the rest
  // half B; the 256-tile GEMM kinds number their items from 0 in each half, and
  // half_total[h][kind] counts them (the other kinds number across the whole table).
  int split_at = 0;
  int64_t half_total[2][3] = {};
  // the largest m among the 256-tile matrices of each half (of the whole list in
  // [0] when it is not split): it picks the GEMM kernel variant
  int32_t max_m[2] = {0, 0};
};
// the GEMM kinds a split plan numbers per half
bool per_half_kind(int kd) { return kd == KIND_SYRK || kd == KIND_POLY || kd == KIND_APPLY; }
// The per-matrix scalars at off_scale: scale[count] (s = 1 / (||M||_F + eps)),
// first[count] (the factor the first NS products apply) and redo[count] (int flags).

// Validate the list and lay out the workspace.  base == nullptr only sizes it.
int build_plan(const mo_matrix* mats, int count, int compute, bool momentum, unsigned char* base,
               Plan& plan, int in_dtype = MO_F32, int out_dtype = MO_F32, bool split = false) {
  if (count < 0) return fail(MO_ERR_INVALID, "count must be >= 0");
  if (count > 0 && !mats) return fail(MO_ERR_INVALID, "mats is NULL");
  if (!valid_dtype(compute)) return fail(MO_ERR_UNSUPPORTED, "compute dtype must be MO_F32 or MO_BF16");
  const size_t es = dtype_size(compute);
  std::vector<int> order(count);
  std::iota(order.begin(), order.end(), 0);
  for (int i = 0; i < count; ++i) {
    const mo_matrix& mt = mats[i];
    if (mt.rows < 1 || mt.cols < 1 || mt.rows > MAX_DIM || mt.cols > MAX_DIM)
      return fail(MO_ERR_INVALID, "matrix " + std::to_string(i) + ": rows and cols must be in [1, 2^24]");
    if (base) {
      if (!mt.out) return fail(MO_ERR_INVALID, "matrix " + std::to_string(i) + ": out is NULL");
      if (momentum && (!mt.grad || !mt.momentum))
        return fail(MO_ERR_INVALID, "matrix " + std::to_string(i) + ": grad or momentum is NULL");
      if (!momentum && !mt.x) return fail(MO_ERR_INVALID, "matrix " + std::to_string(i) + ": x is NULL");
      if (!momentum && mt.x == mt.out && in_dtype != out_dtype)
        return fail(MO_ERR_INVALID, "matrix " + std::to_string(i) + ": x == out needs in_dtype == out_dtype");
    }
  }
  std::stable_sort(order.begin(), order.end(), [&](int p, int q) {
    return mats[p].rows * mats[p].cols > mats[q].rows * mats[q].cols;
  });
  if (split && count >= 2) {
    // half A: every other matrix of the sorted order from the first, half B the
    // rest, so both halves hold the same mix of shapes (each still sorted)
    std::vector<int> halves;
    for (int h = 0; h < 2; ++h)
      for (int k = h; k < count; k += 2) halves.push_back(order[k]);
    order.swap(halves);
    plan.split_at = (count + 1) / 2;
  }
  size_t off = 0;
  plan.off_desc = off;
  off = align_up(off + sizeof(MatDesc) * std::max(count, 1), ALIGN);
  plan.off_scale = off;
  off = align_up(off + (2 * sizeof(float) + sizeof(int)) * std::max(count, 1), ALIGN);
  // one fp64 partial sum per 4096-element chunk (iters == 0) or per 64x64 operand
  // tile (the fused pass)
  int64_t chunks = 0, tiles = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t r = mats[i].rows, c = mats[i].cols;
    chunks += (r * c + CHUNK - 1) / CHUNK;
    tiles += (round_up(std::min(r, c), GEMM_TILE) / PREP_TILE) * (round_up(std::max(r, c), GEMM_TILE) / PREP_TILE);
  }
  plan.off_partial = off;
  off = align_up(off + sizeof(double) * std::max<int64_t>(std::max(chunks, tiles), 1), ALIGN);

  plan.descs.resize(count);
  for (int k = 0; k < count; ++k) {
    const mo_matrix& mt = mats[order[k]];
    MatDesc& d = plan.descs[k];
    std::memset(&d, 0, sizeof(d));
    d.grad = momentum ? mt.grad : mt.x;
    d.mom = momentum ? mt.momentum : nullptr;
    d.out = mt.out;
    d.rows = mt.rows;
    d.cols = mt.cols;
    d.numel = mt.rows * mt.cols;
    d.transposed = mt.rows > mt.cols ? 1 : 0;
    d.m = static_cast<int32_t>(std::min(mt.rows, mt.cols));
    d.n = static_cast<int32_t>(std::max(mt.rows, mt.cols));
    d.mp = static_cast<int32_t>(round_up(d.m, GEMM_TILE));
    d.np = static_cast<int32_t>(round_up(d.n, GEMM_TILE));
    d.vec_ok = (aligned16(d.grad) && aligned16(d.mom) && aligned16(d.out) && (mt.cols % 4 == 0)) ? 1 : 0;
    d.scale_slot = k;
    // k-blocked operands: np / kb blocks of mp rows (X), mp / kb blocks of mp rows
    // (A, B); mp and np are multiples of kb
    const size_t kb = KB_BYTES / es;
    const size_t xb = size_t(d.np) / kb * size_t(d.mp) * KB_BYTES;
    const size_t ab = size_t(d.mp) / kb * size_t(d.mp) * KB_BYTES;
    // the GEMM addresses each operand buffer with 32-bit byte offsets
    if (xb > size_t(0x7fffffff))
      return fail(MO_ERR_UNSUPPORTED, "matrix " + std::to_string(order[k]) +
                                          ": padded operand exceeds 2 GiB (min(rows,cols) * max(rows,cols))");
    d.pX = static_cast<uint32_t>(d.mp) * KB_BYTES;
    d.pM = static_cast<uint32_t>(d.mp) * KB_BYTES;
    auto take = [&](size_t nb) {
      void* p = base ? static_cast<void*>(base + off) : nullptr;
      off = align_up(off + nb, ALIGN);
      return p;
    };
    d.X[0] = take(xb);
    d.X[1] = take(xb);
    d.A = take(ab);
    d.B = take(ab);
    // products: matrices with m <= 256 on 32 x 32 blocks (smallgemm.h), the others
    // on 256 x 256 tiles; the choice depends on the matrix alone, so a matrix's
    // result never depends on the rest of the batch
    const bool small = d.mp == GEMM_TILE;
    const int64_t tm = d.mp / GEMM_TILE, tn = d.np / GEMM_TILE;
    d.items[KIND_SYRK] = small ? 0 : tm * (tm + 1) / 2;
    d.items[KIND_POLY] = small ? 0 : tm * (tm + 1) / 2;
    d.items[KIND_APPLY] = small ? 0 : tm * tn;
    d.items[KIND_SMALL_UPPER] = small ? small_upper_items(d.m) : 0;
    d.items[KIND_SMALL_RECT] = small ? small_rect_items(d.m, d.n) : 0;
    d.items[KIND_PREP] = (int64_t(d.mp) / PREP_TILE) * (int64_t(d.np) / PREP_TILE);
    d.items[KIND_CHUNK] = (d.numel + CHUNK - 1) / CHUNK;
    const int h = (plan.split_at > 0 && k >= plan.split_at) ? 1 : 0;
    if (d.items[KIND_APPLY] > 0) plan.max_m[h] = std::max(plan.max_m[h], d.m);
    for (int kd = 0; kd < NKIND; ++kd) {
      if (plan.split_at > 0 && per_half_kind(kd)) {
        d.begin[kd] = plan.half_total[h][kd - KIND_SYRK];
        plan.half_total[h][kd - KIND_SYRK] += d.items[kd];
      } else {
        d.begin[kd] = plan.total[kd];
      }
      plan.total[kd] += d.items[kd];
    }
  }
  for (int kd = 0; kd < NKIND; ++kd)
    if (plan.total[kd] > 0x7fffffffLL) return fail(MO_ERR_INVALID, "batch too large for one launch");
  plan.bytes = off;
  return MO_OK;
}

// ---- optional per-kernel timing ------------------------------------------------
struct ProfRec {
  int kind;
  hipEvent_t e0, e1;
};
// Profiling state is shared by every thread that calls the library; g_prof_mu guards
// the record list and the event pool.
std::atomic<bool> g_prof{false};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_ev_pool;
const char* const kKindNames[] = {"momentum_sumsq", "norm_scale",  "prep_operand", "scaled_copy",
                                  "ns_syrk",        "ns_poly",     "ns_apply",     "sign_pack",
                                  "sign_vote",      "sign_unpack", "sign_apply",   "momentum_prep"};
enum { PK_MOM = 0, PK_SCALE, PK_PREP, PK_COPY, PK_SYRK, PK_POLY, PK_APPLY, PK_PACK, PK_VOTE, PK_UNPACK,
       PK_SAPPLY, PK_MOMPREP, PK_N };

// (g_prof_mu held)
hipEvent_t take_event() {
  if (!g_ev_pool.empty()) {
    hipEvent_t e = g_ev_pool.back();
    g_ev_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  (void)hipEventCreate(&e);
  return e;
}

// Launch helper: optional event bracket + launch error check.
// Set for the duration of an allocation-free call: its launches record no profiling
// events (creating one may allocate).
thread_local bool g_no_events = false;

template <typename F>
int launch(int pk, hipStream_t stream, F&& f) {
  ProfRec rec{pk, nullptr, nullptr};
  const bool prof = g_prof.load() && !g_no_events;
  if (prof) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    rec.e0 = take_event();
    rec.e1 = take_event();
  }
  if (rec.e0) (void)hipEventRecord(rec.e0, stream);
  f();
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(MO_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(err));
  if (rec.e0 && rec.e1 && hipEventRecord(rec.e1, stream) == hipSuccess) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_recs.push_back(rec);
  }
  return MO_OK;
}

#define MO_TRY(x)            \
  do {                       \
    int rc_ = (x);           \
    if (rc_ != MO_OK) return rc_; \
  } while (0)

// Blocks of a persistent GEMM launch: one per CU (the LDS ring admits no second
// block), rounded down to a multiple of the 8 XCDs, never more than the work items.
int64_t gemm_grid(int64_t total) {
  static std::atomic<int> cus[64];   // per device, 0 until first asked
  int dev = 0;
  (void)hipGetDevice(&dev);
  int n = (dev >= 0 && dev < 64) ? cus[dev].load() : 0;
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 8;
    if (dev >= 0 && dev < 64) cus[dev].store(n);
  }
  const int64_t g = n >= 8 ? n / 8 * 8 : n;
  return std::min<int64_t>(total, g);
}

// Apply mode: the last APPLY (or the iters == 0 copy) updates the caller's weight,
// out <- out - lr * U, instead of writing U.
struct ApplyOpt {
  bool on = false;
  float lr = 0.f;
};

// The second stream of a split call (see split_wanted), per device: created on
// first use with the default priority, kept for the life of the process, with the
// two events that fork it from the caller's stream and join it back.  `mu` is held
// from the fork to the join, so calls from several threads do not interleave their
// use of the events.
struct SideStream {
  std::mutex mu;
  bool tried = false;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream g_side[64];

// This device's side stream, or nullptr if it is unavailable (creating it failed).
SideStream* side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& ss = g_side[dev];
  std::lock_guard<std::mutex> lock(ss.mu);
  if (!ss.tried) {
    ss.tried = true;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      if (ss.join) (void)hipEventDestroy(ss.join);
      if (ss.fork) (void)hipEventDestroy(ss.fork);
      if (ss.s) (void)hipStreamDestroy(ss.s);
      ss.s = nullptr;
      ss.fork = ss.join = nullptr;
      (void)hipGetLastError();
    }
  }
  return ss.s ? &ss : nullptr;
}

// Whether a call's NS products run as two halves on two streams.  Each launch of a
// product deals its tiles to one block per CU in rounds; when a launch holds only a
// few rounds, its last round leaves most CUs idle (1296 APPLY tiles over 256 CUs
// are 5.06 rounds), and a second half running on another stream fills them.
// Measured on one box, two or three rounds each: 125M-class owner set (5 APPLY
// rounds) 2.15-2.17 -> 2.04-2.05 ms per step, 8 x 4096^2 orthogonalisation (8
// rounds) 9.96-10.03 -> 9.48 ms, 1B-class set (49 rounds) 29.53-29.62 -> 29.05-29.25
// ms; as two calls from Python the 7B-class set (386 rounds) gained nothing, and
// three or four streams were slower.  Not under stream capture, and not for the
// allocation-free call.
constexpr int64_t SPLIT_MAX_ROUNDS = 64;
bool split_wanted(const Plan& sizing, int count, const mo_ns_params& ns, hipStream_t stream) {
  if (count < 2 || ns.iters < 1) return false;
  const int64_t ta = sizing.total[KIND_APPLY];
  const int64_t g = gemm_grid(std::numeric_limits<int32_t>::max());
  if (ta == 0 || ta >= SPLIT_MAX_ROUNDS * g) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}

// k NS iterations: per product one persistent 256 x 256-tile launch over the
// matrices with m > 256 and one 32 x 32-block launch (smallgemm.h) over those with
// m <= 256; a launch with no items is skipped.  A split plan launches each
// 256-tile product once per half: half A on the caller's stream, half B on the side
// stream, forked after the first pass and joined before the call returns (the
// small-path launches stay on the caller's stream).
template <typename T, typename TO>
int run_ns(const MatDesc* dd, int count, const Plan& plan, const mo_ns_params& ns, const ApplyOpt& ap,
           const float* first, hipStream_t stream, SideStream* side) {
  const int64_t nu = plan.total[KIND_SMALL_UPPER], nr = plan.total[KIND_SMALL_RECT];
  const dim3 gu(nu), gr(nr);   // one 32 x 32 block per 256-thread block
  // the 256-tile launches of one half: descriptors, their count, item totals, stream
  struct Half {
    const MatDesc* dd;
    int count;
    int64_t ts, tp, ta;
    hipStream_t stream;
    bool smallk;   // SYRK / POLY: bf16 operands and every matrix m <= SMALLK_MAX_M (gemm.h)
  };
  Half halves[2];
  int nh = 1;
  const bool split = plan.split_at > 0 && side != nullptr;
  if (split) {
    halves[0] = {dd, plan.split_at, plan.half_total[0][0], plan.half_total[0][1], plan.half_total[0][2], stream,
                 false};
    halves[1] = {dd + plan.split_at, count - plan.split_at, plan.half_total[1][0], plan.half_total[1][1],
                 plan.half_total[1][2], side->s, false};
    nh = 2;
  } else {
    halves[0] = {dd, count, plan.total[KIND_SYRK], plan.total[KIND_POLY], plan.total[KIND_APPLY], stream, false};
  }
  for (int h = 0; h < nh; ++h) halves[h].smallk = sizeof(T) == 2 && plan.max_m[h] <= SMALLK_MAX_M;
  // one 256-tile product launch of one half, in the kernel variant the half takes
  auto gemm = [&](auto mode, const Half& H, int64_t items, int parity, float ca, float cb, float cc,
                  const float* f) {
    constexpr int M = decltype(mode)::value;
    const dim3 grid(gemm_grid(items));
    if constexpr (sizeof(T) == 2 && (M == GM_SYRK || M == GM_POLY)) {
      if (H.smallk) {
        hipLaunchKernelGGL((k_ns_gemm<T, M, TO, true>), grid, dim3(NTHREADS), 0, H.stream, H.dd, H.count, items,
                           parity, ca, cb, cc, f);
        return;
      }
    }
    hipLaunchKernelGGL((k_ns_gemm<T, M, TO, false>), grid, dim3(NTHREADS), 0, H.stream, H.dd, H.count, items,
                       parity, ca, cb, cc, f);
  };
  std::unique_lock<std::mutex> lock;
  if (split) {
    lock = std::unique_lock<std::mutex>(side->mu);
    if (hipEventRecord(side->fork, stream) != hipSuccess || hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
      return fail(MO_ERR_HIP, "forking the side stream failed");
  }
  auto products = [&]() -> int {
    for (int t = 0; t < ns.iters; ++t) {
      const int parity = t & 1;
      const float* f = t == 0 ? first : nullptr;   // the Frobenius factor, first iteration only
      const bool last = (t + 1 == ns.iters);
      for (int h = 0; h < nh; ++h) {
        const Half& H = halves[h];
        if (H.ts == 0) continue;
        MO_TRY(launch(PK_SYRK, H.stream, [&] { gemm(IC<GM_SYRK>{}, H, H.ts, parity, 0.f, 0.f, 0.f, f); }));
      }
      for (int h = 0; h < nh; ++h) {
        const Half& H = halves[h];
        if (H.tp == 0) continue;
        MO_TRY(launch(PK_POLY, H.stream, [&] { gemm(IC<GM_POLY>{}, H, H.tp, parity, ns.a, ns.b, ns.c, nullptr); }));
      }
      for (int h = 0; h < nh; ++h) {
        const Half& H = halves[h];
        if (H.ta == 0) continue;
        MO_TRY(launch(PK_APPLY, H.stream, [&] {
          if (last && ap.on)
            gemm(IC<GM_APPLY_WEIGHT>{}, H, H.ta, parity, ap.lr, 0.f, 0.f, f);
          else if (last)
            gemm(IC<GM_APPLY_FINAL>{}, H, H.ta, parity, 0.f, 0.f, 0.f, f);
          else
            gemm(IC<GM_APPLY>{}, H, H.ta, parity, 0.f, 0.f, 0.f, f);
        }));
      }
      if (nu > 0) {
        MO_TRY(launch(PK_SYRK, stream, [&] {
          hipLaunchKernelGGL((k_ns_small<T, GM_SYRK, TO>), gu, dim3(256), 0, stream, dd, count, nu, parity, 0.f,
                             0.f, 0.f, f);
        }));
        MO_TRY(launch(PK_POLY, stream, [&] {
          hipLaunchKernelGGL((k_ns_small<T, GM_POLY, TO>), gu, dim3(256), 0, stream, dd, count, nu, parity, ns.a,
                             ns.b, ns.c, nullptr);
        }));
        MO_TRY(launch(PK_APPLY, stream, [&] {
          if (last && ap.on)
            hipLaunchKernelGGL((k_ns_small<T, GM_APPLY_WEIGHT, TO>), gr, dim3(256), 0, stream, dd, count, nr,
                               parity, ap.lr, 0.f, 0.f, f);
          else if (last)
            hipLaunchKernelGGL((k_ns_small<T, GM_APPLY_FINAL, TO>), gr, dim3(256), 0, stream, dd, count, nr,
                               parity, 0.f, 0.f, 0.f, f);
          else
            hipLaunchKernelGGL((k_ns_small<T, GM_APPLY, TO>), gr, dim3(256), 0, stream, dd, count, nr, parity,
                               0.f, 0.f, 0.f, f);
        }));
      }
    }
    return MO_OK;
  };
  const int rc = products();
  if (split) {
    // joined on every path, so no work of this call outlives it on the side stream
    // unordered with the caller's later work
    const bool ok = hipEventRecord(side->join, side->s) == hipSuccess &&
                    hipStreamWaitEvent(stream, side->join, 0) == hipSuccess;
    if (rc == MO_OK && !ok) return fail(MO_ERR_HIP, "joining the side stream failed");
  }
  return rc;
}

// Per-matrix device scalars and partial sums inside the workspace.
struct Scalars {
  float* scale;
  float* first;
  int* redo;
  double* partial;
};

// The launch sequence after the descriptor upload.  TG: the dtype of the input
// (gradient, or x for orthogonalise only); TC: compute; TO: output.
template <typename TG, typename TC, typename TO>
int run_step(const MatDesc* dd, int count, const Plan& plan, const Scalars& sc, bool momentum, float beta,
             const mo_ns_params& ns, const ApplyOpt& ap, hipStream_t stream, SideStream* side) {
  // the NS source after the first pass: the fp32 momentum, or the input itself
  typedef typename std::conditional<std::is_same<TG, float>::value, float, bf16_t>::type TX;
  const int from_mom = momentum ? 1 : 0;
  if (ns.iters == 0) {
    MO_TRY(launch(PK_MOM, stream, [&] {
      const dim3 grid(plan.total[KIND_CHUNK]);
      if (momentum)
        hipLaunchKernelGGL((k_momentum_sumsq<TG, true>), grid, dim3(256), 0, stream, dd, count, beta, sc.partial);
      else
        hipLaunchKernelGGL((k_momentum_sumsq<TG, false>), grid, dim3(256), 0, stream, dd, count, beta, sc.partial);
    }));
    MO_TRY(launch(PK_SCALE, stream, [&] {
      hipLaunchKernelGGL(k_norm_scale, dim3(count), dim3(256), 0, stream, dd, sc.partial, int(KIND_CHUNK), ns.eps,
                         sc.scale, static_cast<float*>(nullptr), static_cast<int*>(nullptr));
    }));
    return launch(PK_COPY, stream, [&] {
      if (momentum)
        hipLaunchKernelGGL((k_scaled_copy<float, TO>), dim3(plan.total[KIND_CHUNK]), dim3(256), 0, stream, dd,
                           count, sc.scale, from_mom, ap.on ? 1 : 0, ap.lr);
      else
        hipLaunchKernelGGL((k_scaled_copy<TX, TO>), dim3(plan.total[KIND_CHUNK]), dim3(256), 0, stream, dd,
                           count, sc.scale, from_mom, ap.on ? 1 : 0, ap.lr);
    });
  }
  MO_TRY(launch(PK_MOMPREP, stream, [&] {
    const dim3 grid(plan.total[KIND_PREP] / MP_TPB);   // a multiple of 16 items per matrix
    if (momentum)
      hipLaunchKernelGGL((k_momentum_prep<TG, TC, true>), grid, dim3(256), 0, stream, dd, count, beta, sc.partial);
    else
      hipLaunchKernelGGL((k_momentum_prep<TG, TC, false>), grid, dim3(256), 0, stream, dd, count, beta, sc.partial);
  }));
  MO_TRY(launch(PK_SCALE, stream, [&] {
    hipLaunchKernelGGL(k_norm_scale, dim3(count), dim3(256), 0, stream, dd, sc.partial, int(KIND_PREP), ns.eps,
                       sc.scale, sc.first, sc.redo);
  }));
  MO_TRY(launch(PK_PREP, stream, [&] {
    const dim3 grid(std::min<int64_t>(plan.total[KIND_PREP], 2048));
    if (momentum)
      hipLaunchKernelGGL((k_prep_redo<float, TC>), grid, dim3(256), 0, stream, dd, count, sc.scale, sc.redo,
                         from_mom);
    else
      hipLaunchKernelGGL((k_prep_redo<TX, TC>), grid, dim3(256), 0, stream, dd, count, sc.scale, sc.redo,
                         from_mom);
  }));
  return run_ns<TC, TO>(dd, count, plan, ns, ap, sc.first, stream, side);
}

template <typename TG>
int dispatch_compute_out(const MatDesc* dd, int count, const Plan& plan, const Scalars& sc, bool momentum,
                         float beta, int compute, int out, const mo_ns_params& ns, const ApplyOpt& ap,
                         hipStream_t stream, SideStream* side) {
  if (compute == MO_BF16) {
    if (out == MO_BF16)
      return run_step<TG, bf16_t, bf16_t>(dd, count, plan, sc, momentum, beta, ns, ap, stream, side);
    return run_step<TG, bf16_t, float>(dd, count, plan, sc, momentum, beta, ns, ap, stream, side);
  }
  if (out == MO_BF16) return run_step<TG, float, bf16_t>(dd, count, plan, sc, momentum, beta, ns, ap, stream, side);
  return run_step<TG, float, float>(dd, count, plan, sc, momentum, beta, ns, ap, stream, side);
}

// Address of this device's copy of `scratch`, looked up once per device with that
// device current and kept.
std::atomic<void*> g_scratch_base[64];

int scratch_base(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MO_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(MO_ERR_UNSUPPORTED, "device index above 63");
  void* p = g_scratch_base[dev].load();
  if (!p) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MO_ERR_HIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
    g_scratch_base[dev].store(p);
  }
  *out = p;
  return MO_OK;
}

int upload_by_args(MatDesc* dst, const MatDesc* src, int count, hipStream_t stream) {
  for (int k0 = 0; k0 < count; k0 += DESC_ARG) {
    const int n = std::min(DESC_ARG, count - k0);
    DescArg a;
    std::memset(&a, 0, sizeof(a));
    std::memcpy(a.d, src + k0, sizeof(MatDesc) * n);
    hipLaunchKernelGGL(k_store_descs, dim3(1), dim3(256), 0, stream, a, n, dst + k0);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(MO_ERR_HIP, std::string("descriptor upload failed: ") + hipGetErrorString(err));
  }
  return MO_OK;
}

// Switches event recording off for this thread while it lives (when `on`).
struct NoEvents {
  bool on;
  explicit NoEvents(bool o) : on(o) {
    if (on) g_no_events = true;
  }
  ~NoEvents() {
    if (on) g_no_events = false;
  }
};

// noalloc: the workspace is this device's `scratch` (workspace and ws_bytes are
// ignored), the descriptor table goes up through kernel arguments, and no call
// below allocates.
int batched(const mo_matrix* mats, int count, int in_dtype, int compute, int out, bool momentum, float beta,
            const mo_ns_params* ns, void* workspace, size_t ws_bytes, void* stream_ptr,
            const ApplyOpt& ap = ApplyOpt(), bool noalloc = false) {
  g_err.clear();
  if (ap.on && !std::isfinite(ap.lr)) return fail(MO_ERR_INVALID, "lr must be finite");
  if (!ns) return fail(MO_ERR_INVALID, "ns params is NULL");
  if (!valid_dtype(in_dtype) || !valid_dtype(compute) || !valid_dtype(out))
    return fail(MO_ERR_UNSUPPORTED, "dtypes must be MO_F32 or MO_BF16");
  if (ns->iters < 0) return fail(MO_ERR_INVALID, "iters must be >= 0");
  if (!std::isfinite(ns->a) || !std::isfinite(ns->b) || !std::isfinite(ns->c) || !std::isfinite(ns->eps) ||
      ns->eps < 0.f || !std::isfinite(beta))
    return fail(MO_ERR_INVALID, "coefficients, beta and eps must be finite, eps >= 0");
  Plan plan;
  MO_TRY(build_plan(mats, count, compute, momentum, nullptr, plan, in_dtype, out));
  if (count == 0) return MO_OK;
  if (noalloc) {
    if (plan.bytes > MO_NOALLOC_SCRATCH_BYTES)
      return fail(MO_ERR_WORKSPACE, "the allocation-free step needs " + std::to_string(plan.bytes) +
                                        " bytes of scratch; it holds " + std::to_string(MO_NOALLOC_SCRATCH_BYTES));
    MO_TRY(scratch_base(&workspace));
    ws_bytes = MO_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace) return fail(MO_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(workspace) & (ALIGN - 1)))
    return fail(MO_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < plan.bytes)
    return fail(MO_ERR_WORKSPACE, "workspace too small: need " + std::to_string(plan.bytes) + " bytes");
  unsigned char* base = static_cast<unsigned char*>(workspace);
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  SideStream* side = (!noalloc && split_wanted(plan, count, *ns, stream)) ? side_stream() : nullptr;
  Plan full;
  MO_TRY(build_plan(mats, count, compute, momentum, base, full, in_dtype, out, side != nullptr));
  MatDesc* dd = reinterpret_cast<MatDesc*>(base + full.off_desc);
  Scalars sc;
  sc.scale = reinterpret_cast<float*>(base + full.off_scale);
  sc.first = sc.scale + count;
  sc.redo = reinterpret_cast<int*>(sc.first + count);
  sc.partial = reinterpret_cast<double*>(base + full.off_partial);
  const NoEvents quiet(noalloc);
  MO_TRY(upload_by_args(dd, full.descs.data(), count, stream));
  if (in_dtype == MO_BF16)
    return dispatch_compute_out<bf16_t>(dd, count, full, sc, momentum, beta, compute, out, *ns, ap, stream, side);
  return dispatch_compute_out<float>(dd, count, full, sc, momentum, beta, compute, out, *ns, ap, stream, side);
}

}  // namespace

extern "C" {

size_t muon_workspace_bytes(const mo_matrix* mats, int32_t count, int32_t compute_dtype) {
  g_err.clear();
  Plan plan;
  if (build_plan(mats, count, compute_dtype, true, nullptr, plan) != MO_OK) return 0;
  return plan.bytes;
}

int32_t muon_step_batched(const mo_matrix* mats, int32_t count, int32_t grad_dtype, int32_t compute_dtype,
                          int32_t out_dtype, float beta, const mo_ns_params* ns, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return batched(mats, count, grad_dtype, compute_dtype, out_dtype, true, beta, ns, workspace, workspace_bytes,
                 stream);
}

int32_t muon_step_batched_noalloc(const mo_matrix* mats, int32_t count, int32_t grad_dtype, int32_t compute_dtype,
                                  int32_t out_dtype, float beta, const mo_ns_params* ns, void* stream) {
  return batched(mats, count, grad_dtype, compute_dtype, out_dtype, true, beta, ns, nullptr, 0, stream, ApplyOpt(),
                 true);
}

int32_t muon_step_apply(const mo_matrix* mats, int32_t count, int32_t grad_dtype, int32_t compute_dtype,
                        int32_t weight_dtype, float beta, const mo_ns_params* ns, float lr, void* workspace,
                        size_t workspace_bytes, void* stream) {
  ApplyOpt ap;
  ap.on = true;
  ap.lr = lr;
  return batched(mats, count, grad_dtype, compute_dtype, weight_dtype, true, beta, ns, workspace, workspace_bytes,
                 stream, ap);
}

int32_t ns_orthogonalize(const mo_matrix* mats, int32_t count, int32_t in_dtype, int32_t compute_dtype,
                         int32_t out_dtype, const mo_ns_params* ns, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return batched(mats, count, in_dtype, compute_dtype, out_dtype, false, 0.f, ns, workspace, workspace_bytes,
                 stream);
}

int32_t sign_pack_batched(const void* u, int32_t dtype, int32_t M, int64_t numel, int64_t u_stride,
                          uint32_t* packed, void* stream_ptr) {
  g_err.clear();
  if (!valid_dtype(dtype)) return fail(MO_ERR_UNSUPPORTED, "dtype must be MO_F32 or MO_BF16");
  if (numel < 1) return fail(MO_ERR_INVALID, "numel must be >= 1");
  if (M < 1 || M > 65535) return fail(MO_ERR_INVALID, "M must be in [1, 65535]");
  if (M > 1 && u_stride < numel) return fail(MO_ERR_INVALID, "u_stride must be >= numel when M > 1");
  if (!u || !packed) return fail(MO_ERR_INVALID, "u or packed is NULL");
  // a block covers 4 waves x PACK_LOADS loads x 64 lanes x 16 bytes
  const int64_t per_block = 256 * PACK_LOADS * (16 / dtype_size(dtype));
  const int64_t blocks = (numel + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return fail(MO_ERR_INVALID, "numel too large");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  // 16-byte loads when every worker's values start 16-byte aligned
  const int64_t stride = M > 1 ? u_stride : 0;
  const int vec = (aligned16(u) && (static_cast<uint64_t>(stride) * dtype_size(dtype)) % 16 == 0) ? 1 : 0;
  return launch(PK_PACK, stream, [&] {
    if (dtype == MO_F32)
      hipLaunchKernelGGL((k_sign_pack<float>), dim3(blocks, M), dim3(256), 0, stream, static_cast<const float*>(u),
                         stride, numel, packed, vec);
    else
      hipLaunchKernelGGL((k_sign_pack<bf16_t>), dim3(blocks, M), dim3(256), 0, stream,
                         static_cast<const bf16_t*>(u), stride, numel, packed, vec);
  });
}

int32_t sign_pack(const void* u, int32_t dtype, int64_t numel, uint32_t* packed, void* stream_ptr) {
  return sign_pack_batched(u, dtype, 1, numel, numel, packed, stream_ptr);
}

int32_t sign_vote(const uint32_t* packed, int32_t M, int64_t numel, uint32_t* out_packed, int8_t* out_sum,
                  void* stream_ptr) {
  g_err.clear();
  if (M < 1 || M > 65535) return fail(MO_ERR_INVALID, "M must be in [1, 65535]");
  if (out_sum && M > 127) return fail(MO_ERR_INVALID, "int8 sums need M <= 127");
  if (numel < 1) return fail(MO_ERR_INVALID, "numel must be >= 1");
  if (!packed || !out_packed) return fail(MO_ERR_INVALID, "packed or out_packed is NULL");
  const int64_t nwords = (numel + 31) / 32;
  // groups of four words with 16-byte loads when every worker's row starts 16-byte
  // aligned (nwords % 4 == 0 and an aligned base); two groups per thread when that
  // still leaves at least 8 blocks of 512 groups per CU (2^20 groups)
  int quad = (nwords % 4 == 0 && aligned16(packed)) ? 1 : 0;
  if (quad && nwords / 4 >= VOTE_PAIR_GROUPS) quad = 2;
  const int64_t per_block = quad == 2 ? 512 : 256;   // groups or words
  const int64_t blocks = ((quad ? nwords / 4 : nwords) + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return fail(MO_ERR_INVALID, "numel too large");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  // the counter needs 2^LV > M: 4 bit planes up to 15 workers, 8 up to 255, else 16
  return launch(PK_VOTE, stream, [&] {
#define MO_VOTE(LV, SUMS)                                                                          \
  hipLaunchKernelGGL((k_sign_vote<LV, SUMS>), dim3(blocks), dim3(256), 0, stream, packed, M, numel, nwords, \
                     out_packed, out_sum, quad)
    if (out_sum) {
      if (M <= 15) MO_VOTE(4, true); else MO_VOTE(8, true);   // sums need M <= 127
    } else if (M <= 15) {
      MO_VOTE(4, false);
    } else if (M <= 255) {
      MO_VOTE(8, false);
    } else {
      MO_VOTE(16, false);
    }
#undef MO_VOTE
  });
}

int32_t sign_unpack(const uint32_t* packed, int64_t numel, int32_t dtype, void* out, void* stream_ptr) {
  g_err.clear();
  if (!valid_dtype(dtype)) return fail(MO_ERR_UNSUPPORTED, "dtype must be MO_F32 or MO_BF16");
  if (numel < 1) return fail(MO_ERR_INVALID, "numel must be >= 1");
  if (!packed || !out) return fail(MO_ERR_INVALID, "packed or out is NULL");
  const int64_t per_block = 256 * UNPACK_PIECES * (16 / dtype_size(dtype));
  const int64_t blocks = (numel + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return fail(MO_ERR_INVALID, "numel too large");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int vec = aligned16(out) ? 1 : 0;
  return launch(PK_UNPACK, stream, [&] {
    if (dtype == MO_F32)
      hipLaunchKernelGGL((k_sign_unpack<float>), dim3(blocks), dim3(256), 0, stream, packed, numel,
                         static_cast<float*>(out), vec);
    else
      hipLaunchKernelGGL((k_sign_unpack<bf16_t>), dim3(blocks), dim3(256), 0, stream, packed, numel,
                         static_cast<bf16_t*>(out), vec);
  });
}

int32_t sign_apply(const uint32_t* packed, int64_t numel, int32_t dtype, void* weight, float lr,
                   void* stream_ptr) {
  g_err.clear();
  if (!valid_dtype(dtype)) return fail(MO_ERR_UNSUPPORTED, "dtype must be MO_F32 or MO_BF16");
  if (numel < 1) return fail(MO_ERR_INVALID, "numel must be >= 1");
  if (!packed || !weight) return fail(MO_ERR_INVALID, "packed or weight is NULL");
  if (!std::isfinite(lr)) return fail(MO_ERR_INVALID, "lr must be finite");
  const int64_t per_block = 256 * SAPPLY_PIECES * (16 / dtype_size(dtype));
  const int64_t blocks = (numel + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return fail(MO_ERR_INVALID, "numel too large");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int vec = aligned16(weight) ? 1 : 0;
  return launch(PK_SAPPLY, stream, [&] {
    if (dtype == MO_F32)
      hipLaunchKernelGGL((k_sign_apply<float>), dim3(blocks), dim3(256), 0, stream, packed, numel,
                         static_cast<float*>(weight), lr, vec);
    else
      hipLaunchKernelGGL((k_sign_apply<bf16_t>), dim3(blocks), dim3(256), 0, stream, packed, numel,
                         static_cast<bf16_t*>(weight), lr, vec);
  });
}

int32_t mo_plan_owners(const int64_t* rows, const int64_t* cols, int32_t count, int32_t ranks, int32_t iters,
                       double bytes_per_element, int32_t* owner, double* rank_work, double* rank_bytes) {
  g_err.clear();
  if (count < 0 || ranks < 1) return fail(MO_ERR_INVALID, "count must be >= 0 and ranks >= 1");
  if (iters < 0) return fail(MO_ERR_INVALID, "iters must be >= 0");
  if (!std::isfinite(bytes_per_element) || bytes_per_element < 0.0)
    return fail(MO_ERR_INVALID, "bytes_per_element must be finite and >= 0");
  if (count > 0 && (!rows || !cols || !owner)) return fail(MO_ERR_INVALID, "rows, cols or owner is NULL");
  for (int i = 0; i < count; ++i)
    if (rows[i] < 1 || cols[i] < 1 || rows[i] > MAX_DIM || cols[i] > MAX_DIM)
      return fail(MO_ERR_INVALID, "matrix " + std::to_string(i) + ": rows and cols must be in [1, 2^24]");
  plan_owners(rows, cols, count, ranks, iters, bytes_per_element, owner, rank_work, rank_bytes);
  return MO_OK;
}

const char* mo_last_error(void) { return g_err.c_str(); }

int32_t mo_version(void) { return MATOPT_VERSION; }

int32_t mo_profile_begin(void) {
  g_prof = true;
  return MO_OK;
}

int32_t mo_profile_end(mo_kernel_time* out, int32_t max) {
  g_err.clear();
  g_prof = false;
  std::lock_guard<std::mutex> lock(g_prof_mu);
  double ms[PK_N] = {0};
  int64_t n[PK_N] = {0};
  // each launch as [start, end) in ms after the first record's start event, for
  // the union per kind; `one_timeline` turns false if an offset cannot be taken
  // (events of another device)
  std::vector<std::pair<double, double>> iv[PK_N];
  bool one_timeline = true;
  int rc = MO_OK;
  const hipEvent_t ref = g_prof_recs.empty() ? nullptr : g_prof_recs.front().e0;
  for (const ProfRec& r : g_prof_recs) {
    float t = 0.f, off = 0.f;
    if (hipEventSynchronize(r.e1) != hipSuccess || hipEventElapsedTime(&t, r.e0, r.e1) != hipSuccess)
      rc = fail(MO_ERR_HIP, "event timing failed");
    if (one_timeline && hipEventElapsedTime(&off, ref, r.e0) != hipSuccess) {
      one_timeline = false;
      (void)hipGetLastError();
    }
    ms[r.kind] += t;
    n[r.kind] += 1;
    iv[r.kind].emplace_back(off, off + t);
  }
  for (const ProfRec& r : g_prof_recs) {
    g_ev_pool.push_back(r.e0);
    g_ev_pool.push_back(r.e1);
  }
  g_prof_recs.clear();
  if (rc != MO_OK) return rc;
  int k = 0;
  for (int i = 0; i < PK_N; ++i) {
    if (!n[i]) continue;
    double busy = ms[i];
    if (one_timeline) {
      std::sort(iv[i].begin(), iv[i].end());
      busy = 0.0;
      double s0 = iv[i].front().first, e0 = iv[i].front().second;
      for (const auto& x : iv[i]) {
        if (x.first > e0) {
          busy += e0 - s0;
          s0 = x.first;
          e0 = x.second;
        } else if (x.second > e0) {
          e0 = x.second;
        }
      }
      busy += e0 - s0;
    }
    if (out && k < max) {
      std::memset(&out[k], 0, sizeof(mo_kernel_time));
      std::strncpy(out[k].name, kKindNames[i], sizeof(out[k].name) - 1);
      out[k].launches = n[i];
      out[k].total_ms = ms[i];
      out[k].busy_ms = busy;
    }
    ++k;
  }
  return k;
}

}  // extern "C"
