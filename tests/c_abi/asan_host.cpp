// Host-side paths of the C ABI under AddressSanitizer: argument validation of every
// entry point, workspace sizing over many shape lists, the owner planner, error
// messages and the profiling calls.  Only calls that the library rejects on the host
// (or that need no device) are made, so the program needs no GPU; it is linked
// against a build of libmatopt.so whose host code carries the sanitizer.  Exit status
// 0 when every check holds (the sanitizer itself aborts on a memory error).

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "matopt.h"

static int failures = 0;

static void check(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL: %s (last error: %s)\n", what, mo_last_error());
    ++failures;
  }
}

static mo_matrix mat(int64_t r, int64_t c, uintptr_t g = 0x1000, uintptr_t m = 0x2000, uintptr_t o = 0x3000) {
  mo_matrix x;
  std::memset(&x, 0, sizeof x);
  x.rows = r;
  x.cols = c;
  x.grad = reinterpret_cast<const void*>(g);
  x.momentum = reinterpret_cast<float*>(m);
  x.out = reinterpret_cast<void*>(o);
  return x;
}

int main() {
  check(mo_version() == MATOPT_VERSION, "mo_version");
  void* fake = reinterpret_cast<void*>(0x1000);
  const mo_ns_params ns = {3.4445f, -4.775f, 2.0315f, 5, 1e-7f};

  // workspace sizing: many lists, both compute dtypes, some invalid
  unsigned seed = 12345;
  auto rnd = [&](int lo, int hi) {
    seed = seed * 1103515245u + 12345u;
    return lo + static_cast<int>((seed >> 8) % static_cast<unsigned>(hi - lo + 1));
  };
  for (int trial = 0; trial < 200; ++trial) {
    const int count = rnd(1, 40);
    std::vector<mo_matrix> list;
    for (int i = 0; i < count; ++i) list.push_back(mat(rnd(1, 5000), rnd(1, 5000)));
    const size_t bf = muon_workspace_bytes(list.data(), count, MO_BF16);
    const size_t f32 = muon_workspace_bytes(list.data(), count, MO_F32);
    check(bf > 0 && f32 > bf, "workspace sizing of a valid list");
  }
  {
    mo_matrix bad[2] = {mat(4, 4), mat(0, 5)};
    check(muon_workspace_bytes(bad, 2, MO_BF16) == 0 && std::strstr(mo_last_error(), "rows and cols"),
          "zero-sized matrix rejected");
    mo_matrix huge = mat(32768, 32768);
    check(muon_workspace_bytes(&huge, 1, MO_BF16) == 0 && std::strstr(mo_last_error(), "2 GiB"),
          "operand beyond 2 GiB rejected");
    check(muon_workspace_bytes(nullptr, 3, MO_BF16) == 0, "null list rejected");
    check(muon_workspace_bytes(bad, 1, 9) == 0, "unsupported compute dtype rejected");
  }

  // the step entry points: each of these fails on the host, before any HIP call
  {
    mo_matrix m = mat(4, 4);
    const mo_ns_params neg = {1.f, 1.f, 1.f, -1, 1e-7f};
    check(muon_step_batched(&m, 1, MO_BF16, MO_BF16, MO_BF16, 0.9f, &neg, fake, 1 << 20, nullptr) == MO_ERR_INVALID,
          "negative iteration count");
    check(muon_step_batched(&m, 1, 7, MO_BF16, MO_BF16, 0.9f, &ns, fake, 1 << 20, nullptr) == MO_ERR_UNSUPPORTED,
          "unsupported gradient dtype");
    check(muon_step_batched(&m, 1, MO_BF16, MO_BF16, MO_BF16, 0.9f, &ns, fake, 16, nullptr) == MO_ERR_WORKSPACE,
          "workspace too small");
    check(muon_step_batched(&m, 1, MO_BF16, MO_BF16, MO_BF16, 0.9f, &ns, nullptr, 1 << 20, nullptr) ==
              MO_ERR_WORKSPACE,
          "missing workspace");
    check(muon_step_batched(&m, 1, MO_BF16, MO_BF16, MO_BF16, 0.9f, nullptr, fake, 1 << 20, nullptr) ==
              MO_ERR_INVALID,
          "missing Newton-Schulz parameters");
    check(muon_step_batched(&m, 0, MO_BF16, MO_BF16, MO_BF16, 0.9f, &ns, nullptr, 0, nullptr) == MO_OK,
          "empty list is a no-op");
    mo_matrix nograd = mat(4, 4, 0);
    check(muon_step_batched(&nograd, 1, MO_BF16, MO_BF16, MO_BF16, 0.9f, &ns, reinterpret_cast<void*>(0x100000),
                            1 << 20, nullptr) == MO_ERR_INVALID,
          "missing gradient pointer");
    const mo_ns_params nan = {NAN, 1.f, 1.f, 1, 1e-7f};
    mo_matrix xm = mat(4, 4);
    xm.x = reinterpret_cast<const void*>(0x100000);
    check(ns_orthogonalize(&xm, 1, MO_BF16, MO_BF16, MO_BF16, &nan, fake, 1 << 20, nullptr) == MO_ERR_INVALID,
          "non-finite coefficient");
    xm.out = const_cast<void*>(xm.x);
    check(ns_orthogonalize(&xm, 1, MO_BF16, MO_BF16, MO_F32, &ns, reinterpret_cast<void*>(0x200000), 1 << 20,
                           nullptr) == MO_ERR_INVALID,
          "in-place call with different dtypes");
    check(muon_step_apply(&m, 1, MO_BF16, MO_BF16, MO_BF16, 0.9f, &ns, INFINITY, fake, 1 << 20, nullptr) ==
              MO_ERR_INVALID,
          "non-finite learning rate");
    check(muon_step_apply(&m, 1, MO_BF16, MO_BF16, 5, 0.9f, &ns, 0.1f, fake, 1 << 20, nullptr) ==
              MO_ERR_UNSUPPORTED,
          "unsupported weight dtype");
    mo_matrix two[2] = {mat(4096, 4096), mat(4096, 4096)};
    check(muon_step_batched_noalloc(two, 2, MO_BF16, MO_BF16, MO_BF16, 0.9f, &ns, nullptr) == MO_ERR_WORKSPACE &&
              std::strstr(mo_last_error(), "allocation-free"),
          "allocation-free step beyond its scratch");
  }

  // the sign tail
  {
    check(sign_pack(fake, MO_BF16, 0, static_cast<uint32_t*>(fake), nullptr) == MO_ERR_INVALID, "sign_pack numel 0");
    check(sign_pack(fake, 5, 10, static_cast<uint32_t*>(fake), nullptr) == MO_ERR_UNSUPPORTED, "sign_pack dtype");
    check(sign_pack(nullptr, MO_BF16, 10, static_cast<uint32_t*>(fake), nullptr) == MO_ERR_INVALID,
          "sign_pack null input");
    check(sign_pack(fake, MO_BF16, int64_t(1) << 45, static_cast<uint32_t*>(fake), nullptr) == MO_ERR_INVALID,
          "sign_pack too large");
    uint32_t* out = reinterpret_cast<uint32_t*>(0x2000);
    check(sign_pack_batched(fake, MO_F32, 0, 64, 64, out, nullptr) == MO_ERR_INVALID, "sign_pack_batched M < 1");
    check(sign_pack_batched(fake, MO_F32, 2, 64, 63, out, nullptr) == MO_ERR_INVALID, "sign_pack_batched overlap");
    const uint32_t* pk = static_cast<const uint32_t*>(fake);
    check(sign_vote(pk, 0, 10, out, nullptr, nullptr) == MO_ERR_INVALID, "sign_vote M < 1");
    check(sign_vote(pk, 70000, 10, out, nullptr, nullptr) == MO_ERR_INVALID, "sign_vote M too large");
    check(sign_vote(pk, 128, 10, out, static_cast<int8_t*>(fake), nullptr) == MO_ERR_INVALID &&
              std::strstr(mo_last_error(), "M <= 127"),
          "sign_vote int8 sums need M <= 127");
    check(sign_unpack(pk, 10, 3, fake, nullptr) == MO_ERR_UNSUPPORTED, "sign_unpack dtype");
    check(sign_unpack(nullptr, 10, MO_BF16, fake, nullptr) == MO_ERR_INVALID, "sign_unpack null input");
    check(sign_apply(pk, 10, MO_BF16, nullptr, 0.1f, nullptr) == MO_ERR_INVALID, "sign_apply null weight");
    check(sign_apply(pk, 10, MO_BF16, fake, NAN, nullptr) == MO_ERR_INVALID, "sign_apply non-finite lr");
  }

  // the owner planner (host only): random sets, every owner in range, work adds up
  for (int trial = 0; trial < 100; ++trial) {
    const int count = rnd(1, 300), ranks = rnd(1, 64);
    std::vector<int64_t> rows(count), cols(count);
    for (int i = 0; i < count; ++i) {
      rows[i] = rnd(1, 12000);
      cols[i] = rnd(1, 12000);
    }
    std::vector<int32_t> owner(count, -1);
    std::vector<double> work(ranks), bytes(ranks);
    const int32_t rc = mo_plan_owners(rows.data(), cols.data(), count, ranks, 5, 4.0, owner.data(), work.data(),
                                      bytes.data());
    check(rc == MO_OK, "planner on a valid set");
    bool in_range = true;
    for (int i = 0; i < count; ++i) in_range = in_range && owner[i] >= 0 && owner[i] < ranks;
    check(in_range, "planner owners in range");
  }
  {
    int64_t r = 4, c = 4;
    int32_t o = 0;
    double w = 0, b = 0;
    check(mo_plan_owners(&r, &c, 1, 0, 5, 4.0, &o, &w, &b) != MO_OK, "planner with no ranks rejected");
    check(mo_plan_owners(nullptr, &c, 1, 2, 5, 4.0, &o, &w, &b) != MO_OK, "planner null rows rejected");
  }

  // profiling without launches
  check(mo_profile_begin() == MO_OK, "mo_profile_begin");
  check(mo_profile_end(nullptr, 0) == 0, "mo_profile_end with no launches");

  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
