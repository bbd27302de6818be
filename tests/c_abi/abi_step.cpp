// Calls libmatopt through its C ABI alone, with no Python and no torch: the HIP
// runtime for device memory, one batched Muon step on three matrices that take both
// product paths (fp32 gradients, momentum, compute and output), a 1-bit pack of one
// result, an argument error, and the version.  Inputs come from a counter-based
// generator (splitmix64); inputs and results are written as raw little-endian arrays
// to the directory given, where the test compares them with the fp64 oracle.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "matopt.h"

#define CK(x)                                                                    \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      return 2;                                                                  \
    }                                                                            \
  } while (0)

namespace {

// splitmix64, mapped to [-1, 1) with 24 significant bits
uint64_t g_state = 0;
float next_uniform() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return static_cast<float>(static_cast<double>(z >> 40) / 16777216.0 * 2.0 - 1.0);
}

bool write_file(const std::string& path, const void* p, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const bool ok = std::fwrite(p, 1, bytes, f) == bytes;
  return std::fclose(f) == 0 && ok;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s OUT_DIR\n", argv[0]);
    return 1;
  }
  const std::string dir = argv[1];
  const int64_t shapes[3][2] = {{300, 200}, {512, 768}, {768, 512}};
  mo_matrix mats[3];
  std::vector<float> g[3], m[3];
  for (int i = 0; i < 3; ++i) {
    const int64_t n = shapes[i][0] * shapes[i][1];
    g[i].resize(n);
    m[i].resize(n);
    for (int64_t e = 0; e < n; ++e) g[i][e] = 0.02f * next_uniform();
    for (int64_t e = 0; e < n; ++e) m[i][e] = 0.02f * next_uniform();
    float *dg = nullptr, *dm = nullptr, *du = nullptr;
    CK(hipMalloc(&dg, n * sizeof(float)));
    CK(hipMalloc(&dm, n * sizeof(float)));
    CK(hipMalloc(&du, n * sizeof(float)));
    CK(hipMemcpy(dg, g[i].data(), n * sizeof(float), hipMemcpyHostToDevice));
    CK(hipMemcpy(dm, m[i].data(), n * sizeof(float), hipMemcpyHostToDevice));
    mats[i] = mo_matrix{shapes[i][0], shapes[i][1], dg, dm, nullptr, du};
    const std::string k = std::to_string(i);
    if (!write_file(dir + "/g" + k + ".f32", g[i].data(), n * sizeof(float)) ||
        !write_file(dir + "/m" + k + ".f32", m[i].data(), n * sizeof(float))) {
      std::fprintf(stderr, "cannot write to %s\n", dir.c_str());
      return 1;
    }
  }
  const mo_ns_params ns = {3.4445f, -4.775f, 2.0315f, 5, 1e-7f};
  const size_t bytes = muon_workspace_bytes(mats, 3, MO_F32);
  if (bytes == 0) {
    std::fprintf(stderr, "muon_workspace_bytes: %s\n", mo_last_error());
    return 3;
  }
  void* ws = nullptr;
  CK(hipMalloc(&ws, bytes));
  int32_t rc = muon_step_batched(mats, 3, MO_F32, MO_F32, MO_F32, 0.95f, &ns, ws, bytes, nullptr);
  if (rc != MO_OK) {
    std::fprintf(stderr, "muon_step_batched: %d %s\n", rc, mo_last_error());
    return 3;
  }
  // the signs of the second matrix's result, 32 per word
  const int64_t n1 = shapes[1][0] * shapes[1][1];
  uint32_t* packed = nullptr;
  CK(hipMalloc(&packed, ((n1 + 31) / 32) * sizeof(uint32_t)));
  rc = sign_pack(mats[1].out, MO_F32, n1, packed, nullptr);
  if (rc != MO_OK) {
    std::fprintf(stderr, "sign_pack: %d %s\n", rc, mo_last_error());
    return 3;
  }
  CK(hipDeviceSynchronize());
  for (int i = 0; i < 3; ++i) {
    const int64_t n = shapes[i][0] * shapes[i][1];
    std::vector<float> mn(n), u(n);
    CK(hipMemcpy(mn.data(), mats[i].momentum, n * sizeof(float), hipMemcpyDeviceToHost));
    CK(hipMemcpy(u.data(), mats[i].out, n * sizeof(float), hipMemcpyDeviceToHost));
    const std::string k = std::to_string(i);
    if (!write_file(dir + "/mnew" + k + ".f32", mn.data(), n * sizeof(float)) ||
        !write_file(dir + "/u" + k + ".f32", u.data(), n * sizeof(float)))
      return 1;
  }
  std::vector<uint32_t> words((n1 + 31) / 32);
  CK(hipMemcpy(words.data(), packed, words.size() * sizeof(uint32_t), hipMemcpyDeviceToHost));
  if (!write_file(dir + "/packed1.u32", words.data(), words.size() * sizeof(uint32_t))) return 1;
  // an argument error is caught on the host, before any launch, with a message
  rc = muon_step_batched(mats, -1, MO_F32, MO_F32, MO_F32, 0.95f, &ns, ws, bytes, nullptr);
  if (rc != MO_ERR_INVALID || mo_last_error()[0] == '\0') {
    std::fprintf(stderr, "negative count: expected MO_ERR_INVALID with a message, got %d\n", rc);
    return 4;
  }
  if (mo_version() != MATOPT_VERSION) {
    std::fprintf(stderr, "version %d, header %d\n", mo_version(), MATOPT_VERSION);
    return 5;
  }
  for (int i = 0; i < 3; ++i) {
    CK(hipFree(const_cast<void*>(mats[i].grad)));
    CK(hipFree(mats[i].momentum));
    CK(hipFree(mats[i].out));
  }
  CK(hipFree(packed));
  CK(hipFree(ws));
  std::printf("abi_step: ok (workspace %zu bytes)\n", bytes);
  return 0;
}
