// Host-side check of the library's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only: the device code is the
// library's own, unsanitized).  Built by sketch_attention_amd/build.py with the
// library's host translation units instrumented; test infrastructure, not
// part of the library.
//
//   sa_host_check validate   argument validation, status strings, planner
//                            queries: no device work (runs without a GPU)
//   sa_host_check full       also create / compute / destroy through every
//                            entry point on device 0 over ragged batches
//                            (empty users, more users than one launch,
//                            two-phase prototype counts), checking statuses and
//                            the mass identity sum_j X~_j = sum_i x_i
//
// Exit status 0 when every check holds; a sanitizer report aborts the run.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "sa.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAIL line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// deterministic values in [-1, 1) (a 64-bit linear congruential sequence)
struct Lcg {
  uint64_t s;
  float next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((s >> 40) & 0xffffff) / 8388608.0f - 1.0f;
  }
};

uint16_t to_bf16(float x) {  // round to nearest even (finite inputs)
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

void validate() {
  for (int s = 0; s <= 5; ++s) EXPECT(sa_status_string((sa_status)s) != nullptr);
  const int ds[] = {0, 1, 64, 96, 128, 256};
  const int ks[] = {-1, 0, 1, 256, 512, 513, 1024, 1025};
  const float taus[] = {0.1f, 0.f, -3.f, NAN, INFINITY};
  for (int d : ds)
    for (int k : ks)
      for (float tau : taus)
        for (int dt = 0; dt < 2; ++dt) {
          const sa_status a = sa_check_config(d, k, tau, (sa_dtype)dt);
          const sa_status g = sa_grad_check_config(d, k, tau, (sa_dtype)dt);
          EXPECT(a >= SA_OK && a <= SA_ERR_DEVICE);
          EXPECT(g >= SA_OK && g <= SA_ERR_DEVICE);
          if (a != SA_OK) EXPECT(g != SA_OK);
        }
  EXPECT(sa_check_config(128, 1024, 0.1f, SA_BF16) == SA_OK);
  EXPECT(sa_check_config(128, 1025, 0.1f, SA_BF16) == SA_ERR_UNSUPPORTED);
  const int64_t good[] = {0, 5, 5, 900};
  const int64_t back[] = {0, 5, 4, 900};
  const int64_t neg[] = {-1, 5};
  EXPECT(sa_check_batch(64, good, 3) == SA_OK);
  EXPECT(sa_check_batch(64, back, 3) == SA_ERR_INVALID_ARG);
  EXPECT(sa_check_batch(64, neg, 1) == SA_ERR_INVALID_ARG);
  EXPECT(sa_check_batch(64, nullptr, 2) == SA_ERR_INVALID_ARG);
  EXPECT(sa_check_batch(64, nullptr, 0) == SA_OK);
  EXPECT(sa_check_batch(64, good, -1) == SA_ERR_INVALID_ARG);
  for (int d : {32, 64, 128})
    for (int da : {0, 16, 64, 200})
      for (int dff : {0, 32, 64, 256, 1000})
        for (int na : {0, 1, 8})
          EXPECT(sa_action_check_config(d, da, dff, na, SA_BF16) <= SA_ERR_DEVICE);
  // null handles and null outputs are refused before any device work
  EXPECT(sa_compress_batch(nullptr, nullptr, good, 3, nullptr, nullptr) == SA_ERR_INVALID_ARG);
  EXPECT(sa_compress_batch_noalloc(nullptr, nullptr, good, 3, nullptr, nullptr) == SA_ERR_INVALID_ARG);
  EXPECT(sa_describe_plan(nullptr, 10, nullptr, nullptr, nullptr, nullptr, nullptr) == SA_ERR_INVALID_ARG);
  EXPECT(sa_create(nullptr, 128, 64, 0.1f, SA_BF16, nullptr, nullptr, nullptr, nullptr) == SA_ERR_INVALID_ARG);
  sa_handle h = reinterpret_cast<sa_handle>(1);
  EXPECT(sa_create(&h, 128, 64, 0.1f, SA_BF16, nullptr, nullptr, nullptr, nullptr) == SA_ERR_INVALID_ARG);
  EXPECT(h == nullptr);
  sa_destroy(nullptr);
  sa_stack_destroy(nullptr);
  sa_grad_destroy(nullptr);
  sa_action_destroy(nullptr);
}

template <typename T>
T* dev_copy(const std::vector<T>& v) {
  void* p = nullptr;
  if (hipMalloc(&p, v.size() * sizeof(T) + 16) != hipSuccess) return nullptr;
  if (!v.empty() && hipMemcpy(p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
  return static_cast<T*>(p);
}

std::vector<uint16_t> bf16_values(size_t n, Lcg& g, float scale) {
  std::vector<uint16_t> v(n);
  for (auto& x : v) x = to_bf16(scale * g.next());
  return v;
}

// sum over prototypes of each user's sketch against the sum of its rows
void mass_identity(const std::vector<uint16_t>& X, const std::vector<int64_t>& off, const std::vector<float>& out, int k,
                   int d) {
  const int users = (int)off.size() - 1;
  for (int u = 0; u < users; ++u) {
    double worst = 0.0, scale = 1e-30;
    for (int c = 0; c < d; ++c) {
      double want = 0.0, have = 0.0;
      for (int64_t i = off[u]; i < off[u + 1]; ++i) want += from_bf16(X[i * d + c]);
      for (int j = 0; j < k; ++j) have += out[((size_t)u * k + j) * d + c];
      worst = std::fmax(worst, std::fabs(have - want));
      scale = std::fmax(scale, std::fabs(want));
    }
    const double rows = (double)(off[u + 1] - off[u]);
    EXPECT(worst <= 2e-2 * std::fmax(scale, std::sqrt(rows + 1.0)));
  }
}

void full() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    std::fprintf(stderr, "full: no device\n");
    ++failures;
    return;
  }
  Lcg g{12345};
  struct Case {
    int d, k;
    std::vector<int64_t> lengths;
  };
  const Case cases[] = {{128, 256, {700, 0, 1, 4100, 63, 64, 65}},
                        {64, 1024, {3000, 0, 17}},
                        {128, 1000, {2500, 1, 0, 640}},
                        {128, 64, std::vector<int64_t>(300, 37)}};  // more users than one launch carries
  for (const Case& c : cases) {
    std::vector<int64_t> off(1, 0);
    for (int64_t len : c.lengths) off.push_back(off.back() + len);
    const int users = (int)c.lengths.size();
    const int64_t rows = off.back();
    const float tau = 1.0f / std::sqrt((float)c.d);
    auto P = bf16_values((size_t)c.k * c.d, g, 1.0f), WQ = bf16_values((size_t)c.d * c.d, g, 0.2f),
         WK = bf16_values((size_t)c.d * c.d, g, 0.2f), X = bf16_values((size_t)rows * c.d, g, 1.0f);
    uint16_t *dP = dev_copy(P), *dWQ = dev_copy(WQ), *dWK = dev_copy(WK), *dX = dev_copy(X);
    float* dout = nullptr;
    EXPECT(dP && dWQ && dWK && dX && hipMalloc((void**)&dout, (size_t)users * c.k * c.d * 4) == hipSuccess);
    sa_handle h = nullptr;
    EXPECT(sa_create(&h, c.d, c.k, tau, SA_BF16, dP, dWQ, dWK, nullptr) == SA_OK);
    if (h) {
      int32_t groups = 0, wk = 0, wr = 0, tr = 0, kp = 0;
      EXPECT(sa_describe_plan(h, rows, &groups, &wk, &wr, &tr, &kp) == SA_OK);
      EXPECT(groups >= 1 && kp >= c.k);
      for (int rep = 0; rep < 2; ++rep) {
        const bool noalloc = rep == 1;
        const sa_status st = noalloc ? sa_compress_batch_noalloc(h, dX, off.data(), users, dout, nullptr)
                                     : sa_compress_batch(h, dX, off.data(), users, dout, nullptr);
        EXPECT(st == SA_OK);
        EXPECT(hipDeviceSynchronize() == hipSuccess);
        std::vector<float> out((size_t)users * c.k * c.d);
        EXPECT(hipMemcpy(out.data(), dout, out.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
        mass_identity(X, off, out, c.k, c.d);
      }
      sa_destroy(h);
    }
    if (c.k >= 256) {  // backward over the same batch
      sa_grad gh = nullptr;
      EXPECT(sa_grad_create(&gh, c.d, c.k, tau, SA_BF16, dP, dWQ, dWK, nullptr) == SA_OK);
      std::vector<float> G((size_t)users * c.k * c.d);
      for (auto& x : G) x = g.next();
      float* dG = dev_copy(G);
      void* dgX = nullptr;
      float *dgP = nullptr, *dgQ = nullptr, *dgK = nullptr;
      EXPECT(dG && hipMalloc(&dgX, (size_t)rows * c.d * 2 + 16) == hipSuccess &&
             hipMalloc((void**)&dgP, (size_t)c.k * c.d * 4) == hipSuccess &&
             hipMalloc((void**)&dgQ, (size_t)c.d * c.d * 4) == hipSuccess &&
             hipMalloc((void**)&dgK, (size_t)c.d * c.d * 4) == hipSuccess);
      if (gh) {
        EXPECT(sa_grad_compute(gh, dX, off.data(), users, dG, dgX, dgP, dgQ, dgK, nullptr) == SA_OK);
        EXPECT(hipDeviceSynchronize() == hipSuccess);
        std::vector<float> gp((size_t)c.k * c.d);
        EXPECT(hipMemcpy(gp.data(), dgP, gp.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
        for (float v : gp) EXPECT(std::isfinite(v));
        sa_grad_destroy(gh);
      }
      for (void* p : {(void*)dG, dgX, (void*)dgP, (void*)dgQ, (void*)dgK}) (void)hipFree(p);
    }
    for (void* p : {(void*)dP, (void*)dWQ, (void*)dWK, (void*)dX, (void*)dout}) (void)hipFree(p);
  }
}

// float32 paths: the comparator (each sketch row a convex combination of the user's rows, so bounded by
// their largest magnitude), the backward (finite weight gradients) and the action fusion (finite rows)
void full_f32() {
  Lcg g{777};
  const int d = 64, k = 300, d_a = 8, d_ff = 64, n_actions = 5;
  const std::vector<int64_t> lengths = {900, 0, 1, 70000};
  std::vector<int64_t> off(1, 0);
  for (int64_t len : lengths) off.push_back(off.back() + len);
  const int users = (int)lengths.size();
  const int64_t rows = off.back();
  auto vals = [&](size_t n, float scale) {
    std::vector<float> v(n);
    for (auto& x : v) x = scale * g.next();
    return v;
  };
  auto P = vals((size_t)k * d, 1.0f), WQ = vals((size_t)d * d, 0.2f), WK = vals((size_t)d * d, 0.2f),
       X = vals((size_t)rows * d, 1.0f), G = vals((size_t)users * k * d, 1.0f);
  float *dP = dev_copy(P), *dWQ = dev_copy(WQ), *dWK = dev_copy(WK), *dX = dev_copy(X), *dG = dev_copy(G);
  float *dout = nullptr, *dgX = nullptr, *dgP = nullptr, *dgQ = nullptr, *dgK = nullptr;
  EXPECT(dP && dWQ && dWK && dX && dG && hipMalloc((void**)&dout, (size_t)users * k * d * 4) == hipSuccess &&
         hipMalloc((void**)&dgX, (size_t)rows * d * 4 + 16) == hipSuccess &&
         hipMalloc((void**)&dgP, (size_t)k * d * 4) == hipSuccess &&
         hipMalloc((void**)&dgQ, (size_t)d * d * 4) == hipSuccess && hipMalloc((void**)&dgK, (size_t)d * d * 4) == hipSuccess);
  const float tau = 0.125f;
  sa_handle h = nullptr;
  EXPECT(sa_create_ex(&h, d, k, tau, SA_F32, dP, dWQ, dWK, SA_NORM_HISTORY, nullptr) == SA_OK);
  if (h) {
    EXPECT(sa_compress_batch(h, dX, off.data(), users, dout, nullptr) == SA_OK);
    EXPECT(hipDeviceSynchronize() == hipSuccess);
    std::vector<float> out((size_t)users * k * d);
    EXPECT(hipMemcpy(out.data(), dout, out.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
    for (int u = 0; u < users; ++u) {
      float bound = 0.f;
      for (int64_t i = off[u] * d; i < off[u + 1] * d; ++i) bound = std::fmax(bound, std::fabs(X[i]));
      for (size_t i = (size_t)u * k * d; i < (size_t)(u + 1) * k * d; ++i) EXPECT(std::fabs(out[i]) <= bound * 1.0001f);
    }
    sa_destroy(h);
  }
  sa_grad gh = nullptr;
  EXPECT(sa_grad_create(&gh, d, k, tau, SA_F32, dP, dWQ, dWK, nullptr) == SA_OK);
  if (gh) {
    for (int rep = 0; rep < 2; ++rep) {
      EXPECT(sa_grad_compute(gh, dX, off.data(), users, dG, dgX, dgP, dgQ, dgK, nullptr) == SA_OK);
      EXPECT(hipDeviceSynchronize() == hipSuccess);
    }
    std::vector<float> gk((size_t)d * d);
    EXPECT(hipMemcpy(gk.data(), dgK, gk.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
    for (float v : gk) EXPECT(std::isfinite(v));
    sa_grad_destroy(gh);
  }
  auto table = vals((size_t)n_actions * d_a, 1.0f), Wg = vals((size_t)(d + d_a) * d_ff, 0.1f),
       Wu = vals((size_t)(d + d_a) * d_ff, 0.1f), Wd = vals((size_t)d_ff * d, 0.1f);
  std::vector<int32_t> acts((size_t)rows);
  for (int64_t i = 0; i < rows; ++i) acts[i] = (int32_t)(i % (n_actions + 2)) - 1;  // some out of range: clamped
  float *dT = dev_copy(table), *dWg = dev_copy(Wg), *dWu = dev_copy(Wu), *dWd = dev_copy(Wd);
  int32_t* dA = dev_copy(acts);
  sa_action ah = nullptr;
  EXPECT(dT && dWg && dWu && dWd && dA &&
         sa_action_create(&ah, d, d_a, d_ff, n_actions, SA_F32, dT, dWg, dWu, dWd, nullptr) == SA_OK);
  if (ah) {
    EXPECT(sa_action_fuse(ah, dX, dA, rows, dgX, nullptr) == SA_OK);
    EXPECT(hipDeviceSynchronize() == hipSuccess);
    std::vector<float> xr((size_t)rows * d);
    EXPECT(hipMemcpy(xr.data(), dgX, xr.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
    for (float v : xr) EXPECT(std::isfinite(v));
    sa_action_destroy(ah);
  }
  for (void* p : {(void*)dP, (void*)dWQ, (void*)dWK, (void*)dX, (void*)dG, (void*)dout, (void*)dgX, (void*)dgP,
                  (void*)dgQ, (void*)dgK, (void*)dT, (void*)dWg, (void*)dWu, (void*)dWd, (void*)dA})
    (void)hipFree(p);
}

}  // namespace

int main(int argc, char** argv) {
  const bool run_full = argc > 1 && std::strcmp(argv[1], "full") == 0;
  validate();
  if (run_full) {
    full();
    full_f32();
  }
  std::printf("sa_host_check %s: %d failure(s)\n", run_full ? "full" : "validate", failures);
  std::fflush(stdout);
  std::fflush(stderr);
  // Every check has run.  The HIP runtime's own teardown after main returns
  // frees device memory through the sanitizer's device allocator after that
  // allocator has shut down, which aborts now and then inside the runtime
  // (not in this program); ending here skips that teardown.
  std::_Exit(failures == 0 ? 0 : 1);
}
