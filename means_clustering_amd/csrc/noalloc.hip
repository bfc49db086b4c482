// kmeans_fit without a caller workspace and without any allocation, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch space that kmeans_fit takes from its `ws` argument lives here
// in a file-scope device array of fixed size instead.  Every GPU the library
// runs on holds its own copy of the array (from module load until the
// process ends); its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address (never the
// array's host-side name) is what the kernels receive.  All calls on one GPU
// share the array, so calls that overlap on one GPU (different streams, or
// different host threads) race on it; calls ordered on one stream do not.
// kmeans_fit reads no scratch value it has not written in the same call, so
// nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/kmeans.h"

namespace km {
km_status fit_args_check(const void* X, km_dtype dt, int64_t N, int64_t D, int64_t K, const float* C, int32_t iters,
                         const int32_t* assign, const int32_t* counts, const double* objective);
km_status fail_with(km_status s, const char* msg);
}  // namespace km

static __device__ __align__(256) unsigned char scratch[KMEANS_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device ordinal; nullptr until looked up

// The device address of this device's copy of `scratch` (looked up on first use with `dev` current).
hipError_t scratch_of(int dev, void** out) {
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[(size_t)dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p) % 256 != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[(size_t)dev] = p;
  }
  *out = g_scratch_ptr[(size_t)dev];
  return hipSuccess;
}
}  // namespace

extern "C" km_status kmeans_fit_noalloc(const void* X, km_dtype dt, int64_t N, int64_t D, int64_t K, float* C,
                                        int32_t iters, int32_t* assign, int32_t* counts, double* objective,
                                        void* stream) {
  km_status st = km::fit_args_check(X, dt, N, D, K, C, iters, assign, counts, objective);
  if (st != KM_OK) return st;
  const size_t need = kmeans_workspace_bytes(KM_OP_FIT, N, D, K, dt, 0);
  if (need > (size_t)KMEANS_NOALLOC_SCRATCH_BYTES)
    return km::fail_with(KM_ERR_UNSUPPORTED,
                         ("kmeans_fit_noalloc: this shape needs " + std::to_string(need) +
                          " bytes of scratch, more than the fixed " + std::to_string(KMEANS_NOALLOC_SCRATCH_BYTES) +
                          " (use kmeans_fit with a workspace)").c_str());
  if (iters == 0) return KM_OK;
  int cur = 0, sdev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) e = hipStreamGetDevice((hipStream_t)stream, &sdev);
  if (e != hipSuccess) return km::fail_with(KM_ERR_HIP, (std::string("kmeans_fit_noalloc: ") + hipGetErrorString(e)).c_str());
  if (sdev != cur)
    return km::fail_with(KM_ERR_INVALID_VALUE, "kmeans_fit_noalloc: the stream must belong to the current device");
  void* ws = nullptr;
  e = scratch_of(cur, &ws);
  if (e != hipSuccess)
    return km::fail_with(KM_ERR_HIP, (std::string("kmeans_fit_noalloc: scratch lookup: ") + hipGetErrorString(e)).c_str());
  return kmeans_fit(X, dt, N, D, K, C, iters, assign, counts, objective, ws, (size_t)KMEANS_NOALLOC_SCRATCH_BYTES,
                    stream);
}
