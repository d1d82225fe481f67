// rmsnorm_matmul for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the same
// call, with the split-K workspace taken from a fixed device array that the
// library owns instead of from the caller.
//
// The array lives in this file's code object, one copy per GPU, for the
// life of the process.  In host code its name is only a stand-in: the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what
// the kernels receive.  The array is zero when the code object is loaded;
// every call leaves the arrival counters in its first 64 KiB at zero again
// (and overwrites its partial sums before reading them), so calls with any
// shapes can follow each other.  Calls that overlap on one GPU (two streams,
// or two threads) share the array and race.
#include <mutex>

#include "rmm.h"
#include "rmm_device.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the array (looked up on the first call per device).
hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

rmm_status rmsnorm_matmul_noalloc(const void* X, const void* g, const void* W, void* Y, float eps,
                                  int64_t M, int64_t N, int64_t K, rmm_dtype dtype,
                                  hipStream_t stream) {
  // Validation first (no HIP call), exactly as rmsnorm_matmul with a
  // workspace of the array's size would do it; the plan also says how much
  // of the array this call uses.
  const rmm_status st = rmm_plan(X, g, W, nullptr, Y, eps, M, N, K, dtype, 0, RMM_VARIANT_AUTO,
                                 0, nullptr, 0, nullptr, nullptr);
  if (st != RMM_OK) return st;
  if (M == 0 || N == 0) return RMM_OK;
  const size_t need = rmm_workspace_bytes_within(dtype, M, N, K, 0, kScratchBytes);
  if (need > kScratchBytes) return RMM_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t err = scratch_for_current_device(&ws);
    if (err != hipSuccess) {
      rmm_set_last_hip_error((int)err);
      return RMM_ERR_HIP;
    }
  }
  return rmsnorm_matmul(X, g, W, Y, eps, M, N, K, dtype, ws, ws ? kScratchBytes : 0, stream);
}

}  // extern "C"
