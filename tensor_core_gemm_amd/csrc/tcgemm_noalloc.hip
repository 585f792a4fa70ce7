// gemm_run_noalloc: gemm_run_ex for callers that cannot allocate device
// memory.  The only scratch memory any kernel of the library uses is the
// split-K workspace (each K range's fp32 partial sums, written by the GEMM
// kernel and read back by the reduction kernel).  Here it comes from one
// fixed device array that the library owns, `scratch`, instead of a buffer
// the caller brings.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy until the process ends.  In host code its name is only
// a host-side stand-in, never a device address; the device address of each
// GPU's copy is fetched once per device with hipGetSymbolAddress (with that
// device current) and kept, and only that address reaches the kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tcgemm.h"

namespace {

constexpr int64_t kScratchBytes = GEMM_NOALLOC_SCRATCH_BYTES;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_ready[kMaxDevices];

// The device address of `dev`'s copy of `scratch` (dev is the current
// device).  Fetched on the first call on that device, then reused.
int scratch_of(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return GEMM_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ready[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return GEMM_E_DEVICE;
    }
    g_scratch_ptr[dev] = p;
    g_scratch_ready[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return GEMM_OK;
}

}  // namespace

extern "C" int gemm_run_noalloc(gemm_plan_t plan, const void* A, const void* B, void* C, const void* bias,
                                void* stream) {
  gemm_plan_info in;
  const int rc = gemm_plan_get_info(plan, &in);
  if (rc != GEMM_OK) return rc;
  // Checked before any device call: a plan whose partial sums do not fit
  // the fixed array is refused, whatever device is current.
  if (in.workspace_bytes > kScratchBytes) return GEMM_E_SCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_E_DEVICE;
  }
  void* ws = nullptr;
  const int src = scratch_of(dev, &ws);
  if (src != GEMM_OK) return src;
  gemm_run_args args = {};
  args.bias = bias;
  if (in.workspace_bytes > 0) {
    // Every element of every K range's M x N sums is written by the GEMM
    // kernel before the reduction reads it, so nothing in the array needs
    // clearing between calls.
    args.workspace = ws;
    args.workspace_bytes = kScratchBytes;
  }
  return gemm_run_ex(plan, A, B, C, &args, stream);
}
