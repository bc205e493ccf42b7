// cce_forward_no_workspace (include/cce.h): cce_forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The forward's only scratch, the per-(range, token) log-sum-exp partials, lives
// in a file-scope device array of kScratchBytes instead of a caller workspace.
//
// The array's name is a host-side stand-in in host code, not a device address: its address on
// each device is looked up once, with that device current, and only that address is ever
// handed to the kernels.  Every GPU holds its own copy of the array for the life of the
// process; calls that overlap on one GPU share it and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cce.h"

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB per GPU
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];

// Address of `scratch` on the current device (nullptr if the lookup failed).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_addr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  return g_addr[dev];
}

}  // namespace

extern "C" {

size_t cce_forward_no_workspace_max_bytes(void) { return kScratchBytes; }

cce_status cce_forward_no_workspace(const void* E, const void* C, const int64_t* targets,
                                    int64_t N, int64_t V, int64_t D, cce_dtype dtype,
                                    int64_t ignore_index, float* loss, float* lse,
                                    float* tile_max, int32_t* err_flag, void* stream) {
  // argument errors first, exactly as cce_forward reports them (it takes no workspace for
  // N == 0 and checks sizes before the workspace)
  const size_t need = cce_forward_workspace_bytes(N, V, D, dtype);
  if (N == 0 || need == 0)
    return cce_forward(E, C, targets, N, V, D, dtype, ignore_index, loss, lse, tile_max,
                       nullptr, 0, err_flag, stream);
  if (need > kScratchBytes) return CCE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = scratch_address();
  if (!ws) return CCE_ERR_HIP;
  return cce_forward(E, C, targets, N, V, D, dtype, ignore_index, loss, lse, tile_max, ws,
                     kScratchBytes, err_flag, stream);
}

}  // extern "C"
