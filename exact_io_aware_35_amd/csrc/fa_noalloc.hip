// fa_noalloc.hip -- fa_backward for callers that cannot allocate device
// memory. The backward's workspace (row statistics and operand copies) comes
// from a static device array of the library instead of a caller buffer; each
// GPU the library runs on holds its own copy of the array until the process
// ends, at an address looked up once per device.

#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.h"

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];          // device address of `scratch` on each GPU
hipError_t g_lookup[kMaxDevices];      // result of the one lookup per GPU
std::once_flag g_once[kMaxDevices];

// Device address of this GPU's `scratch`, looked up on the first call with
// that device current. The host-side symbol is only a stand-in: kernels and
// copies must use the address returned here.
fa_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fa::report(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fa::report(FA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the no-alloc "
                      "path serves", dev, kMaxDevices);
  std::call_once(g_once[dev], [dev] {
    g_lookup[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_lookup[dev] != hipSuccess)
    return fa::report(FA_ERR_HIP, "hipGetSymbolAddress(scratch): %s",
                      hipGetErrorString(g_lookup[dev]));
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" fa_status_t fa_backward_noalloc(const void* q, const void* k, const void* v,
                                           const void* out, const float* lse, const void* dout,
                                           void* dq, void* dk, void* dv,
                                           const int32_t* seqlens_k, int batch, int heads,
                                           int seqlen, int headdim, float softmax_scale,
                                           int causal, int window_left, int window_right,
                                           fa_dtype_t dtype, hipStream_t stream) {
  const size_t need = fa_backward_workspace_size(batch, heads, seqlen, headdim, dtype);
  void* ws = nullptr;
  if (need > FA_NOALLOC_SCRATCH_BYTES)
    return fa::report(FA_ERR_WORKSPACE, "these sizes need %zu bytes of workspace; the no-alloc "
                      "scratch holds %zu", need, (size_t)FA_NOALLOC_SCRATCH_BYTES);
  // need == 0: invalid sizes or an empty call; fa_backward reports or accepts
  // those before it looks at the workspace.
  if (need > 0) {
    fa_status_t s = scratch_address(&ws);
    if (s != FA_OK) return s;
  }
  return fa_backward(q, k, v, out, lse, dout, dq, dk, dv, seqlens_k, batch, heads, seqlen,
                     headdim, softmax_scale, causal, window_left, window_right, dtype, ws,
                     need > 0 ? (size_t)FA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
