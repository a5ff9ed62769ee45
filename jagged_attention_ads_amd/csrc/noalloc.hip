// jfa_forward_noalloc: the forward pass with its scratch space -- the
// offsets-check word and the query-tile work list that jfa_forward keeps in
// the caller's workspace -- in a file-scope device array of this library
// instead, for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation).
// Same kernels, same results, bit for bit.
//
// Every GPU the library runs on holds its own copy of `scratch` until the
// process ends.  In host code the array's name stands for a host-side
// shadow, not a device address, so the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is ever passed on.  Calls on one GPU share its copy: calls that
// overlap on one GPU (several streams, several threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "jfa.h"
#include "jfa_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB per device
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Device address of this device's `scratch`, looked up on the first call
// that runs on it.  `dev` is the device the stream belongs to; if it is not
// the current one, it is made current for the lookup and the previous one
// restored.
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != dev) {
      const hipError_t r = hipSetDevice(prev);
      if (e == hipSuccess) e = r;
    }
    g_status[dev] = e;
    g_scratch[dev] = e == hipSuccess ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess) return g_status[dev];
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int jfa_forward_noalloc(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                                   const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim,
                                   int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len,
                                   float scale, int32_t activation, int32_t causal, int32_t dtype, void* out,
                                   float* lse, hipStream_t stream) {
  const int st = jfa::forward_args_status(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv,
                                          max_q_len, max_kv_len, scale, activation, causal, dtype, out, lse);
  if (st != JFA_OK) return st;
  if (batch == 0 || total_q == 0) return JFA_OK;   // nothing to write
  const size_t need = jfa_workspace_size(batch, heads, head_dim, total_q, total_kv, max_kv_len, dtype, 0);
  if (need > kScratchBytes)
    return jfa::report(JFA_ERR_UNSUPPORTED,
                       "the forward's work list for these sizes exceeds the library's 8 MiB device scratch "
                       "(jfa_workspace_size(..., 0) > 8388608): use jfa_forward with a workspace");
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  void* ws = nullptr;
  if (e == hipSuccess) e = scratch_address(dev, &ws);
  if (e != hipSuccess) return jfa::report(JFA_ERR_HIP, std::string("device scratch lookup: ") + hipGetErrorString(e));
  return jfa_forward(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv, max_q_len,
                     max_kv_len, scale, activation, causal, dtype, out, lse, ws, kScratchBytes, stream);
}
