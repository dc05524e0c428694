// Allocation-free variant of the fused decode layer: the workspace is a
// file-scope device array instead of a caller buffer, for callers that
// cannot allocate (code under HIP-graph capture, tight serving loops,
// harnesses that forbid allocation).  Same kernels and arguments as
// bskv_decode_layer_lookahead otherwise.
//
// The array lives in the library's code object: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels or
// runtime calls; the array's name in host code is a host-side stand-in.
// At that set-up the arrival counters at the start of the array are
// cleared by a fill kernel on the caller's stream; every complete call
// leaves them at zero again.  All calls on one device share the array, so
// calls that overlap in time on one device race.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "bskv_launch.hpp"
#include "../../include/bskv.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;       // 16 MiB per device
// the counter region: the first 2 * 65535 int32 words of every layer
// workspace, whatever the call's shape
constexpr size_t kCounterBytes = size_t(2) * 65535 * 4;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's array; on the first call for a device,
// the lookup and the clearing of the counter region on `stream`.
hipError_t scratch_on_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    const size_t n = kCounterBytes / 4;
    hipLaunchKernelGGL(zero_words, dim3(128), dim3(256), 0, stream, (uint32_t*)p, n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace bskv {
void set_last_error(const char* msg);
int report_hip(hipError_t e);
}  // namespace bskv

extern "C" {

size_t bskv_decode_layer_lookahead_noalloc_capacity(void) { return kScratchBytes; }

int bskv_decode_layer_lookahead_noalloc(const void* q, const void* k, const void* v, int dtype,
                                        const int64_t* kv_strides, int64_t kv_len, const int64_t* seq_len, float* kc,
                                        const float* scores, int32_t* idx, int32_t* cnt, float scale, float* out,
                                        const void* x, const void* w_forecast, int hidden, const float* kc_next,
                                        float* scores_next, int32_t* idx_next, int32_t* cnt_next, int B,
                                        int n_q_heads, int n_kv_heads, int head_dim, int block, int64_t kc_nb_cap,
                                        int topk, int n_init, int n_local, int stages, hipStream_t stream) {
  // sizes first, on the host only: nothing touches the device for a call
  // that cannot fit
  const int U = topk + n_init + n_local;
  const size_t need = bskv_decode_layer_lookahead_workspace(B, n_q_heads, n_kv_heads, head_dim, x ? hidden : 0,
                                                            kc_nb_cap, U, dtype);
  if (need == 0) return BSKV_EINVAL;
  if (need > kScratchBytes) {
    bskv::set_last_error("bskv_decode_layer_lookahead_noalloc: the layer needs more workspace than the 16 MiB "
                         "static scratch holds");
    return BSKV_ENOSPC;
  }
  void* ws = nullptr;
  const hipError_t e = scratch_on_device(stream, &ws);
  if (e != hipSuccess) return bskv::report_hip(e);
  return bskv_decode_layer_lookahead(q, k, v, dtype, kv_strides, kv_len, seq_len, kc, scores, idx, cnt, scale, out, x,
                                     w_forecast, hidden, kc_next, scores_next, idx_next, cnt_next, B, n_q_heads,
                                     n_kv_heads, head_dim, block, kc_nb_cap, topk, n_init, n_local, stages, ws,
                                     kScratchBytes, stream);
}

}  // extern "C"
