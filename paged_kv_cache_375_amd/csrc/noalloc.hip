// pa_decode_step for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, hosts that forbid hipMalloc): the
// split-context workspace is a file-scope device array of the library, one
// per GPU, instead of a buffer the caller brings.
//
// Host code never passes `scratch` itself to a kernel: in host code that name
// is a host-side stand-in, not a device address.  The first call on each
// device looks up that device's copy with hipGetSymbolAddress and keeps the
// address; every kernel receives that address, exactly as the workspace
// argument of pa_decode_step.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "launch.h"

namespace {

// Bytes of the library's scratch on each device: split-context partials and
// arrival counters of pa_decode_step (pa_decode_workspace_size), up to 32 MiB.
constexpr size_t kScratchBytes = size_t{32} << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // each device's address of `scratch`, once looked up and cleared

// Zero `words` 32-bit words from p (a grid-stride fill; a kernel rather than
// a memset so that a stream being captured records a plain kernel node).
__global__ void fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// The device address of `scratch` on the current device.  On a device's
// first call the address is looked up and the whole array cleared with a fill
// kernel on `st`, ordered before the call's decode; the clear is recorded as
// done only when `st` is not being captured (else a captured graph would hold
// the only clear, and it runs again on every replay of that graph).
pa_status scratch_for_device(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "pa_decode_step_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode_step_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev]) {
    *out = g_scratch_ptr[dev];
    return PA_OK;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr)
    return pa::fail(PA_ERR_HIP, "pa_decode_step_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(st, &cap);
  if (e != hipSuccess)
    return pa::fail(PA_ERR_HIP, "pa_decode_step_noalloc: hipStreamIsCapturing: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, st, static_cast<uint32_t*>(p),
                     kScratchBytes / sizeof(uint32_t));
  e = hipGetLastError();
  if (e != hipSuccess)
    return pa::fail(PA_ERR_HIP, "pa_decode_step_noalloc: clearing the scratch: %s", hipGetErrorString(e));
  if (cap == hipStreamCaptureStatusNone) g_scratch_ptr[dev] = p;
  *out = p;
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_step_noalloc(const pa_kv_cache* cache, const void* q, const void* k_new,
                                            const void* v_new, void* out, int32_t act, int32_t num_q_heads,
                                            const int32_t* block_tables, const int32_t* context_lens,
                                            int32_t num_seqs, int32_t max_blocks_per_seq, int32_t max_context_len,
                                            float sm_scale, void* stream) noexcept {
  static const char* fn = "pa_decode_step_noalloc";
  // the size check is host arithmetic only and comes first
  const size_t need = cache && num_seqs > 0 && num_q_heads > 0 && max_context_len >= 0
                          ? pa_decode_workspace_size(num_seqs, num_q_heads, cache->head_dim, max_context_len)
                          : 0;
  if (need > kScratchBytes)
    return pa::fail(PA_ERR_WORKSPACE_TOO_SMALL,
                    "%s: this call needs %zu bytes of split-context scratch, the library holds %zu per device "
                    "(pa_decode_step takes a workspace of any size)",
                    fn, need, kScratchBytes);
  if (need == 0)  // no context is split: the kernels use no workspace (or pa_decode_step reports an argument error)
    return pa_decode_step(cache, q, k_new, v_new, out, act, num_q_heads, block_tables, context_lens, num_seqs,
                          max_blocks_per_seq, max_context_len, sm_scale, nullptr, 0, stream);
  void* ws = nullptr;
  if (pa_status s = scratch_for_device(static_cast<hipStream_t>(stream), &ws)) return s;
  return pa_decode_step(cache, q, k_new, v_new, out, act, num_q_heads, block_tables, context_lens, num_seqs,
                        max_blocks_per_seq, max_context_len, sm_scale, ws, kScratchBytes, stream);
}
