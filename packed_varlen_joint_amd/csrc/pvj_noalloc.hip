// Allocation-free attention backward: the same kernels as pvj_varlen_attn_bwd,
// with the backward's one scratch buffer (Delta = rowsum(dO * O), fp32
// [H, T]) in a library-owned static device array instead of a caller
// workspace.  For callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Its
// host-side name is not a device address, so the entry point looks the
// address up once per device (hipGetSymbolAddress, with that device current)
// and passes only that pointer to the kernels.  Every call on one GPU shares
// that GPU's array: calls that overlap on one GPU (several streams or host
// threads) race on it.  Delta is written in full by the preprocess before the
// kernels read it, so nothing needs clearing between calls.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pvj_internal.h"

namespace pvj {
namespace {

constexpr size_t kScratchBytes = PVJ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// device address of the current device's copy of `scratch`
pvj_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PVJ_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PVJ_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PVJ_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return PVJ_OK;
}

}  // namespace
}  // namespace pvj

using namespace pvj;

extern "C" {

PVJ_API pvj_status_t pvj_varlen_attn_bwd_noalloc(const pvj_plan_t* p, const void* q, const void* k,
                                                 const void* v, const void* o, const float* lse,
                                                 const void* dout, void* dq, void* dk, void* dv,
                                                 float softmax_scale, uint32_t flags,
                                                 void* stream) {
  // size and flag limits first: pure host checks, before anything touches HIP
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (flags & PVJ_FLAG_ROPE_FUSED)
    return fail(PVJ_ERR_UNSUPPORTED,
                "the allocation-free backward takes no PVJ_FLAG_ROPE_FUSED (its rotated Q', K' "
                "do not fit the scratch buffer); pass pre-rotated Q, K with "
                "PVJ_FLAG_ROPE_PREROTATED");
  const size_t need = attn_bwd_delta_bytes(p);
  if (need > kScratchBytes)
    return fail(PVJ_ERR_WORKSPACE_TOO_SMALL,
                "the allocation-free backward needs %zu bytes of scratch (H * T * 4), above "
                "its fixed %zu",
                need, kScratchBytes);
  PVJ_TRY_STATUS(check_attn_bwd_args(p, q, k, v, o, lse, dout, dq, dk, dv, softmax_scale, flags));
  if (p->n_tokens == 0) return PVJ_OK;
  void* ws = nullptr;
  PVJ_TRY_STATUS(scratch_on_current_device(&ws));
  return run_attn_bwd(p, q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(ws), nullptr,
                      nullptr, softmax_scale, flags, stream);
}

}  // extern "C"
