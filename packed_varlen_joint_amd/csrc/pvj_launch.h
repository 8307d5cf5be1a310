// Kernel launchers (host side).  Each enqueues on `stream` and returns the
// launch status reported by the HIP runtime.
#pragma once

#include <hip/hip_runtime.h>

#include "pvj_internal.h"

namespace pvj {

hipError_t launch_pack(const pvj_plan* p, const Meta& m, const void* text, const void* image,
                       void* joint, bool unpack, hipStream_t stream);
hipError_t launch_rope2d(const pvj_plan* p, const Meta& m, const void* x, void* y, bool inverse,
                         hipStream_t stream);
hipError_t launch_attn_fwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, void* o, float* lse, float scale, bool rope,
                           hipStream_t stream);
// Delta = rowsum(dO * O) into delta [H, T], and zero the fp32 dQ accumulator
hipError_t launch_bwd_pre(const pvj_plan* p, const Meta& m, const void* o, const void* dout,
                          float* delta, float* dq_acc, hipStream_t stream);
hipError_t launch_attn_bwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, const void* dout, const float* lse,
                           const float* delta, float* dq_acc, void* dk, void* dv, float scale,
                           bool rope, hipStream_t stream);
// dQ = (inverse RoPE of) the fp32 accumulator, rounded to the plan dtype
hipError_t launch_dq_finalize(const pvj_plan* p, const Meta& m, const float* dq_acc, void* dq,
                              bool rope, hipStream_t stream);

}  // namespace pvj
