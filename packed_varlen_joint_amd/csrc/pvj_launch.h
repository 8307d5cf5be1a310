// Kernel launchers (host side).  Each enqueues on `stream` and returns the
// launch status reported by the HIP runtime.
#pragma once

#include <hip/hip_runtime.h>

#include "pvj_internal.h"

namespace pvj {

hipError_t launch_pack(const pvj_plan* p, const Meta& m, const void* text, const void* image,
                       void* joint, bool unpack, bool rope, bool inverse, hipStream_t stream);
hipError_t launch_rope2d(const pvj_plan* p, const Meta& m, const void* x, void* y, bool inverse,
                         hipStream_t stream);
hipError_t launch_attn_fwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, void* o, float* lse, float scale, bool rope,
                           hipStream_t stream);
// Delta = rowsum(dO * O) into delta [H, T]; with rope also Q' = R Q -> qr and
// K' = R K -> kr (same layout as q, k)
hipError_t launch_bwd_pre(const pvj_plan* p, const Meta& m, const void* o, const void* dout,
                          const void* q, const void* k, float* delta, void* qr, void* kr,
                          bool rope, hipStream_t stream);
// dK, dV (kernel 0) and dQ (kernel 1) from Q', K' (already rotated when rope),
// V, dO, LSE, Delta; with rope the stored dK, dQ are rotated back by R^T
hipError_t launch_attn_bwd(const pvj_plan* p, const Meta& m, int which, const void* q,
                           const void* k, const void* v, const void* dout, const float* lse,
                           const float* delta, void* dq, void* dk, void* dv, float scale,
                           bool rope, hipStream_t stream);

}  // namespace pvj
