// Kernel launchers (host side).  Each enqueues on `stream` and returns the
// launch status reported by the HIP runtime.
#pragma once

#include <hip/hip_runtime.h>

#include "pvj_internal.h"

namespace pvj {

hipError_t launch_pack(const pvj_plan* p, const Meta& m, const void* text, const void* image,
                       void* joint, bool unpack, bool rope, bool inverse, hipStream_t stream);
// sm: x, y in the stream-major layout (all text rows, then all image rows)
hipError_t launch_rope2d(const pvj_plan* p, const Meta& m, const void* x, void* y, bool inverse,
                         bool sm, hipStream_t stream);
// sm: the token tensors (and LSE's token order) in the stream-major layout
hipError_t launch_attn_fwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, void* o, float* lse, float scale, bool rope, bool sm,
                           hipStream_t stream);
// dQ from Q', K' (already rotated when rope), V, O, dO, LSE; it also writes
// Delta = rowsum(dO * O) [H, T], which the dK/dV kernel reads, so it runs first
hipError_t launch_attn_bwd_dq(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                              const void* v, const void* o, const void* dout, const float* lse,
                              float* delta, void* dq, float scale, bool rope, bool sm,
                              hipStream_t stream);
// dK, dV from Q', K', V, dO, LSE and Delta; with rope the stored dK (and, in
// the dQ kernel, dQ) are rotated back by R^T
hipError_t launch_attn_bwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, const void* dout, const float* lse,
                           const float* delta, void* dk, void* dv, float scale, bool rope,
                           bool sm, hipStream_t stream);

// memory-bound chains on one stream (which: 0 text, 1 image) of C columns
// row ranges per sample of the per-sample reductions, from the stream's
// longest sample; workspace for mode 0 (adaln) or 1 (gate)
int chain_splits(int max_sample_rows);
size_t chain_workspace_bytes(int n_samples, int C, int rows, int mode, int splits);
hipError_t launch_adaln_fwd(const pvj_plan* p, int which, int C, const void* x,
                            const void* shift, const void* scale, void* y, float eps,
                            hipStream_t stream);
hipError_t launch_gate_fwd(const pvj_plan* p, int which, int C, const void* x,
                           const void* y, const void* gate, void* out, hipStream_t stream);
hipError_t launch_adaln_bwd(const pvj_plan* p, int which, int C, const void* x,
                            const void* scale, const void* dy, void* dx, float* dshift,
                            float* dscale, float eps, int splits, void* ws, hipStream_t stream);
hipError_t launch_gate_bwd(const pvj_plan* p, int which, int C, const void* y,
                           const void* gate, const void* dout, void* dy, float* dgate, int splits,
                           void* ws, hipStream_t stream);

// projections with the pack / unpack fused (bf16): qkv writes joint Q, K, V rows
// (RoPE on Q, K when rope), out reads the stream's rows from the joint O
hipError_t launch_qkv_proj(const pvj_plan* p, const Meta& m, int which, int C, const void* x,
                           const void* w, const void* bias, void* q, void* k, void* v, bool rope,
                           hipStream_t stream);
hipError_t launch_out_proj(const pvj_plan* p, const Meta& m, int which, int C, const void* o,
                           const void* w, const void* bias, void* y, hipStream_t stream);
// diagnostic: matrix-core-only kernel on every CU; *flop = its bf16 FLOP count
hipError_t launch_mfma_peak(int rounds, int iters, float* sink, double* flop, hipStream_t stream);

}  // namespace pvj
