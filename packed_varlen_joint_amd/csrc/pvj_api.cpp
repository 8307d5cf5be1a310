// C-ABI entry points that touch the device: metadata upload, pack/unpack,
// standalone RoPE, attention forward and backward.  Every argument is
// validated before anything is enqueued; a failing call leaves the stream
// untouched.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "pvj_internal.h"
#include "pvj_launch.h"

using namespace pvj;

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t elt_size(const pvj_plan* p) { return p->desc.dtype == PVJ_BF16 ? 2 : 4; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

pvj_status_t check_ptr(const void* ptr, const char* name, bool needed) {
  if (!needed) return PVJ_OK;
  if (!ptr) return fail(PVJ_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(PVJ_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return PVJ_OK;
}

pvj_status_t check_plan(const pvj_plan* p) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (!p->dev_meta) return fail(PVJ_ERR_NOT_UPLOADED, "plan metadata not uploaded");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PVJ_ERR_HIP, "hipGetDevice failed");
  if (dev != p->dev_id)
    return fail(PVJ_ERR_INVALID_ARG, "plan uploaded on device %d, current device is %d",
                p->dev_id, dev);
  return PVJ_OK;
}

pvj_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PVJ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PVJ_OK;
}

float resolve_scale(const pvj_plan* p, float s) {
  return s > 0.f ? s : 1.0f / std::sqrt((float)p->desc.head_dim);
}

// backward workspace: Delta fp32 [H, T], then the pre-rotated Q' and K' (used
// only with PVJ_FLAG_ROPE_FUSED; always counted so one size serves both)
size_t ws_delta_bytes(const pvj_plan* p) {
  return align256((size_t)p->n_tokens * p->desc.n_heads * sizeof(float));
}
size_t ws_rot_bytes(const pvj_plan* p) {
  return align256((size_t)p->n_tokens * p->desc.n_heads * p->desc.head_dim * elt_size(p));
}
size_t ws_total(const pvj_plan* p) { return ws_delta_bytes(p) + 2 * ws_rot_bytes(p); }

// ---- optional per-kernel event timing ----
struct EventPair {
  int kernel;
  hipEvent_t start, stop;
};
bool g_prof_on = false;
std::vector<EventPair> g_prof_pending;
double g_prof_ms[PVJ_KERNEL_COUNT] = {0};
int64_t g_prof_n[PVJ_KERNEL_COUNT] = {0};

// brackets one launch with events on `stream` when timing is enabled
struct KernelTimer {
  int kernel;
  hipStream_t stream;
  hipEvent_t a = nullptr, b = nullptr;
  KernelTimer(int k, hipStream_t s) : kernel(k), stream(s) {
    if (!g_prof_on) return;
    if (hipEventCreate(&a) != hipSuccess) {
      a = nullptr;
      return;
    }
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      a = b = nullptr;
      return;
    }
    (void)hipEventRecord(a, stream);
  }
  hipError_t done(hipError_t launch_status) {
    if (a && b) {
      (void)hipEventRecord(b, stream);
      g_prof_pending.push_back({kernel, a, b});
    }
    return launch_status;
  }
};

#define PVJ_TRY(x)                  \
  do {                              \
    pvj_status_t st__ = (x);        \
    if (st__ != PVJ_OK) return st__; \
  } while (0)

}  // namespace

namespace pvj {

size_t attn_bwd_delta_bytes(const pvj_plan* p) { return ws_delta_bytes(p); }

// The stream-major layout (PVJ_FLAG_STREAM_MAJOR) is served by the bf16
// kernels that read Q and K already rotated; their per-copy source offsets
// address the whole tensor with 32 bits.
pvj_status_t check_stream_major(const pvj_plan* p, uint32_t flags) {
  if (!(flags & PVJ_FLAG_STREAM_MAJOR)) return PVJ_OK;
  if (p->desc.dtype != PVJ_BF16)
    return fail(PVJ_ERR_UNSUPPORTED, "the stream-major layout needs a bf16 plan");
  if (flags & PVJ_FLAG_ROPE_FUSED)
    return fail(PVJ_ERR_UNSUPPORTED, "the stream-major layout takes rotated Q, K (no ROPE_FUSED)");
  // the kernels form 32-bit byte offsets of rows up to a tile past a sample's end
  if (((int64_t)p->n_tokens + 256) * p->desc.n_heads * p->desc.head_dim * 2 >= (int64_t(1) << 31))
    return fail(PVJ_ERR_UNSUPPORTED,
                "stream-major token tensors need (tokens + 256) * n_heads * head_dim * 2 < 2^31");
  return PVJ_OK;
}

pvj_status_t check_attn_bwd_args(const pvj_plan* p, const void* q, const void* k, const void* v,
                                 const void* o, const float* lse, const void* dout,
                                 const void* dq, const void* dk, const void* dv,
                                 float softmax_scale, uint32_t flags) {
  // flags first: host-only checks, before anything touches HIP
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (flags & ~(PVJ_FLAG_ROPE_FUSED | PVJ_FLAG_ROPE_PREROTATED | PVJ_FLAG_STREAM_MAJOR))
    return fail(PVJ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((flags & PVJ_FLAG_ROPE_FUSED) && (flags & PVJ_FLAG_ROPE_PREROTATED))
    return fail(PVJ_ERR_INVALID_ARG, "ROPE_FUSED and ROPE_PREROTATED exclude each other");
  PVJ_TRY(check_stream_major(p, flags));
  PVJ_TRY(check_plan(p));
  const bool need = p->n_tokens > 0;
  PVJ_TRY(check_ptr(q, "q", need));
  PVJ_TRY(check_ptr(k, "k", need));
  PVJ_TRY(check_ptr(v, "v", need));
  PVJ_TRY(check_ptr(o, "o", need));
  PVJ_TRY(check_ptr(lse, "lse", need));
  PVJ_TRY(check_ptr(dout, "dout", need));
  PVJ_TRY(check_ptr(dq, "dq", need));
  PVJ_TRY(check_ptr(dk, "dk", need));
  PVJ_TRY(check_ptr(dv, "dv", need));
  if (!std::isfinite(softmax_scale)) return fail(PVJ_ERR_INVALID_ARG, "softmax_scale not finite");
  return PVJ_OK;
}

pvj_status_t run_attn_bwd(const pvj_plan* p, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dout, void* dq, void* dk,
                          void* dv, float* delta, void* qr, void* kr, float softmax_scale,
                          uint32_t flags, void* stream) {
  if (p->n_tokens == 0) return PVJ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Meta m = device_meta(p);
  // fused: rotate Q and K in the preprocess; pre-rotated: take them as given.
  // Either way the epilogues rotate dQ' and dK' back (dX = R^T dX').
  const bool rope = (flags & PVJ_FLAG_ROPE_FUSED) != 0;
  const bool unrotate = rope || (flags & PVJ_FLAG_ROPE_PREROTATED) != 0;
  const bool sm = (flags & PVJ_FLAG_STREAM_MAJOR) != 0;
  const float scale = resolve_scale(p, softmax_scale);
  if (rope) {  // Q' = R Q, K' = R K (the standalone rotation, same bits)
    KernelTimer t(PVJ_KERNEL_BWD_PRE, s);
    hipError_t e = launch_rope2d(p, m, q, qr, false, false, s);
    if (e == hipSuccess) e = launch_rope2d(p, m, k, kr, false, false, s);
    PVJ_TRY(launched(t.done(e), "bwd RoPE of Q and K"));
  }
  const void* qq = rope ? qr : q;
  const void* kk = rope ? kr : k;
  {  // dQ first: it also writes Delta = rowsum(dO * O), which dK/dV reads
    KernelTimer t(PVJ_KERNEL_ATTN_BWD_DQ, s);
    PVJ_TRY(launched(t.done(launch_attn_bwd_dq(p, m, qq, kk, v, o, dout, lse, delta, dq, scale,
                                               unrotate, sm, s)),
                     "varlen_attn_bwd dQ"));
  }
  KernelTimer t(PVJ_KERNEL_ATTN_BWD, s);
  return launched(t.done(launch_attn_bwd(p, m, qq, kk, v, dout, lse, delta, dk, dv, scale,
                                         unrotate, sm, s)),
                  "varlen_attn_bwd dK/dV");
}

}  // namespace pvj

extern "C" {

PVJ_API pvj_status_t pvj_plan_upload(pvj_plan_t* p, void* dev_meta, size_t bytes, void* stream) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (!dev_meta) return fail(PVJ_ERR_INVALID_ARG, "dev_meta is NULL");
  if (reinterpret_cast<uintptr_t>(dev_meta) % kMetaAlign)
    return fail(PVJ_ERR_INVALID_ARG, "dev_meta is not %zu-byte aligned", kMetaAlign);
  if (bytes < p->image_bytes + p->part_bytes)
    return fail(PVJ_ERR_WORKSPACE_TOO_SMALL, "metadata buffer %zu < %zu bytes", bytes,
                p->image_bytes + p->part_bytes);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PVJ_ERR_HIP, "hipGetDevice failed");
  hipError_t e = hipMemcpyAsync(dev_meta, p->image, p->image_bytes, hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PVJ_ERR_HIP, "metadata upload: %s", hipGetErrorString(e));
  p->dev_meta = dev_meta;
  p->dev_id = dev;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_pack(const pvj_plan_t* p, const void* text, const void* image,
                              void* joint, void* stream) {
  PVJ_TRY(check_plan(p));
  PVJ_TRY(check_ptr(text, "text", p->n_text > 0));
  PVJ_TRY(check_ptr(image, "image", p->n_img > 0));
  PVJ_TRY(check_ptr(joint, "joint", p->n_tokens > 0));
  KernelTimer t(PVJ_KERNEL_PACK, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_pack(p, device_meta(p), text, image, joint, false, false, false,
                                     static_cast<hipStream_t>(stream))),
                  "pack");
}

PVJ_API pvj_status_t pvj_pack_rope(const pvj_plan_t* p, const void* text, const void* image,
                                   void* joint, int32_t inverse, void* stream) {
  PVJ_TRY(check_plan(p));
  PVJ_TRY(check_ptr(text, "text", p->n_text > 0));
  PVJ_TRY(check_ptr(image, "image", p->n_img > 0));
  PVJ_TRY(check_ptr(joint, "joint", p->n_tokens > 0));
  KernelTimer t(PVJ_KERNEL_PACK, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_pack(p, device_meta(p), text, image, joint, false, true,
                                     inverse != 0, static_cast<hipStream_t>(stream))),
                  "pack_rope");
}

PVJ_API pvj_status_t pvj_unpack(const pvj_plan_t* p, const void* joint, void* text, void* image,
                                void* stream) {
  PVJ_TRY(check_plan(p));
  PVJ_TRY(check_ptr(joint, "joint", p->n_tokens > 0));
  PVJ_TRY(check_ptr(text, "text", p->n_text > 0));
  PVJ_TRY(check_ptr(image, "image", p->n_img > 0));
  KernelTimer t(PVJ_KERNEL_UNPACK, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_pack(p, device_meta(p), text, image, const_cast<void*>(joint),
                                     true, false, false, static_cast<hipStream_t>(stream))),
                  "unpack");
}

PVJ_API pvj_status_t pvj_unpack_rope(const pvj_plan_t* p, const void* joint, void* text,
                                     void* image, int32_t inverse, void* stream) {
  PVJ_TRY(check_plan(p));
  PVJ_TRY(check_ptr(joint, "joint", p->n_tokens > 0));
  PVJ_TRY(check_ptr(text, "text", p->n_text > 0));
  PVJ_TRY(check_ptr(image, "image", p->n_img > 0));
  KernelTimer t(PVJ_KERNEL_UNPACK, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_pack(p, device_meta(p), text, image, const_cast<void*>(joint),
                                     true, true, inverse != 0,
                                     static_cast<hipStream_t>(stream))),
                  "unpack_rope");
}

static pvj_status_t rope2d(const pvj_plan_t* p, const void* x, void* y, int32_t inverse, bool sm,
                           void* stream) {
  PVJ_TRY(check_plan(p));
  PVJ_TRY(check_ptr(x, "x", p->n_tokens > 0));
  PVJ_TRY(check_ptr(y, "y", p->n_tokens > 0));
  if (x != y && p->n_tokens > 0) {
    const size_t n = (size_t)p->n_tokens * p->desc.n_heads * p->desc.head_dim * elt_size(p);
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    if (a < b + n && b < a + n) return fail(PVJ_ERR_INVALID_ARG, "x and y partially overlap");
  }
  KernelTimer t(PVJ_KERNEL_ROPE, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_rope2d(p, device_meta(p), x, y, inverse != 0, sm,
                                       static_cast<hipStream_t>(stream))),
                  "rope2d_apply");
}

PVJ_API pvj_status_t pvj_rope2d_apply(const pvj_plan_t* p, const void* x, void* y,
                                      int32_t inverse, void* stream) {
  return rope2d(p, x, y, inverse, false, stream);
}

PVJ_API pvj_status_t pvj_rope2d_apply_stream_major(const pvj_plan_t* p, const void* x, void* y,
                                                   int32_t inverse, void* stream) {
  return rope2d(p, x, y, inverse, true, stream);
}

PVJ_API pvj_status_t pvj_varlen_attn_fwd(const pvj_plan_t* p, const void* q, const void* k,
                                         const void* v, void* o, float* lse,
                                         float softmax_scale, uint32_t flags, void* stream) {
  // flags first: host-only checks, before anything touches HIP
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (flags & ~(PVJ_FLAG_ROPE_FUSED | PVJ_FLAG_STREAM_MAJOR))
    return fail(PVJ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  PVJ_TRY(check_stream_major(p, flags));
  PVJ_TRY(check_plan(p));
  const bool need = p->n_tokens > 0;
  PVJ_TRY(check_ptr(q, "q", need));
  PVJ_TRY(check_ptr(k, "k", need));
  PVJ_TRY(check_ptr(v, "v", need));
  PVJ_TRY(check_ptr(o, "o", need));
  if (lse && !aligned16(lse)) return fail(PVJ_ERR_INVALID_ARG, "lse is not 16-byte aligned");
  if (!std::isfinite(softmax_scale)) return fail(PVJ_ERR_INVALID_ARG, "softmax_scale not finite");
  KernelTimer t(PVJ_KERNEL_ATTN_FWD, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_attn_fwd(p, device_meta(p), q, k, v, o, lse,
                                         resolve_scale(p, softmax_scale),
                                         (flags & PVJ_FLAG_ROPE_FUSED) != 0,
                                         (flags & PVJ_FLAG_STREAM_MAJOR) != 0,
                                         static_cast<hipStream_t>(stream))),
                  "varlen_attn_fwd");
}

PVJ_API pvj_status_t pvj_varlen_attn_bwd_workspace(const pvj_plan_t* p, size_t* bytes) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (!bytes) return fail(PVJ_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_total(p);
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_varlen_attn_bwd(const pvj_plan_t* p, const void* q, const void* k,
                                         const void* v, const void* o, const float* lse,
                                         const void* dout, void* dq, void* dk, void* dv,
                                         void* workspace, size_t ws_bytes, float softmax_scale,
                                         uint32_t flags, void* stream) {
  PVJ_TRY(check_attn_bwd_args(p, q, k, v, o, lse, dout, dq, dk, dv, softmax_scale, flags));
  const size_t need_ws = ws_total(p);
  if (p->n_tokens > 0) {
    if (!workspace) return fail(PVJ_ERR_INVALID_ARG, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(PVJ_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (ws_bytes < need_ws)
      return fail(PVJ_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need_ws);
  }
  char* ws = static_cast<char*>(workspace);
  return run_attn_bwd(p, q, k, v, o, lse, dout, dq, dk, dv, reinterpret_cast<float*>(ws),
                      ws + ws_delta_bytes(p), ws + ws_delta_bytes(p) + ws_rot_bytes(p),
                      softmax_scale, flags, stream);
}

// ---- memory-bound chains --------------------------------------------------

static bool chain_stream(int32_t which) {
  return which == PVJ_STREAM_TEXT || which == PVJ_STREAM_IMAGE || which == PVJ_STREAM_BOTH;
}

static pvj_status_t check_chain(const pvj_plan* p, int32_t which, int32_t hidden, int* rows) {
  PVJ_TRY(check_plan(p));
  if (!chain_stream(which))
    return fail(PVJ_ERR_INVALID_ARG,
                "stream must be PVJ_STREAM_TEXT, PVJ_STREAM_IMAGE or PVJ_STREAM_BOTH");
  if (hidden < 8 || hidden > 8192 || hidden % 8)
    return fail(PVJ_ERR_UNSUPPORTED, "hidden %d: need a multiple of 8 in [8, 8192]", hidden);
  const int64_t n = chain_rows(p, which, true).rows;
  if (n * hidden * (int64_t)elt_size(p) >= (int64_t(1) << 40))
    return fail(PVJ_ERR_OVERFLOW, "stream tensor too large");
  *rows = (int)n;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_adaln_modulate(const pvj_plan_t* p, int32_t which, int32_t hidden,
                                        const void* x, const void* shift, const void* scale,
                                        void* y, float eps, void* stream) {
  int rows = 0;
  PVJ_TRY(check_chain(p, which, hidden, &rows));
  PVJ_TRY(check_ptr(x, "x", rows > 0));
  PVJ_TRY(check_ptr(y, "y", rows > 0));
  PVJ_TRY(check_ptr(shift, "shift", rows > 0));
  PVJ_TRY(check_ptr(scale, "scale", rows > 0));
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(PVJ_ERR_INVALID_ARG, "eps must be > 0");
  KernelTimer t(PVJ_KERNEL_CHAIN_FWD, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_adaln_fwd(p, which, hidden, x, shift, scale, y,
                                          eps, static_cast<hipStream_t>(stream))),
                  "adaln_modulate");
}

PVJ_API pvj_status_t pvj_gate_residual(const pvj_plan_t* p, int32_t which, int32_t hidden,
                                       const void* x, const void* y, const void* gate, void* out,
                                       void* stream) {
  int rows = 0;
  PVJ_TRY(check_chain(p, which, hidden, &rows));
  PVJ_TRY(check_ptr(x, "x", rows > 0));
  PVJ_TRY(check_ptr(y, "y", rows > 0));
  PVJ_TRY(check_ptr(gate, "gate", rows > 0));
  PVJ_TRY(check_ptr(out, "out", rows > 0));
  KernelTimer t(PVJ_KERNEL_CHAIN_FWD, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_gate_fwd(p, which, hidden, x, y, gate, out,
                                         static_cast<hipStream_t>(stream))),
                  "gate_residual");
}

// row ranges per sample of the chain reductions (from the call's longest segment)
static int stream_splits(const pvj_plan* p, int32_t which) {
  const ChainRows r = chain_rows(p, which, true);
  int mx = 0;
  for (int i = 0; i < r.n_seg; ++i) mx = std::max(mx, (int)(r.cu[i + 1] - r.cu[i]));
  return chain_splits(mx);
}

PVJ_API pvj_status_t pvj_chain_bwd_workspace(const pvj_plan_t* p, int32_t op, int32_t which,
                                             int32_t hidden, size_t* bytes) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (!bytes) return fail(PVJ_ERR_INVALID_ARG, "bytes is NULL");
  if (op != PVJ_CHAIN_ADALN && op != PVJ_CHAIN_GATE)
    return fail(PVJ_ERR_INVALID_ARG, "op must be PVJ_CHAIN_ADALN or PVJ_CHAIN_GATE");
  if (!chain_stream(which))
    return fail(PVJ_ERR_INVALID_ARG,
                "stream must be PVJ_STREAM_TEXT, PVJ_STREAM_IMAGE or PVJ_STREAM_BOTH");
  if (hidden < 8 || hidden > 8192 || hidden % 8)
    return fail(PVJ_ERR_UNSUPPORTED, "hidden %d: need a multiple of 8 in [8, 8192]", hidden);
  const ChainRows r = chain_rows(p, which, true);
  *bytes = chain_workspace_bytes(r.n_seg, hidden, r.rows, op == PVJ_CHAIN_ADALN ? 0 : 1,
                                 stream_splits(p, which));
  return PVJ_OK;
}

static pvj_status_t check_ws(const pvj_plan* p, int32_t op, int32_t which, int32_t hidden,
                             const void* ws, size_t ws_bytes) {
  size_t need = 0;
  PVJ_TRY(pvj_chain_bwd_workspace(p, op, which, hidden, &need));
  if (p->n_samples == 0) return PVJ_OK;
  if (!ws) return fail(PVJ_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(PVJ_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(PVJ_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_adaln_modulate_bwd(const pvj_plan_t* p, int32_t which, int32_t hidden,
                                            const void* x, const void* scale, const void* dy,
                                            void* dx, float* dshift, float* dscale, float eps,
                                            void* workspace, size_t ws_bytes, void* stream) {
  int rows = 0;
  PVJ_TRY(check_chain(p, which, hidden, &rows));
  PVJ_TRY(check_ptr(x, "x", rows > 0));
  PVJ_TRY(check_ptr(dy, "dy", rows > 0));
  PVJ_TRY(check_ptr(dx, "dx", rows > 0));
  PVJ_TRY(check_ptr(scale, "scale", rows > 0));
  PVJ_TRY(check_ptr(dshift, "dshift", p->n_samples > 0));
  PVJ_TRY(check_ptr(dscale, "dscale", p->n_samples > 0));
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(PVJ_ERR_INVALID_ARG, "eps must be > 0");
  PVJ_TRY(check_ws(p, PVJ_CHAIN_ADALN, which, hidden, workspace, ws_bytes));
  KernelTimer t(PVJ_KERNEL_CHAIN_BWD, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_adaln_bwd(p, which, hidden, x, scale, dy, dx,
                                          dshift, dscale, eps, stream_splits(p, which), workspace,
                                          static_cast<hipStream_t>(stream))),
                  "adaln_modulate_bwd");
}

PVJ_API pvj_status_t pvj_gate_residual_bwd(const pvj_plan_t* p, int32_t which, int32_t hidden,
                                           const void* y, const void* gate, const void* dout,
                                           void* dy, float* dgate, void* workspace,
                                           size_t ws_bytes, void* stream) {
  int rows = 0;
  PVJ_TRY(check_chain(p, which, hidden, &rows));
  PVJ_TRY(check_ptr(y, "y", rows > 0));
  PVJ_TRY(check_ptr(dout, "dout", rows > 0));
  PVJ_TRY(check_ptr(dy, "dy", rows > 0));
  PVJ_TRY(check_ptr(gate, "gate", rows > 0));
  PVJ_TRY(check_ptr(dgate, "dgate", p->n_samples > 0));
  PVJ_TRY(check_ws(p, PVJ_CHAIN_GATE, which, hidden, workspace, ws_bytes));
  KernelTimer t(PVJ_KERNEL_CHAIN_BWD, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_gate_bwd(p, which, hidden, y, gate, dout, dy,
                                         dgate, stream_splits(p, which), workspace,
                                         static_cast<hipStream_t>(stream))),
                  "gate_residual_bwd");
}

// ---- projections with the pack / unpack fused ----------------------------------

static pvj_status_t check_proj(const pvj_plan* p, int32_t which, int32_t hidden, int* rows) {
  PVJ_TRY(check_plan(p));
  if (p->desc.dtype != PVJ_BF16)
    return fail(PVJ_ERR_UNSUPPORTED, "the fused projections take bf16 plans only");
  if (which != PVJ_STREAM_TEXT && which != PVJ_STREAM_IMAGE)
    return fail(PVJ_ERR_INVALID_ARG, "stream must be PVJ_STREAM_TEXT or PVJ_STREAM_IMAGE");
  if (hidden < 64 || hidden % 64 || hidden > 65536)
    return fail(PVJ_ERR_UNSUPPORTED, "hidden %d: need a multiple of 64 in [64, 65536]", hidden);
  const int64_t hd = (int64_t)p->desc.n_heads * p->desc.head_dim;
  const int64_t n = which == PVJ_STREAM_TEXT ? p->n_text : p->n_img;
  const int64_t lim = int64_t(1) << 31;
  // 32-bit byte offsets inside every operand
  if ((n + 128) * hidden * 2 >= lim || (p->n_tokens + 128) * hd * 2 >= lim ||
      3 * hd * hidden * 2 >= lim || (n + 128) * 3 * hd * 2 >= lim)
    return fail(PVJ_ERR_UNSUPPORTED, "projection operands must stay below 2 GiB");
  *rows = (int)n;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_qkv_proj_pack(const pvj_plan_t* p, int32_t which, int32_t hidden,
                                       const void* x, const void* w, const void* bias, void* q,
                                       void* k, void* v, uint32_t flags, void* stream) {
  int rows = 0;
  PVJ_TRY(check_proj(p, which, hidden, &rows));
  PVJ_TRY(check_ptr(x, "x", rows > 0));
  PVJ_TRY(check_ptr(w, "w", rows > 0));
  if (bias) PVJ_TRY(check_ptr(bias, "bias", true));
  PVJ_TRY(check_ptr(q, "q", rows > 0));
  PVJ_TRY(check_ptr(k, "k", rows > 0));
  PVJ_TRY(check_ptr(v, "v", rows > 0));
  if (flags & ~PVJ_FLAG_ROPE_FUSED) return fail(PVJ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  KernelTimer t(PVJ_KERNEL_PROJ, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_qkv_proj(p, device_meta(p), which, hidden, x, w, bias, q, k, v,
                                         (flags & PVJ_FLAG_ROPE_FUSED) != 0,
                                         static_cast<hipStream_t>(stream))),
                  "qkv_proj_pack");
}

PVJ_API pvj_status_t pvj_out_proj_unpack(const pvj_plan_t* p, int32_t which, int32_t hidden,
                                         const void* o, const void* w, const void* bias, void* y,
                                         void* stream) {
  int rows = 0;
  PVJ_TRY(check_proj(p, which, hidden, &rows));
  PVJ_TRY(check_ptr(o, "o", rows > 0));
  PVJ_TRY(check_ptr(w, "w", rows > 0));
  if (bias) PVJ_TRY(check_ptr(bias, "bias", true));
  PVJ_TRY(check_ptr(y, "y", rows > 0));
  KernelTimer t(PVJ_KERNEL_PROJ, static_cast<hipStream_t>(stream));
  return launched(t.done(launch_out_proj(p, device_meta(p), which, hidden, o, w, bias, y,
                                         static_cast<hipStream_t>(stream))),
                  "out_proj_unpack");
}

PVJ_API pvj_status_t pvj_diag_mfma_peak(int32_t rounds, int32_t iters, float* sink,
                                        size_t sink_floats, double* flop, void* stream) {
  if (rounds < 1 || rounds > 64 || iters < 1 || iters > (1 << 20))
    return fail(PVJ_ERR_INVALID_ARG, "rounds in [1, 64], iters in [1, 2^20]");
  if (!flop) return fail(PVJ_ERR_INVALID_ARG, "flop is NULL");
  const size_t need = (size_t)256 * 2 * rounds * 256;
  PVJ_TRY(check_ptr(sink, "sink", true));
  if (sink_floats < need)
    return fail(PVJ_ERR_WORKSPACE_TOO_SMALL, "sink %zu < %zu floats", sink_floats, need);
  return launched(launch_mfma_peak(rounds, iters, sink, flop, static_cast<hipStream_t>(stream)),
                  "diag_mfma_peak");
}

PVJ_API pvj_status_t pvj_profile_enable(int32_t on) {
  for (auto& e : g_prof_pending) {
    (void)hipEventSynchronize(e.stop);
    (void)hipEventDestroy(e.start);
    (void)hipEventDestroy(e.stop);
  }
  g_prof_pending.clear();
  for (int i = 0; i < PVJ_KERNEL_COUNT; ++i) {
    g_prof_ms[i] = 0;
    g_prof_n[i] = 0;
  }
  g_prof_on = on != 0;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_profile_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= PVJ_KERNEL_COUNT)
    return fail(PVJ_ERR_INVALID_ARG, "kernel id %d out of range", kernel);
  // entries are removed from the pending list as they are consumed, so a failure
  // part-way leaves only the not yet consumed ones for a later read
  pvj_status_t st = PVJ_OK;
  std::vector<EventPair> keep;
  size_t i = 0;
  for (; i < g_prof_pending.size(); ++i) {
    const EventPair& e = g_prof_pending[i];
    if (e.kernel != kernel) {
      keep.push_back(e);
      continue;
    }
    float ms = 0.f;
    if (hipEventSynchronize(e.stop) != hipSuccess) {
      st = fail(PVJ_ERR_HIP, "event sync");
      break;
    }
    if (hipEventElapsedTime(&ms, e.start, e.stop) != hipSuccess) {
      st = fail(PVJ_ERR_HIP, "event elapsed time");
      break;
    }
    g_prof_ms[kernel] += ms;
    g_prof_n[kernel] += 1;
    (void)hipEventDestroy(e.start);
    (void)hipEventDestroy(e.stop);
  }
  for (; i < g_prof_pending.size(); ++i) keep.push_back(g_prof_pending[i]);
  g_prof_pending.swap(keep);
  if (st != PVJ_OK) return st;
  if (total_ms) *total_ms = g_prof_ms[kernel];
  if (launches) *launches = g_prof_n[kernel];
  return PVJ_OK;
}

}  // extern "C"
