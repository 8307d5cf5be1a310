// Internal declarations shared by the planner, the C-ABI glue and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pvj.h"

namespace pvj {

constexpr int kNumXcd = 8;          // MI355X: 8 XCDs; workgroups are dealt round-robin
constexpr size_t kMetaAlign = 256;  // alignment of every metadata section
constexpr int kMaxLatentSide = 32767;  // h_lat, w_lat, n_frames limit (bounds the RoPE tables)

// Rows of one attention work item.  Forward: query rows per workgroup.
// Backward: key rows per workgroup.
inline int fwd_tile_rows(int dtype, int head_dim) {
  (void)head_dim;
  return dtype == PVJ_BF16 ? 256 : 128;
}
inline int bwd_tile_rows(int dtype, int head_dim) {
  (void)dtype; (void)head_dim;
  return 128;
}

struct Item {  // one attention work item; sample < 0 marks an idle slot
  int32_t sample, head, tile, pad;
};

struct SampleInfo {  // per-sample metadata read by the kernels
  int32_t start;   // first packed row (cu_seqlens[i])
  int32_t len;     // L_i
  int32_t l_text;  // text rows at the start of the sample
  int32_t w_lat;   // latent grid width
  int32_t hw;      // h_lat * w_lat: image token p is at ((p % hw) / w, p % w, p / hw)
  int32_t pad[3];
};

// Device view of an uploaded plan (pointers into the caller's metadata buffer).
struct Meta {
  const int32_t* cu;        // [B+1]
  const int32_t* cu_text;   // [B+1]
  const int32_t* cu_img;    // [B+1]
  const SampleInfo* sinfo;  // [B]
  const float* cos_tab;     // [n_pos][n_pairs]
  const float* sin_tab;     // [n_pos][n_pairs]
  const Item* fwd_items;    // [n_fwd]
  const Item* bwd_items;    // [n_bwd]
  int32_t n_samples, n_tokens, n_heads, head_dim;
  int32_t n_pos, n_pairs, n_fwd, n_bwd;
  int32_t fwd_tile, bwd_tile, n_text, n_img;
  // RoPE axis of head-dim unit u (dims 8u .. 8u+7): row if u < rope_u0, column
  // if u < rope_u1, frame otherwise
  int32_t rope_u0, rope_u1;
};

}  // namespace pvj

// the plan object behind the opaque C handle
struct pvj_plan {
  pvj_plan_desc_t desc;
  int32_t n_samples;
  int64_t n_tokens;
  int32_t max_len;
  int32_t n_pos, n_pairs;
  int32_t rope_axes, rope_dims[3];
  int32_t n_text, n_img;
  int32_t fwd_tile, bwd_tile;
  int32_t n_fwd, n_bwd;
  // host image of the device metadata and section offsets into it
  uint8_t* image;
  size_t image_bytes;
  size_t off_cu, off_cu_text, off_cu_img, off_sinfo, off_cos, off_sin, off_fwd, off_bwd;
  // device copy (set by pvj_plan_upload)
  void* dev_meta;
  int dev_id;
};

// return a failing status from the enclosing function
#define PVJ_TRY_STATUS(x)              \
  do {                                 \
    const pvj_status_t st__ = (x);     \
    if (st__ != PVJ_OK) return st__;   \
  } while (0)

namespace pvj {
// thread-local error detail (pvj_last_error)
pvj_status_t fail(pvj_status_t st, const char* fmt, ...);
Meta device_meta(const pvj_plan* p);

// attention backward, shared by the entry point with a caller workspace and
// the allocation-free one: argument validation (everything but the
// workspace), and the enqueue of preprocess, dK/dV and dQ with Delta at
// `delta` ([H, T] fp32) and, with PVJ_FLAG_ROPE_FUSED, Q' and K' at qr, kr
size_t attn_bwd_delta_bytes(const pvj_plan* p);
pvj_status_t check_attn_bwd_args(const pvj_plan* p, const void* q, const void* k, const void* v,
                                 const void* o, const float* lse, const void* dout,
                                 const void* dq, const void* dk, const void* dv,
                                 float softmax_scale, uint32_t flags);
pvj_status_t run_attn_bwd(const pvj_plan* p, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dout, void* dq, void* dk,
                          void* dv, float* delta, void* qr, void* kr, float softmax_scale,
                          uint32_t flags, void* stream);

template <typename T>
inline const T* host_section(const pvj_plan* p, size_t off) {
  return reinterpret_cast<const T*>(p->image + off);
}
}  // namespace pvj
