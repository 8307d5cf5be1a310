// Internal declarations shared by the planner, the C-ABI glue and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pvj.h"

// helpers used by the host planner (a plain C++ translation unit) and by the
// kernels alike
#ifdef __HIP__
#define PVJ_HD __host__ __device__
#else
#define PVJ_HD
#endif

namespace pvj {

constexpr int kNumXcd = 8;          // MI355X: 8 XCDs; workgroups are dealt round-robin
constexpr size_t kMetaAlign = 256;  // alignment of every metadata section
constexpr int kMaxLatentSide = 32767;  // h_lat, w_lat, n_frames limit (bounds the RoPE tables)

// Rows of one attention work item.  Forward: query rows per workgroup.
// Backward dK/dV: key rows per workgroup (bf16 8 waves x 32, fp32 4 x 32).
inline int fwd_tile_rows(int dtype, int head_dim) {
  (void)head_dim;
  return dtype == PVJ_BF16 ? 256 : 128;
}
inline int bwd_tile_rows(int dtype, int head_dim) {
  (void)head_dim;
  return dtype == PVJ_BF16 ? 256 : 128;
}

struct Item {  // one attention work item; sample < 0 marks an idle slot
  int32_t sample, head, tile;
  // forward: 0 = the tile against all of its sample's keys; otherwise one key
  // range of a split tile: bits 0-3 = parts - 1, bits 4-7 = this part, bits
  // 8-31 = the tile's first partial-result slot.  Backward lists: 0.
  int32_t split;
};

// Forward tail split.  The last query tile of a (sample, head) of a short
// sample (L <= kFwdSplitMaxLen) is cut into up to kMaxFwdSplit ranges of
// consecutive 64-key tiles (each >= kFwdSplitMinTiles tiles); the parts are
// small items that fill the last round of a launch, and a merge pass combines
// their partial softmax states.  Long samples' items run first in the
// largest-first order, so splitting them would only add partial traffic.  The
// part count depends on the sample length only, so a sample's result never
// depends on the rest of the pack.  bf16 plans only.
constexpr int kMaxFwdSplit = 4;
constexpr int kFwdSplitMinTiles = 16;
constexpr int kFwdSplitMaxLen = 8192;
constexpr int kFwdKeyTile = 64;
PVJ_HD inline int fwd_key_tiles(int32_t L) { return (L + kFwdKeyTile - 1) / kFwdKeyTile; }
PVJ_HD inline int fwd_splits(int dtype, int32_t L) {
  if (dtype != PVJ_BF16 || L > kFwdSplitMaxLen) return 1;
  const int s = fwd_key_tiles(L) / kFwdSplitMinTiles;
  return s < 1 ? 1 : (s > kMaxFwdSplit ? kMaxFwdSplit : s);
}
// key tiles [first, end) of part j of n parts over nkt key tiles
// (nkt < 2^25 and j < 16: the product fits 32 bits)
PVJ_HD inline int fwd_split_begin(int nkt, int j, int n) { return nkt * j / n; }
PVJ_HD inline int split_parts(int32_t split) { return (split & 15) + 1; }
PVJ_HD inline int split_part(int32_t split) { return (split >> 4) & 15; }
PVJ_HD inline int split_slot(int32_t split) { return split >> 8; }
// one partial-result slot: O^T unnormalised [D][256 queries], then the
// reference max m (base 2) and the sum l of the 256 queries, fp32
PVJ_HD inline size_t fwd_part_floats(int head_dim) { return (size_t)(head_dim + 2) * 256; }

struct SampleInfo {  // per-sample metadata read by the kernels
  int32_t start;   // first packed row (cu_seqlens[i])
  int32_t len;     // L_i
  int32_t l_text;  // text rows at the start of the sample
  int32_t w_lat;   // latent grid width
  int32_t hw;      // h_lat * w_lat: image token p is at ((p % hw) / w, p % w, p / hw)
  // rows of the sample in a stream-major token tensor (all samples' text rows,
  // then all their image rows): its text at text_row .., its image at img_row ..
  int32_t text_row, img_row;
  int32_t pad;
};

// Device view of an uploaded plan (pointers into the caller's metadata buffer).
struct Meta {
  const int32_t* cu;        // [B+1]
  const int32_t* cu_text;   // [B+1]
  const int32_t* cu_img;    // [B+1]
  const SampleInfo* sinfo;  // [B]
  const float* cos_tab;     // [n_pos][n_pairs]
  const float* sin_tab;     // [n_pos][n_pairs]
  const Item* fwd_items;    // [n_fwd] forward, with split tiles
  const Item* bwd_items;    // [n_bwd] dK/dV
  const Item* dq_items;     // [n_dq] dQ: the forward tiles, none split
  const Item* split_tiles;  // [n_split] {sample, head, tile, slot << 8 | parts - 1}
  float* fwd_part;          // partial-result slots of the split tiles
  int32_t n_samples, n_tokens, n_heads, head_dim;
  int32_t n_pos, n_pairs, n_fwd, n_bwd, n_dq, n_split;
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
  int32_t n_fwd, n_bwd, n_dq, n_split, n_slots;
  // host image of the device metadata and section offsets into it; the device
  // buffer continues past the image with the forward's partial-result slots
  // (off_part, part_bytes), which are not uploaded
  uint8_t* image;
  size_t image_bytes;
  // off_cu_both: the 2B + 1 segment offsets of both streams as one row range
  size_t off_cu, off_cu_text, off_cu_img, off_cu_both, off_sinfo, off_cos, off_sin, off_fwd, off_bwd;
  size_t off_dq, off_split, off_part, part_bytes;
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
// PVJ_FLAG_STREAM_MAJOR's conditions (bf16 plan, no ROPE_FUSED, tensors < 2 GiB)
pvj_status_t check_stream_major(const pvj_plan* p, uint32_t flags);
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

// Rows of one chain call: the text stream, the image stream, or both as one
// range (the text stream's rows, then the image stream's), cut into segments
// that each take one row of the per-sample vectors: the plan's samples for one
// stream; for both, 2B segments, sample i's text rows at i and its image rows
// at B + i.  cu holds the n_seg + 1 segment offsets (device copy, or the host
// image with `host`).
struct ChainRows {
  const int32_t* cu;
  int rows, n_seg;
};
ChainRows chain_rows(const pvj_plan* p, int which, bool host);
}  // namespace pvj
