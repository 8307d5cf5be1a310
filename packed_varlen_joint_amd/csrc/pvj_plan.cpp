// Host planner: offsets, per-sample metadata, RoPE tables and attention work
// lists for one pack.  Pure host code (no device calls), so it is testable on
// a machine without a GPU.
//
// Packing (Mage-Flow review page, section "Native-Resolution MMDiT"): samples
// of different resolutions become variable-length token runs packed into one
// contiguous batch, with per-sample cumulative offsets in place of a
// block-diagonal mask.  Token counts (same page, section "Mage-VAE"): one
// latent token per 16x16 pixels, so a sample is (h_lat, w_lat, l_text) with
// l_text + h_lat * w_lat tokens.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "pvj_internal.h"

namespace pvj {

static thread_local char g_err[512] = "";

pvj_status_t fail(pvj_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Work list for one attention pass.  An item is one tile of `tile_rows` rows of
// one (sample, head); its cost is proportional to the keys (or queries) it
// streams on the other side: the whole sample, or for a forward split tile
// (fwd_splits) the part's key range.  Groups = (sample, head) are dealt to
// the 8 XCDs greedily, largest cost first (LPT), so each group's items share
// one XCD's L2 for the K/V (or Q/dO) they all stream.  Inside an XCD the
// items run largest cost first, so the split parts fill the end.  Launch slot
// b runs on XCD b % 8, so the per-XCD lists are interleaved, with idle slots
// (sample = -1) where a list is shorter than the longest one.  With `split`,
// the split tiles are appended to *split_tiles and their partial-result
// slots numbered from *n_slots on.
static std::vector<Item> build_items(const std::vector<int32_t>& len, int n_heads, int tile_rows,
                                     int dtype, bool split, std::vector<Item>* split_tiles,
                                     int64_t* n_slots) {
  struct Group { int32_t sample, head, n_tiles; int64_t cost; };
  std::vector<Group> groups;
  for (int32_t i = 0; i < (int32_t)len.size(); ++i) {
    if (len[i] == 0) continue;
    int32_t nt = (len[i] + tile_rows - 1) / tile_rows;
    for (int h = 0; h < n_heads; ++h)
      groups.push_back({i, h, nt, (int64_t)nt * (int64_t)len[i]});
  }
  std::stable_sort(groups.begin(), groups.end(), [&](const Group& a, const Group& b) {
    if (len[a.sample] != len[b.sample]) return len[a.sample] > len[b.sample];
    return false;
  });
  struct Work { Item it; int64_t cost; };
  std::vector<std::vector<Work>> per_xcd(kNumXcd);
  int64_t load[kNumXcd] = {0};
  for (const Group& g : groups) {
    int best = 0;
    for (int x = 1; x < kNumXcd; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += g.cost;
    const int32_t L = len[g.sample];
    const int S = split ? fwd_splits(dtype, L) : 1;
    for (int t = 0; t < g.n_tiles; ++t) {
      if (t + 1 < g.n_tiles || S == 1) {
        per_xcd[best].push_back({{g.sample, g.head, t, 0}, L});
        continue;
      }
      const int nkt = fwd_key_tiles(L);
      const int32_t slot = (int32_t)*n_slots;
      *n_slots += S;
      split_tiles->push_back({g.sample, g.head, t, (slot << 8) | (S - 1)});
      for (int j = 0; j < S; ++j) {
        const int64_t k0 = (int64_t)fwd_split_begin(nkt, j, S) * kFwdKeyTile;
        const int64_t k1 = std::min<int64_t>((int64_t)fwd_split_begin(nkt, j + 1, S) * kFwdKeyTile, L);
        per_xcd[best].push_back({{g.sample, g.head, t, (slot << 8) | (j << 4) | (S - 1)}, k1 - k0});
      }
    }
  }
  size_t longest = 0;
  for (auto& l : per_xcd) {
    std::stable_sort(l.begin(), l.end(), [](const Work& a, const Work& b) { return a.cost > b.cost; });
    longest = std::max(longest, l.size());
  }
  std::vector<Item> out;
  out.reserve(longest * kNumXcd);
  for (size_t s = 0; s < longest; ++s)
    for (int x = 0; x < kNumXcd; ++x)
      out.push_back(s < per_xcd[x].size() ? per_xcd[x][s].it : Item{-1, 0, 0, 0});
  return out;
}

ChainRows chain_rows(const pvj_plan* p, int which, bool host) {
  const uint8_t* b = host ? p->image : static_cast<const uint8_t*>(p->dev_meta);
  const size_t off = which == PVJ_STREAM_TEXT    ? p->off_cu_text
                     : which == PVJ_STREAM_IMAGE ? p->off_cu_img
                                                 : p->off_cu_both;
  const int rows = which == PVJ_STREAM_TEXT    ? p->n_text
                   : which == PVJ_STREAM_IMAGE ? p->n_img
                                               : p->n_text + p->n_img;
  const int n_seg = which == PVJ_STREAM_BOTH ? 2 * p->n_samples : p->n_samples;
  return {reinterpret_cast<const int32_t*>(b + off), rows, n_seg};
}

Meta device_meta(const pvj_plan* p) {
  const uint8_t* b = static_cast<const uint8_t*>(p->dev_meta);
  Meta m;
  m.cu = reinterpret_cast<const int32_t*>(b + p->off_cu);
  m.cu_text = reinterpret_cast<const int32_t*>(b + p->off_cu_text);
  m.cu_img = reinterpret_cast<const int32_t*>(b + p->off_cu_img);
  m.sinfo = reinterpret_cast<const SampleInfo*>(b + p->off_sinfo);
  m.cos_tab = reinterpret_cast<const float*>(b + p->off_cos);
  m.sin_tab = reinterpret_cast<const float*>(b + p->off_sin);
  m.fwd_items = reinterpret_cast<const Item*>(b + p->off_fwd);
  m.bwd_items = reinterpret_cast<const Item*>(b + p->off_bwd);
  m.dq_items = reinterpret_cast<const Item*>(b + p->off_dq);
  m.split_tiles = reinterpret_cast<const Item*>(b + p->off_split);
  m.fwd_part = p->n_slots ? reinterpret_cast<float*>(static_cast<uint8_t*>(p->dev_meta) + p->off_part)
                          : nullptr;
  m.n_samples = p->n_samples;
  m.n_tokens = (int32_t)p->n_tokens;
  m.n_heads = p->desc.n_heads;
  m.head_dim = p->desc.head_dim;
  m.n_pos = p->n_pos;
  m.n_pairs = p->n_pairs;
  m.rope_u0 = p->rope_dims[0] / 8;
  m.rope_u1 = (p->rope_dims[0] + p->rope_dims[1]) / 8;
  m.n_fwd = p->n_fwd;
  m.n_bwd = p->n_bwd;
  m.n_dq = p->n_dq;
  m.n_split = p->n_split;
  m.fwd_tile = p->fwd_tile;
  m.bwd_tile = p->bwd_tile;
  m.n_text = p->n_text;
  m.n_img = p->n_img;
  return m;
}

}  // namespace pvj

using namespace pvj;

extern "C" {

PVJ_API const char* pvj_version(void) { return "pvj 0.1 (gfx950)"; }

PVJ_API const char* pvj_last_error(void) { return g_err; }

PVJ_API const char* pvj_status_string(pvj_status_t s) {
  switch (s) {
    case PVJ_OK: return "PVJ_OK";
    case PVJ_ERR_INVALID_ARG: return "PVJ_ERR_INVALID_ARG";
    case PVJ_ERR_UNSUPPORTED: return "PVJ_ERR_UNSUPPORTED";
    case PVJ_ERR_OVERFLOW: return "PVJ_ERR_OVERFLOW";
    case PVJ_ERR_NOT_UPLOADED: return "PVJ_ERR_NOT_UPLOADED";
    case PVJ_ERR_WORKSPACE_TOO_SMALL: return "PVJ_ERR_WORKSPACE_TOO_SMALL";
    case PVJ_ERR_HIP: return "PVJ_ERR_HIP";
  }
  return "PVJ_ERR_UNKNOWN";
}

// shared by pvj_plan_create (frames = 1, 2 RoPE axes) and
// pvj_plan_create_frames (3 RoPE axes)
static pvj_status_t create_plan(const int32_t* hwtf, int32_t n_samples, int axes,
                                const pvj_plan_desc_t* desc, pvj_plan_t** out) {
  if (!out) return fail(PVJ_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!desc) return fail(PVJ_ERR_INVALID_ARG, "desc is NULL");
  if (n_samples < 0) return fail(PVJ_ERR_INVALID_ARG, "n_samples < 0");
  if (n_samples > 0 && !hwtf) return fail(PVJ_ERR_INVALID_ARG, "samples is NULL");
  if (desc->n_heads < 1) return fail(PVJ_ERR_INVALID_ARG, "n_heads must be >= 1");
  if (desc->n_heads > 4096) return fail(PVJ_ERR_UNSUPPORTED, "n_heads > 4096");
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(PVJ_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", desc->head_dim);
  if (desc->dtype != PVJ_BF16 && desc->dtype != PVJ_F32)
    return fail(PVJ_ERR_UNSUPPORTED, "dtype %d unsupported", desc->dtype);
  if (desc->rope_pairing != PVJ_ROPE_INTERLEAVED)
    return fail(PVJ_ERR_UNSUPPORTED, "rope_pairing %d unsupported", desc->rope_pairing);
  if (desc->text_first != 1) return fail(PVJ_ERR_UNSUPPORTED, "text_first must be 1");
  if (!(desc->rope_theta > 0.0f) || !std::isfinite(desc->rope_theta))
    return fail(PVJ_ERR_INVALID_ARG, "rope_theta must be finite and > 0");

  const int B = n_samples;
  std::vector<int32_t> len(B), cu(B + 1), cu_text(B + 1), cu_img(B + 1);
  std::vector<SampleInfo> sinfo(B);
  int64_t T = 0, nt = 0, ni = 0;
  int32_t max_len = 0, max_side = 0, max_frames = 0;
  cu[0] = cu_text[0] = cu_img[0] = 0;
  for (int i = 0; i < B; ++i) {
    const int32_t h = hwtf[4 * i], w = hwtf[4 * i + 1], t = hwtf[4 * i + 2];
    const int32_t f = hwtf[4 * i + 3];
    if (h < 0 || w < 0 || t < 0 || f < 0)
      return fail(PVJ_ERR_INVALID_ARG, "sample %d has a negative size", i);
    // the RoPE tables have one row per position up to the largest side or frame count
    if (h > kMaxLatentSide || w > kMaxLatentSide || f > kMaxLatentSide)
      return fail(PVJ_ERR_UNSUPPORTED, "sample %d: latent side or frames above %d", i,
                  kMaxLatentSide);
    const int64_t hw = (int64_t)h * (int64_t)w;
    const int64_t img = hw * (int64_t)f;
    const int64_t L = img + t;
    // the kernels index rows with int32 and multiply a row by H*D in int64
    if (hw > INT32_MAX || L > INT32_MAX)
      return fail(PVJ_ERR_OVERFLOW, "sample %d length overflows int32", i);
    // the kernels address one (sample, head) with 32-bit byte offsets
    const int64_t elt = desc->dtype == PVJ_BF16 ? 2 : 4;
    if (L * desc->n_heads * desc->head_dim * elt >= (int64_t(1) << 31))
      return fail(PVJ_ERR_UNSUPPORTED, "sample %d spans 2 GiB or more of a token tensor", i);
    T += L;
    nt += t;
    ni += img;
    if (T > INT32_MAX) return fail(PVJ_ERR_OVERFLOW, "packed length T overflows int32");
    len[i] = (int32_t)L;
    cu[i + 1] = (int32_t)T;
    cu_text[i + 1] = (int32_t)nt;
    cu_img[i + 1] = (int32_t)ni;
    sinfo[i] = {cu[i], (int32_t)L, t, w, (int32_t)hw, cu_text[i], cu_img[i], 0};
    max_len = std::max(max_len, (int32_t)L);
    if (img > 0) {
      max_side = std::max(max_side, std::max(h, w));
      max_frames = std::max(max_frames, f);
    }
  }

  for (int i = 0; i < B; ++i) sinfo[i].img_row += (int32_t)nt;  // image rows follow all text rows
  pvj_plan* p = new (std::nothrow) pvj_plan();
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "out of host memory");
  const int D = desc->head_dim;
  p->desc = *desc;
  p->n_samples = B;
  p->n_tokens = T;
  p->max_len = max_len;
  p->n_text = (int32_t)nt;
  p->n_img = (int32_t)ni;
  p->rope_axes = axes;
  if (axes == 2) {
    p->rope_dims[0] = p->rope_dims[1] = D / 2;
    p->rope_dims[2] = 0;
  } else {
    p->rope_dims[0] = p->rope_dims[1] = (D - 16) / 2;
    p->rope_dims[2] = 16;
  }
  p->n_pos = std::max(1, std::max(max_side, axes == 3 ? max_frames : 0));
  p->n_pairs = D / 2;
  p->fwd_tile = fwd_tile_rows(desc->dtype, D);
  p->bwd_tile = bwd_tile_rows(desc->dtype, D);
  p->dev_meta = nullptr;
  p->dev_id = -1;

  std::vector<Item> split_tiles;
  int64_t n_slots = 0;
  std::vector<Item> fwd =
      build_items(len, desc->n_heads, p->fwd_tile, desc->dtype, true, &split_tiles, &n_slots);
  std::vector<Item> bwd =
      build_items(len, desc->n_heads, p->bwd_tile, desc->dtype, false, nullptr, &n_slots);
  std::vector<Item> dq =
      build_items(len, desc->n_heads, p->fwd_tile, desc->dtype, false, nullptr, &n_slots);
  // the slot index has 24 bits in an item
  if (n_slots >= (int64_t(1) << 23)) {
    delete p;
    return fail(PVJ_ERR_UNSUPPORTED, "%lld forward partial-result slots (limit %d)",
                (long long)n_slots, (1 << 23) - 1);
  }
  p->n_fwd = (int32_t)fwd.size();
  p->n_bwd = (int32_t)bwd.size();
  p->n_dq = (int32_t)dq.size();
  p->n_split = (int32_t)split_tiles.size();
  p->n_slots = (int32_t)n_slots;

  size_t off = 0;
  auto section = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 1), kMetaAlign);
    return o;
  };
  const size_t tab = (size_t)p->n_pos * p->n_pairs * sizeof(float);
  p->off_cu = section((B + 1) * sizeof(int32_t));
  p->off_cu_text = section((B + 1) * sizeof(int32_t));
  p->off_cu_img = section((B + 1) * sizeof(int32_t));
  p->off_cu_both = section((2 * B + 1) * sizeof(int32_t));
  p->off_sinfo = section(B * sizeof(SampleInfo));
  p->off_cos = section(tab);
  p->off_sin = section(tab);
  p->off_fwd = section(fwd.size() * sizeof(Item));
  p->off_bwd = section(bwd.size() * sizeof(Item));
  p->off_dq = section(dq.size() * sizeof(Item));
  p->off_split = section(split_tiles.size() * sizeof(Item));
  p->image_bytes = off;
  p->off_part = off;
  p->part_bytes = (size_t)n_slots * fwd_part_floats(D) * sizeof(float);
  p->image = static_cast<uint8_t*>(std::calloc(off, 1));
  if (!p->image) {
    delete p;
    return fail(PVJ_ERR_INVALID_ARG, "out of host memory");
  }
  std::memcpy(p->image + p->off_cu, cu.data(), (B + 1) * sizeof(int32_t));
  std::memcpy(p->image + p->off_cu_text, cu_text.data(), (B + 1) * sizeof(int32_t));
  std::memcpy(p->image + p->off_cu_img, cu_img.data(), (B + 1) * sizeof(int32_t));
  {
    int32_t* cb = reinterpret_cast<int32_t*>(p->image + p->off_cu_both);
    for (int i = 0; i <= B; ++i) cb[i] = cu_text[i];
    for (int i = 1; i <= B; ++i) cb[B + i] = cu_text[B] + cu_img[i];
  }
  if (B) std::memcpy(p->image + p->off_sinfo, sinfo.data(), B * sizeof(SampleInfo));
  // RoPE tables: pair k belongs to axis part a; as pair j of that part its angle
  // is pos * theta^(-j / (d_a/2)), computed in double and rounded to float once
  float* ct = reinterpret_cast<float*>(p->image + p->off_cos);
  float* st = reinterpret_cast<float*>(p->image + p->off_sin);
  int k = 0;
  for (int a = 0; a < 3; ++a) {
    const int half = p->rope_dims[a] / 2;
    for (int j = 0; j < half; ++j, ++k) {
      const double omega = std::pow((double)desc->rope_theta, -(double)j / (double)half);
      for (int pos = 0; pos < p->n_pos; ++pos) {
        const double phi = (double)pos * omega;
        ct[(size_t)pos * p->n_pairs + k] = (float)std::cos(phi);
        st[(size_t)pos * p->n_pairs + k] = (float)std::sin(phi);
      }
    }
  }
  if (!fwd.empty()) std::memcpy(p->image + p->off_fwd, fwd.data(), fwd.size() * sizeof(Item));
  if (!bwd.empty()) std::memcpy(p->image + p->off_bwd, bwd.data(), bwd.size() * sizeof(Item));
  if (!dq.empty()) std::memcpy(p->image + p->off_dq, dq.data(), dq.size() * sizeof(Item));
  if (!split_tiles.empty())
    std::memcpy(p->image + p->off_split, split_tiles.data(), split_tiles.size() * sizeof(Item));
  *out = p;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_plan_create(const pvj_sample_t* samples, int32_t n_samples,
                                     const pvj_plan_desc_t* desc, pvj_plan_t** out) {
  if (n_samples > 0 && !samples) return fail(PVJ_ERR_INVALID_ARG, "samples is NULL");
  std::vector<int32_t> v(4 * (size_t)std::max(n_samples, 0));
  for (int i = 0; i < n_samples; ++i) {
    v[4 * i] = samples[i].h_lat;
    v[4 * i + 1] = samples[i].w_lat;
    v[4 * i + 2] = samples[i].l_text;
    v[4 * i + 3] = 1;
  }
  return create_plan(v.data(), n_samples, 2, desc, out);
}

PVJ_API pvj_status_t pvj_plan_create_frames(const pvj_sample_frames_t* samples, int32_t n_samples,
                                            const pvj_plan_desc_t* desc, pvj_plan_t** out) {
  if (n_samples > 0 && !samples) return fail(PVJ_ERR_INVALID_ARG, "samples is NULL");
  std::vector<int32_t> v(4 * (size_t)std::max(n_samples, 0));
  for (int i = 0; i < n_samples; ++i) {
    v[4 * i] = samples[i].h_lat;
    v[4 * i + 1] = samples[i].w_lat;
    v[4 * i + 2] = samples[i].l_text;
    v[4 * i + 3] = samples[i].n_frames;
  }
  return create_plan(v.data(), n_samples, 3, desc, out);
}

PVJ_API pvj_status_t pvj_plan_info(const pvj_plan_t* p, int64_t* n_tokens, int32_t* max_len,
                                   const int32_t** cu_seqlens_host, size_t* meta_bytes) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (n_tokens) *n_tokens = p->n_tokens;
  if (max_len) *max_len = p->max_len;
  if (cu_seqlens_host) *cu_seqlens_host = host_section<int32_t>(p, p->off_cu);
  if (meta_bytes) *meta_bytes = p->image_bytes + p->part_bytes;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_plan_streams(const pvj_plan_t* p, int64_t* n_text, int64_t* n_image) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (n_text) *n_text = p->n_text;
  if (n_image) *n_image = p->n_img;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_plan_stream_major_rows(const pvj_plan_t* p, int32_t* rows,
                                                int64_t n) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (n != p->n_tokens)
    return fail(PVJ_ERR_INVALID_ARG, "rows holds %lld entries, the plan has %lld tokens",
                (long long)n, (long long)p->n_tokens);
  if (n > 0 && !rows) return fail(PVJ_ERR_INVALID_ARG, "rows is NULL");
  const pvj::SampleInfo* si = pvj::host_section<pvj::SampleInfo>(p, p->off_sinfo);
  for (int32_t i = 0; i < p->n_samples; ++i)
    for (int32_t j = 0; j < si[i].len; ++j)
      rows[si[i].start + j] = j < si[i].l_text ? si[i].text_row + j
                                               : si[i].img_row + (j - si[i].l_text);
  return PVJ_OK;
}

PVJ_API void pvj_plan_destroy(pvj_plan_t* p) {
  if (!p) return;
  std::free(p->image);
  delete p;
}

PVJ_API pvj_status_t pvj_plan_work_items(const pvj_plan_t* p, int32_t which,
                                         const int32_t** items, int32_t* n_items,
                                         int32_t* tile_rows) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (which < 0 || which > 3) return fail(PVJ_ERR_INVALID_ARG, "which must be 0, 1, 2 or 3");
  static const int kTileOf[4] = {0, 1, 0, 0};
  const size_t off[4] = {p->off_fwd, p->off_bwd, p->off_dq, p->off_split};
  const int32_t n[4] = {p->n_fwd, p->n_bwd, p->n_dq, p->n_split};
  if (items) *items = host_section<int32_t>(p, off[which]);
  if (n_items) *n_items = n[which];
  if (tile_rows) *tile_rows = kTileOf[which] ? p->bwd_tile : p->fwd_tile;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_plan_rope_table(const pvj_plan_t* p, const float** cos_tab,
                                         const float** sin_tab, int32_t* n_pos, int32_t* n_pairs) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (cos_tab) *cos_tab = host_section<float>(p, p->off_cos);
  if (sin_tab) *sin_tab = host_section<float>(p, p->off_sin);
  if (n_pos) *n_pos = p->n_pos;
  if (n_pairs) *n_pairs = p->n_pairs;
  return PVJ_OK;
}

PVJ_API pvj_status_t pvj_plan_rope_axes(const pvj_plan_t* p, int32_t* n_axes, int32_t dims[3]) {
  if (!p) return fail(PVJ_ERR_INVALID_ARG, "plan is NULL");
  if (n_axes) *n_axes = p->rope_axes;
  if (dims)
    for (int a = 0; a < 3; ++a) dims[a] = p->rope_dims[a];
  return PVJ_OK;
}

}  // extern "C"
