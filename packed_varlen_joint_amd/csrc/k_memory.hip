// HBM-bound kernels: modality pack/unpack and standalone per-sample 2D RoPE
// (also the attention backward's rotation of Q and K with RoPE on load).
//
// Every kernel walks a block of whole packed rows.  A row is H*D contiguous
// elements and the unit of work is 8 consecutive elements (one 16-byte bf16 or
// 32-byte fp32 access).  The per-row bookkeeping (owning sample, position in
// the text or image stream, RoPE position) is computed once per row into LDS
// at block start; the kernels that rotate issue their first batch's loads
// before it (the lookup is a chain of dependent loads) and load every unit's
// RoPE table entries before rotating any.  Each thread moves up to four units
// per batch, issuing the loads before any store, so every thread keeps
// several independent memory requests in flight; consecutive lanes take
// consecutive units, so every wave touches contiguous spans.  Because D/8
// divides the block size, a thread's unit always covers the same 8 dims of
// the head, so its RoPE axis and frequencies are fixed.

#include <algorithm>

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kThreads = 256;
constexpr int kMaxBatch = 4;       // units in flight per thread, at most
constexpr int kMaxRowsPerBlock = 64;

// Block shape: `rows` whole packed rows per block and `batch` units (8
// elements) in flight per thread, so that one pass of batch x 256 units covers
// the block's rows with as few idle lanes as possible, at about 12 KB per
// block (measured on the training pack: 12 KB beats 6, 24 and 48 KB per block,
// and 2 rows x 384 units in 3 units per thread (no idle lane) beat 4 per
// thread (a quarter of the lanes idle): RoPE 0.134 -> 0.124 ms with the
// non-temporal stores below).
struct BlockShape {
  int rows, batch;
};
static BlockShape block_shape(const Meta& m, size_t elt) {
  const int upr = m.n_heads * m.head_dim / 8;  // units per row
  const size_t row_bytes = (size_t)upr * 8 * elt;
  int target = (int)((12 * 1024) / row_bytes);
  target = target < 1 ? 1 : (target > kMaxRowsPerBlock ? kMaxRowsPerBlock : target);
  BlockShape best = {target, kMaxBatch};
  double best_idle = 2.0;
  // rows from half to twice the target; a block needing more than one pass
  // of kMaxBatch units per thread keeps kMaxBatch (the kernels loop)
  for (int r = (target + 1) / 2; r <= 2 * target && r <= kMaxRowsPerBlock; ++r) {
    const long u = (long)r * upr;
    const int b = (int)((u + kThreads - 1) / kThreads);
    const int bb = b > kMaxBatch ? kMaxBatch : b;
    const long slots = (long)kThreads * bb * ((u + (long)kThreads * bb - 1) / ((long)kThreads * bb));
    const double idle = 1.0 - (double)u / (double)slots + 0.01 * (r > target ? r - target : target - r);
    if (idle < best_idle) {
      best_idle = idle;
      best = {r, bb};
    }
  }
  return best;
}

// outputs are written once and not read again by this kernel: non-temporal
// stores (measured: pack 0.121 -> 0.113 ms, RoPE 0.145 -> 0.134 ms)
template <typename T>
__device__ __forceinline__ void store8_nt(T* p, typename Vec8<T>::type v) {
  __builtin_nontemporal_store(v, reinterpret_cast<typename Vec8<T>::type*>(p));
}

// RoPE position of packed row `tok`
__device__ __forceinline__ RopePos packed_pos(const Meta& m, int tok) {
  const SampleInfo si = m.sinfo[find_sample(m.cu, m.n_samples, tok)];
  return token_pos3(tok - si.start, si);
}
// RoPE position of row `row` of a stream-major tensor (all text rows, then
// all image rows): text tokens sit at (0, 0, 0)
__device__ __forceinline__ RopePos stream_major_pos(const Meta& m, int row) {
  if (row < m.n_text) return RopePos{0, 0, 0};
  const int q = row - m.n_text;
  const int i = find_sample(m.cu_img, m.n_samples, q);
  const SampleInfo si = m.sinfo[i];
  return token_pos3(si.l_text + (q - m.cu_img[i]), si);
}

// ---------------------------------------------------------------------------
// pack / unpack: joint row j of sample i <-> text row cu_text[i] + j (j < t_i)
// or image row cu_img[i] + j - t_i.  Review page, "Native-Resolution MMDiT":
// text and image streams concatenated per sample for the joint attention.
// ---------------------------------------------------------------------------
template <typename T, int kBatch>
__global__ __launch_bounds__(kThreads) void pack_kernel(Meta m, const T* __restrict__ src_text,
                                                        const T* __restrict__ src_img,
                                                        T* __restrict__ joint_out,
                                                        const T* __restrict__ joint_in,
                                                        T* __restrict__ dst_text,
                                                        T* __restrict__ dst_img, int rpb,
                                                        int unpack) {
  __shared__ int s_row[kMaxRowsPerBlock];  // stream row; text rows are stored as -1 - row
  const int upr = m.n_heads * m.head_dim / 8;  // units per packed row
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  if ((int)threadIdx.x < nrows) {
    const int tok = row0 + threadIdx.x;
    const int i = find_sample(m.cu, m.n_samples, tok);
    const SampleInfo si = m.sinfo[i];
    const int j = tok - si.start;
    s_row[threadIdx.x] = j < si.l_text ? -1 - (m.cu_text[i] + j) : m.cu_img[i] + j - si.l_text;
  }
  __syncthreads();
  const int total = nrows * upr;
  for (int e0 = threadIdx.x; e0 < total; e0 += kBatch * kThreads) {
    typename Vec8<T>::type v[kBatch];
    size_t jo[kBatch], so[kBatch];
    bool txt[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = e0 + b * kThreads;
      const int row = e / upr, u = e - row * upr;
      const int sr = e < total ? s_row[row] : 0;
      txt[b] = sr < 0;
      jo[b] = ((size_t)(row0 + row) * upr + u) * 8;
      so[b] = ((size_t)(sr < 0 ? -1 - sr : sr) * upr + u) * 8;
      if (e < total)
        v[b] = unpack ? load8<T>(joint_in + jo[b]) : load8<T>((txt[b] ? src_text : src_img) + so[b]);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (e0 + b * kThreads < total) {
        if (unpack)
          store8_nt<T>((txt[b] ? dst_text : dst_img) + so[b], v[b]);
        else
          store8_nt<T>(joint_out + jo[b], v[b]);
      }
    }
  }
}

// The same with every unit rotated by the plan's RoPE in the pass (review
// page, "Kernel fusion": RoPE application is one of the memory-bound ops
// fused so the data is read and written once): the joint tensor then holds
// R x (pack) or the streams get R^T x (unpack with inverse), with the rounding
// of pvj_rope2d_apply.  The sample of the block's first row is found with
// scalar loads (uniform); when every row of the block lies in it (`one`, the
// common case) each thread forms its units' stream rows itself, so the first
// batch's loads go out before the rows' positions are looked up and passed
// through LDS, and every unit's table entries are loaded before any rotation.
// Measured on the training pack: pack with RoPE 0.1145 -> 0.1115 ms.  (The
// plain pack keeps the per-row lookup through LDS above: with this structure
// it measured 3% slower.)
template <typename T, bool UNPACK, int kBatch>
__global__ __launch_bounds__(kThreads) void pack_rope_kernel(
    Meta m, const T* __restrict__ src_text, const T* __restrict__ src_img,
    T* __restrict__ joint_out, const T* __restrict__ joint_in, T* __restrict__ dst_text,
    T* __restrict__ dst_img, int rpb, int inverse) {
  typedef typename Vec8<T>::type V8;
  __shared__ int s_row[kMaxRowsPerBlock];     // stream row; text rows are stored as -1 - row
  __shared__ int s_pos[3][kMaxRowsPerBlock];  // row, col, frame of each row's token
  const int cpr = m.head_dim / 8;          // units per head row
  const int upr = m.n_heads * cpr;         // units per packed row
  const int chunk = threadIdx.x % cpr;     // fixed for this thread (cpr | kThreads)
  const int axis = unit_axis(chunk, m);
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  const int total = nrows * upr;
  const int s0 = find_sample(m.cu, m.n_samples, row0);
  const SampleInfo si0 = m.sinfo[s0];
  const int ct0 = m.cu_text[s0], ci0 = m.cu_img[s0];
  const bool one = row0 + nrows <= si0.start + si0.len;
  auto stream_row = [&](int j, int ct, int ci, int lt) { return j < lt ? -1 - (ct + j) : ci + j - lt; };
  V8 v[kBatch] = {};
  size_t jo[kBatch], so[kBatch];
  bool txt[kBatch];
  int rw[kBatch];
  // the stream side of a unit (its stream and offset there)
  auto stream_side = [&](int b, int e, int row, int u, bool lds) {
    const int sr = e >= total ? 0
                   : lds      ? s_row[row]
                              : stream_row(row0 + row - si0.start, ct0, ci0, si0.l_text);
    txt[b] = sr < 0;
    so[b] = ((size_t)(sr < 0 ? -1 - sr : sr) * upr + u) * 8;
  };
  auto fetch = [&](int e0, bool lds) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = e0 + b * kThreads;
      const int row = e / upr, u = e - row * upr;
      rw[b] = row;
      jo[b] = ((size_t)(row0 + row) * upr + u) * 8;
      if constexpr (UNPACK) {  // the joint-side loads need no lookup: they go out first
        if (e < total) v[b] = load8<T>(joint_in + jo[b]);
        stream_side(b, e, row, u, lds);
      } else {
        stream_side(b, e, row, u, lds);
        if (e < total) v[b] = load8<T>((txt[b] ? src_text : src_img) + so[b]);
      }
    }
  };
  if (one) fetch(threadIdx.x, false);
  if ((int)threadIdx.x < nrows) {
    const int tok = row0 + threadIdx.x;
    // (each branch forms its values itself, so the rare branch's vector loads
    // are waited for inside it, not where the branches join)
    if (tok < si0.start + si0.len) {
      const int j = tok - si0.start;
      s_row[threadIdx.x] = stream_row(j, ct0, ci0, si0.l_text);
      const RopePos rp = token_pos3(j, si0);
      s_pos[0][threadIdx.x] = rp.r;
      s_pos[1][threadIdx.x] = rp.c;
      s_pos[2][threadIdx.x] = rp.f;
    } else {
      const int i = find_sample(m.cu, m.n_samples, tok);
      const SampleInfo si = m.sinfo[i];
      const int j = tok - si.start;
      s_row[threadIdx.x] = stream_row(j, m.cu_text[i], m.cu_img[i], si.l_text);
      const RopePos rp = token_pos3(j, si);
      s_pos[0][threadIdx.x] = rp.r;
      s_pos[1][threadIdx.x] = rp.c;
      s_pos[2][threadIdx.x] = rp.f;
    }
  }
  __syncthreads();
  for (int e0 = threadIdx.x; e0 < total; e0 += kBatch * kThreads) {
    if (!one || e0 != (int)threadIdx.x) fetch(e0, !one);
    // every unit's table entries before any rotation; out-of-range units use
    // a valid row's position (branch-free) and are not stored
    f32x4 cs[kBatch], sn[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const size_t to = (size_t)s_pos[axis][min(rw[b], nrows - 1)] * m.n_pairs + 4 * chunk;
      cs[b] = *reinterpret_cast<const f32x4*>(m.cos_tab + to);
      sn[b] = *reinterpret_cast<const f32x4*>(m.sin_tab + to);
    }
    __builtin_amdgcn_sched_barrier(0);
    V8 o[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      o[b] = from_f32x8<T>(rope_rotate(to_f32x8(v[b]), cs[b], sn[b], inverse != 0));
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (e0 + b * kThreads < total) {
        if constexpr (UNPACK)
          store8_nt<T>((txt[b] ? dst_text : dst_img) + so[b], o[b]);
        else
          store8_nt<T>(joint_out + jo[b], o[b]);
      }
    }
  }
}

template <typename T, bool ROPE, int B>
static void pack_t(const Meta& m, dim3 grid, int rpb, const void* text, const void* image,
                   void* joint, bool unpack, int inv, hipStream_t stream) {
  if (!ROPE) {
    if (!unpack)
      pack_kernel<T, B><<<grid, kThreads, 0, stream>>>(
          m, (const T*)text, (const T*)image, (T*)joint, nullptr, nullptr, nullptr, rpb, 0);
    else
      pack_kernel<T, B><<<grid, kThreads, 0, stream>>>(
          m, nullptr, nullptr, nullptr, (const T*)joint, (T*)text, (T*)image, rpb, 1);
  } else if (!unpack) {
    pack_rope_kernel<T, false, B><<<grid, kThreads, 0, stream>>>(
        m, (const T*)text, (const T*)image, (T*)joint, nullptr, nullptr, nullptr, rpb, inv);
  } else {
    pack_rope_kernel<T, true, B><<<grid, kThreads, 0, stream>>>(
        m, nullptr, nullptr, nullptr, (const T*)joint, (T*)text, (T*)image, rpb, inv);
  }
}
template <typename T, bool ROPE>
static void pack_b(const Meta& m, BlockShape bs, dim3 grid, const void* text, const void* image,
                   void* joint, bool unpack, int inv, hipStream_t stream) {
  switch (bs.batch) {
    case 1: pack_t<T, ROPE, 1>(m, grid, bs.rows, text, image, joint, unpack, inv, stream); break;
    case 2: pack_t<T, ROPE, 2>(m, grid, bs.rows, text, image, joint, unpack, inv, stream); break;
    case 3: pack_t<T, ROPE, 3>(m, grid, bs.rows, text, image, joint, unpack, inv, stream); break;
    default: pack_t<T, ROPE, 4>(m, grid, bs.rows, text, image, joint, unpack, inv, stream);
  }
}

hipError_t launch_pack(const pvj_plan* p, const Meta& m, const void* text, const void* image,
                       void* joint, bool unpack, bool rope, bool inverse, hipStream_t stream) {
  if (m.n_tokens == 0) return hipSuccess;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const BlockShape bs = block_shape(m, bf ? 2 : 4);
  const dim3 grid((m.n_tokens + bs.rows - 1) / bs.rows);
  const int inv = inverse ? 1 : 0;
  if (bf) {
    if (rope) pack_b<bf16, true>(m, bs, grid, text, image, joint, unpack, inv, stream);
    else pack_b<bf16, false>(m, bs, grid, text, image, joint, unpack, inv, stream);
  } else {
    if (rope) pack_b<float, true>(m, bs, grid, text, image, joint, unpack, inv, stream);
    else pack_b<float, false>(m, bs, grid, text, image, joint, unpack, inv, stream);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// standalone per-sample RoPE (HF paper page "Highlights": per-sample 2D RoPE;
// review page, "Kernel fusion": RoPE application is a memory-bound op; the
// editing plans' third, frame axis comes from the same tables).
// ---------------------------------------------------------------------------
template <typename T, int kBatch, bool SM>
__global__ __launch_bounds__(kThreads) void rope_kernel(Meta m, const T* x, T* y, int rpb,
                                                        int inverse) {
  typedef typename Vec8<T>::type V8;
  __shared__ int s_pos[3][kMaxRowsPerBlock];  // row, col, frame of each row's token
  const int cpr = m.head_dim / 8;              // units per head row
  const int upr = m.n_heads * cpr;             // units per packed row
  const int chunk = threadIdx.x % cpr;         // fixed for this thread (cpr | kThreads)
  const int axis = unit_axis(chunk, m);
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  const int total = nrows * upr;
  V8 v[kBatch] = {};
  size_t off[kBatch];
  int rw[kBatch];
  auto load = [&](int e0) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = e0 + b * kThreads;
      const int row = e / upr, u = e - row * upr;
      rw[b] = row;
      off[b] = ((size_t)(row0 + row) * upr + u) * 8;
      if (e < total) v[b] = load8<T>(x + off[b]);
    }
  };
  // The first batch's loads go out before the rows' RoPE positions are looked
  // up.  The lookup starts from the sample of the block's first row, found
  // with scalar loads (uniform), whose wait does not wait for the data loads
  // as a vector load's would; rows past that sample search on their own.
  // Measured on the training pack: 0.123 -> 0.112 ms.
  load(threadIdx.x);
  const int32_t* cu = SM ? m.cu_img : m.cu;
  const int q0 = SM ? row0 - m.n_text : row0;  // SM: image-stream row (text rows: no lookup)
  const int s0 = q0 >= 0 ? find_sample(cu, m.n_samples, q0) : 0;
  const SampleInfo si0 = m.sinfo[s0];
  const int c0 = cu[s0], c1 = cu[s0 + 1];
  if ((int)threadIdx.x < nrows) {
    const int q = q0 + (int)threadIdx.x;
    RopePos rp = {0, 0, 0};
    // (each branch forms its positions itself, so the rare branch's vector
    // loads are waited for inside it, not where the branches join)
    if (q >= 0 && q0 >= 0 && q < c1) {  // (joint rows are never negative)
      rp = token_pos3(SM ? si0.l_text + (q - c0) : q - si0.start, si0);
    } else if (q >= 0) {  // a row of a later sample
      const int i = find_sample(cu, m.n_samples, q);
      const SampleInfo si = m.sinfo[i];
      rp = token_pos3(SM ? si.l_text + (q - cu[i]) : q - si.start, si);
    }
    s_pos[0][threadIdx.x] = rp.r;
    s_pos[1][threadIdx.x] = rp.c;
    s_pos[2][threadIdx.x] = rp.f;
  }
  __syncthreads();
  for (int e0 = threadIdx.x; e0 < total; e0 += kBatch * kThreads) {
    if (e0 != (int)threadIdx.x) load(e0);
    // every unit's rotation (and so its table loads) before the first store:
    // the tables could alias y for the compiler, which would otherwise wait
    // out one table lookup per store
    // every unit's table entries are loaded before any unit is rotated, out-
    // of-range units with a valid row's position (branch-free, so the table
    // loads are not waited for one at a time; those units are not stored)
    f32x4 cs[kBatch], sn[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const size_t to = (size_t)s_pos[axis][min(rw[b], nrows - 1)] * m.n_pairs + 4 * chunk;
      cs[b] = *reinterpret_cast<const f32x4*>(m.cos_tab + to);
      sn[b] = *reinterpret_cast<const f32x4*>(m.sin_tab + to);
    }
    __builtin_amdgcn_sched_barrier(0);
    V8 o[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      o[b] = from_f32x8<T>(rope_rotate(to_f32x8(v[b]), cs[b], sn[b], inverse != 0));
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (e0 + b * kThreads < total) store8_nt<T>(y + off[b], o[b]);
  }
}

template <typename T, bool SM>
static void rope_b(const Meta& m, BlockShape bs, dim3 grid, const void* x, void* y, int inv,
                   hipStream_t stream) {
  const T* xi = (const T*)x;
  T* yo = (T*)y;
  switch (bs.batch) {
    case 1: rope_kernel<T, 1, SM><<<grid, kThreads, 0, stream>>>(m, xi, yo, bs.rows, inv); break;
    case 2: rope_kernel<T, 2, SM><<<grid, kThreads, 0, stream>>>(m, xi, yo, bs.rows, inv); break;
    case 3: rope_kernel<T, 3, SM><<<grid, kThreads, 0, stream>>>(m, xi, yo, bs.rows, inv); break;
    default: rope_kernel<T, 4, SM><<<grid, kThreads, 0, stream>>>(m, xi, yo, bs.rows, inv);
  }
}

hipError_t launch_rope2d(const pvj_plan* p, const Meta& m, const void* x, void* y, bool inverse,
                         bool sm, hipStream_t stream) {
  if (m.n_tokens == 0) return hipSuccess;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const BlockShape bs = block_shape(m, bf ? 2 : 4);
  const dim3 grid((m.n_tokens + bs.rows - 1) / bs.rows);
  const int inv = inverse ? 1 : 0;
  if (bf) {
    if (sm) rope_b<bf16, true>(m, bs, grid, x, y, inv, stream);
    else rope_b<bf16, false>(m, bs, grid, x, y, inv, stream);
  } else {
    if (sm) rope_b<float, true>(m, bs, grid, x, y, inv, stream);
    else rope_b<float, false>(m, bs, grid, x, y, inv, stream);
  }
  return hipGetLastError();
}

}  // namespace pvj
