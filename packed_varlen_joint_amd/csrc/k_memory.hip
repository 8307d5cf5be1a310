// HBM-bound kernels: modality pack/unpack, standalone per-sample 2D RoPE and
// the attention-backward preprocess (Delta, pre-rotated Q' and K').
//
// Every kernel walks a block of whole packed rows.  A row is H*D contiguous
// elements and the unit of work is 8 consecutive elements (one 16-byte bf16 or
// 32-byte fp32 access).  The per-row bookkeeping (owning sample, position in
// the text or image stream, RoPE position) is computed once per row into LDS
// at block start.  Each thread then moves four units per batch, issuing the
// four loads before any store, so every thread keeps four independent memory
// requests in flight; consecutive lanes take consecutive units, so every wave
// touches contiguous spans.  Because D/8 divides the block size, a thread's
// unit always covers the same 8 dims of the head, so its RoPE axis and
// frequencies are fixed.

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kThreads = 256;
constexpr int kBatch = 4;          // units in flight per thread
constexpr int kMaxRowsPerBlock = 64;

// rows per block: about 12 KB of data (two 6 KB rows at H=24, D=128, bf16);
// measured on the training pack, 12 KB per block beats 6, 24 and 48 KB
// (pack 0.135 -> 0.125 ms against 48 KB)
static int rows_per_block(const Meta& m, size_t elt) {
  const size_t row_bytes = (size_t)m.n_heads * m.head_dim * elt;
  size_t r = (12 * 1024) / row_bytes;
  return (int)(r < 1 ? 1 : (r > (size_t)kMaxRowsPerBlock ? kMaxRowsPerBlock : r));
}

// RoPE position of packed row `tok`
__device__ __forceinline__ RopePos packed_pos(const Meta& m, int tok) {
  const SampleInfo si = m.sinfo[find_sample(m.cu, m.n_samples, tok)];
  return token_pos3(tok - si.start, si);
}

// ---------------------------------------------------------------------------
// pack / unpack: joint row j of sample i <-> text row cu_text[i] + j (j < t_i)
// or image row cu_img[i] + j - t_i.  Review page, "Native-Resolution MMDiT":
// text and image streams concatenated per sample for the joint attention.
// With ROPE the same pass also rotates every unit by the plan's RoPE (review
// page, "Kernel fusion": RoPE application is one of the memory-bound ops
// fused so the data is read and written once): the joint tensor then holds
// R x (pack) or the streams get R^T x (unpack with inverse), with the rounding
// of pvj_rope2d_apply.
// ---------------------------------------------------------------------------
template <typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void pack_kernel(Meta m, const T* __restrict__ src_text,
                                                        const T* __restrict__ src_img,
                                                        T* __restrict__ joint_out,
                                                        const T* __restrict__ joint_in,
                                                        T* __restrict__ dst_text,
                                                        T* __restrict__ dst_img, int rpb,
                                                        int unpack, int inverse) {
  __shared__ int s_row[kMaxRowsPerBlock];  // stream row; text rows are stored as -1 - row
  __shared__ int s_pos[ROPE ? 3 : 1][kMaxRowsPerBlock];  // row, col, frame (ROPE only)
  const int cpr = m.head_dim / 8;          // units per head row
  const int upr = m.n_heads * cpr;         // units per packed row
  const int chunk = threadIdx.x % cpr;     // fixed for this thread (cpr | kThreads)
  const int axis = ROPE ? unit_axis(chunk, m) : 0;
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  if ((int)threadIdx.x < nrows) {
    const int tok = row0 + threadIdx.x;
    const int i = find_sample(m.cu, m.n_samples, tok);
    const SampleInfo si = m.sinfo[i];
    const int j = tok - si.start;
    s_row[threadIdx.x] = j < si.l_text ? -1 - (m.cu_text[i] + j) : m.cu_img[i] + j - si.l_text;
    if (ROPE) {
      const RopePos rp = token_pos3(j, si);
      s_pos[0][threadIdx.x] = rp.r;
      s_pos[1][threadIdx.x] = rp.c;
      s_pos[2][threadIdx.x] = rp.f;
    }
  }
  __syncthreads();
  const int total = nrows * upr;
  for (int e0 = threadIdx.x; e0 < total; e0 += kBatch * kThreads) {
    typename Vec8<T>::type v[kBatch];
    size_t jo[kBatch], so[kBatch];
    bool txt[kBatch];
    int pos[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = e0 + b * kThreads;
      const int row = e / upr, u = e - row * upr;
      const int sr = e < total ? s_row[row] : 0;
      txt[b] = sr < 0;
      jo[b] = ((size_t)(row0 + row) * upr + u) * 8;
      so[b] = ((size_t)(sr < 0 ? -1 - sr : sr) * upr + u) * 8;
      if (ROPE) pos[b] = e < total ? s_pos[axis][row] : 0;
      if (e < total)
        v[b] = unpack ? load8<T>(joint_in + jo[b]) : load8<T>((txt[b] ? src_text : src_img) + so[b]);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (e0 + b * kThreads < total) {
        if (ROPE) v[b] = from_f32x8<T>(rope_unit(to_f32x8(v[b]), chunk, pos[b], m, inverse != 0));
        if (unpack)
          store8<T>((txt[b] ? dst_text : dst_img) + so[b], v[b]);
        else
          store8<T>(joint_out + jo[b], v[b]);
      }
    }
  }
}

hipError_t launch_pack(const pvj_plan* p, const Meta& m, const void* text, const void* image,
                       void* joint, bool unpack, bool rope, bool inverse, hipStream_t stream) {
  if (m.n_tokens == 0) return hipSuccess;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int rpb = rows_per_block(m, bf ? 2 : 4);
  const dim3 grid((m.n_tokens + rpb - 1) / rpb);
  const int inv = inverse ? 1 : 0;
#define PVJ_PACK(TT, RR)                                                                         do {                                                                                             if (!unpack)                                                                                     pack_kernel<TT, RR><<<grid, kThreads, 0, stream>>>(m, (const TT*)text, (const TT*)image,                                                          (TT*)joint, nullptr, nullptr,                                                                  nullptr, rpb, 0, inv);                    else                                                                                             pack_kernel<TT, RR><<<grid, kThreads, 0, stream>>>(m, nullptr, nullptr, nullptr,                                                                  (const TT*)joint, (TT*)text,                                                                   (TT*)image, rpb, 1, inv);               } while (0)
  if (bf) {
    if (rope) PVJ_PACK(bf16, true); else PVJ_PACK(bf16, false);
  } else {
    if (rope) PVJ_PACK(float, true); else PVJ_PACK(float, false);
  }
#undef PVJ_PACK
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// standalone per-sample RoPE (HF paper page "Highlights": per-sample 2D RoPE;
// review page, "Kernel fusion": RoPE application is a memory-bound op; the
// editing plans' third, frame axis comes from the same tables).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(Meta m, const T* x, T* y, int rpb,
                                                        int inverse) {
  __shared__ int s_pos[3][kMaxRowsPerBlock];  // row, col, frame of each row's token
  const int cpr = m.head_dim / 8;              // units per head row
  const int upr = m.n_heads * cpr;             // units per packed row
  const int chunk = threadIdx.x % cpr;         // fixed for this thread (cpr | kThreads)
  const int axis = unit_axis(chunk, m);
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  if ((int)threadIdx.x < nrows) {
    const RopePos rp = packed_pos(m, row0 + threadIdx.x);
    s_pos[0][threadIdx.x] = rp.r;
    s_pos[1][threadIdx.x] = rp.c;
    s_pos[2][threadIdx.x] = rp.f;
  }
  __syncthreads();
  const int total = nrows * upr;
  for (int e0 = threadIdx.x; e0 < total; e0 += kBatch * kThreads) {
    f32x8 v[kBatch];
    size_t off[kBatch];
    int pos[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = e0 + b * kThreads;
      const int row = e / upr, u = e - row * upr;
      off[b] = ((size_t)(row0 + row) * upr + u) * 8;
      pos[b] = e < total ? s_pos[axis][row] : 0;
      if (e < total) v[b] = to_f32x8(load8<T>(x + off[b]));
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (e0 + b * kThreads < total)
        store8<T>(y + off[b], from_f32x8<T>(rope_unit(v[b], chunk, pos[b], m, inverse != 0)));
    }
  }
}

hipError_t launch_rope2d(const pvj_plan* p, const Meta& m, const void* x, void* y, bool inverse,
                         hipStream_t stream) {
  if (m.n_tokens == 0) return hipSuccess;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int rpb = rows_per_block(m, bf ? 2 : 4);
  const dim3 grid((m.n_tokens + rpb - 1) / rpb);
  if (bf)
    rope_kernel<bf16><<<grid, kThreads, 0, stream>>>(m, (const bf16*)x, (bf16*)y, rpb, inverse);
  else
    rope_kernel<float><<<grid, kThreads, 0, stream>>>(m, (const float*)x, (float*)y, rpb, inverse);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// backward preprocess: Delta[h, t] = sum_d dO[t,h,d] * O[t,h,d] (the row term
// of the softmax backward).  With RoPE it also writes Q' = R Q and K' = R K
// once, so the backward kernels stream pre-rotated operands instead of
// rotating every tile again.  The D/8 lanes of one (token, head) are
// consecutive and reduce with xor shuffles (all lanes of a group are in or
// out of range together: totals are multiples of D/8 and batches start at
// multiples of the block size).
// ---------------------------------------------------------------------------
template <typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(Meta m, const T* __restrict__ o,
                                                           const T* __restrict__ dout,
                                                           const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           float* __restrict__ delta,
                                                           T* __restrict__ qr,
                                                           T* __restrict__ kr, int rpb) {
  __shared__ int s_pos[3][kMaxRowsPerBlock];
  const int cpr = m.head_dim / 8;
  const int upr = m.n_heads * cpr;
  const int chunk = threadIdx.x % cpr;
  const int axis = unit_axis(chunk, m);
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  if (ROPE && (int)threadIdx.x < nrows) {
    const RopePos rp = packed_pos(m, row0 + threadIdx.x);
    s_pos[0][threadIdx.x] = rp.r;
    s_pos[1][threadIdx.x] = rp.c;
    s_pos[2][threadIdx.x] = rp.f;
  }
  if (ROPE) __syncthreads();
  const int total = nrows * upr;
  for (int e0 = threadIdx.x; e0 < total; e0 += kBatch * kThreads) {
    f32x8 a[kBatch], g[kBatch], x[kBatch], y[kBatch];
    size_t off[kBatch];
    int rows[kBatch], us[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int e = e0 + b * kThreads;
      rows[b] = e / upr;
      us[b] = e - rows[b] * upr;
      off[b] = ((size_t)(row0 + rows[b]) * upr + us[b]) * 8;
      if (e < total) {
        a[b] = to_f32x8(load8<T>(o + off[b]));
        g[b] = to_f32x8(load8<T>(dout + off[b]));
        if (ROPE) {
          x[b] = to_f32x8(load8<T>(q + off[b]));
          y[b] = to_f32x8(load8<T>(k + off[b]));
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (e0 + b * kThreads >= total) continue;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s += a[b][i] * g[b][i];
      for (int w = 1; w < cpr; w <<= 1) s += __shfl_xor(s, w, 64);
      if ((us[b] % cpr) == 0)
        delta[(size_t)(us[b] / cpr) * m.n_tokens + row0 + rows[b]] = s;
      if (ROPE) {
        const int pos = s_pos[axis][rows[b]];
        store8<T>(qr + off[b], from_f32x8<T>(rope_unit(x[b], chunk, pos, m, false)));
        store8<T>(kr + off[b], from_f32x8<T>(rope_unit(y[b], chunk, pos, m, false)));
      }
    }
  }
}

hipError_t launch_bwd_pre(const pvj_plan* p, const Meta& m, const void* o, const void* dout,
                          const void* q, const void* k, float* delta, void* qr, void* kr,
                          bool rope, hipStream_t stream) {
  if (m.n_tokens == 0) return hipSuccess;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int rpb = rows_per_block(m, bf ? 2 : 4);
  const dim3 grid((m.n_tokens + rpb - 1) / rpb);
#define PVJ_PRE(TT, RR)                                                                      \
  bwd_pre_kernel<TT, RR><<<grid, kThreads, 0, stream>>>(m, (const TT*)o, (const TT*)dout,    \
                                                        (const TT*)q, (const TT*)k, delta,   \
                                                        (TT*)qr, (TT*)kr, rpb)
  if (bf) {
    if (rope) PVJ_PRE(bf16, true); else PVJ_PRE(bf16, false);
  } else {
    if (rope) PVJ_PRE(float, true); else PVJ_PRE(float, false);
  }
#undef PVJ_PRE
  return hipGetLastError();
}

}  // namespace pvj
