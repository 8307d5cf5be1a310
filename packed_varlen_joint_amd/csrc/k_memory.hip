// HBM-bound kernels: modality pack/unpack, standalone per-sample 2D RoPE and
// the attention-backward preprocess (Delta, pre-rotated Q' and K').
//
// Every kernel walks blocks of whole packed rows.  A row is H*D contiguous
// elements; the unit of work is 8 consecutive elements (one 16-byte bf16 or
// 32-byte fp32 access).  Consecutive lanes take consecutive units, so every
// wave reads and writes contiguous spans.  Because D/8 divides the block size,
// a thread always sees the same chunk of the head dimension, and the per-row
// bookkeeping (owning sample, RoPE position, cos/sin) is redone only when the
// thread's row changes.

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kThreads = 256;

// rows per block: about 48 KB of bf16 data (6 KB rows at H=24, D=128)
static int rows_per_block(const Meta& m, size_t elt) {
  const size_t row_bytes = (size_t)m.n_heads * m.head_dim * elt;
  size_t r = (48 * 1024) / row_bytes;
  return (int)(r < 1 ? 1 : (r > 64 ? 64 : r));
}

// ---------------------------------------------------------------------------
// pack / unpack: joint row j of sample i <-> text row cu_text[i] + j (j < t_i)
// or image row cu_img[i] + j - t_i.  Review page, "Native-Resolution MMDiT":
// text and image streams concatenated per sample for the joint attention.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void pack_kernel(Meta m, const T* __restrict__ src_text,
                                                        const T* __restrict__ src_img,
                                                        T* __restrict__ joint_out,
                                                        const T* __restrict__ joint_in,
                                                        T* __restrict__ dst_text,
                                                        T* __restrict__ dst_img, int rpb,
                                                        int unpack) {
  const int upr = m.n_heads * m.head_dim / 8;  // units per row
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  const int total = nrows * upr;
  int e = threadIdx.x;
  int row = e / upr, u = e - (e / upr) * upr;
  int cur = -1;
  size_t other = 0;  // element offset of the row in the text or image stream
  bool is_text = false;
  for (; e < total; e += kThreads) {
    if (row != cur) {
      cur = row;
      const int tok = row0 + row;
      const int i = find_sample(m.cu, m.n_samples, tok);
      const SampleInfo si = m.sinfo[i];
      const int j = tok - si.start;
      is_text = j < si.l_text;
      other = (size_t)(is_text ? m.cu_text[i] + j : m.cu_img[i] + j - si.l_text) * upr * 8;
    }
    const size_t jo = ((size_t)(row0 + row) * upr + u) * 8;
    const size_t so = other + (size_t)u * 8;
    if (!unpack) {
      store8<T>(joint_out + jo, load8<T>((is_text ? src_text : src_img) + so));
    } else {
      store8<T>((is_text ? dst_text : dst_img) + so, load8<T>(joint_in + jo));
    }
    u += kThreads;
    while (u >= upr) {
      u -= upr;
      ++row;
    }
  }
}

hipError_t launch_pack(const pvj_plan* p, const Meta& m, const void* text, const void* image,
                       void* joint, bool unpack, hipStream_t stream) {
  if (m.n_tokens == 0) return hipSuccess;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int rpb = rows_per_block(m, bf ? 2 : 4);
  const dim3 grid((m.n_tokens + rpb - 1) / rpb);
  if (bf) {
    typedef bf16 T;
    if (!unpack)
      pack_kernel<T><<<grid, kThreads, 0, stream>>>(m, (const T*)text, (const T*)image, (T*)joint,
                                                     nullptr, nullptr, nullptr, rpb, 0);
    else
      pack_kernel<T><<<grid, kThreads, 0, stream>>>(m, nullptr, nullptr, nullptr, (const T*)joint,
                                                     (T*)text, (T*)image, rpb, 1);
  } else {
    typedef float T;
    if (!unpack)
      pack_kernel<T><<<grid, kThreads, 0, stream>>>(m, (const T*)text, (const T*)image, (T*)joint,
                                                     nullptr, nullptr, nullptr, rpb, 0);
    else
      pack_kernel<T><<<grid, kThreads, 0, stream>>>(m, nullptr, nullptr, nullptr, (const T*)joint,
                                                     (T*)text, (T*)image, rpb, 1);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// standalone 2D RoPE (HF paper page "Highlights": per-sample 2D RoPE; review
// page, "Kernel fusion": RoPE application is a memory-bound op).
// ---------------------------------------------------------------------------
template <typename TIn, typename TOut, bool ROTATE>
__global__ __launch_bounds__(kThreads) void rope_kernel(Meta m, const TIn* x, TOut* y, int rpb,
                                                        int inverse) {
  const int cpr = m.head_dim / 8;              // chunks per head row
  const int upr = m.n_heads * cpr;             // units per packed row
  const int chunk = threadIdx.x % cpr;         // fixed for this thread (cpr | kThreads)
  const int half_chunks = m.head_dim / 16;
  const bool col = chunk >= half_chunks;
  const int k0 = (chunk - (col ? half_chunks : 0)) * 4;
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  const int total = nrows * upr;
  int e = threadIdx.x;
  int row = e / upr, u = e - (e / upr) * upr;
  int cur = -1;
  f32x4 cs = {1.f, 1.f, 1.f, 1.f}, sn = {0.f, 0.f, 0.f, 0.f};
  for (; e < total; e += kThreads) {
    if (ROTATE && row != cur) {
      cur = row;
      const int tok = row0 + row;
      const SampleInfo si = m.sinfo[find_sample(m.cu, m.n_samples, tok)];
      int r, c;
      token_pos(tok - si.start, si.l_text, si.w_lat, r, c);
      const int pos = col ? c : r;
      cs = *reinterpret_cast<const f32x4*>(m.cos_tab + (size_t)pos * m.n_freq + k0);
      sn = *reinterpret_cast<const f32x4*>(m.sin_tab + (size_t)pos * m.n_freq + k0);
      if (inverse) sn = -sn;
    }
    const size_t off = ((size_t)(row0 + row) * upr + u) * 8;
    f32x8 v = to_f32x8(load8<TIn>(x + off));
    if (ROTATE) {
      f32x8 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = v[2 * q], b = v[2 * q + 1];
        w[2 * q] = a * cs[q] - b * sn[q];
        w[2 * q + 1] = a * sn[q] + b * cs[q];
      }
      v = w;
    }
    store8<TOut>(y + off, from_f32x8<TOut>(v));
    u += kThreads;
    while (u >= upr) {
      u -= upr;
      ++row;
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
    rope_kernel<bf16, bf16, true><<<grid, kThreads, 0, stream>>>(m, (const bf16*)x, (bf16*)y, rpb,
                                                                 inverse);
  else
    rope_kernel<float, float, true><<<grid, kThreads, 0, stream>>>(m, (const float*)x, (float*)y,
                                                                   rpb, inverse);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// backward preprocess: Delta[h, t] = sum_d dO[t,h,d] * O[t,h,d] (the row term
// of the softmax backward).  With RoPE it also writes Q' = R Q and K' = R K
// once, so the backward kernels stream pre-rotated operands instead of
// rotating every tile again.  The D/8 lanes of one (token, head) are
// consecutive and reduce with xor shuffles.
// ---------------------------------------------------------------------------
template <typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(Meta m, const T* __restrict__ o,
                                                           const T* __restrict__ dout,
                                                           const T* __restrict__ q,
                                                           const T* __restrict__ k,
                                                           float* __restrict__ delta,
                                                           T* __restrict__ qr,
                                                           T* __restrict__ kr, int rpb) {
  const int cpr = m.head_dim / 8;
  const int upr = m.n_heads * cpr;
  const int chunk = threadIdx.x % cpr;  // fixed for this thread (cpr | kThreads)
  const int half_chunks = m.head_dim / 16;
  const bool col = chunk >= half_chunks;
  const int k0 = (chunk - (col ? half_chunks : 0)) * 4;
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  const int total = nrows * upr;
  int e = threadIdx.x;
  int row = e / upr, u = e - (e / upr) * upr;
  int cur = -1;
  f32x4 cs = {1.f, 1.f, 1.f, 1.f}, sn = {0.f, 0.f, 0.f, 0.f};
  for (; e < total; e += kThreads) {
    const size_t off = ((size_t)(row0 + row) * upr + u) * 8;
    const f32x8 a = to_f32x8(load8<T>(o + off));
    const f32x8 b = to_f32x8(load8<T>(dout + off));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += a[i] * b[i];
    for (int w = 1; w < cpr; w <<= 1) s += __shfl_xor(s, w, 64);
    if ((u % cpr) == 0) delta[(size_t)(u / cpr) * m.n_tokens + row0 + row] = s;
    if (ROPE) {
      if (row != cur) {
        cur = row;
        const int tok = row0 + row;
        const SampleInfo si = m.sinfo[find_sample(m.cu, m.n_samples, tok)];
        int pr, pc;
        token_pos(tok - si.start, si.l_text, si.w_lat, pr, pc);
        const size_t to = (size_t)(col ? pc : pr) * m.n_freq + k0;
        cs = *reinterpret_cast<const f32x4*>(m.cos_tab + to);
        sn = *reinterpret_cast<const f32x4*>(m.sin_tab + to);
      }
      const f32x8 x = to_f32x8(load8<T>(q + off));
      const f32x8 y = to_f32x8(load8<T>(k + off));
      f32x8 xr, yr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xr[2 * i] = x[2 * i] * cs[i] - x[2 * i + 1] * sn[i];
        xr[2 * i + 1] = x[2 * i] * sn[i] + x[2 * i + 1] * cs[i];
        yr[2 * i] = y[2 * i] * cs[i] - y[2 * i + 1] * sn[i];
        yr[2 * i + 1] = y[2 * i] * sn[i] + y[2 * i + 1] * cs[i];
      }
      store8<T>(qr + off, from_f32x8<T>(xr));
      store8<T>(kr + off, from_f32x8<T>(yr));
    }
    u += kThreads;
    while (u >= upr) {
      u -= upr;
      ++row;
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
