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
// With ROPE the same pass also rotates every unit by the plan's RoPE (review
// page, "Kernel fusion": RoPE application is one of the memory-bound ops
// fused so the data is read and written once): the joint tensor then holds
// R x (pack) or the streams get R^T x (unpack with inverse), with the rounding
// of pvj_rope2d_apply.
// ---------------------------------------------------------------------------
template <typename T, bool ROPE, int kBatch>
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
          store8_nt<T>((txt[b] ? dst_text : dst_img) + so[b], v[b]);
        else
          store8_nt<T>(joint_out + jo[b], v[b]);
      }
    }
  }
}

template <typename T, bool ROPE, int B>
static void pack_t(const Meta& m, dim3 grid, int rpb, const void* text, const void* image,
                   void* joint, bool unpack, int inv, hipStream_t stream) {
  if (!unpack)
    pack_kernel<T, ROPE, B><<<grid, kThreads, 0, stream>>>(
        m, (const T*)text, (const T*)image, (T*)joint, nullptr, nullptr, nullptr, rpb, 0, inv);
  else
    pack_kernel<T, ROPE, B><<<grid, kThreads, 0, stream>>>(
        m, nullptr, nullptr, nullptr, (const T*)joint, (T*)text, (T*)image, rpb, 1, inv);
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
  __shared__ int s_pos[3][kMaxRowsPerBlock];  // row, col, frame of each row's token
  const int cpr = m.head_dim / 8;              // units per head row
  const int upr = m.n_heads * cpr;             // units per packed row
  const int chunk = threadIdx.x % cpr;         // fixed for this thread (cpr | kThreads)
  const int axis = unit_axis(chunk, m);
  const int row0 = blockIdx.x * rpb;
  const int nrows = min(rpb, m.n_tokens - row0);
  if ((int)threadIdx.x < nrows) {
    const RopePos rp =
        SM ? stream_major_pos(m, row0 + threadIdx.x) : packed_pos(m, row0 + threadIdx.x);
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
        store8_nt<T>(y + off[b], from_f32x8<T>(rope_unit(v[b], chunk, pos[b], m, inverse != 0)));
    }
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

// ---------------------------------------------------------------------------
// backward preprocess: Delta[h, t] = sum_d dO[t,h,d] * O[t,h,d] (the row term
// of the softmax backward).  With RoPE it also writes Q' = R Q and K' = R K
// once, so the backward kernels stream pre-rotated operands instead of
// rotating every tile again.  The D/8 lanes of one (token, head) are
// consecutive and reduce with xor shuffles (all lanes of a group are in or
// out of range together: totals are multiples of D/8 and batches start at
// multiples of the block size).
// ---------------------------------------------------------------------------
template <typename T, bool ROPE, int kBatch>
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
        store8_nt<T>(qr + off[b], from_f32x8<T>(rope_unit(x[b], chunk, pos, m, false)));
        store8_nt<T>(kr + off[b], from_f32x8<T>(rope_unit(y[b], chunk, pos, m, false)));
      }
    }
  }
}

// Delta alone (no RoPE): a plain streaming read of O and dO.  Each wave takes
// NB consecutive groups of 64 units; the D/8 lanes of one (token, head) row
// are consecutive and sum their dot products with DPP inside the 16-lane row
// (no LDS); one lane per (token, head) stores Delta[h, t].  No per-row
// bookkeeping: Delta does not depend on the sample.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Delta = rowsum(O * dO) per (token, head) without RoPE: a block takes `tb`
// consecutive tokens with all their heads (tb * H rows of D, contiguous in
// HBM).  Each wave streams groups of 64 units (64 / (D/8) consecutive rows,
// one 16-byte unit per lane) NB groups at a time, the next NB groups' loads
// in flight while the current ones are reduced (DPP sums inside the row's
// lanes), and leaves the row sums in LDS; the block then writes Delta [H, T]
// as one run of tb floats per head (scattered 4-byte stores had been written
// back as partial lines: 3.6x the bytes).
template <typename T, int D, int NB>
__global__ __launch_bounds__(kThreads) void delta_kernel(const T* __restrict__ o,
                                                         const T* __restrict__ dout,
                                                         float* __restrict__ delta, int n_tokens,
                                                         int n_heads, int tb) {
  typedef typename Vec8<T>::type V8;
  constexpr int UPH = D / 8;     // units per (token, head) row: 16 or 8
  constexpr int RPG = 64 / UPH;  // rows per group of 64 units
  extern __shared__ float red[];  // [tb * n_heads] row sums, in row order
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * tb;
  const int nt = min(tb, n_tokens - t0);
  const int rows = nt * n_heads;
  const int groups = (rows + RPG - 1) / RPG;
  const size_t base = (size_t)t0 * n_heads * D + (size_t)(lane % UPH) * 8;
  const int rl = lane / UPH;  // this lane's row inside a group
  V8 a0[NB], b0[NB], a1[NB], b1[NB];
  // rows past the block's end re-read its last row (no branch around the
  // loads, so the waits count them exactly); their sums are not stored
  auto fetch = [&](V8 (&a)[NB], V8 (&b)[NB], int g0) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int r = min((g0 + k * (kThreads / 64)) * RPG + rl, rows - 1);
      a[k] = load8<T>(o + base + (size_t)r * D);
      b[k] = load8<T>(dout + base + (size_t)r * D);
    }
  };
  auto reduce = [&](const V8 (&a)[NB], const V8 (&b)[NB], int g0) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const f32x8 fa = to_f32x8(a[k]), fb = to_f32x8(b[k]);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += fa[i] * fb[i];
      sum += dpp_f<0xB1>(sum);    // quad_perm 1,0,3,2
      sum += dpp_f<0x4E>(sum);    // quad_perm 2,3,0,1
      sum += dpp_f<0x141>(sum);   // row_half_mirror: the other quad of 8 lanes
      if (UPH == 16) sum += dpp_f<0x140>(sum);  // row_mirror: the other 8 of 16
      const int r = (g0 + k * (kThreads / 64)) * RPG + rl;
      if (lane % UPH == 0 && r < rows) red[r] = sum;
    }
  };
  // wave w takes groups w, w + 4, ...: NB of them per step, two register sets
  // alternating (unrolled by two so the set is a compile-time choice)
  constexpr int STEP = NB * (kThreads / 64);
  int g = wave;
  fetch(a0, b0, g);
  for (; g < groups; g += 2 * STEP) {
    fetch(a1, b1, g + STEP);
    reduce(a0, b0, g);
    fetch(a0, b0, g + 2 * STEP);
    reduce(a1, b1, g + STEP);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rows; i += kThreads) {
    const int h = i / nt, t = i - h * nt;
    delta[(size_t)h * n_tokens + t0 + t] = red[t * n_heads + h];
  }
}

template <typename T, bool ROPE>
static void pre_b(const Meta& m, BlockShape bs, dim3 grid, const void* o, const void* dout,
                  const void* q, const void* k, float* delta, void* qr, void* kr,
                  hipStream_t stream) {
#define PVJ_PRE(B)                                                                         \
  bwd_pre_kernel<T, ROPE, B><<<grid, kThreads, 0, stream>>>(                               \
      m, (const T*)o, (const T*)dout, (const T*)q, (const T*)k, delta, (T*)qr, (T*)kr, bs.rows)
  switch (bs.batch) {
    case 1: PVJ_PRE(1); break;
    case 2: PVJ_PRE(2); break;
    case 3: PVJ_PRE(3); break;
    default: PVJ_PRE(4);
  }
#undef PVJ_PRE
}

hipError_t launch_bwd_pre(const pvj_plan* p, const Meta& m, const void* o, const void* dout,
                          const void* q, const void* k, float* delta, void* qr, void* kr,
                          bool rope, hipStream_t stream) {
  if (m.n_tokens == 0) return hipSuccess;
  const bool bf = p->desc.dtype == PVJ_BF16;
  if (!rope) {
    constexpr int NB = 4;  // groups of 64 units per wave and step
    // 128 tokens per block (fewer with many heads: the row sums stay within 16
    // KB of LDS), so each head's Delta is written as 512-byte runs and each wave
    // streams ~200 KB.  Measured on the training pack (H = 24): 8-64 tokens per
    // block 0.125-0.129 ms, 128 tokens 0.122 ms; 2, 4 or 8 groups per step alike
    const int tb = std::max(1, std::min(128, 4096 / m.n_heads));
    const dim3 g((unsigned)((m.n_tokens + tb - 1) / tb));
    const size_t lds = (size_t)tb * m.n_heads * sizeof(float);
#define PVJ_DELTA(TT, DD)                                                                    \
  delta_kernel<TT, DD, NB><<<g, kThreads, lds, stream>>>((const TT*)o, (const TT*)dout, delta, \
                                                          m.n_tokens, m.n_heads, tb)
    if (bf && m.head_dim == 128) PVJ_DELTA(bf16, 128);
    else if (bf) PVJ_DELTA(bf16, 64);
    else if (m.head_dim == 128) PVJ_DELTA(float, 128);
    else PVJ_DELTA(float, 64);
#undef PVJ_DELTA
    return hipGetLastError();
  }
  const BlockShape bs = block_shape(m, bf ? 2 : 4);
  const dim3 grid((m.n_tokens + bs.rows - 1) / bs.rows);
  if (bf) {
    if (rope) pre_b<bf16, true>(m, bs, grid, o, dout, q, k, delta, qr, kr, stream);
    else pre_b<bf16, false>(m, bs, grid, o, dout, q, k, delta, qr, kr, stream);
  } else {
    if (rope) pre_b<float, true>(m, bs, grid, o, dout, q, k, delta, qr, kr, stream);
    else pre_b<float, false>(m, bs, grid, o, dout, q, k, delta, qr, kr, stream);
  }
  return hipGetLastError();
}

}  // namespace pvj
