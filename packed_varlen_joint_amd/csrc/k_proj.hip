// The per-stream projections around the joint attention with the modality
// pack / unpack fused in (Mage-Flow review page, section "Native-Resolution
// MMDiT": modality-specific projection layers for the text and image streams,
// whose tokens are concatenated only for the joint attention).
//
//  * qkv: [Q|K|V] = X_s W_s^T + b_s for one stream s; the epilogue writes each
//    token's row straight into its joint row of Q, K, V ([T, H, D]) and applies
//    the plan's RoPE to Q and K (fp32, one rounding), so no pack pass follows.
//  * out: Y_s = O_s W_s^T + b_s, the A rows gathered from the joint O by the
//    stream's row map, so no unpack pass precedes it.
//
// One bf16 GEMM kernel, C^T = W X^T with v_mfma_f32_32x32x16_bf16: the A
// operand is a tile of W rows (output features), the B operand a tile of
// token rows, so every lane owns one token and its registers hold runs of 4
// consecutive output features (the RoPE pairs are lane-local).  Workgroup
// tile 256 features x 256 tokens, 8 waves of 128 x 64, K in stages of 64
// through double-buffered LDS filled by direct buffer copies (per-lane byte
// offsets fixed once, the stage as an SGPR offset, rows past the end outside
// the buffer resource and read as zeros).  Tile order: each XCD keeps its
// token blocks (G of them) in L2 and walks the feature blocks, so every weight
// slice is fetched once per XCD and band.

#include <type_traits>

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kPjBK = 64;    // K per LDS stage
constexpr int kPjG = 4;      // token blocks per XCD sharing a weight slice

// Tile configuration: WAVES_N x WAVES_M waves, each owning NB x MB blocks of
// 32 features x 32 tokens; the workgroup tile is (32 NB WAVES_N) features x
// (32 MB WAVES_M) tokens.
template <int WAVES_N, int WAVES_M, int NB, int MB>
struct PjCfg {
  static constexpr int WAVES = WAVES_N * WAVES_M;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BN = 32 * NB * WAVES_N;  // output features per workgroup
  static constexpr int BM = 32 * MB * WAVES_M;  // tokens per workgroup
  static constexpr int UW = BN * kPjBK / 8 / THREADS;  // 16-byte units per thread, W tile
  static constexpr int UX = BM * kPjBK / 8 / THREADS;  // 16-byte units per thread, X tile
  static constexpr int NB_ = NB, MB_ = MB, WAVES_M_ = WAVES_M;
};
typedef PjCfg<2, 4, 4, 2> PjBig;    // 256 x 256, 8 waves of 128 x 64

// LDS slot of copy i of this lane: tiles are [rows][64] with the tsw<64>
// swizzle, each copy instruction filling one wave's 64 consecutive slots
template <int WAVES>
__device__ __forceinline__ void pj_slot(int i, int wave, int lane, int& row, int& unit) {
  const int slot = (i * WAVES + wave) * 64 + lane;
  row = slot / 8;
  unit = (slot % 8) ^ tsw<64>(row);
}

template <int WAVES, int UNITS>
__device__ __forceinline__ void pj_copy(__amdgpu_buffer_rsrc_t r, const uint32_t* off, int wave,
                                        bf16* tile, uint32_t soff) {
#pragma unroll
  for (int i = 0; i < UNITS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(tile + (i * WAVES + wave) * 512), 16, off[i],
        soff, 0, 0);
}

// stream row m -> joint row (the stream's rows in sample order)
__device__ __forceinline__ int joint_row(const Meta& m, int which, int r, int& sample) {
  const int32_t* cu = which == 0 ? m.cu_text : m.cu_img;
  const int s = find_sample(cu, m.n_samples, r);
  sample = s;
  const SampleInfo si = m.sinfo[s];
  return si.start + (which == 0 ? 0 : si.l_text) + (r - cu[s]);
}

template <typename CF, int MODE, bool ROPE>
__global__ __launch_bounds__(CF::THREADS) void proj_kernel(
    Meta m, int which, int M, int N, int K, const bf16* __restrict__ A,
    const bf16* __restrict__ W, const bf16* __restrict__ bias, bf16* __restrict__ out0,
    bf16* __restrict__ out1, bf16* __restrict__ out2, int a_rows_total) {
  constexpr int kPjBN = CF::BN, kPjBM = CF::BM, NB = CF::NB_, MB = CF::MB_;
  constexpr int WAVES = CF::WAVES, WM_N = CF::WAVES_M_;
  __shared__ __align__(16) bf16 w_b0[kPjBN * kPjBK], w_b1[kPjBN * kPjBK];
  __shared__ __align__(16) bf16 x_b0[kPjBM * kPjBK], x_b1[kPjBM * kPjBK];

  // tile order (see the header comment)
  const int nM = (M + kPjBM - 1) / kPjBM, nN = (N + kPjBN - 1) / kPjBN;
  const int xcd = blockIdx.x % kNumXcd, q = blockIdx.x / kNumXcd;
  const int band = q / (kPjG * nN), rem = q % (kPjG * nN);
  const int n_blk = rem / kPjG;
  const int m_blk = (band * kNumXcd + xcd) * kPjG + rem % kPjG;
  if (m_blk >= nM) return;
  const int m0 = m_blk * kPjBM, n0 = n_blk * kPjBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int wn = wave / WM_N, wm = wave % WM_N;  // this wave's sub-tile

  // per-lane copy offsets (bytes), fixed for the whole K loop
  uint32_t offw[CF::UW], offx[CF::UX];
#pragma unroll
  for (int i = 0; i < CF::UW; ++i) {
    int row, unit;
    pj_slot<WAVES>(i, wave, lane, row, unit);
    offw[i] = (uint32_t)(((size_t)(n0 + row) * K + unit * 8) * sizeof(bf16));
  }
#pragma unroll
  for (int i = 0; i < CF::UX; ++i) {
    int row, unit;
    pj_slot<WAVES>(i, wave, lane, row, unit);
    const int r = m0 + row;
    if (MODE == 0) {
      offx[i] = (uint32_t)(((size_t)r * K + unit * 8) * sizeof(bf16));
    } else {
      int s;
      const size_t jr = r < M ? (size_t)joint_row(m, which, r, s) : (size_t)a_rows_total;
      offx[i] = (uint32_t)((jr * K + unit * 8) * sizeof(bf16));
    }
  }
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(W), (short)0, (int)((size_t)N * K * sizeof(bf16)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(A), (short)0,
      (int)((size_t)(MODE == 0 ? M : a_rows_total) * K * sizeof(bf16)), 0x00020000);

  // operand read offsets (bytes) inside a tile: row (block*32 + l32), unit
  // 2kk+hi; the blocks of a wave add whole 32-row steps (no swizzle change)
  uint32_t ra[4], rb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    ra[kk] = (uint32_t)(toff<64>(wn * 32 * NB + l32, (2 * kk + hi) * 8) * sizeof(bf16));
    rb[kk] = (uint32_t)(toff<64>(wm * 32 * MB + l32, (2 * kk + hi) * 8) * sizeof(bf16));
  }

  f32x16 acc[NB][MB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[a][b] = f32x16{};

  const int nk = K / kPjBK;
  pj_copy<WAVES, CF::UW>(rw, offw, wave, w_b0, 0);
  pj_copy<WAVES, CF::UX>(rx, offx, wave, x_b0, 0);
  wait_dma();
  __syncthreads();
  auto stage = [&](int ks, auto bc) {
    constexpr int B = decltype(bc)::value;
    if (ks + 1 < nk) {
      const uint32_t so = (uint32_t)((ks + 1) * kPjBK * sizeof(bf16));
      pj_copy<WAVES, CF::UW>(rw, offw, wave, B ? w_b0 : w_b1, so);
      pj_copy<WAVES, CF::UX>(rx, offx, wave, B ? x_b0 : x_b1, so);
    }
    // keep the next stage's copies ahead of this stage's products (left to
    // itself the scheduler sinks them to the stage end, exposing their latency)
    __builtin_amdgcn_sched_barrier(0);
    const char* wt = reinterpret_cast<const char*>(B ? w_b1 : w_b0);
    const char* xt = reinterpret_cast<const char*>(B ? x_b1 : x_b0);
    // operand fragments double-buffered over the four k-steps: the reads of
    // step kk + 1 are issued ahead of the products of step kk
    bf16x8 fa[2][NB], fb[2][MB];
    auto frags = [&](int kk, bf16x8 (&a_)[NB], bf16x8 (&b_)[MB]) {
#pragma unroll
      for (int a = 0; a < NB; ++a)
        a_[a] = *reinterpret_cast<const bf16x8*>(wt + ra[kk] + a * 32 * 64 * sizeof(bf16));
#pragma unroll
      for (int b = 0; b < MB; ++b)
        b_[b] = *reinterpret_cast<const bf16x8*>(xt + rb[kk] + b * 32 * 64 * sizeof(bf16));
    };
    frags(0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) frags(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) mma16(acc[a][b], fa[kk & 1][a], fb[kk & 1][b]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, NB + MB, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) __builtin_amdgcn_sched_group_barrier(0x100, NB + MB, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NB * MB, 0);
    }
    wait_dma();
    __syncthreads();
  };
  int ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    stage(ks, std::integral_constant<int, 0>{});
    stage(ks + 1, std::integral_constant<int, 1>{});
  }
  if (ks < nk) stage(ks, std::integral_constant<int, 0>{});

  // ---- epilogue: lane = token, 4-feature runs per register group ----
  const int HD = m.n_heads * m.head_dim;
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int r = m0 + wm * 32 * MB + b * 32 + l32;
    if (r >= M) continue;
    int sample = 0;
    size_t orow;
    RopePos pos = {0, 0, 0};
    if (MODE == 0) {
      const int j = joint_row(m, which, r, sample);
      orow = (size_t)j * HD;
      if (ROPE) pos = token_pos3(j - m.sinfo[sample].start, m.sinfo[sample]);
    } else {
      orow = (size_t)r * N;
    }
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 32 * NB + a * 32 + 8 * g + 4 * hi;
        if (n >= N) continue;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[a][b][4 * g + e];
        if (bias) {
          const bf16x4 bb = *reinterpret_cast<const bf16x4*>(bias + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] += (float)bb[e];
        }
        bf16* dst;
        if (MODE == 0) {
          const int t = n / HD, w = n - t * HD;
          if (ROPE && t < 2) {
            const int d = w % m.head_dim;
            const size_t to =
                (size_t)axis_pos(pos, unit_axis(d >> 3, m)) * m.n_pairs + (d >> 1);
            const f32x2 cs = *reinterpret_cast<const f32x2*>(m.cos_tab + to);
            const f32x2 sn = *reinterpret_cast<const f32x2*>(m.sin_tab + to);
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const float u = x[2 * p], v = x[2 * p + 1];
              x[2 * p] = __builtin_fmaf(u, cs[p], -(v * sn[p]));
              x[2 * p + 1] = __builtin_fmaf(u, sn[p], v * cs[p]);
            }
          }
          dst = (t == 0 ? out0 : (t == 1 ? out1 : out2)) + orow + w;
        } else {
          dst = out0 + orow + n;
        }
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)x[e];
        *reinterpret_cast<bf16x4*>(dst) = o;
      }
  }
}

template <typename CF>
static int proj_grid(int M, int N) {
  const int nM = (M + CF::BM - 1) / CF::BM, nN = (N + CF::BN - 1) / CF::BN;
  const int per_band = kNumXcd * kPjG;
  const int bands = (nM + per_band - 1) / per_band;
  return bands * per_band * nN;
}

hipError_t launch_qkv_proj(const pvj_plan* p, const Meta& m, int which, int C, const void* x,
                           const void* w, const void* bias, void* q, void* k, void* v, bool rope,
                           hipStream_t st) {
  const int M = which == 0 ? m.n_text : m.n_img;
  const int N = 3 * m.n_heads * m.head_dim;
  if (M == 0) return hipSuccess;
  (void)p;
  typedef PjBig CF;
  const dim3 g(proj_grid<CF>(M, N));
  if (rope)
    proj_kernel<CF, 0, true><<<g, CF::THREADS, 0, st>>>(m, which, M, N, C, (const bf16*)x,
                                                        (const bf16*)w, (const bf16*)bias,
                                                        (bf16*)q, (bf16*)k, (bf16*)v, 0);
  else
    proj_kernel<CF, 0, false><<<g, CF::THREADS, 0, st>>>(m, which, M, N, C, (const bf16*)x,
                                                         (const bf16*)w, (const bf16*)bias,
                                                         (bf16*)q, (bf16*)k, (bf16*)v, 0);
  return hipGetLastError();
}

hipError_t launch_out_proj(const pvj_plan* p, const Meta& m, int which, int C, const void* o,
                           const void* w, const void* bias, void* y, hipStream_t st) {
  const int M = which == 0 ? m.n_text : m.n_img;
  const int K = m.n_heads * m.head_dim;
  if (M == 0) return hipSuccess;
  (void)p;
  typedef PjBig CF;
  const dim3 g(proj_grid<CF>(M, C));
  proj_kernel<CF, 1, false><<<g, CF::THREADS, 0, st>>>(m, which, M, C, K, (const bf16*)o,
                                                       (const bf16*)w, (const bf16*)bias,
                                                       (bf16*)y, nullptr, nullptr, m.n_tokens);
  return hipGetLastError();
}

}  // namespace pvj
