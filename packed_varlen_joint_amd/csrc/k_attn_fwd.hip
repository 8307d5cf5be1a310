// Packed variable-length joint attention, forward, for gfx950.
//
// Mage-Flow review page, section "Native-Resolution MMDiT": joint
// self-attention over each sample's text+image tokens, confined to the sample
// by per-sample cumulative offsets (no block-diagonal mask); HF paper page,
// "Highlights": per-sample 2D RoPE, applied here on load when requested.
//
// One workgroup = one work item (sample, head, 128-query tile); 4 waves, each
// owning 32 queries.  The KV loop streams 64-key tiles of the item's own
// sample only, through double-buffered LDS (separate static buffers).
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16; fp32 inputs use eight
// v_mfma_f32_32x32x2_f32 per k-step of 16):
//  * scores are computed transposed, S^T = K Q^T: the accumulator of lane l
//    holds query l % 32 against 16 keys, and lane l ^ 32 the other 16 keys of
//    the same 32-key block.  Row max and row sum are therefore lane-local plus
//    one v_permlane32_swap per tile; the running max m and sum l (fp32) live in
//    registers of the wave that owns the query.
//  * K rows are stored in LDS in the sigma order (bits 2 and 3 of the row
//    swapped), so accumulator register r of lane l holds key
//    16*(r/8) + 8*(l/32) + r%8 of its 32-key block and the eight probabilities
//    of registers 8s..8s+7 are exactly the B operand (P^T, k = keys) of the
//    output product O^T = V^T P^T.  Its A operand (V^T: rows = d, k = keys) is
//    read from the row-major V tile with two transposing ds_read_b64_tr_b16.
//  * the output accumulator O^T of lane l holds query l % 32, so the online
//    softmax rescale is lane-local too.
//  * bf16 tiles arrive by direct global -> LDS copies (no register round
//    trip), except K with RoPE on load, which is rotated in registers between
//    its global load and its LDS store.
// Online softmax in base 2: x = s * scale * log2(e); p = 2^(x - m);
// LSE = (m + log2 l) * ln 2; the reference max m is only moved (and O, l
// rescaled) when a tile raises some row max by more than 8 (a factor 256).
// Keys at or past the sample end are masked to -inf.

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kFwdBM = 128;  // query rows per workgroup (must match fwd_tile_rows)
constexpr int kFwdBN = 64;   // keys per KV tile
constexpr int kFwdThreads = kTileThreads;

template <typename T, int D>
struct FwdTile {
  static constexpr int UPR = D / 8;                      // 8-element units per row
  static constexpr int NK = kFwdBN * UPR / kFwdThreads;  // units per thread per tile (staged)
  static constexpr int TILE = kFwdBN * D;
};

// bf16 tiles fit two waves per SIMD, so two workgroups share a CU and one's
// softmax VALU work overlaps the other's matrix-core work.
template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(
    sizeof(T) == 2 ? 2 : 1, sizeof(T) == 2 ? 2 : 1))) void attn_fwd_kernel(
    Meta m, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, float scale_log2) {
  typedef typename Vec8<T>::type V8;
  typedef FwdTile<T, D> C;
  constexpr int KS = D / 16;  // k-steps of 16 over the head dim
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int NK = C::NK;
  constexpr int UPR = C::UPR;
  constexpr bool DMA = sizeof(T) == 2;
  constexpr bool K_DMA = DMA && !ROPE;

  __shared__ __align__(16) T k_b0[C::TILE], k_b1[C::TILE], v_b0[C::TILE], v_b1[C::TILE];

  const Item it = m.fwd_items[blockIdx.x];
  if (it.sample < 0) return;
  const SampleInfo si = m.sinfo[it.sample];
  const int L = si.len;
  const size_t RS = (size_t)m.n_heads * D;  // row stride (elements)
  const size_t base = (size_t)si.start * RS + (size_t)it.head * D;
  const T* Qh = Q + base;
  const T* Kh = K + base;
  const T* Vh = V + base;
  T* Oh = O + base;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qi = it.tile * kFwdBM + wave * 32 + l32;  // this lane's query (local index)

  // ---- Q fragments (B operand of S^T = K Q^T), rotated on load if ROPE ----
  V8 qf[KS];
  {
    const RopePos qp = ROPE && qi < L ? token_pos3(qi, si) : RopePos{0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int unit = 2 * ks + hi;
      V8 v = {};
      if (qi < L) {
        v = load8<T>(Qh + (size_t)qi * RS + unit * 8);
        if (ROPE)
          v = from_f32x8<T>(
              rope_unit(to_f32x8(v), unit, axis_pos(qp, unit_axis(unit, m)), m, false));
      }
      qf[ks] = v;
    }
  }

  // ---- tile loaders ----
  // staged path (K with RoPE, fp32): rows k_row0 + i * K_ROW_STEP, one unit each
  const int k_unit = tid % UPR;
  const int k_row0 = tid / UPR;
  constexpr int K_ROW_STEP = kFwdThreads / UPR;
  constexpr int NKR = K_DMA ? 1 : NK;
  constexpr int NVR = DMA ? 1 : NK;
  V8 kreg[NKR], vreg[NVR];
  // RoPE: this thread always handles the same unit of the head dim, so its
  // axis is fixed; only the key position varies
  const int k_axis = unit_axis(k_unit, m);

  auto load_tile = [&](int kv0, int b) {
    if constexpr (K_DMA) {
      dma_tile<D, kFwdBN>(b ? k_b1 : k_b0, Kh, RS, kv0, L);
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int kk = kv0 + k_row0 + i * K_ROW_STEP;
        V8 z = {};
        kreg[i] = kk < L ? load8<T>(Kh + (size_t)kk * RS + k_unit * 8) : z;
      }
    }
    if constexpr (DMA) {
      dma_tile<D, kFwdBN>(b ? v_b1 : v_b0, Vh, RS, kv0, L);
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int kk = kv0 + k_row0 + i * K_ROW_STEP;
        V8 z = {};
        vreg[i] = kk < L ? load8<T>(Vh + (size_t)kk * RS + k_unit * 8) : z;
      }
    }
  };

  auto store_tile = [&](int b, int kv0) {
    if constexpr (!K_DMA) {
      T* kb = b ? k_b1 : k_b0;
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        V8 v = kreg[i];
        if (ROPE) {
          const int kk = kv0 + k_row0 + i * K_ROW_STEP;
          const RopePos kp = kk < L ? token_pos3(kk, si) : RopePos{0, 0, 0};
          v = from_f32x8<T>(rope_unit(to_f32x8(v), k_unit, axis_pos(kp, k_axis), m, false));
        }
        store8<T>(kb + toff<D>(bsigma(k_row0 + i * K_ROW_STEP), k_unit * 8), v);
      }
    }
    if constexpr (!DMA) {
      T* vb = b ? v_b1 : v_b0;
#pragma unroll
      for (int i = 0; i < NK; ++i)
        store8<T>(vb + toff<D>(bsigma(k_row0 + i * K_ROW_STEP), k_unit * 8), vreg[i]);
    }
    if constexpr (DMA) wait_dma();
  };
  auto sig = [](int k) { return bsigma(k); };

  const int nkv = (L + kFwdBN - 1) / kFwdBN;
  load_tile(0, 0);
  store_tile(0, 0);
  __syncthreads();

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int j = 0; j < nkv; ++j) {
    const int b = j & 1;
    const int kv0 = j * kFwdBN;
    if (j + 1 < nkv) load_tile(kv0 + kFwdBN, b ^ 1);
    const T* ks = b ? k_b1 : k_b0;
    const T* vs = b ? v_b1 : v_b0;

    // S^T = K Q^T for the two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int rho = kb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        mma16(s[kb], load8<T>(ks + toff<D>(rho, (2 * kk + hi) * 8)), qf[kk]);
    }
    // mask keys past the sample end (last tile only; their rows hold re-read data)
    if (kv0 + kFwdBN > L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + 16 * (r >> 3) + 8 * hi + (r & 7);
          if (key >= L) s[kb][r] = -INFINITY;
        }
    }
    // online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_pair32(mx) * scale_log2;
    // Rescale only when some query's max grew by more than 2^8: otherwise keep
    // the stale reference max (p <= 256, far from overflow).  O / l is exact
    // for any common reference, so this only skips work.
    if (__any(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    float ls = 0.f;
    V8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kb][r], scale_log2, -m_run));
        ls += p;
        pf[kb][r >> 3][r & 7] = (T)p;
      }
    l_run += ls;

    // O^T += V^T P^T (A = V^T by transposing reads of the row-major V tile)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          mma16(oacc[db], frag_t<D>(vs, kb * 32 + 16 * st, db * 32, sig), pf[kb][st]);
    if (j + 1 < nkv) store_tile(b ^ 1, kv0 + kFwdBN);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE ----
  const float l_tot = sum_pair32(l_run);
  if (qi < L) {
    const float inv = 1.f / l_tot;
    T* orow = Oh + (size_t)qi * RS;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hi;
        if constexpr (sizeof(T) == 2) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)(oacc[db][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + d) = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(orow + d) = w;
        }
      }
    if (hi == 0 && LSE)
      LSE[(size_t)it.head * m.n_tokens + si.start + qi] =
          (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

template <typename T, int D, bool ROPE>
static hipError_t launch_fwd_t(const Meta& m, const void* q, const void* k, const void* v, void* o,
                               float* lse, float scale_log2, hipStream_t stream) {
  attn_fwd_kernel<T, D, ROPE><<<dim3(m.n_fwd), dim3(kFwdThreads), 0, stream>>>(
      m, (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, scale_log2);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, void* o, float* lse, float scale, bool rope,
                           hipStream_t stream) {
  if (m.n_fwd == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int D = p->desc.head_dim;
#define PVJ_FWD(TT, DD)                                                                    \
  return rope ? launch_fwd_t<TT, DD, true>(m, q, k, v, o, lse, sl2, stream)                \
              : launch_fwd_t<TT, DD, false>(m, q, k, v, o, lse, sl2, stream)
  if (bf && D == 128) PVJ_FWD(bf16, 128);
  if (bf && D == 64) PVJ_FWD(bf16, 64);
  if (!bf && D == 128) PVJ_FWD(float, 128);
  PVJ_FWD(float, 64);
#undef PVJ_FWD
}

}  // namespace pvj
