// Packed variable-length joint attention, forward, for gfx950.
//
// Mage-Flow review page, section "Native-Resolution MMDiT": joint
// self-attention over each sample's text+image tokens, confined to the sample
// by per-sample cumulative offsets (no block-diagonal mask); HF paper page,
// "Highlights": per-sample 2D RoPE, applied here on load when requested.
//
// One workgroup = one work item (sample, head, query tile); one wave per 32
// queries: bf16 tiles of 256 queries (8 waves, two per SIMD, all eight
// sharing each K/V tile copy), fp32 tiles of 128.  The KV loop streams 64-key
// tiles of the item's own sample only, through double-buffered LDS (separate
// static buffers).
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

#include <type_traits>

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kFwdBN = 64;  // keys per KV tile

template <typename T, int D>
struct FwdTile {
  // query rows per workgroup (must match fwd_tile_rows): bf16 8 waves x 32
  // queries, so the eight share each K/V tile copy; fp32 4 waves
  static constexpr int BM = sizeof(T) == 2 ? 256 : 128;
  static constexpr int THREADS = BM * 2;               // one wave per 32 queries
  static constexpr int UPR = D / 8;                    // 8-element units per row
  static constexpr int NK = kFwdBN * UPR / THREADS;    // units per thread per tile (staged)
  static constexpr int TILE = kFwdBN * D;
};

// bf16 runs two waves per SIMD (one 8-wave workgroup per CU), so one wave's
// softmax VALU work overlaps the other's matrix-core work.
template <typename T, int D, bool ROPE>
__global__ __launch_bounds__((FwdTile<T, D>::THREADS)) __attribute__((amdgpu_waves_per_eu(
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
  const int qi = it.tile * C::BM + wave * 32 + l32;  // this lane's query (local index)

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
  constexpr int K_ROW_STEP = C::THREADS / UPR;
  constexpr int NKR = K_DMA ? 1 : NK;
  constexpr int NVR = DMA ? 1 : NK;
  V8 kreg[NKR], vreg[NVR];
  // RoPE: this thread always handles the same unit of the head dim, so its
  // axis is fixed; only the key position varies
  const int k_axis = unit_axis(k_unit, m);
  // direct copies: per-thread offsets (K and V tiles share one layout) and
  // one buffer resource per operand spanning this head's L rows
  typedef DmaTile<D, kFwdBN, C::THREADS> DT;
  const DT dma(RS);
  const typename DT::Src rk = DT::src(Kh, RS, L), rv = DT::src(Vh, RS, L);

  // the KV loop is unrolled by two so that every LDS address is a fixed
  // per-lane offset plus a compile-time buffer offset
  auto load_tile = [&](int kv0, auto bc) {
    constexpr int B = decltype(bc)::value;
    if constexpr (K_DMA) {
      dma.copy(B ? k_b1 : k_b0, rk, RS, kv0);
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int kk = kv0 + k_row0 + i * K_ROW_STEP;
        V8 z = {};
        kreg[i] = kk < L ? load8<T>(Kh + (size_t)kk * RS + k_unit * 8) : z;
      }
    }
    if constexpr (DMA) {
      dma.copy(B ? v_b1 : v_b0, rv, RS, kv0);
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int kk = kv0 + k_row0 + i * K_ROW_STEP;
        V8 z = {};
        vreg[i] = kk < L ? load8<T>(Vh + (size_t)kk * RS + k_unit * 8) : z;
      }
    }
  };

  auto store_tile = [&](int kv0, auto bc) {
    constexpr int B = decltype(bc)::value;
    if constexpr (!K_DMA) {
      T* kb = B ? k_b1 : k_b0;
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
      T* vb = B ? v_b1 : v_b0;
#pragma unroll
      for (int i = 0; i < NK; ++i)
        store8<T>(vb + toff<D>(bsigma(k_row0 + i * K_ROW_STEP), k_unit * 8), vreg[i]);
    }
    if constexpr (DMA) wait_dma();
  };
  auto sig = [](int k) { return bsigma(k); };

  const int nkv = (L + kFwdBN - 1) / kFwdBN;
  load_tile(0, std::integral_constant<int, 0>{});
  store_tile(0, std::integral_constant<int, 0>{});
  __syncthreads();

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS addresses of the operand reads, fixed for the whole loop
  // (bf16): K row l32 at unit 2kk+hi, and the V fragment bases of output
  // block db and half t.  The 32-key block kb, the 16-key half st and the
  // buffer only add compile-time offsets (row bits 4-5 do not enter the
  // swizzle, and sigma leaves them in place).  The empty asm pins each value
  // in a register so it is not recomputed every tile.
  uint32_t ka[KS], va[DB][2];
  if constexpr (sizeof(T) == 2) {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      ka[kk] = (uint32_t)(toff<D>(l32, (2 * kk + hi) * 8) * sizeof(T));
      asm volatile("" : "+v"(ka[kk]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        va[db][t] = (uint32_t)(toff<D>(bsigma(8 * (g >> 1) + 4 * t + (sl >> 2)),
                                       db * 32 + 16 * (g & 1) + 4 * (sl & 3)) * sizeof(T));
        asm volatile("" : "+v"(va[db][t]));
      }
  }

  auto step = [&](int j, auto bc, auto mc) {
    constexpr int B = decltype(bc)::value;
    constexpr bool MASK = decltype(mc)::value;
    const int kv0 = j * kFwdBN;
    if (j + 1 < nkv) load_tile(kv0 + kFwdBN, std::integral_constant<int, B ^ 1>{});
    const T* ks = B ? k_b1 : k_b0;
    const T* vs = B ? v_b1 : v_b0;

    // S^T = K Q^T for the two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int rho = kb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        V8 kf;
        if constexpr (sizeof(T) == 2)
          kf = *reinterpret_cast<const V8*>(reinterpret_cast<const char*>(ks) + ka[kk] +
                                            kb * 32 * D * sizeof(T));
        else
          kf = load8<T>(ks + toff<D>(rho, (2 * kk + hi) * 8));
        mma16(s[kb], kf, qf[kk]);
      }
    }
    // mask keys past the sample end (the last, partial tile only; their rows
    // were read as zeros)
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + 16 * (r >> 3) + 8 * hi + (r & 7);
          if (key >= L) s[kb][r] = -INFINITY;
        }
    }
    // online softmax (base 2); max and sum as short independent chains (the
    // maxima associated so that they become three-input v_max3_f32)
    float mx4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float t = fmaxf(fmaxf(s[c >> 1][8 * (c & 1)], s[c >> 1][8 * (c & 1) + 1]),
                      s[c >> 1][8 * (c & 1) + 2]);
      t = fmaxf(fmaxf(t, s[c >> 1][8 * (c & 1) + 3]), s[c >> 1][8 * (c & 1) + 4]);
      t = fmaxf(fmaxf(t, s[c >> 1][8 * (c & 1) + 5]), s[c >> 1][8 * (c & 1) + 6]);
      mx4[c] = fmaxf(t, s[c >> 1][8 * (c & 1) + 7]);
    }
    float mx = fmaxf(fmaxf(fmaxf(mx4[0], mx4[1]), mx4[2]), mx4[3]);
    mx = max_pair32(mx) * scale_log2;
    // Rescale only when some query's max grew by more than 2^8: otherwise keep
    // the stale reference max (p <= 256, far from overflow).  O / l is exact
    // for any common reference, so this only skips work.  (The empty asm keeps
    // this a real branch: folded into selects it would cost the multiplies on
    // every tile.)
    if (__any(mx > m_run + 8.f)) {
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    float ls4[4] = {0.f, 0.f, 0.f, 0.f};
    V8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kb][r], scale_log2, -m_run));
        ls4[r & 3] += p;
        pf[kb][r >> 3][r & 7] = (T)p;
      }
    l_run += (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);

    // O^T += V^T P^T (A = V^T by transposing reads of the row-major V tile)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          V8 vf;
          if constexpr (sizeof(T) == 2) {
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const uint32_t o = (uint32_t)((kb * 32 + 16 * st) * D * sizeof(T));
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const i16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4*)(reinterpret_cast<const char*>(vs) + va[db][t] + o));
              const bf16x4 h = __builtin_bit_cast(bf16x4, w);
#pragma unroll
              for (int e = 0; e < 4; ++e) vf[4 * t + e] = h[e];
            }
          } else {
            vf = frag_t<D>(vs, kb * 32 + 16 * st, db * 32, sig);
          }
          mma16(oacc[db], vf, pf[kb][st]);
        }
    // bf16: keep the transposing reads of V four products ahead of them
    // (measured: 1.3% on the forward)
    if constexpr (sizeof(T) == 2) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 4 * DB - 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    if (j + 1 < nkv) store_tile(kv0 + kFwdBN, std::integral_constant<int, B ^ 1>{});
    __syncthreads();
  };
  // full tiles in pairs (buffers 0, 1), then a leftover full tile, then the
  // partial tile with the key mask
  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  typedef std::integral_constant<bool, false> NoMask;
  typedef std::integral_constant<bool, true> Mask;
  const int nfull = L / kFwdBN;
  int j = 0;
  for (; j + 1 < nfull; j += 2) {
    step(j, B0{}, NoMask{});
    step(j + 1, B1{}, NoMask{});
  }
  if (j < nfull) {
    step(j, B0{}, NoMask{});
    ++j;
  }
  if (j < nkv) {
    if (j & 1) step(j, B1{}, Mask{});
    else step(j, B0{}, Mask{});
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
  attn_fwd_kernel<T, D, ROPE><<<dim3(m.n_fwd), dim3(FwdTile<T, D>::THREADS), 0, stream>>>(
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
