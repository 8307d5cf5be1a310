// Packed variable-length joint attention, backward dQ pass, for gfx950.
//
// Gradient of sum(O * dO) with respect to Q, per sample and head (Mage-Flow
// review page, section "Kernel fusion": training runs forward + backward
// through the joint attention):
//   P = exp(s Q'K'^T - LSE); dP = dO V^T; dS = P * (dP - Delta);
//   dQ' = s dS K'; with RoPE, dQ = R^T dQ'.
//
// attn_bwd_dq_kernel: one workgroup per (sample, head, query tile of the
// forward: 256 bf16, 128 fp32), one wave per 32 queries with Q' and dO in
// registers; streams 64-key tiles of
// K' and V through double-buffered LDS like the forward.  S^T = K'Q'^T and
// dP^T = V dO^T put one query per lane (LSE and Delta are per-lane scalars);
// dQ'^T += K'^T dS^T takes dS^T straight from the accumulators and K'^T by
// transposing reads.  The epilogue scales, applies R^T (rotation pairs are in
// one lane) and stores dQ in the output dtype.  No atomics: each dQ row is
// written by exactly one workgroup.  The kernel also forms Delta =
// rowsum(dO * O) of its queries (it loads their O rows beside the dO rows)
// and stores it for the dK/dV kernel, which runs after it.

#include <type_traits>

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kDqBN = 64;  // keys per streamed tile

template <typename T, int D>
struct DqCfg {
  // queries per workgroup = the forward tile (the kernel walks dq_items):
  // bf16 8 waves x 32 queries share each K'/V tile copy; fp32 4 waves
  static constexpr int BM = sizeof(T) == 2 ? 256 : 128;
  static constexpr int THREADS = BM * 2;
  static constexpr int UPR = D / 8;
  static constexpr int NK = kDqBN * UPR / THREADS;  // units per thread per tile (K and V)
  static constexpr int TILE = kDqBN * D;
};

// bf16 runs two waves per SIMD (one 8-wave workgroup per CU, 64 KB of LDS)
template <typename T, int D, bool SM>
__global__ __launch_bounds__((DqCfg<T, D>::THREADS)) __attribute__((amdgpu_waves_per_eu(
    sizeof(T) == 2 ? 2 : 1, sizeof(T) == 2 ? 2 : 1))) void attn_bwd_dq_kernel(
    Meta m, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ O, const T* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ DELTA, T* __restrict__ dQ, float scale, float scale_log2, int rope) {
  typedef typename Vec8<T>::type V8;
  typedef DqCfg<T, D> C;
  constexpr int KS = D / 16, DB = D / 32, UPR = C::UPR, NK = C::NK;

  // separate static buffers (see the dK/dV kernel)
  __shared__ __align__(16) T k_b0[C::TILE], k_b1[C::TILE], v_b0[C::TILE], v_b1[C::TILE];
  auto ks_of = [&](int b) { return b ? k_b1 : k_b0; };
  auto vs_of = [&](int b) { return b ? v_b1 : v_b0; };

  const Item it = m.dq_items[blockIdx.x];
  if (it.sample < 0) return;
  const SampleInfo si = m.sinfo[it.sample];
  const int L = si.len;
  const size_t RS = (size_t)m.n_heads * D;
  const size_t base = (size_t)si.start * RS + (size_t)it.head * D;
  const size_t hb = (size_t)it.head * D;  // a token's row r is at hb + r * RS
  // stream-major copies (bf16 only): from the head's base to the sample's last image row
  const int tbytes = SM ? sm_bytes<D>(si, RS) : 0;
  const uint32_t rsb = (uint32_t)(RS * sizeof(T));
  (void)tbytes, (void)rsb;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qi = it.tile * C::BM + wave * 32 + l32;  // this lane's query
  const int qrow = qi < L ? token_row<SM>(si, qi) : 0;

  V8 qf[KS], gf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int unit = 2 * ks + hi;
    V8 z = {};
    qf[ks] = qi < L ? load8<T>(Q + hb + (size_t)qrow * RS + unit * 8) : z;
    gf[ks] = qi < L ? load8<T>(dO + hb + (size_t)qrow * RS + unit * 8) : z;
    of[ks] = qi < L ? load8<T>(O + hb + (size_t)qrow * RS + unit * 8) : z;
  }
  // LSE and Delta are [H, T] in the token tensors' row order
  const float lse2 = qi < L ? LSE[(size_t)it.head * m.n_tokens + qrow] * 1.4426950408889634f
                            : INFINITY;

  const int k_unit = tid % UPR;
  const int k_row0 = tid / UPR;
  constexpr int K_ROW_STEP = C::THREADS / UPR;
  constexpr bool DMA = sizeof(T) == 2;
  V8 kreg[DMA ? 1 : NK], vreg[DMA ? 1 : NK];
  // direct copies (K and V tiles share one layout; rows past the end are zeros)
  typedef DmaTile<D, kDqBN, C::THREADS> DT;
  const DT dma(RS);
  const uint32_t c1 = SM ? dma.sm_c1(si, rsb) : 0u;  // stream-major image-row offset
  (void)c1;
  const typename DT::Src rk = DT::src(K + base, RS, L), rv = DT::src(V + base, RS, L);
  auto load_kv = [&](int kv0, int b) {
    if constexpr (DMA && SM) {
#pragma unroll
      for (int c = 0; c < DT::PER; ++c) {
        dma.part_sm(ks_of(b), reinterpret_cast<const bf16*>(K) + hb, tbytes, rsb, c1, si, kv0, c);
        dma.part_sm(vs_of(b), reinterpret_cast<const bf16*>(V) + hb, tbytes, rsb, c1, si, kv0, c);
      }
    } else if constexpr (DMA) {
      dma.copy(ks_of(b), rk, RS, kv0);
      dma.copy(vs_of(b), rv, RS, kv0);
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int kk = kv0 + k_row0 + i * K_ROW_STEP;
        V8 z = {};
        kreg[i] = kk < L ? load8<T>(K + base + (size_t)kk * RS + k_unit * 8) : z;
        vreg[i] = kk < L ? load8<T>(V + base + (size_t)kk * RS + k_unit * 8) : z;
      }
    }
  };
  auto store_kv = [&](int b) {
    if constexpr (DMA) {
      wait_dma();
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int rho = bsigma(k_row0 + i * K_ROW_STEP);
        store8<T>(ks_of(b) + toff<D>(rho, k_unit * 8), kreg[i]);
        store8<T>(vs_of(b) + toff<D>(rho, k_unit * 8), vreg[i]);
      }
    }
  };
  auto sig = [](int k) { return bsigma(k); };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // Per-lane LDS addresses, fixed for the whole loop (bf16): row l32 at unit
  // 2kk+hi of the K and V tiles (same layout), and the K^T fragment bases of
  // output block db and half t; the 32-key block, the 16-key half and the
  // buffer add compile-time offsets.  The empty asm keeps them in registers.
  uint32_t ka[KS], va[DB][2];
  if constexpr (DMA) {
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

  const int nkv = (L + kDqBN - 1) / kDqBN;
  load_kv(0, 0);
  store_kv(0);
  // Delta = rowsum(dO * O) of this lane's query, formed here (this kernel
  // visits each query once; it runs before the dK/dV kernel, which reads it)
  // once the first tile's copies and the row loads are in: the lane pair l,
  // l + 32 holds the even and odd units of the row, every lane adds the two
  // halves in that order, and the first lane of the pair stores it.
  float delta;
  {
    float half = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x8 a = to_f32x8(gf[ks]), b = to_f32x8(of[ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) half += a[e] * b[e];
    }
    delta = sum_pair32(half);
    if (qi < L && hi == 0) DELTA[(size_t)it.head * m.n_tokens + qrow] = delta;
  }
  __syncthreads();
  auto step = [&](int j, auto bc, auto mc) {
    constexpr int B = decltype(bc)::value;
    constexpr bool MASK = decltype(mc)::value;
    const int kv0 = j * kDqBN;
    if (j + 1 < nkv) load_kv(kv0 + kDqBN, B ^ 1);
    const T* ks = B ? k_b1 : k_b0;
    const T* vs = B ? v_b1 : v_b0;
    V8 sfr[2][2];  // dS^T fragments [32-key block][16-key step]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // the products run at raised wave priority: the SIMD's other wave (another
      // workgroup) then fills the gaps with its softmax work instead of
      // delaying these matrix-core issues
      __builtin_amdgcn_s_setprio(1);
      f32x16 s = {}, dp = {};
      const int rho = kb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        V8 kf, vf;
        if constexpr (DMA) {
          const uint32_t o = ka[kk] + kb * 32 * D * sizeof(T);
          kf = *reinterpret_cast<const V8*>(reinterpret_cast<const char*>(ks) + o);
          vf = *reinterpret_cast<const V8*>(reinterpret_cast<const char*>(vs) + o);
        } else {
          const int off = toff<D>(rho, (2 * kk + hi) * 8);
          kf = load8<T>(ks + off);
          vf = load8<T>(vs + off);
        }
        mma16(s, kf, qf[kk]);
        mma16(dp, vf, gf[kk]);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(fmaf(s[r], scale_log2, -lse2));
        // the last tile's rows past the sample end read as zeros: zero weight
        if constexpr (MASK)
          if (kv0 + kb * 32 + 16 * (r >> 3) + 8 * hi + (r & 7) >= L) p = 0.f;
        sfr[kb][r >> 3][r & 7] = (T)(p * (dp[r] - delta));
      }
    }
    // dQ'^T += K'^T dS^T
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          V8 kt;
          if constexpr (DMA) {
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const uint32_t o = (uint32_t)((kb * 32 + 16 * st) * D * sizeof(T));
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const i16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4*)(reinterpret_cast<const char*>(ks) + va[db][t] + o));
              const bf16x4 h = __builtin_bit_cast(bf16x4, w);
#pragma unroll
              for (int e = 0; e < 4; ++e) kt[4 * t + e] = h[e];
            }
          } else {
            kt = frag_t<D>(ks, kb * 32 + 16 * st, db * 32, sig);
          }
          mma16(acc[db], kt, sfr[kb][st]);
        }
    // bf16: keep the transposing K' reads four products ahead of them
    // (measured: 0.8% on this kernel)
    if constexpr (sizeof(T) == 2) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 4 * DB - 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (j + 1 < nkv) store_kv(B ^ 1);
    __syncthreads();
  };
  // full tiles in pairs (buffers 0, 1), a leftover full tile, then the
  // partial tile with the key mask
  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  typedef std::integral_constant<bool, false> NoMask;
  typedef std::integral_constant<bool, true> Mask;
  const int nfull = L / kDqBN;
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

  // ---- epilogue: dQ = R^T (s dQ'); lane holds query qi, d = 32db + 8g + 4hi + e ----
  if (qi < L) {
    const RopePos qp = rope ? token_pos3(qi, si) : RopePos{0, 0, 0};
    T* row = dQ + hb + (size_t)qrow * RS;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hi;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * g + e] * scale;
        if (rope) {
          // pairs (d0, d0+1), (d0+2, d0+3) of unit d0 / 8
          const size_t to =
              (size_t)axis_pos(qp, unit_axis(d0 >> 3, m)) * m.n_pairs + (d0 >> 1);
          const f32x2 cs = *reinterpret_cast<const f32x2*>(m.cos_tab + to);
          const f32x2 sn = *reinterpret_cast<const f32x2*>(m.sin_tab + to);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float a = x[2 * q], bb = x[2 * q + 1];
            x[2 * q] = a * cs[q] + bb * sn[q];        // rotate by -angle
            x[2 * q + 1] = -a * sn[q] + bb * cs[q];
          }
        }
        if constexpr (sizeof(T) == 2) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (bf16)x[e];
          *reinterpret_cast<bf16x4*>(row + d0) = w;
        } else {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = x[e];
          *reinterpret_cast<f32x4*>(row + d0) = w;
        }
      }
  }
}

template <typename T, int D, bool SM>
static hipError_t launch_dq_t(const Meta& m, const void* q, const void* k, const void* v,
                              const void* o, const void* dout, const float* lse, float* delta,
                              void* dq, float scale, bool rope, hipStream_t stream) {
  if (m.n_dq > 0)
    attn_bwd_dq_kernel<T, D, SM><<<dim3(m.n_dq), dim3(DqCfg<T, D>::THREADS), 0, stream>>>(
        m, (const T*)q, (const T*)k, (const T*)v, (const T*)o, (const T*)dout, lse, delta,
        (T*)dq, scale, scale * 1.4426950408889634f, rope ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                              const void* v, const void* o, const void* dout, const float* lse,
                              float* delta, void* dq, float scale, bool rope, bool sm,
                              hipStream_t stream) {
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int D = p->desc.head_dim;
#define PVJ_DQ(TT, DD, SMV) \
  return launch_dq_t<TT, DD, SMV>(m, q, k, v, o, dout, lse, delta, dq, scale, rope, stream)
  // (the stream-major layout is bf16 only; the caller checks)
  if (bf && sm && D == 128) PVJ_DQ(bf16, 128, true);
  if (bf && sm) PVJ_DQ(bf16, 64, true);
  if (bf && D == 128) PVJ_DQ(bf16, 128, false);
  if (bf) PVJ_DQ(bf16, 64, false);
  if (D == 128) PVJ_DQ(float, 128, false);
  PVJ_DQ(float, 64, false);
#undef PVJ_DQ
}

}  // namespace pvj
