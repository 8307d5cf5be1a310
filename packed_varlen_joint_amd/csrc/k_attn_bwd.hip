// Packed variable-length joint attention, backward, for gfx950.
//
// Training runs forward + backward through the joint attention (Mage-Flow
// review page, section "Kernel fusion": 8-GPU training at ~50K packed tokens
// per GPU).  Gradients of sum(O * dO), per sample and head:
//   P = exp(s Q'K'^T - LSE); dV = P^T dO; dP = dO V^T; dS = P * (dP - Delta);
//   dK' = s dS^T Q'; dQ' = s dS K'; with RoPE on load, dK = R^T dK' here and
//   dQ = R^T dQ' in the finalize kernel.
//
// One workgroup = one work item (sample, head, 128-key tile); 4 waves, each
// owning 32 keys.  The loop walks the sample's query tiles (64 rows for bf16,
// 32 for fp32) through LDS.  Matrix-core mapping (32x32 MFMA, k-step 16):
//  * S = Q' K'^T and dP = dO V^T: A = Q' / dO rows from LDS (stored in row
//    order sigma, bits 2 and 3 swapped, as in the forward), B = K' / V rows
//    held in registers.  The accumulator of lane l holds key l % 32, and
//    register r of q-block b holds query 32b + 16(r/8) + 8(l/32) + r%8.
//  * dV += P^T dO and dK' += dS^T Q': the accumulators of P and dS are the A
//    operand directly (rows = keys, k = 16 consecutive queries); B = dO / Q'
//    from transposed LDS copies ([d][query]), one 16-byte read per fragment.
//  * dQ': dS (bf16, [query][key]) goes through LDS once; each wave then
//    computes a 32-wide d-slice of dQ' for the tile's queries over all 128
//    keys (B = K' transposed in LDS) and adds it to the fp32 accumulator with
//    one coalesced atomic per element per workgroup.
//  * LSE and Delta of the tile's queries are staged in LDS.  Keys and queries
//    past the sample end are zero-filled and masked (P = 0).

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kBwdBN = 128;  // keys per workgroup (must match bwd_tile_rows)
constexpr int kBwdThreads = 256;

__device__ __forceinline__ int bsigma(int k) { return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <typename T, int D>
struct BwdCfg {
  static constexpr int QB = sizeof(T) == 2 ? 2 : 1;  // 32-query blocks per tile
  static constexpr int BQ = 32 * QB;                 // queries per tile
  static constexpr int UPR = D / 8;                  // 8-element units per row
  static constexpr int KS = D / 16;                  // k-steps over d
  static constexpr int DB = D / 32;                  // 32-wide d blocks
  static constexpr int QU = BQ / 8;                  // units per transposed row
  static constexpr int KPQ = BQ * UPR / kBwdThreads; // rows per thread in the Q/dO loader
  static constexpr int KPK = kBwdBN * UPR / kBwdThreads;  // keys per thread in the K^T loader
  // LDS element offsets
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + BQ * D;
  static constexpr int OFF_QT = OFF_DO + BQ * D;
  static constexpr int OFF_DOT = OFF_QT + D * BQ;
  static constexpr int OFF_DS = OFF_DOT + D * BQ;
  static constexpr int OFF_KT = OFF_DS + BQ * kBwdBN;
  static constexpr int ELEMS = OFF_KT + D * kBwdBN;
  static constexpr size_t SMEM = (size_t)ELEMS * sizeof(T) + 2 * BQ * sizeof(float);
};

// swizzles of 8-element units
__device__ __forceinline__ int swz_rows(int row) { return row & 7; }             // row-major tiles
__device__ __forceinline__ int swz_t8(int d) { return (d ^ (d >> 3)) & 7; }      // [d][64]
__device__ __forceinline__ int swz_t4(int d) { return (d ^ (d >> 2)) & 3; }      // [d][32]
__device__ __forceinline__ int swz_t16(int d) { return (d ^ (d >> 3)) & 15; }    // [d][128]

template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(kBwdThreads) void attn_bwd_kernel(
    Meta m, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    float* __restrict__ dQacc, T* __restrict__ dK, T* __restrict__ dV, float scale,
    float scale_log2) {
  typedef typename Vec8<T>::type V8;
  typedef BwdCfg<T, D> C;
  constexpr int QB = C::QB, BQ = C::BQ, UPR = C::UPR, KS = C::KS, DB = C::DB, QU = C::QU;
  constexpr int KPQ = C::KPQ, KPK = C::KPK;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* const lds = reinterpret_cast<T*>(smem_raw);
  T* const Qs = lds + C::OFF_Q;
  T* const dOs = lds + C::OFF_DO;
  T* const QTs = lds + C::OFF_QT;
  T* const dOTs = lds + C::OFF_DOT;
  T* const dSs = lds + C::OFF_DS;
  T* const KTs = lds + C::OFF_KT;
  float* const lse2_s = reinterpret_cast<float*>(lds + C::ELEMS);
  float* const delta_s = lse2_s + BQ;

  const Item it = m.bwd_items[blockIdx.x];
  if (it.sample < 0) return;
  const SampleInfo si = m.sinfo[it.sample];
  const int L = si.len;
  const size_t RS = (size_t)m.n_heads * D;
  const size_t base = (size_t)si.start * RS + (size_t)it.head * D;
  const int kv0 = it.tile * kBwdBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // rotate one 8-element unit of local row `row` (RoPE on load)
  auto rot = [&](V8 v, int row, int unit) -> V8 {
    if (!ROPE || row >= L) return v;
    int r, c;
    token_pos(row, si.l_text, si.w_lat, r, c);
    return from_f32x8<T>(rope_chunk(to_f32x8(v), unit, D, r, c, m.cos_tab, m.sin_tab, m.n_freq,
                                    false));
  };

  // ---- this wave's 32 keys: K' and V rows as B operands (registers) ----
  const int my_key = kv0 + wave * 32 + l32;
  V8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int unit = 2 * ks + hi;
    V8 z = {};
    V8 kv = my_key < L ? load8<T>(K + base + (size_t)my_key * RS + unit * 8) : z;
    kf[ks] = rot(kv, my_key, unit);
    vf[ks] = my_key < L ? load8<T>(V + base + (size_t)my_key * RS + unit * 8) : z;
  }
  // ---- K'^T for the whole 128-key tile into LDS ([d][key]) ----
  {
    const int dc = tid % UPR;
    const int k0 = (tid / UPR) * KPK;
    V8 kr[KPK];
#pragma unroll
    for (int i = 0; i < KPK; ++i) {
      const int kk = kv0 + k0 + i;
      V8 z = {};
      kr[i] = rot(kk < L ? load8<T>(K + base + (size_t)kk * RS + dc * 8) : z, kk, dc);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = dc * 8 + j;
      typedef T VK __attribute__((ext_vector_type(KPK)));
      VK w;
#pragma unroll
      for (int i = 0; i < KPK; ++i) w[i] = kr[i][j];
      *reinterpret_cast<VK*>(KTs + d * kBwdBN + (((k0 >> 3) ^ swz_t16(d)) << 3) + (k0 & 7)) = w;
    }
  }

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  const int nq = (L + BQ - 1) / BQ;
  const float* lse_h = LSE + (size_t)it.head * m.n_tokens + si.start;
  const float* delta_h = DELTA + (size_t)it.head * m.n_tokens + si.start;

  for (int qt = 0; qt < nq; ++qt) {
    const int q0 = qt * BQ;
    // ---- load the query tile: Q' and dO, row-major (sigma rows) and transposed ----
    {
      const int dc = tid % UPR;
      const int r0 = (tid / UPR) * KPQ;
      V8 qr[KPQ], gr[KPQ];
#pragma unroll
      for (int i = 0; i < KPQ; ++i) {
        const int qq = q0 + r0 + i;
        V8 z = {};
        qr[i] = rot(qq < L ? load8<T>(Q + base + (size_t)qq * RS + dc * 8) : z, qq, dc);
        gr[i] = qq < L ? load8<T>(dO + base + (size_t)qq * RS + dc * 8) : z;
      }
#pragma unroll
      for (int i = 0; i < KPQ; ++i) {
        const int rho = (r0 + i) ^ (bsigma((r0 + i) & 31) ^ ((r0 + i) & 31));
        store8<T>(Qs + rho * D + ((dc ^ swz_rows(rho)) << 3), qr[i]);
        store8<T>(dOs + rho * D + ((dc ^ swz_rows(rho)) << 3), gr[i]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = dc * 8 + j;
        const int sw = QU == 8 ? swz_t8(d) : swz_t4(d);
        const int off = d * BQ + (((r0 >> 3) ^ sw) << 3) + (r0 & 7);
        typedef T VQ __attribute__((ext_vector_type(KPQ)));
        VQ a, b;
#pragma unroll
        for (int i = 0; i < KPQ; ++i) {
          a[i] = qr[i][j];
          b[i] = gr[i][j];
        }
        *reinterpret_cast<VQ*>(QTs + off) = a;
        *reinterpret_cast<VQ*>(dOTs + off) = b;
      }
      if (tid < BQ) {
        const int qq = q0 + tid;
        // queries past the end: LSE = +inf makes P = 0
        lse2_s[tid] = qq < L ? lse_h[qq] * 1.4426950408889634f : INFINITY;
        delta_s[tid] = qq < L ? delta_h[qq] : 0.f;
      }
    }
    __syncthreads();

    // ---- S = Q' K'^T and dP = dO V^T, then P and dS (lane = key) ----
    V8 pf[QB][2], sf[QB][2];  // A operands of dV / dK: [q-block][k-step of 16 queries]
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 s = {}, dp = {};
      const int rho = qb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int u = ((2 * ks + hi) ^ swz_rows(rho)) << 3;
        mma16(s, load8<T>(Qs + rho * D + u), kf[ks]);
        mma16(dp, load8<T>(dOs + rho * D + u), vf[ks]);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int qbase = qb * 32 + 16 * st + 8 * hi;  // this lane's 8 queries
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse2_s + qbase);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse2_s + qbase + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(delta_s + qbase);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(delta_s + qbase + 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * st + j;
          const float lj = j < 4 ? l0[j] : l1[j - 4];
          const float dj = j < 4 ? d0[j] : d1[j - 4];
          float p = fast_exp2(fmaf(s[r], scale_log2, -lj));
          if (my_key >= L) p = 0.f;
          const float ds = p * (dp[r] - dj);
          pf[qb][st][j] = (T)p;
          sf[qb][st][j] = (T)ds;
        }
      }
    }
    // ---- dV += P^T dO, dK' += dS^T Q' ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + l32;
      const int sw = QU == 8 ? swz_t8(d) : swz_t4(d);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int off = d * BQ + (((4 * qb + 2 * st + hi) ^ sw) << 3);
          mma16(dv_acc[db], pf[qb][st], load8<T>(dOTs + off));
          mma16(dk_acc[db], sf[qb][st], load8<T>(QTs + off));
        }
    }
    // ---- dS -> LDS as [query][key] ----
    {
      const int key = wave * 32 + l32;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int q = qb * 32 + 16 * st + 8 * hi + j;
            dSs[q * kBwdBN + (((key >> 3) ^ (q & 15)) << 3) + (key & 7)] = sf[qb][st][j];
          }
    }
    __syncthreads();
    // ---- dQ' (queries x one 32-wide d block) over the 128 keys; atomics ----
    for (int wu = wave; wu < QB * DB; wu += 4) {
      const int qb = wu / DB, db = wu % DB;
      f32x16 acc = {};
      const int q = qb * 32 + l32;
      const int d = db * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < kBwdBN / 16; ++ks) {
        const int u = 2 * ks + hi;
        const V8 a = load8<T>(dSs + q * kBwdBN + ((u ^ (q & 15)) << 3));
        const V8 b = load8<T>(KTs + d * kBwdBN + ((u ^ swz_t16(d)) << 3));
        mma16(acc, a, b);
      }
      // acc register r: query qb*32 + 8(r/4) + 4 hi + r%4, column d
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = q0 + qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (qq < L) unsafeAtomicAdd(dQacc + base + (size_t)qq * RS + d, acc[r] * scale);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: dK = R^T (s dK'), dV; staged through LDS for row-major stores ----
  float* const stage = reinterpret_cast<float*>(smem_raw);  // [128][D] fp32 fits in the tile LDS
  static_assert((size_t)kBwdBN * D * sizeof(float) <= C::SMEM, "epilogue staging");
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16* acc = pass == 0 ? dk_acc : dv_acc;
    const float mul = pass == 0 ? scale : 1.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = wave * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        stage[key * D + db * 32 + l32] = acc[db][r] * mul;
      }
    __syncthreads();
    T* out = pass == 0 ? dK : dV;
    for (int e = tid; e < kBwdBN * UPR; e += kBwdThreads) {
      const int row = e / UPR, unit = e % UPR;
      const int kk = kv0 + row;
      if (kk < L) {
        f32x8 x = *reinterpret_cast<const f32x8*>(stage + row * D + unit * 8);
        if (ROPE && pass == 0) {
          int r, c;
          token_pos(kk, si.l_text, si.w_lat, r, c);
          x = rope_chunk(x, unit, D, r, c, m.cos_tab, m.sin_tab, m.n_freq, true);
        }
        store8<T>(out + base + (size_t)kk * RS + unit * 8, from_f32x8<T>(x));
      }
    }
    __syncthreads();
  }
}

template <typename T, int D, bool ROPE>
static hipError_t launch_bwd_t(const Meta& m, const void* q, const void* k, const void* v,
                               const void* dout, const float* lse, const float* delta,
                               float* dq_acc, void* dk, void* dv, float scale,
                               hipStream_t stream) {
  auto kern = attn_bwd_kernel<T, D, ROPE>;
  const size_t smem = BwdCfg<T, D>::SMEM;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kern<<<dim3(m.n_bwd), dim3(kBwdThreads), smem, stream>>>(
      m, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse, delta, dq_acc, (T*)dk,
      (T*)dv, scale, scale * 1.4426950408889634f);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, const void* dout, const float* lse,
                           const float* delta, float* dq_acc, void* dk, void* dv, float scale,
                           bool rope, hipStream_t stream) {
  if (m.n_bwd == 0) return hipSuccess;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int D = p->desc.head_dim;
#define PVJ_BWD(TT, DD)                                                                     \
  return rope ? launch_bwd_t<TT, DD, true>(m, q, k, v, dout, lse, delta, dq_acc, dk, dv,    \
                                           scale, stream)                                   \
              : launch_bwd_t<TT, DD, false>(m, q, k, v, dout, lse, delta, dq_acc, dk, dv,   \
                                            scale, stream)
  if (bf && D == 128) PVJ_BWD(bf16, 128);
  if (bf && D == 64) PVJ_BWD(bf16, 64);
  if (!bf && D == 128) PVJ_BWD(float, 128);
  PVJ_BWD(float, 64);
#undef PVJ_BWD
}

}  // namespace pvj
