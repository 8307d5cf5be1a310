// Packed variable-length joint attention, backward, for gfx950.
//
// Training runs forward + backward through the joint attention (Mage-Flow
// review page, section "Kernel fusion": 8-GPU training at ~50K packed tokens
// per GPU).  Gradients of sum(O * dO), per sample and head:
//   P = exp(s Q'K'^T - LSE); dV = P^T dO; dP = dO V^T; dS = P * (dP - Delta);
//   dK' = s dS^T Q'; dQ' = s dS K'; with RoPE, dK = R^T dK' and dQ = R^T dQ'.
//
// Two kernels, no atomics, fully deterministic:
//  * attn_bwd_dkdv_kernel: one workgroup per (sample, head, 128-key tile);
//    4 waves x 32 keys with K' and V in registers; walks the sample's query
//    tiles (64 rows bf16, 32 rows fp32) through double-buffered LDS.
//    S = Q'K'^T and dP = dO V^T put one key per lane (A = Q' / dO rows stored
//    in LDS in sigma row order, bits 2 and 3 swapped), so the accumulators of
//    P and dS are directly the A operands (rows = keys, k = 16 consecutive
//    queries) of dV += P^T dO and dK' += dS^T Q'.  Their B operands (k =
//    queries, n = d) are read from the same row-major LDS tiles with the
//    transposing ds_read_b64_tr_b16.
//  * attn_bwd_dq_kernel: one workgroup per (sample, head, 128-query tile);
//    4 waves x 32 queries with Q' and dO in registers; streams 64-key tiles of
//    K' and V through double-buffered LDS like the forward.  S^T = K'Q'^T and
//    dP^T = V dO^T put one query per lane (LSE and Delta are per-lane scalars);
//    dQ'^T += K'^T dS^T takes dS^T straight from the accumulators and K'^T by
//    transposing reads.  The epilogue scales, applies R^T (rotation pairs are
//    in one lane) and stores dQ in the output dtype.
// With RoPE, the preprocess kernel writes Q' = R Q and K' = R K once into the
// workspace, so both kernels read pre-rotated operands.

#include <type_traits>

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kBwdBN = 128;   // keys per dK/dV workgroup (must match bwd_tile_rows)
constexpr int kDqBM = 128;    // queries per dQ workgroup (= forward tile, uses fwd_items)
constexpr int kDqBN = 64;     // keys per streamed tile in the dQ kernel
constexpr int kBwdThreads = 256;

// ===========================================================================
// dK, dV
// ===========================================================================
template <typename T, int D>
struct DkdvCfg {
  static constexpr int QB = sizeof(T) == 2 ? 2 : 1;  // 32-query blocks per tile
  static constexpr int BQ = 32 * QB;
  static constexpr int UPR = D / 8;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KPQ = BQ * UPR / kBwdThreads;  // rows per thread in the staged loader
  static constexpr int TILE = BQ * D;                 // elements of one Q (or dO) tile
};

template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void attn_bwd_dkdv_kernel(
    Meta m, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    T* __restrict__ dK, T* __restrict__ dV, float scale, float scale_log2, int rope) {
  typedef typename Vec8<T>::type V8;
  typedef DkdvCfg<T, D> C;
  constexpr int QB = C::QB, BQ = C::BQ, UPR = C::UPR, KS = C::KS, DB = C::DB, KPQ = C::KPQ;
  constexpr bool DMA = sizeof(T) == 2;

  // separate static buffers, so the compiler can tell the next tile's
  // direct-to-LDS copies from the current tile's reads
  __shared__ __align__(16) T q_b0[C::TILE], q_b1[C::TILE], g_b0[C::TILE], g_b1[C::TILE];
  __shared__ __align__(16) float l_b0[2 * BQ], l_b1[2 * BQ];  // LSE*log2(e), then Delta
  __shared__ __align__(16) float stage[kBwdBN * D];           // epilogue staging

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

  // this wave's 32 keys as B operands (registers); rows past the end are zero
  // and need no mask: their dK, dV rows are never stored, and dS feeds only
  // dK of its own key
  const int my_key = kv0 + wave * 32 + l32;
  V8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int unit = 2 * ks + hi;
    V8 z = {};
    kf[ks] = my_key < L ? load8<T>(K + base + (size_t)my_key * RS + unit * 8) : z;
    vf[ks] = my_key < L ? load8<T>(V + base + (size_t)my_key * RS + unit * 8) : z;
  }

  // ---- query-tile loader ----
  const int ld_unit = tid % UPR;
  const int ld_r0 = (tid / UPR) * KPQ;
  V8 qr[DMA ? 1 : KPQ], gr[DMA ? 1 : KPQ];
  float lr = 0.f, dr = 0.f;
  const float* lse_h = LSE + (size_t)it.head * m.n_tokens + si.start;
  const float* del_h = DELTA + (size_t)it.head * m.n_tokens + si.start;
  // direct copies: Q and dO tiles share one layout; rows past the sample end
  // arrive as zeros (outside the buffer resources)
  typedef DmaTile<D, BQ> DT;
  const DT dma(RS);
  const typename DT::Src rq = DT::src(Q + base, RS, L), rg = DT::src(dO + base, RS, L);
  auto load_q = [&](int q0, int b) {
    // LSE and Delta first: the wait for them (in-order counter) then leaves the
    // tile copies in flight
    if (tid < BQ) {
      const int qq = q0 + tid;
      // queries past the end: LSE = +inf makes P = 0 (their rows read as zeros)
      lr = qq < L ? lse_h[qq] : INFINITY;
      dr = qq < L ? del_h[qq] : 0.f;
    }
    if constexpr (DMA) {
      dma.copy(b ? q_b1 : q_b0, rq, RS, q0);
      dma.copy(b ? g_b1 : g_b0, rg, RS, q0);
    } else {
#pragma unroll
      for (int i = 0; i < KPQ; ++i) {
        const int qq = q0 + ld_r0 + i;
        V8 z = {};
        qr[i] = qq < L ? load8<T>(Q + base + (size_t)qq * RS + ld_unit * 8) : z;
        gr[i] = qq < L ? load8<T>(dO + base + (size_t)qq * RS + ld_unit * 8) : z;
      }
    }
  };
  auto store_q = [&](int b) {
    if constexpr (DMA) {
      wait_dma();
    } else {
#pragma unroll
      for (int i = 0; i < KPQ; ++i) {
        const int rho = bsigma(ld_r0 + i);
        store8<T>((b ? q_b1 : q_b0) + toff<D>(rho, ld_unit * 8), qr[i]);
        store8<T>((b ? g_b1 : g_b0) + toff<D>(rho, ld_unit * 8), gr[i]);
      }
    }
    if (tid < BQ) {
      (b ? l_b1 : l_b0)[tid] = lr * 1.4426950408889634f;
      (b ? l_b1 : l_b0)[BQ + tid] = dr;
    }
  };
  auto sig = [](int q) { return bsigma(q); };

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  // Per-lane LDS addresses, fixed for the whole loop (bf16): row l32 at unit
  // 2ks+hi of the Q' and dO tiles (same layout), and the transposed fragment
  // bases of output block db and half t; the 32-query block, the 16-query
  // half and the buffer add compile-time offsets.  The empty asm keeps them
  // in registers.
  uint32_t qa[KS], fa[DB][2];
  if constexpr (DMA) {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[ks] = (uint32_t)(toff<D>(l32, (2 * ks + hi) * 8) * sizeof(T));
      asm volatile("" : "+v"(qa[ks]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        fa[db][t] = (uint32_t)(toff<D>(bsigma(8 * (g >> 1) + 4 * t + (sl >> 2)),
                                       db * 32 + 16 * (g & 1) + 4 * (sl & 3)) * sizeof(T));
        asm volatile("" : "+v"(fa[db][t]));
      }
  }
  // A-operand row read (row qb*32 + l32, unit 2ks+hi) and transposed fragment
  // (rows kbase.., columns db*32..) of a Q' or dO tile
  auto rowfrag = [&](const T* t, int qb, int ks) -> V8 {
    if constexpr (DMA)
      return *reinterpret_cast<const V8*>(reinterpret_cast<const char*>(t) + qa[ks] +
                                          qb * 32 * D * sizeof(T));
    else
      return load8<T>(t + toff<D>(qb * 32 + l32, (2 * ks + hi) * 8));
  };
  auto colfrag = [&](const T* t, int kbase, int db) -> V8 {
    if constexpr (DMA) {
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      V8 f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const i16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(reinterpret_cast<const char*>(t) + fa[db][tt] + kbase * D * sizeof(T)));
        const bf16x4 h = __builtin_bit_cast(bf16x4, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[4 * tt + e] = h[e];
      }
      return f;
    } else {
      return frag_t<D>(t, kbase, db * 32, sig);
    }
  };

  // S and dP of one 32-query block (A = Q', dO rows from LDS; B = K', V registers)
  auto sdp = [&](const T* qs, const T* gs, int qb, f32x16& s, f32x16& dp) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      mma16(s, rowfrag(qs, qb, ks), kf[ks]);
      mma16(dp, rowfrag(gs, qb, ks), vf[ks]);
    }
    // keep six operand reads in flight ahead of the products
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // P = 2^(s*scale*log2e - LSE*log2e) and dS = P (dP - Delta) for element r
  // (query qb*32 + 16(r/8) + 8 hi + r%8) into the A fragments of dV and dK
  auto elem = [&](const float* lb, int qb, int r, const f32x16& s, const f32x16& dp,
                  V8 (&pf)[2], V8 (&sf)[2]) {
    const int q = qb * 32 + 16 * (r >> 3) + 8 * hi + (r & 7);
    const float p = fast_exp2(fmaf(s[r], scale_log2, -lb[q]));
    pf[r >> 3][r & 7] = (T)p;
    sf[r >> 3][r & 7] = (T)(p * (dp[r] - lb[BQ + q]));
  };
  // dV += P^T dO and dK' += dS^T Q' for one block (B = transposing reads); the
  // optional `fill` runs between the products (independent VALU work)
  auto dvdk = [&](const T* qs, const T* gs, int qb, V8 (&pf)[2], V8 (&sf)[2], auto fill) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kbase = qb * 32 + 16 * st;
        mma16(dv_acc[db], pf[st], colfrag(gs, kbase, db));
        fill(4 * db + 2 * st);
        mma16(dk_acc[db], sf[st], colfrag(qs, kbase, db));
        fill(4 * db + 2 * st + 1);
      }
  };

  const int nq = (L + BQ - 1) / BQ;
  load_q(0, 0);
  store_q(0);
  __syncthreads();
  // the query-tile loop is unrolled by two so the buffer is a compile-time choice
  auto step = [&](int qt, auto bc) {
    constexpr int B = decltype(bc)::value;
    if (qt + 1 < nq) load_q((qt + 1) * BQ, B ^ 1);
    const T* qs = B ? q_b1 : q_b0;
    const T* gs = B ? g_b1 : g_b0;
    const float* lb = B ? l_b1 : l_b0;
    if constexpr (QB == 2) {
      // software pipeline over the two query blocks: the softmax VALU work of
      // one block sits between the matrix products of the other
      f32x16 s0 = {}, dp0 = {}, s1 = {}, dp1 = {};
      V8 pf0[2], sf0[2], pf1[2], sf1[2];
      sdp(qs, gs, 0, s0, dp0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        mma16(s1, rowfrag(qs, 1, ks), kf[ks]);
        mma16(dp1, rowfrag(gs, 1, ks), vf[ks]);
#pragma unroll
        for (int e = 0; e < 16 / KS; ++e) elem(lb, 0, (16 / KS) * ks + e, s0, dp0, pf0, sf0);
      }
      dvdk(qs, gs, 0, pf0, sf0, [&](int slot) {
        constexpr int PER = 16 / (4 * DB);  // elements of block 1 per product slot
#pragma unroll
        for (int e = 0; e < PER; ++e) elem(lb, 1, PER * slot + e, s1, dp1, pf1, sf1);
      });
      dvdk(qs, gs, 1, pf1, sf1, [](int) {});
    } else {
      f32x16 s0 = {}, dp0 = {};
      V8 pf0[2], sf0[2];
      sdp(qs, gs, 0, s0, dp0);
#pragma unroll
      for (int r = 0; r < 16; ++r) elem(lb, 0, r, s0, dp0, pf0, sf0);
      dvdk(qs, gs, 0, pf0, sf0, [](int) {});
    }
    if (qt + 1 < nq) store_q(B ^ 1);
    __syncthreads();
  };
  int qt = 0;
  for (; qt + 1 < nq; qt += 2) {
    step(qt, std::integral_constant<int, 0>{});
    step(qt + 1, std::integral_constant<int, 1>{});
  }
  if (qt < nq) step(qt, std::integral_constant<int, 0>{});

  // ---- epilogue: dK = R^T (s dK'), dV; staged through LDS for row-major stores ----
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
        if (rope && pass == 0)
          x = rope_unit(x, unit, axis_pos(token_pos3(kk, si), unit_axis(unit, m)), m, true);
        store8<T>(out + base + (size_t)kk * RS + unit * 8, from_f32x8<T>(x));
      }
    }
    __syncthreads();
  }
}

// ===========================================================================
// dQ
// ===========================================================================
template <typename T, int D>
struct DqCfg {
  static constexpr int UPR = D / 8;
  static constexpr int NK = kDqBN * UPR / kBwdThreads;  // units per thread per tile (K and V)
  static constexpr int TILE = kDqBN * D;
};

// bf16 fits two waves per SIMD (two workgroups per CU, 64 KB of LDS each)
template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(
    sizeof(T) == 2 ? 2 : 1, sizeof(T) == 2 ? 2 : 1))) void attn_bwd_dq_kernel(
    Meta m, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    T* __restrict__ dQ, float scale, float scale_log2, int rope) {
  typedef typename Vec8<T>::type V8;
  typedef DqCfg<T, D> C;
  constexpr int KS = D / 16, DB = D / 32, UPR = C::UPR, NK = C::NK;

  // separate static buffers (see the dK/dV kernel)
  __shared__ __align__(16) T k_b0[C::TILE], k_b1[C::TILE], v_b0[C::TILE], v_b1[C::TILE];
  auto ks_of = [&](int b) { return b ? k_b1 : k_b0; };
  auto vs_of = [&](int b) { return b ? v_b1 : v_b0; };

  const Item it = m.fwd_items[blockIdx.x];
  if (it.sample < 0) return;
  const SampleInfo si = m.sinfo[it.sample];
  const int L = si.len;
  const size_t RS = (size_t)m.n_heads * D;
  const size_t base = (size_t)si.start * RS + (size_t)it.head * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qi = it.tile * kDqBM + wave * 32 + l32;  // this lane's query

  V8 qf[KS], gf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int unit = 2 * ks + hi;
    V8 z = {};
    qf[ks] = qi < L ? load8<T>(Q + base + (size_t)qi * RS + unit * 8) : z;
    gf[ks] = qi < L ? load8<T>(dO + base + (size_t)qi * RS + unit * 8) : z;
  }
  const float lse2 = qi < L ? LSE[(size_t)it.head * m.n_tokens + si.start + qi] *
                                  1.4426950408889634f : INFINITY;
  const float delta = qi < L ? DELTA[(size_t)it.head * m.n_tokens + si.start + qi] : 0.f;

  const int k_unit = tid % UPR;
  const int k_row0 = tid / UPR;
  constexpr int K_ROW_STEP = kBwdThreads / UPR;
  constexpr bool DMA = sizeof(T) == 2;
  V8 kreg[DMA ? 1 : NK], vreg[DMA ? 1 : NK];
  // direct copies (K and V tiles share one layout; rows past the end are zeros)
  typedef DmaTile<D, kDqBN> DT;
  const DT dma(RS);
  const typename DT::Src rk = DT::src(K + base, RS, L), rv = DT::src(V + base, RS, L);
  auto load_kv = [&](int kv0, int b) {
    if constexpr (DMA) {
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
    T* row = dQ + base + (size_t)qi * RS;
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

template <typename T, int D>
static hipError_t launch_bwd_t(const Meta& m, int which, const void* q, const void* k,
                               const void* v, const void* dout, const float* lse,
                               const float* delta, void* dq, void* dk, void* dv, float scale,
                               bool rope, hipStream_t stream) {
  const float sl2 = scale * 1.4426950408889634f;
  if (which == 0) {
    auto ka = attn_bwd_dkdv_kernel<T, D>;
    if (m.n_bwd > 0)
      ka<<<dim3(m.n_bwd), dim3(kBwdThreads), 0, stream>>>(
          m, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse, delta, (T*)dk, (T*)dv,
          scale, sl2, rope ? 1 : 0);
  } else {
    auto kb = attn_bwd_dq_kernel<T, D>;
    if (m.n_fwd > 0)
      kb<<<dim3(m.n_fwd), dim3(kBwdThreads), 0, stream>>>(
          m, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse, delta, (T*)dq, scale,
          sl2, rope ? 1 : 0);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const pvj_plan* p, const Meta& m, int which, const void* q,
                           const void* k, const void* v, const void* dout, const float* lse,
                           const float* delta, void* dq, void* dk, void* dv, float scale,
                           bool rope, hipStream_t stream) {
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int D = p->desc.head_dim;
#define PVJ_BWD(TT, DD) \
  return launch_bwd_t<TT, DD>(m, which, q, k, v, dout, lse, delta, dq, dk, dv, scale, rope, stream)
  if (bf && D == 128) PVJ_BWD(bf16, 128);
  if (bf && D == 64) PVJ_BWD(bf16, 64);
  if (!bf && D == 128) PVJ_BWD(float, 128);
  PVJ_BWD(float, 64);
#undef PVJ_BWD
}

}  // namespace pvj
