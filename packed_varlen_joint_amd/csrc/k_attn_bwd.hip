// Packed variable-length joint attention, backward dK/dV pass, for gfx950.
//
// Training runs forward + backward through the joint attention (Mage-Flow
// review page, section "Kernel fusion": 8-GPU training at ~50K packed tokens
// per GPU).  Gradients of sum(O * dO), per sample and head:
//   P = exp(s Q'K'^T - LSE); dV = P^T dO; dP = dO V^T; dS = P * (dP - Delta);
//   dK' = s dS^T Q'; dQ' = s dS K'; with RoPE, dK = R^T dK' and dQ = R^T dQ'.
// Two kernels, no atomics, fully deterministic: this file's dK/dV kernel and
// the dQ kernel (k_attn_dq.hip).  With RoPE, the preprocess kernel writes
// Q' = R Q and K' = R K once into the workspace, so both read pre-rotated
// operands.
//
// attn_bwd_dkdv_kernel: one workgroup per (sample, head, 128-key tile), 4
// waves x 32 keys; bf16 fits two workgroups per CU (two waves per SIMD: 64.5
// KB of LDS and at most 256 registers each), so one wave's softmax work fills
// the other's matrix-core gaps.  K' is held in registers; V (bf16) is copied
// once into LDS (registers cannot hold it beside the 128 accumulators at that
// occupancy).  The sample's query tiles (32 rows) stream through
// double-buffered LDS.  S = Q'K'^T and dP = dO V^T put one key per lane (A =
// Q' / dO rows stored in LDS in sigma row order, bits 2 and 3 swapped), so the
// accumulators of P and dS are directly the A operands (rows = keys, k = 16
// consecutive queries) of dV += P^T dO and dK' += dS^T Q'.  Their B operands
// (k = queries, n = d) are read from the same row-major LDS tiles with the
// transposing ds_read_b64_tr_b16.  The epilogue stages 64 keys at a time
// through the LDS of the V copy.

#include <type_traits>

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kBwdBN = 128;  // keys per dK/dV workgroup (must match bwd_tile_rows)
constexpr int kBwdThreads = kTileThreads;

// ===========================================================================
// dK, dV
// ===========================================================================
template <typename T, int D>
struct DkdvCfg {
  static constexpr int BQ = 32;  // queries per streamed tile
  static constexpr int UPR = D / 8;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KPQ = BQ * UPR / kBwdThreads;  // rows per thread in the staged loader
  static constexpr int TILE = BQ * D;                 // elements of one Q (or dO) tile
};

template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(
    sizeof(T) == 2 ? 2 : 1, sizeof(T) == 2 ? 2 : 1))) void attn_bwd_dkdv_kernel(
    Meta m, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ DELTA,
    T* __restrict__ dK, T* __restrict__ dV, float scale, float scale_log2, int rope) {
  typedef typename Vec8<T>::type V8;
  typedef DkdvCfg<T, D> C;
  constexpr int BQ = C::BQ, UPR = C::UPR, KS = C::KS, DB = C::DB, KPQ = C::KPQ;
  constexpr bool DMA = sizeof(T) == 2;

  // separate static buffers, so the compiler can tell the next tile's
  // direct-to-LDS copies from the current tile's reads
  __shared__ __align__(16) T q_b0[C::TILE], q_b1[C::TILE], g_b0[C::TILE], g_b1[C::TILE];
  __shared__ __align__(16) float l_b0[2 * BQ], l_b1[2 * BQ];  // LSE*log2(e), then Delta
  // bf16: the key tile's V rows (B operands of dP); after the loop the same
  // LDS stages the epilogue, 64 keys of fp32 at a time
  __shared__ __align__(16) T v_t[DMA ? kBwdBN * D : 8];
  __shared__ __align__(16) float stage_own[DMA ? 8 : kBwdBN / 2 * D];
  static_assert(!DMA || sizeof(v_t) >= kBwdBN / 2 * D * sizeof(float), "epilogue staging");
  float* const stage = DMA ? reinterpret_cast<float*>(v_t) : stage_own;

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

  // this wave's 32 keys of K' (and of V for fp32) as B operands in registers;
  // rows past the end are zero and need no mask: their dK, dV rows are never
  // stored, and dS feeds only dK of its own key
  const int my_key = kv0 + wave * 32 + l32;
  V8 kf[KS], vf[DMA ? 1 : KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int unit = 2 * ks + hi;
    V8 z = {};
    kf[ks] = my_key < L ? load8<T>(K + base + (size_t)my_key * RS + unit * 8) : z;
    if constexpr (!DMA)
      vf[ks] = my_key < L ? load8<T>(V + base + (size_t)my_key * RS + unit * 8) : z;
  }
  if constexpr (DMA) {
    // the key tile's V rows, natural order, swizzled units
    constexpr int VPT = kBwdBN * UPR / kBwdThreads;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = i * kBwdThreads + tid;
      const int row = e / UPR, u = e % UPR;
      V8 z = {};
      const V8 x = kv0 + row < L ? load8<T>(V + base + (size_t)(kv0 + row) * RS + u * 8) : z;
      store8<T>(v_t + toff<D>(row, u * 8), x);
    }
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
  // bases of output block db and half t; the 16-query half and the buffer add
  // compile-time offsets.  The empty asm keeps them in registers.
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
  // A-operand row read (row l32, unit 2ks+hi) and transposed fragment (rows
  // kbase.., columns db*32..) of a Q' or dO tile
  auto rowfrag = [&](const T* t, int ks) -> V8 {
    if constexpr (DMA)
      return *reinterpret_cast<const V8*>(reinterpret_cast<const char*>(t) + qa[ks]);
    else
      return load8<T>(t + toff<D>(l32, (2 * ks + hi) * 8));
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

  // the wave's V rows as B operands: from the LDS copy (bf16: its rows use
  // the Q' tiles' unit layout, 32 rows further per wave), else registers
  auto vfrag = [&](int ks) -> V8 {
    if constexpr (DMA)
      return *reinterpret_cast<const V8*>(reinterpret_cast<const char*>(v_t) + qa[ks] +
                                          wave * 32 * D * sizeof(T));
    else
      return vf[ks];
  };
  // S and dP of the 32-query tile (A = Q', dO rows from LDS; B = K', V)
  auto sdp = [&](const T* qs, const T* gs, f32x16& s, f32x16& dp) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      mma16(s, rowfrag(qs, ks), kf[ks]);
      mma16(dp, rowfrag(gs, ks), vfrag(ks));
    }
  };
  // P = 2^(s*scale*log2e - LSE*log2e) and dS = P (dP - Delta) for element r
  // (query 16(r/8) + 8 hi + r%8) into the A fragments of dV and dK
  auto elem = [&](const float* lb, int r, const f32x16& s, const f32x16& dp, V8 (&pf)[2],
                  V8 (&sf)[2]) {
    const int q = 16 * (r >> 3) + 8 * hi + (r & 7);
    const float p = fast_exp2(fmaf(s[r], scale_log2, -lb[q]));
    pf[r >> 3][r & 7] = (T)p;
    sf[r >> 3][r & 7] = (T)(p * (dp[r] - lb[BQ + q]));
  };
  // dV += P^T dO and dK' += dS^T Q' (B operands by transposing reads)
  auto dvdk = [&](const T* qs, const T* gs, V8 (&pf)[2], V8 (&sf)[2]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        mma16(dv_acc[db], pf[st], colfrag(gs, 16 * st, db));
        mma16(dk_acc[db], sf[st], colfrag(qs, 16 * st, db));
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
    // S and dP run at raised wave priority, so the SIMD's other wave (another
    // workgroup) fills their gaps with its softmax and dV/dK work (measured:
    // raising it for the dV/dK products too, or for neither, is slower)
    f32x16 sacc = {}, dpacc = {};
    V8 pf[2], sf[2];
    __builtin_amdgcn_s_setprio(1);
    sdp(qs, gs, sacc, dpacc);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int r = 0; r < 16; ++r) elem(lb, r, sacc, dpacc, pf, sf);
    dvdk(qs, gs, pf, sf);
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
    for (int half = 0; half < 2; ++half) {
      if ((wave >> 1) == half) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = (wave & 1) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            stage[key * D + db * 32 + l32] = acc[db][r] * mul;
          }
      }
      __syncthreads();
      T* out = pass == 0 ? dK : dV;
      for (int e = tid; e < kBwdBN / 2 * UPR; e += kBwdThreads) {
        const int row = e / UPR, unit = e % UPR;
        const int kk = kv0 + half * (kBwdBN / 2) + row;
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
}

template <typename T, int D>
static hipError_t launch_dkdv_t(const Meta& m, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const float* delta, void* dk,
                                void* dv, float scale, bool rope, hipStream_t stream) {
  if (m.n_bwd > 0)
    attn_bwd_dkdv_kernel<T, D><<<dim3(m.n_bwd), dim3(kBwdThreads), 0, stream>>>(
        m, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, lse, delta, (T*)dk, (T*)dv,
        scale, scale * 1.4426950408889634f, rope ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const pvj_plan* p, const Meta& m, int which, const void* q,
                           const void* k, const void* v, const void* dout, const float* lse,
                           const float* delta, void* dq, void* dk, void* dv, float scale,
                           bool rope, hipStream_t stream) {
  if (which != 0)
    return launch_attn_bwd_dq(p, m, q, k, v, dout, lse, delta, dq, scale, rope, stream);
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int D = p->desc.head_dim;
#define PVJ_BWD(TT, DD) \
  return launch_dkdv_t<TT, DD>(m, q, k, v, dout, lse, delta, dk, dv, scale, rope, stream)
  if (bf && D == 128) PVJ_BWD(bf16, 128);
  if (bf && D == 64) PVJ_BWD(bf16, 64);
  if (!bf && D == 128) PVJ_BWD(float, 128);
  PVJ_BWD(float, 64);
#undef PVJ_BWD
}

}  // namespace pvj
