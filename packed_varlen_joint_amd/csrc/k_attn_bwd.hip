// Packed variable-length joint attention, backward dK/dV pass, for gfx950.
//
// Training runs forward + backward through the joint attention (Mage-Flow
// review page, section "Kernel fusion": 8-GPU training at ~50K packed tokens
// per GPU).  Gradients of sum(O * dO), per sample and head:
//   P = exp(s Q'K'^T - LSE); dV = P^T dO; dP = dO V^T; dS = P * (dP - Delta);
//   dK' = s dS^T Q'; dQ' = s dS K'; with RoPE, dK = R^T dK' and dQ = R^T dQ'.
// Two kernels, no atomics, fully deterministic: the dQ kernel
// (k_attn_dq.hip), which also forms Delta, then this file's dK/dV kernel.
// With RoPE on load, Q' = R Q and K' = R K are first written once into the
// workspace by the standalone rotation, so both read pre-rotated operands.
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

constexpr int kBwdBN = 128;  // keys per workgroup of the fp32 kernel (must match bwd_tile_rows)
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

// ---------------------------------------------------------------------------
// bf16 dK/dV with two wave groups offset by half a query tile.
//
// In the kernel above the two workgroups of a CU run in no fixed relation, so
// the two waves of a SIMD often run their softmax work at the same time while
// the matrix cores idle.  Here one workgroup of 8 waves takes 256 keys (32 per
// wave, as above): waves 0-3 (group 0) and 4-7 (group 1) have one wave on every
// SIMD each, and each alternates a matrix phase and a softmax phase:
//   M(j): dV += P_{j-1}^T dO_{j-1} and dK' += dS_{j-1}^T Q'_{j-1} (j >= 1), then
//         S_j = Q'_j K'^T and dP_j = dO_j V^T (j < nq), 32 products (in this
//         order P, dS of tile j - 1 die before S, dP of tile j are live: with
//         the 128 accumulators and K' in registers, both together would not
//         fit 256 registers)
//   E(j): P_j = 2^(S_j s log2e - LSE log2e), dS_j = P_j (dP_j - Delta) (j < nq)
//   group 0: M(j) E(j) | barrier      group 1: M(j) | barrier E(j)
// so after each barrier one wave of a SIMD issues products while the other
// runs its softmax.  M(j) reads query tiles j and j - 1; tile j + 1 is copied
// (by group 0, spread over its products) into the third buffer, whose last
// reader, M(j - 1), both groups finished before barrier j - 1.  Inside M(j)
// the operand reads from LDS run four products ahead.  Every accumulator adds
// the same products in the same order as the kernel above, so both give the
// same bits.
// ---------------------------------------------------------------------------
constexpr int kBwdPpAhead = 4;   // products whose operands are read ahead
constexpr int kBwdPpKeys = 256;  // keys per workgroup (must match bwd_tile_rows)

// LDS reads of product i of a matrix phase with NP transposed-fragment
// products first (two transposing reads each) and then the score products (S
// and dP alternating: one row read for S, a dO row and a V row for dP)
__host__ __device__ constexpr int bwd_pp_reads(int i, int np) {
  return i < np ? 2 : (((i - np) & 1) ? 2 : 1);
}
template <int I, int N, int NP, int NC>
__device__ __forceinline__ void bwd_pp_sched_ops() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I + kBwdPpAhead < N)
      __builtin_amdgcn_sched_group_barrier(0x100, bwd_pp_reads(I + kBwdPpAhead, NP), 0);
    if constexpr (pp_copy_after(I, N, NC)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    bwd_pp_sched_ops<I + 1, N, NP, NC>();
  }
}
__host__ __device__ constexpr int bwd_pp_first_reads(int n, int np) {
  int r = 0;
  for (int i = 0; i < kBwdPpAhead && i < n; ++i) r += bwd_pp_reads(i, np);
  return r;
}
template <int N, int NP, int NC>
__device__ __forceinline__ void bwd_pp_sched() {
  __builtin_amdgcn_sched_group_barrier(0x100, bwd_pp_first_reads(N, NP), 0);
  bwd_pp_sched_ops<0, N, NP, NC>();
}

template <int D, bool SM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_bwd_dkdv_pp_kernel(Meta m, const bf16* __restrict__ Q, const bf16* __restrict__ K,
                        const bf16* __restrict__ V, const bf16* __restrict__ dO,
                        const float* __restrict__ LSE, const float* __restrict__ DELTA,
                        bf16* __restrict__ dK, bf16* __restrict__ dV, float scale,
                        float scale_log2, int rope) {
  constexpr int BQ = 32, THREADS = 512, BN = kBwdPpKeys;
  constexpr int UPR = D / 8, KS = D / 16, DB = D / 32;
  constexpr int TILE = BQ * D;

  // Query-tile buffer B holds Q'_j then dO_j (one object per buffer, so the
  // compiler tells a buffer being copied into from the ones being read; the
  // dO half is a constant offset from the Q' half, so both share each lane's
  // address registers).  Placed below 64 KB (their larger alignment puts them
  // before V), constant offsets inside them fit the reads' offset field.
  __shared__ __align__(64) bf16 qg_b0[2 * TILE], qg_b1[2 * TILE], qg_b2[2 * TILE];
  __shared__ __align__(64) float l_b0[2 * BQ], l_b1[2 * BQ], l_b2[2 * BQ];  // LSE*log2e, Delta
  // the key tile's V rows (B operands of dP); after the loop the same LDS
  // stages the epilogue, 64 keys of fp32 at a time
  __shared__ __align__(16) bf16 v_t[BN * D];
  static_assert(sizeof(v_t) >= 64 * D * sizeof(float), "epilogue staging");
  float* const stage = reinterpret_cast<float*>(v_t);

  const Item it = m.bwd_items[blockIdx.x];
  if (it.sample < 0) return;
  const SampleInfo si = m.sinfo[it.sample];
  const int L = si.len;
  const size_t RS = (size_t)m.n_heads * D;
  const size_t base = (size_t)si.start * RS + (size_t)it.head * D;
  const size_t hb = (size_t)it.head * D;  // a token's row r is at hb + r * RS
  // stream-major copies: from the head's base to the sample's last image row
  const int tbytes = SM ? sm_bytes<D>(si, RS) : 0;
  const uint32_t rsb = (uint32_t)(RS * sizeof(bf16));
  (void)tbytes, (void)rsb;
  const int kv0 = it.tile * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int group = __builtin_amdgcn_readfirstlane(tid >> 8);

  // this wave's 32 keys of K' as B operands in registers (rows past the end
  // are zero: their dK, dV rows are never stored)
  const int my_key = kv0 + wave * 32 + l32;
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 z = {};
    kf[ks] = my_key < L ? load8<bf16>(K + hb + (size_t)token_row<SM>(si, my_key) * RS +
                                      (2 * ks + hi) * 8)
                        : z;
  }
  // the 256 keys' V rows, natural order, swizzled units
  {
    constexpr int VPT = BN * UPR / THREADS;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = i * THREADS + tid;
      const int row = e / UPR, u = e % UPR;
      bf16x8 z = {};
      const bf16x8 x =
          kv0 + row < L ? load8<bf16>(V + hb + (size_t)token_row<SM>(si, kv0 + row) * RS + u * 8)
                        : z;
      store8<bf16>(v_t + toff<D>(row, u * 8), x);
    }
  }

  // query tiles: direct copies by group 0 (rows past the sample end arrive as
  // zeros); LSE and Delta by its first 32 threads through registers
  typedef DmaTile<D, BQ, THREADS / 2> DT;
  constexpr int NC = 2 * DT::PER;  // copy instructions per tile and thread
  const DT dma(RS);
  const uint32_t c1 = SM ? dma.sm_c1(si, rsb) : 0u;  // stream-major image-row offset
  (void)c1;
  const typename DT::Src rq = DT::src(Q + base, RS, L), rg = DT::src(dO + base, RS, L);
  // LSE and Delta are [H, T] in the token tensors' row order
  const float* lse_h = LSE + (size_t)it.head * m.n_tokens;
  const float* del_h = DELTA + (size_t)it.head * m.n_tokens;
  float lr = 0.f, dr = 0.f;
  auto qbuf = [&](auto bc) -> bf16* {
    constexpr int B = decltype(bc)::value;
    return B == 0 ? qg_b0 : (B == 1 ? qg_b1 : qg_b2);
  };
  auto gbuf = [&](auto bc) -> bf16* { return qbuf(bc) + TILE; };
  auto lbuf = [&](auto bc) -> float* {
    constexpr int B = decltype(bc)::value;
    return B == 0 ? l_b0 : (B == 1 ? l_b1 : l_b2);
  };
  // copy instruction c of query tile j into buffer B (a tile at or past the
  // sample end gets an empty buffer resource and reads zeros, into a buffer
  // no later product reads)
  auto copy_part = [&](int j, auto bc, int c) __attribute__((always_inline)) {
    if constexpr (SM) {
      if (c < DT::PER) dma.part_sm(qbuf(bc), Q + hb, tbytes, rsb, c1, si, j * BQ, c);
      else dma.part_sm(gbuf(bc), dO + hb, tbytes, rsb, c1, si, j * BQ, c - DT::PER);
    } else {
      if (c < DT::PER) dma.part(qbuf(bc), rq, RS, j * BQ, c);
      else dma.part(gbuf(bc), rg, RS, j * BQ, c - DT::PER);
    }
  };
  auto load_ld = [&](int j) __attribute__((always_inline)) {
    if (tid < BQ) {
      const int qq = j * BQ + tid;
      // queries past the end: LSE = +inf makes P = 0 (their rows read as zeros)
      const int trow = qq < L ? token_row<SM>(si, qq) : 0;
      lr = qq < L ? lse_h[trow] : INFINITY;
      dr = qq < L ? del_h[trow] : 0.f;
    }
  };
  auto store_ld = [&](auto bc) __attribute__((always_inline)) {
    if (tid < BQ) {
      lbuf(bc)[tid] = lr * 1.4426950408889634f;
      lbuf(bc)[BQ + tid] = dr;
    }
  };

  // per-lane LDS byte offsets of the operand reads (as in the kernel above):
  // row l32 at unit 2ks+hi of a query tile (and of the wave's 32 V rows), and
  // the transposed fragment bases of output block db and half t
  uint32_t qa[KS], fa[DB][2];
  {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qa[ks] = (uint32_t)(toff<D>(l32, (2 * ks + hi) * 8) * sizeof(bf16));
      asm volatile("" : "+v"(qa[ks]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        fa[db][t] = (uint32_t)(toff<D>(bsigma(8 * (g >> 1) + 4 * t + (sl >> 2)),
                                       db * 32 + 16 * (g & 1) + 4 * (sl & 3)) * sizeof(bf16));
        asm volatile("" : "+v"(fa[db][t]));
      }
  }
  const char* vrow = reinterpret_cast<const char*>(v_t) + wave * 32 * D * sizeof(bf16);

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }
  f32x16 sacc, dpacc;
  bf16x8 pf[2], sf[2];

  // M(j): the products of tile j - 1's dV and dK (buffer B + 2 mod 3) and of
  // query tile j's S and dP (tile j in buffer B).  Op x < NP: x even dV, odd
  // dK, of block db = x / 4, half st = (x / 2) & 1; op NP + i: i even S (k-step
  // i / 2), i odd dP (every accumulator adds its products in the order of the
  // kernel above).  Group 0 also copies tile j + 1 into buffer B + 1 mod 3.
  auto mphase = [&](auto gc, int j, auto bc, auto hs, auto hp, const bf16* last)
                    __attribute__((always_inline)) {
    constexpr int G = decltype(gc)::value;
    constexpr int B = decltype(bc)::value;
    constexpr int BP = (B + 2) % 3;
    constexpr int NS = decltype(hs)::value ? 2 * KS : 0;
    constexpr int NP = decltype(hp)::value ? 4 * DB : 0;
    constexpr int N = NS + NP;
    constexpr int NCH = (G == 0 && NS > 0) ? NC : 0;
    typedef std::integral_constant<int, B> BC;
    typedef std::integral_constant<int, BP> BPC;
    typedef std::integral_constant<int, (B + 1) % 3> BN1;
    const char* qs = reinterpret_cast<const char*>(qbuf(BC{}));
    const char* gs = reinterpret_cast<const char*>(gbuf(BC{}));
    // (the last phase, products of tile nq - 1 only, takes that tile's buffer
    // as a run-time choice: no copy is in flight then, and one code path keeps
    // the accumulators in the same registers)
    const char* qp = reinterpret_cast<const char*>(NS > 0 ? qbuf(BPC{}) : last);
    const char* gp = reinterpret_cast<const char*>(NS > 0 ? gbuf(BPC{}) : last + TILE);
    // operand fragment(s) of op o: a (and for dP the V row, b)
    auto fetch = [&](int o, bf16x8& a, bf16x8& b) __attribute__((always_inline)) {
      if (o >= NP) {
        const int i = o - NP;
        const int ks = i >> 1;
        if (i & 1) {
          a = *reinterpret_cast<const bf16x8*>(gs + qa[ks]);
          b = *reinterpret_cast<const bf16x8*>(vrow + qa[ks]);
        } else {
          a = *reinterpret_cast<const bf16x8*>(qs + qa[ks]);
        }
      } else {
        const int x = o;
        const int db = x >> 2, st = (x >> 1) & 1;
        const char* t = (x & 1) ? qp : gp;
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const i16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(t + fa[db][tt] + 16 * st * D * sizeof(bf16)));
          const bf16x4 h = __builtin_bit_cast(bf16x4, w);
#pragma unroll
          for (int e = 0; e < 4; ++e) a[4 * tt + e] = h[e];
        }
      }
    };
    if constexpr (NS > 0) {
      sacc = f32x16{};
      dpacc = f32x16{};
      if constexpr (G == 0) load_ld(j + 1);
    }
    bf16x8 fa_[kBwdPpAhead], fb_[kBwdPpAhead];
#pragma unroll
    for (int o = 0; o < kBwdPpAhead; ++o)
      if (o < N) fetch(o, fa_[o], fb_[o]);
#pragma unroll
    for (int o = 0; o < N; ++o) {
      const bf16x8 a = fa_[o % kBwdPpAhead], b = fb_[o % kBwdPpAhead];
      if (o + kBwdPpAhead < N) fetch(o + kBwdPpAhead, fa_[o % kBwdPpAhead], fb_[o % kBwdPpAhead]);
      if (o >= NP) {
        const int i = o - NP;
        if (i & 1) mma16(dpacc, a, b);
        else mma16(sacc, a, kf[i >> 1]);
      } else {
        const int x = o;
        const int db = x >> 2, st = (x >> 1) & 1;
        if (x & 1) mma16(dk_acc[db], sf[st], a);
        else mma16(dv_acc[db], pf[st], a);
      }
      if (pp_copy_after(o, N, NCH)) copy_part(j + 1, BN1{}, ((o + 1) * NCH) / N - 1);
    }
    bwd_pp_sched<N, NP, NCH>();
  };

  // E(j): P and dS of tile j (LSE, Delta of tile j in buffer B) into the A
  // fragments of dV and dK
  auto ephase = [&](auto bc) __attribute__((always_inline)) {
    const float* lb = lbuf(bc);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = 16 * (r >> 3) + 8 * hi + (r & 7);
      const float p = fast_exp2(fmaf(sacc[r], scale_log2, -lb[q]));
      pf[r >> 3][r & 7] = (bf16)p;
      sf[r >> 3][r & 7] = (bf16)(p * (dpacc[r] - lb[BQ + q]));
    }
    // materialise the phase's results here (their first use is the next M
    // phase; without the pins the optimizer sinks this work below group 0's
    // barrier, which puts both groups back in step)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      i32x4 w = __builtin_bit_cast(i32x4, pf[st]);
      asm volatile("" : "+v"(w));
      pf[st] = __builtin_bit_cast(bf16x8, w);
      i32x4 u = __builtin_bit_cast(i32x4, sf[st]);
      asm volatile("" : "+v"(u));
      sf[st] = __builtin_bit_cast(bf16x8, u);
    }
  };

  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  typedef std::integral_constant<int, 2> B2;
  typedef std::integral_constant<bool, false> F;
  typedef std::integral_constant<bool, true> Tr;
  // one iteration of group G: M(j), then E(j); group 1 takes its barrier
  // between them, group 0 after E(j) (having waited for its copies of tile
  // j + 1 and stored that tile's LSE and Delta)
  auto iter = [&](auto gc, int j, auto bc, auto hs, auto hp, const bf16* last = nullptr)
                  __attribute__((always_inline)) {
    constexpr int G = decltype(gc)::value;
    constexpr int B = decltype(bc)::value;
    __builtin_amdgcn_sched_barrier(0);
    mphase(gc, j, bc, hs, hp, last);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (G == 1) __syncthreads();
    if constexpr (decltype(hs)::value) ephase(bc);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (G == 0) {
      wait_dma();  // tile j + 1 and its LSE, Delta, requested during M(j)
      if constexpr (decltype(hs)::value) store_ld(std::integral_constant<int, (B + 1) % 3>{});
      __syncthreads();
    }
  };
  const int nq = (L + BQ - 1) / BQ;
  // j = 0: S/dP only; then tiles 1 .. nq - 1 (buffers 1, 2, 0, ...); j = nq:
  // the last dV/dK products only
  auto run = [&](auto gc) __attribute__((always_inline)) {
    iter(gc, 0, B0{}, Tr{}, F{});
    int j = 1;
    // whole rounds of three tiles (buffers 1, 2, 0), then up to two more
    // (written out: a loop with exits between its bodies made the compiler
    // shuffle the accumulators between registers and spill)
    for (; j + 2 < nq; j += 3) {
      iter(gc, j, B1{}, Tr{}, Tr{});
      iter(gc, j + 1, B2{}, Tr{}, Tr{});
      iter(gc, j + 2, B0{}, Tr{}, Tr{});
    }
    if (j < nq) {
      iter(gc, j, B1{}, Tr{}, Tr{});
      ++j;
      if (j < nq) {
        iter(gc, j, B2{}, Tr{}, Tr{});
        ++j;
      }
    }
    // j == nq: tile nq - 1 sits in buffer (nq - 1) mod 3
    const int b = (j + 2) % 3;
    iter(gc, j, B0{}, F{}, Tr{}, b == 0 ? qg_b0 : (b == 1 ? qg_b1 : qg_b2));
  };

  if (group == 0) {
    load_ld(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) copy_part(0, B0{}, c);
    wait_dma();
    store_ld(B0{});
  }
  __syncthreads();  // V rows, tile 0 and its LSE, Delta
  if (group == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});

  // ---- epilogue: dK = R^T (s dK'), dV; 64 keys at a time staged through LDS
  // (the V rows are no longer read) for row-major stores ----
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16* acc = pass == 0 ? dk_acc : dv_acc;
    const float mul = pass == 0 ? scale : 1.f;
#pragma unroll
    for (int quarter = 0; quarter < 4; ++quarter) {
      if ((wave >> 1) == quarter) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = (wave & 1) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            stage[key * D + db * 32 + l32] = acc[db][r] * mul;
          }
      }
      __syncthreads();
      bf16* out = pass == 0 ? dK : dV;
      for (int e = tid; e < 64 * UPR; e += THREADS) {
        const int row = e / UPR, unit = e % UPR;
        const int kk = kv0 + quarter * 64 + row;
        if (kk < L) {
          f32x8 x = *reinterpret_cast<const f32x8*>(stage + row * D + unit * 8);
          if (rope && pass == 0)
            x = rope_unit(x, unit, axis_pos(token_pos3(kk, si), unit_axis(unit, m)), m, true);
          store8<bf16>(out + hb + (size_t)token_row<SM>(si, kk) * RS + unit * 8,
                       from_f32x8<bf16>(x));
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

template <int D, bool SM>
static hipError_t launch_dkdv_pp(const Meta& m, const void* q, const void* k, const void* v,
                                 const void* dout, const float* lse, const float* delta, void* dk,
                                 void* dv, float scale, bool rope, hipStream_t stream) {
  attn_bwd_dkdv_pp_kernel<D, SM><<<dim3(m.n_bwd), dim3(512), 0, stream>>>(
      m, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse, delta,
      (bf16*)dk, (bf16*)dv, scale, scale * 1.4426950408889634f, rope ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, const void* dout, const float* lse,
                           const float* delta, void* dk, void* dv, float scale, bool rope,
                           bool sm, hipStream_t stream) {
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int D = p->desc.head_dim;
  if (bf) {  // 256-key work items (the stream-major layout is bf16 only; the caller checks)
    if (m.n_bwd == 0) return hipSuccess;
    if (sm)
      return D == 128 ? launch_dkdv_pp<128, true>(m, q, k, v, dout, lse, delta, dk, dv, scale, rope, stream)
                      : launch_dkdv_pp<64, true>(m, q, k, v, dout, lse, delta, dk, dv, scale, rope, stream);
    return D == 128 ? launch_dkdv_pp<128, false>(m, q, k, v, dout, lse, delta, dk, dv, scale, rope, stream)
                    : launch_dkdv_pp<64, false>(m, q, k, v, dout, lse, delta, dk, dv, scale, rope, stream);
  }
#define PVJ_BWD(TT, DD) \
  return launch_dkdv_t<TT, DD>(m, q, k, v, dout, lse, delta, dk, dv, scale, rope, stream)
  if (D == 128) PVJ_BWD(float, 128);
  PVJ_BWD(float, 64);
#undef PVJ_BWD
}

}  // namespace pvj
