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

// Partial state of one key range of a split tile (bf16, 256 queries): O^T
// unnormalised at slot[d * 256 + q], the reference max m (base 2) at
// slot[D * 256 + q] and the sum l at slot[(D + 1) * 256 + q], for every query
// q of the tile (rows past the sample end too; the merge skips them).  Lane
// (l32, hi) of wave w holds query 32 w + l32 and the d of its accumulators.
template <int DB>
__device__ __forceinline__ void store_partial(float* slot, int ql, int hi, const f32x16 (&oacc)[DB],
                                              float m_run, float l_tot) {
  constexpr int D = DB * 32;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) slot[(db * 32 + 8 * g + 4 * hi + e) * 256 + ql] = oacc[db][4 * g + e];
  if (hi == 0) {
    slot[D * 256 + ql] = m_run;
    slot[(D + 1) * 256 + ql] = l_tot;
  }
}

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

  // key tiles [kt0, kt1) of this item: all of them, or one part of a split tile
  const int nkv = (L + kFwdBN - 1) / kFwdBN;
  const int kt0 = it.split ? fwd_split_begin(nkv, split_part(it.split), split_parts(it.split)) : 0;
  const int kt1 =
      it.split ? fwd_split_begin(nkv, split_part(it.split) + 1, split_parts(it.split)) : nkv;
  load_tile(kt0 * kFwdBN, std::integral_constant<int, 0>{});
  store_tile(kt0 * kFwdBN, std::integral_constant<int, 0>{});
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
    if (j + 1 < kt1) load_tile(kv0 + kFwdBN, std::integral_constant<int, B ^ 1>{});
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
    if (j + 1 < kt1) store_tile(kv0 + kFwdBN, std::integral_constant<int, B ^ 1>{});
    __syncthreads();
  };
  // full tiles in pairs (buffers 0, 1), then a leftover full tile, then the
  // partial tile with the key mask
  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  typedef std::integral_constant<bool, false> NoMask;
  typedef std::integral_constant<bool, true> Mask;
  const int jf = min(kt1, L / kFwdBN);  // tiles [kt0, jf) need no mask
  int j = kt0;
  for (; j + 1 < jf; j += 2) {
    step(j, B0{}, NoMask{});
    step(j + 1, B1{}, NoMask{});
  }
  if (j < jf) {
    step(j, B0{}, NoMask{});
    ++j;
  }
  if (j < kt1) {
    if ((j - kt0) & 1) step(j, B1{}, Mask{});
    else step(j, B0{}, Mask{});
  }

  // ---- epilogue: O = O^T / l, LSE (a split part: its partial state) ----
  const float l_tot = sum_pair32(l_run);
  if constexpr (sizeof(T) == 2) {
    if (it.split) {
      store_partial<DB>(m.fwd_part + (size_t)(split_slot(it.split) + split_part(it.split)) *
                                         fwd_part_floats(D),
                        wave * 32 + l32, hi, oacc, m_run, l_tot);
      return;
    }
  }
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

// ---------------------------------------------------------------------------
// bf16 forward without RoPE on load: two wave groups offset by half a tile.
//
// The kernel above keeps all eight waves in step (one barrier per tile at the
// same point of every wave), so the two waves of a SIMD run their score
// products together, then their softmax together (the matrix cores idle
// meanwhile), then their output products.  Here waves 0-3 (group 0) and 4-7
// (group 1) have one wave on every SIMD each and take the one barrier per
// tile at different points of the same instruction stream:
//   M(k): S_k = K_k Q^T (k < n), then O^T += V_{k-1}^T P_{k-1}^T (k >= 1)
//   V(k): online softmax of S_k into P_k (k < n)
//   group 0: M(k) V(k) | barrier      group 1: M(k) | barrier V(k)
// so after every barrier one wave of a SIMD issues its 32 products while the
// other runs its softmax.  Pipeline set k (read in M(k) by both groups) holds
// K_k and V_{k-1}; set k + 1 goes into the buffers of set k - 1, whose last
// reader (M(k-1) of group 1) is done at barrier k - 1.  Group 0 copies all of
// set k + 1 during its M(k), one copy instruction every few products: issued
// in a burst by all eight waves after a barrier, the copies stalled the
// issuing waves for hundreds of cycles (measured), and a group-1 wave issuing
// them would delay its softmax, which is on the critical path.  Inside M(k)
// the operand reads from LDS run four products ahead of the products.  Per row the
// arithmetic is that of the kernel above, in the same order (O is scaled by
// each tile's alpha before that tile's products are added), so both give the
// same bits.
// ---------------------------------------------------------------------------
constexpr int kPpAhead = 4;  // operand fragments in flight ahead of the products

template <int D, bool SM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_fwd_pp_kernel(Meta m, const bf16* __restrict__ Q, const bf16* __restrict__ K,
                   const bf16* __restrict__ V, bf16* __restrict__ O, float* __restrict__ LSE,
                   float scale_log2) {
  constexpr int BM = 256, THREADS = 512;
  constexpr int KS = D / 16;  // k-steps of 16 over the head dim (score product)
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int TILE = kFwdBN * D;
  static_assert(FwdTile<bf16, D>::BM == BM, "work items are 256-query tiles");

  __shared__ __align__(16) bf16 k_b0[TILE], k_b1[TILE], v_b0[TILE], v_b1[TILE];

  const Item it = m.fwd_items[blockIdx.x];
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

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int group = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int qi = it.tile * BM + wave * 32 + l32;  // this lane's query (local index)

  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 v = {};
    if (qi < L) v = load8<bf16>(Q + hb + (size_t)token_row<SM>(si, qi) * RS + (2 * ks + hi) * 8);
    qf[ks] = v;
  }

  // the copies are issued by group 0 (256 threads) only
  typedef DmaTile<D, kFwdBN, THREADS / 2> DT;
  constexpr int NC = 2 * DT::PER;  // copy instructions per set and wave
  const DT dma(RS);
  const uint32_t c1 = SM ? dma.sm_c1(si, rsb) : 0u;  // stream-major image-row offset
  (void)c1;
  // key tiles kt0 .. kt1 - 1 of the sample: all of them, or one part of a split
  // tile.  Keys are counted from the first one of the part (k below counts
  // tiles from kt0): Lk keys of the sample lie at or after it.
  const int nkv = (L + kFwdBN - 1) / kFwdBN;
  const int kt0 = it.split ? fwd_split_begin(nkv, split_part(it.split), split_parts(it.split)) : 0;
  const int kt1 =
      it.split ? fwd_split_begin(nkv, split_part(it.split) + 1, split_parts(it.split)) : nkv;
  const int n = kt1 - kt0;
  const int Lk = L - kt0 * kFwdBN;
  const size_t kbase = base + (size_t)kt0 * kFwdBN * RS;
  const typename DT::Src rk = DT::src(K + kbase, RS, Lk), rv = DT::src(V + kbase, RS, Lk);
  // copy instruction c of set k into buffer pair B: c < PER copies part c of
  // K_k, the rest part c - PER of V_{k-1}.  A tile at or past the sample end
  // gets an empty buffer resource (it reads zeros, into a buffer no later
  // product reads).
  auto copy_part = [&](int k, auto bc, int c) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    if constexpr (SM) {
      if (c < DT::PER) dma.part_sm(B ? k_b1 : k_b0, K + hb, tbytes, rsb, c1, si, (kt0 + k) * kFwdBN, c);
      else dma.part_sm(B ? v_b1 : v_b0, V + hb, tbytes, rsb, c1, si, (kt0 + k - 1) * kFwdBN, c - DT::PER);
    } else {
      if (c < DT::PER) dma.part(B ? k_b1 : k_b0, rk, RS, k * kFwdBN, c);
      else dma.part(B ? v_b1 : v_b0, rv, RS, (k - 1) * kFwdBN, c - DT::PER);
    }
  };

  // per-lane LDS byte offsets of the operand reads (see the kernel above)
  uint32_t ka[KS], va[DB][2];
  {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      ka[kk] = (uint32_t)(toff<D>(l32, (2 * kk + hi) * 8) * sizeof(bf16));
      asm volatile("" : "+v"(ka[kk]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        va[db][t] = (uint32_t)(toff<D>(bsigma(8 * (g >> 1) + 4 * t + (sl >> 2)),
                                       db * 32 + 16 * (g & 1) + 4 * (sl & 3)) * sizeof(bf16));
        asm volatile("" : "+v"(va[db][t]));
      }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 sacc[2];
  bf16x8 pf[2][2];

  // M(k): the products of pipeline set k.  Op i < NS is the score product
  // (kb = i & 1, kk = i >> 1: the two 32-key chains interleaved); op NS + j
  // the output product (db = j % DB, st = (j / DB) & 1, kb = j / (2 DB):
  // every O block still adds its four terms in the order kb0 st0, kb0 st1,
  // kb1 st0, kb1 st1).  Operand fragments are read kPpAhead ops ahead.
  auto mphase = [&](auto gc, int k, auto bc, auto hs, auto hp) __attribute__((always_inline)) {
    constexpr int G = decltype(gc)::value;
    constexpr int B = decltype(bc)::value;
    constexpr int NS = decltype(hs)::value ? 2 * KS : 0;
    constexpr int NP = decltype(hp)::value ? 4 * DB : 0;
    constexpr int N = NS + NP;
    // group 0 copies set k + 1 (into the other buffer pair) during M(k), k < n
    constexpr int NCH = (G == 0 && NS > 0) ? NC : 0;
    const char* ks = reinterpret_cast<const char*>(B ? k_b1 : k_b0);
    const char* vs = reinterpret_cast<const char*>(B ? v_b1 : v_b0);
    auto fetch = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      if (i < NS) {
        return *reinterpret_cast<const bf16x8*>(ks + ka[i >> 1] + (i & 1) * 32 * D * sizeof(bf16));
      } else {
        const int j = i - NS;
        const int db = j % DB, st = (j / DB) & 1, kb = j / (2 * DB);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const uint32_t o = (uint32_t)((kb * 32 + 16 * st) * D * sizeof(bf16));
        bf16x8 f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const i16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + va[db][t] + o));
          const bf16x4 h = __builtin_bit_cast(bf16x4, w);
#pragma unroll
          for (int e = 0; e < 4; ++e) f[4 * t + e] = h[e];
        }
        return f;
      }
    };
    if constexpr (NS > 0) {
      sacc[0] = f32x16{};
      sacc[1] = f32x16{};
    }
    bf16x8 fr[kPpAhead];
#pragma unroll
    for (int i = 0; i < kPpAhead; ++i)
      if (i < N) fr[i] = fetch(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bf16x8 a = fr[i % kPpAhead];
      if (i + kPpAhead < N) fr[i % kPpAhead] = fetch(i + kPpAhead);
      if (i < NS) {
        mma16(sacc[i & 1], a, qf[i >> 1]);
      } else {
        const int j = i - NS;
        mma16(oacc[j % DB], a, pf[j / (2 * DB)][(j / DB) & 1]);
      }
      if (pp_copy_after(i, N, NCH))
        copy_part(k + 1, std::integral_constant<int, B ^ 1>{}, ((i + 1) * NCH) / N - 1);
    }
    // keep the reads kPpAhead ops ahead of the products, the copies spread
    pp_sched<N, NS, N, kPpAhead, NCH>();
  };

  // V(k): online softmax of S_k (base 2, lazy rescale; see the kernel above)
  auto vphase = [&](int k, auto mc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mc)::value;
    const int kv0 = k * kFwdBN;
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + 16 * (r >> 3) + 8 * hi + (r & 7);
          if (key >= Lk) sacc[kb][r] = -INFINITY;
        }
    }
    float mx4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& sv = sacc[c >> 1];
      const int o = 8 * (c & 1);
      float t = fmaxf(fmaxf(sv[o], sv[o + 1]), sv[o + 2]);
      t = fmaxf(fmaxf(t, sv[o + 3]), sv[o + 4]);
      t = fmaxf(fmaxf(t, sv[o + 5]), sv[o + 6]);
      mx4[c] = fmaxf(t, sv[o + 7]);
    }
    float mx = fmaxf(fmaxf(fmaxf(mx4[0], mx4[1]), mx4[2]), mx4[3]);
    mx = max_pair32(mx) * scale_log2;
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
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[kb][r], scale_log2, -m_run));
        ls4[r & 3] += p;
        pf[kb][r >> 3][r & 7] = (bf16)p;
      }
    l_run += (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
    // Materialise the phase's results here: their first use is the next M
    // phase, and without these empty asm statements the optimizer sinks the
    // whole softmax below group 0's barrier, which puts both groups back in
    // step.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        i32x4 w = __builtin_bit_cast(i32x4, pf[kb][st]);
        asm volatile("" : "+v"(w));
        pf[kb][st] = __builtin_bit_cast(bf16x8, w);
      }
    asm volatile("" : "+v"(m_run), "+v"(l_run));
  };

  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;
  typedef std::integral_constant<bool, false> F;
  typedef std::integral_constant<bool, true> Tr;
  // One iteration of group G: M(k), then V(k); group 1 takes its barrier
  // between them, group 0 after V(k) (having waited for its copies of set
  // k + 1).  Each group runs its own copy of the loop.
  auto iter = [&](auto gc, int k, auto bc, auto hs, auto hp, auto hv, auto mc)
                  __attribute__((always_inline)) {
    constexpr int G = decltype(gc)::value;
    // the phases stay whole: nothing is scheduled across their boundaries
    __builtin_amdgcn_sched_barrier(0);
    mphase(gc, k, bc, hs, hp);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (G == 1) __syncthreads();
    if constexpr (decltype(hv)::value) vphase(k, mc);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (G == 0) {
      wait_dma();  // set k + 1, copied during M(k)
      __syncthreads();
    }
  };
  // k = 0: scores only; full tiles 1 .. n-2 in pairs (buffers 1, 0); the last
  // key tile n-1 (masked when partial); k = n: the last output product only
  const bool tail_mask = kt1 == nkv && (L % kFwdBN) != 0;
  auto run = [&](auto gc) __attribute__((always_inline)) {
    if (n == 1) {
      if (tail_mask) iter(gc, 0, B0{}, Tr{}, F{}, Tr{}, Tr{});
      else iter(gc, 0, B0{}, Tr{}, F{}, Tr{}, F{});
    } else {
      iter(gc, 0, B0{}, Tr{}, F{}, Tr{}, F{});
      int k = 1;
      for (; k + 1 < n - 1; k += 2) {
        iter(gc, k, B1{}, Tr{}, Tr{}, Tr{}, F{});
        iter(gc, k + 1, B0{}, Tr{}, Tr{}, Tr{}, F{});
      }
      if (k < n - 1) {  // one more full tile (odd k)
        iter(gc, k, B1{}, Tr{}, Tr{}, Tr{}, F{});
        ++k;
      }
      // k == n - 1
      if (k & 1) {
        if (tail_mask) iter(gc, k, B1{}, Tr{}, Tr{}, Tr{}, Tr{});
        else iter(gc, k, B1{}, Tr{}, Tr{}, Tr{}, F{});
      } else {
        if (tail_mask) iter(gc, k, B0{}, Tr{}, Tr{}, Tr{}, Tr{});
        else iter(gc, k, B0{}, Tr{}, Tr{}, Tr{}, F{});
      }
    }
    if (n & 1) iter(gc, n, B1{}, F{}, Tr{}, F{}, F{});
    else iter(gc, n, B0{}, F{}, Tr{}, F{}, F{});
  };

  if (group == 0) {
#pragma unroll
    for (int c = 0; c < DT::PER; ++c) copy_part(0, B0{}, c);
    wait_dma();
  }
  __syncthreads();
  if (group == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});

  // ---- epilogue: O = O^T / l, LSE (a split part: its partial state) ----
  const float l_tot = sum_pair32(l_run);
  if (it.split) {
    store_partial<DB>(m.fwd_part + (size_t)(split_slot(it.split) + split_part(it.split)) *
                                       fwd_part_floats(D),
                      wave * 32 + l32, hi, oacc, m_run, l_tot);
    return;
  }
  if (qi < L) {
    const float inv = 1.f / l_tot;
    const int trow = token_row<SM>(si, qi);
    bf16* orow = O + hb + (size_t)trow * RS;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hi;
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(oacc[db][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + d) = w;
      }
    if (hi == 0 && LSE)
      LSE[(size_t)it.head * m.n_tokens + trow] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}


// Merge of the split tiles' partial states, in part order (so deterministic):
// with M = max_j m_j and w_j = 2^(m_j - M), O = sum_j w_j O_j / sum_j w_j l_j
// and LSE = (M + log2 sum_j w_j l_j) ln 2 (the online-softmax combination of
// disjoint key ranges).  Grid: (split tile, 32 columns of the head dim); one
// thread per query of the tile.
template <int D, bool SM>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(Meta m, bf16* __restrict__ O,
                                                             float* __restrict__ LSE) {
  constexpr size_t PS = (size_t)(D + 2) * 256;  // floats per slot
  const Item st = m.split_tiles[blockIdx.x];
  const int S = split_parts(st.split);
  const float* part = m.fwd_part + (size_t)split_slot(st.split) * PS;
  const SampleInfo si = m.sinfo[st.sample];
  const int ql = threadIdx.x;
  const int qi = st.tile * 256 + ql;
  if (qi >= si.len) return;
  const int d0 = blockIdx.y * 32;
  float M = -INFINITY;  // (parts past S re-read the last one: loads issued together)
#pragma unroll
  for (int j = 0; j < kMaxFwdSplit; ++j) M = fmaxf(M, part[min(j, S - 1) * PS + D * 256 + ql]);
  // one part at a time, its 32 loads issued together
  float lt = 0.f, acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  for (int j = 0; j < S; ++j) {
    const float* pj = part + j * PS;
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = pj[(size_t)(d0 + i) * 256 + ql];
    const float wj = fast_exp2(pj[D * 256 + ql] - M);
    lt += wj * pj[(D + 1) * 256 + ql];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] += wj * x[i];
  }
  const float inv = 1.f / lt;
  const int trow = token_row<SM>(si, qi);
  bf16* orow = O + (size_t)trow * m.n_heads * D + (size_t)st.head * D + d0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    bf16x8 o8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = (bf16)(acc[8 * c + e] * inv);
    *reinterpret_cast<bf16x8*>(orow + 8 * c) = o8;
  }
  if (blockIdx.y == 0 && LSE)
    LSE[(size_t)st.head * m.n_tokens + trow] = (M + __log2f(lt)) * 0.69314718055994531f;
}

template <typename T, int D, bool ROPE>
static hipError_t launch_fwd_t(const Meta& m, const void* q, const void* k, const void* v, void* o,
                               float* lse, float scale_log2, hipStream_t stream) {
  attn_fwd_kernel<T, D, ROPE><<<dim3(m.n_fwd), dim3(FwdTile<T, D>::THREADS), 0, stream>>>(
      m, (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, scale_log2);
  return hipGetLastError();
}

template <int D, bool SM>
static hipError_t launch_fwd_pp(const Meta& m, const void* q, const void* k, const void* v,
                                void* o, float* lse, float sl2, hipStream_t stream) {
  attn_fwd_pp_kernel<D, SM><<<dim3(m.n_fwd), dim3(512), 0, stream>>>(
      m, (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, sl2);
  hipError_t e = hipGetLastError();
  // split tiles: combine their parts
  if (e != hipSuccess || m.n_split == 0) return e;
  attn_fwd_merge_kernel<D, SM><<<dim3(m.n_split, D / 32), dim3(256), 0, stream>>>(m, (bf16*)o, lse);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const pvj_plan* p, const Meta& m, const void* q, const void* k,
                           const void* v, void* o, float* lse, float scale, bool rope, bool sm,
                           hipStream_t stream) {
  if (m.n_fwd == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  const bool bf = p->desc.dtype == PVJ_BF16;
  const int D = p->desc.head_dim;
#define PVJ_FWD(TT, DD)                                                                    \
  (rope ? launch_fwd_t<TT, DD, true>(m, q, k, v, o, lse, sl2, stream)                      \
        : launch_fwd_t<TT, DD, false>(m, q, k, v, o, lse, sl2, stream))
  // (the stream-major layout is accepted for bf16 without RoPE on load only;
  // the caller checks)
  if (bf && !rope) {
    if (sm) return D == 128 ? launch_fwd_pp<128, true>(m, q, k, v, o, lse, sl2, stream)
                            : launch_fwd_pp<64, true>(m, q, k, v, o, lse, sl2, stream);
    return D == 128 ? launch_fwd_pp<128, false>(m, q, k, v, o, lse, sl2, stream)
                    : launch_fwd_pp<64, false>(m, q, k, v, o, lse, sl2, stream);
  }
  if (!bf) return D == 128 ? PVJ_FWD(float, 128) : PVJ_FWD(float, 64);
  hipError_t e = D == 128 ? PVJ_FWD(bf16, 128) : PVJ_FWD(bf16, 64);
  // split tiles (bf16 plans only): combine their parts
  if (e != hipSuccess || m.n_split == 0) return e;
  if (D == 128)
    attn_fwd_merge_kernel<128, false><<<dim3(m.n_split, 4), dim3(256), 0, stream>>>(m, (bf16*)o, lse);
  else
    attn_fwd_merge_kernel<64, false><<<dim3(m.n_split, 2), dim3(256), 0, stream>>>(m, (bf16*)o, lse);
  return hipGetLastError();
#undef PVJ_FWD
}

}  // namespace pvj
