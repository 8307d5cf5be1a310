// Memory-bound chains around the joint attention, fused so each tensor is
// read and written once (Mage-Flow review page, section "Kernel fusion":
// normalization, adaptive modulation, gating and residual addition around the
// backbone's main operators; section "Native-Resolution MMDiT": text and image
// streams keep modality-specific parameters).
//
//  * adaln_fwd: y = LN(x) (1 + scale_i) + shift_i per row of one stream
//    (LayerNorm without affine, population variance); one wave per row, the
//    row held in registers (two-pass mean / variance in fp32).
//  * gate_fwd: out = x + gate_i * y, one wave per row.
//  * adaln_bwd (rows up to 3072 columns): one pass per row set.  Each wave
//    owns up to R rows of one sample, every S-th row of it (R sized so the
//    stream's waves fill the chip) and, per row, computes
//    dx = r (g - mean(g) - xhat mean(g xhat)) with g = dy (1 + scale_i),
//    while it keeps the per-sample parameter gradients' column sums
//    (dshift = sum dy, dscale = sum dy xhat) for its rows in registers; it
//    writes them as one partial per wave, so x and dy are read once.  Sample
//    i owns partial slots cu_i / R + i .. + ceil(L_i / R) - 1 (disjoint,
//    increasing), and seg_final_slots adds a sample's partials in a fixed
//    order.
//  * wider rows, and the gate backward: adaln_bwd_rows writes dx and the
//    row's mean and 1/std; the column sums (dshift, dscale; dgate = sum dout
//    y, with dy = gate_i * dout written by the same pass) come from
//    seg_partial, where every sample's rows are cut into `splits` fixed
//    ranges (about 16 rows each for the stream's longest sample, at most 256
//    ranges), one wave per (sample, range, 512-column chunk) writes a partial
//    sum with four rows in flight, and seg_final adds the partials in a fixed
//    order.
// A row's sample i is found by binary search in the call's segment offsets:
// the stream's cumulative offsets (cu_text or cu_img of the plan), or, for
// both streams in one call, 2B segments (sample i's text rows, then at B + i
// its image rows), which also index the per-sample vectors [2, B, C].

#include "pvj_device.h"
#include "pvj_launch.h"

namespace pvj {

constexpr int kChainThreads = 256;     // 4 waves, one row each
constexpr int kColChunk = 512;         // columns per reduction wave (8 per lane)
constexpr int kRowsPerSplit = 16;      // target rows per reduction wave
constexpr int kMaxSplit = 256;

// sum over the wave, in every lane, without LDS round trips: DPP within
// quads, 8- and 16-lane rows, then the 16- and 32-lane swaps of gfx950
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm 1,0,3,2
  v += dpp<0x4E>(v);   // quad_perm 2,3,0,1
  v += dpp<0x141>(v);  // row_half_mirror: the other quad of each 8 lanes
  v += dpp<0x140>(v);  // row_mirror: the other 8 lanes of each 16
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  return sum_pair32(v);
}

template <typename T>
__device__ __forceinline__ f32x8 ld8f(const T* p) { return to_f32x8(load8<T>(p)); }

// row outputs are written once and not read again here: non-temporal stores
template <typename T>
__device__ __forceinline__ void st8nt(T* p, f32x8 v) {
  __builtin_nontemporal_store(from_f32x8<T>(v), reinterpret_cast<typename Vec8<T>::type*>(p));
}

// ---------------------------------------------------------------------------
// forward: adaptive layer norm
// ---------------------------------------------------------------------------
template <typename T, int NU>
__global__ __launch_bounds__(kChainThreads) void adaln_fwd_kernel(
    const int32_t* __restrict__ cu, int n_samples, int rows, int C, const T* __restrict__ x,
    const T* __restrict__ shift, const T* __restrict__ scale, T* y, float eps) {
  const int row = blockIdx.x * (kChainThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int upr = C / 8;
  // the row's loads go out before the sample lookup (a chain of dependent loads)
  const T* xr = x + (size_t)row * C;
  typename Vec8<T>::type xv[NU];
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    typename Vec8<T>::type z = {};
    xv[k] = u < upr ? load8<T>(xr + u * 8) : z;
  }
  const int s = find_sample(cu, n_samples, row);
  f32x8 v[NU];
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    v[k] = to_f32x8(xv[k]);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += v[k][e];
  }
  const float mean = wave_sum(sum) / C;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    if (u < upr) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[k][e] - mean;
        ss += d * d;
      }
    }
  }
  const float rstd = 1.0f / __builtin_sqrtf(wave_sum(ss) / C + eps);
  const T* sh = shift + (size_t)s * C;
  const T* sc = scale + (size_t)s * C;
  T* yr = y + (size_t)row * C;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    if (u < upr) {
      const f32x8 a = ld8f(sc + u * 8), b = ld8f(sh + u * 8);
      f32x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[k][e] - mean) * rstd * (1.f + a[e]) + b[e];
      st8nt<T>(yr + u * 8, o);
    }
  }
}

// ---------------------------------------------------------------------------
// forward: gate + residual
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kChainThreads) void gate_fwd_kernel(
    const int32_t* __restrict__ cu, int n_samples, int rows, int C, const T* x, const T* y,
    const T* __restrict__ gate, T* out) {
  const int row = blockIdx.x * (kChainThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int upr = C / 8;
  const size_t ro = (size_t)row * C;
  // first unit of x and y before the sample lookup (a chain of dependent loads)
  typename Vec8<T>::type x0 = {}, y0 = {};
  if (lane < upr) {
    x0 = load8<T>(x + ro + lane * 8);
    y0 = load8<T>(y + ro + lane * 8);
  }
  const int s = find_sample(cu, n_samples, row);
  const T* g = gate + (size_t)s * C;
  // six units per lane at a time (a 3,072-wide row in one batch; four per
  // batch measured 1.4% slower): all their loads go out before the stores
  // (out may be x or y: every element is read before this lane writes it)
  for (int u0 = lane; u0 < upr; u0 += 384) {
    typename Vec8<T>::type a[6], b[6], w[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int u = u0 + 64 * k;
      typename Vec8<T>::type z = {};
      a[k] = u < upr ? (u == lane ? x0 : load8<T>(x + ro + u * 8)) : z;
      b[k] = u < upr ? (u == lane ? y0 : load8<T>(y + ro + u * 8)) : z;
      w[k] = u < upr ? load8<T>(g + u * 8) : z;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int u = u0 + 64 * k;
      if (u < upr) {
        const f32x8 fa = to_f32x8(a[k]), fb = to_f32x8(b[k]), fw = to_f32x8(w[k]);
        f32x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fa[e] + fw[e] * fb[e];
        st8nt<T>(out + ro + u * 8, o);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// backward: adaptive layer norm, per row (dx and the row statistics)
// ---------------------------------------------------------------------------
template <typename T, int NU>
__global__ __launch_bounds__(kChainThreads) void adaln_bwd_rows_kernel(
    const int32_t* __restrict__ cu, int n_samples, int rows, int C, const T* __restrict__ x,
    const T* __restrict__ scale, const T* __restrict__ dy, T* dx, float2* __restrict__ stats,
    float eps) {
  const int row = blockIdx.x * (kChainThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int upr = C / 8;
  const int s = find_sample(cu, n_samples, row);
  const size_t ro = (size_t)row * C;
  f32x8 v[NU], g[NU];
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    v[k] = u < upr ? ld8f(x + ro + u * 8) : f32x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += v[k][e];
  }
  const float mean = wave_sum(sum) / C;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    if (u < upr) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[k][e] - mean;
        ss += d * d;
      }
    }
  }
  const float rstd = 1.0f / __builtin_sqrtf(wave_sum(ss) / C + eps);
  // g = dy (1 + scale_s); means of g and g * xhat
  float sg = 0.f, sgx = 0.f;
  const T* sc = scale + (size_t)s * C;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    if (u < upr) {
      const f32x8 d = ld8f(dy + ro + u * 8), a = ld8f(sc + u * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[k][e] = (v[k][e] - mean) * rstd;  // xhat from here on
        g[k][e] = d[e] * (1.f + a[e]);
        sg += g[k][e];
        sgx += g[k][e] * v[k][e];
      }
    } else {
      g[k] = f32x8{};
    }
  }
  const float mg = wave_sum(sg) / C, mgx = wave_sum(sgx) / C;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    if (u < upr) {
      f32x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rstd * (g[k][e] - mg - v[k][e] * mgx);
      st8nt<T>(dx + ro + u * 8, o);
    }
  }
  if (lane == 0) stats[row] = make_float2(mean, rstd);
}

// ---------------------------------------------------------------------------
// backward: adaptive layer norm, one pass (dx and the partial column sums)
// ---------------------------------------------------------------------------
// first partial slot of sample i (rows per wave R)
__device__ __forceinline__ int slot_base(const int32_t* cu, int i, int R) { return cu[i] / R + i; }

// Sample i owns slots slot_base(i) .. slot_base(i + 1) - 1; the first
// S = ceil(L_i / R) of them (the ones the final pass reads) take rows
// cu_i + j, cu_i + j + S, ... (at most R each), so a sample's slots sweep its
// rows together (DRAM pages are shared by the concurrent rows: measured 5%
// faster than R consecutive rows per slot); later slots are empty.  The
// sample i of `slot`, its first row r0, stride st and end r1 (empty when
// r0 >= r1; such slots are never read).
__device__ __forceinline__ void slot_rows_strided(const int32_t* cu, int n_samples, int R,
                                                  int slot, int& i, int& r0, int& st, int& r1) {
  int lo = 0, hi = n_samples - 1;  // the last i with slot_base(i) <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_base(cu, mid, R) <= slot) lo = mid;
    else hi = mid - 1;
  }
  i = lo;
  const int j = slot - slot_base(cu, i, R);
  st = (cu[i + 1] - cu[i] + R - 1) / R;
  r1 = cu[i + 1];
  r0 = j < st ? cu[i] + j : r1;
}

template <typename T, int NU>
__global__ __launch_bounds__(kChainThreads) void adaln_bwd_kernel(
    const int32_t* __restrict__ cu, int n_samples, int C, int R, int n_slots,
    const T* __restrict__ x, const T* __restrict__ scale, const T* __restrict__ dy,
    T* __restrict__ dx, float* __restrict__ partial, float eps) {
  typedef typename Vec8<T>::type V8;
  const int slot = blockIdx.x * (kChainThreads / 64) + (threadIdx.x >> 6);
  if (slot >= n_slots) return;
  int i, r0, st, r1;
  slot_rows_strided(cu, n_samples, R, slot, i, r0, st, r1);
  if (r0 >= r1) return;
  const int lane = threadIdx.x & 63;
  const int upr = C / 8;
  const float inv_c = 1.f / C;
  V8 sc[NU];  // scale_i of this lane's columns
  f32x8 acc0[NU], acc1[NU];
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    V8 z = {};
    sc[k] = u < upr ? load8<T>(scale + (size_t)i * C + u * 8) : z;
    acc0[k] = f32x8{};
    acc1[k] = f32x8{};
  }
  // the next row's x and dy are loaded while this row is computed
  V8 xn[NU], dn[NU];
  auto fetch = [&](int r) {
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = lane + 64 * k;
      V8 z = {};
      xn[k] = u < upr ? load8<T>(x + (size_t)r * C + u * 8) : z;
      dn[k] = u < upr ? load8<T>(dy + (size_t)r * C + u * 8) : z;
    }
  };
  fetch(r0);
  for (int r = r0; r < r1; r += st) {
    const size_t ro = (size_t)r * C;
    f32x8 v[NU];
    V8 d[NU];
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      v[k] = to_f32x8(xn[k]);
      d[k] = dn[k];
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += v[k][e];
    }
    if (r + st < r1) fetch(r + st);
    const float mean = wave_sum(sum) * inv_c;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = lane + 64 * k;
      if (u < upr) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = v[k][e] - mean;
          ss += t * t;
        }
      }
    }
    const float rstd = 1.0f / __builtin_sqrtf(wave_sum(ss) * inv_c + eps);
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = lane + 64 * k;
      if (u < upr) {
        const f32x8 dd = to_f32x8(d[k]), a = to_f32x8(sc[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[k][e] = (v[k][e] - mean) * rstd;  // xhat from here on
          const float g = dd[e] * (1.f + a[e]);
          sg += g;
          sgx += g * v[k][e];
          acc0[k][e] += dd[e];
          acc1[k][e] += dd[e] * v[k][e];
        }
      }
    }
    const float mg = wave_sum(sg) * inv_c, mgx = wave_sum(sgx) * inv_c;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = lane + 64 * k;
      if (u < upr) {
        const f32x8 dd = to_f32x8(d[k]), a = to_f32x8(sc[k]);
        f32x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rstd * (dd[e] * (1.f + a[e]) - mg - v[k][e] * mgx);
        st8nt<T>(dx + ro + u * 8, o);
      }
    }
  }
  float* p0 = partial + (size_t)slot * 2 * C;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = lane + 64 * k;
    if (u < upr) {
      *reinterpret_cast<f32x8*>(p0 + u * 8) = acc0[k];
      *reinterpret_cast<f32x8*>(p0 + C + u * 8) = acc1[k];
    }
  }
}

// The same for rows of 2,561-3,072 columns with two waves per slot, each
// holding half of every row (three units per lane): the row statistics are
// summed across the pair through LDS, wave 0's half first so both waves hold
// the same bits.  Half the registers per wave (one wave alone needs ~350, one
// per SIMD, and waits out its dependent passes) let two waves share a SIMD.
// Two exchanges per row: sum x, sum g and sum g x first (sum g xhat =
// r (sum g x - mean sum g) needs no statistic), then sum (x - mean)^2 (two
// passes for the variance).  1 + scale_i is formed once per slot in fp32.
// Only a lane's third unit in wave 1 can lie past the row (C >= 2,561).
// Bounded to two waves per SIMD (256 registers each).
template <typename T>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void
adaln_bwd_pair_kernel(
    const int32_t* __restrict__ cu, int n_samples, int C, int R, int n_slots,
    const T* __restrict__ x, const T* __restrict__ scale, const T* __restrict__ dy,
    T* __restrict__ dx, float* __restrict__ partial, float eps) {
  typedef typename Vec8<T>::type V8;
  constexpr int NU = 3;
  __shared__ float xch[2][2][2][3];  // [row parity][exchange][wave][value]
  const int slot = blockIdx.x;
  if (slot >= n_slots) return;
  int i, r0, st, r1;
  slot_rows_strided(cu, n_samples, R, slot, i, r0, st, r1);
  if (r0 >= r1) return;  // (the whole workgroup: no barrier is left waiting)
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int upr = C / 8;
  const float inv_c = 1.f / C;
  const int ub = w * 192 + lane;  // unit of k = 0; unit k is ub + 64 k
  const bool ok2 = ub + 128 < upr;
  auto ok = [&](int k) { return k < 2 || ok2; };
  f32x8 sp[NU], acc0[NU], acc1[NU];
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const f32x8 a = ok(k) ? ld8f<T>(scale + (size_t)i * C + (ub + 64 * k) * 8) : f32x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) sp[k][e] = 1.f + a[e];
    acc0[k] = f32x8{};
    acc1[k] = f32x8{};
  }
  // x and dy of the next row are loaded into the registers of this one as
  // soon as it is converted.  The loads are unconditional (the slot's last row
  // loads itself again; a unit past the row reads the lane's first unit and
  // is zeroed when converted) and the slot's first row runs before the loop:
  // with conditional loads the compiler moved the loaded values between
  // registers at the loop's end and waited there for every load and store in
  // flight (a second register set, rows two ahead, spilled).  Measured on
  // the training pack's two streams: 0.210 -> 0.206 ms.
  V8 xa[NU], da[NU];
  const int rlast = r0 + (r1 - r0 - 1) / st * st;  // the slot's last row
  const int u2 = ok2 ? ub + 128 : ub;
  auto fetch = [&](V8 (&xs)[NU], V8 (&ds)[NU], int r) __attribute__((always_inline)) {
    const size_t ro = (size_t)min(r, rlast) * C;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = k < 2 ? ub + 64 * k : u2;
      xs[k] = load8<T>(x + ro + u * 8);
      ds[k] = load8<T>(dy + ro + u * 8);
    }
  };
  auto row = [&](int r, V8 (&xs)[NU], V8 (&ds)[NU], int par) __attribute__((always_inline)) {
    f32x8 v[NU], d[NU];
    float s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      v[k] = to_f32x8(xs[k]);
      d[k] = to_f32x8(ds[k]);
      if (!ok(k)) v[k] = d[k] = f32x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = d[k][e] * sp[k][e];
        s1 += v[k][e];
        s2 += g;
        s3 += g * v[k][e];
      }
    }
    fetch(xs, ds, r + st);
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    s3 = wave_sum(s3);
    if (lane == 0) {
      xch[par][0][w][0] = s1;
      xch[par][0][w][1] = s2;
      xch[par][0][w][2] = s3;
    }
    __syncthreads();
    const float mean = (xch[par][0][0][0] + xch[par][0][1][0]) * inv_c;
    const float sg = xch[par][0][0][1] + xch[par][0][1][1];
    const float sgx = xch[par][0][0][2] + xch[par][0][1][2];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NU; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = v[k][e] - mean;
        v[k][e] = ok(k) ? t : 0.f;  // x - mean from here on
        ss += v[k][e] * v[k][e];
      }
    ss = wave_sum(ss);
    if (lane == 0) xch[par][1][w][0] = ss;
    __syncthreads();
    const float rstd =
        1.0f / __builtin_sqrtf((xch[par][1][0][0] + xch[par][1][1][0]) * inv_c + eps);
    const float mg = sg * inv_c;
    const float mgx = rstd * ((sgx - mean * sg) * inv_c);
    const size_t ro = (size_t)r * C;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      f32x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xh = v[k][e] * rstd;
        acc0[k][e] += d[k][e];
        acc1[k][e] += d[k][e] * xh;
        o[e] = rstd * (d[k][e] * sp[k][e] - mg - xh * mgx);
      }
      if (ok(k)) st8nt<T>(dx + ro + (ub + 64 * k) * 8, o);
    }
  };
  fetch(xa, da, r0);
  row(r0, xa, da, 0);
  int r = r0 + st;
  for (; r + st < r1; r += 2 * st) {
    row(r, xa, da, 1);
    row(r + st, xa, da, 0);
  }
  if (r < r1) row(r, xa, da, 1);
  float* p0 = partial + (size_t)slot * 2 * C;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    if (ok(k)) {
      *reinterpret_cast<f32x8*>(p0 + (ub + 64 * k) * 8) = acc0[k];
      *reinterpret_cast<f32x8*>(p0 + C + (ub + 64 * k) * 8) = acc1[k];
    }
  }
}

// final pass over partial slots: 16 waves per (kind, sample, 128-column
// chunk; two columns per lane); wave w adds the sample's slots w + 16 j in
// eight chains j mod 8 (eight loads in flight), then the chains and wave 0 the
// sixteen wave sums, always in the same order (deterministic).  Narrow chunks
// spread the pass over the whole chip (512-column chunks left a few dozen
// workgroups each reading ~650 KB: up to 16 us).  Slot layout [slot][kind][C].
constexpr int kFinalCols = 128;
__global__ __launch_bounds__(1024) void seg_final_slots_kernel(
    const int32_t* __restrict__ cu, int n_samples, int C, int R, int kinds,
    const float* __restrict__ partial, float* __restrict__ out0, float* __restrict__ out1) {
  __shared__ f32x2 red[15][64];
  const int nchunk = (C + kFinalCols - 1) / kFinalCols;
  const int chunk = blockIdx.x % nchunk;
  const int s = (blockIdx.x / nchunk) % n_samples;
  const int kind = blockIdx.x / (nchunk * n_samples);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = chunk * kFinalCols + lane * 2;
  const bool active = col < C;
  const int nsl = (cu[s + 1] - cu[s] + R - 1) / R;
  f32x2 acc = {};
  if (active) {
    const float* p = partial + ((size_t)slot_base(cu, s, R) * kinds + kind) * C + col;
    const size_t stride = (size_t)kinds * C;
    f32x2 a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = f32x2{};
    int k = wave;
    for (; k + 7 * 16 < nsl; k += 8 * 16) {
      f32x2 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const f32x2*>(p + (size_t)(k + 16 * j) * stride);
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] += v[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k + 16 * j < nsl) a[j] += *reinterpret_cast<const f32x2*>(p + (size_t)(k + 16 * j) * stride);
    acc = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0 && active) {
#pragma unroll
    for (int w = 0; w < 15; ++w) acc += red[w][lane];
    *reinterpret_cast<f32x2*>((kind ? out1 : out0) + (size_t)s * C + col) = acc;
  }
}

// ---------------------------------------------------------------------------
// per-sample column sums of the LayerNorm backward for rows wider than the
// one-pass kernel holds: p0 = sum dy, p1 = sum dy * (x - mean) rstd over a
// range of one sample's rows per wave and 512-column chunk.
// partial layout: [kind][sample][split][C] fp32
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void seg_partial_kernel(
    const int32_t* __restrict__ cu, int n_samples, int C, int splits, const T* __restrict__ x,
    const T* __restrict__ dy, const float2* __restrict__ stats, float* __restrict__ partial) {
  const int nchunk = (C + kColChunk - 1) / kColChunk;
  const int chunk = blockIdx.x % nchunk;
  const int split = (blockIdx.x / nchunk) % splits;
  const int s = blockIdx.x / (nchunk * splits);
  const int r0 = cu[s], len = cu[s + 1] - cu[s];
  const int lo = r0 + (int)((long long)len * split / splits);
  const int hi = r0 + (int)((long long)len * (split + 1) / splits);
  const int col = chunk * kColChunk + threadIdx.x * 8;
  if (col >= C) return;
  f32x8 acc0[2] = {}, acc1[2] = {};
  auto add = [&](int k, const f32x8& va, const f32x8& vb, float2 st) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc0[k][e] += vb[e];
      acc1[k][e] += vb[e] * ((va[e] - st.x) * st.y);
    }
  };
  int r = lo;
  for (; r + 4 <= hi; r += 4) {
    f32x8 va[4], vb[4];
    float2 st[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t o = (size_t)(r + k) * C + col;
      va[k] = ld8f(x + o);
      vb[k] = ld8f(dy + o);
      st[k] = stats[r + k];
    }
    // the four rows' loads stay ahead of their uses (see gate_bwd_slots_kernel)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 4; ++k) add(k & 1, va[k], vb[k], st[k]);
  }
  for (; r < hi; ++r) {
    const size_t o = (size_t)r * C + col;
    add(0, ld8f(x + o), ld8f(dy + o), stats[r]);
  }
  const size_t po = ((size_t)s * splits + split) * C + col;
  *reinterpret_cast<f32x8*>(partial + po) = acc0[0] + acc0[1];
  *reinterpret_cast<f32x8*>(partial + (size_t)n_samples * splits * C + po) = acc1[0] + acc1[1];
}

// gate + residual backward, rows in slots (the slots of the one-pass
// LayerNorm backward): wave (slot, 512-column chunk) writes dy = gate_s * dout
// for its rows (at most R, interleaved with the sample's other slots) and the
// partial sum of dout * y over them
template <typename T>
__global__ __launch_bounds__(64) void gate_bwd_slots_kernel(
    const int32_t* __restrict__ cu, int n_samples, int C, int R, const T* __restrict__ dout,
    const T* __restrict__ y, const T* __restrict__ gate, T* __restrict__ dy,
    float* __restrict__ partial) {
  typedef typename Vec8<T>::type V8;
  const int nchunk = (C + kColChunk - 1) / kColChunk;
  const int chunk = blockIdx.x % nchunk;
  const int slot = blockIdx.x / nchunk;
  int s, r0, st, r1;
  slot_rows_strided(cu, n_samples, R, slot, s, r0, st, r1);
  const int col = chunk * kColChunk + threadIdx.x * 8;
  if (r0 >= r1 || col >= C) return;
  const int n = (r1 - r0 + st - 1) / st;  // the slot's rows r0 + t st, t < n
  f32x8 acc[2] = {};
  const f32x8 w = ld8f(gate + (size_t)s * C + col);
  // four rows per step in two alternating register sets: the next four rows'
  // loads are in flight while this step computes and stores (rows past the
  // slot's end re-read its last row, so no branch hides the loads from the
  // waits; they are neither summed nor stored)
  V8 a0[4], b0[4], a1[4], b1[4];
  auto fetch = [&](V8 (&a)[4], V8 (&b)[4], int t0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t o = (size_t)(r0 + min(t0 + k, n - 1) * st) * C + col;
      a[k] = load8<T>(dout + o);
      b[k] = load8<T>(y + o);
    }
  };
  auto use = [&](const V8 (&a)[4], const V8 (&b)[4], int t0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (t0 + k < n) {
        const f32x8 va = to_f32x8(a[k]), vb = to_f32x8(b[k]);
        f32x8 d;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[k & 1][e] += va[e] * vb[e];
          d[e] = w[e] * va[e];
        }
        st8nt<T>(dy + (size_t)(r0 + (t0 + k) * st) * C + col, d);
      }
    }
  };
  fetch(a0, b0, 0);
  for (int t = 0; t < n; t += 8) {
    fetch(a1, b1, t + 4);
    use(a0, b0, t);
    fetch(a0, b0, t + 8);
    use(a1, b1, t + 4);
  }
  *reinterpret_cast<f32x8*>(partial + (size_t)slot * C + col) = acc[0] + acc[1];
}

// final pass: 4 waves per (kind, sample, column chunk); wave w adds the
// partials w, w+4, ... with two loads in flight, then wave 0 adds the four
// wave sums in order (a fixed order: deterministic)
__global__ __launch_bounds__(256) void seg_final_kernel(int n_samples, int C, int splits, int kinds,
                                                        const float* __restrict__ partial,
                                                        float* __restrict__ out0,
                                                        float* __restrict__ out1) {
  __shared__ f32x8 red[3][64];
  const int nchunk = (C + kColChunk - 1) / kColChunk;
  const int chunk = blockIdx.x % nchunk;
  const int s = (blockIdx.x / nchunk) % n_samples;
  const int kind = blockIdx.x / (nchunk * n_samples);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = chunk * kColChunk + lane * 8;
  const bool active = kind < kinds && col < C;
  f32x8 acc0 = {}, acc1 = {};
  if (active) {
    const float* p =
        partial + (size_t)kind * n_samples * splits * C + (size_t)s * splits * C + col;
    int k = wave;
    for (; k + 4 < splits; k += 8) {
      acc0 += *reinterpret_cast<const f32x8*>(p + (size_t)k * C);
      acc1 += *reinterpret_cast<const f32x8*>(p + (size_t)(k + 4) * C);
    }
    if (k < splits) acc0 += *reinterpret_cast<const f32x8*>(p + (size_t)k * C);
    acc0 += acc1;
  }
  if (wave > 0) red[wave - 1][lane] = acc0;
  __syncthreads();
  if (wave == 0 && active) {
    acc0 += red[0][lane];
    acc0 += red[1][lane];
    acc0 += red[2][lane];
    *reinterpret_cast<f32x8*>((kind ? out1 : out0) + (size_t)s * C + col) = acc0;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int chain_splits(int max_sample_rows) {
  const int s = (max_sample_rows + kRowsPerSplit - 1) / kRowsPerSplit;
  return s < 1 ? 1 : (s > kMaxSplit ? kMaxSplit : s);
}

// units per lane for a row of C columns (C / 8 units over 64 lanes)
static int units_per_lane(int C) { return (C / 8 + 63) / 64; }

// the one-pass adaptive-layer-norm backward holds the column sums of a lane
// in registers: rows up to 3072 columns
static bool one_pass(int C) { return units_per_lane(C) <= 6; }

// rows per wave of the one-pass LayerNorm backward: as few as fill the chip's
// waves in a single round (a second, partial round costs a whole round's time;
// measured: 0.31 -> 0.25 ms on the training pack).  The waves that fit at once
// follow the kernel's register use per row width (one wave per SIMD at
// six units per lane, two at four, three at two, four at one); at least 4
// rows per wave.  Correctness does not depend on it.
static bool pair_rows(int C) { return units_per_lane(C) >= 5; }  // adaln_bwd_pair_kernel
static int rows_per_wave(int rows, int n_samples, int C) {
  const int nu = units_per_lane(C);
  // slots that fit at once: waves per SIMD x 1024 SIMDs / waves per slot (the
  // pair kernel: two per SIMD at ~180 registers, two per slot)
  const int per_simd = nu >= 5 ? 2 : (nu >= 4 ? 2 : (nu >= 2 ? 3 : 4));
  const int slots = 256 * 4 * per_simd / (nu >= 5 ? 2 : 1) - n_samples - 1;
  const int r = (rows + slots - 1) / slots;
  return r < 4 ? 4 : r;
}
static int n_slots(int rows, int n_samples, int R) { return rows / R + n_samples + 1; }
// rows per slot of the gate backward (64-lane workgroups, one per slot and
// 512-column chunk), at least 8 rows each: 2048 waves in all, two per SIMD
// (four fit at its ~110 registers; measured on the training pack at hidden
// 3072: 2048 waves 0.199 ms, 4096 0.201, 8192 (two rounds) 0.208, 1024 0.202)
static int gate_rows_per_slot(int rows, int n_samples, int C) {
  const int nchunk = (C + kColChunk - 1) / kColChunk;
  const int slots = 2048 / nchunk - n_samples - 1;
  const int r = slots > 0 ? (rows + slots - 1) / slots : rows;
  return r < 8 ? 8 : r;
}

size_t chain_workspace_bytes(int n_samples, int C, int rows, int mode, int splits) {
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  if (mode == 0 && one_pass(C))
    return al((size_t)n_slots(rows, n_samples, rows_per_wave(rows, n_samples, C)) * 2 * C *
              sizeof(float));
  if (mode == 1)
    return al((size_t)n_slots(rows, n_samples, gate_rows_per_slot(rows, n_samples, C)) * C *
              sizeof(float));
  const size_t part = (size_t)2 * n_samples * splits * C * sizeof(float);
  const size_t st = mode == 0 ? (size_t)rows * sizeof(float2) : 0;
  return al(part) + al(st);
}

template <typename T, int NU>
static void adaln_fwd_t(dim3 g, hipStream_t st, const int32_t* cu, int B, int rows, int C,
                        const void* x, const void* shift, const void* scale, void* y, float eps) {
  adaln_fwd_kernel<T, NU><<<g, kChainThreads, 0, st>>>(cu, B, rows, C, (const T*)x, (const T*)shift,
                                                       (const T*)scale, (T*)y, eps);
}
template <typename T, int NU>
static void adaln_bwd_1p_t(dim3 g, hipStream_t st, const int32_t* cu, int B, int C, int R, int ns,
                           const void* x, const void* scale, const void* dy, void* dx,
                           float* partial, float eps) {
  adaln_bwd_kernel<T, NU><<<g, kChainThreads, 0, st>>>(cu, B, C, R, ns, (const T*)x,
                                                       (const T*)scale, (const T*)dy, (T*)dx,
                                                       partial, eps);
}
template <typename T, int NU>
static void adaln_bwd_t(dim3 g, hipStream_t st, const int32_t* cu, int B, int rows, int C,
                        const void* x, const void* scale, const void* dy, void* dx, float2* stats,
                        float eps) {
  adaln_bwd_rows_kernel<T, NU><<<g, kChainThreads, 0, st>>>(
      cu, B, rows, C, (const T*)x, (const T*)scale, (const T*)dy, (T*)dx, stats, eps);
}

#define PVJ_NU_DISPATCH6(FN, T, ...)                 \
  do {                                               \
    const int nu = units_per_lane(C);                \
    if (nu <= 1) FN<T, 1>(__VA_ARGS__);              \
    else if (nu <= 2) FN<T, 2>(__VA_ARGS__);         \
    else if (nu <= 4) FN<T, 4>(__VA_ARGS__);         \
    else FN<T, 6>(__VA_ARGS__);                      \
  } while (0)

#define PVJ_NU_DISPATCH(FN, T, ...)                  \
  do {                                               \
    const int nu = units_per_lane(C);                \
    if (nu <= 1) FN<T, 1>(__VA_ARGS__);              \
    else if (nu <= 2) FN<T, 2>(__VA_ARGS__);         \
    else if (nu <= 4) FN<T, 4>(__VA_ARGS__);         \
    else if (nu <= 6) FN<T, 6>(__VA_ARGS__);         \
    else if (nu <= 8) FN<T, 8>(__VA_ARGS__);         \
    else if (nu <= 12) FN<T, 12>(__VA_ARGS__);       \
    else FN<T, 16>(__VA_ARGS__);                     \
  } while (0)

hipError_t launch_adaln_fwd(const pvj_plan* p, int which, int C, const void* x,
                            const void* shift, const void* scale, void* y, float eps,
                            hipStream_t st) {
  const ChainRows r = chain_rows(p, which, false);
  const int rows = r.rows;
  if (rows == 0) return hipSuccess;
  const dim3 g((rows + 3) / 4);
  if (p->desc.dtype == PVJ_BF16)
    PVJ_NU_DISPATCH(adaln_fwd_t, bf16, g, st, r.cu, r.n_seg, rows, C, x, shift, scale, y, eps);
  else
    PVJ_NU_DISPATCH(adaln_fwd_t, float, g, st, r.cu, r.n_seg, rows, C, x, shift, scale, y, eps);
  return hipGetLastError();
}

hipError_t launch_gate_fwd(const pvj_plan* p, int which, int C, const void* x,
                           const void* y, const void* gate, void* out, hipStream_t st) {
  const ChainRows r = chain_rows(p, which, false);
  const int rows = r.rows;
  if (rows == 0) return hipSuccess;
  const dim3 g((rows + 3) / 4);
  if (p->desc.dtype == PVJ_BF16)
    gate_fwd_kernel<bf16><<<g, kChainThreads, 0, st>>>(r.cu, r.n_seg, rows, C, (const bf16*)x,
                                                       (const bf16*)y, (const bf16*)gate, (bf16*)out);
  else
    gate_fwd_kernel<float><<<g, kChainThreads, 0, st>>>(r.cu, r.n_seg, rows, C, (const float*)x,
                                                        (const float*)y, (const float*)gate,
                                                        (float*)out);
  return hipGetLastError();
}

hipError_t launch_adaln_bwd(const pvj_plan* p, int which, int C, const void* x,
                            const void* scale, const void* dy, void* dx, float* dshift,
                            float* dscale, float eps, int splits, void* ws, hipStream_t st) {
  const ChainRows r = chain_rows(p, which, false);
  const int rows = r.rows, B = r.n_seg;
  if (B == 0) return hipSuccess;
  const int32_t* cu = r.cu;
  const bool bf = p->desc.dtype == PVJ_BF16;
  if (one_pass(C)) {
    const int R = rows_per_wave(rows, B, C), ns = n_slots(rows, B, R);
    float* partial = static_cast<float*>(ws);
    if (rows > 0) {
      if (pair_rows(C)) {
        if (bf)
          adaln_bwd_pair_kernel<bf16><<<ns, 128, 0, st>>>(cu, B, C, R, ns, (const bf16*)x,
                                                          (const bf16*)scale, (const bf16*)dy,
                                                          (bf16*)dx, partial, eps);
        else
          adaln_bwd_pair_kernel<float><<<ns, 128, 0, st>>>(cu, B, C, R, ns, (const float*)x,
                                                           (const float*)scale,
                                                           (const float*)dy, (float*)dx,
                                                           partial, eps);
      } else {
        const dim3 g((ns + 3) / 4);
        if (bf)
          PVJ_NU_DISPATCH6(adaln_bwd_1p_t, bf16, g, st, cu, B, C, R, ns, x, scale, dy, dx,
                           partial, eps);
        else
          PVJ_NU_DISPATCH6(adaln_bwd_1p_t, float, g, st, cu, B, C, R, ns, x, scale, dy, dx,
                           partial, eps);
      }
    }
    const int nfin = (C + kFinalCols - 1) / kFinalCols;
    seg_final_slots_kernel<<<2 * B * nfin, 1024, 0, st>>>(cu, B, C, R, 2, partial, dshift,
                                                           dscale);
    return hipGetLastError();
  }
  const size_t part = (size_t)2 * B * splits * C * sizeof(float);
  float* partial = static_cast<float*>(ws);
  float2* stats = reinterpret_cast<float2*>(static_cast<char*>(ws) + (part + 255) / 256 * 256);
  if (rows > 0) {
    const dim3 g((rows + 3) / 4);
    if (bf)
      PVJ_NU_DISPATCH(adaln_bwd_t, bf16, g, st, cu, B, rows, C, x, scale, dy, dx, stats, eps);
    else
      PVJ_NU_DISPATCH(adaln_bwd_t, float, g, st, cu, B, rows, C, x, scale, dy, dx, stats, eps);
  }
  const int nchunk = (C + kColChunk - 1) / kColChunk;
  if (bf)
    seg_partial_kernel<bf16><<<B * splits * nchunk, 64, 0, st>>>(
        cu, B, C, splits, (const bf16*)x, (const bf16*)dy, stats, partial);
  else
    seg_partial_kernel<float><<<B * splits * nchunk, 64, 0, st>>>(
        cu, B, C, splits, (const float*)x, (const float*)dy, stats, partial);
  seg_final_kernel<<<2 * B * nchunk, 256, 0, st>>>(B, C, splits, 2, partial, dshift, dscale);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const pvj_plan* p, int which, int C, const void* y,
                           const void* gate, const void* dout, void* dy, float* dgate, int splits,
                           void* ws, hipStream_t st) {
  const ChainRows r = chain_rows(p, which, false);
  const int rows = r.rows, B = r.n_seg;
  if (B == 0) return hipSuccess;
  const int32_t* cu = r.cu;
  float* partial = static_cast<float*>(ws);
  const int nchunk = (C + kColChunk - 1) / kColChunk;
  (void)splits;
  const int R = gate_rows_per_slot(rows, B, C), ns = n_slots(rows, B, R);
  if (rows > 0) {
    if (p->desc.dtype == PVJ_BF16)
      gate_bwd_slots_kernel<bf16><<<ns * nchunk, 64, 0, st>>>(
          cu, B, C, R, (const bf16*)dout, (const bf16*)y, (const bf16*)gate, (bf16*)dy, partial);
    else
      gate_bwd_slots_kernel<float><<<ns * nchunk, 64, 0, st>>>(
          cu, B, C, R, (const float*)dout, (const float*)y, (const float*)gate, (float*)dy,
          partial);
  }
  const int nfin = (C + kFinalCols - 1) / kFinalCols;
  seg_final_slots_kernel<<<B * nfin, 1024, 0, st>>>(cu, B, C, R, 1, partial, dgate, nullptr);
  return hipGetLastError();
}

}  // namespace pvj
