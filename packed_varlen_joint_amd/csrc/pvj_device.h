// Device helpers for the gfx950 kernels: vector types, bf16 conversion,
// matrix-core wrappers, token positions and the per-chunk 2D rotation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pvj_internal.h"

namespace pvj {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Eight consecutive elements of a row: the unit every kernel moves and the
// operand one lane feeds to one 32x32 matrix-core k-step of 16.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<float> { typedef f32x8 type; };

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type load8(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}
template <typename T>
__device__ __forceinline__ void store8(T* p, typename Vec8<T>::type v) {
  *reinterpret_cast<typename Vec8<T>::type*>(p) = v;
}

__device__ __forceinline__ f32x8 to_f32x8(bf16x8 v) {
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (float)v[i];
  return r;
}
__device__ __forceinline__ f32x8 to_f32x8(f32x8 v) { return v; }

template <typename T> __device__ __forceinline__ typename Vec8<T>::type from_f32x8(f32x8 v);
template <> __device__ __forceinline__ bf16x8 from_f32x8<bf16>(f32x8 v) {
  bf16x8 r;  // round to nearest even (v_cvt_pk_bf16_f32)
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)v[i];
  return r;
}
template <> __device__ __forceinline__ f32x8 from_f32x8<float>(f32x8 v) { return v; }

// acc(32x32) += A(32x16) * B(16x32) on the matrix cores.  Lane l feeds row
// (A) or column (B) l % 32 with eight k-values; lanes l and l + 32 feed the
// two k-halves.  bf16: one v_mfma_f32_32x32x16_bf16.  fp32: eight
// v_mfma_f32_32x32x2_f32, element j of both operands forming k-step j.
__device__ __forceinline__ void mma16(f32x16& acc, bf16x8 a, bf16x8 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& acc, f32x8 a, f32x8 b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
}

// exp2 on the transcendental unit (v_exp_f32); exp2(-inf) = 0
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max of a value held by lanes l and l ^ 32 (v_permlane32_swap)
__device__ __forceinline__ float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The sample holding packed row `tok`: the i with cu[i] <= tok < cu[i+1].
__device__ __forceinline__ int find_sample(const int32_t* cu, int n_samples, int tok) {
  int lo = 1, hi = n_samples;  // first j in [1, n] with cu[j] > tok
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] > tok) hi = mid; else lo = mid + 1;
  }
  return lo - 1;
}

// Row of a sample's token (local index j in [0, L)) in a token tensor: the
// joint layout keeps a sample's rows together (text, then image); the
// stream-major layout keeps all text rows first, then all image rows, each in
// sample order.
template <bool SM>
__device__ __forceinline__ int token_row(const SampleInfo& si, int j) {
  if constexpr (SM) return j < si.l_text ? si.text_row + j : si.img_row + (j - si.l_text);
  else return si.start + j;
}

// RoPE position (row, col, frame) of local token j of a sample: text tokens
// first at (0, 0, 0), then the image grids frame after frame, each row-major
// (a plain sample has one frame, so frame = 0).
struct RopePos {
  int r, c, f;
};
__device__ __forceinline__ RopePos token_pos3(int j, const SampleInfo& si) {
  RopePos p = {0, 0, 0};
  if (j >= si.l_text) {  // then the sample has image tokens, so hw > 0
    int q = j - si.l_text;
    const int f = q / si.hw;
    q -= f * si.hw;
    const int r = q / si.w_lat;
    p.r = r;
    p.c = q - r * si.w_lat;
    p.f = f;
  }
  return p;
}

// Position along the RoPE axis of head-dim unit u (dims 8u .. 8u+7): every
// axis part is a whole number of units (row, then column, then frame).
__device__ __forceinline__ int unit_axis(int u, const Meta& m) {
  return u < m.rope_u0 ? 0 : (u < m.rope_u1 ? 1 : 2);
}
__device__ __forceinline__ int axis_pos(const RopePos& p, int axis) {
  return axis == 0 ? p.r : (axis == 1 ? p.c : p.f);
}

// Rotate the 8 dims of unit u (pairs 4u .. 4u+3) at axis position pos with the
// plan's cos/sin tables ([pos][D/2 pairs]); pairs (2k, 2k+1) turn as
// (a, b) -> (a cos - b sin, a sin + b cos); inverse turns by -angle.
// the rotation of one unit by its table entries (cos, sin of the unit's four pairs)
__device__ __forceinline__ f32x8 rope_rotate(f32x8 x, f32x4 cs, f32x4 sn, bool inverse) {
  if (inverse) sn = -sn;
  // explicit fma order, so every kernel that rotates rounds the same way
  f32x8 y;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = x[2 * q], b = x[2 * q + 1];
    y[2 * q] = __builtin_fmaf(a, cs[q], -(b * sn[q]));
    y[2 * q + 1] = __builtin_fmaf(a, sn[q], b * cs[q]);
  }
  return y;
}
__device__ __forceinline__ f32x8 rope_unit(f32x8 x, int u, int pos, const Meta& m, bool inverse) {
  const size_t to = (size_t)pos * m.n_pairs + 4 * u;
  const f32x4 cs = *reinterpret_cast<const f32x4*>(m.cos_tab + to);
  const f32x4 sn = *reinterpret_cast<const f32x4*>(m.sin_tab + to);
  return rope_rotate(x, cs, sn, inverse);
}

// ---------------------------------------------------------------------------
// LDS tiles shared by the attention kernels (all use 256-thread workgroups)
// ---------------------------------------------------------------------------
constexpr int kTileThreads = 256;

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Row order sigma inside every 32-row block: bits 2 and 3 of the row swapped.
// Tiles whose rows feed the A operand of a 32x32 product are stored in this
// order so that accumulator register r of lane l holds row
// 16(r/8) + 8(l/32) + r%8 of the block: the eight registers 8s..8s+7 then
// cover eight consecutive rows, which is exactly one 16-wide k-step operand of
// a following product over those rows.  (sigma is its own inverse.)
__device__ __forceinline__ int bsigma(int k) { return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1); }

// XOR swizzle of the 8-element (16-byte) units of an LDS tile row, chosen
// from the measured bank behaviour of gfx950 LDS (64 banks of 4 bytes):
//  * a ds_read_b128 operand read (lane l: row l%32, one unit) is served 16
//    lanes at a time, so 16 consecutive rows must land on 16 different
//    16-byte slots of a 256-byte bank window;
//  * a transposing ds_read_b64_tr_b16 (16 lanes: 4 consecutive rows x one
//    pair of adjacent units) needs those 4 rows on different unit pairs.
// D = 128 (256-byte rows): unit ^= (row&3)<<2 | (row>>2)&3, a permutation of
// 0..15 over any 16 aligned rows whose bits 1..2 differ within 4 rows.
// D = 64 (128-byte rows, two rows per bank window): rows of one parity need
// 8 different units, and rows 4i, 4i+2 different pairs:
// unit ^= ((row>>1)&1)<<2 | (row>>2)&3.
template <int D>
__device__ __forceinline__ int tsw(int row) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
// element offset of (row, col) in a row-major LDS tile of D columns
template <int D>
__device__ __forceinline__ int toff(int row, int col) {
  return row * D + (((col >> 3) ^ tsw<D>(row)) << 3) + (col & 7);
}

// The 8-slot 32x32x16 operand fragment F[j] = M[kb8 + j][n] of a row-major
// LDS tile M (rows = k, columns = n), where kb8 = kbase + 8*(lane/32) and
// n = nbase + lane%32; `row_of` maps a logical k row to its LDS row.
// bf16: two ds_read_b64_tr_b16.  Inside each 16-lane group, source lane
// s = 4j + c reads row k0 + j, columns n0 + 4c .. n0 + 4c + 3, and lane i
// receives M[k0 .. k0+3][n0 + i] (measured layout of the instruction).
// fp32 (no transposing read for 32-bit data): eight scalar reads.
template <int D, typename RowOf>
__device__ __forceinline__ bf16x8 frag_t(const bf16* M, int kbase, int nbase, RowOf row_of) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, s = lane & 15;
  bf16x8 f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = row_of(kbase + 8 * (g >> 1) + 4 * t + (s >> 2));
    const int col = nbase + 16 * (g & 1) + 4 * (s & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(M + toff<D>(row, col)));
    const bf16x4 b = __builtin_bit_cast(bf16x4, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 * t + e] = b[e];
  }
  return f;
}
template <int D, typename RowOf>
__device__ __forceinline__ f32x8 frag_t(const float* M, int kbase, int nbase, RowOf row_of) {
  const int lane = threadIdx.x & 63;
  const int kb8 = kbase + 8 * (lane >> 5), n = nbase + (lane & 31);
  f32x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = M[toff<D>(row_of(kb8 + j), n)];
  return f;
}

// Direct global -> LDS copy (buffer_load_dwordx4 ... lds, no VGPR round trip)
// of a [ROWS][D] bf16 tile by a workgroup of THREADS threads: rows row0 ..
// row0+ROWS-1 of one (sample, head),
// stored in LDS row sigma(r) with the tsw swizzle.  Each instruction writes
// one wave's 64 consecutive 16-byte LDS slots in lane order, so every lane
// loads the global unit that belongs in its slot.  The copies complete
// asynchronously: wait_dma() before the barrier that publishes the tile.
//
// The source is addressed through a buffer resource built per copy: its base
// is the tile's first row and it spans exactly the sample's remaining rows
// (num_records = ((L-1-row0) RS + D) * 2 bytes).  Each thread's byte offset
// inside a tile is fixed (computed once) and is the only offset the hardware
// range-checks (the scalar offset of a buffer access is outside the check, so
// it is left at zero), hence rows at or past the sample end fall outside the
// resource and read as zeros: no clamp, and no data from the next sample or
// from past the end of the tensor.  The planner keeps a sample's span below
// 2 GiB, so the 32-bit offsets never wrap.
template <int D, int ROWS, int THREADS = kTileThreads>
struct DmaTile {
  static constexpr int UPR = D / 8;
  static constexpr int PER = ROWS * UPR / THREADS;
  // copy instruction i of a thread moves tile row STRIDE * i + rb (source
  // order), unit ub: the swizzle and sigma only touch row bits 0-3
  static constexpr int STRIDE = THREADS / UPR;
  static_assert(STRIDE % 16 == 0, "copy rows of one thread differ in bits 4 and up only");
  uint32_t off[PER];
  int wave;
  // byte offset of copy 0 inside a tile whose first row is at offset 0:
  // rb * RS * 2 + ub for source row rb < STRIDE and unit offset ub < D * 2
  // (kept for the stream-major copies only; 32-bit there)
  uint32_t c0;
  __device__ __forceinline__ explicit DmaTile(size_t RS) {
    wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int slot = (i * (THREADS / 64) + wave) * 64 + lane;
      const int rho = slot / UPR;
      const int u = (slot % UPR) ^ tsw<D>(rho);
      off[i] = (uint32_t)(((size_t)bsigma(rho) * RS + (size_t)u * 8) * sizeof(bf16));
    }
    const int rho0 = (wave * 64 + lane) / UPR;
    const uint32_t ub = (uint32_t)((((wave * 64 + lane) % UPR) ^ tsw<D>(rho0)) * 8 * sizeof(bf16));
    c0 = (uint32_t)bsigma(rho0) * (uint32_t)(RS * sizeof(bf16)) + ub;
  }
  // source: the head whose row 0 is at g, rows 0 .. L-1 (the buffer resource
  // is built where it is used: only device code handles the resource type)
  struct Src {
    const bf16* g;
    int L;
  };
  __device__ __forceinline__ static Src src(const void* g, size_t RS, int L) {
    (void)RS;
    return Src{static_cast<const bf16*>(g), L};
  }
  // copy rows row0 .. row0 + ROWS - 1 (dma_copy below)
  __device__ __forceinline__ void copy(void* tile, Src sr, size_t RS, int row0) const;
  // only the i-th of the PER copy instructions of that tile, so a kernel can
  // spread one tile's copies over its instruction stream
  __device__ __forceinline__ void part(void* tile, Src sr, size_t RS, int row0, int i) const;
  // the same for a stream-major tensor (token_row<true>): the tile's rows
  // row0 .. of the sample lie in two runs (text, image), so each lane picks
  // one of two run bases per copy; g is the tensor's head base and `bytes`
  // (sm_bytes) ends at the sample's last image row, so rows at or past the
  // sample end (always on the image side) read as zeros
  __device__ __forceinline__ void part_sm(void* tile, const bf16* g, int bytes, uint32_t rsb,
                                          uint32_t c1, const SampleInfo& si, int row0,
                                          int i) const;
  // c1 of part_sm: copy 0's offset for an image row, relative to the text run
  __device__ __forceinline__ uint32_t sm_c1(const SampleInfo& si, uint32_t rsb) const {
    return c0 + (uint32_t)(si.img_row - si.l_text - si.text_row) * rsb;
  }
};

// The resource-building copy is a free function template: kept out of the
// kernels' own bodies, the host-side compile of the kernel templates does not
// see the resource type.  g is the tile's first row; bytes spans the rows of
// the sample from there on.
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void dma_copy(const uint32_t* off, int wave, void* tile, const bf16* g,
                                         int bytes) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(g), (short)0, bytes, 0x00020000);
  bf16* t = static_cast<bf16*>(tile);
#pragma unroll
  for (int i = 0; i < DmaTile<D, ROWS, THREADS>::PER; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(t + (i * (THREADS / 64) + wave) * 512),
        16, off[i], 0, 0, 0);
}
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void dma_copy_one(uint32_t off, int wave, int i, void* tile,
                                             const bf16* g, int bytes) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(g), (short)0, bytes, 0x00020000);
  bf16* t = static_cast<bf16*>(tile);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(t + (i * (THREADS / 64) + wave) * 512), 16,
      off, 0, 0, 0);
}
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void DmaTile<D, ROWS, THREADS>::part(void* tile, Src sr, size_t RS,
                                                               int row0, int i) const {
  const int left = sr.L - row0;
  const int bytes = left > 0 ? (int)(((size_t)(left - 1) * RS + D) * sizeof(bf16)) : 0;
  dma_copy_one<D, ROWS, THREADS>(off[i], wave, i, tile, sr.g + (size_t)row0 * RS, bytes);
}
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void DmaTile<D, ROWS, THREADS>::copy(void* tile, Src sr, size_t RS,
                                                               int row0) const {
  // rows of the sample from row0 on (row0 < L at every call site; a tile at or
  // past the end would get an empty resource and read zeros)
  const int left = sr.L - row0;
  const int bytes = left > 0 ? (int)(((size_t)(left - 1) * RS + D) * sizeof(bf16)) : 0;
  dma_copy<D, ROWS, THREADS>(off, wave, tile, sr.g + (size_t)row0 * RS, bytes);
}
// Resource size for stream-major copies of one sample from a tensor's head
// base: up to the end of the sample's last image row.  Every text row of the
// tensor lies below every image row, and the rows past the sample's end that a
// tile covers map past its image run (to the next sample's rows or past the
// tensor), so they fall outside and read as zeros.
template <int D>
__device__ __forceinline__ int sm_bytes(const SampleInfo& si, size_t RS) {
  const int end = si.img_row + (si.len - si.l_text);  // one past the last image row
  return end > 0 ? (int)(((size_t)(end - 1) * RS + D) * sizeof(bf16)) : 0;
}
// The resource of copy i starts at text-run row rr = row0 + STRIDE i of the
// sample (a uniform base, so only the range check needs the lane's row): a
// text row's lane reads at c0 from there, an image row's lane at c1 = c0 +
// (img_row - l_text - text_row) rsb (>= c0: every text row lies below the
// sample's image rows).  Row rr + rb is a text row iff rb < l_text - rr, and
// since 0 <= ub < rsb that is c0 < (l_text - rr) rsb (signed): a uniform
// threshold, then a compare and a select per lane.  32-bit offsets: the caller
// keeps (tokens + 256) * RS * 2 below 2^31, so neither the offsets nor the
// threshold wrap.  A copy whose base is past `bytes` has only rows past the
// sample's end (an image lane's offset is at least the base) and gets an
// empty resource.
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void DmaTile<D, ROWS, THREADS>::part_sm(void* tile, const bf16* g,
                                                                  int bytes, uint32_t rsb,
                                                                  uint32_t c1,
                                                                  const SampleInfo& si, int row0,
                                                                  int i) const {
  const int rr = row0 + STRIDE * i;
  const uint32_t a = (uint32_t)(si.text_row + rr) * rsb;
  const int thr = __builtin_amdgcn_readfirstlane((si.l_text - rr) * (int)rsb);
  const uint32_t o = (int)c0 < thr ? c0 : c1;
  const int left = bytes - (int)a;
  dma_copy_one<D, ROWS, THREADS>(
      o, wave, i, tile,
      reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(g) + a), left > 0 ? left : 0);
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Scheduling groups of one product phase of the phase-shifted attention
// kernels: N products, of which those in [D0, D1) read their operand with two
// transposing reads (ds_read_b64_tr_b16) and the others with one row read
// (ds_read_b128).  First the reads of the first AHEAD products, then per
// product the product and the reads of the product AHEAD further on, and
// after some products one tile copy instruction (NC spread evenly).
__host__ __device__ constexpr int pp_reads(int i, int d0, int d1) {
  return (i >= d0 && i < d1) ? 2 : 1;
}
__host__ __device__ constexpr int pp_first_reads(int n, int d0, int d1, int ahead) {
  int r = 0;
  for (int i = 0; i < ahead && i < n; ++i) r += pp_reads(i, d0, d1);
  return r;
}
// Product i of N is followed by a tile copy instruction when pp_copy_after(i,
// N, NC) (NC copies spread evenly over the N products).
__host__ __device__ constexpr bool pp_copy_after(int i, int n, int nc) {
  return nc > 0 && ((i + 1) * nc) / n != (i * nc) / n;
}
template <int I, int N, int D0, int D1, int AHEAD, int NC>
__device__ __forceinline__ void pp_sched_ops() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I + AHEAD < N)
      __builtin_amdgcn_sched_group_barrier(0x100, pp_reads(I + AHEAD, D0, D1), 0);
    if constexpr (pp_copy_after(I, N, NC)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    pp_sched_ops<I + 1, N, D0, D1, AHEAD, NC>();
  }
}
template <int N, int D0, int D1, int AHEAD, int NC>
__device__ __forceinline__ void pp_sched() {
  __builtin_amdgcn_sched_group_barrier(0x100, pp_first_reads(N, D0, D1, AHEAD), 0);
  pp_sched_ops<0, N, D0, D1, AHEAD, NC>();
}

}  // namespace pvj
