// Device-side helpers shared by the EntmaxKV HIP kernels (gfx950, wave64).
#pragma once

#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "entmaxkv.h"

namespace ekv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element access.  K/V and box metadata are float32 or bfloat16; a bfloat16
// is the high half of a float32, so widening is a shift (exact).
// ---------------------------------------------------------------------------
struct F32 {
  using T = float;
  static constexpr int kBytes = 4;
};
struct BF16 {
  using T = uint16_t;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// Load 8 consecutive elements starting at p (16-byte aligned for bf16,
// 32-byte for f32) and widen them to float.
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8]) {
  const uint4 a = *reinterpret_cast<const uint4 *>(p);
  x[0] = bf16_lo(a.x); x[1] = bf16_hi(a.x);
  x[2] = bf16_lo(a.y); x[3] = bf16_hi(a.y);
  x[4] = bf16_lo(a.z); x[5] = bf16_hi(a.z);
  x[6] = bf16_lo(a.w); x[7] = bf16_hi(a.w);
}

// The 8 coordinates owned by lane li of a group of D/8 lanes that shares a
// row.  A 32-bit row is read as [4 li, 4 li + 4) and [D/2 + 4 li, ...): each
// of the lane's two 16-byte loads is then part of one contiguous span of the
// row across the group.  A 16-bit row is read as 8 consecutive values (one
// 16-byte load).  coord_of gives the coordinate of the lane's j-th value.
template <class T, int D>
__device__ __forceinline__ int coord_of(int li, int j) {
  if constexpr (sizeof(T) == 4) return j < 4 ? 4 * li + j : D / 2 + 4 * li + (j - 4);
  else return 8 * li + j;
}
template <int D>
__device__ __forceinline__ void load8_lane(const float *row, int li, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(row + 4 * li);
  const float4 b = *reinterpret_cast<const float4 *>(row + D / 2 + 4 * li);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <int D>
__device__ __forceinline__ void load8_lane(const uint16_t *row, int li, float (&x)[8]) {
  load8(row + 8 * li, x);
}

__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t *p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
__device__ __forceinline__ void store1(float *p, float x) { *p = x; }
// Only used for values that are already exactly representable in bfloat16
// (minima and maxima of bfloat16 keys), so truncation is exact.
__device__ __forceinline__ void store1(uint16_t *p, float x) {
  *p = static_cast<uint16_t>(__float_as_uint(x) >> 16);
}

// ---------------------------------------------------------------------------
// Lane-group reductions.  W lanes (power of two, <= 64) that are contiguous
// and W-aligned reduce to a value present in every lane of the group.
// Within a row of 16 lanes the data-parallel-primitive (DPP) lane swizzles
// are used: row_mirror pairs lane i with 15-i, row_half_mirror pairs i with
// 7-i inside each half row, and the two quad permutations exchange
// neighbours and pairs; across rows the cross-lane shuffle is used.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuad1032 = 0xB1;  // quad_perm(1, 0, 3, 2)
constexpr int kDppQuad2301 = 0x4E;  // quad_perm(2, 3, 0, 1)

template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: power of two");
  if constexpr (W >= 16) x += dpp_f<kDppRowMirror>(x);
  if constexpr (W >= 8) x += dpp_f<kDppRowHalfMirror>(x);
  if constexpr (W >= 4) x += dpp_f<kDppQuad2301>(x);
  if constexpr (W >= 2) x += dpp_f<kDppQuad1032>(x);
  if constexpr (W >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (W >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}
template <int W>
__device__ __forceinline__ float group_max(float x) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: power of two");
  if constexpr (W >= 16) x = fmaxf(x, dpp_f<kDppRowMirror>(x));
  if constexpr (W >= 8) x = fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
  if constexpr (W >= 4) x = fmaxf(x, dpp_f<kDppQuad2301>(x));
  if constexpr (W >= 2) x = fmaxf(x, dpp_f<kDppQuad1032>(x));
  if constexpr (W >= 32) x = fmaxf(x, __shfl_xor(x, 16, kWave));
  if constexpr (W >= 64) x = fmaxf(x, __shfl_xor(x, 32, kWave));
  return x;
}
// 64-bit values move through DPP as two 32-bit halves.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const unsigned long long v = static_cast<unsigned long long>(__double_as_longlong(x));
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(v >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(static_cast<long long>(
      (static_cast<unsigned long long>(static_cast<unsigned int>(hi)) << 32) |
      static_cast<unsigned int>(lo)));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
// The pairings are symmetric, so every lane of the group ends with the
// bitwise same sum.
template <int W>
__device__ __forceinline__ double group_sum_d(double x) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: power of two");
  if constexpr (W >= 16) x += dpp_d<kDppRowMirror>(x);
  if constexpr (W >= 8) x += dpp_d<kDppRowHalfMirror>(x);
  if constexpr (W >= 4) x += dpp_d<kDppQuad2301>(x);
  if constexpr (W >= 2) x += dpp_d<kDppQuad1032>(x);
  if constexpr (W >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (W >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}
template <int W>
__device__ __forceinline__ int group_sum_i(int x) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: power of two");
  if constexpr (W >= 16) x += dpp_i<kDppRowMirror>(x);
  if constexpr (W >= 8) x += dpp_i<kDppRowHalfMirror>(x);
  if constexpr (W >= 4) x += dpp_i<kDppQuad2301>(x);
  if constexpr (W >= 2) x += dpp_i<kDppQuad1032>(x);
  if constexpr (W >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (W >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

// Whole-wave reductions with the result in every lane.  Each 16-lane row is
// reduced with the swizzles above; then row_bcast:15 carries the last lane
// of rows 0 and 2 into rows 1 and 3, and row_bcast:31 carries lane 31 into
// rows 2 and 3, which leaves the total in lane 63 (read back to all lanes).
// No lane exchange goes through LDS, and the summation order is fixed.
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows(int x, int idle) {
  return __builtin_amdgcn_update_dpp(idle, x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const unsigned long long v = static_cast<unsigned long long>(__double_as_longlong(x));
  const unsigned lo = __builtin_amdgcn_readlane(static_cast<unsigned>(v), l);
  const unsigned hi = __builtin_amdgcn_readlane(static_cast<unsigned>(v >> 32), l);
  return __longlong_as_double(static_cast<long long>(
      (static_cast<unsigned long long>(hi) << 32) | lo));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_rows_d(double x) {  // idle rows read 0.0
  const unsigned long long v = static_cast<unsigned long long>(__double_as_longlong(x));
  const int lo = dpp_rows<CTRL, ROWS>(static_cast<int>(v), 0);
  const int hi = dpp_rows<CTRL, ROWS>(static_cast<int>(v >> 32), 0);
  return __longlong_as_double(static_cast<long long>(
      (static_cast<unsigned long long>(static_cast<unsigned int>(hi)) << 32) |
      static_cast<unsigned int>(lo)));
}
__device__ __forceinline__ double wave_sum_d(double x) {
  x = group_sum_d<16>(x);
  x += dpp_rows_d<kDppRowBcast15, 0xA>(x);
  x += dpp_rows_d<kDppRowBcast31, 0xC>(x);
  return readlane_d(x, kWave - 1);
}
__device__ __forceinline__ float wave_sum_f(float x) {
  x = group_sum<16>(x);
  x += __int_as_float(dpp_rows<kDppRowBcast15, 0xA>(__float_as_int(x), 0));
  x += __int_as_float(dpp_rows<kDppRowBcast31, 0xC>(__float_as_int(x), 0));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x = group_sum_i<16>(x);
  x += dpp_rows<kDppRowBcast15, 0xA>(x, 0);
  x += dpp_rows<kDppRowBcast31, 0xC>(x, 0);
  return __builtin_amdgcn_readlane(x, kWave - 1);
}
__device__ __forceinline__ float wave_min_f(float x) {
  x = -group_max<16>(-x);
  const int idle = __float_as_int(FLT_MAX);
  x = fminf(x, __int_as_float(dpp_rows<kDppRowBcast15, 0xA>(__float_as_int(x), idle)));
  x = fminf(x, __int_as_float(dpp_rows<kDppRowBcast31, 0xC>(__float_as_int(x), idle)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}
// For maxima a lane of a row the broadcast skips keeps its own value.
__device__ __forceinline__ float wave_max_f(float x) {
  x = group_max<16>(x);
  x = fmaxf(x, __int_as_float(dpp_rows<kDppRowBcast15, 0xA>(__float_as_int(x),
                                                            __float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_rows<kDppRowBcast31, 0xC>(__float_as_int(x),
                                                            __float_as_int(x))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_rows_keep_d(double x) {
  const unsigned long long v = static_cast<unsigned long long>(__double_as_longlong(x));
  const int lo = dpp_rows<CTRL, ROWS>(static_cast<int>(v), static_cast<int>(v));
  const int hi = dpp_rows<CTRL, ROWS>(static_cast<int>(v >> 32), static_cast<int>(v >> 32));
  return __longlong_as_double(static_cast<long long>(
      (static_cast<unsigned long long>(static_cast<unsigned int>(hi)) << 32) |
      static_cast<unsigned int>(lo)));
}
__device__ __forceinline__ double wave_max_d(double x) {
  x = fmax(x, dpp_d<kDppRowMirror>(x));
  x = fmax(x, dpp_d<kDppRowHalfMirror>(x));
  x = fmax(x, dpp_d<kDppQuad2301>(x));
  x = fmax(x, dpp_d<kDppQuad1032>(x));
  x = fmax(x, dpp_rows_keep_d<kDppRowBcast15, 0xA>(x));
  x = fmax(x, dpp_rows_keep_d<kDppRowBcast31, 0xC>(x));
  return readlane_d(x, kWave - 1);
}
// Inclusive prefix sum over the wave without LDS: within each 16-lane row
// by shifts of 1, 2, 4 and 8 lanes (a lane with no source adds 0), then the
// row totals carried into the later rows by the two row broadcasts.
__device__ __forceinline__ int wave_incl_scan_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += dpp_rows<kDppRowBcast15, 0xA>(x, 0);
  x += dpp_rows<kDppRowBcast31, 0xC>(x, 0);
  return x;
}

// Workgroup barrier that orders LDS accesses only.  Unlike __syncthreads()
// it does not wait for outstanding global loads, so loads issued before it
// stay in flight.  Use it wherever threads exchange data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) { return wave_incl_scan_dpp(x); }

// Exclusive prefix sum over a block of NT threads; also returns the total.
// `smem` must hold NT/64 ints.  Contains barriers: call from all threads.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int *smem, int &total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int incl = wave_incl_scan(x);
  lds_barrier();
  if (lane == kWave - 1) smem[wid] = incl;
  lds_barrier();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int v = smem[w];
    base += (w < wid) ? v : 0;
    tot += v;
  }
  total = tot;
  return base + incl - x;
}

// Block-wide reductions of NT threads; result valid in every thread.
// `smem` must hold NT/64 elements.  Contain barriers.
template <int NT>
__device__ __forceinline__ float block_max(float x, float *smem) {
  constexpr int NW = NT / kWave;
  x = group_max<kWave>(x);
  lds_barrier();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = x;
  lds_barrier();
  float r = smem[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, smem[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ double block_sum_d(double x, double *smem) {
  constexpr int NW = NT / kWave;
  x = group_sum_d<kWave>(x);
  lds_barrier();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = x;
  lds_barrier();
  double r = smem[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += smem[w];
  return r;
}
template <int NT>
__device__ __forceinline__ int block_sum_i(int x, int *smem) {
  constexpr int NW = NT / kWave;
  x = group_sum_i<kWave>(x);
  lds_barrier();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = x;
  lds_barrier();
  int r = smem[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += smem[w];
  return r;
}

// ---------------------------------------------------------------------------
// Ordered compaction of one tile of NT flags (one per thread): returns the
// flag's rank among the set flags of the tile (in thread order) and the
// tile's total.  `smem` holds NT/64 ints.  Contains barriers.
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ int tile_rank(bool flag, int *smem, int &total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const unsigned long long ball = __ballot(flag);
  const int below = __popcll(ball & ((1ull << lane) - 1ull));
  lds_barrier();
  if (lane == 0) smem[wid] = __popcll(ball);
  lds_barrier();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int v = smem[w];
    base += (w < wid) ? v : 0;
    tot += v;
  }
  total = tot;
  return base + below;
}

// ---------------------------------------------------------------------------
// Range-checked buffer stores.  A raw buffer resource covers `bytes` bytes
// from a wave-uniform base, and the hardware drops a lane's store when the
// lane's byte offset lies past the end.  Streaming kernels use them for
// stores that only some lanes make: behind a branch, a store would make the
// compiler assume it may not have been issued and then wait for more of the
// loads in flight than it needs to.
// ---------------------------------------------------------------------------
constexpr int kDropOffset = 0x7fffffff;  // past the end of every resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_rsrc(void *base,
                                                             size_t bytes) {
  // word 3: 32-bit data format, no swizzle; sizes are capped below the
  // drop offset
  const int n = static_cast<int>(bytes < 0x7fff0000u ? bytes : 0x7fff0000u);
  return __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), n,
                                           0x00020000);
}
__device__ __forceinline__ void store_if(__amdgpu_buffer_rsrc_t r, int byte_off,
                                         bool on, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r,
                                        on ? byte_off : kDropOffset, 0, 0);
}
__device__ __forceinline__ void store_if(__amdgpu_buffer_rsrc_t r, int byte_off,
                                         bool on, int v) {
  __builtin_amdgcn_raw_buffer_store_b32(static_cast<unsigned>(v), r,
                                        on ? byte_off : kDropOffset, 0, 0);
}

// ---------------------------------------------------------------------------
// Paged layout helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int n_pages_of(int len, int P) {
  return (len + P - 1) / P;
}
// Valid tokens of logical page lp of a sequence of length len.
__device__ __forceinline__ int page_tokens(int lp, int len, int P) {
  const int r = len - lp * P;
  return r < P ? r : P;
}
// Element offset of row (slot, head, token) in a [slots][H][P][D] pool.
__device__ __forceinline__ size_t pool_row(int slot, int h, int t, int H,
                                           int P, int D) {
  return ((static_cast<size_t>(slot) * H + h) * P + t) * static_cast<size_t>(D);
}
// Element offset of metadata row (slot, head, which) in [slots][H][2][D].
__device__ __forceinline__ size_t meta_row(int slot, int h, int which, int H,
                                           int D) {
  return ((static_cast<size_t>(slot) * H + h) * 2 + which) *
         static_cast<size_t>(D);
}

}  // namespace ekv
