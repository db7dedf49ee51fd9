// Helpers shared by the decode kernels (kpass.hip, decode.hip): block
// sizes, the flattened work lists over units, the query split for the
// matrix cores, and grid sizing.
#pragma once

#include <float.h>

#include "ekv_device.h"
#include "ekv_kernels.h"

namespace ekv {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kMaxChunkPages = kChunkTokens / 16;  // smallest page size
constexpr int kMaxUnits = 4096;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Work lists.  Work items (pages or chunks of pages) of all units are laid
// end to end, unit by unit; a persistent grid walks them with a stride.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int unit_pages(const int32_t *seq_lens,
                                          const int32_t *sel,
                                          const int32_t *count, int u, int H,
                                          int P) {
  return sel ? count[u] : n_pages_of(seq_lens[u / H], P);
}

// pref[u] = first item of unit u (pref[units] = total); returns the total.
// With `done` (one flag per query head, G per unit), units whose heads are
// all done contribute no items.
template <int NT>
__device__ int build_unit_prefix(int *pref, int *tmp, const int32_t *seq_lens,
                                 const int32_t *sel, const int32_t *count,
                                 int units, int H, int P, int pages_per_item,
                                 const int32_t *done = nullptr, int G = 0) {
  const int per = (units + NT - 1) / NT;
  const int u0 = threadIdx.x * per, u1 = min(units, u0 + per);
  auto items = [&](int u) {
    if (done) {
      bool all = true;
      for (int g = 0; g < G; ++g) all &= done[u * G + g] != 0;
      if (all) return 0;
    }
    return (unit_pages(seq_lens, sel, count, u, H, P) + pages_per_item - 1) /
           pages_per_item;
  };
  int local = 0;
  for (int u = u0; u < u1; ++u) local += items(u);
  int total;
  int base = block_excl_scan<NT>(local, tmp, total);
  for (int u = u0; u < u1; ++u) {
    pref[u] = base;
    base += items(u);
  }
  if (threadIdx.x == 0) pref[units] = total;
  lds_barrier();
  return total;
}

// Largest u with pref[u] <= f.
__device__ __forceinline__ int find_unit(const int *pref, int units, int f) {
  int lo = 0, hi = units - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= f) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Location of a selected page.
struct PageRef {
  int u, j, lp, slot, nt;
};

__device__ __forceinline__ PageRef page_ref(const int *pref, int units, int f,
                                            const int32_t *page_table,
                                            const int32_t *seq_lens,
                                            const int32_t *sel, int H, int P,
                                            int max_pages) {
  PageRef r;
  r.u = find_unit(pref, units, f);
  r.j = f - pref[r.u];
  const int b = r.u / H;
  r.lp = sel ? sel[static_cast<size_t>(r.u) * max_pages + r.j] : r.j;
  r.slot = page_table[static_cast<size_t>(b) * max_pages + r.lp];
  r.nt = page_tokens(r.lp, seq_lens[b], P);
  return r;
}

__device__ __forceinline__ float pow_r(float x, int r, float rg) {
  // x >= 0.  r = 1 (alpha = 2), r = 2 (alpha = 1.5), else x^rg.
  if (r == 1) return x;
  if (r == 2) return x * x;
  return x > 0.f ? powf(x, rg) : 0.f;
}

// ---------------------------------------------------------------------------
// 1a. Scores on the matrix cores (bfloat16 keys).
//
// v_mfma_f32_16x16x32_bf16 multiplies a 16x32 A by a 32x16 B.  B holds 16
// tokens' keys for 32 coordinates: lane l supplies 8 consecutive
// coordinates (one 16-byte load) of token l%16, block l/16.  A holds the
// query: row 4*s + g is the s-th bfloat16 part of (alpha-1)*scale*q_g, where
// q = part0 + part1 + part2 to float32 precision (each part is the bfloat16
// rounding of what the previous parts left over); rows 12..15 are zero.
// Products of bfloat16 values are exact and accumulate in float32, so
// summing the three row results gives z to float32 accuracy.  Output lane l
// holds rows 4*(l/16) + i of column l%16, i.e. part l/16 of head i.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kb_of(int lane) { return lane >> 4; }

__device__ __forceinline__ float bf16_part(float x, int part) {
  const float p0 = static_cast<float>(static_cast<__bf16>(x));
  const float r1 = x - p0;
  const float p1 = static_cast<float>(static_cast<__bf16>(r1));
  const float r2 = r1 - p1;
  const float p2 = static_cast<float>(static_cast<__bf16>(r2));
  return part == 0 ? p0 : part == 1 ? p1 : p2;
}

template <int D, int G>
__device__ __forceinline__ void load_q_parts(bf16x8_t (&a)[(G + 3) / 4][D / 32],
                                             const float *q, int b, int h,
                                             int H, float zscale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, kb = lane >> 4;
  const int Hq = H * G;
#pragma unroll
  for (int ps = 0; ps < (G + 3) / 4; ++ps) {
    const int part = n >> 2, g = (n & 3) + 4 * ps;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float x = 0.f;
        if (part < 3 && g < G)
          x = bf16_part(q[(static_cast<size_t>(b) * Hq + h * G + g) * D +
                          32 * s + 8 * kb + i] * zscale, part);
        a[ps][s][i] = static_cast<__bf16>(x);
      }
  }
}

// ---------------------------------------------------------------------------
// Grid sizing (host)
// ---------------------------------------------------------------------------
// Persistent grid: enough blocks to fill the device, never more than items.
static inline int persistent_blocks(size_t max_items, int per_cu) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess || n_cu <= 0)
    n_cu = 256;
  const size_t cap = static_cast<size_t>(n_cu) * per_cu;
  if (max_items == 0) return 1;
  return static_cast<int>(max_items < cap ? max_items : cap);
}

// Blocks of `kern` the device holds at once, at most `max_items`.
template <class K>
static inline int resident_blocks(K kern, int threads, size_t max_items) {
  int dev = 0, n_cu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess || n_cu <= 0)
    n_cu = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void *>(kern), threads, 0) !=
          hipSuccess || per_cu <= 0)
    per_cu = 1;
  const size_t cap = static_cast<size_t>(n_cu) * per_cu;
  if (max_items == 0) return 1;
  return static_cast<int>(max_items < cap ? max_items : cap);
}

}  // namespace ekv
