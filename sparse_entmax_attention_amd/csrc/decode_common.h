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

// Wave-wide sums of a, b, c and minimum of m, every value in every lane.
// The four reductions are interleaved step by step (each swizzle of one
// value covers the data hazard of the next), with the fixed pattern of the
// single-value reductions: row swizzles, then the row broadcasts into lane 63.
__device__ __forceinline__ void wave_sum3_min(float &a, float &b, float &c, float &m) {
#define EKV_STEP(CTRL)                                  \
  {                                                     \
    const float a_ = dpp_f<CTRL>(a), b_ = dpp_f<CTRL>(b); \
    const float c_ = dpp_f<CTRL>(c), m_ = dpp_f<CTRL>(m); \
    a += a_; b += b_; c += c_; m = fminf(m, m_);         \
  }
  EKV_STEP(kDppRowMirror)
  EKV_STEP(kDppRowHalfMirror)
  EKV_STEP(kDppQuad2301)
  EKV_STEP(kDppQuad1032)
#undef EKV_STEP
  const int big = __float_as_int(FLT_MAX);
#define EKV_BCAST(CTRL, ROWS)                                                \
  {                                                                          \
    const float a_ = __int_as_float(dpp_rows<CTRL, ROWS>(__float_as_int(a), 0)); \
    const float b_ = __int_as_float(dpp_rows<CTRL, ROWS>(__float_as_int(b), 0)); \
    const float c_ = __int_as_float(dpp_rows<CTRL, ROWS>(__float_as_int(c), 0)); \
    const float m_ = __int_as_float(dpp_rows<CTRL, ROWS>(__float_as_int(m), big)); \
    a += a_; b += b_; c += c_; m = fminf(m, m_);                            \
  }
  EKV_BCAST(kDppRowBcast15, 0xA)
  EKV_BCAST(kDppRowBcast31, 0xC)
#undef EKV_BCAST
  a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), kWave - 1));
  b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b), kWave - 1));
  c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), kWave - 1));
  m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), kWave - 1));
}

// Exact threshold by support iteration, one wave, over R register slots of y
// per lane (-inf marks an unused slot), from t0, a lower bound on tau in the
// same origin: over S(t) = {y > t} the closed form t* of the threshold of
// that support (sparsemax: (sum y - 1)/K; 1.5-entmax: the smaller root of
// sum_S (y - t)^2 = 1) is tau once t* < min_S y, since then S(t*) = S;
// otherwise t moves up, to t* for r = 1 (Michelot's step: over a superset of
// the support the terms below tau are negative, so t* <= tau) and by a
// Newton step on F^(1/2) - 1 for r = 2 (convex, so the step stays below
// tau).  Sums are taken in float32 (each lane's R slots in order, then the
// wave in a fixed pattern: the result is the same on every run), the steps
// in float32, and the closed form of the final support in double.  No slot
// is branched on.  Returns false when no support is found in `iters` passes.
template <int R>
__device__ __forceinline__ bool wave_support_iter(const float (&y)[R], float t0,
                                                  int r, int iters, double &tau) {
  float t = t0;
  for (int it = 0; it < iters; ++it) {
    float kf = 0.f, sy = 0.f, sy2 = 0.f, ymin = FLT_MAX;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const bool in = y[k] > t;
      const float yy = in ? y[k] : 0.f;
      kf += in ? 1.f : 0.f;
      sy += yy;
      sy2 = fmaf(yy, yy, sy2);
      ymin = fminf(ymin, in ? y[k] : FLT_MAX);
    }
    wave_sum3_min(kf, sy, sy2, ymin);  // kf: exact count
    if (kf == 0.f) return false;
    const double kd = static_cast<double>(kf);
    const double SY = static_cast<double>(sy), SY2 = static_cast<double>(sy2);
    float tn;
    if (r == 1) {
      tn = (sy - 1.f) / kf;
      if (tn < ymin) { tau = (SY - 1.0) / kd; return true; }
    } else {
      const float disc = sy * sy - kf * (sy2 - 1.f);
      if (disc >= 0.f && (sy - sqrtf(disc)) / kf < ymin) {
        tau = (SY - sqrt(fmax(SY * SY - kd * (SY2 - 1.0), 0.0))) / kd;
        return true;
      }
      const float F = fmaf(kf * t, t, fmaf(-2.f * t, sy, sy2));
      const float Dv = fmaf(-kf, t, sy);
      tn = t + (F - sqrtf(F)) / Dv;
    }
    if (!(tn > t)) { tau = t; return true; }  // converged to rounding
    t = tn;
  }
  return false;
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

// A of the MFMA for the G query heads of KV head h in sequence b: row
// 4 part + e of pass ps is the part-th bfloat16 part of zscale q_{4 ps + e}
// (rows 12..15 and heads past G are zero), lane n + 16 kb holding
// coordinates 32 s + 8 kb .. + 7 of its row for each k-step s.  Every load
// is issued before any is used (rows with no head read head 0 and are zeroed
// afterwards): a load behind a branch would be waited for on its own, one
// memory round trip after another.  q is 16-byte aligned (the entry points
// check it) and D a multiple of 32.
template <int D, int G>
__device__ __forceinline__ void load_q_parts(bf16x8_t (&a)[(G + 3) / 4][D / 32],
                                             const float *q, int b, int h,
                                             int H, float zscale) {
  constexpr int NP = (G + 3) / 4, KS = D / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, kb = lane >> 4;
  const int Hq = H * G;
  float4 raw[NP][KS][2];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int g = (n & 3) + 4 * ps;
    const float *src = q + (static_cast<size_t>(b) * Hq + h * G + (g < G ? g : 0)) * D +
                       8 * kb;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      raw[ps][s][0] = *reinterpret_cast<const float4 *>(src + 32 * s);
      raw[ps][s][1] = *reinterpret_cast<const float4 *>(src + 32 * s + 4);
    }
  }
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int part = n >> 2, g = (n & 3) + 4 * ps;
    const bool on = part < 3 && g < G;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float x[8] = {raw[ps][s][0].x, raw[ps][s][0].y, raw[ps][s][0].z,
                          raw[ps][s][0].w, raw[ps][s][1].x, raw[ps][s][1].y,
                          raw[ps][s][1].z, raw[ps][s][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[ps][s][i] = static_cast<__bf16>(on ? bf16_part(x[i] * zscale, part) : 0.f);
    }
  }
}

// The same operand as load_q_parts in two steps, for a kernel with LDS to
// spare: load_q_rows issues the loads of the unit's G query rows, each
// 16-byte piece once (lanes past the rows re-read the last one), and
// q_parts_from_rows passes them through `stage`, the wave's own G*D/4
// float4s of LDS, to the lanes that need them.  Every wave of a launch
// starts by reading the same few KiB of queries; with the four lanes that
// share a row each reading it (8 KiB per wave) that start waited several
// microseconds on the caches.  Splitting the steps lets the caller issue
// other loads between them.
template <int D, int G>
struct QRows {
  static constexpr int kLoads = (G * D / 4 + kWave - 1) / kWave;  // per lane
  float4 v[kLoads];
};

template <int D, int G>
__device__ __forceinline__ void load_q_rows(QRows<D, G> &r, const float *q, int b,
                                            int h, int H) {
  constexpr int NV = G * D / 4;  // float4s of the unit's rows
  const int lane = threadIdx.x & (kWave - 1);
  const float4 *src = reinterpret_cast<const float4 *>(
      q + (static_cast<size_t>(b) * H * G + h * G) * D);
#pragma unroll
  for (int i = 0; i < QRows<D, G>::kLoads; ++i) r.v[i] = src[min(lane + kWave * i, NV - 1)];
}

template <int D, int G>
__device__ __forceinline__ void q_parts_from_rows(bf16x8_t (&a)[(G + 3) / 4][D / 32],
                                                  const QRows<D, G> &r, float zscale,
                                                  float4 *stage) {
  constexpr int NP = (G + 3) / 4, KS = D / 32;
  constexpr int NV = G * D / 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, kb = lane >> 4;
#pragma unroll
  for (int i = 0; i < QRows<D, G>::kLoads; ++i)
    if (lane + kWave * i < NV) stage[lane + kWave * i] = r.v[i];
  // (the wave's LDS operations complete in order: its reads below see the
  // writes of all its lanes)
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int part = n >> 2, g = (n & 3) + 4 * ps;
    const bool on = part < 3 && g < G;
    const int row = (g < G ? g : 0) * (D / 4) + 2 * kb;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float4 r0 = stage[row + 8 * s], r1 = stage[row + 8 * s + 1];
      const float x[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[ps][s][i] = static_cast<__bf16>(on ? bf16_part(x[i] * zscale, part) : 0.f);
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
