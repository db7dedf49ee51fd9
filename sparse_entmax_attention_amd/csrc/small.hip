// Sparse alpha-entmax attention over a small selection in one launch
// (Technical Summary: EntmaxKV, §2.C "Sparse Entmax Attention", and §2.B.1:
// a fixed budget of k pages).  When the selected tokens of a unit fit on
// chip (at most 2048), NB blocks share the unit: each gathers the keys of
// its share of the selection through the page table and computes z =
// (alpha-1) scale <q, k> for the unit's G query heads on the matrix cores.
// The last of the NB blocks to finish (a per-unit arrival counter) collects
// all of the unit's scores, solves each head's threshold with one wave, and
// sums the value rows of the union of the heads' supports for every head.
// A single block (NB = 1, many units) keeps every score on chip.
#include <float.h>

#include <algorithm>

#include "decode_common.h"

namespace ekv {

constexpr int kSmallThreads = 512;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallIters = 64;  // support iterations before bisection

// One wave's exact threshold of n values y (ys[i] - shift; -inf past n) that
// lie in [-1, 0] or below, with max y = 0, returned in the same offset.
// r in {1, 2}: the support iteration from t = -1 (tau >= max y - 1).  Other
// r, or no clean support after kSmallIters passes: bisection on [-1, 0]
// (sums in float32 per lane, the wave in a fixed pattern).
template <int R>
__device__ __forceinline__ double wave_solve(const float *ys, int n, float shift,
                                             int r, float rg) {
  const int lane = threadIdx.x & (kWave - 1);
  float y[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int i = lane + k * kWave;
    y[k] = ys[i < n ? i : 0] - shift;
    y[k] = i < n ? y[k] : -INFINITY;
  }
  if (r == 1 || r == 2) {
    double tau;
    if (wave_support_iter<R>(y, -1.f, r, kSmallIters, tau)) return tau;
  }
  // bisection: sum max(y - mid, 0)^r >= 1 keeps mid below tau
  double lo = -1.0, hi = 0.0;
  for (int it = 0; it < 30; ++it) {
    const double mid = 0.5 * (lo + hi);
    const float mf = static_cast<float>(mid);
    float fs = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float d = fmaxf(y[k] - mf, 0.f);
      fs += r == 1 ? d : r == 2 ? d * d : (d > 0.f ? powf(d, rg) : 0.f);
    }
    if (wave_sum_f(fs) >= 1.f) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// Exact threshold of one head's scores zs[0 .. n) (-inf past n) by one
// wave: their maximum M, then the threshold of y = z - M.
template <int T>
__device__ __forceinline__ double head_threshold(const float *zs, int n, int r,
                                                 float rg) {
  const int lane = threadIdx.x & (kWave - 1);
  float mloc = -FLT_MAX;
  for (int i = lane; i < n; i += kWave) mloc = fmaxf(mloc, zs[i]);
  const float M = wave_max_f(mloc);
  const double t = n <= T / 2 ? wave_solve<T / 2 / kWave>(zs, n, M, r, rg)
                              : wave_solve<T / kWave>(zs, n, M, r, rg);
  return static_cast<double>(M) + t;
}

template <int D, int G, int P>
__global__ __launch_bounds__(kSmallThreads) void k_entmax_small(
    const uint16_t *__restrict__ kpool, const uint16_t *__restrict__ vpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, const float *__restrict__ q,
    float zscale, int H, int max_pages, int max_count, int nb, int r, float rg,
    float *__restrict__ out, float *__restrict__ tau_out,
    unsigned *__restrict__ arrivals, float *__restrict__ zws) {
  constexpr int T = kSmallTokens;       // token capacity per unit
  constexpr int KS = D / 32;            // k-steps of the MFMA
  constexpr int NPASS = (G + 3) / 4;    // groups of 4 query heads
  constexpr int RING = 4;               // 16-token groups in flight per wave
  constexpr int MAXP = T / 16;          // pages (P >= 16)
  constexpr int LPT = D / 8, TPW = kWave / LPT;  // value rows: lanes per row
  constexpr int RU = G > 4 ? 8 : 16;    // value rows per lane in flight
  __shared__ __align__(16) float zs[G][T];  // scores, then weights
  __shared__ int s_slot[MAXP], s_nt[MAXP];
  __shared__ int s_rows[T];
  __shared__ float s_acc[kSmallWaves][G][D];
  __shared__ float s_psum[kSmallWaves][G];
  __shared__ float s_tau[G];
  __shared__ int s_tmp[kSmallWaves];
  __shared__ int s_last;
  const int u = blockIdx.x / nb, jb = blockIdx.x - u * nb;
  const int b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int n = lane & 15, kb = lane >> 4;
  // 1. q, the unit's count and its selected page numbers are loaded
  // together (sel speculatively, in bounds), then the page-table rows.
  float4 qraw[NPASS][KS][2];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int g = (n & 3) + 4 * ps;
      const float *qp = q + ((static_cast<size_t>(b) * H + h) * G + (g < G ? g : 0)) * D +
                        32 * s + 8 * kb;
      qraw[ps][s][0] = *reinterpret_cast<const float4 *>(qp);
      qraw[ps][s][1] = *reinterpret_cast<const float4 *>(qp + 4);
    }
  const int len = seq_lens[b];
  const int cnt = sel ? count[u] : n_pages_of(len, P);
  int lp = tid;
  if (sel && tid < min(max_count, max_pages))
    lp = sel[static_cast<size_t>(u) * max_pages + tid];
  if (cnt > max_count || cnt > max_pages || cnt * P > T || cnt < 1) {
    // a selection larger than promised: NaN rows (nothing else is read)
    if (jb == 0) {
      float *orow = out + static_cast<size_t>(u) * G * D;
      for (int e = tid; e < G * D; e += kSmallThreads) orow[e] = NAN;
      if (tau_out && tid < G) tau_out[u * G + tid] = NAN;
    }
    return;
  }
  if (tid < cnt) {  // cnt <= 2048 / 16 < kSmallThreads
    s_slot[tid] = page_table[static_cast<size_t>(b) * max_pages + lp];
    s_nt[tid] = page_tokens(lp, len, P);
  }
  // A of the MFMA: row 4 s + g is the s-th bfloat16 part of zscale q_g
  // (parts 0..2; rows 12..15 and heads past G are zero)
  bf16x8_t a[NPASS][KS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int part = n >> 2, g = (n & 3) + 4 * ps;
      const float qv[8] = {qraw[ps][s][0].x, qraw[ps][s][0].y, qraw[ps][s][0].z,
                           qraw[ps][s][0].w, qraw[ps][s][1].x, qraw[ps][s][1].y,
                           qraw[ps][s][1].z, qraw[ps][s][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[ps][s][i] = static_cast<__bf16>(
            part < 3 && g < G ? bf16_part(qv[i] * zscale, part) : 0.f);
    }
  lds_barrier();
  const int ntok = cnt * P;
  const int ngr = ntok / 16;  // P is a multiple of 16
  const size_t zcap = static_cast<size_t>(max_count) * P;
  float *zrow = zws + static_cast<size_t>(u) * G * zcap;

  // 2. this block's 16-token groups, jb + nb (wave + kSmallWaves k), RING at
  // a time per wave: scores on the matrix cores (q in three bfloat16 parts,
  // as in the key pass) into zs and, with NB > 1, into the workspace
  const int gstride = nb * kSmallWaves;
  for (int g0 = jb + nb * wave; g0 < ngr; g0 += RING * gstride) {
    bf16x8_t kv[RING][KS];
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      // past the last group: reload the wave's first one (in bounds; unused)
      const int gr = g0 + k * gstride < ngr ? g0 + k * gstride : g0;
      const int i = 16 * gr + n, j = i / P, t = i - j * P;
      const uint16_t *row = kpool + pool_row(s_slot[j], h, t, H, P, D) + 8 * kb;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kv[k][s] = *reinterpret_cast<const bf16x8_t *>(row + 32 * s);
    }
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      const int gr = g0 + k * gstride;
      const bool live = gr < ngr;
      const int i = 16 * (live ? gr : g0) + n, j = i / P, t = i - j * P;
      const bool valid = t < s_nt[j];
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ps][s2], kv[k][s2], c, 0, 0, 0);
        // lane n + 16 e takes head 4 ps + e's score of token n (the sum of
        // the three q parts, the same butterfly as the key pass)
        float zmine = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s1 = c[e] + __shfl_xor(c[e], 16, kWave);
          const float z = s1 + __shfl_xor(s1, 32, kWave);
          zmine = kb == e ? z : zmine;
        }
        const int g = 4 * ps + kb;
        const float zv = valid ? zmine : -INFINITY;
        if (live && g < G) {
          zs[g][i] = zv;
          if (nb > 1) zrow[g * zcap + i] = zv;
        }
      }
    }
  }

  if (nb > 1) {
    // Arrival: every wave's score stores complete, then one device-scope
    // release (the fence) and the unit's counter.  The block that brings it
    // to NB takes the unit: an acquire, then the other blocks' scores.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      const unsigned before = atomicAdd(arrivals + u, 1u);
      const int last = before == static_cast<unsigned>(nb - 1);
      if (last) {
        __threadfence();
        arrivals[u] = 0u;  // ready for the next call
      }
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    // every score of the unit, four at a time, all loads in flight at once
    constexpr int ZR = (G * T / 4 + kSmallThreads - 1) / kSmallThreads;
    const int n4 = ntok / 4, nch = G * n4;
    float4 zc[ZR];
#pragma unroll
    for (int k = 0; k < ZR; ++k) {
      const int c = tid + k * kSmallThreads, cc = c < nch ? c : 0;
      const int g = cc / n4, i = 4 * (cc - g * n4);
      zc[k] = *reinterpret_cast<const float4 *>(zrow + g * zcap + i);
    }
#pragma unroll
    for (int k = 0; k < ZR; ++k) {
      const int c = tid + k * kSmallThreads;
      if (c < nch) {
        const int g = c / n4, i = 4 * (c - g * n4);
        *reinterpret_cast<float4 *>(&zs[g][i]) = zc[k];
      }
    }
  }
  lds_barrier();

  // 3. one wave per head solves its threshold from its scores in LDS.  The
  // other waves meanwhile load one word of every 128-byte line of the unit's
  // value rows (all in flight together, the words folded into `touch` and
  // consumed at the end), so that the value sum after the solve finds its
  // rows in the L2 instead of a memory round trip away.
  uint32_t touch = 0u;
  if (wave < G) {
    const double tau = head_threshold<T>(zs[wave], ntok, r, rg);
    if (lane == 0) s_tau[wave] = static_cast<float>(tau);
  } else if constexpr (G < kSmallWaves) {
    constexpr int LPR = D * 2 / 128;                    // lines per value row
    constexpr int IDLE = (kSmallWaves - G) * kWave;     // lanes touching
    constexpr int TU = (T * LPR + IDLE - 1) / IDLE;     // loads per lane
    const int nl = ntok * LPR, me = tid - G * kWave;
    uint32_t w[TU];
#pragma unroll
    for (int k = 0; k < TU; ++k) {
      const int e = min(me + k * IDLE, nl - 1);
      const int i = e / LPR, j = i / P, t = i - j * P;
      w[k] = *reinterpret_cast<const uint32_t *>(
          vpool + pool_row(s_slot[j], h, t, H, P, D) + (e - i * LPR) * 64);
    }
#pragma unroll
    for (int k = 0; k < TU; ++k) touch ^= w[k];
  }
  lds_barrier();

  // 4. weights p = max(z - tau, 0)^r in place, their sums, and the ordered
  // list of tokens some head gives weight
  float ps_loc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) ps_loc[g] = 0.f;
  int n_rows = 0;
  for (int base = 0; base < ntok; base += kSmallThreads) {
    const int i = base + tid;
    bool any = false;
    if (i < ntok) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = pow_r(fmaxf(zs[g][i] - s_tau[g], 0.f), r, rg);
        zs[g][i] = p;
        ps_loc[g] += p;
        any |= p > 0.f;
      }
    }
    int tot;
    const int rk = tile_rank<kSmallThreads>(any, s_tmp, tot);
    if (any) s_rows[n_rows + rk] = i;
    n_rows += tot;
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float sg = wave_sum_f(ps_loc[g]);
    if (lane == 0) s_psum[wave][g] = sg;
  }
  lds_barrier();

  // 5. value rows of the union of the supports, LPT lanes per row, RU rows
  // per lane in flight (kept as bfloat16 until used), summed for every head
  // in a fixed order
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  constexpr int STEP = kSmallWaves * TPW * RU;
  n_rows = __builtin_amdgcn_readfirstlane(n_rows);  // block-uniform
  for (int base = 0; base < n_rows; base += STEP) {
    // lanes past the list reload the first listed row (cached) and add
    // nothing: no load is behind a branch
    uint4 x[RU];
    int ri[RU];
    // slot k holds rows [base + 32 k, base + 32 k + 32) of the list across
    // the block: slots past the list are skipped by every wave
#pragma unroll
    for (int k = 0; k < RU; ++k) {
      if (base + k * kSmallWaves * TPW >= n_rows) break;
      const int e = base + (k * kSmallWaves + wave) * TPW + sub;
      ri[k] = s_rows[e < n_rows ? e : 0];
      ri[k] = e < n_rows ? ri[k] : -1;
      const int i = ri[k] >= 0 ? ri[k] : s_rows[0];
      const int j = i / P, t = i - j * P;
      x[k] = *reinterpret_cast<const uint4 *>(
          vpool + pool_row(s_slot[j], h, t, H, P, D) + d0);
    }
#pragma unroll
    for (int k = 0; k < RU; ++k) {
      if (base + k * kSmallWaves * TPW >= n_rows) break;
      const float xv[8] = {bf16_lo(x[k].x), bf16_hi(x[k].x), bf16_lo(x[k].y),
                           bf16_hi(x[k].y), bf16_lo(x[k].z), bf16_hi(x[k].z),
                           bf16_lo(x[k].w), bf16_hi(x[k].w)};
      const int i = ri[k] >= 0 ? ri[k] : 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = ri[k] >= 0 ? zs[g][i] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p, xv[e], acc[g][e]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[g][e];
#pragma unroll
      for (int o = LPT; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
      acc[g][e] = v;
    }
  if (sub == 0)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][g][d0 + e] = acc[g][e];
  lds_barrier();
  float *orow = out + static_cast<size_t>(u) * G * D;
  for (int e = tid; e < G * D; e += kSmallThreads) {
    const int g = e / D, d = e - g * D;
    float v = 0.f, ps = 0.f;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
      v += s_acc[w][g][d];
      ps += s_psum[w][g];
    }
    orow[e] = v / ps;
  }
  if (tau_out && tid < G) tau_out[u * G + tid] = s_tau[tid];
  if (touch == 0x9e3779b9u) s_last = 2;  // keeps the touching loads (never read)
}

// Blocks per unit: enough that the grid covers the device, at most one
// 16-token group per wave.
static int small_blocks_per_unit(int units, int max_count, int P) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess || n_cu <= 0)
    n_cu = 256;
  const int groups = max_count * P / 16;
  const int full = (groups + kSmallWaves - 1) / kSmallWaves;
  const int fill = (n_cu + units - 1) / units;
  return std::max(1, std::min(full, fill));
}

size_t small_ws_bytes(const ekv_paged_kv &kv, int max_count) {
  const size_t units = static_cast<size_t>(kv.batch) * kv.num_kv_heads;
  const size_t ctr = (units * 4 + 255) & ~static_cast<size_t>(255);
  const size_t z = units * kv.group * static_cast<size_t>(max_count) * kv.page_size * 4;
  return ctr + ((z + 255) & ~static_cast<size_t>(255));
}

template <int D, int G>
hipError_t launch_entmax_small(const ekv_paged_kv &kv, const float *q,
                               float scale, float alpha, const int32_t *sel,
                               const int32_t *count, int max_count, float *out,
                               float *tau, void *ws, hipStream_t stream) {
  const float rg = 1.0f / (alpha - 1.0f);
  const int r = alpha == 2.0f ? 1 : alpha == 1.5f ? 2 : 0;
  const int units = kv.batch * kv.num_kv_heads;
  const int nb = small_blocks_per_unit(units, max_count, kv.page_size);
  const size_t units_sz = static_cast<size_t>(units);
  unsigned *arrivals = static_cast<unsigned *>(ws);
  float *zws = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                         ((units_sz * 4 + 255) & ~static_cast<size_t>(255)));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(units * nb), dim3(kSmallThreads), 0, stream,
                       static_cast<const uint16_t *>(kv.k),
                       static_cast<const uint16_t *>(kv.v), kv.page_table,
                       kv.seq_lens, sel, count, q, (alpha - 1.0f) * scale,
                       kv.num_kv_heads, kv.max_pages, max_count, nb, r, rg, out,
                       tau, arrivals, zws);
  };
  switch (kv.page_size) {
    case 16: go(k_entmax_small<D, G, 16>); break;
    case 32: go(k_entmax_small<D, G, 32>); break;
    default: go(k_entmax_small<D, G, 64>); break;
  }
  return hipGetLastError();
}

#define EKV_INST_SMALL(D, G)                                                  \
  template hipError_t launch_entmax_small<D, G>(                              \
      const ekv_paged_kv &, const float *, float, float, const int32_t *,     \
      const int32_t *, int, float *, float *, void *, hipStream_t);
EKV_INST_SMALL(64, 1) EKV_INST_SMALL(64, 2) EKV_INST_SMALL(64, 4) EKV_INST_SMALL(64, 8)
EKV_INST_SMALL(128, 1) EKV_INST_SMALL(128, 2) EKV_INST_SMALL(128, 4) EKV_INST_SMALL(128, 8)

}  // namespace ekv
