// Page metadata and query-aware page scoring
// (Technical Summary: EntmaxKV, §2.A "Query-Aware Page Scoring").
//
// Both kernels stream one small record per (page, KV head): the metadata
// build reads a page's keys once (twice for the variance, the second time
// from cache) and writes 2*D box values and 2*D float32 moments; scoring
// reads those records back and writes G floats (box) or G float pairs
// (Gaussian) per record.  Both are HBM-bound.
#include <float.h>

#include <algorithm>

#include "ekv_device.h"
#include "ekv_kernels.h"

namespace ekv {

// ---------------------------------------------------------------------------
// Metadata build: one block per (sequence, logical page, KV head).  Thread
// (tg, cg) loads coordinates 8cg..8cg+7 of tokens tg, tg+TG, ... (16-byte
// loads, the whole page in flight at once) and keeps partial minima, maxima
// and sums; the TG partials of each coordinate are combined in a fixed
// order, so every page's result is a fixed function of its keys and an
// incremental refresh equals a full build bit for bit.  The variance is
// taken about the mean in a second pass over the registers.
// ---------------------------------------------------------------------------
constexpr int kMetaThreads = 256;

template <class E, int D>
__global__ __launch_bounds__(kMetaThreads) void k_build_meta(
    const typename E::T *__restrict__ kpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ first_page, int H, int P, int max_pages,
    typename E::T *__restrict__ bbox, float *__restrict__ gauss) {
  constexpr int CG = D / 8;                 // coordinate groups
  constexpr int TG = kMetaThreads / CG;     // token groups
  constexpr int MAXT = (64 + TG - 1) / TG;  // tokens per thread (P <= 64)
  __shared__ float s_a[TG][D];
  __shared__ float s_b[TG][D];
  __shared__ float s_c[TG][D];
  __shared__ float s_mean[D];
  const int b = blockIdx.z, h = blockIdx.y;
  const int cg = threadIdx.x % CG, tg = threadIdx.x / CG, d0 = cg * 8;
  const int len = seq_lens[b];
  const int np = n_pages_of(len, P);
  int p0 = first_page ? first_page[b] : 0;
  if (p0 < 0) p0 = 0;
  for (int lp = p0 + blockIdx.x; lp < np; lp += gridDim.x) {
    const int slot = page_table[static_cast<size_t>(b) * max_pages + lp];
    const int n = page_tokens(lp, len, P);
    const typename E::T *base = kpool + pool_row(slot, h, 0, H, P, D);
    float x[MAXT][8];
#pragma unroll
    for (int i = 0; i < MAXT; ++i) {
      const int t = tg + i * TG;
      if (t < n) load8(base + static_cast<size_t>(t) * D + d0, x[i]);
    }
    float mn[8], mx[8], sm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { mn[j] = INFINITY; mx[j] = -INFINITY; sm[j] = 0.f; }
#pragma unroll
    for (int i = 0; i < MAXT; ++i)
      if (tg + i * TG < n)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          mn[j] = fminf(mn[j], x[i][j]);
          mx[j] = fmaxf(mx[j], x[i][j]);
          sm[j] += x[i][j];
        }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s_a[tg][d0 + j] = mn[j];
      s_b[tg][d0 + j] = mx[j];
      s_c[tg][d0 + j] = sm[j];
    }
    lds_barrier();
    if (threadIdx.x < D) {
      const int d = threadIdx.x;
      float a = s_a[0][d], c = s_b[0][d], s = s_c[0][d];
      for (int k = 1; k < TG; ++k) {
        a = fminf(a, s_a[k][d]);
        c = fmaxf(c, s_b[k][d]);
        s += s_c[k][d];
      }
      const float mean = s / static_cast<float>(n);
      s_mean[d] = mean;
      if (bbox) {
        store1(bbox + meta_row(slot, h, 0, H, D) + d, a);
        store1(bbox + meta_row(slot, h, 1, H, D) + d, c);
      }
      if (gauss) gauss[meta_row(slot, h, 0, H, D) + d] = mean;
    }
    lds_barrier();
    if (gauss) {
      float ss[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ss[j] = 0.f;
#pragma unroll
      for (int i = 0; i < MAXT; ++i)
        if (tg + i * TG < n)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float dv = x[i][j] - s_mean[d0 + j];
            ss[j] = fmaf(dv, dv, ss[j]);
          }
#pragma unroll
      for (int j = 0; j < 8; ++j) s_c[tg][d0 + j] = ss[j];
      lds_barrier();
      if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float s = s_c[0][d];
        for (int k = 1; k < TG; ++k) s += s_c[k][d];
        gauss[meta_row(slot, h, 1, H, D) + d] = s / static_cast<float>(n);
      }
    }
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// Page scoring.  Besides the per-page values the kernel writes, for every
// 64-page tile (one block), summaries the selectors use to skip tiles:
//   box:       max over the tile's pages and the group's heads of the bound;
//   Gaussian:  per query head max mu, max (mu + 8.5 sigma) and
//              max (mu + sqrt(2 ln P) sigma).
// They live after the per-page values in the same buffers (see entmaxkv.h).
//
// Page scoring: D/8 lanes per page (8 coordinates per lane, 16-byte loads of
// bf16 box values), 64*8/D pages per wave step.  The box bound uses
// max(q kmin, q kmax) = q+ kmax + q- kmin per coordinate (q+ = max(q, 0),
// q- = min(q, 0)): the same rounded product is picked either way.
// ---------------------------------------------------------------------------
constexpr int kScoreTile = kPageTile;  // pages per block

template <class E, int D, int G, int MODE>
__global__ __launch_bounds__(256) void k_score(
    const typename E::T *__restrict__ bbox, const float *__restrict__ gauss,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const float *__restrict__ q,
    float scale, int H, int P, int max_pages, int batch,
    float *__restrict__ ub, float *__restrict__ gstat) {
  constexpr int LPP = D / 8;          // lanes per page
  constexpr int PPW = kWave / LPP;    // pages per wave step
  constexpr int NWAVE = 4;
  constexpr int NSTEP = kScoreTile / (NWAVE * PPW);
  static_assert(kScoreTile % (NWAVE * PPW) == 0, "tile must fill the waves");
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPP, li = lane % LPP;
  const int Hq = H * G;
  const int n_tiles = (max_pages + kScoreTile - 1) / kScoreTile;
  const int n_items = batch * H * n_tiles;
  __shared__ float s_tile[4][3 * G + 1];

  // Persistent blocks over (sequence, KV head, tile) items.  The page-table
  // entries of a block's next item are read while the current item is
  // scored, so only the first item waits on them before its metadata loads.
  auto page_of = [&](int tile, int k) {
    return tile * kScoreTile + (k * NWAVE + wave) * PPW + sub;
  };
  auto fetch_slots = [&](int item, int (&raw)[NSTEP]) {
    const int b = item / (H * n_tiles);
    const int tile = item % n_tiles;
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      const int lp = page_of(tile, k);
      // entries past the sequence end are in bounds (and unused)
      raw[k] = lp < max_pages ? page_table[static_cast<size_t>(b) * max_pages + lp] : 0;
    }
  };
  int slot_raw[NSTEP];
  int item = blockIdx.x;
  if (item < n_items) fetch_slots(item, slot_raw);
  for (; item < n_items; item += gridDim.x) {
    int slot_next[NSTEP];
    const int nxt = item + gridDim.x;
    if (nxt < n_items) fetch_slots(nxt, slot_next);
    const int b = item / (H * n_tiles);
    const int h = (item / n_tiles) % H;
    const int tile = item % n_tiles;
    const int tile0 = tile * kScoreTile;
    const int len = seq_lens[b];
    const int np = n_pages_of(len, P);
    if (tile0 < np) {

  // scale * q at the coordinates this lane owns in a box row (qb) and in a
  // Gaussian row (qs, float32); see coord_of.
  float qs[G][8], qb[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float *qg = q + (static_cast<size_t>(b) * Hq + h * G + g) * D;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr ((MODE & EKV_SCORE_GAUSS) != 0)
        qs[g][j] = qg[coord_of<float, D>(li, j)] * scale;
      if constexpr ((MODE & EKV_SCORE_BBOX) != 0)
        qb[g][j] = qg[coord_of<typename E::T, D>(li, j)] * scale;
    }
  }

  int lps[NSTEP], slots[NSTEP];
  bool valid[NSTEP];
#pragma unroll
  for (int k = 0; k < NSTEP; ++k) {
    lps[k] = page_of(tile, k);
    valid[k] = lps[k] < np;
    slots[k] = valid[k] ? slot_raw[k] : 0;
  }
  if constexpr ((MODE & EKV_SCORE_BBOX) != 0) {
    float tmax = -FLT_MAX;
    float kmin[NSTEP][8], kmax[NSTEP][8];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      if (valid[k]) {
        load8_lane<D>(bbox + meta_row(slots[k], h, 0, H, D), li, kmin[k]);
        load8_lane<D>(bbox + meta_row(slots[k], h, 1, H, D), li, kmax[k]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { kmin[k][j] = 0.f; kmax[k][j] = 0.f; }
      }
    }
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      float acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          a = fmaf(fmaxf(qb[g][j], 0.f), kmax[k][j], a);
          a = fmaf(fminf(qb[g][j], 0.f), kmin[k][j], a);
        }
        acc[g] = group_sum<LPP>(a);
      }
      if (valid[k]) {
        float gm = acc[0];
#pragma unroll
        for (int g = 1; g < G; ++g) gm = fmaxf(gm, acc[g]);
        tmax = fmaxf(tmax, gm);
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (li == g)
            ub[(static_cast<size_t>(b) * Hq + h * G + g) * max_pages + lps[k]] = acc[g];
      }
    }
    tmax = group_max<kWave>(tmax);
    if (lane == 0) s_tile[wave][3 * G] = tmax;
    lds_barrier();
    if (threadIdx.x == 0) {
      float m = s_tile[0][3 * G];
      for (int w = 1; w < NWAVE; ++w) m = fmaxf(m, s_tile[w][3 * G]);
      ub[static_cast<size_t>(batch) * Hq * max_pages +
         (static_cast<size_t>(b) * H + h) * n_tiles + tile] = m;
    }
  }
  if constexpr ((MODE & EKV_SCORE_GAUSS) != 0) {
    const float cP = sqrtf(2.0f * logf(static_cast<float>(P)));
    float t_mu[G], t_pr[G], t_kp[G];
#pragma unroll
    for (int g = 0; g < G; ++g) { t_mu[g] = -FLT_MAX; t_pr[g] = -FLT_MAX; t_kp[g] = -FLT_MAX; }
    float mean[NSTEP][8], var[NSTEP][8];
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      if (valid[k]) {
        load8_lane<D>(gauss + meta_row(slots[k], h, 0, H, D), li, mean[k]);
        load8_lane<D>(gauss + meta_row(slots[k], h, 1, H, D), li, var[k]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { mean[k][j] = 0.f; var[k][j] = 0.f; }
      }
    }
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      float mu[G], s2[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = qs[g][j];
          a = fmaf(x, mean[k][j], a);
          c = fmaf(x * x, var[k][j], c);
        }
        mu[g] = group_sum<LPP>(a);
        s2[g] = group_sum<LPP>(c);
      }
      if (valid[k]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float sd = sqrtf(fmaxf(s2[g], 0.f));
          t_mu[g] = fmaxf(t_mu[g], mu[g]);
          t_pr[g] = fmaxf(t_pr[g], mu[g] + 8.5f * sd);
          t_kp[g] = fmaxf(t_kp[g], mu[g] + cP * sd);
          if (li == g) {
            float2 rr;
            rr.x = mu[g];
            rr.y = s2[g];
            reinterpret_cast<float2 *>(gstat)[(static_cast<size_t>(b) * Hq + h * G + g) * max_pages + lps[k]] = rr;
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float a0 = group_max<kWave>(t_mu[g]);
      const float a1 = group_max<kWave>(t_pr[g]);
      const float a2 = group_max<kWave>(t_kp[g]);
      if (lane == 0) {
        s_tile[wave][3 * g] = a0;
        s_tile[wave][3 * g + 1] = a1;
        s_tile[wave][3 * g + 2] = a2;
      }
    }
    lds_barrier();
    if (threadIdx.x < G) {
      const int g = threadIdx.x;
      float4 r4;
      r4.x = s_tile[0][3 * g];
      r4.y = s_tile[0][3 * g + 1];
      r4.z = s_tile[0][3 * g + 2];
      r4.w = 0.f;
      for (int w = 1; w < NWAVE; ++w) {
        r4.x = fmaxf(r4.x, s_tile[w][3 * g]);
        r4.y = fmaxf(r4.y, s_tile[w][3 * g + 1]);
        r4.z = fmaxf(r4.z, s_tile[w][3 * g + 2]);
      }
      float4 *gt = reinterpret_cast<float4 *>(
          gstat + gstat_tile_offset(batch, Hq, max_pages));
      gt[(static_cast<size_t>(b) * Hq + h * G + g) * n_tiles + tile] = r4;
    }
  }
    }
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) slot_raw[k] = slot_next[k];
    lds_barrier();  // s_tile is rewritten by the next item
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <class E, int D>
hipError_t launch_build_meta(const ekv_paged_kv &kv, const int32_t *first_page,
                             int span, const ekv_meta &meta,
                             hipStream_t stream) {
  const int pages = span > 0 && span < kv.max_pages ? span : kv.max_pages;
  dim3 grid(pages, kv.num_kv_heads, kv.batch);
  hipLaunchKernelGGL((k_build_meta<E, D>), grid, dim3(kMetaThreads), 0, stream,
                     static_cast<const typename E::T *>(kv.k), kv.page_table,
                     kv.seq_lens, first_page, kv.num_kv_heads, kv.page_size,
                     kv.max_pages, static_cast<typename E::T *>(meta.bbox),
                     meta.gauss);
  return hipGetLastError();
}

template <class E, int D, int G>
hipError_t launch_score(const ekv_paged_kv &kv, const ekv_meta &meta,
                        const float *q, float scale, int mode, float *ub,
                        float *gstat, hipStream_t stream) {
  const int items = ((kv.max_pages + kScoreTile - 1) / kScoreTile) *
                    kv.num_kv_heads * kv.batch;
  auto launch = [&](auto kern) {
    int dev = 0, n_cu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess || n_cu <= 0)
      n_cu = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(kern), 256, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    const int blocks = std::min(items, n_cu * per_cu);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const typename E::T *>(meta.bbox),
                       meta.gauss, kv.page_table, kv.seq_lens, q, scale,
                       kv.num_kv_heads, kv.page_size, kv.max_pages, kv.batch,
                       ub, gstat);
  };
  constexpr int kBoth = EKV_SCORE_BBOX | EKV_SCORE_GAUSS;
  if (mode == EKV_SCORE_BBOX) launch(k_score<E, D, G, EKV_SCORE_BBOX>);
  else if (mode == EKV_SCORE_GAUSS) launch(k_score<E, D, G, EKV_SCORE_GAUSS>);
  else launch(k_score<E, D, G, kBoth>);
  return hipGetLastError();
}

#define EKV_INST_META(E, D)                                                 \
  template hipError_t launch_build_meta<E, D>(const ekv_paged_kv &,         \
                                              const int32_t *, int,         \
                                              const ekv_meta &, hipStream_t);
#define EKV_INST_SCORE(E, D, G)                                             \
  template hipError_t launch_score<E, D, G>(                                \
      const ekv_paged_kv &, const ekv_meta &, const float *, float, int,    \
      float *, float *, hipStream_t);

EKV_FOR_EACH_ED(EKV_INST_META)
EKV_FOR_EACH_EDG(EKV_INST_SCORE)

}  // namespace ekv
