// Page metadata and query-aware page scoring
// (Technical Summary: EntmaxKV, §2.A "Query-Aware Page Scoring").
//
// Both kernels stream one small record per (page, KV head): the metadata
// build reads a page's keys once (twice for the variance, the second time
// from cache) and writes 2*D box values and 2*D float32 moments; scoring
// reads those records back and writes G floats (box) or G float pairs
// (Gaussian) per record.  Both are HBM-bound.
#include "ekv_device.h"
#include "ekv_kernels.h"

namespace ekv {

// ---------------------------------------------------------------------------
// Metadata build: one wave per (sequence, logical page, KV head).  Lanes own
// D/64 coordinates; tokens are walked in order so every page's result is a
// fixed function of its keys (an incremental refresh equals a full build).
// ---------------------------------------------------------------------------
template <class E, int D>
__global__ __launch_bounds__(256) void k_build_meta(
    const typename E::T *__restrict__ kpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ first_page, int H, int P, int max_pages,
    typename E::T *__restrict__ bbox, float *__restrict__ gauss) {
  constexpr int CPL = D / kWave;  // coordinates per lane
  const int b = blockIdx.z, h = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int len = seq_lens[b];
  const int np = n_pages_of(len, P);
  int p0 = first_page ? first_page[b] : 0;
  if (p0 < 0) p0 = 0;
  constexpr int kWavesPerBlock = 4;
  for (int lp = p0 + blockIdx.x * kWavesPerBlock + wave; lp < np;
       lp += gridDim.x * kWavesPerBlock) {
    const int slot = page_table[b * max_pages + lp];
    const int n = page_tokens(lp, len, P);
    const typename E::T *base = kpool + pool_row(slot, h, 0, H, P, D);
    float mn[CPL], mx[CPL], sm[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float x = load1(base + lane * CPL + c);
      mn[c] = x; mx[c] = x; sm[c] = x;
    }
    for (int t = 1; t < n; ++t) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float x = load1(base + static_cast<size_t>(t) * D + lane * CPL + c);
        mn[c] = fminf(mn[c], x);
        mx[c] = fmaxf(mx[c], x);
        sm[c] += x;
      }
    }
    if (bbox) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        store1(bbox + meta_row(slot, h, 0, H, D) + lane * CPL + c, mn[c]);
        store1(bbox + meta_row(slot, h, 1, H, D) + lane * CPL + c, mx[c]);
      }
    }
    if (gauss) {
      float mean[CPL], ss[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        mean[c] = sm[c] / static_cast<float>(n);
        ss[c] = 0.f;
      }
      for (int t = 0; t < n; ++t) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float x = load1(base + static_cast<size_t>(t) * D + lane * CPL + c);
          const float dv = x - mean[c];
          ss[c] = fmaf(dv, dv, ss[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        gauss[meta_row(slot, h, 0, H, D) + lane * CPL + c] = mean[c];
        gauss[meta_row(slot, h, 1, H, D) + lane * CPL + c] =
            ss[c] / static_cast<float>(n);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Page scoring: D/8 lanes per page (8 coordinates per lane, 16-byte loads of
// bf16 box values), 64*8/D pages per wave step.  The box bound uses
// max(q kmin, q kmax) = q+ kmax + q- kmin per coordinate (q+ = max(q, 0),
// q- = min(q, 0)): the same rounded product is picked either way.
// ---------------------------------------------------------------------------
constexpr int kScoreTile = 64;  // pages per block

template <class E, int D, int G>
__global__ __launch_bounds__(256) void k_score(
    const typename E::T *__restrict__ bbox, const float *__restrict__ gauss,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const float *__restrict__ q,
    float scale, int mode, int H, int P, int max_pages,
    float *__restrict__ ub, float *__restrict__ gstat) {
  constexpr int LPP = D / 8;          // lanes per page
  constexpr int PPW = kWave / LPP;    // pages per wave step
  constexpr int NWAVE = 4;
  static_assert(kScoreTile % (NWAVE * PPW) == 0, "tile must fill the waves");
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPP, li = lane % LPP, d0 = li * 8;
  const int len = seq_lens[b];
  const int np = n_pages_of(len, P);
  const int tile0 = blockIdx.x * kScoreTile;
  if (tile0 >= np) return;
  const int Hq = H * G;

  float qp[G][8], qn[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float *qg = q + (static_cast<size_t>(b) * Hq + h * G + g) * D + d0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qg[j] * scale;
      qp[g][j] = fmaxf(x, 0.f);
      qn[g][j] = fminf(x, 0.f);
    }
  }

  for (int i = wave * PPW + sub; i < kScoreTile; i += NWAVE * PPW) {
    const int lp = tile0 + i;
    const bool valid = lp < np;
    const int slot = valid ? page_table[b * max_pages + lp] : 0;
    if (mode & EKV_SCORE_BBOX) {
      float kmin[8], kmax[8];
      if (valid) {
        load8(bbox + meta_row(slot, h, 0, H, D) + d0, kmin);
        load8(bbox + meta_row(slot, h, 1, H, D) + d0, kmax);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { kmin[j] = 0.f; kmax[j] = 0.f; }
      }
      float acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          a = fmaf(qp[g][j], kmax[j], a);
          a = fmaf(qn[g][j], kmin[j], a);
        }
        acc[g] = group_sum<LPP>(a);
      }
      if (valid) {
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (li == g)
            ub[(static_cast<size_t>(b) * Hq + h * G + g) * max_pages + lp] = acc[g];
      }
    }
    if (mode & EKV_SCORE_GAUSS) {
      float mean[8], var[8];
      if (valid) {
        load8(gauss + meta_row(slot, h, 0, H, D) + d0, mean);
        load8(gauss + meta_row(slot, h, 1, H, D) + d0, var);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { mean[j] = 0.f; var[j] = 0.f; }
      }
      float mu[G], s2[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = qp[g][j] + qn[g][j];
          a = fmaf(x, mean[j], a);
          c = fmaf(x * x, var[j], c);
        }
        mu[g] = group_sum<LPP>(a);
        s2[g] = group_sum<LPP>(c);
      }
      if (valid) {
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (li == g) {
            float2 r;
            r.x = mu[g];
            r.y = s2[g];
            reinterpret_cast<float2 *>(gstat)[(static_cast<size_t>(b) * Hq + h * G + g) * max_pages + lp] = r;
          }
      }
    }
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
  dim3 grid((pages + 3) / 4, kv.num_kv_heads, kv.batch);
  hipLaunchKernelGGL((k_build_meta<E, D>), grid, dim3(256), 0, stream,
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
  dim3 grid((kv.max_pages + kScoreTile - 1) / kScoreTile, kv.num_kv_heads,
            kv.batch);
  hipLaunchKernelGGL((k_score<E, D, G>), grid, dim3(256), 0, stream,
                     static_cast<const typename E::T *>(meta.bbox), meta.gauss,
                     kv.page_table, kv.seq_lens, q, scale, mode,
                     kv.num_kv_heads, kv.page_size, kv.max_pages, ub, gstat);
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
