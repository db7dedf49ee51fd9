// Sparse alpha-entmax attention over gathered pages, and the split-K softmax
// baseline (Technical Summary: EntmaxKV, §2.C "Sparse Entmax Attention" and
// §4 "Efficiency").
//
// Entmax has no single-pass running form: the threshold tau depends on every
// score.  The step is therefore split in three launches over "chunks" of
// kChunkTokens token positions of a unit's selected pages:
//   1. scores:    gather K, z = (alpha-1) scale <q, k> for the G query heads,
//                 write z (float32) and each chunk's maximum;
//   2. threshold: per query head, tau from the z of the chunks whose maximum
//                 exceeds max z - 1 (tau >= max z - 1, so no other token can
//                 have p > 0); exact for alpha in {1.5, 2};
//   3. apply:     p = max(z - tau, 0)^r; V rows are read only where some head
//                 has p > 0 (exact: the other rows carry zero weight), chunk
//                 partials are merged in chunk order.
// Reads: selected K once, V only on the support, z twice (from cache).
#include <float.h>

#include "ekv_device.h"
#include "ekv_kernels.h"

namespace ekv {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kMaxChunkPages = kChunkTokens / 16;  // smallest page size

DecodeWs decode_ws_layout(const ekv_paged_kv &kv) {
  const size_t units = static_cast<size_t>(kv.batch) * kv.num_kv_heads;
  const size_t G = kv.group, D = kv.head_dim;
  const size_t cap = static_cast<size_t>(kv.max_pages) * kv.page_size;
  const size_t mc = max_chunks(kv);
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  DecodeWs w;
  w.z = 0;
  w.cmax = al(w.z + units * G * cap * 4);
  w.tau = al(w.cmax + units * G * mc * 4);
  w.part_o = al(w.tau + units * G * 4);
  w.part_s = al(w.part_o + units * mc * G * D * 4);
  w.total = al(w.part_s + units * mc * G * 4);
  return w;
}

SoftmaxWs softmax_ws_layout(const ekv_paged_kv &kv) {
  const size_t units = static_cast<size_t>(kv.batch) * kv.num_kv_heads;
  const size_t G = kv.group, D = kv.head_dim;
  const size_t mc = max_chunks(kv);
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  SoftmaxWs w;
  w.part_m = 0;
  w.part_l = al(units * mc * G * 4);
  w.part_o = al(w.part_l + units * mc * G * 4);
  w.total = al(w.part_o + units * mc * G * D * 4);
  return w;
}

// Pages of one chunk, staged in LDS: logical page, slot, valid tokens.
struct ChunkPages {
  int lp[kMaxChunkPages];
  int slot[kMaxChunkPages];
  int nt[kMaxChunkPages];
};

// Returns false (uniformly for the block) when chunk c is past the unit's
// selection.  Otherwise fills `cp` and sets j0/j1 (selection entries).
__device__ __forceinline__ bool stage_chunk(
    ChunkPages &cp, const int32_t *page_table, const int32_t *seq_lens,
    const int32_t *sel, const int32_t *count, int u, int H, int P,
    int max_pages, int c, int &j0, int &j1, int &len) {
  const int b = u / H;
  len = seq_lens[b];
  const int cnt = sel ? count[u] : n_pages_of(len, P);
  const int ppc = kChunkTokens / P;
  j0 = c * ppc;
  if (j0 >= cnt) return false;
  j1 = min(cnt, j0 + ppc);
  if (threadIdx.x < j1 - j0) {
    const int j = j0 + threadIdx.x;
    const int lp = sel ? sel[static_cast<size_t>(u) * max_pages + j] : j;
    cp.lp[threadIdx.x] = lp;
    cp.slot[threadIdx.x] = page_table[static_cast<size_t>(b) * max_pages + lp];
    cp.nt[threadIdx.x] = page_tokens(lp, len, P);
  }
  __syncthreads();
  return true;
}

__device__ __forceinline__ float pow_r(float x, int r, float rg) {
  // x >= 0.  r = 1 (alpha = 2), r = 2 (alpha = 1.5), else x^rg.
  if (r == 1) return x;
  if (r == 2) return x * x;
  return x > 0.f ? powf(x, rg) : 0.f;
}

// ---------------------------------------------------------------------------
// 1. Scores.  D/8 lanes per token (16-byte K loads), U tokens per lane in
// flight per step.
// ---------------------------------------------------------------------------
constexpr int kUnroll = 4;

template <class E, int D, int G>
__global__ __launch_bounds__(kDecThreads) void k_entmax_scores(
    const typename E::T *__restrict__ kpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, const float *__restrict__ q,
    float zscale, int H, int P, int max_pages, int cap, int maxch,
    float *__restrict__ zbuf, float *__restrict__ cmax) {
  constexpr int LPT = D / 8;
  constexpr int TPW = kWave / LPT;
  constexpr int STEP = kDecWaves * TPW * kUnroll;  // tokens per block step
  static_assert(kChunkTokens % STEP == 0, "chunk must be whole steps");
  __shared__ ChunkPages cp;
  __shared__ float red[kDecWaves][G];
  const int u = blockIdx.y, c = blockIdx.x;
  const int h = u % H, b = u / H;
  int j0, j1, len;
  if (!stage_chunk(cp, page_table, seq_lens, sel, count, u, H, P, max_pages,
                   c, j0, j1, len))
    return;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  const int Hq = H * G;

  float qs[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float *qg = q + (static_cast<size_t>(b) * Hq + h * G + g) * D + d0;
#pragma unroll
    for (int j = 0; j < 8; ++j) qs[g][j] = qg[j] * zscale;
  }
  float mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = -FLT_MAX;
  const int npos = (j1 - j0) * P;
  float *zu = zbuf + static_cast<size_t>(u) * G * cap;

  for (int base = 0; base < kChunkTokens; base += STEP) {
    float x[kUnroll][8];
    bool valid[kUnroll];
    int pos[kUnroll];
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
      const int i = base + (r * kDecWaves + wave) * TPW + sub;
      const int jj = i / P, t = i - jj * P;
      pos[r] = i;
      valid[r] = i < npos && t < cp.nt[jj < kMaxChunkPages ? jj : 0];
      if (valid[r]) {
        load8(kpool + pool_row(cp.slot[jj], h, t, H, P, D) + d0, x[r]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[r][j] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
      float acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaf(qs[g][j], x[r][j], a);
        acc[g] = group_sum<LPT>(a);
      }
      if (pos[r] < npos) {
        const size_t zi = static_cast<size_t>(j0) * P + pos[r];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float z = valid[r] ? acc[g] : -INFINITY;
          if (li == g) zu[static_cast<size_t>(g) * cap + zi] = z;
          if (valid[r]) mx[g] = fmaxf(mx[g], acc[g]);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float m = group_max<kWave>(mx[g]);
    if (lane == 0) red[wave][g] = m;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float m = red[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) m = fmaxf(m, red[w][threadIdx.x]);
    cmax[(static_cast<size_t>(u) * G + threadIdx.x) * maxch + c] = m;
  }
}

// ---------------------------------------------------------------------------
// 2. Threshold.  One block per query head.
//
// With M = max z and L = M - 1, tau lies in [L, M).  The candidates z > L are
// counted into kTauBins equal bins of [L, M].  For the bin edge e_b, token
// values z in bin c >= b satisfy (c-b)/NB <= z - e_b < (c+1-b)/NB, so
//   F_lo(b) = sum_{c>=b} cnt_c ((c-b)/NB)^r  <=  F(e_b)  <=  F_hi(b) = ...(c+1-b)
// with F(t) = sum_i max(z_i - t, 0)^r; for r in {1, 2} both are polynomials in
// b of suffix sums of cnt_c c^k, exact in double.  The largest b with
// F_lo >= 1 and the smallest with F_hi < 1 bracket tau.  Tokens above the
// bracket are certainly in the support (only their count and sums of
// (z-M), (z-M)^2 matter); the few inside it are listed and the support size
// is resolved exactly: for a support of the K largest values, tau has a
// closed form (sparsemax: (sum z - 1)/K; 1.5-entmax: the smaller root of
// sum (z - tau)^2 = 1), and the right K is the one whose tau separates the
// K-th and (K+1)-th values.  Sums are kept in 2^-40 fixed point so that the
// result does not depend on the order the block visits the tokens.
// General alpha, or a bracket holding too many tokens, falls back to
// bisection in double over the candidates.
// ---------------------------------------------------------------------------
constexpr int kTauThreads = 256;
constexpr int kTauBins = 2048;
constexpr int kTauList = 1024;
constexpr int kTauChunkCap = 4096;
constexpr double kFix = 1099511627776.0;  // 2^40

__device__ __forceinline__ long long fixp(double x) {
  return static_cast<long long>(rint(x * kFix));
}

template <int NT>
__device__ __forceinline__ long long block_sum_ll(long long x, long long *smem) {
  constexpr int NW = NT / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = x;
  __syncthreads();
  long long r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) r += smem[w];
  return r;
}

template <int NT>
__device__ __forceinline__ int block_max_i(int x, int *smem) {
  constexpr int NW = NT / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, kWave));
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = x;
  __syncthreads();
  int r = smem[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = max(r, smem[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ int block_min_i(int x, int *smem) {
  return -block_max_i<NT>(-x, smem);
}

// Inclusive scan of a double over the block (NT threads).
template <int NT>
__device__ __forceinline__ double block_incl_scan_d(double x, double *smem) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == kWave - 1) smem[wid] = x;
  __syncthreads();
  double base = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) base += (w < wid) ? smem[w] : 0.0;
  return base + x;
}

__global__ __launch_bounds__(kTauThreads) void k_entmax_tau(
    const float *__restrict__ zbuf, const float *__restrict__ cmax,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, int H, int G, int P, int cap, int maxch,
    int r, float rg, float *__restrict__ tau_ws, float *__restrict__ tau_user) {
  __shared__ unsigned int hist[kTauBins];
  __shared__ int chunks[kTauChunkCap];
  __shared__ float list[kTauList];
  __shared__ int s_nlist;
  __shared__ float red_f[kTauThreads / kWave];
  __shared__ int red_i[kTauThreads / kWave];
  __shared__ double red_d[kTauThreads / kWave];
  __shared__ long long red_ll[kTauThreads / kWave];
  __shared__ int s_bestK;
  __shared__ double s_best_t;
  __shared__ double s_tot[3];

  const int ug = blockIdx.x, u = ug / G;
  const int b = u / H;
  const int tid = threadIdx.x;
  const int len = seq_lens[b];
  const int cnt = sel ? count[u] : n_pages_of(len, P);
  const int ppc = kChunkTokens / P;
  const int nch = (cnt + ppc - 1) / ppc;
  const float *zh = zbuf + static_cast<size_t>(ug) * cap;
  const float *cm = cmax + static_cast<size_t>(ug) * maxch;

  // Largest score and the chunks that may hold candidates.
  float mloc = -FLT_MAX;
  for (int c = tid; c < nch; c += kTauThreads) mloc = fmaxf(mloc, cm[c]);
  const float M = block_max<kTauThreads>(mloc, red_f);
  const double Md = M;
  const double Ld = Md - 1.0;
  const int per = (nch + kTauThreads - 1) / kTauThreads;
  const int c0 = tid * per, c1 = min(nch, c0 + per);
  int ncand = 0;
  for (int c = c0; c < c1; ++c) ncand += static_cast<double>(cm[c]) > Ld;
  int n_chunks;
  int cpos = block_excl_scan<kTauThreads>(ncand, red_i, n_chunks);
  const bool chunk_list = n_chunks <= kTauChunkCap;
  if (chunk_list)
    for (int c = c0; c < c1; ++c)
      if (static_cast<double>(cm[c]) > Ld) chunks[cpos++] = c;
  for (int i = tid; i < kTauBins; i += kTauThreads) hist[i] = 0u;
  if (tid == 0) s_nlist = 0;
  __syncthreads();
  const int n_iter_chunks = chunk_list ? n_chunks : nch;
  const int ctoks = ppc * P;  // == kChunkTokens
  // Visit every candidate token: fn(z) for z > L.
  auto for_candidates = [&](auto fn) {
    for (int k = 0; k < n_iter_chunks; ++k) {
      const int c = chunk_list ? chunks[k] : k;
      if (!chunk_list && !(static_cast<double>(cm[c]) > Ld)) continue;
      const int e = min(cnt * P, (c + 1) * ctoks);
      for (int i = c * ctoks + tid; i < e; i += kTauThreads) {
        const float z = zh[i];
        if (static_cast<double>(z) > Ld) fn(z);
      }
    }
  };
  auto bin_of = [&](float z) {  // z > L on entry, so the bin is >= 0
    const double x = floor((static_cast<double>(z) - Ld) * kTauBins);
    return x < kTauBins ? (x > 0.0 ? static_cast<int>(x) : 0) : kTauBins - 1;
  };

  double t_rel = 0.0;  // tau - M
  bool solved = false;
  double blo = Ld, bhi = Md;  // bisection bracket for the fallback
  if (r == 1 || r == 2) {
    for_candidates([&](float z) { atomicAdd(&hist[bin_of(z)], 1u); });
    __syncthreads();
    // Suffix sums of cnt, cnt*c, cnt*c^2; thread t owns bins [8t, 8t+8).
    constexpr int BPT = kTauBins / kTauThreads;
    double l0 = 0, l1 = 0, l2 = 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const double cb = tid * BPT + k, n = hist[tid * BPT + k];
      l0 += n; l1 += n * cb; l2 += n * cb * cb;
    }
    const double i0 = block_incl_scan_d<kTauThreads>(l0, red_d);
    const double i1 = block_incl_scan_d<kTauThreads>(l1, red_d);
    const double i2 = block_incl_scan_d<kTauThreads>(l2, red_d);
    // Totals (the last thread's inclusive values) via LDS broadcast.
    if (tid == kTauThreads - 1) { s_tot[0] = i0; s_tot[1] = i1; s_tot[2] = i2; }
    __syncthreads();
    // Suffix sums strictly after this thread's bins.
    double S0 = s_tot[0] - i0, S1 = s_tot[1] - i1, S2 = s_tot[2] - i2;
    const double NB = kTauBins, need = (r == 2) ? NB * NB : NB;
    int my_lo = 0, my_hi = kTauBins;  // b = NB always has F_hi = 0 < 1
    for (int k = BPT - 1; k >= 0; --k) {
      const double bb = tid * BPT + k, n = hist[tid * BPT + k];
      S0 += n; S1 += n * bb; S2 += n * bb * bb;
      double flo, fhi;
      if (r == 2) {
        flo = S2 - 2.0 * bb * S1 + bb * bb * S0;
        fhi = S2 - 2.0 * (bb - 1.0) * S1 + (bb - 1.0) * (bb - 1.0) * S0;
      } else {
        flo = S1 - bb * S0;
        fhi = S1 - (bb - 1.0) * S0;
      }
      if (flo >= need) my_lo = max(my_lo, static_cast<int>(bb));
      if (fhi < need) my_hi = min(my_hi, static_cast<int>(bb));
    }
    const int b_lo = block_max_i<kTauThreads>(my_lo, red_i);
    const int b_hi = block_min_i<kTauThreads>(my_hi, red_i);
    blo = Ld + static_cast<double>(b_lo) / kTauBins;
    bhi = Ld + static_cast<double>(b_hi) / kTauBins;

    // Certain support (bin >= b_hi) and the undecided tokens.
    long long nfix = 0, sy = 0, sy2 = 0;
    int minbin_fix = kTauBins;
    for_candidates([&](float z) {
      const int bn = bin_of(z);
      if (bn >= b_hi) {
        const double y = static_cast<double>(z) - Md;
        ++nfix; sy += fixp(y); sy2 += fixp(y * y);
        minbin_fix = min(minbin_fix, bn);
      } else if (bn >= b_lo) {
        const int slot = atomicAdd(&s_nlist, 1);
        if (slot < kTauList) list[slot] = z;
      }
    });
    nfix = block_sum_ll<kTauThreads>(nfix, red_ll);
    sy = block_sum_ll<kTauThreads>(sy, red_ll);
    sy2 = block_sum_ll<kTauThreads>(sy2, red_ll);
    // (block_sum_ll ends with a barrier, so s_nlist is final here.)
    const int nl = s_nlist;
    // Smallest certain value: the least z over bins >= b_hi is needed only
    // through "tau <= every certain value", which holds whenever tau < e_bhi.
    if (nl <= kTauList) {
      if (tid == 0) { s_bestK = -1; s_best_t = 0.0; }
      __syncthreads();
      const double ylo_floor = blo - Md;  // every untracked value is below
      const double ybound_hi = bhi - Md;  // every certain value is >= this
      // Candidate supports: the certain set plus the list values >= z_j
      // (ties ordered by list index), and the certain set alone (j = nl).
      int bestK = -1;
      double best_t = 0.0;
      for (int j = tid; j <= nl; j += kTauThreads) {
        const float zj = j < nl ? list[j] : 0.f;
        long long K = nfix, SY = sy, SY2 = sy2;
        double ynext = ylo_floor;  // largest value left out
        for (int i = 0; i < nl; ++i) {
          const float zi = list[i];
          const bool in = j < nl && (zi > zj || (zi == zj && i <= j));
          if (in) {
            const double y = static_cast<double>(zi) - Md;
            ++K; SY += fixp(y); SY2 += fixp(y * y);
          } else {
            ynext = fmax(ynext, static_cast<double>(zi) - Md);
          }
        }
        if (K == 0) continue;
        const double kd = static_cast<double>(K);
        const double s1 = SY / kFix, s2 = SY2 / kFix;
        double t;
        if (r == 1) {
          t = (s1 - 1.0) / kd;
        } else {
          const double disc = s1 * s1 - kd * (s2 - 1.0);
          if (disc < 0.0) continue;
          t = (s1 - sqrt(disc)) / kd;
        }
        const double ymin_in = j < nl ? static_cast<double>(zj) - Md : ybound_hi;
        if (t <= ymin_in && t >= ynext && K > bestK) {
          bestK = static_cast<int>(K);
          best_t = t;
        }
      }
      const int K_all = block_max_i<kTauThreads>(bestK, red_i);
      if (K_all >= 0 && bestK == K_all) s_best_t = best_t;  // unique K
      __syncthreads();
      if (K_all >= 0) {
        t_rel = s_best_t;
        solved = true;
      }
    }
    (void)minbin_fix;
  }
  if (!solved) {
    // Bisection in double on [blo, bhi] over all candidates.
    double lo = blo, hi = bhi;
    for (int it = 0; it < 64 && hi - lo > 1e-12 * fmax(1.0, fabs(hi)); ++it) {
      const double mid = 0.5 * (lo + hi);
      double f = 0.0;
      for_candidates([&](float z) {
        const double d = static_cast<double>(z) - mid;
        if (d > 0.0) f += (r == 1) ? d : (r == 2) ? d * d : pow(d, static_cast<double>(rg));
      });
      f = block_sum_d<kTauThreads>(f, red_d);
      if (f >= 1.0) lo = mid; else hi = mid;
    }
    t_rel = 0.5 * (lo + hi) - Md;
  }
  if (tid == 0) {
    const float tau = static_cast<float>(Md + t_rel);
    tau_ws[ug] = tau;
    if (tau_user) tau_user[ug] = tau;
  }
}

// ---------------------------------------------------------------------------
// 3a. Apply: chunk partials of sum_i p_i v_i and sum_i p_i.
// ---------------------------------------------------------------------------
template <class E, int D, int G>
__global__ __launch_bounds__(kDecThreads) void k_entmax_apply(
    const typename E::T *__restrict__ vpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, int H, int P, int max_pages, int cap,
    int maxch, int r, float rg, const float *__restrict__ zbuf,
    const float *__restrict__ cmax, const float *__restrict__ tau,
    float *__restrict__ part_o, float *__restrict__ part_s,
    float *__restrict__ probs) {
  constexpr int LPT = D / 8;
  constexpr int TPW = kWave / LPT;
  constexpr int STEP = kDecWaves * TPW * kUnroll;
  __shared__ ChunkPages cp;
  __shared__ float s_acc[kDecWaves][G][D];
  __shared__ float s_sp[kDecWaves][G];
  const int u = blockIdx.y, c = blockIdx.x;
  const int h = u % H, b = u / H;
  int j0, j1, len;
  if (!stage_chunk(cp, page_table, seq_lens, sel, count, u, H, P, max_pages,
                   c, j0, j1, len))
    return;
  float tg[G];
  bool active = false;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    tg[g] = tau[u * G + g];
    active |= cmax[(static_cast<size_t>(u) * G + g) * maxch + c] > tg[g];
  }
  if (!active) return;  // no token of this chunk has p > 0
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  const int Hq = H * G;
  const size_t pstride = static_cast<size_t>(max_pages) * P;
  const int npos = (j1 - j0) * P;
  const float *zu = zbuf + static_cast<size_t>(u) * G * cap;

  float acc[G][8], sp[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    sp[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
  }
  for (int base = 0; base < kChunkTokens; base += STEP) {
    float p[kUnroll][G];
    float x[kUnroll][8];
    bool any[kUnroll];
#pragma unroll
    for (int rr = 0; rr < kUnroll; ++rr) {
      const int i = base + (rr * kDecWaves + wave) * TPW + sub;
      const int jj = i / P, t = i - jj * P;
      const bool valid = i < npos && t < cp.nt[jj < kMaxChunkPages ? jj : 0];
      any[rr] = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float pv = 0.f;
        if (valid) {
          const float z = zu[static_cast<size_t>(g) * cap + static_cast<size_t>(j0) * P + i];
          pv = pow_r(fmaxf(z - tg[g], 0.f), r, rg);
        }
        p[rr][g] = pv;
        any[rr] |= pv > 0.f;
      }
      if (any[rr]) {
        load8(vpool + pool_row(cp.slot[jj], h, t, H, P, D) + d0, x[rr]);
      }
      if (probs && valid) {
        const size_t tok = static_cast<size_t>(cp.lp[jj]) * P + t;
#pragma unroll
        for (int g = 0; g < G; ++g)
          if (li == g)
            probs[(static_cast<size_t>(b) * Hq + h * G + g) * pstride + tok] = p[rr][g];
      }
    }
#pragma unroll
    for (int rr = 0; rr < kUnroll; ++rr) {
      if (any[rr]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[g][j] = fmaf(p[rr][g], x[rr][j], acc[g][j]);
          if (li == 0) sp[g] += p[rr][g];
        }
      }
    }
  }
  // Merge the TPW token groups of the wave (lanes with equal li), then waves.
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = acc[g][j];
#pragma unroll
      for (int o = LPT; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
      acc[g][j] = v;
    }
    const float s = group_sum<kWave>(sp[g]);
    if (lane == 0) s_sp[wave][g] = s;
  }
  if (sub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) s_acc[wave][g][d0 + j] = acc[g][j];
  }
  __syncthreads();
  float *po = part_o + (static_cast<size_t>(u) * maxch + c) * G * D;
  for (int e = threadIdx.x; e < G * D; e += kDecThreads) {
    const int g = e / D, d = e % D;
    float v = s_acc[0][g][d];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) v += s_acc[w][g][d];
    po[e] = v;
  }
  if (threadIdx.x < G) {
    float v = s_sp[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) v += s_sp[w][threadIdx.x];
    part_s[(static_cast<size_t>(u) * maxch + c) * G + threadIdx.x] = v;
  }
}

// ---------------------------------------------------------------------------
// 3b. Merge chunk partials in chunk order: out = sum_c o_c / sum_c s_c over
// the chunks whose maximum exceeds tau (the others contribute exact zeros).
// One block per query head; D threads per chunk slice.
// ---------------------------------------------------------------------------
constexpr int kCombThreads = 1024;

__global__ __launch_bounds__(kCombThreads) void k_entmax_combine(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, int H, int G, int D, int P, int maxch,
    const float *__restrict__ cmax, const float *__restrict__ tau,
    const float *__restrict__ part_o, const float *__restrict__ part_s,
    float *__restrict__ out) {
  __shared__ int act[kTauChunkCap];
  __shared__ int red_i[kCombThreads / kWave];
  __shared__ float s_o[kCombThreads];
  __shared__ float s_s[kCombThreads];
  const int ug = blockIdx.x, u = ug / G, g = ug % G, b = u / H;
  const int tid = threadIdx.x;
  const int len = seq_lens[b];
  const int cnt = sel ? count[u] : n_pages_of(len, P);
  const int ppc = kChunkTokens / P;
  const int nch = (cnt + ppc - 1) / ppc;
  const float t = tau[ug];
  const float *cm = cmax + static_cast<size_t>(ug) * maxch;
  const int per = (nch + kCombThreads - 1) / kCombThreads;
  const int c0 = tid * per, c1 = min(nch, c0 + per);
  int na = 0;
  for (int c = c0; c < c1; ++c) na += cm[c] > t;
  int nact;
  int pos = block_excl_scan<kCombThreads>(na, red_i, nact);
  const bool listed = nact <= kTauChunkCap;
  if (listed)
    for (int c = c0; c < c1; ++c)
      if (cm[c] > t) act[pos++] = c;
  __syncthreads();
  const int slices = kCombThreads / D;
  const int d = tid % D, sl = tid / D;
  float o = 0.f, s = 0.f;
  if (sl < slices) {
    const int n = listed ? nact : nch;
    for (int k = sl; k < n; k += slices) {
      const int c = listed ? act[k] : k;
      if (!listed && !(cm[c] > t)) continue;
      const size_t base = static_cast<size_t>(u) * maxch + c;
      o += part_o[(base * G + g) * D + d];
      if (d == 0) s += part_s[base * G + g];
    }
  }
  s_o[tid] = o;
  s_s[tid] = s;
  __syncthreads();
  if (tid < D) {
    float oo = 0.f, ss = 0.f;
    for (int k = 0; k < slices; ++k) {
      oo += s_o[k * D + tid];
      ss += s_s[k * D];
    }
    out[static_cast<size_t>(ug) * D + tid] = oo / ss;
  }
}

// Zero probs[b][h][0 .. seq_lens[b]) for the debug output.
__global__ void k_fill_probs(const int32_t *__restrict__ seq_lens, int Hq,
                             size_t stride, float *__restrict__ probs) {
  const int bh = blockIdx.y, b = bh / Hq;
  const int len = seq_lens[b];
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < static_cast<size_t>(len); i += static_cast<size_t>(gridDim.x) * blockDim.x)
    probs[static_cast<size_t>(bh) * stride + i] = 0.f;
}

// ---------------------------------------------------------------------------
// Split-K softmax: per chunk, scores to LDS, chunk max m, l = sum exp(s - m),
// acc = sum exp(s - m) v; then a log-sum-exp merge over chunks.
// ---------------------------------------------------------------------------
template <class E, int D, int G>
__global__ __launch_bounds__(kDecThreads) void k_softmax_partial(
    const typename E::T *__restrict__ kpool,
    const typename E::T *__restrict__ vpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, const float *__restrict__ q,
    float scale, int H, int P, int max_pages, int maxch,
    float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_o) {
  constexpr int LPT = D / 8;
  constexpr int TPW = kWave / LPT;
  constexpr int STEP = kDecWaves * TPW * kUnroll;
  __shared__ ChunkPages cp;
  __shared__ float s_sc[G][kChunkTokens];
  __shared__ float s_acc[kDecWaves][G][D];
  __shared__ float red[kDecWaves][G];
  const int u = blockIdx.y, c = blockIdx.x;
  const int h = u % H, b = u / H;
  int j0, j1, len;
  if (!stage_chunk(cp, page_table, seq_lens, sel, count, u, H, P, max_pages,
                   c, j0, j1, len))
    return;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  const int Hq = H * G;
  const int npos = (j1 - j0) * P;
  float qs[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float *qg = q + (static_cast<size_t>(b) * Hq + h * G + g) * D + d0;
#pragma unroll
    for (int j = 0; j < 8; ++j) qs[g][j] = qg[j] * scale;
  }
  float mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = -FLT_MAX;
  for (int base = 0; base < kChunkTokens; base += STEP) {
    float x[kUnroll][8];
    bool valid[kUnroll];
    int pos[kUnroll];
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
      const int i = base + (r * kDecWaves + wave) * TPW + sub;
      const int jj = i / P, t = i - jj * P;
      pos[r] = i;
      valid[r] = i < npos && t < cp.nt[jj < kMaxChunkPages ? jj : 0];
      if (valid[r]) load8(kpool + pool_row(cp.slot[jj], h, t, H, P, D) + d0, x[r]);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[r][j] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaf(qs[g][j], x[r][j], a);
        a = group_sum<LPT>(a);
        if (li == g) s_sc[g][pos[r]] = valid[r] ? a : -INFINITY;
        if (valid[r]) mx[g] = fmaxf(mx[g], a);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float m = group_max<kWave>(mx[g]);
    if (lane == 0) red[wave][g] = m;
  }
  __syncthreads();
  float m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = red[0][g];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) m[g] = fmaxf(m[g], red[w][g]);
  }
  float acc[G][8], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
  }
  for (int base = 0; base < kChunkTokens; base += STEP) {
    float x[kUnroll][8];
    bool valid[kUnroll];
    int pos[kUnroll];
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
      const int i = base + (r * kDecWaves + wave) * TPW + sub;
      const int jj = i / P, t = i - jj * P;
      pos[r] = i;
      valid[r] = i < npos && t < cp.nt[jj < kMaxChunkPages ? jj : 0];
      if (valid[r]) load8(vpool + pool_row(cp.slot[jj], h, t, H, P, D) + d0, x[r]);
    }
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
      if (valid[r]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pw = expf(s_sc[g][pos[r]] - m[g]);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[g][j] = fmaf(pw, x[r][j], acc[g][j]);
          if (li == 0) l[g] += pw;
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = acc[g][j];
#pragma unroll
      for (int o = LPT; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
      acc[g][j] = v;
    }
    l[g] = group_sum<kWave>(l[g]);
  }
  __syncthreads();  // red[] reused below
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) red[wave][g] = l[g];
  }
  if (sub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) s_acc[wave][g][d0 + j] = acc[g][j];
  }
  __syncthreads();
  const size_t pc = static_cast<size_t>(u) * maxch + c;
  float *po = part_o + pc * G * D;
  for (int e = threadIdx.x; e < G * D; e += kDecThreads) {
    const int g = e / D, d = e % D;
    float v = s_acc[0][g][d];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) v += s_acc[w][g][d];
    po[e] = v;
  }
  if (threadIdx.x < G) {
    float v = red[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) v += red[w][threadIdx.x];
    part_l[pc * G + threadIdx.x] = v;
    part_m[pc * G + threadIdx.x] = m[threadIdx.x];
  }
}

__global__ __launch_bounds__(kCombThreads) void k_softmax_combine(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, int H, int G, int D, int P, int maxch,
    const float *__restrict__ part_m, const float *__restrict__ part_l,
    const float *__restrict__ part_o, float *__restrict__ out,
    float *__restrict__ lse) {
  __shared__ float red_f[kCombThreads / kWave];
  __shared__ float s_o[kCombThreads];
  __shared__ float s_l[kCombThreads];
  const int ug = blockIdx.x, u = ug / G, g = ug % G, b = u / H;
  const int tid = threadIdx.x;
  const int len = seq_lens[b];
  const int cnt = sel ? count[u] : n_pages_of(len, P);
  const int ppc = kChunkTokens / P;
  const int nch = (cnt + ppc - 1) / ppc;
  float mloc = -FLT_MAX;
  for (int c = tid; c < nch; c += kCombThreads)
    mloc = fmaxf(mloc, part_m[(static_cast<size_t>(u) * maxch + c) * G + g]);
  const float M = block_max<kCombThreads>(mloc, red_f);
  const int slices = kCombThreads / D;
  const int d = tid % D, sl = tid / D;
  float o = 0.f, l = 0.f;
  if (sl < slices) {
    for (int c = sl; c < nch; c += slices) {
      const size_t base = (static_cast<size_t>(u) * maxch + c) * G + g;
      const float w = expf(part_m[base] - M);
      o = fmaf(w, part_o[base * D + d], o);
      if (d == 0) l = fmaf(w, part_l[base], l);
    }
  }
  s_o[tid] = o;
  s_l[tid] = l;
  __syncthreads();
  if (tid < D) {
    float oo = 0.f, ll = 0.f;
    for (int k = 0; k < slices; ++k) {
      oo += s_o[k * D + tid];
      ll += s_l[k * D];
    }
    out[static_cast<size_t>(ug) * D + tid] = oo / ll;
    if (lse && tid == 0) lse[ug] = M + logf(ll);
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static inline int exponent_code(float alpha, float &rg) {
  rg = 1.0f / (alpha - 1.0f);
  if (alpha == 2.0f) return 1;
  if (alpha == 1.5f) return 2;
  return 0;
}

template <class E, int D, int G>
hipError_t launch_entmax_scores(const ekv_paged_kv &kv, const float *q,
                                float scale, float alpha, const int32_t *sel,
                                const int32_t *count, void *ws,
                                hipStream_t stream) {
  const DecodeWs L = decode_ws_layout(kv);
  char *w = static_cast<char *>(ws);
  const int mc = max_chunks(kv);
  dim3 grid(mc, kv.batch * kv.num_kv_heads);
  hipLaunchKernelGGL((k_entmax_scores<E, D, G>), grid, dim3(kDecThreads), 0,
                     stream, static_cast<const typename E::T *>(kv.k),
                     kv.page_table, kv.seq_lens, sel, count, q,
                     (alpha - 1.0f) * scale, kv.num_kv_heads, kv.page_size,
                     kv.max_pages, kv.max_pages * kv.page_size, mc,
                     reinterpret_cast<float *>(w + L.z),
                     reinterpret_cast<float *>(w + L.cmax));
  return hipGetLastError();
}

template <int G>
hipError_t launch_entmax_threshold(const ekv_paged_kv &kv, float alpha,
                                   const int32_t *sel, const int32_t *count,
                                   float *tau, void *ws, hipStream_t stream) {
  const DecodeWs L = decode_ws_layout(kv);
  char *w = static_cast<char *>(ws);
  float rg;
  const int r = exponent_code(alpha, rg);
  hipLaunchKernelGGL(k_entmax_tau, dim3(kv.batch * kv.num_kv_heads * G),
                     dim3(kTauThreads), 0, stream,
                     reinterpret_cast<const float *>(w + L.z),
                     reinterpret_cast<const float *>(w + L.cmax), kv.seq_lens,
                     sel, count, kv.num_kv_heads, G, kv.page_size,
                     kv.max_pages * kv.page_size, max_chunks(kv), r, rg,
                     reinterpret_cast<float *>(w + L.tau), tau);
  return hipGetLastError();
}

template <class E, int D, int G>
hipError_t launch_entmax_apply(const ekv_paged_kv &kv, float alpha,
                               const int32_t *sel, const int32_t *count,
                               float *out, float *probs, void *ws,
                               hipStream_t stream) {
  const DecodeWs L = decode_ws_layout(kv);
  char *w = static_cast<char *>(ws);
  const int mc = max_chunks(kv);
  const int units = kv.batch * kv.num_kv_heads;
  float rg;
  const int r = exponent_code(alpha, rg);
  const size_t pstride = static_cast<size_t>(kv.max_pages) * kv.page_size;
  if (probs) {
    dim3 g((pstride + 255) / 256 < 1024 ? (pstride + 255) / 256 : 1024,
           kv.batch * kv.num_kv_heads * G);
    hipLaunchKernelGGL(k_fill_probs, g, dim3(256), 0, stream, kv.seq_lens,
                       kv.num_kv_heads * G, pstride, probs);
  }
  hipLaunchKernelGGL((k_entmax_apply<E, D, G>), dim3(mc, units),
                     dim3(kDecThreads), 0, stream,
                     static_cast<const typename E::T *>(kv.v), kv.page_table,
                     kv.seq_lens, sel, count, kv.num_kv_heads, kv.page_size,
                     kv.max_pages, kv.max_pages * kv.page_size, mc, r, rg,
                     reinterpret_cast<const float *>(w + L.z),
                     reinterpret_cast<const float *>(w + L.cmax),
                     reinterpret_cast<const float *>(w + L.tau),
                     reinterpret_cast<float *>(w + L.part_o),
                     reinterpret_cast<float *>(w + L.part_s), probs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_entmax_combine, dim3(units * G), dim3(kCombThreads), 0,
                     stream, kv.seq_lens, sel, count, kv.num_kv_heads, G, D,
                     kv.page_size, mc,
                     reinterpret_cast<const float *>(w + L.cmax),
                     reinterpret_cast<const float *>(w + L.tau),
                     reinterpret_cast<const float *>(w + L.part_o),
                     reinterpret_cast<const float *>(w + L.part_s), out);
  return hipGetLastError();
}

template <class E, int D, int G>
hipError_t launch_softmax(const ekv_paged_kv &kv, const float *q, float scale,
                          const int32_t *sel, const int32_t *count, float *out,
                          float *lse, void *ws, hipStream_t stream) {
  const SoftmaxWs L = softmax_ws_layout(kv);
  char *w = static_cast<char *>(ws);
  const int mc = max_chunks(kv);
  const int units = kv.batch * kv.num_kv_heads;
  hipLaunchKernelGGL((k_softmax_partial<E, D, G>), dim3(mc, units),
                     dim3(kDecThreads), 0, stream,
                     static_cast<const typename E::T *>(kv.k),
                     static_cast<const typename E::T *>(kv.v), kv.page_table,
                     kv.seq_lens, sel, count, q, scale, kv.num_kv_heads,
                     kv.page_size, kv.max_pages, mc,
                     reinterpret_cast<float *>(w + L.part_m),
                     reinterpret_cast<float *>(w + L.part_l),
                     reinterpret_cast<float *>(w + L.part_o));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_softmax_combine, dim3(units * G), dim3(kCombThreads), 0,
                     stream, kv.seq_lens, sel, count, kv.num_kv_heads, G, D,
                     kv.page_size, mc,
                     reinterpret_cast<const float *>(w + L.part_m),
                     reinterpret_cast<const float *>(w + L.part_l),
                     reinterpret_cast<const float *>(w + L.part_o), out, lse);
  return hipGetLastError();
}

#define EKV_INST_DEC(E, D, G)                                                \
  template hipError_t launch_entmax_scores<E, D, G>(                         \
      const ekv_paged_kv &, const float *, float, float, const int32_t *,    \
      const int32_t *, void *, hipStream_t);                                 \
  template hipError_t launch_entmax_apply<E, D, G>(                          \
      const ekv_paged_kv &, float, const int32_t *, const int32_t *, float *, \
      float *, void *, hipStream_t);                                         \
  template hipError_t launch_softmax<E, D, G>(                               \
      const ekv_paged_kv &, const float *, float, const int32_t *,           \
      const int32_t *, float *, float *, void *, hipStream_t);
EKV_FOR_EACH_EDG(EKV_INST_DEC)

#define EKV_INST_TAU(G)                                                      \
  template hipError_t launch_entmax_threshold<G>(                            \
      const ekv_paged_kv &, float, const int32_t *, const int32_t *, float *, \
      void *, hipStream_t);
EKV_FOR_EACH_G(EKV_INST_TAU)

}  // namespace ekv
