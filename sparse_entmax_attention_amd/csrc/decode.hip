// Sparse alpha-entmax attention over gathered pages, and the split-K softmax
// baseline (Technical Summary: EntmaxKV, §2.C "Sparse Entmax Attention" and
// §4 "Efficiency").
//
// Entmax has no single-pass running form: the threshold tau depends on every
// score.  The step is therefore split in three launches:
//   1. scores:    (kpass.hip) the selected pages' keys are gathered and
//                 z = (alpha-1) scale <q, k> is computed for the G query
//                 heads on the matrix cores; z and each page's maximum are
//                 written;
//   2. threshold: per query head, tau from the tokens that can still be in
//                 the support (tau is at least max z - 1, and at least
//                 c - k^-(alpha-1) whenever k page maxima reach c); exact
//                 for alpha in {1.5, 2};
//   3. apply:     per chunk of pages, p = max(z - tau, 0)^r and value rows
//                 are read only where some head has p > 0 (the other rows
//                 carry zero weight); chunk partials are merged in order.
// HBM reads: selected K once, V only on the support, z twice.
#include <float.h>

#include <type_traits>

#include "decode_common.h"

namespace ekv {

DecodeWs decode_ws_layout(const ekv_paged_kv &kv) {
  const size_t units = static_cast<size_t>(kv.batch) * kv.num_kv_heads;
  const size_t G = kv.group, D = kv.head_dim;
  const size_t cap = static_cast<size_t>(kv.max_pages) * kv.page_size;
  const size_t mc = max_chunks(kv);
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  DecodeWs w;
  w.z = 0;
  w.cmax = al(w.z + units * G * cap * 4);  // per-page maxima
  w.tau = al(w.cmax + units * G * static_cast<size_t>(pm_stride(kv.max_pages)) * 4);
  w.part_o = al(w.tau + units * G * 4);
  w.part_s = al(w.part_o + units * mc * G * D * 4);
  w.ctr = al(w.part_s + units * mc * G * 4);  // chunks finished, per unit
  w.done = al(w.ctr + (units + 1) * 4);  // + heads left to the apply step
  w.slot = al(w.done + units * G * 4);  // pool slot per selected page
  w.floor = al(w.slot + units * static_cast<size_t>(kv.max_pages) * 4);  // per head
  w.qz = al(w.floor + units * G * 4);  // (alpha-1) scale q per head
  w.mask = al(w.qz + units * G * D * 4);  // candidate bits per page and head
  w.total = al(w.mask + units * G * static_cast<size_t>(pm_stride(kv.max_pages)) * 8);
  return w;
}

SoftmaxWs softmax_ws_layout(const ekv_paged_kv &kv) {
  const size_t units = static_cast<size_t>(kv.batch) * kv.num_kv_heads;
  const size_t G = kv.group, D = kv.head_dim;
  const size_t mc = max_chunks(kv);
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  // partial slots: one per chunk (float32 K/V) or per streaming segment
  // (bfloat16 K/V), whichever is more
  const size_t slots = std::max(units * mc, softmax_stream_slots(kv));
  SoftmaxWs w;
  w.part_m = 0;
  w.part_l = al(slots * G * 4);
  w.part_o = al(w.part_l + slots * G * 4);
  w.seg = al(w.part_o + slots * G * D * 4);
  w.total = al(w.seg + units * 2 * 4);
  return w;
}

// ---------------------------------------------------------------------------
// 2. Threshold.  One block per query head.
//
// Bracket.  tau >= M - 1 with M = max z.  Moreover, if k page maxima are at
// least c, those k tokens alone give sum (z - t)^r >= 1 at t = c - k^-(1/r),
// so tau >= c - k^-(1/r); a 256-bin count of the page maxima near M gives
// the best such c cheaply.  Only tokens above the resulting L can have
// p > 0; they are staged in LDS.
//
// Exact solve (r in {1, 2}).  The staged values are counted into NB bins of
// width w = 2^-m over [L, L + NB w] (w a power of two, so bin membership is
// exact).  For the bin edge e_b, values in bin c >= b satisfy
// (c-b) w <= z - e_b < (c+1-b) w, hence
//   F_lo(b) = w^r sum_{c>=b} cnt_c (c-b)^r <= F(e_b) <= F_hi(b) = ... (c+1-b)^r
// with F(t) = sum max(z - t, 0)^r; both are polynomials in b of suffix sums
// of cnt_c c^k, exact in double.  The largest b with F_lo >= 1 and the
// smallest with F_hi < 1 bracket tau.  Values above the bracket are in the
// support (only their count, sum of (z - M) and of (z - M)^2 matter); the
// few inside it are listed and the support size is resolved exactly: for a
// support of the K largest values tau has a closed form (sparsemax:
// (sum z - 1)/K; 1.5-entmax: the smaller root of sum (z - tau)^2 = 1), and
// the right K is the one whose tau separates the K-th and (K+1)-th values.
// Sums are kept in 2^-40 fixed point so that the result does not depend on
// the order the block visits the tokens.  General alpha, or a bracket with
// too many undecided tokens, falls back to bisection in double.
// ---------------------------------------------------------------------------
// One pass of the support iteration reduces four values over a wave: the
// count, the sums of y and y^2, and the minimum.  The four are taken through
// each swizzle level together, so their dependency chains overlap, and the
// result (lane 63 after the row broadcasts) is read back to every lane.
__device__ __forceinline__ void wave_reduce_pass(int &k, double &sy, double &sy2,
                                                 float &zmin) {
#define EKV_PASS_LEVEL(CTRL)                            \
  k += dpp_i<CTRL>(k);                                  \
  sy += dpp_d<CTRL>(sy);                                \
  sy2 += dpp_d<CTRL>(sy2);                              \
  zmin = fminf(zmin, dpp_f<CTRL>(zmin));
  EKV_PASS_LEVEL(kDppRowMirror)
  EKV_PASS_LEVEL(kDppRowHalfMirror)
  EKV_PASS_LEVEL(kDppQuad2301)
  EKV_PASS_LEVEL(kDppQuad1032)
#undef EKV_PASS_LEVEL
  const int idle = __float_as_int(FLT_MAX);
  k += dpp_rows<kDppRowBcast15, 0xA>(k, 0);
  sy += dpp_rows_d<kDppRowBcast15, 0xA>(sy);
  sy2 += dpp_rows_d<kDppRowBcast15, 0xA>(sy2);
  zmin = fminf(zmin, __int_as_float(dpp_rows<kDppRowBcast15, 0xA>(__float_as_int(zmin), idle)));
  k += dpp_rows<kDppRowBcast31, 0xC>(k, 0);
  sy += dpp_rows_d<kDppRowBcast31, 0xC>(sy);
  sy2 += dpp_rows_d<kDppRowBcast31, 0xC>(sy2);
  zmin = fminf(zmin, __int_as_float(dpp_rows<kDppRowBcast31, 0xC>(__float_as_int(zmin), idle)));
  k = __builtin_amdgcn_readlane(k, kWave - 1);
  sy = readlane_d(sy, kWave - 1);
  sy2 = readlane_d(sy2, kWave - 1);
  zmin = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zmin), kWave - 1));
}

constexpr int kTauThreads = 512;
constexpr int kTauBins = 2048;
constexpr int kTauList = 1024;
constexpr int kTauPageCap = 4096;
constexpr int kTauCandCap = 8192;
constexpr int kTauMaxBins = 512;
constexpr int kTauIters = 64;  // support iterations before the fallback
constexpr double kFix = 1099511627776.0;  // 2^40

__device__ __forceinline__ long long fixp(double x) {
  return static_cast<long long>(rint(x * kFix));
}

template <int W>
__device__ __forceinline__ long long group_sum_ll(long long x) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

template <int NT>
__device__ __forceinline__ long long block_sum_ll(long long x, long long *smem) {
  constexpr int NW = NT / kWave;
  x = group_sum_ll<kWave>(x);
  lds_barrier();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = x;
  lds_barrier();
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
  lds_barrier();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = x;
  lds_barrier();
  int r = smem[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = max(r, smem[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ int block_min_i(int x, int *smem) {
  return -block_max_i<NT>(-x, smem);
}
template <int NT>
__device__ __forceinline__ double block_max_d(double x, double *smem) {
  constexpr int NW = NT / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o, kWave));
  lds_barrier();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = x;
  lds_barrier();
  double r = smem[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmax(r, smem[w]);
  return r;
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
  lds_barrier();
  if (lane == kWave - 1) smem[wid] = x;
  lds_barrier();
  double base = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) base += (w < wid) ? smem[w] : 0.0;
  return base + x;
}

// Scores of every selected token of one query head, recomputed on the vector
// units from the keys (z = <qz, k>, qz = (alpha-1) scale q) and written in
// the plain layout with -inf past each page's valid tokens, together with
// the page maxima: what an unhinted key pass leaves for that head.  Used
// when a hinted key pass kept too few scores.  Whole block; ends with a
// barrier after which the block sees the new values.
template <class E, int D>
__device__ void recompute_head_scores(const typename E::T *kpool,
                                      const int32_t *page_table,
                                      const int32_t *seq_lens,
                                      const int32_t *sel, const int32_t *slots,
                                      const float *qz, int u, int cnt, int H,
                                      int P, int max_pages, float *zh,
                                      float *pm) {
  constexpr int LPT = D / 8, TPW = kWave / LPT;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  const int nwv = blockDim.x / kWave;
  const int b = u / H, h = u % H;
  float qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] = qz[d0 + j];
  for (int j = wave; j < cnt; j += nwv) {
    const int lp = sel ? sel[static_cast<size_t>(u) * max_pages + j] : j;
    const int nt = page_tokens(lp, seq_lens[b], P);
    const int slot = slots[static_cast<size_t>(u) * max_pages + j];
    float mx = -FLT_MAX;
    for (int t0 = 0; t0 < P; t0 += TPW) {
      const int t = t0 + sub;
      float x[8];
      load8(kpool + pool_row(slot, h, t, H, P, D) + d0, x);
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) a = fmaf(qv[k], x[k], a);
      a = group_sum<LPT>(a);
      const bool valid = t < nt;
      if (li == 0) zh[static_cast<size_t>(j) * P + t] = valid ? a : -INFINITY;
      if (valid) mx = fmaxf(mx, a);
    }
    mx = group_max<kWave>(mx);
    if (lane == 0) pm[j] = mx;
  }
  __threadfence_block();
  __syncthreads();
}

// HALF: half the on-chip capacities (candidates and listed pages), about
// 66 KiB of LDS instead of 128 KiB, so that two blocks share a CU; used when
// there are more query heads than CUs (heads beyond the capacities take the
// same overflow paths as in the full-size form).
template <class E, int D, bool HALF>
__global__ __launch_bounds__(kTauThreads) void k_entmax_tau(
    float *__restrict__ zbuf, float *__restrict__ pmax,
    const typename E::T *__restrict__ vpool,
    const typename E::T *__restrict__ kpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, int H, int G, int P, int max_pages,
    int cap, int r, float rg, float *__restrict__ tau_ws,
    float *__restrict__ tau_user, float *__restrict__ out,
    int32_t *__restrict__ done, int32_t *__restrict__ ctr,
    const int32_t *__restrict__ slots, int32_t *__restrict__ undone,
    const float *__restrict__ floor_ws, const float *__restrict__ qz,
    const unsigned long long *__restrict__ pmask) {
  constexpr int NW = kTauThreads / kWave;
  constexpr int CandCap = HALF ? kTauCandCap / 2 : kTauCandCap;
  constexpr int PageCap = HALF ? kTauPageCap / 2 : kTauPageCap;
  constexpr int SEGP = PageCap / NW;  // listed pages per wave
  constexpr int CSEG = CandCap / NW;  // staged candidates per wave
  __shared__ unsigned int hist[kTauBins];
  __shared__ int cpages[NW][SEGP];
  __shared__ float cand[CandCap];   // z of the staged candidates
  __shared__ int cpos[CandCap];     // their positions jj * P + t
  __shared__ float s_vacc[NW][D];
  __shared__ float s_vsum[NW];
  __shared__ float list[kTauList];
  __shared__ int s_nlist;
  __shared__ int s_npg[NW];
  __shared__ int dense[PageCap];   // listed pages (selection index j)
  __shared__ int dslot[PageCap];   // their pool slots
  __shared__ float s_wmax[NW];
  __shared__ int s_wscan[NW];
  __shared__ double s_wL[NW];
  __shared__ int red_i[NW];
  __shared__ double red_d[NW];
  __shared__ long long red_ll[NW];
  __shared__ double s_best_t;
  __shared__ double s_tot[3];
  __shared__ int s_ccnt[NW];
  __shared__ int s_wsolved;
  __shared__ double s_wtau;

  const int ug = blockIdx.x, u = ug / G;
  const int lgP = __builtin_ctz(P);  // page sizes are powers of two
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int mps = pm_stride(max_pages);
  float *zh = zbuf + static_cast<size_t>(ug) * cap;
  float *pm = pmax + static_cast<size_t>(ug) * mps;
  constexpr int U = 32, U4 = U / 4;
  const int cnt = unit_pages(seq_lens, sel, count, u, H, P);
  const unsigned long long below = (1ull << lane) - 1ull;

  // Results of the front end: the largest score M, a lower bound L on tau
  // (Lf: the largest float not above L) and, in LDS, every score above L
  // (per-wave segments of cand / cpos, counts in s_ccnt).  With `listed`,
  // cpos holds (index into dense) * P + t, else (selection index) * P + t.
  float M = -FLT_MAX, Lf = -FLT_MAX;
  double Md = 0.0, L = 0.0;
  bool listed = false;
  int n_pg = cnt;

  // Hinted key pass: only scores above the floor f were kept, packed per
  // page with a bit mask.  They are staged here; if they alone give
  // sum (z - f)_+^r >= 1, then tau >= f (the full sum is larger), every
  // score of the support is among them and f serves as L.  Otherwise the
  // head's scores are recomputed in full and the plain front end runs.
  const float fl = floor_ws[ug];
  bool hinted = fl > -INFINITY;
  if (hinted) {
    constexpr int MCAP = (NW * SEGP * static_cast<int>(sizeof(int))) /
                         static_cast<int>(sizeof(unsigned long long));
    unsigned long long *dmask = reinterpret_cast<unsigned long long *>(&cpages[0][0]);
    const unsigned long long *mk = pmask + static_cast<size_t>(ug) * mps;
    // 1. pages holding candidates, in page order, with their masks and pool
    // slots (the slots loaded beside the masks, all in flight together)
    const int32_t *uslots = slots + static_cast<size_t>(u) * max_pages;
    int n_cp = 0;
    for (int base = 0; base < cnt; base += kTauThreads * 4) {
      unsigned long long m4[4];
      int s4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = min(base + k * kTauThreads + tid, cnt - 1);
        m4[k] = mk[j];
        s4[k] = uslots[j];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = base + k * kTauThreads + tid;
        const bool has = j < cnt && m4[k] != 0ull;
        int tot;
        const int rk = tile_rank<kTauThreads>(has, red_i, tot);
        if (has && n_cp + rk < MCAP) {
          dense[n_cp + rk] = j;
          dmask[n_cp + rk] = m4[k];
          dslot[n_cp + rk] = s4[k];
        }
        n_cp += tot;
      }
    }
    lds_barrier();
    // 2. stage them in page order, candidate e of the head going to segment
    // e / per_seg (per_seg = ceil(C / NW)): the per-page counts are scanned
    // (each thread owns 4 consecutive listed pages, offsets kept in dslot),
    // then every thread takes candidates tid, tid + kTauThreads, ..., finds
    // its page by bisection over the offsets and its token as the rank-th
    // set bit of the page's mask; all of a thread's loads are in flight
    // together.
    int *coff = reinterpret_cast<int *>(hist);  // kTauBins >= MCAP entries
    int C = 0;
    if (n_cp <= MCAP) {
      int cnt4[4], loc = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int li = 4 * tid + k;
        cnt4[k] = li < n_cp ? __popcll(dmask[li]) : 0;
        loc += cnt4[k];
      }
      int pre = block_excl_scan<kTauThreads>(loc, red_i, C);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int li = 4 * tid + k;
        if (li < n_cp) coff[li] = pre;
        pre += cnt4[k];
      }
    }
    lds_barrier();
    int nc = 0;
    float mloc = -FLT_MAX;
    const int per_seg = (C + NW - 1) / NW;
    if (n_cp <= MCAP && per_seg <= CSEG) {
      constexpr int EU = 4;  // candidates per thread per round
      for (int e0 = 0; e0 < C; e0 += EU * kTauThreads) {
        float zv[EU];
        int posv[EU];
#pragma unroll
        for (int k = 0; k < EU; ++k) {
          const int e = min(e0 + k * kTauThreads + tid, C - 1);
          int lo = 0, hi = n_cp - 1;  // last listed page with coff <= e
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (coff[mid] <= e) lo = mid; else hi = mid - 1;
          }
          int rk = e - coff[lo];
          unsigned long long m = dmask[lo];
          int t = 0;  // position of the rk-th set bit of m
#pragma unroll
          for (int w = 32; w >= 1; w >>= 1) {
            const unsigned long long lowm = m & ((1ull << w) - 1ull);
            const int c = __popcll(lowm);
            if (rk >= c) {
              rk -= c;
              m >>= w;
              t += w;
            } else {
              m = lowm;
            }
          }
          // position: listed page index * P + token (slots in dslot)
          zv[k] = zh[static_cast<size_t>(dense[lo]) * P + (e - coff[lo])];
          posv[k] = lo * P + t;
        }
#pragma unroll
        for (int k = 0; k < EU; ++k) {
          const int e = e0 + k * kTauThreads + tid;
          if (e < C) {
            const int w = e / per_seg, i = e - w * per_seg;
            cand[w * CSEG + i] = zv[k];
            cpos[w * CSEG + i] = posv[k];
            mloc = fmaxf(mloc, zv[k]);
          }
        }
      }
      nc = max(0, min(per_seg, C - wave * per_seg));
    }
    if (lane == 0) s_ccnt[wave] = (n_cp <= MCAP && per_seg <= CSEG) ? nc : CSEG + 1;
    lds_barrier();
    bool fits = n_cp <= MCAP;
#pragma unroll
    for (int w = 0; w < NW; ++w) fits &= s_ccnt[w] <= CSEG;
    // 3. M and the check sum (z - f)_+^r >= 1 (double), over the staged
    // candidates.
    double fs = 0.0;
    if (fits) {
      const int ncw = s_ccnt[wave];
      for (int i = lane; i < ncw; i += kWave) {
        const double y = static_cast<double>(cand[wave * CSEG + i]) - fl;
        fs += (r == 1) ? y : (r == 2) ? y * y : pow(y, static_cast<double>(rg));
      }
    }
    fs = wave_sum_d(fs);
    mloc = wave_max_f(mloc);
    if (lane == 0) {
      red_d[wave] = fs;
      s_wmax[wave] = mloc;
    }
    lds_barrier();
    double fsum = 0.0;
    float mall = -FLT_MAX;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      fsum += red_d[w];
      mall = fmaxf(mall, s_wmax[w]);
    }
    if (fits && fsum >= 1.0) {
      M = mall;
      Md = M;
      L = fl;
      Lf = fl;
      listed = true;
      n_pg = n_cp;
    } else {
      recompute_head_scores<E, D>(kpool, page_table, seq_lens, sel, slots,
                                  qz + static_cast<size_t>(ug) * D, u, cnt, H,
                                  P, max_pages, zh, pm);
      hinted = false;
    }
  }

  if (!hinted) {

  // Page maxima, read once with 16-byte loads, issued before the page count
  // is known (rows are padded to a multiple of 4; entries past the count
  // are masked): thread tid holds pages 4 tid + e + 4 k kTauThreads
  // (e < 4, k < U/4); pages beyond U * kTauThreads (very long selections)
  // are re-read when needed.
  static_assert(kTauMaxBins <= kTauBins, "page-maximum bins reuse hist");
  static_assert(kTauBins * sizeof(unsigned int) >= 2048 * sizeof(int),
                "hinted candidate offsets reuse hist");
  constexpr int CACHED = kTauThreads * U;
  auto page_k = [&](int k, int e) { return 4 * tid + e + 4 * k * kTauThreads; };
  float pv[U];
#pragma unroll
  for (int k = 0; k < U4; ++k) {
    // unconditional (clamped into the row, whose length mps is a multiple
    // of 4), so that all U4 loads are in flight together
    const float4 v = *reinterpret_cast<const float4 *>(pm + min(page_k(k, 0), mps - 4));
    pv[4 * k] = v.x; pv[4 * k + 1] = v.y; pv[4 * k + 2] = v.z; pv[4 * k + 3] = v.w;
  }
  // Slices k (4 kTauThreads pages each) that hold selected pages: the others
  // are skipped (the test is uniform, and no load depends on it).
  const int nsl = min(U4, (cnt + 4 * kTauThreads - 1) / (4 * kTauThreads));
#pragma unroll
  for (int k = 0; k < U4; ++k)
    if (k < nsl)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (page_k(k, e) >= cnt) pv[4 * k + e] = -FLT_MAX;
  for (int i = tid; i < kTauMaxBins; i += kTauThreads) hist[i] = 0u;
  // Largest score (the barrier also orders the clearing of hist).
  float mloc = -FLT_MAX;
#pragma unroll
  for (int k = 0; k < U4; ++k)
    if (k < nsl)
#pragma unroll
      for (int e = 0; e < 4; ++e) mloc = fmaxf(mloc, pv[4 * k + e]);
  for (int j = CACHED + tid; j < cnt; j += kTauThreads) mloc = fmaxf(mloc, pm[j]);
  mloc = wave_max_f(mloc);
  if (lane == 0) s_wmax[wave] = mloc;
  lds_barrier();
  M = s_wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, s_wmax[w]);
  Md = M;

  // Tighter lower bracket from the page maxima within 1 of M: with C_b the
  // number of page maxima in bins >= b (all at least the bin's lower edge
  // e_b), tau >= e_b - C_b^(-1/r).
  auto count_max = [&](float v) {
    const double x = (static_cast<double>(v) - (Md - 1.0)) * kTauMaxBins;
    if (x > 0.0) {
      const int bn = x < kTauMaxBins ? static_cast<int>(x) : kTauMaxBins - 1;
      atomicAdd(&hist[bn], 1u);
    }
  };
#pragma unroll
  for (int k = 0; k < U4; ++k)
    if (k < nsl)
#pragma unroll
      for (int e = 0; e < 4; ++e) count_max(pv[4 * k + e]);
  for (int j = CACHED + tid; j < cnt; j += kTauThreads) count_max(pm[j]);
  lds_barrier();
  double Lloc = Md - 1.0;
  {
    static_assert(kTauMaxBins == kTauThreads, "one bin per thread");
    const int bin = kTauMaxBins - 1 - tid;  // thread 0 owns the top bin
    const int x = static_cast<int>(hist[bin]);
    // page maxima in bins >= bin: a scan in thread order
    const int incl = wave_incl_scan_dpp(x);
    if (lane == kWave - 1) s_wscan[wave] = incl;
    lds_barrier();
    int c = incl;
#pragma unroll
    for (int w = 0; w < NW; ++w) c += (w < wave) ? s_wscan[w] : 0;
    if (c > 0) {
      const double edge = (Md - 1.0) + static_cast<double>(bin) / kTauMaxBins;
      const double kk = static_cast<double>(c);
      const double drop = (r == 1) ? 1.0 / kk : (r == 2) ? 1.0 / sqrt(kk)
                                   : pow(kk, -1.0 / static_cast<double>(rg));
      Lloc = fmax(Lloc, edge - drop);
    }
  }
  Lloc = wave_max_d(Lloc);
  if (lane == 0) s_wL[wave] = Lloc;
  lds_barrier();
  L = s_wL[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) L = fmax(L, s_wL[w]);
  // Snap down to a multiple of 2^-24 so that z - L is exact in double.
  L = floor(L * 16777216.0) / 16777216.0;
  // For a float z, z > L exactly when z > Lf, the largest float <= L.
  Lf = static_cast<float>(L);
  if (static_cast<double>(Lf) > L) Lf = nextafterf(Lf, -INFINITY);

  // Pages whose maximum exceeds L: each wave lists those it holds, then the
  // lists are laid end to end in `dense`.  The order is fixed but not
  // ascending: lane l of wave w holds pages 4 (64 w + l) + e + 4 k
  // kTauThreads, and the wave lists them slice k by slice k and, within a
  // slice, e by e (pages 256 w + 4 l, then 256 w + 4 l + 1, ...).  Nothing
  // that reads `dense` or `dslot` relies on their order.
  int npw = 0;
  auto list_page = [&](int j, float v) {  // called by whole waves
    const bool flag = j < cnt && v > Lf;
    const unsigned long long ball = __ballot(flag);
    const int rk = npw + __popcll(ball & below);
    if (flag && rk < SEGP) cpages[wave][rk] = j;
    npw += __popcll(ball);
  };
#pragma unroll
  for (int k = 0; k < U4; ++k)
    if (k < nsl)
#pragma unroll
      for (int e = 0; e < 4; ++e) list_page(page_k(k, e), pv[4 * k + e]);
  for (int jb = CACHED + wave * kWave; jb < cnt; jb += kTauThreads) {
    const int j = jb + lane;
    list_page(j, j < cnt ? pm[j] : -FLT_MAX);
  }
  if (lane == 0) s_npg[wave] = npw;
  if (tid == 0) s_nlist = 0;
  lds_barrier();
  listed = true;
  int n_listed = 0, seg0 = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = s_npg[w];
    listed &= c <= SEGP;
    seg0 += (w < wave) ? c : 0;
    n_listed += c;
  }
  if (listed)
    for (int i = lane; i < npw; i += kWave) dense[seg0 + i] = cpages[wave][i];
  lds_barrier();
  n_pg = listed ? n_listed : cnt;

  // Stage the candidates z > L in LDS, wave w appending to its own segment
  // cand[w * CSEG ..] in a fixed order (no atomics, so the order does not
  // change from run to run).  Each lane loads 4 consecutive scores (16 bytes)
  // of a page, so a wave step covers 4 kWave / P listed pages; US steps are
  // in flight.
  {
    constexpr int US = 8;
    const int lpp = P / 4, ppw = kWave / lpp;
    const int sub = lane / lpp, t4 = 4 * (lane - sub * lpp);
    const int steps = (n_pg + ppw - 1) / ppw;
    int nc = 0;
    for (int s0 = wave; s0 < steps; s0 += NW * US) {
      float4 zv[US];
      int zs[US];
      if (listed) {
        // The listed pages all hold candidates: their scores and pool slots
        // (written by the score pass, for the value gather at the end) are
        // loaded unconditionally, from a clamped index past the list, so
        // that all of them are in flight together.
#pragma unroll
        for (int k = 0; k < US; ++k) {
          const int jj = (s0 + k * NW) * ppw + sub;
          const int j = dense[min(jj, n_pg - 1)];
          const float4 v = *reinterpret_cast<const float4 *>(zh + static_cast<size_t>(j) * P + t4);
          zs[k] = slots[static_cast<size_t>(u) * max_pages + j];
          zv[k] = jj < n_pg ? v : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
      } else {
#pragma unroll
        for (int k = 0; k < US; ++k) {
          const int jj = (s0 + k * NW) * ppw + sub;
          zv[k] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
          zs[k] = 0;
          if (jj < n_pg && pm[jj] > Lf)
            zv[k] = *reinterpret_cast<const float4 *>(zh + static_cast<size_t>(jj) * P + t4);
        }
      }
#pragma unroll
      for (int k = 0; k < US; ++k) {
        const int jj = (s0 + k * NW) * ppw + sub;
        const float ze[4] = {zv[k].x, zv[k].y, zv[k].z, zv[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool hit = ze[e] > Lf;
          const unsigned long long ball = __ballot(hit);
          const int sidx = nc + __popcll(ball & below);
          if (hit && sidx < CSEG) {
            cand[wave * CSEG + sidx] = ze[e];
            cpos[wave * CSEG + sidx] = jj * P + t4 + e;
          }
          nc += __popcll(ball);
        }
        if (listed && t4 == 0 && jj < n_pg) dslot[jj] = zs[k];
      }
    }
    if (lane == 0) s_ccnt[wave] = nc;
  }
  lds_barrier();
  }  // plain front end
  auto page_of = [&](int jj) { return listed ? dense[jj] : jj; };
  bool staged = true;
#pragma unroll
  for (int w = 0; w < NW; ++w) staged &= s_ccnt[w] <= CSEG;
  // Visit every candidate z > L: from LDS when staged, else from memory.
  auto for_candidates = [&](auto fn) {
    if (staged) {
      for (int w = 0; w < NW; ++w)
        for (int i = tid; i < s_ccnt[w]; i += kTauThreads) fn(cand[w * CSEG + i]);
    } else {
      const int span = n_pg * P;
      for (int fi = tid; fi < span; fi += kTauThreads) {
        const int jj = fi / P, t = fi - jj * P;
        const int j = page_of(jj);
        if (!listed && !(pm[j] > Lf)) continue;
        const float z = zh[static_cast<size_t>(j) * P + t];
        if (z > Lf) fn(z);
      }
    }
  };

  double t_rel = 0.0;  // tau - M
  bool solved = false;
  double blo = L, bhi = Md;  // bracket for the fallback

  // Exact solve by support iteration (r in {1, 2}, candidates staged), by
  // wave 0 alone, in y = z - M from t = L - M (a lower bound on tau - M):
  // wave_support_iter over the candidates in registers (float32 sums, the
  // final support's closed form in double), or, beyond 2048 candidates, the
  // same iteration over LDS in double.  Lanes sum their candidates in a
  // fixed order and the wave reduces in a fixed pattern, so the result is
  // the same on every run.
  if (staged && (r == 1 || r == 2)) {
    if (wave == 0) {
      // Up to 2048 candidates are held in registers: candidate e (in
      // segment order) goes to lane e % 64, slot e / 64, as y = z - M; the
      // slot count is the smallest power of two that holds them.  Segment
      // starts in scalar registers (wave-uniform), so that locating a
      // candidate is a compare chain rather than dependent LDS reads.
      int segs[NW + 1];
      segs[0] = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        segs[w + 1] = segs[w] + __builtin_amdgcn_readfirstlane(s_ccnt[w]);
      const int n_all = segs[NW];
      // the start, L - M rounded down to a float (a lower bound on tau - M)
      float t0 = static_cast<float>(L - Md);
      if (static_cast<double>(t0) > L - Md) t0 = nextafterf(t0, -INFINITY);
      double res = 0.0;
      bool ok = false;
      auto solve_in_regs = [&](auto slots) {
        constexpr int RR = decltype(slots)::value;
        float y[RR];
#pragma unroll
        for (int k = 0; k < RR; ++k) {
          const int e = lane + k * kWave;
          int base = 0, w = 0;
#pragma unroll
          for (int v = 1; v < NW; ++v)
            if (e >= segs[v]) { w = v; base = segs[v]; }
          const bool on = e < n_all;
          const float zc = cand[on ? w * CSEG + (e - base) : 0];
          y[k] = on ? zc - M : -INFINITY;
        }
        ok = wave_support_iter<RR>(y, t0, r, kTauIters, res);
      };
      if (n_all <= 4 * kWave) solve_in_regs(std::integral_constant<int, 4>());
      else if (n_all <= 8 * kWave) solve_in_regs(std::integral_constant<int, 8>());
      else if (n_all <= 16 * kWave) solve_in_regs(std::integral_constant<int, 16>());
      else if (n_all <= 32 * kWave) solve_in_regs(std::integral_constant<int, 32>());
      else {
        // more candidates than registers: the same iteration over LDS, in
        // double
        double t = static_cast<double>(t0);
        for (int it = 0; it < kTauIters; ++it) {
          int K = 0;
          double SY = 0.0, SY2 = 0.0;
          float zmin = FLT_MAX;
          for (int w = 0; w < NW; ++w)
            for (int i = lane; i < s_ccnt[w]; i += kWave) {
              const float zc = cand[w * CSEG + i];
              const double y = static_cast<double>(zc) - Md;
              const bool in = y > t;
              const double yy = in ? y : 0.0;
              K += in ? 1 : 0;
              SY += yy;
              SY2 = fma(yy, yy, SY2);
              zmin = in ? fminf(zmin, zc) : zmin;
            }
          wave_reduce_pass(K, SY, SY2, zmin);
          if (K == 0) break;
          const double kd = static_cast<double>(K);
          const double ymin = static_cast<double>(zmin) - Md;
          double tn;
          if (r == 1) {
            tn = (SY - 1.0) / kd;
            if (tn < ymin) { res = tn; ok = true; break; }
          } else {
            const double disc = SY * SY - kd * (SY2 - 1.0);
            if (disc >= 0.0) {
              const double ts = (SY - sqrt(disc)) / kd;
              if (ts < ymin) { res = ts; ok = true; break; }
            }
            const double F = SY2 - 2.0 * t * SY + kd * t * t;
            const double Dv = SY - kd * t;
            tn = t + (F - sqrt(F)) / Dv;
          }
          if (!(tn > t)) { res = t; ok = true; break; }
          t = tn;
        }
      }
      if (lane == 0) {
        s_wsolved = ok ? 1 : 0;
        s_wtau = res;
      }
    } else if (listed) {
      // Meanwhile the other waves bring the value rows of every candidate
      // (a superset of the support) into the L2, so that the gather after
      // the solve does not wait on memory: one 4-byte load per 128-byte line
      // of a row.  The loaded values are not used: the empty asm only keeps
      // the loads.
      constexpr int ROWB = D * static_cast<int>(sizeof(typename E::T));
      constexpr int LNR = ROWB >= 128 ? ROWB / 128 : 1;  // lines of a row
      constexpr int TPW = kWave / LNR, KP = 4;             // rows per load
      const int sub = lane / LNR, li = lane % LNR;
      int segs[NW + 1];
      segs[0] = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        segs[w + 1] = segs[w] + __builtin_amdgcn_readfirstlane(s_ccnt[w]);
      const int n_all = segs[NW];
      const int h = u % H;
      for (int e0 = (wave - 1) * TPW + sub; e0 < n_all; e0 += (NW - 1) * TPW * KP) {
        unsigned x[KP];
#pragma unroll
        for (int k = 0; k < KP; ++k) {
          // unconditional (candidates past the last repeat it), so that the
          // KP loads are in flight together
          const int e = min(e0 + k * (NW - 1) * TPW, n_all - 1);
          int w = 0, base = 0;
#pragma unroll
          for (int v = 1; v < NW; ++v)
            if (e >= segs[v]) { w = v; base = segs[v]; }
          const int pos = cpos[w * CSEG + (e - base)];
          const int slot = dslot[pos >> lgP];  // listed positions (also hinted)
          const char *row = reinterpret_cast<const char *>(
              vpool + pool_row(slot, h, pos & (P - 1), H, P, D));
          x[k] = *reinterpret_cast<const unsigned *>(row + 128 * li);
        }
#pragma unroll
        for (int k = 0; k < KP; ++k) asm volatile("" ::"v"(x[k]));
      }
    }
    lds_barrier();
    solved = s_wsolved != 0;
    t_rel = s_wtau;
  }

  // Bin width: the smallest power of two w with NB * w >= M - L.
  double w = 1.0;
  for (int it = 0; it < 64 && w * kTauBins < Md - L; ++it) w *= 2.0;
  for (int it = 0; it < 64 && w * 0.5 * kTauBins >= Md - L; ++it) w *= 0.5;
  const double inv_w = 1.0 / w;
  auto bin_of = [&](float z) {  // z > L on entry
    const double x = floor((static_cast<double>(z) - L) * inv_w);
    return x < kTauBins ? (x > 0.0 ? static_cast<int>(x) : 0) : kTauBins - 1;
  };

  if (!solved && (r == 1 || r == 2)) {
    for (int i = tid; i < kTauBins; i += kTauThreads) hist[i] = 0u;
    lds_barrier();
    for_candidates([&](float z) { atomicAdd(&hist[bin_of(z)], 1u); });
    lds_barrier();
    constexpr int BPT = kTauBins / kTauThreads;
    double l0 = 0, l1 = 0, l2 = 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const double cb = tid * BPT + k, nn = hist[tid * BPT + k];
      l0 += nn; l1 += nn * cb; l2 += nn * cb * cb;
    }
    const double i0 = block_incl_scan_d<kTauThreads>(l0, red_d);
    const double i1 = block_incl_scan_d<kTauThreads>(l1, red_d);
    const double i2 = block_incl_scan_d<kTauThreads>(l2, red_d);
    if (tid == kTauThreads - 1) { s_tot[0] = i0; s_tot[1] = i1; s_tot[2] = i2; }
    lds_barrier();
    double S0 = s_tot[0] - i0, S1 = s_tot[1] - i1, S2 = s_tot[2] - i2;
    // F_lo(b) >= 1  <=>  sum cnt (c-b)^r >= w^-r
    const double need = (r == 2) ? inv_w * inv_w : inv_w;
    int my_lo = 0, my_hi = kTauBins;  // F_hi at the top edge is <= 0 < 1
    for (int k = BPT - 1; k >= 0; --k) {
      const double bb = tid * BPT + k, nn = hist[tid * BPT + k];
      S0 += nn; S1 += nn * bb; S2 += nn * bb * bb;
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
    blo = L + b_lo * w;
    bhi = fmin(Md, L + b_hi * w);

    long long nfix = 0, sy = 0, sy2 = 0;
    for_candidates([&](float z) {
      const int bn = bin_of(z);
      if (bn >= b_hi) {
        const double y = static_cast<double>(z) - Md;
        ++nfix; sy += fixp(y); sy2 += fixp(y * y);
      } else if (bn >= b_lo) {
        const int slot = atomicAdd(&s_nlist, 1);
        if (slot < kTauList) list[slot] = z;
      }
    });
    nfix = block_sum_ll<kTauThreads>(nfix, red_ll);
    sy = block_sum_ll<kTauThreads>(sy, red_ll);
    sy2 = block_sum_ll<kTauThreads>(sy2, red_ll);
    const int nl = s_nlist;  // final: block_sum_ll ends with a barrier
    if (nl <= kTauList) {
      const double ylo_floor = blo - Md;             // untracked values are below
      const double ybound_hi = (L + b_hi * w) - Md;  // certain values are >= this
      int bestK = -1;
      double best_t = 0.0;
      for (int j = tid; j <= nl; j += kTauThreads) {
        const float zj = j < nl ? list[j] : 0.f;
        long long K = nfix, SY = sy, SY2 = sy2;
        double ynext = ylo_floor;
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
      if (K_all >= 0 && bestK == K_all) s_best_t = best_t;
      lds_barrier();
      if (K_all >= 0) {
        t_rel = s_best_t;
        solved = true;
      }
    }
  }
  if (!solved) {
    // Bisection in double on [blo, bhi] over the candidates.
    double lo = blo, hi = bhi;
    for (int it = 0; it < 64 && hi - lo > 1e-12 * fmax(1.0, fabs(hi)); ++it) {
      const double mid = 0.5 * (lo + hi);
      double fsum = 0.0;
      for_candidates([&](float z) {
        const double d = static_cast<double>(z) - mid;
        if (d > 0.0)
          fsum += (r == 1) ? d : (r == 2) ? d * d
                                          : pow(d, static_cast<double>(rg));
      });
      fsum = block_sum_d<kTauThreads>(fsum, red_d);
      if (fsum >= 1.0) lo = mid; else hi = mid;
    }
    t_rel = 0.5 * (lo + hi) - Md;
  }
  const float tau = static_cast<float>(Md + t_rel);
  if (tid == 0) {
    tau_ws[ug] = tau;
    if (tau_user) tau_user[ug] = tau;
  }

  // Weighted value sum over the support, p = max(z - tau, 0)^r as in the
  // chunked path, value rows gathered through the page table.  Each wave
  // compacts (p, position) of support tokens into its own LDS segment and
  // reads their rows with D/8 lanes per row and many rows in flight.  When
  // every candidate is staged the support is among them and is compacted in
  // place; otherwise, with a selection, the wave walks its share of the
  // kept pages again and gathers whenever its segment fills.  Sums run in a
  // fixed order, so the result is the same on every run.  Only the full
  // cache (no selection) leaves such heads to the apply step, whose per-unit
  // chunk counter is reset here for it.
  if (tid == 0 && ug % G == 0) ctr[u] = 0;
  if (!staged && sel == nullptr) {
    if (tid == 0) {
      done[ug] = 0;
      atomicAdd(undone, 1);
    }
    return;
  }
  constexpr int LPT = D / 8, TPW = kWave / LPT, RU = 8;
  const int h = u % H;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  float *seg_p = cand + wave * CSEG;
  int *seg_pos = cpos + wave * CSEG;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  float psum = 0.f;
  // adds sum p v over entries [0, n) of the wave's segment
  auto gather = [&](int n) {
    for (int base = 0; base < n; base += TPW * RU) {
      float x[RU][8];
      float pw[RU];
#pragma unroll
      for (int rr = 0; rr < RU; ++rr) {
        // unconditional loads (entries past n repeat entry n - 1, with
        // weight 0), all in flight together
        const int k = base + rr * TPW + sub;
        const int kc = min(k, n - 1);
        pw[rr] = k < n ? seg_p[kc] : 0.f;
        const int pos = seg_pos[kc];
        const int jj = pos >> lgP, t = pos & (P - 1);
        const int slot =
            listed ? dslot[jj] : slots[static_cast<size_t>(u) * max_pages + jj];
        load8(vpool + pool_row(slot, h, t, H, P, D) + d0, x[rr]);
      }
#pragma unroll
      for (int rr = 0; rr < RU; ++rr) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(pw[rr], x[rr][j], acc[j]);
        if (li == 0) psum += pw[rr];
      }
    }
  };
  if (staged) {
    int nk = 0;
    const int nc = s_ccnt[wave];
    for (int i0 = 0; i0 < nc; i0 += kWave) {
      const int i = i0 + lane;
      float pv = 0.f;
      int pos = 0;
      if (i < nc) {
        pv = pow_r(fmaxf(seg_p[i] - tau, 0.f), r, rg);
        pos = seg_pos[i];
      }
      const bool keep = pv > 0.f;
      const unsigned long long ball = __ballot(keep);
      if (keep) {
        const int k = nk + __popcll(ball & below);
        seg_p[k] = pv;  // k <= i: written after this chunk's reads
        seg_pos[k] = pos;
      }
      nk += __popcll(ball);
    }
    gather(nk);
  } else {
    // Steps of 4 kWave / P listed pages (4 scores per lane), dealt to the
    // waves in turn, US at a time; a step adds at most 4 kWave entries.
    constexpr int US = CSEG >= 2 * 2 * 4 * kWave ? 2 : 1;
    static_assert(CSEG >= 2 * US * 4 * kWave, "segment holds two passes");
    const int lpp = P / 4, ppw = kWave / lpp;
    const int sp = lane / lpp, t4 = 4 * (lane - sp * lpp);
    const int steps = (n_pg + ppw - 1) / ppw;
    int nk = 0;
    for (int s0 = wave; s0 < steps; s0 += NW * US) {
      float4 zv[US];
#pragma unroll
      for (int k = 0; k < US; ++k) {
        const int jj = (s0 + k * NW) * ppw + sp;
        zv[k] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (jj < n_pg) {
          const int j = page_of(jj);
          if (pm[j] > tau)
            zv[k] = *reinterpret_cast<const float4 *>(zh + static_cast<size_t>(j) * P + t4);
        }
      }
#pragma unroll
      for (int k = 0; k < US; ++k) {
        const int jj = (s0 + k * NW) * ppw + sp;
        const float ze[4] = {zv[k].x, zv[k].y, zv[k].z, zv[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = pow_r(fmaxf(ze[e] - tau, 0.f), r, rg);
          const bool keep = pv > 0.f;
          const unsigned long long ball = __ballot(keep);
          if (keep) {
            const int kk = nk + __popcll(ball & below);
            seg_p[kk] = pv;
            seg_pos[kk] = jj * P + t4 + e;
          }
          nk += __popcll(ball);
        }
      }
      if (nk > CSEG - US * 4 * kWave) {  // uniform
        gather(nk);
        nk = 0;
      }
    }
    gather(nk);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v = acc[j];
#pragma unroll
    for (int o = LPT; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
    acc[j] = v;
  }
  psum = group_sum<kWave>(psum);
  if (sub == 0)
#pragma unroll
    for (int j = 0; j < 8; ++j) s_vacc[wave][d0 + j] = acc[j];
  if (lane == 0) s_vsum[wave] = psum;
  lds_barrier();
  float psum_all = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) psum_all += s_vsum[w];
  for (int d = tid; d < D; d += kTauThreads) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += s_vacc[w][d];
    out[static_cast<size_t>(ug) * D + d] = v / psum_all;
  }
  if (tid == 0) done[ug] = 1;
}

// ---------------------------------------------------------------------------
// Chunks: kChunkTokens token positions (kChunkTokens / P pages) of one unit.
// ---------------------------------------------------------------------------
struct ChunkPages {
  int lp[kMaxChunkPages];
  int slot[kMaxChunkPages];
  int nt[kMaxChunkPages];
};

// Stages the pages of chunk c of unit u; returns the number of pages.
__device__ __forceinline__ int stage_chunk(ChunkPages &cp,
                                           const int32_t *page_table,
                                           const int32_t *seq_lens,
                                           const int32_t *sel, int u, int c,
                                           int cnt, int H, int P,
                                           int max_pages) {
  const int b = u / H;
  const int ppc = kChunkTokens / P;
  const int j0 = c * ppc;
  const int npg = min(cnt - j0, ppc);
  if (threadIdx.x < npg) {
    const int j = j0 + threadIdx.x;
    const int lp = sel ? sel[static_cast<size_t>(u) * max_pages + j] : j;
    cp.lp[threadIdx.x] = lp;
    cp.slot[threadIdx.x] = page_table[static_cast<size_t>(b) * max_pages + lp];
    cp.nt[threadIdx.x] = page_tokens(lp, seq_lens[b], P);
  }
  return npg;
}

// ---------------------------------------------------------------------------
// 3a. Apply: chunk partials of sum_i p_i v_i and sum_i p_i.  Persistent
// blocks over the chunks of the units the threshold step did not finish.
// A chunk none of whose pages has a maximum above tau for any head only
// records a zero partial.  Otherwise p is computed once per (token, head)
// into LDS from the z of the chunk's active pages, the rows with some p > 0
// are compacted, and all their value loads are issued together.  The block
// that completes a unit's last chunk merges the unit's partials.
// ---------------------------------------------------------------------------
constexpr int kRowUnroll = 4;

// Merge of one unit's chunk partials: out = sum_c o_c / sum_c s_c over the
// chunks with some p > 0 (the others add exact zeros), in chunk order, for
// every query head not already finished by the threshold step.  One block;
// `list` holds kChunkTokens ints and `tmp` kDecWaves ints.
template <int G, int D>
__device__ void merge_unit_partials(int u, int nch, int maxch,
                                    const float *part_o, const float *part_s,
                                    const int32_t *done, float *out, int *list,
                                    int *tmp) {
  int nact = 0;
  for (int base = 0; base < nch; base += kDecThreads) {
    const int c = base + threadIdx.x;
    bool flag = false;
    if (c < nch)
#pragma unroll
      for (int g = 0; g < G; ++g)
        flag |= part_s[(static_cast<size_t>(u) * maxch + c) * G + g] > 0.f;
    int tot;
    const int rk = tile_rank<kDecThreads>(flag, tmp, tot);
    if (flag && nact + rk < kChunkTokens) list[nact + rk] = c;
    nact += tot;
  }
  lds_barrier();
  const bool listed = nact <= kChunkTokens;
  const int n = listed ? nact : nch;
  for (int e = threadIdx.x; e < G * D; e += kDecThreads) {
    const int g = e / D, d = e - g * D;
    if (done && done[u * G + g]) continue;
    float o = 0.f, sum = 0.f;
    for (int k = 0; k < n; ++k) {
      const int c = listed ? list[k] : k;
      const size_t cb = static_cast<size_t>(u) * maxch + c;
      o += part_o[(cb * G + g) * D + d];
      sum += part_s[cb * G + g];
    }
    out[(static_cast<size_t>(u) * G + g) * D + d] = o / sum;
  }
}

template <class E, int D, int G>
__global__ __launch_bounds__(kDecThreads) void k_entmax_apply(
    const typename E::T *__restrict__ vpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, int units, int H, int P, int max_pages,
    int cap, int maxch, int r, float rg, const float *__restrict__ zbuf,
    const float *__restrict__ pmax, const float *__restrict__ tau,
    float *__restrict__ part_o, float *__restrict__ part_s,
    float *__restrict__ probs, const int32_t *__restrict__ done,
    int32_t *__restrict__ ctr, const int32_t *__restrict__ undone,
    float *__restrict__ out) {
  constexpr int LPT = D / 8;
  constexpr int TPW = kWave / LPT;
  constexpr int ROWS_STEP = kDecWaves * TPW * kRowUnroll;
  // Nothing to do when the threshold step finished every head.
  if (done && *undone == 0) return;
  __shared__ int pref[kMaxUnits + 1];
  __shared__ int tmp[kDecWaves];
  __shared__ ChunkPages cp;
  __shared__ int s_act[kMaxChunkPages];
  __shared__ float s_p[G][kChunkTokens];
  __shared__ int s_rows[kChunkTokens];
  __shared__ float s_acc[kDecWaves][G][D];
  __shared__ float s_sp[kDecWaves][G];
  __shared__ int s_last;
  const int ppc = kChunkTokens / P;
  // Units whose query heads were all finished by the threshold step are
  // skipped (done == NULL: none is).
  const int total = build_unit_prefix<kDecThreads>(
      pref, tmp, seq_lens, sel, count, units, H, P, ppc, done, G);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  const int Hq = H * G;
  const size_t pstride = static_cast<size_t>(max_pages) * P;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int u = find_unit(pref, units, w);
    const int c = w - pref[u];
    const int h = u % H, b = u / H;
    const int cnt = unit_pages(seq_lens, sel, count, u, H, P);
    const int j0 = c * ppc;
    const int npg = min(cnt - j0, ppc);
    // Active pages: some head's page maximum above its tau.
    bool act = false;
    if (threadIdx.x < npg) {
      const int jj = threadIdx.x;
#pragma unroll
      for (int g = 0; g < G; ++g)
        act |= pmax[(static_cast<size_t>(u) * G + g) * pm_stride(max_pages) + j0 + jj] >
               tau[u * G + g];
      s_act[jj] = act;
    }
    if (__syncthreads_or(act)) {
    stage_chunk(cp, page_table, seq_lens, sel, u, c, cnt, H, P, max_pages);
    float tg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) tg[g] = tau[u * G + g];
    lds_barrier();
    const int npos = npg * P;
    const float *zu = zbuf + static_cast<size_t>(u) * G * cap +
                      static_cast<size_t>(j0) * P;
    // p for every position of the chunk (zero outside active pages).
    float spl[G];
#pragma unroll
    for (int g = 0; g < G; ++g) spl[g] = 0.f;
    int n_rows = 0;
    for (int base = 0; base < kChunkTokens; base += kDecThreads) {
      const int i = base + threadIdx.x;
      const int jj = i / P, t = i - jj * P;
      const bool on = i < npos && s_act[jj] && t < cp.nt[jj];
      float pv[G];
      bool any = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        pv[g] = 0.f;
        if (on) pv[g] = pow_r(fmaxf(zu[static_cast<size_t>(g) * cap + i] - tg[g], 0.f), r, rg);
        s_p[g][i] = pv[g];
        spl[g] += pv[g];
        any |= pv[g] > 0.f;
      }
      if (probs && on) {
        const size_t tok = static_cast<size_t>(cp.lp[jj]) * P + t;
#pragma unroll
        for (int g = 0; g < G; ++g)
          probs[(static_cast<size_t>(b) * Hq + h * G + g) * pstride + tok] = pv[g];
      }
      int tot;
      const int rk = tile_rank<kDecThreads>(any, tmp, tot);
      if (any) s_rows[n_rows + rk] = i;
      n_rows += tot;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sg = group_sum<kWave>(spl[g]);
      if (lane == 0) s_sp[wave][g] = sg;
    }
    lds_barrier();
    // Value rows with some p > 0: LPT lanes per row, all loads in flight.
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
    for (int base = 0; base < n_rows; base += ROWS_STEP) {
      float x[kRowUnroll][8];
      int ri[kRowUnroll];
#pragma unroll
      for (int rr = 0; rr < kRowUnroll; ++rr) {
        const int k = base + (rr * kDecWaves + wave) * TPW + sub;
        ri[rr] = k < n_rows ? s_rows[k] : -1;
        if (ri[rr] >= 0) {
          const int jj = ri[rr] / P, t = ri[rr] - jj * P;
          load8(vpool + pool_row(cp.slot[jj], h, t, H, P, D) + d0, x[rr]);
        }
      }
#pragma unroll
      for (int rr = 0; rr < kRowUnroll; ++rr)
        if (ri[rr] >= 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pw = s_p[g][ri[rr]];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[g][j] = fmaf(pw, x[rr][j], acc[g][j]);
          }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[g][j];
#pragma unroll
        for (int o = LPT; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
        acc[g][j] = v;
      }
    if (sub == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) s_acc[wave][g][d0 + j] = acc[g][j];
    }
    lds_barrier();
    float *po = part_o + (static_cast<size_t>(u) * maxch + c) * G * D;
    for (int e = threadIdx.x; e < G * D; e += kDecThreads) {
      const int g = e / D, d = e % D;
      float v = s_acc[0][g][d];
#pragma unroll
      for (int ww = 1; ww < kDecWaves; ++ww) v += s_acc[ww][g][d];
      po[e] = v;
    }
    if (threadIdx.x < G) {
      float v = s_sp[0][threadIdx.x];
#pragma unroll
      for (int ww = 1; ww < kDecWaves; ++ww) v += s_sp[ww][threadIdx.x];
      part_s[(static_cast<size_t>(u) * maxch + c) * G + threadIdx.x] = v;
    }
    } else if (threadIdx.x < G) {  // no page of the chunk can hold p > 0
      part_s[(static_cast<size_t>(u) * maxch + c) * G + threadIdx.x] = 0.f;
    }
    // The block that finishes the unit's last chunk merges its partials
    // (in chunk order) into out.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = atomicAdd(&ctr[u], 1) == pref[u + 1] - pref[u] - 1;
    __syncthreads();
    if (s_last) {
      __threadfence();
      merge_unit_partials<G, D>(u, pref[u + 1] - pref[u], maxch, part_o, part_s,
                                done, out, s_rows, tmp);
      if (threadIdx.x == 0) ctr[u] = 0;
    }
    __syncthreads();  // LDS of this chunk is reused by the next one
  }
}

// ---------------------------------------------------------------------------
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
// Split-K softmax over float32 K/V (bfloat16 K/V stream through softmax.hip).
// Persistent blocks over chunks: scores into LDS, the chunk maximum m, the
// weights exp(s - m) once per (token, head), then the weighted value sum on
// the vector units.  The chunk partials (m, l, acc) are merged in
// log-sum-exp form.
// ---------------------------------------------------------------------------
template <class E, int D, int G>
__device__ __forceinline__ void chunk_scores_valu(
    const ChunkPages &cp, const typename E::T *kpool, const float *q, int b,
    int h, int H, int P, int npos, float scale, float (*s_sc)[kChunkTokens]) {
  constexpr int LPT = D / 8;
  constexpr int TPW = kWave / LPT;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  const int Hq = H * G;
  float qs[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      qs[g][j] = q[(static_cast<size_t>(b) * Hq + h * G + g) * D + d0 + j] * scale;
  for (int i0 = wave * TPW; i0 < kChunkTokens; i0 += kDecWaves * TPW) {
    const int i = i0 + sub;
    const int jj = i / P, t = i - jj * P;
    const bool valid = i < npos && t < cp.nt[jj < kMaxChunkPages ? jj : 0];
    float x[8];
    if (valid) {
      load8(kpool + pool_row(cp.slot[jj], h, t, H, P, D) + d0, x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fmaf(qs[g][j], x[j], a);
      a = group_sum<LPT>(a);
      if (li == g) s_sc[g][i] = valid ? a : -INFINITY;
    }
  }
}

// Eight consecutive elements kept packed until use (fewer registers while
// many rows are in flight).
template <class E>
struct Packed8;
template <>
struct Packed8<BF16> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t *p) {
    w = *reinterpret_cast<const uint4 *>(p);
  }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
};
template <>
struct Packed8<F32> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

template <class E, int D, int G>
__global__ __launch_bounds__(kDecThreads) void k_softmax_partial(
    const typename E::T *__restrict__ kpool,
    const typename E::T *__restrict__ vpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, const float *__restrict__ q,
    float scale, int units, int H, int P, int max_pages, int maxch,
    float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_o) {
  constexpr int LPT = D / 8;
  constexpr int TPW = kWave / LPT;
  constexpr int VSTEP = 256;                      // value rows per sub-tile
  constexpr int VUN = VSTEP / (kDecWaves * TPW);  // rows per lane in flight
  __shared__ int pref[kMaxUnits + 1];
  __shared__ int tmp[kDecWaves];
  __shared__ ChunkPages cp;
  __shared__ float s_sc[G][kChunkTokens];
  __shared__ float s_acc[kDecWaves][G][D];
  __shared__ float red[kDecWaves][G];
  const int ppc = kChunkTokens / P;
  const int total = build_unit_prefix<kDecThreads>(pref, tmp, seq_lens, sel,
                                                   count, units, H, P, ppc);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int u = find_unit(pref, units, w);
    const int c = w - pref[u];
    const int h = u % H, b = u / H;
    const int cnt = unit_pages(seq_lens, sel, count, u, H, P);
    const int npg = stage_chunk(cp, page_table, seq_lens, sel, u, c, cnt, H, P,
                                max_pages);
    lds_barrier();
    const int npos = npg * P;
    chunk_scores_valu<E, D, G>(cp, kpool, q, b, h, H, P, npos, scale, s_sc);
    lds_barrier();
    // chunk maximum per head, then the weights and their sum
    float m[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = -FLT_MAX;
      for (int i = threadIdx.x; i < kChunkTokens; i += kDecThreads)
        x = fmaxf(x, s_sc[g][i]);
      x = group_max<kWave>(x);
      if (lane == 0) red[wave][g] = x;
    }
    lds_barrier();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = red[0][g];
#pragma unroll
      for (int ww = 1; ww < kDecWaves; ++ww) m[g] = fmaxf(m[g], red[ww][g]);
    }
    lds_barrier();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = 0.f;
      for (int i = threadIdx.x; i < kChunkTokens; i += kDecThreads) {
        const float pw = expf(s_sc[g][i] - m[g]);  // exp(-inf) = 0
        s_sc[g][i] = pw;
        x += pw;
      }
      x = group_sum<kWave>(x);
      if (lane == 0) red[wave][g] = x;
    }
    lds_barrier();
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
    for (int base = 0; base < npos; base += VSTEP) {
      Packed8<E> x[VUN];
      bool valid[VUN];
      int pos[VUN];
#pragma unroll
      for (int rr = 0; rr < VUN; ++rr) {
        const int i = base + (rr * kDecWaves + wave) * TPW + sub;
        const int jj = i / P, t = i - jj * P;
        pos[rr] = i;
        valid[rr] = i < npos && t < cp.nt[jj < kMaxChunkPages ? jj : 0];
        if (valid[rr]) x[rr].load(vpool + pool_row(cp.slot[jj], h, t, H, P, D) + d0);
      }
#pragma unroll
      for (int rr = 0; rr < VUN; ++rr) {
        if (valid[rr]) {
          float xv[8];
          x[rr].unpack(xv);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pw = s_sc[g][pos[rr]];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[g][j] = fmaf(pw, xv[j], acc[g][j]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[g][j];
#pragma unroll
        for (int o = LPT; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
        acc[g][j] = v;
      }
    if (sub == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) s_acc[wave][g][d0 + j] = acc[g][j];
    }
    lds_barrier();
    const size_t pc = static_cast<size_t>(u) * maxch + c;
    float *po = part_o + pc * G * D;
    for (int e = threadIdx.x; e < G * D; e += kDecThreads) {
      const int g = e / D, d = e % D;
      float v = s_acc[0][g][d];
#pragma unroll
      for (int ww = 1; ww < kDecWaves; ++ww) v += s_acc[ww][g][d];
      po[e] = v;
    }
    if (threadIdx.x < G) {
      float v = red[0][threadIdx.x];
#pragma unroll
      for (int ww = 1; ww < kDecWaves; ++ww) v += red[ww][threadIdx.x];
      part_l[pc * G + threadIdx.x] = v;
      part_m[pc * G + threadIdx.x] = m[threadIdx.x];
    }
    lds_barrier();
  }
}

// Merge: grid (units*G, D/kCombD); kCombSlices slices of chunks per block.
constexpr int kCombD = 16;
constexpr int kCombSlices = 64;

__global__ __launch_bounds__(kCombD * kCombSlices) void k_softmax_combine(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, int H, int G, int D, int P, int maxch,
    const float *__restrict__ part_m, const float *__restrict__ part_l,
    const float *__restrict__ part_o, float *__restrict__ out,
    float *__restrict__ lse) {
  constexpr int NT = kCombD * kCombSlices;
  __shared__ float red_f[NT / kWave];
  __shared__ float s_o[kCombSlices][kCombD];
  __shared__ float s_l[kCombSlices];
  const int ug = blockIdx.x, u = ug / G, g = ug % G;
  const int tid = threadIdx.x;
  const int cnt = unit_pages(seq_lens, sel, count, u, H, P);
  const int ppc = kChunkTokens / P;
  const int nch = (cnt + ppc - 1) / ppc;
  const size_t ub = static_cast<size_t>(u) * maxch;
  float mloc = -FLT_MAX;
  for (int c = tid; c < nch; c += NT) mloc = fmaxf(mloc, part_m[(ub + c) * G + g]);
  const float M = block_max<NT>(mloc, red_f);
  const int dl = tid % kCombD, sl = tid / kCombD;
  const int d = blockIdx.y * kCombD + dl;
  float o = 0.f, l = 0.f;
#pragma unroll 4
  for (int c = sl; c < nch; c += kCombSlices) {
    const size_t base = (ub + c) * G + g;
    const float wgt = expf(part_m[base] - M);
    o = fmaf(wgt, part_o[base * D + d], o);
    l = fmaf(wgt, part_l[base], l);
  }
  s_o[sl][dl] = o;
  if (dl == 0) s_l[sl] = l;
  lds_barrier();
  if (tid < kCombD) {
    float oo = 0.f, ll = 0.f;
    for (int k = 0; k < kCombSlices; ++k) {
      oo += s_o[k][tid];
      ll += s_l[k];
    }
    out[static_cast<size_t>(ug) * D + blockIdx.y * kCombD + tid] = oo / ll;
    if (lse && blockIdx.y == 0 && tid == 0) lse[ug] = M + logf(ll);
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
hipError_t launch_entmax_threshold(const ekv_paged_kv &kv, float alpha,
                                   const int32_t *sel, const int32_t *count,
                                   float *tau, float *out, void *ws,
                                   hipStream_t stream) {
  const DecodeWs L = decode_ws_layout(kv);
  char *w = static_cast<char *>(ws);
  float rg;
  const int r = exponent_code(alpha, rg);
  // one block per query head: with more heads than CUs the half-capacity
  // form lets two blocks share a CU
  const int n_heads = kv.batch * kv.num_kv_heads * G;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n_cu <= 0)
    n_cu = 256;
  auto kern = n_heads > n_cu ? k_entmax_tau<E, D, true> : k_entmax_tau<E, D, false>;
  hipLaunchKernelGGL(kern, dim3(n_heads), dim3(kTauThreads), 0, stream,
                     reinterpret_cast<float *>(w + L.z),
                     reinterpret_cast<float *>(w + L.cmax),
                     static_cast<const typename E::T *>(kv.v),
                     static_cast<const typename E::T *>(kv.k), kv.page_table,
                     kv.seq_lens, sel, count, kv.num_kv_heads, G, kv.page_size,
                     kv.max_pages, kv.max_pages * kv.page_size, r, rg,
                     reinterpret_cast<float *>(w + L.tau), tau, out,
                     reinterpret_cast<int32_t *>(w + L.done),
                     reinterpret_cast<int32_t *>(w + L.ctr),
                     reinterpret_cast<const int32_t *>(w + L.slot),
                     reinterpret_cast<int32_t *>(w + L.ctr) + kv.batch * kv.num_kv_heads,
                     reinterpret_cast<const float *>(w + L.floor),
                     reinterpret_cast<const float *>(w + L.qz),
                     reinterpret_cast<const unsigned long long *>(w + L.mask));
  return hipGetLastError();
}

template <class E, int D, int G>
hipError_t launch_entmax_apply(const ekv_paged_kv &kv, float alpha,
                               const int32_t *sel, const int32_t *count,
                               float *out, float *probs, void *ws,
                               hipStream_t stream) {
  // With a selection the threshold step has written every row of out.
  if (sel && !probs) return hipSuccess;
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
  // With the debug probabilities every chunk is visited (they are written
  // there); otherwise heads finished by the threshold step are skipped.
  const int32_t *done =
      probs ? nullptr : reinterpret_cast<const int32_t *>(w + L.done);
  const int blocks = persistent_blocks(static_cast<size_t>(units) * mc, 4);
  hipLaunchKernelGGL((k_entmax_apply<E, D, G>), dim3(blocks),
                     dim3(kDecThreads), 0, stream,
                     static_cast<const typename E::T *>(kv.v), kv.page_table,
                     kv.seq_lens, sel, count, units, kv.num_kv_heads,
                     kv.page_size, kv.max_pages, kv.max_pages * kv.page_size,
                     mc, r, rg, reinterpret_cast<const float *>(w + L.z),
                     reinterpret_cast<const float *>(w + L.cmax),
                     reinterpret_cast<const float *>(w + L.tau),
                     reinterpret_cast<float *>(w + L.part_o),
                     reinterpret_cast<float *>(w + L.part_s), probs, done,
                     reinterpret_cast<int32_t *>(w + L.ctr),
                     reinterpret_cast<const int32_t *>(w + L.ctr) + units, out);
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
  const int blocks = persistent_blocks(static_cast<size_t>(units) * mc, 4);
  if constexpr (sizeof(typename E::T) == 2) {
    return launch_softmax_stream<D, G>(
        kv, q, scale, sel, count, out, lse, reinterpret_cast<float *>(w + L.part_m),
        reinterpret_cast<float *>(w + L.part_l), reinterpret_cast<float *>(w + L.part_o),
        reinterpret_cast<int32_t *>(w + L.seg), stream);
  } else
  hipLaunchKernelGGL((k_softmax_partial<E, D, G>), dim3(blocks),
                     dim3(kDecThreads), 0, stream,
                     static_cast<const typename E::T *>(kv.k),
                     static_cast<const typename E::T *>(kv.v), kv.page_table,
                     kv.seq_lens, sel, count, q, scale, units, kv.num_kv_heads,
                     kv.page_size, kv.max_pages, mc,
                     reinterpret_cast<float *>(w + L.part_m),
                     reinterpret_cast<float *>(w + L.part_l),
                     reinterpret_cast<float *>(w + L.part_o));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_softmax_combine, dim3(units * G, D / kCombD),
                     dim3(kCombD * kCombSlices), 0, stream, kv.seq_lens, sel,
                     count, kv.num_kv_heads, G, D, kv.page_size, mc,
                     reinterpret_cast<const float *>(w + L.part_m),
                     reinterpret_cast<const float *>(w + L.part_l),
                     reinterpret_cast<const float *>(w + L.part_o), out, lse);
  return hipGetLastError();
}

#define EKV_INST_DEC(E, D, G)                                                \
  template hipError_t launch_entmax_threshold<E, D, G>(                      \
      const ekv_paged_kv &, float, const int32_t *, const int32_t *, float *, \
      float *, void *, hipStream_t);                                         \
  template hipError_t launch_entmax_apply<E, D, G>(                          \
      const ekv_paged_kv &, float, const int32_t *, const int32_t *, float *, \
      float *, void *, hipStream_t);                                         \
  template hipError_t launch_softmax<E, D, G>(                               \
      const ekv_paged_kv &, const float *, float, const int32_t *,           \
      const int32_t *, float *, float *, void *, hipStream_t);
EKV_FOR_EACH_EDG(EKV_INST_DEC)


}  // namespace ekv
