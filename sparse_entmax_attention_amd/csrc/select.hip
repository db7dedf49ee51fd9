// Candidate selection (Technical Summary: EntmaxKV, §2.B).
//
//  * Top-k (§2.B.1): per unit, rank pages by the largest box bound over the
//    unit's query heads and keep the k best (ties to the lower page index).
//  * Gaussian-aware (§2.B.2): per query head, the threshold estimate tau_hat
//    solves sum_p n_p E[max(Z_p - tau, 0)^r] = 1 over page score Gaussians;
//    per unit, pages whose estimated largest score clears tau_hat - delta for
//    some query head are kept.
//
// Both read the 64-page tile summaries written by the scoring kernel and
// look at the pages of a tile only when its summary says the tile can
// matter, which removes most of the pages of a long context from the work.
#include <float.h>

#include "ekv_device.h"
#include "ekv_kernels.h"
#include "gauss_rule.h"

namespace ekv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// Order-preserving map float -> uint32 (larger float, larger key).  -0 is
// folded onto +0 so that the two compare equal, as they do as floats.  Every
// non-NaN float maps above 0, which is used as "no page".
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest unsigned value over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_max_u(uint32_t x) {
  x = max(x, static_cast<uint32_t>(dpp_i<kDppRowMirror>(static_cast<int>(x))));
  x = max(x, static_cast<uint32_t>(dpp_i<kDppRowHalfMirror>(static_cast<int>(x))));
  x = max(x, static_cast<uint32_t>(dpp_i<kDppQuad2301>(static_cast<int>(x))));
  x = max(x, static_cast<uint32_t>(dpp_i<kDppQuad1032>(static_cast<int>(x))));
  x = max(x, static_cast<uint32_t>(dpp_rows<kDppRowBcast15, 0xA>(static_cast<int>(x),
                                                                static_cast<int>(x))));
  x = max(x, static_cast<uint32_t>(dpp_rows<kDppRowBcast31, 0xC>(static_cast<int>(x),
                                                                static_cast<int>(x))));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), kWave - 1));
}

// Ordered list of the indices i < n with pred(i), written to out (at most
// cap entries are stored); returns the count.  Rounds of one index per
// thread; contains barriers.
template <class F>
__device__ int ordered_list(int n, F pred, int *out, int cap, int *tmp) {
  int total = 0;
  for (int base = 0; base < n; base += kSelThreads) {
    const int i = base + threadIdx.x;
    const bool flag = i < n && pred(i);
    int tot;
    const int rk = tile_rank<kSelThreads>(flag, tmp, tot);
    if (flag && total + rk < cap) out[total + rk] = i;
    total += tot;
  }
  return total;
}

// kk-th largest of n keys key_at(i) (kk <= n): returns the key T, in need
// how many keys equal to T belong to the kk largest, and in n_at how many
// keys equal T.  Most significant digit first, 8 bits per pass, from the
// digit at bit shift_hi down to the one at shift_lo (the bits below shift_lo
// are returned as 0, a lower bound of T); keys whose bits above shift_hi + 7
// differ from prefix0 are left out (the caller knows every key of the kk
// largest has them).  hist holds two 256-bin
// histograms and s_digit / s_need (need, count) two slots, used in turn, so that a pass
// needs two barriers: one after its histogram (then wave 0 finds the digit
// while the other waves clear the next histogram), one after the digit.
// A wave whose keys all share the digit adds them with one atomic.
// Contains barriers.
template <class F>
__device__ uint32_t radix_select(F key_at, int n, int kk, int *hist,
                                 uint32_t *s_digit, int *s_need, int &need,
                                 int &n_at, int shift_hi = 24, int shift_lo = 0,
                                 uint32_t prefix0 = 0u) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t mask = shift_hi >= 24 ? 0u : ~((256u << shift_hi) - 1u);
  uint32_t prefix = prefix0 & mask;
  need = kk;
  for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
  lds_barrier();
  int pass = 0;
  n_at = 0;
  for (int shift = shift_hi; shift >= shift_lo; shift -= 8, ++pass) {
    int *hc = hist + 256 * (pass & 1), *hn = hist + 256 * ((pass + 1) & 1);
    for (int base = 0; base < n; base += kSelThreads) {
      const int i = base + threadIdx.x;
      const uint32_t key = i < n ? key_at(i) : 0u;
      const bool act = i < n && (key & mask) == prefix;
      const uint32_t dg = (key >> shift) & 255u;
      const unsigned long long on = __ballot(act);
      if (on) {
        const int first = __ffsll(static_cast<long long>(on)) - 1;
        const uint32_t d0 = static_cast<uint32_t>(
            __builtin_amdgcn_readlane(static_cast<int>(dg), first));
        if ((__ballot(act && dg != d0)) == 0ull) {
          if (lane == first) atomicAdd(&hc[d0], __popcll(on));
        } else if (act) {
          atomicAdd(&hc[dg], 1);
        }
      }
    }
    lds_barrier();
    if (threadIdx.x < kWave) {
      // Lane l owns digits 255-4l .. 252-4l (descending).
      int c[4], local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hc[255 - 4 * lane - j];
        local += c[j];
      }
      const int incl = wave_incl_scan(local);
      int before = incl - local;  // keys with a larger digit
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < need && before + c[j] >= need) {
          s_digit[pass & 1] = static_cast<uint32_t>(255 - 4 * lane - j);
          s_need[pass & 1] = need - before;
          s_need[2 + (pass & 1)] = c[j];
        }
        before += c[j];
      }
    } else {
      for (int i = threadIdx.x - kWave; i < 256; i += kSelThreads - kWave) hn[i] = 0;
    }
    lds_barrier();
    prefix |= s_digit[pass & 1] << shift;
    mask |= 255u << shift;
    need = s_need[pass & 1];
    n_at = s_need[2 + (pass & 1)];
  }
  return prefix;
}

// ---------------------------------------------------------------------------
// Top-k.  One block per unit.
//   1. T0 = the k-th largest tile maximum.  k tiles reach T0, each through
//      a page of its own, so the k-th largest page bound is >= T0 and only
//      tiles whose maximum is >= T0 can hold a selected page.
//   2. The pages of those tiles (in page order) are the candidates; their
//      keys go to LDS (all pages of the unit when the candidates do not
//      fit, in LDS or else in the workspace).
//   3. Radix select of the k-th largest candidate key, then an ordered
//      compaction; ties at the cut go to the lower page index.
// ---------------------------------------------------------------------------
constexpr int kTopkCand = 20480;  // candidate keys held in LDS
constexpr int kTopkTileCap = 4096;

__device__ __forceinline__ int pad16(int p) { return p + (p >> 4); }

template <int G>
__global__ __launch_bounds__(kSelThreads) void k_select_topk(
    const float *__restrict__ ub, const int32_t *__restrict__ seq_lens,
    int batch, int H, int P, int max_pages, int k, int32_t *__restrict__ sel,
    int32_t *__restrict__ count, uint32_t *__restrict__ keys_ws) {
  __shared__ uint32_t s_keys[kTopkCand + kTopkCand / 16];
  __shared__ int s_tiles[kTopkTileCap];
  __shared__ int hist[512];
  __shared__ int tmp[kSelWaves];
  __shared__ uint32_t s_digit[2];
  __shared__ int s_need[4];
  __shared__ uint32_t s_wmax[kSelWaves];
  const int u = blockIdx.x, b = u / H, h = u % H;
  const int tid = threadIdx.x;
  const int np = n_pages_of(seq_lens[b], P);
  const int kk = k < np ? k : np;
  const int Hq = H * G;
  const int n_tiles = (max_pages + kPageTile - 1) / kPageTile;
  const int nt = (np + kPageTile - 1) / kPageTile;
  int32_t *out = sel + static_cast<size_t>(u) * max_pages;
  const float *ubt = ub + static_cast<size_t>(batch) * Hq * max_pages +
                     static_cast<size_t>(u) * n_tiles;

  if (kk == np) {  // every page is kept
    for (int p = tid; p < np; p += kSelThreads) out[p] = p;
    if (tid == 0) count[u] = np;
    return;
  }
  auto page_key = [&](int p) {
    float g = ub[(static_cast<size_t>(b) * Hq + h * G) * max_pages + p];
#pragma unroll
    for (int j = 1; j < G; ++j)
      g = fmaxf(g, ub[(static_cast<size_t>(b) * Hq + h * G + j) * max_pages + p]);
    return order_key(g);
  };

  // 1-2. candidate tiles and their pages
  int n_ct = nt;
  bool tiles_listed = false;
  uint32_t T0 = 0u;
  if (nt > kk && nt <= kTopkTileCap) {
    for (int t = tid; t < nt; t += kSelThreads) s_keys[t] = order_key(ubt[t]);
    lds_barrier();
    // T0 to 16 bits (rounded down): a few more tiles may reach it, all of
    // the k best pages still do
    int nd, nat;
    T0 = radix_select([&](int i) { return s_keys[i]; }, nt, kk,
                      hist, s_digit, s_need, nd, nat, 24, 16);
    n_ct = ordered_list(nt, [&](int t) { return s_keys[t] >= T0; }, s_tiles,
                        kTopkTileCap, tmp);
    tiles_listed = true;
    lds_barrier();
  }
  // Candidate slots: slot s is page tile(s / 64) * 64 + s % 64.
  const int n_slots = n_ct * kPageTile;
  auto page_of_slot = [&](int s) {
    const int ti = s / kPageTile;
    return (tiles_listed ? s_tiles[ti] : ti) * kPageTile + (s % kPageTile);
  };
  const bool in_lds = n_slots <= kTopkCand;
  uint32_t *gkeys = keys_ws + static_cast<size_t>(u) * n_tiles * kPageTile;
  constexpr int KU = 4;
  uint32_t kmax = 0u;
  for (int s0 = tid; s0 < n_slots; s0 += kSelThreads * KU) {
    uint32_t kv[KU];
#pragma unroll
    for (int k2 = 0; k2 < KU; ++k2) {
      const int s = s0 + k2 * kSelThreads;
      const int p = s < n_slots ? page_of_slot(s) : np;
      kv[k2] = p < np ? page_key(p) : 0u;
      kmax = max(kmax, kv[k2]);
    }
#pragma unroll
    for (int k2 = 0; k2 < KU; ++k2) {
      const int s = s0 + k2 * kSelThreads;
      if (s < n_slots) {
        if (in_lds) s_keys[pad16(s)] = kv[k2];
        else gkeys[s] = kv[k2];
      }
    }
  }
  kmax = wave_max_u(kmax);
  if ((tid & (kWave - 1)) == 0) s_wmax[tid / kWave] = kmax;
  if (in_lds) lds_barrier(); else __syncthreads();
  auto key_at = [&](int s) { return in_lds ? s_keys[pad16(s)] : gkeys[s]; };
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) kmax = max(kmax, s_wmax[w]);

  // 3. k-th largest candidate, then the ordered compaction over slots.  The
  // k best keys lie in [T0, kmax]: the digits those two share are skipped.
  int shift_hi = 24;
  while (shift_hi > 0 && ((T0 ^ kmax) >> shift_hi) == 0u) shift_hi -= 8;
  int need, n_at;
  const uint32_t T = radix_select(key_at, n_slots, kk, hist, s_digit, s_need,
                                  need, n_at, shift_hi, 0, kmax);
  const int per = (n_slots + kSelThreads - 1) / kSelThreads;
  const int s_beg = tid * per, s_end = min(n_slots, s_beg + per);
  if (n_at == need) {  // every key equal to T is taken: keys >= T, in order
    int n_sel = 0;
    for (int s = s_beg; s < s_end; ++s) n_sel += (key_at(s) >= T);
    int tot;
    int pos = block_excl_scan<kSelThreads>(n_sel, tmp, tot);
    for (int s = s_beg; s < s_end; ++s)
      if (key_at(s) >= T) out[pos++] = page_of_slot(s);
    if (tid == 0) count[u] = kk;
    return;
  }
  int n_eq = 0;
  for (int s = s_beg; s < s_end; ++s) n_eq += (key_at(s) == T);
  int tot;
  const int eq_rank = block_excl_scan<kSelThreads>(n_eq, tmp, tot);
  int n_sel = 0;
  {
    int r = eq_rank;
    for (int s = s_beg; s < s_end; ++s) {
      const uint32_t key = key_at(s);
      if (key > T) ++n_sel;
      else if (key == T) { n_sel += (r < need); ++r; }
    }
  }
  int pos = block_excl_scan<kSelThreads>(n_sel, tmp, tot);
  {
    int r = eq_rank;
    for (int s = s_beg; s < s_end; ++s) {
      const uint32_t key = key_at(s);
      bool take = key > T;
      if (key == T) { take = r < need; ++r; }
      if (take) out[pos++] = page_of_slot(s);
    }
  }
  if (tid == 0) count[u] = kk;
}

// ---------------------------------------------------------------------------
// Gaussian-aware selection.
//
// Threshold estimate per query head:
//   m_p = (alpha-1) mu_p, s_p = (alpha-1) sigma_p, n_p valid tokens,
//   F(tau) = sum_p n_p E[max(Z_p - tau, 0)^r],  Z_p ~ N(m_p, s_p^2).
// F is decreasing and convex, and so is F^(1/r) (an L^r norm of a convex
// non-negative function of tau).  By Jensen, n E[(Z - tau)_+^r] >=
// n (m - tau)_+^r, so F(m_p - n_p^(-1/r)) >= 1 for every page p: tau_lo =
// max_p (m_p - n_p^(-1/r)) is a lower bound on the root, and Newton's method
// on F^(1/r) - 1 started there climbs monotonically to the root without
// overshooting.  (tau_lo is taken from the largest mean over the full pages
// and over the last page, with their token counts.)  Pages with
// m_p + 8.5 s_p <= tau_lo add less than ~1e-17 each for every tau >= tau_lo
// and are left out ("survivors" are the others), first tile by tile from the
// tile summaries, then page by page.
//
// Keep test: zhat = (alpha-1)(mu + sigma sqrt(2 ln n_p)) > tau_hat - delta
// for some head.  Since tau_hat >= tau_lo, only tiles whose summary
// max(mu + sqrt(2 ln P) sigma) clears tau_lo - delta can hold a kept page
// (sqrt(2 ln n_p) <= sqrt(2 ln P)).
//
// Two kernels:
//   k_gauss_tau, one block per (unit, query head): tau_lo from the tile
//     summaries; ordered lists of the survivor tiles and of the keep
//     candidate tiles; their pages loaded at once into LDS; Newton from LDS;
//     tau_hat and, per tile, the 64-bit mask of the pages this head keeps
//     (in the workspace).
//   k_gauss_collect, one block per unit: the union of the heads' masks,
//     written out in page order.
// Lists or page data beyond the LDS capacities are read from global memory
// instead (same arithmetic, slower).
// ---------------------------------------------------------------------------
constexpr int kGtThreads = 1024;
constexpr int kGtWaves = kGtThreads / kWave;
constexpr int kGtSvItems = 128;   // survivor tiles whose (m, s) sit in LDS
constexpr int kGtKzItems = 128;   // keep-candidate tiles whose zhat sit in LDS
constexpr int kGtListCap = 4096;  // entries of each tile list
constexpr float kPruneSigmas = 8.5f;
constexpr float kGtDrop = 1e-12f;  // page terms dropped from later passes

// Standard normal tail pieces at c: Phi(c) and the density phi(c).
// For a = |c|, the upper tail Q(a) = phi(a) R(a) with R the Mills ratio,
// approximated by a degree 4 / degree 5 rational function with positive
// coefficients, fitted for least maximum relative error on [0, 14] against
// R(x) = sqrt(pi/2) erfcx(x / sqrt(2)): fit error 1.1e-8, about 4e-7 as
// evaluated here in float32.  Its large-x behaviour is R ~ 1/x, as it should
// be, and phi(a) underflows to 0 past a ~ 13.2.  Because Q is a product,
// its relative accuracy holds far into the tail; Phi(c) = Q(-c) for c < 0
// and 1 - Q(c) otherwise.  fit_mills.py (beside this file) refits such a
// rational function and checks these constants.
__device__ __forceinline__ void norm_cdf_pdf(float c, float &Phi, float &phi) {
  const float a = fabsf(c);
  phi = 0.39894228040143268f *
        __builtin_amdgcn_exp2f(-0.72134752044448170f * a * a);
  float num = 9.571634593e-03f;
  num = fmaf(num, a, 9.694951865e-02f);
  num = fmaf(num, a, 4.449650583e-01f);
  num = fmaf(num, a, 1.079636338e+00f);
  num = fmaf(num, a, 1.253314139e+00f);
  float den = 9.571468318e-03f;
  den = fmaf(den, a, 9.695800140e-02f);
  den = fmaf(den, a, 4.543498346e-01f);
  den = fmaf(den, a, 1.178967137e+00f);
  den = fmaf(den, a, 1.659309722e+00f);
  den = fmaf(den, a, 1.0f);
  const float q = phi * num * __builtin_amdgcn_rcpf(den);
  Phi = c < 0.f ? q : 1.0f - q;
}

// Adds n E[(Z - tau)_+^r] to f and n r E[(Z - tau)_+^(r-1)] to df for
// Z ~ N(m, s^2) (closed forms: E[(Z-tau)_+] = u Phi + s phi and
// E[(Z-tau)_+^2] = (u^2 + s^2) Phi + u s phi, u = m - tau, at c = u / s).
__device__ __forceinline__ void gauss_term(float m, float s, float n, float tau,
                                           int r, float &f, float &df) {
  const float u = m - tau;
  float Phi, phi;
  if (s > 0.f) {
    norm_cdf_pdf(u * __builtin_amdgcn_rcpf(s), Phi, phi);
  } else {
    Phi = u > 0.f ? 1.f : 0.f;
    phi = 0.f;
  }
  const float e1 = fmaf(u, Phi, s * phi);  // E[(Z - tau)_+]
  if (r == 2) {
    const float e2 = fmaf(fmaf(u, u, s * s), Phi, u * s * phi);
    f = fmaf(n, e2, f);
    df = fmaf(2.0f * n, e1, df);
  } else {
    f = fmaf(n, e1, f);
    df = fmaf(n, Phi, df);
  }
}

// The same two terms at any r >= 1 (r code 0), from the Gauss rules in q.
// With c = (tau - m)/s, E[(Z - tau)_+^r] = s^r J_r(c) for
// J_r(c) = int_0^inf y^r phi(y + c) dy, and -dE/dtau = s^(r-1) K with
// K = int_0^inf y^r (y + c) phi(y + c) dy (differentiating under the
// integral).  Where c >= -6 both integrands are negligible past
// y + c = 10, and y = h (1 + x), h = (10 - c)/2, turns them into
// h^(r+1) times Gauss-Jacobi sums over x with weight (1 + x)^r of the
// smooth factors phi(y + c) and (y + c) phi(y + c).  Further below the page
// mean (c < -6), and for s = 0, the expectations are taken over Z directly
// with the Gauss-Hermite rule: sum_i w_i (u + s x_i)_+^r and
// r sum_i w_i (u + s x_i)_+^(r-1), u = m - tau (the nodes below -6 carry
// under 1e-9 of the mass).
__device__ __forceinline__ void gauss_term_rule(float m, float s, float n,
                                                float tau, const GaussRule &q,
                                                float &f, float &df) {
  constexpr float kInvSqrt2Pi = 0.39894228040143268f;
  constexpr float kHalfLog2e = 0.72134752044448170f;  // log2(e) / 2
  const float u = m - tau;
  const float r = q.r;
  if (s > 0.f && u < 6.0f * s) {
    const float c = -u * __builtin_amdgcn_rcpf(s);
    const float h = 0.5f * (10.0f - c);
    if (!(h > 0.f)) return;
    float j = 0.f, k = 0.f;
#pragma unroll
    for (int i = 0; i < kJacobiNodes; ++i) {
      const float t = fmaf(h, 1.0f + q.jx[i], c);  // y + c
      const float e = q.jw[i] * __builtin_amdgcn_exp2f(-kHalfLog2e * t * t);
      j += e;
      k = fmaf(t, e, k);
    }
    // s^(r-1) h^(r+1) / sqrt(2 pi), in the log domain
    const float sc = kInvSqrt2Pi * __builtin_amdgcn_exp2f(
                                       (r - 1.0f) * __builtin_amdgcn_logf(s) +
                                       (r + 1.0f) * __builtin_amdgcn_logf(h));
    f = fmaf(n * sc * s, j, f);
    df = fmaf(n * sc, k, df);
  } else {
    float e0 = 0.f, e1 = 0.f;
#pragma unroll
    for (int i = 0; i < kHermiteNodes; ++i) {
      const float v = fmaf(s, q.hx[i], u);
      if (v > 0.f) {
        const float pv = __builtin_amdgcn_exp2f((r - 1.0f) * __builtin_amdgcn_logf(v));
        e1 = fmaf(q.hw[i], pv, e1);
        e0 = fmaf(q.hw[i] * v, pv, e0);
      }
    }
    f = fmaf(n, e0, f);
    df = fmaf(n * r, e1, df);
  }
}

// Exclusive prefix sums of L counters over a block of NT threads (thread
// order) and their totals.  smem holds L * NT / 64 ints.  Contains barriers.
template <int NT, int L>
__device__ __forceinline__ void block_scan_multi(const int (&x)[L], int (&pre)[L],
                                                 int (&tot)[L], int *smem) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  int incl[L];
#pragma unroll
  for (int l = 0; l < L; ++l) incl[l] = wave_incl_scan(x[l]);
  if (lane == kWave - 1)
#pragma unroll
    for (int l = 0; l < L; ++l) smem[l * NW + wid] = incl[l];
  lds_barrier();
#pragma unroll
  for (int l = 0; l < L; ++l) {
    int base = 0, t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int v = smem[l * NW + w];
      base += (w < wid) ? v : 0;
      t += v;
    }
    pre[l] = base + incl[l] - x[l];
    tot[l] = t;
  }
}

// HALF: half the LDS capacities (about 65 KiB instead of 129 KiB), so that
// two blocks share a CU (eight waves per SIMD); used when there are more
// query heads than CUs.
template <int G, bool RULE, bool HALF>
__global__ __launch_bounds__(kGtThreads, HALF ? 8 : 1) void k_gauss_tau(
    const float *__restrict__ gstat, const int32_t *__restrict__ seq_lens,
    int batch, int H, int P, int max_pages, float am1, int r, float delta,
    float *__restrict__ tau_hat, unsigned long long *__restrict__ masks,
    const GaussRule rule) {
  constexpr int SvItems = HALF ? kGtSvItems / 2 : kGtSvItems;
  constexpr int KzItems = HALF ? kGtKzItems / 2 : kGtKzItems;
  constexpr int ListCap = HALF ? kGtListCap / 2 : kGtListCap;
  __shared__ float2 s_sv[SvItems * kPageTile];  // (m, s); s < 0: last page
  __shared__ float s_kz[KzItems * kPageTile];
  __shared__ int s_slist[ListCap];
  __shared__ int s_klist[ListCap];
  __shared__ int s_scan[2 * kGtWaves];
  __shared__ float s_red[2][kGtWaves];
  __shared__ float2 s_fd[2][kGtWaves];
  const int u = blockIdx.x / G, g = blockIdx.x % G, b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int len = seq_lens[b];
  const int np = n_pages_of(len, P);
  const int nt = (np + kPageTile - 1) / kPageTile;
  const int Hq = H * G;
  const int n_tiles = (max_pages + kPageTile - 1) / kPageTile;
  const size_t row = static_cast<size_t>(b) * Hq + h * G + g;
  const float2 *st = reinterpret_cast<const float2 *>(gstat) + row * max_pages;
  const float4 *gt = reinterpret_cast<const float4 *>(
                         gstat + gstat_tile_offset(batch, Hq, max_pages)) +
                     row * n_tiles;
  unsigned long long *mk = masks + (static_cast<size_t>(u) * G + g) * n_tiles;
  const float last_n = static_cast<float>(page_tokens(np - 1, len, P));
  const bool ragged = last_n < static_cast<float>(P);
  const float full_c = sqrtf(2.0f * logf(static_cast<float>(P)));
  const float last_c = sqrtf(2.0f * logf(last_n));

  // 1. tau_lo.  Each thread owns a contiguous range of tiles and keeps the
  // (.y, .z) summaries of its first one.  The last tile's summary may come
  // from the partial last page, so that tile is read page by page.
  const int per = (nt + kGtThreads - 1) / kGtThreads;
  const int t_beg = min(nt, tid * per), t_end = min(nt, t_beg + per);
  float2 c2 = make_float2(-FLT_MAX, -FLT_MAX);
  float mx = -FLT_MAX, ml = -FLT_MAX;
  for (int t = t_beg; t < t_end; ++t) {
    const float4 v = gt[t];
    if (t == t_beg) c2 = make_float2(v.y, v.z);
    if (!(ragged && t == nt - 1)) mx = fmaxf(mx, v.x);
  }
  if (ragged && wave == 0) {
    const int p = (nt - 1) * kPageTile + lane;
    if (p < np) {
      const float x = st[p].x;
      if (p == np - 1) ml = x;
      else mx = fmaxf(mx, x);
    }
  }
  mx = group_max<kWave>(mx);
  ml = group_max<kWave>(ml);
  if (lane == 0) {
    s_red[0][wave] = mx;
    s_red[1][wave] = ml;
  }
  lds_barrier();
  float M = s_red[0][0], ML = s_red[1][0];
#pragma unroll
  for (int w = 1; w < kGtWaves; ++w) {
    M = fmaxf(M, s_red[0][w]);
    ML = fmaxf(ML, s_red[1][w]);
  }
  // n^(-1/r) for the full and the last page (r code 0: rule.r)
  auto inv_root = [&](float n) {
    if constexpr (RULE) return __builtin_amdgcn_exp2f(-__builtin_amdgcn_logf(n) / rule.r);
    return r == 2 ? rsqrtf(n) : 1.0f / n;
  };
  const float inv_full = inv_root(static_cast<float>(P));
  const float inv_last = inv_root(last_n);
  const float tau_lo = fmaxf(am1 * M - inv_full, am1 * ML - inv_last);
  // Tile tests get a small margin: they only prune, the page tests decide.
  const float s_thr = tau_lo - 1e-5f * fmaxf(fabsf(tau_lo), 1.0f);
  const float kc0 = tau_lo - delta;
  const float k_thr = kc0 - 1e-5f * fmaxf(fabsf(kc0), 1.0f);

  // 2. ordered lists of survivor tiles and keep-candidate tiles.
  auto tile_flags = [&](int t, bool &sf, bool &kf) {
    float2 v = c2;
    if (t != t_beg) {
      const float4 w = gt[t];
      v = make_float2(w.y, w.z);
    }
    sf = am1 * v.x > s_thr;
    kf = am1 * v.y > k_thr;
  };
  int cnt[2] = {0, 0}, pre[2], tot[2];
  for (int t = t_beg; t < t_end; ++t) {
    bool sf, kf;
    tile_flags(t, sf, kf);
    cnt[0] += sf;
    cnt[1] += kf;
  }
  block_scan_multi<kGtThreads, 2>(cnt, pre, tot, s_scan);
  const bool s_listed = tot[0] <= ListCap;
  const bool k_listed = tot[1] <= ListCap;
  const int n_st = s_listed ? tot[0] : nt;  // otherwise every tile, in order
  const int n_kt = k_listed ? tot[1] : nt;
  for (int t = t_beg; t < t_end; ++t) {
    bool sf, kf;
    tile_flags(t, sf, kf);
    if (sf && s_listed) s_slist[pre[0]++] = t;
    if (kf && k_listed) s_klist[pre[1]++] = t;
    // Tiles that cannot hold a kept page get an empty mask here; the
    // listed ones are written after the threshold is known.
    if (!kf && k_listed) mk[t] = 0ull;
  }
  lds_barrier();
  auto surv_tile = [&](int i) { return s_listed ? s_slist[i] : i; };
  auto keep_tile = [&](int k) { return k_listed ? s_klist[k] : k; };
  // (m, s) of page p, m = -inf if it is not a survivor, s < 0 (stored as
  // -1 - s) tags the last page.
  auto surv_entry = [&](int p) -> float2 {
    if (p >= np) return make_float2(-INFINITY, 0.f);
    const float2 v = st[p];
    const float m = am1 * v.x, sd = am1 * sqrtf(fmaxf(v.y, 0.f));
    if (!(m + kPruneSigmas * sd > tau_lo)) return make_float2(-INFINITY, 0.f);
    return make_float2(m, p == np - 1 ? -1.0f - sd : sd);
  };
  auto zhat = [&](int p, const float2 v) {
    const float c = (p == np - 1) ? last_c : full_c;
    return am1 * (v.x + sqrtf(fmaxf(v.y, 0.f)) * c);
  };

  // 3. load the pages of both lists into LDS, loads of a round in flight
  // together (entries wave, wave + 8, ...).
  {
    constexpr int KS = 4, KK = 4;
    const int s_lim = min(n_st, SvItems), k_lim = min(n_kt, KzItems);
    for (int c = 0;; ++c) {
      const int si0 = wave + c * KS * kGtWaves;
      const int ki0 = wave + c * KK * kGtWaves;
      if (si0 >= s_lim && ki0 >= k_lim) break;
      float2 kv[KK];
      int kp[KK];
#pragma unroll
      for (int k = 0; k < KK; ++k) {
        const int ki = ki0 + k * kGtWaves;
        kp[k] = ki < k_lim ? keep_tile(ki) * kPageTile + lane : np;
        kv[k] = kp[k] < np ? st[kp[k]] : make_float2(0.f, 0.f);
      }
      float2 sv[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int si = si0 + k * kGtWaves;
        sv[k] = si < s_lim ? surv_entry(surv_tile(si) * kPageTile + lane)
                           : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int si = si0 + k * kGtWaves;
        if (si < s_lim) s_sv[si * kPageTile + lane] = sv[k];
      }
#pragma unroll
      for (int k = 0; k < KK; ++k) {
        const int ki = ki0 + k * kGtWaves;
        if (ki < k_lim)
          s_kz[ki * kPageTile + lane] = kp[k] < np ? zhat(kp[k], kv[k]) : -INFINITY;
      }
    }
  }
  lds_barrier();

  // 4. Newton on F^(1/r) - 1 from tau_lo.  The step for r = 2,
  // 2 (F - sqrt F) / (-F'), is taken as 2 sqrt(F) (F - 1) / ((sqrt F + 1)
  // (-F')), which keeps its relative accuracy in float32 as F -> 1; every
  // thread takes the same step from the same sums.  All waves share the
  // pages, with one barrier per iteration (s_fd is double-buffered).
  auto step_from = [&](float ff, float dd, float t, float &next) {
    if (!(ff > 1.0f) || !(dd > 0.0f)) return false;
    float step;
    if constexpr (RULE) {
      // r F (1 - F^(-1/r)) / (-F'), with 1 - F^(-1/r) = -expm1(-ln F / r)
      step = rule.r * ff * -expm1f(-logf(ff) / rule.r) / dd;
    } else if (r == 2) {
      const float sf = sqrtf(ff);
      step = 2.0f * sf * (ff - 1.0f) / ((sf + 1.0f) * dd);
    } else {
      step = (ff - 1.0f) / dd;
    }
    next = t + step;
    return next > t;
  };
  auto page_terms = [&](int i, float t, float &f, float &df) {
    const float2 e = i < SvItems ? s_sv[i * kPageTile + lane]
                                    : surv_entry(surv_tile(i) * kPageTile + lane);
    if (e.x == -INFINITY) return;
    const bool last = e.y < 0.f;
    const float sd = last ? -1.0f - e.y : e.y;
    const float nn = last ? last_n : static_cast<float>(P);
    float tf = 0.f, tdf = 0.f;
    if constexpr (RULE) gauss_term_rule(e.x, sd, nn, t, rule, tf, tdf);
    else gauss_term(e.x, sd, nn, t, r, tf, tdf);
    f += tf;
    df += tdf;
    // A page's term only falls as tau rises (every step is upward): once
    // below kGtDrop it is dropped for the remaining passes.  Together the
    // dropped terms stay under 16384 kGtDrop, far below float rounding of
    // F ~ 1.
    if (i < SvItems && tf < kGtDrop) s_sv[i * kPageTile + lane].x = -INFINITY;
  };
  float tau = tau_lo, prev_step = INFINITY;
  for (int it = 0; it < 64; ++it) {
    float f = 0.f, df = 0.f;
    for (int i = wave; i < n_st; i += kGtWaves) page_terms(i, tau, f, df);
    f = wave_sum_f(f);
    df = wave_sum_f(df);
    if (lane == 0) s_fd[it & 1][wave] = make_float2(f, df);
    lds_barrier();
    float ff = 0.f, dd = 0.f;
#pragma unroll
    for (int w = 0; w < kGtWaves; ++w) {
      const float2 v = s_fd[it & 1][w];
      ff += v.x;
      dd += v.y;
    }
    float next;
    if (!step_from(ff, dd, tau, next)) break;
    // In the quadratic phase of the iteration a step s that is rho times
    // the one before is followed by one of about rho^2 s.  With s below
    // 1e-4 max(1, |tau|) and rho below 0.01 that is about 1e-8 (relative),
    // under float rounding, so the iteration ends here rather than spend a
    // pass confirming it.  (A small step alone would not do: from below, a
    // convex F's Newton step falls short of the distance to the root where
    // F flattens out; a sharp drop in the step shows that it does not.)
    const float step = next - tau;
    const bool last = step <= 1e-4f * fmaxf(1.0f, fabsf(tau)) && step <= 0.01f * prev_step;
    prev_step = step;
    tau = next;
    if (last) break;
  }
  if (tid == 0) tau_hat[row] = tau;

  // 5. this head's keep masks of the candidate tiles.
  const float cut = tau - delta;
  for (int k = wave; k < n_kt; k += kGtWaves) {
    const int t = keep_tile(k);
    const int p = t * kPageTile + lane;
    float z = -INFINITY;
    if (k < KzItems) z = s_kz[k * kPageTile + lane];
    else if (p < np) z = zhat(p, st[p]);
    const unsigned long long ball = __ballot(z > cut);
    if (lane == 0) mk[t] = ball;
  }
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void k_gauss_collect(
    const float *__restrict__ gstat, const int32_t *__restrict__ seq_lens,
    int batch, int H, int P, int max_pages, float am1,
    const unsigned long long *__restrict__ masks,
    const float *__restrict__ tau_hat, int32_t *__restrict__ sel,
    int32_t *__restrict__ count) {
  __shared__ unsigned long long s_mask[kSelThreads];
  __shared__ int s_off[kSelThreads];
  __shared__ int tmp[kSelWaves];
  __shared__ float s_gap[kSelWaves];
  __shared__ int s_idx[kSelWaves];
  const int u = blockIdx.x, b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int len = seq_lens[b];
  const int np = n_pages_of(len, P);
  const int nt = (np + kPageTile - 1) / kPageTile;
  const int n_tiles = (max_pages + kPageTile - 1) / kPageTile;
  const unsigned long long *mk = masks + static_cast<size_t>(u) * G * n_tiles;
  const unsigned long long below = (1ull << lane) - 1ull;
  int32_t *out = sel + static_cast<size_t>(u) * max_pages;

  // Chunks of kSelThreads tiles: union of the heads' masks, exclusive scan
  // of the page counts, then one wave per tile writes its pages in order.
  int total = 0;
  for (int c0 = 0; c0 < nt; c0 += kSelThreads) {
    const int t = c0 + tid;
    unsigned long long m = 0ull;
    if (t < nt) {
#pragma unroll
      for (int g = 0; g < G; ++g) m |= mk[static_cast<size_t>(g) * n_tiles + t];
    }
    int ctot;
    const int pre = block_excl_scan<kSelThreads>(__popcll(m), tmp, ctot);
    s_mask[tid] = m;
    s_off[tid] = total + pre;
    lds_barrier();
    const int n_c = min(kSelThreads, nt - c0);
    for (int j = wave; j < n_c; j += kSelWaves) {
      const unsigned long long mm = s_mask[j];
      if ((mm >> lane) & 1ull)
        out[s_off[j] + __popcll(mm & below)] = (c0 + j) * kPageTile + lane;
    }
    total += ctot;
    lds_barrier();  // s_mask and s_off are rewritten by the next chunk
  }
  if (total > 0) {
    if (tid == 0) count[u] = total;
    return;
  }
  // Nothing kept: the page with the largest margin
  // max_g (zhat_g - tau_hat_g), lower index on ties (all pages scanned).
  const int Hq = H * G;
  const float2 *st = reinterpret_cast<const float2 *>(gstat) +
                     (static_cast<size_t>(b) * Hq + h * G) * max_pages;
  const float *th = tau_hat + static_cast<size_t>(b) * Hq + h * G;
  const float last_n = static_cast<float>(page_tokens(np - 1, len, P));
  const float full_c = sqrtf(2.0f * logf(static_cast<float>(P)));
  const float last_c = sqrtf(2.0f * logf(last_n));
  float best = -FLT_MAX;
  int bi = np;
  for (int p = tid; p < np; p += kSelThreads) {
    const float c = (p == np - 1) ? last_c : full_c;
    float mg = -FLT_MAX;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float2 v = st[static_cast<size_t>(g) * max_pages + p];
      mg = fmaxf(mg, am1 * (v.x + sqrtf(fmaxf(v.y, 0.f)) * c) - th[g]);
    }
    if (mg > best) { best = mg; bi = p; }
  }
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float om = __shfl_xor(best, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    if (om > best || (om == best && oi < bi)) { best = om; bi = oi; }
  }
  if (lane == 0) {
    s_gap[wave] = best;
    s_idx[wave] = bi;
  }
  lds_barrier();
  if (tid == 0) {
    for (int w = 0; w < kSelWaves; ++w)
      if (s_gap[w] > best || (s_gap[w] == best && s_idx[w] < bi)) {
        best = s_gap[w];
        bi = s_idx[w];
      }
    out[0] = bi < np ? bi : 0;
    count[u] = 1;
  }
}

// ---------------------------------------------------------------------------
template <int G>
hipError_t launch_select_topk(const ekv_paged_kv &kv, const float *ub, int k,
                              int32_t *sel, int32_t *count, void *ws,
                              hipStream_t stream) {
  const int units = kv.batch * kv.num_kv_heads;
  hipLaunchKernelGGL((k_select_topk<G>), dim3(units), dim3(kSelThreads), 0,
                     stream, ub, kv.seq_lens, kv.batch, kv.num_kv_heads,
                     kv.page_size, kv.max_pages, k, sel, count,
                     static_cast<uint32_t *>(ws));
  return hipGetLastError();
}

template <int G>
hipError_t launch_select_gauss(const ekv_paged_kv &kv, const float *gstat,
                               float alpha, float delta, int32_t *sel,
                               int32_t *count, float *tau_hat, void *ws,
                               hipStream_t stream) {
  // r code: 1 and 2 have closed forms; 0 sums the Gauss rules built here
  const int r = alpha == 2.0f ? 1 : alpha == 1.5f ? 2 : 0;
  GaussRule rule{};
  rule.r = 1.0f / (alpha - 1.0f);
  if (r == 0) {
    double x[kJacobiNodes], w[kJacobiNodes], hx[kHermiteNodes], hw[kHermiteNodes];
    if (!gauss_jacobi_rule(static_cast<double>(rule.r), kJacobiNodes, x, w) ||
        !gauss_hermite_rule(kHermiteNodes, hx, hw))
      return hipErrorInvalidValue;
    for (int i = 0; i < kJacobiNodes; ++i) {
      rule.jx[i] = static_cast<float>(x[i]);
      rule.jw[i] = static_cast<float>(w[i]);
    }
    for (int i = 0; i < kHermiteNodes; ++i) {
      rule.hx[i] = static_cast<float>(hx[i]);
      rule.hw[i] = static_cast<float>(hw[i]);
    }
  }
  const int units = kv.batch * kv.num_kv_heads;
  auto *masks = static_cast<unsigned long long *>(ws);
  // one block per query head: with more heads than CUs the half-capacity
  // form lets two blocks share a CU (the closed forms only: the quadrature
  // form does not fit eight waves per SIMD without spilling)
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n_cu <= 0)
    n_cu = 256;
  const bool half = units * G > n_cu;
  auto gt = r == 0 ? k_gauss_tau<G, true, false>
                   : (half ? k_gauss_tau<G, false, true> : k_gauss_tau<G, false, false>);
  hipLaunchKernelGGL(gt, dim3(units * G), dim3(kGtThreads), 0, stream, gstat,
                     kv.seq_lens, kv.batch, kv.num_kv_heads, kv.page_size,
                     kv.max_pages, alpha - 1.0f, r, delta, tau_hat, masks,
                     rule);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gauss_collect<G>), dim3(units), dim3(kSelThreads), 0,
                     stream, gstat, kv.seq_lens, kv.batch, kv.num_kv_heads,
                     kv.page_size, kv.max_pages, alpha - 1.0f, masks, tau_hat,
                     sel, count);
  return hipGetLastError();
}

#define EKV_INST_SEL(G)                                                      \
  template hipError_t launch_select_topk<G>(const ekv_paged_kv &,            \
                                            const float *, int, int32_t *,   \
                                            int32_t *, void *, hipStream_t); \
  template hipError_t launch_select_gauss<G>(                                \
      const ekv_paged_kv &, const float *, float, float, int32_t *,          \
      int32_t *, float *, void *, hipStream_t);
EKV_FOR_EACH_G(EKV_INST_SEL)

}  // namespace ekv
