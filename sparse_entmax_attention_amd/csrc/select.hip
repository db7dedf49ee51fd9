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

// kk-th largest of n keys key_at(i) (kk <= n): returns the key T and, in
// need, how many keys equal to T belong to the kk largest.  Most
// significant digit first, 8 bits per pass.  Contains barriers.
template <class F>
__device__ uint32_t radix_select(F key_at, int n, int kk, int *hist,
                                 uint32_t *s_digit, int *s_need, int &need) {
  uint32_t prefix = 0, mask = 0;
  need = kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
    lds_barrier();
    for (int i = threadIdx.x; i < n; i += kSelThreads) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    lds_barrier();
    if (threadIdx.x < kWave) {
      // Lane l owns digits 255-4l .. 252-4l (descending).
      const int l = threadIdx.x;
      int c[4], local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * l - j];
        local += c[j];
      }
      const int incl = wave_incl_scan(local);
      int before = incl - local;  // keys with a larger digit
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < need && before + c[j] >= need) {
          *s_digit = static_cast<uint32_t>(255 - 4 * l - j);
          *s_need = need - before;
        }
        before += c[j];
      }
    }
    lds_barrier();
    prefix |= *s_digit << shift;
    mask |= 255u << shift;
    need = *s_need;
    lds_barrier();
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
  __shared__ int hist[256];
  __shared__ int tmp[kSelWaves];
  __shared__ uint32_t s_digit;
  __shared__ int s_need;
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
  if (nt > kk && nt <= kTopkTileCap) {
    for (int t = tid; t < nt; t += kSelThreads) s_keys[t] = order_key(ubt[t]);
    lds_barrier();
    int nd;
    const uint32_t T0 = radix_select([&](int i) { return s_keys[i]; }, nt, kk,
                                     hist, &s_digit, &s_need, nd);
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
  for (int s0 = tid; s0 < n_slots; s0 += kSelThreads * KU) {
    uint32_t kv[KU];
#pragma unroll
    for (int k2 = 0; k2 < KU; ++k2) {
      const int s = s0 + k2 * kSelThreads;
      const int p = s < n_slots ? page_of_slot(s) : np;
      kv[k2] = p < np ? page_key(p) : 0u;
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
  if (in_lds) lds_barrier(); else __syncthreads();
  auto key_at = [&](int s) { return in_lds ? s_keys[pad16(s)] : gkeys[s]; };

  // 3. k-th largest candidate, then the ordered compaction over slots.
  int need;
  const uint32_t T = radix_select(key_at, n_slots, kk, hist, &s_digit, &s_need, need);
  const int per = (n_slots + kSelThreads - 1) / kSelThreads;
  const int s_beg = tid * per, s_end = min(n_slots, s_beg + per);
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
// Gaussian-aware selection, one block per unit.
//
// Threshold estimate per query head:
//   m_p = (alpha-1) mu_p, s_p = (alpha-1) sigma_p, n_p valid tokens,
//   F(tau) = sum_p n_p E[max(Z_p - tau, 0)^r],  Z_p ~ N(m_p, s_p^2).
// F is decreasing and convex, and so is F^(1/r) (an L^r norm of a convex
// non-negative function of tau).  Newton's method on F^(1/r) - 1 started at
// tau_lo = max_p m_p - 1 (where F >= 1) therefore climbs monotonically to
// the root without overshooting.  Pages with m_p + 8.5 s_p <= tau_lo add
// less than ~1e-17 each for every tau >= tau_lo and are left out, first
// tile by tile from the tile summaries, then page by page.
//
// Keep test: zhat = (alpha-1)(mu + sigma sqrt(2 ln n_p)) > tau_hat - delta
// for some head; a tile is examined only if its summary
// max(mu + sqrt(2 ln P) sigma) (an upper bound on every page's mu + sigma
// sqrt(2 ln n_p), as n_p <= P) can pass for some head.
// ---------------------------------------------------------------------------
constexpr int kSurvCap = 8192;    // survivor pages (all heads) in LDS
constexpr int kTileListCap = 4096;

struct GaussTerm {
  double f, df;  // contribution to F and to -dF/dtau
};

// n * E[(Z - tau)_+^r] and n * r * E[(Z - tau)_+^(r-1)] for Z ~ N(m, s^2).
__device__ __forceinline__ GaussTerm gauss_term(float m, float s, float n,
                                                float tau, int r) {
  const float u = m - tau;
  float Phi, phi;
  if (s > 0.f) {
    const float c = u / s;
    Phi = 0.5f * erfcf(-c * 0.70710678118654752f);
    phi = 0.39894228040143268f * expf(-0.5f * c * c);
  } else {
    Phi = u > 0.f ? 1.f : 0.f;
    phi = 0.f;
  }
  const float e1 = u * Phi + s * phi;  // E[(Z - tau)_+]
  GaussTerm t;
  if (r == 2) {
    const float e2 = (u * u + s * s) * Phi + u * s * phi;
    t.f = static_cast<double>(n) * e2;
    t.df = 2.0 * static_cast<double>(n) * e1;
  } else {
    t.f = static_cast<double>(n) * e1;
    t.df = static_cast<double>(n) * Phi;
  }
  return t;
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void k_select_gauss(
    const float *__restrict__ gstat, const int32_t *__restrict__ seq_lens,
    int batch, int H, int P, int max_pages, float am1, int r, float delta,
    int32_t *__restrict__ sel, int32_t *__restrict__ count,
    float *__restrict__ tau_hat) {
  __shared__ float2 s_surv[kSurvCap];  // (m, s); s < 0 tags the last page
  __shared__ int s_tiles[kTileListCap];
  __shared__ int s_soff[G + 1];
  __shared__ int s_cnt[kSelWaves];
  __shared__ float s_red[kSelWaves][G];
  __shared__ double s_fd[2][G][kSelWaves];
  __shared__ float s_tau[G];
  __shared__ int tmp[kSelWaves];
  __shared__ float s_gap[kSelWaves];
  __shared__ int s_idx[kSelWaves];
  const int u = blockIdx.x, b = u / H, h = u % H;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int len = seq_lens[b];
  const int np = n_pages_of(len, P);
  const int nt = (np + kPageTile - 1) / kPageTile;
  const int Hq = H * G;
  const int n_tiles = (max_pages + kPageTile - 1) / kPageTile;
  const float2 *st = reinterpret_cast<const float2 *>(gstat) +
                     (static_cast<size_t>(b) * Hq + h * G) * max_pages;
  const float4 *gt = reinterpret_cast<const float4 *>(
                         gstat + gstat_tile_offset(batch, Hq, max_pages)) +
                     (static_cast<size_t>(b) * Hq + h * G) * n_tiles;
  const float last_n = static_cast<float>(page_tokens(np - 1, len, P));
  const unsigned long long below = (1ull << lane) - 1ull;

  // 1. largest page mean per head, from the tile summaries
  float mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = -FLT_MAX;
  for (int t = tid; t < nt; t += kSelThreads)
#pragma unroll
    for (int g = 0; g < G; ++g)
      mx[g] = fmaxf(mx[g], gt[static_cast<size_t>(g) * n_tiles + t].x);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float m = group_max<kWave>(mx[g]);
    if (lane == 0) s_red[wave][g] = m;
  }
  lds_barrier();
  float tau_lo[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = s_red[0][g];
    for (int w = 1; w < kSelWaves; ++w) m = fmaxf(m, s_red[w][g]);
    tau_lo[g] = am1 * m - 1.0f;
  }

  // 2. survivors of every head, in (head, page) order, in LDS: tiles whose
  // summary passes, then one tile per wave and an ordered write per round.
  bool surv_ok = true;
  int n_surv = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (tid == 0) s_soff[g] = n_surv;
    const float tl = tau_lo[g];
    const int n_st = ordered_list(
        nt, [&](int t) { return am1 * gt[static_cast<size_t>(g) * n_tiles + t].y > tl; },
        s_tiles, kTileListCap, tmp);
    if (n_st > kTileListCap) surv_ok = false;
    const int n_use = surv_ok ? n_st : 0;
    for (int r0 = 0; r0 < n_use; r0 += kSelWaves) {
      const int ti = r0 + wave;
      const int p = ti < n_use ? s_tiles[ti] * kPageTile + lane : np;
      float m = 0.f, sd = 0.f;
      bool ok = false;
      if (p < np) {
        const float2 v = st[static_cast<size_t>(g) * max_pages + p];
        m = am1 * v.x;
        sd = am1 * sqrtf(fmaxf(v.y, 0.f));
        ok = m + 8.5f * sd > tl;
      }
      const unsigned long long ball = __ballot(ok);
      if (lane == 0) s_cnt[wave] = __popcll(ball);
      lds_barrier();
      int off = n_surv, tot = 0;
      for (int w = 0; w < kSelWaves; ++w) {
        off += (w < wave) ? s_cnt[w] : 0;
        tot += s_cnt[w];
      }
      const int pos = off + __popcll(ball & below);
      if (ok && pos < kSurvCap)
        s_surv[pos] = make_float2(m, p == np - 1 ? -1.0f - sd : sd);
      n_surv += tot;
      lds_barrier();
    }
    if (n_surv > kSurvCap) surv_ok = false;
  }
  if (tid == 0) s_soff[G] = n_surv;
  lds_barrier();

  // 3. Newton for all heads together, one block reduction per iteration.
  float tau[G];
  bool done[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { tau[g] = tau_lo[g]; done[g] = false; }
  for (int it = 0; it < 64; ++it) {
    double f[G], df[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      f[g] = 0.0;
      df[g] = 0.0;
      if (done[g]) continue;
      if (surv_ok) {
        for (int i = s_soff[g] + tid; i < s_soff[g + 1]; i += kSelThreads) {
          const float2 e = s_surv[i];
          const bool last = e.y < 0.f;
          const GaussTerm t = gauss_term(e.x, last ? -1.0f - e.y : e.y,
                                         last ? last_n : static_cast<float>(P),
                                         tau[g], r);
          f[g] += t.f;
          df[g] += t.df;
        }
      } else {
        for (int p = tid; p < np; p += kSelThreads) {
          const float2 v = st[static_cast<size_t>(g) * max_pages + p];
          const float m = am1 * v.x, sd = am1 * sqrtf(fmaxf(v.y, 0.f));
          if (m + 8.5f * sd > tau_lo[g]) {
            const GaussTerm t = gauss_term(
                m, sd, p == np - 1 ? last_n : static_cast<float>(P), tau[g], r);
            f[g] += t.f;
            df[g] += t.df;
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      f[g] = group_sum_d<kWave>(f[g]);
      df[g] = group_sum_d<kWave>(df[g]);
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) { s_fd[0][g][wave] = f[g]; s_fd[1][g][wave] = df[g]; }
    }
    lds_barrier();
    bool all_done = true;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (done[g]) continue;
      double ff = 0.0, dd = 0.0;
      for (int w = 0; w < kSelWaves; ++w) { ff += s_fd[0][g][w]; dd += s_fd[1][g][w]; }
      if (!(ff > 1.0) || !(dd > 0.0)) { done[g] = true; continue; }
      const double step = (r == 2) ? 2.0 * (ff - sqrt(ff)) / dd : (ff - 1.0) / dd;
      const float next = static_cast<float>(static_cast<double>(tau[g]) + step);
      if (!(next > tau[g])) { done[g] = true; continue; }
      tau[g] = next;
      all_done = false;
    }
    lds_barrier();  // s_fd is rewritten by the next iteration
    if (all_done) break;
  }
  if (tid < G) {
    float tg = tau[0];
#pragma unroll
    for (int g = 1; g < G; ++g) if (g == tid) tg = tau[g];
    s_tau[tid] = tg;
    tau_hat[b * Hq + h * G + tid] = tg;
  }
  lds_barrier();

  // 4. keep test over the tiles that can pass, ordered write per round.
  float cut[G];
#pragma unroll
  for (int g = 0; g < G; ++g) cut[g] = s_tau[g] - delta;
  const float full_c = sqrtf(2.0f * logf(static_cast<float>(P)));
  const float last_c = sqrtf(2.0f * logf(last_n));
  const int n_kt = ordered_list(
      nt,
      [&](int t) {
        bool any = false;
#pragma unroll
        for (int g = 0; g < G; ++g)
          any |= am1 * gt[static_cast<size_t>(g) * n_tiles + t].z > cut[g];
        return any;
      },
      s_tiles, kTileListCap, tmp);
  const bool kt_listed = n_kt <= kTileListCap;
  const int n_scan = kt_listed ? n_kt : nt;
  int32_t *out = sel + static_cast<size_t>(u) * max_pages;
  int total = 0;
  for (int r0 = 0; r0 < n_scan; r0 += kSelWaves) {
    const int ti = r0 + wave;
    const int tile = ti < n_scan ? (kt_listed ? s_tiles[ti] : ti) : nt;
    const int p = tile * kPageTile + lane;
    bool keep = false;
    if (p < np) {
      const float c = (p == np - 1) ? last_c : full_c;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float2 v = st[static_cast<size_t>(g) * max_pages + p];
        keep |= am1 * (v.x + sqrtf(fmaxf(v.y, 0.f)) * c) > cut[g];
      }
    }
    const unsigned long long ball = __ballot(keep);
    if (lane == 0) s_cnt[wave] = __popcll(ball);
    lds_barrier();
    int off = total, tot = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      off += (w < wave) ? s_cnt[w] : 0;
      tot += s_cnt[w];
    }
    if (keep) out[off + __popcll(ball & below)] = p;
    total += tot;
    lds_barrier();
  }
  if (total > 0) {
    if (tid == 0) count[u] = total;
    return;
  }
  // Nothing kept: the page with the largest margin
  // max_g (zhat_g - tau_hat_g), lower index on ties (all pages scanned).
  float best = -FLT_MAX;
  int bi = np;
  for (int p = tid; p < np; p += kSelThreads) {
    const float c = (p == np - 1) ? last_c : full_c;
    float mg = -FLT_MAX;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float2 v = st[static_cast<size_t>(g) * max_pages + p];
      mg = fmaxf(mg, am1 * (v.x + sqrtf(fmaxf(v.y, 0.f)) * c) - s_tau[g]);
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
                               int32_t *count, float *tau_hat,
                               hipStream_t stream) {
  const int r = alpha == 2.0f ? 1 : 2;
  hipLaunchKernelGGL((k_select_gauss<G>), dim3(kv.batch * kv.num_kv_heads),
                     dim3(kSelThreads), 0, stream, gstat, kv.seq_lens,
                     kv.batch, kv.num_kv_heads, kv.page_size, kv.max_pages,
                     alpha - 1.0f, r, delta, sel, count, tau_hat);
  return hipGetLastError();
}

#define EKV_INST_SEL(G)                                                      \
  template hipError_t launch_select_topk<G>(const ekv_paged_kv &,            \
                                            const float *, int, int32_t *,   \
                                            int32_t *, void *, hipStream_t); \
  template hipError_t launch_select_gauss<G>(                                \
      const ekv_paged_kv &, const float *, float, float, int32_t *,          \
      int32_t *, float *, hipStream_t);
EKV_FOR_EACH_G(EKV_INST_SEL)

}  // namespace ekv
