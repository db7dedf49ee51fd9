// Candidate selection (Technical Summary: EntmaxKV, §2.B).
//
//  * Top-k (§2.B.1): per unit, rank pages by the largest box bound over the
//    unit's query heads and keep the k best.  Exact k-th-largest search by a
//    4 x 8-bit radix select on order-preserving integer keys of the float32
//    bounds, then an ordered compaction (ties go to the lower page index).
//  * Gaussian-aware (§2.B.2): per query head, the threshold estimate tau_hat
//    solves sum_p n_p E[max(Z_p - tau, 0)^r] = 1 over page score Gaussians;
//    per unit, pages whose estimated largest score clears tau_hat - delta for
//    some query head are kept.
#include <float.h>

#include "ekv_device.h"
#include "ekv_kernels.h"

namespace ekv {

// Order-preserving map float -> uint32 (larger float, larger key).  -0 is
// folded onto +0 so that the two compare equal, as they do as floats.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Top-k.  One 1024-thread block per unit.  Keys of the unit's pages are
// written once to the workspace and re-read (from cache) by each pass.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;

template <int G>
__global__ __launch_bounds__(kTopkThreads) void k_select_topk(
    const float *__restrict__ ub, const int32_t *__restrict__ seq_lens, int H,
    int P, int max_pages, int k, int32_t *__restrict__ sel,
    int32_t *__restrict__ count, uint32_t *__restrict__ keys_ws) {
  __shared__ int hist[256];
  __shared__ int scan_tmp[kTopkThreads / kWave];
  __shared__ uint32_t s_digit;
  __shared__ int s_need;
  const int u = blockIdx.x, b = u / H, h = u % H;
  const int tid = threadIdx.x;
  const int np = n_pages_of(seq_lens[b], P);
  const int kk = k < np ? k : np;
  const int Hq = H * G;
  int32_t *out = sel + static_cast<size_t>(u) * max_pages;
  uint32_t *keys = keys_ws + static_cast<size_t>(u) * max_pages;

  if (kk == np) {  // every page is kept
    for (int p = tid; p < np; p += kTopkThreads) out[p] = p;
    if (tid == 0) count[u] = np;
    return;
  }
  for (int p = tid; p < np; p += kTopkThreads) {
    float g = ub[(static_cast<size_t>(b) * Hq + h * G) * max_pages + p];
#pragma unroll
    for (int j = 1; j < G; ++j)
      g = fmaxf(g, ub[(static_cast<size_t>(b) * Hq + h * G + j) * max_pages + p]);
    keys[p] = order_key(g);
  }
  __syncthreads();

  // Radix select of the kk-th largest key, most significant digit first.
  uint32_t prefix = 0, mask = 0;
  int need = kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int p = tid; p < np; p += kTopkThreads) {
      const uint32_t key = keys[p];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < kWave) {
      // Lane l owns digits 255-4l .. 252-4l (descending).
      int c[4], local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * tid - j];
        local += c[j];
      }
      const int incl = wave_incl_scan(local);
      int before = incl - local;  // keys with a larger digit
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < need && before + c[j] >= need) {
          s_digit = static_cast<uint32_t>(255 - 4 * tid - j);
          s_need = need - before;
        }
        before += c[j];
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    need = s_need;
    __syncthreads();
  }
  const uint32_t T = prefix;  // key of the kk-th largest; `need` ties taken

  // Ordered compaction.  Thread t owns pages [t*per, (t+1)*per).
  const int per = (np + kTopkThreads - 1) / kTopkThreads;
  const int p0 = tid * per, p1 = min(np, p0 + per);
  int n_eq = 0;
  for (int p = p0; p < p1; ++p) n_eq += (keys[p] == T);
  int tot;
  int eq_rank = block_excl_scan<kTopkThreads>(n_eq, scan_tmp, tot);
  int n_sel = 0;
  {
    int r = eq_rank;
    for (int p = p0; p < p1; ++p) {
      const uint32_t key = keys[p];
      if (key > T) ++n_sel;
      else if (key == T) { n_sel += (r < need); ++r; }
    }
  }
  int pos = block_excl_scan<kTopkThreads>(n_sel, scan_tmp, tot);
  {
    int r = eq_rank;
    for (int p = p0; p < p1; ++p) {
      const uint32_t key = keys[p];
      bool take = key > T;
      if (key == T) { take = r < need; ++r; }
      if (take) out[pos++] = p;
    }
  }
  if (tid == 0) count[u] = kk;
}

// ---------------------------------------------------------------------------
// Gaussian threshold estimate.  One 256-thread block per query head.
//   m_p = (alpha-1) mu_p, s_p = (alpha-1) sigma_p, n_p valid tokens.
//   F(tau) = sum_p n_p E[max(Z_p - tau, 0)^r],  Z_p ~ N(m_p, s_p^2).
// F is decreasing and convex, and so is F^(1/r) (an L^r norm of a convex
// non-negative function of tau).  Newton's method on F^(1/r) - 1 started at
// tau_lo = max_p m_p - 1 (where F >= 1) therefore climbs monotonically to the
// root without overshooting.  Pages with m_p + 8.5 s_p <= tau_lo contribute
// less than ~1e-17 each for every tau >= tau_lo and are left out; the others
// are compacted, in page order, into LDS (global fallback when too many).
// ---------------------------------------------------------------------------
constexpr int kGaussThreads = 256;
constexpr int kGaussCap = 4096;  // pages kept in LDS per head

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

__global__ __launch_bounds__(kGaussThreads) void k_gauss_tau(
    const float *__restrict__ gstat, const int32_t *__restrict__ seq_lens,
    int Hq, int P, int max_pages, float am1, int r,
    float *__restrict__ tau_hat) {
  __shared__ float s_m[kGaussCap], s_s[kGaussCap], s_n[kGaussCap];
  __shared__ float red_f[kGaussThreads / kWave];
  __shared__ double red_d[kGaussThreads / kWave];
  __shared__ int red_i[kGaussThreads / kWave];
  const int bh = blockIdx.x, b = bh / Hq;
  const int tid = threadIdx.x;
  const int len = seq_lens[b];
  const int np = n_pages_of(len, P);
  const float2 *st = reinterpret_cast<const float2 *>(gstat) +
                     static_cast<size_t>(bh) * max_pages;

  // 1. Largest page mean.
  float mmax = -FLT_MAX;
  for (int p = tid; p < np; p += kGaussThreads) mmax = fmaxf(mmax, am1 * st[p].x);
  mmax = block_max<kGaussThreads>(mmax, red_f);
  const float tau_lo = mmax - 1.0f;

  // 2. Ordered compaction of the pages that can matter.
  const int per = (np + kGaussThreads - 1) / kGaussThreads;
  const int p0 = tid * per, p1 = min(np, p0 + per);
  auto alive = [&](int p, float &m, float &s) {
    const float2 v = st[p];
    m = am1 * v.x;
    s = am1 * sqrtf(fmaxf(v.y, 0.f));
    return m + 8.5f * s > tau_lo;
  };
  int n_alive = 0;
  for (int p = p0; p < p1; ++p) {
    float m, s;
    n_alive += alive(p, m, s);
  }
  int n_surv;
  int pos = block_excl_scan<kGaussThreads>(n_alive, red_i, n_surv);
  const bool in_lds = n_surv <= kGaussCap;
  if (in_lds) {
    for (int p = p0; p < p1; ++p) {
      float m, s;
      if (alive(p, m, s)) {
        s_m[pos] = m;
        s_s[pos] = s;
        s_n[pos] = static_cast<float>(page_tokens(p, len, P));
        ++pos;
      }
    }
  }
  __syncthreads();

  // 3. Newton on F^(1/r) - 1 from tau_lo.
  float tau = tau_lo;
  for (int it = 0; it < 64; ++it) {
    double f = 0.0, df = 0.0;
    if (in_lds) {
      for (int i = tid; i < n_surv; i += kGaussThreads) {
        const GaussTerm t = gauss_term(s_m[i], s_s[i], s_n[i], tau, r);
        f += t.f;
        df += t.df;
      }
    } else {
      for (int p = p0; p < p1; ++p) {
        float m, s;
        if (alive(p, m, s)) {
          const GaussTerm t = gauss_term(
              m, s, static_cast<float>(page_tokens(p, len, P)), tau, r);
          f += t.f;
          df += t.df;
        }
      }
    }
    f = block_sum_d<kGaussThreads>(f, red_d);
    df = block_sum_d<kGaussThreads>(df, red_d);
    if (!(f > 1.0) || !(df > 0.0)) break;  // at (or rounding past) the root
    const double step = (r == 2) ? 2.0 * (f - sqrt(f)) / df : (f - 1.0) / df;
    const float next = static_cast<float>(static_cast<double>(tau) + step);
    if (!(next > tau)) break;  // no representable progress left
    tau = next;
  }
  if (tid == 0) tau_hat[bh] = tau;
}

// ---------------------------------------------------------------------------
// Gaussian keep test and ordered compaction.  One block per unit.
// ---------------------------------------------------------------------------
constexpr int kKeepThreads = 1024;

template <int G>
__global__ __launch_bounds__(kKeepThreads) void k_gauss_keep(
    const float *__restrict__ gstat, const int32_t *__restrict__ seq_lens,
    const float *__restrict__ tau_hat, int H, int P, int max_pages, float am1,
    float delta, int32_t *__restrict__ sel, int32_t *__restrict__ count) {
  __shared__ int scan_tmp[kKeepThreads / kWave];
  __shared__ float s_gap[kKeepThreads / kWave];
  __shared__ int s_idx[kKeepThreads / kWave];
  const int u = blockIdx.x, b = u / H, h = u % H;
  const int tid = threadIdx.x;
  const int len = seq_lens[b];
  const int np = n_pages_of(len, P);
  const int Hq = H * G;
  const float2 *st = reinterpret_cast<const float2 *>(gstat) +
                     (static_cast<size_t>(b) * Hq + h * G) * max_pages;
  float cut[G];
#pragma unroll
  for (int g = 0; g < G; ++g) cut[g] = tau_hat[b * Hq + h * G + g];
  const float full_c = sqrtf(2.0f * logf(static_cast<float>(P)));

  // Largest margin (alpha-1) mhat - tau_hat over the group for page p.
  auto margin = [&](int p) {
    const float c = (p == np - 1) ? sqrtf(2.0f * logf(static_cast<float>(
                                        page_tokens(p, len, P))))
                                  : full_c;
    float best = -FLT_MAX;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float2 v = st[static_cast<size_t>(g) * max_pages + p];
      const float zhat = am1 * (v.x + sqrtf(fmaxf(v.y, 0.f)) * c);
      best = fmaxf(best, zhat - cut[g]);
    }
    return best;
  };
  // keep <=> exists g: zhat_g > cut_g - delta; evaluated per head to match
  // the definition rather than through the margin.
  auto keep = [&](int p) {
    const float c = (p == np - 1) ? sqrtf(2.0f * logf(static_cast<float>(
                                        page_tokens(p, len, P))))
                                  : full_c;
    bool k = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float2 v = st[static_cast<size_t>(g) * max_pages + p];
      const float zhat = am1 * (v.x + sqrtf(fmaxf(v.y, 0.f)) * c);
      k |= zhat > cut[g] - delta;
    }
    return k;
  };

  const int per = (np + kKeepThreads - 1) / kKeepThreads;
  const int p0 = tid * per, p1 = min(np, p0 + per);
  int n_keep = 0;
  for (int p = p0; p < p1; ++p) n_keep += keep(p);
  int total;
  int pos = block_excl_scan<kKeepThreads>(n_keep, scan_tmp, total);
  int32_t *out = sel + static_cast<size_t>(u) * max_pages;
  for (int p = p0; p < p1; ++p)
    if (keep(p)) out[pos++] = p;
  if (total > 0) {
    if (tid == 0) count[u] = total;
    return;
  }
  // Nothing kept: the page with the largest margin, lower index on ties.
  float best = -FLT_MAX;
  int bi = np;
  for (int p = p0; p < p1; ++p) {
    const float m = margin(p);
    if (m > best) { best = m; bi = p; }
  }
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float om = __shfl_xor(best, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    if (om > best || (om == best && oi < bi)) { best = om; bi = oi; }
  }
  if ((tid & (kWave - 1)) == 0) {
    s_gap[tid / kWave] = best;
    s_idx[tid / kWave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kKeepThreads / kWave; ++w)
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
  hipLaunchKernelGGL((k_select_topk<G>), dim3(units), dim3(kTopkThreads), 0,
                     stream, ub, kv.seq_lens, kv.num_kv_heads, kv.page_size,
                     kv.max_pages, k, sel, count,
                     static_cast<uint32_t *>(ws));
  return hipGetLastError();
}

template <int G>
hipError_t launch_select_gauss(const ekv_paged_kv &kv, const float *gstat,
                               float alpha, float delta, int32_t *sel,
                               int32_t *count, float *tau_hat,
                               hipStream_t stream) {
  const int Hq = kv.num_kv_heads * G;
  const int r = alpha == 2.0f ? 1 : 2;
  const float am1 = alpha - 1.0f;
  hipLaunchKernelGGL(k_gauss_tau, dim3(kv.batch * Hq), dim3(kGaussThreads), 0,
                     stream, gstat, kv.seq_lens, Hq, kv.page_size,
                     kv.max_pages, am1, r, tau_hat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gauss_keep<G>), dim3(kv.batch * kv.num_kv_heads),
                     dim3(kKeepThreads), 0, stream, gstat, kv.seq_lens,
                     tau_hat, kv.num_kv_heads, kv.page_size, kv.max_pages,
                     am1, delta, sel, count);
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
