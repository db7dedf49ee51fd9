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
    const int32_t *__restrict__ first_page, int last_only, int H, int P,
    int max_pages, typename E::T *__restrict__ bbox,
    float *__restrict__ gauss) {
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
  int p0 = last_only ? np - 1 : first_page ? first_page[b] : 0;
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
// 64-page tile, summaries the selectors use to skip tiles:
//   box:       max over the tile's pages and the group's heads of the bound;
//   Gaussian:  per query head max mu, max (mu + 8.5 sigma) and
//              max (mu + sqrt(2 ln P) sigma).
// They live after the per-page values in the same buffers (see entmaxkv.h).
//
// Two waves score one tile of one (sequence, KV head) unit at a time, each
// half of its pages: D/8 lanes per page (8 coordinates per lane, see
// coord_of), 64*8/D pages per step.  (Twice as many waves as tiles keep the
// read stream fuller: with one wave per tile a 1M-token batch gives only two
// waves per SIMD.)  The two waves of a tile sit in one block and merge their
// halves' tile summaries through LDS; all waves of a block walk their items
// in the same rounds, so every wave reaches every barrier.  The box bound uses max(q kmin, q kmax) per coordinate, that is
// q kmax where q > 0 and q kmin elsewhere (kmin <= kmax): one product per
// coordinate, the larger of the two rounded ones.
//
// The metadata loads run kScoreRing steps ahead of the arithmetic: as soon
// as a step's registers have been used they are refilled with the step
// kScoreRing further on, past the end of a half tile with the first steps of
// the wave's next one, so each wave streams its records without a break.  Every
// load is unconditional (pages past a sequence's end re-read its last page),
// which keeps the compiler's counts of loads in flight exact; a load behind a
// branch would make it wait for all of them.  Tiles are numbered over those
// that hold at least one page (a per-sequence prefix that every block builds
// in LDS), KV head fastest, and dealt to the wave pairs in turn: the waves
// running together read every head's record of the same slots, one
// contiguous stretch of the pool.  The query heads of a wave's next tile are
// staged through the wave's own LDS rows while the current tile is scored.
// ---------------------------------------------------------------------------
constexpr int kScoreTile = kPageTile;
constexpr int kScoreWaves = 4;
constexpr int kScoreThreads = kScoreWaves * kWave;
constexpr int kScoreRing = 2;
constexpr int kScorePairs = kScoreWaves / 2;
constexpr int kScoreHalf = kPageTile / 2;  // pages per wave of a tile
// Waves per SIMD the compiler is held to where that costs no spills: one
// kind of record with up to four query heads per KV head (not float32 boxes
// with four, whose 32-byte rows need more registers); four for bfloat16
// keys, three for float32 keys (whose tail-page rebuild holds a coordinate's
// 64 values).  Elsewhere it may use the whole register file.
template <class T, int G, int MODE>
constexpr int score_min_waves() {
  if (MODE != EKV_SCORE_BBOX && MODE != EKV_SCORE_GAUSS) return 1;
  if (G > 4) return 1;
  if (G == 4 && MODE == EKV_SCORE_BBOX && sizeof(T) == 4) return 1;
  return sizeof(T) == 2 ? 4 : 3;
}

// The 8 coordinates of a row that a lane holds, as loaded (see coord_of).
template <class T> struct Raw8;
template <> struct Raw8<float> { float4 a, b; };
template <> struct Raw8<uint16_t> { uint4 a; };

template <int D>
__device__ __forceinline__ Raw8<float> load_raw8(const float *row, int li) {
  Raw8<float> r;
  r.a = *reinterpret_cast<const float4 *>(row + 4 * li);
  r.b = *reinterpret_cast<const float4 *>(row + D / 2 + 4 * li);
  return r;
}
template <int D>
__device__ __forceinline__ Raw8<uint16_t> load_raw8(const uint16_t *row, int li) {
  Raw8<uint16_t> r;
  r.a = *reinterpret_cast<const uint4 *>(row + 8 * li);
  return r;
}
__device__ __forceinline__ void unpack8(const Raw8<float> &r, float (&x)[8]) {
  x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
  x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}
__device__ __forceinline__ void unpack8(const Raw8<uint16_t> &r, float (&x)[8]) {
  x[0] = bf16_lo(r.a.x); x[1] = bf16_hi(r.a.x);
  x[2] = bf16_lo(r.a.y); x[3] = bf16_hi(r.a.y);
  x[4] = bf16_lo(r.a.z); x[5] = bf16_hi(r.a.z);
  x[6] = bf16_lo(r.a.w); x[7] = bf16_hi(r.a.w);
}

// Max over the lane groups of a wave of a value that is uniform within each
// group of W lanes.
template <int W>
__device__ __forceinline__ float cross_group_max(float x) {
  if constexpr (W < 16) x = fmaxf(x, dpp_f<kDppRowMirror>(x));
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  return fmaxf(x, __shfl_xor(x, 32, kWave));
}

// Keeps a running tile maximum computed at the step that produced it.  The
// maxima are only read after a tile's last step, and without this the
// compiler moves every step's update there, holding all the steps' sums in
// registers at once.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

// One step's records as loaded: box rows (min, max) and/or Gaussian rows
// (mean, variance).  Members a mode does not use are never touched.
template <class T>
struct ScoreStep {
  Raw8<T> lo, hi;
  Raw8<float> mean, var;
};

struct ScoreItem {
  int b, h, tile, np;
};

// Rebuild of one page's metadata for one KV head by a single wave, equal bit
// for bit to what k_build_meta computes: per coordinate, partial sums over
// the token groups tg, tg + TG, ... of a k_build_meta block, each taken in
// token order from zero, then added in group order; the variance the same
// way about the mean; minima and maxima do not depend on order.  Lane l
// owns coordinates l*CPL .. l*CPL + CPL - 1 and holds all n <= 64 tokens of
// them.  Null bbox or gauss skips that part.
template <class E, int D>
__device__ __forceinline__ void rebuild_page_meta(const typename E::T *kpool, int slot, int h,
                                  int H, int P, int n, typename E::T *bbox,
                                  float *gauss) {
  using T = typename E::T;
  constexpr int CPL = D / kWave;            // coordinates per lane
  constexpr int CG = D / 8;                 // coordinate groups of a block
  constexpr int TG = kMetaThreads / CG;     // token groups of a block
  constexpr int MAXT = (64 + TG - 1) / TG;  // tokens per group (P <= 64)
  const int lane = threadIdx.x & (kWave - 1);
  // The page's n valid rows as a range-checked buffer: rows past n read as
  // zero (and are masked below), so all 64 loads are unconditional and in
  // flight at once, each with the lane's offset and a constant row offset.
  const __amdgpu_buffer_rsrc_t rows = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(kpool + pool_row(slot, h, 0, H, P, D)),
      static_cast<short>(0), n * D * static_cast<int>(sizeof(T)), 0x00020000);
  // Statistics of coordinate lane * CPL + c from its n values xv(t).
  auto stats = [&](auto xv, int c) {
    float mn = INFINITY, mx = -INFINITY, s = 0.f;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < MAXT; ++i) {
        const int t = tg + i * TG;
        if (t < 64 && t < n) {
          const float x = xv(t);
          mn = fminf(mn, x);
          mx = fmaxf(mx, x);
          part += x;
        }
      }
      s = tg == 0 ? part : s + part;
    }
    const float mean = s / static_cast<float>(n);
    float v = 0.f;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < MAXT; ++i) {
        const int t = tg + i * TG;
        if (t < 64 && t < n) {
          const float dv = xv(t) - mean;
          part = fmaf(dv, dv, part);
        }
      }
      v = tg == 0 ? part : v + part;
    }
    const int d = lane * CPL + c;
    if (bbox) {
      store1(bbox + meta_row(slot, h, 0, H, D) + d, mn);
      store1(bbox + meta_row(slot, h, 1, H, D) + d, mx);
    }
    if (gauss) {
      gauss[meta_row(slot, h, 0, H, D) + d] = mean;
      gauss[meta_row(slot, h, 1, H, D) + d] = v / static_cast<float>(n);
    }
  };
  if constexpr (sizeof(T) == 2 && CPL == 2) {
    // A lane's two bfloat16 coordinates are adjacent: one 4-byte load per
    // token brings both (the lower address in the low half), so the page is
    // read once, with all 64 loads in flight together.
    uint32_t w[64];
#pragma unroll
    for (int t = 0; t < 64; ++t)
      w[t] = __builtin_amdgcn_raw_buffer_load_b32(rows, lane * 4, t * D * 2, 0);
    // (the values are unpacked at each use rather than kept unpacked: the
    // empty asm stops the compiler from holding 64 more registers)
    auto half = [&](int t, uint32_t mask, int sh) {
      uint32_t x = w[t];
      asm volatile("" : "+v"(x));
      return __uint_as_float((x << sh) & mask);
    };
    stats([&](int t) { return half(t, 0xffff0000u, 16); }, 0);
    stats([&](int t) { return half(t, 0xffff0000u, 0); }, 1);
  } else {
    // One coordinate at a time, its n tokens in registers (the second read
    // of the rows comes from the cache).
#pragma unroll 1
    for (int c = 0; c < CPL; ++c) {
      const int voff = (lane * CPL + c) * static_cast<int>(sizeof(T));
      float x[64];
#pragma unroll
      for (int t = 0; t < 64; ++t) {
        const int soff = t * D * static_cast<int>(sizeof(T));
        if constexpr (sizeof(T) == 2)
          x[t] = __uint_as_float(static_cast<uint32_t>(
                                     __builtin_amdgcn_raw_buffer_load_b16(rows, voff, soff, 0))
                                 << 16);
        else
          x[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rows, voff, soff, 0));
      }
      stats([&](int t) { return x[t]; }, c);
    }
  }
}

template <class E, int D, int G, int MODE, bool REFRESH>
__global__ __launch_bounds__(kScoreThreads, (score_min_waves<typename E::T, G, MODE>())) void k_score(
    const typename E::T *bbox, const float *gauss,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const float *__restrict__ q,
    float scale, int H, int P, int max_pages, int batch,
    float *__restrict__ ub, float *__restrict__ gstat,
    const typename E::T *__restrict__ kpool, typename E::T *bbox_w,
    float *gauss_w) {
  using T = typename E::T;
  constexpr bool kBox = (MODE & EKV_SCORE_BBOX) != 0;
  constexpr bool kGauss = (MODE & EKV_SCORE_GAUSS) != 0;
  constexpr int LPP = D / 8;               // lanes per page
  constexpr int PPS = kWave / LPP;         // pages per step
  constexpr int NSTEP = kScoreHalf / PPS;  // steps per half tile
  constexpr int R = kScoreRing;
  constexpr int QF = G * D / kWave;        // staged query floats per lane
  static_assert(kScoreTile == kWave, "one page-table entry per lane");
  static_assert(NSTEP >= R, "the ring must fit in a half tile");
  static_assert(QF == 1 || QF == 2 || QF % 4 == 0, "query staging width");
  // the wave index (and everything derived from it) is wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int pair = wave >> 1, half = wave & 1;
  const int sub = lane / LPP, li = lane % LPP;
  const int Hq = H * G;
  const int n_tiles = (max_pages + kScoreTile - 1) / kScoreTile;

  constexpr bool refresh = REFRESH;
  // LDS: per wave G*D staged query floats, then per sequence the prefix of
  // its tiles (batch + 1 entries), its page count (batch entries) and, when
  // refreshing, the prefix of non-empty sequences (batch + 1 entries).  When
  // refreshing, the last tile of every non-empty sequence comes first in the
  // numbering (and the main prefix counts the other tiles), so that each is
  // the first item of some wave pair (the host checks there are enough pairs).
  extern __shared__ float4 s_dyn4[];
  float *s_q = reinterpret_cast<float *>(s_dyn4) + wave * G * D;
  int *s_pref = reinterpret_cast<int *>(s_dyn4) + kScoreWaves * G * D;
  int *s_np = s_pref + batch + 1;
  int *s_plast = s_np + batch;
  __shared__ int s_tmp[kScoreWaves];
  // the second half's tile summaries, for the first half to merge (two
  // buffers, alternating by round)
  __shared__ float4 s_tg[2][kScorePairs][G];
  __shared__ float s_tb[2][kScorePairs];
  // a wave's (mu, sigma^2) of its half tile, [query head][page], written
  // out in two coalesced stores at the half tile's end (a store per step,
  // four scattered 32-byte pieces each, held up the record loads behind it)
  __shared__ float2 s_gp[kScoreWaves][kGauss ? G * kScoreHalf : 1];
  {
    const int per = (batch + kScoreThreads - 1) / kScoreThreads;
    const int b0 = min(batch, threadIdx.x * per), b1 = min(batch, b0 + per);
    auto tiles_main = [&](int np) {
      const int nt = (np + kScoreTile - 1) / kScoreTile;
      return refresh ? max(nt - 1, 0) : nt;
    };
    int local = 0, local_last = 0;
    for (int b = b0; b < b1; ++b) {
      // pages of sequence b, clamped to its page-table row
      const int np = max(0, min(n_pages_of(seq_lens[b], P), max_pages));
      s_np[b] = np;
      local += tiles_main(np);
      local_last += refresh && np > 0;
    }
    int total, total_last = 0, base_last = 0;
    int base = block_excl_scan<kScoreThreads>(local, s_tmp, total);
    if constexpr (REFRESH)
      base_last = block_excl_scan<kScoreThreads>(local_last, s_tmp, total_last);
    for (int b = b0; b < b1; ++b) {
      s_pref[b] = base;
      base += tiles_main(s_np[b]);
      s_plast[b] = base_last;
      base_last += refresh && s_np[b] > 0;
    }
    if (threadIdx.x == 0) {
      s_pref[batch] = total;
      s_plast[batch] = total_last;
    }
    lds_barrier();
  }
  const int n_last = REFRESH ? s_plast[batch] : 0;
  const int n_items = (s_pref[batch] + n_last) * H;
  const int n_pairs = gridDim.x * kScorePairs;
  // The block's items this round are itb .. itb + kScorePairs - 1; a pair
  // whose item is past the end re-reads the last item and stores nothing.
  int itb = blockIdx.x * kScorePairs;
  if (itb >= n_items) return;  // the whole block
  int it = itb + pair;

  // items only move forward, and so do their sequences in each part
  int blast = 0, bscan = 0;
  auto describe = [&](int i) {
    const int ts = i / H;
    ScoreItem d;
    d.h = i - ts * H;
    if (REFRESH && ts < n_last) {  // a sequence's last tile (refreshing only)
      while (s_plast[blast + 1] <= ts) ++blast;
      d.b = __builtin_amdgcn_readfirstlane(blast);
      d.np = __builtin_amdgcn_readfirstlane(s_np[blast]);
      d.tile = (d.np - 1) / kScoreTile;
    } else {
      const int tm = ts - n_last;
      while (s_pref[bscan + 1] <= tm) ++bscan;
      d.b = __builtin_amdgcn_readfirstlane(bscan);
      d.np = __builtin_amdgcn_readfirstlane(s_np[bscan]);
      d.tile = __builtin_amdgcn_readfirstlane(tm - s_pref[bscan]);
    }
    return d;
  };
  // Slot of page (tile * 64 + lane), clamped to the sequence's last page
  // (each wave loads the whole tile's and uses its half).
  auto load_slots = [&](const ScoreItem &d) {
    const int lp = min(d.tile * kScoreTile + lane, d.np - 1);
    return page_table[static_cast<size_t>(d.b) * max_pages + lp];
  };
  auto issue = [&](ScoreStep<T> &st, const ScoreItem &d, int slots, int t) {
    const int slot = __shfl(slots, half * kScoreHalf + t * PPS + sub, kWave);
    if constexpr (kBox) {
      const T *rb = bbox + meta_row(slot, d.h, 0, H, D);
      st.lo = load_raw8<D>(rb, li);
      st.hi = load_raw8<D>(rb + D, li);
    }
    if constexpr (kGauss) {
      const float *rg = gauss + meta_row(slot, d.h, 0, H, D);
      st.mean = load_raw8<D>(rg, li);
      st.var = load_raw8<D>(rg + D, li);
    }
  };
  // The G query rows of a unit are contiguous; lane l holds floats
  // [l QF, (l + 1) QF) of them.
  auto load_q = [&](const ScoreItem &d, float (&v)[QF]) {
    const float *src = q + (static_cast<size_t>(d.b) * Hq + d.h * G) * D + lane * QF;
    if constexpr (QF % 4 == 0) {
#pragma unroll
      for (int c = 0; c < QF / 4; ++c) {
        const float4 x = reinterpret_cast<const float4 *>(src)[c];
        v[4 * c] = x.x; v[4 * c + 1] = x.y; v[4 * c + 2] = x.z; v[4 * c + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < QF; ++j) v[j] = src[j];
    }
  };
  auto stage_q = [&](const float (&v)[QF]) {
#pragma unroll
    for (int j = 0; j < QF; ++j) s_q[lane * QF + j] = v[j] * scale;
  };

  float qv[QF];
  ScoreItem cur = describe(min(it, n_items - 1));
  bool real = it < n_items;
  if (REFRESH && real && it < n_last * H &&
      half == ((cur.np - 1) % kScoreTile) / kScoreHalf) {
    // This pair's first tile is the last tile of its sequence, and this
    // wave's half holds the last page: rebuild that page's metadata for this
    // KV head before any of the half's records is read (the other half never
    // uses the page).  The fence makes the wave's stores visible to its own
    // later loads.
    // (read by every lane from one address: uniform, kept in scalars)
    const int lp = cur.np - 1;
    const int slot = __builtin_amdgcn_readfirstlane(
        page_table[static_cast<size_t>(cur.b) * max_pages + lp]);
    const int n = __builtin_amdgcn_readfirstlane(page_tokens(lp, seq_lens[cur.b], P));
    rebuild_page_meta<E, D>(kpool, slot, cur.h, H, P, n, bbox_w, gauss_w);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  // The first records are requested as soon as the page-table rows are in;
  // the query rows, requested after those rows, are staged behind them.
  int slots_cur = load_slots(cur);
  load_q(cur, qv);
  ScoreStep<T> ring[R];
#pragma unroll
  for (int t = 0; t < R; ++t) issue(ring[t], cur, slots_cur, t);
  __builtin_amdgcn_sched_barrier(0);
  stage_q(qv);
  const float cP = sqrtf(2.0f * logf(static_cast<float>(P)));
  float2 *gpage = reinterpret_cast<float2 *>(gstat);
  float4 *gtile = reinterpret_cast<float4 *>(gstat + gstat_tile_offset(batch, Hq, max_pages));

  int par = 0;
  while (true) {
    const int it_next = it + n_pairs;
    const bool more = itb + n_pairs < n_items;  // the same for the block
    const ScoreItem nxt = more ? describe(min(it_next, n_items - 1)) : cur;
    const int slots_next = load_slots(nxt);
    load_q(nxt, qv);

    // this tile's query heads: scale * q at the lane's coordinates
    float qs[G][8], qb[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (kGauss) qs[g][j] = s_q[g * D + coord_of<float, D>(li, j)];
        if constexpr (kBox) {
          const float x = s_q[g * D + coord_of<T, D>(li, j)];
          qb[g][j] = x;
        }
      }
    const size_t row0 = (static_cast<size_t>(cur.b) * Hq + cur.h * G) * max_pages;
    float tmax = -FLT_MAX;
    float t_mu[G], t_pr[G], t_kp[G];
#pragma unroll
    for (int g = 0; g < G; ++g) { t_mu[g] = -FLT_MAX; t_pr[g] = -FLT_MAX; t_kp[g] = -FLT_MAX; }

#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      ScoreStep<T> &st = ring[s % R];
      const int lp = cur.tile * kScoreTile + half * kScoreHalf + s * PPS + sub;
      const bool valid = real && lp < cur.np;
      if constexpr (kBox) {
        float kmin[8], kmax[8];
        unpack8(st.lo, kmin);
        unpack8(st.hi, kmax);
        float acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            a = fmaf(qb[g][j], qb[g][j] > 0.f ? kmax[j] : kmin[j], a);
          }
          acc[g] = group_sum<LPP>(a);
        }
        float gm = acc[0], mine = acc[0];
#pragma unroll
        for (int g = 1; g < G; ++g) {
          gm = fmaxf(gm, acc[g]);
          mine = li == g ? acc[g] : mine;
        }
        tmax = valid ? fmaxf(tmax, gm) : tmax;
        pin(tmax);
        if (valid && li < G) ub[row0 + static_cast<size_t>(li) * max_pages + lp] = mine;
      }
      if constexpr (kGauss) {
        float mean[8], var[8];
        unpack8(st.mean, mean);
        unpack8(st.var, var);
        float mu[G], s2[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = 0.f, c = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = qs[g][j];
            a = fmaf(x, mean[j], a);
            c = fmaf(x, x * var[j], c);
          }
          mu[g] = group_sum<LPP>(a);
          s2[g] = group_sum<LPP>(c);
        }
        float2 mine = make_float2(mu[0], s2[0]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float sd = sqrtf(fmaxf(s2[g], 0.f));
          t_mu[g] = valid ? fmaxf(t_mu[g], mu[g]) : t_mu[g];
          t_pr[g] = valid ? fmaxf(t_pr[g], mu[g] + 8.5f * sd) : t_pr[g];
          t_kp[g] = valid ? fmaxf(t_kp[g], mu[g] + cP * sd) : t_kp[g];
          if (g > 0 && li == g) mine = make_float2(mu[g], s2[g]);
          pin(t_mu[g]);
          pin(t_pr[g]);
          pin(t_kp[g]);
        }
        if (li < G) s_gp[wave][li * kScoreHalf + s * PPS + sub] = mine;
      }
      // refill: the step R further on, in this half tile or the wave's next
      // one (none after its last)
      if (s + R < NSTEP) issue(st, cur, slots_cur, s + R);
      else if (more) issue(st, nxt, slots_next, s + R - NSTEP);
    }

    if constexpr (kGauss) {
      const int base = cur.tile * kScoreTile + half * kScoreHalf;
#pragma unroll
      for (int e0 = 0; e0 < G * kScoreHalf; e0 += kWave) {
        const int e = e0 + lane;
        const int gg = e / kScoreHalf, pg = e % kScoreHalf;
        if (e < G * kScoreHalf && real && base + pg < cur.np)
          gpage[row0 + static_cast<size_t>(gg) * max_pages + base + pg] = s_gp[wave][e];
      }
    }
    // Tile summaries: the second half's go through LDS to the first half,
    // which writes the tile's (its first page is valid, so the first half
    // holds at least one valid page; a half without one contributes
    // -FLT_MAX).
    float4 gsum = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (kBox) {
      tmax = cross_group_max<LPP>(tmax);
      if (half == 1 && lane == 0) s_tb[par][pair] = tmax;
    }
    if constexpr (kGauss) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float a0 = cross_group_max<LPP>(t_mu[g]);
        const float a1 = cross_group_max<LPP>(t_pr[g]);
        const float a2 = cross_group_max<LPP>(t_kp[g]);
        if (lane == g) gsum = make_float4(a0, a1, a2, 0.f);
      }
      if (half == 1 && lane < G) s_tg[par][pair][lane] = gsum;
    }
    lds_barrier();
    if (half == 0 && real) {
      if constexpr (kBox) {
        if (lane == 0)
          ub[static_cast<size_t>(batch) * Hq * max_pages +
             (static_cast<size_t>(cur.b) * H + cur.h) * n_tiles + cur.tile] =
              fmaxf(tmax, s_tb[par][pair]);
      }
      if constexpr (kGauss) {
        if (lane < G) {
          const float4 o = s_tg[par][pair][lane];
          gsum = make_float4(fmaxf(gsum.x, o.x), fmaxf(gsum.y, o.y), fmaxf(gsum.z, o.z), 0.f);
          gtile[(static_cast<size_t>(cur.b) * Hq + cur.h * G + lane) * n_tiles + cur.tile] = gsum;
        }
      }
    }
    if (!more) break;
    // this tile's query reads are done (their values are in registers)
    stage_q(qv);
    cur = nxt;
    slots_cur = slots_next;
    it = it_next;
    itb += n_pairs;
    real = it < n_items;
    par ^= 1;
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
                     kv.seq_lens, first_page, 0, kv.num_kv_heads, kv.page_size,
                     kv.max_pages, static_cast<typename E::T *>(meta.bbox),
                     meta.gauss);
  return hipGetLastError();
}

// Waves stay resident and walk their tiles; the grid is as many blocks as fit
// on the device at once (fewer if there are fewer tiles than waves).
// With `refresh`, the metadata of every sequence's last page is rebuilt
// first: inside the scoring launch when every (sequence, KV head) gets a
// wave of its own, else by a one-page metadata launch before it.
template <class E, int D, int G>
hipError_t launch_score(const ekv_paged_kv &kv, const ekv_meta &meta,
                        const float *q, float scale, int mode, float *ub,
                        float *gstat, bool refresh, hipStream_t stream) {
  using T = typename E::T;
  const long long items = static_cast<long long>(page_tiles(kv)) *
                          kv.num_kv_heads * kv.batch;
  const size_t lds = static_cast<size_t>(kScoreWaves) * G * D * sizeof(float) +
                     (3 * static_cast<size_t>(kv.batch) + 2) * sizeof(int);
  hipError_t err = hipSuccess;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n_cu <= 0)
    n_cu = 256;
  auto grid_of = [&](auto kern) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(kern), kScoreThreads, lds) !=
            hipSuccess || per_cu <= 0)
      per_cu = 1;
    const long long want = (items + kScorePairs - 1) / kScorePairs;
    return static_cast<int>(
        std::min<long long>(want, static_cast<long long>(n_cu) * per_cu));
  };
  auto launch = [&](auto kern, int blocks) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kScoreThreads), lds, stream,
                       static_cast<const T *>(meta.bbox), meta.gauss,
                       kv.page_table, kv.seq_lens, q, scale, kv.num_kv_heads,
                       kv.page_size, kv.max_pages, kv.batch, ub, gstat,
                       static_cast<const T *>(kv.k), static_cast<T *>(meta.bbox),
                       meta.gauss);
    err = hipGetLastError();
  };
  // the fused form needs a wave pair for every (sequence, KV head)
  auto run = [&](auto plain, auto fused) {
    if (refresh) {
      const int nb = grid_of(fused);
      if (static_cast<long long>(kv.batch) * kv.num_kv_heads <=
          static_cast<long long>(nb) * kScorePairs) {
        launch(fused, nb);
        return;
      }
      hipLaunchKernelGGL((k_build_meta<E, D>), dim3(1, kv.num_kv_heads, kv.batch),
                         dim3(kMetaThreads), 0, stream,
                         static_cast<const T *>(kv.k), kv.page_table,
                         kv.seq_lens, nullptr, 1, kv.num_kv_heads, kv.page_size,
                         kv.max_pages, static_cast<T *>(meta.bbox), meta.gauss);
      if ((err = hipGetLastError()) != hipSuccess) return;
    }
    launch(plain, grid_of(plain));
  };
  constexpr int kBoth = EKV_SCORE_BBOX | EKV_SCORE_GAUSS;
  if (mode == EKV_SCORE_BBOX)
    run(k_score<E, D, G, EKV_SCORE_BBOX, false>, k_score<E, D, G, EKV_SCORE_BBOX, true>);
  else if (mode == EKV_SCORE_GAUSS)
    run(k_score<E, D, G, EKV_SCORE_GAUSS, false>, k_score<E, D, G, EKV_SCORE_GAUSS, true>);
  else
    run(k_score<E, D, G, kBoth, false>, k_score<E, D, G, kBoth, true>);
  return err;
}

#define EKV_INST_META(E, D)                                                 \
  template hipError_t launch_build_meta<E, D>(const ekv_paged_kv &,         \
                                              const int32_t *, int,         \
                                              const ekv_meta &, hipStream_t);
#define EKV_INST_SCORE(E, D, G)                                             \
  template hipError_t launch_score<E, D, G>(                                \
      const ekv_paged_kv &, const ekv_meta &, const float *, float, int,    \
      float *, float *, bool, hipStream_t);

EKV_FOR_EACH_ED(EKV_INST_META)
EKV_FOR_EACH_EDG(EKV_INST_SCORE)

}  // namespace ekv
