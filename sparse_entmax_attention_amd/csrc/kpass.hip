// Key scores of the selected pages (Technical Summary: EntmaxKV, §2.C
// "Sparse Entmax Attention"): z = (alpha-1) scale <q, k> for every token of
// every selected page and query head, each page's maximum per head, and the
// page's pool slot, for the threshold and apply steps of decode.hip.  Reads
// the selected keys once; HBM-bound.
//
// With a threshold hint per query head (the Gaussian selector's estimate
// tau_hat), only the scores above f = hint - kHintMargin are written: each
// page's candidates are packed at the start of the page's own score range, in
// token order, and a 64-bit mask per page and head records which tokens they
// are.  Scores at or below f cannot be in the support as long as tau >= f,
// which the threshold step checks from the candidates themselves
// (sum (z - f)_+^r >= 1 over them implies tau >= f).  Without a hint (f =
// -inf) every valid token is a candidate and the layout is the plain one.
#include <float.h>

#include <type_traits>

#include "decode_common.h"

namespace ekv {

// Each wave takes a contiguous run of the flattened list of selected pages
// (units in order, so a run seldom crosses into another unit) and walks it in
// chunks of up to 64 pages.  A chunk's page references are loaded first, one
// page per lane (selection entry, sequence length, then page-table entry),
// and read back with readlane; its keys then stream in bodies of kKRing
// 16-token groups (one page of 64 tokens, two of 32 or four of 16).  As soon
// as a group has been used its registers are refilled with the same group of
// the next body, so one body of keys is always in flight.  Every load in the
// stream is unconditional (the refill after a chunk's last body repeats that
// body and is never used), so the compiler's counts of loads in flight stay
// exact and the wait for one group never waits for the groups behind it.
constexpr int kKRing = 4;

// Score floor of query head ug from the hint: hint - kHintMargin, or -inf
// without a hint (or for a NaN hint).  The threshold step reads the value
// stored by block 0 of the key pass, computed by this same function.
__device__ __forceinline__ float hint_floor(const float *tau_hint, int ug) {
  if (!tau_hint) return -INFINITY;
  const float t = tau_hint[ug];
  return t == t ? t - kHintMargin : -INFINITY;
}

// Block 0 records, for the threshold step, every head's score floor and its
// query scaled by (alpha-1) scale (used to recompute scores when a hint
// proves too high), and clears the count of heads left to the apply step.
template <int D>
__device__ __forceinline__ void record_heads(const float *q, const float *tau_hint,
                                             float zscale, int n_heads,
                                             float *floor_ws, float *qz,
                                             int32_t *undone) {
  if (blockIdx.x != 0) return;
  if (threadIdx.x == 0) *undone = 0;
  for (int i = threadIdx.x; i < n_heads; i += blockDim.x)
    floor_ws[i] = hint_floor(tau_hint, i);
  for (int i = threadIdx.x; i < n_heads * D; i += blockDim.x) qz[i] = q[i] * zscale;
}

template <int D, int G, int P, bool SEL>
__global__ __launch_bounds__(kDecThreads) void k_entmax_scores_mfma(
    const uint16_t *__restrict__ kpool, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, const float *__restrict__ q,
    const float *__restrict__ tau_hint, float zscale, int units, int H,
    int max_pages, int cap, float *__restrict__ zbuf, float *__restrict__ pmax,
    int32_t *__restrict__ slots, int32_t *__restrict__ undone,
    float *__restrict__ floor_ws, float *__restrict__ qz,
    unsigned long long *__restrict__ pmask) {
  constexpr int KS = D / 32;            // k-steps of 32 coordinates
  constexpr int NPASS = (G + 3) / 4;    // groups of 4 query heads
  constexpr int NT16 = P / 16;          // 16-token groups per page
  constexpr int U = kKRing / NT16;      // pages per body
  record_heads<D>(q, tau_hint, zscale, units * G, floor_ws, qz, undone);
  static_assert(kKRing % NT16 == 0, "a body holds whole pages");
  __shared__ int pref[kMaxUnits + 1];
  __shared__ int tmp[kDecWaves];
  const int total = build_unit_prefix<kDecThreads>(pref, tmp, seq_lens, sel,
                                                   count, units, H, P, 1);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, kb = lane >> 4;
  const int nwaves = gridDim.x * kDecWaves;
  const int wg = blockIdx.x * kDecWaves + wave;
  const int per = ((total + U - 1) / U + nwaves - 1) / nwaves;  // bodies
  const int f0 = wg * per * U;
  const int f1 = min(total, f0 + per * U);
  if (f0 >= f1) return;  // whole waves; no block barrier follows

  auto issue = [&](bf16x8_t (&bv)[KS], int slot, int h, int t) {
    const uint16_t *row = kpool + pool_row(slot, h, 16 * t + n, H, P, D) + 8 * kb;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      bv[s] = *reinterpret_cast<const bf16x8_t *>(row + 32 * s);
  };
  auto lane_val = [](int x, int i) { return __builtin_amdgcn_readlane(x, i); };

  bf16x8_t a[NPASS][KS];
  bf16x8_t ring[kKRing][KS];
  float flo[NPASS];                 // score floor of this lane's head 4 ps + kb
  int run[NPASS];                   // candidates so far in the page, per head
  unsigned long long pbits[NPASS];  // the page's candidate mask, per head
  int cur_u = -1;
  for (int c0 = f0; c0 < f1; c0 += kWave) {
    const int nc = min(kWave, f1 - c0);        // pages in this chunk
    const int nbc = (nc + U - 1) / U;          // bodies in this chunk
    // page references, one page per lane (lanes past the chunk repeat its last)
    const int f = c0 + min(lane, nc - 1);
    const int ru = find_unit(pref, units, f);
    const int rj = f - pref[ru];
    const int rb = ru / H;
    int rlp;
    if constexpr (SEL) rlp = sel[static_cast<size_t>(ru) * max_pages + rj];
    else rlp = rj;
    const int rnt = page_tokens(rlp, seq_lens[rb], P);
    const int rslot = page_table[static_cast<size_t>(rb) * max_pages + rlp];
    auto body_page = [&](int k, int t) { return min(k * U + t, nc - 1); };
#pragma unroll
    for (int s = 0; s < kKRing; ++s) {
      const int i = body_page(0, s / NT16);
      issue(ring[s], lane_val(rslot, i), lane_val(ru, i) % H, s % NT16);
    }
    for (int k = 0; k < nbc; ++k) {
      float pm[NPASS][4];
#pragma unroll
      for (int s = 0; s < kKRing; ++s) {
        const int t = s / NT16, tt = s % NT16;
        const int i = k * U + t;               // page of the chunk
        const bool live = i < nc;
        const int ic = min(i, nc - 1);
        const int u = lane_val(ru, ic);
        const int j = lane_val(rj, ic);
        const int h = u % H;
        if (tt == 0) {
          if (u != cur_u) {  // rare: the run enters another unit
            cur_u = u;
            load_q_parts<D, G>(a, q, u / H, h, H, zscale);
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
              const int g = 4 * ps + kb;
              flo[ps] = g < G ? hint_floor(tau_hint, u * G + g) : -INFINITY;
            }
          }
#pragma unroll
          for (int ps = 0; ps < NPASS; ++ps) {
            run[ps] = 0;
            pbits[ps] = 0ull;
#pragma unroll
            for (int e = 0; e < 4; ++e) pm[ps][e] = -FLT_MAX;
          }
        }
        const bool valid = 16 * tt + n < lane_val(rnt, ic);
        const __amdgpu_buffer_rsrc_t zr = store_rsrc(
            zbuf + static_cast<size_t>(u) * G * cap,
            static_cast<size_t>(G) * cap * sizeof(float));
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < KS; ++s2)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ps][s2], ring[s][s2], c,
                                                        0, 0, 0);
          // c[e] of lane n + 16 kb is q-part kb's share of head 4 ps + e on
          // token n (part 3 is zero).  A butterfly over the four lane groups
          // leaves every lane with the same sum (c0 + c1) + (c2 + c3), so
          // lane n + 16 e can write head 4 ps + e's score of token n: one
          // store with every lane active instead of one per head.
          float zmine = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float s1 = c[e] + __shfl_xor(c[e], 16, kWave);
            const float z = s1 + __shfl_xor(s1, 32, kWave);
            if (valid) pm[ps][e] = fmaxf(pm[ps][e], z);
            zmine = kb == e ? z : zmine;
          }
          // Candidates (z above the head's floor) go to the next free entry
          // of the page's range; without a hint every valid token is one, at
          // its own position, and the invalid tail keeps -inf as before.
          const int g = 4 * ps + kb;
          const bool cand = valid && zmine > flo[ps];
          const unsigned long long ball = __ballot(cand);
          const unsigned gb = static_cast<unsigned>(ball >> (16 * kb)) & 0xffffu;
          const int rank = run[ps] + __popc(gb & ((1u << n) - 1u));
          const bool keep = cand || (!valid && flo[ps] == -INFINITY);
          store_if(zr, 4 * (g * cap + j * P + (cand ? rank : 16 * tt + n)),
                   keep && g < G && live, valid ? zmine : -INFINITY);
          run[ps] += __popc(gb);
          pbits[ps] |= static_cast<unsigned long long>(gb) << (16 * tt);
        }
        if (tt == NT16 - 1) {
          // the page's maxima, lane g holding head g's
          float mine = 0.f;
#pragma unroll
          for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int g = 4 * ps + e;
              if (g < G) {
                const float m = group_max<16>(pm[ps][e]);
                const float m0 = __shfl(m, 0, kWave);
                mine = lane == g ? m0 : mine;
              }
            }
          const int ps_ = pm_stride(max_pages);
          const __amdgpu_buffer_rsrc_t pr = store_rsrc(
              pmax + static_cast<size_t>(u) * G * ps_,
              static_cast<size_t>(G) * ps_ * sizeof(float));
          store_if(pr, 4 * (lane * ps_ + j), lane < G && live, mine);
          // candidate masks: lane 16 e of pass ps writes head 4 ps + e's
          const __amdgpu_buffer_rsrc_t mr = store_rsrc(
              pmask + static_cast<size_t>(u) * G * ps_,
              static_cast<size_t>(G) * ps_ * sizeof(unsigned long long));
#pragma unroll
          for (int ps = 0; ps < NPASS; ++ps) {
            typedef unsigned v2u __attribute__((ext_vector_type(2)));
            const int g = 4 * ps + kb;
            const v2u w = {static_cast<unsigned>(pbits[ps]),
                           static_cast<unsigned>(pbits[ps] >> 32)};
            __builtin_amdgcn_raw_buffer_store_b64(
                w, mr, (n == 0 && g < G && live) ? 8 * (g * ps_ + j) : kDropOffset, 0, 0);
          }
          const __amdgpu_buffer_rsrc_t sr = store_rsrc(
              slots + static_cast<size_t>(u) * max_pages,
              static_cast<size_t>(max_pages) * sizeof(int32_t));
          store_if(sr, 4 * j, lane == 0 && live, lane_val(rslot, ic));
        }
        // refill: the same group of the next body
        const int inx = body_page(k + 1, t);
        issue(ring[s], lane_val(rslot, inx), lane_val(ru, inx) % H, tt);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 1b. Scores on the vector units (float32 keys).  One wave per page; D/8
// lanes per token, 8 coordinates per lane.
// ---------------------------------------------------------------------------
template <class E, int D, int G>
__global__ __launch_bounds__(kDecThreads) void k_entmax_scores_valu(
    const typename E::T *__restrict__ kpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, const float *__restrict__ q,
    float zscale, int units, int H, int P, int max_pages, int cap,
    float *__restrict__ zbuf, float *__restrict__ pmax,
    int32_t *__restrict__ slots, int32_t *__restrict__ undone,
    float *__restrict__ floor_ws, float *__restrict__ qz) {
  // float32 keys: every score is written (no hint is used)
  record_heads<D>(q, nullptr, zscale, units * G, floor_ws, qz, undone);
  constexpr int LPT = D / 8;
  constexpr int TPW = kWave / LPT;
  __shared__ int pref[kMaxUnits + 1];
  __shared__ int tmp[kDecWaves];
  const int total = build_unit_prefix<kDecThreads>(pref, tmp, seq_lens, sel,
                                                   count, units, H, P, 1);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int sub = lane / LPT, li = lane % LPT, d0 = li * 8;
  const int Hq = H * G;
  const int nwaves = gridDim.x * kDecWaves;
  for (int f = blockIdx.x * kDecWaves + wave; f < total; f += nwaves) {
    const PageRef r = page_ref(pref, units, f, page_table, seq_lens, sel, H, P,
                               max_pages);
    const int u = r.u, h = u % H, b = u / H;
    float qs[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        qs[g][j] = q[(static_cast<size_t>(b) * Hq + h * G + g) * D + d0 + j] * zscale;
    float mx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) mx[g] = -FLT_MAX;
    float *zu = zbuf + static_cast<size_t>(u) * G * cap +
                static_cast<size_t>(r.j) * P;
    for (int t0 = 0; t0 < P; t0 += TPW) {
      const int t = t0 + sub;
      float x[8];
      load8(kpool + pool_row(r.slot, h, t, H, P, D) + d0, x);
      const bool valid = t < r.nt;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaf(qs[g][j], x[j], a);
        a = group_sum<LPT>(a);
        if (li == g) zu[static_cast<size_t>(g) * cap + t] = valid ? a : -INFINITY;
        if (valid) mx[g] = fmaxf(mx[g], a);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m = group_max<kWave>(mx[g]);
      if (lane == 0) pmax[(static_cast<size_t>(u) * G + g) * pm_stride(max_pages) + r.j] = m;
    }
    if (lane == 0) slots[static_cast<size_t>(u) * max_pages + r.j] = r.slot;
  }
}

template <class E, int D, int G>
hipError_t launch_entmax_scores(const ekv_paged_kv &kv, const float *q,
                                float scale, float alpha, const int32_t *sel,
                                const int32_t *count, const float *tau_hint,
                                void *ws, hipStream_t stream) {
  const DecodeWs L = decode_ws_layout(kv);
  char *w = static_cast<char *>(ws);
  const int units = kv.batch * kv.num_kv_heads;
  const size_t pages = static_cast<size_t>(units) * kv.max_pages;
  const int blocks = persistent_blocks((pages + kDecWaves - 1) / kDecWaves, 4);
  const int cap = kv.max_pages * kv.page_size;
  float *z = reinterpret_cast<float *>(w + L.z);
  float *pm = reinterpret_cast<float *>(w + L.cmax);
  int32_t *sl = reinterpret_cast<int32_t *>(w + L.slot);
  int32_t *und = reinterpret_cast<int32_t *>(w + L.ctr) + units;
  float *fl = reinterpret_cast<float *>(w + L.floor);
  float *qz = reinterpret_cast<float *>(w + L.qz);
  auto *mk = reinterpret_cast<unsigned long long *>(w + L.mask);
  const float zs = (alpha - 1.0f) * scale;
  if constexpr (sizeof(typename E::T) == 2) {
    const uint16_t *k = static_cast<const uint16_t *>(kv.k);
    // resident waves walk contiguous runs of pages
    auto go = [&](auto kern) {
      const int nb = resident_blocks(kern, kDecThreads,
                                     (pages + kDecWaves - 1) / kDecWaves);
      hipLaunchKernelGGL(kern, dim3(nb), dim3(kDecThreads), 0, stream, k,
                         kv.page_table, kv.seq_lens, sel, count, q, tau_hint,
                         zs, units, kv.num_kv_heads, kv.max_pages, cap, z, pm,
                         sl, und, fl, qz, mk);
    };
    auto by_page = [&](auto has_sel) {
      constexpr bool S = decltype(has_sel)::value;
      switch (kv.page_size) {
        case 16: go(k_entmax_scores_mfma<D, G, 16, S>); break;
        case 32: go(k_entmax_scores_mfma<D, G, 32, S>); break;
        default: go(k_entmax_scores_mfma<D, G, 64, S>); break;
      }
    };
    if (sel) by_page(std::true_type());
    else by_page(std::false_type());
  } else {
    hipLaunchKernelGGL((k_entmax_scores_valu<E, D, G>), dim3(blocks),
                       dim3(kDecThreads), 0, stream,
                       static_cast<const typename E::T *>(kv.k), kv.page_table,
                       kv.seq_lens, sel, count, q, zs, units, kv.num_kv_heads,
                       kv.page_size, kv.max_pages, cap, z, pm, sl, und, fl,
                       qz);
  }
  return hipGetLastError();
}

#define EKV_INST_KPASS(E, D, G)                                              \
  template hipError_t launch_entmax_scores<E, D, G>(                         \
      const ekv_paged_kv &, const float *, float, float, const int32_t *,    \
      const int32_t *, const float *, void *, hipStream_t);
EKV_FOR_EACH_EDG(EKV_INST_KPASS)

}  // namespace ekv
