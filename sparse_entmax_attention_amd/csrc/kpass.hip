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

// Records, for the threshold step, every head's score floor and its query
// scaled by (alpha-1) scale (used to recompute scores when a hint proves too
// high), and clears the count of heads left to the apply step.  The heads are
// spread over the grid, block b taking heads b, b + gridDim.x, ...: one
// 16-byte load and store per lane and head.  (Block 0 alone, one float per
// thread and round, made a chain of dependent round trips, 64 of them at
// 128 heads, that held its own keys back by some 30 us.)  q and qz are
// 16-byte aligned (checked at the entry points; qz sits in the workspace).
template <int D>
__device__ __forceinline__ void record_heads(const float *q, const float *tau_hint,
                                             float zscale, int n_heads,
                                             float *floor_ws, float *qz,
                                             int32_t *undone) {
  constexpr int V = D / 4;  // float4s per head
  static_assert(V < kDecThreads, "one lane per float4 of a head, one for the floor");
  if (blockIdx.x == 0 && threadIdx.x == 0) *undone = 0;
  for (int hd = blockIdx.x; hd < n_heads; hd += gridDim.x) {
    if (threadIdx.x < V) {
      float4 x = reinterpret_cast<const float4 *>(q)[static_cast<size_t>(hd) * V + threadIdx.x];
      x.x *= zscale;
      x.y *= zscale;
      x.z *= zscale;
      x.w *= zscale;
      reinterpret_cast<float4 *>(qz)[static_cast<size_t>(hd) * V + threadIdx.x] = x;
    } else if (threadIdx.x == V) {
      floor_ws[hd] = hint_floor(tau_hint, hd);
    }
  }
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
  // Per wave: the current page's kept scores (G rows of P), and the page
  // maxima and candidate masks of the chunk's pages (G rows of 64).  The
  // scores leave in one 16-byte store per lane per page and the page
  // records once per chunk: stores cost the key stream more by their
  // number than by their bytes.
  constexpr int ZS = G * P < 256 ? 256 : G * P;
  __shared__ __align__(16) float s_z[kDecWaves][ZS];
  __shared__ float s_pm[kDecWaves][G][kWave];
  __shared__ unsigned long long s_mk[kDecWaves][G][kWave];
  __shared__ float4 s_qs[kDecWaves][G * D / 4];  // the unit's queries, staged
  const int total = build_unit_prefix<kDecThreads>(pref, tmp, seq_lens, sel,
                                                   count, units, H, P, 1);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, kb = lane >> 4;
  const int nwaves = gridDim.x * kDecWaves;
  float *zst = s_z[wave];
  const int wg = blockIdx.x * kDecWaves + wave;
  const int per = ((total + U - 1) / U + nwaves - 1) / nwaves;  // bodies
  const int pw = per * U;                                        // pages per wave
  int f0 = wg * pw;
  int f1 = min(total, f0 + pw);
  // A wave whose run crosses into another unit pays the whole start again
  // (selection entries, page table, query rows) in the middle of the stream,
  // and those waves ended last.  When the grid has waves enough, each unit
  // gets its own ceil(pages / pw) waves instead, none crossing a unit
  // boundary, no wave taking more than pw pages.  The waves-per-unit prefix
  // lives in the query staging area, before any wave stages its queries
  // (the same for the whole block, barriers included; skipped when there is
  // nothing to do, pw = 0).
  if (units < kDecWaves * G * D && pw > 0) {
    int *wpref = reinterpret_cast<int *>(&s_qs[0][0]);
    const int pt = (units + kDecThreads - 1) / kDecThreads;
    const int u0 = min(units, static_cast<int>(threadIdx.x) * pt), u1 = min(units, u0 + pt);
    auto waves_of = [&](int u) { return (pref[u + 1] - pref[u] + pw - 1) / pw; };
    int local = 0;
    for (int u = u0; u < u1; ++u) local += waves_of(u);
    int need;
    int base = block_excl_scan<kDecThreads>(local, tmp, need);
    for (int u = u0; u < u1; ++u) {
      wpref[u] = base;
      base += waves_of(u);
    }
    lds_barrier();
    if (need <= nwaves) {
      if (wg < need) {
        const int u = find_unit(wpref, units, wg);
        f0 = pref[u] + (wg - wpref[u]) * pw;
        f1 = min(pref[u + 1], f0 + pw);
      } else {
        f0 = f1 = total;
      }
    }
    lds_barrier();  // every wave has read wpref
  }
  if (f0 >= f1) return;  // whole waves; no block barrier follows

  // Keys of 16-token group t of page (slot, h) through a buffer resource on
  // the page: the page's address stays in scalar registers and every load
  // of the stream shares one per-lane offset register.
  const int key_off = 2 * (n * D + 8 * kb);
  auto issue = [&](bf16x8_t (&bv)[KS], int slot, int h, int t) {
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(kpool + pool_row(slot, h, 0, H, P, D)),
        static_cast<short>(0), 2 * P * D, 0x00020000);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      bv[s] = __builtin_bit_cast(
          bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(pr, key_off + 64 * s,
                                                          32 * D * t, 0));
  };
  auto lane_val = [](int x, int i) { return __builtin_amdgcn_readlane(x, i); };

  bf16x8_t a[NPASS][KS];
  bf16x8_t ring[kKRing][KS];
  float flo[NPASS];                 // score floor of this lane's head 4 ps + kb
  int run[NPASS];                   // candidates so far in the page, per head
  unsigned long long pbits[NPASS];  // the page's candidate mask, per head
  for (int c0 = f0; c0 < f1;) {
    // A chunk is up to 64 pages of one unit, so the unit's query parts and
    // score floors are loaded here, while no keys are in flight: loading
    // them inside the stream would hold their float32 sources in registers
    // beside the ring, and the extra registers cost a wave per SIMD.  The
    // page references go first (the selection entries, then the page-table
    // rows they name, are the chain to the first keys); the query rows and
    // floors travel beside them and are turned into the matrix operand
    // while the page-table rows are on their way.
    const int u = __builtin_amdgcn_readfirstlane(find_unit(pref, units, c0));
    const int c1 = min(min(c0 + kWave, f1), pref[u + 1]);
    const int nc = c1 - c0;                    // pages in this chunk
    const int nbc = (nc + U - 1) / U;          // bodies in this chunk
    const int h = u % H, b = u / H;
    // page references, one page per lane (lanes past the chunk repeat its last)
    const int rj = c0 + min(lane, nc - 1) - pref[u];
    int rlp;
    if constexpr (SEL) rlp = sel[static_cast<size_t>(u) * max_pages + rj];
    else rlp = rj;
    QRows<D, G> qrow;
    load_q_rows<D, G>(qrow, q, b, h, H);
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int g = 4 * ps + kb;
      flo[ps] = g < G ? hint_floor(tau_hint, u * G + g) : -INFINITY;
    }
    __builtin_amdgcn_sched_barrier(0);
    const int rnt = page_tokens(rlp, seq_lens[b], P);
    const int rslot = page_table[static_cast<size_t>(b) * max_pages + rlp];
    __builtin_amdgcn_sched_barrier(0);
    q_parts_from_rows<D, G>(a, qrow, zscale, s_qs[wave]);
    auto body_page = [&](int k, int t) { return min(k * U + t, nc - 1); };
#pragma unroll
    for (int s = 0; s < kKRing; ++s) {
      __builtin_amdgcn_sched_barrier(0);  // issued in the order they are used
      issue(ring[s], lane_val(rslot, body_page(0, s / NT16)), h, s % NT16);
    }
    for (int k = 0; k < nbc; ++k) {
      float pm[NPASS];  // the page's maximum so far of this lane's head 4 ps + kb
#pragma unroll
      for (int s = 0; s < kKRing; ++s) {
        // Groups stay in program order: the compiler's scheduler would
        // otherwise gather the refills at the end of the body, and the wait
        // for the first group would then cover the whole body, leaving no
        // keys in flight while the body is scored.
        __builtin_amdgcn_sched_barrier(0);
        const int t = s / NT16, tt = s % NT16;
        const int i = k * U + t;               // page of the chunk
        const bool live = i < nc;
        const int ic = min(i, nc - 1);
        const int j = lane_val(rj, ic);
        if (tt == 0) {
#pragma unroll
          for (int ps = 0; ps < NPASS; ++ps) {
            run[ps] = 0;
            pbits[ps] = 0ull;
            pm[ps] = -FLT_MAX;
          }
        }
        const bool valid = 16 * tt + n < lane_val(rnt, ic);
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
            zmine = kb == e ? z : zmine;
          }
          // Candidates (z above the head's floor) go to the next free entry
          // of the page's range; without a hint every valid token is one, at
          // its own position, and the invalid tail keeps -inf as before.
          const int g = 4 * ps + kb;
          if (valid) pm[ps] = fmaxf(pm[ps], zmine);
          const bool cand = valid && zmine > flo[ps];
          const unsigned long long ball = __ballot(cand);
          const unsigned gb = static_cast<unsigned>(ball >> (16 * kb)) & 0xffffu;
          const int rank = run[ps] + __popc(gb & ((1u << n) - 1u));
          const bool keep = cand || (!valid && flo[ps] == -INFINITY);
          if (keep && g < G) zst[g * P + (cand ? rank : 16 * tt + n)] = valid ? zmine : -INFINITY;
          run[ps] += __popc(gb);
          pbits[ps] |= static_cast<unsigned long long>(gb) << (16 * tt);
        }
        if (tt == NT16 - 1) {
          // the page's maxima and candidate masks, kept for the chunk's end
#pragma unroll
          for (int ps = 0; ps < NPASS; ++ps) {
            const float m = group_max<16>(pm[ps]);  // head 4 ps + kb's, in every lane of the group
            if (n == 0 && 4 * ps + kb < G) s_pm[wave][4 * ps + kb][i] = m;
          }
#pragma unroll
          for (int ps = 0; ps < NPASS; ++ps) {
            const int g = 4 * ps + kb;
            if (n == 0 && g < G) s_mk[wave][g][i] = pbits[ps];
          }
          // The page's kept scores: lane l writes floats 4 l .. 4 l + 3 of
          // the G rows of P (of row 4 l / P), those of a row up to its count
          // of kept scores rounded up to 4 (the rest of the page's range is
          // never read) or, without a hint, the whole row.
          int lim[NPASS];
#pragma unroll
          for (int ps = 0; ps < NPASS; ++ps) lim[ps] = flo[ps] == -INFINITY ? P : run[ps];
          const __amdgpu_buffer_rsrc_t zr = store_rsrc(
              zbuf + static_cast<size_t>(u) * G * cap,
              static_cast<size_t>(G) * cap * sizeof(float));
#pragma unroll
          for (int k2 = 0; k2 < (G * P + 255) / 256; ++k2) {
            const int f = 256 * k2 + 4 * lane;
            const int g2 = f / P, pos = f - g2 * P;
            int lg;
            if constexpr (P == 64) {
              lg = lim[k2 < NPASS ? k2 : 0];  // row 4 k2 + kb: this lane's own
            } else {
              // both shuffles on every lane (a lane that reads from an
              // inactive one gets 0), then the pass of this lane's row
              const int src = 16 * (g2 & 3);
              const int l0 = __shfl(lim[0], src, kWave);
              const int l1 = __shfl(lim[NPASS - 1], src, kWave);
              lg = g2 >= 4 ? l1 : l0;
            }
            // read as floats, the type the rows were written with, so that
            // the read stays ordered after those writes
            const float *zf = zst + min(f, ZS - 4);
            const f32x4_t v = {zf[0], zf[1], zf[2], zf[3]};
            __builtin_amdgcn_raw_buffer_store_b128(
                v, zr,
                (live && g2 < G && pos < lg) ? 4 * (g2 * cap + j * P + pos) : kDropOffset,
                0, 0);
          }
        }
        // refill: the same group of the next body
        issue(ring[s], lane_val(rslot, body_page(k + 1, t)), h, tt);
      }
    }
    // the chunk's page records: lane l holds page l of the chunk
    {
      const int j0 = c0 - pref[u];
      const bool on = lane < nc;
      const int ps_ = pm_stride(max_pages);
      const __amdgpu_buffer_rsrc_t sr = store_rsrc(
          slots + static_cast<size_t>(u) * max_pages,
          static_cast<size_t>(max_pages) * sizeof(int32_t));
      store_if(sr, 4 * (j0 + lane), on, rslot);
      const __amdgpu_buffer_rsrc_t pr = store_rsrc(
          pmax + static_cast<size_t>(u) * G * ps_,
          static_cast<size_t>(G) * ps_ * sizeof(float));
      const __amdgpu_buffer_rsrc_t mr = store_rsrc(
          pmask + static_cast<size_t>(u) * G * ps_,
          static_cast<size_t>(G) * ps_ * sizeof(unsigned long long));
#pragma unroll
      for (int g = 0; g < G; ++g) {
        store_if(pr, 4 * (g * ps_ + j0 + lane), on, s_pm[wave][g][lane]);
        typedef unsigned v2u __attribute__((ext_vector_type(2)));
        const unsigned long long mk = s_mk[wave][g][lane];
        const v2u w = {static_cast<unsigned>(mk), static_cast<unsigned>(mk >> 32)};
        __builtin_amdgcn_raw_buffer_store_b64(
            w, mr, on ? 8 * (g * ps_ + j0 + lane) : kDropOffset, 0, 0);
      }
    }
    c0 = c1;
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
