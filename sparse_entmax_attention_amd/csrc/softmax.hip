// Split-K softmax attention over bfloat16 K/V: the full-cache baseline the
// Technical Summary (EntmaxKV, §4) compares against, and softmax over a
// selection of pages (§2.B.1's budget, for the matched-budget comparison).
//
// Streaming pass.  The selected pages of all units form one flattened list
// (units in order); each wave takes a contiguous run of it, like the key
// pass of kpass.hip, in chunks of up to 64 pages of one unit (page
// references one per lane, the unit's query parts loaded at the chunk's
// start).  Keys and values of 16-token groups stream through a ring of
// kSmRing groups, refilled in the order they are used.  Per group: scores
// on the matrix cores (q in three bfloat16 parts, float32 accuracy), then an
// online softmax per head (running maximum m, sum of exponentials l, and the
// weighted value sum, rescaled when m grows).  A wave's run crosses a unit
// boundary at most a few times: each (wave w, unit u) piece of it, a
// segment, ends with its (m, l, o) written to slot w + u (slots increase
// along the list, so a unit's segments have consecutive slots), and the
// pieces holding a unit's first and last page record the unit's slot range.
//
// Combine.  Per (unit, query head) and slice of head_dim: the unit's
// segments merged in log-sum-exp form, o / l and lse = m + log l.
#include <float.h>

#include "decode_common.h"

namespace ekv {

constexpr int kSmRing = 2;         // 16-token groups of keys and values in flight
constexpr int kSmMaxWaves = 8192;  // waves of the streaming pass, at most

size_t softmax_stream_slots(const ekv_paged_kv &kv) {
  return static_cast<size_t>(kSmMaxWaves) +
         static_cast<size_t>(kv.batch) * kv.num_kv_heads;
}

template <int D, int G, int P>
__global__ __launch_bounds__(kDecThreads) void k_softmax_stream(
    const uint16_t *__restrict__ kpool, const uint16_t *__restrict__ vpool,
    const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, const float *__restrict__ q,
    float scale, int units, int H, int max_pages,
    float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_o, int32_t *__restrict__ seg_range) {
  constexpr int KS = D / 32;          // k-steps of the MFMA
  constexpr int NPASS = (G + 3) / 4;  // groups of 4 query heads
  constexpr int NT16 = P / 16;        // 16-token groups per page
  constexpr int LPR = D / 8;          // lanes per value row (8 coordinates each)
  constexpr int RPI = kWave / LPR;    // value rows per load instruction
  constexpr int NVI = 16 / RPI;       // value loads per 16-token group
  constexpr int R = kSmRing;
  __shared__ int pref[kMaxUnits + 1];
  __shared__ int tmp[kDecWaves];
  __shared__ float s_p[kDecWaves][16][G];  // a group's weights, token-major
  const int total = build_unit_prefix<kDecThreads>(pref, tmp, seq_lens, sel,
                                                   count, units, H, P, 1);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, kb = lane >> 4;
  const int sub = lane / LPR, li = lane % LPR;
  const int nwaves = gridDim.x * kDecWaves;
  const int wg = blockIdx.x * kDecWaves + wave;
  const int per = (total + nwaves - 1) / nwaves;
  const int f0 = wg * per;
  const int f1 = min(total, f0 + per);
  if (f0 >= f1) return;  // whole waves; no block barrier follows
  float(*sp)[G] = s_p[wave];

  // keys of group t of page (slot, h): lane n + 16 kb takes coordinates
  // 32 s + 8 kb .. + 7 of token 16 t + n (the MFMA's B layout); values:
  // lane takes coordinates 8 li .. + 7 of token 16 t + RPI k + sub
  const int key_off = 2 * (n * D + 8 * kb);
  const int val_off = 2 * (sub * D + 8 * li);
  struct Group {
    bf16x8_t k[KS];
    uint4 v[NVI];
  };
  auto issue = [&](Group &gr, int slot, int h, int t) {
    const size_t page = pool_row(slot, h, 0, H, P, D);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(kpool + page), static_cast<short>(0), 2 * P * D, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(vpool + page), static_cast<short>(0), 2 * P * D, 0x00020000);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      gr.k[s] = __builtin_bit_cast(
          bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(kr, key_off + 64 * s, 32 * D * t, 0));
#pragma unroll
    for (int k = 0; k < NVI; ++k)
      gr.v[k] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, val_off + 2 * RPI * D * k,
                                                       32 * D * t, 0));
  };
  auto lane_val = [](int x, int i) { return __builtin_amdgcn_readlane(x, i); };
  auto lane_valf = [](float x, int i) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i));
  };

  bf16x8_t a[NPASS][KS];
  Group ring[R];
  float m[NPASS], l[NPASS];  // head 4 ps + kb's, uniform in each lane group
  float acc[G][8];           // weighted value sums, coordinates 8 li .. + 7
  auto reset = [&]() {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      m[ps] = -INFINITY;
      l[ps] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  };
  reset();

  for (int c0 = f0; c0 < f1;) {
    const int u = __builtin_amdgcn_readfirstlane(find_unit(pref, units, c0));
    const int c1 = min(min(c0 + kWave, f1), pref[u + 1]);
    const int nc = c1 - c0;  // pages in this chunk
    const int ng = nc * NT16;
    const int h = u % H, b = u / H;
    load_q_parts<D, G>(a, q, b, h, H, scale);
    const int rj = c0 + min(lane, nc - 1) - pref[u];
    const int rlp = sel ? sel[static_cast<size_t>(u) * max_pages + rj] : rj;
    const int rnt = page_tokens(rlp, seq_lens[b], P);
    const int rslot = page_table[static_cast<size_t>(b) * max_pages + rlp];
    auto group_page = [&](int gq) { return min(gq / NT16, nc - 1); };
#pragma unroll
    for (int r = 0; r < R; ++r) {
      __builtin_amdgcn_sched_barrier(0);  // issued in the order they are used
      const int gq = min(r, ng - 1);
      issue(ring[r], lane_val(rslot, group_page(gq)), h, gq % NT16);
    }
    for (int q0 = 0; q0 < ng; q0 += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // groups in program order: each is waited for alone
        __builtin_amdgcn_sched_barrier(0);
        const int gq = q0 + r;
        if (gq < ng) {  // uniform
          const int i = gq / NT16, t = gq - i * NT16;
          const int nt = lane_val(rnt, i);
          const bool valid = 16 * t + n < nt;
          float sc[NPASS];
#pragma unroll
          for (int ps = 0; ps < NPASS; ++ps) {
            f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2)
              c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ps][s2], ring[r].k[s2], c, 0, 0, 0);
            // lane n + 16 e takes head 4 ps + e's score of token n (the sum
            // of the three q parts, as in the key pass)
            float zmine = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float s1 = c[e] + __shfl_xor(c[e], 16, kWave);
              const float z = s1 + __shfl_xor(s1, 32, kWave);
              zmine = kb == e ? z : zmine;
            }
            const float z = valid ? zmine : -INFINITY;
            const float mn = fmaxf(m[ps], group_max<16>(z));
            // no valid token yet: nothing to rescale and nothing to add
            sc[ps] = mn == -INFINITY ? 1.f : expf(m[ps] - mn);
            const float p = valid ? expf(z - mn) : 0.f;
            l[ps] = fmaf(l[ps], sc[ps], group_sum<16>(p));
            m[ps] = mn;
            if (4 * ps + kb < G) sp[n][4 * ps + kb] = p;
          }
          // rescale the sums of every head whose maximum grew, then add the
          // group's value rows (rows past the sequence add nothing: their
          // values are replaced by zeros, whatever the pool holds there)
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float s = lane_valf(sc[g / 4], 16 * (g % 4));
            if (s != 1.f) {
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[g][e] *= s;
            }
          }
          const bool full = 16 * t + 16 <= nt;  // uniform
#pragma unroll
          for (int k = 0; k < NVI; ++k) {
            const int tok = RPI * k + sub;
            float x[8] = {bf16_lo(ring[r].v[k].x), bf16_hi(ring[r].v[k].x),
                          bf16_lo(ring[r].v[k].y), bf16_hi(ring[r].v[k].y),
                          bf16_lo(ring[r].v[k].z), bf16_hi(ring[r].v[k].z),
                          bf16_lo(ring[r].v[k].w), bf16_hi(ring[r].v[k].w)};
            if (!full && 16 * t + tok >= nt) {
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] = 0.f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const float pw = sp[tok][g];
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pw, x[e], acc[g][e]);
            }
          }
        }
        // refill: the group R further on (past the chunk: its last group
        // again, never used)
        const int gn = min(gq + R, ng - 1);
        issue(ring[r], lane_val(rslot, group_page(gn)), h, gn % NT16);
      }
    }
    const bool seg_end = c1 == f1 || c1 == pref[u + 1];
    if (seg_end) {
      // the segment's sums over its lane subgroups (lanes with equal li),
      // then slot wg + u
      const int slot = wg + u;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = acc[g][e];
#pragma unroll
          for (int o = LPR; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
          acc[g][e] = v;
        }
      if (sub == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float4 *dst = reinterpret_cast<float4 *>(
              part_o + (static_cast<size_t>(slot) * G + g) * D + 8 * li);
          dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
          dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mg = lane_valf(m[g / 4], 16 * (g % 4));
        const float lg = lane_valf(l[g / 4], 16 * (g % 4));
        if (lane == g) {
          part_m[static_cast<size_t>(slot) * G + g] = mg;
          part_l[static_cast<size_t>(slot) * G + g] = lg;
        }
      }
      const int seg_start = max(f0, pref[u]);
      if (lane == 0 && seg_start == pref[u]) seg_range[2 * u] = slot;
      if (lane == 0 && c1 == pref[u + 1]) seg_range[2 * u + 1] = slot;
      reset();
    }
    c0 = c1;
  }
}

// One block per (unit, query head) and kSmCombD coordinates: the unit's
// segments merged in log-sum-exp form, kSmCombSlices threads per coordinate
// taking every kSmCombSlices-th segment (a full cache has hundreds of
// segments per unit).
constexpr int kSmCombD = 16;
constexpr int kSmCombSlices = 64;

__global__ __launch_bounds__(kSmCombD * kSmCombSlices) void k_softmax_stream_combine(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel,
    const int32_t *__restrict__ count, int H, int G, int D, int P,
    const float *__restrict__ part_m, const float *__restrict__ part_l,
    const float *__restrict__ part_o, const int32_t *__restrict__ seg_range,
    float *__restrict__ out, float *__restrict__ lse) {
  constexpr int NT = kSmCombD * kSmCombSlices;
  __shared__ float red_f[NT / kWave];
  __shared__ float s_o[kSmCombSlices][kSmCombD];
  __shared__ float s_l[kSmCombSlices];
  const int ug = blockIdx.x, u = ug / G, g = ug % G;
  const int tid = threadIdx.x;
  // a unit with no pages has no segments (its range is left from before)
  const int cnt = unit_pages(seq_lens, sel, count, u, H, P);
  const int s0 = cnt > 0 ? seg_range[2 * u] : 0;
  const int ns = cnt > 0 ? seg_range[2 * u + 1] - s0 + 1 : 0;
  float mloc = -FLT_MAX;
  for (int c = tid; c < ns; c += NT)
    mloc = fmaxf(mloc, part_m[static_cast<size_t>(s0 + c) * G + g]);
  const float M = block_max<NT>(mloc, red_f);
  const int dl = tid % kSmCombD, sl = tid / kSmCombD;
  const int d = blockIdx.y * kSmCombD + dl;
  float o = 0.f, lsum = 0.f;
  for (int c = sl; c < ns; c += kSmCombSlices) {
    const size_t base = static_cast<size_t>(s0 + c) * G + g;
    const float mc = part_m[base];
    const float wgt = mc == -INFINITY ? 0.f : expf(mc - M);
    o = fmaf(wgt, part_o[base * D + d], o);
    lsum = fmaf(wgt, part_l[base], lsum);
  }
  s_o[sl][dl] = o;
  if (dl == 0) s_l[sl] = lsum;
  lds_barrier();
  if (tid < kSmCombD) {
    float oo = 0.f, ll = 0.f;
    for (int k = 0; k < kSmCombSlices; ++k) {
      oo += s_o[k][tid];
      ll += s_l[k];
    }
    out[static_cast<size_t>(ug) * D + blockIdx.y * kSmCombD + tid] = oo / ll;
    if (lse && blockIdx.y == 0 && tid == 0) lse[ug] = M + logf(ll);
  }
}

template <int D, int G>
hipError_t launch_softmax_stream(const ekv_paged_kv &kv, const float *q,
                                 float scale, const int32_t *sel,
                                 const int32_t *count, float *out, float *lse,
                                 float *part_m, float *part_l, float *part_o,
                                 int32_t *seg_range, hipStream_t stream) {
  const int units = kv.batch * kv.num_kv_heads;
  const size_t pages = static_cast<size_t>(units) * kv.max_pages;
  auto go = [&](auto kern) {
    int nb = resident_blocks(kern, kDecThreads, (pages + kDecWaves - 1) / kDecWaves);
    nb = std::min(nb, kSmMaxWaves / kDecWaves);
    hipLaunchKernelGGL(kern, dim3(nb), dim3(kDecThreads), 0, stream,
                       static_cast<const uint16_t *>(kv.k),
                       static_cast<const uint16_t *>(kv.v), kv.page_table,
                       kv.seq_lens, sel, count, q, scale, units,
                       kv.num_kv_heads, kv.max_pages, part_m, part_l, part_o,
                       seg_range);
  };
  switch (kv.page_size) {
    case 16: go(k_softmax_stream<D, G, 16>); break;
    case 32: go(k_softmax_stream<D, G, 32>); break;
    default: go(k_softmax_stream<D, G, 64>); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_softmax_stream_combine, dim3(units * G, D / kSmCombD),
                     dim3(kSmCombD * kSmCombSlices), 0, stream, kv.seq_lens,
                     sel, count, kv.num_kv_heads, G, D, kv.page_size, part_m,
                     part_l, part_o, seg_range, out, lse);
  return hipGetLastError();
}

#define EKV_INST_SM(D, G)                                                     \
  template hipError_t launch_softmax_stream<D, G>(                            \
      const ekv_paged_kv &, const float *, float, const int32_t *,            \
      const int32_t *, float *, float *, float *, float *, float *, int32_t *, \
      hipStream_t);
EKV_INST_SM(64, 1) EKV_INST_SM(64, 2) EKV_INST_SM(64, 4) EKV_INST_SM(64, 8)
EKV_INST_SM(128, 1) EKV_INST_SM(128, 2) EKV_INST_SM(128, 4) EKV_INST_SM(128, 8)

}  // namespace ekv
