// Host-side launchers of the EntmaxKV kernels, one template instance per
// (element type, head_dim, group) combination the library is built for.
#pragma once

#include <hip/hip_runtime.h>

#include "entmaxkv.h"

namespace ekv {

struct F32;
struct BF16;

// Pages summarised together by the scoring kernel (one tile per block).
constexpr int kPageTile = 64;

// Float offset of the Gaussian tile summaries in gstat: after the per-page
// (mu, sigma^2) pairs, rounded up to 4 floats so the float4 rows are aligned.
__host__ __device__ inline size_t gstat_tile_offset(int batch, int Hq,
                                                    int max_pages) {
  const size_t n = static_cast<size_t>(batch) * Hq * max_pages * 2;
  return (n + 3) & ~static_cast<size_t>(3);
}

inline int page_tiles(const ekv_paged_kv &kv) {
  return (kv.max_pages + kPageTile - 1) / kPageTile;
}

// Tokens covered by one decode work item (a "chunk" of selected pages).
constexpr int kChunkTokens = 512;

inline int chunk_pages(int P) { return kChunkTokens / P; }
inline int max_chunks(const ekv_paged_kv &kv) {
  const int ppc = chunk_pages(kv.page_size);
  return (kv.max_pages + ppc - 1) / ppc;
}

// Decode workspace layout (offsets in bytes, each 256-byte aligned).
// Row stride of the per-page score maxima in the decode workspace: a
// multiple of 4 entries, so that rows can be read with 16-byte loads.
__host__ __device__ inline int pm_stride(int max_pages) {
  return (max_pages + 3) & ~3;
}

struct DecodeWs {
  size_t z, cmax, tau, part_o, part_s, ctr, done, slot, floor, qz, mask, total;
};

// Scores below (tau hint - kHintMargin) are not kept by a hinted key pass.
// The margin is in z units; the Gaussian selector's estimate lies within
// about 0.01 of the exact threshold on the clustered workloads, and a hint
// that proves too high is caught and repaired by the threshold step.
constexpr float kHintMargin = 0.03125f;
DecodeWs decode_ws_layout(const ekv_paged_kv &kv);
struct SoftmaxWs {
  size_t part_m, part_l, part_o, seg, total;
};
size_t softmax_stream_slots(const ekv_paged_kv &kv);
template <int D, int G>
hipError_t launch_softmax_stream(const ekv_paged_kv &kv, const float *q,
                                 float scale, const int32_t *sel,
                                 const int32_t *count, float *out, float *lse,
                                 float *part_m, float *part_l, float *part_o,
                                 int32_t *seg_range, hipStream_t stream);
SoftmaxWs softmax_ws_layout(const ekv_paged_kv &kv);

template <class E, int D>
hipError_t launch_build_meta(const ekv_paged_kv &kv, const int32_t *first_page,
                             int span, const ekv_meta &meta,
                             hipStream_t stream);
template <class E, int D, int G>
hipError_t launch_score(const ekv_paged_kv &kv, const ekv_meta &meta,
                        const float *q, float scale, int mode, float *ub,
                        float *gstat, bool refresh, hipStream_t stream);
template <int G>
hipError_t launch_select_topk(const ekv_paged_kv &kv, const float *ub, int k,
                              int32_t *sel, int32_t *count, void *ws,
                              hipStream_t stream);
template <int G>
hipError_t launch_select_gauss(const ekv_paged_kv &kv, const float *gstat,
                               float alpha, float delta, int32_t *sel,
                               int32_t *count, float *tau_hat, void *ws,
                               hipStream_t stream);
template <class E, int D, int G>
hipError_t launch_entmax_scores(const ekv_paged_kv &kv, const float *q,
                                float scale, float alpha, const int32_t *sel,
                                const int32_t *count, const float *tau_hint,
                                void *ws, hipStream_t stream);
// Tokens of one unit the single-launch small-selection decode holds on chip.
constexpr int kSmallTokens = 2048;

template <int D, int G>
hipError_t launch_entmax_small(const ekv_paged_kv &kv, const float *q,
                               float scale, float alpha, const int32_t *sel,
                               const int32_t *count, int max_count, float *out,
                               float *tau, void *ws, hipStream_t stream);
// Workspace of the small-selection decode: per-unit arrival counters, then
// the units' scores.
size_t small_ws_bytes(const ekv_paged_kv &kv, int max_count);
template <class E, int D, int G>
hipError_t launch_entmax_threshold(const ekv_paged_kv &kv, float alpha,
                                   const int32_t *sel, const int32_t *count,
                                   float *tau, float *out, void *ws,
                                   hipStream_t stream);
template <class E, int D, int G>
hipError_t launch_entmax_apply(const ekv_paged_kv &kv, float alpha,
                               const int32_t *sel, const int32_t *count,
                               float *out, float *probs, void *ws,
                               hipStream_t stream);
template <class E, int D, int G>
hipError_t launch_softmax(const ekv_paged_kv &kv, const float *q, float scale,
                          const int32_t *sel, const int32_t *count, float *out,
                          float *lse, void *ws, hipStream_t stream);

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                             hipStream_t stream);

#define EKV_FOR_EACH_G(X) X(1) X(2) X(4) X(8)
#define EKV_FOR_EACH_ED(X) X(F32, 64) X(F32, 128) X(BF16, 64) X(BF16, 128)
#define EKV_FOR_EACH_EDG(X)                                                \
  X(F32, 64, 1) X(F32, 64, 2) X(F32, 64, 4) X(F32, 64, 8)                  \
  X(F32, 128, 1) X(F32, 128, 2) X(F32, 128, 4) X(F32, 128, 8)              \
  X(BF16, 64, 1) X(BF16, 64, 2) X(BF16, 64, 4) X(BF16, 64, 8)              \
  X(BF16, 128, 1) X(BF16, 128, 2) X(BF16, 128, 4) X(BF16, 128, 8)

}  // namespace ekv
