// C ABI of the EntmaxKV paged decode library: host-side validation,
// workspace sizing and dispatch to the kernel instances.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "ekv_device.h"
#include "ekv_kernels.h"
#include "gauss_rule.h"

namespace {

thread_local std::string g_last_error;

ekv_status fail(ekv_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ekv_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return EKV_OK;
  return fail(EKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Checks of the paged cache common to every entry point.
ekv_status check_kv(const ekv_paged_kv *kv, bool need_k, bool need_v) {
  if (!kv) return fail(EKV_ERR_INVALID_ARG, "kv is NULL");
  if (kv->batch < 1 || kv->num_kv_heads < 1 || kv->group < 1 ||
      kv->head_dim < 1 || kv->page_size < 1 || kv->num_slots < 1 ||
      kv->max_pages < 1)
    return fail(EKV_ERR_INVALID_ARG,
                "sizes must be >= 1 (batch %d, heads %d, group %d, D %d, P %d, "
                "slots %d, max_pages %d)",
                kv->batch, kv->num_kv_heads, kv->group, kv->head_dim,
                kv->page_size, kv->num_slots, kv->max_pages);
  if (kv->kv_dtype != EKV_F32 && kv->kv_dtype != EKV_BF16)
    return fail(EKV_ERR_INVALID_ARG, "kv_dtype %d is not an ekv_dtype",
                kv->kv_dtype);
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(EKV_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)",
                kv->head_dim);
  if (kv->page_size != 16 && kv->page_size != 32 && kv->page_size != 64)
    return fail(EKV_ERR_UNSUPPORTED, "page_size %d (built: 16, 32, 64)",
                kv->page_size);
  if (kv->group != 1 && kv->group != 2 && kv->group != 4 && kv->group != 8)
    return fail(EKV_ERR_UNSUPPORTED, "group %d (built: 1, 2, 4, 8)",
                kv->group);
  if (static_cast<long long>(kv->batch) * kv->num_kv_heads > 4096)
    return fail(EKV_ERR_UNSUPPORTED, "batch * num_kv_heads exceeds 4096");
  // one unit's float32 scores must be addressable by a 32-bit byte offset
  // of a buffer store (kernels write them through range-checked stores)
  const double unit_bytes =
      static_cast<double>(kv->max_pages) * kv->page_size * kv->group * 4.0;
  if (unit_bytes > 2147418112.0)
    return fail(EKV_ERR_UNSUPPORTED,
                "group * max_pages * page_size * 4 bytes exceeds 2 GiB - 64 KiB");
  if (!kv->page_table || !kv->seq_lens)
    return fail(EKV_ERR_INVALID_ARG, "page_table and seq_lens are required");
  if (need_k && (!kv->k || !aligned(kv->k, 16)))
    return fail(EKV_ERR_INVALID_ARG, "k must be non-NULL and 16-byte aligned");
  if (need_v && (!kv->v || !aligned(kv->v, 16)))
    return fail(EKV_ERR_INVALID_ARG, "v must be non-NULL and 16-byte aligned");
  return EKV_OK;
}

ekv_status check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return EKV_OK;
  if (!ws) return fail(EKV_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  if (ws_bytes < need)
    return fail(EKV_ERR_WORKSPACE, "workspace has %zu bytes, %zu required",
                ws_bytes, need);
  if (!aligned(ws, 256))
    return fail(EKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return EKV_OK;
}

ekv_status check_alpha(float alpha) {
  if (!std::isfinite(alpha) || !(alpha > 1.0f))
    return fail(EKV_ERR_INVALID_ARG, "alpha must be finite and > 1 (got %g)",
                static_cast<double>(alpha));
  return EKV_OK;
}

ekv_status check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(EKV_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)",
                static_cast<double>(scale));
  return EKV_OK;
}

ekv_status check_sel(const int32_t *sel, const int32_t *count) {
  if (sel && !count)
    return fail(EKV_ERR_INVALID_ARG, "count is required with sel");
  return EKV_OK;
}

template <int V>
using IC = std::integral_constant<int, V>;

// Calls f(E{}, IC<D>{}, IC<G>{}) for the runtime (dtype, D, G).
template <class F>
hipError_t with_edg(const ekv_paged_kv &kv, F &&f) {
  auto on_g = [&](auto e, auto d) -> hipError_t {
    switch (kv.group) {
      case 1: return f(e, d, IC<1>{});
      case 2: return f(e, d, IC<2>{});
      case 4: return f(e, d, IC<4>{});
      default: return f(e, d, IC<8>{});
    }
  };
  auto on_d = [&](auto e) -> hipError_t {
    if (kv.head_dim == 64) return on_g(e, IC<64>{});
    return on_g(e, IC<128>{});
  };
  if (kv.kv_dtype == EKV_F32) return on_d(ekv::F32{});
  return on_d(ekv::BF16{});
}

template <class F>
hipError_t with_g(const ekv_paged_kv &kv, F &&f) {
  switch (kv.group) {
    case 1: return f(IC<1>{});
    case 2: return f(IC<2>{});
    case 4: return f(IC<4>{});
    default: return f(IC<8>{});
  }
}

#define EKV_TRY(x)                        \
  do {                                    \
    const ekv_status s_ = (x);            \
    if (s_ != EKV_OK) return s_;          \
  } while (0)

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

// Workspace of ekv_entmax_decode_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` is only
// a host-side stand-in for the symbol; its device address on a GPU comes
// from hipGetSymbolAddress with that GPU current, taken once per device and
// kept in g_scratch.
constexpr size_t kScratchBytes = static_cast<size_t>(EKV_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

// Device address of `scratch` on the GPU that runs `stream`.
ekv_status scratch_on(hipStream_t stream, void **ptr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "finding the stream's device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(EKV_ERR_UNSUPPORTED, "device %d: the scratch is kept for devices 0..%d",
                dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess)
      return hip_status(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return hip_status(e, "hipSetDevice");
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(EKV_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return EKV_OK;
}

}  // namespace

extern "C" {

size_t ekv_workspace_size(int32_t op, const ekv_paged_kv *kv, int32_t k_or_0) {
  if (check_kv(kv, false, false) != EKV_OK) return 0;
  const size_t units = static_cast<size_t>(kv->batch) * kv->num_kv_heads;
  switch (op) {
    case EKV_OP_SELECT_TOPK:  // candidate keys, whole tiles of pages
      return ((units * ekv::page_tiles(*kv) * ekv::kPageTile * 4) + 255) &
             ~static_cast<size_t>(255);
    case EKV_OP_SELECT_GAUSS:  // per (unit, query head) 64-bit page masks per tile
      return ((units * kv->group * ekv::page_tiles(*kv) * 8) + 255) &
             ~static_cast<size_t>(255);
    case EKV_OP_ENTMAX_DECODE:
      return ekv::decode_ws_layout(*kv).total;
    case EKV_OP_SOFTMAX_DECODE:
      return ekv::softmax_ws_layout(*kv).total;
    case EKV_OP_ENTMAX_DECODE_SMALL:  // k_or_0: max_count
      return k_or_0 >= 1 ? ekv::small_ws_bytes(*kv, k_or_0) : 0;
    default:
      return 0;
  }
}

size_t ekv_score_size(const ekv_paged_kv *kv, int32_t mode) {
  if (check_kv(kv, false, false) != EKV_OK) return 0;
  const size_t Hq = static_cast<size_t>(kv->num_kv_heads) * kv->group;
  const size_t B = kv->batch, H = kv->num_kv_heads, MP = kv->max_pages;
  const size_t T = ekv::page_tiles(*kv);
  if (mode == EKV_SCORE_BBOX) return B * Hq * MP + B * H * T;
  if (mode == EKV_SCORE_GAUSS)
    return ekv::gstat_tile_offset(kv->batch, static_cast<int>(Hq), kv->max_pages) +
           B * Hq * T * 4;
  return 0;
}

ekv_status ekv_build_meta(const ekv_paged_kv *kv, const int32_t *first_page,
                          int32_t span_hint, const ekv_meta *meta,
                          void *stream) {
  EKV_TRY(check_kv(kv, true, false));
  if (!meta) return fail(EKV_ERR_INVALID_ARG, "meta is NULL");
  if (!meta->bbox && !meta->gauss)
    return fail(EKV_ERR_INVALID_ARG, "meta has neither bbox nor gauss");
  if ((meta->bbox && !aligned(meta->bbox, 16)) ||
      (meta->gauss && !aligned(meta->gauss, 16)))
    return fail(EKV_ERR_INVALID_ARG, "metadata must be 16-byte aligned");
  const hipError_t e = with_edg(*kv, [&](auto E, auto D, auto) {
    return ekv::launch_build_meta<decltype(E), decltype(D)::value>(
        *kv, first_page, span_hint, *meta, as_stream(stream));
  });
  return hip_status(e, "ekv_build_meta launch");
}

namespace {
ekv_status score_pages(const char *who, const ekv_paged_kv *kv,
                       const ekv_meta *meta, const float *q, float scale,
                       int32_t mode, float *ub, float *gstat, bool refresh,
                       void *stream) {
  EKV_TRY(check_kv(kv, refresh, false));
  EKV_TRY(check_scale(scale));
  if (!meta || !q) return fail(EKV_ERR_INVALID_ARG, "meta and q are required");
  if (mode <= 0 || (mode & ~(EKV_SCORE_BBOX | EKV_SCORE_GAUSS)))
    return fail(EKV_ERR_INVALID_ARG, "mode %d is not a set of EKV_SCORE_*", mode);
  if ((mode & EKV_SCORE_BBOX) && (!meta->bbox || !ub))
    return fail(EKV_ERR_INVALID_ARG, "box scoring needs meta->bbox and ub");
  if ((mode & EKV_SCORE_GAUSS) && (!meta->gauss || !gstat))
    return fail(EKV_ERR_INVALID_ARG, "Gaussian scoring needs meta->gauss and gstat");
  if ((meta->bbox && !aligned(meta->bbox, 16)) ||
      (meta->gauss && !aligned(meta->gauss, 16)) || !aligned(q, 16) ||
      (gstat && !aligned(gstat, 16)))
    return fail(EKV_ERR_INVALID_ARG, "q, metadata and gstat must be 16-byte aligned");
  const hipError_t e = with_edg(*kv, [&](auto E, auto D, auto G) {
    return ekv::launch_score<decltype(E), decltype(D)::value,
                             decltype(G)::value>(*kv, *meta, q, scale, mode,
                                                 ub, gstat, refresh,
                                                 as_stream(stream));
  });
  return hip_status(e, who);
}
}  // namespace

ekv_status ekv_score_pages(const ekv_paged_kv *kv, const ekv_meta *meta,
                           const float *q, float scale, int32_t mode,
                           float *ub, float *gstat, void *stream) {
  return score_pages("ekv_score_pages launch", kv, meta, q, scale, mode, ub,
                     gstat, false, stream);
}

ekv_status ekv_refresh_score_pages(const ekv_paged_kv *kv, const ekv_meta *meta,
                                   const float *q, float scale, int32_t mode,
                                   float *ub, float *gstat, void *stream) {
  return score_pages("ekv_refresh_score_pages launch", kv, meta, q, scale,
                     mode, ub, gstat, true, stream);
}

ekv_status ekv_select_topk(const ekv_paged_kv *kv, const float *ub, int32_t k,
                           int32_t *sel, int32_t *count, void *ws,
                           size_t ws_bytes, void *stream) {
  EKV_TRY(check_kv(kv, false, false));
  if (!ub || !sel || !count)
    return fail(EKV_ERR_INVALID_ARG, "ub, sel and count are required");
  if (k < 1) return fail(EKV_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  EKV_TRY(check_ws(ws, ws_bytes, ekv_workspace_size(EKV_OP_SELECT_TOPK, kv, k)));
  const hipError_t e = with_g(*kv, [&](auto G) {
    return ekv::launch_select_topk<decltype(G)::value>(*kv, ub, k, sel, count,
                                                      ws, as_stream(stream));
  });
  return hip_status(e, "ekv_select_topk launch");
}

ekv_status ekv_select_gauss(const ekv_paged_kv *kv, const float *gstat,
                            float alpha, float delta, int32_t *sel,
                            int32_t *count, float *tau_hat, void *ws,
                            size_t ws_bytes, void *stream) {
  EKV_TRY(check_kv(kv, false, false));
  EKV_TRY(check_alpha(alpha));
  if (!(alpha >= 1.1f && alpha <= 2.0f))
    return fail(EKV_ERR_UNSUPPORTED,
                "Gaussian selector built for 1.1 <= alpha <= 2 (got %g)",
                static_cast<double>(alpha));
  if (std::isnan(delta) || delta < 0.0f)
    return fail(EKV_ERR_INVALID_ARG, "delta must be >= 0 (got %g)",
                static_cast<double>(delta));
  if (!gstat || !sel || !count || !tau_hat)
    return fail(EKV_ERR_INVALID_ARG, "gstat, sel, count and tau_hat are required");
  if (!aligned(gstat, 16)) return fail(EKV_ERR_INVALID_ARG, "gstat must be 16-byte aligned");
  EKV_TRY(check_ws(ws, ws_bytes, ekv_workspace_size(EKV_OP_SELECT_GAUSS, kv, 0)));
  const hipError_t e = with_g(*kv, [&](auto G) {
    return ekv::launch_select_gauss<decltype(G)::value>(
        *kv, gstat, alpha, delta, sel, count, tau_hat, ws, as_stream(stream));
  });
  return hip_status(e, "ekv_select_gauss launch");
}

ekv_status ekv_entmax_scores(const ekv_paged_kv *kv, const float *q,
                             float scale, float alpha, const int32_t *sel,
                             const int32_t *count, const float *tau_hint,
                             void *ws, size_t ws_bytes, void *stream) {
  EKV_TRY(check_kv(kv, true, false));
  EKV_TRY(check_scale(scale));
  EKV_TRY(check_alpha(alpha));
  EKV_TRY(check_sel(sel, count));
  if (!q || !aligned(q, 16))
    return fail(EKV_ERR_INVALID_ARG, "q must be non-NULL and 16-byte aligned");
  EKV_TRY(check_ws(ws, ws_bytes, ekv_workspace_size(EKV_OP_ENTMAX_DECODE, kv, 0)));
  const hipError_t e = with_edg(*kv, [&](auto E, auto D, auto G) {
    return ekv::launch_entmax_scores<decltype(E), decltype(D)::value,
                                     decltype(G)::value>(
        *kv, q, scale, alpha, sel, count, tau_hint, ws, as_stream(stream));
  });
  return hip_status(e, "ekv_entmax_scores launch");
}

ekv_status ekv_entmax_threshold(const ekv_paged_kv *kv, float alpha,
                                const int32_t *sel, const int32_t *count,
                                float *tau, float *out, void *ws,
                                size_t ws_bytes, void *stream) {
  EKV_TRY(check_kv(kv, true, true));
  EKV_TRY(check_alpha(alpha));
  EKV_TRY(check_sel(sel, count));
  if (!out) return fail(EKV_ERR_INVALID_ARG, "out is required");
  EKV_TRY(check_ws(ws, ws_bytes, ekv_workspace_size(EKV_OP_ENTMAX_DECODE, kv, 0)));
  const hipError_t e = with_edg(*kv, [&](auto E, auto D, auto G) {
    return ekv::launch_entmax_threshold<decltype(E), decltype(D)::value,
                                        decltype(G)::value>(
        *kv, alpha, sel, count, tau, out, ws, as_stream(stream));
  });
  return hip_status(e, "ekv_entmax_threshold launch");
}

ekv_status ekv_entmax_apply(const ekv_paged_kv *kv, float alpha,
                            const int32_t *sel, const int32_t *count,
                            float *out, float *probs, void *ws,
                            size_t ws_bytes, void *stream) {
  EKV_TRY(check_kv(kv, false, true));
  EKV_TRY(check_alpha(alpha));
  EKV_TRY(check_sel(sel, count));
  if (!out) return fail(EKV_ERR_INVALID_ARG, "out is required");
  EKV_TRY(check_ws(ws, ws_bytes, ekv_workspace_size(EKV_OP_ENTMAX_DECODE, kv, 0)));
  const hipError_t e = with_edg(*kv, [&](auto E, auto D, auto G) {
    return ekv::launch_entmax_apply<decltype(E), decltype(D)::value,
                                    decltype(G)::value>(
        *kv, alpha, sel, count, out, probs, ws, as_stream(stream));
  });
  return hip_status(e, "ekv_entmax_apply launch");
}

ekv_status ekv_entmax_decode(const ekv_paged_kv *kv, const float *q,
                             float scale, float alpha, const int32_t *sel,
                             const int32_t *count, const float *tau_hint,
                             float *out, float *tau, float *probs, void *ws,
                             size_t ws_bytes, void *stream) {
  EKV_TRY(check_kv(kv, true, true));
  if (!out) return fail(EKV_ERR_INVALID_ARG, "out is required");
  // the debug probabilities need every score: the hint is not used then
  EKV_TRY(ekv_entmax_scores(kv, q, scale, alpha, sel, count,
                            probs ? nullptr : tau_hint, ws, ws_bytes, stream));
  EKV_TRY(ekv_entmax_threshold(kv, alpha, sel, count, tau, out, ws, ws_bytes, stream));
  return ekv_entmax_apply(kv, alpha, sel, count, out, probs, ws, ws_bytes, stream);
}

ekv_status ekv_entmax_decode_noalloc(const ekv_paged_kv *kv, const float *q,
                                     float scale, float alpha,
                                     const int32_t *sel, const int32_t *count,
                                     const float *tau_hint, float *out,
                                     float *tau, float *probs, void *stream) {
  EKV_TRY(check_kv(kv, true, true));
  const size_t need = ekv_workspace_size(EKV_OP_ENTMAX_DECODE, kv, 0);
  if (need > kScratchBytes)
    return fail(EKV_ERR_WORKSPACE,
                "this cache needs %zu bytes of decode workspace; the static "
                "scratch holds %zu (use ekv_entmax_decode with a workspace)",
                need, kScratchBytes);
  void *ws = nullptr;
  EKV_TRY(scratch_on(as_stream(stream), &ws));
  return ekv_entmax_decode(kv, q, scale, alpha, sel, count, tau_hint, out, tau,
                           probs, ws, kScratchBytes, stream);
}

ekv_status ekv_entmax_decode_small(const ekv_paged_kv *kv, const float *q,
                                   float scale, float alpha,
                                   const int32_t *sel, const int32_t *count,
                                   int32_t max_count, float *out, float *tau,
                                   void *ws, size_t ws_bytes, void *stream) {
  EKV_TRY(check_kv(kv, true, true));
  EKV_TRY(check_scale(scale));
  EKV_TRY(check_alpha(alpha));
  EKV_TRY(check_sel(sel, count));
  if (!q || !aligned(q, 16) || !out)
    return fail(EKV_ERR_INVALID_ARG, "q (16-byte aligned) and out are required");
  if (kv->kv_dtype != EKV_BF16)
    return fail(EKV_ERR_UNSUPPORTED, "the small-selection decode is built for bfloat16 keys");
  if (max_count < 1)
    return fail(EKV_ERR_INVALID_ARG, "max_count must be >= 1 (got %d)", max_count);
  if (static_cast<long long>(max_count) * kv->page_size > ekv::kSmallTokens)
    return fail(EKV_ERR_UNSUPPORTED,
                "max_count %d * page_size %d exceeds the %d tokens held on chip",
                max_count, kv->page_size, ekv::kSmallTokens);
  EKV_TRY(check_ws(ws, ws_bytes, ekv::small_ws_bytes(*kv, max_count)));
  const hipError_t e = with_edg(*kv, [&](auto, auto D, auto G) {
    return ekv::launch_entmax_small<decltype(D)::value, decltype(G)::value>(
        *kv, q, scale, alpha, sel, count, max_count, out, tau, ws, as_stream(stream));
  });
  return hip_status(e, "ekv_entmax_decode_small launch");
}

ekv_status ekv_softmax_decode(const ekv_paged_kv *kv, const float *q,
                              float scale, const int32_t *sel,
                              const int32_t *count, float *out, float *lse,
                              void *ws, size_t ws_bytes, void *stream) {
  EKV_TRY(check_kv(kv, true, true));
  EKV_TRY(check_scale(scale));
  EKV_TRY(check_sel(sel, count));
  if (!q || !aligned(q, 16) || !out)
    return fail(EKV_ERR_INVALID_ARG, "q (16-byte aligned) and out are required");
  EKV_TRY(check_ws(ws, ws_bytes, ekv_workspace_size(EKV_OP_SOFTMAX_DECODE, kv, 0)));
  const hipError_t e = with_edg(*kv, [&](auto E, auto D, auto G) {
    return ekv::launch_softmax<decltype(E), decltype(D)::value,
                               decltype(G)::value>(*kv, q, scale, sel, count,
                                                   out, lse, ws,
                                                   as_stream(stream));
  });
  return hip_status(e, "ekv_softmax_decode launch");
}

ekv_status ekv_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                          void *stream) {
  if (!buf || !sink || !aligned(buf, 16) || (bytes & 15) != 0)
    return fail(EKV_ERR_INVALID_ARG,
                "buf (16-byte aligned), sink and a multiple of 16 bytes required");
  return hip_status(ekv::launch_read_probe(buf, bytes, sink, as_stream(stream)),
                    "ekv_read_probe launch");
}

ekv_status ekv_quadrature_rule(int32_t kind, double param, int32_t n,
                               double *nodes, double *weights) {
  if (!nodes || !weights || n < 1 || n > ekv::kMaxRuleNodes)
    return fail(EKV_ERR_INVALID_ARG, "nodes, weights and 1 <= n <= %d required",
                ekv::kMaxRuleNodes);
  bool ok = false;
  if (kind == EKV_RULE_JACOBI) ok = ekv::gauss_jacobi_rule(param, n, nodes, weights);
  else if (kind == EKV_RULE_HERMITE) ok = ekv::gauss_hermite_rule(n, nodes, weights);
  if (!ok) return fail(EKV_ERR_INVALID_ARG, "unknown rule kind or parameter out of range");
  return EKV_OK;
}

const char *ekv_status_string(ekv_status s) {
  switch (s) {
    case EKV_OK: return "EKV_OK";
    case EKV_ERR_INVALID_ARG: return "EKV_ERR_INVALID_ARG";
    case EKV_ERR_UNSUPPORTED: return "EKV_ERR_UNSUPPORTED";
    case EKV_ERR_WORKSPACE: return "EKV_ERR_WORKSPACE";
    case EKV_ERR_HIP: return "EKV_ERR_HIP";
  }
  return "EKV_UNKNOWN_STATUS";
}

const char *ekv_last_error(void) { return g_last_error.c_str(); }

int32_t ekv_version(void) { return EKV_VERSION; }

}  // extern "C"
