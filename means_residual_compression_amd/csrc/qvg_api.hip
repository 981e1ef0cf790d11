// C ABI of the QVG library (declared in include/qvg.h): argument validation,
// workspace carve-up and the stage x iteration orchestration of the compress
// path.  All device work is enqueued on the caller's stream; nothing here
// synchronises or allocates device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <type_traits>
#include <vector>

#include "qvg.h"
#include "qvg_attn.h"
#include "qvg_internal.h"

using namespace qvg;

namespace {

thread_local char g_err[512];

qvg_status fail(qvg_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

qvg_status hip_fail(const char *what) {
  return fail(QVG_ERR_HIP, "%s: %s", what, hipGetErrorString(hipGetLastError()));
}

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Workspace layout shared by the size query and the carve-up.
struct Layout {
  size_t rt, tb, cent, ctab, cinit, cbnd, stats, recheck, fallback, counters, sorted, offs, hist,
      cofs, chunk_j, part, pflag, stage_re, stage_fb, span, idx, isum, lminv, prev, mcnt;
  size_t total;
  bool incremental;
};

// incremental: room for the state of the incremental centroid update (the
// compress paths; the lone assign has no update).
Layout make_layout(int64_t H, int64_t N, int64_t d, int64_t C, int64_t T, bool need_idx,
                   bool incremental = true) {
  const int64_t Cp = std::max<int64_t>(32, pad32((int)C));
  const int64_t NT = (N + kTile - 1) / kTile;
  const int64_t Ts = std::max<int64_t>(T, 1);
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = up(o + bytes); return at; };
  L.rt = take((size_t)(H * NT * kTile * d * 2));
  L.tb = take((size_t)(H * NT * kTile * 8));
  L.cent = take((size_t)(H * Cp * d * 4));
  L.ctab = take((size_t)(H * Cp * d * 2));
  L.cinit = take((size_t)(H * Cp * 4));
  L.cbnd = take((size_t)(H * Cp * 16));
  L.stats = take((size_t)(H * Ts * kStatWords * 4));
  L.recheck = take((size_t)(H * NT * kTile * 16));
  L.fallback = take((size_t)(H * NT * kTile * 8));
  L.counters = take(kCounterWords * 4);
  L.sorted = take((size_t)(H * N * 4));
  L.offs = take((size_t)(H * (Cp + 1) * 4));
  L.hist = take((size_t)(H * ((N + kSortChunk - 1) / kSortChunk) * kMaxC * 4));
  L.cofs = take((size_t)(H * (Cp + 1) * 4));
  L.chunk_j = take((size_t)(H * max_chunks((int)N, (int)Cp) * 4));
  L.part = take((size_t)(H * max_chunks((int)N, (int)Cp) * d * 8));
  L.pflag = take((size_t)(H * max_chunks((int)N, (int)Cp) * d * 4));
  L.stage_re = take((size_t)(H * (NT + 15) * kTile * 16));
  L.stage_fb = take((size_t)(H * (NT + 15) * kTile * 8));
  L.span = take((size_t)(H * kSpanParts * d * 4));
  L.idx = take(need_idx ? (size_t)(H * T * C * 4) : 0);
  L.incremental = incremental;
  L.isum = take(incremental ? (size_t)(H * Cp * d * 8) : 0);
  L.lminv = take(incremental ? (size_t)(H * d * 4) : 0);
  L.prev = take(incremental ? (size_t)(2 * H * N) : 0);
  L.mcnt = take(incremental ? (size_t)(H * ((N + kSortChunk - 1) / kSortChunk) * 4) : 0);
  L.total = o;
  return L;
}

Ws carve(void *ws, const Layout &L) {
  char *b = (char *)ws;
  Ws w;
  w.rt = (half8 *)(b + L.rt);
  w.tb = (float2 *)(b + L.tb);
  w.cent = (float *)(b + L.cent);
  w.ctab = (half8 *)(b + L.ctab);
  w.cinit = (float *)(b + L.cinit);
  w.cbnd = (float4 *)(b + L.cbnd);
  w.stats = (uint32_t *)(b + L.stats);
  w.recheck = (int4 *)(b + L.recheck);
  w.fallback = (int2 *)(b + L.fallback);
  w.counters = (uint32_t *)(b + L.counters);
  w.sorted = (int32_t *)(b + L.sorted);
  w.offs = (int32_t *)(b + L.offs);
  w.hist = (uint32_t *)(b + L.hist);
  w.cofs = (int32_t *)(b + L.cofs);
  w.chunk_j = (int32_t *)(b + L.chunk_j);
  w.part = (double *)(b + L.part);
  w.pflag = (uint32_t *)(b + L.pflag);
  w.stage_re = (int4 *)(b + L.stage_re);
  w.stage_fb = (int2 *)(b + L.stage_fb);
  w.span = (uint32_t *)(b + L.span);
  w.idx = (int32_t *)(b + L.idx);
  const bool inc = L.incremental;
  w.isum = inc ? (long long *)(b + L.isum) : nullptr;
  w.lminv = inc ? (uint32_t *)(b + L.lminv) : nullptr;
  w.prev = inc ? (uint8_t *)(b + L.prev) : nullptr;
  w.mcnt = inc ? (uint32_t *)(b + L.mcnt) : nullptr;
  return w;
}

qvg_status check_dims(int64_t H, int64_t N, int64_t d, qvg_dtype dt) {
  if (H < 1 || H > 65535) return fail(QVG_ERR_INVALID_ARG, "H=%lld must be in [1, 65535]", (long long)H);
  if (N < 1 || N > (1 << 30)) return fail(QVG_ERR_INVALID_ARG, "N=%lld must be in [1, 2^30]", (long long)N);
  if (d != 64 && d != 128) return fail(QVG_ERR_UNSUPPORTED, "d=%lld: supported head dims are 64 and 128", (long long)d);
  if (dt != QVG_F32 && dt != QVG_BF16) return fail(QVG_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  return QVG_OK;
}

qvg_status check_quant(int64_t d, int32_t bits, int32_t G) {
  if (bits != 2 && bits != 4) return fail(QVG_ERR_UNSUPPORTED, "bits=%d: only 2 and 4", bits);
  if (G < 8 || G > d || G % 8 != 0 || d % G != 0)
    return fail(QVG_ERR_UNSUPPORTED, "group=%d must be a multiple of 8 dividing d=%lld", G, (long long)d);
  return QVG_OK;
}

qvg_status check_params(int64_t H, int64_t N, int64_t d, qvg_dtype dt, const qvg_params *p,
                        int32_t iters) {
  if (!p) return fail(QVG_ERR_INVALID_ARG, "params is NULL");
  qvg_status s = check_dims(H, N, d, dt);
  if (s != QVG_OK) return s;
  if (p->T < 0 || p->T > kMaxT) return fail(QVG_ERR_UNSUPPORTED, "T=%d must be in [0, %d]", p->T, kMaxT);
  if (p->C < 1 || p->C > kMaxC) return fail(QVG_ERR_UNSUPPORTED, "C=%d must be in [1, 256]", p->C);
  if (p->T > 0 && p->C > N) return fail(QVG_ERR_INVALID_ARG, "C=%d exceeds N=%lld", p->C, (long long)N);
  if (p->T > 0 && iters < 1) return fail(QVG_ERR_INVALID_ARG, "iterations must be >= 1 (got %d)", iters);
  return check_quant(d, p->bits, p->group);
}

// Relative error coefficient of an MFMA key (see k_assign): fp32
// accumulation of K = d products plus the init (2 gamma_{K+1}, doubled for
// the unknown internal order), the 8-bit index embedding (2^-15) and the
// rounding of the accumulator init (2^-22 covers it).
float kappa_for(int64_t d) {
  const double K = (double)d + 1.0, u = std::ldexp(1.0, -24);
  const double gamma = K * u / (1.0 - K * u);
  const double k = 2.0 * gamma + std::ldexp(1.0, -15) + std::ldexp(1.0, -22);
  return std::nextafter((float)k, 1.0f);
}

// True when p is device (or managed) memory that kernels can read; pageable
// or pinned host memory is false.  The query's error for unregistered host
// pointers is cleared.
bool device_resident(const void *p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged;
}

// idx: device rows [H][T][C] of every stage start, or nullptr when the
// stages start from init_c.
template <typename Tin, typename Tc, int D>
qvg_status run_compress(const void *x, int64_t H, int64_t N, const qvg_params *p, int32_t iters,
                        const int32_t *idx, const float *init_c, float *cache_out,
                        const qvg_record *out, const Ws &w, hipStream_t s) {
  const int T = p->T, C = p->C;
  const int Cp = std::max(32, pad32(C));
  const int NT = (int)((N + kTile - 1) / kTile);
  const bool x_bf16 = std::is_same<Tin, uint16_t>::value;
  const int stat_stride = std::max(T, 1) * kStatWords;
  if (!launch_fill_u32(w.stats, (int64_t)H * stat_stride, s) || !launch_fill_u32(w.counters, kCounterWords, s))
    return hip_fail("fill");
  if (T == 0) {
    if (!launch_quant(x, x_bf16, (int)H, (int)N, D, 1, nullptr, nullptr, 1, 0, p->bits,
                      p->group, out->codes, out->scales, s))
      return hip_fail("group_quant_pack");
    return QVG_OK;
  }
  if (!launch_absmax<Tin>(x, (int)H, N * D, w.stats, stat_stride, S_MAXR, s))
    return hip_fail("absmax");
  const int64_t rec_hstride = (int64_t)T * C * D;
  for (int t = 0; t < T; ++t) {
    if (t > 0 && !launch_stage_bound(w.stats + (int64_t)(t - 1) * kStatWords, stat_stride,
                                     (int)H, s))
      return hip_fail("stage bound");
    KmArgs a;
    a.H = (int)H; a.N = (int)N; a.C = C; a.Cp = Cp; a.NT = NT;
    a.x = x; a.rec_pi = out->assign; a.rec_cent = out->centroids; a.Ts = T; a.nsub = t;
    a.idx = idx ? idx + (int64_t)t * C : nullptr;
    a.idx_hstride = (int64_t)T * C;
    a.init = idx ? nullptr : init_c + (int64_t)t * C * D;
    a.init_hstride = rec_hstride;
    a.assign = out->assign + (int64_t)t * N;
    a.assign_hstride = (int64_t)T * N;
    a.ws = w;
    a.ws_stats = w.stats + (int64_t)t * kStatWords;
    a.stat_stride = stat_stride;
    a.kappa = kappa_for(D);
    const bool in_bf16 = x_bf16;
    bool ok = in_bf16 ? launch_kmeans_stage_begin<uint16_t, D>(a, s)
                      : launch_kmeans_stage_begin<float, D>(a, s);
    if (!ok) return hip_fail("k-means stage init");
    Tc *rec_c = (Tc *)out->centroids + (int64_t)t * C * D;
    float *cache_t = cache_out ? cache_out + (int64_t)t * C * D : nullptr;
    for (int it = 0; it < iters; ++it) {
      const int bslot = S_B0 + 4 * (it & 1), next = S_B0 + 4 * ((it + 1) & 1);
      const bool last = it == iters - 1;
      ok = in_bf16 ? launch_assign<uint16_t, D>(a, bslot, s) : launch_assign<float, D>(a, bslot, s);
      if (!ok) return hip_fail("kmeans_assign");
      const int log_slot = t * iters + it;
      ok = in_bf16 ? launch_update<uint16_t, Tc, D>(a, next, !last, last ? rec_c : nullptr,
                                                    rec_hstride, last ? cache_t : nullptr,
                                                    rec_hstride, log_slot, it, s)
                   : launch_update<float, Tc, D>(a, next, !last, last ? rec_c : nullptr,
                                                 rec_hstride, last ? cache_t : nullptr,
                                                 rec_hstride, log_slot, it, s);
      if (!ok) return hip_fail("kmeans_update");
    }
  }
  // R(T), recomputed from x and the record, quantized and packed
  if (!launch_quant(x, x_bf16, (int)H, (int)N, D, C, out->assign, out->centroids, T, T,
                    p->bits, p->group, out->codes, out->scales, s))
    return hip_fail("group_quant_pack");
  return QVG_OK;
}

qvg_status compress_impl(const void *x, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                         const qvg_params *p, int32_t iters, const int32_t *init_idx,
                         const float *init_c, float *cache_out, const qvg_record *out, void *ws,
                         size_t ws_bytes, void *stream) {
  qvg_status st = check_params(H, N, d, dtype, p, iters);
  if (st != QVG_OK) return st;
  if (!x || !out || !out->codes || !out->scales)
    return fail(QVG_ERR_INVALID_ARG, "x, out, out->codes and out->scales must be non-NULL");
  if (p->T > 0) {
    if (!out->assign || !out->centroids)
      return fail(QVG_ERR_INVALID_ARG, "out->assign and out->centroids must be non-NULL when T >= 1");
    if (init_idx && init_c)
      return fail(QVG_ERR_INVALID_ARG, "give at most one of init_idx and init_centroids");
  }
  // stage starts: host rows (validated, then copied), device rows (read by
  // the kernels), caller centroids, or rows drawn from p->seed on the device
  const bool rows = p->T > 0 && init_c == nullptr;
  const bool rows_dev = rows && init_idx != nullptr && device_resident(init_idx);
  const bool rows_host = rows && init_idx != nullptr && !rows_dev;
  const bool rows_seeded = rows && init_idx == nullptr;
  const Layout L = make_layout(H, N, d, p->C, p->T, rows_host || rows_seeded);
  if (!ws) return fail(QVG_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < L.total)
    return fail(QVG_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, L.total);
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(QVG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (rows_host) {
    const int64_t n = H * p->T * p->C;
    for (int64_t q = 0; q < n; ++q)
      if (init_idx[q] < 0 || init_idx[q] >= N)
        return fail(QVG_ERR_INVALID_ARG, "init_idx[%lld]=%d is outside [0, N=%lld)", (long long)q,
                    init_idx[q], (long long)N);
  }
  const Ws w = carve(ws, L);
  hipStream_t s = (hipStream_t)stream;
  if (rows_host &&
      hipMemcpyAsync(w.idx, init_idx, (size_t)(H * p->T * p->C) * 4, hipMemcpyHostToDevice, s) != hipSuccess)
    return hip_fail("copy init_idx");
  if (rows_seeded && !launch_sample_rows((int)H, p->T, (int)N, p->C, p->seed, w.idx, s))
    return hip_fail("seeded rows");
  const int32_t *idx = rows_dev ? init_idx : (rows ? w.idx : nullptr);
  const bool bf = dtype == QVG_BF16;
  if (d == 64)
    return bf ? run_compress<uint16_t, uint16_t, 64>(x, H, N, p, iters, idx, init_c, cache_out, out, w, s)
              : run_compress<float, float, 64>(x, H, N, p, iters, idx, init_c, cache_out, out, w, s);
  return bf ? run_compress<uint16_t, uint16_t, 128>(x, H, N, p, iters, idx, init_c, cache_out, out, w, s)
            : run_compress<float, float, 128>(x, H, N, p, iters, idx, init_c, cache_out, out, w, s);
}

// Device scratch of qvg_compress_stream_static: one array per GPU, held until
// the process ends.  In host code `scratch` only names the symbol; its device
// address on each GPU comes from hipGetSymbolAddress with that GPU current.
static __device__ __align__(256) unsigned char scratch[QVG_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Address of the current device's scratch (looked up once per device).
qvg_status static_scratch(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hip_fail("hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QVG_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return hip_fail("hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QVG_OK;
}

}  // namespace

extern "C" {

const char *qvg_status_string(qvg_status s) {
  switch (s) {
    case QVG_OK: return "QVG_OK";
    case QVG_ERR_INVALID_ARG: return "QVG_ERR_INVALID_ARG";
    case QVG_ERR_UNSUPPORTED: return "QVG_ERR_UNSUPPORTED";
    case QVG_ERR_WORKSPACE: return "QVG_ERR_WORKSPACE";
    case QVG_ERR_HIP: return "QVG_ERR_HIP";
  }
  return "QVG_UNKNOWN_STATUS";
}

const char *qvg_last_error(void) { return g_err; }

size_t qvg_workspace_size(int64_t H, int64_t N, int64_t d, qvg_dtype dtype, const qvg_params *p) {
  if (check_params(H, N, d, dtype, p, p ? std::max(p->iters, 1) : 1) != QVG_OK) return 0;
  return make_layout(H, N, d, p->C, p->T, p->T > 0).total;
}

qvg_status qvg_compress(const void *x, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                        const qvg_params *p, const int32_t *init_idx, const float *init_centroids,
                        float *cache_out, const qvg_record *out, void *ws, size_t ws_bytes,
                        void *stream) {
  g_err[0] = 0;
  return compress_impl(x, dtype, H, N, d, p, p ? p->iters : 0, init_idx, init_centroids,
                       cache_out, out, ws, ws_bytes, stream);
}

qvg_status qvg_compress_stream(const void *chunk, qvg_dtype dtype, int64_t H, int64_t N,
                               int64_t d, const qvg_params *p, int32_t iters_warm, float *cache,
                               int warm, const int32_t *init_idx, const qvg_record *out, void *ws,
                               size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (!p) return fail(QVG_ERR_INVALID_ARG, "params is NULL");
  if (p->T > 0 && !cache) return fail(QVG_ERR_INVALID_ARG, "cache must be non-NULL when T >= 1");
  if (warm)
    return compress_impl(chunk, dtype, H, N, d, p, iters_warm, nullptr, cache, cache, out, ws,
                         ws_bytes, stream);
  return compress_impl(chunk, dtype, H, N, d, p, p->iters, init_idx, nullptr, cache, out, ws,
                       ws_bytes, stream);
}

qvg_status qvg_compress_stream_static(const void *chunk, qvg_dtype dtype, int64_t H, int64_t N,
                                      int64_t d, const qvg_params *p, int32_t iters_warm,
                                      float *cache, int warm, const int32_t *init_idx,
                                      const qvg_record *out, void *stream) {
  g_err[0] = 0;
  if (!p) return fail(QVG_ERR_INVALID_ARG, "params is NULL");
  if (p->T > 0 && !cache) return fail(QVG_ERR_INVALID_ARG, "cache must be non-NULL when T >= 1");
  qvg_status st = check_params(H, N, d, dtype, p, warm ? iters_warm : p->iters);
  if (st != QVG_OK) return st;
  const size_t need = make_layout(H, N, d, p->C, p->T, p->T > 0).total;
  if (need > (size_t)QVG_STATIC_SCRATCH_BYTES)
    return fail(QVG_ERR_WORKSPACE,
                "these sizes need %zu bytes of scratch, more than the %u of the static array",
                need, (unsigned)QVG_STATIC_SCRATCH_BYTES);
  void *ws = nullptr;
  st = static_scratch(&ws);
  if (st != QVG_OK) return st;
  return qvg_compress_stream(chunk, dtype, H, N, d, p, iters_warm, cache, warm, init_idx, out, ws,
                             (size_t)QVG_STATIC_SCRATCH_BYTES, stream);
}

qvg_status qvg_decompress(const qvg_record *rec, qvg_dtype rec_dtype, int64_t H, int64_t N,
                          int64_t d, const qvg_params *p, void *out, qvg_dtype out_dtype,
                          void *stream) {
  g_err[0] = 0;
  if (!p) return fail(QVG_ERR_INVALID_ARG, "params is NULL");
  qvg_status st = check_dims(H, N, d, rec_dtype);
  if (st != QVG_OK) return st;
  if (out_dtype != QVG_F32 && out_dtype != QVG_BF16) return fail(QVG_ERR_INVALID_ARG, "unknown out dtype");
  if (p->T < 0 || p->T > kMaxT) return fail(QVG_ERR_UNSUPPORTED, "T=%d must be in [0, 8]", p->T);
  if (p->T > 0 && (p->C < 1 || p->C > kMaxC)) return fail(QVG_ERR_UNSUPPORTED, "C=%d must be in [1, 256]", p->C);
  st = check_quant(d, p->bits, p->group);
  if (st != QVG_OK) return st;
  if (!rec || !rec->codes || !rec->scales || !out) return fail(QVG_ERR_INVALID_ARG, "NULL record or output");
  if (p->T > 0 && (!rec->assign || !rec->centroids)) return fail(QVG_ERR_INVALID_ARG, "NULL assign/centroids");
  if (!launch_dequant(rec->codes, rec->scales, rec->assign, rec->centroids, rec_dtype == QVG_BF16,
                      (int)H, (int)N, (int)d, p->C, p->T, p->bits, p->group, out,
                      out_dtype == QVG_BF16, (hipStream_t)stream))
    return hip_fail("fused_dequant");
  return QVG_OK;
}

qvg_status qvg_decompress_chunks(const qvg_record *recs, const int64_t *n_tokens,
                                 int32_t n_chunks, qvg_dtype rec_dtype, int64_t H, int64_t d,
                                 const qvg_params *p, void *out, qvg_dtype out_dtype,
                                 void *stream) {
  g_err[0] = 0;
  if (!p || !recs || !n_tokens || !out) return fail(QVG_ERR_INVALID_ARG, "NULL argument");
  if (n_chunks < 1) return fail(QVG_ERR_INVALID_ARG, "n_chunks=%d must be >= 1", n_chunks);
  int64_t total = 0;
  for (int32_t c = 0; c < n_chunks; ++c) {
    if (n_tokens[c] < 1) return fail(QVG_ERR_INVALID_ARG, "chunk %d has %lld tokens", c, (long long)n_tokens[c]);
    total += n_tokens[c];
    if (total > (1 << 30)) return fail(QVG_ERR_UNSUPPORTED, "more than 2^30 tokens per head");
  }
  qvg_status st = check_dims(H, total, d, rec_dtype);
  if (st != QVG_OK) return st;
  if (out_dtype != QVG_F32 && out_dtype != QVG_BF16) return fail(QVG_ERR_INVALID_ARG, "unknown out dtype");
  if (p->T < 0 || p->T > kMaxT) return fail(QVG_ERR_UNSUPPORTED, "T=%d must be in [0, 8]", p->T);
  if (p->T > 0 && (p->C < 1 || p->C > kMaxC)) return fail(QVG_ERR_UNSUPPORTED, "C=%d must be in [1, 256]", p->C);
  st = check_quant(d, p->bits, p->group);
  if (st != QVG_OK) return st;
  for (int32_t c = 0; c < n_chunks; ++c) {
    const qvg_record &r = recs[c];
    if (!r.codes || !r.scales) return fail(QVG_ERR_INVALID_ARG, "chunk %d: NULL codes/scales", c);
    if (p->T > 0 && (!r.assign || !r.centroids))
      return fail(QVG_ERR_INVALID_ARG, "chunk %d: NULL assign/centroids", c);
  }
  int64_t done = 0;
  for (int32_t c0 = 0; c0 < n_chunks; c0 += kMaxChunksPerLaunch) {
    ChunkTable tbl{};
    tbl.n = std::min<int32_t>(kMaxChunksPerLaunch, n_chunks - c0);
    tbl.out_off = done;
    tbl.out_hstride = total;
    tbl.off[0] = 0;
    for (int q = 0; q < tbl.n; ++q) {
      const qvg_record &r = recs[c0 + q];
      tbl.codes[q] = r.codes;
      tbl.scales[q] = r.scales;
      tbl.assign[q] = r.assign;
      tbl.cent[q] = r.centroids;
      tbl.off[q + 1] = tbl.off[q] + n_tokens[c0 + q];
    }
    if (!launch_dequant_chunks(tbl, rec_dtype == QVG_BF16, (int)H, (int)d, p->C, p->T, p->bits,
                               p->group, out, out_dtype == QVG_BF16, (hipStream_t)stream))
      return hip_fail("fused_dequant (chunks)");
    done += tbl.off[tbl.n];
  }
  return QVG_OK;
}

size_t qvg_attention_workspace_size(int64_t H, int64_t Nq, int64_t N, int64_t d,
                                    const qvg_params *vp) {
  if (!vp || H < 1 || H > 65535 || N < 1 || N > (1 << 30) || (d != 64 && d != 128) || Nq < 1 ||
      Nq > kAttnMaxQueries || vp->T < 0 || vp->T > kMaxT || (vp->T > 0 && (vp->C < 1 || vp->C > kMaxC)))
    return 0;
  return up(attn_scratch_floats((int)H, N, (int)Nq, (int)d, vp->T, std::max(vp->C, 1)) *
            sizeof(float));
}

qvg_status qvg_attention(const float *q, int64_t H, int64_t Nq, int64_t d,
                         const qvg_record *k_rec, const qvg_params *kp,
                         const qvg_record *v_rec, const qvg_params *vp, qvg_dtype rec_dtype,
                         int64_t N, float scale, const float *rope_cos, const float *rope_sin,
                         float *out, void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (!q || !out || !k_rec || !v_rec || !kp || !vp) return fail(QVG_ERR_INVALID_ARG, "NULL argument");
  if (!rope_cos != !rope_sin) return fail(QVG_ERR_INVALID_ARG, "give both rope tables or neither");
  if (Nq < 1 || Nq > kAttnMaxQueries)
    return fail(QVG_ERR_INVALID_ARG, "Nq=%lld must be in [1, %d]", (long long)Nq, kAttnMaxQueries);
  qvg_status st = check_dims(H, N, d, rec_dtype);
  if (st != QVG_OK) return st;
  const qvg_record *recs[2] = {k_rec, v_rec};
  const qvg_params *ps[2] = {kp, vp};
  AttnRec ar[2];
  for (int i = 0; i < 2; ++i) {
    const qvg_params *p = ps[i];
    const qvg_record &r = *recs[i];
    const char *who = i ? "values" : "keys";
    if (p->T < 0 || p->T > kMaxT) return fail(QVG_ERR_UNSUPPORTED, "%s: T=%d must be in [0, 8]", who, p->T);
    if (p->T > 0 && (p->C < 1 || p->C > kMaxC))
      return fail(QVG_ERR_UNSUPPORTED, "%s: C=%d must be in [1, 256]", who, p->C);
    st = check_quant(d, p->bits, p->group);
    if (st != QVG_OK) return st;
    if (!r.codes || !r.scales) return fail(QVG_ERR_INVALID_ARG, "%s: NULL codes/scales", who);
    if (p->T > 0 && (!r.assign || !r.centroids)) return fail(QVG_ERR_INVALID_ARG, "%s: NULL assign/centroids", who);
    if (((uintptr_t)r.codes & 3) || (p->T > 0 && ((uintptr_t)r.centroids & 15)))
      return fail(QVG_ERR_INVALID_ARG, "%s: codes must be 4-byte and centroids 16-byte aligned", who);
    ar[i] = AttnRec{r.codes, r.scales, r.assign, r.centroids, p->T, p->bits, p->group, std::max(p->C, 1)};
  }
  if (((uintptr_t)q & 15) || ((uintptr_t)rope_cos & 15) || ((uintptr_t)rope_sin & 15))
    return fail(QVG_ERR_INVALID_ARG, "q and the rope tables must be 16-byte aligned");
  const size_t need = qvg_attention_workspace_size(H, Nq, N, d, vp);
  if (!ws || ws_bytes < need) return fail(QVG_ERR_WORKSPACE, "workspace smaller than %zu bytes", need);
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(QVG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (!launch_attention(q, (int)H, (int)Nq, (int)N, (int)d, ar[0], ar[1], rec_dtype == QVG_BF16,
                        scale, rope_cos, rope_sin, static_cast<float *>(ws), out,
                        (hipStream_t)stream))
    return hip_fail("attention");
  return QVG_OK;
}

qvg_status qvg_candidate_counts(const void *ws, int64_t H, int64_t N, int64_t d, qvg_dtype dtype,
                                const qvg_params *p, uint32_t *out, int32_t n_iters) {
  g_err[0] = 0;
  qvg_status st = check_params(H, N, d, dtype, p, p ? std::max(p->iters, 1) : 1);
  if (st != QVG_OK) return st;
  if (!ws || !out || n_iters < 0 || n_iters > kCounterLog)
    return fail(QVG_ERR_INVALID_ARG, "ws/out NULL or n_iters outside [0, %d]", kCounterLog);
  const Layout L = make_layout(H, N, d, p->C, p->T, p->T > 0);
  if (hipMemcpy(out, (const char *)ws + L.counters + 16, (size_t)n_iters * 8,
                hipMemcpyDeviceToHost) != hipSuccess)
    return hip_fail("read candidate counts");
  return QVG_OK;
}

size_t qvg_assign_workspace_size(int64_t H, int64_t N, int64_t d, int32_t C) {
  if (check_dims(H, N, d, QVG_F32) != QVG_OK || C < 1 || C > kMaxC || C > N) return 0;
  return make_layout(H, N, d, C, 1, false, false).total;
}

qvg_status qvg_kmeans_assign(const void *r, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                             const float *centroids, int32_t C, uint8_t *assign, void *ws,
                             size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  qvg_status st = check_dims(H, N, d, dtype);
  if (st != QVG_OK) return st;
  if (C < 1 || C > kMaxC || C > N) return fail(QVG_ERR_UNSUPPORTED, "C=%d must be in [1, min(256, N)]", C);
  if (!r || !centroids || !assign) return fail(QVG_ERR_INVALID_ARG, "NULL pointer argument");
  const Layout L = make_layout(H, N, d, C, 1, false, false);
  if (!ws || ws_bytes < L.total) return fail(QVG_ERR_WORKSPACE, "workspace smaller than %zu bytes", L.total);
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(QVG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const Ws w = carve(ws, L);
  hipStream_t s = (hipStream_t)stream;
  KmArgs a;
  a.H = (int)H; a.N = (int)N; a.C = C; a.Cp = std::max(32, pad32(C));
  a.NT = (int)((N + kTile - 1) / kTile);
  a.x = r; a.rec_pi = nullptr; a.rec_cent = nullptr; a.Ts = 1; a.nsub = 0;
  a.idx = nullptr; a.idx_hstride = 0; a.init = centroids; a.init_hstride = (int64_t)C * d;
  a.assign = assign; a.assign_hstride = N; a.ws = w; a.ws_stats = w.stats;
  a.stat_stride = kStatWords; a.kappa = kappa_for(d);
  if (!launch_fill_u32(w.stats, H * kStatWords, s) || !launch_fill_u32(w.counters, kCounterWords, s)) return hip_fail("fill");
  const bool bf = dtype == QVG_BF16;
  bool ok;
  if (d == 64)
    ok = bf ? (launch_absmax<uint16_t>(r, (int)H, N * d, w.stats, kStatWords, S_MAXR, s) &&
               launch_kmeans_stage_begin<uint16_t, 64>(a, s) && launch_assign<uint16_t, 64>(a, S_B0, s))
            : (launch_absmax<float>(r, (int)H, N * d, w.stats, kStatWords, S_MAXR, s) &&
               launch_kmeans_stage_begin<float, 64>(a, s) && launch_assign<float, 64>(a, S_B0, s));
  else
    ok = bf ? (launch_absmax<uint16_t>(r, (int)H, N * d, w.stats, kStatWords, S_MAXR, s) &&
               launch_kmeans_stage_begin<uint16_t, 128>(a, s) && launch_assign<uint16_t, 128>(a, S_B0, s))
            : (launch_absmax<float>(r, (int)H, N * d, w.stats, kStatWords, S_MAXR, s) &&
               launch_kmeans_stage_begin<float, 128>(a, s) && launch_assign<float, 128>(a, S_B0, s));
  return ok ? QVG_OK : hip_fail("kmeans_assign");
}

size_t qvg_update_workspace_size(int64_t H, int64_t N, int64_t d, int32_t C) {
  if (check_dims(H, N, d, QVG_F32) != QVG_OK || C < 1 || C > kMaxC) return 0;
  size_t o = 0;
  o = up(o + (size_t)(H * kStatWords * 4));  // stats
  o = up(o + kCounterWords * 4);             // counters
  o = up(o + (size_t)(H * N * 4));           // sorted
  o = up(o + (size_t)(H * (C + 1) * 4));     // offs
  o = up(o + (size_t)(H * ((N + kSortChunk - 1) / kSortChunk) * kMaxC * 4));  // hist
  o = up(o + (size_t)(H * (C + 1) * 4));                                        // cofs
  o = up(o + (size_t)(H * max_chunks((int)N, C) * 4));                           // chunk_j
  o = up(o + (size_t)(H * max_chunks((int)N, C) * d * 8));                       // part
  o = up(o + (size_t)(H * max_chunks((int)N, C) * d * 4));                       // pflag
  return o;
}

qvg_status qvg_kmeans_update(const void *r, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                             const uint8_t *assign, int32_t C, float *centroids, void *ws,
                             size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  qvg_status st = check_dims(H, N, d, dtype);
  if (st != QVG_OK) return st;
  if (C < 1 || C > kMaxC) return fail(QVG_ERR_UNSUPPORTED, "C=%d must be in [1, 256]", C);
  if (!r || !assign || !centroids) return fail(QVG_ERR_INVALID_ARG, "NULL pointer argument");
  const size_t need = qvg_update_workspace_size(H, N, d, C);
  if (!ws || ws_bytes < need) return fail(QVG_ERR_WORKSPACE, "workspace smaller than %zu bytes", need);
  char *b = (char *)ws;
  Ws w{};
  size_t o = 0;
  w.stats = (uint32_t *)(b + o); o = up(o + (size_t)(H * kStatWords * 4));
  w.counters = (uint32_t *)(b + o); o = up(o + kCounterWords * 4);
  w.sorted = (int32_t *)(b + o); o = up(o + (size_t)(H * N * 4));
  w.offs = (int32_t *)(b + o); o = up(o + (size_t)(H * (C + 1) * 4));
  w.hist = (uint32_t *)(b + o); o = up(o + (size_t)(H * ((N + kSortChunk - 1) / kSortChunk) * kMaxC * 4));
  w.cofs = (int32_t *)(b + o); o = up(o + (size_t)(H * (C + 1) * 4));
  w.chunk_j = (int32_t *)(b + o); o = up(o + (size_t)(H * max_chunks((int)N, C) * 4));
  w.part = (double *)(b + o); o = up(o + (size_t)(H * max_chunks((int)N, C) * d * 8));
  w.pflag = (uint32_t *)(b + o);
  w.cent = centroids;
  KmArgs a;
  a.H = (int)H; a.N = (int)N; a.C = C; a.Cp = C; a.NT = 0;
  a.x = r; a.rec_pi = nullptr; a.rec_cent = nullptr; a.Ts = 1; a.nsub = 0;
  a.idx = nullptr; a.idx_hstride = 0; a.init = nullptr; a.init_hstride = 0;
  a.assign = (uint8_t *)assign; a.assign_hstride = N; a.ws = w; a.ws_stats = w.stats;
  a.stat_stride = kStatWords; a.kappa = 0.0f;
  hipStream_t s = (hipStream_t)stream;
  // cleared stats: the sums' spans are tracked per chunk (S_SPAN unset)
  if (!launch_fill_u32(w.stats, H * kStatWords, s)) return hip_fail("fill");
  const bool bf = dtype == QVG_BF16;
  bool ok;
  if (d == 64)
    ok = bf ? launch_update<uint16_t, float, 64>(a, S_B0, false, nullptr, 0, nullptr, 0, -1, -1, s)
            : launch_update<float, float, 64>(a, S_B0, false, nullptr, 0, nullptr, 0, -1, -1, s);
  else
    ok = bf ? launch_update<uint16_t, float, 128>(a, S_B0, false, nullptr, 0, nullptr, 0, -1, -1, s)
            : launch_update<float, float, 128>(a, S_B0, false, nullptr, 0, nullptr, 0, -1, -1, s);
  return ok ? QVG_OK : hip_fail("kmeans_update");
}

qvg_status qvg_sas_subtract(const void *r, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                            const uint8_t *assign, const void *chat, qvg_dtype cdtype, int32_t C,
                            float *r_out, void *stream) {
  g_err[0] = 0;
  qvg_status st = check_dims(H, N, d, dtype);
  if (st != QVG_OK) return st;
  if (cdtype != QVG_F32 && cdtype != QVG_BF16) return fail(QVG_ERR_INVALID_ARG, "unknown centroid dtype");
  if (C < 1 || C > kMaxC) return fail(QVG_ERR_UNSUPPORTED, "C=%d must be in [1, 256]", C);
  if (!r || !assign || !chat || !r_out) return fail(QVG_ERR_INVALID_ARG, "NULL pointer argument");
  if (!launch_subtract(r, dtype == QVG_BF16, (int)H, (int)N, (int)d, C, assign, N, chat,
                       cdtype == QVG_BF16, (int64_t)C * d, r_out, nullptr, 0, 0, (hipStream_t)stream))
    return hip_fail("sas_subtract");
  return QVG_OK;
}

qvg_status qvg_group_quant_pack(const void *r, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                                int32_t bits, int32_t group, uint8_t *codes, uint8_t *scales,
                                void *stream) {
  g_err[0] = 0;
  qvg_status st = check_dims(H, N, d, dtype);
  if (st != QVG_OK) return st;
  st = check_quant(d, bits, group);
  if (st != QVG_OK) return st;
  if (!r || !codes || !scales) return fail(QVG_ERR_INVALID_ARG, "NULL pointer argument");
  if (!launch_quant(r, dtype == QVG_BF16, (int)H, (int)N, (int)d, 1, nullptr, nullptr, 1, 0,
                    bits, group, codes, scales, (hipStream_t)stream))
    return hip_fail("group_quant_pack");
  return QVG_OK;
}

}  // extern "C"
