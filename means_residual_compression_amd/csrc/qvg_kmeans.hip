// k-means kernels of Semantic-Aware Smoothing for gfx950.
//
// note.zhuruihan.top "Semantic-Aware Smoothing" step 1 (k-means over tokens
// along the sequence axis) and step 2 (centroid = group mean);
// paper.rainbus.top method paragraph, SAS (a)-(b).
//
// Assignment: the distance ranking argmin_j ||r - c_j||^2 equals
// argmax_j (r.c_j - ||c_j||^2 / 2).  The dot products run on MFMA
// (v_mfma_f32_32x32x16_f16) over fp16 copies of r and c scaled by a per-head
// power of two; the accumulator starts at -||c_j||^2/2.  Each key carries its
// centroid index in the low 8 mantissa bits, so top-3 tracking is one max and
// two med3 per value.  A rigorous per-token error bound eps then decides:
//   key1 - key2 > 2 eps  -> the top-1 is the exact argmin;
//   key1 - key3 > 2 eps  -> the exact argmin is one of the top-2: both are
//                           re-checked with fp64 distances in channel order;
//   otherwise            -> exact fp64 scan over all centroids.
// The fp64 distances are computed exactly as a plain channel-order sum, so the
// result is the exact argmin with ties to the smallest index.
//
// Update: tokens are grouped by cluster with a stable counting sort (one
// workgroup per head), then one wave per cluster sums its members' rows in
// token order in fp64 and divides: the mean is the same fp64 token-order sum
// as a sequential loop.
#include "qvg_common.h"
#include "qvg_internal.h"

namespace qvg {

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ void atomic_max_pos(uint32_t *p, float v) {
  atomicMax(p, __float_as_uint(v));
}

template <typename Tin>
__device__ __forceinline__ float head_scale(const uint32_t *st) {
  return ldexpf(1.0f, -scale_exp(fmaxf(stat_f(st, S_MAXR), stat_f(st, S_MAXC))));
}

// ------------------------------------------------------------- abs max
// stats[h][slot] = max |x| over x[h] ([N*d] elements).
template <typename Tin>
__global__ void k_absmax(const Tin *__restrict__ x, int64_t per_head, uint32_t *stats,
                         int stat_stride, int slot) {
  const int h = blockIdx.y;
  const Tin *xh = x + (int64_t)h * per_head;
  float m = 0.0f;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < per_head;
       i += (int64_t)gridDim.x * blockDim.x * 8) {
    float v[8];
    load8(xh, i, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) atomic_max_pos(stats + (int64_t)h * stat_stride + slot, m);
}

// --------------------------------------------------------------- init
// Wave per (head, centroid): cent[h][j] = R[h][idx[h][j]] (gather) or
// init[h][j] (copy); stats max |c| into S_MAXC.  Padded centroids j >= C
// are zeroed.
template <typename Tin, int D>
__global__ void k_init(const Tin *__restrict__ r, int N, const int32_t *__restrict__ idx,
                       int64_t idx_hstride, const float *__restrict__ init,
                       int64_t init_hstride, int C, int Cp, float *__restrict__ cent,
                       uint32_t *stats, int stat_stride) {
  const int h = blockIdx.y;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= Cp) return;
  float *dst = cent + ((int64_t)h * Cp + j) * D;
  float m = 0.0f;
  for (int k = lane; k < D; k += 64) {
    float v = 0.0f;
    if (j < C) {
      if (idx) {
        const int64_t row = idx[(int64_t)h * idx_hstride + j];
        v = Elem<Tin>::get(r, ((int64_t)h * N + row) * D + k);
      } else {
        v = init[(int64_t)h * init_hstride + (int64_t)j * D + k];
      }
    }
    dst[k] = v;
    m = fmaxf(m, fabsf(v));
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) atomic_max_pos(stats + (int64_t)h * stat_stride + S_MAXC, m);
}

// ------------------------------------------------------------ prepare
// Thread per token: fp16 fragments of r * 2^-e for the MFMA B operand and the
// token's bounds (||r~||, ||r*2^-e - r~||), both rounded up.
// Fragment layout: [h][tile][kc][lane][8]; lane l holds token tile*32 + l%32
// and channels kc*16 + 8*(l/32) + 0..7.
template <typename Tin, int D>
__global__ void k_prepare(const Tin *__restrict__ r, int N, int NT, const uint32_t *stats,
                          int stat_stride, half8 *__restrict__ rt, float2 *__restrict__ tb) {
  constexpr int KC = D / 16;
  const int h = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= NT * kTile) return;
  const float sc = head_scale<Tin>(stats + (int64_t)h * stat_stride);
  const int tile = i / kTile, col = i % kTile;
  half8 *frag = rt + ((int64_t)h * NT + tile) * KC * 64;
  float n2 = 0.0f, e2 = 0.0f;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float v[8];
      if (i < N) {
        load8(r, ((int64_t)h * N + i) * D + kc * 16 + hf * 8, v);
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) v[m] = 0.0f;
      }
      half8 o;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float s = v[m] * sc;
        const _Float16 q = (_Float16)s;
        const float b = (float)q;
        o[m] = q;
        n2 += b * b;
        e2 += (s - b) * (s - b);
      }
      frag[kc * 64 + col + 32 * hf] = o;
    }
  }
  // sequential fp32 sums of D squares: relative error below 2^-12; the
  // 1e-30 absolute term covers values that underflowed when scaled
  const float up = 1.0f + 0x1p-12f;
  tb[(int64_t)h * NT * kTile + i] =
      make_float2(sqrtf(n2 * up) * (1.0f + 0x1p-20f), sqrtf(e2 * up) * (1.0f + 0x1p-20f) + 1e-30f);
}

// -------------------------------------------------------------- tables
// Given centroid j's values (lane holds channels k = lane*D/64 + 0..), write
// its fp16 fragment, its accumulator init -||c*sc||^2/2 and the per-head
// bounds.  Called by one full wave.
template <int D>
__device__ __forceinline__ void emit_tables(int h, int j, int Cp, const float *cv, float sc,
                                            half8 *__restrict__ ctab, float *__restrict__ cinit,
                                            uint32_t *bounds) {
  constexpr int KC = D / 16, PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int CB = Cp / kTile;
  double n2 = 0.0;
  float e2 = 0.0f, t2 = 0.0f;
  _Float16 q[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const float s = cv[m] * sc;
    q[m] = (_Float16)s;
    const float b = (float)q[m];
    n2 += (double)s * (double)s;
    e2 += (s - b) * (s - b);
    t2 += b * b;
  }
  // fragment position of channel k: kc = k/16, half = (k%16)/8, elem = k%8;
  // A operand lane = (j%32) + 32*half
  const int k0 = lane * PER;
  const int kc = k0 / 16, hf = (k0 % 16) / 8, el = k0 % 8;
  _Float16 *dst = reinterpret_cast<_Float16 *>(
      ctab + (((int64_t)h * CB + j / kTile) * KC + kc) * 64 + (j % kTile) + 32 * hf);
#pragma unroll
  for (int m = 0; m < PER; ++m) dst[el + m] = q[m];
  for (int o = 32; o > 0; o >>= 1) {
    n2 += __shfl_xor(n2, o);
    e2 += __shfl_xor(e2, o);
    t2 += __shfl_xor(t2, o);
  }
  if (lane == 0) {
    // accumulator init for row j: rows of a 32x32 output tile map to
    // (half, a) with row = 8*(a/4) + 4*half + a%4
    const int rr = j % kTile, hf2 = (rr / 4) % 2, a = 4 * (rr / 8) + rr % 4;
    cinit[(((int64_t)h * CB + j / kTile) * 2 + hf2) * 16 + a] = (float)(-0.5 * n2);
    const float up = 1.0f + 0x1p-12f;
    atomic_max_pos(bounds + 0, (float)sqrt(n2) * (1.0f + 0x1p-20f));
    atomic_max_pos(bounds + 1, sqrtf(e2 * up) * (1.0f + 0x1p-20f) + 1e-30f);
    atomic_max_pos(bounds + 2, sqrtf(t2 * up) * (1.0f + 0x1p-20f));
    atomic_max_pos(bounds + 3, (float)n2 * (1.0f + 0x1p-20f));
  }
}

// Padded centroid rows (j >= C): zero fragment and an init of -3e38 so their
// keys never enter the top-2.
template <int D>
__device__ __forceinline__ void emit_pad(int h, int j, int Cp, half8 *__restrict__ ctab,
                                         float *__restrict__ cinit) {
  constexpr int KC = D / 16, PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int CB = Cp / kTile;
  const int k0 = lane * PER;
  const int kc = k0 / 16, hf = (k0 % 16) / 8, el = k0 % 8;
  _Float16 *dst = reinterpret_cast<_Float16 *>(
      ctab + (((int64_t)h * CB + j / kTile) * KC + kc) * 64 + (j % kTile) + 32 * hf);
#pragma unroll
  for (int m = 0; m < PER; ++m) dst[el + m] = (_Float16)0.0f;
  if (lane == 0) {
    const int rr = j % kTile, hf2 = (rr / 4) % 2, a = 4 * (rr / 8) + rr % 4;
    cinit[(((int64_t)h * CB + j / kTile) * 2 + hf2) * 16 + a] = -3.0e38f;
  }
}

// Wave per (head, centroid): tables for the stage's initial centroids.
template <int D>
__global__ void k_tables(const float *__restrict__ cent, int C, int Cp, const uint32_t *stats,
                         uint32_t *stats_w, int stat_stride, int bslot, half8 *__restrict__ ctab,
                         float *__restrict__ cinit) {
  constexpr int PER = D / 64;
  const int h = blockIdx.y;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= Cp) return;
  if (j >= C) {
    emit_pad<D>(h, j, Cp, ctab, cinit);
    return;
  }
  const uint32_t *st = stats + (int64_t)h * stat_stride;
  const float sc = ldexpf(1.0f, -scale_exp(fmaxf(stat_f(st, S_MAXR), stat_f(st, S_MAXC))));
  float cv[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) cv[m] = cent[((int64_t)h * Cp + j) * D + lane * PER + m];
  emit_tables<D>(h, j, Cp, cv, sc, ctab, cinit, stats_w + (int64_t)h * stat_stride + bslot);
}

// ------------------------------------------------------------- assign
// Workgroup: 4 waves, one head, `tiles_per_wg` consecutive 32-token tiles.
// Each wave handles two tiles at a time against every 32-centroid block held
// in LDS (fp16 fragments + accumulator inits).
template <int D>
__global__ __launch_bounds__(256, 2) void k_assign(
    const half8 *__restrict__ rt, const float2 *__restrict__ tb, const half8 *__restrict__ ctab,
    const float *__restrict__ cinit, const uint32_t *__restrict__ stats, int stat_stride,
    int bslot, int N, int NT, int CB, int tiles_per_wg, uint8_t *__restrict__ assign,
    int64_t assign_hstride, int4 *__restrict__ recheck, int2 *__restrict__ fallback,
    uint32_t *__restrict__ counters, float kappa) {
  constexpr int KC = D / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  half8 *ctab_s = reinterpret_cast<half8 *>(smem);
  float *cinit_s = reinterpret_cast<float *>(smem + (size_t)CB * KC * 64 * sizeof(half8));

  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  {
    const half8 *src = ctab + (int64_t)h * CB * KC * 64;
    for (int q = threadIdx.x; q < CB * KC * 64; q += 256) ctab_s[q] = src[q];
    const float *ci = cinit + (int64_t)h * CB * 32;
    for (int q = threadIdx.x; q < CB * 32; q += 256) cinit_s[q] = ci[q];
  }
  __syncthreads();

  const uint32_t *st = stats + (int64_t)h * stat_stride + bslot;
  const float cmax = __uint_as_float(st[0]), ecmax = __uint_as_float(st[1]);
  const float ctmax = __uint_as_float(st[2]), nmax = __uint_as_float(st[3]);
  const int half = lane >> 5;
  const uint32_t halfbits = (uint32_t)half << 2;

  const int tile_lo = blockIdx.x * tiles_per_wg;
  const int tile_hi = min(NT, tile_lo + tiles_per_wg);
  for (int t0 = tile_lo + 2 * wave; t0 < tile_hi; t0 += 8) {
    const bool has1 = t0 + 1 < tile_hi;
    half8 b0[KC], b1[KC];
    const half8 *f0 = rt + ((int64_t)h * NT + t0) * KC * 64 + lane;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      b0[kc] = f0[kc * 64];
      b1[kc] = has1 ? f0[(KC + kc) * 64] : b0[kc];
    }
    float a1 = -3.4e38f, a2 = -3.4e38f, a3 = -3.4e38f;
    float c1 = -3.4e38f, c2 = -3.4e38f, c3 = -3.4e38f;
    for (int cb = 0; cb < CB; ++cb) {
      const floatx4 *cp = reinterpret_cast<const floatx4 *>(cinit_s + cb * 32 + half * 16);
      const floatx4 i0 = cp[0], i1 = cp[1], i2 = cp[2], i3 = cp[3];
      floatx16 init;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        init[q] = i0[q];
        init[4 + q] = i1[q];
        init[8 + q] = i2[q];
        init[12 + q] = i3[q];
      }
      floatx16 acc0 = init, acc1 = init;
      const half8 *ap = ctab_s + cb * KC * 64 + lane;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const half8 a = ap[kc * 64];
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b0[kc], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b1[kc], acc1, 0, 0, 0);
      }
      const uint32_t base = (uint32_t)cb << 5;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const uint32_t enc = base | (uint32_t)(8 * (a / 4) + (a % 4));
        const float x0 = __uint_as_float((__float_as_uint(acc0[a]) & 0xFFFFFF00u) | enc);
        const float x1 = __uint_as_float((__float_as_uint(acc1[a]) & 0xFFFFFF00u) | enc);
        a3 = __builtin_amdgcn_fmed3f(a2, a3, x0);
        a2 = __builtin_amdgcn_fmed3f(a1, a2, x0);
        a1 = fmaxf(a1, x0);
        c3 = __builtin_amdgcn_fmed3f(c2, c3, x1);
        c2 = __builtin_amdgcn_fmed3f(c1, c2, x1);
        c1 = fmaxf(c1, x1);
      }
    }
    // lanes >= 32 saw the rows with bit 2 set
    a1 = __uint_as_float(__float_as_uint(a1) | halfbits);
    a2 = __uint_as_float(__float_as_uint(a2) | halfbits);
    a3 = __uint_as_float(__float_as_uint(a3) | halfbits);
    c1 = __uint_as_float(__float_as_uint(c1) | halfbits);
    c2 = __uint_as_float(__float_as_uint(c2) | halfbits);
    c3 = __uint_as_float(__float_as_uint(c3) | halfbits);
    // merge with the other half (same token column); lanes < 32 keep tile t0,
    // lanes >= 32 keep tile t0+1
    float m1 = half ? c1 : a1, m2 = half ? c2 : a2, m3 = half ? c3 : a3;
    const float s1 = half ? a1 : c1, s2 = half ? a2 : c2, s3 = half ? a3 : c3;
    const float o1 = __shfl_xor(s1, 32), o2 = __shfl_xor(s2, 32), o3 = __shfl_xor(s3, 32);
    const float oo[3] = {o1, o2, o3};
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      m3 = __builtin_amdgcn_fmed3f(m2, m3, oo[q]);
      m2 = __builtin_amdgcn_fmed3f(m1, m2, oo[q]);
      m1 = fmaxf(m1, oo[q]);
    }
    const int tile = t0 + half;
    const int tok = tile * kTile + (lane & 31);
    if (tile < tile_hi && tok < N) {
      const float2 b = tb[(int64_t)h * NT * kTile + tok];
      const float rn = b.x, er = b.y;
      const float big = fmaf(rn, ctmax, 0.5f * nmax);
      const float rc = rn + ctmax + er + ecmax;
      float eps = er * cmax + rn * ecmax + kappa * big + 0x1p-40f * rc * rc;
      eps = eps * (1.0f + 0x1p-20f) + 1e-37f;
      const int j1 = (int)(__float_as_uint(m1) & 0xFFu);
      const int j2 = (int)(__float_as_uint(m2) & 0xFFu);
      const float g12 = (m1 - m2) * (1.0f - 0x1p-20f);
      const float g13 = (m1 - m3) * (1.0f - 0x1p-20f);
      uint8_t *dst = assign + (int64_t)h * assign_hstride + tok;
      if (g12 > 2.0f * eps) {
        *dst = (uint8_t)j1;
      } else if (g13 > 2.0f * eps) {
        const uint32_t pos = atomicAdd(counters + 0, 1u);
        recheck[pos] = make_int4(h, tok, j1, j2);
      } else {
        const uint32_t pos = atomicAdd(counters + 1, 1u);
        fallback[pos] = make_int2(h, tok);
      }
    }
  }
}

// ------------------------------------------------------------ resolve
// Exact fp64 squared distance, channel order, no fused multiply-add.
template <typename Tin, int D>
__device__ __forceinline__ double exact_dist(const Tin *__restrict__ row,
                                             const float *__restrict__ c) {
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < D; k += 8) {
    float v[8], w[8];
    load8(row, k, v);
    load8(c, k, w);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const double df = (double)v[m] - (double)w[m];
      acc = __dadd_rn(acc, __dmul_rn(df, df));
    }
  }
  return acc;
}

// Thread per re-check entry: the nearer of the two candidates.
template <typename Tin, int D>
__global__ void k_recheck(const Tin *__restrict__ r, int N, const float *__restrict__ cent,
                          int Cp, const int4 *__restrict__ list,
                          const uint32_t *__restrict__ counters, uint8_t *__restrict__ assign,
                          int64_t assign_hstride) {
  const uint32_t n = counters[0];
  for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) {
    const int4 q = list[e];
    const Tin *row = r + ((int64_t)q.x * N + q.y) * D;
    const float *cb = cent + (int64_t)q.x * Cp * D;
    const double d1 = exact_dist<Tin, D>(row, cb + (int64_t)q.z * D);
    const double d2 = exact_dist<Tin, D>(row, cb + (int64_t)q.w * D);
    const int j = (d2 < d1 || (d2 == d1 && q.w < q.z)) ? q.w : q.z;
    assign[(int64_t)q.x * assign_hstride + q.y] = (uint8_t)j;
  }
}

// Wave per fallback entry: exact scan over all C centroids.
template <typename Tin, int D>
__global__ void k_fallback(const Tin *__restrict__ r, int N, const float *__restrict__ cent,
                           int C, int Cp, const int2 *__restrict__ list,
                           const uint32_t *__restrict__ counters, uint8_t *__restrict__ assign,
                           int64_t assign_hstride) {
  const uint32_t n = counters[1];
  const int lane = threadIdx.x & 63;
  const uint32_t nw = gridDim.x * (blockDim.x >> 6);
  for (uint32_t e = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); e < n; e += nw) {
    const int2 q = list[e];
    const Tin *row = r + ((int64_t)q.x * N + q.y) * D;
    const float *cb = cent + (int64_t)q.x * Cp * D;
    double best = 0.0;
    int bj = -1;
    for (int j = lane; j < C; j += 64) {
      const double dj = exact_dist<Tin, D>(row, cb + (int64_t)j * D);
      if (bj < 0 || dj < best) {
        best = dj;
        bj = j;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oj = __shfl_xor(bj, o);
      if (oj >= 0 && (bj < 0 || ob < best || (ob == best && oj < bj))) {
        best = ob;
        bj = oj;
      }
    }
    if (lane == 0) assign[(int64_t)q.x * assign_hstride + q.y] = (uint8_t)bj;
  }
}

// --------------------------------------------------------------- sort
// One workgroup (16 waves) per head: stable counting sort of token ids by
// cluster.  Each wave owns a contiguous token range; ranks inside a 64-token
// group come from ballots, so token order is kept within every cluster.
// Also clears the next bound slot and (head 0) the candidate-list counters.
__global__ __launch_bounds__(1024) void k_sort(const uint8_t *__restrict__ assign,
                                               int64_t assign_hstride, int N, int C, int Cp,
                                               int32_t *__restrict__ sorted,
                                               int32_t *__restrict__ offs, uint32_t *stats,
                                               int stat_stride, int clear_slot,
                                               uint32_t *counters) {
  __shared__ uint32_t hist[16][kMaxC];
  __shared__ uint32_t tot[kMaxC];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t *a = assign + (int64_t)h * assign_hstride;
  const int chunk = (((N + 15) / 16) + 63) & ~63;
  const int lo = min(N, wave * chunk), hi = min(N, lo + chunk);
  for (int q = threadIdx.x; q < 16 * kMaxC; q += 1024) (&hist[0][0])[q] = 0;
  if (threadIdx.x < 4) stats[(int64_t)h * stat_stride + clear_slot + threadIdx.x] = 0;
  if (h == 0 && threadIdx.x < 2) counters[threadIdx.x] = 0;
  __syncthreads();
  for (int i = lo + lane; i < hi; i += 64) atomicAdd(&hist[wave][a[i]], 1u);
  __syncthreads();
  if (threadIdx.x < kMaxC) {
    uint32_t s = 0;
    for (int w = 0; w < 16; ++w) s += hist[w][threadIdx.x];
    tot[threadIdx.x] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // exclusive scan over all 256 byte values, so that assignment bytes >= C
    // (possible only for corrupt input) still get in-range slots after the
    // real clusters' segments
    uint32_t run = 0;
    for (int j = 0; j < kMaxC; ++j) {
      const uint32_t t = tot[j];
      tot[j] = run;
      if (j <= Cp) offs[(int64_t)h * (Cp + 1) + j] = (int32_t)run;
      run += t;
    }
    if (Cp == kMaxC) offs[(int64_t)h * (Cp + 1) + Cp] = (int32_t)run;
  }
  __syncthreads();
  if (threadIdx.x < kMaxC) {
    uint32_t run = tot[threadIdx.x];
    for (int w = 0; w < 16; ++w) {
      const uint32_t c = hist[w][threadIdx.x];
      hist[w][threadIdx.x] = run;
      run += c;
    }
  }
  __syncthreads();
  int32_t *out = sorted + (int64_t)h * N;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int g = lo; g < hi; g += 64) {
    const int i = g + lane;
    const bool valid = i < hi;
    const uint32_t j = valid ? a[i] : 0u;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bb = __ballot(valid && ((j >> b) & 1u));
      m &= ((j >> b) & 1u) ? bb : ~bb;
    }
    if (valid) {
      const uint32_t rank = __popcll(m & lt);
      out[hist[wave][j] + rank] = i;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (m >> lane) == 1ull) hist[wave][j] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------- accumulate
// Wave per (head, cluster): c_j = fp32(sum of members in token order / n_j)
// with fp64 sums; an empty cluster keeps its centroid.  Then emits the
// centroid's tables for the next assign.  On the stage's last iteration it
// also stores the record centroid (rounded to the record dtype) and the fp32
// cache entry.
template <typename Tin, typename Tc, int D>
__global__ void k_accumulate(const Tin *__restrict__ r, int N, const int32_t *__restrict__ sorted,
                             const int32_t *__restrict__ offs, int C, int Cp,
                             float *__restrict__ cent, const uint32_t *stats, uint32_t *stats_w,
                             int stat_stride, int bslot, half8 *__restrict__ ctab,
                             float *__restrict__ cinit, Tc *__restrict__ rec_c,
                             int64_t rec_hstride, float *__restrict__ cache,
                             int64_t cache_hstride) {
  constexpr int PER = D / 64;
  const int h = blockIdx.y;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= Cp) return;
  if (j >= C) {
    if (ctab) emit_pad<D>(h, j, Cp, ctab, cinit);
    return;
  }
  const int32_t lo = offs[(int64_t)h * (Cp + 1) + j], hi = offs[(int64_t)h * (Cp + 1) + j + 1];
  const int32_t *mem = sorted + (int64_t)h * N;
  const Tin *rh = r + (int64_t)h * N * D + lane * PER;
  double s[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) s[m] = 0.0;
  int32_t p = lo;
  for (; p + 8 <= hi; p += 8) {
    float v[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t row = (int64_t)mem[p + u] * D;
#pragma unroll
      for (int m = 0; m < PER; ++m) v[u][m] = Elem<Tin>::get(rh, row + m);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int m = 0; m < PER; ++m) s[m] = __dadd_rn(s[m], (double)v[u][m]);
  }
  for (; p < hi; ++p) {
    const int64_t row = (int64_t)mem[p] * D;
#pragma unroll
    for (int m = 0; m < PER; ++m) s[m] = __dadd_rn(s[m], (double)Elem<Tin>::get(rh, row + m));
  }
  float *cj = cent + ((int64_t)h * Cp + j) * D + lane * PER;
  float cv[PER];
  const int32_t n = hi - lo;
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    cv[m] = n > 0 ? (float)(s[m] / (double)n) : cj[m];
    cj[m] = cv[m];
  }
  if (ctab) {
    const uint32_t *st = stats + (int64_t)h * stat_stride;
    const float sc = ldexpf(1.0f, -scale_exp(fmaxf(stat_f(st, S_MAXR), stat_f(st, S_MAXC))));
    emit_tables<D>(h, j, Cp, cv, sc, ctab, cinit, stats_w + (int64_t)h * stat_stride + bslot);
  }
  if (rec_c) {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      Elem<Tc>::put(rec_c + (int64_t)h * rec_hstride, (int64_t)j * D + lane * PER + m, cv[m]);
      if (cache) cache[(int64_t)h * cache_hstride + (int64_t)j * D + lane * PER + m] = cv[m];
    }
  }
}

// ============================================================ launchers
namespace {
template <int D> int kc_of() { return D / 16; }
}

#define QVG_CHECK_LAUNCH() \
  do { if (hipGetLastError() != hipSuccess) return false; } while (0)

template <typename Tin>
bool launch_absmax(const void *x, int H, int64_t per_head, uint32_t *stats, int stat_stride,
                   int slot, hipStream_t s) {
  int64_t blocks = (per_head / 8 + 255) / 256;
  dim3 grid((unsigned)std::min<int64_t>(blocks, 1024), H);
  { TimerScope ts_("absmax", s);
  hipLaunchKernelGGL(k_absmax<Tin>, grid, dim3(256), 0, s, (const Tin *)x, per_head, stats,
                     stat_stride, slot); }
  QVG_CHECK_LAUNCH();
  return true;
}

template <typename Tin, int D>
bool launch_kmeans_stage_begin(const KmArgs &a, hipStream_t s) {
  dim3 gc((a.Cp + 3) / 4, a.H);
  { TimerScope ts_("kmeans_init", s);
  hipLaunchKernelGGL((k_init<Tin, D>), gc, dim3(256), 0, s, (const Tin *)a.r, a.N, a.idx,
                     a.idx_hstride, a.init, a.init_hstride, a.C, a.Cp, a.ws.cent, a.ws_stats,
                     a.stat_stride); }
  QVG_CHECK_LAUNCH();
  dim3 gp((a.NT * kTile + 255) / 256, a.H);
  { TimerScope ts_("kmeans_prepare", s);
  hipLaunchKernelGGL((k_prepare<Tin, D>), gp, dim3(256), 0, s, (const Tin *)a.r, a.N, a.NT,
                     a.ws_stats, a.stat_stride, a.ws.rt, a.ws.tb); }
  QVG_CHECK_LAUNCH();
  { TimerScope ts_("kmeans_tables", s);
  hipLaunchKernelGGL((k_tables<D>), gc, dim3(256), 0, s, a.ws.cent, a.C, a.Cp, a.ws_stats,
                     a.ws_stats, a.stat_stride, (int)S_B0, a.ws.ctab, a.ws.cinit); }
  QVG_CHECK_LAUNCH();
  return true;
}

template <typename Tin, int D>
bool launch_assign(const KmArgs &a, int bslot, hipStream_t s) {
  constexpr int KC = D / 16;
  const int CB = a.Cp / kTile;
  const size_t lds = (size_t)CB * KC * 64 * sizeof(half8) + (size_t)CB * 32 * sizeof(float);
  const int tiles_per_wg = 16;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void *)k_assign<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            96 * 1024) != hipSuccess)
      return false;
    attr_set = true;
  }
  dim3 grid((a.NT + tiles_per_wg - 1) / tiles_per_wg, a.H);
  { TimerScope ts_("kmeans_assign", s);
  hipLaunchKernelGGL((k_assign<D>), grid, dim3(256), lds, s, a.ws.rt, a.ws.tb, a.ws.ctab,
                     a.ws.cinit, a.ws_stats, a.stat_stride, bslot, a.N, a.NT, CB, tiles_per_wg,
                     a.assign, a.assign_hstride, a.ws.recheck, a.ws.fallback, a.ws.counters,
                     a.kappa); }
  QVG_CHECK_LAUNCH();
  { TimerScope ts_("kmeans_recheck", s);
  hipLaunchKernelGGL((k_recheck<Tin, D>), dim3(512), dim3(256), 0, s, (const Tin *)a.r, a.N,
                     a.ws.cent, a.Cp, a.ws.recheck, a.ws.counters, a.assign, a.assign_hstride); }
  QVG_CHECK_LAUNCH();
  { TimerScope ts_("kmeans_fallback", s);
  hipLaunchKernelGGL((k_fallback<Tin, D>), dim3(512), dim3(256), 0, s, (const Tin *)a.r, a.N,
                     a.ws.cent, a.C, a.Cp, a.ws.fallback, a.ws.counters, a.assign,
                     a.assign_hstride); }
  QVG_CHECK_LAUNCH();
  return true;
}

template <typename Tin, typename Tc, int D>
bool launch_update(const KmArgs &a, int next_bslot, bool tables, Tc *rec_c, int64_t rec_hstride,
                   float *cache, int64_t cache_hstride, hipStream_t s) {
  { TimerScope ts_("kmeans_sort", s);
  hipLaunchKernelGGL(k_sort, dim3(a.H), dim3(1024), 0, s, a.assign, a.assign_hstride, a.N, a.C,
                     a.Cp, a.ws.sorted, a.ws.offs, a.ws_stats, a.stat_stride, next_bslot,
                     a.ws.counters); }
  QVG_CHECK_LAUNCH();
  dim3 gc((a.Cp + 3) / 4, a.H);
  { TimerScope ts_("kmeans_accumulate", s);
  hipLaunchKernelGGL((k_accumulate<Tin, Tc, D>), gc, dim3(256), 0, s, (const Tin *)a.r, a.N,
                     a.ws.sorted, a.ws.offs, a.C, a.Cp, a.ws.cent, a.ws_stats, a.ws_stats,
                     a.stat_stride, next_bslot, tables ? a.ws.ctab : nullptr, a.ws.cinit, rec_c,
                     rec_hstride, cache, cache_hstride); }
  QVG_CHECK_LAUNCH();
  return true;
}

#define QVG_INST(Tin, D)                                                                      \
  template bool launch_kmeans_stage_begin<Tin, D>(const KmArgs &, hipStream_t);               \
  template bool launch_assign<Tin, D>(const KmArgs &, int, hipStream_t);                      \
  template bool launch_update<Tin, float, D>(const KmArgs &, int, bool, float *, int64_t,     \
                                             float *, int64_t, hipStream_t);                  \
  template bool launch_update<Tin, uint16_t, D>(const KmArgs &, int, bool, uint16_t *,        \
                                                int64_t, float *, int64_t, hipStream_t);
QVG_INST(float, 64)
QVG_INST(float, 128)
QVG_INST(uint16_t, 64)
QVG_INST(uint16_t, 128)
template bool launch_absmax<float>(const void *, int, int64_t, uint32_t *, int, int, hipStream_t);
template bool launch_absmax<uint16_t>(const void *, int, int64_t, uint32_t *, int, int,
                                      hipStream_t);

}  // namespace qvg
