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
// Update: tokens are grouped by cluster with a stable counting sort, each
// cluster's members (token order) are summed in fp64 in chunks of 64 and the
// chunk sums added in chunk order.  Alongside, every chunk records per channel
// the largest exponent and a lower bound on the lowest set bit of its values;
// when those show that some partial sum of the cluster could round, the
// cluster is summed again in one sequential token-order pass.  Either way the
// sum equals the sequential fp64 sum of a plain loop.
//
// The first iteration of a stage also reduces those spans over each head.
// When they show that the cluster sums fit int64 in units of each channel's
// lowest bit (the usual case), the sums are kept as such integers, and later
// iterations of the stage only move the tokens whose assignment changed from
// their old cluster's sum to the new one (k_hist lists them, k_accum_delta adds
// them): integer sums do not depend on the order, and when every cluster's
// member count keeps its fp64 partial sums exact they are the sequential fp64
// sums.  k_scatter decides per head and iteration; heads that fail those
// conditions, or with more than a quarter of their tokens moved, take the full
// update.
#include "qvg_common.h"
#include "qvg_internal.h"

namespace qvg {

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ void atomic_max_pos(uint32_t *p, float v) {
  atomicMax(p, __float_as_uint(v));
}

// Workgroup copy global -> LDS with U loads in flight per thread.
template <int U, typename T>
__device__ __forceinline__ void block_copy(T *__restrict__ dst, const T *__restrict__ src, int n) {
  const int step = U * (int)blockDim.x;
  int base = 0;
  for (; base + step <= n; base += step) {  // full rounds: no per-load condition
    T tmp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) tmp[u] = src[base + u * (int)blockDim.x + (int)threadIdx.x];
#pragma unroll
    for (int u = 0; u < U; ++u) dst[base + u * (int)blockDim.x + (int)threadIdx.x] = tmp[u];
  }
  for (int q = base + (int)threadIdx.x; q < n; q += (int)blockDim.x) dst[q] = src[q];
}

// Max over a workgroup of up to 1024 threads (result valid in thread 0).
__device__ __forceinline__ float block_max(float m) {
  __shared__ float part[16];
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, part[w]);
  return m;
}

// A head whose stage spans are known to keep every cluster sum exact (S_SPAN
// == 1): it skips the per-chunk span tracking.
__device__ __forceinline__ bool head_sums_exact(const uint32_t *stats, int stat_stride, int h) {
  return (__builtin_amdgcn_readfirstlane(stats[(int64_t)h * stat_stride + S_SPAN]) & 3u) == 1u;
}
// This iteration updates the head incrementally (set by k_scatter).
__device__ __forceinline__ bool head_incremental(const uint32_t *stats, int stat_stride, int h) {
  return __builtin_amdgcn_readfirstlane(stats[(int64_t)h * stat_stride + S_INC]) == 1u;
}
__device__ __forceinline__ int ceil_log2(uint32_t n) {
  return n > 1 ? 32 - __builtin_clz(n - 1) : 0;
}
// The head's cluster sums fit int64 in units of each channel's lowest bit for
// any set of up to N members (|v| < 2^(span + 24) units each): sums of them
// are exact in any order.
__device__ __forceinline__ bool head_int_sums(const uint32_t *stats, int stat_stride, int h,
                                              int N) {
  const uint32_t *st = stats + (int64_t)h * stat_stride;
  const uint32_t chk = __builtin_amdgcn_readfirstlane(st[S_SPAN]);
  const int w = (int)__builtin_amdgcn_readfirstlane(st[S_SPANW]);
  return (chk & 1u) && w + 24 + ceil_log2((uint32_t)N) <= 62;
}
// A head that may be updated incrementally in this iteration: integer sums
// possible and exact after its last full update.
__device__ __forceinline__ bool head_inc_candidate(const uint32_t *stats, int stat_stride, int h,
                                                   int N) {
  return head_int_sums(stats, stat_stride, h, N) &&
         __builtin_amdgcn_readfirstlane(stats[(int64_t)h * stat_stride + S_ISUM]) == 1u;
}

// Sum over a workgroup of up to 1024 threads, returned to every thread.
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v) {
  __shared__ uint32_t part[16];
  __shared__ uint32_t total;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += part[w];
    total = t;
  }
  __syncthreads();
  return total;
}

// Max over a workgroup of up to 1024 threads, returned to every thread.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t part[16];
  __shared__ uint32_t best;
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = max(m, part[w]);
    best = m;
  }
  __syncthreads();
  return best;
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
  m = block_max(m);
  if (threadIdx.x == 0) atomic_max_pos(stats + (int64_t)h * stat_stride + slot, m);
}

// --------------------------------------------------------- stage bound
// Scale bound for stage t >= 1: R(t) = R(t-1) - C^[pi] with |C^| at most the
// larger of max|R(t-1)| and max|init centroids| (a centroid is a mean of rows
// or an untouched initial value) times bf16 rounding, so
// max|R(t)| <= (max|R(t-1)| + max(max|R(t-1)|, max|C0(t-1)|)) * (1 + 2^-7).
__global__ void k_stage_bound(uint32_t *stats, int stat_stride, int H) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  uint32_t *st = stats + (int64_t)h * stat_stride;
  const float r = __uint_as_float(st[S_MAXR]), c = __uint_as_float(st[S_MAXC]);
  st[kStatWords + S_MAXR] = __float_as_uint((r + fmaxf(r, c)) * (1.0f + 0x1p-7f));
}

// ------------------------------------------------------- seeded rows
// Cold-start rows of stage t (1-based) of head h: a partial Fisher-Yates
// shuffle of 0..N-1 driven by splitmix64 (Steele, Lea and Flood 2014; output
// j is the generator state seed_ht + (j+1)*0x9E3779B97F4A7C15 passed through
// the two published xor-shift-multiply rounds and a final xor-shift), with
// seed_ht = seed ^ (0x9E3779B97F4A7C15*(h+1)) ^ (0xD1B54A32D192ED03*t).  Step j
// swaps positions j and j + (z_j mod (N-j)); row j is the value then at
// position j.  One wave per (head, stage): the C offsets are computed in
// parallel (the generator is a counter), the swaps run in order on a sparse
// permutation: positions below C in a dense LDS array, positions from C on in
// a list of at most C (position, value) pairs searched by the whole wave.
__device__ __forceinline__ uint64_t splitmix_at(uint64_t s, uint64_t k) {
  uint64_t z = s + 0x9E3779B97F4A7C15ull * k;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(64) void k_sample(int N, int C, int T, uint64_t seed,
                                               int32_t *__restrict__ idx) {
  __shared__ uint32_t off[kMaxC];
  __shared__ int32_t front[kMaxC], bpos[kMaxC], bval[kMaxC];
  const int h = blockIdx.y, t = blockIdx.x + 1, lane = threadIdx.x;
  const uint64_t s0 = seed ^ (0x9E3779B97F4A7C15ull * (uint64_t)(h + 1)) ^
                      (0xD1B54A32D192ED03ull * (uint64_t)t);
  for (int j = lane; j < C; j += 64) {
    off[j] = (uint32_t)(splitmix_at(s0, (uint64_t)j + 1) % (uint64_t)(N - j));
    front[j] = j;
  }
  __syncthreads();
  int32_t *out = idx + ((int64_t)h * T + (t - 1)) * C;
  int nb = 0;  // entries of the list (wave-uniform)
  for (int j = 0; j < C; ++j) {
    const int k = j + (int)off[j];
    const int32_t vj = front[j];
    int32_t vk;
    if (k < C) {
      vk = front[k];
      __syncthreads();
      if (lane == 0) front[k] = vj;
    } else {
      int at = -1;
      for (int q = lane; q < nb; q += 64)
        if (bpos[q] == k) at = q;
      const uint64_t m = __ballot(at >= 0);
      const int pos = m ? __shfl(at, __builtin_ctzll(m)) : -1;
      if (pos >= 0) {
        vk = bval[pos];
        __syncthreads();
        if (lane == 0) bval[pos] = vj;
      } else {
        vk = k;
        __syncthreads();
        if (lane == 0) {
          bpos[nb] = k;
          bval[nb] = vj;
        }
        ++nb;
      }
    }
    if (lane == 0) {
      front[j] = vk;
      out[j] = vk;
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------- init
// Wave per (head, centroid): cent[h][j] = R[h][idx[h][j]] (gather) or
// init[h][j] (copy); stats max |c| into S_MAXC.  Padded centroids j >= C
// are zeroed.
template <typename Tin, int D>
__global__ void k_init(ResView<Tin> rv, const int32_t *__restrict__ idx,
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
        // rows outside [0, N) only arrive from unchecked device arrays: clamped
        const int64_t row = min(max((int64_t)idx[(int64_t)h * idx_hstride + j], (int64_t)0),
                                (int64_t)rv.N - 1);
        v = rv.get(h, row, k);
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
// fp16 fragments of r * 2^-e for the MFMA B operand and each token's bounds
// (||r~||, ||r*2^-e - r~||), rounded up.  D/8 lanes per token, each 8
// channels, so a token row is read contiguously.
// Fragment layout: [h][tile][kc][lane][8]; lane l holds token tile*32 + l%32
// and channels kc*16 + 8*(l/32) + 0..7.
template <typename Tin, int D, int NSUB>
__global__ void k_prepare(ResView<Tin> rv, int NT, const uint32_t *stats, int stat_stride,
                          half8 *__restrict__ rt, float2 *__restrict__ tb) {
  const int N = rv.N;
  constexpr int KC = D / 16, LPT = D / 8;
  const int h = blockIdx.y;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = g < (int64_t)NT * kTile * LPT;
  const int i = live ? (int)(g / LPT) : 0;
  const int q = (int)(g % LPT);
  const float sc = head_scale<Tin>(stats + (int64_t)h * stat_stride);
  float v[8];
  if (live && i < N) {
    rv.template load8_n<NSUB>(h, i, q * 8, v);
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = 0.0f;
  }
  float n2 = 0.0f, e2 = 0.0f;
  half8 o;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float s = v[m] * sc;
    const _Float16 hq = (_Float16)s;
    const float b = (float)hq;
    o[m] = hq;
    n2 += b * b;
    e2 += (s - b) * (s - b);
  }
#pragma unroll
  for (int off = 1; off < LPT; off <<= 1) {
    n2 += __shfl_xor(n2, off);
    e2 += __shfl_xor(e2, off);
  }
  if (!live) return;
  const int tile = i / kTile, col = i % kTile, kc = q / 2, hf = q % 2;
  rt[((int64_t)h * NT + tile) * KC * 64 + kc * 64 + col + 32 * hf] = o;
  if (q == 0) {
    // fp32 sums of D squares in any order: relative error below 2^-12; the
    // 1e-30 absolute term covers values that underflowed when scaled
    const float up = 1.0f + 0x1p-12f;
    tb[(int64_t)h * NT * kTile + i] = make_float2(sqrtf(n2 * up) * (1.0f + 0x1p-20f),
                                                  sqrtf(e2 * up) * (1.0f + 0x1p-20f) + 1e-30f);
  }
}

// -------------------------------------------------------------- tables
// Given centroid j's values (lane holds channels k = lane*D/64 + 0..), write
// its fp16 fragment, its accumulator init -||c*sc||^2/2 and the per-head
// bounds.  Called by one full wave.
template <int D>
__device__ __forceinline__ void emit_tables(int h, int j, int Cp, const float *cv, float sc,
                                            half8 *__restrict__ ctab, float *__restrict__ cinit,
                                            float4 *__restrict__ cbnd, uint32_t *bounds) {
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
    const float4 bd = make_float4((float)sqrt(n2) * (1.0f + 0x1p-20f),
                                  sqrtf(e2 * up) * (1.0f + 0x1p-20f) + 1e-30f,
                                  sqrtf(t2 * up) * (1.0f + 0x1p-20f),
                                  (float)n2 * (1.0f + 0x1p-20f));
    cbnd[(int64_t)h * Cp + j] = bd;
  }
}

// Padded centroid rows (j >= C): zero fragment and an init of -3e38 so their
// keys never enter the top-2.
template <int D>
__device__ __forceinline__ void emit_pad(int h, int j, int Cp, half8 *__restrict__ ctab,
                                         float *__restrict__ cinit, float4 *__restrict__ cbnd) {
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
    cbnd[(int64_t)h * Cp + j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
}

// Wave per (head, centroid): tables for the stage's initial centroids.
template <int D>
__global__ void k_tables(const float *__restrict__ cent, int C, int Cp, const uint32_t *stats,
                         uint32_t *stats_w, int stat_stride, int bslot, half8 *__restrict__ ctab,
                         float *__restrict__ cinit, float4 *__restrict__ cbnd) {
  constexpr int PER = D / 64;
  const int h = blockIdx.y;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= Cp) return;
  if (j >= C) {
    emit_pad<D>(h, j, Cp, ctab, cinit, cbnd);
    return;
  }
  const uint32_t *st = stats + (int64_t)h * stat_stride;
  const float sc = ldexpf(1.0f, -scale_exp(fmaxf(stat_f(st, S_MAXR), stat_f(st, S_MAXC))));
  float cv[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) cv[m] = cent[((int64_t)h * Cp + j) * D + lane * PER + m];
  emit_tables<D>(h, j, Cp, cv, sc, ctab, cinit, cbnd, stats_w + (int64_t)h * stat_stride + bslot);
}

// ------------------------------------------------------------- assign
// Per-candidate error bound of a key (see the file header):
//   E = er*||c|| + rn*||c - c~|| + kappa*(rn*||c~|| + n/2) + 2^-40*(rn+||c~||+er+ec)^2
// with rn = ||r~||, er = ||r*sc - r~||; every factor is an upper bound.  The
// kappa term covers fp32 accumulation of the MFMA (any order) and the 8-bit
// index embedded in the key; the last term covers the fp64 rounding of the
// exact distances the decision has to agree with.
__device__ __forceinline__ float key_bound(float rn, float er, float cn, float ec, float ctn,
                                           float n, float kappa) {
  const float rc = rn + ctn + er + ec;
  const float e = er * cn + rn * ec + kappa * fmaf(rn, ctn, 0.5f * n) + 0x1p-40f * rc * rc;
  return e * (1.0f + 0x1p-20f) + 1e-37f;
}

// Persistent workgroups of 8 waves.  A work item is (head, 16 consecutive
// 32-token tiles); each workgroup takes a contiguous range of work items and
// reloads the head's tables into LDS only when the head changes.  Each wave
// multiplies two token tiles (B operand, registers) by every 32-centroid
// block (A operand, LDS).
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_assign(
    const half8 *__restrict__ rt, const float2 *__restrict__ tb, const half8 *__restrict__ ctab,
    const float *__restrict__ cinit, const float4 *__restrict__ cbnd,
    const uint32_t *__restrict__ stats, int stat_stride, int bslot, int N, int NT, int CB,
    int groups_per_head, int total_groups, int groups_per_wg, uint8_t *__restrict__ assign,
    int64_t assign_hstride, int4 *__restrict__ recheck, int2 *__restrict__ fallback,
    int4 *__restrict__ stage_re, int2 *__restrict__ stage_fb, uint32_t *__restrict__ counters,
    float kappa) {
  constexpr int KC = D / 16;
  constexpr int TPG = 16;  // tiles per work item
  extern __shared__ __align__(16) unsigned char smem[];
  half8 *ctab_s = reinterpret_cast<half8 *>(smem);
  float *cinit_s = reinterpret_cast<float *>(smem + (size_t)CB * KC * 64 * sizeof(half8));
  float4 *cbnd_s = reinterpret_cast<float4 *>(cinit_s + CB * 32);
  __shared__ float4 hmax_s;
  // unsettled tokens are staged in this workgroup's segment of stage_re /
  // stage_fb (slots from LDS counters) and copied to the compact lists once
  // at the end, with one global atomic per list
  __shared__ uint32_t lcnt[2], gbase[2];
  if (threadIdx.x == 0) lcnt[0] = lcnt[1] = 0u;  // read after the first barrier
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const uint32_t halfbits = (uint32_t)half << 2;
  // +inf and the mask live in VGPRs the compiler cannot see through, so that
  // a max is one v_med3_f32 (no canonicalising moves) and inserting the index
  // is one v_and_or_b32
  float INF;
  asm volatile("v_mov_b32 %0, 0x7f800000" : "=v"(INF));
  uint32_t vmask;
  asm volatile("v_mov_b32 %0, 0xffffff00" : "=v"(vmask));
  const int Cp = CB * kTile;
  int cached_h = -1;
  const int g_lo = blockIdx.x * groups_per_wg;
  const int g_hi = min(total_groups, g_lo + groups_per_wg);
  const int64_t seg = (int64_t)g_lo * TPG * kTile;  // this workgroup's staging segment
  for (int g = g_lo; g < g_hi; ++g) {
    const int h = g / groups_per_head;
    const int tile_lo = (g % groups_per_head) * TPG;
    if (h != cached_h) {  // uniform over the workgroup
      __syncthreads();
      block_copy<8>(ctab_s, ctab + (int64_t)h * CB * KC * 64, CB * KC * 64);
      block_copy<1>(cinit_s, cinit + (int64_t)h * CB * 32, CB * 32);
      block_copy<1>(cbnd_s, cbnd + (int64_t)h * Cp, Cp);
      __syncthreads();
      // per-head maxima of the per-centroid bounds (bound for all centroids)
      if (wave == 0) {
        float4 mx = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int q = lane; q < Cp; q += 64) {
          const float4 b = cbnd_s[q];
          mx.x = fmaxf(mx.x, b.x);
          mx.y = fmaxf(mx.y, b.y);
          mx.z = fmaxf(mx.z, b.z);
          mx.w = fmaxf(mx.w, b.w);
        }
        for (int o = 32; o > 0; o >>= 1) {
          mx.x = fmaxf(mx.x, __shfl_xor(mx.x, o));
          mx.y = fmaxf(mx.y, __shfl_xor(mx.y, o));
          mx.z = fmaxf(mx.z, __shfl_xor(mx.z, o));
          mx.w = fmaxf(mx.w, __shfl_xor(mx.w, o));
        }
        if (lane == 0) hmax_s = mx;
      }
      __syncthreads();
      cached_h = h;
    }
    const int t0 = tile_lo + 2 * wave;
    if (t0 >= NT) continue;
    const int t1 = min(t0 + 1, NT - 1);
    const half8 *f0 = rt + ((int64_t)h * NT + t0) * KC * 64 + lane;
    const half8 *f1 = rt + ((int64_t)h * NT + t1) * KC * 64 + lane;
    half8 b0[KC], b1[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) b0[kc] = f0[kc * 64];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) b1[kc] = f1[kc * 64];
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
        const float x0 = __uint_as_float((__float_as_uint(acc0[a]) & vmask) | enc);
        const float x1 = __uint_as_float((__float_as_uint(acc1[a]) & vmask) | enc);
        a3 = __builtin_amdgcn_fmed3f(a2, a3, x0);
        a2 = __builtin_amdgcn_fmed3f(a1, a2, x0);
        a1 = __builtin_amdgcn_fmed3f(a1, x0, INF);
        c3 = __builtin_amdgcn_fmed3f(c2, c3, x1);
        c2 = __builtin_amdgcn_fmed3f(c1, c2, x1);
        c1 = __builtin_amdgcn_fmed3f(c1, x1, INF);
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
    const float oo[3] = {__shfl_xor(s1, 32), __shfl_xor(s2, 32), __shfl_xor(s3, 32)};
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      m3 = __builtin_amdgcn_fmed3f(m2, m3, oo[q]);
      m2 = __builtin_amdgcn_fmed3f(m1, m2, oo[q]);
      m1 = __builtin_amdgcn_fmed3f(m1, oo[q], INF);
    }
    const int tile = t0 + half;
    const int tok = tile * kTile + (lane & 31);
    const bool live = tile < NT && tok < N;
    int kind = 0;  // 0 settled, 1 re-check, 2 full scan
    int j1 = 0, j2 = 0;
    if (live) {
      const float4 hm = hmax_s;
      const float2 b = tb[(int64_t)h * NT * kTile + tok];
      j1 = min((int)(__float_as_uint(m1) & 0xFFu), Cp - 1);
      j2 = min((int)(__float_as_uint(m2) & 0xFFu), Cp - 1);
      const float4 B1 = cbnd_s[j1], B2 = cbnd_s[j2];
      const float e1 = key_bound(b.x, b.y, B1.x, B1.y, B1.z, B1.w, kappa);
      const float e2 = key_bound(b.x, b.y, B2.x, B2.y, B2.z, B2.w, kappa);
      const float eg = key_bound(b.x, b.y, hm.x, hm.y, hm.z, hm.w, kappa);
      const float g12 = (m1 - m2) * (1.0f - 0x1p-20f);
      const float g13 = (m1 - m3) * (1.0f - 0x1p-20f);
      if (g12 > e1 + e2) {
        assign[(int64_t)h * assign_hstride + tok] = (uint8_t)j1;
      } else {
        kind = g13 > e1 + eg ? 1 : 2;
      }
    }
    // staged appends: one LDS atomic per wave and list, slots from mbcnt
    const uint64_t m_re = __ballot(kind == 1), m_fb = __ballot(kind == 2);
    const uint32_t lt_re = __builtin_amdgcn_mbcnt_hi((uint32_t)(m_re >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m_re, 0u));
    const uint32_t lt_fb = __builtin_amdgcn_mbcnt_hi((uint32_t)(m_fb >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m_fb, 0u));
    uint32_t base_re = 0, base_fb = 0;
    if (lane == 0) {
      if (m_re) base_re = atomicAdd(&lcnt[0], (uint32_t)__popcll(m_re));
      if (m_fb) base_fb = atomicAdd(&lcnt[1], (uint32_t)__popcll(m_fb));
    }
    base_re = __shfl(base_re, 0);
    base_fb = __shfl(base_fb, 0);
    if (kind == 1) stage_re[seg + base_re + lt_re] = make_int4(h, tok, j1, j2);
    if (kind == 2) stage_fb[seg + base_fb + lt_fb] = make_int2(h, tok);
  }
  // the workgroup's staged entries go to the compact lists
  __syncthreads();
  if (threadIdx.x == 0) {
    gbase[0] = lcnt[0] ? atomicAdd(counters + 0, lcnt[0]) : 0u;
    gbase[1] = lcnt[1] ? atomicAdd(counters + 1, lcnt[1]) : 0u;
  }
  __syncthreads();
  const uint32_t n_re = lcnt[0], n_fb = lcnt[1];
  for (uint32_t q = threadIdx.x; q < n_re; q += blockDim.x) recheck[gbase[0] + q] = stage_re[seg + q];
  for (uint32_t q = threadIdx.x; q < n_fb; q += blockDim.x) fallback[gbase[1] + q] = stage_fb[seg + q];
}

// ------------------------------------------------------------ resolve
// Exact fp64 squared distances of token i to NC centroid rows, channel order,
// no fused multiply-add: the same arithmetic as a plain sequential loop per
// centroid.  The residual row is rebuilt in fp32 (x minus the NSUB stage rows
// in stage order) KC channels at a time, every load of a chunk issued
// together (the stage indices are read once, so no load waits on another),
// and the NC distances share the residual loads.
template <typename Tin, int D, int NC, int NSUB>
__device__ __forceinline__ void exact_dist_n(const ResView<Tin> &rv, int h, int64_t i,
                                             const float *c0, const float *c1, double *out) {
  constexpr int KC = 8;
  const float *cr[2] = {c0, c1};
  const Tin *sr[NSUB > 0 ? NSUB : 1];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) sr[s] = rv.stage_row(h, s, rv.stage_j(h, s, i));
  const Tin *xr = rv.x + rv.xrow(h, i);
  double acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = 0.0;
#pragma unroll 1
  for (int k0 = 0; k0 < D; k0 += KC) {
    float v[KC], w[NC][KC], cs[NSUB > 0 ? NSUB : 1][KC];
#pragma unroll
    for (int q = 0; q < KC / 8; ++q) {
      ::qvg::load8(xr, k0 + 8 * q, v + 8 * q);
#pragma unroll
      for (int c = 0; c < NC; ++c) load8(cr[c], k0 + 8 * q, w[c] + 8 * q);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) ::qvg::load8(sr[s], k0 + 8 * q, cs[s] + 8 * q);
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int m = 0; m < KC; ++m) v[m] = v[m] - cs[s][m];
#pragma unroll
    for (int m = 0; m < KC; ++m)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const double df = (double)v[m] - (double)w[c][m];
        acc[c] = __dadd_rn(acc[c], __dmul_rn(df, df));
      }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) out[c] = acc[c];
}

// The view's stage count (runtime) dispatched to the compile-time form.
template <typename Tin, int D, int NC>
__device__ __forceinline__ void exact_dist(const ResView<Tin> &rv, int h, int64_t i,
                                                     const float *c0, const float *c1,
                                                     double *out) {
  switch (rv.nsub) {
    case 0: exact_dist_n<Tin, D, NC, 0>(rv, h, i, c0, c1, out); break;
    case 1: exact_dist_n<Tin, D, NC, 1>(rv, h, i, c0, c1, out); break;
    case 2: exact_dist_n<Tin, D, NC, 2>(rv, h, i, c0, c1, out); break;
    case 3: exact_dist_n<Tin, D, NC, 3>(rv, h, i, c0, c1, out); break;
    case 4: exact_dist_n<Tin, D, NC, 4>(rv, h, i, c0, c1, out); break;
    case 5: exact_dist_n<Tin, D, NC, 5>(rv, h, i, c0, c1, out); break;
    case 6: exact_dist_n<Tin, D, NC, 6>(rv, h, i, c0, c1, out); break;
    default: exact_dist_n<Tin, D, NC, kMaxT - 1>(rv, h, i, c0, c1, out); break;
  }
}

// Both the sequential fp64 sum and any other fp64 summation order of the D
// non-negative terms lie within gamma_{D+2} of the exact distance, so when two
// distances computed in another order differ by more than
// 2*gamma*(D1 + D2) (with slack), the sequential ones order the same way.
template <int D>
__device__ __forceinline__ double order_tol() {
  return (2.0 * (D + 4) * 0x1p-53) * 1.01;
}

// Re-check of the two candidates: D/8 lanes per entry, each lane 8 channels,
// fp64 partial sums combined by a fixed butterfly; the sequential fp64 replica
// decides only when the margin is too thin to settle the order.
template <typename Tin, int D>
__device__ __forceinline__ void recheck_part(const ResView<Tin> &rv, const float *__restrict__ cent,
                                             int Cp, const int4 *__restrict__ list,
                                             const uint32_t *__restrict__ counters,
                                             uint8_t *__restrict__ assign, int64_t assign_hstride,
                                             uint32_t b0, uint32_t nb) {
  constexpr int LPE = D / 8, EPW = 64 / LPE;
  const uint32_t n = counters[0];
  const int lane = threadIdx.x & 63, sub = lane / LPE, li = lane % LPE;
  const uint32_t gw = ((blockIdx.x - b0) * blockDim.x + threadIdx.x) >> 6;
  const uint32_t nw = (nb * blockDim.x) >> 6;
  for (uint32_t base = gw * EPW; base < n; base += nw * EPW) {
    const uint32_t e = base + sub;
    const bool live = e < n;
    const int4 q = live ? list[e] : make_int4(0, 0, 0, 0);
    const float *cb = cent + (int64_t)q.x * Cp * D;
    double s1 = 0.0, s2 = 0.0;
    if (live) {
      float v[8], w1[8], w2[8];
      rv.load8(q.x, q.y, li * 8, v);
      load8(cb + (int64_t)q.z * D, li * 8, w1);
      load8(cb + (int64_t)q.w * D, li * 8, w2);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const double d1 = (double)v[m] - (double)w1[m];
        const double d2 = (double)v[m] - (double)w2[m];
        s1 = __dadd_rn(s1, __dmul_rn(d1, d1));
        s2 = __dadd_rn(s2, __dmul_rn(d2, d2));
      }
    }
#pragma unroll
    for (int o = 1; o < LPE; o <<= 1) {
      s1 = __dadd_rn(s1, __shfl_xor(s1, o));
      s2 = __dadd_rn(s2, __shfl_xor(s2, o));
    }
    if (live && li == 0) {
      const double diff = s2 - s1, tol = (s1 + s2) * order_tol<D>();
      int j;
      if (diff > tol) {
        j = q.z;
      } else if (diff < -tol) {
        j = q.w;
      } else {
        double dd[2];
        exact_dist<Tin, D, 2>(rv, q.x, q.y, cb + (int64_t)q.z * D, cb + (int64_t)q.w * D, dd);
        const double d1 = dd[0], d2 = dd[1];
        j = (d2 < d1 || (d2 == d1 && q.w < q.z)) ? q.w : q.z;
      }
      assign[(int64_t)q.x * assign_hstride + q.y] = (uint8_t)j;
    }
  }
}

// Exact scan over all centroids for the tokens the bound could not settle:
// one workgroup per entry (grid-stride), thread j owns centroid j.  fp64
// distances with 4 interleaved partial sums (within gamma_{D+4} of the exact
// distance in any order) pick the best; any centroid whose order against the
// best is not settled by that margin gets the sequential fp64 distance, the
// same arithmetic as a plain loop.  Smallest distance wins, ties to the
// smallest index.
template <typename Tin, int D>
__device__ __forceinline__ void fallback_part(const ResView<Tin> &rv,
                                              const float *__restrict__ cent, int C, int Cp,
                                              const int2 *__restrict__ list,
                                              const uint32_t *__restrict__ counters,
                                              uint8_t *__restrict__ assign,
                                              int64_t assign_hstride, uint32_t b0, uint32_t nb) {
  constexpr int D4 = D / 4, HB = D4 / 2;
  __shared__ float4 rs[D4];
  __shared__ double wbest[4];
  __shared__ int wbj[4], wnear[4];
  const uint32_t n = counters[1];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const double tol = order_tol<D>();
  for (uint32_t e = blockIdx.x - b0; e < n; e += nb) {
    const int2 q = list[e];
    const float *ch = cent + (int64_t)q.x * Cp * D;
    // the first half of this thread's centroid row goes out before the
    // token's residual row
    const int j = min(t, C - 1);
    const float4 *c4 = reinterpret_cast<const float4 *>(ch + (int64_t)j * D);
    float4 c[HB];
#pragma unroll
    for (int k = 0; k < HB; ++k) c[k] = c4[k];
    if (t < D4) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = rv.get(q.x, q.y, t * 4 + u);
      rs[t] = make_float4(v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
    double p0 = 0.0, p1 = 0.0, p2 = 0.0, p3 = 0.0;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      if (hb == 1) {
#pragma unroll
        for (int k = 0; k < HB; ++k) c[k] = c4[HB + k];
      }
#pragma unroll
      for (int k = 0; k < HB; ++k) {
        const float4 x = rs[hb * HB + k];
        const double dx = (double)x.x - (double)c[k].x, dy = (double)x.y - (double)c[k].y;
        const double dz = (double)x.z - (double)c[k].z, dw = (double)x.w - (double)c[k].w;
        p0 = __dadd_rn(p0, __dmul_rn(dx, dx));
        p1 = __dadd_rn(p1, __dmul_rn(dy, dy));
        p2 = __dadd_rn(p2, __dmul_rn(dz, dz));
        p3 = __dadd_rn(p3, __dmul_rn(dw, dw));
      }
    }
    const double dp = t < C ? (p0 + p1) + (p2 + p3) : __builtin_inf();
    // workgroup argmin of (dp, j)
    double best = dp;
    int bj = t < C ? t : 0x7fffffff;
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oj = __shfl_xor(bj, o);
      if (ob < best || (ob == best && oj < bj)) {
        best = ob;
        bj = oj;
      }
    }
    if (lane == 0) {
      wbest[wave] = best;
      wbj[wave] = bj;
    }
    __syncthreads();
    best = wbest[0];
    bj = wbj[0];
    for (int w = 1; w < 4; ++w)
      if (wbest[w] < best || (wbest[w] == best && wbj[w] < bj)) {
        best = wbest[w];
        bj = wbj[w];
      }
    // centroids whose order against the best is not settled by the margin
    const bool near = t < C && t != bj && dp - best <= tol * (dp + best);
    const uint64_t nb = __ballot(near);
    if (lane == 0) wnear[wave] = nb != 0ull;
    __syncthreads();
    const bool any_near = wnear[0] | wnear[1] | wnear[2] | wnear[3];
    if (any_near) {  // uniform over the workgroup
      const bool mine = t < C && (t == bj || dp - best <= tol * (dp + best));
      double sb = __builtin_inf();
      if (mine) exact_dist<Tin, D, 1>(rv, q.x, q.y, ch + (int64_t)t * D, nullptr, &sb);
      int sj = mine ? t : 0x7fffffff;
      for (int o = 32; o > 0; o >>= 1) {
        const double ob = __shfl_xor(sb, o);
        const int oj = __shfl_xor(sj, o);
        if (ob < sb || (ob == sb && oj < sj)) {
          sb = ob;
          sj = oj;
        }
      }
      __syncthreads();
      if (lane == 0) {
        wbest[wave] = sb;
        wbj[wave] = sj;
      }
      __syncthreads();
      sb = wbest[0];
      sj = wbj[0];
      for (int w = 1; w < 4; ++w)
        if (wbest[w] < sb || (wbest[w] == sb && wbj[w] < sj)) {
          sb = wbest[w];
          sj = wbj[w];
        }
      bj = sj;
    }
    if (t == 0) assign[(int64_t)q.x * assign_hstride + q.y] = (uint8_t)bj;
    __syncthreads();
  }
}

// Both kinds of unsettled tokens in one launch: re-checks of two candidates
// (a wave per EPW entries, grid-stride over the re-check workgroups) and exact
// scans (a workgroup per entry, grid-stride over the scan workgroups).
// Iterations with few or no candidates cost one small launch.  Held to 128
// registers (4 waves per SIMD, the whole grid resident) with the sequential
// replica inlined.
template <typename Tin, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_resolve(ResView<Tin> rv, const float *__restrict__ cent,
                                                 int C, int Cp, const int4 *__restrict__ rlist,
                                                 const int2 *__restrict__ flist,
                                                 const uint32_t *__restrict__ counters,
                                                 uint8_t *__restrict__ assign,
                                                 int64_t assign_hstride) {
  // The two lists go concurrently: each exact scan is one workgroup's latency
  // chain, so scans take up to three quarters of the workgroups (all of them
  // when there are no re-checks) and the re-checks the rest.
  const uint32_t nre = counters[0], nfb = counters[1], G = gridDim.x;
  const uint32_t fw = min(nfb, nre ? G - G / 4 : G);
  if (blockIdx.x < fw)
    fallback_part<Tin, D>(rv, cent, C, Cp, flist, counters, assign, assign_hstride, 0u, fw);
  else
    recheck_part<Tin, D>(rv, cent, Cp, rlist, counters, assign, assign_hstride, fw, G - fw);
}

// --------------------------------------------------------------- sort
// Stable counting sort of token ids by cluster, in two kernels over chunks of
// kSortChunk tokens: k_hist counts each chunk; k_scatter derives every
// chunk's start position per cluster from the counts and writes the ids with
// ranks taken from ballots, so token order is kept within every cluster.
// k_hist also clears the next bound slot of the head and (first chunk of head
// 0) logs and clears the candidate-list counters.  With prev set it copies the
// assignments to prev[par ^ 1]; with `delta` set, a head that may be updated
// incrementally (head_inc_candidate) also lists the tokens of this block whose
// assignment differs from prev[par] (the previous update's) in its own segment
// moved[h][lo ..) (in no particular order), and their number in mcnt[h][b].
__global__ __launch_bounds__(256) void k_hist(const uint8_t *__restrict__ assign,
                                              int64_t assign_hstride, int N,
                                              uint32_t *__restrict__ hist, uint32_t *stats,
                                              int stat_stride, int clear_slot,
                                              uint32_t *counters, int log_slot,
                                              uint8_t *__restrict__ prev, int par, int delta,
                                              int32_t *__restrict__ moved,
                                              uint32_t *__restrict__ mcnt) {
  __shared__ uint32_t cnt[kMaxC];
  __shared__ uint32_t nmv;
  const int h = blockIdx.y, b = blockIdx.x;
  const int nb = gridDim.x, H = gridDim.y;
  cnt[threadIdx.x] = 0;
  if (threadIdx.x == 0) nmv = 0u;
  if (b == 0 && threadIdx.x < 4) stats[(int64_t)h * stat_stride + clear_slot + threadIdx.x] = 0;
  if (b == 0 && h == 0 && threadIdx.x < 2) {
    // keep the finished iteration's candidate counts for diagnostics
    if (log_slot >= 0 && log_slot < kCounterLog)
      counters[4 + 2 * log_slot + threadIdx.x] = counters[threadIdx.x];
    counters[threadIdx.x] = 0;
  }
  const bool track = prev && delta && head_inc_candidate(stats, stat_stride, h, N);
  __syncthreads();
  const uint8_t *a = assign + (int64_t)h * assign_hstride;
  const uint8_t *pr = prev ? prev + ((int64_t)par * H + h) * N : nullptr;
  uint8_t *pw = prev ? prev + ((int64_t)(par ^ 1) * H + h) * N : nullptr;
  const int lo = b * kSortChunk, hi = min(N, lo + kSortChunk);
  int32_t *seg = moved + (int64_t)h * N + lo;
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = lo; i0 < hi; i0 += 256) {  // uniform trip count (ballots below)
    const int i = i0 + (int)threadIdx.x;
    const bool in = i < hi;
    const uint32_t j = in ? (uint32_t)a[i] : 0u;
    if (in) {
      atomicAdd(&cnt[j], 1u);
      if (pw) pw[i] = (uint8_t)j;
    }
    if (track) {
      const bool ch = in && (uint32_t)pr[i] != j;
      const uint64_t m = __ballot(ch);
      uint32_t base = 0;
      if (m && lane == 0) base = atomicAdd(&nmv, (uint32_t)__popcll(m));
      base = __shfl(base, 0);
      if (ch) seg[base + __popcll(m & lt)] = i;
    }
  }
  __syncthreads();
  hist[((int64_t)h * nb + b) * kMaxC + threadIdx.x] = cnt[threadIdx.x];
  if (track && threadIdx.x == 0) mcnt[(int64_t)h * nb + b] = nmv;
}

// Inclusive scan of one value per thread over a 256-thread workgroup: a
// shuffle scan inside each wave, then the totals of the lower waves (two
// barriers; ws holds at least 4 words of shared memory).  Integer adds, so
// the result does not depend on the order.
__device__ __forceinline__ uint32_t scan256_incl(uint32_t v, uint32_t *ws) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) ws[wave] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; ++w) add += ws[w];
  __syncthreads();  // ws may be written again by the next scan
  return v + add;
}

// With stats set, k_scatter decides how this iteration updates the head
// (written to S_INC by block 0): incrementally when `delta` is set, the head is
// a candidate (head_inc_candidate), every cluster's fp64 sum is exact (its
// member count n satisfies span + ceil(log2 n) <= 29, so the integer sum is
// the sequential one) and at most N/4 of its tokens moved (the sum of the
// blocks' counts mcnt[h][..]); then only the full update sorts.  Past a
// quarter of the tokens, gathering every moved row once per channel slice
// costs more than one pass over all.
__global__ __launch_bounds__(256) void k_scatter(const uint8_t *__restrict__ assign,
                                                 int64_t assign_hstride, int N, int Cp,
                                                 const uint32_t *__restrict__ hist,
                                                 int32_t *__restrict__ sorted,
                                                 int32_t *__restrict__ offs,
                                                 int32_t *__restrict__ cofs,
                                                 int32_t *__restrict__ chunk_j, int maxch,
                                                 uint32_t *stats, int stat_stride, int delta,
                                                 const uint32_t *__restrict__ mcnt) {
  __shared__ uint32_t scan[4];
  __shared__ uint32_t wbase[4][kMaxC];
  const int h = blockIdx.y, b = blockIdx.x, nb = gridDim.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // heads that are no candidate, or whose sums are exact for any member set
  // (then every cluster's are), are decided before the counts are read
  bool decided = true;
  if (stats) {
    const bool cand = delta && head_inc_candidate(stats, stat_stride, h, N);  // uniform
    decided = !cand || head_sums_exact(stats, stat_stride, h);
    if (decided) {
      bool inc = false;
      if (cand) {
        uint32_t m = 0;
        for (int q = t; q < nb; q += 256) m += mcnt[(int64_t)h * nb + q];
        inc = block_sum_u32(m) <= (uint32_t)(N / 4);
      }
      if (b == 0 && t == 0) stats[(int64_t)h * stat_stride + S_INC] = inc ? 1u : 0u;
      if (inc) return;
    }
  }
  const uint8_t *a = assign + (int64_t)h * assign_hstride;
  const int lo = b * kSortChunk, hi = min(N, lo + kSortChunk);
  // this wave's quarter of the chunk: token wlo + lane + 64k is jk[k] (loaded
  // first, so the loads overlap the count reads below; kSortChunk / 4 = 4 * 64)
  static_assert(kSortChunk % 256 == 0, "four waves of whole 64-token rounds");
  constexpr int QW = kSortChunk / 4, KW = QW / 64;
  const int wlo = min(hi, lo + wave * QW), whi = min(hi, wlo + QW);
  uint32_t jk[KW];
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int i = wlo + lane + 64 * k;
    jk[k] = i < whi ? (uint32_t)a[i] : 0u;
  }
  // this chunk's predecessors and all chunks, for byte value t
  const uint32_t *hh = hist + (int64_t)h * nb * kMaxC + t;
  uint32_t pre = 0, tot = 0;
  int bb = 0;
  for (; bb + 32 <= nb; bb += 32) {  // 32 loads in flight per round
    uint32_t c[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) c[u] = hh[(int64_t)(bb + u) * kMaxC];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      tot += c[u];
      pre += bb + u < b ? c[u] : 0u;
    }
  }
  for (; bb + 8 <= nb; bb += 8) {
    uint32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = hh[(int64_t)(bb + u) * kMaxC];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      tot += c[u];
      pre += bb + u < b ? c[u] : 0u;
    }
  }
  for (; bb < nb; ++bb) {
    const uint32_t c = hh[(int64_t)bb * kMaxC];
    tot += c;
    pre += bb < b ? c : 0u;
  }
  if (!decided) {  // a candidate whose sums are exact cluster by cluster
    uint32_t m = 0;
    for (int q = t; q < nb; q += 256) m += mcnt[(int64_t)h * nb + q];
    const uint32_t moved = block_sum_u32(m);
    const uint32_t most = block_max_u32(tot);  // largest cluster of this iteration
    const int w = (int)__builtin_amdgcn_readfirstlane(stats[(int64_t)h * stat_stride + S_SPANW]);
    const bool inc = moved <= (uint32_t)(N / 4) && w + ceil_log2(most) <= 29;
    if (b == 0 && t == 0) stats[(int64_t)h * stat_stride + S_INC] = inc ? 1u : 0u;
    if (inc) return;
  }
  // exclusive scan of the totals over the 256 byte values; assignment bytes
  // >= C (corrupt input only) get slots after the clusters
  const uint32_t mine = scan256_incl(tot, scan);
  const uint32_t excl = mine - tot;
  if (b == 0) {
    if (t <= Cp) offs[(int64_t)h * (Cp + 1) + t] = (int32_t)excl;
    if (Cp == kMaxC && t == kMaxC - 1) offs[(int64_t)h * (Cp + 1) + Cp] = (int32_t)mine;
    // chunks of kAccChunk consecutive members per cluster: exclusive scan of
    // the chunk counts of clusters 0..Cp-1, and the chunk -> cluster map
    const uint32_t nch = t < Cp ? (tot + kAccChunk - 1) / kAccChunk : 0u;
    const uint32_t cm = scan256_incl(nch, scan);
    const uint32_t cex = cm - nch;
    if (t <= Cp) cofs[(int64_t)h * (Cp + 1) + t] = (int32_t)cex;
    if (Cp == kMaxC && t == kMaxC - 1) cofs[(int64_t)h * (Cp + 1) + Cp] = (int32_t)cm;
    for (uint32_t q = 0; q < nch; ++q) chunk_j[(int64_t)h * maxch + cex + q] = t;
  }
  // per-wave counts inside the chunk (each wave owns a quarter, in order)
  for (int w = 0; w < 4; ++w) wbase[w][t] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < KW; ++k)
    if (wlo + lane + 64 * k < whi) atomicAdd(&wbase[wave][jk[k]], 1u);
  __syncthreads();
  {
    uint32_t run = excl + pre;
    for (int w = 0; w < 4; ++w) {
      const uint32_t c = wbase[w][t];
      wbase[w][t] = run;
      run += c;
    }
  }
  __syncthreads();
  int32_t *out = sorted + (int64_t)h * N;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int g = wlo + 64 * k;
    if (g >= whi) break;  // wave-uniform
    const int i = g + lane;
    const bool valid = i < whi;
    const uint32_t j = jk[k];
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t bb = __ballot(valid && ((j >> bit) & 1u));
      m &= ((j >> bit) & 1u) ? bb : ~bb;
    }
    if (valid) out[wbase[wave][j] + __popcll(m & lt)] = i;
    __builtin_amdgcn_wave_barrier();
    if (valid && (m >> lane) == 1ull) wbase[wave][j] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------- accumulate
// The members of each cluster (token order, from the counting sort) are cut
// into chunks of kAccChunk.  k_chunk_sum: one wave per chunk sums its members'
// rows in fp64 (a lane takes 8 channels of every (64/(D/8))-th member; the
// lane groups are combined at the end).  k_finalize: one wave per cluster
// adds its chunk sums in chunk order, divides in fp64 and rounds to fp32 (an
// empty cluster keeps its
// centroid).  Exactness: every value is an integer multiple of 2^(lmin-150)
// and smaller than 2^(emax-126) in magnitude (lmin = exponent field + trailing
// zeros of the significand, a lower bound for subnormals; emax = largest
// exponent field; zeros excluded), so for n members every partial sum, in any
// order, is a multiple of 2^(lmin-150) below n*2^(emax-126); when
// emax - lmin + ceil(log2 n) <= 29 all of them fit in 53 bits and the chunked
// sum is the sequential one.  Otherwise the wave re-sums the cluster in one
// token-order pass.  It then emits the centroid's tables for the next assign
// and, on the stage's last iteration, the record centroid (rounded to the
// record dtype) and the fp32 cache entry.

// Exponent field and lowest-bit bound of an fp32 value (0xFFFF for zeros).
__device__ __forceinline__ void exact_span(float v, uint32_t &emax, uint32_t &lmin) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t e = (b >> 23) & 0xFFu;
  const uint32_t l = e + (uint32_t)__builtin_ctz(b | 0x800000u);
  emax = max(emax, e);
  lmin = min(lmin, v != 0.0f ? l : 0xFFFFu);
}
// TRACK: also record the chunk's per-channel spans (not needed once the whole
// head's spans have shown every cluster sum of this stage exact).
template <typename Tin, int D, int NSUB, bool TRACK>
__device__ __forceinline__ void chunk_sum_body(const ResView<Tin> &rv, int Cp,
                                               const int32_t *__restrict__ sorted,
                                               const int32_t *__restrict__ offs,
                                               const int32_t *__restrict__ cofs,
                                               const int32_t *__restrict__ chunk_j, int maxch,
                                               double *__restrict__ part,
                                               uint32_t *__restrict__ pflag, int h, int g) {
  constexpr int LPR = D / 8;              // lanes per member row (8 channels each)
  constexpr int RPI = 64 / LPR;           // member rows per load instruction
  constexpr int MPL = kAccChunk / RPI;    // members per lane
  constexpr int MB = 4;                   // members per lane in flight
  const int lane = threadIdx.x & 63;
  const int total = __builtin_amdgcn_readfirstlane(cofs[(int64_t)h * (Cp + 1) + Cp]);
  if (g >= total) return;
  const int j = __builtin_amdgcn_readfirstlane(chunk_j[(int64_t)h * maxch + g]);
  const int c0 = __builtin_amdgcn_readfirstlane(cofs[(int64_t)h * (Cp + 1) + j]);
  const int o0 = __builtin_amdgcn_readfirstlane(offs[(int64_t)h * (Cp + 1) + j]);
  const int o1 = __builtin_amdgcn_readfirstlane(offs[(int64_t)h * (Cp + 1) + j + 1]);
  const int start = o0 + (g - c0) * kAccChunk;
  const int cnt = min(kAccChunk, o1 - start);
  const int N = rv.N;
  // lane u holds member u's token id and its cluster in every earlier stage
  // (NSUB = the stage index, a template parameter, so the loads below are
  // issued without branches)
  const int32_t id = sorted[(int64_t)h * N + start + min(lane, cnt - 1)];
  int pj[NSUB > 0 ? NSUB : 1];
#pragma unroll
  for (int st = 0; st < NSUB; ++st) pj[st] = rv.stage_j(h, st, id);
  // this lane: channels q*8 .. q*8+7 of members sub, sub + RPI, ...
  const int sub = lane / LPR, q = lane % LPR;
  const Tin *xh = rv.x + (int64_t)h * N * D + q * 8;
  double s[8];
  uint32_t emax[8], lmin[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0, emax[e] = 0, lmin[e] = 0xFFFFu;
#pragma unroll
  for (int k0 = 0; k0 < MPL; k0 += MB) {
    float v[MB][8];
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const int src = min(sub + RPI * (k0 + k), cnt - 1);
      const int64_t row = __shfl(id, src);
      load8(xh, row * D, v[k]);
#pragma unroll
      for (int st = 0; st < NSUB; ++st) {  // R(t) = x - C(1)[pi(1)] - ... in stage order
        float c[8];
        load8(rv.stage_row(h, st, __shfl(pj[st], src)), q * 8, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[k][e] = v[k][e] - c[e];
      }
    }
#pragma unroll
    for (int k = 0; k < MB; ++k)
      if (sub + RPI * (k0 + k) < cnt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s[e] = __dadd_rn(s[e], (double)v[k][e]);
          if constexpr (TRACK) exact_span(v[k][e], emax[e], lmin[e]);
        }
  }
  // combine the RPI member slots (in any order: the finalize pass only uses
  // these sums when the spans prove every partial sum exact)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[e] = __dadd_rn(s[e], __shfl_xor(s[e], off));
      if constexpr (TRACK) {
        emax[e] = max(emax[e], (uint32_t)__shfl_xor((int)emax[e], off));
        lmin[e] = min(lmin[e], (uint32_t)__shfl_xor((int)lmin[e], off));
      }
    }
  if (sub == 0) {
    double *dst = part + ((int64_t)h * maxch + g) * D + q * 8;
    uint32_t *fl = pflag + ((int64_t)h * maxch + g) * D + q * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dst[e] = s[e];
      if constexpr (TRACK) fl[e] = emax[e] | (lmin[e] << 16);
    }
  }
}

template <typename Tin, int D, int NSUB>
__global__ __launch_bounds__(256) void k_chunk_sum(ResView<Tin> rv, int Cp,
                                                   const int32_t *__restrict__ sorted,
                                                   const int32_t *__restrict__ offs,
                                                   const int32_t *__restrict__ cofs,
                                                   const int32_t *__restrict__ chunk_j,
                                                   int maxch, double *__restrict__ part,
                                                   uint32_t *__restrict__ pflag,
                                                   uint32_t *stats, int stat_stride) {
  const int h = blockIdx.y, g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (head_incremental(stats, stat_stride, h)) return;  // updated from its moved tokens
  // summed in full: its integer sums are exact unless k_finalize has to sum a
  // cluster again in token order (it then clears the flag)
  if (blockIdx.x == 0 && threadIdx.x == 0) stats[(int64_t)h * stat_stride + S_ISUM] = 1u;
  if (head_sums_exact(stats, stat_stride, h))
    chunk_sum_body<Tin, D, NSUB, false>(rv, Cp, sorted, offs, cofs, chunk_j, maxch, part, pflag,
                                        h, g);
  else
    chunk_sum_body<Tin, D, NSUB, true>(rv, Cp, sorted, offs, cofs, chunk_j, maxch, part, pflag,
                                       h, g);
}

// Head-wide spans of a stage's residual, from the per-chunk spans of its first
// iteration: every token is in exactly one chunk, and the residual is the same
// in all iterations of the stage, so if emax - lmin + ceil(log2 N) <= 29 in
// every channel, every partial sum of any cluster (at most N members) of any
// later iteration is exact.  k_span_part reduces kSpanParts groups of chunks,
// k_span_final the groups, and sets S_SPAN.
template <int D>
__global__ __launch_bounds__(256) void k_span_part(const uint32_t *__restrict__ pflag,
                                                   const int32_t *__restrict__ cofs, int Cp,
                                                   int maxch, uint32_t *__restrict__ span) {
  constexpr int RPP = 256 / D;  // chunk rows per pass
  const int h = blockIdx.y, y = blockIdx.x;
  const int total = cofs[(int64_t)h * (Cp + 1) + Cp];
  const int per = (total + kSpanParts - 1) / kSpanParts;
  const int g0 = y * per, g1 = min(total, g0 + per);
  const int ch = threadIdx.x % D, r = threadIdx.x / D;
  uint32_t emax = 0u, lmin = 0xFFFFu;
  for (int g = g0 + r; g < g1; g += RPP) {
    const uint32_t f = pflag[((int64_t)h * maxch + g) * D + ch];
    emax = max(emax, f & 0xFFFFu);
    lmin = min(lmin, f >> 16);
  }
  __shared__ uint32_t se[256], sl[256];
  se[threadIdx.x] = emax;
  sl[threadIdx.x] = lmin;
  __syncthreads();
  if (threadIdx.x < D) {
    for (int q = 1; q < RPP; ++q) {
      emax = max(emax, se[threadIdx.x + q * D]);
      lmin = min(lmin, sl[threadIdx.x + q * D]);
    }
    span[((int64_t)h * kSpanParts + y) * D + threadIdx.x] = emax | (lmin << 16);
  }
}
template <int D>
__global__ __launch_bounds__(D) void k_span_final(const uint32_t *__restrict__ span, int N,
                                                  uint32_t *__restrict__ stats, int stat_stride,
                                                  uint32_t *__restrict__ lminv) {
  const int h = blockIdx.x;
  uint32_t emax = 0u, lmin = 0xFFFFu;
#pragma unroll 8
  for (int y = 0; y < kSpanParts; ++y) {
    const uint32_t f = span[((int64_t)h * kSpanParts + y) * D + threadIdx.x];
    emax = max(emax, f & 0xFFFFu);
    lmin = min(lmin, f >> 16);
  }
  const int lg = N > 1 ? 32 - __builtin_clz((uint32_t)(N - 1)) : 0;
  const int risky = (int)emax - (int)lmin + lg > 29;
  if (lminv) lminv[(int64_t)h * D + threadIdx.x] = lmin;
  // the widest span over the channels that hold a nonzero value
  __shared__ int wmax;
  if (threadIdx.x == 0) wmax = 0;
  const int any = __syncthreads_or(risky);
  if (lmin != 0xFFFFu) atomicMax(&wmax, (int)emax - (int)lmin);
  __syncthreads();
  if (threadIdx.x == 0) {
    stats[(int64_t)h * stat_stride + S_SPAN] = 1u | (any ? 2u : 0u);
    stats[(int64_t)h * stat_stride + S_SPANW] = (uint32_t)max(wmax, 0);
  }
}

// ------------------------------------------------------ incremental update
// For a head whose stage sums are exact (S_SPAN == 1), every value of channel
// k of the stage residual is an integer multiple of 2^(lmin_k - 150) and every
// sum of distinct members is below 2^53 of those units (the span condition),
// so the cluster sums are kept as int64 multiples of 2^(lmin_k - 150): integer
// adds are exact in any order, and the fp64 value of a sum is the sequential
// fp64 sum.  From the second iteration of the stage on, only the tokens whose
// assignment changed since the previous update (listed by k_hist) move their
// rows: subtracted from the old cluster's sum, added to the new one.
__device__ __forceinline__ long long to_units(double v, uint32_t lmin) {
  return (long long)ldexp(v, 150 - (int)lmin);  // an integer below 2^53: exact
}
__device__ __forceinline__ double from_units(long long q, uint32_t lmin) {
  return ldexp((double)q, (int)lmin - 150);
}

// One workgroup per (8 channels, head), all workgroups of a head on one XCD
// (workgroups are dealt to the 8 XCDs in turn by id), so the moved rows they
// share come from HBM once and from that XCD's L2 afterwards.  The sums of the
// workgroup's channels for every cluster live in LDS (rows padded to 9 words
// against bank conflicts); the moved tokens of up to 512 sort blocks at a time
// are located through a prefix sum of the blocks' counts; up to four tokens
// per lane are in flight (fewer for later stages, which hold more rows), each
// row rebuilt as R(t) = x - C(1)[pi(1)] - ... (the arithmetic of the full
// update) and added with 64-bit LDS atomics.  The workgroup then adds its
// slice to isum (it is the slice's only writer; the slice is loaded first).
constexpr int kDeltaRow = 9;
constexpr int kDeltaThreads = 512;
__host__ __device__ inline int delta_grid(int H, int D) { return 8 * ((H + 7) / 8) * (D / 8); }

template <typename Tin, int D, int NSUB>
__device__ __forceinline__ void delta_body(
    const ResView<Tin> &rv, int H, int Cp, const uint8_t *__restrict__ assign,
    int64_t assign_hstride, const uint8_t *__restrict__ prev, int par,
    const int32_t *__restrict__ moved, const uint32_t *__restrict__ mcnt, int nb,
    const uint32_t *__restrict__ lminv, long long *__restrict__ isum,
    const uint32_t *__restrict__ stats, int stat_stride, int id) {
  constexpr int U = NSUB <= 1 ? 4 : (NSUB <= 3 ? 2 : 1);
  constexpr int S = D / 8;                       // channel slices per head
  constexpr int QS = kMaxC * 8 / kDeltaThreads;  // isum words per thread
  __shared__ unsigned long long acc[kMaxC * kDeltaRow];
  __shared__ uint32_t pre[kDeltaThreads + 1];
  __shared__ uint32_t wsum[kDeltaThreads / 64];
  const int xcd = id % 8, k = id / 8;
  const int h = xcd + 8 * (k / S), k0 = (k % S) * 8;
  if (h >= H) return;
  const int N = rv.N;
  // independent loads first: the slice of isum and the channel bounds
  long long *dst = isum + (int64_t)h * Cp * D + k0;
  long long old[QS];
#pragma unroll
  for (int r = 0; r < QS; ++r) {
    const int q = r * kDeltaThreads + (int)threadIdx.x;
    old[r] = q < Cp * 8 ? dst[(int64_t)(q >> 3) * D + (q & 7)] : 0ll;
  }
  uint32_t lm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) lm[e] = lminv[(int64_t)h * D + k0 + e];
  if (!head_incremental(stats, stat_stride, h)) return;
  for (int q = threadIdx.x; q < Cp * kDeltaRow; q += kDeltaThreads) acc[q] = 0ull;
  const uint8_t *ah = assign + (int64_t)h * assign_hstride;
  const uint8_t *ph = prev + ((int64_t)par * H + h) * N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bool any = false;
  for (int b0 = 0; b0 < nb; b0 += kDeltaThreads) {
    // exclusive prefix of the counts of blocks b0 .. b0+511
    uint32_t c = b0 + (int)threadIdx.x < nb ? mcnt[(int64_t)h * nb + b0 + threadIdx.x] : 0u;
    c = min(c, (uint32_t)kSortChunk);
    uint32_t v = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint32_t add = 0;
    for (int w = 0; w < wave; ++w) add += wsum[w];
    pre[threadIdx.x + 1] = v + add;
    if (threadIdx.x == 0) pre[0] = 0u;
    __syncthreads();
    const int tot = (int)pre[kDeltaThreads];
    any |= tot > 0;
    for (int f0 = 0; f0 < tot; f0 += U * kDeltaThreads) {
      int tok[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = min(f0 + u * kDeltaThreads + (int)threadIdx.x, tot - 1);
        ok[u] = f0 + u * kDeltaThreads + (int)threadIdx.x < tot;
        int lo = 0, hi = kDeltaThreads;  // last block with pre[block] <= f
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if ((int)pre[mid] <= f) lo = mid; else hi = mid;
        }
        const int64_t at = (int64_t)(b0 + lo) * kSortChunk + (f - (int)pre[lo]);
        tok[u] = min(max(moved[(int64_t)h * N + min(at, (int64_t)N - 1)], 0), N - 1);
      }
      uint32_t jn[U], jo[U];
      float v8[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        jn[u] = ah[tok[u]];
        jo[u] = ph[tok[u]];
        rv.template load8_n<NSUB>(h, tok[u], k0, v8[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u] || jn[u] >= (uint32_t)Cp || jo[u] >= (uint32_t)Cp) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const long long q = to_units((double)v8[u][e], lm[e]);
          atomicAdd(&acc[jn[u] * kDeltaRow + e], (unsigned long long)q);
          atomicAdd(&acc[jo[u] * kDeltaRow + e], (unsigned long long)(-q));
        }
      }
    }
    __syncthreads();  // pre and wsum are rewritten by the next pass
  }
  if (!any) return;  // uniform: nothing moved
#pragma unroll
  for (int r = 0; r < QS; ++r) {
    const int q = r * kDeltaThreads + (int)threadIdx.x;
    if (q < Cp * 8)
      dst[(int64_t)(q >> 3) * D + (q & 7)] = old[r] + (long long)acc[(q >> 3) * kDeltaRow + (q & 7)];
  }
}

// The incremental update on its own (stages with more than three earlier
// stages, whose chunk sums keep 256-thread workgroups).
template <typename Tin, int D, int NSUB>
__global__ __launch_bounds__(kDeltaThreads) void k_delta(
    ResView<Tin> rv, int H, int Cp, const uint8_t *__restrict__ assign, int64_t assign_hstride,
    const uint8_t *__restrict__ prev, int par, const int32_t *__restrict__ moved,
    const uint32_t *__restrict__ mcnt, int nb, const uint32_t *__restrict__ lminv,
    long long *__restrict__ isum, const uint32_t *__restrict__ stats, int stat_stride) {
  delta_body<Tin, D, NSUB>(rv, H, Cp, assign, assign_hstride, prev, par, moved, mcnt, nb, lminv,
                           isum, stats, stat_stride, blockIdx.x);
}

// The accumulate launch of the iterations after a stage's first (stages with
// at most three earlier stages): workgroups 0 .. H*gx-1 sum the member chunks
// of heads updated in full (8 waves, one chunk each, as k_chunk_sum),
// workgroups from doff (a multiple of 8, so that the XCD of a delta workgroup
// follows its id) update the others from their moved tokens.
template <typename Tin, int D, int NSUB>
__global__ __launch_bounds__(kDeltaThreads) void k_accum_delta(
    ResView<Tin> rv, int H, int Cp, const int32_t *__restrict__ sorted,
    const int32_t *__restrict__ offs, const int32_t *__restrict__ cofs,
    const int32_t *__restrict__ chunk_j, int maxch, double *__restrict__ part,
    uint32_t *__restrict__ pflag, int gx, int doff, const uint8_t *__restrict__ assign,
    int64_t assign_hstride, const uint8_t *__restrict__ prev, int par,
    const uint32_t *__restrict__ mcnt, int nb, const uint32_t *__restrict__ lminv,
    long long *__restrict__ isum, uint32_t *stats, int stat_stride) {
  const int bid = blockIdx.x;
  if (bid < gx * H) {
    const int h = bid / gx, g = (bid % gx) * (kDeltaThreads / 64) + (int)(threadIdx.x >> 6);
    if (head_incremental(stats, stat_stride, h)) return;
    if (bid % gx == 0 && threadIdx.x == 0) stats[(int64_t)h * stat_stride + S_ISUM] = 1u;
    if (head_sums_exact(stats, stat_stride, h))
      chunk_sum_body<Tin, D, NSUB, false>(rv, Cp, sorted, offs, cofs, chunk_j, maxch, part,
                                          pflag, h, g);
    else
      chunk_sum_body<Tin, D, NSUB, true>(rv, Cp, sorted, offs, cofs, chunk_j, maxch, part,
                                         pflag, h, g);
  } else if (bid >= doff) {
    delta_body<Tin, D, NSUB>(rv, H, Cp, assign, assign_hstride, prev, par, sorted, mcnt, nb,
                             lminv, isum, stats, stat_stride, bid - doff);
  }
}

template <typename Tin, typename Tc, int D>
__global__ __launch_bounds__(256) void k_finalize(
    ResView<Tin> rv, const int32_t *__restrict__ sorted, const uint32_t *__restrict__ pflag,
    int C, int Cp, const int32_t *__restrict__ offs, const int32_t *__restrict__ cofs, int maxch,
    const double *__restrict__ part, float *__restrict__ cent, const uint32_t *stats,
    uint32_t *stats_w, int stat_stride, int bslot, half8 *__restrict__ ctab,
    float *__restrict__ cinit, float4 *__restrict__ cbnd, Tc *__restrict__ rec_c,
    int64_t rec_hstride, float *__restrict__ cache, int64_t cache_hstride,
    long long *__restrict__ isum, const uint32_t *__restrict__ lminv,
    const uint32_t *__restrict__ hist, int nb) {
  constexpr int PER = D / 64;
  const int h = blockIdx.y;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= Cp) return;
  if (j >= C) {
    if (ctab) emit_pad<D>(h, j, Cp, ctab, cinit, cbnd);
    return;
  }
  const bool head_exact = head_sums_exact(stats, stat_stride, h);
  // with the incremental state (isum set): a head updated incrementally in
  // this iteration (k_accum_delta) reads its integer sums; a head updated in
  // full whose sums fit the integers stores them for the iterations after, or
  // marks them unusable when a cluster had to be summed again in token order
  // (that sum may have rounded)
  const bool from_isum = isum && head_incremental(stats, stat_stride, h);
  long long *isj = isum ? isum + ((int64_t)h * Cp + j) * D + lane * PER : nullptr;
  const uint32_t *lmj = lminv ? lminv + (int64_t)h * D + lane * PER : nullptr;
  double s[PER];
  int n;
  if (from_isum) {
    // member count: the column of this iteration's per-chunk histograms
    uint32_t c = 0u;
    for (int b = lane; b < nb; b += 64) c += hist[((int64_t)h * nb + b) * kMaxC + j];
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    n = (int)__builtin_amdgcn_readfirstlane(c);
#pragma unroll
    for (int m = 0; m < PER; ++m) s[m] = from_units(isj[m], lmj[m]);
  } else {
  n = __builtin_amdgcn_readfirstlane(offs[(int64_t)h * (Cp + 1) + j + 1] -
                                     offs[(int64_t)h * (Cp + 1) + j]);
  const int c0 = __builtin_amdgcn_readfirstlane(cofs[(int64_t)h * (Cp + 1) + j]);
  const int nch = __builtin_amdgcn_readfirstlane(cofs[(int64_t)h * (Cp + 1) + j + 1]) - c0;
  const double *ph = part + ((int64_t)h * maxch + c0) * D + lane * PER;
  const uint32_t *pf = pflag + ((int64_t)h * maxch + c0) * D + lane * PER;
  int emax[PER], lmin[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) s[m] = 0.0, emax[m] = 0, lmin[m] = 0xFFFF;
  for (int q = 0; q < nch; q += 8) {
    double v[8][PER];
    uint32_t f[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        v[u][m] = ph[(int64_t)min(q + u, nch - 1) * D + m];
        f[u][m] = head_exact ? 0u : pf[(int64_t)min(q + u, nch - 1) * D + m];
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q + u < nch)
#pragma unroll
        for (int m = 0; m < PER; ++m) {
          s[m] = __dadd_rn(s[m], v[u][m]);
          emax[m] = max(emax[m], (int)(f[u][m] & 0xFFFFu));
          lmin[m] = min(lmin[m], (int)(f[u][m] >> 16));
        }
  }
  // Some partial sum might round: sum the cluster again, sequentially in
  // token order (rare; members are read 32 at a time, added one by one).
  const int lg = n > 1 ? 32 - __builtin_clz((uint32_t)(n - 1)) : 0;
  bool risky = false;
#pragma unroll
  for (int m = 0; m < PER; ++m) risky |= !head_exact && emax[m] - lmin[m] + lg > 29;
  if (__ballot(risky)) {
    const int o0 = __builtin_amdgcn_readfirstlane(offs[(int64_t)h * (Cp + 1) + j]);
    const int32_t *ids = sorted + (int64_t)h * rv.N + o0;
#pragma unroll
    for (int m = 0; m < PER; ++m) s[m] = 0.0;
    for (int q = 0; q < n; q += 32) {
      const int32_t myid = ids[min(q + (lane & 31), n - 1)];
      float v[32][PER];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int64_t row = __builtin_amdgcn_readlane(myid, u);
#pragma unroll
        for (int m = 0; m < PER; ++m) v[u][m] = rv.get(h, row, lane * PER + m);
      }
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (q + u < n)
#pragma unroll
          for (int m = 0; m < PER; ++m) s[m] = __dadd_rn(s[m], (double)v[u][m]);
    }
  }
  if (isum && head_int_sums(stats, stat_stride, h, rv.N)) {
    if (__ballot(risky)) {
      if (lane == 0) stats_w[(int64_t)h * stat_stride + S_ISUM] = 0u;
    } else {
#pragma unroll
      for (int m = 0; m < PER; ++m) isj[m] = to_units(s[m], lmj[m]);
    }
  }
  }
  float *cj = cent + ((int64_t)h * Cp + j) * D + lane * PER;
  float cv[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    cv[m] = n > 0 ? (float)(s[m] / (double)n) : cj[m];
    cj[m] = cv[m];
  }
  if (ctab) {
    const uint32_t *st = stats + (int64_t)h * stat_stride;
    const float sc = ldexpf(1.0f, -scale_exp(fmaxf(stat_f(st, S_MAXR), stat_f(st, S_MAXC))));
    emit_tables<D>(h, j, Cp, cv, sc, ctab, cinit, cbnd, stats_w + (int64_t)h * stat_stride + bslot);
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
#define QVG_CHECK_LAUNCH() \
  do { if (hipGetLastError() != hipSuccess) return false; } while (0)

namespace {
// Compute units of the current device (cached per device id).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Raise a kernel's dynamic LDS limit once per process.
bool allow_lds(const void *fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) ==
         hipSuccess;
}
}  // namespace

bool launch_sample_rows(int H, int T, int N, int C, uint64_t seed, int32_t *idx, hipStream_t s) {
  TimerScope ts_("kmeans_init", s);
  hipLaunchKernelGGL(k_sample, dim3(T, H), dim3(64), 0, s, N, C, T, seed, idx);
  QVG_CHECK_LAUNCH();
  return true;
}

bool launch_stage_bound(uint32_t *prev_stats, int stat_stride, int H, hipStream_t s) {
  TimerScope ts_("kmeans_init", s);
  hipLaunchKernelGGL(k_stage_bound, dim3((H + 63) / 64), dim3(64), 0, s, prev_stats,
                     stat_stride, H);
  QVG_CHECK_LAUNCH();
  return true;
}

template <typename Tin>
bool launch_absmax(const void *x, int H, int64_t per_head, uint32_t *stats, int stat_stride,
                   int slot, hipStream_t s) {
  const int64_t blocks = (per_head / 8 + 255) / 256;
  dim3 grid((unsigned)std::min<int64_t>(blocks, 64), H);
  TimerScope ts_("absmax", s);
  hipLaunchKernelGGL(k_absmax<Tin>, grid, dim3(256), 0, s, (const Tin *)x, per_head, stats,
                     stat_stride, slot);
  QVG_CHECK_LAUNCH();
  return true;
}

template <typename T>
ResView<T> view_of(const KmArgs &a, int D) {
  ResView<T> v;
  v.x = (const T *)a.x;
  v.pi = a.rec_pi;
  v.cent = (const T *)a.rec_cent;
  v.N = a.N;
  v.D = D;
  v.dlog2 = __builtin_ctz(D);
  v.C = a.C;
  v.Ts = a.Ts;
  v.nsub = a.nsub;
  return v;
}

template <typename Tin, int D>
bool launch_kmeans_stage_begin(const KmArgs &a, hipStream_t s) {
  const ResView<Tin> rv = view_of<Tin>(a, D);
  dim3 gc((a.Cp + 3) / 4, a.H);
  {
    TimerScope ts_("kmeans_init", s);
    hipLaunchKernelGGL((k_init<Tin, D>), gc, dim3(256), 0, s, rv, a.idx,
                       a.idx_hstride, a.init, a.init_hstride, a.C, a.Cp, a.ws.cent, a.ws_stats,
                       a.stat_stride);
    QVG_CHECK_LAUNCH();
  }
  {
    const int64_t threads = (int64_t)a.NT * kTile * (D / 8);
    dim3 gp((unsigned)((threads + 255) / 256), a.H);
    TimerScope ts_("kmeans_prepare", s);
    dispatch_nsub(a.nsub, [&]<int NS>() {
      hipLaunchKernelGGL((k_prepare<Tin, D, NS>), gp, dim3(256), 0, s, rv, a.NT, a.ws_stats,
                         a.stat_stride, a.ws.rt, a.ws.tb);
    });
    QVG_CHECK_LAUNCH();
  }
  {
    TimerScope ts_("kmeans_tables", s);
    hipLaunchKernelGGL((k_tables<D>), gc, dim3(256), 0, s, a.ws.cent, a.C, a.Cp, a.ws_stats,
                       a.ws_stats, a.stat_stride, (int)S_B0, a.ws.ctab, a.ws.cinit, a.ws.cbnd);
    QVG_CHECK_LAUNCH();
  }
  return true;
}

template <typename Tin, int D>
bool launch_assign(const KmArgs &a, int bslot, hipStream_t s) {
  const ResView<Tin> rv = view_of<Tin>(a, D);
  constexpr int KC = D / 16, TPG = 16;
  const int CB = a.Cp / kTile;
  const size_t lds = (size_t)CB * KC * 64 * sizeof(half8) + (size_t)CB * 32 * sizeof(float) +
                     (size_t)a.Cp * sizeof(float4);
  static bool attr_assign = allow_lds((const void *)k_assign<D>, 96 * 1024);
  if (!attr_assign) return false;
  const int groups_per_head = (a.NT + TPG - 1) / TPG;
  const int total = groups_per_head * a.H;
  const int target = 2 * cu_count();
  const int per_wg = (total + target - 1) / target;
  const int grid = (total + per_wg - 1) / per_wg;
  {
    TimerScope ts_("kmeans_assign", s);
    hipLaunchKernelGGL((k_assign<D>), dim3(grid), dim3(512), lds, s, a.ws.rt, a.ws.tb,
                       a.ws.ctab, a.ws.cinit, a.ws.cbnd, a.ws_stats, a.stat_stride, bslot, a.N,
                       a.NT, CB, groups_per_head, total, per_wg, a.assign, a.assign_hstride,
                       a.ws.recheck, a.ws.fallback, a.ws.stage_re, a.ws.stage_fb, a.ws.counters,
                       a.kappa);
    QVG_CHECK_LAUNCH();
  }
  {
    TimerScope ts_("kmeans_resolve", s);
    // every workgroup resident at once (four per CU at <= 128 VGPRs), so that
    // the scan and re-check workgroups run concurrently
    hipLaunchKernelGGL((k_resolve<Tin, D>), dim3(4 * cu_count()), dim3(256), 0, s, rv, a.ws.cent, a.C,
                       a.Cp, a.ws.recheck, a.ws.fallback, a.ws.counters, a.assign,
                       a.assign_hstride);
    QVG_CHECK_LAUNCH();
  }
  return true;
}

template <typename Tin, typename Tc, int D>
bool launch_update(const KmArgs &a, int next_bslot, bool tables, Tc *rec_c, int64_t rec_hstride,
                   float *cache, int64_t cache_hstride, int log_slot, int iter, hipStream_t s) {
  // after the first iteration of a stage (with the incremental state), each
  // head is updated either from its changed tokens (k_accum_delta) or in full (sort
  // and chunk sums), as k_scatter decides from its exactness and moved count
  const bool inc = a.ws.isum != nullptr && iter >= 0;
  const bool delta = inc && iter > 0;
  const int par = iter > 0 ? iter & 1 : 0;
  const int nb = (a.N + kSortChunk - 1) / kSortChunk;
  const int maxch = max_chunks(a.N, a.Cp);
  // the iterations after a stage's first are timed as one unit, kmeans_delta
  // (their heads may take either update)
  {
    TimerScope ts_(delta ? "kmeans_delta" : "kmeans_sort", s);
    hipLaunchKernelGGL(k_hist, dim3(nb, a.H), dim3(256), 0, s, a.assign, a.assign_hstride, a.N,
                       a.ws.hist, a.ws_stats, a.stat_stride, next_bslot, a.ws.counters, log_slot,
                       inc ? a.ws.prev : nullptr, par, delta ? 1 : 0, a.ws.sorted, a.ws.mcnt);
    QVG_CHECK_LAUNCH();
    hipLaunchKernelGGL(k_scatter, dim3(nb, a.H), dim3(256), 0, s, a.assign, a.assign_hstride,
                       a.N, a.Cp, a.ws.hist, a.ws.sorted, a.ws.offs, a.ws.cofs, a.ws.chunk_j,
                       maxch, a.ws_stats, a.stat_stride, delta ? 1 : 0, a.ws.mcnt);
    QVG_CHECK_LAUNCH();
  }
  {
    TimerScope ts_(delta ? "kmeans_delta" : "kmeans_accumulate", s);
    if (delta && a.nsub <= 3) {
      const int gx = (maxch + kDeltaThreads / 64 - 1) / (kDeltaThreads / 64);
      const int doff = (gx * a.H + 7) / 8 * 8;
      dispatch_nsub(a.nsub, [&]<int NS>() {
        if constexpr (NS <= 3)
          hipLaunchKernelGGL((k_accum_delta<Tin, D, NS>), dim3(doff + delta_grid(a.H, D)),
                             dim3(kDeltaThreads), 0, s, view_of<Tin>(a, D), a.H, a.Cp,
                             a.ws.sorted, a.ws.offs, a.ws.cofs, a.ws.chunk_j, maxch, a.ws.part,
                             a.ws.pflag, gx, doff, a.assign, a.assign_hstride, a.ws.prev, par,
                             a.ws.mcnt, nb, a.ws.lminv, a.ws.isum, a.ws_stats, a.stat_stride);
      });
      QVG_CHECK_LAUNCH();
    } else {
      const dim3 gcs((maxch + 3) / 4, a.H);
#define QVG_CS(NS)                                                                           \
  hipLaunchKernelGGL((k_chunk_sum<Tin, D, NS>), gcs, dim3(256), 0, s, view_of<Tin>(a, D), a.Cp, \
                     a.ws.sorted, a.ws.offs, a.ws.cofs, a.ws.chunk_j, maxch, a.ws.part,      \
                     a.ws.pflag, a.ws_stats, a.stat_stride)
      switch (a.nsub) {
        case 0: QVG_CS(0); break;
        case 1: QVG_CS(1); break;
        case 2: QVG_CS(2); break;
        case 3: QVG_CS(3); break;
        case 4: QVG_CS(4); break;
        case 5: QVG_CS(5); break;
        case 6: QVG_CS(6); break;
        default: QVG_CS(7); break;
      }
#undef QVG_CS
      QVG_CHECK_LAUNCH();
      if (iter == 0) {
        hipLaunchKernelGGL((k_span_part<D>), dim3(kSpanParts, a.H), dim3(256), 0, s, a.ws.pflag,
                           a.ws.cofs, a.Cp, maxch, a.ws.span);
        QVG_CHECK_LAUNCH();
        hipLaunchKernelGGL((k_span_final<D>), dim3(a.H), dim3(D), 0, s, a.ws.span, a.N,
                           a.ws_stats, a.stat_stride, inc ? a.ws.lminv : nullptr);
        QVG_CHECK_LAUNCH();
      }
      if (delta) {
        dispatch_nsub(a.nsub, [&]<int NS>() {
          hipLaunchKernelGGL((k_delta<Tin, D, NS>), dim3(delta_grid(a.H, D)),
                             dim3(kDeltaThreads), 0, s, view_of<Tin>(a, D), a.H, a.Cp, a.assign,
                             a.assign_hstride, a.ws.prev, par, a.ws.sorted, a.ws.mcnt, nb,
                             a.ws.lminv, a.ws.isum, a.ws_stats, a.stat_stride);
        });
        QVG_CHECK_LAUNCH();
      }
    }
    hipLaunchKernelGGL((k_finalize<Tin, Tc, D>), dim3((a.Cp + 3) / 4, a.H), dim3(256), 0, s,
                       view_of<Tin>(a, D), a.ws.sorted, a.ws.pflag, a.C, a.Cp, a.ws.offs,
                       a.ws.cofs, maxch, a.ws.part, a.ws.cent, a.ws_stats, a.ws_stats,
                       a.stat_stride, next_bslot, tables ? a.ws.ctab : nullptr, a.ws.cinit,
                       a.ws.cbnd, rec_c, rec_hstride, cache, cache_hstride,
                       inc ? a.ws.isum : nullptr, inc ? a.ws.lminv : nullptr, a.ws.hist, nb);
    QVG_CHECK_LAUNCH();
  }
  return true;
}

#define QVG_INST(Tin, D)                                                                      \
  template bool launch_kmeans_stage_begin<Tin, D>(const KmArgs &, hipStream_t);               \
  template bool launch_assign<Tin, D>(const KmArgs &, int, hipStream_t);                      \
  template bool launch_update<Tin, float, D>(const KmArgs &, int, bool, float *, int64_t,     \
                                             float *, int64_t, int, int, hipStream_t);       \
  template bool launch_update<Tin, uint16_t, D>(const KmArgs &, int, bool, uint16_t *,        \
                                                int64_t, float *, int64_t, int, int,          \
                                                hipStream_t);
QVG_INST(float, 64)
QVG_INST(float, 128)
QVG_INST(uint16_t, 64)
QVG_INST(uint16_t, 128)
template bool launch_absmax<float>(const void *, int, int64_t, uint32_t *, int, int, hipStream_t);
template bool launch_absmax<uint16_t>(const void *, int, int64_t, uint32_t *, int, int,
                                      hipStream_t);

}  // namespace qvg
