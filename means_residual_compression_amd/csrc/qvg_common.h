// Internal definitions shared by the QVG HIP kernels and host code (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qvg {

constexpr int kMaxC = 256;  // assignments are uint8
constexpr int kMaxT = 8;
constexpr int kTile = 32;   // tokens (and centroids) per 32x32 MFMA tile
constexpr int kSortChunk = 1024; // tokens per block of the counting sort
constexpr int kAccChunk = 64;    // cluster members per partial sum of the update
constexpr int kCounterLog = 64;  // iterations whose candidate counts are kept
constexpr int kCounterWords = 4 + 2 * kCounterLog;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Per-head statistics, one row of kStatWords uint32 per (head, stage).
// Non-negative floats are stored as their bit patterns so that integer
// atomicMax is an order-independent (deterministic) float max.
enum StatSlot : int {
  S_MAXR = 0,    // max |r| over the stage's input residual
  S_MAXC = 1,    // max |c| over the stage's initial centroids
  S_B0 = 2,      // bounds of the current centroid table, double-buffered:
                 // [2 + 4*p + 0] max ||c*sc||, [+1] max ||c*sc - fp16(c*sc)||,
                 // [+2] max ||fp16(c*sc)||, [+3] max ||c*sc||^2
  S_SPAN = 10,   // exactness of the stage's centroid sums over the whole head:
                 // bit 0 set once checked, bit 1 when some channel's span
                 // leaves a partial sum of up to N members able to round
  S_INC = 11,    // 1 when this iteration's update of the head is incremental
  S_SPANW = 12,  // the stage's widest channel span, max over channels of emax - lmin
  S_ISUM = 13,   // 1 while the head's integer sums are exact (no cluster of its last
                 // full update had to be summed again in token order)
  kStatWords = 16,
};

// Device scratch carved from the caller's workspace.
struct Ws {
  half8 *rt;          // fp16 fragments [H][NT][KC][64] of the scaled residual
  float2 *tb;         // [H][NT*32]        per-token (||r~||, ||r*sc - r~||) bounds
  float *cent;        // fp32 [H][Cp][d]   working centroids
  half8 *ctab;        // fp16 fragments [H][CB][KC][64] of the scaled centroids
  float *cinit;       // fp32 [H][CB][2][16] accumulator init -||c*sc||^2 / 2
  float4 *cbnd;       // [H][Cp] per-centroid bounds (||c*sc||, ||c*sc - c~||, ||c~||, ||c*sc||^2)
  uint32_t *stats;    // [H][T'][kStatWords]
  int4 *recheck;      // [H*NT*32] (head, token, j1, j2)
  int2 *fallback;     // [H*NT*32] (head, token)
  uint32_t *counters; // [kCounterWords]: 0 recheck entries, 1 fallback entries of
                      // the running assign; 4 + 2k (+1): counts of iteration k
  int32_t *sorted;    // [H][N] token ids grouped by cluster, token order inside
  int32_t *offs;      // [H][Cp+1] cluster segment offsets into `sorted`
  uint32_t *hist;     // [H][ceil(N/kSortChunk)][256] per-chunk cluster counts
  int32_t *cofs;      // [H][Cp+1] first member-chunk of each cluster
  int32_t *chunk_j;   // [H][max_chunks] cluster of each member-chunk
  double *part;       // [H][max_chunks][d] fp64 partial sums of member-chunks
  uint32_t *pflag;    // [H][max_chunks][d] per chunk and channel: max exponent | min lowest-bit << 16
  int4 *stage_re;     // [H*(NT+15)*32] recheck entries staged per assign workgroup
  int2 *stage_fb;     // [H*(NT+15)*32] fallback entries staged per assign workgroup
  uint32_t *span;     // [H][kSpanParts][D] per-channel emax | lmin << 16 of chunk groups
  int32_t *idx;       // [H][T][C] device copy of the seeded init indices
  // Incremental update of heads whose stage sums are exact (null: always the
  // full update).
  long long *isum;    // [H][Cp][D] cluster sums as integers, units 2^(lmin - 150)
  uint32_t *lminv;    // [H][D] per-channel lowest-bit bound lmin of the stage residual
  uint8_t *prev;      // [2][H][N] assignments at the last two updates (iteration parity)
  uint32_t *mcnt;     // [H][ceil(N/kSortChunk)] moved tokens listed by each sort block
};

constexpr int kSpanParts = 32;  // chunk groups per head in the span reduction

__host__ __device__ inline int pad32(int x) { return (x + 31) & ~31; }
// Upper bound on member-chunks per head: every cluster adds at most one
// partially filled chunk.
__host__ __device__ inline int max_chunks(int N, int Cp) {
  return (N + kAccChunk - 1) / kAccChunk + Cp;
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
// Round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float get(const float *p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void put(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float get(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ static __forceinline__ void put(uint16_t *p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// Load 8 consecutive elements starting at p[i] (i multiple of 8) as fp32.
__device__ __forceinline__ void load8(const float *p, int64_t i, float v[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p + i);
  const float4 b = *reinterpret_cast<const float4 *>(p + i + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t *p, int64_t i, float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4 *>(p + i);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    v[2 * m] = __uint_as_float(w[m] << 16);
    v[2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void store8(float *p, int64_t i, const float v[8]) {
  *reinterpret_cast<float4 *>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4 *>(p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
// Round-to-nearest-even fp32 -> bf16 with gfx950's v_cvt_pk_bf16_f32 (two
// values per instruction); fp32 stores are unchanged.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  const bf16x2_t r = __builtin_convertvector((floatx2_t){a, b}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}
__device__ __forceinline__ void store8(uint16_t *p, int64_t i, const float v[8]) {
  *reinterpret_cast<uint4 *>(p + i) = make_uint4(pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]),
                                                 pack_bf16_rne(v[4], v[5]), pack_bf16_rne(v[6], v[7]));
}
// The same as non-temporal stores: for streamed output that no later kernel
// of the pass reads, so it does not displace cached data on its way out.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store8_stream(uint16_t *p, const float v[8]) {
  const u32x4_t w = {pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]), pack_bf16_rne(v[4], v[5]),
                     pack_bf16_rne(v[6], v[7])};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(p));
}
__device__ __forceinline__ void store8_stream(float *p, const float v[8]) {
  const u32x4_t a = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  const u32x4_t b = {__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
  __builtin_nontemporal_store(a, reinterpret_cast<u32x4_t *>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<u32x4_t *>(p + 4));
}

// ------------------------------------------------------- stage residuals
// The input residual of stage t, recomputed on the fly from the stage-0
// input X and the record:  R(t) = X - C(1)[pi(1)] - ... - C(t)[pi(t)], one fp32
// subtraction per stage in stage order (the same arithmetic as subtracting
// stage by stage).  nsub = t; pi and cent are the record's assignments
// [H][Ts][N] and centroids [H][Ts][C][D] (rounded to the record dtype T).
template <typename T>
struct ResView {
  const T *x;
  const uint8_t *pi;
  const T *cent;
  int N, D, C, Ts, nsub;
  int dlog2;  // log2(D): D is 64 or 128, so row offsets are shifts

  __device__ __forceinline__ int stage_j(int h, int s, int64_t i) const {
    return min((int)pi[((int64_t)h * Ts + s) * N + i], C - 1);
  }
  // Row j of stage s of head h: a per-(head, stage) base (uniform) plus a
  // 32-bit row offset (j < 256).
  __device__ __forceinline__ const T *stage_row(int h, int s, int j) const {
    return cent + (((int64_t)h * Ts + s) * C << dlog2) + ((uint32_t)j << dlog2);
  }
  // Element offset of row i of head h of x.
  __device__ __forceinline__ int64_t xrow(int h, int64_t i) const {
    return ((int64_t)h * N + i) << dlog2;
  }
  __device__ __forceinline__ float get(int h, int64_t i, int k) const {
    float v = Elem<T>::get(x, xrow(h, i) + k);
    for (int s = 0; s < nsub; ++s) v = v - Elem<T>::get(stage_row(h, s, stage_j(h, s, i)), k);
    return v;
  }
  __device__ __forceinline__ void load8(int h, int64_t i, int k0, float v[8]) const {
    ::qvg::load8(x, xrow(h, i) + k0, v);
    for (int s = 0; s < nsub; ++s) {
      float c[8];
      ::qvg::load8(stage_row(h, s, stage_j(h, s, i)), k0, c);
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = v[m] - c[m];
    }
  }
  // Same with the stage count fixed at compile time (branch-free, so the
  // loads of all stages are issued together).
  template <int NSUB>
  __device__ __forceinline__ void load8_n(int h, int64_t i, int k0, float v[8]) const {
    int js[NSUB > 0 ? NSUB : 1];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) js[s] = stage_j(h, s, i);
    float c[NSUB > 0 ? NSUB : 1][8];
    ::qvg::load8(x, xrow(h, i) + k0, v);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) ::qvg::load8(stage_row(h, s, js[s]), k0, c[s]);
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = v[m] - c[s][m];
  }
};

// Calls F.template operator()<NS>() with NS = n (0..8) as a compile-time value.
template <typename F>
inline void dispatch_nsub(int n, F &&f) {
  switch (n) {
    case 0: f.template operator()<0>(); break;
    case 1: f.template operator()<1>(); break;
    case 2: f.template operator()<2>(); break;
    case 3: f.template operator()<3>(); break;
    case 4: f.template operator()<4>(); break;
    case 5: f.template operator()<5>(); break;
    case 6: f.template operator()<6>(); break;
    case 7: f.template operator()<7>(); break;
    default: f.template operator()<8>(); break;
  }
}

// -------------------------------------------------------------- FP8 E4M3
// OCP E4M3 ("e4m3fn"): 4 exponent bits (bias 7), 3 mantissa bits, largest
// finite 448.  Encode s >= 0 with round-to-nearest-even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  if (!(s < 464.0f)) return 0x7Eu;  // >= 464 (and the tie at 464) -> 448
  if (s < 0.015625f) {              // below 2^-6: subnormal grid m * 2^-9
    return (uint32_t)__builtin_rintf(s * 512.0f);  // 0..8; 8 is 2^-6 (code 8)
  }
  const uint32_t u = __float_as_uint(s);
  // keep 3 mantissa bits with round-to-nearest-even (carries into the exponent)
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
  return r - ((127u - 7u) << 3);
}
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Branch-free decode of a non-negative E4M3 code: placing the 7 code bits at
// fp32 bit 20 gives 2^(e-127)(1 + m/8) for e > 0 and the fp32 subnormal
// m * 2^-129 for e = 0; scaling by 2^120 (exact) yields 2^(e-7)(1 + m/8) and
// m * 2^-9 respectively.  Needs fp32 subnormals preserved (the default).
__device__ __forceinline__ float e4m3_decode_bits(uint32_t c) {
  return __uint_as_float((c & 0x7Fu) << 20) * 0x1p120f;
}

// Power-of-two exponent e such that values up to `m` scaled by 2^-e stay
// below 2^14 (well inside fp16 range).
__device__ __forceinline__ int scale_exp(float m) {
  if (!(m > 0.0f)) return 0;
  return ilogbf(m) - 13;
}

__device__ __forceinline__ float stat_f(const uint32_t *s, int slot) {
  return __uint_as_float(s[slot]);
}

}  // namespace qvg
