// Attention of a few queries over a compressed history.  Per token and head
// the kernel reads only the packed codes, the FP8 scales and the T
// assignment bytes of K and of V (plus centroid rows, which stay in L2); the
// reconstructed keys and values are never written to HBM.
//
// note.zhuruihan.top "Algorithm-System Co-design" (dequantization fused into
// the kernels that consume the cache); paper.rainbus.top novelty paragraph
// and the howistudyai.com explainer, "Required resources" (keys are cached
// before the rotary position embedding, which is applied after
// reconstruction); paper.rainbus.top method paragraph, DQ (the
// reconstruction level * s_hat + C(T)[pi(T)] + ... + C(1)[pi(1)]).
//
// Keys are rebuilt bit for bit as qvg_decompress rebuilds them in bf16 and
// rotated (rotate-half form, fp32 products and difference/sum, then bf16).
// Values enter unrounded, in one of two ways:
//  * weight sums (up to kAttnSumQueries queries, Nq*T*C <= kAttnSumEntries):
//    sum_n p_n V_n = sum_n p_n (level*s_hat)_n + sum_t sum_c W_t[c] C(t)[c]
//    with W_t[c] the summed weights of the tokens assigned to c at stage t.
//    Only the residual level*s_hat (exact in bf16) is staged per token; W
//    lives in LDS and is contracted with the tables once per head at the end.
//  * rebuilt values: level*s_hat + stage rows in fp32 (the dequant's
//    arithmetic without the bf16 rounding), staged per token.
//
// k_attn_split: one workgroup per (head, run of consecutive 64-token tiles).
// Per tile it (1) stages the keys and the value rows in LDS; (2) scores every
// query against every token in fp32 (one wave per query group, one lane per
// token) and folds the tile into a running softmax per query: a reference
// maximum m, raised (with the factor e^(m_old - m_new) applied to everything
// accumulated) only when a tile's maximum exceeds it by more than
// kLazyRescale; (3) accumulates the un-normalised output, one thread per
// (channel, half or quarter of the tile), and with weight sums adds each
// token's weight to W_t[pi_t] (wave w owns the stages t = w mod 4, so every
// slot has one writer and a fixed order).  At the end of its run it writes
// (m, l, o[d], W) per query.  k_attn_contract merges W over the runs and
// contracts it with the value tables; k_attn_combine merges the runs.
//
// Summation order (for error bounds): an output element of one run is a
// fused multiply-add chain over the tokens a thread owns (32 or 16 per tile,
// d = 128 or 64), rescaled at most once per tile, then the 2 or 4 thread
// parts are added, then the runs are combined with one more multiply-add
// chain.  A weight sum is a chain of adds over the run's tokens assigned to
// its slot (rescaled at most once per tile), combined over runs with a
// multiply-add chain, then contracted with the table rows in 2048/d row
// ranges of T*C*d/2048 rows each, the ranges added in order.
#include "qvg_common.h"
#include "qvg_attn.h"
#include "qvg_internal.h"

namespace qvg {

namespace {

__device__ __forceinline__ float bf16f(uint32_t b) { return __uint_as_float(b << 16); }

// First-level loads of one item (token ti, channel groups [k0, k0+8) and
// [k1, k1+8)) of one record: the two code words, the two scale bytes and the
// assignment bytes of stages T-1 .. T-4 (those that exist).
struct RawItem {
  uint32_t w0, w1, e0, e1;
  uint32_t j[4];
};

template <int D>
__device__ __forceinline__ void load_raw(const AttnRec &r, int h, int N, int64_t ti, int k0, int k1,
                                         int glog2, RawItem &w) {
  const int64_t row = (int64_t)h * N + ti;
  if (r.bits == 2) {
    const uint16_t *c = reinterpret_cast<const uint16_t *>(r.codes + row * (D / 4));
    w.w0 = c[k0 >> 3];
    w.w1 = c[k1 >> 3];
  } else {
    const uint32_t *c = reinterpret_cast<const uint32_t *>(r.codes + row * (D / 2));
    w.w0 = c[k0 >> 3];
    w.w1 = c[k1 >> 3];
  }
  const uint8_t *sc = r.scales + (row << (__builtin_ctz(D) - glog2));
  w.e0 = sc[k0 >> glog2];
  w.e1 = sc[k1 >> glog2];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    w.j[u] = u < r.T ? r.assign[((int64_t)h * r.T + (r.T - 1 - u)) * N + ti] : 0u;
}

// Centroid rows of 8 channels as loaded (bf16 pairs or fp32), unpacked at use.
template <typename Tc> struct Row8;
template <> struct Row8<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
  __device__ __forceinline__ void get(float f[8]) const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f[2 * m] = __uint_as_float(w[m] << 16);
      f[2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
    }
  }
};
template <> struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ __forceinline__ void get(float f[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// Gathers of stages T-1 .. T-4 for both channel groups of an item.
template <typename Tc, int D>
__device__ __forceinline__ void gather4(const AttnRec &r, int h, int k0, int k1, const RawItem &w,
                                        Row8<Tc> ga[4], Row8<Tc> gb[4]) {
  const Tc *cent = static_cast<const Tc *>(r.cent);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u < r.T) {
      const int j = min((int)w.j[u], r.C - 1);
      const Tc *crow = cent + (((int64_t)h * r.T + (r.T - 1 - u)) * r.C + j) * D;
      ga[u].load(crow + k0);
      gb[u].load(crow + k1);
    }
  }
}

// The item's 16 channels, rebuilt as the fused dequant rebuilds them: level
// (2q - L) times the decoded scale plus the stage-T centroid in one fused
// multiply-add (the product is exact), then + C(t)[pi(t)] for t = T-1..1,
// each an fp32 add.
// Signed levels 2q - L of the 8 codes of a code word, from the byte tables
// (lut2: a byte's 4 INT2 levels; lut4: a byte's 2 INT4 levels).
__device__ __forceinline__ void levels8(uint32_t w, int bits, const float4 *lut2,
                                        const float2 *lut4, float v[8]) {
  if (bits == 2) {
    const float4 x = lut2[w & 0xFFu], y = lut2[(w >> 8) & 0xFFu];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float2 x = lut4[(w >> (8 * m)) & 0xFFu];
      v[2 * m] = x.x;
      v[2 * m + 1] = x.y;
    }
  }
}

template <typename Tc, int D>
__device__ __forceinline__ void rebuild(const AttnRec &r, int h, int N, int64_t ti, int k0, int k1,
                                        const RawItem &w, const Row8<Tc> ga[4],
                                        const Row8<Tc> gb[4], const float4 *lut2,
                                        const float2 *lut4, float a[8], float b[8]) {
  const float s0 = e4m3_decode_bits(w.e0), s1 = e4m3_decode_bits(w.e1);
  levels8(w.w0, r.bits, lut2, lut4, a);
  levels8(w.w1, r.bits, lut2, lut4, b);
  if (r.T == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = a[e] * s0;
      b[e] = b[e] * s1;
    }
    return;
  }
  float ca[8], cb[8];
  ga[0].get(ca);
  gb[0].get(cb);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = __builtin_fmaf(a[e], s0, ca[e]);
    b[e] = __builtin_fmaf(b[e], s1, cb[e]);
  }
#pragma unroll
  for (int u = 1; u < 4; ++u) {
    if (u < r.T) {
      ga[u].get(ca);
      gb[u].get(cb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = a[e] + ca[e];
        b[e] = b[e] + cb[e];
      }
    }
  }
  // stages below T-4 (T > 4), one at a time
  const Tc *cent = static_cast<const Tc *>(r.cent);
  for (int t = r.T - 5; t >= 0; --t) {
    const int j = min((int)r.assign[((int64_t)h * r.T + t) * N + ti], r.C - 1);
    const Tc *crow = cent + (((int64_t)h * r.T + t) * r.C + j) * D;
    Row8<Tc> x, y;
    x.load(crow + k0);
    y.load(crow + k1);
    x.get(ca);
    y.get(cb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = a[e] + ca[e];
      b[e] = b[e] + cb[e];
    }
  }
}

// Rotary embedding, rotate-half form, on bf16 inputs x (channel k) and y
// (channel k + d/2): x' = x c - y s, y' = y c + x s with each product and the
// difference/sum rounded to fp32 separately, then each result to bf16.
__device__ __forceinline__ void rotate8(const float x[8], const float y[8], const float c[8],
                                        const float s[8], uint32_t xo[4], uint32_t yo[4]) {
#pragma clang fp contract(off)
  float xr[8], yr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xc = x[e] * c[e], ys = y[e] * s[e], yc = y[e] * c[e], xs = x[e] * s[e];
    xr[e] = xc - ys;
    yr[e] = yc + xs;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    xo[m] = pack_bf16_rne(xr[2 * m], xr[2 * m + 1]);
    yo[m] = pack_bf16_rne(yr[2 * m], yr[2 * m + 1]);
  }
}

__device__ __forceinline__ void unpack8(const uint32_t w[4], float v[8]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    v[2 * m] = bf16f(w[m] & 0xFFFFu);
    v[2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
  }
}

// bf16 rounding (RNE) of x, as the fp32 value: v_cvt_pk_bf16_f32 of (0, x)
// leaves bf16(x) in the high half and zero in the low half.
__device__ __forceinline__ float round_bf16(float x) {
  return __uint_as_float(pack_bf16_rne(0.0f, x));
}

__device__ __forceinline__ void pack8(const float v[8], uint32_t w[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) w[m] = pack_bf16_rne(v[2 * m], v[2 * m + 1]);
}

__device__ __forceinline__ void st16(uint16_t *p, const uint32_t w[4]) {
  *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

constexpr float kLazyRescale = 8.0f;  // weights stay below e^8 between rescales

template <typename Tc, int D, int NQ, bool SUMS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NQ == 16 ? 2 : 3)))
void k_attn_split(const float *__restrict__ q, int Nq, int N, int H, AttnRec kr, AttnRec vr,
                  float scale, const float *__restrict__ rcos, const float *__restrict__ rsin,
                  int nsplit, int tiles_per_split, int pf, float *__restrict__ part) {
  constexpr int BN = kAttnBN, RS = D + 8, RSF = D + 4, HD = D / 2, NG = D / 16;
  constexpr int P = 256 / D, TPP = BN / P;  // output thread parts, tokens each
  constexpr int QW = NQ >= 4 ? NQ / 4 : 1, NW = NQ >= 4 ? 4 : NQ;  // queries per wave, waves
  constexpr int NIT = BN * NG / 256;                                 // rebuild items per thread
  extern __shared__ float4 smem_a[];
  float4 *lut2 = smem_a;                                   // [256] INT2 levels of a byte
  float2 *lut4 = reinterpret_cast<float2 *>(lut2 + 256);   // [256] INT4 levels of a byte
  uint16_t *kt = reinterpret_cast<uint16_t *>(lut4 + 256); // [BN][RS] keys
  // values: the residuals level * s_hat ([BN][RS] bf16, exact) with weight
  // sums, else the rebuilt values ([BN][RSF] fp32)
  uint16_t *vh = kt + BN * RS;
  float *vf = reinterpret_cast<float *>(kt + BN * RS);
  float *qs = SUMS ? reinterpret_cast<float *>(vh + BN * RS) : vf + BN * RSF;  // [NQ][D]
  float *ps = qs + NQ * D;   // [NQ][BN] tile weights
  float *st = ps + NQ * BN;  // [NQ][4] reference max, sum, rescale factor
  float *ws = st + 4 * NQ;   // weight sums [Nq][T][C]

  // XCD-aware order: workgroups dispatch round-robin over the 8 XCDs, and
  // each XCD takes a contiguous range of items.  Items run group-major (heads
  // in groups of ceil(H/8)), then run, then head within the group: an XCD
  // works on a few heads at a time (their centroid rows stay in its L2), all
  // at the same runs of tokens (the rotary rows they share are fetched once),
  // and the XCDs move through the tokens together.
  const int total = H * nsplit, wg = blockIdx.x, xcd = wg & 7, slot = wg >> 3;
  const int base = total >> 3, rem = total & 7;
  const int item = xcd * base + min(xcd, rem) + slot;
  const int HG = (H + 7) >> 3;
  const int grp = item / (HG * nsplit), r0 = item - grp * HG * nsplit;
  const int gh = min(HG, H - grp * HG);
  const int sp = r0 / gh, h = grp * HG + (r0 - sp * gh);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int kg = __builtin_ctz(kr.G), vg = __builtin_ctz(vr.G);
  const int TC = vr.T * vr.C;
  AttnRec vq = vr;
  if (SUMS) vq.T = 0;  // the residual only: no assignment bytes, no rows

  // byte -> levels tables (blockDim.x == 256: one entry per thread)
  lut2[t] = make_float4((float)(2 * (t & 3) - 3), (float)(2 * ((t >> 2) & 3) - 3),
                        (float)(2 * ((t >> 4) & 3) - 3), (float)(2 * ((t >> 6) & 3) - 3));
  lut4[t] = make_float2((float)(2 * (t & 15) - 15), (float)(2 * ((t >> 4) & 15) - 15));
  for (int x = t; x < NQ * D; x += 256) qs[x] = x < Nq * D ? q[(int64_t)h * Nq * D + x] : 0.0f;
  if (t < NQ) {
    st[4 * t] = -__builtin_inff();
    st[4 * t + 1] = 0.0f;
    st[4 * t + 2] = 0.0f;
  }
  if (SUMS)
    for (int x = t; x < Nq * TC; x += 256) ws[x] = 0ull;
  float o[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) o[j] = 0.0f;
  const int ntiles = (N + BN - 1) / BN;
  const int tb = sp * tiles_per_split, te = min(tb + tiles_per_split, ntiles);
  const int ko = t % D, kp = t / D;  // output role: channel, token part
  __syncthreads();

  for (int tile = tb; tile < te; ++tile) {
    const int64_t i0 = (int64_t)tile * BN;
    const int nt = (int)min((int64_t)BN, (int64_t)N - i0);
    // (1) stage: item = (token, channel pair-group g): channels g*8.. and
    // d/2 + g*8..; tokens past the end repeat the last one.  All first-level
    // loads of the tile go out first, then each item's K gathers (with its
    // rotary rows), then its values.
    RawItem rk[NIT], rv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int w = t + 256 * it, i = w / NG, g = w - i * NG;
      const int64_t ti = i0 + min(i, nt - 1);
      load_raw<D>(kr, h, N, ti, g * 8, HD + g * 8, kg, rk[it]);
      load_raw<D>(vq, h, N, ti, g * 8, HD + g * 8, vg, rv[it]);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int w = t + 256 * it, i = w / NG, g = w - i * NG;
      const int64_t ti = i0 + min(i, nt - 1);
      const int k0 = g * 8, k1 = HD + g * 8;
      Row8<Tc> ga[4], gb[4];
      gather4<Tc, D>(kr, h, k0, k1, rk[it], ga, gb);
      float c[8], sn[8];
      if (rcos) {
        load8(rcos + ti * HD, k0, c);
        load8(rsin + ti * HD, k0, sn);
      }
      float a[8], b[8];
      uint32_t wa[4], wb[4];
      rebuild<Tc, D>(kr, h, N, ti, k0, k1, rk[it], ga, gb, lut2, lut4, a, b);
      pack8(a, wa);
      pack8(b, wb);
      if (rcos) {
        unpack8(wa, a);
        unpack8(wb, b);
        rotate8(a, b, c, sn, wa, wb);
      }
      st16(kt + i * RS + k0, wa);
      st16(kt + i * RS + k1, wb);
      __builtin_amdgcn_sched_barrier(0);  // keep the value loads out of the key phase's registers
      if constexpr (SUMS) {
        rebuild<Tc, D>(vq, h, N, ti, k0, k1, rv[it], ga, gb, lut2, lut4, a, b);  // level * s_hat
        pack8(a, wa);  // exact: at most 8 significant bits
        pack8(b, wb);
        st16(vh + i * RS + k0, wa);
        st16(vh + i * RS + k1, wb);
      } else {
        gather4<Tc, D>(vr, h, k0, k1, rv[it], ga, gb);
        rebuild<Tc, D>(vr, h, N, ti, k0, k1, rv[it], ga, gb, lut2, lut4, a, b);
        store8(vf, i * RSF + k0, a);
        store8(vf, i * RSF + k1, b);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // (2) scores and the running softmax: wave w owns queries w, w+4, ...;
    // lane = token; tokens past the end score -inf (weight 0)
    if (wave < NW) {
      float s[QW];
#pragma unroll
      for (int j = 0; j < QW; ++j) s[j] = 0.0f;
      const uint16_t *krow = kt + lane * RS;
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 8) {
        const uint4 kw = *reinterpret_cast<const uint4 *>(krow + k0);
        const uint32_t ww[4] = {kw.x, kw.y, kw.z, kw.w};
        float kf[8];
        unpack8(ww, kf);
#pragma unroll
        for (int j = 0; j < QW; ++j) {
          const float4 qa = *reinterpret_cast<const float4 *>(qs + (wave + 4 * j) * D + k0);
          const float4 qb = *reinterpret_cast<const float4 *>(qs + (wave + 4 * j) * D + k0 + 4);
          s[j] = __builtin_fmaf(qa.x, kf[0], s[j]);
          s[j] = __builtin_fmaf(qa.y, kf[1], s[j]);
          s[j] = __builtin_fmaf(qa.z, kf[2], s[j]);
          s[j] = __builtin_fmaf(qa.w, kf[3], s[j]);
          s[j] = __builtin_fmaf(qb.x, kf[4], s[j]);
          s[j] = __builtin_fmaf(qb.y, kf[5], s[j]);
          s[j] = __builtin_fmaf(qb.z, kf[6], s[j]);
          s[j] = __builtin_fmaf(qb.w, kf[7], s[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < QW; ++j) {
        const int qq = wave + 4 * j;
        const float sc = lane < nt ? s[j] * scale : -__builtin_inff();
        float mt = sc;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
        const float m_ref = st[4 * qq];
        const bool raise = mt > m_ref + kLazyRescale;  // always on the first tile
        const float m_new = raise ? mt : m_ref;
        const float alpha = raise ? __expf(m_ref - m_new) : 1.0f;
        const float p = __expf(sc - m_new);
        float sum = p;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        ps[qq * BN + lane] = p;
        if (lane == 0) {
          st[4 * qq] = m_new;
          st[4 * qq + 1] = __builtin_fmaf(st[4 * qq + 1], alpha, sum);
          st[4 * qq + 2] = alpha;
        }
      }
    }
    __syncthreads();
    // (3) output: thread = (channel ko, token part kp)
#pragma unroll
    for (int j = 0; j < NQ; ++j) o[j] = o[j] * st[4 * j + 2];
    const float *pw = ps + kp * TPP;
#pragma unroll 2
    for (int i = 0; i < TPP; i += 4) {
      const int r = kp * TPP + i;
      float v0, v1, v2, v3;
      if constexpr (SUMS) {
        const uint16_t *vc = vh + r * RS + ko;
        v0 = bf16f(vc[0]);
        v1 = bf16f(vc[RS]);
        v2 = bf16f(vc[2 * RS]);
        v3 = bf16f(vc[3 * RS]);
      } else {
        const float *vc = vf + r * RSF + ko;
        v0 = vc[0];
        v1 = vc[RSF];
        v2 = vc[2 * RSF];
        v3 = vc[3 * RSF];
      }
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const float4 pj = *reinterpret_cast<const float4 *>(pw + j * BN + i);
        o[j] = __builtin_fmaf(pj.x, v0, o[j]);
        o[j] = __builtin_fmaf(pj.y, v1, o[j]);
        o[j] = __builtin_fmaf(pj.z, v2, o[j]);
        o[j] = __builtin_fmaf(pj.w, v3, o[j]);
      }
    }
    if constexpr (SUMS) {
      // weight sums: wave w owns stages w, w+4, ...; lane = token
      const int64_t ti = i0 + min(lane, nt - 1);
      for (int ts = wave; ts < vr.T; ts += 4) {
        const int c = min((int)vr.assign[((int64_t)h * vr.T + ts) * N + ti], vr.C - 1);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          if (j >= Nq) break;
          float *wq = ws + (j * vr.T + ts) * vr.C;
          const float al = st[4 * j + 2];
          if (al != 1.0f)
            for (int cc = lane; cc < vr.C; cc += 64) wq[cc] *= al;
          if (lane < nt) atomicAdd(wq + c, ps[j * BN + lane]);
        }
      }
    }
    __syncthreads();
  }

  // merge the token parts in a fixed order, write (m, l, o[], W) per query
  float *oh = reinterpret_cast<float *>(kt);  // [P-1][NQ][D], over the staged rows
  if (kp > 0) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) oh[((kp - 1) * NQ + j) * D + ko] = o[j];
  }
  __syncthreads();
  float *rec = part + ((int64_t)h * nsplit + sp) * Nq * pf;
  if (kp == 0) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (j >= Nq) break;
      float r = o[j];
#pragma unroll
      for (int p2 = 1; p2 < P; ++p2) r += oh[((p2 - 1) * NQ + j) * D + ko];
      float *dst = rec + j * pf;
      dst[2 + ko] = r;
      if (ko == 0) {
        dst[0] = st[4 * j];
        dst[1] = st[4 * j + 1];
      }
    }
  }
  if (SUMS)
    for (int x = t; x < Nq * TC; x += 256) {
      const int j = x / TC;
      rec[j * pf + 2 + D + (x - j * TC)] = ws[x];
    }
}

// Largest run maximum m_b of one (head, query): blockDim.x threads load the
// runs' maxima in parallel, then reduce through `red` (blockDim.x floats).
__device__ __forceinline__ float runs_max(const float *p, int64_t stride, int nsplit, float *red) {
  float m = -__builtin_inff();
  for (int b = threadIdx.x; b < nsplit; b += blockDim.x) m = fmaxf(m, p[b * stride]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();  // red may be written again by the caller
  return r;
}

// Weight-sum term, cut into kContractParts row ranges (one workgroup each):
// with M the largest run maximum and w_b = e^(m_b - M), each range's rows r
// get W[r] = sum_b w_b W_b[r] (merged in run order) and its share of
// sum_r W[r] C[r][k] goes to cpart[h][q][z][k]; 256/d threads per channel
// take consecutive sub-ranges, added in order.
constexpr int kContractParts = 8;

template <typename Tc>
__global__ __launch_bounds__(256) void k_attn_contract(const float *__restrict__ part, int nsplit,
                                                       int Nq, int D, int pf, AttnRec vr,
                                                       float *__restrict__ cpart) {
  __shared__ float wl[2048 / kContractParts];  // T*C <= 2048
  __shared__ float red[256];
  __shared__ float wb[kAttnMaxSplit];            // w_b per run
  const int qq = blockIdx.x, h = blockIdx.y, z = blockIdx.z, t = threadIdx.x;
  const int64_t stride = (int64_t)Nq * pf;
  const float *p = part + ((int64_t)h * nsplit * Nq + qq) * pf;
  const float M = runs_max(p, stride, nsplit, red);
  for (int b = t; b < nsplit; b += 256) wb[b] = __expf(p[b * stride] - M);
  __syncthreads();
  const int TC = vr.T * vr.C;
  const int r0 = z * TC / kContractParts, r1 = (z + 1) * TC / kContractParts, n = r1 - r0;
  for (int r = t; r < n; r += 256) {
    float acc = 0.0f;
    for (int b0 = 0; b0 < nsplit; b0 += 8) {  // 8 loads in flight, added in run order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[min(b0 + u, nsplit - 1) * stride + 2 + D + r0 + r];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b0 + u < nsplit) acc = __builtin_fmaf(v[u], wb[b0 + u], acc);
    }
    wl[r] = acc;
  }
  __syncthreads();
  const int k = t % D, kp = t / D, np = 256 / D;
  const int a0 = kp * n / np, a1 = (kp + 1) * n / np;
  const Tc *cent = static_cast<const Tc *>(vr.cent) + ((size_t)h * TC + r0) * D;
  float acc = 0.0f;
#pragma unroll 8
  for (int r = a0; r < a1; ++r) {
    float c;
    if constexpr (sizeof(Tc) == 2)
      c = __uint_as_float((uint32_t)cent[(size_t)r * D + k] << 16);
    else
      c = cent[(size_t)r * D + k];
    acc = __builtin_fmaf(wl[r], c, acc);
  }
  red[t] = acc;
  __syncthreads();
  if (kp == 0) {
    float o = 0.0f;
    for (int j2 = 0; j2 < np; ++j2) o += red[j2 * D + k];
    cpart[(((int64_t)h * Nq + qq) * kContractParts + z) * D + k] = o;
  }
}

// Merges the runs of each (query, head): with M the largest run maximum and
// w_b = e^(m_b - M), O = (sum_b w_b o_b + the weight-sum term) / sum_b w_b l_b,
// the weight-sum term (with weight sums only) being the contraction parts
// added in order.
template <bool SUMS>
__global__ __launch_bounds__(128) void k_attn_combine(const float *__restrict__ part, int nsplit,
                                                      int Nq, int D, int pf,
                                                      const float *__restrict__ cpart,
                                                      float *__restrict__ out) {
  __shared__ float red[128];
  const int qq = blockIdx.x, h = blockIdx.y, k = threadIdx.x;
  const int64_t stride = (int64_t)Nq * pf;
  const float *p = part + ((int64_t)h * nsplit * Nq + qq) * pf;
  const float M = runs_max(p, stride, nsplit, red);
  if (k >= D) return;
  float l = 0.0f, o = 0.0f;
  for (int b0 = 0; b0 < nsplit; b0 += 8) {  // 8 runs' loads in flight, merged in run order
    float m[8], lb[8], ob[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t b = min(b0 + u, nsplit - 1) * stride;
      m[u] = p[b];
      lb[u] = p[b + 1];
      ob[u] = p[b + 2 + k];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (b0 + u < nsplit) {
        const float w = __expf(m[u] - M);
        l = __builtin_fmaf(lb[u], w, l);
        o = __builtin_fmaf(ob[u], w, o);
      }
  }
  if (SUMS) {
    const float *cp = cpart + ((int64_t)h * Nq + qq) * kContractParts * D + k;
    for (int z = 0; z < kContractParts; ++z) o += cp[z * D];
  }
  out[((int64_t)h * Nq + qq) * D + k] = o / l;
}

// ------------------------------------------------------------- two passes
// With bf16 centroid tables, keys of 1 to 4 stages and weight sums (up to
// 16 queries, kAttnSumQueries at a time), the attention takes two passes
// over the records instead of k_attn_split:
//  * k_attn_scores (keys only, one query): a workgroup takes a run of tokens
//    for a group of heads (score_group).  Eight lanes per token (d = 128;
//    four for d = 64), each holding 8 rotate-half channel pairs (channels
//    k .. k+7 and d/2 + k ..), rebuild the key in registers as k_attn_split
//    does, rotate it and take its product with the query in a chain of 16
//    fused multiply-adds; butterfly adds give all lanes of the token the
//    same score, which is scaled and written to the scratch.  A lane loads
//    its token's rotary rows once and keeps them while it scores the token
//    for every head of the group.  Only the level tables and the queries go
//    through LDS, and every wave scores its own tokens.
//    k_attn_scores_mq does the same for 2 to 16 queries on the matrix cores.
//  * k_attn_values1 (one query) and k_attn_values_mq (up to
//    kAttnSumQueries per launch): with m the run's largest score (read back
//    from the scores), every weight is p_n = e^(s_n - m), so no running
//    maximum is kept and nothing is rescaled.  The residual term
//    sum_n (p_n s_hat_n) level_n is accumulated in registers (fused
//    multiply-add chains for one query, matrix-core products otherwise);
//    each token's weight, rounded to a multiple of 2^-40, is added to
//    W_t[pi_t(n)] in LDS as a 64-bit integer (integer LDS atomics are an
//    order of magnitude faster than float ones here, and integer sums do not
//    depend on the order of the adds).  The run's (m, l, o, W) record, W
//    converted back to fp32 once, is merged by k_attn_contract and
//    k_attn_combine.
// Summation orders are given with each kernel; a weight sum of a run is
// exact in units of 2^-40 (each weight within 2^-41 of its unit multiple),
// rounded once to fp32.

// Workgroup -> (head, run), XCD-aware as in k_attn_split.
__device__ __forceinline__ void attn_item(int H, int nsplit, int &h, int &sp) {
  const int total = H * nsplit, wg = blockIdx.x, xcd = wg & 7, slot = wg >> 3;
  const int base = total >> 3, rem = total & 7;
  const int item = xcd * base + min(xcd, rem) + slot;
  const int HG = (H + 7) >> 3;
  const int grp = item / (HG * nsplit), r0 = item - grp * HG * nsplit;
  const int gh = min(HG, H - grp * HG);
  sp = r0 / gh;
  h = grp * HG + (r0 - sp * gh);
}

// Code words of GPT consecutive groups of 8 channels starting at channel k of
// a record row (16 bits per group for INT2, 32 for INT4).
template <int BITS, int GPT>
__device__ __forceinline__ void load_codes(const uint8_t *rowp, int k, uint32_t w[GPT]) {
  const uint8_t *p = rowp + k * BITS / 8;
  if constexpr (BITS == 2 && GPT == 2) {
    const uint32_t x = *reinterpret_cast<const uint32_t *>(p);
    w[0] = x & 0xFFFFu;
    w[1] = x >> 16;
  } else if constexpr (BITS == 2) {
    w[0] = *reinterpret_cast<const uint16_t *>(p);
  } else if constexpr (GPT == 2) {
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    w[0] = x.x;
    w[1] = x.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t *>(p);
  }
}

template <int BITS>
__device__ __forceinline__ void init_level_lut(float4 *lut2, float2 *lut4) {
  const int t = threadIdx.x;  // blockDim.x == 256
  if constexpr (BITS == 2)
    lut2[t] = make_float4((float)(2 * (t & 3) - 3), (float)(2 * ((t >> 2) & 3) - 3),
                          (float)(2 * ((t >> 4) & 3) - 3), (float)(2 * ((t >> 6) & 3) - 3));
  else
    lut4[t] = make_float2((float)(2 * (t & 15) - 15), (float)(2 * ((t >> 4) & 15) - 15));
}

// Heads per scores workgroup: half of them (at most 32, and at most 32 KB of
// queries in LDS).  Each token's rotary rows are then read by the XCDs
// of two groups, and an XCD's L2 holds the tables of one group; smaller
// groups re-read the rotary rows on more XCDs, larger ones lose the tables
// from L2 (measured on the decode-side records: 5, 10, 20 and 40 heads per
// group fetch 1.69, 1.36, 1.29 and 1.26 GB and take 663, 654, 655 and 708 us).
__host__ __device__ inline int score_group(int H, int NQ, int D) {
  const int cap = 8192 / (NQ * D) < 32 ? 8192 / (NQ * D) : 32;
  return (H + 1) / 2 < cap ? (H + 1) / 2 : cap;
}

// The rebuilt key channels x (a) and their rotate-half partners y (b) as
// bf16 operand words: each rounded to bf16, then (with rotation) x c - y s
// and y c + x s from fp32 products and an fp32 difference/sum, rounded to
// bf16 in the packing.
__device__ __forceinline__ void rotate_pack(float a[8], float b[8], bool rot, const float c[8],
                                            const float sn[8], uint32_t wa[4], uint32_t wb[4]) {
  if (rot) {
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = round_bf16(a[e]), y = round_bf16(b[e]);
      const float xc = x * c[e], ys = y * sn[e], yc = y * c[e], xs = x * sn[e];
      a[e] = xc - ys;
      b[e] = yc + xs;
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    wa[m] = pack_bf16_rne(a[2 * m], a[2 * m + 1]);
    wb[m] = pack_bf16_rne(b[2 * m], b[2 * m + 1]);
  }
}

// Scores: workgroup -> (group of heads, run of tiles), consecutive items on
// one XCD.  A lane keeps its token's rotary rows in registers while it
// scores the token for every head of the group.
template <int D, int NQ, int KT, int BITS>
__global__ __launch_bounds__(256) void k_attn_scores(const float *__restrict__ q, int Nq, int N,
                                                     int H, AttnRec kr, float scale,
                                                     const float *__restrict__ rcos,
                                                     const float *__restrict__ rsin, int nsplit,
                                                     int tps, float *__restrict__ scores) {
  constexpr int HD = D / 2, LPT = D / 16;  // lanes per token: 8 pair positions each
  constexpr int TB = 256 / LPT;            // tokens per workgroup pass
  __shared__ float4 lut2[BITS == 2 ? 256 : 1];
  __shared__ float2 lut4[BITS == 4 ? 256 : 1];
  extern __shared__ float qs[];  // [gh][NQ][D] queries of the group's heads
  const int HG = score_group(H, NQ, D), ngroups = (H + HG - 1) / HG;
  const int total = ngroups * nsplit, wg = blockIdx.x, xcd = wg & 7, slot = wg >> 3;
  const int item = xcd * (total >> 3) + min(xcd, total & 7) + slot;
  const int grp = item / nsplit, sp = item - grp * nsplit;
  const int h0 = grp * HG, gh = min(HG, H - h0);
  const int t = threadIdx.x;
  const int part = t % LPT, tok = t / LPT;
  const int ka = part * 8, kb = HD + part * 8;  // this lane's channels ka.., kb..
  init_level_lut<BITS>(lut2, lut4);
  for (int x = t; x < gh * NQ * D; x += 256) {
    const int hq = x / D, k = x - hq * D, hh = hq / NQ, jq = hq - hh * NQ;
    qs[x] = jq < Nq ? q[((int64_t)(h0 + hh) * Nq + jq) * D + k] : 0.0f;
  }
  __syncthreads();
  const int C = kr.C, kg = __builtin_ctz(kr.G);
  const int ntiles = (N + kAttnBN - 1) / kAttnBN;
  const int t0 = sp * tps * kAttnBN, t1 = min(min(sp * tps + tps, ntiles) * kAttnBN, N);
  const char *rc = reinterpret_cast<const char *>(rcos), *rs = reinterpret_cast<const char *>(rsin);
  // First-level loads of one (pass, head) step: code words, scale bytes and
  // assignment bytes of this lane's token (tokens past the run repeat its
  // last one).  Head bases are uniform, lane offsets 32-bit (the launcher
  // keeps every offset below 2^32 bytes).
  struct Raw {
    uint32_t wa, wb, ea, eb, j[KT];
  };
  auto fetch = [&](int b0, int h, Raw &r) {
    const uint32_t ti = (uint32_t)min(b0 + tok, t1 - 1);
    const uint8_t *crow = kr.codes + (int64_t)h * N * (D * BITS / 8) + ti * (uint32_t)(D * BITS / 8);
    load_codes<BITS, 1>(crow, ka, &r.wa);
    load_codes<BITS, 1>(crow, kb, &r.wb);
    const uint8_t *scl = kr.scales + ((int64_t)h * N << (__builtin_ctz(D) - kg));
    const uint32_t so = ti << (__builtin_ctz(D) - kg);
    r.ea = scl[so + (ka >> kg)];
    r.eb = scl[so + (kb >> kg)];
    const uint8_t *asg = kr.assign + (int64_t)h * KT * N;
#pragma unroll
    for (int u = 0; u < KT; ++u) r.j[u] = asg[(uint32_t)(KT - 1 - u) * (uint32_t)N + ti];  // u = 0: last stage
  };
  Raw cur;
  fetch(t0, h0, cur);
  float c[8], sn[8];
  int b0 = t0, hh = 0;       // this step
  int nb0 = t0, nhh = 0;     // the next step
  while (b0 < t1) {
    if (++nhh == gh) nhh = 0, nb0 += TB;
    const int h = h0 + hh;
    const uint32_t ti = (uint32_t)min(b0 + tok, t1 - 1);
    // this step's table rows (and, for the group's first head, the token's
    // rotary rows) go out first, then the next step's first-level loads,
    // which stay in flight while this step computes
    Row8<uint16_t> ga[KT], gb[KT];
    const char *cent = reinterpret_cast<const char *>(static_cast<const uint16_t *>(kr.cent) +
                                                      (int64_t)h * KT * C * D);
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      const uint32_t ju = min(cur.j[u], (uint32_t)C - 1);
      const uint32_t off = (((uint32_t)(KT - 1 - u) * (uint32_t)C + ju) * D + ka) * 2u;
      ga[u].load(reinterpret_cast<const uint16_t *>(cent + off));
      gb[u].load(reinterpret_cast<const uint16_t *>(cent + off + HD * 2));
    }
    if (rcos && hh == 0) {
      const uint32_t ro = (ti * HD + ka) * 4u;
      load8(reinterpret_cast<const float *>(rc + ro), 0, c);
      load8(reinterpret_cast<const float *>(rs + ro), 0, sn);
    }
    Raw nx;
    fetch(min(nb0, t1 - 1), h0 + nhh, nx);
    float a[8], b[8], ca[8], cb[8];
    levels8(cur.wa, BITS, lut2, lut4, a);
    levels8(cur.wb, BITS, lut2, lut4, b);
    const float s0 = e4m3_decode_bits(cur.ea), s1 = e4m3_decode_bits(cur.eb);
    ga[0].get(ca);
    gb[0].get(cb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = __builtin_fmaf(a[e], s0, ca[e]);
      b[e] = __builtin_fmaf(b[e], s1, cb[e]);
    }
#pragma unroll
    for (int u = 1; u < KT; ++u) {
      ga[u].get(ca);
      gb[u].get(cb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = a[e] + ca[e];
        b[e] = b[e] + cb[e];
      }
    }
    // the bf16 key, rotated (fp32 products and difference/sum, then bf16)
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = round_bf16(a[e]), b[e] = round_bf16(b[e]);
    if (rcos) {
#pragma clang fp contract(off)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xc = a[e] * c[e], ys = b[e] * sn[e], yc = b[e] * c[e], xs = a[e] * sn[e];
        a[e] = round_bf16(xc - ys);
        b[e] = round_bf16(yc + xs);
      }
    }
    const bool valid = b0 + tok < t1;
    const float *qh = qs + hh * NQ * D;
#pragma unroll
    for (int jq = 0; jq < NQ; ++jq) {
      float qa[8], qb[8];
      load8(qh + jq * D, ka, qa);
      load8(qh + jq * D, kb, qb);
      float v = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) v = __builtin_fmaf(qa[e], a[e], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v = __builtin_fmaf(qb[e], b[e], v);
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) v = v + __shfl_xor(v, off);
      v = v * scale;
      if (part == 0 && valid && jq < Nq) scores[((int64_t)h * Nq + jq) * N + ti] = v;
    }
    cur = nx;
    b0 = nb0;
    hh = nhh;
  }
}

// Scores of 2 to 16 queries on the matrix cores (v_mfma_f32_16x16x32_bf16):
// the same workgroups, runs and head groups as k_attn_scores, but a wave
// step covers 16 tokens with four lanes per token.  Lane l holds token
// l % 16 and, in each 32-channel block kb, channels kb*32 + 8*(l/16) .. +7,
// which is the B-operand layout of the instruction; a rotate-half partner
// (k + d/2) lies in block kb + d/64 of the same lane.  The lane rebuilds its
// d/4 key channels with k_attn_scores' arithmetic, rotates them and packs
// the bf16 results straight into operands.  Each query is split into two
// bf16 parts (hi = bf16(q), lo = bf16(q - hi), so |q - hi - lo| <= 2^-16 |q|),
// kept in LDS in A-operand layout; 2 d/32 products give a 16 x 16 tile of
// (query, token) scores in fp32, scaled and written like k_attn_scores'.
template <int D, int KT, int BITS>
__global__ __launch_bounds__(256) void k_attn_scores_mq(const float *__restrict__ q, int Nq, int N,
                                                        int H, AttnRec kr, float scale,
                                                        const float *__restrict__ rcos,
                                                        const float *__restrict__ rsin, int nsplit,
                                                        int tps, float *__restrict__ scores) {
  constexpr int HD = D / 2, KB = D / 32, HKB = KB / 2;
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float floatx4_t __attribute__((ext_vector_type(4)));
  __shared__ float4 lut2[BITS == 2 ? 256 : 1];
  __shared__ float2 lut4[BITS == 4 ? 256 : 1];
  extern __shared__ uint4 qop[];  // [gh][2 parts][KB][64 lanes] A operands
  const int HG = score_group(H, kAttnMaxQueries, D), ngroups = (H + HG - 1) / HG;
  const int total = ngroups * nsplit, wg = blockIdx.x, xcd = wg & 7, slot = wg >> 3;
  const int item = xcd * (total >> 3) + min(xcd, total & 7) + slot;
  const int grp = item / nsplit, sp = item - grp * nsplit;
  const int h0 = grp * HG, gh = min(HG, H - h0);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int tok = wave * 16 + (lane & 15);  // token of the 64-token step
  const int c0 = (lane >> 4) * 8;           // channel offset within each block
  init_level_lut<BITS>(lut2, lut4);
  // the queries as two bf16 parts in A-operand layout: lane l of block kb
  // holds query l % 16, channels kb*32 + 8*(l/16) .. +7 (zero past Nq)
  for (int x = t; x < gh * KB * 64; x += 256) {
    const int hh = x / (KB * 64), r = x - hh * (KB * 64), kb = r >> 6, ln = r & 63;
    const int i = ln & 15, k = kb * 32 + (ln >> 4) * 8;
    float v[8];
    if (i < Nq) {
      load8(q + ((int64_t)(h0 + hh) * Nq + i) * D, k, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      hi[m] = pack_bf16_rne(v[2 * m], v[2 * m + 1]);
      const float r0 = v[2 * m] - __uint_as_float(hi[m] << 16);  // exact
      const float r1 = v[2 * m + 1] - __uint_as_float(hi[m] & 0xFFFF0000u);
      lo[m] = pack_bf16_rne(r0, r1);
    }
    qop[((hh * 2 + 0) * KB + kb) * 64 + ln] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    qop[((hh * 2 + 1) * KB + kb) * 64 + ln] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  __syncthreads();
  const int C = kr.C, kg = __builtin_ctz(kr.G);
  const int ntiles = (N + kAttnBN - 1) / kAttnBN;
  const int t0 = sp * tps * kAttnBN, t1 = min(min(sp * tps + tps, ntiles) * kAttnBN, N);
  const char *rc = reinterpret_cast<const char *>(rcos), *rs = reinterpret_cast<const char *>(rsin);
  // First-level loads of one (pass, head) step, as in k_attn_scores.
  struct Raw {
    uint32_t w[KB], e[KB], j[KT];
  };
  auto fetch = [&](int b0, int h, Raw &r) {
    const uint32_t ti = (uint32_t)min(b0 + tok, t1 - 1);
    const uint8_t *crow = kr.codes + (int64_t)h * N * (D * BITS / 8) + ti * (uint32_t)(D * BITS / 8);
    const uint8_t *scl = kr.scales + ((int64_t)h * N << (__builtin_ctz(D) - kg));
    const uint32_t so = ti << (__builtin_ctz(D) - kg);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      load_codes<BITS, 1>(crow, kb * 32 + c0, &r.w[kb]);
      r.e[kb] = scl[so + ((kb * 32 + c0) >> kg)];
    }
    const uint8_t *asg = kr.assign + (int64_t)h * KT * N;
#pragma unroll
    for (int u = 0; u < KT; ++u) r.j[u] = asg[(uint32_t)(KT - 1 - u) * (uint32_t)N + ti];  // u = 0: last stage
  };
  Raw cur;
  fetch(t0, h0, cur);
  float c[HKB][8], sn[HKB][8];
  int b0 = t0, hh = 0;
  int nb0 = t0, nhh = 0;
  while (b0 < t1) {
    if (++nhh == gh) nhh = 0, nb0 += kAttnBN;
    const int h = h0 + hh;
    const uint32_t ti = (uint32_t)min(b0 + tok, t1 - 1);
    const char *cent = reinterpret_cast<const char *>(static_cast<const uint16_t *>(kr.cent) +
                                                      (int64_t)h * KT * C * D);
    uint32_t kop[KB][4];  // the lane's rotated bf16 key channels, B operands
    Raw nx;
#pragma unroll
    for (int hb = 0; hb < HKB; ++hb) {
      // channels hb*32 + c0 .. (x) and their partners d/2 later (y): the
      // table rows (and, for the group's first head, the rotary rows) go out
      // first; after the last half's, the next step's first-level loads,
      // which stay in flight while this step computes
      Row8<uint16_t> ga[KT], gb[KT];
#pragma unroll
      for (int u = 0; u < KT; ++u) {
        const uint32_t ju = min(cur.j[u], (uint32_t)C - 1);
        const uint32_t off = (((uint32_t)(KT - 1 - u) * (uint32_t)C + ju) * D + hb * 32 + c0) * 2u;
        ga[u].load(reinterpret_cast<const uint16_t *>(cent + off));
        gb[u].load(reinterpret_cast<const uint16_t *>(cent + off + HD * 2));
      }
      if (rcos && hh == 0) {
        const uint32_t ro = (ti * HD + hb * 32 + c0) * 4u;
        load8(reinterpret_cast<const float *>(rc + ro), 0, c[hb]);
        load8(reinterpret_cast<const float *>(rs + ro), 0, sn[hb]);
      }
      if (hb == HKB - 1) fetch(min(nb0, t1 - 1), h0 + nhh, nx);
      float a[8], b[8], ca[8], cb[8];
      levels8(cur.w[hb], BITS, lut2, lut4, a);
      levels8(cur.w[hb + HKB], BITS, lut2, lut4, b);
      const float s0 = e4m3_decode_bits(cur.e[hb]), s1 = e4m3_decode_bits(cur.e[hb + HKB]);
      ga[0].get(ca);
      gb[0].get(cb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = __builtin_fmaf(a[e], s0, ca[e]);
        b[e] = __builtin_fmaf(b[e], s1, cb[e]);
      }
#pragma unroll
      for (int u = 1; u < KT; ++u) {
        ga[u].get(ca);
        gb[u].get(cb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a[e] = a[e] + ca[e];
          b[e] = b[e] + cb[e];
        }
      }
      rotate_pack(a, b, rcos != nullptr, c[hb], sn[hb], kop[hb], kop[hb + HKB]);
    }
    cur = nx;
    // 16 queries x 16 tokens: the hi parts of every block, then the lo parts
    floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint4 *qa = qop + (hh * 2) * KB * 64 + lane;
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint4 av = qa[(part * KB + kb) * 64];
        const uint4 bv = make_uint4(kop[kb][0], kop[kb][1], kop[kb][2], kop[kb][3]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                      __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0,
                                                      0);
      }
    // lane l: token l % 16 of the wave, queries 4*(l/16) .. +3
    const uint32_t tw = (uint32_t)b0 + (uint32_t)(wave * 16 + (lane & 15));
    if (tw < (uint32_t)t1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = (lane >> 4) * 4 + r;
        if (i < Nq) scores[((int64_t)h * Nq + i) * N + tw] = acc[r] * scale;
      }
    }
    b0 = nb0;
    hh = nhh;
  }
}

// Values of 2 to kAttnSumQueries queries, the residual term on the matrix
// cores.  Each wave owns d/4 channels and
// runs without workgroup barriers: per 64-token tile it
//  * takes the weights p = e^(s - m) of every token (lane) and query, and
//    stores them as two bf16 parts (hi = bf16(p), lo = bf16(p - hi),
//    |p - hi - lo| <= 2^-16 p) in its own P tile; wave 0 adds them to l;
//  * adds each weight, rounded to a multiple of 2^-40, to the weight sum of
//    the token's cluster in the stages t = w mod 4 (64-bit LDS integers,
//    exact in any order);
//  * decodes level * s_hat of its channels (exact in bf16: an odd level
//    below 16 times an E4M3 value) into its own transposed tile V^T;
//  * multiplies P (A: queries x tokens) by V^T (B: tokens x channels) with
//    v_mfma_f32_16x16x32_bf16, hi parts then lo parts of each 32-token
//    block, accumulating in fp32.
// A wave's LDS writes and later reads of its own tiles are ordered by the
// in-order LDS queue of the wave.  The tiles' 16-byte granules are
// XOR-swizzled by row so that the operand reads spread over the banks.
constexpr int kValuesAhead = 4;
template <int D, int BITS, int PT>
__global__ __launch_bounds__(256) void k_attn_values_mq(const float *__restrict__ scores, int Nq,
                                                        int N, int H, AttnRec vr, int nsplit,
                                                        int tps, int pf,
                                                        float *__restrict__ part) {
  constexpr int NQG = kAttnSumQueries;  // queries per launch
  constexpr int CW = D / 4;              // channels per wave
  constexpr int CTW = CW / 16;           // 16-channel tiles per wave
  constexpr int TPL = CW / 8;            // tokens per lane in the decode
  constexpr int NTG = kAttnBN / TPL;     // token groups
  constexpr int SPW = (PT + 3) / 4;      // stages per wave
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float floatx4_t __attribute__((ext_vector_type(4)));
  // INT2 levels by nibble (two codes per float2 entry): 16 entries cover the
  // banks once, so random lookups do not conflict; INT4 by byte
  __shared__ float2 lutn[BITS == 2 ? 16 : 1];
  __shared__ float4 lut4v[BITS == 4 ? 128 : 1];
  __shared__ __align__(16) uint16_t vt_all[4][CW * kAttnBN];        // per wave V^T
  __shared__ __align__(16) uint16_t pt_all[4][2 * NQG * kAttnBN];   // per wave P
  __shared__ float mred[4][NQG], lred[NQG];
  float2 *lut4 = reinterpret_cast<float2 *>(lut4v);
  extern __shared__ unsigned long long ws[];  // [Nq][T][C] weight sums in units of 2^-40
  int h, sp;
  attn_item(H, nsplit, h, sp);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int T = vr.T, C = vr.C, TC = T * C, vg = __builtin_ctz(vr.G);
  uint16_t *vt = vt_all[wave], *pt = pt_all[wave];
  if constexpr (BITS == 2) {
    if (t < 16) lutn[t] = make_float2((float)(2 * (t & 3) - 3), (float)(2 * (t >> 2) - 3));
  } else {
    init_level_lut<BITS>(nullptr, lut4);
  }
  for (int x = t; x < Nq * TC; x += 256) ws[x] = 0ull;
  const float *sh = scores + (int64_t)h * Nq * N;
  const int ntiles = (N + kAttnBN - 1) / kAttnBN;
  const int tb = sp * tps, te = min(tb + tps, ntiles);
  // M: the run's largest score per query
  const int r0 = tb * kAttnBN, r1 = min(te * kAttnBN, N);
  float M[NQG];
#pragma unroll
  for (int jq = 0; jq < NQG; ++jq) {
    float m = -__builtin_inff();
    if (jq < Nq)
      for (int i0 = r0 + t; i0 < r1; i0 += 256 * 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = sh[(int64_t)jq * N + min(i0 + 256 * u, r1 - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) m = fmaxf(m, v[u]);
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) mred[wave][jq] = m;
  }
  __syncthreads();  // also orders the LUT and the cleared sums before use
#pragma unroll
  for (int jq = 0; jq < NQG; ++jq)
    M[jq] = fmaxf(fmaxf(mred[0][jq], mred[1][jq]), fmaxf(mred[2][jq], mred[3][jq]));
  // decode role: tokens TPL*g .. +TPL-1, channels wave*CW + 8*c8 .. +7
  const int g = lane % NTG, c8 = lane / NTG;
  const int kw = wave * CW + c8 * 8;  // first channel of the lane's group
  const int dv = __builtin_ctz(D) - vg;
  const uint8_t *codes = vr.codes + (int64_t)h * N * (D * BITS / 8);
  const uint8_t *scl = vr.scales + ((int64_t)h * N << dv);
  const uint8_t *asg = vr.assign + (int64_t)h * T * N;
  // one tile's global loads: the scores of token `lane`, its assignment
  // bytes in this wave's stages (past T: the last stage, unused), the
  // decode role's code words and scale bytes
  struct Raw {
    float s[NQG];
    uint32_t a[SPW];
    uint32_t w[TPL], e[TPL];
  };
  const int Tl = max(T - 1, 0);
  auto fetch = [&](int tile, Raw &r) {
    const int i0 = tile * kAttnBN, nt = min(kAttnBN, N - i0);
    const int tl = i0 + min(lane, nt - 1);
#pragma unroll
    for (int jq = 0; jq < NQG; ++jq) r.s[jq] = jq < Nq ? sh[(int64_t)jq * N + tl] : 0.0f;
    if (T > 0) {  // uniform
#pragma unroll
      for (int u = 0; u < SPW; ++u) r.a[u] = asg[(int64_t)min(wave + 4 * u, Tl) * N + tl];
    }
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
      const int ti = i0 + min(TPL * g + u, nt - 1);
      load_codes<BITS, 1>(codes + (int64_t)ti * (D * BITS / 8), kw, &r.w[u]);
      r.e[u] = scl[((int64_t)ti << dv) + (kw >> vg)];
    }
  };
  float lsum[NQG];
#pragma unroll
  for (int jq = 0; jq < NQG; ++jq) lsum[jq] = 0.0f;
  floatx4_t acc[CTW];
#pragma unroll
  for (int c = 0; c < CTW; ++c) acc[c] = (floatx4_t){0.0f, 0.0f, 0.0f, 0.0f};
  const int qi = lane & 15, kq = lane >> 4;  // operand row / column, 8-token granule
  auto process = [&](int tile, const Raw &r) {
    const int nt = min(kAttnBN, N - tile * kAttnBN);
    // weights of token `lane`: P tile (granules swizzled by query) and sums
    unsigned long long pq[NQG];
#pragma unroll
    for (int jq = 0; jq < NQG; ++jq) {
      const bool ok = jq < Nq && lane < nt;
      const float p = ok ? __expf(r.s[jq] - M[jq]) : 0.0f;
      lsum[jq] += p;
      const uint32_t hi = pack_bf16_rne(0.0f, p) >> 16;
      const float rem = p - __uint_as_float(hi << 16);  // exact
      const uint32_t lo = pack_bf16_rne(0.0f, rem) >> 16;
      const int col = (((lane >> 3) ^ jq) << 3) | (lane & 7);
      pt[(0 * NQG + jq) * kAttnBN + col] = (uint16_t)hi;
      pt[(1 * NQG + jq) * kAttnBN + col] = (uint16_t)lo;
      pq[jq] = __float2ull_rn(p * 0x1p40f);
    }
    if (lane < nt) {
#pragma unroll
      for (int u = 0; u < SPW; ++u) {
        const int ts = wave + 4 * u;
        if (ts < T) {
          const int c = min((int)r.a[u], C - 1);
#pragma unroll
          for (int jq = 0; jq < NQG; ++jq)
            if (jq < Nq) atomicAdd(ws + (jq * T + ts) * C + c, pq[jq]);
        }
      }
    }
    // level * s_hat of this lane's tokens and channels into V^T (row k =
    // channel within the wave, granules swizzled by k mod 8)
    {
      float v[TPL][8];
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        if constexpr (BITS == 2) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {  // codes 2m, 2m+1
            const float2 x = lutn[(r.w[u] >> (4 * m)) & 0xFu];
            v[u][2 * m] = x.x;
            v[u][2 * m + 1] = x.y;
          }
        } else {
          levels8(r.w[u], BITS, nullptr, lut4, v[u]);
        }
        const float shat = e4m3_decode_bits(r.e[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = v[u][e] * shat;  // exact
      }
      const int n0 = TPL * g;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = c8 * 8 + e;
        uint16_t *dst = vt + k * kAttnBN + ((((n0 >> 3) ^ e) << 3) | (n0 & 7));
        if constexpr (TPL == 4) {
          *reinterpret_cast<uint2 *>(dst) =
              make_uint2(pack_bf16_rne(v[0][e], v[1][e]), pack_bf16_rne(v[2][e], v[3][e]));
        } else {
          *reinterpret_cast<uint32_t *>(dst) = pack_bf16_rne(v[0][e], v[1][e]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // O[q][k] += sum_n P[q][n] V[n][k] over the two 32-token blocks
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int gr = ks * 4 + kq;  // 8-token granule of the block
      uint4 ah = make_uint4(0u, 0u, 0u, 0u), al = ah;
      if (qi < Nq) {
        const int col = (gr ^ qi) << 3;
        ah = *reinterpret_cast<const uint4 *>(pt + (0 * NQG + qi) * kAttnBN + col);
        al = *reinterpret_cast<const uint4 *>(pt + (1 * NQG + qi) * kAttnBN + col);
      }
#pragma unroll
      for (int c = 0; c < CTW; ++c) {
        const int k = c * 16 + qi;
        const uint4 bv =
            *reinterpret_cast<const uint4 *>(vt + k * kAttnBN + ((gr ^ (k & 7)) << 3));
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                         __builtin_bit_cast(bf16x8_t, bv), acc[c],
                                                         0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                         __builtin_bit_cast(bf16x8_t, bv), acc[c],
                                                         0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  };
  // tile k's loads sit in buffer k mod kValuesAhead, issued kValuesAhead
  // tiles before its use; every path issues the same loads, so that the
  // compiler's waits stay counted
  Raw buf[kValuesAhead];
#pragma unroll
  for (int k = 0; k < kValuesAhead; ++k) fetch(min(tb + k, te - 1), buf[k]);
  for (int tile = tb; tile < te; tile += kValuesAhead) {
#pragma unroll
    for (int k = 0; k < kValuesAhead; ++k) {
      if (tile + k < te) process(tile + k, buf[k]);  // uniform
      fetch(min(tile + k + kValuesAhead, te - 1), buf[k]);
    }
  }
  // l per query: wave 0's lanes, pairwise
  if (wave == 0) {
#pragma unroll
    for (int jq = 0; jq < NQG; ++jq) {
      float v = lsum[jq];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) v = v + __shfl_xor(v, off);
      if (lane == 0) lred[jq] = v;
    }
  }
  __syncthreads();  // l, and every weight sum, are complete
  float *rec = part + ((int64_t)h * nsplit + sp) * Nq * pf;
  // lanes 0..15 hold rows (queries) 0..3 of their channel columns
  if (lane < 16) {
#pragma unroll
    for (int c = 0; c < CTW; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r < Nq) rec[r * pf + 2 + wave * CW + c * 16 + lane] = acc[c][r];
  }
#pragma unroll
  for (int jq = 0; jq < NQG; ++jq)
    if (t == jq && jq < Nq) {
      rec[jq * pf] = M[jq];
      rec[jq * pf + 1] = lred[jq];
    }
  for (int x = t; x < Nq * TC; x += 256) {
    const int jq = x / TC;
    rec[jq * pf + 2 + D + (x - jq * TC)] = __ull2float_rn(ws[x]) * 0x1p-40f;
  }
}

// Values of 2 to 16 queries in one launch, the residual term on the matrix
// cores.  A workgroup of d/16 waves takes one run; every query's weight sums
// sit in LDS at once (Nq*T*C 64-bit integers), so the value record is read
// once per call.  Per 64-token tile:
//  * thread (query q = w + k*d/16, token = lane) takes its weight
//    p = e^(s - m_q), adds it to its l, stores it as two bf16 parts (hi =
//    bf16(p), lo = bf16(p - hi), |p - hi - lo| <= 2^-16 p) in the shared P
//    tile (double-buffered: one barrier per tile), and adds it, rounded to a
//    multiple of 2^-40, to the weight sum of the token's cluster in every
//    stage (exact in any order);
//  * wave w decodes level * s_hat of its 16 channels (exact in bf16) into its
//    own transposed tile V^T, ordered before its reads by the wave's in-order
//    LDS queue;
//  * after the barrier, wave w multiplies P (A: 16 queries x tokens) by its
//    V^T (B: tokens x 16 channels) with v_mfma_f32_16x16x32_bf16, hi parts
//    then lo parts of each 32-token block, accumulating in fp32.
// Tile granules are XOR-swizzled by row (bank spread); loads run
// kValuesAhead tiles ahead.
template <int D, int BITS, int PT>
__global__ __launch_bounds__(D * 4) void k_attn_values_all(const float *__restrict__ scores, int Nq,
                                                           int N, int H, AttnRec vr, int nsplit,
                                                           int tps, int pf,
                                                           float *__restrict__ part) {
  constexpr int NW = D / 16;             // waves, one 16-channel tile each
  constexpr int NT = NW * 64;            // threads
  constexpr int QPT = kAttnMaxQueries / NW;  // (query, token) weights per thread and tile
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float floatx4_t __attribute__((ext_vector_type(4)));
  __shared__ float2 lutn[BITS == 2 ? 16 : 1];
  __shared__ float4 lut4v[BITS == 4 ? 128 : 1];
  __shared__ __align__(16) uint16_t vt_all[NW][16 * kAttnBN];  // per wave V^T
  __shared__ __align__(16) uint16_t pt_all[2][2 * 16 * kAttnBN];  // P: [buf][part][query][token]
  __shared__ float mred[NW][kAttnMaxQueries], lred[kAttnMaxQueries], Ms[kAttnMaxQueries];
  float2 *lut4 = reinterpret_cast<float2 *>(lut4v);
  extern __shared__ unsigned long long ws[];  // [Nq][T][C] weight sums in units of 2^-40
  int h, sp;
  attn_item(H, nsplit, h, sp);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int T = vr.T, C = vr.C, TC = T * C, vg = __builtin_ctz(vr.G);
  uint16_t *vt = vt_all[wave];
  if constexpr (BITS == 2) {
    if (t < 16) lutn[t] = make_float2((float)(2 * (t & 3) - 3), (float)(2 * (t >> 2) - 3));
  } else {
    if (t < 256) lut4[t] = make_float2((float)(2 * (t & 15) - 15), (float)(2 * ((t >> 4) & 15) - 15));
  }
  for (int x = t; x < Nq * TC; x += NT) ws[x] = 0ull;
  const float *sh = scores + (int64_t)h * Nq * N;
  const int ntiles = (N + kAttnBN - 1) / kAttnBN;
  const int tb = sp * tps, te = min(tb + tps, ntiles);
  // the run's largest score per query
  const int r0 = tb * kAttnBN, r1 = min(te * kAttnBN, N);
  for (int jq = 0; jq < Nq; ++jq) {
    float m = -__builtin_inff();
    for (int i0 = r0 + t; i0 < r1; i0 += NT * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = sh[(int64_t)jq * N + min(i0 + NT * u, r1 - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) m = fmaxf(m, v[u]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) mred[wave][jq] = m;
  }
  __syncthreads();
  if (t < kAttnMaxQueries) {
    float m = -__builtin_inff();
    if (t < Nq)
#pragma unroll
      for (int w = 0; w < NW; ++w) m = fmaxf(m, mred[w][t]);
    Ms[t] = m;
  }
  __syncthreads();  // also orders the level table and the cleared sums
  float Mq[QPT];
  bool qok[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int qq = wave + k * NW;
    qok[k] = qq < Nq;
    Mq[k] = qok[k] ? Ms[qq] : 0.0f;
  }
  // decode role: tokens 2g, 2g+1, channels 16*wave + 8*c8 .. +7
  const int g = lane & 31, c8 = lane >> 5;
  const int kw = wave * 16 + c8 * 8;
  const int dv = __builtin_ctz(D) - vg;
  const uint8_t *codes = vr.codes + (int64_t)h * N * (D * BITS / 8);
  const uint8_t *scl = vr.scales + ((int64_t)h * N << dv);
  const uint8_t *asg = vr.assign + (int64_t)h * T * N;
  const int Tl = max(T - 1, 0);
  struct Raw {
    float s[QPT];
    uint32_t a[PT];
    uint32_t w[2], e[2];
  };
  auto fetch = [&](int tile, Raw &r) {
    const int i0 = tile * kAttnBN, nt = min(kAttnBN, N - i0);
    const int tl = i0 + min(lane, nt - 1);
#pragma unroll
    for (int k = 0; k < QPT; ++k)
      r.s[k] = qok[k] ? sh[(int64_t)(wave + k * NW) * N + tl] : 0.0f;
    if (T > 0) {  // uniform; stages past T repeat the last one (unused)
#pragma unroll
      for (int u = 0; u < PT; ++u) r.a[u] = asg[(int64_t)min(u, Tl) * N + tl];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ti = i0 + min(2 * g + u, nt - 1);
      load_codes<BITS, 1>(codes + (int64_t)ti * (D * BITS / 8), kw, &r.w[u]);
      r.e[u] = scl[((int64_t)ti << dv) + (kw >> vg)];
    }
  };
  float lsum[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) lsum[k] = 0.0f;
  floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int qi = lane & 15, kq = lane >> 4;
  auto process = [&](int tile, const Raw &r) {
    const int nt = min(kAttnBN, N - tile * kAttnBN);
    uint16_t *pt = pt_all[(tile - tb) & 1];
    // weights of (query wave + k*NW, token lane)
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int qq = wave + k * NW;
      const bool ok = qok[k] && lane < nt;
      const float p = ok ? __expf(r.s[k] - Mq[k]) : 0.0f;
      lsum[k] += p;
      const uint32_t hi = pack_bf16_rne(0.0f, p) >> 16;
      const float rem = p - __uint_as_float(hi << 16);  // exact
      const uint32_t lo = pack_bf16_rne(0.0f, rem) >> 16;
      const int col = (((lane >> 3) ^ (qq & 7)) << 3) | (lane & 7);
      pt[(0 * 16 + qq) * kAttnBN + col] = (uint16_t)hi;
      pt[(1 * 16 + qq) * kAttnBN + col] = (uint16_t)lo;
      if (ok) {
        const unsigned long long pq = __float2ull_rn(p * 0x1p40f);
#pragma unroll
        for (int ts = 0; ts < PT; ++ts)
          if (ts < T) atomicAdd(ws + (qq * T + ts) * C + min((int)r.a[ts], C - 1), pq);
      }
    }
    // level * s_hat of tokens 2g, 2g+1 and this lane's 8 channels into V^T
    {
      float v[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if constexpr (BITS == 2) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {  // codes 2m, 2m+1
            const float2 x = lutn[(r.w[u] >> (4 * m)) & 0xFu];
            v[u][2 * m] = x.x;
            v[u][2 * m + 1] = x.y;
          }
        } else {
          levels8(r.w[u], BITS, nullptr, lut4, v[u]);
        }
        const float shat = e4m3_decode_bits(r.e[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = v[u][e] * shat;  // exact
      }
      const int n0 = 2 * g;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = c8 * 8 + e;
        *reinterpret_cast<uint32_t *>(vt + k * kAttnBN + ((((n0 >> 3) ^ e) << 3) | (n0 & 7))) =
            pack_bf16_rne(v[0][e], v[1][e]);
      }
    }
    __syncthreads();  // the P tile is complete (it is rewritten two tiles on)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int gr = ks * 4 + kq;  // 8-token granule of the block
      uint4 ah = make_uint4(0u, 0u, 0u, 0u), al = ah;
      if (qi < Nq) {
        const int col = (gr ^ (qi & 7)) << 3;
        ah = *reinterpret_cast<const uint4 *>(pt + (0 * 16 + qi) * kAttnBN + col);
        al = *reinterpret_cast<const uint4 *>(pt + (1 * 16 + qi) * kAttnBN + col);
      }
      const uint4 bv = *reinterpret_cast<const uint4 *>(vt + qi * kAttnBN + ((gr ^ (qi & 7)) << 3));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ah),
                                                    __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, al),
                                                    __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
    }
  };
  Raw buf[kValuesAhead];
#pragma unroll
  for (int k = 0; k < kValuesAhead; ++k) fetch(min(tb + k, te - 1), buf[k]);
  for (int tile = tb; tile < te; tile += kValuesAhead) {
#pragma unroll
    for (int k = 0; k < kValuesAhead; ++k) {
      if (tile + k < te) process(tile + k, buf[k]);  // uniform
      fetch(min(tile + k + kValuesAhead, te - 1), buf[k]);
    }
  }
  // l of queries wave + k*NW: the wave's lanes, pairwise
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    float v = lsum[k];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = v + __shfl_xor(v, off);
    if (lane == 0) lred[wave + k * NW] = v;
  }
  __syncthreads();  // l, and every weight sum, are complete
  float *rec = part + ((int64_t)h * nsplit + sp) * Nq * pf;
  // lane l holds queries 4*(l/16) .. +3 of channel 16*wave + l % 16
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qq = kq * 4 + r;
    if (qq < Nq) rec[qq * pf + 2 + wave * 16 + qi] = acc[r];
  }
  if (t < Nq) {
    rec[t * pf] = Ms[t];
    rec[t * pf + 1] = lred[t];
  }
  for (int x = t; x < Nq * TC; x += NT) {
    const int jq = x / TC;
    rec[jq * pf + 2 + D + (x - jq * TC)] = __ull2float_rn(ws[x]) * 0x1p-40f;
  }
}

// Values of one query: a lane owns 32 consecutive channels of one token per
// pass (four lanes per token for d = 128, two for d = 64), so a token's
// weight is computed by 4 (or 2) lanes, and the lane accumulates its 32
// channels in registers; the wave that owns stage t (t = w mod 4, lane =
// token) adds the weights to the stage's sums.  Summation order: an output
// element of one run is a fused multiply-add chain over the run's tokens of
// that lane position (one per pass), the 16 (or 32) lane chains of a wave
// added pairwise, then the 4 waves in order.
template <int D, int BITS>
__global__ __launch_bounds__(256) void k_attn_values1(const float *__restrict__ scores, int N,
                                                      int H, AttnRec vr, int nsplit, int tps,
                                                      int pf, float *__restrict__ part) {
  constexpr int LPT = D / 32, TPP = 256 / LPT;  // lanes per token, tokens per pass
  constexpr int NW = BITS == 2 ? 2 : 4;         // code words (32 bits) per lane
  constexpr int WCH = TPP / 64;                 // 64-token chunks per pass (weight sums)
  __shared__ float2 lutn[BITS == 2 ? 16 : 1];     // INT2 levels by nibble
  __shared__ float4 lut4v[BITS == 4 ? 128 : 1];  // [256] float2, 16-byte aligned
  __shared__ float mred[4];
  __shared__ float lred;
  float2 *lut4 = reinterpret_cast<float2 *>(lut4v);
  // [T][C] weight sums in units of 2^-40, then [4][D] wave outputs
  extern __shared__ unsigned long long ws[];
  int h, sp;
  attn_item(H, nsplit, h, sp);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int part_ = t % LPT, tok = t / LPT, k0 = part_ * 32;
  const int T = vr.T, C = vr.C, TC = T * C, vg = __builtin_ctz(vr.G);
  if constexpr (BITS == 2) {
    if (t < 16) lutn[t] = make_float2((float)(2 * (t & 3) - 3), (float)(2 * (t >> 2) - 3));
  } else {
    init_level_lut<BITS>(nullptr, lut4);
  }
  for (int x = t; x < TC; x += 256) ws[x] = 0ull;
  const float *sh = scores + (int64_t)h * N;
  const int ntiles = (N + kAttnBN - 1) / kAttnBN;
  const int tb = sp * tps, te = min(tb + tps, ntiles);
  const int r0 = tb * kAttnBN, r1 = min(te * kAttnBN, N);
  const uint8_t *codes = vr.codes + (int64_t)h * N * (D * BITS / 8);
  const uint8_t *scl = vr.scales + ((int64_t)h * N << (__builtin_ctz(D) - vg));
  const int dv = __builtin_ctz(D) - vg;
  // A pass's loads: this lane's code words, scale bytes and score, and for
  // the weight sums the score and stage-`wave` assignment byte of token
  // `lane` of each 64-token chunk; tokens past the run repeat its last one.
  struct Raw {
    uint32_t w[NW], e[4], a[WCH];
    float s, sw[WCH];
  };
  auto fetch = [&](int b0, Raw &r) {
    const uint32_t ti = (uint32_t)min(b0 + tok, r1 - 1);
    const uint8_t *crow = codes + ti * (uint32_t)(D * BITS / 8) + k0 * BITS / 8;
    if constexpr (BITS == 2) {
      const uint2 x = *reinterpret_cast<const uint2 *>(crow);
      r.w[0] = x.x, r.w[1] = x.y;
    } else {
      const uint4 x = *reinterpret_cast<const uint4 *>(crow);
      r.w[0] = x.x, r.w[1] = x.y, r.w[2] = x.z, r.w[3] = x.w;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) r.e[g] = scl[(ti << dv) + ((k0 + 8 * g) >> vg)];
    r.s = sh[ti];
#pragma unroll
    for (int c = 0; c < WCH; ++c) {
      const uint32_t tl = (uint32_t)min(b0 + 64 * c + lane, r1 - 1);
      r.sw[c] = sh[tl];
      r.a[c] = wave < T ? vr.assign[((int64_t)h * T + wave) * N + tl] : 0u;
    }
  };
  // m: the run's largest score (8 loads in flight per round)
  {
    float m = -__builtin_inff();
    for (int i0 = r0 + t; i0 < r1; i0 += 256 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = sh[min(i0 + 256 * u, r1 - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) m = fmaxf(m, v[u]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) mred[wave] = m;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(mred[0], mred[1]), fmaxf(mred[2], mred[3]));
  float o[32], l = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) o[e] = 0.0f;
  // pass k's loads sit in buffer k mod kValuesAhead, issued kValuesAhead
  // passes before its use; every path issues the same loads
  auto process = [&](int b0, const Raw &r) {
    // residual term: this lane's 32 channels of its token
    const float p = b0 + tok < r1 ? __expf(r.s - M) : 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float lv[8];
      const uint32_t w = BITS == 2 ? (r.w[g >> 1] >> (16 * (g & 1))) & 0xFFFFu : r.w[g];
      if constexpr (BITS == 2) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {  // codes 2m, 2m+1
          const float2 x = lutn[(w >> (4 * m)) & 0xFu];
          lv[2 * m] = x.x;
          lv[2 * m + 1] = x.y;
        }
      } else {
        levels8(w, BITS, nullptr, lut4, lv);
      }
      const float ps = p * e4m3_decode_bits(r.e[g]);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[8 * g + e] = __builtin_fmaf(ps, lv[e], o[8 * g + e]);
    }
    // weight sums (wave w: stages w, w + 4, ...) and l (wave 0); lane = token
    if (wave == 0 || wave < T) {
#pragma unroll
      for (int c = 0; c < WCH; ++c) {
        const bool valid = b0 + 64 * c + lane < r1;
        const float pw = valid ? __expf(r.sw[c] - M) : 0.0f;
        if (wave == 0) l += pw;
        const unsigned long long pq = __float2ull_rn(pw * 0x1p40f);
        const int tl = min(b0 + 64 * c + lane, r1 - 1);
        for (int ts = wave; ts < T; ts += 4) {
          const uint32_t raw = ts == wave ? r.a[c] : vr.assign[((int64_t)h * T + ts) * N + tl];
          if (valid) atomicAdd(ws + ts * C + min((int)raw, C - 1), pq);
        }
      }
    }
  };
  Raw buf[kValuesAhead];
#pragma unroll
  for (int q = 0; q < kValuesAhead; ++q) fetch(min(r0 + q * TPP, r1 - 1), buf[q]);
  for (int b0 = r0; b0 < r1; b0 += kValuesAhead * TPP) {
#pragma unroll
    for (int q = 0; q < kValuesAhead; ++q) {
      const int bq = b0 + q * TPP;
      if (bq < r1) process(bq, buf[q]);  // uniform
      fetch(min(bq + kValuesAhead * TPP, r1 - 1), buf[q]);
    }
  }
  // combine: lanes of one channel range are lane % LPT apart by multiples of
  // LPT within a wave (added pairwise), then the 4 waves in order
  float *wout = reinterpret_cast<float *>(ws + TC);  // [4][D]
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = o[e] + __shfl_xor(o[e], off);
  if (lane < LPT)
#pragma unroll
    for (int e = 0; e < 32; ++e) wout[wave * D + k0 + e] = o[e];
  if (wave == 0) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l = l + __shfl_xor(l, off);
    if (lane == 0) lred = l;
  }
  __syncthreads();
  float *rec = part + ((int64_t)h * nsplit + sp) * pf;
  for (int k = t; k < D; k += 256)
    rec[2 + k] = ((wout[k] + wout[D + k]) + wout[2 * D + k]) + wout[3 * D + k];
  if (t == 0) {
    rec[0] = M;
    rec[1] = lred;
  }
  for (int x = t; x < TC; x += 256) rec[2 + D + x] = __ull2float_rn(ws[x]) * 0x1p-40f;
}

namespace {

int nq_bucket(int Nq) { return Nq <= 1 ? 1 : Nq <= 4 ? 4 : 16; }

size_t attn_lds_bytes(int NQ, int D, bool sums, int Nq, int TC) {
  const size_t vals = sums ? (size_t)kAttnBN * (D + 8) * 2 : (size_t)kAttnBN * (D + 4) * 4;
  return (size_t)256 * 24 + (size_t)kAttnBN * (D + 8) * 2 + vals + (size_t)NQ * D * 4 + (size_t)NQ * kAttnBN * 4 +
         (size_t)NQ * 16 + (sums ? (size_t)Nq * TC * 4 : 0);
}

template <typename Tc, int D, int NQ, bool SUMS>
bool launch_attn_t(const float *q, int H, int Nq, int N, const AttnRec &kr, const AttnRec &vr,
                   float scale, const float *rcos, const float *rsin, float *part, float *out,
                   hipStream_t s) {
  const AttnSplit sp = attn_split(H, N);
  const int pf = attn_part_floats(Nq, D, vr.T, vr.C, false);
  const int TC = vr.T * vr.C;
  static const bool lds_ok =
      hipFuncSetAttribute((const void *)k_attn_split<Tc, D, NQ, SUMS>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024) == hipSuccess;
  if (!lds_ok) return false;
  hipLaunchKernelGGL((k_attn_split<Tc, D, NQ, SUMS>), dim3(H * sp.nsplit), dim3(256),
                     attn_lds_bytes(NQ, D, SUMS, Nq, TC), s, q, Nq, N, H, kr, vr, scale, rcos,
                     rsin, sp.nsplit, sp.tiles_per_split, pf, part);
  if (hipGetLastError() != hipSuccess) return false;
  float *cpart = part + (size_t)H * sp.nsplit * Nq * pf;
  if (SUMS && TC > 0) {
    hipLaunchKernelGGL((k_attn_contract<Tc>), dim3(Nq, H, kContractParts), dim3(256), 0, s, part,
                       sp.nsplit, Nq, D, pf, vr, cpart);
    if (hipGetLastError() != hipSuccess) return false;
  }
  if (SUMS && TC > 0)
    hipLaunchKernelGGL(k_attn_combine<true>, dim3(Nq, H), dim3(128), 0, s, part, sp.nsplit, Nq, D,
                       pf, cpart, out);
  else
    hipLaunchKernelGGL(k_attn_combine<false>, dim3(Nq, H), dim3(128), 0, s, part, sp.nsplit, Nq, D,
                       pf, cpart, out);
  return hipGetLastError() == hipSuccess;
}

// The two-pass path (scores, then values); the scratch holds the
// run records, the contraction parts and the scores [H][Nq][N], in that
// order.  The scores pass cuts each head group's tiles into its own runs, so
// that about kAttnTargetGroups workgroups fill the chip.
template <int D, int NQ, int KT>
bool launch_scores_t(const float *q, int H, int Nq, int N, const AttnRec &kr, float scale,
                     const float *rcos, const float *rsin, float *scores, hipStream_t s) {
  const int HG = score_group(H, NQ, D), ngroups = (H + HG - 1) / HG;
  const int ntiles = (N + kAttnBN - 1) / kAttnBN;
  const int want = std::min(std::min(std::max(1, (kAttnTargetGroups + ngroups - 1) / ngroups),
                                     kAttnMaxSplit), ntiles);
  const int tps = (ntiles + want - 1) / want, nsplit = (ntiles + tps - 1) / tps;
  const size_t lds = (size_t)HG * NQ * D * sizeof(float);
  if (kr.bits == 2)
    hipLaunchKernelGGL((k_attn_scores<D, NQ, KT, 2>), dim3(ngroups * nsplit), dim3(256), lds, s, q,
                       Nq, N, H, kr, scale, rcos, rsin, nsplit, tps, scores);
  else
    hipLaunchKernelGGL((k_attn_scores<D, NQ, KT, 4>), dim3(ngroups * nsplit), dim3(256), lds, s, q,
                       Nq, N, H, kr, scale, rcos, rsin, nsplit, tps, scores);
  return hipGetLastError() == hipSuccess;
}

template <int D, int KT>
bool launch_scores_mq_t(const float *q, int H, int Nq, int N, const AttnRec &kr, float scale,
                        const float *rcos, const float *rsin, float *scores, hipStream_t s) {
  const int HG = score_group(H, kAttnMaxQueries, D), ngroups = (H + HG - 1) / HG;
  const int ntiles = (N + kAttnBN - 1) / kAttnBN;
  const int want = std::min(std::min(std::max(1, (kAttnTargetGroups + ngroups - 1) / ngroups),
                                     kAttnMaxSplit), ntiles);
  const int tps = (ntiles + want - 1) / want, nsplit = (ntiles + tps - 1) / tps;
  const size_t lds = (size_t)HG * 2 * (D / 32) * 64 * sizeof(uint4);
  if (kr.bits == 2)
    hipLaunchKernelGGL((k_attn_scores_mq<D, KT, 2>), dim3(ngroups * nsplit), dim3(256), lds, s, q,
                       Nq, N, H, kr, scale, rcos, rsin, nsplit, tps, scores);
  else
    hipLaunchKernelGGL((k_attn_scores_mq<D, KT, 4>), dim3(ngroups * nsplit), dim3(256), lds, s, q,
                       Nq, N, H, kr, scale, rcos, rsin, nsplit, tps, scores);
  return hipGetLastError() == hipSuccess;
}

template <int D, int NQ>
bool launch_attn_2p(const float *q, int H, int Nq, int N, const AttnRec &kr, const AttnRec &vr,
                    float scale, const float *rcos, const float *rsin, float *part, float *out,
                    hipStream_t s) {
  const AttnSplit sp = attn_split(H, N);
  const int pf = attn_part_floats(Nq, D, vr.T, vr.C, true);
  const int TC = vr.T * vr.C;
  float *cpart = part + (size_t)H * sp.nsplit * Nq * pf;
  float *scores = cpart + (size_t)H * Nq * kContractParts * D;
  bool ok = false;
  if (NQ == 1) {
    switch (kr.T) {
      case 1: ok = launch_scores_t<D, 1, 1>(q, H, Nq, N, kr, scale, rcos, rsin, scores, s); break;
      case 2: ok = launch_scores_t<D, 1, 2>(q, H, Nq, N, kr, scale, rcos, rsin, scores, s); break;
      case 3: ok = launch_scores_t<D, 1, 3>(q, H, Nq, N, kr, scale, rcos, rsin, scores, s); break;
      case 4: ok = launch_scores_t<D, 1, 4>(q, H, Nq, N, kr, scale, rcos, rsin, scores, s); break;
    }
  } else {
    switch (kr.T) {
      case 1: ok = launch_scores_mq_t<D, 1>(q, H, Nq, N, kr, scale, rcos, rsin, scores, s); break;
      case 2: ok = launch_scores_mq_t<D, 2>(q, H, Nq, N, kr, scale, rcos, rsin, scores, s); break;
      case 3: ok = launch_scores_mq_t<D, 3>(q, H, Nq, N, kr, scale, rcos, rsin, scores, s); break;
      case 4: ok = launch_scores_mq_t<D, 4>(q, H, Nq, N, kr, scale, rcos, rsin, scores, s); break;
    }
  }
  if (!ok) return false;
  if (NQ == 1) {
    const size_t lds = (size_t)TC * sizeof(unsigned long long) + (size_t)4 * D * sizeof(float);
    if (vr.bits == 2)
      hipLaunchKernelGGL((k_attn_values1<D, 2>), dim3(H * sp.nsplit), dim3(256), lds, s, scores,
                         N, H, vr, sp.nsplit, sp.tiles_per_split, pf, part);
    else
      hipLaunchKernelGGL((k_attn_values1<D, 4>), dim3(H * sp.nsplit), dim3(256), lds, s, scores,
                         N, H, vr, sp.nsplit, sp.tiles_per_split, pf, part);
  } else {
    // more than kAttnSumQueries queries: one launch with every query's
    // weight sums at once (Nq*T*C <= 16384 64-bit words), so the value record
    // is read once; otherwise one launch of the per-wave kernel
    if (Nq > kAttnSumQueries) {
      static const bool lds_ok =
          hipFuncSetAttribute((const void *)k_attn_values_all<D, 2, 4>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024) == hipSuccess &&
          hipFuncSetAttribute((const void *)k_attn_values_all<D, 2, kMaxT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024) == hipSuccess &&
          hipFuncSetAttribute((const void *)k_attn_values_all<D, 4, 4>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024) == hipSuccess &&
          hipFuncSetAttribute((const void *)k_attn_values_all<D, 4, kMaxT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024) == hipSuccess;
      if (!lds_ok) return false;
      const size_t lds = (size_t)Nq * TC * sizeof(unsigned long long);
      const dim3 grid(H * sp.nsplit), block(D * 4);
      if (vr.bits == 2 && vr.T <= 4)
        hipLaunchKernelGGL((k_attn_values_all<D, 2, 4>), grid, block, lds, s, scores, Nq, N, H, vr,
                           sp.nsplit, sp.tiles_per_split, pf, part);
      else if (vr.bits == 2)
        hipLaunchKernelGGL((k_attn_values_all<D, 2, kMaxT>), grid, block, lds, s, scores, Nq, N, H,
                           vr, sp.nsplit, sp.tiles_per_split, pf, part);
      else if (vr.T <= 4)
        hipLaunchKernelGGL((k_attn_values_all<D, 4, 4>), grid, block, lds, s, scores, Nq, N, H, vr,
                           sp.nsplit, sp.tiles_per_split, pf, part);
      else
        hipLaunchKernelGGL((k_attn_values_all<D, 4, kMaxT>), grid, block, lds, s, scores, Nq, N, H,
                           vr, sp.nsplit, sp.tiles_per_split, pf, part);
    } else {
      const size_t lds = (size_t)Nq * TC * sizeof(unsigned long long);
      const dim3 grid(H * sp.nsplit);
      if (vr.bits == 2 && vr.T <= 4)
        hipLaunchKernelGGL((k_attn_values_mq<D, 2, 4>), grid, dim3(256), lds, s, scores, Nq, N, H,
                           vr, sp.nsplit, sp.tiles_per_split, pf, part);
      else if (vr.bits == 2)
        hipLaunchKernelGGL((k_attn_values_mq<D, 2, kMaxT>), grid, dim3(256), lds, s, scores, Nq, N,
                           H, vr, sp.nsplit, sp.tiles_per_split, pf, part);
      else if (vr.T <= 4)
        hipLaunchKernelGGL((k_attn_values_mq<D, 4, 4>), grid, dim3(256), lds, s, scores, Nq, N, H,
                           vr, sp.nsplit, sp.tiles_per_split, pf, part);
      else
        hipLaunchKernelGGL((k_attn_values_mq<D, 4, kMaxT>), grid, dim3(256), lds, s, scores, Nq, N,
                           H, vr, sp.nsplit, sp.tiles_per_split, pf, part);
    }
  }
  if (hipGetLastError() != hipSuccess) return false;
  if (TC > 0) {
    hipLaunchKernelGGL((k_attn_contract<uint16_t>), dim3(Nq, H, kContractParts), dim3(256), 0, s,
                       part, sp.nsplit, Nq, D, pf, vr, cpart);
    if (hipGetLastError() != hipSuccess) return false;
    hipLaunchKernelGGL(k_attn_combine<true>, dim3(Nq, H), dim3(128), 0, s, part, sp.nsplit, Nq, D,
                       pf, cpart, out);
  } else {
    hipLaunchKernelGGL(k_attn_combine<false>, dim3(Nq, H), dim3(128), 0, s, part, sp.nsplit, Nq, D,
                       pf, cpart, out);
  }
  return hipGetLastError() == hipSuccess;
}

template <typename Tc, int D>
bool launch_attn_d(const float *q, int H, int Nq, int N, const AttnRec &kr, const AttnRec &vr,
                   float scale, const float *rcos, const float *rsin, float *part, float *out,
                   hipStream_t s) {
  if (attn_two_pass(H, Nq, kr.T, vr.T, vr.C, sizeof(Tc) == 2, N, D)) {
    if (Nq == 1) return launch_attn_2p<D, 1>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
    return launch_attn_2p<D, kAttnMaxQueries>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
  }
  if (attn_sums_one_pass(Nq, vr.T, vr.C)) {
    if (Nq == 1)
      return launch_attn_t<Tc, D, 1, true>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
    return launch_attn_t<Tc, D, 4, true>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
  }
  switch (nq_bucket(Nq)) {
    case 1: return launch_attn_t<Tc, D, 1, false>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
    case 4: return launch_attn_t<Tc, D, 4, false>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
    default: return launch_attn_t<Tc, D, 16, false>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
  }
}

}  // namespace

AttnSplit attn_split(int H, int64_t N) {
  const int ntiles = (int)((N + kAttnBN - 1) / kAttnBN);
  const int want = std::min(std::min(std::max(1, (kAttnTargetGroups + H - 1) / H), kAttnMaxSplit),
                            ntiles);
  const int tps = (ntiles + want - 1) / want;
  return AttnSplit{(ntiles + tps - 1) / tps, tps};
}

bool attn_sums_one_pass(int Nq, int T, int C) {
  return Nq <= kAttnSumQueries && (int64_t)Nq * T * C <= kAttnSumEntries;
}

bool attn_sums_two_pass(int Nq, int T, int C) {
  return Nq <= kAttnMaxQueries &&
         (int64_t)std::min(Nq, kAttnSumQueries) * T * C <= kAttnSumEntries;
}

bool attn_two_pass(int H, int Nq, int kT, int vT, int vC, bool c_bf16, int64_t N, int D) {
  // k_attn_scores addresses the rotary rows with 32-bit byte offsets and
  // keeps a head group's queries in LDS
  return c_bf16 && kT >= 1 && kT <= 4 && attn_sums_two_pass(Nq, vT, vC) &&
         N * 2 * D < ((int64_t)1 << 32) && H <= 256;
}

int attn_part_floats(int Nq, int D, int T, int C, bool two_pass) {
  const bool sums = two_pass ? attn_sums_two_pass(Nq, T, C) : attn_sums_one_pass(Nq, T, C);
  return D + 2 + (sums ? T * C : 0);
}

size_t attn_scratch_floats(int H, int64_t N, int Nq, int D, int T, int C) {
  // sized for the larger of the two paths' layouts: the two-pass path uses
  // weight sums whenever the one-pass path does, and for more queries
  const AttnSplit sp = attn_split(H, N);
  const bool sums = attn_sums_two_pass(Nq, T, C);
  const size_t runs = (size_t)H * sp.nsplit * Nq * attn_part_floats(Nq, D, T, C, true);
  const size_t contract = sums ? (size_t)H * Nq * kContractParts * D : 0;
  const size_t two = sums ? (size_t)H * Nq * N : 0;  // the two-pass path's scores
  return runs + contract + two;
}

bool launch_attention(const float *q, int H, int Nq, int N, int D, const AttnRec &kr,
                      const AttnRec &vr, bool c_bf16, float scale, const float *rcos,
                      const float *rsin, float *part, float *out, hipStream_t s) {
  TimerScope ts_("attention", s);
  if (D == 64)
    return c_bf16 ? launch_attn_d<uint16_t, 64>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s)
                  : launch_attn_d<float, 64>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
  return c_bf16 ? launch_attn_d<uint16_t, 128>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s)
                : launch_attn_d<float, 128>(q, H, Nq, N, kr, vr, scale, rcos, rsin, part, out, s);
}

}  // namespace qvg
