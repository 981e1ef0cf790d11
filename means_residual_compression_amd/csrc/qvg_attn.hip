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
    for (int x = t; x < Nq * TC; x += 256) ws[x] = 0.0f;
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
  const int qq = blockIdx.x, h = blockIdx.y, z = blockIdx.z, t = threadIdx.x;
  const int64_t stride = (int64_t)Nq * pf;
  const float *p = part + ((int64_t)h * nsplit * Nq + qq) * pf;
  float M = -__builtin_inff();
  for (int b = 0; b < nsplit; ++b) M = fmaxf(M, p[b * stride]);
  const int TC = vr.T * vr.C;
  const int r0 = z * TC / kContractParts, r1 = (z + 1) * TC / kContractParts, n = r1 - r0;
  for (int r = t; r < n; r += 256) {
    float acc = 0.0f;
#pragma unroll 4
    for (int b = 0; b < nsplit; ++b)
      acc = __builtin_fmaf(p[b * stride + 2 + D + r0 + r], __expf(p[b * stride] - M), acc);
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
  const int qq = blockIdx.x, h = blockIdx.y, k = threadIdx.x;
  if (k >= D) return;
  const int64_t stride = (int64_t)Nq * pf;
  const float *p = part + ((int64_t)h * nsplit * Nq + qq) * pf;
  float M = -__builtin_inff();
  for (int b = 0; b < nsplit; ++b) M = fmaxf(M, p[b * stride]);
  float l = 0.0f, o = 0.0f;
  for (int b = 0; b < nsplit; ++b) {
    const float w = __expf(p[b * stride] - M);
    l = __builtin_fmaf(p[b * stride + 1], w, l);
    o = __builtin_fmaf(p[b * stride + 2 + k], w, o);
  }
  if (SUMS) {
    const float *cp = cpart + ((int64_t)h * Nq + qq) * kContractParts * D + k;
    for (int z = 0; z < kContractParts; ++z) o += cp[z * D];
  }
  out[((int64_t)h * Nq + qq) * D + k] = o / l;
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
  const int pf = attn_part_floats(Nq, D, vr.T, vr.C);
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

template <typename Tc, int D>
bool launch_attn_d(const float *q, int H, int Nq, int N, const AttnRec &kr, const AttnRec &vr,
                   float scale, const float *rcos, const float *rsin, float *part, float *out,
                   hipStream_t s) {
  if (attn_uses_sums(Nq, vr.T, vr.C)) {
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

bool attn_uses_sums(int Nq, int T, int C) {
  return Nq <= kAttnSumQueries && (int64_t)Nq * T * C <= kAttnSumEntries;
}

int attn_part_floats(int Nq, int D, int T, int C) {
  return D + 2 + (attn_uses_sums(Nq, T, C) ? T * C : 0);
}

size_t attn_scratch_floats(int H, int64_t N, int Nq, int D, int T, int C) {
  const AttnSplit sp = attn_split(H, N);
  const size_t runs = (size_t)H * sp.nsplit * Nq * attn_part_floats(Nq, D, T, C);
  const size_t contract = attn_uses_sums(Nq, T, C) ? (size_t)H * Nq * kContractParts * D : 0;
  return runs + contract;
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
