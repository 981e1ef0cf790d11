// Memory-bound kernels of the QVG path for gfx950: centroid subtraction,
// fused subtract + per-group quantization + packing, and fused
// dequantization with stage-T..1 centroid add-back.
//
// paper.rainbus.top method paragraph: SAS (c) residual R = X - C[pi]; Q:
// symmetric per-group integer quantization of R(T) (X_INT, S_x); DQ:
// X^(t-1) = X^(t) + C(t)[pi(t)] from t = T down to 1.  note.zhuruihan.top
// "Algorithm-System Co-design": fused dequantization keeps intermediates in
// registers; scales are FP8 E4M3.
//
// Thread layout for all three: one lane per 8 consecutive channels of one
// token (16 B of bf16 / 32 B of fp32), so a token row of d=128 is 16 lanes
// and every global access of a wave is contiguous.
#include <type_traits>

#include "qvg_common.h"
#include "qvg_internal.h"

namespace qvg {

__global__ void k_fill_u32(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ------------------------------------------------------------ subtract
template <typename Tin, typename Tc>
__global__ void k_subtract(const Tin *__restrict__ r, int N, int D, int C, const uint8_t *__restrict__ assign,
                           int64_t assign_hstride, const Tc *__restrict__ chat,
                           int64_t chat_hstride, float *__restrict__ out, uint32_t *stats,
                           int stat_stride, int slot) {
  const int h = blockIdx.y;
  const int lpt = D / 8;  // lanes per token
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float m = 0.0f;
  if (g < (int64_t)N * lpt) {
    const int64_t i = g / lpt;
    const int q = (int)(g % lpt);
    // an assignment byte >= C (corrupt input) is clamped so no read leaves the table
    const int j = min((int)assign[(int64_t)h * assign_hstride + i], C - 1);
    const int64_t off = ((int64_t)h * N + i) * D + q * 8;
    float v[8], c[8];
    load8(r, off, v);
    load8(chat + (int64_t)h * chat_hstride, (int64_t)j * D + q * 8, c);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = v[k] - c[k];
      m = fmaxf(m, fabsf(v[k]));
    }
    store8(out, off, v);
  }
  if (stats) {  // one atomic per workgroup
    __shared__ float part[4];
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
      atomicMax(stats + (int64_t)h * stat_stride + slot, __float_as_uint(m));
    }
  }
}

// --------------------------------------------------------- quant + pack
// floor(u / 2) of an fp32 u, exact also where u/2 underflows to -0.
__device__ __forceinline__ int floor_half(float u) {
  const float hh = u * 0.5f;
  int f = (int)floorf(hh);
  if (hh == 0.0f && u < 0.0f) f = -1;
  return f;
}

// Quantizes the residual R(T) = x - C(1)[pi(1)] - ... - C(T)[pi(T)] (the
// view's nsub = T), recomputed from the input and the record.  A lane covers
// 8 channels of QU tokens: the stage indices of all QU tokens are loaded
// first, then their input rows and centroid rows, so each wave has QU
// independent chains of loads in flight.  Per group of G channels (G/8
// adjacent lanes): a = max |r|, s = a / (2^b - 1) (IEEE division), E4M3
// scale, codes floor(u / 2) + 2^(b-1) with u = r / s_hat, clamped.
constexpr int QU = 4;
template <typename T, int BITS, int NSUB>
__global__ __launch_bounds__(256) void k_quant(ResView<T> rv, int G, uint8_t *__restrict__ codes,
                                               uint8_t *__restrict__ scales) {
  constexpr int L = (1 << BITS) - 1, MID = 1 << (BITS - 1);
  const int h = blockIdx.y;
  const int N = rv.N, D = rv.D;
  const int lpt = D / 8, lpg = G / 8, glog2 = __builtin_ctz(G);
  const int tpb = (int)blockDim.x / lpt;  // tokens per block and slot
  const int q = (int)threadIdx.x % lpt;
  const int64_t t0 = (int64_t)blockIdx.x * tpb * QU + threadIdx.x / lpt;
  int64_t tok[QU];
  int js[QU][NSUB > 0 ? NSUB : 1];
#pragma unroll
  for (int u = 0; u < QU; ++u) {
    tok[u] = t0 + (int64_t)u * tpb;
    const int64_t i = min(tok[u], (int64_t)N - 1);
#pragma unroll
    for (int st = 0; st < NSUB; ++st) js[u][st] = rv.stage_j(h, st, i);
  }
  float v[QU][8];
#pragma unroll
  for (int u = 0; u < QU; ++u) load8(rv.x, rv.xrow(h, min(tok[u], (int64_t)N - 1)) + q * 8, v[u]);
  float c[QU][NSUB > 0 ? NSUB : 1][8];
#pragma unroll
  for (int u = 0; u < QU; ++u)
#pragma unroll
    for (int st = 0; st < NSUB; ++st) load8(rv.stage_row(h, st, js[u][st]), q * 8, c[u][st]);
#pragma unroll
  for (int u = 0; u < QU; ++u) {
#pragma unroll
    for (int st = 0; st < NSUB; ++st)  // R(t) = x - C(1)[pi(1)] - ... in stage order
#pragma unroll
      for (int k = 0; k < 8; ++k) v[u][k] = v[u][k] - c[u][st][k];
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[u][k]));
    for (int o = 1; o < lpg; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
    const float sc = a / (float)L;
    const uint32_t e = e4m3_encode(sc);
    const float sh = e4m3_decode(e);
    uint32_t packed = 0;
    if constexpr (BITS == 2) {
      // code = #{B in {-2, 0, 2} : fl(r / s_hat) >= B} (the clamped floor(u/2)
      // + 2).  With round-to-nearest-even, fl(x) >= B exactly when x >= tau(B):
      // tau(-2) = -2 - 2^-23, tau(0) = -2^-150, tau(2) = 2 - 2^-24 (half the gap
      // to B's lower neighbour; a tie rounds to B, whose last bit is even).
      // So fl(r / s_hat) >= B iff r >= tau(B) * s_hat, a product exact in fp64
      // (at most 25 + 4 significant bits): no division.  s_hat = 0 gives 2.
      const double sd = (double)sh;
      const double t1 = (-2.0 - 0x1p-23) * sd, t2 = -0x1p-150 * sd, t3 = (2.0 - 0x1p-24) * sd;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const double r = (double)v[u][k];
        int cd = (r >= t1) + (r >= t2) + (r >= t3);
        if (sh == 0.0f) cd = MID;
        packed |= (uint32_t)cd << (2 * k);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        int cd = MID;
        if (sh != 0.0f) cd = min(max(floor_half(v[u][k] / sh) + MID, 0), L);
        packed |= (uint32_t)cd << (BITS * k);
      }
    }
    if (tok[u] >= N) continue;
    const int64_t row = (int64_t)h * N + tok[u];
    if (BITS == 2) {
      reinterpret_cast<uint16_t *>(codes + (row << (rv.dlog2 - 2)))[q] = (uint16_t)packed;
    } else {
      reinterpret_cast<uint32_t *>(codes + (row << (rv.dlog2 - 1)))[q] = packed;
    }
    if (q % lpg == 0) scales[(row << (rv.dlog2 - glog2)) + q / lpg] = (uint8_t)e;
  }
}

// ------------------------------------------------------------- dequant
// The H*N token rows are cut into equal contiguous ranges, one per resident
// workgroup slot; each range is processed in slices of `ch` channels by
// separate workgroups that sit consecutively on one XCD (so a range's code
// bytes come from HBM once).  A workgroup keeps in LDS (a) its head's
// centroid tables of all T stages for its slice, in the centroid dtype
// (re-staged where the range crosses into the next head), and (b) a
// 256-entry table from a code
// byte to the signed levels 2q - L of the codes it packs.  One lane handles 8
// consecutive channels (so a wave's stores cover whole lines) of U
// consecutive tokens per step; every global load of a step is issued before
// the first use, and the U tokens are computed together so their LDS reads
// overlap (tokens past the end are clamped; only their stores are skipped);
// output goes out through non-temporal stores.
// Per element:
// x = fma(level, s_hat, C(T)[pi]) -- level * s_hat is exact, so this is the
// rounded sum level*s_hat + C(T) -- then x += C(t)[pi(t)] for t = T-1..1 in
// fp32, rounded once (RNE) to the output dtype.
template <typename Tc, typename TL>
__device__ __forceinline__ void stage_tables(TL *tab, const Tc *__restrict__ cent, int h, int T,
                                             int C, int D, int ch, int c0) {
  const int qpr = ch >> 2;  // 4-element quads per table row
  const int nq = T * C * qpr;
  for (int v0 = threadIdx.x; v0 < nq; v0 += 4 * blockDim.x) {
    uint4 tmp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = min(v0 + i * (int)blockDim.x, nq - 1);
      const int row = v / qpr, part = v - row * qpr;  // row = t*C + j
      const Tc *src = cent + ((int64_t)h * T * C + row) * D + c0 + part * 4;
      if constexpr (sizeof(Tc) == 2) {
        const uint2 w = *reinterpret_cast<const uint2 *>(src);
        tmp[i] = make_uint4(w.x, w.y, 0, 0);
      } else {
        tmp[i] = *reinterpret_cast<const uint4 *>(src);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = v0 + i * (int)blockDim.x;
      if (v >= nq) continue;
      if constexpr (sizeof(TL) == 2) {  // bf16 -> bf16, natural order
        reinterpret_cast<uint2 *>(tab)[v] = make_uint2(tmp[i].x, tmp[i].y);
      } else {
        // fp32 rows are stored as two halves: quad 2m (channels 8m..8m+3) at
        // quad m, quad 2m+1 at quad qpr/2 + m, so that the 8 lanes of a token
        // read one contiguous 128-byte run per instruction (no bank conflicts).
        const int row = v / qpr, part = v - row * qpr;
        const int pq = row * qpr + (part & 1) * (qpr >> 1) + (part >> 1);
        if constexpr (sizeof(Tc) == 2)  // bf16 -> fp32 (exact)
          reinterpret_cast<uint4 *>(tab)[pq] =
              make_uint4(tmp[i].x << 16, tmp[i].x & 0xFFFF0000u, tmp[i].y << 16, tmp[i].y & 0xFFFF0000u);
        else
          reinterpret_cast<uint4 *>(tab)[pq] = tmp[i];
      }
    }
  }
}

// The 8 table values of channels kl..kl+7 of a row, as fp32 (fp32 rows use
// the split layout written by stage_tables).
__device__ __forceinline__ void lds_row8(const float *row, uint32_t kl, uint32_t ch, float c[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(row + (kl >> 1));
  const float4 b = *reinterpret_cast<const float4 *>(row + (ch >> 1) + (kl >> 1));
  c[0] = a.x, c[1] = a.y, c[2] = a.z, c[3] = a.w, c[4] = b.x, c[5] = b.y, c[6] = b.z, c[7] = b.w;
}
__device__ __forceinline__ void lds_row8(const uint16_t *row, uint32_t kl, uint32_t, float c[8]) {
  const uint4 w = *reinterpret_cast<const uint4 *>(row + kl);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = __uint_as_float(u[i] << 16);
    c[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

// Row j of a stage table from a lane's base (the table plus the lane's channel
// offset, in bytes) with one shift-add: bf16 rows are 2^rsh bytes.
__device__ __forceinline__ void lds_row8_at(const char *lane_base, uint32_t j, uint32_t rsh,
                                            float c[8]) {
  const uint4 w = *reinterpret_cast<const uint4 *>(lane_base + (j << rsh));
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = __uint_as_float(u[i] << 16);
    c[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

template <int BITS>
constexpr int dequant_lut_bytes() {
  return 256 * (8 / BITS) * 4;
}

template <typename Tc, typename TL, typename To, int BITS, int T, typename Tab>
__global__ __launch_bounds__(1024) void k_dequant(const uint8_t *__restrict__ codes,
                                                  const uint8_t *__restrict__ scales,
                                                  const uint8_t *__restrict__ assign,
                                                  const Tc *__restrict__ cent, int H, int N, int D,
                                                  int C, int G, int ch_log2, int nranges,
                                                  To *__restrict__ out, Tab tbl) {
  // Tab = ChunkTable: the rows are those of tbl.n chunk records laid end to
  // end per head (N = their total), each record with its own tables
  constexpr bool CH = !std::is_same<Tab, NoChunks>::value;
  constexpr int L = (1 << BITS) - 1;
  constexpr int U = 4;         // consecutive tokens per lane per step
  constexpr int PB = 8 / BITS; // codes per byte
  extern __shared__ float4 smem4[];
  float *lut = reinterpret_cast<float *>(smem4);  // [256][PB]
  TL *tab = reinterpret_cast<TL *>(lut + 256 * PB);  // [T][C][ch]
  const int ch = 1 << ch_log2;
  const int slices = D >> ch_log2;
  const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int sl = k % slices;
  const int r = (k / slices) * 8 + xcd;
  if (r >= nranges) return;
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
#pragma unroll
    for (int i = 0; i < PB; ++i) lut[b * PB + i] = (float)(2 * ((b >> (BITS * i)) & L) - L);
  }
  if (T == 0) __syncthreads();
  const int64_t total = (int64_t)H * N;
  const int64_t per = (total + nranges - 1) / nranges;
  const int64_t a = r * per, b = min(total, a + per);
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lpt_log2 = ch_log2 - 3;  // lanes per token = ch / 8
  const int tpw = 64 >> lpt_log2;    // tokens per wave per unrolled slot
  const uint32_t kl = (uint32_t)(lane & ((1 << lpt_log2) - 1)) * 8;  // lane's channel in the slice
  const uint32_t k0 = (uint32_t)(sl * ch) + kl;                      // ... and in the row
  // All per-row strides are powers of two: D, D*BITS/8 code bytes, D/G scale bytes.
  const int d_log2 = __builtin_ctz(D);
  const int db_log2 = d_log2 + __builtin_ctz(BITS) - 3;
  const int dg_log2 = d_log2 - __builtin_ctz(G);
  const uint32_t coff = k0 * BITS / 8, soff = k0 >> __builtin_ctz(G);
  for (int64_t seg = a; seg < b;) {
    // the segment: rows [lo, hi) of one head of one record (nrec rows per head)
    const int h = (int)(seg / N);
    int64_t lo = seg - (int64_t)h * N, hi = min(b - (int64_t)h * N, (int64_t)N), nrec = N;
    int64_t orow0 = (int64_t)h * N + lo, next = (int64_t)h * N + hi;
    const uint8_t *rc = codes, *rs = scales, *ra = assign;
    const Tc *rcent = cent;
    if constexpr (CH) {
      int c = 0;
      for (int q = 1; q < tbl.n; ++q) c = tbl.off[q] <= lo ? q : c;
      const int64_t c0 = tbl.off[c];
      nrec = tbl.off[c + 1] - c0;
      hi = min(hi, c0 + nrec) - c0;
      lo -= c0;
      orow0 = (int64_t)h * tbl.out_hstride + tbl.out_off + c0 + lo;
      next = (int64_t)h * N + c0 + hi;
      rc = tbl.codes[c];
      rs = tbl.scales[c];
      ra = tbl.assign[c];
      rcent = static_cast<const Tc *>(tbl.cent[c]);
    }
    if (T > 0) {
      __syncthreads();  // the previous segment's tables are no longer read
      stage_tables<Tc, TL>(tab, rcent, h, T, C, D, ch, sl * ch);
      __syncthreads();
    }
    // Segment-relative addressing: uniform 64-bit bases, 32-bit lane offsets
    // (the launcher keeps a range's output below 2^31 bytes).
    const int64_t row0 = (int64_t)h * nrec + lo;
    const uint8_t *cbase = rc + (row0 << db_log2);
    const uint8_t *sbase = rs + (row0 << dg_log2);
    const uint8_t *abase[T > 0 ? T : 1];
#pragma unroll
    for (int t = 0; t < T; ++t) abase[t] = ra + ((int64_t)h * T + t) * nrec + lo;
    char *obase = reinterpret_cast<char *>(out + (orow0 << d_log2));
    const TL *tabt[T > 0 ? T : 1];  // stage tables of this slice
#pragma unroll
    for (int t = 0; t < T; ++t) tabt[t] = tab + (uint32_t)t * C * ch;
    // bf16 tables: each stage's table plus this lane's channel offset, in bytes
    constexpr bool TB = std::is_same<TL, uint16_t>::value;
    const uint32_t rsh = (uint32_t)ch_log2 + 1;
    const char *tlane[T > 0 ? T : 1];
#pragma unroll
    for (int t = 0; t < T; ++t) tlane[t] = reinterpret_cast<const char *>(tabt[t] + kl);
    const uint32_t n = (uint32_t)(hi - lo);
    const uint32_t step_w = (uint32_t)(tpw * U);  // tokens per wave step
    const uint32_t step = (uint32_t)nw * step_w;
    // One step's loads, kept as loaded: fetch_* only issue them and emit()
    // takes the bytes apart, so that a prefetched step's loads stay in flight
    // while the current step computes.  aw[t]: stage t's assignment bytes of
    // the U tokens (byte u = token u); sw[u], packed[u]: token u's scale byte
    // and code bytes.
    struct Batch {
      uint32_t aw[T > 0 ? T : 1];
      uint32_t sw[U];
      uint32_t packed[U];
    };
    // Global loads of one step; a lane's U tokens are rel .. rel+U-1.  Where
    // the whole wave step lies inside the segment (fetch_full) each stage's
    // assignment bytes come in one load; the last, partial step (fetch_tail)
    // loads them per token, clamped to the last token, and packs them alike.
    // Both load in one fixed sequence (no data-dependent control flow), so
    // the compiler can leave a prefetched step's loads in flight.
    auto fetch_token = [&](uint32_t i, int u, Batch &bt) {
      if constexpr (BITS == 2)
        bt.packed[u] = *reinterpret_cast<const uint16_t *>(cbase + ((i << db_log2) + coff));
      else
        bt.packed[u] = *reinterpret_cast<const uint32_t *>(cbase + ((i << db_log2) + coff));
      bt.sw[u] = sbase[(i << dg_log2) + soff];
    };
    auto fetch_full = [&](uint32_t rel, Batch &bt) {
#pragma unroll
      for (int u = 0; u < U; ++u) fetch_token(rel + (uint32_t)u, u, bt);
#pragma unroll
      for (int t = 0; t < T; ++t) __builtin_memcpy(&bt.aw[t], abase[t] + rel, U);
    };
    auto fetch_tail = [&](uint32_t rel, Batch &bt) {
#pragma unroll
      for (int t = 0; t < T; ++t) bt.aw[t] = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = min(rel + (uint32_t)u, n - 1);
        fetch_token(i, u, bt);
#pragma unroll
        for (int t = 0; t < T; ++t) bt.aw[t] |= (uint32_t)abase[t][i] << (8 * u);
      }
    };
    auto emit = [&](uint32_t rel, const Batch &bt) {
      // All U tokens are computed unconditionally (clamped inputs) so their
      // LDS reads overlap; only the stores are guarded.
      float v[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float sh = e4m3_decode_bits(bt.sw[u]);
#pragma unroll
        for (int m = 0; m < 8 / PB; ++m) {  // code bytes of the 8 channels
          const uint32_t byte = (bt.packed[u] >> (8 * m)) & 0xFFu;
          if constexpr (PB == 4) {
            const float4 l4 = reinterpret_cast<const float4 *>(lut)[byte];
            v[u][4 * m] = l4.x, v[u][4 * m + 1] = l4.y, v[u][4 * m + 2] = l4.z, v[u][4 * m + 3] = l4.w;
          } else {
            const float2 l2 = reinterpret_cast<const float2 *>(lut)[byte];
            v[u][2 * m] = l2.x, v[u][2 * m + 1] = l2.y;
          }
        }
        if constexpr (T > 0) {
          float c[8];
          const uint32_t jT = min((bt.aw[T - 1] >> (8 * u)) & 0xFFu, (uint32_t)C - 1);
          if constexpr (TB) lds_row8_at(tlane[T - 1], jT, rsh, c);
          else lds_row8(tabt[T - 1] + (jT << ch_log2), kl, ch, c);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[u][e] = __builtin_fmaf(v[u][e], sh, c[e]);
#pragma unroll
          for (int t = T - 2; t >= 0; --t) {
            const uint32_t jt = min((bt.aw[t] >> (8 * u)) & 0xFFu, (uint32_t)C - 1);
            if constexpr (TB) lds_row8_at(tlane[t], jt, rsh, c);
            else lds_row8(tabt[t] + (jt << ch_log2), kl, ch, c);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[u][e] = v[u][e] + c[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[u][e] = v[u][e] * sh;
        }
      }
      // Keep the arithmetic of all U tokens ahead of the guarded stores (the
      // compiler would otherwise sink each token's work into its store's
      // branch and serialize the LDS reads).
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(v[u][e]));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = rel + (uint32_t)u;
        if (i < n)
          store8_stream(reinterpret_cast<To *>(obase + (((i << d_log2) + k0) * (uint32_t)sizeof(To))), v[u]);
      }
    };
    // Steps run in wave-uniform control flow (rw is the wave's first token);
    // lanes past the end of the partial step load clamped tokens and skip
    // their stores.
    const uint32_t tl = ((uint32_t)lane >> lpt_log2) * U;
    uint32_t rw = (uint32_t)(wave * step_w);
    auto full = [&](uint32_t r) { return __builtin_amdgcn_readfirstlane(r + step_w <= n ? 1 : 0) != 0; };
    if constexpr (T >= 3) {
      // long add chains: the next full step's loads go out before this
      // step's arithmetic and stores (after the last full step they re-read
      // it).  Two batches alternate, so that no loaded register is copied.
      if (full(rw)) {
        Batch b0, b1;
        fetch_full(rw + tl, b0);
        for (;;) {
          uint32_t rn = rw + step;
          bool more = full(rn);
          fetch_full((more ? rn : rw) + tl, b1);
          emit(rw + tl, b0);
          rw = rn;
          if (!more) break;
          rn = rw + step;
          more = full(rn);
          fetch_full((more ? rn : rw) + tl, b0);
          emit(rw + tl, b1);
          rw = rn;
          if (!more) break;
        }
      }
    } else {
      for (; full(rw); rw += step) {
        Batch bt;
        fetch_full(rw + tl, bt);
        emit(rw + tl, bt);
      }
    }
    if (rw < n) {  // the partial step
      Batch bt;
      fetch_tail(rw + tl, bt);
      emit(rw + tl, bt);
    }
    seg = next;
  }
}

// ============================================================ launchers
#define QVG_CHECK_LAUNCH() \
  do { if (hipGetLastError() != hipSuccess) return false; } while (0)

bool launch_fill_u32(uint32_t *p, int64_t n, hipStream_t s) {
  if (n <= 0) return true;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  TimerScope ts_("fill", s);
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  QVG_CHECK_LAUNCH();
  return true;
}

bool launch_subtract(const void *r, bool r_bf16, int H, int N, int D, int C, const uint8_t *assign,
                     int64_t assign_hstride, const void *chat, bool c_bf16, int64_t chat_hstride,
                     float *r_out, uint32_t *stats, int stat_stride, int slot, hipStream_t s) {
  const int64_t threads = (int64_t)N * (D / 8);
  dim3 grid((unsigned)((threads + 255) / 256), H);
  TimerScope ts_("sas_subtract", s);
#define QVG_SUB(TI, TC)                                                                       \
  hipLaunchKernelGGL((k_subtract<TI, TC>), grid, dim3(256), 0, s, (const TI *)r, N, D, C, assign, \
                     assign_hstride, (const TC *)chat, chat_hstride, r_out, stats, stat_stride, \
                     slot)
  if (r_bf16 && c_bf16) QVG_SUB(uint16_t, uint16_t);
  else if (r_bf16) QVG_SUB(uint16_t, float);
  else if (c_bf16) QVG_SUB(float, uint16_t);
  else QVG_SUB(float, float);
#undef QVG_SUB
  QVG_CHECK_LAUNCH();
  return true;
}

template <typename T>
static void launch_quant_t(const void *x, int H, int N, int D, int C, const uint8_t *pi,
                           const void *cent, int Ts, int nsub, int bits, int G, uint8_t *codes,
                           uint8_t *scales, hipStream_t s) {
  ResView<T> rv;
  rv.x = (const T *)x;
  rv.pi = pi;
  rv.cent = (const T *)cent;
  rv.N = N;
  rv.D = D;
  rv.dlog2 = __builtin_ctz(D);
  rv.C = C;
  rv.Ts = Ts;
  rv.nsub = nsub;
  const int tpb = 256 / (D / 8);  // tokens per block and slot
  dim3 grid((unsigned)(((int64_t)N + (int64_t)tpb * QU - 1) / ((int64_t)tpb * QU)), H);
  dispatch_nsub(nsub, [&]<int NS>() {
    if (bits == 2)
      hipLaunchKernelGGL((k_quant<T, 2, NS>), grid, dim3(256), 0, s, rv, G, codes, scales);
    else
      hipLaunchKernelGGL((k_quant<T, 4, NS>), grid, dim3(256), 0, s, rv, G, codes, scales);
  });
}

bool launch_quant(const void *x, bool bf16, int H, int N, int D, int C, const uint8_t *pi,
                  const void *cent, int Ts, int nsub, int bits, int G, uint8_t *codes,
                  uint8_t *scales, hipStream_t s) {
  TimerScope ts_("group_quant_pack", s);
  if (bf16)
    launch_quant_t<uint16_t>(x, H, N, D, C, pi, cent, Ts, nsub, bits, G, codes, scales, s);
  else
    launch_quant_t<float>(x, H, N, D, C, pi, cent, Ts, nsub, bits, G, codes, scales, s);
  QVG_CHECK_LAUNCH();
  return true;
}

// Channel slice of the dequant's LDS tables (kept in the centroid dtype).
// Slices of at least 64 channels keep a token's share of a bf16 output row a
// whole 128-byte line; among those, one whose tables leave room for two
// workgroups per CU is preferred, then one that fits at all; only when none
// fits do slices drop below 64 channels.
static int dequant_slice(int D, int C, int T, size_t esz, size_t lut) {
  for (size_t cap : {80 * 1024, 160 * 1024})
    for (int ch = D; ch >= 64; ch /= 2)
      if (lut + (size_t)T * C * ch * esz <= cap) return ch;
  for (int ch = 32; ch >= 16; ch /= 2)
    if (lut + (size_t)T * C * ch * esz <= 160 * 1024) return ch;
  return 16;
}

template <typename Tc, typename TL, typename To, int BITS, int T, typename Tab>
static bool launch_dequant_t(const uint8_t *codes, const uint8_t *scales, const uint8_t *assign,
                             const void *cent, int H, int N, int D, int C, int G, int ch, void *out,
                             const Tab &tbl, hipStream_t s) {
  const size_t lds = dequant_lut_bytes<BITS>() + (size_t)T * C * ch * sizeof(TL);
  static const bool attr =
      hipFuncSetAttribute((const void *)k_dequant<Tc, TL, To, BITS, T, Tab>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
  if (!attr) return false;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(2, (160 * 1024) / lds));
  const int slices = D / ch;
  const int64_t rows = (int64_t)H * N;
  int64_t want = (int64_t)per_cu * cus / slices;
  // a range's output must stay below 2^31 bytes (32-bit offsets in the kernel)
  want = std::max<int64_t>(want, (rows * D * (int64_t)sizeof(To) >> 30) + 1);
  const int nranges = (int)std::max<int64_t>(1, std::min<int64_t>(rows, want));
  const int grid = (nranges + 7) / 8 * 8 * slices;
  hipLaunchKernelGGL((k_dequant<Tc, TL, To, BITS, T, Tab>), dim3(grid), dim3(1024), lds, s,
                     codes, scales, assign, (const Tc *)cent, H, N, D, C, G, __builtin_ctz(ch),
                     nranges, (To *)out, tbl);
  return true;
}

template <typename Tc, typename To, int BITS, typename Tab>
static bool launch_dequant_b(const uint8_t *codes, const uint8_t *scales, const uint8_t *assign,
                             const void *cent, int H, int N, int D, int C, int T, int G, void *out,
                             const Tab &tbl, hipStream_t s) {
  const int ch = dequant_slice(D, C, T, sizeof(Tc), dequant_lut_bytes<BITS>());
  bool ok = false;
  dispatch_nsub(T, [&]<int TT>() {
    ok = launch_dequant_t<Tc, Tc, To, BITS, TT, Tab>(codes, scales, assign, cent, H, N, D, C, G,
                                                     ch, out, tbl, s);
  });
  return ok;
}

bool launch_dequant(const uint8_t *codes, const uint8_t *scales, const uint8_t *assign,
                    const void *cent, bool c_bf16, int H, int N, int D, int C, int T, int bits,
                    int G, void *out, bool out_bf16, hipStream_t s) {
  TimerScope ts_("fused_dequant", s);
  if (T == 0) C = 1;
  bool ok;
#define QVG_DQ(TC, TO)                                                                          \
  ok = bits == 2 ? launch_dequant_b<TC, TO, 2>(codes, scales, assign, cent, H, N, D, C, T, G, out, \
                                               NoChunks{}, s)                                      \
                 : launch_dequant_b<TC, TO, 4>(codes, scales, assign, cent, H, N, D, C, T, G, out, \
                                               NoChunks{}, s)
  if (c_bf16 && out_bf16) QVG_DQ(uint16_t, uint16_t);
  else if (c_bf16) QVG_DQ(uint16_t, float);
  else if (out_bf16) QVG_DQ(float, uint16_t);
  else QVG_DQ(float, float);
#undef QVG_DQ
  if (!ok) return false;
  QVG_CHECK_LAUNCH();
  return true;
}

bool launch_dequant_chunks(const ChunkTable &tbl, bool c_bf16, int H, int D, int C, int T,
                           int bits, int G, void *out, bool out_bf16, hipStream_t s) {
  TimerScope ts_("fused_dequant", s);
  if (T == 0) C = 1;
  const int N = (int)tbl.off[tbl.n];
  bool ok;
#define QVG_DQ(TC, TO)                                                                         \
  ok = bits == 2 ? launch_dequant_b<TC, TO, 2>(nullptr, nullptr, nullptr, nullptr, H, N, D, C, T, \
                                               G, out, tbl, s)                                    \
                 : launch_dequant_b<TC, TO, 4>(nullptr, nullptr, nullptr, nullptr, H, N, D, C, T, \
                                               G, out, tbl, s)
  if (c_bf16 && out_bf16) QVG_DQ(uint16_t, uint16_t);
  else if (c_bf16) QVG_DQ(uint16_t, float);
  else if (out_bf16) QVG_DQ(float, uint16_t);
  else QVG_DQ(float, float);
#undef QVG_DQ
  if (!ok) return false;
  QVG_CHECK_LAUNCH();
  return true;
}

}  // namespace qvg
