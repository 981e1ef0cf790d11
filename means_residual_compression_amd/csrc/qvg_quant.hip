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
// view's nsub = T), recomputed from the input and the record.
template <typename T, int BITS, int NSUB>
__global__ void k_quant(ResView<T> rv, int G, uint8_t *__restrict__ codes,
                        uint8_t *__restrict__ scales) {
  constexpr int L = (1 << BITS) - 1, MID = 1 << (BITS - 1);
  const int h = blockIdx.y;
  const int N = rv.N, D = rv.D;
  const int lpt = D / 8, lpg = G / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = g < (int64_t)N * lpt;
  const int64_t i = live ? g / lpt : 0;
  const int q = (int)(g % lpt);
  float v[8];
  if (live) {
    rv.template load8_n<NSUB>(h, i, q * 8, v);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[k]));
  for (int o = 1; o < lpg; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
  const float s = a / (float)L;
  const uint32_t e = e4m3_encode(s);
  const float sh = e4m3_decode(e);
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    int c = MID;
    if (sh != 0.0f) c = min(max(floor_half(v[k] / sh) + MID, 0), L);
    packed |= (uint32_t)c << (BITS * k);
  }
  if (!live) return;
  const int64_t row = (int64_t)h * N + i;
  if (BITS == 2) {
    reinterpret_cast<uint16_t *>(codes + row * (D / 4))[q] = (uint16_t)packed;
  } else {
    reinterpret_cast<uint32_t *>(codes + row * (D / 2))[q] = packed;
  }
  if (q % lpg == 0) scales[row * (D / G) + q / lpg] = (uint8_t)e;
}

// ------------------------------------------------------------- dequant
template <typename Tc, typename To, int BITS>
__global__ void k_dequant(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                          const uint8_t *__restrict__ assign, const Tc *__restrict__ cent, int N,
                          int D, int C, int T, int G, To *__restrict__ out) {
  constexpr int L = (1 << BITS) - 1;
  const int h = blockIdx.y;
  const int lpt = D / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)N * lpt) return;
  const int64_t i = g / lpt;
  const int q = (int)(g % lpt);
  const int64_t row = (int64_t)h * N + i;
  uint32_t packed;
  if (BITS == 2) {
    packed = reinterpret_cast<const uint16_t *>(codes + row * (D / 4))[q];
  } else {
    packed = reinterpret_cast<const uint32_t *>(codes + row * (D / 2))[q];
  }
  const float sh = e4m3_decode(scales[row * (D / G) + (q * 8) / G]);
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = (int)((packed >> (BITS * k)) & (uint32_t)L);
    v[k] = (float)(2 * c - L) * sh;  // exact: small integer times an E4M3 value
  }
  for (int t = T - 1; t >= 0; --t) {
    const int j = min((int)assign[((int64_t)h * T + t) * N + i], C - 1);
    float c[8];
    load8(cent, (((int64_t)h * T + t) * C + j) * D + q * 8, c);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = v[k] + c[k];
  }
  store8(out, row * D + q * 8, v);
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
  rv.C = C;
  rv.Ts = Ts;
  rv.nsub = nsub;
  const int64_t threads = (int64_t)N * (D / 8);
  dim3 grid((unsigned)((threads + 255) / 256), H);
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

bool launch_dequant(const uint8_t *codes, const uint8_t *scales, const uint8_t *assign,
                    const void *cent, bool c_bf16, int H, int N, int D, int C, int T, int bits,
                    int G, void *out, bool out_bf16, hipStream_t s) {
  const int64_t threads = (int64_t)N * (D / 8);
  dim3 grid((unsigned)((threads + 255) / 256), H);
  TimerScope ts_("fused_dequant", s);
#define QVG_DQ(TC, TO, B)                                                                      \
  hipLaunchKernelGGL((k_dequant<TC, TO, B>), grid, dim3(256), 0, s, codes, scales, assign,    \
                     (const TC *)cent, N, D, C, T, G, (TO *)out)
#define QVG_DQB(TC, TO) \
  do { if (bits == 2) QVG_DQ(TC, TO, 2); else QVG_DQ(TC, TO, 4); } while (0)
  if (c_bf16 && out_bf16) QVG_DQB(uint16_t, uint16_t);
  else if (c_bf16) QVG_DQB(uint16_t, float);
  else if (out_bf16) QVG_DQB(float, uint16_t);
  else QVG_DQB(float, float);
#undef QVG_DQB
#undef QVG_DQ
  QVG_CHECK_LAUNCH();
  return true;
}

}  // namespace qvg
