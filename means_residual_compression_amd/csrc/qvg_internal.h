// Host-side launcher interface between the C ABI and the kernel files.
#pragma once

#include <algorithm>

#include "qvg_common.h"

namespace qvg {

// Brackets one kernel launch with HIP events on its stream while timing is
// enabled (qvg_timing_enable); a no-op otherwise.
class TimerScope {
 public:
  TimerScope(const char *name, hipStream_t s);
  ~TimerScope();
  TimerScope(const TimerScope &) = delete;
  TimerScope &operator=(const TimerScope &) = delete;

 private:
  const char *name_;
  hipStream_t s_;
  hipEvent_t a_;
};

// Everything one stage of k-means needs.  `r` is the stage input residual
// [H][N][D] (bf16 X at the first stage, fp32 afterwards).
struct KmArgs {
  int H, N, C, Cp, NT;
  // stage input residual R(t) = x - C(1)[pi(1)] - ... - C(t)[pi(t)] (see
  // ResView): x [H][N][D] in the record dtype, record assignments and
  // centroids with Ts stages, nsub = t
  const void *x;
  const uint8_t *rec_pi;
  const void *rec_cent;
  int Ts, nsub;
  const int32_t *idx;  // device [H][..][C] init rows, or nullptr
  int64_t idx_hstride;
  const float *init;   // device [H][..][C][D] init centroids, or nullptr
  int64_t init_hstride;
  uint8_t *assign;     // stage slice of [H][T][N]
  int64_t assign_hstride;
  Ws ws;
  uint32_t *ws_stats;  // stats row of this stage; per-head stride stat_stride
  int stat_stride;
  float kappa;         // relative error coefficient of the MFMA keys
};

bool launch_stage_bound(uint32_t *prev_stats, int stat_stride, int H, hipStream_t s);
// Seeded cold-start rows idx[h][t][0..C) for every head and stage (the draw
// documented with qvg_params.seed).
bool launch_sample_rows(int H, int T, int N, int C, uint64_t seed, int32_t *idx, hipStream_t s);
template <typename Tin>
bool launch_absmax(const void *x, int H, int64_t per_head, uint32_t *stats, int stat_stride,
                   int slot, hipStream_t s);
template <typename Tin, int D>
bool launch_kmeans_stage_begin(const KmArgs &a, hipStream_t s);
template <typename Tin, int D>
bool launch_assign(const KmArgs &a, int bslot, hipStream_t s);
template <typename Tin, typename Tc, int D>
// iter: the iteration within the stage, or -1 for a lone update.  Iteration 0
// reduces the chunk sums' spans over each head, so later iterations skip the
// tracking; with a.ws.isum set it also keeps the sums of heads whose stage
// sums are exact, and later iterations update those heads from the tokens
// whose assignment changed.
bool launch_update(const KmArgs &a, int next_bslot, bool tables, Tc *rec_c, int64_t rec_hstride,
                   float *cache, int64_t cache_hstride, int log_slot, int iter, hipStream_t s);

// Records of consecutive chunks of one stream for one reconstruction launch:
// chunk c holds tokens [off[c], off[c+1]) of the launch's span, which starts
// at token out_off of an output with out_hstride tokens per head.
constexpr int kMaxChunksPerLaunch = 32;
struct NoChunks {};
struct ChunkTable {
  const uint8_t *codes[kMaxChunksPerLaunch];
  const uint8_t *scales[kMaxChunksPerLaunch];
  const uint8_t *assign[kMaxChunksPerLaunch];
  const void *cent[kMaxChunksPerLaunch];
  int64_t off[kMaxChunksPerLaunch + 1];
  int64_t out_off, out_hstride;
  int n;
};

// Elementwise kernels (qvg_quant.hip).
bool launch_fill_u32(uint32_t *p, int64_t n, hipStream_t s);
// r_out = r - chat[assign] (fp32), stats max|r_out| into stats[h*stride+slot]
// when stats is non-null.
bool launch_subtract(const void *r, bool r_bf16, int H, int N, int D, int C, const uint8_t *assign,
                     int64_t assign_hstride, const void *chat, bool c_bf16, int64_t chat_hstride,
                     float *r_out, uint32_t *stats, int stat_stride, int slot, hipStream_t s);
// codes/scales of the residual x - C(1)[pi(1)] - ... - C(nsub)[pi(nsub)]
// (record assignments [H][Ts][N], centroids [H][Ts][C][D] in x's dtype).
// Assignment bytes >= C are clamped to C-1 in every kernel that gathers
// centroids.
bool launch_quant(const void *x, bool bf16, int H, int N, int D, int C, const uint8_t *pi,
                  const void *cent, int Ts, int nsub, int bits, int G, uint8_t *codes,
                  uint8_t *scales, hipStream_t s);
bool launch_dequant(const uint8_t *codes, const uint8_t *scales, const uint8_t *assign,
                    const void *cent, bool c_bf16, int H, int N, int D, int C, int T, int bits,
                    int G, void *out, bool out_bf16, hipStream_t s);
// The same over the records of tbl.n consecutive chunks (at most
// kMaxChunksPerLaunch); all share T, C, bits, G and the dtypes.
bool launch_dequant_chunks(const ChunkTable &tbl, bool c_bf16, int H, int D, int C, int T,
                           int bits, int G, void *out, bool out_bf16, hipStream_t s);

}  // namespace qvg
