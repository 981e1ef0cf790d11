// Launcher interface of the fused dequant-attention (qvg_attn.hip).
#pragma once

#include "qvg_common.h"

namespace qvg {

// Attention of Nq queries over one compressed history (qvg_attn.hip): the
// keys are rebuilt per tile of kAttnBN tokens in LDS, as launch_dequant
// rebuilds them (bf16), and never stored; the values enter unrounded.  Each
// head's tiles are cut into nsplit runs of tiles_per_split consecutive
// tiles, one workgroup each, so that about kAttnTargetGroups workgroups fill
// the chip whatever the head count; the split count depends on H and N only.
constexpr int kAttnBN = 64;
constexpr int kAttnTargetGroups = 2048;
constexpr int kAttnMaxSplit = 1024;
constexpr int kAttnMaxQueries = 16;
// Value path by per-centroid weight sums: on the one-pass path up to this
// many queries, while their T * C weight sums fit kAttnSumEntries entries of
// LDS in all; on the two-pass path up to kAttnMaxQueries queries while this
// many (or Nq, if fewer) queries' sums would fit, i.e. all Nq queries' sums
// fit 4 * kAttnSumEntries (k_attn_values_mq takes up to this many queries,
// k_attn_values_all more).
constexpr int kAttnSumQueries = 4;
constexpr int kAttnSumEntries = 4096;
struct AttnRec {
  const uint8_t *codes, *scales, *assign;
  const void *cent;
  int T, bits, G, C;
};
struct AttnSplit {
  int nsplit, tiles_per_split;
};
AttnSplit attn_split(int H, int64_t N);
// Whether the values go through per-centroid weight sums on the one-pass
// path and on the two-pass path (see qvg_attn.hip).
bool attn_sums_one_pass(int Nq, int T, int C);
bool attn_sums_two_pass(int Nq, int T, int C);
// Whether the call takes the two-pass path (scores, then values):
// bf16 centroids, keys of 1 to 4 stages, weight sums, N * 2d < 2^32 and at
// most 256 heads.
bool attn_two_pass(int H, int Nq, int kT, int vT, int vC, bool c_bf16, int64_t N, int D);
// Floats of one (run, query) record in the scratch: m, l, o[D], then the
// T*C weight sums when the path uses them.
int attn_part_floats(int Nq, int D, int T, int C, bool two_pass);
// fp32 scratch floats of one call (the larger of the two paths' layouts):
// the run records, then (with weight sums) the contraction parts
// [H][Nq][8][D] and the scores [H][Nq][N] of the two-pass path.
size_t attn_scratch_floats(int H, int64_t N, int Nq, int D, int T, int C);
// q [H][Nq][D] fp32, part [H][nsplit][Nq][attn_part_floats] fp32 scratch
// (attn_scratch_floats in all),
// out [H][Nq][D] fp32; rcos/rsin [N][D/2] fp32 or both null (no rotation).
// Both records hold centroids of the same dtype (c_bf16).
bool launch_attention(const float *q, int H, int Nq, int N, int D, const AttnRec &kr,
                      const AttnRec &vr, bool c_bf16, float scale, const float *rcos,
                      const float *rsin, float *part, float *out, hipStream_t s);

}  // namespace qvg
