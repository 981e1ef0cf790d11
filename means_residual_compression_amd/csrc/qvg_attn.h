// Launcher interface of the fused dequant-attention (qvg_attn.hip).
#pragma once

#include "qvg_common.h"

namespace qvg {

// Attention of Nq queries over one compressed history (qvg_attn.hip): the
// keys and values are rebuilt per tile of kAttnBN tokens in LDS, as
// launch_dequant rebuilds them (bf16), and never stored.  Each head's tiles
// are cut into nsplit runs of tiles_per_split consecutive tiles, one
// workgroup each, so that about kAttnTargetGroups workgroups fill the chip
// whatever the head count; the split count depends on H and N only.
constexpr int kAttnBN = 64;
constexpr int kAttnTargetGroups = 2048;
constexpr int kAttnMaxSplit = 1024;
constexpr int kAttnMaxQueries = 16;
struct AttnRec {
  const uint8_t *codes, *scales, *assign;
  const void *cent;
  int T, bits, G, C;
};
struct AttnSplit {
  int nsplit, tiles_per_split;
};
AttnSplit attn_split(int H, int64_t N);
// LDS bytes of one split workgroup (NQ query rows, head dim D).
size_t attn_lds_bytes(int NQ, int D);
// q [H][Nq][D] fp32, part [H][nsplit][Nq][D+2] fp32 scratch, out [H][Nq][D]
// fp32; rcos/rsin [N][D/2] fp32 or both null (no rotation).  Both records
// hold centroids of the same dtype (c_bf16).
bool launch_attention(const float *q, int H, int Nq, int N, int D, const AttnRec &kr,
                      const AttnRec &vr, bool c_bf16, float scale, const float *rcos,
                      const float *rsin, float *part, float *out, hipStream_t s);

}  // namespace qvg
