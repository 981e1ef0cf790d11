/*
 * qvg.h -- C ABI of the QVG KV-cache compress/decompress library for MI355X
 * (gfx950).  Implements the hot path of Quant VideoGen ("Auto-Regressive Long
 * Video Generation via 2-Bit KV-Cache Quantization"), as described on:
 *
 *   note.zhuruihan.top  -- sections "Semantic-Aware Smoothing",
 *                          "Progressive Residual Quantization",
 *                          "Algorithm-System Co-design";
 *   paper.rainbus.top   -- method paragraph (SAS steps a-c, PRQ, Q, DQ);
 *   howistudyai.com     -- "Step-by-step" (chunking, C=256, uint8 assignments).
 *
 * One "head-tensor" is one X in R^{N x d} (one attention head of K or of V).
 * H head-tensors are processed per call, all independent.
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device memory owned by the caller, contiguous,
 *    row-major, with the shapes given below.  Host pointers are marked (host).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously and no entry point synchronises the stream.  The one
 *    array argument that may live on the host (init_idx) is then read by a
 *    host-to-device copy enqueued on `stream`: from pageable memory the HIP
 *    runtime stages it before the call returns; from pinned memory the caller
 *    must keep it unchanged until the stream has passed the call.  Given in
 *    device memory it is read by the kernels (no copy), and the seeded draw
 *    (neither init_idx nor init_centroids) runs on the device too.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call returns a status and enqueues nothing.  The library never
 *    aborts and allocates no device memory: scratch comes from the caller's
 *    workspace.  qvg_last_error() describes the most recent failure of the
 *    calling thread.
 *  - Inputs must be finite.  Results for NaN/Inf inputs are unspecified.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *  - Calls that share a workspace or an output buffer on the same stream are
 *    ordered by the stream; concurrent calls on different streams need their
 *    own workspaces.
 */
#ifndef QVG_H
#define QVG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QVG_OK = 0,
    QVG_ERR_INVALID_ARG = 1, /* null pointer, bad size or inconsistent arguments */
    QVG_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels implement */
    QVG_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the size query */
    QVG_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} qvg_status;

typedef enum { QVG_F32 = 0, QVG_BF16 = 1 } qvg_dtype;

/* Method parameters.
 *   C      clusters per stage (k-means k), 1 <= C <= 256 (assignments are
 *          stored as uint8, howistudyai.com "Step-by-step"), C <= N.
 *   T      progressive residual stages, 0 <= T <= 8 (T = 0 is plain
 *          per-group quantization of X).
 *   iters  k-means iterations per stage, each one assign followed by one
 *          update; >= 1 when T >= 1.  The stored assignments come from the
 *          last assign, the stored centroids from the last update.
 *   bits   2 or 4 (INT2 / INT4 codes).
 *   group  G, channels per quantization group along d; d % G == 0 and
 *          G % 8 == 0, 8 <= G <= 256.
 *   seed   seed of the cold-start draw (used when a compress call is given
 *          neither init_idx nor init_centroids): stage t (1-based) of head h
 *          (0-based within the call) starts from the rows perm[0..C) of a
 *          partial Fisher-Yates shuffle of 0..N-1, where step j swaps
 *          perm[j] with perm[j + (z_j mod (N - j))] and z_j is output j of
 *          splitmix64 (Steele, Lea and Flood 2014) started from
 *          seed ^ (0x9E3779B97F4A7C15 * (h+1)) ^ (0xD1B54A32D192ED03 * t),
 *          all arithmetic modulo 2^64.  The pages only say the start is a
 *          set of seeded token rows; this draw is the pinned reading.
 * Supported head dims: d in {64, 128}. */
typedef struct {
    int32_t C;
    int32_t T;
    int32_t iters;
    int32_t bits;
    int32_t group;
    uint64_t seed;
} qvg_params;

/* A compressed record of H head-tensors (paper.rainbus.top, method paragraph:
 * X_INT and S_x, plus C(t) and pi(t) for every stage).
 *   codes      [H][N][d*bits/8]  packed codes; element k of a token row sits
 *                                in byte k*bits/8 at bit offset
 *                                bits*(k mod 8/bits), little-endian.
 *   scales     [H][N][d/G]       FP8 E4M3 (OCP e4m3fn) scale codes, >= 0.
 *   assign     [H][T][N]         uint8 cluster index of each token per stage.
 *   centroids  [H][T][C][d]      stage centroids in the record dtype (the
 *                                dtype of X: bf16 or fp32).
 * Quantized level of code q: (2q - (2^bits - 1)) * scale. */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    uint8_t *assign;
    void *centroids;
} qvg_record;

/* Human-readable name of a status code (static string). */
const char *qvg_status_string(qvg_status s);

/* Message for the calling thread's most recent non-OK status (static
 * thread-local buffer; "" if none). */
const char *qvg_last_error(void);

/* Bytes of device workspace that qvg_compress / qvg_compress_stream need for
 * these sizes; 0 if the arguments are invalid.  The workspace must be 256-byte
 * aligned. */
size_t qvg_workspace_size(int64_t H, int64_t N, int64_t d, qvg_dtype dtype,
                          const qvg_params *p);

/* Compress H head-tensors X [H][N][d] (bf16 or fp32) into `out`.
 *
 * note.zhuruihan.top "Semantic-Aware Smoothing" and "Progressive Residual
 * Quantization"; paper.rainbus.top method paragraph.  R(0) = X; for stage
 * t = 1..T: k-means (squared Euclidean, ties to the smallest index, empty
 * clusters keep their centroid) over the tokens of R(t-1) for `iters`
 * iterations; the centroids rounded to the record dtype are stored and
 * subtracted, R(t) = R(t-1) - C(t)[pi(t)] in fp32.  R(T) is quantized per
 * group of G channels: s = max|r| / (2^b - 1) rounded to the nearest finite
 * E4M3 value (ties to even, saturating at 448); code q = nearest level, a tie
 * going to the upper level; a zero scale gives the middle code everywhere.
 *
 * Stage-t k-means starts from:
 *   init_idx (int32 [H][T][C], host or device memory): rows
 *            init_idx[h][t][0..C) of R(t-1); duplicates allowed.  Host
 *            indices outside [0, N) are rejected (QVG_ERR_INVALID_ARG);
 *            device indices are not read by the host and are clamped to
 *            [0, N-1] by the kernel;
 *   else init_centroids (device, fp32 [H][T][C][d]);
 *   else (both NULL) rows of R(t-1) drawn from p->seed (see qvg_params).
 * At most one of init_idx and init_centroids may be non-NULL.
 * cache_out (device, fp32 [H][T][C][d], nullable) receives each stage's final
 * fp32 centroids before rounding (the streaming centroid cache).
 * Workspace: `ws` of at least qvg_workspace_size() bytes. */
qvg_status qvg_compress(const void *x, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                        const qvg_params *p, const int32_t *init_idx,
                        const float *init_centroids, float *cache_out, const qvg_record *out,
                        void *ws, size_t ws_bytes, void *stream);

/* Streaming compress of one chunk [H][N][d] with the centroid cache
 * (note.zhuruihan.top "Algorithm-System Co-design": the previous chunk's
 * centroids initialise the next chunk's k-means).
 *   cache (device, fp32 [H][T][C][d]) is read as the stage initialisation when
 *   warm != 0 and is overwritten with this chunk's final centroids.
 *   warm != 0: k-means runs `iters_warm` iterations from the cache.
 *   warm == 0: k-means runs p->iters iterations from init_idx (host or
 *   device, as in qvg_compress), or from rows drawn from p->seed when
 *   init_idx is NULL.
 * The record is self-contained: decompress needs no other chunk. */
qvg_status qvg_compress_stream(const void *chunk, qvg_dtype dtype, int64_t H, int64_t N,
                               int64_t d, const qvg_params *p, int32_t iters_warm, float *cache,
                               int warm, const int32_t *init_idx, const qvg_record *out, void *ws,
                               size_t ws_bytes, void *stream);

/* Bytes of the device array qvg_compress_stream_static uses as scratch. */
#define QVG_STATIC_SCRATCH_BYTES (64u << 20)

/* qvg_compress_stream without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, results and errors are those
 * of qvg_compress_stream.  Scratch is a file-scope device array of
 * QVG_STATIC_SCRATCH_BYTES (64 MiB) per GPU, held until the process ends;
 * its address is looked up once per device on the first call made with
 * that device current.  Nothing is allocated: sizes whose workspace
 * (qvg_workspace_size) exceeds the array return QVG_ERR_WORKSPACE before
 * anything is enqueued; 24 head-tensors of 4680 tokens, d = 128, C = 256
 * need 57 MiB.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (different streams, or host threads without ordering)
 * race and must be serialised by the caller.  The array keeps the last
 * call's contents; the call clears what must start at zero itself.  For
 * a call free of host-to-device copies, give init_idx in device memory or
 * leave it NULL (seeded draw). */
qvg_status qvg_compress_stream_static(const void *chunk, qvg_dtype dtype, int64_t H, int64_t N,
                                      int64_t d, const qvg_params *p, int32_t iters_warm,
                                      float *cache, int warm, const int32_t *init_idx,
                                      const qvg_record *out, void *stream);

/* Fused decompression (paper.rainbus.top method paragraph, DQ;
 * note.zhuruihan.top "Algorithm-System Co-design", fused dequantization
 * kernel): per element x = level(q) * scale, then x += C(t)[pi(t)] for
 * t = T down to 1 in fp32, rounded once (RNE) to out_dtype.
 *   rec_dtype: dtype of rec->centroids.  out: device [H][N][d] in out_dtype. */
qvg_status qvg_decompress(const qvg_record *rec, qvg_dtype rec_dtype, int64_t H, int64_t N,
                          int64_t d, const qvg_params *p, void *out, qvg_dtype out_dtype,
                          void *stream);

/* Reconstruction of a stream's history from its chunk records (the chunked
 * streaming of note.zhuruihan.top "Algorithm-System Co-design" and the
 * howistudyai.com explainer, "Step-by-step": each chunk of frames is
 * compressed on its own, and reading the cache means reconstructing every
 * stored chunk).  Chunk c (0 <= c < n_chunks) is a record of n_tokens[c]
 * tokens as written by qvg_compress / qvg_compress_stream with params p; all
 * chunks share p, H, d and rec_dtype.  out: device [H][sum n_tokens][d] in
 * out_dtype; head h's tokens of chunk c start at row h*sum + (n_tokens[0] +
 * ... + n_tokens[c-1]).  Every element is computed exactly as qvg_decompress
 * of that chunk computes it.  recs and n_tokens are host arrays, read during
 * the call only; the records' buffers are device memory.  Chunks go out in
 * launches of up to 32.  Errors: QVG_ERR_INVALID_ARG for NULL pointers,
 * n_chunks < 1 or a chunk with n_tokens < 1; QVG_ERR_UNSUPPORTED as in
 * qvg_decompress, or when the total exceeds 2^30 tokens per head. */
qvg_status qvg_decompress_chunks(const qvg_record *recs, const int64_t *n_tokens,
                                 int32_t n_chunks, qvg_dtype rec_dtype, int64_t H, int64_t d,
                                 const qvg_params *p, void *out, qvg_dtype out_dtype,
                                 void *stream);

/* ---- single steps of the path (each is one piece of the compress above) ---- */

/* Bytes of workspace qvg_kmeans_assign needs. */
size_t qvg_assign_workspace_size(int64_t H, int64_t N, int64_t d, int32_t C);

/* k-means assignment step (paper.rainbus.top method paragraph, SAS a):
 * assign[h][i] = argmin_j ||r_hi - c_hj||^2 with fp64 distances, ties to the
 * smallest j.  r: device [H][N][d] (dtype); centroids: device fp32 [H][C][d];
 * assign: device uint8 [H][N]. */
qvg_status qvg_kmeans_assign(const void *r, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                             const float *centroids, int32_t C, uint8_t *assign, void *ws,
                             size_t ws_bytes, void *stream);

/* Bytes of workspace qvg_kmeans_update needs. */
size_t qvg_update_workspace_size(int64_t H, int64_t N, int64_t d, int32_t C);

/* k-means update step (note.zhuruihan.top SAS step 2, centroid = mean value):
 * centroids[h][j] = fp32(sum_{i: assign=j} r_hi / n_j) with fp64 sums: the
 * members, in token order, are summed in fp64 in chunks of 64 and the chunk
 * sums are added in order (identical to one sequential fp64 sum whenever the
 * fp64 sums are exact, e.g. for bf16 inputs); the fp64 mean is rounded to
 * fp32.  Clusters with no member keep their value.
 * centroids: device fp32 [H][C][d], read and written. */
qvg_status qvg_kmeans_update(const void *r, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                             const uint8_t *assign, int32_t C, float *centroids, void *ws,
                             size_t ws_bytes, void *stream);

/* Centroid subtraction (paper.rainbus.top method paragraph, SAS c):
 * r_out[h][i] = fp32(r[h][i] - chat[h][assign[h][i]]).  chat: device
 * [H][C][d] in cdtype; r_out: device fp32 [H][N][d] (may alias r when r is
 * fp32). */
qvg_status qvg_sas_subtract(const void *r, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                            const uint8_t *assign, const void *chat, qvg_dtype cdtype, int32_t C,
                            float *r_out, void *stream);

/* Group quantization and packing of a residual (paper.rainbus.top method
 * paragraph, Q) as in qvg_compress.  r: device [H][N][d] (dtype); codes
 * [H][N][d*bits/8]; scales [H][N][d/group]. */
qvg_status qvg_group_quant_pack(const void *r, qvg_dtype dtype, int64_t H, int64_t N, int64_t d,
                                int32_t bits, int32_t group, uint8_t *codes, uint8_t *scales,
                                void *stream);

/* Attention of Nq queries over one compressed history, with the keys and
 * values reconstructed on chip and never written out (note.zhuruihan.top
 * "Algorithm-System Co-design": dequantization fused into the kernels that
 * read the cache; paper.rainbus.top novelty paragraph and the howistudyai.com
 * explainer, "Required resources": keys are cached before the rotary
 * position embedding, which is applied after reconstruction).
 *   q: device fp32 [H][Nq][d], 1 <= Nq <= 16.
 *   k_rec, v_rec: records of the same N tokens (from qvg_compress /
 *   qvg_compress_stream) with params kp and vp, centroids in rec_dtype.
 *   Each key is the bf16 value qvg_decompress(..., QVG_BF16) gives.  Each
 *   value is the reconstruction level * s_hat + C(T)[pi(T)] + ... +
 *   C(1)[pi(1)] taken unrounded (paper.rainbus.top method paragraph, DQ).
 *   rope_cos, rope_sin: device fp32 [N][d/2], both NULL for none; else key
 *   channels k and k + d/2 (k < d/2) become x c - y s and y c + x s, each
 *   product and the difference/sum rounded to fp32, the results to bf16.
 *   out: device fp32 [H][Nq][d] = softmax(scale q K^T) V per head, computed
 *   in fp32, so not bit-reproducible against another summation order (the
 *   same inputs give the same bits on every call).  The order:
 *   - Runs: each head's ntiles = ceil(N/64) tiles of 64 tokens go in runs of
 *     tps = ceil(ntiles / min(ntiles, ceil(2048/H), 1024)) consecutive tiles
 *     (nsplit = ceil(ntiles/tps) runs).
 *   - Scores: a d-term fused multiply-add chain, times scale.
 *   - Output within a run: a fused multiply-add chain over 64*d/256 tokens
 *     per tile, rescaled at most once per tile. The 256/d thread parts are
 *     then added, and the runs merged with one more chain.
 *   - Weight sums (one pass: Nq <= 4 and Nq*T*C <= 4096, values' T and C;
 *     two passes, below: min(Nq, 4)*T*C <= 4096): the value
 *     term sum_n p_n C(t)[pi_t(n)] is taken as sum_c C(t)[c] * (the weights
 *     of the tokens assigned to c). Each weight sum is an add chain over a
 *     run's tokens (rescaled at most once per tile), merged over runs with a
 *     chain, then contracted with the table rows in 2048/d ranges of
 *     T*C*d/2048 rows, added in order.
 *   - Otherwise the values are rebuilt in fp32 (the dequant's fused
 *     multiply-add and adds).
 *   With bf16 centroids, keys of 1 to 4 stages, weight sums, N*2d < 2^32
 *   and H <= 256, the call takes two passes instead (same runs for the
 *   values; every query's weight sums held at once).
 *   The scores first: for one query, d/8 (d/4 for d = 64) fused
 *   multiply-add chains of 16 terms added pairwise, times scale; for 2 to
 *   16 queries, each query split into two bf16 parts, hi = bf16(q) and
 *   lo = bf16(q - hi) (so |q - hi - lo| <= 2^-16 |q|), and the 2d exact
 *   products of the parts with the bf16 key summed in fp32 on the matrix
 *   cores (the hi parts of the 32-channel blocks in order, then the lo
 *   parts; the order within a block is the hardware's), times scale.  Then,
 *   with m the run's largest score, weights e^(s - m) (never rescaled): for
 *   one query, per run a fused multiply-add chain of (weight * s_hat) *
 *   level over 1 token per pass of 64 or 128, the chains of a wave added
 *   pairwise and the 4 waves in order; for 2 to 16 queries, each weight
 *   split into two bf16 parts (|p - hi - lo| <= 2^-16 p) and the products
 *   with s_hat * level (exact in bf16) summed in fp32 on the matrix cores
 *   over the run (per 32-token block the hi parts, then the lo parts).
 *   Weight sums are kept exactly in units of 2^-40 (each weight rounded to
 *   the nearest unit) and rounded to fp32 once per run; runs merged as
 *   above.
 *   ws: device scratch of qvg_attention_workspace_size(H, Nq, N, d, vp)
 *   bytes, 256-byte aligned; all device pointers 16-byte aligned.
 * Errors: QVG_ERR_INVALID_ARG for NULL pointers, one rope table without the
 * other, Nq outside [1, 16] or misaligned pointers; QVG_ERR_UNSUPPORTED as
 * in qvg_decompress for kp or vp; QVG_ERR_WORKSPACE for a small or
 * misaligned workspace.  Inputs must be finite. */
qvg_status qvg_attention(const float *q, int64_t H, int64_t Nq, int64_t d,
                         const qvg_record *k_rec, const qvg_params *kp,
                         const qvg_record *v_rec, const qvg_params *vp, qvg_dtype rec_dtype,
                         int64_t N, float scale, const float *rope_cos, const float *rope_sin,
                         float *out, void *ws, size_t ws_bytes, void *stream);
/* Workspace bytes qvg_attention needs for value params vp; 0 for
 * unsupported sizes. */
size_t qvg_attention_workspace_size(int64_t H, int64_t Nq, int64_t N, int64_t d,
                                    const qvg_params *vp);

/* ---- diagnostics ---- */

/* After a qvg_compress / qvg_compress_stream call that used workspace `ws`
 * with these arguments has completed (this call synchronises the device),
 * copies out[2k] = tokens whose assignment needed the top-2 exact re-check and
 * out[2k+1] = tokens that needed the exact scan over all centroids, for the
 * call's k-means iterations k = 0..n_iters-1 (stage-major; at most 64). */
qvg_status qvg_candidate_counts(const void *ws, int64_t H, int64_t N, int64_t d, qvg_dtype dtype,
                                const qvg_params *p, uint32_t *out, int32_t n_iters);

/* Per-kernel launch timing.  While enabled, every kernel launch of the
 * library is bracketed by two HIP events recorded on its launch stream (the
 * caller's stream).  Kernel names: "kmeans_assign", "kmeans_resolve" (the
 * exact re-checks and scans), "kmeans_sort" and "kmeans_accumulate" (the
 * update of a stage's first iteration, which sorts and sums every member),
 * "kmeans_delta" (the updates of the later iterations, which move only the
 * tokens whose assignment changed where that is exact and cheaper), "kmeans_init",
 * "kmeans_prepare", "kmeans_tables", "absmax", "sas_subtract",
 * "group_quant_pack", "fused_dequant", "attention", "fill".  Host-side
 * bookkeeping only; results of the path are unchanged. */
void qvg_timing_enable(int on);
/* Forget all recorded launches (waits for their events). */
void qvg_timing_reset(void);
/* Waits for the recorded launches of `kernel`, stores the sum of their
 * durations in *total_ms and returns how many there were (-1 on a HIP
 * error). */
int64_t qvg_timing_read(const char *kernel, double *total_ms);

#ifdef __cplusplus
}
#endif

#endif /* QVG_H */
