/*
 * QVG CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, deliberately unoptimised C implementation of what the Quant
 * VideoGen compress/decompress path computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it; the product library
 * never links, calls or reads anything here, and this file shares no code,
 * header, table or helper with the HIP path.
 *
 * Sources (web pages about "Quant VideoGen: Auto-Regressive Long Video
 * Generation via 2-Bit KV-Cache Quantization"):
 *   [SAS]  note.zhuruihan.top, section "Semantic-Aware Smoothing" (k-means on
 *          tokens along the sequence axis, subtract each group's mean);
 *          paper.rainbus.top, method paragraph, steps (a)-(c).
 *   [PRQ]  note.zhuruihan.top, "Progressive Residual Quantization"; paper.rainbus.top
 *          method paragraph: R(0) = X, stage t applies SAS to R(t-1) and yields
 *          R(t), C(t), pi(t); only R(T) is quantized; C(t), pi(t) are stored.
 *   [Q]    paper.rainbus.top method paragraph: symmetric per-group integer
 *          quantization X_INT, S_x = Q(R(T)); note.zhuruihan.top "Algorithm-System
 *          Co-design": per-group scales stored as FP8 E4M3.
 *   [DQ]   paper.rainbus.top method paragraph and note.zhuruihan.top PRQ section:
 *          dequantize, then add back C(t)[pi(t)] from stage T down to stage 1.
 *   [FMT]  howistudyai.com "Step-by-step": assignments stored as uint8 (K=256).
 *
 * Readings taken where the pages are silent:
 *   - distance is squared Euclidean; argmin ties go to the smallest index;
 *   - one k-means iteration = assign then update; the returned pi comes from
 *     the last assign and the returned centroids from the last update;
 *   - an empty cluster keeps its previous centroid;
 *   - values are fp32; distances and centroid sums accumulate in fp64, sums
 *     in token order, distances in channel order;
 *   - centroids are stored rounded to the input dtype (bf16 RNE or fp32), and
 *     that rounded centroid is what is subtracted, so decompression inverts
 *     compression exactly; the fp32 centroid goes to the streaming cache;
 *   - quantization groups are G contiguous channels of one token; the scale is
 *     s = max|r| / (2^b - 1) rounded to the nearest finite E4M3 value (ties to
 *     even code, saturating at 448); codes select the nearest of the 2^b
 *     levels (2q - (2^b - 1)) * s_hat, a tie going to the upper level; s_hat = 0
 *     gives the middle code 2^(b-1) everywhere;
 *   - packing: element k of a token row lives in byte k*b/8 at bit offset
 *     b*(k mod 8/b) (little-endian within the byte).
 *
 * Built with: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread
 * (x86-64 SSE2 arithmetic: fp32 ops round to fp32, fp64 to fp64, no FMA).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define DT_F32 0
#define DT_BF16 1

/* ------------------------------------------------------------------ bf16 */
static float bits_to_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t float_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float qvgo_bf16_to_f32(uint16_t b) { return bits_to_float((uint32_t)b << 16); }

/* Round a finite float to the nearest bf16; on an exact tie pick the
 * candidate whose last mantissa bit is 0.  The two candidates are the value
 * truncated toward zero and the next bf16 away from zero.  Above the largest
 * finite bf16 the next candidate is 2^128 as if the exponent were unbounded;
 * choosing it means overflow, which IEEE 754 round-to-nearest turns into an
 * infinity of the same sign (bits 0x7F80 / 0xFF80). */
uint16_t qvgo_f32_to_bf16(float x)
{
    uint32_t u = float_to_bits(x);
    uint32_t lo = u & 0xFFFF0000u;
    uint32_t hi = lo + 0x10000u;
    double vhi = ((hi & 0x7FFFFFFFu) == 0x7F800000u) ? ldexp(x < 0 ? -1.0 : 1.0, 128)
                                                     : (double)bits_to_float(hi);
    double dlo = fabs((double)x - (double)bits_to_float(lo));
    double dhi = fabs(vhi - (double)x);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1u) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

/* ------------------------------------------------------------- FP8 E4M3 */
/* Value of a non-negative OCP E4M3 ("e4m3fn") code 0..126: exponent bias 7,
 * 3 mantissa bits, subnormals m * 2^-9 when the exponent field is 0. */
double qvgo_e4m3_value(int code)
{
    int e = (code >> 3) & 15, m = code & 7;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp((double)(8 + m), e - 10);
}

/* Nearest finite non-negative E4M3 value to s >= 0 (ties to the even code);
 * values above the largest finite 448 therefore saturate to code 0x7E. */
uint8_t qvgo_e4m3_encode(float s)
{
    int best = 0;
    double bestd = fabs((double)s);
    for (int code = 1; code <= 126; ++code) {
        double d = fabs((double)s - qvgo_e4m3_value(code));
        if (d < bestd || (d == bestd && (code & 1) == 0)) { best = code; bestd = d; }
    }
    return (uint8_t)best;
}

float qvgo_e4m3_decode(uint8_t code)
{
    double v = qvgo_e4m3_value(code & 0x7F);
    return (float)((code & 0x80) ? -v : v);
}

/* --------------------------------------------------------------- k-means */
/* Squared Euclidean distance, fp64, summed over channels in order. */
double qvgo_dist(const float *r, const float *c, int d)
{
    double D = 0.0;
    for (int k = 0; k < d; ++k) {
        double diff = (double)r[k] - (double)c[k];
        D += diff * diff;
    }
    return D;
}

/* [SAS] step (a): each token goes to its nearest centroid, ties to the
 * smallest index. */
void qvgo_assign(const float *R, int64_t N, int d, const float *C, int nC, int32_t *pi)
{
    for (int64_t i = 0; i < N; ++i) {
        int best = 0;
        double bd = qvgo_dist(R + i * d, C, d);
        for (int j = 1; j < nC; ++j) {
            double D = qvgo_dist(R + i * d, C + (int64_t)j * d, d);
            if (D < bd) { bd = D; best = j; }
        }
        pi[i] = best;
    }
}

/* [SAS] step (b): each centroid becomes the mean of its members (fp64 sum in
 * token order, fp64 divide, rounded to fp32); an empty cluster keeps its
 * previous centroid.  counts may be NULL. */
void qvgo_update(const float *R, int64_t N, int d, const int32_t *pi, int nC, float *C,
                 int64_t *counts)
{
    double *sum = (double *)calloc((size_t)nC * d, sizeof(double));
    int64_t *cnt = (int64_t *)calloc((size_t)nC, sizeof(int64_t));
    for (int64_t i = 0; i < N; ++i) {
        int j = pi[i];
        cnt[j] += 1;
        for (int k = 0; k < d; ++k) sum[(int64_t)j * d + k] += (double)R[i * d + k];
    }
    for (int j = 0; j < nC; ++j) {
        if (cnt[j] > 0)
            for (int k = 0; k < d; ++k)
                C[(int64_t)j * d + k] = (float)(sum[(int64_t)j * d + k] / (double)cnt[j]);
        if (counts) counts[j] = cnt[j];
    }
    free(sum);
    free(cnt);
}

/* [SAS] step (c): residual of each token, r - C[pi(r)], one fp32 subtraction
 * per element; C given as fp32 values (already rounded to the storage dtype). */
void qvgo_subtract(const float *R, int64_t N, int d, const int32_t *pi, const float *C,
                   float *out)
{
    for (int64_t i = 0; i < N; ++i)
        for (int k = 0; k < d; ++k)
            out[i * d + k] = R[i * d + k] - C[(int64_t)pi[i] * d + k];
}

/* The assignment of tokens [lo, hi) by one thread (each token's argmin is
 * independent of the others, so splitting the tokens changes nothing). */
typedef struct {
    const float *R; int64_t lo, hi; int d; const float *C; int nC; int32_t *pi;
} assign_part_t;

static void *assign_part(void *arg)
{
    assign_part_t *a = (assign_part_t *)arg;
    qvgo_assign(a->R + a->lo * a->d, a->hi - a->lo, a->d, a->C, a->nC, a->pi + a->lo);
    return NULL;
}

static void assign_threads(const float *R, int64_t N, int d, const float *C, int nC, int32_t *pi,
                           int nthreads)
{
    if (nthreads <= 1 || N < 2 * nthreads) {
        qvgo_assign(R, N, d, C, nC, pi);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    assign_part_t *parts = (assign_part_t *)malloc(sizeof(assign_part_t) * nthreads);
    for (int t = 0; t < nthreads; ++t) {
        parts[t].R = R; parts[t].d = d; parts[t].C = C; parts[t].nC = nC; parts[t].pi = pi;
        parts[t].lo = N * t / nthreads;
        parts[t].hi = N * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, assign_part, &parts[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(parts);
}

/* Lloyd's k-means from the given initial centroids: iters x (assign, update);
 * the assignment may use `threads` threads over token ranges. */
static void kmeans_threads(const float *R, int64_t N, int d, float *C, int nC, int iters,
                           int32_t *pi, int threads)
{
    for (int it = 0; it < iters; ++it) {
        assign_threads(R, N, d, C, nC, pi, threads);
        qvgo_update(R, N, d, pi, nC, C, NULL);
    }
}

void qvgo_kmeans(const float *R, int64_t N, int d, float *C, int nC, int iters, int32_t *pi)
{
    kmeans_threads(R, N, d, C, nC, iters, pi, 1);
}

/* ------------------------------------------------------ seeded sampler */
/* Cold-start rows of stage t (1-based) of head h (0-based): C distinct token
 * indices drawn without replacement.  The pages only say the initial
 * centroids are seeded token rows; the draw is pinned as follows.
 * splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014; constants as published by Vigna): the state advances
 * by 0x9E3779B97F4A7C15 and each output is the state passed through two
 * xor-shift-multiply rounds and a final xor-shift.  All arithmetic is
 * modulo 2^64. */
uint64_t qvgo_splitmix64(uint64_t *state)
{
    uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* The generator of (seed, h, t) starts from seed ^ (0x9E3779B97F4A7C15 *
 * (h+1)) ^ (0xD1B54A32D192ED03 * t).  A partial Fisher-Yates shuffle of
 * perm = 0..N-1 then picks the rows: for j = 0..C-1 it swaps perm[j] with
 * perm[j + (next() mod (N - j))], and row j is perm[j].  (The slight
 * modulo bias is part of the definition.)  Requires 1 <= C <= N. */
void qvgo_sample_rows(int64_t N, int C, uint64_t seed, int64_t h, int t, int32_t *rows)
{
    int32_t *perm = (int32_t *)malloc((size_t)N * sizeof(int32_t));
    uint64_t st = seed ^ (0x9E3779B97F4A7C15ull * (uint64_t)(h + 1)) ^
                  (0xD1B54A32D192ED03ull * (uint64_t)t);
    for (int64_t i = 0; i < N; ++i) perm[i] = (int32_t)i;
    for (int j = 0; j < C; ++j) {
        uint64_t r = qvgo_splitmix64(&st) % (uint64_t)(N - j);
        int64_t k = j + (int64_t)r;
        int32_t tmp = perm[j];
        perm[j] = perm[k];
        perm[k] = tmp;
        rows[j] = perm[j];
    }
    free(perm);
}

/* ---------------------------------------------------------- quantization */
/* [Q] symmetric per-group quantization of one token row r[0..d) with b bits
 * and G channels per group, writing packed codes (d*b/8 bytes) and E4M3
 * scale bytes (d/G). */
void qvgo_quantize_row(const float *r, int d, int bits, int G, uint8_t *codes, uint8_t *scales)
{
    const int levels = (1 << bits) - 1; /* 2^b - 1 */
    const int mid = 1 << (bits - 1);
    const int per_byte = 8 / bits;
    memset(codes, 0, (size_t)d * bits / 8);
    for (int g = 0; g < d / G; ++g) {
        float a = 0.0f;
        for (int k = g * G; k < (g + 1) * G; ++k) {
            float v = fabsf(r[k]);
            if (v > a) a = v;
        }
        float s = a / (float)levels;
        uint8_t e = qvgo_e4m3_encode(s);
        float sh = qvgo_e4m3_decode(e);
        scales[g] = e;
        for (int k = g * G; k < (g + 1) * G; ++k) {
            int q;
            if (sh == 0.0f) {
                q = mid;
            } else {
                float u = r[k] / sh;
                q = (int)floor((double)u / 2.0) + mid;
                if (q < 0) q = 0;
                if (q > levels) q = levels;
            }
            codes[k / per_byte] |= (uint8_t)(q << (bits * (k % per_byte)));
        }
    }
}

/* Dequantized level of element k of a row (before any centroid is added). */
static float dequant_elem(const uint8_t *codes, const uint8_t *scales, int k, int bits, int G)
{
    const int per_byte = 8 / bits;
    int q = (codes[k / per_byte] >> (bits * (k % per_byte))) & ((1 << bits) - 1);
    float sh = qvgo_e4m3_decode(scales[k / G]);
    return (float)(2 * q - ((1 << bits) - 1)) * sh;
}

void qvgo_quantize(const float *R, int64_t N, int d, int bits, int G, uint8_t *codes,
                   uint8_t *scales)
{
    for (int64_t i = 0; i < N; ++i)
        qvgo_quantize_row(R + i * d, d, bits, G, codes + i * (d * bits / 8), scales + i * (d / G));
}

/* ------------------------------------------------------- whole-path, per head */
typedef struct {
    int C, T, iters, bits, G;
    int assign_threads; /* threads of one head's assignment step */
} qvgo_params;

static float load_val(const void *base, int dtype, int64_t idx)
{
    if (dtype == DT_BF16) return qvgo_bf16_to_f32(((const uint16_t *)base)[idx]);
    return ((const float *)base)[idx];
}

static float round_store(float v, int dtype, void *base, int64_t idx)
{
    if (dtype == DT_BF16) {
        uint16_t b = qvgo_f32_to_bf16(v);
        ((uint16_t *)base)[idx] = b;
        return qvgo_bf16_to_f32(b);
    }
    ((float *)base)[idx] = v;
    return v;
}

/* [PRQ] + [Q] for one head-tensor X[N][d].
 * Stage t (0-based) initialises from rows init_idx[t][0..C) of R(t-1) when
 * init_idx is non-NULL, else from init_c[t] (fp32 [C][d]).
 * Outputs: codes [N][d*b/8], scales [N][d/G], assign [T][N] (uint8),
 * cent [T][C][d] in the input dtype, cache [T][C][d] fp32 (may be NULL). */
static void compress_head(const void *X, int dtype, int64_t N, int d, const qvgo_params *p,
                          const int32_t *init_idx, const float *init_c, int seeded,
                          uint64_t seed, int64_t h, uint8_t *codes, uint8_t *scales,
                          uint8_t *assign, void *cent, float *cache)
{
    const int C = p->C;
    float *R = (float *)malloc((size_t)N * d * sizeof(float));
    float *Cc = (float *)malloc((size_t)C * d * sizeof(float));
    float *Ch = (float *)malloc((size_t)C * d * sizeof(float));
    int32_t *pi = (int32_t *)malloc((size_t)N * sizeof(int32_t));
    for (int64_t i = 0; i < N * d; ++i) R[i] = load_val(X, dtype, i);

    int32_t *rows = (int32_t *)malloc((size_t)C * sizeof(int32_t));
    for (int t = 0; t < p->T; ++t) {
        if (init_idx || seeded) {
            /* rows of R(t-1): the stage input, i.e. the previous stage's residual */
            if (seeded) qvgo_sample_rows(N, C, seed, h, t + 1, rows);
            else memcpy(rows, init_idx + (int64_t)t * C, (size_t)C * sizeof(int32_t));
            for (int j = 0; j < C; ++j)
                memcpy(Cc + (int64_t)j * d, R + (int64_t)rows[j] * d, d * sizeof(float));
        } else {
            memcpy(Cc, init_c + (int64_t)t * C * d, (size_t)C * d * sizeof(float));
        }
        kmeans_threads(R, N, d, Cc, C, p->iters, pi, p->assign_threads);
        if (cache) memcpy(cache + (int64_t)t * C * d, Cc, (size_t)C * d * sizeof(float));
        for (int64_t q = 0; q < (int64_t)C * d; ++q)
            Ch[q] = round_store(Cc[q], dtype, cent, (int64_t)t * C * d + q);
        for (int64_t i = 0; i < N; ++i) {
            assign[(int64_t)t * N + i] = (uint8_t)pi[i];
            for (int k = 0; k < d; ++k) R[i * d + k] = R[i * d + k] - Ch[(int64_t)pi[i] * d + k];
        }
    }
    qvgo_quantize(R, N, d, p->bits, p->G, codes, scales);
    free(rows);
    free(R);
    free(Cc);
    free(Ch);
    free(pi);
}

/* [DQ] for one head: x = level * s_hat, then + C(t)[pi(t)] for t = T..1, in
 * fp32, rounded once to the output dtype. */
static void decompress_head(const uint8_t *codes, const uint8_t *scales, const uint8_t *assign,
                            const void *cent, int cdtype, int64_t N, int d, const qvgo_params *p,
                            void *out, int odtype)
{
    const int rowb = d * p->bits / 8, rows = d / p->G;
    for (int64_t i = 0; i < N; ++i) {
        for (int k = 0; k < d; ++k) {
            float v = dequant_elem(codes + i * rowb, scales + i * rows, k, p->bits, p->G);
            for (int t = p->T - 1; t >= 0; --t) {
                int j = assign[(int64_t)t * N + i];
                v = v + load_val(cent, cdtype, ((int64_t)t * p->C + j) * d + k);
            }
            round_store(v, odtype, out, i * d + k);
        }
    }
}

/* ------------------------------------------------------ threads over heads */
typedef struct {
    int mode; /* 0 compress, 1 decompress */
    int tid, nthreads;
    const void *X; int dtype; int64_t H, N; int d; qvgo_params p;
    const int32_t *init_idx; const float *init_c; int seeded; uint64_t seed;
    uint8_t *codes, *scales, *assign; void *cent; float *cache;
    void *out; int odtype;
} job_t;

static size_t esize(int dtype) { return dtype == DT_BF16 ? 2 : 4; }

static void *worker(void *arg)
{
    job_t *j = (job_t *)arg;
    const int64_t N = j->N, d = j->d, C = j->p.C, T = j->p.T;
    const int64_t rowb = d * j->p.bits / 8, rows = d / j->p.G;
    for (int64_t h = j->tid; h < j->H; h += j->nthreads) {
        uint8_t *codes = j->codes + h * N * rowb;
        uint8_t *scales = j->scales + h * N * rows;
        uint8_t *assign = j->assign + h * T * N;
        char *cent = (char *)j->cent + h * T * C * d * esize(j->dtype);
        if (j->mode == 0) {
            compress_head((const char *)j->X + h * N * d * esize(j->dtype), j->dtype, N, (int)d,
                          &j->p, j->init_idx ? j->init_idx + h * T * C : NULL,
                          j->init_c ? j->init_c + h * T * C * d : NULL, j->seeded, j->seed, h,
                          codes, scales, assign, cent,
                          j->cache ? j->cache + h * T * C * d : NULL);
        } else {
            decompress_head(codes, scales, assign, cent, j->dtype, N, (int)d, &j->p,
                            (char *)j->out + h * N * d * esize(j->odtype), j->odtype);
        }
    }
    return NULL;
}

static void run_jobs(job_t *proto, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * nthreads);
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].tid = t;
        jobs[t].nthreads = nthreads;
        pthread_create(&th[t], NULL, worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/* Whole compress over H head-tensors X[H][N][d] (dtype 0 = fp32, 1 = bf16).
 * Stage starts: init_idx [H][T][C] int32 rows, else init_c [H][T][C][d] fp32,
 * else (both NULL) rows drawn by qvgo_sample_rows(N, C, seed, h, t).
 * codes [H][N][d*b/8], scales [H][N][d/G], assign [H][T][N], cent [H][T][C][d]
 * (input dtype), cache [H][T][C][d] fp32 or NULL. */
void qvgo_compress(const void *X, int dtype, int64_t H, int64_t N, int d, int C, int T,
                   int iters, int bits, int G, const int32_t *init_idx, const float *init_c,
                   uint64_t seed, uint8_t *codes, uint8_t *scales, uint8_t *assign, void *cent,
                   float *cache, int nthreads)
{
    job_t j;
    memset(&j, 0, sizeof j);
    j.mode = 0; j.X = X; j.dtype = dtype; j.H = H; j.N = N; j.d = d;
    j.p.C = C; j.p.T = T; j.p.iters = iters; j.p.bits = bits; j.p.G = G;
    j.init_idx = init_idx; j.init_c = init_c;
    j.seeded = init_idx == NULL && init_c == NULL; j.seed = seed;
    /* fewer heads than threads: the spare threads split each head's tokens */
    if (nthreads < 1) nthreads = 1;
    j.p.assign_threads = H < nthreads ? (int)(nthreads / H) : 1;
    if (H < nthreads) nthreads = (int)H;
    j.codes = codes; j.scales = scales; j.assign = assign; j.cent = cent; j.cache = cache;
    run_jobs(&j, nthreads);
}

/* Whole decompress: centroids in cdtype, output in odtype. */
void qvgo_decompress(const uint8_t *codes, const uint8_t *scales, const uint8_t *assign,
                     const void *cent, int cdtype, int64_t H, int64_t N, int d, int C, int T,
                     int bits, int G, void *out, int odtype, int nthreads)
{
    job_t j;
    memset(&j, 0, sizeof j);
    j.mode = 1; j.dtype = cdtype; j.H = H; j.N = N; j.d = d;
    j.p.C = C; j.p.T = T; j.p.bits = bits; j.p.G = G;
    j.codes = (uint8_t *)codes; j.scales = (uint8_t *)scales; j.assign = (uint8_t *)assign;
    j.cent = (void *)cent; j.out = out; j.odtype = odtype;
    run_jobs(&j, nthreads);
}
