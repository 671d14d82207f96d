/*
 * Seeded synthetic inputs for the FP8 W8A8 linear layer.
 *
 * This module only draws random numbers and lays them out; it holds none of
 * the quantization or GEMM arithmetic.  Both the CPU oracle and the HIP path
 * consume the buffers it fills, so the two sides see identical inputs.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used counter-style: the i-th draw of a
 * stream is the i-th output of a SplitMix64 sequence whose state starts at
 * the stream key, so any element can be produced independently (and in
 * parallel) from (key, i).  Uniforms take the top 53 bits, offset by half an
 * ulp so they lie strictly inside (0, 1).  Normals use the Box-Muller
 * transform on consecutive uniform pairs.
 *
 * Distributions (the workloads of the "unified low-precision dataflow" pages:
 * Llama-3 / DeepSeek-style linear layers with per-token activations and
 * per-output-channel weight magnitudes):
 *   activations  x[m,k] ~ N(0,1), with a fixed set of outlier channels
 *                (the same columns for every token) multiplied by a factor;
 *   weights      w[n,k] = 0.02 * z[n,k] * exp(0.5 * g[n]), z, g ~ N(0,1)
 *                (log-normal(0, 0.5) magnitude per output channel);
 *   MoE routing  each token picks `topk` distinct experts with Zipf(s)
 *                weights p_r ~ r^-s (expert id = rank - 1), sampled without
 *                replacement by Efraimidis-Spirakis keys u^(1/p).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* i-th output (0-based) of SplitMix64 started at state `key`. */
static inline uint64_t sm64_at(uint64_t key, uint64_t i) {
    return sm64_mix(key + (i + 1) * SM64_GAMMA);
}

/* Key of sub-stream `stream` under `seed`: distinct tensors never share draws. */
uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
    return sm64_at(sm64_mix(seed ^ 0x5DEECE66DULL), stream);
}

static inline double u01(uint64_t key, uint64_t i) {
    return ((double)(sm64_at(key, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* i-th standard normal of the stream: Box-Muller on the uniform pair (2j, 2j+1). */
static inline double normal_at(uint64_t key, uint64_t i) {
    uint64_t j = i >> 1;
    double u1 = u01(key, 2 * j), u2 = u01(key, 2 * j + 1);
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(t) : r * cos(t);
}

uint64_t synth_u64(uint64_t key, uint64_t i) { return sm64_at(key, i); }
double synth_uniform(uint64_t key, uint64_t i) { return u01(key, i); }
double synth_normal(uint64_t key, uint64_t i) { return normal_at(key, i); }

/* out[i] = mul * N_(offset+i), i < n. */
void synth_normal_f32(uint64_t key, uint64_t offset, int64_t n, float mul, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(mul * normal_at(key, offset + (uint64_t)i));
}

/* Choose `count` distinct indices of [0, n) (partial Fisher-Yates), written sorted. */
void synth_choose(uint64_t key, int64_t n, int64_t count, int64_t* chosen) {
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) perm[i] = i;
    for (int64_t i = 0; i < count && i < n; ++i) {
        uint64_t span = (uint64_t)(n - i);
        int64_t j = i + (int64_t)(sm64_at(key, (uint64_t)i) % span);
        int64_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
    for (int64_t i = 0; i < count; ++i) chosen[i] = perm[i];
    /* insertion sort: count is small */
    for (int64_t i = 1; i < count; ++i) {
        int64_t v = chosen[i], j = i - 1;
        while (j >= 0 && chosen[j] > v) { chosen[j + 1] = chosen[j]; --j; }
        chosen[j + 1] = v;
    }
    free(perm);
}

/*
 * Activations X [M, K] (row stride ldx), N(0,1) with `n_out` outlier columns
 * scaled by `out_mult`.  Streams: base for the values, base+1 for the columns.
 * `cols` (n_out entries, may be NULL) receives the chosen columns.
 */
void synth_activations(uint64_t seed, uint64_t stream, int64_t M, int64_t K, int64_t ldx,
                       int64_t n_out, float out_mult, float* x, int64_t* cols) {
    uint64_t kv = synth_stream_key(seed, stream), kc = synth_stream_key(seed, stream + 1);
    int64_t* c = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_out > 0 ? n_out : 1));
    synth_choose(kc, K, n_out, c);
    char* is_out = (char*)calloc((size_t)(K > 0 ? K : 1), 1);
    for (int64_t i = 0; i < n_out; ++i) is_out[c[i]] = 1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            double v = normal_at(kv, (uint64_t)(m * K + k));
            if (is_out[k]) v *= (double)out_mult;
            x[m * ldx + k] = (float)v;
        }
    }
    if (cols) memcpy(cols, c, sizeof(int64_t) * (size_t)n_out);
    free(is_out);
    free(c);
}

/*
 * Weights W [N, K] (row stride ldw): 0.02 * z[n,k] * exp(0.5 * g[n]).
 * Rows [n0, n0+N) of the stream (so a big matrix can be drawn in slabs).
 * Streams: base for z, base+1 for g.
 */
void synth_weights(uint64_t seed, uint64_t stream, int64_t n0, int64_t N, int64_t K, int64_t ldw,
                   float* w) {
    uint64_t kz = synth_stream_key(seed, stream), kg = synth_stream_key(seed, stream + 1);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        int64_t gn = n0 + n;
        double mag = 0.02 * exp(0.5 * normal_at(kg, (uint64_t)gn));
        for (int64_t k = 0; k < K; ++k)
            w[n * ldw + k] = (float)(mag * normal_at(kz, (uint64_t)(gn * K + k)));
    }
}

/*
 * MoE routing: T tokens, E experts, `topk` distinct experts per token with
 * Zipf(s) weights over expert rank.  Outputs (expert-sorted routed rows, rows
 * of one expert in token order):
 *   token_expert [T*topk]  chosen experts of token t, by decreasing key
 *   row_token    [T*topk]  source token of routed row r
 *   offsets      [E+1]     rows of expert e are [offsets[e], offsets[e+1])
 * Returns 0, or -1 when topk > E or topk > 64.
 */
int synth_routing(uint64_t seed, uint64_t stream, int64_t T, int64_t E, int64_t topk, double s,
                  int32_t* token_expert, int32_t* row_token, int32_t* offsets) {
    if (topk > E || topk < 0 || topk > 64 || E <= 0) return -1;
    uint64_t ku = synth_stream_key(seed, stream);
    double* logw = (double*)malloc(sizeof(double) * (size_t)E);
    for (int64_t e = 0; e < E; ++e) logw[e] = -s * log((double)(e + 1));
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        /* Efraimidis-Spirakis: key = u^(1/w), compared as log(u)/w. */
        double best_key[64];
        int32_t best_e[64];
        int64_t nb = 0;
        for (int64_t e = 0; e < E; ++e) {
            double key = log(u01(ku, (uint64_t)(t * E + e))) / exp(logw[e]);
            if (nb < topk) {
                int64_t j = nb++;
                while (j > 0 && best_key[j - 1] < key) { best_key[j] = best_key[j - 1]; best_e[j] = best_e[j - 1]; --j; }
                best_key[j] = key; best_e[j] = (int32_t)e;
            } else if (topk > 0 && key > best_key[topk - 1]) {
                int64_t j = topk - 1;
                while (j > 0 && best_key[j - 1] < key) { best_key[j] = best_key[j - 1]; best_e[j] = best_e[j - 1]; --j; }
                best_key[j] = key; best_e[j] = (int32_t)e;
            }
        }
        for (int64_t i = 0; i < topk; ++i) token_expert[t * topk + i] = best_e[i];
    }
    /* counting sort of the routed rows by expert, stable in token order */
    for (int64_t e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t i = 0; i < T * topk; ++i) offsets[token_expert[i] + 1] += 1;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int64_t e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int64_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < topk; ++i) row_token[fill[token_expert[t * topk + i]]++] = (int32_t)t;
    free(fill);
    free(logw);
    return 0;
}

/*
 * KV activations [T, C] (row stride ld): N(0,1) times a per-channel gain
 * exp(0.5 g_c), g_c ~ N(0,1), with `n_out` outlier channels further scaled by
 * `out_mult`.  Streams: base (values), base+1 (gains), base+2 (outliers).
 */
void synth_kv(uint64_t seed, uint64_t stream, int64_t T, int64_t C, int64_t ld, int64_t n_out, float out_mult,
              float* kv) {
    uint64_t kz = synth_stream_key(seed, stream), kg = synth_stream_key(seed, stream + 1);
    uint64_t kc = synth_stream_key(seed, stream + 2);
    double* gain = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    int64_t* c = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_out > 0 ? n_out : 1));
    for (int64_t j = 0; j < C; ++j) gain[j] = exp(0.5 * normal_at(kg, (uint64_t)j));
    synth_choose(kc, C, n_out, c);
    for (int64_t i = 0; i < n_out; ++i) gain[c[i]] *= (double)out_mult;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < C; ++j) kv[t * ld + j] = (float)(gain[j] * normal_at(kz, (uint64_t)(t * C + j)));
    free(c);
    free(gain);
}

/* A uniformly random permutation of 0..n-1 (Fisher-Yates). */
void synth_permutation(uint64_t key, int64_t n, int64_t* perm) {
    for (int64_t i = 0; i < n; ++i) perm[i] = i;
    for (int64_t i = n - 1; i > 0; --i) {
        int64_t j = (int64_t)(sm64_at(key, (uint64_t)i) % (uint64_t)(i + 1));
        int64_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
}
