/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle of the DeepSeek Sparse Attention (DSA)
 * indexer hot path: store (RMSNorm -> RoPE -> fp8/bf16 paged store), score (per-head dot,
 * ReLU, weighted head sum over causally visible compressed keys) and top-k selection.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code with the HIP kernels: no headers, helpers, tables or
 * constant generators.  Everything is computed in fp64 with plain loops; the only rounding steps
 * are the ones the stored formats define (fp32 canonical key, bf16, fp8 e4m3, fp32 scale).
 *
 * Sources (the four blog pages on the DSA indexer):
 *  - "When the Fused Kernel Isn't Enough", Input Knowledge Required: the indexer has a store path
 *    that writes compressed keys and a read path that computes logits; fp8 keys are 128 B of codes
 *    plus a 4 B scale (132 B/token), bf16 keys are 256 B/token.
 *  - "The Moment of Validation", Input Knowledge Required: the fused kernel normalises, applies
 *    RoPE and stores; fp8 keys carry a shared scale per group; bf16 storage has no quantisation.
 *  - "The Crash That Changed Direction", Experiment / Assumptions / Input Knowledge: scores are a
 *    batched q.k product followed by ReLU over the head dimension, then top-k; keys are e4m3.
 *  - "The Fused Kernel Decision", Message / Assumptions: the indexer cache is paged, 64 tokens per
 *    page, [npages, 64*128]; a token maps to (page, offset); q and k must share one element order.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - RMSNorm over all 128 dims with eps passed in, then RoPE (theta = 1e4) on dims 64..127 as
 *    interleaved pairs (64+2j, 65+2j) at position 4s; inv_freq_j = fp32(theta^(-2j/64)).
 *  - canonical key k32 = fp32 round-to-nearest-even of the fp64 result.
 *  - bf16 code = round-to-nearest-even of k32.
 *  - fp8: scale = fp32(absmax(k32) / 448); code_i = e4m3fn RNE (saturating) of fp32(k32_i / scale);
 *    scale = 0 and codes 0x00 for an all-zero key.  Page = 64 x 128 code bytes then 64 fp32
 *    scales (8448 B).
 *  - visibility: key s is visible to the query at token t iff 4s + 3 <= t, i.e. s < (t+1)/4;
 *    queries of sequence b are its last q_len_b tokens.
 *  - logit(t, s) = sum_h w[t,h] * max(0, sum_i q[t,h,i] * k[s,i]), no softmax scale.
 *  - top-k: the k largest logits of a row, ties to the lower s; rows with fewer than k entries are
 *    padded with index -1 and value -inf.
 *  - keys whose page-table entry lies outside the pool score -inf; keys with an out-of-range
 *    sequence, index or page are not stored.
 *  - the rotated store ("The Fused Kernel Decision", Assumptions: the Hadamard transform's output
 *    order is kept through the pipeline so that q and k stay aligned; "When the Fused Kernel
 *    Isn't Enough", the fused vs. non-fused paths: normalisation, RoPE, Hadamard transform and
 *    store in one kernel): after RoPE, the 128 dims are multiplied by the normalised Sylvester
 *    Walsh-Hadamard matrix H / sqrt(128), H[i][j] = (-1)^popcount(i & j), computed in fp64 as the
 *    fast transform (butterfly stages of spans 1, 2, ..., 64, (a, b) -> (a + b, a - b)) followed
 *    by one multiplication with the fp64 value of 2^-3.5; the canonical key is the fp32 rounding
 *    of that.  q is rotated by the same map (fp64, then fp32, then bf16 RNE) so that q.k is kept.
 *  - fp4 keys ("The Fused Kernel Decision", Input Knowledge: the indexer also has an fp4 variant
 *    for more aggressive compression; its format is not given): OCP e2m1 codes, RNE, saturating
 *    at +-6, with one fp32 scale per key, fp32(absmax / 6), the fp8 rule with 6 for 448; dims 2i
 *    and 2i+1 in the low and high nibble of byte i; page = 64 x 64 code bytes, then 64 scales
 *    (4352 B, 68 B per key).
 *  - sparse attention over the selected keys ("When the Fused Kernel Isn't Enough", Input
 *    Knowledge: the sparse attention attends to the top-K entries the indexer picks, and the main
 *    KV cache is bf16 with head_dim 512; "The Fused Kernel Decision", Message: that cache is
 *    unpaged, [num_slots, 512] bf16, one slot per entry): for query row i of sequence b and head
 *    h, each listed entry j with 0 <= idx[i][j] < max_keys whose slot kv_slot[b][idx] lies in
 *    [0, n_slots) contributes the 512-dim latent v_j = kv[slot]; logit_j = scale * q[i][h] . v_j,
 *    o[i][h] = sum_j softmax(logit)_j * v_j (the latent is key and value, shared by all heads),
 *    lse[i][h] = log sum_j exp(logit_j).  No listed entry: o = 0, lse = -inf.
 *  - fp8 x fp8 scoring ("The Crash That Changed Direction", Experiment: fp8 keys go into the
 *    product; the read path as a matrix product over heads): q of each (query, head) is quantised
 *    like a key (one fp32 scale = absmax / 448, e4m3 codes of q_i / scale) and the logit is
 *    sum_h w_h * max(0, sum_i (code_q * scale_q) * (code_k * scale_k)) with both operands taken
 *    exactly in fp64.  The pages never quantise q; this variant is the fp8 product itself.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_D 128          /* index-key head dim */
#define OR_H 64           /* indexer heads */
#define OR_PAGE 64        /* keys per cache page */
#define OR_RATIO 4        /* tokens per compressed key ("c4") */
#define OR_FP8 0
#define OR_BF16 1
#define OR_FP4 2          /* e2m1 codes, two per byte, then one fp32 scale per key */
#define OR_DV 512         /* main-KV latent dim of the sparse attention */

/* Planted-mistake switch used only by the test that checks the pins catch mistakes. 0 = none. */
static int g_mutation = 0;
void oracle_set_mutation(int m) { g_mutation = m; }
int oracle_get_mutation(void) { return g_mutation; }

/* Threads the OpenMP loops below run on. */
int oracle_num_threads(void) { return omp_get_max_threads(); }

int64_t oracle_page_bytes(int dtype) {
    if (dtype == OR_FP4) return (int64_t)OR_PAGE * (OR_D / 2 + 4);
    return dtype == OR_FP8 ? (int64_t)OR_PAGE * (OR_D + 4) : (int64_t)OR_PAGE * OR_D * 2;
}

/* ---------------------------------------------------------------------------------------------
 * Number formats
 * ------------------------------------------------------------------------------------------- */

/* OCP FP8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; S.1111.111 is NaN.
 * Normal: 2^(E-7) * (1 + M/8); subnormal (E = 0): 2^-6 * M/8. */
double oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round v to the nearest e4m3fn value, ties to the even code, saturating at +-448.  The 127
 * non-negative finite magnitudes increase with the code, so a binary search finds the pair that
 * brackets |v|; the two distances are exact in fp64. */
uint8_t oracle_e4m3_encode(float v) {
    double a = fabs((double)v);
    int sign = signbit(v) ? 1 : 0;
    int c;
    if (a >= oracle_e4m3_decode(126)) {
        c = 126;
    } else {
        int lo = 0, hi = 126;              /* mag(lo) <= a < mag(hi) */
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
        }
        double dlo = a - oracle_e4m3_decode((uint8_t)lo);
        double dhi = oracle_e4m3_decode((uint8_t)hi) - a;
        if (dlo < dhi) c = lo;
        else if (dhi < dlo) c = hi;
        else if (g_mutation == 9) c = hi;                /* planted: ties away from zero */
        else c = (lo % 2 == 0) ? lo : hi;
    }
    return (uint8_t)(c | (sign << 7));
}

/* OCP FP4 e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no infinities or NaN; largest 6.
 * Normal (E > 0): 2^(E-1) * (1 + M/2); subnormal (E = 0): M / 2.  Code bits: S.EE.M. */
double oracle_e2m1_decode(uint8_t c) {
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = e ? ldexp(1.0 + (double)m / 2.0, e - 1) : (double)m / 2.0;
    return s ? -v : v;
}

/* Nearest e2m1 value, ties to the even code, saturating at +-6: the 8 magnitudes increase with
 * the code, so the bracketing pair is found by a scan; distances are exact in fp64. */
uint8_t oracle_e2m1_encode(float v) {
    double a = fabs((double)v);
    int sign = signbit(v) ? 1 : 0;
    int c;
    if (a >= 6.0) {
        c = 7;
    } else {
        int lo = 0;
        while (lo < 6 && oracle_e2m1_decode((uint8_t)(lo + 1)) <= a) lo++;
        int hi = lo + 1;                      /* mag(lo) <= a < mag(hi) */
        double dlo = a - oracle_e2m1_decode((uint8_t)lo);
        double dhi = oracle_e2m1_decode((uint8_t)hi) - a;
        if (dlo < dhi) c = lo;
        else if (dhi < dlo) c = hi;
        else if (g_mutation == 19) c = hi;                /* planted: ties away from zero */
        else c = (lo % 2 == 0) ? lo : hi;
    }
    return (uint8_t)(c | (sign << 3));
}

static double bf16_bits_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* bfloat16 = the upper 16 bits of an fp32 pattern.  Round a finite fp32 to the nearest bf16,
 * ties to the even pattern: compare the two candidates that bracket it. */
uint16_t oracle_bf16_encode(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    uint16_t lo = (uint16_t)(u >> 16);        /* truncation: the neighbour toward zero */
    uint16_t hi = (uint16_t)(lo + 1);         /* next magnitude away from zero */
    double a = fabs((double)v);
    double dlo = a - fabs(bf16_bits_value(lo));
    double dhi = fabs(bf16_bits_value(hi)) - a;
    if (g_mutation == 11) return lo;          /* planted: truncation instead of RNE */
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1) == 0 ? lo : hi;
}

/* ---------------------------------------------------------------------------------------------
 * S1: RMSNorm -> RoPE -> canonical fp32 key -> bf16 or fp8 + scale, scattered to a paged pool.
 * ------------------------------------------------------------------------------------------- */

void oracle_rope_inv_freq(float out[32]) {
    for (int j = 0; j < 32; j++) out[j] = (float)pow(10000.0, -(2.0 * j) / 64.0);
}

/* 2^-3.5 = sqrt(2^-7): the square root of an exact power of two, correctly rounded. */
double oracle_hadamard_scale(void) { return sqrt(1.0 / 128.0); }

/* In-place normalised Walsh-Hadamard transform of 128 fp64 values (Sylvester order): butterfly
 * stages of span h = 1, 2, 4, ..., 64, each mapping (v[i], v[i+h]) to (v[i] + v[i+h],
 * v[i] - v[i+h]) for every i whose bit h is clear, then one multiplication by 2^-3.5. */
void oracle_hadamard128(double* v) {
    const double c = oracle_hadamard_scale();
    for (int h = 1; h < OR_D; h *= 2) {
        if (g_mutation == 14 && h == 8) continue;                 /* planted: a stage skipped */
        for (int i = 0; i < OR_D; i++) {
            if (i & h) continue;
            double a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = (g_mutation == 15) ? b - a : a - b;        /* planted: difference sign */
        }
    }
    for (int i = 0; i < OR_D; i++) v[i] *= (g_mutation == 16) ? 1.0 / 128.0 : c;  /* planted */
}

/* q rotated like the keys: each 128-dim bf16 vector to fp64, transformed, rounded to fp32 and
 * then to bf16 (nearest-even). */
void oracle_rotate_q(const uint16_t* q, int64_t n_vec, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_vec; n++) {
        double v[OR_D];
        for (int i = 0; i < OR_D; i++) v[i] = bf16_bits_value(q[n * OR_D + i]);
        oracle_hadamard128(v);
        for (int i = 0; i < OR_D; i++) out[n * OR_D + i] = oracle_bf16_encode((float)v[i]);
    }
}

/* The canonical key of one row: fp64 RMSNorm over the 128 dims, scaled by gamma, then rotation of
 * the interleaved pairs of dims 64..127 by angle (4s) * inv_freq_j, then (rotated store) the
 * normalised Hadamard transform, rounded once to fp32. */
static void canonical_key(const float* x, const float* gamma, float eps, int32_t s,
                          const float* inv_freq, int hadamard, float* k32) {
    double y[OR_D];
    double ss = 0.0;
    int n_norm = (g_mutation == 3) ? 64 : OR_D;  /* planted: mean over half the dims */
    for (int i = 0; i < n_norm; i++) ss += (double)x[i] * (double)x[i];
    double r = (g_mutation == 27) ? 1.0 / (sqrt(ss / (double)n_norm) + (double)eps)  /* planted */
                                  : 1.0 / sqrt(ss / (double)n_norm + (double)eps);
    for (int i = 0; i < OR_D; i++) {
        double g = (g_mutation == 4) ? 1.0 : (double)gamma[i];   /* planted: gamma dropped */
        y[i] = (double)x[i] * r * g;
    }
    double pos = (double)OR_RATIO * (double)s;
    for (int j = 0; j < 32; j++) {
        int i0 = 64 + 2 * j, i1 = i0 + 1;
        if (g_mutation == 2) { i0 = 63 + 2 * j; i1 = i0 + 1; }   /* planted: pairs shifted */
        double phi = pos * (double)inv_freq[j];
        double c = cos(phi), sn = sin(phi);
        if (g_mutation == 1) sn = -sn;                          /* planted: rotation sign */
        double a = y[i0], b = y[i1];
        y[i0] = a * c - b * sn;
        y[i1] = a * sn + b * c;
    }
    if (hadamard) oracle_hadamard128(y);
    for (int i = 0; i < OR_D; i++) k32[i] = (float)y[i];
}

/* Writes every key whose (seq, s, page) is in range; returns the number of keys skipped.
 * k32_out (nullable) receives the canonical fp32 key of every input row (zeros when skipped). */
int64_t oracle_store_keys(const float* x, const float* gamma, float eps, const int32_t* key_idx,
                          const int32_t* key_seq, int64_t n_keys, const int32_t* page_table,
                          int32_t n_seq, int32_t max_pages, int dtype, uint8_t* pool,
                          int64_t n_pages_pool, float* k32_out, int hadamard) {
    float inv_freq[32];
    oracle_rope_inv_freq(inv_freq);
    int64_t skipped = 0;
    const int64_t pb = oracle_page_bytes(dtype);
#pragma omp parallel for schedule(static) reduction(+ : skipped)
    for (int64_t n = 0; n < n_keys; n++) {
        float k32[OR_D];
        int32_t b = key_seq ? key_seq[n] : 0;
        int32_t s = key_idx[n];
        if (k32_out) memset(k32_out + n * OR_D, 0, sizeof(float) * OR_D);
        if (b < 0 || b >= n_seq || s < 0 || (int64_t)s >= (int64_t)max_pages * OR_PAGE) {
            skipped++;
            continue;
        }
        int32_t page = page_table[(int64_t)b * max_pages + s / OR_PAGE];
        if (page < 0 || page >= n_pages_pool) {
            skipped++;
            continue;
        }
        canonical_key(x + n * OR_D, gamma, eps, s, inv_freq, hadamard, k32);
        if (k32_out) memcpy(k32_out + n * OR_D, k32, sizeof(float) * OR_D);
        uint8_t* pg = pool + (int64_t)page * pb;
        int slot = s % OR_PAGE;
        if (dtype == OR_BF16) {
            for (int i = 0; i < OR_D; i++) {
                uint16_t h = oracle_bf16_encode(k32[i]);
                pg[slot * 256 + 2 * i] = (uint8_t)(h & 0xFF);
                pg[slot * 256 + 2 * i + 1] = (uint8_t)(h >> 8);
            }
        } else if (dtype == OR_FP4) {
            /* fp4: scale = fp32(absmax / 6), codes e2m1 of fp32(k32 / scale); dims 2i and 2i+1
             * in the low and high nibble of byte i; codes at slot * 64, scales after the 4096 */
            double amax = 0.0;
            for (int i = 0; i < OR_D; i++) amax = fmax(amax, fabs((double)k32[i]));
            float scale = (float)(amax / 6.0);
            for (int i = 0; i < OR_D / 2; i++) {
                uint8_t c0 = 0, c1 = 0;
                if (scale > 0.0f) {
                    c0 = oracle_e2m1_encode((float)((double)k32[2 * i] / (double)scale));
                    c1 = oracle_e2m1_encode((float)((double)k32[2 * i + 1] / (double)scale));
                }
                pg[slot * (OR_D / 2) + i] = (g_mutation == 20) ? (uint8_t)(c1 | (c0 << 4))
                                                               : (uint8_t)(c0 | (c1 << 4));
            }
            memcpy(pg + OR_PAGE * (OR_D / 2) + slot * 4, &scale, 4);
        } else {
            double amax = 0.0;
            for (int i = 0; i < OR_D; i++) amax = fmax(amax, fabs((double)k32[i]));
            double fmax_code = (g_mutation == 10) ? 240.0 : 448.0;  /* planted: FNUZ max */
            /* fp64 quotient of fp32 operands rounded once to fp32 = correctly rounded fp32 div */
            float scale = (float)(amax / fmax_code);
            for (int i = 0; i < OR_D; i++) {
                uint8_t c = 0;
                if (scale > 0.0f)
                    c = oracle_e4m3_encode((g_mutation == 26) ? k32[i] * (1.0f / scale)  /* planted */
                                                              : (float)((double)k32[i] / (double)scale));
                pg[slot * OR_D + i] = c;
            }
            memcpy(pg + OR_PAGE * OR_D + slot * 4, &scale, 4);
        }
    }
    return skipped;
}

/* ---------------------------------------------------------------------------------------------
 * S2: logits.  Key source is either the paged pool (dequantised exactly to fp64) or a dense array
 * of canonical fp32 keys laid out [n_seq][ref_stride][128] (the "unquantised" ranking).
 * ------------------------------------------------------------------------------------------- */

/* Dequantise key s of sequence b from the pool.  Returns 0 if its page is out of range. */
static int fetch_key(const uint8_t* pool, int dtype, int64_t n_pages_pool, const int32_t* page_table,
                     int32_t max_pages, int32_t b, int32_t s, double* k) {
    int32_t page = page_table[(int64_t)b * max_pages + s / OR_PAGE];
    if (page < 0 || page >= n_pages_pool) return 0;
    const uint8_t* pg = pool + (int64_t)page * oracle_page_bytes(dtype);
    int slot = s % OR_PAGE;
    if (dtype == OR_BF16) {
        for (int i = 0; i < OR_D; i++) {
            uint16_t h = (uint16_t)(pg[slot * 256 + 2 * i] | (pg[slot * 256 + 2 * i + 1] << 8));
            k[i] = bf16_bits_value(h);
        }
    } else if (dtype == OR_FP4) {
        float scale;
        memcpy(&scale, pg + OR_PAGE * (OR_D / 2) + slot * 4, 4);
        for (int i = 0; i < OR_D / 2; i++) {
            uint8_t byte = pg[slot * (OR_D / 2) + i];
            k[2 * i] = oracle_e2m1_decode(byte & 15) * (double)scale;
            k[2 * i + 1] = oracle_e2m1_decode(byte >> 4) * (double)scale;
        }
    } else {
        float scale;
        memcpy(&scale, pg + OR_PAGE * OR_D + slot * 4, 4);
        for (int i = 0; i < OR_D; i++) {
            double v = oracle_e4m3_decode(pg[slot * OR_D + i]) * (double)scale;
            if (g_mutation == 13) v = oracle_e4m3_decode(pg[slot * OR_D + i]);  /* planted */
            k[i] = v;
        }
    }
    return 1;
}

/* Sequence of flattened query row i: the b with cu_q[b] <= i < cu_q[b+1]. */
static int32_t seq_of_row(const int32_t* cu_q, int32_t n_seq, int64_t i) {
    for (int32_t b = 0; b < n_seq; b++)
        if (i >= cu_q[b] && i < cu_q[b + 1]) return b;
    return -1;
}

/* Number of keys the query at token t of a sequence with max_pages pages sees. */
int64_t oracle_n_visible(int64_t t, int32_t max_pages) {
    if (t < 0) return 0;
    int64_t n = (t + 1) / OR_RATIO;
    if (g_mutation == 12) n = (t + 1) / OR_RATIO + 1;   /* planted: off by one */
    int64_t cap = (int64_t)max_pages * OR_PAGE;
    return n < cap ? n : cap;
}

/* fp8 x fp8 scoring: q of query i, head h is e4m3 codes times one fp32 scale, taken exactly in
 * fp64 (decoded once per query row). */
static void decode_q_fp8(const uint8_t* qc, const float* qs, double* qd) {
    for (int h = 0; h < OR_H; h++) {
        double sq = (g_mutation == 18) ? 1.0 : (double)qs[h];      /* planted: q scale dropped */
        for (int i = 0; i < OR_D; i++) qd[h * OR_D + i] = oracle_e4m3_decode(qc[h * OR_D + i]) * sq;
    }
}

static double score_one_f64(const double* qd, const float* w, const double* k) {
    double l = 0.0;
    for (int h = 0; h < OR_H; h++) {
        double d = 0.0;
        for (int i = 0; i < OR_D; i++) d += qd[h * OR_D + i] * k[i];
        l += (double)w[h] * fmax(0.0, d);
    }
    return l;
}

static double score_one(const uint16_t* q, const float* w, const double* k) {
    double l = 0.0;
    for (int h = 0; h < OR_H; h++) {
        double d = 0.0;
        for (int i = 0; i < OR_D; i++) {
            double qv = bf16_bits_value(q[h * OR_D + i]);
            if (g_mutation == 6) qv = bf16_bits_value(q[i * OR_H + h]);  /* planted: [128][64] read */
            d += qv * k[i];
        }
        double wv = (double)w[(g_mutation == 7) ? (h + 1) % OR_H : h];  /* planted: head shift */
        double r = (g_mutation == 5) ? d : fmax(0.0, d);                  /* planted: no ReLU */
        l += wv * r;
    }
    return l;
}

/* Logits for the query rows listed in rows[0..n_rows): out[r * row_len + s], s < row_len, is the
 * logit of visible key s, -inf otherwise (and for keys on out-of-pool pages).  n_vis_out[r]
 * (nullable) receives the row's visible count.  If keys_ref is non-NULL the keys are read from
 * it ([n_seq][ref_stride][128] fp32) instead of the pool. */
/* Rows of logits; q is bf16 (q) or fp8 codes with per-(query, head) scales (qc, qs). */
static void logits_rows(const uint16_t* q, const uint8_t* qc, const float* qs, const float* w,
                        const uint8_t* pool, int dtype, int64_t n_pages_pool,
                        const int32_t* page_table, int32_t n_seq, int32_t max_pages,
                        const int32_t* seq_lens, const int32_t* cu_q, const int64_t* rows,
                        int64_t n_rows, int64_t row_len, const float* keys_ref, int64_t ref_stride,
                        double* out, int64_t* n_vis_out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; r++) {
        int64_t i = rows[r];
        double* o = out + r * row_len;
        for (int64_t s = 0; s < row_len; s++) o[s] = -INFINITY;
        int32_t b = seq_of_row(cu_q, n_seq, i);
        int64_t n_vis = 0;
        if (b >= 0) {
            int64_t q_len = cu_q[b + 1] - cu_q[b];
            int64_t t = (int64_t)seq_lens[b] - q_len + (i - cu_q[b]);
            n_vis = oracle_n_visible(t, max_pages);
        }
        if (n_vis_out) n_vis_out[r] = n_vis;
        double k[OR_D];
        double qd[OR_H * OR_D];
        if (!q) decode_q_fp8(qc + i * OR_H * OR_D, qs + i * OR_H, qd);
        for (int64_t s = 0; s < n_vis && s < row_len; s++) {
            if (keys_ref) {
                const float* kr = keys_ref + ((int64_t)b * ref_stride + s) * OR_D;
                for (int d = 0; d < OR_D; d++) k[d] = (double)kr[d];
            } else if (!fetch_key(pool, dtype, n_pages_pool, page_table, max_pages, b, (int32_t)s, k)) {
                continue;
            }
            o[s] = q ? score_one(q + i * OR_H * OR_D, w + i * OR_H, k)
                     : score_one_f64(qd, w + i * OR_H, k);
        }
    }
}

void oracle_logits(const uint16_t* q, const float* w, const uint8_t* pool, int dtype,
                   int64_t n_pages_pool, const int32_t* page_table, int32_t n_seq,
                   int32_t max_pages, const int32_t* seq_lens, const int32_t* cu_q,
                   const int64_t* rows, int64_t n_rows, int64_t row_len, const float* keys_ref,
                   int64_t ref_stride, double* out, int64_t* n_vis_out) {
    logits_rows(q, NULL, NULL, w, pool, dtype, n_pages_pool, page_table, n_seq, max_pages,
                seq_lens, cu_q, rows, n_rows, row_len, keys_ref, ref_stride, out, n_vis_out);
}

void oracle_logits_fp8q(const uint8_t* q_codes, const float* q_scales, const float* w,
                        const uint8_t* pool, int dtype, int64_t n_pages_pool,
                        const int32_t* page_table, int32_t n_seq, int32_t max_pages,
                        const int32_t* seq_lens, const int32_t* cu_q, const int64_t* rows,
                        int64_t n_rows, int64_t row_len, double* out, int64_t* n_vis_out) {
    logits_rows(NULL, q_codes, q_scales, w, pool, dtype, n_pages_pool, page_table, n_seq,
                max_pages, seq_lens, cu_q, rows, n_rows, row_len, NULL, 0, out, n_vis_out);
}

/* q for fp8 x fp8 scoring: each 128-dim bf16 vector (one query head) gets one fp32 scale,
 * fp32(absmax / 448), and e4m3 codes of the correctly rounded fp32 quotients q_i / scale, the
 * rule of the fp8 key store; an all-zero vector gets scale 0 and codes 0. */
void oracle_quantize_q(const uint16_t* q, int64_t n_vec, uint8_t* codes, float* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_vec; n++) {
        double amax = 0.0;
        for (int i = 0; i < OR_D; i++) amax = fmax(amax, fabs(bf16_bits_value(q[n * OR_D + i])));
        float scale = (float)(amax / 448.0);
        scales[n] = scale;
        for (int i = 0; i < OR_D; i++) {
            double v = bf16_bits_value(q[n * OR_D + i]);
            uint8_t c = 0;
            if (scale > 0.0f)
                c = oracle_e4m3_encode(g_mutation == 17 ? (float)v : (float)(v / (double)scale));
            codes[n * OR_D + i] = c;   /* planted (17): the quotient skipped */
        }
    }
}

/* ---------------------------------------------------------------------------------------------
 * S3: top-k by full sort of (-value, index) over the first row_len[r] entries of each row.
 * ------------------------------------------------------------------------------------------- */

typedef struct { double v; int32_t s; } or_pair;

static int cmp_pair(const void* a, const void* b) {
    const or_pair* x = (const or_pair*)a;
    const or_pair* y = (const or_pair*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    if (g_mutation == 8) return (x->s > y->s) ? -1 : (x->s < y->s);   /* planted: ties to high s */
    return (x->s < y->s) ? -1 : (x->s > y->s);
}

void oracle_topk(const double* scores, int64_t n_rows, int64_t row_stride, const int64_t* row_len,
                 int32_t k, int32_t* out_idx, double* out_val) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; r++) {
        int64_t n = row_len ? row_len[r] : row_stride;
        if (n > row_stride) n = row_stride;
        if (n < 0) n = 0;
        or_pair* p = (or_pair*)malloc(sizeof(or_pair) * (size_t)(n > 0 ? n : 1));
        for (int64_t s = 0; s < n; s++) {
            double v = scores[r * row_stride + s];
            p[s].v = (v == 0.0) ? 0.0 : v;     /* -0 and +0 compare equal */
            p[s].s = (int32_t)s;
        }
        qsort(p, (size_t)n, sizeof(or_pair), cmp_pair);
        for (int32_t j = 0; j < k; j++) {
            if (j < n) {
                out_idx[r * k + j] = p[j].s;
                if (out_val) out_val[r * k + j] = scores[r * row_stride + p[j].s];
            } else {
                out_idx[r * k + j] = -1;
                if (out_val) out_val[r * k + j] = -INFINITY;
            }
        }
        free(p);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Test-harness helper: pre-norm activations whose stored key points along a given direction.
 * x = R_{4s}^{-1}(kstar) / gamma, so that RMSNorm then RoPE return r * kstar for a positive r.
 * ------------------------------------------------------------------------------------------- */
void oracle_plant_keys(const double* kstar, const int32_t* key_idx, int64_t n, const float* gamma,
                       float* x_out) {
    float inv_freq[32];
    oracle_rope_inv_freq(inv_freq);
    for (int64_t r = 0; r < n; r++) {
        double y[OR_D];
        for (int i = 0; i < OR_D; i++) y[i] = kstar[r * OR_D + i];
        double pos = (double)OR_RATIO * (double)key_idx[r];
        for (int j = 0; j < 32; j++) {
            int i0 = 64 + 2 * j, i1 = i0 + 1;
            double phi = pos * (double)inv_freq[j];
            double c = cos(phi), sn = sin(phi);
            double a = y[i0], b = y[i1];
            y[i0] = a * c + b * sn;        /* rotation by -phi */
            y[i1] = -a * sn + b * c;
        }
        for (int i = 0; i < OR_D; i++) x_out[r * OR_D + i] = (float)(y[i] / (double)gamma[i]);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Sparse attention over the selected keys, for the query rows listed in rows[0..n_rows).
 * q: [n_q][n_heads][512] bf16 bits; kv: [n_slots][512] bf16 bits; kv_slot: [n_seq][max_keys];
 * idx: [n_q][k] logical key indices (-1 = none).  out: [n_rows][n_heads][512], lse:
 * [n_rows][n_heads], both fp64.  Every product of two bf16 values is exact in fp64; the softmax
 * subtracts the largest logit before exponentiating.
 * ------------------------------------------------------------------------------------------- */
void oracle_sparse_attn(const uint16_t* q, const uint16_t* kv, int64_t n_slots,
                        const int32_t* kv_slot, int32_t n_seq, int32_t max_keys,
                        const int32_t* cu_q, const int32_t* idx, int32_t n_heads, int32_t k,
                        double scale, const int64_t* rows, int64_t n_rows, double* out,
                        double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; r++) {
        int64_t i = rows[r];
        int32_t b = seq_of_row(cu_q, n_seq, i);
        /* the rows of kv this query attends to, in list order */
        int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)(k > 0 ? k : 1));
        int n = 0;
        for (int32_t j = 0; j < k; j++) {
            int32_t s = idx[i * k + j];
            if (g_mutation == 22 && s < 0) s = 0;                 /* planted: -1 read as key 0 */
            if (b < 0 || s < 0 || s >= max_keys) continue;
            int64_t sl = kv_slot[(int64_t)b * max_keys + s];
            if (g_mutation == 23) sl = kv_slot[(int64_t)b * max_keys + (s + 1) % max_keys];
            if (sl < 0 || sl >= n_slots) continue;
            slot[n++] = sl;
        }
        double* logit = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        for (int32_t h = 0; h < n_heads; h++) {
            const uint16_t* qh = q + (i * n_heads + h) * OR_DV;
            double* o = out + (r * n_heads + h) * OR_DV;
            for (int d = 0; d < OR_DV; d++) o[d] = 0.0;
            if (n == 0) {
                lse[r * n_heads + h] = -INFINITY;
                continue;
            }
            double mx = -INFINITY;
            for (int j = 0; j < n; j++) {
                const uint16_t* v = kv + slot[j] * OR_DV;
                double dot = 0.0;
                for (int d = 0; d < OR_DV; d++) {
                    double qv = bf16_bits_value(qh[d]);
                    if (g_mutation == 25) qv = bf16_bits_value(q[(i * OR_DV + d) * n_heads + h]);
                    dot += qv * bf16_bits_value(v[d]);
                }
                logit[j] = (g_mutation == 21) ? dot : scale * dot;  /* planted: scale dropped */
                if (logit[j] > mx) mx = logit[j];
            }
            double sum = 0.0;
            for (int j = 0; j < n; j++) sum += exp(logit[j] - mx);
            for (int j = 0; j < n; j++) {
                double p = exp(logit[j] - mx) / sum;
                const uint16_t* v = kv + slot[j] * OR_DV;
                for (int d = 0; d < OR_DV; d++) o[d] += p * bf16_bits_value(v[d]);
            }
            lse[r * n_heads + h] = (g_mutation == 24) ? log(sum) : mx + log(sum);
        }
        free(logit);
        free(slot);
    }
}
