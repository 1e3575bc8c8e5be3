/*
 * CPU oracle for the routed int4 Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product path never does.  It
 * shares no code, header or table with the GPU library and reads only the
 * public weight layout (documented in routed_expert_int4_amd/synth.py).
 *
 * What is computed (all arithmetic in double precision after an exact
 * dequantisation; the pages fix no precision, so fp64 is the reference):
 *
 *  - Router.  The colibri summary ("Principales fonctionnalites": a sigmoid
 *    router in the style of DeepSeek-V3 with noaux_tc, routed_scaling_factor
 *    and a shared expert) and the LightLX README ("How it works": mlx-lm's
 *    noaux_tc sigmoid router) name the router but do not spell out its
 *    arithmetic.  We take the DeepSeek-V3 gating rule as the reading:
 *      s_e  = sigmoid(x . W_r[e])                 affinity
 *      sb_e = s_e + bias_e                        used only to choose experts
 *      group score = sum of the two largest sb in the group (contiguous groups)
 *      keep the topk_group best groups; experts outside them cannot be chosen
 *      choose the top_k eligible experts by sb (ties: lower index)
 *      weight_j = routed_scaling_factor * s_j / sum_selected s      (no epsilon)
 *  - Experts.  SwiGLU with no biases, as mlx-lm's SwitchGLU (LightLX "Run any
 *    model"): h = silu(W_g x) * (W_u x), d = W_d h, silu(z) = z * sigmoid(z).
 *  - Combine.  y = sum_j weight_j * d_{e_j} + sum over shared experts d_s
 *    (the shared expert is always applied with weight 1; colibri summary,
 *    "Principales fonctionnalites"; LightLX "How it works" keeps all shared
 *    experts resident).
 *  - Int4 format.  Symmetric int4 codes with one fp16 scale per 32 inputs
 *    (the colibri summary lists packed int4 kernels with dequant-on-use; the
 *    group size and scale type are the layer's stated format).  A code byte
 *    holds the even column in its low nibble, two's complement.  The weight
 *    value is fp32(scale) * q, which is exact in fp32.
 *
 *  - MXFP4 format (codec 1).  The LargerLM README ("What It Proves") runs a
 *    GLM-5.2 MXFP4 layout; the pages name it only.  Reading: the OCP
 *    Microscaling (MX) v1.0 MXFP4 element and scale types over blocks of 32
 *    consecutive inputs, packed as the int4 codes are (even column in the
 *    low nibble).  An E2M1 element has a sign bit, a 2-bit exponent (bias 1)
 *    and a 1-bit mantissa: value (-1)^s * 2^(e-1) * (1 + m/2) for e > 0 and
 *    (-1)^s * m/2 for e = 0 (no infinities or NaNs).  An E8M0 scale byte b
 *    is 2^(b-127), b = 255 is NaN.  Weight value = scale * element, exact in
 *    double.
 *
 *  - Int8 format (codec 2).  The colibri summary ("Principales
 *    fonctionnalites": the quantisation kernels cover int8, packed int4 and
 *    packed int2 with dequant-on-use; the MTP head must be int8) names the
 *    width only.  Reading: one two's complement byte per weight, the same
 *    fp16 scale per 32 inputs as int4; weight = fp32(scale) * q (exact: an
 *    11-bit significand times an 8-bit integer).
 *
 *  - Int2 format (codec 3), the packed int2 of the same list.  Reading: four
 *    two's complement 2-bit codes per byte (values -2..1), column 4j + t in
 *    bits [2t, 2t + 2) of byte j, the same fp16 scale per 32 inputs;
 *    weight = fp32(scale) * q.
 *
 *  - Adaptive expert top-p (colibri summary, options list: --topp, an
 *    adaptive expert top-p that cuts the expert reads).  Reading: with
 *    top_p < 1, the selected experts are ranked by their share s_j / sum_sel s
 *    (descending, ties: lower index) and only the smallest leading set whose
 *    shares reach top_p is kept (an expert is kept when the shares ranked
 *    before it sum to less than top_p); the kept weights are renormalised,
 *    weight_j = routed_scaling_factor * s_j / sum_kept s, and a dropped slot
 *    holds id -1 and weight 0.  top_p = 1 is plain top-k.
 *
 * Diagnostics per token: the boundary gap of the selection (the smallest
 * margin by which a different choice of groups or experts would have been
 * made), used to excuse index mismatches caused by rounding, and with top-p
 * the margin of the keep decisions, min_j |shares ranked before j - top_p|.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoding */

/* IEEE binary16 bits -> value (exact). */
static double half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 31;
    int man = h & 1023;
    double v;
    if (ex == 0) {
        v = ldexp((double)man, -24);
    } else if (ex == 31) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + man), ex - 25);
    }
    return sign ? -v : v;
}

/* bfloat16 bits -> value (exact). */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* int4 code of column c in a packed row (two's complement nibble). */
static int code_at(const uint8_t* row, int c) {
    int nib = (row[c >> 1] >> ((c & 1) * 4)) & 15;
    return nib >= 8 ? nib - 16 : nib;
}

/* y[r] = sum_c W[r][c] x[c] for an int4 matrix [rows][cols] with group-32
 * fp16 scales, where W[r][c] = fp32(scale[r][c/32]) * q[r][c] is formed in
 * float (exact: an 11-bit significand times a 4-bit integer) and widened to
 * double before the product. */
static void int4_matvec(const uint8_t* q, const uint16_t* s, int rows, int cols, const double* x, double* y) {
    for (int r = 0; r < rows; ++r) {
        const uint8_t* qr = q + (size_t)r * (cols / 2);
        const uint16_t* sr = s + (size_t)r * (cols / 32);
        double acc = 0.0;
        for (int g = 0; g < cols / 32; ++g) {
            float scale = (float)half_to_double(sr[g]);
            for (int c = 32 * g; c < 32 * g + 32; ++c) {
                float wv = scale * (float)code_at(qr, c);
                acc += (double)wv * x[c];
            }
        }
        y[r] = acc;
    }
}

/* MXFP4: E2M1 element of column c in a packed row, and an E8M0 scale. */
static double e2m1_at(const uint8_t* row, int c) {
    int nib = (row[c >> 1] >> ((c & 1) * 4)) & 15;
    int sgn = nib >> 3, ex = (nib >> 1) & 3, man = nib & 1;
    double v = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
    return sgn ? -v : v;
}
static double e8m0_value(uint8_t b) { return b == 255 ? NAN : ldexp(1.0, (int)b - 127); }

/* y[r] = sum_c W[r][c] x[c] for an MXFP4 matrix [rows][cols]: W[r][c] =
 * E8M0(scale[r][c/32]) * E2M1(code[r][c]), formed exactly in double. */
static void mxfp4_matvec(const uint8_t* q, const uint8_t* s, int rows, int cols, const double* x, double* y) {
    for (int r = 0; r < rows; ++r) {
        const uint8_t* qr = q + (size_t)r * (cols / 2);
        const uint8_t* sr = s + (size_t)r * (cols / 32);
        double acc = 0.0;
        for (int g = 0; g < cols / 32; ++g) {
            double scale = e8m0_value(sr[g]);
            for (int c = 32 * g; c < 32 * g + 32; ++c) acc += (scale * e2m1_at(qr, c)) * x[c];
        }
        y[r] = acc;
    }
}

/* Int8: y[r] = sum_c W[r][c] x[c], codes [rows][cols] two's complement
 * bytes, W[r][c] = fp32(scale[r][c/32]) * q[r][c] formed in float (exact). */
static void int8_matvec(const uint8_t* q, const uint16_t* s, int rows, int cols, const double* x, double* y) {
    for (int r = 0; r < rows; ++r) {
        const int8_t* qr = (const int8_t*)(q + (size_t)r * cols);
        const uint16_t* sr = s + (size_t)r * (cols / 32);
        double acc = 0.0;
        for (int g = 0; g < cols / 32; ++g) {
            float scale = (float)half_to_double(sr[g]);
            for (int c = 32 * g; c < 32 * g + 32; ++c) acc += (double)(scale * (float)qr[c]) * x[c];
        }
        y[r] = acc;
    }
}

/* Int2: code of column c in a packed row (two's complement 2-bit field). */
static int code2_at(const uint8_t* row, int c) {
    int v = (row[c >> 2] >> ((c & 3) * 2)) & 3;
    return v >= 2 ? v - 4 : v;
}
static void int2_matvec(const uint8_t* q, const uint16_t* s, int rows, int cols, const double* x, double* y) {
    for (int r = 0; r < rows; ++r) {
        const uint8_t* qr = q + (size_t)r * (cols / 4);
        const uint16_t* sr = s + (size_t)r * (cols / 32);
        double acc = 0.0;
        for (int g = 0; g < cols / 32; ++g) {
            float scale = (float)half_to_double(sr[g]);
            for (int c = 32 * g; c < 32 * g + 32; ++c) acc += (double)(scale * (float)code2_at(qr, c)) * x[c];
        }
        y[r] = acc;
    }
}

/* Codec 0: int4 codes with fp16 scales; codec 1: MXFP4 (E2M1 codes, E8M0
 * scales); codec 2: int8 codes, codec 3: int2 codes, both with fp16 scales.
 * Scale arrays are uint16 (codecs 0, 2, 3) or uint8 (codec 1); code arrays
 * hold cols/2 bytes per row (codecs 0 and 1), cols (codec 2) or cols/4
 * (codec 3). */
static void codec_matvec(int codec, const uint8_t* q, const void* s, int rows, int cols, const double* x,
                         double* y) {
    if (codec == 1)
        mxfp4_matvec(q, (const uint8_t*)s, rows, cols, x, y);
    else if (codec == 2)
        int8_matvec(q, (const uint16_t*)s, rows, cols, x, y);
    else if (codec == 3)
        int2_matvec(q, (const uint16_t*)s, rows, cols, x, y);
    else
        int4_matvec(q, (const uint16_t*)s, rows, cols, x, y);
}

/* Public matvec of one quantised matrix (for pins of the decoding). */
void oracle_matvec(int codec, const uint8_t* q, const void* s, int rows, int cols, const double* x, double* y) {
    codec_matvec(codec, q, s, rows, cols, x, y);
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ---------------------------------------------------------------- public API */

/* One expert on one token: d = W_d (silu(W_g x) * (W_u x)).
 * gate/up: [inter][hidden/2] codes, [inter][hidden/32] scales;
 * down: [hidden][inter/2] codes, [hidden][inter/32] scales.
 * h (optional, [inter]) receives the intermediate activation. */
void oracle_expert_ffn(int codec, int hidden, int inter,
                       const uint8_t* gate_q, const void* gate_s,
                       const uint8_t* up_q, const void* up_s,
                       const uint8_t* down_q, const void* down_s,
                       const double* x, double* d, double* h_out) {
    double* g = (double*)malloc(sizeof(double) * (size_t)inter);
    double* u = (double*)malloc(sizeof(double) * (size_t)inter);
    codec_matvec(codec, gate_q, gate_s, inter, hidden, x, g);
    codec_matvec(codec, up_q, up_s, inter, hidden, x, u);
    for (int i = 0; i < inter; ++i) g[i] = g[i] * sigmoid(g[i]) * u[i];
    codec_matvec(codec, down_q, down_s, hidden, inter, g, d);
    if (h_out) memcpy(h_out, g, sizeof(double) * (size_t)inter);
    free(g);
    free(u);
}

/* Router scores of one token: logit, s = sigmoid(logit), sb = s + bias. */
void oracle_router_scores(int hidden, int n_experts, const float* router_w, const float* bias,
                          const double* x, double* logit, double* s, double* sb) {
    for (int e = 0; e < n_experts; ++e) {
        double acc = 0.0;
        const float* w = router_w + (size_t)e * hidden;
        for (int c = 0; c < hidden; ++c) acc += (double)w[c] * x[c];
        logit[e] = acc;
        s[e] = sigmoid(acc);
        sb[e] = s[e] + (double)bias[e];
    }
}

/* "a ranks before b": larger value first, ties to the lower index. */
static int ranks_before(double va, int a, double vb, int b) {
    return va > vb || (va == vb && a < b);
}

/* Group-limited top-k selection of one token from its scores.
 * Writes ids[top_k] (sb descending, ties to the lower index), w[top_k], and
 * the boundary gap: min over the group boundary and the expert boundary of
 * (last kept score - first rejected score); +inf where there is no rejected
 * candidate.  Returns 0, or -1 when the arguments are inconsistent. */
int oracle_select(int n_experts, int n_groups, int topk_group, int top_k, double rsf, double top_p,
                  const double* s, const double* sb, int32_t* ids, double* w, double* gap, double* pgap) {
    if (n_experts <= 0 || n_groups <= 0 || n_experts % n_groups) return -1;
    int gsize = n_experts / n_groups;
    if (gsize < 2 || topk_group < 1 || topk_group > n_groups) return -1;
    if (top_k < 1 || top_k > topk_group * gsize || top_k > 64 || !(top_p > 0.0 && top_p <= 1.0)) return -1;

    double* gscore = (double*)malloc(sizeof(double) * (size_t)n_groups);
    int* gorder = (int*)malloc(sizeof(int) * (size_t)n_groups);
    int* eorder = (int*)malloc(sizeof(int) * (size_t)n_experts);
    char* eligible = (char*)calloc((size_t)n_experts, 1);

    /* Group score: the two largest biased scores in the group. */
    for (int g = 0; g < n_groups; ++g) {
        double best = -INFINITY, second = -INFINITY;
        for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
            if (sb[e] > best) { second = best; best = sb[e]; }
            else if (sb[e] > second) second = sb[e];
        }
        gscore[g] = best + second;
    }
    /* Order groups (insertion sort on the ranking relation). */
    for (int g = 0; g < n_groups; ++g) {
        int p = g;
        while (p > 0 && ranks_before(gscore[g], g, gscore[gorder[p - 1]], gorder[p - 1])) {
            gorder[p] = gorder[p - 1];
            --p;
        }
        gorder[p] = g;
    }
    for (int r = 0; r < topk_group; ++r) {
        int g = gorder[r];
        for (int e = g * gsize; e < (g + 1) * gsize; ++e) eligible[e] = 1;
    }
    double gap_g = INFINITY;
    if (topk_group < n_groups) gap_g = gscore[gorder[topk_group - 1]] - gscore[gorder[topk_group]];

    /* Order eligible experts by sb. */
    int n_el = 0;
    for (int e = 0; e < n_experts; ++e) {
        if (!eligible[e]) continue;
        int p = n_el++;
        while (p > 0 && ranks_before(sb[e], e, sb[eorder[p - 1]], eorder[p - 1])) {
            eorder[p] = eorder[p - 1];
            --p;
        }
        eorder[p] = e;
    }
    double denom = 0.0;
    for (int j = 0; j < top_k; ++j) {
        ids[j] = eorder[j];
        denom += s[eorder[j]];
    }
    for (int j = 0; j < top_k; ++j) w[j] = rsf * s[ids[j]] / denom;
    double gap_e = INFINITY;
    if (top_k < n_el) gap_e = sb[eorder[top_k - 1]] - sb[eorder[top_k]];
    *gap = gap_e < gap_g ? gap_e : gap_g;

    /* Adaptive top-p over the selected experts. */
    *pgap = INFINITY;
    if (top_p < 1.0) {
        int keep[64];
        double kept = 0.0;
        for (int j = 0; j < top_k; ++j) {
            double before = 0.0;
            for (int k = 0; k < top_k; ++k)
                if (ranks_before(s[ids[k]], ids[k], s[ids[j]], ids[j])) before += s[ids[k]] / denom;
            keep[j] = before < top_p;
            if (fabs(before - top_p) < *pgap) *pgap = fabs(before - top_p);
            if (keep[j]) kept += s[ids[j]];
        }
        for (int j = 0; j < top_k; ++j) {
            w[j] = keep[j] ? rsf * s[ids[j]] / kept : 0.0;
            if (!keep[j]) ids[j] = -1;
        }
    }

    free(gscore);
    free(gorder);
    free(eorder);
    free(eligible);
    return 0;
}

/* Full layer on T tokens.
 *
 * Expert arrays are stacked: expert e (0 <= e < n_experts) then the shared
 * experts at n_experts .. n_experts+n_shared-1; gate_q has shape
 * [n_experts+n_shared][inter][hidden/2] and so on.
 * forced_ids (optional, [T][top_k]): use these experts instead of the
 * router's choice; the weights are still rsf * s / sum s over them.
 * Outputs: y [T][hidden], ids [T][top_k], w [T][top_k], gap [T],
 * logits (optional) [T][n_experts].  Returns 0 or -1 on bad arguments. */
int oracle_layer_forward(int codec, int hidden, int inter, int n_experts, int n_groups, int topk_group, int top_k,
                         int n_shared, double rsf, double top_p,
                         const float* router_w, const float* bias,
                         const uint8_t* gate_q, const void* gate_s,
                         const uint8_t* up_q, const void* up_s,
                         const uint8_t* down_q, const void* down_s,
                         const uint16_t* x_bf16, int T, const int32_t* forced_ids,
                         double* y, int32_t* ids, double* w, double* gap, double* pgap, double* logits,
                         int n_threads) {
    if (hidden % 32 || inter % 32 || T < 0 || n_shared < 0 || codec < 0 || codec > 3) return -1;
    const size_t ssz = codec == 1 ? 1 : 2;                       /* bytes per scale */
    const size_t cpb = codec == 2 ? 1 : codec == 3 ? 4 : 2;      /* codes per byte */
    const uint8_t *gs_b = (const uint8_t*)gate_s, *us_b = (const uint8_t*)up_s, *ds_b = (const uint8_t*)down_s;
    const size_t gq_n = (size_t)inter * (hidden / cpb), gs_n = (size_t)inter * (hidden / 32);
    const size_t dq_n = (size_t)hidden * (inter / cpb), ds_n = (size_t)hidden * (inter / 32);
    int status = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int t = 0; t < T; ++t) {
        double* x = (double*)malloc(sizeof(double) * (size_t)hidden);
        double* lg = (double*)malloc(sizeof(double) * (size_t)n_experts);
        double* s = (double*)malloc(sizeof(double) * (size_t)n_experts);
        double* sb = (double*)malloc(sizeof(double) * (size_t)n_experts);
        double* d = (double*)malloc(sizeof(double) * (size_t)hidden);
        double* yt = y + (size_t)t * hidden;
        int32_t* it = ids + (size_t)t * top_k;
        double* wt = w + (size_t)t * top_k;

        for (int c = 0; c < hidden; ++c) x[c] = bf16_to_double(x_bf16[(size_t)t * hidden + c]);
        oracle_router_scores(hidden, n_experts, router_w, bias, x, lg, s, sb);
        if (logits) memcpy(logits + (size_t)t * n_experts, lg, sizeof(double) * (size_t)n_experts);
        if (oracle_select(n_experts, n_groups, topk_group, top_k, rsf, top_p, s, sb, it, wt, gap + t,
                          pgap + t) != 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = -1;
        } else {
            if (forced_ids) {
                /* forced experts (-1: empty slot), weights over the forced set */
                double denom = 0.0;
                for (int j = 0; j < top_k; ++j) {
                    it[j] = forced_ids[(size_t)t * top_k + j];
                    if (it[j] >= 0) denom += s[it[j]];
                }
                for (int j = 0; j < top_k; ++j) wt[j] = it[j] >= 0 ? rsf * s[it[j]] / denom : 0.0;
            }
            for (int c = 0; c < hidden; ++c) yt[c] = 0.0;
            for (int j = 0; j < top_k + n_shared; ++j) {
                if (j < top_k && it[j] < 0) continue; /* slot dropped by top-p */
                int e = j < top_k ? it[j] : n_experts + (j - top_k);
                double scale = j < top_k ? wt[j] : 1.0;
                oracle_expert_ffn(codec, hidden, inter, gate_q + e * gq_n, gs_b + e * gs_n * ssz, up_q + e * gq_n,
                                  us_b + e * gs_n * ssz, down_q + e * dq_n, ds_b + e * ds_n * ssz, x, d, NULL);
                for (int c = 0; c < hidden; ++c) yt[c] += scale * d[c];
            }
        }
        free(x);
        free(lg);
        free(s);
        free(sb);
        free(d);
    }
    return status;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Router and selection only, for T tokens (no expert math): ids [T][top_k],
 * w [T][top_k], gap [T].  Same steps as oracle_layer_forward. */
int oracle_route(int hidden, int n_experts, int n_groups, int topk_group, int top_k, double rsf, double top_p,
                 const float* router_w, const float* bias, const uint16_t* x_bf16, int T,
                 int32_t* ids, double* w, double* gap, double* pgap, int n_threads) {
    int status = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 4)
#endif
    for (int t = 0; t < T; ++t) {
        double* x = (double*)malloc(sizeof(double) * (size_t)hidden);
        double* lg = (double*)malloc(sizeof(double) * (size_t)n_experts);
        double* s = (double*)malloc(sizeof(double) * (size_t)n_experts);
        double* sb = (double*)malloc(sizeof(double) * (size_t)n_experts);
        for (int c = 0; c < hidden; ++c) x[c] = bf16_to_double(x_bf16[(size_t)t * hidden + c]);
        oracle_router_scores(hidden, n_experts, router_w, bias, x, lg, s, sb);
        if (oracle_select(n_experts, n_groups, topk_group, top_k, rsf, top_p, s, sb, ids + (size_t)t * top_k,
                          w + (size_t)t * top_k, gap + t, pgap + t) != 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = -1;
        }
        free(x);
        free(lg);
        free(s);
        free(sb);
    }
    return status;
}
