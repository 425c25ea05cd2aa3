/*
 * oracle.c -- plain CPU oracle for the W8A8 INT8 mixture-of-experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package
 * entry file and the cpu_baseline leg of bench.py may load or call this code.  The
 * GPU library never links, includes or calls it, and this file includes nothing
 * from the GPU library: the two share no headers, helpers, tables or constants.
 *
 * Every step is written as the plainest loop that states what the scheme
 * computes.  There is no blocking, fusion or reordering.  The only
 * parallelism is an OpenMP "parallel for" over independent rows (tokens or
 * routed pairs): every row is computed by one thread in the same order as in
 * a serial run, so the results do not depend on the thread count.
 *
 * Sources (web pages; each cited by its title and section):
 *   [30B-W8A8]   "Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer:
 *                section 1 (model profile), 2 (quantisation config), 3.1-3.3
 *                (why mlp.gate stays bf16), 7 (FAQ).
 *   [3.6-CFG]    "Qwen3.6-35B-A3B-w8a8 config.json and recipe.yaml" walkthrough:
 *                the quantization_config group_0 block, its "weights" and
 *                "input_activations" parameter lists.
 *   [235B-FILES] "Qwen3-235B-A22B-quantized.w8a8" file-structure guide: model
 *                overview table, shard contents, W8A8 section.
 *   [1.7B-W4A8]  "Qwen3-1.7B-W4A8 on Ascend": the W4A8 variant (4-bit weights
 *                in groups of 128 with scale/offset, two's-complement packing).
 *   [NEXT-AMCT]  "Qwen3-Next-80B-A3B-Instruct in AMCT" adaptation case:
 *                section 2.2 (packed gate_up_proj / down_proj), section 6
 *                (packed MoE GMM performance note).
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *   R1  codes are clamped to [-127, 127]; -128 is never produced (symmetric).
 *   R2  rounding of x/s to an integer is round-half-to-even (rintf in the
 *       default rounding mode).
 *   R3  scale s = amax / 127 is one IEEE fp32 divide, and the code is
 *       rint(x / s) with a second IEEE fp32 divide (not x * (127 / amax)).
 *   R4  a row whose amax is 0 gets s = 0 and all codes 0.
 *   R5  scales are fp32.
 *   R6  router logits: fp32.  The hidden index is cut into chunks of 512
 *       (the last may be shorter); each chunk is one fused multiply-add chain
 *       over its indices in ascending order, starting from +0.0f, and the
 *       chunk sums are added in ascending chunk order (fp32 adds, the first
 *       chunk's sum as the start).  For H <= 512 this is the single chain.
 *   R7  top-k selects on the fp32 logits, larger first, equal logits ordered
 *       by the lower expert index.
 *   R8  the k selected softmax probabilities are renormalised to sum to 1.
 *   R9  the expert MLP is SwiGLU: h = silu(gate) * up, silu(g) = g / (1 + e^-g).
 *   R10 h is rounded once to bf16 (round-half-to-even) before it is quantised
 *       for down_proj; down_proj is int8 like gate/up ([235B-FILES]).
 *   R11 the permutation inside one expert's group is by ascending pair index
 *       p = t * k + j.
 *   R17 W4A8 (the next row after the W8A8 layer): gate_up_proj expert weights
 *       in 4 bits, groups of 128 consecutive inputs of one output channel
 *       (the last group of a row may be shorter), each with an fp32 scale and
 *       an integer offset ([1.7B-W4A8] "4bit 权重" items 1-2: group_size 128
 *       with a scale/offset per group, two's-complement 4-bit codes).  The
 *       plainest asymmetric min-max reading: the range [min(w, 0), max(w, 0)]
 *       (zero always representable) is split into 15 steps, s = (max - min)/15
 *       (one fp32 divide), z = rint(-min / s) in [0, 15], u = clamp(rint(w / s)
 *       + z, 0, 15); stored code q = u - 8 in [-8, 7], offset o = z - 8 in
 *       [-8, 7]; w ~ (q - o) * s.  A group of zeros has s = 0, codes and
 *       offset 0.  down_proj stays W8A8 (the page keeps down_proj in higher
 *       precision); activations are the same per-token int8 codes.
 *   R18 shared expert (the next row after W4A8): the layers of the pages'
 *       Qwen3.6 and Qwen3-Next models add an always-on shared expert whose
 *       Linears are W8A8 like a routed expert's ([NEXT-AMCT] 2.2: the shared
 *       expert is a dense path quantised directly) while shared_expert_gate
 *       stays bf16 ([3.6-CFG] ignore list).  The plainest reading of the
 *       pair: the shared expert is a SwiGLU FFN of its own intermediate size
 *       Is over every token's int8 codes from step 2, with the steps of a
 *       routed expert (h rounded to bf16, quantised per row, int8 down_proj),
 *       and the gate is one bf16 Linear [H] -> 1 whose sigmoid weights the
 *       shared output: out = sum_j w_j y_j + sigmoid(x . w_sg) * z.
 *   R19 the gate logit x . w_sg is not a decision (no integer depends on
 *       it), so here it is the exact fp64 sum of the products (bf16 x bf16 and
 *       fp32 x bf16 products are exact in fp64); the shared term is added after
 *       the k routed slots.
 *   Floating-point results that are compared within a tolerance (dequantised
 *   GEMM outputs, SwiGLU, softmax weights, the combine) are computed here in
 *   fp64.  Floating-point work that decides an integer (int8 codes, top-k
 *   ids) is done in fp32, the precision the GPU takes the same decision in.
 *
 * Preconditions: inputs are finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the OpenMP loops below use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the OpenMP loops below (n >= 1).  The results do not depend on
 * it: every row is computed by one thread in the serial order. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ bf16 --- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static float or_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a double to the nearest bf16 (8 significant bits, binary32 exponent
 * range), ties to even, in one rounding.  Results beyond the largest finite
 * bf16 become infinity. */
static uint16_t or_f64_to_bf16(double v)
{
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    uint16_t bits;
    if (a == 0.0) {
        bits = 0;
    } else {
        int e;
        (void)frexp(a, &e);              /* a = m * 2^e with 0.5 <= m < 1 */
        int quantum = e - 8;             /* weight of the last of 8 significant bits */
        if (quantum < -133) quantum = -133; /* bf16 subnormal spacing is 2^-133 */
        double r = ldexp(nearbyint(ldexp(a, -quantum)), quantum);
        if (r >= ldexp(1.0, 128)) {
            bits = 0x7f80;               /* overflow to +inf */
        } else {
            float f = (float)r;          /* exact: r has at most 8 significant bits */
            uint32_t u;
            memcpy(&u, &f, sizeof u);
            bits = (uint16_t)(u >> 16);
        }
    }
    return (uint16_t)(bits | (neg ? 0x8000 : 0));
}

uint16_t oracle_f64_to_bf16(double v) { return or_f64_to_bf16(v); }
double oracle_bf16_to_f64(uint16_t b) { return (double)or_bf16_to_f32(b); }

/* Load element i of a row given as bf16 (dtype 0) or fp32 (dtype 1). */
static float or_load(const void *x, int dtype, int64_t i)
{
    if (dtype == 0) return or_bf16_to_f32(((const uint16_t *)x)[i]);
    return ((const float *)x)[i];
}

/* ------------------------------------------------------ row quantisation --- */

/*
 * Symmetric int8 quantisation of one row (R1-R5).
 * Static per-output-channel weight quantisation ([3.6-CFG] group_0 "weights":
 * 8 bits, strategy channel, symmetric, minmax observer, not dynamic; [30B-W8A8]
 * section 2) and dynamic per-token activation quantisation ([3.6-CFG] group_0
 * "input_activations": 8 bits, strategy token, symmetric, dynamic) are the same
 * computation on a row: a row of W is one output channel, a row of x is one token.
 */
static void or_quant_row(const void *x, int dtype, int64_t cols, int8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
        float a = fabsf(or_load(x, dtype, c));
        if (a > amax) amax = a;
    }
    float s = amax / 127.0f;
    *scale = s;
    for (int64_t c = 0; c < cols; ++c) {
        if (s == 0.0f) {
            q[c] = 0;
            continue;
        }
        float v = rintf(or_load(x, dtype, c) / s);
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        q[c] = (int8_t)v;
    }
}

/* Quantise `rows` rows of `cols` elements, row stride ld (elements). */
void oracle_quant_rows(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       int8_t *q, float *scales)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const void *row = (dtype == 0) ? (const void *)((const uint16_t *)x + r * ld)
                                       : (const void *)((const float *)x + r * ld);
        or_quant_row(row, dtype, cols, q + r * cols, &scales[r]);
    }
}

/* ---------------------------------------------------------------- router --- */

/*
 * The unquantised router ([30B-W8A8] sections 3.1-3.3; [235B-FILES] shard
 * contents: mlp.gate stays bf16): hidden state -> one score per expert ->
 * softmax -> the top-k experts, whose weights are renormalised (R6-R8).
 *   x      [T][H]  bf16 (dtype 0) or fp32 (dtype 1)
 *   wg     [E][H]  bf16 bits
 *   ids    [T][k]  out, expert ids by descending logit
 *   w      [T][k]  out, routing weights
 *   logits [T][E]  out, may be NULL
 */
/* R6: hidden indices per chain of the router score */
#define OR_ROUTE_CHUNK 512

/* The router with chains of `chunk` hidden indices (R6 is chunk = 512; a
 * chunk <= 0 or >= H gives the single fma chain over all of h, kept to study
 * how far the choice of order moves the selected experts). */
void oracle_route_topk_chunked(const void *x, int dtype, const uint16_t *wg, int64_t T, int64_t H,
                               int E, int k, int renormalize, int32_t *ids, float *w, float *logits,
                               int64_t chunk)
{
    int64_t t;
    if (chunk <= 0 || chunk > H) chunk = H;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        float *l = (float *)malloc(sizeof(float) * (size_t)E);
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        const void *xrow = (dtype == 0) ? (const void *)((const uint16_t *)x + t * H)
                                        : (const void *)((const float *)x + t * H);
        for (int e = 0; e < E; ++e) {
            float total = 0.0f;
            for (int64_t c0 = 0; c0 < H; c0 += chunk) {
                const int64_t c1 = (c0 + chunk < H) ? c0 + chunk : H;
                float acc = 0.0f;
                for (int64_t h = c0; h < c1; ++h)
                    acc = fmaf(or_load(xrow, dtype, h), or_bf16_to_f32(wg[(int64_t)e * H + h]), acc);
                total = (c0 == 0) ? acc : total + acc;
            }
            l[e] = total;
            if (logits) logits[t * E + e] = total;
        }
        /* top-k by repeated selection: strict ">" over ascending e keeps the
         * lower index first among equal logits. */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            ids[t * k + j] = best;
        }
        /* softmax over all E scores (fp64) */
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m) m = l[e];
        double Z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - m);
            Z += p[e];
        }
        for (int e = 0; e < E; ++e) p[e] = p[e] / Z;
        double S = 0.0;
        for (int j = 0; j < k; ++j) S += p[ids[t * k + j]];
        for (int j = 0; j < k; ++j) {
            double v = p[ids[t * k + j]];
            w[t * k + j] = (float)(renormalize ? v / S : v);
        }
        free(l);
        free(p);
        free(taken);
    }
}

void oracle_route_topk(const void *x, int dtype, const uint16_t *wg, int64_t T, int64_t H,
                       int E, int k, int renormalize, int32_t *ids, float *w, float *logits)
{
    oracle_route_topk_chunked(x, dtype, wg, T, H, E, k, renormalize, ids, w, logits, OR_ROUTE_CHUNK);
}

/* --------------------------------------------------------------- permute --- */

/*
 * Group the routed pairs by expert so that each expert's rows are contiguous
 * ([NEXT-AMCT] section 6: the packed MoE GMM runs one grouped matmul over all
 * experts).  Pair p = t*k + j goes to expert ids[p].  Within a group the
 * pairs keep ascending p (R11).
 *   offsets     [E+1] out, exclusive prefix of the group sizes
 *   sorted_pair [T*k] out, pair index at each grouped row
 *   pair_pos    [T*k] out, grouped row of each pair
 */
void oracle_permute(const int32_t *ids, int64_t T, int k, int E,
                    int32_t *offsets, int32_t *sorted_pair, int32_t *pair_pos)
{
    int64_t P = T * k;
    int64_t pos = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = (int32_t)pos;
        for (int64_t p = 0; p < P; ++p)
            if (ids[p] == e) sorted_pair[pos++] = (int32_t)p;
    }
    offsets[E] = (int32_t)pos;
    for (int64_t r = 0; r < P; ++r) pair_pos[sorted_pair[r]] = (int32_t)r;
}

/* ---------------------------------------------------------- int8 matmul --- */

/* Exact int8 x int8 dot product with an int32 sum ([30B-W8A8] FAQ Q1: W8A8
 * runs the matmul on integers).  |sum| <= K * 127^2 < 2^31 for K < 133144. */
static int32_t or_dot_i8(const int8_t *a, const int8_t *b, int64_t K)
{
    int32_t acc = 0;
    for (int64_t i = 0; i < K; ++i) acc += (int32_t)a[i] * (int32_t)b[i];
    return acc;
}

/* -------------------------------------------------------------- W4 codes --- */

/* One group of n <= 128 weights of one output channel (R17). */
static void or_quant_w4_group(const float *w, int64_t n, int8_t *q, float *scale, int8_t *off)
{
    float mn = 0.0f, mx = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (w[i] < mn) mn = w[i];
        if (w[i] > mx) mx = w[i];
    }
    float s = (mx - mn) / 15.0f;
    *scale = s;
    if (s == 0.0f) {
        *off = 0;
        for (int64_t i = 0; i < n; ++i) q[i] = 0;
        return;
    }
    float z = rintf(-mn / s);
    *off = (int8_t)(z - 8.0f);
    for (int64_t i = 0; i < n; ++i) {
        float u = rintf(w[i] / s) + z;
        if (u < 0.0f) u = 0.0f;
        if (u > 15.0f) u = 15.0f;
        q[i] = (int8_t)(u - 8.0f);
    }
}

/* rows x cols fp32 weights -> codes [rows][cols] in [-8, 7] (one per byte),
 * scales and offsets [rows][ceil(cols / 128)]. */
void oracle_quant_w4_rows(const float *w, int64_t rows, int64_t cols, int8_t *q, float *scales, int8_t *offs)
{
    int64_t ng = (cols + 127) / 128, r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * 128, n = cols - c0 < 128 ? cols - c0 : 128;
            or_quant_w4_group(w + r * cols + c0, n, q + r * cols + c0, &scales[r * ng + g], &offs[r * ng + g]);
        }
}

/* sum over the groups g of s_g * sum_{k in g} a_k * (q_k - o_g): each group's
 * integer sum is exact, the sum over groups is fp64. */
static double or_dot_w4(const int8_t *a, const int8_t *q, const float *scale, const int8_t *off, int64_t K)
{
    double acc = 0.0;
    int64_t ng = (K + 127) / 128;
    for (int64_t g = 0; g < ng; ++g) {
        int32_t sum = 0;
        for (int64_t kk = g * 128; kk < K && kk < (g + 1) * 128; ++kk)
            sum += (int32_t)a[kk] * ((int32_t)q[kk] - (int32_t)off[g]);
        acc += (double)scale[g] * (double)sum;
    }
    return acc;
}

static double or_silu(double g) { return g / (1.0 + exp(-g)); }

/* Output casts: dtype 0 bf16 (one RNE rounding of the fp64 value), 1 fp32. */
static void or_store(void *out, int dtype, int64_t i, double v)
{
    if (dtype == 0) ((uint16_t *)out)[i] = or_f64_to_bf16(v);
    else ((float *)out)[i] = (float)v;
}

/*
 * Grouped W8A8 GEMM.  Group g owns grouped rows [offsets[g], offsets[g+1]).
 * Grouped row r reads activation row a = gather ? gather[r] / gather_div : r.
 *   A        [*][K]    int8 codes, a_scales[a] its per-token scale
 *   B        [G][N][K] int8 codes (nn.Linear [out][in]), b_scales[g][n]
 * Epilogues (acc is the exact int32 dot product):
 *   0 RAW_I32        out[r][n] = acc                              (int32 [M][N])
 *   1 DEQUANT        out[r][n] = acc * a_scales[a] * b_scales[g][n] (out dtype [M][N])
 *   2 DEQUANT_SWIGLU N = 2*Ih; gate = columns [0, Ih), up = [Ih, 2*Ih) of the
 *                    packed gate_up_proj ([NEXT-AMCT] section 2.2);
 *                    out[r][n] = silu(gate_n) * up_n              (out dtype [M][Ih])
 */
void oracle_grouped_gemm(const int8_t *A, const float *a_scales, const int32_t *gather, int gather_div,
                         const int8_t *B, const float *b_scales, const int32_t *offsets, int G,
                         int64_t N, int64_t K, int epilogue, int out_dtype, void *out)
{
    for (int g = 0; g < G; ++g) {
        int64_t r;
#pragma omp parallel for schedule(static)
        for (r = offsets[g]; r < offsets[g + 1]; ++r) {
            int64_t a = gather ? gather[r] / gather_div : r;
            const int8_t *arow = A + a * K;
            const int8_t *Bg = B + (int64_t)g * N * K;
            const float *sg = b_scales ? b_scales + (int64_t)g * N : NULL;
            if (epilogue == 0) {
                for (int64_t n = 0; n < N; ++n)
                    ((int32_t *)out)[r * N + n] = or_dot_i8(arow, Bg + n * K, K);
            } else if (epilogue == 1) {
                for (int64_t n = 0; n < N; ++n) {
                    int32_t acc = or_dot_i8(arow, Bg + n * K, K);
                    or_store(out, out_dtype, r * N + n, (double)acc * (double)a_scales[a] * (double)sg[n]);
                }
            } else {
                int64_t Ih = N / 2;
                for (int64_t n = 0; n < Ih; ++n) {
                    int32_t ag = or_dot_i8(arow, Bg + n * K, K);
                    int32_t au = or_dot_i8(arow, Bg + (Ih + n) * K, K);
                    double gate = (double)ag * (double)a_scales[a] * (double)sg[n];
                    double up = (double)au * (double)a_scales[a] * (double)sg[Ih + n];
                    or_store(out, out_dtype, r * Ih + n, or_silu(gate) * up);
                }
            }
        }
    }
}

/*
 * Grouped W4A8 GEMM: as the W8A8 one with epilogue 1 or 2, the weights being
 * W4 codes Bq [G][N][K] (one per byte) with scales / offsets [G][N][ceil(K/128)]:
 *   acc(r, n) = sum_g s[g][n][kg] * sum_{k in kg} A[a][k] * (Bq[g][n][k] - o[g][n][kg])
 *   1 DEQUANT        out = acc * a_scales[a]
 *   2 DEQUANT_SWIGLU out = silu(gate) * up on columns [0, N/2) and [N/2, N)
 */
void oracle_w4a8_grouped_gemm(const int8_t *A, const float *a_scales, const int32_t *gather, int gather_div,
                              const int8_t *Bq, const float *b_scales, const int8_t *b_offs,
                              const int32_t *offsets, int G, int64_t N, int64_t K, int epilogue, int out_dtype,
                              void *out)
{
    int64_t ng = (K + 127) / 128;
    for (int g = 0; g < G; ++g) {
        int64_t r;
#pragma omp parallel for schedule(static)
        for (r = offsets[g]; r < offsets[g + 1]; ++r) {
            int64_t a = gather ? gather[r] / gather_div : r;
            const int8_t *arow = A + a * K;
            const int8_t *Bg = Bq + (int64_t)g * N * K;
            const float *sg = b_scales + (int64_t)g * N * ng;
            const int8_t *og = b_offs + (int64_t)g * N * ng;
            if (epilogue == 1) {
                for (int64_t n = 0; n < N; ++n) {
                    double acc = or_dot_w4(arow, Bg + n * K, sg + n * ng, og + n * ng, K);
                    or_store(out, out_dtype, r * N + n, acc * (double)a_scales[a]);
                }
            } else {
                int64_t Ih = N / 2;
                for (int64_t n = 0; n < Ih; ++n) {
                    double gate = or_dot_w4(arow, Bg + n * K, sg + n * ng, og + n * ng, K) * (double)a_scales[a];
                    double up = or_dot_w4(arow, Bg + (Ih + n) * K, sg + (Ih + n) * ng, og + (Ih + n) * ng, K) *
                                (double)a_scales[a];
                    or_store(out, out_dtype, r * Ih + n, or_silu(gate) * up);
                }
            }
        }
    }
}

/* ---------------------------------------------------------------- combine --- */

/*
 * out[t][n] = sum over the token's k slots of w[t][j] * y[pair_pos[t*k+j]][n],
 * summed in fp64 in slot order, then cast once to the output dtype.
 * y is given as fp64 (oracle-internal) or as bf16/fp32 (y_dtype 0/1).
 */
static double or_load_y(const void *y, int y_dtype, int64_t i)
{
    if (y_dtype == 2) return ((const double *)y)[i];
    return (double)or_load(y, y_dtype, i);
}

void oracle_combine(const void *y, int y_dtype, const float *w, const int32_t *pair_pos,
                    int64_t T, int k, int64_t H, void *out, int out_dtype)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        for (int64_t n = 0; n < H; ++n) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += (double)w[t * k + j] * or_load_y(y, y_dtype, (int64_t)pair_pos[t * k + j] * H + n);
            or_store(out, out_dtype, t * H + n, acc);
        }
    }
}

/* ------------------------------------------------------------ whole layer --- */

/*
 * The W8A8 MoE layer, step by step:
 *   1 route (bf16 router, fp32 logits, softmax, top-k, renormalise)
 *   2 quantise x per token
 *   3 group the (token, slot) pairs by expert
 *   4 gate_up_proj int8 GEMM -> dequantise -> SwiGLU -> h (bf16);
 *     quantise h per row; down_proj int8 GEMM -> dequantise -> y (fp64)
 *   5 combine y with the routing weights.
 * Weights: wgu [E][2I][H] int8 (gate rows then up rows), sgu [E][2I];
 *          wd [E][H][I] int8, sd [E][H]; wg [E][H] bf16.
 * Optional outputs (any may be NULL) expose the intermediate results:
 *   ids/w [T][k], xq [T][H] + sx [T], offsets [E+1], sorted_pair/pair_pos [T*k],
 *   acc_gu [T*k][2I] int32, h [T*k][I] bf16, hq [T*k][I] + sh [T*k],
 *   acc_d [T*k][H] int32.
 * out [T][H] has the dtype of x.
 */
/* The shared expert of R18 (NULL when the layer has none); the *_o members
 * are optional outputs: gate [T] (the sigmoid), h [T][Is] bf16, hq [T][Is]
 * with scales sh [T], and the down_proj int32 sums acc_d [T][H]. */
typedef struct {
    int64_t Is;
    const int8_t *wgu;   /* [2Is][H] codes, gate rows then up rows */
    const float *sgu;    /* [2Is] */
    const int8_t *wd;    /* [H][Is] */
    const float *sd;     /* [H] */
    const uint16_t *wsg; /* [H] bf16, shared_expert_gate */
    double *gate_o;
    uint16_t *h_o;
    int8_t *hq_o;
    float *sh_o;
    int32_t *acc_d_o;
} or_shared_t;

static void or_moe_layer(const void *x, int dtype, int64_t T, int64_t H, int E, int k, int64_t I,
                         const uint16_t *wg, const int8_t *wgu, const float *sgu,
                         const int8_t *wgu4, const float *sgu4, const int8_t *ogu4,
                         const int8_t *wd, const float *sd, void *out,
                         int32_t *ids_o, float *w_o, int8_t *xq_o, float *sx_o,
                         int32_t *offsets_o, int32_t *sorted_o, int32_t *pos_o,
                         int32_t *acc_gu_o, uint16_t *h_o, int8_t *hq_o, float *sh_o, int32_t *acc_d_o,
                         const or_shared_t *se)
{
    int64_t P = T * k;
    int32_t *ids = ids_o ? ids_o : (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
    float *w = w_o ? w_o : (float *)malloc(sizeof(float) * (size_t)P);
    int8_t *xq = xq_o ? xq_o : (int8_t *)malloc((size_t)(T * H));
    float *sx = sx_o ? sx_o : (float *)malloc(sizeof(float) * (size_t)T);
    int32_t *offsets = offsets_o ? offsets_o : (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sorted = sorted_o ? sorted_o : (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
    int32_t *pos = pos_o ? pos_o : (int32_t *)malloc(sizeof(int32_t) * (size_t)P);
    uint16_t *h = h_o ? h_o : (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(P * I));
    int8_t *hq = hq_o ? hq_o : (int8_t *)malloc((size_t)(P * I));
    float *sh = sh_o ? sh_o : (float *)malloc(sizeof(float) * (size_t)P);
    double *y = (double *)malloc(sizeof(double) * (size_t)(P * H));

    /* 1 */
    oracle_route_topk(x, dtype, wg, T, H, E, k, 1, ids, w, NULL);
    /* 2 */
    oracle_quant_rows(x, dtype, T, H, H, xq, sx);
    /* 3 */
    oracle_permute(ids, T, k, E, offsets, sorted, pos);
    /* 4 gate_up + SwiGLU, one grouped row at a time */
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < P; ++r) {
        int64_t p = sorted[r];
        int64_t t = p / k;
        int64_t e = ids[p];
        const int8_t *arow = xq + t * H;
        if (wgu4) {   /* W4A8 gate_up (R17) */
            int64_t ng = (H + 127) / 128;
            for (int64_t n = 0; n < I; ++n) {
                int64_t rg = e * 2 * I + n, ru = e * 2 * I + I + n;
                double gate = or_dot_w4(arow, wgu4 + rg * H, sgu4 + rg * ng, ogu4 + rg * ng, H) * (double)sx[t];
                double up = or_dot_w4(arow, wgu4 + ru * H, sgu4 + ru * ng, ogu4 + ru * ng, H) * (double)sx[t];
                h[r * I + n] = or_f64_to_bf16(or_silu(gate) * up);
            }
            continue;
        }
        for (int64_t n = 0; n < I; ++n) {
            int32_t ag = or_dot_i8(arow, wgu + (e * 2 * I + n) * H, H);
            int32_t au = or_dot_i8(arow, wgu + (e * 2 * I + I + n) * H, H);
            if (acc_gu_o) {
                acc_gu_o[r * 2 * I + n] = ag;
                acc_gu_o[r * 2 * I + I + n] = au;
            }
            double gate = (double)ag * (double)sx[t] * (double)sgu[e * 2 * I + n];
            double up = (double)au * (double)sx[t] * (double)sgu[e * 2 * I + I + n];
            h[r * I + n] = or_f64_to_bf16(or_silu(gate) * up);
        }
    }
    /* 4 quantise h per grouped row, then down_proj */
    oracle_quant_rows(h, 0, P, I, I, hq, sh);
#pragma omp parallel for schedule(static)
    for (r = 0; r < P; ++r) {
        int64_t e = ids[sorted[r]];
        for (int64_t n = 0; n < H; ++n) {
            int32_t ad = or_dot_i8(hq + r * I, wd + (e * H + n) * I, I);
            if (acc_d_o) acc_d_o[r * H + n] = ad;
            y[r * H + n] = (double)ad * (double)sh[r] * (double)sd[e * H + n];
        }
    }
    /* 5 */
    if (!se) {
        oracle_combine(y, 2, w, pos, T, k, H, out, dtype);
    } else {
        /* R18: the shared expert on every token, then its gated output is
         * added after the routed slots */
        int64_t Is = se->Is;
        uint16_t *hs = se->h_o ? se->h_o : (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(T * Is));
        int8_t *hqs = se->hq_o ? se->hq_o : (int8_t *)malloc((size_t)(T * Is));
        float *shs = se->sh_o ? se->sh_o : (float *)malloc(sizeof(float) * (size_t)T);
        double *z = (double *)malloc(sizeof(double) * (size_t)(T * H));
        double *sig = (double *)malloc(sizeof(double) * (size_t)T);
        int64_t t;
#pragma omp parallel for schedule(static)
        for (t = 0; t < T; ++t) {
            for (int64_t n = 0; n < Is; ++n) {
                double gate = (double)or_dot_i8(xq + t * H, se->wgu + n * H, H) * (double)sx[t] * (double)se->sgu[n];
                double up = (double)or_dot_i8(xq + t * H, se->wgu + (Is + n) * H, H) * (double)sx[t] *
                            (double)se->sgu[Is + n];
                hs[t * Is + n] = or_f64_to_bf16(or_silu(gate) * up);
            }
        }
        oracle_quant_rows(hs, 0, T, Is, Is, hqs, shs);
#pragma omp parallel for schedule(static)
        for (t = 0; t < T; ++t) {
            for (int64_t n = 0; n < H; ++n) {
                int32_t ad = or_dot_i8(hqs + t * Is, se->wd + n * Is, Is);
                if (se->acc_d_o) se->acc_d_o[t * H + n] = ad;
                z[t * H + n] = (double)ad * (double)shs[t] * (double)se->sd[n];
            }
            double g = 0.0; /* R19 */
            for (int64_t c = 0; c < H; ++c)
                g += (double)or_load(x, dtype, t * H + c) * (double)or_bf16_to_f32(se->wsg[c]);
            sig[t] = 1.0 / (1.0 + exp(-g));
            if (se->gate_o) se->gate_o[t] = sig[t];
        }
#pragma omp parallel for schedule(static)
        for (t = 0; t < T; ++t) {
            for (int64_t n = 0; n < H; ++n) {
                double acc = 0.0;
                for (int j = 0; j < k; ++j) acc += (double)w[t * k + j] * y[(int64_t)pos[t * k + j] * H + n];
                acc += sig[t] * z[t * H + n];
                or_store(out, dtype, t * H + n, acc);
            }
        }
        if (!se->h_o) free(hs);
        if (!se->hq_o) free(hqs);
        if (!se->sh_o) free(shs);
        free(z);
        free(sig);
    }

    if (!ids_o) free(ids);
    if (!w_o) free(w);
    if (!xq_o) free(xq);
    if (!sx_o) free(sx);
    if (!offsets_o) free(offsets);
    if (!sorted_o) free(sorted);
    if (!pos_o) free(pos);
    if (!h_o) free(h);
    if (!hq_o) free(hq);
    if (!sh_o) free(sh);
    free(y);
}

void oracle_moe_layer(const void *x, int dtype, int64_t T, int64_t H, int E, int k, int64_t I,
                      const uint16_t *wg, const int8_t *wgu, const float *sgu,
                      const int8_t *wd, const float *sd, void *out,
                      int32_t *ids_o, float *w_o, int8_t *xq_o, float *sx_o,
                      int32_t *offsets_o, int32_t *sorted_o, int32_t *pos_o,
                      int32_t *acc_gu_o, uint16_t *h_o, int8_t *hq_o, float *sh_o, int32_t *acc_d_o)
{
    or_moe_layer(x, dtype, T, H, E, k, I, wg, wgu, sgu, NULL, NULL, NULL, wd, sd, out, ids_o, w_o, xq_o, sx_o,
                 offsets_o, sorted_o, pos_o, acc_gu_o, h_o, hq_o, sh_o, acc_d_o, NULL);
}

/* The layer with W4A8 gate_up weights (R17): codes wgu4 [E][2I][H], scales
 * and offsets [E][2I][ceil(H/128)]; down_proj W8A8 as above. */
void oracle_moe_layer_w4(const void *x, int dtype, int64_t T, int64_t H, int E, int k, int64_t I,
                         const uint16_t *wg, const int8_t *wgu4, const float *sgu4, const int8_t *ogu4,
                         const int8_t *wd, const float *sd, void *out,
                         int32_t *ids_o, float *w_o, int8_t *xq_o, float *sx_o,
                         int32_t *offsets_o, int32_t *sorted_o, int32_t *pos_o,
                         uint16_t *h_o, int8_t *hq_o, float *sh_o)
{
    or_moe_layer(x, dtype, T, H, E, k, I, wg, NULL, NULL, wgu4, sgu4, ogu4, wd, sd, out, ids_o, w_o, xq_o, sx_o,
                 offsets_o, sorted_o, pos_o, NULL, h_o, hq_o, sh_o, NULL, NULL);
}

/* The layer with a shared expert (R18, R19): wsgu [2Is][H] int8 + ssgu [2Is],
 * wsd [H][Is] int8 + ssd [H], wsg [H] bf16.  The routed intermediates are the
 * same optional outputs as oracle_moe_layer's; gate_o [T] (fp64 sigmoid),
 * hs_o [T][Is] bf16, hqs_o [T][Is] + shs_o [T], accs_d_o [T][H] those of the
 * shared expert. */
void oracle_moe_layer_shared(const void *x, int dtype, int64_t T, int64_t H, int E, int k, int64_t I,
                             const uint16_t *wg, const int8_t *wgu, const float *sgu,
                             const int8_t *wd, const float *sd,
                             int64_t Is, const int8_t *wsgu, const float *ssgu, const int8_t *wsd, const float *ssd,
                             const uint16_t *wsg, void *out,
                             int32_t *ids_o, float *w_o, int8_t *xq_o, float *sx_o,
                             int32_t *offsets_o, int32_t *sorted_o, int32_t *pos_o,
                             uint16_t *h_o, int8_t *hq_o, float *sh_o,
                             double *gate_o, uint16_t *hs_o, int8_t *hqs_o, float *shs_o, int32_t *accs_d_o)
{
    or_shared_t se = {Is, wsgu, ssgu, wsd, ssd, wsg, gate_o, hs_o, hqs_o, shs_o, accs_d_o};
    or_moe_layer(x, dtype, T, H, E, k, I, wg, wgu, sgu, NULL, NULL, NULL, wd, sd, out, ids_o, w_o, xq_o, sx_o,
                 offsets_o, sorted_o, pos_o, NULL, h_o, hq_o, sh_o, NULL, &se);
}

/*
 * The same layer restricted to a subset of tokens.  The layer has no term that
 * couples tokens (each token's output depends on its own row of x only), so the
 * rows of `out` for tokens `tok[0..n)` equal those of the full layer.  Used to
 * check full-size runs on a sample.  out is [n][H].
 */
void oracle_moe_layer_tokens(const void *x, int dtype, int64_t H, int E, int k, int64_t I,
                             const uint16_t *wg, const int8_t *wgu, const float *sgu,
                             const int8_t *wd, const float *sd,
                             const int64_t *tok, int64_t n, void *out)
{
    size_t esz = dtype == 0 ? 2 : 4;
    unsigned char *xs = (unsigned char *)malloc(esz * (size_t)(n * H));
    for (int64_t i = 0; i < n; ++i)
        memcpy(xs + esz * (size_t)(i * H), (const unsigned char *)x + esz * (size_t)(tok[i] * H), esz * (size_t)H);
    oracle_moe_layer(xs, dtype, n, H, E, k, I, wg, wgu, sgu, wd, sd, out,
                     NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    free(xs);
}

void oracle_moe_layer_w4_tokens(const void *x, int dtype, int64_t H, int E, int k, int64_t I,
                                const uint16_t *wg, const int8_t *wgu4, const float *sgu4, const int8_t *ogu4,
                                const int8_t *wd, const float *sd, const int64_t *tok, int64_t n, void *out)
{
    size_t esz = dtype == 0 ? 2 : 4;
    unsigned char *xs = (unsigned char *)malloc(esz * (size_t)(n * H));
    for (int64_t i = 0; i < n; ++i)
        memcpy(xs + esz * (size_t)(i * H), (const unsigned char *)x + esz * (size_t)(tok[i] * H), esz * (size_t)H);
    oracle_moe_layer_w4(xs, dtype, n, H, E, k, I, wg, wgu4, sgu4, ogu4, wd, sd, out,
                        NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    free(xs);
}

void oracle_moe_layer_shared_tokens(const void *x, int dtype, int64_t H, int E, int k, int64_t I,
                                    const uint16_t *wg, const int8_t *wgu, const float *sgu,
                                    const int8_t *wd, const float *sd,
                                    int64_t Is, const int8_t *wsgu, const float *ssgu, const int8_t *wsd,
                                    const float *ssd, const uint16_t *wsg,
                                    const int64_t *tok, int64_t n, void *out)
{
    size_t esz = dtype == 0 ? 2 : 4;
    unsigned char *xs = (unsigned char *)malloc(esz * (size_t)(n * H));
    for (int64_t i = 0; i < n; ++i)
        memcpy(xs + esz * (size_t)(i * H), (const unsigned char *)x + esz * (size_t)(tok[i] * H), esz * (size_t)H);
    oracle_moe_layer_shared(xs, dtype, n, H, E, k, I, wg, wgu, sgu, wd, sd, Is, wsgu, ssgu, wsd, ssd, wsg, out,
                            NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    free(xs);
}
