/*
 * w8a8moe.h -- C ABI of the W8A8 INT8 mixture-of-experts feed-forward layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (sources are web pages, cited by title and section):
 *   1. an unquantised bf16 router scores every expert, applies softmax, keeps
 *      the top-k experts and renormalises their weights
 *      ("Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer, sections
 *      3.1-3.3; "Qwen3-235B-A22B-quantized.w8a8" file guide, shard contents);
 *   2. activations are quantised to int8 per token at run time, symmetric,
 *      scale = max|x| / 127 ("Qwen3.6-35B-A3B-w8a8 config.json and
 *      recipe.yaml" walkthrough, group_0 "input_activations");
 *   3. the (token, slot) pairs are grouped by expert (the packed MoE grouped
 *      matmul of the "Qwen3-Next-80B-A3B-Instruct in AMCT" case, section 6);
 *   4. gate_proj / up_proj / down_proj run as int8 x int8 -> int32 grouped
 *      GEMMs against static per-output-channel symmetric int8 weights
 *      (group_0 "weights" of the same walkthrough), with a per-token x
 *      per-channel dequantisation and SwiGLU;
 *   5. each token's output is the sum of its k selected experts' outputs,
 *      weighted by their routing weights (the same explainer, section 3.1:
 *      the top-k experts the router picks are the ones that take part in the
 *      token's forward pass).
 *
 * Conventions shared by every call
 *   - Every pointer argument named as device memory is a device pointer owned
 *     by the caller; the library allocates nothing and keeps no state between
 *     calls.  Calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream) and never synchronise the host.
 *   - Matrices are row-major and contiguous unless a leading dimension is
 *     given.  Weights use the nn.Linear [out][in] layout.
 *   - Contraction lengths (H, I, K, cols of a quantised row) and output widths
 *     N must be multiples of 16, and every device pointer must be 16-byte
 *     aligned.  1 <= k <= E <= 256.  A zero row/token count is a valid no-op.
 *   - Inputs must be finite; results for non-finite inputs are unspecified.
 *   - Arguments are checked before anything is launched; a rejected call
 *     returns a negative status and writes nothing.  W8A8_ERR_HIP reports a
 *     failed launch (the HIP error is cleared).  Kernel faults surface on the
 *     caller's next synchronisation, like any HIP kernel.
 *   - Number formats (the one scheme supported, nothing else is accepted):
 *     int8 codes in [-127, 127] (-128 never produced), round-half-to-even,
 *     fp32 scales, bf16 stored as its 16-bit pattern.
 */
#ifndef W8A8MOE_H
#define W8A8MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define W8A8_OK 0
#define W8A8_ERR_INVALID_ARG (-1)        /* null pointer, bad enum, k > E, negative size */
#define W8A8_ERR_UNSUPPORTED_SHAPE (-2)  /* contraction or width not a multiple of 16, E > 256 */
#define W8A8_ERR_ALIGNMENT (-3)          /* a pointer or leading dimension not 16-byte aligned */
#define W8A8_ERR_WORKSPACE_TOO_SMALL (-4)
#define W8A8_ERR_HIP (-5)                /* a HIP launch failed */
#define W8A8_ERR_SCRATCH_LIMIT (-6)      /* more scratch than w8a8_grouped_gemm_noalloc's fixed buffer */

/* element types */
#define W8A8_BF16 0
#define W8A8_F32 1
#define W8A8_I32 2

/* weight layouts of the grouped GEMM */
#define W8A8_B_ROWMAJOR 0 /* [G][N][K], nn.Linear [out][in] per group */
#define W8A8_B_PACKED 1   /* the MFMA-fragment layout written by w8a8_pack_weights */

/* grouped GEMM epilogues */
#define W8A8_EPI_RAW_I32 0        /* out = int32 accumulator */
#define W8A8_EPI_DEQUANT 1        /* out = acc * a_scale[row] * b_scale[group][col] */
#define W8A8_EPI_DEQUANT_SWIGLU 2 /* N = 2*I packed gate|up; out[:, n] = silu(gate_n) * up_n */

/* Text of a status code (static storage). */
const char *w8a8_status_string(int status);

/*
 * Per-row symmetric int8 quantisation: for each row r,
 *   scales[r] = max_c |x[r][c]| / 127   (fp32 divide; 0 for an all-zero row)
 *   q[r][c]   = clamp(round_half_even(x[r][c] / scales[r]), -127, 127)
 * Used for the per-token dynamic activation quantisation and, with the rows
 * of a weight matrix, for the static per-output-channel weight quantisation
 * (the same computation; "Qwen3.6-35B-A3B-w8a8 config.json and recipe.yaml"
 * walkthrough, group_0 "input_activations" and "weights").
 *   x       device, [rows][ld_x] of x_dtype (W8A8_BF16 or W8A8_F32), read
 *   q       device, [rows][cols] int8, written
 *   scales  device, [rows] fp32, written
 * cols % 16 == 0, ld_x >= cols, ld_x * element size % 16 == 0.
 */
int w8a8_quant_act(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   int8_t *q, float *scales, void *stream);

/*
 * MoE router ("Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer,
 * section 3.1: hidden state -> one score per expert -> softmax -> top-k).
 *   logit[t][e] = sum over the chunks h = 512c .. min(H, 512c + 512) - 1, in
 *                 ascending c (fp32 adds, the first chunk's sum as the start),
 *                 of each chunk's fp32 fused multiply-add chain in ascending h
 *                 from +0 of x[t][h] * w_gate[e][h] (bf16 operands widened
 *                 exactly; fp32 x used as is); for H <= 512 one chain
 *   topk_ids[t][0..k) = the k largest logits, larger first, equal logits by
 *                 lower expert index
 *   topk_w[t][j]  = softmax probability of topk_ids[t][j]; with renormalize != 0
 *                 divided by the sum over the k selected
 *   x         device, [T][H] x_dtype (W8A8_BF16 or W8A8_F32)
 *   w_gate    device, [E][H] bf16 (unquantised router weight)
 *   topk_ids  device, [T][k] int32, written
 *   topk_w    device, [T][k] fp32, written
 *   logits_out device, [T][E] fp32, written when not NULL
 * T * H * 4 and E * H * 2 must stay below 2^31 (32-bit byte offsets).
 */
int moe_route_topk(const void *x, int x_dtype, const uint16_t *w_gate, int64_t T, int64_t H,
                   int E, int k, int renormalize, int32_t *topk_ids, float *topk_w,
                   float *logits_out, void *stream);

/*
 * The same router with the weight's moe_router_pack copy as well
 * (w_gate_packed, device, [H/8][E][8] bf16, or NULL for moe_route_topk's
 * behaviour): with bf16 tokens, few-token calls then read it (coalesced, the
 * chunks of each score on several waves).  The results are identical.  Same
 * arguments and limits otherwise.
 */
int moe_route_topk_packed(const void *x, int x_dtype, const uint16_t *w_gate, const uint16_t *w_gate_packed,
                          int64_t T, int64_t H, int E, int k, int renormalize, int32_t *topk_ids,
                          float *topk_w, float *logits_out, void *stream);

/*
 * The router weight widened once to fp32 for the layer (w8a8_moe_weights
 * .w_gate_f32): w_gate_f32[i] = w_gate[i] exactly (a bf16 value is the upper
 * half of an fp32).  w_gate device [E][H] bf16; w_gate_f32 device [E][H] fp32,
 * written.  H % 16 == 0.
 */
int moe_router_widen(const uint16_t *w_gate, int E, int64_t H, float *w_gate_f32, void *stream);

/*
 * The router weight re-laid once for few-token layers (w8a8_moe_weights
 * .w_gate_packed): w_gate_packed[(j * E + e) * 8 + i] = w_gate[e * H + 8 j + i]
 * for j < H / 8, i < 8, i.e. [H/8][E][8] bf16: per group of 8 hidden indices
 * the experts' 16-byte pieces lie side by side, so a wavefront that runs 64
 * experts' score chains reads one contiguous kilobyte per step.  A pure copy:
 * the scores do not change.  w_gate device [E][H] bf16; w_gate_packed device,
 * E * H bf16, written.  H % 16 == 0.
 */
int moe_router_pack(const uint16_t *w_gate, int E, int64_t H, uint16_t *w_gate_packed, void *stream);

/*
 * Group the routed pairs by expert (the packed MoE grouped matmul,
 * "Qwen3-Next-80B-A3B-Instruct in AMCT" case, section 6).  Pair p = t*k + j is
 * routed to expert topk_ids[p]; pairs are stably sorted by (expert, p).
 *   offsets     device, [E+1] int32, written: offsets[e] = first grouped row of
 *               expert e, offsets[E] = T*k
 *   sorted_pair device, [T*k] int32, written: pair index at each grouped row
 *   pair_pos    device, [T*k] int32, written: grouped row of each pair
 *   ws          device scratch of at least moe_permute_workspace_size() bytes
 * Every id must lie in [0, E) (ids out of range are not detected).
 */
size_t moe_permute_workspace_size(int64_t T, int k, int E);
int moe_permute(const int32_t *topk_ids, int64_t T, int k, int E, int32_t *offsets,
                int32_t *sorted_pair, int32_t *pair_pos, void *ws, size_t ws_bytes, void *stream);

/*
 * Static weights are re-laid once, after quantisation, so that every
 * wavefront of the grouped GEMM fetches its matrix-core operand as 1 KiB of
 * contiguous memory.  For group g, 32-row block nb and 128-byte K step ks, a
 * 4 KiB chunk at byte ((g * NB + nb) * KS + ks) * 4096 holds, at offset
 * s * 1024 + l * 16 (s = 0..3, l = 0..63), bytes [64 * (l / 32) + 16 * s, +16)
 * of step ks of row 32 * nb + l % 32; rows beyond N and bytes beyond K are
 * zero.  NB = ceil(N / 32), KS = ceil(K / 128).
 *   B       device, [G][N][K] int8, read
 *   packed  device, w8a8_packed_weights_size(G, N, K) bytes, written
 * K % 16 == 0, N % 16 == 0.
 */
size_t w8a8_packed_weights_size(int G, int64_t N, int64_t K);
int w8a8_pack_weights(const int8_t *B, int G, int64_t N, int64_t K, int8_t *packed, void *stream);

/*
 * Grouped W8A8 GEMM: for group g and every grouped row r in
 * [group_offsets[g], group_offsets[g+1]), with activation row
 * a = a_row_gather ? a_row_gather[r] / gather_div : r,
 *   acc[r][n] = sum_k A[a][k] * B[g][n][k]     (exact int32)
 * then the epilogue (W8A8_EPI_*):
 *   RAW_I32        out [M_total][N] int32 = acc
 *   DEQUANT        out [M_total][N] out_dtype = acc * a_scales[a] * b_scales[g][n]
 *   DEQUANT_SWIGLU out [M_total][N/2] out_dtype = silu(gate) * up with
 *                  gate = dequant(acc[r][n]), up = dequant(acc[r][N/2 + n]) (the
 *                  packed gate_up_proj layout of the AMCT case, section 2.2)
 *   A             device, [A_rows][K] int8 (rows addressed by a, all < A_rows)
 *   a_scales      device, fp32 per activation row (unused for RAW_I32)
 *   a_row_gather  device, [M_total] int32 or NULL
 *   B             device, int8 in layout b_layout (W8A8_B_ROWMAJOR [G][N][K] or
 *                 W8A8_B_PACKED as written by w8a8_pack_weights);
 *   b_scales      device [G][N] fp32
 *   group_offsets device, [G+1] int32, non-decreasing, group_offsets[0] = 0,
 *                 group_offsets[G] = M_total (not checked: device memory)
 *   ws            device scratch of at least w8a8_grouped_gemm_workspace_size() bytes
 * out_dtype: W8A8_BF16 or W8A8_F32 (W8A8_I32 with RAW_I32).  K % 16 == 0,
 * N % 16 == 0, N % 64 == 0 for SWIGLU, G <= 4096.  A_rows * K and one group of B must stay
 * below 2^31 bytes (the kernels address them with 32-bit byte offsets); larger
 * shapes return W8A8_ERR_UNSUPPORTED_SHAPE.
 */
size_t w8a8_grouped_gemm_workspace_size(int64_t M_total, int64_t N, int G);
int w8a8_grouped_gemm(const int8_t *A, int64_t A_rows, const float *a_scales,
                      const int32_t *a_row_gather, int gather_div, const int8_t *B, int b_layout,
                      const float *b_scales, const int32_t *group_offsets, int G, int64_t M_total,
                      int64_t N, int64_t K, int epilogue, int out_dtype, void *out, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code being captured into a
 * HIP graph, tight serving loops, hosts that forbid allocation): the same
 * grouped GEMM without a workspace argument.  Its only scratch, the tile table
 * that a first kernel builds from group_offsets on the device, lives in a
 * fixed array of W8A8_NOALLOC_SCRATCH_BYTES in each GPU's memory, reserved
 * with the library's code and held until the process ends; the call allocates
 * nothing.  Arguments, results and limits are those of w8a8_grouped_gemm (the
 * same kernels, the same bits).  A problem whose tile table would exceed the
 * array (w8a8_grouped_gemm_workspace_size(M_total, N, G) >
 * W8A8_NOALLOC_SCRATCH_BYTES) returns W8A8_ERR_SCRATCH_LIMIT before anything
 * is launched.  Every call on one GPU shares that GPU's array: calls on one
 * stream are ordered, but calls that may overlap on one GPU (other streams,
 * other host threads) race and must not be issued.  Nothing in the array has
 * to start cleared: each call writes every table entry it reads.
 */
#define W8A8_NOALLOC_SCRATCH_BYTES (4 << 20)
int w8a8_grouped_gemm_noalloc(const int8_t *A, int64_t A_rows, const float *a_scales,
                              const int32_t *a_row_gather, int gather_div, const int8_t *B, int b_layout,
                              const float *b_scales, const int32_t *group_offsets, int G, int64_t M_total,
                              int64_t N, int64_t K, int epilogue, int out_dtype, void *out, void *stream);

/*
 * W4A8 weights ("Qwen3-1.7B-W4A8 on Ascend", section on 4bit weights, items 1
 * and 2: groups of 128 weights share a scale and an offset; 4-bit codes in
 * two's complement).  Per output channel (row of w) and group of 128
 * consecutive inputs (the last group of a row may be shorter), over the range
 * [min(w, 0), max(w, 0)]: s = (max - min) / 15, z = rint(-min / s),
 * u = clamp(rint(w / s) + z, 0, 15) (IEEE fp32 divides, round half to even);
 * code u - 8 and offset z - 8, both in [-8, 7]; w ~ (code - offset) * s.  A
 * group of zeros has s = 0, codes and offset 0.
 *   w        device [rows][cols] fp32 (cols % 16 == 0)
 *   q        device [rows][cols] int8 codes (one per byte)
 *   scales   device [rows][ceil(cols / 128)] fp32;  offsets the same, int8
 */
int w4a8_quant_weights(const float *w, int64_t rows, int64_t cols, int8_t *q, float *scales,
                       int8_t *offsets, void *stream);

/*
 * W4 codes [G][N][K] (one per byte) packed two per byte for the W4A8 GEMM:
 * for group g, 32-row block nb and 128-column step ks, a 2 KiB chunk at byte
 * ((g * NB + nb) * KS + ks) * 2048 holds at l * 32 + 16 * p + 4 * j + i
 * (l = 0..63, p = 0..1, j, i = 0..3) the code of column
 * 128 ks + 64 (l / 32) + 32 p + 4 j + i of row 32 nb + l % 32 in the low
 * nibble and the code 16 columns further in the high nibble; zero padding.
 * NB = ceil(N / 32), KS = ceil(K / 128).  After the codes (at the next
 * multiple of 256 bytes) the buffer holds the group scales re-laid step-major,
 * [G][KS][N] fp32, then (256-byte aligned) the offsets [G][KS][N] int8: one
 * 128-column step of a wave's 64 columns is then one contiguous read.
 *   q        device [G][N][K] codes;  scales / offsets device [G][N][KS] (as
 *            w4a8_quant_weights writes them, rows = G*N)
 *   packed   device, w4a8_packed_weights_size(G, N, K) bytes
 */
size_t w4a8_packed_weights_size(int G, int64_t N, int64_t K);
int w4a8_pack_weights(const int8_t *q, const float *scales, const int8_t *offsets, int G, int64_t N, int64_t K,
                      uint8_t *packed, void *stream);

/*
 * Grouped W4A8 GEMM: as w8a8_grouped_gemm with epilogue DEQUANT or
 * DEQUANT_SWIGLU, B the packed buffer of w4a8_pack_weights (codes q, group
 * scales s and offsets o, groups of 128 inputs kg):
 *   acc[r][n] = sum_kg s[g][n][kg] * sum_{k in kg} A[a][k] * (q[g][n][k] - o[g][n][kg])
 *   DEQUANT out = acc * a_scales[a];  DEQUANT_SWIGLU out = silu(gate) * up
 * The workspace is w8a8_grouped_gemm_workspace_size(M_total, N, G).  Same
 * limits as w8a8_grouped_gemm.
 */
int w4a8_grouped_gemm(const int8_t *A, int64_t A_rows, const float *a_scales,
                      const int32_t *a_row_gather, int gather_div, const uint8_t *B_packed,
                      const int32_t *group_offsets, int G, int64_t M_total, int64_t N, int64_t K, int epilogue,
                      int out_dtype, void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Dense W8A8 linear: the other Linears of the scheme, e.g. an attention
 * block's q_proj / k_proj / v_proj / o_proj, which the "Qwen3-235B-A22B-
 * quantized.w8a8" guide lists as INT8 next to the experts, and which the
 * recipe's targets [Linear] cover ("Qwen3.6-35B-A3B-w8a8" recipe.yaml).
 *   out[m][n] = (sum_k xq[m][k] * w[n][k]) * s_x[m] * w_scales[n]
 * with xq, s_x the per-row int8 codes of x (as w8a8_quant_act).  A fused QKV
 * projection is one call over the concatenated [q; k; v] weight rows: with
 * per-output-channel scales its columns are exactly those of the three
 * separate linears.
 *   x        device [M][K] x_dtype (row-major, contiguous)
 *   w_packed int8 codes [N][K] packed by w8a8_pack_weights (one group)
 *   w_scales device [N] fp32;  out device [M][N] out_dtype (W8A8_BF16 or W8A8_F32)
 *   ws       device scratch of w8a8_linear_workspace_size(M, N, K) bytes (the
 *            codes and scales of x; with few rows also the int32 partial sums
 *            of slices of K: such a linear has too few output tiles for the
 *            chip, so K is split and a second kernel adds the slices exactly
 *            and dequantises, with the same result bit for bit)
 * K % 16 == 0, N % 16 == 0, 16-byte aligned pointers, M*K and the packed
 * weight bytes below 2^31.  Returns 0 (also for M = 0) or a negative status;
 * nothing is launched on error.
 */
size_t w8a8_linear_workspace_size(int64_t M, int64_t N, int64_t K);
int w8a8_linear(const void *x, int x_dtype, int64_t M, int64_t K, const int8_t *w_packed,
                const float *w_scales, int64_t N, void *out, int out_dtype, void *ws, size_t ws_bytes,
                void *stream);
/* The same GEMM on rows already quantised (xq [M][K] int8, x_scales [M] fp32,
 * e.g. by w8a8_quant_act).  ws: w8a8_linear_q_workspace_size(M, N, K) bytes
 * for the split of K (0 when the shape is not split), or NULL: then K is
 * never split (same result, fewer tiles in flight). */
size_t w8a8_linear_q_workspace_size(int64_t M, int64_t N, int64_t K);
int w8a8_linear_q(const int8_t *xq, const float *x_scales, int64_t M, int64_t K, const int8_t *w_packed,
                  const float *w_scales, int64_t N, void *out, int out_dtype, void *ws, size_t ws_bytes,
                  void *stream);

/*
 * Weighted combine of the expert outputs ("Qwen3-30B-A3B-Instruct-2507-
 * quantized.w8a8" explainer, section 3.1: only the top-k experts the router
 * picks take part in a token's forward pass, weighted by its scores):
 *   out[t][n] = sum_{j<k} topk_w[t][j] * y[pair_pos[t*k+j]][n]
 * accumulated in fp32 in slot order, then rounded once to out_dtype.
 *   y device [T*k][H] y_dtype;  topk_w device [T][k];  pair_pos device [T*k]
 *   out device [T][H] out_dtype
 */
int moe_combine(const void *y, int y_dtype, const float *topk_w, const int32_t *pair_pos,
                int64_t T, int k, int64_t H, void *out, int out_dtype, void *stream);

/*
 * Layer weights (caller-owned device memory):
 *   w_gate    [E][H]    bf16 router (not quantised)
 *   w_gate_up int8 gate_up_proj codes [E][2I][H] (rows 0..I-1 gate_proj, rows
 *             I..2I-1 up_proj) in the packed layout of w8a8_pack_weights
 *   s_gate_up [E][2I]   fp32 per-output-channel scales
 *   w_down    int8 down_proj codes [E][H][I], packed the same way
 *   s_down    [E][H]    fp32
 *   w_gate_f32 [E][H]   fp32: w_gate widened by moe_router_widen (exact), or
 *             NULL.  When given, the router stages it as is instead of
 *             widening w_gate inside every call; the scores are identical.
 *   w_gate_packed  w_gate re-laid by moe_router_pack, or NULL.  When given,
 *             few-token layers read it instead of w_gate's rows (coalesced,
 *             and the chunks of each score run on several waves); the scores
 *             are identical.
 *   w4_gate_up W4A8 gate_up_proj: the w4a8_pack_weights buffer of its codes
 *             [E][2I][H] with their scales and offsets, or NULL.  When given,
 *             gate_up runs as the W4A8 GEMM and w_gate_up, s_gate_up may be
 *             NULL; down_proj stays W8A8.
 *   Shared expert ("Qwen3-Next-80B-A3B-Instruct in AMCT" section 2.2: the
 *   shared expert is a dense path quantised like the other Linears; the
 *   "Qwen3.6-35B-A3B-w8a8" recipe keeps shared_expert_gate out of the
 *   quantisation), all NULL / I_shared = 0 for a layer without one:
 *   I_shared  its intermediate size (multiple of 32)
 *   w_shared_gate_up  int8 codes [2*I_shared][H] (gate rows then up rows),
 *             packed by w8a8_pack_weights as one group;  s_shared_gate_up [2*I_shared]
 *   w_shared_down     int8 codes [H][I_shared], packed;  s_shared_down [H]
 *   w_shared_gate     [H] bf16 shared_expert_gate (not quantised)
 *   Every token runs through the shared expert with its int8 codes (the
 *   steps of a routed expert) and the layer adds sigmoid(x . w_shared_gate)
 *   times its output after the k routed slots; the logit is an fp32 sum.
 *   A shared expert with W4A8 routed gate_up weights is not supported
 *   (W8A8_ERR_UNSUPPORTED_SHAPE).
 * H % 16 == 0, I % 32 == 0.  32-bit byte offsets address the operands, so
 * T * H * 4, E * H * 2 (E * H * 4 with w_gate_f32), T * k * I and one
 * expert's packed weights must stay below 2^31; larger layers return
 * W8A8_ERR_UNSUPPORTED_SHAPE.
 */
typedef struct {
    int E, k;
    int64_t H, I;
    const uint16_t *w_gate;
    const int8_t *w_gate_up;
    const float *s_gate_up;
    const int8_t *w_down;
    const float *s_down;
    const float *w_gate_f32;
    const uint8_t *w4_gate_up;
    int64_t I_shared;
    const int8_t *w_shared_gate_up;
    const float *s_shared_gate_up;
    const int8_t *w_shared_down;
    const float *s_shared_down;
    const uint16_t *w_shared_gate;
    const uint16_t *w_gate_packed;
} w8a8_moe_weights;

/*
 * The whole layer ("Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer,
 * sections 2 and 3.1: a bf16 router picks the top-k experts of each token,
 * whose int8 gate/up/down Linears run on per-token int8 activations, and the
 * token's output sums their outputs with the routing weights; the steps and
 * their sources are listed at the top of this header):
 * route -> quantise x -> permute -> gate_up GEMM + SwiGLU ->
 * quantise h -> down GEMM -> combine, all launched on `stream` (with a shared
 * expert, its GEMMs and h quantisation run in the same stages as the routed
 * ones and the combine adds its gated output).
 *   x   device [T][H] x_dtype (W8A8_BF16 or W8A8_F32);  out device [T][H] x_dtype
 *   ws  device scratch of at least w8a8_moe_layer_workspace_size() bytes
 * Returns 0 (also for T = 0) or a negative status.
 */
size_t w8a8_moe_layer_workspace_size(const w8a8_moe_weights *W, int64_t T, int x_dtype);
int w8a8_moe_layer(const w8a8_moe_weights *W, const void *x, int x_dtype, int64_t T, void *out,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * The same layer (same sources), recording `n_events` (<= W8A8_LAYER_STAGES + 1) hipEvent_t
 * handles on `stream`: events[0] before the first stage and events[i] after
 * stage i, stages in the order route, quantise x, permute, gate_up GEMM,
 * quantise h, down GEMM, combine.  A null entry skips that mark, so a caller
 * can bracket one stage without adding records between the others.  Used to
 * time the stages from the host.  Marks recorded while `stream` is being
 * captured into a HIP graph only order the graph's nodes; they do not time
 * its replays.
 */
#define W8A8_LAYER_STAGES 7
int w8a8_moe_layer_events(const w8a8_moe_weights *W, const void *x, int x_dtype, int64_t T,
                          void *out, void *ws, size_t ws_bytes, void *stream,
                          void *const *events, int n_events);

/*
 * Pointers into the layer workspace (the layer's steps, see w8a8_moe_layer)
 * of the intermediate results of the last
 * call with the same (W, T, x_dtype, ws): ids [T][k] i32, w [T][k] f32,
 * xq [T][H] i8, sx [T] f32, offsets [E+1] i32, sorted_pair / pair_pos [T*k] i32,
 * h [T*k][I] bf16, hq [T*k][I] i8, sh [T*k] f32,
 * y [T*k][H] i16 and y_exp [T*k][ceil(H/64)] i8: the down projection's
 * output (grouped row order) as 16-bit fixed point, value = y * 2^y_exp of its
 * row and 64-column segment, the exponent chosen so that the segment's largest
 * magnitude lies in [2^13, 2^14) (absolute error at most 2^-14 of it).
 * With a shared expert y and y_exp have T*k + T rows, rows T*k + t holding
 * the shared expert's output for token t, and four more entries follow:
 * hs [T][I_shared] bf16, hqs [T][I_shared] i8, shs [T] f32 (its h, codes and
 * scales) and gate [T] f32 (the sigmoid of each token's gate logit); without
 * one they point at zero-sized parts.
 * Index order of `ptrs`: as listed.  For inspection and stage-by-stage checks.
 */
#define W8A8_LAYER_INTERMEDIATES 16
int w8a8_moe_layer_intermediates(const w8a8_moe_weights *W, int64_t T, int x_dtype, void *ws,
                                 void **ptrs);

#ifdef __cplusplus
}
#endif

#endif /* W8A8MOE_H */
