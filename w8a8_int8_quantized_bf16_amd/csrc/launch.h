// Host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w8a8 {

hipError_t launch_quant_rows(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                             int8_t *q, float *scales, hipStream_t st);
// W4 codes [rows][cols] (one per byte, in [-8, 7]), scales and offsets
// [rows][ceil(cols / 128)] of fp32 weights; cols even
hipError_t launch_quant_w4(const float *w, int64_t rows, int64_t cols, int8_t *q, float *scales, int8_t *offs,
                           hipStream_t st);

// wg_f32: the same router weight widened to fp32, or nullptr (then the
// kernel widens wg while staging it).  wg_packed: the same weight in the
// moe_router_pack layout ([H/8][E][8] bf16), or nullptr.  xq/sx: when
// route_fuses_quant() holds, the router may also write the tokens' int8 codes
// [T,H] and scales [T] (pass nullptr otherwise; non-null where it does not
// hold is an error).
bool route_fuses_quant(int dtype, int64_t T, int64_t H, int E);
hipError_t launch_route_topk(const void *x, int dtype, const uint16_t *wg, const float *wg_f32, int64_t T,
                             int64_t H, int E, int k, int renormalize, int32_t *ids, float *w, float *logits,
                             hipStream_t st, int8_t *xq = nullptr, float *sx = nullptr,
                             const uint16_t *wg_packed = nullptr);
// n bf16 values (n % 8 == 0, 16-byte aligned) widened to fp32
hipError_t launch_widen_bf16(const uint16_t *src, int64_t n, float *dst, hipStream_t st);
// router weight [E][H] bf16 -> [H/8][E][8] bf16 (H % 8 == 0, 16-byte aligned)
hipError_t launch_pack_router(const uint16_t *wg, int E, int64_t H, uint16_t *dst, hipStream_t st);

size_t permute_ws_bytes(int64_t T, int k, int E);
// Tile tables the permutation builds for grouped GEMMs (up to four): over its
// E expert groups, plus one extra group of extra_rows rows after them when
// launch_permute's extra_rows > 0; or, with dense_rows > 0, over one group of
// dense_rows rows (a dense linear).
struct TileTableReq {
    int BM, nblocks_n;
    int32_t *prefix;   // [groups + 1]
    int4 *tiles;
    int32_t dense_rows;
};
// extra_rows > 0: also sorted_pair[T*k + t] = t*k for t < extra_rows (an
// extra group that every token visits once, in token order).
hipError_t launch_permute(const int32_t *ids, int64_t T, int k, int E, int32_t *offsets,
                          int32_t *sorted_pair, int32_t *pair_pos, void *ws, hipStream_t st,
                          const TileTableReq *req = nullptr, int nreq = 0, int32_t extra_rows = 0);

size_t gemm_ws_bytes(int64_t M_total, int64_t N, int G);
void gemm_tile_params(int64_t M_total, int64_t N, int G, int epilogue, int *BM, int *nblocks_n);
void *gemm_tiles_ptr(void *ws, int G);
// tile map of a grouped GEMM (into ws), then the GEMM itself reading that map
// (offsets == nullptr: one group of M_total rows, a dense linear)
hipError_t launch_gemm_tilemap(const int32_t *offsets, int G, int64_t M_total, int64_t N, int epilogue, void *ws,
                               hipStream_t st);
// Internal epilogue of the layer's down GEMM (not a public W8A8_EPI_* code):
// the dequantised value v as 16-bit fixed point, out = rint(v * 2^-e) (int16)
// with one exponent e per row and 64-column segment in out_exp
// ([M][ceil(N/64)] int8), e chosen so the segment's largest |v| maps into
// [2^13, 2^14).  Absolute error per element <= 2^-14 of the segment maximum.
constexpr int EPI_FIXED16 = 3;
// B_extra: the last of the G groups takes its weights (one group's worth, the
// same layout) and scales from B_extra / b_extra_scales instead of B, b_scales.
hipError_t launch_gemm_main(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                            int gather_div, const int8_t *B, int b_packed, const float *b_scales,
                            const int32_t *offsets, int G, int64_t M_total, int64_t N, int64_t K, int epilogue,
                            int out_dtype, void *out, const void *ws, hipStream_t st, int8_t *out_exp = nullptr,
                            const int8_t *B_extra = nullptr, const float *b_extra_scales = nullptr);
// The layer's down GEMM (EPI_FIXED16, packed weights) with its A given as the
// bf16 rows of h in grouped order [M_total][K]: each tile quantises its rows
// itself (per-row scale amax / 127, the quantiser's arithmetic) and the tiles
// of column block 0 store the int8 codes [M_total][K] and scales [M_total] to
// a_codes_out / a_scales_out.  Only where gemm_down_fuses_quant holds (tiles
// of 32 rows: few rows per expert, the weight stream bounds the tile); the
// tile table in ws is the one the permutation builds for EPI_FIXED16.
bool gemm_down_fuses_quant(int64_t M_total, int64_t N, int64_t K, int G);
hipError_t launch_gemm_down_qa(const uint16_t *A_h, int64_t M_total, int8_t *a_codes_out, float *a_scales_out,
                               const int8_t *B, const float *b_scales, const int32_t *offsets, int G, int64_t N,
                               int64_t K, void *out, int8_t *out_exp, const void *ws, hipStream_t st,
                               const int8_t *B_extra = nullptr, const float *b_extra_scales = nullptr);
hipError_t launch_grouped_gemm(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                               int gather_div, const int8_t *B, int b_packed, const float *b_scales,
                               const int32_t *offsets, int G, int64_t M_total, int64_t N, int64_t K, int epilogue,
                               int out_dtype, void *out, void *ws, hipStream_t st);
// Dense W8A8 linear on quantised rows: out [M][N] = (xq . W^T) * sx[m] * s[n]
// (packed weights, one group), tiles from the block index (no table).  With
// few tiles K is split into slices whose int32 sums go to `partials`
// (linear_partials_bytes(M, N, K) bytes; 0: no split) and a second kernel adds
// them and dequantises; partials == nullptr never splits.
size_t linear_partials_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear(const int8_t *xq, const float *sx, int64_t M, int64_t K, const int8_t *Bp,
                         const float *b_scales, int64_t N, int out_dtype, void *out, hipStream_t st,
                         int32_t *partials = nullptr);
size_t packed_weights_bytes(int64_t G, int64_t N, int64_t K);
hipError_t launch_pack_weights(const int8_t *B, int64_t G, int64_t N, int64_t K, int8_t *P, hipStream_t st);

// W4A8: packed 4-bit weights (pack_w4_kernel layout) followed by the group
// scales and offsets re-laid step-major ([G][KS][N]); the grouped GEMM with
// per-(column, 128-step) scales and offsets; epilogue 1 (dequant) or 2
// (dequant + SwiGLU).  The tile table comes from gemm_tile_params_w4.
size_t packed_w4_bytes(int64_t G, int64_t N, int64_t K);
hipError_t launch_pack_w4(const int8_t *B, const float *scales, const int8_t *offs, int64_t G, int64_t N, int64_t K,
                          uint8_t *P, hipStream_t st);
void gemm_tile_params_w4(int64_t M_total, int64_t N, int G, int epilogue, int *BM, int *nblocks_n);
hipError_t launch_gemm_w4_main(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                               int gather_div, const uint8_t *Bp, const int32_t *offsets, int G, int64_t M_total,
                               int64_t N, int64_t K, int epilogue, int out_dtype, void *out, const void *ws,
                               hipStream_t st);
hipError_t launch_grouped_gemm_w4(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *gather,
                                  int gather_div, const uint8_t *Bp, const int32_t *offsets, int G, int64_t M_total,
                                  int64_t N, int64_t K, int epilogue, int out_dtype, void *out, void *ws,
                                  hipStream_t st);

hipError_t launch_combine(const void *y, int y_dtype, const float *w, const int32_t *pair_pos, int64_t T,
                          int k, int64_t H, void *out, int out_dtype, hipStream_t st);
// combine of y in the EPI_FIXED16 format: y16 [T*k][H] int16, y_exp [T*k][ceil(H/64)].
// With a shared expert (w_sg non-null): y has T*k + T rows, row T*k + t the
// shared expert's output for token t, added with weight sigmoid(x[t] . w_sg)
// after the routed slots; x [T][H] has out's dtype, gate_out [T] receives the
// sigmoids.
hipError_t launch_combine_fixed16(const int16_t *y16, const int8_t *y_exp, const float *w, const int32_t *pair_pos,
                                  int64_t T, int k, int64_t H, void *out, int out_dtype, hipStream_t st,
                                  const void *x = nullptr, const uint16_t *w_sg = nullptr,
                                  float *gate_out = nullptr);

}  // namespace w8a8
