// C ABI of the W8A8 MoE library: argument checks, workspace layout and the
// launch sequence of the layer.  Every entry point validates its arguments
// completely before the first launch; nothing here synchronises the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/w8a8moe.h"
#include "launch.h"

using namespace w8a8;

// Scratch memory of the allocation-free grouped GEMM (its tile table): a
// fixed array in every GPU's memory, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it names a stand-in,
// not device memory): it uses the device address that hipGetSymbolAddress
// returns, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[W8A8_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mutex;
void *scratch_addr[SCRATCH_MAX_DEVICES];   // per device, filled on its first use

// The current device's copy of `scratch`.
hipError_t scratch_of_current_device(void **addr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_addr[dev] = p;
    }
    *addr = scratch_addr[dev];
    return hipSuccess;
}
}  // namespace

namespace {

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool act_dtype_ok(int d) { return d == W8A8_BF16 || d == W8A8_F32; }
inline size_t elem_size(int d) { return d == W8A8_BF16 ? 2 : 4; }
inline size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return W8A8_OK;
    (void)hipGetLastError();
    return W8A8_ERR_HIP;
}

int check_route(const void *x, int x_dtype, const uint16_t *w_gate, int64_t T, int64_t H, int E, int k,
                const int32_t *ids, const float *w, const float *logits)
{
    if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E || !act_dtype_ok(x_dtype)) return W8A8_ERR_INVALID_ARG;
    if (E > 256) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (H % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    // activations and router rows are addressed with 32-bit byte offsets
    if (T * H * 4 > INT32_MAX - 256 || (int64_t)E * H * 2 > INT32_MAX - 256) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (T > 0 && (!x || !w_gate || !ids || !w)) return W8A8_ERR_INVALID_ARG;
    if (T > 0 && (!aligned16(x) || !aligned16(w_gate) || !aligned16(ids) || !aligned16(w) ||
                  (logits && !aligned16(logits))))
        return W8A8_ERR_ALIGNMENT;
    return W8A8_OK;
}

// Arguments of a grouped GEMM, everything but its workspace.
int check_grouped_gemm(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *a_row_gather,
                       int gather_div, const int8_t *B, int b_layout, const float *b_scales,
                       const int32_t *group_offsets, int G, int64_t M_total, int64_t N, int64_t K, int epilogue,
                       int out_dtype, const void *out)
{
    if (M_total < 0 || A_rows < 0 || N <= 0 || K <= 0 || G <= 0) return W8A8_ERR_INVALID_ARG;
    if (G > 4096) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (b_layout != W8A8_B_ROWMAJOR && b_layout != W8A8_B_PACKED) return W8A8_ERR_INVALID_ARG;
    if (epilogue < W8A8_EPI_RAW_I32 || epilogue > W8A8_EPI_DEQUANT_SWIGLU) return W8A8_ERR_INVALID_ARG;
    if (epilogue == W8A8_EPI_RAW_I32 ? out_dtype != W8A8_I32 : !act_dtype_ok(out_dtype))
        return W8A8_ERR_INVALID_ARG;
    if (a_row_gather && gather_div <= 0) return W8A8_ERR_INVALID_ARG;
    if (K % 16 || N % 16 || (epilogue == W8A8_EPI_DEQUANT_SWIGLU && N % 64)) return W8A8_ERR_UNSUPPORTED_SHAPE;
    const int64_t group_bytes = b_layout == W8A8_B_PACKED ? (int64_t)packed_weights_bytes(1, N, K) : N * K;
    if (A_rows * K > INT32_MAX - 256 || group_bytes > INT32_MAX - 256) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (!B || !group_offsets) return W8A8_ERR_INVALID_ARG;
    if (M_total > 0 && (!A || !out)) return W8A8_ERR_INVALID_ARG;
    if (epilogue != W8A8_EPI_RAW_I32 && (!b_scales || (M_total > 0 && !a_scales))) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(A) || !aligned16(B) || !aligned16(out) || !aligned16(group_offsets) ||
        (a_row_gather && !aligned16(a_row_gather)) || (a_scales && !aligned16(a_scales)) ||
        (b_scales && !aligned16(b_scales)))
        return W8A8_ERR_ALIGNMENT;
    return W8A8_OK;
}

// Layer workspace layout (every part 256-byte aligned).
struct LayerWs {
    size_t ids, w, xq, sx, offsets, sorted, pos, h, hq, sh, y, yexp, perm, gemm1, gemm2;
    size_t hs, hqs, shs, sgate, gemm3, gemm4;   // shared expert (zero-sized without one)
    size_t total;
};

inline bool has_shared(const w8a8_moe_weights *W) { return W->I_shared > 0; }
// A shared expert as wide as the routed ones, with int8 gate_up weights, runs
// as one extra group of the routed grouped GEMMs (rows P .. P+T of the
// grouped order, each token once); otherwise as GEMMs of its own.
inline bool shared_in_groups(const w8a8_moe_weights *W)
{
    return has_shared(W) && W->I_shared == W->I && W->w4_gate_up == nullptr;
}

LayerWs layer_ws(const w8a8_moe_weights *W, int64_t T, int x_dtype)
{
    const int64_t P = T * W->k;
    LayerWs L;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o += round256(bytes);
        return at;
    };
    L.ids = take(sizeof(int32_t) * P);
    L.w = take(sizeof(float) * P);
    L.xq = take((size_t)(T * W->H));
    L.sx = take(sizeof(float) * T);
    // a shared expert's rows follow the P routed ones: in the grouped rows
    // (sorted_pair, h, hq, sh) when it runs as an extra group, and in y always
    const int64_t Ts = has_shared(W) ? T : 0, Is = has_shared(W) ? W->I_shared : 0;
    const int64_t Tg = shared_in_groups(W) ? T : 0;   // extra grouped rows
    const int Gx = shared_in_groups(W) ? 1 : 0;
    L.offsets = take(sizeof(int32_t) * (W->E + 1));
    L.sorted = take(sizeof(int32_t) * (P + Tg));
    L.pos = take(sizeof(int32_t) * P);
    L.h = take(2 * (size_t)((P + Tg) * W->I));
    L.hq = take((size_t)((P + Tg) * W->I));
    L.sh = take(sizeof(float) * (P + Tg));
    // y: 16-bit fixed point with a power-of-two exponent per row and 64 columns
    L.y = take(sizeof(int16_t) * (size_t)((P + Ts) * W->H));
    L.yexp = take((size_t)((P + Ts) * ((W->H + 63) / 64)));
    L.perm = take(permute_ws_bytes(T, W->k, W->E));
    L.gemm1 = take(gemm_ws_bytes(P + Tg, 2 * W->I, W->E + Gx));
    L.gemm2 = take(gemm_ws_bytes(P + Tg, W->H, W->E + Gx));
    if (Gx) {   // the shared expert's h, codes and scales are the extra group's rows
        L.hs = L.h + 2 * (size_t)(P * W->I);
        L.hqs = L.hq + (size_t)(P * W->I);
        L.shs = L.sh + sizeof(float) * P;
    } else {
        L.hs = take(2 * (size_t)(Ts * Is));
        L.hqs = take((size_t)(Ts * Is));
        L.shs = take(sizeof(float) * (size_t)Ts);
    }
    L.sgate = take(sizeof(float) * (size_t)Ts);
    L.gemm3 = Ts && !Gx ? take(gemm_ws_bytes(Ts, 2 * Is, 1)) : o;
    L.gemm4 = Ts && !Gx ? take(gemm_ws_bytes(Ts, W->H, 1)) : o;
    L.total = o;
    return L;
}

int check_layer(const w8a8_moe_weights *W, const void *x, int x_dtype, int64_t T, const void *out)
{
    if (!W || T < 0 || !act_dtype_ok(x_dtype)) return W8A8_ERR_INVALID_ARG;
    if (W->E <= 0 || W->k <= 0 || W->k > W->E || W->H <= 0 || W->I <= 0) return W8A8_ERR_INVALID_ARG;
    if (W->E > 256 || W->H % 16 || W->I % 32) return W8A8_ERR_UNSUPPORTED_SHAPE;
    // the grouped GEMMs address one expert's weights and the activation codes
    // with 32-bit byte offsets
    if ((int64_t)packed_weights_bytes(1, 2 * W->I, W->H) > INT32_MAX - 256 ||
        (int64_t)packed_weights_bytes(1, W->H, W->I) > INT32_MAX - 256 || T * W->k * W->I > INT32_MAX - 256 ||
        T * W->H > INT32_MAX - 256)
        return W8A8_ERR_UNSUPPORTED_SHAPE;
    // the router kernels the layer launches address the token rows (up to fp32
    // wide) and the router weight (bf16, or its fp32 copy) the same way: the
    // bounds of moe_route_topk
    if (T * W->H * 4 > INT32_MAX - 256 || (int64_t)W->E * W->H * (W->w_gate_f32 ? 4 : 2) > INT32_MAX - 256)
        return W8A8_ERR_UNSUPPORTED_SHAPE;
    const bool w4 = W->w4_gate_up != nullptr;
    if (w4 && ((int64_t)packed_w4_bytes(1, 2 * W->I, W->H) > INT32_MAX - 256 ||
               2 * W->I * ((W->H + 127) / 128) * 4 > INT32_MAX - 256))
        return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (!W->w_gate || !W->w_down || !W->s_down) return W8A8_ERR_INVALID_ARG;
    if (!w4 && (!W->w_gate_up || !W->s_gate_up)) return W8A8_ERR_INVALID_ARG;
    if (T > 0 && (!x || !out)) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(W->w_gate) || !aligned16(W->w_down) || !aligned16(W->s_down) ||
        (W->w_gate_f32 && !aligned16(W->w_gate_f32)) || (W->w_gate_packed && !aligned16(W->w_gate_packed)))
        return W8A8_ERR_ALIGNMENT;
    if (w4 ? !aligned16(W->w4_gate_up) : (!aligned16(W->w_gate_up) || !aligned16(W->s_gate_up)))
        return W8A8_ERR_ALIGNMENT;
    if (T > 0 && (!aligned16(x) || !aligned16(out))) return W8A8_ERR_ALIGNMENT;
    // shared expert: all of its weights, or none
    const bool any_shared = W->I_shared != 0 || W->w_shared_gate_up || W->s_shared_gate_up || W->w_shared_down ||
                            W->s_shared_down || W->w_shared_gate;
    if (any_shared) {
        if (W->I_shared <= 0 || !W->w_shared_gate_up || !W->s_shared_gate_up || !W->w_shared_down ||
            !W->s_shared_down || !W->w_shared_gate)
            return W8A8_ERR_INVALID_ARG;
        if (W->I_shared % 32 || w4) return W8A8_ERR_UNSUPPORTED_SHAPE;   // with W4A8 routed weights: not built
        if ((int64_t)packed_weights_bytes(1, 2 * W->I_shared, W->H) > INT32_MAX - 256 ||
            (int64_t)packed_weights_bytes(1, W->H, W->I_shared) > INT32_MAX - 256 ||
            T * W->I_shared > INT32_MAX - 256)
            return W8A8_ERR_UNSUPPORTED_SHAPE;
        if (!aligned16(W->w_shared_gate_up) || !aligned16(W->s_shared_gate_up) || !aligned16(W->w_shared_down) ||
            !aligned16(W->s_shared_down) || !aligned16(W->w_shared_gate))
            return W8A8_ERR_ALIGNMENT;
    }
    return W8A8_OK;
}

int run_layer(const w8a8_moe_weights *W, const void *x, int x_dtype, int64_t T, void *out, void *ws,
              size_t ws_bytes, hipStream_t st, void *const *events, int n_events)
{
    int rc = check_layer(W, x, x_dtype, T, out);
    if (rc) return rc;
    if (n_events < 0 || n_events > W8A8_LAYER_STAGES + 1 || (n_events > 0 && !events)) return W8A8_ERR_INVALID_ARG;
    if (T == 0) return W8A8_OK;
    const LayerWs L = layer_ws(W, T, x_dtype);
    if (!ws) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(ws)) return W8A8_ERR_ALIGNMENT;
    if (ws_bytes < L.total) return W8A8_ERR_WORKSPACE_TOO_SMALL;

    char *base = (char *)ws;
    int32_t *ids = (int32_t *)(base + L.ids);
    float *w = (float *)(base + L.w);
    int8_t *xq = (int8_t *)(base + L.xq);
    float *sx = (float *)(base + L.sx);
    int32_t *offsets = (int32_t *)(base + L.offsets);
    int32_t *sorted = (int32_t *)(base + L.sorted);
    int32_t *pos = (int32_t *)(base + L.pos);
    uint16_t *h = (uint16_t *)(base + L.h);
    int8_t *hq = (int8_t *)(base + L.hq);
    float *sh = (float *)(base + L.sh);
    int16_t *y = (int16_t *)(base + L.y);
    int8_t *yexp = (int8_t *)(base + L.yexp);
    void *perm = base + L.perm;
    void *gws1 = base + L.gemm1;
    void *gws2 = base + L.gemm2;
    const int64_t P = T * W->k;
    const int E = W->E, k = W->k;
    const int64_t H = W->H, I = W->I;
    const bool shared = has_shared(W);
    const int64_t Is = W->I_shared;
    uint16_t *hs = (uint16_t *)(base + L.hs);
    int8_t *hqs = (int8_t *)(base + L.hqs);
    float *shs = (float *)(base + L.shs);
    float *sgate = (float *)(base + L.sgate);
    void *gws3 = base + L.gemm3;
    void *gws4 = base + L.gemm4;

    int ev = 0;
    auto mark = [&]() -> hipError_t {
        if (ev >= n_events) return hipSuccess;
        void *h = events[ev++];
        return h ? hipEventRecord((hipEvent_t)h, st) : hipSuccess;   // a null entry skips the mark
    };
    hipError_t e;
    if ((e = mark()) != hipSuccess) return hip_status(e);
    // 1 route; with bf16 tokens the router also quantises them (stage 2 is then empty)
    const bool fused_q = route_fuses_quant(x_dtype, T, H, E);
    if ((e = launch_route_topk(x, x_dtype, W->w_gate, W->w_gate_f32, T, H, E, k, 1, ids, w, nullptr, st,
                               fused_q ? xq : nullptr, fused_q ? sx : nullptr, W->w_gate_packed)) != hipSuccess ||
        (e = mark()) != hipSuccess)
        return hip_status(e);
    // 2 quantise x once per token (before the permutation: one scale per token
    //   serves all k experts)
    if ((!fused_q && (e = launch_quant_rows(x, x_dtype, T, H, H, xq, sx, st)) != hipSuccess) ||
        (e = mark()) != hipSuccess)
        return hip_status(e);
    // 3 permute; its scan also builds the tile tables of the grouped GEMMs
    //   (over E groups, or E + 1 with the shared expert as the extra group;
    //   one-group tables for a shared expert with GEMMs of its own)
    const bool w4 = W->w4_gate_up != nullptr;
    const bool sg = shared_in_groups(W);
    const int Gg = sg ? E + 1 : E;         // groups of the grouped GEMMs
    const int64_t Pg = sg ? P + T : P;     // their rows
    TileTableReq req[4] = {};
    if (w4) gemm_tile_params_w4(Pg, 2 * I, Gg, W8A8_EPI_DEQUANT_SWIGLU, &req[0].BM, &req[0].nblocks_n);
    else gemm_tile_params(Pg, 2 * I, Gg, W8A8_EPI_DEQUANT_SWIGLU, &req[0].BM, &req[0].nblocks_n);
    gemm_tile_params(Pg, H, Gg, EPI_FIXED16, &req[1].BM, &req[1].nblocks_n);
    req[0].prefix = (int32_t *)gws1;
    req[0].tiles = (int4 *)gemm_tiles_ptr(gws1, Gg);
    req[1].prefix = (int32_t *)gws2;
    req[1].tiles = (int4 *)gemm_tiles_ptr(gws2, Gg);
    int nreq = 2;
    if (shared && !sg) {
        gemm_tile_params(T, 2 * Is, 1, W8A8_EPI_DEQUANT_SWIGLU, &req[2].BM, &req[2].nblocks_n);
        gemm_tile_params(T, H, 1, EPI_FIXED16, &req[3].BM, &req[3].nblocks_n);
        req[2].prefix = (int32_t *)gws3;
        req[2].tiles = (int4 *)gemm_tiles_ptr(gws3, 1);
        req[3].prefix = (int32_t *)gws4;
        req[3].tiles = (int4 *)gemm_tiles_ptr(gws4, 1);
        req[2].dense_rows = req[3].dense_rows = (int32_t)T;
        nreq = 4;
    }
    if ((e = launch_permute(ids, T, k, E, offsets, sorted, pos, perm, st, req, nreq, sg ? (int32_t)T : 0)) !=
            hipSuccess ||
        (e = mark()) != hipSuccess)
        return hip_status(e);
    // 4a gate_up GEMM + SwiGLU -> h (bf16), W8A8 or W4A8 weights
    e = w4 ? launch_gemm_w4_main(xq, T, sx, sorted, k, W->w4_gate_up, offsets, E, P, 2 * I, H,
                                 W8A8_EPI_DEQUANT_SWIGLU, W8A8_BF16, h, gws1, st)
           : launch_gemm_main(xq, T, sx, sorted, k, W->w_gate_up, 1, W->s_gate_up, offsets, Gg, Pg, 2 * I, H,
                              W8A8_EPI_DEQUANT_SWIGLU, W8A8_BF16, h, gws1, st, nullptr,
                              sg ? W->w_shared_gate_up : nullptr, sg ? W->s_shared_gate_up : nullptr);
    if (e != hipSuccess) return hip_status(e);
    // a shared expert with GEMMs of its own, on every token's codes (no gather)
    if (shared && !sg &&
        (e = launch_gemm_main(xq, T, sx, nullptr, 1, W->w_shared_gate_up, 1, W->s_shared_gate_up, nullptr, 1, T,
                              2 * Is, H, W8A8_EPI_DEQUANT_SWIGLU, W8A8_BF16, hs, gws3, st)) != hipSuccess)
        return hip_status(e);
    if ((e = mark()) != hipSuccess) return hip_status(e);
    // quantise h per grouped row (and a separate shared expert's h per token);
    // with few rows per expert the down GEMM's tiles quantise their own rows
    // (and still store hq and sh), so the pass is skipped
    const bool down_qa = gemm_down_fuses_quant(Pg, H, I, Gg);
    if ((!down_qa && (e = launch_quant_rows(h, W8A8_BF16, Pg, I, I, hq, sh, st)) != hipSuccess) ||
        (shared && !sg && (e = launch_quant_rows(hs, W8A8_BF16, T, Is, Is, hqs, shs, st)) != hipSuccess) ||
        (e = mark()) != hipSuccess)
        return hip_status(e);
    // 4b down GEMM -> y (16-bit fixed point + exponents); the shared expert's
    //    rows follow the routed ones
    const int64_t nseg = (H + 63) / 64;
    e = down_qa ? launch_gemm_down_qa(h, Pg, hq, sh, W->w_down, W->s_down, offsets, Gg, H, I, y, yexp, gws2, st,
                                      sg ? W->w_shared_down : nullptr, sg ? W->s_shared_down : nullptr)
                : launch_gemm_main(hq, Pg, sh, nullptr, 1, W->w_down, 1, W->s_down, offsets, Gg, Pg, H, I, EPI_FIXED16,
                                   W8A8_F32, y, gws2, st, yexp, sg ? W->w_shared_down : nullptr,
                                   sg ? W->s_shared_down : nullptr);
    if (e != hipSuccess ||
        (shared && !sg &&
         (e = launch_gemm_main(hqs, T, shs, nullptr, 1, W->w_shared_down, 1, W->s_shared_down, nullptr, 1, T, H, Is,
                               EPI_FIXED16, W8A8_F32, y + P * H, gws4, st, yexp + P * nseg)) != hipSuccess) ||
        (e = mark()) != hipSuccess)
        return hip_status(e);
    // 5 combine (with the shared expert's gated output)
    if ((e = launch_combine_fixed16(y, yexp, w, pos, T, k, H, out, x_dtype, st, shared ? x : nullptr,
                                    shared ? W->w_shared_gate : nullptr, shared ? sgate : nullptr)) != hipSuccess ||
        (e = mark()) != hipSuccess)
        return hip_status(e);
    return W8A8_OK;
}

}  // namespace

extern "C" {

const char *w8a8_status_string(int status)
{
    switch (status) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_INVALID_ARG: return "invalid argument";
    case W8A8_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case W8A8_ERR_ALIGNMENT: return "pointer or leading dimension not 16-byte aligned";
    case W8A8_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case W8A8_ERR_HIP: return "HIP launch failed";
    case W8A8_ERR_SCRATCH_LIMIT: return "problem needs more scratch than the fixed buffer of the allocation-free entry point";
    default: return "unknown status";
    }
}

int w8a8_quant_act(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, int8_t *q, float *scales,
                   void *stream)
{
    if (rows < 0 || cols <= 0 || ld_x < cols || !act_dtype_ok(x_dtype)) return W8A8_ERR_INVALID_ARG;
    if (cols % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (rows == 0) return W8A8_OK;
    if (!x || !q || !scales) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || ((size_t)ld_x * elem_size(x_dtype)) % 16) return W8A8_ERR_ALIGNMENT;
    return hip_status(launch_quant_rows(x, x_dtype, rows, cols, ld_x, q, scales, (hipStream_t)stream));
}

int moe_route_topk(const void *x, int x_dtype, const uint16_t *w_gate, int64_t T, int64_t H, int E, int k,
                   int renormalize, int32_t *topk_ids, float *topk_w, float *logits_out, void *stream)
{
    int rc = check_route(x, x_dtype, w_gate, T, H, E, k, topk_ids, topk_w, logits_out);
    if (rc) return rc;
    if (T == 0) return W8A8_OK;
    return hip_status(launch_route_topk(x, x_dtype, w_gate, nullptr, T, H, E, k, renormalize, topk_ids, topk_w,
                                        logits_out,
                                        (hipStream_t)stream));
}

int moe_route_topk_packed(const void *x, int x_dtype, const uint16_t *w_gate, const uint16_t *w_gate_packed,
                          int64_t T, int64_t H, int E, int k, int renormalize, int32_t *topk_ids, float *topk_w,
                          float *logits_out, void *stream)
{
    int rc = check_route(x, x_dtype, w_gate, T, H, E, k, topk_ids, topk_w, logits_out);
    if (rc) return rc;
    if (w_gate_packed && !aligned16(w_gate_packed)) return W8A8_ERR_ALIGNMENT;
    if (T == 0) return W8A8_OK;
    return hip_status(launch_route_topk(x, x_dtype, w_gate, nullptr, T, H, E, k, renormalize, topk_ids, topk_w,
                                        logits_out, (hipStream_t)stream, nullptr, nullptr, w_gate_packed));
}

int moe_router_widen(const uint16_t *w_gate, int E, int64_t H, float *w_gate_f32, void *stream)
{
    if (E <= 0 || H <= 0 || !w_gate || !w_gate_f32) return W8A8_ERR_INVALID_ARG;
    if (H % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(w_gate) || !aligned16(w_gate_f32)) return W8A8_ERR_ALIGNMENT;
    return hip_status(launch_widen_bf16(w_gate, (int64_t)E * H, w_gate_f32, (hipStream_t)stream));
}

int moe_router_pack(const uint16_t *w_gate, int E, int64_t H, uint16_t *w_gate_packed, void *stream)
{
    if (E <= 0 || H <= 0 || !w_gate || !w_gate_packed) return W8A8_ERR_INVALID_ARG;
    if (H % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(w_gate) || !aligned16(w_gate_packed)) return W8A8_ERR_ALIGNMENT;
    return hip_status(launch_pack_router(w_gate, E, H, w_gate_packed, (hipStream_t)stream));
}

size_t moe_permute_workspace_size(int64_t T, int k, int E)
{
    if (T < 0 || k <= 0 || E <= 0) return 0;
    return round256(permute_ws_bytes(T, k, E));
}

int moe_permute(const int32_t *topk_ids, int64_t T, int k, int E, int32_t *offsets, int32_t *sorted_pair,
                int32_t *pair_pos, void *ws, size_t ws_bytes, void *stream)
{
    if (T < 0 || k <= 0 || E <= 0 || k > E) return W8A8_ERR_INVALID_ARG;
    if (E > 256) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (!offsets) return W8A8_ERR_INVALID_ARG;
    if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos || !ws)) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(offsets) || (T > 0 && (!aligned16(topk_ids) || !aligned16(sorted_pair) || !aligned16(pair_pos) ||
                                          !aligned16(ws))))
        return W8A8_ERR_ALIGNMENT;
    if (ws_bytes < permute_ws_bytes(T, k, E)) return W8A8_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(
        launch_permute(topk_ids, T, k, E, offsets, sorted_pair, pair_pos, ws, (hipStream_t)stream));
}

size_t w8a8_packed_weights_size(int G, int64_t N, int64_t K)
{
    if (G <= 0 || N <= 0 || K <= 0) return 0;
    return packed_weights_bytes(G, N, K);
}

int w8a8_pack_weights(const int8_t *B, int G, int64_t N, int64_t K, int8_t *packed, void *stream)
{
    if (G <= 0 || N <= 0 || K <= 0 || !B || !packed) return W8A8_ERR_INVALID_ARG;
    if (N % 16 || K % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(B) || !aligned16(packed)) return W8A8_ERR_ALIGNMENT;
    return hip_status(launch_pack_weights(B, G, N, K, packed, (hipStream_t)stream));
}

size_t w8a8_grouped_gemm_workspace_size(int64_t M_total, int64_t N, int G)
{
    if (M_total < 0 || N <= 0 || G <= 0) return 0;
    return gemm_ws_bytes(M_total, N, G);
}

int w8a8_grouped_gemm(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *a_row_gather,
                      int gather_div, const int8_t *B, int b_layout, const float *b_scales,
                      const int32_t *group_offsets, int G, int64_t M_total, int64_t N, int64_t K, int epilogue,
                      int out_dtype, void *out, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_grouped_gemm(A, A_rows, a_scales, a_row_gather, gather_div, B, b_layout, b_scales, group_offsets,
                                G, M_total, N, K, epilogue, out_dtype, out);
    if (rc) return rc;
    if (!ws) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(ws)) return W8A8_ERR_ALIGNMENT;
    if (ws_bytes < gemm_ws_bytes(M_total, N, G)) return W8A8_ERR_WORKSPACE_TOO_SMALL;
    if (M_total == 0) return W8A8_OK;
    return hip_status(launch_grouped_gemm(A, A_rows, a_scales, a_row_gather, gather_div, B, b_layout, b_scales,
                                          group_offsets, G, M_total, N, K, epilogue, out_dtype, out, ws,
                                          (hipStream_t)stream));
}

int w8a8_grouped_gemm_noalloc(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *a_row_gather,
                              int gather_div, const int8_t *B, int b_layout, const float *b_scales,
                              const int32_t *group_offsets, int G, int64_t M_total, int64_t N, int64_t K,
                              int epilogue, int out_dtype, void *out, void *stream)
{
    int rc = check_grouped_gemm(A, A_rows, a_scales, a_row_gather, gather_div, B, b_layout, b_scales, group_offsets,
                                G, M_total, N, K, epilogue, out_dtype, out);
    if (rc) return rc;
    if (gemm_ws_bytes(M_total, N, G) > (size_t)W8A8_NOALLOC_SCRATCH_BYTES) return W8A8_ERR_SCRATCH_LIMIT;
    if (M_total == 0) return W8A8_OK;
    void *table = nullptr;
    hipError_t e = scratch_of_current_device(&table);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_grouped_gemm(A, A_rows, a_scales, a_row_gather, gather_div, B, b_layout, b_scales,
                                          group_offsets, G, M_total, N, K, epilogue, out_dtype, out, table,
                                          (hipStream_t)stream));
}

int w4a8_quant_weights(const float *w, int64_t rows, int64_t cols, int8_t *q, float *scales, int8_t *offsets,
                       void *stream)
{
    if (rows < 0 || cols <= 0) return W8A8_ERR_INVALID_ARG;
    if (cols % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (rows == 0) return W8A8_OK;
    if (!w || !q || !scales || !offsets) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(q) || ((uintptr_t)scales & 3u)) return W8A8_ERR_ALIGNMENT;
    return hip_status(launch_quant_w4(w, rows, cols, q, scales, offsets, (hipStream_t)stream));
}

size_t w4a8_packed_weights_size(int G, int64_t N, int64_t K)
{
    if (G <= 0 || N <= 0 || K <= 0) return 0;
    return packed_w4_bytes(G, N, K);
}

int w4a8_pack_weights(const int8_t *q, const float *scales, const int8_t *offsets, int G, int64_t N, int64_t K,
                      uint8_t *packed, void *stream)
{
    if (G <= 0 || N <= 0 || K <= 0 || !q || !scales || !offsets || !packed) return W8A8_ERR_INVALID_ARG;
    if (N % 16 || K % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(q) || !aligned16(packed) || ((uintptr_t)scales & 3u)) return W8A8_ERR_ALIGNMENT;
    return hip_status(launch_pack_w4(q, scales, offsets, G, N, K, packed, (hipStream_t)stream));
}

int w4a8_grouped_gemm(const int8_t *A, int64_t A_rows, const float *a_scales, const int32_t *a_row_gather,
                      int gather_div, const uint8_t *B_packed, const int32_t *group_offsets, int G, int64_t M_total,
                      int64_t N, int64_t K, int epilogue, int out_dtype, void *out, void *ws, size_t ws_bytes,
                      void *stream)
{
    if (M_total < 0 || A_rows < 0 || N <= 0 || K <= 0 || G <= 0) return W8A8_ERR_INVALID_ARG;
    if (G > 4096) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (epilogue != W8A8_EPI_DEQUANT && epilogue != W8A8_EPI_DEQUANT_SWIGLU) return W8A8_ERR_INVALID_ARG;
    if (!act_dtype_ok(out_dtype)) return W8A8_ERR_INVALID_ARG;
    if (a_row_gather && gather_div <= 0) return W8A8_ERR_INVALID_ARG;
    if (K % 16 || N % 16 || (epilogue == W8A8_EPI_DEQUANT_SWIGLU && N % 64)) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (A_rows * K > INT32_MAX - 256 || (int64_t)packed_w4_bytes(1, N, K) > INT32_MAX - 256 ||
        N * ((K + 127) / 128) * 4 > INT32_MAX - 256)
        return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (!B_packed || !group_offsets || !ws) return W8A8_ERR_INVALID_ARG;
    if (M_total > 0 && (!A || !out || !a_scales)) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(A) || !aligned16(B_packed) || !aligned16(out) || !aligned16(ws) || !aligned16(group_offsets) ||
        (a_row_gather && !aligned16(a_row_gather)) || !aligned16(a_scales))
        return W8A8_ERR_ALIGNMENT;
    if (ws_bytes < gemm_ws_bytes(M_total, N, G)) return W8A8_ERR_WORKSPACE_TOO_SMALL;
    if (M_total == 0) return W8A8_OK;
    return hip_status(launch_grouped_gemm_w4(A, A_rows, a_scales, a_row_gather, gather_div, B_packed, group_offsets,
                                             G, M_total, N, K, epilogue, out_dtype, out, ws, (hipStream_t)stream));
}

static int check_linear(int64_t M, int64_t K, int64_t N, const int8_t *w_packed, const float *w_scales, const void *out,
                        int out_dtype)
{
    if (M < 0 || K <= 0 || N <= 0 || !act_dtype_ok(out_dtype)) return W8A8_ERR_INVALID_ARG;
    if (K % 16 || N % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (M * K > INT32_MAX - 256 || (int64_t)packed_weights_bytes(1, N, K) > INT32_MAX - 256 || M > INT32_MAX / 2)
        return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (M > 0 && (!w_packed || !w_scales || !out)) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && (!aligned16(w_packed) || !aligned16(w_scales) || !aligned16(out))) return W8A8_ERR_ALIGNMENT;
    return W8A8_OK;
}

static bool linear_sizes_ok(int64_t M, int64_t N, int64_t K) { return M >= 0 && N > 0 && K > 0; }

size_t w8a8_linear_q_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (!linear_sizes_ok(M, N, K)) return 0;
    return round256(linear_partials_bytes(M, N, K));
}

size_t w8a8_linear_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (!linear_sizes_ok(M, N, K)) return 0;
    return round256((size_t)(M * K)) + round256(sizeof(float) * (size_t)M) + w8a8_linear_q_workspace_size(M, N, K);
}

int w8a8_linear(const void *x, int x_dtype, int64_t M, int64_t K, const int8_t *w_packed, const float *w_scales,
                int64_t N, void *out, int out_dtype, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_linear(M, K, N, w_packed, w_scales, out, out_dtype);
    if (rc) return rc;
    if (!act_dtype_ok(x_dtype)) return W8A8_ERR_INVALID_ARG;
    if (M == 0) return W8A8_OK;
    if (!x || !ws) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(ws)) return W8A8_ERR_ALIGNMENT;
    if (ws_bytes < w8a8_linear_workspace_size(M, N, K)) return W8A8_ERR_WORKSPACE_TOO_SMALL;
    int8_t *xq = (int8_t *)ws;
    float *sx = (float *)((char *)ws + round256((size_t)(M * K)));
    int32_t *part = (int32_t *)((char *)sx + round256(sizeof(float) * (size_t)M));
    hipError_t e = launch_quant_rows(x, x_dtype, M, K, K, xq, sx, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_linear(xq, sx, M, K, w_packed, w_scales, N, out_dtype, out, (hipStream_t)stream,
                                    linear_partials_bytes(M, N, K) ? part : nullptr));
}

int w8a8_linear_q(const int8_t *xq, const float *x_scales, int64_t M, int64_t K, const int8_t *w_packed,
                  const float *w_scales, int64_t N, void *out, int out_dtype, void *ws, size_t ws_bytes,
                  void *stream)
{
    int rc = check_linear(M, K, N, w_packed, w_scales, out, out_dtype);
    if (rc) return rc;
    if (M == 0) return W8A8_OK;
    if (!xq || !x_scales) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(x_scales) || (ws && !aligned16(ws))) return W8A8_ERR_ALIGNMENT;
    const size_t need = linear_partials_bytes(M, N, K);
    if (ws && ws_bytes < need) return W8A8_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(launch_linear(xq, x_scales, M, K, w_packed, w_scales, N, out_dtype, out, (hipStream_t)stream,
                                    ws && need ? (int32_t *)ws : nullptr));
}

int moe_combine(const void *y, int y_dtype, const float *topk_w, const int32_t *pair_pos, int64_t T, int k, int64_t H,
                void *out, int out_dtype, void *stream)
{
    if (T < 0 || k <= 0 || H <= 0 || !act_dtype_ok(y_dtype) || !act_dtype_ok(out_dtype)) return W8A8_ERR_INVALID_ARG;
    if (H % 16) return W8A8_ERR_UNSUPPORTED_SHAPE;
    if (T == 0) return W8A8_OK;
    if (!y || !topk_w || !pair_pos || !out) return W8A8_ERR_INVALID_ARG;
    if (!aligned16(y) || !aligned16(topk_w) || !aligned16(pair_pos) || !aligned16(out)) return W8A8_ERR_ALIGNMENT;
    return hip_status(launch_combine(y, y_dtype, topk_w, pair_pos, T, k, H, out, out_dtype, (hipStream_t)stream));
}

size_t w8a8_moe_layer_workspace_size(const w8a8_moe_weights *W, int64_t T, int x_dtype)
{
    if (!W || T < 0 || !act_dtype_ok(x_dtype) || W->E <= 0 || W->k <= 0 || W->H <= 0 || W->I <= 0) return 0;
    return layer_ws(W, T, x_dtype).total;
}

int w8a8_moe_layer(const w8a8_moe_weights *W, const void *x, int x_dtype, int64_t T, void *out, void *ws,
                   size_t ws_bytes, void *stream)
{
    return run_layer(W, x, x_dtype, T, out, ws, ws_bytes, (hipStream_t)stream, nullptr, 0);
}

int w8a8_moe_layer_events(const w8a8_moe_weights *W, const void *x, int x_dtype, int64_t T, void *out, void *ws,
                          size_t ws_bytes, void *stream, void *const *events, int n_events)
{
    return run_layer(W, x, x_dtype, T, out, ws, ws_bytes, (hipStream_t)stream, events, n_events);
}

int w8a8_moe_layer_intermediates(const w8a8_moe_weights *W, int64_t T, int x_dtype, void *ws, void **ptrs)
{
    if (!W || !ws || !ptrs || T < 0 || !act_dtype_ok(x_dtype)) return W8A8_ERR_INVALID_ARG;
    const LayerWs L = layer_ws(W, T, x_dtype);
    char *b = (char *)ws;
    const size_t offs[W8A8_LAYER_INTERMEDIATES] = {L.ids, L.w,  L.xq, L.sx,   L.offsets, L.sorted, L.pos, L.h,
                                                   L.hq,  L.sh, L.y,  L.yexp, L.hs,      L.hqs,    L.shs, L.sgate};
    for (int i = 0; i < W8A8_LAYER_INTERMEDIATES; ++i) ptrs[i] = b + offs[i];
    return W8A8_OK;
}

}  // extern "C"
