// MoE router: unquantised bf16 gate -> fp32 scores -> top-k -> softmax weights
// ("Qwen3-30B-A3B-Instruct-2507-quantized.w8a8" explainer, sections 3.1-3.3:
// the gate maps the hidden state to one score per expert, softmax, top-8; it
// stays in bf16 because a swapped ranking is a discrete error).
//
// Scores: the hidden index is cut into chunks of RT_CHUNK = 512; each chunk is
// an fp32 fused multiply-add chain over its indices, ascending, from +0, and
// the chunk sums are added in ascending chunk order.  The order is fixed so
// that every implementation that follows it produces bit-identical scores,
// and therefore identical expert ids; the chunks let several waves share one
// score when there are few tokens.
//
// Two kernels compute the same chains: route_mfma_kernel for bf16 x (matrix
// cores, below) and route_topk_kernel for fp32 x (vector FMA: a bf16 x fp32
// product is not exact in fp32, so only a true fused multiply-add reproduces
// the chain).  In the vector kernel a block holds 16 tokens x all E (<= 256)
// experts; thread (wave w, lane l) owns tokens 4w..4w+3 and experts l, l+64,
// l+128, l+192, with x and W_g staged through LDS in 32-wide slices of the
// hidden dimension.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "quant_common.h"

namespace w8a8 {

namespace {
constexpr int RT_TOK = 16;   // tokens per block
constexpr int RT_KC = 32;    // hidden slice staged per step
constexpr int RT_CHUNK = 512;   // hidden indices per chain of a score
}

template <typename T>
__device__ __forceinline__ float load_elem(const T *p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p) { return bf16_bits_to_float(*p); }
template <>
__device__ __forceinline__ float load_elem<float>(const float *p) { return *p; }

// Top-k of one token whose E (<= 256) scores sit in one wavefront, lane l
// holding experts l + 64 j in l4[j].
//   1. Scores map to order-preserving 32-bit keys (-0 read as +0, so equal
//      scores give equal keys); absent experts get key 0, below every score.
//   2. The k-th largest key is found bit by bit from the top: a candidate is
//      kept when at least k keys reach it, counted with wave ballots (no
//      cross-lane data movement, so each of the 32 steps is a few cycles).
//   3. The selection is every key above that threshold plus, among keys equal
//      to it, the lowest expert indices up to k in total.
//   4. The k selected (key, expert) pairs are compacted into the wave's LDS
//      scratch.  Every lane then reads all k pairs: a pair's output position
//      is the number of pairs that order before it (larger score, or equal
//      score and lower index), the largest score is their maximum, and the
//      renormalised softmax denominator is their sum of exponentials.
// Weights are softmax probabilities of the selected experts, optionally
// renormalised over the k (then only the k scores enter).  scr: this wave's
// LDS scratch of 2 x 256 words.
__device__ __forceinline__ uint32_t score_key(float v, bool valid)
{
    const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    return !valid ? 0u : ((u >> 31) ? ~u : (u | 0x80000000u));
}

// inverse of score_key for a present expert (the score's exact bits)
__device__ __forceinline__ float key_score(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

template <int S>   // 64-expert slots per lane (E <= 64 S)
__device__ __forceinline__ void select_topk(const float l4[4], int64_t t, int E, int k, int renorm,
                                            int32_t *__restrict__ ids, float *__restrict__ wout,
                                            float *__restrict__ logits_out, uint32_t *scr)
{
    const int lane = threadIdx.x & 63;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t key[S];
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const bool valid = lane + 64 * j < E;
        key[j] = score_key(l4[j], valid);
        if (valid && logits_out) logits_out[t * E + lane + 64 * j] = l4[j];
    }
    // k-th largest key (straight-line: 32 ballot rounds)
    uint32_t thr = 0;
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = thr | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < S; ++j) cnt += __popcll(__ballot(key[j] >= cand));
        thr = cnt >= k ? cand : thr;
    }
    // selection and compaction (expert order: slot j major, lane minor)
    int above = 0;
#pragma unroll
    for (int j = 0; j < S; ++j) above += __popcll(__ballot(key[j] > thr));
    const int need_eq = k - above;
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const uint64_t eq = __ballot(key[j] == thr);
        const bool sel = key[j] > thr || (key[j] == thr && eq_before + __popcll(eq & lt) < need_eq);
        const uint64_t sm = __ballot(sel);
        if (sel) {
            const int slot = sel_before + __popcll(sm & lt);
            scr[slot] = key[j];
            scr[256 + slot] = lane + 64 * j;
        }
        eq_before += __popcll(eq);
        sel_before += __popcll(sm);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (k <= 8) {
        // the (at most 8) pairs in registers, unused slots ordered last
        uint32_t kq[8];
        int eqi[8];
        const uint4 ka = *reinterpret_cast<const uint4 *>(scr), kb = *reinterpret_cast<const uint4 *>(scr + 4);
        const uint4 ia = *reinterpret_cast<const uint4 *>(scr + 256), ib = *reinterpret_cast<const uint4 *>(scr + 260);
        kq[0] = ka.x; kq[1] = ka.y; kq[2] = ka.z; kq[3] = ka.w; kq[4] = kb.x; kq[5] = kb.y; kq[6] = kb.z; kq[7] = kb.w;
        eqi[0] = ia.x; eqi[1] = ia.y; eqi[2] = ia.z; eqi[3] = ia.w; eqi[4] = ib.x; eqi[5] = ib.y; eqi[6] = ib.z; eqi[7] = ib.w;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q >= k) kq[q] = 0u;
        uint32_t kmax = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) kmax = max(kmax, kq[q]);
        const float mx = key_score(kmax);
        float denom = 0.0f;
        if (renorm) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q < k) denom += expf(key_score(kq[q]) - mx);
        } else {
            float zsum = 0.0f;
#pragma unroll
            for (int j = 0; j < S; ++j)
                if (lane + 64 * j < E) zsum += expf(l4[j] - mx);
            denom = wave_sum(zsum);
        }
        if (lane < k) {
            uint32_t ki = kq[0];
            int ei = eqi[0];
#pragma unroll
            for (int q = 1; q < 8; ++q)
                if (lane == q) { ki = kq[q]; ei = eqi[q]; }
            int pos = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                pos += (q < k && (kq[q] > ki || (kq[q] == ki && eqi[q] < ei))) ? 1 : 0;
            ids[t * k + pos] = ei;
            wout[t * k + pos] = expf(key_score(ki) - mx) / denom;
        }
    } else {
        uint32_t kmax = 0;
        for (int q = 0; q < k; ++q) kmax = max(kmax, scr[q]);
        const float mx = key_score(kmax);
        float denom = 0.0f;
        if (renorm) {
            for (int q = 0; q < k; ++q) denom += expf(key_score(scr[q]) - mx);
        } else {
            float zsum = 0.0f;
#pragma unroll
            for (int j = 0; j < S; ++j)
                if (lane + 64 * j < E) zsum += expf(l4[j] - mx);
            denom = wave_sum(zsum);
        }
        for (int i = lane; i < k; i += 64) {
            const uint32_t ki = scr[i];
            const int ei = (int)scr[256 + i];
            int pos = 0;
            for (int q = 0; q < k; ++q) {
                const uint32_t kq = scr[q];
                pos += (kq > ki || (kq == ki && (int)scr[256 + q] < ei)) ? 1 : 0;
            }
            ids[t * k + pos] = ei;
            wout[t * k + pos] = expf(key_score(ki) - mx) / denom;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Top-k for k <= 8 with renormalised weights (the layer's case), 8 / S
// tokens per wavefront at once, lanes working side by side instead of one
// token's 32 ballot rounds at a time.  Lane l takes token l / (8 S) and its
// experts 8 (l % (8 S)) .. + 7.  A (score, expert) pair is coded as the
// double whose bits are 1.0's with key << 8 | (255 - expert) in the low
// mantissa bits: a positive normal number, so doubles order like the codes,
// larger scores first and, among equal scores, lower expert indices, and
// the k largest are the selection in output order; one max and one min
// (v_max_f64, v_min_f64, exact: they return an operand) order a pair.  Each
// lane sorts its 8 values (Batcher's 19-comparator network), then exchanges
// its list with a lane of the other half of a growing lane group (DPP moves:
// xor 1, xor 2, mirror in 8, mirror in 16) and keeps the 8 largest of both:
// the elementwise maximum of its list and the partner's reversed one holds
// them as a bitonic sequence, which 12 comparators sort.  After log2(8 S)
// rounds each lane of a token holds the token's sorted top 8.  The weights
// take select_topk's arithmetic, so both give the same bits: the largest
// score as the offset, and the k exponentials (one per lane) summed in
// ascending expert order, which a 19-comparator sort of (expert, value)
// codes gives.
namespace {
constexpr int kBatcher8[19][2] = {{0, 1}, {2, 3}, {4, 5}, {6, 7}, {0, 2}, {1, 3}, {4, 6}, {5, 7}, {1, 2}, {5, 6},
                                  {0, 4}, {1, 5}, {2, 6}, {3, 7}, {2, 4}, {3, 5}, {1, 2}, {3, 4}, {5, 6}};
constexpr int kBitonic8[12][2] = {{0, 4}, {1, 5}, {2, 6}, {3, 7}, {0, 2}, {1, 3},
                                  {4, 6}, {5, 7}, {0, 1}, {2, 3}, {4, 5}, {6, 7}};
constexpr uint64_t kOneBits = 0x3ff0000000000000ull;   // 1.0
}

template <int CTRL>
__device__ __forceinline__ double dpp_move_f64(double v)
{
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// larger first
__device__ __forceinline__ void cmpx_desc(double &a, double &b)
{
    const double x = __builtin_fmax(a, b), y = __builtin_fmin(a, b);
    a = x;
    b = y;
}

// one exchange round: the 8 largest of this lane's and the partner's lists
template <int CTRL>
__device__ __forceinline__ void topk8_round(double (&c)[8])
{
    double p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = dpp_move_f64<CTRL>(c[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_fmax(c[i], p[7 - i]);
#pragma unroll
    for (int n = 0; n < 12; ++n) cmpx_desc(c[kBitonic8[n][0]], c[kBitonic8[n][1]]);
}

// Tokens tt0 .. tt0 + 8 / S - 1 of a block (block row tt holds the scores of
// token tb + tt, expert 64 j + c at score(j, tt, c)).  Every lane of the wave
// must call it (DPP and the lane exchange read the neighbours); rows past T_
// write nothing.
template <int S, typename ScoreFn>
__device__ __forceinline__ void topk8_renorm_tokens(ScoreFn score, int tt0, int64_t tb, int64_t T_, int E, int k,
                                                    int32_t *__restrict__ ids, float *__restrict__ wout,
                                                    float *__restrict__ logits_out)
{
    constexpr int NSUB = 8 * S;   // lanes per token
    const int lane = threadIdx.x & 63;
    const int sub = lane % NSUB, tt = tt0 + lane / NSUB;
    const int64_t t = tb + tt;
    const bool live = t < T_;
    double c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = 8 * sub + i;
        const float v = score(e >> 6, tt, e & 63);
        const bool valid = e < E;
        c[i] = __longlong_as_double(
            (long long)(kOneBits | ((uint64_t)score_key(v, valid) << 8) | (uint64_t)(255 - e)));
        if (live && valid && logits_out) logits_out[t * E + e] = v;
    }
#pragma unroll
    for (int n = 0; n < 19; ++n) cmpx_desc(c[kBatcher8[n][0]], c[kBatcher8[n][1]]);
    topk8_round<0xB1>(c);    // xor 1
    topk8_round<0x4E>(c);    // xor 2
    topk8_round<0x141>(c);   // mirror within 8 lanes
    if constexpr (S == 2) topk8_round<0x140>(c);   // mirror within 16 lanes
    auto key_of = [](double d) { return (uint32_t)((uint64_t)__double_as_longlong(d) >> 8); };
    auto expert_of = [](double d) { return 255 - (int)((uint64_t)__double_as_longlong(d) & 0xff); };
    const float mx = key_score(key_of(c[0]));
    // this lane's selection (lane sub < k takes the sub-th) and its exponential
    double mine = c[0];
#pragma unroll
    for (int q = 1; q < 8; ++q)
        if (sub == q) mine = c[q];
    const int my_e = expert_of(mine);
    const float my_x = sub < k ? expf(key_score(key_of(mine)) - mx) : 0.0f;
    // the token's k exponentials (lanes sub = 0 .. 7 of its group), coded as
    // (expert << 32 | value bits) in the same way and sorted by expert
    const int base = lane - sub;
    double d[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int eq = __shfl(my_e, base + q, 64);
        const float xq = __shfl(my_x, base + q, 64);
        d[q] = __longlong_as_double((long long)(kOneBits | ((uint64_t)(q < k ? eq : 256 + q) << 32) |
                                                (uint64_t)__float_as_uint(xq)));
    }
#pragma unroll
    for (int n = 0; n < 19; ++n) cmpx_desc(d[kBatcher8[n][1]], d[kBatcher8[n][0]]);   // ascending
    float denom = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) denom += __uint_as_float((uint32_t)__double_as_longlong(d[q]));
    if (live && sub < k) {
        ids[t * k + sub] = my_e;
        wout[t * k + sub] = my_x / denom;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void route_topk_kernel(const T *__restrict__ x, const uint16_t *__restrict__ wg,
                                                         int64_t T_, int64_t H, int E, int k, int renorm,
                                                         int32_t *__restrict__ ids, float *__restrict__ wout,
                                                         float *__restrict__ logits_out)
{
    __shared__ float xs[RT_TOK][RT_KC];
    __shared__ float wsl[256][RT_KC + 1];
    __shared__ __attribute__((aligned(16))) uint32_t tk_scr[4][512];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t t0 = (int64_t)blockIdx.x * RT_TOK;

    float acc[4][4], tot[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = tot[i][j] = 0.0f;

    static_assert(RT_CHUNK % RT_KC == 0, "chunks end at slice ends");
    for (int64_t k0 = 0; k0 < H; k0 += RT_KC) {
        const int kend = (int)((H - k0) < RT_KC ? (H - k0) : RT_KC);
        for (int idx = tid; idx < RT_TOK * RT_KC; idx += 256) {
            const int i = idx / RT_KC, kk = idx % RT_KC;
            const int64_t t = t0 + i;
            xs[i][kk] = (t < T_ && kk < kend) ? load_elem<T>(x + t * H + k0 + kk) : 0.0f;
        }
        for (int idx = tid; idx < E * RT_KC; idx += 256) {
            const int e = idx / RT_KC, kk = idx % RT_KC;
            wsl[e][kk] = kk < kend ? bf16_bits_to_float(wg[(int64_t)e * H + k0 + kk]) : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < kend; ++kk) {
            float xv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = xs[wave * 4 + i][kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (lane + 64 * j < E) {
                    const float wv = wsl[lane + 64 * j][kk];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i][j] = fmaf(xv[i], wv, acc[i][j]);
                }
            }
        }
        if ((k0 + RT_KC) % RT_CHUNK == 0 || k0 + RT_KC >= H) {   // a chunk ends: add its sums
            const bool first = k0 < RT_CHUNK;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    tot[i][j] = first ? acc[i][j] : tot[i][j] + acc[i][j];
                    acc[i][j] = 0.0f;
                }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + wave * 4 + i;
        if (t >= T_) break;
        select_topk<4>(tot[i], t, E, k, renorm, ids, wout, logits_out, tk_scr[wave]);
    }
}

// bf16 activations: the score chains run on the matrix cores.  With bf16
// operands every product is exact in fp32, so one v_mfma_f32_4x4x1_16b step
// (c += a * b, one rounding) is exactly one fused multiply-add of the chain;
// the instruction keeps 16 independent 4x4 outer products: lane l feeds
// token l % 4 and expert 64 s + l, and after the H steps holds the scores of
// tokens 0..3 for expert 64 s + l.
//
// A block is 8 wavefronts (two per SIMD, so that one wave's staging work and
// LDS waits overlap the other's matrix work); each owns one slice of 64
// experts (S slices) and one chunk of 4 tokens (8 / S chunks per block).
// x and W_g are staged through LDS in 32- or 64-wide
// hidden slices, widened to fp32 once when staged (so the inner loop is LDS
// reads and MFMAs only), rows padded to an odd number of 16-byte units (144
// or 272 bytes: the 16-byte reads of 16 consecutive rows hit distinct bank
// groups), three slices in flight in
// registers.  Zero padding beyond H or E adds +0 * 0 terms, which leave every
// chain unchanged.
namespace {
constexpr int RM_STAGES = 3;               // slices in flight (registers)
}

// WF32: W_g is given already widened to fp32 ([E][H]), staged by plain copies.
// KC: hidden indices per staged slice, 32 or 64 (64 halves the barriers and
// staging rounds of the chain; its LDS allows one block per CU, and 256
// experts do not fit).
template <int S, bool WF32, int KC>   // 64-expert slices (E <= 64 S), S in {1, 2, 4}
__global__ __launch_bounds__(512) void route_mfma_kernel(const uint16_t *__restrict__ x,
                                                         const void *__restrict__ wg, int64_t T_, int64_t H,
                                                         int E, int k, int renorm, int32_t *__restrict__ ids,
                                                         float *__restrict__ wout, float *__restrict__ logits_out,
                                                         int8_t *__restrict__ xq, float *__restrict__ sx)
{
    static_assert(KC == 32 || (KC == 64 && S <= 2), "slice width");
    constexpr int RM_KC = KC;
    constexpr int RM_ROW = RM_KC * 4 + 16;   // padded fp32 LDS row, bytes (an odd number of 16-byte units)
    constexpr int RM_PPR = RM_KC / 8;        // 16-byte bf16 pieces per row slice
    constexpr int NT = 512;                                    // threads
    constexpr int TC = 8 / S;                                  // 4-token chunks per block
    constexpr int WROWS = 64 * S, XROWS = 4 * TC;
    constexpr int WPR = WF32 ? 2 * RM_PPR : RM_PPR;            // 16-byte pieces per W_g row slice
    constexpr int WPIECES = WROWS * WPR, XPIECES = XROWS * RM_PPR;   // 16-byte pieces per slice
    constexpr int WPT = (WPIECES + NT - 1) / NT, XPT = (XPIECES + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) unsigned char wl[2][WROWS * RM_ROW];
    __shared__ __attribute__((aligned(16))) unsigned char xl[2][XROWS * RM_ROW];
    __shared__ float lg[XROWS][WROWS + 1];
    __shared__ __attribute__((aligned(16))) uint32_t tk_scr[8][512];
    __shared__ float qmax[XROWS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int sl = wave % S, ch = wave / S;
    static_assert(XPT == 1, "one x piece per thread and slice");
    float xmax = 0.0f;   // largest |x| of the pieces this thread stages (one token row)
    const int64_t tb = (int64_t)blockIdx.x * XROWS;
    const int nsl = (int)((H + RM_KC - 1) / RM_KC);

    // buffer resources: an out-of-range offset reads zero without a branch
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x), 0, 0x7ffffff0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(wg), 0, 0x7ffffff0, 0x00020000);
    // staging assignment: piece p = row * 4 + c holds hidden 8c..8c+7 of the slice
    int woff[WPT], xoff[XPT];
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int p = tid + j * NT, row = p / WPR, c = p % WPR;
        woff[j] = (p < WPIECES && row < E) ? (int)((int64_t)row * H * (WF32 ? 4 : 2)) + 16 * c : 0x7fffffff;
    }
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
        const int p = tid + j * NT, row = p / RM_PPR, c = p % RM_PPR;
        xoff[j] = (p < XPIECES && tb + row < T_) ? (int)((tb + row) * H * 2) + 16 * c : 0x7fffffff;
    }
    uint4 wr[RM_STAGES][WPT], xr[RM_STAGES][XPT];
    auto load = [&](int st, int slc) {
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const int c = (tid + j * NT) % WPR;
            const bool ok = woff[j] != 0x7fffffff && slc * RM_KC + (WF32 ? 4 : 8) * c < H;
            wr[st][j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rw, ok ? woff[j] + slc * RM_KC * (WF32 ? 4 : 2) : 0x7fffffff, 0, 0));
        }
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            const int c = (tid + j * NT) % RM_PPR;
            const bool ok = xoff[j] != 0x7fffffff && slc * RM_KC + 8 * c < H;
            xr[st][j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? xoff[j] + slc * RM_KC * 2 : 0x7fffffff, 0, 0));
        }
    };
    // widen 8 bf16 to fp32 (exact) into LDS row `row`, hidden 8c..8c+7
    auto put = [&](unsigned char *base, int p, const uint4 &v) {
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
        uint4 lo, hi;
        lo.x = u[0] << 16; lo.y = u[0] & 0xffff0000u; lo.z = u[1] << 16; lo.w = u[1] & 0xffff0000u;
        hi.x = u[2] << 16; hi.y = u[2] & 0xffff0000u; hi.z = u[3] << 16; hi.w = u[3] & 0xffff0000u;
        unsigned char *d = base + (p / RM_PPR) * RM_ROW + 32 * (p % RM_PPR);
        *reinterpret_cast<uint4 *>(d) = lo;
        *reinterpret_cast<uint4 *>(d + 16) = hi;
    };
    // staging work of one slice: WPT pieces of W_g, then XPT of x
    constexpr int NITEMS = WPT + XPT;
    auto stage_item = [&](int item, int st, int buf) {
        if (item < WPT) {
            const int p = tid + item * NT;
            if constexpr (WF32) {
                if (p < WPIECES)
                    *reinterpret_cast<uint4 *>(wl[buf] + (p / WPR) * RM_ROW + 16 * (p % WPR)) = wr[st][item];
            } else {
                if (p < WPIECES) put(wl[buf], p, wr[st][item]);
            }
        } else {
            const int p = tid + (item - WPT) * NT;
            if (p < XPIECES) {
                const uint4 v = xr[st][item - WPT];
                put(xl[buf], p, v);
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xmax = fmaxf(xmax, fmaxf(__uint_as_float((u[i] << 16) & 0x7fffffffu),
                                             __uint_as_float(u[i] & 0x7fff0000u)));
            }
        }
    };

#pragma unroll
    for (int st = 0; st < RM_STAGES; ++st) load(st, st);
#pragma unroll
    for (int it = 0; it < NITEMS; ++it) stage_item(it, 0, 0);
    load(0, RM_STAGES);
    __syncthreads();

    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f}, tot = acc;
    constexpr int SPC = RT_CHUNK / RM_KC;   // slices per chunk of the score
    static_assert(RT_CHUNK % RM_KC == 0, "chunks end at slice ends");
    const unsigned char *wrow0 = &wl[0][(sl * 64 + lane) * RM_ROW];
    const unsigned char *xrow0 = &xl[0][(ch * 4 + (lane & 3)) * RM_ROW];
    const int nsl_pad = (nsl + RM_STAGES - 1) / RM_STAGES * RM_STAGES;
    for (int s0 = 0; s0 < nsl_pad; s0 += RM_STAGES) {
#pragma unroll
        for (int d = 0; d < RM_STAGES; ++d) {
            const int slc = s0 + d;
            const int buf = slc & 1;
            const int dn = (d + 1) % RM_STAGES;   // register slot of slice slc+1
            if (slc < nsl) {
                const unsigned char *wrow = wrow0 + buf * (WROWS * RM_ROW);
                const unsigned char *xrow = xrow0 + buf * (XROWS * RM_ROW);
                // operands of the next 4 hidden indices are read while the
                // current ones feed the chain
                v4f wv = *reinterpret_cast<const v4f *>(wrow);
                v4f xa = *reinterpret_cast<const v4f *>(xrow);
#pragma unroll
                for (int c = 0; c < RM_KC / 4; ++c) {
                    v4f wn = wv, xan = xa;
                    if (c + 1 < RM_KC / 4) {
                        wn = *reinterpret_cast<const v4f *>(wrow + 16 * (c + 1));
                        xan = *reinterpret_cast<const v4f *>(xrow + 16 * (c + 1));
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[j], wv[j], acc, 0, 0, 0);
                    wv = wn;
                    xa = xan;
                }
                if ((slc + 1) % SPC == 0 || slc + 1 == nsl) {   // a chunk ends: add its sums
                    if (slc < SPC) tot = acc;
                    else tot = tot + acc;
                    acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
            // slice slc+1 (loaded RM_STAGES slices ago) into the other buffer
#pragma unroll
            for (int it = 0; it < NITEMS; ++it) stage_item(it, dn, (slc + 1) & 1);
            load(dn, slc + 1 + RM_STAGES);
            __syncthreads();
        }
    }
    // lane l, value i: score of token 4 ch + i for expert 64 sl + l
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[ch * 4 + i][sl * 64 + lane] = tot[i];
    __syncthreads();
    for (int tt = wave; tt < XROWS; tt += 8) {
        const int64_t t = tb + tt;
        if (t >= T_) break;
        float l4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) l4[j] = (j < S) ? lg[tt][lane + 64 * j] : 0.0f;
        select_topk<S>(l4, t, E, k, renorm, ids, wout, logits_out, tk_scr[wave]);
    }

    // Per-token int8 codes of the block's tokens, when asked for: every x
    // element passed through this block's staging, whose pieces of one token
    // row are staged by RM_PPR consecutive lanes, so the row maxima are a
    // reduction over those lanes; the codes then take a second (L2-resident)
    // read of the rows, with the quantisation kernels' arithmetic.
    if (xq) {
        float m = xmax;
#pragma unroll
        for (int o = 1; o < RM_PPR; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if (tid < XPIECES && tid % RM_PPR == 0) qmax[tid / RM_PPR] = m;
        __syncthreads();
        constexpr int TPR = NT / XROWS;   // threads per token row
        const int row = tid / TPR, t8 = tid % TPR;
        const int64_t t = tb + row;
        if (t < T_) {
            const float amax = qmax[row];
            const float s = amax / 127.0f;
            const float y = s > 0.0f ? 1.0f / s : 0.0f;
            const bool fast = s >= QUANT_FAST_MIN_SCALE;
            if (t8 == 0) sx[t] = s;
            for (int64_t c = (int64_t)t8 * 8; c < H; c += TPR * 8) {
                float v[8];
                load8_f32(x + t * H + c, v);
                *reinterpret_cast<uint2 *>(xq + t * H + c) = s != 0.0f ? pack8(v, s, y, fast) : make_uint2(0u, 0u);
            }
        }
    }
}

// bf16 activations, many tokens: the score chains on the 32 x 32 x 1 fp32
// matrix instruction (v_mfma_f32_32x32x1_2b_f32).  Its two blocks each add a
// 32 x 32 outer product of one hidden index to their accumulators; every
// product of two bf16 values is exact in fp32, so each step is exactly one
// fused multiply-add of each of the 2048 chains it holds.  A wave takes 32
// tokens (lane l feeds token l % 32 to both blocks), all 64 S experts (S
// accumulators; lane l feeds expert 64 j + l of slice j: block l / 32; with
// SPLIT one slice per wave), and one run of CPW of the score's 512-index
// chunks.  Each x operand is used 64 S times and each W_g operand 32 times, so
// the lanes load them straight from memory (x rows and W_g, both L2-resident
// after the first touch) into registers, D steps of 8 indices ahead, and widen
// the bf16 pairs in registers: no LDS staging and no barrier until the chains
// end.
//
// A block is 32 tokens and NCW waves, one per chunk run (SPLIT: 2 NCW waves,
// one per run and slice).  The chunk sums meet in LDS in ascending chunk order
// (the run of wave 0 first, each later run adding its chunks one at a time to
// the running total as soon as the runs before it are in), and the top-k runs
// on the totals.  The waves of a block
// share their compute unit's matrix cores unevenly (measured: the first wave
// on each SIMD ends its chain about a fifth of the chain time before the
// second), so with xq the waves that are done quantise the block's tokens
// while the others finish (each row read and coded by one wave).
//
// Output layout of the instruction: block b of the result sits in registers
// 16 b .. 16 b + 15; register 16 b + 4 q + r of lane l holds row 8 q + 4 (l / 32)
// + r, column l % 32 (rows: tokens, columns: experts).
namespace {
constexpr int R32_STEPS = RT_CHUNK / 8;
constexpr int r32_max_waves(int S) { return S == 1 ? 16 : 8; }
// 8-index steps in flight per lane: 8 with two slices (a block of at most 8
// waves, 256 registers each) or with 16-token blocks (16-register
// accumulators), 4 with one slice of 32 tokens (16 waves, 128 registers)
constexpr int r32_depth(int TOK, int S) { return (S == 1 && TOK == 32) ? 4 : 8; }
}

// TOK: tokens per block, 32 (the 32 x 32 x 1 instruction) or 16 (its
// 16 x 16 x 1 four-block form, for fewer tokens: twice the blocks).  QX: the
// block also quantises its tokens (xq and sx are then given).  SPLIT (two
// slices): each chunk run takes two waves, one per 64-expert slice (wave w:
// run w / 2, slice w % 2), so a SIMD interleaves twice the waves, each with
// one chain; both waves load the run's x operands.
template <int TOK, int S, int CPW, bool PACKED, bool QX, bool SPLIT = false>   // S: 64-expert slices (E <= 64 S), CPW: chunks per wave
__global__ __launch_bounds__(64 * (SPLIT ? 16 : r32_max_waves(S))) void route_mfma_k1_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ wg, int64_t T_, int64_t H,
                                                            int E, int k, int renorm, int NCW,
                                                            int32_t *__restrict__ ids, float *__restrict__ wout,
                                                            float *__restrict__ logits_out, int8_t *__restrict__ xq,
                                                            float *__restrict__ sx)
{
    static_assert(S == 1 || S == 2, "slices");
    static_assert(TOK == 32 || TOK == 16, "tokens per block");
    static_assert(!SPLIT || S == 2, "a split run is two slices");
    constexpr int SW = SPLIT ? 1 : S;   // slices per wave
    constexpr int R32_D = r32_depth(TOK, S);
    static_assert(R32_STEPS % R32_D == 0, "chunks end at pass ends");
    // a lane's accumulator: TOK x 64 results over 64 lanes
    typedef float vacc __attribute__((ext_vector_type(TOK)));
    __shared__ float rt[S][TOK][64 + 1];    // running totals, then the scores
    __shared__ __attribute__((aligned(16))) uint32_t tk_scr[8][512];
    __shared__ int q_next;   // next token row of the block to quantise
    __shared__ int r_done[SPLIT ? 2 : 1];   // chunk runs added to the running totals (per slice if split)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the run bounds stay scalar
    const int nwv = NCW * (SPLIT ? 2 : 1);                      // waves of the block
    const int run = SPLIT ? wv >> 1 : wv;
    const int js = SPLIT ? wv & 1 : 0;                          // the wave's first slice
    const int64_t tb = (int64_t)blockIdx.x * TOK;
    const int nst = (int)(H / 8);
    const int nch = (nst + R32_STEPS - 1) / R32_STEPS;
    const int c_beg = min(nch, run * CPW), c_end = min(nch, c_beg + CPW);
    const int s_beg = c_beg * R32_STEPS, s_end = min(nst, c_end * R32_STEPS);

    // offsets: an out-of-range one (absent token or expert, or a step past the
    // run) starts at OOB and stays above the resource size, so it reads zeros
    constexpr uint32_t OOB = 0x80000000u;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x), 0, 0x7ffffff0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(wg), 0, 0x7ffffff0, 0x00020000);
    const int tok = lane & (TOK - 1);
    const uint32_t xrow = tb + tok < T_ ? (uint32_t)((tb + tok) * H * 2) : OOB;
    uint32_t wrow[SW];
#pragma unroll
    for (int j = 0; j < SW; ++j) {
        const int e = 64 * (js + j) + lane;
        wrow[j] = e < E ? (PACKED ? (uint32_t)e * 16u : (uint32_t)((int64_t)e * H * 2)) : OOB;
    }
    const uint32_t wstep = PACKED ? (uint32_t)E * 16u : 16u;   // bytes between steps of one expert
    if (tid == 0) {
        q_next = 0;
        r_done[0] = 0;
        if constexpr (SPLIT) r_done[1] = 0;
    }
    __syncthreads();
    uint4 xr[R32_D], wr[R32_D][SW];
    auto load = [&](int slot, int st) {
        const bool live = st < s_end;
        xr[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rx, live ? xrow + (uint32_t)st * 16u : OOB, 0, 0));
#pragma unroll
        for (int j = 0; j < SW; ++j)
            wr[slot][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rw, live ? wrow[j] + (uint32_t)st * wstep : OOB, 0, 0));
    };
#pragma unroll
    for (int d = 0; d < R32_D; ++d) load(d, s_beg + d);

    vacc acc[CPW][SW];
    // c += a * b for one hidden index: TOK tokens x 64 experts
    auto mfma = [](float av, float bv, const vacc &c) -> vacc {
        if constexpr (TOK == 32) return __builtin_amdgcn_mfma_f32_32x32x1f32(av, bv, c, 0, 0, 0);
        else return __builtin_amdgcn_mfma_f32_16x16x1f32(av, bv, c, 0, 0, 0);
    };
    // one step: the 8 indices of slot d into the chains, then the slot's
    // refill with step st + R32_D (st % R32_D == d: chunks start at multiples)
    auto step = [&](vacc (&a)[SW], int d, int st) {
        const uint32_t u[4] = {xr[d].x, xr[d].y, xr[d].z, xr[d].w};
        // hidden 8 st + 2 i is the low half of word i, 8 st + 2 i + 1 the high half
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = __uint_as_float(u[i] << 16), x1 = __uint_as_float(u[i] & 0xffff0000u);
#pragma unroll
            for (int j = 0; j < SW; ++j) {
                const uint32_t w = (&wr[d][j].x)[i];
                a[j] = mfma(x0, __uint_as_float(w << 16), a[j]);
            }
#pragma unroll
            for (int j = 0; j < SW; ++j) {
                const uint32_t w = (&wr[d][j].x)[i];
                a[j] = mfma(x1, __uint_as_float(w & 0xffff0000u), a[j]);
            }
        }
        load(d, st + R32_D);
        // keep the refill here: scheduled to the end of the pass, each load
        // would be waited for right after it is issued
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci) {
        vacc a[SW];
#pragma unroll
        for (int j = 0; j < SW; ++j) a[j] = vacc{};
        const int cs = s_beg + ci * R32_STEPS;
        const int ce = min(s_end, cs + R32_STEPS);
        const int cf = cs + max(0, ce - cs) / R32_D * R32_D;   // end of the whole passes
        for (int st0 = cs; st0 < cf; st0 += R32_D) {
#pragma unroll
            for (int d = 0; d < R32_D; ++d) step(a, d, st0 + d);
        }
#pragma unroll
        for (int d = 0; d < R32_D; ++d)   // a chunk's last, partial pass (only where H ends inside it)
            if (cf + d < ce) step(a, d, cf + d);
#pragma unroll
        for (int j = 0; j < SW; ++j) acc[ci][j] = a[j];
    }
    // Chunk sums into the running totals, runs in ascending order: run r waits
    // until runs 0 .. r - 1 are in (r_done == r), adds its chunks one at a
    // time, then lets run r + 1 go (split: the runs of each slice in order, a
    // counter per slice).  Every earlier run ends without waiting on a later
    // one, so each wait ends.
    if (run > 0)
        while (__hip_atomic_load(&r_done[js], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < run)
            __builtin_amdgcn_s_sleep(1);
    if (c_beg < c_end) {
        // lane l's element reg of slice j (reg = 4 q + i).  32 tokens: row
        // 8 (q & 3) + 4 (l / 32) + i, column 32 (q / 4) + l % 32; 16 tokens
        // (block q of the instruction): row 4 (l / 16) + i, column 16 q + l % 16
        auto rt_at = [&](int j, int reg) -> float & {
            const int q = reg >> 2, i = reg & 3;
            if constexpr (TOK == 32)
                return rt[j][8 * (q & 3) + 4 * (lane >> 5) + i][32 * (q >> 2) + (lane & 31)];
            else
                return rt[j][4 * (lane >> 4) + i][16 * q + (lane & 15)];
        };
        // the run's chunk sums added in order to what the earlier runs left
        // (all loads first, then the sums and stores)
        auto add_run = [&](const float(&before)[SW][TOK], bool first) {
#pragma unroll
            for (int j = 0; j < SW; ++j)
#pragma unroll
                for (int reg = 0; reg < TOK; ++reg) {
                    float t = first ? acc[0][j][reg] : before[j][reg] + acc[0][j][reg];
#pragma unroll
                    for (int ci = 1; ci < CPW; ++ci)
                        if (c_beg + ci < c_end) t = t + acc[ci][j][reg];
                    rt_at(js + j, reg) = t;
                }
        };
        float tot[SW][TOK];
        if (run == 0) {
            add_run(tot, true);
        } else {
#pragma unroll
            for (int j = 0; j < SW; ++j)
#pragma unroll
                for (int reg = 0; reg < TOK; ++reg) tot[j][reg] = rt_at(js + j, reg);
            add_run(tot, false);
        }
    }
    __hip_atomic_store(&r_done[js], run + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);

    // Per-token int8 codes, when asked for, with the quantisation kernels'
    // arithmetic: a wave that has added its chunk sums takes the block's token
    // rows one at a time (a shared counter) while the waves behind it still
    // run their chains, so the codes cost little time after the chains.  A
    // wave reads a row in pieces of 8 elements, QP per lane at a time, the
    // next row's first pieces while it codes the current one: one read where
    // the row fits (H <= 512 QP), else one read for the largest magnitude and
    // one for the codes.  (QP: 8, or 4 in the 128-register waves of one-slice
    // blocks.)
    if constexpr (QX) {
        constexpr int QP = S == 1 ? 4 : 8;
        const int npc = (int)(H / 8);   // 8-element pieces per row
        auto grab = [&]() {
            int u = 0;
            if (lane == 0) u = atomicAdd(&q_next, 1);
            return __builtin_amdgcn_readfirstlane(u);
        };
        // pieces p0 + lane + 64 i of the block's row u (zeros past the row or the tokens)
        auto qload = [&](uint4(&v)[QP], int u, int p0) {
            const bool live = u < TOK && tb + u < T_;
            const uint32_t rb = live ? (uint32_t)((tb + u) * H * 2) : 0u;
#pragma unroll
            for (int i = 0; i < QP; ++i) {
                const int p = p0 + lane + 64 * i;
                v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rx, (live && p < npc) ? rb + (uint32_t)p * 16u : OOB, 0, 0));
            }
        };
        auto widen = [](const uint4 &q, float f[8]) {
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[2 * i] = __uint_as_float(w[i] << 16);
                f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        };
        // codes of row u, whose first QP pieces per lane are in v
        auto qrow = [&](uint4(&v)[QP], int u) {
            const int64_t t = tb + u;
            if (t >= T_) return;
            float amax = 0.0f;
            for (int p0 = 0; p0 < npc; p0 += 64 * QP) {
                if (p0 > 0) qload(v, u, p0);
#pragma unroll
                for (int i = 0; i < QP; ++i) {
                    float f[8];
                    widen(v[i], f);
#pragma unroll
                    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
                }
            }
            amax = wave_max_nonneg(amax);
            const float s = amax / 127.0f;
            const float y = s > 0.0f ? 1.0f / s : 0.0f;
            const bool fast = s >= QUANT_FAST_MIN_SCALE;
            if (lane == 0) sx[t] = s;
            int8_t *qdst = xq + t * H;
            for (int p0 = 0; p0 < npc; p0 += 64 * QP) {
                if (npc > 64 * QP) qload(v, u, p0);   // the row did not fit: read this part again
#pragma unroll
                for (int i = 0; i < QP; ++i) {
                    const int p = p0 + lane + 64 * i;
                    if (p < npc) {
                        float f[8];
                        widen(v[i], f);
                        *reinterpret_cast<uint2 *>(qdst + 8 * p) =
                            s != 0.0f ? pack8(f, s, y, fast) : make_uint2(0u, 0u);
                    }
                }
            }
        };
        uint4 va[QP], vb[QP];
        int u = grab();
        qload(va, u, 0);
        while (u < TOK) {
            const int u2 = grab();
            qload(vb, u2, 0);
            qrow(va, u);
            if (u2 >= TOK) break;
            u = grab();
            qload(va, u, 0);
            qrow(vb, u2);
        }
    }
    __syncthreads();

    if (renorm && k <= 8) {
        // 8 / S tokens per wave at once, every wave taking groups in turn
        constexpr int TPW = 8 / S;
        auto score = [&](int j, int tt, int c) { return rt[j][tt][c]; };
        for (int tt0 = wv * TPW; tt0 < TOK; tt0 += nwv * TPW)
            topk8_renorm_tokens<S>(score, tt0, tb, T_, E, k, ids, wout, logits_out);
        return;
    }
    const int ntk = min(nwv, 8);   // waves that run the top-k
    for (int tt = wv; tt < TOK && wv < 8; tt += ntk) {
        const int64_t t = tb + tt;
        if (t >= T_) break;
        float l4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) l4[j] = (j < S) ? rt[j][tt][lane] : 0.0f;
        select_topk<S>(l4, t, E, k, renorm, ids, wout, logits_out, tk_scr[wv]);
    }
}

// Vector-ALU router for few tokens.  A wavefront owns TPW tokens, one slice
// of 64 experts and a run of the score's 512-index chunks: lane l runs the TPW
// fma chains of expert 64 sl + l over those chunks (v_fma_f32 is exactly the
// chain's fmaf), so every W_g value a lane loads feeds TPW chains.  With few
// tokens the router is bound by one wave's issue of its chain, so the chunks
// of a score can be spread over CW waves (the launch's choice, up to 8 / S)
// that run side by side; their chunk sums meet in LDS and are added in chunk
// order.  That pays only with PACKED W_g ([H/8][E][8], a wave's step one
// contiguous kilobyte): read from the [E][H] rows every lane's 16-byte step
// lies on its own cache line, and more waves streaming rows at once slow the
// loads down more than the shorter chains gain (so the launch takes CW = 1).
// The block first widens its tokens' rows of x into LDS (fp32); the chains
// then take them as broadcast LDS reads issued XP steps ahead, while each lane
// streams its expert's bf16 W_g values D steps of 8 ahead and widens them in
// registers.  A step holds as few instructions as it can: 8 fmas, 8 widening
// ops, one W load at a fixed offset from the pass base, two LDS reads.  (The
// fp32 copy of W_g would double the load instructions; the bf16 rows are
// faster here.)
//
// Waves: S * CW chain waves (wave w: slice w % S, chunk run w / S), then, with
// xq != nullptr, one more that quantises the staged token rows (per-token int8
// codes and scale, the same arithmetic as the quantisation kernels) while the
// others run their chains.
namespace {
constexpr int RV_MAX_CHUNKS = 16;   // H <= 8192
constexpr int RV_STEPS_PER_CHUNK = RT_CHUNK / 8;
}

template <int S, int TPW, bool PACKED>
__global__ __launch_bounds__(576) void route_valu_kernel(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ wg, int64_t T_, int64_t H,
                                                         int E, int k, int renorm, int CW,
                                                         int32_t *__restrict__ ids, float *__restrict__ wout,
                                                         float *__restrict__ logits_out, int8_t *__restrict__ xq,
                                                         float *__restrict__ sx)
{
    constexpr int D = 16;   // W_g steps (8 values each) in flight per lane
    constexpr int XP = 2;   // x steps read ahead from LDS
    static_assert(RV_STEPS_PER_CHUNK % D == 0, "passes end at chunk ends");
    // [TPW][H] fp32, plus the XP * 8 floats that the read-ahead past the last row touches
    extern __shared__ __attribute__((aligned(16))) float xs[];
    __shared__ float lg[RV_MAX_CHUNKS][TPW][64 * S + 1];   // chunk sums
    __shared__ __attribute__((aligned(16))) uint32_t tk_scr[S][512];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nchain = S * CW;
    const int sl = wave % S, run = wave / S;
    const int e = 64 * sl + lane;
    const int64_t tb = (int64_t)blockIdx.x * TPW;
    const int nst = (int)(H / 8);
    const int nch = (nst + RV_STEPS_PER_CHUNK - 1) / RV_STEPS_PER_CHUNK;
    const int cpw = (nch + CW - 1) / CW;   // chunks per wave
    const int c_beg = min(nch, run * cpw), c_end = min(nch, c_beg + cpw);
    const int st_b = c_beg * RV_STEPS_PER_CHUNK, st_e = min(nst, c_end * RV_STEPS_PER_CHUNK);
    // the resource spans W_g exactly: a read past its end (the look-ahead of
    // the last steps, the lanes past E) returns zeros
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(wg), 0, (int)(E * H * 2), 0x00020000);
    // byte offset of this lane's step st: wrow + st * stepb
    const uint32_t stepb = PACKED ? (uint32_t)E * 16u : 16u;
    const uint32_t wrow = e < E ? (PACKED ? (uint32_t)e * 16u : (uint32_t)((int64_t)e * H * 2)) : 0x80000000u;

    uint4 wr[D];
    // within a pass the offset is the pass base plus a uniform d * stepb
    auto load_w = [&](int slot, uint32_t base, uint32_t soff) {
        wr[slot] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, base, soff, 0));
    };
    if (wave < nchain) {
#pragma unroll
        for (int d = 0; d < D; ++d) load_w(d, wrow + (uint32_t)st_b * stepb, (uint32_t)d * stepb);
    }
    // x rows into LDS (a token past T stages zeros; its result is never stored)
    for (int64_t i = (int64_t)tid * 8; i < TPW * H; i += (int64_t)blockDim.x * 8) {
        const int t = (int)(i / H);
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (tb + t < T_) load8_f32(x + (tb + t) * H + (i - (int64_t)t * H), v);
        *reinterpret_cast<float4 *>(xs + i) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(xs + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    __syncthreads();

    if (wave == nchain) {   // the quantisation wave (present only when xq is given)
        for (int t = 0; t < TPW && tb + t < T_; ++t) {
            const float *xr = xs + t * H;
            float amax = 0.0f;
            for (int64_t c = (int64_t)lane * 8; c < H; c += 512) {
                const float4 a = *reinterpret_cast<const float4 *>(xr + c);
                const float4 b = *reinterpret_cast<const float4 *>(xr + c + 4);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
            }
            amax = wave_max_nonneg(amax);
            const float s = amax / 127.0f;
            const float y = s > 0.0f ? 1.0f / s : 0.0f;
            const bool fast = s >= QUANT_FAST_MIN_SCALE;
            if (lane == 0) sx[tb + t] = s;
            int8_t *qr = xq + (tb + t) * H;
            for (int64_t c = (int64_t)lane * 8; c < H; c += 512) {
                const float4 a = *reinterpret_cast<const float4 *>(xr + c);
                const float4 b = *reinterpret_cast<const float4 *>(xr + c + 4);
                const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                *reinterpret_cast<uint2 *>(qr + c) = s != 0.0f ? pack8(v, s, y, fast) : make_uint2(0u, 0u);
            }
        }
    }
    if (wave >= nchain) {   // no chain: meet the chain waves at the barrier before the top-k
        __syncthreads();
        return;
    }

    auto widen_w = [&](int slot, float w8[8]) {
        const uint32_t u[4] = {wr[slot].x, wr[slot].y, wr[slot].z, wr[slot].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w8[2 * i] = __uint_as_float(u[i] << 16);
            w8[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    };
    float4 xr[XP][TPW][2];
    auto load_x = [&](int slot, int st) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            xr[slot][t][0] = *reinterpret_cast<const float4 *>(xs + t * H + st * 8);
            xr[slot][t][1] = *reinterpret_cast<const float4 *>(xs + t * H + st * 8 + 4);
        }
    };
    auto chain8 = [&](const float4 (&xv)[TPW][2], const float w8[8], float acc[TPW]) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const float x8[8] = {xv[t][0].x, xv[t][0].y, xv[t][0].z, xv[t][0].w,
                                 xv[t][1].x, xv[t][1].y, xv[t][1].z, xv[t][1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[t] = fmaf(x8[i], w8[i], acc[t]);
        }
    };
    // the sum of the chunk that ends here goes to LDS; the next chain starts at +0
    auto close_chunk = [&](int c, float acc[TPW]) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            lg[c][t][e] = acc[t];
            acc[t] = 0.0f;
        }
    };
    float acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int p = 0; p < XP; ++p) load_x(p, st_b + p);
    const int nmain = st_b + (st_e - st_b) / D * D;
    for (int st0 = st_b; st0 < nmain; st0 += D) {
        const uint32_t base = wrow + (uint32_t)(st0 + D) * stepb;   // the next pass's steps
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float w8[8];
            widen_w(d, w8);
            float4 xv[TPW][2];
#pragma unroll
            for (int t = 0; t < TPW; ++t) xv[t][0] = xr[d % XP][t][0], xv[t][1] = xr[d % XP][t][1];
            load_x(d % XP, st0 + d + XP);   // past the rows it reads the pad (unused)
            chain8(xv, w8, acc);
            load_w(d, base, (uint32_t)d * stepb);   // after the fmas: the slot's registers are free again
            // keep each step's loads in place: the scheduler would otherwise batch
            // them at the end of the body, and every pass would wait for them all
            __builtin_amdgcn_sched_barrier(0);
        }
        if ((st0 + D) % RV_STEPS_PER_CHUNK == 0) close_chunk((st0 + D) / RV_STEPS_PER_CHUNK - 1, acc);
    }
    // tail: the last st_e - nmain (< D) steps; slot d holds step nmain + d
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (nmain + d < st_e) {
            float w8[8];
            widen_w(d, w8);
            float4 xv[TPW][2];
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                xv[t][0] = *reinterpret_cast<const float4 *>(xs + t * H + (nmain + d) * 8);
                xv[t][1] = *reinterpret_cast<const float4 *>(xs + t * H + (nmain + d) * 8 + 4);
            }
            chain8(xv, w8, acc);
        }
    }
    if (st_e > st_b && st_e % RV_STEPS_PER_CHUNK != 0) close_chunk(c_end - 1, acc);   // the short last chunk
    __syncthreads();
    if (wave >= S) return;
    for (int tt = wave; tt < TPW; tt += S) {
        const int64_t t = tb + tt;
        if (t >= T_) break;
        float l4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = 0.0f;
            if (j < S) {
                v = lg[0][tt][lane + 64 * j];
                for (int c = 1; c < nch; ++c) v = v + lg[c][tt][lane + 64 * j];
            }
            l4[j] = v;
        }
        select_topk<S>(l4, t, E, k, renorm, ids, wout, logits_out, tk_scr[wave]);
    }
}

// W_g widened to fp32 once (exact): the bf16 pattern becomes the upper half.
__global__ __launch_bounds__(256) void widen_bf16_kernel(const uint16_t *__restrict__ src, int64_t n,
                                                         float *__restrict__ dst)
{
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (int64_t)gridDim.x * 256 * 8) {
        float v[8];
        load8_f32(src + i, v);
        store8(dst + i, v);
    }
}

// [E][H] -> [H/8][E][8]: thread i copies the 16-byte piece (j, e) = (i / E, i % E)
__global__ __launch_bounds__(256) void pack_router_kernel(const uint16_t *__restrict__ src, int E, int64_t H,
                                                          uint16_t *__restrict__ dst)
{
    const int64_t n = H / 8 * E;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t j = i / E, e = i % E;
        *reinterpret_cast<uint4 *>(dst + i * 8) = *reinterpret_cast<const uint4 *>(src + e * H + j * 8);
    }
}

hipError_t launch_pack_router(const uint16_t *wg, int E, int64_t H, uint16_t *dst, hipStream_t st)
{
    const int64_t n = H / 8 * E;
    if (n == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(pack_router_kernel, dim3((unsigned)blocks), dim3(256), 0, st, wg, E, H, dst);
    return hipGetLastError();
}

hipError_t launch_widen_bf16(const uint16_t *src, int64_t n, float *dst, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n / 8 + 255) / 256, 4096);
    hipLaunchKernelGGL(widen_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, n, dst);
    return hipGetLastError();
}

// Up to 512 (token, 64-expert slice) pairs and H <= 8192 (the token row in
// LDS) the vector-ALU router runs, above that the matrix-core one; with bf16
// tokens both can also quantise them.
static bool route_valu_path(int64_t T, int64_t H, int E)
{
    const int S = E <= 64 ? 1 : (E <= 128 ? 2 : 4);
    return T * S <= 512 && H <= 8192;
}

bool route_fuses_quant(int dtype, int64_t, int64_t, int) { return dtype == 0; }

hipError_t launch_route_topk(const void *x, int dtype, const uint16_t *wg, const float *wg_f32, int64_t T,
                             int64_t H, int E, int k, int renormalize, int32_t *ids, float *w, float *logits,
                             hipStream_t st, int8_t *xq, float *sx, const uint16_t *wg_packed)
{
    if (T == 0) return hipSuccess;
    if (dtype == 0) {
        const int S = E <= 64 ? 1 : (E <= 128 ? 2 : 4);
        const uint16_t *xb = (const uint16_t *)x;
        const void *wp = wg_f32 ? (const void *)wg_f32 : (const void *)wg;
        if (route_valu_path(T, H, E)) {
            // few tokens: vector-ALU chains over the bf16 W_g, one token per
            // block; with the packed W_g the score's chunks are spread over up
            // to 8 / S waves per slice
            constexpr int TP = 1;
            const size_t lds = ((size_t)TP * H + 16) * sizeof(float);
            const int nch = (int)((H + RT_CHUNK - 1) / RT_CHUNK);
            const int cwmax = wg_packed ? std::max(1, 8 / S) : 1;
            const int cpw = (nch + cwmax - 1) / cwmax;
            const int CW = (nch + cpw - 1) / cpw;
            const dim3 blk(64 * (S * CW + (xq ? 1 : 0)));
            const uint16_t *wv = wg_packed ? wg_packed : wg;
            auto go = [&](auto kern) {
                hipLaunchKernelGGL(kern, dim3((unsigned)((T + TP - 1) / TP)), blk, lds, st, xb, wv, T, H, E, k,
                                   renormalize, CW, ids, w, logits, xq, sx);
            };
            if (wg_packed) {
                if (S == 1) go(route_valu_kernel<1, TP, true>);
                else if (S == 2) go(route_valu_kernel<2, TP, true>);
                else go(route_valu_kernel<4, TP, true>);
            } else {
                if (S == 1) go(route_valu_kernel<1, TP, false>);
                else if (S == 2) go(route_valu_kernel<2, TP, false>);
                else go(route_valu_kernel<4, TP, false>);
            }
            return hipGetLastError();
        }
        // up to 128 experts: the K = 1 matrix-core kernel, a wave per run of
        // one or two chunks (with one chunk per wave and two slices, a wave per
        // run and slice; at most 16 waves), on 32-token blocks where they fill
        // the chip, else on 16-token blocks where H spans two chunks or more
        const int nch = (int)((H / 8 + R32_STEPS - 1) / R32_STEPS);
        const int64_t ngrp32 = (T + 31) / 32;
        if (S <= 2 && nch <= 2 * r32_max_waves(S) && (ngrp32 >= 256 || nch >= 2)) {
            const int cpw = nch <= r32_max_waves(S) ? 1 : 2;
            const int ncw = (nch + cpw - 1) / cpw;
            const bool t32 = ngrp32 >= 256;
            // two slices, one chunk per wave: a wave per (run, slice), up to 16
            const bool split = S == 2 && cpw == 1;
            const dim3 g32((unsigned)(t32 ? ngrp32 : (T + 15) / 16)), b32(64 * ncw * (split ? 2 : 1));
            const uint16_t *wv = wg_packed ? wg_packed : wg;
            auto go32 = [&](auto kern) {
                hipLaunchKernelGGL(kern, g32, b32, 0, st, xb, wv, T, H, E, k, renormalize, ncw, ids, w, logits, xq,
                                   sx);
            };
            auto pick = [&](auto tok, auto qx) {
                constexpr int TK = decltype(tok)::value;
                constexpr bool QX = decltype(qx)::value;
                if (split)
                    wg_packed ? go32(route_mfma_k1_kernel<TK, 2, 1, true, QX, true>)
                              : go32(route_mfma_k1_kernel<TK, 2, 1, false, QX, true>);
                else if (S == 1 && cpw == 1)
                    wg_packed ? go32(route_mfma_k1_kernel<TK, 1, 1, true, QX>)
                              : go32(route_mfma_k1_kernel<TK, 1, 1, false, QX>);
                else if (S == 1)
                    wg_packed ? go32(route_mfma_k1_kernel<TK, 1, 2, true, QX>)
                              : go32(route_mfma_k1_kernel<TK, 1, 2, false, QX>);
                else   // two slices, two chunks per wave
                    wg_packed ? go32(route_mfma_k1_kernel<TK, 2, 2, true, QX>)
                              : go32(route_mfma_k1_kernel<TK, 2, 2, false, QX>);
            };
            using T32 = std::integral_constant<int, 32>;
            using T16 = std::integral_constant<int, 16>;
            if (t32) xq ? pick(T32{}, std::true_type{}) : pick(T32{}, std::false_type{});
            else xq ? pick(T16{}, std::true_type{}) : pick(T16{}, std::false_type{});
            return hipGetLastError();
        }
        const int64_t nblk = (T + 32 / S - 1) / (32 / S);
        dim3 g((unsigned)nblk), b(512);
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, g, b, 0, st, xb, wp, T, H, E, k, renormalize, ids, w, logits, xq, sx);
        };
        // 64-wide slices while the blocks fit one per CU; 32-wide (two blocks
        // per CU) beyond
        const bool wide = S <= 2 && nblk <= 256;
        if (S == 1 && wide) wg_f32 ? go(route_mfma_kernel<1, true, 64>) : go(route_mfma_kernel<1, false, 64>);
        else if (S == 1) wg_f32 ? go(route_mfma_kernel<1, true, 32>) : go(route_mfma_kernel<1, false, 32>);
        else if (S == 2 && wide) wg_f32 ? go(route_mfma_kernel<2, true, 64>) : go(route_mfma_kernel<2, false, 64>);
        else if (S == 2) wg_f32 ? go(route_mfma_kernel<2, true, 32>) : go(route_mfma_kernel<2, false, 32>);
        else wg_f32 ? go(route_mfma_kernel<4, true, 32>) : go(route_mfma_kernel<4, false, 32>);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((T + RT_TOK - 1) / RT_TOK)), block(256);
    if (dtype == 0)
        hipLaunchKernelGGL(route_topk_kernel<uint16_t>, grid, block, 0, st, (const uint16_t *)x, wg, T, H, E, k,
                           renormalize, ids, w, logits);
    else
        hipLaunchKernelGGL(route_topk_kernel<float>, grid, block, 0, st, (const float *)x, wg, T, H, E, k,
                           renormalize, ids, w, logits);
    return hipGetLastError();
}

}  // namespace w8a8
