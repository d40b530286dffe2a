// Router: logits = x * W_r^T + b, then per token the top-k experts and their
// renormalised softmax weights.  The pages give no gate formula; the gate here is
// softmax top-k with the weights renormalised over the chosen k.
//
// Logits: prefill batches use the tiled MFMA kernels of gemm.hip.  A decode-sized
// batch (T <= 256 tokens, bf16) would give those only a few workgroups, each
// walking all of K, so it uses a split-K kernel here: 16 x 16 tiles with the K range
// split over the workgroup's 16 waves (router_splitk16_kernel; the 32 x 32 form with
// 8 waves, router_splitk_kernel, is the build option DWDP_ROUTER_SPLITK_TILE=32 and
// took the 64-token route stage 47 us against 29 us), partial tiles summed through
// LDS in wave order (a fixed order, so the logits are reproducible bit for bit).
//
// Top-k: one wavefront per token.  Lane l holds logits l, l+64, l+128, ...;
// k rounds of (lane-local best, then a 64-lane butterfly max on (value desc,
// index asc)) pick the experts in slot order.  Equal logits go to the lower
// expert index, which makes the selection unique and bitwise reproducible.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace dwdp {
int router_gemm(const void* x, const void* w, int dtype, const float* bias, int64_t T, int H, int E, float* logits,
                hipStream_t st);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSplitMaxT = 256;    // batches up to this many tokens take the split-K router
constexpr int kSplitWaves = 8;

// logits[T, E] for one 32-token x 32-expert tile.  Wave w multiplies K columns [w H/8, (w+1) H/8)
// with v_mfma_f32_32x32x16_bf16, operands loaded straight from global memory (lane l: row l % 32,
// 8 columns at 8 (l / 32)); rows past T or E are clamped for loads and skipped for stores.
__global__ __launch_bounds__(kSplitWaves * 64) void router_splitk_kernel(const uint16_t* __restrict__ x,
                                                                        const uint16_t* __restrict__ wr,
                                                                        const float* __restrict__ bias, int T,
                                                                        int H, int E, float* __restrict__ logits) {
    __shared__ float part[kSplitWaves][64][17];   // 17: consecutive lanes fall on different banks
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, hi = lane >> 5;
    const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
    const uint16_t* arow = x + (size_t)min(m0 + l32, T - 1) * H + hi * 8;
    const uint16_t* brow = wr + (size_t)min(n0 + l32, E - 1) * H + hi * 8;
    const int kw = H / kSplitWaves;
    const int kb = wave * kw, ke = kb + kw;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    constexpr int U = 8;                           // K16 steps per batch of loads
    int k = kb;
    for (; k + 16 * U <= ke; k += 16 * U) {
        bf16x8 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = *reinterpret_cast<const bf16x8*>(arow + k + 16 * u);
            b[u] = *reinterpret_cast<const bf16x8*>(brow + k + 16 * u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], acc, 0, 0, 0);
    }
    for (; k < ke; k += 16) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + k);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(brow + k);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    // element r of lane (l32, hi): token m0 + 8 (r / 4) + 4 hi + r % 4, expert n0 + l32
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave][lane][r] = acc[r];
    __syncthreads();
    if (wave == 0) {
        const int e = n0 + l32;
        const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = part[0][lane][r];
#pragma unroll
            for (int w = 1; w < kSplitWaves; ++w) s += part[w][lane][r];
            const int t = m0 + (r >> 2) * 8 + hi * 4 + (r & 3);
            if (t < T && e < E) logits[(size_t)t * E + e] = s + b;
        }
    }
}

// The same with 16 x 16 tiles (v_mfma_f32_16x16x32_bf16) and the K range split over 16 waves: four
// times the workgroups of the 32 x 32 form, so a 64-token batch spreads its loads over 64 compute
// units instead of 16, and each wave walks H/16 columns in batches of 8 K steps.  Wave w takes the
// 32-column K steps [w S / 16, (w+1) S / 16) of the S = H / 32 (any H % 32 == 0).  Operand lanes:
// row (or expert) l % 16, 8 columns at 8 (l / 16) of the step; result element r of lane l: token
// m0 + 4 (l / 16) + r, expert n0 + l % 16.  Partials are summed through LDS in wave order.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kSplit16Waves = 16;

__global__ __launch_bounds__(kSplit16Waves * 64) void router_splitk16_kernel(const uint16_t* __restrict__ x,
                                                                            const uint16_t* __restrict__ wr,
                                                                            const float* __restrict__ bias, int T,
                                                                            int H, int E,
                                                                            float* __restrict__ logits) {
    __shared__ float part[kSplit16Waves][64][5];   // 5: consecutive lanes fall on different banks
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, q = lane >> 4;
    const int m0 = blockIdx.x * 16, n0 = blockIdx.y * 16;
    const uint16_t* arow = x + (size_t)min(m0 + l16, T - 1) * H + q * 8;
    const uint16_t* brow = wr + (size_t)min(n0 + l16, E - 1) * H + q * 8;
    const int steps = H / 32;
    const int sb = wave * steps / kSplit16Waves, se = (wave + 1) * steps / kSplit16Waves;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int U = 8;                           // K steps per batch of loads
    for (int s0 = sb; s0 < se; s0 += U) {
        bf16x8 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s0 + u < se) {
                a[u] = *reinterpret_cast<const bf16x8*>(arow + (s0 + u) * 32);
                b[u] = *reinterpret_cast<const bf16x8*>(brow + (s0 + u) * 32);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s0 + u < se) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][lane][r] = acc[r];
    __syncthreads();
    if (wave == 0) {
        const int e = n0 + l16;
        const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s = part[0][lane][r];
            for (int w = 1; w < kSplit16Waves; ++w) s += part[w][lane][r];
            const int t = m0 + q * 4 + r;
            if (t < T && e < E) logits[(size_t)t * E + e] = s + b;
        }
    }
}

#ifndef DWDP_ROUTER_SPLITK_TILE
#define DWDP_ROUTER_SPLITK_TILE 16
#endif

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// PL logits per lane (E <= 64 PL): the per-lane scan of every round walks only the slots E needs.
template <int PL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
    constexpr int kPerLane = PL;
    const int lane = threadIdx.x & 63;
    for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += (int64_t)gridDim.x * 4) {
        const float* row = logits + t * E;
        float v[kPerLane];
        bool live[kPerLane];
#pragma unroll
        for (int s = 0; s < kPerLane; ++s) {
            const int e = lane + 64 * s;
            live[s] = e < E;
            v[s] = live[s] ? row[e] : 0.0f;
        }
        // round j picks slot j; lane j keeps it
        float my_v = 0.0f, top_v = 0.0f;
        int my_i = 0;
        for (int j = 0; j < k; ++j) {
            float bv = 0.0f;
            int bi = 0x7fffffff;
#pragma unroll
            for (int s = 0; s < kPerLane; ++s) {
                const int e = lane + 64 * s;
                if (live[s] && (bi == 0x7fffffff || better(v[s], e, bv, bi))) {
                    bv = v[s];
                    bi = e;
                }
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const float ov = __shfl_xor(bv, d);
                const int oi = __shfl_xor(bi, d);
                if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (j == 0) top_v = bv;
            if (lane == j) {
                my_v = bv;
                my_i = bi;
            }
#pragma unroll
            for (int s = 0; s < kPerLane; ++s)
                if (lane + 64 * s == bi) live[s] = false;
        }
        // weights: softmax over the chosen k, shifted by the largest; summed in slot order
        const float ex = lane < k ? expf(my_v - top_v) : 0.0f;
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) sum += __shfl(ex, j);
        if (lane < k) {
            idx[t * k + lane] = my_i;
            w[t * k + lane] = ex / sum;
        }
    }
}

}  // namespace
}  // namespace dwdp

using namespace dwdp;

extern "C" int dwdp_route_topk(const void* x, const void* w_router, int in_dtype, const float* bias, int64_t T, int H,
                               int E, int k, float* logits_out, int32_t* topk_idx, float* topk_w, void* stream) {
    clear_error();
    DWDP_REQUIRE(in_dtype == DWDP_F32 || in_dtype == DWDP_BF16, "in_dtype must be DWDP_F32 or DWDP_BF16");
    DWDP_REQUIRE(T >= 0 && T < ((int64_t)1 << 31), "T out of range");
    DWDP_REQUIRE(E >= 1 && E <= kMaxE, "E must be in [1, 1024]");
    DWDP_REQUIRE(k >= 1 && k <= E && k <= kMaxK, "k must be in [1, min(E, 32)]");
    DWDP_REQUIRE(H > 0, "H must be positive");
    if (in_dtype == DWDP_BF16) DWDP_REQUIRE(H % 64 == 0, "bf16 routing needs H % 64 == 0");
    else DWDP_REQUIRE(H % 16 == 0, "f32 routing needs H % 16 == 0");
    if (T == 0) return DWDP_OK;
    DWDP_REQUIRE(x && w_router && logits_out && topk_idx && topk_w, "null pointer argument");
    DWDP_REQUIRE(aligned16(x) && aligned16(w_router), "x and w_router must be 16-byte aligned");
    hipStream_t st = as_stream(stream);
    if (DWDP_ROUTER_SPLITK_TILE == 16 && in_dtype == DWDP_BF16 && T <= kSplitMaxT) {
        hipLaunchKernelGGL(router_splitk16_kernel, dim3((unsigned)((T + 15) / 16), (unsigned)((E + 15) / 16)),
                           dim3(kSplit16Waves * 64), 0, st, static_cast<const uint16_t*>(x),
                           static_cast<const uint16_t*>(w_router), bias, (int)T, H, E, logits_out);
        DWDP_LAUNCHED();
    } else if (in_dtype == DWDP_BF16 && T <= kSplitMaxT && H % (kSplitWaves * 16) == 0) {
        hipLaunchKernelGGL(router_splitk_kernel, dim3((unsigned)((T + 31) / 32), (unsigned)((E + 31) / 32)),
                           dim3(kSplitWaves * 64), 0, st, static_cast<const uint16_t*>(x),
                           static_cast<const uint16_t*>(w_router), bias, (int)T, H, E, logits_out);
        DWDP_LAUNCHED();
    } else {
        int rc = router_gemm(x, w_router, in_dtype, bias, T, H, E, logits_out, st);
        if (rc != DWDP_OK) return rc;
    }
    const dim3 tgrid((unsigned)std::min<int64_t>((T + 3) / 4, kMaxRowGrid));
    if (E <= 64) hipLaunchKernelGGL(topk_kernel<1>, tgrid, dim3(256), 0, st, logits_out, T, E, k, topk_idx, topk_w);
    else if (E <= 128) hipLaunchKernelGGL(topk_kernel<2>, tgrid, dim3(256), 0, st, logits_out, T, E, k, topk_idx, topk_w);
    else if (E <= 256) hipLaunchKernelGGL(topk_kernel<4>, tgrid, dim3(256), 0, st, logits_out, T, E, k, topk_idx, topk_w);
    else if (E <= 512) hipLaunchKernelGGL(topk_kernel<8>, tgrid, dim3(256), 0, st, logits_out, T, E, k, topk_idx, topk_w);
    else hipLaunchKernelGGL(topk_kernel<kMaxE / 64>, tgrid, dim3(256), 0, st, logits_out, T, E, k, topk_idx, topk_w);
    DWDP_LAUNCHED();
    return DWDP_OK;
}
