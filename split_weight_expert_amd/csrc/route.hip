// Router: logits = x * W_r^T + b (gemm.hip), then per token the top-k experts and
// their renormalised softmax weights.  The pages give no gate formula; the gate
// here is softmax top-k with the weights renormalised over the chosen k.
//
// Top-k: one wavefront per token.  Lane l holds logits l, l+64, l+128, ...;
// k rounds of (lane-local best, then a 64-lane butterfly max on (value desc,
// index asc)) pick the experts in slot order.  Equal logits go to the lower
// expert index, which makes the selection unique and bitwise reproducible.
#include "common.h"
#include "internal.h"

namespace dwdp {
int router_gemm(const void* x, const void* w, int dtype, const float* bias, int64_t T, int H, int E, float* logits,
                hipStream_t st);

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kPerLane = kMaxE / 64;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
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
    int rc = router_gemm(x, w_router, in_dtype, bias, T, H, E, logits_out, st);
    if (rc != DWDP_OK) return rc;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, logits_out, T, E, k, topk_idx,
                       topk_w);
    DWDP_LAUNCHED();
    return DWDP_OK;
}
