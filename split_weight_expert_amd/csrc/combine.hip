// Weighted unpermute: y[t] = sum_j w[t,j] * y_perm[inv_perm[t,j]] (+ y_perm[T*k + t]),
// summed in fp32 in slot order, then the shared row, rounded once.  One
// workgroup per token; each thread owns 8 consecutive columns (16-byte bf16
// vectors).  Entries with inv_perm < 0 (dropped assignments) contribute nothing.
#include "common.h"
#include "internal.h"

namespace dwdp {
namespace {

constexpr int kMaxK = 64;

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint8_t* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ topk_w, int64_t T, int k, int shared,
                                                      int H, int64_t rows, uint8_t* __restrict__ y) {
    const int64_t t = blockIdx.x;
    __shared__ int32_t s_row[kMaxK];
    __shared__ float s_w[kMaxK];
    if (threadIdx.x < k) {
        const int32_t p = inv_perm[t * k + threadIdx.x];
        s_row[threadIdx.x] = (p >= 0 && p < rows) ? p : -1;
        s_w[threadIdx.x] = topk_w[t * k + threadIdx.x];
    }
    __syncthreads();
    const int64_t shared_row = T * k + t;
    const int nvec = H / 8;
    for (int c = threadIdx.x; c < nvec; c += 256) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        auto add_row = [&](int64_t row, float wt) {
            if (BF16) {
                const uint4 raw = *reinterpret_cast<const uint4*>(y_perm + (row * H + c * 8) * 2);
                const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += wt * bf16_to_f32((uint16_t)(wd[i] & 0xffffu));
                    acc[2 * i + 1] += wt * bf16_to_f32((uint16_t)(wd[i] >> 16));
                }
            } else {
                const float4* p = reinterpret_cast<const float4*>(y_perm + (row * H + c * 8) * 4);
                const float4 a = p[0], b = p[1];
                const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += wt * v[i];
            }
        };
        for (int j = 0; j < k; ++j)
            if (s_row[j] >= 0) add_row(s_row[j], s_w[j]);
        if (shared) add_row(shared_row, 1.0f);
        if (BF16) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16);
            *reinterpret_cast<uint4*>(y + (t * H + c * 8) * 2) = uint4{o[0], o[1], o[2], o[3]};
        } else {
            float4* out = reinterpret_cast<float4*>(y + (t * H + c * 8) * 4);
            out[0] = float4{acc[0], acc[1], acc[2], acc[3]};
            out[1] = float4{acc[4], acc[5], acc[6], acc[7]};
        }
    }
}

}  // namespace
}  // namespace dwdp

using namespace dwdp;

extern "C" int dwdp_combine(const void* y_perm, const int32_t* inv_perm, const float* topk_w, int64_t T, int k,
                            int shared, int H, int out_dtype, void* y, void* stream) {
    clear_error();
    DWDP_REQUIRE(out_dtype == DWDP_F32 || out_dtype == DWDP_BF16, "out_dtype must be DWDP_F32 or DWDP_BF16");
    DWDP_REQUIRE(T >= 0 && T < ((int64_t)1 << 31), "T out of range");
    DWDP_REQUIRE(k >= 1 && k <= kMaxK, "k must be in [1, 64]");
    DWDP_REQUIRE(shared == 0 || shared == 1, "shared must be 0 or 1");
    DWDP_REQUIRE(H > 0 && H % 8 == 0, "H must be a positive multiple of 8");
    if (T == 0) return DWDP_OK;
    DWDP_REQUIRE(y_perm && inv_perm && topk_w && y, "null pointer argument");
    DWDP_REQUIRE(aligned16(y_perm) && aligned16(y), "y_perm and y must be 16-byte aligned");
    const int64_t rows = T * k + shared * T;
    if (out_dtype == DWDP_BF16)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)T), dim3(256), 0, as_stream(stream),
                           static_cast<const uint8_t*>(y_perm), inv_perm, topk_w, T, k, shared, H, rows,
                           static_cast<uint8_t*>(y));
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)T), dim3(256), 0, as_stream(stream),
                           static_cast<const uint8_t*>(y_perm), inv_perm, topk_w, T, k, shared, H, rows,
                           static_cast<uint8_t*>(y));
    DWDP_LAUNCHED();
    return DWDP_OK;
}
