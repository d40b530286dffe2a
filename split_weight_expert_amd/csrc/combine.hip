// Weighted unpermute: y[t] = sum_j w[t,j] * y_perm[inv_perm[t,j]] (+ y_perm[T*k + t]),
// summed in fp32 in slot order, then the shared row, rounded once.  One
// workgroup per token (a bounded grid walks the tokens); each thread owns 8 consecutive columns (16-byte bf16
// vectors) and issues the loads of up to 16 source rows together before summing
// them in slot order.  Entries with inv_perm < 0 (dropped assignments) contribute
// nothing.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace dwdp {
namespace {

constexpr int kMaxK = 64;
#ifndef DWDP_COMBINE_NT
#define DWDP_COMBINE_NT 1
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(const uint4* q) {
    if constexpr (DWDP_COMBINE_NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
        return uint4{v[0], v[1], v[2], v[3]};
    }
    return *q;
}

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint8_t* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ topk_w, int64_t T, int k, int shared,
                                                      int H, int64_t rows, uint8_t* __restrict__ y) {
    __shared__ int32_t s_row[kMaxK];
    __shared__ float s_w[kMaxK];
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        __syncthreads();                                      // the previous token's reads of s_row / s_w are done
        if (threadIdx.x < k) {
            const int32_t p = inv_perm[t * k + threadIdx.x];
            s_row[threadIdx.x] = (p >= 0 && p < rows) ? p : -1;
            s_w[threadIdx.x] = topk_w[t * k + threadIdx.x];
        }
        __syncthreads();
        const int64_t shared_row = T * k + t;
        const int nvec = H / 8;
        const int nsrc = k + (shared ? 1 : 0);                // source rows: the k slots, then the shared row
        constexpr int B = 16;                                 // rows whose loads are in flight together
        for (int c = threadIdx.x; c < nvec; c += 256) {
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int j0 = 0; j0 < nsrc; j0 += B) {
                // all loads of the batch first (a dropped slot loads row 0 and is skipped below) ...
                uint4 raw[BF16 ? B : 2 * B];
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const int j = j0 + u;
                    if (j < nsrc) {
                        const int64_t row = j < k ? (s_row[j] >= 0 ? s_row[j] : 0) : shared_row;
                        // each y_perm element is read once: non-temporal loads (DWDP_COMBINE_NT) stream it
                        if (BF16) {
                            const uint4* q = reinterpret_cast<const uint4*>(y_perm + (row * H + c * 8) * 2);
                            raw[u] = load16(q);
                        } else {
                            const uint4* q = reinterpret_cast<const uint4*>(y_perm + (row * H + c * 8) * 4);
                            raw[2 * u] = load16(q);
                            raw[2 * u + 1] = load16(q + 1);
                        }
                    }
                }
                // ... then the sums, in slot order
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const int j = j0 + u;
                    if (j >= nsrc || (j < k && s_row[j] < 0)) continue;
                    const float wt = j < k ? s_w[j] : 1.0f;
                    if (BF16) {
                        const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[2 * i] += wt * bf16_to_f32((uint16_t)(wd[i] & 0xffffu));
                            acc[2 * i + 1] += wt * bf16_to_f32((uint16_t)(wd[i] >> 16));
                        }
                    } else {
                        const uint32_t wd[8] = {raw[2 * u].x, raw[2 * u].y, raw[2 * u].z, raw[2 * u].w,
                                                raw[2 * u + 1].x, raw[2 * u + 1].y, raw[2 * u + 1].z, raw[2 * u + 1].w};
#pragma unroll
                        for (int i = 0; i < 8; ++i) acc[i] += wt * __uint_as_float(wd[i]);
                    }
                }
            }
            if (BF16) {
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[i] = bf16x2(acc[2 * i], acc[2 * i + 1]);
                *reinterpret_cast<uint4*>(y + (t * H + c * 8) * 2) = uint4{o[0], o[1], o[2], o[3]};
            } else {
                float4* out = reinterpret_cast<float4*>(y + (t * H + c * 8) * 4);
                out[0] = float4{acc[0], acc[1], acc[2], acc[3]};
                out[1] = float4{acc[4], acc[5], acc[6], acc[7]};
            }
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
    const unsigned grid = (unsigned)std::min<int64_t>(T, kMaxRowGrid);
    if (out_dtype == DWDP_BF16)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, as_stream(stream),
                           static_cast<const uint8_t*>(y_perm), inv_perm, topk_w, T, k, shared, H, rows,
                           static_cast<uint8_t*>(y));
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, as_stream(stream),
                           static_cast<const uint8_t*>(y_perm), inv_perm, topk_w, T, k, shared, H, rows,
                           static_cast<uint8_t*>(y));
    DWDP_LAUNCHED();
    return DWDP_OK;
}
