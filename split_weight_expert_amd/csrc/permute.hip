// Permutation of the routed (token, slot) pairs by expert -- a counting sort
// that is stable in the flattened index t*k+j -- and the row gather that
// builds x_perm, optionally quantising each row to fp8 E4M3 per 128 columns.
//
//   count    one workgroup per expert, 16 waves; wave w scans a fixed slice of
//            topk_idx, each lane 16 consecutive entries, and counts matches
//   offsets  one workgroup: per-expert totals, their exclusive scan (the group
//            row offsets) and the base row of every (expert, wave) slice
//   scatter  the count walk again, now with a 64-lane prefix scan of the
//            per-lane match counts: rank = slice base + lanes before + matches
//            before inside the lane, which keeps the t*k+j order
//   gather   one workgroup per x_perm row: bitwise row copy, or per-row fp8
//            quantisation (scale = amax/448 over 128 columns, code = E4M3(v/s))
// No atomics are involved, so every output is bitwise reproducible.
#include "common.h"
#include "internal.h"

namespace dwdp {
namespace {

constexpr int kWaves = kPermuteWaves;   // waves per count / scatter workgroup
constexpr int kPerLane = 16;        // consecutive entries per lane per step
constexpr int kStep = 64 * kPerLane;

__device__ __forceinline__ void load16(const int32_t* __restrict__ idx, int64_t first, int64_t lo, int64_t hi,
                                       int32_t (&v)[kPerLane]) {
    if (first >= lo && first + kPerLane <= hi) {
        const int4* p = reinterpret_cast<const int4*>(idx + first);
#pragma unroll
        for (int q = 0; q < kPerLane / 4; ++q) {
            const int4 x = p[q];
            v[4 * q] = x.x;
            v[4 * q + 1] = x.y;
            v[4 * q + 2] = x.z;
            v[4 * q + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) {
            const int64_t f = first + q;
            v[q] = (f >= lo && f < hi) ? idx[f] : -1;
        }
    }
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    return v;
}

__global__ __launch_bounds__(1024) void count_kernel(const int32_t* __restrict__ idx, int64_t N, int64_t seg,
                                                     int32_t* __restrict__ wave_counts) {
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t lo = (int64_t)w * seg, hi = min(N, lo + seg);
    int c = 0;
    for (int64_t cb = lo; cb < hi; cb += kStep) {
        int32_t v[kPerLane];
        load16(idx, cb + (int64_t)lane * kPerLane, lo, hi, v);
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) c += v[q] == e;
    }
    c = wave_sum(c);
    if (lane == 0) wave_counts[e * kWaves + w] = c;
}

__global__ __launch_bounds__(1024) void offsets_kernel(const int32_t* __restrict__ wave_counts, int E, int shared,
                                                       int64_t T, int64_t R, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ wave_base, int32_t* __restrict__ perm_src) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < E; base += 1024) {
        const int e = base + tid;
        int tot = 0;
        if (e < E)
            for (int w = 0; w < kWaves; ++w) tot += wave_counts[e * kWaves + w];
        const int incl = wave_incl_scan(tot, lane);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int before = carry_s;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        const int excl = before + incl - tot;
        if (e < E) {
            offsets[e] = excl;
            int b = excl;
            for (int w = 0; w < kWaves; ++w) {
                wave_base[e * kWaves + w] = b;
                b += wave_counts[e * kWaves + w];
            }
        }
        __syncthreads();
        if (tid == 0) {
            int s = 0;
            for (int w = 0; w < 16; ++w) s += wsum[w];
            carry_s += s;
        }
        __syncthreads();
    }
    if (tid == 0) {
        offsets[E] = (int32_t)R;                 // equals the count total when every index is valid
        if (shared) offsets[E + 1] = (int32_t)(R + T);
    }
    // Rows of dropped entries (indices outside [0, E)): the count total falls short of R by their
    // number, and rows [total, R) close the last routed group.  They read token 0, so every row the
    // grouped FFN computes has a defined source; the combine never reads them (their inv_perm is -1).
    for (int64_t r = (int64_t)carry_s + tid; r < R; r += 1024) perm_src[r] = 0;
}

__global__ __launch_bounds__(1024) void scatter_kernel(const int32_t* __restrict__ idx, int64_t N, int k, int E,
                                                       int64_t seg, const int32_t* __restrict__ wave_base,
                                                       int32_t* __restrict__ perm_src, int32_t* __restrict__ inv_perm) {
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t lo = (int64_t)w * seg, hi = min(N, lo + seg);
    int base = wave_base[e * kWaves + w];
    for (int64_t cb = lo; cb < hi; cb += kStep) {
        const int64_t first = cb + (int64_t)lane * kPerLane;
        int32_t v[kPerLane];
        load16(idx, first, lo, hi, v);
        int c = 0;
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) c += v[q] == e;
        const int incl = wave_incl_scan(c, lane);
        int pos = base + incl - c;
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) {
            if (v[q] == e) {
                perm_src[pos] = (int32_t)((first + q) / k);
                inv_perm[first + q] = pos;
                ++pos;
            } else if (e == 0 && (v[q] < 0 || v[q] >= E) && first + q >= lo && first + q < hi) {
                inv_perm[first + q] = -1;        // out-of-range expert index: dropped
            }
        }
        base += __shfl(incl, 63);
    }
}

// Row gather.  One workgroup (256 threads) per x_perm row, 16-byte vectors.
__global__ __launch_bounds__(256) void gather_copy_kernel(const uint8_t* __restrict__ x, int64_t T, int64_t R,
                                                          int64_t row_bytes, int32_t* __restrict__ perm_src,
                                                          uint8_t* __restrict__ x_perm) {
    const int64_t r = blockIdx.x;
    int64_t src;
    if (r < R) {
        src = perm_src[r];
    } else {
        src = r - R;
        if (threadIdx.x == 0) perm_src[r] = (int32_t)src;
    }
    const bool ok = src >= 0 && src < T;
    const uint4* in = reinterpret_cast<const uint4*>(x + (ok ? src : 0) * row_bytes);
    uint4* out = reinterpret_cast<uint4*>(x_perm + r * row_bytes);
    const int64_t nvec = row_bytes / 16;
    for (int64_t i = threadIdx.x; i < nvec; i += 256) out[i] = ok ? in[i] : uint4{0, 0, 0, 0};
}

// Shared-expert rows of perm_src (token t at row R + t) when no rows are gathered.
__global__ __launch_bounds__(256) void shared_rows_kernel(int32_t* __restrict__ perm_src, int64_t R, int64_t T) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < T) perm_src[R + t] = (int32_t)t;
}

// fp8 gather: 16 lanes per 128-column group, 8 bf16 values (16 bytes) per lane.  perm_src == NULL
// quantises x row by row (output row r = token r).
__global__ __launch_bounds__(256) void gather_fp8_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t R, int H,
                                                         int32_t* __restrict__ perm_src, uint8_t* __restrict__ q,
                                                         float* __restrict__ qs) {
    const int64_t r = blockIdx.x;
    int64_t src;
    if (r < R) {
        src = perm_src[r];
    } else {
        src = r - R;
        if (perm_src != nullptr && threadIdx.x == 0) perm_src[r] = (int32_t)src;
    }
    const bool ok = src >= 0 && src < T;
    const int G = H / kFp8Group;
    const int sub = threadIdx.x & 15;
    for (int g = threadIdx.x >> 4; g < G; g += 16) {
        float v[8];
        if (ok) {
            const uint4 raw = *reinterpret_cast<const uint4*>(x + src * H + g * kFp8Group + sub * 8);
            const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_to_f32((uint16_t)(wds[i] & 0xffffu));
                v[2 * i + 1] = bf16_to_f32((uint16_t)(wds[i] >> 16));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        }
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 16));
        const float s = m == 0.0f ? 1.0f : m / 448.0f;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo |= (uint32_t)f32_to_e4m3(v[i] / s) << (8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) hi |= (uint32_t)f32_to_e4m3(v[4 + i] / s) << (8 * i);
        *reinterpret_cast<uint2*>(q + r * H + g * kFp8Group + sub * 8) = uint2{lo, hi};
        if (sub == 0) qs[r * G + g] = s;
    }
}

}  // namespace

}  // namespace dwdp

using namespace dwdp;

extern "C" int dwdp_permute(const int32_t* topk_idx, int64_t T, int k, int E, int shared, const void* x, int x_dtype,
                            int act_dtype, int H, void* x_perm, float* x_perm_scale, int32_t* offsets,
                            int32_t* perm_src, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    DWDP_REQUIRE(T >= 0 && k >= 1 && E >= 1 && (shared == 0 || shared == 1), "bad T, k, E or shared");
    DWDP_REQUIRE(E <= 65536, "E must be at most 65536");
    DWDP_REQUIRE(T * (k + shared) < ((int64_t)1 << 31), "T*(k+shared) must fit in int32");
    DWDP_REQUIRE(x_dtype == DWDP_F32 || x_dtype == DWDP_BF16, "x_dtype must be DWDP_F32 or DWDP_BF16");
    DWDP_REQUIRE(act_dtype == x_dtype || (act_dtype == DWDP_FP8_E4M3 && x_dtype == DWDP_BF16),
                 "act_dtype must equal x_dtype, or be DWDP_FP8_E4M3 with bf16 x");
    DWDP_REQUIRE(H > 0 && (H * elem_bytes(x_dtype)) % 16 == 0, "H * element size must be a multiple of 16");
    if (act_dtype == DWDP_FP8_E4M3) DWDP_REQUIRE(H % kFp8Group == 0, "fp8 quantisation needs H % 128 == 0");
    DWDP_REQUIRE(offsets != nullptr, "offsets is NULL");
    const size_t need = permute_ws_bytes(T, k, E);
    if (T == 0) return DWDP_OK;
    DWDP_REQUIRE(topk_idx && perm_src && inv_perm && ws, "null pointer argument");
    const bool gather = x_perm != nullptr;
    if (gather) {
        DWDP_REQUIRE(x != nullptr, "x is NULL");
        DWDP_REQUIRE(aligned16(x) && aligned16(x_perm), "x and x_perm must be 16-byte aligned");
        if (act_dtype == DWDP_FP8_E4M3) DWDP_REQUIRE(x_perm_scale != nullptr, "fp8 needs x_perm_scale");
    }
    DWDP_REQUIRE(aligned16(topk_idx) && aligned16(ws), "topk_idx and ws must be 16-byte aligned");
    if (ws_bytes < need) return fail(DWDP_ERR_WORKSPACE, "dwdp_permute: workspace too small");
    hipStream_t st = as_stream(stream);
    const int64_t N = T * k, R = N, rows = R + shared * T;
    const int64_t seg = ((N + kWaves - 1) / kWaves + kStep - 1) / kStep * kStep;
    int32_t* wave_counts = static_cast<int32_t*>(ws);
    int32_t* wave_base = wave_counts + (size_t)E * kWaves;
    hipLaunchKernelGGL(count_kernel, dim3(E), dim3(1024), 0, st, topk_idx, N, seg, wave_counts);
    hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(1024), 0, st, wave_counts, E, shared, T, R, offsets, wave_base,
                       perm_src);
    hipLaunchKernelGGL(scatter_kernel, dim3(E), dim3(1024), 0, st, topk_idx, N, k, E, seg, wave_base, perm_src, inv_perm);
    if (!gather) {
        if (shared) hipLaunchKernelGGL(shared_rows_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, perm_src, R, T);
    } else if (act_dtype == DWDP_FP8_E4M3) {
        hipLaunchKernelGGL(gather_fp8_kernel, dim3((unsigned)rows), dim3(256), 0, st,
                           static_cast<const uint16_t*>(x), T, R, H, perm_src, static_cast<uint8_t*>(x_perm),
                           x_perm_scale);
    } else {
        hipLaunchKernelGGL(gather_copy_kernel, dim3((unsigned)rows), dim3(256), 0, st, static_cast<const uint8_t*>(x), T,
                           R, (int64_t)H * (int64_t)elem_bytes(x_dtype), perm_src, static_cast<uint8_t*>(x_perm));
    }
    DWDP_LAUNCHED();
    return DWDP_OK;
}

extern "C" int dwdp_quantize_tokens_fp8(const void* x, int64_t T, int H, void* q, float* q_scale, void* stream) {
    clear_error();
    DWDP_REQUIRE(T >= 0 && T < ((int64_t)1 << 31), "T out of range");
    DWDP_REQUIRE(H > 0 && H % kFp8Group == 0, "H must be a positive multiple of 128");
    if (T == 0) return DWDP_OK;
    DWDP_REQUIRE(x && q && q_scale, "null pointer argument");
    DWDP_REQUIRE(aligned16(x) && aligned16(q), "x and q must be 16-byte aligned");
    hipLaunchKernelGGL(gather_fp8_kernel, dim3((unsigned)T), dim3(256), 0, as_stream(stream),
                       static_cast<const uint16_t*>(x), T, (int64_t)0, H, static_cast<int32_t*>(nullptr),
                       static_cast<uint8_t*>(q), q_scale);
    DWDP_LAUNCHED();
    return DWDP_OK;
}
