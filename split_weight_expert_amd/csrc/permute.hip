// Permutation of the routed (token, slot) pairs by expert -- a counting sort
// that is stable in the flattened index t*k+j -- and the row gather that
// builds x_perm, optionally quantising each row to fp8 E4M3 per 128 columns.
//
// Up to kHistMaxE experts the sort works on chunk histograms, O(T*k) work:
//   chunk_count    one wave per chunk of consecutive entries: its expert
//                  histogram in LDS, written out as row c of [chunks][E]
//   chunk_offsets  one workgroup: per-expert totals, their exclusive scan (the
//                  group row offsets), and the histogram rewritten in place as
//                  the first row of every (chunk, expert) pair
//   chunk_scatter  each wave walks its chunk again, 64 entries at a time; the
//                  lanes that hold the same expert find each other with one
//                  ballot per bit of the expert index, so an entry's row is its
//                  (chunk, expert) base + entries of that expert before it in
//                  the chunk, which keeps the t*k+j order
// Above kHistMaxE (the histograms would not fit in LDS) one workgroup per
// expert scans all entries, O(E*T*k):
//   count    16 waves; wave w scans a fixed slice of topk_idx, each lane 16
//            consecutive entries, and counts matches
//   offsets  one workgroup: per-expert totals, their exclusive scan and the base
//            row of every (expert, wave) slice
//   scatter  the count walk again, now with a 64-lane prefix scan of the
//            per-lane match counts: rank = slice base + lanes before + matches
//            before inside the lane
//   gather   one workgroup per x_perm row: bitwise row copy, or per-row fp8
//            quantisation (scale = amax/448 over 128 columns, code = E4M3(v/s))
// Every output is bitwise reproducible: the only atomics add integers in LDS.
#include <algorithm>

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

// ---------------------------------------------------------------- chunk histograms (E <= kHistMaxE)
constexpr int kHistWaves = 4;   // chunks (waves) per workgroup

// Row c of hist [chunks][E]: how many entries of chunk c name each expert (entries outside [0, E)
// are dropped and counted nowhere).
__global__ __launch_bounds__(256) void chunk_count_kernel(const int32_t* __restrict__ idx, int64_t N, int E,
                                                          int64_t chunk, int64_t C, int32_t* __restrict__ hist) {
    __shared__ int32_t cnt_s[kHistWaves * kHistMaxE];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * kHistWaves + w;
    int32_t* cnt = cnt_s + w * E;
    for (int e = lane; e < E; e += 64) cnt[e] = 0;
    __syncthreads();
    if (c < C) {
        const int64_t lo = c * chunk, hi = min(N, lo + chunk);
        for (int64_t i = lo + lane; i < hi; i += 64) {
            const int v = idx[i];
            if (v >= 0 && v < E) atomicAdd(&cnt[v], 1);
        }
    }
    __syncthreads();
    if (c < C)
        for (int e = lane; e < E; e += 64) hist[c * E + e] = cnt[e];
}

// offsets[e] = exclusive scan of the expert totals; hist[c][e] becomes the first row of chunk c's
// entries of expert e (offsets[e] + the entries of e in chunks before c).  Experts are taken EB at a
// time, and the chunks of each expert are split into P = 1024 / EB segments with a thread each, so that
// a thread's loads are a few batches of independent ones rather than one chain over all chunks.
constexpr int kOffBatch = 16;
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(int32_t* __restrict__ hist, int64_t C, int E, int shared,
                                                             int64_t T, int64_t R, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm_src) {
    __shared__ int part_s[1024];     // segment sums, [segment][expert of the block]
    __shared__ int excl_s[1024];     // offsets of the block's experts
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = E >= 1024 ? 1 : 1024 / E, EB = 1024 / P;
    const int sg = tid / EB, el = tid % EB;
    const int64_t SC = (C + P - 1) / P;                     // chunks per segment
    const int64_t c_lo = min(C, (int64_t)sg * SC), c_hi = min(C, c_lo + SC);
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < E; base += EB) {
        const int e = base + el;
        const bool mine = sg < P && e < E;
        int sum = 0;
        if (mine) {
            for (int64_t c0 = c_lo; c0 < c_hi; c0 += kOffBatch) {
                int h[kOffBatch];
#pragma unroll
                for (int q = 0; q < kOffBatch; ++q) h[q] = c0 + q < c_hi ? hist[(c0 + q) * E + e] : 0;
#pragma unroll
                for (int q = 0; q < kOffBatch; ++q) sum += h[q];
            }
        }
        part_s[tid] = sum;
        __syncthreads();
        int tot = 0;                                       // thread el < EB of segment 0 holds expert el's total
        if (sg == 0 && e < E)
            for (int q = 0; q < P; ++q) tot += part_s[q * EB + el];
        const int incl = wave_incl_scan(tot, lane);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int before = carry_s;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        if (sg == 0) {
            const int excl = before + incl - tot;
            excl_s[el] = excl;
            if (e < E) offsets[e] = excl;
        }
        __syncthreads();
        if (mine) {
            int run = excl_s[el];
            for (int q = 0; q < sg; ++q) run += part_s[q * EB + el];
            for (int64_t c0 = c_lo; c0 < c_hi; c0 += kOffBatch) {
                int h[kOffBatch];
#pragma unroll
                for (int q = 0; q < kOffBatch; ++q) h[q] = c0 + q < c_hi ? hist[(c0 + q) * E + e] : 0;
#pragma unroll
                for (int q = 0; q < kOffBatch; ++q) {
                    if (c0 + q < c_hi) hist[(c0 + q) * E + e] = run;
                    run += h[q];
                }
            }
        }
        __syncthreads();
        if (tid == 0) {
            int total = 0;
            for (int w = 0; w < 16; ++w) total += wsum[w];
            carry_s += total;
        }
        __syncthreads();
    }
    if (tid == 0) {
        offsets[E] = (int32_t)R;                 // equals the count total when every index is valid
        if (shared) offsets[E + 1] = (int32_t)(R + T);
    }
    // rows of dropped entries close the last routed group and read token 0 (as in offsets_kernel)
    for (int64_t r = (int64_t)carry_s + tid; r < R; r += 1024) perm_src[r] = 0;
}

// ebits: bits that tell apart the keys 0 .. E (E stands for every entry outside [0, E)).
__global__ __launch_bounds__(256) void chunk_scatter_kernel(const int32_t* __restrict__ idx, int64_t N, int k, int E,
                                                            int ebits, int64_t chunk, int64_t C,
                                                            const int32_t* __restrict__ first_row, int64_t R,
                                                            int32_t* __restrict__ perm_src,
                                                            int32_t* __restrict__ inv_perm) {
    __shared__ int32_t next_s[kHistWaves * kHistMaxE];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * kHistWaves + w;
    int32_t* next = next_s + w * E;               // next free row of each expert in this chunk
    if (c < C)
        for (int e = lane; e < E; e += 64) next[e] = first_row[c * E + e];
    __syncthreads();
    if (c >= C) return;
    const int64_t lo = c * chunk, hi = min(N, lo + chunk);
    const uint64_t below = (1ull << lane) - 1;    // lanes before this one
    for (int64_t i0 = lo; i0 < hi; i0 += 64) {    // uniform trip count: every lane takes part in the ballots
        const int64_t i = i0 + lane;
        const bool in = i < hi;
        const int v = in ? idx[i] : -1;
        const bool ok = v >= 0 && v < E;
        const int key = ok ? v : E;
        uint64_t same = ~0ull;                    // lanes whose key equals this lane's
        for (int b = 0; b < ebits; ++b) {
            const bool bit = (key >> b) & 1;
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        if (ok) {
            // one LDS read per lane, then the group's last lane moves the counter past the group (the
            // wave's LDS operations complete in order, so every read sees the value before the write)
            const int pos = next[v] + __popcll(same & below);
            if (pos < R) {
                perm_src[pos] = (int32_t)(i / k);
                inv_perm[i] = pos;
            }
            if ((same >> lane) == 1ull) next[v] = pos + 1;
        } else if (in) {
            inv_perm[i] = -1;                     // out-of-range expert index: dropped
        }
    }
}

// Row gather.  One workgroup (256 threads) per x_perm row (a bounded grid walks the rows), 16-byte vectors.
__global__ __launch_bounds__(256) void gather_copy_kernel(const uint8_t* __restrict__ x, int64_t T, int64_t R,
                                                          int64_t rows, int64_t row_bytes, int32_t* __restrict__ perm_src,
                                                          uint8_t* __restrict__ x_perm) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
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
}

// Shared-expert rows of perm_src (token t at row R + t) when no rows are gathered.
__global__ __launch_bounds__(256) void shared_rows_kernel(int32_t* __restrict__ perm_src, int64_t R, int64_t T) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < T) perm_src[R + t] = (int32_t)t;
}

// fp8 gather: 16 lanes per 128-column group, 8 bf16 values (16 bytes) per lane; the 16 lane groups of
// the workgroup take the row's column groups in batches of 4 each (all 4 loads issued before the first
// is used, so a 7168-wide row costs one memory round trip, not four).  perm_src == NULL quantises x row
// by row (output row r = token r).
__global__ __launch_bounds__(256) void gather_fp8_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t R,
                                                         int64_t rows, int H, int32_t* __restrict__ perm_src,
                                                         uint8_t* __restrict__ q, float* __restrict__ qs) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
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
        constexpr int U = 4;
        for (int g0 = threadIdx.x >> 4; g0 < G; g0 += 16 * U) {
            uint4 raw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = g0 + 16 * u;
                raw[u] = (ok && g < G) ? *reinterpret_cast<const uint4*>(x + src * H + g * kFp8Group + sub * 8)
                                       : uint4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = g0 + 16 * u;
                if (g >= G) break;                 // the same for all 16 lanes of the group
                float v[8];
                const uint32_t wds[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = bf16_to_f32((uint16_t)(wds[i] & 0xffffu));
                    v[2 * i + 1] = bf16_to_f32((uint16_t)(wds[i] >> 16));
                }
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
                for (int d = 8; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 16));
                const float s = m == 0.0f ? 1.0f : m / 448.0f;
                const uint32_t lo = e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
                const uint32_t hi = e4m3x4(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
                *reinterpret_cast<uint2*>(q + r * H + g * kFp8Group + sub * 8) = uint2{lo, hi};
                if (sub == 0) qs[r * G + g] = s;
            }
        }
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
    const unsigned row_grid = (unsigned)std::min<int64_t>(rows, kMaxRowGrid);
    if (E <= kHistMaxE) {
        const int64_t chunk = hist_chunk(N), C = hist_chunks(N);
        int ebits = 0;
        while ((E >> ebits) != 0) ++ebits;        // E itself needs ebits bits
        int32_t* hist = static_cast<int32_t*>(ws);
        const dim3 grid((unsigned)((C + kHistWaves - 1) / kHistWaves));
        hipLaunchKernelGGL(chunk_count_kernel, grid, dim3(64 * kHistWaves), 0, st, topk_idx, N, E, chunk, C, hist);
        hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, st, hist, C, E, shared, T, R, offsets,
                           perm_src);
        hipLaunchKernelGGL(chunk_scatter_kernel, grid, dim3(64 * kHistWaves), 0, st, topk_idx, N, k, E, ebits, chunk, C,
                           hist, R, perm_src, inv_perm);
    } else {
        const int64_t seg = ((N + kWaves - 1) / kWaves + kStep - 1) / kStep * kStep;
        int32_t* wave_counts = static_cast<int32_t*>(ws);
        int32_t* wave_base = wave_counts + (size_t)E * kWaves;
        hipLaunchKernelGGL(count_kernel, dim3(E), dim3(1024), 0, st, topk_idx, N, seg, wave_counts);
        hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(1024), 0, st, wave_counts, E, shared, T, R, offsets,
                           wave_base, perm_src);
        hipLaunchKernelGGL(scatter_kernel, dim3(E), dim3(1024), 0, st, topk_idx, N, k, E, seg, wave_base, perm_src,
                           inv_perm);
    }
    if (!gather) {
        if (shared) hipLaunchKernelGGL(shared_rows_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, perm_src, R, T);
    } else if (act_dtype == DWDP_FP8_E4M3) {
        hipLaunchKernelGGL(gather_fp8_kernel, dim3(row_grid), dim3(256), 0, st, static_cast<const uint16_t*>(x), T, R,
                           rows, H, perm_src, static_cast<uint8_t*>(x_perm), x_perm_scale);
    } else {
        hipLaunchKernelGGL(gather_copy_kernel, dim3(row_grid), dim3(256), 0, st, static_cast<const uint8_t*>(x), T, R,
                           rows, (int64_t)H * (int64_t)elem_bytes(x_dtype), perm_src, static_cast<uint8_t*>(x_perm));
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
    hipLaunchKernelGGL(gather_fp8_kernel, dim3((unsigned)std::min<int64_t>(T, kMaxRowGrid)), dim3(256), 0,
                       as_stream(stream), static_cast<const uint16_t*>(x), T, (int64_t)0, T, H,
                       static_cast<int32_t*>(nullptr), static_cast<uint8_t*>(q), q_scale);
    DWDP_LAUNCHED();
    return DWDP_OK;
}
