// Layer-ahead expert prefetch (DWDP paper summary, §2) with time-division
// multiplexed slices (§4.3.2): every source is cut into fixed-size slices and
// the slices are issued round-robin over the sources.
//
// Two engines walk the same plan:
//   DWDP_COPY_HIPMEMCPY  one hipMemcpyAsync per slice on the copy stream -- the
//                        pages' pull mechanism.  On MI355X a same-device copy is
//                        served by the runtime's blit kernel, one launch per slice.
//   DWDP_COPY_KERNEL     one launch of a slice-copy kernel with a bounded grid:
//                        workgroup b copies plan slices b, b+grid, ... with
//                        non-temporal 16-byte loads and stores, so the copy
//                        takes a fixed, small share of the CUs and does not
//                        evict the expert GEMM's working set from L2.
// Also here: block quantisation of weights to fp8 (an offline weight-preparation
// step, not part of the per-layer path).
#include <algorithm>
#include <cstring>

#include "common.h"
#include "internal.h"

namespace dwdp {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct CopyArgs {
    const uint8_t* src[kMaxCopySources];
    uint64_t dst_off[kMaxCopySources];
    uint64_t bytes[kMaxCopySources];
    int32_t nchunks[kMaxCopySources];
    uint8_t* dst;
    uint64_t chunk;
    int64_t total_chunks;
    int32_t n_src;
    int32_t max_rounds;
};

// Plan slice P -> (source, slice index): round c holds slice c of every source
// that has more than c slices, in source order.
__device__ void plan_entry(const CopyArgs& a, int64_t P, int& src, int64_t& c) {
    int64_t lo = 0, hi = a.max_rounds;      // find the round: before(c) <= P < before(c+1)
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        int64_t before = 0;
        for (int s = 0; s < a.n_src; ++s) before += min((int64_t)a.nchunks[s], mid);
        if (before <= P) lo = mid;
        else hi = mid;
    }
    c = lo;
    int64_t before = 0;
    for (int s = 0; s < a.n_src; ++s) before += min((int64_t)a.nchunks[s], c);
    int64_t i = P - before;
    src = 0;
    for (int s = 0; s < a.n_src; ++s) {
        if (a.nchunks[s] > c) {
            if (i == 0) {
                src = s;
                break;
            }
            --i;
        }
    }
}

constexpr int kCopyUnroll = 16;

__global__ __launch_bounds__(256) void slice_copy_kernel(CopyArgs a) {
    __shared__ int s_src;
    __shared__ int64_t s_c;
    for (int64_t P = blockIdx.x; P < a.total_chunks; P += gridDim.x) {
        if (threadIdx.x == 0) {
            int s;
            int64_t c;
            plan_entry(a, P, s, c);
            s_src = s;
            s_c = c;
        }
        __syncthreads();
        const int s = s_src;
        const uint64_t off = (uint64_t)s_c * a.chunk;
        const uint64_t n = min(a.chunk, a.bytes[s] - off);
        const uint8_t* from = a.src[s] + off;
        uint8_t* to = a.dst + a.dst_off[s] + off;
        __syncthreads();
        const uint64_t nvec = n / 16;
        const v4u* f4 = reinterpret_cast<const v4u*>(from);
        v4u* t4 = reinterpret_cast<v4u*>(to);
        uint64_t i = threadIdx.x;
        // kCopyUnroll loads per lane in flight (64 KB per workgroup): one workgroup then moves about
        // as much as a CU can pull from HBM, so a few workgroups carry the whole copy
        for (; i + (kCopyUnroll - 1) * 256 < nvec; i += kCopyUnroll * 256) {
            v4u v[kCopyUnroll];
#pragma unroll
            for (int j = 0; j < kCopyUnroll; ++j) v[j] = __builtin_nontemporal_load(f4 + i + j * 256);
#pragma unroll
            for (int j = 0; j < kCopyUnroll; ++j) __builtin_nontemporal_store(v[j], t4 + i + j * 256);
        }
        for (; i < nvec; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(f4 + i), t4 + i);
        for (uint64_t b = nvec * 16 + threadIdx.x; b < n; b += 256) to[b] = from[b];
    }
}

__global__ __launch_bounds__(256) void quantize_block_kernel(const float* __restrict__ w, int64_t cols,
                                                             uint8_t* __restrict__ q, float* __restrict__ s) {
    const int64_t br = blockIdx.y, bc = blockIdx.x;
    const int t = threadIdx.x, r = t >> 1, h = t & 1;
    const float* row = w + (br * kFp8Group + r) * cols + bc * kFp8Group + h * 64;
    float v[64];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float4 x = reinterpret_cast<const float4*>(row)[i];
        v[4 * i] = x.x;
        v[4 * i + 1] = x.y;
        v[4 * i + 2] = x.z;
        v[4 * i + 3] = x.w;
        m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
    __shared__ float red[4];
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
    uint8_t* out = q + (br * kFp8Group + r) * cols + bc * kFp8Group + h * 64;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        reinterpret_cast<uint32_t*>(out)[i] =
            e4m3x4(v[4 * i] / sc, v[4 * i + 1] / sc, v[4 * i + 2] / sc, v[4 * i + 3] / sc);
    }
    if (t == 0) s[br * (cols / kFp8Group) + bc] = sc;
}

}  // namespace
}  // namespace dwdp

using namespace dwdp;

extern "C" int dwdp_prefetch_chunks(void* dst, const dwdp_copy_src* srcs, int n_src, size_t chunk_bytes, int engine,
                                    int max_workgroups, void* copy_stream, void* wait_event, void* done_event) {
    clear_error();
    int rc = check_sources(srcs, n_src, chunk_bytes);
    if (rc != DWDP_OK) return rc;
    DWDP_REQUIRE(engine == DWDP_COPY_HIPMEMCPY || engine == DWDP_COPY_KERNEL || engine == DWDP_COPY_SDMA,
                 "unknown engine");
    DWDP_REQUIRE(max_workgroups >= 0, "max_workgroups must be >= 0");
    hipStream_t st = as_stream(copy_stream);
    std::vector<dwdp_chunk> plan = make_plan(srcs, n_src, chunk_bytes);
    if (!plan.empty()) DWDP_REQUIRE(dst != nullptr, "dst is NULL");
    CopyArgs a{};
    if (engine == DWDP_COPY_KERNEL && !plan.empty()) {
        // validate everything before anything is enqueued
        DWDP_REQUIRE(chunk_bytes % 16 == 0, "kernel engine needs chunk_bytes % 16 == 0");
        DWDP_REQUIRE(aligned16(dst), "kernel engine needs a 16-byte aligned dst");
        a.dst = static_cast<uint8_t*>(dst);
        a.chunk = chunk_bytes;
        a.n_src = n_src;
        a.total_chunks = (int64_t)plan.size();
        int64_t rounds = 0;
        for (int s = 0; s < n_src; ++s) {
            DWDP_REQUIRE(srcs[s].bytes == 0 || (aligned16(srcs[s].src) && srcs[s].dst_offset % 16 == 0),
                         "kernel engine needs 16-byte aligned sources and destination offsets");
            a.src[s] = static_cast<const uint8_t*>(srcs[s].src);
            a.dst_off[s] = srcs[s].dst_offset;
            a.bytes[s] = srcs[s].bytes;
            const size_t nc = n_slices(srcs[s].bytes, chunk_bytes);
            DWDP_REQUIRE(nc < ((size_t)1 << 31), "too many slices for one source");
            a.nchunks[s] = (int32_t)nc;
            rounds = std::max(rounds, (int64_t)nc);
        }
        a.max_rounds = (int32_t)rounds;
    }
    if (wait_event) DWDP_HIP(hipStreamWaitEvent(st, reinterpret_cast<hipEvent_t>(wait_event), 0));
    if (engine == DWDP_COPY_HIPMEMCPY || engine == DWDP_COPY_SDMA) {
        // SDMA: the copy kind that keeps compute units out of it (the DMA engines move the bytes)
        const hipMemcpyKind kind = engine == DWDP_COPY_SDMA ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
        for (const dwdp_chunk& c : plan) {
            DWDP_HIP(hipMemcpyAsync(static_cast<uint8_t*>(dst) + c.dst_offset,
                                    static_cast<const uint8_t*>(srcs[c.source].src) + c.src_offset, c.bytes, kind,
                                    st));
        }
    } else if (!plan.empty()) {
        const int grid = (int)std::min<int64_t>(max_workgroups > 0 ? max_workgroups : 48, a.total_chunks);
        hipLaunchKernelGGL(slice_copy_kernel, dim3(grid), dim3(256), 0, st, a);
        DWDP_LAUNCHED();
    }
    if (done_event) DWDP_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(done_event), st));
    return DWDP_OK;
}

extern "C" int dwdp_quantize_weight_fp8(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* s,
                                        void* stream) {
    clear_error();
    DWDP_REQUIRE(rows > 0 && cols > 0 && rows % kFp8Group == 0 && cols % kFp8Group == 0,
                 "rows and cols must be positive multiples of 128");
    DWDP_REQUIRE(rows / kFp8Group < 65536, "too many block rows");
    DWDP_REQUIRE(w && q && s, "null pointer argument");
    DWDP_REQUIRE(aligned16(w) && aligned16(q), "w and q must be 16-byte aligned");
    hipLaunchKernelGGL(quantize_block_kernel, dim3((unsigned)(cols / kFp8Group), (unsigned)(rows / kFp8Group)),
                       dim3(256), 0, as_stream(stream), w, cols, q, s);
    DWDP_LAUNCHED();
    return DWDP_OK;
}
