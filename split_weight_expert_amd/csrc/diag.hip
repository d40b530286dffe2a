// Diagnostics of the machine (not steps of the MoE block).
//
// Operand-stream probe: how fast workgroups move bytes from device memory into LDS with
// global_load_lds, the path every operand of the expert GEMM takes (a diagnostic, not a step of the
// MoE block).  Each workgroup has the GEMM's shape -- 512 threads, one per compute unit, a ring of
// 32 KB LDS slots -- and does nothing but load, so the rate it reaches is the ceiling of the GEMM's
// operand stream for the same source of bytes: lines that hit the XCD's L2, or lines that miss it.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace dwdp {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeSlots = 5;
constexpr int kProbeStep = 32768;        // bytes per step: 8 waves x 4 loads of 1 KB
constexpr int kProbePerWave = 4;

template <int CPOL>
__device__ __forceinline__ void probe_dma16(const uint8_t* g, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, CPOL);
#endif
}

template <int N>
__device__ __forceinline__ void probe_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup b streams [b*stride, b*stride + span) of src `iters` times.  Step s goes to slot s % 5;
// after issuing step s a wave waits until at most INFL-1 of its steps are outstanding, so a slot is
// rewritten only after the load that last filled it has landed (INFL <= 5 slots).  The bytes are
// never read from LDS: only the arrival rate is measured.
template <int INFL, int CPOL>
__global__ __launch_bounds__(kProbeThreads) void operand_stream_kernel(const uint8_t* __restrict__ src, size_t span,
                                                                       size_t stride, int iters) {
    static_assert(INFL >= 1 && INFL <= kProbeSlots, "in-flight steps");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kProbeSlots * kProbeStep];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* base = src + (size_t)blockIdx.x * stride + wave * (kProbePerWave * 1024) + lane * 16;
    uint8_t* lbase = ring + wave * (kProbePerWave * 1024);
    const size_t steps = span / kProbeStep;
    size_t s_all = 0;
    for (int it = 0; it < iters; ++it) {
        for (size_t s = 0; s < steps; ++s, ++s_all) {
            const uint8_t* g = base + s * kProbeStep;
            uint8_t* l = lbase + (s_all % kProbeSlots) * kProbeStep;
#pragma unroll
            for (int q = 0; q < kProbePerWave; ++q) probe_dma16<CPOL>(g + q * 1024, l + q * 1024);
            probe_wait_vmcnt<(INFL - 1) * kProbePerWave>();
        }
    }
    probe_wait_vmcnt<0>();
}

template <int CPOL>
void launch_probe(int in_flight, dim3 grid, hipStream_t st, const uint8_t* src, size_t span, size_t stride,
                  int iters) {
    switch (in_flight) {
        case 1: hipLaunchKernelGGL((operand_stream_kernel<1, CPOL>), grid, dim3(kProbeThreads), 0, st, src, span, stride, iters); break;
        case 2: hipLaunchKernelGGL((operand_stream_kernel<2, CPOL>), grid, dim3(kProbeThreads), 0, st, src, span, stride, iters); break;
        case 3: hipLaunchKernelGGL((operand_stream_kernel<3, CPOL>), grid, dim3(kProbeThreads), 0, st, src, span, stride, iters); break;
        case 4: hipLaunchKernelGGL((operand_stream_kernel<4, CPOL>), grid, dim3(kProbeThreads), 0, st, src, span, stride, iters); break;
        default: hipLaunchKernelGGL((operand_stream_kernel<5, CPOL>), grid, dim3(kProbeThreads), 0, st, src, span, stride, iters); break;
    }
}

// LDS read probe: every wave reads 16-byte slots of a 128 KB LDS array with ds_read_b128, each lane a
// consecutive slot (no bank conflicts), Q reads in flight between uses; thread 0 stores the workgroup's
// shader-clock (s_memtime) and real-time (s_memrealtime, 100 MHz) deltas over the loop.
constexpr int kLdsSlots = 8192;
constexpr int kLdsQ = 16;

template <int THREADS>
__global__ __launch_bounds__(THREADS) void lds_read_kernel(int iters, uint32_t* __restrict__ sink,
                                                           unsigned long long* __restrict__ clocks) {
    __shared__ __attribute__((aligned(16))) uint4 buf[kLdsSlots];
    for (int i = threadIdx.x; i < kLdsSlots; i += THREADS) buf[i] = uint4{(uint32_t)i, (uint32_t)i + 1u, 2u, 3u};
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint4 acc{0, 0, 0, 0};
    const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < kLdsQ; ++q) {
            const uint4 v = buf[((it * kLdsQ + q) * 64 + w * 1024 + lane) & (kLdsSlots - 1)];
            acc.x ^= v.x;
            acc.y ^= v.y;
            acc.z ^= v.z;
            acc.w ^= v.w;
        }
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    // a store the compiler cannot drop, taken (almost) never: keeps the reads
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[blockIdx.x] = acc.x;
    if (threadIdx.x == 0) {
        clocks[2 * (size_t)blockIdx.x] = c1 - c0;
        clocks[2 * (size_t)blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace
}  // namespace dwdp

using namespace dwdp;

extern "C" int dwdp_diag_lds_read(int grid, int waves, int iters, uint32_t* sink, unsigned long long* clocks,
                                  void* stream) {
    clear_error();
    DWDP_REQUIRE(grid >= 1 && grid <= 65536, "grid must be in [1, 65536]");
    DWDP_REQUIRE(waves == 4 || waves == 8 || waves == 16, "waves must be 4, 8 or 16");
    DWDP_REQUIRE(iters >= 1, "iters must be at least 1");
    DWDP_REQUIRE(sink != nullptr && clocks != nullptr, "null pointer argument");
    DWDP_REQUIRE(aligned16(clocks), "clocks must be 16-byte aligned");
    hipStream_t st = as_stream(stream);
    if (waves == 4) hipLaunchKernelGGL(lds_read_kernel<256>, dim3(grid), dim3(256), 0, st, iters, sink, clocks);
    else if (waves == 8) hipLaunchKernelGGL(lds_read_kernel<512>, dim3(grid), dim3(512), 0, st, iters, sink, clocks);
    else hipLaunchKernelGGL(lds_read_kernel<1024>, dim3(grid), dim3(1024), 0, st, iters, sink, clocks);
    DWDP_LAUNCHED();
    return DWDP_OK;
}

extern "C" int dwdp_diag_operand_stream(const void* src, size_t span, size_t stride, int iters, int grid,
                                        int in_flight, int cpol, void* stream) {
    clear_error();
    DWDP_REQUIRE(src != nullptr, "src is NULL");
    DWDP_REQUIRE(aligned16(src), "src must be 16-byte aligned");
    DWDP_REQUIRE(span > 0 && span % kProbeStep == 0, "span must be a positive multiple of 32768");
    DWDP_REQUIRE(stride % 16 == 0, "stride must be a multiple of 16");
    DWDP_REQUIRE(iters >= 1, "iters must be at least 1");
    DWDP_REQUIRE(grid >= 1 && grid <= 65536, "grid must be in [1, 65536]");
    DWDP_REQUIRE(in_flight >= 1 && in_flight <= kProbeSlots, "in_flight must be in [1, 5]");
    DWDP_REQUIRE(cpol == 0 || cpol == 2, "cpol must be 0 or 2");
    hipStream_t st = as_stream(stream);
    const auto* s = static_cast<const uint8_t*>(src);
    if (cpol == 0) launch_probe<0>(in_flight, dim3(grid), st, s, span, stride, iters);
    else launch_probe<2>(in_flight, dim3(grid), st, s, span, stride, iters);
    DWDP_LAUNCHED();
    return DWDP_OK;
}
