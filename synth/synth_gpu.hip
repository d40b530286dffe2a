// Seeded synthetic tensors on the GPU: the element generator of synth_host.c
// written again for gfx950, so that full-size inputs can be produced in HBM
// without a host round trip.  Test and benchmark infrastructure only; it holds
// none of the MoE layer's arithmetic.  Both implementations follow the same
// definition (SplitMix64 counter draw, four 16-bit fields summed, one fp32
// multiply, optional round-to-nearest-even to bf16) and must agree bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float synth_value(uint64_t key, uint64_t i, float c) {
    uint64_t z = mix64(key + (i + 1) * kGamma);
    int32_t s = (int32_t)(z & 0xFFFFu) + (int32_t)((z >> 16) & 0xFFFFu) +
                (int32_t)((z >> 32) & 0xFFFFu) + (int32_t)(z >> 48);
    return __fmul_rn((float)(s - 131070), c);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__global__ void fill_f32(uint64_t key, uint64_t first, uint64_t n, float c, float* out) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        out[j] = synth_value(key, first + j, c);
}

__global__ void fill_bf16(uint64_t key, uint64_t first, uint64_t n, float c, uint16_t* out) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        out[j] = f32_to_bf16_rne(synth_value(key, first + j, c));
}

unsigned grid_for(uint64_t n) {
    uint64_t g = (n + 255) / 256;
    if (g > 65536) g = 65536;
    if (g == 0) g = 1;
    return (unsigned)g;
}

}  // namespace

extern "C" {

// out[j] = element (first + j) for j < n, fp32, on `stream`.  Returns a
// hipError_t code (0 on success).
int synth_gpu_fill_f32(uint64_t key, uint64_t first, uint64_t n, float c, void* out, void* stream) {
    if (n == 0) return 0;
    if (out == nullptr) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, first, n, c,
                       (float*)out);
    return (int)hipGetLastError();
}

// out[j] = bf16 bits of element (first + j) for j < n, on `stream`.
int synth_gpu_fill_bf16(uint64_t key, uint64_t first, uint64_t n, float c, void* out, void* stream) {
    if (n == 0) return 0;
    if (out == nullptr) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fill_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, first, n, c,
                       (uint16_t*)out);
    return (int)hipGetLastError();
}

}  // extern "C"
