// Device-side helpers shared by the library's HIP translation units: HIP error checks and the
// number conversions (bf16, E4M3).  The host-only helpers are in errors.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <string>

#include "errors.h"

namespace dwdp {

#define DWDP_HIP(call)                                                                \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess)                                                         \
            return ::dwdp::fail(DWDP_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
    } while (0)

#define DWDP_LAUNCHED()                                                               \
    do {                                                                              \
        hipError_t e_ = hipGetLastError();                                            \
        if (e_ != hipSuccess)                                                         \
            return ::dwdp::fail(DWDP_ERR_HIP, std::string(__func__) + ": launch: " + hipGetErrorString(e_)); \
    } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ------------------------------------------------------------ device: numbers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 -> OCP E4M3 code: round to nearest even, saturating at +-448, NaN -> 0x7F.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7f;
    if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);          // |x| >= 448
    if (a < 0x3c800000u) {                                           // |x| < 2^-6: subnormal step 2^-9
        float m = __builtin_rintf(__uint_as_float(a) * 512.0f);      // exact scaling, rint = ties to even
        return (uint8_t)(sign | (uint32_t)m);                        // m == 8 is the smallest normal
    }
    uint32_t mant = a & 0x7fffffu;
    uint32_t expf = (a >> 23) - 127u + 7u;                           // 1..15
    uint32_t r = mant + 0x7ffffu + ((mant >> 20) & 1u);              // round to 3 fraction bits
    uint32_t code = (expf << 3) + (r >> 20);                         // carry bumps the exponent
    if (code > 0x7eu) code = 0x7eu;
    return (uint8_t)(sign | code);
}

__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
    uint32_t s = (uint32_t)(c & 0x80u) << 24;
    uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
    if (e == 0) return __uint_as_float(s) + (s ? -1.0f : 1.0f) * (float)m * 0.001953125f;
    return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// Wavefront helpers (64 lanes).
__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace dwdp
