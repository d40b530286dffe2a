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

// Two fp32 values -> bf16 bits packed little-endian (a in the low half), round to nearest even, NaN
// stays a quiet NaN: one hardware v_cvt_pk_bf16_f32.
typedef float dwdp_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 dwdp_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((dwdp_f32x2){a, b}, dwdp_bf16x2));
}

// Four fp32 values -> OCP E4M3 codes (round to nearest even, subnormals kept), packed little-endian
// (a in byte 0).  The hardware conversion v_cvt_pk_fp8_f32, two values per instruction.  Callers pass
// x / (amax / 448), so |x| <= 448 up to the rounding of that division, well below 464 where the
// conversion would stop rounding to the largest code 0x7E (448).  The GPU tests compare its codes with
// the oracle's E4M3 rounding on every fp32 value of magnitude <= 448, both signs.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
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
