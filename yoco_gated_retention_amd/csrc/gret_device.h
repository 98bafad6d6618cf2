// gret_device.h -- small device helpers shared by the gRet kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gret {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// fp32 -> bf16 with round-to-nearest-even (the default rounding mode; gfx950
// lowers this to its packed convert instruction).
__device__ inline bf16_t to_bf16(float x) { return static_cast<bf16_t>(x); }
__device__ inline float from_bf16(bf16_t x) { return static_cast<float>(x); }

__device__ inline float load_as_float(const float* p, int64_t i) { return p[i]; }
__device__ inline float load_as_float(const bf16_t* p, int64_t i) { return from_bf16(p[i]); }

__device__ inline void store_from_float(float* p, int64_t i, float x) { p[i] = x; }
__device__ inline void store_from_float(bf16_t* p, int64_t i, float x) { p[i] = to_bf16(x); }

// Clamp of the log-gate to [floor, 0]. fmaxf returns its non-NaN operand, so
// a NaN log-gate is treated as the floor (gate ~ 0).
__device__ inline float clamp_log_gamma(float l, float floor_v) {
    return fminf(fmaxf(l, floor_v), 0.0f);
}

}  // namespace gret
