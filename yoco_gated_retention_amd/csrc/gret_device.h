// gret_device.h -- device types and primitives shared by the gRet kernels (gfx950):
// vector types, matrix-core and LDS helpers, buffer descriptors, waits and the
// LDS barrier.
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

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// v_mfma_f32_16x16x32_bf16. Operand lanes: A row (B column) = lane % 16, the
// 8 k-values of a lane are 8 (lane / 16) .. +7; C column = lane % 16, rows
// 4 (lane / 16) .. +3.
__device__ inline f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: A row / B column = lane % 32 with contraction
// index 8 (lane / 32) + e for element e; C column = lane % 32, register r holds
// row 8 (r / 4) + 4 (lane / 32) + r % 4.
__device__ inline f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 lds_read8(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ inline bf16x4 lds_read4(const bf16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }

// Transposing LDS read: within each 16-lane group, lane l receives element
// (l % 4) of the 8-byte pieces addressed by lanes 4e + l/4 (e = 0..3). With
// lane s pointing at row t0 + s/4, column n0 + 4(s % 4) of a row-major tile,
// lane l gets column n0 + l of rows t0..t0+3.
__device__ inline bf16x4 lds_read_tr4(const bf16_t* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ inline bf16x8 cat44(const bf16x4& a, const bf16x4& b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// swish(x) = x * sigmoid(x), with the hardware reciprocal (about 1 ulp).
__device__ inline float swish(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Sum over aligned groups of L adjacent lanes (L = 8, 16 or 32), every lane of
// a group receiving the total. Within a 16-lane DPP row: exchange with lane^1
// and lane^2 (quad permutations), then with the mirrored lane of the half row
// and of the row; across rows (L = 32) one cross-lane permute.
template <int L>
__device__ inline float group_sum(float v) {
    static_assert(L == 8 || L == 16 || L == 32, "group size");
    constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kXor1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kXor2, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kHalfMirror, 0xF, 0xF, false));
    if constexpr (L >= 16)
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kMirror, 0xF, 0xF, false));
    if constexpr (L == 32) v += __shfl_xor(v, 16);
    return v;
}

// Range-checked buffer access (CDNA buffer resources): a load past the
// descriptor's byte size returns zeros and a store past it is dropped.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, gfx9-family data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferWord3);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wavefront are outstanding (gfx9 encoding; expcnt and lgkmcnt left alone).
constexpr int vm_wait_imm(int n) {
    return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8);
}
constexpr int kLgkmWaitZero = 0xC07F;  // lgkmcnt(0) only

template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(N));
}

// Workgroup barrier for LDS data: this wavefront's LDS writes complete, then
// s_barrier; compiler-only fences keep memory accesses on their side. Unlike
// __syncthreads it carries no release fence, so it does not drain the loads
// still in flight for later tiles.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kLgkmWaitZero);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace gret
