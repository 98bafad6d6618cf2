// gret_stream.hip -- streaming kernels that measure what HBM delivers for the
// access mix of the chunkwise prefill: three read streams (q, k, v) and one
// write stream (the output) of equal size, 16 bytes per lane, so each
// wavefront instruction moves 1 KB of contiguous rows. They compute nothing of
// the method (the output is the bitwise XOR of the three inputs, so no load
// can be dropped); they give the measured bandwidth ceiling the prefill is
// compared against. Built into libgret_stream.so, used only by the benchmark.
//
// Variants: cache policy of the loads and of the stores (default write-back
// or nontemporal), rows per lane and iteration (U), and workgroups per
// compute unit (the grid is persistent: CUs x W workgroups of 256 threads
// walk the arrays with a grid stride).
//
// The segmented form mirrors the prefill's own memory pattern: each of G
// workgroups (8 wavefronts, one per compute unit) streams its own contiguous
// 1/G of the arrays (segments assigned to workgroups as the prefill assigns
// them: one contiguous run of segments per XCD), the loads go from HBM straight into LDS with
// buffer_load ... lds, D 1 KB blocks per stream and wavefront in flight, and
// the output leaves from LDS through the registers with 16-byte stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ inline i32x4 ld(const i32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__device__ inline void st(i32x4* p, const i32x4& v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// R read streams (1..3) and, if W_OUT, one write stream; n16 16-byte units each.
template <int R, bool W_OUT, bool NT_LOAD, bool NT_STORE, int U>
__global__ __launch_bounds__(256) void stream_kernel(const i32x4* __restrict__ a,
                                                     const i32x4* __restrict__ b,
                                                     const i32x4* __restrict__ c,
                                                     i32x4* __restrict__ o, int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * U;
    i32x4 sink = {0, 0, 0, 0};
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x; base < n16;
         base += stride) {
        i32x4 x[U], y[U], z[U];
        if (base + 256 * (U - 1) < n16) {
            // whole iteration in range: every load is issued before any use
#pragma unroll
            for (int u = 0; u < U; ++u) {
                x[u] = ld<NT_LOAD>(a + base + 256 * u);
                if constexpr (R > 1) y[u] = ld<NT_LOAD>(b + base + 256 * u);
                if constexpr (R > 2) z[u] = ld<NT_LOAD>(c + base + 256 * u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (R > 1) x[u] ^= y[u];
                if constexpr (R > 2) x[u] ^= z[u];
                if constexpr (W_OUT)
                    st<NT_STORE>(o + base + 256 * u, x[u]);
                else
                    sink ^= x[u];
            }
        } else {
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + 256 * u;
                if (i >= n16) break;
                i32x4 t = ld<NT_LOAD>(a + i);
                if constexpr (R > 1) t ^= ld<NT_LOAD>(b + i);
                if constexpr (R > 2) t ^= ld<NT_LOAD>(c + i);
                if constexpr (W_OUT)
                    st<NT_STORE>(o + i, t);
                else
                    sink ^= t;
            }
        }
    }
    if constexpr (!W_OUT) {
        // keeps the loads of a read-only variant alive; one store per thread
        if ((sink.x | sink.y | sink.z | sink.w) == 0x7fffffff) o[threadIdx.x] = sink;
    }
}

// Write-only: fills o with a constant (no read stream).
template <bool NT_STORE, int U>
__global__ __launch_bounds__(256) void fill_kernel(i32x4* __restrict__ o, int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * U;
    const i32x4 v = {1, 2, 3, 4};
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x; base < n16;
         base += stride) {
        if (base + 256 * (U - 1) < n16) {
#pragma unroll
            for (int u = 0; u < U; ++u) st<NT_STORE>(o + base + 256 * u, v);
        } else {
            for (int u = 0; u < U && base + 256 * u < n16; ++u) st<NT_STORE>(o + base + 256 * u, v);
        }
    }
}

typedef __attribute__((address_space(3))) void lds_void;

constexpr int vm_wait_imm(int n) {
    return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8);
}
template <int N>
__device__ inline void wait_vm() {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(N));
}

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Segmented 3-read/1-write stream through LDS: D iterations in flight per
// wavefront; at least 96 KB of LDS per workgroup, so one workgroup per CU.
template <int D, int POL_L, int POL_S>
__global__ __launch_bounds__(512) void seg_stream_kernel(const char* a, const char* b,
                                                         const char* c, char* o, int64_t nblk) {
    constexpr int kSlots = D < 4 ? 4 : D;
    __shared__ __attribute__((aligned(16))) char lds[8 * kSlots * 3072];
    // segment of this workgroup in the prefill's order: the ids that land on
    // one XCD (id mod 8) take one contiguous run of segments
    const int64_t G = gridDim.x, x = blockIdx.x % 8, per = G / 8, rem = G % 8;
    const int64_t seg = x * per + (x < rem ? x : rem) + blockIdx.x / 8;
    const int64_t lo = seg * nblk / G;
    const int64_t hi = (seg + 1) * nblk / G;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    char* mine = lds + w * D * 3072;
    const int64_t nit = (hi - lo + 7) / 8;
    const uint32_t sbytes = static_cast<uint32_t>((hi - lo) * 1024);
    const __amdgpu_buffer_rsrc_t ra = rsrc(a + lo * 1024, sbytes), rb = rsrc(b + lo * 1024, sbytes),
                                 rc = rsrc(c + lo * 1024, sbytes), ro = rsrc(o + lo * 1024, sbytes);
    auto issue = [&](int64_t it, int slot) {
        const uint32_t off = static_cast<uint32_t>((it * 8 + w) * 1024 + lane * 16);
        char* d = mine + slot * 3072;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(d), 16, off, 0, 0, POL_L);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(d + 1024), 16, off, 0, 0, POL_L);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void*)(d + 2048), 16, off, 0, 0, POL_L);
    };
    // iterations past the segment read zeros and store nothing (range checks)
#pragma unroll
    for (int i = 0; i < D; ++i) issue(i, i);
    for (int64_t it = 0; it < nit; it += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            // operations younger than iteration it+s's loads: in the prologue at
            // least 3 (D-1) loads, afterwards (D-1) x (3 loads + 1 store)
            if (it == 0)
                wait_vm<(D - 1) * 3>();
            else
                wait_vm<(D - 1) * 4>();
            const i32x4* p = reinterpret_cast<const i32x4*>(mine + s * 3072 + lane * 16);
            const i32x4 v = p[0] ^ p[64] ^ p[128];
            const uint32_t off = static_cast<uint32_t>(((it + s) * 8 + w) * 1024 + lane * 16);
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, off, 0, POL_S);
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): slot read before it is refilled
            issue(it + s + D, s);
        }
    }
    wait_vm<0>();
}

template <int D>
hipError_t launch_seg(int nt_load, int nt_store, int groups, const void* a, const void* b,
                      const void* c, void* o, int64_t nblk, hipStream_t s) {
    auto A = static_cast<const char*>(a);
    auto B = static_cast<const char*>(b);
    auto C = static_cast<const char*>(c);
    auto O = static_cast<char*>(o);
    const dim3 g(groups), t(512);
    if (nt_load && nt_store) hipLaunchKernelGGL((seg_stream_kernel<D, 2, 2>), g, t, 0, s, A, B, C, O, nblk);
    else if (nt_load) hipLaunchKernelGGL((seg_stream_kernel<D, 2, 0>), g, t, 0, s, A, B, C, O, nblk);
    else if (nt_store) hipLaunchKernelGGL((seg_stream_kernel<D, 0, 2>), g, t, 0, s, A, B, C, O, nblk);
    else hipLaunchKernelGGL((seg_stream_kernel<D, 0, 0>), g, t, 0, s, A, B, C, O, nblk);
    return hipGetLastError();
}

template <int R, bool W_OUT, bool NL, bool NS>
hipError_t launch_u(int u, int groups, const void* a, const void* b, const void* c, void* o,
                    int64_t n16, hipStream_t s) {
    const dim3 g(groups), t(256);
    auto A = static_cast<const i32x4*>(a);
    auto B = static_cast<const i32x4*>(b);
    auto C = static_cast<const i32x4*>(c);
    auto O = static_cast<i32x4*>(o);
    switch (u) {
        case 1: hipLaunchKernelGGL((stream_kernel<R, W_OUT, NL, NS, 1>), g, t, 0, s, A, B, C, O, n16); break;
        case 2: hipLaunchKernelGGL((stream_kernel<R, W_OUT, NL, NS, 2>), g, t, 0, s, A, B, C, O, n16); break;
        case 4: hipLaunchKernelGGL((stream_kernel<R, W_OUT, NL, NS, 4>), g, t, 0, s, A, B, C, O, n16); break;
        case 8: hipLaunchKernelGGL((stream_kernel<R, W_OUT, NL, NS, 8>), g, t, 0, s, A, B, C, O, n16); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int R, bool W_OUT>
hipError_t launch_pol(int nt_load, int nt_store, int u, int groups, const void* a, const void* b,
                      const void* c, void* o, int64_t n16, hipStream_t s) {
    if (nt_load && nt_store) return launch_u<R, W_OUT, true, true>(u, groups, a, b, c, o, n16, s);
    if (nt_load) return launch_u<R, W_OUT, true, false>(u, groups, a, b, c, o, n16, s);
    if (nt_store) return launch_u<R, W_OUT, false, true>(u, groups, a, b, c, o, n16, s);
    return launch_u<R, W_OUT, false, false>(u, groups, a, b, c, o, n16, s);
}

}  // namespace

extern "C" {

// Streams `reads` (1..3) input arrays of `bytes` bytes each and, when `write`
// is nonzero, writes one output array of the same size; reads == 0 with write
// is a plain fill. Pointers must be 16-byte aligned and bytes a multiple of
// 16. `groups` workgroups of 256 threads; `unroll` in {1, 2, 4, 8}. Returns 0
// when enqueued on `stream`, else a nonzero hipError_t value.
int gret_stream_run(int reads, int write, int nt_load, int nt_store, int unroll, int groups,
                    const void* a, const void* b, const void* c, void* out, int64_t bytes,
                    void* stream) {
    if (bytes <= 0 || bytes % 16 != 0 || groups < 1 || !out) return hipErrorInvalidValue;
    const int64_t n16 = bytes / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (reads == 0) {
        if (!write) return hipErrorInvalidValue;
        const dim3 g(groups), t(256);
        auto O = static_cast<i32x4*>(out);
        if (unroll != 4) return hipErrorInvalidValue;
        if (nt_store)
            hipLaunchKernelGGL((fill_kernel<true, 4>), g, t, 0, s, O, n16);
        else
            hipLaunchKernelGGL((fill_kernel<false, 4>), g, t, 0, s, O, n16);
        return hipGetLastError();
    }
    if (!a || (reads > 1 && !b) || (reads > 2 && !c)) return hipErrorInvalidValue;
    if (reads == 1)
        return write ? launch_pol<1, true>(nt_load, nt_store, unroll, groups, a, b, c, out, n16, s)
                     : launch_pol<1, false>(nt_load, nt_store, unroll, groups, a, b, c, out, n16, s);
    if (reads == 2)
        return write ? launch_pol<2, true>(nt_load, nt_store, unroll, groups, a, b, c, out, n16, s)
                     : launch_pol<2, false>(nt_load, nt_store, unroll, groups, a, b, c, out, n16, s);
    if (reads == 3)
        return write ? launch_pol<3, true>(nt_load, nt_store, unroll, groups, a, b, c, out, n16, s)
                     : launch_pol<3, false>(nt_load, nt_store, unroll, groups, a, b, c, out, n16, s);
    return hipErrorInvalidValue;
}

// The segmented form: `groups` workgroups each stream their own contiguous
// 1/groups of three input arrays into one output array (bytes each, a multiple
// of 1 KB, each workgroup's share below 4 GB), `depth` in {2, 3, 4, 6}.
int gret_stream_segmented_run(int depth, int nt_load, int nt_store, int groups, const void* a,
                              const void* b, const void* c, void* out, int64_t bytes,
                              void* stream) {
    if (bytes <= 0 || bytes % 1024 != 0 || groups < 1 || !a || !b || !c || !out)
        return hipErrorInvalidValue;
    const int64_t nblk = bytes / 1024;
    // every offset a workgroup forms (its share plus the blocks issued past it)
    if ((nblk / groups + 64) * 1024 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (depth) {
        case 2: return launch_seg<2>(nt_load, nt_store, groups, a, b, c, out, nblk, s);
        case 3: return launch_seg<3>(nt_load, nt_store, groups, a, b, c, out, nblk, s);
        case 4: return launch_seg<4>(nt_load, nt_store, groups, a, b, c, out, nblk, s);
        case 6: return launch_seg<6>(nt_load, nt_store, groups, a, b, c, out, nblk, s);
        default: return hipErrorInvalidValue;
    }
}

}  // extern "C"
