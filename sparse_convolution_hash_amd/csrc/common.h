// Internal helpers shared by the libspc HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

#include "spc.h"

namespace spc {

// ---------------------------------------------------------------- host errors

// Records a printf-style message in the thread-local error string and
// returns `st`, so host checks read `return fail(SPC_ERR_ARG, "...")`.
spc_status fail(spc_status st, const char* fmt, ...);
void clear_error();

#define SPC_HIP(call)                                                              \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess)                                                      \
            return ::spc::fail(SPC_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// Checks the launch that was just issued.
#define SPC_LAUNCHED(name)                                                            \
    do {                                                                              \
        hipError_t e_ = hipGetLastError();                                            \
        if (e_ != hipSuccess)                                                         \
            return ::spc::fail(SPC_ERR_HIP, "launch of %s: %s", name, hipGetErrorString(e_)); \
    } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, queried once per device (256 when the
// query fails); sizes the grids of the persistent kernels.
inline int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// ---------------------------------------------------------------- device side

constexpr int WAVE = 64;

// Load of a[min(i, n - 1)] (n >= 1): an unconditional load, so a batch of
// them issues back to back; the caller discards the value when i >= n.
template <typename T>
__device__ __forceinline__ T ld_clamped(const T* __restrict__ a, int64_t i, int64_t n) {
    return a[i < n ? i : n - 1];
}

// Workgroup barrier that waits for LDS operations only: a release/acquire
// fence scoped to the workgroup and to LDS around s_barrier.  Unlike
// __syncthreads(), which waits for every outstanding memory operation first,
// it lets global loads into registers stay in flight across it, so loads can
// be issued steps ahead of their use.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Block-wide exclusive scan of one int per thread; returns the block total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_waves, int& total) {
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    int incl = v;
    for (int off = 1; off < WAVE; off <<= 1) {
        const int u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
    }
    if (lane == WAVE - 1) lds_waves[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < NT / WAVE; ++w) {
        const int s = lds_waves[w];
        if (w < wave) before += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// 16 bytes moved as one unit (one dwordx4 load/store).
struct alignas(16) u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st16(void* p, const u32x4& v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// fp32 -> fp16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
    _Float16 h = static_cast<_Float16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

// Element types: T is the storage type seen by the kernels; 16-bit types are
// carried as raw bits and only the MFMA reads them as numbers.
struct F32 {
    using storage = float;
    static constexpr int E = 4;  // elements per 16 bytes
    static constexpr spc_dtype id = SPC_F32;
};
struct F16 {
    using storage = uint16_t;
    static constexpr int E = 8;
    static constexpr spc_dtype id = SPC_F16;
};
struct BF16 {
    using storage = uint16_t;
    static constexpr int E = 8;
    static constexpr spc_dtype id = SPC_BF16;
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// One 16x16 MFMA tile step over the 16-byte fragments a (rows of D) and b
// (columns of D).  Lane l supplies, for D-row (resp. column) l%16, the
// contraction elements of lane group l/16: 8 consecutive values for the
// 16-bit types (v_mfma_f32_16x16x32_{f16,bf16}), 4 for fp32, which are
// consumed by four v_mfma_f32_16x16x4_f32 steps, one element each.  Any
// assignment of contraction indices to (lane group, element) works as long as
// a and b use the same one, and these two do.
template <typename TT>
__device__ __forceinline__ f32x4_t mfma16(const u32x4& a, const u32x4& b, f32x4_t c);

template <>
__device__ __forceinline__ f32x4_t mfma16<BF16>(const u32x4& a, const u32x4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4_t mfma16<F16>(const u32x4& a, const u32x4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4_t mfma16<F32>(const u32x4& a, const u32x4& b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
}

// Stores four consecutive fp32 values as the element type (one RNE rounding).
template <typename TT>
__device__ __forceinline__ void store4(void* p, f32x4_t v);

template <>
__device__ __forceinline__ void store4<F32>(void* p, f32x4_t v) {
    *reinterpret_cast<f32x4_t*>(p) = v;
}

template <>
__device__ __forceinline__ void store4<BF16>(void* p, f32x4_t v) {
    uint2 w;
    w.x = uint32_t(f32_to_bf16_rne(v.x)) | (uint32_t(f32_to_bf16_rne(v.y)) << 16);
    w.y = uint32_t(f32_to_bf16_rne(v.z)) | (uint32_t(f32_to_bf16_rne(v.w)) << 16);
    *reinterpret_cast<uint2*>(p) = w;
}

template <>
__device__ __forceinline__ void store4<F16>(void* p, f32x4_t v) {
    uint2 w;
    w.x = uint32_t(f32_to_f16_rne(v.x)) | (uint32_t(f32_to_f16_rne(v.y)) << 16);
    w.y = uint32_t(f32_to_f16_rne(v.z)) | (uint32_t(f32_to_f16_rne(v.w)) << 16);
    *reinterpret_cast<uint2*>(p) = w;
}

// Loads four consecutive elements of the element type as fp32 (exact).
template <typename TT>
__device__ __forceinline__ f32x4_t load4(const void* p);

template <>
__device__ __forceinline__ f32x4_t load4<F32>(const void* p) {
    return *reinterpret_cast<const f32x4_t*>(p);
}

template <>
__device__ __forceinline__ f32x4_t load4<BF16>(const void* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                   __uint_as_float(w.y & 0xffff0000u)};
}

template <>
__device__ __forceinline__ f32x4_t load4<F16>(const void* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    auto h = [](uint32_t b) { return float(__builtin_bit_cast(_Float16, uint16_t(b))); };
    return f32x4_t{h(w.x & 0xffffu), h(w.x >> 16), h(w.y & 0xffffu), h(w.y >> 16)};
}

inline int dtype_size(spc_dtype d) { return d == SPC_F32 ? 4 : 2; }

}  // namespace spc
