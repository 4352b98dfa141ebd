// Device helpers shared by the ZHA HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define ZHA_D 128            // head dimension the kernels are written for
#define ZHA_MAX_GROUP 16     // query heads per KV head (rows of one MFMA tile)
#define ZHA_SCORE_MAXB 256   // max score-kernel blocks per KV group
#define ZHA_ATTN_MAXB 512    // max attention split blocks per KV group
// gather workgroups resident per compute unit: three for bf16 K/V; two for fp32,
// whose wider rows need the registers of the lower occupancy
#ifndef ZHA_ATTN_BLOCKS_BF16
#define ZHA_ATTN_BLOCKS_BF16 3
#endif
#ifndef ZHA_ATTN_BLOCKS_F32
#define ZHA_ATTN_BLOCKS_F32 2
#endif

typedef __attribute__((ext_vector_type(8))) __bf16 zha_bf16x8;
typedef __attribute__((ext_vector_type(4))) float zha_f32x4;

__device__ __forceinline__ float zha_bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t zha_f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ zha_bf16x8 zha_as_bf16x8(uint4 v) {
    return __builtin_bit_cast(zha_bf16x8, v);
}

__device__ __forceinline__ float zha_neg_inf() { return -__builtin_inff(); }

// Make this wave's LDS writes visible to its other lanes before they read.
__device__ __forceinline__ void zha_wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Wait until this wave's global stores and atomics have completed.  A
// workgroup barrier does not wait for them, so before one thread of a workgroup
// publishes the workgroup's results to other workgroups (release fence, then a
// counter atomic) every wave calls this first.  s_waitcnt immediate for gfx9:
// vmcnt(0), expcnt and lgkmcnt left at their no-wait maxima.
__device__ __forceinline__ void zha_wave_mem_wait() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename T>
__device__ __forceinline__ T zha_shfl_xor(T v, int mask, int width = 64) {
    return __shfl_xor(v, mask, width);
}

// DPP moves within a wave (row = 16 lanes): lanes whose source is outside the
// row, or whose row is masked off, receive `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t zha_dpp(uint32_t old, uint32_t src) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum of a 64-bit value across a full wave (all lanes active):
// row_shr 1, 2, 4, 8 inside each row of 16, then row_bcast 15 and 31 across rows.
__device__ __forceinline__ uint64_t zha_wave_incl_scan_u64(uint64_t x) {
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
#define ZHA_SCAN_STEP(CTRL, RM)                            \
    {                                                      \
        const uint32_t tl = zha_dpp<CTRL, RM>(0u, lo);     \
        const uint32_t th = zha_dpp<CTRL, RM>(0u, hi);     \
        const uint32_t nl = lo + tl;                       \
        hi = hi + th + (nl < lo ? 1u : 0u);                \
        lo = nl;                                           \
    }
    ZHA_SCAN_STEP(0x111, 0xF)
    ZHA_SCAN_STEP(0x112, 0xF)
    ZHA_SCAN_STEP(0x114, 0xF)
    ZHA_SCAN_STEP(0x118, 0xF)
    ZHA_SCAN_STEP(0x142, 0xA)
    ZHA_SCAN_STEP(0x143, 0xC)
#undef ZHA_SCAN_STEP
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t zha_readlane_u64(uint64_t x, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)x, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Maximum over a full wave (all lanes active), returned to every lane.
__device__ __forceinline__ float zha_wave_max(float v) {
    const uint32_t ninf = 0xFF800000u;
    uint32_t x = __float_as_uint(v);
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x111, 0xF>(ninf, x))));
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x112, 0xF>(ninf, x))));
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x114, 0xF>(ninf, x))));
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x118, 0xF>(ninf, x))));
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x142, 0xA>(ninf, x))));
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x143, 0xC>(ninf, x))));
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)x, 63));
}

// Reductions over each row of 16 lanes (DPP row_ror); every lane of the row
// receives its row's result.
__device__ __forceinline__ float zha_row16_max(float v) {
    uint32_t x = __float_as_uint(v);
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x128, 0xF>(x, x))));
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x124, 0xF>(x, x))));
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x122, 0xF>(x, x))));
    x = __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(zha_dpp<0x121, 0xF>(x, x))));
    return __uint_as_float(x);
}

__device__ __forceinline__ float zha_row16_sum(float v) {
    v += __uint_as_float(zha_dpp<0x128, 0xF>(__float_as_uint(v), __float_as_uint(v)));
    v += __uint_as_float(zha_dpp<0x124, 0xF>(__float_as_uint(v), __float_as_uint(v)));
    v += __uint_as_float(zha_dpp<0x122, 0xF>(__float_as_uint(v), __float_as_uint(v)));
    v += __uint_as_float(zha_dpp<0x121, 0xF>(__float_as_uint(v), __float_as_uint(v)));
    return v;
}

__device__ __forceinline__ float zha_wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ uint64_t zha_wave_sum_u64(uint64_t v) {
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
        v += ((uint64_t)hi << 32) | lo;
    }
    return v;
}

// Relaxed device-scope load that bypasses the non-coherent vector L1, for data
// other workgroups of the same kernel wrote with device-scope atomics.
__device__ __forceinline__ uint32_t zha_load_coherent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
