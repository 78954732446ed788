// q4mi_device.h -- device-side helpers shared by the library's kernels
// (gfx950 / CDNA4, wave64).  Internal to libq4mi; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4mi {

constexpr int kWave = 64;
constexpr int kGroup = 256;  // weights per (scale, minimum) group along K
constexpr int kBlock = 32;   // activations per Q8_1 block along K

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int16_t_v __attribute__((ext_vector_type(16)));

// DPP controls (GCN/CDNA encoding of the dpp_ctrl field).
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowRor8 = 0x128;     // row_ror:8 (rotate right by 8 within 16 lanes)

template <int ctrl>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 ctrl, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 8 or 16) of one DPP row; every lane
// of the group ends with the same bits (each step adds a commuted pair).
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(G == 8 || G == 16, "group of 8 or 16 lanes");
    v += dpp_f32<kDppQuadSwap1>(v);
    v += dpp_f32<kDppQuadSwap2>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    if (G == 16) v += dpp_f32<kDppRowMirror>(v);
    return v;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f)
{
    // v_cvt_f16_f32: IEEE round-to-nearest-even, fp16 subnormals kept.
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// Q8_1 decisions for one block of 32 values, in IEEE fp32 with correctly
// rounded division (every kernel that produces Q8_1 uses these, so their codes
// agree bit for bit): d16 = fp16(amax / 127); a = clamp(rint(x / d), -127, 127)
// (0 when d is 0); s16 = fp16(d * sum a), the product exact in fp32.
__device__ __forceinline__ uint16_t q8_1_scale(float amax) { return f32_to_f16_bits(__fdiv_rn(amax, 127.0f)); }

// 1/d for q8_1_code: the hardware reciprocal, within one ulp.
__device__ __forceinline__ float q8_1_rcp(float df) { return __builtin_amdgcn_rcpf(df); }

// rint of the correctly rounded quotient x / d, mostly without dividing.  With
// rdf within one ulp of 1/d, q = x * rdf is within 1.5 * 2^-23 |x / d| of the
// exact quotient, and the rounded quotient within 2^-24 |x / d|: below 256 the
// two lie within 2^-14 of each other, so wherever q is more than 2^-11 from a
// half-integer both round to the same integer.  The rare quotients nearer a
// half-integer (exact ties among them) are divided exactly.  From 256 up both
// clamp.  d is an fp16 value, so 1/d is finite whenever d is not 0.
__device__ __forceinline__ int q8_1_code(float x, float df, float rdf)
{
    if (df == 0.0f) return 0;
    const float q = x * rdf;
    float r = rintf(q);
    if (__builtin_expect(!(fabsf(fabsf(q - r) - 0.5f) > 0x1p-11f), 0)) r = rintf(__fdiv_rn(x, df));
    return r < -127.0f ? -127 : (r > 127.0f ? 127 : (int)r);
}

__device__ __forceinline__ uint32_t q8_1_ds(uint16_t d16, float df, int sum)
{
    const uint16_t s16 = f32_to_f16_bits(__fmul_rn(df, (float)sum));
    return (uint32_t)d16 | ((uint32_t)s16 << 16);
}

// Raw buffer loads.  The descriptor carries the buffer size; a load whose
// bytes fall outside it returns zeros, so edge rows need no branch (a branch
// around a load makes the compiler wait for every outstanding load).
// 0x00020000 is the gfx9-family descriptor word 3 (32-bit data format).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off)
{
    const int4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return __builtin_bit_cast(uint4, v);
}

__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Raw buffer store; bytes outside the descriptor are dropped.  A buffer (not
// flat) store keeps the compiler's wait analysis exact: flat accesses count
// against both the vector-memory and the LDS counters, after which every
// later load or LDS read is awaited down to zero outstanding.
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
}

// Streaming variants for data read exactly once (the GEMV weights): the
// non-temporal cache policy (gfx940-family NT bit) keeps them from displacing
// reused lines; on MI355X it also lifts the streamed read rate by about 8 %.
constexpr int kCachePolicyNT = 2;

__device__ __forceinline__ uint4 buf_load16_nt(rsrc_t r, uint32_t off)
{
    const int4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicyNT);
    return __builtin_bit_cast(uint4, v);
}

__device__ __forceinline__ uint32_t buf_load4_nt(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCachePolicyNT);
}

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Loads straight into LDS: lane i's 16 (4) bytes at buffer offset voff + soff
// go to LDS byte address base + 16 i (4 i); soff and base are the same for the
// whole wave.  Written as asm so that the compiler neither tracks nor waits
// for them: a kernel orders them itself (s_waitcnt vmcnt before the barrier
// that publishes the LDS data).  No vector registers are written; M0 (the LDS
// base of the load) is saved in a scratch SGPR and restored, so the compiler's
// own use of M0, if any, is undisturbed, and one wait state separates the
// SALU write of M0 from the load that reads it.  Bytes outside the
// descriptor's range arrive as zeros.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t base)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %4 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(base)),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory");
}

__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t base)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %4 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(base)),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory");
}

// Wait until at most kN vector-memory loads of this wave are outstanding,
// then a workgroup barrier; no memory access moves across it.
template <int kN>
__device__ __forceinline__ void wait_vm_barrier()
{
    static_assert(kN >= 0 && kN < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(kN) : "memory");
}

// Largest byte count a single launch addresses through one descriptor with
// 32-bit offsets; launchers split bigger weight matrices into row ranges.
constexpr int64_t kMaxBufferBytes = (int64_t)1 << 31;

}  // namespace q4mi
