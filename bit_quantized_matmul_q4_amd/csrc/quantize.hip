// quantize.hip -- weight packing (4-bit, groups of 256 or 32, fp16 scale + minimum) and
// Q8_1 activation quantization for gfx950.
//
// Both kernels are HBM-streaming passes that must reproduce the defining fp32
// arithmetic bit for bit: every decision (min/max, the fp32 divisions, the
// fp16 rounding, the round-half-to-even of the codes) uses correctly rounded
// IEEE operations (__fdiv_rn, __fsub_rn, __fmul_rn, rintf, v_cvt_f16_f32 with
// round-to-nearest-even) and nothing is contracted into an FMA.
//
// Formats: the HFQ4-G256 weight format and the Q8_1 activation format of the
// hipfire MMQ-prefill note (ai-navigate-news.com article, list of changes);
// the byte layout is this library's (see q4mi.h).
#include "q4mi_device.h"
#include "q4mi_kernels.h"

namespace q4mi {

// One wave per run of 256 weights: lane l holds elements 4l .. 4l+3 (one
// 16-byte load per lane, 1 KiB per wave).  Codes of elements 32j+i and
// 32j+i+16 share byte 16j+i, so the lane holding elements 32j+16+4u.. (lane%8
// >= 4) hands its codes to lane-4, which writes one dword of four bytes.  GS
// is the (scale, minimum) group: 256 (the whole wave) or 32 (eight lanes).
template <int GS>
__global__ __launch_bounds__(256) void k_q4_pack(const float *__restrict__ W,
                                                 uint8_t *__restrict__ qs,
                                                 uint32_t *__restrict__ sm, int64_t ngroups)
{
    static_assert(GS == 256 || GS == 32, "group of 256 or 32");
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * (blockDim.x / kWave);
    for (int64_t grp = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
         grp < ngroups; grp += stride) {
        // rows are K = 256 * G floats long, so group grp starts at grp * 256
        const float4 v = *reinterpret_cast<const float4 *>(W + grp * kGroup + lane * 4);
        float mn = fminf(fminf(v.x, v.y), fminf(v.z, v.w));
        float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
#pragma unroll
        for (int o = GS / 8; o >= 1; o >>= 1) {
            mn = fminf(mn, __shfl_xor(mn, o));
            mx = fmaxf(mx, __shfl_xor(mx, o));
        }
        mn = __fadd_rn(mn, 0.0f);  // a zero minimum or maximum counts as +0
        mx = __fadd_rn(mx, 0.0f);
        const float range = __fsub_rn(mx, mn);
        const uint16_t s16 = f32_to_f16_bits(__fdiv_rn(range, 15.0f));
        const uint16_t m16 = f32_to_f16_bits(mn);
        const float sf = f16_bits_to_f32(s16), mf = f16_bits_to_f32(m16);
        const float e[4] = {v.x, v.y, v.z, v.w};
        uint32_t codes = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            int q = 0;
            if (sf != 0.0f) {
                const float r = rintf(__fdiv_rn(__fsub_rn(e[t], mf), sf));
                q = r < 0.0f ? 0 : (r > 15.0f ? 15 : (int)r);
            }
            codes |= (uint32_t)q << (8 * t);
        }
        const uint32_t high = __shfl_down(codes, 4);
        if ((lane & 7) < 4) {
            const int64_t byte = grp * (kGroup / 2) + 16 * (lane >> 3) + 4 * (lane & 7);
            *reinterpret_cast<uint32_t *>(qs + byte) = codes | (high << 4);
        }
        if (GS == 256 && lane == 0) sm[grp] = (uint32_t)s16 | ((uint32_t)m16 << 16);
        if (GS == 32 && (lane & 7) == 0) sm[grp * 8 + (lane >> 3)] = (uint32_t)s16 | ((uint32_t)m16 << 16);
    }
}

// Eight lanes per block of 32 activations, four per lane.  A wave takes 128
// consecutive float4 per step, two 16-byte loads per lane 1 KB apart, both in
// flight before any arithmetic (non-temporal: x is read once).  The flat element index works across rows
// because K is a multiple of 32, so the eight lanes of a block are all inside
// or all outside [0, nvec4); lanes past the end reload the last vector and
// store nothing.  Block max and sum: DPP within each group of eight lanes.
__global__ __launch_bounds__(256) void k_q8_1_quantize(const float *__restrict__ x,
                                                       int8_t *__restrict__ qa,
                                                       uint32_t *__restrict__ ds, int64_t nvec4)
{
    constexpr int kLoads = 2;
    const int lane = threadIdx.x & 63;
    const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    for (int64_t base = wave0 * (kWave * kLoads); base < nvec4; base += nwaves * (kWave * kLoads)) {
        float4 v[kLoads];
#pragma unroll
        for (int h = 0; h < kLoads; ++h)
            v[h] = __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const float4_t *>(x4) +
                                                                         min(base + kWave * h + lane, nvec4 - 1)));
#pragma unroll
        for (int h = 0; h < kLoads; ++h) {
            const int64_t i = base + kWave * h + lane;
            float amax = fmaxf(fmaxf(fabsf(v[h].x), fabsf(v[h].y)), fmaxf(fabsf(v[h].z), fabsf(v[h].w)));
            amax = fmaxf(amax, dpp_f32<kDppQuadSwap1>(amax));
            amax = fmaxf(amax, dpp_f32<kDppQuadSwap2>(amax));
            amax = fmaxf(amax, dpp_f32<kDppRowHalfMirror>(amax));
            const uint16_t d16 = q8_1_scale(amax);
            const float df = f16_bits_to_f32(d16), rdf = q8_1_rcp(df);
            const float e[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
            uint32_t packed = 0;
            int sum = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int a = q8_1_code(e[t], df, rdf);
                sum += a;
                packed |= ((uint32_t)a & 0xFFu) << (8 * t);
            }
            sum += __builtin_amdgcn_update_dpp(0, sum, kDppQuadSwap1, 0xF, 0xF, false);
            sum += __builtin_amdgcn_update_dpp(0, sum, kDppQuadSwap2, 0xF, 0xF, false);
            sum += __builtin_amdgcn_update_dpp(0, sum, kDppRowHalfMirror, 0xF, 0xF, false);
            if (i < nvec4) {
                reinterpret_cast<uint32_t *>(qa)[i] = packed;
                if ((i & 7) == 0) ds[i >> 3] = q8_1_ds(d16, df, sum);
            }
        }
    }
}

hipError_t launch_q4_pack(const float *W, int64_t N, int64_t K, int group, uint8_t *qs, uint16_t *sm,
                          int num_cus, hipStream_t stream)
{
    const int64_t ngroups = N * (K / kGroup);  // runs of 256 weights, one wave each
    int64_t blocks = (ngroups + 3) / 4;
    const int64_t cap = (int64_t)num_cus * 32;
    if (blocks > cap) blocks = cap;
    if (group == 32)
        hipLaunchKernelGGL(k_q4_pack<32>, dim3((unsigned)blocks), dim3(256), 0, stream, W, qs,
                           reinterpret_cast<uint32_t *>(sm), ngroups);
    else
        hipLaunchKernelGGL(k_q4_pack<256>, dim3((unsigned)blocks), dim3(256), 0, stream, W, qs,
                           reinterpret_cast<uint32_t *>(sm), ngroups);
    return hipGetLastError();
}

hipError_t launch_q8_1_quantize(const float *x, int64_t M, int64_t K, int8_t *qa, uint16_t *ds,
                                int num_cus, hipStream_t stream)
{
    const int64_t nvec4 = M * K / 4;
    int64_t blocks = (nvec4 + 511) / 512;  // 512 float4 per workgroup step
    const int64_t cap = (int64_t)num_cus * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(k_q8_1_quantize, dim3((unsigned)blocks), dim3(256), 0, stream, x, qa,
                       reinterpret_cast<uint32_t *>(ds), nvec4);
    return hipGetLastError();
}

}  // namespace q4mi
