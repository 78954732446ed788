// mmq.hip -- prefill GEMM on Q8_1 activations and 4-bit group-256 weights
// with gfx950 int8 matrix cores ("MMQ": the hipfire MMQ-prefill note, list of
// changes -- Q8_1 pre-quantized activations, LDS staging, i8 matrix products
// over 128x128 output tiles).
//
//   y[m][n] = sum_g ( s[n][g] * sum_{b in g} d[m][b] * I[m][n][b]
//                     + mn[n][g] * sum_{b in g} d[m][b] * A[m][b] )
//   I[m][n][b] = sum_{k in block b} a[m][k] * q[n][k]     (exact int32, MFMA)
//   A[m][b]    = sum_{k in block b} a[m][k]
//
// Design for CDNA4:
//   * One v_mfma_i32_32x32x32_i8 covers exactly one Q8_1 block (K = 32), so its
//     int32 result is the block dot I, which the epilogue scales by d[m][b].
//   * Weights are the A operand (output rows = n), activations the B operand
//     (output columns = m), so each lane owns one activation row m and its
//     block scale d[m][b] is a scalar per lane.
//   * The packed format puts elements i and i+16 of a block in one byte, so
//     the A operand of lane group 0 (k 0..15) is (chunk & 0x0F0F0F0F) and that
//     of lane group 1 (k 16..31) is ((chunk >> 4) & 0x0F0F0F0F): K-contiguous
//     int8 runs, matching a straight 16-byte load of qa for the B operand.
//   * A workgroup computes a 128x128 tile with 4 waves of 64x64 (2x2 MFMA
//     tiles).  Each K step stages one 256-wide group in LDS: 128 rows of packed
//     weights (128 B each), 128 rows of int8 activations (256 B each), the
//     block scales and the group's (scale, minimum).  Row strides are padded
//     by 16 bytes so 16-byte LDS reads of consecutive rows hit distinct banks.
//   * The sum of the activation codes of a block, A[m][b], is taken from the B
//     operand registers with v_dot4 against 0x01010101 (no extra load).
#include "q4mi_device.h"
#include "q4mi_kernels.h"

namespace q4mi {

namespace {

constexpr int kTile = 128;             // output tile: 128 (n) x 128 (m)
constexpr int kBlocks = 8;             // Q8_1 blocks per group (per K step)
constexpr int kRowA = 128 + 16;        // LDS bytes per weight row per step
constexpr int kRowB = 256 + 16;        // LDS bytes per activation row per step
constexpr int kLdsA = kTile * kRowA;
constexpr int kLdsB = kTile * kRowB;
constexpr int kLdsD = kTile * kBlocks * 4;   // d as fp32
constexpr int kLdsSM = kTile * 4;            // (scale, minimum) fp16 pair
constexpr int kLdsTotal = kLdsA + kLdsB + kLdsD + kLdsSM;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

template <bool kDots>
__global__ __launch_bounds__(256) void k_mmq(const int8_t *__restrict__ qa,
                                             const uint32_t *__restrict__ ds,
                                             const uint8_t *__restrict__ qs,
                                             const uint32_t *__restrict__ sm, float *__restrict__ y,
                                             int32_t *__restrict__ idot, int M, int N, int K,
                                             int vec_store)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsTotal];
    uint8_t *sA = lds;
    uint8_t *sB = lds + kLdsA;
    float *sD = reinterpret_cast<float *>(lds + kLdsA + kLdsB);
    uint32_t *sSM = reinterpret_cast<uint32_t *>(lds + kLdsA + kLdsB + kLdsD);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;      // wave's 64x64 quadrant
    const int l32 = lane & 31, half = lane >> 5;  // MFMA column / k-half
    const int n0 = blockIdx.x * kTile, m0 = blockIdx.y * kTile;
    const int G = K / kGroup, B = K / kBlock;
    const int64_t rowA = K / 2;

    float yacc[2][2][16];
    float gacc[2][2][16];
    float xsum[2];
#pragma unroll
    for (int ta = 0; ta < 2; ++ta)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int e = 0; e < 16; ++e) yacc[ta][tb][e] = 0.0f;

    for (int g = 0; g < G; ++g) {
        __syncthreads();
        // ---- stage one group of weights, activations and scales in LDS ----
#pragma unroll
        for (int p = 0; p < 4; ++p) {  // weights: 128 rows x 8 x 16 B
            const int idx = tid + 256 * p, row = idx >> 3, seg = idx & 7;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (n0 + row < N)
                v = *reinterpret_cast<const uint4 *>(qs + (int64_t)(n0 + row) * rowA + g * 128 + seg * 16);
            *reinterpret_cast<uint4 *>(sA + row * kRowA + seg * 16) = v;
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {  // activations: 128 rows x 16 x 16 B
            const int idx = tid + 256 * p, row = idx >> 4, seg = idx & 15;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m0 + row < M)
                v = *reinterpret_cast<const uint4 *>(qa + (int64_t)(m0 + row) * K + g * 256 + seg * 16);
            *reinterpret_cast<uint4 *>(sB + row * kRowB + seg * 16) = v;
        }
        if (!kDots) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {  // block scales d: 128 rows x 8 blocks
                const int idx = tid + 256 * p, row = idx >> 3, b = idx & 7;
                float d = 0.0f;
                if (m0 + row < M)
                    d = f16_bits_to_f32(ds[(int64_t)(m0 + row) * B + g * kBlocks + b] & 0xFFFFu);
                sD[row * kBlocks + b] = d;
            }
            if (tid < kTile)
                sSM[tid] = (n0 + tid < N) ? sm[(int64_t)(n0 + tid) * G + g] : 0u;
        }
        __syncthreads();

        // ---- 8 blocks of 32: MFMA + per-block epilogue ----
        if (!kDots) {
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) gacc[ta][tb][e] = 0.0f;
            xsum[0] = xsum[1] = 0.0f;
        }
        for (int b = 0; b < kBlocks; ++b) {
            v4i av[2], bv[2];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta) {
                const int row = wn * 64 + ta * 32 + l32;
                const uint4 c = *reinterpret_cast<const uint4 *>(sA + row * kRowA + b * 16);
                const int sh = half * 4;
                av[ta] = v4i{(int)((c.x >> sh) & 0x0F0F0F0Fu), (int)((c.y >> sh) & 0x0F0F0F0Fu),
                             (int)((c.z >> sh) & 0x0F0F0F0Fu), (int)((c.w >> sh) & 0x0F0F0F0Fu)};
            }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int row = wm * 64 + tb * 32 + l32;
                bv[tb] = *reinterpret_cast<const v4i *>(sB + row * kRowB + b * 32 + half * 16);
            }
            float dm[2] = {0.0f, 0.0f};
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                if (!kDots) {
                    dm[tb] = sD[(wm * 64 + tb * 32 + l32) * kBlocks + b];
                    int s = 0;
                    s = __builtin_amdgcn_sdot4(bv[tb].x, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4(bv[tb].y, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4(bv[tb].z, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4(bv[tb].w, 0x01010101, s, false);
                    s += __shfl_xor(s, 32);
                    xsum[tb] = fmaf(dm[tb], (float)s, xsum[tb]);
                }
            }
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                    const v16i I = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[ta], bv[tb], zero, 0, 0, 0);
                    if (kDots) {
                        const int m = m0 + wm * 64 + tb * 32 + l32;
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int n = n0 + wn * 64 + ta * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
                            if (m < M && n < N)
                                idot[((int64_t)m * N + n) * B + g * kBlocks + b] = I[e];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            gacc[ta][tb][e] = fmaf(dm[tb], (float)I[e], gacc[ta][tb][e]);
                    }
                }
        }
        if (!kDots) {
            // ---- group epilogue: weight scale and minimum ----
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t smv = sSM[wn * 64 + ta * 32 + 8 * (e >> 2) + 4 * half + (e & 3)];
                    const float sf = f16_bits_to_f32(smv & 0xFFFFu), mf = f16_bits_to_f32(smv >> 16);
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
                        yacc[ta][tb][e] = fmaf(sf, gacc[ta][tb][e], fmaf(mf, xsum[tb], yacc[ta][tb][e]));
                }
        }
    }

    if (!kDots) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int m = m0 + wm * 64 + tb * 32 + l32;
            if (m >= M) continue;
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int n = n0 + wn * 64 + ta * 32 + 8 * r4 + 4 * half;
                    float *dst = y + (int64_t)m * N + n;
                    if (vec_store && n + 3 < N) {
                        *reinterpret_cast<float4 *>(dst) =
                            make_float4(yacc[ta][tb][4 * r4], yacc[ta][tb][4 * r4 + 1],
                                        yacc[ta][tb][4 * r4 + 2], yacc[ta][tb][4 * r4 + 3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (n + i < N) dst[i] = yacc[ta][tb][4 * r4 + i];
                    }
                }
        }
    }
}

}  // namespace

size_t mmq_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_mmq(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                      const uint16_t *sm, int64_t N, int K, float *y, void *, const DeviceInfo &,
                      hipStream_t stream)
{
    const dim3 grid((unsigned)((N + kTile - 1) / kTile), (unsigned)((M + kTile - 1) / kTile));
    // 16-byte stores of y need N % 4 == 0 and a 16-byte aligned y
    const int vec_store = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
    hipLaunchKernelGGL(k_mmq<false>, grid, dim3(256), 0, stream, qa,
                       reinterpret_cast<const uint32_t *>(ds), qs,
                       reinterpret_cast<const uint32_t *>(sm), y, (int32_t *)nullptr, (int)M,
                       (int)N, K, vec_store);
    return hipGetLastError();
}

hipError_t launch_block_dots(const int8_t *qa, int64_t M, const uint8_t *qs, int64_t N, int K,
                             int32_t *idot, const DeviceInfo &, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + kTile - 1) / kTile), (unsigned)((M + kTile - 1) / kTile));
    hipLaunchKernelGGL(k_mmq<true>, grid, dim3(256), 0, stream, qa, (const uint32_t *)nullptr, qs,
                       (const uint32_t *)nullptr, (float *)nullptr, idot, (int)M, (int)N, K, 0);
    return hipGetLastError();
}

}  // namespace q4mi
