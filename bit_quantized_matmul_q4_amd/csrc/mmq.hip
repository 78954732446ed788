// mmq.hip -- prefill GEMM on Q8_1 activations and 4-bit group-256 weights
// with gfx950 int8 matrix cores ("MMQ": the hipfire MMQ-prefill note, list of
// changes -- Q8_1 pre-quantized activations, LDS staging, i8 matrix products
// over 128x128 output tiles).
//
//   y[m][n] = sum_g ( s[n][g] * sum_{b in g} d[m][b] * I[m][n][b]
//                     + mn[n][g] * X[m][g] )
//   I[m][n][b] = sum_{k in block b} a[m][k] * q[n][k]     (exact int32, MFMA)
//   X[m][g]    = sum_{b in g} d[m][b] * sum_{k in block b} a[m][k]
//
// Design for CDNA4:
//   * One v_mfma_i32_32x32x32_i8 covers exactly one Q8_1 block (K = 32), so its
//     int32 result is the block dot I.  Weights are the A operand (output rows
//     n), activations the B operand (output columns m): each lane owns one
//     activation row m, so the block scale d[m][b] is a scalar per lane.
//   * The VALU epilogue, not the matrix core, bounds the kernel: one 32x32x32
//     int8 MFMA takes 32 cycles per SIMD, while one VALU op over its 1024
//     outputs takes 64.  Scaling each block dot in fp32 (acc += d * (float)I)
//     costs two ops per output and block (at most 25 % of the int8 peak), so
//     the fp32-output kernels combine the blocks of a group in integers:
//       - the weights enter the MFMA centred, q - 8 in [-8, 7], so
//         |I'| = |sum a (q - 8)| <= 32 * 127 * 8 = 32512;
//       - each row's block scales in the group become 13-bit integers
//         D[m][b] = rint(d[m][b] / step[m][g]), step = max_b d[m][b] / 8191;
//       - acc = sum_b D * I' by one v_mad_i32_i24 per output and block
//         (8 * 32512 * 8191 < 2^31 for any input: no overflow);
//       - per group: y += scale * step * acc + (minimum + 8 scale) * X.
//     Each block's scale is then exact to within step / 2, which on the
//     N(0, 1) activations with 1 % 20x outliers against N(0, 0.02) weights
//     gives NMSE ~3e-8 and max error ~2e-4 of max |y| (fp32 block scaling:
//     ~1e-13).  Centring matters: uncentred codes carry a mean of 7.5 * sum a
//     that cancels against the minimum term and amplifies the scale rounding
//     (NMSE ~2e-7 at 13 bits).  The integer block dots themselves (the test
//     hook) and the group-32 kernel, whose scale changes every block, keep the
//     uncentred codes and the fp32 per-block epilogue.
//   * Per 128x128 tile and 256-wide K step (one weight group) the workgroup
//     stages in LDS: the weights unpacked to int8 (each 16-byte packed block
//     becomes the low-nibble run k 0..15 and the high-nibble run k 16..31), the
//     int8 activations, the block scales (integer D, or fp32 d), the group's
//     per-row X[m][g] and step, and the (scale, minimum) pairs as fp32.  Rows
//     are padded to 272 bytes so 16-byte reads of consecutive rows hit
//     distinct banks.  Everything per (row, block) is computed once per
//     workgroup, so the MFMA loop itself does only LDS reads, MFMAs and the
//     epilogue.
//   * Loads are raw buffer loads: rows past M or N read as zeros without a
//     branch.  Tiles are mapped so each XCD works on a contiguous run of
//     tiles (m fastest), which keeps the shared activation and weight tiles in
//     that XCD's L2.
//   * 256 threads = 2 x 2 waves of 64x64 outputs (2x2 MFMA tiles); about 75 KB
//     of LDS, so two workgroups share a CU and hide each other's staging.
#include "q4mi_device.h"
#include "q4mi_kernels.h"
#include "mmq_tiles.h"

namespace q4mi {

namespace {

constexpr int kTile = 128;             // output tile: 128 (n) x 128 (m)
constexpr int kBlocks = 8;             // Q8_1 blocks per group (per K step)
constexpr int kRow = 256 + 16;         // LDS bytes per row per step (A and B)
constexpr int kLdsA = kTile * kRow;
constexpr int kLdsB = kTile * kRow;
constexpr int kLdsD = kTile * kBlocks * 4;   // block scales: integer D, or d as fp32
constexpr int kLdsX = kTile * 4;             // X[m][g] as fp32
constexpr int kLdsStep = kTile * 4;          // step[m][g] as fp32
constexpr int kLdsSM = kTile * 8;            // (scale, minimum) as fp32 pairs
constexpr int kLdsStage = kLdsA + kLdsB + kLdsD + kLdsX + kLdsStep + kLdsSM;
constexpr int kDMax = 8191;                  // integer block scales D in [0, 8191]

// q - 8 for four codes q in [0, 15] held one per byte, as int8 bytes (the
// bytes cannot carry into each other)
__device__ __forceinline__ uint32_t centre_codes(uint32_t q) { return (q + 0x78787878u) ^ 0x80808080u; }
// Group-32 weights: the kLdsD region holds d16 | (sum a) << 16 per (block,
// row) and the (scale, minimum) pairs are fp32 per (block, weight row):
// 80 KiB, so two workgroups still share a CU.
constexpr int kLdsSM32 = kTile * kBlocks * 8;
__host__ __device__ constexpr int mmq_lds_bytes(bool g32) { return g32 ? kLdsA + kLdsB + kLdsD + kLdsSM32 : kLdsStage; }

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// y and idot point at the sub-problem's first output; ldy / ldi are the row
// strides (elements) of the full outputs.
//
// 512 threads = 8 waves: wave (wn, wm) computes weight rows 64wn .. 64wn+63
// (two 32-row MFMA tiles) and activation rows 32wm .. 32wm+31 (one tile).
// One LDS stage of ~75 KB and at most 128 VGPRs per lane, so two workgroups
// share a CU (4 waves per SIMD) and one's staging and barriers overlap the
// other's MFMA loop.
// Output modes: fp32 y; the int32 block dots (test hook); or y quantized to
// Q8_1 along n in the epilogue (qo int8 [M][ldy], dso [M][ldy/32]) for a
// consumer that takes Q8_1 activations.
enum { kOutY = 0, kOutDots = 1, kOutQ8 = 2 };

// kG32: group-32 weights, one (scale, minimum) pair per Q8_1 block, applied in
// the per-block epilogue: y += scale * (d * I) + minimum * (d * sum a).
template <int kMode, bool kG32 = false>
__global__ __launch_bounds__(512, kMode == kOutDots ? 1 : 4) void k_mmq(
    const int8_t *__restrict__ qa, const uint32_t *__restrict__ ds, const uint8_t *__restrict__ qs,
    const uint32_t *__restrict__ sm, float *__restrict__ y, int32_t *__restrict__ idot,
    int8_t *__restrict__ qo, uint32_t *__restrict__ dso, int M, int N, int K, int tiles_m, int64_t ldy,
    int64_t ldi, int vec_store, int gps)
{
    constexpr bool kDots = kMode == kOutDots;
    constexpr bool kInt = !kDots && !kG32;  // centred codes, integer block scales
    static_assert(!kG32 || kMode == kOutY, "group-32 weights: fp32 output");
    __shared__ __attribute__((aligned(16))) uint8_t lds[mmq_lds_bytes(kG32)];
    uint8_t *const sA = lds;
    uint8_t *const sB = lds + kLdsA;
    float *const sD = reinterpret_cast<float *>(lds + kLdsA + kLdsB);    // [block][row]
    int *const sDi = reinterpret_cast<int *>(lds + kLdsA + kLdsB);  // kInt: [block][row]
    float *const sX = reinterpret_cast<float *>(lds + kLdsA + kLdsB + kLdsD);
    float *const sStep = reinterpret_cast<float *>(lds + kLdsA + kLdsB + kLdsD + kLdsX);
    float2 *const sSM = reinterpret_cast<float2 *>(lds + kLdsA + kLdsB + kLdsD + kLdsX + kLdsStep);
    uint32_t *const sDA = reinterpret_cast<uint32_t *>(lds + kLdsA + kLdsB);      // kG32: [block][row]
    float2 *const sSM32 = reinterpret_cast<float2 *>(lds + kLdsA + kLdsB + kLdsD);  // kG32: [block][row]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;      // 64 weight rows x 32 activation rows
    const int l32 = lane & 31, half = lane >> 5;  // MFMA column / k-half
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int mt = tile % tiles_m, nt = tile / tiles_m;
    const int n0 = nt * kTile, m0 = mt * kTile;
    const int G = K / kGroup, B = K / kBlock;
    // K split blockIdx.y covers groups [g_lo, g_hi); its partial sums go to
    // their own [M][ldy] slice of y (the caller's workspace when split)
    const int g_lo = blockIdx.y * gps, g_hi = min(G, g_lo + gps);
    if (kMode == kOutY) y += (int64_t)blockIdx.y * M * ldy;
    const uint32_t rowA = K / 2;

    const rsrc_t r_qs = make_rsrc(qs, (uint32_t)N * rowA);
    const rsrc_t r_qa = make_rsrc(qa, (uint32_t)M * (uint32_t)K);
    const rsrc_t r_ds = make_rsrc(ds, kDots ? 0u : (uint32_t)M * B * 4u);
    const rsrc_t r_sm = make_rsrc(sm, kDots ? 0u : (uint32_t)N * (kG32 ? B : G) * 4u);

    // ---- stage one group (256 of K) in LDS ----
    // weights: chunks tid and tid+512 (row idx/8, block idx%8), unpacked to int8;
    // activations: row tid/4, blocks 2(tid%4) and 2(tid%4)+1, with d and sum(a)
    auto stage_group = [&](int g) {
        const int arow = tid >> 2, aq = tid & 3;
        const int m = min(m0 + arow, M);  // rows past M or N read zeros
        uint4 w[2], a[4];
        uint32_t dsw[2] = {0, 0}, psm = 0, psm32[2] = {0, 0};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int idx = tid + 512 * p;
            const int n = min(n0 + (idx >> 3), N);
            w[p] = buf_load16(r_qs, (uint32_t)n * rowA + g * 128 + (idx & 7) * 16);
        }
        const uint32_t base = (uint32_t)m * (uint32_t)K + g * 256 + aq * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = buf_load16(r_qa, base + i * 16);
        if (!kDots) {
            const uint32_t o = ((uint32_t)m * B + g * kBlocks + aq * 2) * 4u;
            dsw[0] = buf_load4(r_ds, o);
            dsw[1] = buf_load4(r_ds, o + 4);
            if (kG32) {
                // pair of (weight row idx / 8, block idx % 8) for idx = tid, tid + 512
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int idx = tid + 512 * p;
                    psm32[p] = buf_load4(r_sm, ((uint32_t)min(n0 + (idx >> 3), N) * B + g * kBlocks + (idx & 7)) * 4u);
                }
            } else if (tid < kTile) {
                psm = buf_load4(r_sm, ((uint32_t)min(n0 + tid, N) * G + g) * 4u);
            }
        }
        __syncthreads();  // every wave is done reading the previous group
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int idx = tid + 512 * p, row = idx >> 3, blk = idx & 7;
            uint4 lo = make_uint4(w[p].x & 0x0F0F0F0Fu, w[p].y & 0x0F0F0F0Fu,
                                  w[p].z & 0x0F0F0F0Fu, w[p].w & 0x0F0F0F0Fu);
            uint4 hi = make_uint4((w[p].x >> 4) & 0x0F0F0F0Fu, (w[p].y >> 4) & 0x0F0F0F0Fu,
                                  (w[p].z >> 4) & 0x0F0F0F0Fu, (w[p].w >> 4) & 0x0F0F0F0Fu);
            if (kInt) {
                lo = make_uint4(centre_codes(lo.x), centre_codes(lo.y), centre_codes(lo.z), centre_codes(lo.w));
                hi = make_uint4(centre_codes(hi.x), centre_codes(hi.y), centre_codes(hi.z), centre_codes(hi.w));
            }
            *reinterpret_cast<uint4 *>(sA + row * kRow + blk * 32) = lo;
            *reinterpret_cast<uint4 *>(sA + row * kRow + blk * 32 + 16) = hi;
        }
        float xpart = 0.0f, dblk[2] = {0.0f, 0.0f};
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            const uint4 c0 = a[2 * b2], c1 = a[2 * b2 + 1];
            *reinterpret_cast<uint4 *>(sB + arow * kRow + aq * 64 + b2 * 32) = c0;
            *reinterpret_cast<uint4 *>(sB + arow * kRow + aq * 64 + b2 * 32 + 16) = c1;
            if (!kDots) {
                int sa = 0;
                sa = __builtin_amdgcn_sdot4((int)c0.x, 0x01010101, sa, false);
                sa = __builtin_amdgcn_sdot4((int)c0.y, 0x01010101, sa, false);
                sa = __builtin_amdgcn_sdot4((int)c0.z, 0x01010101, sa, false);
                sa = __builtin_amdgcn_sdot4((int)c0.w, 0x01010101, sa, false);
                sa = __builtin_amdgcn_sdot4((int)c1.x, 0x01010101, sa, false);
                sa = __builtin_amdgcn_sdot4((int)c1.y, 0x01010101, sa, false);
                sa = __builtin_amdgcn_sdot4((int)c1.z, 0x01010101, sa, false);
                sa = __builtin_amdgcn_sdot4((int)c1.w, 0x01010101, sa, false);
                const float d = f16_bits_to_f32(dsw[b2] & 0xFFFFu);
                dblk[b2] = d;
                if (kG32)  // |sum a| <= 4064 fits 16 bits
                    sDA[(aq * 2 + b2) * kTile + arow] = (dsw[b2] & 0xFFFFu) | ((uint32_t)sa << 16);
                else if (!kInt)
                    sD[(aq * 2 + b2) * kTile + arow] = d;  // block-major: conflict-free reads
                xpart = fmaf(d, (float)sa, xpart);
            }
        }
        if (kInt) {
            // the row's eight blocks sit in four consecutive lanes (one quad):
            // D = rint(d * 8191 / max d) and step = max d / 8191, so that
            // D * step is within step / 2 of d (any rounding of the factors
            // only moves which integer D is, not that bound)
            float dmax = fmaxf(dblk[0], dblk[1]);
            dmax = fmaxf(dmax, dpp_f32<kDppQuadSwap1>(dmax));
            dmax = fmaxf(dmax, dpp_f32<kDppQuadSwap2>(dmax));
            const float inv = dmax > 0.0f ? (float)kDMax * __builtin_amdgcn_rcpf(dmax) : 0.0f;
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2)
                sDi[(aq * 2 + b2) * kTile + arow] = min(kDMax, (int)rintf(dblk[b2] * inv));
            if (aq == 0) sStep[arow] = dmax * (1.0f / (float)kDMax);
        }
        if (!kDots) {
            // the row's eight blocks sit in four consecutive lanes
            xpart += dpp_f32<kDppQuadSwap1>(xpart);
            xpart += dpp_f32<kDppQuadSwap2>(xpart);
            if (kG32) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int idx = tid + 512 * p;
                    sSM32[(idx & 7) * kTile + (idx >> 3)] =
                        make_float2(f16_bits_to_f32(psm32[p] & 0xFFFFu), f16_bits_to_f32(psm32[p] >> 16));
                }
            } else {
                if (aq == 0) sX[arow] = xpart;
                if (tid < kTile) {
                    // centred codes: w = scale * (q - 8) + (minimum + 8 scale)
                    const float sc = f16_bits_to_f32(psm & 0xFFFFu), mn = f16_bits_to_f32(psm >> 16);
                    sSM[tid] = make_float2(sc, kInt ? fmaf(8.0f, sc, mn) : mn);
                }
            }
        }
        __syncthreads();
    };

    float yacc[2][16];
#pragma unroll
    for (int ta = 0; ta < 2; ++ta)
#pragma unroll
        for (int e = 0; e < 16; ++e) yacc[ta][e] = 0.0f;

    const int arow_w = wm * 32 + l32;  // this lane's activation row in the tile
#pragma unroll 1
    for (int g = g_lo; g < g_hi; ++g) {
        stage_group(g);

        // ---- 8 blocks x 2 tiles: MFMA + per-block epilogue ----
        // the MFMA of the next tile is issued before the epilogue of the last.
        // iacc: the group's integer sums sum_b D * I' (kInt; block 0 assigns
        // them); in the other modes only the fence below touches it
        int iacc[2][16];
        if (!kInt) {
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int e = 0; e < 16; ++e) iacc[ta][e] = 0;
        }
        const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        auto a_op = [&](int b, int ta) {
            return *reinterpret_cast<const v4i *>(sA + (wn * 64 + ta * 32 + l32) * kRow + b * 32 + half * 16);
        };
        auto b_op = [&](int b) {
            return *reinterpret_cast<const v4i *>(sB + arow_w * kRow + b * 32 + half * 16);
        };
        // per block: d and (group-32 only) d * sum a of this lane's activation
        // row; with kInt the integer scale D (its bits in .x)
        auto dscale = [&](int b) -> float2 {
            if (kDots) return make_float2(0.0f, 0.0f);
            if (kInt) return make_float2(__int_as_float(sDi[b * kTile + arow_w]), 0.0f);
            if (kG32) {
                const uint32_t v = sDA[b * kTile + arow_w];
                const float d = f16_bits_to_f32(v & 0xFFFFu);
                return make_float2(d, d * (float)(int)(int16_t)(v >> 16));  // exact: 11 x 12 bits
            }
            return make_float2(sD[b * kTile + arow_w], 0.0f);
        };
        auto epilogue = [&](const v16i &I, int ta, float2 dd, int b) {
            const float d = dd.x;
            if (kG32) {
                // y += scale[n][b] * (d * I) + minimum[n][b] * (d * sum a); rows
                // 8q + 4 half + r, two (scale, minimum) pairs per 16-byte read
#pragma unroll
                for (int p2 = 0; p2 < 8; ++p2) {
                    const int e = 2 * p2;
                    const float4 v = *reinterpret_cast<const float4 *>(
                        sSM32 + b * kTile + wn * 64 + ta * 32 + 8 * (e >> 2) + 4 * half + (e & 3));
                    yacc[ta][e] = fmaf(v.x, d * (float)I[e], fmaf(v.y, dd.y, yacc[ta][e]));
                    yacc[ta][e + 1] = fmaf(v.z, d * (float)I[e + 1], fmaf(v.w, dd.y, yacc[ta][e + 1]));
                }
            } else if (kDots) {
                const int m = m0 + arow_w;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int n = n0 + wn * 64 + ta * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
                    if (m < M && n < N) idot[(int64_t)m * ldi + (int64_t)n * B + g * kBlocks + b] = I[e];
                }
            } else {
                // |I'| < 2^15 and D < 2^13: exact in the 24-bit multiplier
                const int D = __float_as_int(dd.x);
                if (b == 0) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) iacc[ta][e] = __mul24(I[e], D);
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) iacc[ta][e] = __mul24(I[e], D) + iacc[ta][e];
                }
            }
        };
        v4i a1 = a_op(0, 1), bv = b_op(0);
        float2 dcur = dscale(0);
        v16i prev = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op(0, 0), bv, zero, 0, 0, 0);
        float2 dprev = dcur;
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
            // tile 1 of block b
            const v16i t1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bv, zero, 0, 0, 0);
            epilogue(prev, 0, dprev, b);
            prev = t1;
            dprev = dcur;
            if (b + 1 < kBlocks) {
                // tile 0 of block b+1; its operands are read after the running
                // sums exist, so no MFMA is hoisted above an earlier epilogue
                if (kInt && b == 0)  // tile 1's sums do not exist yet
                    asm volatile("" : "+v"(iacc[0][0]), "+v"(iacc[0][15])::"memory");
                else
                    asm volatile("" : "+v"(iacc[0][0]), "+v"(iacc[0][15]), "+v"(iacc[1][0]),
                                 "+v"(iacc[1][15])::"memory");
                bv = b_op(b + 1);
                a1 = a_op(b + 1, 1);
                dcur = dscale(b + 1);
                const v16i t0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_op(b + 1, 0), bv, zero, 0, 0, 0);
                epilogue(prev, 1, dprev, b);
                prev = t0;
                dprev = dcur;
            }
        }
        epilogue(prev, 1, dprev, kBlocks - 1);

        if (kInt) {
            // ---- group epilogue: y += scale * step * acc + (minimum + 8 scale) * X ----
            // rows 8q + 4 half + r (r = 0..3) of each tile are consecutive:
            // two (scale, minimum) pairs per 16-byte read
            const float xm = sX[arow_w], step = sStep[arow_w];
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int p2 = 0; p2 < 8; ++p2) {
                    const int e = 2 * p2;
                    const float4 v = *reinterpret_cast<const float4 *>(sSM + wn * 64 + ta * 32 + 8 * (e >> 2) + 4 * half + (e & 3));
                    yacc[ta][e] = fmaf(v.x, step * (float)iacc[ta][e], fmaf(v.y, xm, yacc[ta][e]));
                    yacc[ta][e + 1] = fmaf(v.z, step * (float)iacc[ta][e + 1], fmaf(v.w, xm, yacc[ta][e + 1]));
                }
        }
    }

    if (kMode == kOutQ8) {
        // Each 32-row MFMA tile is one Q8_1 block along n for this lane's row
        // m: 16 values here and 16 in lane ^ 32.  N is a multiple of 32, so a
        // block lies wholly inside or outside [0, N).
        const int m = m0 + arow_w;
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {
            const int nb = n0 + wn * 64 + ta * 32;  // first n of the block
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(yacc[ta][e]));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const uint16_t d16 = q8_1_scale(amax);
            const float df = f16_bits_to_f32(d16), rdf = q8_1_rcp(df);
            int sum = 0;
            uint32_t packed[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                packed[q] = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int a = q8_1_code(yacc[ta][4 * q + r], df, rdf);
                    sum += a;
                    packed[q] |= ((uint32_t)a & 0xFFu) << (8 * r);
                }
            }
            sum += __shfl_xor(sum, 32);
            if (m < M && nb < N) {
                // rows n = nb + 8q + 4 half + r: four runs of four codes
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint32_t *>(qo + (int64_t)m * ldy + nb + 8 * q + 4 * half) = packed[q];
                if (half == 0) dso[(int64_t)m * (ldy / kBlock) + nb / kBlock] = q8_1_ds(d16, df, sum);
            }
        }
    } else if (!kDots) {
        const int m = m0 + arow_w;
        if (m < M) {
#pragma unroll
            for (int ta = 0; ta < 2; ++ta)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int n = n0 + wn * 64 + ta * 32 + 8 * r4 + 4 * half;
                    float *dst = y + (int64_t)m * ldy + n;
                    if (vec_store && n + 3 < N) {
                        *reinterpret_cast<float4 *>(dst) =
                            make_float4(yacc[ta][4 * r4], yacc[ta][4 * r4 + 1], yacc[ta][4 * r4 + 2],
                                        yacc[ta][4 * r4 + 3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (n + i < N) dst[i] = yacc[ta][4 * r4 + i];
                    }
                }
        }
    }
}

// y[m][n] (row stride ldy) = sum over splits of partial[s][m][n] (dense
// [nsplit][M][N]), in split order
__global__ __launch_bounds__(256) void k_mmq_split_sum(const float *__restrict__ partial,
                                                       float *__restrict__ y, int M, int N,
                                                       int64_t ldy, int nsplit)
{
    const int64_t count = (int64_t)M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        float v = 0.0f;
        for (int s = 0; s < nsplit; ++s) v += partial[(int64_t)s * count + i];
        y[(i / N) * ldy + i % N] = v;
    }
}

// As k_mmq_split_sum, then the sums quantized to Q8_1 along n: eight lanes per
// block of 32 outputs, four per lane (N is a multiple of 32).
__global__ __launch_bounds__(256) void k_mmq_split_sum_q8(const float *__restrict__ partial,
                                                          int8_t *__restrict__ qo,
                                                          uint32_t *__restrict__ dso, int M, int N,
                                                          int64_t ldq, int nsplit)
{
    const int64_t count = (int64_t)M * N, nvec4 = count / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    // stride and nvec4 are multiples of 8: the 8 lanes of a block iterate together
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec4; i += stride) {
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int s = 0; s < nsplit; ++s) {
            const float4 p = reinterpret_cast<const float4 *>(partial + (int64_t)s * count)[i];
            v[0] += p.x;
            v[1] += p.y;
            v[2] += p.z;
            v[3] += p.w;
        }
        float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        const uint16_t d16 = q8_1_scale(amax);
        const float df = f16_bits_to_f32(d16), rdf = q8_1_rcp(df);
        uint32_t packed = 0;
        int sum = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int a = q8_1_code(v[t], df, rdf);
            sum += a;
            packed |= ((uint32_t)a & 0xFFu) << (8 * t);
        }
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        const int64_t m = (4 * i) / N, n = (4 * i) % N;
        *reinterpret_cast<uint32_t *>(qo + m * ldq + n) = packed;
        if ((i & 7) == 0) dso[m * (ldq / kBlock) + n / kBlock] = q8_1_ds(d16, df, sum);
    }
}

// K is split while the grid has at most one workgroup per CU of a full MI355X
// (one resident workgroup cannot hide its own staging; beyond that the
// partials' extra traffic costs more than the split gains).  The split
// depends only on the shape, so the workspace size does too.
constexpr int64_t kSplitCus = 256;

struct SplitCfg {
    int nsplit, gps;
};

SplitCfg choose_split(int64_t M, int64_t N, int K)
{
    const int G = K / kGroup;
    const int64_t tiles = ((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile);
    int s = 1;
    // halve K ranges while the grid is at most one workgroup per CU and each keeps >= 2 groups
    while (tiles * s <= kSplitCus && (G + 2 * s - 1) / (2 * s) >= 2) s *= 2;
    SplitCfg c;
    c.gps = (G + s - 1) / s;
    c.nsplit = (G + c.gps - 1) / c.gps;  // every split non-empty
    return c;
}

// Run over sub-problems whose weights (N rows) and activations (M rows) each
// stay below 2 GiB, the reach of a buffer descriptor with 32-bit offsets.
// With a K split, each sub-problem's partials go to the workspace (dense
// [nsplit][mm][nn]) and a second kernel sums them into y (or into Q8_1).
hipError_t run_tiles(int mode, bool g32, const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                     const uint16_t *sm, int64_t N, int K, float *y, int32_t *idot, int8_t *qo,
                     uint16_t *dso, void *workspace, int num_cus, hipStream_t stream)
{
    const int SPR = K / (g32 ? kBlock : kGroup);  // (scale, minimum) pairs per weight row
    const int64_t n_max = ((kMaxBufferBytes - 1) / (K / 2)) / kTile * kTile;
    const int64_t m_max = ((kMaxBufferBytes - 1) / K) / kTile * kTile;
    const int B = K / kBlock;
    const SplitCfg sc = mode == kOutDots ? SplitCfg{1, K / kGroup} : choose_split(M, N, K);
    uint32_t *dso32 = reinterpret_cast<uint32_t *>(dso);
    for (int64_t m0 = 0; m0 < M; m0 += m_max) {
        const int64_t mm = M - m0 < m_max ? M - m0 : m_max;
        for (int64_t n0 = 0; n0 < N; n0 += n_max) {
            const int64_t nn = N - n0 < n_max ? N - n0 : n_max;
            const int tiles_m = (int)((mm + kTile - 1) / kTile);
            const int64_t tiles = (int64_t)tiles_m * ((nn + kTile - 1) / kTile);
            if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
            const int8_t *qa0 = qa + m0 * K;
            const uint8_t *qs0 = qs + n0 * (K / 2);
            const uint32_t *ds0 = reinterpret_cast<const uint32_t *>(ds + m0 * B * 2);
            const uint32_t *sm0 = reinterpret_cast<const uint32_t *>(sm + n0 * SPR * 2);
            if (mode == kOutDots) {
                hipLaunchKernelGGL(k_mmq<kOutDots>, dim3((unsigned)tiles), dim3(512), 0, stream, qa0,
                                   (const uint32_t *)nullptr, qs0, (const uint32_t *)nullptr,
                                   (float *)nullptr, idot + (m0 * N + n0) * B, (int8_t *)nullptr,
                                   (uint32_t *)nullptr, (int)mm, (int)nn, K, tiles_m, (int64_t)0, N * B, 0,
                                   sc.gps);
            } else if (sc.nsplit > 1) {
                // partials [nsplit][mm][nn] in the workspace, then the sum
                float *part = static_cast<float *>(workspace);
                const int vec_store = (nn % 4 == 0) ? 1 : 0;
                if (g32)
                    hipLaunchKernelGGL((k_mmq<kOutY, true>), dim3((unsigned)tiles, (unsigned)sc.nsplit), dim3(512),
                                       0, stream, qa0, ds0, qs0, sm0, part, (int32_t *)nullptr, (int8_t *)nullptr,
                                       (uint32_t *)nullptr, (int)mm, (int)nn, K, tiles_m, nn, (int64_t)0,
                                       vec_store, sc.gps);
                else
                    hipLaunchKernelGGL(k_mmq<kOutY>, dim3((unsigned)tiles, (unsigned)sc.nsplit), dim3(512), 0,
                                       stream, qa0, ds0, qs0, sm0, part, (int32_t *)nullptr, (int8_t *)nullptr,
                                       (uint32_t *)nullptr, (int)mm, (int)nn, K, tiles_m, nn, (int64_t)0,
                                       vec_store, sc.gps);
                if (hipGetLastError() == hipSuccess) {
                    int64_t sb = (mm * nn + 255) / 256;
                    if (sb > (int64_t)num_cus * 8) sb = (int64_t)num_cus * 8;
                    if (mode == kOutY)
                        hipLaunchKernelGGL(k_mmq_split_sum, dim3((unsigned)sb), dim3(256), 0, stream, part,
                                           y + m0 * N + n0, (int)mm, (int)nn, N, sc.nsplit);
                    else
                        hipLaunchKernelGGL(k_mmq_split_sum_q8, dim3((unsigned)sb), dim3(256), 0, stream, part,
                                           qo + m0 * N + n0, dso32 + m0 * (N / kBlock) + n0 / kBlock,
                                           (int)mm, (int)nn, N, sc.nsplit);
                }
            } else if (mode == kOutY) {
                float *y0 = y + m0 * N + n0;
                const int vec_store = (N % 4 == 0) && (nn % 4 == 0) &&
                                      ((reinterpret_cast<uintptr_t>(y0) & 15) == 0);
                if (g32)
                    hipLaunchKernelGGL((k_mmq<kOutY, true>), dim3((unsigned)tiles, 1u), dim3(512), 0, stream, qa0,
                                       ds0, qs0, sm0, y0, (int32_t *)nullptr, (int8_t *)nullptr, (uint32_t *)nullptr,
                                       (int)mm, (int)nn, K, tiles_m, N, (int64_t)0, vec_store, sc.gps);
                else
                    hipLaunchKernelGGL(k_mmq<kOutY>, dim3((unsigned)tiles, 1u), dim3(512), 0, stream, qa0, ds0,
                                       qs0, sm0, y0, (int32_t *)nullptr, (int8_t *)nullptr, (uint32_t *)nullptr,
                                       (int)mm, (int)nn, K, tiles_m, N, (int64_t)0, vec_store, sc.gps);
            } else {
                hipLaunchKernelGGL(k_mmq<kOutQ8>, dim3((unsigned)tiles, 1u), dim3(512), 0, stream, qa0, ds0,
                                   qs0, sm0, (float *)nullptr, (int32_t *)nullptr, qo + m0 * N + n0,
                                   dso32 + m0 * (N / kBlock) + n0 / kBlock, (int)mm, (int)nn, K, tiles_m, N,
                                   (int64_t)0, 0, sc.gps);
            }
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

// The fp16 matrix-core kernels (mmq_f16.hip) take q4_mmq_gemm and its Q8_1
// variant when their grid of 256 x 128 tiles (one workgroup per CU) keeps
// the CUs evenly busy: at least 128 tiles and either at most one round of
// 256 or rounds at least 80 % full.  Elsewhere (small grids, which the K
// split here keeps busy, and grids that leave most of a last round idle)
// the int8 kernels here are faster.  Measured on MI355X (q4_mmq_gemm incl.
// its prep kernels, us): M = 2048 4096 -> 12288 (768 tiles) 275 vs 319;
// 12288 -> 4096 (256) 240 vs 283; M = 4096 (1536) 512 vs 562; M = 512
// 2560 -> 9216 (144) 56 vs 62; M = 1024 (384, 1.5 rounds) 153 vs 145;
// M = 768 (288) 146 vs 136; M = 256 12288 -> 4096 (32) 148 vs 54.
bool mmq_uses_f16(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    constexpr int64_t kCus = 256;
    const int64_t tiles = ((M + 255) / 256) * ((N + 127) / 128);
    if (tiles < kCus / 2) return false;
    if (tiles <= kCus) return true;
    const int64_t slots = (tiles + kCus - 1) / kCus * kCus;
    return tiles * 5 >= slots * 4;
}

// The int8 design's fp32-output kernels: the pipelined k_mmqi (mmq_i8.hip,
// 128 x 128 tiles, one workgroup per CU) when its grid has at least one tile
// per CU, otherwise k_mmq here (128 x 128 tiles, two per CU, K split for
// small grids).  Grids of more than one but less than two rounds of k_mmqi
// (257 to 511 tiles) also take k_mmq, which runs them in one round (M 512,
// 2560 -> 9216, 288 tiles: 62.5 -> 60.0 us; 384 tiles: the same time; the
// same integer sums, bit-identical).  A function of the shape only.
bool mmq_int8_pipelined(int64_t M, int64_t N, int64_t K)
{
    constexpr int64_t kCus = 256;
    const int64_t tiles = ((M + 255) / 256) * ((N + 127) / 128);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (t128 > kCus && t128 < 2 * kCus) return false;
    return tiles >= 128 && mmqi_supported(M, N, K);
}

// fp32 and Q8_1 output (group-32 weights have no pipelined integer kernel):
// where the pipelined kernel's 128 x 128 tiles fill the CUs in one round (at
// most 256) it beats the fp16 design, whose 256 x 128 tiles then leave at
// least half the CUs idle (measured, q4_mmq_gemm_int8 vs the fp16 route, us:
// 1024 x 12288 -> 4096 152 vs 188; 512 x 4096 -> 8192 57 vs 72; 2048 x 4096
// -> 2048 56 vs 74; 256 x 4096 -> 16384 56 vs 69; 640 x 4096 -> 6144, 240
// tiles, 53 vs 70; with 288 tiles, 512 x 2560 -> 9216, the fp16 design stays
// faster, 53 vs 65).
bool mmq_int8_one_round(int64_t M, int64_t N, int64_t K)
{
    constexpr int64_t kCus = 256;
    return mmq_int8_pipelined(M, N, K) && ((M + 127) / 128) * ((N + 127) / 128) <= kCus;
}

// the fp32- and Q8_1-output routes' choice
bool mmq_f32_uses_f16(int64_t M, int64_t N, int64_t K)
{
    return mmq_uses_f16(M, N, K) && !mmq_int8_one_round(M, N, K);
}

size_t mmq_int8_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || K < kGroup) return 0;
    if (mmq_int8_pipelined(M, N, K)) return mmqi_workspace_bytes(M, N, K);
    const SplitCfg sc = choose_split(M, N, (int)K);
    if (sc.nsplit == 1) return 0;
    // the largest sub-problem's partials (sub-problems split at < 2 GiB reach)
    const int64_t n_max = ((kMaxBufferBytes - 1) / (K / 2)) / kTile * kTile;
    const int64_t m_max = ((kMaxBufferBytes - 1) / K) / kTile * kTile;
    const int64_t mm = M < m_max ? M : m_max, nn = N < n_max ? N : n_max;
    return (size_t)sc.nsplit * mm * nn * sizeof(float);
}

size_t mmq_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || K < kGroup) return 0;
    // the K-split partials of k_mmq (Q8_1 output and group-32 weights take it
    // at any grid the other designs do not), what k_mmqi needs where the fp32
    // and Q8_1 routes take it, the fp16 design's image (the group-32 route
    // takes it wherever mmq_uses_f16 holds)
    size_t need = mmq_f32_uses_f16(M, N, K) ? 0 : mmq_int8_workspace_bytes(M, N, K);
    {
        const SplitCfg sc = choose_split(M, N, (int)K);
        if (sc.nsplit > 1) {
            const int64_t n_max = ((kMaxBufferBytes - 1) / (K / 2)) / kTile * kTile;
            const int64_t m_max = ((kMaxBufferBytes - 1) / K) / kTile * kTile;
            const int64_t mm = M < m_max ? M : m_max, nn = N < n_max ? N : n_max;
            const size_t part = (size_t)sc.nsplit * mm * nn * sizeof(float);
            if (part > need) need = part;
        }
    }
    if (mmq_uses_f16(M, N, K)) {
        const size_t f = mmqf_workspace_bytes(M, N, K);
        if (f > need) need = f;
    }
    return need;
}

hipError_t launch_mmq_int8(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                           const uint16_t *sm, int64_t N, int K, float *y, void *workspace,
                           const DeviceInfo &dev, hipStream_t stream)
{
    if (mmq_int8_pipelined(M, N, K))
        return launch_mmqi(qa, ds, M, qs, sm, N, K, y, nullptr, nullptr, workspace, stream);
    return run_tiles(kOutY, false, qa, ds, M, qs, sm, N, K, y, nullptr, nullptr, nullptr, workspace,
                     dev.num_cus, stream);
}

hipError_t launch_mmq(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                      const uint16_t *sm, int64_t N, int K, float *y, void *workspace,
                      const DeviceInfo &dev, hipStream_t stream)
{
    if (mmq_f32_uses_f16(M, N, K))
        return launch_mmqf(qa, ds, M, qs, sm, N, K, false, y, nullptr, nullptr, workspace, dev.num_cus, stream);
    return launch_mmq_int8(qa, ds, M, qs, sm, N, K, y, workspace, dev, stream);
}

hipError_t launch_mmq_g32(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                          const uint16_t *sm, int64_t N, int K, float *y, void *workspace,
                          const DeviceInfo &dev, hipStream_t stream)
{
    if (mmq_uses_f16(M, N, K))
        return launch_mmqf(qa, ds, M, qs, sm, N, K, true, y, nullptr, nullptr, workspace, dev.num_cus, stream);
    return run_tiles(kOutY, true, qa, ds, M, qs, sm, N, K, y, nullptr, nullptr, nullptr, workspace,
                     dev.num_cus, stream);
}

hipError_t launch_mmq_q8_1(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                           const uint16_t *sm, int64_t N, int K, int8_t *qo, uint16_t *dso,
                           void *workspace, const DeviceInfo &dev, hipStream_t stream)
{
    // the design the fp32 route takes for the shape, so the result is that
    // route's fp32 output quantized
    if (!mmq_f32_uses_f16(M, N, K) && mmq_int8_pipelined(M, N, K))
        return launch_mmqi(qa, ds, M, qs, sm, N, K, nullptr, qo, dso, workspace, stream);
    if (mmq_f32_uses_f16(M, N, K))
        return launch_mmqf(qa, ds, M, qs, sm, N, K, false, nullptr, qo, dso, workspace, dev.num_cus, stream);
    return run_tiles(kOutQ8, false, qa, ds, M, qs, sm, N, K, nullptr, nullptr, qo, dso, workspace,
                     dev.num_cus, stream);
}

hipError_t launch_block_dots(const int8_t *qa, int64_t M, const uint8_t *qs, int64_t N, int K,
                             int32_t *idot, const DeviceInfo &dev, hipStream_t stream)
{
    return run_tiles(kOutDots, false, qa, nullptr, M, qs, nullptr, N, K, nullptr, idot, nullptr, nullptr,
                     nullptr, dev.num_cus, stream);
}

}  // namespace q4mi
