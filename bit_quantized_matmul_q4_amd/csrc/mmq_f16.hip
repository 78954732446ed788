// mmq_f16.hip -- prefill GEMM on Q8_1 activations and 4-bit group-256 weights
// with gfx950 fp16 matrix cores (the MMQ path of the hipfire MMQ-prefill note,
// list of changes: Q8_1 pre-quantized activations, LDS-staged tiles, matrix
// core products over output tiles).
//
//   y[m][n] = sum_k (d[m][k/32] * a[m][k]) * (scale[n][k/256] * q[n][k] + minimum[n][k/256])
//
// Why fp16 and not int8 matrix cores on CDNA4: an int8 MFMA can only contract
// within one Q8_1 block (32 of K), because the activation scale d changes
// every block; scaling its 1024 int32 results costs at least one VALU op per
// output and block, 64 cycles per SIMD against the MFMA's 32, so that design
// is bound by the VALU at no more than half the int8 peak (measured: 14 %).
// Here both scales move into the operands instead, where a whole tile shares
// the cost:
//   * activations: a prep pass writes x'[m][k] = fp16(d * a * F[m]) with one
//     power of two F[m] = 2^(8 - e) per row (e the binary exponent of the
//     row's largest d), so every |x'| < 2^15 and the products d * a (11 x 7
//     bits, exact in fp32) are rounded once;
//   * weights: each 4-bit code goes straight into an fp16 lane as a subnormal
//     (bits q, value q * 2^-24; a code in the high nibble has bits 16 q), and
//     one packed fp16 FMA per pair of codes makes fp16(q * s' + mn') with
//     s' = scale * 2^E[n] and mn' = minimum * 2^E[n], one rounding, where
//     2^E[n] puts the row's largest |minimum| + 15 |scale| in [2^-7, 2^-6)
//     (so the FMA's scale operand s' * 2^24 stays below 2^15);
//   * y = acc * 2^-E[n] / F[m], both exact powers of two.
// Each operand value is within half an fp16 ulp (2^-11 relative) of the exact
// one; on the prefill workloads NMSE ~8e-8 and max |dy| ~3e-4 of max |y|
// against the fp64 definition.
//
// Design for CDNA4:
//   * One v_mfma_f32_32x32x16_f16 takes 32 cycles per SIMD, the same as the
//     int8 32x32x32; per 64-wide K step a computing wave runs 32 of them
//     against about 40 VALU ops (36 to unpack its weights), so the VALU is
//     not the limit.
//   * The K order inside an MFMA is free as long as both operands agree, so
//     each lane unpacks one 32-bit word of packed weights (codes k, k+1, k+2,
//     k+3 and k+16 .. k+19 of a block) into one MFMA's 8 operand slots with
//     four masks, and the prep pass writes the activations in that order.
//   * Tile 256 (m) x 128 (n), 512 threads = 8 waves, two per SIMD: one wave
//     per SIMD loads, one computes 128 x 64 outputs (4 x 2 MFMA tiles).
//   * Each K step (32 KB of image, 4 KB of packed weights) is loaded straight
//     into one of 4 LDS stages (no registers in flight, two steps ahead);
//     the computing waves read and unpack each MFMA round's operands during
//     the round before.
//   * The image is laid out per (256-row tile, K step) in LDS order: the
//     loads are contiguous 1 KB per instruction and the LDS reads (16 bytes
//     per lane, consecutive rows) are conflict-free.
//   * Tiles are mapped so each XCD works on a contiguous run of tiles (m
//     fastest), which keeps the shared activation and weight tiles in its L2.
#include "q4mi_device.h"
#include "q4mi_kernels.h"

namespace q4mi {

namespace {

constexpr int kFm = 256;           // activation rows per tile
constexpr int kFn = 128;           // weight rows per tile
constexpr int kFk = 64;            // K per step: two Q8_1 blocks
constexpr int kFThreads = 256;
constexpr int kStepVecs = 8 * kFm; // 16-byte vectors of the image per (tile, step)
constexpr int kGemmThreads = 512;
constexpr int kStages = 4;                      // K steps in LDS at once
constexpr int kStageVecs = kStepVecs + 2 * kFn; // image + packed weights of a step
constexpr int kSmVecs32 = 2 * kFn / 4;          // group 32: the step's (scale, minimum) pairs
// 144 KB of stages; with group-32 weights 148 KB
__host__ __device__ constexpr int stage_vecs(bool g32) { return kStageVecs + (g32 ? kSmVecs32 : 0); }
static_assert(kStages * stage_vecs(true) * 16 + 3 * kFn * 4 + kFn * 8 <= 160 * 1024, "LDS of a CU");
// largest activation image per launch; bigger M runs in row chunks
constexpr int64_t kImageMaxBytes = (int64_t)256 << 20;

enum { kFOutY = 0, kFOutQ8 = 1 };

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int xcd_tile_f(int pid, int ntiles)
{
    constexpr int kXcd = 8;
    const int per = ntiles / kXcd, rem = ntiles % kXcd;
    const int xcd = pid % kXcd, local = pid / kXcd;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// F[r] for rows r < rows: 2^(8 - e) with e the binary exponent of the row's
// largest block scale (d = f * 2^e, f in [0.5, 1)), so 127 * d * F < 2^15;
// 1 for rows past M, all-zero rows and non-finite scales.  One wave per row.
__device__ __forceinline__ float row_factor(uint32_t dm)
{
    float f = 1.0f;
    if (dm != 0 && dm < 0x7C00u) {
        int e;
        frexpf(f16_bits_to_f32(dm), &e);
        f = ldexpf(1.0f, 8 - e);
    }
    return f;
}

__global__ __launch_bounds__(256) void k_mmqf_rowscale(const uint32_t *__restrict__ ds, int M, int B, int rows,
                                                       float *__restrict__ fs)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    uint32_t dm = 0;
    if (row < M) {
        const uint32_t *p = ds + (int64_t)row * B;
        for (int b = lane; b < B; b += kWave) dm = max(dm, p[b] & 0x7FFFu);  // |d| bits order as values
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dm = max(dm, (uint32_t)__shfl_xor((int)dm, o));
    if (lane == 0) fs[row] = row_factor(dm);
}

// The fp16 activation image of one (256-row tile mt, K step s): thread r
// converts row mt * 256 + r, k in [64 s, 64 s + 64).  Vector (t, h, r) of the
// step (t = 0..3 MFMA of the step, h = Q8_1 block of the step) holds
// x'[k] for k = 64 s + 32 h + {4t, 4t+2, 16+4t, 18+4t, 4t+1, 4t+3, 17+4t, 19+4t}:
// the order in which the GEMM unpacks one 32-bit word of packed weights.
// kRowScale: each thread also finds its row's factor itself (all the row's
// block scales, loaded a round of 8 vectors at a time) and the step-0
// workgroups store it for the GEMM's epilogue, in place of k_mmqf_rowscale;
// taken when those repeated reads stay small (short K, few row tiles).
template <bool kRowScale>
__global__ __launch_bounds__(kFThreads) void k_mmqf_image(const int8_t *__restrict__ qa,
                                                          const uint32_t *__restrict__ ds,
                                                          float *__restrict__ fs, int M, int K,
                                                          uint4 *__restrict__ img)
{
    const int s = blockIdx.x, mt = blockIdx.y, r = threadIdx.x;
    const int S = K / kFk;
    const int m = mt * kFm + r;
    uint4 q[4] = {};
    uint32_t dw[2] = {0, 0};
    float F = 1.0f;
    if (m < M) {
        const uint4 *src = reinterpret_cast<const uint4 *>(qa + (int64_t)m * K + (int64_t)s * kFk);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = src[i];
        const uint32_t *dp = ds + (int64_t)m * (K / kBlock) + 2 * s;
        dw[0] = dp[0];
        dw[1] = dp[1];
        if (kRowScale) {
            const int B4 = K / kBlock / 4;  // 16-byte vectors of the row's (d, s) pairs
            const uint4 *p = reinterpret_cast<const uint4 *>(ds + (int64_t)m * (K / kBlock));
            uint32_t dm = 0;
            for (int b0 = 0; b0 < B4; b0 += 8) {
                uint4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = b0 + u < B4 ? p[b0 + u] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    dm = max(dm, max(max(v[u].x & 0x7FFFu, v[u].y & 0x7FFFu), max(v[u].z & 0x7FFFu, v[u].w & 0x7FFFu)));
            }
            F = row_factor(dm);
            if (s == 0) fs[m] = F;
        } else {
            F = fs[m];
        }
    }
    uint4 *dst = img + ((int64_t)mt * S + s) * kStepVecs + r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float df = f16_bits_to_f32(dw[h] & 0xFFFFu) * F;  // exact: F is a power of two
        const uint32_t w8[8] = {q[2 * h].x, q[2 * h].y, q[2 * h].z, q[2 * h].w,
                                q[2 * h + 1].x, q[2 * h + 1].y, q[2 * h + 1].z, q[2 * h + 1].w};
        // d * a is exact in fp32 (11 x 7 bits); one rounding to fp16
        auto cv = [&](uint32_t w, int byte) -> uint32_t {
            return f32_to_f16_bits(df * (float)(int8_t)(w >> (8 * byte)));
        };
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t lo = w8[t], hi = w8[t + 4];
            uint4 o;
            o.x = cv(lo, 0) | (cv(lo, 2) << 16);
            o.y = cv(hi, 0) | (cv(hi, 2) << 16);
            o.z = cv(lo, 1) | (cv(lo, 3) << 16);
            o.w = cv(hi, 1) | (cv(hi, 3) << 16);
            dst[(2 * t + h) * kFm] = o;
        }
    }
}

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Loads straight into LDS: lane i's 16 (4) bytes at buffer offset voff + soff go to
// LDS byte address base + 16 i (4 i); soff and base are the same for the
// whole wave.
// Written as asm so that the compiler neither tracks nor waits for them: the
// kernel orders them itself with wait_vm_barrier.  No registers are written.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t base)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(base)),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}

__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t base)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, %3 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(base)),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}

// Wait until at most kN vector-memory loads of this wave are outstanding,
// then a workgroup barrier; no memory access moves across it.
template <int kN>
__device__ __forceinline__ void wait_vm_barrier()
{
    static_assert(kN >= 0 && kN < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(kN) : "memory");
}

// y (row stride ldy) for activation rows [0, M) and weight rows [0, N) of
// this sub-problem; img/fs are its activation image and row factors.
// Output modes: fp32 y, or y quantized to Q8_1 along n (qo int8 [M][ldy],
// dso [M][ldy/32]) as q8_1_quantize would do it.  kG32: group-32 weights,
// one (scale, minimum) pair per Q8_1 block; the pairs of a step travel with
// it and the operand constants change per step.
//
// 512 threads = 8 waves, two per SIMD.  Waves 4-7 (one per SIMD) only load
// K steps into LDS; waves 0-3 (one per SIMD) only compute, wave (wm, wn)
// owning activation rows 128 wm .. 128 wm + 127 (four MFMA tiles) x weight
// rows 64 wn .. 64 wn + 63 (two) over whole K steps (4 MFMA rounds per
// step), so the computing waves never issue a vector-memory instruction.
template <int kMode, bool kG32 = false>
__global__ __launch_bounds__(kGemmThreads) void k_mmqf(
    const uint4 *__restrict__ img, uint32_t img_bytes, const float *__restrict__ fs,
    const uint8_t *__restrict__ qs, const uint32_t *__restrict__ sm, float *__restrict__ y,
    int8_t *__restrict__ qo, uint32_t *__restrict__ dso, int M, int N, int K, int tiles_m, int64_t ldy,
    int vec_store)
{
    constexpr int kSV = stage_vecs(kG32);
    __shared__ int4_t lds[kStages * kSV];
    __shared__ uint32_t sSM[2][kFn];
    __shared__ float sScale[kFn];
    __shared__ int sE[kFn];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool consumer = wave < 4;
    const int wn = wave & 1, wm = (wave >> 1) & 1, pw = wave - 4;
    const int l32 = lane & 31, h = lane >> 5;
    const int tile = xcd_tile_f(blockIdx.x, gridDim.x);
    const int mt = tile % tiles_m, nt = tile / tiles_m;
    const int n0 = nt * kFn, m0 = mt * kFm;
    const int S = K / kFk, G = K / kGroup;
    const int P = kG32 ? K / kBlock : G;
    const uint32_t rowq = (uint32_t)K / 2;
    const rsrc_t r_img = make_rsrc(img, img_bytes);
    const rsrc_t r_qs = make_rsrc(qs, (uint32_t)N * rowq);
    const rsrc_t r_sm = make_rsrc(sm, (uint32_t)N * P * 4u);
    uint32_t nrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) nrow[j] = (uint32_t)(n0 + wn * 64 + 32 * j + l32);

    auto pair_bound = [](uint32_t v) {
        return fabsf(f16_bits_to_f32(v >> 16)) + 15.0f * fabsf(f16_bits_to_f32(v & 0xFFFFu));
    };
    auto exponent_of = [](float wmax) {
        int e = 0;
        if (wmax > 0.0f && wmax <= 3.0e38f) {
            frexpf(wmax, &e);
            return -6 - e;
        }
        return 0;
    };
    int E[2] = {0, 0};
    if (kG32) {
        const int r = tid >> 2, q = tid & 3;
        const uint32_t base = (uint32_t)(n0 + r) * (uint32_t)P * 4u;
        float wmax = 0.0f;
        for (int i = q; 4 * i < P; i += 4) {
            const uint4 v = buf_load16(r_sm, base + 16u * (uint32_t)i);
            wmax = fmaxf(fmaxf(wmax, fmaxf(pair_bound(v.x), pair_bound(v.y))), fmaxf(pair_bound(v.z), pair_bound(v.w)));
        }
        wmax = fmaxf(wmax, dpp_f32<kDppQuadSwap1>(wmax));
        wmax = fmaxf(wmax, dpp_f32<kDppQuadSwap2>(wmax));
        if (q == 0) {
            const int e = exponent_of(wmax);
            sE[r] = e;
            sScale[r] = ldexpf(1.0f, -e);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j) E[j] = sE[wn * 64 + 32 * j + l32];
    } else if (consumer) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float wmax = 0.0f;
            for (int g = h; g < G; g += 2) wmax = fmaxf(wmax, pair_bound(buf_load4(r_sm, (nrow[j] * G + g) * 4u)));
            wmax = fmaxf(wmax, __shfl_xor(wmax, 32));
            E[j] = exponent_of(wmax);
            if (h == 0 && wm == 0) sScale[wn * 64 + 32 * j + l32] = ldexpf(1.0f, -E[j]);
        }
    }

    const uint32_t lds0 = lds_addr(lds);
    const uint32_t sm0 = lds_addr(&sSM[0][0]);

    if (!consumer) {
        // ---- producer: step s in stage s % kStages; 8 image pieces (2048
        // vectors / 4 producers), one weight piece, with group-32 weights one
        // piece of pairs: at least 9 loads per step.  Barrier B_s (the
        // consumers' barrier between rounds 2 and 3 of step s) needs step
        // s + 1 in LDS; after it, step s + kStages - 1 goes into the stage of
        // step s - 1, whose reads the consumers finished before B_s. ----
        const uint32_t wcol = (uint32_t)((pw * 64 + lane) & 127), wblk = (uint32_t)((pw * 64 + lane) >> 7);
        const uint32_t wts_v = (n0 + wcol) * rowq + wblk * 16u;
        const uint32_t sm32_v = (n0 + wcol) * (uint32_t)P * 4u + wblk * 4u;
        auto issue = [&](int s) {
            const int sl = min(s, S - 1);
            const uint32_t stage = lds0 + (uint32_t)((s % kStages) * kSV) * 16u;
            const uint32_t goff = (uint32_t)((mt * S + sl) * kStepVecs) * 16u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t v = (uint32_t)(pw * 512 + i * 64);
                dma16(r_img, (v + lane) * 16u, goff, stage + v * 16u);
            }
            dma16(r_qs, wts_v, (uint32_t)sl * 32u, stage + (uint32_t)(kStepVecs + pw * 64) * 16u);
            if (kG32) dma4(r_sm, sm32_v, (uint32_t)sl * 8u, stage + (uint32_t)(kStageVecs * 16 + pw * 256));
        };
        auto issue_sm = [&](int g) {
            if (!kG32 && pw < 2 && g < G) {
                const uint32_t c = (uint32_t)(pw * 64 + lane);
                dma4(r_sm, (n0 + c) * G * 4u, (uint32_t)g * 4u, sm0 + (uint32_t)((g & 1) * kFn + pw * 64) * 4u);
            }
        };
        issue_sm(0);
        for (int s = 0; s < kStages - 2; ++s) issue(s);
        wait_vm_barrier<9 * (kStages - 3)>();  // B_init: step 0
        issue(kStages - 2);
        for (int s = 0; s < S; ++s) {
            wait_vm_barrier<9 * (kStages - 3)>();  // B_s: step s + 1
            issue(s + kStages - 1);
            if ((s & 3) == 0) issue_sm((s >> 2) + 1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }

    // ---- consumer ----
    float16_t acc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;
    auto read_frags = [&](int s, int t, f16x8 (&bv)[4]) {
        const int4_t *act = lds + (s % kStages) * kSV + wm * 128 + l32;
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[i] = __builtin_bit_cast(f16x8, act[(2 * t + h) * kFm + 32 * i]);
    };
    auto read_wts = [&](int s, int4_t (&wq)[2]) {
        const int4_t *wv = lds + (s % kStages) * kSV + kStepVecs + h * kFn + wn * 64 + l32;
#pragma unroll
        for (int j = 0; j < 2; ++j) wq[j] = wv[32 * j];
    };
    half2_t cs[2], cs16[2], cmn[2];
    auto consts = [&](int s) {
        // group 256: the constants of step s's group; group 32: of step s
        const uint32_t *sm32 = reinterpret_cast<const uint32_t *>(lds + (s % kStages) * kSV + kStageVecs);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w = kG32 ? sm32[h * kFn + wn * 64 + 32 * j + l32] : sSM[(s >> 2) & 1][wn * 64 + 32 * j + l32];
            const float sc = f16_bits_to_f32(w & 0xFFFFu), mn = f16_bits_to_f32(w >> 16);
            const _Float16 a = (_Float16)ldexpf(sc, E[j] + 24), b = (_Float16)ldexpf(sc, E[j] + 20),
                           c = (_Float16)ldexpf(mn, E[j]);
            cs[j] = half2_t{a, a};
            cs16[j] = half2_t{b, b};
            cmn[j] = half2_t{c, c};
        }
    };
    auto unpack = [&](int t, const int4_t (&wq)[2], f16x8 (&av)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w = (uint32_t)wq[j][t], w8 = w >> 8;
            const half2_t p0 = __builtin_elementwise_fma(as_half2(w & 0x000F000Fu), cs[j], cmn[j]);
            const half2_t p1 = __builtin_elementwise_fma(as_half2(w & 0x00F000F0u), cs16[j], cmn[j]);
            const half2_t p2 = __builtin_elementwise_fma(as_half2(w8 & 0x000F000Fu), cs[j], cmn[j]);
            const half2_t p3 = __builtin_elementwise_fma(as_half2(w8 & 0x00F000F0u), cs16[j], cmn[j]);
            av[j] = f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
        }
    };
    auto mfmas = [&](const f16x8 (&av)[2], const f16x8 (&bv)[4]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[j], bv[i], acc[j][i], 0, 0, 0);
    };

    // Each round's fragments and weights are read and unpacked during the
    // round before: one scheduling region holds a round's 8 MFMAs and the
    // next round's LDS reads and unpack, interleaved one MFMA, one read and
    // three VALU ops at a time so the VALU runs in the MFMAs' shadow.  B_s
    // falls between rounds 2 and 3, and step s + 1's first operands are read
    // after it, during round 3.
    auto interleave = [&]() {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
        }
    };
    wait_vm_barrier<63>();  // B_init (consumers issue no loads: no wait)
    f16x8 bv0[4], bv1[4], av0[2], av1[2];
    int4_t wq[2];
    read_wts(0, wq);
    consts(0);
    read_frags(0, 0, bv0);
    unpack(0, wq, av0);
#pragma unroll 1
    for (int s = 0; s < S; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        mfmas(av0, bv0);                       // round 0
        read_frags(s, 1, bv1);
        unpack(1, wq, av1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        mfmas(av1, bv1);                       // round 1
        read_frags(s, 2, bv0);
        unpack(2, wq, av0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        mfmas(av0, bv0);                       // round 2
        read_frags(s, 3, bv1);
        unpack(3, wq, av1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_barrier<63>();                 // B_s: step s + 1 in LDS
        int4_t wqn[2];
        read_wts(s + 1, wqn);
        if (kG32 || ((s + 1) & 3) == 0) consts(s + 1);
        mfmas(av1, bv1);                       // round 3
        read_frags(s + 1, 0, bv0);
        unpack(0, wqn, av0);
        interleave();
        wq[0] = wqn[0];
        wq[1] = wqn[1];
    }

#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int nl = wn * 64 + 32 * j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 128 + 32 * i + l32;
            const float fi = m < M ? 1.0f / fs[m] : 0.0f;
            const float16_t &a = acc[j][i];
            float v[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 sc = *reinterpret_cast<const float4 *>(sScale + nl + 8 * r4 + 4 * h);
                v[4 * r4] = a[4 * r4] * fi * sc.x;
                v[4 * r4 + 1] = a[4 * r4 + 1] * fi * sc.y;
                v[4 * r4 + 2] = a[4 * r4 + 2] * fi * sc.z;
                v[4 * r4 + 3] = a[4 * r4 + 3] * fi * sc.w;
            }
            if (kMode == kFOutQ8) {
                const int nb = n0 + nl;
                float amax = 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
                amax = fmaxf(amax, __shfl_xor(amax, 32));
                const uint16_t d16 = q8_1_scale(amax);
                const float df = f16_bits_to_f32(d16);
                int sum = 0;
                uint32_t packed[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    packed[q] = 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int c = q8_1_code(v[4 * q + r], df);
                        sum += c;
                        packed[q] |= ((uint32_t)c & 0xFFu) << (8 * r);
                    }
                }
                sum += __shfl_xor(sum, 32);
                if (m < M && nb < N) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint32_t *>(qo + (int64_t)m * ldy + nb + 8 * q + 4 * h) = packed[q];
                    if (h == 0) dso[(int64_t)m * (ldy / kBlock) + nb / kBlock] = q8_1_ds(d16, df, sum);
                }
            } else if (m < M) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int n = n0 + nl + 8 * r4 + 4 * h;
                    float *dst = y + (int64_t)m * ldy + n;
                    if (vec_store && n + 3 < N) {
                        *reinterpret_cast<float4 *>(dst) =
                            make_float4(v[4 * r4], v[4 * r4 + 1], v[4 * r4 + 2], v[4 * r4 + 3]);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (n + c < N) dst[c] = v[4 * r4 + c];
                    }
                }
            }
        }
    }
}

int64_t round_up(int64_t v, int64_t u) { return (v + u - 1) / u * u; }

constexpr int64_t kFusedScaleBytes = (int64_t)8 << 20;

// activation rows per launch: the whole (padded) M, or as many 256-row tiles
// as keep the image within kImageMaxBytes (at least one tile)
int64_t chunk_rows(int64_t M, int64_t K)
{
    int64_t per = (kImageMaxBytes / (2 * K)) / kFm * kFm;
    if (per < kFm) per = kFm;
    const int64_t mp = round_up(M, kFm);
    return mp < per ? mp : per;
}

}  // namespace

size_t mmqf_workspace_bytes(int64_t M, int64_t K)
{
    if (M < 1 || K < kGroup) return 0;
    const int64_t rows = chunk_rows(M, K);
    return (size_t)(rows * K * 2 + rows * (int64_t)sizeof(float));
}

hipError_t launch_mmqf(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                       const uint16_t *sm, int64_t N, int K, bool g32, float *y, int8_t *qo, uint16_t *dso,
                       void *workspace, hipStream_t stream)
{
    const int B = K / kBlock, S = K / kFk;
    const int P = g32 ? B : K / kGroup;  // (scale, minimum) pairs per weight row
    if (g32 && !y) return hipErrorInvalidValue;  // group 32: fp32 output only
    const int64_t rows_max = chunk_rows(M, K);
    uint4 *img = static_cast<uint4 *>(workspace);
    float *fs = reinterpret_cast<float *>(static_cast<char *>(workspace) + rows_max * K * 2);
    const uint32_t *ds32 = reinterpret_cast<const uint32_t *>(ds);
    const uint32_t *sm32 = reinterpret_cast<const uint32_t *>(sm);
    uint32_t *dso32 = reinterpret_cast<uint32_t *>(dso);
    // weight rows per launch: 32-bit offsets into qs (2 GiB descriptor reach)
    const int64_t n_max = ((kMaxBufferBytes - 1) / (K / 2)) / kFn * kFn;
    for (int64_t m0 = 0; m0 < M; m0 += rows_max) {
        const int64_t mm = M - m0 < rows_max ? M - m0 : rows_max;
        const int64_t mp = round_up(mm, kFm);
        const int tiles_m = (int)(mp / kFm);
        const uint32_t img_bytes = (uint32_t)(mp * K * 2);  // <= kImageMaxBytes (or one tile's)
        // the image workgroups find the row factors themselves while the
        // row-scale reads they repeat (each step re-reads its rows' scales)
        // stay within kFusedScaleBytes and the scales allow 16-byte loads;
        // otherwise a separate pass
        if (mp * S * B * 4 <= kFusedScaleBytes && (reinterpret_cast<uintptr_t>(ds) & 15) == 0) {
            hipLaunchKernelGGL(k_mmqf_image<true>, dim3((unsigned)S, (unsigned)tiles_m), dim3(kFThreads), 0,
                               stream, qa + m0 * K, ds32 + m0 * B, fs, (int)mm, K, img);
        } else {
            hipLaunchKernelGGL(k_mmqf_rowscale, dim3((unsigned)(mp / 4)), dim3(256), 0, stream, ds32 + m0 * B,
                               (int)mm, B, (int)mp, fs);
            hipLaunchKernelGGL(k_mmqf_image<false>, dim3((unsigned)S, (unsigned)tiles_m), dim3(kFThreads), 0,
                               stream, qa + m0 * K, ds32 + m0 * B, fs, (int)mm, K, img);
        }
        for (int64_t n0 = 0; n0 < N; n0 += n_max) {
            const int64_t nn = N - n0 < n_max ? N - n0 : n_max;
            const int64_t tiles = (int64_t)tiles_m * ((nn + kFn - 1) / kFn);
            if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
            if (y) {
                float *y0 = y + m0 * N + n0;
                const int vec_store = (N % 4 == 0) && (nn % 4 == 0) &&
                                      ((reinterpret_cast<uintptr_t>(y0) & 15) == 0);
                auto kern = g32 ? k_mmqf<kFOutY, true> : k_mmqf<kFOutY, false>;
                hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kGemmThreads), 0, stream, img, img_bytes, fs,
                                   qs + n0 * (K / 2), sm32 + n0 * P, y0, (int8_t *)nullptr, (uint32_t *)nullptr,
                                   (int)mm, (int)nn, K, tiles_m, N, vec_store);
            } else {
                hipLaunchKernelGGL((k_mmqf<kFOutQ8, false>), dim3((unsigned)tiles), dim3(kGemmThreads), 0, stream,
                                   img, img_bytes, fs,
                                   qs + n0 * (K / 2), sm32 + n0 * P, (float *)nullptr, qo + m0 * N + n0,
                                   dso32 + m0 * (N / kBlock) + n0 / kBlock, (int)mm, (int)nn, K, tiles_m, N, 0);
            }
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace q4mi
