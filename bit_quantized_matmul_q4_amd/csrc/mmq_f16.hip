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
//     Grids whose 256-row tiles would leave CUs idle in their last round
//     (at most two rounds) take 192-row tiles where that means fewer rows x
//     rounds (96 x 64 per computing wave): M 512 at N 9216 runs 216 tiles
//     of 192 rows in one round instead of 144 of 256.  The arithmetic is
//     the same per output, so the results are identical bit for bit.
//   * Each K step (32 KB of image, 4 KB of packed weights) is loaded straight
//     into one of 4 LDS stages (no registers in flight, two steps ahead);
//     the computing waves read and unpack each MFMA round's operands during
//     the round before.
//   * The image is laid out per (256-row tile, K step) in LDS order: the
//     loads are contiguous 1 KB per instruction and the LDS reads (16 bytes
//     per lane, consecutive rows) are conflict-free.
//   * Tiles are mapped so each XCD works on a contiguous run of tiles in
//     groups of few activation-row tiles (m fastest within a group), which
//     keeps the shared activation and weight tiles in its L2 and reads each
//     XCD's activation slice and each weight tile once.
#include "q4mi_device.h"
#include "q4mi_kernels.h"
#include "mmq_tiles.h"

namespace q4mi {

namespace {

// activation rows per tile: 256, or 192 where the grid of 256-row tiles
// leaves CUs idle in its last round (the launcher's choice, tile_rows)
constexpr int kFm = 256;
constexpr int kFmSmall = 192;
constexpr int kFn = 128;           // weight rows per tile
constexpr int kFk = 64;            // K per step: two Q8_1 blocks
// K steps per image workgroup: two (128 B of a row per thread, whole cache
// lines) while that still leaves kImgMinGroups workgroups, else one
constexpr int kImgMaxSteps = 2;
constexpr int kImgMinGroups = 256;
static_assert(kGroup % (kFk * kImgMaxSteps) == 0, "K (a multiple of 256) holds whole image workgroups");
// 16-byte vectors of the image per (tile of fm rows, step)
__host__ __device__ constexpr int step_vecs(int fm) { return 8 * fm; }
// Computing waves (one per SIMD) and the 32-row activation tiles each owns.
// Eight computing waves (two per SIMD, 64 x 64 each, 129 registers) were
// 3-6 % slower at M 512-2048: each weight tile's fragments are then read and
// unpacked by four waves instead of two.
constexpr int kCW = 4;
constexpr int kGemmThreads = (kCW + 4) * kWave;  // and one loading wave per SIMD
constexpr int kStages = 4;                      // K steps in LDS at once
constexpr int kSmVecs32 = 2 * kFn / 4;          // group 32: the step's (scale, minimum) pairs
// image + packed weights of a step (+ group-32 pairs): 144 KB of stages at
// 256 rows, 148 KB with group-32 weights
__host__ __device__ constexpr int stage_vecs(int fm, bool g32)
{
    return step_vecs(fm) + 2 * kFn + (g32 ? kSmVecs32 : 0);
}
static_assert(kStages * stage_vecs(kFm, true) * 16 + 3 * kFn * 4 + kFn * 8 <= 160 * 1024, "LDS of a CU");
static_assert(kFmSmall % 64 == 0 && kFmSmall < kFm, "whole 32-row MFMA tiles per computing wave");
// largest activation image per launch; bigger M runs in row chunks
constexpr int64_t kImageMaxBytes = (int64_t)256 << 20;

enum { kFOutY = 0, kFOutQ8 = 1 };

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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

// Bound on a weight row's dequantized magnitudes from one (scale, minimum)
// pair: |minimum| + 15 |scale|.
__device__ __forceinline__ float pair_bound(uint32_t v)
{
    return fabsf(f16_bits_to_f32(v >> 16)) + 15.0f * fabsf(f16_bits_to_f32(v & 0xFFFFu));
}

// E[n] with 2^E * (the row's largest pair bound) in [2^-7, 2^-6), or 0 for
// all-zero and non-finite rows.
__device__ __forceinline__ int weight_exponent(float wmax)
{
    int e = 0;
    if (wmax > 0.0f && wmax <= 3.0e38f) {
        frexpf(wmax, &e);
        return -6 - e;
    }
    return 0;
}

// The fp16 activation image of one 256-row tile mt and kSteps K steps s0,
// s0 + 1, ...: thread r converts row mt * 256 + r, k in [64 s0, 64 s0 +
// 64 kSteps) (with two steps, whole 128-byte lines of its row).
// Vector (t, h, r) of step s (t = 0..3 MFMA of the step, h = Q8_1 block of
// the step) holds
// x'[k] for k = 64 s + 32 h + {4t, 4t+2, 16+4t, 18+4t, 4t+1, 4t+3, 17+4t, 19+4t}:
// the order in which the GEMM unpacks one 32-bit word of packed weights.
// kRowScale: each thread also finds its row's factor itself (all the row's
// block scales, loaded a round of 8 vectors at a time) and the step-0
// workgroups store it for the GEMM's epilogue, in place of k_mmqf_rowscale;
// taken when those repeated reads stay small (short K, few row tiles).
// The last row of workgroups (blockIdx.y == tiles_m) instead finds each
// weight row's exponent E (weight_exponent over its P pairs) for rows [0,
// Np), Np = N rounded up to whole 128-row tiles: wexp[n] = (E, 2^-E as fp32
// bits), (0, 1.0) past N.
template <bool kRowScale, int kSteps, int FM>
__global__ __launch_bounds__(kFm) void k_mmqf_image(const int8_t *__restrict__ qa,
                                                          const uint32_t *__restrict__ ds,
                                                          float *__restrict__ fs, int M, int K,
                                                          uint4 *__restrict__ img,
                                                          const uint32_t *__restrict__ sm, int N, int P,
                                                          int Np, int2 *__restrict__ wexp)
{
    constexpr int kFm = FM, kStepVecs = step_vecs(FM);
    if ((int)blockIdx.y == (int)gridDim.y - 1) {
        const int stride = (int)gridDim.x * FM;
        for (int n = (int)blockIdx.x * FM + (int)threadIdx.x; n < Np; n += stride) {
            float wmax = 0.0f;
            if (n < N) {
                // eight loads in flight at a time
                const uint32_t *row = sm + (int64_t)n * P;
                int i = 0;
                for (; i + 8 <= P; i += 8) {
                    uint32_t v[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = row[i + j];
#pragma unroll
                    for (int j = 0; j < 8; ++j) wmax = fmaxf(wmax, pair_bound(v[j]));
                }
                for (; i < P; ++i) wmax = fmaxf(wmax, pair_bound(row[i]));
            }
            const int e = n < N ? weight_exponent(wmax) : 0;
            wexp[n] = make_int2(e, __float_as_int(ldexpf(1.0f, -e)));
        }
        return;
    }
    const int s0 = blockIdx.x * kSteps, mt = blockIdx.y, r = threadIdx.x;
    const int S = K / kFk;
    const int m = mt * kFm + r;
    uint4 q[4 * kSteps] = {};
    uint32_t dw[2 * kSteps] = {};
    float F = 1.0f;
    if (m < M) {
        const uint4 *src = reinterpret_cast<const uint4 *>(qa + (int64_t)m * K + (int64_t)s0 * kFk);
#pragma unroll
        for (int i = 0; i < 4 * kSteps; ++i) q[i] = src[i];
        const uint32_t *dp = ds + (int64_t)m * (K / kBlock) + 2 * s0;
#pragma unroll
        for (int i = 0; i < 2 * kSteps; ++i) dw[i] = dp[i];
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
            if (s0 == 0) fs[m] = F;
        } else {
            F = fs[m];
        }
    }
#pragma unroll
    for (int ss = 0; ss < kSteps; ++ss) {
        uint4 *dst = img + ((int64_t)mt * S + s0 + ss) * kStepVecs + r;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float df = f16_bits_to_f32(dw[2 * ss + h] & 0xFFFFu) * F;  // exact: F is a power of two
            const uint4 *qh = q + 4 * ss + 2 * h;
            const uint32_t w8[8] = {qh[0].x, qh[0].y, qh[0].z, qh[0].w, qh[1].x, qh[1].y, qh[1].z, qh[1].w};
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
}

// y (row stride ldy) for activation rows [0, M) and weight rows [0, N) of
// this sub-problem; img/fs are its activation image and row factors, wexp
// its weight rows' exponents.  Output modes: fp32 y, or y quantized to Q8_1
// along n (qo int8 [M][ldy], dso [M][ldy/32]) as q8_1_quantize would do it.
// kG32: group-32 weights, one (scale, minimum) pair per Q8_1 block; the pairs
// of a step travel with it and the operand constants change per step.
//
// 512 threads = 8 waves, two per SIMD.  Waves 4-7 (one per SIMD) only load
// K steps into LDS; waves 0-3 (one per SIMD) only compute, wave (wm, wn)
// owning activation rows 128 wm .. 128 wm + 127 (four MFMA tiles) x weight
// rows 64 wn .. 64 wn + 63 (two) over whole K steps (4 MFMA rounds per
// step).  Workgroups are persistent: workgroup b takes tiles b, b + grid,
// b + 2 grid, ... (through the XCD mapping), and the K steps of its tiles
// form one stream: the loading waves run into the next tile's steps while
// the computing waves write the last tile's outputs, whose stores drain
// while the next tile computes.
template <int kMode, bool kG32, int FM>
__global__ __launch_bounds__(kGemmThreads) void k_mmqf(
    const uint4 *__restrict__ img, uint32_t img_bytes, const float *__restrict__ fs,
    const uint8_t *__restrict__ qs, const uint32_t *__restrict__ sm, const int2 *__restrict__ wexp,
    float *__restrict__ y, int8_t *__restrict__ qo, uint32_t *__restrict__ dso, int M, int N, int K,
    int tiles_m, int ntiles, int64_t ldy, int vec_store)
{
    // tile of FM activation rows: kTI 32-row MFMA tiles per computing wave,
    // kIP image pieces of 64 vectors per loading wave and step
    constexpr int kFm = FM, kStepVecs = step_vecs(FM), kTI = FM / 32 / (kCW / 2), kIP = FM / 32;
    constexpr int kStageVecs = step_vecs(FM) + 2 * kFn;
    constexpr int kSV = stage_vecs(FM, kG32);
    __shared__ int4_t lds[kStages * kSV];
    __shared__ uint32_t sSM[2][kFn];
    __shared__ int2 sWE[2][kFn];  // (E, 2^-E) of the weight rows of tiles with even / odd index

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool consumer = wave < kCW;
    const int wn = wave & 1, wm = (wave >> 1) & (kCW / 2 - 1), pw = wave - kCW;
    const int l32 = lane & 31, h = lane >> 5;
    const int S = K / kFk, G = K / kGroup;
    const int P = kG32 ? K / kBlock : G;
    // this workgroup's tiles: k = 0 .. nk-1; global step u = k S + s
    const int nk = (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int U = nk * S;
    // each XCD runs a contiguous stretch of tiles in grouped order (about one
    // 256-row image slice against many weight tiles, so each XCD reads its
    // image slice and each weight tile once), returned as the m-fastest index
    // the rest uses
    auto tile_of = [&](int k) {
        int mt, nt;
        grouped_tile(xcd_tile((int)blockIdx.x + k * (int)gridDim.x, ntiles), tiles_m, ntiles / tiles_m, mt, nt);
        return mt + nt * tiles_m;
    };
    const uint32_t rowq = (uint32_t)K / 2;
    const int Np = (N + kFn - 1) / kFn * kFn;
    const rsrc_t r_img = make_rsrc(img, img_bytes);
    const rsrc_t r_qs = make_rsrc(qs, (uint32_t)N * rowq);
    const rsrc_t r_sm = make_rsrc(sm, (uint32_t)N * P * 4u);
    const rsrc_t r_we = make_rsrc(wexp, (uint32_t)Np * 8u);

    const uint32_t lds0 = lds_addr(lds);
    const uint32_t sm0 = lds_addr(&sSM[0][0]);
    const uint32_t we0 = lds_addr(&sWE[0][0]);

    if (!consumer) {
        // ---- producer: step u in stage u % kStages; kIP image pieces (8 FM
        // vectors / 4 producers), one weight piece, with group-32 weights one
        // piece of pairs: at least kIP + 1 loads per step.  Barrier B_u (the
        // consumers' barrier between rounds 2 and 3 of step u) needs step
        // u + 1 in LDS; after it, step u + kStages - 1 goes into the stage of
        // step u - 1, whose reads the consumers finished before B_u.  Steps
        // past the last read the last step again (uniform load counts). ----
        const uint32_t wcol = (uint32_t)((pw * 64 + lane) & 127), wblk = (uint32_t)((pw * 64 + lane) >> 7);
        auto issue = [&](int u) {
            const int ul = min(u, U - 1);
            const int tile = tile_of(ul / S), sl = ul % S;
            const int mt = tile % tiles_m, n0 = (tile / tiles_m) * kFn;
            const uint32_t stage = lds0 + (uint32_t)((u % kStages) * kSV) * 16u;
            const uint32_t goff = (uint32_t)((mt * S + sl) * kStepVecs) * 16u;
#pragma unroll
            for (int i = 0; i < kIP; ++i) {
                const uint32_t v = (uint32_t)(pw * kIP * 64 + i * 64);
                dma16(r_img, (v + lane) * 16u, goff, stage + v * 16u);
            }
            dma16(r_qs, ((uint32_t)n0 + wcol) * rowq + wblk * 16u, (uint32_t)sl * 32u,
                  stage + (uint32_t)(kStepVecs + pw * 64) * 16u);
            if (kG32)
                dma4(r_sm, ((uint32_t)n0 + wcol) * (uint32_t)P * 4u + wblk * 4u, (uint32_t)sl * 8u,
                     stage + (uint32_t)(kStageVecs * 16 + pw * 256));
        };
        // group gg of the stream (tile gg / G, group gg % G): its pairs into sSM[gg & 1]
        auto issue_sm = [&](int gg) {
            if (!kG32 && pw < 2 && gg < nk * G) {
                const int n0 = (tile_of(gg / G) / tiles_m) * kFn;
                const uint32_t c = (uint32_t)(pw * 64 + lane);
                dma4(r_sm, ((uint32_t)n0 + c) * (uint32_t)G * 4u, (uint32_t)(gg % G) * 4u,
                     sm0 + (uint32_t)((gg & 1) * kFn + pw * 64) * 4u);
            }
        };
        // tile k's weight-row exponents into sWE[k & 1] (1 KB, one load per lane of wave 6)
        auto issue_we = [&](int k) {
            if (pw == 2 && k < nk) {
                const int n0 = (tile_of(k) / tiles_m) * kFn;
                dma16(r_we, (uint32_t)n0 * 8u + (uint32_t)lane * 16u, 0u, we0 + (uint32_t)((k & 1) * kFn * 8));
            }
        };
        issue_we(0);
        issue_sm(0);
        for (int u = 0; u < kStages - 2; ++u) issue(u);
        wait_vm_barrier<(kIP + 1) * (kStages - 3)>();  // B_init: step 0, its pairs and exponents
        issue(kStages - 2);
        for (int u = 0; u < U; ++u) {
            wait_vm_barrier<(kIP + 1) * (kStages - 3)>();  // B_u: step u + 1
            issue(u + kStages - 1);
            if ((u & 3) == 0) issue_sm((u >> 2) + 1);
            // from B_{k S} on the consumers are past tile k - 1's epilogue,
            // the last reader of sWE[(k + 1) & 1]
            if (u % S == 0) issue_we(u / S + 1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }

    // ---- consumer ----
    float16_t acc[2][kTI];
    auto zero_acc = [&]() {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < kTI; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;
    };
    zero_acc();
    auto read_frags = [&](int u, int t, f16x8 (&bv)[kTI]) {
        const int4_t *act = lds + (u % kStages) * kSV + wm * (32 * kTI) + l32;
#pragma unroll
        for (int i = 0; i < kTI; ++i) bv[i] = __builtin_bit_cast(f16x8, act[(2 * t + h) * kFm + 32 * i]);
    };
    auto read_wts = [&](int u, int4_t (&wq)[2]) {
        const int4_t *wv = lds + (u % kStages) * kSV + kStepVecs + h * kFn + wn * 64 + l32;
#pragma unroll
        for (int j = 0; j < 2; ++j) wq[j] = wv[32 * j];
    };
    half2_t cs[2], cs16[2], cmn[2];
    auto consts = [&](int u) {
        // group 256: the constants of step u's group; group 32: of step u
        const uint32_t *sm32 = reinterpret_cast<const uint32_t *>(lds + (u % kStages) * kSV + kStageVecs);
        const int2 *we = sWE[(u / S) & 1];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = wn * 64 + 32 * j + l32;
            const uint32_t w = kG32 ? sm32[h * kFn + r] : sSM[(u >> 2) & 1][r];
            const int E = we[r].x;
            const float sc = f16_bits_to_f32(w & 0xFFFFu), mn = f16_bits_to_f32(w >> 16);
            const _Float16 a = (_Float16)ldexpf(sc, E + 24), b = (_Float16)ldexpf(sc, E + 20),
                           c = (_Float16)ldexpf(mn, E);
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
    auto mfmas = [&](const f16x8 (&av)[2], const f16x8 (&bv)[kTI]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < kTI; ++i)
                acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[j], bv[i], acc[j][i], 0, 0, 0);
    };
    // the row factors of tile k's activation rows, loaded when the tile
    // starts and used by its epilogue
    float fin[kTI];
    auto load_factors = [&](int k) {
        const int m0 = (tile_of(k) % tiles_m) * kFm;
#pragma unroll
        for (int i = 0; i < kTI; ++i) {
            const int m = m0 + wm * (32 * kTI) + 32 * i + l32;
            fin[i] = m < M ? fs[m] : 1.0f;
        }
    };
    // tile k's outputs from acc: y[m][n] = acc * 2^-E[n] / F[m]
    auto epilogue = [&](int k) {
        const int tile = tile_of(k);
        const int m0 = (tile % tiles_m) * kFm, n0 = (tile / tiles_m) * kFn;
        const int2 *we = sWE[k & 1];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int nl = wn * 64 + 32 * j;
#pragma unroll
            for (int i = 0; i < kTI; ++i) {
                const int m = m0 + wm * (32 * kTI) + 32 * i + l32;
                const float fi = m < M ? 1.0f / fin[i] : 0.0f;
                const float16_t &a = acc[j][i];
                float v[16];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        v[4 * r4 + c] = a[4 * r4 + c] * fi * __int_as_float(we[nl + 8 * r4 + 4 * h + c].y);
                }
                if (kMode == kFOutQ8) {
                    const int nb = n0 + nl;
                    float amax = 0.0f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
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
                            const int c = q8_1_code(v[4 * q + r], df, rdf);
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
    };

    // Each round's activation fragments are read two rounds ahead (four
    // fragment buffers; one round ahead, the loading waves' LDS writes left
    // the reads late: M 2048 4096 -> 12288 261 -> 254 us, 12288 -> 4096 257
    // -> 246 us, bit-identical) and its weights unpacked during the round
    // before: one scheduling region holds a round's 8 MFMAs, LDS reads and
    // unpack, interleaved one MFMA, one read and three VALU ops at a time so
    // the VALU runs in the MFMAs' shadow.  B_u falls between rounds 1 and 2,
    // and step u + 1's first fragments are read after it, during rounds 2 and
    // 3 (the next tile's first step after a tile's last); the group
    // constants of step u + 1 change only after round 2 has unpacked step u's
    // last weights.
    auto interleave = [&]() {
#pragma unroll
        for (int k = 0; k < 2 * kTI; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
        }
    };
    load_factors(0);
    wait_vm_barrier<63>();  // B_init (consumers wait for no loads of their own)
    f16x8 bv0[kTI], bv1[kTI], bv2[kTI], bv3[kTI], av0[2], av1[2];
    int4_t wq[2];
    read_wts(0, wq);
    consts(0);
    read_frags(0, 0, bv0);
    read_frags(0, 1, bv1);
    unpack(0, wq, av0);
#pragma unroll 1
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        mfmas(av0, bv0);                       // round 0
        read_frags(u, 2, bv2);
        unpack(1, wq, av1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        mfmas(av1, bv1);                       // round 1
        read_frags(u, 3, bv3);
        unpack(2, wq, av0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_barrier<63>();                 // B_u: step u + 1 in LDS
        int4_t wqn[2];
        read_wts(u + 1, wqn);
        mfmas(av0, bv2);                       // round 2
        read_frags(u + 1, 0, bv0);
        unpack(3, wq, av1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        if (kG32 || ((u + 1) & 3) == 0) consts(u + 1);
        mfmas(av1, bv3);                       // round 3
        read_frags(u + 1, 1, bv1);
        unpack(0, wqn, av0);
        interleave();
        wq[0] = wqn[0];
        wq[1] = wqn[1];
        if ((u + 1) % S == 0) {
            // tile u / S is complete: its outputs go out while the loading
            // waves already fill the next tile's steps
            __builtin_amdgcn_sched_barrier(0);
            const int k = u / S;
            epilogue(k);
            zero_acc();
            if (k + 1 < nk) load_factors(k + 1);
        }
    }
}

int64_t round_up(int64_t v, int64_t u) { return (v + u - 1) / u * u; }

constexpr int64_t kFusedScaleBytes = (int64_t)8 << 20;

// Activation rows per tile, from the shape alone (the workspace size follows
// it): 192 where the grid of 256-row tiles fills at most two rounds of the
// CUs and 192-row tiles take fewer rows x rounds, e.g. M 512 at N 9216 (144
// tiles of 256 rows on 256 CUs, 216 of 192 rows: one round either way);
// otherwise 256.
int tile_rows(int64_t M, int64_t N)
{
    constexpr int64_t kCus = 256;
    const int64_t nt = (N + kFn - 1) / kFn;
    const int64_t t256 = (M + kFm - 1) / kFm * nt, t192 = (M + kFmSmall - 1) / kFmSmall * nt;
    if (t256 > 2 * kCus) return kFm;
    const int64_t c256 = (t256 + kCus - 1) / kCus * kFm, c192 = (t192 + kCus - 1) / kCus * kFmSmall;
    return c192 < c256 ? kFmSmall : kFm;
}

// activation rows per launch: the whole (padded) M, or as many fm-row tiles
// as keep the image within kImageMaxBytes (at least one tile)
int64_t chunk_rows(int64_t M, int64_t K, int fm)
{
    int64_t per = (kImageMaxBytes / (2 * K)) / fm * fm;
    if (per < fm) per = fm;
    const int64_t mp = round_up(M, fm);
    return mp < per ? mp : per;
}

template <int FM>
hipError_t launch_mmqf_t(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                         const uint16_t *sm, int64_t N, int K, bool g32, float *y, int8_t *qo, uint16_t *dso,
                         void *workspace, int num_cus, hipStream_t stream);

}  // namespace

// [image: rows x K fp16][row factors: rows fp32][weight-row (E, 2^-E): N
// rounded up to whole tiles]
size_t mmqf_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || K < kGroup) return 0;
    const int64_t rows = chunk_rows(M, K, tile_rows(M, N));
    return (size_t)(rows * K * 2 + rows * (int64_t)sizeof(float) + round_up(N, kFn) * (int64_t)sizeof(int2));
}

hipError_t launch_mmqf(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                       const uint16_t *sm, int64_t N, int K, bool g32, float *y, int8_t *qo, uint16_t *dso,
                       void *workspace, int num_cus, hipStream_t stream)
{
    if (tile_rows(M, N) == kFmSmall)
        return launch_mmqf_t<kFmSmall>(qa, ds, M, qs, sm, N, K, g32, y, qo, dso, workspace, num_cus, stream);
    return launch_mmqf_t<kFm>(qa, ds, M, qs, sm, N, K, g32, y, qo, dso, workspace, num_cus, stream);
}

namespace {

template <int FM>
hipError_t launch_mmqf_t(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                         const uint16_t *sm, int64_t N, int K, bool g32, float *y, int8_t *qo, uint16_t *dso,
                         void *workspace, int num_cus, hipStream_t stream)
{
    constexpr int kFm = FM;
    const int B = K / kBlock, S = K / kFk;
    const int P = g32 ? B : K / kGroup;  // (scale, minimum) pairs per weight row
    if (g32 && !y) return hipErrorInvalidValue;  // group 32: fp32 output only
    const int64_t rows_max = chunk_rows(M, K, FM);
    const int64_t npad = round_up(N, kFn);
    if (npad > 0x7FFFFFFF) return hipErrorInvalidValue;
    uint4 *img = static_cast<uint4 *>(workspace);
    float *fs = reinterpret_cast<float *>(static_cast<char *>(workspace) + rows_max * K * 2);
    int2 *wexp = reinterpret_cast<int2 *>(static_cast<char *>(workspace) + rows_max * K * 2 + rows_max * 4);
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
        const bool two = (int64_t)(S / kImgMaxSteps) * tiles_m >= kImgMinGroups;
        const dim3 igrid((unsigned)(two ? S / kImgMaxSteps : S), (unsigned)(tiles_m + 1));
        if (mp * S * B * 4 <= kFusedScaleBytes && (reinterpret_cast<uintptr_t>(ds) & 15) == 0) {
            auto kimg = two ? k_mmqf_image<true, kImgMaxSteps, FM> : k_mmqf_image<true, 1, FM>;
            hipLaunchKernelGGL(kimg, igrid, dim3(FM), 0, stream, qa + m0 * K, ds32 + m0 * B, fs, (int)mm,
                               K, img, sm32, (int)N, P, (int)npad, wexp);
        } else {
            hipLaunchKernelGGL(k_mmqf_rowscale, dim3((unsigned)(mp / 4)), dim3(256), 0, stream, ds32 + m0 * B,
                               (int)mm, B, (int)mp, fs);
            auto kimg = two ? k_mmqf_image<false, kImgMaxSteps, FM> : k_mmqf_image<false, 1, FM>;
            hipLaunchKernelGGL(kimg, igrid, dim3(FM), 0, stream, qa + m0 * K, ds32 + m0 * B, fs, (int)mm,
                               K, img, sm32, (int)N, P, (int)npad, wexp);
        }
        for (int64_t n0 = 0; n0 < N; n0 += n_max) {
            const int64_t nn = N - n0 < n_max ? N - n0 : n_max;
            const int64_t tiles = (int64_t)tiles_m * ((nn + kFn - 1) / kFn);
            if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
            // persistent: one workgroup per CU (the LDS of one), each taking
            // every grid-th tile
            const unsigned grid = (unsigned)(tiles < num_cus ? tiles : num_cus);
            if (y) {
                float *y0 = y + m0 * N + n0;
                const int vec_store = (N % 4 == 0) && (nn % 4 == 0) &&
                                      ((reinterpret_cast<uintptr_t>(y0) & 15) == 0);
                auto kern = g32 ? k_mmqf<kFOutY, true, FM> : k_mmqf<kFOutY, false, FM>;
                hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), 0, stream, img, img_bytes, fs,
                                   qs + n0 * (K / 2), sm32 + n0 * P, wexp + n0, y0, (int8_t *)nullptr,
                                   (uint32_t *)nullptr, (int)mm, (int)nn, K, tiles_m, (int)tiles, N, vec_store);
            } else {
                hipLaunchKernelGGL((k_mmqf<kFOutQ8, false, FM>), dim3(grid), dim3(kGemmThreads), 0, stream, img,
                                   img_bytes, fs, qs + n0 * (K / 2), sm32 + n0 * P, wexp + n0, (float *)nullptr,
                                   qo + m0 * N + n0, dso32 + m0 * (N / kBlock) + n0 / kBlock, (int)mm, (int)nn, K,
                                   tiles_m, (int)tiles, N, 0);
            }
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

}  // namespace q4mi
