// mmq_i8.hip -- prefill GEMM on Q8_1 activations and 4-bit group-256 weights
// with gfx950 int8 matrix cores, pipelined: the MMQ of the hipfire
// MMQ-prefill note (list of changes: Q8_1 pre-quantized activations,
// LDS-staged 128x128 output tiles, i8 matrix products) with the block
// products exact in int32.
//
//   I[m][n][b] = sum_{k in block b} a[m][k] * q[n][k]              (one i8 MFMA)
//   acc[m][n][g] = sum_{b in g} D[m][b] * I[m][n][b] - 8 T[m][g]     (int32)
//               = sum_{b in g} D[m][b] * sum_{k in b} a[m][k] (q[n][k] - 8)
//   y[m][n] = sum_g ( s[n][g] * step[m][g] * acc + (mn[n][g] + 8 s[n][g]) * X[m][g] )
//
// with the per-(row, group) quantities of the int8 design (see mmq.hip):
// D = min(8191, rint(d * 8191 / max d)) the 13-bit block scales, step =
// max d / 8191, X = sum_b d * A, T = sum_b D * A, A = sum of a block's codes.
// The MFMA takes the codes q as they are and the -8 T start value of each
// group's sum does the centring: after k blocks the sum is
// sum_{b<k} D I'_b - 8 sum_{b>=k} D A_b with I' = sum a (q - 8), and each
// block contributes at most 8191 * 32 * 127 * 8 < 2^28 in magnitude either
// way, so no partial sum reaches 2^31.
//
// Where the work goes, per output and Q8_1 block: one v_mad_i32_i24 (the VALU
// bound of this design); per output and group: four fp32 ops.  Everything
// that depends only on (row, group) -- the integer block scales, step, X,
// T -- and on (weight row, group) -- scale and minimum + 8 scale in fp32 --
// is computed once by k_mmqi_prep instead of by every tile that uses it.
//
// k_mmqi: 128 (n) x 128 (m) tiles, 512 threads = 8 waves, wave (wn, wm)
// owning weight rows 64 wn .. 64 wn + 63 (two 32-row MFMA tiles) x
// activation rows 32 wm .. 32 wm + 31.  Each wave software-pipelines its
// products: the MFMA of the next (block, tile) is issued before the
// multiply-adds of the current one.  K runs in stages of one group (256,
// eight blocks), double-buffered in LDS (about 138 KB, one workgroup per CU,
// one barrier per group): activations and the per-group records go straight
// to LDS by buffer_load ... lds (no registers), the packed weights through
// registers where they are split into int8 codes.  Rows are 256 bytes with
// their 16-byte chunks XOR-swizzled by the row's low four bits: a 1 KB run of
// LDS is four whole source rows (every load instruction fetches whole
// 128-byte lines), and the 16-byte fragment reads of sixteen consecutive rows
// at one chunk cover all 64 banks once.  The minimum term of each group,
// (mn + 8 s) X, is a rank-1 update of the tile: one fp32 MFMA per 32 x 32
// tile and group on the otherwise idle matrix core, accumulating into y.
#include <type_traits>

#include "q4mi_device.h"
#include "q4mi_kernels.h"
#include "mmq_tiles.h"

namespace q4mi {

namespace {

constexpr int kPn = 128;                 // weight rows (n) per tile
constexpr int kPm = 128;                 // activation rows (m) per tile
constexpr int kPk = 256;                 // K per stage: one group, eight Q8_1 blocks
constexpr int kPThreads = 512;
// per (activation row, group): D pairs (D[2i] | D[2i+1] << 16) x 4, X, step, -8 T, 0
constexpr int kRecBytes = 32;
constexpr int kLdsW = kPn * kPk;         // 32 KB: int8 weight codes of a stage
constexpr int kLdsA = kPm * kPk;         // 32 KB: int8 activations of a stage
constexpr int kLdsRec = kPm * kRecBytes; // 4 KB: the tile's row records of the group
constexpr int kLdsSm = kPn * 8;          // 1 KB: (scale, minimum + 8 scale) of the group
constexpr int kOffA = kLdsW;
constexpr int kOffRec = kOffA + kLdsA;
constexpr int kOffSm = kOffRec + kLdsRec;
constexpr int kLdsStage = kOffSm + kLdsSm;  // 69 KB
constexpr int kLdsTotal = 2 * kLdsStage;    // 138 KB: one workgroup per CU
constexpr int kDMaxI = 8191;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// LDS byte offset of 16-byte chunk c (0..15) of row r in a [rows][256 B]
// array.  A 16-byte LDS read serves 16 lanes per cycle across 64 banks (256
// bytes), so every row starts on bank 0; the chunks are XOR-swizzled by the
// row's low four bits, and sixteen consecutive rows at one chunk cover all 64
// banks once.
__device__ __forceinline__ uint32_t swz(uint32_t r, uint32_t c) { return r * 256u + 16u * (c ^ (r & 15u)); }

// LDS byte offset of 16-byte chunk c (0..1) of row r's 32-byte record, chunks
// XOR-swizzled by bit 3 of the row so that sixteen consecutive rows at one
// chunk cover all 64 banks once
__device__ __forceinline__ uint32_t recoff(uint32_t r, uint32_t c) { return r * 32u + 16u * (c ^ ((r >> 3) & 1u)); }

// Blocks [0, rowblocks): eight lanes per (activation row m, group g), lane b
// taking block b, records [g][Mp] of kRecBytes (rows >= M are zeros: their
// loads fall outside the buffers).  Blocks [rowblocks, ...): one thread per
// (weight row n, group g): per group and 128-row tile, the 128 scales then
// the 128 (minimum + 8 scale), fp32 (rows >= N zero).
__global__ __launch_bounds__(256) void k_mmqi_prep(const int8_t *__restrict__ qa, const uint32_t *__restrict__ ds,
                                                   const uint32_t *__restrict__ sm, int M, int N, int K, int Mp,
                                                   int Np, int rowblocks, uint32_t *__restrict__ rec,
                                                   float2 *__restrict__ smrec)
{
    const int G = K / kGroup;
    if ((int)blockIdx.x < rowblocks) {
        // Mp * G * 8 is a multiple of 256: every lane of the grid has a row
        const uint32_t t = blockIdx.x * 256u + threadIdx.x;
        const int b = (int)(t & 7u);
        const uint32_t mg = t >> 3;  // g * Mp + m
        const uint32_t m = mg % (uint32_t)Mp, g = mg / (uint32_t)Mp;
        const rsrc_t r_qa = make_rsrc(qa, (uint32_t)M * (uint32_t)K);
        const rsrc_t r_ds = make_rsrc(ds, (uint32_t)M * (uint32_t)(K / kBlock) * 4u);
        const uint32_t off = m * (uint32_t)K + g * kGroup + (uint32_t)b * kBlock;
        const uint4 c0 = buf_load16(r_qa, off), c1 = buf_load16(r_qa, off + 16);
        const uint32_t dw = buf_load4(r_ds, (m * (uint32_t)(K / kBlock) + g * 8u + (uint32_t)b) * 4u);
        int sa = 0;
        sa = __builtin_amdgcn_sdot4((int)c0.x, 0x01010101, sa, false);
        sa = __builtin_amdgcn_sdot4((int)c0.y, 0x01010101, sa, false);
        sa = __builtin_amdgcn_sdot4((int)c0.z, 0x01010101, sa, false);
        sa = __builtin_amdgcn_sdot4((int)c0.w, 0x01010101, sa, false);
        sa = __builtin_amdgcn_sdot4((int)c1.x, 0x01010101, sa, false);
        sa = __builtin_amdgcn_sdot4((int)c1.y, 0x01010101, sa, false);
        sa = __builtin_amdgcn_sdot4((int)c1.z, 0x01010101, sa, false);
        sa = __builtin_amdgcn_sdot4((int)c1.w, 0x01010101, sa, false);
        const float d = f16_bits_to_f32(dw & 0xFFFFu);
        float dmax = d;
        dmax = fmaxf(dmax, __shfl_xor(dmax, 1));
        dmax = fmaxf(dmax, __shfl_xor(dmax, 2));
        dmax = fmaxf(dmax, __shfl_xor(dmax, 4));
        // D * step is within step / 2 of d whatever the rounding of the factors
        const float inv = dmax > 0.0f ? (float)kDMaxI * __builtin_amdgcn_rcpf(dmax) : 0.0f;
        const int D = min(kDMaxI, (int)rintf(d * inv));
        float X = d * (float)sa;  // exact: 11 x 13 bits
        int T = D * sa;           // |T| <= 8 * 8191 * 4064 < 2^28
        X += __shfl_xor(X, 1);
        X += __shfl_xor(X, 2);
        X += __shfl_xor(X, 4);
        T += __shfl_xor(T, 1);
        T += __shfl_xor(T, 2);
        T += __shfl_xor(T, 4);
        // D pairs: lane b takes the neighbour's D by one shuffle
        const int Dn = __shfl_xor(D, 1);
        uint32_t *r = rec + (size_t)mg * (kRecBytes / 4);
        if ((b & 1) == 0) r[b >> 1] = (uint32_t)D | ((uint32_t)Dn << 16);
        if (b == 1) r[4] = __float_as_uint(X);
        if (b == 3) r[5] = __float_as_uint(dmax * (1.0f / (float)kDMaxI));
        if (b == 5) r[6] = (uint32_t)(-8 * T);
        if (b == 7) r[7] = 0u;
    } else {
        const uint32_t t = (blockIdx.x - (uint32_t)rowblocks) * 256u + threadIdx.x;
        if (t >= (uint32_t)Np * (uint32_t)G) return;
        const uint32_t n = t % (uint32_t)Np, g = t / (uint32_t)Np;
        const rsrc_t r_sm = make_rsrc(sm, (uint32_t)N * (uint32_t)G * 4u);
        const uint32_t v = buf_load4(r_sm, (n * (uint32_t)G + g) * 4u);
        const float sc = f16_bits_to_f32(v & 0xFFFFu), mn = f16_bits_to_f32(v >> 16);
        // per (group, 128-row tile): 128 scales, then 128 minimum + 8 scale
        float *tileplane = reinterpret_cast<float *>(smrec) + ((size_t)g * (Np / kPn) + n / kPn) * (2 * kPn);
        tileplane[n % kPn] = sc;
        tileplane[kPn + n % kPn] = fmaf(8.0f, sc, mn);
    }
}

// y (row stride ldy) for activation rows [0, M) and weight rows [0, N), or
// with kQ8 y quantized to Q8_1 along n (qo int8 [M][ldy], dso [M][ldy/32]) as
// q8_1_quantize would do it; rec / smrec from k_mmqi_prep (Mp, Np: M and N
// padded to whole tiles).
template <bool kQ8>
__global__ __launch_bounds__(kPThreads, 2) void k_mmqi(const int8_t *__restrict__ qa, const uint8_t *__restrict__ qs,
                                                       const uint32_t *__restrict__ rec,
                                                       const float2 *__restrict__ smrec, float *__restrict__ y,
                                                       int8_t *__restrict__ qo, uint32_t *__restrict__ dso,
                                                       int M, int N, int K, int Mp, int Np, int tiles_m,
                                                       int64_t ldy, int vec_store)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsTotal];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int l32 = lane & 31, half = lane >> 5;
    // each XCD runs a contiguous stretch of tiles in grouped order: its one
    // or two 128-row activation tiles against every weight tile, each read
    // once per XCD
    int mt, nt;
    grouped_tile(xcd_tile(blockIdx.x, gridDim.x), tiles_m, (int)gridDim.x / tiles_m, mt, nt);
    const int m0 = mt * kPm, n0 = nt * kPn;
    const int G = K / kGroup;
    const uint32_t rowq = (uint32_t)K / 2;

    const rsrc_t r_qa = make_rsrc(qa, (uint32_t)M * (uint32_t)K);
    const rsrc_t r_qs = make_rsrc(qs, (uint32_t)N * rowq);
    const rsrc_t r_rec = make_rsrc(rec, (uint32_t)Mp * (uint32_t)G * kRecBytes);
    const rsrc_t r_sm = make_rsrc(smrec, (uint32_t)Np * (uint32_t)G * 8u);
    const uint32_t lds0 = lds_addr(lds);

    // ---- loads of group g into stage buffer g & 1 ----
    // activations: wave w moves rows 16 w .. 16 w + 15 as four 1 KB runs of 4 rows
    const uint32_t arow = (uint32_t)(lane >> 4), aslot = (uint32_t)(lane & 15);
    auto load_acts = [&](int g) {
        const uint32_t dst = lds0 + (uint32_t)(g & 1) * kLdsStage + kOffA;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t r = (uint32_t)(wave * 4 + i) * 4u + arow;
            const uint32_t c = aslot ^ (r & 15u);
            dma16(r_qa, ((uint32_t)m0 + r) * (uint32_t)K + (uint32_t)g * kPk + 16u * c, 0u,
                  dst + (uint32_t)(wave * 4 + i) * 1024u);
        }
    };
    // weights: thread t takes row t / 4, blocks 2 (t % 4) and 2 (t % 4) + 1 of the group
    const uint32_t wrow = (uint32_t)(tid >> 2), wq = (uint32_t)(tid & 3);
    struct W2 {
        uint4 a, b;
    };
    auto load_wts = [&](int g) {
        const uint32_t o = ((uint32_t)n0 + wrow) * rowq + (uint32_t)g * (kPk / 2) + 32u * wq;
        return W2{buf_load16(r_qs, o), buf_load16(r_qs, o + 16u)};
    };
    // codes of block q of a packed 16-byte run: byte i holds element i (low
    // nibble) and i + 16 (high nibble); elements 0..15 are chunk 2q, 16..31 chunk 2q+1
    auto store_wts = [&](int g, const W2 &w) {
        uint8_t *dst = lds + (uint32_t)(g & 1) * kLdsStage;
        const uint4 v[2] = {w.a, w.b};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint4 x = v[k];
            const uint32_t blk = 2u * wq + (uint32_t)k;
            const uint4 lo = make_uint4(x.x & 0x0F0F0F0Fu, x.y & 0x0F0F0F0Fu, x.z & 0x0F0F0F0Fu, x.w & 0x0F0F0F0Fu);
            const uint4 hi = make_uint4((x.x >> 4) & 0x0F0F0F0Fu, (x.y >> 4) & 0x0F0F0F0Fu,
                                        (x.z >> 4) & 0x0F0F0F0Fu, (x.w >> 4) & 0x0F0F0F0Fu);
            *reinterpret_cast<uint4 *>(dst + swz(wrow, 2u * blk)) = lo;
            *reinterpret_cast<uint4 *>(dst + swz(wrow, 2u * blk + 1u)) = hi;
        }
    };
    // the group's records: 4 KB of rows (waves 0-3, one 1 KB run of 32
    // records each) and 1 KB of weight-row pairs (wave 4)
    auto load_group = [&](int g) {
        const uint32_t base = lds0 + (uint32_t)(g & 1) * kLdsStage;
        if (wave < 4) {
            const uint32_t r = (uint32_t)wave * 32u + (uint32_t)(lane >> 1);
            const uint32_t c = (uint32_t)(lane & 1) ^ ((r >> 3) & 1u);
            const uint32_t rbase = ((uint32_t)g * (uint32_t)Mp + (uint32_t)m0) * kRecBytes;
            dma16(r_rec, rbase + r * kRecBytes + 16u * c, 0u, base + kOffRec + (uint32_t)wave * 1024u);
        } else if (wave == 4) {
            dma16(r_sm, ((uint32_t)g * (uint32_t)Np + (uint32_t)n0) * 8u + 16u * (uint32_t)lane, 0u,
                  base + kOffSm);
        }
    };

    int acc[2][16];
    float16_t yacc[2];
#pragma unroll
    for (int ta = 0; ta < 2; ++ta)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            acc[ta][e] = 0;
            yacc[ta][e] = 0.0f;
        }
    // fragment rows: the two weight tiles are 32 rows apart (the low four bits
    // of the row, and so the swizzle, agree), one activation tile
    const uint32_t nrow = (uint32_t)(wn * 64 + l32);
    const uint32_t mrow = (uint32_t)(wm * 32 + l32);
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    // Per group, the values the group epilogue needs are read into registers
    // before the barrier that ends the group (their LDS buffer is refilled
    // right after it), and the epilogue runs at the start of the next
    // group, in the shadow of that group's first LDS reads and MFMA.
    struct GroupEpi {
        float4 sc[2][4];  // scales of rows 8 q + 4 half + r of each tile
        float mnv[2];     // minimum + 8 scale of row l32 of each tile
        float X, step;
    };
    auto read_epi = [&](int g, GroupEpi &e) {
        const uint8_t *S = lds + (g & 1) * kLdsStage;
        const float *P = reinterpret_cast<const float *>(S + kOffSm);
        const float2 xs = *reinterpret_cast<const float2 *>(S + kOffRec + recoff(mrow, 1));
        e.X = xs.x;
        e.step = xs.y;
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {
            e.mnv[ta] = P[kPn + wn * 64 + ta * 32 + l32];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                e.sc[ta][q] = *reinterpret_cast<const float4 *>(P + wn * 64 + ta * 32 + 8 * q + 4 * half);
        }
    };
    // y += s * (step * acc) on the VALU and y += (mn + 8 s) X as a rank-1
    // update on the matrix core (k = 0 of a 32x32x2 fp32 product, k = 1 zero)
    auto group_epilogue = [&](const GroupEpi &e) {
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {
            yacc[ta] = __builtin_amdgcn_mfma_f32_32x32x2f32(half == 0 ? e.mnv[ta] : 0.0f, half == 0 ? e.X : 0.0f,
                                                            yacc[ta], 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float sc[4] = {e.sc[ta][q].x, e.sc[ta][q].y, e.sc[ta][q].z, e.sc[ta][q].w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int el = 4 * q + r;
                    yacc[ta][el] = fmaf(sc[r], e.step * (float)acc[ta][el], yacc[ta][el]);
                }
            }
        }
    };

    // the eight blocks of group g from stage buffer g & 1; first (with_prev)
    // the epilogue of the previous group, between the first reads and
    // products of this one
    GroupEpi epi;
    auto compute = [&](int g, bool with_prev) {
        const uint8_t *S = lds + (g & 1) * kLdsStage;
        const uint8_t *W = S, *A = S + kOffA, *R = S + kOffRec;
        const uint4 dp = *reinterpret_cast<const uint4 *>(R + recoff(mrow, 0));
        const int start = *reinterpret_cast<const int *>(R + recoff(mrow, 1) + 8);  // -8 T
        const uint32_t dpw[4] = {dp.x, dp.y, dp.z, dp.w};
        auto frag_b = [&](int j) { return *reinterpret_cast<const v4i *>(A + swz(mrow, 2u * j + half)); };
        auto frag_a = [&](int j, int ta) {
            return *reinterpret_cast<const v4i *>(W + swz(nrow + 32u * ta, 2u * j + half));
        };
        auto mads = [&](const v16i &I, int ta, int j) {
            const int D = (int)((j & 1) ? (dpw[j >> 1] >> 16) : (dpw[j >> 1] & 0xFFFFu));
            // |I| <= 32 * 127 * 15 and D <= 8191: exact in the 24-bit
            // multiplier (one v_mad_i32_i24 per output)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[ta][e] = __mul24(I[e], D) + (j == 0 ? start : acc[ta][e]);
            // the block's sums are final here: the compiler may not regroup
            // the eight additions of a group (that would keep several blocks'
            // products alive and split each multiply-add)
#pragma unroll
            for (int e = 0; e < 16; e += 4)
                asm volatile("" : "+v"(acc[ta][e]), "+v"(acc[ta][e + 1]), "+v"(acc[ta][e + 2]), "+v"(acc[ta][e + 3]));
        };
        // software pipeline over (block, tile): two products live, and the
        // LDS fragments of block j + 2 are read while block j is multiplied
        v4i fb[8], fa0[8], fa1[8];
        fb[0] = frag_b(0);
        fa0[0] = frag_a(0, 0);
        fa1[0] = frag_a(0, 1);
        fb[1] = frag_b(1);
        fa0[1] = frag_a(1, 0);
        fa1[1] = frag_a(1, 1);
        v16i I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa0[0], fb[0], zero, 0, 0, 0);
        if (with_prev) group_epilogue(epi);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa1[j], fb[j], zero, 0, 0, 0);
            if (j + 2 < 8) {
                fb[j + 2] = frag_b(j + 2);
                fa0[j + 2] = frag_a(j + 2, 0);
                fa1[j + 2] = frag_a(j + 2, 1);
            }
            mads(I0, 0, j);
            if (j + 1 < 8) I0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa0[j + 1], fb[j + 1], zero, 0, 0, 0);
            mads(I1, 1, j);
        }
    };

    // ---- prologue: group 0 ----
    load_group(0);
    load_acts(0);
    {
        const W2 w = load_wts(0);
        store_wts(0, w);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

#pragma unroll 1
    for (int g = 0; g < G; ++g) {
        // group g from buffer g & 1; group g + 1 loads into the other buffer,
        // whose last reader (group g - 1) finished before the last barrier
        const bool more = g + 1 < G;
        W2 w;
        if (more) {
            load_group(g + 1);
            load_acts(g + 1);
            w = load_wts(g + 1);
        }
        compute(g, g > 0);
        read_epi(g, epi);
        __builtin_amdgcn_sched_barrier(0);
        if (more) store_wts(g + 1, w);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    group_epilogue(epi);

    // ---- y: lane (l32, half) holds column m = l32 of each tile, rows 8 q + 4 half + r ----
    const int m = m0 + (int)mrow;
    if constexpr (kQ8) {
        // each 32-row tile of the lane's column is one Q8_1 block along n:
        // 16 values here, 16 in lane ^ 32; the same fp32 decisions as
        // q8_1_quantize (N is a multiple of 32, so a block is wholly inside
        // or outside [0, N))
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {
            const int nb = n0 + wn * 64 + ta * 32;
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
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint32_t *>(qo + (int64_t)m * ldy + nb + 8 * q + 4 * half) = packed[q];
                if (half == 0) dso[(int64_t)m * (ldy / kBlock) + nb / kBlock] = q8_1_ds(d16, df, sum);
            }
        }
    } else if (m < M) {
#pragma unroll
        for (int ta = 0; ta < 2; ++ta)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 64 + ta * 32 + 8 * q + 4 * half;
                float *dst = y + (int64_t)m * ldy + n;
                const float v0 = yacc[ta][4 * q], v1 = yacc[ta][4 * q + 1];
                const float v2 = yacc[ta][4 * q + 2], v3 = yacc[ta][4 * q + 3];
                if (vec_store && n + 3 < N) {
                    *reinterpret_cast<float4 *>(dst) = make_float4(v0, v1, v2, v3);
                } else {
                    if (n < N) dst[0] = v0;
                    if (n + 1 < N) dst[1] = v1;
                    if (n + 2 < N) dst[2] = v2;
                    if (n + 3 < N) dst[3] = v3;
                }
            }
    }
}

int64_t round_up_i(int64_t v, int64_t u) { return (v + u - 1) / u * u; }

}  // namespace

bool mmqi_supported(int64_t M, int64_t N, int64_t K)
{
    // one descriptor per operand: activations, weights and the row records
    // within 2^31 bytes
    const int64_t G = K / kGroup, Mp = round_up_i(M, kPm), Np = round_up_i(N, kPn);
    return M >= 1 && N >= 1 && K >= kGroup && K % kGroup == 0 && (Mp + kPm) * K < ((int64_t)1 << 31) &&
           (Np + kPn) * (K / 2) < ((int64_t)1 << 31) && Mp * G * kRecBytes < ((int64_t)1 << 31) &&
           ((Mp / kPm) * (Np / kPn)) < ((int64_t)1 << 31);
}

size_t mmqi_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    const int64_t G = K / kGroup, Mp = round_up_i(M, kPm), Np = round_up_i(N, kPn);
    return (size_t)(Mp * G * kRecBytes + Np * G * 8);
}

hipError_t launch_mmqi(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs, const uint16_t *sm,
                       int64_t N, int K, float *y, int8_t *qo, uint16_t *dso, void *workspace, hipStream_t stream)
{
    const int G = K / kGroup;
    const int64_t Mp = round_up_i(M, kPm), Np = round_up_i(N, kPn);
    uint32_t *rec = static_cast<uint32_t *>(workspace);
    float2 *smrec = reinterpret_cast<float2 *>(static_cast<char *>(workspace) + Mp * G * kRecBytes);
    const int64_t rowblocks = Mp * G * 8 / 256;
    const int64_t smblocks = (Np * G + 255) / 256;
    hipLaunchKernelGGL(k_mmqi_prep, dim3((unsigned)(rowblocks + smblocks)), dim3(256), 0, stream, qa,
                       reinterpret_cast<const uint32_t *>(ds), reinterpret_cast<const uint32_t *>(sm), (int)M,
                       (int)N, K, (int)Mp, (int)Np, (int)rowblocks, rec, smrec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tiles_m = (int)(Mp / kPm);
    const int64_t tiles = (int64_t)tiles_m * (Np / kPn);
    if (y) {
        const int vec_store = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
        hipLaunchKernelGGL(k_mmqi<false>, dim3((unsigned)tiles), dim3(kPThreads), 0, stream, qa, qs, rec, smrec, y,
                           (int8_t *)nullptr, (uint32_t *)nullptr, (int)M, (int)N, K, (int)Mp, (int)Np, tiles_m,
                           (int64_t)N, vec_store);
    } else {
        // Q8_1 output (N a multiple of 32)
        hipLaunchKernelGGL(k_mmqi<true>, dim3((unsigned)tiles), dim3(kPThreads), 0, stream, qa, qs, rec, smrec,
                           (float *)nullptr, qo, reinterpret_cast<uint32_t *>(dso), (int)M, (int)N, K, (int)Mp,
                           (int)Np, tiles_m, (int64_t)N, 0);
    }
    return hipGetLastError();
}

}  // namespace q4mi
