// gemv.hip -- dequant-fused GEMV for decode: y[m][n] = sum_k x[m][k] * w[n][k]
// with 4-bit group-256 weights, 1..16 fp32 activation rows, fp32 output.
//
// This is the "tiny-N f32-out GEMV" / "split-K GEMM" arm pair of the vllm.cpp
// decode campaign (vllm.cpp issue 5, "Starting position") re-designed for
// gfx950.  It is bound by HBM: every weight byte is read once (0.516 B per
// weight), so the kernels are built around coalesced 16-byte loads and a VALU
// budget of about 2.5 lane-ops per weight (256 CUs x 64 lanes x 2.4 GHz
// against 8 TB/s).
//
// Shared techniques:
//   * Nibble widening by masking alone.  A dword of qs holds 8 codes; masking
//     it with 0x000F000F or 0x00F000F0 leaves two codes in the mantissas of two
//     fp16 halves, i.e. the exact fp16 subnormals q * 2^-24 and q * 2^-20
//     (widening codes to fp16 subnormals follows the gfx942 trick of the vLLM
//     Octave KV page, "Design choices", where one v_perm makes each code byte
//     an exact fp16 subnormal).  Activations paired with the high nibbles are
//     stored pre-multiplied by 2^-4 so both land on one scale.
//   * Activations are split into an fp16 "hi" part and an fp16 "lo" residual
//     (about 22 significant bits) after scaling each chunk (arm A) or group
//     (arm B) by a power of two that puts its largest magnitude in
//     [2^14, 2^15).  A single fp16 copy is not accurate enough: scale * q has
//     a large mean that cancels against minimum * sum(x), which amplifies the
//     fp16 rounding of x about threefold in the result.
//   * Per group: y += (scale * 2^(24+e)) * dot + minimum * sum(x_group), the
//     minimum term using the exact fp32 sum of the activations.
//   * Fixed reduction orders, no atomics: reruns are bit-identical.
//
// Arm A, "dot2" (M = 1, VALU): G lanes (16, or 8 when K/32 is not a multiple of
// 16) share one row; lane j owns the 16-byte chunks s*G*CPT + t*G + j (t < CPT)
// of every row, a fixed K-slice s, so its activations (hi and lo, 2*CPT*16
// VGPRs) are loaded once and reused for every row.  v_dot2_f32_f16 multiplies
// a widened pair by the activation pair: 0.63 unpack + 1 multiply op per
// weight.  Row partials are reduced across the G lanes with DPP and, with
// several K-slices, across waves through LDS in slice order.
//
// Arm B, "mfma" (M = 2..16, matrix cores): with several activation rows the
// VALU can no longer keep up with HBM, so the contraction goes to
// v_mfma_f32_16x16x32_f16: A = 16 weight rows x 32 k (one qs dword per lane,
// widened as above), B = 32 k x 16 activation columns (hi, then lo, chained
// into one fp32 accumulator).  Each wave keeps the B operands of GPW groups of
// K in registers and visits every 16-row block of the workgroup's tile; the
// waves' per-group partials meet in LDS once per row block.  When K has more
// groups than one workgroup's waves hold, the K range is split over
// workgroups and a second pass sums the fp32 partials in split order.
#include "q4mi_device.h"
#include "q4mi_kernels.h"

namespace q4mi {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

// widened pairs of one qs dword (bytes b0..b3 of a 32-element chunk, dword t):
//   p0 = (e[4t], e[4t+2])            scale 2^-24
//   p1 = (e[16+4t], e[16+4t+2])      scale 2^-20
//   p2 = (e[4t+1], e[4t+3])          scale 2^-24
//   p3 = (e[16+4t+1], e[16+4t+3])    scale 2^-20
__device__ __forceinline__ void widen(uint32_t w, uint32_t (&p)[4])
{
    const uint32_t w8 = w >> 8;
    p[0] = w & 0x000F000Fu;
    p[1] = w & 0x00F000F0u;
    p[2] = w8 & 0x000F000Fu;
    p[3] = w8 & 0x00F000F0u;
}

// element index (within a chunk) of slot (pair p, half h) of dword t
__device__ __forceinline__ int slot_elem(int t, int p, int h)
{
    return ((p & 1) ? 16 : 0) + 4 * t + ((p & 2) ? 1 : 0) + 2 * h;
}

// power-of-two exponent sc with amax * 2^-sc in [2^14, 2^15)
__device__ __forceinline__ int chunk_exp(float amax)
{
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);
    return e - 15;
}

__device__ __forceinline__ void split_hi_lo(float v, _Float16 &hi, _Float16 &lo)
{
    hi = (_Float16)v;
    lo = (_Float16)(v - (float)hi);  // exact residual, rounded to fp16
}

// ------------------------------------------------------------------ arm A --

// LDS image of the activations for arm A: per 32-element chunk, 16 hi dwords
// and 16 lo dwords (fp16 pairs in widening order), the chunk's 2^(24+e) factor
// and its fp32 sum.  The 144-byte stride (128 + 16) makes 16-byte reads of
// consecutive chunks by consecutive lanes fall on distinct LDS banks.
constexpr int kChunkLds = 144;

// Four threads per chunk; thread i converts dword i of it (elements 4i..4i+3
// and 16+4i..16+4i+3).  C is a multiple of 8 and blockDim a multiple of 64,
// so the four threads of a chunk are always active together.
__device__ __forceinline__ void fill_x_chunks(const float *__restrict__ x, int C, uint8_t *lds)
{
    for (int idx = threadIdx.x; idx < C * 4; idx += blockDim.x) {
        const int c = idx >> 2, i = idx & 3;
        const float4 a = *reinterpret_cast<const float4 *>(x + c * 32 + 4 * i);
        const float4 b = *reinterpret_cast<const float4 *>(x + c * 32 + 16 + 4 * i);
        float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                           fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
        float sum = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        const int sc = chunk_exp(amax);
        const float ls = ldexpf(1.0f, -sc), hs = ldexpf(1.0f, -sc - 4);
        // pairs of dword i: (4i, 4i+2) (16+4i, 16+4i+2) (4i+1, 4i+3) (16+4i+1, 16+4i+3)
        const float v[8] = {a.x * ls, a.z * ls, b.x * hs, b.z * hs, a.y * ls, a.w * ls, b.y * hs, b.w * hs};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            _Float16 h0, l0, h1, l1;
            split_hi_lo(v[2 * p], h0, l0);
            split_hi_lo(v[2 * p + 1], h1, l1);
            hw[p] = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
            lw[p] = __builtin_bit_cast(uint32_t, half2_t{l0, l1});
        }
        uint8_t *dst = lds + c * kChunkLds;
        *reinterpret_cast<uint4 *>(dst + 16 * i) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4 *>(dst + 64 + 16 * i) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        if (i == 0) *reinterpret_cast<float2 *>(dst + 128) = make_float2(ldexpf(1.0f, 24 + sc), sum);
    }
}

// Work of one wave: "batches" of RB = (64/G)*U consecutive rows.  A batch is
// covered in P passes of CB chunks per lane (lane j of a row owns chunks
// j + G*t, t < CB*P, so every chunk of the row once).  The registers of each
// (row step u, chunk t) are refilled with the next pass's data as soon as they
// are consumed, which keeps about U*CB*16 bytes per lane in flight.
template <int CB, int U, int G>
__global__ __launch_bounds__(256) void k_gemv_dot2(const float *__restrict__ x,
                                                   const uint8_t *__restrict__ qs,
                                                   const uint32_t *__restrict__ sm,
                                                   float *__restrict__ y, int N, int K, int P,
                                                   int nbatches)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
    constexpr int RPW = kWave / G;
    constexpr int RB = RPW * U;
    const int lane = threadIdx.x & 63, j = lane % G, rq = lane / G;
    const int C = K / 32, gpr = K / kGroup;
    const int64_t rowbytes = K / 2;
    const int W = gridDim.x * (blockDim.x / kWave);
    const int wb = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);

    const rsrc_t rq_qs = make_rsrc(qs, (uint32_t)(N * rowbytes));
    const rsrc_t rq_sm = make_rsrc(sm, (uint32_t)N * gpr * 4u);
    uint4 q[U][CB];
    uint32_t smv[U][CB];
    // rows past the end (including every row of a batch past the last) read
    // as zeros through the descriptor bounds
    auto load_item = [&](int b, int pass, int u, int t) {
        const int n = min(b * RB + u * RPW + rq, N);
        const int c = j + G * (pass * CB + t);
        q[u][t] = buf_load16(rq_qs, (uint32_t)n * (uint32_t)rowbytes + c * 16);
        smv[u][t] = buf_load4(rq_sm, ((uint32_t)n * gpr + (c >> 3)) * 4u);
    };
    // first item's loads go out before the activation fill
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < CB; ++t) load_item(wb, 0, u, t);
    fill_x_chunks(x, C, xl);
    __syncthreads();

    float p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) p[u] = 0.0f;
    int b = wb, pass = 0;
    while (b < nbatches) {
        int nb = b, np = pass + 1;
        if (np == P) { np = 0; nb = b + W; }
#pragma unroll
        for (int t = 0; t < CB; ++t) {
            // The partial sums of chunk t-1 must exist before chunk t's
            // activation reads are issued: only one chunk's 32 activation
            // registers are live, and the loads refilled below stay in flight.
#pragma unroll
            for (int u = 0; u < U; ++u) asm volatile("" : "+v"(p[u])::"memory");
            const int c = j + G * (pass * CB + t);
            const uint8_t *xc = xl + c * kChunkLds;
            uint4 hv[4], lv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hv[i] = *reinterpret_cast<const uint4 *>(xc + 16 * i);
                lv[i] = *reinterpret_cast<const uint4 *>(xc + 64 + 16 * i);
            }
            const float2 fx = *reinterpret_cast<const float2 *>(xc + 128);
            const uint32_t xh[16] = {hv[0].x, hv[0].y, hv[0].z, hv[0].w, hv[1].x, hv[1].y, hv[1].z, hv[1].w,
                                     hv[2].x, hv[2].y, hv[2].z, hv[2].w, hv[3].x, hv[3].y, hv[3].z, hv[3].w};
            const uint32_t xo[16] = {lv[0].x, lv[0].y, lv[0].z, lv[0].w, lv[1].x, lv[1].y, lv[1].z, lv[1].w,
                                     lv[2].x, lv[2].y, lv[2].z, lv[2].w, lv[3].x, lv[3].y, lv[3].z, lv[3].w};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float acc = 0.0f;
                const uint32_t w4[4] = {q[u][t].x, q[u][t].y, q[u][t].z, q[u][t].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t pw[4];
                    widen(w4[d], pw);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        acc = __builtin_amdgcn_fdot2(as_half2(pw[k]), as_half2(xh[4 * d + k]), acc, false);
                        acc = __builtin_amdgcn_fdot2(as_half2(pw[k]), as_half2(xo[4 * d + k]), acc, false);
                    }
                }
                const uint32_t sv = smv[u][t];
                const float sf = f16_bits_to_f32(sv & 0xFFFFu), mf = f16_bits_to_f32(sv >> 16);
                p[u] = fmaf(sf * fx.x, acc, p[u]);
                p[u] = fmaf(mf, fx.y, p[u]);
            }
            // registers of chunk t are consumed: refill them in place with the
            // next item (the fence keeps the loads below the compute, so the
            // loaded registers are the loop-carried ones and need no copy)
#pragma unroll
            for (int u = 0; u < U; ++u) asm volatile("" : "+v"(p[u])::"memory");
#pragma unroll
            for (int u = 0; u < U; ++u) load_item(nb, np, u, t);
        }
        if (np == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float v = group_sum<G>(p[u]);
                const int n = b * RB + u * RPW + rq;
                if (j == 0 && n < N) y[n] = v;
                p[u] = 0.0f;
            }
        }
        b = nb;
        pass = np;
    }
}

// row steps U per chunk-block size CB: about 8-10 loads of 16 B in flight per lane
constexpr int kRowStepsFor[9] = {0, 8, 4, 2, 2, 1, 1, 1, 1};

struct Dot2Cfg {
    int G, CB, U, P, nbatches, grid;
    size_t lds;
};

Dot2Cfg choose_dot2(int64_t N, int K, const DeviceInfo &dev)
{
    Dot2Cfg c{};
    const int C = K / 32;
    c.G = (C % 16 == 0) ? 16 : 8;
    const int cpt = C / c.G;  // chunks per lane per row
    static const int cbs[] = {8, 6, 5, 4, 3, 2, 1};
    c.CB = 1;
    for (int cb : cbs)
        if (cpt % cb == 0) { c.CB = cb; break; }
    c.P = cpt / c.CB;
    c.U = kRowStepsFor[c.CB];
    const int rb = (kWave / c.G) * c.U;
    c.nbatches = (int)((N + rb - 1) / rb);
    // persistent waves, at most 6 workgroups of 4 waves per CU; every wave
    // gets the same number of batches (rounds) so no round runs half empty
    const int waves_per_wg = 4;
    const int64_t max_waves = (int64_t)dev.num_cus * 6 * waves_per_wg;
    const int64_t rounds = (c.nbatches + max_waves - 1) / max_waves;
    const int64_t waves = (c.nbatches + rounds - 1) / rounds;
    c.grid = (int)((waves + waves_per_wg - 1) / waves_per_wg);
    c.lds = (size_t)C * kChunkLds;
    return c;
}

template <int CB, int U, int G>
hipError_t run_dot2(const Dot2Cfg &c, const float *x, const uint8_t *qs, const uint16_t *sm,
                    int64_t N, int K, float *y, hipStream_t stream)
{
    hipLaunchKernelGGL((k_gemv_dot2<CB, U, G>), dim3(c.grid), dim3(256), c.lds, stream, x, qs,
                       reinterpret_cast<const uint32_t *>(sm), y, (int)N, K, c.P, c.nbatches);
    return hipGetLastError();
}

template <int G>
hipError_t dispatch_dot2(const Dot2Cfg &c, const float *x, const uint8_t *qs, const uint16_t *sm,
                         int64_t N, int K, float *y, hipStream_t stream)
{
    switch (c.CB) {
    case 1: return run_dot2<1, kRowStepsFor[1], G>(c, x, qs, sm, N, K, y, stream);
    case 2: return run_dot2<2, kRowStepsFor[2], G>(c, x, qs, sm, N, K, y, stream);
    case 3: return run_dot2<3, kRowStepsFor[3], G>(c, x, qs, sm, N, K, y, stream);
    case 4: return run_dot2<4, kRowStepsFor[4], G>(c, x, qs, sm, N, K, y, stream);
    case 5: return run_dot2<5, kRowStepsFor[5], G>(c, x, qs, sm, N, K, y, stream);
    case 6: return run_dot2<6, kRowStepsFor[6], G>(c, x, qs, sm, N, K, y, stream);
    case 8: return run_dot2<8, kRowStepsFor[8], G>(c, x, qs, sm, N, K, y, stream);
    }
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ arm B --

constexpr int kMfmaRows = 16;  // weight rows per MFMA block

// One 16-row block per step.  Lane l: A row / B column j = l % 16, k-group
// kg = l / 16 (chunks 2kg, 2kg+1 of each group), D rows 4kg .. 4kg+3.
template <int GPW>
__global__ __launch_bounds__(512) void k_gemv_mfma(const float *__restrict__ x,
                                                   const uint8_t *__restrict__ qs,
                                                   const uint32_t *__restrict__ sm,
                                                   float *__restrict__ out, int M, int N, int K,
                                                   int groups_per_split, int ntiles)
{
    extern __shared__ float red[];  // [2][W][16 rows][16 columns]
    const int W = blockDim.x / kWave;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, kg = lane >> 4;
    const int split = blockIdx.y;
    const int GK = K / kGroup;
    const int gbeg = split * groups_per_split;
    const int gend = min(GK, gbeg + groups_per_split);
    const int64_t rowbytes = K / 2;
    float *dst = out + (int64_t)split * M * N;

    half8_t bh[GPW][8], bl[GPW][8];
    float fsc[GPW], xs[GPW];
    bool gvalid[GPW];

    // ---- activations of this wave's groups, as B operands (column m = j) ----
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int g = gbeg + wave * GPW + i;
        gvalid[i] = g < gend;
        const bool live = gvalid[i] && j < M;
        float v[64];  // chunks 2kg and 2kg+1 of group g, row j
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live) f = reinterpret_cast<const float4 *>(x + (int64_t)j * K + g * kGroup + kg * 64)[q];
            v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
        float amax = 0.0f, sum = 0.0f;
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            amax = fmaxf(amax, fabsf(v[q]));
            sum += v[q];
        }
        // the four k-groups of column j sit in lanes j, j+16, j+32, j+48
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        const int sc = chunk_exp(amax);
        const float lo_s = ldexpf(1.0f, -sc), hi_s = ldexpf(1.0f, -sc - 4);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const int ch = d >> 2, t = d & 3;
            half8_t h, l;
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const float sc2 = (p & 1) ? hi_s : lo_s;
                    _Float16 a, b;
                    split_hi_lo(v[ch * 32 + slot_elem(t, p, hh)] * sc2, a, b);
                    h[2 * p + hh] = a;
                    l[2 * p + hh] = b;
                }
            bh[i][d] = h;
            bl[i][d] = l;
        }
        fsc[i] = ldexpf(1.0f, 24 + sc);
        xs[i] = sum;
    }

    int buf = 0;
    uint4 cur[GPW][2];
    auto load_block = [&](int tile, uint4 (&dstv)[GPW][2]) {
        const int n = tile * kMfmaRows + j;
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            const int g = gbeg + wave * GPW + i;
            if (gvalid[i] && n < N && tile < ntiles) {
                const uint4 *p = reinterpret_cast<const uint4 *>(qs + (int64_t)n * rowbytes + g * 128 + kg * 32);
                dstv[i][0] = p[0];
                dstv[i][1] = p[1];
            } else {
                dstv[i][0] = make_uint4(0, 0, 0, 0);
                dstv[i][1] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    load_block(blockIdx.x, cur);

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        uint4 nxt[GPW][2];
        load_block(tile + gridDim.x, nxt);  // prefetch the next row block

        float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            const int g = gbeg + wave * GPW + i;
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            const uint32_t w8[8] = {cur[i][0].x, cur[i][0].y, cur[i][0].z, cur[i][0].w,
                                    cur[i][1].x, cur[i][1].y, cur[i][1].z, cur[i][1].w};
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                uint32_t p[4];
                widen(w8[d], p);
                const half8_t a = __builtin_bit_cast(half8_t, uint4{p[0], p[1], p[2], p[3]});
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh[i][d], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl[i][d], acc, 0, 0, 0);
            }
            if (gvalid[i]) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = tile * kMfmaRows + 4 * kg + e;
                    const uint32_t smv = n < N ? sm[(int64_t)n * GK + g] : 0u;
                    const float sf = f16_bits_to_f32(smv & 0xFFFFu), mf = f16_bits_to_f32(smv >> 16);
                    part[e] = fmaf(sf * fsc[i], acc[e], part[e]);
                    part[e] = fmaf(mf, xs[i], part[e]);
                }
            }
        }
        float *rb = red + (size_t)buf * W * 256;
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[wave * 256 + (4 * kg + e) * 16 + j] = part[e];
        __syncthreads();
        for (int idx = threadIdx.x; idx < kMfmaRows * M; idx += blockDim.x) {
            const int r = idx / M, m = idx % M;
            const int n = tile * kMfmaRows + r;
            float v = 0.0f;
            for (int w = 0; w < W; ++w) v += rb[w * 256 + r * 16 + m];
            if (n < N) dst[(int64_t)m * N + n] = v;
        }
        buf ^= 1;
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            cur[i][0] = nxt[i][0];
            cur[i][1] = nxt[i][1];
        }
    }
}

// y[m][n] = sum over splits of partial[s][m][n], in split order
__global__ __launch_bounds__(256) void k_splitk_sum(const float *__restrict__ partial,
                                                    float *__restrict__ y, int64_t count, int nsplit)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        float v = 0.0f;
        for (int s = 0; s < nsplit; ++s) v += partial[(int64_t)s * count + i];
        y[i] = v;
    }
}

constexpr int kGpw = 2;         // groups of K per wave (B operands in registers)
constexpr int kMaxWaves = 8;    // waves per workgroup

struct MfmaCfg {
    int waves, groups_per_split, nsplit, ntiles, grid;
    size_t lds;
};

MfmaCfg choose_mfma(int64_t N, int K, const DeviceInfo &dev)
{
    MfmaCfg c{};
    const int GK = K / kGroup;
    const int cap_groups = kGpw * kMaxWaves;
    c.nsplit = (GK + cap_groups - 1) / cap_groups;
    c.groups_per_split = (GK + c.nsplit - 1) / c.nsplit;
    c.waves = (c.groups_per_split + kGpw - 1) / kGpw;
    c.ntiles = (int)((N + kMfmaRows - 1) / kMfmaRows);
    const int wgs_per_cu = 16 / c.waves > 0 ? 16 / c.waves : 1;
    int64_t cap = (int64_t)dev.num_cus * wgs_per_cu;
    cap = (cap + c.nsplit - 1) / c.nsplit;
    c.grid = (int)(c.ntiles < cap ? c.ntiles : cap);
    c.lds = (size_t)2 * c.waves * 256 * sizeof(float);
    return c;
}

}  // namespace

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 1) return 0;
    const int GK = (int)(K / kGroup);
    const int nsplit = (GK + kGpw * kMaxWaves - 1) / (kGpw * kMaxWaves);
    return nsplit > 1 ? (size_t)nsplit * M * N * sizeof(float) : 0;
}

hipError_t launch_gemv(const float *x, int M, const uint8_t *qs, const uint16_t *sm, int64_t N,
                       int K, float *y, void *workspace, const DeviceInfo &dev, hipStream_t stream)
{
    if (M == 1) {
        // one descriptor addresses < 2 GiB of weights: split taller matrices
        const int64_t rows_max = (kMaxBufferBytes - 1) / (K / 2);
        for (int64_t n0 = 0; n0 < N; n0 += rows_max) {
            const int64_t nn = N - n0 < rows_max ? N - n0 : rows_max;
            const uint8_t *q = qs + n0 * (K / 2);
            const uint16_t *s = sm + n0 * (K / kGroup) * 2;
            const Dot2Cfg c = choose_dot2(nn, K, dev);
            const hipError_t e = c.G == 16 ? dispatch_dot2<16>(c, x, q, s, nn, K, y + n0, stream)
                                           : dispatch_dot2<8>(c, x, q, s, nn, K, y + n0, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const MfmaCfg c = choose_mfma(N, K, dev);
    float *out = c.nsplit > 1 ? static_cast<float *>(workspace) : y;
    hipLaunchKernelGGL((k_gemv_mfma<kGpw>), dim3(c.grid, c.nsplit), dim3(kWave * c.waves), c.lds,
                       stream, x, qs, reinterpret_cast<const uint32_t *>(sm), out, M, (int)N, K,
                       c.groups_per_split, c.ntiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.nsplit == 1) return e;
    const int64_t count = (int64_t)M * N;
    int64_t blocks = (count + 255) / 256;
    if (blocks > (int64_t)dev.num_cus * 8) blocks = (int64_t)dev.num_cus * 8;
    hipLaunchKernelGGL(k_splitk_sum, dim3((unsigned)blocks), dim3(256), 0, stream, out, y, count,
                       c.nsplit);
    return hipGetLastError();
}

}  // namespace q4mi
