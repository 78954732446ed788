// gemv.hip -- dequant-fused GEMV for decode: y[m][n] = sum_k x[m][k] * w[n][k]
// with 4-bit group-256 weights, 1..16 fp32 activation rows, fp32 output (the
// "tiny-N f32-out GEMV" and "split-K GEMM" arms of the vllm.cpp issue
// "GFX1100-TG200", section "Starting position"), designed for gfx950.  It is bound by
// HBM: every weight byte is read once (0.516 B per weight), so the kernels are
// built around coalesced 16-byte buffer loads kept in flight in register rings.
//
// Shared techniques:
//   * Nibble widening by masking alone.  A dword of qs holds 8 codes; masking
//     it with 0x000F000F or 0x00F000F0 leaves two codes in the mantissas of two
//     fp16 halves, i.e. the exact fp16 subnormals q * 2^-24 and q * 2^-20
//     (the same idea as the vLLM "ROCM_OCTAVE" KV-cache pull request, "Design
//     choices", where one v_perm makes each code byte an exact fp16 subnormal).  Activations paired
//     with the high nibbles are stored pre-multiplied by 2^-4, so both land on
//     one scale.
//   * Activations become fp16 after scaling a chunk (arm A: 32 elements) or a
//     group (arm B: 256) by a power of two that puts its largest magnitude in
//     [2^14, 2^15).  fp16 rounding alone is not accurate enough: scale * q has
//     mean about 7.5 * scale, which cancels against minimum * sum(x) and
//     amplifies the rounding of x.  So each chunk / group also carries
//     c = 7.5 * sum(x - fp16(x)), computed exactly in fp32; it restores the
//     rounding's share on the mean code, and what remains is
//     sum (x - fp16(x)) * (q - 7.5) over centred codes (NMSE ~5e-8 on the
//     N(0, 0.02) / N(0, 1) workloads, against a 1e-6 budget).
//   * Per group: y += scale * (f * dot + c) + minimum * X, where f = 2^(24+e)
//     undoes the scalings and X is the exact fp32 sum of the activations.
//     The running sums carry y * 2^-kYShift (f, c and X are stored that
//     much smaller) and the stores multiply by 2^kYShift, so f stays finite
//     for every finite activation (f = 2^(24+e) alone overflows once a chunk
//     reaches 2^118); the exponent e is clamped at -127 so 2^-e stays finite
//     for the smallest chunks (all-zero up to fp32 subnormals).  Powers of
//     two change no rounding in the normal range.
//   * Fixed reduction orders, no atomics: reruns are bit-identical.
//
// Arm A, "dot2" (M = 1, VALU): the workgroup converts x once into LDS; G lanes
// (16, or 8 when K/32 is not a multiple of 16) share a weight row, lane j owning
// its 16-byte chunks j, j+G, ...; v_dot2_f32_f16 multiplies a widened pair by an
// activation pair (0.63 unpack + 0.5 multiply op per weight).  Row partials are
// summed across the G lanes with DPP.  Waves are persistent, with the same
// number of row batches each.
//
// Arm B, "mfma" (M = 2..16, matrix cores): v_mfma_f32_16x16x32_f16 with the
// activations as A (16 rows, zeros past M) read from an LDS image the
// workgroup builds once, and 16 weight rows as B straight from the widened
// registers.  Each wave streams (16-row unit, group) items through a ring of
// register slots refilled as soon as they are consumed, so the weights of
// several items stay in flight with no barrier in the loop.  K is split over
// workgroups when LDS cannot hold all of it or N gives too few units; a second
// pass then sums the fp32 partials in split order.
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

// power-of-two exponent sc with amax * 2^-sc in [2^14, 2^15), but at least
// -127 so that 2^-sc is finite: a chunk below 2^-113 (fp32 subnormals
// included) is scaled by 2^127 and still lands in fp16's normal range down to
// about 2^-141.  At most 2^128 / 2^14: sc <= 113.
constexpr int kMinChunkExp = -127;
__device__ __forceinline__ int chunk_exp(float amax)
{
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);
    return max(e - 15, kMinChunkExp);
}

// Partial sums are carried at 2^-kYShift of their value: f = 2^(24-kYShift+sc)
// <= 2^127, X and c (computed from the scaled activations) below 2^127 for
// any finite x; the stored outputs are multiplied back by 2^kYShift.
constexpr int kYShift = 10;
__device__ __forceinline__ float unshift(float v) { return v * (float)(1 << kYShift); }

// ------------------------------------------------------------------ arm A --

// LDS image of the activations for arm A: per 32-element chunk, 16 dwords of
// fp16 pairs in widening order and a float4 (f, X, c, 0): f = 2^(24+e) undoes
// the chunk's power-of-two scaling and the subnormal weights, X is the fp32
// sum of the chunk and c = 7.5 * sum of (x - hi), the centred codes' share of
// the fp16 rounding of x (the error left is sum (x - hi)(q - 7.5)).  The
// 80-byte stride puts 16-byte reads of consecutive chunks by consecutive lanes
// on distinct LDS banks.
constexpr int kChunkLds = 80;
// activation items per thread whose loads go out ahead of the weight loads
constexpr int kFillRegs = 2;

// Item idx = (row r, chunk c, dword i), idx = (r C + c) 4 + i, of the image
// needs x[r][32c+4i..+3] (low nibbles) and x[r][32c+16+4i..+3] (high
// nibbles); the image holds the rows one after another, so item idx belongs
// to chunk idx / 4 of it.  Thread t takes items base + t + it * nthr;
// items past the end (nitems) read zeros and are not stored, rows >= M read
// zeros.
struct XItems {
    float4 a[kFillRegs], b[kFillRegs];
};

template <int MR>
__device__ __forceinline__ void load_x_items(rsrc_t rx, int C, int K, int M, int nitems, int nthr, int base, XItems &v)
{
#pragma unroll
    for (int it = 0; it < kFillRegs; ++it) {
        const int idx = base + threadIdx.x + it * nthr;
        uint32_t off;
        if (MR == 1) {
            off = idx < nitems ? (uint32_t)((idx >> 2) * 32 + 4 * (idx & 3)) * 4u : 0x80000000u;
        } else {
            const int r = idx / (C * 4), e = idx - r * (C * 4);
            off = idx < nitems && r < M ? (uint32_t)(r * K + (e >> 2) * 32 + 4 * (e & 3)) * 4u : 0x80000000u;
        }
        v.a[it] = __builtin_bit_cast(float4, buf_load16(rx, off));
        v.b[it] = __builtin_bit_cast(float4, buf_load16(rx, off + 64));
    }
}

// Four consecutive threads hold the four dwords of one chunk (nthr is a
// multiple of 64, so they are active together).
__device__ __forceinline__ void convert_x_items(int nitems, int nthr, int base, const XItems &v, uint8_t *lds)
{
#pragma unroll
    for (int it = 0; it < kFillRegs; ++it) {
        const int idx = base + threadIdx.x + it * nthr;
        const float4 a = v.a[it], b = v.b[it];
        float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                           fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
        // the chunk's four dwords sit in one lane quad: quad-swap DPP, not LDS
        amax = fmaxf(amax, dpp_f32<kDppQuadSwap1>(amax));
        amax = fmaxf(amax, dpp_f32<kDppQuadSwap2>(amax));
        const int sc = chunk_exp(amax);
        const float ls = ldexpf(1.0f, -sc), hs = ldexpf(1.0f, -sc - 4);
        // the sum of x, taken on the scaled values (no overflow; the same
        // roundings as on x itself), then brought to 2^-kYShift of its value
        float sum = ((a.x * ls + a.y * ls) + (a.z * ls + a.w * ls)) +
                    ((b.x * ls + b.y * ls) + (b.z * ls + b.w * ls));
        sum += dpp_f32<kDppQuadSwap1>(sum);
        sum += dpp_f32<kDppQuadSwap2>(sum);
        // pairs of dword i: (4i, 4i+2) (16+4i, 16+4i+2) (4i+1, 4i+3) (16+4i+1, 16+4i+3)
        const float w[8] = {a.x * ls, a.z * ls, b.x * hs, b.z * hs, a.y * ls, a.w * ls, b.y * hs, b.w * hs};
        uint32_t hw[4];
        float dl = 0.0f, dh = 0.0f;  // residuals of low / high slots, in scaled units
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const _Float16 h0 = (_Float16)w[2 * p], h1 = (_Float16)w[2 * p + 1];
            const float r = (w[2 * p] - (float)h0) + (w[2 * p + 1] - (float)h1);
            if (p & 1) dh += r; else dl += r;
            hw[p] = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
        }
        float delta = ldexpf(dl, sc - kYShift) + ldexpf(dh, sc + 4 - kYShift);
        delta += dpp_f32<kDppQuadSwap1>(delta);
        delta += dpp_f32<kDppQuadSwap2>(delta);
        if (idx < nitems) {
            uint8_t *dst = lds + (idx >> 2) * kChunkLds;
            const int i = idx & 3;
            *reinterpret_cast<uint4 *>(dst + 16 * i) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            if (i == 0)
                *reinterpret_cast<float4 *>(dst + 64) = make_float4(
                    ldexpf(1.0f, 24 - kYShift + sc), ldexpf(sum, sc - kYShift), 7.5f * delta, 0.0f);
        }
    }
}

// A workgroup has B x S waves: wave w works on K slice s = w % S of row batch
// w / S.  A batch is RB = (64/G)*U rows; lane j of a row owns the 16-byte
// chunks j + G*t.  Slice s of a row covers chunk steps [s*P*CB, (s+1)*P*CB),
// taken in P passes of CB chunks; the registers of each (row step u, chunk t)
// are refilled with the next pass (or the next round's batch) as soon as they
// are consumed.  The activation loads go out first, the weight loads next, so
// the fp16 image is built while the weights are in flight.  Row partials are
// summed over the G lanes with DPP and, with S > 1, over the slices through
// LDS in slice order.  All waves run the same number of rounds (batches past
// the end read zeros), so the slice barriers are uniform.  MR activation rows
// (1 or 2; rows >= M are zeros and not written) share every widened weight
// pair: the image holds one copy per row, y row r starts at y + r * ldy.
// cfg = S | P << 8 | M << 16 | B << 24 and bstride = gridDim.x * B: the
// arguments fit the 14 dwords the library preloads into SGPRs at wave launch
// (a build flag), and the kernel reads no block or grid size, so no argument
// is fetched by a scalar-load round trip (each costs a small launch ~0.3 us).
template <int CB, int U, int G, int GS, int MR>
__global__ __launch_bounds__(1024) void k_gemv_dot2(const float *__restrict__ x,
                                                    const uint8_t *__restrict__ qs,
                                                    const uint32_t *__restrict__ sm,
                                                    float *__restrict__ y, int N, int K, int rounds,
                                                    int ldy, int cfg, int bstride)
{
    const int S = cfg & 255, P = (cfg >> 8) & 255, M = (cfg >> 16) & 255, B = cfg >> 24;
    const int nthr = kWave * B * S;
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
    constexpr int RPW = kWave / G;
    constexpr int RB = RPW * U;
    const int lane = threadIdx.x & 63, j = lane % G, rq = lane / G;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = wave % S, bi = wave / S;
    const int C = K / 32, gpr = K / GS;  // (scale, minimum) pairs per row
    const int nx = MR * C * 4;           // activation image items
    const uint32_t rowbytes = K / 2;

    const rsrc_t r_qs = make_rsrc(qs, (uint32_t)N * rowbytes);
    const rsrc_t r_sm = make_rsrc(sm, (uint32_t)N * gpr * 4u);
    const rsrc_t r_x = make_rsrc(x, (uint32_t)M * K * 4u);
    uint4 q[U][CB];
    uint32_t smv[U][CB];
    // rows past the end (every row of a batch past the last) read zeros
    auto load_item = [&](int b, int pass, int u, int t) {
        const int n = min(b * RB + u * RPW + rq, N);
        const int c = j + G * ((s * P + pass) * CB + t);
        q[u][t] = buf_load16_nt(r_qs, (uint32_t)n * rowbytes + c * 16);
        smv[u][t] = buf_load4_nt(r_sm, ((uint32_t)n * gpr + (GS == kGroup ? (c >> 3) : c)) * 4u);
    };
    XItems xv;
    load_x_items<MR>(r_x, C, K, M, nx, nthr, 0, xv);
    int b = blockIdx.x * B + bi;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < CB; ++t) load_item(b, 0, u, t);
    convert_x_items(nx, nthr, 0, xv, xl);
    for (int base = kFillRegs * nthr; base < nx; base += kFillRegs * nthr) {
        load_x_items<MR>(r_x, C, K, M, nx, nthr, base, xv);
        convert_x_items(nx, nthr, base, xv, xl);
    }
    __syncthreads();
    float *red = reinterpret_cast<float *>(xl + MR * C * kChunkLds);  // [B][S][RB][MR] slice partials

    float p[U][MR];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < MR; ++r) p[u][r] = 0.0f;
    auto fence = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < MR; ++r) asm volatile("" : "+v"(p[u][r])::"memory");
    };
    for (int rd = 0; rd < rounds; ++rd) {
        const int nb = b + bstride;  // past the end in the last round: zeros
        for (int pass = 0; pass < P; ++pass) {
            const int lb = pass + 1 < P ? b : nb, lp = pass + 1 < P ? pass + 1 : 0;
#pragma unroll
            for (int t = 0; t < CB; ++t) {
                // The partial sums of chunk t-1 must exist before chunk t's
                // activation reads are issued: only one chunk's activation
                // registers are live, and the loads refilled below stay in flight.
                fence();
                const int c = j + G * ((s * P + pass) * CB + t);
                uint32_t xh[MR][16];
                float4 fx[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    const uint8_t *xc = xl + (r * C + c) * kChunkLds;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 hv = *reinterpret_cast<const uint4 *>(xc + 16 * i);
                        xh[r][4 * i] = hv.x;
                        xh[r][4 * i + 1] = hv.y;
                        xh[r][4 * i + 2] = hv.z;
                        xh[r][4 * i + 3] = hv.w;
                    }
                    fx[r] = *reinterpret_cast<const float4 *>(xc + 64);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float acc[MR];
#pragma unroll
                    for (int r = 0; r < MR; ++r) acc[r] = 0.0f;
                    const uint32_t w4[4] = {q[u][t].x, q[u][t].y, q[u][t].z, q[u][t].w};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        uint32_t pw[4];
                        widen(w4[d], pw);
#pragma unroll
                        for (int k = 0; k < 4; ++k)
#pragma unroll
                            for (int r = 0; r < MR; ++r)
                                acc[r] = __builtin_amdgcn_fdot2(as_half2(pw[k]), as_half2(xh[r][4 * d + k]), acc[r],
                                                                false);
                    }
                    const uint32_t sv = smv[u][t];
                    const float sf = f16_bits_to_f32(sv & 0xFFFFu), mf = f16_bits_to_f32(sv >> 16);
#pragma unroll
                    for (int r = 0; r < MR; ++r)
                        p[u][r] = fmaf(sf, fmaf(fx[r].x, acc[r], fx[r].z), fmaf(mf, fx[r].y, p[u][r]));
                }
                // registers of chunk t are consumed: refill them in place (the
                // fence keeps the loads below the compute, so the loaded
                // registers are the loop-carried ones and need no copy)
                fence();
#pragma unroll
                for (int u = 0; u < U; ++u) load_item(lb, lp, u, t);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const float v = group_sum<G>(p[u][r]);
                p[u][r] = 0.0f;
                const int n = b * RB + u * RPW + rq;
                if (S == 1) {
                    if (j == 0 && n < N && r < M) y[(int64_t)r * ldy + n] = unshift(v);
                } else if (j == 0) {
                    red[((bi * S + s) * RB + u * RPW + rq) * MR + r] = v;
                }
            }
        if (S > 1) {
            __syncthreads();
            if (s == 0 && j == 0) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int r = 0; r < MR; ++r) {
                        float v = 0.0f;
                        for (int k = 0; k < S; ++k) v += red[((bi * S + k) * RB + u * RPW + rq) * MR + r];
                        const int n = b * RB + u * RPW + rq;
                        if (n < N && r < M) y[(int64_t)r * ldy + n] = unshift(v);
                    }
            }
            __syncthreads();
        }
        b = nb;
    }
}

// row steps U per chunk-block size CB in the persistent mode: about 8-10 loads
// of 16 B in flight per lane
constexpr int kRowStepsFor[9] = {0, 8, 4, 2, 2, 1, 1, 1, 1};
// with four activation rows (64 activation registers) fewer row steps fit
constexpr int kRowStepsFor4[9] = {0, 4, 2, 2, 2, 1, 1, 1, 1};
__host__ __device__ constexpr int row_steps(int CB, int MR) { return MR == 4 ? kRowStepsFor4[CB] : kRowStepsFor[CB]; }

struct Dot2Cfg {
    int G, CB, U, S, P, B, rounds, grid;
    size_t lds;
};

// Two modes.  Small N (up to about 12 row batches per CU): one round, CB the
// largest chunk block dividing the lane's chunks (for rows of 12 or more
// chunk steps at most a sixth of them), K split over S waves of P passes;
// four batches per workgroup, which amortises the activation image over 4 S
// waves, or one batch per workgroup when that leaves fewer workgroups than an
// eighth of the CUs.
// Large N: persistent waves (S = 1), every wave the same number of batches.
// MR activation rows only change the LDS the image takes.
Dot2Cfg choose_dot2(int64_t N, int K, int MR, const DeviceInfo &dev)
{
    Dot2Cfg c{};
    const int C = K / 32;
    c.G = (C % 16 == 0) ? 16 : 8;
    const int cpt = C / c.G;  // chunks per lane per row
    static const int cbs[] = {8, 6, 5, 4, 3, 2, 1};
    const int rpw = kWave / c.G;
    const int64_t nb1 = (N + rpw - 1) / rpw;  // batches at U = 1
    c.CB = 1;
    for (int cb : cbs)
        if (cpt % cb == 0) { c.CB = cb; break; }
    if (nb1 <= (int64_t)dev.num_cus * 12) {
        c.U = 1;
        c.B = 4;
        if (cpt >= 12) {
            // long rows: at least 6 chunk steps per row, so each of the (up
            // to 4) slices makes two passes and refills while it computes
            // (9216 -> 2560: 6.4 -> 5.7 us)
            for (int cb : cbs)
                if (cpt % cb == 0 && cb * 6 <= cpt) { c.CB = cb; break; }
        }
        if ((nb1 + c.B - 1) / c.B < dev.num_cus / 8) {
            // very few rows: one batch per workgroup, K over more slices
            c.B = 1;
            c.CB = 1;
        }
        // slices: the largest divisor of the chunk steps that fits 16 / B waves
        const int m = cpt / c.CB;
        c.S = 1;
        for (int sl = 1; sl <= m && sl * c.B <= 16; ++sl)
            if (m % sl == 0) c.S = sl;
        c.P = m / c.S;
        c.rounds = 1;
        c.grid = (int)((nb1 + c.B - 1) / c.B);
    } else {
        c.U = row_steps(c.CB, MR);
        c.S = 1;
        c.P = cpt / c.CB;
        c.B = 4;
        if (nb1 >= (int64_t)dev.num_cus * 64) {
            // very large N (the lm_head): 8 waves per activation image, and
            // with 5-chunk rows two row steps (10 loads in flight per lane),
            // measured 3-5 % faster; smaller N keeps more, smaller workgroups
            c.B = 8;
            if (c.CB == 5) c.U = 2;
            if (MR == 2) {
                // two rows: 16 waves per image, and at most 4 chunks per row
                // step (tiny-M M = 2, K = 4096: 59.6 -> 55.3 us)
                c.B = 16;
                if (c.CB == 8) c.CB = 4;
                c.U = c.CB == 5 ? 1 : row_steps(c.CB, MR);
                c.P = cpt / c.CB;
            }
        }
        c.rounds = 0;  // set at launch from the kernel's occupancy
    }
    c.lds = (size_t)MR * C * kChunkLds + (size_t)c.B * c.S * rpw * c.U * MR * sizeof(float);
    return c;
}

template <int CB, int U, int G, int GS, int MR>
hipError_t run_dot2(Dot2Cfg c, const float *x, int M, const uint8_t *qs, const uint16_t *sm, int64_t N,
                    int64_t ldy, int K, float *y, const DeviceInfo &dev, hipStream_t stream)
{
    const auto kernel = k_gemv_dot2<CB, U, G, GS, MR>;
    if (c.rounds == 0) {
        // persistent: as many workgroups as fit on the chip at once, every wave
        // the same number of row batches (rounds) so no round runs half empty
        // (a host-side query of the kernel's register and LDS needs; only
        // large launches take this path)
        int wgs_per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&wgs_per_cu, reinterpret_cast<const void *>(kernel),
                                                         kWave * c.B * c.S, c.lds) != hipSuccess ||
            wgs_per_cu < 1)
            wgs_per_cu = 1;
        const int64_t rb = (int64_t)(kWave / G) * U;
        const int64_t nbatches = (N + rb - 1) / rb;
        const int64_t max_waves = (int64_t)dev.num_cus * wgs_per_cu * c.B;
        c.rounds = (int)((nbatches + max_waves - 1) / max_waves);
        const int64_t waves = (nbatches + c.rounds - 1) / c.rounds;
        c.grid = (int)((waves + c.B - 1) / c.B);
    }
    // S <= 16, P <= 252 chunk steps, M <= 4, B <= 16
    const int cfg = c.S | (c.P << 8) | (M << 16) | (c.B << 24);
    hipLaunchKernelGGL(kernel, dim3(c.grid), dim3(kWave * c.B * c.S), c.lds, stream, x, qs,
                       reinterpret_cast<const uint32_t *>(sm), y, (int)N, K, c.rounds, (int)ldy, cfg,
                       c.grid * c.B);
    return hipGetLastError();
}

template <int G, int GS, int MR>
hipError_t dispatch_dot2(const Dot2Cfg &c, const float *x, int M, const uint8_t *qs, const uint16_t *sm,
                         int64_t N, int64_t ldy, int K, float *y, const DeviceInfo &dev, hipStream_t stream)
{
    if (c.CB == 5 && c.U == 2) return run_dot2<5, 2, G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
    if (c.U == 1) {
        switch (c.CB) {
        case 1: return run_dot2<1, 1, G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 2: return run_dot2<2, 1, G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 3: return run_dot2<3, 1, G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 4: return run_dot2<4, 1, G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 5: return run_dot2<5, 1, G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 6: return run_dot2<6, 1, G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 8: return run_dot2<8, 1, G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        }
    } else {
        switch (c.CB) {
        case 1: return run_dot2<1, row_steps(1, MR), G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 2: return run_dot2<2, row_steps(2, MR), G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 3: return run_dot2<3, row_steps(3, MR), G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        case 4: return run_dot2<4, row_steps(4, MR), G, GS, MR>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        }
    }
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ arm B --

// One workgroup of kBWaves waves per CU holds the activations of its K range in
// LDS as MFMA A operands (MP = 1, 2, 4, 8 or 16 activation rows x 32 k per step,
// fp16, zeros for rows >= M; the MFMA's other rows read copies of these, so
// the fragment reads of a small M are mostly broadcasts, and are never
// stored), so every weight byte fetched from HBM meets its activations without
// another global read.  Weights are the B operand (16 weight rows x 32
// k), so the lane that loads a weight row also loads that row's scale and
// minimum and owns the row's outputs.  GS is the (scale, minimum) group along
// K: 256, or 32 for the group-32 format, where each MFMA step is one run of 32
// and carries its own pair.
constexpr int kBRows = 16;                      // weight rows per unit (one MFMA column block)
constexpr int kBWaves = 8;                      // waves per workgroup
constexpr int kBThreads = kBWaves * kWave;
constexpr int kBDepth = 4;                      // (unit, group) items in flight per wave
constexpr int kBTargetUnits = 256 * kBWaves;    // units wanted before K is split further
constexpr int kBTileRow = 9 * 16;               // weight tile row: 8 chunks of 16 B + 16 B pad

// per group of 256: f[16] (and with GS 256: X[16], c[16]; with GS 32: X and c
// per run, [8][16] each), fp32
__host__ __device__ constexpr int arm_b_fac_floats(int GS) { return GS == 32 ? 16 + 2 * 8 * kBRows : 3 * kBRows; }
// groups of 256 one workgroup holds in LDS
__host__ __device__ constexpr int arm_b_max_groups(int GS) { return GS == 32 ? 14 : 16; }
// per-wave tile: 16 weight rows x 144 B, and with GS 32 their 16 x 8 pairs
__host__ __device__ constexpr int arm_b_tile_bytes(int GS) { return kBRows * kBTileRow + (GS == 32 ? kBRows * 8 * 4 : 0); }
// A image of one group with MP activation rows: [step 8][kg 4][m MP] x 16 B
__host__ __device__ constexpr int arm_b_group_lds(int MP) { return 8 * 4 * MP * 16; }
__host__ __device__ constexpr size_t arm_b_x_lds_bytes(int gps, int GS, int MP)
{
    return (size_t)gps * (arm_b_group_lds(MP) + 4 * arm_b_fac_floats(GS));
}
__host__ __device__ constexpr size_t arm_b_lds_bytes(int gps, int GS, int MP)
{
    return arm_b_x_lds_bytes(gps, GS, MP) + (size_t)kBWaves * arm_b_tile_bytes(GS);
}

// Activations of groups g0 .. g0+gc-1 into LDS.  32 threads per (row m, group):
// thread (c, t) converts dword t of chunk c, i.e. elements 32c+4t..32c+4t+3
// (low nibbles) and 32c+16+4t..+3 (high nibbles, pre-scaled by 2^-4), in the
// slot order the weight widening produces.  Per (group, row): the factor
// f = 2^(24+e) that undoes the group's power-of-two scaling and the subnormal
// weights; per (group or run, row): X = sum of x and c = 7.5 * sum of (x - hi),
// the codes' mean share of the fp16 rounding of x, folded back in exactly (the
// remaining error is sum (x - hi) (q - 7.5), with centred codes).  Items are
// taken up to four per thread at a time, all their loads issued before any is
// used; rows >= M and items past the end read zeros (buffer bounds), and rows
// of items wholly past the image are skipped.  Only the MP image rows are
// converted.  Maxima and sums over a run's 32 (or 4) lanes go by DPP within
// rows of 16 lanes and one exchange between the two rows: the same pairs as
// an xor butterfly, so every lane ends with the same bits.  (With five
// shuffles per reduction this prologue took ~10 us of a 73 us call at 16
// rows, tiny-M K 4096 N 151936; now 68.6 us in all.  All items in one round
// trip held 110 more registers and was slower.)
template <int NB>
struct XGroupItems {
    float4 a[NB], b[NB];
};
// items per thread in one round trip
constexpr int x_batch(int MP) { return MP < 4 ? MP : 4; }

__device__ __forceinline__ float run32_max(float v)
{
    v = fmaxf(v, dpp_f32<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp_f32<kDppQuadSwap2>(v));
    v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
    return fmaxf(v, __shfl_xor(v, 16));
}

template <int L>
__device__ __forceinline__ float run_sum(float v)
{
    static_assert(L == 4 || L == 32, "runs of 4 or 32 lanes");
    v += dpp_f32<kDppQuadSwap1>(v);
    v += dpp_f32<kDppQuadSwap2>(v);
    if (L == 32) {
        v += dpp_f32<kDppRowHalfMirror>(v);
        v += dpp_f32<kDppRowMirror>(v);
        v += __shfl_xor(v, 16);
    }
    return v;
}

template <int MP>
__device__ __forceinline__ void load_x_groups(rsrc_t rx, int M, int K, int g0, int gc, int base,
                                              XGroupItems<x_batch(MP)> &v)
{
#pragma unroll
    for (int it = 0; it < x_batch(MP); ++it) {
        const int idx = base + threadIdx.x + it * kBThreads;
        const int pair = idx >> 5, sub = idx & 31;
        const int m = pair & (MP - 1), gl = pair / MP;
        const int c = sub >> 2, t = sub & 3;
        const bool ok = m < M && gl < gc;
        const uint32_t off =
            ok ? (uint32_t)(m * K + (g0 + gl) * kGroup + c * 32 + 4 * t) * 4u : 0x80000000u;
        v.a[it] = __builtin_bit_cast(float4, buf_load16(rx, off));
        v.b[it] = __builtin_bit_cast(float4, buf_load16(rx, off + 64));
    }
}

template <int GS, int MP>
__device__ __forceinline__ void convert_x_groups(int gc, int base, const XGroupItems<x_batch(MP)> &v, uint8_t *lds)
{
    float *fac = reinterpret_cast<float *>(lds + (size_t)gc * arm_b_group_lds(MP));
    constexpr int F = arm_b_fac_floats(GS);
    const int nx = MP * gc * 32;
#pragma unroll
    for (int it = 0; it < x_batch(MP); ++it) {
        // rows of items wholly past the image (few groups per K split): skipped
        // by the whole workgroup
        if (base + it * kBThreads >= nx) break;
        const int idx = base + threadIdx.x + it * kBThreads;
        const int pair = idx >> 5, sub = idx & 31;
        const int m = pair & (MP - 1), gl = pair / MP;
        const int c = sub >> 2, t = sub & 3;
        const float4 a = v.a[it], b = v.b[it];
        float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                           fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
        // the power-of-two scale is per group of 256; the sums per (scale, minimum) group
        amax = run32_max(amax);
        const int sc = chunk_exp(amax);
        const float ls = ldexpf(1.0f, -sc), hs = ldexpf(1.0f, -sc - 4);
        // sum of x on the scaled values (as in arm A)
        float sum = ((a.x * ls + a.y * ls) + (a.z * ls + a.w * ls)) +
                    ((b.x * ls + b.y * ls) + (b.z * ls + b.w * ls));
        sum = run_sum<GS / 8>(sum);
        sum = ldexpf(sum, sc - kYShift);
        // slot order of one widened dword: (4t, 4t+2) (16+4t, 16+4t+2) (4t+1, 4t+3) (16+4t+1, 16+4t+3)
        const float w[8] = {a.x * ls, a.z * ls, b.x * hs, b.z * hs, a.y * ls, a.w * ls, b.y * hs, b.w * hs};
        uint32_t hw[4];
        float dl = 0.0f, dh = 0.0f;  // residuals of low / high slots, in scaled units
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const _Float16 h0 = (_Float16)w[2 * p], h1 = (_Float16)w[2 * p + 1];
            const float r = (w[2 * p] - (float)h0) + (w[2 * p + 1] - (float)h1);
            if (p & 1) dh += r; else dl += r;
            hw[p] = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
        }
        float delta = ldexpf(dl, sc - kYShift) + ldexpf(dh, sc + 4 - kYShift);
        delta = run_sum<GS / 8>(delta);
        if (gl < gc) {
            // GS 256: step d mixes runs (kg = run & 3, d = (run >> 2) * 4 + dword);
            // GS 32: step d is run d, lane kg its dword kg
            const int kg = GS == 32 ? t : (c & 3), d = GS == 32 ? c : (c >> 2) * 4 + t;
            *reinterpret_cast<uint4 *>(lds + (size_t)gl * arm_b_group_lds(MP) + ((d * 4 + kg) * MP + m) * 16) =
                make_uint4(hw[0], hw[1], hw[2], hw[3]);
            float *fg = fac + gl * F;
            if (sub == 0) fg[m] = ldexpf(1.0f, 24 - kYShift + sc);
            if (GS == 32 && t == 0) {
                fg[kBRows + c * kBRows + m] = sum;
                fg[kBRows + 8 * kBRows + c * kBRows + m] = 7.5f * delta;
            }
            if (GS != 32 && sub == 0) {
                fg[kBRows + m] = sum;
                fg[2 * kBRows + m] = 7.5f * delta;
            }
        }
    }
}

// Workgroup b covers K split b % nsplit; with wps workgroups per split, wave
// w of workgroup r is wave gw = r * kBWaves + w of the split and takes the
// 16-row units gw, gw + GW, ... (GW = wps * kBWaves), so the chip sweeps the
// matrix front to back.  A wave streams (unit, group) items through a ring of
// D register slots: each slot is refilled with the item D places later as
// soon as it is consumed, so D items of weights stay in flight with no
// barrier in the loop.  The weights of an item (16 rows x 128 B) arrive as
// whole 128-byte lines, 8 rows per load instruction, and are turned into the
// MFMA B layout through a small per-wave LDS tile.  GS 256: lane (j, kg) takes
// chunks kg and 4 + kg of row j; with kSmQuad (groups per split a multiple of
// 4) the (scale, minimum) pairs come 4 groups per load, lane (j, kg) holding
// group 4q + kg of row j, and reach the other lanes by a cross-lane read.
// GS 32: step d is run d (lane (j, kg) its dword kg); the lane that loads a
// run also loads the run's pair, which goes through the tile with the codes.
// Items past the wave's end load out of range (zeros) and write nothing.
template <int D, bool kSmQuad, int GS, int MP>
__global__ __launch_bounds__(kBThreads) void k_gemv_mfma(const float *__restrict__ x,
                                                         const uint8_t *__restrict__ qs,
                                                         const uint32_t *__restrict__ sm,
                                                         float *__restrict__ out, int64_t ldo, int M,
                                                         int N, int K, int gps, int nsplit, int wps)
{
    static_assert(!kSmQuad || (D % 4 == 0 && GS == kGroup), "quads of slots, groups of 256");
    constexpr bool kG32 = GS == 32;
    constexpr int F = arm_b_fac_floats(GS);
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
    const int lane = threadIdx.x & 63, j = lane & 15, kg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x % nsplit, wr = blockIdx.x / nsplit;
    const int GK = K / kGroup;
    const int SPR = K / GS;  // (scale, minimum) pairs per row
    const int g0 = split * gps;
    const int gc = min(GK, g0 + gps) - g0;  // >= 1: the host makes every split non-empty
    const int R = (N + kBRows - 1) / kBRows;
    const int gw = wr * kBWaves + wave, GW = wps * kBWaves;
    const int nunits = R > gw ? (R - gw + GW - 1) / GW : 0;
    const int nitems = nunits * gc;
    const uint32_t rowbytes = K / 2;
    // partials [split][M][ldo] (or y itself): the host keeps every offset below 2^31
    const rsrc_t r_out = make_rsrc(out + (int64_t)split * M * ldo, (uint32_t)(((int64_t)(M - 1) * ldo + N) * 4));
    uint8_t *tile = xl + arm_b_x_lds_bytes(gc, GS, MP) + wave * arm_b_tile_bytes(GS);
    uint32_t *tile_sm = reinterpret_cast<uint32_t *>(tile + kBRows * kBTileRow);  // GS 32: [row][run]

    const rsrc_t r_qs = make_rsrc(qs, (uint32_t)N * rowbytes);
    const rsrc_t r_sm = make_rsrc(sm, (uint32_t)N * SPR * 4u);
    uint4 wq[D][2];  // rows 16 u + (lane >> 3) and + 8, chunk lane & 7
    // (scale, minimum) pairs: GS 256 per slot or per quad of slots; GS 32 the
    // pairs of this lane's two rows and run
    uint32_t wsm[kG32 ? 2 * D : (kSmQuad ? D / 4 : D)];
    auto load_item = [&](int s, int unit, int gl) {
        const bool ok = unit < nunits;
        const int r0 = (gw + GW * unit) * kBRows + (lane >> 3);
        const uint32_t gb = (uint32_t)(g0 + gl) * 128u + (lane & 7) * 16;
        // rows past N read zeros (row N is out of the descriptor's range)
        const uint32_t o0 = ok ? (uint32_t)min(r0, N) * rowbytes + gb : 0x80000000u;
        const uint32_t o1 = ok ? (uint32_t)min(r0 + 8, N) * rowbytes + gb : 0x80000000u;
        wq[s][0] = buf_load16_nt(r_qs, o0);
        wq[s][1] = buf_load16_nt(r_qs, o1);
        if (kG32) {
            const uint32_t run = (uint32_t)(g0 + gl) * 8u + (lane & 7);
            wsm[2 * s] = buf_load4_nt(r_sm, ok ? ((uint32_t)min(r0, N) * SPR + run) * 4u : 0x80000000u);
            wsm[2 * s + 1] = buf_load4_nt(r_sm, ok ? ((uint32_t)min(r0 + 8, N) * SPR + run) * 4u : 0x80000000u);
        } else if (!kSmQuad) {
            const int n = min((gw + GW * unit) * kBRows + j, N);
            wsm[s] = buf_load4_nt(r_sm, ok ? ((uint32_t)n * SPR + g0 + gl) * 4u : 0x80000000u);
        }
    };
    // pairs of groups gl .. gl+3 of the unit: lane (j, kg) takes group gl + kg of row j
    auto load_quad = [&](int q, int unit, int gl) {
        const bool ok = unit < nunits;
        const int n = min((gw + GW * unit) * kBRows + j, N);
        wsm[q] = buf_load4_nt(r_sm, ok ? ((uint32_t)n * SPR + g0 + gl + kg) * 4u : 0x80000000u);
    };
    // activation loads first, then the weight ring, then the conversion
    const rsrc_t r_x = make_rsrc(x, (uint32_t)M * K * 4u);
    const int nx = MP * gc * 32;
    XGroupItems<x_batch(MP)> xv;
    load_x_groups<MP>(r_x, M, K, g0, gc, 0, xv);
    int lu = 0, lg = 0;  // next item to load
#pragma unroll
    for (int s = 0; s < D; ++s) {
        load_item(s, lu, lg);
        if (kSmQuad && s % 4 == 3) load_quad(s / 4, lu, lg - 3);
        if (++lg == gc) { lg = 0; ++lu; }
    }
    convert_x_groups<GS, MP>(gc, 0, xv, xl);
    for (int base = x_batch(MP) * kBThreads; base < nx; base += x_batch(MP) * kBThreads) {
        load_x_groups<MP>(r_x, M, K, g0, gc, base, xv);
        convert_x_groups<GS, MP>(gc, base, xv, xl);
    }
    __syncthreads();

    const float *fac = reinterpret_cast<const float *>(xl + (size_t)gc * arm_b_group_lds(MP));
    float4_t yacc = {0.f, 0.f, 0.f, 0.f};
    int cu = 0, cg = 0;  // item being computed
    for (int base = 0; base < nitems; base += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            // the previous item's epilogue completes before this item's LDS
            // traffic is issued (only one item's operands are live at a time)
            asm volatile("" : "+v"(yacc)::"memory");
            // weights of slot s through the tile: row r at r * kBTileRow, chunk c at 16 c
            *reinterpret_cast<uint4 *>(tile + (lane >> 3) * kBTileRow + (lane & 7) * 16) = wq[s][0];
            *reinterpret_cast<uint4 *>(tile + (8 + (lane >> 3)) * kBTileRow + (lane & 7) * 16) = wq[s][1];
            uint4 bw0, bw1;
            uint32_t smv = 0;
            if (kG32) {
                tile_sm[(lane >> 3) * 8 + (lane & 7)] = wsm[2 * s];
                tile_sm[(8 + (lane >> 3)) * 8 + (lane & 7)] = wsm[2 * s + 1];
                // dword kg of runs 0..7 of row j
                const uint32_t *tr = reinterpret_cast<const uint32_t *>(tile + j * kBTileRow) + kg;
                bw0 = make_uint4(tr[0], tr[4], tr[8], tr[12]);
                bw1 = make_uint4(tr[16], tr[20], tr[24], tr[28]);
            } else {
                bw0 = *reinterpret_cast<const uint4 *>(tile + j * kBTileRow + kg * 16);
                bw1 = *reinterpret_cast<const uint4 *>(tile + j * kBTileRow + (4 + kg) * 16);
                smv = kSmQuad ? (uint32_t)__shfl((int)wsm[s / 4], j + 16 * (s % 4)) : wsm[s];
            }
            // slot s is consumed: refill it in place with the item D later
            // (its (scale, minimum) quad once the last item using it is read)
            asm volatile("" : "+v"(yacc)::"memory");
            load_item(s, lu, lg);
            if (kSmQuad && s % 4 == 3) load_quad(s / 4, lu, lg - 3);
            if (++lg == gc) { lg = 0; ++lu; }

            // lane (j, kg) reads image row j mod MP; its factors those of rows
            // 4 kg' .. 4 kg' + 3, kg' = kg mod MP/4 (0 below four rows; rows
            // past MP are copies or unset, and never stored)
            const int kq = MP >= 4 ? (kg & (MP / 4 - 1)) : 0;
            const uint8_t *ag = xl + (size_t)cg * arm_b_group_lds(MP) + (kg * MP + (j & (MP - 1))) * 16;
            const float *fg = fac + cg * F;
            const float4 f = *reinterpret_cast<const float4 *>(fg + 4 * kq);
            if (kG32) {
                // one MFMA per run, each with its own (scale, minimum): the
                // group's T = sum over runs of scale * dot on the VALU (two
                // accumulators so a run's scaling overlaps the next product),
                // its minimum and correction terms sum over runs of (c scale +
                // X minimum) as four fp32 MFMAs of rank 2 accumulating into y
                // (A[m][k] = c or X of run 2q + k/2 for row m, B[k][n] = scale
                // or minimum of that run for row n), then y += f T
                float4_t accs[2];
                float4_t T = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    const half8_t a = *reinterpret_cast<const half8_t *>(ag + d * 4 * MP * 16);
                    const uint4 c4 = d < 4 ? bw0 : bw1;
                    const uint32_t w = (d & 3) == 0 ? c4.x : (d & 3) == 1 ? c4.y : (d & 3) == 2 ? c4.z : c4.w;
                    uint32_t p[4];
                    widen(w, p);
                    const half8_t b = __builtin_bit_cast(half8_t, uint4{p[0], p[1], p[2], p[3]});
                    accs[d & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if (d > 0) {
                        const float sf = f16_bits_to_f32(tile_sm[j * 8 + d - 1] & 0xFFFFu);
                        const float4_t acc = accs[(d - 1) & 1];
#pragma unroll
                        for (int e = 0; e < 4; ++e) T[e] = fmaf(sf, acc[e], T[e]);
                    }
                }
                {
                    const float sf = f16_bits_to_f32(tile_sm[j * 8 + 7] & 0xFFFFu);
                    const float4_t acc = accs[1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) T[e] = fmaf(sf, acc[e], T[e]);
                }
                const int ki = lane >> 4, mi = j & (MP - 1);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int run = 2 * q + (ki >> 1);
                    const float av = fg[((ki & 1) ? kBRows : 9 * kBRows) + run * kBRows + mi];
                    const uint32_t sv = tile_sm[j * 8 + run];
                    const float bv = f16_bits_to_f32((ki & 1) ? (sv >> 16) : (sv & 0xFFFFu));
                    yacc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, yacc, 0, 0, 0);
                }
                yacc[0] = fmaf(f.x, T[0], yacc[0]);
                yacc[1] = fmaf(f.y, T[1], yacc[1]);
                yacc[2] = fmaf(f.z, T[2], yacc[2]);
                yacc[3] = fmaf(f.w, T[3], yacc[3]);
            } else {
                // two independent accumulator chains (even / odd steps)
                float4_t acc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    const half8_t a = *reinterpret_cast<const half8_t *>(ag + d * 4 * MP * 16);
                    const uint4 c4 = d < 4 ? bw0 : bw1;
                    const uint32_t w = (d & 3) == 0 ? c4.x : (d & 3) == 1 ? c4.y : (d & 3) == 2 ? c4.z : c4.w;
                    uint32_t p[4];
                    widen(w, p);
                    const half8_t b = __builtin_bit_cast(half8_t, uint4{p[0], p[1], p[2], p[3]});
                    acc2[d & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc2[d & 1], 0, 0, 0);
                }
                const float4_t acc = acc2[0] + acc2[1];
                const float4 X = *reinterpret_cast<const float4 *>(fg + kBRows + 4 * kq);
                const float4 cc = *reinterpret_cast<const float4 *>(fg + 2 * kBRows + 4 * kq);
                const float sf = f16_bits_to_f32(smv & 0xFFFFu), mf = f16_bits_to_f32(smv >> 16);
                yacc[0] = fmaf(sf, fmaf(f.x, acc[0], cc.x), fmaf(mf, X.x, yacc[0]));
                yacc[1] = fmaf(sf, fmaf(f.y, acc[1], cc.y), fmaf(mf, X.y, yacc[1]));
                yacc[2] = fmaf(sf, fmaf(f.z, acc[2], cc.z), fmaf(mf, X.z, yacc[2]));
                yacc[3] = fmaf(sf, fmaf(f.w, acc[3], cc.w), fmaf(mf, X.w, yacc[3]));
            }
            if (cg == gc - 1) {
                // unit complete: lane (j, kg) holds rows m = 4kg+e of column n
                const int n = (gw + GW * cu) * kBRows + j;
                if (cu < nunits && n < N) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * kg + e < M)
                            buf_store4(r_out, ((uint32_t)(4 * kg + e) * (uint32_t)ldo + (uint32_t)n) * 4u, unshift(yacc[e]));
                }
                yacc = float4_t{0.f, 0.f, 0.f, 0.f};
                cg = 0;
                ++cu;
            } else {
                ++cg;
            }
        }
    }
}

// y[m][n] (row stride ldy) = sum over splits of partial[s][m][n] (dense
// [nsplit][M][N]), in split order
__global__ __launch_bounds__(256) void k_splitk_sum(const float *__restrict__ partial,
                                                    float *__restrict__ y, int M, int N, int64_t ldy,
                                                    int nsplit)
{
    const int64_t count = (int64_t)M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        float v = 0.0f;
        for (int s = 0; s < nsplit; ++s) v += partial[(int64_t)s * count + i];
        y[(i / N) * ldy + i % N] = v;
    }
}

struct MfmaCfg {
    int nsplit, gps;
};

// K split: as few splits as LDS allows, more while the 16-row units are too
// few to give every wave of the chip one (small N), every split non-empty.
// Independent of the device so the workspace size is too.
MfmaCfg choose_mfma(int64_t N, int K, int GS)
{
    MfmaCfg c{};
    const int GK = K / kGroup;
    const int64_t R = (N + kBRows - 1) / kBRows;
    const int maxg = arm_b_max_groups(GS);
    int ns = (GK + maxg - 1) / maxg;
    while (R * ns < kBTargetUnits && ns * 2 <= GK) ns *= 2;
    c.gps = (GK + ns - 1) / ns;
    c.nsplit = (GK + c.gps - 1) / c.gps;
    return c;
}

// Activation rows of the image for an M-row call.  With fewer rows than the
// MFMA's 16 the fragment reads repeat rows: tiny-M K 4096 N 151936 at M = 4
// 72.3 -> 60.6 us, M = 8 70.4 -> 63.0 us, bit-identical (12 or 16 waves per
// workgroup, in the LDS this frees, were slower).
constexpr int arm_b_image_rows(int M) { return M <= 2 ? M : (M <= 4 ? 4 : (M <= 8 ? 8 : 16)); }

template <int GS, int MP>
hipError_t launch_arm_b_mp(const MfmaCfg &c, const float *x, int M, const uint8_t *qs, const uint16_t *sm,
                           int64_t N, int64_t ldy, int K, float *y, void *workspace, size_t ws_bytes,
                           const DeviceInfo &dev, hipStream_t stream)
{
    const size_t lds = arm_b_lds_bytes(c.gps, GS, MP);
    if (lds > (size_t)dev.lds_bytes) return hipErrorInvalidConfiguration;
    const int64_t R = (N + kBRows - 1) / kBRows;
    // workgroups per split: one per CU overall, at most one per kBWaves units
    int64_t wps = dev.num_cus / c.nsplit;
    if (wps < 1) wps = 1;
    if (wps > (R + kBWaves - 1) / kBWaves) wps = (R + kBWaves - 1) / kBWaves;
    // split-K partials are dense [nsplit][M][N] in the workspace (which must
    // hold them: the plan was made for the whole matrix, this is one row range
    // of it); otherwise y is written directly
    if (c.nsplit > 1 && (workspace == nullptr || (size_t)c.nsplit * M * N * sizeof(float) > ws_bytes))
        return hipErrorInvalidValue;
    float *out = c.nsplit > 1 ? static_cast<float *>(workspace) : y;
    const int64_t ldo = c.nsplit > 1 ? N : ldy;
    const uint32_t *sm32 = reinterpret_cast<const uint32_t *>(sm);
    // the kernel addresses its output through one descriptor with 32-bit
    // offsets (the C ABI rejects shapes beyond it, so this does not trigger)
    if (((int64_t)(M - 1) * ldo + N) * 4 > kMaxBufferBytes) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(wps * c.nsplit)), block(kBThreads);
    if constexpr (GS == 32) {
        hipLaunchKernelGGL((k_gemv_mfma<kBDepth, false, 32, MP>), grid, block, lds, stream, x, qs, sm32, out,
                           ldo, M, (int)N, K, c.gps, c.nsplit, (int)wps);
    } else {
        if ((K / kGroup) % c.gps == 0 && c.gps % 4 == 0) {
            // (scale, minimum) quads need every split's group count to be a multiple of 4
            hipLaunchKernelGGL((k_gemv_mfma<kBDepth, true, kGroup, MP>), grid, block, lds, stream, x, qs, sm32,
                               out, ldo, M, (int)N, K, c.gps, c.nsplit, (int)wps);
        } else {
            hipLaunchKernelGGL((k_gemv_mfma<kBDepth, false, kGroup, MP>), grid, block, lds, stream, x, qs,
                               sm32, out, ldo, M, (int)N, K, c.gps, c.nsplit, (int)wps);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.nsplit == 1) return e;
    const int64_t count = (int64_t)M * N;
    int64_t sb = (count + 255) / 256;
    if (sb > (int64_t)dev.num_cus * 8) sb = (int64_t)dev.num_cus * 8;
    hipLaunchKernelGGL(k_splitk_sum, dim3((unsigned)sb), dim3(256), 0, stream, out, y, M, (int)N, ldy,
                       c.nsplit);
    return hipGetLastError();
}

template <int GS>
hipError_t launch_arm_b(const MfmaCfg &c, const float *x, int M, const uint8_t *qs, const uint16_t *sm, int64_t N,
                        int64_t ldy, int K, float *y, void *workspace, size_t ws_bytes, const DeviceInfo &dev,
                        hipStream_t stream)
{
    switch (arm_b_image_rows(M)) {
    case 1: return launch_arm_b_mp<GS, 1>(c, x, M, qs, sm, N, ldy, K, y, workspace, ws_bytes, dev, stream);
    case 2: return launch_arm_b_mp<GS, 2>(c, x, M, qs, sm, N, ldy, K, y, workspace, ws_bytes, dev, stream);
    case 4: return launch_arm_b_mp<GS, 4>(c, x, M, qs, sm, N, ldy, K, y, workspace, ws_bytes, dev, stream);
    case 8: return launch_arm_b_mp<GS, 8>(c, x, M, qs, sm, N, ldy, K, y, workspace, ws_bytes, dev, stream);
    default: return launch_arm_b_mp<GS, 16>(c, x, M, qs, sm, N, ldy, K, y, workspace, ws_bytes, dev, stream);
    }
}

}  // namespace

// Largest K whose activation image arm A holds in LDS (80 B per 32 of K and
// activation row plus at most 2 KB of slice partials per row, within a
// workgroup's 160 KB), for one and for two rows; longer K takes the
// matrix-core arm, which splits K over workgroups.
constexpr int kArmAMaxK = 64512;
constexpr int kArmAMaxK2 = 31744;
constexpr int kArmAMaxK4 = 15360;

// Activation rows arm A's image holds for an M-row call (0: the matrix-core
// arm).  One row always (measured faster at every N).  Three and four rows
// only below 65536 weight rows: there the matrix-core arm's fixed costs
// (activation image per workgroup, K split with a second pass) dominate
// (4096 x 4096 at M = 4: 9.8 vs 20.6 us), while on the lm_head widths four
// rows make arm A VALU-bound (88 vs 72 us at K = 4096).  Two rows likewise,
// except that from 65536 weight rows the matrix-core arm's two-row image wins
// only where it takes K without a split (K <= 4096: tiny-M K 4096 N 151936
// 62.9 -> 56.9 us, K 2560 42.1 -> 39.3 us; K 12288 N 65536, three splits,
// 82.0 vs 86.5 us).
constexpr int64_t kArmA4MaxN = 65536;
int arm_a_rows(int64_t M, int64_t N, int64_t K)
{
    if (M == 1 && K <= kArmAMaxK) return 1;
    if (M == 2 && K <= kArmAMaxK2 && (N < kArmA4MaxN || K > 16 * kGroup)) return 2;
    if (M >= 3 && M <= 4 && K <= kArmAMaxK4 && N < kArmA4MaxN) return 4;
    return 0;
}

// Weight rows one launch addresses: one descriptor reaches < 2 GiB of qs,
// so taller matrices run as row ranges of at most this many rows.
int64_t gemv_range_rows(int64_t K) { return ((kMaxBufferBytes - 1) / (K / 2)) / 64 * 64; }

// The plan of an M x N x K call, a function of the whole shape only: every
// row range of a tall matrix runs the same arm with the same K split, and the
// workspace query, the argument check and the launch all agree.
GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int group)
{
    GemvPlan p{};
    p.MR = arm_a_rows(M, N, K);
    if (p.MR == 0) {
        const MfmaCfg c = choose_mfma(N, (int)K, group);
        p.nsplit = c.nsplit;
        p.gps = c.gps;
    } else {
        p.nsplit = 1;
        p.gps = 0;
    }
    return p;
}

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int group)
{
    if (M < 1 || N < 1 || K < kGroup) return 0;
    const GemvPlan p = plan_gemv(M, N, K, group);
    if (p.MR != 0 || p.nsplit == 1) return 0;
    // partials [nsplit][M][rows of the largest range]; the ranges run one
    // after another on the stream and reuse the same bytes
    const int64_t rows = N < gemv_range_rows(K) ? N : gemv_range_rows(K);
    return (size_t)p.nsplit * (size_t)M * (size_t)rows * sizeof(float);
}

bool gemv_shape_supported(int64_t M, int64_t N, int64_t K, int group)
{
    if (M < 1 || N < 1 || K < kGroup) return true;
    const GemvPlan p = plan_gemv(M, N, K, group);
    // the matrix-core arm without a K split writes y through one descriptor
    return !(p.MR == 0 && p.nsplit == 1 && M * N > kMaxBufferBytes / 4);
}

namespace {

template <int GS>
hipError_t launch_gemv_rows(const GemvPlan &p, const float *x, int M, const uint8_t *qs, const uint16_t *sm,
                            int64_t N, int64_t ldy, int K, float *y, void *workspace, size_t ws_bytes,
                            const DeviceInfo &dev, hipStream_t stream)
{
    const int MR = p.MR;
    if (MR != 0) {
        const Dot2Cfg c = choose_dot2(N, K, MR, dev);
        if (MR == 1)
            return c.G == 16 ? dispatch_dot2<16, GS, 1>(c, x, M, qs, sm, N, ldy, K, y, dev, stream)
                             : dispatch_dot2<8, GS, 1>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        if (MR == 2)
            return c.G == 16 ? dispatch_dot2<16, GS, 2>(c, x, M, qs, sm, N, ldy, K, y, dev, stream)
                             : dispatch_dot2<8, GS, 2>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
        return c.G == 16 ? dispatch_dot2<16, GS, 4>(c, x, M, qs, sm, N, ldy, K, y, dev, stream)
                         : dispatch_dot2<8, GS, 4>(c, x, M, qs, sm, N, ldy, K, y, dev, stream);
    }
    return launch_arm_b<GS>(MfmaCfg{p.nsplit, p.gps}, x, M, qs, sm, N, ldy, K, y, workspace, ws_bytes, dev,
                            stream);
}

}  // namespace

hipError_t launch_gemv(const float *x, int M, const uint8_t *qs, const uint16_t *sm, int64_t N,
                       int K, int group, float *y, void *workspace, size_t ws_bytes, const DeviceInfo &dev,
                       hipStream_t stream)
{
    const GemvPlan p = plan_gemv(M, N, K, group);
    // one descriptor addresses < 2 GiB of weights: split taller matrices into
    // row ranges (y keeps its row stride N)
    const int64_t rows_max = gemv_range_rows(K);
    for (int64_t n0 = 0; n0 < N; n0 += rows_max) {
        const int64_t nn = N - n0 < rows_max ? N - n0 : rows_max;
        const uint8_t *qs0 = qs + n0 * (K / 2);
        const uint16_t *sm0 = sm + n0 * (K / group) * 2;
        const hipError_t e =
            group == 32
                ? launch_gemv_rows<32>(p, x, M, qs0, sm0, nn, N, K, y + n0, workspace, ws_bytes, dev, stream)
                : launch_gemv_rows<kGroup>(p, x, M, qs0, sm0, nn, N, K, y + n0, workspace, ws_bytes, dev, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4mi
