/*
 * q4mi.h -- C ABI of the MI355X (gfx950) 4-bit weight-quantized matmul library
 * (libq4mi.so): weight packing, Q8_1 activation quantization, the
 * dequant-fused GEMV used in decode and the integer "MMQ" GEMM used in prefill.
 *
 * Sources of the operations (pages cited by title and section):
 *   - 4-bit weights in groups of 256 along K with an fp16 scale and an fp16
 *     minimum per group, two codes per byte: the HFQ4-G256 format named in the
 *     hipfire MMQ-prefill note (ai-navigate-news.com article, list of changes
 *     and benchmark table).  The page gives no byte layout; the layout below is
 *     this library's.
 *   - Q8_1 pre-quantized activations and i8 matrix-core tile products over
 *     128x128 output tiles with LDS staging: same note, list of changes.
 *   - A quantized GEMV arm with fp32 output for few activation rows, and a
 *     split-K arm for shapes with too few output rows to fill the GPU:
 *     vllm.cpp issue 5 ("GFX1100-TG200 campaign"), "Starting position".
 *   - Integer dot products bit-exact against a CPU implementation: vllm.cpp
 *     pull request 4 ("spec(GFX1100-TG150)"), "Design", correctness policy.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller.  The library never allocates, frees or synchronizes; work
 *     is enqueued on `stream` (a hipStream_t passed as void*, NULL = the null
 *     stream) and the call returns before it runs.
 *   - Arrays are dense and row-major.  K must be a positive multiple of 256.
 *   - Arguments are validated before any HIP call; an invalid call enqueues
 *     nothing and returns a negative Q4_ERR_* code.  A call with M == 0 or
 *     N == 0 (an empty product) is valid and enqueues nothing.
 *   - The device must be gfx950 (MI355X class); any other returns Q4_ERR_ARCH.
 *   - Non-finite inputs are outside the contract.
 *   - Calls are stateless apart from a per-device cache of device properties,
 *     and are safe to issue from several host threads.
 *
 * Data layouts:
 *   W   fp32 [N][K]               weights before packing
 *   qs  u8   [N][K/2]             4-bit codes.  Group g of row n occupies bytes
 *                                 128g .. 128g+127 of the row.  Within a group,
 *                                 elements 32j .. 32j+31 take bytes 16j .. 16j+15;
 *                                 byte i of them holds element 32j+i in its low
 *                                 nibble and element 32j+i+16 in its high nibble.
 *   sm  fp16 [N][K/256][2]        (scale, minimum) per group, as IEEE binary16 bits.
 *                                 Dequantized weight: w = scale * q + minimum.
 *   x   fp32 [M][K]               activations
 *   qa  i8   [M][K]               Q8_1 codes
 *   ds  fp16 [M][K/32][2]         (d, s) per block of 32: x ~= d * a, s = d * sum(a)
 *   y   fp32 [M][N]               y = x * W^T
 */
#ifndef Q4MI_H
#define Q4MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4MI_ABI_VERSION 1

enum {
    Q4_OK = 0,
    Q4_ERR_ARG = -1,       /* null pointer, bad dimension or size out of range   */
    Q4_ERR_ALIGN = -2,     /* pointer not aligned as required                     */
    Q4_ERR_WORKSPACE = -3, /* workspace missing or smaller than required          */
    Q4_ERR_ARCH = -4,      /* current device is not gfx950                        */
    Q4_ERR_LAUNCH = -5,    /* the HIP runtime rejected the kernel launch          */
    Q4_ERR_DEVICE = -6     /* no usable HIP device / runtime query failed         */
};

/* Largest supported dimensions. */
#define Q4_MAX_K (1 << 20)          /* K <= 1048576                               */
#define Q4_MAX_N ((1LL << 31) - 1)  /* N rows of weights                          */
#define Q4_MAX_M_MMQ ((1LL << 31) - 1)
#define Q4_GEMV_MAX_M 16            /* q4_gemv takes 1..16 activation rows        */

/* ABI version of the loaded library (Q4MI_ABI_VERSION it was built with). */
int q4_abi_version(void);

/* Static text for an error code (never NULL). */
const char *q4_strerror(int code);

/*
 * q4_pack -- quantize W [N][K] fp32 to 4-bit codes with a scale and a minimum
 * per group of 256 consecutive k (the HFQ4-G256 weight format of the hipfire
 * MMQ-prefill note).  For each group, in IEEE fp32 with round-to-nearest-even:
 *     mn = min w, mx = max w              (a zero counts as +0)
 *     scale16 = fp16(fp32(mx - mn) / 15), min16 = fp16(mn)
 *     q = 0 if scale16 == 0, else clamp(rint((w - min16) / scale16), 0, 15)
 * Output is bit-exact with the definition.
 *   W:  device fp32 [N][K], 16-byte aligned.
 *   qs: device u8 [N][K/2], 16-byte aligned.   sm: device u16 [N][K/256][2],
 *   4-byte aligned.  Outputs must not overlap W.
 * Errors: Q4_ERR_ARG (null, N < 0, K not a positive multiple of 256, K or N too
 * large), Q4_ERR_ALIGN, Q4_ERR_ARCH, Q4_ERR_DEVICE, Q4_ERR_LAUNCH.
 */
int q4_pack(const float *W, int64_t N, int64_t K, uint8_t *qs, uint16_t *sm, void *stream);

/*
 * q8_1_quantize -- quantize activations x [M][K] fp32 to Q8_1 (the activation
 * format the hipfire MMQ-prefill note pre-quantizes prefill inputs into).
 * Per block of 32 consecutive k, in IEEE fp32 with round-to-nearest-even:
 *     amax = max |x|, d16 = fp16(amax / 127)
 *     a = 0 if d16 == 0, else clamp(rint(x / d16), -127, 127)
 *     s16 = fp16(d16 * sum(a))
 * Output is bit-exact with the definition.  K must be a positive multiple of
 * 32 here (256 for the matmuls that consume it).
 *   x:  device fp32 [M][K], 16-byte aligned.
 *   qa: device i8 [M][K], 16-byte aligned.  ds: device u16 [M][K/32][2],
 *   4-byte aligned.
 * Errors: Q4_ERR_ARG, Q4_ERR_ALIGN, Q4_ERR_ARCH, Q4_ERR_DEVICE, Q4_ERR_LAUNCH.
 */
int q8_1_quantize(const float *x, int64_t M, int64_t K, int8_t *qa, uint16_t *ds, void *stream);

/*
 * q4_gemv_workspace_bytes -- device workspace q4_gemv needs for this shape
 * (0 when the shape runs without one).  Pure host function, no HIP call.
 * Returns 0 for shapes q4_gemv would reject.
 */
size_t q4_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * q4_gemv -- y [M][N] = x [M][K] * dequant(qs, sm)^T for 1 <= M <= 16 fp32
 * activation rows: the dequant-fused decode GEMV with fp32 output (the
 * "tiny-N f32-out GEMV" and "split-K" arms of vllm.cpp issue 5, "Starting
 * position"), streaming the 4-bit weights once from HBM.
 * The fp32 sum order is the library's; results match the fp64 definition
 * sum_k x[m][k] * (scale * q + minimum) to max|dy| / max|y| <= 2e-3 and
 * sum(dy^2) / sum(y^2) <= 1e-6 on well-scaled inputs (activations are rounded
 * to fp16 with a power-of-two scale per 32-element chunk inside the kernel).
 * Every finite x gives finite y unless the exact y itself overflows fp32:
 * chunks anywhere from fp32 subnormals to the fp32 maximum are scaled into
 * fp16's range (chunks below 2^-113 by 2^127), and the partial sums are
 * carried at 2^-10 of their value; rows whose outputs fall below about 1e-37
 * are accurate to about 2^-130 absolute rather than relatively.
 * Reruns with the same inputs are bit-identical.
 * Shape limit: when the shape runs on the matrix-core arm without a K split
 * (M >= 5, or M = 3..4 with N >= 65536 or K > 15360, or M = 2 with
 * K > 31744, or M = 1 with K > 64512; and N large enough that K is not
 * split), M * N must not exceed 2^29 (y is addressed through one 2 GiB
 * buffer descriptor); larger shapes return Q4_ERR_ARG.  Weights beyond
 * 2 GiB are fine: they run as row ranges of one plan.
 *   x:  device fp32 [M][K], 16-byte aligned.   qs: device u8 [N][K/2],
 *   16-byte aligned.   sm: device u16 [N][K/256][2], 4-byte aligned.
 *   y:  device fp32 [M][N], 4-byte aligned; must not overlap the inputs.
 *   workspace: device buffer of at least q4_gemv_workspace_bytes(M, N, K)
 *   bytes, 16-byte aligned (may be NULL when that is 0).  Its contents on entry
 *   are ignored and on exit are unspecified.  Two calls that run concurrently
 *   must not share a workspace.
 * Errors: Q4_ERR_ARG (M outside 0..16, N < 0, K not a positive multiple of
 * 256, the shape limit above, null pointer), Q4_ERR_ALIGN, Q4_ERR_WORKSPACE,
 * Q4_ERR_ARCH, Q4_ERR_DEVICE, Q4_ERR_LAUNCH.
 */
int q4_gemv(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm, int64_t N,
            int64_t K, float *y, void *workspace, size_t ws_bytes, void *stream);

/*
 * q4_gemv_noalloc -- q4_gemv for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels, plan and results (bit for bit) as q4_gemv,
 * with no workspace argument.  Shapes that split K keep their partial sums in
 * a fixed device array of Q4_NOALLOC_SCRATCH_BYTES inside the library, one
 * per device, allocated when the library's code is loaded on that device and
 * held until the process ends; the call itself allocates nothing.
 * A shape whose q4_gemv_workspace_bytes exceeds Q4_NOALLOC_SCRATCH_BYTES is
 * refused with Q4_ERR_WORKSPACE (use q4_gemv with a workspace).  Every call
 * on one device shares that array: two calls that may run at the same time on
 * one device (different streams, or graphs replayed concurrently) race and
 * must be ordered by the caller.  Nothing in the array needs to start at
 * zero (each call writes every partial it later reads).
 * Arguments and errors otherwise as q4_gemv.
 */
#define Q4_NOALLOC_SCRATCH_BYTES (32u << 20)
int q4_gemv_noalloc(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm, int64_t N,
                    int64_t K, float *y, void *stream);

/*
 * Group-32 variant (the "W4A16, asymmetric, group 32" int4 checkpoints the vLLM
 * ROCM_OCTAVE pull request validates on, "Validation" and the QSA evaluation
 * setup).  The code bytes qs are laid out exactly as for group 256; the
 * (scale, minimum) pairs come one per 32 consecutive k: sm u16 [N][K/32][2].
 * K must still be a positive multiple of 256.  Definitions, accuracy, argument
 * rules and errors are those of the group-256 functions with "group of 256"
 * read as "group of 32".
 *   q4_pack_g32                  -- q4_pack over groups of 32.
 *   q4_gemv_g32_workspace_bytes  -- workspace q4_gemv_g32 needs (host only).
 *   q4_gemv_g32                  -- q4_gemv on group-32 weights.
 *   q4_mmq_gemm_g32              -- q4_mmq_gemm on group-32 weights; each Q8_1
 *                                   block meets its own weight pair, so the
 *                                   scales apply per block:
 *       y[m][n] = sum_b ( scale[n][b] * d[m][b] * I[m][n][b]
 *                         + minimum[n][b] * d[m][b] * sum_{k in b} a[m][k] )
 *     (workspace: q4_mmq_workspace_bytes(M, N, K)).
 */
int q4_pack_g32(const float *W, int64_t N, int64_t K, uint8_t *qs, uint16_t *sm, void *stream);
size_t q4_gemv_g32_workspace_bytes(int64_t M, int64_t N, int64_t K);
int q4_gemv_g32(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm, int64_t N,
                int64_t K, float *y, void *workspace, size_t ws_bytes, void *stream);
int q4_mmq_gemm_g32(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                    const uint16_t *sm, int64_t N, int64_t K, float *y, void *workspace,
                    size_t ws_bytes, void *stream);

/*
 * q4_mmq_workspace_bytes -- device workspace q4_mmq_gemm (and
 * q4_mmq_gemm_q8_1, q4_mmq_gemm_g32) needs for this shape: the fp16
 * activation image of the fp16 path (2 * K bytes per activation row, rows
 * padded to whole tiles of 256 or 192, at most 256 MiB + 2 * K * 256
 * bytes, plus 4 bytes per row) and 8 bytes per
 * weight row (N rounded up to 128), or what the int8 path needs
 * (q4_mmq_int8_workspace_bytes).  Pure host function.  Returns 0
 * for shapes q4_mmq_gemm would reject.
 */
size_t q4_mmq_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * q4_mmq_gemm -- prefill GEMM on Q8_1 activations (the MMQ path of the hipfire
 * note: pre-quantized Q8_1 activations, LDS-staged tiles, matrix-core
 * products over output tiles):
 *     y[m][n] = sum_k (d[m][k/32] * a[m][k]) * (scale[n][k/256] * q[n][k] + minimum[n][k/256])
 * Two designs, chosen from the shape alone (so the workspace size, and the
 * result, depend only on the inputs):
 *   - fp16 matrix cores, for grids of 256 x 128 output tiles that keep every
 *     CU evenly busy (at least 128 tiles, and at most 256 or rounds of 256
 *     at least 80 % full; e.g. M = 2048 at N = 4096 or 12288, M = 512 at
 *     N = 9216), unless the int8 design's 128 x 128 tiles fill the CUs in
 *     one round (at most 256 tiles; e.g. M = 1024 at N = 4096), with
 *     192-row tiles where those fill the CUs better (e.g. M = 512 at
 *     N = 9216; the result is the same bit for bit): a prep pass
 *     writes each activation as fp16(d * a * 2^f[m]),
 *     one power of two per row so that the largest is below 2^15; the GEMM
 *     turns each weight into fp16((scale * q + minimum) * 2^e[n]) in one
 *     fused multiply-add, one power of two per weight row so that the
 *     largest is below 2^-6; it multiplies in fp16, sums in fp32 and scales
 *     y by 2^-(f[m] + e[n]).  Each operand is within 2^-11 relative of its
 *     exact value; weights below about 2^-7 and activations below about
 *     2^-28 of their row's largest are fp16 subnormals, exact to 2^-25
 *     absolute.  Measured
 *     NMSE ~8e-8, max|dy| / max|y| ~3e-4.
 *   - int8 matrix cores elsewhere, as q4_mmq_gemm_int8:
 *     per-block products sum_{k in block} a * (q - 8) are exact int32 (i8
 *     MFMA); the eight blocks of a weight group are combined
 *     in int32 with each row's block scales as 13-bit integers relative to
 *     the group's largest (D = rint(d / step), step = max d / 8191), then
 *     the group's scale, step and minimum term are applied in fp32.  So every
 *     activation may move by up to 1/16382 of the largest |x| in its group of
 *     256 on top of Q8_1's own rounding; measured NMSE ~3e-8 on N(0,1)
 *     activations with outliers up to 1000x.
 * Either way results match the fp64 definition to max|dy| / max|y| <= 2e-3
 * and NMSE <= 1e-6.  The s field of ds is not read.  Reruns are
 * bit-identical.
 *   qa: device i8 [M][K], 16-byte aligned.  ds: device u16 [M][K/32][2],
 *   4-byte aligned.  qs/sm as for q4_gemv.  y: device fp32 [M][N], 4-byte
 *   aligned.  workspace: at least q4_mmq_workspace_bytes(M, N, K) bytes,
 *   16-byte aligned (NULL allowed when that is 0); same rules as q4_gemv.
 * Errors: Q4_ERR_ARG, Q4_ERR_ALIGN, Q4_ERR_WORKSPACE, Q4_ERR_ARCH,
 * Q4_ERR_DEVICE, Q4_ERR_LAUNCH.
 */
int q4_mmq_gemm(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                const uint16_t *sm, int64_t N, int64_t K, float *y, void *workspace,
                size_t ws_bytes, void *stream);

/*
 * q4_mmq_gemm_int8 -- q4_mmq_gemm on int8 matrix cores at every shape: the
 * hipfire note's MMQ arithmetic as written ("list of changes": Q8_1
 * pre-quantized activations, LDS-staged tiles, i8 matrix products over
 * 128x128 output tiles).  Each 32-wide block product
 *     I[m][n][b] = sum_{k in block b} a[m][k] * (q[n][k] - 8)
 * is an exact int32 from one int8 MFMA; the eight blocks of a weight group
 * are combined in int32 with each row's block scales as 13-bit integers
 * relative to the group's largest (D = rint(d / step), step = max d / 8191),
 * and the group's scale, step and minimum term are applied in fp32:
 *     y[m][n] = sum_g ( scale * step * sum_b D * I + (minimum + 8 scale) * X[m][g] ),
 *     X[m][g] = sum_{b in g} d[m][b] * sum_{k in b} a[m][k].
 * Every activation may move by up to 1/16382 of the largest |x| in its group
 * of 256 on top of Q8_1's own rounding; results match the fp64 definition to
 * max|dy| / max|y| <= 2e-3 and NMSE <= 1e-6 (measured NMSE ~3e-8 on N(0,1)
 * activations with outliers up to 1000x).  Reruns are bit-identical.
 * Grids of at least 256 tiles of 128 x 128 (but not 257 to 511, which the
 * unpipelined kernel runs in one round) whose activations, packed weights
 * and records each stay below 2 GiB run a pipelined kernel whose prep
 * pass writes, per (activation row, group), the block scales D, step, X and
 * the centring term 8 * sum_b D * sum_{k in b} a, and per (weight row, group)
 * scale and minimum + 8 scale in fp32, into the workspace (32 bytes per
 * activation row and 8 bytes per weight row, per group, rows rounded up to
 * 128).  Other shapes run an unpipelined kernel over row ranges of less
 * than 2 GiB of each operand; small grids split K over workgroups into fp32
 * partials in the workspace, summed in split order by a second kernel (no
 * workspace when K is not split).
 *   Arguments, layouts and errors as q4_mmq_gemm; workspace: at least
 *   q4_mmq_int8_workspace_bytes(M, N, K) bytes (pure host function, 0 for
 *   shapes the call would reject).
 */
size_t q4_mmq_int8_workspace_bytes(int64_t M, int64_t N, int64_t K);
int q4_mmq_gemm_int8(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                     const uint16_t *sm, int64_t N, int64_t K, float *y, void *workspace,
                     size_t ws_bytes, void *stream);

/*
 * q4_mmq_gemm_q8_1 -- q4_mmq_gemm whose epilogue hands its result on as Q8_1
 * activations for a following MMQ layer instead of writing fp32: the
 * quantization step that the hipfire MMQ note runs ahead of the prefill GEMM
 * ("list of changes": activations pre-quantized to Q8_1 in MMQ layout), moved
 * into the producing GEMM.  The output is exactly
 *     q8_1_quantize(q4_mmq_gemm(qa, ds, qs, sm))
 * bit for bit: the same fp32 y, quantized along n in blocks of 32 with the
 * same decisions (d = fp16(amax/127), a = clamp(rint(y/d), -127, 127),
 * s = fp16(d * sum a)).  N must be a multiple of 32.
 *   qa, ds, qs, sm: as for q4_mmq_gemm.  qa_out: device i8 [M][N], 4-byte
 *   aligned.  ds_out: device u16 [M][N/32][2] = (d, s), 4-byte aligned.
 *   workspace: at least q4_mmq_workspace_bytes(M, N, K) bytes (used as by
 *   q4_mmq_gemm, which takes the same design for the shape), 16-byte
 *   aligned, NULL allowed when 0.
 * Errors: Q4_ERR_ARG (also N not a multiple of 32), Q4_ERR_ALIGN,
 * Q4_ERR_WORKSPACE, Q4_ERR_ARCH, Q4_ERR_DEVICE, Q4_ERR_LAUNCH.
 */
int q4_mmq_gemm_q8_1(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                     const uint16_t *sm, int64_t N, int64_t K, int8_t *qa_out, uint16_t *ds_out,
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * q4_mmq_block_dots -- the integer core of q4_mmq_gemm on its own, for
 * checking it bit-exactly (the "keep-quant integer core" the vllm.cpp TG150
 * campaign keeps bit-exact against the CPU, pull request 4, "Design"):
 *     idot[m][n][b] = sum_{k = 32b}^{32b+31} a[m][k] * q[n][k]      (exact int32)
 * It runs the same i8 MFMA tile code as q4_mmq_gemm's int8 design with an
 * epilogue that stores the per-block sums instead of scaling them.
 *   qa: device i8 [M][K], 16-byte aligned.  qs: device u8 [N][K/2], 16-byte
 *   aligned.  idot: device i32 [M][N][K/32], 4-byte aligned (M*N*K/32 entries
 *   must not exceed 2^31).
 * Errors: Q4_ERR_ARG, Q4_ERR_ALIGN, Q4_ERR_ARCH, Q4_ERR_DEVICE, Q4_ERR_LAUNCH.
 */
int q4_mmq_block_dots(const int8_t *qa, int64_t M, const uint8_t *qs, int64_t N, int64_t K,
                      int32_t *idot, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4MI_H */
