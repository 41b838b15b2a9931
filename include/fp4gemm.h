/*
 * fp4gemm.h -- C ABI of the BF16 / FP16 x FP4 block-scaled GEMM for AMD MI355X (gfx950),
 * with its grouped mixture-of-experts variant, the offline repack and the
 * offline quantizer.
 *
 *   Y[m][N] = A[m][K] . dequant(W)[N][K]^T,   dequant(W)[n][k] = e2m1(code[n][k]) * scale[n][k / G]
 *
 * A and Y are BF16 (fp4_gemm) or FP16 (fp4_gemm_f16), accumulation is FP32.  W is stored as FP4 E2M1 codes with
 * one scale per G consecutive K-elements of a row:
 *   NVFP4: G = 16, scale = FP8 E4M3 (OCP "E4M3FN")  -- Petit blog ("Optimizing
 *          FP4 Mixed-Precision Inference on AMD GPUs"), section "Detailed
 *          performance analysis": 16 elements share one FP8 scale.
 *   MXFP4: G = 32, scale = E8M0 (2^(byte - 127))     -- petit-kernel PyPI page,
 *          "Features": dense GEMM with MXFP4 weights (OCP MX definition).
 * E2M1 (1 sign, 2 exponent, 1 mantissa bit; values +-{0, .5, 1, 1.5, 2, 3, 4, 6})
 * follows the mhpq.cn FP4 GEMM article, section 2.1.
 *
 * Canonical (source) weight layout, as produced by a quantizer:
 *   codes  uint8 [N][K/2]  byte j of row n: element k = 2j in bits 3..0,
 *                          element k = 2j+1 in bits 7..4
 *   scales uint8 [N][K/G]  byte g of row n scales elements [g*G, (g+1)*G)
 * The GEMM consumes the "packed" layout written by fp4_repack: the same bytes
 * permuted into the order in which the gfx950 matrix-core fragments consume
 * them, so that each wavefront load is one contiguous 1 KiB block (the
 * offline weight shuffle of the Petit blog, section "Efficient dequantization
 * through preprocessing", and of the petit-kernel page, "Techniques and
 * performance").  The packed layout pads N to a multiple of 16 and K to a
 * multiple of 512 with zero bytes; it is an internal format, described in
 * the library sources, and may change between versions: persist the
 * canonical layout (fp4_unpack restores it exactly).
 *
 * Conventions for every call:
 *   - All sizes are element counts unless named *_bytes.  Return value is an
 *     fp4_status; no call aborts, throws or prints.
 *   - Every argument check happens before any HIP call.  A failed check
 *     leaves every output untouched.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronizes in any device entry (fp4_gemm*, fp4_moe_gemm,
 *     fp4_quantize, fp4_dequant*): they only queue kernels on `stream`.
 *   - "device" pointers must be HIP device memory on the current device;
 *     "host" pointers must be ordinary host memory.
 *   - Functions are reentrant and thread-safe; the only global state is a
 *     per-device "is gfx950" cache, an atomic launch counter that tags the
 *     split-K arrival words, a 64-entry cache of the kernel shape chosen per
 *     (m, N, K, format) (behind a mutex), and the tuning overrides
 *     FP4GEMM_DECODE / FP4GEMM_PREFILL, read from the environment once per
 *     process.
 */
#ifndef FP4GEMM_H
#define FP4GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats. */
enum {
    FP4_NVFP4 = 0, /* G = 16, E4M3 scales */
    FP4_MXFP4 = 1  /* G = 32, E8M0 scales */
};

/* Status codes. */
enum {
    FP4_OK = 0,
    FP4_ERR_NULL = 1,      /* a required pointer is NULL */
    FP4_ERR_SHAPE = 2,     /* N < 1, K < G, K % G != 0, m < 0, a size over the limits below,
                              or a device pointer not aligned as its entry requires */
    FP4_ERR_FORMAT = 3,    /* format is neither FP4_NVFP4 nor FP4_MXFP4 (or, fp4_gemm_ex, an
                              activation type other than 0 / 1) */
    FP4_ERR_VALUE = 4,     /* fp4_repack: a scale byte is negative or NaN; fp4_gemm_ex /
                              fp4_quantize: alpha outside its documented range */
    FP4_ERR_WORKSPACE = 5, /* workspace smaller than fp4_gemm_workspace_size */
    FP4_ERR_DEVICE = 6,    /* no current HIP device, or it is not gfx950 */
    FP4_ERR_HIP = 7        /* a HIP runtime call or kernel launch failed */
};

/* Size limits (checked; FP4_ERR_SHAPE beyond them):
 *   K <= 2^20, N <= 2^24, m <= 2^20, and m*K*2 and m*N*2 (bytes of A and Y,
 *   after m is rounded up to the kernel's row block) below 2^31, because the
 *   kernels address A and Y through 32-bit ranged buffer offsets. */

/* Human-readable name of a status code (static string, never NULL). */
const char* fp4_status_string(int status);

/* Bytes of the packed code and scale arrays for an N x K weight.
 * wq_bytes = Np*Kp/2 and sq_bytes = Np*Kp/G with Np = roundup(N, 16),
 * Kp = roundup(K, 512).  Either output pointer may be NULL. */
int fp4_repack_size(int64_t N, int64_t K, int format, size_t* wq_bytes, size_t* sq_bytes);

/* Offline, host to host: permute canonical codes [N][K/2] and scales [N][K/G]
 * into the packed layout wq / sq (sizes from fp4_repack_size; every byte of
 * both outputs is written, padding with zeros).  Pure integer permutation:
 * no value changes.  Scale bytes must be non-negative and not NaN (the
 * petit-kernel page, "Known limitations", assumes positive scales):
 * NVFP4 rejects bytes with bit 7 set and 0x7F; MXFP4 rejects 0xFF; zero
 * scales are accepted.  All 16 code values are accepted (a negative-zero code
 * dequantizes to -0.0).  On FP4_ERR_VALUE nothing is written.
 * MXFP4 scale bytes outside 2..252 (exponent outside -125..125) are accepted
 * but give BF16 results that overflow or fall below the normal range. */
int fp4_repack(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, int format,
               uint8_t* wq, uint8_t* sq);

/* Exact inverse of fp4_repack (host to host): writes codes [N][K/2] and
 * scales [N][K/G].  unpack(repack(x)) == x byte for byte. */
int fp4_unpack(const uint8_t* wq, const uint8_t* sq, int64_t N, int64_t K, int format,
               uint8_t* codes, uint8_t* scales);

/* Workspace bytes fp4_gemm needs for this problem (a pure function of its
 * arguments; no device is queried).  The library may split K over S
 * workgroups (split-K; not described on the pages: a narrow layer at the
 * decode batch m = 16 has too few 16-row output tiles to give each of the
 * 256 compute units its own): each writes FP32
 * partial sums of its K range, which are added in a fixed order s = 0, 1, ...
 * With the decode kernels (m <= 64, except 33 <= m <= 64 on layers whose
 * decode grid would fill the GPU poorly or whose K exceeds 16384) the last
 * workgroup of each output group adds them (it finds out through an 8-byte
 * arrival word per group, after the partials); with the prefill kernel a
 * second kernel does.  The size is about S * m * N * 4 bytes, or 0 when no
 * split is chosen.  The contents need no initialization (the arrival words
 * carry a tag unique to each launch, and the last workgroup of a group
 * leaves its word at zero, so a call captured in a HIP graph can be
 * replayed with its workspace) and are not preserved between calls. */
int fp4_gemm_workspace_size(int64_t m, int64_t N, int64_t K, int format, size_t* bytes);

/* Y = A . dequant(W)^T on `stream` (a hipStream_t; NULL = default stream).
 *   A   device, BF16 [m][K] row-major, contiguous
 *   wq  device, packed codes from fp4_repack (uploaded by the caller)
 *   sq  device, packed scales from fp4_repack
 *   C   device, BF16 [m][N] row-major, contiguous; every element is written
 *   workspace / workspace_bytes: device scratch, 16-byte aligned, of at
 *       least fp4_gemm_workspace_size bytes (may be NULL when that size is
 *       0); FP4_ERR_WORKSPACE otherwise.  Calls that may run concurrently
 *       (different streams) need separate workspaces.
 * A, wq, sq and C must be 16-byte aligned (the kernels use 16-byte vector
 * loads and 8-byte stores).
 * m == 0 is a no-op returning FP4_OK.  Asynchronous: returns once the kernels
 * are queued; faults surface at the caller's next synchronization.
 * Accumulation is FP32; the output is rounded to BF16 to nearest even.
 * Results are deterministic: the same inputs give the same bits on every
 * call (fixed summation order; the only atomics count split-K arrivals). */
int fp4_gemm(const void* A, const void* wq, const void* sq, void* C,
             int64_t m, int64_t N, int64_t K, int format,
             void* workspace, size_t workspace_bytes, void* stream);

/* fp4_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and results (bit for bit) as fp4_gemm, without
 * workspace arguments.  The split-K scratch (fp4_gemm_workspace_size bytes)
 * lives in a 64 MiB device array of the library instead, one per GPU the
 * library runs on, held until the process ends; problems whose workspace
 * size exceeds fp4_gemm_noalloc_max_workspace() return FP4_ERR_WORKSPACE
 * (checked before any HIP call).  The call allocates and frees nothing.
 * All calls on one GPU share its array: calls that overlap in time on one
 * GPU (several streams or threads at once) race and give wrong results;
 * serialize them.  The array keeps the last call's contents; nothing in it
 * needs clearing between calls (the split-K arrival words carry launch tags
 * and are left at zero).  The first call on each device looks the array's
 * address up (hipGetSymbolAddress); make that first call outside a graph
 * capture.  Other arguments, errors and determinism as fp4_gemm. */
int fp4_gemm_noalloc(const void* A, const void* wq, const void* sq, void* C,
                     int64_t m, int64_t N, int64_t K, int format, void* stream);

/* Size in bytes of fp4_gemm_noalloc's per-GPU scratch array (64 MiB). */
size_t fp4_gemm_noalloc_max_workspace(void);

/* Same as fp4_gemm with FP16 activations and output: A device FP16 [m][K],
 * C device FP16 [m][N] (the Petit blog, "Introduction": FP16/BF16 x FP4
 * kernels).  The weights use the same packed layout; they are dequantized
 * to FP16 (exact for every NVFP4 code x scale product, and for MXFP4 scale
 * exponents -23 .. 13; outside that range products round or overflow in
 * FP16).  Accumulation FP32, output rounded to FP16 to nearest even.
 * Workspace, alignment, errors and determinism as for fp4_gemm (the
 * workspace size is the same). */
int fp4_gemm_f16(const void* A, const void* wq, const void* sq, void* C,
                 int64_t m, int64_t N, int64_t K, int format,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Debug/test entry: write dequant(W) as BF16 [N][K] row-major to device
 * memory W_bf16 with the same device dequantization the GEMM uses (the
 * per-block debug dump suggested by the mhpq.cn article, section 7).
 * Every code x scale product is exact in BF16 for valid scales. */
int fp4_dequant(const void* wq, const void* sq, void* W_bf16, int64_t N, int64_t K, int format,
                void* stream);

/* As fp4_dequant, writing FP16 [N][K] with the dequantization fp4_gemm_f16
 * uses. */
int fp4_dequant_f16(const void* wq, const void* sq, void* W_f16, int64_t N, int64_t K, int format,
                    void* stream);

/* fp4_gemm / fp4_gemm_f16 with a per-tensor output scale:
 *     C = alpha * (A . dequant(W)^T)
 * act_type 0: BF16 A and C (as fp4_gemm), 1: FP16 (as fp4_gemm_f16).  alpha
 * is the second-level FP32 scale of a two-level NVFP4 checkpoint (not on the
 * pages; the offline quantizer below takes the same alpha), applied to the
 * FP32 accumulator before rounding.  alpha must be finite with |alpha| in
 * [2^-100, 2^100], else FP4_ERR_VALUE; alpha = 1 gives bit-identical results
 * to fp4_gemm / fp4_gemm_f16.  act_type outside {0, 1} is FP4_ERR_FORMAT.
 * Everything else (workspace, alignment, errors, determinism) as fp4_gemm. */
int fp4_gemm_ex(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N, int64_t K,
                int format, int act_type, float alpha, void* workspace, size_t workspace_bytes, void* stream);

/* Offline quantizer on the device: BF16 weights -> FP4 codes and block scales
 * in the source order fp4_repack takes (mhpq.cn FP4 GEMM article: block
 * scaling with the block maximum, section 2.2; nearest grid point, section
 * 2.1; no zero scale for an all-zero block, section 5.2).
 *   W       device, BF16 [N][K] row-major, 16-byte aligned
 *   codes   device, uint8 [N][K/2] (element 2j in the low nibble), aligned
 *           to G/2 bytes
 *   scales  device, uint8 [N][K/G]
 * Per block of G elements, in IEEE FP32 (correctly rounded operations):
 *   NVFP4: scale = E4M3 round-to-nearest-even of (amax / 6) / alpha,
 *          saturated at 448 and at least 2^-9 (never zero);
 *   MXFP4: scale byte = clamp(floor(log2(amax / alpha)) - 2 + 127, 0, 254)
 *          (the OCP MX rule); byte 0 is the scale 2^-127 (any amax / alpha
 *          below 2^-124) and its block is rounded like every other;
 *   code = nearest E2M1 value to |x| / (alpha * scale), ties to the even
 *   mantissa bit, saturating at +-6; no negative zero; NaN -> 0, +-Inf ->
 *   +-6 with the largest scale.
 * alpha > 0, finite, in [2^-100, 2^100] (else FP4_ERR_VALUE); quantizing with
 * alpha and multiplying by it with fp4_gemm_ex reproduces the tensor's scale.
 * N, K in 1 .. 2^24 with K % G == 0 (else FP4_ERR_SHAPE).  Asynchronous on
 * `stream`. */
int fp4_quantize(const void* W, void* codes, void* scales, int64_t N, int64_t K, int format, float alpha,
                 void* stream);

/* ---- Native FP4 path (FP4 x FP4 on the gfx950 matrix cores) ----------------
 * The Petit blog's introduction: MI350 multiplies FP4 natively.  Unlike the
 * entries above, this path quantizes the activations: each 32-element K block
 * of every row of A becomes MXFP4 by the fp4_quantize rule (alpha 1), and the
 * product of the two MXFP4 operands is accumulated in FP32:
 *     C = alpha * (dequant(quantize(A)) . dequant(W)^T)
 * MXFP4 weights only (the matrix core's block scale is E8M0 per 32), in their
 * own packed layout (fp4_native_repack). */

/* Bytes of the native packed codes and scales (the MXFP4 sizes of
 * fp4_repack_size). */
int fp4_native_repack_size(int64_t N, int64_t K, size_t* wq_bytes, size_t* sq_bytes);

/* Offline, host to host: canonical MXFP4 codes [N][K/2] and scales [N][K/32]
 * -> the native packed layout (a pure permutation plus zero padding; scale
 * byte 0xFF rejected with FP4_ERR_VALUE, nothing written then). */
int fp4_native_repack(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, uint8_t* wq,
                      uint8_t* sq);

/* Exact inverse of fp4_native_repack (host to host). */
int fp4_native_unpack(const uint8_t* wq, const uint8_t* sq, int64_t N, int64_t K, uint8_t* codes,
                      uint8_t* scales);

/* Workspace of fp4_gemm_native: the quantized activations (m x Kp/2 code
 * bytes and m x Kp/32 scale bytes, Kp = K rounded up to 512) plus FP32
 * partials when K is split; 0 for m == 0. */
int fp4_gemm_native_workspace_size(int64_t m, int64_t N, int64_t K, size_t* bytes);

/* C = alpha * (dequant(quantize(A)) . dequant(W)^T) on `stream`:
 *   A  device BF16 [m][K]; wq / sq from fp4_native_repack (device);
 *   C  device BF16 [m][N], every element written; alpha as fp4_gemm_ex;
 *   workspace: device, 256-byte aligned, at least
 *   fp4_gemm_native_workspace_size bytes (FP4_ERR_WORKSPACE otherwise);
 *   its contents are scratch.  A, wq, sq and C 16-byte aligned.
 * K % 32 == 0, m <= 2^20, m * Kp / 2 and m * N * 2 below 2^31 (else
 * FP4_ERR_SHAPE).  Two kernels (activation quantizer, FP4 GEMM; a third sums
 * the K-split partials); deterministic. */
int fp4_gemm_native(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N, int64_t K,
                    float alpha, void* workspace, size_t workspace_bytes, void* stream);

/* Grouped mixture-of-experts GEMM with BF16 activations (the petit-kernel
 * page, "Features": fused MoE kernels for BF16 and MXFP4 workloads; both FP4
 * formats are accepted).  For expert e = 0 .. E-1 and every assignment id
 * in sorted_ids[expert_offsets[e] .. expert_offsets[e+1]):
 *     C[id][:] = w(id) * A[id / a_div] . dequant(W_e)^T
 * with w(id) = topk_weights[id] (FP32, multiplied before rounding) or 1 when
 * topk_weights is NULL.  a_div is the number of experts per token when A
 * holds one row per token (gate/up projection), 1 when A holds one row per
 * assignment (down projection).
 *   A              device, BF16 [a_rows][K] row-major
 *   wq, sq         device, E experts' packed weights back to back, each
 *                  exactly the fp4_repack_size(N, K, format) bytes of one
 *                  N x K matrix (expert e at e * wq_bytes / e * sq_bytes)
 *   sorted_ids     device, int32 [P], assignment ids grouped by expert; each
 *                  id at most once (a repeated id is a write race)
 *   expert_offsets device, int32 [E + 1], non-decreasing, from 0 to P
 *                  (values are clamped to [0, P])
 *   topk_weights   device, FP32 [out_rows] indexed by id, or NULL
 *   C              device, BF16 [out_rows][N]; only the rows listed in
 *                  sorted_ids are written; ids outside [0, out_rows) are
 *                  skipped, rows id / a_div >= a_rows read as zeros
 * A, wq, sq and C 16-byte aligned, the int32 / FP32 arrays 4-byte aligned.
 * P == 0 is a no-op.  No workspace (no K split).  Asynchronous on `stream`;
 * deterministic.  Errors as for fp4_gemm; FP4_ERR_SHAPE also for E outside
 * 1 .. 4096, P > 2^24, a_div < 1, out_rows * N * 2 bytes of C at or above
 * 2^31, or a grid that would need more than 65535 row blocks (P / 16 + E). */
int fp4_moe_gemm(const void* A, const void* wq, const void* sq, const int32_t* sorted_ids,
                 const int32_t* expert_offsets, const float* topk_weights, void* C, int64_t a_rows, int64_t a_div,
                 int64_t out_rows, int64_t P, int64_t E, int64_t N, int64_t K, int format, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4GEMM_H */
