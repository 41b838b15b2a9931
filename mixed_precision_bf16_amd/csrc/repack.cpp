// Offline weight repack / unpack and the host-only parts of the C ABI.
//
// The repack is the offline weight arrangement of the Petit blog ("Optimizing
// FP4 Mixed-Precision Inference on AMD GPUs", section "Efficient
// dequantization through preprocessing") and of the petit-kernel PyPI page
// ("Techniques and performance": weights are shuffled offline).  Here it is a
// pure permutation of 4-byte words (plus zero padding) into the layout of layout.h, so it
// is exactly invertible and never changes a value.
#include <string.h>

#include "../../include/fp4gemm.h"
#include "layout.h"

using namespace fp4;

extern "C" const char* fp4_status_string(int status) {
    switch (status) {
        case FP4_OK: return "ok";
        case FP4_ERR_NULL: return "null pointer argument";
        case FP4_ERR_SHAPE: return "invalid shape (need N >= 1, K >= G, K % G == 0, m >= 0, within size limits)";
        case FP4_ERR_FORMAT: return "unknown FP4 format (expected FP4_NVFP4 or FP4_MXFP4)";
        case FP4_ERR_VALUE: return "invalid scale byte (negative or NaN)";
        case FP4_ERR_WORKSPACE: return "workspace too small";
        case FP4_ERR_DEVICE: return "no gfx950 HIP device is current";
        case FP4_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

// Shared by the host and the device entry points (fp4gemm.hip declares it).
int fp4_check_weight_shape(int64_t N, int64_t K, int format) {
    if (format != FP4_NVFP4 && format != FP4_MXFP4) return FP4_ERR_FORMAT;
    const int64_t G = group_of(format);
    if (N < 1 || N > (int64_t(1) << 24)) return FP4_ERR_SHAPE;
    if (K < G || K % G != 0 || K > (int64_t(1) << 20)) return FP4_ERR_SHAPE;
    return FP4_OK;
}

extern "C" int fp4_repack_size(int64_t N, int64_t K, int format, size_t* wq_bytes, size_t* sq_bytes) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    const int64_t Np = padded_n(N), Kp = padded_k(K);
    if (wq_bytes) *wq_bytes = size_t(Np * Kp / 2);
    if (sq_bytes) *sq_bytes = size_t(Np * Kp / group_of(format));
    return FP4_OK;
}

static bool scale_byte_ok(uint8_t b, int format) {
    if (format == FP4_NVFP4) return (b & 0x80) == 0 && b != 0x7F;  // sign clear, not NaN
    return b != 0xFF;                                              // E8M0 NaN
}

extern "C" int fp4_repack(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, int format,
                          uint8_t* wq, uint8_t* sq) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (!codes || !scales || !wq || !sq) return FP4_ERR_NULL;
    const int64_t G = group_of(format);
    const int64_t ng = K / G;
    for (int64_t i = 0; i < N * ng; ++i)
        if (!scale_byte_ok(scales[i], format)) return FP4_ERR_VALUE;

    const int64_t Np = padded_n(N), Kp = padded_k(K);
    const int64_t KB = Kp / kChunkK, SB = Kp / kScaleBlockK;
    memset(wq, 0, size_t(Np * Kp / 2));
    memset(sq, 0, size_t(Np * Kp / G));
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t* row = codes + n * (K / 2);
        // one packed dword holds 8 consecutive k of the row
        for (int64_t k = 0; k < K; k += 8) memcpy(wq + wq_offset(n, k, KB), row + k / 2, 4);
        const uint8_t* srow = scales + n * ng;
        for (int64_t g = 0; g < ng; ++g) sq[sq_offset(n, g * G, SB, format)] = srow[g];
    }
    return FP4_OK;
}

extern "C" int fp4_unpack(const uint8_t* wq, const uint8_t* sq, int64_t N, int64_t K, int format,
                          uint8_t* codes, uint8_t* scales) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (!codes || !scales || !wq || !sq) return FP4_ERR_NULL;
    const int64_t G = group_of(format);
    const int64_t ng = K / G;
    const int64_t Kp = padded_k(K);
    const int64_t KB = Kp / kChunkK, SB = Kp / kScaleBlockK;
    for (int64_t n = 0; n < N; ++n) {
        uint8_t* row = codes + n * (K / 2);
        for (int64_t k = 0; k < K; k += 8) memcpy(row + k / 2, wq + wq_offset(n, k, KB), 4);
        uint8_t* srow = scales + n * ng;
        for (int64_t g = 0; g < ng; ++g) srow[g] = sq[sq_offset(n, g * G, SB, format)];
    }
    return FP4_OK;
}

// ------------------------------------------------------------ native layout
// Layout of MXFP4 weights for the FP4 matrix-core path (fp4_gemm_native).
// The gfx950 scaled 16x16x128 FP4 MFMA gives lane l = 16 j + r of a wave
// row r of its operand and 32 consecutive k (128-k step, k = 32 j .. 32 j +
// 31), two codes per byte with the even element in the low nibble, and one
// E8M0 scale per lane (checked on the device).  So the canonical row bytes
// are kept, only moved: per (16-row tile t, 128-k chunk c) one 1 KiB block
// whose 16-byte lane slot l holds row 16 t + r, canonical bytes
// [64 c + 16 j, 64 c + 16 j + 16); per (tile t, 512-k group q) one 256-byte
// block whose lane dword l holds, in byte s, the scale of row 16 t + r, block
// 16 q + 4 s + j (the lane's scale for chunk 4 q + s).  N is padded to 16 and
// K to 512 with zero bytes.
static int native_shape(int64_t N, int64_t K) { return fp4_check_weight_shape(N, K, FP4_MXFP4); }

static inline int64_t native_code_offset(int64_t n, int64_t k, int64_t KB) {  // k a multiple of 32
    const int64_t t = n / kTileN, r = n % kTileN, c = k / kChunkK, j = (k % kChunkK) / 32;
    return (t * KB + c) * 1024 + (16 * j + r) * 16;
}
static inline int64_t native_scale_offset(int64_t n, int64_t blk, int64_t QB) {  // blk = k / 32
    const int64_t t = n / kTileN, r = n % kTileN, q = blk / 16, s = (blk % 16) / 4, j = blk % 4;
    return (t * QB + q) * 256 + (16 * j + r) * 4 + s;
}

extern "C" int fp4_native_repack_size(int64_t N, int64_t K, size_t* wq_bytes, size_t* sq_bytes) {
    return fp4_repack_size(N, K, FP4_MXFP4, wq_bytes, sq_bytes);
}

extern "C" int fp4_native_repack(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, uint8_t* wq,
                                 uint8_t* sq) {
    int st = native_shape(N, K);
    if (st != FP4_OK) return st;
    if (!codes || !scales || !wq || !sq) return FP4_ERR_NULL;
    const int64_t ng = K / 32;
    for (int64_t i = 0; i < N * ng; ++i)
        if (!scale_byte_ok(scales[i], FP4_MXFP4)) return FP4_ERR_VALUE;
    const int64_t Np = padded_n(N), Kp = padded_k(K);
    const int64_t KB = Kp / kChunkK, QB = Kp / kScaleBlockK;
    memset(wq, 0, size_t(Np * Kp / 2));
    memset(sq, 0, size_t(Np * Kp / 32));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; k += 32) memcpy(wq + native_code_offset(n, k, KB), codes + n * (K / 2) + k / 2, 16);
        for (int64_t b = 0; b < ng; ++b) sq[native_scale_offset(n, b, QB)] = scales[n * ng + b];
    }
    return FP4_OK;
}

extern "C" int fp4_native_unpack(const uint8_t* wq, const uint8_t* sq, int64_t N, int64_t K, uint8_t* codes,
                                 uint8_t* scales) {
    int st = native_shape(N, K);
    if (st != FP4_OK) return st;
    if (!codes || !scales || !wq || !sq) return FP4_ERR_NULL;
    const int64_t ng = K / 32;
    const int64_t Kp = padded_k(K);
    const int64_t KB = Kp / kChunkK, QB = Kp / kScaleBlockK;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; k += 32) memcpy(codes + n * (K / 2) + k / 2, wq + native_code_offset(n, k, KB), 16);
        for (int64_t b = 0; b < ng; ++b) scales[n * ng + b] = sq[native_scale_offset(n, b, QB)];
    }
    return FP4_OK;
}
