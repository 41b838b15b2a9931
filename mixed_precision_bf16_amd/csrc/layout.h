// Packed weight layout shared by the offline repack (host) and the kernels.
//
// Why a repack at all: a wavefront load wants one contiguous block (1 KiB for
// 64 lanes x 16 bytes) while the matrix core wants each lane to hold a
// fragment of a 16-row tile.  The Petit blog ("Optimizing FP4 Mixed-Precision
// Inference on AMD GPUs", section "Efficient dequantization through
// preprocessing") resolves this by arranging the weights offline; this file
// is the gfx950 arrangement used here.
//
// gfx950 MFMA v_mfma_f32_16x16x32_bf16 (checked on the device): lane l holds
// operand row (l % 16) and eight K-values in slots 8*(l/16) .. 8*(l/16)+7 of
// a 32-deep step; the output lane l holds column (l % 16), rows 4*(l/16)..+3.
// The K reduction does not care which real k each (lane, slot) carries, as
// long as both operands agree.  Within a 128-wide K chunk, lane (j = l/16,
// r = l%16) carries k = 32*i + 8*j + e in MFMA step i = 0..3, slot e = 0..7.
// For a fixed step the four lanes j = 0..3 of a row then cover 32 consecutive
// k, so an activation fragment load touches 64 contiguous bytes per row.
//
//   N is padded to Np = roundup(N, 16) (zero codes), K to Kp = roundup(K, 512)
//   (zero codes, zero scales).  Tile t = n / 16, row r = n % 16.
//
//   Codes (wq), one 1 KiB block per (tile t, chunk b = k / 128), KB = Kp / 128:
//     lane (j, r) = 16 j + r owns 16 bytes at ((t * KB + b) * 64 + lane) * 16;
//     its dword i holds the 8 codes of row n for k in [128 b + 32 i + 8 j, +8)
//     (4 source bytes, low nibble = even k).  The repack is a permutation of
//     source dwords.
//
//   Scales (sq), one block per (tile t, scale block sb = k / 512), SB = Kp / 512:
//     NVFP4 (G = 16): 512 bytes as two halves h = 0, 1 of 256 bytes; row r
//       owns 16 bytes at h * 256 + r * 16; byte 4 c + i of them is the scale
//       of group 32 sb + 8 c + 2 i + h (chunk c = 0..3 of the block, step i).
//       Lane (j, r) loads half h = j / 2: the scales of all 16 dwords it
//       multiplies in the block, with one 16-byte load; the 16 lanes of one j
//       read 256 contiguous bytes.
//     MXFP4 (G = 32): 256 bytes; row r owns 16 bytes at r * 16; byte 4 c + i
//       is the scale of group 16 sb + 4 c + i.  All four lanes j of a row
//       load the same 16 bytes.
//   No scale byte is stored twice.
#pragma once

#include <stdint.h>

namespace fp4 {

constexpr int kTileN = 16;        // rows per n-tile
constexpr int kChunkK = 128;      // K per 1 KiB code block
constexpr int kScaleBlockK = 512; // K per scale block
constexpr int kLanes = 64;

inline int group_of(int fmt) { return fmt == 0 ? 16 : 32; }
inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
inline int64_t padded_n(int64_t N) { return round_up(N, kTileN); }
inline int64_t padded_k(int64_t K) { return round_up(K, kScaleBlockK); }
// packed scale bytes per (tile, scale block)
inline int scale_block_bytes(int fmt) { return fmt == 0 ? 512 : 256; }

// Byte offset in wq of the byte holding element (n, k) (k even/odd share it).
inline int64_t wq_offset(int64_t n, int64_t k, int64_t KB) {
    const int64_t t = n / kTileN, r = n % kTileN;
    const int64_t b = k / kChunkK, kk = k % kChunkK;
    const int64_t i = kk / 32, j = (kk % 32) / 8;
    const int64_t lane = 16 * j + r;
    return ((t * KB + b) * kLanes + lane) * 16 + 4 * i + (k % 8) / 2;
}

// Byte offset in sq of the scale of element (n, k).
inline int64_t sq_offset(int64_t n, int64_t k, int64_t SB, int fmt) {
    const int64_t t = n / kTileN, r = n % kTileN;
    const int64_t sb = k / kScaleBlockK, c = (k % kScaleBlockK) / kChunkK, i = (k % kChunkK) / 32;
    if (fmt == 0) {
        const int64_t h = (k % 32) / 16;
        return (t * SB + sb) * 512 + h * 256 + r * 16 + 4 * c + i;
    }
    return (t * SB + sb) * 256 + r * 16 + 4 * c + i;
}

}  // namespace fp4
