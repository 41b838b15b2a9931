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
// operand row (l % 16) and the eight K-values 8*(l/16) .. 8*(l/16)+7 of a
// 32-deep step; the output lane l holds column (l % 16), rows 4*(l/16)..+3.
// The K reduction does not care which real k each (lane, slot) carries, as
// long as both operands agree, so within a 128-wide K chunk lane (j = l/16,
// r = l%16) carries k = 32*j + 8*i + e for MFMA step i = 0..3, slot e = 0..7:
// 32 consecutive k of one row, i.e. 16 consecutive source bytes.
//
//   N is padded to Np = roundup(N, 16) (zero codes), K to Kp = roundup(K, 512)
//   (zero codes, zero scales).  Tile t = n / 16, row r = n % 16.
//
//   Codes (wq), one 1 KiB block per (tile t, chunk b = k / 128):
//     block (t, b) at byte ((t * KB + b) * 64 + lane) * 16,  KB = Kp / 128,
//     lane = 16 * j + r with j = (k % 128) / 32; the 16 bytes of a lane are
//     the source bytes of row n covering k in [128 b + 32 j, +32), in source
//     order (low nibble = even k).  Dword i of a lane is MFMA step i.
//
//   Scales (sq), one block per (tile t, scale block sb = k / 512), SB = Kp / 512:
//     NVFP4 (G = 16): 8 bytes per lane at ((t * SB + sb) * 64 + lane) * 8;
//       byte 2c + h is the scale of row n, group (512 sb + 128 c + 32 j)/16 + h,
//       i.e. chunk c = 0..3 of the block, half h = 0/1 of the lane's 32 k
//       (h selects dwords 0-1 vs 2-3).
//     MXFP4 (G = 32): 4 bytes per lane at ((t * SB + sb) * 64 + lane) * 4;
//       byte c is the scale of row n, group (512 sb + 128 c + 32 j) / 32.
//   A lane thus reads all its scales for 512 K with one 8- or 4-byte load and
//   no scale byte is stored twice.
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
// scale bytes per lane per scale block
inline int scale_lane_bytes(int fmt) { return fmt == 0 ? 8 : 4; }

// Byte offset in wq of the byte holding element (n, k) (k even/odd share it).
inline int64_t wq_offset(int64_t n, int64_t k, int64_t KB) {
    int64_t t = n / kTileN, r = n % kTileN;
    int64_t b = k / kChunkK, j = (k % kChunkK) / 32;
    int64_t lane = 16 * j + r;
    return ((t * KB + b) * kLanes + lane) * 16 + (k % 32) / 2;
}

// Byte offset in sq of the scale of element (n, k).
inline int64_t sq_offset(int64_t n, int64_t k, int64_t SB, int fmt) {
    int64_t t = n / kTileN, r = n % kTileN;
    int64_t sb = k / kScaleBlockK, c = (k % kScaleBlockK) / kChunkK, j = (k % kChunkK) / 32;
    int64_t lane = 16 * j + r;
    if (fmt == 0) {
        int64_t h = (k % 32) / 16;
        return ((t * SB + sb) * kLanes + lane) * 8 + 2 * c + h;
    }
    return ((t * SB + sb) * kLanes + lane) * 4 + c;
}

}  // namespace fp4
