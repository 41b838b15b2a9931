// BF16 x FP4 (NVFP4 / MXFP4) GEMM kernels for gfx950 and the device-side C ABI.
//
//   Y[m][N] = A[m][K] . dequant(W)[N][K]^T, FP32 accumulation, BF16 output.
//
// Design (MI355X-first; the Petit blog "Optimizing FP4 Mixed-Precision
// Inference on AMD GPUs" is prior art written for MI300):
//  * Weights stay FP4 in HBM and are dequantized in registers to BF16 right
//    before the BF16 matrix-core instruction (the blog's section "Efficient
//    dequantization through preprocessing": no native FP4 x BF16 matrix core,
//    so FP4 -> BF16 in registers, then BF16 MFMA).  Activations are never
//    re-quantized.
//  * The weight layout is pre-arranged offline (layout.h) so that each lane
//    loads its MFMA fragment straight from HBM into VGPRs with one 16-byte
//    load and a wave reads one contiguous 1 KiB block.
//  * Activations are read with ranged buffer loads: rows >= m and K-padding
//    read as zero without branches (the blog's section "Generating
//    high-quality machine code": ranged buffer loads drop out-of-bounds
//    accesses).
//  * The activation tile of the large-m kernel is staged in LDS with an XOR
//    swizzle so that both the 16-byte writes and the fragment reads are free
//    of bank conflicts (the blog's section "Mastering the memory hierarchy").
//  * Dequant: gfx950 v_cvt_scalef32_pk_{f32,bf16}_fp4 converts two E2M1 codes
//    per instruction.  Its scale operand only contributes its exponent
//    (checked on the device), which is exactly an E8M0 scale, so MXFP4 is
//    one instruction per two weights.  E4M3 scales carry mantissa bits, so
//    NVFP4 converts exactly to FP32, multiplies by the decoded scale (exact:
//    at most 6 significant bits) and keeps the upper halves (exact BF16).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <type_traits>

#include "../../include/fp4gemm.h"
#include "layout.h"

int fp4_check_weight_shape(int64_t N, int64_t K, int format);  // repack.cpp

namespace fp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource word 3 for raw (stride 0) 32-bit buffer access on gfx9-family
// parts; an offset at or past the buffer's byte range reads zero.
constexpr int kBufWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kXcdCount = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

// ------------------------------------------------------------------ dequant
// Keep the upper 16 bits of two FP32 values (exact when both are BF16 values).
__device__ __forceinline__ uint32_t upper_halves(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// NVFP4: eight codes (low nibble of byte 0 first) times FP32 scale s -> eight
// BF16 values in K order, packed two per dword.
__device__ __forceinline__ u32x4 dequant_nvfp4(uint32_t w, float s) {
    const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    u32x4 o;
    o.x = upper_halves(f0.x * s, f0.y * s);
    o.y = upper_halves(f1.x * s, f1.y * s);
    o.z = upper_halves(f2.x * s, f2.y * s);
    o.w = upper_halves(f3.x * s, f3.y * s);
    return o;
}

// MXFP4: the scale operand is an FP32 whose exponent field is the E8M0 byte.
__device__ __forceinline__ u32x4 dequant_mxfp4(uint32_t w, float sexp) {
    u32x4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sexp, 0));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sexp, 1));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sexp, 2));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sexp, 3));
    return o;
}

// Scales of one lane for one 512-K scale block: 16 bytes; byte 4 c + i is the
// scale of MFMA step i of chunk c (layout.h).  Lane byte offset inside the
// block: NVFP4 r * 32 + (j / 2) * 16, MXFP4 r * 16.
template <int FMT>
__device__ __forceinline__ int scale_lane_offset(int r, int j) {
    return FMT == 0 ? r * 32 + (j >> 1) * 16 : r * 16;
}
template <int FMT>
constexpr int scale_block_bytes() { return FMT == 0 ? 512 : 256; }

// Dequantize MFMA step I (dword I of the lane's 16 bytes) of chunk C.
// NVFP4: OCP E4M3 -> FP32 with the hardware FP8 convert (OCP encoding on
// gfx950, checked on the device).  MXFP4: the E8M0 byte becomes the exponent
// field of the FP32 scale operand.
template <int FMT, int C, int I>
__device__ __forceinline__ u32x4 dequant_step(const u32x4& w, const u32x4& s) {
    if constexpr (FMT == 0) {
        return dequant_nvfp4(w[I], __builtin_amdgcn_cvt_f32_fp8((int)s[C], I));
    } else {
        return dequant_mxfp4(w[I], __uint_as_float(((s[C] >> (8 * I)) & 0xFFu) << 23));
    }
}

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ u32x4 load_a(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Store one 16x16 output fragment: lane holds Y[m][n0 .. n0+3] (MFMA output
// rows are n, columns are m).
__device__ __forceinline__ void store_frag(uint16_t* __restrict__ C, const f32x4& v, int m, int n0, int M, int N) {
    if (m >= M) return;
    const uint32_t p0 = pack_bf16_rne(v.x, v.y), p1 = pack_bf16_rne(v.z, v.w);
    uint16_t* dst = C + (size_t)m * N + n0;
    if ((N & 3) == 0 && n0 + 3 < N) {
        u32x2 pv = {p0, p1};
        *reinterpret_cast<u32x2*>(dst) = pv;
    } else {
        const uint16_t h[4] = {(uint16_t)(p0 & 0xFFFF), (uint16_t)(p0 >> 16), (uint16_t)(p1 & 0xFFFF),
                               (uint16_t)(p1 >> 16)};
        for (int e = 0; e < 4; ++e)
            if (n0 + e < N) dst[e] = h[e];
    }
}

// ------------------------------------------------------------ skinny GEMM
// Small m (<= 16*MB): each workgroup owns TN n-tiles (16 rows each) and its NW
// waves split K into contiguous ranges of 512-K scale blocks.  Every wave
// streams its tiles' 1 KiB code blocks straight into VGPRs one scale block
// ahead of the block it is multiplying (so 4*TN KiB per wave are in flight
// while it computes), reads the matching activation fragments (64 contiguous
// bytes per lane per chunk) one chunk ahead with ranged buffer loads, and the
// partial 16x16 products of the waves are summed through LDS in a fixed order
// (deterministic).  Chunk offsets live in scalar registers; only the chunk
// holding the end of K masks lanes.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufWord3);
}

template <int FMT>
__device__ __forceinline__ u32x4 load_scale_block(__amdgpu_buffer_rsrc_t r, int soff_lane, int sb) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, soff_lane, sb * scale_block_bytes<FMT>(), 0);
}

template <int FMT, int MB, int C, int I>
__device__ __forceinline__ void mma_step(const u32x4& w, const u32x4& s,
                                         const u32x4 (&a)[MB][4], f32x4 (&acc)[MB]) {
    const u32x4 wf = dequant_step<FMT, C, I>(w, s);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_bf16(wf, a[mb][I], acc[mb]);
}

template <int FMT, int MB, int C>
__device__ __forceinline__ void mma_chunk(const u32x4& w, const u32x4& s,
                                          const u32x4 (&a)[MB][4], f32x4 (&acc)[MB]) {
    mma_step<FMT, MB, C, 0>(w, s, a, acc);
    mma_step<FMT, MB, C, 1>(w, s, a, acc);
    mma_step<FMT, MB, C, 2>(w, s, a, acc);
    mma_step<FMT, MB, C, 3>(w, s, a, acc);
}

// Activation fragments of chunk b for the lane: rows mb*16 + r, K = 128 b + 32 i + 8 j.
// KTAIL (K not a multiple of 512): lanes whose 8 K-values lie at or past K read
// zeros through an out-of-range offset instead of the next row's data.
template <int MB, bool KTAIL>
__device__ __forceinline__ void load_a_chunk(__amdgpu_buffer_rsrc_t ra, const uint32_t (&arow)[MB], int b, int j,
                                             int K, u32x4 (&a)[MB][4]) {
    const int kb = b * kChunkK + j * 8;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = kb + 32 * i;
            const uint32_t off = arow[mb] + (uint32_t)k * 2u;
            a[mb][i] = load_a(ra, (!KTAIL || k < K) ? off : kOutOfRange);
        }
}

template <int FMT, int MB, int TN, int NW, bool KTAIL>
__global__ __launch_bounds__(64 * NW) void gemm_skinny(const uint16_t* __restrict__ A, const u32x4* __restrict__ wq,
                                                      const uint8_t* __restrict__ sq, uint16_t* __restrict__ C,
                                                      int M, int N, int K, int KB, int SB, int NT) {
    typedef u32x4 SW;
    constexpr int kScaleBlockBytes = scale_block_bytes<FMT>();  // per tile per scale block
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane & 15, j = lane >> 4;
    const int tile0 = blockIdx.x * TN;
    const int soff = scale_lane_offset<FMT>(r, j);

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)(M * K * 2));
    uint32_t arow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) arow[mb] = (uint32_t)((mb * 16 + r) * K) * 2u;

    // Tiles past the end re-read the last tile; their stores are masked by n < N.
    __amdgpu_buffer_rsrc_t rw[TN], rs[TN];
#pragma unroll
    for (int tt = 0; tt < TN; ++tt) {
        const int t = min(tile0 + tt, NT - 1);
        rw[tt] = make_rsrc(reinterpret_cast<const uint8_t*>(wq) + (size_t)t * KB * 1024, (uint32_t)KB * 1024u);
        rs[tt] = make_rsrc(sq + (size_t)t * SB * kScaleBlockBytes, (uint32_t)(SB * kScaleBlockBytes));
    }

    f32x4 acc[TN][MB];
#pragma unroll
    for (int tt = 0; tt < TN; ++tt)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[tt][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Software pipeline over 128-K chunks, three chunks deep: register slot
    // c % 4 holds the code blocks and activation fragments of chunk c; at the
    // step that multiplies chunk c, chunk c+3 is issued into slot (c+3) % 4.
    // Vector-memory loads complete in issue order, and every wait is for a
    // slot filled three steps earlier, so no wait covers a younger prefetch.
    // Scales alternate between two register sets, one 512-K block ahead, and
    // the loop body covers two blocks so that no loaded register is copied
    // across the loop back edge (that keeps the compiler's wait counts exact).
    // The tail re-reads the wave's last chunk (a cache hit) instead of
    // branching.
    const int sb0 = (wave * SB) / NW, sb1 = ((wave + 1) * SB) / NW;
    if (sb0 < sb1) {
        const int clast = 4 * sb1 - 1;
        u32x4 wr[4][TN];
        u32x4 ar[4][MB][4];
        SW sa[TN], sbs[TN];
        auto issue = [&](auto slot_c, int chunk) {
            constexpr int S = decltype(slot_c)::value;
            chunk = min(chunk, clast);
#pragma unroll
            for (int tt = 0; tt < TN; ++tt)
                wr[S][tt] = __builtin_amdgcn_raw_buffer_load_b128(rw[tt], lane * 16, chunk * 1024, 0);
            load_a_chunk<MB, KTAIL>(ra, arow, chunk, j, K, ar[S]);
        };
        // one 512-K block: multiply chunks 4 sbx .. 4 sbx + 3 with scales cur,
        // prefetch the scales of block nsb into nxt
        auto block = [&](int sbx, const SW (&cur)[TN], SW (&nxt)[TN], int nsb) {
            const int base = 4 * sbx;
            issue(std::integral_constant<int, 3>{}, base + 3);
#pragma unroll
            for (int tt = 0; tt < TN; ++tt) nxt[tt] = load_scale_block<FMT>(rs[tt], soff, nsb);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tt = 0; tt < TN; ++tt) mma_chunk<FMT, MB, 0>(wr[0][tt], cur[tt], ar[0], acc[tt]);
            __builtin_amdgcn_sched_barrier(0);
            issue(std::integral_constant<int, 0>{}, base + 4);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tt = 0; tt < TN; ++tt) mma_chunk<FMT, MB, 1>(wr[1][tt], cur[tt], ar[1], acc[tt]);
            __builtin_amdgcn_sched_barrier(0);
            issue(std::integral_constant<int, 1>{}, base + 5);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tt = 0; tt < TN; ++tt) mma_chunk<FMT, MB, 2>(wr[2][tt], cur[tt], ar[2], acc[tt]);
            __builtin_amdgcn_sched_barrier(0);
            issue(std::integral_constant<int, 2>{}, base + 6);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tt = 0; tt < TN; ++tt) mma_chunk<FMT, MB, 3>(wr[3][tt], cur[tt], ar[3], acc[tt]);
            __builtin_amdgcn_sched_barrier(0);
        };
#pragma unroll
        for (int tt = 0; tt < TN; ++tt) sa[tt] = load_scale_block<FMT>(rs[tt], soff, sb0);
        issue(std::integral_constant<int, 0>{}, 4 * sb0 + 0);
        issue(std::integral_constant<int, 1>{}, 4 * sb0 + 1);
        issue(std::integral_constant<int, 2>{}, 4 * sb0 + 2);
        int sb = sb0;
        for (; sb + 1 < sb1; sb += 2) {
            block(sb, sa, sbs, sb + 1);
            block(sb + 1, sbs, sa, min(sb + 2, sb1 - 1));
        }
        if (sb < sb1) block(sb, sa, sbs, sb);  // odd block count
    }

    if constexpr (NW > 1) {
        __shared__ f32x4 red[(NW - 1) * TN * MB * kLanes];
        if (wave > 0) {
#pragma unroll
            for (int tt = 0; tt < TN; ++tt)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) red[(((wave - 1) * TN + tt) * MB + mb) * kLanes + lane] = acc[tt][mb];
        }
        __syncthreads();
        if (wave != 0) return;
        for (int w = 1; w < NW; ++w)
#pragma unroll
            for (int tt = 0; tt < TN; ++tt)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[tt][mb] += red[(((w - 1) * TN + tt) * MB + mb) * kLanes + lane];
    }
#pragma unroll
    for (int tt = 0; tt < TN; ++tt)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) store_frag(C, acc[tt][mb], mb * 16 + r, (tile0 + tt) * kTileN + 4 * j, M, N);
}

// ------------------------------------------------------------- tiled GEMM
// Larger m.  A 256-thread workgroup computes a BM x BN output tile with its
// four waves in a WM x WN grid; a wave owns MBW 16-row blocks of m and TNW
// 16-row tiles of n.  Per 128-K chunk:
//   * the activation tile (BM rows x 128 K, BF16) lives in LDS, double
//     buffered, with its 16-byte columns XOR-swizzled by row so that both the
//     16-byte writes and the fragment reads are free of bank conflicts (the
//     Petit blog, "Mastering the memory hierarchy": permuted LDS layout);
//   * the next chunk's activations and code blocks are loaded into registers
//     while the current chunk is multiplied (activations first, so the wait
//     before they are written to LDS never covers the code-block prefetch);
//   * barriers fence LDS only, so they never drain the prefetch.
// Work items are ordered so that each XCD gets a contiguous band of n-tiles
// (all m-tiles of it): the band's codes are fetched by one L2 only and the
// activations stay L2-resident per XCD (the blog's topology-aware partition).
template <int FMT, int WM, int WN, int MBW, int TNW, bool KTAIL>
__global__ __launch_bounds__(256) void gemm_tiled(const uint16_t* __restrict__ A, const u32x4* __restrict__ wq,
                                                 const uint8_t* __restrict__ sq, uint16_t* __restrict__ C, int M,
                                                 int N, int K, int KB, int SB, int NT) {
    static_assert(WM * WN == 4, "four waves");
    constexpr int BM = WM * MBW * 16;  // m rows per workgroup
    constexpr int BNT = WN * TNW;      // n-tiles per workgroup
    constexpr int kBuf = BM * 256;     // one LDS activation buffer (BM x 128 K x 2 B)
    constexpr int kStage = BM / 16;    // 16-byte activation pieces per thread per chunk
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * kBuf];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, j = lane >> 4;
    const int wm = wave % WM, wn = wave / WM;

    // XCD-banded work order
    const int MT = (M + BM - 1) / BM, NG = (NT + BNT - 1) / BNT;
    const int total = MT * NG;
    int L = blockIdx.x;
    if (total % kXcdCount == 0) L = (blockIdx.x % kXcdCount) * (total / kXcdCount) + blockIdx.x / kXcdCount;
    const int mt = L % MT, ng = L / MT;
    const int m0 = mt * BM;
    const int tile0 = ng * BNT + wn * TNW;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)(M * K * 2));
    constexpr int kScaleBlockBytes = scale_block_bytes<FMT>();
    const int soff = scale_lane_offset<FMT>(r, j);
    __amdgpu_buffer_rsrc_t rw[TNW], rs[TNW];
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) {
        const int t = min(tile0 + tt, NT - 1);
        rw[tt] = make_rsrc(reinterpret_cast<const uint8_t*>(wq) + (size_t)t * KB * 1024, (uint32_t)KB * 1024u);
        rs[tt] = make_rsrc(sq + (size_t)t * SB * kScaleBlockBytes, (uint32_t)(SB * kScaleBlockBytes));
    }

    // activation staging: piece q of this thread = (row, 16-byte column)
    uint32_t aoff[kStage];
    int lds_off[kStage];
#pragma unroll
    for (int q = 0; q < kStage; ++q) {
        const int idx = tid + 256 * q;
        const int row = idx >> 4, col = idx & 15;
        aoff[q] = (uint32_t)((m0 + row) * K + col * 8) * 2u;
        lds_off[q] = row * 256 + ((col ^ (row & 15)) << 4);
    }
    auto load_stage = [&](int b, u32x4 (&st)[kStage]) {
#pragma unroll
        for (int q = 0; q < kStage; ++q) {
            const int col = ((tid + 256 * q) & 15);
            const int k = b * kChunkK + col * 8;
            const uint32_t off = aoff[q] + (uint32_t)(b * kChunkK) * 2u;
            st[q] = load_a(ra, (!KTAIL || k < K) ? off : kOutOfRange);
        }
    };
    auto store_stage = [&](int buf, const u32x4 (&st)[kStage]) {
#pragma unroll
        for (int q = 0; q < kStage; ++q) *reinterpret_cast<u32x4*>(lds_a + buf * kBuf + lds_off[q]) = st[q];
    };
    auto lds_barrier = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    f32x4 acc[TNW][MBW];
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) acc[tt][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // multiply chunk b (activations in LDS buffer buf) with code blocks w
    auto compute = [&](auto cc, int buf, const u32x4 (&w)[TNW], const u32x4 (&sc)[TNW]) {
        constexpr int CC = decltype(cc)::value;
        const uint8_t* base = lds_a + buf * kBuf;
        auto step = [&](auto ii) {
            constexpr int I = decltype(ii)::value;
            u32x4 a[MBW];
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                const int row = wm * MBW * 16 + mb * 16 + r;
                const int col = 4 * I + j;
                a[mb] = *reinterpret_cast<const u32x4*>(base + row * 256 + ((col ^ (row & 15)) << 4));
            }
#pragma unroll
            for (int tt = 0; tt < TNW; ++tt) {
                const u32x4 wf = dequant_step<FMT, CC, I>(w[tt], sc[tt]);
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) acc[tt][mb] = mfma_bf16(wf, a[mb], acc[tt][mb]);
            }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
    };

    const int last = KB - 1;
    u32x4 st[kStage];
    u32x4 w0[TNW], w1[TNW], sc[TNW], scn[TNW];
    load_stage(0, st);
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) {
        w0[tt] = __builtin_amdgcn_raw_buffer_load_b128(rw[tt], lane * 16, 0, 0);
        sc[tt] = load_scale_block<FMT>(rs[tt], soff, 0);
    }
    store_stage(0, st);
    lds_barrier();
    // chunk pairs (b even in w0, b odd in w1); a scale block is 4 chunks
    for (int sb = 0; sb < SB; ++sb) {
        const int nsb = min(sb + 1, SB - 1);
        auto half = [&](auto cc, const u32x4 (&wc)[TNW], u32x4 (&wn)[TNW]) {
            constexpr int CC = decltype(cc)::value;
            const int b = 4 * sb + CC;
            const int bn = min(b + 1, last);
            load_stage(bn, st);
#pragma unroll
            for (int tt = 0; tt < TNW; ++tt) {
                wn[tt] = __builtin_amdgcn_raw_buffer_load_b128(rw[tt], lane * 16, bn * 1024, 0);
                if constexpr (CC == 3) scn[tt] = load_scale_block<FMT>(rs[tt], soff, nsb);
            }
            compute(cc, b & 1, wc, sc);
            store_stage((b + 1) & 1, st);
            lds_barrier();
        };
        half(std::integral_constant<int, 0>{}, w0, w1);
        half(std::integral_constant<int, 1>{}, w1, w0);
        half(std::integral_constant<int, 2>{}, w0, w1);
        half(std::integral_constant<int, 3>{}, w1, w0);
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt) sc[tt] = scn[tt];
    }
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
            store_frag(C, acc[tt][mb], m0 + wm * MBW * 16 + mb * 16 + r, (tile0 + tt) * kTileN + 4 * j, M, N);
}

// ------------------------------------------------------------ debug dequant
// One wave per (n-tile, 128-K chunk): writes the BF16 weights it would feed to
// the matrix core, using the GEMM's own dequant functions.
template <int FMT>
__global__ __launch_bounds__(64) void dequant_kernel(const u32x4* __restrict__ wq, const uint8_t* __restrict__ sq,
                                                     uint16_t* __restrict__ W, int N, int K, int KB, int SB) {
    typedef u32x4 SW;
    const int t = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x, r = lane & 15, j = lane >> 4;
    const int n = t * kTileN + r;
    const u32x4 w = wq[((size_t)t * KB + b) * kLanes + lane];
    const SW s = *reinterpret_cast<const u32x4*>(sq + ((size_t)t * SB + b / 4) * scale_block_bytes<FMT>() +
                                                 scale_lane_offset<FMT>(r, j));
    u32x4 o[4];
    switch (b & 3) {
        case 0: o[0] = dequant_step<FMT, 0, 0>(w, s); o[1] = dequant_step<FMT, 0, 1>(w, s);
                o[2] = dequant_step<FMT, 0, 2>(w, s); o[3] = dequant_step<FMT, 0, 3>(w, s); break;
        case 1: o[0] = dequant_step<FMT, 1, 0>(w, s); o[1] = dequant_step<FMT, 1, 1>(w, s);
                o[2] = dequant_step<FMT, 1, 2>(w, s); o[3] = dequant_step<FMT, 1, 3>(w, s); break;
        case 2: o[0] = dequant_step<FMT, 2, 0>(w, s); o[1] = dequant_step<FMT, 2, 1>(w, s);
                o[2] = dequant_step<FMT, 2, 2>(w, s); o[3] = dequant_step<FMT, 2, 3>(w, s); break;
        default: o[0] = dequant_step<FMT, 3, 0>(w, s); o[1] = dequant_step<FMT, 3, 1>(w, s);
                 o[2] = dequant_step<FMT, 3, 2>(w, s); o[3] = dequant_step<FMT, 3, 3>(w, s); break;
    }
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = b * kChunkK + 32 * i + 8 * j;
        if (k < K) *reinterpret_cast<u32x4*>(W + (size_t)n * K + k) = o[i];
    }
}

// ------------------------------------------------------------- host side
std::atomic<int> g_device_state[64];  // 0 unknown, 1 gfx950, 2 other

static int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP4_ERR_DEVICE;
    int st = g_device_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FP4_ERR_DEVICE;
        st = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? FP4_OK : FP4_ERR_DEVICE;
}

static int launch_status() {
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

// Row block the kernels for this m read A in (A offsets are 32-bit).
static int64_t a_row_block(int64_t M) {
    if (M <= 16) return 16;
    if (M <= 32) return 32;
    if (M <= 64) return 64;
    return 256;  // largest tiled m-block
}

// Skinny-kernel shape: TN n-tiles per workgroup, NW waves splitting K.
struct SkinnyShape {
    int tn, nw;
};

// Tuning override "TN,NW" from FP4GEMM_SKINNY (read once; used by sweeps).
static SkinnyShape skinny_override() {
    static const SkinnyShape ov = [] {
        SkinnyShape s{0, 0};
        const char* e = getenv("FP4GEMM_SKINNY");
        if (e) sscanf(e, "%d,%d", &s.tn, &s.nw);
        return s;
    }();
    return ov;
}

// Measured on MI355X over the Llama-3-70B decode shapes (m = 16): many
// n-tiles favour fewer, wider waves; long K favours more waves per tile.
static SkinnyShape pick_skinny(int MB, int NT, int SB) {
    SkinnyShape ov = skinny_override();
    if (ov.tn > 0) return ov;
    if (MB > 1) return {1, 4};
    if (NT >= 2048) return {4, 2};
    if (SB >= 32) return {2, 4};
    if (NT >= 640) return {4, 4};
    return {2, 4};
}

#define FP4_SKINNY_CASE(MB_, TN_, NW_)                                                                   \
    if (sh.tn == TN_ && sh.nw == NW_) {                                                                  \
        gemm_skinny<FMT, MB_, TN_, NW_, false><<<dim3((NT + TN_ - 1) / TN_), dim3(64 * NW_), 0, s>>>(    \
            A, wq, sq, C, M, N, K, KB, SB, NT);                                                          \
        return true;                                                                                     \
    }

template <int FMT>
static bool launch_skinny(int MB, SkinnyShape sh, const uint16_t* A, const u32x4* wq, const uint8_t* sq,
                          uint16_t* C, int M, int N, int K, int KB, int SB, int NT, hipStream_t s) {
    if (MB == 1) {
        FP4_SKINNY_CASE(1, 1, 2) FP4_SKINNY_CASE(1, 1, 4) FP4_SKINNY_CASE(1, 1, 8)
        FP4_SKINNY_CASE(1, 2, 2) FP4_SKINNY_CASE(1, 2, 4) FP4_SKINNY_CASE(1, 2, 8)
        FP4_SKINNY_CASE(1, 4, 2) FP4_SKINNY_CASE(1, 4, 4) FP4_SKINNY_CASE(1, 4, 8)
    } else if (MB == 2) {
        FP4_SKINNY_CASE(2, 1, 4) FP4_SKINNY_CASE(2, 1, 8) FP4_SKINNY_CASE(2, 2, 4) FP4_SKINNY_CASE(2, 2, 8)
    } else {
        FP4_SKINNY_CASE(4, 1, 4)
    }
    return false;
}
#undef FP4_SKINNY_CASE

// Tiled-kernel shape: WM x WN waves, MBW m-blocks and TNW n-tiles per wave.
struct TiledShape {
    int wm, wn, mbw, tnw;
};

static TiledShape tiled_override() {
    static const TiledShape ov = [] {
        TiledShape t{0, 0, 0, 0};
        const char* e = getenv("FP4GEMM_TILED");
        if (e) sscanf(e, "%d,%d,%d,%d", &t.wm, &t.wn, &t.mbw, &t.tnw);
        return t;
    }();
    return ov;
}

// Measured on MI355X over the Llama-3-70B prefill shapes (m = 256): one wave
// over all 128 rows of the block amortizes each dequantized code over 128
// products; wide-N shapes take two n-tiles per wave.
static TiledShape pick_tiled(int M, int NT) {
    (void)M;
    TiledShape ov = tiled_override();
    if (ov.wm > 0) return ov;
    return NT >= 640 ? TiledShape{1, 4, 8, 2} : TiledShape{1, 4, 8, 1};
}

template <int FMT, int WM, int WN, int MBW, int TNW>
static void launch_tiled_t(const uint16_t* A, const u32x4* wq, const uint8_t* sq, uint16_t* C, int M, int N, int K,
                           int KB, int SB, int NT, hipStream_t s) {
    constexpr int BM = WM * MBW * 16, BNT = WN * TNW;
    const int grid = ((M + BM - 1) / BM) * ((NT + BNT - 1) / BNT);
    if (K % kScaleBlockK == 0)
        gemm_tiled<FMT, WM, WN, MBW, TNW, false><<<dim3(grid), dim3(256), 0, s>>>(A, wq, sq, C, M, N, K, KB, SB, NT);
    else
        gemm_tiled<FMT, WM, WN, MBW, TNW, true><<<dim3(grid), dim3(256), 0, s>>>(A, wq, sq, C, M, N, K, KB, SB, NT);
}

template <int FMT>
static void launch_tiled(TiledShape t, const uint16_t* A, const u32x4* wq, const uint8_t* sq, uint16_t* C, int M,
                         int N, int K, int KB, int SB, int NT, hipStream_t s) {
#define FP4_TILED_CASE(WM_, WN_, MBW_, TNW_)                                                         \
    if (t.wm == WM_ && t.wn == WN_ && t.mbw == MBW_ && t.tnw == TNW_)                                \
        return launch_tiled_t<FMT, WM_, WN_, MBW_, TNW_>(A, wq, sq, C, M, N, K, KB, SB, NT, s);
    FP4_TILED_CASE(1, 4, 8, 1) FP4_TILED_CASE(1, 4, 8, 2) FP4_TILED_CASE(1, 4, 4, 1) FP4_TILED_CASE(1, 4, 4, 2)
    FP4_TILED_CASE(2, 2, 4, 4) FP4_TILED_CASE(2, 2, 4, 2)
#undef FP4_TILED_CASE
    launch_tiled_t<FMT, 1, 4, 8, 1>(A, wq, sq, C, M, N, K, KB, SB, NT, s);  // shape not compiled: default
}

template <int FMT>
static int launch_gemm(const uint16_t* A, const u32x4* wq, const uint8_t* sq, uint16_t* C, int M, int N, int K,
                       int KB, int SB, int NT, hipStream_t s) {
    if (M <= 64 && K % kScaleBlockK != 0) {  // ragged K: masked activation loads
        if (M <= 16)
            gemm_skinny<FMT, 1, 1, 4, true><<<dim3(NT), dim3(256), 0, s>>>(A, wq, sq, C, M, N, K, KB, SB, NT);
        else if (M <= 32)
            gemm_skinny<FMT, 2, 1, 4, true><<<dim3(NT), dim3(256), 0, s>>>(A, wq, sq, C, M, N, K, KB, SB, NT);
        else
            gemm_skinny<FMT, 4, 1, 4, true><<<dim3(NT), dim3(256), 0, s>>>(A, wq, sq, C, M, N, K, KB, SB, NT);
    } else if (M <= 64) {
        const int MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
        SkinnyShape sh = pick_skinny(MB, NT, SB);
        if (!launch_skinny<FMT>(MB, sh, A, wq, sq, C, M, N, K, KB, SB, NT, s)) {
            sh = SkinnyShape{1, 4};  // an override naming no compiled shape falls back to the default
            launch_skinny<FMT>(MB, sh, A, wq, sq, C, M, N, K, KB, SB, NT, s);
        }
    } else {
        launch_tiled<FMT>(pick_tiled(M, NT), A, wq, sq, C, M, N, K, KB, SB, NT, s);
    }
    return FP4_OK;
}

}  // namespace fp4

using namespace fp4;

extern "C" int fp4_gemm_workspace_size(int64_t m, int64_t N, int64_t K, int format, size_t* bytes) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (m < 0 || m > (int64_t(1) << 20)) return FP4_ERR_SHAPE;
    if (!bytes) return FP4_ERR_NULL;
    *bytes = 0;
    return FP4_OK;
}

extern "C" int fp4_gemm(const void* A, const void* wq, const void* sq, void* C, int64_t m, int64_t N, int64_t K,
                        int format, void* workspace, size_t workspace_bytes, void* stream) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (m < 0 || m > (int64_t(1) << 20)) return FP4_ERR_SHAPE;
    if (m == 0) return FP4_OK;
    if (!A || !wq || !sq || !C) return FP4_ERR_NULL;
    if (round_up(m, a_row_block(m)) * K * 2 >= (int64_t(1) << 31)) return FP4_ERR_SHAPE;
    (void)workspace;
    (void)workspace_bytes;
    st = check_device();
    if (st != FP4_OK) return st;
    const int64_t Np = padded_n(N), Kp = padded_k(K);
    const int KB = int(Kp / kChunkK), SB = int(Kp / kScaleBlockK), NT = int(Np / kTileN);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (format == FP4_NVFP4)
        launch_gemm<0>((const uint16_t*)A, (const u32x4*)wq, (const uint8_t*)sq, (uint16_t*)C, int(m), int(N), int(K),
                       KB, SB, NT, s);
    else
        launch_gemm<1>((const uint16_t*)A, (const u32x4*)wq, (const uint8_t*)sq, (uint16_t*)C, int(m), int(N), int(K),
                       KB, SB, NT, s);
    return launch_status();
}

extern "C" int fp4_dequant(const void* wq, const void* sq, void* W_bf16, int64_t N, int64_t K, int format,
                           void* stream) {
    int st = fp4_check_weight_shape(N, K, format);
    if (st != FP4_OK) return st;
    if (!wq || !sq || !W_bf16) return FP4_ERR_NULL;
    st = check_device();
    if (st != FP4_OK) return st;
    const int64_t Np = padded_n(N), Kp = padded_k(K);
    const int KB = int(Kp / kChunkK), SB = int(Kp / kScaleBlockK), NT = int(Np / kTileN);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    dim3 grid(NT, KB);
    if (format == FP4_NVFP4)
        dequant_kernel<0><<<grid, dim3(64), 0, s>>>((const u32x4*)wq, (const uint8_t*)sq, (uint16_t*)W_bf16, int(N),
                                                    int(K), KB, SB);
    else
        dequant_kernel<1><<<grid, dim3(64), 0, s>>>((const u32x4*)wq, (const uint8_t*)sq, (uint16_t*)W_bf16, int(N),
                                                    int(K), KB, SB);
    return launch_status();
}
