// BF16 / FP16 x FP4 (NVFP4 / MXFP4) GEMM kernels for gfx950 (device code).
//
//   Y[m][N] = A[m][K] . dequant(W)[N][K]^T, FP32 accumulation, output in the
//   activation type (ACT = 0: BF16, ACT = 1: FP16).
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
//    FP16 activations (the Petit blog, "Introduction": FP16/BF16 x FP4): the
//    FP4 -> FP16 convert applies the scale's exponent and one packed FP16
//    multiply applies its mantissa, both exact.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "../../include/fp4gemm.h"
#include "dispatch.h"
#include "layout.h"

namespace fp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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
// Cache-policy operand of buffer loads that stream data read once (the decode
// kernels' weight codes and scales): the nontemporal hint.  The prefill
// kernels load theirs with the default policy instead (kLoadReused): the
// m-tiles of a weight tile read the same bytes, and with the hint the later
// reads missed L2 more often (MI355X, the four Llama-3-70B layers at
// m = 256, interleaved: 411 against 419 us; the decode step with the default
// policy 119 against 115 us).
constexpr int kLoadStream = 2;
constexpr int kLoadReused = 0;
constexpr int kXcdCount = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin
// Cache-policy operand sc1 (device scope): the access is coherent across the
// XCDs' separate L2 caches (stores write through, loads do not hit a line
// another XCD may have changed).  Used for the split-K partial sums.
constexpr int kDeviceCoherent = 16;

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
// block: NVFP4 (j / 2) * 256 + r * 16, MXFP4 r * 16.
template <int FMT>
__device__ __forceinline__ int scale_lane_offset(int r, int j) {
    return FMT == 0 ? (j >> 1) * 256 + r * 16 : r * 16;
}
template <int FMT>
constexpr int scale_block_bytes() { return FMT == 0 ? 512 : 256; }

// FP16 targets.  NVFP4: the convert's scale operand is the decoded E4M3
// scale s, of which it applies the exponent (c x 2^e, exact in FP16: between
// 2^-10 and 1536); the packed multiply applies s / 2^e in [1, 2) (at most 4
// significant bits; the product has at most 6: exact).  A zero scale gives
// c x 2^-127, which rounds to zero in FP16.  MXFP4: the E8M0 scale is the
// convert's scale operand; exact for exponents -23 .. 13.
__device__ __forceinline__ u32x4 dequant_nvfp4_f16(uint32_t w, float s) {
    const uint32_t mant = 0x3C00u | ((__float_as_uint(s) >> 13) & 0x3FFu);  // FP16 bits of s / 2^e
    const f16x2 m2 = __builtin_bit_cast(f16x2, mant | (mant << 16));
    u32x4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 0) * m2);
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 1) * m2);
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 2) * m2);
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 3) * m2);
    return o;
}

__device__ __forceinline__ u32x4 dequant_mxfp4_f16(uint32_t w, float sexp) {
    u32x4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sexp, 0));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sexp, 1));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sexp, 2));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sexp, 3));
    return o;
}

// Dequantize MFMA step I (dword I of the lane's 16 bytes) of chunk C into the
// activation type ACT.  NVFP4: OCP E4M3 -> FP32 with the hardware FP8
// convert (OCP encoding on gfx950, checked on the device).  MXFP4: the E8M0
// byte becomes the exponent field of the FP32 scale operand.
template <int FMT, int C, int I, int ACT = 0>
__device__ __forceinline__ u32x4 dequant_step(const u32x4& w, const u32x4& s) {
    if constexpr (FMT == 0) {
        const float sf = __builtin_amdgcn_cvt_f32_fp8((int)s[C], I);
        if constexpr (ACT == 0) return dequant_nvfp4(w[I], sf);
        else return dequant_nvfp4_f16(w[I], sf);
    } else {
        const float se = __uint_as_float(((s[C] >> (8 * I)) & 0xFFu) << 23);
        if constexpr (ACT == 0) return dequant_mxfp4(w[I], se);
        else return dequant_mxfp4_f16(w[I], se);
    }
}

// 16x16x32 matrix-core product in the activation type, FP32 accumulate.
template <int ACT = 0>
__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
    if constexpr (ACT == 0)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

__device__ __forceinline__ u32x4 load_a(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Two FP32 values rounded to nearest even into the output type, packed.
template <int ACT = 0>
__device__ __forceinline__ uint32_t pack_out(float lo, float hi) {
    if constexpr (ACT == 0) {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

// ------------------------------------------------------------ buffer access
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufWord3);
}

// Store one 16x16 output fragment: lane holds Y[m][n0 .. n0+3] (MFMA output
// rows are n, columns are m) of the [M][N] output (M * N * 2 < 2^31 bytes).
// Ranged buffer stores: an element at or past row M or column N gets an
// offset past the buffer's range and the hardware drops it, so the epilogue
// has no branches (the Petit blog, "Generating high-quality machine code":
// ranged memory instructions discard out-of-bounds accesses).
template <int ACT = 0>
__device__ __forceinline__ void store_frag(uint16_t* __restrict__ C, const f32x4& v, int m, int n0, int M, int N) {
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C, (uint32_t)M * (uint32_t)N * 2u);
    const uint32_t p0 = pack_out<ACT>(v.x, v.y), p1 = pack_out<ACT>(v.z, v.w);
    const uint32_t base = ((uint32_t)m * (uint32_t)N + (uint32_t)n0) * 2u;  // used only when in range
    if ((N & 3) == 0) {  // the four columns are all inside or all past N
        const uint32_t off = (m < M && n0 < N) ? base : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{p0, p1}, rc, off, 0, 0);
    } else {
        const uint32_t h[4] = {p0 & 0xFFFFu, p0 >> 16, p1 & 0xFFFFu, p1 >> 16};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)h[e], rc,
                                                  (m < M && n0 + e < N) ? base + 2u * e : kOutOfRange, 0, 0);
    }
}

template <int FMT, int POL = kLoadStream>
__device__ __forceinline__ u32x4 load_scale_block(__amdgpu_buffer_rsrc_t r, int soff_lane, int sb) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, soff_lane, sb * scale_block_bytes<FMT>(), POL);
}

// ------------------------------------------------------------ split-K fixup
// A K split over S workgroups without a second kernel.  Each workgroup of a
// group writes its FP32 partial sums P[ks][m][n] with device-coherent stores,
// waits until they are complete and counts itself in at the group's arrival
// word; the workgroup that arrives last adds the S partials in the fixed
// order s = 0, 1, ... (device-coherent loads), scales by alpha and writes
// the output.  Because every access to the partials and to the arrival word
// is device-coherent, no cache-wide write-back or invalidate is needed.
// The arrival word is (tag << 32) | count with a tag unique to the launch
// (never 0): a word holding any other tag (stale words of earlier launches,
// partial sums of other shapes, uninitialized memory) counts as zero, so the
// workspace needs no initialization.  The last arrival writes 0 instead of
// the full count, so a launch replayed with the same tag (a captured HIP
// graph bakes the tag into the kernel arguments) finds the word at zero
// again.  The arrival words follow the partials at a 256-byte aligned
// offset (in floats):
__host__ __device__ inline size_t split_counter_floats(int S, int M, int N) {
    return ((size_t)S * (size_t)M * (size_t)N + 63) / 64 * 64;
}

// Partial plane ks of an S-way split (M x N FP32, M * N < 2^29).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t split_plane(const float* P, int ks, int M, int N) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(P) + (size_t)ks * M * N, 0, M * N * 4, kBufWord3);
}

// Store the FP32 partials of one 16x16 output fragment (lane: row m, columns
// n0 .. n0 + 3) into plane `pl` with device-coherent ranged stores; rows at
// or past M and columns at or past N are dropped.
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t pl, const f32x4& v, int m, int n0, int M,
                                              int N) {
    const uint32_t off = ((uint32_t)m * (uint32_t)N + (uint32_t)n0) * 4u;  // used only when in range
    if ((N & 3) == 0) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), pl,
                                               (m < M && n0 < N) ? off : kOutOfRange, 0, kDeviceCoherent);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), pl,
                                                  (m < M && n0 + e < N) ? off + 4 * e : kOutOfRange, 0,
                                                  kDeviceCoherent);
    }
}

// Count one arrival at word w; true for the S-th arrival of this launch,
// which leaves the word at 0 (no other workgroup of the launch touches it
// after that).  A word that already carries this launch's tag is counted
// with one atomic add (its count is below S, so no reset can intervene and
// the add never carries into the tag); a word with another tag is claimed
// with a compare-exchange that installs (tag, 1).  Workgroups that arrive
// together thus pay at most one failed exchange each, then one add, instead
// of retrying an exchange once per earlier arrival.
__device__ __forceinline__ bool split_arrive(unsigned long long* w, uint32_t tag, int S) {
    const unsigned long long mine = (unsigned long long)tag << 32;
    unsigned long long cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {  // a failed exchange means another workgroup changed the word: at most S - 1 turns
        uint32_t cnt;
        if ((cur >> 32) == (unsigned long long)tag) {
            cnt = (uint32_t)__hip_atomic_fetch_add(w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        } else if (__hip_atomic_compare_exchange_strong(w, &cur, S == 1 ? 0ull : mine | 1ull, __ATOMIC_RELAXED,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            cnt = 1u;
        } else {
            continue;  // cur now holds the word's value
        }
        if (cnt == (uint32_t)S && S > 1)
            __hip_atomic_store(w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return cnt == (uint32_t)S;
    }
}

// Y[m][n] = alpha * sum_s P[s][m][n] over the rows [m_begin, m_end) and
// columns [n_begin, n_end), in the order s = 0, 1, ... (SS: S known at
// compile time, else 0).
template <int ACT, int kThreads, int SS>
__device__ __forceinline__ void split_sum(const float* P, uint16_t* __restrict__ C, int M, int N, int S, int m_begin,
                                          int m_end, int n_begin, int n_end, float alpha) {
    const int quads = (n_end - n_begin + 3) >> 2;
    const int total = (m_end - m_begin) * quads;
    for (int e = threadIdx.x; e < total; e += kThreads) {
        const int m = m_begin + e / quads, n = n_begin + 4 * (e % quads);
        const uint32_t off = (uint32_t)(m * N + n) * 4u;
        if ((N & 3) == 0 && n + 3 < N) {
            f32x4 v;
            if constexpr (SS > 0) {
                u32x4 p[SS];
#pragma unroll
                for (int s = 0; s < SS; ++s)
                    p[s] = __builtin_amdgcn_raw_buffer_load_b128(split_plane(P, s, M, N), off, 0, kDeviceCoherent);
                v = __builtin_bit_cast(f32x4, p[0]);
#pragma unroll
                for (int s = 1; s < SS; ++s) v += __builtin_bit_cast(f32x4, p[s]);
            } else {
                v = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(split_plane(P, 0, M, N), off, 0, kDeviceCoherent));
                for (int s = 1; s < S; ++s)
                    v += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(split_plane(P, s, M, N), off,
                                                                                         0, kDeviceCoherent));
            }
            v *= alpha;
            u32x2 o = {pack_out<ACT>(v.x, v.y), pack_out<ACT>(v.z, v.w)};
            *reinterpret_cast<u32x2*>(C + (size_t)m * N + n) = o;
        } else {
            for (int x = 0; x < 4 && n + x < n_end; ++x) {
                float v = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(split_plane(P, 0, M, N), off + 4 * x, 0, kDeviceCoherent));
                for (int s = 1; s < S; ++s)
                    v += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(split_plane(P, s, M, N), off + 4 * x,
                                                                              0, kDeviceCoherent));
                v *= alpha;
                C[(size_t)m * N + n + x] = (uint16_t)(pack_out<ACT>(v, 0.f) & 0xFFFF);
            }
        }
    }
}

// Called by every thread of the workgroup after its partial stores (no
// thread may have exited).  Returns in all threads; the last arriving
// workgroup of the group first writes Y[m][n] = alpha * sum_s P[s][m][n]
// for m in [m_begin, m_end), n in [n_begin, n_end).
template <int ACT, int kThreads>
__device__ __forceinline__ void split_finish(const float* P, uint16_t* __restrict__ C, int M, int N, int S, int grp,
                                             int m_begin, int m_end, int n_begin, int n_end, float alpha,
                                             uint32_t tag) {
    __shared__ int last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long* words =
            reinterpret_cast<unsigned long long*>(const_cast<float*>(P) + split_counter_floats(S, M, N));
        last = split_arrive(words + grp, tag, S);
    }
    __syncthreads();
    if (!last) return;
    asm volatile("" ::: "memory");
    switch (S) {  // a compile-time S keeps all S loads of an output in flight at once
        case 2: split_sum<ACT, kThreads, 2>(P, C, M, N, S, m_begin, m_end, n_begin, n_end, alpha); break;
        case 4: split_sum<ACT, kThreads, 4>(P, C, M, N, S, m_begin, m_end, n_begin, n_end, alpha); break;
        case 8: split_sum<ACT, kThreads, 8>(P, C, M, N, S, m_begin, m_end, n_begin, n_end, alpha); break;
        case 16: split_sum<ACT, kThreads, 16>(P, C, M, N, S, m_begin, m_end, n_begin, n_end, alpha); break;
        default: split_sum<ACT, kThreads, 0>(P, C, M, N, S, m_begin, m_end, n_begin, n_end, alpha); break;
    }
}

// ------------------------------------------------------------ MoE routing
// Grouped mixture-of-experts GEMM (the petit-kernel page, "Features": fused
// MoE kernels for BF16 x MXFP4): expert e owns the packed weights at
// wq + e * w_stride / sq + e * s_stride (each the dense layout of N x K) and
// the assignment ids sorted_ids[offsets[e] .. offsets[e+1]); assignment id
// reads activation row id / a_div and writes output row id, scaled by
// topw[id] when topw is given.
// (MoeArgs is declared in dispatch.h, shared with the host.)

// Row block `item` of the grouped problem: blocks of `rows` assignments are
// numbered expert by expert.  Returns the expert (or -1 past the last
// block) and its first assignment and row count.  Every lane of the wave
// computes the same result: lane x of a 64-expert window counts the blocks
// of expert base + x and a wave prefix sum finds the owner.
__device__ __forceinline__ int moe_find_block(const MoeArgs& moe, int item, int rows, int& first_row, int& nrows) {
    const int lane = threadIdx.x & 63;
    int before = 0;
    for (int base = 0; base < moe.E; base += 64) {
        const int x = base + lane;
        int nb = 0, o0 = 0, o1 = 0;
        if (x < moe.E) {
            o0 = min(max(moe.offsets[x], 0), moe.P);
            o1 = min(max(moe.offsets[x + 1], o0), moe.P);
            nb = (o1 - o0 + rows - 1) / rows;
        }
        int inc = nb;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(inc, d, 64);
            if (lane >= d) inc += t;
        }
        const int start = before + inc - nb;
        const unsigned long long own = __ballot(x < moe.E && item >= start && item < start + nb);
        if (own) {
            const int src = __ffsll(own) - 1;
            const int e = __shfl(x, src, 64);
            const int blk = item - __shfl(start, src, 64);
            const int o0s = __shfl(o0, src, 64), o1s = __shfl(o1, src, 64);
            first_row = __builtin_amdgcn_readfirstlane(o0s + blk * rows);
            nrows = __builtin_amdgcn_readfirstlane(min(rows, o1s - o0s - blk * rows));
            return __builtin_amdgcn_readfirstlane(e);
        }
        before += __shfl(inc, 63, 64);
    }
    return -1;
}

// ------------------------------------------------------------ decode GEMM
// Small m (<= 16*MB) with the activations shared through LDS.  A workgroup has
// NWK groups of NWN waves.  The waves of one group cover the same K range and
// different n-tiles (TN each), so one activation chunk in LDS feeds
// TN*NWN tiles: each activation byte crosses the L1/L2 path once per
// workgroup instead of once per wave, and the loads that bring it in read
// whole 128-byte lines (1 KiB of one row per wave instruction).  The NWK
// groups split the workgroup's K range and are summed through LDS in a fixed
// order.  Narrow layers also split K over S workgroups: each writes FP32
// partial sums to the caller's workspace and the group's last workgroup to
// arrive adds them in the fixed order s = 0, 1, ... (split-K fixup above;
// the only atomics count arrivals, so results are deterministic).
//
// Pipeline.  Code blocks stream through a four-slot register ring, three
// 128-K chunks ahead of the multiply.  Activations move one 512-K scale block
// at a time through two LDS buffers: at the start of block x the
// activations of block x+1 are issued into registers (before the code blocks
// issued during block x, so waiting for them never waits for a younger code
// prefetch), and at the end of block x they are written to the buffer block
// x-1 used.  One barrier per block (LDS only: the prefetches stay in flight)
// separates those writes from the reads of block x+1 and the reads of block
// x-1 from the writes.
//
// MOE: the same kernel over one row block of one expert (MoeArgs above):
// blockIdx.y numbers the row blocks, the activation rows are gathered by
// assignment id and the output rows scattered by it; no K split.
template <int FMT, int ACT, int MB, int TN, int NWN, int NWK, bool MOE = false>
__global__ __launch_bounds__(64 * NWN * NWK) void gemm_decode(const uint16_t* __restrict__ A,
                                                             const u32x4* __restrict__ wq,
                                                             const uint8_t* __restrict__ sq,
                                                             uint16_t* __restrict__ C, float* __restrict__ P, int M,
                                                             int N, int K, int KB, int SB, int NT, int S,
                                                             float alpha, uint32_t tag, MoeArgs moe = MoeArgs{}) {
    typedef u32x4 SW;
    constexpr int kRows = 16 * MB;  // activation rows; one 1 KiB load per row per block
    // Activation load instructions per wave per block (row wn + NWN u).  When
    // NWN does not divide the row count, a wave's last slot may fall past
    // the last row: it loads and stores nothing (every row has exactly one
    // owner, and each load costs the CU's vector-memory path as much as a
    // code load does).
    constexpr int QB = (kRows + NWN - 1) / NWN;
    constexpr int kBuf = MB * 4096;  // one chunk: 16*MB rows x 128 K x 2 B
    constexpr int kBlk = 4 * kBuf;     // one 512-K block
    constexpr int kScaleBlockBytes = scale_block_bytes<FMT>();
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[NWK * 2 * kBlk];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % NWN, wk = wave / NWN;
    const int r = lane & 15, j = lane >> 4;
    const int ks = blockIdx.x % S, grp = blockIdx.x / S;
    const int tile0 = grp * (TN * NWN) + wn * TN;
    const int soff = scale_lane_offset<FMT>(r, j);
    int row0 = 0;  // MOE: first entry of ids in this row block
    if constexpr (MOE) {
        int nrows = 0;
        const int e = moe_find_block(moe, blockIdx.y, kRows, row0, nrows);
        if (e < 0) return;  // whole workgroup, before any barrier
        M = nrows;
        wq = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(wq) + (size_t)e * moe.w_stride);
        sq += (size_t)e * moe.s_stride;
    }

    // K range of the workgroup and of this wave's group, in 512-K scale blocks.
    // Every group runs nblk blocks so that all waves meet at every barrier; a
    // group with fewer blocks skips the multiply of the extra ones.
    const int wsb0 = (ks * SB) / S, wsb1 = ((ks + 1) * SB) / S;
    const int span = wsb1 - wsb0;
    const int sb0 = wsb0 + (wk * span) / NWK, sb1 = wsb0 + ((wk + 1) * span) / NWK;
    const int nblk = (span + NWK - 1) / NWK;
    const int own = sb1 - sb0;
    const int sbmax = own > 0 ? sb1 - 1 : wsb0;         // last block this group may read
    const int cmax = own > 0 ? 4 * sb1 - 1 : 4 * wsb0;  // last chunk this group may read

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)((MOE ? moe.a_rows : M) * K * 2));
    __amdgpu_buffer_rsrc_t rw[TN], rs[TN];
#pragma unroll
    for (int tt = 0; tt < TN; ++tt) {
        const int t = min(tile0 + tt, NT - 1);
        rw[tt] = make_rsrc(reinterpret_cast<const uint8_t*>(wq) + (size_t)t * KB * 1024, (uint32_t)KB * 1024u);
        rs[tt] = make_rsrc(sq + (size_t)t * SB * kScaleBlockBytes, (uint32_t)(SB * kScaleBlockBytes));
    }

    // Activations in LDS, per 128-K chunk: the 16-byte fragment of MFMA step
    // I, m-block mb, lane (j, r) sits in slot 16 j + (r ^ (4 I + j)) of the
    // 1 KiB run (I, mb).  The XOR spreads the 16 octets of one row over all
    // 16 bank groups, so the row-contiguous writes below and the fragment
    // reads are both free of bank conflicts.
    // Load u of this wave brings row q = wn + NWN u of a 512-K block: lane l
    // reads the 16 contiguous bytes at k = 512 sb + 8 l (chunk l / 16, octet
    // l % 16), so one instruction is 1 KiB of one row.
    const int a_oct = lane & 15;
    const int a_base = (lane >> 4) * kBuf + (((a_oct >> 2) * MB) * 64 + 16 * (a_oct & 3)) * 16;
    // Rows at or past m are neither loaded nor stored: they only feed MFMA
    // output columns that are never written back.
    uint32_t aoff[QB];
    int ldst[QB];
    bool alive[QB];
#pragma unroll
    for (int u = 0; u < QB; ++u) {
        const int row = min(wn + NWN * u, kRows - 1);
        alive[u] = wn + NWN * u < kRows && row < M;
        aoff[u] = (uint32_t)(row * K + 8 * lane) * 2u;
        if constexpr (MOE) {
            // gathered row; an id outside [0, a_div * a_rows) reads zeros
            const int id = alive[u] ? moe.ids[row0 + row] : 0;
            const bool in_a = id >= 0 && id / moe.a_div < moe.a_rows;
            aoff[u] = in_a ? (uint32_t)((id / moe.a_div) * K + 8 * lane) * 2u : kOutOfRange;
        }
        ldst[u] = a_base + ((row >> 4) * 64 + ((row & 15) ^ a_oct)) * 16;
    }
    uint8_t* const ring = lds_a + wk * 2 * kBlk;

    f32x4 acc[TN][MB];
#pragma unroll
    for (int tt = 0; tt < TN; ++tt)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[tt][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Code ring: kSlots slots, chunks issued kAhead = kSlots - 1 steps ahead
    // (a ring of 8 measured no faster on MI355X).
    constexpr int kSlots = 4;
    constexpr int kAhead = kSlots - 1;
    u32x4 wr[kSlots][TN];
    u32x4 ar[QB];
    SW sa[TN], sbs[TN];
    // activations of block sbx into registers
    auto a_issue = [&](int sbx) {
        const bool in_k = sbx * kScaleBlockK + 8 * lane < K;  // K tail reads zeros
#pragma unroll
        for (int u = 0; u < QB; ++u) {
            const uint32_t off = aoff[u] + (uint32_t)sbx * (kScaleBlockK * 2);
            if (alive[u]) ar[u] = load_a(ra, in_k ? off : kOutOfRange);
        }
    };
    auto a_store = [&](int buf) {
        uint8_t* dst = ring + buf * kBlk;
#pragma unroll
        for (int u = 0; u < QB; ++u)
            if (alive[u]) *reinterpret_cast<u32x4*>(dst + ldst[u]) = ar[u];
    };
    // Code blocks wholly past K (the zero padding of K to 512) are not
    // fetched: an out-of-range offset makes the load return zeros without a
    // memory access.
    // Prefetches past the group's last chunk are never multiplied: they too
    // read nothing.
    const int kb_valid = (K + kChunkK - 1) / kChunkK;
    auto w_issue = [&](auto slot_c, int chunk) {
        constexpr int SL = decltype(slot_c)::value;
        const bool live = chunk <= cmax && chunk < kb_valid;
        chunk = min(chunk, cmax);
        const uint32_t voff = (uint32_t)lane * 16u + (live ? 0u : kOutOfRange);
#pragma unroll
        for (int tt = 0; tt < TN; ++tt)
            wr[SL][tt] = __builtin_amdgcn_raw_buffer_load_b128(rw[tt], voff, chunk * 1024, kLoadStream);
    };
    auto lds_barrier = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    // multiply chunk T of the block in LDS buffer buf with code slot SL
    auto compute = [&](auto t_c, auto slot_c, const uint8_t* blk_base, const SW (&sc)[TN]) {
        constexpr int T = decltype(t_c)::value;
        constexpr int SL = decltype(slot_c)::value;
        const uint8_t* base = blk_base + T * kBuf;
        auto step = [&](auto ii) {
            constexpr int I = decltype(ii)::value;
            u32x4 a[MB];
            const int slot = 16 * j + (r ^ (4 * I + j));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                a[mb] = *reinterpret_cast<const u32x4*>(base + ((I * MB + mb) * 64 + slot) * 16);
#pragma unroll
            for (int tt = 0; tt < TN; ++tt) {
                const u32x4 wf = dequant_step<FMT, T, I, ACT>(wr[SL][tt], sc[tt]);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[tt][mb] = mfma<ACT>(wf, a[mb], acc[tt][mb]);
            }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
    };
    // chunk T of a block of parity PAR: the ring slot of the chunk c0 + 4 blk
    // + T is (4 PAR + T) % kSlots (blocks alternate parity from blk = 0)
    auto pstep = [&](auto par_c, auto t_c, int base, bool valid, const uint8_t* blk_base, const SW (&cur)[TN]) {
        constexpr int PAR = decltype(par_c)::value;
        constexpr int T = decltype(t_c)::value;
        w_issue(std::integral_constant<int, (4 * PAR + T + kAhead) % kSlots>{}, base + T + kAhead);
        __builtin_amdgcn_sched_barrier(0);
        if (valid) compute(t_c, std::integral_constant<int, (4 * PAR + T) % kSlots>{}, blk_base, cur);
        __builtin_amdgcn_sched_barrier(0);
    };
    // one 512-K block (x = blk, LDS buffer PAR = blk % 2): chunks 4 (sb0 + blk)
    // .. +3 with scales cur; prefetches the next block's scales into nxt and
    // its activations into registers, and stores those to the other buffer.
    auto block = [&](auto par_c, int blk, const SW (&cur)[TN], SW (&nxt)[TN]) {
        constexpr int PAR = decltype(par_c)::value;
        const int base = 4 * (sb0 + blk);
        const bool valid = blk < own;
        const int nsb = min(sb0 + blk + 1, sbmax);
        lds_barrier();
        a_issue(nsb);
#pragma unroll
        for (int tt = 0; tt < TN; ++tt) nxt[tt] = load_scale_block<FMT>(rs[tt], soff, nsb);
        const uint8_t* blk_base = ring + PAR * kBlk;
        pstep(par_c, std::integral_constant<int, 0>{}, base, valid, blk_base, cur);
        pstep(par_c, std::integral_constant<int, 1>{}, base, valid, blk_base, cur);
        pstep(par_c, std::integral_constant<int, 2>{}, base, valid, blk_base, cur);
        pstep(par_c, std::integral_constant<int, 3>{}, base, valid, blk_base, cur);
        a_store(1 - PAR);
    };

    const int c0 = 4 * sb0;
    a_issue(min(sb0, sbmax));
#pragma unroll
    for (int tt = 0; tt < TN; ++tt) sa[tt] = load_scale_block<FMT>(rs[tt], soff, min(sb0, sbmax));
    w_issue(std::integral_constant<int, 0>{}, c0);
    w_issue(std::integral_constant<int, 1>{}, c0 + 1);
    w_issue(std::integral_constant<int, 2>{}, c0 + 2);
    a_store(0);
    int blk = 0;
    for (; blk + 1 < nblk; blk += 2) {
        block(std::integral_constant<int, 0>{}, blk, sa, sbs);
        block(std::integral_constant<int, 1>{}, blk + 1, sbs, sa);
    }
    if (blk < nblk) block(std::integral_constant<int, 0>{}, blk, sa, sbs);

    if constexpr (NWK > 1) {
        __shared__ f32x4 red[(NWK - 1) * NWN * TN * MB * kLanes];
        if (wk > 0) {
#pragma unroll
            for (int tt = 0; tt < TN; ++tt)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    red[((((wk - 1) * NWN + wn) * TN + tt) * MB + mb) * kLanes + lane] = acc[tt][mb];
        }
        __syncthreads();
        if (wk == 0)
            for (int g = 1; g < NWK; ++g)
#pragma unroll
                for (int tt = 0; tt < TN; ++tt)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[tt][mb] += red[((((g - 1) * NWN + wn) * TN + tt) * MB + mb) * kLanes + lane];
    }
    // the waves of K group 0 hold the workgroup's sums
    if constexpr (MOE) {
        if (wk != 0) return;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = mb * 16 + r;
            if (m >= M) continue;
            const int id = moe.ids[row0 + m];
            if (id < 0 || id >= moe.out_rows) continue;
            const float w = (moe.topw ? moe.topw[id] : 1.0f) * alpha;
#pragma unroll
            for (int tt = 0; tt < TN; ++tt) store_frag<ACT>(C, acc[tt][mb] * w, id, (tile0 + tt) * kTileN + 4 * j,
                                                            moe.out_rows, N);
        }
        return;
    }
    if (P == nullptr) {
        if (wk != 0) return;
#pragma unroll
        for (int tt = 0; tt < TN; ++tt)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                store_frag<ACT>(C, acc[tt][mb] * alpha, mb * 16 + r, (tile0 + tt) * kTileN + 4 * j, M, N);
        return;
    }
    // K split: partials, then the group's last workgroup writes the output
    if (wk == 0) {
        const __amdgpu_buffer_rsrc_t pl = split_plane(P, ks, M, N);
#pragma unroll
        for (int tt = 0; tt < TN; ++tt)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                store_partial(pl, acc[tt][mb], mb * 16 + r, (tile0 + tt) * kTileN + 4 * j, M, N);
    }
    const int n_begin = grp * (TN * NWN) * kTileN;
    split_finish<ACT, 64 * NWN * NWK>(P, C, M, N, S, grp, 0, M, n_begin, min(N, n_begin + TN * NWN * kTileN), alpha,
                                      tag);
}

// Y = alpha x the sum over s of the S partial products P[s][M][N] (in order
// s = 0, 1, ...), rounded to the output type.  Four consecutive elements of
// the flattened [M][N] array per thread.
template <int ACT>
__global__ __launch_bounds__(256) void reduce_partials(const float* __restrict__ P, uint16_t* __restrict__ C,
                                                       int64_t total, int S, float alpha) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= total) return;
    if (e + 3 < total) {
        f32x4 v = *reinterpret_cast<const f32x4*>(P + e);
        for (int s = 1; s < S; ++s) v += *reinterpret_cast<const f32x4*>(P + (size_t)s * total + e);
        v *= alpha;
        u32x2 o = {pack_out<ACT>(v.x, v.y), pack_out<ACT>(v.z, v.w)};
        *reinterpret_cast<u32x2*>(C + e) = o;
    } else {
        for (int64_t x = e; x < total; ++x) {
            float v = P[x];
            for (int s = 1; s < S; ++s) v += P[(size_t)s * total + x];
            v *= alpha;
            C[x] = (uint16_t)(pack_out<ACT>(v, 0.f) & 0xFFFF);
        }
    }
}

// ----------------------------------------------------------- prefill GEMM
// Larger m.  A workgroup of four or eight waves computes a BM (m) x BN (n)
// tile with its waves in a WM x WN grid (a wave owns MBW 16-row m-blocks and
// TNW n-tiles), over a K range (the whole K, or 1/S of it with FP32
// partials).  Eight waves run two per SIMD, so one wave's dequant and memory
// instructions issue while the other's matrix instructions execute.
// Activations go global -> LDS by DMA (three chunk buffers in rotation,
// XOR-swizzled by row: conflict-free fragment reads; the Petit blog,
// "Mastering the memory hierarchy"), so they take no registers; codes go
// global -> registers through a 4-slot ring, three chunks ahead; scales one
// 512-K block ahead.  Per 128-K chunk c (four MFMA steps i = 0..3), with the
// activation fragments of each step read from LDS one step ahead:
//   issue the code blocks of chunk c+3;
//   steps 0..2 of chunk c, each reading the fragments of the next step;
//   wait for this wave's DMA of chunk c+1, then barrier: every wave is done
//     with chunk c's buffer and chunk c+1 is in LDS;
//   DMA chunk c+3 into chunk c's buffer (two chunks of time to land);
//   step 3 of chunk c, reading step 0 of chunk c+1.
// So no fragment read waits on its own step's products, and the one barrier
// per chunk sits where three steps' products are still in flight.
template <int FMT, int ACT, int WM, int WN, int MBW, int TNW, bool KTAIL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_prefill(const uint16_t* __restrict__ A,
                                                            const u32x4* __restrict__ wq,
                                                            const uint8_t* __restrict__ sq, uint16_t* __restrict__ C,
                                                            float* __restrict__ P, int M, int N, int K, int KB,
                                                            int SB, int NT, int S, float alpha) {
    static_assert(WM * WN == 4 || WM * WN == 8, "four or eight waves");
    typedef u32x4 SW;
    constexpr int kThreads = 64 * WM * WN;
    constexpr int BM = WM * MBW * 16;          // m rows per workgroup
    constexpr int BNT = WN * TNW;              // n-tiles per workgroup
    constexpr int kBuf = BM * 256;             // one LDS activation buffer (BM x 128 K x 2 B)
    constexpr int kStage = BM * 16 / kThreads;  // 16-byte activation pieces per thread per chunk
    static_assert(kStage * kThreads == BM * 16, "whole pieces per thread");
    constexpr int kScaleBlockBytes = scale_block_bytes<FMT>();
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[3 * kBuf];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, j = lane >> 4;
    const int wm = wave % WM, wn = wave / WM;

    // work item: K split ks (innermost), then an XCD-banded (m-tile, n-group) order
    const int MT = (M + BM - 1) / BM, NG = (NT + BNT - 1) / BNT;
    const int ks = blockIdx.x % S;
    const int item = blockIdx.x / S;
    const int total = MT * NG;
    int L = item;
    if (total % kXcdCount == 0 && S == 1)
        L = (item % kXcdCount) * (total / kXcdCount) + item / kXcdCount;
    const int mt = L % MT, ng = L / MT;
    const int m0 = mt * BM;
    const int tile0 = ng * BNT + wn * TNW;
    const int sb0 = (ks * SB) / S, sb1 = ((ks + 1) * SB) / S;
    const int c0 = 4 * sb0, clast = 4 * sb1 - 1;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)(M * K * 2));
    const int soff = scale_lane_offset<FMT>(r, j);
    __amdgpu_buffer_rsrc_t rw[TNW], rs[TNW];
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) {
        const int t = min(tile0 + tt, NT - 1);
        rw[tt] = make_rsrc(reinterpret_cast<const uint8_t*>(wq) + (size_t)t * KB * 1024, (uint32_t)KB * 1024u);
        rs[tt] = make_rsrc(sq + (size_t)t * SB * kScaleBlockBytes, (uint32_t)(SB * kScaleBlockBytes));
    }

    // Activations move HBM/L2 -> LDS by DMA (buffer loads that write LDS, no
    // registers): piece q of a wave is one 1 KiB instruction, lane l writing
    // the 16 bytes at LDS slot p = q * kThreads + 64 * wave + l of the chunk
    // buffer (row p / 16, physical column p % 16).  The tile is XOR-swizzled
    // by row (physical column = logical column ^ (row % 16): conflict-free
    // fragment reads; the Petit blog, "Mastering the memory hierarchy"), so
    // the lane fetches logical column (p % 16) ^ (row % 16) of its row.
    uint32_t aoff[kStage];
    int acol[kStage];
#pragma unroll
    for (int q = 0; q < kStage; ++q) {
        const int idx = tid + kThreads * q;
        const int row = idx >> 4, col = (idx & 15) ^ (row & 15);
        acol[q] = col;
        aoff[q] = (uint32_t)((m0 + row) * K + col * 8) * 2u;
    }
    // chunk -> LDS buffer at byte offset buf (three buffers in rotation).
    // A prefetch past the range repeats the last chunk into a buffer nobody
    // reads again.
    auto a_dma = [&](int chunk, int buf) {
        chunk = min(chunk, clast);
#pragma unroll
        for (int q = 0; q < kStage; ++q) {
            const int k = chunk * kChunkK + acol[q] * 8;
            const uint32_t off = aoff[q] + (uint32_t)(chunk * kChunkK) * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(lds_a + buf + (q * kThreads + 64 * wave) * 16), 16,
                (!KTAIL || k < K) ? off : kOutOfRange, 0, 0, 0);
        }
    };
    u32x4 wr[4][TNW];
    auto w_issue = [&](auto slot_c, int chunk) {
        constexpr int SL = decltype(slot_c)::value;
        chunk = min(chunk, clast);
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt)
            wr[SL][tt] = __builtin_amdgcn_raw_buffer_load_b128(rw[tt], lane * 16, chunk * 1024, kLoadReused);
    };
    // Barrier between the waves' LDS accesses.  Written without a fence: a
    // workgroup fence would also make every wave wait for its newest LDS DMA
    // (issued one chunk earlier), which the schedule waits for one chunk
    // later, explicitly (kYounger below).  The waits here cover this wave's
    // fragment reads; the memory clobbers keep LDS accesses on their side.
    auto lds_barrier = [] {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // this lane's fragments (16-byte column 4 I + j of its rows) of step I
    // of the chunk in the LDS buffer at byte offset buf
    auto read_frags = [&](auto i_c, int buf, u32x4 (&a)[MBW]) {
        constexpr int I = decltype(i_c)::value;
        const uint8_t* base = lds_a + buf + (wm * MBW * 16 + r) * 256 + (((4 * I + j) ^ r) << 4);
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) a[mb] = *reinterpret_cast<const u32x4*>(base + mb * 16 * 256);
    };

    f32x4 acc[TNW][MBW];
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) acc[tt][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Dequantized weight fragments of the current MFMA step (one per n-tile).
    // Each step's products use them while the next step's codes are
    // dequantized, and the scheduler is asked to alternate one matrix
    // instruction with two vector instructions: the dequant runs while the
    // matrix core works, inside each wave.
    u32x4 wcur[TNW];
    // Products of step I of chunk position T with fragments a and wcur, and
    // the dequant of the next step (chunk position NT, step NI, its scales
    // sn: the next 512-K block's after the last step of a block) into wcur.
    auto mma = [&](auto t_c, auto i_c, const u32x4 (&a)[MBW], const SW (&sn)[TNW]) {
        constexpr int T = decltype(t_c)::value;
        constexpr int I = decltype(i_c)::value;
        constexpr int NT = I == 3 ? (T + 1) % 4 : T;
        constexpr int NI = (I + 1) % 4;
        u32x4 wn[TNW];
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt) wn[tt] = dequant_step<FMT, NT, NI, ACT>(wr[NT][tt], sn[tt]);
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt)
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) acc[tt][mb] = mfma<ACT>(wcur[tt], a[mb], acc[tt][mb]);
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt) wcur[tt] = wn[tt];
    };
    auto interleave = [] {
        __builtin_amdgcn_sched_group_barrier(0x100, MBW, 0);  // next step's fragment reads first
#pragma unroll
        for (int q = 0; q < MBW * TNW; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // Each step's fragments are read one step ahead (two fragment sets).
    u32x4 fa[MBW], fb[MBW];
    // LDS buffers (byte offsets): chunk c in b_cur, c+1 in b_nxt, the DMA of
    // c+2 in flight to b_far.
    int b_cur = 0, b_nxt = kBuf, b_far = 2 * kBuf;
    // Vector-memory instructions certainly issued after the DMA of chunk c+1
    // by the time chunk c waits for it: the DMA of chunk c+2.  Loads complete
    // in issue order, so at most this many may then be outstanding.  (The code
    // loads in between are not counted: the compiler deletes the prefetches
    // of the last block whose results are never used.)
    constexpr int kYounger = kStage;
    // chunk c = base + T (T = c % 4, also its code-ring slot); fa holds step
    // 0's fragments and wcur its dequantized weights on entry; nxt are the
    // next block's scales (used by the dequant ahead of the block's end)
    auto pstep = [&](auto t_c, int base, const SW (&cur)[TNW], const SW (&nxt)[TNW]) {
        constexpr int T = decltype(t_c)::value;
        w_issue(std::integral_constant<int, (T + 3) % 4>{}, base + T + 3);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(I1{}, b_cur, fb);
        mma(t_c, I0{}, fa, cur);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(I2{}, b_cur, fa);
        mma(t_c, I1{}, fb, cur);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(I3{}, b_cur, fb);
        mma(t_c, I2{}, fa, cur);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        // this wave's DMA of chunk c+1 has landed; after the barrier every
        // wave's has, and every wave has read all of chunk c
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kYounger) : "memory");
        lds_barrier();
        a_dma(base + T + 3, b_cur);  // into the buffer chunk c just freed
        const int b_free = b_cur;
        b_cur = b_nxt;
        b_nxt = b_far;
        b_far = b_free;
        __builtin_amdgcn_sched_barrier(0);
        read_frags(I0{}, b_cur, fa);
        if constexpr (T == 3) mma(t_c, I3{}, fb, nxt);
        else mma(t_c, I3{}, fb, cur);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
    };
    SW sa[TNW], sbs[TNW];
    auto block = [&](int sbx, const SW (&cur)[TNW], SW (&nxt)[TNW]) {
        const int base = 4 * sbx;
        const int nsb = min(sbx + 1, sb1 - 1);
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt) nxt[tt] = load_scale_block<FMT, kLoadReused>(rs[tt], soff, nsb);
        pstep(I0{}, base, cur, nxt);
        pstep(I1{}, base, cur, nxt);
        pstep(I2{}, base, cur, nxt);
        pstep(I3{}, base, cur, nxt);
    };

    // prologue: code blocks c0 .. c0+2 and the DMA of chunks c0 .. c0+2 in
    // flight (in the order the steady state expects); chunk c0 in LDS first.
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) sa[tt] = load_scale_block<FMT, kLoadReused>(rs[tt], soff, sb0);
    w_issue(I0{}, c0);
    a_dma(c0, 0);
    w_issue(I1{}, c0 + 1);
    a_dma(c0 + 1, kBuf);
    w_issue(I2{}, c0 + 2);
    a_dma(c0 + 2, 2 * kBuf);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kStage) : "memory");  // DMA of chunk c0
    lds_barrier();
    read_frags(I0{}, b_cur, fa);
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) wcur[tt] = dequant_step<FMT, 0, 0, ACT>(wr[0][tt], sa[tt]);
    int sb = sb0;
    for (; sb + 1 < sb1; sb += 2) {
        block(sb, sa, sbs);
        block(sb + 1, sbs, sa);
    }
    if (sb < sb1) block(sb, sa, sbs);
    // no DMA may still write this workgroup's LDS after it exits
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
    for (int tt = 0; tt < TNW; ++tt)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            const int m = m0 + wm * MBW * 16 + mb * 16 + r, n0 = (tile0 + tt) * kTileN + 4 * j;
            if (P == nullptr) {
                store_frag<ACT>(C, acc[tt][mb] * alpha, m, n0, M, N);
            } else if (m < M) {  // FP32 partials for the reduce kernel (plain stores: measured faster here)
                float* dst = P + ((size_t)ks * M + m) * N + n0;
                if ((N & 3) == 0 && n0 + 3 < N) {
                    *reinterpret_cast<f32x4*>(dst) = acc[tt][mb];
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (n0 + e < N) dst[e] = acc[tt][mb][e];
                }
            }
        }
}

// ------------------------------------------------------ tall prefill GEMM
// 256-row tiles: a workgroup of NW waves computes a 256 (m) x 16 NW TNW (n)
// tile, each wave over all 16 m-blocks and TNW n-tiles, so every weight is
// dequantized once per 256 rows (half as often as with 128-row tiles) and
// every dequantized fragment feeds 16 products.  Activations: two 64 KiB LDS
// chunk buffers (256 rows x 128 K, XOR-swizzled by row as in gemm_prefill),
// filled by DMA one chunk ahead; codes in a two-slot ring two chunks ahead.
// An MFMA step (32 K) runs in 16 / FG groups of FG m-blocks whose fragments
// are read one group ahead; the next step's weights are dequantized during
// the current step.  Per 128-K chunk c (LDS buffer c % 2):
//   step 0, each group also issuing its share of the DMA of chunk c+1 into
//     the other buffer (freed by the previous barrier): spread over the
//     step, the DMA competes less with the fragment reads than in one burst
//     (gate_up 3.4 % faster at m = 256, 1.8 % at m = 512);
//   steps 1..2 and step 3 up to its last group;
//   wait for every load issued so far (the DMA of chunk c+1, the codes of
//     chunk c+1), barrier: chunk c+1 is in LDS and every wave has read all
//     of chunk c;
//   codes of chunk c+2 into chunk c's ring slot;
//   the last group of step 3, reading the first group of chunk c+1.
template <int FMT, int ACT, int NW, int TNW, int FG, bool KTAIL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void gemm_prefill_tall(
    const uint16_t* __restrict__ A, const u32x4* __restrict__ wq, const uint8_t* __restrict__ sq,
    uint16_t* __restrict__ C, float* __restrict__ P, int M, int N, int K, int KB, int SB, int NT, int S,
    float alpha) {
    typedef u32x4 SW;
    constexpr int kThreads = 64 * NW, MBW = 16, BM = 256, BNT = NW * TNW;
    constexpr int kGroups = MBW / FG;           // fragment groups per MFMA step
    constexpr int kBuf = BM * 256;              // one LDS activation buffer (BM x 128 K x 2 B)
    constexpr int kStage = BM * 16 / kThreads;  // 16-byte activation pieces per thread per chunk
    constexpr int kScaleBlockBytes = scale_block_bytes<FMT>();
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert((kGroups == 2 || kGroups == 4) && kGroups % TNW == 0, "group / n-tile split");
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * kBuf];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, j = lane >> 4;

    // work item: K split ks (innermost), then an XCD-banded (m-tile, n-group) order
    const int MT = (M + BM - 1) / BM, NG = (NT + BNT - 1) / BNT;
    const int ks = blockIdx.x % S;
    const int item = blockIdx.x / S;
    const int total = MT * NG;
    int L = item;
    if (total % kXcdCount == 0 && S == 1)
        L = (item % kXcdCount) * (total / kXcdCount) + item / kXcdCount;
    const int mt = L % MT, ng = L / MT;
    const int m0 = mt * BM;
    const int tile0 = ng * BNT + wave * TNW;
    const int sb0 = (ks * SB) / S, sb1 = ((ks + 1) * SB) / S;
    const int c0 = 4 * sb0, clast = 4 * sb1 - 1;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)(M * K * 2));
    const int soff = scale_lane_offset<FMT>(r, j);
    __amdgpu_buffer_rsrc_t rw[TNW], rs[TNW];
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) {
        const int t = min(tile0 + tt, NT - 1);
        rw[tt] = make_rsrc(reinterpret_cast<const uint8_t*>(wq) + (size_t)t * KB * 1024, (uint32_t)KB * 1024u);
        rs[tt] = make_rsrc(sq + (size_t)t * SB * kScaleBlockBytes, (uint32_t)(SB * kScaleBlockBytes));
    }

    // Activation DMA: piece q of the thread is LDS slot p = tid + kThreads q
    // of the chunk buffer (row p / 16, physical column p % 16, logical column
    // (p % 16) ^ (row % 16)); rows step by a multiple of 16 with q, so the
    // logical column is the same for every piece of the thread.  Offsets are
    // 32-bit unsigned: the host bounds round_up(M, 128) * K * 2 below 2^31,
    // so rows below M are exact; a padding row of the last 256-row tile may
    // wrap, and its load then reads zeros or another row's values that only
    // feed outputs at rows >= M, which are never stored.
    const int arow = tid >> 4, acol = (tid & 15) ^ (arow & 15);
    const uint32_t aoff = ((uint32_t)(m0 + arow) * (uint32_t)K + (uint32_t)(acol * 8)) * 2u;
    const uint32_t arow_step = (uint32_t)(kThreads / 16 * K) * 2u;
    auto a_dma = [&](int chunk, int buf) {
        chunk = min(chunk, clast);
        const bool in_k = !KTAIL || chunk * kChunkK + acol * 8 < K;
        const uint32_t off0 = aoff + (uint32_t)(chunk * kChunkK) * 2u;
#pragma unroll
        for (int q = 0; q < kStage; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(lds_a + buf + (q * kThreads + 64 * wave) * 16), 16,
                in_k ? off0 + q * arow_step : kOutOfRange, 0, 0, 0);
    };
    auto a_dma_part = [&](int chunk, int buf, auto g_c) {
        constexpr int G = decltype(g_c)::value;
        chunk = min(chunk, clast);
        // a chunk past K reads zeros: its offsets start at 2^31 and stay
        // past the buffer's range (below 2^31) for every piece
        const uint32_t off0 = (!KTAIL || chunk * kChunkK + acol * 8 < K)
                                  ? aoff + (uint32_t)(chunk * kChunkK) * 2u : kOutOfRange;
#pragma unroll
        for (int q = G * (kStage / kGroups); q < (G + 1) * (kStage / kGroups); ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(lds_a + buf + (q * kThreads + 64 * wave) * 16), 16,
                off0 + q * arow_step, 0, 0, 0);
    };
    u32x4 wr[2][TNW];
    auto w_issue = [&](auto slot_c, int chunk) {
        constexpr int SL = decltype(slot_c)::value;
        chunk = min(chunk, clast);
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt)
            wr[SL][tt] = __builtin_amdgcn_raw_buffer_load_b128(rw[tt], lane * 16, chunk * 1024, kLoadReused);
    };
    auto lds_barrier = [] {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // fragments of group G (m-blocks FG G .. FG G + FG - 1) of step I of the
    // chunk in the LDS buffer at byte offset buf
    auto read_group = [&](auto i_c, auto g_c, int buf, u32x4 (&a)[FG]) {
        constexpr int I = decltype(i_c)::value;
        constexpr int G = decltype(g_c)::value;
        const uint8_t* base = lds_a + buf + (G * FG * 16 + r) * 256 + (((4 * I + j) ^ r) << 4);
#pragma unroll
        for (int mb = 0; mb < FG; ++mb) a[mb] = *reinterpret_cast<const u32x4*>(base + mb * 16 * 256);
    };

    f32x4 acc[TNW][MBW];
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) acc[tt][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wcur[TNW], wnx[TNW];
    // Products of group G with fragments a and wcur; n-tile G / (kGroups /
    // TNW) of the next step (chunk position NTP, step NI, scales sn) is
    // dequantized into wnx in the group that starts its share.
    auto group = [&](auto t_c, auto i_c, auto g_c, const u32x4 (&a)[FG], const SW (&sn)[TNW]) {
        constexpr int T = decltype(t_c)::value;
        constexpr int I = decltype(i_c)::value;
        constexpr int G = decltype(g_c)::value;
        constexpr int NTP = I == 3 ? (T + 1) % 4 : T;
        constexpr int NI = (I + 1) % 4;
        if constexpr (G % (kGroups / TNW) == 0) {
            constexpr int tt = G / (kGroups / TNW);
            wnx[tt] = dequant_step<FMT, NTP, NI, ACT>(wr[NTP % 2][tt], sn[tt]);
        }
#pragma unroll
        for (int mb = 0; mb < FG; ++mb)
#pragma unroll
            for (int tt = 0; tt < TNW; ++tt)
                acc[tt][G * FG + mb] = mfma<ACT>(wcur[tt], a[mb], acc[tt][G * FG + mb]);
    };
    auto interleave = [] {
        __builtin_amdgcn_sched_group_barrier(0x100, FG, 0);  // the next group's fragment reads first
#pragma unroll
        for (int q = 0; q < FG * TNW; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    u32x4 fa[FG], fb[FG];  // fragments of the even / odd groups
    int b_cur = 0, b_nxt = kBuf;
    // group G of MFMA step I of chunk position T (chunk base + T); on entry
    // its fragments are in fa (G even) or fb (G odd)
    auto one_group = [&](auto t_c, auto i_c, auto g_c, int base, const SW (&sn)[TNW]) {
        constexpr int T = decltype(t_c)::value;
        constexpr int I = decltype(i_c)::value;
        constexpr int G = decltype(g_c)::value;
        u32x4(&cur_f)[FG] = G % 2 == 0 ? fa : fb;
        u32x4(&nxt_f)[FG] = G % 2 == 0 ? fb : fa;
        if constexpr (G + 1 < kGroups) {
            read_group(i_c, std::integral_constant<int, G + 1>{}, b_cur, nxt_f);
        } else if constexpr (I < 3) {
            read_group(std::integral_constant<int, I + 1>{}, I0{}, b_cur, nxt_f);
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            w_issue(std::integral_constant<int, T % 2>{}, base + T + 2);
            const int b_free = b_cur;
            b_cur = b_nxt;
            b_nxt = b_free;
            __builtin_amdgcn_sched_barrier(0);
            read_group(I0{}, I0{}, b_cur, nxt_f);
        }
        if constexpr (I == 0) a_dma_part(base + T + 1, b_nxt, g_c);
        group(t_c, i_c, g_c, cur_f, sn);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto step = [&](auto t_c, auto i_c, int base, const SW (&cur)[TNW], const SW (&nxt)[TNW]) {
        constexpr int T = decltype(t_c)::value;
        constexpr int I = decltype(i_c)::value;
        const SW(&sn)[TNW] = T == 3 && I == 3 ? nxt : cur;
        one_group(t_c, i_c, I0{}, base, sn);
        one_group(t_c, i_c, I1{}, base, sn);
        if constexpr (kGroups > 2) {
            one_group(t_c, i_c, I2{}, base, sn);
            one_group(t_c, i_c, I3{}, base, sn);
        }
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt) wcur[tt] = wnx[tt];
    };
    auto chunk = [&](auto t_c, int base, const SW (&cur)[TNW], const SW (&nxt)[TNW]) {
        step(t_c, I0{}, base, cur, nxt);
        step(t_c, I1{}, base, cur, nxt);
        step(t_c, I2{}, base, cur, nxt);
        step(t_c, I3{}, base, cur, nxt);
    };
    SW sa[TNW], sbs[TNW];
    auto block = [&](int sbx, const SW (&cur)[TNW], SW (&nxt)[TNW]) {
        const int base = 4 * sbx;
        const int nsb = min(sbx + 1, sb1 - 1);
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt) nxt[tt] = load_scale_block<FMT, kLoadReused>(rs[tt], soff, nsb);
        chunk(I0{}, base, cur, nxt);
        chunk(I1{}, base, cur, nxt);
        chunk(I2{}, base, cur, nxt);
        chunk(I3{}, base, cur, nxt);
    };

    // prologue: codes of chunks c0, c0+1 and the DMA of chunk c0 (chunk
    // c0+1's comes with step 0 of chunk c0)
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) sa[tt] = load_scale_block<FMT, kLoadReused>(rs[tt], soff, sb0);
    w_issue(I0{}, c0);
    w_issue(I1{}, c0 + 1);
    a_dma(c0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    read_group(I0{}, I0{}, b_cur, fa);
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) wcur[tt] = dequant_step<FMT, 0, 0, ACT>(wr[0][tt], sa[tt]);
    int sb = sb0;
    for (; sb + 1 < sb1; sb += 2) {
        block(sb, sa, sbs);
        block(sb + 1, sbs, sa);
    }
    if (sb < sb1) block(sb, sa, sbs);
    // no DMA may still write this workgroup's LDS after it exits
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
    for (int tt = 0; tt < TNW; ++tt)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            const int m = m0 + mb * 16 + r, n0 = (tile0 + tt) * kTileN + 4 * j;
            if (P == nullptr) {
                store_frag<ACT>(C, acc[tt][mb] * alpha, m, n0, M, N);
            } else if (m < M) {  // FP32 partials for the reduce kernel
                float* dst = P + ((size_t)ks * M + m) * N + n0;
                if ((N & 3) == 0 && n0 + 3 < N) {
                    *reinterpret_cast<f32x4*>(dst) = acc[tt][mb];
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (n0 + e < N) dst[e] = acc[tt][mb][e];
                }
            }
        }
}

// ------------------------------------------------------------ quantizer
// Offline quantizer: BF16 weights -> E2M1 codes (two per byte, element 2j in
// the low nibble) and one scale byte per G-element block, in the source
// order fp4_repack takes.  Block scaling with the block's largest magnitude
// and nearest-grid rounding (mhpq.cn FP4 GEMM article, sections 2.1, 2.2); an
// all-zero block never gets a zero NVFP4 scale (section 5.2).  Every decision
// is taken in IEEE FP32 with correctly rounded operations:
//   NVFP4: scale byte = E4M3 round-to-nearest-even of (amax / 6) / alpha,
//          saturated at 448, at least 2^-9 (byte 1);
//   MXFP4: scale byte = clamp(floor(log2(amax / alpha)) - 2 + 127, 0, 254),
//          255 never; byte 0 is the scale 2^-127 (an FP32 subnormal) and
//          its block is rounded like any other;
//   S = alpha * scale, q = |x| / S, code = nearest E2M1 value to q with
//   ties to the even mantissa bit, saturating at 6; the sign bit only on
//   non-zero codes.  Zero and NaN elements give code 0 (amax ignores NaN);
//   infinities give the largest scale.
// One thread per block of G elements: the blocks of a row are consecutive
// in memory, so a wave reads and writes contiguous bytes.

// E4M3 byte of the nearest value to t >= 0 (ties to the even mantissa),
// saturating at 448 (byte 0x7E).
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
    if (!(t < 448.0f)) return 0x7Eu;
    const uint32_t b = __float_as_uint(t);
    const int e = int((b >> 23) & 0xFF) - 127;
    if (e >= -6) {  // E4M3 normal range: keep 3 mantissa bits, round to nearest even
        const uint32_t m3 = (b >> 20) & 7u, rem = b & 0xFFFFFu;
        const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ? 1u : 0u;
        return ((uint32_t)(e + 7) << 3) + m3 + up;  // a mantissa carry moves into the exponent
    }
    // subnormal range: value = f x 2^-9, f = round-half-even(t x 2^9) in 0 .. 8
    // (f = 8 is 2^-6, whose byte 0x08 is the same integer)
    return (uint32_t)rintf(t * 512.0f);
}

__device__ __forceinline__ float e4m3_decode(uint32_t byte) {
    const uint32_t e = byte >> 3, m = byte & 7u;
    return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

template <int FMT>
// Output rows hold gpr_out >= gpr_in blocks: blocks past the input row's
// gpr_in are written as zero blocks (codes 0, scale byte 0), which pads K for
// the native FP4 path; gpr_out == gpr_in is the canonical layout.
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ W, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int64_t groups, float alpha,
                                                       int64_t gpr_in, int64_t gpr_out) {
    constexpr int G = FMT == 0 ? 16 : 32;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= groups) return;
    const int64_t row = g / gpr_out, blk = g - row * gpr_out;
    if (blk >= gpr_in) {
        if constexpr (FMT == 0) *reinterpret_cast<u32x2*>(codes + g * (G / 2)) = u32x2{0u, 0u};
        else *reinterpret_cast<u32x4*>(codes + g * (G / 2)) = u32x4{0u, 0u, 0u, 0u};
        scales[g] = 0;
        return;
    }
    u32x4 v[G / 8];
    const u32x4* src = reinterpret_cast<const u32x4*>(W + (row * gpr_in + blk) * G);
#pragma unroll
    for (int i = 0; i < G / 8; ++i) v[i] = src[i];
    float x[G];
#pragma unroll
    for (int i = 0; i < G / 2; ++i) {
        const uint32_t d = v[i / 4][i % 4];
        x[2 * i] = __uint_as_float(d << 16);
        x[2 * i + 1] = __uint_as_float(d & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) amax = fmaxf(amax, fabsf(x[i]));  // fmaxf drops NaN operands
    uint32_t sb;
    float sval;
    if constexpr (FMT == 0) {
        sb = e4m3_rne(__fdiv_rn(__fdiv_rn(amax, 6.0f), alpha));
        sb = sb == 0 ? 1u : sb;
        sval = e4m3_decode(sb);
    } else {
        const float t = __fdiv_rn(amax, alpha);
        const int ef = int((__float_as_uint(t) >> 23) & 0xFF);  // 0: zero or below 2^-126; 255: infinite
        sb = ef == 255 ? 254u : (uint32_t)max(ef - 2, 0);
        // 2^(sb - 127); byte 0 is 2^-127, the FP32 subnormal 0x00400000
        sval = __uint_as_float(sb != 0 ? sb << 23 : 0x00400000u);
    }
    const float S = __fmul_rn(alpha, sval);
    uint32_t out[G / 8];
#pragma unroll
    for (int w = 0; w < G / 8; ++w) out[w] = 0;
    if constexpr (FMT == 0) {
        // alpha a power of two: S = 2^es x M with M in [1, 2) of at most 4
        // significant bits (the E4M3 mantissa).  y = x x rcp(M) is within 4
        // ulps of x / M; a quotient that is not a midpoint (at most 3
        // significant bits) lies at least 2^-8 / 300 relative, over 100 ulps,
        // from every midpoint (as for the thresholds below), so y decides like
        // x / M once values within 4 ulps of a 3-significant-bit number are
        // snapped to it (that restores an exact midpoint and moves no other
        // quotient across one).  Then the FP32 -> FP4 convert with scale 2^es
        // rounds y / 2^es as the rule does (see the MXFP4 branch).
        const uint32_t ab = __float_as_uint(alpha), Sb = __float_as_uint(S);
        if ((ab & 0x007FFFFFu) == 0u && ((ab >> 23) & 0xFF) != 0u && ((Sb >> 23) & 0xFF) != 0u) {
            const float sc = __uint_as_float(Sb & 0x7F800000u);  // 2^es (S is normal: >= 2^-109)
            const float r = __builtin_amdgcn_rcpf(__uint_as_float((Sb & 0x007FFFFFu) | 0x3F800000u));
            bool nan_any = false;
#pragma unroll
            for (int i = 0; i < G / 2; ++i) nan_any |= __builtin_isunordered(x[2 * i], x[2 * i + 1]);
            float y[G];
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const uint32_t yb = __float_as_uint(x[i] * r);
                const uint32_t y3 = (yb + 0x00100000u) & 0xFFE00000u;  // nearest with 3 significant bits
                y[i] = __uint_as_float(yb - y3 + 4u <= 8u ? y3 : yb);  // |yb - y3| <= 4
            }
#pragma unroll
            for (int w = 0; w < G / 8; ++w) {
                uint32_t o = 0;
                o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[8 * w + 0], y[8 * w + 1], sc, 0);
                o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[8 * w + 2], y[8 * w + 3], sc, 1);
                o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[8 * w + 4], y[8 * w + 5], sc, 2);
                o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[8 * w + 6], y[8 * w + 7], sc, 3);
                const uint32_t mag = o & 0x77777777u;
                out[w] = mag | (o & ((mag + 0x77777777u) & 0x88888888u));
            }
            if (nan_any) {
#pragma unroll
                for (int i = 0; i < G; ++i)
                    if (__builtin_isnan(x[i])) out[i / 8] &= ~(0xFu << (4 * (i % 8)));
            }
            *reinterpret_cast<u32x2*>(codes + g * (G / 2)) = u32x2{out[0], out[1]};
            scales[g] = (uint8_t)sb;
            return;
        }
    }
    if constexpr (FMT == 1) {
        // alpha a power of two: S = 2^es is one too, so q = |x| / S is exact
        // and the gfx950 FP32 -> FP4 convert with S as its (E8M0) scale gives
        // the nearest E2M1 code with ties to the even mantissa, saturating at
        // 6 (checked on the device against this rule for every BF16 value and
        // scale bytes 0 .. 254); it differs only in writing the sign bit on
        // codes of magnitude 0 and in converting NaN to code 7, both undone.
        const uint32_t ab = __float_as_uint(alpha);
        const int es = int((ab >> 23) & 0xFF) - 127 + int(sb) - 127;  // log2 S when alpha = 2^(exp)
        if ((ab & 0x007FFFFFu) == 0u && ((ab >> 23) & 0xFF) != 0u && es >= -127 && es <= 127) {
            const float sc = __uint_as_float((uint32_t)(es + 127) << 23);
            bool nan_any = false;
#pragma unroll
            for (int i = 0; i < G / 2; ++i) nan_any |= __builtin_isunordered(x[2 * i], x[2 * i + 1]);
#pragma unroll
            for (int w = 0; w < G / 8; ++w) {
                // FP32 operands (the BF16 values, exact): a bit cast of single
                // elements of the loaded vectors into the BF16 form was
                // mis-folded by clang into one element for all four converts
                uint32_t o = 0;
                o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, x[8 * w + 0], x[8 * w + 1], sc, 0);
                o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, x[8 * w + 2], x[8 * w + 3], sc, 1);
                o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, x[8 * w + 4], x[8 * w + 5], sc, 2);
                o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, x[8 * w + 6], x[8 * w + 7], sc, 3);
                // keep a nibble's sign bit only where its magnitude is non-zero
                // (magnitude + 7 carries into bit 3 exactly when it is >= 1)
                const uint32_t mag = o & 0x77777777u;
                out[w] = mag | (o & ((mag + 0x77777777u) & 0x88888888u));
            }
            if (nan_any) {
#pragma unroll
                for (int i = 0; i < G; ++i)
                    if (__builtin_isnan(x[i])) out[i / 8] &= ~(0xFu << (4 * (i % 8)));
            }
            *reinterpret_cast<u32x4*>(codes + g * (G / 2)) = u32x4{out[0], out[1], out[2], out[3]};
            scales[g] = (uint8_t)sb;
            return;
        }
    }
    // With alpha a power of two, S has at most 4 significant bits and x at
    // most 8, so q = fl(|x| / S) lies on the same side of every midpoint c
    // (at most 3 significant bits) as |x| does of c x S, which is exact in
    // FP32: a quotient that is not c differs from it by at least 2^-8 / 300
    // relative, far more than the half-ulp the division rounds by.  Then the
    // decision needs no division (S below 2^120 keeps 5 S finite; S of a
    // block with a non-zero element is at least about amax / 8 >= 2^-136,
    // so every threshold c x S is an exact FP32 value, subnormals included;
    // only an all-zero block's S can underflow to 0, and zero elements get
    // code 0 below whatever the thresholds are).
    const bool exact_thresholds = (__float_as_uint(alpha) & 0x007FFFFFu) == 0u && S < 0x1p120f;
    const float t0 = 0.25f * S, t1 = 0.75f * S, t2 = 1.25f * S, t3 = 1.75f * S, t4 = 2.5f * S, t5 = 3.5f * S,
                t6 = 5.0f * S;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const float ax = fabsf(x[i]);
        uint32_t c;
        if (exact_thresholds) {
            c = (uint32_t)(ax > t0) + (uint32_t)(ax >= t1) + (uint32_t)(ax > t2) + (uint32_t)(ax >= t3) +
                (uint32_t)(ax > t4) + (uint32_t)(ax >= t5) + (uint32_t)(ax > t6);
        } else {
            const float q = __fdiv_rn(ax, S);
            c = (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f) + (uint32_t)(q > 1.25f) + (uint32_t)(q >= 1.75f) +
                (uint32_t)(q > 2.5f) + (uint32_t)(q >= 3.5f) + (uint32_t)(q > 5.0f);
        }
        if (!(ax > 0.0f)) c = 0;  // zero or NaN (q = 0 or NaN)
        if (c != 0 && x[i] < 0.0f) c |= 8u;
        out[i / 8] |= c << (4 * (i % 8));
    }
    if constexpr (FMT == 0) {
        *reinterpret_cast<u32x2*>(codes + g * (G / 2)) = u32x2{out[0], out[1]};
    } else {
        *reinterpret_cast<u32x4*>(codes + g * (G / 2)) = u32x4{out[0], out[1], out[2], out[3]};
    }
    scales[g] = (uint8_t)sb;
}

// ------------------------------------------------------------ native FP4 GEMM
// The FP4 matrix-core path of gfx950 (the Petit blog's introduction: MI350
// multiplies FP4 natively).  Both operands are MXFP4: the weights in the
// native layout (fp4_native_repack; one 1 KiB block per 16-row tile and
// 128-K chunk, one 256-byte scale block per tile and 512 K), the activations
// quantized to MXFP4 by quantize_kernel<1> into rows of Kp / 2 code bytes
// and Kp / 32 scale bytes (K zero-padded to Kp = 512 multiple).  One
// v_mfma_scale_f32_16x16x128_f8f6f4 per (tile, m-block, chunk) multiplies
// 16 x 128 FP4 weights by 16 x 128 FP4 activations with one E8M0 scale per
// lane and operand (lane l = 16 j + r: row r, k = 32 j .. 32 j + 31 of the
// chunk; the weight scale is byte (chunk % 4) of the lane's scale dword, the
// activation scale the low byte after shifting by 8 j).
// Workgroup: four waves, WN n-groups x WM m-groups, a wave owns MBW m-blocks
// and TNW n-tiles.  The activations of one 512-K group (four chunks: BM rows x
// 256 code bytes + 16 scale bytes per row) go through registers into a
// double-buffered LDS tile one group ahead (one barrier per group; the
// 16-byte code slots are XOR-swizzled by row, so fragment reads are free of
// bank conflicts); the code blocks stream three chunks ahead in a four-slot
// register ring; K split over S workgroups as in the prefill kernel.
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int WM, int WN, int MBW, int TNW>
__global__ __launch_bounds__(256) void gemm_native(const uint8_t* __restrict__ Aq, const uint8_t* __restrict__ As,
                                                  const u32x4* __restrict__ wq, const uint8_t* __restrict__ sq,
                                                  uint16_t* __restrict__ C, float* __restrict__ P, int M, int N,
                                                  int KB, int NT, int S, float alpha) {
    static_assert(WM * WN == 4, "four waves");
    constexpr int BM = WM * MBW * 16;
    constexpr int BNT = WN * TNW;
    constexpr int kCodeBuf = BM * 256;              // one 512-K group of activation codes
    constexpr int kBuf = kCodeBuf + BM * 16;        // plus its scale bytes
    constexpr int kPieces = BM * 16 / 256;          // 16-byte code pieces per thread per group
    static_assert(kPieces >= 1 && BM * 16 % 256 == 0 && BM <= 256, "whole pieces");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBuf];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, j = lane >> 4;
    const int wm = wave % WM, wn = wave / WM;
    const int MT = (M + BM - 1) / BM, NG = (NT + BNT - 1) / BNT;
    const int ks = blockIdx.x % S, item = blockIdx.x / S;
    const int total = MT * NG;
    int L = item;
    if (total % kXcdCount == 0 && S == 1) L = (item % kXcdCount) * (total / kXcdCount) + item / kXcdCount;
    const int mt = L % MT, ng = L / MT;
    const int m0 = mt * BM, tile0 = ng * BNT + wn * TNW;
    const int QB = KB / 4;                          // 512-K groups
    const int q0 = (ks * QB) / S, q1 = ((ks + 1) * QB) / S;
    const int clast = 4 * q1 - 1;
    const int row_bytes = KB * 64, srow_bytes = KB * 4;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Aq, (uint32_t)(M * row_bytes));
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(As, (uint32_t)(M * srow_bytes));
    __amdgpu_buffer_rsrc_t rw[TNW], rs[TNW];
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) {
        const int t = min(tile0 + tt, NT - 1);
        rw[tt] = make_rsrc(reinterpret_cast<const uint8_t*>(wq) + (size_t)t * KB * 1024, (uint32_t)KB * 1024u);
        rs[tt] = make_rsrc(sq + (size_t)t * QB * 256, (uint32_t)QB * 256u);
    }

    // staging: code piece p of this thread = (row, 16-byte slot s of the
    // group's 256 bytes: chunk s / 4, lane group s % 4); threads 0 .. BM-1
    // also bring their row's 16 scale bytes
    u32x4 st[kPieces];
    u32x4 sst = u32x4{0u, 0u, 0u, 0u};
    auto a_issue = [&](int q) {
        q = min(q, q1 - 1);
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
            const int idx = tid + 256 * p, row = idx >> 4, slot = idx & 15;
            st[p] = __builtin_amdgcn_raw_buffer_load_b128(ra, (uint32_t)((m0 + row) * row_bytes + q * 256 + slot * 16),
                                                          0, 0);
        }
        if (tid < BM)
            sst = __builtin_amdgcn_raw_buffer_load_b128(rsa, (uint32_t)((m0 + tid) * srow_bytes + q * 16), 0, 0);
    };
    auto a_store = [&](int buf) {
        uint8_t* base = lds + buf * kBuf;
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
            const int idx = tid + 256 * p, row = idx >> 4, slot = idx & 15;
            *reinterpret_cast<u32x4*>(base + row * 256 + ((slot ^ (row & 15)) << 4)) = st[p];
        }
        if (tid < BM) *reinterpret_cast<u32x4*>(base + kCodeBuf + tid * 16) = sst;
    };
    u32x4 wr[4][TNW];
    auto w_issue = [&](auto slot_c, int chunk) {
        constexpr int SL = decltype(slot_c)::value;
        chunk = min(chunk, clast);
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt)
            wr[SL][tt] = __builtin_amdgcn_raw_buffer_load_b128(rw[tt], lane * 16, chunk * 1024, kLoadStream);
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

    // chunk T (0..3) of the group in LDS buffer `base`
    auto compute = [&](auto t_c, const uint8_t* base, const uint32_t (&wsc)[TNW]) {
        constexpr int T = decltype(t_c)::value;
        i32x8 a[MBW];
        int asc[MBW];
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            const int row = wm * MBW * 16 + mb * 16 + r;
            const u32x4 v = *reinterpret_cast<const u32x4*>(base + row * 256 + (((4 * T + j) ^ (row & 15)) << 4));
            a[mb] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            asc[mb] = (int)(*reinterpret_cast<const uint32_t*>(base + kCodeBuf + row * 16 + T * 4) >> (8 * j));
        }
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt) {
            const u32x4 w = wr[T][tt];
            const i32x8 b = i32x8{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                acc[tt][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a[mb], acc[tt][mb], 4, 4, T,
                                                                               (int)wsc[tt], 0, asc[mb]);
        }
    };
    uint32_t sa[TNW], sb[TNW];
    auto group = [&](int q, int buf, const uint32_t (&cur)[TNW], uint32_t (&nxt)[TNW]) {
        const int base = 4 * q;
        const int nq = min(q + 1, q1 - 1);
        const uint8_t* lb = lds + buf * kBuf;
#pragma unroll
        for (int tt = 0; tt < TNW; ++tt)
            nxt[tt] = __builtin_amdgcn_raw_buffer_load_b32(rs[tt], lane * 4, nq * 256, kLoadStream);
        a_issue(q + 1);
        auto step = [&](auto t_c) {
            constexpr int T = decltype(t_c)::value;
            w_issue(std::integral_constant<int, (T + 3) % 4>{}, base + T + 3);
            __builtin_amdgcn_sched_barrier(0);
            compute(t_c, lb, cur);
            __builtin_amdgcn_sched_barrier(0);
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
        a_store(1 - buf);
        lds_barrier();
    };

    const int c0 = 4 * q0;
#pragma unroll
    for (int tt = 0; tt < TNW; ++tt) sa[tt] = __builtin_amdgcn_raw_buffer_load_b32(rs[tt], lane * 4, q0 * 256, kLoadStream);
    a_issue(q0);
    w_issue(std::integral_constant<int, 0>{}, c0);
    w_issue(std::integral_constant<int, 1>{}, c0 + 1);
    w_issue(std::integral_constant<int, 2>{}, c0 + 2);
    a_store(0);
    lds_barrier();
    int q = q0;
    for (; q + 1 < q1; q += 2) {
        group(q, 0, sa, sb);
        group(q + 1, 1, sb, sa);
    }
    if (q < q1) group(q, 0, sa, sb);

#pragma unroll
    for (int tt = 0; tt < TNW; ++tt)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            const int m = m0 + wm * MBW * 16 + mb * 16 + r, n0 = (tile0 + tt) * kTileN + 4 * j;
            if (P == nullptr) {
                store_frag<0>(C, acc[tt][mb] * alpha, m, n0, M, N);
            } else if (m < M) {  // FP32 partials for the reduce kernel (plain stores: measured faster here)
                float* dst = P + ((size_t)ks * M + m) * N + n0;
                if ((N & 3) == 0 && n0 + 3 < N) {
                    *reinterpret_cast<f32x4*>(dst) = acc[tt][mb];
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (n0 + e < N) dst[e] = acc[tt][mb][e];
                }
            }
        }
}

// ------------------------------------------------------------ debug dequant
// One wave per (n-tile, 128-K chunk): writes the BF16 weights it would feed to
// the matrix core, using the GEMM's own dequant functions.
template <int FMT, int ACT>
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
        case 0: o[0] = dequant_step<FMT, 0, 0, ACT>(w, s); o[1] = dequant_step<FMT, 0, 1, ACT>(w, s);
                o[2] = dequant_step<FMT, 0, 2, ACT>(w, s); o[3] = dequant_step<FMT, 0, 3, ACT>(w, s); break;
        case 1: o[0] = dequant_step<FMT, 1, 0, ACT>(w, s); o[1] = dequant_step<FMT, 1, 1, ACT>(w, s);
                o[2] = dequant_step<FMT, 1, 2, ACT>(w, s); o[3] = dequant_step<FMT, 1, 3, ACT>(w, s); break;
        case 2: o[0] = dequant_step<FMT, 2, 0, ACT>(w, s); o[1] = dequant_step<FMT, 2, 1, ACT>(w, s);
                o[2] = dequant_step<FMT, 2, 2, ACT>(w, s); o[3] = dequant_step<FMT, 2, 3, ACT>(w, s); break;
        default: o[0] = dequant_step<FMT, 3, 0, ACT>(w, s); o[1] = dequant_step<FMT, 3, 1, ACT>(w, s);
                 o[2] = dequant_step<FMT, 3, 2, ACT>(w, s); o[3] = dequant_step<FMT, 3, 3, ACT>(w, s); break;
    }
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = b * kChunkK + 32 * i + 8 * j;
        if (k < K) *reinterpret_cast<u32x4*>(W + (size_t)n * K + k) = o[i];
    }
}

}  // namespace fp4
