// Host-side launch interface between the C ABI (fp4gemm.hip) and the kernel
// instantiations, one translation unit per kernel family and activation type
// (decode_bf16.hip, decode_f16.hip, prefill_bf16.hip, prefill_f16.hip), which
// are compiled in parallel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

// Decode kernel: TN n-tiles per wave, NWN waves per K group, NWK K groups per
// workgroup, K split over S workgroups.
struct DecodeShape {
    int tn, nwn, nwk, s;
};

// Prefill kernel: WM x WN waves, MBW m-blocks and TNW n-tiles per wave, K split
// over S workgroups.
struct PrefillShape {
    int wm, wn, mbw, tnw, s;
};

// Grouped MoE problem (see the MoE routing note in kernels.h): expert e owns
// the packed weights at wq + e * w_stride / sq + e * s_stride and the
// assignment ids ids[offsets[e] .. offsets[e+1]); assignment id reads
// activation row id / a_div and writes output row id, scaled by topw[id]
// when topw is not null.
struct MoeArgs {
    const int32_t* ids;
    const int32_t* offsets;
    const float* topw;
    int E, P;      // experts; entries of ids
    int a_div;     // activation row of an assignment = id / a_div
    int a_rows;    // rows of A
    int out_rows;  // rows of C; ids outside [0, out_rows) are skipped
    int64_t w_stride, s_stride;
};

// Compiled decode shapes: X(MB, TN, NWN, NWK).
#define FP4_DECODE_SHAPES(X)                                                                         \
    X(1, 1, 4, 1) X(1, 2, 4, 1) X(1, 1, 4, 2) X(1, 2, 4, 2) X(1, 1, 4, 4) X(1, 2, 1, 4) X(1, 2, 1, 1)  \
    X(1, 2, 7, 1) X(1, 1, 7, 1) X(1, 2, 7, 2) X(1, 2, 5, 1) X(1, 1, 5, 2) X(1, 1, 8, 1) X(1, 2, 8, 1)  \
    X(1, 1, 8, 2) X(2, 1, 4, 1) X(2, 1, 4, 2) X(2, 1, 8, 1) X(2, 2, 4, 1) X(4, 1, 4, 1) X(4, 1, 8, 1)  \
    X(4, 2, 4, 1)

// Compiled prefill shapes: X(WM, WN, MBW, TNW).
#define FP4_PREFILL_SHAPES(X) \
    X(1, 4, 8, 2) X(1, 4, 8, 4) X(2, 2, 4, 4) X(2, 2, 4, 2) X(1, 4, 8, 1) X(2, 2, 4, 1) X(1, 4, 4, 4) \
    X(1, 8, 8, 2) X(1, 8, 8, 1) X(1, 8, 4, 2) X(1, 8, 16, 2)

// Launch one GEMM kernel on stream s (P: FP32 partials of a K split, else
// null).  False when the shape is not compiled.  The decode kernel finishes
// its K split itself (arrival words after the partials, `tag` unique to the
// launch); the prefill kernel leaves the partials to reduce_partials.
bool launch_decode_bf16(int fmt, int MB, const DecodeShape& d, const void* A, const void* wq, const void* sq,
                        void* C, float* P, int M, int N, int K, int KB, int SB, int NT, float alpha, uint32_t tag,
                        hipStream_t s);
bool launch_decode_f16(int fmt, int MB, const DecodeShape& d, const void* A, const void* wq, const void* sq, void* C,
                       float* P, int M, int N, int K, int KB, int SB, int NT, float alpha, uint32_t tag,
                       hipStream_t s);
bool launch_prefill_bf16(int fmt, const PrefillShape& t, const void* A, const void* wq, const void* sq, void* C,
                         float* P, int M, int N, int K, int KB, int SB, int NT, float alpha, hipStream_t s);
bool launch_prefill_f16(int fmt, const PrefillShape& t, const void* A, const void* wq, const void* sq, void* C,
                        float* P, int M, int N, int K, int KB, int SB, int NT, float alpha, hipStream_t s);

// Compiled MoE shapes (BF16 activations): X(MB, TN, NWN); one K group, no K
// split.  `items` bounds the number of row blocks (grid height).
#define FP4_MOE_SHAPES(X) \
    X(1, 1, 2) X(1, 1, 4) X(1, 1, 8) X(1, 2, 8) X(2, 1, 4) X(2, 1, 8) X(2, 2, 8) X(4, 1, 4) X(4, 1, 8) X(4, 2, 8)
bool launch_moe_bf16(int fmt, int MB, int tn, int nwn, const void* A, const void* wq, const void* sq, void* C,
                     const MoeArgs& moe, int N, int K, int KB, int SB, int NT, int items, hipStream_t s);

}  // namespace fp4
