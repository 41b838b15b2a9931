// Instantiates the grouped MoE GEMM (the decode kernel's MOE variant) for BF16
// activations over the compiled MoE shapes and both weight formats.
#include "dispatch.h"
#include "kernels.h"

namespace fp4 {
namespace {

template <int FMT, int MB, int TN, int NWN>
void launch_moe_t(const void* A, const void* wq, const void* sq, void* C, const MoeArgs& moe, int N, int K, int KB,
                  int SB, int NT, int items, hipStream_t s) {
    const int groups = (NT + TN * NWN - 1) / (TN * NWN);
    gemm_decode<FMT, 0, MB, TN, NWN, 1, true><<<dim3(groups, items), dim3(64 * NWN), 0, s>>>(
        (const uint16_t*)A, (const u32x4*)wq, (const uint8_t*)sq, (uint16_t*)C, nullptr, 0, N, K, KB, SB, NT, 1, 1.0f, 0u, moe);
}

template <int FMT>
bool launch_moe_fmt(int MB, int tn, int nwn, const void* A, const void* wq, const void* sq, void* C,
                    const MoeArgs& moe, int N, int K, int KB, int SB, int NT, int items, hipStream_t s) {
#define FP4_MOE_CASE(MB_, TN_, NWN_)                                                         \
    if (MB == MB_ && tn == TN_ && nwn == NWN_) {                                             \
        launch_moe_t<FMT, MB_, TN_, NWN_>(A, wq, sq, C, moe, N, K, KB, SB, NT, items, s);    \
        return true;                                                                         \
    }
    FP4_MOE_SHAPES(FP4_MOE_CASE)
#undef FP4_MOE_CASE
    return false;
}

}  // namespace

bool launch_moe_bf16(int fmt, int MB, int tn, int nwn, const void* A, const void* wq, const void* sq, void* C,
                     const MoeArgs& moe, int N, int K, int KB, int SB, int NT, int items, hipStream_t s) {
    return fmt == 0 ? launch_moe_fmt<0>(MB, tn, nwn, A, wq, sq, C, moe, N, K, KB, SB, NT, items, s)
                    : launch_moe_fmt<1>(MB, tn, nwn, A, wq, sq, C, moe, N, K, KB, SB, NT, items, s);
}

}  // namespace fp4
