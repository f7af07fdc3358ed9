// Compiled variants of the weight-streaming products of the context path
// (EPI_FC: context projection; EPI_KV: K/V injection).
#include "gemm_kernel.h"

namespace dflash {
template hipError_t launch_gemm_epi<bf16_t, EPI_FC>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<float, EPI_FC>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<bf16_t, EPI_KV>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<float, EPI_KV>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
}  // namespace dflash
