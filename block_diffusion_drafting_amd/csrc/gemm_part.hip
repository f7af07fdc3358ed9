// Compiled variants of the weight-streaming product with the EPI_PART epilogue.
#include "gemm_kernel.h"

namespace dflash {
template hipError_t launch_gemm_epi<bf16_t, EPI_PART>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<float, EPI_PART>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
}  // namespace dflash
