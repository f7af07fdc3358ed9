// Compiled variants of the output-side products: EPI_PART (split-K partial
// tiles), EPI_RESNORM (full-K, residual add and the next norm's inputs) and
// EPI_PARTRES (split-K, the last split adding the partials into the
// residual).
#include "gemm_kernel.h"

namespace dflash {
template hipError_t launch_gemm_epi<bf16_t, EPI_PART>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<float, EPI_PART>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<bf16_t, EPI_RESNORM>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<float, EPI_RESNORM>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<bf16_t, EPI_PARTRES>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm_epi<float, EPI_PARTRES>(const GemmPlan&, GemmArgs, const EpiArgs&, hipStream_t);
}  // namespace dflash
