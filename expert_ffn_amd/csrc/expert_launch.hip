// One group of variants of the fused expert kernel (expert_kernel.h): compiled once
// per (dtype, kernel, shared experts) with -DMOE_K_BF16=0|1 -DMOE_K_MODE=0|1
// -DMOE_K_SH=0|1, so that the variant groups compile in parallel.  Each compilation
// defines the one launcher its macros name.
#include "expert_kernel.h"

#if !defined(MOE_K_BF16) || !defined(MOE_K_MODE) || !defined(MOE_K_SH)
#error "build with -DMOE_K_BF16=0|1 -DMOE_K_MODE=0|1 -DMOE_K_SH=0|1"
#endif

#define MOE_K_NAME2(b, m, s) launch_expert_##b##_##m##_##s
#define MOE_K_NAME(b, m, s) MOE_K_NAME2(b, m, s)

namespace moe_k {

void MOE_K_NAME(MOE_K_BF16, MOE_K_MODE, MOE_K_SH)(const Args& a, const Plan& p, int grid, hipStream_t st, int lay) {
    launch_nt<MOE_K_BF16 != 0, MOE_K_MODE, MOE_K_SH != 0>(a, p, grid, st, lay);
}

}  // namespace moe_k
