// walk_mfma_i8_gumbel.hip -- the kernels of walk_mfma_i8.hip with Gumbel-max sampling (flag
// DSW_FLAG_GUMBEL; "Keeping the Draft Walk on Chip", section "The idea: make
// the walk resident": small batches sample by per-row Gumbel-max).
#define DSW_SAMPLER 1
#define DSW_LOOKUP dsw_internal_mfma_i8_kernel_gumbel
#include "walk_mfma_i8.hip"
