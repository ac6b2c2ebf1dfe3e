// walk_mfma_b1_i8_gumbel.hip -- the kernels of walk_mfma_b1_i8.hip with
// Gumbel-max sampling (flag DSW_FLAG_GUMBEL).
#define DSW_SAMPLER 1
#define DSW_DT 1
#define DSW_LOOKUP dsw_internal_mfma_kernel_b1_i8_gumbel
#include "walk_mfma_b1.hip"
