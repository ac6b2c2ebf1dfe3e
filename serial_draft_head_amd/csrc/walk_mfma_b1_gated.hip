// walk_mfma_b1_gated.hip -- the kernels of walk_mfma_b1.hip for DSpark's gated
// serial head ("Keeping the Draft Walk on Chip", section "Beyond DSpark: other
// serial heads"): one request, the whole state updated in every workgroup
// through one int8 gate matrix held in LDS.
#define DSW_SAMPLER 0
#define DSW_CELL 3
#define DSW_LOOKUP dsw_internal_mfma_kernel_b1_gated
#include "walk_mfma_b1.hip"
