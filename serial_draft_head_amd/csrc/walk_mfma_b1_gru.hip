// walk_mfma_b1_gru.hip -- the kernels of walk_mfma_b1.hip for the GRU serial
// head ("Keeping the Draft Walk on Chip", section "Beyond DSpark: other serial
// heads"): one request, the state updated by a GRU cell every step.
#define DSW_SAMPLER 0
#define DSW_CELL 1
#define DSW_LOOKUP dsw_internal_mfma_kernel_b1_gru
#include "walk_mfma_b1.hip"
