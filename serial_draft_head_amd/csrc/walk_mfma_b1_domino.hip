// walk_mfma_b1_domino.hip -- the kernels of walk_mfma_b1.hip for Domino's
// serial head ("Keeping the Draft Walk on Chip", section "Beyond DSpark: other
// serial heads"): one request, the GRU head whose input also carries the
// drafter's hidden state of each block position.
#define DSW_SAMPLER 0
#define DSW_CELL 4
#define DSW_LOOKUP dsw_internal_mfma_kernel_b1_domino
#include "walk_mfma_b1.hip"
