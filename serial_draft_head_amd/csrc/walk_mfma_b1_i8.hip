// walk_mfma_b1_i8.hip -- the kernels of walk_mfma_b1.hip for int8 rows with
// fp32 row scales: one request, the rows widened to bf16 once when the shard is
// loaded (exact), the bias bf16(scale * fp32 dot) (the int8-plus-row-scale
// table of "Keeping the Draft Walk on Chip", section "V = 248,320: 62% on
// chip, the rest streamed").
#define DSW_SAMPLER 0
#define DSW_DT 1
#define DSW_LOOKUP dsw_internal_mfma_kernel_b1_i8
#include "walk_mfma_b1.hip"
