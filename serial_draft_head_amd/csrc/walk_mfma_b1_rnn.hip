// walk_mfma_b1_rnn.hip -- the kernels of walk_mfma_b1.hip for the RNN serial
// head ("Keeping the Draft Walk on Chip", section "Beyond DSpark: other serial
// heads"): one request, the state updated by a tanh RNN cell every step.
#define DSW_SAMPLER 0
#define DSW_CELL 2
#define DSW_LOOKUP dsw_internal_mfma_kernel_b1_rnn
#include "walk_mfma_b1.hip"
