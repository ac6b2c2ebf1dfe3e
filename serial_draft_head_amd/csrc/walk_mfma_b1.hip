// walk_mfma_b1.hip -- MFMA-engine walk kernels (walk_kernel.h) for one request
// per launch: register tiles in AGPRs and VGPRs, four tiles' results gathered
// into one register per epilogue.
#include "walk_kernel.h"

// DSW_SAMPLER 0: inverse-CDF sampling; 1: Gumbel-max (the *_gumbel.hip twin
// defines it and the lookup name, then includes this file)
#ifndef DSW_SAMPLER
#define DSW_SAMPLER 0
#define DSW_LOOKUP dsw_internal_mfma_kernel_b1
#endif
// DSW_CELL 0: the Markov head; 1: the GRU head (walk_mfma_b1_gru.hip); 2: the
// RNN head (walk_mfma_b1_rnn.hip); 3: the gated head (walk_mfma_b1_gated.hip);
// 4: Domino's head (walk_mfma_b1_domino.hip)
#ifndef DSW_CELL
#define DSW_CELL 0
#endif
// DSW_DT 0: bf16 rows; 1: int8 rows with fp32 row scales (walk_mfma_b1_i8.hip)
#ifndef DSW_DT
#define DSW_DT 0
#endif

// Host-side lookup used by the launcher: the kernel for (register tiles,
// tiles per wave) at batch tile 1, or nullptr when that shape is not compiled.
extern "C" const void* DSW_LOOKUP(int reg_tiles, int max_tiles) {
#define DSW_PICK(R, M) \
    if (reg_tiles == (R) && max_tiles == (M)) return (const void*)dsw::walk_kernel<dsw::kEngineMfma, (R), (M), 1, DSW_DT, DSW_SAMPLER, DSW_CELL>;
    DSW_MFMA_ONE_SHAPES(DSW_PICK)
#undef DSW_PICK
    return nullptr;
}
