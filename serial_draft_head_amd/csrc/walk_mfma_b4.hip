// walk_mfma_b4.hip -- MFMA-engine walk kernels (walk_kernel.h) for batch
// tile 4 (up to 4 requests per launch).
#include "walk_kernel.h"

// DSW_SAMPLER 0: inverse-CDF sampling; 1: Gumbel-max (the *_gumbel.hip twin
// defines it and the lookup name, then includes this file)
#ifndef DSW_SAMPLER
#define DSW_SAMPLER 0
#define DSW_LOOKUP dsw_internal_mfma_kernel_b4
#endif

// Host-side lookup used by the launcher: the kernel for (register tiles,
// tiles per wave) at batch tile 4, or nullptr when that shape is not compiled.
extern "C" const void* DSW_LOOKUP(int reg_tiles, int max_tiles) {
#define DSW_PICK(R, M) \
    if (reg_tiles == (R) && max_tiles == (M)) return (const void*)dsw::walk_kernel<dsw::kEngineMfma, (R), (M), 4, 0, DSW_SAMPLER>;
    DSW_MFMA_SHAPES(DSW_PICK)
#undef DSW_PICK
    return nullptr;
}
