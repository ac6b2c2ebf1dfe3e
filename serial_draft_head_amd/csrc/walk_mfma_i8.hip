// walk_mfma_i8.hip -- MFMA-engine walk kernels (walk_kernel.h) for int8
// weights with fp32 row scales, batch tiles 4 and 16.
#include "walk_kernel.h"

// DSW_SAMPLER 0: inverse-CDF sampling; 1: Gumbel-max (the *_gumbel.hip twin
// defines it and the lookup name, then includes this file)
#ifndef DSW_SAMPLER
#define DSW_SAMPLER 0
#define DSW_LOOKUP dsw_internal_mfma_i8_kernel
#endif

// Host-side lookup used by the launcher: the int8 kernel for (batch tile,
// register tiles, tiles per wave), or nullptr when that shape is not compiled.
extern "C" const void* DSW_LOOKUP(int batch_tile, int reg_tiles, int max_tiles) {
#define DSW_PICK4(R, M)                                                   \
    if (batch_tile == 4 && reg_tiles == (R) && max_tiles == (M))          \
        return (const void*)dsw::walk_kernel<dsw::kEngineMfma, (R), (M), 4, 1, DSW_SAMPLER>;
#define DSW_PICK16(R, M)                                                  \
    if (batch_tile == 16 && reg_tiles == (R) && max_tiles == (M))         \
        return (const void*)dsw::walk_kernel<dsw::kEngineMfma, (R), (M), 16, 1, DSW_SAMPLER>;
    DSW_MFMA_I8_SHAPES(DSW_PICK4)
    DSW_MFMA_I8_SHAPES(DSW_PICK16)
#undef DSW_PICK4
#undef DSW_PICK16
    return nullptr;
}
