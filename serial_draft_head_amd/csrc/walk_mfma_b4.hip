// walk_mfma_b4.hip -- MFMA-engine walk kernels (walk_kernel.h) for batch
// tile 4 (up to 4 requests per launch).
#include "walk_kernel.h"

// Host-side lookup used by the launcher: the kernel for (register tiles,
// tiles per wave) at batch tile 4, or nullptr when that shape is not compiled.
extern "C" const void* dsw_internal_mfma_kernel_b4(int reg_tiles, int max_tiles) {
#define DSW_PICK(R, M) \
    if (reg_tiles == (R) && max_tiles == (M)) return (const void*)dsw::walk_kernel<dsw::kEngineMfma, (R), (M), 4>;
    DSW_MFMA_SHAPES(DSW_PICK)
#undef DSW_PICK
    return nullptr;
}
