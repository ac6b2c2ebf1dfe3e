// walk_batched.hip -- batched walk kernels (walk_batched.h): bf16 and int8
// weights, every compiled (register tiles, tiles per wave) shape.
#include "walk_batched.h"

// Host-side lookup used by the launcher: the batched kernel for (W2 dtype,
// register tiles, tiles per wave, single rounding, four tiles per epilogue,
// Gumbel-max), or nullptr when that shape is not compiled.  The four-tile
// epilogue (up to 4 requests) and Gumbel-max are compiled for bf16 with double
// rounding.
extern "C" const void* dsw_internal_batched_kernel(int w2_dtype, int reg_tiles, int max_tiles, int single_round,
                                                   int fold, int gumbel) {
#define DSW_PICK(R, M)                                                                       \
    if (w2_dtype == 0 && reg_tiles == (R) && max_tiles == (M)) {                             \
        if (single_round) return gumbel ? nullptr : (const void*)dsw::walk_batched<(R), (M), 0, 1>; \
        if (gumbel)                                                                          \
            return fold ? (const void*)dsw::walk_batched<(R), (M), 0, 0, 4, 1>                \
                        : (const void*)dsw::walk_batched<(R), (M), 0, 0, 1, 1>;               \
        return fold ? (const void*)dsw::walk_batched<(R), (M), 0, 0, 4>                      \
                    : (const void*)dsw::walk_batched<(R), (M), 0, 0>;                        \
    }
#define DSW_PICK_I8(R, M)                                                \
    if (w2_dtype == 1 && reg_tiles == (R) && max_tiles == (M))           \
        return gumbel ? nullptr                                          \
                      : (single_round ? (const void*)dsw::walk_batched<(R), (M), 1, 1> \
                                      : (const void*)dsw::walk_batched<(R), (M), 1, 0>);
    DSW_BATCHED_SHAPES(DSW_PICK)
    DSW_BATCHED_I8_SHAPES(DSW_PICK_I8)
#undef DSW_PICK
#undef DSW_PICK_I8
    return nullptr;
}
