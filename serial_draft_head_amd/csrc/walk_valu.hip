// walk_valu.hip -- VALU-engine walk kernels (walk_kernel.h) for every
// (VGPR row groups per lane, batch tile) the planner may pick.
#include "walk_kernel.h"

// DSW_SAMPLER 0: inverse-CDF sampling; 1: Gumbel-max (the *_gumbel.hip twin
// defines it and the lookup name, then includes this file)
#ifndef DSW_SAMPLER
#define DSW_SAMPLER 0
#define DSW_LOOKUP dsw_internal_walk_kernel
#endif

// Host-side lookup used by the launcher: the kernel for (register row groups,
// batch tile, W2 dtype), or nullptr when it is not compiled.  int8 rows are
// compiled for one request.
extern "C" const void* DSW_LOOKUP(int reg_slots, int batch_tile, int w2_dtype) {
#define DSW_PICK(R, NB)                                                  \
    if (w2_dtype == 0 && reg_slots == (R) && batch_tile == (NB))          \
        return (const void*)dsw::walk_kernel<dsw::kEngineValu, (R), 0, (NB), 0, DSW_SAMPLER>;
#define DSW_PICK_I8(R)                                                   \
    if (w2_dtype == 1 && reg_slots == (R) && batch_tile == 1)            \
        return (const void*)dsw::walk_kernel<dsw::kEngineValu, (R), 0, 1, 1, DSW_SAMPLER>;
    DSW_PICK(0, 1) DSW_PICK(1, 1) DSW_PICK(2, 1) DSW_PICK(3, 1)
    DSW_PICK(0, 4) DSW_PICK(1, 4) DSW_PICK(2, 4)
    DSW_PICK(0, 16) DSW_PICK(1, 16)
    DSW_PICK_I8(0) DSW_PICK_I8(1) DSW_PICK_I8(2)
#undef DSW_PICK
#undef DSW_PICK_I8
    return nullptr;
}
