// launch.h -- the one persistent launch of a walk round, shared by the
// handle-based entry points (api.cpp) and the allocation-free entry point
// (walk_static.hip).  Host code only.
#pragma once
#include <stdint.h>

#include "../../include/dsw.h"
#include "walk_params.h"

namespace dsw {

constexpr unsigned kSpinLimit = 1u << 20;  // polls before a device wait gives up; each costs well over 100 ns

// Everything a launch needs besides the call's tensors: the walk's sizes and
// flags, the device description, the workspace, and the diagnostics knobs.
struct LaunchCtx {
    int device;
    int V, gamma_max, B_max, dtype;
    unsigned flags;
    const dsw_devinfo* dev;
    Workspace ws;
    unsigned spin_limit, skew;
    int seeded;
    unsigned long long seed;
    unsigned long long* trace;
    long long trace_bytes;
};

// A recurrent head's extra arguments (dsw_walk_gru, dsw_walk_rnn: the cell;
// dsw_walk_gated: the gate matrix, its scales and biases; dsw_walk_domino:
// the GRU cell and the drafter's hidden states).
struct GruArgs {
    const uint16_t* wih;
    const uint16_t* whh;
    const float* bih;
    const float* bhh;
    const float* h0;
    float* states;
    const int8_t* gq;
    const float* gs;
    const float* gb;
    const uint16_t* hidden;  // Domino's head: H [gamma][d]
    int d;
};

// Plans and launches one round (B requests, gamma steps) on `stream`; gru is
// null for the Markov head.  Checks dtype/scale agreement and null tensors,
// returns a DSW_* code; B == 0 or gamma == 0 launches nothing.  plan_out, if
// not null, receives the plan.  Allocates nothing.
int launch_walk(const LaunchCtx& x, const void* W1, const void* W2, const float* w2_scale, const void* base,
                const int32_t* anchor, const float* T, const float* uniforms, int32_t* tokens, void* logits,
                int B, int gamma, void* stream, const GruArgs* gru, dsw_plan_info* plan_out);

}  // namespace dsw
