// walk_params.h -- launch parameters of the persistent walk kernel and the
// layout of the device workspace the handle owns.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace dsw {

constexpr int kRank = 256;          // r: latent width of the Markov head
constexpr int kBlock = 256;         // threads per workgroup (4 wave64, one per SIMD)
constexpr int kRowChunks = 32;      // 16-byte chunks in one bf16 row of 256
constexpr int kMaxSlots = 4;        // 256-row groups per workgroup (rows <= 1024)
constexpr int kMaxGrid = 256;       // one workgroup per CU; partial scans assume <= 256
constexpr int kLdsWork = 16384;     // LDS bytes reserved for u vectors and reductions

// Device workspace.  Every cross-workgroup slot exists twice, indexed by the
// parity of a device-side round counter: a launch uses parity p and clears
// parity 1-p for the next launch, so repeated launches (and graph replays)
// need no memset.
struct Workspace {
    unsigned long long* keys;      // [2][gamma_max][B_max]  packed {ordered logit, ~index}
    unsigned* counts;              // [2][gamma_max]         arrivals per step
    unsigned long long* partials;  // [2][gamma_max][B_max][kMaxGrid] {m_c, s_c} per shard
    unsigned* tok_slots;           // [2][gamma_max][B_max]  sampled token + 1
    unsigned* round_ctr;           // [1]
    unsigned* status;              // [1]  latched DSW_DEV_* bits
};

// Status bits latched by the device (translated to DSW_ERR_DEV_* on the host).
constexpr unsigned kStatusTimeout = 1u;
constexpr unsigned kStatusToken = 2u;
constexpr unsigned kStatusUniforms = 4u;

// Byte offsets of the workspace regions (each 256-byte aligned) for a handle
// serving at most gamma_max steps and B_max requests.
struct WorkspaceLayout {
    size_t keys, counts, partials, tok_slots, round_ctr, status, total;
};
inline WorkspaceLayout workspace_layout(int gamma_max, int B_max) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t gb = (size_t)gamma_max * (size_t)B_max;
    WorkspaceLayout L;
    size_t o = 0;
    L.keys = o;      o = up(o + 2 * gb * 8);
    L.counts = o;    o = up(o + 2 * (size_t)gamma_max * 4);
    L.partials = o;  o = up(o + 2 * gb * kMaxGrid * 8);
    L.tok_slots = o; o = up(o + 2 * gb * 4);
    L.round_ctr = o; o = up(o + 4);
    L.status = o;    o = up(o + 4);
    L.total = o;
    return L;
}

struct WalkParams {
    const uint16_t* W1;
    const void* W2;          // bf16 or int8 rows
    const float* w2_scale;   // int8 only
    const uint16_t* base;
    const int32_t* anchor;
    const float* T;
    const float* uniforms;
    int32_t* tokens;
    uint16_t* logits;
    Workspace ws;
    int V;
    int B;
    int gamma;
    int gamma_max;
    int B_max;
    int rows_per_wg;
    int lds_rows;            // rows per workgroup resident in LDS (after the register slots)
    unsigned spin_limit;     // polls before a wait gives up and latches kStatusTimeout
};

}  // namespace dsw
