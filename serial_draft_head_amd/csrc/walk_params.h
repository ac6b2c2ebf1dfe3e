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
constexpr int kTileRows = 16;       // MFMA engine: vocabulary rows per 16x16x32 tile
constexpr int kTileBytes = kTileRows * kRank * 2;   // 8 KiB of bf16 weights per tile
constexpr int kMaxRegTiles = 8;     // weight tiles per wave in the 256 AGPRs
constexpr int kMaxVgprTiles = 4;    // one request, MFMA engine: further tiles per wave in VGPRs
constexpr int kTraceSteps = 16;    // steps the optional phase trace records

// Device workspace.  Cross-workgroup traffic goes through per-workgroup
// mailboxes tagged with a step epoch: workgroup c writes its words for step
// s into mail[s & 1][c], and readers wait until a word carries the epoch of
// s.  The host clears nothing between steps, launches or graph replays.
//
// Epochs.  Step k of a launch has sequence number s = n * gamma_max + k
// (mod 2^32), n the launch count of the kernel family that owns the region
// (the all-to-all kernels and the batched kernel keep separate counts), and
// epoch(s) = (s mod 2^27) + 1: never 0, and since 2^27 divides 2^32 two steps
// share an epoch only if their sequence numbers are 2^27 apart, also across
// the 32-bit wrap.  At entry every workgroup zeroes each word it will post in
// this launch (both parities), before its first post and behind a barrier, so
// a word a reader polls holds 0, a post of this launch or a post of the
// family's previous launch -- fewer than 2 gamma_max steps from the current
// one, never a full period.  Every word has one writing workgroup.
constexpr int kMailKeys = 0;        // word b: request b's key (or Gumbel score)
constexpr int kMailSums = 16;       // word 16 + b: its exp-sum (or Gumbel ~id)
constexpr int kMailWords = 32;      // per workgroup and parity (256 bytes: measured faster to
                                    // poll than a 384-byte stride)
constexpr int kMaxBatchPersistent = 16;  // requests per launch of the all-to-all kernel
constexpr int kCellMaxPerWg = 4;   // recurrent heads: state elements per workgroup (one per wave; grid >= 64)
constexpr int kDominoMaxGamma = 16;  // Domino's head: steps per round (its drafters' blocks)
constexpr int kDominoMaxD = 4096;    // Domino's head: the drafter's hidden width, bound
constexpr int kMaxBatch = 256;           // requests per launch of the batched kernel
// Batched kernel: words of one owner workgroup's region (one per request it
// owns, rounded up to whole 128-byte lines), and a bound on G * owner_stride(G)
// over every grid of up to kMaxGrid workgroups.
constexpr int owner_stride(int G) { return (((kMaxBatch + G - 1) / G) + 15) / 16 * 16; }
constexpr int kOwnWords = 4096;
constexpr int max_owner_words() {
    int m = 0;
    for (int G = 1; G <= kMaxGrid; ++G) m = G * owner_stride(G) > m ? G * owner_stride(G) : m;
    return m;
}
static_assert(max_owner_words() <= kOwnWords, "owner regions of every grid fit kOwnWords");
constexpr int kGroup = 16;               // batched kernel: requests per MFMA column block
constexpr int kBatchedFrom = 2;          // the planner's default: the batched kernel from this many requests
constexpr unsigned kEpochMod = 0x0FFFFFFFu;   // the 28-bit epoch field of a mailbox word
constexpr unsigned kEpochPeriod = 1u << 27;   // epochs repeat after this many steps
constexpr int kMaxGammaMax = 4096;            // gamma_max bound: 2 gamma_max stays far below the period
constexpr int kFamAll = 0;                    // family counter of the all-to-all kernels
constexpr int kFamBatched = 1;                // family counter of the batched kernel
constexpr unsigned epoch_of(unsigned seq) { return (seq & (kEpochPeriod - 1u)) + 1u; }
// The control block: one 16-byte aligned line that a kernel reads with a single
// load when it starts (a kernel boundary makes the previous launch's updates
// visible): {round counter, family counters [2], status word}.
constexpr int kCtlRound = 0, kCtlFam = 1, kCtlStatus = 3;
struct Workspace {
    unsigned long long* mail;      // [2][kMaxGrid][kMailWords]
    unsigned long long* tokw;      // [2][kMaxGrid][kMaxBatchPersistent]  sampled token << 32 | epoch,
                                   // in the row of the shard that found it
    unsigned* round_ctr;           // ctl[0]  completed launches (keys the device-drawn noise)
    unsigned* fam_ctr;             // ctl[1..2]  completed launches per kernel family (the epochs)
    unsigned* status;              // ctl[3]  latched kStatus* bits
    // batched kernel (requests owned by workgroups): every workgroup posts one
    // key word and next to it one exp-sum word per request (a reader takes both
    // with one 16-byte load); the owner of request b reads column b, and for a
    // sampled request the token shard's logits from blog, and publishes the
    // token
    unsigned long long* bkey;      // [2][kMaxGrid][kMaxBatch][2]  key << 28 | epoch, then exp-sum
                                   // bits << 32 | epoch (Gumbel-max: ord32(score) << 28 | epoch,
                                   // then ~id << 32 | epoch)
    unsigned long long* bdec;      // [2][kOwnWords]  per owner workgroup c, a region of
                                   // owner_stride(G) words (whole 128-byte lines, one
                                   // writer each; 1 word for up to 16 requests); request
                                   // b = c + i G takes word i: its decision, token << 24 |
                                   // a 24-bit epoch
    uint16_t* blog;                // batched kernel: this step's logits of the 16-request
                                   // groups with a sampled request (agent-scope stores,
                                   // complete before the key words), read back by the
                                   // requests' owners, batched_logits_bytes() long;
                                   // NULL if the handle never runs the batched kernel.
                                   // Per workgroup c, 16-request group, wave and tile j:
                                   // 64 lanes x 4 bf16 (rows 4g .. 4g+3 of request n),
                                   // [c][group][wave][j][lane], so that each store of the
                                   // epilogue is one contiguous 512-byte block
};

// Status bits latched by the device (translated to DSW_ERR_DEV_* on the host).
constexpr unsigned kStatusTimeout = 1u;
constexpr unsigned kStatusToken = 2u;
constexpr unsigned kStatusUniforms = 4u;

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WorkspaceLayout {
    size_t mail, tokw, ctl, bkey, bdec, total;
};
inline WorkspaceLayout workspace_layout() {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    WorkspaceLayout L;
    size_t o = 0;
    L.mail = o;      o = up(o + 2 * (size_t)kMaxGrid * kMailWords * 8);
    L.tokw = o;      o = up(o + 2 * (size_t)kMaxGrid * kMaxBatchPersistent * 8);
    L.ctl = o;       o = up(o + 16);
    L.bkey = o;      o = up(o + 2 * (size_t)kMaxGrid * kMaxBatch * 16);
    L.bdec = o;      o = up(o + 2 * (size_t)kOwnWords * 8);
    L.total = o;
    return L;
}

// Bytes of Workspace::blog for up to B_max requests over any grid: per
// workgroup its 16-request groups x ceil(V / grid) rows rounded up to 64
// (four waves of whole 16-row tiles) x 2 bytes.
constexpr size_t batched_logits_bytes(int V, int B_max) {
    return (size_t)((B_max + 15) / 16 * 16) * ((size_t)V + 64u * (size_t)kMaxGrid) * 2u;
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
    int tiles_per_wave;      // MFMA engine: 16-row tiles per wave (contiguous rows)
    int lds_tiles;           // MFMA engine: tiles per wave held in LDS after the VGPR tiles
    int pf_tiles;            // MFMA engine, one bf16 request: streamed tiles per wave loaded
                             // into LDS one step ahead (after the LDS tiles' slots)
    int rows_pad;            // batched kernel: shard rows rounded up to a multiple of 128
    int ring;                // batched kernel: LDS slots for u rows and base logits of groups
    int aligned;             // batched kernel: V % 8 == 0 (16-byte aligned base rows)
    unsigned spin_limit;     // polls before a wait gives up and latches kStatusTimeout
    unsigned skew;           // diagnostics: 0, or each workgroup sleeps a pseudo-random
                             // multiple of this many s_sleep units before it posts
    int single_round;        // 1: logit = bf16(base + fp32 dot), rounded once
    int seeded;              // 1: uniforms == NULL draws them on the device from seed
    unsigned long long seed; // key of the device-drawn uniforms and of the Gumbel noise
    // Recurrent serial heads (one request): the cell's weights [g*r][r] bf16
    // and biases [g*r] f32 -- g = 3 for the GRU (CELL = 1; gates r, z, n),
    // g = 1 for the tanh RNN (CELL = 2) -- the initial state [r] f32, and an
    // optional [gamma][r] f32 output of every step's state
    const uint16_t* gru_wih;         // rows of cell_in values (r, or r + d for Domino's head)
    const uint16_t* gru_whh;
    const float* gru_bih;
    const float* gru_bhh;
    const float* h0;
    float* states;
    // gated head (CELL = 3): the r x r gate matrix as int8 codes (row-major,
    // 16-byte aligned) with fp32 row scales and biases; h0 and states as above
    const int8_t* gate_q;
    const float* gate_scale;
    const float* gate_bias;
    // Domino's head (CELL = 4; the GRU with the drafter's hidden states appended
    // to its input): hidden states [gamma][hidden_d] bf16, 16-byte aligned
    const uint16_t* hidden;
    int hidden_d;
    int cell_in;             // Wih row length: r, or r + hidden_d
    unsigned long long* trace;  // optional [grid][gamma+1][8] phase timestamps, or null
};

// Phase timestamps recorded per workgroup and step when a trace buffer is set
// (s_memrealtime, the device-wide 100 MHz clock, so that workgroups on
// different XCDs compare; slot 7 holds the core-clock counter s_memtime).
enum TracePhase {
    kTrStepStart = 0,   // top of the step
    kTrGathered = 1,    // u and the base logits staged (after the barrier)
    kTrGemvDone = 2,    // GEMV and epilogue done (wave 0)
    kTrReduced = 3,     // workgroup argmax known
    kTrPosted = 4,      // key posted and arrival counted
    kTrArrived = 5,     // every workgroup has arrived
    kTrSelected = 6,    // tokens known (end of step)
    kTrReal = 7,        // s_memtime (core clock) at the end of the step
};

}  // namespace dsw
