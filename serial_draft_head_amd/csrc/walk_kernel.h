// walk_kernel.h -- one persistent launch per round of DSpark's serial Markov
// draft walk on gfx950 (MI355X), with two shard-GEMV engines.
//
// What is computed ("Keeping the Draft Walk on Chip", tie-pilot-qxw.github.io,
// section "The serial part of a parallel drafter"): for k < gamma,
// u = W1[prev], logit = bf16(base_k + bf16(W2 . u)), tok = argmax (T = 0) or an
// inverse-CDF sample of softmax(logit / T) (vLLM PR #64442, "Details"),
// prev = tok.
//
// Residency (section "The idea: make the walk resident"): workgroup c owns the
// contiguous rows [c*R, c*R + R) of W2 and keeps them on chip for the whole
// walk, so W2 crosses HBM once per round.
//
// GEMV engines:
//   VALU (A = VGPR row groups per lane): lane t owns rows s*256 + t; the
//     first A groups live in VGPR/AGPRs (128 dwords per row), then rows in LDS
//     (16-byte chunks XOR-swizzled), then rows re-read every step.  Each lane
//     forms whole dot products with v_dot2_f32_bf16 against u broadcast from
//     LDS, so the GEMV needs no cross-lane reduction.
//   MFMA (A = VGPR tiles per wave, M = tiles per wave): rows in 16-row tiles,
//     each the B operand of v_mfma_f32_16x16x32_bf16 (N = rows, K = 32 latent
//     values); u of up to 16 requests is the A operand, so extra requests cost
//     no extra matrix work (section "B200: the bf16 table fits on chip":
//     batching is almost free on the tensor cores).  Each request's results
//     land in one 16-lane DPP row.
// int8 weights (MFMA engine): one fp32 scale per row; each lane widens its
//   int8 codes to bf16 (exact: |q| <= 127 needs 7 significant bits) before the
//   MFMA, and the shard bias is bf16(scale * fp32 dot) (the int8-plus-row-scale
//   table of section "V = 248,320: 62% on chip, the rest streamed").
// Both engines round twice to bf16 (bias, then base + bias) and reduce their
// rows to workgroup-local keys {order-preserving bf16 logit, ~row}, so equal
// logits resolve to the smallest id (section "The idea").
//
// Rendezvous: each workgroup stores one word per request {logit, ~id, epoch}
// (and the shard's exp-sum for sampled requests) into its own mailbox region;
// every workgroup reads all regions until each carries the step's epoch.
// Regions alternate by step parity and epochs come from a device round
// counter, so nothing is cleared between steps, launches or graph replays.
// Sampling scans shard masses in vocabulary order; the owner shard of u*Z finds
// the token and publishes it through a token mailbox (vLLM PR #64442,
// "Details": block masses, then a token inside the block).  The GUM = 1
// instantiations sample by Gumbel-max instead (section "The idea: make the
// walk resident": per-row Gumbel-max for small batches): each workgroup posts
// its best {l / T + G, ~id} in the two words, and the largest such key across
// the grid names the token, with no owner hop; up to 4 requests, the noise G
// of the next step is drawn while the current step's words travel.
#pragma once
#include <type_traits>

#include "walk_device.h"

namespace dsw {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kEngineValu = 0;
constexpr int kEngineMfma = 1;

__device__ __forceinline__ f32x4_t mfma_tile(const uint4 a, const uint4 b, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// MFMA engine: the 8-latent chunk that lane group gg (lanes 16gg .. 16gg+15)
// supplies in K block kb.  Chunks are dealt so that each lane's 8 K blocks are
// 8 consecutive chunks of its row (128 contiguous bytes of bf16 weights), not
// every fourth chunk; A (u) and B (W2) use the same map, so the contraction
// covers every latent once.
#define DSW_KC(kb, gg) ((gg) * 8 + (kb))

// Workgroup-local 32-bit key: {order-preserving bf16 logit, ~row in shard}.
__device__ __forceinline__ uint32_t local_key(uint32_t lbits, int r) {
    return (ord16(lbits) << 16) | (0xFFFFu - (uint32_t)r);
}
__device__ __forceinline__ float local_key_logit(uint32_t lk) { return bf16_to_f32(unord16(lk >> 16)); }

// Global 36-bit key {ordered bf16 logit, ~vocabulary id} from a local key; 0 stays 0.
__device__ __forceinline__ unsigned long long global_key(uint32_t lk, int v0) {
    if (lk == 0u) return 0ull;
    const uint32_t v = (uint32_t)v0 + (0xFFFFu - (lk & 0xFFFFu));
    return ((unsigned long long)(lk >> 16) << kIdxBits) | (unsigned long long)(kIdxMask - v);
}

// Pin a weight in AGPRs: the compiler may not re-load it from memory later.
__device__ __forceinline__ void pin_agpr(uint4& v) {
    asm volatile("" : "+a"(v.x), "+a"(v.y), "+a"(v.z), "+a"(v.w));
}
__device__ __forceinline__ void pin_agpr(uint2& v) { asm volatile("" : "+a"(v.x), "+a"(v.y)); }
__device__ __forceinline__ void pin_vgpr(uint4& v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ __forceinline__ void pin_vgpr(uint2& v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }

// One request on the MFMA engine: tile j's 16 results sit in lanes 0..15 of
// its accumulator's first register.  Two permlane16 swaps and one permlane32
// swap gather four tiles into one register, lane l holding row l%16 of tile
// l/16, i.e. the 64 consecutive rows of the four tiles.
__device__ __forceinline__ float combine4(float t0, float t1, float t2, float t3) {
    const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t0), __float_as_uint(t1), false, false);
    const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t2), __float_as_uint(t3), false, false);
    const auto s = __builtin_amdgcn_permlane32_swap(s01[0], s23[0], false, false);
    return __uint_as_float(s[0]);
}

// One K block of a lane's tile row as the MFMA's 8 bf16 values.
__device__ __forceinline__ uint4 as_bf16x8(const uint4& w) { return w; }
// Signed byte `i` of w as an exact fp32 value.
__device__ __forceinline__ float i8_at(uint32_t w, int i) { return (float)(int)(int8_t)(w >> (8 * i)); }
// Two fp32 values with zero low halves as a bf16 pair (lo in the low half).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ uint4 as_bf16x8(const uint2& q) {
    return make_uint4(bf16_pair(i8_at(q.x, 0), i8_at(q.x, 1)), bf16_pair(i8_at(q.x, 2), i8_at(q.x, 3)),
                      bf16_pair(i8_at(q.y, 0), i8_at(q.y, 1)), bf16_pair(i8_at(q.y, 2), i8_at(q.y, 3)));
}

// GUM = 1: sampled requests draw by Gumbel-max instead of the inverse CDF (a
// separate instantiation, so that the default kernels carry none of its code).
// CELL = 1, 2: recurrent serial heads ("Keeping the Draft Walk on Chip",
// section "Beyond DSpark: other serial heads": the same walk with a state
// update; the state is spread across the workgroups and gathered once per
// step).  The state h goes through a standard cell fed with x = W1[prev] --
// CELL = 1 the GRU (Cho et al. 2014; gates r, z, n; the reset gate scales
// Whn h + bhn), CELL = 2 the tanh RNN, h' = tanh(Wih x + bih + Whh h + bhh) --
// and the vocabulary matrix reads bf16(h).  Workgroup c updates state
// elements c, c + G, ... (one per wave), posts them with the step's epoch, and
// every workgroup gathers all r of them before its GEMV.  CELL = 3: DSpark's
// gated head, whose one r x r matrix is small enough in int8 for every
// workgroup to hold it and update the whole state itself (no state exchange):
// g = sigmoid(s (Gq h) + b) from the state, h' = g h + (1 - g) x.  CELL = 4:
// Domino's head, the GRU of CELL = 1 whose input also carries the drafter's
// hidden state H_k of block position k, x = [W1[prev]; H_k]; the hidden
// states' part of the input pre-activations is formed for every step when the
// kernel starts (one state element per workgroup).  One request.
template <int ENGINE, int A, int M, int NB, int DT = 0, int GUM = 0, int CELL = 0>
__global__ void __launch_bounds__(kBlock, 1) walk_kernel(WalkParams p) {
    constexpr bool kMfma = ENGINE == kEngineMfma;
    constexpr bool kI8 = DT == 1;  // int8 rows + fp32 row scales
    static_assert(!kI8 || kMfma || NB == 1, "int8 rows on the VALU engine: one request");
    static_assert(NB == 1 || NB == 4 || NB == 16, "batch tile");
    // one request on the MFMA engine: tiles gathered four at a time, up to
    // kMaxRegTiles tiles per wave in AGPRs and kMaxVgprTiles more in VGPRs
    constexpr bool kOne = kMfma && NB == 1;
    // MT: one K block of 8 weights of a lane's tile row as stored in memory
    // (MFMA: 8 int8 codes or 8 bf16), or 16 bytes of a row (VALU).  WT: the
    // same on chip -- the MFMA engine with up to 16 requests keeps int8 codes
    // and widens them every step; one request keeps rows widened to bf16 once,
    // at entry (exact: |q| <= 127), as does the VALU engine
    using MT = typename std::conditional<kI8 && kMfma, uint2, uint4>::type;
    using WT = typename std::conditional<kI8 && kMfma && !kOne, uint2, uint4>::type;
    static_assert(!kMfma || (A <= M && A <= (kI8 && !kOne ? 2 : 1) * kMaxRegTiles + (kOne ? kMaxVgprTiles : 0)),
                  "MFMA shape");
    static_assert(kMfma || (A >= 0 && A <= kMaxSlots), "VALU shape");
    constexpr bool kCell = CELL != 0;                           // a recurrent head
    constexpr bool kDomino = CELL == 4;                         // the GRU reading the drafter's hidden states
    constexpr bool kGru = CELL == 1 || kDomino;
    constexpr bool kGated = CELL == 3;                          // the whole state in every workgroup
    constexpr bool kShard = kCell && !kGated;                   // the state spread over the workgroups
    // One request (not the gated head, which polls before forming its gates):
    // the second word sits next to the key, and a reader fetches both with one
    // 16-byte load -- half the polls through the fabric (V = 151,936, gamma
    // 16, mixed T: 106.2 -> 99.9 us; Gumbel-max: 83.0 -> 76.9 us).  The
    // recurrent heads' state words follow at 2 .. 5.
    constexpr bool kPair = NB == 1 && !kGated;
    constexpr int kStateWord = 2;
    constexpr int kSumWord = kPair ? 1 : kMailSums;
    constexpr int kGates = kGru ? 3 : 1;                         // cell rows per input, per element
    static_assert(CELL >= 0 && CELL <= 4, "cell");
    static_assert(!kCell || (kOne && GUM == 0), "recurrent heads: the one-request MFMA engine");
    static_assert(!kCell || kBlock == kRank, "recurrent heads: one state element per thread in the gather");
    constexpr int RPAD = kMfma ? M * 4 * kTileRows : kMaxSlots * kBlock;  // rows per shard, bound
    constexpr int CHMAX = (RPAD + kBlock - 1) / kBlock;                    // scan rows per thread
    constexpr int US = kRowChunks + 1;                                     // padded u row (uint4)
    constexpr int KPL = (kMfma && !kOne) ? 4 : NB;                         // request keys per lane
    constexpr int NQ = kOne ? (M + 3) / 4 : 1;                             // 4-tile groups per wave
    extern __shared__ uint4 s_w[];  // LDS-resident weights (engine-specific layout)

    __shared__ uint4 s_u[NB * US];
    __shared__ uint16_t s_base[kMfma && !kOne ? NB * RPAD : 1];
    __shared__ float s_scale[kI8 ? RPAD : 1];
    __shared__ uint16_t s_logit[NB * RPAD];
    // Gumbel-max, up to 4 requests: the noise G of the shard's rows for the
    // coming step, drawn while the previous rendezvous is in flight
    constexpr bool kPreG = GUM != 0 && NB <= 4;
    __shared__ float s_G[kPreG ? NB * RPAD : 1];
    // recurrent heads: the state h (r floats), and this workgroup's rows of the
    // cell (per owned element: the kGates rows of Wih, then those of Whh --
    // GRU Wir, Wiz, Win, Whr, Whz, Whn) with their biases
    __shared__ float s_h[kCell ? kRank : 1];
    __shared__ uint16_t s_cw[kShard ? kCellMaxPerWg * 2 * kGates * kRank : 1];
    __shared__ float s_cb[kShard ? kCellMaxPerWg * 2 * kGates : 1];
    // recurrent heads: Whh h + bhh of the owned elements for the coming step,
    // formed while the previous step's keys travel
    __shared__ float s_gh[kShard ? kCellMaxPerWg * kGates : 1];
    // Domino's head (one state element per workgroup): the hidden states' part
    // of the element's three input pre-activations for every step, and the
    // waves' partial sums that form it
    __shared__ float s_P[kDomino ? kDominoMaxGamma * 3 : 1];
    __shared__ float s_pp[kDomino ? 4 * kDominoMaxGamma * 3 : 1];
    // gated head: the matrix widened once from int8 to bf16 (exact), as 16
    // MFMA B-operand tiles of 16 rows in the order [tile][K block][lane]; the
    // row scales and biases; the gates of the coming step; and the state's
    // three bf16 pieces hi, lo, lo2 (h = hi + lo + lo2 exactly; hi = bf16(h)
    // is also the vocabulary GEMV's operand in s_u)
    __shared__ uint4 s_gw[kGated ? (kRank / kTileRows) * 8 * 64 : 1];
    __shared__ float s_gs[kGated ? kRank : 1];
    __shared__ float s_gb[kGated ? kRank : 1];
    __shared__ float s_gg[kGated ? kRank : 1];
    __shared__ uint4 s_hp[kGated ? 3 * kRowChunks : 1];
    __shared__ uint32_t s_wbest[4][NB];
    __shared__ unsigned long long s_red64[4][NB];
    __shared__ float s_redf[4][NB];
    // shard masses (inverse CDF); Gumbel-max: the waves' best {score, ~id} keys
    __shared__ __attribute__((aligned(16))) float s_S[NB * kBlock];
    __shared__ int s_own[NB];
    __shared__ float s_pex[NB];
    __shared__ float s_tgt[NB];
    __shared__ float s_Mg[NB];
    __shared__ float s_excl[NB * kBlock];
    __shared__ int s_redi[4];
    __shared__ int s_redj[4];
    __shared__ float s_T[NB];
    __shared__ float s_tot[NB];
    __shared__ int s_anchor[NB];
    __shared__ int s_prev[NB];
    __shared__ unsigned s_round;
    __shared__ unsigned s_fam;
    __shared__ int s_abort;
    DSW_TRACE_DECL;
    // one request, up to 10 register tiles: the branch-free epilogue's logits
    // of lanes past the shard
    __shared__ uint16_t s_lj[kMfma && kOne && A <= 10 ? 64 : 1];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // provably wave-uniform
    const int g = lane >> 4;  // MFMA: DPP row holding requests 4g .. 4g+3
    const int n = lane & 15;  // MFMA: row within a tile
    const int c = blockIdx.x;
    const int G = gridDim.x;
    const int V = p.V;
    const int B = p.B;
    const int gamma = p.gamma;
    const int v0 = c * p.rows_per_wg;
    const uint32_t dbl_round = p.single_round ? 0u : 0xFFFFFFFFu;  // see bias_round
    constexpr bool gum = GUM != 0;  // sampled requests: Gumbel-max instead of the inverse CDF
    const int nrows = max(0, min(V, v0 + p.rows_per_wg) - v0);
    // register slots beyond the shard load its last row (a cache hit), never
    // another shard's rows (extra HBM reads); an empty shard loads row V - 1
    const int last_row = nrows > 0 ? v0 + nrows - 1 : V - 1;
    const MT* __restrict__ W2 = reinterpret_cast<const MT*>(p.W2);
    WT* s_wt = reinterpret_cast<WT*>(s_w);
    const uint4* __restrict__ W1 = reinterpret_cast<const uint4*>(p.W1);
    const uint16_t* __restrict__ base = p.base;
    unsigned* status = p.ws.status;
    // VALU layout
    const int reg_cap = kMfma ? 0 : A * kBlock;
    const int reg_rows = kMfma ? 0 : min(nrows, reg_cap);
    const int lds_rows = kMfma ? 0 : min(nrows - reg_rows, p.lds_rows);
    // MFMA layout
    const int TW = kMfma ? p.tiles_per_wave : 0;
    const int LT = kMfma ? p.lds_tiles : 0;
    // one bf16 request, no register tiles (the shape that streams): streamed
    // tiles LT .. LT + PF - 1 of this wave come from LDS slots after the LDS
    // tiles', filled one step ahead while the previous step's keys travel
    // ("Keeping the Draft Walk on Chip", section "V = 248,320: 62% on chip,
    // the rest streamed": the ring keeps refilling across steps).  Only in
    // that shape is LDS left over; elsewhere the code would cost registers.
    constexpr bool kPf = kMfma && kOne && !kI8 && A == 0;
    const int PF = kPf ? p.pf_tiles : 0;
    const int wrow0 = wave * TW * kTileRows;
    const int nt_w = kMfma ? max(0, min(TW, (nrows - wrow0 + kTileRows - 1) / kTileRows)) : 0;

    // The control block (round counter, family counters, status word) and this
    // thread's anchor and temperature are requested first and used only after
    // the shard's loads have been issued, so that their round trip overlaps the
    // shard load.  A plain load: the previous launch's updates are visible at
    // a kernel boundary.
    uint4 ctl = make_uint4(0u, 0u, 0u, 0u);
    if (t == 0) ctl = *reinterpret_cast<const uint4*>(p.ws.round_ctr);
    int a_in = 0;
    float t_in = 0.0f;
    if (t < NB && t < B) {
        a_in = p.anchor[t];
        t_in = p.T[t];
    }
    // one bf16 request (the Markov head, up to 10 register tiles per wave:
    // wider shapes have no registers to spare): thread t < 32 fetches chunk t
    // of the anchor's W1 row for the first step, and the first step's base
    // logits, right after the shard's loads are issued, so that these round
    // trips overlap the shard load instead of following it
    constexpr bool kEarly = kMfma && kOne && !kI8 && !kCell && A <= 10;
    int a_pre = 0;
    if (kEarly && B > 0 && t < kRowChunks) a_pre = p.anchor[0];
    uint4 u_pre = make_uint4(0u, 0u, 0u, 0u);
    // every word this workgroup posts in this launch, both parities, starts
    // at 0 (the barriers before the first post order these stores first)
    if (t < 2 * kMailWords)
        st_agent64(p.ws.mail + ((size_t)(t / kMailWords) * kMaxGrid + c) * kMailWords + t % kMailWords, 0ull);
    else if (t < 2 * kMailWords + 2 * kMaxBatchPersistent) {
        const int i = t - 2 * kMailWords;
        st_agent64(p.ws.tokw + ((size_t)(i / kMaxBatchPersistent) * kMaxGrid + c) * kMaxBatchPersistent +
                       i % kMaxBatchPersistent, 0ull);
    }
    DSW_TRACE(gamma, 0);
    for (int j = t; j < NB * US; j += kBlock) s_u[j] = make_uint4(0u, 0u, 0u, 0u);
    // gated head: the exact split h = hi + lo + lo2 into bf16 pieces (fp32 h
    // has 24 significant bits, each piece takes the next 8), stored by thread m
    auto split_state = [&](int m, float hv) {
        uint16_t* s_x = reinterpret_cast<uint16_t*>(s_u);
        uint16_t* s_lo = reinterpret_cast<uint16_t*>(s_hp);
        const uint32_t hi = f32_to_bf16(hv);
        const float r1 = hv - bf16_to_f32(hi);
        const uint32_t lo = f32_to_bf16(r1);
        s_x[m] = (uint16_t)hi;
        s_lo[m] = (uint16_t)hi;
        s_lo[kRank + m] = (uint16_t)lo;
        s_lo[2 * kRank + m] = (uint16_t)f32_to_bf16(r1 - bf16_to_f32(lo));
    };
    if constexpr (kGated) {
        // h0 and the whole gate matrix (every workgroup updates the whole state)
        __syncthreads();  // s_u is zeroed by other threads just above
        for (int m = t; m < kRank; m += kBlock) {
            const float hv = p.h0[m];
            s_h[m] = hv;
            split_state(m, hv);  // the first gates read it (s_u is zero until the first gather)
            s_gs[m] = p.gate_scale[m];
            s_gb[m] = p.gate_bias[m];
        }
        // B-operand entry (tile * 8 + kb) * 64 + lane holds the codes of chunk
        // KC(kb, g) = 8 g + kb of row 16 tile + n (n = lane % 16, g = lane / 16),
        // widened to bf16: item (tile, lane) is the 64 contiguous codes 64 g ..
        // of that row, K blocks 0..7.  Every load is issued before any is used.
        const uint4* gq = reinterpret_cast<const uint4*>(p.gate_q);
        constexpr int kItems = (kRank / kTileRows) * 64 / kBlock;
        uint4 raw[kItems][4];
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = t + it * kBlock, ln = i & 63;
            const int m = (i >> 6) * kTileRows + (ln & 15);
#pragma unroll
            for (int q = 0; q < 4; ++q) raw[it][q] = gq[m * (kRank / 16) + 4 * (ln >> 4) + q];
        }
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int i = t + it * kBlock, ln = i & 63, tile = i >> 6;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                s_gw[(tile * 8 + 2 * q) * 64 + ln] = as_bf16x8(make_uint2(raw[it][q].x, raw[it][q].y));
                s_gw[(tile * 8 + 2 * q + 1) * 64 + ln] = as_bf16x8(make_uint2(raw[it][q].z, raw[it][q].w));
            }
        }
    }
    if constexpr (kShard) {
        // h0, and the cell rows of state elements c + i G (i < kCellMaxPerWg)
        constexpr int kRows = 2 * kGates;
        for (int m = t; m < kRank; m += kBlock) s_h[m] = p.h0[m];
        for (int e = t; e < kCellMaxPerWg * kRows * kRank; e += kBlock) {
            const int i = e / (kRows * kRank), q = (e / kRank) % kRows, m = e % kRank;
            const int j = c + i * G;
            uint16_t wv = 0;
            if (j < kRank) {
                const uint16_t* W = q < kGates ? p.gru_wih : p.gru_whh;
                wv = W[(size_t)((q % kGates) * kRank + j) * (q < kGates ? p.cell_in : kRank) + m];
            }
            s_cw[e] = wv;
        }
        if (t < kCellMaxPerWg * kRows) {
            const int i = t / kRows, q = t % kRows, j = c + i * G;
            s_cb[t] = j < kRank ? (q < kGates ? p.gru_bih : p.gru_bhh)[(q % kGates) * kRank + j] : 0.0f;
        }
    }
    if constexpr (kDomino) {
        // P[k][q] = Wih[q r + c][r .. r + d) . H[k]: thread t takes the 16-byte
        // slices t and t + kBlock of the d hidden columns (d <= 2 * 8 * kBlock),
        // eight steps' hidden states loaded at a time; fp32 sums of exact
        // products, reduced over each wave and then over the four waves
        const int d8 = p.hidden_d / 8, in8 = p.cell_in / 8;
        const uint4* Wr = reinterpret_cast<const uint4*>(p.gru_wih);
        const uint4* Hh = reinterpret_cast<const uint4*>(p.hidden);
        const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
        auto dot8 = [](const uint4 a, const uint4 b, float acc) {
            const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = fmaf(bf16_to_f32(aw[i] & 0xFFFFu), bf16_to_f32(bw[i] & 0xFFFFu), acc);
                acc = fmaf(bf16_to_f32(aw[i] >> 16), bf16_to_f32(bw[i] >> 16), acc);
            }
            return acc;
        };
        uint4 wq[3][2];
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int e8 = t + s * kBlock;
                wq[q][s] = e8 < d8 ? Wr[(size_t)(q * kRank + c) * in8 + kRank / 8 + e8] : z4;
            }
#pragma unroll 1
        for (int k0 = 0; k0 < gamma; k0 += 8) {
            uint4 hv[8][2];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int e8 = t + s * kBlock;
                    hv[kk][s] = (k0 + kk < gamma && e8 < d8) ? Hh[(size_t)(k0 + kk) * d8 + e8] : z4;
                }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    const float part = dot8(wq[q][1], hv[kk][1], dot8(wq[q][0], hv[kk][0], 0.0f));
                    const float tot = __shfl(wave_incl_scan_dpp(part), 63);
                    if (lane == 0) s_pp[(wave * kDominoMaxGamma + k0 + kk) * 3 + q] = tot;
                }
        }
        __syncthreads();
        if (t < kDominoMaxGamma * 3)
            s_P[t] = (s_pp[t] + s_pp[kDominoMaxGamma * 3 + t]) +
                     (s_pp[2 * kDominoMaxGamma * 3 + t] + s_pp[3 * kDominoMaxGamma * 3 + t]);
    }

    // ---- entry: this workgroup's shard on chip -------------------------
    WT wr[A > 0 ? A : 1][kMfma ? 8 : kRowChunks];
    uint32_t bs[kMfma ? 1 : NB][kMfma ? 1 : kMaxSlots];  // VALU: base logits of the lane's rows
    uint32_t bq[NQ];  // one request, MFMA: base logits of rows wrow0 + 64q + lane
    // one request, MFMA: does group q's row for this lane exist in the shard
#define DSW_ONE_ROW_OK(q) ((4 * (q) + (lane >> 4)) < nt_w && wrow0 + 64 * (q) + lane < nrows)
    if constexpr (kMfma && kOne && kI8) {
        // int8 codes widened to bf16 on chip, in two passes (the AGPR tiles,
        // then the VGPR tiles) so that the codes in flight and the widened
        // tiles fit in the registers together; within a pass every load is
        // issued before the first widening
        constexpr int P1 = A < kMaxRegTiles ? A : kMaxRegTiles;
        {
            uint2 raw[P1 > 0 ? P1 : 1][8];
#pragma unroll
            for (int j = 0; j < P1; ++j) {
                const int row = min(v0 + wrow0 + j * kTileRows + n, last_row);
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) raw[j][kb] = W2[(size_t)row * kRowChunks + DSW_KC(kb, g)];
            }
#pragma unroll
            for (int j = 0; j < P1; ++j)
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    wr[j][kb] = as_bf16x8(raw[j][kb]);
                    pin_agpr(wr[j][kb]);
                }
        }
        if constexpr (A > kMaxRegTiles) {
            uint2 raw[A - P1][8];
#pragma unroll
            for (int j = P1; j < A; ++j) {
                const int row = min(v0 + wrow0 + j * kTileRows + n, last_row);
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) raw[j - P1][kb] = W2[(size_t)row * kRowChunks + DSW_KC(kb, g)];
            }
#pragma unroll
            for (int j = P1; j < A; ++j)
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    wr[j][kb] = as_bf16x8(raw[j - P1][kb]);
                    pin_vgpr(wr[j][kb]);
                }
        }
    } else if constexpr (kMfma) {
#pragma unroll
        for (int j = 0; j < A; ++j) {
            // rows outside the shard load the shard's last row instead (no
            // second, zeroed copy of the registers); their results are never used
            const int row = min(v0 + wrow0 + j * kTileRows + n, last_row);
            const MT* src = W2 + (size_t)row * kRowChunks;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) wr[j][kb] = src[DSW_KC(kb, g)];
        }
        if constexpr (kEarly) {
            // an anchor out of range walks from row 0 (and is flagged below)
            const int a0 = (a_pre >= 0 && a_pre < V) ? a_pre : 0;
            if (B > 0 && t < kRowChunks) u_pre = W1[(size_t)a0 * kRowChunks + t];
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                bq[q] = (B > 0 && DSW_ONE_ROW_OK(q)) ? (uint32_t)base[v0 + wrow0 + 64 * q + lane] : 0u;
        }
        // pinned only once every tile's loads are in flight: a pin waits for
        // its registers, so pinning tile by tile would turn the shard load
        // into one memory round trip per tile
#pragma unroll
        for (int j = 0; j < A; ++j)
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                if (j < kMaxRegTiles) pin_agpr(wr[j][kb]);
                else pin_vgpr(wr[j][kb]);
            }
    }
    if constexpr (kMfma) {
        if constexpr (kOne && !kEarly) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                bq[q] = (B > 0 && DSW_ONE_ROW_OK(q)) ? (uint32_t)base[v0 + wrow0 + 64 * q + lane] : 0u;
        }
        // LDS tiles: 8 loads per thread in flight before their stores; only
        // tiles that exist in this shard have an LDS slot
        for (int i0 = 0; i0 < 4 * LT * 512; i0 += 8 * kBlock) {
            MT v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = i0 + q * kBlock + t;
                const int s = idx >> 9, kb = (idx >> 6) & 7, ln = idx & 63;
                const int ws = s / max(LT, 1);
                const int j = A + (s - ws * LT);
                const int r = ws * TW * kTileRows + j * kTileRows + (ln & 15);
                v[q] = MT{};
                if (idx < 4 * LT * 512 && j < TW && r < nrows)
                    v[q] = W2[(size_t)(v0 + r) * kRowChunks + DSW_KC(kb, ln >> 4)];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                // only tiles that exist in this shard have an LDS slot
                const int idx = i0 + q * kBlock + t;
                const int s = idx >> 9;
                const int ws = s / max(LT, 1);
                const int j = A + (s - ws * LT);
                if (idx < 4 * LT * 512 && j < TW && ws * TW * kTileRows + j * kTileRows < nrows) {
                    if constexpr (kOne && kI8) s_wt[idx] = as_bf16x8(v[q]);  // widened once
                    else s_wt[idx] = v[q];
                }
            }
        }
        if constexpr (kI8)
            for (int r = t; r < RPAD; r += kBlock) s_scale[r] = r < nrows ? p.w2_scale[v0 + r] : 0.0f;
        for (int i0 = 0; i0 < (kOne ? 0 : NB * RPAD); i0 += 8 * kBlock) {
            uint16_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = i0 + q * kBlock + t;
                const int b = idx / RPAD, r = idx - b * RPAD;
                v[q] = (idx < NB * RPAD && b < B && r < nrows) ? base[((size_t)b * gamma) * V + v0 + r] : (uint16_t)0;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int idx = i0 + q * kBlock + t;
                if (idx < NB * RPAD) s_base[idx] = v[q];
            }
        }
    } else if constexpr (kI8) {
        // int8 rows: HBM carries half the bytes; each row is widened to bf16
        // once (exact) and the walk then runs the bf16 dot products
        const uint4* __restrict__ Wq = reinterpret_cast<const uint4*>(p.W2);  // 16 codes per uint4
        // slot by slot: one slot's codes in flight, then widened (holding every
        // slot's codes at once would not fit beside the widened rows)
#pragma unroll
        for (int s = 0; s < A; ++s) {
            const int row = min(v0 + s * kBlock + t, last_row);  // rows past the shard: its last row
            uint4 qv[kRowChunks / 2];
#pragma unroll
            for (int c2 = 0; c2 < kRowChunks / 2; ++c2) qv[c2] = Wq[(size_t)row * (kRowChunks / 2) + c2];
#pragma unroll
            for (int c2 = 0; c2 < kRowChunks / 2; ++c2) {
                wr[s][2 * c2] = as_bf16x8(make_uint2(qv[c2].x, qv[c2].y));
                wr[s][2 * c2 + 1] = as_bf16x8(make_uint2(qv[c2].z, qv[c2].w));
            }
        }
        for (int j = t; j < lds_rows * (kRowChunks / 2); j += kBlock) {
            const int il = j >> 4, c2 = j & 15;
            const uint4 qv = Wq[(size_t)(v0 + reg_cap + il) * (kRowChunks / 2) + c2];
            s_w[il * kRowChunks + ((2 * c2) ^ (il & 31))] = as_bf16x8(make_uint2(qv.x, qv.y));
            s_w[il * kRowChunks + ((2 * c2 + 1) ^ (il & 31))] = as_bf16x8(make_uint2(qv.z, qv.w));
        }
        // row scales in LDS: four more registers per lane would spill the widest shape
        for (int r = t; r < RPAD; r += kBlock) s_scale[r] = r < nrows ? p.w2_scale[v0 + r] : 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxSlots; ++s) {
            const int i = s * kBlock + t;
            bs[0][s] = (B > 0 && i < nrows) ? (uint32_t)base[v0 + i] : 0u;
        }
    } else {
        // no pin here: A = 3 needs 384 registers, more than the 256 VGPRs a "v"
        // constraint would force them through; the loads land in AGPRs directly
#pragma unroll
        for (int s = 0; s < A; ++s) {
            const int i = s * kBlock + t;
            if (i < reg_rows) {
                const MT* src = W2 + (size_t)(v0 + i) * kRowChunks;
#pragma unroll
                for (int ch = 0; ch < kRowChunks; ++ch) wr[s][ch] = src[ch];
            } else {
#pragma unroll
                for (int ch = 0; ch < kRowChunks; ++ch) wr[s][ch] = make_uint4(0u, 0u, 0u, 0u);
            }

        }
        for (int j = t; j < lds_rows * kRowChunks; j += kBlock) {
            const int il = j >> 5, ch = j & 31;
            s_w[il * kRowChunks + (ch ^ (il & 31))] = W2[(size_t)(v0 + reg_cap + il) * kRowChunks + ch];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int s = 0; s < kMaxSlots; ++s) {
                const int i = s * kBlock + t;
                bs[b][s] = (b < B && i < nrows) ? (uint32_t)base[((size_t)b * gamma) * V + v0 + i] : 0u;
            }
    }
    if (t == 0) {
        s_round = ctl.x;
        s_fam = (kFamAll == 0 ? ctl.y : ctl.z);
        // a device error latched by an earlier launch stands until dsw_status
        // clears the workspace: this launch then does nothing
        s_abort = ctl.w != 0u;
    }
    if (t < NB) {
        int a = a_in;
        float temp = t_in;
        if (t < B) {
            if (a < 0 || a >= V) {
                if (c == 0) latch(status, kStatusToken);
                a = 0;
            }
            if (temp > 0.0f && p.uniforms == nullptr && !p.seeded) {
                if (c == 0) latch(status, kStatusUniforms);
                temp = 0.0f;
            }
            if (!(temp > 0.0f)) temp = 0.0f;
        }
        s_anchor[t] = a;
        s_prev[t] = a;
        s_T[t] = temp;
    }
    __syncthreads();
    if (s_abort) return;  // uniform: read after the barrier
    // diagnostics: a pseudo-random delay per workgroup before the walk, so that
    // the workgroups reach the first rendezvous in a scrambled order (a hook
    // inside the step loop measurably slowed every step, even when off)
    walk_skew(p, c, 0, 0);
    // this wave's prefetched tiles for the next step, straight into its LDS
    // slots (wave-local: the same wave reads them after its next gather);
    // rows past the shard load its last row, whose results are dropped
    auto prefetch_streamed = [&]() {
        if constexpr (kPf) {
            for (int i = 0; i < PF; ++i) {
                const int row = min(v0 + wrow0 + (A + LT + i) * kTileRows + n, last_row);
                const uint4* src = reinterpret_cast<const uint4*>(p.W2) + (size_t)row * kRowChunks;
                const uint32_t dst = lds_addr(s_w + (size_t)(4 * LT + wave * PF + i) * 512);
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) dma16(src + DSW_KC(kb, g), dst + kb * 64 * 16);
            }
        }
    };
    prefetch_streamed();
    const unsigned round = s_round;
    const unsigned fam = s_fam;
    bool any_samp = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) any_samp |= (b < B) && (s_T[b] > 0.0f);
    const int CH = (nrows + kBlock - 1) / kBlock;  // rows per thread in vocabulary-order scans

    // Gumbel-max noise of step kk for every sampled request: rows in aligned
    // groups of four ids, one Philox call per group (see gumbel_of_word)
    const int m0 = v0 >> 2;
    const int ng = nrows > 0 ? ((v0 + nrows - 1) >> 2) - m0 + 1 : 0;
    auto draw_noise = [&](int kk) {
#pragma unroll 1
        for (int b = 0; b < B; ++b) {
            if (!(s_T[b] > 0.0f)) continue;
#pragma unroll 1
            for (int gi = t; gi < ng; gi += kBlock) {
                uint32_t w[4] = {(uint32_t)(m0 + gi), ((uint32_t)kk << 8) | (uint32_t)b, round, 0x47554D42u};
                philox4(w, (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * (m0 + gi) + e - v0;
                    if (r >= 0 && r < nrows) s_G[b * RPAD + r] = gumbel_of_word(w[e]);
                }
            }
        }
    };
    if constexpr (kPreG) {
        if (any_samp && gamma > 0) draw_noise(0);  // read after the first step's barriers
    }

    // recurrent heads: wave i forms Whh h + bhh for its element c + i G from
    // the state in s_h (kGates dot products of r terms), for the coming step
    constexpr int kCellUnroll = A <= 10 ? 4 : 1;  // the widest shapes have no registers to spare
    auto cell_recurrent = [&]() {
        const int j = c + wave * G;
        if (wave < kCellMaxPerWg && j < kRank) {
            float acc[kGates];
#pragma unroll
            for (int q = 0; q < kGates; ++q) acc[q] = 0.0f;
#pragma unroll kCellUnroll
            for (int mm = 0; mm < kRank / 64; ++mm) {
                const int m = mm * 64 + lane;
                const float hv = s_h[m];
#pragma unroll
                for (int q = 0; q < kGates; ++q)
                    acc[q] = fmaf(bf16_to_f32(s_cw[(wave * 2 * kGates + kGates + q) * kRank + m]), hv, acc[q]);
            }
#pragma unroll
            for (int q = 0; q < kGates; ++q) {
                const float tot = __shfl(wave_incl_scan_dpp(acc[q]), 63);
                if (lane == 0) s_gh[wave * kGates + q] = tot + s_cb[wave * 2 * kGates + kGates + q];
            }
        }
    };
    if constexpr (kShard) {
        if (gamma > 0) cell_recurrent();  // from h0; read by the same wave in step 0
    }
    // gated head: wave w forms the gates of state elements 64 w .. 64 w + 63 for
    // the coming step on the matrix cores.  A-operand rows 0, 1, 2 carry the
    // state's three bf16 pieces, so row i of the result is the gate matrix
    // times piece i: products exact, sums in fp32, and their sum is the
    // matrix times the fp32 state.
    // Rows 3..15 of A repeat lo2: their results are never read.  K block
    // kb + 1's operands are read from LDS before block kb's products are
    // issued.  (KT tiles per pass: the widest shapes have no registers for
    // four accumulators.)
    auto gate_update = [&]() {
        constexpr int KT = A <= 10 ? 4 : 1;
        const uint4* ap = s_hp + min(lane & 15, 2) * kRowChunks + DSW_KC(0, lane >> 4);
#pragma unroll 1
        for (int t0 = 0; t0 < 4; t0 += KT) {
            const uint4* bp = s_gw + (wave * 4 + t0) * 8 * 64 + lane;
            f32x4_t d[KT];
            uint4 a = ap[0], b[KT];
#pragma unroll
            for (int tl = 0; tl < KT; ++tl) {
                d[tl] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                b[tl] = bp[tl * 8 * 64];
            }
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                uint4 a2 = a, b2[KT];
#pragma unroll
                for (int tl = 0; tl < KT; ++tl) b2[tl] = b[tl];
                if (kb + 1 < 8) {
                    a2 = ap[kb + 1];  // DSW_KC(kb + 1, g) = DSW_KC(0, g) + kb + 1
#pragma unroll
                    for (int tl = 0; tl < KT; ++tl) b2[tl] = bp[tl * 8 * 64 + (kb + 1) * 64];
                }
                __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of the products
#pragma unroll
                for (int tl = 0; tl < KT; ++tl) d[tl] = mfma_tile(a, b[tl], d[tl]);
                __builtin_amdgcn_sched_barrier(0);
                a = a2;
#pragma unroll
                for (int tl = 0; tl < KT; ++tl) b[tl] = b2[tl];
            }
            if (lane < kTileRows) {
#pragma unroll
                for (int tl = 0; tl < KT; ++tl) {
                    const int m = (wave * 4 + t0 + tl) * kTileRows + lane;
                    const float dot = (d[tl][0] + d[tl][1]) + d[tl][2];
                    s_gg[m] = 1.0f / (1.0f + expf(-(s_gs[m] * dot + s_gb[m])));
                }
            }
        }
    };
    if constexpr (kGated) {
        if (gamma > 0) gate_update();  // from h0; read after the first gather's barrier
        __syncthreads();               // every wave has read bf16(h0) before the gather replaces it
    }

    // token of request b at the end of the current step (after the winner
    // reduction and, for sampled requests, the owner's publication)
#define DSW_TOKEN(b)                                                                             \
    ((s_T[b] > 0.0f && !gum)                                                                     \
         ? s_prev[b]                                                                             \
         : checked_token(key_index(max(max(s_red64[0][b], s_red64[1][b]),                        \
                                       max(s_red64[2][b], s_red64[3][b]))),                      \
                         V, status))

    // ---- the walk --------------------------------------------------------
    for (int k = 0; k < gamma; ++k) {
        DSW_TRACE(k, kTrStepStart);
        const unsigned seq = fam * (unsigned)p.gamma_max + (unsigned)k;
        const unsigned long long epoch = epoch_of(seq);
        const int q = (int)(seq & 1u);
        unsigned long long* mail_q = p.ws.mail + (size_t)q * kMaxGrid * kMailWords;

        if constexpr (kMfma && !kOne) {
            if (k > 0) {  // this step's base logits for the shard, loads batched
                for (int b = 0; b < B; ++b) {
                    const uint16_t* src = base + ((size_t)b * gamma + k) * V + v0;
                    uint16_t v[CHMAX];
#pragma unroll
                    for (int q = 0; q < CHMAX; ++q) {
                        const int r = q * kBlock + t;
                        if (r < nrows) v[q] = src[r];
                    }
#pragma unroll
                    for (int q = 0; q < CHMAX; ++q) {
                        const int r = q * kBlock + t;
                        if (r < nrows) s_base[b * RPAD + r] = v[q];
                    }
                }
            }
        }
        // gather u = W1[prev] for every request
        if (kEarly && k == 0) {
            if (t < B * kRowChunks) s_u[t] = u_pre;  // fetched at entry
        } else {
            for (int j = t; j < B * kRowChunks; j += kBlock) {
                const int b = j >> 5, ch = j & 31;
                const int prev = (k == 0) ? s_anchor[b] : DSW_TOKEN(b);
                s_u[b * US + ch] = W1[(size_t)prev * kRowChunks + ch];
            }
        }
        if (PF > 0) wait_vmcnt(0);  // the prefetched tiles are in LDS (issued a step ago)
        __syncthreads();
        if constexpr (kGated) {
            // ---- the gated update, one state element per thread ---------------
            const uint16_t* s_x = reinterpret_cast<const uint16_t*>(s_u);  // x = W1[prev]
            const float gg = s_gg[t];
            const float hn = gg * s_h[t] + (1.0f - gg) * bf16_to_f32(s_x[t]);
            s_h[t] = hn;
            split_state(t, hn);  // bf16(h') replaces x as the GEMV operand
            if (c == 0 && p.states != nullptr) p.states[(size_t)k * kRank + t] = hn;
            __syncthreads();
        }
        if constexpr (kShard) {
            // ---- the cell: wave i updates state element c + i G ---------------
            const uint16_t* s_x = reinterpret_cast<const uint16_t*>(s_u);  // x = W1[prev]
            const int j = c + wave * G;
            unsigned long long* box = mail_q + (size_t)c * kMailWords;
            if (wave < kCellMaxPerWg && j < kRank) {
                // Wih x + bih (the recurrent half was formed ahead, in s_gh)
                float acc[kGates];
#pragma unroll
                for (int q = 0; q < kGates; ++q) acc[q] = 0.0f;
#pragma unroll kCellUnroll
                for (int mm = 0; mm < kRank / 64; ++mm) {
                    const int m = mm * 64 + lane;
                    const float xv = bf16_to_f32(s_x[m]);
#pragma unroll
                    for (int q = 0; q < kGates; ++q)
                        acc[q] = fmaf(bf16_to_f32(s_cw[(wave * 2 * kGates + q) * kRank + m]), xv, acc[q]);
                }
#pragma unroll
                for (int q = 0; q < kGates; ++q) acc[q] = __shfl(wave_incl_scan_dpp(acc[q]), 63);
                if constexpr (kDomino) {  // the hidden states' part of the input (one element, wave 0)
#pragma unroll
                    for (int q = 0; q < kGates; ++q) acc[q] += s_P[k * 3 + q];
                }
                const float* cb = s_cb + wave * 2 * kGates;
                const float* gh = s_gh + wave * kGates;
                float hn;
                if constexpr (kGru) {
                    const float rg = 1.0f / (1.0f + expf(-((acc[0] + cb[0]) + gh[0])));
                    const float zg = 1.0f / (1.0f + expf(-((acc[1] + cb[1]) + gh[1])));
                    const float ng = tanhf((acc[2] + cb[2]) + rg * gh[2]);
                    hn = (1.0f - zg) * ng + zg * s_h[j];
                } else {
                    hn = tanhf((acc[0] + cb[0]) + gh[0]);
                }
                if (lane == 0) {
                    st_agent64(&box[kStateWord + wave], ((unsigned long long)__float_as_uint(hn) << 32) | epoch);
                    if (p.states != nullptr) p.states[(size_t)k * kRank + j] = hn;
                }
            }
            // ---- gather the new state: thread m reads element m ------------------
            float hnew = 0.0f;
            {
                // as before the key polls: nothing can have arrived this early
                // (measured: GRU head, V = 151,936, gamma 7: 58.8 -> 58.1 us)
                __builtin_amdgcn_s_sleep(8);
                const unsigned long long* sbox = mail_q + (size_t)(t % G) * kMailWords + kStateWord + t / G;
                unsigned it = 0;
                unsigned long long v = 0ull;
                bool ok = true;
                while (((v = ld_agent64(sbox)) & kEpochMod) != epoch) {
                    if (++it >= p.spin_limit) {
                        latch(status, kStatusTimeout);
                        ok = false;
                        break;
                    }
                    if ((it & 255u) == 0u && ld_agent(status) != 0u) {
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (!ok) s_abort = 1;
                hnew = __uint_as_float((uint32_t)(v >> 32));
            }
            __syncthreads();  // the cell has read x and h
            if (s_abort) break;
            s_h[t] = hnew;  // kBlock == kRank: one element per thread
            reinterpret_cast<uint16_t*>(s_u)[t] = (uint16_t)f32_to_bf16(hnew);
            __syncthreads();
        }
        DSW_TRACE(k, kTrGathered);

        uint32_t best[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) best[i] = 0u;

        if constexpr (kMfma) {
            // A operand: lane l carries u of request l%16, latent 8*(l/16).. of each K block
            uint4 a[8];
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) a[kb] = (n < B) ? s_u[n * US + DSW_KC(kb, g)] : make_uint4(0u, 0u, 0u, 0u);
          if constexpr (kOne) {
            if constexpr (A <= 10) {
                // Groups of four tiles: four independent MFMA chains, gathered into
                // one register, then one 64-lane epilogue.  Register tiles are
                // multiplied even beyond nt_w (they hold valid rows; results are
                // masked), LDS and streamed tiles only where they exist.  Up to 10
                // register tiles per wave, groups that start with a register tile
                // run without a branch, and every epilogue is branch-free, so that
                // the scheduler can overlap one group's epilogue with the next
                // group's MFMAs (the wider shapes have no registers for it).
#pragma unroll
                for (int gq = 0; gq < NQ; ++gq) {
                    if (4 * gq < A || 4 * gq < nt_w) {
                        f32x4_t d[4];
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int j = 4 * gq + jj;
                            d[jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                            if (j < A) {
#pragma unroll
                                for (int kb = 0; kb < 8; ++kb) d[jj] = mfma_tile(a[kb], wr[j < A ? j : 0][kb], d[jj]);
                            } else if (j < M && j < nt_w) {
                                if (j - A < LT) {
                                    const int sb = (wave * LT + (j - A)) * 512 + lane;
#pragma unroll
                                    for (int kb = 0; kb < 8; ++kb) d[jj] = mfma_tile(a[kb], s_w[sb + kb * 64], d[jj]);
                                } else if (j - A - LT < PF) {
                                    const int sb = (4 * LT + wave * PF + (j - A - LT)) * 512 + lane;
#pragma unroll
                                    for (int kb = 0; kb < 8; ++kb) d[jj] = mfma_tile(a[kb], s_w[sb + kb * 64], d[jj]);
                                } else {
                                    const int r = wrow0 + j * kTileRows + n;
                                    const bool ok = r < nrows;
                                    const MT* src = W2 + (size_t)(v0 + (ok ? r : 0)) * kRowChunks;
#pragma unroll
                                    for (int kb = 0; kb < 8; ++kb)
                                        d[jj] = mfma_tile(a[kb], ok ? as_bf16x8(src[DSW_KC(kb, g)]) : make_uint4(0u, 0u, 0u, 0u),
                                                          d[jj]);
                                }
                            }
                        }
                        const float acc1 = combine4(d[0][0], d[1][0], d[2][0], d[3][0]);
                        const bool ok = DSW_ONE_ROW_OK(gq);
                        const int r = wrow0 + 64 * gq + lane;
                        const float bias = bias_round(kI8 ? s_scale[ok ? r : 0] * acc1 : acc1, dbl_round);
                        const uint32_t lbits = f32_to_bf16(bf16_to_f32(bq[gq]) + bias);
                        const uint32_t key = local_key(lbits, r);
                        best[0] = ok ? max(best[0], key) : best[0];
                        *(ok ? &s_logit[r] : &s_lj[lane]) = (uint16_t)lbits;  // lanes past the shard: junk
                    }
                }
            } else {
                // the same with a branch per group and per epilogue (12 register
                // tiles per wave leave no registers for the straight-line form)
#pragma unroll
                for (int gq = 0; gq < NQ; ++gq) {
                    if (4 * gq < nt_w) {
                        f32x4_t d[4];
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int j = 4 * gq + jj;
                            d[jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                            if (j < A) {
#pragma unroll
                                for (int kb = 0; kb < 8; ++kb) d[jj] = mfma_tile(a[kb], wr[j < A ? j : 0][kb], d[jj]);
                            } else if (j < M && j < nt_w) {
                                if (j - A < LT) {
                                    const int sb = (wave * LT + (j - A)) * 512 + lane;
#pragma unroll
                                    for (int kb = 0; kb < 8; ++kb) d[jj] = mfma_tile(a[kb], s_w[sb + kb * 64], d[jj]);
                                } else if (j - A - LT < PF) {
                                    const int sb = (4 * LT + wave * PF + (j - A - LT)) * 512 + lane;
#pragma unroll
                                    for (int kb = 0; kb < 8; ++kb) d[jj] = mfma_tile(a[kb], s_w[sb + kb * 64], d[jj]);
                                } else {
                                    const int r = wrow0 + j * kTileRows + n;
                                    const bool ok = r < nrows;
                                    const MT* src = W2 + (size_t)(v0 + (ok ? r : 0)) * kRowChunks;
#pragma unroll
                                    for (int kb = 0; kb < 8; ++kb)
                                        d[jj] = mfma_tile(a[kb], ok ? as_bf16x8(src[DSW_KC(kb, g)]) : make_uint4(0u, 0u, 0u, 0u),
                                                          d[jj]);
                                }
                            }
                        }
                        const float acc1 = combine4(d[0][0], d[1][0], d[2][0], d[3][0]);
                        if (DSW_ONE_ROW_OK(gq)) {
                            const int r = wrow0 + 64 * gq + lane;
                            const float bias = bias_round(kI8 ? s_scale[r] * acc1 : acc1, dbl_round);
                            const uint32_t lbits = f32_to_bf16(bf16_to_f32(bq[gq]) + bias);
                            best[0] = max(best[0], local_key(lbits, r));
                            s_logit[r] = (uint16_t)lbits;
                        }
                    }
                }
            }
            // the next step's base logits land while the rendezvous is in flight
            if (k + 1 < gamma) {
#pragma unroll
                for (int gq = 0; gq < NQ; ++gq)
                    bq[gq] = DSW_ONE_ROW_OK(gq)
                                 ? (uint32_t)base[(size_t)(k + 1) * V + v0 + wrow0 + 64 * gq + lane]
                                 : 0u;
            }
          } else {
            const int lofs = 4 * g * RPAD + wrow0 + n;
#define DSW_EPI_MFMA(dv, j)                                                                      \
    do {                                                                                         \
        const int r_ = wrow0 + (j) * kTileRows + n;                                              \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                          \
            if (4 * g + i < B && r_ < nrows) {                                                   \
                const int e_ = lofs + i * RPAD + (j) * kTileRows;                                \
                const float a_ = kI8 ? s_scale[r_] * (dv)[i] : (dv)[i];                          \
                const float bias_ = bias_round(a_, dbl_round);                                   \
                const uint32_t lb_ = f32_to_bf16(bf16_to_f32(s_base[e_]) + bias_);               \
                best[i] = max(best[i], local_key(lb_, r_));                                      \
                s_logit[e_] = (uint16_t)lb_;                                                     \
            }                                                                                    \
        }                                                                                        \
    } while (0)
            // Register tiles two at a time, each pair's epilogue right after its
            // MFMAs, so that few accumulators and widened operands are live.
            // Tiles beyond nt_w hold other rows: multiplying them keeps the MFMA
            // sequence free of branches, and their results are dropped.
#pragma unroll
            for (int j0 = 0; j0 < A; j0 += 2) {
                f32x4_t d0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, d1 = d0;
                if constexpr (kI8) {
                    // opaque every step, so that the widening to bf16 is not
                    // hoisted out of the walk (that would hold twice the registers)
#pragma unroll
                    for (int j = j0; j < j0 + 2 && j < A; ++j)
#pragma unroll
                        for (int kb = 0; kb < 8; ++kb) pin_agpr(wr[j][kb]);
                }
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    d0 = mfma_tile(a[kb], as_bf16x8(wr[j0][kb]), d0);
                    if (j0 + 1 < A) d1 = mfma_tile(a[kb], as_bf16x8(wr[j0 + 1][kb]), d1);
                }
                if (j0 < nt_w) DSW_EPI_MFMA(d0, j0);
                if (j0 + 1 < A && j0 + 1 < nt_w) DSW_EPI_MFMA(d1, j0 + 1);
                __builtin_amdgcn_sched_barrier(0);  // keep the pairs apart
            }
#pragma unroll 1
            for (int j = A; j < M; ++j) {
                if (j < nt_w) {
                    f32x4_t dd = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    if (j - A < LT) {
                        const int sb = (wave * LT + (j - A)) * 512 + lane;
#pragma unroll
                        for (int kb = 0; kb < 8; ++kb) dd = mfma_tile(a[kb], as_bf16x8(s_wt[sb + kb * 64]), dd);
                    } else {
                        const int r = wrow0 + j * kTileRows + n;
                        const bool ok = r < nrows;
                        const MT* src = W2 + (size_t)(v0 + (ok ? r : 0)) * kRowChunks;
#pragma unroll
                        for (int kb = 0; kb < 8; ++kb)
                            dd = mfma_tile(a[kb], as_bf16x8(ok ? src[DSW_KC(kb, g)] : MT{}), dd);
                    }
                    DSW_EPI_MFMA(dd, j);
                }
            }
#undef DSW_EPI_MFMA
          }
        } else {
            float acc[NB][kMaxSlots];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int s = 0; s < kMaxSlots; ++s) acc[b][s] = 0.0f;
            if (A > 0) {
                if constexpr (NB == 1) {
                    // u read kUPre chunks ahead of its dot products: each LDS read
                    // is in flight while earlier chunks are multiplied (the
                    // scheduling barriers keep the compiler from sinking the
                    // reads back next to their use)
                    constexpr int kUPre = 2;
                    uint4 ub[kUPre + 1];
#pragma unroll
                    for (int q = 0; q < kUPre; ++q) ub[q] = s_u[q];
#pragma unroll
                    for (int ch = 0; ch < kRowChunks; ++ch) {
                        if (ch + kUPre < kRowChunks) ub[(ch + kUPre) % (kUPre + 1)] = s_u[ch + kUPre];
                        __builtin_amdgcn_sched_barrier(0);
                        const uint4 u4 = ub[ch % (kUPre + 1)];
#pragma unroll
                        for (int s = 0; s < A; ++s) acc[0][s] = dot8(wr[s][ch], u4, acc[0][s]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
#pragma unroll
                    for (int ch = 0; ch < kRowChunks; ++ch) {
#pragma unroll
                        for (int b = 0; b < NB; ++b) {
                            if (b < B) {
                                const uint4 u4 = s_u[b * US + ch];
#pragma unroll
                                for (int s = 0; s < A; ++s) acc[b][s] = dot8(wr[s][ch], u4, acc[b][s]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int s = A; s < kMaxSlots; ++s) {
                const int i = s * kBlock + t;
                if (i < nrows) {
                    const int il = i - reg_cap;
                    // weights in groups of kGrp chunks: every load of a group is
                    // issued before the first dot product waits on it
                    constexpr int kGrp = NB == 16 ? 4 : 8;
                    if (il < lds_rows) {
#pragma unroll 1
                        for (int c0 = 0; c0 < kRowChunks; c0 += kGrp) {
                            uint4 w4[kGrp];
#pragma unroll
                            for (int q = 0; q < kGrp; ++q) w4[q] = s_w[il * kRowChunks + ((c0 + q) ^ (il & 31))];
#pragma unroll
                            for (int q = 0; q < kGrp; ++q)
#pragma unroll
                                for (int b = 0; b < NB; ++b)
                                    if (NB == 1 || b < B) acc[b][s] = dot8(w4[q], s_u[b * US + c0 + q], acc[b][s]);
                        }
                    } else {
                        const MT* src = W2 + (size_t)(v0 + i) * kRowChunks;
                        const uint2* srcq = reinterpret_cast<const uint2*>(p.W2) + (size_t)(v0 + i) * kRowChunks;
#pragma unroll 1
                        for (int c0 = 0; c0 < kRowChunks; c0 += kGrp) {
                            uint4 w4[kGrp];
#pragma unroll
                            for (int q = 0; q < kGrp; ++q) {
                                if constexpr (kI8) w4[q] = as_bf16x8(srcq[c0 + q]);
                                else w4[q] = src[c0 + q];
                            }
#pragma unroll
                            for (int q = 0; q < kGrp; ++q)
#pragma unroll
                                for (int b = 0; b < NB; ++b)
                                    if (NB == 1 || b < B) acc[b][s] = dot8(w4[q], s_u[b * US + c0 + q], acc[b][s]);
                        }
                    }
                }
            }
            // int8: the scale reads stay after the dot products (issued earlier,
            // they would be live across the GEMV and spill the widest shape)
            if constexpr (kI8) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
#pragma unroll
                for (int s = 0; s < kMaxSlots; ++s) {
                    const int i = s * kBlock + t;
                    if ((NB == 1 || b < B) && i < nrows) {
                        float a = acc[b][s];
                        if constexpr (kI8) a *= s_scale[i];
                        // double rounding (the default walk's), or one rounding of the sum
                        const float bias = bias_round(a, dbl_round);
                        const uint32_t lbits = f32_to_bf16(bf16_to_f32(bs[b][s]) + bias);
                        best[b] = max(best[b], local_key(lbits, i));
                        s_logit[b * RPAD + i] = (uint16_t)lbits;
                    }
                }
            }
            // the next step's base logits land while the rendezvous is in flight
            if (k + 1 < gamma) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int s = 0; s < kMaxSlots; ++s) {
                        const int i = s * kBlock + t;
                        bs[b][s] = (b < B && i < nrows)
                                       ? (uint32_t)base[((size_t)b * gamma + k + 1) * V + v0 + i]
                                       : 0u;
                    }
            }
        }
        DSW_TRACE(k, kTrGemvDone);

        // workgroup argmax per request: DPP within the wave, then 4 waves via LDS
        if constexpr (kMfma && !kOne) {
#pragma unroll
            for (int i = 0; i < 4; ++i) best[i] = row16_max_u32(best[i]);
            if (n == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i < NB) s_wbest[wave][4 * g + i] = best[i];
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint32_t m = wave_max_u32(best[b]);
                if (lane == 0) s_wbest[wave][b] = m;
            }
        }
        __syncthreads();
        DSW_TRACE(k, kTrReduced);

        // Gumbel-max (sampled requests): the shard's best key {ord32(l / T + G),
        // ~id}, rows in aligned groups of four ids, one Philox call per group
        unsigned long long* s_gk = reinterpret_cast<unsigned long long*>(s_S);  // [4][NB]
        if (any_samp && gum) {
#pragma unroll 1
            for (int b = 0; b < B; ++b) {
                if (!(s_T[b] > 0.0f)) continue;
                const float invT = 1.0f / s_T[b];
                unsigned long long bk = 0ull;
                if constexpr (kPreG) {  // the noise is already in LDS
#pragma unroll 1
                    for (int r = t; r < nrows; r += kBlock) {
                        const float sc = bf16_to_f32(s_logit[b * RPAD + r]) * invT + s_G[b * RPAD + r];
                        const unsigned long long key = ((unsigned long long)ord32(sc) << kIdxBits) |
                                                       (unsigned long long)(kIdxMask - (uint32_t)(v0 + r));
                        bk = key > bk ? key : bk;
                    }
                }
#pragma unroll 1
                for (int gi = t; gi < (kPreG ? 0 : ng); gi += kBlock) {
                    uint32_t w[4] = {(uint32_t)(m0 + gi), ((uint32_t)k << 8) | (uint32_t)b, round, 0x47554D42u};
                    philox4(w, (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = 4 * (m0 + gi) + e;
                        const int r = v - v0;
                        if (r >= 0 && r < nrows) {
                            const float sc = bf16_to_f32(s_logit[b * RPAD + r]) * invT + gumbel_of_word(w[e]);
                            const unsigned long long key =
                                ((unsigned long long)ord32(sc) << kIdxBits) | (unsigned long long)(kIdxMask - (uint32_t)v);
                            bk = key > bk ? key : bk;
                        }
                    }
                }
                bk = wave_max_u64_dpp(bk);
                if (lane == 0) s_gk[wave * NB + b] = bk;
            }
            __syncthreads();
        }

        // sampled requests: masses w = exp((l - m_c) / T) of the shard's rows in
        // vocabulary order, CH consecutive rows per thread
        if (any_samp && !gum) {
            float part[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                part[b] = 0.0f;
                if (b < B && s_T[b] > 0.0f) {
                    const uint32_t lk = max(max(s_wbest[0][b], s_wbest[1][b]), max(s_wbest[2][b], s_wbest[3][b]));
                    const float ml = local_key_logit(lk);
                    const float Tb = s_T[b];
#pragma unroll
                    for (int rr = 0; rr < CHMAX; ++rr) {
                        const int r = t * CH + rr;
                        if (rr < CH && r < nrows)
                            part[b] += __expf((bf16_to_f32(s_logit[b * RPAD + r]) - ml) / Tb);
                    }
                }
            }
            float incl[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                incl[b] = 0.0f;
                if (b < B && s_T[b] > 0.0f) {
                    incl[b] = wave_incl_scan_dpp(part[b]);
                    if (lane == 63) s_redf[wave][b] = incl[b];
                }
            }
            __syncthreads();
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b < B && s_T[b] > 0.0f) {
                    float off = 0.0f, tot = 0.0f;
                    for (int w = 0; w < 4; ++w) {
                        if (w < wave) off += s_redf[w][b];
                        tot += s_redf[w][b];
                    }
                    s_excl[b * kBlock + t] = off + (incl[b] - part[b]);
                    if (t == 0) s_tot[b] = tot;
                }
            }
        }

        // ---- rendezvous: post, write the logits out, read every mailbox ------
        if (wave == 0 && lane < B) {
            const uint32_t lk = max(max(s_wbest[0][lane], s_wbest[1][lane]), max(s_wbest[2][lane], s_wbest[3][lane]));
            unsigned long long* box = mail_q + (size_t)c * kMailWords;
            if (gum && s_T[lane] > 0.0f) {
                // Gumbel-max: {score, epoch} and {~id, epoch}
                const unsigned long long gk = max(max(s_gk[lane], s_gk[NB + lane]),
                                                  max(s_gk[2 * NB + lane], s_gk[3 * NB + lane]));
                st_agent64(&box[kMailKeys + lane], ((gk >> kIdxBits) << 32) | epoch);
                st_agent64(&box[kSumWord + lane], ((gk & kIdxMask) << 32) | epoch);
            } else {
                st_agent64(&box[kMailKeys + lane], (global_key(lk, v0) << 28) | epoch);
                if (s_T[lane] > 0.0f)
                    st_agent64(&box[kSumWord + lane],
                               ((unsigned long long)__float_as_uint(s_tot[lane]) << 32) | epoch);
            }
        }
        DSW_TRACE(k, kTrPosted);
        if (k + 1 < gamma) prefetch_streamed();  // the next step's, while the keys travel
        // the previous step's tokens, stored while this step's rendezvous is in
        // flight (a store at the end of a step would hold up the next gather)
        if (c == 0 && k > 0 && t < B) p.tokens[(size_t)t * gamma + k - 1] = DSW_TOKEN(t);
        if (p.logits != nullptr) {  // the exact values the tokens are selected from
            for (int b = 0; b < B; ++b) {
                uint16_t* dst = p.logits + ((size_t)b * gamma + k) * V + v0;
                for (int r = t; r < nrows; r += kBlock) dst[r] = s_logit[b * RPAD + r];
            }
        }
        if constexpr (kPreG) {
            // the next step's noise, while this step's words travel (this
            // step's noise was last read before the barrier ahead of the post)
            if (any_samp && k + 1 < gamma) draw_noise(k + 1);
        }
        if constexpr (kShard) {
            // the next step's recurrent half from this step's state, while the keys travel
            if (k + 1 < gamma) cell_recurrent();
        }
        // Up to 4 requests: two polls in flight, each check waiting only for the
        // older load, so a word that lands is seen about half a round trip
        // sooner than with one poll at a time.  16 requests: one poll at a time
        // (a second set of words would not fit in registers).  Thread t < G
        // reads workgroup t's mailbox.
        constexpr int kDepth = NB <= 4 ? 2 : 1;
        // ~0.2 us before the first poll: no word can have arrived yet, and
        // polls issued meanwhile (256 per workgroup) only slow the posts
        // through the fabric (measured: V = 151,936, gamma 7: 38.9 -> 37.5
        // us; V = 32,000: 25.8 -> 23.7 us; gamma 16 mixed T: 125 -> 107 us)
        __builtin_amdgcn_s_sleep(8);
        const unsigned long long* box = mail_q + (size_t)t * kMailWords;
        unsigned long long pa[kDepth == 2 ? NB : 1][2], pb[kDepth == 2 ? NB : 1][2];
        bool smp[NB];  // requests with a second word (in registers: no LDS read per poll)
#pragma unroll
        for (int b = 0; b < NB; ++b) smp[b] = s_T[b] > 0.0f;
#define DSW_POLL(WV)                                                                       \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                       \
        if (NB == 1 || b < B) {                                                            \
            WV[b][0] = ld_agent64(&box[kMailKeys + b]);                                    \
            if (smp[b]) WV[b][1] = ld_agent64(&box[kSumWord + b]);                         \
        }                                                                                  \
    }
        if constexpr (kGated) {
            // the first polls go out, then the next step's gates are formed while
            // the keys travel
            static_assert(kDepth == 2, "gated head: one request");
            if (t < G) DSW_POLL(pa);
            if (k + 1 < gamma) gate_update();
        }
        unsigned long long kw[NB];
        uint32_t sw[NB];  // the second word's payload: exp-sum bits, or ~id (Gumbel-max)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            kw[b] = 0ull;
            sw[b] = 0u;
        }
        if (t < G) {
#define DSW_READY(w, ready)                                                                \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                       \
        if (NB == 1 || b < B) {                                                            \
            if ((w[b][0] & kEpochMod) == epoch) kw[b] = w[b][0] >> 28;                     \
            else ready = false;                                                            \
            if (smp[b]) {                                                                  \
                if ((w[b][1] & kEpochMod) == epoch) sw[b] = (uint32_t)(w[b][1] >> 32);          \
                else ready = false;                                                        \
            }                                                                              \
        }                                                                                  \
    }
            unsigned it = 0;
            if (kPair && smp[0]) {
                // one request with a second word: both with one 16-byte load
                // per poll (its own loop, so that the one-word loop below keeps
                // two polls in flight)
                for (;;) {
                    unsigned long long w0, w1;
                    ld_agent64_pair(&box[kMailKeys], w0, w1);
                    if ((w0 & kEpochMod) == epoch && (w1 & kEpochMod) == epoch) {
                        kw[0] = w0 >> 28;
                        sw[0] = (uint32_t)(w1 >> 32);
                        break;
                    }
                    if (++it >= p.spin_limit) {
                        latch(status, kStatusTimeout);
                        s_abort = 1;
                        break;
                    }
                    if ((it & 127u) == 0u && ld_agent(status) != 0u) {
                        s_abort = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            } else {
            if constexpr (kDepth == 2 && !kGated) DSW_POLL(pa);  // (the gated head polled above)
            for (;;) {
                if constexpr (kDepth == 2) {
                    DSW_POLL(pb);
                    bool ready = true;
                    DSW_READY(pa, ready);
                    if (ready) break;
                    __builtin_amdgcn_s_sleep(1);
                    DSW_POLL(pa);
                    ready = true;
                    DSW_READY(pb, ready);
                    if (ready) break;
                } else {
                    bool ready = true;
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if (b < B) {
                            const unsigned long long wk = ld_agent64(&box[kMailKeys + b]);
                            if ((wk & kEpochMod) == epoch) kw[b] = wk >> 28;
                            else ready = false;
                            if (smp[b]) {
                                const unsigned long long ws = ld_agent64(&box[kSumWord + b]);
                                if ((ws & kEpochMod) == epoch) sw[b] = (uint32_t)(ws >> 32);
                                else ready = false;
                            }
                        }
                    }
                    if (ready) break;
                }
                if (++it >= p.spin_limit) {
                    latch(status, kStatusTimeout);
                    s_abort = 1;
                    break;
                }
                if ((it & 127u) == 0u && ld_agent(status) != 0u) {
                    s_abort = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            }
#undef DSW_POLL
#undef DSW_READY
        }
        DSW_TRACE(k, kTrArrived);
        if (any_samp && gum) {
            // Gumbel-max keys {score (32), ~id (20)}: ~id is decoded like a greedy key's
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if ((NB == 1 || b < B) && s_T[b] > 0.0f) kw[b] = ((kw[b] >> 4) << kIdxBits) | sw[b];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const unsigned long long m = wave_max_u64_dpp(kw[b]);
            if (lane == 0) s_red64[wave][b] = m;
        }
        __syncthreads();
        if (s_abort) break;

        // ---- sampled requests: owner shard of u*Z ------------------------
        // Every workgroup derives the same owner from the same mailbox words
        // with the same code, so they agree without another exchange.
        if (any_samp && !gum) {
            // shard masses S_c = s_c * exp((m_c - M) / T), one request per row of s_S
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if ((b < B) && (s_T[b] > 0.0f)) {
                    const unsigned long long win =
                        max(max(s_red64[0][b], s_red64[1][b]), max(s_red64[2][b], s_red64[3][b]));
                    float S = 0.0f;
                    if (t < G && kw[b] != 0ull) S = __uint_as_float(sw[b]) * __expf((key_logit(kw[b]) - key_logit(win)) / s_T[b]);
                    s_S[b * kBlock + t] = S;
                }
            }
            __syncthreads();
            // wave w scans the shard masses of requests w, w + 4, ...; lane l holds
            // shards 4l .. 4l+3.  The owner is the first shard with positive mass
            // whose inclusive prefix exceeds u*Z, else the last one with positive mass.
            for (int b = wave; b < B; b += 4) {
                if (!(s_T[b] > 0.0f)) continue;
                const float4 m4 = reinterpret_cast<const float4*>(s_S + b * kBlock)[lane];
                const float q0 = m4.x, q1 = q0 + m4.y, q2 = q1 + m4.z, q3 = q2 + m4.w;
                const float incl = wave_incl_scan_dpp(q3);
                const float ex = incl - q3;
                const float Z = __shfl(incl, 63);
                const float target = walk_uniform(p, b, k, gamma, round) * Z;
                const float c4[4] = {ex + q0, ex + q1, ex + q2, ex + q3};
                const float w4[4] = {m4.x, m4.y, m4.z, m4.w};
                uint32_t first = 0u, lastp = 0u;  // shard + 1, 0 = none
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    if (w4[i] > 0.0f && c4[i] > target) first = (uint32_t)(4 * lane + i) + 1u;
                    if (lastp == 0u && w4[i] > 0.0f) lastp = (uint32_t)(4 * lane + i) + 1u;
                }
                const uint32_t fmin = wave_max_u32(first ? 0xFFFFFFFFu - first : 0u);
                const uint32_t lmax = wave_max_u32(lastp);
                const int owner = fmin ? (int)(0xFFFFFFFFu - fmin) - 1 : (int)lmax - 1;
                // exclusive prefix of the owner: c4 of shard owner - 1
                const int pj = max(owner - 1, 0);
                const float cj = (pj & 3) == 0 ? c4[0] : ((pj & 3) == 1 ? c4[1] : ((pj & 3) == 2 ? c4[2] : c4[3]));
                const float pexcl = __shfl(cj, pj >> 2);
                if (lane == 0) {
                    s_own[b] = owner;
                    s_pex[b] = owner > 0 ? pexcl : 0.0f;
                    s_tgt[b] = target;
                    s_Mg[b] = key_logit(max(max(s_red64[0][b], s_red64[1][b]), max(s_red64[2][b], s_red64[3][b])));
                }
            }
            __syncthreads();
            // the owner finds the token inside its rows and publishes it
            for (int b = 0; b < B; ++b) {
                if (!(s_T[b] > 0.0f) || s_own[b] != c) continue;
                const float Tb = s_T[b];
                const float target = s_tgt[b];
                const float pexcl = s_pex[b];
                const uint32_t lk = max(max(s_wbest[0][b], s_wbest[1][b]), max(s_wbest[2][b], s_wbest[3][b]));
                const float ml = local_key_logit(lk);
                const float scale = __expf((ml - s_Mg[b]) / Tb);
                float run = s_excl[b * kBlock + t];
                uint32_t first = 0u, lastw = 0u;  // row + 1, 0 = none
#pragma unroll
                for (int rr = 0; rr < CHMAX; ++rr) {
                    const int r = t * CH + rr;
                    if (rr < CH && r < nrows) {
                        const float w = __expf((bf16_to_f32(s_logit[b * RPAD + r]) - ml) / Tb);
                        run += w;
                        if (first == 0u && pexcl + scale * run > target) first = (uint32_t)r + 1u;
                        if (w > 0.0f) lastw = (uint32_t)r + 1u;
                    }
                }
                // smallest crossing row: max over the complement
                const uint32_t fmin = wave_max_u32(first ? 0xFFFFFFFFu - first : 0u);
                const uint32_t lmax = wave_max_u32(lastw);
                if (lane == 0) {
                    s_redi[wave] = (int)fmin;
                    s_redj[wave] = (int)lmax;
                }
                __syncthreads();
                uint32_t fm = 0u, lm = 0u;
                for (int w = 0; w < 4; ++w) {
                    fm = max(fm, (uint32_t)s_redi[w]);
                    lm = max(lm, (uint32_t)s_redj[w]);
                }
                // no crossing row (rounding): the last row with positive mass;
                // none at all cannot happen for the owner, flag it if it does
                const int row = fm ? (int)(0xFFFFFFFFu - fm) - 1 : (lm ? (int)lm - 1 : -1);
                const int tok = checked_token(row < 0 ? -1 : v0 + row, V, status);
                __syncthreads();
                if (t == 0) s_prev[b] = tok;
                if (t == b) {  // into this workgroup's own row of token words
                    st_agent64(p.ws.tokw + ((size_t)q * kMaxGrid + c) * kMaxBatchPersistent + b,
                               ((unsigned long long)(unsigned)tok << 32) | epoch);
                }
            }
            // every other sampled request: thread b reads its owner's token word
            if (t < B && s_T[t] > 0.0f && s_own[t] != c) {
                // (an owner of -1, no shard with mass, cannot occur: the winner's
                // shard always has mass >= 1; the clamp keeps the read in bounds)
                const unsigned long long* tbox =
                    p.ws.tokw + ((size_t)q * kMaxGrid + max(s_own[t], 0)) * kMaxBatchPersistent + t;
                unsigned it = 0;
                unsigned long long v = 0ull;
                bool ok = true;
                while (((v = ld_agent64(tbox)) & kEpochMod) != epoch) {
                    if (++it >= p.spin_limit) {
                        latch(status, kStatusTimeout);
                        ok = false;
                        break;
                    }
                    if ((it & 255u) == 0u && ld_agent(status) != 0u) {
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (!ok) s_abort = 1;
                s_prev[t] = ok ? checked_token((int)(v >> 32), V, status) : 0;
            }
            __syncthreads();
            if (s_abort) break;
        }
        DSW_TRACE(k, kTrSelected);
        DSW_TRACE_REAL(k);
    }
    if (PF > 0) wait_vmcnt(0);  // no LDS load may land after the workgroup ends
    if (c == 0 && t < B && !s_abort && gamma > 0) p.tokens[(size_t)t * gamma + gamma - 1] = DSW_TOKEN(t);
#undef DSW_TOKEN
#undef DSW_ONE_ROW_OK

    DSW_TRACE_FLUSH();
    if (c == 0 && t == 0 && !s_abort) {
        __hip_atomic_fetch_add(p.ws.round_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(p.ws.fam_ctr + kFamAll, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// (register tiles, tiles per wave) shapes of the MFMA engine, per batch tile
#define DSW_MFMA_SHAPES(X) X(2, 2) X(4, 4) X(8, 8) X(8, 10) X(8, 16) X(0, 16)
// the same for int8 weights (a tile row is half as large)
#define DSW_MFMA_I8_SHAPES(X) X(4, 4) X(8, 8) X(16, 16) X(0, 16)
// one request: up to kMaxRegTiles AGPR tiles plus kMaxVgprTiles VGPR tiles per wave
#define DSW_MFMA_ONE_SHAPES(X) X(2, 2) X(4, 4) X(8, 8) X(10, 10) X(12, 12) X(12, 16) X(0, 16)

}  // namespace dsw
