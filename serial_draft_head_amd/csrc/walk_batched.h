// walk_batched.h -- one persistent launch per round of DSpark's serial Markov
// draft walk for large batches (up to 256 requests), on gfx950 (MI355X).
//
// The per-request computation is the one of walk_kernel.h ("Keeping the Draft
// Walk on Chip", tie-pilot-qxw.github.io, section "The serial part of a
// parallel drafter"; sampler of vLLM PR #64442, "Details").  What changes with
// the batch size (section "B200: the bf16 table fits on chip": batching is
// almost free for the matrix cores, everything around the GEMV grows):
//
// * GEMV: requests go through in groups of 16.  A weight tile is the A operand
//   of v_mfma_f32_16x16x32_bf16 (16 rows x 32 latent values, the same register
//   layout as walk_kernel.h) and the u vectors of the group are the B operand,
//   so lane (n, g) ends with rows 4g .. 4g+3 of a tile for request n: four
//   adjacent base logits, one 8-byte LDS read.
// * Streaming: every step reads B * rows * 2 bytes of base logits per shard.
//   The u rows and base logits of a group go straight from memory into a ring
//   of LDS slots (global_load_lds_dwordx4), several groups ahead, while the
//   matrix cores work on the current group; XOR swizzles keep the 16 lanes of
//   one request column on distinct LDS banks.
// * Exchange: an all-to-all of B keys per workgroup would read B * 2 KiB per
//   workgroup and step.  Here request b is owned by workgroup b % G: every
//   workgroup stores its B key words (and exp-sum words) in one row, the owner
//   reads column b and publishes the token in one word.  Greedy: the best key.
//   Sampled: the owner finds the shard whose mass holds u*Z and the mass that
//   shard accumulates, in its own scale, before the token, reads that shard's
//   logits of request b (every shard writes the logits of its groups with a
//   sampled request to the workspace with agent-scope stores before its key
//   words) and scans them for the token.  Gumbel-max: the owner reduces
//   {score, ~id} words.  Every step takes two exchanges.
#pragma once
#include "walk_kernel.h"

namespace dsw {

constexpr int kSlotUBytes = kGroup * kRowChunks * 16;  // u rows of one group: 8 KiB
// Decision words carry a 24-bit epoch, (seq mod 2^23) + 1: never 0, and two
// steps share it only 2^23 steps apart (the words a reader can meet are fewer
// than 2 gamma_max <= 8192 steps apart).  Above it: the request's token
// (bits 24..43).
constexpr unsigned long long kDecEpochMask = 0xFFFFFFull;
__device__ __forceinline__ unsigned long long dec_epoch(unsigned seq) { return (seq & 0x7FFFFFu) + 1u; }

// Four 16x16 results whose columns 0..3 alone are needed: lane column 4q + b
// of each 16-lane row takes column b of t_q (DPP row shifts by 4q, written
// into bank q only).
__device__ __forceinline__ f32x4_t fold4(const f32x4_t& t0, const f32x4_t& t1, const f32x4_t& t2,
                                         const f32x4_t& t3) {
    f32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int v = __float_as_int(t0[i]);
        v = __builtin_amdgcn_update_dpp(v, __float_as_int(t1[i]), 0x114, 0xF, 0x2, false);  // row_shr:4
        v = __builtin_amdgcn_update_dpp(v, __float_as_int(t2[i]), 0x118, 0xF, 0x4, false);  // row_shr:8
        v = __builtin_amdgcn_update_dpp(v, __float_as_int(t3[i]), 0x11C, 0xF, 0x8, false);  // row_shr:12
        r[i] = __int_as_float(v);
    }
    return r;
}
// column4_max_u32 for 64-bit keys (both halves through the same swaps)
__device__ __forceinline__ unsigned long long column4_max_u64(unsigned long long x) {
    const auto ah = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
    const auto al = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    const unsigned long long a0 = ((unsigned long long)(uint32_t)ah[0] << 32) | (uint32_t)al[0];
    const unsigned long long a1 = ((unsigned long long)(uint32_t)ah[1] << 32) | (uint32_t)al[1];
    x = a0 > a1 ? a0 : a1;
    const auto bh = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
    const auto bl = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    const unsigned long long b0 = ((unsigned long long)(uint32_t)bh[0] << 32) | (uint32_t)bl[0];
    const unsigned long long b1 = ((unsigned long long)(uint32_t)bh[1] << 32) | (uint32_t)bl[1];
    return b0 > b1 ? b0 : b1;
}
// The maximum and the sum over lane columns n, n + 4, n + 8, n + 12 of each
// 16-lane row (DPP row rotations by 4 and 8).
__device__ __forceinline__ uint32_t fold4_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xF, 0xF, false));  // row_ror:4
    return max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false));  // row_ror:8
}
template <int CTL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
    const uint32_t h = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTL, 0xF, 0xF, false);
    const uint32_t l = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTL, 0xF, 0xF, false);
    return ((unsigned long long)h << 32) | l;
}
__device__ __forceinline__ unsigned long long fold4_max_u64(unsigned long long x) {
    unsigned long long y = dpp_u64<0x124>(x);  // row_ror:4
    x = x > y ? x : y;
    y = dpp_u64<0x128>(x);                     // row_ror:8
    return x > y ? x : y;
}
__device__ __forceinline__ float fold4_sum_f32(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}

// SR = 1: single rounding (logit = bf16(base + fp32 dot)), DSW_FLAG_SINGLE_ROUND.
// FD = 4 (bf16, up to 4 requests): only columns 0..3 of a tile's result hold
// requests, so four tiles share one epilogue: tile j0 + q's column b moves to
// lane column 4q + b (DPP row shifts), and each lane works on its own tile and
// request.
// GU = 1: sampled requests draw by Gumbel-max (DSW_FLAG_GUMBEL): the epilogue
// adds each row's noise to l / T and keeps the best score, the owner of a
// request reduces the shards' {score, ~id} and publishes the token itself, so
// every step takes two exchanges and no token shard scans its rows.
template <int A, int M, int DT, int SR, int FD = 1, int GU = 0>
__global__ void __launch_bounds__(kBlock, 1) walk_batched(WalkParams p) {
    static_assert(FD == 1 || (FD == 4 && DT == 0), "fold: bf16");
    static_assert(GU == 0 || (DT == 0 && SR == 0), "Gumbel-max: bf16, double rounding");
    constexpr bool kI8 = DT == 1;
    using WT = typename std::conditional<kI8, uint2, uint4>::type;
    // register tiles in bf16 (int8 rows widened once at entry): up to
    // kMaxRegTiles in AGPRs and two more in VGPRs
    static_assert(A <= M && A <= kMaxRegTiles + 2 && (A % 2) == 0, "shape");
    constexpr int kA4 = (A + 3) / 4 * 4;  // FD = 4: the first tile after the register groups
    constexpr int RPAD = M * 4 * kTileRows;  // shard rows, bound
    extern __shared__ uint4 s_dyn[];  // [LDS weight tiles][ring slots]

    __shared__ uint32_t s_rkey[4][kMaxBatch];  // per wave and request: local key
    // per wave and request: max logit and exp-sum relative to it (sampled
    // requests, inverse CDF), or (Gumbel-max) the best {ord32(score), ~id}
    __shared__ float s_rm[GU ? 1 : 4][GU ? 1 : kMaxBatch];
    __shared__ float s_rs[GU ? 1 : 4][GU ? 1 : kMaxBatch];
    __shared__ unsigned long long s_gk[GU ? 4 : 1][GU ? kMaxBatch : 1];
    __shared__ int s_prev[kMaxBatch];
    __shared__ unsigned long long s_rowb[kMaxBatch];  // request b's base logits of step 0 at this shard, in 16 B
    __shared__ int s_next[kMaxBatch];
    __shared__ float s_T[kMaxBatch];
    __shared__ float s_scl[kMaxBatch];             // log2(e) / T of sampled requests, else 0
    __shared__ float s_invT[GU ? kMaxBatch : 1];   // Gumbel-max: 1 / T of sampled requests
    __shared__ float s_S[kMaxGrid];
    __shared__ float s_E[kMaxGrid];
    __shared__ float s_M[kMaxGrid];            // owner: the shards' max logits of the request
    __shared__ float s_wsum[4];                // owner: per-wave mass totals of the token search
    __shared__ uint32_t s_wfirst[4], s_wlast[4];
    __shared__ float s_scale[kI8 ? RPAD : 1];
    __shared__ uint2 s_junk[4][64];            // base logits (-inf) of tiles beyond a wave's rows
    __shared__ unsigned long long s_red64[4];
    __shared__ int s_own;
    __shared__ float s_qown;
    __shared__ unsigned s_round;
    __shared__ unsigned s_fam;
    __shared__ int s_abort;
    DSW_TRACE_DECL;
    __shared__ int s_any_samp;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // provably wave-uniform
    const int g = lane >> 4;  // rows 4g .. 4g+3 of a tile
    const int n = lane & 15;  // request column within a group (MFMA B operand)
    // the lane's request within its group and its tile offset in the epilogue
    const int nreq = FD == 4 ? (n & 3) : n;
    const int qf = FD == 4 ? (n >> 2) : 0;
    const int c = blockIdx.x;
    const int G = gridDim.x;
    const int V = p.V;
    const int B = p.B;
    const int gamma = p.gamma;
    const int R = p.rows_per_wg;  // multiple of 16
    const int Rpad = p.rows_pad;  // multiple of 128
    const int CPR = Rpad >> 3;    // 16-byte chunks per request row of a base slot
    const int v0 = c * R;
    const int nrows = max(0, min(V, v0 + R) - v0);
    // register slots beyond the shard load its last row (a cache hit), never
    // another shard's rows (extra HBM reads); an empty shard loads row V - 1
    const int last_row = nrows > 0 ? v0 + nrows - 1 : V - 1;
    const int TW = p.tiles_per_wave;
    const int LT = p.lds_tiles;
    const int wrow0 = wave * TW * kTileRows;
    const int nt_w = max(0, min(TW, (nrows - wrow0 + kTileRows - 1) / kTileRows));
    const int NG = (B + kGroup - 1) / kGroup;
    // Owner words: request b's decision word at b / G in owner b % G's region
    // of OS words, whole lines with one writer each (253 requests: 335 -> 329
    // us, 64: 136 -> 131 us against one line shared by 16 owners; 16 requests:
    // 224 -> 216 us against their 16 words in one line).
    const int OS = owner_stride(G);
    const int D = p.ring;
    const bool aligned = p.aligned != 0;
    const bool al4 = (V & 3) == 0;  // 8-byte stores of 4 logits (rows 4g .. 4g+3)
    const int P = 2 + (aligned ? CPR / 16 : 0);  // DMA instructions per wave and group
    // x / CPR as (x * cpr_mul) >> 20, exact for x < 16 * CPR (CPR <= 128: rows_pad <= 1024)
    const unsigned cpr_mul = ((1u << 20) + (unsigned)CPR - 1u) / (unsigned)CPR;
    const WT* __restrict__ W2 = reinterpret_cast<const WT*>(p.W2);
    const uint4* __restrict__ W1 = reinterpret_cast<const uint4*>(p.W1);
    const uint16_t* __restrict__ base = p.base;
    unsigned* status = p.ws.status;
    WT* s_wt = reinterpret_cast<WT*>(s_dyn);
    char* ring = reinterpret_cast<char*>(s_dyn) + 4 * LT * 512 * (int)sizeof(WT);
    const int slot_bytes = kSlotUBytes + kGroup * Rpad * 2;

    // The control block (round counter, family counters, status word) and this
    // thread's anchor and temperature are requested first and used only after
    // the shard's loads have been issued, so that their round trip overlaps the
    // shard load.  A plain load: the previous launch's updates are visible at
    // a kernel boundary.
    uint4 ctl = make_uint4(0u, 0u, 0u, 0u);
    if (t == 0) ctl = *reinterpret_cast<const uint4*>(p.ws.round_ctr);
    int a_in = 0;
    float t_in = 0.0f;
    if (t < B) {
        a_in = p.anchor[t];
        t_in = p.T[t];
    }
    if (t == 0) s_any_samp = 0;
    s_junk[t >> 6][t & 63] = make_uint2(0xFF80FF80u, 0xFF80FF80u);  // -inf base logits
    // every word this workgroup posts in this launch, both parities, starts at
    // 0 (the barriers before the first post order these stores first): its row
    // of keys and exp-sums, and the decision words of the requests it owns
    for (int i = t; i < 2 * p.B_max; i += kBlock) {
        const size_t o = ((size_t)(i / p.B_max) * kMaxGrid + c) * kMaxBatch + i % p.B_max;
        st_agent64(p.ws.bkey + 2 * o, 0ull);
        st_agent64(p.ws.bkey + 2 * o + 1, 0ull);
    }
    for (int i = t; i < 2 * OS; i += kBlock)
        st_agent64(p.ws.bdec + (size_t)(i / OS) * kOwnWords + (size_t)c * OS + i % OS, 0ull);
    __syncthreads();  // s_any_samp and s_junk set (LDS only: no wait for the loads above)
    DSW_TRACE(gamma, 0);

    // ---- entry: this workgroup's shard on chip (as walk_kernel.h) --------
    // Register tiles hold bf16 operands: int8 rows are widened once here
    // (exactly: every int8 value is a bf16 value), not before every MFMA.
    uint4 wr[A > 0 ? A : 1][8];
    {
        WT raw[A > 0 ? A : 1][8];
#pragma unroll
        for (int j = 0; j < A; ++j) {
            const int row = min(v0 + wrow0 + j * kTileRows + n, last_row);
            const WT* src = W2 + (size_t)row * kRowChunks + g;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) raw[j][kb] = src[kb * 4];
        }
#pragma unroll
        for (int j = 0; j < A; ++j)
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) wr[j][kb] = as_bf16x8(raw[j][kb]);
    }
    // pinned once every tile's loads are in flight (a pin waits for its registers)
#pragma unroll
    for (int j = 0; j < A; ++j)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            if (j < kMaxRegTiles) pin_agpr(wr[j][kb]);
    for (int i0 = 0; i0 < 4 * LT * 512; i0 += 8 * kBlock) {
        WT v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int idx = i0 + q * kBlock + t;
            const int s = idx >> 9, kb = (idx >> 6) & 7, ln = idx & 63;
            const int ws = s / max(LT, 1);
            const int j = A + (s - ws * LT);
            const int r = ws * TW * kTileRows + j * kTileRows + (ln & 15);
            v[q] = WT{};
            if (idx < 4 * LT * 512 && j < TW && r < nrows)
                v[q] = W2[(size_t)(v0 + r) * kRowChunks + kb * 4 + (ln >> 4)];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int idx = i0 + q * kBlock + t;
            if (idx < 4 * LT * 512) s_wt[idx] = v[q];
        }
    }
    if constexpr (kI8)
        for (int r = t; r < RPAD; r += kBlock) s_scale[r] = r < nrows ? p.w2_scale[v0 + r] : 0.0f;
    if (t == 0) {
        s_round = ctl.x;
        s_fam = ctl.z;  // the batched family's counter
        // a device error latched by an earlier launch stands until dsw_status
        // clears the workspace: this launch then does nothing
        s_abort = ctl.w != 0u;
    }
    if (t < B) {
        int a = a_in;
        float temp = t_in;
        if (a < 0 || a >= V) {
            if (c == 0) latch(status, kStatusToken);
            a = 0;
        }
        if (temp > 0.0f && p.uniforms == nullptr && !p.seeded) {
            if (c == 0) latch(status, kStatusUniforms);
            temp = 0.0f;
        }
        if (!(temp > 0.0f)) temp = 0.0f;
        s_prev[t] = a;
        s_T[t] = temp;
        s_scl[t] = temp > 0.0f ? kLog2e / temp : 0.0f;
        if constexpr (GU) s_invT[t] = temp > 0.0f ? 1.0f / temp : 1.0f;
        if (temp > 0.0f) s_any_samp = 1;
        s_rowb[t] = (unsigned long long)t * (unsigned)gamma * (unsigned)(V >> 3) + (unsigned)(v0 >> 3);
    }
    __syncthreads();
    if (s_abort) return;  // uniform: read after the barrier
    const unsigned round = s_round;
    const unsigned fam = s_fam;
    const bool any_samp = s_any_samp != 0;

    // acc_ += tile j >= A (in LDS, else streamed from W2) times ub
#define DSW_TILE_OFFCHIP(j_, acc_)                                                               \
    do {                                                                                         \
        if ((j_) - A < LT) {                                                                     \
            const int sb_ = (wave * LT + ((j_) - A)) * 512 + lane;                               \
            _Pragma("unroll") for (int kb = 0; kb < 8; ++kb)                                     \
                acc_ = mfma_tile(as_bf16x8(s_wt[sb_ + kb * 64]), ub[kb], acc_);                  \
        } else {                                                                                 \
            const int row_ = min(v0 + wrow0 + (j_) * kTileRows + n, last_row);                   \
            const WT* src_ = W2 + (size_t)row_ * kRowChunks + g;                                 \
            _Pragma("unroll") for (int kb = 0; kb < 8; ++kb)                                     \
                acc_ = mfma_tile(as_bf16x8(src_[kb * 4]), ub[kb], acc_);                         \
        }                                                                                        \
    } while (0)

    // MFMA over every tile of this wave with B operand ub[8]; EPI(d, j) gets
    // the four results (rows 4g .. 4g+3 of tile j, request column n)
#define DSW_TILES(EPI)                                                                           \
    do {                                                                                         \
        {                                                                                        \
            /* the MFMAs of a pair of tiles are issued before the epilogue of the    */          \
            /* previous pair, whose VALU work then overlaps them;                    */          \
            /* their base logits are read from LDS with the MFMAs, a pair ahead     */          \
            f32x4_t p0_ = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, p1_ = p0_;                            \
            uint2 pb0_ = make_uint2(0u, 0u), pb1_ = pb0_;                                        \
            _Pragma("unroll") for (int j0 = 0; j0 < A; j0 += 2) {                                \
                const uint2 nb0_ = *DSW_BASE_PTR(j0), nb1_ = *DSW_BASE_PTR(j0 + 1);              \
                f32x4_t c0_ = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, c1_ = c0_;                        \
                _Pragma("unroll") for (int kb = 0; kb < 8; ++kb) {                               \
                    c0_ = mfma_tile(as_bf16x8(wr[j0][kb]), ub[kb], c0_);                         \
                    c1_ = mfma_tile(as_bf16x8(wr[j0 + 1][kb]), ub[kb], c1_);                     \
                }                                                                                \
                if (j0 > 0) {                                                                    \
                    EPI(p0_, j0 - 2, pb0_);                                                      \
                    EPI(p1_, j0 - 1, pb1_);                                                      \
                }                                                                                \
                p0_ = c0_;                                                                       \
                p1_ = c1_;                                                                       \
                pb0_ = nb0_;                                                                     \
                pb1_ = nb1_;                                                                     \
            }                                                                                    \
            if (A > 0) {                                                                         \
                EPI(p0_, A - 2, pb0_);                                                           \
                EPI(p1_, A - 1, pb1_);                                                           \
            }                                                                                    \
        }                                                                                        \
        _Pragma("unroll 1") for (int j = A; j < nt_w; ++j) {                                     \
            f32x4_t dd = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};                                        \
            if (j - A < LT) {                                                                    \
                const int sb_ = (wave * LT + (j - A)) * 512 + lane;                              \
                _Pragma("unroll") for (int kb = 0; kb < 8; ++kb)                                 \
                    dd = mfma_tile(as_bf16x8(s_wt[sb_ + kb * 64]), ub[kb], dd);                   \
            } else {                                                                             \
                const int row_ = min(v0 + wrow0 + j * kTileRows + n, last_row);                  \
                const WT* src_ = W2 + (size_t)row_ * kRowChunks + g;                             \
                _Pragma("unroll") for (int kb = 0; kb < 8; ++kb)                                 \
                    dd = mfma_tile(as_bf16x8(src_[kb * 4]), ub[kb], dd);                          \
            }                                                                                    \
            EPI(dd, j, *DSW_BASE_PTR(j));                                                        \
        }                                                                                        \
    } while (0)

    // FD = 4: four tiles per epilogue (the lane's tile is j0 + qf); the MFMAs
    // of four register tiles are issued before the epilogue of the previous
    // four.  A last group of four that holds fewer than four register tiles
    // (A % 4 == 2) takes its other tiles from LDS or W2.
#define DSW_TILES_F4(EPI)                                                                        \
    do {                                                                                         \
        f32x4_t e_ = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};                                            \
        uint2 eb_ = make_uint2(0u, 0u);                                                          \
        _Pragma("unroll") for (int j0 = 0; j0 < A; j0 += 4) {                                    \
            const uint2 nb_ = *DSW_BASE_PTR(j0 + qf);                                            \
            f32x4_t c_[4];                                                                       \
            _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) {                                   \
                c_[jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};                                        \
                if (j0 + jj < A) {                                                               \
                    _Pragma("unroll") for (int kb = 0; kb < 8; ++kb)                             \
                        c_[jj] = mfma_tile(as_bf16x8(wr[min(j0 + jj, A - 1)][kb]), ub[kb], c_[jj]); \
                } else if (j0 + jj < nt_w) {                                                     \
                    DSW_TILE_OFFCHIP(j0 + jj, c_[jj]);                                           \
                }                                                                                \
            }                                                                                    \
            if (j0 > 0) EPI(e_, j0 - 4 + qf, eb_);                                               \
            e_ = fold4(c_[0], c_[1], c_[2], c_[3]);                                              \
            eb_ = nb_;                                                                           \
        }                                                                                        \
        if (A > 0) EPI(e_, kA4 - 4 + qf, eb_);                                                   \
        _Pragma("unroll 1") for (int j0 = kA4; j0 < nt_w; j0 += 4) {                             \
            f32x4_t c_[4];                                                                       \
            _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) {                                   \
                const int j = j0 + jj;                                                           \
                c_[jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};                                        \
                if (j < nt_w) DSW_TILE_OFFCHIP(j, c_[jj]);                                       \
            }                                                                                    \
            EPI(fold4(c_[0], c_[1], c_[2], c_[3]), j0 + qf, *DSW_BASE_PTR(j0 + qf));             \
        }                                                                                        \
    } while (0)

    // ---- the walk --------------------------------------------------------
    for (int k = 0; k < gamma; ++k) {
        DSW_TRACE(k, kTrStepStart);
        const unsigned seq = fam * (unsigned)p.gamma_max + (unsigned)k;
        const unsigned long long epoch = epoch_of(seq);
        const int q = (int)(seq & 1u);
        // workgroup c's words for request b: bkey[2 (c kMaxBatch + b)] (key), + 1 (exp-sum or ~id)
        unsigned long long* bkey = p.ws.bkey + (size_t)q * kMaxGrid * kMaxBatch * 2;
        unsigned long long* bown = p.ws.bdec + (size_t)q * kOwnWords;
#define DSW_OWN(b_) (bown + (size_t)((b_) % G) * OS + (b_) / G)

        // group gq's u rows (U_) and base logits (BASE_, of the step whose rows
        // start koff_ 16-byte chunks into a request's base) into ring slot
        // gq % D.  Each lane names its own source; the wave's 64 chunks land
        // contiguously.
#define DSW_ISSUE_GROUP(grp_, U_, BASE_, koff_)                                                  \
    do {                                                                                         \
        const int gq_ = (grp_);                                                                  \
        char* slot_ = ring + (gq_ % D) * slot_bytes;                                             \
        if (U_) _Pragma("unroll") for (int ii = 0; ii < 2; ++ii) {                               \
            const int inst_ = wave * 2 + ii;                                                     \
            const int pos_ = inst_ * 64 + lane;                                                  \
            const int nn_ = pos_ >> 5, pc_ = pos_ & 31;                                          \
            const int b_ = min(gq_ * kGroup + nn_, B - 1);                                       \
            dma16(W1 + (size_t)s_prev[b_] * kRowChunks + (pc_ ^ nn_),                            \
                  __builtin_amdgcn_readfirstlane(lds_addr(slot_ + inst_ * 1024)));               \
        }                                                                                        \
        if (!(BASE_)) {                                                                          \
        } else if (aligned) {                                                                    \
            /* 16-byte chunk (pc ^ nn) of request nn's row past the shard start, */             \
            /* clamped to the row's last chunk; 24-bit products (pos < 16 CPR)   */             \
            const int per_ = CPR / 16;                                                           \
            for (int ii = 0; ii < per_; ++ii) {                                                  \
                const int inst_ = wave * per_ + ii;                                              \
                const int pos_ = inst_ * 64 + lane;                                              \
                const int nn_ = (int)((unsigned)__umul24((unsigned)pos_, cpr_mul) >> 20);        \
                const int pc_ = pos_ - __umul24((unsigned)nn_, (unsigned)CPR);                   \
                const int b_ = min(gq_ * kGroup + nn_, B - 1);                                   \
                const int x_ = min(pc_ ^ nn_, lastc);                                            \
                const uint4* src_ = reinterpret_cast<const uint4*>(base) + (s_rowb[b_] + (koff_)) + x_; \
                dma16(src_, __builtin_amdgcn_readfirstlane(lds_addr(slot_ + kSlotUBytes + inst_ * 1024))); \
            }                                                                                    \
        } else {                                                                                 \
            uint16_t* sb_ = reinterpret_cast<uint16_t*>(slot_ + kSlotUBytes);                    \
            for (int e_ = t; e_ < kGroup * Rpad; e_ += kBlock) {                                 \
                const int nn_ = e_ / Rpad, r_ = e_ - nn_ * Rpad;  /* fallback path only */      \
                const int b_ = min(gq_ * kGroup + nn_, B - 1);                                   \
                sb_[(nn_ * CPR + ((r_ >> 3) ^ nn_)) * 8 + (r_ & 7)] =                            \
                    r_ < nrows ? base[((size_t)b_ * gamma + k) * V + v0 + r_] : (uint16_t)0;     \
            }                                                                                    \
        }                                                                                        \
    } while (0)

        const unsigned long long koff = (unsigned long long)k * (unsigned)(V >> 3);  // step k's rows, in 16 B
        const int lastc = (V >> 3) - 1 - (v0 >> 3);  // the row's last chunk past the shard start (< 0: empty shard)
        // one group (up to 16 requests, DMA-able base rows): its base logits of
        // steps after the first were fetched during the previous step's
        // exchange (below)
        const bool pref = NG == 1 && aligned;
        for (int gq = 0; gq < min(D - 1, NG); ++gq) DSW_ISSUE_GROUP(gq, true, !(pref && k > 0), koff);

        for (int grp = 0; grp < NG; ++grp) {
            wait_vmcnt(P * min(D - 2, NG - 1 - grp));
            barrier_keep_vm();
            if (grp + D - 1 < NG) DSW_ISSUE_GROUP(grp + D - 1, true, true, koff);
            const char* slot = ring + (grp % D) * slot_bytes;
            const uint4* su = reinterpret_cast<const uint4*>(slot);
            uint16_t* sb = reinterpret_cast<uint16_t*>(const_cast<char*>(slot) + kSlotUBytes);
            const int b = grp * kGroup + nreq;
            const bool bval = b < B;
            uint4 ub[8];
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) ub[kb] = su[n * kRowChunks + ((kb * 4 + g) ^ n)];
            // The partial tile of the vocabulary's last shard: base rows past the
            // vocabulary read -inf, so that their logits lose every max and add
            // nothing to an exp-sum.  Only the wave whose tiles hold them fills
            // them, after the group's DMA has landed and before it reads them.
            if (nt_w > 0 && nrows < wrow0 + nt_w * kTileRows) {
                const int nfill = wrow0 + nt_w * kTileRows - nrows;  // 1 .. 15 rows
                for (int e = lane; e < kGroup * nfill; e += 64) {
                    const int nn = e & (kGroup - 1), r = nrows + (e >> 4);
                    sb[(nn * CPR + ((r >> 3) ^ nn)) * 8 + (r & 7)] = (uint16_t)0xFF80u;
                }
            }
            // Lane's best (first) logit of request n: the tile whose four logits
            // hold the largest value first (tiles in row order, a strictly larger
            // maximum replaces it), that tile's logits, and after the tiles the
            // first of its four rows with that value.
            float bestv = -__builtin_inff();
            int bestj = -1;
            uint32_t bq01 = 0u, bq23 = 0u;
            // Gumbel-max: the lane's best score and its row (-1: none finite)
            float bestS = -__builtin_inff();
            int bestR = -1;
// Base logits of tile j for this lane's request: the slot, or s_junk (-inf)
// for a tile beyond this wave's rows.
#define DSW_BASE_PTR(j)                                                                          \
    (((j) < nt_w) ? reinterpret_cast<uint2*>(sb + (nreq * CPR + (((wrow0 + (j) * kTileRows + 4 * g) >> 3) ^ nreq)) * 8 + \
                                             ((wrow0 + (j) * kTileRows + 4 * g) & 7))            \
                  : &s_junk[wave][lane])
// Branch-free, so that the matrix cores' work and this VALU work can be
// interleaved; a tile beyond this wave's rows has -inf base logits and its
// logits lose every max.  bw: the tile's four base logits.  STORE (a
// constant): the logits go out -- when the caller wants them, back into the
// slot over the base logits (a tile beyond the wave's rows rewrites s_junk's
// -inf), copied out row-contiguously after the tiles; otherwise, in a group
// with a sampled request, to the group's private block `lblog` with
// agent-scope stores (the wave's 64 lanes write 512 contiguous bytes); the
// owners of sampled requests read them from either -- and the lane's running
// exp-sum of them, relative to its running maximum, is updated (sampled
// lanes: sc > 0; it is rescaled when the maximum grows).
#define DSW_EPI(dv, j, bw, STORE, NOISE)                                                         \
    do {                                                                                         \
        const int rb_ = wrow0 + (j) * kTileRows + 4 * g;                                         \
        const bool live_ = (j) < nt_w;                                                           \
        const uint2 bw_ = (bw);                                                                  \
        float x0_ = (dv)[0], x1_ = (dv)[1], x2_ = (dv)[2], x3_ = (dv)[3];                        \
        if constexpr (kI8) {                                                                     \
            const int rs_ = live_ ? rb_ : 0;                                                     \
            x0_ *= s_scale[rs_];                                                                 \
            x1_ *= s_scale[rs_ + 1];                                                             \
            x2_ *= s_scale[rs_ + 2];                                                             \
            x3_ *= s_scale[rs_ + 3];                                                             \
        }                                                                                        \
        if constexpr (!SR) {  /* double rounding: the bias to bf16 first */                    \
            const uint32_t p01_ = pack_bf16_rne(x0_, x1_), p23_ = pack_bf16_rne(x2_, x3_);       \
            x0_ = bf16_lo(p01_);                                                                 \
            x1_ = bf16_hi(p01_);                                                                 \
            x2_ = bf16_lo(p23_);                                                                 \
            x3_ = bf16_hi(p23_);                                                                 \
        }                                                                                        \
        const uint32_t q01_ = pack_bf16_rne(bf16_lo(bw_.x) + x0_, bf16_hi(bw_.x) + x1_);         \
        const uint32_t q23_ = pack_bf16_rne(bf16_lo(bw_.y) + x2_, bf16_hi(bw_.y) + x3_);         \
        const float tm_ = fmaxf(fmaxf(bf16_lo(q01_), bf16_hi(q01_)), fmaxf(bf16_lo(q23_), bf16_hi(q23_))); \
        if (STORE) {                                                                             \
            if (priv) {  /* wave-uniform */                                                      \
                if (tolog && live_)  /* for the owners' token search */                         \
                    st_agent64(&lblog[(j) * 64], ((unsigned long long)q23_ << 32) | q01_);       \
            } else {                                                                             \
                *DSW_BASE_PTR(j) = make_uint2(q01_, q23_);  /* for the caller's copy */          \
            }                                                                                    \
            if constexpr (!GU) {                                                                 \
            /* finite, since mrun starts at -FLT_MAX: no -inf - -inf */                         \
            const float mn_ = fmaxf(mrun, tm_);                                                  \
            srun = srun * __builtin_amdgcn_exp2f((mrun - mn_) * sc) +                            \
                   ((__builtin_amdgcn_exp2f((bf16_lo(q01_) - mn_) * sc) +                         \
                     __builtin_amdgcn_exp2f((bf16_hi(q01_) - mn_) * sc)) +                        \
                    (__builtin_amdgcn_exp2f((bf16_lo(q23_) - mn_) * sc) +                         \
                     __builtin_amdgcn_exp2f((bf16_hi(q23_) - mn_) * sc)));                        \
            mrun = mn_;                                                                          \
        }                                                                                        \
        }                                                                                        \
        if constexpr (GU) {                                                                      \
            /* score l / T + G of the tile's four rows (sampled lanes; l itself */             \
            /* otherwise), the first best kept; NOISE: some lane samples      */                 \
            float s_[4] = {bf16_lo(q01_), bf16_hi(q01_), bf16_lo(q23_), bf16_hi(q23_)};          \
            if (NOISE) {                                                                         \
                uint32_t w_[4] = {(uint32_t)(v0 + rb_) >> 2, gc1, round, 0x47554D42u};          \
                philox4(w_, (uint32_t)p.seed, (uint32_t)(p.seed >> 32));                         \
                _Pragma("unroll") for (int e_ = 0; e_ < 4; ++e_)                                 \
                    s_[e_] = samp ? s_[e_] * invT + gumbel_of_word(w_[e_]) : s_[e_];             \
            }                                                                                    \
            _Pragma("unroll") for (int e_ = 0; e_ < 4; ++e_) {                                   \
                const bool gt_ = s_[e_] > bestS;                                                 \
                bestS = gt_ ? s_[e_] : bestS;                                                    \
                bestR = gt_ ? rb_ + e_ : bestR;                                                  \
            }                                                                                    \
        } else {                                                                                 \
            const bool gt_ = tm_ > bestv;                                                        \
            bestv = gt_ ? tm_ : bestv;                                                           \
            bestj = gt_ ? (j) : bestj;                                                           \
            bq01 = gt_ ? q01_ : bq01;                                                            \
            bq23 = gt_ ? q23_ : bq23;                                                            \
        }                                                                                        \
    } while (0)
#define DSW_EPI_G(dv, j, bw) DSW_EPI(dv, j, bw, 0, 0)
#define DSW_EPI_GS(dv, j, bw) DSW_EPI(dv, j, bw, 1, 0)
#define DSW_EPI_N(dv, j, bw) DSW_EPI(dv, j, bw, 0, 1)
#define DSW_EPI_NS(dv, j, bw) DSW_EPI(dv, j, bw, 1, 1)
            // Logits go out straight from the epilogue: to `logits` when asked
            // for (with agent-scope stores in a group with a sampled request),
            // else for such groups to the workspace's private blocks, where the
            // owners read them back.  A group with
            // nothing to store runs the epilogue without the stores and
            // without exp-sums (their branches cost a greedy batch ~12% even
            // when no lane stores).
            // Gumbel-max: the logits go out only when the caller wants them, and
            // the noise is drawn only in groups with a sampled request.
            const bool samp = bval && s_T[b] > 0.0f;
            const float sc = bval ? s_scl[b] : 0.0f;
            const float invT = GU && bval ? s_invT[GU ? b : 0] : 1.0f;  // Gumbel-max: l / T
            const uint32_t gc1 = ((uint32_t)k << 8) | (uint32_t)b;    // Gumbel-max: the noise counter
            const bool priv = p.logits == nullptr;  // no caller logits (wave-uniform)
            // this lane's column of the group's private block: tile j at 64 j
            unsigned long long* lblog = reinterpret_cast<unsigned long long*>(p.ws.blog) +
                                        (((size_t)c * NG + grp) * 4 + wave) * TW * 64 + g * 16 + nreq;
            float mrun = -__FLT_MAX__, srun = 0.0f;  // the lane's running maximum and exp-sum
            const bool anys = __builtin_amdgcn_ballot_w64(samp) != 0ull;
            const bool tolog = !GU && anys;  // owners read these logits (wave-uniform)
            const bool stored = !priv || tolog;
            if constexpr (GU) {
                if (FD == 4) {
                    if (stored) {
                        if (anys) DSW_TILES_F4(DSW_EPI_NS); else DSW_TILES_F4(DSW_EPI_GS);
                    } else {
                        if (anys) DSW_TILES_F4(DSW_EPI_N); else DSW_TILES_F4(DSW_EPI_G);
                    }
                } else {
                    if (stored) {
                        if (anys) DSW_TILES(DSW_EPI_NS); else DSW_TILES(DSW_EPI_GS);
                    } else {
                        if (anys) DSW_TILES(DSW_EPI_N); else DSW_TILES(DSW_EPI_G);
                    }
                }
            } else if constexpr (FD == 4) {
                if (stored) {
                    DSW_TILES_F4(DSW_EPI_GS);
                } else {
                    DSW_TILES_F4(DSW_EPI_G);
                }
            } else {
                if (stored) {
                    DSW_TILES(DSW_EPI_GS);
                } else {
                    DSW_TILES(DSW_EPI_G);
                }
            }
#undef DSW_EPI_G
#undef DSW_EPI_GS
#undef DSW_EPI_N
#undef DSW_EPI_NS
#undef DSW_EPI
#undef DSW_BASE_PTR
            if constexpr (GU) {
                // {ord32(score), ~id} of the lane's best row, reduced over the
                // request's lanes
                unsigned long long gk = bestR >= 0 ? (((unsigned long long)ord32(bestS) << kIdxBits) |
                                                      (unsigned long long)(kIdxMask - (uint32_t)(v0 + bestR)))
                                                   : 0ull;
                gk = column4_max_u64(gk);
                if constexpr (FD == 4) gk = fold4_max_u64(gk);
                if (g == 0 && qf == 0 && bval) s_gk[wave][b] = gk;
            }
            // the first of the best tile's four rows with the best value
            uint32_t best = 0u;
            if constexpr (!GU) {
                const int bi = bf16_lo(bq01) == bestv ? 0 : (bf16_hi(bq01) == bestv ? 1 : (bf16_lo(bq23) == bestv ? 2 : 3));
                const int bestr = bestj >= 0 ? wrow0 + bestj * kTileRows + 4 * g + bi : -1;
                best = bestr >= 0 ? local_key(__float_as_uint(bestv) >> 16, bestr) : 0u;
                // the four lanes of request column n: rows 4g .. 4g+3 for g = 0..3
                // (and, folded, the four tiles of each epilogue)
                best = column4_max_u32(best);
                if constexpr (FD == 4) best = fold4_max_u32(best);
                if (g == 0 && qf == 0 && bval) s_rkey[wave][b] = best;
            }
            if (!priv) {
                // the caller's logits of the group's requests over this wave's
                // rows, from the slot: four consecutive rows per lane, so that
                // the wave's stores to one request's row are contiguous; with
                // agent-scope stores when an owner reads them
                const int rend = min(wrow0 + nt_w * kTileRows, nrows);
                for (int nn = 0; nn < kGroup && grp * kGroup + nn < B; ++nn) {
                    uint16_t* dst = p.logits + ((size_t)(grp * kGroup + nn) * gamma + k) * V + v0;
                    for (int r0 = wrow0 + 4 * lane; r0 < rend; r0 += 256) {
                        const uint2 v = *reinterpret_cast<const uint2*>(sb + (nn * CPR + ((r0 >> 3) ^ nn)) * 8 + (r0 & 7));
                        if (al4 && r0 + 4 <= rend) {
                            if (tolog)
                                st_agent64(reinterpret_cast<unsigned long long*>(dst + r0),
                                           ((unsigned long long)v.y << 32) | v.x);
                            else
                                *reinterpret_cast<uint2*>(dst + r0) = v;
                        } else {
                            const uint32_t l4[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                if (r0 + i < rend) {
                                    if (tolog)
                                        st_agent16(dst + r0 + i, (uint16_t)l4[i]);
                                    else
                                        dst[r0 + i] = (uint16_t)l4[i];
                                }
                            }
                        }
                    }
                }
            }
            const float Tb = bval ? s_T[b] : 0.0f;
            const bool on = !GU && Tb > 0.0f && best != 0u;
            if (!GU && stored && __builtin_amdgcn_ballot_w64(on) != 0ull) {
                // exp-sum of this wave's logits of request n relative to its
                // maximum: the four lanes' running sums, rescaled to it (a lane
                // whose rows all lie past the vocabulary holds 0 at -FLT_MAX)
                const float mw = local_key_logit(best);
                float sw = on ? srun * __builtin_amdgcn_exp2f((mrun - mw) * sc) : 0.0f;
                sw = column4_sum_f32(sw);
                if constexpr (FD == 4) sw = fold4_sum_f32(sw);
                if constexpr (!GU) {
                    if (g == 0 && qf == 0 && bval) {
                        s_rm[wave][b] = mw;
                        s_rs[wave][b] = sw;
                    }
                }
            }
        }
        // the logits' agent-scope stores (private blocks or the caller's
        // logits) complete before any key word of this step is posted
        if (!GU && any_samp) wait_vmcnt(0);
        __syncthreads();
        DSW_TRACE(k, kTrGemvDone);

        // ---- post: one key word (and exp-sum word) per request -----------
        walk_skew(p, c, k, 0);
        if (t < B) {
            if constexpr (GU) {
                // Gumbel-max, every request: ord32(best score) in the key word,
                // ~id in the second
                const unsigned long long gk = max(max(s_gk[0][t], s_gk[1][t]), max(s_gk[2][t], s_gk[3][t]));
                st_agent64(&bkey[2 * ((size_t)c * kMaxBatch + t)], ((gk >> kIdxBits) << 28) | epoch);
                st_agent64(&bkey[2 * ((size_t)c * kMaxBatch + t) + 1], ((gk & kIdxMask) << 32) | epoch);
            } else {
                // every LDS read issued at once, the sum branch-free (a wave
                // without rows adds nothing)
                uint32_t kk[4];
                float rm[4], rs[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    kk[w] = s_rkey[w][t];
                    rm[w] = s_rm[w][t];
                    rs[w] = s_rs[w][t];
                }
                const float scl = s_scl[t];
                const bool smp = s_T[t] > 0.0f;
                const uint32_t lk = max(max(kk[0], kk[1]), max(kk[2], kk[3]));
                st_agent64(&bkey[2 * ((size_t)c * kMaxBatch + t)], (global_key(lk, v0) << 28) | epoch);
                if (smp) {
                    const float mc = local_key_logit(lk);
                    float sc = 0.0f;
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        sc += kk[w] != 0u ? rs[w] * __builtin_amdgcn_exp2f((rm[w] - mc) * scl) : 0.0f;
                    st_agent64(&bkey[2 * ((size_t)c * kMaxBatch + t) + 1],
                               ((unsigned long long)__float_as_uint(sc) << 32) | epoch);
                }
            }
        }
        DSW_TRACE(k, kTrPosted);
        // One group: the next step's base logits go into its slot now (every
        // wave is done with the slot), so that the next step waits only for
        // its u rows.  The polls below wait for these loads too (vmcnt counts
        // in order), but the exchange takes longer than they do.
        if (pref && k + 1 < gamma) DSW_ISSUE_GROUP(0, false, true, koff + (unsigned long long)(unsigned)(V >> 3));
        // ~0.2 us before the first poll of the columns: no other workgroup's
        // words can be there yet, and early polls only load the fabric
        // (measured: V = 129,280, gamma 5, B = 16: 231.5 -> 229.7 us)
        __builtin_amdgcn_s_sleep(8);

        // read column b of every workgroup's row: kw, sw of shard t (t < G); a
        // request with a second word takes both with one 16-byte load per poll
#define DSW_READ_COLUMN(b_, kw_, sw_)                                                            \
    do {                                                                                         \
        kw_ = 0ull;                                                                              \
        sw_ = 0.0f;                                                                              \
        if (t < G) {                                                                             \
            const bool samp_ = GU || s_T[b_] > 0.0f;  /* Gumbel-max: both words, always */       \
            const unsigned long long* pk_ = &bkey[2 * ((size_t)t * kMaxBatch + (b_))];           \
            unsigned it_ = 0;                                                                    \
            if (samp_) {                                                                         \
                for (;;) {                                                                       \
                    unsigned long long k_, s_;                                                   \
                    ld_agent64_pair(pk_, k_, s_);                                                \
                    if ((k_ & kEpochMod) == epoch && (s_ & kEpochMod) == epoch) {                \
                        kw_ = k_ >> 28;                                                          \
                        sw_ = __uint_as_float((uint32_t)(s_ >> 32));                             \
                        break;                                                                   \
                    }                                                                            \
                    if (++it_ >= p.spin_limit) { latch(status, kStatusTimeout); s_abort = 1; break; } \
                    if ((it_ & 255u) == 0u && ld_agent(status) != 0u) { s_abort = 1; break; }    \
                    __builtin_amdgcn_s_sleep(1);                                                 \
                }                                                                                \
            } else {                                                                             \
                for (;;) {                                                                       \
                    const unsigned long long w_ = ld_agent64(pk_);                               \
                    if ((w_ & kEpochMod) == epoch) {                                             \
                        kw_ = w_ >> 28;                                                          \
                        break;                                                                   \
                    }                                                                            \
                    if (++it_ >= p.spin_limit) { latch(status, kStatusTimeout); s_abort = 1; break; } \
                    if ((it_ & 255u) == 0u && ld_agent(status) != 0u) { s_abort = 1; break; }    \
                    __builtin_amdgcn_s_sleep(1);                                                 \
                }                                                                                \
            }                                                                                    \
        }                                                                                        \
    } while (0)

        // shard masses S_t of sampled request b_ into s_S (their scales
        // exp((m_t - M) / T) into s_E, their maxima m_t into s_M), then wave 0
        // finds the first shard with
        // positive mass whose prefix exceeds u*Z (else the last with positive
        // mass): s_own, and s_qown = (u*Z - mass before it) / its scale.
#define DSW_OWNER_SHARD(b_, kw_, sw_, M_)                                                        \
    do {                                                                                         \
        const float e_ = (t < G && kw_ != 0ull)                                                  \
                             ? __builtin_amdgcn_exp2f((key_logit(kw_) - (M_)) * s_scl[b_])          \
                             : 0.0f;                                                             \
        s_S[t] = (t < G && kw_ != 0ull) ? sw_ * e_ : 0.0f;                                       \
        s_E[t] = e_;                                                                             \
        s_M[t] = (t < G && kw_ != 0ull) ? key_logit(kw_) : 0.0f;                                 \
        __syncthreads();                                                                         \
        if (wave == 0) {                                                                         \
            const float4 m4_ = reinterpret_cast<const float4*>(s_S)[lane];                       \
            const float q0_ = m4_.x, q1_ = q0_ + m4_.y, q2_ = q1_ + m4_.z, q3_ = q2_ + m4_.w;    \
            const float incl_ = wave_incl_scan_dpp(q3_);                                         \
            const float ex_ = incl_ - q3_;                                                       \
            const float Z_ = __shfl(incl_, 63);                                                  \
            const float tgt_ = walk_uniform(p, (b_), k, gamma, round) * Z_;                      \
            const float c4_[4] = {ex_ + q0_, ex_ + q1_, ex_ + q2_, ex_ + q3_};                   \
            const float w4_[4] = {m4_.x, m4_.y, m4_.z, m4_.w};                                   \
            uint32_t first_ = 0u, lastp_ = 0u;                                                   \
            _Pragma("unroll") for (int i = 3; i >= 0; --i) {                                     \
                if (w4_[i] > 0.0f && c4_[i] > tgt_) first_ = (uint32_t)(4 * lane + i) + 1u;      \
                if (lastp_ == 0u && w4_[i] > 0.0f) lastp_ = (uint32_t)(4 * lane + i) + 1u;       \
            }                                                                                    \
            const uint32_t fmin_ = wave_max_u32(first_ ? 0xFFFFFFFFu - first_ : 0u);             \
            const uint32_t lmax_ = wave_max_u32(lastp_);                                         \
            const int own_ = fmin_ ? (int)(0xFFFFFFFFu - fmin_) - 1 : (int)lmax_ - 1;            \
            const int pj_ = max(own_ - 1, 0);                                                    \
            const float cj_ = (pj_ & 3) == 0 ? c4_[0] : ((pj_ & 3) == 1 ? c4_[1] : ((pj_ & 3) == 2 ? c4_[2] : c4_[3])); \
            const float pex_ = __shfl(cj_, pj_ >> 2);                                            \
            if (lane == 0) {                                                                     \
                s_own = own_;                                                                    \
                /* own_ >= 0: the winner's shard has mass >= 1 */                               \
                s_qown = (tgt_ - (own_ > 0 ? pex_ : 0.0f)) * __builtin_amdgcn_rcpf(s_E[max(own_, 0)]); \
            }                                                                                    \
        }                                                                                        \
        __syncthreads();                                                                         \
    } while (0)

        // workgroup max of kw_ into win_ (all threads)
#define DSW_BLOCK_MAX64(kw_, win_)                                                               \
    do {                                                                                         \
        const unsigned long long m_ = wave_max_u64_dpp(kw_);                                     \
        if (lane == 0) s_red64[wave] = m_;                                                       \
        __syncthreads();                                                                         \
        win_ = max(max(s_red64[0], s_red64[1]), max(s_red64[2], s_red64[3]));                    \
    } while (0)

        // ---- owners: the winner of every request this workgroup owns -------
        // (the decision words' epoch, formed here: a scalar pair less held
        // through the group loop)
        const unsigned long long dep = dec_epoch(fam * (unsigned)p.gamma_max + (unsigned)k);
        for (int b = c; b < B; b += G) {
            unsigned long long kw;
            float sw;
            DSW_READ_COLUMN(b, kw, sw);
            if constexpr (GU) {  // the shard's {ord32(score), ~id}
                kw = t < G ? ((kw << kIdxBits) | (unsigned long long)(__float_as_uint(sw) & kIdxMask)) : 0ull;
            }
            unsigned long long win;
            DSW_BLOCK_MAX64(kw, win);
            if (s_abort) break;
            if (GU || !(s_T[b] > 0.0f)) {
                if (t == 0) {
                    const int tok = checked_token(key_index(win), V, status);
                    walk_skew(p, c, k, 1);
                    st_agent64(DSW_OWN(b), ((unsigned long long)(unsigned)tok << 24) | dep);
                }
            } else {
                DSW_OWNER_SHARD(b, kw, sw, key_logit(win));
                // The token: shard s_own's logits of request b, read back from
                // the caller's logits or its private block (written before its
                // key word), scanned in
                // vocabulary order for the first cumulative mass, relative to
                // the shard's maximum, above s_qown -- rows 4t .. 4t+3 per
                // thread; no crossing row (rounding): the last row with mass.
                const int own = s_own;
                const int ov0 = max(own, 0) * R;
                const int onr = own < 0 ? 0 : max(0, min(V, ov0 + R) - ov0);
                const float sc2 = s_scl[b];
                const float mo = s_M[max(own, 0)];
                const float qo = s_qown;
                const int r0 = 4 * t;
                float w4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (r0 < onr) {
                    unsigned long long v;
                    if (p.logits != nullptr) {
                        // row ov0 + r0 of request b's step-k logits (8-byte
                        // aligned when 4 | V: ov0 and r0 are multiples of 4)
                        const uint16_t* src = p.logits + ((size_t)b * gamma + k) * V + ov0 + r0;
                        if (al4) {
                            v = ld_agent64(reinterpret_cast<const unsigned long long*>(src));
                        } else {
                            v = 0ull;
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (r0 + i < onr) v |= (unsigned long long)ld_agent16(src + i) << (16 * i);
                        }
                    } else {
                        // row r0 of the shard: wave r0 / (16 TW), tile rem / 16,
                        // lane 16 ((rem / 4) % 4) + b % 16 of that block, its
                        // four logits
                        const int wv = r0 / (TW * kTileRows), rem = r0 - wv * TW * kTileRows;
                        v = ld_agent64(reinterpret_cast<const unsigned long long*>(p.ws.blog) +
                                       ((((size_t)own * NG + (b >> 4)) * 4 + wv) * TW + (rem >> 4)) * 64 +
                                       ((rem >> 2) & 3) * 16 + (b & 15));
                    }
                    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
                    const float l4[4] = {bf16_lo(lo), bf16_hi(lo), bf16_lo(hi), bf16_hi(hi)};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        w4[i] = r0 + i < onr ? __builtin_amdgcn_exp2f((l4[i] - mo) * sc2) : 0.0f;
                }
                const float part = ((w4[0] + w4[1]) + w4[2]) + w4[3];
                const float incl = wave_incl_scan_dpp(part);
                if (lane == 63) s_wsum[wave] = incl;
                __syncthreads();
                float run = incl - part;
                for (int w = 0; w < wave; ++w) run += s_wsum[w];
                uint32_t first = 0u, lastw = 0u;  // row + 1, 0 = none
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    run += w4[i];
                    if (first == 0u && w4[i] > 0.0f && run > qo) first = (uint32_t)(r0 + i) + 1u;
                    if (w4[i] > 0.0f) lastw = (uint32_t)(r0 + i) + 1u;
                }
                const uint32_t fmin = wave_max_u32(first ? 0xFFFFFFFFu - first : 0u);
                const uint32_t lmax = wave_max_u32(lastw);
                if (lane == 0) {
                    s_wfirst[wave] = fmin;
                    s_wlast[wave] = lmax;
                }
                __syncthreads();
                if (t == 0) {
                    const uint32_t f = max(max(s_wfirst[0], s_wfirst[1]), max(s_wfirst[2], s_wfirst[3]));
                    const uint32_t l = max(max(s_wlast[0], s_wlast[1]), max(s_wlast[2], s_wlast[3]));
                    const int row = f ? (int)(0xFFFFFFFFu - f) - 1 : (l ? (int)l - 1 : -1);
                    const int tok = checked_token(row < 0 ? -1 : ov0 + row, V, status);
                    walk_skew(p, c, k, 1);
                    st_agent64(DSW_OWN(b), ((unsigned long long)(unsigned)tok << 24) | dep);
                }
            }
            __syncthreads();
        }
        __syncthreads();
        if (s_abort) break;

        // ---- decisions of every request: its token ---------------------------
        if (t < B) {
            unsigned it = 0;
            unsigned long long w = 0ull;
            bool ok = true;
            while (((w = ld_agent64(DSW_OWN(t))) & kDecEpochMask) != dep) {
                if (++it >= p.spin_limit) { latch(status, kStatusTimeout); ok = false; break; }
                if ((it & 255u) == 0u && ld_agent(status) != 0u) { ok = false; break; }
                __builtin_amdgcn_s_sleep(1);
            }
            if (!ok) s_abort = 1;
            const int tok = ok ? checked_token((int)((w >> 24) & 0xFFFFFu), V, status) : 0;
            if constexpr (FD == 4) {
                // up to 4 requests: straight into the next step's previous
                // token (nothing reads s_prev between this step's DMA issue and
                // the barrier below), one barrier per step fewer
                s_prev[t] = tok;
                if (c == 0 && ok) p.tokens[(size_t)t * gamma + k] = tok;
            } else {
                s_next[t] = tok;
            }
        }
        __syncthreads();
        if (s_abort) break;
        DSW_TRACE(k, kTrArrived);

        if constexpr (FD != 4) {
            if (t < B) {
                if (c == 0) p.tokens[(size_t)t * gamma + k] = s_next[t];
                s_prev[t] = s_next[t];
            }
            __syncthreads();
        }
        DSW_TRACE(k, kTrSelected);
        DSW_TRACE_REAL(k);
    }
#undef DSW_OWN
#undef DSW_ISSUE_GROUP
#undef DSW_READ_COLUMN
#undef DSW_OWNER_SHARD
#undef DSW_BLOCK_MAX64
#undef DSW_TILES
#undef DSW_TILES_F4
#undef DSW_TILE_OFFCHIP

    wait_vmcnt(0);  // a walk that gave up may still have a prefetch in flight
    DSW_TRACE_FLUSH();
    if (c == 0 && t == 0 && !s_abort) {
        __hip_atomic_fetch_add(p.ws.round_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(p.ws.fam_ctr + kFamBatched, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// (register tiles, tiles per wave) shapes of the batched kernel
#define DSW_BATCHED_SHAPES(X) X(4, 4) X(8, 8) X(8, 12) X(10, 12) X(0, 12)
#define DSW_BATCHED_I8_SHAPES(X) X(8, 8) X(8, 12) X(0, 12)

}  // namespace dsw
