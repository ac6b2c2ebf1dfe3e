// walk_mfma.h -- the persistent walk with its shard GEMV on the matrix cores
// (v_mfma_f32_16x16x32_bf16, gfx950).  Instantiated in walk_mfma_b4.hip and
// walk_mfma_b16.hip.
//
// What is computed ("Keeping the Draft Walk on Chip", tie-pilot-qxw.github.io,
// section "The serial part of a parallel drafter"): for k < gamma,
// u = W1[prev], logit = bf16(base_k + bf16(W2 . u)), tok = argmax (T = 0) or an
// inverse-CDF sample of softmax(logit / T) (vLLM PR #64442, "Details"),
// prev = tok.
//
// Layout on chip.  Workgroup c owns the contiguous rows [c*R, c*R + R) of W2
// (section "The idea: make the walk resident": one slice of vocabulary rows
// per CTA, loaded once per round).  Its rows are cut into 16-row tiles and each
// of the 4 waves takes a contiguous run of tiles_per_wave tiles.  A tile is
// the B operand of a 16x16x32 MFMA (N = 16 rows, K = 32 of the latent), so one
// lane holds 8 bf16 of one row per 32-wide K block: 32 registers per tile.
// The first REG_T tiles of a wave live in VGPR/AGPRs, the next lds_tiles in
// LDS in operand order (conflict-free 16-byte reads), any further tiles are
// re-read from memory every step.
//
// Per step.  u = W1[prev] of every request is the A operand (M = request, so
// up to 16 requests share every MFMA at no extra cost: batching is almost free
// on the matrix cores, section "B200: the bf16 table fits on chip").  Lane l
// receives the fp32 dot products of row l%16 for requests 4*(l/16)..+3, so
// each request's results sit in one 16-lane DPP row: the workgroup argmax is a
// DPP row max plus a 4-way LDS step, no cross-row shuffles.  The epilogue
// rounds twice to bf16 (bias, then base + bias) and packs {ordered bf16 logit,
// ~row} keys (ties resolve to the smallest id, section "The idea").
//
// Rendezvous.  Every workgroup stores its keys (and, for sampled requests, the
// shard's exp-sum) into its own mailbox line tagged with the step epoch; every
// workgroup reads all lines.  Sampling scans the shard masses in vocabulary
// order; the shard holding u*Z finds the token inside its rows and publishes it
// through a token mailbox.
#pragma once
#include "walk_device.h"

namespace dsw {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_tile(const uint4 a, const uint4 b, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// Global 36-bit key (ordered bf16 logit, ~vocabulary id) from a workgroup-local
// 32-bit key (ordered bf16 logit, ~row within the shard); 0 stays 0.
__device__ __forceinline__ unsigned long long global_key(uint32_t lk, int v0) {
    if (lk == 0u) return 0ull;
    const uint32_t row = 0xFFFFu - (lk & 0xFFFFu);
    const uint32_t v = (uint32_t)v0 + row;
    return ((unsigned long long)(lk >> 16) << kIdxBits) | (unsigned long long)(kIdxMask - v);
}

template <int REG_T, int MAXT, int NB>
__global__ void __launch_bounds__(kBlock, 1) walk_mfma(WalkParams p) {
    static_assert(NB == 4 || NB == 16, "batch tile");
    static_assert(REG_T <= MAXT && REG_T <= kMaxRegTiles, "register tiles");
    constexpr int RPAD = MAXT * 4 * kTileRows;          // rows per workgroup, upper bound
    constexpr int CHMAX = (RPAD + kBlock - 1) / kBlock; // shard rows per thread in a scan
    constexpr int US = kRowChunks + 1;                  // padded u row, in uint4
    extern __shared__ uint4 s_w[];                      // LDS tiles [wave*lds_tiles + j][8][64]

    __shared__ uint4 s_u[NB * US];
    __shared__ uint16_t s_base[NB * RPAD];
    __shared__ uint16_t s_logit[NB * RPAD];
    __shared__ uint32_t s_best[4][NB];
    __shared__ unsigned long long s_red64[4][NB];
    __shared__ float s_redf[4][NB];
    __shared__ float s_scan[kMaxGrid];
    __shared__ int s_redi[4];
    __shared__ float s_T[NB];
    __shared__ float s_tot[NB];
    __shared__ float s_excl[NB * kBlock];  // exclusive prefix of each thread's rows' masses
    __shared__ int s_prev[NB];
    __shared__ unsigned s_round;
    __shared__ int s_abort;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int g = lane >> 4;  // DPP row: requests 4g .. 4g+3 in the accumulators
    const int n = lane & 15;  // row within a tile
    const int c = blockIdx.x;
    const int G = gridDim.x;
    const int V = p.V;
    const int B = p.B;
    const int gamma = p.gamma;
    const int v0 = c * p.rows_per_wg;
    const int nrows = max(0, min(V, v0 + p.rows_per_wg) - v0);
    const int TW = p.tiles_per_wave;
    const int LT = p.lds_tiles;
    const int wrow0 = wave * TW * kTileRows;
    const int nt_w = max(0, min(TW, (nrows - wrow0 + kTileRows - 1) / kTileRows));
    const uint4* __restrict__ W2 = reinterpret_cast<const uint4*>(p.W2);
    const uint4* __restrict__ W1 = reinterpret_cast<const uint4*>(p.W1);
    const uint16_t* __restrict__ base = p.base;
    unsigned* status = p.ws.status;

    if (t == 0) {
        s_round = ld_agent(p.ws.round_ctr);
        s_abort = 0;
    }
    DSW_TRACE(gamma, 0);
    if (t < NB) {
        int a = 0;
        float temp = 0.0f;
        if (t < B) {
            a = p.anchor[t];
            temp = p.T[t];
            if (a < 0 || a >= V) {
                if (c == 0) latch(status, kStatusToken);
                a = 0;
            }
            if (temp > 0.0f && p.uniforms == nullptr) {
                if (c == 0) latch(status, kStatusUniforms);
                temp = 0.0f;
            }
            if (!(temp > 0.0f)) temp = 0.0f;
        }
        s_prev[t] = a;
        s_T[t] = temp;
    }
    for (int j = t; j < NB * US; j += kBlock) s_u[j] = make_uint4(0u, 0u, 0u, 0u);

    // ---- entry: this workgroup's shard on chip -------------------------
    uint4 wr[REG_T > 0 ? REG_T : 1][8];
#pragma unroll
    for (int j = 0; j < REG_T; ++j) {
        const int r = wrow0 + j * kTileRows + n;
        if (j < nt_w && r < nrows) {
            const uint4* src = W2 + (size_t)(v0 + r) * kRowChunks + g;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) wr[j][kb] = src[kb * 4];
        } else {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) wr[j][kb] = make_uint4(0u, 0u, 0u, 0u);
        }
        // The tile must stay in registers for the whole walk: hide where the
        // values came from, so the compiler cannot re-load them from W2 later.
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            asm volatile("" : "+v"(wr[j][kb].x), "+v"(wr[j][kb].y), "+v"(wr[j][kb].z), "+v"(wr[j][kb].w));
    }
    for (int idx = t; idx < 4 * LT * 512; idx += kBlock) {
        const int s = idx >> 9, kb = (idx >> 6) & 7, ln = idx & 63;
        const int ws = s / LT;
        const int j = REG_T + (s - ws * LT);
        const int nt_ws = max(0, min(TW, (nrows - ws * TW * kTileRows + kTileRows - 1) / kTileRows));
        if (j < nt_ws) {  // only tiles that exist in this shard have an LDS slot
            const int r = ws * TW * kTileRows + j * kTileRows + (ln & 15);
            s_w[idx] = (r < nrows) ? W2[(size_t)(v0 + r) * kRowChunks + kb * 4 + (ln >> 4)] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    for (int idx = t; idx < NB * RPAD; idx += kBlock) {
        const int b = idx / RPAD, r = idx - b * RPAD;
        s_base[idx] = (b < B && r < nrows) ? base[((size_t)b * gamma) * V + v0 + r] : (uint16_t)0;
    }
    __syncthreads();
    const unsigned round = s_round;
    bool any_samp = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) any_samp |= (b < B) && (s_T[b] > 0.0f);
    const int CH = (nrows + kBlock - 1) / kBlock;  // rows per thread in vocabulary-order scans


    // ---- the walk --------------------------------------------------------
    for (int k = 0; k < gamma; ++k) {
        DSW_TRACE(k, kTrStepStart);
        const unsigned seq = round * (unsigned)p.gamma_max + (unsigned)k;
        const unsigned long long epoch = (unsigned long long)(seq % kEpochMod + 1u);
        const int q = (int)(seq & 1u);
        unsigned long long* mail_q = p.ws.mail + (size_t)q * kMaxGrid * kMailWords;

        if (k > 0) {  // this step's base logits for the shard (step 0 was staged at entry)
            for (int b = 0; b < B; ++b) {
                const uint16_t* src = base + ((size_t)b * gamma + k) * V + v0;
                for (int r = t; r < nrows; r += kBlock) s_base[b * RPAD + r] = src[r];
            }
        }
        // gather u = W1[prev] for every request
        for (int j = t; j < B * kRowChunks; j += kBlock) {
            const int b = j >> 5, ch = j & 31;
            s_u[b * US + ch] = W1[(size_t)s_prev[b] * kRowChunks + ch];
        }
        __syncthreads();
        DSW_TRACE(k, kTrGathered);

        // A operand: lane l carries u of request l%16, latent 8*(l/16).. of each K block
        uint4 a[8];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) a[kb] = (n < B) ? s_u[n * US + kb * 4 + g] : make_uint4(0u, 0u, 0u, 0u);

        uint32_t best[4] = {0u, 0u, 0u, 0u};
        // lane's first staged (request 4g, row wrow0 + n) element; tile j and
        // request 4g+i sit at constant offsets from it
        const int lofs = 4 * g * RPAD + wrow0 + n;
        // bias = bf16(acc), logit = bf16(base + bias) for the lane's four
        // requests of tile j; keys {ordered logit, ~row}; logits staged in LDS
#define DSW_EPILOGUE(dv, j)                                                                     \
    do {                                                                                        \
        const int r_ = wrow0 + (j) * kTileRows + n;                                             \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                         \
            if (4 * g + i < B && r_ < nrows) {                                                  \
                const int e_ = lofs + i * RPAD + (j) * kTileRows;                               \
                const uint32_t bias_ = f32_to_bf16((dv)[i]);                                    \
                const uint32_t lb_ = f32_to_bf16(bf16_to_f32(s_base[e_]) + bf16_to_f32(bias_)); \
                best[i] = max(best[i], (ord16(lb_) << 16) | (0xFFFFu - (uint32_t)r_));          \
                s_logit[e_] = (uint16_t)lb_;                                                    \
            }                                                                                   \
        }                                                                                       \
    } while (0)

        // register tiles: K-block outer so the MFMAs of different tiles overlap
        f32x4_t d[REG_T > 0 ? REG_T : 1];
#pragma unroll
        for (int j = 0; j < (REG_T > 0 ? REG_T : 1); ++j) d[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int j = 0; j < REG_T; ++j)
                if (j < nt_w) d[j] = mfma_tile(a[kb], wr[j][kb], d[j]);
#pragma unroll
        for (int j = 0; j < REG_T; ++j)
            if (j < nt_w) DSW_EPILOGUE(d[j], j);
        // LDS and streamed tiles, one at a time
#pragma unroll 1
        for (int j = REG_T; j < MAXT; ++j) {
            if (j < nt_w) {
                f32x4_t dd = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                if (j - REG_T < LT) {
                    const int sb = (wave * LT + (j - REG_T)) * 512 + lane;
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) dd = mfma_tile(a[kb], s_w[sb + kb * 64], dd);
                } else {
                    const int r = wrow0 + j * kTileRows + n;
                    const bool ok = r < nrows;
                    const uint4* src = W2 + (size_t)(v0 + (ok ? r : 0)) * kRowChunks + g;
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) dd = mfma_tile(a[kb], ok ? src[kb * 4] : make_uint4(0u, 0u, 0u, 0u), dd);
                }
                DSW_EPILOGUE(dd, j);
            }
        }
#undef DSW_EPILOGUE
        DSW_TRACE(k, kTrGemvDone);

        // workgroup argmax per request: DPP row max, then the 4 waves
#pragma unroll
        for (int i = 0; i < 4; ++i) best[i] = row16_max_u32(best[i]);
        if (n == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * g + i < NB) s_best[wave][4 * g + i] = best[i];
        }
        __syncthreads();
        DSW_TRACE(k, kTrReduced);

        // sampled requests: masses w = exp((l - m_c) / T) of the shard's rows in
        // vocabulary order; each thread owns CH consecutive rows
        if (any_samp) {
            float part[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                part[b] = 0.0f;
                if (b < B && s_T[b] > 0.0f) {
                    const uint32_t lk = max(max(s_best[0][b], s_best[1][b]), max(s_best[2][b], s_best[3][b]));
                    const float ml = bf16_to_f32(unord16(lk >> 16));
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
                    incl[b] = wave_incl_scan(part[b], lane);
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
            __syncthreads();
        }

        // ---- rendezvous: post, prefetch the next base, read every mailbox ----
        if (wave == 0 && lane < B) {
            const uint32_t lk = max(max(s_best[0][lane], s_best[1][lane]), max(s_best[2][lane], s_best[3][lane]));
            unsigned long long* box = mail_q + (size_t)c * kMailWords;
            st_agent64(&box[lane], (global_key(lk, v0) << 28) | epoch);
            if (s_T[lane] > 0.0f)
                st_agent64(&box[kMaxBatchPersistent + lane],
                           ((unsigned long long)__float_as_uint(s_tot[lane]) << 32) | epoch);
        }
        DSW_TRACE(k, kTrPosted);
        if (p.logits != nullptr) {  // the exact values the tokens are selected from
            for (int b = 0; b < B; ++b) {
                uint16_t* dst = p.logits + ((size_t)b * gamma + k) * V + v0;
                for (int r = t; r < nrows; r += kBlock) dst[r] = s_logit[b * RPAD + r];
            }
        }
        unsigned long long kw[NB];
        float sw[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            kw[b] = 0ull;
            sw[b] = 0.0f;
        }
        if (t < G) {
            const unsigned long long* box = mail_q + (size_t)t * kMailWords;
            unsigned it = 0;
            for (;;) {
                bool ready = true;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < B) {
                        const unsigned long long wk = ld_agent64(&box[b]);
                        if ((wk & kEpochMod) == epoch) kw[b] = wk >> 28;
                        else ready = false;
                        if (s_T[b] > 0.0f) {
                            const unsigned long long ws = ld_agent64(&box[kMaxBatchPersistent + b]);
                            if ((ws & kEpochMod) == epoch) sw[b] = __uint_as_float((uint32_t)(ws >> 32));
                            else ready = false;
                        }
                    }
                }
                if (ready) break;
                if (++it >= p.spin_limit) {
                    latch(status, kStatusTimeout);
                    s_abort = 1;
                    break;
                }
                if ((it & 255u) == 0u && ld_agent(status) != 0u) {
                    s_abort = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        DSW_TRACE(k, kTrArrived);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const unsigned long long m = wave_max_u64(kw[b]);
            if (lane == 0) s_red64[wave][b] = m;
        }
        __syncthreads();
        if (s_abort) break;
        unsigned long long win[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            unsigned long long m = s_red64[0][b];
#pragma unroll
            for (int w = 1; w < 4; ++w) m = s_red64[w][b] > m ? s_red64[w][b] : m;
            win[b] = m;
        }

        // ---- selection ----------------------------------------------------
        if (t < B) {
            unsigned long long mine = 0ull;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b == t) mine = win[b];
            if (!(s_T[t] > 0.0f)) s_prev[t] = checked_token(key_index(mine), V, status);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (!((b < B) && (s_T[b] > 0.0f))) continue;
            const float Tb = s_T[b];
            const float M = key_logit(win[b]);
            unsigned long long* tbox = p.ws.tok_mail + (size_t)q * kMaxBatchPersistent + b;
            // shard masses S_c = s_c * exp((m_c - M) / T), scanned in shard order
            float S = 0.0f;
            if (t < G && kw[b] != 0ull) S = sw[b] * __expf((key_logit(kw[b]) - M) / Tb);
            float P = wave_incl_scan(S, lane);
            if (lane == 63) s_redf[wave][0] = P;
            __syncthreads();
            float off = 0.0f, Z = 0.0f;
            for (int w = 0; w < 4; ++w) {
                if (w < wave) off += s_redf[w][0];
                Z += s_redf[w][0];
            }
            P += off;
            s_scan[t] = P;  // inclusive prefix over shards 0..t
            const float target = p.uniforms[(size_t)b * gamma + k] * Z;
            const int below = (t < G && P <= target) ? 1 : 0;
            const int last_pos = (t < G && S > 0.0f) ? t : -1;
            const int nb = __popcll(__ballot(below));
            const int lp = wave_max_i(last_pos);
            if (lane == 0) s_redi[wave] = nb;
            __syncthreads();
            int owner = s_redi[0] + s_redi[1] + s_redi[2] + s_redi[3];
            __syncthreads();
            if (lane == 0) s_redi[wave] = lp;
            __syncthreads();
            const int last_c = max(max(s_redi[0], s_redi[1]), max(s_redi[2], s_redi[3]));
            if (owner >= G) owner = last_c;
            __syncthreads();
            if (c == owner) {
                // the first row of this shard whose cumulative mass exceeds target
                const float pexcl = (owner == 0) ? 0.0f : s_scan[owner - 1];
                const uint32_t lk = max(max(s_best[0][b], s_best[1][b]), max(s_best[2][b], s_best[3][b]));
                const float ml = bf16_to_f32(unord16(lk >> 16));
                const float scale = __expf((ml - M) / Tb);
                float run = s_excl[b * kBlock + t];
                int first = 0x7FFFFFFF, lastw = -1;
#pragma unroll
                for (int rr = 0; rr < CHMAX; ++rr) {
                    const int r = t * CH + rr;
                    if (rr < CH && r < nrows) {
                        const float w = __expf((bf16_to_f32(s_logit[b * RPAD + r]) - ml) / Tb);
                        run += w;
                        if (first == 0x7FFFFFFF && pexcl + scale * run > target) first = r;
                        if (w > 0.0f) lastw = r;
                    }
                }
                first = wave_min_i(first);
                lastw = wave_max_i(lastw);
                if (lane == 0) s_redi[wave] = first;
                __syncthreads();
                first = min(min(s_redi[0], s_redi[1]), min(s_redi[2], s_redi[3]));
                __syncthreads();
                if (lane == 0) s_redi[wave] = lastw;
                __syncthreads();
                lastw = max(max(s_redi[0], s_redi[1]), max(s_redi[2], s_redi[3]));
                const int tok = checked_token(v0 + (first != 0x7FFFFFFF ? first : lastw), V, status);
                if (t == 0) {
                    s_prev[b] = tok;
                    st_agent64(tbox, ((unsigned long long)(unsigned)tok << 32) | epoch);
                }
            } else if (t == 0) {
                unsigned it = 0;
                unsigned long long v = 0ull;
                while (((v = ld_agent64(tbox)) & kEpochMod) != epoch) {
                    if (++it >= p.spin_limit) {
                        latch(status, kStatusTimeout);
                        s_abort = 1;
                        break;
                    }
                    if ((it & 255u) == 0u && ld_agent(status) != 0u) {
                        s_abort = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                s_prev[b] = s_abort ? 0 : checked_token((int)(v >> 32), V, status);
            }
            __syncthreads();
        }
        if (s_abort) break;
        if (c == 0)
            for (int b = t; b < B; b += kBlock) p.tokens[(size_t)b * gamma + k] = s_prev[b];
        __syncthreads();
        DSW_TRACE(k, kTrSelected);
        if (p.trace != nullptr && t == 0)
            p.trace[((size_t)c * (gamma + 1) + k) * 8 + kTrReal] = __builtin_amdgcn_s_memrealtime();
    }

    if (c == 0 && t == 0 && !s_abort)
        __hip_atomic_fetch_add(p.ws.round_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// (register tiles, tiles per wave) shapes compiled for every batch tile
#define DSW_MFMA_SHAPES(X) X(2, 2) X(4, 4) X(8, 8) X(8, 10) X(8, 16) X(0, 16)

}  // namespace dsw
