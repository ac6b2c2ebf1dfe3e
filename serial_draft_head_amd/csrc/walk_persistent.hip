// walk_persistent.hip -- one persistent launch per round of DSpark's serial
// Markov draft walk, written for gfx950 (MI355X).
//
// What is computed ("Keeping the Draft Walk on Chip", tie-pilot-qxw.github.io,
// section "The serial part of a parallel drafter"): for k < gamma,
// u = W1[prev], logit = bf16(base_k + bf16(W2 . u)), tok = argmax (T = 0) or an
// inverse-CDF sample of softmax(logit / T) (vLLM PR #64442, "Details"),
// prev = tok.
//
// How it runs (the resident design of section "The idea: make the walk
// resident", re-planned for CDNA4):
//   * one workgroup of 4 wave64 per CU; workgroup c owns the contiguous rows
//     [c*R, c*R + R) of W2 and keeps them on chip for the whole walk:
//     REG_SLOTS groups of 256 rows in VGPRs (one row per lane, 128 dwords),
//     then up to lds_rows rows in LDS (XOR-swizzled 16-byte chunks), and any
//     rows left over are re-read from memory every step;
//   * per step every lane computes whole dot products for its rows with
//     v_dot2_f32_bf16 against u broadcast from LDS (fp32 accumulation), then
//     rounds twice to bf16 as the pages' default walk does;
//   * the workgroup reduces its rows to one key per request: the
//     order-preserving bits of the bf16 logit, then the inverted row index, so
//     equal logits resolve to the smallest id (section "The idea");
//   * rendezvous: instead of the pages' atomic {key, count} pair, every
//     workgroup stores its keys into its own mailbox line, tagged with the
//     step's epoch, and every workgroup reads all mailboxes until each carries
//     the epoch.  On MI355X device-scope atomics on one line serialise across
//     the 8 XCDs, so 256 posters cost far more than 256 independent stores;
//   * sampled requests also post each shard's exp-sum (the per-block max and
//     exp-sum of vLLM's sample kernel); every workgroup scans the shard masses
//     in vocabulary order, the shard that holds u*Z finds the token inside its
//     rows and publishes it through a token mailbox;
//   * mailboxes alternate between two buffers by step parity and carry the
//     epoch, so launches and graph replays need no memset (section "The idea").
#include <hip/hip_runtime.h>

#include "walk_device.h"

namespace dsw {

// ------------------------------------------------------------ the kernel
template <int REG_SLOTS, int NB>
__global__ void __launch_bounds__(kBlock, 1) walk_persistent(WalkParams p) {
    static_assert(REG_SLOTS >= 0 && REG_SLOTS <= kMaxSlots, "register slots");
    static_assert(NB <= kMaxBatchPersistent, "batch tile");
    extern __shared__ uint4 s_w[];  // LDS-resident rows: [lds_rows][32] swizzled chunks

    __shared__ uint4 s_u[NB * kRowChunks];  // u = W1[prev] per request
    __shared__ unsigned long long s_red64[4][NB];
    __shared__ float s_redf[4][NB * kMaxSlots];
    __shared__ float s_scan[kMaxGrid];
    __shared__ int s_redi[4];
    __shared__ float s_T[NB];
    __shared__ float s_sloc[NB];
    __shared__ int s_prev[NB];
    __shared__ unsigned s_round;
    __shared__ int s_abort;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int c = blockIdx.x;
    const int G = gridDim.x;
    const int V = p.V;
    const int B = p.B;
    const int gamma = p.gamma;
    const int v0 = c * p.rows_per_wg;
    const int nrows = max(0, min(V, v0 + p.rows_per_wg) - v0);
    const int reg_cap = REG_SLOTS * kBlock;
    const int reg_rows = min(nrows, reg_cap);
    const int lds_rows = min(nrows - reg_rows, p.lds_rows);
    const uint4* __restrict__ W2 = reinterpret_cast<const uint4*>(p.W2);
    const uint4* __restrict__ W1 = reinterpret_cast<const uint4*>(p.W1);
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
    for (int j = t; j < NB * kRowChunks; j += kBlock) s_u[j] = make_uint4(0u, 0u, 0u, 0u);

    // ---- entry: load this workgroup's shard on chip ----------------------
    uint4 wr[REG_SLOTS > 0 ? REG_SLOTS : 1][kRowChunks];
#pragma unroll
    for (int s = 0; s < REG_SLOTS; ++s) {
        const int i = s * kBlock + t;
        if (i < reg_rows) {
            const uint4* src = W2 + (size_t)(v0 + i) * kRowChunks;
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
    // base logits of step 0 for the lane's rows (later steps are prefetched
    // one step ahead, while the rendezvous is in flight)
    uint32_t bs[NB][kMaxSlots];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int s = 0; s < kMaxSlots; ++s) {
            const int i = s * kBlock + t;
            bs[b][s] = (b < B && i < nrows) ? (uint32_t)p.base[((size_t)b * gamma) * V + v0 + i] : 0u;
        }
    __syncthreads();
    const unsigned round = s_round;

    // ---- the walk --------------------------------------------------------
    for (int k = 0; k < gamma; ++k) {
        DSW_TRACE(k, kTrStepStart);
        const unsigned seq = round * (unsigned)p.gamma_max + (unsigned)k;
        const unsigned long long epoch = (unsigned long long)(seq % kEpochMod + 1u);
        const int q = (int)(seq & 1u);
        unsigned long long* mail_q = p.ws.mail + (size_t)q * kMaxGrid * kMailWords;

        // gather u = W1[prev] for every request into LDS
        for (int j = t; j < B * kRowChunks; j += kBlock) {
            const int b = j >> 5, ch = j & 31;
            s_u[j] = W1[(size_t)s_prev[b] * kRowChunks + ch];
        }
        __syncthreads();
        DSW_TRACE(k, kTrGathered);

        // shard GEMV, fp32 accumulation
        float acc[NB][kMaxSlots];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int s = 0; s < kMaxSlots; ++s) acc[b][s] = 0.0f;

        if (REG_SLOTS > 0) {
#pragma unroll
            for (int ch = 0; ch < kRowChunks; ++ch) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < B) {
                        const uint4 u4 = s_u[b * kRowChunks + ch];
#pragma unroll
                        for (int s = 0; s < REG_SLOTS; ++s) acc[b][s] = dot8(wr[s][ch], u4, acc[b][s]);
                    }
                }
            }
        }
#pragma unroll
        for (int s = REG_SLOTS; s < kMaxSlots; ++s) {
            const int i = s * kBlock + t;
            if (i < nrows) {
                const int il = i - reg_cap;
                if (il < lds_rows) {
                    for (int ch = 0; ch < kRowChunks; ++ch) {
                        const uint4 w4 = s_w[il * kRowChunks + (ch ^ (il & 31))];
#pragma unroll
                        for (int b = 0; b < NB; ++b)
                            if (b < B) acc[b][s] = dot8(w4, s_u[b * kRowChunks + ch], acc[b][s]);
                    }
                } else {
                    const uint4* src = W2 + (size_t)(v0 + i) * kRowChunks;
                    for (int ch = 0; ch < kRowChunks; ++ch) {
                        const uint4 w4 = src[ch];
#pragma unroll
                        for (int b = 0; b < NB; ++b)
                            if (b < B) acc[b][s] = dot8(w4, s_u[b * kRowChunks + ch], acc[b][s]);
                    }
                }
            }
        }

        // epilogue: bias = bf16(acc), logit = bf16(base + bias); local best key
        float lg[NB][kMaxSlots];
        unsigned long long best[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            best[b] = 0ull;
#pragma unroll
            for (int s = 0; s < kMaxSlots; ++s) {
                const int i = s * kBlock + t;
                const uint32_t bias = f32_to_bf16(acc[b][s]);
                const uint32_t lbits = f32_to_bf16(bf16_to_f32(bs[b][s]) + bf16_to_f32(bias));
                const bool valid = (b < B) && (i < nrows);
                lg[b][s] = valid ? bf16_to_f32(lbits) : -INFINITY;
                if (valid) {
                    const unsigned long long key = make_key(lbits, (uint32_t)(v0 + i));
                    best[b] = key > best[b] ? key : best[b];
                    if (p.logits != nullptr)
                        p.logits[((size_t)b * gamma + k) * V + v0 + i] = (uint16_t)lbits;
                }
            }
        }
        DSW_TRACE(k, kTrGemvDone);
        // prefetch the next step's base logits; they land during the rendezvous
        if (k + 1 < gamma) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int s = 0; s < kMaxSlots; ++s) {
                    const int i = s * kBlock + t;
                    bs[b][s] = (b < B && i < nrows)
                                   ? (uint32_t)p.base[((size_t)b * gamma + k + 1) * V + v0 + i]
                                   : 0u;
                }
        }
        // workgroup max of the keys
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const unsigned long long m = wave_max_u64(best[b]);
            if (lane == 0) s_red64[wave][b] = m;
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            unsigned long long m = s_red64[0][b];
#pragma unroll
            for (int w = 1; w < 4; ++w) m = s_red64[w][b] > m ? s_red64[w][b] : m;
            best[b] = m;
        }
        DSW_TRACE(k, kTrReduced);

        // sampled requests: local weights w = exp((l - m_c) / T), their
        // inclusive prefix in vocabulary order (slot-major, then lane), and
        // the shard total s_c
        float cw[NB][kMaxSlots];
        bool any_sampled = false;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float Tb = s_T[b];
            const bool samp = (b < B) && (Tb > 0.0f);
            any_sampled |= samp;
            const float m = (best[b] != 0ull) ? key_logit(best[b]) : 0.0f;
#pragma unroll
            for (int s = 0; s < kMaxSlots; ++s) {
                cw[b][s] = 0.0f;
                if (samp) {  // uniform across the workgroup
                    const float w = (lg[b][s] != -INFINITY) ? __expf((lg[b][s] - m) / Tb) : 0.0f;
                    cw[b][s] = wave_incl_scan(w, lane);
                    if (lane == 63) s_redf[wave][b * kMaxSlots + s] = cw[b][s];
                }
            }
        }
        if (any_sampled) {
            __syncthreads();
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if ((b < B) && (s_T[b] > 0.0f)) {
                    float carry = 0.0f;
#pragma unroll
                    for (int s = 0; s < kMaxSlots; ++s) {
                        float before = carry;
                        for (int w = 0; w < 4; ++w) {
                            if (w < wave) before += s_redf[w][b * kMaxSlots + s];
                            carry += s_redf[w][b * kMaxSlots + s];
                        }
                        cw[b][s] += before;
                    }
                    if (t == 0) s_sloc[b] = carry;
                }
            }
            __syncthreads();
        }

        // ---- rendezvous: post this workgroup's mailbox words ---------------
        if (wave == 0 && lane < B) {
            unsigned long long mine = 0ull;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b == lane) mine = best[b];
            unsigned long long* box = mail_q + (size_t)c * kMailWords;
            st_agent64(&box[lane], (mine << 28) | epoch);
            if (s_T[lane] > 0.0f)
                st_agent64(&box[kMaxBatchPersistent + lane],
                           ((unsigned long long)__float_as_uint(s_sloc[lane]) << 32) | epoch);
        }
        DSW_TRACE(k, kTrPosted);
        // ... and read every workgroup's words: thread t reads workgroup t
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
            bool ready = false;
            while (!ready) {
                ready = true;
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
        // global argmax per request
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
            // owner shard: the first c whose inclusive prefix exceeds target
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
                const float mloc = key_logit(best[b]);
                const float scale = __expf((mloc - M) / Tb);
                int first = 0x7FFFFFFF, lastw = -1;
#pragma unroll
                for (int s = 0; s < kMaxSlots; ++s) {
                    const int i = s * kBlock + t;
                    if (i < nrows && lg[b][s] != -INFINITY) {
                        if (pexcl + scale * cw[b][s] > target) first = min(first, i);
                        if (__expf((lg[b][s] - mloc) / Tb) > 0.0f) lastw = max(lastw, i);
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

// ------------------------------------------------------------ dispatch
typedef void (*walk_fn)(WalkParams);

template <int R>
static walk_fn pick_nb(int nb) {
    switch (nb) {
        case 1: return walk_persistent<R, 1>;
        case 4: return walk_persistent<R, 4>;
        case 16: return walk_persistent<R, 16>;
        default: return nullptr;
    }
}

}  // namespace dsw

// Host-side lookup used by the launcher (api.cpp).  Returns the kernel for
// (register slots, batch tile) or nullptr when it is not compiled.
extern "C" const void* dsw_internal_walk_kernel(int reg_slots, int batch_tile) {
    using namespace dsw;
    switch (reg_slots) {
        case 0: return (const void*)pick_nb<0>(batch_tile);
        case 1: return (const void*)pick_nb<1>(batch_tile);
        case 2: return (const void*)pick_nb<2>(batch_tile);
        case 3: return (const void*)pick_nb<3>(batch_tile);
        default: return nullptr;
    }
}
