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
//   * the workgroup reduces its rows to one 64-bit key per request
//     (order-preserving bits of the fp32 logit, then the inverted row index,
//     so equal logits resolve to the smallest id: section "The idea"), posts
//     it with a device-scope atomic max, counts its arrival with an atomic
//     add and waits until every workgroup has arrived;
//   * sampled requests also post each shard's {local max, local exp-sum}
//     (the per-block max and exp-sum of vLLM's sample kernel); after the
//     rendezvous every workgroup scans the shard masses in vocabulary order,
//     the shard that holds u*Z finds the token inside its rows and publishes
//     it through a mailbox;
//   * the cross-workgroup slots alternate with the parity of a device round
//     counter, so repeated launches need no memset (section "The idea").
#include <hip/hip_runtime.h>

#include "walk_params.h"

namespace dsw {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; inf stays inf).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float dot8(const uint4 w, const uint4 u, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x),
                                          __builtin_bit_cast(bf16x2_t, u.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y),
                                          __builtin_bit_cast(bf16x2_t, u.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z),
                                          __builtin_bit_cast(bf16x2_t, u.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w),
                                          __builtin_bit_cast(bf16x2_t, u.w), acc, false);
    return acc;
}

// 64-bit selection key: order-preserving bits of the logit, then ~index.
__device__ __forceinline__ unsigned long long make_key(float logit, uint32_t v) {
    uint32_t b = __float_as_uint(logit);
    if (b == 0x80000000u) b = 0u;  // -0 and +0 compare equal
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - v);
}
__device__ __forceinline__ float key_logit(unsigned long long key) {
    const uint32_t ord = (uint32_t)(key >> 32);
    const uint32_t b = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    return __uint_as_float(b);
}
__device__ __forceinline__ int key_index(unsigned long long key) {
    return (int)(0xFFFFFFFFu - (uint32_t)key);
}

// ------------------------------------------------------- wave reductions
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long y = __shfl_xor(x, off, 64);
        x = x > y ? x : y;
    }
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off, 64));
    return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
    return x;
}
// inclusive prefix sum across the 64 lanes of a wave
__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// A token id that will index W1: out-of-range ids latch kStatusToken and
// are replaced by 0 so that no access leaves the table.
__device__ __forceinline__ int checked_token(int tok, int V, unsigned* status) {
    if (tok < 0 || tok >= V) {
        __hip_atomic_fetch_or(status, kStatusToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
    }
    return tok;
}

// ------------------------------------------------------ device atomics
__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent64(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll *p until it reaches `target`; gives up after `limit` polls (or when
// another workgroup has already latched a status) and returns false.
__device__ __noinline__ bool wait_at_least(const unsigned* p, unsigned target, unsigned limit,
                                           unsigned* status) {
    unsigned it = 0;
    while (ld_agent(p) < target) {
        if (++it >= limit) {
            __hip_atomic_fetch_or(status, kStatusTimeout, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        if ((it & 255u) == 0u && ld_agent(status) != 0u) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}
__device__ __noinline__ unsigned wait_nonzero(const unsigned* p, unsigned limit, unsigned* status) {
    unsigned it = 0, v;
    while ((v = ld_agent(p)) == 0u) {
        if (++it >= limit) {
            __hip_atomic_fetch_or(status, kStatusTimeout, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            return 0u;
        }
        if ((it & 255u) == 0u && ld_agent(status) != 0u) return 0u;
        __builtin_amdgcn_s_sleep(1);
    }
    return v;
}

// ------------------------------------------------------------ the kernel
template <int REG_SLOTS, int NB>
__global__ void __launch_bounds__(kBlock, 1) walk_persistent(WalkParams p) {
    static_assert(REG_SLOTS >= 0 && REG_SLOTS <= kMaxSlots, "register slots");
    extern __shared__ uint4 s_w[];  // LDS-resident rows: [lds_rows][32] swizzled chunks

    __shared__ uint4 s_u[NB * kRowChunks];            // u = W1[prev] per request
    __shared__ unsigned long long s_red64[4][NB];
    __shared__ float s_redf[4][NB * kMaxSlots];
    __shared__ float s_scan[kMaxGrid];
    __shared__ int s_redi[4];
    __shared__ unsigned long long s_key[NB];
    __shared__ float s_T[NB];
    __shared__ float s_mloc[NB];
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
    if (t < NB) {
        int a = 0;
        float temp = 0.0f;
        if (t < B) {
            a = p.anchor[t];
            temp = p.T[t];
            if (a < 0 || a >= V) {
                if (c == 0)
                    __hip_atomic_fetch_or(status, kStatusToken, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                a = 0;
            }
            if (temp > 0.0f && p.uniforms == nullptr) {
                if (c == 0)
                    __hip_atomic_fetch_or(status, kStatusUniforms, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                temp = 0.0f;
            }
            if (!(temp > 0.0f)) temp = 0.0f;
        }
        s_prev[t] = a;
        s_T[t] = temp;
    }
    for (int j = t; j < NB * kRowChunks; j += kBlock) s_u[j] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const unsigned par = s_round & 1u;
    const size_t slot_base = (size_t)par * p.gamma_max * p.B_max;

    // Clear the other parity's slots for the next launch (the previous
    // launch, which used them, has finished).
    if (c == 0) {
        const size_t other = (size_t)(1u - par) * p.gamma_max * p.B_max;
        for (int j = t; j < p.gamma_max * p.B_max; j += kBlock) {
            p.ws.keys[other + j] = 0ull;
            p.ws.tok_slots[other + j] = 0u;
        }
        for (int j = t; j < p.gamma_max; j += kBlock)
            p.ws.counts[(size_t)(1u - par) * p.gamma_max + j] = 0u;
    }

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

    // ---- the walk --------------------------------------------------------
    for (int k = 0; k < gamma; ++k) {
        // gather u = W1[prev] for every request into LDS
        for (int j = t; j < B * kRowChunks; j += kBlock) {
            const int b = j >> 5, ch = j & 31;
            s_u[j] = W1[(size_t)s_prev[b] * kRowChunks + ch];
        }
        // this step's base logits for the lane's rows
        uint32_t bs[NB][kMaxSlots];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int s = 0; s < kMaxSlots; ++s) {
                const int i = s * kBlock + t;
                bs[b][s] = (b < B && i < nrows)
                               ? (uint32_t)p.base[((size_t)b * gamma + k) * V + v0 + i]
                               : 0u;
            }
        __syncthreads();

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
                const float l = bf16_to_f32(lbits);
                const bool valid = (b < B) && (i < nrows);
                lg[b][s] = valid ? l : -INFINITY;
                if (valid) {
                    const unsigned long long key = make_key(l, (uint32_t)(v0 + i));
                    best[b] = key > best[b] ? key : best[b];
                    if (p.logits != nullptr)
                        p.logits[((size_t)b * gamma + k) * V + v0 + i] = (uint16_t)lbits;
                }
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

        // sampled requests: local weights w = exp((l - m_c) / T), their
        // inclusive prefix in vocabulary order (slot-major, then lane), and
        // the shard total s_c
        float cw[NB][kMaxSlots];   // inclusive prefix of w within the shard (rows of this lane)
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
                    if (t == 0) {
                        s_mloc[b] = (best[b] != 0ull) ? key_logit(best[b]) : -INFINITY;
                        s_sloc[b] = carry;
                    }
                }
            }
        }

        // ---- rendezvous: post keys (and shard masses), count, wait -------
        if (wave == 0) {
            if (lane < B) {
                unsigned long long mine = 0ull;
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b == lane) mine = best[b];
                const size_t slot = slot_base + (size_t)k * p.B_max + lane;
                __hip_atomic_fetch_max(&p.ws.keys[slot], mine, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                if (s_T[lane] > 0.0f) {
                    const unsigned long long pk =
                        ((unsigned long long)__float_as_uint(s_sloc[lane]) << 32) |
                        (unsigned long long)__float_as_uint(s_mloc[lane]);
                    __hip_atomic_store(&p.ws.partials[slot * kMaxGrid + c], pk, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            if (lane == 0) {
                unsigned* cnt = &p.ws.counts[(size_t)par * p.gamma_max + k];
                __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                if (!wait_at_least(cnt, (unsigned)G, p.spin_limit, status)) s_abort = 1;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            if (lane < B) s_key[lane] = ld_agent64(&p.ws.keys[slot_base + (size_t)k * p.B_max + lane]);
        }
        __syncthreads();
        if (s_abort) break;

        // ---- selection ----------------------------------------------------
        for (int b = t; b < B; b += kBlock)
            if (!(s_T[b] > 0.0f)) s_prev[b] = checked_token(key_index(s_key[b]), V, status);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (!((b < B) && (s_T[b] > 0.0f))) continue;
            const float Tb = s_T[b];
            const float M = key_logit(s_key[b]);
            const size_t slot = slot_base + (size_t)k * p.B_max + b;
            // shard masses S_c = s_c * exp((m_c - M) / T), scanned in shard order
            float S = 0.0f;
            if (t < G) {
                const unsigned long long pk = ld_agent64(&p.ws.partials[slot * kMaxGrid + t]);
                const float mc = __uint_as_float((uint32_t)pk);
                const float sc = __uint_as_float((uint32_t)(pk >> 32));
                S = (mc == -INFINITY) ? 0.0f : sc * __expf((mc - M) / Tb);
            }
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
            int nb = __popcll(__ballot(below));
            int lp = wave_max_i(last_pos);
            if (lane == 0) {
                s_redi[wave] = nb;
            }
            __syncthreads();
            int owner = s_redi[0] + s_redi[1] + s_redi[2] + s_redi[3];
            __syncthreads();
            if (lane == 0) s_redi[wave] = lp;
            __syncthreads();
            const int last_c = max(max(s_redi[0], s_redi[1]), max(s_redi[2], s_redi[3]));
            if (owner >= G) owner = last_c;
            __syncthreads();
            if (c == owner) {
                // find the first row of this shard whose cumulative mass exceeds target
                const float pexcl = (owner == 0) ? 0.0f : s_scan[owner - 1];
                const float scale = __expf((s_mloc[b] - M) / Tb);
                int first = 0x7FFFFFFF, lastw = -1;
#pragma unroll
                for (int s = 0; s < kMaxSlots; ++s) {
                    const int i = s * kBlock + t;
                    if (i < nrows && lg[b][s] != -INFINITY) {
                        if (pexcl + scale * cw[b][s] > target) first = min(first, i);
                        if (__expf((lg[b][s] - s_mloc[b]) / Tb) > 0.0f) lastw = max(lastw, i);
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
                    __hip_atomic_store(&p.ws.tok_slots[slot], (unsigned)(tok + 1), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            } else if (t == 0) {
                const unsigned v = wait_nonzero(&p.ws.tok_slots[slot], p.spin_limit, status);
                if (v == 0u) s_abort = 1;
                s_prev[b] = (v == 0u) ? 0 : checked_token((int)(v - 1u), V, status);
            }
            __syncthreads();
        }
        if (s_abort) break;
        if (c == 0)
            for (int b = t; b < B; b += kBlock) p.tokens[(size_t)b * gamma + k] = s_prev[b];
        __syncthreads();
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
