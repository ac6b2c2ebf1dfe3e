// walk_device.h -- device helpers shared by the walk kernels: bf16 rounding,
// the selection key, device-coherent mailbox I/O, wave reductions, and
// loads from global memory straight into LDS.
#pragma once
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

// The bias as the epilogue adds it: rounded to bf16 (dbl = ~0u, the default
// walk's double rounding) or kept in fp32 (dbl = 0, single rounding of the
// sum).  Branch-free with a uniform mask, so it costs no extra registers.
__device__ __forceinline__ float bias_round(float a, uint32_t dbl) {
    uint32_t u = __float_as_uint(a);
    u += (0x7FFFu + ((u >> 16) & 1u)) & dbl;
    return __uint_as_float(u & (0xFFFF0000u | ~dbl));
}

// Two fp32 values -> a bf16 pair (lo in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32.  It agrees bit for bit with f32_to_bf16 on finite
// inputs, ties and denormals included (checked on the device).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

constexpr float kLog2e = 1.4426950408889634f;

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

// ------------------------------------------------------ device uniforms
// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011): per round, counter words 0 and 2 are
// multiplied by the round constants; the high halves of the products are mixed
// with words 3 and 1 and the key, the low halves carried over; the key
// advances by the Weyl constants between rounds.  Returns output word 0.
// All four output words, in place of the counter.
__device__ __forceinline__ void philox4(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint32_t h0 = __umulhi(0xD2511F53u, c[0]), l0 = 0xD2511F53u * c[0];
        const uint32_t h1 = __umulhi(0xCD9E8D57u, c[2]), l1 = 0xCD9E8D57u * c[2];
        const uint32_t n0 = h1 ^ c[1] ^ k0, n2 = h0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = l1;
        c[2] = n2;
        c[3] = l0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
    uint32_t c[4] = {c0, c1, c2, c3};
    philox4(c, k0, k1);
    return c[0];
}

// The uniform of request b at step k: supplied by the caller, or drawn on the
// device, keyed by (seed, request, step, round counter) as the pages' kernel
// keys its noise ("Keeping the Draft Walk on Chip", section "The idea: make
// the walk resident"), so every launch and graph replay draws fresh values:
// the top 24 bits of Philox word 0, as a multiple of 2^-24 in [0, 1).
__device__ __forceinline__ float walk_uniform(const WalkParams& p, int b, int k, int gamma, unsigned round) {
    if (p.uniforms != nullptr) return p.uniforms[(size_t)b * gamma + k];
    const uint32_t w = philox_word0((uint32_t)k, (uint32_t)b, round, 0x44535721u, (uint32_t)p.seed,
                                    (uint32_t)(p.seed >> 32));
    return (float)(w >> 8) * (1.0f / 16777216.0f);
}

// Gumbel-max noise ("Keeping the Draft Walk on Chip", section "The idea: make
// the walk resident": small batches sample by per-row Gumbel-max from Philox
// noise keyed by seed, row, step and round counter).  Vocabulary rows 4m ..
// 4m+3 of request b at step k share the call on counter (m, 256 k + b, round,
// 0x47554D42); word e maps to U = (2 (w >> 9) + 1) 2^-24, strictly inside
// (0, 1) and exact in fp32.  Returns the variate G = -ln(-ln U), both
// logarithms taken with the hardware base-2 logarithm (v_log_f32) times ln 2,
// straight on U.  Over all 2^23 values U can take, -ln U stays within 2e-7
// relative and G within 2e-6 absolute of binary64 (a GPU test evaluates this
// function on every one of them, dsw_debug_gumbel_table).
__device__ __forceinline__ float gumbel_of_word(uint32_t w) {
    const float U = (float)(2u * (w >> 9) + 1u) * (1.0f / 16777216.0f);
    const float e = -0.69314718f * __builtin_amdgcn_logf(U);
    return -0.69314718f * __builtin_amdgcn_logf(e);
}

// Order-preserving 32-bit image of an fp32 score (-0 maps like +0; every
// finite score maps above 0, so a zero key never wins).
__device__ __forceinline__ uint32_t ord32(float s) {
    uint32_t b = __float_as_uint(s);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Selection key (36 bits): order-preserving bits of the bf16 logit, then the
// inverted row index (rows < 2^20).  Larger key = larger logit, then smaller id.
constexpr int kIdxBits = 20;
constexpr unsigned kIdxMask = (1u << kIdxBits) - 1u;
__device__ __forceinline__ unsigned long long make_key(uint32_t lbits, uint32_t v) {
    if (lbits == 0x8000u) lbits = 0u;  // -0 and +0 compare equal
    const uint32_t ord = (lbits & 0x8000u) ? (~lbits & 0xFFFFu) : (lbits | 0x8000u);
    return ((unsigned long long)ord << kIdxBits) | (unsigned long long)(kIdxMask - v);
}
__device__ __forceinline__ float key_logit(unsigned long long key) {
    const uint32_t ord = (uint32_t)(key >> kIdxBits) & 0xFFFFu;
    const uint32_t b = (ord & 0x8000u) ? (ord & 0x7FFFu) : (~ord & 0xFFFFu);
    return bf16_to_f32(b);
}
__device__ __forceinline__ int key_index(unsigned long long key) {
    return (int)(kIdxMask - ((uint32_t)key & kIdxMask));
}

// ------------------------------------------------------- wave reductions
// Over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one 16-lane column in each
// row of 16): v_permlane16_swap of a value with itself leaves rows {0, 0, 2,
// 2} in one result and {1, 1, 3, 3} in the other, v_permlane32_swap halves
// {lo, lo} and {hi, hi}; combining the two results after each swap gives
// every lane the column's maximum (or sum) with VALU work only.
__device__ __forceinline__ uint32_t column4_max_u32(uint32_t x) {
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)a[0], (uint32_t)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((uint32_t)b[0], (uint32_t)b[1]);
}
__device__ __forceinline__ float column4_sum_f32(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long y = __shfl_xor(x, off, 64);
        x = x > y ? x : y;
    }
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

// Diagnostics (dsw_set_debug): with p.skew != 0, the calling wave sleeps
// before a post for a pseudo-random number (0..7, from the workgroup, step and
// call site) of units of s_sleep 127 (~8k clocks each), so that workgroups
// reach the rendezvous in a scrambled order.  No loop: three fixed sleeps
// guarded by the bits of the count (a loop nested in the step loop measurably
// slowed the walk even when it never ran).
__device__ __forceinline__ void walk_skew(const WalkParams& p, int c, int k, int site) {
    if (p.skew == 0u) return;
    uint32_t h = (uint32_t)c * 0x9E3779B1u ^ ((uint32_t)k * 0x85EBCA77u + (uint32_t)site * 0xC2B2AE3Du);
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    if (h & 1u) __builtin_amdgcn_s_sleep(127);
    if (h & 2u) {
        __builtin_amdgcn_s_sleep(127);
        __builtin_amdgcn_s_sleep(127);
    }
    if (h & 4u) {
        __builtin_amdgcn_s_sleep(127);
        __builtin_amdgcn_s_sleep(127);
        __builtin_amdgcn_s_sleep(127);
        __builtin_amdgcn_s_sleep(127);
    }
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

// --------------------------------------------------- device-coherent I/O
__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_agent64(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two adjacent mailbox words (16-byte aligned) with one agent-scope load: each
// word carries its own epoch, so a read that sees one half updated and not
// the other is simply not ready yet.  The asm waits for its own load, so its
// outputs are complete when it returns (and the wait also covers this wave's
// earlier memory operations).
__device__ __forceinline__ void ld_agent64_pair(const unsigned long long* p, unsigned long long& lo,
                                                unsigned long long& hi) {
    uint4 v;
    asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p));
    lo = ((unsigned long long)v.y << 32) | v.x;
    hi = ((unsigned long long)v.w << 32) | v.z;
}
__device__ __forceinline__ void st_agent64(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint16_t ld_agent16(const uint16_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent16(uint16_t* p, uint16_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void latch(unsigned* status, unsigned bits) {
    __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Max of a 32-bit value over the 16 lanes of a DPP row; every lane of the
// row receives it (quad swaps, then half-row and row mirrors).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, false));
    return x;
}

// DPP controls (gfx9 encoding)
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;

// Max of a 32-bit value over the whole wave, returned to every lane: a DPP
// row max, then the four row results read out as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = row16_max_u32(x);
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane(x, 0), b = (uint32_t)__builtin_amdgcn_readlane(x, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane(x, 32), d = (uint32_t)__builtin_amdgcn_readlane(x, 48);
    return max(max(a, b), max(c, d));
}

// 64-bit max over the whole wave, returned to every lane.
__device__ __forceinline__ unsigned long long wave_max_u64_dpp(unsigned long long x) {
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
#define DSW_STEP64(ctrl)                                                                      \
    do {                                                                                      \
        const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, ctrl, 0xF, 0xF, false); \
        const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, ctrl, 0xF, 0xF, false); \
        const bool gt = (ohi > hi) || (ohi == hi && olo > lo);                                \
        lo = gt ? olo : lo;                                                                   \
        hi = gt ? ohi : hi;                                                                   \
    } while (0)
    DSW_STEP64(kDppQuadSwap1);
    DSW_STEP64(kDppQuadSwap2);
    DSW_STEP64(kDppRowHalfMirror);
    DSW_STEP64(kDppRowMirror);
#undef DSW_STEP64
    unsigned long long best = 0ull;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t rh = (uint32_t)__builtin_amdgcn_readlane(hi, 16 * r);
        const uint32_t rl = (uint32_t)__builtin_amdgcn_readlane(lo, 16 * r);
        const unsigned long long v = ((unsigned long long)rh << 32) | (unsigned long long)rl;
        best = v > best ? v : best;
    }
    return best;
}

// Inclusive prefix sum over the 64 lanes in lane order: DPP row shifts, then
// the row broadcasts carry row totals forward.
__device__ __forceinline__ float wave_incl_scan_dpp(float x) {
#define DSW_ADD(ctrl, rmask)                                                                   \
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rmask, 0xF, false))
    DSW_ADD(kDppRowShr1, 0xF);
    DSW_ADD(kDppRowShr2, 0xF);
    DSW_ADD(kDppRowShr4, 0xF);
    DSW_ADD(kDppRowShr8, 0xF);
    DSW_ADD(kDppRowBcast15, 0xA);
    DSW_ADD(kDppRowBcast31, 0xC);
#undef DSW_ADD
    return x;
}

// Order-preserving 16-bit image of a bf16 pattern (-0 maps like +0).
__device__ __forceinline__ uint32_t ord16(uint32_t lbits) {
    if (lbits == 0x8000u) lbits = 0u;
    return (lbits & 0x8000u) ? (~lbits & 0xFFFFu) : (lbits | 0x8000u);
}
__device__ __forceinline__ uint32_t unord16(uint32_t ord) {
    return (ord & 0x8000u) ? (ord & 0x7FFFu) : (~ord & 0xFFFFu);
}

// Phase timestamps of the optional trace (thread 0 of each workgroup).  They
// are kept in LDS during the walk and written out once at the end, so that
// tracing adds no global stores (and no waits on them) inside the steps.
// Steps beyond kTraceSteps are not recorded; row kTraceSteps holds the kernel
// start, written out as step `gamma`.
#define DSW_TRACE_DECL __shared__ unsigned long long s_trace[kTraceSteps + 1][8]
#define DSW_TRACE_AT(k, ph, clock)                                                          \
    do {                                                                                    \
        if (p.trace != nullptr && t == 0) {                                                 \
            const int kk_ = (k) >= gamma ? kTraceSteps : ((k) < kTraceSteps ? (k) : -1);    \
            if (kk_ >= 0) s_trace[kk_][ph] = clock;                                         \
        }                                                                                   \
    } while (0)
#define DSW_TRACE(k, ph) DSW_TRACE_AT(k, ph, __builtin_amdgcn_s_memrealtime())
#define DSW_TRACE_REAL(k) DSW_TRACE_AT(k, kTrReal, __builtin_amdgcn_s_memtime())
#define DSW_TRACE_FLUSH()                                                                   \
    do {                                                                                    \
        if (p.trace != nullptr && t == 0) {                                                 \
            for (int k_ = 0; k_ < gamma && k_ < kTraceSteps; ++k_)                          \
                for (int ph_ = 0; ph_ < 8; ++ph_)                                           \
                    p.trace[((size_t)c * (gamma + 1) + k_) * 8 + ph_] = s_trace[k_][ph_];   \
            p.trace[((size_t)c * (gamma + 1) + gamma) * 8] = s_trace[kTraceSteps][0];       \
        }                                                                                   \
    } while (0)

// ------------------------------------------- vector-memory waits, LDS DMA
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int waitcnt_vm_imm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x3 << 14);

// Wait until at most n vector-memory instructions of this wave are in flight.
// No memory access moves across it (a load issued later must not be counted
// as issued earlier).
__device__ __forceinline__ void wait_vmcnt(int n) {
    asm volatile("" ::: "memory");
    switch (n < 0 ? 0 : (n > 31 ? 31 : n)) {
#define DSW_W(i) \
    case i: __builtin_amdgcn_s_waitcnt(waitcnt_vm_imm(i)); break;
        DSW_W(0) DSW_W(1) DSW_W(2) DSW_W(3) DSW_W(4) DSW_W(5) DSW_W(6) DSW_W(7)
        DSW_W(8) DSW_W(9) DSW_W(10) DSW_W(11) DSW_W(12) DSW_W(13) DSW_W(14) DSW_W(15)
        DSW_W(16) DSW_W(17) DSW_W(18) DSW_W(19) DSW_W(20) DSW_W(21) DSW_W(22) DSW_W(23)
        DSW_W(24) DSW_W(25) DSW_W(26) DSW_W(27) DSW_W(28) DSW_W(29) DSW_W(30) DSW_W(31)
#undef DSW_W
        default: break;
    }
}

// Workgroup barrier that keeps vector-memory loads (and LDS DMA) in flight:
// this wave's LDS accesses are complete, and the compiler moves no memory
// access across it.  (__syncthreads would also wait for every outstanding
// load, which would drain the prefetch ring at every group.)
__device__ __forceinline__ void barrier_keep_vm() {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16 bytes from global memory straight into LDS: this lane's data lands at
// lds_base + 16 * lane (lds_base is wave-uniform).  Written as inline assembly
// so that the compiler does not treat every later LDS access as waiting on
// it (it would drain the whole ring at each group); the kernel waits for
// these loads itself with wait_vmcnt.  M0 needs one wait state before use.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

}  // namespace dsw
