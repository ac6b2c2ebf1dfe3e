// api.cpp -- the C ABI of include/dsw.h: device probing, handle and workspace
// management, argument checks and the one persistent launch per round.
#include <hip/hip_runtime_api.h>
#include <string.h>

#include <mutex>
#include <new>

#include "../../include/dsw.h"
#include "launch.h"
#include "walk_params.h"

extern "C" const void* dsw_internal_walk_kernel(int reg_slots, int batch_tile, int w2_dtype);
extern "C" const void* dsw_internal_mfma_kernel_b1(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_kernel_b4(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_kernel_b16(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_i8_kernel(int batch_tile, int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_batched_kernel(int w2_dtype, int reg_tiles, int max_tiles, int single_round,
                                                   int fold, int gumbel);
// the same all-to-all kernels with Gumbel-max sampling
extern "C" const void* dsw_internal_walk_kernel_gumbel(int reg_slots, int batch_tile, int w2_dtype);
extern "C" const void* dsw_internal_mfma_kernel_b1_gumbel(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_kernel_b4_gumbel(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_kernel_b16_gumbel(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_i8_kernel_gumbel(int batch_tile, int reg_tiles, int max_tiles);
// the one-request kernels for the GRU and RNN serial heads
extern "C" const void* dsw_internal_mfma_kernel_b1_gru(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_kernel_b1_rnn(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_kernel_b1_gated(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_kernel_b1_domino(int reg_tiles, int max_tiles);
// one request with int8 rows widened to bf16 at entry
extern "C" const void* dsw_internal_mfma_kernel_b1_i8(int reg_tiles, int max_tiles);
extern "C" const void* dsw_internal_mfma_kernel_b1_i8_gumbel(int reg_tiles, int max_tiles);

namespace {
// The compiled kernel a plan runs (with Gumbel-max sampling when `gumbel`), or
// nullptr.  The planner never gives a Gumbel-max handle the batched kernel.
// The head a handle's flags select: 0 the Markov head, 1 the GRU head, 2 the
// RNN head, 3 the gated head, 4 Domino's head.
int cell_of(unsigned flags) {
    if (flags & DSW_FLAG_GRU) return 1;
    if (flags & DSW_FLAG_RNN) return 2;
    if (flags & DSW_FLAG_GATED) return 3;
    return (flags & DSW_FLAG_DOMINO) ? 4 : 0;
}

// cell: as cell_of; single: DSW_FLAG_SINGLE_ROUND (the batched kernel is
// compiled for each rounding)
const void* kernel_for(const dsw_plan_info& pl, bool gumbel, int cell, bool single, int B) {
    if (cell) {  // the planner gives the recurrent heads only the one-request MFMA engine
        if (pl.engine != DSW_ENGINE_MFMA || pl.batch_tile != 1 || pl.w2_dtype != DSW_BF16) return nullptr;
        const void* (*const lookup[])(int, int) = {dsw_internal_mfma_kernel_b1_gru, dsw_internal_mfma_kernel_b1_rnn,
                                                   dsw_internal_mfma_kernel_b1_gated,
                                                   dsw_internal_mfma_kernel_b1_domino};
        return cell <= 4 ? lookup[cell - 1](pl.reg_tiles, pl.max_tiles) : nullptr;
    }
    if (pl.batch_tile == dsw::kMaxBatch) {
        // up to 4 requests share one epilogue per four tiles (bf16, double
        // rounding)
        return dsw_internal_batched_kernel(pl.w2_dtype, pl.reg_tiles, pl.max_tiles, single, B <= 4, gumbel);
    }
    if (pl.engine == DSW_ENGINE_VALU)
        return gumbel ? dsw_internal_walk_kernel_gumbel(pl.reg_slots, pl.batch_tile, pl.w2_dtype)
                      : dsw_internal_walk_kernel(pl.reg_slots, pl.batch_tile, pl.w2_dtype);
    if (pl.w2_dtype == DSW_INT8 && pl.batch_tile == 1)
        return gumbel ? dsw_internal_mfma_kernel_b1_i8_gumbel(pl.reg_tiles, pl.max_tiles)
                      : dsw_internal_mfma_kernel_b1_i8(pl.reg_tiles, pl.max_tiles);
    if (pl.w2_dtype == DSW_INT8)
        return gumbel ? dsw_internal_mfma_i8_kernel_gumbel(pl.batch_tile, pl.reg_tiles, pl.max_tiles)
                      : dsw_internal_mfma_i8_kernel(pl.batch_tile, pl.reg_tiles, pl.max_tiles);
    if (pl.batch_tile == 1)
        return gumbel ? dsw_internal_mfma_kernel_b1_gumbel(pl.reg_tiles, pl.max_tiles)
                      : dsw_internal_mfma_kernel_b1(pl.reg_tiles, pl.max_tiles);
    if (pl.batch_tile == 4)
        return gumbel ? dsw_internal_mfma_kernel_b4_gumbel(pl.reg_tiles, pl.max_tiles)
                      : dsw_internal_mfma_kernel_b4(pl.reg_tiles, pl.max_tiles);
    if (pl.batch_tile == 16)
        return gumbel ? dsw_internal_mfma_kernel_b16_gumbel(pl.reg_tiles, pl.max_tiles)
                      : dsw_internal_mfma_kernel_b16(pl.reg_tiles, pl.max_tiles);
    return nullptr;
}
}  // namespace

struct dsw_handle {
    int device;
    int V, r, gamma_max, B_max, dtype;
    unsigned flags;
    dsw_devinfo dev;
    dsw_devinfo pdev;  // what the planner sees: dev, with the workgroup count capped by dsw_set_grid
    char* ws_mem;
    size_t ws_bytes;
    uint16_t* blog_mem;  // batched kernel: logits of sampled requests, [B_max][V] bf16
    dsw::Workspace ws;
    unsigned long long seed;    // key of device-drawn uniforms (when seeded)
    int seeded;
    unsigned long long* trace;  // optional device trace buffer (caller-owned)
    long long trace_bytes;
    unsigned spin_limit;        // polls before a device wait gives up
    unsigned skew;              // diagnostics: pseudo-random delays before posts (0 = none)
};

namespace {

// Makes `device` current for the lifetime of the guard and restores the
// caller's device afterwards.
struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int device) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        ok = hipSetDevice(device) == hipSuccess;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

int clear_workspace(dsw_handle* h) {
    if (hipMemset(h->ws_mem, 0, h->ws_bytes) != hipSuccess) return DSW_ERR_HIP;
    if (hipDeviceSynchronize() != hipSuccess) return DSW_ERR_HIP;
    return DSW_OK;
}

}  // namespace

extern "C" int dsw_device_info(int device, dsw_devinfo* out) {
    if (!out) return DSW_ERR_NULL;
    memset(out, 0, sizeof(*out));
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return DSW_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return DSW_ERR_HIP;
    out->cu_count = prop.multiProcessorCount;
    out->simds_per_cu = 4;
    out->wave_size = prop.warpSize;
    out->vgprs_per_simd_lane = 512;
    int lds_cu = 0, lds_blk = 0, coop = 0, clock = 0;
    (void)hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device);
    (void)hipDeviceGetAttribute(&lds_blk, hipDeviceAttributeMaxSharedMemoryPerBlock, device);
    (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device);
    (void)hipDeviceGetAttribute(&clock, hipDeviceAttributeClockRate, device);
    out->lds_bytes_per_cu = lds_cu > 0 ? lds_cu : (int)prop.sharedMemPerBlock;
    out->max_lds_per_block = lds_blk > 0 ? lds_blk : (int)prop.sharedMemPerBlock;
    out->xcd_count = 8;
    out->clock_khz = clock;
    out->l2_bytes = prop.l2CacheSize;
    out->hbm_bytes = (long long)prop.totalGlobalMem;
    out->cooperative = coop;
    return DSW_OK;
}

extern "C" int dsw_create(dsw_handle_t* out, int device, int V, int r, int gamma_max, int B_max,
                          int w2_dtype, unsigned flags) {
    if (!out) return DSW_ERR_NULL;
    *out = nullptr;
    if (r != dsw::kRank) return DSW_ERR_RANK;
    if (w2_dtype != DSW_BF16 && w2_dtype != DSW_INT8) return DSW_ERR_DTYPE;
    if (V < 1) return DSW_ERR_VOCAB;
    if (gamma_max < 1 || gamma_max > dsw::kMaxGammaMax) return DSW_ERR_GAMMA;
    if (B_max < 1 || B_max > dsw::kMaxBatch) return DSW_ERR_BATCH;
    dsw_devinfo dev;
    int rc = dsw_device_info(device, &dev);
    if (rc) return rc;
    dsw_plan_info plan;
    rc = dsw_plan_compute(&dev, V, r, gamma_max, B_max, w2_dtype, flags, &plan);
    if (rc) return rc;
    if ((flags & DSW_FLAG_COOPERATIVE) && !dev.cooperative) return DSW_ERR_LAUNCH;

    dsw_handle* h = new (std::nothrow) dsw_handle();
    if (!h) return DSW_ERR_ARG;
    h->device = device;
    h->V = V;
    h->r = r;
    h->gamma_max = gamma_max;
    h->B_max = B_max;
    h->dtype = w2_dtype;
    h->flags = flags;
    h->dev = dev;
    h->pdev = dev;
    h->trace = nullptr;
    h->trace_bytes = 0;
    h->spin_limit = dsw::kSpinLimit;
    h->skew = 0u;
    h->seed = 0ull;
    h->seeded = 0;

    DeviceGuard g(device);
    if (!g.ok) { delete h; return DSW_ERR_DEVICE; }
    const dsw::WorkspaceLayout L = dsw::workspace_layout();
    h->ws_bytes = L.total;
    if (hipMalloc(&h->ws_mem, L.total) != hipSuccess) { delete h; return DSW_ERR_HIP; }
    h->ws.mail = reinterpret_cast<unsigned long long*>(h->ws_mem + L.mail);
    h->ws.tokw = reinterpret_cast<unsigned long long*>(h->ws_mem + L.tokw);
    h->ws.round_ctr = reinterpret_cast<unsigned*>(h->ws_mem + L.ctl) + dsw::kCtlRound;
    h->ws.fam_ctr = reinterpret_cast<unsigned*>(h->ws_mem + L.ctl) + dsw::kCtlFam;
    h->ws.status = reinterpret_cast<unsigned*>(h->ws_mem + L.ctl) + dsw::kCtlStatus;
    h->ws.bkey = reinterpret_cast<unsigned long long*>(h->ws_mem + L.bkey);
    h->ws.bdec = reinterpret_cast<unsigned long long*>(h->ws_mem + L.bdec);
    // the batched kernel writes the current step's logits of its sampled
    // requests here for their owners
    h->blog_mem = nullptr;
    if (B_max >= dsw::kBatchedFrom || (flags & DSW_FLAG_BATCHED)) {
        if (hipMalloc(&h->blog_mem, dsw::batched_logits_bytes(V, B_max)) != hipSuccess) {
            (void)hipFree(h->ws_mem);
            delete h;
            return DSW_ERR_HIP;
        }
    }
    h->ws.blog = h->blog_mem;
    if (clear_workspace(h) != DSW_OK) {
        (void)hipFree(h->ws_mem);
        if (h->blog_mem) (void)hipFree(h->blog_mem);
        delete h;
        return DSW_ERR_HIP;
    }
    // Residency: every batch size this handle serves must fit one workgroup
    // on each CU within the LDS limit, and the grid must not exceed the CUs;
    // short walks (up to 3 steps) may plan another kernel, so they are checked too.
    const int n_g = gamma_max > 3 ? 2 : 1;
    for (int i = 0; i < B_max * n_g; ++i) {
        const int B = 1 + i / n_g;
        const int gm = (i % n_g) == 0 ? gamma_max : 3;
        dsw_plan_info pl;
        int prc = dsw_plan_compute(&dev, V, r, gm, B, w2_dtype, flags, &pl);
        const void* fn = prc == DSW_OK ? kernel_for(pl, (flags & DSW_FLAG_GUMBEL) != 0, cell_of(flags),
                                                    (flags & DSW_FLAG_SINGLE_ROUND) != 0, B)
                                        : nullptr;
        hipFuncAttributes attr;
        int per_cu = 0;
        bool ok = fn != nullptr && hipFuncGetAttributes(&attr, fn) == hipSuccess &&
                  (int)attr.sharedSizeBytes <= pl.static_lds_bytes &&
                  (int)attr.sharedSizeBytes + pl.lds_bytes <= dev.max_lds_per_block && pl.grid <= dev.cu_count;
        if (ok) {
            (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, pl.lds_bytes);
            ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, pl.block, (size_t)pl.lds_bytes) ==
                     hipSuccess && per_cu >= 1;
        }
        if (!ok) {
            (void)hipGetLastError();
            (void)hipFree(h->ws_mem);
            if (h->blog_mem) (void)hipFree(h->blog_mem);
            delete h;
            return prc != DSW_OK ? prc : DSW_ERR_LAUNCH;
        }
    }
    *out = h;
    return DSW_OK;
}

extern "C" int dsw_query_plan(dsw_handle_t h, int B, dsw_plan_info* out) {
    if (!h || !out) return DSW_ERR_NULL;
    if (B < 0 || B > h->B_max) return DSW_ERR_BATCH;
    return dsw_plan_compute(&h->pdev, h->V, h->r, h->gamma_max, B, h->dtype, h->flags, out);
}

namespace {
using dsw::GruArgs;

// Kernels whose dynamic-LDS ceiling was raised, per device (process-wide).
std::mutex g_lds_mu;
struct LdsEntry {
    const void* fn;
    int device;
    int bytes;
};
LdsEntry g_lds[256];
int g_n_lds = 0;

void raise_lds_ceiling(const void* fn, int device, int bytes) {
    std::lock_guard<std::mutex> lock(g_lds_mu);
    int slot = -1;
    for (int i = 0; i < g_n_lds; ++i)
        if (g_lds[i].fn == fn && g_lds[i].device == device) slot = i;
    if (slot >= 0 && g_lds[slot].bytes >= bytes) return;
    // Raises the dynamic-LDS ceiling where the runtime enforces one; a
    // failure here surfaces as a launch error.
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    (void)hipGetLastError();
    if (slot < 0 && g_n_lds < 256) slot = g_n_lds++;
    if (slot >= 0) g_lds[slot] = LdsEntry{fn, device, bytes};
}

dsw::LaunchCtx ctx_of(const dsw_handle* h) {
    dsw::LaunchCtx x;
    x.device = h->device;
    x.V = h->V;
    x.gamma_max = h->gamma_max;
    x.B_max = h->B_max;
    x.dtype = h->dtype;
    x.flags = h->flags;
    x.dev = &h->pdev;
    x.ws = h->ws;
    x.spin_limit = h->spin_limit;
    x.skew = h->skew;
    x.seeded = h->seeded;
    x.seed = h->seed;
    x.trace = h->trace;
    x.trace_bytes = h->trace_bytes;
    return x;
}

int walk_impl(dsw_handle_t h, const void* W1, const void* W2, const float* w2_scale, const void* base,
              const int32_t* anchor, const float* T, const float* uniforms, int32_t* tokens, void* logits,
              int B, int gamma, void* stream, const GruArgs* gru) {
    if (!h) return DSW_ERR_NULL;
    if (B < 0 || B > h->B_max) return DSW_ERR_BATCH;
    if (gamma < 0 || gamma > h->gamma_max) return DSW_ERR_GAMMA;
    const dsw::LaunchCtx x = ctx_of(h);
    return dsw::launch_walk(x, W1, W2, w2_scale, base, anchor, T, uniforms, tokens, logits, B, gamma, stream, gru,
                            nullptr);
}
}  // namespace

namespace dsw {

int launch_walk(const LaunchCtx& x, const void* W1, const void* W2, const float* w2_scale, const void* base,
                const int32_t* anchor, const float* T, const float* uniforms, int32_t* tokens, void* logits,
                int B, int gamma, void* stream, const GruArgs* gru, dsw_plan_info* plan_out) {
    if (x.dtype == DSW_BF16 && w2_scale != nullptr) return DSW_ERR_DTYPE;
    if (x.dtype == DSW_INT8 && w2_scale == nullptr) return DSW_ERR_DTYPE;
    if (B == 0 || gamma == 0) return DSW_OK;
    if (!W1 || !W2 || !base || !anchor || !T || !tokens) return DSW_ERR_NULL;
    if ((x.flags & DSW_FLAG_GUMBEL) && !x.seeded) return DSW_ERR_ARG;  // the noise needs a seed

    dsw_plan_info plan;
    int rc = dsw_plan_compute(x.dev, x.V, kRank, gamma, B, x.dtype, x.flags, &plan);
    if (rc) return rc;
    if (plan_out) *plan_out = plan;
    const void* fn = kernel_for(plan, (x.flags & DSW_FLAG_GUMBEL) != 0, gru != nullptr ? cell_of(x.flags) : 0,
                                (x.flags & DSW_FLAG_SINGLE_ROUND) != 0, B);
    if (!fn) return DSW_ERR_PLAN;
    if (plan.batch_tile == kMaxBatch && x.ws.blog == nullptr) return DSW_ERR_PLAN;

    DeviceGuard g(x.device);
    if (!g.ok) return DSW_ERR_DEVICE;
    raise_lds_ceiling(fn, x.device, plan.lds_bytes);

    WalkParams p;
    p.W1 = static_cast<const uint16_t*>(W1);
    p.W2 = W2;
    p.w2_scale = w2_scale;
    p.base = static_cast<const uint16_t*>(base);
    p.anchor = anchor;
    p.T = T;
    p.uniforms = uniforms;
    p.tokens = tokens;
    p.logits = static_cast<uint16_t*>(logits);
    p.ws = x.ws;
    p.V = x.V;
    p.B = B;
    p.gamma = gamma;
    p.gamma_max = x.gamma_max;
    p.B_max = x.B_max;
    p.rows_per_wg = plan.rows_per_wg;
    p.lds_rows = plan.lds_rows;
    p.tiles_per_wave = plan.tiles_per_wave;
    p.lds_tiles = plan.lds_tiles;
    p.pf_tiles = plan.prefetch_tiles;
    p.rows_pad = plan.rows_pad;
    p.ring = plan.ring_slots;
    p.aligned = (x.V % 8) == 0;
    p.spin_limit = x.spin_limit;
    p.skew = x.skew;
    p.single_round = (x.flags & DSW_FLAG_SINGLE_ROUND) ? 1 : 0;
    p.seeded = x.seeded;
    p.seed = x.seed;
    p.gru_wih = gru ? gru->wih : nullptr;
    p.gru_whh = gru ? gru->whh : nullptr;
    p.gru_bih = gru ? gru->bih : nullptr;
    p.gru_bhh = gru ? gru->bhh : nullptr;
    p.h0 = gru ? gru->h0 : nullptr;
    p.states = gru ? gru->states : nullptr;
    p.gate_q = gru ? gru->gq : nullptr;
    p.gate_scale = gru ? gru->gs : nullptr;
    p.gate_bias = gru ? gru->gb : nullptr;
    p.hidden = gru ? gru->hidden : nullptr;
    p.hidden_d = gru ? gru->d : 0;
    p.cell_in = kRank + p.hidden_d;
    p.trace = nullptr;
    if (x.trace != nullptr && (long long)plan.grid * (gamma + 1) * 8 * 8 <= x.trace_bytes) p.trace = x.trace;
    void* args[] = {&p};
    hipError_t e;
    if (x.flags & DSW_FLAG_COOPERATIVE)
        e = hipLaunchCooperativeKernel(fn, dim3(plan.grid), dim3(plan.block), args,
                                       (unsigned)plan.lds_bytes, static_cast<hipStream_t>(stream));
    else
        e = hipLaunchKernel(fn, dim3(plan.grid), dim3(plan.block), args, (size_t)plan.lds_bytes,
                            static_cast<hipStream_t>(stream));
    if (e == hipErrorCooperativeLaunchTooLarge) return DSW_ERR_LAUNCH;
    return e == hipSuccess ? DSW_OK : DSW_ERR_HIP;
}

}  // namespace dsw

extern "C" int dsw_walk(dsw_handle_t h, const void* W1, const void* W2, const float* w2_scale,
                        const void* base, const int32_t* anchor, const float* T,
                        const float* uniforms, int32_t* tokens, void* logits, int B, int gamma,
                        void* stream) {
    if (h && cell_of(h->flags)) return DSW_ERR_ARG;  // the heads' own entry points serve these handles
    return walk_impl(h, W1, W2, w2_scale, base, anchor, T, uniforms, tokens, logits, B, gamma, stream, nullptr);
}

extern "C" int dsw_walk_gru(dsw_handle_t h, const void* W1, const void* W2, const void* Wih, const void* Whh,
                            const float* bih, const float* bhh, const float* h0, const void* base,
                            const int32_t* anchor, const float* T, const float* uniforms, int32_t* tokens,
                            void* logits, float* states, int B, int gamma, void* stream) {
    if (!h) return DSW_ERR_NULL;
    if (cell_of(h->flags) != 1) return DSW_ERR_ARG;
    if (B > 0 && gamma > 0 && (!Wih || !Whh || !bih || !bhh || !h0)) return DSW_ERR_NULL;
    const GruArgs g{static_cast<const uint16_t*>(Wih), static_cast<const uint16_t*>(Whh), bih, bhh, h0, states,
                    nullptr, nullptr, nullptr, nullptr, 0};
    return walk_impl(h, W1, W2, nullptr, base, anchor, T, uniforms, tokens, logits, B, gamma, stream, &g);
}

extern "C" int dsw_walk_rnn(dsw_handle_t h, const void* W1, const void* W2, const void* Wih, const void* Whh,
                            const float* bih, const float* bhh, const float* h0, const void* base,
                            const int32_t* anchor, const float* T, const float* uniforms, int32_t* tokens,
                            void* logits, float* states, int B, int gamma, void* stream) {
    if (!h) return DSW_ERR_NULL;
    if (cell_of(h->flags) != 2) return DSW_ERR_ARG;
    if (B > 0 && gamma > 0 && (!Wih || !Whh || !bih || !bhh || !h0)) return DSW_ERR_NULL;
    const GruArgs g{static_cast<const uint16_t*>(Wih), static_cast<const uint16_t*>(Whh), bih, bhh, h0, states,
                    nullptr, nullptr, nullptr, nullptr, 0};
    return walk_impl(h, W1, W2, nullptr, base, anchor, T, uniforms, tokens, logits, B, gamma, stream, &g);
}

extern "C" int dsw_walk_gated(dsw_handle_t h, const void* W1, const void* W2, const void* Gq,
                              const float* gate_scale, const float* gate_bias, const float* h0, const void* base,
                              const int32_t* anchor, const float* T, const float* uniforms, int32_t* tokens,
                              void* logits, float* states, int B, int gamma, void* stream) {
    if (!h) return DSW_ERR_NULL;
    if (cell_of(h->flags) != 3) return DSW_ERR_ARG;
    if (B > 0 && gamma > 0) {
        if (!Gq || !gate_scale || !gate_bias || !h0) return DSW_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(Gq) % 16 != 0) return DSW_ERR_ARG;  // read as 16-byte words
    }
    const GruArgs g{nullptr, nullptr, nullptr, nullptr, h0, states, static_cast<const int8_t*>(Gq), gate_scale,
                    gate_bias, nullptr, 0};
    return walk_impl(h, W1, W2, nullptr, base, anchor, T, uniforms, tokens, logits, B, gamma, stream, &g);
}

extern "C" int dsw_walk_domino(dsw_handle_t h, const void* W1, const void* W2, const void* Wih, const void* Whh,
                               const float* bih, const float* bhh, const float* h0, const void* H, int d,
                               const void* base, const int32_t* anchor, const float* T, const float* uniforms,
                               int32_t* tokens, void* logits, float* states, int B, int gamma, void* stream) {
    if (!h) return DSW_ERR_NULL;
    if (cell_of(h->flags) != 4) return DSW_ERR_ARG;
    if (d < 8 || d > dsw::kDominoMaxD || d % 8 != 0) return DSW_ERR_ARG;
    if (B > 0 && gamma > 0) {
        if (!Wih || !Whh || !bih || !bhh || !h0 || !H) return DSW_ERR_NULL;
        // read as 16-byte words
        if (reinterpret_cast<uintptr_t>(Wih) % 16 != 0 || reinterpret_cast<uintptr_t>(H) % 16 != 0)
            return DSW_ERR_ARG;
    }
    const GruArgs g{static_cast<const uint16_t*>(Wih), static_cast<const uint16_t*>(Whh), bih, bhh, h0, states,
                    nullptr, nullptr, nullptr, static_cast<const uint16_t*>(H), d};
    return walk_impl(h, W1, W2, nullptr, base, anchor, T, uniforms, tokens, logits, B, gamma, stream, &g);
}

extern "C" int dsw_set_seed(dsw_handle_t h, unsigned long long seed, int enable) {
    if (!h) return DSW_ERR_NULL;
    h->seed = seed;
    h->seeded = enable ? 1 : 0;
    return DSW_OK;
}

extern "C" int dsw_round_counter(dsw_handle_t h, unsigned* out) {
    if (!h || !out) return DSW_ERR_NULL;
    DeviceGuard g(h->device);
    if (!g.ok) return DSW_ERR_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return DSW_ERR_HIP;
    if (hipMemcpy(out, h->ws.round_ctr, sizeof *out, hipMemcpyDeviceToHost) != hipSuccess) return DSW_ERR_HIP;
    return DSW_OK;
}

extern "C" int dsw_set_debug(dsw_handle_t h, unsigned spin_limit, unsigned skew) {
    if (!h) return DSW_ERR_NULL;
    if (skew > 1u) return DSW_ERR_ARG;
    h->spin_limit = spin_limit ? spin_limit : dsw::kSpinLimit;
    h->skew = skew;
    return DSW_OK;
}

extern "C" int dsw_set_grid(dsw_handle_t h, int grid) {
    if (!h) return DSW_ERR_NULL;
    if (grid < 0 || grid > h->dev.cu_count) return DSW_ERR_ARG;
    h->pdev = h->dev;
    if (grid > 0) h->pdev.cu_count = grid;
    return DSW_OK;
}

extern "C" int dsw_set_round_counter(dsw_handle_t h, unsigned value) {
    if (!h) return DSW_ERR_NULL;
    DeviceGuard g(h->device);
    if (!g.ok) return DSW_ERR_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return DSW_ERR_HIP;
    const unsigned v[3] = {value, value, value};
    if (hipMemcpy(h->ws.round_ctr, &v[0], sizeof v[0], hipMemcpyHostToDevice) != hipSuccess) return DSW_ERR_HIP;
    if (hipMemcpy(h->ws.fam_ctr, &v[1], 2 * sizeof v[0], hipMemcpyHostToDevice) != hipSuccess) return DSW_ERR_HIP;
    return DSW_OK;
}

extern "C" unsigned dsw_debug_epoch(unsigned seq) { return dsw::epoch_of(seq); }

extern "C" int dsw_internal_gumbel_table(float* out, void* stream);
extern "C" int dsw_debug_gumbel_table(float* out, void* stream) {
    if (!out) return DSW_ERR_NULL;
    return dsw_internal_gumbel_table(out, stream) == 0 ? DSW_OK : DSW_ERR_HIP;
}

extern "C" int dsw_set_trace(dsw_handle_t h, void* trace, long long bytes) {
    if (!h) return DSW_ERR_NULL;
    if (trace != nullptr && bytes < 0) return DSW_ERR_ARG;
    h->trace = static_cast<unsigned long long*>(trace);
    h->trace_bytes = trace ? bytes : 0;
    return DSW_OK;
}

extern "C" int dsw_status(dsw_handle_t h) {
    if (!h) return DSW_ERR_NULL;
    DeviceGuard g(h->device);
    if (!g.ok) return DSW_ERR_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return DSW_ERR_HIP;
    unsigned st = 0;
    if (hipMemcpy(&st, h->ws.status, sizeof st, hipMemcpyDeviceToHost) != hipSuccess) return DSW_ERR_HIP;
    if (st == 0) return DSW_OK;
    // the parity state may be half-written after a failed round: start clean
    if (clear_workspace(h) != DSW_OK) return DSW_ERR_HIP;
    if (st & dsw::kStatusTimeout) return DSW_ERR_DEV_TIMEOUT;
    if (st & dsw::kStatusToken) return DSW_ERR_DEV_TOKEN;
    return DSW_ERR_DEV_UNIFORMS;
}

extern "C" int dsw_destroy(dsw_handle_t h) {
    if (!h) return DSW_OK;
    {
        DeviceGuard g(h->device);
        if (h->ws_mem) {
            (void)hipDeviceSynchronize();
            (void)hipFree(h->ws_mem);
        }
        if (h->blog_mem) (void)hipFree(h->blog_mem);
    }
    delete h;
    return DSW_OK;
}

extern "C" const char* dsw_strerror(int code) {
    switch (code) {
        case DSW_OK: return "ok";
        case DSW_ERR_NULL: return "a required pointer is NULL";
        case DSW_ERR_BATCH: return "batch size out of range";
        case DSW_ERR_GAMMA: return "walk length out of range";
        case DSW_ERR_RANK: return "rank must be 256";
        case DSW_ERR_DTYPE: return "unsupported W2 dtype or scale mismatch";
        case DSW_ERR_VOCAB: return "vocabulary size out of range for this device";
        case DSW_ERR_LAUNCH: return "the persistent grid cannot be co-resident";
        case DSW_ERR_HIP: return "HIP runtime error";
        case DSW_ERR_DEVICE: return "no such device";
        case DSW_ERR_PLAN: return "no execution plan fits";
        case DSW_ERR_ARG: return "invalid argument";
        case DSW_ERR_SCRATCH: return "the walk needs more workspace than the static scratch array holds";
        case DSW_ERR_DEV_TIMEOUT: return "device: a cross-workgroup wait exceeded its bound";
        case DSW_ERR_DEV_TOKEN: return "device: token id outside [0, V)";
        case DSW_ERR_DEV_UNIFORMS: return "device: T > 0 but uniforms is NULL";
        default: return "unknown error";
    }
}
