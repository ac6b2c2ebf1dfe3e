// plan.cpp -- residency planner: a pure host function of the device
// description and the walk's sizes (no HIP calls, so it can be exercised with
// invented devices on a machine without a GPU).
//
// Each workgroup (one per CU) owns ceil(V / grid) contiguous vocabulary rows,
// the slice-per-CTA split of "Keeping the Draft Walk on Chip", section "The
// idea: make the walk resident".  The slice goes to registers first, then to
// LDS, and whatever is left is streamed from memory every step, as the pages'
// partially resident kernel does when the table does not fit (section
// "V = 248,320: 62% on chip, the rest streamed").
//
// Two shard-GEMV engines share that plan:
//   MFMA (default): rows in 16-row tiles, a contiguous run of tiles per wave;
//     up to kMaxRegTiles tiles per wave in AGPRs, then LDS tiles, then streamed.
//   VALU: one row per lane in 256-row groups ("slots") in VGPR/AGPRs, then LDS
//     rows, then streamed rows.
#include <string.h>

#include "../../include/dsw.h"
#include "walk_params.h"

namespace dsw {

// LDS of the phase trace's timestamps (kTraceSteps + 1 rows of 8 u64), in every kernel.
static const int kTraceLds = (kTraceSteps + 1) * 8 * 8;

// ---- VALU engine ----------------------------------------------------------
// Largest number of VGPR row groups per lane a compiled kernel holds without
// spilling to scratch (checked in the compiled code objects).  int8 rows are
// widened to bf16 in registers; three widened groups beside the row scales
// spill, so int8 stops at two.
static int valu_reg_slot_cap(int batch_tile, bool i8) {
    if (i8) return 2;
    switch (batch_tile) {
        case 1: return 3;
        case 4: return 2;
        default: return 1;
    }
}
// Gumbel-max kernels of up to 4 requests keep one step's noise per row in LDS.
static int gumbel_noise_lds(int nb, int rpad, bool gum) { return gum && nb <= 4 ? nb * rpad * 4 : 0; }
// Upper bound of the VALU kernel's static LDS for a batch tile (int8 rows add
// their fp32 scales).
static int valu_static_lds(int nb, bool i8, bool gum) {
    return nb * ((kRowChunks + 1) * 16 + kMaxSlots * kBlock * 2 + 2 * 4 * kBlock + 144) + 1104 +
           (i8 ? 4 * kMaxSlots * kBlock : 0) + kTraceLds + gumbel_noise_lds(nb, kMaxSlots * kBlock, gum);
}
static int valu_tile_for(int B) { return B <= 1 ? 1 : (B <= 4 ? 4 : 16); }

// ---- MFMA engine ----------------------------------------------------------
// (register tiles, tiles per wave) shapes compiled for each batch tile; must
// match DSW_MFMA_SHAPES in walk_kernel.h.
static const int kShapes[][2] = {{2, 2}, {4, 4}, {8, 8}, {8, 10}, {8, 16}};
// one request (DSW_MFMA_ONE_SHAPES): AGPR tiles, then up to kMaxVgprTiles VGPR tiles
static const int kShapesOne[][2] = {{2, 2}, {4, 4}, {8, 8}, {10, 10}, {12, 12}, {12, 16}};
// int8 rows (DSW_MFMA_I8_SHAPES): a tile row takes half the registers
static const int kShapesI8[][2] = {{4, 4}, {8, 8}, {16, 16}};
static const int kStreamShape[2] = {0, 16};
// one request (bf16 or int8 rows widened at entry), or 4 / 16 requests
static int mfma_tile_for(int B) { return B <= 1 ? 1 : (B <= 4 ? 4 : 16); }
// Upper bound of the MFMA kernel's static LDS for (batch tile, tiles per
// wave, int8 rows with their fp32 scales).
// A recurrent head keeps its state (r floats) and its cell rows in LDS: per
// owned state element 2 x gates bf16 rows and biases, and the gates' recurrent
// pre-activations of the coming step (GRU: 3 gates, RNN: 1).
// The gated head holds its whole r x r matrix (widened to bf16), the row
// scales and biases, the state, its two low bf16 pieces and the coming
// step's gates.
static int cell_lds(unsigned flags) {
    if (flags & DSW_FLAG_GATED) return kRank * kRank * 2 + 4 * kRank * 4 + 2 * kRank * 2;
    const int gates = (flags & (DSW_FLAG_GRU | DSW_FLAG_DOMINO)) ? 3 : ((flags & DSW_FLAG_RNN) ? 1 : 0);
    // Domino's head: the hidden states' pre-activations of every step and their partial sums
    const int domino = (flags & DSW_FLAG_DOMINO) ? 5 * kDominoMaxGamma * 3 * 4 : 0;
    return gates ? kRank * 4 + kCellMaxPerWg * 2 * gates * (kRank * 2 + 4) + kCellMaxPerWg * gates * 4 + domino : 0;
}
static int mfma_static_lds(int nb, int max_tiles, bool i8, bool gum, unsigned flags) {
    const int rpad = max_tiles * 4 * kTileRows;
    return nb * ((kRowChunks + 1) * 16 + 4 * rpad + 2 * 4 * kBlock + 144) + 1048 + 96 + 128 + (i8 ? 4 * rpad : 0) +
           kTraceLds + gumbel_noise_lds(nb, rpad, gum) + cell_lds(flags);
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Rows of tile j of wave w in the first (largest) shard.
static int tile_rows(int R, int TW, int w, int j) {
    const int r0 = (w * TW + j) * kTileRows;
    const int n = R - r0;
    return n <= 0 ? 0 : (n < kTileRows ? n : kTileRows);
}

static int plan_mfma(const dsw_devinfo* dev, int V, int B, unsigned flags, int grid, int R, bool i8,
                     dsw_plan_info* out) {
    const int tiles = ceil_div(R, kTileRows);
    const int TW = ceil_div(tiles, 4);
    const int nb = mfma_tile_for(B);
    // one request keeps int8 rows widened to bf16 on chip; more requests keep the codes
    const int tile_bytes = (i8 && nb != 1) ? kTileBytes / 2 : kTileBytes;
    int reg_t = -1, max_t = -1;
    if (flags & DSW_FLAG_FORCE_STREAM) {
        reg_t = kStreamShape[0];
        max_t = kStreamShape[1];
    } else if (nb == 1) {
        for (const auto& sh : kShapesOne)
            if (sh[1] >= TW) {
                reg_t = sh[0];
                max_t = sh[1];
                break;
            }
    } else if (i8) {
        for (const auto& sh : kShapesI8)
            if (sh[1] >= TW) {
                reg_t = sh[0];
                max_t = sh[1];
                break;
            }
    } else {
        for (const auto& sh : kShapes)
            if (sh[1] >= TW) {
                reg_t = sh[0];
                max_t = sh[1];
                break;
            }
    }
    if (max_t < TW) return DSW_ERR_VOCAB;
    const int lds_static = mfma_static_lds(nb, max_t, i8, (flags & DSW_FLAG_GUMBEL) != 0, flags);
    int avail = dev->max_lds_per_block - lds_static;
    if (avail < 0) return DSW_ERR_PLAN;

    int n_w[4];
    for (int w = 0; w < 4; ++w) {
        int n = tiles - w * TW;
        n_w[w] = n < 0 ? 0 : (n > TW ? TW : n);
    }
    auto slots = [&](int L) {
        int s = 0;
        for (int w = 0; w < 4; ++w) {
            int extra = n_w[w] - reg_t;
            if (extra < 0) extra = 0;
            s += extra < L ? extra : L;
        }
        return s;
    };
    int LT = TW - reg_t;
    if (LT < 0) LT = 0;
    if (flags & DSW_FLAG_FORCE_STREAM) LT = 0;
    while (LT > 0 && slots(LT) * tile_bytes > avail) --LT;

    int reg_rows = 0, lds_rows = 0, stream_rows = 0;
    for (int w = 0; w < 4; ++w)
        for (int j = 0; j < TW; ++j) {
            const int n = tile_rows(R, TW, w, j);
            if (j < reg_t) reg_rows += n;
            else if (j < reg_t + LT) lds_rows += n;
            else stream_rows += n;
        }

    // one bf16 request in the shape without register tiles: LDS left over
    // takes the first streamed tiles of every wave one step ahead (their
    // slots follow the 4 x LT slots of LDS tiles)
    int PF = 0;
    if (nb == 1 && !i8 && reg_t == 0 && stream_rows > 0) {  // the kernel has it only without register tiles
        const int streamed = TW - reg_t - LT;
        const int room = (avail - 4 * LT * tile_bytes) / (4 * tile_bytes);
        PF = streamed < room ? streamed : room;
        if (PF < 0) PF = 0;
    }
    int lds_bytes = slots(LT) * tile_bytes;
    const int half = dev->lds_bytes_per_cu / 2 + 1024 - lds_static;  // one workgroup per CU
    if (lds_bytes < half) lds_bytes = half;
    if (PF > 0 && lds_bytes < 4 * (LT + PF) * tile_bytes) lds_bytes = 4 * (LT + PF) * tile_bytes;
    if (lds_bytes > avail) lds_bytes = avail;
    if (lds_bytes < slots(LT) * tile_bytes || lds_bytes < 4 * (LT + PF) * tile_bytes * (PF > 0)) return DSW_ERR_PLAN;

    out->engine = DSW_ENGINE_MFMA;
    out->path = stream_rows > 0 ? DSW_PATH_PARTIAL : DSW_PATH_RESIDENT;
    out->grid = grid;
    out->block = kBlock;
    out->rows_per_wg = R;
    out->reg_slots = 0;
    out->reg_rows = reg_rows;
    out->lds_rows = lds_rows;
    out->stream_rows = stream_rows;
    out->batch_tile = nb;
    out->lds_bytes = lds_bytes;
    out->tiles_per_wave = TW;
    out->reg_tiles = reg_t;
    out->lds_tiles = LT;
    out->max_tiles = max_t;
    out->static_lds_bytes = lds_static;
    out->prefetch_tiles = PF;
    return DSW_OK;
}

// ---- batched kernel (walk_batched.h) ---------------------------------------
// (register tiles, tiles per wave); must match DSW_BATCHED_SHAPES and
// DSW_BATCHED_I8_SHAPES.
static const int kBShapes[][2] = {{4, 4}, {8, 8}, {8, 12}};
static const int kBShapesI8[][2] = {{8, 8}, {8, 12}};
static const int kBStreamShape[2] = {0, 12};
static int batched_static_lds(int max_tiles, bool i8) {
    const int rpad = max_tiles * 4 * kTileRows;
    // per-request keys, maxima and exp-sums per wave; tokens (two),
    // temperatures and their two scales; base-row offsets (8 bytes); the shard
    // masses, scales and maxima; int8 row scales; the -inf base rows of dead
    // tiles (4 waves x 64 lanes x 8 bytes) and a few scalars; the trace
    return 4 * kMaxBatch * 4 * 3 + 5 * kMaxBatch * 4 + kMaxBatch * 8 + 3 * kMaxGrid * 4 +
           (i8 ? 4 * rpad : 0) + 4 * 64 * 8 + 1024 + kTraceLds;
}
static int round_up(int x, int m) { return (x + m - 1) / m * m; }

static int plan_batched(const dsw_devinfo* dev, int V, int B, unsigned flags, int grid, bool i8,
                        dsw_plan_info* out) {
    const int R = round_up((V + grid - 1) / grid, kTileRows);  // 16-row aligned shards
    const int Rpad = round_up(R, 128);
    if (Rpad > 1024) return DSW_ERR_VOCAB;  // the kernel's slot indexing assumes <= 1024
    const int tiles = R / kTileRows;
    const int TW = ceil_div(tiles, 4);
    const int tile_bytes = i8 ? kTileBytes / 2 : kTileBytes;
    int reg_t = -1, max_t = -1;
    if (flags & DSW_FLAG_FORCE_STREAM) {
        reg_t = kBStreamShape[0];
        max_t = kBStreamShape[1];
    } else if (i8) {
        for (const auto& sh : kBShapesI8)
            if (sh[1] >= TW) {
                reg_t = sh[0];
                max_t = sh[1];
                break;
            }
    } else {
        for (const auto& sh : kBShapes)
            if (sh[1] >= TW) {
                reg_t = sh[0];
                max_t = sh[1];
                break;
            }
        // 10 to 12 tiles per wave: two more register tiles (in VGPRs), so that
        // a shard of 10 tiles needs no LDS tiles -- except for Gumbel-max beyond
        // 4 requests, whose one-tile epilogue leaves no registers for them
        if (reg_t == 8 && max_t == 12 && TW >= 10 && !((flags & DSW_FLAG_GUMBEL) && B > 4)) reg_t = 10;
    }
    if (max_t < TW) return DSW_ERR_VOCAB;
    const int lds_static = batched_static_lds(max_t, i8);
    const int avail = dev->max_lds_per_block - lds_static;
    const int slot_bytes = 16 * kRowChunks * 16 + 16 * Rpad * 2;  // u rows + base of 16 requests
    // LDS tiles first (4 waves x LT), then at least two ring slots
    int LT = TW - reg_t;
    if (LT < 0) LT = 0;
    if (flags & DSW_FLAG_FORCE_STREAM) LT = 0;
    while (LT > 0 && 4 * LT * tile_bytes + 2 * slot_bytes > avail) --LT;
    int ring = (avail - 4 * LT * tile_bytes) / slot_bytes;
    if (ring > 4) ring = 4;
    if (ring < 2) return DSW_ERR_PLAN;

    int reg_rows = 0, lds_rows = 0, stream_rows = 0;
    for (int w = 0; w < 4; ++w)
        for (int j = 0; j < TW; ++j) {
            const int n = tile_rows(R, TW, w, j);
            if (j < reg_t) reg_rows += n;
            else if (j < reg_t + LT) lds_rows += n;
            else stream_rows += n;
        }
    out->engine = DSW_ENGINE_MFMA;
    out->path = stream_rows > 0 ? DSW_PATH_PARTIAL : DSW_PATH_RESIDENT;
    out->grid = grid;
    out->block = kBlock;
    out->rows_per_wg = R;
    out->reg_rows = reg_rows;
    out->lds_rows = lds_rows;
    out->stream_rows = stream_rows;
    out->batch_tile = kMaxBatch;
    int lds_bytes = 4 * LT * tile_bytes + ring * slot_bytes;
    const int half = dev->lds_bytes_per_cu / 2 + 1024 - lds_static;  // one workgroup per CU
    if (lds_bytes < half) lds_bytes = half < avail ? half : avail;
    out->lds_bytes = lds_bytes;
    out->tiles_per_wave = TW;
    out->reg_tiles = reg_t;
    out->lds_tiles = LT;
    out->max_tiles = max_t;
    out->static_lds_bytes = lds_static;
    out->ring_slots = ring;
    out->rows_pad = Rpad;
    return DSW_OK;
}

static int plan_valu(const dsw_devinfo* dev, int B, unsigned flags, int grid, int R, bool i8,
                     dsw_plan_info* out) {
    if (R > kMaxSlots * kBlock) return DSW_ERR_VOCAB;
    const int row_bytes = kRank * 2;
    const int tile = valu_tile_for(B);
    const int slots = ceil_div(R, kBlock);
    const int cap = valu_reg_slot_cap(tile, i8);
    int reg_slots = slots < cap ? slots : cap;
    if (flags & DSW_FLAG_FORCE_STREAM) reg_slots = 0;
    const int reg_rows = R < reg_slots * kBlock ? R : reg_slots * kBlock;

    const int lds_static = valu_static_lds(tile, i8, (flags & DSW_FLAG_GUMBEL) != 0);
    int lds_avail = dev->max_lds_per_block - lds_static;
    if (lds_avail < 0) lds_avail = 0;
    int lds_rows = R - reg_rows;
    if (lds_rows > lds_avail / row_bytes) lds_rows = lds_avail / row_bytes;
    if (lds_rows > (kMaxSlots - reg_slots) * kBlock) lds_rows = (kMaxSlots - reg_slots) * kBlock;
    if (flags & DSW_FLAG_FORCE_STREAM) lds_rows = 0;
    if (lds_rows < 0) lds_rows = 0;
    const int stream_rows = R - reg_rows - lds_rows;

    int lds_bytes = lds_rows * row_bytes;
    const int half = dev->lds_bytes_per_cu / 2 + 1024 - lds_static;
    if (lds_bytes < half) lds_bytes = half;
    if (lds_bytes + lds_static > dev->max_lds_per_block) lds_bytes = dev->max_lds_per_block - lds_static;
    if (lds_bytes < lds_rows * row_bytes) return DSW_ERR_PLAN;

    out->engine = DSW_ENGINE_VALU;
    out->path = stream_rows > 0 ? DSW_PATH_PARTIAL : DSW_PATH_RESIDENT;
    out->grid = grid;
    out->block = kBlock;
    out->rows_per_wg = R;
    out->reg_slots = reg_slots;
    out->reg_rows = reg_rows;
    out->lds_rows = lds_rows;
    out->stream_rows = stream_rows;
    out->batch_tile = tile;
    out->lds_bytes = lds_bytes;
    out->static_lds_bytes = lds_static;
    return DSW_OK;
}

}  // namespace dsw

extern "C" int dsw_plan_compute(const dsw_devinfo* dev, int V, int r, int gamma, int B,
                                int w2_dtype, unsigned flags, dsw_plan_info* out) {
    using namespace dsw;
    if (!dev || !out) return DSW_ERR_NULL;
    memset(out, 0, sizeof(*out));
    if (r != kRank) return DSW_ERR_RANK;
    if (w2_dtype != DSW_BF16 && w2_dtype != DSW_INT8) return DSW_ERR_DTYPE;
    const bool i8 = w2_dtype == DSW_INT8;
    if (i8 && (flags & DSW_FLAG_VALU_GEMV) && B > 1) return DSW_ERR_DTYPE;  // VALU int8: one request
    if (V < 1 || V > (1 << 20)) return DSW_ERR_VOCAB;  // row ids live in 20 key bits
    if (gamma < 0) return DSW_ERR_GAMMA;
    if (B < 0 || B > kMaxBatch) return DSW_ERR_BATCH;
    if (dev->cu_count < 1 || dev->max_lds_per_block < 1) return DSW_ERR_DEVICE;

    const int grid = dev->cu_count < kMaxGrid ? dev->cu_count : kMaxGrid;
    const long long rows = ((long long)V + grid - 1) / grid;
    if (rows > 4 * 16 * kTileRows) return DSW_ERR_VOCAB;  // 4 waves x 16 tiles x 16 rows
    if ((flags & DSW_FLAG_VALU_GEMV) && (flags & DSW_FLAG_MFMA_GEMV)) return DSW_ERR_ARG;
    const int R = (int)rows;
    // kernel: the batched one beyond 16 requests or when asked for; an engine
    // flag forces the all-to-all kernel (up to 16 requests).  Otherwise, as
    // measured on MI355X: one request on the MFMA engine (V = 151,936,
    // gamma = 7: 39.7 against 42.5 us per round on VALU; int8 rows widened to
    // bf16 on chip when the shard is loaded), the batched kernel from 2
    // requests (V = 151,936, gamma = 16, mixed T: 2 requests 107.2 against
    // 175.1 us on the all-to-all kernel, 3: 130.6 against 254.5; greedy and at
    // V = 32,000 as well), falling back to the all-to-all kernel where it has
    // no shape (e.g. int8 rows beyond 12 tiles per wave).
    const bool forced = (flags & (DSW_FLAG_VALU_GEMV | DSW_FLAG_MFMA_GEMV)) != 0;
    const bool batched = B > kMaxBatchPersistent || (flags & DSW_FLAG_BATCHED);
    if (batched && (flags & DSW_FLAG_VALU_GEMV)) return DSW_ERR_ARG;
    // Gumbel-max: the batched kernel has it for bf16 rows with double rounding
    // (from kBatchedFrom requests, as the inverse CDF); otherwise the
    // all-to-all kernels, up to 16 requests
    const bool gumbel = (flags & DSW_FLAG_GUMBEL) != 0;
    const bool gumbel_batched = gumbel && !i8 && !(flags & DSW_FLAG_SINGLE_ROUND);
    if (batched && gumbel && !gumbel_batched) return DSW_ERR_ARG;
    // the recurrent heads: one bf16 request on the one-request MFMA engine, and
    // (GRU, RNN) a grid of at least r / kCellMaxPerWg workgroups to hold the
    // state; the gated head keeps the whole state in every workgroup
    const unsigned heads = flags & (DSW_FLAG_GRU | DSW_FLAG_RNN | DSW_FLAG_GATED | DSW_FLAG_DOMINO);
    const bool cell = heads != 0;
    if (heads & (heads - 1)) return DSW_ERR_ARG;  // one head per handle
    if (cell) {
        if (B > 1 || batched || gumbel || (flags & DSW_FLAG_VALU_GEMV)) return DSW_ERR_ARG;
        if (i8) return DSW_ERR_DTYPE;
        if (!(flags & DSW_FLAG_GATED) && grid * kCellMaxPerWg < kRank) return DSW_ERR_PLAN;
        // Domino's head: one state element per workgroup, its drafters' block length
        if ((flags & DSW_FLAG_DOMINO) && grid < kRank) return DSW_ERR_PLAN;
        if ((flags & DSW_FLAG_DOMINO) && gamma > kDominoMaxGamma) return DSW_ERR_GAMMA;
    }
    bool valu = (flags & DSW_FLAG_VALU_GEMV) != 0;
    // one request: the MFMA engine's step is ~1 us shorter, but its shard load
    // ~3 us longer (measured at V = 151,936 in bf16), so walks of up to 3 steps
    // take the VALU engine; both widen int8 rows to bf16 once, at entry
    if (!forced) valu = B <= 1 && gamma <= 3 && !cell;
    int rc;
    if (batched) {
        rc = plan_batched(dev, V, B, flags, grid, i8, out);
    } else if (!forced && (!gumbel || gumbel_batched) && B >= kBatchedFrom) {
        rc = plan_batched(dev, V, B, flags, grid, i8, out);
        if (rc != DSW_OK) {
            memset(out, 0, sizeof(*out));
            rc = plan_mfma(dev, V, B, flags, grid, R, i8, out);
        }
    } else {
        rc = valu ? plan_valu(dev, B, flags, grid, R, i8, out) : plan_mfma(dev, V, B, flags, grid, R, i8, out);
    }
    if (rc != DSW_OK) {
        memset(out, 0, sizeof(*out));
        return rc;
    }
    out->w2_dtype = w2_dtype;
    const int row_bytes = i8 ? kRank : kRank * 2;
    const int Rs = out->rows_per_wg;  // the plan's shard size
    long long onchip = 0, streamed = 0;
    // every shard but the last is full; shards beyond V are empty
    for (int c = 0; c < grid; ++c) {
        long long n = (long long)V - (long long)c * Rs;
        if (n <= 0) break;
        if (n > Rs) n = Rs;
        // a short shard keeps its first rows in the same classes as the first shard
        long long on = out->reg_rows + out->lds_rows;
        if (out->engine == DSW_ENGINE_MFMA) {
            on = 0;
            const int TW = out->tiles_per_wave;
            for (int w = 0; w < 4; ++w)
                for (int j = 0; j < TW && j < out->reg_tiles + out->lds_tiles; ++j)
                    on += tile_rows((int)n, TW, w, j);
        } else if (on > n) {
            on = n;
        }
        onchip += on * row_bytes;
        streamed += (n - on) * row_bytes;
    }
    out->onchip_bytes = onchip;
    out->stream_bytes = streamed;
    out->workspace_bytes = (long long)workspace_layout().total;
    return DSW_OK;
}
