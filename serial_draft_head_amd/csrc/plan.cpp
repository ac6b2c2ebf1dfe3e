// plan.cpp -- residency planner: a pure host function of the device
// description and the walk's sizes (no HIP calls, so it can be exercised with
// invented devices on a machine without a GPU).
//
// Each workgroup (one per CU) owns ceil(V / grid) contiguous vocabulary rows,
// the slice-per-CTA split of "Keeping the Draft Walk on Chip", section "The
// idea: make the walk resident".  The slice is placed in VGPRs first (whole
// 256-row groups, one row per lane), then in LDS, and whatever is left is
// streamed from memory every step, as the pages' partially resident kernel
// does when the table does not fit (section "V = 248,320: 62% on chip, the
// rest streamed").
#include <string.h>

#include "../../include/dsw.h"
#include "walk_params.h"

namespace dsw {

// Largest number of VGPR row groups a compiled kernel holds without spilling
// to scratch, by batch tile (the GEMV keeps batch_tile x 4 accumulators, the
// weights take 128 registers per group).
static int reg_slot_cap(int batch_tile) {
    switch (batch_tile) {
        case 1: return 3;
        case 4: return 2;
        default: return 1;
    }
}

// Upper bound of the kernel's static LDS (u vectors, reduction scratch).
static int static_lds_bytes(int batch_tile) { return 1024 + 672 * batch_tile; }

static int batch_tile_for(int B) {
    if (B <= 1) return 1;
    if (B <= 4) return 4;
    return 16;
}


}  // namespace dsw

extern "C" int dsw_plan_compute(const dsw_devinfo* dev, int V, int r, int gamma, int B,
                                int w2_dtype, unsigned flags, dsw_plan_info* out) {
    using namespace dsw;
    if (!dev || !out) return DSW_ERR_NULL;
    memset(out, 0, sizeof(*out));
    if (r != kRank) return DSW_ERR_RANK;
    if (w2_dtype != DSW_BF16) return DSW_ERR_DTYPE;
    if (V < 1 || V > (1 << 20)) return DSW_ERR_VOCAB;  // row ids live in 20 key bits
    if (gamma < 0) return DSW_ERR_GAMMA;
    if (B < 0 || B > 16) return DSW_ERR_BATCH;
    if (dev->cu_count < 1 || dev->max_lds_per_block < 1) return DSW_ERR_DEVICE;

    const int grid = dev->cu_count < kMaxGrid ? dev->cu_count : kMaxGrid;
    const long long rows = ((long long)V + grid - 1) / grid;
    if (rows > (long long)kMaxSlots * kBlock) return DSW_ERR_VOCAB;
    const int R = (int)rows;
    const int row_bytes = kRank * 2;
    const int tile = batch_tile_for(B);
    const int slots = (R + kBlock - 1) / kBlock;

    int reg_slots = slots < reg_slot_cap(tile) ? slots : reg_slot_cap(tile);
    if (flags & DSW_FLAG_FORCE_STREAM) reg_slots = 0;
    const int reg_rows = R < reg_slots * kBlock ? R : reg_slots * kBlock;

    const int lds_static = static_lds_bytes(tile);
    int lds_avail = dev->max_lds_per_block - lds_static;
    if (lds_avail < 0) lds_avail = 0;
    int lds_rows = R - reg_rows;
    if (lds_rows > lds_avail / row_bytes) lds_rows = lds_avail / row_bytes;
    if (lds_rows > (kMaxSlots - reg_slots) * kBlock) lds_rows = (kMaxSlots - reg_slots) * kBlock;
    if (flags & DSW_FLAG_FORCE_STREAM) lds_rows = 0;
    if (lds_rows < 0) lds_rows = 0;
    const int stream_rows = R - reg_rows - lds_rows;

    // Dynamic LDS: the resident rows, but at least half of the CU's LDS so
    // that two workgroups can never share a CU.
    int lds_bytes = lds_rows * row_bytes;
    const int half = dev->lds_bytes_per_cu / 2 + 1024 - lds_static;
    if (lds_bytes < half) lds_bytes = half;
    if (lds_bytes + lds_static > dev->max_lds_per_block) lds_bytes = dev->max_lds_per_block - lds_static;
    if (lds_bytes < lds_rows * row_bytes) return DSW_ERR_PLAN;

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
    // bytes over the grid, counting only rows that exist (the last shards may be short)
    long long onchip = 0, streamed = 0;
    for (int c = 0; c < grid; ++c) {
        long long n = (long long)V - (long long)c * R;
        if (n <= 0) break;
        if (n > R) n = R;
        long long on = n < reg_rows + lds_rows ? n : reg_rows + lds_rows;
        onchip += on * row_bytes;
        streamed += (n - on) * row_bytes;
    }
    out->onchip_bytes = onchip;
    out->stream_bytes = streamed;
    out->workspace_bytes = (long long)workspace_layout().total;
    return DSW_OK;
}
