// Host-side argument validation and launch planning. Pure C++: no HIP calls,
// so every rule here can be exercised on a machine without a GPU.
#include <string.h>

#include "tp_internal.hpp"

namespace tp {
namespace {

bool overlaps(uintptr_t a, uint64_t a_bytes, uintptr_t b, uint64_t b_bytes)
{
    if (a_bytes == 0 || b_bytes == 0)
        return false;
    return a < b + b_bytes && b < a + a_bytes;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int path_bits(uintptr_t load_ptr, uintptr_t store_ptr)
{
    return ((load_ptr % 16) ? TP_PATH_SCALAR_LOAD : 0) | ((store_ptr % 16) ? TP_PATH_SCALAR_STORE : 0);
}

bool valid_tile(int tile_elems)
{
    switch (tile_elems) {
    case 256: case 512: case 1024: case 2048: case 4096: case 8192:
        return true;
    default:
        return false;
    }
}

int resolve_tiles_per_block(int tiles_per_block, int default_value)
{
    if (tiles_per_block == 0)
        return default_value;
    if (tiles_per_block < 0 || tiles_per_block > kMaxTilesPerBlock)
        return -1;
    return tiles_per_block;
}

// Mean number of a run's tiles loading at a wave's stage waits: at the wait
// of iteration t, tiles t .. min(t+S-1, T-1) are in flight (refill-first
// order; loads past the run's end move nothing).
double mean_tiles_in_flight(int64_t T, int64_t S)
{
    const int64_t sum = T <= S ? T * (T + 1) / 2 : S * (S + 1) / 2 + (T - S) * S;
    return (double)sum / (double)T;
}

// LDS a workgroup reserves so that at most `cap` workgroups fit on a CU.
int32_t reserve_for_cap(int32_t ring_bytes, int cap, int64_t lds_budget)
{
    int64_t pad = (int64_t)kLdsPerCu / cap / kLdsReserveGranule * kLdsReserveGranule;
    if (pad > lds_budget)
        pad = lds_budget;
    return pad > ring_bytes ? (int32_t)pad : ring_bytes;
}

}  // namespace

int map_policy_resident_cap(int op, int tile_elems, int stages, int tiles_per_block, int waves)
{
    // A wave of the streaming ops is almost always waiting on memory, so the
    // resident workgroups decide how much traffic is in flight; past roughly
    // 27 KiB per CU (with headroom for the start and end of short runs) the
    // extra requests only queue, and HBM efficiency drops. horner32 spends
    // most of a wave's time in FMAs and needs every wave to hide it; a run of
    // one tile has no pipeline and lives too briefly to be bounded; and where
    // a lane moves several 16-byte chunks per tile (tiles of 2048 floats and
    // more) its wave already keeps several loads in flight, and bounding the
    // workgroups was measured to cost bandwidth instead.
    const MapGeometry g = map_geometry(tile_elems);
    if (op == TP_OP_HORNER32 || tiles_per_block <= 1 || g.lane_chunks > 1)
        return 0;
    const double moving = mean_tiles_in_flight(tiles_per_block, stages) + 1.0;   // loads + stores
    const double target = kInflightTargetBytes * (1.0 + 1.0 / tiles_per_block);
    int cap = (int)(target / (moving * tile_elems * 4.0) + 0.5);
    int floor_wgs = (kMinResidentWaves + waves - 1) / waves;
    if (floor_wgs < kMinResidentWorkgroups)
        floor_wgs = kMinResidentWorkgroups;
    if (cap < floor_wgs)
        cap = floor_wgs;
    return cap >= kMaxWavesPerCu / waves ? 0 : cap;
}

int plan_row_shift(uintptr_t a, uintptr_t b, int64_t rows, int64_t lds_budget, tp_plan *plan)
{
    if (rows < 0 || rows > kMaxRowShiftRows)
        return TP_ERR_INVALID_ARG;
    tp_plan p;
    memset(&p, 0, sizeof p);
    p.stages = 1;
    p.tile_units = (int32_t)rows;
    p.lane_chunks = 1;
    p.tiles_per_block = 1;
    if (rows > 0) {
        if (!a || !b)
            return TP_ERR_INVALID_ARG;
        if (a % 4 || b % 4)
            return TP_ERR_MISALIGNED;
        const uint64_t bytes = (uint64_t)rows * 16;
        if (a != b && overlaps(a, bytes, b, bytes))
            return TP_ERR_OVERLAP;
        p.threads = (int32_t)(ceil_div(rows, 64) * 64);
        p.lds_bytes = p.threads * 16;
        p.ring_bytes = p.lds_bytes;
        if (p.lds_bytes > lds_budget)
            return TP_ERR_LDS_BUDGET;
        p.path = path_bits(a, b);
        p.num_tiles = 1;
        p.grid = 1;
    }
    if (plan)
        *plan = p;
    return TP_OK;
}

int plan_map(uintptr_t in, uintptr_t out, int64_t n, int op, int tile_elems, int stages,
             int tiles_per_block, int resident_cap, int schedule, int align,
             int64_t lds_budget, tp_plan *plan)
{
    if (resident_cap < -1 || (schedule != TP_SCHED_UNIFORM && schedule != TP_SCHED_ROLE_SPLIT))
        return TP_ERR_INVALID_ARG;
    if (align != TP_ALIGN_REALIGN && align != TP_ALIGN_WORDS)
        return TP_ERR_INVALID_ARG;
    if (n < 0 || n > kMaxMapElems)
        return TP_ERR_INVALID_ARG;
    if (op != TP_OP_SCALE2 && op != TP_OP_HORNER32 && op != TP_OP_COPY)
        return TP_ERR_INVALID_ARG;
    if (!valid_tile(tile_elems) || stages < 1 || stages > kMaxStages)
        return TP_ERR_INVALID_ARG;
    const int tpb = resolve_tiles_per_block(tiles_per_block, default_map_run(tile_elems));
    if (tpb < 0)
        return TP_ERR_INVALID_ARG;
    // a workgroup's run (plus S-1 tiles of out-of-range prefetch) must stay
    // well inside 32-bit buffer offsets
    if ((int64_t)tpb * tile_elems * 4 > kMaxRunBytes)
        return TP_ERR_INVALID_ARG;
    const MapGeometry g = map_geometry(tile_elems);
    tp_plan p;
    memset(&p, 0, sizeof p);
    p.stages = stages;
    p.tile_units = tile_elems;
    // the role split adds one wave that only loads
    p.threads = g.threads + (schedule == TP_SCHED_ROLE_SPLIT ? 64 : 0);
    p.lane_chunks = g.lane_chunks;
    p.schedule = schedule;
    p.align = align;
    p.tiles_per_block = tpb;
    p.ring_bytes = stages * tile_elems * 4 + kMapEdgeLdsBytes;
    if (n > 0) {
        if (!in || !out)
            return TP_ERR_INVALID_ARG;
        if (in % 4 || out % 4)
            return TP_ERR_MISALIGNED;
        const uint64_t bytes = (uint64_t)n * 4;
        if (in != out && overlaps(in, bytes, out, bytes))
            return TP_ERR_OVERLAP;
    }
    if (p.ring_bytes > lds_budget)
        return TP_ERR_LDS_BUDGET;
    p.path = TP_PATH_X4;
    if (n > 0 && align == TP_ALIGN_WORDS) {
        p.path = path_bits(in, out);
    } else if (n > 0) {
        // 16-byte loads at any 4-byte alignment. The body starts at out's first
        // line boundary, so its stores fill whole lines; or at in's, when that
        // puts out on a half-line boundary: a store stream split at half lines
        // cost less than a load stream split inside lines
        const uintptr_t skew = (out - in) % kRealignBytes;
        const uintptr_t anchor = skew == kRealignBytes / 2 ? in : out;
        const int64_t to_boundary =
            (int64_t)((kRealignBytes - anchor % kRealignBytes) % kRealignBytes / 4);
        p.head = (int32_t)(to_boundary < n ? to_boundary : n);
    }
    const int waves = p.threads / 64;
    const int cap = resident_cap == 0 ? map_policy_resident_cap(op, tile_elems, stages, tpb, waves)
                                      : resident_cap;
    p.resident_cap = cap >= kMaxWavesPerCu / waves ? 0 : (cap < 0 ? 0 : cap);
    p.lds_bytes = p.resident_cap ? reserve_for_cap(p.ring_bytes, p.resident_cap, lds_budget)
                                 : p.ring_bytes;
    const bool load_x4 = !(p.path & TP_PATH_SCALAR_LOAD);
    const bool store_x4 = !(p.path & TP_PATH_SCALAR_STORE);
    if (schedule == TP_SCHED_ROLE_SPLIT) {
        // the loading wave covers the whole tile and issues no stores
        const int ld = map_loads_per_tile(load_x4, g.lane_chunks) * (g.threads / 64);
        p.wait_steady = stages == 1 ? 0 : stage_wait_count(stages, ld, 0, 0);
    } else {
        p.wait_steady = stage_wait_count(stages, map_loads_per_tile(load_x4, g.lane_chunks),
                                         map_stores_per_tile(store_x4, g.lane_chunks), stages,
                                         map_wave_local(load_x4, store_x4));
    }
    const int64_t n_main = (n - p.head) & ~int64_t(3);   // the body's whole 16-byte chunks
    p.num_tiles = ceil_div(n_main, tile_elems);
    p.grid = n == 0 ? 0 : (p.num_tiles == 0 ? 1 : ceil_div(p.num_tiles, tpb));
    if (p.grid > INT32_MAX)        // more workgroups than one launch can name
        return TP_ERR_INVALID_ARG;
    if (plan)
        *plan = p;
    return TP_OK;
}

void map2d_resolve_box(int64_t cols, int *box_rows, int *box_cols)
{
    if (*box_rows != 0 || *box_cols != 0)
        return;
    int bc = 4;
    while (bc < 1024 && bc < cols)
        bc *= 2;
    *box_cols = bc;
    *box_rows = 1024 / bc;
}

int plan_map_2d(uintptr_t src, int64_t src_stride, uintptr_t dst, int64_t dst_stride,
                int64_t rows, int64_t cols, int op, int box_rows, int box_cols, int stages,
                int tiles_per_block, int align, int64_t lds_budget, tp_plan *plan)
{
    if (align != TP_ALIGN_REALIGN && align != TP_ALIGN_WORDS)
        return TP_ERR_INVALID_ARG;
    map2d_resolve_box(cols, &box_rows, &box_cols);
    if (rows < 0 || cols < 0 || rows > kMaxMapElems || cols > kMaxMapElems)
        return TP_ERR_INVALID_ARG;
    if (op != TP_OP_SCALE2 && op != TP_OP_HORNER32 && op != TP_OP_COPY)
        return TP_ERR_INVALID_ARG;
    if (stages < 1 || stages > kMaxStages)
        return TP_ERR_INVALID_ARG;
    const int64_t tile = (int64_t)box_rows * box_cols;
    if (box_rows < 1 || box_cols < 4 || (box_rows & (box_rows - 1)) || (box_cols & (box_cols - 1)) ||
        !valid_tile((int)(tile > 8192 ? 0 : tile)))
        return TP_ERR_INVALID_ARG;
    const int tpb = resolve_tiles_per_block(tiles_per_block, kDefaultMap2dBoxesPerBlock);
    if (tpb < 0)
        return TP_ERR_INVALID_ARG;
    const MapGeometry g = map_geometry((int)tile);
    tp_plan p;
    memset(&p, 0, sizeof p);
    p.stages = stages;
    p.tile_units = (int32_t)tile;
    p.threads = g.threads;
    p.lane_chunks = g.lane_chunks;
    p.tiles_per_block = tpb;
    p.ring_bytes = (int32_t)(stages * tile * 4);
    p.schedule = TP_SCHED_UNIFORM;
    p.align = align;
    if (p.ring_bytes > lds_budget)
        return TP_ERR_LDS_BUDGET;
    p.lds_bytes = p.ring_bytes;
    p.path = TP_PATH_X4;
    if (rows > 0 && cols > 0) {
        if (!src || !dst)
            return TP_ERR_INVALID_ARG;
        if (src % 4 || dst % 4)
            return TP_ERR_MISALIGNED;
        if (src_stride < cols || dst_stride < cols || src_stride > kMaxStride ||
            dst_stride > kMaxStride)
            return TP_ERR_INVALID_ARG;
        // one workgroup's band, up to its run's last column, stays well inside
        // 32-bit buffer offsets on both sides
        const int64_t run_cols = (int64_t)tpb * box_cols;
        if (((box_rows - 1) * src_stride + run_cols) * 4 > kMaxRunBytes ||
            ((box_rows - 1) * dst_stride + run_cols) * 4 > kMaxRunBytes)
            return TP_ERR_INVALID_ARG;
        const uint64_t src_bytes = (uint64_t)((rows - 1) * src_stride + cols) * 4;
        const uint64_t dst_bytes = (uint64_t)((rows - 1) * dst_stride + cols) * 4;
        if (!(src == dst && src_stride == dst_stride) && overlaps(src, src_bytes, dst, dst_bytes))
            return TP_ERR_OVERLAP;
        const int64_t bands = ceil_div(rows, box_rows);
        const int64_t boxes_per_band = ceil_div(cols, box_cols);
        const int64_t runs = ceil_div(boxes_per_band, tpb);
        if (bands * runs > INT32_MAX)
            return TP_ERR_INVALID_ARG;
        p.num_tiles = bands * boxes_per_band;
        p.grid = bands * runs;
        // a 16-byte chunk is 4 floats of one row: cols % 4 == 0 keeps every chunk
        // inside its row; the pages' rule also wants it 16-byte aligned
        const bool words = align == TP_ALIGN_WORDS;
        const bool load_x4 = cols % 4 == 0 && (!words || (src % 16 == 0 && src_stride % 4 == 0));
        const bool store_x4 = cols % 4 == 0 && (!words || (dst % 16 == 0 && dst_stride % 4 == 0));
        p.path = (load_x4 ? 0 : TP_PATH_SCALAR_LOAD) | (store_x4 ? 0 : TP_PATH_SCALAR_STORE);
    }
    const bool load_x4 = !(p.path & TP_PATH_SCALAR_LOAD);
    const bool store_x4 = !(p.path & TP_PATH_SCALAR_STORE);
    p.wait_steady = stage_wait_count(stages, map_loads_per_tile(load_x4, g.lane_chunks),
                                     map_stores_per_tile(store_x4, g.lane_chunks), stages,
                                     map_wave_local(load_x4, store_x4));
    const int cap = map_policy_resident_cap(op, (int)tile, stages, tpb, g.threads / 64);
    p.resident_cap = cap;
    if (cap)
        p.lds_bytes = reserve_for_cap(p.ring_bytes, cap, lds_budget);
    if (plan)
        *plan = p;
    return TP_OK;
}

int plan_chunk_copy(uintptr_t src, uintptr_t dst, int64_t n_chunks, int chunk_bytes,
                    uintptr_t pred, uintptr_t src_size, uintptr_t ignore_src, int stages,
                    int tiles_per_block, int64_t lds_budget, tp_plan *plan)
{
    if (n_chunks < 0 || n_chunks > kMaxChunks)
        return TP_ERR_INVALID_ARG;
    if (chunk_bytes != 4 && chunk_bytes != 8 && chunk_bytes != 16)
        return TP_ERR_INVALID_ARG;
    if (stages < 1 || stages > kMaxStages)
        return TP_ERR_INVALID_ARG;
    // The default run is max(S-1, m) tiles. With S-1 tiles the prologue puts
    // the whole run in flight: every metadata load, then every data load,
    // then the stores. For 16-byte chunks under the masked writes that a false
    // pred leaves this measured fastest on MI355X at every stage count (runs
    // of 64 tiles ran about 1.45x slower). Narrower chunks make smaller tiles
    // (2 and 1 KiB) whose per-workgroup metadata round trip needs longer runs
    // to amortize: m = 1, 2 and 8 tiles for 16-, 8- and 4-byte chunks
    // (measured best, or within a few percent of it, at 1-6 stages).
    const int min_run = chunk_bytes == 16 ? 1 : chunk_bytes == 8 ? 2 : 8;
    const int tpb = resolve_tiles_per_block(tiles_per_block,
                                            stages - 1 > min_run ? stages - 1 : min_run);
    if (tpb < 0)
        return TP_ERR_INVALID_ARG;
    if ((int64_t)tpb * chunk_data_slot_bytes(chunk_bytes) > kMaxRunBytes)
        return TP_ERR_INVALID_ARG;
    // A ring deeper than the run plus one slot holds nothing more (the
    // prologue already issues the whole run), and a run of one tile moves with
    // the same instructions on the one-stage schedule: the ring is cut to what
    // the run can use, which only frees LDS.
    if (tpb == 1)
        stages = 1;
    else if (stages > tpb + 1)
        stages = tpb + 1;
    tp_plan p;
    memset(&p, 0, sizeof p);
    p.stages = stages;
    p.tile_units = kChunkTile;
    p.threads = kChunkTile;
    p.lane_chunks = 1;
    p.tiles_per_block = tpb;
    p.chunk_bytes = chunk_bytes;
    p.lds_bytes = chunk_lds_bytes(stages, chunk_bytes);
    p.ring_bytes = p.lds_bytes;
    if (n_chunks > 0) {
        if (!src || !dst)
            return TP_ERR_INVALID_ARG;
        if (src % 4 || dst % 4)
            return TP_ERR_MISALIGNED;
        const uint64_t bytes = (uint64_t)n_chunks * chunk_bytes;
        if (src != dst && overlaps(src, bytes, dst, bytes))
            return TP_ERR_OVERLAP;
        const uintptr_t meta[3] = {pred, src_size, ignore_src};
        for (uintptr_t m : meta)
            if (m && overlaps(dst, bytes, m, (uint64_t)n_chunks))
                return TP_ERR_OVERLAP;
    }
    if (p.lds_bytes > lds_budget)
        return TP_ERR_LDS_BUDGET;
    // 16-byte chunks move as one 16-byte access per side when that side is
    // aligned; narrower chunks always move as words
    if (chunk_bytes == 16)
        p.path = n_chunks > 0 ? path_bits(src, dst) : TP_PATH_X4;
    else
        p.path = TP_PATH_SCALAR;
    const bool load_x4 = !(p.path & TP_PATH_SCALAR_LOAD);
    const bool store_x4 = !(p.path & TP_PATH_SCALAR_STORE);
    p.wait_steady = stage_wait_count(stages, chunk_loads_per_tile(load_x4, chunk_bytes),
                                     chunk_stores_per_tile(store_x4, chunk_bytes), stages);
    p.num_tiles = ceil_div(n_chunks, kChunkTile);
    p.grid = ceil_div(p.num_tiles, tpb);
    if (p.grid > INT32_MAX)
        return TP_ERR_INVALID_ARG;
    if (plan)
        *plan = p;
    return TP_OK;
}

int plan_workgroup_copy(uintptr_t src, uintptr_t dst, int64_t n_chunks, uintptr_t workspace,
                        int64_t workspace_bytes, uintptr_t status, int64_t spin_limit,
                        tp_plan *plan)
{
    if (n_chunks < 0 || n_chunks > kWgMaxChunks)
        return TP_ERR_INVALID_ARG;
    if (spin_limit < 0 || spin_limit > (int64_t)kWgMaxSpinLimit)
        return TP_ERR_INVALID_ARG;
    tp_plan p;
    memset(&p, 0, sizeof p);
    p.stages = 1;
    p.tile_units = kWgChunkBytes;
    p.threads = 64;
    p.lane_chunks = 1;
    p.tiles_per_block = 1;
    p.lds_bytes = 2 * kWgChunkBytes;   // the own chunk and the received one
    p.ring_bytes = p.lds_bytes;
    p.path = TP_PATH_SCALAR;
    if (n_chunks > 0) {
        const int64_t need = wg_workspace_bytes(n_chunks);
        if (!src || !dst || !workspace || !status || workspace_bytes < need)
            return TP_ERR_INVALID_ARG;
        // the tagged words are 8-byte accesses, which land whole only when aligned
        if (src % 4 || dst % 4 || workspace % 8 || status % 4)
            return TP_ERR_MISALIGNED;
        const uint64_t bytes = (uint64_t)n_chunks * kWgChunkBytes;
        if (src != dst && overlaps(src, bytes, dst, bytes))
            return TP_ERR_OVERLAP;
        const uintptr_t data[2] = {src, dst};
        for (uintptr_t a : data)
            if (overlaps(a, bytes, workspace, (uint64_t)need) || overlaps(a, bytes, status, 4))
                return TP_ERR_OVERLAP;
        if (overlaps(workspace, (uint64_t)need, status, 4))
            return TP_ERR_OVERLAP;
        p.num_tiles = n_chunks;
        p.grid = n_chunks;
    }
    if (plan)
        *plan = p;
    return TP_OK;
}

void horner32_coefficients(float c[32])
{
    for (int k = 0; k < 32; ++k)
        c[k] = 1.0f / (float)(k + 1);
}

int arch_status(const char *arch)
{
    return arch && strncmp(arch, "gfx950", 6) == 0 && (arch[6] == '\0' || arch[6] == ':')
               ? TP_OK
               : TP_ERR_UNSUPPORTED_DEVICE;
}

MapParams map_params(const tp_plan &plan, const float *in, float *out, int64_t n)
{
    MapParams p;
    memset(&p, 0, sizeof p);
    p.in = in + plan.head;        // the tiled body
    p.out = out + plan.head;
    p.n = n - plan.head;
    p.n_main = p.n & ~int64_t(3);
    p.head = plan.head;
    p.tiles_per_block = plan.tiles_per_block;
    horner32_coefficients(p.coef);
    return p;
}

Map2dParams map2d_params(const tp_plan &plan, const float *src, int64_t src_stride, float *dst,
                         int64_t dst_stride, int64_t rows, int64_t cols, int box_rows, int box_cols)
{
    Map2dParams p;
    memset(&p, 0, sizeof p);
    p.src = src;
    p.dst = dst;
    p.src_stride = src_stride;
    p.dst_stride = dst_stride;
    p.rows = rows;
    p.cols = cols;
    map2d_resolve_box(cols, &box_rows, &box_cols);
    int lg = 0;
    while ((1 << lg) < box_cols)
        ++lg;
    p.box_cols_log2 = lg;
    p.tiles_per_block = plan.tiles_per_block;
    p.runs_per_band = (int32_t)((((cols + box_cols - 1) / box_cols) + plan.tiles_per_block - 1) /
                                plan.tiles_per_block);
    horner32_coefficients(p.coef);
    return p;
}

}  // namespace tp
