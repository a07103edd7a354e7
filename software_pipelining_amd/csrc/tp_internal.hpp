// Internal declarations shared by the host planner, the C ABI and the kernels.
// Nothing here is part of the public ABI (that is include/tilepipe.h).
#pragma once

#include <stdint.h>

#include "tilepipe.h"

#if defined(__HIPCC__)
#define TP_HD __host__ __device__
#else
#define TP_HD
#endif

namespace tp {

constexpr int kMaxStages = 8;
// Default run of the pipelined map (tiles_per_block == 0): 4 tiles of at most
// 2 KiB, else 2. Measured on MI355X (scale2 over 2^28 floats, 2 stages):
// tile 256 streams 1.0-1.6 % faster in runs of 4 (4 KiB) than of 2, tile 512
// 1.4 % faster in runs of 4 (8 KiB); tile 1024 is fastest in runs of 2
// (8 KiB) and runs of 4 lose 7 %. Runs of 3, 5 or 6 tiles lost 4-9 %.
constexpr int default_map_run(int tile_elems) { return tile_elems * 4 <= 2048 ? 4 : 2; }
constexpr int kDefaultMap2dBoxesPerBlock = 2;    // 2-D map, boxes_per_block == 0
constexpr int kMaxTilesPerBlock = 65536;
constexpr int kMaxRowShiftRows = 1024;
constexpr int kChunkTile = 256;            // chunks per tile of the chunk copy (one per lane)
constexpr int kChunkMetaArrays = 3;        // pred, src_size, ignore_src
constexpr int kMapEdgeLdsBytes = 256;      // LDS area of the floats outside the whole 16-byte chunks
// The 1-D map's tiled body starts at a boundary of this many bytes (the L2
// line) of out, or of in when out then sits on a half-line boundary. On
// MI355X a stream of 16-byte stores that splits lines ran up to a fifth
// slower (1-2 % when split at half lines), a stream of loads that does up to
// 4 % slower.
constexpr int kRealignBytes = 128;
constexpr int kVmcntMax = 63;              // vmcnt is a 6-bit counter on gfx9-family parts
constexpr int64_t kMaxMapElems = int64_t(1) << 40;
constexpr int64_t kMaxChunks = int64_t(1) << 36;
constexpr int64_t kMaxStride = int64_t(1) << 36;     // elements between rows of a 2-D window
constexpr int64_t kMaxRunBytes = int64_t(1) << 30;   // bytes one workgroup streams
constexpr int kLdsPerCu = 160 * 1024;      // gfx950: LDS of one CU, all of it usable by one workgroup
constexpr int kMaxWavesPerCu = 32;         // gfx950: 8 wave slots on each of 4 SIMDs
constexpr int kLdsReserveGranule = 1024;   // padding to bound residency is whole KiB
constexpr int kInflightTargetBytes = 27 * 1024;   // streaming map: tile traffic in flight per CU
constexpr int kMinResidentWaves = 8;       // ... but never fewer resident waves per CU
constexpr int kMinResidentWorkgroups = 4;  // ... nor fewer resident workgroups

// Memory instructions each lane issues per tile of a pipelined loop.
//   ld: loads per tile (LDS-DMA loads, plus metadata loads for the chunk copy)
//   st: stores per tile
// Wait count of the stage wait in iteration t of a loop with `stages` slots,
// before tile t is consumed. Every load is issued unconditionally (tiles
// outside a workgroup's range are out-of-range buffer loads that move no
// data), so the number of memory instructions issued after tile t's last load
// is fixed:
//   loads of tiles t+1 .. t+S-2                    -> (S-2) * ld
//   (refill-first order: the refill of tile t+S-1 is issued before the wait,
//    one more tile of loads                        -> (S-1) * ld)
//   stores of the iterations issued after tile t   -> min(t, S-1) * st
// Vector-memory operations of one wave retire in issue order on this
// architecture (loads and stores share the single vmcnt counter), so
// "at most that many outstanding" means tile t has landed in LDS. The count is
// clamped to the counter's width; a smaller count only waits longer.
TP_HD constexpr int stage_wait_count(int stages, int ld, int st, int t, bool refill_first = false)
{
    const int after_loads = (stages - 2 + (refill_first ? 1 : 0)) * ld;
    const int after_stores = (t < stages - 1 ? t : stages - 1) * st;
    const int k = after_loads + after_stores;
    return k > kVmcntMax ? kVmcntMax : (k < 0 ? 0 : k);
}

// ---------------------------------------------------------------- map
struct MapGeometry {
    int threads;      // workgroup size: min(256, tile_elems / 4)
    int lane_chunks;  // L: 16-byte chunks per lane per tile
};

TP_HD constexpr MapGeometry map_geometry(int tile_elems)
{
    const int threads = tile_elems / 4 < 256 ? tile_elems / 4 : 256;
    return MapGeometry{threads, tile_elems / (4 * threads)};
}

TP_HD constexpr int map_loads_per_tile(bool load_x4, int lane_chunks)
{
    return load_x4 ? lane_chunks : 4 * lane_chunks;
}

TP_HD constexpr int map_stores_per_tile(bool store_x4, int lane_chunks)
{
    return store_x4 ? lane_chunks : 4 * lane_chunks;
}

// Loads and stores of the same width give every lane back exactly the bytes it
// copied itself: the tile needs no exchange between waves.
TP_HD constexpr bool map_wave_local(bool load_x4, bool store_x4)
{
    return load_x4 == store_x4;
}

// The tiled body of a 1-D map starts at in/out; `head` floats just before it
// (when the output was realigned to 16 bytes) belong to the problem too.
struct MapParams {
    const float *in;         // first float of the body
    float *out;
    int64_t n_main;          // body elements in whole 16-byte chunks: n rounded down to a multiple of 4
    int64_t n;               // body elements; [n_main, n) is the final partial chunk
    int32_t tiles_per_block; // consecutive tiles per workgroup
    int32_t head;            // 0..31 floats at in[-head .. -1] / out[-head .. -1]
    float coef[32];          // Horner coefficients (used by TP_OP_HORNER32 only)
};

struct Map2dParams {
    const float *src;
    float *dst;
    int64_t src_stride;      // elements between rows
    int64_t dst_stride;
    int64_t rows;
    int64_t cols;
    int32_t box_cols_log2;   // box_cols = 1 << box_cols_log2; box_rows follows from the tile size
    int32_t tiles_per_block; // boxes per workgroup, side by side in one band of box_rows rows
    int32_t runs_per_band;   // workgroups per band
    int32_t pad;
    float coef[32];          // Horner coefficients (used by TP_OP_HORNER32 only)
};

// ---------------------------------------------------------- chunk copy
// Memory instructions per lane and tile of the chunk copy, for chunks of
// `width` = 4, 8 or 16 bytes: three metadata bytes, then the chunk as one
// 16-byte load when that is aligned, else as width / 4 words.
TP_HD constexpr int chunk_loads_per_tile(bool load_x4, int width = 16)
{
    return kChunkMetaArrays + (width == 16 && load_x4 ? 1 : width / 4);
}

TP_HD constexpr int chunk_stores_per_tile(bool store_x4, int width = 16)
{
    return width == 16 && store_x4 ? 1 : width / 4;
}

TP_HD constexpr int chunk_meta_slots(int stages)
{
    return stages == 1 ? 1 : 2 * stages - 1;
}

TP_HD constexpr int chunk_data_slot_bytes(int width = 16) { return kChunkTile * width; }
constexpr int kChunkDataSlotBytes = kChunkTile * 16;                    // 4 KiB (16-byte chunks)
constexpr int kChunkMetaSlotBytes = kChunkMetaArrays * kChunkTile * 4;  // 3 KiB (4 bytes per lane)

TP_HD constexpr int chunk_lds_bytes(int stages, int width = 16)
{
    return stages * chunk_data_slot_bytes(width) + chunk_meta_slots(stages) * kChunkMetaSlotBytes;
}

enum ChunkFlags : int32_t {
    kHasPred = 1,
    kHasSize = 2,
    kHasIgnore = 4,
};

struct ChunkParams {
    const uint8_t *src;
    uint8_t *dst;
    const uint8_t *pred;
    const uint8_t *src_size;
    const uint8_t *ignore_src;
    int64_t n_chunks;
    int32_t tiles_per_block;
    int32_t flags;           // ChunkFlags
};

// Kernel arguments of a planned chunk copy (an absent metadata array is a
// null pointer and a cleared flag).
inline ChunkParams chunk_params(const tp_plan &plan, const void *src, void *dst, int64_t n_chunks,
                                const uint8_t *pred, const uint8_t *src_size,
                                const uint8_t *ignore_src)
{
    ChunkParams p{};
    p.src = static_cast<const uint8_t *>(src);
    p.dst = static_cast<uint8_t *>(dst);
    p.pred = pred;
    p.src_size = src_size;
    p.ignore_src = ignore_src;
    p.n_chunks = n_chunks;
    p.tiles_per_block = plan.tiles_per_block;
    p.flags = (pred ? kHasPred : 0) | (src_size ? kHasSize : 0) | (ignore_src ? kHasIgnore : 0);
    return p;
}

// ------------------------------------------------ copies between workgroups
constexpr int kWgChunkBytes = 256;             // the chunk one workgroup hands on
constexpr int kWgSlotBytes = 2 * kWgChunkBytes;   // its staging slot: 64 tagged 8-byte words
constexpr uint32_t kWgTag = 1u;                // the tag of a word a sender has stored
constexpr int64_t kWgMaxChunks = int64_t(1) << 26;
constexpr uint32_t kWgDefaultSpinLimit = 1u << 16;   // polls of a slot before giving up
constexpr uint32_t kWgMaxSpinLimit = 1u << 24;
constexpr uint32_t kWgStatusPollEvery = 8;     // a waiting receiver reads the status every 8th poll
constexpr int64_t kWgClearThreads = 256;       // lanes of a workgroup of the clearing kernel
constexpr int64_t kWgClearSlotsPerPass = 8;    // slots (4 KiB) a clearing workgroup zeroes per pass
constexpr int64_t kWgClearMaxGroups = 65536;   // the clearing kernel's grid at most (they loop)

// Workspace of a copy between n workgroups: n staging slots of 512 bytes.
// Slot k holds chunk k as 64 words {data, tag} of 8 bytes each, lane l's at
// byte 8 l; the clearing kernel zeroes every slot, and a word is the sender's
// once its tag reads kWgTag.
TP_HD constexpr int64_t wg_workspace_bytes(int64_t n) { return n <= 0 ? 0 : kWgSlotBytes * n; }

// Grid of the clearing kernel for n chunks.
TP_HD constexpr int64_t wg_clear_groups(int64_t n)
{
    return (n + kWgClearSlotsPerPass - 1) / kWgClearSlotsPerPass < kWgClearMaxGroups
               ? (n + kWgClearSlotsPerPass - 1) / kWgClearSlotsPerPass
               : kWgClearMaxGroups;
}

// The allocation-free variant keeps its workspace in a static device array
// sized for this many chunks.
constexpr int64_t kWgNoAllocMaxChunks = 16384;
constexpr int64_t kWgNoAllocScratchBytes = wg_workspace_bytes(kWgNoAllocMaxChunks);

struct WgCopyParams {
    const uint8_t *src;
    uint8_t *dst;
    uint8_t *stage;          // n staging slots of kWgSlotBytes
    int32_t *status;         // 0, or 1 once a receiver gave up waiting
    int64_t n_chunks;
    uint32_t spin_limit;     // polls of a slot before a receiver gives up
    uint32_t pad;
};

// -------------------------------------------------------------- row shift
struct RowShiftParams {
    const float *a;
    float *b;
    int32_t rows;
    int32_t pad;
};

// ---------------------------------------------------------- host planner
// Pure host code (no HIP): argument validation and launch geometry.
int plan_row_shift(uintptr_t a, uintptr_t b, int64_t rows, int64_t lds_budget, tp_plan *plan);
int plan_map(uintptr_t in, uintptr_t out, int64_t n, int op, int tile_elems, int stages,
             int tiles_per_block, int resident_cap, int schedule, int align,
             int64_t lds_budget, tp_plan *plan);
// The library's residency bound for a map launch (0: none); see tp_pipelined_map_ex.
int map_policy_resident_cap(int op, int tile_elems, int stages, int tiles_per_block, int waves);
// Box of a 2-D map when the caller passes 0 x 0: 1024 floats, as wide as the
// window allows (box_cols the smallest power of two >= min(cols, 1024), at
// least 4). Leaves the arguments alone otherwise.
void map2d_resolve_box(int64_t cols, int *box_rows, int *box_cols);
int plan_map_2d(uintptr_t src, int64_t src_stride, uintptr_t dst, int64_t dst_stride,
                int64_t rows, int64_t cols, int op, int box_rows, int box_cols, int stages,
                int tiles_per_block, int align, int64_t lds_budget, tp_plan *plan);
int plan_chunk_copy(uintptr_t src, uintptr_t dst, int64_t n_chunks, int chunk_bytes,
                    uintptr_t pred, uintptr_t src_size, uintptr_t ignore_src, int stages,
                    int tiles_per_block, int64_t lds_budget, tp_plan *plan);

// Validates a copy between workgroups (the workspace is caller memory of
// workspace_bytes; spin_limit 0 means the default) and plans its main kernel:
// n_chunks one-wave workgroups with 512 bytes of LDS.
int plan_workgroup_copy(uintptr_t src, uintptr_t dst, int64_t n_chunks, uintptr_t workspace,
                        int64_t workspace_bytes, uintptr_t status, int64_t spin_limit,
                        tp_plan *plan);

// TP_OK for a device whose architecture name is gfx950 (optionally followed by
// ":feature..." suffixes), TP_ERR_UNSUPPORTED_DEVICE for any other name.
int arch_status(const char *arch);

// Horner coefficients c_k = RN(1/(k+1)), k = 0..31.
void horner32_coefficients(float c[32]);

// Kernel arguments of a planned launch, as the C ABI builds them.
MapParams map_params(const tp_plan &plan, const float *in, float *out, int64_t n);
Map2dParams map2d_params(const tp_plan &plan, const float *src, int64_t src_stride, float *dst,
                         int64_t dst_stride, int64_t rows, int64_t cols, int box_rows, int box_cols);

// ------------------------------------------------------- kernel launchers
// Each returns a hipError_t value (0 = success). `stream` is a hipStream_t.
int launch_row_shift(const tp_plan &plan, const RowShiftParams &p, void *stream);
// One entry per kernel family, op and half of the stage range (S 1-4, 5-8),
// each defined by its own compilation of tp_*_inst.hip.
int launch_map_scale2_s1_4(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_scale2_s5_8(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_horner32_s1_4(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_horner32_s5_8(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_copy_s1_4(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_copy_s5_8(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_split_scale2_s1_4(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_split_scale2_s5_8(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_split_horner32_s1_4(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_split_horner32_s5_8(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_split_copy_s1_4(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map_split_copy_s5_8(const tp_plan &plan, const MapParams &p, void *stream);
int launch_map2d_scale2_s1_4(const tp_plan &plan, const Map2dParams &p, void *stream);
int launch_map2d_scale2_s5_8(const tp_plan &plan, const Map2dParams &p, void *stream);
int launch_map2d_horner32_s1_4(const tp_plan &plan, const Map2dParams &p, void *stream);
int launch_map2d_horner32_s5_8(const tp_plan &plan, const Map2dParams &p, void *stream);
int launch_map2d_copy_s1_4(const tp_plan &plan, const Map2dParams &p, void *stream);
int launch_map2d_copy_s5_8(const tp_plan &plan, const Map2dParams &p, void *stream);
int launch_chunk_copy(const tp_plan &plan, const ChunkParams &p, void *stream);
// The clearing kernel (staging slots and status to zero), then, for two
// chunks or more, the hand-off kernel.
int launch_workgroup_copy(const tp_plan &plan, const WgCopyParams &p, void *stream);
// Device address of the current device's static workspace for the
// allocation-free variant (looked up once per device); a hipError_t value.
int workgroup_copy_scratch(void **ptr);

}  // namespace tp
