/*
 * libtilepipe: software-pipelined global->LDS tile streaming on MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only; HIP types are hidden behind void* so a
 * caller needs no HIP headers. Every compute entry point is stream-ordered: it
 * validates its arguments on the host, enqueues one kernel on `stream` and
 * returns without synchronizing (the pages' copy interface likewise returns at
 * once and completion is observed later: "Asynchronous Data Movement",
 * section "cuda::memcpy_async"). Completion and any device fault are observed
 * through the stream (hipStreamSynchronize, an event, or a later blocking
 * call), as for any other stream operation.
 *
 * Conventions shared by all entry points
 *  - Ownership: the caller owns every buffer (device memory from hipMalloc,
 *    torch, or any allocator). The library never allocates, frees, or
 *    synchronizes, and keeps no state other than a per-device cache of device
 *    properties, so calls from several host threads are safe.
 *  - Errors: argument errors are found on the host before anything is
 *    enqueued; the call then returns a nonzero tp_status and enqueues nothing.
 *    A failed launch returns TP_ERR_HIP; tp_last_hip_error() then gives the
 *    hipError_t value (per calling thread). A device that is not gfx950 gives
 *    TP_ERR_UNSUPPORTED_DEVICE. An empty problem (n == 0) returns TP_OK and
 *    launches nothing.
 *  - Alignment: float and chunk buffers must be 4-byte aligned
 *    (TP_ERR_MISALIGNED otherwise). A buffer that is 4- but not 16-byte
 *    aligned is not an error. The pages send such a copy down a slower
 *    element-wise path ("Asynchronous Data Movement", section "Alignment
 *    requirements"). The maps do not need to by default (TP_ALIGN_REALIGN):
 *    gfx950 serves 16-byte global accesses at any 4-byte alignment, and the
 *    1-D map moves the floats before out's first 128-byte boundary (at most
 *    31) element-wise, so that its 16-byte stores fill whole 128-byte lines
 *    (on MI355X a store stream that splits lines ran up to a fifth slower,
 *    even 16-byte aligned). When out - in is 64 modulo 128 it starts at in's
 *    first 128-byte boundary instead, which leaves the stores split at half
 *    lines, the cheaper of the two splits. With TP_ALIGN_WORDS
 *    the maps follow the pages' rule, and the row exchange and the chunk copy
 *    always do: a side whose pointer is not 16-byte aligned moves 4-byte
 *    words. The choice is reported through path_out (the pages' fallback is
 *    silent; here it is observable). Results never depend on the path.
 *  - Aliasing: an output may be exactly the same buffer as the input (every
 *    unit is read into LDS before it is written). Any partial overlap between
 *    an output and another argument is TP_ERR_OVERLAP.
 *  - `stream` is a hipStream_t (NULL = the null stream of the current device).
 *    Kernels run on the device that is current on the calling thread.
 *  - path_out (may be NULL) receives a tp_path value for the launch made.
 */
#ifndef TILEPIPE_H
#define TILEPIPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TP_API __attribute__((visibility("default")))

#define TP_VERSION 1

typedef enum tp_status {
    TP_OK = 0,
    TP_ERR_INVALID_ARG = 1,        /* null pointer, negative size, value out of range */
    TP_ERR_MISALIGNED = 2,         /* a float/chunk buffer not 4-byte aligned */
    TP_ERR_LDS_BUDGET = 3,         /* stages x tile bytes exceeds the device's LDS per workgroup */
    TP_ERR_OVERLAP = 4,            /* output partially overlaps another argument */
    TP_ERR_UNSUPPORTED_DEVICE = 5, /* current device is not gfx950 */
    TP_ERR_HIP = 6                 /* a HIP runtime call or launch failed */
} tp_status;

typedef enum tp_op {
    TP_OP_SCALE2 = 0,   /* y = 2 * x */
    TP_OP_HORNER32 = 1, /* y = 0; for k = 0..31: y = fma(y, x, c_k), c_k = RN(1/(k+1)) */
    TP_OP_COPY = 2      /* y = x (copy-bandwidth ceiling) */
} tp_op;

/* Which side of the copy uses 16-byte accesses: bit 0 set = loads use the
 * 4-byte fallback (source not 16-byte aligned), bit 1 set = stores do. */
typedef enum tp_path {
    TP_PATH_X4 = 0,
    TP_PATH_SCALAR_LOAD = 1,
    TP_PATH_SCALAR_STORE = 2,
    TP_PATH_SCALAR = 3
} tp_path;

/* How the maps move a buffer that is 4- but not 16-byte aligned. */
typedef enum tp_align {
    TP_ALIGN_REALIGN = 0, /* 16-byte accesses at any 4-byte alignment; the 1-D map moves
                             the floats before out's first 128-byte boundary (in's when
                             out - in is 64 mod 128) element-wise */
    TP_ALIGN_WORDS = 1    /* the pages' rule: 4-byte words on a side not 16-byte aligned */
} tp_align;

/* How the waves of a map workgroup share the work ("Asynchronous Data
 * Movement", section "Barriers and pipelines": producer and consumer roles). */
typedef enum tp_schedule {
    TP_SCHED_UNIFORM = 0,    /* every wave loads, computes and stores its own part of each tile */
    TP_SCHED_ROLE_SPLIT = 1  /* one extra wave issues all loads; the others compute and store */
} tp_schedule;

/* Launch plan of one call: what the entry point would enqueue (host-only). */
typedef struct tp_plan {
    int32_t path;            /* tp_path */
    int32_t stages;          /* LDS ring slots S (1 = no overlap inside a workgroup) */
    int32_t tile_units;      /* floats per tile (map), chunks per tile (chunk copy), rows (row shift) */
    int32_t threads;         /* workgroup size */
    int32_t lane_chunks;     /* 16-byte chunks each lane moves per tile */
    int32_t tiles_per_block; /* consecutive tiles one workgroup streams */
    int32_t lds_bytes;       /* dynamic LDS per workgroup */
    int32_t wait_steady;     /* vmcnt immediate of the steady-state stage wait */
    int64_t num_tiles;       /* tiles over the whole problem */
    int64_t grid;            /* workgroups launched (0: nothing to launch) */
    int32_t ring_bytes;      /* LDS the kernel itself needs (the ring and its tail area) */
    int32_t resident_cap;    /* about this many workgroups per CU (0: hardware limits only);
                                lds_bytes is padded up to bound residency */
    int32_t schedule;        /* tp_schedule (map); 0 for the other entry points */
    int32_t chunk_bytes;     /* bytes per chunk (chunk copy); 0 for the other entry points */
    int32_t align;           /* tp_align (maps); 0 for the other entry points */
    int32_t head;            /* 1-D map, TP_ALIGN_REALIGN: floats before the first 128-byte
                                boundary of out (or of in, when out - in is 64 mod 128),
                                0..31, moved element-wise; 0 otherwise */
} tp_plan;

/* Human-readable name of a tp_status value ("TP_OK", ...); never NULL. */
TP_API const char *tp_status_string(int status);

/* hipError_t of the last TP_ERR_HIP returned on the calling thread (0 if none). */
TP_API int tp_last_hip_error(void);

/* Library ABI version (TP_VERSION). */
TP_API int tp_version(void);

/* TP_OK if `device` is a gfx950 GPU, TP_ERR_UNSUPPORTED_DEVICE if it is another
 * GPU, TP_ERR_HIP if it cannot be queried (no such device, no driver). The
 * asynchronous-copy path exists only on hardware that has it ("Asynchronous
 * Data Movement", section "Genuinely asynchronous from CC 8.0+"); this library
 * targets only gfx950 and refuses other devices instead of degrading. */
TP_API int tp_device_check(int device);

/* Bytes of LDS one workgroup may use on `device` (written to *bytes), the
 * budget the entry points check stages x tile bytes against. Returns TP_OK or
 * TP_ERR_HIP; bytes must not be NULL (TP_ERR_INVALID_ARG). */
TP_API int tp_device_lds_budget(int device, int64_t *bytes);

/*
 * Neighbour-row exchange ("Asynchronous Copies", section "A Global-to-Shared
 * Copy"): each lane copies its 16-byte row of A into LDS asynchronously, waits
 * for its copies, synchronizes the workgroup, then writes row (i+1) mod rows:
 *     b[i][j] = a[(i + 1) % rows][j],   0 <= i < rows, 0 <= j < 4.
 * a, b: device buffers of rows x 4 float32, row-major (16 bytes per row); data
 * moves as raw 32-bit words. 0 <= rows <= 1024 (one workgroup; rows > 1024 is
 * TP_ERR_INVALID_ARG). b == a is allowed (in place).
 */
TP_API int tp_row_shift(const float *a, float *b, int64_t rows, void *stream, int *path_out);

/*
 * Software-pipelined tiled map ("Asynchronous Data Movement", sections
 * "Double buffering" and "Barriers and pipelines"; "CUDA Async Copy and
 * Pipeline Guide", section "Implementation Comparison"):
 *     out[i] = op(in[i]),   0 <= i < n.
 * Each workgroup streams tiles_per_block consecutive tiles of tile_elems
 * floats through an LDS ring of `stages` slots: the loads of the next
 * stages-1 tiles are in flight while the current tile is computed on and
 * stored. in, out: device buffers of n float32. op: tp_op.
 * tile_elems: 256, 512, 1024, 2048, 4096 or 8192. stages: 1..8 ("Typically 2-4
 * stages": the guide's FAQ; 1 = load, wait, compute, store with no overlap).
 * tiles_per_block: 1..65536, or 0 for the library default: runs of 4 tiles
 * of at most 512 floats, of 2 larger tiles. On MI355X short runs dispatched in
 * order keep the memory traffic of all resident workgroups within a narrow
 * window and stream fastest; runs of 4 KiB (tile 256) to 8 KiB (tiles 512
 * and 1024) were measured fastest, and runs of 3, 5 or 6 tiles 4-9 % slower.
 * stages * tile_elems * 4 must fit the device's LDS per workgroup
 * (TP_ERR_LDS_BUDGET). out == in is allowed. Buffers off a 128-byte boundary
 * are moved as TP_ALIGN_REALIGN describes: the floats before out's first
 * 128-byte boundary (at most 31) are moved element-wise and the rest is tiled
 * from there, so the 16-byte stores fill whole lines, while the loads are 16
 * bytes at whatever 4-byte alignment in then has (in's boundary is taken
 * instead when out - in is 64 modulo 128). The result does not depend
 * on tile_elems, stages, tiles_per_block or the path.
 */
TP_API int tp_pipelined_map(const float *in, float *out, int64_t n, int op,
                            int tile_elems, int stages, int tiles_per_block,
                            void *stream, int *path_out);

/*
 * tp_pipelined_map with an explicit bound on resident workgroups per CU
 * (tp_pipelined_map is this call with resident_cap 0). The bound is applied by
 * reserving LDS: each workgroup is given floor(160 KiB / cap) rounded down to
 * whole KiB (so about cap workgroups fit on a CU, a few more where the
 * rounding leaves room), or the ring's own size if that is larger, and never
 * more than the device's LDS per workgroup. It changes how much tile traffic
 * is in flight at once on a CU, never the result.
 *   resident_cap  0: the library's policy. For the streaming ops (scale2,
 *                    copy) with runs of 2 or more tiles of at most 1024
 *                    floats it keeps about 27 KiB x (1 + 1/T) of tile traffic
 *                    per CU in flight: each resident workgroup has a(T,S) + 1
 *                    tiles moving on average (a = mean over a run of
 *                    min(S, tiles left) loads, plus the stores behind them),
 *                    with at least 4 workgroups and 8 waves resident per CU.
 *                    horner32, runs of one tile and larger tiles (several
 *                    loads per lane per tile) are not bounded.
 *               -1: no bound (hardware limits only);
 *              k>0: at most k workgroups per CU;
 *          below -1: TP_ERR_INVALID_ARG.
 * schedule: TP_SCHED_UNIFORM (what tp_pipelined_map runs), or
 * TP_SCHED_ROLE_SPLIT: the workgroup gets one more wave, which issues every
 * load of every tile and waits for them; the other waves only read tiles from
 * LDS, compute and store. One workgroup barrier per iteration publishes the
 * landed tile and frees the slot the loading wave refills next (two per
 * iteration with one stage). Other values: TP_ERR_INVALID_ARG.
 * align: TP_ALIGN_REALIGN (what tp_pipelined_map does), or TP_ALIGN_WORDS:
 * a side whose pointer is not 16-byte aligned moves 4-byte words, and the
 * tiles start at in[0]. Other values: TP_ERR_INVALID_ARG.
 * The other arguments, errors and results are those of tp_pipelined_map.
 */
TP_API int tp_pipelined_map_ex(const float *in, float *out, int64_t n, int op,
                               int tile_elems, int stages, int tiles_per_block,
                               int resident_cap, int schedule, int align, void *stream,
                               int *path_out);

/*
 * Strided 2-D map ("Asynchronous Data Movement", section "The Tensor Memory
 * Accelerator": a tile transfer described by a base, a shape and strides
 * rather than by per-thread addresses):
 *     dst[r * dst_stride + c] = op(src[r * src_stride + c]),  0 <= r < rows, 0 <= c < cols.
 * src, dst: device float32 buffers; strides in elements, cols <= stride <= 2^36.
 * The window is cut into boxes of box_rows x box_cols floats (powers of two,
 * box_cols >= 4, box_rows * box_cols one of 256 .. 8192; 0 x 0 picks boxes of
 * 1024 floats as wide as the window allows: box_cols the smallest power of
 * two >= min(cols, 1024), at least 4, box_rows = 1024 / box_cols); a workgroup streams
 * boxes_per_block boxes side by side in one band of box_rows rows (0: the
 * default of 2) through an LDS ring of `stages` slots, each box read by
 * LDS-DMA loads from row * stride + column. Elements of an edge box outside
 * the matrix are neither read nor written, and dst outside the window is not
 * touched. With align TP_ALIGN_REALIGN both sides use 16-byte accesses
 * whenever cols is a multiple of 4, at any 4-byte alignment of the pointers
 * and any strides; with TP_ALIGN_WORDS a side uses them only when its pointer
 * is also 16-byte aligned and its stride a multiple of 4. Otherwise the side
 * moves 4-byte words (reported in path_out; bit 0 loads, bit 1 stores). Other
 * align values: TP_ERR_INVALID_ARG. The library's bound on
 * resident workgroups per CU (tp_pipelined_map_ex) applies. Errors:
 * TP_ERR_INVALID_ARG (bad shape, box, stages, a band of box_rows rows up to
 * the run's last column spanning more than 1 GiB on either side, or more than
 * 2^31 - 1 workgroups), TP_ERR_MISALIGNED (a pointer not 4-byte aligned),
 * TP_ERR_OVERLAP (the byte ranges of the windows overlap, unless dst == src
 * with equal strides, which is allowed), TP_ERR_LDS_BUDGET (stages x box bytes
 * exceeds the device's LDS per workgroup). rows or cols 0: TP_OK, nothing
 * launched (pointers may then be NULL).
 */
TP_API int tp_map_2d(const float *src, int64_t src_stride, float *dst, int64_t dst_stride,
                     int64_t rows, int64_t cols, int op, int box_rows, int box_cols,
                     int stages, int boxes_per_block, int align, void *stream,
                     int *path_out);

/*
 * Predicated 16-byte chunk copy ("Asynchronous Copies", section "A
 * Global-to-Shared Copy", the paragraph on pred, src_size and ignore_src).
 * For each chunk i < n_chunks:
 *   pred[i] == 0           -> dst chunk i is not written at all;
 *   else ignore_src[i] != 0 -> dst chunk i = 16 zero bytes;
 *   else                    -> dst bytes [0, s) = src bytes [0, s), bytes
 *                              [s, 16) = 0, with s = min(src_size[i], 16).
 * src, dst: device buffers of n_chunks x 16 bytes (4-byte aligned; 16-byte
 * alignment selects the fast path). pred, src_size, ignore_src: device arrays
 * of n_chunks bytes (any alignment), or NULL for "all 1", "all 16" and "all 0".
 * The whole 16-byte source chunk must be readable memory whatever the operands
 * say (the paragraph's bounds-check sentence); the kernel may read it (the
 * 16-byte load path skips a chunk whose bytes would all be dropped, the word
 * path reads every chunk). stages: 1..8.
 * tiles_per_block (256-chunk tiles): 1..65536, or 0 for the default of
 * max(stages - 1, 1) tiles, so that the ring's prologue holds the whole run
 * (on MI355X the masked writes that false preds leave are served fastest when
 * a wave's loads come as one burst before its stores; runs of 64 tiles ran
 * about 1.45x slower). The ring is cut to what the run can use: at most
 * tiles_per_block + 1 slots, and one slot for runs of one tile (the same
 * instructions in less LDS); the plan reports the stages that run. Each
 * workgroup of 256 lanes moves one chunk per lane per tile; a 16-byte
 * destination takes one 16-byte store per chunk, otherwise each store
 * instruction writes 64 consecutive words of the wave's chunks.
 * dst == src is allowed; dst overlapping a metadata array is TP_ERR_OVERLAP.
 */
TP_API int tp_chunk_copy(const void *src, void *dst, int64_t n_chunks,
                         const uint8_t *pred, const uint8_t *src_size,
                         const uint8_t *ignore_src, int stages, int tiles_per_block,
                         void *stream, int *path_out);

/*
 * tp_chunk_copy for chunks of chunk_bytes = 4, 8 or 16 bytes (tp_chunk_copy is
 * chunk_bytes 16), the element sizes the pages name for the fast copy path
 * ("Asynchronous Data Movement", section "Alignment requirements"). The
 * operands keep their meaning with 16 replaced by chunk_bytes: s =
 * min(src_size[i], chunk_bytes) bytes are copied and the rest of the chunk is
 * zeroed. src and dst hold n_chunks x chunk_bytes bytes, 4-byte aligned; 4-
 * and 8-byte chunks always move as 4-byte words (path_out TP_PATH_SCALAR).
 * Their tiles are smaller (2 and 1 KiB), so the default run is longer:
 * max(stages - 1, 2) tiles of 8-byte and max(stages - 1, 8) tiles of 4-byte
 * chunks. Other chunk_bytes: TP_ERR_INVALID_ARG.
 */
TP_API int tp_chunk_copy_ex(const void *src, void *dst, int64_t n_chunks, int chunk_bytes,
                            const uint8_t *pred, const uint8_t *src_size,
                            const uint8_t *ignore_src, int stages, int tiles_per_block,
                            void *stream, int *path_out);

/*
 * Copies between workgroups ("Asynchronous Copies", section "Copies between
 * CTAs": one group copies a 256-byte chunk of its shared memory into another
 * group's, and the receiver waits until the bytes have arrived before reading
 * them). Over n_chunks chunks of 256 bytes, workgroup k copies chunk k of src
 * into its LDS and hands it to workgroup k + 1, which writes what it received
 * as chunk k + 1 of dst:
 *     dst[k] = src[k - 1]   (256 bytes each),  1 <= k < n_chunks;
 * chunk 0 of dst receives nothing and is not written. CDNA4 workgroups cannot
 * address each other's LDS, so the chunk passes through a staging slot in
 * `workspace`: each 4-byte word of it is stored together with a 4-byte tag in
 * one 8-byte device-scope store (coherent across the XCDs' L2s), which lands
 * as a whole. The receiver loads the slot the same way until every word's tag
 * is set, so the arrival of the bytes is read off the bytes themselves; it
 * puts them into its LDS and stores them. A workgroup waits only for the one
 * numbered just below it, which was dispatched before it, and a sender waits
 * for nothing but its own source load.
 *   src, dst: device buffers of n_chunks x 256 bytes, 4-byte aligned; dst ==
 *     src is allowed (each workgroup reads its own chunk before its receiver
 *     role writes it); a partial overlap is TP_ERR_OVERLAP.
 *   workspace: caller-owned device memory of at least
 *     tp_workgroup_copy_workspace_bytes(n_chunks) bytes (512 per chunk), 8-byte
 *     aligned. The call zeroes the slots itself (a kernel on `stream` before
 *     the hand-off), so the workspace needs no preparation and may be used
 *     for anything else between calls. Calls that share a workspace must not
 *     overlap in time.
 *   status: caller-owned device int32. The call sets it to 0 and a receiver
 *     that gives up waiting sets it to 1; read it after the stream has
 *     finished. 1 means some dst chunks were not written.
 *   spin_limit: polls of its sender's slot before a receiver gives up
 *     (0 = the default of 65536; at most 2^24). A waiting receiver also reads
 *     the status every 8 polls and stops once it is set, so the kernel always
 *     finishes.
 * n_chunks 0: TP_OK, nothing launched. More than 2^26 chunks, a missing
 * pointer or a short workspace: TP_ERR_INVALID_ARG; src, dst or status not
 * 4-byte aligned, or the workspace not 8-byte aligned: TP_ERR_MISALIGNED;
 * workspace or status overlapping src or dst, or each other: TP_ERR_OVERLAP.
 */
TP_API int tp_workgroup_copy(const void *src, void *dst, int64_t n_chunks, void *workspace,
                             int64_t workspace_bytes, int32_t *status, int spin_limit,
                             void *stream);

/* Bytes of workspace tp_workgroup_copy needs for n_chunks chunks, 512 per
 * chunk (-1 if n_chunks is out of range). */
TP_API int64_t tp_workgroup_copy_workspace_bytes(int64_t n_chunks);

/*
 * tp_workgroup_copy without a workspace argument and without allocating, for
 * callers that cannot allocate (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc). The staging slots live in a static
 * device array of 8 388 608 bytes that the library holds on each GPU it runs
 * on, for up to 16384 chunks; n_chunks above that is TP_ERR_INVALID_ARG. The
 * array is found once per device with hipGetSymbolAddress (with that device
 * current) and never allocated or freed.
 * Every call on one GPU shares that GPU's array and zeroes its slots first:
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race and may give wrong results. src, dst, status, spin_limit, results and
 * the other errors are those of tp_workgroup_copy.
 */
TP_API int tp_workgroup_copy_noalloc(const void *src, void *dst, int64_t n_chunks,
                                     int32_t *status, int spin_limit, void *stream);

/*
 * Host-only planning: the same validation and launch plan as the entry point
 * of the same name, for the given pointer values and LDS budget (bytes per
 * workgroup), without touching any device. Pointers are only inspected for
 * null, alignment and overlap. Returns the status the entry point would return
 * for argument errors; on TP_OK, *plan describes the launch (plan may be NULL).
 */
TP_API int tp_plan_row_shift(const void *a, const void *b, int64_t rows,
                             int64_t lds_budget, tp_plan *plan);
TP_API int tp_plan_pipelined_map(const void *in, const void *out, int64_t n, int op,
                                 int tile_elems, int stages, int tiles_per_block,
                                 int resident_cap, int schedule, int align,
                                 int64_t lds_budget, tp_plan *plan);
TP_API int tp_plan_map_2d(const void *src, int64_t src_stride, const void *dst,
                          int64_t dst_stride, int64_t rows, int64_t cols, int op, int box_rows,
                          int box_cols, int stages, int boxes_per_block, int align,
                          int64_t lds_budget, tp_plan *plan);
TP_API int tp_plan_chunk_copy(const void *src, const void *dst, int64_t n_chunks,
                              int chunk_bytes, const void *pred, const void *src_size,
                              const void *ignore_src, int stages, int tiles_per_block,
                              int64_t lds_budget, tp_plan *plan);
TP_API int tp_plan_workgroup_copy(const void *src, const void *dst, int64_t n_chunks,
                                  const void *workspace, int64_t workspace_bytes,
                                  const int32_t *status, int spin_limit, tp_plan *plan);

#ifdef __cplusplus
}
#endif

#endif /* TILEPIPE_H */
