/*
 * A plain C client of libtilepipe: TEST CODE. It drives the library through
 * include/tilepipe.h alone, with memory from the HIP runtime's C API, and
 * compares every result bit for bit with the CPU oracle (oracle/liboracle.so,
 * which tests may link). It is built as a shared object linked against
 * libtilepipe.so and liboracle.so, and the tests call its one entry point:
 *
 *   tp_c_client_run("host", ...)  planning and error paths only (tp_plan_*,
 *                                 status strings, workspace sizes); touches
 *                                 no device
 *   tp_c_client_run("gpu", ...)   every entry point on device 0, checked
 *                                 against the oracle
 *
 * It prints one line per case passed and returns 0 when every case passes, 1
 * with the first mismatch or unexpected status described in `msg`, 2 for an
 * unknown mode. Device memory of a failed case is not freed.
 */
#include <setjmp.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tilepipe.h"

/* The oracle's entry points (oracle/oracle.c); it ships no header. */
void oracle_row_shift(const uint32_t *a, uint32_t *b, int64_t rows);
void oracle_map_scale2(const float *in, float *out, int64_t lo, int64_t hi);
void oracle_map_copy(const float *in, float *out, int64_t lo, int64_t hi);
void oracle_map_horner32(const float *in, float *out, int64_t lo, int64_t hi);
void oracle_map_2d(const float *src, int64_t src_stride, float *dst, int64_t dst_stride,
                   int64_t cols, int op, int64_t lo, int64_t hi);
void oracle_chunk_copy_w(const uint8_t *src, uint8_t *dst, int width, const uint8_t *pred,
                         const uint8_t *src_size, const uint8_t *ignore_src, int64_t lo,
                         int64_t hi);
void oracle_workgroup_copy(const uint8_t *src, uint8_t *dst, int64_t lo, int64_t hi);

static jmp_buf fail_jmp;
static char fail_msg[512];

#define CHECK(cond, ...)                                                                 \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            int at_ = snprintf(fail_msg, sizeof fail_msg, "%s:%d: ", __FILE__, __LINE__); \
            snprintf(fail_msg + at_, sizeof fail_msg - at_, __VA_ARGS__);                \
            longjmp(fail_jmp, 1);                                                        \
        }                                                                                \
    } while (0)

#define HIP(call)                                                                   \
    do {                                                                            \
        hipError_t e_ = (call);                                                     \
        CHECK(e_ == hipSuccess, "%s -> %s", #call, hipGetErrorString(e_));          \
    } while (0)

#define TP(call, expect)                                                            \
    do {                                                                            \
        int s_ = (call);                                                            \
        CHECK(s_ == (expect), "%s -> %s, expected %s (hip error %d)", #call,        \
              tp_status_string(s_), tp_status_string(expect), tp_last_hip_error()); \
    } while (0)

static void ok(const char *what)
{
    printf("c_client: %s ok\n", what);
    fflush(stdout);
}

/* splitmix64: test inputs only (no part of what the library computes) */
static uint64_t rng_state;
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* uniform on [-1, 1) on a 2^-23 grid */
static float next_pm1(void)
{
    return (float)((int64_t)(next_u64() >> 40) - (1 << 23)) * 0x1p-23f;
}

static void *host_alloc(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    CHECK(p != NULL, "malloc(%zu)", bytes);
    return p;
}

static void *dev_alloc(size_t bytes)
{
    void *p = NULL;
    HIP(hipMalloc(&p, bytes ? bytes : 4));
    return p;
}

static void expect_same(const void *got, const void *want, size_t bytes, const char *what)
{
    const uint8_t *g = got, *w = want;
    for (size_t i = 0; i < bytes; ++i)
        CHECK(g[i] == w[i], "%s: byte %zu is 0x%02x, the oracle gives 0x%02x", what, i, g[i],
              w[i]);
}

/* ---- host mode: the ABI from C without a device ---- */

static void host_mode(void)
{
    CHECK(tp_version() == TP_VERSION, "tp_version %d", tp_version());
    CHECK(strcmp(tp_status_string(TP_OK), "TP_OK") == 0, "status string of TP_OK");
    CHECK(strcmp(tp_status_string(TP_ERR_OVERLAP), "TP_ERR_OVERLAP") == 0, "overlap string");
    CHECK(tp_status_string(12345) != NULL, "unknown status string is NULL");
    ok("status strings and version");

    const int64_t lds = 160 * 1024;
    tp_plan p;
    /* a 4 KiB-aligned stand-in address: planning only inspects pointer values */
    const char *base = (const char *)(uintptr_t)0x100000000ull;
    const char *out = base + (64 << 20);
    const int32_t *status = (const int32_t *)(base + (192 << 20));
    TP(tp_plan_pipelined_map(base, out, 1 << 24, TP_OP_SCALE2, 256, 2, 0, 0, 0, 0, lds, &p),
       TP_OK);
    CHECK(p.tiles_per_block == 4 && p.grid == (1 << 24) / 1024 && p.path == TP_PATH_X4,
          "map plan: runs %d grid %lld path %d", p.tiles_per_block, (long long)p.grid, p.path);
    TP(tp_plan_pipelined_map(base + 2, out, 100, TP_OP_SCALE2, 256, 2, 0, 0, 0, 0, lds, &p),
       TP_ERR_MISALIGNED);
    TP(tp_plan_pipelined_map(base, base + 64, 100, TP_OP_SCALE2, 256, 2, 0, 0, 0, 0, lds, &p),
       TP_ERR_OVERLAP);
    TP(tp_plan_pipelined_map(base, out, 100, TP_OP_SCALE2, 8192, 8, 0, 0, 0, 0, lds, &p),
       TP_ERR_LDS_BUDGET);
    TP(tp_plan_pipelined_map(base, out, 100, 7, 256, 2, 0, 0, 0, 0, lds, &p), TP_ERR_INVALID_ARG);
    ok("map planning and argument errors");

    TP(tp_plan_map_2d(base, 1037, out, 1000, 300, 1000, TP_OP_HORNER32, 0, 0, 2,
                      0, TP_ALIGN_REALIGN, lds, &p),
       TP_OK);
    CHECK(p.tile_units == 1024, "2-D default box %d floats", p.tile_units);
    TP(tp_plan_chunk_copy(base, out, 100003, 16, NULL, NULL, NULL, 2, 0, lds, &p), TP_OK);
    CHECK(p.chunk_bytes == 16, "chunk plan width %d", p.chunk_bytes);
    TP(tp_plan_chunk_copy(base, out, 100, 12, NULL, NULL, NULL, 2, 0, lds, &p),
       TP_ERR_INVALID_ARG);
    TP(tp_plan_row_shift(base, base + 4096, 64, lds, &p), TP_OK);
    TP(tp_plan_row_shift(base, base + 4096, 1025, lds, &p), TP_ERR_INVALID_ARG);
    ok("2-D map, chunk copy and row exchange planning");

    const int64_t ws = tp_workgroup_copy_workspace_bytes(1000);
    CHECK(ws >= 1000 * (256 + 4), "workspace bytes %lld", (long long)ws);
    CHECK(tp_workgroup_copy_workspace_bytes(-1) == -1, "workspace bytes of -1 chunks");
    TP(tp_plan_workgroup_copy(base, out, 1000, base + (128 << 20), ws, status, 0, &p), TP_OK);
    TP(tp_plan_workgroup_copy(base, out, 1000, base + (128 << 20), ws - 4, status, 0, &p),
       TP_ERR_INVALID_ARG);
    ok("workgroup copy planning");
}

/* ---- gpu mode ---- */

static void gpu_row_shift(hipStream_t st)
{
    const int64_t rows = 64;
    uint32_t a[256], b[256], want[256];
    for (int i = 0; i < 256; ++i)
        a[i] = i; /* the bit patterns of 0 .. 255 */
    void *da = dev_alloc(sizeof a), *db = dev_alloc(sizeof b);
    HIP(hipMemcpy(da, a, sizeof a, hipMemcpyHostToDevice));
    int path = -1;
    TP(tp_row_shift(da, db, rows, st, &path), TP_OK);
    HIP(hipStreamSynchronize(st));
    HIP(hipMemcpy(b, db, sizeof b, hipMemcpyDeviceToHost));
    oracle_row_shift(a, want, rows);
    expect_same(b, want, sizeof b, "row exchange 64 x 4");
    HIP(hipFree(da));
    HIP(hipFree(db));
    ok("row exchange 64 x 4");
}

static void gpu_map(hipStream_t st)
{
    const int64_t n = 3 * (1 << 18) + 37;
    float *x = host_alloc((n + 1) * sizeof(float)), *y = host_alloc(n * sizeof(float));
    float *want = host_alloc(n * sizeof(float));
    for (int64_t i = 0; i < n + 1; ++i)
        x[i] = next_pm1();
    float *dx = dev_alloc((n + 1) * sizeof(float)), *dy = dev_alloc(n * sizeof(float));
    HIP(hipMemcpy(dx, x, (n + 1) * sizeof(float), hipMemcpyHostToDevice));
    static const char *names[] = {"scale2", "horner32", "copy"};
    for (int op = 0; op < 3; ++op) {
        /* the source 4 bytes past the allocation's start: off every 16-byte boundary */
        int path = -1;
        TP(tp_pipelined_map(dx + 1, dy, n, op, 1024, 2, 0, st, &path), TP_OK);
        HIP(hipStreamSynchronize(st));
        HIP(hipMemcpy(y, dy, n * sizeof(float), hipMemcpyDeviceToHost));
        if (op == TP_OP_SCALE2)
            oracle_map_scale2(x + 1, want, 0, n);
        else if (op == TP_OP_HORNER32)
            oracle_map_horner32(x + 1, want, 0, n);
        else
            oracle_map_copy(x + 1, want, 0, n);
        char what[96];
        snprintf(what, sizeof what, "pipelined map %s, %lld floats, source at +4 B", names[op],
                 (long long)n);
        expect_same(y, want, n * sizeof(float), what);
        ok(what);
    }
    /* in place, the pages' 4-byte fallback on the misaligned side */
    int path = -1;
    TP(tp_pipelined_map_ex(dx + 1, dx + 1, n, TP_OP_SCALE2, 256, 3, 0, 0, TP_SCHED_UNIFORM,
                           TP_ALIGN_WORDS, st, &path),
       TP_OK);
    CHECK(path == TP_PATH_SCALAR, "words path reported %d", path);
    HIP(hipStreamSynchronize(st));
    HIP(hipMemcpy(y, dx + 1, n * sizeof(float), hipMemcpyDeviceToHost));
    oracle_map_scale2(x + 1, want, 0, n);
    expect_same(y, want, n * sizeof(float), "in place, 4-byte words");
    ok("pipelined map in place with the 4-byte fallback");
    /* errors are reported before anything is enqueued */
    TP(tp_pipelined_map((const float *)((char *)dx + 2), dy, n, TP_OP_SCALE2, 1024, 2, 0, st,
                        NULL),
       TP_ERR_MISALIGNED);
    TP(tp_pipelined_map(dx, dx + 16, n, TP_OP_SCALE2, 1024, 2, 0, st, NULL), TP_ERR_OVERLAP);
    TP(tp_pipelined_map(dx, dy, 0, TP_OP_SCALE2, 1024, 2, 0, st, NULL), TP_OK);
    ok("map argument errors");
    HIP(hipFree(dx));
    HIP(hipFree(dy));
    free(x);
    free(y);
    free(want);
}

static void gpu_map_2d(hipStream_t st)
{
    const int64_t rows = 300, cols = 1000, ss = 1037, ds = 1000;
    float *src = host_alloc(rows * ss * sizeof(float));
    float *dst = host_alloc(rows * ds * sizeof(float));
    float *want = host_alloc(rows * ds * sizeof(float));
    for (int64_t i = 0; i < rows * ss; ++i)
        src[i] = next_pm1();
    float *dsrc = dev_alloc(rows * ss * sizeof(float));
    float *ddst = dev_alloc(rows * ds * sizeof(float));
    HIP(hipMemcpy(dsrc, src, rows * ss * sizeof(float), hipMemcpyHostToDevice));
    int path = -1;
    TP(tp_map_2d(dsrc, ss, ddst, ds, rows, cols, TP_OP_HORNER32, 0, 0, 2, 0, TP_ALIGN_REALIGN, st,
                 &path),
       TP_OK);
    HIP(hipStreamSynchronize(st));
    HIP(hipMemcpy(dst, ddst, rows * ds * sizeof(float), hipMemcpyDeviceToHost));
    oracle_map_2d(src, ss, want, ds, cols, TP_OP_HORNER32, 0, rows);
    expect_same(dst, want, rows * ds * sizeof(float), "2-D map");
    ok("2-D map horner32, 300 x 1000 window of rows 1037 floats apart");
    HIP(hipFree(dsrc));
    HIP(hipFree(ddst));
    free(src);
    free(dst);
    free(want);
}

static void gpu_chunk_copy(hipStream_t st, int width)
{
    const int64_t n = 100003;
    const size_t bytes = (size_t)n * width;
    uint8_t *src = host_alloc(bytes), *dst = host_alloc(bytes), *want = host_alloc(bytes);
    uint8_t *pred = host_alloc(n), *size = host_alloc(n), *ign = host_alloc(n);
    for (size_t i = 0; i < bytes; ++i)
        src[i] = (uint8_t)next_u64();
    for (int64_t i = 0; i < n; ++i) {
        pred[i] = next_u64() % 10 != 0;               /* true with probability 0.9 */
        size[i] = (uint8_t)(next_u64() % (width + 2)); /* 0 .. width + 1 (above width clamps) */
        ign[i] = next_u64() % 100 == 0;               /* true with probability 0.01 */
    }
    static const uint8_t fill[4] = {0xEF, 0xBE, 0xAD, 0xDE};
    for (size_t i = 0; i < bytes; ++i)
        want[i] = fill[i % 4];
    uint8_t *dsrc = dev_alloc(bytes), *ddst = dev_alloc(bytes);
    uint8_t *dpred = dev_alloc(n), *dsize = dev_alloc(n), *dign = dev_alloc(n);
    HIP(hipMemcpy(dsrc, src, bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(ddst, want, bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dpred, pred, n, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dsize, size, n, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dign, ign, n, hipMemcpyHostToDevice));
    int path = -1;
    if (width == 16)
        TP(tp_chunk_copy(dsrc, ddst, n, dpred, dsize, dign, 2, 0, st, &path), TP_OK);
    else
        TP(tp_chunk_copy_ex(dsrc, ddst, n, width, dpred, dsize, dign, 2, 0, st, &path), TP_OK);
    HIP(hipStreamSynchronize(st));
    HIP(hipMemcpy(dst, ddst, bytes, hipMemcpyDeviceToHost));
    oracle_chunk_copy_w(src, want, width, pred, size, ign, 0, n);
    char what[96];
    snprintf(what, sizeof what, "predicated chunk copy, %lld chunks of %d bytes", (long long)n,
             width);
    expect_same(dst, want, bytes, what);
    ok(what);
    HIP(hipFree(dsrc));
    HIP(hipFree(ddst));
    HIP(hipFree(dpred));
    HIP(hipFree(dsize));
    HIP(hipFree(dign));
    free(src);
    free(dst);
    free(want);
    free(pred);
    free(size);
    free(ign);
}

static void gpu_workgroup_copy(hipStream_t st, int noalloc)
{
    const int64_t n = noalloc ? 300 : 1000;
    const size_t bytes = (size_t)n * 256;
    uint8_t *src = host_alloc(bytes), *dst = host_alloc(bytes), *want = host_alloc(bytes);
    for (size_t i = 0; i < bytes; ++i) {
        src[i] = (uint8_t)next_u64();
        want[i] = 0x5A;
    }
    uint8_t *dsrc = dev_alloc(bytes), *ddst = dev_alloc(bytes);
    int32_t *dstatus = dev_alloc(sizeof(int32_t));
    HIP(hipMemcpy(dsrc, src, bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(ddst, want, bytes, hipMemcpyHostToDevice));
    void *ws = NULL;
    if (noalloc) {
        TP(tp_workgroup_copy_noalloc(dsrc, ddst, n, dstatus, 0, st), TP_OK);
    } else {
        const int64_t wsb = tp_workgroup_copy_workspace_bytes(n);
        ws = dev_alloc(wsb);
        TP(tp_workgroup_copy(dsrc, ddst, n, ws, wsb, dstatus, 0, st), TP_OK);
    }
    HIP(hipStreamSynchronize(st));
    int32_t status = -1;
    HIP(hipMemcpy(&status, dstatus, sizeof status, hipMemcpyDeviceToHost));
    CHECK(status == 0, "workgroup copy status %d", status);
    HIP(hipMemcpy(dst, ddst, bytes, hipMemcpyDeviceToHost));
    oracle_workgroup_copy(src, want, 0, n);
    const char *what = noalloc ? "copy between workgroups without allocating, 300 chunks"
                               : "copy between workgroups, 1000 chunks";
    expect_same(dst, want, bytes, what);
    ok(what);
    if (ws)
        HIP(hipFree(ws));
    HIP(hipFree(dsrc));
    HIP(hipFree(ddst));
    HIP(hipFree(dstatus));
    free(src);
    free(dst);
    free(want);
}

static void gpu_mode(void)
{
    HIP(hipSetDevice(0));
    TP(tp_device_check(0), TP_OK);
    int64_t lds = 0;
    TP(tp_device_lds_budget(0, &lds), TP_OK);
    CHECK(lds >= 64 * 1024, "LDS budget %lld", (long long)lds);
    ok("device check");
    hipStream_t st;
    HIP(hipStreamCreate(&st));
    gpu_row_shift(st);
    gpu_map(st);
    gpu_map_2d(st);
    gpu_chunk_copy(st, 16);
    gpu_chunk_copy(st, 8);
    gpu_chunk_copy(st, 4);
    gpu_workgroup_copy(st, 0);
    gpu_workgroup_copy(st, 1);
    /* the same call on the default stream (a null stream argument) */
    gpu_row_shift(NULL);
    HIP(hipStreamDestroy(st));
}

int tp_c_client_run(const char *mode, char *msg, int msglen)
{
    rng_state = 20261202;
    fail_msg[0] = 0;
    if (setjmp(fail_jmp)) {
        snprintf(msg, msglen, "%s", fail_msg);
        return 1;
    }
    if (strcmp(mode, "host") == 0)
        host_mode();
    else if (strcmp(mode, "gpu") == 0)
        gpu_mode();
    else {
        snprintf(msg, msglen, "unknown mode %s (host or gpu)", mode);
        return 2;
    }
    printf("c_client: all cases passed\n");
    fflush(stdout);
    return 0;
}
