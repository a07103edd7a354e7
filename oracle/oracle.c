/*
 * CPU oracle for libtilepipe: TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct C definitions of what the GPU entry points
 * compute. Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's library; the product path never does.
 * It shares no code, header, table or helper with the HIP library: it has its
 * own coefficient table, its own loops and no notion of tiles, stages, lanes
 * or alignment, because those change only the speed of the GPU path, never
 * its result ("Asynchronous Data Movement", section "Alignment requirements":
 * the slow fallback is still correct; "Asynchronous Copies", section "A
 * Global-to-Shared Copy": the async version gives the same row shift as the
 * synchronous one).
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * No contraction and no fast-math, so every float operation below is exactly
 * one IEEE-754 binary32 operation rounded to nearest-even (x86-64 SSE default,
 * no flush-to-zero). The only fused operation is the explicit fmaf().
 *
 * Every range-taking function works on [lo, hi) so a harness may split the
 * index space over threads; results do not depend on the split.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

/*
 * Row exchange ("Asynchronous Copies", section "A Global-to-Shared Copy":
 * each thread copies its four-float row, then writes the next thread's row;
 * the check compares against a roll of -1 along the row axis).
 *   b[i][j] = a[(i + 1) mod rows][j],  0 <= i < rows, 0 <= j < 4
 * Rows are moved as raw 32-bit words so any bit pattern (NaN payloads
 * included) must come through unchanged. a and b must not overlap.
 */
void oracle_row_shift(const uint32_t *a, uint32_t *b, int64_t rows)
{
    for (int64_t i = 0; i < rows; ++i) {
        int64_t src = (i + 1) % rows;
        for (int j = 0; j < 4; ++j)
            b[4 * i + j] = a[4 * src + j];
    }
}

/*
 * Scale-by-2 map ("CUDA Async Copy and Pipeline Guide", section
 * "Implementation Comparison": both the synchronous and the pipelined kernel
 * compute out = in * 2 on each float of the tile).
 */
void oracle_map_scale2(const float *in, float *out, int64_t lo, int64_t hi)
{
    for (int64_t i = lo; i < hi; ++i)
        out[i] = 2.0f * in[i];
}

/* Identity map: out[i] = in[i], bit for bit (a copy-bandwidth ceiling op). */
void oracle_map_copy(const float *in, float *out, int64_t lo, int64_t hi)
{
    for (int64_t i = lo; i < hi; ++i)
        out[i] = in[i];
}

/*
 * Coefficients of the compute-heavy map: c_k = 1/(k+1) rounded to the nearest
 * binary32 (ties to even), k = 0..31. The pages leave the tile's compute
 * open ("Asynchronous Data Movement", section "Double buffering": the compute
 * step is elided); the 32-step Horner chain is the workload's own definition.
 */
void oracle_horner32_coeffs(float c[32])
{
    for (int k = 0; k < 32; ++k)
        c[k] = 1.0f / (float)(k + 1);
}

/*
 * Compute-heavy map: y = +0; for k = 0, 1, ..., 31: y = fmaf(y, x, c_k);
 * out = y. With ascending k this is Horner's rule for
 *   p(x) = sum_{k=0}^{31} c_k x^(31-k),
 * so p(0) = c_31 = 1/32. Each step is one correctly rounded fused multiply-add.
 */
void oracle_map_horner32(const float *in, float *out, int64_t lo, int64_t hi)
{
    float c[32];
    oracle_horner32_coeffs(c);
    for (int64_t i = lo; i < hi; ++i) {
        const float x = in[i];
        float y = 0.0f;
        for (int k = 0; k < 32; ++k)
            y = fmaf(y, x, c[k]);
        out[i] = y;
    }
}

/*
 * Strided 2-D map: the maps above applied to a window of a row-major matrix
 * whose rows lie a stride apart, the tile described by a base, a shape and
 * strides ("Asynchronous Data Movement", section "The Tensor Memory
 * Accelerator"):
 *   dst[r * dst_stride + c] = op(src[r * src_stride + c]),  lo <= r < hi, 0 <= c < cols
 * op: 0 scale2, 1 horner32, 2 copy. Elements of dst outside the window are
 * not written. Rows are independent, so [lo, hi) splits the rows over threads.
 */
void oracle_map_2d(const float *src, int64_t src_stride, float *dst, int64_t dst_stride,
                   int64_t cols, int op, int64_t lo, int64_t hi)
{
    for (int64_t r = lo; r < hi; ++r) {
        const float *s = src + r * src_stride;
        float *d = dst + r * dst_stride;
        if (op == 0)
            oracle_map_scale2(s, d, 0, cols);
        else if (op == 1)
            oracle_map_horner32(s, d, 0, cols);
        else
            oracle_map_copy(s, d, 0, cols);
    }
}

/*
 * Diagnostic for the rounding reading: how many Horner steps over [lo, hi)
 * produce a subnormal result or a subnormal (nonzero) exact product y*x.
 * If this is zero on a workload, a flush-to-zero mode on either side could not
 * have changed any result there. The product is formed in double, where the
 * product of two binary32 values is exact.
 * The check on y cannot fire for finite inputs: y = fma(y', x, c_k) with
 * c_k >= 2^-5 is below 2^-126 only if y'x cancels c_k, which needs
 * |y'x| > 2^-6; both terms then lie on a grid no finer than 2^-53, so their
 * sum is zero or at least 2^-53. It stays as a guard; the product count is
 * the one that inputs such as subnormal x reach (31 steps for any subnormal x).
 */
int64_t oracle_horner32_subnormal_steps(const float *in, int64_t lo, int64_t hi)
{
    float c[32];
    oracle_horner32_coeffs(c);
    int64_t count = 0;
    for (int64_t i = lo; i < hi; ++i) {
        const float x = in[i];
        float y = 0.0f;
        for (int k = 0; k < 32; ++k) {
            const double prod = (double)y * (double)x;
            if (prod != 0.0 && fabs(prod) < (double)FLT_MIN)
                ++count;
            y = fmaf(y, x, c[k]);
            if (y != 0.0f && fabsf(y) < FLT_MIN)
                ++count;
        }
    }
    return count;
}

/*
 * Predicated chunk copy ("Asynchronous Copies", section "A Global-to-Shared
 * Copy", the paragraph on the copy's optional operands), for chunks of
 * `width` = 4, 8 or 16 bytes, the element sizes the pages name for the fast
 * copy path ("Asynchronous Data Movement", section "Alignment requirements"):
 *   - a false predicate skips the copy and leaves the destination chunk as it
 *     was (it is not written at all);
 *   - otherwise, ignore_src set: the whole chunk becomes zero bytes;
 *   - otherwise, the first s = min(src_size, width) bytes come from the source
 *     chunk and the remaining width - s bytes become zero.
 * pred and ignore_src are bytes read as nonzero = true. A NULL array means its
 * default for every chunk: pred all true, src_size all `width`, ignore_src all
 * false. src and dst hold `width` bytes per chunk; they may be the same
 * buffer (every chunk is computed from its own source bytes only).
 * oracle_chunk_copy is the 16-byte case.
 */
void oracle_chunk_copy_w(const uint8_t *src, uint8_t *dst, int width,
                         const uint8_t *pred, const uint8_t *src_size,
                         const uint8_t *ignore_src, int64_t lo, int64_t hi)
{
    for (int64_t i = lo; i < hi; ++i) {
        const int p = pred ? (pred[i] != 0) : 1;
        if (!p)
            continue;
        const int ign = ignore_src ? (ignore_src[i] != 0) : 0;
        int s = src_size ? (int)src_size[i] : width;
        if (s > width)
            s = width;
        if (ign)
            s = 0;
        uint8_t chunk[16];
        for (int b = 0; b < width; ++b)
            chunk[b] = (b < s) ? src[(int64_t)width * i + b] : 0;
        memcpy(dst + (int64_t)width * i, chunk, (size_t)width);
    }
}

void oracle_chunk_copy(const uint8_t *src, uint8_t *dst,
                       const uint8_t *pred, const uint8_t *src_size,
                       const uint8_t *ignore_src, int64_t lo, int64_t hi)
{
    oracle_chunk_copy_w(src, dst, 16, pred, src_size, ignore_src, lo, hi);
}

/*
 * Copies between workgroups ("Asynchronous Copies", section "Copies between
 * CTAs": one group's shared-memory chunk of 256 bytes is copied into another
 * group's shared memory, and the receiver waits until those bytes have
 * arrived before it reads them). Over n chunks, group k holds chunk k of src
 * and hands it to group k + 1, which writes what it received as chunk k + 1
 * of dst:
 *   dst[k] = src[k - 1]  (256 bytes each),  1 <= k < n;
 * dst chunk 0 receives nothing and is not written. src and dst must not
 * overlap. [lo, hi) ranges over the receiving chunks k.
 */
void oracle_workgroup_copy(const uint8_t *src, uint8_t *dst, int64_t lo, int64_t hi)
{
    for (int64_t k = lo; k < hi; ++k) {
        if (k < 1)
            continue;
        memcpy(dst + 256 * k, src + 256 * (k - 1), 256);
    }
}
