// Neighbour-row exchange: b[i][:] = a[(i + 1) % rows][:], rows of 4 floats.
//
// "Asynchronous Copies", section "A Global-to-Shared Copy": each thread copies
// its own 16-byte row from global memory into shared memory asynchronously,
// waits for its copy group, synchronizes the block, then reads the next
// thread's row. Here: one workgroup of ceil(rows/64) waves; lane i's row lands
// at LDS byte 16*i by a direct-to-LDS load; vmcnt(0) (the lane's own copies are
// complete) then s_barrier (every other wave's copies are complete too: a
// barrier alone would not wait for outstanding copies) before the exchange.
// The whole input is in LDS before anything is written, so b == a works.
#include "tp_engine.hpp"
#include "tp_internal.hpp"

namespace tp {
namespace dev {

template <bool LX4, bool SX4>
__global__ void __launch_bounds__(1024) row_shift_kernel(RowShiftParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const uint32_t rows = (uint32_t)p.rows;
    const uint32_t tid = threadIdx.x;
    const uint32_t wave_first = uniform(tid & ~63u);
    const uint32_t ring = uniform(lds_offset(lds));
    const BufferRes ra = make_buffer_res(p.a, rows * 16);
    const BufferRes rb = make_buffer_res(p.b, rows * 16);

    if constexpr (LX4) {
        dma_b128(ra, tid * 16, uniform(ring + wave_first * 16));
    } else {
        // 4-byte fallback: the wave's 64 rows are 256 floats, four loads per lane
        static_for<0, 4>([&](auto q) {
            const uint32_t e0 = wave_first * 4 + q * 64;
            dma_b32(ra, (e0 + (tid - wave_first)) * 4, uniform(ring + e0 * 4));
        });
    }
    vm_wait<0>();
    block_sync();

    if constexpr (SX4) {
        const uint32_t src = tid + 1 < rows ? tid + 1 : 0;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + src * 16);
        store_b128(rb, tid * 16, v);
    } else {
        static_for<0, 4>([&](auto q) {
            const uint32_t e = wave_first * 4 + q * 64 + (tid - wave_first);
            const uint32_t r = e / 4;
            const uint32_t src = r + 1 < rows ? r + 1 : 0;
            const uint32_t v = *reinterpret_cast<const uint32_t *>(lds + src * 16 + (e % 4) * 4);
            store_b32(rb, e * 4, v);
        });
    }
}

}  // namespace dev

int launch_row_shift(const tp_plan &plan, const RowShiftParams &p, void *stream)
{
    using Fn = void (*)(RowShiftParams);
    static constexpr Fn table[4] = {
        &dev::row_shift_kernel<true, true>, &dev::row_shift_kernel<false, true>,
        &dev::row_shift_kernel<true, false>, &dev::row_shift_kernel<false, false>};
    RowShiftParams args = p;
    void *kargs[] = {&args};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(table[plan.path]), dim3(1),
                                dim3((uint32_t)plan.threads), kargs, (size_t)plan.lds_bytes,
                                (hipStream_t)stream);
}

}  // namespace tp
