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
//
// This header holds the kernel body, written against an engine: the gfx950
// engine of tp_engine.hpp, or the CPU emulator in tests/emu.
#pragma once

#include "tp_engine.hpp"
#include "tp_internal.hpp"

namespace tp {
namespace dev {

// The kernel body, written against an engine (tp_engine.hpp).
template <class E, bool LX4, bool SX4>
TP_HD __forceinline__ void row_shift_body(const E &e, const RowShiftParams &p)
{
    const uint32_t rows = (uint32_t)p.rows;
    const uint32_t tid = e.tid();
    const uint32_t wave_first = e.uniform(tid & ~63u);
    const uint32_t ring = e.uniform(e.lds_base());
    const auto ra = e.res(p.a, rows * 16);
    const auto rb = e.res(p.b, rows * 16);

    if constexpr (LX4) {
        e.dma_b128(ra, tid * 16, e.uniform(ring + wave_first * 16));
    } else {
        // 4-byte fallback: the wave's 64 rows are 256 floats, four loads per lane
        static_for<0, 4>([&](auto q) TP_INLINE {
            const uint32_t e0 = wave_first * 4 + q * 64;
            e.dma_b32(ra, (e0 + (tid - wave_first)) * 4, e.uniform(ring + e0 * 4));
        });
    }
    e.template wait<0>();
    e.barrier();

    if constexpr (SX4) {
        const uint32_t src = tid + 1 < rows ? tid + 1 : 0;
        const u32x4 v = e.template lds_load<u32x4>(src * 16);
        e.store_b128(rb, tid * 16, v);
    } else {
        static_for<0, 4>([&](auto q) TP_INLINE {
            const uint32_t el = wave_first * 4 + q * 64 + (tid - wave_first);
            const uint32_t r = el / 4;
            const uint32_t src = r + 1 < rows ? r + 1 : 0;
            const uint32_t v = e.template lds_load<uint32_t>(src * 16 + (el % 4) * 4);
            e.store_b32(rb, el * 4, v);
        });
    }
}

}  // namespace dev
}  // namespace tp
