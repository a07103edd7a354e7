// Copies between workgroups: the kernel bodies, written against an engine
// (tp_engine.hpp on the GPU, tests/emu on the host).
//
// The pages let one group of a cluster copy a chunk of its shared memory into
// another group's shared memory; the receiver waits until the expected bytes
// have arrived before it reads them, and both stay until the transfer is done
// ("Asynchronous Copies", section "Copies between CTAs"). CDNA4 has no
// clusters and no way to address another workgroup's LDS, so the chunk goes
// through a staging slot in memory the two share:
//   workgroup k   copies chunk k of src into its LDS (LDS-DMA) and waits for
//                 it; if k + 1 < n it stores the LDS bytes into staging slot
//                 k at device scope, waits until those stores have completed
//                 and sets flags[k] (a device-scope store);
//   workgroup k   (k >= 1) polls flags[k - 1] at device scope; once it is set,
//                 copies staging slot k - 1 into its LDS with device-scope
//                 LDS-DMA loads, waits, and stores those bytes as chunk k of
//                 dst.
// (tp_engine.hpp explains why device-scope accesses and these waits order the
// hand-off across XCDs.)
// A workgroup only ever waits for the one numbered just below it. Workgroups
// are dispatched in order of their index, so the lowest one not yet finished
// is running or has room to start, and the chain always moves. The wait is
// still bounded: after spin_limit polls the receiver gives up, sets the status
// word and writes nothing, and a receiver that sees the status set stops
// waiting too, so every wave ends whatever happens. Each staging slot is used
// once per call; the flags and the status start at zero (the clearing kernel
// runs first on the same stream).
#pragma once

#include "tp_engine.hpp"
#include "tp_internal.hpp"

namespace tp {
namespace dev {

// Zero flags [0, n) and the status word: workgroups of kWgClearThreads lanes,
// one flag word per lane.
template <class E>
TP_HD __forceinline__ void workgroup_copy_clear_body(const E &e, const WgCopyParams &p)
{
    const uint32_t tid = e.tid();
    const int64_t first = (int64_t)e.block() * kWgClearThreads;
    const int64_t left = p.n_chunks - first;
    const uint32_t count = (uint32_t)(left < kWgClearThreads ? left : kWgClearThreads);
    const auto rflags = e.res(p.flags + first, count * 4);
    e.store_b32(rflags, tid * 4, 0u);
    if (e.block() == 0) {
        const auto rstatus = e.res(p.status, 4);
        e.store_b32(rstatus, tid == 0 ? 0u : 4u, 0u);
    }
}

// One 64-lane workgroup per chunk; lane l moves bytes [4l, 4l + 4) of it.
// LDS: the own chunk at [0, 256), the received one at [256, 512).
template <class E>
TP_HD __forceinline__ void workgroup_copy_body(const E &e, const WgCopyParams &p)
{
    const uint32_t lane = e.tid();
    const int64_t k = e.block();
    const uint32_t base = e.uniform(e.lds_base());
    const uint32_t off = lane * 4;

    const auto rsrc = e.res(p.src + kWgChunkBytes * k, kWgChunkBytes);
    e.dma_b32(rsrc, off, base);
    e.template wait<0>();

    if (k + 1 < p.n_chunks) {             // send chunk k to workgroup k + 1
        const auto rstage = e.res(p.stage + kWgChunkBytes * k, kWgChunkBytes);
        e.store_b32_device(rstage, off, e.template lds_load<uint32_t>(off));
        e.template wait<0>();             // the staged bytes are written before the flag
        const auto rflag = e.res(p.flags + k, 4);
        e.store_b32_device(rflag, lane == 0 ? 0u : 4u, 1u);
    }

    if (k >= 1) {                         // receive chunk k - 1 from workgroup k - 1
        const auto rflag = e.res(p.flags + (k - 1), 4);
        const auto rstatus = e.res(p.status, 4);
        uint32_t got = 0, stop = 0;
        for (uint32_t i = 0; i < p.spin_limit; ++i) {
            got = e.uniform(e.load_b32_device(rflag, 0));
            if (got)
                break;
            stop = e.uniform(e.load_b32_device(rstatus, 0));
            if (stop)
                break;
            e.pause();
        }
        if (got) {
            const auto rstage = e.res(p.stage + kWgChunkBytes * (k - 1), kWgChunkBytes);
            e.dma_b32_device(rstage, off, e.uniform(base + kWgChunkBytes));
            e.template wait<0>();
            const auto rdst = e.res(p.dst + kWgChunkBytes * k, kWgChunkBytes);
            e.store_b32(rdst, off, e.template lds_load<uint32_t>(kWgChunkBytes + off));
        } else if (!stop) {
            const auto rstatus_w = e.res(p.status, 4);
            e.store_b32_device(rstatus_w, lane == 0 ? 0u : 4u, 1u);   // gave up waiting
        }
    }
    // no copy into LDS is in flight when the workgroup ends
    e.template wait<0>();
}

}  // namespace dev
}  // namespace tp
