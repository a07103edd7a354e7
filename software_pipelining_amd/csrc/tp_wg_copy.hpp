// Copies between workgroups: the kernel bodies, written against an engine
// (tp_engine.hpp on the GPU, tests/emu on the host).
//
// The pages let one group of a cluster copy a chunk of its shared memory into
// another group's shared memory; the receiver waits until the expected bytes
// have arrived before it reads them ("Asynchronous Copies", section "Copies
// between CTAs"). CDNA4 has no clusters and no way to address another
// workgroup's LDS, so the chunk goes through a staging slot in memory both
// can reach, and "the bytes have arrived" is read off the bytes themselves:
// every 4-byte word of the chunk travels with a 4-byte tag in one 8-byte
// device-scope access, which lands whole (tp_engine.hpp), so a word whose tag
// is set is the sender's word.
//   clearing      zeroes every staging slot and the status word;
//   workgroup k   copies chunk k of src into its LDS (LDS-DMA) and waits for
//                 it; if k + 1 < n each lane stores its word with the tag into
//                 staging slot k (no wait, no flag);
//   workgroup k   (k >= 1) loads slot k - 1, one tagged word per lane, until
//                 every lane's tag is set, puts the words into its LDS and
//                 stores them as chunk k of dst.
// A workgroup only ever waits for the one numbered just below it. Workgroups
// are dispatched in order of their index, so the lowest one not yet finished
// is running or has room to start, and the chain always moves; a sender
// never waits for anything but its own source load. The wait is still
// bounded: after spin_limit polls the receiver gives up, sets the status word
// and writes nothing, and a receiver that finds the status set (it looks
// every kWgStatusPollEvery polls) stops waiting too, so every wave ends
// whatever happens.
#pragma once

#include "tp_engine.hpp"
#include "tp_internal.hpp"

namespace tp {
namespace dev {

// Zero the n staging slots and the status word. Workgroups of kWgClearThreads
// lanes zero kWgClearSlotsPerPass slots (4 KiB, 16 bytes a lane) per pass and
// step over the slots by the grid.
template <class E>
TP_HD __forceinline__ void workgroup_copy_clear_body(const E &e, const WgCopyParams &p)
{
    constexpr int64_t kPassBytes = kWgClearSlotsPerPass * kWgSlotBytes;
    static_assert(kPassBytes == kWgClearThreads * 16, "one 16-byte store per lane and pass");
    const uint32_t tid = e.tid();
    const int64_t total = p.n_chunks * kWgSlotBytes;
    for (int64_t at = (int64_t)e.block() * kPassBytes; at < total;
         at += (int64_t)e.blocks() * kPassBytes) {
        const int64_t left = total - at;
        const auto rslots = e.res(p.stage + at, (uint32_t)(left < kPassBytes ? left : kPassBytes));
        e.store_b128(rslots, tid * 16, u32x4{0u, 0u, 0u, 0u});
    }
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
        const auto rslot = e.res(p.stage + kWgSlotBytes * k, kWgSlotBytes);
        const uint64_t word = (uint64_t)kWgTag << 32 | e.template lds_load<uint32_t>(off);
        e.store_b64_device(rslot, lane * 8, word);
    }

    if (k >= 1) {                         // receive chunk k - 1 from workgroup k - 1
        const auto rslot = e.res(p.stage + kWgSlotBytes * (k - 1), kWgSlotBytes);
        const auto rstatus = e.res(p.status, 4);
        uint64_t word = 0;
        bool got = false, stop = false;
        for (uint32_t i = 0; i < p.spin_limit; ++i) {
            word = e.load_b64_device(rslot, lane * 8);
            got = e.all_lanes((uint32_t)(word >> 32) == kWgTag);
            if (got)
                break;
            if (i % kWgStatusPollEvery == kWgStatusPollEvery - 1) {
                stop = e.uniform(e.load_b32_device(rstatus, 0)) != 0;
                if (stop)
                    break;
            }
            e.pause();
        }
        if (got) {
            e.template lds_store<uint32_t>(kWgChunkBytes + off, (uint32_t)word);
            const auto rdst = e.res(p.dst + kWgChunkBytes * k, kWgChunkBytes);
            e.store_b32(rdst, off, e.template lds_load<uint32_t>(kWgChunkBytes + off));
        } else if (!stop) {
            e.store_b32_device(rstatus, lane == 0 ? 0u : 4u, 1u);   // gave up waiting
        }
    }
}

}  // namespace dev
}  // namespace tp
