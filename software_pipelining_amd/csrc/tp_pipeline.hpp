// The stage loop shared by the pipelined kernels: a workgroup streams its
// run of `cnt` consecutive tiles through an LDS ring of S slots ("Asynchronous Data Movement", section "Double buffering": the
// first copy is issued before the loop, and each iteration issues the next
// stage's copy before waiting on the current one; S slots generalize the two
// buffers, the "N-buffering" of "CUDA Async Copy and Pipeline Guide", section
// "Optimization Techniques"). Two schedules, chosen by the load/store widths:
//
// Refill-first (loads and stores of the same width). Every lane reads back
// exactly the bytes it copied itself, so no wave needs another wave's data and
// the slot a wave has just consumed is free for that wave at once:
//   prologue   issue tiles 0 .. S-2 into slots 0 .. S-2
//   iteration t:
//     issue    tile t+S-1 into slot (t+S-1) mod S = (t-1) mod S   (just consumed)
//     wait     vmcnt(k_t): this wave's loads of tile t have landed
//     consume  read tile t from slot t mod S, apply op, store
// so all S slots are loading while the wave waits for tile t.
//
// Exchange (a 16-byte side and a 4-byte side: lanes read bytes other waves
// copied), the pages' protocol with a workgroup barrier:
//   prologue   issue tiles 0 .. S-2 into slots 0 .. S-2
//   iteration t:
//     wait     vmcnt(k_t): this wave's loads of tile t have landed  (consumer_wait)
//     barrier  every wave's part of tile t is visible; every wave has finished
//              reading slot (t-1) mod S in iteration t-1              (consumer_release)
//     issue    tile t+S-1 into slot (t-1) mod S                       (producer side)
//     consume  read tile t from slot t mod S, apply op, store
// so S-1 tiles are in flight while tile t is computed and stored; with S = 1
// it is the classic load -> barrier -> compute -> barrier ("Asynchronous Data
// Movement", opening paragraph).
//
// Tiles past the end of the workgroup's run are still "issued" as out-of-range
// loads that move no data: the count of memory instructions between tile t's
// loads and its wait is then the same for every t, and k_t is a compile-time
// immediate (the first S-1 iterations, whose loads were issued before any
// store, are peeled with their own smaller counts).
//
// The caller supplies the engine (tp_engine.hpp) and the tile: issue(j, slot_address) issues the LD loads of
// tile j into the slot at that LDS byte address (out-of-range loads for j past
// the run move nothing), and consume(j, slot_offset) reads tile j from the
// slot at that byte offset of the workgroup's LDS, computes and issues its ST
// stores. Every lane issues the same LD loads and ST stores per tile, whatever
// its data, so the wait counts are those of stage_wait_count.
#pragma once

#include "tp_engine.hpp"
#include "tp_internal.hpp"

namespace tp {
namespace dev {

// Runs the loop for cnt >= 1 tiles; on return no load issued here is still in
// flight (only the last tiles' stores may be), so the LDS may be released.
template <int S, int LD, int ST, bool WAVE_LOCAL, class E, class Issue, class Consume>
TP_HD __forceinline__ void pipeline_run(const E &e, int cnt, uint32_t ring, uint32_t slot_bytes,
                                        Issue &issue, Consume &consume)
{
    if constexpr (WAVE_LOCAL) {
        static_for<0, S - 1>([&](auto s) TP_INLINE { issue(s, ring + s * slot_bytes); });
        // Warm-up iterations 0 .. S-2 with their own wait counts (cnt >= 1, so
        // iteration 0 always runs). Every iteration issues before it stores,
        // so whichever iteration runs last leaves only its stores behind its
        // final load.
        static_for<0, S - 1>([&](auto T) TP_INLINE {
            if ((int)T == 0 || (int)T < cnt) {
                issue(T + S - 1, ring + ((T + S - 1) % S) * slot_bytes);
                e.template wait<stage_wait_count(S, LD, ST, T, true)>();
                consume(T, (T % S) * slot_bytes);
            }
        });
        // Byte offsets of the slots of tiles t and t - 1, carried from one
        // iteration to the next; tile t + S - 1 goes into tile t - 1's slot.
        // Kept as offsets (adds and a wrap, no multiply) so that they stay
        // scalar and M0 is set straight from them.
        uint32_t cur = ((S - 1) % S) * slot_bytes;
        uint32_t prev = ((2 * S - 2) % S) * slot_bytes;
        const uint32_t ring_bytes = S * slot_bytes;
        for (int t = S - 1; t < cnt; ++t) {
            issue(t + S - 1, ring + prev);
            e.template wait<stage_wait_count(S, LD, ST, S - 1, true)>();
            consume(t, cur);
            prev = cur;
            cur = cur + slot_bytes == ring_bytes ? 0 : cur + slot_bytes;
        }
    } else if constexpr (S == 1) {
        for (int t = 0; t < cnt; ++t) {
            issue(t, ring);
            e.template wait<0>();
            e.barrier();
            consume(t, 0);
            e.barrier();
        }
    } else {
        static_for<0, S - 1>([&](auto s) TP_INLINE { issue(s, ring + s * slot_bytes); });
        static_for<0, S - 1>([&](auto T) TP_INLINE {
            if ((int)T == 0 || (int)T < cnt) {    // cnt is uniform: every wave takes the barrier
                e.template wait<stage_wait_count(S, LD, ST, T)>();
                e.barrier();
                issue(T + S - 1, ring + ((T + S - 1) % S) * slot_bytes);
                consume(T, (T % S) * slot_bytes);
            }
        });
        uint32_t cur = ((S - 1) % S) * slot_bytes;        // as above
        uint32_t prev = ((2 * S - 2) % S) * slot_bytes;
        const uint32_t ring_bytes = S * slot_bytes;
        for (int t = S - 1; t < cnt; ++t) {
            e.template wait<stage_wait_count(S, LD, ST, S - 1)>();
            e.barrier();
            issue(t + S - 1, ring + prev);
            consume(t, cur);
            prev = cur;
            cur = cur + slot_bytes == ring_bytes ? 0 : cur + slot_bytes;
        }
    }
    // Operations retire in issue order and every path above ends with one
    // tile's ST stores issued after the last load, so at most ST outstanding
    // means every load has landed.
    e.template wait<ST>();
}

}  // namespace dev
}  // namespace tp
