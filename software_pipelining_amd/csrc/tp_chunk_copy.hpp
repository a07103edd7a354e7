// Predicated chunk copy through the LDS copy pipeline, for chunks of W = 16
// bytes and, with the same schedule, W = 8 and 4 bytes.
//
// This header holds the kernel body, written against an engine: the gfx950
// engine of tp_engine.hpp, or the CPU emulator in tests/emu that compiles the
// same body.
//
// Semantics ("Asynchronous Copies", section "A Global-to-Shared Copy", the
// paragraph on the copy's operands): a false pred skips the copy and leaves
// the destination unchanged; src_size copies a byte prefix and zero-fills the
// rest; ignore_src zero-fills the whole chunk. The copy itself is skipped
// whenever it would bring no byte that survives (pred false, ignore_src set,
// or src_size 0): those lanes get the first out-of-range offset (the end of
// the workgroup's run), so the load moves nothing, while the instruction still
// issues and the wait counts hold.
//
// One lane owns one chunk of a 256-chunk tile. Per tile, each wave issues
//   three 1-byte LDS-DMA loads (pred, src_size, ignore_src of its 64 chunks)
//   one 16-byte LDS-DMA load of its 64 chunks (W = 16 with a 16-byte-aligned
//   source), or else W/4 4-byte loads covering the wave's 64 * W bytes, word
//   after word, so every chunk lands contiguously at LDS byte tid * W
// and on consumption reads its chunk and the three bytes back from LDS,
// zeroes the bytes past the prefix and stores W bytes, with the store's
// offset out of range when pred is false, so the destination is never
// written there. A 16-byte store writes the lane's chunk whole. Word stores
// (8-byte chunks, or a destination that is not 16-byte aligned) are laid out
// across the wave instead: each lane writes its masked chunk back over its own
// LDS bytes, and store q then writes word q * 64 + lane of the wave's
// 64 * W / 4 words, so every store instruction covers whole 64-byte blocks
// except where pred is false (a lane storing its own chunk's words would
// leave every instruction's blocks partly written, and the memory side serves
// such masked writes much more slowly). Everything a lane reads from LDS was
// loaded or written by its own wave, so the per-wave vmcnt wait is the whole
// synchronization; no workgroup barrier is needed.
//
// Schedule (S data slots, 2S-1 metadata slots). A run of at most S-1 tiles
// fits the prologue: the metadata of every tile of the run, a wait, the data
// of every tile, a wait, then every tile is consumed; nothing is issued past
// the run. A longer run is pipelined: a tile's metadata is loaded S-1
// iterations before its data, in the same issue group as the data of an
// earlier tile. Because loads retire in order, the wait for tile t's data
// also guarantees that the metadata of tile t+S-1, needed to mask that tile's
// data load in the same iteration, has landed.
//   prologue: meta 0 .. S-2; wait for all; then groups g = 0 .. S-2:
//             {meta g+S-1, data g}
//   iteration t: wait (data t landed)
//                issue group {meta t+2S-2, data t+S-1 masked by meta t+S-1}
//                consume t (meta t, data t)
#pragma once

#include "tp_engine.hpp"
#include "tp_internal.hpp"

namespace tp {
namespace dev {

template <class E, int S, int W, bool LX4, bool SX4>
TP_HD __forceinline__ void chunk_copy_body(const E &e, const ChunkParams &p)
{
    static_assert(W == 16 || ((W == 8 || W == 4) && !LX4 && !SX4), "narrow chunks move as words");
    constexpr int R = chunk_meta_slots(S);
    constexpr int LD = chunk_loads_per_tile(LX4, W);
    constexpr int ST = chunk_stores_per_tile(SX4, W);
    constexpr int WPC = W / 4;                        // words per chunk
    constexpr uint32_t kData = chunk_data_slot_bytes(W);   // 256 chunks per data slot
    constexpr uint32_t kMeta = kChunkMetaSlotBytes;   // 3 KiB per metadata slot

    const uint32_t tid = e.tid();
    const uint32_t wave_first = e.uniform(tid & ~63u);
    const uint32_t lane = tid - wave_first;
    const int64_t first = (int64_t)e.block() * p.tiles_per_block * kChunkTile;
    const int64_t rem = p.n_chunks - first;
    const int64_t run = (int64_t)p.tiles_per_block * kChunkTile;
    const uint32_t span = (uint32_t)(rem < run ? rem : run);   // chunks of this workgroup
    const int cnt = (int)((span + kChunkTile - 1) / kChunkTile);
    const bool has_pred = p.flags & kHasPred;
    const bool has_size = p.flags & kHasSize;
    const bool has_ign = p.flags & kHasIgnore;

    const uint32_t run_end = span * W;            // first out-of-range byte of src/dst
    const auto rsrc = e.res(p.src + W * first, run_end);
    const auto rdst = e.res(p.dst + W * first, run_end);
    // An absent metadata array still gets its loads issued (so counts stay
    // fixed); they read the run's own source bytes, and those LDS bytes are
    // ignored.
    const uint8_t *src_run = p.src + W * first;
    const auto rpred = e.res(has_pred ? p.pred + first : src_run, span);
    const auto rsize = e.res(has_size ? p.src_size + first : src_run, span);
    const auto rign = e.res(has_ign ? p.ignore_src + first : src_run, span);

    const uint32_t base = e.uniform(e.lds_base());
    const uint32_t data_ring = 0;                 // offsets from the start of the LDS
    const uint32_t meta_ring = S * kData;
    // metadata slot layout: [wave][array][64 lanes x 4 bytes]
    const uint32_t meta_wave = wave_first * 12;   // = (wave_first / 64) * 768

    auto issue_meta = [&](uint32_t j, uint32_t mslot) TP_INLINE {
        const uint32_t voff = j * kChunkTile + tid;
        const uint32_t m0 = base + meta_ring + mslot * kMeta + meta_wave;
        e.dma_u8(rpred, voff, e.uniform(m0));
        e.dma_u8(rsize, voff, e.uniform(m0 + 256));
        e.dma_u8(rign, voff, e.uniform(m0 + 512));
    };

    // Effective byte count of the lane's chunk (0..W) and whether it is stored.
    struct Meta {
        uint32_t keep;
        bool store;
    };
    auto read_meta = [&](uint32_t mslot) TP_INLINE {
        const uint32_t m = meta_ring + mslot * kMeta + meta_wave + lane * 4;
        const bool pr = has_pred ? e.template lds_load<uint8_t>(m) != 0 : true;
        const bool ig = has_ign ? e.template lds_load<uint8_t>(m + 512) != 0 : false;
        uint32_t s = has_size ? e.template lds_load<uint8_t>(m + 256) : (uint32_t)W;
        s = s > (uint32_t)W ? (uint32_t)W : s;
        return Meta{ig ? 0u : s, pr};
    };

    auto issue_data = [&](uint32_t j, uint32_t dslot, uint32_t mslot) TP_INLINE {
        const uint32_t slot = base + data_ring + dslot * kData;
        if constexpr (LX4) {
            const Meta m = read_meta(mslot);
            const bool needed = m.store && m.keep != 0;
            e.dma_b128(rsrc, needed ? j * kData + tid * 16 : run_end, e.uniform(slot + wave_first * 16));
        } else {
            static_for<0, WPC>([&](auto q) TP_INLINE {
                const uint32_t w0 = wave_first * WPC + q * 64;   // first word of this load
                e.dma_b32(rsrc, j * kData + (w0 + lane) * 4, e.uniform(slot + w0 * 4));
            });
        }
    };

    auto consume = [&](uint32_t j, uint32_t dslot, uint32_t mslot) TP_INLINE {
        const Meta m = read_meta(mslot);
        const uint32_t slot = data_ring + dslot * kData;
        u32x4 v;
        if constexpr (W == 16) {
            v = e.template lds_load<u32x4>(slot + tid * 16);
        } else {
            static_for<0, WPC>([&](auto w) TP_INLINE {
                v[(int)w] = e.template lds_load<uint32_t>(slot + tid * W + w * 4);
            });
        }
        // keep bytes [0, keep): word w keeps min(max(keep - 4w, 0), 4) bytes
#pragma unroll
        for (int w = 0; w < WPC; ++w) {
            const int kb = (int)m.keep - 4 * w;
            const uint32_t mask = kb >= 4 ? 0xFFFFFFFFu : kb <= 0 ? 0u : ((1u << (8 * kb)) - 1u);
            v[w] &= mask;
        }
        const uint32_t off = j * kData + tid * W;
        if constexpr (SX4) {
            e.store_b128(rdst, m.store ? off : run_end, v);
        } else if constexpr (WPC == 1) {
            e.store_b32(rdst, m.store ? off : run_end, v[0]);
        } else {
            // the masked chunk back over the lane's own bytes, then the
            // wave's words in order: word q * 64 + lane belongs to the wave's
            // chunk (q * 64 + lane) / WPC, whose pred decides the store
            if constexpr (W == 16) {
                e.template lds_store<u32x4>(slot + tid * 16, v);
            } else {
                static_for<0, WPC>([&](auto w) TP_INLINE {
                    e.template lds_store<uint32_t>(slot + tid * W + w * 4, v[(int)w]);
                });
            }
            const uint32_t wave_bytes = wave_first * W;   // the wave's chunks in the slot and in dst
            const uint32_t meta = meta_ring + mslot * kMeta + meta_wave;
            static_for<0, WPC>([&](auto q) TP_INLINE {
                const uint32_t wi = q * 64 + lane;
                const bool st = has_pred ? e.template lds_load<uint8_t>(meta + wi / WPC * 4) != 0
                                         : true;
                const uint32_t word = e.template lds_load<uint32_t>(slot + wave_bytes + wi * 4);
                e.store_b32(rdst, st ? j * kData + wave_bytes + wi * 4 : run_end, word);
            });
        }
    };

    if constexpr (S == 1) {
        for (int t = 0; t < cnt; ++t) {
            issue_meta(t, 0);
            e.template wait<0>();
            issue_data(t, 0, 0);
            e.template wait<0>();
            consume(t, 0, 0);
        }
    } else if (cnt <= S - 1) {
        // the whole run in the prologue: nothing is issued past its last tile
        static_for<0, S - 1>([&](auto m) TP_INLINE {
            if ((int)m < cnt)
                issue_meta(m, m);
        });
        e.template wait<0>();
        static_for<0, S - 1>([&](auto g) TP_INLINE {
            if ((int)g < cnt)
                issue_data(g, g, g);
        });
        e.template wait<0>();
        static_for<0, S - 1>([&](auto g) TP_INLINE {
            if ((int)g < cnt)
                consume(g, g, g);
        });
    } else {
        static_for<0, S - 1>([&](auto m) TP_INLINE { issue_meta(m, m); });
        e.template wait<0>();
        static_for<0, S - 1>([&](auto g) TP_INLINE {
            issue_meta(g + S - 1, g + S - 1);
            issue_data(g, g, g);
        });
        bool stop = false;
        static_for<0, S - 1>([&](auto T) TP_INLINE {
            if (!stop) {
                if ((int)T >= cnt) {
                    stop = true;
                } else {
                    e.template wait<stage_wait_count(S, LD, ST, T)>();
                    issue_meta(T + 2 * S - 2, (T + 2 * S - 2) % R);
                    issue_data(T + S - 1, (T + S - 1) % S, (T + S - 1) % R);
                    consume(T, T % S, T % R);
                }
            }
        });
        uint32_t dcur = (S - 1) % S;   // data slot of tile t
        uint32_t mcur = (S - 1) % R;   // metadata slot of tile t
        for (int t = S - 1; t < cnt; ++t) {
            const uint32_t dnxt = dcur == 0 ? S - 1 : dcur - 1;              // (t + S - 1) mod S
            const uint32_t mnxt = mcur + S - 1 >= R ? mcur + S - 1 - R : mcur + S - 1;  // (t + S - 1) mod R
            const uint32_t mfar = mcur == 0 ? R - 1 : mcur - 1;              // (t + 2S - 2) mod R
            e.template wait<stage_wait_count(S, LD, ST, S - 1)>();
            issue_meta(t + 2 * S - 2, mfar);
            issue_data(t + S - 1, dnxt, mnxt);
            consume(t, dcur, mcur);
            dcur = dcur + 1 == S ? 0 : dcur + 1;
            mcur = mcur + 1 == R ? 0 : mcur + 1;
        }
    }
    // No copy into LDS may still be in flight when the workgroup's LDS is freed.
    e.template wait<0>();
}

}  // namespace dev
}  // namespace tp
