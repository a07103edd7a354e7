// Software-pipelined tiled map with a producer/consumer role split:
// out[i] = op(in[i]).
//
// The pages name two roles around a pipeline: a producer that acquires a
// stage, starts its copies and commits them, and consumers that wait for a
// stage, use it and release it ("Asynchronous Data Movement", section
// "Barriers and pipelines"; "CUDA Async Copy and Pipeline Guide", section
// "Optimization Techniques"). Here the roles go to whole waves of one
// workgroup: the last wave only issues LDS-DMA loads, for every chunk of every
// tile, and the other C waves only read tiles from LDS, compute and store.
//
// One workgroup barrier per iteration is both hand-offs:
//   producer  prologue: issue tiles 0 .. S-2 into slots 0 .. S-2
//             iteration t: wait vmcnt((S-2) * loads per tile)   tile t landed
//                          barrier                              (commit / release)
//                          issue tile t+S-1 into slot (t-1) mod S
//   consumers iteration t: barrier                              (wait / release)
//                          read tile t from slot t mod S, apply op, store
// The barrier of iteration t follows the producer's wait for tile t and each
// consumer's use of tile t-1, so it publishes tile t and frees the slot the
// producer refills next. With S = 1 the producer loads, waits and meets the
// consumers at a barrier, and a second barrier frees the single slot.
//
// The producer issues no stores, so its wait count is (S-2) x its loads per
// tile in every iteration. As in the uniform schedule, tiles past the run's
// end are still issued as out-of-range loads that move nothing, which keeps
// that count fixed; the producer drains them before it ends. Every wave takes
// the same number of barriers, and no wave spins on a flag.
//
// Layout is that of the uniform schedule: a tile of TILE floats sits
// contiguously in its slot; consumer lane tid reads chunk i*NC + tid (i < L),
// or float i*NC + tid with 4-byte stores; producer lane l loads chunk k*64 + l
// (k < C*L), or float k*64 + l with 4-byte loads.
#pragma once

#include "tp_map.hpp"

namespace tp {
namespace dev {

template <int TILE>
struct SplitGeometry {
    static constexpr int NC = TILE / 4 < 256 ? TILE / 4 : 256;  // consumer threads
    static constexpr int C = NC / 64;                           // consumer waves
    static constexpr int L = TILE / (4 * NC);                   // 16-byte chunks per consumer lane
};

// The kernel body, written against an engine (tp_engine.hpp).
template <class E, int OP, int S, int TILE, bool LX4, bool SX4>
TP_HD __forceinline__ void map_split_body(const E &e, const MapParams &p)
{
    using G = SplitGeometry<TILE>;
    constexpr int NC = G::NC;
    constexpr int L = G::L;
    constexpr int LDP = LX4 ? G::C * L : 4 * G::C * L;   // producer loads per tile
    constexpr uint32_t tile_bytes = TILE * 4;
    constexpr int64_t tile_elems = TILE;

    const uint32_t tid = e.tid();
    const uint32_t wave_first = e.uniform(tid & ~63u);
    const bool producer = wave_first >= (uint32_t)NC;

    // This workgroup's run: tiles [b T, (b + 1) T), as in the uniform schedule.
    const uint32_t b = e.block();
    const int64_t run_first = (int64_t)b * p.tiles_per_block * tile_elems;
    const int64_t rem = p.n_main - run_first;
    const int64_t run_bytes = (int64_t)p.tiles_per_block * tile_bytes;
    const uint32_t span = rem <= 0 ? 0u : (uint32_t)(rem * 4 < run_bytes ? rem * 4 : run_bytes);
    const int64_t base = rem > 0 ? run_first : 0;
    const int cnt = (int)((span + tile_bytes - 1) / tile_bytes);
    const auto rin = e.res(p.in + base, span);
    const auto rout = e.res(p.out + base, span);
    const uint32_t ring = e.uniform(e.lds_base());

    // Producer: every chunk of tile j into the LDS slot at byte address `slot`.
    auto issue = [&](uint32_t j, uint32_t slot) TP_INLINE {
        const uint32_t toff = j * tile_bytes;
        const uint32_t pl = tid - NC;
        if constexpr (LX4) {
            static_for<0, LDP>([&](auto k) TP_INLINE {
                e.dma_b128(rin, toff + (k * 64 + pl) * 16, e.uniform(slot + k * 64 * 16));
            });
        } else {
            static_for<0, LDP>([&](auto k) TP_INLINE {
                e.dma_b32(rin, toff + (k * 64 + pl) * 4, e.uniform(slot + k * 64 * 4));
            });
        }
    };

    // Consumer: tile j from the slot at LDS byte offset `slot_off` -> op -> store.
    auto consume = [&](uint32_t j, uint32_t slot_off) TP_INLINE {
        const uint32_t toff = j * tile_bytes;
        float v[4 * L];
        if constexpr (SX4) {
            static_for<0, L>([&](auto i) TP_INLINE {
                const f32x4 x = e.template lds_load<f32x4>(slot_off + (i * NC + tid) * 16);
                v[4 * i + 0] = x.x;
                v[4 * i + 1] = x.y;
                v[4 * i + 2] = x.z;
                v[4 * i + 3] = x.w;
            });
            MapOp<OP>::apply(v, p.coef);
            static_for<0, L>([&](auto i) TP_INLINE {
                const u32x4 o = {f2u(v[4 * i]), f2u(v[4 * i + 1]), f2u(v[4 * i + 2]), f2u(v[4 * i + 3])};
                e.store_b128(rout, toff + (i * NC + tid) * 16, o);
            });
        } else {
            static_for<0, 4 * L>([&](auto i) TP_INLINE {
                v[i] = e.template lds_load<float>(slot_off + (i * NC + tid) * 4);
            });
            MapOp<OP>::apply(v, p.coef);
            static_for<0, 4 * L>([&](auto i) TP_INLINE { e.store_b32(rout, toff + (i * NC + tid) * 4, f2u(v[i])); });
        }
    };

    if (cnt > 0) {
        if (producer) {
            if constexpr (S == 1) {
                for (int t = 0; t < cnt; ++t) {
                    issue(t, ring);
                    e.template wait<0>();
                    e.barrier();   // tile t is in LDS
                    e.barrier();   // the consumers are done with it
                }
            } else {
                static_for<0, S - 1>([&](auto s) TP_INLINE { issue(s, ring + s * tile_bytes); });
                uint32_t nxt = S - 1;  // slot of tile t + S - 1
                for (int t = 0; t < cnt; ++t) {
                    e.template wait<stage_wait_count(S, LDP, 0, 0)>();
                    e.barrier();
                    issue(t + S - 1, ring + nxt * tile_bytes);
                    nxt = nxt + 1 == S ? 0 : nxt + 1;
                }
            }
            e.template wait<0>();   // the loads issued past the run's end
        } else {
            uint32_t cur = 0;  // slot of tile t
            for (int t = 0; t < cnt; ++t) {
                e.barrier();
                consume(t, cur * tile_bytes);
                if constexpr (S == 1)
                    e.barrier();
                cur = cur + 1 == S ? 0 : cur + 1;
            }
        }
    }

    // The floats outside the body's whole 16-byte chunks (before the body and
    // its final partial chunk), moved by the first consumer wave as in the
    // uniform schedule.
    if (wave_first == 0) {
        const uint32_t edge_off = S * tile_bytes;
        if (b == 0 && p.head > 0)
            map_edge<OP>(e, p.in - p.head, p.out - p.head, (uint32_t)p.head, edge_off, tid, p.coef);
        if (b == e.blocks() - 1 && p.n > p.n_main)
            map_edge<OP>(e, p.in + p.n_main, p.out + p.n_main, (uint32_t)(p.n - p.n_main), edge_off,
                         tid, p.coef);
    }
}

template <int OP, int S, int TILE, bool LX4, bool SX4>
__global__ void __launch_bounds__(320) map_split_kernel(MapParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    map_split_body<GpuEngine, OP, S, TILE, LX4, SX4>(TP_GPU_ENGINE(lds), p);
}

// Kernel table of one op over stage counts SLO..SHI:
// index ((S - SLO) * 6 + log2(tile / 256)) * 4 + path.
template <int OP, int SLO, int I>
constexpr MapKernelFn map_split_entry()
{
    constexpr int path = I % 4;
    constexpr int TILE = 256 << ((I / 4) % 6);
    constexpr int S = SLO + I / 24;
    return &map_split_kernel<OP, S, TILE, !(path & TP_PATH_SCALAR_LOAD), !(path & TP_PATH_SCALAR_STORE)>;
}

template <int OP, int SLO, int... I>
constexpr std::array<MapKernelFn, sizeof...(I)> map_split_table(std::integer_sequence<int, I...>)
{
    return {map_split_entry<OP, SLO, I>()...};
}

template <int OP, int SLO, int SHI>
int launch_map_split_stages(const tp_plan &plan, const MapParams &p, void *stream)
{
    static constexpr auto table =
        map_split_table<OP, SLO>(std::make_integer_sequence<int, (SHI - SLO + 1) * 6 * 4>{});
    int ti = 0;
    while ((256 << ti) < plan.tile_units)
        ++ti;
    return launch_planned(table[((plan.stages - SLO) * 6 + ti) * 4 + plan.path], plan, p, stream);
}

}  // namespace dev
}  // namespace tp
