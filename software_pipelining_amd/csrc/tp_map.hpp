// Software-pipelined tiled map: out[i] = op(in[i]).
//
// A workgroup streams its run of consecutive tiles through an LDS ring of S
// slots with the stage loop of tp_pipeline.hpp ("Asynchronous Data Movement",
// section "Double buffering"); this file supplies what one tile is: where its
// bytes live in global memory and in its slot, how the lanes split it, and
// the op applied between the LDS read and the store.
//
// Layout: a tile is tile_elems contiguous floats of global memory and sits
// contiguously in its LDS slot. With the 16-byte path, lane `tid` moves chunk
// i*threads + tid (i < L) of the tile; with the 4-byte fallback it moves float
// i*threads + tid (i < 4L). Loads and stores choose their width
// independently. The 16-byte accesses need only 4-byte alignment; the host
// starts the body at out's first 128-byte line boundary, so its stores fill
// whole lines.
#pragma once

#include <array>
#include <utility>

#include "tp_engine.hpp"
#include "tp_internal.hpp"
#include "tp_pipeline.hpp"

namespace tp {
namespace dev {

template <int OP>
struct MapOp;

template <>
struct MapOp<TP_OP_SCALE2> {
    template <int N>
    TP_HD __forceinline__ static void apply(float (&v)[N], const float *)
    {
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = v[i] * 2.0f;
    }
};

template <>
struct MapOp<TP_OP_COPY> {
    template <int N>
    TP_HD __forceinline__ static void apply(float (&)[N], const float *) {}
};

// y = 0; y = fma(y, x, c_k) for k = 0..31. The N elements of a lane form N
// independent chains, interleaved so consecutive FMAs do not depend on each
// other.
template <>
struct MapOp<TP_OP_HORNER32> {
    template <int N>
    TP_HD __forceinline__ static void apply(float (&v)[N], const float *c)
    {
        float y[N];
#pragma unroll
        for (int i = 0; i < N; ++i)
            y[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const float ck = c[k];
#pragma unroll
            for (int i = 0; i < N; ++i)
                y[i] = __builtin_fmaf(y[i], v[i], ck);
        }
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = y[i];
    }
};

TP_HD __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }

// `count` (at most 64) floats outside the body's whole 16-byte chunks, moved
// element-wise by one wave: lane l loads src[l] into the LDS area at byte
// offset `area_off` of the workgroup's LDS (lanes past `count` are out of
// range: they move nothing and store nothing), waits for its own copy, applies
// the op and stores dst[l].
template <int OP, class E>
TP_HD __forceinline__ void map_edge(const E &e, const float *src, float *dst, uint32_t count,
                                    uint32_t area_off, uint32_t lane, const float *coef)
{
    const auto ri = e.res(src, count * 4);
    const auto ro = e.res(dst, count * 4);
    e.dma_b32(ri, lane * 4, e.uniform(e.lds_base() + area_off));
    e.template wait<0>();
    float v[1] = {e.template lds_load<float>(area_off + lane * 4)};
    MapOp<OP>::apply(v, coef);
    e.store_b32(ro, lane * 4, f2u(v[0]));
}

// The kernel body, written against an engine (tp_engine.hpp).
template <class E, int OP, int S, int L, bool LX4, bool SX4>
TP_HD __forceinline__ void map_body(const E &e, const MapParams &p)
{
    constexpr int LD = map_loads_per_tile(LX4, L);
    constexpr int ST = map_stores_per_tile(SX4, L);

    const uint32_t nt = e.nthreads();
    const uint32_t tid = e.tid();
    const uint32_t wave_first = e.uniform(tid & ~63u);
    const uint32_t tile_bytes = nt * L * 16;
    const int64_t tile_elems = (int64_t)nt * L * 4;

    // This workgroup's run: tiles [b T, (b + 1) T) of the input, tile j at
    // byte j * tile_bytes of the resource window [base, base + span).
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

    // Producer: copy tile j of the run into the LDS slot at byte address `slot`.
    auto issue = [&](uint32_t j, uint32_t slot) TP_INLINE {
        const uint32_t toff = j * tile_bytes;
        if constexpr (LX4) {
            static_for<0, L>([&](auto i) TP_INLINE {
                e.dma_b128(rin, toff + (i * nt + tid) * 16, e.uniform(slot + (i * nt + wave_first) * 16));
            });
        } else {
            static_for<0, 4 * L>([&](auto i) TP_INLINE {
                e.dma_b32(rin, toff + (i * nt + tid) * 4, e.uniform(slot + (i * nt + wave_first) * 4));
            });
        }
    };

    // Consumer: tile j from the slot at LDS byte offset `slot_off` -> op -> store.
    auto consume = [&](uint32_t j, uint32_t slot_off) TP_INLINE {
        const uint32_t toff = j * tile_bytes;
        float v[4 * L];
        if constexpr (SX4) {
            static_for<0, L>([&](auto i) TP_INLINE {
                const f32x4 x = e.template lds_load<f32x4>(slot_off + (i * nt + tid) * 16);
                v[4 * i + 0] = x.x;
                v[4 * i + 1] = x.y;
                v[4 * i + 2] = x.z;
                v[4 * i + 3] = x.w;
            });
            MapOp<OP>::apply(v, p.coef);
            static_for<0, L>([&](auto i) TP_INLINE {
                const u32x4 o = {f2u(v[4 * i]), f2u(v[4 * i + 1]), f2u(v[4 * i + 2]), f2u(v[4 * i + 3])};
                e.store_b128(rout, toff + (i * nt + tid) * 16, o);
            });
        } else {
            static_for<0, 4 * L>([&](auto i) TP_INLINE {
                v[i] = e.template lds_load<float>(slot_off + (i * nt + tid) * 4);
            });
            MapOp<OP>::apply(v, p.coef);
            static_for<0, 4 * L>([&](auto i) TP_INLINE { e.store_b32(rout, toff + (i * nt + tid) * 4, f2u(v[i])); });
        }
    };

    if (cnt > 0)
        pipeline_run<S, LD, ST, map_wave_local(LX4, SX4)>(e, cnt, ring, tile_bytes, issue, consume);

    // The floats outside the body's whole 16-byte chunks, moved element-wise
    // by the first wave through an LDS area of its own: the 0-31 floats before
    // the body (workgroup 0) and the body's final partial chunk (the last
    // workgroup; both when there is one workgroup).
    if (wave_first == 0) {
        const uint32_t edge_off = S * tile_bytes;
        if (b == 0 && p.head > 0)
            map_edge<OP>(e, p.in - p.head, p.out - p.head, (uint32_t)p.head, edge_off, tid, p.coef);
        if (b == e.blocks() - 1 && p.n > p.n_main)
            map_edge<OP>(e, p.in + p.n_main, p.out + p.n_main, (uint32_t)(p.n - p.n_main), edge_off,
                         tid, p.coef);
    }
    // No copy into LDS is in flight here: pipeline_run retires its last load
    // before it returns, and each edge pass waits for its own.
}

template <int OP, int S, int L, bool LX4, bool SX4>
__global__ void __launch_bounds__(256) map_kernel(MapParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    map_body<GpuEngine, OP, S, L, LX4, SX4>(TP_GPU_ENGINE(lds), p);
}

// Kernel table of one op over stage counts SLO..SHI:
// index ((S - SLO) * 4 + log2 L) * 4 + path.
using MapKernelFn = void (*)(MapParams);

template <int OP, int SLO, int I>
constexpr MapKernelFn map_entry()
{
    constexpr int path = I % 4;
    constexpr int L = 1 << ((I / 4) % 4);
    constexpr int S = SLO + I / 16;
    return &map_kernel<OP, S, L, !(path & TP_PATH_SCALAR_LOAD), !(path & TP_PATH_SCALAR_STORE)>;
}

template <int OP, int SLO, int... I>
constexpr std::array<MapKernelFn, sizeof...(I)> map_table(std::integer_sequence<int, I...>)
{
    return {map_entry<OP, SLO, I>()...};
}

constexpr int lane_chunks_index(int lane_chunks)
{
    return lane_chunks == 1 ? 0 : lane_chunks == 2 ? 1 : lane_chunks == 4 ? 2 : 3;
}

// Launch a kernel of `fn`'s signature with the plan's grid, block and LDS.
template <class Fn, class Params>
int launch_planned(Fn fn, const tp_plan &plan, const Params &p, void *stream)
{
    if (plan.lds_bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 plan.lds_bytes);
        if (e != hipSuccess)
            return (int)e;
    }
    Params args = p;
    void *kargs[] = {&args};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((uint32_t)plan.grid),
                                dim3((uint32_t)plan.threads), kargs, (size_t)plan.lds_bytes,
                                (hipStream_t)stream);
}

template <int OP, int SLO, int SHI>
int launch_map_stages(const tp_plan &plan, const MapParams &p, void *stream)
{
    static constexpr auto table = map_table<OP, SLO>(std::make_integer_sequence<int, (SHI - SLO + 1) * 16>{});
    const int i = ((plan.stages - SLO) * 4 + lane_chunks_index(plan.lane_chunks)) * 4 + plan.path;
    return launch_planned(table[i], plan, p, stream);
}

}  // namespace dev
}  // namespace tp
