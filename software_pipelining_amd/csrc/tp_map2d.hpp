// Strided 2-D map through the LDS pipeline:
//   dst[r * dst_stride + c] = op(src[r * src_stride + c]),  r < rows, c < cols.
//
// The tile is a box of box_rows x box_cols floats of a row-major matrix,
// described by a base, a shape and the row strides, as the pages describe a
// tensor tile transfer ("Asynchronous Data Movement", section "The Tensor
// Memory Accelerator"). CDNA4 has no engine that walks such a description, so
// the lanes of the workgroup do it: each lane turns its chunk (or float) of
// the box into a row and a column and issues an LDS-DMA buffer load from
// row * stride + column. The box sits in its LDS slot contiguously, row after
// row, exactly as a 1-D tile of box_rows * box_cols floats does, and the stage
// loop is the shared one (tp_pipeline.hpp).
//
// A workgroup owns a run of tiles_per_block boxes side by side in one band of
// box_rows rows. Its two buffer descriptors are rebased at the band's first
// element and cover exactly the band's rows up to the run's last column, so
// every offset fits 32 bits and an element past the matrix's last row or
// column, in an edge box, is given the descriptor's first out-of-range offset:
// its load moves nothing (the LDS gets zeros) and its store is dropped. Every
// lane still issues the same instructions per box, so the wait counts hold.
// With 16-byte accesses a chunk never straddles the matrix's last column
// (cols is a multiple of 4 on that path).
#pragma once

#include "tp_map.hpp"
#include "tp_pipeline.hpp"

namespace tp {
namespace dev {

// The kernel body, written against an engine (tp_engine.hpp).
template <class E, int OP, int S, int L, bool LX4, bool SX4>
TP_HD __forceinline__ void map2d_body(const E &e, const Map2dParams &p)
{
    constexpr int LD = map_loads_per_tile(LX4, L);
    constexpr int ST = map_stores_per_tile(SX4, L);

    const uint32_t nt = e.nthreads();
    const uint32_t tid = e.tid();
    const uint32_t wave_first = e.uniform(tid & ~63u);
    const uint32_t tile_bytes = nt * L * 16;
    const uint32_t bc_log2 = p.box_cols_log2;
    const uint32_t box_cols = 1u << bc_log2;
    const uint32_t box_rows = (nt * L * 4) >> bc_log2;

    // This workgroup's run: boxes [first_box, first_box + T) of band `band`.
    const uint32_t b = e.block();
    const uint32_t band = b / p.runs_per_band;
    const uint32_t first_box = (b - band * p.runs_per_band) * p.tiles_per_block;
    const int64_t r0 = (int64_t)band * box_rows;
    const int64_t c0 = (int64_t)first_box * box_cols;
    const int64_t rows_left = p.rows - r0;
    const int64_t cols_left = p.cols - c0;
    const int64_t run_cols = (int64_t)p.tiles_per_block * box_cols;
    const uint32_t rr = (uint32_t)(rows_left < box_rows ? rows_left : box_rows);    // >= 1
    const uint32_t cc = (uint32_t)(cols_left < run_cols ? cols_left : run_cols);    // >= 1
    const int cnt = (int)((cc + box_cols - 1) >> bc_log2);
    const uint32_t ss = (uint32_t)p.src_stride;
    const uint32_t ds = (uint32_t)p.dst_stride;
    const uint32_t src_end = ((rr - 1) * ss + cc) * 4;   // first out-of-range byte
    const uint32_t dst_end = ((rr - 1) * ds + cc) * 4;
    const auto rin = e.res(p.src + r0 * p.src_stride + c0, src_end);
    const auto rout = e.res(p.dst + r0 * p.dst_stride + c0, dst_end);
    const uint32_t ring = e.uniform(e.lds_base());

    // Element e of box j (row-major in the box, 4-aligned on the 16-byte
    // path): its byte offset in a descriptor with row stride `stride`, or
    // `end` when it lies outside the matrix.
    auto elem_offset = [&](uint32_t j, uint32_t e, uint32_t stride, uint32_t end) TP_INLINE {
        const uint32_t row = e >> bc_log2;
        const uint32_t col = (j << bc_log2) + (e & (box_cols - 1));
        return row < rr && col < cc ? (row * stride + col) * 4 : end;
    };

    auto issue = [&](uint32_t j, uint32_t slot) TP_INLINE {
        if constexpr (LX4) {
            static_for<0, L>([&](auto i) TP_INLINE {
                const uint32_t q = i * nt + tid;   // 16-byte chunk of the box
                e.dma_b128(rin, elem_offset(j, q * 4, ss, src_end), e.uniform(slot + (i * nt + wave_first) * 16));
            });
        } else {
            static_for<0, 4 * L>([&](auto i) TP_INLINE {
                const uint32_t f = i * nt + tid;   // float of the box
                e.dma_b32(rin, elem_offset(j, f, ss, src_end), e.uniform(slot + (i * nt + wave_first) * 4));
            });
        }
    };

    auto consume = [&](uint32_t j, uint32_t slot_off) TP_INLINE {
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
                e.store_b128(rout, elem_offset(j, (i * nt + tid) * 4, ds, dst_end), o);
            });
        } else {
            static_for<0, 4 * L>([&](auto i) TP_INLINE {
                v[i] = e.template lds_load<float>(slot_off + (i * nt + tid) * 4);
            });
            MapOp<OP>::apply(v, p.coef);
            static_for<0, 4 * L>([&](auto i) TP_INLINE {
                e.store_b32(rout, elem_offset(j, i * nt + tid, ds, dst_end), f2u(v[i]));
            });
        }
    };

    pipeline_run<S, LD, ST, map_wave_local(LX4, SX4)>(e, cnt, ring, tile_bytes, issue, consume);
}

template <int OP, int S, int L, bool LX4, bool SX4>
__global__ void __launch_bounds__(256) map2d_kernel(Map2dParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    map2d_body<GpuEngine, OP, S, L, LX4, SX4>(TP_GPU_ENGINE(lds), p);
}

// Kernel table of one op over stage counts SLO..SHI:
// index ((S - SLO) * 4 + log2 L) * 4 + path.
using Map2dKernelFn = void (*)(Map2dParams);

template <int OP, int SLO, int I>
constexpr Map2dKernelFn map2d_entry()
{
    constexpr int path = I % 4;
    constexpr int L = 1 << ((I / 4) % 4);
    constexpr int S = SLO + I / 16;
    return &map2d_kernel<OP, S, L, !(path & TP_PATH_SCALAR_LOAD), !(path & TP_PATH_SCALAR_STORE)>;
}

template <int OP, int SLO, int... I>
constexpr std::array<Map2dKernelFn, sizeof...(I)> map2d_table(std::integer_sequence<int, I...>)
{
    return {map2d_entry<OP, SLO, I>()...};
}

template <int OP, int SLO, int SHI>
int launch_map2d_stages(const tp_plan &plan, const Map2dParams &p, void *stream)
{
    static constexpr auto table = map2d_table<OP, SLO>(std::make_integer_sequence<int, (SHI - SLO + 1) * 16>{});
    const int i = ((plan.stages - SLO) * 4 + lane_chunks_index(plan.lane_chunks)) * 4 + plan.path;
    return launch_planned(table[i], plan, p, stream);
}

}  // namespace dev
}  // namespace tp
