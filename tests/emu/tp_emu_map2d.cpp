// Emulated launches of the strided 2-D map (tp_emu.hpp). Every stage count,
// lane-chunk count and path is compiled in for scale2; horner32 and copy for
// the subsets listed, which share scale2's memory schedule.
#include "tp_emu.hpp"
#include "tp_map2d.hpp"

using emu::EmuEngine;

namespace {

template <int OP, int S, int L, int P>
std::function<void()> body_of(const tp::Map2dParams &p)
{
    return [p] {
        tp::dev::map2d_body<EmuEngine, OP, S, L, !(P & TP_PATH_SCALAR_LOAD), !(P & TP_PATH_SCALAR_STORE)>(
            EmuEngine{}, p);
    };
}

}  // namespace

// Compiled twice (EMU_PART 0 and 1) so the instances build in parallel: part 1
// holds scale2 at stages 5-8, part 0 everything else and the entry point.
std::function<void()> map2d_part1(const tp_plan &plan, int op, const tp::Map2dParams &p);

#if EMU_PART == 1
std::function<void()> map2d_part1(const tp_plan &plan, int op, const tp::Map2dParams &p)
{
    std::function<void()> b;
    if (op == TP_OP_SCALE2)
        emu::pick<5, 6, 7, 8>(plan.stages, [&](auto s) {
            emu::pick<1, 2, 4, 8>(plan.lane_chunks, [&](auto l) {
                emu::pick<0, 1, 2, 3>(plan.path, [&](auto q) { b = body_of<TP_OP_SCALE2, s, l, q>(p); });
            });
        });
    return b;
}
#else
extern "C" {

// Plans the 2-D map as tp_map_2d does (with the whole 160 KiB of LDS as the
// budget) and runs its kernel body under the emulator.
int emu_map_2d(const float *src, int64_t src_stride, float *dst, int64_t dst_stride, int64_t rows,
               int64_t cols, int op, int box_rows, int box_cols, int stages, int boxes_per_block,
               int align, const emu::Options *o, tp_plan *plan_out, char *err, int errlen)
{
    tp_plan plan;
    const int st = tp::plan_map_2d((uintptr_t)src, src_stride, (uintptr_t)dst, dst_stride, rows,
                                   cols, op, box_rows, box_cols, stages, boxes_per_block, align,
                                   tp::kLdsPerCu, &plan);
    if (st != TP_OK)
        return st;
    *plan_out = plan;
    if (plan.grid == 0)
        return 0;
    const tp::Map2dParams p = tp::map2d_params(plan, src, src_stride, dst, dst_stride, rows, cols,
                                               box_rows, box_cols);
    std::function<void()> b;
    const int S = plan.stages, L = plan.lane_chunks, P = plan.path;
    if (op == TP_OP_SCALE2)
        emu::pick<1, 2, 3, 4>(S, [&](auto s) {
            emu::pick<1, 2, 4, 8>(L, [&](auto l) {
                emu::pick<0, 1, 2, 3>(P, [&](auto q) { b = body_of<TP_OP_SCALE2, s, l, q>(p); });
            });
        });
    else if (op == TP_OP_HORNER32)
        emu::pick<2>(S, [&](auto s) {
            emu::pick<1>(L, [&](auto l) {
                emu::pick<0, 3>(P, [&](auto q) { b = body_of<TP_OP_HORNER32, s, l, q>(p); });
            });
        });
    else
        emu::pick<2>(S, [&](auto s) {
            emu::pick<1>(L, [&](auto l) {
                emu::pick<0>(P, [&](auto q) { b = body_of<TP_OP_COPY, s, l, q>(p); });
            });
        });
    if (!b)
        b = map2d_part1(plan, op, p);
    if (!b)
        return emu::kNotInstantiated;
    return emu::launch(plan, *o, b, err, errlen);
}

}  // extern "C"
#endif
