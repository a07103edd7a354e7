// Emulated launches of the 1-D pipelined map, both schedules (tp_emu.hpp).
// Compiled three times: EMU_PART 0 holds the entry point, the role split and
// the ops other than scale2; parts 1 and 2 the uniform scale2 instances of
// stages 1-4 and 5-8.
// Every stage count, lane-chunk count and path is compiled in for scale2 (for
// the role split: tiles of 256, 1024 and 8192 floats); horner32 and copy for
// the subsets listed, which share scale2's memory schedule.
#include "tp_emu.hpp"
#include "tp_map.hpp"
#include "tp_map_split.hpp"

using emu::EmuEngine;

namespace {

template <int OP, int S, int L, int P>
std::function<void()> uniform_body(const tp::MapParams &p)
{
    return [p] {
        tp::dev::map_body<EmuEngine, OP, S, L, !(P & TP_PATH_SCALAR_LOAD), !(P & TP_PATH_SCALAR_STORE)>(
            EmuEngine{}, p);
    };
}

template <int OP, int S, int TILE, int P>
std::function<void()> split_body(const tp::MapParams &p)
{
    return [p] {
        tp::dev::map_split_body<EmuEngine, OP, S, TILE, !(P & TP_PATH_SCALAR_LOAD),
                                !(P & TP_PATH_SCALAR_STORE)>(EmuEngine{}, p);
    };
}

}  // namespace

// Kernel instances are spread over three compilations of this file
// (EMU_PART 0, 1, 2) so that they build in parallel; parts 1 and 2 return the
// body they hold for a plan, or an empty function.
std::function<void()> map_part1(const tp_plan &plan, int op, const tp::MapParams &p);
std::function<void()> map_part2(const tp_plan &plan, int op, const tp::MapParams &p);

#if EMU_PART == 1 || EMU_PART == 2
#if EMU_PART == 1
std::function<void()> map_part1(const tp_plan &plan, int op, const tp::MapParams &p)
#else
std::function<void()> map_part2(const tp_plan &plan, int op, const tp::MapParams &p)
#endif
{
    std::function<void()> b;
    if (plan.schedule != TP_SCHED_UNIFORM || op != TP_OP_SCALE2)
        return b;
    auto pick_l = [&](auto s) {
        emu::pick<1, 2, 4, 8>(plan.lane_chunks, [&](auto l) {
            emu::pick<0, 1, 2, 3>(plan.path, [&](auto q) { b = uniform_body<TP_OP_SCALE2, s, l, q>(p); });
        });
    };
#if EMU_PART == 1
    emu::pick<1, 2, 3, 4>(plan.stages, pick_l);
#else
    emu::pick<5, 6, 7, 8>(plan.stages, pick_l);
#endif
    return b;
}
#else
namespace {

std::function<void()> part0(const tp_plan &plan, int op, const tp::MapParams &p)
{
    std::function<void()> b;
    const int S = plan.stages, L = plan.lane_chunks, T = plan.tile_units, P = plan.path;
    if (plan.schedule == TP_SCHED_ROLE_SPLIT) {
        if (op == TP_OP_SCALE2)
            emu::pick<1, 2, 3, 4, 5, 6, 7, 8>(S, [&](auto s) {
                emu::pick<256, 1024, 8192>(T, [&](auto t) {
                    emu::pick<0, 1, 2, 3>(P, [&](auto q) { b = split_body<TP_OP_SCALE2, s, t, q>(p); });
                });
            });
        else if (op == TP_OP_HORNER32)
            emu::pick<1, 2, 4>(S, [&](auto s) {
                emu::pick<1024>(T, [&](auto t) {
                    emu::pick<0>(P, [&](auto q) { b = split_body<TP_OP_HORNER32, s, t, q>(p); });
                });
            });
    } else if (op == TP_OP_HORNER32) {
        emu::pick<1, 2, 4>(S, [&](auto s) {
            emu::pick<1, 2>(L, [&](auto l) {
                emu::pick<0, 3>(P, [&](auto q) { b = uniform_body<TP_OP_HORNER32, s, l, q>(p); });
            });
        });
    } else if (op == TP_OP_COPY) {
        emu::pick<2>(S, [&](auto s) {
            emu::pick<1>(L, [&](auto l) {
                emu::pick<0, 1, 2, 3>(P, [&](auto q) { b = uniform_body<TP_OP_COPY, s, l, q>(p); });
            });
        });
    }
    return b;
}

}  // namespace

extern "C" {

// Plans the map as tp_pipelined_map_ex does (with the whole 160 KiB of LDS as
// the budget) and runs its kernel body under the emulator.
int emu_pipelined_map(const float *in, float *out, int64_t n, int op, int tile_elems, int stages,
                      int tiles_per_block, int resident_cap, int schedule, int align,
                      const emu::Options *o, tp_plan *plan_out, char *err, int errlen)
{
    tp_plan plan;
    const int st = tp::plan_map((uintptr_t)in, (uintptr_t)out, n, op, tile_elems, stages,
                                tiles_per_block, resident_cap, schedule, align, tp::kLdsPerCu,
                                &plan);
    if (st != TP_OK)
        return st;
    *plan_out = plan;
    if (plan.grid == 0)
        return 0;
    const tp::MapParams p = tp::map_params(plan, in, out, n);
    std::function<void()> body = part0(plan, op, p);
    if (!body)
        body = map_part1(plan, op, p);
    if (!body)
        body = map_part2(plan, op, p);
    if (!body)
        return emu::kNotInstantiated;
    return emu::launch(plan, *o, body, err, errlen);
}

}  // extern "C"
#endif
