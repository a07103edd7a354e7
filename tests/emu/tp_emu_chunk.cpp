// Emulated launches of the chunk copy and the row exchange (tp_emu.hpp).
#include "tp_chunk_copy.hpp"
#include "tp_emu.hpp"
#include "tp_row_shift.hpp"
#include "tp_wg_copy.hpp"

using emu::EmuEngine;

namespace {

template <int S, int W, int P>
std::function<void()> chunk_body(const tp::ChunkParams &p)
{
    return [p] {
        tp::dev::chunk_copy_body<EmuEngine, S, W, !(P & TP_PATH_SCALAR_LOAD),
                                 !(P & TP_PATH_SCALAR_STORE)>(EmuEngine{}, p);
    };
}

template <int P>
std::function<void()> row_shift_body(const tp::RowShiftParams &p)
{
    return [p] {
        tp::dev::row_shift_body<EmuEngine, !(P & TP_PATH_SCALAR_LOAD), !(P & TP_PATH_SCALAR_STORE)>(
            EmuEngine{}, p);
    };
}

}  // namespace

extern "C" {

// Plans the chunk copy as tp_chunk_copy_ex does and runs its kernel body under
// the emulator. Returns a tp_status from planning, 0 with the destination
// written, or emu::kViolation with `err` describing the first violation.
int emu_chunk_copy(const void *src, void *dst, int64_t n_chunks, int chunk_bytes,
                   const uint8_t *pred, const uint8_t *src_size, const uint8_t *ignore_src,
                   int stages, int tiles_per_block, const emu::Options *o, tp_plan *plan_out,
                   char *err, int errlen)
{
    tp_plan plan;
    const int st = tp::plan_chunk_copy((uintptr_t)src, (uintptr_t)dst, n_chunks, chunk_bytes,
                                       (uintptr_t)pred, (uintptr_t)src_size,
                                       (uintptr_t)ignore_src, stages, tiles_per_block,
                                       tp::kLdsPerCu, &plan);
    if (st != TP_OK)
        return st;
    *plan_out = plan;
    if (plan.grid == 0)
        return 0;
    const tp::ChunkParams p = tp::chunk_params(plan, src, dst, n_chunks, pred, src_size, ignore_src);
    std::function<void()> body;
    emu::pick<1, 2, 3, 4, 5, 6, 7, 8>(plan.stages, [&](auto s) {
        if (plan.chunk_bytes == 8)
            body = chunk_body<s, 8, TP_PATH_SCALAR>(p);
        else if (plan.chunk_bytes == 4)
            body = chunk_body<s, 4, TP_PATH_SCALAR>(p);
        else
            emu::pick<0, 1, 2, 3>(plan.path, [&](auto q) { body = chunk_body<s, 16, q>(p); });
    });
    return emu::launch(plan, *o, body, err, errlen);
}

// The row exchange, planned as tp_row_shift does.
int emu_row_shift(const float *a, float *b, int64_t rows, const emu::Options *o, tp_plan *plan_out,
                  char *err, int errlen)
{
    tp_plan plan;
    const int st = tp::plan_row_shift((uintptr_t)a, (uintptr_t)b, rows, tp::kLdsPerCu, &plan);
    if (st != TP_OK)
        return st;
    *plan_out = plan;
    if (plan.grid == 0)
        return 0;
    const tp::RowShiftParams p{a, b, (int32_t)rows, 0};
    std::function<void()> body;
    emu::pick<0, 1, 2, 3>(plan.path, [&](auto q) { body = row_shift_body<q>(p); });
    return emu::launch(plan, *o, body, err, errlen);
}

// Copies between workgroups, planned as tp_workgroup_copy does: the clearing
// kernel over every workgroup, then the hand-off kernel over the workgroups
// of `o` in its order (the emulator runs one workgroup after another, so a
// receiver run before its sender finds no flag and gives up after spin_limit
// polls, as the GPU kernel would).
int emu_workgroup_copy(const void *src, void *dst, int64_t n_chunks, void *workspace,
                       int64_t workspace_bytes, int32_t *status, int spin_limit,
                       const emu::Options *o, tp_plan *plan_out, char *err, int errlen)
{
    tp_plan plan;
    const int st = tp::plan_workgroup_copy((uintptr_t)src, (uintptr_t)dst, n_chunks,
                                           (uintptr_t)workspace, workspace_bytes,
                                           (uintptr_t)status, spin_limit, &plan);
    if (st != TP_OK)
        return st;
    *plan_out = plan;
    if (n_chunks == 0)
        return 0;
    tp::WgCopyParams p{};
    p.src = static_cast<const uint8_t *>(src);
    p.dst = static_cast<uint8_t *>(dst);
    p.stage = static_cast<uint8_t *>(workspace);
    p.status = status;
    p.n_chunks = n_chunks;
    p.spin_limit = spin_limit == 0 ? tp::kWgDefaultSpinLimit : (uint32_t)spin_limit;
    tp_plan clear = plan;
    clear.threads = (int32_t)tp::kWgClearThreads;
    clear.grid = tp::wg_clear_groups(n_chunks);
    clear.lds_bytes = 0;
    emu::Options co = *o;
    co.blocks = nullptr;
    co.n_blocks = 0;
    int r = emu::launch(clear, co, [p] { tp::dev::workgroup_copy_clear_body(EmuEngine{}, p); }, err,
                        errlen);
    if (r != 0 || n_chunks < 2)
        return r;
    return emu::launch(plan, *o, [p] { tp::dev::workgroup_copy_body(EmuEngine{}, p); }, err, errlen);
}

// The library's device check on an architecture name, as the device would
// report it (the check itself needs no device).
int emu_arch_status(const char *arch) { return tp::arch_status(arch); }

}  // extern "C"
