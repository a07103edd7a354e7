// C ABI of libtilepipe: validation, device checks and launches.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <string.h>

#include "tp_internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;

struct DeviceInfo {
    bool known;
    int status;            // TP_OK or TP_ERR_UNSUPPORTED_DEVICE
    int64_t lds_budget;    // bytes of LDS one workgroup may use
};

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
DeviceInfo g_devices[kMaxDevices];

int hip_failure(hipError_t e)
{
    g_last_hip_error = (int)e;
    return TP_ERR_HIP;
}

int query_device(int device, int64_t *lds_budget)
{
    if (device < 0 || device >= kMaxDevices)
        return hip_failure(hipErrorInvalidDevice);
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (g_devices[device].known) {
            if (lds_budget)
                *lds_budget = g_devices[device].lds_budget;
            return g_devices[device].status;
        }
    }
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
        return hip_failure(e);
    int lds = 0;
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, device);
    if (e != hipSuccess)
        return hip_failure(e);
    DeviceInfo info{true, tp::arch_status(prop.gcnArchName), lds};
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        g_devices[device] = info;
    }
    if (lds_budget)
        *lds_budget = info.lds_budget;
    return info.status;
}

int current_device(int64_t *lds_budget)
{
    int device = 0;
    const hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return hip_failure(e);
    return query_device(device, lds_budget);
}

int finish_launch(int hip_error)
{
    if (hip_error != 0) {
        (void)hipGetLastError();
        return hip_failure((hipError_t)hip_error);
    }
    return TP_OK;
}

// The kernel instances of each family, op and half of the stage range live in
// separate objects; these pick the one a plan needs.
int launch_map(const tp_plan &plan, const tp::MapParams &p, int op, void *stream)
{
    const bool hi = plan.stages > 4;
    if (plan.schedule == TP_SCHED_ROLE_SPLIT) {
        switch (op) {
        case TP_OP_SCALE2:
            return hi ? tp::launch_map_split_scale2_s5_8(plan, p, stream)
                      : tp::launch_map_split_scale2_s1_4(plan, p, stream);
        case TP_OP_HORNER32:
            return hi ? tp::launch_map_split_horner32_s5_8(plan, p, stream)
                      : tp::launch_map_split_horner32_s1_4(plan, p, stream);
        default:
            return hi ? tp::launch_map_split_copy_s5_8(plan, p, stream)
                      : tp::launch_map_split_copy_s1_4(plan, p, stream);
        }
    }
    switch (op) {
    case TP_OP_SCALE2:
        return hi ? tp::launch_map_scale2_s5_8(plan, p, stream) : tp::launch_map_scale2_s1_4(plan, p, stream);
    case TP_OP_HORNER32:
        return hi ? tp::launch_map_horner32_s5_8(plan, p, stream)
                  : tp::launch_map_horner32_s1_4(plan, p, stream);
    default:
        return hi ? tp::launch_map_copy_s5_8(plan, p, stream) : tp::launch_map_copy_s1_4(plan, p, stream);
    }
}

int launch_map2d(const tp_plan &plan, const tp::Map2dParams &p, int op, void *stream)
{
    const bool hi = plan.stages > 4;
    switch (op) {
    case TP_OP_SCALE2:
        return hi ? tp::launch_map2d_scale2_s5_8(plan, p, stream) : tp::launch_map2d_scale2_s1_4(plan, p, stream);
    case TP_OP_HORNER32:
        return hi ? tp::launch_map2d_horner32_s5_8(plan, p, stream)
                  : tp::launch_map2d_horner32_s1_4(plan, p, stream);
    default:
        return hi ? tp::launch_map2d_copy_s5_8(plan, p, stream) : tp::launch_map2d_copy_s1_4(plan, p, stream);
    }
}

// Argument errors are decided with an unlimited LDS budget first, so a bad
// call never touches the device; the device's real budget is checked after.
constexpr int64_t kNoBudget = INT64_MAX;

}  // namespace

extern "C" {

TP_API const char *tp_status_string(int status)
{
    switch (status) {
    case TP_OK: return "TP_OK";
    case TP_ERR_INVALID_ARG: return "TP_ERR_INVALID_ARG";
    case TP_ERR_MISALIGNED: return "TP_ERR_MISALIGNED";
    case TP_ERR_LDS_BUDGET: return "TP_ERR_LDS_BUDGET";
    case TP_ERR_OVERLAP: return "TP_ERR_OVERLAP";
    case TP_ERR_UNSUPPORTED_DEVICE: return "TP_ERR_UNSUPPORTED_DEVICE";
    case TP_ERR_HIP: return "TP_ERR_HIP";
    default: return "TP_ERR_UNKNOWN";
    }
}

TP_API int tp_last_hip_error(void) { return g_last_hip_error; }

TP_API int tp_version(void) { return TP_VERSION; }

TP_API int tp_device_check(int device) { return query_device(device, nullptr); }

TP_API int tp_device_lds_budget(int device, int64_t *bytes)
{
    if (!bytes)
        return TP_ERR_INVALID_ARG;
    const int st = query_device(device, bytes);
    return st == TP_ERR_UNSUPPORTED_DEVICE ? TP_OK : st;
}

TP_API int tp_plan_row_shift(const void *a, const void *b, int64_t rows, int64_t lds_budget,
                             tp_plan *plan)
{
    return tp::plan_row_shift((uintptr_t)a, (uintptr_t)b, rows, lds_budget, plan);
}

TP_API int tp_plan_pipelined_map(const void *in, const void *out, int64_t n, int op,
                                 int tile_elems, int stages, int tiles_per_block,
                                 int resident_cap, int schedule, int align,
                                 int64_t lds_budget, tp_plan *plan)
{
    return tp::plan_map((uintptr_t)in, (uintptr_t)out, n, op, tile_elems, stages, tiles_per_block,
                        resident_cap, schedule, align, lds_budget, plan);
}

TP_API int tp_plan_map_2d(const void *src, int64_t src_stride, const void *dst,
                          int64_t dst_stride, int64_t rows, int64_t cols, int op, int box_rows,
                          int box_cols, int stages, int boxes_per_block, int align,
                          int64_t lds_budget, tp_plan *plan)
{
    return tp::plan_map_2d((uintptr_t)src, src_stride, (uintptr_t)dst, dst_stride, rows, cols, op,
                           box_rows, box_cols, stages, boxes_per_block, align, lds_budget, plan);
}

TP_API int tp_plan_chunk_copy(const void *src, const void *dst, int64_t n_chunks,
                              int chunk_bytes, const void *pred, const void *src_size,
                              const void *ignore_src, int stages, int tiles_per_block,
                              int64_t lds_budget, tp_plan *plan)
{
    return tp::plan_chunk_copy((uintptr_t)src, (uintptr_t)dst, n_chunks, chunk_bytes,
                               (uintptr_t)pred, (uintptr_t)src_size, (uintptr_t)ignore_src,
                               stages, tiles_per_block, lds_budget, plan);
}

TP_API int tp_row_shift(const float *a, float *b, int64_t rows, void *stream, int *path_out)
{
    tp_plan plan;
    int st = tp::plan_row_shift((uintptr_t)a, (uintptr_t)b, rows, kNoBudget, &plan);
    if (st != TP_OK)
        return st;
    if (path_out)
        *path_out = plan.path;
    if (plan.grid == 0)
        return TP_OK;
    int64_t lds = 0;
    if ((st = current_device(&lds)) != TP_OK)
        return st;
    if (plan.lds_bytes > lds)
        return TP_ERR_LDS_BUDGET;
    tp::RowShiftParams p{a, b, (int32_t)rows, 0};
    return finish_launch(tp::launch_row_shift(plan, p, stream));
}

TP_API int tp_pipelined_map(const float *in, float *out, int64_t n, int op, int tile_elems,
                            int stages, int tiles_per_block, void *stream, int *path_out)
{
    return tp_pipelined_map_ex(in, out, n, op, tile_elems, stages, tiles_per_block, 0,
                               TP_SCHED_UNIFORM, TP_ALIGN_REALIGN, stream, path_out);
}

TP_API int tp_pipelined_map_ex(const float *in, float *out, int64_t n, int op, int tile_elems,
                               int stages, int tiles_per_block, int resident_cap, int schedule,
                               int align, void *stream, int *path_out)
{
    tp_plan plan;
    int st = tp::plan_map((uintptr_t)in, (uintptr_t)out, n, op, tile_elems, stages,
                          tiles_per_block, resident_cap, schedule, align, kNoBudget, &plan);
    if (st != TP_OK)
        return st;
    if (path_out)
        *path_out = plan.path;
    if (plan.grid == 0)
        return TP_OK;
    int64_t lds = 0;
    if ((st = current_device(&lds)) != TP_OK)
        return st;
    // again with the device's budget: the ring must fit, and the LDS reserved
    // to bound residency never exceeds it
    st = tp::plan_map((uintptr_t)in, (uintptr_t)out, n, op, tile_elems, stages, tiles_per_block,
                      resident_cap, schedule, align, lds, &plan);
    if (st != TP_OK)
        return st;
    const tp::MapParams p = tp::map_params(plan, in, out, n);
    return finish_launch(launch_map(plan, p, op, stream));
}

TP_API int tp_map_2d(const float *src, int64_t src_stride, float *dst, int64_t dst_stride,
                     int64_t rows, int64_t cols, int op, int box_rows, int box_cols, int stages,
                     int boxes_per_block, int align, void *stream, int *path_out)
{
    tp_plan plan;
    int st = tp::plan_map_2d((uintptr_t)src, src_stride, (uintptr_t)dst, dst_stride, rows, cols,
                             op, box_rows, box_cols, stages, boxes_per_block, align, kNoBudget,
                             &plan);
    if (st != TP_OK)
        return st;
    if (path_out)
        *path_out = plan.path;
    if (plan.grid == 0)
        return TP_OK;
    int64_t lds = 0;
    if ((st = current_device(&lds)) != TP_OK)
        return st;
    st = tp::plan_map_2d((uintptr_t)src, src_stride, (uintptr_t)dst, dst_stride, rows, cols, op,
                         box_rows, box_cols, stages, boxes_per_block, align, lds, &plan);
    if (st != TP_OK)
        return st;
    const tp::Map2dParams p = tp::map2d_params(plan, src, src_stride, dst, dst_stride, rows, cols,
                                               box_rows, box_cols);
    return finish_launch(launch_map2d(plan, p, op, stream));
}

TP_API int tp_chunk_copy(const void *src, void *dst, int64_t n_chunks, const uint8_t *pred,
                         const uint8_t *src_size, const uint8_t *ignore_src, int stages,
                         int tiles_per_block, void *stream, int *path_out)
{
    return tp_chunk_copy_ex(src, dst, n_chunks, 16, pred, src_size, ignore_src, stages,
                            tiles_per_block, stream, path_out);
}

TP_API int tp_chunk_copy_ex(const void *src, void *dst, int64_t n_chunks, int chunk_bytes,
                            const uint8_t *pred, const uint8_t *src_size,
                            const uint8_t *ignore_src, int stages, int tiles_per_block,
                            void *stream, int *path_out)
{
    tp_plan plan;
    int st = tp::plan_chunk_copy((uintptr_t)src, (uintptr_t)dst, n_chunks, chunk_bytes,
                                 (uintptr_t)pred, (uintptr_t)src_size, (uintptr_t)ignore_src,
                                 stages, tiles_per_block, kNoBudget, &plan);
    if (st != TP_OK)
        return st;
    if (path_out)
        *path_out = plan.path;
    if (plan.grid == 0)
        return TP_OK;
    int64_t lds = 0;
    if ((st = current_device(&lds)) != TP_OK)
        return st;
    if (plan.lds_bytes > lds)
        return TP_ERR_LDS_BUDGET;
    const tp::ChunkParams p = tp::chunk_params(plan, src, dst, n_chunks, pred, src_size, ignore_src);
    return finish_launch(tp::launch_chunk_copy(plan, p, stream));
}

TP_API int64_t tp_workgroup_copy_workspace_bytes(int64_t n_chunks)
{
    return n_chunks < 0 || n_chunks > tp::kWgMaxChunks ? -1 : tp::wg_workspace_bytes(n_chunks);
}

TP_API int tp_plan_workgroup_copy(const void *src, const void *dst, int64_t n_chunks,
                                  const void *workspace, int64_t workspace_bytes,
                                  const int32_t *status, int spin_limit, tp_plan *plan)
{
    return tp::plan_workgroup_copy((uintptr_t)src, (uintptr_t)dst, n_chunks,
                                   (uintptr_t)workspace, workspace_bytes, (uintptr_t)status,
                                   spin_limit, plan);
}

TP_API int tp_workgroup_copy(const void *src, void *dst, int64_t n_chunks, void *workspace,
                             int64_t workspace_bytes, int32_t *status, int spin_limit,
                             void *stream)
{
    tp_plan plan;
    int st = tp::plan_workgroup_copy((uintptr_t)src, (uintptr_t)dst, n_chunks,
                                     (uintptr_t)workspace, workspace_bytes, (uintptr_t)status,
                                     spin_limit, &plan);
    if (st != TP_OK)
        return st;
    if (n_chunks == 0)
        return TP_OK;
    int64_t lds = 0;
    if ((st = current_device(&lds)) != TP_OK)
        return st;
    if (plan.lds_bytes > lds)
        return TP_ERR_LDS_BUDGET;
    tp::WgCopyParams p{};
    p.src = static_cast<const uint8_t *>(src);
    p.dst = static_cast<uint8_t *>(dst);
    p.stage = static_cast<uint8_t *>(workspace);
    p.status = status;
    p.n_chunks = n_chunks;
    p.spin_limit = spin_limit == 0 ? tp::kWgDefaultSpinLimit : (uint32_t)spin_limit;
    return finish_launch(tp::launch_workgroup_copy(plan, p, stream));
}

TP_API int tp_workgroup_copy_noalloc(const void *src, void *dst, int64_t n_chunks,
                                     int32_t *status, int spin_limit, void *stream)
{
    if (n_chunks < 0 || n_chunks > tp::kWgNoAllocMaxChunks)
        return TP_ERR_INVALID_ARG;
    if (n_chunks == 0)
        return tp::plan_workgroup_copy((uintptr_t)src, (uintptr_t)dst, 0, 0, 0,
                                       (uintptr_t)status, spin_limit, nullptr);
    // argument errors first, with a stand-in address that overlaps nothing
    int st = tp::plan_workgroup_copy((uintptr_t)src, (uintptr_t)dst, n_chunks, 256,
                                     tp::kWgNoAllocScratchBytes, (uintptr_t)status, spin_limit,
                                     nullptr);
    if (st == TP_ERR_OVERLAP)
        st = TP_OK;   // decided again below, against the real address
    if (st != TP_OK)
        return st;
    int64_t lds = 0;
    if ((st = current_device(&lds)) != TP_OK)
        return st;
    void *ws = nullptr;
    const int e = tp::workgroup_copy_scratch(&ws);
    if (e != 0)
        return hip_failure((hipError_t)e);
    tp_plan plan;
    st = tp::plan_workgroup_copy((uintptr_t)src, (uintptr_t)dst, n_chunks, (uintptr_t)ws,
                                 tp::kWgNoAllocScratchBytes, (uintptr_t)status, spin_limit, &plan);
    if (st != TP_OK)
        return st;
    if (plan.lds_bytes > lds)
        return TP_ERR_LDS_BUDGET;
    tp::WgCopyParams p{};
    p.src = static_cast<const uint8_t *>(src);
    p.dst = static_cast<uint8_t *>(dst);
    p.stage = static_cast<uint8_t *>(ws);
    p.status = status;
    p.n_chunks = n_chunks;
    p.spin_limit = spin_limit == 0 ? tp::kWgDefaultSpinLimit : (uint32_t)spin_limit;
    return finish_launch(tp::launch_workgroup_copy(plan, p, stream));
}

}  // extern "C"
