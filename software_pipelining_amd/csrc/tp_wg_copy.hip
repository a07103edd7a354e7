// Copies between workgroups: the gfx950 kernels (their bodies are in
// tp_wg_copy.hpp) and their launches.
#include "tp_wg_copy.hpp"

namespace tp {
namespace dev {

__global__ void __launch_bounds__(256) workgroup_copy_clear_kernel(WgCopyParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    workgroup_copy_clear_body(TP_GPU_ENGINE(lds), p);
}

__global__ void __launch_bounds__(64) workgroup_copy_kernel(WgCopyParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    workgroup_copy_body(TP_GPU_ENGINE(lds), p);
}

}  // namespace dev

int launch_workgroup_copy(const tp_plan &plan, const WgCopyParams &p, void *stream)
{
    WgCopyParams args = p;
    void *kargs[] = {&args};
    const int64_t clear_groups = (p.n_chunks + kWgClearThreads - 1) / kWgClearThreads;
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&dev::workgroup_copy_clear_kernel),
                                   dim3((uint32_t)clear_groups), dim3((uint32_t)kWgClearThreads),
                                   kargs, 0, (hipStream_t)stream);
    if (e != hipSuccess || p.n_chunks < 2)
        return (int)e;
    e = hipLaunchKernel(reinterpret_cast<const void *>(&dev::workgroup_copy_kernel),
                        dim3((uint32_t)plan.grid), dim3((uint32_t)plan.threads), kargs,
                        (size_t)plan.lds_bytes, (hipStream_t)stream);
    return (int)e;
}

}  // namespace tp
