// Copies between workgroups: the gfx950 kernels (their bodies are in
// tp_wg_copy.hpp) and their launches.
#include <mutex>

#include "tp_wg_copy.hpp"

namespace tp {

// Workspace of tp_workgroup_copy_noalloc: the staging slots of at most
// kWgNoAllocMaxChunks chunks. Each GPU the library runs on holds its own copy
// until the process ends. In host code `scratch` names a host-side stand-in,
// not the device array: only the address hipGetSymbolAddress returns for the
// current device is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kWgNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices];
}  // namespace

int workgroup_copy_scratch(void **ptr)
{
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return (int)e;
    if (device < 0 || device >= kMaxScratchDevices)
        return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `device` current
        if (e != hipSuccess)
            return (int)e;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return 0;
}
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
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&dev::workgroup_copy_clear_kernel),
                                   dim3((uint32_t)wg_clear_groups(p.n_chunks)),
                                   dim3((uint32_t)kWgClearThreads), kargs, 0, (hipStream_t)stream);
    if (e != hipSuccess || p.n_chunks < 2)
        return (int)e;
    e = hipLaunchKernel(reinterpret_cast<const void *>(&dev::workgroup_copy_kernel),
                        dim3((uint32_t)plan.grid), dim3((uint32_t)plan.threads), kargs,
                        (size_t)plan.lds_bytes, (hipStream_t)stream);
    return (int)e;
}

}  // namespace tp
