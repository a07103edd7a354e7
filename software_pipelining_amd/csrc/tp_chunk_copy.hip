// Predicated chunk copy: the gfx950 kernels (their body is in
// tp_chunk_copy.hpp) and their launch table.
#include "tp_chunk_copy.hpp"

namespace tp {
namespace dev {

template <int S, int W, bool LX4, bool SX4>
__global__ void __launch_bounds__(256) chunk_copy_kernel(ChunkParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    chunk_copy_body<GpuEngine, S, W, LX4, SX4>(TP_GPU_ENGINE(lds), p);
}

}  // namespace dev

int launch_chunk_copy(const tp_plan &plan, const ChunkParams &p, void *stream)
{
    using Fn = void (*)(ChunkParams);
    // per stage count: the four 16-byte-chunk paths, then 8- and 4-byte chunks (words only)
#define TP_CHUNK_ROW(S)                                                                        \
    &dev::chunk_copy_kernel<S, 16, true, true>, &dev::chunk_copy_kernel<S, 16, false, true>,   \
        &dev::chunk_copy_kernel<S, 16, true, false>, &dev::chunk_copy_kernel<S, 16, false, false>, \
        &dev::chunk_copy_kernel<S, 8, false, false>, &dev::chunk_copy_kernel<S, 4, false, false>
    static constexpr Fn table[kMaxStages * 6] = {TP_CHUNK_ROW(1), TP_CHUNK_ROW(2), TP_CHUNK_ROW(3),
                                                 TP_CHUNK_ROW(4), TP_CHUNK_ROW(5), TP_CHUNK_ROW(6),
                                                 TP_CHUNK_ROW(7), TP_CHUNK_ROW(8)};
#undef TP_CHUNK_ROW
    const int col = plan.chunk_bytes == 16 ? plan.path : plan.chunk_bytes == 8 ? 4 : 5;
    const Fn fn = table[(plan.stages - 1) * 6 + col];
    if (plan.lds_bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 plan.lds_bytes);
        if (e != hipSuccess)
            return (int)e;
    }
    ChunkParams args = p;
    void *kargs[] = {&args};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((uint32_t)plan.grid),
                                dim3((uint32_t)plan.threads), kargs, (size_t)plan.lds_bytes,
                                (hipStream_t)stream);
}

}  // namespace tp
