// Neighbour-row exchange: the gfx950 kernels (their body is in
// tp_row_shift.hpp) and their launch table.
#include "tp_row_shift.hpp"

namespace tp {
namespace dev {

template <bool LX4, bool SX4>
__global__ void __launch_bounds__(1024) row_shift_kernel(RowShiftParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    row_shift_body<GpuEngine, LX4, SX4>(TP_GPU_ENGINE(lds), p);
}

}  // namespace dev

int launch_row_shift(const tp_plan &plan, const RowShiftParams &p, void *stream)
{
    using Fn = void (*)(RowShiftParams);
    static constexpr Fn table[4] = {
        &dev::row_shift_kernel<true, true>, &dev::row_shift_kernel<false, true>,
        &dev::row_shift_kernel<true, false>, &dev::row_shift_kernel<false, false>};
    RowShiftParams args = p;
    void *kargs[] = {&args};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(table[plan.path]), dim3(1),
                                dim3((uint32_t)plan.threads), kargs, (size_t)plan.lds_bytes,
                                (hipStream_t)stream);
}

}  // namespace tp
