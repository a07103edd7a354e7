// Strided 2-D map kernels for op = horner32 (every stage count, lane width and path).
#include "tp_map2d.hpp"

namespace tp {

int launch_map2d_horner32(const tp_plan &plan, const Map2dParams &p, void *stream)
{
    return dev::launch_map2d_op<TP_OP_HORNER32>(plan, p, stream);
}

}  // namespace tp
