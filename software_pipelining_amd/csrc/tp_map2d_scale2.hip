// Strided 2-D map kernels for op = scale2 (every stage count, lane width and path).
#include "tp_map2d.hpp"

namespace tp {

int launch_map2d_scale2(const tp_plan &plan, const Map2dParams &p, void *stream)
{
    return dev::launch_map2d_op<TP_OP_SCALE2>(plan, p, stream);
}

}  // namespace tp
