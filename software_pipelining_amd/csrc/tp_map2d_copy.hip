// Strided 2-D map kernels for op = copy (every stage count, lane width and path).
#include "tp_map2d.hpp"

namespace tp {

int launch_map2d_copy(const tp_plan &plan, const Map2dParams &p, void *stream)
{
    return dev::launch_map2d_op<TP_OP_COPY>(plan, p, stream);
}

}  // namespace tp
