// Pipelined map kernels for op = copy (every stage count, lane width and path).
#include "tp_map.hpp"

namespace tp {

int launch_map_copy(const tp_plan &plan, const MapParams &p, void *stream)
{
    return dev::launch_map_op<TP_OP_COPY>(plan, p, stream);
}

}  // namespace tp
