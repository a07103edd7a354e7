// Role-split pipelined map kernels for op = copy (every stage count, tile size and path).
#include "tp_map_split.hpp"

namespace tp {

int launch_map_split_copy(const tp_plan &plan, const MapParams &p, void *stream)
{
    return dev::launch_map_split_op<TP_OP_COPY>(plan, p, stream);
}

}  // namespace tp
