// Role-split pipelined map kernels for op = horner32 (every stage count, tile size and path).
#include "tp_map_split.hpp"

namespace tp {

int launch_map_split_horner32(const tp_plan &plan, const MapParams &p, void *stream)
{
    return dev::launch_map_split_op<TP_OP_HORNER32>(plan, p, stream);
}

}  // namespace tp
