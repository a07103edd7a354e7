// Pipelined map kernels for op = horner32 (every stage count, lane width and path).
#include "tp_map.hpp"

namespace tp {

int launch_map_horner32(const tp_plan &plan, const MapParams &p, void *stream)
{
    return dev::launch_map_op<TP_OP_HORNER32>(plan, p, stream);
}

}  // namespace tp
