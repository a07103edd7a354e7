// Instantiates the pipelined-map kernels of one op and one range of stage counts.
// The build compiles this unit once per op and per half of the stage range
// (TP_INST_OP, TP_INST_SLO..TP_INST_SHI, entry point TP_INST_FN), so the
// kernel instances compile in parallel pieces of similar size.
#include "tp_map.hpp"

#if !defined(TP_INST_OP) || !defined(TP_INST_SLO) || !defined(TP_INST_SHI) || !defined(TP_INST_FN)
#error "the build defines TP_INST_OP, TP_INST_SLO, TP_INST_SHI and TP_INST_FN"
#endif

namespace tp {

int TP_INST_FN(const tp_plan &plan, const MapParams &p, void *stream)
{
    return dev::launch_map_stages<TP_INST_OP, TP_INST_SLO, TP_INST_SHI>(plan, p, stream);
}

}  // namespace tp
