// Explicit instantiations of the scan and decode launchers for head_dim 64.
#include "ssd_scan.hpp"
#include "ssd_step.hpp"

namespace ssd {
#define SSD_INST(IO, NN)                                                                  \
    template hipError_t launch_scan<IO, 64, NN>(const ScanPlan &, const ScanArgs &,      \
                                                 hipStream_t);                            \
    template hipError_t launch_step<IO, 64, NN>(const StepArgs &, hipStream_t);
SSD_INST(float, 32)
SSD_INST(float, 64)
SSD_INST(float, 128)
SSD_INST(bf16, 32)
SSD_INST(bf16, 64)
SSD_INST(bf16, 128)
#undef SSD_INST
}  // namespace ssd
