// Explicit instantiations of the scan and decode launchers for head_dim 32.
#include "ssd_scan.hpp"
#include "ssd_scan16.hpp"
#include "ssd_step.hpp"

namespace ssd {
#define SSD_INST(NN)                                                                      \
    template hipError_t launch_scan<float, 32, NN>(const ScanPlan &, const ScanArgs &,   \
                                                    hipStream_t);                         \
    template hipError_t launch_scan16<32, NN>(const ScanPlan &, const ScanArgs &,        \
                                               hipStream_t);                              \
    template hipError_t launch_step<float, 32, NN>(const StepArgs &, hipStream_t);       \
    template hipError_t launch_step<bf16, 32, NN>(const StepArgs &, hipStream_t);
SSD_INST(32)
SSD_INST(64)
SSD_INST(128)
#undef SSD_INST
}  // namespace ssd
