// Fine-grained FP8 grouped GEMMs (placeholder until the e4m3 MFMA kernels land).
#include "common.h"
#include "launch.h"

namespace moe {

int fp8_tile_rows_gateup() { return 128; }
int fp8_tile_rows_down() { return 128; }

hipError_t launch_experts_fp8(const ExpertsLaunch&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe
