// ns_kernels.h - launch interface between the host driver and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "ns_layout.h"
#include "ns_plan.h"

namespace ns {

hipError_t launch_gemm(int dtype, const StageKind& k, const GemmArgs& g, hipStream_t st);
// n groups of slices, each with its own arguments, one kernel instance (k)
hipError_t launch_gemm_grouped(int dtype, const StageKind& k, const GemmArgs* gs, int n, hipStream_t st);
hipError_t launch_sumsq(int dtype, const NormArgs& g, int batch, hipStream_t st);
hipError_t launch_sumsq_grouped(int dtype, const NormArgs* gs, const int* batch, int n, hipStream_t st);
hipError_t launch_scale(int dtype, const NormArgs& g, int batch, hipStream_t st);
hipError_t launch_pad(int dtype, const PadArgs& g, hipStream_t st);

}  // namespace ns
