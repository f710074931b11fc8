// ns_kernels.h - launch interface between the host driver and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "ns_layout.h"
#include "ns_plan.h"

namespace ns {

// Events that the next launches of this thread record in their dispatch
// packets (start: the first one's start; stop: the last one's end); both
// null: plain launches.  The caller clears them after the launches it times.
void set_launch_events(hipEvent_t start, hipEvent_t stop);

hipError_t launch_gemm(int dtype, const StageKind& k, const GemmArgs& g, hipStream_t st);
// n groups of slices, each with its own arguments, one kernel instance (k)
hipError_t launch_gemm_grouped(int dtype, const StageKind& k, const GemmArgs* gs, int n, hipStream_t st);
hipError_t launch_sumsq(int dtype, const NormArgs& g, int batch, hipStream_t st);
hipError_t launch_sumsq_grouped(int dtype, const NormArgs* gs, const int* batch, int n, hipStream_t st);
hipError_t launch_scale(int dtype, const NormArgs& g, int batch, hipStream_t st);
// odd shapes: the zero-padded copy fused with the sum-of-squares pass (g
// over the padded copy), and the caller's block out of the padded result
hipError_t launch_pad_sumsq(int dtype, const PadArgs& p, const NormArgs& g, int batch, hipStream_t st);
hipError_t launch_unpad(int dtype, const PadArgs& p, hipStream_t st);

// Device address of the fixed scratch array (ns_noalloc.hip) on device
// `dev`, which must be the current device.  The first call per device takes
// it with hipGetSymbolAddress; later calls return the kept value.
hipError_t noalloc_scratch(int dev, char** ptr);

// matrix-core calibration loop (ns_peak.hip): `blocks` workgroups of
// kPeakThreads threads, each wave `iters` (a multiple of 4) rounds of
// mfma_peak_acc() MFMAs; sink takes one float per thread, clocks four
// counters per workgroup (shader clock and wall clock, before and after)
constexpr int kPeakThreads = 256;
hipError_t launch_mfma_peak(int dtype, int blocks, int iters, float* sink, unsigned long long* clocks,
                            hipStream_t st);
long long mfma_peak_flops_per_inst(int dtype);
int mfma_peak_acc();

}  // namespace ns
