// atlas_mem_linear.h -- entry of the linear memory on phi precomputed per
// call (atlas_mem_linear.hip): the same parameters and workspace scheme as
// the grouped MLP kernels (GroupedParams), WP window rows per coefficient block.
#pragma once

#include "atlas_mem_internal.h"

namespace atlas {

template <int PHI, int DK, int PD, int DV, int WP>
hipError_t launch_linear(const GroupedParams& gp, const CoeffParams& kp, hipStream_t stream, hipEvent_t ev0,
                         hipEvent_t ev1);
template <int PHI, int DK, int PD, int DV, int WP>
size_t linear_seq_bytes(int nchunks);

}  // namespace atlas
