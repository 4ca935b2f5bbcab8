// Launchers of the gfx950 kernels (kernels.hip).  Each returns the HIP
// runtime's status of the launch; none synchronises.
#pragma once
#include <hip/hip_runtime_api.h>

#include "args.hpp"

namespace ulysses {

// Most blocks along grid.y (batch planes) of one launch; callers split
// larger batches over several launches.
constexpr uint32_t kMaxGridY = 65535;

// Relayout pass over `tensors` tensors of one geometry: grid (grid_x,
// planes, tensors) of kRelayoutBlock threads, from the planes src and dst
// point at.
hipError_t launch_relayout(const RelayoutArgs &a, uint32_t grid_x, uint32_t planes,
                           uint32_t tensors, hipStream_t stream);

// Copy of nvec[r] vectors per rank: grid (grid_x, 1, 1) of kRelayoutBlock
// threads.
hipError_t launch_plane_copy(const CopyArgs &a, uint32_t grid_x, hipStream_t stream);

// Device address of the static window array (kStaticWindowBytes) on the
// device of `stream` (the current device for the null stream), looked up
// once per device and kept.  The library allocates nothing here: the array
// is part of the library's code object on each GPU.
hipError_t static_windows(hipStream_t stream, unsigned char **ptr);

// Fused QK RMSNorm + RoPE mode-0 pass over q and k for head dimension d
// (d / 8 a power of two from 1 to 64): grid (grid_x, planes, 1) of
// kFusedBlock threads.
hipError_t launch_fused(const FusedArgs &a, uint32_t d, uint32_t grid_x, uint32_t planes,
                        hipStream_t stream);

}  // namespace ulysses
