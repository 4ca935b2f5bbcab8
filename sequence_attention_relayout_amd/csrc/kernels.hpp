// Launchers of the gfx950 kernels (kernels.hip).  Each returns the HIP
// runtime's status of the launch; none synchronises.
#pragma once
#include <hip/hip_runtime_api.h>

#include "args.hpp"

namespace ulysses {

// 16-byte vectors one block of the relayout / copy kernels moves.
uint32_t relayout_vectors_per_block();
// 16-byte vectors (one per lane) one block of the fused kernel handles.
uint32_t fused_vectors_per_block();

// Relayout pass: grid (grid_x, planes).
hipError_t launch_relayout(const RelayoutArgs &a, uint32_t grid_x, uint32_t planes,
                           hipStream_t stream);

// Fused QK RMSNorm + RoPE mode-0 pass over q and k: grid (grid_x, planes, 2).
hipError_t launch_fused(const FusedArgs &a, uint32_t grid_x, uint32_t planes,
                        hipStream_t stream);

}  // namespace ulysses
