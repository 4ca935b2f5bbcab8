// Launchers of the gfx950 kernels (kernels.hip).  Each returns the HIP
// runtime's status of the launch; none synchronises.
#pragma once
#include <hip/hip_runtime_api.h>

#include "args.hpp"

namespace ulysses {

// Most blocks along grid.y (batch planes) of one launch; callers split
// larger batches over several launches.
constexpr uint32_t kMaxGridY = 65535;
// Threads per block of the relayout / copy kernels and of the fused kernel
// chosen for head dimension d (for the grid.x * block <= 2^32 bound).
uint32_t relayout_block_threads();
uint32_t fused_block_threads(uint32_t d);

// 16-byte vectors one block of the relayout / copy kernels moves.
uint32_t relayout_vectors_per_block();
// Units one block of the fused kernel handles (one unit per lane); a unit is
// fused_vectors_per_lane(d) consecutive 16-byte vectors of one head row.
uint32_t fused_units_per_block();
uint32_t fused_vectors_per_lane(uint32_t d);
// Vectors per band of the band kernel that takes head dimension d = 128 (it
// reads a vector-band table, fill_relayout_vbands, in 16-byte vectors, and
// moves q and k in one block), or 0 when d takes fused_kernel.
uint32_t fused_band_vectors(uint32_t d);

// Relayout pass over `tensors` tensors of one geometry: grid (grid_x,
// planes, tensors).
hipError_t launch_relayout(const RelayoutArgs &a, uint32_t grid_x, uint32_t planes,
                           uint32_t tensors, hipStream_t stream);

// Fused QK RMSNorm + RoPE mode-0 pass over q and k: grid (grid_x, planes, 2),
// or (grid_x, planes, 1) for the band kernel.
hipError_t launch_fused(const FusedArgs &a, uint32_t grid_x, uint32_t planes,
                        hipStream_t stream);

}  // namespace ulysses
