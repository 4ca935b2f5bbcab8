// Host-side plan of the Ulysses 4D relayout: validation, offsets, the piece
// table and the kernels' launch tables.  No HIP headers: it builds and is
// tested on a machine without a GPU.
//
// The addressing follows the pages' description of the exchange as pitched
// copies whose source and destination strides perform the sequence/head
// permutation (fast-ulysses 0.1.0 introduction and "What it does";
// fast-ulysses 0.2.1 "Key features"), with one region per (source rank,
// destination rank) pair.
#pragma once
#include <cstdint>
#include <string>

#include "args.hpp"

namespace ulysses {

// Status codes; the same values as enum ulysses_status in ulysses.h.
enum Status : int {
    kOk = 0,
    kEInval = -1,
    kEAlign = -2,
    kEDtype = -3,
    kEWindow = -4,
    kEOverlap = -5,
    kEHip = -6,
};

// Bytes per element of an ulysses_dtype value, or -1 if unknown.
int64_t dtype_size(int dtype);

// One (j -> r) region of a batch plane, in bytes: `rows` rows of `row_bytes`
// contiguous bytes on both sides.  Its first byte is at src_off within
// source plane j and at dst_off within destination plane r, consecutive rows
// src_pitch and dst_pitch apart.  In the frame of each shard (rows of its
// own pitch) the region is the rectangle of rows from *_row0 and bytes from
// *_col0, so *_off = *_row0 * *_pitch + *_col0.
struct Piece {
    int j = 0, r = 0;
    int64_t rows = 0;
    int64_t row_bytes = 0;
    int64_t src_off = 0, dst_off = 0;
    int64_t src_pitch = 0, dst_pitch = 0;
    int64_t src_row0 = 0, src_col0 = 0;
    int64_t dst_row0 = 0, dst_col0 = 0;
};

struct ModeGeom {
    Piece piece[kMaxWorld * kMaxWorld];   // index j * world + r
    int64_t src_plane[kMaxWorld] = {};    // bytes per batch plane, source shard j
    int64_t dst_plane[kMaxWorld] = {};    // bytes per batch plane, destination shard r
    int64_t src_shape[kMaxWorld][4] = {};
    int64_t dst_shape[kMaxWorld][4] = {};
    int64_t window_bytes = 0;             // max_r dst_plane[r]
};

struct Plan {
    int world = 0;
    int64_t b = 0, d = 0;
    int dtype = 0;
    int64_t esz = 0;
    int64_t window_cap = 0;
    int64_t S[kMaxWorld] = {}, H[kMaxWorld] = {};
    int64_t seq_off[kMaxWorld + 1] = {}, head_off[kMaxWorld + 1] = {};
    int64_t s_global = 0, n_global = 0;
    int64_t G = 0;                  // bytes of a sequence-sharded row: n_global*d*esz
    int64_t R[kMaxWorld] = {};      // bytes of a head-sharded row of rank r: H_r*d*esz
    ModeGeom mode[2];
};

// Validates and fills *p.  On failure returns a negative Status and sets *msg.
int plan_build(Plan *p, int world, int64_t b, int64_t d, const int64_t *seq_splits,
               const int64_t *head_splits, int dtype, int64_t window_cap, std::string *msg);

// Launch table of one relayout pass of `mode` (the gather of RelayoutArgs).
// Pointers are left to the caller.  Returns the number of blocks along grid.x
// (0 when nothing moves) as a 64-bit count that the caller checks against the
// launch limits.
uint64_t fill_relayout(const Plan &p, int mode, RelayoutArgs *a);

// Launch table of the copy of one batch plane from each of the W windows
// into the destination shards of `mode` (CopyArgs).  Returns grid.x.
uint64_t fill_plane_copy(const Plan &p, int mode, CopyArgs *a);

// Launch table of the fused mode-0 gather (FusedArgs) with kFusedBlock
// vectors per block; pointers, gains, tables and eps are left to the caller.
// Returns grid.x.
uint64_t fill_fused(const Plan &p, FusedArgs *a);

// Magic multiplier of the kernels' lane division by vpr (see RowSplit).
uint32_t row_magic(uint32_t vpr);

// The full row split of vpr vectors per row (vpr >= 1).
RowSplit row_split(uint32_t vpr);

}  // namespace ulysses
