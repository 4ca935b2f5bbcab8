// Host-side plan of the Ulysses 4D relayout: validation, offsets, the piece
// table and launch tables.  No HIP headers: it builds and is tested on a
// machine without a GPU.
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

// One (j -> r) region of a batch plane, in bytes.
struct Piece {
    int j = 0, r = 0;
    int64_t rows = 0;        // rows of the region
    int64_t row_bytes = 0;   // contiguous bytes per row (same on both sides)
    int64_t src_off = 0;     // byte offset of the first row within source plane j
    int64_t dst_off = 0;     // byte offset of the first row within destination plane r
    int64_t src_pitch = 0;   // bytes between consecutive source rows
    int64_t dst_pitch = 0;   // bytes between consecutive destination rows
    int64_t seq_pos0 = 0;    // global sequence position of the region's first row
};

struct ModeGeom {
    Piece piece[kMaxPieces];            // index j * world + r
    int64_t src_plane[kMaxWorld] = {};  // bytes per batch plane, source shard j
    int64_t dst_plane[kMaxWorld] = {};  // bytes per batch plane, destination shard r
    int64_t src_shape[kMaxWorld][4] = {};
    int64_t dst_shape[kMaxWorld][4] = {};
    int64_t window_bytes = 0;           // max_r dst_plane[r]
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

// Order in which pieces take consecutive blocks of the grid.
enum PieceOrder : int {
    kDstMajor = 0,   // for r: for j   (destination shards filled one after another)
    kSrcMajor = 1,   // for j: for r   (source shards drained one after another)
};

// Launch table of one relayout pass of `mode` with `vec_per_block` 16-byte
// vectors per block.  Pointers and plane bases are left to the caller.
// Returns the number of blocks along grid.x (0 when nothing moves), as a
// 64-bit count: the caller checks it against the launch limits before use.
uint64_t fill_relayout(const Plan &p, int mode, uint32_t vec_per_block, PieceOrder order,
                       RelayoutArgs *a);

// Row-band launch table of one relayout pass of `mode` (see
// RelayoutArgs::grp_begin): bands of `band_rows` rows.  Returns grid.x.
uint64_t fill_relayout_bands(const Plan &p, int mode, uint32_t band_rows, RelayoutArgs *a);

// Vector-band launch table: bands of `band_vecs` vectors of each piece,
// interleaved over the group as for row bands.  Returns grid.x.
uint64_t fill_relayout_vbands(const Plan &p, int mode, uint32_t band_vecs, RelayoutArgs *a);

// Row-aligned chunk table (see RelayoutArgs::chunk_begin) when the pieces of
// a group differ in row width: bands of R rows, R the fewest rows that make
// every piece's band a whole number of chunk_vecs-vector chunks, one chunk
// per block, so blocks running side by side cover the same rows of every
// piece.  Returns grid.x, or 0 without touching *a when the pieces of a group
// all have the same width, or when max_chunks != 0 and some piece's band
// would hold more than max_chunks chunks (then fill_relayout_vbands applies).
uint64_t fill_relayout_aligned(const Plan &p, int mode, uint32_t chunk_vecs, uint32_t max_chunks,
                               RelayoutArgs *a);

// Band height so that one band of the widest piece moves about
// `target_vectors` 16-byte vectors (at least one row).
uint32_t band_rows_for(const Plan &p, int mode, uint32_t target_vectors);

// Launch table of the plane copy from the W windows (one destination plane
// each) into the destination shards, for the band kernel: group r holds the
// one piece copying window r (equal row pitches on both sides), in bands of
// `band_vecs` vectors.
uint64_t fill_window_copy(const Plan &p, int mode, uint32_t band_vecs, RelayoutArgs *a);

// Rescales a launch table from 16-byte vectors to units of `vpl` vectors
// (vector counts, offsets, pitches, plane sizes and band width divided by
// vpl, magic multipliers recomputed); block ranges are unchanged, so the
// table must have been filled with vec_per_block (or band_vecs) = units per
// block * vpl.  Returns
// false, leaving *a unusable, if any count is not a multiple of vpl.
bool to_units(RelayoutArgs *a, uint32_t vpl);

// Magic multiplier for the kernels' division by vpr (see PieceArgs::magic).
uint32_t row_magic(uint32_t vpr);

}  // namespace ulysses
