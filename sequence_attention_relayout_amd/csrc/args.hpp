// Kernel argument blocks shared by the host plan and the HIP kernels.
//
// Plain C++ types only (no HIP headers), so the plan that fills them builds
// and is unit-tested without a GPU.  Every block is passed to its kernel by
// value through the kernarg segment; each stays under 4 KiB (checked below).
#pragma once
#include <cstdint>

namespace ulysses {

constexpr int kMaxWorld = 8;
constexpr int kMaxPieces = kMaxWorld * kMaxWorld;
// Tensors one relayout launch can move (q, k, v and a gate: QKVG).
constexpr int kMaxTensors = 4;
// A row of any shard is at most this many 16-byte vectors (512 KiB).  The
// kernels split a block's vector range into rows with a 32-bit
// multiply-high whose numerators stay below 2^16 under this bound.
constexpr uint32_t kMaxRowVectors = 32768;

// One (source rank j -> destination rank r) region of one batch plane: `rows`
// rows of `vpr` 16-byte vectors, contiguous within each row on both sides.
// Offsets and pitches are in 16-byte vectors.
struct PieceArgs {
    uint32_t nvec;        // rows * vpr
    uint32_t vpr;         // vectors per row
    uint32_t magic;       // floor(2^32 / vpr) + 1 when vpr >= 2, unused when vpr == 1
    uint32_t src_pitch;   // row pitch in the source shard
    uint32_t dst_pitch;   // row pitch in the destination shard
    uint32_t src_off;     // first vector within the source plane
    uint32_t dst_off;     // first vector within the destination plane
    uint32_t src_row0;    // sequence position of the piece's first source row
                          // (global position of row 0; used by the fused path)
    uint8_t j, r;         // source and destination rank
    uint8_t vpr_s1, vpr_s2;   // shifts of the exact division by vpr (div32)
    uint32_t vpr_m;           // multiplier of the exact division by vpr (div32)
};

// floor(n / d) for every 32-bit n, from the multiplier and shifts that
// div32_magic gives for d (Granlund & Montgomery, "Division by invariant
// integers using multiplication", 1994, Figure 4.1).  constexpr, so the HIP
// kernels call the same function; on the GPU a block-uniform n compiles to
// scalar instructions.
constexpr uint32_t div32(uint32_t n, uint32_t m, uint32_t s1, uint32_t s2) {
    const uint32_t t = static_cast<uint32_t>((uint64_t{n} * m) >> 32);
    return (t + ((n - t) >> s1)) >> s2;
}

struct Div32Magic {
    uint32_t m;
    uint8_t s1, s2;
};

// Multiplier and shifts of div32 for a divisor 1 <= d <= 2^31:
// l = ceil(log2 d), m = floor(2^32 * (2^l - d) / d) + 1, s1 = min(l, 1),
// s2 = max(l - 1, 0).
constexpr Div32Magic div32_magic(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d) ++l;
    const uint64_t m = ((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1;
    return Div32Magic{static_cast<uint32_t>(m), static_cast<uint8_t>(l > 0 ? 1 : 0),
                      static_cast<uint8_t>(l > 0 ? l - 1 : 0)};
}

// Launch table for one relayout pass: grid.x walks the pieces' blocks, grid.y
// the batch planes, grid.z the tensors (all of one plan's geometry).  Block x
// belongs to the piece p with blk_begin[p] <= x < blk_begin[p + 1]; unused
// entries hold 0xFFFFFFFF.
struct RelayoutArgs {
    const unsigned char *src[kMaxTensors][kMaxWorld];
    unsigned char *dst[kMaxTensors][kMaxWorld];
    uint64_t src_plane[kMaxWorld];   // vectors per batch plane of source shard j
    uint64_t dst_plane[kMaxWorld];   // vectors per batch plane of destination shard r
    uint32_t blk_begin[kMaxPieces];
    PieceArgs piece[kMaxPieces];
    uint32_t src_plane0;             // batch plane of grid.y == 0, source side
    uint32_t dst_plane0;             // batch plane of grid.y == 0, destination side
    // Row-band traversal (fill_relayout_bands): the pieces sharing one
    // row-sharded shard g (source j in mode 0, destination r in mode 1) sit
    // at piece[g * world + k]; their blocks interleave band by band: block
    // grp_begin[g] + band * world + k moves rows [band*band_rows,
    // (band+1)*band_rows) of piece (g, k).  Unused entries hold 0xFFFFFFFF.
    // With band_vecs != 0 a band is instead band_vecs consecutive vectors of
    // the piece (the same rows across the group when its rows are equally
    // wide); a block whose band starts past its piece does nothing.
    uint32_t grp_begin[kMaxWorld];
    uint32_t world;
    uint32_t band_rows;
    uint32_t band_vecs;
    // Row-aligned chunk traversal (fill_relayout_aligned; band_vecs == 0 and
    // chunks_per_band != 0), for groups whose pieces have unequal row widths:
    // a band is band_rows rows of every piece of the group, cut into chunks
    // of chunk_vecs vectors (a whole number per piece);
    // block grp_begin[g] + band * chunks_per_band + q takes chunk
    // q - chunk_begin[k] of piece (g, k), k being the last piece with
    // chunk_begin[k] <= q.  band_m/band_s1/band_s2 divide exactly by
    // chunks_per_band (div32).
    uint32_t chunk_begin[kMaxWorld + 1];
    uint32_t chunks_per_band;
    uint32_t chunk_vecs;
    uint32_t band_m;
    uint32_t band_s1, band_s2;
};

// The fused QK-norm + RoPE mode-0 pass: the same piece table for q and k
// (grid.z picks the tensor), plus the row-op parameters.  Vector counts,
// offsets and pitches of the pieces are in units of the kernel's vectors per
// lane (see to_units in the plan).
struct FusedArgs {
    const unsigned char *src[2][kMaxWorld];
    unsigned char *dst[2][kMaxWorld];
    uint64_t src_plane[kMaxWorld];
    uint64_t dst_plane[kMaxWorld];
    uint32_t blk_begin[kMaxPieces];
    PieceArgs piece[kMaxPieces];
    const float *gamma[2];
    const float *rope_cos;
    const float *rope_sin;
    float eps;
    float inv_d;                     // 1/d, exact (d is a power of two)
    uint32_t d;                      // head dimension
    uint32_t plane0;                 // batch plane of grid.y == 0
    // band traversal as in RelayoutArgs (band_vecs != 0), else blk_begin
    uint32_t grp_begin[kMaxWorld];
    uint32_t world;
    uint32_t band_vecs;
    // exact division by world (div32): a block's band within its group
    uint32_t world_m;
    uint32_t world_s1, world_s2;
};

static_assert(sizeof(RelayoutArgs) <= 4096, "kernel argument block over 4 KiB");
static_assert(sizeof(FusedArgs) <= 4096, "kernel argument block over 4 KiB");

}  // namespace ulysses
