// Kernel argument blocks shared by the host plan and the HIP kernels.
//
// Plain C++ types only (no HIP headers), so the plan that fills them builds
// and is unit-tested without a GPU.  Every block is passed to its kernel by
// value through the kernarg segment; each stays under 4 KiB (checked below).
// Offsets, pitches and sizes are in 16-byte vectors.
#pragma once
#include <cstdint>

namespace ulysses {

constexpr int kMaxWorld = 8;
// Tensors one relayout launch can move (q, k, v and a gate: QKVG).
constexpr int kMaxTensors = 4;
// A row of any shard is at most this many 16-byte vectors (512 KiB).  The
// kernels split a block's vectors into rows with a 32-bit multiply-high whose
// numerators stay below 2^16 under this bound.
constexpr uint32_t kMaxRowVectors = 32768;
// Threshold entries past the world; no key reaches them.
constexpr uint32_t kNone = 0xFFFFFFFFu;
// Threads per block: one wave per block for the relayout and the plane copy,
// two for the fused pass.
constexpr uint32_t kRelayoutBlock = 64;
constexpr uint32_t kFusedBlock = 128;
// Bytes of the static device array that holds the windows of the
// plane-at-a-time call for callers that cannot allocate (one array per GPU
// the library runs on, kept until the process ends), and the alignment of
// each window within it.
constexpr uint64_t kStaticWindowBytes = uint64_t{64} << 20;
constexpr uint64_t kStaticWindowAlign = 256;

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

// Row split of the vectors of one shard: vector v of a plane sits at row
// v / vpr, column v % vpr.  The block's first vector is split with div32
// (any 32-bit numerator); a lane's offset from there (below 2^16) with one
// multiply-high by magic = floor(2^32 / vpr) + 1 (exact for numerators below
// 2^16 and 2 <= vpr <= 2^16; vpr == 1 is handled directly).
struct RowSplit {
    uint32_t vpr;
    uint32_t magic;
    uint32_t m;
    uint8_t s1, s2;
    uint16_t pad;
};

// One relayout pass, walking every destination vector once (a gather):
// grid.x takes the destination shards one after another, 64 consecutive
// vectors of a shard per block; grid.y the batch planes; grid.z the tensors
// (all of one plan's geometry).  The caller points src and dst at the first
// batch plane of the launch, so a launch of one plane needs no plane terms.
//
// Destination shard r is partitioned among the source ranks: piece (j -> r)
// covers the destination rows (mode 0) or columns (mode 1) from
// bound[j] up to bound[j + 1].  The owner of a destination vector at (row,
// col) is the number of q in [1, world) with bound[q] <= key, key = row in
// mode 0 and col in mode 1 (an empty piece has bound[j] == bound[j + 1] and
// is never chosen).  Its source vector within source plane j is
// off[r][j] + row * pitch[r][j] + col: the piece's source offset, moved to
// the destination frame's origin (it may be negative).
struct RelayoutArgs {
    const unsigned char *src[kMaxTensors][kMaxWorld];
    unsigned char *dst[kMaxTensors][kMaxWorld];
    uint64_t src_plane[kMaxWorld];          // vectors per batch plane of source shard j
    uint64_t dst_plane[kMaxWorld];          // vectors per batch plane of destination shard r
    int64_t off[kMaxWorld][kMaxWorld];      // [r][j]
    uint32_t pitch[kMaxWorld][kMaxWorld];   // [r][j]
    uint32_t blk_begin[kMaxWorld];          // first block of destination r; kNone past the world
    uint32_t nvec[kMaxWorld];               // vectors per plane of destination r
    RowSplit row[kMaxWorld];                // rows of destination r
    uint32_t bound[kMaxWorld];              // [0] unused; kNone past the world
    uint32_t key_col;                       // 0: owner by row (mode 0), 1: by column (mode 1)
};

// A contiguous copy of nvec[r] vectors per rank, src[r] to dst[r] (one batch
// plane: the window and the plane the caller points dst at); grid.x takes the
// ranks one after another, 64 vectors per block.
struct CopyArgs {
    const unsigned char *src[kMaxWorld];
    unsigned char *dst[kMaxWorld];
    uint32_t blk_begin[kMaxWorld];
    uint32_t nvec[kMaxWorld];
};

// The fused QK-norm + RoPE mode-0 pass, walking every destination vector
// once (a gather, like RelayoutArgs in mode 0): grid.x takes the destination
// shards one after another, kFusedBlock consecutive vectors of a shard per
// block; grid.y the batch planes (the caller points src and dst at the
// launch's first plane).  Each lane moves the same vector of q and of k.
//
// Destination shard r's rows are sequence positions s, of
// row[r].vpr = H_r * d / 8 vectors.  Row s comes from source rank j = the
// number of q in [1, world) with bound[q] <= s, vector (s, col) at
// off[r][j] + s * pitch + col of source plane j, and takes rotary row s.
struct FusedArgs {
    const unsigned char *src[2][kMaxWorld];   // [0] q, [1] k
    unsigned char *dst[2][kMaxWorld];
    uint64_t src_plane[kMaxWorld];            // vectors per batch plane of source shard j
    uint64_t dst_plane[kMaxWorld];            // vectors per batch plane of destination shard r
    int64_t off[kMaxWorld][kMaxWorld];        // [r][j]
    uint32_t pitch;                           // vectors per source row (every j)
    uint32_t blk_begin[kMaxWorld];            // first block of destination r; kNone past the world
    uint32_t nvec[kMaxWorld];                 // vectors per plane of destination r
    RowSplit row[kMaxWorld];                  // rows of destination r
    uint32_t bound[kMaxWorld];                // [0] unused; kNone past the world
    const float *gamma[2];
    const float *rope_cos;
    const float *rope_sin;
    float eps;
    float inv_d;                              // 1/d, exact (d is a power of two)
    uint32_t half_d;                          // d / 2: floats per rotary row
};

static_assert(sizeof(RelayoutArgs) <= 4096, "kernel argument block over 4 KiB");
static_assert(sizeof(CopyArgs) <= 4096, "kernel argument block over 4 KiB");
static_assert(sizeof(FusedArgs) <= 4096, "kernel argument block over 4 KiB");

}  // namespace ulysses
