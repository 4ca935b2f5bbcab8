// Host-side plan of the Ulysses 4D relayout (see plan.hpp).
#include "plan.hpp"

#include <cstring>

namespace ulysses {

int64_t dtype_size(int dtype) {
    switch (dtype) {
    case 0: return 2;   // bf16
    case 1: return 2;   // fp16
    case 2: return 4;   // fp32
    case 3: return 1;   // fp8 e4m3fn
    case 4: return 1;   // fp8 e5m2
    case 5: return 1;   // int8
    case 6: return 1;   // uint8
    default: return -1;
    }
}

static int fail(std::string *msg, int code, const std::string &text) {
    if (msg) *msg = text;
    return code;
}

uint32_t row_magic(uint32_t vpr) {
    // floor(n / vpr) == (n * m) >> 32 for every n < 2^16 when
    // m = floor(2^32 / vpr) + 1 and 2 <= vpr <= 2^16 (Granlund & Montgomery,
    // "Division by invariant integers using multiplication", 1994, Thm 4.2
    // with N = 16, l = 16).  vpr == 1 is handled by the kernels directly.
    if (vpr < 2) return 0;
    return static_cast<uint32_t>((uint64_t{1} << 32) / vpr + 1);
}

RowSplit row_split(uint32_t vpr) {
    if (vpr < 1) vpr = 1;
    const Div32Magic dm = div32_magic(vpr);
    RowSplit s;
    s.vpr = vpr;
    s.magic = row_magic(vpr);
    s.m = dm.m;
    s.s1 = dm.s1;
    s.s2 = dm.s2;
    s.pad = 0;
    return s;
}

// Sizes are bounded before they are multiplied, so no product below
// overflows: a head row d*esz and a full row G at most 512 KiB (2^19), a
// split at most 2^40 positions or 2^24 heads, one batch plane of a shard
// below 2^31 vectors, and a whole shard (all planes) at most 2^58 bytes.
constexpr int64_t kMaxRowBytes = int64_t{kMaxRowVectors} * 16;
constexpr int64_t kMaxSeqSplit = int64_t{1} << 40;
constexpr int64_t kMaxHeadSplit = int64_t{1} << 24;
constexpr int64_t kMaxPlaneBytes = (int64_t{1} << 31) * 16;
constexpr int64_t kMaxShardBytes = int64_t{1} << 58;

int plan_build(Plan *p, int world, int64_t b, int64_t d, const int64_t *seq_splits,
               const int64_t *head_splits, int dtype, int64_t window_cap, std::string *msg) {
    if (!p) return fail(msg, kEInval, "plan output pointer is null");
    *p = Plan{};
    if (world < 1 || world > kMaxWorld)
        return fail(msg, kEInval, "world must be in [1, 8], got " + std::to_string(world));
    if (b < 1) return fail(msg, kEInval, "batch b must be >= 1");
    if (b > (int64_t{1} << 31)) return fail(msg, kEInval, "batch b must be at most 2^31");
    if (d < 1) return fail(msg, kEInval, "head dimension d must be >= 1");
    if (!seq_splits || !head_splits) return fail(msg, kEInval, "split arrays must be non-null");
    if (window_cap < 0) return fail(msg, kEInval, "window_cap_bytes must be >= 0");
    const int64_t esz = dtype_size(dtype);
    if (esz < 0) return fail(msg, kEDtype, "unknown dtype " + std::to_string(dtype));
    if (d > kMaxRowBytes / esz)
        return fail(msg, kEInval, "a head row of d = " + std::to_string(d) +
                                      " elements exceeds the 512 KiB row limit");
    const int64_t hb = d * esz;   // one head row of one position
    if (hb % 16 != 0)
        return fail(msg, kEAlign, "d * elem_size = " + std::to_string(hb) +
                                      " bytes is not a multiple of 16");
    p->world = world;
    p->b = b;
    p->d = d;
    p->dtype = dtype;
    p->esz = esz;
    p->window_cap = window_cap;
    for (int j = 0; j < world; ++j) {
        if (seq_splits[j] < 0 || head_splits[j] < 0)
            return fail(msg, kEInval, "splits must be >= 0 (rank " + std::to_string(j) + ")");
        if (seq_splits[j] > kMaxSeqSplit || head_splits[j] > kMaxHeadSplit)
            return fail(msg, kEInval, "split too large (rank " + std::to_string(j) + ")");
        p->S[j] = seq_splits[j];
        p->H[j] = head_splits[j];
        p->seq_off[j + 1] = p->seq_off[j] + seq_splits[j];
        p->head_off[j + 1] = p->head_off[j] + head_splits[j];
    }
    p->s_global = p->seq_off[world];
    p->n_global = p->head_off[world];
    if (p->s_global < 1) return fail(msg, kEInval, "sum of seq_splits must be >= 1");
    if (p->n_global < 1) return fail(msg, kEInval, "sum of head_splits must be >= 1");

    p->G = p->n_global * hb;   // at most 2^27 * 2^19
    if (p->G > kMaxRowBytes)
        return fail(msg, kEInval, "a row of n_global*d*elem_size = " + std::to_string(p->G) +
                                      " bytes exceeds the 512 KiB limit");
    for (int r = 0; r < world; ++r) p->R[r] = p->H[r] * hb;

    // Per-plane shard sizes: below 2^31 vectors each (vector offsets within a
    // plane fit in 31 bits); all b planes of a shard at most 2^58 bytes.
    for (int r = 0; r < world; ++r) {
        const int64_t seq_plane = p->S[r] * p->G;          // (S_r, n_global, d): <= 2^59
        const int64_t head_plane = p->s_global * p->R[r];  // (s_global, H_r, d): <= 2^62
        if (seq_plane >= kMaxPlaneBytes || head_plane >= kMaxPlaneBytes)
            return fail(msg, kEInval, "one batch plane of a shard must stay below 32 GiB");
        const int64_t big = seq_plane > head_plane ? seq_plane : head_plane;
        if (big > 0 && b > kMaxShardBytes / big)
            return fail(msg, kEInval, "batch too large: a shard would exceed 2^58 bytes");
        // mode 0: sequence-sharded in, head-sharded out; mode 1 the reverse
        p->mode[0].src_plane[r] = seq_plane;
        p->mode[0].dst_plane[r] = head_plane;
        p->mode[1].src_plane[r] = head_plane;
        p->mode[1].dst_plane[r] = seq_plane;
        const int64_t seq_shape[4] = {b, p->S[r], p->n_global, d};
        const int64_t head_shape[4] = {b, p->s_global, p->H[r], d};
        std::memcpy(p->mode[0].src_shape[r], seq_shape, sizeof seq_shape);
        std::memcpy(p->mode[0].dst_shape[r], head_shape, sizeof head_shape);
        std::memcpy(p->mode[1].src_shape[r], head_shape, sizeof head_shape);
        std::memcpy(p->mode[1].dst_shape[r], seq_shape, sizeof seq_shape);
    }
    for (int m = 0; m < 2; ++m) {
        int64_t w = 0;
        for (int r = 0; r < world; ++r)
            if (p->mode[m].dst_plane[r] > w) w = p->mode[m].dst_plane[r];
        p->mode[m].window_bytes = w;
    }

    // The piece table.  Mode 0, piece j -> r: rows of source shard j (every
    // local row s, global position seq_off_j + s), taking the head block of
    // r (bytes from head_off_r * d * esz within a row of G bytes) into rows
    // seq_off_j .. seq_off_j + S_j of destination r (rows of R_r bytes).
    // Mode 1, piece j -> r: the rows seq_off_r .. seq_off_r + S_r of source j
    // (rows of R_j bytes) land at head block j of the rows of destination r.
    for (int j = 0; j < world; ++j)
        for (int r = 0; r < world; ++r) {
            Piece &a = p->mode[0].piece[j * world + r];
            a.j = j;
            a.r = r;
            a.rows = p->S[j];
            a.row_bytes = p->R[r];
            a.src_pitch = p->G;
            a.src_row0 = 0;
            a.src_col0 = p->head_off[r] * hb;
            a.dst_pitch = p->R[r];
            a.dst_row0 = p->seq_off[j];
            a.dst_col0 = 0;

            Piece &c = p->mode[1].piece[j * world + r];
            c.j = j;
            c.r = r;
            c.rows = p->S[r];
            c.row_bytes = p->R[j];
            c.src_pitch = p->R[j];
            c.src_row0 = p->seq_off[r];
            c.src_col0 = 0;
            c.dst_pitch = p->G;
            c.dst_row0 = 0;
            c.dst_col0 = p->head_off[j] * hb;
        }
    for (int m = 0; m < 2; ++m)
        for (int q = 0; q < world * world; ++q) {
            Piece &pc = p->mode[m].piece[q];
            pc.src_off = pc.src_row0 * pc.src_pitch + pc.src_col0;
            pc.dst_off = pc.dst_row0 * pc.dst_pitch + pc.dst_col0;
        }
    return kOk;
}

uint64_t fill_relayout(const Plan &p, int mode, RelayoutArgs *a) {
    std::memset(a, 0, sizeof *a);
    const ModeGeom &g = p.mode[mode];
    const int w = p.world;
    for (int q = 0; q < kMaxWorld; ++q) {
        a->blk_begin[q] = kNone;
        a->bound[q] = kNone;
    }
    a->key_col = mode == 0 ? 0u : 1u;
    // Pieces sharing destination r partition its rows (mode 0: by source
    // sequence range) or columns (mode 1: by source head block); the same
    // bounds hold for every r.
    for (int j = 1; j < w; ++j) {
        const Piece &pc = g.piece[j * w + 0];
        a->bound[j] = static_cast<uint32_t>(mode == 0 ? pc.dst_row0 : pc.dst_col0 / 16);
    }
    uint64_t blocks = 0;
    for (int r = 0; r < w; ++r) {
        a->src_plane[r] = static_cast<uint64_t>(g.src_plane[r] / 16);
        a->dst_plane[r] = static_cast<uint64_t>(g.dst_plane[r] / 16);
        const int64_t row_bytes = mode == 0 ? p.R[r] : p.G;
        a->row[r] = row_split(static_cast<uint32_t>(row_bytes / 16));
        a->nvec[r] = static_cast<uint32_t>(g.dst_plane[r] / 16);
        a->blk_begin[r] = static_cast<uint32_t>(blocks);
        blocks += (uint64_t(a->nvec[r]) + kRelayoutBlock - 1) / kRelayoutBlock;
        for (int j = 0; j < w; ++j) {
            // destination (row, col) of piece j -> r reads source vector
            // src_off + (row - dst_row0) * src_pitch + (col - dst_col0)
            const Piece &pc = g.piece[j * w + r];
            a->off[r][j] =
                (pc.src_off - pc.dst_row0 * pc.src_pitch - pc.dst_col0) / 16;
            a->pitch[r][j] = static_cast<uint32_t>(pc.src_pitch / 16);
        }
    }
    return blocks;
}

uint64_t fill_plane_copy(const Plan &p, int mode, CopyArgs *a) {
    std::memset(a, 0, sizeof *a);
    const ModeGeom &g = p.mode[mode];
    for (int q = 0; q < kMaxWorld; ++q) a->blk_begin[q] = kNone;
    uint64_t blocks = 0;
    for (int r = 0; r < p.world; ++r) {
        a->nvec[r] = static_cast<uint32_t>(g.dst_plane[r] / 16);
        a->blk_begin[r] = static_cast<uint32_t>(blocks);
        blocks += (uint64_t(a->nvec[r]) + kRelayoutBlock - 1) / kRelayoutBlock;
    }
    return blocks;
}

uint64_t fill_fused(const Plan &p, FusedArgs *a) {
    std::memset(a, 0, sizeof *a);
    const ModeGeom &g = p.mode[0];
    const int w = p.world;
    for (int q = 0; q < kMaxWorld; ++q) {
        a->blk_begin[q] = kNone;
        a->bound[q] = kNone;
    }
    // the source sequence ranges partition every destination's rows
    for (int j = 1; j < w; ++j) a->bound[j] = static_cast<uint32_t>(g.piece[j * w].dst_row0);
    a->pitch = static_cast<uint32_t>(p.G / 16);
    a->half_d = static_cast<uint32_t>(p.d / 2);
    a->inv_d = 1.0f / static_cast<float>(p.d);   // exact for the power-of-two d accepted
    uint64_t blocks = 0;
    for (int r = 0; r < w; ++r) {
        a->src_plane[r] = static_cast<uint64_t>(g.src_plane[r] / 16);
        a->dst_plane[r] = static_cast<uint64_t>(g.dst_plane[r] / 16);
        a->row[r] = row_split(static_cast<uint32_t>(p.R[r] / 16));
        a->nvec[r] = static_cast<uint32_t>(g.dst_plane[r] / 16);
        a->blk_begin[r] = static_cast<uint32_t>(blocks);
        blocks += (uint64_t(a->nvec[r]) + kFusedBlock - 1) / kFusedBlock;
        for (int j = 0; j < w; ++j) {
            // destination (row, col) of piece j -> r reads source vector
            // src_off + (row - dst_row0) * src_pitch + (col - dst_col0)
            const Piece &pc = g.piece[j * w + r];
            a->off[r][j] = (pc.src_off - pc.dst_row0 * pc.src_pitch - pc.dst_col0) / 16;
        }
    }
    return blocks;
}

}  // namespace ulysses
