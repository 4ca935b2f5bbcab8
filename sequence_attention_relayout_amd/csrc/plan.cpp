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

int plan_build(Plan *p, int world, int64_t b, int64_t d, const int64_t *seq_splits,
               const int64_t *head_splits, int dtype, int64_t window_cap, std::string *msg) {
    if (!p) return fail(msg, kEInval, "plan output pointer is null");
    *p = Plan{};
    if (world < 1 || world > kMaxWorld)
        return fail(msg, kEInval, "world must be in [1, 8], got " + std::to_string(world));
    if (b < 1) return fail(msg, kEInval, "batch b must be >= 1");
    if (d < 1) return fail(msg, kEInval, "head dimension d must be >= 1");
    if (!seq_splits || !head_splits) return fail(msg, kEInval, "split arrays must be non-null");
    if (window_cap < 0) return fail(msg, kEInval, "window_cap_bytes must be >= 0");
    const int64_t esz = dtype_size(dtype);
    if (esz < 0) return fail(msg, kEDtype, "unknown dtype " + std::to_string(dtype));
    if ((d * esz) % 16 != 0)
        return fail(msg, kEAlign, "d * elem_size = " + std::to_string(d * esz) +
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
        if (seq_splits[j] > (int64_t{1} << 40) || head_splits[j] > (int64_t{1} << 24))
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

    const int64_t hb = d * esz;   // one head row of one position
    p->G = p->n_global * hb;
    const int64_t max_row = int64_t{kMaxRowVectors} * 16;
    if (p->G > max_row)
        return fail(msg, kEInval, "a row of n_global*d*elem_size = " + std::to_string(p->G) +
                                      " bytes exceeds the 512 KiB limit");
    for (int r = 0; r < world; ++r) p->R[r] = p->H[r] * hb;

    // Per-plane shard sizes, bounded so that vector offsets fit in 31 bits.
    const int64_t max_plane = (int64_t{1} << 31) * 16;
    for (int r = 0; r < world; ++r) {
        const int64_t seq_plane = p->S[r] * p->G;          // (S_r, n_global, d)
        const int64_t head_plane = p->s_global * p->R[r];  // (s_global, H_r, d)
        if (seq_plane >= max_plane || head_plane >= max_plane)
            return fail(msg, kEInval, "one batch plane of a shard must stay below 32 GiB");
        if (b > (int64_t{1} << 31))
            return fail(msg, kEInval, "batch too large");
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
    // r (offset head_off_r * d * esz within a row of G bytes) into rows
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
            a.src_off = p->head_off[r] * hb;
            a.src_pitch = p->G;
            a.dst_off = p->seq_off[j] * p->R[r];
            a.dst_pitch = p->R[r];
            a.seq_pos0 = p->seq_off[j];

            Piece &c = p->mode[1].piece[j * world + r];
            c.j = j;
            c.r = r;
            c.rows = p->S[r];
            c.row_bytes = p->R[j];
            c.src_off = p->seq_off[r] * p->R[j];
            c.src_pitch = p->R[j];
            c.dst_off = p->head_off[j] * hb;
            c.dst_pitch = p->G;
            c.seq_pos0 = p->seq_off[r];
        }
    return kOk;
}

// The exact 32-bit division by o->vpr (a piece without rows keeps d = 1).
static void set_vpr_division(PieceArgs *o) {
    const Div32Magic dm = div32_magic(o->vpr > 0 ? o->vpr : 1);
    o->vpr_m = dm.m;
    o->vpr_s1 = dm.s1;
    o->vpr_s2 = dm.s2;
}

static void fill_piece_args(const Piece &pc, PieceArgs *o) {
    const uint32_t vpr = static_cast<uint32_t>(pc.row_bytes / 16);
    o->vpr = vpr;
    o->nvec = static_cast<uint32_t>(pc.rows * vpr);
    o->magic = row_magic(vpr);
    o->src_pitch = static_cast<uint32_t>(pc.src_pitch / 16);
    o->dst_pitch = static_cast<uint32_t>(pc.dst_pitch / 16);
    o->src_off = static_cast<uint32_t>(pc.src_off / 16);
    o->dst_off = static_cast<uint32_t>(pc.dst_off / 16);
    o->src_row0 = static_cast<uint32_t>(pc.seq_pos0);
    o->j = static_cast<uint8_t>(pc.j);
    o->r = static_cast<uint8_t>(pc.r);
    set_vpr_division(o);
}

static void clear_table(RelayoutArgs *a) {
    std::memset(a, 0, sizeof *a);
    for (int q = 0; q < kMaxPieces; ++q) a->blk_begin[q] = 0xFFFFFFFFu;
    for (int q = 0; q < kMaxWorld; ++q) a->grp_begin[q] = 0xFFFFFFFFu;
}

uint32_t band_rows_for(const Plan &p, int mode, uint32_t target_vectors) {
    int64_t widest = 1;
    for (int q = 0; q < p.world * p.world; ++q) {
        const int64_t vpr = p.mode[mode].piece[q].row_bytes / 16;
        if (vpr > widest) widest = vpr;
    }
    const int64_t t = target_vectors / widest;
    return static_cast<uint32_t>(t < 1 ? 1 : t);
}

uint64_t fill_relayout_bands(const Plan &p, int mode, uint32_t band_rows, RelayoutArgs *a) {
    clear_table(a);
    const ModeGeom &g = p.mode[mode];
    for (int r = 0; r < p.world; ++r) {
        a->src_plane[r] = static_cast<uint64_t>(g.src_plane[r] / 16);
        a->dst_plane[r] = static_cast<uint64_t>(g.dst_plane[r] / 16);
    }
    a->world = static_cast<uint32_t>(p.world);
    a->band_rows = band_rows;
    uint64_t blocks = 0;
    for (int grp = 0; grp < p.world; ++grp) {
        // every piece of the group has S_grp rows (mode 0: source rank j =
        // grp; mode 1: destination rank r = grp)
        const int64_t rows = p.S[grp];
        const int64_t bands = (rows + band_rows - 1) / band_rows;
        for (int k = 0; k < p.world; ++k) {
            const int j = mode == 0 ? grp : k;
            const int r = mode == 0 ? k : grp;
            fill_piece_args(g.piece[j * p.world + r], &a->piece[grp * p.world + k]);
        }
        a->grp_begin[grp] = static_cast<uint32_t>(blocks);
        blocks += static_cast<uint64_t>(bands) * p.world;
    }
    return blocks;
}

uint64_t fill_relayout(const Plan &p, int mode, uint32_t vec_per_block, PieceOrder order,
                       RelayoutArgs *a) {
    clear_table(a);
    const ModeGeom &g = p.mode[mode];
    for (int r = 0; r < p.world; ++r) {
        a->src_plane[r] = static_cast<uint64_t>(g.src_plane[r] / 16);
        a->dst_plane[r] = static_cast<uint64_t>(g.dst_plane[r] / 16);
    }
    uint64_t blocks = 0;
    int n = 0;
    for (int outer = 0; outer < p.world; ++outer)
        for (int inner = 0; inner < p.world; ++inner) {
            const int j = order == kDstMajor ? inner : outer;
            const int r = order == kDstMajor ? outer : inner;
            const Piece &pc = g.piece[j * p.world + r];
            if (pc.rows == 0 || pc.row_bytes == 0) continue;   // empty piece
            PieceArgs &o = a->piece[n];
            fill_piece_args(pc, &o);
            a->blk_begin[n] = static_cast<uint32_t>(blocks);
            blocks += (o.nvec + vec_per_block - 1) / vec_per_block;
            ++n;
        }
    return blocks;
}

uint64_t fill_relayout_vbands(const Plan &p, int mode, uint32_t band_vecs, RelayoutArgs *a) {
    clear_table(a);
    const ModeGeom &g = p.mode[mode];
    for (int r = 0; r < p.world; ++r) {
        a->src_plane[r] = static_cast<uint64_t>(g.src_plane[r] / 16);
        a->dst_plane[r] = static_cast<uint64_t>(g.dst_plane[r] / 16);
    }
    a->world = static_cast<uint32_t>(p.world);
    a->band_vecs = band_vecs;
    uint64_t blocks = 0;
    for (int grp = 0; grp < p.world; ++grp) {
        uint64_t bands = 0;
        for (int k = 0; k < p.world; ++k) {
            const int j = mode == 0 ? grp : k;
            const int r = mode == 0 ? k : grp;
            PieceArgs &o = a->piece[grp * p.world + k];
            fill_piece_args(g.piece[j * p.world + r], &o);
            const uint64_t nb = (uint64_t(o.nvec) + band_vecs - 1) / band_vecs;
            if (nb > bands) bands = nb;
        }
        a->grp_begin[grp] = static_cast<uint32_t>(blocks);
        blocks += bands * p.world;
    }
    return blocks;
}

uint64_t fill_relayout_aligned(const Plan &p, int mode, uint32_t chunk_vecs, uint32_t max_chunks,
                               RelayoutArgs *a) {
    const ModeGeom &g = p.mode[mode];
    // Row widths of the k-th piece of a group: the same for every group
    // (mode 0: destination r = k; mode 1: source j = k).
    uint32_t vpr[kMaxWorld] = {};
    uint32_t common = 0;   // gcd of the non-zero widths
    uint32_t first = 0;
    bool uneven = false;
    for (int k = 0; k < p.world; ++k) {
        vpr[k] = static_cast<uint32_t>(p.R[k] / 16);
        if (vpr[k] == 0) continue;
        if (first == 0) first = vpr[k];
        else if (vpr[k] != first) uneven = true;
        uint32_t x = common, y = vpr[k];
        while (y != 0) { const uint32_t t = x % y; x = y; y = t; }
        common = x;
    }
    if (!uneven || chunk_vecs == 0) return 0;
    uint32_t gc = common, y = chunk_vecs;   // gcd(chunk_vecs, common)
    while (y != 0) { const uint32_t t = gc % y; gc = y; y = t; }
    // R * vpr_k is a multiple of chunk_vecs for R = chunk_vecs / gc
    const uint32_t rows_per_band = chunk_vecs / gc;
    if (max_chunks != 0) {
        for (int k = 0; k < p.world; ++k)
            if (uint64_t(rows_per_band) * vpr[k] > uint64_t(max_chunks) * chunk_vecs) return 0;
    }
    clear_table(a);
    for (int r = 0; r < p.world; ++r) {
        a->src_plane[r] = static_cast<uint64_t>(g.src_plane[r] / 16);
        a->dst_plane[r] = static_cast<uint64_t>(g.dst_plane[r] / 16);
    }
    a->world = static_cast<uint32_t>(p.world);
    a->band_rows = rows_per_band;
    a->chunk_vecs = chunk_vecs;
    uint32_t n = 0;
    for (int k = 0; k < p.world; ++k) {
        a->chunk_begin[k] = n;
        n += static_cast<uint32_t>(uint64_t(rows_per_band) * vpr[k] / chunk_vecs);
    }
    for (int k = p.world; k <= kMaxWorld; ++k) a->chunk_begin[k] = n;
    a->chunks_per_band = n;
    const Div32Magic dm = div32_magic(n);
    a->band_m = dm.m;
    a->band_s1 = dm.s1;
    a->band_s2 = dm.s2;
    uint64_t blocks = 0;
    for (int grp = 0; grp < p.world; ++grp) {
        const int64_t rows = p.S[grp];
        const int64_t bands = (rows + rows_per_band - 1) / rows_per_band;
        for (int k = 0; k < p.world; ++k) {
            const int j = mode == 0 ? grp : k;
            const int r = mode == 0 ? k : grp;
            fill_piece_args(g.piece[j * p.world + r], &a->piece[grp * p.world + k]);
        }
        a->grp_begin[grp] = static_cast<uint32_t>(blocks);
        blocks += static_cast<uint64_t>(bands) * n;
    }
    return blocks;
}

bool to_units(RelayoutArgs *a, uint32_t vpl) {
    if (vpl == 0 || a->band_vecs % vpl) return false;
    a->band_vecs /= vpl;
    for (int r = 0; r < kMaxWorld; ++r) {
        if (a->src_plane[r] % vpl || a->dst_plane[r] % vpl) return false;
        a->src_plane[r] /= vpl;
        a->dst_plane[r] /= vpl;
    }
    for (int q = 0; q < kMaxPieces; ++q) {
        PieceArgs &o = a->piece[q];
        if (o.nvec % vpl || o.vpr % vpl || o.src_pitch % vpl || o.dst_pitch % vpl ||
            o.src_off % vpl || o.dst_off % vpl)
            return false;
        o.nvec /= vpl;
        o.vpr /= vpl;
        o.src_pitch /= vpl;
        o.dst_pitch /= vpl;
        o.src_off /= vpl;
        o.dst_off /= vpl;
        o.magic = row_magic(o.vpr);
        set_vpr_division(&o);
    }
    return true;
}

uint64_t fill_window_copy(const Plan &p, int mode, uint32_t band_vecs, RelayoutArgs *a) {
    clear_table(a);
    const ModeGeom &g = p.mode[mode];
    a->world = 1;   // one piece per group: group r copies window r
    a->band_vecs = band_vecs;
    uint64_t blocks = 0;
    for (int r = 0; r < p.world; ++r) {
        // the window of r holds one destination plane of r, rows of the
        // destination's own width, packed: copy it as (rows x row) with
        // equal pitches on both sides.
        const int64_t row_bytes = mode == 0 ? p.R[r] : p.G;
        const int64_t rows = mode == 0 ? p.s_global : p.S[r];
        a->src_plane[r] = static_cast<uint64_t>(g.dst_plane[r] / 16);
        a->dst_plane[r] = static_cast<uint64_t>(g.dst_plane[r] / 16);
        Piece pc;
        pc.j = r;
        pc.r = r;
        pc.rows = rows;
        pc.row_bytes = row_bytes;
        pc.src_pitch = pc.dst_pitch = row_bytes;
        PieceArgs &o = a->piece[r];
        fill_piece_args(pc, &o);
        a->grp_begin[r] = static_cast<uint32_t>(blocks);
        blocks += (uint64_t(o.nvec) + band_vecs - 1) / band_vecs;
    }
    return blocks;
}

}  // namespace ulysses
