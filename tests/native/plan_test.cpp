// Host-only test of the relayout plan (no GPU, no HIP headers).
//
// For many geometries it replays, on the CPU, the index arithmetic the
// kernels perform for every (block, lane) of the launch tables the plan
// fills, and checks that
//   - every destination vector is written exactly once, and
//   - it is read from the source address the definition names:
//       mode 0: out_r[bi][S][h] = in_j[bi][S - seq_off_j][head_off_r + h],
//       mode 1: out_r[bi][s][H] = in_j[bi][seq_off_r + s][H - head_off_j];
//   - the window copy of the plane-at-a-time mode covers each destination
//     plane once from the same offset in the window;
//   - the fused path's lane of a vector within its head row is the thread's
//     lane modulo d/8, and the band kernel's block order, exact divisions
//     and 32-bit offsets are valid;
//   - the multiply-high division by the row length is exact at every
//     quotient boundary, hence everywhere (both sides are monotone).
// Prints "OK <checks>" and exits 0, or a message and exits 1.
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <random>
#include <vector>

#include "plan.hpp"

using namespace ulysses;

static long g_checks = 0;
static long g_aligned = 0;   // geometries that took the row-aligned table

#define REQUIRE(c, ...)                                              \
    do {                                                             \
        ++g_checks;                                                  \
        if (!(c)) {                                                  \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                       \
            std::fprintf(stderr, "\n");                              \
            std::exit(1);                                            \
        }                                                            \
    } while (0)

static uint32_t umulhi(uint32_t a, uint32_t b) {
    return static_cast<uint32_t>((uint64_t(a) * b) >> 32);
}

// The kernels' mapping of (block x, plane y, linear lane lin) to vector
// offsets; returns false when the lane is past its piece.
struct Hit {
    int j, r;
    uint64_t src_vec, dst_vec;   // vector offsets from the shard bases
    uint32_t col;
    uint32_t row, pos0;          // piece-local row, piece's first position
};

static bool replay(const RelayoutArgs &a, uint32_t vpb, uint32_t x, uint32_t y, uint32_t lin,
                   Hit *h) {
    uint32_t p = 0;
    for (int q = 1; q < kMaxPieces; ++q) p += a.blk_begin[q] <= x ? 1u : 0u;
    const PieceArgs &pc = a.piece[p];
    const uint32_t s0 = (x - a.blk_begin[p]) * vpb;
    const uint32_t row0 = s0 / pc.vpr;
    const uint32_t col0 = s0 - row0 * pc.vpr;
    const uint32_t t = col0 + lin;
    if (t >= 65536u) {
        std::fprintf(stderr, "numerator %u out of range\n", t);
        std::exit(1);
    }
    const uint32_t dr = pc.vpr == 1 ? t : umulhi(t, pc.magic);
    const uint32_t col = t - dr * pc.vpr;
    const uint32_t row = row0 + dr;
    if (s0 + lin >= pc.nvec) return false;
    h->j = pc.j;
    h->r = pc.r;
    h->src_vec = (uint64_t(a.src_plane0) + y) * a.src_plane[pc.j] + pc.src_off +
                 uint64_t(row) * pc.src_pitch + col;
    h->dst_vec = (uint64_t(a.dst_plane0) + y) * a.dst_plane[pc.r] + pc.dst_off +
                 uint64_t(row) * pc.dst_pitch + col;
    h->col = col;
    h->row = row;
    h->pos0 = pc.src_row0;
    return true;
}

// The band kernel's mapping: block x, chunk-relative lane `lin` of chunk
// `c`; returns false when the lane (or the whole chunk) is past the band.
static bool replay_band(const RelayoutArgs &a, uint32_t chunk, uint32_t x, uint32_t y,
                        uint32_t c, uint32_t lin, Hit *h) {
    uint32_t g = 0;
    for (int q = 1; q < kMaxWorld; ++q) g += a.grp_begin[q] <= x ? 1u : 0u;
    const uint32_t local = x - a.grp_begin[g];
    uint32_t k, begin, end;
    if (a.chunks_per_band != 0) {   // row-aligned chunks, as the kernel decodes them
        const uint32_t band = div32(local, a.band_m, a.band_s1, a.band_s2);
        REQUIRE(band == local / a.chunks_per_band, "aligned band division");
        const uint32_t q = local - band * a.chunks_per_band;
        k = 0;
        for (int i = 1; i < kMaxWorld; ++i) k += a.chunk_begin[i] <= q ? 1u : 0u;
        REQUIRE(k < a.world && a.chunk_begin[k + 1] > q, "aligned chunk lands in a piece");
        const uint32_t c = q - a.chunk_begin[k];
        const uint32_t vpr = a.piece[g * a.world + k].vpr;
        const uint32_t band0 = band * a.band_rows * vpr;
        begin = band0 + c * a.chunk_vecs;
        REQUIRE(c * a.chunk_vecs < a.band_rows * vpr, "chunk past its band");
        end = std::min(std::min(begin + a.chunk_vecs, band0 + a.band_rows * vpr),
                       a.piece[g * a.world + k].nvec);
    } else {
        const uint32_t band = local / a.world;
        k = local - band * a.world;
        const uint32_t vpr = a.piece[g * a.world + k].vpr;
        const uint32_t span = a.band_vecs != 0 ? a.band_vecs : a.band_rows * vpr;
        begin = band * span;
        end = std::min(begin + span, a.piece[g * a.world + k].nvec);
    }
    const PieceArgs &pc = a.piece[g * a.world + k];
    const uint32_t s0 = begin + c * chunk;
    if (s0 >= end) return false;
    const uint32_t row0 = s0 / pc.vpr;
    const uint32_t col0 = s0 - row0 * pc.vpr;
    const uint32_t t = col0 + lin;
    if (t >= 65536u) {
        std::fprintf(stderr, "numerator %u out of range\n", t);
        std::exit(1);
    }
    const uint32_t dr = pc.vpr == 1 ? t : umulhi(t, pc.magic);
    const uint32_t col = t - dr * pc.vpr;
    const uint32_t row = row0 + dr;
    if (s0 + lin >= end) return false;
    h->j = pc.j;
    h->r = pc.r;
    h->src_vec = (uint64_t(a.src_plane0) + y) * a.src_plane[pc.j] + pc.src_off +
                 uint64_t(row) * pc.src_pitch + col;
    h->dst_vec = (uint64_t(a.dst_plane0) + y) * a.dst_plane[pc.r] + pc.dst_off +
                 uint64_t(row) * pc.dst_pitch + col;
    h->col = col;
    h->row = row;
    h->pos0 = pc.src_row0;
    return true;
}

static void check_magic() {
    for (uint32_t v = 2; v <= kMaxRowVectors; ++v) {
        const uint32_t m = row_magic(v);
        for (uint64_t k = 1; k * v <= 65536; ++k) {
            const uint32_t lo = static_cast<uint32_t>(k * v - 1), hi = static_cast<uint32_t>(k * v);
            REQUIRE(umulhi(lo, m) == k - 1, "magic vpr=%u t=%u", v, lo);
            if (hi < 65536) REQUIRE(umulhi(hi, m) == k, "magic vpr=%u t=%u", v, hi);
        }
    }
}

static void check_geometry(int world, int64_t b, int64_t d, int dtype,
                           const std::vector<int64_t> &S, const std::vector<int64_t> &H,
                           uint32_t vpb) {
    Plan p;
    std::string msg;
    const int rc = plan_build(&p, world, b, d, S.data(), H.data(), dtype, 1 << 30, &msg);
    REQUIRE(rc == kOk, "plan_build failed: %s", msg.c_str());
    const int64_t esz = dtype_size(dtype);
    const int64_t hb = d * esz;
    const int64_t n_global = p.n_global, s_global = p.s_global;
    REQUIRE(hb % 16 == 0, "row alignment");
    const int64_t hv = hb / 16;   // vectors per head row
    for (int mode = 0; mode < 2; ++mode) {
        // traversals 0, 1: flat in both piece orders; 2, 3: row bands of
        // two heights, with chunks of vpb vectors; 4: bands of vpb vectors;
        // 5: row-aligned chunks (pieces of unequal width only)
        for (int trav = 0; trav < 6; ++trav) {
            RelayoutArgs a;
            uint32_t gx, nchunks = 1;
            if (trav < 2) {
                gx = fill_relayout(p, mode, vpb, static_cast<PieceOrder>(trav), &a);
            } else if (trav == 4) {
                gx = fill_relayout_vbands(p, mode, vpb, &a);
            } else if (trav == 5) {
                gx = fill_relayout_aligned(p, mode, vpb, 0, &a);
                if (gx == 0) continue;   // equal widths: the vector bands apply
                for (int q = 0; q < p.world; ++q)
                    REQUIRE(a.band_rows * a.piece[q].vpr % vpb == 0, "aligned band not whole chunks");
                ++g_aligned;
            } else {
                const uint32_t rows = trav == 2 ? band_rows_for(p, mode, vpb) : 3;
                gx = fill_relayout_bands(p, mode, rows, &a);
                uint32_t widest = 1;
                for (int q = 0; q < kMaxPieces; ++q) widest = std::max(widest, a.piece[q].vpr);
                nchunks = (rows * widest + vpb - 1) / vpb;
            }
            std::vector<std::vector<int>> hits(world);
            for (int r = 0; r < world; ++r)
                hits[r].assign(static_cast<size_t>(b * p.mode[mode].dst_plane[r] / 16), 0);
            for (uint32_t y = 0; y < b; ++y)
                for (uint32_t x = 0; x < gx; ++x)
                    for (uint32_t c = 0; c < nchunks; ++c)
                    for (uint32_t lin = 0; lin < vpb; ++lin) {
                        Hit h;
                        const bool in = trav < 2 ? replay(a, vpb, x, y, lin, &h)
                                                 : replay_band(a, vpb, x, y, c, lin, &h);
                        if (!in) continue;
                        REQUIRE(h.dst_vec < hits[h.r].size(), "dst out of range");
                        hits[h.r][h.dst_vec] += 1;
                        // decode the destination vector and derive its source
                        int64_t v = static_cast<int64_t>(h.dst_vec);
                        int64_t want_j, want_src;
                        if (mode == 0) {   // dst (b, s_global, H_r, hv)
                            const int64_t e = v % hv; v /= hv;
                            const int64_t hh = v % p.H[h.r]; v /= p.H[h.r];
                            const int64_t Sg = v % s_global; const int64_t bi = v / s_global;
                            int j = 0;
                            while (!(p.seq_off[j] <= Sg && Sg < p.seq_off[j + 1])) ++j;
                            want_j = j;
                            want_src = ((bi * p.S[j] + (Sg - p.seq_off[j])) * n_global +
                                        p.head_off[h.r] + hh) * hv + e;
                        } else {           // dst (b, S_r, n_global, hv)
                            const int64_t e = v % hv; v /= hv;
                            const int64_t Hg = v % n_global; v /= n_global;
                            const int64_t s = v % p.S[h.r]; const int64_t bi = v / p.S[h.r];
                            int j = 0;
                            while (!(p.head_off[j] <= Hg && Hg < p.head_off[j + 1])) ++j;
                            want_j = j;
                            want_src = ((bi * s_global + p.seq_off[h.r] + s) * p.H[j] +
                                        (Hg - p.head_off[j])) * hv + e;
                        }
                        REQUIRE(h.j == want_j && static_cast<int64_t>(h.src_vec) == want_src,
                                "mode %d W=%d: src (%d,%llu) want (%lld,%lld)", mode, world, h.j,
                                (unsigned long long)h.src_vec, (long long)want_j,
                                (long long)want_src);
                        // fused lanes: lane within the head row == lin mod hv
                        if (trav < 2 && mode == 0 && (hv & (hv - 1)) == 0 && hv <= 64 &&
                            vpb % hv == 0)
                            REQUIRE(int64_t(h.col % hv) == int64_t(lin % hv), "lane mapping");
                    }
            for (int r = 0; r < world; ++r)
                for (size_t i = 0; i < hits[r].size(); ++i)
                    REQUIRE(hits[r][i] == 1, "trav %d mode %d rank %d vector %zu written %d times",
                            trav, mode, r, i, hits[r][i]);
        }
        // window copy: plane y of dst r from window r plane 0, same offset
        RelayoutArgs c;
        const uint32_t gc = fill_window_copy(p, mode, vpb, &c);
        for (uint32_t y = 0; y < b; ++y) {
            c.src_plane0 = 0;
            c.dst_plane0 = y;
            std::vector<std::vector<int>> hits(world);
            for (int r = 0; r < world; ++r)
                hits[r].assign(static_cast<size_t>(p.mode[mode].dst_plane[r] / 16), 0);
            for (uint32_t x = 0; x < gc; ++x)
                for (uint32_t lin = 0; lin < vpb; ++lin) {
                    Hit h;
                    if (!replay_band(c, vpb, x, 0, 0, lin, &h)) continue;
                    REQUIRE(h.j == h.r, "copy crosses ranks");
                    const uint64_t plane = p.mode[mode].dst_plane[h.r] / 16;
                    REQUIRE(h.dst_vec == y * plane + h.src_vec, "copy offset");
                    REQUIRE(h.src_vec < plane, "copy source past the window");
                    hits[h.r][h.src_vec] += 1;
                }
            for (int r = 0; r < world; ++r)
                for (size_t i = 0; i < hits[r].size(); ++i)
                    REQUIRE(hits[r][i] == 1, "copy coverage");
        }
    }
}

// The fused kernel's tables: mode-0 pieces in units of vpl vectors.  Every
// destination vector is covered once, from the source the definition
// names, and a lane's position within its head row is threadIdx % (hv/vpl).
static void check_fused_units(int world, int64_t b, int64_t d, const std::vector<int64_t> &S,
                              const std::vector<int64_t> &H, uint32_t upb) {
    Plan p;
    std::string msg;
    REQUIRE(plan_build(&p, world, b, d, S.data(), H.data(), 0, 0, &msg) == kOk, "plan");
    const int64_t hv = d / 8, n_global = p.n_global, s_global = p.s_global;
    for (uint32_t vpl = 1; vpl <= 4; vpl *= 2) {
        if (hv % vpl) continue;
        const uint32_t L = static_cast<uint32_t>(hv / vpl);
      for (int banded = 0; banded < 2; ++banded) {
        RelayoutArgs a;
        const uint32_t gx = banded ? fill_relayout_vbands(p, 0, upb * vpl, &a)
                                   : fill_relayout(p, 0, upb * vpl, kSrcMajor, &a);
        REQUIRE(to_units(&a, vpl), "to_units");
        std::vector<std::vector<int>> hits(world);
        for (int r = 0; r < world; ++r)
            hits[r].assign(static_cast<size_t>(b * p.mode[0].dst_plane[r] / 16), 0);
        for (uint32_t y = 0; y < b; ++y)
            for (uint32_t x = 0; x < gx; ++x)
                for (uint32_t lin = 0; lin < upb; ++lin) {
                    Hit h;
                    const bool in = banded ? replay_band(a, upb, x, y, 0, lin, &h)
                                           : replay(a, upb, x, y, lin, &h);
                    if (!in) continue;
                    REQUIRE(h.col % L == lin % L, "fused lane mapping");
                    for (uint32_t v = 0; v < vpl; ++v) {
                        int64_t dv = static_cast<int64_t>(h.dst_vec * vpl + v);
                        const int64_t sv = static_cast<int64_t>(h.src_vec * vpl + v);
                        REQUIRE(dv < static_cast<int64_t>(hits[h.r].size()), "unit past shard");
                        hits[h.r][dv] += 1;
                        const int64_t e = dv % hv; dv /= hv;
                        const int64_t hh = dv % p.H[h.r]; dv /= p.H[h.r];
                        const int64_t Sg = dv % s_global, bi = dv / s_global;
                        int j = 0;
                        while (!(p.seq_off[j] <= Sg && Sg < p.seq_off[j + 1])) ++j;
                        const int64_t want = ((bi * p.S[j] + (Sg - p.seq_off[j])) * n_global +
                                              p.head_off[h.r] + hh) * hv + e;
                        REQUIRE(h.j == j && sv == want, "fused unit source");
                        // the table row the kernel reads is the global position
                        REQUIRE(int64_t(h.pos0) + int64_t(h.row) == Sg, "fused rotary position");
                    }
                }
        for (int r = 0; r < world; ++r)
            for (size_t i = 0; i < hits[r].size(); ++i)
                REQUIRE(hits[r][i] == 1, "fused coverage vpl=%u rank %d vec %zu: %d", vpl, r, i,
                        hits[r][i]);
      }
    }
}

// The band kernel of the fused path (d = 128): a vector-band table with
// 64 * unroll vectors per band, blocks taken in the XCD-aware order, each
// block moving its band of q and of k (the same offsets for both).  Checks
// that the order is a bijection, the exact divisions agree with '/', every
// destination vector is written once from the defined source, the rotary
// row is the row's global position, and the kernel's 32-bit byte offsets and
// 16-bit division numerators stay in range.
static uint32_t band_xcd_order(uint32_t x, uint32_t n, uint32_t w, const Div32Magic &dm) {
    const uint32_t full = div32(n >> 3, dm.m, dm.s1, dm.s2) * (8 * w);
    if (x >= full) return x;
    const uint32_t c = div32(x >> 3, dm.m, dm.s1, dm.s2);
    const uint32_t rem = x - c * (8 * w);
    return (8 * c + (rem & 7)) * w + (rem >> 3);
}

static void check_fused_band(int world, int64_t b, const std::vector<int64_t> &S,
                             const std::vector<int64_t> &H, uint32_t unroll) {
    Plan p;
    std::string msg;
    REQUIRE(plan_build(&p, world, b, 128, S.data(), H.data(), 0, 0, &msg) == kOk, "plan");
    const int64_t hv = 16, n_global = p.n_global, s_global = p.s_global;
    const uint32_t band_v = 64 * unroll;
    RelayoutArgs a;
    const uint64_t gx64 = fill_relayout_vbands(p, 0, band_v, &a);
    REQUIRE(to_units(&a, 1), "to_units");
    REQUIRE(gx64 % a.world == 0, "band table not a multiple of world");
    const uint32_t gx = static_cast<uint32_t>(gx64);
    const Div32Magic wm = div32_magic(a.world);
    std::vector<int> order_hits(gx, 0);
    std::vector<std::vector<int>> hits(world);
    for (int r = 0; r < world; ++r)
        hits[r].assign(static_cast<size_t>(b * p.mode[0].dst_plane[r] / 16), 0);
    for (uint32_t y = 0; y < b; ++y)
        for (uint32_t xb = 0; xb < gx; ++xb) {
            const uint32_t x = band_xcd_order(xb, gx, a.world, wm);
            REQUIRE(x < gx, "block order past the grid");
            if (y == 0) order_hits[x] += 1;
            uint32_t g = 0;
            for (int q = 1; q < kMaxWorld; ++q) g += a.grp_begin[q] <= x ? 1u : 0u;
            const uint32_t local = x - a.grp_begin[g];
            const uint32_t band = div32(local, wm.m, wm.s1, wm.s2);
            REQUIRE(band == local / a.world, "band division");
            const PieceArgs &pc = a.piece[g * a.world + (local - band * a.world)];
            const uint32_t s0 = band * band_v;
            if (s0 >= pc.nvec) continue;
            const uint32_t last = std::min(band_v, pc.nvec - s0) - 1;
            const uint32_t row0 = div32(s0, pc.vpr_m, pc.vpr_s1, pc.vpr_s2);
            REQUIRE(row0 == s0 / pc.vpr, "row division");
            const uint32_t col0 = s0 - row0 * pc.vpr;
            for (uint32_t lin = 0; lin < band_v; ++lin) {
                const bool ok = lin <= last;
                const uint32_t t = col0 + std::min(lin, last);
                REQUIRE(t < 65536u, "band numerator %u out of range", t);
                const uint32_t dr = pc.vpr == 1 ? t : umulhi(t, pc.magic);
                REQUIRE(dr == t / pc.vpr, "row split");
                REQUIRE(dr <= band_v / 16, "band spans %u rows", dr + 1);
                const uint32_t col = t - dr * pc.vpr;
                const uint64_t soff = (uint64_t(dr) * pc.src_pitch + col) << 4;
                const uint64_t doff = (uint64_t(dr) * pc.dst_pitch + col) << 4;
                REQUIRE(soff < (uint64_t{1} << 32) && doff < (uint64_t{1} << 32),
                        "32-bit offsets");
                // lanes past the piece reload its last vector and store
                // nothing; valid lanes come in whole 16-lane rows
                if (!ok) continue;
                REQUIRE(col % 16 == (lin & 15), "band lane within its head row");
                REQUIRE(lin / 16 * 16 + 15 <= last, "16-lane row partly past the piece");
                const uint32_t row = row0 + dr;
                const uint64_t sv = uint64_t(y) * a.src_plane[pc.j] + pc.src_off +
                                    uint64_t(row) * pc.src_pitch + col;
                const uint64_t dvv = uint64_t(y) * a.dst_plane[pc.r] + pc.dst_off +
                                     uint64_t(row) * pc.dst_pitch + col;
                REQUIRE(dvv < hits[pc.r].size(), "band kernel past shard");
                hits[pc.r][dvv] += 1;
                int64_t dv = static_cast<int64_t>(dvv);
                const int64_t e = dv % hv; dv /= hv;
                const int64_t hh = dv % p.H[pc.r]; dv /= p.H[pc.r];
                const int64_t Sg = dv % s_global, bi = dv / s_global;
                int j = 0;
                while (!(p.seq_off[j] <= Sg && Sg < p.seq_off[j + 1])) ++j;
                const int64_t want = ((bi * p.S[j] + (Sg - p.seq_off[j])) * n_global +
                                      p.head_off[pc.r] + hh) * hv + e;
                REQUIRE(pc.j == j && int64_t(sv) == want, "band kernel source");
                REQUIRE(int64_t(pc.src_row0) + int64_t(row) == Sg, "band kernel position");
            }
        }
    for (uint32_t x = 0; x < gx; ++x) REQUIRE(order_hits[x] == 1, "block order not a bijection");
    for (int r = 0; r < world; ++r)
        for (size_t i = 0; i < hits[r].size(); ++i)
            REQUIRE(hits[r][i] == 1, "band kernel coverage rank %d vec %zu: %d", r, i, hits[r][i]);
}

// The exact 32-bit division against '/', at quotient boundaries and at random.
static void check_div32(std::mt19937_64 &rng) {
    std::vector<uint32_t> ds;
    for (uint32_t v = 1; v <= 4096; ++v) ds.push_back(v);
    for (int i = 0; i < 2000; ++i) ds.push_back(1 + static_cast<uint32_t>(rng() % 0x80000000u));
    ds.push_back(0x80000000u);
    for (uint32_t v : ds) {
        const Div32Magic dm = div32_magic(v);
        const uint32_t probes[] = {0u, 1u, v - 1, v, v + 1, 0xFFFFFFFFu, 0xFFFFFFFFu - v,
                                   0x80000000u, static_cast<uint32_t>(rng()),
                                   static_cast<uint32_t>(rng())};
        for (uint32_t n : probes) REQUIRE(div32(n, dm.m, dm.s1, dm.s2) == n / v, "div32 %u / %u", n, v);
        for (uint64_t k = 1; k * v <= 0xFFFFFFFFull && k < 64; ++k) {
            const uint32_t lo = static_cast<uint32_t>(k * v - 1), hi = static_cast<uint32_t>(k * v);
            REQUIRE(div32(lo, dm.m, dm.s1, dm.s2) == k - 1 && div32(hi, dm.m, dm.s1, dm.s2) == k,
                    "div32 boundary %u", v);
        }
    }
}

// When the row-aligned table applies: pieces of unequal width whose
// whole-chunk bands hold at most max_chunks chunks of 64 vectors per piece.
static void check_aligned_choice() {
    struct Case { int64_t d; std::vector<int64_t> H; uint32_t max_chunks; uint32_t rows; };
    const Case cases[] = {
        {128, {6, 6, 6, 6, 4, 4, 4, 4}, 4, 2},   // widths 96/64 vectors: 2 rows, 3/2 chunks
        {128, {4, 4, 4, 4, 2, 2, 2, 2}, 4, 2},   // 64/32: 2 rows, 2/1 chunks
        {128, {8, 8, 4, 4}, 4, 1},               // 128/64: 1 row, 2/1 chunks
        {128, {8, 8, 8, 6}, 4, 2},               // 128/96: 2 rows, 4/3 chunks
        {128, {6, 6, 6, 6, 5, 5, 5, 5}, 4, 0},   // 96/80: 4 rows, 6/5 chunks: vector bands
        {128, {6, 6, 6, 6, 5, 5, 5, 5}, 0, 4},   // ... unless uncapped
        {256, {6, 6, 6, 6, 6, 5, 5}, 4, 0},      // 192/160: 2 rows but 6/5 chunks
        {128, {5, 5, 5, 5}, 4, 0},               // equal widths: vector bands
        {128, {5, 0, 5, 5}, 4, 0},               // an empty piece does not count
    };
    for (const Case &c : cases) {
        const int world = static_cast<int>(c.H.size());
        std::vector<int64_t> S(world, 7);
        Plan p;
        std::string msg;
        REQUIRE(plan_build(&p, world, 1, c.d, S.data(), c.H.data(), 0, 0, &msg) == kOk, "plan");
        for (int mode = 0; mode < 2; ++mode) {
            RelayoutArgs a;
            std::memset(&a, 0x5A, sizeof a);
            const uint64_t gx = fill_relayout_aligned(p, mode, 64, c.max_chunks, &a);
            if (c.rows == 0) {
                REQUIRE(gx == 0, "aligned table where vector bands apply");
            } else {
                REQUIRE(gx != 0 && a.band_rows == c.rows, "aligned band of %u rows, want %u",
                        a.band_rows, c.rows);
            }
        }
    }
}

static void check_errors() {
    Plan p;
    std::string m;
    const int64_t s2[2] = {4, 4}, h2[2] = {2, 2};
    REQUIRE(plan_build(&p, 0, 1, 8, s2, h2, 0, 0, &m) == kEInval, "world 0");
    REQUIRE(plan_build(&p, 9, 1, 8, s2, h2, 0, 0, &m) == kEInval, "world 9");
    REQUIRE(plan_build(&p, 2, 0, 8, s2, h2, 0, 0, &m) == kEInval, "b 0");
    REQUIRE(plan_build(&p, 2, 1, 4, s2, h2, 0, 0, &m) == kEAlign, "d*esz 8");
    REQUIRE(plan_build(&p, 2, 1, 8, s2, h2, 9, 0, &m) == kEDtype, "dtype");
    REQUIRE(plan_build(&p, 2, 1, 8, s2, h2, 3, 0, &m) == kEAlign, "fp8 d=8");
    const int64_t neg[2] = {-1, 5}, zero[2] = {0, 0};
    REQUIRE(plan_build(&p, 2, 1, 8, neg, h2, 0, 0, &m) == kEInval, "negative split");
    REQUIRE(plan_build(&p, 2, 1, 8, zero, h2, 0, 0, &m) == kEInval, "zero sum");
    const int64_t big[2] = {1024, 1025};
    REQUIRE(plan_build(&p, 2, 1, 128, s2, big, 0, 0, &m) == kEInval, "row over 512 KiB");
    REQUIRE(plan_build(&p, 2, 1, 8, s2, h2, 0, -1, &m) == kEInval, "negative cap");
    // the FastVideo geometry: 896,000,000 bytes per rank per plane
    const int64_t s4[4] = {62500, 62500, 62500, 62500}, h4[4] = {14, 14, 14, 14};
    REQUIRE(plan_build(&p, 4, 3, 128, s4, h4, 0, 1 << 30, &m) == kOk, "fastvideo plan");
    REQUIRE(p.mode[0].window_bytes == 896000000 && p.mode[1].window_bytes == 896000000,
            "window bytes");
}

int main() {
    check_magic();
    check_errors();
    check_aligned_choice();
    std::mt19937_64 rng(12345);
    const uint32_t vpbs[] = {64, 256, 1024, 2048};
    const int dtypes[] = {0, 2, 3, 5};
    for (int it = 0; it < 160; ++it) {
        const int world = 1 + static_cast<int>(rng() % 8);
        const int dtype = dtypes[rng() % 4];
        const int64_t esz = dtype_size(dtype);
        const int64_t unit = 16 / esz;   // smallest legal d
        const int64_t d = unit * (1 + static_cast<int64_t>(rng() % 3));
        const int64_t b = 1 + static_cast<int64_t>(rng() % 3);
        std::vector<int64_t> S(world), H(world);
        int64_t ss = 0, hs = 0;
        for (int r = 0; r < world; ++r) {
            S[r] = static_cast<int64_t>(rng() % 40) - (it % 3 == 0 ? 5 : 0);
            if (S[r] < 0) S[r] = 0;
            H[r] = static_cast<int64_t>(rng() % 5);
            ss += S[r];
            hs += H[r];
        }
        if (ss == 0) S[0] = 3;
        if (hs == 0) H[world - 1] = 2;
        check_geometry(world, b, d, dtype, S, H, vpbs[rng() % 4]);
    }
    // long rows: row length near the 32768-vector limit, vpr == 1 rows
    check_geometry(2, 1, 2048, 2, {3, 2}, {40, 24}, 2048);
    check_geometry(3, 2, 16, 5, {5, 1, 7}, {1, 1, 1}, 64);
    for (int it = 0; it < 40; ++it) {
        const int world = 1 + static_cast<int>(rng() % 8);
        const int64_t d = int64_t{8} << (rng() % 6);   // 8 .. 256
        const int64_t b = 1 + static_cast<int64_t>(rng() % 2);
        std::vector<int64_t> S(world), H(world);
        for (int r = 0; r < world; ++r) {
            S[r] = static_cast<int64_t>(rng() % 30);
            H[r] = static_cast<int64_t>(rng() % 4);
        }
        S[0] += 1;
        H[world - 1] += 1;
        check_fused_units(world, b, d, S, H, 128);
    }
    for (int it = 0; it < 30; ++it) {
        const int world = 1 + static_cast<int>(rng() % 8);
        std::vector<int64_t> S(world), H(world);
        for (int r = 0; r < world; ++r) {
            S[r] = static_cast<int64_t>(rng() % 23);
            H[r] = static_cast<int64_t>(rng() % 19);   // up to 18 heads: several head chunks
        }
        S[0] += 1;
        H[world - 1] += 1;
        check_fused_band(world, 1 + static_cast<int64_t>(rng() % 2), S, H, 1u << (it % 3));
    }
    // many equal pieces: full runs of 8 bands in the XCD order, and a tail
    check_fused_band(8, 1, std::vector<int64_t>(8, 40), std::vector<int64_t>(8, 5), 1);
    check_fused_band(7, 2, {9, 40, 3, 17, 0, 22, 31}, {6, 6, 6, 6, 6, 5, 5}, 2);
    check_div32(rng);
    REQUIRE(g_aligned > 50, "too few geometries exercised the row-aligned table: %ld", g_aligned);
    std::printf("OK %ld\n", g_checks);
    return 0;
}
