// Host-only test of the relayout plan (no GPU, no HIP headers).
//
// For many geometries it replays, on the CPU, the index arithmetic the
// kernels perform for every (block, plane, lane) of the launch tables the
// plan fills, and checks that
//   - every destination vector is written exactly once, and
//   - it is read from the source address the definition names:
//       mode 0: out_r[bi][S][h] = in_j[bi][S - seq_off_j][head_off_r + h],
//       mode 1: out_r[bi][s][H] = in_j[bi][seq_off_r + s][H - head_off_j];
//   - every address stays inside its shard (loads of the lanes the kernels
//     clamp included);
//   - the plane copy of the plane-at-a-time mode covers each destination
//     plane once from the same offset in the window;
//   - the fused gather's lane within its head row is the thread's lane
//     modulo d/8, valid lanes come in whole head rows, and the rotary row is
//     the global position of the destination row;
//   - the divisions are exact (the multiply-high by the row length at every
//     quotient boundary, hence everywhere, both sides being monotone; the
//     32-bit division of div32 against '/').
// It also checks the plan's validation, including sizes whose products
// would overflow.  Prints "OK <checks>" and exits 0, or a message and exits 1.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "plan.hpp"

using namespace ulysses;

static long g_checks = 0;

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

static uint32_t find_group(const uint32_t *begin, uint32_t x) {
    uint32_t g = 0;
    for (int q = 1; q < kMaxWorld; ++q) g += begin[q] <= x ? 1u : 0u;
    return g;
}

// The kernels' two-halves block order: of a launch's n blocks, block x
// takes block x / 2 (x even) or ceil(n / 2) + x / 2 (x odd).  Mode 0 of the
// relayout, the plane copy and the fused pass run their blocks in this
// order; replaying them through it checks, for every geometry here, that
// each vector is still written exactly once.
static uint32_t halves(uint32_t x, uint32_t n) {
    return (x & 1) ? ((n + 1) >> 1) + (x >> 1) : (x >> 1);
}

// The kernels' split_rows, with the bound on the multiply-high numerator.
static void split_rows(const RowSplit &rs, uint32_t s0, uint32_t lane, uint32_t *row,
                       uint32_t *col) {
    const uint32_t row0 = div32(s0, rs.m, rs.s1, rs.s2);
    REQUIRE(row0 == s0 / rs.vpr, "row division of %u by %u", s0, rs.vpr);
    const uint32_t t = s0 - row0 * rs.vpr + lane;
    REQUIRE(t < 65536u, "lane numerator %u out of range", t);
    const uint32_t dr = rs.vpr == 1 ? t : umulhi(t, rs.magic);
    REQUIRE(dr == t / rs.vpr, "lane division of %u by %u", t, rs.vpr);
    *row = row0 + dr;
    *col = t - dr * rs.vpr;
}

// Source of destination vector dv (within all b planes of shard r) by the
// definition, as (rank, vector within all b planes of that source shard).
static void defined_source(const Plan &p, int mode, int r, int64_t dv, int *want_j,
                           int64_t *want_src) {
    const int64_t hv = p.d * p.esz / 16;   // vectors per head row
    int64_t v = dv;
    if (mode == 0) {   // dst (b, s_global, H_r, hv)
        const int64_t e = v % hv; v /= hv;
        const int64_t hh = v % p.H[r]; v /= p.H[r];
        const int64_t Sg = v % p.s_global; const int64_t bi = v / p.s_global;
        int j = 0;
        while (!(p.seq_off[j] <= Sg && Sg < p.seq_off[j + 1])) ++j;
        *want_j = j;
        *want_src = ((bi * p.S[j] + (Sg - p.seq_off[j])) * p.n_global + p.head_off[r] + hh) * hv + e;
    } else {           // dst (b, S_r, n_global, hv)
        const int64_t e = v % hv; v /= hv;
        const int64_t Hg = v % p.n_global; v /= p.n_global;
        const int64_t s = v % p.S[r]; const int64_t bi = v / p.S[r];
        int j = 0;
        while (!(p.head_off[j] <= Hg && Hg < p.head_off[j + 1])) ++j;
        *want_j = j;
        *want_src = ((bi * p.s_global + p.seq_off[r] + s) * p.H[j] + (Hg - p.head_off[j])) * hv + e;
    }
}

// The relayout kernel over every (block, plane, tensor, lane) of its grid,
// with planes handed out in launches of `per_launch` planes: each launch's
// shards start at its first plane p0 (the caller moves the pointers), and a
// launch of several planes adds blockIdx.y planes in the kernel.
static void check_relayout(const Plan &p, int mode, uint32_t per_launch, uint32_t tensors) {
    RelayoutArgs a;
    const uint64_t gx = fill_relayout(p, mode, &a);
    const ModeGeom &g = p.mode[mode];
    std::vector<std::vector<std::vector<int>>> hits(tensors, std::vector<std::vector<int>>(p.world));
    for (uint32_t tt = 0; tt < tensors; ++tt)
        for (int r = 0; r < p.world; ++r)
            hits[tt][r].assign(static_cast<size_t>(p.b * g.dst_plane[r] / 16), 0);
    for (int64_t p0 = 0; p0 < p.b; p0 += per_launch) {
        const uint32_t planes = static_cast<uint32_t>(std::min<int64_t>(per_launch, p.b - p0));
        for (uint32_t t = 0; t < tensors; ++t)
            for (uint32_t y = 0; y < planes; ++y)
                for (uint32_t xb = 0; xb < gx; ++xb)
                    for (uint32_t lane = 0; lane < kRelayoutBlock; ++lane) {
                        const uint32_t x = mode == 0 ? halves(xb, uint32_t(gx)) : xb;
                        const uint32_t r = find_group(a.blk_begin, x);
                        REQUIRE(r < uint32_t(p.world), "block past the world");
                        const uint32_t s0 = (x - a.blk_begin[r]) * kRelayoutBlock;
                        REQUIRE(s0 < a.nvec[r], "block starts past its shard");
                        const uint32_t v = s0 + lane;
                        uint32_t row, col;
                        split_rows(a.row[r], s0, lane, &row, &col);
                        if (v >= a.nvec[r]) continue;
                        const uint32_t key = a.key_col ? col : row;
                        const uint32_t j = find_group(a.bound, key);
                        REQUIRE(j < uint32_t(p.world), "owner past the world");
                        // planes past the launch's first: only in launches of several
                        const uint64_t ky = planes > 1 ? y : 0;
                        REQUIRE(a.src_plane[j] < (uint64_t{1} << 32), "plane size past 32 bits");
                        const int64_t sv = int64_t(uint64_t(p0) * a.src_plane[j]) + a.off[r][j] +
                                           int64_t(uint64_t(row) * a.pitch[r][j] + col) +
                                           int64_t(ky * uint32_t(a.src_plane[j]));
                        const uint64_t dv = uint64_t(p0) * a.dst_plane[r] + v + ky * a.dst_plane[r];
                        REQUIRE(dv < hits[t][r].size(), "destination past shard %u", r);
                        hits[t][r][dv] += 1;
                        int want_j;
                        int64_t want_src;
                        defined_source(p, mode, int(r), int64_t(dv), &want_j, &want_src);
                        REQUIRE(int(j) == want_j && sv == want_src,
                                "mode %d W=%d: dst (%u,%llu) reads (%u,%lld), want (%d,%lld)",
                                mode, p.world, r, (unsigned long long)dv, j, (long long)sv,
                                want_j, (long long)want_src);
                        REQUIRE(sv >= 0 && sv < p.b * g.src_plane[j] / 16, "source past shard");
                    }
    }
    for (uint32_t tt = 0; tt < tensors; ++tt)
        for (int r = 0; r < p.world; ++r)
            for (size_t i = 0; i < hits[tt][r].size(); ++i)
                REQUIRE(hits[tt][r][i] == 1, "mode %d tensor %u rank %d vector %zu written %d times",
                        mode, tt, r, i, hits[tt][r][i]);
}

// The plane copy: window r (one plane) to the plane the caller points dst r
// at, every vector once.
static void check_plane_copy(const Plan &p, int mode) {
    CopyArgs c;
    const uint64_t gc = fill_plane_copy(p, mode, &c);
    std::vector<std::vector<int>> hits(p.world);
    for (int r = 0; r < p.world; ++r)
        hits[r].assign(static_cast<size_t>(p.mode[mode].dst_plane[r] / 16), 0);
    for (uint32_t xb = 0; xb < gc; ++xb)
        for (uint32_t lane = 0; lane < kRelayoutBlock; ++lane) {
            const uint32_t x = halves(xb, uint32_t(gc));
            const uint32_t r = find_group(c.blk_begin, x);
            REQUIRE(r < uint32_t(p.world), "copy block past the world");
            const uint32_t v = (x - c.blk_begin[r]) * kRelayoutBlock + lane;
            if (v >= c.nvec[r]) continue;
            REQUIRE(uint64_t(c.nvec[r]) * 16 == uint64_t(p.mode[mode].dst_plane[r]), "copy size");
            hits[r][v] += 1;
        }
    for (int r = 0; r < p.world; ++r)
        for (size_t i = 0; i < hits[r].size(); ++i) REQUIRE(hits[r][i] == 1, "copy coverage");
}

// The fused gather (mode 0, bf16, L = d/8 lanes per head row).
static void check_fused(const Plan &p) {
    FusedArgs a;
    const uint64_t gx = fill_fused(p, &a);
    const uint32_t L = static_cast<uint32_t>(p.d / 8);
    const ModeGeom &g = p.mode[0];
    REQUIRE(a.half_d == uint32_t(p.d / 2) && a.inv_d * float(p.d) == 1.0f, "fused constants");
    REQUIRE(a.pitch == uint32_t(p.G / 16), "fused source pitch");
    // the kernel takes the last q with bound[q] <= row, which is the count
    // of such q only for ascending bounds
    for (int q = 2; q < kMaxWorld; ++q) REQUIRE(a.bound[q] >= a.bound[q - 1], "fused bounds ascend");
    std::vector<std::vector<int>> hits(p.world);
    for (int r = 0; r < p.world; ++r) hits[r].assign(static_cast<size_t>(p.b * g.dst_plane[r] / 16), 0);
    for (uint32_t y = 0; y < p.b; ++y)
        for (uint32_t xb = 0; xb < gx; ++xb) {
            const uint32_t x = halves(xb, uint32_t(gx));
            const uint32_t r = find_group(a.blk_begin, x);
            REQUIRE(r < uint32_t(p.world), "fused block past the world");
            const uint32_t s0 = (x - a.blk_begin[r]) * kFusedBlock;
            REQUIRE(s0 < a.nvec[r], "fused block starts past its shard");
            const uint32_t last = a.nvec[r] - 1;
            REQUIRE(int64_t(a.row[r].vpr) == p.H[r] * L, "fused destination row length");
            for (uint32_t tid = 0; tid < kFusedBlock; ++tid) {
                const bool ok = s0 + tid <= last;
                const uint32_t lt = std::min(s0 + tid, last) - s0;
                const uint32_t lane = tid & (L - 1);
                uint32_t row, col;
                split_rows(a.row[r], s0, lt, &row, &col);
                const uint32_t j = find_group(a.bound, row);
                REQUIRE(j < uint32_t(p.world), "fused source past the world");
                // the loads of every lane (clamped ones too) stay in bounds
                // (one launch holds every plane here: b <= 65535)
                const int64_t sv = int64_t(uint64_t(y) * a.src_plane[j]) + a.off[r][j] +
                                   int64_t(uint64_t(row) * a.pitch + col);
                REQUIRE(sv >= 0 && sv < int64_t(uint64_t(p.b) * a.src_plane[j]),
                        "fused load past shard");
                REQUIRE(row < uint64_t(p.s_global), "rotary row past the table");
                REQUIRE(4 * lane + 3 < a.half_d && 8 * lane + 7 < uint32_t(p.d), "lane past d");
                if (!ok) {
                    // a clamped lane's whole head row is past the shard
                    REQUIRE(s0 + (tid & ~(L - 1)) > last, "head row partly past the shard");
                    continue;
                }
                REQUIRE(col % L == lane, "lane %u holds column %u of a %u-lane row", tid, col, L);
                const uint64_t dv = uint64_t(y) * a.dst_plane[r] + s0 + lt;
                REQUIRE(dv < hits[r].size(), "fused store past shard");
                REQUIRE(uint64_t(row) * a.row[r].vpr + col == s0 + lt, "fused row split");
                hits[r][dv] += 1;
                int want_j;
                int64_t want_src;
                defined_source(p, 0, int(r), int64_t(dv), &want_j, &want_src);
                REQUIRE(int(j) == want_j && sv == want_src, "fused source");
                // rotary row of the destination row's global position
                const int64_t Sg = (int64_t(dv) / (p.H[r] * L)) % p.s_global;
                REQUIRE(int64_t(row) == Sg, "fused rotary position");
            }
        }
    for (int r = 0; r < p.world; ++r)
        for (size_t i = 0; i < hits[r].size(); ++i)
            REQUIRE(hits[r][i] == 1, "fused coverage rank %d vector %zu: %d", r, i, hits[r][i]);
}

static void check_geometry(int world, int64_t b, int64_t d, int dtype,
                           const std::vector<int64_t> &S, const std::vector<int64_t> &H) {
    Plan p;
    std::string msg;
    const int rc = plan_build(&p, world, b, d, S.data(), H.data(), dtype, 1 << 30, &msg);
    REQUIRE(rc == kOk, "plan_build failed: %s", msg.c_str());
    for (int mode = 0; mode < 2; ++mode) {
        check_relayout(p, mode, 1 << 16, 1);
        for (uint32_t t : {2u, 3u, 4u}) check_relayout(p, mode, 1 << 16, t);   // tensors in one launch
        if (b > 1) check_relayout(p, mode, 1, 1);   // one plane per launch (the chunked passes)
        check_plane_copy(p, mode);
    }
    const int64_t L = d / 8;
    if (dtype == 0 && L >= 1 && L <= 64 && (L & (L - 1)) == 0 && d % 8 == 0) check_fused(p);
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
    // sizes whose products would overflow 64 bits are refused before any
    // multiplication: a huge d (d * esz wraps), a huge batch, huge splits
    const int64_t one[1] = {1};
    REQUIRE(plan_build(&p, 1, 1, (int64_t{1} << 59) + 8, one, one, 0, 0, &m) == kEInval,
            "d = 2^59 + 8");
    REQUIRE(plan_build(&p, 1, 1, INT64_MAX, one, one, 0, 0, &m) == kEInval, "d = INT64_MAX");
    REQUIRE(plan_build(&p, 1, 1, 262144, one, one, 2, 0, &m) == kEInval, "fp32 d over 512 KiB");
    REQUIRE(plan_build(&p, 1, 1, 262144, one, one, 0, 0, &m) == kOk, "bf16 d at 512 KiB");
    REQUIRE(plan_build(&p, 2, INT64_MAX, 8, s2, h2, 0, 0, &m) == kEInval, "b = INT64_MAX");
    REQUIRE(plan_build(&p, 2, int64_t{1} << 31, 8, s2, h2, 0, 0, &m) == kOk, "b = 2^31");
    REQUIRE(plan_build(&p, 2, (int64_t{1} << 31) + 1, 8, s2, h2, 0, 0, &m) == kEInval, "b > 2^31");
    const int64_t huge_s[2] = {INT64_MAX, 1}, huge_h[2] = {INT64_MAX, 1};
    REQUIRE(plan_build(&p, 2, 1, 8, huge_s, h2, 0, 0, &m) == kEInval, "seq split INT64_MAX");
    REQUIRE(plan_build(&p, 2, 1, 8, s2, huge_h, 0, 0, &m) == kEInval, "head split INT64_MAX");
    // a plane of 2^31 vectors or more is refused; just below is accepted
    const int64_t s_big[1] = {int64_t{1} << 31}, h_one[1] = {1};
    REQUIRE(plan_build(&p, 1, 1, 8, s_big, h_one, 0, 0, &m) == kEInval, "plane of 2^31 vectors");
    const int64_t s_ok[1] = {(int64_t{1} << 31) - 1};
    REQUIRE(plan_build(&p, 1, 1, 8, s_ok, h_one, 0, 0, &m) == kOk, "plane below 2^31 vectors");
    // whole shards beyond 2^58 bytes
    const int64_t s_plane[1] = {(int64_t{1} << 31) - 1};
    REQUIRE(plan_build(&p, 1, int64_t{1} << 27, 8, s_plane, h_one, 0, 0, &m) == kEInval,
            "shard beyond 2^58 bytes");
    // every accepted plan has positive sizes
    REQUIRE(plan_build(&p, 2, 3, 8, s2, h2, 0, 0, &m) == kOk, "small plan");
    for (int mm = 0; mm < 2; ++mm)
        for (int r = 0; r < 2; ++r)
            REQUIRE(p.mode[mm].src_plane[r] > 0 && p.mode[mm].dst_plane[r] > 0, "sizes");
    // the FastVideo geometry: 896,000,000 bytes per rank per plane
    const int64_t s4[4] = {62500, 62500, 62500, 62500}, h4[4] = {14, 14, 14, 14};
    REQUIRE(plan_build(&p, 4, 3, 128, s4, h4, 0, 1 << 30, &m) == kOk, "fastvideo plan");
    REQUIRE(p.mode[0].window_bytes == 896000000 && p.mode[1].window_bytes == 896000000,
            "window bytes");
}

// The piece table against the definition: each piece's rectangle in both
// frames, and the pieces sharing a shard tile it exactly.
static void check_pieces(const Plan &p) {
    const int w = p.world;
    const int64_t hb = p.d * p.esz;
    for (int mode = 0; mode < 2; ++mode)
        for (int j = 0; j < w; ++j)
            for (int r = 0; r < w; ++r) {
                const Piece &pc = p.mode[mode].piece[j * w + r];
                REQUIRE(pc.src_off == pc.src_row0 * pc.src_pitch + pc.src_col0, "src_off");
                REQUIRE(pc.dst_off == pc.dst_row0 * pc.dst_pitch + pc.dst_col0, "dst_off");
                if (mode == 0) {
                    REQUIRE(pc.rows == p.S[j] && pc.row_bytes == p.R[r], "mode 0 extent");
                    REQUIRE(pc.src_col0 == p.head_off[r] * hb && pc.src_pitch == p.G, "mode 0 src");
                    REQUIRE(pc.dst_row0 == p.seq_off[j] && pc.dst_pitch == p.R[r], "mode 0 dst");
                } else {
                    REQUIRE(pc.rows == p.S[r] && pc.row_bytes == p.R[j], "mode 1 extent");
                    REQUIRE(pc.src_row0 == p.seq_off[r] && pc.src_pitch == p.R[j], "mode 1 src");
                    REQUIRE(pc.dst_col0 == p.head_off[j] * hb && pc.dst_pitch == p.G, "mode 1 dst");
                }
            }
}

int main() {
    check_magic();
    check_errors();
    std::mt19937_64 rng(12345);
    const int dtypes[] = {0, 2, 3, 5, 1};
    for (int it = 0; it < 200; ++it) {
        const int world = 1 + static_cast<int>(rng() % 8);
        const int dtype = dtypes[rng() % 5];
        const int64_t esz = dtype_size(dtype);
        const int64_t unit = 16 / esz;   // smallest legal d
        const int64_t d = unit * (1 + static_cast<int64_t>(rng() % 3)) * (it % 4 == 0 ? 8 : 1);
        const int64_t b = 1 + static_cast<int64_t>(rng() % 3);
        std::vector<int64_t> S(world), H(world);
        int64_t ss = 0, hs = 0;
        for (int r = 0; r < world; ++r) {
            S[r] = static_cast<int64_t>(rng() % 40) - (it % 3 == 0 ? 5 : 0);
            if (S[r] < 0) S[r] = 0;
            H[r] = static_cast<int64_t>(rng() % 7) - (it % 5 == 0 ? 2 : 0);
            if (H[r] < 0) H[r] = 0;
            ss += S[r];
            hs += H[r];
        }
        if (ss == 0) S[0] = 3;
        if (hs == 0) H[world - 1] = 2;
        Plan p;
        std::string msg;
        REQUIRE(plan_build(&p, world, b, d, S.data(), H.data(), dtype, 0, &msg) == kOk, "plan");
        check_pieces(p);
        check_geometry(world, b, d, dtype, S, H);
    }
    // long rows: row length at the 32768-vector limit, one-vector rows
    check_geometry(2, 1, 2048, 2, {3, 2}, {40, 24});
    check_geometry(3, 2, 8, 0, {50, 1, 77}, {1, 1, 1});
    check_geometry(4, 1, 16, 5, {9, 0, 33, 5}, {1, 1, 1, 1});
    // the fused pass at every head dimension it takes, with zero splits
    for (int it = 0; it < 60; ++it) {
        const int world = 1 + static_cast<int>(rng() % 8);
        const int64_t d = int64_t{8} << (it % 7);   // 8 .. 512
        std::vector<int64_t> S(world), H(world);
        for (int r = 0; r < world; ++r) {
            S[r] = static_cast<int64_t>(rng() % 23);
            H[r] = static_cast<int64_t>(rng() % (d >= 256 ? 4 : 19));
        }
        S[0] += 1;
        H[world - 1] += 1;
        check_geometry(world, 1 + static_cast<int64_t>(rng() % 2), d, 0, S, H);
    }
    // the shapes of the timed workloads, scaled down in sequence length
    check_geometry(8, 1, 128, 0, std::vector<int64_t>(8, 95), std::vector<int64_t>(8, 5));
    check_geometry(7, 2, 128, 0, {9, 40, 3, 17, 1, 22, 31}, {6, 6, 6, 6, 6, 5, 5});
    check_geometry(7, 2, 128, 3, {9, 40, 3, 17, 1, 22, 31}, {6, 6, 6, 6, 6, 5, 5});
    check_geometry(4, 3, 128, 0, {25, 25, 25, 25}, {14, 14, 14, 14});
    check_div32(rng);
    std::printf("OK %ld\n", g_checks);
    return 0;
}
