// gfx950 (CDNA4) kernels of the Ulysses 4D relayout.
//
// The relayout is pure data movement: every byte is read once and written
// once, so HBM bandwidth bounds it and there is no contraction for MFMA.
// Each (source rank j -> destination rank r) piece is a set of rows that are
// contiguous on both sides (at least d*elem_size >= 16 bytes, in practice
// 640 B and up), so every lane moves whole 16-byte vectors with coalesced
// loads and stores and no LDS staging is needed: the source and destination
// strides already agree at 16-byte granularity.  The permutation itself is
// only addressing, as the pages put it (fast-ulysses 0.1.0 introduction: the
// sequence/head relayout is expressed as copy strides instead of separate
// permute kernels).
//
// Work split: grid.x walks the blocks of all pieces (a piece table in the
// kernarg segment), grid.y the batch planes, grid.z the tensors.  The default
// walk is in bands: the W pieces that share one row-sharded shard (source j
// in mode 0, destination r in mode 1) take consecutive blocks band by band,
// one band of ULY_BLOCK * ULY_UNROLL consecutive vectors of a piece per
// block, so neighbouring blocks sweep whole rows of that shard and W
// contiguous streams of the head-sharded side.  Each thread issues its
// ULY_UNROLL 16-byte loads, ULY_BLOCK apart, before its stores; each load
// instruction of a wavefront covers 1 KiB of contiguous memory.  A flat walk
// (each piece's blocks in turn, relayout_kernel) remains for comparison.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

// Launch shape, chosen by measurement on MI355X (W=8, 75,600 tokens, bf16):
// one-wave blocks moving one vector per thread, in bands of 64 vectors (see
// the band table in the plan), beat every larger block, deeper unroll,
// longer band, XCD-aware block permutation and capped occupancy tried.
#ifndef ULY_BLOCK
#define ULY_BLOCK 64
#endif
#ifndef ULY_UNROLL
#define ULY_UNROLL 1
#endif
// bit 0: non-temporal loads, bit 1: non-temporal stores
#ifndef ULY_NT
#define ULY_NT 3
#endif
// The generic fused kernel (head dimensions other than 128) keeps two rows
// per thread so that they share one divide/sqrt sequence (128 x 2 measured
// best for it).
#ifndef ULY_FUSED_BLOCK
#define ULY_FUSED_BLOCK 128
#endif
#ifndef ULY_FUSED_UNROLL
#define ULY_FUSED_UNROLL 2
#endif
// 16-byte vectors of one head row per lane in the generic fused kernel (1, 2
// or 4).
// One is fastest on MI355X: two or four make each load instruction of a
// wave touch two or four times the cache lines.
#ifndef ULY_FUSED_VPL
#define ULY_FUSED_VPL 1
#endif
// Share one divide/sqrt sequence between the unroll slots of a 16-lane row.
#ifndef ULY_FUSED_SHARE_INV
#define ULY_FUSED_SHARE_INV 1
#endif
// Vectors per lane of the band kernel for d = 128 (1, 2 or 4; each lane
// handles that many head rows of q and as many of k).  One measured best.
#ifndef ULY_FUSED_BAND_UNROLL
#define ULY_FUSED_BAND_UNROLL 1
#endif

namespace ulysses {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 load16(const unsigned char *p) {
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
}

template <bool NT>
__device__ __forceinline__ void store16(unsigned char *p, u32x4 v) {
    u32x4 *q = reinterpret_cast<u32x4 *>(p);
    if constexpr (NT) __builtin_nontemporal_store(v, q);
    else *q = v;
}

// The piece owning block x: the last entry of blk_begin that is <= x.
// blk_begin is strictly ascending over used entries (blk_begin[0] == 0) and
// 0xFFFFFFFF past them.  Six dependent scalar loads of a binary search; a
// full 64-entry scan would hold 64 SGPRs and spill.
__device__ __forceinline__ uint32_t find_piece(const uint32_t *blk_begin, uint32_t x) {
    uint32_t p = 0;
#pragma unroll
    for (uint32_t step = kMaxPieces / 2; step > 0; step /= 2)
        if (blk_begin[p + step] <= x) p += step;
    return p;
}

// Splits t (< 2^16) into (t / vpr, t % vpr) with one multiply-high; see
// row_magic() in the plan for the bound.
__device__ __forceinline__ uint32_t div_vpr(uint32_t t, uint32_t vpr, uint32_t magic) {
    return vpr == 1 ? t : __umulhi(t, magic);
}

// --------------------------------------------------------------------------
// Relayout (modes 0 and 1, and the window copy of the chunked mode)
// --------------------------------------------------------------------------

template <int BLOCK, int UNROLL, bool NTL, bool NTS>
__global__ void __launch_bounds__(BLOCK) relayout_kernel(const RelayoutArgs a) {
    const uint32_t x = blockIdx.x;
    const uint32_t p = find_piece(a.blk_begin, x);
    const PieceArgs pc = a.piece[p];
    const uint64_t ps = uint64_t(a.src_plane0) + blockIdx.y;
    const uint64_t pd = uint64_t(a.dst_plane0) + blockIdx.y;
    const unsigned char *sb = a.src[blockIdx.z][pc.j] + (ps * a.src_plane[pc.j] + pc.src_off) * 16;
    unsigned char *db = a.dst[blockIdx.z][pc.r] + (pd * a.dst_plane[pc.r] + pc.dst_off) * 16;
    const uint32_t s0 = (x - a.blk_begin[p]) * uint32_t(BLOCK * UNROLL);
    // Row and column of the block's first vector (uniform); per-lane offsets
    // from there stay below 2^16 (row length <= 32768 vectors).
    const uint32_t row0 = s0 / pc.vpr;
    const uint32_t col0 = s0 - row0 * pc.vpr;
    u32x4 v[UNROLL];
    uint64_t doff[UNROLL];
    bool ok[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
        const uint32_t lin = threadIdx.x + uint32_t(k * BLOCK);
        const uint32_t t = col0 + lin;
        const uint32_t dr = div_vpr(t, pc.vpr, pc.magic);
        const uint32_t col = t - dr * pc.vpr;
        const uint32_t row = row0 + dr;
        ok[k] = s0 + lin < pc.nvec;
        const uint64_t soff = uint64_t(row) * pc.src_pitch + col;
        doff[k] = uint64_t(row) * pc.dst_pitch + col;
        if (ok[k]) v[k] = load16<NTL>(sb + soff * 16);
    }
#pragma unroll
    for (int k = 0; k < UNROLL; ++k)
        if (ok[k]) store16<NTS>(db + doff[k] * 16, v[k]);
}

// Band traversals: the W pieces that share a row-sharded shard take
// consecutive blocks band by band, so blocks running side by side sweep whole
// contiguous rows of that shard and W contiguous streams of the head-sharded
// side.  A band is band_vecs vectors of a piece (the default), band_rows rows
// of a piece (walked in chunks of BLOCK * UNROLL vectors), or, when the
// pieces differ in row width, band_rows rows of every piece cut into chunks
// with one chunk per block (RelayoutArgs describes the three tables).
template <int BLOCK, int UNROLL, bool NTL, bool NTS>
__global__ void __launch_bounds__(BLOCK) relayout_band_kernel(const RelayoutArgs a) {
    const uint32_t x = blockIdx.x;
    uint32_t g = 0;
#pragma unroll
    for (int q = 1; q < kMaxWorld; ++q) g += (a.grp_begin[q] <= x) ? 1u : 0u;
    const uint32_t local = x - a.grp_begin[g];
    uint32_t k, begin, end;
    if (a.chunks_per_band != 0) {
        // row-aligned chunks: band of band_rows rows of every piece, chunk c
        // of piece k (chunk_begin is non-decreasing; the last entry <= q
        // always belongs to a piece with chunks)
        const uint32_t band = div32(local, a.band_m, a.band_s1, a.band_s2);
        const uint32_t q = local - band * a.chunks_per_band;
        k = 0;
#pragma unroll
        for (int i = 1; i < kMaxWorld; ++i) k += (a.chunk_begin[i] <= q) ? 1u : 0u;
        const uint32_t c = q - a.chunk_begin[k];
        const uint32_t vpr = a.piece[g * a.world + k].vpr;
        const uint32_t band0 = band * a.band_rows * vpr;
        begin = band0 + c * a.chunk_vecs;
        end = min(min(begin + a.chunk_vecs, band0 + a.band_rows * vpr),
                  a.piece[g * a.world + k].nvec);
    } else {
        const uint32_t band = local / a.world;
        k = local - band * a.world;
        const uint32_t vpr = a.piece[g * a.world + k].vpr;
        const uint32_t span = a.band_vecs != 0 ? a.band_vecs : a.band_rows * vpr;
        begin = band * span;
        end = min(begin + span, a.piece[g * a.world + k].nvec);
    }
    const PieceArgs pc = a.piece[g * a.world + k];
    const uint64_t ps = uint64_t(a.src_plane0) + blockIdx.y;
    const uint64_t pd = uint64_t(a.dst_plane0) + blockIdx.y;
    const unsigned char *sb = a.src[blockIdx.z][pc.j] + (ps * a.src_plane[pc.j] + pc.src_off) * 16;
    unsigned char *db = a.dst[blockIdx.z][pc.r] + (pd * a.dst_plane[pc.r] + pc.dst_off) * 16;

    for (uint32_t s0 = begin; s0 < end; s0 += uint32_t(BLOCK * UNROLL)) {
        const uint32_t row0 = s0 / pc.vpr;
        const uint32_t col0 = s0 - row0 * pc.vpr;
        u32x4 v[UNROLL];
        uint64_t doff[UNROLL];
        bool ok[UNROLL];
#pragma unroll
        for (int kk = 0; kk < UNROLL; ++kk) {
            const uint32_t lin = threadIdx.x + uint32_t(kk * BLOCK);
            const uint32_t t = col0 + lin;
            const uint32_t dr = div_vpr(t, pc.vpr, pc.magic);
            const uint32_t col = t - dr * pc.vpr;
            const uint32_t row = row0 + dr;
            ok[kk] = s0 + lin < end;
            const uint64_t soff = uint64_t(row) * pc.src_pitch + col;
            doff[kk] = uint64_t(row) * pc.dst_pitch + col;
            if (ok[kk]) v[kk] = load16<NTL>(sb + soff * 16);
        }
#pragma unroll
        for (int kk = 0; kk < UNROLL; ++kk)
            if (ok[kk]) store16<NTS>(db + doff[kk] * 16, v[kk]);
    }
}

uint32_t relayout_vectors_per_block() { return ULY_BLOCK * ULY_UNROLL; }
uint32_t relayout_block_threads() { return ULY_BLOCK; }

hipError_t launch_relayout(const RelayoutArgs &a, uint32_t grid_x, uint32_t planes,
                           uint32_t tensors, hipStream_t stream) {
    if (grid_x == 0 || planes == 0 || tensors == 0) return hipSuccess;
    void *argv[] = {const_cast<RelayoutArgs *>(&a)};
    const void *fn =
        (a.band_rows != 0 || a.band_vecs != 0)
            ? reinterpret_cast<const void *>(
                  &relayout_band_kernel<ULY_BLOCK, ULY_UNROLL, (ULY_NT & 1) != 0,
                                        (ULY_NT & 2) != 0>)
            : reinterpret_cast<const void *>(
                  &relayout_kernel<ULY_BLOCK, ULY_UNROLL, (ULY_NT & 1) != 0, (ULY_NT & 2) != 0>);
    return hipLaunchKernel(fn, dim3(grid_x, planes, tensors), dim3(ULY_BLOCK, 1, 1), argv, 0,
                           stream);
}

// --------------------------------------------------------------------------
// Fused mode 0 with QK RMSNorm + RoPE (bf16 in, bf16 out, fp32 arithmetic)
// --------------------------------------------------------------------------
//
// A head row of d bf16 elements is d/8 16-byte vectors.  Each lane holds VPL
// consecutive vectors of one row ("a unit": elements 8*VPL*l .. 8*VPL*l +
// 8*VPL - 1 of lane l, rotary pairs 4*VPL*l ..), so L = d / (8*VPL)
// consecutive lanes hold one row.  The piece table arrives in units of VPL
// vectors; rows are whole numbers of units and blocks start on multiples of
// L, so a thread's lane within its row is threadIdx.x % L for every unit.
// The operation order is fixed so the result is reproducible bit for bit:
//   partial p_m, one per vector: fma chain over its 8 squares, ascending;
//   ss = pairwise tree over p_0 .. p_{d/8-1} with adjacent pairing: the
//        first log2(VPL) levels inside the lane, the rest as an xor
//        butterfly over the L lanes (every lane ends with the same bits,
//        fp32 + being commutative);
//   ms = ss * (1/d), which equals ss / d exactly since d is a power of two;
//   inv = 1 / sqrt(ms + eps), correctly rounded sqrt and division;
//   y = (x * inv) * gamma;  rotation products rounded one by one.
// The library is compiled with -ffp-contract=off so no product is fused.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two floats to bf16 (nearest even) and pack them, lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = {lo, hi};
    const bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over groups of L consecutive lanes; every lane of a group gets the
// same bits.  Within a 16-lane DPP row: neighbours (quad_perm 1,0,3,2), pairs
// of neighbours (quad_perm 2,3,0,1), then the mirrored half-row and row;
// after each stage all lanes of a half are equal, so the mirror adds the two
// halves, as an xor butterfly would.  Wider groups continue with shuffles.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (L >= 2) v = v + dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (L >= 4) v = v + dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (L >= 8) v = v + dpp<0x141>(v);   // row_half_mirror
    if constexpr (L >= 16) v = v + dpp<0x140>(v);  // row_mirror
    if constexpr (L >= 32) v = v + __shfl_xor(v, 16, L);
    if constexpr (L >= 64) v = v + __shfl_xor(v, 32, L);
    return v;
}

template <int BLOCK, int UNROLL, int VPL, int L>
__global__ void __launch_bounds__(BLOCK) fused_kernel(const FusedArgs a) {
    constexpr int E = 8 * VPL;   // elements per lane
    const uint32_t x = blockIdx.x;
    const uint32_t tensor = blockIdx.z;
    // the block's piece (in units of VPL vectors) and first unit: a band of
    // the piece when the table is banded, else a flat block of it
    PieceArgs pc;
    uint32_t s0, end;
    if (a.band_vecs != 0) {
        uint32_t g = 0;
#pragma unroll
        for (int q = 1; q < kMaxWorld; ++q) g += (a.grp_begin[q] <= x) ? 1u : 0u;
        const uint32_t local = x - a.grp_begin[g];
        const uint32_t band = local / a.world;
        pc = a.piece[g * a.world + (local - band * a.world)];
        s0 = band * a.band_vecs;
        end = min(s0 + a.band_vecs, pc.nvec);
        if (s0 >= end) return;   // uniform: the whole block is past its piece
    } else {
        const uint32_t p = find_piece(a.blk_begin, x);
        pc = a.piece[p];
        s0 = (x - a.blk_begin[p]) * uint32_t(BLOCK * UNROLL);
        end = pc.nvec;
    }
    const uint32_t row0 = s0 / pc.vpr;
    const uint32_t col0 = s0 - row0 * pc.vpr;
    const uint64_t plane = uint64_t(a.plane0) + blockIdx.y;
    const unsigned char *sb =
        a.src[tensor][pc.j] + (plane * a.src_plane[pc.j] + pc.src_off) * (16 * VPL);
    unsigned char *db =
        a.dst[tensor][pc.r] + (plane * a.dst_plane[pc.r] + pc.dst_off) * (16 * VPL);
    const uint32_t lane = threadIdx.x & (L - 1);
    const uint32_t half_d = a.d / 2;

    // this lane's gains
    float g[E];
    {
        const f32x4 *gp = reinterpret_cast<const f32x4 *>(a.gamma[tensor] + E * lane);
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
            const f32x4 t = gp[i];
            g[4 * i] = t.x; g[4 * i + 1] = t.y; g[4 * i + 2] = t.z; g[4 * i + 3] = t.w;
        }
    }
    const float eps = a.eps;
    const float inv_d = a.inv_d;

    u32x4 xv[UNROLL][VPL];
    f32x4 cv[UNROLL][VPL], sv[UNROLL][VPL];
    uint64_t doff[UNROLL];
    bool ok[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
        const uint32_t lin = threadIdx.x + uint32_t(k * BLOCK);
        const uint32_t t = col0 + lin;
        const uint32_t dr = div_vpr(t, pc.vpr, pc.magic);
        const uint32_t col = t - dr * pc.vpr;
        const uint32_t row = row0 + dr;
        ok[k] = s0 + lin < end;
        const uint64_t soff = uint64_t(row) * pc.src_pitch + col;
        doff[k] = uint64_t(row) * pc.dst_pitch + col;
        // global sequence position of this source row
        const uint64_t tab = uint64_t(pc.src_row0 + row) * half_d + 4 * VPL * lane;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            xv[k][v] = u32x4{0, 0, 0, 0};
            cv[k][v] = f32x4{0.f, 0.f, 0.f, 0.f};
            sv[k][v] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (ok[k]) {
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                xv[k][v] = load16<true>(sb + soff * (16 * VPL) + 16 * v);
                cv[k][v] = *reinterpret_cast<const f32x4 *>(a.rope_cos + tab + 4 * v);
                sv[k][v] = *reinterpret_cast<const f32x4 *>(a.rope_sin + tab + 4 * v);
            }
        }
    }
    // Squares and row sums of every slot first, then 1/sqrt once per row.
    float xs[UNROLL][E];
    float ss[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
        float *xf = xs[k];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            xf[8 * v + 0] = bf16_lo(xv[k][v].x); xf[8 * v + 1] = bf16_hi(xv[k][v].x);
            xf[8 * v + 2] = bf16_lo(xv[k][v].y); xf[8 * v + 3] = bf16_hi(xv[k][v].y);
            xf[8 * v + 4] = bf16_lo(xv[k][v].z); xf[8 * v + 5] = bf16_hi(xv[k][v].z);
            xf[8 * v + 6] = bf16_lo(xv[k][v].w); xf[8 * v + 7] = bf16_hi(xv[k][v].w);
        }
        float part[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            part[v] = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                part[v] = __builtin_fmaf(xf[8 * v + i], xf[8 * v + i], part[v]);
        }
        // adjacent-pairing levels inside the lane
#pragma unroll
        for (int n = VPL; n > 1; n /= 2)
#pragma unroll
            for (int q = 0; q < n / 2; ++q) part[q] = part[2 * q] + part[2 * q + 1];
        ss[k] = group_sum<L>(part[0]);
    }
    // '/' and __builtin_sqrtf lower to the IEEE-exact sequences under hipcc's
    // default correctly rounded fp32 divide and sqrt (div_scale/div_fmas/
    // div_fixup; v_sqrt_f32 plus a one-ulp residual correction); __fsqrt_rn
    // would carry a 3-ulp fpmath bound.  ms = ss * (1/d) equals ss / d
    // exactly because d is a power of two.
    float invs[UNROLL];
    if constexpr (L == 16 && (UNROLL == 2 || UNROLL == 4) && ULY_FUSED_SHARE_INV) {
        // Every lane of a 16-lane row holds the same ss of each slot: lane k
        // of the row computes slot k's 1/sqrt and DPP row_newbcast:k hands it
        // back to the whole row (the same operations on the same value, so
        // the same bits), one divide/sqrt sequence for UNROLL slots.
        const uint32_t q = threadIdx.x & (UNROLL - 1);
        float sel = ss[0];
#pragma unroll
        for (int k = 1; k < UNROLL; ++k) sel = (q == uint32_t(k)) ? ss[k] : sel;
        const float mine = 1.0f / __builtin_sqrtf(sel * inv_d + eps);
        invs[0] = dpp<0x150>(mine);
        if constexpr (UNROLL >= 2) invs[1] = dpp<0x151>(mine);
        if constexpr (UNROLL >= 4) {
            invs[2] = dpp<0x152>(mine);
            invs[3] = dpp<0x153>(mine);
        }
    } else {
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) invs[k] = 1.0f / __builtin_sqrtf(ss[k] * inv_d + eps);
    }
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
        const float *xf = xs[k];
        const float inv = invs[k];
        float y[E];
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] = (xf[i] * inv) * g[i];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const float c[4] = {cv[k][v].x, cv[k][v].y, cv[k][v].z, cv[k][v].w};
            const float sn[4] = {sv[k][v].x, sv[k][v].y, sv[k][v].z, sv[k][v].w};
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float y0 = y[8 * v + 2 * q], y1 = y[8 * v + 2 * q + 1];
                const float e0 = y0 * c[q];
                const float e1 = y1 * sn[q];
                const float e2 = y0 * sn[q];
                const float e3 = y1 * c[q];
                o[q] = pack_bf16x2(e0 - e1, e2 + e3);
            }
            if (ok[k])
                store16<true>(db + doff[k] * (16 * VPL) + 16 * v, u32x4{o[0], o[1], o[2], o[3]});
        }
    }
}

// Block order that puts the W consecutive blocks of one band (the pieces of
// one band) on one XCD.  Workgroups go round-robin over the 8 XCDs by linear
// id, so within each run of 8 bands (8*W blocks) physical block x takes band
// 8c + (x mod 8) and piece (x mod 8W) / 8; the last, partial run keeps the
// identity order.  A bijection on [0, n); x / (8W) is taken as (x / 8) / W
// through the exact division by W.
__device__ __forceinline__ uint32_t band_xcd_order(uint32_t x, uint32_t n, const FusedArgs &a) {
    const uint32_t w = a.world;
    // x / (8w) == (x / 8) / w, through the exact division by w
    const uint32_t full = div32(n >> 3, a.world_m, a.world_s1, a.world_s2) * (8 * w);
    if (x >= full) return x;
    const uint32_t c = div32(x >> 3, a.world_m, a.world_s1, a.world_s2);
    const uint32_t rem = x - c * (8 * w);
    return (8 * c + (rem & 7)) * w + (rem >> 3);
}

// Band form for d = 128, with the relayout kernel's access shape: a one-wave
// block takes one band of 64 * UNROLL consecutive vectors of a piece, UNROLL
// vectors per lane 64 apart, 16 lanes per head row, and moves that band of
// both q and k, so the band's rotary entries are read once for the two.
// Blocks follow band_xcd_order: the W pieces of a band share an XCD, and
// with it the L2 that holds their rotary rows.  Everything block-uniform (the
// piece, the band's first row and column, the base addresses of sources,
// destinations and rotary rows) is computed once per block with scalar
// instructions, the divisions by runtime values through host-computed exact
// multipliers (div32); each lane then adds 32-bit offsets.  Lanes past the
// end of a piece reload its last vector and skip their stores, so no lane
// works on uninitialised registers and no load is predicated.  Operation
// order and rounding are those of fused_kernel; the 2 * UNROLL rows of a
// lane share one divide/sqrt sequence (lane i of each 16-lane row computes
// the i-th and DPP row_newbcast:i hands it out).
template <int UNROLL>
__global__ void __launch_bounds__(64) fused_band_kernel(const FusedArgs a) {
    static_assert(UNROLL == 1 || UNROLL == 2 || UNROLL == 4, "slots per lane");
    constexpr int T = 2;                         // q and k
    constexpr int S = T * UNROLL;                // rows per lane sharing one 1/sqrt pass
    static_assert(S <= 8, "at most 8 slots share the divide/sqrt sequence");
    constexpr uint32_t kBand = 64 * UNROLL;
    const uint32_t tid = threadIdx.x;
    const uint32_t x = band_xcd_order(blockIdx.x, gridDim.x, a);
    uint32_t g = 0;
#pragma unroll
    for (int q = 1; q < kMaxWorld; ++q) g += (a.grp_begin[q] <= x) ? 1u : 0u;
    const uint32_t local = x - a.grp_begin[g];
    const uint32_t band = div32(local, a.world_m, a.world_s1, a.world_s2);
    const PieceArgs pc = a.piece[g * a.world + (local - band * a.world)];
    const uint32_t s0 = band * kBand;
    if (s0 >= pc.nvec) return;                   // uniform: band past the piece (or empty)
    const uint32_t last = min(kBand, pc.nvec - s0) - 1;   // last valid lane index
    const uint32_t row0 = div32(s0, pc.vpr_m, pc.vpr_s1, pc.vpr_s2);
    const uint32_t col0 = s0 - row0 * pc.vpr;
    const uint64_t plane = uint64_t(a.plane0) + blockIdx.y;
    const uint64_t src_v = plane * a.src_plane[pc.j] + pc.src_off + uint64_t(row0) * pc.src_pitch;
    const uint64_t dst_v = plane * a.dst_plane[pc.r] + pc.dst_off + uint64_t(row0) * pc.dst_pitch;
    const uint32_t t0 = 0;
    const unsigned char *sb[T];
    unsigned char *db[T];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        sb[tt] = a.src[t0 + tt][pc.j] + (src_v << 4);
        db[tt] = a.dst[t0 + tt][pc.r] + (dst_v << 4);
    }
    const uint64_t trow = uint64_t(pc.src_row0 + row0) * 64;   // global position * d/2
    const unsigned char *cb = reinterpret_cast<const unsigned char *>(a.rope_cos + trow);
    const unsigned char *snb = reinterpret_cast<const unsigned char *>(a.rope_sin + trow);
    const uint32_t lane = tid & 15;

    float gm[T][8];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        const f32x4 *gp = reinterpret_cast<const f32x4 *>(a.gamma[t0 + tt] + 8 * lane);
        const f32x4 g0 = gp[0], g1 = gp[1];
        gm[tt][0] = g0.x; gm[tt][1] = g0.y; gm[tt][2] = g0.z; gm[tt][3] = g0.w;
        gm[tt][4] = g1.x; gm[tt][5] = g1.y; gm[tt][6] = g1.z; gm[tt][7] = g1.w;
    }
    const float eps = a.eps;
    const float inv_d = a.inv_d;

    u32x4 xv[T][UNROLL];
    f32x4 cv[UNROLL], sv[UNROLL];
    uint32_t doff[UNROLL];
    bool ok[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
        const uint32_t lin = tid + uint32_t(k * 64);
        ok[k] = lin <= last;
        // below 2^16: col0 < vpr <= 32768 and lin < kBand
        const uint32_t t = col0 + min(lin, last);
        const uint32_t dr = div_vpr(t, pc.vpr, pc.magic);   // rows past row0
        // 24-bit products and 32-bit byte offsets: a head row is 16 vectors,
        // so dr <= kBand / 16 <= 16, and pitches and vpr are at most 32768
        // vectors; every offset stays below 17 rows of 512 KiB
        const uint32_t col = t - __umul24(dr, pc.vpr);
        const uint32_t soff = (__umul24(dr, pc.src_pitch) + col) << 4;
        doff[k] = (__umul24(dr, pc.dst_pitch) + col) << 4;
        const uint32_t toff = (dr * 64 + 4 * lane) * 4;
#pragma unroll
        for (int tt = 0; tt < T; ++tt) xv[tt][k] = load16<true>(sb[tt] + soff);
        cv[k] = *reinterpret_cast<const f32x4 *>(cb + toff);
        sv[k] = *reinterpret_cast<const f32x4 *>(snb + toff);
    }
    // every load of the block is in flight before any arithmetic starts
    __builtin_amdgcn_sched_barrier(0);
    float ss[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const u32x4 v = xv[i / UNROLL][i % UNROLL];
        const float xf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                             bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf(xf[e], xf[e], part);
        ss[i] = group_sum<16>(part);
    }
    // lane i of each 16-lane row computes slot i's 1/sqrt(ms + eps) and DPP
    // row_newbcast:i hands it to the row (the same operations on the same
    // value, so the same bits as every lane computing its own)
    float invs[S];
    {
        float sel = ss[0];
#pragma unroll
        for (int i = 1; i < S; ++i) sel = (lane == uint32_t(i)) ? ss[i] : sel;
        const float mine = 1.0f / __builtin_sqrtf(sel * inv_d + eps);
        invs[0] = dpp<0x150>(mine);
        if constexpr (S > 1) invs[1] = dpp<0x151>(mine);
        if constexpr (S > 2) invs[2] = dpp<0x152>(mine);
        if constexpr (S > 3) invs[3] = dpp<0x153>(mine);
        if constexpr (S > 4) invs[4] = dpp<0x154>(mine);
        if constexpr (S > 5) invs[5] = dpp<0x155>(mine);
        if constexpr (S > 6) invs[6] = dpp<0x156>(mine);
        if constexpr (S > 7) invs[7] = dpp<0x157>(mine);
    }
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int tt = i / UNROLL, k = i % UNROLL;
        const u32x4 v = xv[tt][k];
        const float xf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                             bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
        const float cc[4] = {cv[k].x, cv[k].y, cv[k].z, cv[k].w};
        const float sn[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (xf[e] * invs[i]) * gm[tt][e];
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float e0 = y[2 * q] * cc[q];
            const float e1 = y[2 * q + 1] * sn[q];
            const float e2 = y[2 * q] * sn[q];
            const float e3 = y[2 * q + 1] * cc[q];
            o[q] = pack_bf16x2(e0 - e1, e2 + e3);
        }
        if (ok[k]) store16<true>(db[tt] + doff[k], u32x4{o[0], o[1], o[2], o[3]});
    }
}

uint32_t fused_band_vectors(uint32_t d) { return d == 128 ? 64 * ULY_FUSED_BAND_UNROLL : 0; }

uint32_t fused_units_per_block() { return ULY_FUSED_BLOCK * ULY_FUSED_UNROLL; }
uint32_t fused_block_threads(uint32_t d) {
    return fused_band_vectors(d) != 0 ? 64 : ULY_FUSED_BLOCK;
}

uint32_t fused_vectors_per_lane(uint32_t d) {
    const uint32_t per_row = d / 8;
    return per_row >= ULY_FUSED_VPL ? ULY_FUSED_VPL : per_row;
}

template <int VPL, int L>
static hipError_t launch_fused_l(const FusedArgs &a, uint32_t grid_x, uint32_t planes,
                                 hipStream_t stream) {
    void *argv[] = {const_cast<FusedArgs *>(&a)};
    return hipLaunchKernel(
        reinterpret_cast<const void *>(&fused_kernel<ULY_FUSED_BLOCK, ULY_FUSED_UNROLL, VPL, L>),
        dim3(grid_x, planes, 2), dim3(ULY_FUSED_BLOCK, 1, 1), argv, 0, stream);
}

template <int VPL>
static hipError_t launch_fused_vpl(const FusedArgs &a, uint32_t grid_x, uint32_t planes,
                                   hipStream_t stream) {
    switch (a.d / (8 * VPL)) {
    case 1: return launch_fused_l<VPL, 1>(a, grid_x, planes, stream);
    case 2: return launch_fused_l<VPL, 2>(a, grid_x, planes, stream);
    case 4: return launch_fused_l<VPL, 4>(a, grid_x, planes, stream);
    case 8: return launch_fused_l<VPL, 8>(a, grid_x, planes, stream);
    case 16: return launch_fused_l<VPL, 16>(a, grid_x, planes, stream);
    case 32: return launch_fused_l<VPL, 32>(a, grid_x, planes, stream);
    case 64: return launch_fused_l<VPL, 64>(a, grid_x, planes, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fused(const FusedArgs &a, uint32_t grid_x, uint32_t planes,
                        hipStream_t stream) {
    if (grid_x == 0 || planes == 0) return hipSuccess;
    void *argv[] = {const_cast<FusedArgs *>(&a)};
    if (fused_band_vectors(a.d) != 0)   // q and k in one block: grid.z = 1
        return hipLaunchKernel(
            reinterpret_cast<const void *>(&fused_band_kernel<ULY_FUSED_BAND_UNROLL>),
            dim3(grid_x, planes, 1), dim3(64, 1, 1), argv, 0, stream);
    switch (fused_vectors_per_lane(a.d)) {
    case 1: return launch_fused_vpl<1>(a, grid_x, planes, stream);
#if ULY_FUSED_VPL >= 2
    case 2: return launch_fused_vpl<2>(a, grid_x, planes, stream);
#endif
#if ULY_FUSED_VPL >= 4
    case 4: return launch_fused_vpl<4>(a, grid_x, planes, stream);
#endif
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ulysses
