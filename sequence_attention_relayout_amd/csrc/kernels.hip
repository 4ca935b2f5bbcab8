// gfx950 (CDNA4) kernels of the Ulysses 4D relayout.
//
// The relayout is pure data movement: every byte is read once and written
// once, so HBM bandwidth bounds it and there is no contraction for MFMA.
// Every (source rank j -> destination rank r) piece is a set of rows that are
// contiguous on both sides (d * elem_size >= 16 bytes, in practice 128 B and
// up), so each lane moves whole 16-byte vectors and no LDS staging is needed:
// the source and destination strides agree at 16-byte granularity.  The
// permutation itself is only addressing, as the pages put it (fast-ulysses
// 0.1.0 introduction: the sequence/head relayout is expressed as copy
// strides instead of separate permute kernels).
//
// Both passes walk the destination shards in address order, 64 consecutive
// 16-byte vectors per wave (each load or store instruction of a wave covers
// 1 KiB), and find for each lane the source rank that owns its vector (a
// gather): every store of a wave is one contiguous KiB, and each lane reads
// from the piece that owns its destination row (mode 0, and the fused pass)
// or column (mode 1).  Measured on MI355X, walking the destinations beats
// walking the sources (a scatter) and the earlier per-piece band walk, for
// the relayout in both modes and for the fused pass.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace ulysses {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Non-temporal 16-byte loads and stores through the global address space:
// each byte is touched once, so streaming hints keep the caches for the
// index tables and rotary rows (+5-10% measured over plain accesses), and
// global (not flat) instructions leave the scalar loads' counter alone.
// Stores also carry device scope (sc1), so each line is written through the
// XCD's L2 at once instead of staying dirty there until evicted: measured on
// MI355X, 0.4-1.4% faster on every relayout geometry and dtype, and on the
// fused pass, than non-temporal stores alone (load scope bits change nothing).
typedef __attribute__((address_space(1))) const u32x4 global_cu32x4;

__device__ __forceinline__ u32x4 load16(uint64_t addr) {
    return __builtin_nontemporal_load(reinterpret_cast<global_cu32x4 *>(addr));
}

// A vector-memory store (global_store_dwordx4) the compiler does not see.
// Two things it would otherwise take care of:
//  - a VALU write to the data registers of a store of more than 8 bytes needs
//    one wait state after the store (gfx9 hazard); the s_nop 0 gives it;
//  - on gfx950 stores and loads share one in-order counter, so any wait the
//    compiler places after the store only waits longer, never too little.
__device__ __forceinline__ void store16(uint64_t addr, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 0" ::"v"(addr), "v"(v)
                 : "memory");
}

// Cached 16-byte loads through the global address space (the rotary rows
// and the gains, which many waves read).
typedef __attribute__((address_space(1))) const f32x4 global_cf32x4;

__device__ __forceinline__ f32x4 loadf4(uint64_t addr) {
    return *reinterpret_cast<global_cf32x4 *>(addr);
}

__device__ __forceinline__ uint64_t addr_of(const unsigned char *p) {
    return reinterpret_cast<uint64_t>(p);
}

// Index of the last entry of a kMaxWorld-entry ascending table that is <= x
// (entries past the world hold kNone).
__device__ __forceinline__ uint32_t find_group(const uint32_t *begin, uint32_t x) {
    uint32_t g = 0;
#pragma unroll
    for (int q = 1; q < kMaxWorld; ++q) g += (begin[q] <= x) ? 1u : 0u;
    return g;
}

// Launch order of the blocks: block x takes block halves(x, n) of the
// launch's n, so even blocks walk the first half of the destination vectors
// and odd blocks the second half (a bijection of [0, n)).  Workgroups go to
// the 8 XCDs round robin, so the even XCDs stream through one half and the
// odd XCDs through the other.  Measured on MI355X, a plain copy split this
// way runs 0.5-1.6% faster than one stream at every distance between the
// halves tried (256 MiB to 1.8 GiB), while alternating in groups of 8 or 64
// blocks, where every XCD sees both halves, does not.  Four parts gain less
// than two, and eight (one range per XCD) lose to the plain order.
__device__ __forceinline__ uint32_t halves(uint32_t x, uint32_t n) {
    return (x & 1) ? ((n + 1) >> 1) + (x >> 1) : (x >> 1);
}

// Row and column of vector s0 + lane of a shard whose rows hold rs.vpr
// vectors; s0 is uniform and lane < 2^16 - rs.vpr.
struct RowCol {
    uint32_t row, col;
};

__device__ __forceinline__ RowCol split_rows(const RowSplit &rs, uint32_t s0, uint32_t lane) {
    const uint32_t row0 = div32(s0, rs.m, rs.s1, rs.s2);
    const uint32_t t = s0 - row0 * rs.vpr + lane;   // < rs.vpr + lane < 2^16
    const uint32_t dr = rs.vpr == 1 ? t : __umulhi(t, rs.magic);
    return RowCol{row0 + dr, t - dr * rs.vpr};
}

// --------------------------------------------------------------------------
// Relayout (modes 0 and 1, and the window pass of the plane-at-a-time mode)
// --------------------------------------------------------------------------

// Each wave moves 1 KiB, so what a wave does before its load issues bounds
// the bytes in flight: every block-uniform value is read once up front and
// the per-rank choice is a select, with no branch.  A launch of one batch
// plane (PLANES false) has no plane arithmetic at all, the caller having
// pointed the shards at that plane; a launch of several adds one multiply
// per lane on the selected rank's plane size.  Measured on MI355X, each
// scalar 64-bit product or branch taken out of that path moved the pass by
// about a percent.
// HALVES (mode 0) runs the blocks in halves() order, where the two halves
// read different column slices of the same source rows at the same time.
// Measured on MI355X in mode 0: 1.0-1.3% faster at W=8 for 640- to
// 1,536-byte destination rows (fp8, bf16 with d = 64 and 128, unequal
// heads), 3% for 2,560-byte fp32 rows, 1% at W=7 in fp32, even in bf16 at
// W=7, and 0.1-0.75% slower at W=7 in fp8.  In mode 1 the same order reads
// twice the source regions at once and lost 1-3%, so mode 1 keeps the plain
// order.
template <bool PLANES, bool HALVES>
__global__ void __launch_bounds__(kRelayoutBlock) relayout_kernel(const RelayoutArgs a) {
    const uint32_t x = HALVES ? halves(blockIdx.x, gridDim.x) : blockIdx.x;
    const uint32_t r = find_group(a.blk_begin, x);
    const uint32_t s0 = (x - a.blk_begin[r]) * kRelayoutBlock;
    const uint32_t t = blockIdx.z;
    // every source rank's piece origin in this destination's frame
    uint64_t base[kMaxWorld];
    uint32_t pitch[kMaxWorld], bound[kMaxWorld], splane[kMaxWorld];
#pragma unroll
    for (int q = 0; q < kMaxWorld; ++q) {
        base[q] = addr_of(a.src[t][q]) + (static_cast<uint64_t>(a.off[r][q]) << 4);
        pitch[q] = a.pitch[r][q];
        bound[q] = a.bound[q];
        if constexpr (PLANES) splane[q] = static_cast<uint32_t>(a.src_plane[q]);
    }
    const RowCol rc = split_rows(a.row[r], s0, threadIdx.x);
    // the source rank owning this destination vector, and its piece
    const uint32_t key = a.key_col ? rc.col : rc.row;
    uint64_t b = base[0];
    uint32_t pt = pitch[0], pl = 0;
    if constexpr (PLANES) pl = splane[0];
#pragma unroll
    for (int q = 1; q < kMaxWorld; ++q) {
        const bool c = bound[q] <= key;
        b = c ? base[q] : b;
        pt = c ? pitch[q] : pt;
        if constexpr (PLANES) pl = c ? splane[q] : pl;
    }
    const uint32_t v = s0 + threadIdx.x;
    if (v < a.nvec[r]) {
        uint64_t so = uint64_t(rc.row) * pt + rc.col;
        uint64_t dv = v;
        if constexpr (PLANES) {
            so += uint64_t(blockIdx.y) * pl;
            dv += uint64_t(blockIdx.y) * a.dst_plane[r];
        }
        store16(addr_of(a.dst[t][r]) + (dv << 4), load16(b + (so << 4)));
    }
}

hipError_t launch_relayout(const RelayoutArgs &a, uint32_t grid_x, uint32_t planes,
                           uint32_t tensors, hipStream_t stream) {
    if (grid_x == 0 || planes == 0 || tensors == 0) return hipSuccess;
    void *argv[] = {const_cast<RelayoutArgs *>(&a)};
    const bool h = a.key_col == 0;   // mode 0
    const void *fn =
        planes > 1 ? (h ? reinterpret_cast<const void *>(&relayout_kernel<true, true>)
                        : reinterpret_cast<const void *>(&relayout_kernel<true, false>))
                   : (h ? reinterpret_cast<const void *>(&relayout_kernel<false, true>)
                        : reinterpret_cast<const void *>(&relayout_kernel<false, false>));
    return hipLaunchKernel(fn, dim3(grid_x, planes, tensors), dim3(kRelayoutBlock, 1, 1), argv, 0,
                           stream);
}

// One batch plane per rank, window -> destination plane, contiguous, in
// halves() order (a plain copy is the case that order was measured on).
__global__ void __launch_bounds__(kRelayoutBlock) plane_copy_kernel(const CopyArgs a) {
    const uint32_t x = halves(blockIdx.x, gridDim.x);
    const uint32_t r = find_group(a.blk_begin, x);
    const uint32_t v = (x - a.blk_begin[r]) * kRelayoutBlock + threadIdx.x;
    if (v < a.nvec[r])
        store16(addr_of(a.dst[r]) + (uint64_t(v) << 4), load16(addr_of(a.src[r]) + (uint64_t(v) << 4)));
}

// The windows of the plane-at-a-time call for callers that cannot allocate.
// In host code `scratch` only stands in for the symbol: its device address
// on a GPU comes from hipGetSymbolAddress with that GPU current, once per
// device, and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[kStaticWindowBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t static_windows(hipStream_t stream, unsigned char **ptr) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = static_cast<unsigned char *>(g_scratch[dev]);
    return hipSuccess;
}

hipError_t launch_plane_copy(const CopyArgs &a, uint32_t grid_x, hipStream_t stream) {
    if (grid_x == 0) return hipSuccess;
    void *argv[] = {const_cast<CopyArgs *>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&plane_copy_kernel), dim3(grid_x, 1, 1),
                           dim3(kRelayoutBlock, 1, 1), argv, 0, stream);
}

// --------------------------------------------------------------------------
// Fused mode 0 with QK RMSNorm + RoPE (bf16 in, bf16 out, fp32 arithmetic)
// --------------------------------------------------------------------------
//
// The pass is the mode-0 gather of the relayout with the arithmetic on the
// way: each lane takes one destination vector of q and the same one of k,
// reads both from the source rank that owns the row's sequence position, and
// stores them normalised and rotated, so every store of a wave is one
// contiguous KiB.  Measured on MI355X it beats walking the sources (a
// scatter) by 3-6%.  With the arithmetic and the tables taken out, the data
// movement alone runs only 2-6% faster: moving two tensors per lane is what
// bounds the pass, and layouts with one tensor per lane or per block, or
// with more concurrent streams, measured slower.
//
// A head row of d bf16 elements is L = d/8 16-byte vectors held by L
// consecutive lanes: lane l of the row holds elements 8l .. 8l+7 and rotary
// pairs 4l .. 4l+3.  Blocks start on multiples of kFusedBlock and rows are
// whole head rows, so a lane's place within its head row is threadIdx % L.
// The operation order is fixed so the result is reproducible bit for bit:
//   partial p_l, one per lane: fused multiply-add chain over its 8 squares,
//        ascending;
//   ss = pairwise tree over p_0 .. p_{L-1} with adjacent pairing, as an xor
//        butterfly over the L lanes (every lane ends with the same bits, fp32
//        + being commutative);
//   ms = ss * (1/d), which equals ss / d exactly since d is a power of two;
//   inv = 1 / sqrt(ms + eps), correctly rounded sqrt and division;
//   y = (x * inv) * gamma;  rotation products rounded one by one.
// The library is compiled with -ffp-contract=off so no product is fused.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two floats to bf16 (nearest even, gfx950's v_cvt_pk_bf16_f32) and
// pack them, lo in bits 0..15.
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

__device__ __forceinline__ void widen(u32x4 v, float xf[8]) {
    xf[0] = bf16_lo(v.x); xf[1] = bf16_hi(v.x);
    xf[2] = bf16_lo(v.y); xf[3] = bf16_hi(v.y);
    xf[4] = bf16_lo(v.z); xf[5] = bf16_hi(v.z);
    xf[6] = bf16_lo(v.w); xf[7] = bf16_hi(v.w);
}

template <int L, bool PLANES>
__global__ void __launch_bounds__(kFusedBlock) fused_kernel(const FusedArgs a) {
    // halves() order: measured on MI355X 0.3-2.5% faster than the plain
    // order on every geometry tried
    const uint32_t x = halves(blockIdx.x, gridDim.x);
    const uint32_t r = find_group(a.blk_begin, x);
    const uint32_t s0 = (x - a.blk_begin[r]) * kFusedBlock;
    const uint32_t last = a.nvec[r] - 1;
    const uint32_t tid = threadIdx.x;
    // lanes past the shard redo its last vector and store nothing; valid
    // lanes come in whole L-lane head rows (s0 and the shard are multiples)
    const bool ok = s0 + tid <= last;
    const uint32_t lt = min(s0 + tid, last) - s0;
    const uint32_t lane = tid & (L - 1);
    // rc.row: the sequence position
    const RowCol rc = split_rows(a.row[r], s0, lt);
    // a launch of one batch plane has no plane terms (the caller points
    // the shards at it)
    const uint64_t plane = PLANES ? blockIdx.y : 0;
    // the source rank owning this sequence position, and its piece
    uint64_t bq = 0, bk = 0;
#pragma unroll
    for (int q = 0; q < kMaxWorld; ++q) {
        uint64_t o = static_cast<uint64_t>(a.off[r][q]);
        if constexpr (PLANES) o += plane * a.src_plane[q];
        const bool c = q == 0 || a.bound[q] <= rc.row;
        bq = c ? addr_of(a.src[0][q]) + (o << 4) : bq;
        bk = c ? addr_of(a.src[1][q]) + (o << 4) : bk;
    }
    const uint64_t so = (uint64_t(rc.row) * a.pitch + rc.col) << 4;
    const u32x4 xq = load16(bq + so);
    const u32x4 xk = load16(bk + so);
    // rotary row of the sequence position
    const uint64_t to = (uint64_t(rc.row) * a.half_d + 4 * lane) * 4;
    const f32x4 cv = loadf4(reinterpret_cast<uint64_t>(a.rope_cos) + to);
    const f32x4 sv = loadf4(reinterpret_cast<uint64_t>(a.rope_sin) + to);
    f32x4 gv[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint64_t gp = reinterpret_cast<uint64_t>(a.gamma[t]) + 32 * lane;
        gv[t][0] = loadf4(gp);
        gv[t][1] = loadf4(gp + 16);
    }
    // every load of the block is in flight before any arithmetic starts
    __builtin_amdgcn_sched_barrier(0);

    const u32x4 xv[2] = {xq, xk};
    float ss[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float xf[8];
        widen(xv[t], xf);
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf(xf[e], xf[e], part);
        ss[t] = group_sum<L>(part);
    }
    // '/' and __builtin_sqrtf lower to the IEEE-exact sequences under hipcc's
    // default correctly rounded fp32 divide and sqrt (div_scale/div_fmas/
    // div_fixup; v_sqrt_f32 plus a one-ulp residual correction).
    float inv[2];
    if constexpr (L >= 16) {
        // every lane of a 16-lane DPP row holds the same ss of q and of k:
        // lane 0 of the row computes q's 1/sqrt, lane 1 k's, and DPP
        // row_newbcast hands them to the row (the same operations on the
        // same value, so the same bits as every lane computing its own)
        const float sel = (tid & 15) == 1 ? ss[1] : ss[0];
        const float mine = 1.0f / __builtin_sqrtf(sel * a.inv_d + a.eps);
        inv[0] = dpp<0x150>(mine);
        inv[1] = dpp<0x151>(mine);
    } else {
        inv[0] = 1.0f / __builtin_sqrtf(ss[0] * a.inv_d + a.eps);
        inv[1] = 1.0f / __builtin_sqrtf(ss[1] * a.inv_d + a.eps);
    }
    const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
    const float sn[4] = {sv.x, sv.y, sv.z, sv.w};
    const uint64_t dv = ((PLANES ? plane * a.dst_plane[r] : 0) + s0 + lt) << 4;
    // q is stored as soon as it is ready: measured on MI355X, 2-4% faster
    // than storing q and k together at the end
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float xf[8];
        widen(xv[t], xf);
        const float g[8] = {gv[t][0].x, gv[t][0].y, gv[t][0].z, gv[t][0].w,
                            gv[t][1].x, gv[t][1].y, gv[t][1].z, gv[t][1].w};
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (xf[e] * inv[t]) * g[e];
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float e0 = y[2 * q] * cc[q];
            const float e1 = y[2 * q + 1] * sn[q];
            const float e2 = y[2 * q] * sn[q];
            const float e3 = y[2 * q + 1] * cc[q];
            o[q] = pack_bf16x2(e0 - e1, e2 + e3);
        }
        if (ok) store16(addr_of(a.dst[t][r]) + dv, u32x4{o[0], o[1], o[2], o[3]});
    }
}

template <int L>
static hipError_t launch_fused_l(const FusedArgs &a, uint32_t grid_x, uint32_t planes,
                                 hipStream_t stream) {
    void *argv[] = {const_cast<FusedArgs *>(&a)};
    const void *fn = planes > 1 ? reinterpret_cast<const void *>(&fused_kernel<L, true>)
                                : reinterpret_cast<const void *>(&fused_kernel<L, false>);
    return hipLaunchKernel(fn, dim3(grid_x, planes, 1), dim3(kFusedBlock, 1, 1), argv, 0, stream);
}

hipError_t launch_fused(const FusedArgs &a, uint32_t d, uint32_t grid_x, uint32_t planes,
                        hipStream_t stream) {
    if (grid_x == 0 || planes == 0) return hipSuccess;
    switch (d / 8) {
    case 1: return launch_fused_l<1>(a, grid_x, planes, stream);
    case 2: return launch_fused_l<2>(a, grid_x, planes, stream);
    case 4: return launch_fused_l<4>(a, grid_x, planes, stream);
    case 8: return launch_fused_l<8>(a, grid_x, planes, stream);
    case 16: return launch_fused_l<16>(a, grid_x, planes, stream);
    case 32: return launch_fused_l<32>(a, grid_x, planes, stream);
    case 64: return launch_fused_l<64>(a, grid_x, planes, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ulysses
