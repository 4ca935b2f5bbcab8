// extern "C" boundary of libulysses.so (declared in include/ulysses.h).
//
// Every entry point validates everything on the host first and only then
// enqueues; a failed call has launched nothing.  No C++ exception leaves
// this file.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/ulysses.h"
#include "kernels.hpp"
#include "plan.hpp"

struct ulysses_plan {
    ulysses::Plan p;
};

namespace {

thread_local std::string g_last_error;

int set_error(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

template <typename F>
int guarded(F &&f) {
    try {
        return f();
    } catch (const std::bad_alloc &) {
        return set_error(ULYSSES_EINVAL, "host allocation failed");
    } catch (...) {
        return set_error(ULYSSES_EINVAL, "internal error");
    }
}

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
    bool written;
    std::string name;
};

// Pointer checks for one buffer: non-null, 16-byte aligned and not running
// past the top of the address space when non-empty.
int check_ptr(const void *ptr, int64_t bytes, const std::string &name) {
    if (bytes <= 0) return ULYSSES_OK;
    if (!ptr) return set_error(ULYSSES_EINVAL, name + " is null");
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
    if (lo % 16 != 0) return set_error(ULYSSES_EALIGN, name + " is not 16-byte aligned");
    if (lo + static_cast<uintptr_t>(bytes) < lo)
        return set_error(ULYSSES_EINVAL, name + " runs past the end of the address space");
    return ULYSSES_OK;
}

void add_range(std::vector<Range> *v, const void *ptr, int64_t bytes, bool written,
               const std::string &name) {
    if (bytes <= 0 || !ptr) return;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
    v->push_back(Range{lo, lo + static_cast<uintptr_t>(bytes), written, name});
}

// Every written range must be disjoint from every other range.
int check_overlap(const std::vector<Range> &v) {
    for (size_t a = 0; a < v.size(); ++a) {
        if (!v[a].written) continue;
        for (size_t b = 0; b < v.size(); ++b) {
            if (a == b) continue;
            if (v[a].lo < v[b].hi && v[b].lo < v[a].hi)
                return set_error(ULYSSES_EOVERLAP, v[a].name + " overlaps " + v[b].name);
        }
    }
    return ULYSSES_OK;
}

int launch_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ULYSSES_OK;
    return set_error(ULYSSES_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// One launch covers grid_x * block threads along x; HIP bounds that by 2^32.
// grid_x comes from a 64-bit block count and is narrowed only after this.
int check_grid(uint64_t grid_x, uint32_t block, const char *what) {
    if (grid_x > 0xFFFFFFFFull || grid_x * block > 0xFFFFFFFFull)
        return set_error(ULYSSES_EINVAL, std::string(what) +
                                             ": one batch plane is too large for one launch");
    return ULYSSES_OK;
}

// `base` moved forward by `planes` batch planes of `plane_bytes` each (an
// empty shard keeps its pointer: its planes are 0 bytes).
template <typename T>
T *plane_ptr(T *base, int64_t planes, int64_t plane_bytes) {
    return reinterpret_cast<T *>(reinterpret_cast<uintptr_t>(base) +
                                 static_cast<uintptr_t>(planes * plane_bytes));
}

// Planes per launch.  A plane that moves at least kPlaneLaunchBytes (about
// 10 us of HBM time) gets a launch of its own: the kernels' one-plane form
// has no per-lane plane arithmetic, and measured on MI355X (W=7, b=2, 1.5-6 GB
// per launch) it beats one launch over both planes by 1-2% despite the launch
// boundary.  Smaller planes share launches, up to kMaxGridY each.
constexpr int64_t kPlaneLaunchBytes = int64_t{64} << 20;

int64_t planes_per_launch(const ulysses::ModeGeom &g, int world, int tensors) {
    int64_t plane = 0;
    for (int r = 0; r < world; ++r) plane += 2 * g.dst_plane[r];
    return plane * tensors >= kPlaneLaunchBytes ? 1 : ulysses::kMaxGridY;
}

// A relayout over the plan's b batch planes, planes_per_launch() per launch,
// each launch's shards pointed at its first plane.
int launch_planes(const ulysses::Plan &p, int mode, ulysses::RelayoutArgs a, uint32_t gx,
                  int tensors, const void *const *src, void *const *dst, hipStream_t stream,
                  const char *what) {
    const ulysses::ModeGeom &g = p.mode[mode];
    const int64_t per = planes_per_launch(g, p.world, tensors);
    for (int64_t p0 = 0; p0 < p.b; p0 += per) {
        const int64_t n = p.b - p0 < per ? p.b - p0 : per;
        for (int t = 0; t < tensors; ++t)
            for (int r = 0; r < p.world; ++r) {
                a.src[t][r] = plane_ptr(static_cast<const unsigned char *>(src[t * p.world + r]),
                                        p0, g.src_plane[r]);
                a.dst[t][r] = plane_ptr(static_cast<unsigned char *>(dst[t * p.world + r]), p0,
                                        g.dst_plane[r]);
            }
        const int rc = launch_status(
            ulysses::launch_relayout(a, gx, static_cast<uint32_t>(n), static_cast<uint32_t>(tensors),
                                     stream),
            what);
        if (rc) return rc;
    }
    return ULYSSES_OK;
}

int check_plan_mode(const ulysses_plan *plan, int mode) {
    if (!plan) return set_error(ULYSSES_EINVAL, "plan is null");
    if (mode != 0 && mode != 1) return set_error(ULYSSES_EINVAL, "mode must be 0 or 1");
    return ULYSSES_OK;
}

// Checks src/dst pointer arrays of a relayout of `mode` and records ranges.
int check_shards(const ulysses::Plan &p, int mode, const void *const *src, void *const *dst,
                 const char *sname, const char *dname, std::vector<Range> *ranges) {
    if (!src || !dst) return set_error(ULYSSES_EINVAL, "pointer arrays must be non-null");
    const ulysses::ModeGeom &g = p.mode[mode];
    for (int r = 0; r < p.world; ++r) {
        const int64_t sb = p.b * g.src_plane[r];
        const int64_t db = p.b * g.dst_plane[r];
        const std::string si = std::string(sname) + "[" + std::to_string(r) + "]";
        const std::string di = std::string(dname) + "[" + std::to_string(r) + "]";
        int rc = check_ptr(src[r], sb, si);
        if (rc) return rc;
        rc = check_ptr(dst[r], db, di);
        if (rc) return rc;
        add_range(ranges, src[r], sb, false, si);
        add_range(ranges, dst[r], db, true, di);
    }
    return ULYSSES_OK;
}

// Validation and launch shared by the one-tensor and multi-tensor calls.
int relayout_tensors(const ulysses_plan *plan, int mode, int tensors, const void *const *src,
                     void *const *dst, hipStream_t stream) {
    int rc = check_plan_mode(plan, mode);
    if (rc) return rc;
    if (tensors < 1 || tensors > ulysses::kMaxTensors)
        return set_error(ULYSSES_EINVAL, "ntensors must be in [1, 4]");
    if (!src || !dst) return set_error(ULYSSES_EINVAL, "pointer arrays must be non-null");
    const ulysses::Plan &p = plan->p;
    std::vector<Range> ranges;
    for (int t = 0; t < tensors; ++t) {
        const std::string sn = tensors == 1 ? "src" : "src" + std::to_string(t);
        const std::string dn = tensors == 1 ? "dst" : "dst" + std::to_string(t);
        rc = check_shards(p, mode, src + t * p.world, dst + t * p.world, sn.c_str(), dn.c_str(),
                          &ranges);
        if (rc) return rc;
    }
    rc = check_overlap(ranges);
    if (rc) return rc;
    ulysses::RelayoutArgs a;
    const uint64_t gx = ulysses::fill_relayout(p, mode, &a);
    rc = check_grid(gx, ulysses::kRelayoutBlock, "relayout");
    if (rc) return rc;
    return launch_planes(p, mode, a, static_cast<uint32_t>(gx), tensors, src, dst, stream,
                         "relayout");
}

// The plane-at-a-time passes of a validated call: for each batch plane p,
// the relayout of plane p into the W windows and a copy of window r into
// plane p of dst r; with window == nullptr the relayout of plane p writes
// straight into plane p of the destinations (the window is the output slice).
int chunked_planes(const ulysses::Plan &p, int mode, const void *const *src, void *const *dst,
                   const void *const *window, hipStream_t stream) {
    const ulysses::ModeGeom &g = p.mode[mode];
    ulysses::RelayoutArgs to_window;
    ulysses::CopyArgs copy;
    const uint64_t gs = ulysses::fill_relayout(p, mode, &to_window);
    const uint64_t gc = ulysses::fill_plane_copy(p, mode, &copy);
    int rc = check_grid(gs > gc ? gs : gc, ulysses::kRelayoutBlock, "chunked relayout");
    if (rc) return rc;
    for (int64_t plane = 0; plane < p.b; ++plane) {
        for (int r = 0; r < p.world; ++r) {
            unsigned char *out = plane_ptr(static_cast<unsigned char *>(dst[r]), plane,
                                           g.dst_plane[r]);
            to_window.src[0][r] =
                plane_ptr(static_cast<const unsigned char *>(src[r]), plane, g.src_plane[r]);
            to_window.dst[0][r] =
                window ? static_cast<unsigned char *>(const_cast<void *>(window[r])) : out;
            if (window) {
                copy.src[r] = static_cast<const unsigned char *>(window[r]);
                copy.dst[r] = out;
            }
        }
        rc = launch_status(
            ulysses::launch_relayout(to_window, static_cast<uint32_t>(gs), 1, 1, stream),
            "plane relayout");
        if (rc) return rc;
        if (!window) continue;
        rc = launch_status(ulysses::launch_plane_copy(copy, static_cast<uint32_t>(gc), stream),
                           "window copy");
        if (rc) return rc;
    }
    return ULYSSES_OK;
}

}  // namespace

extern "C" {

int ulysses_plan_create(ulysses_plan **out, int world, int64_t b, int64_t d,
                        const int64_t *seq_splits, const int64_t *head_splits, int dtype,
                        int64_t window_cap_bytes) {
    return guarded([&]() -> int {
        if (!out) return set_error(ULYSSES_EINVAL, "out is null");
        *out = nullptr;
        auto *plan = new ulysses_plan;
        std::string msg;
        const int rc = ulysses::plan_build(&plan->p, world, b, d, seq_splits, head_splits,
                                           dtype, window_cap_bytes, &msg);
        if (rc != ULYSSES_OK) {
            delete plan;
            return set_error(rc, msg);
        }
        *out = plan;
        return ULYSSES_OK;
    });
}

void ulysses_plan_destroy(ulysses_plan *plan) { delete plan; }

int ulysses_plan_shape(const ulysses_plan *plan, int mode, int rank, int is_dst,
                       int64_t shape[4]) {
    return guarded([&]() -> int {
        int rc = check_plan_mode(plan, mode);
        if (rc) return rc;
        if (!shape) return set_error(ULYSSES_EINVAL, "shape is null");
        if (rank < 0 || rank >= plan->p.world)
            return set_error(ULYSSES_EINVAL, "rank out of range");
        const ulysses::ModeGeom &g = plan->p.mode[mode];
        std::memcpy(shape, is_dst ? g.dst_shape[rank] : g.src_shape[rank], 4 * sizeof(int64_t));
        return ULYSSES_OK;
    });
}

int64_t ulysses_plan_window_bytes(const ulysses_plan *plan, int mode) {
    int64_t v = 0;
    const int rc = guarded([&]() -> int {
        int r = check_plan_mode(plan, mode);
        if (r) return r;
        v = plan->p.mode[mode].window_bytes;
        return ULYSSES_OK;
    });
    return rc ? rc : v;
}

int64_t ulysses_plan_bytes(const ulysses_plan *plan, int mode) {
    int64_t v = 0;
    const int rc = guarded([&]() -> int {
        int r = check_plan_mode(plan, mode);
        if (r) return r;
        const ulysses::Plan &p = plan->p;
        v = 2 * p.b * p.s_global * p.n_global * p.d * p.esz;
        return ULYSSES_OK;
    });
    return rc ? rc : v;
}

int ulysses_a2a_4d(const ulysses_plan *plan, int mode, const void *const *src,
                   void *const *dst, hipStream_t stream) {
    return guarded([&]() -> int { return relayout_tensors(plan, mode, 1, src, dst, stream); });
}

int ulysses_a2a_4d_multi(const ulysses_plan *plan, int mode, int ntensors,
                         const void *const *src, void *const *dst, hipStream_t stream) {
    return guarded(
        [&]() -> int { return relayout_tensors(plan, mode, ntensors, src, dst, stream); });
}

int ulysses_a2a_4d_chunked(const ulysses_plan *plan, int mode, const void *const *src,
                           void *const *dst, void *const *window, hipStream_t stream) {
    return guarded([&]() -> int {
        int rc = check_plan_mode(plan, mode);
        if (rc) return rc;
        const ulysses::Plan &p = plan->p;
        if (p.window_cap <= 0)
            return set_error(ULYSSES_EINVAL, "the plan has no window cap (window_cap_bytes = 0)");
        const int64_t wb = p.mode[mode].window_bytes;
        if (wb > p.window_cap)
            return set_error(ULYSSES_EWINDOW, "window bytes per rank per plane " +
                                                  std::to_string(wb) + " exceed the cap " +
                                                  std::to_string(p.window_cap));
        std::vector<Range> ranges;
        rc = check_shards(p, mode, src, dst, "src", "dst", &ranges);
        if (rc) return rc;
        if (window) {
            for (int r = 0; r < p.world; ++r) {
                const std::string wi = "window[" + std::to_string(r) + "]";
                const int64_t need = p.mode[mode].dst_plane[r];
                rc = check_ptr(window[r], need, wi);
                if (rc) return rc;
                add_range(&ranges, window[r], need, true, wi);
            }
        }
        rc = check_overlap(ranges);
        if (rc) return rc;
        return chunked_planes(p, mode, src, dst, window, stream);
    });
}

int ulysses_a2a_4d_chunked_static(const ulysses_plan *plan, int mode, const void *const *src,
                                  void *const *dst, hipStream_t stream) {
    return guarded([&]() -> int {
        int rc = check_plan_mode(plan, mode);
        if (rc) return rc;
        const ulysses::Plan &p = plan->p;
        if (p.window_cap <= 0)
            return set_error(ULYSSES_EINVAL, "the plan has no window cap (window_cap_bytes = 0)");
        const int64_t wb = p.mode[mode].window_bytes;
        if (wb > p.window_cap)
            return set_error(ULYSSES_EWINDOW, "window bytes per rank per plane " +
                                                  std::to_string(wb) + " exceed the cap " +
                                                  std::to_string(p.window_cap));
        // the W windows, each rounded up to the array's alignment, must fit
        const uint64_t align = ulysses::kStaticWindowAlign;
        const uint64_t slot = (static_cast<uint64_t>(wb) + align - 1) / align * align;
        if (slot * static_cast<uint64_t>(p.world) > ulysses::kStaticWindowBytes)
            return set_error(ULYSSES_EWINDOW,
                             std::to_string(p.world) + " windows of " + std::to_string(wb) +
                                 " bytes exceed the static window array of " +
                                 std::to_string(ulysses::kStaticWindowBytes) + " bytes");
        std::vector<Range> ranges;
        rc = check_shards(p, mode, src, dst, "src", "dst", &ranges);
        if (rc) return rc;
        unsigned char *base = nullptr;
        rc = launch_status(ulysses::static_windows(stream, &base), "static windows");
        if (rc) return rc;
        add_range(&ranges, base, static_cast<int64_t>(ulysses::kStaticWindowBytes), true,
                  "the static windows");
        rc = check_overlap(ranges);
        if (rc) return rc;
        const void *window[ulysses::kMaxWorld];
        for (int r = 0; r < p.world; ++r) window[r] = base + slot * static_cast<uint64_t>(r);
        return chunked_planes(p, mode, src, dst, window, stream);
    });
}

int ulysses_a2a_4d_qknorm_rope(const ulysses_plan *plan, const void *const *q_src,
                               void *const *q_dst, const void *const *k_src,
                               void *const *k_dst, const float *gamma_q, const float *gamma_k,
                               float eps, const float *rope_cos, const float *rope_sin,
                               hipStream_t stream) {
    return guarded([&]() -> int {
        int rc = check_plan_mode(plan, 0);
        if (rc) return rc;
        const ulysses::Plan &p = plan->p;
        if (p.dtype != ULYSSES_BF16)
            return set_error(ULYSSES_EDTYPE, "the fused QK-norm + RoPE path takes bf16 only");
        const int64_t lanes = p.d / 8;
        if (p.d % 8 != 0 || lanes < 1 || lanes > 64 || (lanes & (lanes - 1)) != 0)
            return set_error(ULYSSES_EINVAL, "the fused path needs d/8 a power of two in [1, 64]");
        if (!(eps >= 0.0f) || !std::isfinite(eps))
            return set_error(ULYSSES_EINVAL, "eps must be finite and >= 0");
        std::vector<Range> ranges;
        rc = check_shards(p, 0, q_src, q_dst, "q_src", "q_dst", &ranges);
        if (rc) return rc;
        rc = check_shards(p, 0, k_src, k_dst, "k_src", "k_dst", &ranges);
        if (rc) return rc;
        const int64_t gbytes = p.d * 4;
        const int64_t tbytes = p.s_global * (p.d / 2) * 4;
        const struct { const void *ptr; int64_t bytes; const char *name; } params[] = {
            {gamma_q, gbytes, "gamma_q"}, {gamma_k, gbytes, "gamma_k"},
            {rope_cos, tbytes, "rope_cos"}, {rope_sin, tbytes, "rope_sin"}};
        for (const auto &q : params) {
            rc = check_ptr(q.ptr, q.bytes, q.name);
            if (rc) return rc;
            add_range(&ranges, q.ptr, q.bytes, false, q.name);
        }
        rc = check_overlap(ranges);
        if (rc) return rc;

        ulysses::FusedArgs a;
        const uint64_t gx = ulysses::fill_fused(p, &a);
        rc = check_grid(gx, ulysses::kFusedBlock, "fused relayout");
        if (rc) return rc;
        a.gamma[0] = gamma_q;
        a.gamma[1] = gamma_k;
        a.rope_cos = rope_cos;
        a.rope_sin = rope_sin;
        a.eps = eps;
        const ulysses::ModeGeom &g = p.mode[0];
        const int64_t per = planes_per_launch(g, p.world, 2);
        for (int64_t p0 = 0; p0 < p.b; p0 += per) {
            const int64_t n = p.b - p0 < per ? p.b - p0 : per;
            for (int r = 0; r < p.world; ++r) {
                a.src[0][r] =
                    plane_ptr(static_cast<const unsigned char *>(q_src[r]), p0, g.src_plane[r]);
                a.dst[0][r] = plane_ptr(static_cast<unsigned char *>(q_dst[r]), p0, g.dst_plane[r]);
                a.src[1][r] =
                    plane_ptr(static_cast<const unsigned char *>(k_src[r]), p0, g.src_plane[r]);
                a.dst[1][r] = plane_ptr(static_cast<unsigned char *>(k_dst[r]), p0, g.dst_plane[r]);
            }
            rc = launch_status(ulysses::launch_fused(a, static_cast<uint32_t>(p.d),
                                                     static_cast<uint32_t>(gx),
                                                     static_cast<uint32_t>(n), stream),
                               "fused relayout");
            if (rc) return rc;
        }
        return ULYSSES_OK;
    });
}

int ulysses_rope_table(double theta, int64_t s_global, int64_t d, float *cos_out,
                       float *sin_out) {
    return guarded([&]() -> int {
        if (!(theta > 0.0) || !std::isfinite(theta))
            return set_error(ULYSSES_EINVAL, "theta must be finite and > 0");
        if (s_global < 0 || d < 2 || d % 2 != 0)
            return set_error(ULYSSES_EINVAL, "need s_global >= 0 and an even d >= 2");
        if (s_global > 0 && (!cos_out || !sin_out))
            return set_error(ULYSSES_EINVAL, "output tables are null");
        const int64_t half = d / 2;
        // frequencies once per pair, then one double-precision angle per entry
        std::vector<double> w(static_cast<size_t>(half));
        for (int64_t i = 0; i < half; ++i)
            w[static_cast<size_t>(i)] =
                std::pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(d));
        for (int64_t s = 0; s < s_global; ++s) {
            float *cr = cos_out + s * half;
            float *sr = sin_out + s * half;
            for (int64_t i = 0; i < half; ++i) {
                const double ang = static_cast<double>(s) * w[static_cast<size_t>(i)];
                cr[i] = static_cast<float>(std::cos(ang));
                sr[i] = static_cast<float>(std::sin(ang));
            }
        }
        return ULYSSES_OK;
    });
}

const char *ulysses_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
