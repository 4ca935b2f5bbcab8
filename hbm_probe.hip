// HBM ceilings of this GPU for the relayout's access pattern: pure read,
// pure write and contiguous copy kernels moving 16-byte vectors with
// non-temporal hints, in three launch shapes (64 x 1, 128 x 1 and 128 x 2
// threads x vectors per thread), two block orders (plain, and the library's
// two-halves order: even blocks walk the first half, odd blocks the second)
// and, for the kernels that store, two store policies (non-temporal, and
// non-temporal at device scope as the library stores), each moving
// 1,548,288,000 bytes (one
// relayout launch of the W=8, 75,600-token bf16 workload).  Measurement
// infrastructure for the benchmark: it prints one JSON line per kernel and
// shape (median of 20 timed runs after 3 warm-ups) and is not part of the
// library.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                    \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            std::printf("{\"error\": \"%s\", \"line\": %d}\n", hipGetErrorString(e_), \
                        __LINE__);                                                  \
            return 1;                                                               \
        }                                                                           \
    } while (0)

// Store policy SC1: 0 non-temporal; 1 non-temporal at device scope (written
// through the XCD's L2 at once).
template <int SC1>
__device__ __forceinline__ void store(u32x4 *p, u32x4 v) {
    if constexpr (SC1)
        // s_nop 0: the wait state a VALU write to the store's data registers
        // needs after a store of more than 8 bytes (the compiler does not see
        // this store to insert it)
        asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 0" ::"v"(p), "v"(v)
                     : "memory");
    else
        __builtin_nontemporal_store(v, p);
}

// Order H: 0 plain; 1 block x takes block x/2 (x even) or ceil(n/2) + x/2
// (x odd) of the n blocks, so the even XCDs (workgroups go to the 8 XCDs
// round robin) walk the first half and the odd XCDs the second.
template <int H>
__device__ __forceinline__ size_t block_of() {
    const uint32_t x = blockIdx.x, n = gridDim.x;
    return H ? ((x & 1) ? ((n + 1) >> 1) + (x >> 1) : (x >> 1)) : x;
}

// Block b moves vectors [B*U*b, B*U*(b+1)); lane t takes t, t + B, ...
template <int B, int U, int SC1, int H>
__global__ void __launch_bounds__(B) copy_kernel(const u32x4 *__restrict__ s,
                                                 u32x4 *__restrict__ d, size_t n) {
    const size_t i = block_of<H>() * (B * U) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k)
        if (i + k * B < n) v[k] = __builtin_nontemporal_load(s + i + k * B);
#pragma unroll
    for (int k = 0; k < U; ++k)
        if (i + k * B < n) store<SC1>(d + i + k * B, v[k]);
}

template <int B, int U, int H>
__global__ void __launch_bounds__(B) read_kernel(const u32x4 *__restrict__ s,
                                                 u32x4 *__restrict__ sink, size_t n) {
    const size_t i = block_of<H>() * (B * U) + threadIdx.x;
    u32x4 c = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < U; ++k)
        if (i + k * B < n) c ^= __builtin_nontemporal_load(s + i + k * B);
    // keeps the loads alive; the buffers never hold this pattern
    if ((c.x & c.y & c.z & c.w) == 0xDEADBEEFu) sink[threadIdx.x] = c;
}

template <int B, int U, int SC1, int H>
__global__ void __launch_bounds__(B) write_kernel(u32x4 *__restrict__ d, size_t n) {
    const size_t i = block_of<H>() * (B * U) + threadIdx.x;
    const u32x4 v = {static_cast<unsigned>(i), 1u, 2u, 3u};
#pragma unroll
    for (int k = 0; k < U; ++k)
        if (i + k * B < n) store<SC1>(d + i + k * B, v);
}

int main() {
    // The peak the runtime reports: memory clock (kHz) x bus width, two
    // transfers per clock.
    {
        hipDeviceProp_t prop;
        CHECK(hipGetDeviceProperties(&prop, 0));
        const double peak = 2.0 * double(prop.memoryClockRate) * 1e3 *
                            double(prop.memoryBusWidth) / 8.0 / 1e9;
        std::printf("{\"device_props\": {\"memory_clock_khz\": %d, \"memory_bus_bits\": %d, "
                    "\"peak_gbs\": %.1f}}\n",
                    prop.memoryClockRate, prop.memoryBusWidth, peak);
        std::fflush(stdout);
    }
    const size_t moved = 1548288000ull;
    const size_t n_all = moved / 16;   // vectors read (or written) by the one-sided kernels
    const size_t n_copy = n_all / 2;   // vectors read and written by the copy
    unsigned char *a = nullptr, *b = nullptr;
    u32x4 *sink = nullptr;
    CHECK(hipMalloc(&a, moved));
    CHECK(hipMalloc(&b, moved));
    CHECK(hipMalloc(&sink, 128 * sizeof(u32x4)));
    CHECK(hipMemset(a, 1, moved));
    CHECK(hipMemset(b, 2, moved));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    auto run = [&](const char *kind, int blk, int u, const char *st, const char *order,
                   auto launch) -> int {
        std::vector<float> t;
        for (int r = 0; r < 23; ++r) {
            CHECK(hipEventRecord(e0, 0));
            launch();
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1, 0));
            CHECK(hipEventSynchronize(e1));
            float ms = 0;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            if (r >= 3) t.push_back(ms);
        }
        std::sort(t.begin(), t.end());
        const float med = t[t.size() / 2];
        std::printf("{\"kernel\": \"%s\", \"block\": %d, \"per_thread\": %d, \"store\": \"%s\", "
                    "\"order\": \"%s\", \"bytes\": %zu, \"median_us\": %.1f, \"gbs\": %.1f}\n",
                    kind, blk, u, st, order, moved, med * 1e3, moved / (med * 1e-3) / 1e9);
        std::fflush(stdout);
        return 0;
    };
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a);
    u32x4 *dst = reinterpret_cast<u32x4 *>(b);
#define STORES(B, U, SC1, ST, H, ORD)                                                      \
    if (run("copy", B, U, ST, ORD, [&] {                                                   \
            copy_kernel<B, U, SC1, H>                                                      \
                <<<dim3(unsigned((n_copy + B * U - 1) / (B * U))), B>>>(src, dst, n_copy); \
        }))                                                                                \
        return 1;                                                                          \
    if (run("write", B, U, ST, ORD, [&] {                                                  \
            write_kernel<B, U, SC1, H>                                                     \
                <<<dim3(unsigned((n_all + B * U - 1) / (B * U))), B>>>(dst, n_all);        \
        }))                                                                                \
        return 1;
#define KINDS(B, U, H, ORD)                                                                \
    STORES(B, U, 0, "nt", H, ORD)                                                          \
    STORES(B, U, 1, "sc1 nt", H, ORD)                                                      \
    if (run("read", B, U, "-", ORD, [&] {                                                  \
            read_kernel<B, U, H>                                                           \
                <<<dim3(unsigned((n_all + B * U - 1) / (B * U))), B>>>(src, sink, n_all);  \
        }))                                                                                \
        return 1;
#define SHAPE(B, U)                                                                        \
    KINDS(B, U, 0, "plain")                                                                \
    KINDS(B, U, 1, "halves")
    SHAPE(64, 1)
    SHAPE(128, 1)
    SHAPE(128, 2)
#undef SHAPE
#undef KINDS
#undef STORES
    CHECK(hipDeviceSynchronize());
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    CHECK(hipFree(sink));
    return 0;
}
