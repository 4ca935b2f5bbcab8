// HBM ceilings of this GPU for the relayout's access shape: pure read, pure
// write and contiguous copy kernels with the relayout kernel's launch shape
// (128 threads, 2 x 16-byte vectors per thread, non-temporal hints), each
// moving 1,548,288,000 bytes (one relayout launch of the W=8, 75,600-token
// bf16 workload).  Measurement infrastructure for the benchmark: it prints
// one JSON line per kernel (median of 20 timed runs after 3 warm-ups) and is
// not part of the library.
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

// Block b moves vectors [256 b, 256 b + 256); lanes take i and i + 128.
__global__ void __launch_bounds__(128) copy_kernel(const u32x4 *__restrict__ s,
                                                   u32x4 *__restrict__ d, size_t n) {
    const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (i < n) a = __builtin_nontemporal_load(s + i);
    if (i + 128 < n) b = __builtin_nontemporal_load(s + i + 128);
    if (i < n) __builtin_nontemporal_store(a, d + i);
    if (i + 128 < n) __builtin_nontemporal_store(b, d + i + 128);
}

__global__ void __launch_bounds__(128) read_kernel(const u32x4 *__restrict__ s,
                                                   u32x4 *__restrict__ sink, size_t n) {
    const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (i < n) a = __builtin_nontemporal_load(s + i);
    if (i + 128 < n) b = __builtin_nontemporal_load(s + i + 128);
    const u32x4 c = a ^ b;
    // keeps the loads alive; the buffers never hold this pattern
    if ((c.x & c.y & c.z & c.w) == 0xDEADBEEFu) sink[threadIdx.x] = c;
}

__global__ void __launch_bounds__(128) write_kernel(u32x4 *__restrict__ d, size_t n) {
    const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
    const u32x4 v = {static_cast<unsigned>(i), 1u, 2u, 3u};
    if (i < n) __builtin_nontemporal_store(v, d + i);
    if (i + 128 < n) __builtin_nontemporal_store(v, d + i + 128);
}

int main() {
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
    auto blocks = [](size_t n) { return dim3(static_cast<unsigned>((n + 255) / 256)); };
    auto run = [&](const char *name, auto launch) -> int {
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
        std::printf("{\"kernel\": \"%s\", \"bytes\": %zu, \"median_us\": %.1f, \"gbs\": %.1f}\n",
                    name, moved, med * 1e3, moved / (med * 1e-3) / 1e9);
        std::fflush(stdout);
        return 0;
    };
    if (run("copy", [&] {
            copy_kernel<<<blocks(n_copy), 128>>>(reinterpret_cast<const u32x4 *>(a),
                                                 reinterpret_cast<u32x4 *>(b), n_copy);
        }))
        return 1;
    if (run("read", [&] {
            read_kernel<<<blocks(n_all), 128>>>(reinterpret_cast<const u32x4 *>(a), sink, n_all);
        }))
        return 1;
    if (run("write", [&] {
            write_kernel<<<blocks(n_all), 128>>>(reinterpret_cast<u32x4 *>(b), n_all);
        }))
        return 1;
    CHECK(hipDeviceSynchronize());
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    CHECK(hipFree(sink));
    return 0;
}
