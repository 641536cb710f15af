// Paged-read floor of this device at the decode kernel's shape: a standalone
// program (not part of the library).  It reads 77,824 tiles (the (block, KV
// head) tiles of a 64-sequence Llama-3-8B decode step) of one size, 8 KiB
// (bf16 K+V at head dim 128), 4 KiB (fp8 / int8) or 2 KiB (int4), at random
// positions of one of three 768 MiB regions taken in turn, so no launch finds
// the previous launch's tiles in the 256 MB Infinity Cache.  Like the decode
// kernel, each work-group of 4 waves takes an equal run of tiles, its waves
// take them round robin, 16 bytes per lane per load, with 1 or 2 tiles in
// flight per wave while one is consumed; the grid holds 2, 3 or 4 work-groups
// per CU (set with the dynamic LDS size).  Every index is checked against the
// region on the host.  Prints the median launch time over 30 launches and
// the rate, per tile size and configuration.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); exit(1); } } while (0)

template <int S> struct Tile { u32x4 w[S / 1024]; };   // 1 KiB per wave load

template <int S>
__device__ __forceinline__ void load_tile(Tile<S>& t, const unsigned char* buf, int id, bool valid, int lane) {
    // a zero-sized resource returns zeros without touching memory
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(buf + static_cast<long>(id) * S), 0, valid ? S : 0, 0x00020000);
#pragma unroll
    for (int s = 0; s < S / 1024; ++s)
        t.w[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 1024 * s, 0));
}

template <int S>
__device__ __forceinline__ unsigned fold(const Tile<S>& t) {
    unsigned a = 0;
#pragma unroll
    for (int s = 0; s < S / 1024; ++s) a ^= t.w[s][0] ^ t.w[s][1] ^ t.w[s][2] ^ t.w[s][3];
    return a;
}

// Work-group b reads tiles idx[b * per .. (b + 1) * per); wave w takes w, w + 4, ...
template <int S, int DEPTH>
__global__ __launch_bounds__(256) void read_tiles(const unsigned char* buf, const int* idx, int per, unsigned* out) {
    extern __shared__ int lds_pad[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int* my = idx + static_cast<long>(blockIdx.x) * per;
    const int cnt = (per - wave + 3) / 4;
    auto id = [&](int i) { return i < cnt ? my[wave + 4 * i] : 0; };
    unsigned acc = 0;
    Tile<S> ta, tb, tc;
    load_tile<S>(ta, buf, id(0), cnt > 0, lane);
    if (DEPTH == 2) load_tile<S>(tb, buf, id(1), cnt > 1, lane);
    int i = 0;
    if (DEPTH == 2) {
        for (; i + 2 < cnt; i += 3) {
            load_tile<S>(tc, buf, id(i + 2), true, lane);
            acc += fold<S>(ta);
            load_tile<S>(ta, buf, id(i + 3), i + 3 < cnt, lane);
            acc += fold<S>(tb);
            load_tile<S>(tb, buf, id(i + 4), i + 4 < cnt, lane);
            acc += fold<S>(tc);
        }
        if (i < cnt) acc += fold<S>(ta);
        if (i + 1 < cnt) acc += fold<S>(tb);
    } else {
        for (; i + 1 < cnt; i += 2) {
            load_tile<S>(tb, buf, id(i + 1), true, lane);
            acc += fold<S>(ta);
            load_tile<S>(ta, buf, id(i + 2), i + 2 < cnt, lane);
            acc += fold<S>(tb);
        }
        if (i < cnt) acc += fold<S>(ta);
    }
    if (acc == 0x12345678u) out[blockIdx.x] = acc + static_cast<unsigned>(lds_pad[0]);   // keeps the loads
}

constexpr long kRegionBytes = 768L << 20;
constexpr int kRegions = 3;
constexpr long kTiles = 77824;

template <int S>
void run(unsigned char* buf, unsigned* d_out, int wgs_per_cu, int depth, std::mt19937_64& rng) {
    const long region_tiles = kRegionBytes / S;
    const int grid = 256 * wgs_per_cu;
    const int per = static_cast<int>(kTiles / grid);
    const long n = static_cast<long>(per) * grid;
    std::vector<int*> d_idx(kRegions);
    std::vector<int> perm(region_tiles), h(n);
    for (int r = 0; r < kRegions; ++r) {
        for (long i = 0; i < region_tiles; ++i) perm[i] = static_cast<int>(i);
        std::shuffle(perm.begin(), perm.end(), rng);
        for (long i = 0; i < n; ++i) {
            h[i] = static_cast<int>(r * region_tiles + perm[i]);
            if (h[i] < 0 || h[i] >= region_tiles * kRegions) { printf("bad index\n"); exit(1); }
        }
        CK(hipMalloc(&d_idx[r], sizeof(int) * n));
        CK(hipMemcpy(d_idx[r], h.data(), sizeof(int) * n, hipMemcpyHostToDevice));
    }
    // LDS per work-group that lets exactly wgs_per_cu of them share a CU's 160 KB
    const size_t lds = wgs_per_cu == 2 ? 64 * 1024 : (wgs_per_cu == 3 ? 48 * 1024 : 36 * 1024);
    auto launch = [&](int r) {
        if (depth == 2) hipLaunchKernelGGL((read_tiles<S, 2>), dim3(grid), dim3(256), lds, 0, buf, d_idx[r], per, d_out);
        else hipLaunchKernelGGL((read_tiles<S, 1>), dim3(grid), dim3(256), lds, 0, buf, d_idx[r], per, d_out);
        CK(hipGetLastError());
    };
    for (int w = 0; w < 6; ++w) launch(w % kRegions);
    CK(hipDeviceSynchronize());
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    std::vector<float> ts;
    for (int rep = 0; rep < 30; ++rep) {
        CK(hipEventRecord(e0));
        launch(rep % kRegions);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        float ms = 0;
        CK(hipEventElapsedTime(&ms, e0, e1));
        ts.push_back(ms);
    }
    std::sort(ts.begin(), ts.end());
    const double gb = static_cast<double>(n) * S / 1e9;
    printf("tile %5d B  %6.1f MB  %d work-groups/CU  %d in flight/wave: %6.1f us (%5.0f GB/s), p10 %.1f p90 %.1f us\n",
           S, gb * 1e3, wgs_per_cu, depth, ts[15] * 1e3, gb / (ts[15] * 1e-3), ts[3] * 1e3, ts[27] * 1e3);
    fflush(stdout);
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
    for (int r = 0; r < kRegions; ++r) CK(hipFree(d_idx[r]));
}

int main() {
    unsigned char* buf;
    unsigned* d_out;
    CK(hipMalloc(&buf, kRegionBytes * kRegions));
    CK(hipMemset(buf, 1, kRegionBytes * kRegions));
    CK(hipMalloc(&d_out, sizeof(unsigned) * 1024));
    std::mt19937_64 rng(293);
    for (int wpc = 2; wpc <= 4; ++wpc)
        for (int depth = 1; depth <= 2; ++depth) {
            run<8192>(buf, d_out, wpc, depth, rng);
            run<4096>(buf, d_out, wpc, depth, rng);
            run<2048>(buf, d_out, wpc, depth, rng);
        }
    CK(hipFree(buf));
    CK(hipFree(d_out));
    return 0;
}
