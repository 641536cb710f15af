// HBM read ceilings of this device, for the attention kernels' rooflines: a
// standalone program (not part of the library).  Each wave reads whole tiles
// of S bytes (K and V tile of one block and KV head: 2 KiB int4, 4 KiB int8 /
// fp8, 8 KiB bf16 at head dim 128) at tile indices from a host-made list,
// four tiles in flight per wave, 8 waves per SIMD, from a 2 GiB buffer:
// "random" draws the indices uniformly (paged placement), "stream" takes them
// in order (a contiguous read).  Every index is checked against the tile
// count on the host.  Prints GB/s per mode and tile size.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <random>
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); exit(1); } } while (0)

template <int S>
__global__ __launch_bounds__(256) void probe(const u32x4* __restrict__ buf, const int* __restrict__ idx,
                                             int tiles_per_wave, unsigned* out) {
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * 4) + (threadIdx.x >> 6);
    const int* my = idx + static_cast<long>(wave) * tiles_per_wave;
    constexpr int PER = S / 1024;          // 1 KiB per wave instruction
    unsigned acc = 0;
    for (int t = 0; t < tiles_per_wave; t += 4) {
        u32x4 v[4][PER];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4* base = buf + static_cast<long>(my[t + u]) * (S / 16);
#pragma unroll
            for (int p = 0; p < PER; ++p) v[u][p] = base[p * 64 + lane];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int p = 0; p < PER; ++p) acc ^= v[u][p][0] ^ v[u][p][1] ^ v[u][p][2] ^ v[u][p][3];
    }
    if (acc == 0x12345678u) out[wave] = acc;     // keeps the loads alive
}

template <int S>
void run(const u32x4* buf, size_t bytes, int* d_idx, std::vector<int>& h_idx, unsigned* d_out, bool random) {
    const long n_tiles = static_cast<long>(bytes / S);
    const int waves = 256 * 4 * 8;              // 8 waves per SIMD
    const int tpw = static_cast<int>((1L << 30) / S / waves) / 4 * 4;   // ~1 GiB read per launch
    std::mt19937_64 rng(293);
    for (long i = 0; i < static_cast<long>(waves) * tpw; ++i)
        h_idx[i] = static_cast<int>(random ? rng() % n_tiles : i % n_tiles);
    for (long i = 0; i < static_cast<long>(waves) * tpw; ++i)
        if (h_idx[i] < 0 || h_idx[i] >= n_tiles) { printf("bad index\n"); exit(1); }
    CK(hipMemcpy(d_idx, h_idx.data(), sizeof(int) * waves * tpw, hipMemcpyHostToDevice));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
    for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(probe<S>, dim3(waves / 4), dim3(256), 0, 0, buf, d_idx, tpw, d_out);
    CK(hipDeviceSynchronize());
    const int reps = 10;
    CK(hipEventRecord(e0));
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(probe<S>, dim3(waves / 4), dim3(256), 0, 0, buf, d_idx, tpw, d_out);
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float ms = 0; CK(hipEventElapsedTime(&ms, e0, e1));
    const double gb = static_cast<double>(waves) * tpw * S * reps / 1e9;
    printf("%-6s tile %6d B: %8.1f GB/s (%.3f ms per launch)\n", random ? "random" : "stream", S,
           gb / (ms * 1e-3), ms / reps);
    fflush(stdout);
}

int main() {
    const size_t bytes = 2ull << 30;
    u32x4* buf; int* d_idx; unsigned* d_out;
    CK(hipMalloc(&buf, bytes));
    CK(hipMemset(buf, 1, bytes));
    const size_t max_idx = (1ull << 30) / 2048;    // tile >= 2 KiB
    CK(hipMalloc(&d_idx, sizeof(int) * max_idx));
    CK(hipMalloc(&d_out, sizeof(unsigned) * 256 * 4 * 8));
    std::vector<int> h_idx(max_idx);
    for (int random = 1; random >= 0; --random) {
        run<2048>(buf, bytes, d_idx, h_idx, d_out, random);
        run<4096>(buf, bytes, d_idx, h_idx, d_out, random);
        run<8192>(buf, bytes, d_idx, h_idx, d_out, random);
        run<16384>(buf, bytes, d_idx, h_idx, d_out, random);
    }
    CK(hipFree(buf)); CK(hipFree(d_idx)); CK(hipFree(d_out));
    return 0;
}
