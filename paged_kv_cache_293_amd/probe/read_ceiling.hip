// HBM read ceiling of this device: a standalone program (not part of the
// library).  Each launch reads one whole 768 MiB region once, in 8 KiB
// pieces (16 bytes per lane per load, 1 KiB per wave load), in one of three
// orders:
//   stream  : pieces in address order (the region read front to back);
//   random8 : a random permutation of the pieces (each read once);
//   random64: a random permutation of 64 KiB blocks, each block's 8 pieces
//             in order (the pool's (block, 8 KV heads) runs at bf16 d 128).
// Piece p of the list is read by wave p mod W of the grid (W waves in all),
// so at any moment adjacent list entries are read by waves running side by
// side.  Three regions are read in turn, so no launch finds the previous
// one's bytes in the 256 MB Infinity Cache.  Grids of 2 work-groups per CU
// (three pieces per wave, two in flight while one is consumed) and 8 per CU
// (one piece per wave at a time); a work-group is one wave on each SIMD.
// The 2 per CU grid also runs with the loads' cache-policy bits set:
// non-temporal (2), sc0 (1), sc0 + non-temporal (3), sc0 + sc1 (17).
// Every piece index is checked against the region on the host.  Prints the
// median launch time over 30 launches and the rate.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); exit(1); } } while (0)

constexpr int kPiece = 8192;
constexpr long kRegionBytes = 768L << 20;
constexpr int kRegions = 3;
constexpr int kPieces = static_cast<int>(kRegionBytes / kPiece);

struct Piece { u32x4 w[kPiece / 1024]; };

// POL: the load's cache-policy bits (0 default; 2 non-temporal; 1, 3, 17, 19
// with the coherence bits sc0 (1) and sc1 (16)).
template <int POL>
__device__ __forceinline__ void load_piece(Piece& t, const unsigned char* region, int piece, bool valid, int lane) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(region + static_cast<long>(piece) * kPiece), 0, valid ? kPiece : 0, 0x00020000);
#pragma unroll
    for (int s = 0; s < kPiece / 1024; ++s)
        t.w[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 1024 * s, POL));
}

__device__ __forceinline__ unsigned fold(const Piece& t) {
    unsigned a = 0;
#pragma unroll
    for (int s = 0; s < kPiece / 1024; ++s) a ^= t.w[s][0] ^ t.w[s][1] ^ t.w[s][2] ^ t.w[s][3];
    return a;
}

// Wave g reads list[g], list[g + W], ...  (cnt of them).
template <int DEPTH, int POL>
__global__ __launch_bounds__(256) void read_region(const unsigned char* region, const int* list, int n, unsigned* out) {
    const int lane = threadIdx.x & 63;
    const int W = static_cast<int>(gridDim.x) * 4;
    const int g = static_cast<int>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int cnt = g < n ? (n - g + W - 1) / W : 0;
    auto id = [&](int i) { return i < cnt ? list[g + i * W] : 0; };
    unsigned acc = 0;
    if constexpr (DEPTH == 2) {
        Piece ta, tb, tc;
        load_piece<POL>(ta, region, id(0), cnt > 0, lane);
        load_piece<POL>(tb, region, id(1), cnt > 1, lane);
        int i = 0;
        for (; i + 2 < cnt; i += 3) {
            load_piece<POL>(tc, region, id(i + 2), true, lane);
            acc += fold(ta);
            load_piece<POL>(ta, region, id(i + 3), i + 3 < cnt, lane);
            acc += fold(tb);
            load_piece<POL>(tb, region, id(i + 4), i + 4 < cnt, lane);
            acc += fold(tc);
        }
        if (i < cnt) acc += fold(ta);
        if (i + 1 < cnt) acc += fold(tb);
    } else {
        for (int i = 0; i < cnt; ++i) {
            Piece t;
            load_piece<POL>(t, region, id(i), true, lane);
            acc += fold(t);
        }
    }
    if (acc == 0x12345678u) out[blockIdx.x] = acc;   // keeps the loads
}

int main() {
    unsigned char* buf;
    unsigned* d_out;
    int* d_list;
    CK(hipMalloc(&buf, kRegionBytes * kRegions));
    CK(hipMemset(buf, 1, kRegionBytes * kRegions));
    CK(hipMalloc(&d_out, sizeof(unsigned) * 256 * 8));
    CK(hipMalloc(&d_list, sizeof(int) * kPieces));
    std::mt19937_64 rng(293);
    const char* names[3] = {"stream", "random8", "random64"};
    for (int pol : {0, 2, 1, 3, 17}) {
    for (int mode = 0; mode < 3; ++mode) {
        std::vector<int> list(kPieces);
        if (mode == 0) {
            for (int i = 0; i < kPieces; ++i) list[i] = i;
        } else if (mode == 1) {
            for (int i = 0; i < kPieces; ++i) list[i] = i;
            std::shuffle(list.begin(), list.end(), rng);
        } else {
            std::vector<int> blocks(kPieces / 8);
            for (int i = 0; i < kPieces / 8; ++i) blocks[i] = i;
            std::shuffle(blocks.begin(), blocks.end(), rng);
            for (int i = 0; i < kPieces; ++i) list[i] = blocks[i / 8] * 8 + i % 8;
        }
        std::vector<char> seen(kPieces, 0);
        for (int x : list) {
            if (x < 0 || x >= kPieces || seen[x]) { printf("bad piece list\n"); exit(1); }
            seen[x] = 1;
        }
        CK(hipMemcpy(d_list, list.data(), sizeof(int) * kPieces, hipMemcpyHostToDevice));
        for (int wpc : {2, 8}) {
            if (pol != 0 && wpc != 2) continue;
            const int grid = 256 * wpc;
            auto launch = [&](int r) {
                const unsigned char* region = buf + r * kRegionBytes;
                if (wpc == 8) hipLaunchKernelGGL((read_region<0, 0>), dim3(grid), dim3(256), 0, 0, region, d_list, kPieces, d_out);
                else if (pol == 0) hipLaunchKernelGGL((read_region<2, 0>), dim3(grid), dim3(256), 0, 0, region, d_list, kPieces, d_out);
                else if (pol == 2) hipLaunchKernelGGL((read_region<2, 2>), dim3(grid), dim3(256), 0, 0, region, d_list, kPieces, d_out);
                else if (pol == 1) hipLaunchKernelGGL((read_region<2, 1>), dim3(grid), dim3(256), 0, 0, region, d_list, kPieces, d_out);
                else if (pol == 3) hipLaunchKernelGGL((read_region<2, 3>), dim3(grid), dim3(256), 0, 0, region, d_list, kPieces, d_out);
                else hipLaunchKernelGGL((read_region<2, 17>), dim3(grid), dim3(256), 0, 0, region, d_list, kPieces, d_out);
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
            const double gb = static_cast<double>(kRegionBytes) / 1e9;
            printf("%-8s %d WG/CU policy %2d: %.1f MB per launch, median %7.1f us (%5.0f GB/s), p10 %7.1f  p90 %7.1f us\n",
                   names[mode], wpc, pol, gb * 1e3, ts[15] * 1e3, gb / (ts[15] * 1e-3), ts[3] * 1e3, ts[27] * 1e3);
            fflush(stdout);
            CK(hipEventDestroy(e0));
            CK(hipEventDestroy(e1));
        }
    }
    }
    CK(hipFree(buf));
    CK(hipFree(d_out));
    CK(hipFree(d_list));
    return 0;
}
