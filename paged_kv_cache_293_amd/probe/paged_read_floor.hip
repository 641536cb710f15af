// Paged-read floor at the decode step's shape: a standalone program (not part
// of the library).  It reads exactly the tiles a Llama-3-8B decode step reads
// (64 sequences, lengths uniform in [512, 4096], 16-token blocks, 8 KV heads,
// blocks placed by a random permutation over a pool of 1.25x the blocks in
// use) and nothing else: no scores, no softmax, no output.  Pool layout as the
// library's: the 8 KV heads' tiles of a block are adjacent, so one block is
// 8 x S contiguous bytes (S = 8 KiB for bf16 K+V at head dim 128, 4 KiB for
// one-byte codes, 2 KiB for int4).
//
// The tiles are listed in one of two orders and cut into equal runs, one run
// per work-group; a work-group's 4 waves take its run's tiles round robin,
// 16 bytes per lane per load (at 2 work-groups per CU with two tiles in flight
// per wave while a third is consumed: the decode kernel's pipeline):
//   head : sequence, then KV head, then block (the decode kernel's order: a
//          work-group walks one head of one sequence, reading one S-byte tile
//          of each 8 x S-byte block);
//   block: sequence, then block, then KV head (a work-group's waves read the
//          adjacent tiles of one block together: 8 x S contiguous bytes).
// Three pool copies are read in turn, so no launch finds the previous one's
// tiles in the 256 MB Infinity Cache.  Grids of 2, 4 and 8 work-groups per CU
// (a work-group is one wave on each SIMD, so 2, 4 and 8 waves per SIMD); so
// that every work-group of the grid is resident at once, the 4 per CU grid
// keeps one tile per wave in flight while one is consumed, and the 8 per CU
// grid one tile per wave (load, consume).  Every tile index is checked
// against the pool on the host.
// Every configuration runs with the default cache policy of the loads and
// with the non-temporal one the decode kernel uses.  Prints the median launch
// time over 30 launches, p10 and p90, and the rate.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); exit(1); } } while (0)

constexpr int kHeads = 8;
constexpr int kSeqs = 64;
constexpr int kCopies = 3;

template <int S> struct Tile { u32x4 w[S / 1024]; };   // 1 KiB per wave load

// POL: the loads' cache-policy bits (0 default, 2 non-temporal).
template <int S, int POL>
__device__ __forceinline__ void load_tile(Tile<S>& t, const unsigned char* pool, long tile, bool valid, int lane) {
    // a zero-sized resource returns zeros without touching memory
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(pool + tile * S), 0, valid ? S : 0, 0x00020000);
#pragma unroll
    for (int s = 0; s < S / 1024; ++s)
        t.w[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 1024 * s, POL));
}

template <int S>
__device__ __forceinline__ unsigned fold(const Tile<S>& t) {
    unsigned a = 0;
#pragma unroll
    for (int s = 0; s < S / 1024; ++s) a ^= t.w[s][0] ^ t.w[s][1] ^ t.w[s][2] ^ t.w[s][3];
    return a;
}

// Work-group b reads tiles list[b * per .. b * per + run), run <= per (the
// last runs may be shorter); wave w takes w, w + 4, ...  DEPTH 2: three tile
// buffers (two tiles in flight while one is consumed); DEPTH 1: two buffers;
// DEPTH 0: one buffer (load, consume, load).
template <int S, int DEPTH, int POL>
__global__ __launch_bounds__(256) void read_tiles(const unsigned char* pool, const int* list, int per, int total,
                                                  unsigned* out) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int* my = list + static_cast<long>(blockIdx.x) * per;
    const int run = max(0, min(per, total - static_cast<int>(blockIdx.x) * per));
    const int cnt = (run - wave + 3) / 4;
    auto id = [&](int i) { return i < cnt ? static_cast<long>(my[wave + 4 * i]) : 0L; };
    unsigned acc = 0;
    if constexpr (DEPTH == 2) {
        Tile<S> ta, tb, tc;
        load_tile<S, POL>(ta, pool, id(0), cnt > 0, lane);
        load_tile<S, POL>(tb, pool, id(1), cnt > 1, lane);
        int i = 0;
        for (; i + 2 < cnt; i += 3) {
            load_tile<S, POL>(tc, pool, id(i + 2), true, lane);
            acc += fold<S>(ta);
            load_tile<S, POL>(ta, pool, id(i + 3), i + 3 < cnt, lane);
            acc += fold<S>(tb);
            load_tile<S, POL>(tb, pool, id(i + 4), i + 4 < cnt, lane);
            acc += fold<S>(tc);
        }
        if (i < cnt) acc += fold<S>(ta);
        if (i + 1 < cnt) acc += fold<S>(tb);
    } else if constexpr (DEPTH == 1) {
        Tile<S> ta, tb;
        load_tile<S, POL>(ta, pool, id(0), cnt > 0, lane);
        int i = 0;
        for (; i + 1 < cnt; i += 2) {
            load_tile<S, POL>(tb, pool, id(i + 1), true, lane);
            acc += fold<S>(ta);
            load_tile<S, POL>(ta, pool, id(i + 2), i + 2 < cnt, lane);
            acc += fold<S>(tb);
        }
        if (i < cnt) acc += fold<S>(ta);
    } else {
        for (int i = 0; i < cnt; ++i) {
            Tile<S> t;
            load_tile<S, POL>(t, pool, id(i), true, lane);
            acc += fold<S>(t);
        }
    }
    if (acc == 0x12345678u) out[blockIdx.x] = acc;   // keeps the loads
}

struct Step {
    std::vector<int> lens;      // tokens per sequence
    std::vector<std::vector<int>> table;   // physical block of each logical block
    int num_blocks = 0;         // pool blocks
};

Step make_step(std::mt19937_64& rng) {
    Step st;
    std::uniform_int_distribution<int> len(512, 4096);
    int used = 0;
    for (int s = 0; s < kSeqs; ++s) {
        st.lens.push_back(len(rng));
        used += (st.lens.back() + 15) / 16;
    }
    st.num_blocks = (used * 5 + 3) / 4;
    std::vector<int> perm(st.num_blocks);
    for (int i = 0; i < st.num_blocks; ++i) perm[i] = i;
    std::shuffle(perm.begin(), perm.end(), rng);
    int cursor = 0;
    for (int s = 0; s < kSeqs; ++s) {
        const int nb = (st.lens[s] + 15) / 16;
        st.table.emplace_back(perm.begin() + cursor, perm.begin() + cursor + nb);
        cursor += nb;
    }
    return st;
}

// Tile index = block * kHeads + head, in the chosen order.
std::vector<int> tile_list(const Step& st, bool block_major) {
    std::vector<int> out;
    for (int s = 0; s < kSeqs; ++s) {
        const std::vector<int>& t = st.table[s];
        if (block_major) {
            for (int b : t)
                for (int h = 0; h < kHeads; ++h) out.push_back(b * kHeads + h);
        } else {
            for (int h = 0; h < kHeads; ++h)
                for (int b : t) out.push_back(b * kHeads + h);
        }
    }
    return out;
}

template <int S, int POL>
void run(const Step& st, bool block_major, int wgs_per_cu, unsigned* d_out) {
    const long copy_bytes = static_cast<long>(st.num_blocks) * kHeads * S;
    unsigned char* buf;
    CK(hipMalloc(&buf, copy_bytes * kCopies));
    CK(hipMemset(buf, 1, copy_bytes * kCopies));
    std::vector<int> list = tile_list(st, block_major);
    const int grid = 256 * wgs_per_cu;
    const int per = static_cast<int>((list.size() + grid - 1) / grid);
    const int total = static_cast<int>(list.size());
    const long tiles = total;
    for (int x : list)
        if (x < 0 || static_cast<long>(x) >= static_cast<long>(st.num_blocks) * kHeads) { printf("bad tile\n"); exit(1); }
    if (static_cast<long>(per) * grid < total) { printf("bad runs\n"); exit(1); }
    int* d_list;
    CK(hipMalloc(&d_list, sizeof(int) * list.size()));
    CK(hipMemcpy(d_list, list.data(), sizeof(int) * list.size(), hipMemcpyHostToDevice));
    auto launch = [&](int c) {
        if (wgs_per_cu >= 8)
            hipLaunchKernelGGL((read_tiles<S, 0, POL>), dim3(grid), dim3(256), 0, 0, buf + c * copy_bytes, d_list, per,
                               total, d_out);
        else if (wgs_per_cu >= 4)
            hipLaunchKernelGGL((read_tiles<S, 1, POL>), dim3(grid), dim3(256), 0, 0, buf + c * copy_bytes, d_list, per,
                               total, d_out);
        else
            hipLaunchKernelGGL((read_tiles<S, 2, POL>), dim3(grid), dim3(256), 0, 0, buf + c * copy_bytes, d_list, per,
                               total, d_out);
        CK(hipGetLastError());
    };
    for (int w = 0; w < 6; ++w) launch(w % kCopies);
    CK(hipDeviceSynchronize());
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    std::vector<float> ts;
    for (int rep = 0; rep < 30; ++rep) {
        CK(hipEventRecord(e0));
        launch(rep % kCopies);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        float ms = 0;
        CK(hipEventElapsedTime(&ms, e0, e1));
        ts.push_back(ms);
    }
    std::sort(ts.begin(), ts.end());
    const double gb = static_cast<double>(tiles) * S / 1e9;
    printf("tile %5d B  order %-5s  %d WG/CU  policy %d: %6.1f MB  median %6.1f us (%5.0f GB/s)  p10 %6.1f  p90 %6.1f us\n",
           S, block_major ? "block" : "head", wgs_per_cu, POL, gb * 1e3, ts[15] * 1e3, gb / (ts[15] * 1e-3),
           ts[3] * 1e3, ts[27] * 1e3);
    fflush(stdout);
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
    CK(hipFree(d_list));
    CK(hipFree(buf));
}

int main() {
    std::mt19937_64 rng(293002);
    const Step st = make_step(rng);
    long tokens = 0;
    for (int n : st.lens) tokens += n;
    printf("decode step: %d sequences, %ld tokens, pool of %d blocks\n", kSeqs, tokens, st.num_blocks);
    unsigned* d_out;
    CK(hipMalloc(&d_out, sizeof(unsigned) * 256 * 8));
    for (int wpc : {2, 4, 8})
        for (int bm = 0; bm <= 1; ++bm) {
            run<8192, 0>(st, bm == 1, wpc, d_out);
            run<4096, 0>(st, bm == 1, wpc, d_out);
            run<2048, 0>(st, bm == 1, wpc, d_out);
        }
    for (int wpc : {2, 4, 8})
        for (int bm = 0; bm <= 1; ++bm) {
            run<8192, 2>(st, bm == 1, wpc, d_out);
            run<4096, 2>(st, bm == 1, wpc, d_out);
            run<2048, 2>(st, bm == 1, wpc, d_out);
        }
    CK(hipFree(d_out));
    return 0;
}
