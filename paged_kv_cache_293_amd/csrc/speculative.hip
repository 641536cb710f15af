// Exact speculative acceptance for gfx950.
//
// Method (page "LLM Serving - KV Cache, Batching, Speculative Decoding",
// section "Speculative decoding: distribution and break-even"; page "KV cache
// & continuous batching", section "5. Speculative decoding"): position i of a
// drafted block accepts its token x_i with probability min(1, p_i(x_i) /
// q_i(x_i)); the first rejected position emits a token drawn from the
// normalised positive residual (p_i - q_i)+; a fully accepted block emits a
// bonus token drawn from p_{K+1}.  Random draws come in as arrays.
//
// Steps, one work-group of 16 waves per sequence:
//  1. thread i < K tests position i:  u_i * q_i(x_i) < p_i(x_i) in float32;
//     the first failing position (or K) is a;
//  2. the emitted token's weights are w = max(p_a - q_a, 0) (a < K) or p_K;
//     the row is split into 16 contiguous segments, one per wave; a wave
//     walks its segment in tiles of 1024 weights (four coalesced float4
//     loads per lane) and keeps each tile's total (lane sums, then a fixed
//     butterfly over the lanes) in LDS;
//  3. S = sum of the segment totals (fixed order), T = u * S; the wave whose
//     segment crosses T finds the crossing tile from its totals, re-reads that
//     tile and scans it in index order: the emitted token is the first index
//     whose running sum exceeds T.  Where float32 rounding leaves T at or past
//     the end of a scan (u close to 1), the last segment, tile or index with
//     weight is taken, so a row with mass always yields a token; only a
//     residual with no mass (S = 0) falls back to p_a.
// The row is read once (plus one tile); the kernel is bound by HBM.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kSpWaves = 16;
constexpr int kSpThreads = 64 * kSpWaves;
constexpr int kSpSub = 256;           // weights per coalesced wave load (64 lanes x float4)
constexpr int kSpTile = 4 * kSpSub;   // weights per tile (four loads per lane)

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Inclusive scan of v over the 64 lanes (lane order), fixed association.
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    return v;
}

// Sum of v over the 64 lanes (fixed butterfly association; every lane gets it).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d);
    return v;
}

// The four weights at e0 .. e0+3 of the row (0 past the vocabulary).
template <bool VEC>
__device__ __forceinline__ f32x4 load_weights(const float* p, const float* q, int64_t e0, int vocab, bool resid) {
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if constexpr (VEC) {
        if (e0 < vocab) {
            w = *reinterpret_cast<const f32x4*>(p + e0);
            if (resid) {
                const f32x4 b = *reinterpret_cast<const f32x4*>(q + e0);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = fmaxf(w[i] - b[i], 0.f);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (e0 + i < vocab) {
                const float x = p[e0 + i];
                w[i] = resid ? fmaxf(x - q[e0 + i], 0.f) : x;
            }
        }
    }
    return w;
}

template <bool VEC>
__global__ __launch_bounds__(kSpThreads) void speculative_accept_kernel(SpecArgs a) {
    extern __shared__ float sp_tile_tot[];   // [kSpWaves][tiles per segment]
    __shared__ int first_reject;
    __shared__ float seg_total[kSpWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int b = blockIdx.x;
    const int K = a.k;
    const int64_t V = a.vocab;

    // 1. acceptance tests
    if (tid == 0) first_reject = K;
    __syncthreads();
    if (tid < K) {
        const int x = a.draft[static_cast<int64_t>(b) * K + tid];
        bool ok = false;
        if (x >= 0 && x < V) {
            const int64_t row = static_cast<int64_t>(b) * K + tid;
            const float pu = a.p[(static_cast<int64_t>(b) * (K + 1) + tid) * V + x];
            const float qu = a.q[row * V + x];
            ok = __fmul_rn(a.u_accept[row], qu) < pu;
        }
        if (!ok) atomicMin(&first_reject, tid);
    }
    __syncthreads();
    const int acc = first_reject;

    const float* prow = a.p + (static_cast<int64_t>(b) * (K + 1) + acc) * V;
    const float* qrow = acc < K ? a.q + (static_cast<int64_t>(b) * K + acc) * V : nullptr;
    const int64_t seg = a.seg_len;            // multiple of kSpTile
    const int tiles = static_cast<int>(seg / kSpTile);
    float* my_tot = sp_tile_tot + wave * tiles;
    const float u = a.u_sample[b];

    int token = -1;
    for (int attempt = 0; attempt < 2 && token < 0; ++attempt) {
        const bool resid = acc < K && attempt == 0;
        // 2. tile totals of this wave's segment
        const int64_t s0 = wave * seg;
        float run = 0.f;
        for (int t = 0; t < tiles; ++t) {
            const int64_t tb0 = s0 + static_cast<int64_t>(t) * kSpTile + 4 * lane;
            f32x4 w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w[k] = load_weights<VEC>(prow, qrow, tb0 + k * kSpSub, static_cast<int>(V), resid);
            float ls = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) ls += ((w[k][0] + w[k][1]) + w[k][2]) + w[k][3];
            const float tt = wave_sum(ls);
            if (lane == 0) my_tot[t] = tt;
            run += tt;
        }
        if (lane == 0) seg_total[wave] = run;
        __syncthreads();
        float S = 0.f;
        for (int w = 0; w < kSpWaves; ++w) S += seg_total[w];
        if (S > 0.f) {
            const float T = __fmul_rn(u, S);
            // 3. the crossing segment, tile and index.  Partial sums are
            // formed in the order S and the segment totals were (segment
            // totals from 0 in segment order; tile totals from 0 in tile
            // order), so a segment found crossing holds a crossing tile.
            // Where rounding leaves T at or past the end (u close to 1),
            // the fallback is the last segment, then tile, with weight.
            float base = 0.f, base_last = 0.f;
            int cw = -1, last_w = -1;
            for (int w = 0; w < kSpWaves; ++w) {
                if (seg_total[w] > 0.f) { last_w = w; base_last = base; }
                if (cw < 0 && base + seg_total[w] > T) cw = w;
                if (cw < 0) base += seg_total[w];
            }
            if (cw < 0) { cw = last_w; base = base_last; }
            if (wave == cw) {
                int ct = -1, last_t = -1;
                float r = 0.f, r_ct = 0.f, r_last = 0.f;   // tile totals before t
                for (int t = 0; t < tiles; ++t) {
                    if (my_tot[t] > 0.f) { last_t = t; r_last = r; }
                    if (ct < 0 && base + (r + my_tot[t]) > T) { ct = t; r_ct = r; }
                    r += my_tot[t];
                }
                if (ct < 0) { ct = last_t; r_ct = r_last; }
                const float tb = base + r_ct;
                // scan the crossing tile in index order: its four 256-weight parts in turn
                int pick = -1;
                int last_pick = -1;
                float c0 = tb;
                for (int k = 0; k < 4 && pick < 0; ++k) {
                    const int64_t e0 = s0 + static_cast<int64_t>(ct) * kSpTile + k * kSpSub + 4 * lane;
                    const f32x4 w = load_weights<VEC>(prow, qrow, e0, static_cast<int>(V), resid);
                    const float ls = ((w[0] + w[1]) + w[2]) + w[3];
                    const float incl = wave_inclusive_scan(ls, lane);
                    float c = c0 + (incl - ls);
                    int hit = -1;
                    int last_pos = -1;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        c += w[i];
                        if (hit < 0 && w[i] > 0.f && c > T) hit = i;
                        if (w[i] > 0.f) last_pos = i;
                    }
                    const unsigned long long found = __ballot(hit >= 0);
                    if (found) {
                        const int l = __ffsll(static_cast<long long>(found)) - 1;
                        pick = __shfl(static_cast<int>(e0) + hit, l);
                    }
                    const unsigned long long any = __ballot(last_pos >= 0);
                    if (any) {
                        const int l = 63 - __clzll(static_cast<long long>(any));
                        last_pick = __shfl(static_cast<int>(e0) + last_pos, l);
                    }
                    c0 += __shfl(incl, 63);
                }
                // rounding put T at the tile's end: its last weighted index
                if (pick < 0) pick = last_pick;
                if (lane == 0) first_reject = pick;   // reuse as the result slot
            }
            __syncthreads();
            token = first_reject;
            __syncthreads();
        } else {
            __syncthreads();
        }
    }

    if (tid == 0) a.num_accepted[b] = acc;
    for (int i = tid; i <= K; i += kSpThreads) {
        int v = -1;
        if (i < acc) v = a.draft[static_cast<int64_t>(b) * K + i];
        else if (i == acc) v = token;
        a.tokens[static_cast<int64_t>(b) * (K + 1) + i] = v;
    }
}

}  // namespace

hipError_t launch_speculative_accept(const SpecArgs& a, hipStream_t stream) {
    if (a.num_seqs <= 0) return hipSuccess;
    const size_t lds = static_cast<size_t>(kSpWaves) * (a.seg_len / kSpTile) * sizeof(float);
    if (a.vocab % 4 == 0)
        hipLaunchKernelGGL(speculative_accept_kernel<true>, dim3(a.num_seqs), dim3(kSpThreads), lds, stream, a);
    else
        hipLaunchKernelGGL(speculative_accept_kernel<false>, dim3(a.num_seqs), dim3(kSpThreads), lds, stream, a);
    return hipGetLastError();
}

int64_t speculative_segment_len(int64_t vocab) {
    const int64_t per_wave = (vocab + kSpWaves - 1) / kSpWaves;
    return (per_wave + kSpTile - 1) / kSpTile * kSpTile;
}

}  // namespace pkv
