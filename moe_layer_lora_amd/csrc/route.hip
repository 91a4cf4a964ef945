// route.hip - top-k routing and expert grouping on gfx950.
//
// The grouping follows the flatten / stable sort by expert id / bincount /
// offset-slice formulation of the Unsloth x NVIDIA blog (d9249.github.io,
// section "core idea / structure / how it works", MoE routing paragraph), as
// three kernels with no host synchronisation:
//   1. topk:    per token, top-k experts by (logit desc, id asc) and softmax
//               over the k selected logits; per-block expert histogram in
//               LDS (the bincount, split over token blocks).
//   2. scan:    one exclusive scan over the expert-major [E x nblk]
//               histogram gives every (expert, block) its first output row;
//               counts and offsets fall out of the same pass.
//   3. scatter: each block ranks its slots within their expert with wave64
//               ballots (match on the expert-id bits, popcount below the
//               lane) plus a cross-wave prefix in LDS; the rank is stable
//               (slot order = token order), so the result is the stable sort.
#include "kernels.hpp"
#include "common.hpp"

#include <climits>

namespace moe {

constexpr int kRouteThreads = 1024;  // 16 waves per block: few blocks, so a small block histogram to scan
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / kWave;  // 16 logits per lane

int route_tokens_per_block(int T, int E) {
    // 2 tokens per wave: 256 blocks at 8192 tokens fill every CU (64 tokens per
    // block, half of them, made top-k 50% slower; 16 per block made the scan
    // of the larger histogram cost more than top-k gained)
    int tpb = 32;
    while ((long long)E * ((T + tpb - 1) / tpb) > 65536) tpb *= 2;
    return tpb;
}

// The router's order: larger logit first, ties to the lower id. Logits are
// compared through an order-preserving 32-bit key: larger logit, larger key.
// -0.0 is first made +0.0 (the two compare equal, so the lower id must win);
// 0 is below every finite logit's key and marks taken or absent entries.
__device__ __forceinline__ uint32_t route_key(float v) {
    const uint32_t b = __float_as_uint(v + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float route_key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Maximum over the wave by DPP: row_shr 1, 2, 4, 8 leave each row's maximum
// in its lane 15, row_bcast 15 and 31 carry it to lane 63. Out-of-range
// sources read 0, the smallest key.
__device__ __forceinline__ uint32_t wave_max_key(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));  // row_shr:1
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));  // row_shr:2
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));  // row_shr:4
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));  // row_shr:8
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false)); // row_bcast:15
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false)); // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// NPL: logits per lane (E <= 64 NPL); KS: result slots per lane (k <= 64 KS)
template <int NPL, int KS>
__global__ __launch_bounds__(kRouteThreads) void k_route_topk(const float *__restrict__ logits, int T, int E,
                                                              int k, int tpb, int nblk,
                                                              int32_t *__restrict__ topk_idx,
                                                              float *__restrict__ topk_w,
                                                              int32_t *__restrict__ hist) {
    __shared__ int s_hist[kMaxE];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    for (int e = tid; e < E; e += kRouteThreads) s_hist[e] = 0;
    __syncthreads();
    const int b = blockIdx.x;
    const int t0 = b * tpb, t1 = min(T, t0 + tpb);
    for (int t = t0 + wave; t < t1; t += kRouteWaves) {
        const float *row = logits + (size_t)t * E;
        // entry i of this lane is expert lane + 64 i: ids rise with i
        uint32_t key[NPL];
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int e = lane + kWave * i;
            key[i] = e < E ? route_key(row[e]) : 0u;
        }
        int my_idx[KS];
        float my_val[KS];
        float v0 = 0.0f;
        for (int j = 0; j < k; ++j) {
            // the best key left, then the lowest id holding it (ballots in id order)
            uint32_t m = key[0];
#pragma unroll
            for (int i = 1; i < NPL; ++i) m = max(m, key[i]);
            m = wave_max_key(m);
            int bid = -1;
#pragma unroll
            for (int i = 0; i < NPL; ++i) {
                const uint64_t hit = __ballot(key[i] == m);
                if (bid < 0 && hit != 0) bid = __builtin_ctzll(hit) + kWave * i;
            }
            const float bv = route_key_value(m);
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (bid == lane + kWave * i) key[i] = 0u;  // taken
            if (j == 0) v0 = bv;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                if (s == (j / kWave) && lane == (j & (kWave - 1))) {
                    my_idx[s] = bid;
                    my_val[s] = bv;
                }
            if (lane == 0) atomicAdd(&s_hist[bid], 1);
        }
        // softmax over the k selected logits, shifted by the largest
        float sum = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            if (s * kWave + lane < k) sum += expf(my_val[s] - v0);
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int j = s * kWave + lane;
            if (j < k) {
                topk_idx[(size_t)t * k + j] = my_idx[s];
                topk_w[(size_t)t * k + j] = expf(my_val[s] - v0) / sum;
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) hist[(size_t)b * E + e] = s_hist[e];  // block-major
}

// exclusive scan of one value per thread over a 1024-thread block
__device__ int block_excl_scan_1024(int v, int *s_wsum) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int w = lane < 16 ? s_wsum[lane] : 0;
        int wi = w;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int o = __shfl_up(wi, off, kWave);
            if (lane >= off) wi += o;
        }
        if (lane < 16) s_wsum[lane] = wi - w;  // exclusive over waves
    }
    __syncthreads();
    const int r = s_wsum[wave] + incl - v;
    __syncthreads();
    return r;
}

// Scan of the block-major [nblk x E] histogram. Thread (g, e) owns expert e
// over the g-th range of token blocks; per-column passes are coalesced across
// the lanes (consecutive experts). host_counts, if not null, is page-locked
// host memory mapped for the device at its host address: the counts are
// stored there too (vector stores over the bus), in place of a copy.
__global__ __launch_bounds__(1024) void k_route_scan(const int32_t *__restrict__ hist, int E, int nblk, int S,
                                                     int32_t *__restrict__ base, int32_t *__restrict__ counts,
                                                     int32_t *__restrict__ offsets, int32_t *__restrict__ host_counts) {
    __shared__ int s_wsum[16];
    __shared__ int s_part[1024];
    const int tid = threadIdx.x;
    const int G = max(1, 1024 / E);            // block ranges
    const int g = tid / E, e = tid % E;
    const bool act = g < G;
    const int per = (nblk + G - 1) / G;
    const int b0 = min(nblk, g * per), b1 = min(nblk, b0 + per);
    int part = 0;
    if (act) {
#pragma unroll 16
        for (int b = b0; b < b1; ++b) part += hist[(size_t)b * E + e];  // unrolled: many loads in flight
    }
    s_part[tid] = act ? part : 0;
    __syncthreads();
    int c = 0;
    if (tid < E)
        for (int q = 0; q < G; ++q) c += s_part[q * E + tid];
    const int off = block_excl_scan_1024(tid < E ? c : 0, s_wsum);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = off;
        if (host_counts) host_counts[tid] = c;
    }
    if (tid == 0) offsets[E] = S;
    // bases: offset of e plus the counts of e in earlier blocks
    __shared__ int s_off[1024];
    if (tid < E) s_off[tid] = off;
    __syncthreads();
    if (act) {
        int run = s_off[e];
        for (int q = 0; q < g; ++q) run += s_part[q * E + e];
#pragma unroll 16
        for (int b = b0; b < b1; ++b) {
            const int h = hist[(size_t)b * E + e];
            base[(size_t)b * E + e] = run;
            run += h;
        }
    }
}

__global__ __launch_bounds__(kRouteThreads) void k_route_scatter(const int32_t *__restrict__ topk_idx,
                                                                 const int32_t *__restrict__ base, int T, int E,
                                                                 int k, int tpb, int nblk,
                                                                 int32_t *__restrict__ sorted_slot,
                                                                 int32_t *__restrict__ slot_row) {
    __shared__ int s_base[kMaxE], s_run[kMaxE], s_wcnt[kRouteWaves][kMaxE];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int b = blockIdx.x;
    for (int e = tid; e < E; e += kRouteThreads) {
        s_base[e] = base[(size_t)b * E + e];  // block-major
        s_run[e] = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) s_wcnt[w][e] = 0;
    }
    __syncthreads();
    const int q0 = b * tpb * k, q1 = min(T, (b + 1) * tpb) * k;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int rb = q0; rb < q1; rb += kRouteThreads) {
        const int q = rb + tid;
        const bool valid = q < q1;
        const int e = valid ? topk_idx[q] : 0;
        unsigned long long m = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool set = (e >> bit) & 1;
            const unsigned long long bb = __ballot(valid && set);
            m &= set ? bb : ~bb;
        }
        const int rank_w = __popcll(m & below);
        if (valid && rank_w == 0) s_wcnt[wave][e] = __popcll(m);
        __syncthreads();
        if (valid) {
            int pre = 0;
            for (int w = 0; w < wave; ++w) pre += s_wcnt[w][e];
            const int pos = s_base[e] + s_run[e] + pre + rank_w;
            sorted_slot[pos] = q;
            slot_row[q] = pos;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kRouteThreads) {
            int add = 0;
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) {
                add += s_wcnt[w][x];
                s_wcnt[w][x] = 0;
            }
            s_run[x] += add;
        }
        __syncthreads();
    }
}

hipError_t launch_route_topk(const float *logits, int T, int E, int k, int32_t *topk_idx, float *topk_w,
                             int32_t *hist, hipStream_t st) {
    const int nblk = route_nblk(T, E);
    if (nblk == 0) return hipSuccess;
    const int tpb = route_tokens_per_block(T, E);
#define MOE_TOPK(NPL, KS)                                                                                  \
    hipLaunchKernelGGL((k_route_topk<NPL, KS>), dim3(nblk), dim3(kRouteThreads), 0, st, logits, T, E, k, tpb,    \
                       nblk, topk_idx, topk_w, hist)
    if (E <= 64) MOE_TOPK(1, 1);
    else if (E <= 128) { if (k <= 64) MOE_TOPK(2, 1); else MOE_TOPK(2, 2); }
    else if (E <= 256) { if (k <= 64) MOE_TOPK(4, 1); else MOE_TOPK(4, 4); }
    else if (E <= 512) { if (k <= 64) MOE_TOPK(8, 1); else MOE_TOPK(8, 8); }
    else { if (k <= 64) MOE_TOPK(16, 1); else MOE_TOPK(16, 16); }
#undef MOE_TOPK
    return hipGetLastError();
}

hipError_t launch_route_scan(const int32_t *hist, int T, int E, int k, int32_t *base, int32_t *counts,
                             int32_t *offsets, int32_t *host_counts, hipStream_t st) {
    const int nblk = route_nblk(T, E);
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, st, hist, E, nblk, T * k, base, counts, offsets,
                       host_counts);
    return hipGetLastError();
}

hipError_t launch_route_scatter(const int32_t *topk_idx, const int32_t *base, int T, int E, int k,
                                int32_t *sorted_slot, int32_t *slot_row, hipStream_t st) {
    const int nblk = route_nblk(T, E);
    if (nblk == 0) return hipSuccess;
    const int tpb = route_tokens_per_block(T, E);
    hipLaunchKernelGGL(k_route_scatter, dim3(nblk), dim3(kRouteThreads), 0, st, topk_idx, base, T, E, k, tpb, nblk,
                       sorted_slot, slot_row);
    return hipGetLastError();
}

}  // namespace moe
