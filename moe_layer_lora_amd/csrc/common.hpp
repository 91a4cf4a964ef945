// common.hpp - element types, MFMA fragments and the grouped-tile scheduler
// shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace moe {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));  // one 16-byte chunk
// 16-byte store marked non-temporal (no L2 allocation): for grouped-GEMM
// outputs that only a later kernel reads, so they do not evict the operand
// lines the other tiles on the same L2 are still streaming
__device__ __forceinline__ void st_stream(void *p, const chunk_t &v) {
    __builtin_nontemporal_store(v, reinterpret_cast<chunk_t *>(p));
}
// 16-byte load marked non-temporal: for data a kernel reads exactly once
__device__ __forceinline__ chunk_t ld_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const chunk_t *>(p));
}

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// two values, same rounding, lo in bits 0-15: one v_cvt_pk_bf16_f32 (two
// scalar conversions cost two of them plus a shift and an or)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------------------
// Element traits. A "chunk" is 16 bytes: VEC elements. Both MFMA operands
// are read from LDS one chunk per lane: lane l holds VEC consecutive k of
// row (l % 32), at k offset (l / 32) * VEC within a k-group of 2*VEC.
template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int VEC = 4;
    __device__ static float load_f32(const float *p, int i) { return p[i]; }
    __device__ static float to_f32(float v) { return v; }
    __device__ static float from_f32(float v) { return v; }
    // acc(32x32) += A(32 x 8) * B(8 x 32); the 8 k of a group are split as
    // lane-half h holding k = 4h .. 4h+3; instruction i takes element i of
    // both chunks, so it covers k in {i, 4+i}: the same k-permutation on both
    // operands, hence the exact sum over the group.
    __device__ static void mma(f32x16_t &acc, const chunk_t &a, const chunk_t &b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), acc, 0, 0, 0);
    }
    // VEC fp32 values -> one chunk
    __device__ static chunk_t pack(const float *v) {
        return chunk_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                       __float_as_uint(v[3])};
    }
};

template <> struct Elem<bf16_t> {
    static constexpr int VEC = 8;
    __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
    __device__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
    // acc(32x32) += A(32 x 16) * B(16 x 32), one v_mfma_f32_32x32x16_bf16
    __device__ static void mma(f32x16_t &acc, const chunk_t &a, const chunk_t &b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
    __device__ static chunk_t pack(const float *v) {
        chunk_t c;
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = f32x2_to_bf16x2(v[2 * i], v[2 * i + 1]);
        return c;
    }
};

// unpack one chunk into VEC floats
template <typename T> __device__ __forceinline__ void unpack(const chunk_t &c, float *v);
template <> __device__ __forceinline__ void unpack<float>(const chunk_t &c, float *v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(c[i]);
}
template <> __device__ __forceinline__ void unpack<bf16_t>(const chunk_t &c, float *v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(c[i] << 16);
        v[2 * i + 1] = __uint_as_float(c[i] & 0xffff0000u);
    }
}

// Row and column of accumulator register i of a 32x32 MFMA tile held by `lane`.
__device__ __forceinline__ int acc_row(int i, int lane) { return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Logistic function from the hardware exp and reciprocal (about 1 ulp each)
// instead of an IEEE-exact division: for epilogues whose results are stored
// as bf16 (8 mantissa bits), where the exact division's ~10 VALU
// instructions per element would dominate the tile's epilogue.
__device__ __forceinline__ float sigmoid_fast(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// SwiGLU h = silu(g) u of one element: the fast logistic for bf16 layers,
// IEEE exp and division for fp32 layers.
__device__ __forceinline__ float swiglu_fast(float g, float u) { return g * sigmoid_fast(g) * u; }
__device__ __forceinline__ float swiglu_ieee(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// One 16-byte chunk of H from the chunks of G and U as stored. H is a
// function of the stored (rounded) G and U, not of the accumulators, so the
// forward's epilogue and a later rebuild from the stored G and U (the reload
// of offloaded activations) give bit-identical H.
template <typename T> __device__ __forceinline__ chunk_t swiglu_chunk(const chunk_t &cg, const chunk_t &cu);
template <> __device__ __forceinline__ chunk_t swiglu_chunk<bf16_t>(const chunk_t &cg, const chunk_t &cu) {
    float g[8], u[8], h[8];
    unpack<bf16_t>(cg, g);
    unpack<bf16_t>(cu, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = swiglu_fast(g[e], u[e]);
    return Elem<bf16_t>::pack(h);
}
template <> __device__ __forceinline__ chunk_t swiglu_chunk<float>(const chunk_t &cg, const chunk_t &cu) {
    chunk_t h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = __float_as_uint(swiglu_ieee(__uint_as_float(cg[e]), __uint_as_float(cu[e])));
    return h;
}

// ---------------------------------------------------------------------------
// Grouped-tile scheduler. Expert e owns rows offsets[e] .. offsets[e+1]-1,
// cut into mt_e = ceil(n_e / BM) row tiles; each row tile is crossed with NT
// column tiles. Work items are ordered expert-major, then column tile, then
// row tile, so the row tiles that share one expert weight strip are
// consecutive. Hardware hands workgroups to the 8 XCDs round-robin by block
// id; the remap below gives each XCD a contiguous range of work items, so a
// weight strip (and an expert's rows) is fetched into one XCD's L2 and
// reused there. Empty experts own no work and their weights are never read.
struct Tile {
    int e;      // expert
    int mt;     // row tile within the expert
    int nt;     // column tile
    int row0;   // first row p of the tile
    int rows;   // valid rows in the tile (1..BM)
    int gmt;    // row tile index over all experts (expert-major)
};

// Inclusive scan of s[1..E] in place (__shared__, E <= 1024) by one wave,
// lane l taking the l-th sequential segment of up to 16 entries.
__device__ __forceinline__ void wave_scan_shared(int *s, int E, int lane) {
    const int per = (E + kWave - 1) / kWave;
    const int lo = 1 + lane * per, hi = min(E + 1, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += s[i];
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
    }
    int run = incl - sum;
    for (int i = lo; i < hi; ++i) {
        run += s[i];
        s[i] = run;
    }
}

// Per-expert row-tile counts ceil(n_e / BM) and their inclusive scan into
// s_start[0..E] (__shared__ int[E+1], E <= 1024); ends with a barrier.
template <int BM, int NTHREADS>
__device__ void scan_row_tiles(const int *__restrict__ offsets, int E, int *s_start) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += NTHREADS) {
        const int n = offsets[e + 1] - offsets[e];
        s_start[e + 1] = (n + BM - 1) / BM;
    }
    if (tid == 0) s_start[0] = 0;
    __syncthreads();
    if (tid < kWave) wave_scan_shared(s_start, E, tid);
    __syncthreads();
}

// XCD-contiguous remap of block ids (a bijection on [0, total))
__device__ __forceinline__ int xcd_item(int b, int total) {
    const int xcd = b & 7, local = b >> 3;
    const int q = total >> 3, rem = total & 7;
    return xcd * q + min(xcd, rem) + local;
}

// s_start: __shared__ int[E+1] scratch. Returns false if block b has no work.
template <int BM, int NTHREADS>
__device__ bool schedule_tile(const int *__restrict__ offsets, int E, int NT, int b, int *s_start,
                              Tile &tile) {
    scan_row_tiles<BM, NTHREADS>(offsets, E, s_start);
    const int total = s_start[E] * NT;
    if (b >= total) return false;
    const int lam = xcd_item(b, total);
    // find expert: largest e with s_start[e] * NT <= lam
    int lo = 0, hi = E;  // invariant: s_start[lo]*NT <= lam < s_start[hi]*NT
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_start[mid] * NT <= lam) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int mte = s_start[e + 1] - s_start[e];
    const int rem2 = lam - s_start[e] * NT;
    tile.e = e;
    tile.nt = rem2 / mte;
    tile.mt = rem2 % mte;
    tile.row0 = offsets[e] + tile.mt * BM;
    tile.rows = min(BM, offsets[e + 1] - tile.row0);
    tile.gmt = s_start[e] + tile.mt;
    // the same in every lane; say so, so that buffer descriptors built from
    // them stay in scalar registers (else the compiler wraps every load
    // using them in a loop over lanes)
    tile.e = __builtin_amdgcn_readfirstlane(tile.e);
    tile.nt = __builtin_amdgcn_readfirstlane(tile.nt);
    tile.mt = __builtin_amdgcn_readfirstlane(tile.mt);
    tile.row0 = __builtin_amdgcn_readfirstlane(tile.row0);
    tile.rows = __builtin_amdgcn_readfirstlane(tile.rows);
    tile.gmt = __builtin_amdgcn_readfirstlane(tile.gmt);
    return true;
}

// ---------------------------------------------------------------------------
// Row-tile table of the grouped GEMMs (kRowTile-row tiles), int4 entries:
// entry 0 = {number of row tiles, 0, 0, 0}; entry 1 + g, g a row tile over
// all experts in expert order, = {its expert e, e's first row tile, e's
// first row, e's row count}; capacity 1 + max_row_tiles(S, E, kRowTile).
// Built once per pass by block 0 of the pass's first kernel, so that each
// GEMM block finds its work item with two table loads instead of rescanning
// the counts.
template <int NTHREADS>
__device__ void build_row_tiles(const int *__restrict__ offsets, int E, int *s_start, int32_t *table) {
    scan_row_tiles<kRowTile, NTHREADS>(offsets, E, s_start);
    int4 *t4 = reinterpret_cast<int4 *>(table);
    for (int e = threadIdx.x; e < E; e += NTHREADS) {
        const int o = offsets[e], n = offsets[e + 1] - o;
        for (int g = s_start[e]; g < s_start[e + 1]; ++g) t4[1 + g] = make_int4(e, s_start[e], o, n);
    }
    if (threadIdx.x == 0) t4[0] = make_int4(s_start[E], 0, 0, 0);
    __syncthreads();  // s_start is reused by the caller
}

// Work items that each XCD's first blocks run as two 128-row halves. At the
// large workloads nearly every tile costs the same (experts hold 1.8-2.2
// tiles of rows), so all CUs would reach their epilogues - VALU-bound SwiGLU
// math and a burst of output stores - together, tile after tile. Running the
// first kPhaseSplit items of each XCD as halves on 2 kPhaseSplit of its 32
// CUs puts those CUs half a tile out of phase with the rest for the whole
// launch (measured: gate/up 2%, down backward 3% faster). Launch grids
// carry kPhaseSplitBlocks extra blocks for the halves.
constexpr int kPhaseSplit = 8;
constexpr int kPhaseSplitBlocks = 8 * (kPhaseSplit + 1);

// The work item of block b, ordered as schedule_tile<kRowTile> orders them,
// from the table. Expert e owns items [s*NT, (s+mte)*NT), s its first row
// tile, so the item lam belongs to the expert of row tile lam / NT. Each XCD
// (block b on XCD b mod 8) takes a contiguous range of items; its local
// blocks 0 .. 2 sp - 1 run the range's first sp items as halves (the second
// half of an item of at most 128 rows has no work).
__device__ __forceinline__ bool table_tile(const int32_t *__restrict__ table, int NT, int b, Tile &tile) {
    const int total = __builtin_amdgcn_readfirstlane(table[0]) * NT;
    const int xcd = b & 7, l = b >> 3;
    const int q = total >> 3, rem = total & 7;
    const int nx = q + (xcd < rem ? 1 : 0), start = xcd * q + min(xcd, rem);
    const int sp = min(kPhaseSplit, nx);
    int li, half = -1;
    if (l < 2 * sp) {
        li = l >> 1;
        half = l & 1;
    } else {
        li = l - sp;
        if (li >= nx) return false;
    }
    const int lam = start + li;
    const int4 te = reinterpret_cast<const int4 *>(table)[1 + lam / NT];
    const int e = __builtin_amdgcn_readfirstlane(te.x);
    const int s = __builtin_amdgcn_readfirstlane(te.y);
    const int off = __builtin_amdgcn_readfirstlane(te.z);
    const int n = __builtin_amdgcn_readfirstlane(te.w);
    const int mte = (n + kRowTile - 1) / kRowTile;
    const int rem2 = lam - s * NT;
    tile.e = e;
    tile.nt = rem2 / mte;
    tile.mt = rem2 - tile.nt * mte;
    tile.row0 = off + tile.mt * kRowTile;
    tile.rows = min(kRowTile, n - tile.mt * kRowTile);
    tile.gmt = s + tile.mt;
    if (half >= 0) {
        if (tile.rows <= kRowTile / 2) {
            if (half) return false;
        } else {
            tile.row0 += half * (kRowTile / 2);
            tile.rows = min(kRowTile / 2, tile.rows - half * (kRowTile / 2));
        }
    }
    return true;
}

}  // namespace moe
