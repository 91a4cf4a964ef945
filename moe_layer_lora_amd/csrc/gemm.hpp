// gemm.hpp - LDS-staged MFMA tile engine for the grouped GEMMs.
//
// A workgroup computes a BM x BN tile of C = A * B^T where both operands are
// staged in LDS "K-contiguous": LDS row i of the A tile holds A[m0+i][k..k+BK)
// and LDS row j of the B tile holds B[n0+j][k..k+BK). Each wave owns a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles.
//
// The K dimension is the concatenation of two segments. Segment 0 is the
// main contraction (x W^T and friends); segment 1 is the rank-r LoRA
// expansion s * Z B^T, so that  C = [A0 | s Z] [W | B]^T  adds the LoRA term
// in the same accumulators after the base product: the Split-LoRA order,
// with W + s B A never formed.
#pragma once

#include "common.hpp"

namespace moe {

template <typename T_, int BM_, int BN_, int BK_, int WM_, int WN_>
struct GemmCfg {
    using T = T_;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NTHREADS = WM * WN * kWave;
    static constexpr int VEC = Elem<T>::VEC;   // elements per 16-byte chunk
    static constexpr int KG = 2 * VEC;         // k per MFMA group
    static constexpr int LDK = BK + VEC;       // LDS row pitch (one chunk of padding)
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int CPR = BK / VEC;       // chunks per LDS row
    static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
    static_assert(BK % KG == 0, "BK must hold whole MFMA k-groups");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
};

__device__ __forceinline__ chunk_t zero4() { return chunk_t{0u, 0u, 0u, 0u}; }

// ---------------------------------------------------------------------------
// K-contiguous operand loader for a tile of ROWS rows.
// Segment 0: rows of T with K0 elements (row pointer, or nullptr for a zero row).
// Segment 1: either rows of T valid on k in [klo, khi) (SEG1_F32 = false), or
// rows of float32 valid on [0, K1), multiplied by `scale1` and rounded to T.
template <class Cfg, int ROWS, bool SEG1_F32>
struct KLoader {
    using T = typename Cfg::T;
    static constexpr int VEC = Cfg::VEC, CPR = Cfg::CPR, NT = Cfg::NTHREADS, BK = Cfg::BK;
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int PER = (CHUNKS + NT - 1) / NT;

    const T *p0[PER];
    const void *p1[PER];
    int klo1[PER], khi1[PER];
    int K0, K1, nk0;
    float scale1;

    struct Regs { chunk_t c[PER]; };

    __device__ static int chunk(int i) { return (int)threadIdx.x + i * NT; }
    __device__ static bool active(int i) { return chunk(i) < CHUNKS; }
    __device__ static int row_of(int i) { return chunk(i) / CPR; }
    __device__ static int kc_of(int i) { return chunk(i) % CPR; }

    __device__ void load(int kt, Regs &r) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (!active(i)) continue;
            const int kc = kc_of(i);
            if (kt < nk0) {
                const int k = kt * BK + kc * VEC;
                r.c[i] = (p0[i] && k < K0) ? *reinterpret_cast<const chunk_t *>(p0[i] + k) : zero4();
            } else {
                const int k = (kt - nk0) * BK + kc * VEC;
                if constexpr (SEG1_F32) {
                    float v[VEC];
                    if (p1[i] && k < K1) {
                        const float4 *src = reinterpret_cast<const float4 *>(
                            static_cast<const float *>(p1[i]) + k);
#pragma unroll
                        for (int h = 0; h < VEC / 4; ++h) {
                            const float4 f = src[h];
                            v[4 * h + 0] = f.x * scale1; v[4 * h + 1] = f.y * scale1;
                            v[4 * h + 2] = f.z * scale1; v[4 * h + 3] = f.w * scale1;
                        }
                    } else {
#pragma unroll
                        for (int h = 0; h < VEC; ++h) v[h] = 0.0f;
                    }
                    r.c[i] = Elem<T>::pack(v);
                } else {
                    r.c[i] = (p1[i] && k >= klo1[i] && k + VEC <= khi1[i])
                                 ? *reinterpret_cast<const chunk_t *>(static_cast<const T *>(p1[i]) + (k - klo1[i]))
                                 : zero4();
                }
            }
        }
    }

    __device__ void store(const Regs &r, T *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (active(i))
                *reinterpret_cast<chunk_t *>(lds + row_of(i) * Cfg::LDK + kc_of(i) * VEC) = r.c[i];
    }
};

// ---------------------------------------------------------------------------
// Transposing loader for an operand stored N-contiguous in memory
// (element (k, n) at row k, column n). The LDS tile is still K-contiguous:
// each thread reads a VEC x VEC block (VEC k-rows of 16 bytes) and writes its
// transpose (VEC n-rows of 16 bytes). Each K segment is up to two matrices
// stacked along k (rows [0, split) from `a`, [split, K) from `b`); each
// matrix covers a window of tile columns [clo, chi) (block-diagonal
// placements), its pointer addressing tile column clo.
struct NSeg {
    const void *a, *b;
    int split, K, ld;
    int a_clo, a_chi, b_clo, b_chi;
};

template <class Cfg, int ROWS>
struct NLoader {
    using T = typename Cfg::T;
    static constexpr int VEC = Cfg::VEC, NT = Cfg::NTHREADS, BK = Cfg::BK;
    static constexpr int KB = BK / VEC, NB = ROWS / VEC, NBLK = KB * NB;
    static constexpr int PER = (NBLK + NT - 1) / NT;

    NSeg s0, s1;
    int nk0;

    struct Regs { chunk_t c[PER][VEC]; };

    __device__ static int blk(int i) { return (int)threadIdx.x + i * NT; }

    __device__ void load(int kt, Regs &r) const {
        const bool first = kt < nk0;
        const NSeg &sg = first ? s0 : s1;
        const int kt0 = (first ? kt : kt - nk0) * BK;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            if (b >= NBLK) continue;
            const int nb = b % NB, kb = b / NB;
            const int n = nb * VEC;
#pragma unroll
            for (int ii = 0; ii < VEC; ++ii) {
                const int k = kt0 + kb * VEC + ii;
                const T *src = nullptr;
                if (k < sg.K) {
                    if (k < sg.split) {
                        if (sg.a && n >= sg.a_clo && n + VEC <= sg.a_chi)
                            src = static_cast<const T *>(sg.a) + (size_t)k * sg.ld + (n - sg.a_clo);
                    } else {
                        if (sg.b && n >= sg.b_clo && n + VEC <= sg.b_chi)
                            src = static_cast<const T *>(sg.b) + (size_t)(k - sg.split) * sg.ld + (n - sg.b_clo);
                    }
                }
                r.c[i][ii] = src ? *reinterpret_cast<const chunk_t *>(src) : zero4();
            }
        }
    }

    __device__ void store(const Regs &r, T *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            if (b >= NBLK) continue;
            const int nb = b % NB, kb = b / NB;
            chunk_t o[VEC];
            transpose(r.c[i], o);
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj)
                *reinterpret_cast<chunk_t *>(lds + (nb * VEC + jj) * Cfg::LDK + kb * VEC) = o[jj];
        }
    }

    // in[ii] = VEC n-values of k-row ii; out[jj] = VEC k-values of n-column jj
    __device__ static void transpose(const chunk_t (&in)[VEC], chunk_t (&out)[VEC]) {
        if constexpr (VEC == 8) {  // 16-bit elements
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                uint32_t w[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t lw = in[2 * v][jj >> 1], hw = in[2 * v + 1][jj >> 1];
                    w[v] = (jj & 1) ? ((lw >> 16) | (hw & 0xffff0000u)) : ((lw & 0xffffu) | (hw << 16));
                }
                out[jj] = chunk_t{w[0], w[1], w[2], w[3]};
            }
        } else {  // 32-bit elements, VEC == 4
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                out[jj] = chunk_t{in[0][jj], in[1][jj], in[2][jj], in[3][jj]};
        }
    }
};

// ---------------------------------------------------------------------------
// One BK slice of MFMA work from LDS.
template <class Cfg>
__device__ __forceinline__ void mma_tile(const typename Cfg::T *sA, const typename Cfg::T *sB,
                                         f32x16_t (&acc)[Cfg::TM][Cfg::TN]) {
    using T = typename Cfg::T;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const T *a_base = sA + (wm * Cfg::WTM + (lane & 31)) * Cfg::LDK + (lane >> 5) * Cfg::VEC;
    const T *b_base = sB + (wn * Cfg::WTN + (lane & 31)) * Cfg::LDK + (lane >> 5) * Cfg::VEC;
#pragma unroll
    for (int kg = 0; kg < Cfg::BK / Cfg::KG; ++kg) {
        chunk_t af[Cfg::TM], bfr[Cfg::TN];
#pragma unroll
        for (int mi = 0; mi < Cfg::TM; ++mi)
            af[mi] = *reinterpret_cast<const chunk_t *>(a_base + mi * 32 * Cfg::LDK + kg * Cfg::KG);
#pragma unroll
        for (int ni = 0; ni < Cfg::TN; ++ni)
            bfr[ni] = *reinterpret_cast<const chunk_t *>(b_base + ni * 32 * Cfg::LDK + kg * Cfg::KG);
#pragma unroll
        for (int mi = 0; mi < Cfg::TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < Cfg::TN; ++ni)
                Elem<T>::mma(acc[mi][ni], af[mi], bfr[ni]);
    }
}

// Double-buffered main loop over nk K-tiles: the next tile's global loads are
// in flight while the current tile is multiplied out of LDS.
template <class Cfg, class LA, class LB>
__device__ void gemm_mainloop(const LA &la, const LB &lb, int nk, typename Cfg::T *sA,
                              typename Cfg::T *sB, f32x16_t (&acc)[Cfg::TM][Cfg::TN]) {
#pragma unroll
    for (int mi = 0; mi < Cfg::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < Cfg::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;
    if (nk <= 0) return;
    typename LA::Regs ra;
    typename LB::Regs rb;
    la.load(0, ra);
    lb.load(0, rb);
    la.store(ra, sA);
    lb.store(rb, sB);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(kt + 1, ra);
            lb.load(kt + 1, rb);
        }
        mma_tile<Cfg>(sA + cur * Cfg::A_ELEMS, sB + cur * Cfg::B_ELEMS, acc);
        if (more) {
            la.store(ra, sA + (cur ^ 1) * Cfg::A_ELEMS);
            lb.store(rb, sB + (cur ^ 1) * Cfg::B_ELEMS);
        }
        __syncthreads();
    }
}

// Visit every accumulator element: f(tile_row, tile_col, mi, ni, i, value).
template <class Cfg, class Fn>
__device__ __forceinline__ void for_each_acc(const f32x16_t (&acc)[Cfg::TM][Cfg::TN], Fn &&f) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
#pragma unroll
    for (int mi = 0; mi < Cfg::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < Cfg::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                f(wm * Cfg::WTM + mi * 32 + acc_row(i, lane), wn * Cfg::WTN + ni * 32 + acc_col(lane), mi,
                  ni, i, acc[mi][ni][i]);
}

}  // namespace moe
