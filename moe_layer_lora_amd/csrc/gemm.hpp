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
// Each thread owns PER chunks of the tile (chunk c -> row c / CPR, k-chunk
// c % CPR, so 8 consecutive lanes fill 128 contiguous bytes of one row).
// A row is addressed as base[sel] + off, with 32-bit element offsets whose
// top bit picks one of two bases (e.g. gate / up weights); a row whose bit in
// `valid` is clear reads as zeros.
// Segment 0: rows of T with K0 elements.
// Segment 1: rows of float32 on k in [0, K1), multiplied by `scale1` and
// rounded to T (SEG1_F32), or rows of T valid on k in [wlo[sel], wlo[sel] + wwidth).
constexpr uint32_t kSel = 0x80000000u;

template <class Cfg, int ROWS, bool SEG1_F32>
struct KLoader {
    using T = typename Cfg::T;
    static constexpr int VEC = Cfg::VEC, CPR = Cfg::CPR, NT = Cfg::NTHREADS, BK = Cfg::BK;
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int PER = (CHUNKS + NT - 1) / NT;
    static_assert(PER <= 32, "valid masks are 32 bits");

    const T *b0[2];
    const void *b1[2];
    uint32_t off0[PER], off1[PER];
    uint32_t valid0 = 0, valid1 = 0;
    int K0 = 0, K1 = 0, nk0 = 0, wwidth = 0;
    int wlo[2] = {0, 0};
    float scale1 = 1.0f;

    struct Regs { chunk_t c[PER]; };

    __device__ KLoader() {
#pragma unroll
        for (int i = 0; i < PER; ++i) off0[i] = off1[i] = 0u;
    }

    __device__ static int chunk(int i) { return (int)threadIdx.x + i * NT; }
    __device__ static bool active(int i) { return chunk(i) < CHUNKS; }
    __device__ static int row_of(int i) { return chunk(i) / CPR; }
    __device__ static int kc_of(int i) { return chunk(i) % CPR; }

    __device__ void set0(int i, uint32_t off, int sel) {
        off0[i] = off | (sel ? kSel : 0u);
        valid0 |= 1u << i;
    }
    __device__ void set1(int i, uint32_t off, int sel) {
        off1[i] = off | (sel ? kSel : 0u);
        valid1 |= 1u << i;
    }

    // Branch-free: every lane loads from a real address (the segment base when
    // its row or k is out of range) and zeroes the value afterwards.
    __device__ __forceinline__ void load(int kt, Regs &r) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (!active(i)) continue;
            const int kc = kc_of(i);
            if (kt < nk0) {
                const int k = kt * BK + kc * VEC;
                const bool ok = ((valid0 >> i) & 1u) && k < K0;
                const T *src = ok ? ((off0[i] & kSel) ? b0[1] : b0[0]) + (off0[i] & ~kSel) + k : b0[0];
                const chunk_t v = *reinterpret_cast<const chunk_t *>(src);
                r.c[i] = ok ? v : zero4();
            } else {
                const int k = (kt - nk0) * BK + kc * VEC;
                const bool sel = (off1[i] & kSel) != 0;  // selects, not indexing: keeps b1 in registers
                const uint32_t o = off1[i] & ~kSel;
                if constexpr (SEG1_F32) {
                    const bool ok = ((valid1 >> i) & 1u) && k < K1;
                    const float4 *src = reinterpret_cast<const float4 *>(
                        ok ? static_cast<const float *>(sel ? b1[1] : b1[0]) + o + k
                           : static_cast<const float *>(b1[0]));
                    float v[VEC];
#pragma unroll
                    for (int h = 0; h < VEC / 4; ++h) {
                        const float4 f = src[h];
                        v[4 * h + 0] = ok ? f.x * scale1 : 0.0f;
                        v[4 * h + 1] = ok ? f.y * scale1 : 0.0f;
                        v[4 * h + 2] = ok ? f.z * scale1 : 0.0f;
                        v[4 * h + 3] = ok ? f.w * scale1 : 0.0f;
                    }
                    r.c[i] = Elem<T>::pack(v);
                } else {
                    const int kl = k - (sel ? wlo[1] : wlo[0]);
                    const bool ok = ((valid1 >> i) & 1u) && kl >= 0 && kl + VEC <= wwidth;
                    const T *src = ok ? static_cast<const T *>(sel ? b1[1] : b1[0]) + o + kl
                                      : static_cast<const T *>(b1[0]);
                    const chunk_t v = *reinterpret_cast<const chunk_t *>(src);
                    r.c[i] = ok ? v : zero4();
                }
            }
        }
    }

    __device__ __forceinline__ void store(const Regs &r, T *lds) const {
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
// transpose (VEC n-rows of 16 bytes). Consecutive lanes take consecutive k
// blocks of one n block, so the 16-byte LDS writes of 8 lanes fill one
// padded LDS row segment (no bank conflicts) and, per k-row, 8 lanes with
// consecutive n blocks read 128 contiguous bytes. Each K segment is up to two matrices
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

    __device__ __forceinline__ void load(int kt, Regs &r) const {
        const bool first = kt < nk0;
        // pick the segment field by field (a reference would force the
        // structs into scratch memory)
        NSeg sg;
        sg.a = first ? s0.a : s1.a;
        sg.b = first ? s0.b : s1.b;
        sg.split = first ? s0.split : s1.split;
        sg.K = first ? s0.K : s1.K;
        sg.ld = first ? s0.ld : s1.ld;
        sg.a_clo = first ? s0.a_clo : s1.a_clo;
        sg.a_chi = first ? s0.a_chi : s1.a_chi;
        sg.b_clo = first ? s0.b_clo : s1.b_clo;
        sg.b_chi = first ? s0.b_chi : s1.b_chi;
        const int kt0 = (first ? kt : kt - nk0) * BK;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            if (b >= NBLK) continue;
            const int kb = b % KB, nb = b / KB;
            const int n = nb * VEC;
#pragma unroll
            for (int ii = 0; ii < VEC; ++ii) {
                const int k = kt0 + kb * VEC + ii;
                const bool in_a = k < sg.split;
                const bool ok = k < sg.K && (in_a ? (sg.a && n >= sg.a_clo && n + VEC <= sg.a_chi)
                                                  : (sg.b && n >= sg.b_clo && n + VEC <= sg.b_chi));
                const T *src = !ok ? static_cast<const T *>(s0.a)
                               : in_a ? static_cast<const T *>(sg.a) + (size_t)k * sg.ld + (n - sg.a_clo)
                                      : static_cast<const T *>(sg.b) + (size_t)(k - sg.split) * sg.ld + (n - sg.b_clo);
                const chunk_t v = *reinterpret_cast<const chunk_t *>(src);
                r.c[i][ii] = ok ? v : zero4();
            }
        }
    }

    __device__ __forceinline__ void store(const Regs &r, T *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            if (b >= NBLK) continue;
            const int kb = b % KB, nb = b / KB;
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
// Raw-buffer operand loaders for the steady-state K loop of the large GEMMs.
// A buffer resource carries the base address and byte size of one tensor
// slice; an offset at or beyond the size reads as zero in hardware, which
// handles ragged rows, columns and K without branches or selects on data.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kInvalid = 0x80000000u;  // any offset >= the slice size reads 0

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // dword 3 = 0x00020000: untyped 32-bit data format, as gfx9-family raw buffers expect
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ chunk_t buf_load16(rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(chunk_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// K-contiguous tile of ROWS rows. Steady-state tiles come from up to two K
// segments (uniform per tile): segment s reads k in [0, K[s]) at column base
// col[s] of the rows, through descriptor rs[s][sel]. With ALT32 the rows
// alternate between descriptor 0 and 1 in blocks of 32 tile rows (gate / up
// weights); every lane's chunk i then lies in the same block, so sel is a
// compile-time function of i and the descriptors stay scalar. Row byte
// offsets are per chunk; rows outside the tile hold kInvalid.
template <class Cfg, int ROWS, bool ALT32 = false>
struct BufKLoader {
    using T = typename Cfg::T;
    static constexpr int VEC = Cfg::VEC, CPR = Cfg::CPR, NT = Cfg::NTHREADS, BK = Cfg::BK;
    static constexpr int PER = ROWS * CPR / NT;
    static_assert(ROWS * CPR % NT == 0, "whole chunks per thread");
    static_assert(!ALT32 || NT / CPR == 32, "ALT32 needs 32 tile rows per chunk index");
    rsrc_t rs[2][2];
    uint32_t off[PER];
    int K[2] = {0, 0}, col[2] = {0, 0};
    int nt0 = 0;  // tiles of segment 0

    struct Regs { chunk_t c[PER]; };
    __device__ static int row_of(int i) { return ((int)threadIdx.x + i * NT) / CPR; }
    __device__ static int kc_of(int i) { return ((int)threadIdx.x + i * NT) % CPR; }
    static constexpr bool sel_of(int i) { return ALT32 && (i & 1); }

    __device__ __forceinline__ void load(int t, Regs &r) const {
        const bool s1 = t >= nt0;
        const int kt = s1 ? t - nt0 : t;
        const int Ks = s1 ? K[1] : K[0];
        const uint32_t cb = (uint32_t)(s1 ? col[1] : col[0]) * sizeof(T);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int k = kt * BK + kc_of(i) * VEC;
            const bool ok = off[i] != kInvalid && k < Ks;
            const uint32_t vo = ok ? off[i] + cb + (uint32_t)k * sizeof(T) : kInvalid;
            const rsrc_t d = s1 ? (sel_of(i) ? rs[1][1] : rs[1][0]) : (sel_of(i) ? rs[0][1] : rs[0][0]);
            r.c[i] = buf_load16(d, vo);
        }
    }
    __device__ __forceinline__ void store(const Regs &r, T *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            *reinterpret_cast<chunk_t *>(lds + row_of(i) * Cfg::LDK + kc_of(i) * VEC) = r.c[i];
    }
};

// N-contiguous (transposed) tile of ROWS n-rows: element (k, n) of segment s
// at byte (k * ld[s] + n) * sizeof(T) of descriptor rs[s], valid for
// k < K[s] and n < ncol. Thread b loads the VEC x VEC block (kb = b % KB,
// nb = b / KB) and writes its transpose.
template <class Cfg, int ROWS>
struct BufNLoader {
    using T = typename Cfg::T;
    static constexpr int VEC = Cfg::VEC, NT = Cfg::NTHREADS, BK = Cfg::BK;
    static constexpr int KB = BK / VEC, NB = ROWS / VEC, NBLK = KB * NB;
    static constexpr int PER = NBLK / NT;
    static_assert(NBLK % NT == 0, "whole blocks per thread");
    rsrc_t rs[2];
    int K[2] = {0, 0}, ld[2] = {0, 0};
    int ncol = 0, nt0 = 0;

    struct Regs { chunk_t c[PER][VEC]; };
    __device__ static int kb_of(int i) { return ((int)threadIdx.x + i * NT) % KB; }
    __device__ static int nb_of(int i) { return ((int)threadIdx.x + i * NT) / KB; }

    __device__ __forceinline__ void load(int t, Regs &r) const {
        const bool s1 = t >= nt0;
        const int kt = s1 ? t - nt0 : t;
        const int Ks = s1 ? K[1] : K[0];
        const uint32_t ldb = (uint32_t)(s1 ? ld[1] : ld[0]) * sizeof(T);
        const rsrc_t d = s1 ? rs[1] : rs[0];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int n = nb_of(i) * VEC;
            const bool nok = n + VEC <= ncol;
#pragma unroll
            for (int ii = 0; ii < VEC; ++ii) {
                const int k = kt * BK + kb_of(i) * VEC + ii;
                const uint32_t vo = (nok && k < Ks) ? (uint32_t)k * ldb + (uint32_t)n * sizeof(T) : kInvalid;
                r.c[i][ii] = buf_load16(d, vo);
            }
        }
    }
    __device__ __forceinline__ void store(const Regs &r, T *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            chunk_t o[VEC];
            NLoader<Cfg, ROWS>::transpose(r.c[i], o);
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj)
                *reinterpret_cast<chunk_t *>(lds + (nb_of(i) * VEC + jj) * Cfg::LDK + kb_of(i) * VEC) = o[jj];
        }
    }
};

// ---------------------------------------------------------------------------
// One BK slice of MFMA work from LDS.
template <class Cfg>
__device__ __forceinline__ void mma_tile(const typename Cfg::T *sA, const typename Cfg::T *sB,
                                         f32x16_t (&acc)[Cfg::TM][Cfg::TN]) {
    using T = typename Cfg::T;
    constexpr int NKG = Cfg::BK / Cfg::KG;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const T *a_base = sA + (wm * Cfg::WTM + (lane & 31)) * Cfg::LDK + (lane >> 5) * Cfg::VEC;
    const T *b_base = sB + (wn * Cfg::WTN + (lane & 31)) * Cfg::LDK + (lane >> 5) * Cfg::VEC;
    // fragments of k-group kg+1 are read while k-group kg is multiplied;
    // the fences keep the compiler from hoisting further reads (registers)
    chunk_t af[2][Cfg::TM], bfr[2][Cfg::TN];
#pragma unroll
    for (int mi = 0; mi < Cfg::TM; ++mi) af[0][mi] = *reinterpret_cast<const chunk_t *>(a_base + mi * 32 * Cfg::LDK);
#pragma unroll
    for (int ni = 0; ni < Cfg::TN; ++ni) bfr[0][ni] = *reinterpret_cast<const chunk_t *>(b_base + ni * 32 * Cfg::LDK);
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
        const int c = kg & 1;
        if (kg + 1 < NKG) {
#pragma unroll
            for (int mi = 0; mi < Cfg::TM; ++mi)
                af[c ^ 1][mi] = *reinterpret_cast<const chunk_t *>(a_base + mi * 32 * Cfg::LDK + (kg + 1) * Cfg::KG);
#pragma unroll
            for (int ni = 0; ni < Cfg::TN; ++ni)
                bfr[c ^ 1][ni] = *reinterpret_cast<const chunk_t *>(b_base + ni * 32 * Cfg::LDK + (kg + 1) * Cfg::KG);
        }
#pragma unroll
        for (int mi = 0; mi < Cfg::TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < Cfg::TN; ++ni)
                Elem<T>::mma(acc[mi][ni], af[c][mi], bfr[c][ni]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Double-buffered main loop over nk K-tiles: the next tile's global loads are
// in flight while the current tile is multiplied out of LDS.
template <class Cfg, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(const LA &la, const LB &lb, int nk, typename Cfg::T *sA,
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

// Pipelined K loop over nt steady-state tiles (loaders SA, SB), preceded by
// one rank-r LoRA tile from loaders PA, PB when `lora` is set: the LoRA
// expansion adds into the same accumulators as the base product. Two LDS
// stages; the next tile's global loads are in flight while the current one
// is multiplied.
template <class Cfg, class SA, class SB, class PA, class PB>
__device__ __forceinline__ void gemm_pipeline(const SA &sa, const SB &sb, int nt, const PA &pa, const PB &pb, int nlora,
                              typename Cfg::T *sA, typename Cfg::T *sB, f32x16_t (&acc)[Cfg::TM][Cfg::TN]) {
#pragma unroll
    for (int mi = 0; mi < Cfg::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < Cfg::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;
    typename SA::Regs ra;
    typename SB::Regs rb;
    int t = 0;
    if (nlora > 0) {
        typename PA::Regs pra;
        typename PB::Regs prb;
        // LoRA tiles beyond the first (rank above BK / 2): one at a time
        for (int lt = 0; lt + 1 < nlora; ++lt) {
            pa.load(lt, pra);
            pb.load(lt, prb);
            pa.store(pra, sA);
            pb.store(prb, sB);
            __syncthreads();
            mma_tile<Cfg>(sA, sB, acc);
            __syncthreads();
        }
        pa.load(nlora - 1, pra);
        pb.load(nlora - 1, prb);
        pa.store(pra, sA);
        pb.store(prb, sB);
        t = -1;  // the LoRA tile sits in stage 0 ahead of steady tile 0
    } else {
        if (nt <= 0) return;
        sa.load(0, ra);
        sb.load(0, rb);
        sa.store(ra, sA);
        sb.store(rb, sB);
    }
    __syncthreads();
    int cur = 0;
    for (; t < nt; ++t) {
        const bool more = t + 1 < nt;
        if (more) {
            sa.load(t + 1, ra);
            sb.load(t + 1, rb);
        }
        mma_tile<Cfg>(sA + cur * Cfg::A_ELEMS, sB + cur * Cfg::B_ELEMS, acc);
        if (more) {
            sa.store(ra, sA + (cur ^ 1) * Cfg::A_ELEMS);
            sb.store(rb, sB + (cur ^ 1) * Cfg::B_ELEMS);
        }
        __syncthreads();
        cur ^= 1;
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
