// layer.hip - expert-layer kernels on gfx950: grouped GEMMs with Split-LoRA,
// SwiGLU epilogues, combines, router-weight gradient and LoRA weight
// gradients, plus the forward / backward drivers.
//
// All experts run in ONE launch per projection (the grouped_mm form of the
// Unsloth 2026 wiki chapter, "Optimisation 3: grouped_mm and Split-LoRA in
// MoE training"): a block picks an (expert, row tile, column tile) from the
// device-side offsets, so no per-expert launch and no host sync exist.
// Split-LoRA (same chapter, Split-LoRA subsection): each projection runs the
// frozen W first and adds s * (x A^T) B^T as a second K segment of the same
// accumulation; W + s B A is never formed.
#include "kernels.hpp"
#include "gemm.hpp"
#include "gemm_lds.hpp"
#include "moe.h"

#include <algorithm>
#include <type_traits>

namespace moe {

constexpr int kMaxE = 1024;

// The large tiles hold a 128x128 fp32 accumulator per wave (256 registers):
// one wave per SIMD, so the full 512-entry register file (256 VGPR + 256
// AGPR) is available to it.
#define MOE_ONE_WAVE_PER_SIMD __attribute__((amdgpu_waves_per_eu(1, 1)))
// ring-engine kernels: C::NWAVES waves per block, one block per CU (the ring
// fills the LDS), so C::NWAVES / 4 waves on each SIMD
#define MOE_LDS_BLOCK(C) __launch_bounds__(C::NTHREADS) __attribute__((amdgpu_waves_per_eu(C::NWAVES / 4, C::NWAVES / 4)))

// Main grouped-GEMM tile shapes.
template <typename T> struct MainCfg;
template <> struct MainCfg<bf16_t> { using type = GemmCfg<bf16_t, 128, 128, 32, 2, 2>; };  // (bf16 runs the LDS-ring kernels)
template <> struct MainCfg<float> { using type = GemmCfg<float, 128, 128, 32, 2, 2>; };
// Skinny projections (N = r or 2r) and LoRA weight gradients (N = r or 2r).
template <typename T, int BN> struct SkinnyCfg;
template <int BN> struct SkinnyCfg<bf16_t, BN> { using type = GemmCfg<bf16_t, 128, BN, 32, 4 / (BN / 32), BN / 32>; };
template <int BN> struct SkinnyCfg<float, BN> { using type = GemmCfg<float, 128, BN, 16, 4 / (BN / 32), BN / 32>; };

template <class Cfg> struct Smem {
    __align__(16) typename Cfg::T a[2 * Cfg::A_ELEMS];
    __align__(16) typename Cfg::T b[2 * Cfg::B_ELEMS];
    int start[kMaxE + 1];
};

__device__ __forceinline__ int token_of(const int32_t *sorted_slot, int p, int k) { return sorted_slot[p] / k; }

// ===========================================================================
// Gate/up grouped GEMM: G = Xp W_g^T + s Zg B_g^T, U likewise, H = silu(G) U.
// The B tile interleaves 32-column blocks of gate and up rows for the same f,
// so each lane holds g and u of one element and the SwiGLU is fused.
// ===========================================================================
struct GateUpP {
    const void *x, *wg, *wu, *bg, *bu;
    const float *zgu;
    const int32_t *sorted_slot, *offsets;
    void *G, *U, *H;
    int T, E, k, d, F, r;
    float s;
    const int32_t *tiles;  // bf16 path: row-tile table (build_row_tiles)
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS) MOE_ONE_WAVE_PER_SIMD void k_gateup(GateUpP p) {
    using T = typename Cfg::T;
    static_assert(std::is_same<T, float>::value, "fp32 layers (bf16 gate/up runs on the LDS ring)");
    __shared__ Smem<Cfg> sm;
    constexpr int HALF = Cfg::BN / 2;
    static_assert(Cfg::TN % 2 == 0, "gate/up pairs");
    static_assert(Cfg::NTHREADS / Cfg::CPR == 32, "one 32-row gate or up block per chunk index");
    Tile tl;
    if (!schedule_tile<Cfg::BM, Cfg::NTHREADS>(p.offsets, p.E, cdiv(p.F, HALF), blockIdx.x, sm.start, tl)) return;
    const int f_base = tl.nt * HALF;

    // steady state: x rows (gathered by token) against W_gate / W_up rows
    BufKLoader<Cfg, Cfg::BM> sa;
    sa.rs[0][0] = sa.rs[0][1] = make_rsrc(p.x, (uint32_t)p.T * p.d * sizeof(T));
    sa.K[0] = p.d; sa.nt0 = cdiv(p.d, Cfg::BK);
#pragma unroll
    for (int i = 0; i < sa.PER; ++i) {
        const int m = sa.row_of(i);
        sa.off[i] = m < tl.rows ? (uint32_t)token_of(p.sorted_slot, tl.row0 + m, p.k) * p.d * sizeof(T) : kInvalid;
    }
    BufKLoader<Cfg, Cfg::BN, true> sb;
    const size_t wofs = (size_t)tl.e * p.F * p.d;
    sb.rs[0][0] = make_rsrc(static_cast<const T *>(p.wg) + wofs, (uint32_t)p.F * p.d * sizeof(T));
    sb.rs[0][1] = make_rsrc(static_cast<const T *>(p.wu) + wofs, (uint32_t)p.F * p.d * sizeof(T));
    sb.K[0] = p.d; sb.nt0 = sa.nt0;
#pragma unroll
    for (int i = 0; i < sb.PER; ++i) {
        const int n = sb.row_of(i);
        const int wn = n / Cfg::WTN, ni = (n % Cfg::WTN) / 32;
        const int f = f_base + wn * (Cfg::WTN / 2) + (ni / 2) * 32 + (n % 32);
        sb.off[i] = f < p.F ? (uint32_t)f * p.d * sizeof(T) : kInvalid;
    }
    // LoRA tile: [s Zg | s Zu] rows against [B_g | 0] (gate rows) and [0 | B_u] (up rows)
    KLoader<Cfg, Cfg::BM, true> la;
    la.K1 = 2 * p.r; la.nk0 = 0; la.scale1 = p.s;
    la.b1[0] = la.b1[1] = p.zgu;
#pragma unroll
    for (int i = 0; i < la.PER; ++i) {
        const int m = la.row_of(i);
        if (la.active(i) && m < tl.rows) la.set1(i, (uint32_t)(tl.row0 + m) * 2 * p.r, 0);
    }
    KLoader<Cfg, Cfg::BN, false> lb;
    lb.K1 = 2 * p.r; lb.nk0 = 0;
    lb.b1[0] = static_cast<const T *>(p.bg) + (size_t)tl.e * p.F * p.r;
    lb.b1[1] = static_cast<const T *>(p.bu) + (size_t)tl.e * p.F * p.r;
    lb.wlo[0] = 0; lb.wlo[1] = p.r; lb.wwidth = p.r;
#pragma unroll
    for (int i = 0; i < lb.PER; ++i) {
        const int n = lb.row_of(i);
        const int wn = n / Cfg::WTN, ni = (n % Cfg::WTN) / 32;
        const int f = f_base + wn * (Cfg::WTN / 2) + (ni / 2) * 32 + (n % 32);
        if (lb.active(i) && f < p.F) lb.set1(i, (uint32_t)f * p.r, ni & 1);
    }
    f32x16_t acc[Cfg::TM][Cfg::TN];
    gemm_pipeline<Cfg>(sa, sb, sa.nt0, la, lb, cdiv(2 * p.r, Cfg::BK), sm.a, sm.b, acc);

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    T *G = static_cast<T *>(p.G), *U = static_cast<T *>(p.U), *H = static_cast<T *>(p.H);
#pragma unroll
    for (int mi = 0; mi < Cfg::TM; ++mi)
#pragma unroll
        for (int c = 0; c < Cfg::TN / 2; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = wm * Cfg::WTM + mi * 32 + acc_row(i, lane);
                const int f = f_base + wn * (Cfg::WTN / 2) + c * 32 + acc_col(lane);
                if (m < tl.rows && f < p.F) {
                    const float g = acc[mi][2 * c][i], u = acc[mi][2 * c + 1][i];
                    const size_t o = (size_t)(tl.row0 + m) * p.F + f;
                    if (G) G[o] = g;
                    if (U) U[o] = u;
                    H[o] = swiglu_ieee(g, u);
                }
            }
}

// ===========================================================================
// Down grouped GEMM: Y = H W_d^T + s Zd B_d^T.
// ===========================================================================
struct DownP {
    const void *H, *wd, *bd;
    const float *zd;
    const int32_t *offsets;
    void *Y;
    int S, E, d, F, r;
    float s;
    const int32_t *tiles;  // bf16 path: row-tile table (build_row_tiles)
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS) MOE_ONE_WAVE_PER_SIMD void k_down(DownP p) {
    using T = typename Cfg::T;
    __shared__ Smem<Cfg> sm;
    Tile tl;
    if (!schedule_tile<Cfg::BM, Cfg::NTHREADS>(p.offsets, p.E, cdiv(p.d, Cfg::BN), blockIdx.x, sm.start, tl)) return;
    const int n_base = tl.nt * Cfg::BN;
    BufKLoader<Cfg, Cfg::BM> sa;
    sa.rs[0][0] = sa.rs[0][1] = make_rsrc(p.H, (uint32_t)p.S * p.F * sizeof(T));
    sa.K[0] = p.F; sa.nt0 = cdiv(p.F, Cfg::BK);
#pragma unroll
    for (int i = 0; i < sa.PER; ++i) {
        const int m = sa.row_of(i);
        sa.off[i] = m < tl.rows ? (uint32_t)(tl.row0 + m) * p.F * sizeof(T) : kInvalid;
    }
    BufKLoader<Cfg, Cfg::BN> sb;
    sb.rs[0][0] = sb.rs[0][1] = make_rsrc(static_cast<const T *>(p.wd) + (size_t)tl.e * p.d * p.F,
                                          (uint32_t)p.d * p.F * sizeof(T));
    sb.K[0] = p.F; sb.nt0 = sa.nt0;
#pragma unroll
    for (int i = 0; i < sb.PER; ++i) {
        const int n = n_base + sb.row_of(i);
        sb.off[i] = n < p.d ? (uint32_t)n * p.F * sizeof(T) : kInvalid;
    }
    KLoader<Cfg, Cfg::BM, true> la;
    la.K1 = p.r; la.nk0 = 0; la.scale1 = p.s;
    la.b1[0] = la.b1[1] = p.zd;
#pragma unroll
    for (int i = 0; i < la.PER; ++i) {
        const int m = la.row_of(i);
        if (la.active(i) && m < tl.rows) la.set1(i, (uint32_t)(tl.row0 + m) * p.r, 0);
    }
    KLoader<Cfg, Cfg::BN, false> lb;
    lb.K1 = p.r; lb.nk0 = 0; lb.wwidth = p.r;
    lb.b1[0] = lb.b1[1] = static_cast<const T *>(p.bd) + (size_t)tl.e * p.d * p.r;
#pragma unroll
    for (int i = 0; i < lb.PER; ++i) {
        const int n = n_base + lb.row_of(i);
        if (lb.active(i) && n < p.d) lb.set1(i, (uint32_t)n * p.r, 0);
    }
    f32x16_t acc[Cfg::TM][Cfg::TN];
    gemm_pipeline<Cfg>(sa, sb, sa.nt0, la, lb, cdiv(p.r, Cfg::BK), sm.a, sm.b, acc);
    T *Y = static_cast<T *>(p.Y);
    for_each_acc<Cfg>(acc, [&](int m, int n, int, int, int, float v) {
        if (m < tl.rows && n_base + n < p.d) Y[(size_t)(tl.row0 + m) * p.d + n_base + n] = Elem<T>::from_f32(v);
    });
}

// ===========================================================================
// Down backward: dH = w * (dout W_d + s P'd A_d), with P'd = dout B_d, then
// the SwiGLU backward  dG = dH u sig(g) (1 + g (1 - sig(g))),  dU = dH silu(g).
// The row scale w (combine weight of the slot) is applied in the epilogue.
// ===========================================================================
struct DownBwdP {
    const void *dout, *wd, *ad, *G, *U;
    const float *pd, *topk_w;
    const int32_t *sorted_slot, *offsets;
    void *dGU;
    int T, E, k, d, F, r;
    float s;
    const float *w_row;  // bf16 path: combine weight of each row p (topk_w[sorted_slot[p]])
    const int32_t *tiles;  // bf16 path: row-tile table (build_row_tiles)
    // bf16 path with r in {16, 32}: the epilogue also projects the tile's dG,
    // dU onto B_g, B_u; ppart [cdiv(F, 256), S, 2r] fp32 gets each column
    // strip's share of Pgu = [dG B_g | dU B_u] (k_pgu_sum adds them up)
    const void *bg, *bu;
    float *ppart;
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS) MOE_ONE_WAVE_PER_SIMD void k_down_bwd(DownBwdP p) {
    using T = typename Cfg::T;
    __shared__ Smem<Cfg> sm;
    Tile tl;
    if (!schedule_tile<Cfg::BM, Cfg::NTHREADS>(p.offsets, p.E, cdiv(p.F, Cfg::BN), blockIdx.x, sm.start, tl)) return;
    const int n_base = tl.nt * Cfg::BN;
    const int ncol = min(Cfg::BN, p.F - n_base);
    BufKLoader<Cfg, Cfg::BM> sa;
    sa.rs[0][0] = sa.rs[0][1] = make_rsrc(p.dout, (uint32_t)p.T * p.d * sizeof(T));
    sa.K[0] = p.d; sa.nt0 = cdiv(p.d, Cfg::BK);
#pragma unroll
    for (int i = 0; i < sa.PER; ++i) {
        const int m = sa.row_of(i);
        sa.off[i] = m < tl.rows ? (uint32_t)token_of(p.sorted_slot, tl.row0 + m, p.k) * p.d * sizeof(T) : kInvalid;
    }
    // W_d[e] is [d, F]: element (k = model dim, n = f)
    BufNLoader<Cfg, Cfg::BN> sb;
    sb.rs[0] = sb.rs[1] = make_rsrc(static_cast<const T *>(p.wd) + (size_t)tl.e * p.d * p.F + n_base,
                                    (uint32_t)((size_t)p.d * p.F - n_base) * sizeof(T));
    sb.K[0] = p.d; sb.ld[0] = p.F; sb.ncol = ncol; sb.nt0 = sa.nt0;
    KLoader<Cfg, Cfg::BM, true> la;
    la.K1 = p.r; la.nk0 = 0; la.scale1 = p.s;
    la.b1[0] = la.b1[1] = p.pd;
#pragma unroll
    for (int i = 0; i < la.PER; ++i) {
        const int m = la.row_of(i);
        if (la.active(i) && m < tl.rows) la.set1(i, (uint32_t)(tl.row0 + m) * p.r, 0);
    }
    NLoader<Cfg, Cfg::BN> lb;
    lb.nk0 = 1 << 30;
    lb.s0 = NSeg{static_cast<const T *>(p.ad) + (size_t)tl.e * p.r * p.F + n_base, nullptr, p.r, p.r, p.F,
                 0, ncol, 0, 0};
    lb.s1 = lb.s0;
    f32x16_t acc[Cfg::TM][Cfg::TN];
    gemm_pipeline<Cfg>(sa, sb, sa.nt0, la, lb, cdiv(p.r, Cfg::BK), sm.a, sm.b, acc);
    const T *G = static_cast<const T *>(p.G), *U = static_cast<const T *>(p.U);
    T *dGU = static_cast<T *>(p.dGU);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
#pragma unroll
    for (int mi = 0; mi < Cfg::TM; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = wm * Cfg::WTM + mi * 32 + acc_row(i, lane);
            if (m >= tl.rows) continue;
            const int pr = tl.row0 + m;
            const float w = p.topk_w[p.sorted_slot[pr]];
#pragma unroll
            for (int ni = 0; ni < Cfg::TN; ++ni) {
                const int f = n_base + wn * Cfg::WTN + ni * 32 + acc_col(lane);
                if (f < p.F) {
                    const float dh = w * acc[mi][ni][i];
                    const size_t o = (size_t)pr * p.F + f;
                    const float g = Elem<T>::to_f32(G[o]), u = Elem<T>::to_f32(U[o]);
                    const float sg = 1.0f / (1.0f + expf(-g));
                    dGU[(size_t)pr * 2 * p.F + f] = Elem<T>::from_f32(dh * u * sg * (1.0f + g * (1.0f - sg)));
                    dGU[(size_t)pr * 2 * p.F + p.F + f] = Elem<T>::from_f32(dh * g * sg);
                }
            }
        }
    }
}

// ===========================================================================
// Gate/up backward: dXp = [dG | dU] [W_g ; W_u] + s [Pg | Pu] [A_g ; A_u].
// ===========================================================================
struct GateUpBwdP {
    const void *dGU, *wg, *wu, *ag, *au;
    const float *pgu;
    const int32_t *offsets;
    void *dXp;
    int S, E, d, F, r;
    float s;
    const int32_t *tiles;  // bf16 path: row-tile table (build_row_tiles)
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS) MOE_ONE_WAVE_PER_SIMD void k_gateup_bwd(GateUpBwdP p) {
    using T = typename Cfg::T;
    __shared__ Smem<Cfg> sm;
    Tile tl;
    if (!schedule_tile<Cfg::BM, Cfg::NTHREADS>(p.offsets, p.E, cdiv(p.d, Cfg::BN), blockIdx.x, sm.start, tl)) return;
    const int n_base = tl.nt * Cfg::BN;
    const int ncol = min(Cfg::BN, p.d - n_base);
    const int ntf = cdiv(p.F, Cfg::BK);
    // two K segments: dG (columns 0..F of dGU) against W_g, then dU (F..2F) against W_u
    BufKLoader<Cfg, Cfg::BM> sa;
    sa.rs[0][0] = sa.rs[0][1] = sa.rs[1][0] = sa.rs[1][1] =
        make_rsrc(p.dGU, (uint32_t)p.S * 2 * p.F * sizeof(T));
    sa.K[0] = sa.K[1] = p.F; sa.col[0] = 0; sa.col[1] = p.F; sa.nt0 = ntf;
#pragma unroll
    for (int i = 0; i < sa.PER; ++i) {
        const int m = sa.row_of(i);
        sa.off[i] = m < tl.rows ? (uint32_t)(tl.row0 + m) * 2 * p.F * sizeof(T) : kInvalid;
    }
    // W_g[e], W_u[e] are [F, d]: element (k = f, n = model dim)
    BufNLoader<Cfg, Cfg::BN> sb;
    const size_t wofs = (size_t)tl.e * p.F * p.d + n_base;
    const uint32_t wbytes = (uint32_t)((size_t)p.F * p.d - n_base) * sizeof(T);
    sb.rs[0] = make_rsrc(static_cast<const T *>(p.wg) + wofs, wbytes);
    sb.rs[1] = make_rsrc(static_cast<const T *>(p.wu) + wofs, wbytes);
    sb.K[0] = sb.K[1] = p.F; sb.ld[0] = sb.ld[1] = p.d; sb.ncol = ncol; sb.nt0 = ntf;
    KLoader<Cfg, Cfg::BM, true> la;
    la.K1 = 2 * p.r; la.nk0 = 0; la.scale1 = p.s;
    la.b1[0] = la.b1[1] = p.pgu;
#pragma unroll
    for (int i = 0; i < la.PER; ++i) {
        const int m = la.row_of(i);
        if (la.active(i) && m < tl.rows) la.set1(i, (uint32_t)(tl.row0 + m) * 2 * p.r, 0);
    }
    NLoader<Cfg, Cfg::BN> lb;
    lb.nk0 = 1 << 30;
    const size_t aofs = (size_t)tl.e * p.r * p.d + n_base;
    lb.s0 = NSeg{static_cast<const T *>(p.ag) + aofs, static_cast<const T *>(p.au) + aofs, p.r, 2 * p.r, p.d,
                 0, ncol, 0, ncol};
    lb.s1 = lb.s0;
    f32x16_t acc[Cfg::TM][Cfg::TN];
    gemm_pipeline<Cfg>(sa, sb, 2 * ntf, la, lb, cdiv(2 * p.r, Cfg::BK), sm.a, sm.b, acc);
    T *dXp = static_cast<T *>(p.dXp);
    for_each_acc<Cfg>(acc, [&](int m, int n, int, int, int, float v) {
        if (m < tl.rows && n_base + n < p.d) dXp[(size_t)(tl.row0 + m) * p.d + n_base + n] = Elem<T>::from_f32(v);
    });
}

// ===========================================================================
// bf16 versions of the four grouped GEMMs on the direct-to-LDS ring engine
// (gemm_lds.hpp). Same math and epilogues as the kernels above.
// ===========================================================================
// All four run 64-deep steps, so every K-contiguous row segment a load
// touches is a whole 128-byte line (about twice the L2-to-LDS rate of 64-byte
// segments), through five 32 KB operand slots (B tiles two steps ahead, A
// tiles one). The backward GEMMs read their N-contiguous weights with
// transposing LDS reads.
// Waves: 2 x 4 per block (each wave 128 x 64 of the tile, two waves per SIMD,
// so one wave's waits are covered by the other's MFMAs) for down, down
// backward and gate/up backward; gate/up forward keeps 2 x 2 waves of
// 128 x 128 (fewer LDS fragment reads per MFMA; measured faster there).
using LdsGU = lds::Cfg<256, 256, 5, false, 64>;
using LdsGUh = lds::Cfg<128, 256, 5, false, 64>;  // 128-row tail tiles
using LdsNT = lds::Cfg<256, 256, 5, false, 64, 2, 4>;
using LdsNTh = lds::Cfg<128, 256, 5, false, 64, 2, 4>;
using LdsNN64 = lds::Cfg<256, 256, 5, true, 64, 2, 4>;
using LdsNN64h = lds::Cfg<128, 256, 5, true, 64, 2, 4>;

template <class C> union LdsSmem {  // the tile scheduler's table is dead once the ring starts
    __align__(16) char ring[C::SMEM_BYTES];
    int start[kMaxE + 1];
};


// NF4 frozen weights (4-bit NormalFloat codes and per-64 fp32 scales) for the
// four grouped GEMMs: the B operand is dequantised while it is staged to LDS
// (lds::Q4B); c1 / s1 are the second weight of the gate/up pair.
struct Q4P {
    const uint8_t *c0, *c1;
    const float *s0, *s1;
    lds::Nf4Lv lv;
};

// codes and scales descriptors of expert e's [rows, cols] NF4 weight. The
// sizes go through readfirstlane: the compiler may otherwise reuse a copy of
// cols / 2 that a lane-dependent branch left in a vector register, and a
// descriptor in vector registers turns every load into a loop over lanes.
__device__ __forceinline__ rsrc_t q4_codes(const uint8_t *c, int e, int rows, int cols) {
    const uint32_t n = __builtin_amdgcn_readfirstlane((uint32_t)rows * (uint32_t)(cols / 2));
    return make_rsrc(c + (size_t)e * n, n);
}
__device__ __forceinline__ rsrc_t q4_scales(const float *s, int e, int rows, int cols) {
    const uint32_t n = __builtin_amdgcn_readfirstlane((uint32_t)rows * (uint32_t)(cols / 64));
    return make_rsrc(s + (size_t)e * n, n * 4);
}

// --- gate/up -----------------------------------------------------------------
// B rows interleave gate / up in 32-row blocks: tile row n -> FFN index f and
// which weight (up = second) it comes from
template <class C> __device__ __forceinline__ int gateup_f(int f_base, int n, bool &up) {
    const int wn = n / C::WTN, ni = (n % C::WTN) / 32;
    up = ni & 1;
    return f_base + wn * (C::WTN / 2) + (ni / 2) * 32 + (n % 32);
}

template <class C> __device__ __forceinline__ void gateup_a(const GateUpP &p, const Tile &tl, lds::Operands<C> &op) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t aro[C::A_INSTR];
#pragma unroll
    for (int j = 0; j < C::A_INSTR; ++j) {
        const int m = lds_row<C>(wave, lane, j, C::A_INSTR);
        aro[j] = m < tl.rows ? (uint32_t)token_of(p.sorted_slot, tl.row0 + m, p.k) * p.d * 2 : kInvalid;
    }
    op.a.init_rows(wave, lane, aro);
    op.ra[0] = op.ra[1] = make_rsrc(p.x, (uint32_t)p.T * p.d * 2);
    op.K[0] = op.K[1] = p.d;
    op.nt0 = op.nt = cdiv(p.d, C::BK);
}

template <class C> using GateUpLora = lds::LoraTile<lds::LoraA<typename C::LoraCfg>, lds::LoraBK<typename C::LoraCfg>>;

// LoRA tile: [s Zg | s Zu] rows against [B_g | 0] (gate rows) and [0 | B_u] (up rows)
template <class C> __device__ __forceinline__ GateUpLora<C> gateup_lora(const GateUpP &p, const Tile &tl) {
    const int f_base = tl.nt * (C::BN / 2);
    const bf16_t *bg = static_cast<const bf16_t *>(p.bg) + (size_t)tl.e * p.F * p.r;
    const bf16_t *bu = static_cast<const bf16_t *>(p.bu) + (size_t)tl.e * p.F * p.r;
    GateUpLora<C> lora;
    lora.pa = {p.zgu, 2 * p.r, tl.row0, tl.rows, p.s};
    lora.pb.r = p.r;
    lora.pb.safe = bg;
#pragma unroll
    for (int i = 0; i < lds::LoraBK<typename C::LoraCfg>::PER; ++i) {
        bool up;
        const int f = gateup_f<C>(f_base, ((int)threadIdx.x + C::NTHREADS * i) >> 2, up);
        lora.pb.rowp[i] = f < p.F ? (up ? bu : bg) + (size_t)f * p.r : nullptr;
        lora.pb.klo[i] = up ? p.r : 0;
    }
    return lora;
}

// SwiGLU epilogue: wave columns are pairs [gate 32 | up 32] for
// f = f_base + wn * WTN / 2 + (0 .. WTN / 2 - 1); writes G, U (training) and H
template <class C>
__device__ __forceinline__ void gateup_epilogue(const GateUpP &p, const Tile &tl, const f32x16_t (&acc)[C::TM][C::TN],
                                                char *ring) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int f_base = tl.nt * (C::BN / 2);
    bf16_t *G = static_cast<bf16_t *>(p.G), *U = static_cast<bf16_t *>(p.U), *H = static_cast<bf16_t *>(p.H);
    const int wn = wave % C::WN, wm = wave / C::WN;
    float *buf = reinterpret_cast<float *>(ring) + wave * 32 * C::WTN;
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi) {
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                buf[acc_row(i, lane) * C::WTN + ni * 32 + acc_col(lane)] = acc[mi][ni][i];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // WTN / 2 f per row = LPR lanes x 8 f; RPP rows per pass
        constexpr int LPR = C::WTN / 16, RPP = 64 / LPR;
#pragma unroll
        for (int pass = 0; pass < 32 / RPP; ++pass) {
            const int r = pass * RPP + lane / LPR, q = lane % LPR;  // q: 8-f group
            const int gc = (q / 4) * 64 + (q % 4) * 8;             // gate column in the wave tile
            const float4 g0 = *reinterpret_cast<const float4 *>(buf + r * C::WTN + gc);
            const float4 g1 = *reinterpret_cast<const float4 *>(buf + r * C::WTN + gc + 4);
            const float4 u0 = *reinterpret_cast<const float4 *>(buf + r * C::WTN + gc + 32);
            const float4 u1 = *reinterpret_cast<const float4 *>(buf + r * C::WTN + gc + 36);
            const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            const int m = wm * C::WTM + mi * 32 + r;
            const int f = f_base + wn * (C::WTN / 2) + (q / 4) * 32 + (q % 4) * 8;
            if (m < tl.rows && f < p.F) {
                const chunk_t cg = Elem<bf16_t>::pack(g), cu = Elem<bf16_t>::pack(u);
                const size_t o = (size_t)(tl.row0 + m) * p.F + f;
                if (G) st_stream(G + o, cg);
                if (U) st_stream(U + o, cu);
                st_stream(H + o, swiglu_chunk<bf16_t>(cg, cu));  // from G and U as stored
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

template <class C>
__device__ __forceinline__ void gateup_tile(const GateUpP &p, const Tile &tl, char *ring) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int f_base = tl.nt * (C::BN / 2);
    lds::Operands<C> op;
    gateup_a<C>(p, tl, op);
    uint32_t bro[C::B_INSTR];
    // one load covers 16 rows of one 32-row gate or up block
#pragma unroll
    for (int j = 0; j < C::B_INSTR; ++j) {
        bool up;
        const int f = gateup_f<C>(f_base, lds_row<C>(wave, lane, j, C::B_INSTR), up);
        bro[j] = f < p.F ? (uint32_t)f * p.d * 2 : kInvalid;
        const int n0 = (wave * C::B_INSTR + j) * C::RPI;  // first row of the load (same block for every lane)
        op.bsel_mask |= (uint32_t)(((n0 % C::WTN) / 32) & 1) << j;
    }
    op.bk.init_rows(wave, lane, bro);
    const size_t wofs = (size_t)tl.e * p.F * p.d;
    op.rb[0][0] = op.rb[1][0] = make_rsrc(static_cast<const bf16_t *>(p.wg) + wofs, (uint32_t)p.F * p.d * 2);
    op.rb[0][1] = op.rb[1][1] = make_rsrc(static_cast<const bf16_t *>(p.wu) + wofs, (uint32_t)p.F * p.d * 2);
    f32x16_t acc[C::TM][C::TN];
    lds::run<C>(op, cdiv(2 * p.r, C::LoraCfg::BK), gateup_lora<C>(p, tl), ring, acc);
    gateup_epilogue<C>(p, tl, acc, ring);
}

// NF4 weights: each thread dequantises one 32-element group of a B row
template <class C>
__device__ __forceinline__ void gateup_tile_q4(const GateUpP &p, const Q4P &q, const Tile &tl, char *ring) {
    lds::Operands<C> op;
    gateup_a<C>(p, tl, op);
    lds::Q4B<C> qb;
    bool up;
    const int f = gateup_f<C>(tl.nt * (C::BN / 2), qb.row(), up);
    // a wave's 32 rows are one gate or one up block: its weight is uniform
    const bool wup = __builtin_amdgcn_readfirstlane((int)up) != 0;
    qb.coff = f < p.F ? (uint32_t)f * (p.d / 2) + ((int)threadIdx.x & 1) * 16 : kInvalid;
    qb.soff = f < p.F ? (uint32_t)f * (p.d / 64) * 4 : 0;
    qb.rc[0] = q4_codes(wup ? q.c1 : q.c0, tl.e, p.F, p.d);
    qb.rs[0] = q4_scales(wup ? q.s1 : q.s0, tl.e, p.F, p.d);
    qb.nt0 = qb.nt = op.nt;
    f32x16_t acc[C::TM][C::TN];
    lds::run_q4<C>(op, qb, q.lv, cdiv(2 * p.r, C::LoraCfg::BK), gateup_lora<C>(p, tl), ring, acc);
    gateup_epilogue<C>(p, tl, acc, ring);
}

// full 256-row tiles run C, an expert's last tile with at most CH::BM rows runs CH
template <class C, class CH>
__global__ MOE_LDS_BLOCK(C) void k_gateup_lds(GateUpP p) {
    static_assert(C::NTHREADS == CH::NTHREADS, "one block size for both tile shapes");
    // an expert's last tile of at most 64 rows runs a 64-row shape: half the
    // padded MFMA work of the 128-row one (the 8-wave kernels cannot split
    // a 64-row tile's loads evenly, so only this 4-wave kernel has it)
    using CQ = lds::Cfg<64, 256, 5, false, 64>;
    __shared__ LdsSmem<C> sm;
    static_assert(C::BM == kRowTile, "tiles come from the row-tile table");
    Tile tl;
    if (!table_tile(p.tiles, cdiv(p.F, C::BN / 2), blockIdx.x, tl)) return;
    if (tl.rows > CH::BM) gateup_tile<C>(p, tl, sm.ring);
    else if (tl.rows > CQ::BM) gateup_tile<CH>(p, tl, sm.ring);
    else gateup_tile<CQ>(p, tl, sm.ring);
}

template <class C, class CH>
__global__ MOE_LDS_BLOCK(C) void k_gateup_q4(GateUpP p, Q4P q) {
    static_assert(C::NTHREADS == CH::NTHREADS, "one block size for both tile shapes");
    __shared__ LdsSmem<C> sm;
    static_assert(C::BM == kRowTile, "tiles come from the row-tile table");
    Tile tl;
    if (!table_tile(p.tiles, cdiv(p.F, C::BN / 2), blockIdx.x, tl)) return;
    if (tl.rows > CH::BM) gateup_tile_q4<C>(p, q, tl, sm.ring);
    else gateup_tile_q4<CH>(p, q, tl, sm.ring);
}

// --- down ----------------------------------------------------------------------
template <class C> __device__ __forceinline__ void down_a(const DownP &p, const Tile &tl, lds::Operands<C> &op) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t aro[C::A_INSTR];
#pragma unroll
    for (int j = 0; j < C::A_INSTR; ++j) {
        const int m = lds_row<C>(wave, lane, j, C::A_INSTR);
        aro[j] = m < tl.rows ? (uint32_t)(tl.row0 + m) * p.F * 2 : kInvalid;
    }
    op.a.init_rows(wave, lane, aro);
    op.ra[0] = op.ra[1] = make_rsrc(p.H, (uint32_t)p.S * p.F * 2);
    op.K[0] = op.K[1] = p.F;
    op.nt0 = op.nt = cdiv(p.F, C::BK);
}

template <class C> using KLora = lds::LoraTile<lds::LoraA<typename C::LoraCfg>, lds::LoraBK<typename C::LoraCfg>>;

template <class C> __device__ __forceinline__ KLora<C> down_lora(const DownP &p, const Tile &tl) {
    const int n_base = tl.nt * C::BN;
    const bf16_t *bd = static_cast<const bf16_t *>(p.bd) + (size_t)tl.e * p.d * p.r;
    KLora<C> lora;
    lora.pa = {p.zd, p.r, tl.row0, tl.rows, p.s};
    lora.pb.r = p.r;
    lora.pb.safe = bd;
#pragma unroll
    for (int i = 0; i < lds::LoraBK<typename C::LoraCfg>::PER; ++i) {
        const int n = n_base + (((int)threadIdx.x + C::NTHREADS * i) >> 2);
        lora.pb.rowp[i] = n < p.d ? bd + (size_t)n * p.r : nullptr;
        lora.pb.klo[i] = 0;
    }
    return lora;
}

template <class C>
__device__ __forceinline__ void down_epilogue(const DownP &p, const Tile &tl, const f32x16_t (&acc)[C::TM][C::TN],
                                              char *ring) {
    const int n_base = tl.nt * C::BN;
    bf16_t *Y = static_cast<bf16_t *>(p.Y);
    lds::epilogue_rows<C>(acc, ring, [&](int m, int n, const float *v) {
        if (m < tl.rows && n_base + n < p.d)
            st_stream(Y + (size_t)(tl.row0 + m) * p.d + n_base + n, Elem<bf16_t>::pack(v));
    });
}

template <class C>
__device__ __forceinline__ void down_tile(const DownP &p, const Tile &tl, char *ring) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_base = tl.nt * C::BN;
    lds::Operands<C> op;
    down_a<C>(p, tl, op);
    uint32_t bro[C::B_INSTR];
#pragma unroll
    for (int j = 0; j < C::B_INSTR; ++j) {
        const int n = n_base + lds_row<C>(wave, lane, j, C::B_INSTR);
        bro[j] = n < p.d ? (uint32_t)n * p.F * 2 : kInvalid;
    }
    op.bk.init_rows(wave, lane, bro);
    op.rb[0][0] = op.rb[0][1] = op.rb[1][0] = op.rb[1][1] =
        make_rsrc(static_cast<const bf16_t *>(p.wd) + (size_t)tl.e * p.d * p.F, (uint32_t)p.d * p.F * 2);
    f32x16_t acc[C::TM][C::TN];
    lds::run<C>(op, cdiv(p.r, C::LoraCfg::BK), down_lora<C>(p, tl), ring, acc);
    down_epilogue<C>(p, tl, acc, ring);
}

template <class C>
__device__ __forceinline__ void down_tile_q4(const DownP &p, const Q4P &q, const Tile &tl, char *ring) {
    lds::Operands<C> op;
    down_a<C>(p, tl, op);
    lds::Q4B<C> qb;
    const int n = tl.nt * C::BN + qb.row();
    qb.coff = n < p.d ? (uint32_t)n * (p.F / 2) + ((int)threadIdx.x & 1) * 16 : kInvalid;
    qb.soff = n < p.d ? (uint32_t)n * (p.F / 64) * 4 : 0;
    qb.rc[0] = q4_codes(q.c0, tl.e, p.d, p.F);
    qb.rs[0] = q4_scales(q.s0, tl.e, p.d, p.F);
    qb.nt0 = qb.nt = op.nt;
    f32x16_t acc[C::TM][C::TN];
    lds::run_q4<C>(op, qb, q.lv, cdiv(p.r, C::LoraCfg::BK), down_lora<C>(p, tl), ring, acc);
    down_epilogue<C>(p, tl, acc, ring);
}

// full 256-row tiles run C, an expert's last tile with at most CH::BM rows runs CH
template <class C, class CH>
__global__ MOE_LDS_BLOCK(C) void k_down_lds(DownP p) {
    static_assert(C::NTHREADS == CH::NTHREADS, "one block size for both tile shapes");
    __shared__ LdsSmem<C> sm;
    static_assert(C::BM == kRowTile, "tiles come from the row-tile table");
    Tile tl;
    if (!table_tile(p.tiles, cdiv(p.d, C::BN), blockIdx.x, tl)) return;
    if (tl.rows > CH::BM) down_tile<C>(p, tl, sm.ring);
    else down_tile<CH>(p, tl, sm.ring);
}

template <class C, class CH>
__global__ MOE_LDS_BLOCK(C) void k_down_q4(DownP p, Q4P q) {
    static_assert(C::NTHREADS == CH::NTHREADS, "one block size for both tile shapes");
    __shared__ LdsSmem<C> sm;
    static_assert(C::BM == kRowTile, "tiles come from the row-tile table");
    Tile tl;
    if (!table_tile(p.tiles, cdiv(p.d, C::BN), blockIdx.x, tl)) return;
    if (tl.rows > CH::BM) down_tile_q4<C>(p, q, tl, sm.ring);
    else down_tile_q4<CH>(p, q, tl, sm.ring);
}

// --- down backward ---------------------------------------------------------------
template <class C> __device__ __forceinline__ void down_bwd_a(const DownBwdP &p, const Tile &tl, lds::Operands<C> &op) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t aro[C::A_INSTR];
#pragma unroll
    for (int j = 0; j < C::A_INSTR; ++j) {
        const int m = lds_row<C>(wave, lane, j, C::A_INSTR);
        aro[j] = m < tl.rows ? (uint32_t)token_of(p.sorted_slot, tl.row0 + m, p.k) * p.d * 2 : kInvalid;
    }
    op.a.init_rows(wave, lane, aro);
    op.ra[0] = op.ra[1] = make_rsrc(p.dout, (uint32_t)p.T * p.d * 2);
    op.K[0] = op.K[1] = p.d;
    op.nt0 = op.nt = cdiv(p.d, C::BK);
}

template <class C> using NLora = lds::LoraTile<lds::LoraA<typename C::LoraCfg>, lds::LoraBN<typename C::LoraCfg>>;

template <class C> __device__ __forceinline__ NLora<C> down_bwd_lora(const DownBwdP &p, const Tile &tl) {
    const int n_base = tl.nt * C::BN;
    const int ncol = min(C::BN, p.F - n_base);
    const bf16_t *ad = static_cast<const bf16_t *>(p.ad) + (size_t)tl.e * p.r * p.F + n_base;
    NLora<C> lora;
    lora.pa = {p.pd, p.r, tl.row0, tl.rows, p.s};
    lora.pb = {ad, ad, p.r, p.r, p.F, ncol};
    return lora;
}

// SwiGLU backward epilogue. Per 32-row slab of each wave: the fp32 tile goes
// through LDS to 16-byte row chunks; G, U and the row weight of the next
// slab are loaded while this slab is computed and stored.
template <class C>
__device__ __forceinline__ void down_bwd_epilogue(const DownBwdP &p, const Tile &tl,
                                                  const f32x16_t (&acc)[C::TM][C::TN], char *ring) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_base = tl.nt * C::BN;
    const bf16_t *G = static_cast<const bf16_t *>(p.G), *U = static_cast<const bf16_t *>(p.U);
    bf16_t *dGU = static_cast<bf16_t *>(p.dGU);
    constexpr int LPR = C::WTN / 8, RPP = 64 / LPR, NPASS = 32 / RPP;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int c8 = (lane % LPR) * 8, f = n_base + wn * C::WTN + c8;
    // Projection of dG | dU onto B_g | B_u (when p.ppart is set). Past the
    // per-wave fp32 slabs the ring holds, per row group wm, the current 32
    // rows of bf16 dG (k = f - n_base) and dU (k = 256 + f - n_base), and the
    // tile's slices of B_g and B_u transposed: sbt[n][f - n_base], rows n < r
    // from B_g, r <= n < 2r from B_u. Both swap 16-byte chunks within groups
    // of 16 (256 bytes, all 64 banks): staged row r by ((r & 1) << 3) |
    // ((r >> 1) & 7), so the two rows a write instruction's 16-lane groups
    // cover fall in different bank halves and any 16 rows a fragment read
    // covers fall on distinct chunks; sbt row n by n & 15. Each slab gives r / 4 jobs of 16 rows x 16 columns (a column
    // block uses the dG half of k if it is below r, else the dU half), spread
    // over the WN waves of the row group; each job is 8 MFMAs over 256 k.
    constexpr int SLABS = C::NWAVES * 32 * C::WTN * 4;
    static_assert(C::BN == 256 && C::WN * C::WTN == 256, "one 256-column strip per tile");
    static_assert(SLABS + C::WM * 32 * 1024 + 64 * 512 <= C::SMEM_BYTES, "staging fits the ring");
    const bool fuse = p.ppart != nullptr;
    char *stage = ring + SLABS + wm * 32 * 1024;
    char *sbt = ring + SLABS + C::WM * 32 * 1024;
    const int r2 = 2 * p.r;
    struct Pre {
        chunk_t g[NPASS], u[NPASS];
        float w[NPASS];
    };
    auto prefetch = [&](int mi, Pre &q) {
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            const int m = wm * C::WTM + mi * 32 + pass * RPP + lane / LPR;
            const bool ok = m < tl.rows && f < p.F;
            const size_t o = (size_t)(tl.row0 + (ok ? m : 0)) * p.F + (ok ? f : 0);
            q.g[pass] = ld_stream(G + o);
            q.u[pass] = ld_stream(U + o);
            q.w[pass] = p.w_row[tl.row0 + (ok ? m : 0)];
        }
    };
    float *buf = reinterpret_cast<float *>(ring) + wave * 32 * C::WTN;
    __syncthreads();  // every wave is done with the ring
    if (fuse) {
        // B_x[e] is [F, r]: thread w takes two rows f, f + 1 of eight columns
        // and writes them as eight column pairs of sbt
        const int ng = r2 / 8;
        for (int w = threadIdx.x; w < ng * 128; w += C::NTHREADS) {
            const int fp = w % 128, g8 = w / 128, n0 = g8 * 8;
            const bool up = n0 >= p.r;
            const bf16_t *src = static_cast<const bf16_t *>(up ? p.bu : p.bg) + (size_t)tl.e * p.F * p.r +
                                (up ? n0 - p.r : n0);
            const int f0 = n_base + 2 * fp;
            const chunk_t zero = {0u, 0u, 0u, 0u};
            const chunk_t v0 = f0 < p.F ? *reinterpret_cast<const chunk_t *>(src + (size_t)f0 * p.r) : zero;
            const chunk_t v1 = f0 + 1 < p.F ? *reinterpret_cast<const chunk_t *>(src + (size_t)(f0 + 1) * p.r) : zero;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t lo = (v0[i >> 1] >> ((i & 1) * 16)) & 0xffffu;
                const uint32_t hi = (v1[i >> 1] >> ((i & 1) * 16)) & 0xffffu;
                const int n = n0 + i;
                *reinterpret_cast<uint32_t *>(sbt + n * 512 + (((fp >> 2) ^ (n & 15)) * 16) + (fp & 3) * 4) =
                    lo | (hi << 16);
            }
        }
    }
    Pre q[2];
    prefetch(0, q[0]);
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi) {
        if (mi + 1 < C::TM) prefetch(mi + 1, q[(mi + 1) & 1]);
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) buf[acc_row(i, lane) * C::WTN + ni * 32 + acc_col(lane)] = acc[mi][ni][i];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            const int r = pass * RPP + lane / LPR;
            const int m = wm * C::WTM + mi * 32 + r;
            const float4 a = *reinterpret_cast<const float4 *>(buf + r * C::WTN + c8);
            const float4 b4 = *reinterpret_cast<const float4 *>(buf + r * C::WTN + c8 + 4);
            const float v[8] = {a.x, a.y, a.z, a.w, b4.x, b4.y, b4.z, b4.w};
            chunk_t pg = {0u, 0u, 0u, 0u}, pu = {0u, 0u, 0u, 0u};
            if (m < tl.rows && f < p.F) {
                const Pre &cq = q[mi & 1];
                float g[8], u[8], dg[8], du[8];
                unpack<bf16_t>(cq.g[pass], g);
                unpack<bf16_t>(cq.u[pass], u);
                const float w = cq.w[pass];
#pragma unroll
                for (int h = 0; h < 8; ++h) {
                    const float dh = w * v[h];
                    const float sg = sigmoid_fast(g[h]);
                    dg[h] = dh * u[h] * sg * (1.0f + g[h] * (1.0f - sg));
                    du[h] = dh * g[h] * sg;
                }
                pg = Elem<bf16_t>::pack(dg);
                pu = Elem<bf16_t>::pack(du);
                const size_t pr = (size_t)(tl.row0 + m);
                st_stream(dGU + pr * 2 * p.F + f, pg);
                st_stream(dGU + pr * 2 * p.F + p.F + f, pu);
            }
            if (fuse) {
                const int cg = (wn * C::WTN + c8) / 8, cu = 32 + cg, sw = ((r & 1) << 3) | ((r >> 1) & 7);
                *reinterpret_cast<chunk_t *>(stage + r * 1024 + ((cg ^ sw) * 16)) = pg;
                *reinterpret_cast<chunk_t *>(stage + r * 1024 + ((cu ^ sw) * 16)) = pu;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next slab overwrites
        if (fuse) {
            __syncthreads();  // both row groups' slabs (and sbt) are staged
            const int jobs = p.r / 4;
            for (int job = wn; job < jobs; job += C::WN) {
                const int rh = job & 1, nb = job >> 1;
                const int half = nb * 16 >= p.r ? 1 : 0;
                const int row = rh * 16 + (lane & 15), n = nb * 16 + (lane & 15);
                f32x4_t pacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kq = 0; kq < 8; ++kq) {
                    const int ca = half * 32 + kq * 4 + (lane >> 4), sw = ((row & 1) << 3) | ((row >> 1) & 7);
                    const int cb = kq * 4 + (lane >> 4);
                    const chunk_t av = *reinterpret_cast<const chunk_t *>(stage + row * 1024 + ((ca ^ sw) * 16));
                    const chunk_t bv = *reinterpret_cast<const chunk_t *>(sbt + n * 512 + ((cb ^ (n & 15)) * 16));
                    pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                   __builtin_bit_cast(bf16x8_t, bv), pacc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = wm * C::WTM + mi * 32 + rh * 16 + (lane >> 4) * 4 + i;
                    if (m < tl.rows)
                        p.ppart[((size_t)tl.nt * (p.T * p.k) + tl.row0 + m) * r2 + n] = pacc[i];
                }
            }
            __syncthreads();  // every job has read the staged slab
        }
    }
}

template <class C>
__device__ __forceinline__ void down_bwd_tile(const DownBwdP &p, const Tile &tl, char *ring) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_base = tl.nt * C::BN;
    const int ncol = min(C::BN, p.F - n_base);
    lds::Operands<C> op;
    down_bwd_a<C>(p, tl, op);
    // W_d[e] is [d, F]: k = model dim, n = f
    op.bn.init(wave, lane, ncol);
    op.rb[0][0] = op.rb[1][0] = make_rsrc(static_cast<const bf16_t *>(p.wd) + (size_t)tl.e * p.d * p.F + n_base,
                                          (uint32_t)((size_t)p.d * p.F - n_base) * 2);
    op.ldb[0] = op.ldb[1] = (uint32_t)p.F * 2;
    f32x16_t acc[C::TM][C::TN];
    lds::run<C>(op, cdiv(p.r, C::LoraCfg::BK), down_bwd_lora<C>(p, tl), ring, acc);
    down_bwd_epilogue<C>(p, tl, acc, ring);
}

template <class C>
__device__ __forceinline__ void down_bwd_tile_q4(const DownBwdP &p, const Q4P &q, const Tile &tl, char *ring) {
    lds::Operands<C> op;
    down_bwd_a<C>(p, tl, op);
    lds::Q4B<C> qb;
    // W_d[e] is [d, F]: the tile's k-rows are weight rows, its columns f
    const int n = tl.nt * C::BN + ((int)threadIdx.x & 7) * 32;
    qb.coff = n < p.F ? (uint32_t)n / 2 : kInvalid;
    qb.soff = (uint32_t)(n / 64) * 4;
    qb.ldc[0] = qb.ldc[1] = (uint32_t)p.F / 2;
    qb.ldsc[0] = qb.ldsc[1] = (uint32_t)(p.F / 64) * 4;
    qb.rc[0] = q4_codes(q.c0, tl.e, p.d, p.F);
    qb.rs[0] = q4_scales(q.s0, tl.e, p.d, p.F);
    qb.nt0 = qb.nt = op.nt;
    f32x16_t acc[C::TM][C::TN];
    lds::run_q4<C>(op, qb, q.lv, cdiv(p.r, C::LoraCfg::BK), down_bwd_lora<C>(p, tl), ring, acc);
    down_bwd_epilogue<C>(p, tl, acc, ring);
}

// full 256-row tiles run C, an expert's last tile with at most CH::BM rows runs CH
template <class C, class CH>
__global__ MOE_LDS_BLOCK(C) void k_down_bwd_lds(DownBwdP p) {
    static_assert(C::NTHREADS == CH::NTHREADS, "one block size for both tile shapes");
    __shared__ LdsSmem<C> sm;
    static_assert(C::BM == kRowTile, "tiles come from the row-tile table");
    Tile tl;
    if (!table_tile(p.tiles, cdiv(p.F, C::BN), blockIdx.x, tl)) return;
    if (tl.rows > CH::BM) down_bwd_tile<C>(p, tl, sm.ring);
    else down_bwd_tile<CH>(p, tl, sm.ring);
}

template <class C, class CH>
__global__ MOE_LDS_BLOCK(C) void k_down_bwd_q4(DownBwdP p, Q4P q) {
    static_assert(C::NTHREADS == CH::NTHREADS, "one block size for both tile shapes");
    __shared__ LdsSmem<C> sm;
    static_assert(C::BM == kRowTile, "tiles come from the row-tile table");
    Tile tl;
    if (!table_tile(p.tiles, cdiv(p.F, C::BN), blockIdx.x, tl)) return;
    if (tl.rows > CH::BM) down_bwd_tile_q4<C>(p, q, tl, sm.ring);
    else down_bwd_tile_q4<CH>(p, q, tl, sm.ring);
}

// --- gate/up backward --------------------------------------------------------------
template <class C>
__device__ __forceinline__ void gateup_bwd_a(const GateUpBwdP &p, const Tile &tl, lds::Operands<C> &op) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t aro[C::A_INSTR];
#pragma unroll
    for (int j = 0; j < C::A_INSTR; ++j) {
        const int m = lds_row<C>(wave, lane, j, C::A_INSTR);
        aro[j] = m < tl.rows ? (uint32_t)(tl.row0 + m) * 2 * p.F * 2 : kInvalid;
    }
    op.a.init_rows(wave, lane, aro);
    // segment 0: dG (columns 0..F) x W_g ; segment 1: dU (columns F..2F) x W_u
    op.ra[0] = op.ra[1] = make_rsrc(p.dGU, (uint32_t)p.S * 2 * p.F * 2);
    op.acol[0] = 0; op.acol[1] = (uint32_t)p.F * 2;
    op.K[0] = op.K[1] = p.F;
    op.nt0 = cdiv(p.F, C::BK);
    op.nt = 2 * op.nt0;
}

template <class C> __device__ __forceinline__ NLora<C> gateup_bwd_lora(const GateUpBwdP &p, const Tile &tl) {
    const int n_base = tl.nt * C::BN;
    const int ncol = min(C::BN, p.d - n_base);
    const size_t aofs = (size_t)tl.e * p.r * p.d + n_base;
    const bf16_t *ag = static_cast<const bf16_t *>(p.ag) + aofs, *au = static_cast<const bf16_t *>(p.au) + aofs;
    NLora<C> lora;
    lora.pa = {p.pgu, 2 * p.r, tl.row0, tl.rows, p.s};
    lora.pb = {ag, au, p.r, 2 * p.r, p.d, ncol};
    return lora;
}

template <class C>
__device__ __forceinline__ void gateup_bwd_epilogue(const GateUpBwdP &p, const Tile &tl,
                                                    const f32x16_t (&acc)[C::TM][C::TN], char *ring) {
    const int n_base = tl.nt * C::BN;
    bf16_t *dXp = static_cast<bf16_t *>(p.dXp);
    lds::epilogue_rows<C>(acc, ring, [&](int m, int n, const float *v) {
        if (m < tl.rows && n_base + n < p.d)
            st_stream(dXp + (size_t)(tl.row0 + m) * p.d + n_base + n, Elem<bf16_t>::pack(v));
    });
}

template <class C>
__device__ __forceinline__ void gateup_bwd_tile(const GateUpBwdP &p, const Tile &tl, char *ring) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_base = tl.nt * C::BN;
    const int ncol = min(C::BN, p.d - n_base);
    lds::Operands<C> op;
    gateup_bwd_a<C>(p, tl, op);
    op.bn.init(wave, lane, ncol);
    const size_t wofs = (size_t)tl.e * p.F * p.d + n_base;
    const uint32_t wbytes = (uint32_t)((size_t)p.F * p.d - n_base) * 2;
    op.rb[0][0] = make_rsrc(static_cast<const bf16_t *>(p.wg) + wofs, wbytes);
    op.rb[1][0] = make_rsrc(static_cast<const bf16_t *>(p.wu) + wofs, wbytes);
    op.ldb[0] = op.ldb[1] = (uint32_t)p.d * 2;
    f32x16_t acc[C::TM][C::TN];
    lds::run<C>(op, cdiv(2 * p.r, C::LoraCfg::BK), gateup_bwd_lora<C>(p, tl), ring, acc);
    gateup_bwd_epilogue<C>(p, tl, acc, ring);
}

template <class C>
__device__ __forceinline__ void gateup_bwd_tile_q4(const GateUpBwdP &p, const Q4P &q, const Tile &tl, char *ring) {
    lds::Operands<C> op;
    gateup_bwd_a<C>(p, tl, op);
    lds::Q4B<C, 2> qb;
    // W_g[e], W_u[e] are [F, d]: the tile's k-rows are weight rows (segment 0
    // gate, 1 up), its columns the model dim
    const int n = tl.nt * C::BN + ((int)threadIdx.x & 7) * 32;
    qb.coff = n < p.d ? (uint32_t)n / 2 : kInvalid;
    qb.soff = (uint32_t)(n / 64) * 4;
    qb.ldc[0] = qb.ldc[1] = (uint32_t)p.d / 2;
    qb.ldsc[0] = qb.ldsc[1] = (uint32_t)(p.d / 64) * 4;
    qb.rc[0] = q4_codes(q.c0, tl.e, p.F, p.d);
    qb.rc[1] = q4_codes(q.c1, tl.e, p.F, p.d);
    qb.rs[0] = q4_scales(q.s0, tl.e, p.F, p.d);
    qb.rs[1] = q4_scales(q.s1, tl.e, p.F, p.d);
    qb.nt0 = op.nt0;
    qb.nt = op.nt;
    f32x16_t acc[C::TM][C::TN];
    lds::run_q4<C>(op, qb, q.lv, cdiv(2 * p.r, C::LoraCfg::BK), gateup_bwd_lora<C>(p, tl), ring, acc);
    gateup_bwd_epilogue<C>(p, tl, acc, ring);
}

// full 256-row tiles run C, an expert's last tile with at most CH::BM rows runs CH
template <class C, class CH>
__global__ MOE_LDS_BLOCK(C) void k_gateup_bwd_lds(GateUpBwdP p) {
    static_assert(C::NTHREADS == CH::NTHREADS, "one block size for both tile shapes");
    __shared__ LdsSmem<C> sm;
    static_assert(C::BM == kRowTile, "tiles come from the row-tile table");
    Tile tl;
    if (!table_tile(p.tiles, cdiv(p.d, C::BN), blockIdx.x, tl)) return;
    if (tl.rows > CH::BM) gateup_bwd_tile<C>(p, tl, sm.ring);
    else gateup_bwd_tile<CH>(p, tl, sm.ring);
}

template <class C, class CH>
__global__ MOE_LDS_BLOCK(C) void k_gateup_bwd_q4(GateUpBwdP p, Q4P q) {
    static_assert(C::NTHREADS == CH::NTHREADS, "one block size for both tile shapes");
    __shared__ LdsSmem<C> sm;
    static_assert(C::BM == kRowTile, "tiles come from the row-tile table");
    Tile tl;
    if (!table_tile(p.tiles, cdiv(p.d, C::BN), blockIdx.x, tl)) return;
    if (tl.rows > CH::BM) gateup_bwd_tile_q4<C>(p, q, tl, sm.ring);
    else gateup_bwd_tile_q4<CH>(p, q, tl, sm.ring);
}

// ===========================================================================
// Skinny projections onto the LoRA rank (fp32 out [S, nr]):
//   PROJ_GU:   Zgu = Xp [A_g ; A_u]^T            (B rows K-contiguous)
//   PROJ_D:    Zd  = H A_d^T                     (B rows K-contiguous)
//   PROJ_DOUT: P'd = dout_gathered B_d           (B N-contiguous)
//   PROJ_DGU:  Pgu = [dG B_g | dU B_u]           (B N-contiguous, block-diagonal)
// ===========================================================================
enum ProjKind { PROJ_GU = 0, PROJ_D = 1, PROJ_DOUT = 2, PROJ_DGU = 3 };

struct ProjP {
    const void *a;            // x, H, dout or dGU
    const void *b0, *b1;      // A_g/A_u, A_d, B_d, B_g/B_u
    const int32_t *sorted_slot, *offsets;
    float *out;
    int E, k, d, F, r;
    // optional bf16 transposed copy [nr, ldT] of the output (ldT = S rounded
    // up to a multiple of 8), each row p scaled by wt[sorted_slot[p]] when wt
    // is set: the small operand of the LoRA-gradient kernel
    bf16_t *outT;
    const float *wt;
    int ldT, S;
    float *w_row_out;  // optional: wt[sorted_slot[p]] for every row p (written by the first column tile)
    int32_t *tiles_out;  // optional: block 0 builds the grouped GEMMs' row-tile table here
};

template <class Cfg, int KIND>
__global__ __launch_bounds__(Cfg::NTHREADS) void k_proj(ProjP p) {
    using T = typename Cfg::T;
    __shared__ Smem<Cfg> sm;
    constexpr bool GATHER = KIND == PROJ_GU || KIND == PROJ_DOUT;
    constexpr bool BN_CONTIG = KIND == PROJ_DOUT || KIND == PROJ_DGU;
    const int nr = (KIND == PROJ_GU || KIND == PROJ_DGU) ? 2 * p.r : p.r;
    const int K = (KIND == PROJ_GU || KIND == PROJ_DOUT) ? p.d : (KIND == PROJ_D ? p.F : 2 * p.F);
    Tile tl;
    if (p.tiles_out && blockIdx.x == 0) build_row_tiles<Cfg::NTHREADS>(p.offsets, p.E, sm.start, p.tiles_out);
    if (!schedule_tile<Cfg::BM, Cfg::NTHREADS>(p.offsets, p.E, cdiv(nr, Cfg::BN), blockIdx.x, sm.start, tl)) return;
    const int n_base = tl.nt * Cfg::BN;
    const int nk = cdiv(K, Cfg::BK);
    KLoader<Cfg, Cfg::BM, true> la;
    la.K0 = K; la.K1 = 0; la.nk0 = nk; la.scale1 = 0.0f;
    la.b0[0] = la.b0[1] = static_cast<const T *>(p.a);
    la.b1[0] = la.b1[1] = nullptr;
#pragma unroll
    for (int i = 0; i < la.PER; ++i) {
        const int m = la.row_of(i);
        if (la.active(i) && m < tl.rows) {
            const int pr = tl.row0 + m;
            const uint32_t row = GATHER ? (uint32_t)token_of(p.sorted_slot, pr, p.k) : (uint32_t)pr;
            la.set0(i, row * K, 0);
        }
    }
    f32x16_t acc[Cfg::TM][Cfg::TN];
    if constexpr (!BN_CONTIG) {
        KLoader<Cfg, Cfg::BN, false> lb;
        lb.K0 = K; lb.K1 = 0; lb.nk0 = nk;
        // rows n < r from b0 (A_gate or A_down), rows r..2r from b1 (A_up)
        lb.b0[0] = static_cast<const T *>(p.b0) + (size_t)tl.e * p.r * K;
        lb.b0[1] = KIND == PROJ_GU ? static_cast<const T *>(p.b1) + (size_t)tl.e * p.r * K : lb.b0[0];
        lb.b1[0] = lb.b1[1] = nullptr;
#pragma unroll
        for (int i = 0; i < lb.PER; ++i) {
            const int n = n_base + lb.row_of(i);
            if (lb.active(i) && n < nr) {
                const int hi = n >= p.r;
                lb.set0(i, (uint32_t)(hi ? n - p.r : n) * K, hi);
            }
        }
        gemm_mainloop<Cfg>(la, lb, nk, sm.a, sm.b, acc);
    } else {
        NLoader<Cfg, Cfg::BN> lb;
        lb.nk0 = nk;
        if (KIND == PROJ_DOUT) {
            // B_d[e] is [d, r]: element (k = model dim, n = rank)
            lb.s0 = NSeg{static_cast<const T *>(p.b0) + (size_t)tl.e * p.d * p.r, nullptr, p.d, p.d, p.r,
                         -n_base, p.r - n_base, 0, 0};
        } else {
            // rows f < F from B_g (columns [0, r)), rows f >= F from B_u (columns [r, 2r))
            const size_t o = (size_t)tl.e * p.F * p.r;
            lb.s0 = NSeg{static_cast<const T *>(p.b0) + o, static_cast<const T *>(p.b1) + o, p.F, 2 * p.F, p.r,
                         -n_base, p.r - n_base, p.r - n_base, 2 * p.r - n_base};
        }
        lb.s1 = lb.s0;
        gemm_mainloop<Cfg>(la, lb, nk, sm.a, sm.b, acc);
    }
    for_each_acc<Cfg>(acc, [&](int m, int n, int, int, int, float v) {
        if (m < tl.rows && n_base + n < nr) p.out[(size_t)(tl.row0 + m) * nr + n_base + n] = v;
    });
    if (p.w_row_out && tl.nt == 0)
        for (int m = threadIdx.x; m < tl.rows; m += Cfg::NTHREADS)
            p.w_row_out[tl.row0 + m] = p.wt[p.sorted_slot[tl.row0 + m]];
    if (p.outT) {
        // the padding columns [S, ldT) are read as operands (times zero rows):
        // they must hold finite values
        const int pad = p.ldT - p.S;
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < nr * pad; i += Cfg::NTHREADS)
                p.outT[(size_t)(i / pad) * p.ldT + p.S + i % pad] = Elem<bf16_t>::from_f32(0.0f);
        for_each_acc<Cfg>(acc, [&](int m, int n, int, int, int, float v) {
            if (m < tl.rows && n_base + n < nr) {
                const int pr = tl.row0 + m;
                const float sc = p.wt ? p.wt[p.sorted_slot[pr]] : 1.0f;
                p.outT[(size_t)(n_base + n) * p.ldT + pr] = Elem<bf16_t>::from_f32(v * sc);
            }
        });
    }
}

// bf16 projections on the direct-load ring: 128-row tiles, 64 output
// columns (nr <= 64 per tile), A rows gathered by token for PROJ_GU and
// PROJ_DOUT, B K-contiguous (A_g | A_u, A_d) or N-contiguous (B_d; B_g and B_u
// as two K segments over the dG and dU columns of dGU, block-diagonal).
using ProjNT = lds::Cfg<128, 64, 4, false>;
using ProjNN = lds::Cfg<128, 64, 4, true>;

template <class C, int KIND>
__global__ __launch_bounds__(256) void k_proj_lds(ProjP p) {
    __shared__ LdsSmem<C> sm;
    constexpr bool GATHER = KIND == PROJ_GU || KIND == PROJ_DOUT;
    const int nr = (KIND == PROJ_GU || KIND == PROJ_DGU) ? 2 * p.r : p.r;
    Tile tl;
    if (p.tiles_out && blockIdx.x == 0) build_row_tiles<256>(p.offsets, p.E, sm.start, p.tiles_out);
    if (!schedule_tile<C::BM, 256>(p.offsets, p.E, cdiv(nr, C::BN), blockIdx.x, sm.start, tl)) return;
    __syncthreads();  // every thread has read the scheduler table
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int n_base = tl.nt * C::BN;
    // A: rows of length lda (elements); K per segment
    const int lda = (KIND == PROJ_GU || KIND == PROJ_DOUT) ? p.d : (KIND == PROJ_D ? p.F : 2 * p.F);
    const int K = (KIND == PROJ_GU || KIND == PROJ_DOUT) ? p.d : p.F;
    const int arows = GATHER ? p.S / p.k : p.S;
    lds::Operands<C, KIND == PROJ_DGU> op;
    uint32_t aro[C::A_INSTR];
#pragma unroll
    for (int j = 0; j < C::A_INSTR; ++j) {
        const int m = lds_row<C>(wave, lane, j, C::A_INSTR);
        const uint32_t row = m < tl.rows ? (GATHER ? (uint32_t)token_of(p.sorted_slot, tl.row0 + m, p.k)
                                                   : (uint32_t)(tl.row0 + m))
                                         : 0u;
        aro[j] = m < tl.rows ? row * (uint32_t)lda * 2u : kInvalid;
    }
    op.a.init_rows(wave, lane, aro);
    op.ra[0] = op.ra[1] = make_rsrc(p.a, (uint32_t)arows * (uint32_t)lda * 2u);
    op.K[0] = op.K[1] = K;
    op.nt0 = op.nt = cdiv(K, C::BK);
    if constexpr (!C::B_NCONTIG) {
        // B rows n: n < r from b0 (A_gate / A_down), r <= n < 2r from b1 (A_up);
        // one load covers 16 rows of one matrix (r is a multiple of 16 here)
        uint32_t bro[C::B_INSTR];
#pragma unroll
        for (int j = 0; j < C::B_INSTR; ++j) {
            const int n = n_base + lds_row<C>(wave, lane, j, C::B_INSTR);
            bro[j] = n < nr ? (uint32_t)(n % p.r) * (uint32_t)K * 2u : kInvalid;
            const int n0 = n_base + (wave * C::B_INSTR + j) * C::RPI;
            op.bsel_mask |= (uint32_t)(KIND == PROJ_GU && n0 >= p.r) << j;
        }
        op.bk.init_rows(wave, lane, bro);
        const size_t bofs = (size_t)tl.e * p.r * K;
        op.rb[0][0] = op.rb[1][0] = make_rsrc(static_cast<const bf16_t *>(p.b0) + bofs, (uint32_t)p.r * K * 2u);
        op.rb[0][1] = op.rb[1][1] =
            make_rsrc(static_cast<const bf16_t *>(KIND == PROJ_GU ? p.b1 : p.b0) + bofs, (uint32_t)p.r * K * 2u);
    } else {
        const size_t bofs = (size_t)tl.e * K * p.r;
        op.ldb[0] = op.ldb[1] = (uint32_t)p.r * 2u;
        if (KIND == PROJ_DOUT) {
            // B_d[e] is [d, r]: k = model dim, columns j < r
            op.bn.init(wave, lane, min(C::BN, p.r - n_base));
            op.rb[0][0] = op.rb[1][0] =
                make_rsrc(static_cast<const bf16_t *>(p.b0) + bofs + n_base, (uint32_t)(K * p.r - n_base) * 2u);
        } else {
            // segment 0: dG (columns [0, F) of dGU) x B_g -> output columns [0, r)
            // segment 1: dU (columns [F, 2F)) x B_u -> output columns [r, 2r)
            op.acol[0] = 0;
            op.acol[1] = (uint32_t)p.F * 2u;
            op.bn.init(wave, lane, max(0, min(C::BN, p.r - n_base)));
            op.bn1.init(wave, lane, min(C::BN, 2 * p.r - n_base), max(0, p.r - n_base));
            const bf16_t *bg = static_cast<const bf16_t *>(p.b0) + bofs;
            const bf16_t *bu = static_cast<const bf16_t *>(p.b1) + bofs;
            op.rb[0][0] = make_rsrc(bg + n_base, (uint32_t)(K * p.r - min(n_base, K * p.r)) * 2u);
            // column n of the tile is column n_base + n - r of B_u (n >= r - n_base only)
            op.rb[1][0] = make_rsrc(bu + (n_base - p.r), (uint32_t)(K * p.r + p.r - n_base) * 2u);
            const int nk = cdiv(K, C::BK);
            const bool has0 = n_base < p.r, has1 = n_base + C::BN > p.r;
            op.nt0 = has0 ? nk : 0;
            op.nt = op.nt0 + (has1 ? nk : 0);
        }
    }
    f32x16_t acc[C::TM][C::TN];
    lds::NoLora nolora;
    lds::run<C>(op, 0, nolora, sm.ring, acc);
    if (p.w_row_out && tl.nt == 0)
        for (int m = threadIdx.x; m < tl.rows; m += 256) p.w_row_out[tl.row0 + m] = p.wt[p.sorted_slot[tl.row0 + m]];
    const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = wm * C::WTM + mi * 32 + acc_row(i, lane);
                const int n = n_base + wn * C::WTN + ni * 32 + acc_col(lane);
                if (m < tl.rows && n < nr) p.out[(size_t)(tl.row0 + m) * nr + n] = acc[mi][ni][i];
            }
    if (p.outT) {
        const int pad = p.ldT - p.S;
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < nr * pad; i += 256)
                p.outT[(size_t)(i / pad) * p.ldT + p.S + i % pad] = Elem<bf16_t>::from_f32(0.0f);
        // Transposed store through LDS (the ring is drained): the tile goes
        // in column-major as fp32, then each wave writes 64 adjacent rows of
        // one column, a run of 128 contiguous bytes of outT, where stores
        // straight from the accumulators put 2 bytes into each of 32 outT rows
        constexpr int P = C::BM + 4;  // float pitch: 16-byte aligned, rotates the banks
        static_assert(C::BN * P * 4 <= C::SMEM_BYTES, "the staged tile fits the ring");
        float *stg = reinterpret_cast<float *>(sm.ring);
#pragma unroll
        for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {  // accumulator rows 4q .. 4q+3 are consecutive
                    const int m = wm * C::WTM + mi * 32 + acc_row(4 * q, lane);
                    const int n = wn * C::WTN + ni * 32 + acc_col(lane);
                    *reinterpret_cast<f32x4_t *>(stg + n * P + m) =
                        f32x4_t{acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                                acc[mi][ni][4 * q + 3]};
                }
        __syncthreads();
        // each thread keeps one row (and its weight) over the columns
        static_assert(256 % C::BM == 0, "whole tile columns per pass");
        const int ncols = min(C::BN, nr - n_base), m = threadIdx.x % C::BM;
        if (m < tl.rows) {
            const int pr = tl.row0 + m;
            const float sc = p.wt ? p.wt[p.sorted_slot[pr]] : 1.0f;
            for (int n = threadIdx.x / C::BM; n < ncols; n += 256 / C::BM)
                p.outT[(size_t)(n_base + n) * p.ldT + pr] = Elem<bf16_t>::from_f32(stg[n * P + m] * sc);
        }
    }
}

// Pgu = sum over the column strips of the down-backward epilogues' shares
// (strip order, fixed), as fp32 [S, 2r] and as the bf16 transpose [2r, ldT]
// the LoRA-gradient kernel reads (columns S .. ldT-1 set to zero). A block
// owns 64 rows; the transpose goes through LDS so each store instruction
// writes 64 consecutive rows of one column.
__global__ __launch_bounds__(256) void k_pgu_sum(const float *__restrict__ part, int nstrip, int S, int r2,
                                                 float *__restrict__ pgu, bf16_t *__restrict__ pguT, int ldT) {
    __shared__ float t[64][65];
    const int row0 = blockIdx.x * 64, nq = r2 / 4;
    const size_t ss = (size_t)S * nq;  // strip stride in float4
    // a thread sums four consecutive j of one row, strip by strip in order;
    // the loads of four strips are issued before their adds
    for (int i = threadIdx.x; i < 64 * nq; i += 256) {
        const int m = i / nq, j = (i % nq) * 4, pr = row0 + m;
        f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (pr < S) {
            const f32x4_t *src = reinterpret_cast<const f32x4_t *>(part + (size_t)pr * r2 + j);
            int sidx = 0;
            for (; sidx + 4 <= nstrip; sidx += 4) {
                const f32x4_t a = src[sidx * ss], b = src[(sidx + 1) * ss], c = src[(sidx + 2) * ss],
                              d = src[(sidx + 3) * ss];
                v += a;
                v += b;
                v += c;
                v += d;
            }
            for (; sidx < nstrip; ++sidx) v += src[sidx * ss];
            *reinterpret_cast<f32x4_t *>(pgu + (size_t)pr * r2 + j) = v;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) t[j + c][m] = v[c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * r2; i += 256) {
        const int j = i / 64, m = i % 64, pr = row0 + m;
        if (pr < S) pguT[(size_t)j * ldT + pr] = Elem<bf16_t>::from_f32(t[j][m]);
    }
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < r2 * (ldT - S); i += 256)
            pguT[(size_t)(i / (ldT - S)) * ldT + S + i % (ldT - S)] = Elem<bf16_t>::from_f32(0.0f);
}

// ===========================================================================
// Weighted combine / dX gather-sum: out[t] = sum_j w[t,j] Y[slot_row[t*k+j]]
// (w = 1 for dX), fp32 accumulation in ascending j.
// ===========================================================================
template <typename T>
__global__ __launch_bounds__(256) void k_combine(const T *__restrict__ Y, const int32_t *__restrict__ slot_row,
                                                 const float *__restrict__ w, int k, int d, T *__restrict__ out) {
    constexpr int VEC = Elem<T>::VEC;
    constexpr int KU = 8;  // choices loaded together (independent loads in flight)
    const int t = blockIdx.x;
    for (int c = threadIdx.x; c < d / VEC; c += blockDim.x) {
        float acc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += KU) {
            chunk_t ch[KU];
            float wj[KU];
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int j = j0 + u;
                const int q = t * k + min(j, k - 1);
                ch[u] = ld_stream(Y + (size_t)slot_row[q] * d + c * VEC);  // each row read once
                wj[u] = j < k ? (w ? w[q] : 1.0f) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < KU; ++u) {  // j ascending
                float y[VEC];
                unpack<T>(ch[u], y);
                if (j0 + u < k) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[v] += wj[u] * y[v];
                }
            }
        }
        st_stream(out + (size_t)t * d + c * VEC, Elem<T>::pack(acc));
    }
}

// ===========================================================================
// Router-weight gradient: d_topk_w[t,j] = <dout[t], Y[row of (t,j)]>, and
// its chain through the softmax over the selected logits:
// d_logits[t, e_j] = w_j (dw_j - sum_i w_i dw_i); zero for unselected experts.
// One wave per token.
// ===========================================================================
template <typename T>
__global__ __launch_bounds__(256) void k_router_grad(const T *__restrict__ dout, const T *__restrict__ Y,
                                                     const int32_t *__restrict__ slot_row,
                                                     const int32_t *__restrict__ topk_idx,
                                                     const float *__restrict__ topk_w, int Tn, int E, int k, int d,
                                                     float *__restrict__ d_topk_w, float *__restrict__ d_logits) {
    constexpr int VEC = Elem<T>::VEC;
    __shared__ float s_dw[4][kMaxE];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int t = blockIdx.x * 4 + wave;
    const bool valid = t < Tn;
    float dot = 0.0f;
    if (valid) {
        // four choices per pass: each dOut chunk is loaded once for the four,
        // and their expert rows (each read once, so non-temporal) are in
        // flight together; each choice sums in the same order as alone
        constexpr int JU = 4;
        const T *gr = dout + (size_t)t * d;
        for (int j0 = 0; j0 < k; j0 += JU) {
            const T *yr[JU];
#pragma unroll
            for (int u = 0; u < JU; ++u) yr[u] = Y + (size_t)slot_row[t * k + min(j0 + u, k - 1)] * d;
            float acc[JU];
#pragma unroll
            for (int u = 0; u < JU; ++u) acc[u] = 0.0f;
            for (int c = lane; c < d / VEC; c += kWave) {
                float a[VEC];
                unpack<T>(*reinterpret_cast<const chunk_t *>(gr + c * VEC), a);
                chunk_t yc[JU];
#pragma unroll
                for (int u = 0; u < JU; ++u) yc[u] = ld_stream(yr[u] + c * VEC);
#pragma unroll
                for (int u = 0; u < JU; ++u) {
                    float b[VEC];
                    unpack<T>(yc[u], b);
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[u] += a[v] * b[v];
                }
            }
#pragma unroll
            for (int u = 0; u < JU; ++u) {
                float a = acc[u];
#pragma unroll
                for (int off = kWave / 2; off > 0; off >>= 1) a += __shfl_xor(a, off, kWave);
                if (j0 + u < k) {  // past k: a repeat of choice k-1, dropped
                    if (lane == 0) s_dw[wave][j0 + u] = a;
                    dot += topk_w[t * k + j0 + u] * a;
                }
            }
        }
    }
    __syncthreads();
    if (!valid) return;
    if (d_topk_w)
        for (int j = lane; j < k; j += kWave) d_topk_w[(size_t)t * k + j] = s_dw[wave][j];
    if (d_logits)
        for (int e = lane; e < E; e += kWave) {
            float v = 0.0f;
            for (int j = 0; j < k; ++j)
                if (topk_idx[(size_t)t * k + j] == e) v = topk_w[(size_t)t * k + j] * (s_dw[wave][j] - dot);
            d_logits[(size_t)t * E + e] = v;
        }
}

// ===========================================================================
// LoRA weight gradients, reduced over each expert's rows (K = rows):
//   mode 0: [dA_g ; dA_u]^T = s Xp^T [Pg | Pu]        (D = d,  nr = 2r)
//   mode 1: [dB_g , dB_u]   = s [dG | dU]^T [Zg | Zu] (D = 2F, nr = 2r, diagonal blocks kept)
//   mode 2: dA_d^T          = s H^T (w P'd)           (D = F,  nr = r)
//   mode 3: dB_d            = s (w dout)^T Zd         (D = d,  nr = r)
// A block takes (expert, chunk of RC rows, D tile); an expert with one chunk
// writes its gradient directly, larger experts write partial sums that the
// finalize kernel adds in chunk order (deterministic). Experts with no rows
// get exact zeros from the finalize kernel.
// ===========================================================================
constexpr int kLoraRC = 1024;  // rows per chunk

struct LGradP {
    const void *big;                 // [*, ldbig] rows (gathered by token if gather)
    const float *small;              // [S, ldsmall] fp32
    const int32_t *sorted_slot, *offsets;
    const float *topk_w;
    float *partial;
    float *out0, *out1;
    int E, k, d, F, r, D, nr, ldbig, ldsmall;
    float s;
    const bf16_t *smallT;            // bf16 path: [nr, ldT] transposed small operand
    int ldT, mode;                   // ldT = S rounded up to a multiple of 8
    int j0;                          // bf16 path: first small-operand column of this slice
};

__device__ __forceinline__ void lgrad_store(int mode, const LGradP &p, int e, int m, int n, float v) {
    switch (mode) {
    case 0:
        if (n < p.r) p.out0[((size_t)e * p.r + n) * p.d + m] = v;
        else p.out1[((size_t)e * p.r + n - p.r) * p.d + m] = v;
        break;
    case 1:
        if (m < p.F && n < p.r) p.out0[((size_t)e * p.F + m) * p.r + n] = v;
        else if (m >= p.F && n >= p.r) p.out1[((size_t)e * p.F + m - p.F) * p.r + n - p.r] = v;
        break;
    case 2: p.out0[((size_t)e * p.r + n) * p.F + m] = v; break;
    default: p.out0[((size_t)e * p.d + m) * p.r + n] = v; break;
    }
}

// The same mapping as strides, set up once per block: element (m, n) of
// expert e goes to (n < split ? o0 : o1) + (n mod split) * sn + (m - mo_h) * sm,
// where half 1 (n >= split) shifts m by mo; mode 1 keeps only the diagonal
// blocks (m < F with n < r, m >= F with n >= r).
struct LgOut {
    float *o0, *o1;
    int split, sn, sm, mo;
    bool diag;
    __device__ LgOut(const LGradP &p, int e) {
        switch (p.mode) {
        case 0:
            o0 = p.out0 + (size_t)e * p.r * p.d; o1 = p.out1 + (size_t)e * p.r * p.d;
            split = p.r; sn = p.d; sm = 1; mo = 0; diag = false; break;
        case 1:
            o0 = p.out0 + (size_t)e * p.F * p.r; o1 = p.out1 + (size_t)e * p.F * p.r;
            split = p.r; sn = 1; sm = p.r; mo = p.F; diag = true; break;
        case 2:
            o0 = o1 = p.out0 + (size_t)e * p.r * p.F;
            split = p.nr; sn = p.F; sm = 1; mo = 0; diag = false; break;
        default:
            o0 = o1 = p.out0 + (size_t)e * p.d * p.r;
            split = p.nr; sn = 1; sm = p.r; mo = 0; diag = false; break;
        }
    }
    __device__ __forceinline__ void store(int m, int n, float v) const {
        const bool h = n >= split;
        if (diag && h != (m >= mo)) return;
        (h ? o1 : o0)[(size_t)(h ? n - split : n) * sn + (size_t)(h ? m - mo : m) * sm] = v;
    }
    // rows m .. m+3 of column n of an output laid out [n][m] (sm == 1, m a
    // multiple of 4): one 16-byte store
    __device__ __forceinline__ void store4m(int m, int n, f32x4_t v) const {
        const bool h = n >= split;
        if (diag && h != (m >= mo)) return;
        *reinterpret_cast<f32x4_t *>((h ? o1 : o0) + (size_t)(h ? n - split : n) * sn + (h ? m - mo : m)) = v;
    }
    // columns n .. n+3 (n a multiple of 4, as split is): one 16-byte store
    // where they are adjacent in memory ([m][n] outputs), four otherwise
    __device__ __forceinline__ void store4(int m, int n, f32x4_t v) const {
        if (sn != 1) {
            for (int u = 0; u < 4; ++u) store(m, n + u, v[u]);
            return;
        }
        const bool h = n >= split;
        if (diag && h != (m >= mo)) return;
        *reinterpret_cast<f32x4_t *>((h ? o1 : o0) + (size_t)(h ? n - split : n) + (size_t)(h ? m - mo : m) * sm) = v;
    }
};

// Transposing loader whose k index is a row p of the current chunk:
// element (k = row, col) is src_row(p)[col], for ROWS tile columns.
template <class Cfg, int ROWS, typename SrcT>
struct RowTLoader {
    using T = typename Cfg::T;
    static constexpr int VEC = Cfg::VEC, NT = Cfg::NTHREADS, BK = Cfg::BK;
    static constexpr int KB = BK / VEC, NB = ROWS / VEC, NBLK = KB * NB;
    static constexpr int PER = (NBLK + NT - 1) / NT;
    const void *base;
    int ld, col0, ncol;          // columns [col0, col0 + ROWS) of rows of length ld; valid < ncol
    int row0, rows, k;           // chunk rows p in [row0, row0 + rows)
    bool gather, wscale;
    const int32_t *sorted_slot;
    const float *topk_w;
    struct Regs { chunk_t c[PER][VEC]; };
    __device__ void load(int kt, Regs &r) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = (int)threadIdx.x + i * NT;
            if (b >= NBLK) continue;
            const int nb = b % NB, kb = b / NB;
            const int c = col0 + nb * VEC;
#pragma unroll
            for (int ii = 0; ii < VEC; ++ii) {
                const int pl = kt * BK + kb * VEC + ii;
                chunk_t v = zero4();
                if (pl < rows && c + VEC <= ncol) {
                    const int pr = row0 + pl;
                    const size_t row = gather ? (size_t)(sorted_slot[pr] / k) : (size_t)pr;
                    if constexpr (sizeof(SrcT) == sizeof(T)) {
                        v = *reinterpret_cast<const chunk_t *>(static_cast<const SrcT *>(base) + row * ld + c);
                    } else {  // fp32 source, T = bf16: 32 bytes -> one chunk
                        const float *src = static_cast<const float *>(base) + row * ld + c;
                        const float sc = wscale ? topk_w[sorted_slot[pr]] : 1.0f;
                        float f[VEC];
#pragma unroll
                        for (int h = 0; h < VEC; ++h) f[h] = src[h] * sc;
                        v = Elem<T>::pack(f);
                    }
                    if constexpr (sizeof(SrcT) == sizeof(T)) {
                        if (wscale) {
                            float f[VEC];
                            unpack<T>(v, f);
                            const float sc = topk_w[sorted_slot[pr]];
#pragma unroll
                            for (int h = 0; h < VEC; ++h) f[h] *= sc;
                            v = Elem<T>::pack(f);
                        }
                    }
                }
                r.c[i][ii] = v;
            }
        }
    }
    __device__ void store(const Regs &r, T *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = (int)threadIdx.x + i * NT;
            if (b >= NBLK) continue;
            const int nb = b % NB, kb = b / NB;
            chunk_t o[VEC];
            NLoader<Cfg, ROWS>::transpose(r.c[i], o);
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj)
                *reinterpret_cast<chunk_t *>(lds + (nb * VEC + jj) * Cfg::LDK + kb * VEC) = o[jj];
        }
    }
};

template <class Cfg, int MODE>
__global__ __launch_bounds__(Cfg::NTHREADS) void k_lora_grad(LGradP p) {
    using T = typename Cfg::T;
    __shared__ Smem<Cfg> sm;
    const int ntm = cdiv(p.D, Cfg::BM), ntn = cdiv(p.nr, Cfg::BN);
    Tile tl;
    if (!schedule_tile<kLoraRC, Cfg::NTHREADS>(p.offsets, p.E, ntm * ntn, blockIdx.x, sm.start, tl)) return;
    const int m_base = (tl.nt % ntm) * Cfg::BM, n_base = (tl.nt / ntm) * Cfg::BN;
    constexpr bool BIG_GATHER = MODE == 0 || MODE == 3;
    constexpr bool SMALL_W = MODE == 2 || MODE == 3;
    RowTLoader<Cfg, Cfg::BM, T> la;
    la.base = p.big; la.ld = p.ldbig; la.col0 = m_base; la.ncol = p.D;
    la.row0 = tl.row0; la.rows = tl.rows; la.k = p.k; la.gather = BIG_GATHER; la.wscale = MODE == 3;
    la.sorted_slot = p.sorted_slot; la.topk_w = p.topk_w;
    RowTLoader<Cfg, Cfg::BN, float> lb;
    lb.base = p.small; lb.ld = p.ldsmall; lb.col0 = n_base; lb.ncol = p.nr;
    lb.row0 = tl.row0; lb.rows = tl.rows; lb.k = p.k; lb.gather = false; lb.wscale = MODE == 2;
    lb.sorted_slot = p.sorted_slot; lb.topk_w = p.topk_w;
    (void)SMALL_W;
    f32x16_t acc[Cfg::TM][Cfg::TN];
    gemm_mainloop<Cfg>(la, lb, cdiv(tl.rows, Cfg::BK), sm.a, sm.b, acc);
    const bool single = (p.offsets[tl.e + 1] - p.offsets[tl.e]) <= kLoraRC;
    for_each_acc<Cfg>(acc, [&](int m, int n, int, int, int, float v) {
        const int gm = m_base + m, gn = n_base + n;
        if (gm < p.D && gn < p.nr) {
            if (single) lgrad_store(MODE, p, tl.e, gm, gn, p.s * v);
            else p.partial[((size_t)tl.gmt * p.D + gm) * p.nr + gn] = v;
        }
    });
}

// bf16 LoRA weight gradients, all modes in one launch. A block takes
// (mode, expert, chunk of up to kLgRC of its rows, a group of lg_ntb tiles
// of 256 columns of the big operand) and forms out^T[j][c] = sum_p SmallT[j][p]
// Big[p][c] tile after tile (the chunk's row table and the tile scheduler's
// work are shared by the block's tiles). Both
// operands stream through a ring of direct loads, one 32-row step per stage:
//  - the big rows (gathered by token for modes 0 and 3), 32 x 256 bf16,
//    N-contiguous, read back with transposing LDS reads;
//  - the matching 32 columns of SmallT, the bf16 [nr, S] transposed copy of
//    the small operand that the projection kernels write (with the combine
//    weight already applied for modes 2 and 3), K-contiguous.
// Rows past the chunk load as zeros on the big side, which zeroes their
// products whatever the SmallT columns hold.
constexpr int kLgRC = 1024;         // rows per chunk
constexpr int kLgRows = kLgRC + 8;   // chunk rows plus the alignment lead-in
constexpr int kLgBN = 256;           // big-operand columns per tile
#ifndef MOE_LG_ITEM
#define MOE_LG_ITEM 2048
#endif
// Column tiles per block (one ring, one row table): about kLgItem / (rows of
// the expert's chunks), at most kLgNTB, so that the blocks' costs stay close
// whatever the routing: an expert of ~500 rows takes 4 tiles a block, the
// full 1024-row chunks of a large expert 2.
constexpr int kLgNTB = 4;
constexpr int kLgItem = MOE_LG_ITEM;
__host__ __device__ constexpr int lg_ntb(int chunk_rows) {
    const int t = (kLgItem + chunk_rows / 2) / chunk_rows;
    return t < 1 ? 1 : (t > kLgNTB ? kLgNTB : t);
}
constexpr int kLgNTBMin = lg_ntb(kLgRC);  // chunks hold at most kLgRC rows

template <int NR> struct LgRing {
    static constexpr int NSTAGE = NR <= 32 ? 4 : 3;
    static constexpr int BIG = 32 * kLgBN * 2;           // 16 KB
    static constexpr int SMALL = NR * 64;                // NR rows j x 32 p
    static constexpr int STAGE = BIG + SMALL;
    static constexpr int SMALL_INSTR = SMALL / 1024;     // 4-byte direct loads (256 B) per wave
    static constexpr int LOADS = 4 + SMALL_INSTR;        // direct loads per wave per step
};

// Slices of the four modes in one launch: a slice covers NR columns j of a
// mode's small operand (nr up to 2r = 512 takes several slices).
constexpr int kLgMaxSlices = 24;
constexpr int kLgSliceMax = 64;  // columns per slice of the NR = 64 kernel (NR = 32 slices take nr <= 32)

// the work-item scheduler's tables (LDS)
struct LgSched {
    int item[kMaxE + 1];   // first work item of each expert in the block's slice
    int chunk[kMaxE + 1];  // first chunk of each expert (over all experts)
    int ntb[kMaxE];        // column tiles per item of each expert
    int tot[kLgMaxSlices]; // items of each slice
};

template <int NR> struct LgSmem {
    union {  // the scheduler's tables are dead once the ring starts
        __align__(16) char ring[LgRing<NR>::NSTAGE * LgRing<NR>::STAGE];
        LgSched sch;
    };
    uint32_t rowoff[kLgRows];  // byte offset of each step row in Big (kInvalid outside the chunk)
};

struct LGradSet {
    LGradP m[kLgMaxSlices];
    int n;
};

template <int NR>
__device__ __forceinline__ void lg_issue(const LGradP &p, int p0, const uint32_t *__restrict__ rowoff, rsrc_t rs,
                                         rsrc_t rsm, int c_base, int ncol, bool live, int t,
                                         char *__restrict__ st, int wave, int lane) {
    using R = LgRing<NR>;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // big: 2 rows of 512 B per 1 KB load
        const int q = wave * 4 + j;
        const int kr = q * 2 + (lane >> 5);
        const int lch = (lane & 31) ^ lds::swz_n<kLgBN>(kr);
        const uint32_t ro = rowoff[min(t * 32 + kr, kLgRows - 1)];
        const uint32_t vo =
            (live && ro != kInvalid && lch * 8 + 8 <= ncol) ? ro + (uint32_t)(c_base + lch * 8) * 2u : kInvalid;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MOE_LDS_PTR(st + q * 1024), 16, vo, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < R::SMALL_INSTR; ++i) {  // SmallT: 4 rows j of 64 B per 256 B load
        const int q = wave * R::SMALL_INSTR + i;
        const int jr = q * 4 + (lane >> 4);
        const int lc = ((lane & 15) >> 2) ^ lds::swz_k(jr);
        const uint32_t pr = (uint32_t)(p0 + t * 32 + lc * 8);  // 8-aligned: 16-byte aligned chunks
        const uint32_t vo = (live && p.j0 + jr < p.nr)
                                ? ((uint32_t)(p.j0 + jr) * (uint32_t)p.ldT + pr) * 2u + (uint32_t)(lane & 3) * 4u
                                : kInvalid;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsm, MOE_LDS_PTR(st + R::BIG + q * 256), 4, vo, 0, 0, 0);
    }
}

// One steady step: the loads of a later step (t, c_base, ncol, live: the
// step NSTAGE - 1 ahead) into `dst` (a different ring slot from `st`, as the
// restrict qualifiers state, so the compiler inserts no vmcnt drain before
// the LDS reads) and the MFMA work of the step in `st`.
template <int NR>
__device__ __forceinline__ void lg_iter(const LGradP &p, int p0, const uint32_t *__restrict__ rowoff, rsrc_t rs,
                                        rsrc_t rsm, int c_base, int ncol, bool live, int t,
                                        char *__restrict__ dst, const char *__restrict__ st, int wave, int lane,
                                        f32x16_t (&acc)[NR / 32][2]) {
    using R = LgRing<NR>;
    constexpr int TM = NR / 32;
    lg_issue<NR>(p, p0, rowoff, rs, rsm, c_base, ncol, live, t, dst, wave, lane);
    const char *sa = st + R::BIG;
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
        chunk_t af[TM], bfr[2];
#pragma unroll
        for (int mi2 = 0; mi2 < TM; ++mi2) {
            const int row = mi2 * 32 + (lane & 31);
            const int c = kg * 2 + (lane >> 5);
            af[mi2] = *reinterpret_cast<const chunk_t *>(sa + row * 64 + ((c ^ lds::swz_k(row)) * 16));
        }
        const int kbase = kg * 16 + (g >> 1) * 8 + (sl >> 2);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const int n = wave * 64 + ni * 32 + (g & 1) * 16 + 4 * (sl & 3);
            lds::s16x4_t h[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int k = kbase + 4 * half;
                h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) lds::s16x4_t *)(st + k * kLgBN * 2 +
                                                                       (((n >> 3) ^ lds::swz_n<kLgBN>(k)) * 16) + (n & 7) * 2));
            }
            bfr[ni] = chunk_t{(uint32_t)(uint16_t)h[0].x | ((uint32_t)(uint16_t)h[0].y << 16),
                              (uint32_t)(uint16_t)h[0].z | ((uint32_t)(uint16_t)h[0].w << 16),
                              (uint32_t)(uint16_t)h[1].x | ((uint32_t)(uint16_t)h[1].y << 16),
                              (uint32_t)(uint16_t)h[1].z | ((uint32_t)(uint16_t)h[1].w << 16)};
        }
#pragma unroll
        for (int mi2 = 0; mi2 < TM; ++mi2)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) Elem<bf16_t>::mma(acc[mi2][ni], af[mi2], bfr[ni]);
    }
}

// Work item of block b. A slice's items are (expert e, group of column
// tiles, chunk of up to kLgRC rows of e), ordered expert-major, then group,
// then chunk; the slices' items follow one another in slice order and the
// blocks past them have no work, so they come last in dispatch order. Items
// run on XCD b mod 8, so each XCD takes every eighth item: items differ in
// cost (tail chunks, groups of fewer tiles), and the items of one chunk read
// disjoint columns of the big operand, so an even spread matters and L2
// locality does not. Sets mi (the slice), tl.e, tl.nt (the group), tl.mt
// (the chunk within e), tl.row0, tl.rows, tl.gmt (the chunk over all
// experts) and ntb (tiles per item of e). Returns false if the block has no
// work; ends with every thread past the tables' last read.
__device__ bool lg_schedule(const LGradSet &set, int b, LgSched &sc, int &mi, Tile &tl, int &ntb) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int *__restrict__ offsets = set.m[0].offsets;  // the slices share the routing
    const int E = set.m[0].E;
    for (int e = tid; e < E; e += 256) {
        const int n = offsets[e + 1] - offsets[e];
        sc.chunk[e + 1] = (n + kLgRC - 1) / kLgRC;
        sc.ntb[e] = n > 0 ? lg_ntb(min(n, kLgRC)) : 1;
    }
    if (tid == 0) sc.chunk[0] = 0;
    __syncthreads();
    for (int m = wave; m < set.n; m += 4) {  // items of each slice, one wave a slice
        const int ntn = cdiv(set.m[m].D, kLgBN);
        int t = 0;
        for (int e = lane; e < E; e += kWave) t += sc.chunk[e + 1] * cdiv(ntn, sc.ntb[e]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, kWave);
        if (lane == 0) sc.tot[m] = t;
    }
    __syncthreads();
    int s = 0, base = 0;
    while (s < set.n && b >= base + sc.tot[s]) base += sc.tot[s++];
    if (s == set.n) return false;  // the same in every thread
    mi = __builtin_amdgcn_readfirstlane(s);
    const int item = b - base, ntn = cdiv(set.m[mi].D, kLgBN);
    for (int e = tid; e < E; e += 256) sc.item[e + 1] = sc.chunk[e + 1] * cdiv(ntn, sc.ntb[e]);
    if (tid == 0) sc.item[0] = 0;
    __syncthreads();
    if (tid < kWave) wave_scan_shared(sc.item, E, tid);
    else if (tid < 2 * kWave) wave_scan_shared(sc.chunk, E, tid - kWave);
    __syncthreads();
    int lo = 0, hi = E;  // invariant: item[lo] <= item < item[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sc.item[mid] <= item) lo = mid; else hi = mid;
    }
    const int e = lo, nch = sc.chunk[e + 1] - sc.chunk[e], rem = item - sc.item[e];
    tl.e = __builtin_amdgcn_readfirstlane(e);
    tl.nt = __builtin_amdgcn_readfirstlane(rem / nch);
    tl.mt = __builtin_amdgcn_readfirstlane(rem % nch);
    tl.row0 = __builtin_amdgcn_readfirstlane(offsets[e] + tl.mt * kLgRC);
    tl.rows = __builtin_amdgcn_readfirstlane(min(kLgRC, offsets[e + 1] - tl.row0));
    tl.gmt = __builtin_amdgcn_readfirstlane(sc.chunk[e] + tl.mt);
    ntb = __builtin_amdgcn_readfirstlane(sc.ntb[e]);
    __syncthreads();  // every thread has read the tables before the ring overwrites them
    return true;
}

template <int NR>
__global__ __launch_bounds__(256) void k_lgrad(LGradSet set) {
    using R = LgRing<NR>;
    __shared__ LgSmem<NR> sm;
    Tile tl;
    int mi, ntb;
    if (!lg_schedule(set, blockIdx.x, sm.sch, mi, tl, ntb)) return;
    const LGradP &p = set.m[mi];
    const int ntn = cdiv(p.D, kLgBN);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool gather = p.mode == 0 || p.mode == 3;
    // the block's column tiles nt0 .. nt0 + ntiles - 1, one after the other
    // through one ring (the next tile's loads are in flight while a tile's
    // results are stored)
    const int nt0 = tl.nt * ntb, ntiles = min(ntb, ntn - nt0);
    // steps start at p0, the chunk's first row rounded down to a multiple of
    // 8, so SmallT columns load as aligned 16-byte chunks; the lead-in rows
    // (previous expert) load as zeros on the big side
    const int p0 = tl.row0 & ~7, lead = tl.row0 - p0;
    for (int i = tid; i < kLgRows; i += 256) {
        uint32_t o = kInvalid;
        if (i >= lead && i < lead + tl.rows) {
            const int pr = p0 + i;
            o = (gather ? (uint32_t)(p.sorted_slot[pr] / p.k) : (uint32_t)pr) * (uint32_t)p.ldbig * 2u;
        }
        sm.rowoff[i] = o;
    }
    __syncthreads();
    // rows are range-checked through rowoff; the range is the 2 GiB every
    // tensor fits, so the last 16-byte chunk of a tensor of exactly 2^31
    // bytes is in range and the kInvalid offset (2^31) is not
    const rsrc_t rs = make_rsrc(p.big, 0x80000000u);
    const rsrc_t rsm = make_rsrc(p.smallT, (uint32_t)p.nr * (uint32_t)p.ldT * 2u);
    const int nsteps = cdiv(lead + tl.rows, 32), total = ntiles * nsteps;
    auto stage = [&](int t) { return sm.ring + (t % R::NSTAGE) * R::STAGE; };
    // global step u -> (column tile, step within it); past the last tile the
    // loads are issued as zeros so every step waits on the same count
    auto issue_at = [&](int u, int &cb, int &nc, bool &live, int &t) {
        live = u < total;
        const int jt = live ? u / nsteps : 0;
        t = live ? u - jt * nsteps : 0;
        cb = (nt0 + jt) * kLgBN;
        nc = min(kLgBN, p.D - cb);
    };
    constexpr int TM = NR / 32;
    f32x16_t acc[TM][2];
#pragma unroll
    for (int mi2 = 0; mi2 < TM; ++mi2)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi2][ni][i] = 0.0f;
#pragma unroll
    for (int u = 0; u < R::NSTAGE - 1; ++u) {
        int cb, nc, t;
        bool live;
        issue_at(u, cb, nc, live, t);
        lg_issue<NR>(p, p0, sm.rowoff, rs, rsm, cb, nc, live, t, stage(u), wave, lane);
    }
    const bool single = (p.offsets[tl.e + 1] - p.offsets[tl.e]) <= kLgRC;
    const LgOut dst(p, tl.e);
    int tt = 0, jt = 0;  // step within the current tile, current tile
    for (int u = 0; u < total; ++u) {
        // every step issues the same loads (zeros past the end): a fixed wait count
        lds::wait_vm<(R::NSTAGE - 2) * R::LOADS>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        int cb, nc, t;
        bool live;
        issue_at(u + R::NSTAGE - 1, cb, nc, live, t);
        lg_iter<NR>(p, p0, sm.rowoff, rs, rsm, cb, nc, live, t, stage(u + R::NSTAGE - 1), stage(u), wave, lane,
                    acc);
        if (++tt < nsteps) continue;
        tt = 0;
        // tile jt done: acc[mi2][ni] holds out^T rows j = mi2*32 + ..,
        // columns c = wave*64 + ni*32 + ..; a lane's accumulator rows 4q ..
        // 4q+3 are four consecutive j of one column m; nr, NR and j0 are
        // multiples of 8, so the four share a fate
        const int c_base = (nt0 + jt) * kLgBN, ncol = min(kLgBN, p.D - c_base);
        ++jt;
#pragma unroll
        for (int mi2 = 0; mi2 < TM; ++mi2)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = p.j0 + mi2 * 32 + acc_row(4 * q, lane);
                    const int cl = wave * 64 + ni * 32 + acc_col(lane);
                    if (j < p.nr && j < p.j0 + NR && cl < ncol) {
                        const int m = c_base + cl;
                        const f32x4_t v{acc[mi2][ni][4 * q], acc[mi2][ni][4 * q + 1], acc[mi2][ni][4 * q + 2],
                                        acc[mi2][ni][4 * q + 3]};
                        if (single) {
                            dst.store4(m, j, p.s * v);
                        } else if (!dst.diag || (j >= dst.split) == (m >= dst.mo)) {
                            // [chunk][j][m]: lanes of consecutive m store 128-byte
                            // runs (the off-diagonal blocks of mode 1 are dropped)
#pragma unroll
                            for (int u = 0; u < 4; ++u) p.partial[((size_t)tl.gmt * p.nr + j + u) * p.D + m] = v[u];
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mi2][ni][i] = 0.0f;
            }
    }
    lds::wait_vm<0>();  // the zero loads of the last steps
}

// Finalize of the bf16 path. A unit is (expert, kLgFinM columns m of the
// big operand); block g of a slice takes units g, g + gridDim.x, ... Units
// of experts with one chunk were written by the gradient kernel and are
// skipped, empty experts get exact zeros, multi-chunk experts the
// chunk-ordered sums of their [chunk][j][m] fp32 partials: a thread sums
// four consecutive m of one j with 16-byte loads, eight chunks' loads in
// flight at a time. Outputs laid out [j][m] take 16-byte stores from
// there; outputs laid out [m][j] go through an LDS transpose and take
// 16-byte stores of four adjacent j. Empty experts' zeros are 16-byte
// stores too.
constexpr int kLgFinM = 64;        // m per unit
constexpr int kLgFinBlocks = 512;  // blocks per slice

__global__ __launch_bounds__(256) void k_lgrad_finalize(LGradSet set) {
    __shared__ int s_chunk[kMaxE + 1];  // first chunk of each expert
    __shared__ float s_t[kLgSliceMax][kLgFinM + 1];
    const LGradP &p = set.m[blockIdx.y];
    const int tid = threadIdx.x;
    constexpr int M4 = kLgFinM / 4;
    const int ntm = cdiv(p.D, kLgFinM), ns = min(p.nr - p.j0, kLgSliceMax);
    {  // leave at once if every unit of the block belongs to an expert of one chunk
        bool need = false;
        for (int u = blockIdx.x + tid * gridDim.x; u < p.E * ntm; u += 256 * gridDim.x) {
            const int n = p.offsets[u / ntm + 1] - p.offsets[u / ntm];
            need = need || n == 0 || n > kLgRC;
        }
        if (!__syncthreads_or(need)) return;
    }
    for (int e = tid; e < p.E; e += 256) s_chunk[e + 1] = cdiv(p.offsets[e + 1] - p.offsets[e], kLgRC);
    if (tid == 0) s_chunk[0] = 0;
    __syncthreads();
    if (tid < kWave) wave_scan_shared(s_chunk, p.E, tid);
    __syncthreads();
    const size_t cs4 = (size_t)p.nr * p.D / 4;  // chunk stride of the partials in 16-byte units
    for (int u = blockIdx.x; u < p.E * ntm; u += gridDim.x) {
        const int e = u / ntm, m0 = (u - e * ntm) * kLgFinM;
        const int c0 = s_chunk[e], nch = s_chunk[e + 1] - c0;
        if (nch == 1) continue;  // uniform per block
        const LgOut dst(p, e);
        const bool mrow = dst.sn == 1;  // output [m][j]
        if (nch == 0) {  // no rows: exact zeros, 16-byte stores in the output's own order
            const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int i = tid; i < ns * M4; i += 256) {
                if (mrow) {  // four adjacent j of one m (ns, j0 and split are multiples of 4)
                    const int ml = i / (ns / 4), m = m0 + ml;
                    if (m < p.D) dst.store4(m, p.j0 + (i - ml * (ns / 4)) * 4, z);
                } else {  // four adjacent m of one j (D is a multiple of 8)
                    const int n = i / M4, m = m0 + (i - n * M4) * 4;
                    if (m < p.D) dst.store4m(m, p.j0 + n, z);
                }
            }
            continue;
        }
        for (int i = tid; i < ns * M4; i += 256) {
            const int n = i / M4, ml = (i - n * M4) * 4, m = m0 + ml, j = p.j0 + n;
            // D is a multiple of 8 and so are split and mo: the four m share a fate
            const bool live = m < p.D && (!dst.diag || (j >= dst.split) == (m >= dst.mo));
            f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (live) {
                const f32x4_t *src = reinterpret_cast<const f32x4_t *>(p.partial + ((size_t)c0 * p.nr + j) * p.D + m);
                int c = 0;
                for (; c + 8 <= nch; c += 8) {
                    f32x4_t a[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) a[q] = src[(size_t)(c + q) * cs4];
#pragma unroll
                    for (int q = 0; q < 8; ++q) v += a[q];  // chunk order
                }
                if (c + 4 <= nch) {
                    f32x4_t a[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) a[q] = src[(size_t)(c + q) * cs4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) v += a[q];
                    c += 4;
                }
                for (; c < nch; ++c) v += src[(size_t)c * cs4];
            }
            v = p.s * v;
            if (mrow) {
#pragma unroll
                for (int q = 0; q < 4; ++q) s_t[n][ml + q] = v[q];
            } else if (live) {
                dst.store4m(m, j, v);
            }
        }
        if (mrow) {
            // LDS-only barriers: the global stores need not land before the
            // next unit, so the waves do not wait for them
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            for (int i = tid; i < ns / 4 * kLgFinM; i += 256) {  // four adjacent j of one m
                const int ml = i / (ns / 4), n = (i - ml * (ns / 4)) * 4, m = m0 + ml;
                if (m < p.D) dst.store4(m, p.j0 + n, f32x4_t{s_t[n][ml], s_t[n + 1][ml], s_t[n + 2][ml], s_t[n + 3][ml]});
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();  // the tile is read before the next unit overwrites it
            asm volatile("" ::: "memory");
        }
    }
}

// Finalize: zeros for empty experts, chunk-ordered sums for multi-chunk experts.
template <int MODE, int RC>
__global__ __launch_bounds__(256) void k_lora_grad_finalize(LGradP p) {
    __shared__ int s_start[kMaxE + 1];
    const int e = blockIdx.y;
    const int ne = p.offsets[e + 1] - p.offsets[e];
    if (ne > 0 && ne <= RC) return;  // written by the GEMM directly
    // chunk start of expert e: sum of ceil(n/RC) over earlier experts
    for (int x = threadIdx.x; x < p.E; x += 256)
        s_start[x] = (p.offsets[x + 1] - p.offsets[x] + RC - 1) / RC;
    __syncthreads();
    int c0 = 0;
    for (int x = 0; x < e; ++x) c0 += s_start[x];
    const int nch = s_start[e];
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= p.D * p.nr) return;
    const int m = idx / p.nr, n = idx % p.nr;
    float v = 0.0f;
    for (int c = 0; c < nch; ++c) v += p.partial[((size_t)(c0 + c) * p.D + m) * p.nr + n];
    lgrad_store(MODE, p, e, m, n, p.s * v);
}

// Partial-sum regions of the four gradient modes (byte offsets; the bf16
// kernel runs the modes concurrently, the fp32 path reuses region 0).
static void lgrad_partial_layout(const Dims &D, size_t off[5]) {
    const size_t tiles = (size_t)max_row_tiles(D.S(), D.E, std::min(kLoraRC, kLgRC));
    const size_t w[4] = {(size_t)D.d * 2 * D.r, (size_t)2 * D.F * 2 * D.r, (size_t)D.F * D.r, (size_t)D.d * D.r};
    off[0] = 0;
    for (int m = 0; m < 4; ++m) off[m + 1] = off[m] + ((tiles * w[m] * sizeof(float) + 255) & ~(size_t)255);
}

size_t lora_grad_partial_bytes(const Dims &D) {
    size_t off[5];
    lgrad_partial_layout(D, off);
    return off[4];
}

// ===========================================================================
// drivers
// ===========================================================================
struct TraceScope {
    const Trace *tr;
    int id;
    hipStream_t st;
    TraceScope(const Trace *t, int i, hipStream_t s) : tr(t), id(i), st(s) {
        if (tr && tr->start[id] && tr->stop[id]) (void)hipEventRecord(tr->start[id], st);
    }
    ~TraceScope() {
        if (tr && tr->start[id] && tr->stop[id]) (void)hipEventRecord(tr->stop[id], st);
    }
};

enum {
    K_PROJ_GU = MOE_K_PROJ_GU, K_GATEUP = MOE_K_GATEUP, K_PROJ_D = MOE_K_PROJ_D, K_DOWN = MOE_K_DOWN,
    K_COMBINE = MOE_K_COMBINE, K_ROUTER_GRAD = MOE_K_ROUTER_GRAD, K_PROJ_DOUT = MOE_K_PROJ_DOUT,
    K_DOWN_BWD = MOE_K_DOWN_BWD, K_PROJ_DGU = MOE_K_PROJ_DGU, K_GATEUP_BWD = MOE_K_GATEUP_BWD,
    K_DX_COMBINE = MOE_K_DX_COMBINE, K_LORA_GRAD = MOE_K_LORA_GRAD
};

// blocks of a grouped-GEMM launch: every work item, plus the phase-split halves
template <class Cfg> static int grid_for(const Dims &D, int BM, int NT) {
    return max_row_tiles(D.S(), D.E, BM) * NT + kPhaseSplitBlocks;
}

#define MOE_LAUNCH(kern, grid, block, ...)                   \
    do {                                                     \
        if ((grid) > 0) {                                    \
            kern<<<dim3(grid), dim3(block), 0, st>>>(__VA_ARGS__); \
            hipError_t _e = hipGetLastError();               \
            if (_e != hipSuccess) return _e;                 \
        }                                                    \
    } while (0)

template <typename T, int KIND>
static hipError_t launch_proj(const Dims &D, const ProjP &pp, hipStream_t st) {
    const int nr = (KIND == PROJ_GU || KIND == PROJ_DGU) ? 2 * D.r : D.r;
    if constexpr (std::is_same<T, bf16_t>::value) {
        if (KIND != PROJ_GU || D.r % 16 == 0) {
            using C = typename std::conditional<KIND == PROJ_DOUT || KIND == PROJ_DGU, ProjNN, ProjNT>::type;
            MOE_LAUNCH((k_proj_lds<C, KIND>), max_row_tiles(D.S(), D.E, C::BM) * cdiv(nr, C::BN), 256, pp);
            return hipSuccess;
        }
    }
    if (nr <= 32) {
        using Cfg = typename SkinnyCfg<T, 32>::type;
        MOE_LAUNCH((k_proj<Cfg, KIND>), grid_for<Cfg>(D, Cfg::BM, cdiv(nr, Cfg::BN)), Cfg::NTHREADS, pp);
    } else {
        using Cfg = typename SkinnyCfg<T, 64>::type;
        MOE_LAUNCH((k_proj<Cfg, KIND>), grid_for<Cfg>(D, Cfg::BM, cdiv(nr, Cfg::BN)), Cfg::NTHREADS, pp);
    }
    return hipSuccess;
}

static Q4P q4_params(const uint8_t *c0, const uint8_t *c1, const float *s0, const float *s1) {
    Q4P q{c0, c1, s0, s1, {}};
    nf4_level_values(q.lv.v);
    return q;
}

template <typename T>
hipError_t run_fwd(const Dims &D, const FwdBufs &b, hipStream_t st, const Trace *tr) {
    using Cfg = typename MainCfg<T>::type;
    if (D.T == 0) return hipSuccess;
    {
        TraceScope ts(tr, K_PROJ_GU, st);
        ProjP pp{b.x, b.ag, b.au, b.sorted_slot, b.offsets, b.Zgu, D.E, D.k, D.d, D.F, D.r,
                 static_cast<bf16_t *>(b.ZguT), nullptr, lgrad_ldT(D), D.S()};
        pp.tiles_out = b.tiles;
        hipError_t e = launch_proj<T, PROJ_GU>(D, pp, st);
        if (e != hipSuccess) return e;
    }
    {
        TraceScope ts(tr, K_GATEUP, st);
        GateUpP gp{b.x, b.wg, b.wu, b.bg, b.bu, b.Zgu, b.sorted_slot, b.offsets, b.G, b.U, b.H,
                   D.T, D.E, D.k, D.d, D.F, D.r, D.s, b.tiles};
        if constexpr (std::is_same<T, bf16_t>::value) {
            if (b.q4) {
                const Q4P q = q4_params(b.q4->cg, b.q4->cu, b.q4->sg, b.q4->su);
                MOE_LAUNCH((k_gateup_q4<LdsNT, LdsNTh>), grid_for<Cfg>(D, LdsNT::BM, cdiv(D.F, LdsNT::BN / 2)),
                           LdsNT::NTHREADS, gp, q);
            } else {
                MOE_LAUNCH((k_gateup_lds<LdsGU, LdsGUh>), grid_for<Cfg>(D, LdsGU::BM, cdiv(D.F, LdsGU::BN / 2)),
                           LdsGU::NTHREADS, gp);
            }
        } else
            MOE_LAUNCH(k_gateup<Cfg>, grid_for<Cfg>(D, Cfg::BM, cdiv(D.F, Cfg::BN / 2)), Cfg::NTHREADS, gp);
    }
    {
        TraceScope ts(tr, K_PROJ_D, st);
        ProjP pp{b.H, b.ad, nullptr, b.sorted_slot, b.offsets, b.Zd, D.E, D.k, D.d, D.F, D.r,
                 static_cast<bf16_t *>(b.wZdT), b.topk_w, lgrad_ldT(D), D.S()};
        hipError_t e = launch_proj<T, PROJ_D>(D, pp, st);
        if (e != hipSuccess) return e;
    }
    {
        TraceScope ts(tr, K_DOWN, st);
        DownP dp{b.H, b.wd, b.bd, b.Zd, b.offsets, b.Y, D.S(), D.E, D.d, D.F, D.r, D.s, b.tiles};
        if constexpr (std::is_same<T, bf16_t>::value) {
            if (b.q4) {
                const Q4P q = q4_params(b.q4->cd, b.q4->cd, b.q4->sd, b.q4->sd);
                MOE_LAUNCH((k_down_q4<LdsNT, LdsNTh>), grid_for<Cfg>(D, LdsNT::BM, cdiv(D.d, LdsNT::BN)),
                           LdsNT::NTHREADS, dp, q);
            } else {
                MOE_LAUNCH((k_down_lds<LdsNT, LdsNTh>), grid_for<Cfg>(D, LdsNT::BM, cdiv(D.d, LdsNT::BN)),
                           LdsNT::NTHREADS, dp);
            }
        } else
            MOE_LAUNCH(k_down<Cfg>, grid_for<Cfg>(D, Cfg::BM, cdiv(D.d, Cfg::BN)), Cfg::NTHREADS, dp);
    }
    {
        TraceScope ts(tr, K_COMBINE, st);
        MOE_LAUNCH(k_combine<T>, D.T, 256, static_cast<const T *>(b.Y), b.slot_row, b.topk_w, D.k, D.d,
                   static_cast<T *>(b.out));
    }
    return hipSuccess;
}

template <int MODE>
static hipError_t launch_lgrad_f32(const Dims &D, const LGradP &lp, hipStream_t st) {
    using T = float;
    const int ntm = cdiv(lp.D, 128);
    if (lp.nr <= 32) {
        using Cfg = typename SkinnyCfg<T, 32>::type;
        MOE_LAUNCH((k_lora_grad<Cfg, MODE>), max_row_tiles(D.S(), D.E, kLoraRC) * ntm * cdiv(lp.nr, Cfg::BN),
                   Cfg::NTHREADS, lp);
    } else {
        using Cfg = typename SkinnyCfg<T, 64>::type;
        MOE_LAUNCH((k_lora_grad<Cfg, MODE>), max_row_tiles(D.S(), D.E, kLoraRC) * ntm * cdiv(lp.nr, Cfg::BN),
                   Cfg::NTHREADS, lp);
    }
    k_lora_grad_finalize<MODE, kLoraRC><<<dim3(cdiv(lp.D * lp.nr, 256), D.E), dim3(256), 0, st>>>(lp);
    return hipGetLastError();
}

// the bf16 modes whose small operand has at most NR columns, in one launch
// The bf16 modes with nr <= 32 (NR = 32) or nr > 32 (NR = 64, in 64-column
// slices), in one launch plus one finalize launch.
template <int NR>
static hipError_t launch_lgrad_set(const Dims &D, const LGradP (&lp)[4], hipStream_t st) {
    LGradSet set{};
    int grid = 0;  // the most items the slices can have together
    for (int m = 0; m < 4; ++m) {
        const bool mine = NR == 32 ? lp[m].nr <= 32 : lp[m].nr > 32;
        if (!mine) continue;
        for (int j0 = 0; j0 < lp[m].nr; j0 += NR) {
            if (set.n == kLgMaxSlices) return hipErrorInvalidValue;
            set.m[set.n] = lp[m];
            set.m[set.n].j0 = j0;
            ++set.n;
            grid += max_row_tiles(D.S(), D.E, kLgRC) * cdiv(cdiv(lp[m].D, kLgBN), kLgNTBMin);
        }
    }
    if (set.n == 0) return hipSuccess;
    MOE_LAUNCH(k_lgrad<NR>, grid, 256, set);
    k_lgrad_finalize<<<dim3(kLgFinBlocks, set.n), dim3(256), 0, st>>>(set);
    return hipGetLastError();
}

template <typename T>
hipError_t run_bwd(const Dims &D, const BwdBufs &b, hipStream_t st, const Trace *tr) {
    using Cfg = typename MainCfg<T>::type;
    const int S = D.S();
    if (D.T > 0 && (b.d_topk_w || b.d_logits)) {
        TraceScope ts(tr, K_ROUTER_GRAD, st);
        MOE_LAUNCH(k_router_grad<T>, cdiv(D.T, 4), 256, static_cast<const T *>(b.dout),
                   static_cast<const T *>(b.Y), b.slot_row, b.topk_idx, b.topk_w, D.T, D.E, D.k, D.d, b.d_topk_w,
                   b.d_logits);
    }
    if (D.T > 0) {
        {
            TraceScope ts(tr, K_PROJ_DOUT, st);
            ProjP pp{b.dout, b.bd, nullptr, b.sorted_slot, b.offsets, b.Pd, D.E, D.k, D.d, D.F, D.r,
                     static_cast<bf16_t *>(b.wPdT), b.topk_w, lgrad_ldT(D), D.S(), b.w_row, b.tiles};
            hipError_t e = launch_proj<T, PROJ_DOUT>(D, pp, st);
            if (e != hipSuccess) return e;
        }
        {
            TraceScope ts(tr, K_DOWN_BWD, st);
            DownBwdP dp{b.dout, b.wd, b.ad, b.G, b.U, b.Pd, b.topk_w, b.sorted_slot, b.offsets, b.dGU,
                        D.T, D.E, D.k, D.d, D.F, D.r, D.s, b.w_row, b.tiles, b.bg, b.bu, b.ppart};
            if constexpr (std::is_same<T, bf16_t>::value) {
                if (b.q4) {
                    const Q4P q = q4_params(b.q4->cd, b.q4->cd, b.q4->sd, b.q4->sd);
                    MOE_LAUNCH((k_down_bwd_q4<LdsNN64, LdsNN64h>), grid_for<Cfg>(D, LdsNN64::BM, cdiv(D.F, LdsNN64::BN)),
                               LdsNN64::NTHREADS, dp, q);
                } else {
                    MOE_LAUNCH((k_down_bwd_lds<LdsNN64, LdsNN64h>), grid_for<Cfg>(D, LdsNN64::BM, cdiv(D.F, LdsNN64::BN)),
                               LdsNN64::NTHREADS, dp);
                }
            } else
                MOE_LAUNCH(k_down_bwd<Cfg>, grid_for<Cfg>(D, Cfg::BM, cdiv(D.F, Cfg::BN)), Cfg::NTHREADS, dp);
        }
        {
            TraceScope ts(tr, K_PROJ_DGU, st);
            if (b.ppart) {
                // the down-backward epilogues left Pgu's column-strip shares
                MOE_LAUNCH(k_pgu_sum, cdiv(S, 64), 256, b.ppart, cdiv(D.F, 256), S, 2 * D.r, b.Pgu,
                           static_cast<bf16_t *>(b.PguT), lgrad_ldT(D));
            } else {
                ProjP pp{b.dGU, b.bg, b.bu, b.sorted_slot, b.offsets, b.Pgu, D.E, D.k, D.d, D.F, D.r,
                         static_cast<bf16_t *>(b.PguT), nullptr, lgrad_ldT(D), D.S()};
                hipError_t e = launch_proj<T, PROJ_DGU>(D, pp, st);
                if (e != hipSuccess) return e;
            }
        }
        {
            TraceScope ts(tr, K_GATEUP_BWD, st);
            GateUpBwdP gp{b.dGU, b.wg, b.wu, b.ag, b.au, b.Pgu, b.offsets, b.dXp, D.S(), D.E, D.d, D.F, D.r, D.s,
                          b.tiles};
            if constexpr (std::is_same<T, bf16_t>::value) {
                if (b.q4) {
                    const Q4P q = q4_params(b.q4->cg, b.q4->cu, b.q4->sg, b.q4->su);
                    MOE_LAUNCH((k_gateup_bwd_q4<LdsNN64, LdsNN64h>), grid_for<Cfg>(D, LdsNN64::BM, cdiv(D.d, LdsNN64::BN)),
                               LdsNN64::NTHREADS, gp, q);
                } else {
                    MOE_LAUNCH((k_gateup_bwd_lds<LdsNN64, LdsNN64h>), grid_for<Cfg>(D, LdsNN64::BM, cdiv(D.d, LdsNN64::BN)),
                               LdsNN64::NTHREADS, gp);
                }
            } else
                MOE_LAUNCH(k_gateup_bwd<Cfg>, grid_for<Cfg>(D, Cfg::BM, cdiv(D.d, Cfg::BN)), Cfg::NTHREADS, gp);
        }
        {
            TraceScope ts(tr, K_DX_COMBINE, st);
            MOE_LAUNCH(k_combine<T>, D.T, 256, static_cast<const T *>(b.dXp), b.slot_row,
                       static_cast<const float *>(nullptr), D.k, D.d, static_cast<T *>(b.dx));
        }
    }
    {
        TraceScope ts(tr, K_LORA_GRAD, st);
        size_t po[5];
        lgrad_partial_layout(D, po);
        const bool bf = std::is_same<T, bf16_t>::value;
        auto part = [&](int m) { return reinterpret_cast<float *>(reinterpret_cast<char *>(b.partial) + (bf ? po[m] : 0)); };
        const LGradP lp[4] = {
            {b.x, b.Pgu, b.sorted_slot, b.offsets, b.topk_w, part(0), b.da_g, b.da_u, D.E, D.k, D.d, D.F, D.r, D.d,
             2 * D.r, D.d, 2 * D.r, D.s, static_cast<const bf16_t *>(b.PguT), lgrad_ldT(D), 0},
            {b.dGU, b.Zgu, b.sorted_slot, b.offsets, b.topk_w, part(1), b.db_g, b.db_u, D.E, D.k, D.d, D.F, D.r,
             2 * D.F, 2 * D.r, 2 * D.F, 2 * D.r, D.s, static_cast<const bf16_t *>(b.ZguT), lgrad_ldT(D), 1},
            {b.H, b.Pd, b.sorted_slot, b.offsets, b.topk_w, part(2), b.da_d, nullptr, D.E, D.k, D.d, D.F, D.r, D.F,
             D.r, D.F, D.r, D.s, static_cast<const bf16_t *>(b.wPdT), lgrad_ldT(D), 2},
            {b.dout, b.Zd, b.sorted_slot, b.offsets, b.topk_w, part(3), b.db_d, nullptr, D.E, D.k, D.d, D.F, D.r, D.d,
             D.r, D.d, D.r, D.s, static_cast<const bf16_t *>(b.wZdT), lgrad_ldT(D), 3}};
        hipError_t e = hipSuccess;
        if constexpr (std::is_same<T, bf16_t>::value) {
            e = launch_lgrad_set<32>(D, lp, st);
            if (e == hipSuccess) e = launch_lgrad_set<64>(D, lp, st);
        } else {
            e = launch_lgrad_f32<0>(D, lp[0], st);
            if (e == hipSuccess) e = launch_lgrad_f32<1>(D, lp[1], st);
            if (e == hipSuccess) e = launch_lgrad_f32<2>(D, lp[2], st);
            if (e == hipSuccess) e = launch_lgrad_f32<3>(D, lp[3], st);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// H = silu(G) U rebuilt from G and U as stored, one 16-byte chunk per
// thread and step (S F is a multiple of 8, so whole chunks): the reload of
// offloaded activations moves G and U only, and the same chunk function as
// the gate/up epilogue makes the rebuilt H bit-identical to the forward's.
template <typename T>
__global__ __launch_bounds__(256) void k_rebuild_h(const chunk_t *__restrict__ G, const chunk_t *__restrict__ U,
                                                   chunk_t *__restrict__ H, size_t nchunk) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nchunk; i += (size_t)gridDim.x * 256)
        st_stream(H + i, swiglu_chunk<T>(ld_stream(G + i), ld_stream(U + i)));
}

template <typename T>
hipError_t run_rebuild_h(size_t elems, const void *G, const void *U, void *H, hipStream_t st) {
    const size_t nchunk = elems * sizeof(T) / sizeof(chunk_t);
    if (nchunk == 0) return hipSuccess;
    const int grid = (int)std::min<size_t>((nchunk + 255) / 256, 8192);
    k_rebuild_h<T><<<dim3(grid), dim3(256), 0, st>>>(static_cast<const chunk_t *>(G), static_cast<const chunk_t *>(U),
                                                     static_cast<chunk_t *>(H), nchunk);
    return hipGetLastError();
}

template hipError_t run_rebuild_h<float>(size_t, const void *, const void *, void *, hipStream_t);
template hipError_t run_rebuild_h<bf16_t>(size_t, const void *, const void *, void *, hipStream_t);
template hipError_t run_fwd<float>(const Dims &, const FwdBufs &, hipStream_t, const Trace *);
template hipError_t run_fwd<bf16_t>(const Dims &, const FwdBufs &, hipStream_t, const Trace *);
template hipError_t run_bwd<float>(const Dims &, const BwdBufs &, hipStream_t, const Trace *);
template hipError_t run_bwd<bf16_t>(const Dims &, const BwdBufs &, hipStream_t, const Trace *);

}  // namespace moe
