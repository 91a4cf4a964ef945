// router.hip - the router projection in front of the routing (the linear gate
// logits = x W_r^T, no bias) and its backward: the router's share of dX and
// the gradient of W_r. The pages start the MoE layer from a per-token routing
// decision over router logits (Unsloth x NVIDIA blog, MoE routing paragraph;
// Unsloth 2026 wiki chapter, "Optimisation 3: grouped_mm and Split-LoRA in
// MoE training", opening paragraph); this is the plain linear gate.
//
// bf16 logits and dW_r run on the direct-load ring (gemm_lds.hpp); dx and
// every fp32 product on the register-staged MFMA tile engine (gemm.hpp),
// tiles of 4 waves (64 x 64 for the logits, else 128 x 128), fp32
// accumulation:
//   logits [T,E]   = x [T,d] . W_r[E,d]^T          (both K-contiguous)
//   dx     [T,d]   = dx_in + d_logits [T,E] . W_r  (d_logits fp32, rounded
//                    to the storage type as it is staged; W_r N-contiguous)
//   dW_r   [E,d]   = d_logits^T . x                (K = tokens: d_logits is
//                    transposed once into the workspace; the token range is
//                    split into chunks whose fp32 partial products are summed
//                    in chunk order, so the result is deterministic)
#include "gemm.hpp"
#include "gemm_lds.hpp"
#include "kernels.hpp"
#include "moe.h"

namespace moe {
namespace {

template <typename T> struct RouterCfg { using type = GemmCfg<T, 128, 128, 32, 2, 2>; };
// dx has K = E only: 64-deep steps halve its chain of dependent steps
template <typename T> struct DxCfg { using type = GemmCfg<T, 128, 128, 64, 2, 2>; };
// the logits have only E columns: 64 x 64 tiles give 4x the blocks of 128 x 128
template <typename T> struct LogitsCfg { using type = GemmCfg<T, 64, 64, 32, 2, 2>; };

template <class Cfg> struct RSmem {
    __align__(16) typename Cfg::T a[2 * Cfg::A_ELEMS];
    __align__(16) typename Cfg::T b[2 * Cfg::B_ELEMS];
};

struct RouterP {
    const void *x, *wr;
    const float *dl;      // d_logits [T,E]
    void *dlT;            // workspace [E,Tp]: d_logits transposed (fp32 for fp32 layers, bf16 for
                          // bf16 layers), zero for T <= t < Tp
    const void *dx_in;
    void *dx;
    float *logits, *dw, *partial;
    int T, d, E, Tp, chunk, nch;
};

// logits = x W_r^T: tile (m0, n0) of [T, E]
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS) void k_router_logits(RouterP p) {
    using T = typename Cfg::T;
    __shared__ RSmem<Cfg> sm;
    const int ntn = cdiv(p.E, Cfg::BN);
    const int m0 = (int)(blockIdx.x / ntn) * Cfg::BM, n0 = (int)(blockIdx.x % ntn) * Cfg::BN;
    const int nk = cdiv(p.d, Cfg::BK);
    KLoader<Cfg, Cfg::BM, false> la;
    la.K0 = p.d; la.K1 = 0; la.nk0 = nk; la.scale1 = 0.0f;
    la.b0[0] = la.b0[1] = static_cast<const T *>(p.x);
    la.b1[0] = la.b1[1] = nullptr;
#pragma unroll
    for (int i = 0; i < la.PER; ++i) {
        const int m = la.row_of(i);
        if (la.active(i) && m0 + m < p.T) la.set0(i, (uint32_t)(m0 + m) * (uint32_t)p.d, 0);
    }
    KLoader<Cfg, Cfg::BN, false> lb;
    lb.K0 = p.d; lb.K1 = 0; lb.nk0 = nk; lb.scale1 = 0.0f;
    lb.b0[0] = lb.b0[1] = static_cast<const T *>(p.wr);
    lb.b1[0] = lb.b1[1] = nullptr;
#pragma unroll
    for (int i = 0; i < lb.PER; ++i) {
        const int n = lb.row_of(i);
        if (lb.active(i) && n0 + n < p.E) lb.set0(i, (uint32_t)(n0 + n) * (uint32_t)p.d, 0);
    }
    f32x16_t acc[Cfg::TM][Cfg::TN];
    gemm_mainloop<Cfg>(la, lb, nk, sm.a, sm.b, acc);
    for_each_acc<Cfg>(acc, [&](int m, int n, int, int, int, float v) {
        if (m0 + m < p.T && n0 + n < p.E) p.logits[(size_t)(m0 + m) * p.E + n0 + n] = v;
    });
}

// bf16 logits on the direct-load ring: 64 x 64 tiles (x rows by experts),
// 32-deep steps through an 8-stage ring, so seven steps of loads (56 KB per
// block) are in flight while one is multiplied. The product is a stream over
// x (W_r stays in L2), and the register-staged engine, which waits on each
// step's loads, reaches a fraction of the HBM rate on it.
using LogitsLds = lds::Cfg<64, 64, 8, false>;

template <class C>
__global__ __launch_bounds__(C::NTHREADS) void k_router_logits_lds(RouterP p) {
    __shared__ __align__(16) char ring[C::SMEM_BYTES];
    // the hardware deals blocks to the 8 XCDs round-robin: each XCD takes a
    // contiguous range of tiles, so the column tiles of one row tile (same x
    // rows) share that XCD's L2; the grid is 8 * per
    const int ntn = cdiv(p.E, C::BN), ntiles = cdiv(p.T, C::BM) * ntn, per = cdiv(ntiles, 8);
    const int tile = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (tile >= ntiles) return;
    const int m0 = (tile / ntn) * C::BM, n0 = (tile % ntn) * C::BN;
    const int lane = (int)threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    lds::Operands<C> op;
    uint32_t aro[C::A_INSTR], bro[C::B_INSTR];
#pragma unroll
    for (int j = 0; j < C::A_INSTR; ++j) {
        const int m = m0 + lds_row<C>(wave, lane, j, C::A_INSTR);
        aro[j] = m < p.T ? (uint32_t)m * (uint32_t)p.d * 2u : kInvalid;
    }
#pragma unroll
    for (int j = 0; j < C::B_INSTR; ++j) {
        const int n = n0 + lds_row<C>(wave, lane, j, C::B_INSTR);
        bro[j] = n < p.E ? (uint32_t)n * (uint32_t)p.d * 2u : kInvalid;
    }
    op.a.init_rows(wave, lane, aro);
    op.bk.init_rows(wave, lane, bro);
    op.ra[0] = op.ra[1] = make_rsrc(p.x, (uint32_t)p.T * (uint32_t)p.d * 2u);
    op.rb[0][0] = op.rb[0][1] = op.rb[1][0] = op.rb[1][1] = make_rsrc(p.wr, (uint32_t)p.E * (uint32_t)p.d * 2u);
    op.K[0] = op.K[1] = p.d;
    op.nt0 = op.nt = cdiv(p.d, C::BK);
    f32x16_t acc[C::TM][C::TN];
    lds::NoLora nolora;
    lds::run<C>(op, 0, nolora, ring, acc);
    // lane: column acc_col of rows acc_row(i) of each 32 x 32 piece, so each
    // store instruction writes 128-byte runs of two rows
    const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + wm * C::WTM + mi * 32 + acc_row(i, lane);
                const int n = n0 + wn * C::WTN + ni * 32 + acc_col(lane);
                if (m < p.T && n < p.E) p.logits[(size_t)m * p.E + n] = acc[mi][ni][i];
            }
}

// dx = dx_in + d_logits W_r: tile (m0, n0) of [T, d], K = E
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS) void k_router_dx(RouterP p) {
    using T = typename Cfg::T;
    __shared__ RSmem<Cfg> sm;
    const int ntn = cdiv(p.d, Cfg::BN);
    const int m0 = (int)(blockIdx.x / ntn) * Cfg::BM, n0 = (int)(blockIdx.x % ntn) * Cfg::BN;
    const int ncol = min(Cfg::BN, p.d - n0);
    // A: only the fp32 segment (rows of d_logits, scale 1)
    KLoader<Cfg, Cfg::BM, true> la;
    la.K0 = 0; la.nk0 = 0; la.K1 = p.E; la.scale1 = 1.0f;
    la.b0[0] = la.b0[1] = static_cast<const T *>(p.wr);  // never read (no segment 0)
    la.b1[0] = la.b1[1] = p.dl;
#pragma unroll
    for (int i = 0; i < la.PER; ++i) {
        const int m = la.row_of(i);
        if (la.active(i) && m0 + m < p.T) la.set1(i, (uint32_t)(m0 + m) * (uint32_t)p.E, 0);
    }
    // B: W_r [E, d], element (k = e, n) at row e, column n0 + n
    NLoader<Cfg, Cfg::BN> lb;
    lb.nk0 = 1 << 30;
    lb.s0 = NSeg{static_cast<const T *>(p.wr) + n0, nullptr, p.E, p.E, p.d, 0, ncol, 0, 0};
    lb.s1 = lb.s0;
    f32x16_t acc[Cfg::TM][Cfg::TN];
    gemm_mainloop<Cfg>(la, lb, cdiv(p.E, Cfg::BK), sm.a, sm.b, acc);
    // Epilogue through LDS (the tiles are dead after the loop's last barrier):
    // each wave parks 32 rows x WTN fp32 of its sub-tile, then every lane adds
    // VEC consecutive columns of one row to dx_in with 16-byte accesses.
    constexpr int VEC = Cfg::VEC, WTN = Cfg::WTN, LPR = WTN / VEC, RPP = 64 / LPR;
    static_assert(32 * WTN * 4 * Cfg::WM * Cfg::WN <= (int)sizeof(RSmem<Cfg>), "staging fits the tiles");
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    float *buf = reinterpret_cast<float *>(&sm) + wave * 32 * WTN;
    const T *dxi = static_cast<const T *>(p.dx_in);
    T *dxo = static_cast<T *>(p.dx);
#pragma unroll
    for (int mi = 0; mi < Cfg::TM; ++mi) {
#pragma unroll
        for (int ni = 0; ni < Cfg::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) buf[acc_row(i, lane) * WTN + ni * 32 + acc_col(lane)] = acc[mi][ni][i];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int pass = 0; pass < 32 / RPP; ++pass) {
            const int r = pass * RPP + lane / LPR, c = (lane % LPR) * VEC;
            const int m = m0 + wm * Cfg::WTM + mi * 32 + r, n = n0 + wn * WTN + c;
            if (m < p.T && n < p.d) {  // d is a multiple of 8: the whole chunk is inside
                const size_t o = (size_t)m * p.d + n;
                float a[VEC];
                unpack<T>(*reinterpret_cast<const chunk_t *>(dxi + o), a);
#pragma unroll
                for (int h = 0; h < VEC; ++h) a[h] += buf[r * WTN + c + h];
                *reinterpret_cast<chunk_t *>(dxo + o) = Elem<T>::pack(a);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next slab
    }
}

// dlT[e][t] = d_logits[t][e] for t < T, 0 for T <= t < Tp; 32 x 32 tiles;
// TO = bf16 rounds to nearest even, as the fp32 product's staging does
template <typename TO>
__global__ __launch_bounds__(256) void k_router_dlT(RouterP p) {
    __shared__ float tile[32][33];
    TO *dlT = static_cast<TO *>(p.dlT);
    const int t0 = (int)blockIdx.x * 32, e0 = (int)blockIdx.y * 32;
    const int tx = (int)threadIdx.x & 31, ty = (int)threadIdx.x >> 5;
#pragma unroll
    for (int i = ty; i < 32; i += 8) {
        const int t = t0 + i, e = e0 + tx;
        tile[i][tx] = (t < p.T && e < p.E) ? p.dl[(size_t)t * p.E + e] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int i = ty; i < 32; i += 8) {
        const int e = e0 + i, t = t0 + tx;
        if (e < p.E && t < p.Tp) dlT[(size_t)e * p.Tp + t] = Elem<TO>::from_f32(tile[tx][i]);
    }
}

// dW_r (one chunk of tokens): tile (m0 = expert, n0 = model dim) of [E, d],
// K = the chunk's tokens; written to dw directly when there is one chunk,
// else to partial[c]
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS) void k_router_dw(RouterP p) {
    using T = typename Cfg::T;
    __shared__ RSmem<Cfg> sm;
    const int ntn = cdiv(p.d, Cfg::BN), ntm = cdiv(p.E, Cfg::BM);
    const int c = (int)blockIdx.x / (ntm * ntn), rem = (int)blockIdx.x % (ntm * ntn);
    const int m0 = (rem / ntn) * Cfg::BM, n0 = (rem % ntn) * Cfg::BN;
    const int t0 = c * p.chunk, kc = min(p.chunk, p.T - t0);
    const int ncol = min(Cfg::BN, p.d - n0);
    // A: rows e of dlT from token t0 (zero-padded past T, so a chunk's last
    // partial vector reads zeros, never the next chunk)
    KLoader<Cfg, Cfg::BM, true> la;
    la.K0 = 0; la.nk0 = 0; la.K1 = kc; la.scale1 = 1.0f;
    la.b0[0] = la.b0[1] = static_cast<const T *>(p.x);  // never read (no segment 0)
    la.b1[0] = la.b1[1] = static_cast<const float *>(p.dlT) + t0;
#pragma unroll
    for (int i = 0; i < la.PER; ++i) {
        const int m = la.row_of(i);
        if (la.active(i) && m0 + m < p.E) la.set1(i, (uint32_t)(m0 + m) * (uint32_t)p.Tp, 0);
    }
    // B: x rows t0 .. t0 + kc - 1, element (k = token, n) at column n0 + n
    NLoader<Cfg, Cfg::BN> lb;
    lb.nk0 = 1 << 30;
    lb.s0 = NSeg{static_cast<const T *>(p.x) + (size_t)t0 * p.d + n0, nullptr, kc, kc, p.d, 0, ncol, 0, 0};
    lb.s1 = lb.s0;
    f32x16_t acc[Cfg::TM][Cfg::TN];
    gemm_mainloop<Cfg>(la, lb, cdiv(kc, Cfg::BK), sm.a, sm.b, acc);
    float *dst = p.nch == 1 ? p.dw : p.partial + (size_t)c * p.E * p.d;
    for_each_acc<Cfg>(acc, [&](int m, int n, int, int, int, float v) {
        if (m0 + m < p.E && n0 + n < p.d) dst[(size_t)(m0 + m) * p.d + n0 + n] = v;
    });
}

// bf16 dW_r (one chunk of tokens) on the direct-load ring: tile of 128
// experts x 128 model columns; A = the experts' rows of the bf16 transposed
// d_logits over the chunk's tokens (K-contiguous), B = the chunk's x rows as
// k-rows (N-contiguous, read with transposing LDS reads), so x streams
// through once. A 16-byte A chunk may run past the chunk's last token into
// the next chunk's; the B k-rows past the chunk read as zero, so those
// products vanish. Written to dw directly when there is one chunk, else to
// partial[c].
using DwLds = lds::Cfg<128, 128, 5, true>;

template <class C>
__global__ __launch_bounds__(C::NTHREADS) void k_router_dw_lds(RouterP p) {
    __shared__ __align__(16) char ring[C::SMEM_BYTES];
    const int ntn = cdiv(p.d, C::BN), ntm = cdiv(p.E, C::BM);
    const int c = (int)blockIdx.x / (ntm * ntn), rem = (int)blockIdx.x % (ntm * ntn);
    const int m0 = (rem / ntn) * C::BM, n0 = (rem % ntn) * C::BN;
    const int t0 = c * p.chunk, kc = min(p.chunk, p.T - t0);
    const int lane = (int)threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    lds::Operands<C> op;
    uint32_t aro[C::A_INSTR];
#pragma unroll
    for (int j = 0; j < C::A_INSTR; ++j) {
        const int e = m0 + lds_row<C>(wave, lane, j, C::A_INSTR);
        aro[j] = e < p.E ? (uint32_t)e * (uint32_t)p.Tp * 2u : kInvalid;
    }
    op.a.init_rows(wave, lane, aro);
    op.ra[0] = op.ra[1] = make_rsrc(p.dlT, (uint32_t)p.E * (uint32_t)p.Tp * 2u);
    op.acol[0] = op.acol[1] = (uint32_t)t0 * 2u;
    op.K[0] = op.K[1] = kc;
    op.nt0 = op.nt = cdiv(kc, C::BK);
    op.bn.init(wave, lane, min(C::BN, p.d - n0));
    op.ldb[0] = op.ldb[1] = (uint32_t)p.d * 2u;
    const bf16_t *xb = static_cast<const bf16_t *>(p.x) + (size_t)t0 * p.d + n0;
    op.rb[0][0] = op.rb[0][1] = op.rb[1][0] = op.rb[1][1] =
        make_rsrc(xb, (uint32_t)((size_t)(p.T - t0) * p.d - n0) * 2u);
    f32x16_t acc[C::TM][C::TN];
    lds::NoLora nolora;
    lds::run<C>(op, 0, nolora, ring, acc);
    float *dst = p.nch == 1 ? p.dw : p.partial + (size_t)c * p.E * p.d;
    const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + wm * C::WTM + mi * 32 + acc_row(i, lane);
                const int n = n0 + wn * C::WTN + ni * 32 + acc_col(lane);
                if (m < p.E && n < p.d) dst[(size_t)m * p.d + n] = acc[mi][ni][i];
            }
}

// dw = sum of the chunk partials in chunk order (zeros when there are no tokens)
__global__ __launch_bounds__(256) void k_router_dw_sum(RouterP p) {
    const size_t n = (size_t)p.E * p.d;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        float acc = 0.0f;
        for (int c = 0; c < p.nch; ++c) acc += p.partial[(size_t)c * n + i];
        p.dw[i] = acc;
    }
}

struct Scope {  // event pair around one launch, if asked for
    const Trace *tr; int id; hipStream_t st;
    Scope(const Trace *t, int i, hipStream_t s) : tr(t), id(i), st(s) {
        if (tr && tr->start[id] && tr->stop[id]) (void)hipEventRecord(tr->start[id], st);
    }
    ~Scope() { if (tr && tr->start[id] && tr->stop[id]) (void)hipEventRecord(tr->stop[id], st); }
};

#define MOE_RLAUNCH(kern, grid, block, ...)                                 \
    do {                                                                    \
        kern<<<(grid), dim3(block), 0, st>>>(__VA_ARGS__);                  \
        const hipError_t _e = hipGetLastError();                            \
        if (_e != hipSuccess) return _e;                                    \
    } while (0)

}  // namespace

RouterWs router_ws(const Dims &D) {
    RouterWs w{};
    w.Tp = (D.T + 7) & ~7;
    // token chunks: enough for about 256 blocks of 128 x 128 dW_r tiles, at
    // most 32, at least about 256 tokens each
    const int tiles = cdiv(D.E, 128) * cdiv(D.d, 128);
    const int nch0 = D.T > 0 ? min(min(32, cdiv(256, tiles)), max(1, cdiv(D.T, 256))) : 1;
    w.chunk = D.T > 0 ? ((D.T + nch0 - 1) / nch0 + 31) & ~31 : 32;
    w.nch = D.T > 0 ? (D.T + w.chunk - 1) / w.chunk : 1;
    w.dlT_bytes = (size_t)D.E * w.Tp * sizeof(float);
    w.partial_bytes = w.nch > 1 ? (size_t)w.nch * D.E * D.d * sizeof(float) : 0;
    return w;
}

template <typename T>
hipError_t run_router_fwd(const Dims &D, const void *x, const void *wr, float *logits, hipStream_t st,
                          const Trace *tr) {
    using Cfg = typename LogitsCfg<T>::type;
    if (D.T == 0) return hipSuccess;
    RouterP p{};
    p.x = x; p.wr = wr; p.logits = logits; p.T = D.T; p.d = D.d; p.E = D.E;
    Scope sc(tr, MOE_K_ROUTER_LOGITS, st);
    if constexpr (std::is_same<T, bf16_t>::value) {
        using C = LogitsLds;
        MOE_RLAUNCH(k_router_logits_lds<C>, dim3(8 * cdiv(cdiv(D.T, C::BM) * cdiv(D.E, C::BN), 8)), C::NTHREADS, p);
    } else {
        MOE_RLAUNCH(k_router_logits<Cfg>, dim3(cdiv(D.T, Cfg::BM) * cdiv(D.E, Cfg::BN)), Cfg::NTHREADS, p);
    }
    return hipSuccess;
}

template <typename T>
hipError_t run_router_bwd(const Dims &D, const void *x, const void *wr, const float *d_logits, const void *dx_in,
                          void *dx, float *dw, void *dlT, void *partial, hipStream_t st, const Trace *tr) {
    using Cfg = typename RouterCfg<T>::type;
    const RouterWs w = router_ws(D);
    RouterP p{};
    p.x = x; p.wr = wr; p.dl = d_logits; p.dlT = dlT; p.dx_in = dx_in; p.dx = dx;
    p.dw = dw; p.partial = static_cast<float *>(partial);
    p.T = D.T; p.d = D.d; p.E = D.E; p.Tp = w.Tp; p.chunk = w.chunk; p.nch = w.nch;
    if (dx && D.T > 0) {
        Scope sc(tr, MOE_K_ROUTER_DX, st);
        using CfgX = typename DxCfg<T>::type;
        MOE_RLAUNCH(k_router_dx<CfgX>, dim3(cdiv(D.T, CfgX::BM) * cdiv(D.d, CfgX::BN)), CfgX::NTHREADS, p);
    }
    if (dw) {
        Scope sc(tr, MOE_K_ROUTER_DW, st);
        if (D.T == 0) {  // an empty sum: zeros
            p.nch = 0;
            MOE_RLAUNCH(k_router_dw_sum, dim3(min(1024, cdiv(D.E * D.d, 256))), 256, p);
            return hipSuccess;
        }
        MOE_RLAUNCH(k_router_dlT<T>, dim3(cdiv(w.Tp, 32), cdiv(D.E, 32)), 256, p);
        if constexpr (std::is_same<T, bf16_t>::value) {
            using C = DwLds;
            MOE_RLAUNCH(k_router_dw_lds<C>, dim3(w.nch * cdiv(D.E, C::BM) * cdiv(D.d, C::BN)), C::NTHREADS, p);
        } else {
            MOE_RLAUNCH(k_router_dw<Cfg>, dim3(w.nch * cdiv(D.E, Cfg::BM) * cdiv(D.d, Cfg::BN)), Cfg::NTHREADS, p);
        }
        if (w.nch > 1) MOE_RLAUNCH(k_router_dw_sum, dim3(min(1024, cdiv(D.E * D.d, 256))), 256, p);
    }
    return hipSuccess;
}

template hipError_t run_router_fwd<float>(const Dims &, const void *, const void *, float *, hipStream_t, const Trace *);
template hipError_t run_router_fwd<bf16_t>(const Dims &, const void *, const void *, float *, hipStream_t, const Trace *);
template hipError_t run_router_bwd<float>(const Dims &, const void *, const void *, const float *, const void *, void *,
                                          float *, void *, void *, hipStream_t, const Trace *);
template hipError_t run_router_bwd<bf16_t>(const Dims &, const void *, const void *, const float *, const void *, void *,
                                           float *, void *, void *, hipStream_t, const Trace *);

}  // namespace moe
