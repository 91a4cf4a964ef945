// gemm_lds.hpp - bf16 grouped-GEMM engine for gfx950 built on direct
// global->LDS loads and transposing LDS reads.
//
// Tile: BM x BN per workgroup of WM x WN waves: 2 x 2 waves of 128 x 128 for
// the 256 x 256 shape (16 v_mfma_f32_32x32x16_bf16 accumulators, 256
// registers, one wave per SIMD) or 2 x 4 waves of 128 x 64 (8 accumulators,
// two waves per SIMD). K advances BK (32 or 64) per step through a ring of LDS
// stages or operand slots filled by buffer_load_dwordx4 ... lds (no staging
// registers), with later steps in flight while one is multiplied.
//
// LDS layouts (byte offsets inside a stage):
//  K-contiguous operand [rows][BK]: 64-byte rows of 4 16-byte chunks; chunk c
//    of row r sits at physical chunk c ^ ((r >> 2) & 3). The LDS serves a
//    16-byte read for 16 lanes (16 consecutive rows, one chunk column) per
//    cycle across 64 banks; with this swizzle those 16 rows hit 16 distinct
//    16-byte bank groups (measured: half of all LDS cycles were conflicts
//    with a swizzle that only separated 8 rows).
//  N-contiguous operand [BK][BN] (k-rows of BN elements): 16-byte chunk c of
//    k-row k sits at physical chunk c ^ (4 * (k & 3)). A ds_read_b64_tr_b16
//    cycle serves 32 lanes = 4 k-rows x 4 chunks; the XOR puts them in 16
//    distinct 16-byte bank groups.
// A direct load writes 1 KB contiguous per wave instruction (lane l at 16 l),
// so each lane loads the global chunk that belongs at its LDS slot.
#pragma once

#include <utility>

#include "gemm.hpp"

namespace moe {
namespace lds {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
#define MOE_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int BM_, int BN_, int NSTAGE_, bool BN_CONTIG_, int BK_ = 32, int WM_ = 2, int WN_ = 2>
struct Cfg {
    using T = bf16_t;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, NSTAGE = NSTAGE_;
    static constexpr bool B_NCONTIG = BN_CONTIG_;
    static constexpr int WM = WM_, WN = WN_, NWAVES = WM_ * WN_, NTHREADS = 64 * NWAVES;
    static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
    static constexpr int NKG = BK / 16;                      // 16-deep MFMA k groups per step
    static constexpr int CPR = BK / 8;                       // 16-byte chunks per K-contig row
    static constexpr int RPI = 64 / CPR;                     // K-contig rows per 1 KB load
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_INSTR = A_BYTES / 1024 / NWAVES;  // direct loads per wave per step
    static constexpr int B_INSTR = B_BYTES / 1024 / NWAVES;
    static constexpr int LOADS_PER_STEP = A_INSTR + B_INSTR;
    static constexpr int KROWS_PER_INSTR = 1024 / (BN * 2);  // N-contig k-rows per 1 KB
    // The rank-r LoRA tiles always use 32-deep steps (LoraCfg) and go
    // through one ring slot before the K loop.
    using LoraCfg = Cfg<BM_, BN_, NSTAGE_, BN_CONTIG_, 32, WM_, WN_>;
    // 32-deep steps: a ring of NSTAGE whole stages (A and B of one step).
    // 64-deep steps (SPLIT): a ring of NSTAGE operand slots, each holding the
    // A tile or the B tile of one step (or the LoRA tile), so the B tiles can
    // be loaded two steps ahead and the A tiles one step ahead.
    static constexpr bool SPLIT = BK == 64;
    static constexpr int SLOT_BYTES = SPLIT ? cmax(cmax(A_BYTES, B_BYTES), (BM + BN) * 32 * 2) : STAGE_BYTES;
    static constexpr int SMEM_BYTES = NSTAGE * SLOT_BYTES;
    static_assert(!SPLIT || NSTAGE == 5, "the split ring holds five operand slots");
    static_assert(A_BYTES % (1024 * NWAVES) == 0 && B_BYTES % (1024 * NWAVES) == 0, "whole loads per wave");
    static_assert(CPR == 4 || CPR == 8, "64- or 128-byte K-contig rows");
    static_assert(!B_NCONTIG || (BN * 2) % 1024 == 0 || 1024 % (BN * 2) == 0, "k-rows tile 1 KB loads");
};

// K-contiguous rows: XOR the 16-byte chunk index by (row >> 2) & 3 (64-byte
// rows) or (row >> 1) & 7 (128-byte rows): 16 consecutive rows of one
// logical chunk then hit 16 distinct 16-byte bank groups
template <int CPR> __device__ __forceinline__ int swz_kc(int row) {
    return CPR == 4 ? (row >> 2) & 3 : (row >> 1) & 7;
}
__device__ __forceinline__ int swz_k(int row) { return swz_kc<4>(row); }
// N-contiguous k-rows: XOR the 16-byte chunk index by 4 (k & 3) (rows of at
// least 16 chunks) or by 4 (k & 1) (8-chunk rows of 64-column tiles)
template <int BN> __device__ __forceinline__ int swz_n(int krow) {
    static_assert(BN >= 64, "at least 8 chunks per k-row");
    return BN >= 128 ? 4 * (krow & 3) : 4 * (krow & 1);
}

// ---------------------------------------------------------------------------
// Direct loads of one K-contiguous operand tile (ROWS x BK) into LDS.
// Each thread owns INSTR rows (one per wave instruction); their byte offsets
// (row start + segment column base handled by the caller) are fixed for the
// whole K loop.
template <int ROWS, int INSTR, int CPR = 4>
struct KDirect {
    static constexpr int RPI = 64 / CPR;  // rows per 1 KB load
    uint32_t off[INSTR];   // byte offset of the thread's row, kInvalid if outside
    int pchunk;            // this lane's physical chunk within its row
    // chunk of the row this lane fetches: logical = physical ^ swizzle(row)
    int lchunk[INSTR];

    __device__ void init_rows(int wave, int lane, const uint32_t (&rowoff)[INSTR]) {
        pchunk = lane % CPR;
#pragma unroll
        for (int j = 0; j < INSTR; ++j) {
            const int row = (wave * INSTR + j) * RPI + lane / CPR;
            lchunk[j] = pchunk ^ swz_kc<CPR>(row);
            off[j] = rowoff[j];
        }
    }

    // issue loads [J0, J1) of the INSTR of one step (k elements [k0, k0 + 8 CPR)
    // of the segment, valid for k < K) into the stage region at `lds`
    template <int J0 = 0, int J1 = INSTR>
    __device__ __forceinline__ void issue(rsrc_t rs, uint32_t colbytes, int k0, int K, char *lds, int wave) const {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int k = k0 + lchunk[j] * 8;
            const uint32_t vo = (off[j] != kInvalid && k < K) ? off[j] + colbytes + (uint32_t)k * 2 : kInvalid;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MOE_LDS_PTR(lds + (wave * INSTR + j) * 1024), 16, vo, 0, 0, 0);
        }
    }
};

// Direct loads of one N-contiguous operand tile (BK k-rows x BN) into LDS:
// element (k, n) of the segment at byte k * ldb + n * 2 of the descriptor
// (the descriptor base already at the tile's first column).
template <int BN, int INSTR>
struct NDirect {
    static constexpr int KR = 1024 / (BN * 2);  // k-rows per 1 KB instruction
    int krow[INSTR];
    int ncol_off[INSTR];   // element offset n of this lane's chunk
    bool nok[INSTR];

    // tile columns [c_lo, c_hi) are loaded (8-aligned bounds), the rest read as zero
    __device__ void init(int wave, int lane, int ncol, int c_lo = 0) {
#pragma unroll
        for (int j = 0; j < INSTR; ++j) {
            const int q = wave * INSTR + j;
            const int byte = lane * 16;               // within the 1 KB block
            krow[j] = q * KR + byte / (BN * 2);
            const int pch = (byte % (BN * 2)) / 16;   // physical chunk in the k-row
            const int lch = pch ^ swz_n<BN>(krow[j]);
            ncol_off[j] = lch * 8;
            nok[j] = ncol_off[j] >= c_lo && ncol_off[j] + 8 <= ncol;
        }
    }
    template <int J0 = 0, int J1 = INSTR>
    __device__ __forceinline__ void issue(rsrc_t rs, uint32_t ldb, int k0, int K, char *lds, int wave) const {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            const int k = k0 + krow[j];
            const uint32_t vo = (nok[j] && k < K) ? (uint32_t)k * ldb + (uint32_t)ncol_off[j] * 2 : kInvalid;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MOE_LDS_PTR(lds + (wave * INSTR + j) * 1024), 16, vo, 0, 0, 0);
        }
    }
};

// ---------------------------------------------------------------------------
// Register-staged stores into the same layouts (used for the rank-r LoRA
// tile, whose A side is fp32 scaled by s and so cannot be loaded directly).
// K-contiguous: chunk (row, logical c) -> physical c ^ swz_k(row).
template <int CPR = 4>
__device__ __forceinline__ void st_kcontig(char *lds, int row, int c, const chunk_t &v) {
    *reinterpret_cast<chunk_t *>(lds + row * CPR * 16 + ((c ^ swz_kc<CPR>(row)) * 16)) = v;
}
// N-contiguous: 8 consecutive n at (k, n0) -> physical chunk (n0 / 8) ^ swz_n(k).
template <int BN>
__device__ __forceinline__ void st_ncontig(char *lds, int k, int n0, const chunk_t &v) {
    *reinterpret_cast<chunk_t *>(lds + k * BN * 2 + (((n0 >> 3) ^ swz_n<BN>(k)) * 16)) = v;
}

// ---------------------------------------------------------------------------
// MFMA work of one K step out of a stage.
// MFMA operand fragments of one 16-deep k group of a step, for one wave.
template <class C> struct Frags {
    chunk_t a[C::TM], b[C::TN];
};

// LDS reads of the fragments of k group kg (k = 16 kg .. 16 kg + 15 of the step).
template <class C>
__device__ __forceinline__ void read_frags(const char *sa, const char *sb, int kg, Frags<C> &f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    // A fragments: row (wm*WTM + mi*32 + lane%32), logical chunk kg*2 + lane/32
    const int arow0 = wm * C::WTM + (lane & 31);
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi) {
        const int row = arow0 + mi * 32;
        const int c = kg * 2 + (lane >> 5);
        f.a[mi] = *reinterpret_cast<const chunk_t *>(sa + row * C::CPR * 16 + ((c ^ swz_kc<C::CPR>(row)) * 16));
    }
    if constexpr (!C::B_NCONTIG) {
        const int brow0 = wn * C::WTN + (lane & 31);
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) {
            const int row = brow0 + ni * 32;
            const int c = kg * 2 + (lane >> 5);
            f.b[ni] = *reinterpret_cast<const chunk_t *>(sb + row * C::CPR * 16 + ((c ^ swz_kc<C::CPR>(row)) * 16));
        }
    } else {
        // transposing reads: 16-lane group g gets 4 k of 16 columns per read
        const int g = lane >> 4, s = lane & 15;
        const int kbase = kg * 16 + (g >> 1) * 8 + (s >> 2);
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) {
            const int n = wn * C::WTN + ni * 32 + (g & 1) * 16 + 4 * (s & 3);
            s16x4_t h[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int k = kbase + 4 * half;
                const char *p = sb + k * C::BN * 2 + (((n >> 3) ^ swz_n<C::BN>(k)) * 16) + (n & 7) * 2;
                h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)(p));
            }
            f.b[ni] = chunk_t{(uint32_t)(uint16_t)h[0].x | ((uint32_t)(uint16_t)h[0].y << 16),
                              (uint32_t)(uint16_t)h[0].z | ((uint32_t)(uint16_t)h[0].w << 16),
                              (uint32_t)(uint16_t)h[1].x | ((uint32_t)(uint16_t)h[1].y << 16),
                              (uint32_t)(uint16_t)h[1].z | ((uint32_t)(uint16_t)h[1].w << 16)};
        }
    }
}

template <class C>
__device__ __forceinline__ void mma_frags(const Frags<C> &f, f32x16_t (&acc)[C::TM][C::TN]) {
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni) Elem<bf16_t>::mma(acc[mi][ni], f.a[mi], f.b[ni]);
}

// One whole step (both k groups) from one stage.
template <class C>
__device__ __forceinline__ void mma_step(const char *sa, const char *sb, f32x16_t (&acc)[C::TM][C::TN]) {
#pragma unroll
    for (int kg = 0; kg < C::NKG; ++kg) {
        Frags<C> f;
        read_frags<C>(sa, sb, kg, f);
        mma_frags<C>(f, acc);
    }
}

// wait until at most N direct loads of this wave are outstanding
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace lds
}  // namespace moe

namespace moe {
namespace lds {

// Operands of one grouped-GEMM tile for the ring driver below. Up to two K
// segments; step t < nt0 is segment 0 at k = BK t, else segment 1.
template <class C, bool NSPLIT = false>
struct Operands {
    KDirect<C::BM, C::A_INSTR, C::CPR> a;
    rsrc_t ra[2];
    uint32_t acol[2] = {0, 0};     // byte column base of the A rows per segment
    int K[2] = {0, 0};
    int nt0 = 0, nt = 0;
    // B, K-contiguous: rows through rb[seg][sel] with sel a per-instruction
    // choice (bit j of bsel_mask for this wave)
    KDirect<C::BN, C::B_INSTR, C::CPR> bk;
    uint32_t bsel_mask = 0;
    // B, N-contiguous (bn1: segment 1's columns, used when NSPLIT)
    NDirect<C::BN, C::B_INSTR> bn, bn1;
    uint32_t ldb[2] = {0, 0};
    rsrc_t rb[2][2];

    // Loads of step t (A tile into `sa`, B tile into `sb`). Steps at or
    // beyond nt load zeros (every offset out of range), so the steady loop can
    // issue unconditionally. Operands are used as values (no runtime index
    // into the arrays: that would put the descriptors in scratch).
    template <int J0 = 0, int J1 = C::A_INSTR>
    __device__ __forceinline__ void issue_a(int t, char *sa, int wave) const {
        const bool s1 = t >= nt0;
        const int k0 = (s1 ? t - nt0 : t) * C::BK;
        const int Ks = t < nt ? (s1 ? K[1] : K[0]) : 0;
        const rsrc_t ra0 = ra[0], ra1 = ra[1];
        const uint32_t ac0 = acol[0], ac1 = acol[1];
        a.template issue<J0, J1>(s1 ? ra1 : ra0, s1 ? ac1 : ac0, k0, Ks, sa, wave);
    }
    template <int J0 = 0, int J1 = C::B_INSTR>
    __device__ __forceinline__ void issue_b(int t, char *sb, int wave) const {
        const bool s1 = t >= nt0;
        const int k0 = (s1 ? t - nt0 : t) * C::BK;
        const int Ks = t < nt ? (s1 ? K[1] : K[0]) : 0;
        const rsrc_t r00 = rb[0][0], r01 = rb[0][1], r10 = rb[1][0], r11 = rb[1][1];
        const uint32_t lb0 = ldb[0], lb1 = ldb[1];
        if constexpr (C::B_NCONTIG) {
            if (NSPLIT && s1) bn1.template issue<J0, J1>(r10, lb1, k0, Ks, sb, wave);
            else bn.template issue<J0, J1>(s1 ? r10 : r00, s1 ? lb1 : lb0, k0, Ks, sb, wave);
        } else {
#pragma unroll
            for (int j = J0; j < J1; ++j) {
                const bool sel = (bsel_mask >> j) & 1u;
                const rsrc_t d = s1 ? (sel ? r11 : r10) : (sel ? r01 : r00);
                const int k = k0 + bk.lchunk[j] * 8;
                const uint32_t vo = (bk.off[j] != kInvalid && k < Ks) ? bk.off[j] + (uint32_t)k * 2 : kInvalid;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(d, MOE_LDS_PTR(sb + (wave * C::B_INSTR + j) * 1024), 16, vo,
                                                         0, 0, 0);
            }
        }
    }
    // both tiles of step t into one stage (A first, then B)
    __device__ __forceinline__ void issue(int t, char *stage, int wave) const {
        issue_a(t, stage, wave);
        issue_b(t, stage + C::A_BYTES, wave);
    }
};

template <int N> struct KGroup { static constexpr int value = N; };

// One 16-deep k group of a step out of its A tile `sa` and B tile `sb`,
// skewed by one group: the LDS reads of group KG go under the MFMAs of the
// group before it (the previous step's last group when KG = 0; zeros in the
// first step). issue(KGroup<KG>) issues NL direct loads of a later step,
// spread evenly over the group's MFMAs: a wave issues in order, so a burst
// of loads the address and L1 path cannot take at once would hold back the
// MFMAs behind it.
template <class C, int KG, int NL, class Issue>
__device__ __forceinline__ void kg_group(const Issue &issue, const char *sa, const char *sb, Frags<C> (&f)[2],
                                         f32x16_t (&acc)[C::TM][C::TN]) {
    constexpr int NMMA = C::TM * C::TN, NRD = C::TM + (C::B_NCONTIG ? 2 : 1) * C::TN;
    static_assert(NL <= NMMA, "at most one load per MFMA");
    constexpr int LSTEP = NL > 0 ? NMMA / NL : NMMA;
    constexpr int HALF = NMMA > 1 ? NMMA / 2 : 1;
    constexpr int RPM = (NRD + HALF - 1) / HALF;  // LDS reads per MFMA over the first half
    issue(KGroup<KG>{});
    read_frags<C>(sa, sb, KG, f[KG & 1]);
    mma_frags<C>(f[(KG + 1) & 1], acc);
#pragma unroll
    for (int i = 0; i < NMMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, KG);                           // MFMA
        if (NL > 0 && i % LSTEP == 0 && i / LSTEP < NL)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, KG);                       // direct load
        if (i < HALF) __builtin_amdgcn_sched_group_barrier(0x100, RPM, KG);           // LDS reads
    }
    __builtin_amdgcn_sched_barrier(0);
}

// The NKG k groups of a step; NLA loads per group in the first half of the
// groups, NLB in the second.
template <class C, int NLA, int NLB, class Issue, int... G>
__device__ __forceinline__ void kg_groups(const Issue &issue, const char *sa, const char *sb, Frags<C> (&f)[2],
                                          f32x16_t (&acc)[C::TM][C::TN], std::integer_sequence<int, G...>) {
    static_assert(C::NKG % 2 == 0, "k groups alternate between two fragment sets");
    (kg_group<C, G, (G < C::NKG / 2 ? NLA : NLB)>(issue, sa, sb, f, acc), ...);
}

// MFMA work of one step with the loads of later steps: the A tile's loads
// in the first half of the k groups, the B tile's in the second.
template <class C, class IssueA, class IssueB>
__device__ __forceinline__ void kg_loop(const IssueA &issue_a, const IssueB &issue_b, const char *sa, const char *sb,
                                        Frags<C> (&f)[2], f32x16_t (&acc)[C::TM][C::TN]) {
    constexpr int H = C::NKG / 2;
    static_assert(C::A_INSTR % H == 0 && C::B_INSTR % H == 0, "loads split evenly over the k groups");
    auto issue = [&](auto g) {
        constexpr int G = decltype(g)::value;
        if constexpr (G < H) issue_a(KGroup<G * C::A_INSTR / H>{}, KGroup<(G + 1) * C::A_INSTR / H>{});
        else issue_b(KGroup<(G - H) * C::B_INSTR / H>{}, KGroup<(G - H + 1) * C::B_INSTR / H>{});
    };
    kg_groups<C, C::A_INSTR / H, C::B_INSTR / H>(issue, sa, sb, f, acc, std::make_integer_sequence<int, C::NKG>{});
}

// One steady iteration of the whole-stage ring: the loads of step t_issue
// into `dst` and the MFMA work of the step in `src`. The two stages are
// distinct ring slots, which the restrict qualifiers state: the compiler
// then knows the LDS reads of `src` cannot see the direct loads into `dst`
// and inserts no vmcnt drain before them (the loop's own vmcnt waits order
// the stages).
template <class C, class Op>
__device__ __forceinline__ void ring_iter(const Op &op, int t_issue, char *__restrict__ dst,
                                          const char *__restrict__ src, int wave, Frags<C> (&f)[2],
                                          f32x16_t (&acc)[C::TM][C::TN]) {
    kg_loop<C>(
        [&](auto j0, auto j1) { op.template issue_a<decltype(j0)::value, decltype(j1)::value>(t_issue, dst, wave); },
        [&](auto j0, auto j1) {
            op.template issue_b<decltype(j0)::value, decltype(j1)::value>(t_issue, dst + C::A_BYTES, wave);
        },
        src, src + C::A_BYTES, f, acc);
}

// One steady iteration of the operand-slot ring, at step t: the A tile of
// step t + 1 into `da`, the B tile of step t + 2 into `db`, and the MFMA work
// of step t out of `sa` / `sb`. Four distinct slots (restrict, as above).
template <class C, class Op>
__device__ __forceinline__ void split_iter(const Op &op, int t, char *__restrict__ da, char *__restrict__ db,
                                           const char *__restrict__ sa, const char *__restrict__ sb, int wave,
                                           Frags<C> (&f)[2], f32x16_t (&acc)[C::TM][C::TN]) {
    kg_loop<C>([&](auto j0, auto j1) { op.template issue_a<decltype(j0)::value, decltype(j1)::value>(t + 1, da, wave); },
               [&](auto j0, auto j1) { op.template issue_b<decltype(j0)::value, decltype(j1)::value>(t + 2, db, wave); },
               sa, sb, f, acc);
}

// The rank-r LoRA tiles, staged through registers into `slot` and
// multiplied, while the ring loads the prologue issued stay in flight. The
// caller issued the first LoRA tile's global loads before the ring's: loads
// complete in order, so waiting for the LoRA data does not wait for the ring.
// `slot` is not a slot those ring loads write (restrict in the callers).
template <class C, class Lora>
__device__ __forceinline__ void lora_tiles(int nlora, const Lora &lora, typename Lora::Regs &lr, char *slot,
                                           f32x16_t (&acc)[C::TM][C::TN]) {
    for (int lt = 0; lt < nlora; ++lt) {
        if (lt > 0) lora.load(lt, lr);
        lora.store(lr, slot);
        // LDS writes done, then a bare barrier: the ring loads stay in flight
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        mma_step<typename C::LoraCfg>(slot, slot + C::LoraCfg::A_BYTES, acc);
        if (lt + 1 < nlora) {  // the slot is refilled by the next LoRA tile
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    }
}

// Whole-stage ring prologue: steps 0 .. NSTAGE-2 go to stages 1 .. NSTAGE-1
// (`rest`) while the LoRA tiles go through stage 0 (`s0`).
template <class C, class Op, class Lora>
__device__ __forceinline__ void ring_prologue(const Op &op, int nlora, const Lora &lora, char *__restrict__ s0,
                                              char *__restrict__ rest, int wave, f32x16_t (&acc)[C::TM][C::TN]) {
    typename Lora::Regs lr;
    if (nlora > 0) lora.load(0, lr);
    __builtin_amdgcn_sched_barrier(0);  // LoRA loads ahead of the ring loads
#pragma unroll
    for (int t = 0; t < C::NSTAGE - 1; ++t) op.issue(t, rest + t * C::STAGE_BYTES, wave);  // zeros past nt
    lora_tiles<C>(nlora, lora, lr, s0, acc);
}

// Operand-slot ring prologue: B of step 0, A of step 0 and B of step 1 into
// slots 0, 1, 2 while the LoRA tiles go through slot 4.
template <class C, class Op, class Lora>
__device__ __forceinline__ void split_prologue(const Op &op, int nlora, const Lora &lora, char *__restrict__ s0,
                                               char *__restrict__ s1, char *__restrict__ s2,
                                               char *__restrict__ s4, int wave, f32x16_t (&acc)[C::TM][C::TN]) {
    typename Lora::Regs lr;
    if (nlora > 0) lora.load(0, lr);
    __builtin_amdgcn_sched_barrier(0);  // LoRA loads ahead of the ring loads
    op.issue_b(0, s0, wave);
    op.issue_a(0, s1, wave);
    op.issue_b(1, s2, wave);
    lora_tiles<C>(nlora, lora, lr, s4, acc);
}

// Ring driver: the LoRA tiles first, then nt steady steps. Every iteration
// issues one step of loads (zeros past the end), so the wait count is the
// same in every iteration. After the barrier of step t the wave issues its
// loads and the LDS reads of step t's k groups, each interleaved with the
// MFMAs of the group before it (the previous step's last group first,
// already in registers), so the MFMA pipe has work while the barrier
// resolves and the reads are in flight.
//  - Whole-stage ring (32-deep steps): step t in stage (t + 1) % NSTAGE, the
//    LoRA tiles in stage 0; NSTAGE - 1 steps in flight.
//  - Operand-slot ring (64-deep steps, five slots): half-tile h in slot
//    h % 5, with h = 2 t the B tile and h = 2 t + 1 the A tile of step t; the
//    LoRA tiles in slot 4 before its first ring use. Iteration t issues
//    halves 2 t + 3 (A of t + 1) and 2 t + 4 (B of t + 2) into the slots of
//    step t - 1, so B tiles have two steps to land and A tiles one.
template <class C, class Op, class Lora>
__device__ __forceinline__ void run(const Op &op, int nlora, const Lora &lora, char *smem,
                                    f32x16_t (&acc)[C::TM][C::TN]) {
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    Frags<C> f[2];
    if constexpr (C::SPLIT) {
        auto slot = [&](int h) { return smem + (h % C::NSTAGE) * C::SLOT_BYTES; };
        split_prologue<C>(op, nlora, lora, slot(0), slot(1), slot(2), slot(4), wave, acc);
#pragma unroll
        for (int i = 0; i < C::TM; ++i) f[1].a[i] = chunk_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < C::TN; ++i) f[1].b[i] = chunk_t{0u, 0u, 0u, 0u};
        for (int t = 0; t < op.nt; ++t) {
            // halves up to 2 t + 1 have landed; half 2 t + 2 (a B tile) may be in flight
            wait_vm<C::B_INSTR>();
            // Every LDS read of step t-1 has completed (lgkmcnt) before the
            // bare barrier, so after it that step's slots can be refilled. A
            // full __syncthreads() would add a release fence, i.e. a vmcnt(0)
            // drain of the loads still in flight. The asm keeps LDS accesses
            // in place.
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            split_iter<C>(op, t, slot(2 * t + 3), slot(2 * t + 4), slot(2 * t + 1), slot(2 * t), wave, f, acc);
        }
    } else {
        auto stage_of = [&](int t) { return smem + ((t + 1) % C::NSTAGE) * C::STAGE_BYTES; };
        ring_prologue<C>(op, nlora, lora, smem, stage_of(0), wave, acc);
#pragma unroll
        for (int i = 0; i < C::TM; ++i) f[1].a[i] = chunk_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < C::TN; ++i) f[1].b[i] = chunk_t{0u, 0u, 0u, 0u};
        for (int t = 0; t < op.nt; ++t) {
            wait_vm<(C::NSTAGE - 2) * C::LOADS_PER_STEP>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // as above
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            ring_iter<C>(op, t + C::NSTAGE - 1, stage_of(t + C::NSTAGE - 1), stage_of(t), wave, f, acc);
        }
    }
    if (op.nt > 0) mma_frags<C>(f[1], acc);
    // the zero loads of the last iterations land in the ring: drain them
    // before the epilogue reuses its memory
    wait_vm<0>();
    __syncthreads();
}

// ---------------------------------------------------------------------------
// 4-bit NormalFloat (NF4) B operand, dequantised while it is staged to LDS.
// A frozen weight is stored as codes (two per byte, element 2i of a row in
// the low nibble of byte i) and one fp32 scale per 64 consecutive elements of
// a row; element = bf16(level[code] * scale), the rounding the standalone
// dequantisation kernel applies, so the GEMM reads exactly the bf16 tile the
// unfused path would have loaded.
struct Nf4Lv { float v[16]; };

// The 16 products bf16(level[j] * s) of one scale block as byte planes:
// byte i of lo[m] / hi[m] is the low / high byte of entry 4m + i.
struct Nf4Table { uint32_t lo[4], hi[4]; };

__device__ __forceinline__ Nf4Table nf4_table(float s, const Nf4Lv &lv) {
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        p[i] = f32x2_to_bf16x2(lv.v[2 * i] * s, lv.v[2 * i + 1] * s);
    Nf4Table t;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        // v_perm_b32(a, b, sel): byte i of the result is byte sel[i] of the
        // 8-byte value a:b (b = bytes 0-3, a = bytes 4-7)
        t.lo[m] = __builtin_amdgcn_perm(p[2 * m + 1], p[2 * m], 0x06040200u);
        t.hi[m] = __builtin_amdgcn_perm(p[2 * m + 1], p[2 * m], 0x07050301u);
    }
    return t;
}

// one byte plane looked up for 4 codes (one per byte of c, 0..15): entries
// 0-7 and 8-15 by the low 3 bits, then bit 3 (m = 0xff in the bytes whose
// code has it) picks between them
__device__ __forceinline__ uint32_t nf4_plane(const uint32_t (&pl)[4], uint32_t c7, uint32_t m) {
    const uint32_t a = __builtin_amdgcn_perm(pl[1], pl[0], c7);
    const uint32_t b = __builtin_amdgcn_perm(pl[3], pl[2], c7);
    return (m & b) | (~m & a);
}

// 8 codes (one dword, element i in nibble i) -> 8 bf16 in element order.
// The bit-3 masks come from v_perm's sign selectors (8, 9, 10, 11 give
// 0xff or 0x00 from bit 7 of bytes 1, 3, 5, 7 of the 8-byte source): for
// the odd elements that bit is bit 7 of each code byte already, for the even
// ones it is moved there by a 4-bit shift (a multiply by 0xff would be a
// quarter-rate instruction).
__device__ __forceinline__ chunk_t nf4_lookup8(uint32_t q, const Nf4Table &t) {
    const uint32_t ce = q & 0x07070707u, co = (q >> 4) & 0x07070707u;  // elements 0,2,4,6 / 1,3,5,7
    const uint32_t me = __builtin_amdgcn_perm(q << 4, q << 12, 0x0B090A08u);
    const uint32_t mo = __builtin_amdgcn_perm(q, q << 8, 0x0B090A08u);
    const uint32_t lo_e = nf4_plane(t.lo, ce, me), hi_e = nf4_plane(t.hi, ce, me);
    const uint32_t lo_o = nf4_plane(t.lo, co, mo), hi_o = nf4_plane(t.hi, co, mo);
    const uint32_t e02 = __builtin_amdgcn_perm(hi_e, lo_e, 0x05010400u), e46 = __builtin_amdgcn_perm(hi_e, lo_e, 0x07030602u);
    const uint32_t o13 = __builtin_amdgcn_perm(hi_o, lo_o, 0x05010400u), o57 = __builtin_amdgcn_perm(hi_o, lo_o, 0x07030602u);
    return chunk_t{__builtin_amdgcn_perm(o13, e02, 0x05040100u), __builtin_amdgcn_perm(o13, e02, 0x07060302u),
                   __builtin_amdgcn_perm(o57, e46, 0x05040100u), __builtin_amdgcn_perm(o57, e46, 0x07060302u)};
}

// The B tile of one 64-deep step from NF4 weights. Every thread owns one
// group of 32 elements that share a scale block:
//  K-contiguous B (rows of the tile = weight rows, k along the row): tile
//    row tid / 2, k half tid % 2 of the step;
//  N-contiguous B (k-rows of the tile = weight rows, n along the row): k-row
//    tid / 8, columns 32 (tid % 8) .. + 31.
// NSEG K segments (like Operands), each through one codes and one scales
// descriptor (the weight of the segment; for K-contiguous gate/up, whose tile
// interleaves gate and up rows in 32-row blocks, the weight of this wave's
// block). Few descriptors: they must stay in scalar registers.
template <class C, int NSEG = 1>
struct Q4B {
    static_assert(C::BK == 64, "one 64-element scale block per weight row and step");
    static_assert(C::BN * C::BK == 32 * C::NTHREADS, "one 32-element group per thread");
    static_assert(NSEG == 1 || NSEG == 2, "one or two K segments");
    rsrc_t rc[NSEG], rs[NSEG];
    uint32_t coff = kInvalid;   // K-contig: byte offset of the group's codes at k = 0; N-contig: column bytes
    uint32_t soff = 0;          // K-contig: byte offset of the row's scales; N-contig: column-block bytes
    uint32_t ldc[2] = {0, 0}, ldsc[2] = {0, 0};  // N-contig: code / scale bytes per weight row
    int nt0 = 0, nt = 0;
    struct Regs { chunk_t c; float s; };

    __device__ __forceinline__ int row() const { return (int)threadIdx.x >> (C::B_NCONTIG ? 3 : 1); }

    // global loads of step t's codes and scale into r (zeros past the end or
    // outside the weight)
    __device__ __forceinline__ void load(int t, Regs &r) const {
        const bool s1 = NSEG == 2 && t >= nt0, ok = t < nt && coff != kInvalid;
        const int tt = s1 ? t - nt0 : t;
        rsrc_t cd = rc[0], sd = rs[0];
        if constexpr (NSEG == 2) {
            const rsrc_t c1 = rc[1], sc1 = rs[1];
            cd = s1 ? c1 : cd;
            sd = s1 ? sc1 : sd;
        }
        uint32_t co, so;
        if constexpr (C::B_NCONTIG) {
            const uint32_t krow = (uint32_t)(tt * 64 + row());
            co = krow * (s1 ? ldc[1] : ldc[0]) + coff;
            so = krow * (s1 ? ldsc[1] : ldsc[0]) + soff;
        } else {
            co = coff + (uint32_t)tt * 32;
            so = soff + (uint32_t)tt * 4;
        }
        r.c = buf_load16(cd, ok ? co : kInvalid);
        r.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sd, ok ? so : kInvalid, 0, 0));
    }

    // elements 8i .. 8i+7 of the group (codes dword i) as bf16 into the B
    // tile at `sb`, in the layout the direct loads produce
    __device__ __forceinline__ void store8(const Regs &r, const Nf4Table &tb, int i, char *sb) const {
        const chunk_t v = nf4_lookup8(r.c[i], tb);
        if constexpr (C::B_NCONTIG) st_ncontig<C::BN>(sb, row(), ((int)threadIdx.x & 7) * 32 + i * 8, v);
        else st_kcontig<C::CPR>(sb, row(), ((int)threadIdx.x & 1) * 4 + i, v);
    }
    // the whole group
    __device__ __forceinline__ void store(const Regs &r, char *sb, const Nf4Lv &lv) const {
        const Nf4Table tb = nf4_table(r.s, lv);
#pragma unroll
        for (int i = 0; i < 4; ++i) store8(r, tb, i, sb);
    }
};

// A k group (as kg_group) whose extra work is VALU-heavy: NV vector ALU
// instructions are placed after each MFMA and the group's NW LDS writes are
// spread over its MFMAs, so the dequantisation runs under the matrix pipe
// instead of in one block before it.
template <class C, int KG, int NL, int NV, int NW, class Issue>
__device__ __forceinline__ void kg_group_v(const Issue &issue, const char *sa, const char *sb, Frags<C> (&f)[2],
                                           f32x16_t (&acc)[C::TM][C::TN]) {
    constexpr int NMMA = C::TM * C::TN, NRD = C::TM + (C::B_NCONTIG ? 2 : 1) * C::TN;
    constexpr int LSTEP = NL > 0 ? NMMA / NL : NMMA;
    constexpr int WSTEP = NW > 0 ? NMMA / NW : NMMA;
    constexpr int HALF = NMMA > 1 ? NMMA / 2 : 1;
    constexpr int RPM = (NRD + HALF - 1) / HALF;
    issue(KGroup<KG>{});
    read_frags<C>(sa, sb, KG, f[KG & 1]);
    mma_frags<C>(f[(KG + 1) & 1], acc);
#pragma unroll
    for (int i = 0; i < NMMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, KG);                           // MFMA
        if (NL > 0 && i % LSTEP == 0 && i / LSTEP < NL)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, KG);                       // direct / vector load
        if (i < HALF) __builtin_amdgcn_sched_group_barrier(0x100, RPM, KG);           // LDS reads
        if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, KG);              // VALU
        if (NW > 0 && i % WSTEP == WSTEP - 1 && i / WSTEP < NW)
            __builtin_amdgcn_sched_group_barrier(0x200, 1, KG);                       // LDS write
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One steady iteration of the operand-slot ring with an NF4 B operand, at
// step t: the A tile of step t + 1 into `da` (direct loads, as split_iter),
// the codes of step t + 2 into `fill`, and the B tile of step t + 1 from
// `use` (its codes, loaded one iteration earlier) dequantised into `db`;
// the MFMA work of step t out of `sa` / `sb`. Five distinct slots (restrict).
template <class C, class Op, class QB>
__device__ __forceinline__ void q4_iter(const Op &op, const QB &qb, const Nf4Lv &lv, int t,
                                        char *__restrict__ da, char *__restrict__ db, const char *__restrict__ sa,
                                        const char *__restrict__ sb, int wave, const typename QB::Regs &use,
                                        typename QB::Regs &fill, Frags<C> (&f)[2], f32x16_t (&acc)[C::TM][C::TN]) {
    static_assert(C::NKG == 4, "64-deep steps");
    constexpr int AH = C::A_INSTR / 2;
    constexpr int NMMA = C::TM * C::TN;
    // the codes of step t + 2 first (a whole iteration to arrive), the table
    // (~32 VALU) with the first half of A(t + 1), then one code dword (8
    // weights, ~31 VALU + one LDS write) with the rest of A(t + 1), one more,
    // and the last two
    Nf4Table tb;
    kg_group_v<C, 0, AH + 2, (32 + NMMA - 1) / NMMA, 0>(
        [&](auto) {
            qb.load(t + 2, fill);
            op.template issue_a<0, AH>(t + 1, da, wave);
            tb = nf4_table(use.s, lv);
        },
        sa, sb, f, acc);
    kg_group_v<C, 1, C::A_INSTR - AH, (32 + NMMA - 1) / NMMA, 1>(
        [&](auto) {
            op.template issue_a<AH, C::A_INSTR>(t + 1, da, wave);
            qb.store8(use, tb, 0, db);
        },
        sa, sb, f, acc);
    kg_group_v<C, 2, 0, (32 + NMMA - 1) / NMMA, 1>([&](auto) { qb.store8(use, tb, 1, db); }, sa, sb, f, acc);
    kg_group_v<C, 3, 0, (64 + NMMA - 1) / NMMA, 2>(
        [&](auto) {
            qb.store8(use, tb, 2, db);
            qb.store8(use, tb, 3, db);
        },
        sa, sb, f, acc);
}

// Ring driver for an NF4 B operand: like run() with 64-deep steps, except
// that B tiles are written by the threads (dequantised) one iteration ahead
// instead of loaded directly two ahead. Half-tile h in slot h % 5 as in run();
// iteration t writes B of step t + 1 (half 2t + 2, the slot of A(t - 2)).
template <class C, class Op, class QB, class Lora>
__device__ __forceinline__ void run_q4(const Op &op, const QB &qb, const Nf4Lv &lv, int nlora, const Lora &lora,
                                       char *smem, f32x16_t (&acc)[C::TM][C::TN]) {
    static_assert(C::SPLIT, "64-deep operand-slot ring");
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    auto slot = [&](int h) { return smem + (h % C::NSTAGE) * C::SLOT_BYTES; };
    Frags<C> f[2];
    typename QB::Regs q0, q1;
    {
        typename Lora::Regs lr;
        if (nlora > 0) lora.load(0, lr);
        __builtin_amdgcn_sched_barrier(0);
        qb.load(0, q0);
        op.issue_a(0, slot(1), wave);
        qb.load(1, q1);
        qb.store(q0, slot(0), lv);  // B of step 0
        lora_tiles<C>(nlora, lora, lr, slot(4), acc);
    }
#pragma unroll
    for (int i = 0; i < C::TM; ++i) f[1].a[i] = chunk_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < C::TN; ++i) f[1].b[i] = chunk_t{0u, 0u, 0u, 0u};
    // every load of the previous iteration (the codes of step t + 1, then A(t))
    // has landed at the top of iteration t: nothing is issued after A(t)
    for (int t = 0; t < op.nt; t += 2) {
        wait_vm<0>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        q4_iter<C>(op, qb, lv, t, slot(2 * t + 3), slot(2 * t + 2), slot(2 * t + 1), slot(2 * t), wave, q1, q0, f,
                   acc);
        if (t + 1 < op.nt) {
            wait_vm<0>();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            q4_iter<C>(op, qb, lv, t + 1, slot(2 * t + 5), slot(2 * t + 4), slot(2 * t + 3), slot(2 * t + 2), wave,
                       q0, q1, f, acc);
        }
    }
    if (op.nt > 0) mma_frags<C>(f[1], acc);
    wait_vm<0>();
    __syncthreads();
}

// ---------------------------------------------------------------------------
// LoRA tile pieces (register-staged). A side: rows p of an fp32 [S, nz]
// matrix times s, k = 32 lt + ..., into the K-contiguous A tile.
template <class C>
struct LoraA {
    static_assert(C::BK == 32, "LoRA tiles use 32-deep steps");
    static constexpr int PER = C::BM * 4 / C::NTHREADS;
    static_assert(C::BM * 4 % C::NTHREADS == 0, "whole 16-byte chunks per thread");
    const float *z;
    int nz, row0, rows;
    float s;
    struct Regs { float4 v[PER][2]; uint32_t ok; };
    // raw loads only (invalid chunks read a valid address); zeroing happens in
    // store(), so issuing these needs no wait on their data
    __device__ __forceinline__ void load(int lt, Regs &r) const {
        r.ok = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = (int)threadIdx.x + C::NTHREADS * i;
            const int row = c >> 2, k = lt * 32 + (c & 3) * 8;
            const bool ok = row < rows && k < nz;
            const float4 *src = reinterpret_cast<const float4 *>(ok ? z + (size_t)(row0 + row) * nz + k : z);
            r.v[i][0] = src[0];
            r.v[i][1] = src[1];
            r.ok |= (uint32_t)ok << i;
        }
    }
    __device__ __forceinline__ void store(const Regs &r, char *st) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = (int)threadIdx.x + C::NTHREADS * i;
            const float m = ((r.ok >> i) & 1u) ? s : 0.0f;
            const float4 a = r.v[i][0], b = r.v[i][1];
            const float v[8] = {a.x * m, a.y * m, a.z * m, a.w * m, b.x * m, b.y * m, b.z * m, b.w * m};
            st_kcontig(st, c >> 2, c & 3, Elem<bf16_t>::pack(v));
        }
    }
};

// B side, K-contiguous rows of rank r: tile row n holds row_of(n) of a [*, r]
// matrix (a or b) placed at k in [klo, klo + r) of the 32 lt + ... range.
// The row map comes from the kernel as per-chunk pointers and offsets.
template <class C>
struct LoraBK {
    static_assert(C::BK == 32, "LoRA tiles use 32-deep steps");
    static constexpr int PER = C::BN * 4 / C::NTHREADS;
    static_assert(C::BN * 4 % C::NTHREADS == 0, "whole 16-byte chunks per thread");
    const bf16_t *rowp[PER];  // row start (element k = klo), nullptr outside
    int klo[PER];
    int r;
    const bf16_t *safe;       // any readable address (loaded, then discarded, for empty chunks)
    struct Regs { chunk_t v[PER]; uint32_t ok; };
    __device__ __forceinline__ void load(int lt, Regs &rg) const {
        rg.ok = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = (int)threadIdx.x + C::NTHREADS * i;
            const int k = lt * 32 + (c & 3) * 8 - klo[i];
            const bool ok = rowp[i] && k >= 0 && k < r;
            rg.v[i] = *reinterpret_cast<const chunk_t *>(ok ? rowp[i] + k : safe);
            rg.ok |= (uint32_t)ok << i;
        }
    }
    __device__ __forceinline__ void store(const Regs &rg, char *st) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = (int)threadIdx.x + C::NTHREADS * i;
            st_kcontig(st + C::A_BYTES, c >> 2, c & 3, ((rg.ok >> i) & 1u) ? rg.v[i] : zero4());
        }
    }
};

// B side, N-contiguous: k-rows j of up to two stacked [*, ld] matrices (rows
// < split from a, the rest from b, K rows in all), tile columns [0, ncol).
template <class C>
struct LoraBN {
    static_assert(C::BK == 32, "LoRA tiles use 32-deep steps");
    static constexpr int PER = 32 * C::BN / 8 / C::NTHREADS;
    static_assert(32 * C::BN / 8 % C::NTHREADS == 0, "whole 16-byte chunks per thread");
    const bf16_t *a, *b;
    int split, K, ld, ncol;
    struct Regs { chunk_t v[PER]; uint32_t ok; };
    __device__ __forceinline__ void load(int lt, Regs &rg) const {
        rg.ok = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = (int)threadIdx.x + C::NTHREADS * i;
            const int kr = c / (C::BN / 8), n = (c % (C::BN / 8)) * 8;
            const int j = lt * 32 + kr;
            const bool ok = j < K && n + 8 <= ncol;
            const bf16_t *src = ok ? (j < split ? a + (size_t)j * ld : b + (size_t)(j - split) * ld) + n : a;
            rg.v[i] = *reinterpret_cast<const chunk_t *>(src);
            rg.ok |= (uint32_t)ok << i;
        }
    }
    __device__ __forceinline__ void store(const Regs &rg, char *st) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = (int)threadIdx.x + C::NTHREADS * i;
            st_ncontig<C::BN>(st + C::A_BYTES, c / (C::BN / 8), (c % (C::BN / 8)) * 8,
                              ((rg.ok >> i) & 1u) ? rg.v[i] : zero4());
        }
    }
};

// a LoRA tile = its A piece and its B piece
template <class PA, class PB>
struct LoraTile {
    PA pa;
    PB pb;
    struct Regs { typename PA::Regs a; typename PB::Regs b; };
    __device__ __forceinline__ void load(int lt, Regs &r) const { pa.load(lt, r.a); pb.load(lt, r.b); }
    __device__ __forceinline__ void store(const Regs &r, char *st) const { pa.store(r.a, st); pb.store(r.b, st); }
};

// No rank-r tile (plain grouped GEMMs such as the LoRA projections).
struct NoLora {
    struct Regs {};
    __device__ __forceinline__ void load(int, Regs &) const {}
    __device__ __forceinline__ void store(const Regs &, char *) const {}
};

// ---------------------------------------------------------------------------
// Epilogue through LDS: the accumulators of one wave, 32 rows at a time, are
// parked in the wave's own LDS region (32 x WTN fp32, 16 KB for WTN = 128)
// and read back row-major, so each lane holds 8 consecutive columns of one
// row and global traffic uses 16-byte accesses. fn(tile_row, tile_col, v[8])
// is called for every (row, 8-column group) of the wave's sub-tile. Call
// after the K loop on all threads (the ring is reused: one barrier first).
template <class C, class Fn>
__device__ __forceinline__ void epilogue_rows(const f32x16_t (&acc)[C::TM][C::TN], char *smem, Fn &&fn) {
    static_assert(C::WTN % 64 == 0, "8-column groups per 16 lanes");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    float *buf = reinterpret_cast<float *>(smem) + wave * 32 * C::WTN;
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi) {
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) buf[acc_row(i, lane) * C::WTN + ni * 32 + acc_col(lane)] = acc[mi][ni][i];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int LPR = C::WTN / 8;  // lanes per row
        constexpr int RPP = 64 / LPR;    // rows per pass
#pragma unroll
        for (int pass = 0; pass < 32 / RPP; ++pass) {
            const int r = pass * RPP + lane / LPR, c8 = (lane % LPR) * 8;
            const float4 a = *reinterpret_cast<const float4 *>(buf + r * C::WTN + c8);
            const float4 b = *reinterpret_cast<const float4 *>(buf + r * C::WTN + c8 + 4);
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            fn(wm * C::WTM + mi * 32 + r, wn * C::WTN + c8, v);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next slab overwrites
    }
}

}  // namespace lds

// K-contiguous tile row that load j (of instr per wave) of this lane covers
template <class C> __device__ __forceinline__ int lds_row(int wave, int lane, int j, int instr) {
    return (wave * instr + j) * C::RPI + lane / C::CPR;
}

}  // namespace moe
