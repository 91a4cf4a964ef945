// nf4.hip - 4-bit NormalFloat frozen base weights: dequantisation to bf16.
//
// The pages name 4-bit QLoRA as the frozen-base variant of MoE fine-tuning
// (Unsloth 2026 wiki chapter, model-support table) and QLoRA's NF4 code
// (GPU MODE lecture 32 notes, closing open questions) without giving the
// format. The code is the NormalFloat one of the QLoRA paper (section 3,
// values listed in its appendix): 16 levels that are quantiles of N(0, 1),
// asymmetric so that zero is exact, scaled into [-1, 1]:
//   q = 0 .. 6  : -Q(0.5 + j/7 (p - 0.5)) / Q(p), j = 7 .. 1
//   q = 7       : 0
//   q = 8 .. 15 : +Q(0.5 + j/8 (p - 0.5)) / Q(p), j = 1 .. 8
// with Q the standard normal quantile and p = 0.9677083, the top probability
// for which this construction gives the paper's published levels (to float32
// rounding). A weight is level[code] * scale, one fp32 scale per 64
// consecutive weights of a row.
// Codes are packed two per byte, element 2i in the low nibble of byte i.
//
// The kernel is a stream: 4 code bytes in, 16 bytes of bf16 out per thread
// (HBM-bound: 0.5 + 2 bytes per weight plus a scale per 64).
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

struct Nf4Levels {
    float v[16];
};

// standard normal quantile by Newton's method on the complementary error
// function (p in (0, 1), here at most 0.9677083)
double normal_quantile(double p) {
    double x = 0.0;
    for (int it = 0; it < 60; ++it) {
        const double f = 0.5 * std::erfc(-x / std::sqrt(2.0)) - p;
        const double d = std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
        const double step = f / d;
        x -= step;
        if (std::fabs(step) < 1e-15) break;
    }
    return x;
}

Nf4Levels nf4_levels() {
    static const Nf4Levels lv = [] {
        Nf4Levels l{};
        const double p = 0.9677083, qmax = normal_quantile(p);
        for (int j = 7; j >= 1; --j) l.v[7 - j] = (float)(-normal_quantile(0.5 + j / 7.0 * (p - 0.5)) / qmax);
        l.v[7] = 0.0f;
        for (int j = 1; j <= 8; ++j) l.v[7 + j] = (float)(normal_quantile(0.5 + j / 8.0 * (p - 0.5)) / qmax);
        return l;
    }();
    return lv;
}

// out[row][c] = level[code(row, c)] * scale[row][c / 64], 8 elements per
// thread, so the 4-byte code loads and 16-byte stores of a wave are
// contiguous (32 elements per thread with four strided stores measured 40%
// slower)
__global__ __launch_bounds__(256) void k_nf4_dequant(const uint8_t *__restrict__ codes,
                                                     const float *__restrict__ scales, int64_t rows, int cols,
                                                     Nf4Levels lv, bf16_t *__restrict__ out) {
    __shared__ float lvl[16];
    if (threadIdx.x < 16) lvl[threadIdx.x] = lv.v[threadIdx.x];
    __syncthreads();
    const int per_row = cols / 8;
    const int64_t n8 = rows * per_row;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / per_row;
        const int c8 = (int)(i - row * per_row) * 8;
        const uint32_t q = *reinterpret_cast<const uint32_t *>(codes + row * (cols / 2) + c8 / 2);
        const float s = scales[row * (cols / 64) + c8 / 64];
        float v[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) v[h] = lvl[(q >> (4 * h)) & 15u] * s;
        st_stream(out + row * cols + c8, Elem<bf16_t>::pack(v));  // written once, read by a later pass
    }
}

}  // namespace

void nf4_level_values(float out[16]) {
    const Nf4Levels lv = nf4_levels();
    for (int i = 0; i < 16; ++i) out[i] = lv.v[i];
}

hipError_t run_nf4_dequant(const uint8_t *codes, const float *scales, int64_t rows, int cols, bf16_t *out,
                           hipStream_t st) {
    const int64_t n8 = rows * (cols / 8);
    if (n8 == 0) return hipSuccess;
    const int64_t want = (n8 + 255) / 256;
    const int grid = (int)(want < 8192 ? want : 8192);
    k_nf4_dequant<<<grid, 256, 0, st>>>(codes, scales, rows, cols, nf4_levels(), out);
    return hipGetLastError();
}

}  // namespace moe
