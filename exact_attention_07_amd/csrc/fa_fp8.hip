// Block quantization of bf16 rows to FP8 (E4M3), with optional incoherent
// processing.
//
// FlashAttention from Scratch, section 10.3 "Treat FP8 as a second lesson",
// and FlashAttention 1-4, FlashAttention-3 point 3: one FP8 scale per tile
// instead of one per tensor, and Q and K multiplied by the same random
// orthogonal matrix -- a Hadamard transform with random sign flips -- before
// quantizing, which leaves QK^T unchanged and spreads an outlier coordinate
// over all of them.
//
// One workgroup per (head, block of block_rows rows); each wavefront takes
// whole rows, with element i of a row in lane i % 64 (slot i / 64).
//  * Transform (when signs are given): x' = H (sigma * x) with H the
//    Sylvester Hadamard matrix (entries +-1), as a fast Walsh-Hadamard
//    transform in fp64: butterflies (a, b) -> (a + b, a - b) over each bit of
//    the index, across lanes by xor-shuffles and, for bit 6 (D = 128), within
//    a lane.  Every partial sum of +-x of bf16 inputs is exact in fp64 when
//    their exponents span at most 38 binades, so the result, rounded once to
//    fp32, does not depend on the order of the butterflies.  The 1/sqrt(D)
//    of the orthogonal matrix is not applied: the caller divides the softmax
//    scale by D.
//  * Scale: the smallest power of two 2^k with max|x'| 2^-k <= 448 (E4M3's
//    largest finite value), found from the exponent of the block maximum;
//    the scaled values are exact and only the E4M3 rounding loses
//    information.
//  * Codes: v_cvt_pk_fp8_f32, which rounds to the nearest E4M3 value with
//    ties to even, keeps subnormals and the sign of zero (checked on gfx950).
// The block is read twice (the transform is recomputed in the second pass)
// rather than held in LDS: a quantization pass reads 4 and writes 1 byte per
// element and is bound by HBM either way.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

template <int D>
struct RowXf {
    static constexpr int E = D / 64;        // elements per lane
    float y[E];

    // Row `row` of head `head`, transformed (if signs) and rounded to fp32.
    __device__ __forceinline__ void load(const QuantParams& p, size_t row_base, int l) {
        double x[E];
#pragma unroll
        for (int s = 0; s < E; ++s) x[s] = (double)(float)p.x[row_base + l + 64 * s];
        if (p.signs) {
#pragma unroll
            for (int s = 0; s < E; ++s) x[s] *= (double)p.signs[l + 64 * s];
#pragma unroll
            for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
                for (int s = 0; s < E; ++s) {
                    const double o = __shfl_xor(x[s], h, 64);
                    x[s] = (l & h) ? o - x[s] : x[s] + o;
                }
            }
            if (E == 2) {
                const double a = x[0], b = x[E - 1];
                x[0] = a + b;
                x[E - 1] = a - b;
            }
        }
#pragma unroll
        for (int s = 0; s < E; ++s) y[s] = (float)x[s];
    }
};

template <int D>
__global__ void __launch_bounds__(256) quantize_fp8_kernel(QuantParams p) {
    constexpr int E = D / 64;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int head = blockIdx.x / p.nblk;
    const int blk = blockIdx.x - head * p.nblk;
    const int row0 = blk * p.block_rows;
    const int rows = min(p.block_rows, p.L - row0);
    const size_t base = ((size_t)head * p.L + row0) * D;

    // Pass 1: the block maximum of |x'|.
    float amax = 0.0f;
    for (int r = w; r < rows; r += 4) {
        RowXf<D> xf;
        xf.load(p, base + (size_t)r * D, l);
#pragma unroll
        for (int s = 0; s < E; ++s) amax = fmaxf(amax, fabsf(xf.y[s]));
    }
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) amax = fmaxf(amax, __shfl_xor(amax, h, 64));
    __shared__ float wmax[4];
    if (l == 0) wmax[w] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

    // Smallest k with amax 2^-k <= 448: amax in [2^(e-1), 2^e) and
    // 448 2^(e-9) = 0.875 2^e, while 448 2^(e-10) < 2^(e-1).
    int k = 0;
    if (amax > 0.0f) {
        int e;
        (void)frexpf(amax, &e);
        k = (amax <= ldexpf(0.875f, e)) ? e - 9 : e - 8;
    }
    if (threadIdx.x == 0) p.scales[(size_t)head * p.nblk + blk] = ldexpf(1.0f, k);

    // Pass 2: codes of x' 2^-k (exact scaling, E4M3 rounding).
    for (int r = w; r < rows; r += 4) {
        RowXf<D> xf;
        xf.load(p, base + (size_t)r * D, l);
#pragma unroll
        for (int s = 0; s < E; ++s) {
            const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(xf.y[s], -k), 0.0f, 0, false);
            p.x8[base + (size_t)r * D + l + 64 * s] = (uint8_t)(packed & 0xFF);
        }
    }
}

}  // namespace

hipError_t launch_quantize_fp8(int D, const QuantParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)((long long)p.heads * p.nblk)), block(256);
    if (D == 64) hipLaunchKernelGGL(quantize_fp8_kernel<64>, grid, block, 0, stream, p);
    else         hipLaunchKernelGGL(quantize_fp8_kernel<128>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
