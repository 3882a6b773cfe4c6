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
// One workgroup per (head, block of block_rows rows).  A row is held by D / 32
// consecutive lanes, 32 consecutive elements each (16-byte loads and code
// stores), so a wavefront holds 16 (D = 128) or 32 (D = 64) rows at a time.
//  * Transform (when signs are given): x' = H (sigma * x) with H the
//    Sylvester Hadamard matrix (entries +-1), as a fast Walsh-Hadamard
//    transform in fp64: butterflies (a, b) -> (a + b, a - b) over each bit of
//    the index, in registers for bits 0..4 and between the row's lanes (quad
//    DPP moves) for bits 5 and 6.  Every partial sum of +-x of bf16 inputs is
//    exact in fp64 when their exponents span at most 38 binades, so the
//    result, rounded once to fp32, does not depend on the order of the
//    butterflies.  The 1/sqrt(D)
//    of the orthogonal matrix is not applied: the caller divides the softmax
//    scale by D.
//  * Scale: the smallest power of two 2^k with max|x'| 2^-k <= 448 (E4M3's
//    largest finite value), found from the exponent of the block maximum;
//    the scaled values are exact and only the E4M3 rounding loses
//    information.
//  * Codes: v_cvt_pk_fp8_f32, which rounds to the nearest E4M3 value with
//    ties to even, keeps subnormals and the sign of zero (checked on gfx950).
// The block is read twice (the transform is recomputed in the second pass,
// the rows coming from cache) rather than held on chip.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

// Lane-pair exchange of a double through two quad-permute DPP moves (lanes
// xor 1 or xor 2 within each group of four).
template <int XOR>
__device__ __forceinline__ double dpp_xor(double v) {
    constexpr int ctrl = XOR == 1 ? 0xB1 : 0x4E;    // quad_perm [1,0,3,2] / [2,3,0,1]
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)b, ctrl, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), ctrl, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned)lo);
}

// A row of D elements is held by LPR = D / 32 consecutive lanes, element
// i = 32 q + e in lane quarter q = lane % LPR, register e; a wavefront holds
// 64 / LPR rows at once.
template <int D>
struct RowSlice {
    static constexpr int LPR = D / 32;
    double x[32];

    // Row `r` of the block (zeros past `rows`), transformed if signs are given.
    __device__ __forceinline__ void load(const QuantParams& p, size_t base, int r, int rows, int q,
                                         const float (&sg)[32]) {
        const bool ok = r < rows;
        const bf16x8* src = reinterpret_cast<const bf16x8*>(p.x + base + (size_t)(ok ? r : 0) * D + 32 * q);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8 v = src[c];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * c + e] = ok ? (double)(float)v[e] : 0.0;
        }
        if (!p.signs) return;
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] *= (double)sg[e];
        // Index bits 0..4: butterflies inside the lane.
#pragma unroll
        for (int h = 1; h < 32; h <<= 1)
#pragma unroll
            for (int e = 0; e < 32; ++e)
                if ((e & h) == 0) {
                    const double a = x[e], b = x[e + h];
                    x[e] = a + b;
                    x[e + h] = a - b;
                }
        // Index bits 5 (and 6): between the lanes of the row.
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const double o = dpp_xor<1>(x[e]);
            x[e] = (q & 1) ? o - x[e] : x[e] + o;
        }
        if (LPR == 4) {
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const double o = dpp_xor<2>(x[e]);
                x[e] = (q & 2) ? o - x[e] : x[e] + o;
            }
        }
    }
};

template <int D>
__global__ void __launch_bounds__(256) quantize_fp8_kernel(QuantParams p) {
    constexpr int LPR = RowSlice<D>::LPR;
    constexpr int RPW = 64 / LPR;           // rows per wavefront at a time
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int q = l % LPR;
    const int head = blockIdx.x / p.nblk;
    const int blk = blockIdx.x - head * p.nblk;
    const int row0 = blk * p.block_rows;
    const int rows = min(p.block_rows, p.L - row0);
    const size_t base = ((size_t)head * p.L + row0) * D;
    float sg[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) sg[e] = p.signs ? p.signs[32 * q + e] : 1.0f;

    // Pass 1: the block maximum of |x'| (rounded to fp32).
    float amax = 0.0f;
    for (int r0 = w * RPW; r0 < rows; r0 += 4 * RPW) {
        RowSlice<D> rs;
        rs.load(p, base, r0 + l / LPR, rows, q, sg);
#pragma unroll
        for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf((float)rs.x[e]));
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

    // Pass 2: codes of x' 2^-k (exact scaling, E4M3 rounding), 32 bytes per lane.
    for (int r0 = w * RPW; r0 < rows; r0 += 4 * RPW) {
        const int r = r0 + l / LPR;
        RowSlice<D> rs;
        rs.load(p, base, r, rows, q, sg);
        if (r < rows) {
            int packed[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf((float)rs.x[4 * c], -k),
                                                               ldexpf((float)rs.x[4 * c + 1], -k), 0, false);
                packed[c] = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf((float)rs.x[4 * c + 2], -k),
                                                            ldexpf((float)rs.x[4 * c + 3], -k), lo, true);
            }
            i32x4* dst = reinterpret_cast<i32x4*>(p.x8 + base + (size_t)r * D + 32 * q);
            dst[0] = i32x4{packed[0], packed[1], packed[2], packed[3]};
            dst[1] = i32x4{packed[4], packed[5], packed[6], packed[7]};
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
