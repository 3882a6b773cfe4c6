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
// One workgroup per (head, block of block_rows rows).  A row is held by
// D / 32 consecutive lanes, 32 consecutive elements each (16-byte loads and
// code stores), so a wavefront covers a slice of 16 (D = 128) or 32 (D = 64)
// rows at a time.  The workgroup has one wavefront per slice for up to eight
// slices, else eight wavefronts taking every eighth slice.
//  * Transform (when signs are given): x' = H (sigma * x) with H the
//    Sylvester Hadamard matrix (entries +-1), as a fast Walsh-Hadamard
//    transform in fp64: butterflies (a, b) -> (a + b, a - b) over each bit of
//    the index, in registers for bits 0..4 and between the row's lanes (quad
//    DPP moves) for bits 5 and 6.  Every partial sum of +-x of bf16 inputs is
//    exact in fp64 when their exponents span at most 38 binades, so the
//    result, rounded once to fp32, does not depend on the order of the
//    butterflies.  The sign flips act on the bf16 sign bits.  The 1/sqrt(D)
//    of the orthogonal matrix is not applied: the caller divides the softmax
//    scale by D.
//  * Scale: the smallest power of two 2^k with max|x'| 2^-k <= 448 (E4M3's
//    largest finite value), found from the exponent of the block maximum;
//    the scaled values are exact and only the E4M3 rounding loses
//    information.
//  * Codes: v_cvt_pk_fp8_f32, which rounds to the nearest E4M3 value with
//    ties to even, keeps subnormals and the sign of zero (checked on gfx950).
// Each wavefront keeps the fp32 x' of its first one or two slices in
// registers between the maximum and the codes; only a block of more than 16
// slices transforms its further slices twice (their rows come from cache the
// second time).
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

constexpr int kQuantMaxWaves = 8;

// x' (rounded to fp32) of the lane's 32 elements i = 32 q + e (e = 0..31).
// The lane's 32 bf16 inputs of row r of the block (zeros past `rows`), with
// the sign bits in `flip` (bit 15 and bit 31 of each pair) flipped.
template <int D>
__device__ __forceinline__ void load_slice(const QuantParams& p, size_t base, int r, int rows, int q,
                                           const i32x4 (&flip)[4], i32x4 (&raw)[4]) {
    const bool ok = r < rows;
    const i32x4* src = reinterpret_cast<const i32x4*>(p.x + base + (size_t)(ok ? r : 0) * D + 32 * q);
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = ok ? (src[c] ^ flip[c]) : i32x4{0, 0, 0, 0};
}

template <int D>
__device__ __forceinline__ void transform_slice(const QuantParams& p, int q, const i32x4 (&raw)[4],
                                                float (&out)[32]) {
    constexpr int LPR = D / 32;
    double x[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned w = (unsigned)raw[c][e];
            x[8 * c + 2 * e] = (double)__builtin_bit_cast(float, w << 16);
            x[8 * c + 2 * e + 1] = (double)__builtin_bit_cast(float, w & 0xFFFF0000u);
        }
    }
    if (p.signs) {
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
        // Index bits 5 (and 6): between the lanes of the row; the lane with
        // the bit set keeps partner - own.
        const double s1 = (q & 1) ? -1.0 : 1.0;
#pragma unroll
        for (int e = 0; e < 32; ++e) x[e] = __builtin_fma(x[e], s1, dpp_xor<1>(x[e]));
        if (LPR == 4) {
            const double s2 = (q & 2) ? -1.0 : 1.0;
#pragma unroll
            for (int e = 0; e < 32; ++e) x[e] = __builtin_fma(x[e], s2, dpp_xor<2>(x[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) out[e] = (float)x[e];
}

template <int D>
__device__ __forceinline__ void store_codes(const QuantParams& p, size_t base, int r, int q, int k,
                                            const float (&v)[32]) {
    int packed[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * c], -k), ldexpf(v[4 * c + 1], -k), 0, false);
        packed[c] = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * c + 2], -k), ldexpf(v[4 * c + 3], -k), lo, true);
    }
    i32x4* dst = reinterpret_cast<i32x4*>(p.x8 + base + (size_t)r * D + 32 * q);
    dst[0] = i32x4{packed[0], packed[1], packed[2], packed[3]};
    dst[1] = i32x4{packed[4], packed[5], packed[6], packed[7]};
}

template <int D, int KEEP>
__global__ void __launch_bounds__(64 * kQuantMaxWaves) quantize_fp8_kernel(QuantParams p) {
    constexpr int LPR = D / 32;
    constexpr int RPW = 64 / LPR;           // rows per wavefront at a time
    const int nw = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int q = l % LPR;
    const int head = blockIdx.x / p.nblk;
    const int blk = blockIdx.x - head * p.nblk;
    const int row0 = blk * p.block_rows;
    const int rows = min(p.block_rows, p.L - row0);
    const size_t base = ((size_t)head * p.L + row0) * D;
    i32x4 flip[4] = {};                     // sign bits of sigma for this lane's elements
    if (p.signs) {
        const f32x4* sg = reinterpret_cast<const f32x4*>(p.signs + 32 * q);
        f32x4 sv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] = sg[i];          // all eight loads in flight at once
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float s0 = sv[2 * c + e / 2][2 * (e % 2)], s1 = sv[2 * c + e / 2][2 * (e % 2) + 1];
                flip[c][e] = (int)((s0 < 0.0f ? 0x8000u : 0u) | (s1 < 0.0f ? 0x80000000u : 0u));
            }
    }

    // Pass 1: the block maximum of |x'|, keeping the first KEEP slices (their
    // loads all issued first).
    float keep[KEEP][32];
    float amax = 0.0f;
    const int stride = nw * RPW;
    {
        i32x4 raw[KEEP][4];
#pragma unroll
        for (int j = 0; j < KEEP; ++j) load_slice<D>(p, base, w * RPW + j * stride + l / LPR, rows, q, flip, raw[j]);
#pragma unroll
        for (int j = 0; j < KEEP; ++j) {
            transform_slice<D>(p, q, raw[j], keep[j]);
#pragma unroll
            for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(keep[j][e]));
        }
    }
    for (int r0 = w * RPW + KEEP * stride; r0 < rows; r0 += stride) {
        i32x4 raw[4];
        float v[32];
        load_slice<D>(p, base, r0 + l / LPR, rows, q, flip, raw);
        transform_slice<D>(p, q, raw, v);
#pragma unroll
        for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) amax = fmaxf(amax, __shfl_xor(amax, h, 64));
    __shared__ float wmax[kQuantMaxWaves];
    if (l == 0) wmax[w] = amax;
    __syncthreads();
    amax = 0.0f;
    for (int i = 0; i < nw; ++i) amax = fmaxf(amax, wmax[i]);

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
#pragma unroll
    for (int j = 0; j < KEEP; ++j) {
        const int r = w * RPW + j * stride + l / LPR;
        if (r < rows) store_codes<D>(p, base, r, q, k, keep[j]);
    }
    for (int r0 = w * RPW + KEEP * stride; r0 < rows; r0 += stride) {
        i32x4 raw[4];
        float v[32];
        load_slice<D>(p, base, r0 + l / LPR, rows, q, flip, raw);
        transform_slice<D>(p, q, raw, v);
        if (r0 + l / LPR < rows) store_codes<D>(p, base, r0 + l / LPR, q, k, v);
    }
}

}  // namespace

hipError_t launch_quantize_fp8(int D, const QuantParams& p, hipStream_t stream) {
    // Slices of 64 / (D / 32) rows: one per wavefront for up to
    // kQuantMaxWaves of them, else two per wavefront (held in registers) on
    // kQuantMaxWaves wavefronts.
    const int rpw = 64 / (D / 32);
    const int slices = (p.block_rows + rpw - 1) / rpw;
    const bool two = slices > kQuantMaxWaves;
    const int waves = two ? kQuantMaxWaves : slices;
    const dim3 grid((unsigned)((long long)p.heads * p.nblk)), block(64 * waves);
    if (D == 64) {
        if (two) hipLaunchKernelGGL((quantize_fp8_kernel<64, 2>), grid, block, 0, stream, p);
        else     hipLaunchKernelGGL((quantize_fp8_kernel<64, 1>), grid, block, 0, stream, p);
    } else {
        if (two) hipLaunchKernelGGL((quantize_fp8_kernel<128, 2>), grid, block, 0, stream, p);
        else     hipLaunchKernelGGL((quantize_fp8_kernel<128, 1>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
