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
// Rows are held by D / 64 lanes, 64 elements each (at D = 128 the two lanes
// split each 32-element run into halves; 16-byte loads and code stores), so a
// wavefront covers a slice of 32 (D = 128) or 64 (D = 64) rows at a time.  A workgroup has one wavefront per slice of a
// block, up to eight (beyond that, eight wavefronts take every eighth slice),
// and works through blocks of the tensor in turn, the loads of its next
// block in flight while it transforms and stores the current one.
//  * Transform (when signs are given): x' = H (sigma * x) with H the
//    Sylvester Hadamard matrix (entries +-1), as a fast Walsh-Hadamard
//    transform in fp64: butterflies (a, b) -> (a + b, a - b) over each bit of
//    the index, in registers for all bits but one and, at D = 128, between
//    the two lanes of the row (a quad DPP move) for bit 4.  Every partial sum of +-x
//    of bf16 inputs is exact in fp64 when their exponents span at most 38
//    binades, so the result, rounded once to fp32, does not depend on the
//    order of the butterflies.  The sign flips act on the bf16 sign bits.
//    The 1/sqrt(D) of the orthogonal matrix is not applied: the caller
//    divides the softmax scale by D.
//  * Scale: the smallest power of two 2^k with max|x'| 2^-k <= 448 (E4M3's
//    largest finite value), found from the exponent of the block maximum;
//    the scaled values are exact and only the E4M3 rounding loses
//    information.
//  * Codes: v_cvt_pk_fp8_f32, which rounds to the nearest E4M3 value with
//    ties to even, keeps subnormals and the sign of zero (checked on gfx950).
// Each wavefront keeps the fp32 x' of its first slice of a block in
// registers between the maximum and the codes; only a block of more than
// eight slices transforms its further slices twice (their rows come from
// cache the second time).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

// The double held by lane l ^ 1, through two quad-permute DPP moves.
__device__ __forceinline__ double lane_pair_swap(double v) {
    constexpr int ctrl = 0xB1;              // quad_perm [1,0,3,2]
    // Every lane reads a valid partner, so no lane keeps an old value: a plain
    // DPP move (no initialisation of the destination).
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)b, ctrl, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), ctrl, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned)lo);
}

constexpr int kQuantMaxWaves = 8;

// Element of the row held at position e (0..63) of lane half h.  At D = 128
// the two lanes of a row split it by index bit 4 (16-element halves of each
// 32), so each lane's code stores and pairs of input words are contiguous
// and the two lanes' are adjacent; position bits 0-3 and 4-5 are index bits
// 0-3 and 5-6.
template <int D>
__device__ __forceinline__ int elem_index(int e, int h) {
    return D == 128 ? (e & 15) | (h << 4) | ((e >> 4) << 5) : e;
}

// The lane's 64 bf16 inputs of row r of a block, as eight 16-byte words,
// through a buffer descriptor over the block's valid rows (rows past them
// read as zeros).
template <int D>
__device__ __forceinline__ void load_row(rsrc_t blk, int r, int h, i32x4 (&raw)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t at = (uint32_t)(r * D + elem_index<D>(8 * c, h)) * 2;
        raw[c] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(blk, at, 0, 0));
    }
}

// x' (rounded to fp32) of the lane's 64 elements, i = elem_index(e, h).
// Bit e of `sgn` is the sign of sigma for element e (flipped on the bf16
// sign bit).
template <int D>
__device__ __forceinline__ void transform_row(const QuantParams& p, int h, const i32x4 (&raw)[8],
                                              uint64_t sgn, float (&out)[64]) {
    if (!p.signs) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned w = (unsigned)raw[c][e];
                out[8 * c + 2 * e] = __builtin_bit_cast(float, w << 16);
                out[8 * c + 2 * e + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
            }
        return;
    }
    double x[64];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 8 * c + 2 * e;
            const unsigned bits = (unsigned)(sgn >> i);
            const unsigned w = (unsigned)raw[c][e] ^ (((bits & 1u) << 15) | ((bits & 2u) << 30));
            x[i] = (double)__builtin_bit_cast(float, w << 16);
            x[i + 1] = (double)__builtin_bit_cast(float, w & 0xFFFF0000u);
        }
    // Position bits 0..5: butterflies inside the lane.
#pragma unroll
    for (int b = 1; b < 64; b <<= 1)
#pragma unroll
        for (int e = 0; e < 64; ++e)
            if ((e & b) == 0) {
                const double a = x[e], c = x[e + b];
                x[e] = a + c;
                x[e + b] = a - c;
            }
    if (D == 128) {
        // Index bit 4: between the two lanes of the row; the lane with the
        // bit set keeps partner - own.
        const double s1 = h ? -1.0 : 1.0;
#pragma unroll
        for (int e = 0; e < 64; ++e) x[e] = __builtin_fma(x[e], s1, lane_pair_swap(x[e]));
    }
#pragma unroll
    for (int e = 0; e < 64; ++e) out[e] = (float)x[e];
}

// E4M3 codes of v 2^-k, four per 32-bit word.
__device__ __forceinline__ void encode_row(int k, const float (&v)[64], int (&packed)[16]) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * c], -k), ldexpf(v[4 * c + 1], -k), 0, false);
        packed[c] = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * c + 2], -k), ldexpf(v[4 * c + 3], -k), lo, true);
    }
}

// The codes of row r through a descriptor over the block's valid rows
// (stores past them are dropped): always four store instructions.
template <int D>
__device__ __forceinline__ void store_codes(rsrc_t out, int r, int h, const int (&packed)[16]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned,
                               i32x4{packed[4 * c], packed[4 * c + 1], packed[4 * c + 2], packed[4 * c + 3]}),
            out, (uint32_t)(r * D + elem_index<D>(16 * c, h)), 0, 0);
}

template <int D>
__global__ void __launch_bounds__(64 * kQuantMaxWaves) quantize_fp8_kernel(QuantParams p) {
    constexpr int LPR = D / 64;             // lanes per row
    constexpr int RPW = 64 / LPR;           // rows per wavefront at a time
    const int nw = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int h = l % LPR;                  // which 64 elements of the row
    const int lr = l / LPR;                 // row within the slice
    const int total = p.heads * p.nblk;
    const int stride = nw * RPW;
    uint64_t sgn = 0;                       // bit e: sigma of this lane's element e is -1
    if (p.signs) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(p.signs + elem_index<D>(4 * c, h));
#pragma unroll
            for (int e = 0; e < 4; ++e) sgn |= (uint64_t)(a[e] < 0.0f) << (4 * c + e);
        }
    }
    __shared__ float wmax[2][kQuantMaxWaves];
    auto block_base = [&](int id, int& rows) -> size_t {
        const int head = id / p.nblk;
        const int blk = id - head * p.nblk;
        const int row0 = blk * p.block_rows;
        rows = min(p.block_rows, p.L - row0);
        return ((size_t)head * p.L + row0) * D;
    };

    // Smallest k with amax 2^-k <= 448: amax in [2^(e-1), 2^e) and
    // 448 2^(e-9) = 0.875 2^e, while 448 2^(e-10) < 2^(e-1).
    auto scale_exponent = [](float amax) {
        int k = 0;
        if (amax > 0.0f) {
            int e;
            (void)frexpf(amax, &e);
            k = (amax <= ldexpf(0.875f, e)) ? e - 9 : e - 8;
        }
        return k;
    };
    // The block maximum over the workgroup (wmax buffer `buf`).
    auto block_max = [&](float amax, int buf) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        if (l == 0) wmax[buf][w] = amax;
        __syncthreads();                    // also: every wavefront has read wmax[buf ^ 1]
        amax = 0.0f;
        for (int i = 0; i < nw; ++i) amax = fmaxf(amax, wmax[buf][i]);
        return amax;
    };

    if (p.block_rows <= stride) {
        // One slice per wavefront and block, software-pipelined over the
        // workgroup's blocks: the wavefront's slice of the next block is
        // copied straight into its LDS stage (no registers) while the current
        // one is transformed, and the codes of a block are stored during the
        // next block's transform.
        extern __shared__ __attribute__((aligned(16))) i32x4 stage[];   // [wave][512] 16-byte words
        const uint32_t lds_stage = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) i32x4*)stage) +
                                   (uint32_t)w * 8 * 64 * 16;
        // The stage holds the wavefront's slice (RPW rows of CPR 16-byte words)
        // with word q of row j at position CPR j + (q ^ swz(j)): copy i of
        // a lane fills position 64 i + lane, so each copy instruction reads 1 KB
        // of consecutive rows, and the lanes of a row-word read land on
        // distinct bank groups.
        constexpr int CPR = D / 8;
        auto swz = [](int j) { return D == 128 ? (j & 15) : ((j >> 1) & 7); };
        uint32_t at[8];                     // byte offsets of the lane's copies in a block
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int P = 64 * c + l;
            const int j = P / CPR;
            at[c] = (uint32_t)((w * RPW + j) * D + 8 * ((P % CPR) ^ swz(j))) * 2;
        }
        int rd[8];                          // stage positions of the lane's words
#pragma unroll
        for (int c = 0; c < 8; ++c) rd[c] = w * 8 * 64 + CPR * lr + ((elem_index<D>(8 * c, h) / 8) ^ swz(lr));
        auto copy_slice = [&](int id) {
            int rows;
            const size_t base = block_base(min(id, total - 1), rows);
            const i32x4 d = make_desc(p.x + base, id < total ? (uint32_t)rows * D * 2 : 0u);
#pragma unroll
            for (int c = 0; c < 8; ++c) copy16_to_lds_async(d, at[c], lds_stage + (uint32_t)c * 64 * 16);
        };
        const int r = w * RPW + lr;
        int codes[16];                      // the previous block's codes of row r
        rsrc_t prev_out = make_rsrc(p.x8, 0u);
        int id = blockIdx.x;
        copy_slice(id);
        for (int it = 0; id < total; id += gridDim.x, ++it) {
            int rows;
            const size_t base = block_base(id, rows);
            // This block's copy has landed.  Vector memory operations complete
            // in issue order, and only the previous block's four code stores
            // were issued after it (from the second block on).
            if (it >= 2) wait_vector_loads_until<4>();
            else         wait_vector_loads_until<0>();
            i32x4 raw[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) raw[c] = stage[rd[c]];
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the stage is read before it is refilled
            copy_slice(id + gridDim.x);
            if (it >= 1) store_codes<D>(prev_out, r, h, codes);
            float keep[64];
            transform_row<D>(p, h, raw, sgn, keep);
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 64; ++e) amax = fmaxf(amax, fabsf(keep[e]));
            const int k = scale_exponent(block_max(amax, it & 1));
            if (threadIdx.x == 0) p.scales[id] = ldexpf(1.0f, k);
            encode_row(k, keep, codes);
            prev_out = make_rsrc(p.x8 + base, (uint32_t)rows * D);   // rows past the block's are dropped
        }
        if (id != (int)blockIdx.x) store_codes<D>(prev_out, r, h, codes);
        wait_vector_loads_until<0>();       // the copy past the last block (zero range) drained
    } else {
        // Blocks of more than one slice per wavefront: the maximum over every
        // slice, then the codes, each slice transformed in both passes.
        for (int id = blockIdx.x, it = 0; id < total; id += gridDim.x, ++it) {
            int rows;
            const size_t base = block_base(id, rows);
            const rsrc_t blk = make_rsrc(p.x + base, (uint32_t)rows * D * 2);
            float amax = 0.0f;
            for (int r0 = w * RPW; r0 < rows; r0 += stride) {
                i32x4 raw[8];
                float v[64];
                load_row<D>(blk, r0 + lr, h, raw);
                transform_row<D>(p, h, raw, sgn, v);
#pragma unroll
                for (int e = 0; e < 64; ++e) amax = fmaxf(amax, fabsf(v[e]));
            }
            const int k = scale_exponent(block_max(amax, it & 1));
            if (threadIdx.x == 0) p.scales[id] = ldexpf(1.0f, k);
            for (int r0 = w * RPW; r0 < rows; r0 += stride) {
                i32x4 raw[8];
                float v[64];
                load_row<D>(blk, r0 + lr, h, raw);
                transform_row<D>(p, h, raw, sgn, v);
                int codes[16];
                encode_row(k, v, codes);
                store_codes<D>(make_rsrc(p.x8 + base, (uint32_t)rows * D), r0 + lr, h, codes);
            }
        }
    }
}

}  // namespace

hipError_t launch_quantize_fp8(int D, const QuantParams& p, int cus, hipStream_t stream) {
    // Slices of 64 / (D / 64) rows: one wavefront per slice of a block, up to
    // kQuantMaxWaves.  Two wavefronts per SIMD fit, so a CU holds
    // 8 / waves workgroups; the grid fills every CU once with them and each
    // workgroup takes every grid-th block.
    const int rpw = 64 / (D / 64);
    const int slices = (p.block_rows + rpw - 1) / rpw;
    const int waves = slices < kQuantMaxWaves ? slices : kQuantMaxWaves;
    const long long total = (long long)p.heads * p.nblk;
    const long long fill = (long long)cus * (8 / waves);
    const dim3 grid((unsigned)(total < fill ? total : fill)), block(64 * waves);
    const size_t lds = slices <= kQuantMaxWaves ? (size_t)waves * 8 * 64 * 16 : 0;   // the LDS stages
    if (D == 64) hipLaunchKernelGGL((quantize_fp8_kernel<64>), grid, block, lds, stream, p);
    else         hipLaunchKernelGGL((quantize_fp8_kernel<128>), grid, block, lds, stream, p);
    return hipGetLastError();
}

}  // namespace fa
