// Split-KV forward (Flash-Decoding) and the log-sum-exp combine.
//
// FlashAttention from Scratch, section 9.1 "Split the long dimension that
// remains": with one query per head there is no query-tile parallelism, so
// the valid keys of every sequence are cut into partitions; each partition
// computes a normalised partial output O_s and its log-sum-exp L_s, and a
// reduction merges them by section 4.3's rule, L = log sum_s e^{L_s},
// O = sum_s e^{L_s - L} O_s.  Section 9.2: the r query heads that share a KV
// head are packed into one matrix-core tile so each K/V byte is read once for
// all of them.
//
// split kernel: one wavefront per (batch, KV head, 32-row group, partition).
// Packed row rho = head_in_group * Lq + query enumerates the rows that read
// this KV head; they are contiguous in Q, O and LSE memory.  Per 32-key tile:
//   K rows go straight from global memory into MFMA A-operand registers (one
//   16-byte load per lane per k-step, rows in the bit-2/3 swapped order);
//   V rows are loaded with coalesced 16-byte loads and written transposed into
//   a wave-private LDS tile, then read back as the A operand of O^T += V^T P^T;
//   the next tile's loads are issued before the current tile's arithmetic.
// The online-softmax update is the same as the prefill kernel's.
// Partials are kept in base-2 units: part_lse = m*c + log2 l.
//
// combine kernel: one wavefront per output row merges the active partitions
// (partitions that start before the sequence's valid length) and writes bf16 O
// and the natural-log LSE; a row with no valid key gets O = 0, LSE = -inf.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <int D>
__global__ void __launch_bounds__(64) splitkv_kernel(SplitParams p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int DG = D / 8;               // 16-byte groups per row
    constexpr int VBLK = D / 64;            // (4 keys x 8 columns) blocks per lane
    constexpr int VST = 32 + 8;             // LDS row stride of V^T in bf16

    __shared__ __attribute__((aligned(16))) bf16 vt[D * VST];

    const int l = threadIdx.x;
    const int hi = l >> 5;
    int L = blockIdx.x;
    const int s = L % p.num_splits;
    L /= p.num_splits;
    const int rg = L % p.n_groups;
    L /= p.n_groups;
    const int g = L % p.Hkv;
    const int b = L / p.Hkv;

    int n = p.Lk;
    if (p.kv_lens) {
        n = p.kv_lens[b];
        n = n < 0 ? 0 : (n > p.Lk ? p.Lk : n);
    }
    const int kbeg = s * p.chunk;
    if (kbeg >= n) return;                  // an empty partition: the combine skips it
    const int kend = min(n, kbeg + p.chunk);
    const int ntiles = (kend - kbeg + 31) / 32;

    const int rho = rg * 32 + (l & 31);     // packed row of this lane's column
    const bool row_ok = rho < p.rows;
    const int qi = row_ok ? rho % p.Lq : 0;
    const size_t grow = (size_t)(b * p.Hq + g * p.r) * p.Lq + rho;  // row in [B*Hq*Lq]
    const size_t kvoff = (size_t)(b * p.Hkv + g) * p.Lk * D;
    const int qpos = n - p.Lq + qi;         // bottom-right causal position
    // Range-checked buffers: keys >= kend (past this partition) read as zero.
    const rsrc_t kbuf = make_rsrc(p.k + kvoff, (uint32_t)kend * D * 2);
    const rsrc_t vbuf = make_rsrc(p.v + kvoff, (uint32_t)kend * D * 2);
    const size_t qbase = (size_t)(b * p.Hq + g * p.r) * p.Lq;      // first packed row of this KV head
    const rsrc_t qbuf = make_rsrc(p.q + qbase * D, (uint32_t)p.rows * D * 2);

    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = load16(qbuf, (uint32_t)(rho * D + ks * 16 + hi * 8) * 2);

    const int krow = swap_bits_2_3(l & 31);
    bf16x8 kreg[KS];
    bf16x8 vreg[VBLK][4];
    auto load_tile = [&](int t) {
        const int k0 = kbeg + t * 32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kreg[ks] = load16(kbuf, (uint32_t)((k0 + krow) * D + ks * 16 + hi * 8) * 2);
#pragma unroll
        for (int i = 0; i < VBLK; ++i) {
            const int blk = l + 64 * i;
            const int dg = blk % DG, kg = blk / DG;
#pragma unroll
            for (int j = 0; j < 4; ++j)   // rows past the partition read as zero
                vreg[i][j] = load16(vbuf, (uint32_t)((k0 + kg * 4 + j) * D + dg * 8) * 2);
        }
    };

    const float c = p.c;
    float m = kNegInf, ell = 0.0f;
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();

    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = kbeg + t * 32;
        // Stage V^T of this tile in LDS (after every lane finished reading the previous one).
        __syncthreads();
#pragma unroll
        for (int i = 0; i < VBLK; ++i) {
            const int blk = l + 64 * i;
            const int dg = blk % DG, kg = blk / DG;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 col;
#pragma unroll
                for (int j = 0; j < 4; ++j) col[j] = vreg[i][j][e];
                *reinterpret_cast<bf16x4*>(vt + (dg * 8 + e) * VST + kg * 4) = col;
            }
        }
        __syncthreads();
        bf16x8 kcur[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kcur[ks] = kreg[ks];
        if (t + 1 < ntiles) load_tile(t + 1);

        f32x16 sacc = zero_f32x16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = mfma_32x32x16(kcur[ks], qf[ks], sacc);

        const bool need_mask = (k0 + 32 > kend) || p.causal;
        if (need_mask) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = k0 + 16 * (v >> 3) + 8 * hi + (v & 7);
                const bool ok = key < kend && (!p.causal || key <= qpos);
                if (!ok) sacc[v] = kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
        mx = fmaxf(mx, lane_xor32(mx));
        const float m_new = fmaxf(m, mx);
        const float mc = (m_new == kNegInf) ? 0.0f : m_new * c;
        const float alpha = exp2_fast(m * c - mc);
        float psum = 0.0f;
        bf16x8 pb[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                e[j] = exp2_fast(__builtin_fmaf(sacc[8 * half + j], c, -mc));
                psum += e[j];
            }
            pb[half] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        }
        ell = alpha * ell + psum;
        m = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    vt + (db * 32 + (l & 31)) * VST + half * 16 + hi * 8);
                acc[db] = mfma_32x32x16(a, pb[half], acc[db]);
            }
    }

    const float ell_t = ell + lane_xor32(ell);
    const float inv = ell_t > 0.0f ? 1.0f / ell_t : 0.0f;
    if (row_ok) {
        float* Op = p.part_o + (grow * p.num_splits + s) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                f32x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = acc[db][4 * grp + j] * inv;
                *reinterpret_cast<f32x4*>(Op + db * 32 + 8 * grp + 4 * hi) = ov;
            }
        if (hi == 0)
            p.part_lse[grow * p.num_splits + s] = ell_t > 0.0f ? m * c + log2_fast(ell_t) : kNegInf;
    }
}

template <int D>
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p) {
    constexpr int PER_LANE = D / 64;
    const int w = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const long long rows = (long long)p.B * p.Hq * p.Lq;
    const long long row = (long long)blockIdx.x * 4 + w;
    if (row >= rows) return;
    const int b = (int)(row / ((long long)p.Hq * p.Lq));
    int n = p.Lk;
    if (p.kv_lens) {
        n = p.kv_lens[b];
        n = n < 0 ? 0 : (n > p.Lk ? p.Lk : n);
    }
    int active = (n + p.chunk - 1) / p.chunk;
    active = active < p.num_splits ? active : p.num_splits;
    const float* ls = p.part_lse + row * p.num_splits;
    float M = kNegInf;
    for (int s = 0; s < active; ++s) M = fmaxf(M, ls[s]);
    float out[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) out[j] = 0.0f;
    float lse = kNegInf;
    if (M != kNegInf) {
        float W = 0.0f;
        const float* po = p.part_o + row * p.num_splits * D;
        for (int s = 0; s < active; ++s) {
            const float wgt = exp2_fast(ls[s] - M);  // an empty partition (-inf) weighs 0
            W += wgt;
#pragma unroll
            for (int j = 0; j < PER_LANE; ++j) out[j] += wgt * po[(size_t)s * D + l * PER_LANE + j];
        }
        const float inv = 1.0f / W;
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j) out[j] *= inv;
        lse = (M + log2_fast(W)) * kLn2;
    }
    bf16* Op = p.o + row * D + l * PER_LANE;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) Op[j] = (bf16)out[j];
    if (p.lse && l == 0) p.lse[row] = lse;
}

hipError_t launch_splitkv(int D, const SplitParams& p, hipStream_t stream) {
    const long long total = (long long)p.B * p.Hkv * p.n_groups * p.num_splits;
    const dim3 grid((unsigned)total), block(64);
    if (D == 64) hipLaunchKernelGGL((splitkv_kernel<64>), grid, block, 0, stream, p);
    else         hipLaunchKernelGGL((splitkv_kernel<128>), grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_combine(int D, const CombineParams& p, hipStream_t stream) {
    const long long rows = (long long)p.B * p.Hq * p.Lq;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (D == 64) hipLaunchKernelGGL((combine_kernel<64>), grid, block, 0, stream, p);
    else         hipLaunchKernelGGL((combine_kernel<128>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
