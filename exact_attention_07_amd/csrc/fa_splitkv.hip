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
// this KV head; they are contiguous in Q, O and LSE memory.  The kernel is
// bound by HBM bandwidth, so it keeps many bytes in flight with few
// instructions: per 32-key tile each lane issues 16-byte range-checked,
// non-temporal loads of K and V straight into registers (fully coalesced: one
// instruction reads 1 KB of consecutive rows; keys past the partition read as
// zero), and the loads of tile t + 1 are issued as soon as the registers of
// tile t are consumed, so they are in flight during all of tile t's work.
// Both tiles then go to wavefront-private LDS tiles (16-byte writes,
// XOR-swizzled) from which K is read in the MFMA A-operand layout (rows
// through the bit-2/3 swap) and V through the transposing read.  Register use
// is capped at 256 so that two wavefronts share each SIMD.  Per tile,
// S^T = K Q^T and O^T += V^T P^T run on the matrix cores as in the prefill
// kernel, with the same online-softmax update.
// Partials are kept in base-2 units: part_lse = m*c + log2 l; a partition that
// starts past the sequence's valid length writes part_lse = -inf and nothing
// else, so the combine needs no lengths.
//
// Causal window (section 12, width w: key j is allowed for the query at
// position i when 0 <= i - j < w): partitions start at the 32-key tile that
// holds the lowest key any packed row can see, n - Lq - w + 1, so the
// partition plan covers only the window's span; keys before a row's own
// window are masked in the tiles that cross it.
//
// Paged cache (section 9.3, "Paging changes where keys live"): logical token
// t of sequence b lives in physical page table[b][t / P], row t % P, of a
// cache laid out [num_pages, Hkv, P, D].  With P a multiple of 16 and tiles
// starting at multiples of 32, each 16-key half of a tile lies in one page:
// the loader looks up that page (a wave-uniform scalar load) and reads the
// half through its own range-checked descriptor, so the loads stay 16-byte
// and coalesced and everything after the loader is the contiguous kernel.
// A table entry outside [0, num_pages) is never dereferenced: its keys are
// read as zeros and masked.
//
// combine kernel: one wavefront per output row.  Lanes load the partition
// log-sum-exps together, reduce their max and the weight sum across the
// wavefront, then every lane accumulates its columns over all partitions with
// independent loads (a partition of weight 0 is selected away, so the stale
// data of an empty partition is never used).  A row with no valid key gets
// O = 0, LSE = -inf.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <int D, bool PAGED>
__global__ void __launch_bounds__(64, 2) splitkv_kernel(SplitParams p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int CH = D / 8;               // 16-byte chunks per row
    constexpr int BN = 32;                  // keys per tile
    constexpr int NV = BN * CH / 64;        // 16-byte V loads per lane and tile

    __shared__ __attribute__((aligned(16))) bf16 kt[BN * D];   // K tile, row-major, swizzled
    __shared__ __attribute__((aligned(16))) bf16 vt[BN * D];   // V tile, row-major, swizzled

    const int l = threadIdx.x;
    const int hi = l >> 5;
    // Partition-major order: consecutive workgroups (dealt round-robin to the
    // eight XCDs) take the same partition of different (batch, KV head, row
    // group) units, so every XCD gets a like mix of long and short sequences.
    const int units = p.B * p.Hkv * p.n_groups;
    const int s = blockIdx.x / units;
    int L = blockIdx.x - s * units;
    const int g = L % p.Hkv;
    L /= p.Hkv;
    const int rg = L % p.n_groups;
    const int b = L / p.n_groups;

    int n = p.Lk;
    if (p.kv_lens) {
        n = p.kv_lens[b];
        n = n < 0 ? 0 : (n > p.Lk ? p.Lk : n);
    }
    const int rho = rg * 32 + (l & 31);     // packed row of this lane's column
    const bool row_ok = rho < p.rows;
    const size_t grow = (size_t)(b * p.Hq + g * p.r) * p.Lq + rho;  // row in [B*Hq*Lq]
    int lo = 0;                             // first key of partition 0
    if (p.window > 0) lo = max(n - p.Lq - p.window + 1, 0) & ~(BN - 1);
    const int kbeg = lo + s * p.chunk;
    if (kbeg >= n) {                        // an empty partition: weight 0 in the combine
        if (row_ok && hi == 0) p.part_lse[grow * p.num_splits + s] = kNegInf;
        return;
    }
    const int kend = min(n, kbeg + p.chunk);
    const int ntiles = (kend - kbeg + BN - 1) / BN;

    const int qi = row_ok ? rho % p.Lq : 0;
    const size_t kvoff = (size_t)(b * p.Hkv + g) * p.Lk * D;
    const int qpos = n - p.Lq + qi;         // bottom-right causal position
    const size_t qbase = (size_t)(b * p.Hq + g * p.r) * p.Lq;      // first packed row of this KV head
    const rsrc_t qbuf = make_rsrc(p.q + qbase * D, (uint32_t)p.rows * D * 2);

    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = load16(qbuf, (uint32_t)(rho * D + ks * 16 + hi * 8) * 2);

    // Tile t as 16-byte chunks: chunk i * 64 + lane of the row-major K and V
    // tiles; past kend the range is 0.
    bf16x8 kr[NV], vr[NV];
    int pv_next = 3;                        // paged: bit h = half h of the loaded tile is usable
    auto load_tile = [&](int t) __attribute__((always_inline)) {
        const int k0 = kbeg + t * BN;
        if constexpr (!PAGED) {
            const int rows = kend - k0;
            const uint32_t bytes = (uint32_t)(rows > 0 ? rows : 0) * D * 2;
            const size_t src = kvoff + (size_t)(rows > 0 ? k0 : 0) * D;
            const rsrc_t kb = make_rsrc(p.k + src, bytes);
            const rsrc_t vb = make_rsrc(p.v + src, bytes);
#pragma unroll
            for (int i = 0; i < NV; ++i) kr[i] = load16_stream(kb, (uint32_t)(i * 64 + l) * 16);
#pragma unroll
            for (int i = 0; i < NV; ++i) vr[i] = load16_stream(vb, (uint32_t)(i * 64 + l) * 16);
        } else {
            // Load i covers tile rows 64 i / CH ..: the first NV / 2 loads
            // read rows 0-15, the rest rows 16-31.
            constexpr int NH = NV / 2;
            rsrc_t kb[2], vb[2];
            int pv = 0;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int r0 = k0 + 16 * hf;
                // Wave-uniform by construction; readfirstlane keeps the
                // descriptor in scalar registers (a clamp folded into a
                // vector op would otherwise force a per-lane loop).
                int rows = __builtin_amdgcn_readfirstlane(min(kend - r0, 16));
                int page = 0;
                if (rows > 0)
                    page = __builtin_amdgcn_readfirstlane(p.page_table[(size_t)b * p.max_pages + r0 / p.page_size]);
                const bool ok = (page >= 0) & (page < p.num_pages);
                if (ok || rows <= 0) pv |= 1 << hf;
                if (!ok) { page = 0; rows = 0; }
                const size_t src = ((size_t)page * p.Hkv + g) * p.page_size * D +
                                   (size_t)(r0 % p.page_size) * D;
                const uint32_t bytes = (uint32_t)(rows > 0 ? rows : 0) * D * 2;
                kb[hf] = make_rsrc(p.k + src, bytes);
                vb[hf] = make_rsrc(p.v + src, bytes);
            }
            pv_next = pv;
#pragma unroll
            for (int i = 0; i < NV; ++i) kr[i] = load16_stream(kb[i / NH], (uint32_t)((i % NH) * 64 + l) * 16);
#pragma unroll
            for (int i = 0; i < NV; ++i) vr[i] = load16_stream(vb[i / NH], (uint32_t)((i % NH) * 64 + l) * 16);
        }
    };
    // Chunk i * 64 + lane of either tile goes to row P / CH, chunk P % CH xor the swizzle.
    auto store_tile = [&](bf16* tile, const bf16x8 (&r)[NV], auto swz) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int P = i * 64 + l;
            const int row = P / CH;
            *reinterpret_cast<bf16x8*>(tile + row * D + (((P % CH) ^ swz(row)) * 8)) = r[i];
        }
    };

    const int krow = swap_bits_2_3(l & 31);
    const int kxor = k_swizzle<D>(krow);
    const int vrow = 8 * hi + ((l & 15) >> 2);
    const int vxor = v_swizzle<D>(vrow);
    const int vcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

    const float c = p.c;
    float m = kNegInf, ell = 0.0f;
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();

    load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = kbeg + t * BN;
        const int pv = pv_next;
        // K(t) and V(t) into the LDS tiles (the previous tile's reads are
        // ordered before these writes: one wavefront's LDS operations execute
        // in order), then the registers take tile t + 1.
        store_tile(kt, kr, [](int row) { return k_swizzle<D>(row); });
        store_tile(vt, vr, [](int row) { return v_swizzle<D>(row); });
        load_tile(t + 1);                   // zeros and no traffic past the last tile

        f32x16 sacc = zero_f32x16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + krow * D + (((2 * ks + hi) ^ kxor) * 8));
            sacc = mfma_32x32x16(a, qf[ks], sacc);
        }

        const bool need_mask = (k0 + BN > kend) || (p.causal && k0 + BN - 1 > n - p.Lq) ||
                               (p.window > 0 && n - 1 - k0 >= p.window) || (PAGED && pv != 3);
        if (need_mask) {
            // Branch-free per element (bitwise &, then a select): every
            // element's test is a straight-line select.
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = k0 + 16 * (v >> 3) + 8 * hi + (v & 7);
                const bool ok = (key < kend) & (!p.causal | (key <= qpos)) &
                                ((p.window == 0) | (qpos - key < p.window)) & (((pv >> (v >> 3)) & 1) != 0);
                sacc[v] = ok ? sacc[v] : kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
        mx = max_with_partner(mx);
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
                const int col = db * 32 + vcol;
                const bf16* base = vt + (half * 16 + vrow) * D + (((col >> 3) ^ vxor) * 8) + (col & 7);
                const bf16x4 lo = lds_read_transposed(base);
                const bf16x4 up = lds_read_transposed(base + 4 * D);
                bf16x8 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) { a[e] = lo[e]; a[4 + e] = up[e]; }
                acc[db] = mfma_32x32x16(a, pb[half], acc[db]);
            }
    }

    const float ell_t = sum_with_partner(ell);
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D>
__global__ void __launch_bounds__(256) combine_kernel(CombineParams p) {
    constexpr int PER_LANE = D / 64;
    const int w = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const long long rows = (long long)p.B * p.Hq * p.Lq;
    const long long row = (long long)blockIdx.x * 4 + w;
    if (row >= rows) return;
    const int S = p.num_splits;
    const float* ls = p.part_lse + row * S;
    const float* po = p.part_o + row * S * D + l * PER_LANE;

    float M = kNegInf;
    for (int s0 = 0; s0 < S; s0 += 64)
        if (s0 + l < S) M = fmaxf(M, ls[s0 + l]);
    M = wave_max(M);

    float out[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) out[j] = 0.0f;
    float lse = kNegInf;
    if (M != kNegInf) {
        float W = 0.0f;
        for (int s0 = 0; s0 < S; s0 += 64) {
            // Lane i holds the weight of partition s0 + i (0 for an empty one).
            const float wl = (s0 + l < S) ? exp2_fast(ls[s0 + l] - M) : 0.0f;
            W += wl;
            const int cnt = S - s0 < 64 ? S - s0 : 64;
            for (int i0 = 0; i0 < cnt; i0 += 4) {
                // Four partitions per pass with independent loads; indices past
                // cnt are clamped to a valid partition and weighted 0.
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = i0 + u < cnt ? i0 + u : cnt - 1;
                    const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i));
                    const float wgt = i0 + u < cnt ? wi : 0.0f;
#pragma unroll
                    for (int j = 0; j < PER_LANE; ++j) {
                        const float x = po[(size_t)(s0 + i) * D + j];
                        out[j] += wgt != 0.0f ? wgt * x : 0.0f;
                    }
                }
            }
        }
        W = wave_sum(W);
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

hipError_t launch_splitkv(int D, bool paged, const SplitParams& p, hipStream_t stream) {
    const long long total = (long long)p.B * p.Hkv * p.n_groups * p.num_splits;
    const dim3 grid((unsigned)total), block(64);
    if (D == 64) {
        if (paged) hipLaunchKernelGGL((splitkv_kernel<64, true>), grid, block, 0, stream, p);
        else       hipLaunchKernelGGL((splitkv_kernel<64, false>), grid, block, 0, stream, p);
    } else {
        if (paged) hipLaunchKernelGGL((splitkv_kernel<128, true>), grid, block, 0, stream, p);
        else       hipLaunchKernelGGL((splitkv_kernel<128, false>), grid, block, 0, stream, p);
    }
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
