// Backward of the attention forward by recomputation.
//
// FlashAttention from Scratch, section 8 "Backward: spend arithmetic to save
// memory" (no dropout, fixed mask): with G = dL/dO, the probabilities of every
// allowed pair are rebuilt from the forward's saved row normaliser,
// P_ij = exp(c s_ij - LSE_i); then dV = P^T G, dP = G V^T,
// delta_i = G_i . O_i, dS = P (dP - delta), dQ = c dS K and dK = c dS^T Q --
// five matrix products per tile (S, dP, dV, dQ, dK).  The section leaves the
// ownership open: a query-owned block finishes dQ, a KV-owned block finishes
// dK and dV.  Here each gets its own kernel, so neither needs atomics and the
// result is deterministic:
//
// dq kernel: one wavefront per (batch, query head, 32 queries).  Q and G of
// the wavefront's queries stay in registers as B operands; K and V tiles of 32
// keys go through wavefront-private LDS.  Per tile, on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation: S^T = K Q^T and dP^T = V G^T (K and V rows fed
// through the bit-2/3 swap, as in the forward, so that key 16*(v/8) + 8*hi +
// (v%8) sits in accumulator entry v), P^T and dS^T elementwise with one query
// per lane (its LSE and delta in registers), then dQ^T += K^T dS^T with K^T
// from the transposing LDS read and dS^T rounded to bf16 as the B operand.
// The wavefront also forms delta_i = G_i . O_i for its queries (one dot
// product per lane pair) and stores it for the second kernel.
//
// dk/dv kernel: one wavefront per (batch, KV head, 32 keys).  K and V of the
// wavefront's keys stay in registers as B operands; it visits every query
// tile of every query head that reads this KV head (section 9.2's grouping,
// so the GQA sum happens in registers) and skips tiles no query of which can
// see the block (causal, window).  Per 32-query tile, through wavefront-private
// LDS: S = Q K^T and dP = G V^T with the query rows fed through the bit-2/3
// swap, which makes the P and dS accumulators, rounded to bf16, exactly the A
// operands of dV += P^T G and dK += dS^T Q; G and Q enter those as B operands
// through the transposing LDS read.  Keys past a sequence's valid length get
// zero gradient.
//
// Exponentials are base 2 with the scale folded in: p = 2^(s c2 - L2) with
// c2 = c log2(e) and L2 = LSE log2(e); a row with LSE = -inf (no allowed key)
// has every pair masked and gets p = 0.  Masks are the forward's: valid
// length, bottom-right causal, causal window; they are branch-free selects.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// A 32-row tile of a [rows, D] bf16 tensor into wavefront-private LDS,
// row-major with the K swizzle: every lane loads D/16 16-byte chunks
// (coalesced, range-checked: rows past `valid` read as zero) and stores them.
template <int D>
__device__ __forceinline__ void stage_tile(bf16* tile, const bf16* src, int valid, int l) {
    constexpr int CH = D / 8;
    constexpr int NV = 32 * CH / 64;
    const rsrc_t rs = make_rsrc(src, (uint32_t)(valid > 0 ? valid : 0) * D * 2);
    bf16x8 r[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) r[i] = load16(rs, (uint32_t)(i * 64 + l) * 16);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int P = i * 64 + l;
        const int row = P / CH;
        *reinterpret_cast<bf16x8*>(tile + row * D + (((P % CH) ^ k_swizzle<D>(row)) * 8)) = r[i];
    }
}

// A-operand fragment: row `row` of a K-swizzled tile, 16-byte chunk `chunk`.
template <int D>
__device__ __forceinline__ bf16x8 read_row_chunk(const bf16* tile, int row, int chunk) {
    return *reinterpret_cast<const bf16x8*>(tile + row * D + ((chunk ^ k_swizzle<D>(row)) * 8));
}

// Transposed fragment of a K-swizzled tile: lane l receives column
// col0 + (l % 32) of rows row0 + 8*(l/32) + e, e = 0..7 (the operand layout of
// an MFMA whose k index runs down the tile's rows).  Each lane's two 8-byte
// reads are addressed through the swizzle of their own rows.
template <int D>
__device__ __forceinline__ bf16x8 read_transposed(const bf16* tile, int row0, int col0, int l) {
    const int hi = l >> 5;
    const int r = row0 + 8 * hi + ((l & 15) >> 2);
    const int col = col0 + 16 * ((l >> 4) & 1) + 4 * (l & 3);
    const bf16* a = tile + r * D + (((col >> 3) ^ k_swizzle<D>(r)) * 8) + (col & 7);
    const bf16* b = tile + (r + 4) * D + (((col >> 3) ^ k_swizzle<D>(r + 4)) * 8) + (col & 7);
    const bf16x4 lo = lds_read_transposed(a);
    const bf16x4 up = lds_read_transposed(b);
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[e] = lo[e]; f[4 + e] = up[e]; }
    return f;
}

__device__ __forceinline__ int clamp_len(const int* kv_lens, int b, int Lk) {
    if (!kv_lens) return Lk;
    const int n = kv_lens[b];
    return n < 0 ? 0 : (n > Lk ? Lk : n);
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(64) bwd_dq_kernel(BwdParams p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    __shared__ __attribute__((aligned(16))) bf16 kt[32 * D];
    __shared__ __attribute__((aligned(16))) bf16 vt[32 * D];

    const int l = threadIdx.x;
    const int hi = l >> 5;
    const int nqb = (p.Lq + 31) / 32;
    const int qb = blockIdx.x % nqb;
    const int bh = blockIdx.x / nqb;           // b * Hq + h
    const int h = bh % p.Hq;
    const int b = bh / p.Hq;
    const int g = h / p.r;
    const int n = clamp_len(p.kv_lens, b, p.Lk);
    const int off = n - p.Lq;                   // query i sits at key position i + off
    const int q0 = qb * 32;
    const int qrow = q0 + (l & 31);
    const bool row_ok = qrow < p.Lq;
    const int qpos = qrow + off;

    const size_t qoff = (size_t)bh * p.Lq * D;
    const size_t kvoff = (size_t)(b * p.Hkv + g) * p.Lk * D;
    const rsrc_t qbuf = make_rsrc(p.q + qoff, (uint32_t)p.Lq * D * 2);
    const rsrc_t obuf = make_rsrc(p.o + qoff, (uint32_t)p.Lq * D * 2);
    const rsrc_t gbuf = make_rsrc(p.dout + qoff, (uint32_t)p.Lq * D * 2);

    // Q and G of this lane's query as B operands; delta = G . O.
    bf16x8 qf[KS], gf[KS];
    float dpart = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint32_t at = (uint32_t)(qrow * D + ks * 16 + hi * 8) * 2;
        qf[ks] = load16(qbuf, at);
        gf[ks] = load16(gbuf, at);
        const bf16x8 of = load16(obuf, at);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart += (float)gf[ks][e] * (float)of[e];
    }
    const float delta = sum_with_partner(dpart);
    float lse2 = 0.0f;
    if (row_ok) {
        const float L = p.lse[(size_t)bh * p.Lq + qrow];
        lse2 = L == kNegInf ? 0.0f : L * kLog2e;      // an empty row has every pair masked
        if (hi == 0) p.delta[(size_t)bh * p.Lq + qrow] = delta;
    }

    // Keys this block can see: [k_lo, k_hi).
    int k_hi = n, k_lo = 0;
    if (p.causal) k_hi = min(n, max(min(q0 + 32, p.Lq) + off, 0));
    if (p.window > 0) k_lo = max(q0 + off - p.window + 1, 0);
    const int t_lo = k_lo / 32;
    const int t_hi = (k_hi + 31) / 32;

    const int krow = swap_bits_2_3(l & 31);
    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero_f32x16();
    const float c2 = p.c;

    for (int t = t_lo; t < t_hi; ++t) {
        const int k0 = t * 32;
        // One wavefront's LDS operations run in order: the reads of the
        // previous tile are done before these writes land.
        stage_tile<D>(kt, p.k + kvoff + (size_t)k0 * D, n - k0, l);
        stage_tile<D>(vt, p.v + kvoff + (size_t)k0 * D, n - k0, l);

        f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s = mfma_32x32x16(read_row_chunk<D>(kt, krow, 2 * ks + hi), qf[ks], s);
            dp = mfma_32x32x16(read_row_chunk<D>(vt, krow, 2 * ks + hi), gf[ks], dp);
        }
        float ds[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = k0 + 16 * (v >> 3) + 8 * hi + (v & 7);
            const bool ok = row_ok & (key < n) & (!p.causal | (key <= qpos)) &
                            ((p.window == 0) | (qpos - key < p.window));
            const float pr = ok ? exp2_fast(__builtin_fmaf(s[v], c2, -lse2)) : 0.0f;
            ds[v] = pr * (dp[v] - delta);
        }
        const bf16x8 dsb0 = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
        const bf16x8 dsb1 = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            dq[db] = mfma_32x32x16(read_transposed<D>(kt, 0, db * 32, l), dsb0, dq[db]);
            dq[db] = mfma_32x32x16(read_transposed<D>(kt, 16, db * 32, l), dsb1, dq[db]);
        }
    }

    if (row_ok) {
        bf16* out = p.dq + qoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                bf16x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = (bf16)(dq[db][4 * gq + j] * p.scale);
                *reinterpret_cast<bf16x4*>(out + db * 32 + 8 * gq + 4 * hi) = ov;
            }
    }
}

template <int D>
__global__ void __launch_bounds__(64) bwd_dkdv_kernel(BwdParams p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    __shared__ __attribute__((aligned(16))) bf16 qt[32 * D];
    __shared__ __attribute__((aligned(16))) bf16 gt[32 * D];
    __shared__ __attribute__((aligned(16))) float stat[64];   // L2 and delta of the tile's 32 queries

    const int l = threadIdx.x;
    const int hi = l >> 5;
    const int nkb = (p.Lk + 31) / 32;
    const int kb = blockIdx.x % nkb;
    const int bg = blockIdx.x / nkb;           // b * Hkv + g
    const int g = bg % p.Hkv;
    const int b = bg / p.Hkv;
    const int n = clamp_len(p.kv_lens, b, p.Lk);
    const int off = n - p.Lq;
    const int k0 = kb * 32;
    const int key = k0 + (l & 31);              // this lane's key (accumulator column of S, dP)

    const size_t kvoff = (size_t)bg * p.Lk * D;
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dk[db] = zero_f32x16(); dv[db] = zero_f32x16(); }

    if (k0 < n) {
        // K and V of this lane's key as B operands (rows past n read as zero).
        const rsrc_t kbuf = make_rsrc(p.k + kvoff, (uint32_t)n * D * 2);
        const rsrc_t vbuf = make_rsrc(p.v + kvoff, (uint32_t)n * D * 2);
        bf16x8 kf[KS], vf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint32_t at = (uint32_t)(key * D + ks * 16 + hi * 8) * 2;
            kf[ks] = load16(kbuf, at);
            vf[ks] = load16(vbuf, at);
        }
        // Queries that can see some key of [k0, k0 + 32): position >= k0
        // (causal) and position < k0 + 31 + window (window).
        int i_lo = 0, i_hi = p.Lq;
        if (p.causal) i_lo = max(k0 - off, 0);
        if (p.window > 0) i_hi = min(p.Lq, max(k0 + 31 + p.window - off, 0));
        const int qrow = swap_bits_2_3(l & 31);   // A-operand row of this lane
        const float c2 = p.c;

        for (int hh = 0; hh < p.r; ++hh) {
            const int h = g * p.r + hh;
            const size_t bh = (size_t)b * p.Hq + h;
            const size_t qoff = bh * p.Lq * D;
            for (int q0 = (i_lo / 32) * 32; q0 < i_hi; q0 += 32) {
                stage_tile<D>(qt, p.q + qoff + (size_t)q0 * D, p.Lq - q0, l);
                stage_tile<D>(gt, p.dout + qoff + (size_t)q0 * D, p.Lq - q0, l);
                if (l < 32) {
                    const int i = q0 + l;
                    float L2 = 0.0f, dl = 0.0f;
                    if (i < p.Lq) {
                        const float L = p.lse[bh * p.Lq + i];
                        L2 = L == kNegInf ? 0.0f : L * kLog2e;
                        dl = p.delta[bh * p.Lq + i];
                    }
                    stat[l] = L2;
                    stat[32 + l] = dl;
                }

                f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s = mfma_32x32x16(read_row_chunk<D>(qt, qrow, 2 * ks + hi), kf[ks], s);
                    dp = mfma_32x32x16(read_row_chunk<D>(gt, qrow, 2 * ks + hi), vf[ks], dp);
                }
                // Entry v of this lane holds query q0 + 16*(v/8) + 8*hi + (v%8).
                float pr[16], ds[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int qi = 16 * (v >> 3) + 8 * hi + (v & 7);
                    const int i = q0 + qi;
                    const int qpos = i + off;
                    const bool ok = (i < p.Lq) & (key < n) & (!p.causal | (key <= qpos)) &
                                    ((p.window == 0) | (qpos - key < p.window));
                    pr[v] = ok ? exp2_fast(__builtin_fmaf(s[v], c2, -stat[qi])) : 0.0f;
                    ds[v] = pr[v] * (dp[v] - stat[32 + qi]);
                }
                const bf16x8 pb0 = to_bf16x8(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
                const bf16x8 pb1 = to_bf16x8(pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]);
                const bf16x8 db0 = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
                const bf16x8 db1 = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dv[db] = mfma_32x32x16(pb0, read_transposed<D>(gt, 0, db * 32, l), dv[db]);
                    dv[db] = mfma_32x32x16(pb1, read_transposed<D>(gt, 16, db * 32, l), dv[db]);
                    dk[db] = mfma_32x32x16(db0, read_transposed<D>(qt, 0, db * 32, l), dk[db]);
                    dk[db] = mfma_32x32x16(db1, read_transposed<D>(qt, 16, db * 32, l), dk[db]);
                }
            }
        }
    }

    // Accumulator entry v of lane l: key k0 + 8*(v/4) + 4*hi + (v%4), column
    // 32*db + (l % 32).  Keys past n hold zeros.
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int kr = k0 + 8 * (v >> 2) + 4 * hi + (v & 3);
        if (kr < p.Lk) {
            bf16* dkp = p.dk + kvoff + (size_t)kr * D + (l & 31);
            bf16* dvp = p.dv + kvoff + (size_t)kr * D + (l & 31);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dkp[db * 32] = (bf16)(dk[db][v] * p.scale);
                dvp[db * 32] = (bf16)dv[db][v];
            }
        }
    }
}

hipError_t launch_backward(int D, const BwdParams& p, hipStream_t stream) {
    const long long nq = (long long)p.B * p.Hq * ((p.Lq + 31) / 32);
    const long long nk = (long long)p.B * p.Hkv * ((p.Lk + 31) / 32);
    if (D == 64) {
        hipLaunchKernelGGL((bwd_dq_kernel<64>), dim3((unsigned)nq), dim3(64), 0, stream, p);
        if (nk > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<64>), dim3((unsigned)nk), dim3(64), 0, stream, p);
    } else {
        hipLaunchKernelGGL((bwd_dq_kernel<128>), dim3((unsigned)nq), dim3(64), 0, stream, p);
        if (nk > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<128>), dim3((unsigned)nk), dim3(64), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
