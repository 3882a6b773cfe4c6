// Prefill forward: one workgroup per (batch, query head, 128-row query block).
//
// Schedule (FlashAttention Cheat Sheet, section 4 "The complete FlashAttention
// flow"; FlashAttention from Scratch, section 6.3): the Q tile is loaded once
// and stays in registers; K and V tiles stream through LDS, double-buffered
// (section 10, "fill one buffer while consuming another"); each KV tile goes
// through S = Q K^T, masking, the online-softmax update and A += P V; O = A / l
// and the LSE are written once at the end.  Each of the four wavefronts owns 32
// complete query rows (FA2's split-Q ownership, section 7.3), so no partial
// outputs are exchanged between wavefronts.
//
// gfx950 mapping.  The score tile is computed transposed, S^T = K Q^T, on
// v_mfma_f32_32x32x16_bf16: the accumulator puts one query per lane (column
// l % 32) with 16 keys per 32-key block, so a row's max and sum are in-lane
// reductions plus one exchange between lanes l and l ^ 32, and the softmax
// state (m, l) is one scalar per lane.  K rows are fed to the MFMA through the
// bit-2/3 swap of fa_device.h, which makes the S^T accumulator, converted to
// bf16, exactly the B operand (P^T, keys as the reduction index) of the second
// product O^T += V^T P^T: the probabilities never leave registers.  V is
// transposed once per tile while it is written to LDS so that each lane's
// A-operand read of V^T is one 16-byte LDS load.
//
// Softmax in base 2 with the scale folded into the exponent: p = 2^(s*c - m*c),
// c = scale * log2(e) (FlashAttention from Scratch, section 6.3, base-2
// exponentials); the LSE is converted back to natural log once
// (LSE = (m*c + log2 l) * ln 2).  alpha = 2^((m_old - m_new) * c) rescales the
// running sum and the accumulator; the accumulator multiply is skipped when no
// row of the wavefront changed its max.  The running max is always the true
// max, so the largest probability of every tile is exactly 1.0 and passes
// through the bf16 P operand unrounded.  (FA4's conditional rescaling keeps a
// stale reference, which puts the dominant probability in (1, 256] where bf16
// rounds it; measured on peaky rows it doubles the worst output error, so it
// is not used.)
//
// Causal work (section 7.3; FlashAttention-4 summary, "LPT scheduling for
// imbalanced grids"): KV tiles past the block's last visible key are never
// visited, elementwise masks are applied only on tiles that cross the
// diagonal or the valid length, a wavefront whose rows all precede a tile
// skips that tile's arithmetic, and query blocks are launched last-first so
// the longest workgroups start earliest.  Workgroups of the query heads that
// share a KV head are adjacent, and when B * Hkv is a multiple of 8 each of
// the eight XCDs (round-robin workgroup dispatch) receives whole KV heads, so
// K/V re-reads across query blocks hit that XCD's L2.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <int D, int BN, bool CAUSAL>
__global__ void __launch_bounds__(256, 2) prefill_kernel(PrefillParams p) {
    constexpr int BM = 128;                 // query rows per workgroup
    constexpr int KS = D / 16;              // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;              // 32-row blocks of O^T
    constexpr int KB = BN / 32;             // 32-key blocks per KV tile
    constexpr int KST = D + 8;              // LDS row stride of K in bf16 (16-byte pad)
    constexpr int VST = BN + 8;             // LDS row stride of V^T in bf16
    constexpr int BUF = BN * KST + D * VST; // one K + V^T buffer, bf16 elements
    constexpr int DG = D / 8;               // 16-byte groups per row
    constexpr int KCH = BN * DG / 256;      // 16-byte K chunks per thread
    constexpr int KPT = BN * DG / 256;      // keys per thread in the V transpose
    static_assert(KCH >= 1 && (BN * DG) % 256 == 0, "tile must split evenly over 256 threads");
    static_assert((BN / KPT) * DG == 256, "V transpose blocks must cover the tile");
    typedef __bf16 bf16xk __attribute__((ext_vector_type(KPT)));

    __shared__ __attribute__((aligned(16))) bf16 smem[2 * BUF];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int hi = l >> 5;                  // which half of the wave (0 or 1)

    // ---- workgroup -> (b, h, query block) ---------------------------------
    const int L = blockIdx.x;
    int qb_rev, unit, hg;
    if (p.xcd_units > 0) {
        const int xcd = L & 7, slot = L >> 3;
        const int per = p.xcd_units * p.r;
        qb_rev = slot / per;
        const int rem = slot - qb_rev * per;
        unit = xcd * p.xcd_units + rem / p.r;
        hg = rem % p.r;
    } else {
        const int per = p.B * p.Hq;
        qb_rev = L / per;
        const int rem = L - qb_rev * per;
        unit = rem / p.r;
        hg = rem % p.r;
    }
    const int qb = p.n_qblocks - 1 - qb_rev;
    const int b = unit / p.Hkv;
    const int g = unit - b * p.Hkv;
    const int h = g * p.r + hg;

    int n = p.Lk;
    if (p.kv_lens) {
        n = p.kv_lens[b];
        n = n < 0 ? 0 : (n > p.Lk ? p.Lk : n);
    }
    const int off = n - p.Lq;               // query i sits at key position i + off
    const int q0 = qb * BM;
    const int qw0 = q0 + w * 32;            // first row of this wavefront
    const int qrow = qw0 + (l & 31);        // the row this lane's column holds
    int kv_end = n;
    if (CAUSAL) {
        const int last = min(q0 + BM, p.Lq) + off;  // keys < last are visible to some row
        kv_end = min(n, max(last, 0));
    }
    const int ntiles = (kv_end + BN - 1) / BN;

    const size_t qoff = (size_t)(b * p.Hq + h) * p.Lq * D;
    const size_t kvoff = (size_t)(b * p.Hkv + g) * p.Lk * D;

    // Range-checked buffers: Q rows >= Lq and K/V rows >= n read as zero.
    const rsrc_t qbuf = make_rsrc(p.q + qoff, (uint32_t)p.Lq * D * 2);
    const rsrc_t kbuf = make_rsrc(p.k + kvoff, (uint32_t)n * D * 2);
    const rsrc_t vbuf = make_rsrc(p.v + kvoff, (uint32_t)n * D * 2);

    // ---- Q tile: B operand of S^T, resident in registers -------------------
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = load16(qbuf, (uint32_t)(qrow * D + ks * 16 + hi * 8) * 2);

    // ---- K/V tile staging: global -> registers -> LDS -----------------------
    bf16x8 kreg[KCH];
    bf16x8 vreg[KPT];
    // V: this thread's KPT-key group and 8-column group.  Consecutive lanes take
    // consecutive key groups, so one transposed LDS store of a wavefront covers
    // contiguous bytes of V^T rows (all 64 banks, no conflicts).
    constexpr int KG = BN / KPT;
    const int vkg = tid % KG;
    const int vdg = tid / KG;

    auto load_tile = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + 256 * i;
            const int row = c / DG, col = c % DG;
            kreg[i] = load16(kbuf, (uint32_t)((k0 + row) * D + col * 8) * 2);
        }
#pragma unroll
        for (int i = 0; i < KPT; ++i)   // rows past n read as zero: 0 * garbage would be NaN
            vreg[i] = load16(vbuf, (uint32_t)((k0 + vkg * KPT + i) * D + vdg * 8) * 2);
    };
    auto store_tile = [&](int buf) {
        bf16* Ks = smem + buf * BUF;
        bf16* Vs = Ks + BN * KST;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + 256 * i;
            const int row = c / DG, col = c % DG;
            *reinterpret_cast<bf16x8*>(Ks + row * KST + col * 8) = kreg[i];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16xk col;
#pragma unroll
            for (int i = 0; i < KPT; ++i) col[i] = vreg[i][e];
            *reinterpret_cast<bf16xk*>(Vs + (vdg * 8 + e) * VST + vkg * KPT) = col;
        }
    };

    // ---- online-softmax state ----------------------------------------------
    const float c = p.c;
    float m = kNegInf;                      // running max of raw scores q.k (this lane's row)
    float ell = 0.0f;                       // this lane's half of the running sum
    f32x16 acc[DB];                         // O^T accumulator: rows d, column = this lane's query
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();

    const int krow = swap_bits_2_3(l & 31);

    // Prologue, unconditional: with range-checked loads an empty tile reads as
    // zeros, and every Q load is then complete before the loop starts.
    load_tile(0);
    store_tile(0);
    wait_all_vector_loads();   // Q is resident: no wait on it inside the loop
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) load_tile(t + 1);
        const int k0 = t * BN;
        const bool wave_active = !CAUSAL || (k0 <= qw0 + 31 + off);
        if (wave_active) {
            const bf16* Ks = smem + buf * BUF;
            const bf16* Vs = Ks + BN * KST;

            // S^T = K Q^T
            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                s[kb] = zero_f32x16();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        Ks + (kb * 32 + krow) * KST + ks * 16 + hi * 8);
                    s[kb] = mfma_32x32x16(a, qf[ks], s[kb]);
                }
            }

            // Masks: valid length, and causal on tiles crossing the diagonal.
            const bool need_mask = (k0 + BN > n) || (CAUSAL && (k0 + BN - 1 > qw0 + off));
            if (need_mask) {
                const int qpos = qrow + off;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = k0 + kb * 32 + 16 * (v >> 3) + 8 * hi + (v & 7);
                        const bool ok = key < n && (!CAUSAL || key <= qpos);
                        if (!ok) s[kb][v] = kNegInf;
                    }
            }

            // Row max: in-lane, then across the two lanes holding this row.
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
            mx = fmaxf(mx, lane_xor32(mx));

            const float m_new = fmaxf(m, mx);
            const float mc = (m_new == kNegInf) ? 0.0f : m_new * c;  // never form -inf - (-inf)
            const float alpha = exp2_fast(m * c - mc);               // 0 while the row was empty

            // p = 2^(s c - m c), row sum, and P^T as the B operand of the PV product.
            float psum = 0.0f;
            bf16x8 pb[KB][2];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        e[j] = exp2_fast(__builtin_fmaf(s[kb][8 * half + j], c, -mc));
                        psum += e[j];
                    }
                    pb[kb][half] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
                }
            ell = alpha * ell + psum;
            m = m_new;

            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
            }

            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                            Vs + (db * 32 + (l & 31)) * VST + kb * 32 + half * 16 + hi * 8);
                        acc[db] = mfma_32x32x16(a, pb[kb][half], acc[db]);
                    }
        }
        if (t + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = A / l, LSE = ln 2 * (m c + log2 l) -------------------
    const float ell_t = ell + lane_xor32(ell);
    const float inv = ell_t > 0.0f ? 1.0f / ell_t : 0.0f;
    if (qrow < p.Lq) {
        bf16* Op = p.o + qoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                bf16x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = (bf16)(acc[db][4 * grp + j] * inv);
                *reinterpret_cast<bf16x4*>(Op + db * 32 + 8 * grp + 4 * hi) = ov;
            }
        if (p.lse && hi == 0)
            p.lse[(size_t)(b * p.Hq + h) * p.Lq + qrow] =
                ell_t > 0.0f ? (m * c + log2_fast(ell_t)) * kLn2 : kNegInf;
    }
}

hipError_t launch_prefill(int D, bool causal, const PrefillParams& p, hipStream_t stream) {
    const long long total = (long long)p.B * p.Hq * p.n_qblocks;
    const dim3 grid((unsigned)total), block(256);
    if (D == 64) {
        if (causal) hipLaunchKernelGGL((prefill_kernel<64, 128, true>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((prefill_kernel<64, 128, false>), grid, block, 0, stream, p);
    } else {
        if (causal) hipLaunchKernelGGL((prefill_kernel<128, 64, true>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((prefill_kernel<128, 64, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
