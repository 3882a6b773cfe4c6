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
// Pipelining (section 10.2's dependency sketch, applied on one wavefront):
// the score product of tile t+1 is issued in the same basic block as the
// softmax of tile t, so the matrix cores work while the vector ALUs compute
// exponentials; K therefore runs one tile ahead of V.  K and V each have two
// LDS buffers and are copied HBM -> LDS directly (buffer loads with the LDS
// destination, range-checked so rows past the valid length arrive as zeros);
// the copies for tiles t+2 (K) and t+1 (V) are issued at the top of step t
// and waited for at its end.
//
// gfx950 mapping.  The score tile is computed transposed, S^T = K Q^T, on
// v_mfma_f32_32x32x16_bf16: the accumulator puts one query per lane (column
// l % 32) with 16 keys per 32-key block, so a row's max and sum are in-lane
// reductions plus one exchange between lanes l and l ^ 32, and the softmax
// state (m, l) is one scalar per lane.  K rows are fed to the MFMA through the
// bit-2/3 swap of fa_device.h, which makes the S^T accumulator, converted to
// bf16, exactly the B operand (P^T, keys as the reduction index) of the second
// product O^T += V^T P^T: the probabilities never leave registers.  V stays
// row-major in LDS; its A-operand fragments (four keys of one column per read)
// come from ds_read_b64_tr_b16, the gfx950 transposing LDS read.  Both tiles
// are XOR-swizzled in 16-byte units so every LDS read is bank-conflict-free.
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

template <int N>
struct Const { static constexpr int value = N; };

template <int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(64 * NW, 512 / (64 * NW)) prefill_kernel(PrefillParams p) {
    constexpr int NT = 64 * NW;             // threads per workgroup
    constexpr int BM = 32 * NW;             // query rows per workgroup
    constexpr int BN = 64;                  // keys per KV tile
    constexpr int KS = D / 16;              // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;              // 32-row blocks of O^T
    constexpr int KB = BN / 32;             // 32-key blocks per KV tile
    constexpr int CH = D / 8;               // 16-byte chunks per K/V row
    constexpr int TILE = BN * D;            // bf16 elements of one K or V tile
    constexpr int NI = BN * CH / NT;        // 16-byte direct copies per thread per tile
    static_assert(NI >= 1 && (BN * CH) % NT == 0, "a tile must split evenly over the workgroup");
    // LDS stages per operand: K(t) lives in K buffer t % NB, V(t) in V buffer t % NB.
    // Step t copies K(t + NB) and V(t + NB - 1), so copies run NB - 2 steps
    // ahead of the step that first needs them.
#ifdef FA_PREFILL_STAGES
    constexpr int NB = FA_PREFILL_STAGES;
#else
    constexpr int NB = D == 64 ? 4 : 3;
#endif
    // Copies issued after the pair a step waits for: NB - 2 steps of 2 * NI.
    constexpr int kPendingAfter = (NB - 2) * 2 * NI;

    // K buffers at [0, NB TILE), V buffers at [NB TILE, 2 NB TILE).
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * NB * TILE];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
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

    // ---- Q tile: B operand of S^T, resident in registers -------------------
    const rsrc_t qbuf = make_rsrc(p.q + qoff, (uint32_t)p.Lq * D * 2);   // rows >= Lq read as zero
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = load16(qbuf, (uint32_t)(qrow * D + ks * 16 + hi * 8) * 2);

    // ---- direct HBM -> LDS copies -----------------------------------------
    // Copy i of wavefront w fills LDS chunk positions P = (w*NI + i)*64 + lane of
    // a tile buffer; position P holds chunk (P % CH) ^ swizzle(row) of row P / CH.
    // The per-lane source offsets are fixed; each tile gets its own buffer
    // descriptor (base advanced by the tile, range = the valid rows left), so
    // rows past n arrive as zeros and the per-tile work is scalar.
    uint32_t koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int P = (w * NI + i) * 64 + l;
        const int row = P / CH;
        koff[i] = (uint32_t)(row * D + (((P % CH) ^ k_swizzle<D>(row)) * 8)) * 2;
        voff[i] = (uint32_t)(row * D + (((P % CH) ^ v_swizzle<D>(row)) * 8)) * 2;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) bf16*)smem);
    auto copy_tile = [&](const bf16* base, int t, int buf, const uint32_t (&offs)[NI]) {
        const int rows = n - t * BN;        // valid rows from the tile start; <= 0 past the end
        const i32x4 d = make_desc(base + kvoff + (size_t)t * BN * D,
                                  (uint32_t)(rows > 0 ? rows : 0) * D * 2);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            copy16_to_lds_async(d, offs[i], lds0 + (uint32_t)(buf * TILE + (w * NI + i) * 512) * 2);
    };
    auto copy_k = [&](int t, int buf) { copy_tile(p.k, t, buf, koff); };
    auto copy_v = [&](int t, int buf) { copy_tile(p.v, t, NB + buf, voff); };

    // ---- per-lane LDS read offsets (constant over the loop) -----------------
    // K (A operand of S^T): row kb*32 + krow, chunk 2*ks + hi.
    const int krow = swap_bits_2_3(l & 31);
    const int kxor = k_swizzle<D>(krow);    // swizzle of rows kb*32 + krow does not depend on kb
    // V (A operand of O^T via the transposing read): row
    // kbase + 8*hi + 4*hh + (l & 15) / 4, column db*32 + 16*((l >> 4) & 1) + 4*(l & 3).
    const int vrow = 8 * hi + ((l & 15) >> 2);
    const int vxor = v_swizzle<D>(vrow);    // rows differ from vrow by multiples of 4
    const int vcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

    auto score_tile = [&](int buf, f32x16 (&s)[KB]) {
        const bf16* Ks = smem + buf * TILE;     // buf: K buffer index
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[kb] = zero_f32x16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    Ks + (kb * 32 + krow) * D + (((2 * ks + hi) ^ kxor) * 8));
                s[kb] = mfma_32x32x16(a, qf[ks], s[kb]);
            }
        }
    };
    // Masks of tile t: valid length, and causal on tiles crossing the diagonal.
    // Tiles past the last one are masked entirely by the same rule.
    auto mask_tile = [&](int t, f32x16 (&s)[KB]) {
        const int k0 = t * BN;
        const bool need = (k0 + BN > n) || (CAUSAL && (k0 + BN - 1 > qw0 + off));
        if (need) {
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
    };
    auto row_max = [&](const f32x16 (&s)[KB]) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
        return max_with_partner(mx);
    };

    // ---- online-softmax state ----------------------------------------------
    const float c = p.c;
    float m = kNegInf;                      // running max of raw scores q.k (this lane's row)
    float ell = 0.0f;                       // this lane's half of the running sum
    f32x16 acc[DB];                         // O^T accumulator: rows d, column = this lane's query
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();

    // One step for tile t, entered with sc = masked S(t) and (m, ell, acc)
    // referenced to the max over tiles 0..t-1.  One basic block holds:
    //   the score product of tile t + 1 (matrix cores), and on the vector ALUs
    //   the row max of tile t, alpha, p = 2^(s c - m c) with the row sum and
    //   P -> bf16, and the rescale of A by alpha;
    //   then O^T += V^T P^T of tile t, each accumulator block rescaled just
    //   before its first product.
    // The rescale is unconditional (no branch), so nothing splits the block and
    // the vector work of tile t overlaps the matrix work.  Tile t + 1 is masked
    // at the end of the step (a branch taken only on diagonal and tail tiles).
    // PH = t % lcm(2, NB) makes every buffer index a compile-time constant.
    // Copies are issued for every step, also past the last tile (they then
    // read zeros), so the number of copies in flight, and with it the wait
    // count at the end of a step, is a constant.
    auto step = [&](int t, f32x16 (&sc)[KB], f32x16 (&sn)[KB], auto phase) {
        constexpr int PH = decltype(phase)::value;
        copy_k(t + NB, PH % NB);                         // into the buffer of K(t), last read in step t - 1
        copy_v(t + NB - 1, (PH + NB - 1) % NB);          // into the buffer of V(t - 1)

        score_tile((PH + 1) % NB, sn);                   // K(t+1) is resident

        const float mx = row_max(sc);
        const float m_new = fmaxf(m, mx);
        const float mc = (m_new == kNegInf) ? 0.0f : m_new * c;    // never form -inf - (-inf)
        const float alpha = exp2_fast(m * c - mc);                 // 0 while the row was empty
        m = m_new;
        float psum = 0.0f;
        bf16x8 pb[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    e[j] = exp2_fast(__builtin_fmaf(sc[kb][8 * half + j], c, -mc));
                    psum += e[j];
                }
                pb[kb][half] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
            }
        ell = alpha * ell + psum;

        const bf16* Vs = smem + (NB + PH % NB) * TILE;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int row0 = kb * 32 + half * 16 + vrow;
                    const int col = db * 32 + vcol;
                    const bf16* base = Vs + row0 * D + (((col >> 3) ^ vxor) * 8) + (col & 7);
                    const bf16x4 lo = lds_read_transposed(base);
                    const bf16x4 up = lds_read_transposed(base + 4 * D);
                    bf16x8 a;
#pragma unroll
                    for (int e = 0; e < 4; ++e) { a[e] = lo[e]; a[4 + e] = up[e]; }
                    acc[db] = mfma_32x32x16(a, pb[kb][half], acc[db]);
                }
        }
        // Interleave: LDS reads run three MFMAs ahead; every MFMA is followed by
        // an even share of the vector work.
        constexpr int kQk = KB * KS, kPv = DB * KB * 2;
        constexpr int kValu = 7 * KB * 8 + 16 * DB + 2 * KB * 8 + 12;
        constexpr int kPer = (kValu + kQk + kPv - 1) / (kQk + kPv);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int i = 0; i < kQk; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // score MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, kPer, 0);   // VALU
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // next LDS read
        }
#pragma unroll
        for (int i = 0; i < kPv; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // PV MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, kPer, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);      // next transposing V reads
        }

        mask_tile(t + 1, sn);
        wait_vector_loads_until<kPendingAfter>();        // K(t+2) and V(t+1) have landed
        __syncthreads();
    };

    // ---- prologue: copies K(0..NB-1), V(0..NB-2); S(0) masked ------------------
    copy_k(0, 0);
    copy_k(1, 1);
    copy_v(0, 0);
#pragma unroll
    for (int j = 2; j < NB; ++j) {
        copy_k(j, j);
        copy_v(j - 1, j - 1);
    }
    wait_vector_loads_until<kPendingAfter>();            // Q, K(0), K(1), V(0) have landed
    __syncthreads();
    f32x16 s0[KB], s1[KB];
    score_tile(0, s0);
    mask_tile(0, s0);
    __syncthreads();                        // step 0 refills K buffer 0

    constexpr int NU = NB % 2 == 0 ? NB : 2 * NB;       // lcm(2, NB)
    auto run = [&](int t, auto phase) {
        if constexpr (decltype(phase)::value % 2 == 0) step(t, s0, s1, phase);
        else step(t, s1, s0, phase);
    };
    for (int t = 0; t < ntiles; t += NU) {
        run(t, Const<0>{});
        if (t + 1 < ntiles) run(t + 1, Const<1>{});
        if (t + 2 < ntiles) run(t + 2, Const<2 % NU>{});
        if (t + 3 < ntiles) run(t + 3, Const<3 % NU>{});
        if constexpr (NU > 4) {
            if (t + 4 < ntiles) run(t + 4, Const<4 % NU>{});
            if (t + 5 < ntiles) run(t + 5, Const<5 % NU>{});
        }
    }

    // ---- epilogue: O = A / l, LSE = ln 2 * (m c + log2 l) -------------------
    const float ell_t = sum_with_partner(ell);
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
    constexpr int NW = kPrefillWaves;
    const dim3 grid((unsigned)total), block(64 * NW);
    if (D == 64) {
        if (causal) hipLaunchKernelGGL((prefill_kernel<64, true, NW>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((prefill_kernel<64, false, NW>), grid, block, 0, stream, p);
    } else {
        if (causal) hipLaunchKernelGGL((prefill_kernel<128, true, NW>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((prefill_kernel<128, false, NW>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
