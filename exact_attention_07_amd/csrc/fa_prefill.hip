// Prefill forward: one workgroup per (batch, query head, 256-row query block).
//
// Schedule (FlashAttention Cheat Sheet, section 4 "The complete FlashAttention
// flow"; FlashAttention from Scratch, section 6.3): the Q tile is loaded once
// and stays in registers; K and V tiles stream through LDS in three stages
// (section 10, "fill one buffer while consuming another"), copied HBM -> LDS
// directly (buffer loads with the LDS destination, range-checked so rows past
// the valid length arrive as zeros); each KV tile goes through S = Q K^T,
// masking, the online-softmax update and A += P V; O = A / l and the LSE are
// written once at the end.  Each of the eight wavefronts owns 32 complete
// query rows (FA2's split-Q ownership, section 7.3), so no partial outputs are
// exchanged between wavefronts.
//
// Ping-pong (FlashAttention-3 summary, "ping-pong scheduling" of two warp
// groups): the wavefronts form two groups of four, one wavefront of each group
// per SIMD, and every wavefront alternates a matrix phase M(t) -- the score
// product of tile t+1 and O^T += V^T P^T of tile t -- with a vector phase
// V(t) -- mask, row max and p = 2^(s c - r) for tile t+1.  The second group
// runs one phase behind the first, and a workgroup barrier ends every phase,
// so while one wavefront of a SIMD keeps the matrix cores busy the other one
// computes exponentials on the vector ALUs.  The matrix phase runs at raised
// wave priority so its products issue first.
//
// LDS stages.  K(j) lives in K buffer j % 3, V(j) in V buffer j % 3.  With the
// first group's M(t) in phase 2t and the second's in 2t+1, K(j) is read in
// phases 2j-2, 2j-1 and V(j) in 2j, 2j+1.  M(t) copies K(t+3) (into the
// buffer of K(t), free since phase 2t) and V(t+2) (into that of V(t-1), free
// since phase 2t); every wavefront waits for the copies of M(t-1) at the end
// of M(t), so all of K(t+2) and V(t+1) are resident after phase 2t+1, before
// their first reader in phase 2t+2.
//
// gfx950 mapping.  Scores are computed transposed, S^T = K Q^T, on
// v_mfma_f32_32x32x16_bf16: the accumulator puts one query per lane (column
// l % 32) with 16 keys per 32-key block, so a row's max and sum are in-lane
// reductions plus one exchange between lanes l and l ^ 32.  K rows are fed
// through the bit-2/3 swap of fa_device.h, which makes the S^T accumulator,
// converted to bf16, exactly the B operand (P^T) of the second product
// O^T += V^T P^T: the probabilities never leave registers.  V stays row-major
// in LDS; its A-operand fragments come from ds_read_b64_tr_b16, the gfx950
// transposing LDS read.  Both tiles are XOR-swizzled in 16-byte units so every
// LDS read is bank-conflict-free.
//
// Softmax in base 2 with the scale folded into the exponent: p = 2^(s c - r),
// c = scale * log2(e), r = the row's reference (FlashAttention from Scratch,
// section 6.3, base-2 exponentials).  The reference is a past row max plus
// kTau of headroom; it is only moved (to kTau above the current max), and A
// and l rescaled by
// alpha = 2^(r_old - r_new), when a tile's probabilities for the row sum to
// more than 2^kTau (the conditional rescaling of the FlashAttention-4 summary,
// with the sum as the test so that the common path needs no row max); between
// moves every p <= 2^kTau, far from fp32 overflow.  Because p is rounded to bf16 for the PV product, O is
// normalised by the sum of the rounded probabilities (one v_dot2 per pair),
// so numerator and denominator carry the same weights and a dominant key
// passes through exactly; the LSE uses the fp32 sum of the unrounded ones.
//
// Causal work (section 7.3; FlashAttention-4 summary, "LPT scheduling for
// imbalanced grids"): KV tiles past the block's last visible key are never
// visited, nor, under a causal window of width w (section 12: a key is
// allowed when it is at most w - 1 positions before the query), the tiles
// wholly before the window of the block's first row; tile indices below are
// counted from that first visited tile, so the LDS stage of a tile stays a
// compile-time function of the loop position, elementwise masks are applied only on tiles that cross the
// diagonal or the valid length, and query blocks are launched last-first so
// the longest workgroups start earliest.  Workgroups of the query heads that
// share a KV head are adjacent, and when B * Hkv is a multiple of 8 each of
// the eight XCDs (round-robin workgroup dispatch) receives whole KV heads, so
// K/V re-reads across query blocks hit that XCD's L2.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <int N>
struct Const { static constexpr int value = N; };

// The reference sits kTau (base 2) above the row max when it is set, and a
// tile's probabilities may sum to at most kTauSum = 2^kTau per row before it
// moves again.
constexpr float kTau = 8.0f;
constexpr float kTauSum = 256.0f;

// Exact probabilities for rows that a few keys dominate (D = 128 kernels).  P
// enters the PV product rounded to bf16 (relative error up to 2^-8), which
// moves O by up to 2^-8 sum_j P_j |v_j - O|: on rows that a few keys dominate
// that reaches a few 1e-3 of an output of magnitude 2-4.  Such a row is
// recognised when its reference moves (the row max is known exactly then):
// its largest p is at least kPeakFrac of its running sum, judged only once
// the row has seen kJudgeKeys of its keys (or all, if it has fewer), since a
// row whose first tile holds a few of its keys is dominated there whatever
// the rest.  Once kSplitRows rows of a workgroup are (a head whose scores
// spread widely), the workgroup switches, for the rest of its KV loop, to
// split probabilities: the residual p - bf16(p), itself rounded to bf16, goes
// through a second product with the same V fragments, so every weight is
// exact to ~2^-16, and the tile's normaliser is the fp32 sum of p (which its
// weights then match to ~2^-18).  The switch is one counter in LDS that every wavefront adds to; each
// reads it after the prologue's tile and then once per cycle of LDS stages,
// and moves from the plain tile loop to a split one (whose matrix phase
// follows every PV product by its residual product on the same fragment), so
// the plain loop carries no residual code.  All wavefronts of a workgroup
// then do the same work per tile, so the phases stay balanced.  The modifier
// and FP8 kernels keep bf16 probabilities (their bars account for them).
constexpr float kPeakFrac = 1.0f / 2.0f;
constexpr int kSplitRows = 16;              // dominated rows that switch a workgroup to split probabilities
constexpr int kJudgeKeys = 32;              // keys a row must have seen to be judged dominated

typedef int i32x8 __attribute__((ext_vector_type(8)));

// FP8 instantiation: S^T = K Q^T from E4M3 codes on
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales in the instruction; the
// tile's dequantisation factor s_q s_k goes into the exponent's scale).  A
// lane holds 32 bytes of its K row (A) or Q row (B); the instruction pairs
// byte e of lane half hi in A with the same in B, so giving both the bytes
// 64 ks + 32 hi + e of a row makes the product a dot product over D.  K rows
// of D bytes sit in LDS in 16-byte chunks XOR-swizzled by k8_swizzle, so 16
// lanes reading one chunk column of 16 rows hit 16 distinct bank groups (of
// 16 bytes: group (D/16) row + chunk, mod 16).  V and P stay bf16 (the PV
// product is the bf16 one).
template <int D>
__device__ __forceinline__ int k8_swizzle(int row) {
    return D == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}
template <bool FP8>
struct ScoreOperand { typedef bf16x8 type; };
template <>
struct ScoreOperand<true> { typedef i32x8 type; };

// Score modifiers (FlashAttention from Scratch, section 12: S' = f(S, i, j)
// before the softmax), applied to the tile's raw scores before the masks, in
// the units the exponent uses (x = s c - r):
//   MOD 1, ALiBi:     s -= (slope_h / scale) |pos_i - pos_j|
//   MOD 2, soft-cap:  s  = (cap / scale) tanh(s scale / cap)
//                        = (cap / scale) (1 - 2 / (1 + 2^(s 2 scale log2(e) / cap)))
// (an exponential and a reciprocal per score; 2^(large) = inf gives 1, and
// 2^(-large) = 0 gives -1).
constexpr int kModNone = 0, kModAlibi = 1, kModSoftcap = 2;
constexpr float kPosInf = __builtin_inff();

template <int D, bool CAUSAL, bool WINDOW, bool FP8 = false, int MOD = kModNone, bool VARLEN = false,
          bool QQ = false>
__global__ void __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(PrefillParams p) {
    constexpr int NW = 8;                   // wavefronts: two groups of four
    constexpr int NT = 64 * NW;             // threads per workgroup
    constexpr int BM = 32 * NW;             // query rows per workgroup
    constexpr int BN = 64;                  // keys per KV tile
    constexpr int KS = D / 16;              // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;              // 32-row blocks of O^T
    constexpr int KB = BN / 32;             // 32-key blocks per KV tile
    constexpr int CH = D / 8;               // 16-byte chunks per K/V row
    constexpr int TILE = BN * D;            // bf16 elements of one K or V tile
    constexpr int NI = BN * CH / NT;        // 16-byte direct copies per thread per tile
    constexpr int NB = 3;                   // LDS stages per operand (the tile loop is unrolled by NB)
    static_assert(BM == kPrefillRows, "host and kernel disagree on the query block");
    static_assert(NI >= 1 && (BN * CH) % NT == 0, "a tile must split evenly over the workgroup");
    static_assert(CAUSAL || !WINDOW, "the window is causal");
    static_assert(!FP8 || !WINDOW, "the FP8 scores are built without a window");
    static_assert(MOD == kModNone || (!FP8 && !WINDOW), "score modifiers are built for the bf16 kernel without a window");
    static_assert(!VARLEN || (!FP8 && !WINDOW && MOD == kModNone), "packed batches are built for the plain bf16 kernel");
    static_assert(!QQ || FP8, "Q is quantized in the kernel only for FP8 scores");
    constexpr bool QBF16 = !FP8 || QQ;      // Q arrives in bf16 (staged through LDS)
    // Split probabilities in the bf16 kernels at D = 128 without modifiers: the
    // modifier and FP8 instantiations keep bf16 probabilities throughout.
    constexpr bool CORR = D == 128 && !FP8 && MOD == kModNone;
    constexpr int KSQ = FP8 ? D / 64 : KS;  // k-steps of S^T
    // 16-byte copies per thread per K tile.  An E4M3 tile at D = 64 (4 KB) is
    // half a copy per thread: the copies of its second half of positions fall
    // on rows past the tile, outside the descriptor's range (nothing is
    // read), into the unused second half of the stage buffer.
    constexpr int NIK = FP8 ? (BN * D + NT * 16 - 1) / (NT * 16) : NI;
    static_assert(NIK >= 1, "a K tile must split evenly over the workgroup");
    typedef typename ScoreOperand<FP8>::type SA;

    // K buffers at [0, NB TILE), V buffers at [NB TILE, 2 NB TILE).
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * NB * TILE];
    // bf16 residuals of corrected 16-key chunks: [wave][chunk][lane], written in
    // a wavefront's vector phase and read in its next matrix phase.
    constexpr int NCH = KB * 2;                     // 16-key chunks per tile
    __shared__ __attribute__((aligned(16))) bf16x8 plo_lds[D == 128 ? NW * NCH * 64 : 1];
    __shared__ __attribute__((aligned(16))) bf16 qst[(QBF16 && D == 64) ? 256 * 64 : 8];   // Q staging at D = 64
    __shared__ float qmax_w[QQ ? NW : 1];   // QQ: each wavefront's largest |transformed Q|
    __shared__ int split_rows;              // rows of the workgroup found dominated by a few keys

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
    const int grp = w >> 2;                 // ping-pong group; waves w and w + 4 share a SIMD
    const int l = tid & 63;
    const int hi = l >> 5;                  // which half of the wave (0 or 1)
    if (tid == 0) split_rows = 0;           // visible after the prologue's first barrier

    // ---- workgroup -> (b, h, query block) ---------------------------------
    const int L = blockIdx.x;
    // Within an XCD, workgroups go to its four shader engines round-robin by
    // dispatch position, whatever their load, and when the engine next in
    // turn is full, dispatch to the others waits too.  So the heads of a query
    // block are laid out with the higher bits of the head index folded into
    // its two low bits by XOR (an involution that keeps every aligned group of
    // four together, so the r query heads of a KV head stay adjacent): heads
    // whose cost differs with a period of 2, 4 or 8 (every 8th head scaled,
    // say) then cover all four engines within every block.
    auto spread_heads = [](int rem, int per) {
        if (per & 3) return rem;
        const int x = rem >> 2;
        return rem ^ ((x ^ (x >> 2) ^ (x >> 4) ^ (x >> 6)) & 3);
    };
    int qblk, b, g, h;                      // query block, sequence, KV head, query head
    int Lq, n;                              // the sequence's query rows and valid keys
    size_t qoff, kvoff, lse_off;            // element offsets of its Q/O rows, K/V rows and LSE
    if constexpr (VARLEN) {
        // Packed batch.  Work item `it` is one query block of one sequence
        // with all its query heads (Hq consecutive workgroups); the items run
        // through the sequences in the schedule's longest-tile-first order,
        // each sequence's query blocks last-first (the longest first under the
        // causal rule).  The grid is an upper bound: workgroups past the
        // batch's items, or that a schedule inconsistent with the offsets
        // leaves without a query block, exit at once.
        const int it = L / p.Hq;
        const int s = L - it * p.Hq;
        const int* prefix = p.schedule + p.B;
        if (it >= prefix[p.B]) return;
        int lo = 0, up = p.B - 1;           // the last position whose items start at or before it
        while (lo < up) {
            const int mid = (lo + up + 1) >> 1;
            if (prefix[mid] <= it) lo = mid; else up = mid - 1;
        }
        b = min(max(p.schedule[lo], 0), p.B - 1);
        int q_start, k_start;
        varlen_segment(p.cu_q, b, p.Lq, q_start, Lq);
        varlen_segment(p.cu_k, b, p.Lk, k_start, n);
        const int nqb = (Lq + BM - 1) / BM;
        const int j = it - prefix[lo];
        if (j < 0 || j >= nqb) return;
        qblk = nqb - 1 - j;
        // Heads.  The XCD of a workgroup is s % 8 (round-robin dispatch, Hq a
        // multiple of 8); it takes one block of Hq / 8 adjacent query heads --
        // whole KV heads, so their K/V tiles are shared in its L2 -- and the
        // block rotates with the item, so heads that differ in cost are spread
        // over the XCDs; within the block, the position rotates every second
        // item, which spreads them over the XCD's shader engines too.
        const int per = p.Hq >> 3;
        if ((p.Hq & 7) == 0 && per % p.r == 0) {
            const int blk = ((s & 7) + it) & 7;
            h = blk * per + ((s >> 3) + (it >> 1)) % per;
        } else {
            h = s;
        }
        g = h / p.r;
        qoff = ((size_t)h * p.Lq + q_start) * D;
        kvoff = ((size_t)g * p.Lk + k_start) * D;
        lse_off = (size_t)h * p.Lq + q_start;
    } else {
        int qb_rev, unit, hg;
        if (p.xcd_spread) {
            // XCD x owns the query-block pairs (n-1-q, q) for q = x, x+8, ...: first
            // its heavy blocks in descending order, then its light ones; within a
            // block, every (batch, KV head) with its r query heads adjacent.
            const int xcd = L & 7, slot = L >> 3;
            const int per = p.B * p.Hq;
            const int j = slot / per;
            const int rem = spread_heads(slot - j * per, per);
            const int M = p.n_qblocks >> 4;      // pairs per XCD
            const int q = j < M ? xcd + 8 * j : xcd + 8 * (2 * M - 1 - j);
            qb_rev = j < M ? q : p.n_qblocks - 1 - q;
            unit = rem / p.r;
            hg = rem % p.r;
        } else if (p.xcd_units > 0) {
            const int xcd = L & 7, slot = L >> 3;
            const int per = p.xcd_units * p.r;
            qb_rev = slot / per;
            const int rem = spread_heads(slot - qb_rev * per, per);
            unit = xcd * p.xcd_units + rem / p.r;
            hg = rem % p.r;
        } else {
            const int per = p.B * p.Hq;
            qb_rev = L / per;
            const int rem = spread_heads(L - qb_rev * per, per);
            unit = rem / p.r;
            hg = rem % p.r;
        }
        qblk = p.n_qblocks - 1 - qb_rev;
        b = unit / p.Hkv;
        g = unit - b * p.Hkv;
        h = g * p.r + hg;
        Lq = p.Lq;
        n = p.Lk;
        if (p.kv_lens) {
            n = p.kv_lens[b];
            n = n < 0 ? 0 : (n > p.Lk ? p.Lk : n);
        }
        qoff = (size_t)(b * p.Hq + h) * p.Lq * D;
        kvoff = (size_t)(b * p.Hkv + g) * p.Lk * D;
        lse_off = (size_t)(b * p.Hq + h) * p.Lq;
    }
    const int off = n - Lq;                 // query i sits at key position i + off
    const int q0 = qblk * BM;
    const int qw0 = q0 + w * 32;            // first row of this wavefront
    const int qrow = qw0 + (l & 31);        // the row this lane's column holds
    int kv_end = n;
    if (CAUSAL) {
        const int last = min(q0 + BM, Lq) + off;    // keys < last are visible to some row
        kv_end = min(n, max(last, 0));
    }
    // First visited tile: under a window, the one holding the lowest key
    // visible to the block's first row (q0 + off - w + 1).
    int tb = 0;
    if (WINDOW) tb = max(q0 + off - p.window + 1, 0) / BN;
    const int ntiles = (kv_end + BN - 1) / BN - tb;   // tiles visited, counted from tb
    // Visit order.  With ALiBi the tiles run from the last one down: under
    // the bias the nearest keys score highest, so the row maxima are found
    // first and the reference rarely moves afterwards (in key order the max
    // of a steep head rises by tens of binades per tile, a move every tile).
    // Positions t >= ntiles (the prologue's tile when the block sees no key,
    // and copies past the end) map past the visited range in either order, so
    // the masks treat them as in key order.
    constexpr bool REV = MOD == kModAlibi;
    auto tile_abs = [&](int t) { return (REV && t < ntiles) ? tb + ntiles - 1 - t : tb + t; };

    // FP8: exponent scale of tile t = c s_q s_k(t); s_k is read one tile ahead
    // (QQ: s_q is found in the prologue).
    float cq = (FP8 && !QQ) ? p.c * p.q_scale[(size_t)(b * p.Hq + h) * p.n_qblocks + qblk] : p.c;

    // ---- Q tile: B operand of S^T, resident in registers -------------------
    SA qf[KSQ];
    if constexpr (FP8 && !QQ) {
        const rsrc_t qbuf = make_rsrc(p.q8 + qoff, (uint32_t)Lq * D);   // rows >= Lq read as zero
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
            const uint32_t at = (uint32_t)(qrow * D + 64 * ks + 32 * hi);
            const i32x4 lo = __builtin_bit_cast(i32x4, load16(qbuf, at));
            const i32x4 up = __builtin_bit_cast(i32x4, load16(qbuf, at + 16));
            qf[ks] = i32x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
        }
    }
    // bf16 kernels: each wavefront copies its 32 rows of Q straight into LDS
    // as whole rows (1 KB of consecutive rows per copy instruction; rows past
    // Lq arrive as zeros), 16-byte chunks XOR-swizzled by the row so the
    // fragment reads below hit distinct banks, and reads its B-operand
    // fragments back once they have landed (wavefront-local, in the
    // prologue).  Staging: at D = 128 the residual buffer (wavefronts 0-3)
    // and V buffers 1-2 (wavefronts 4-7; V(1) is copied after the prologue's
    // barrier), at D = 64 a buffer of its own.
    constexpr int NQC = 32 * D * 2 / 1024;  // copies per lane
    bf16* qs_w = D == 128 ? (w < 4 ? reinterpret_cast<bf16*>(plo_lds) + w * 32 * D
                                   : smem + (NB + 1) * TILE + (w - 4) * 32 * D)
                          : qst + w * 32 * D;
    // Chunk swizzle of a staged row: with 256-byte rows (D = 128) the row's
    // low bits; with 128-byte rows two rows share the 64 banks, so bits 1-3.
    // The 16 rows of one 16-lane group of a fragment read then hit 16
    // distinct 16-byte bank groups.
    auto q_swz = [](int row) { return D == 128 ? row & 15 : (row >> 1) & 7; };
    if constexpr (QBF16) {
        const int vq = min(max(Lq - qw0, 0), 32);
        const i32x4 qd = make_desc(p.q + qoff + (size_t)min(qw0, Lq) * D, (uint32_t)vq * D * 2);
        const uint32_t qs_addr = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) bf16*)qs_w);
#pragma unroll
        for (int i = 0; i < NQC; ++i) {
            const int P = i * 64 + l;
            const int row = P / CH;
            copy16_to_lds_async(qd, (uint32_t)(row * D + ((P % CH) ^ q_swz(row)) * 8) * 2, qs_addr + i * 1024);
        }
    }
    // QQ: the E4M3 codes of Q made here, exactly as the block quantizer makes
    // them (one power-of-two scale per 256-row block, the workgroup's query
    // block; the optional random-sign Hadamard transform, FlashAttention-3's
    // incoherent processing).  A lane takes the D / 2 elements of its row that
    // its E4M3 operand holds, 64 ks + 32 hi + e (e < 32), from the staged bf16
    // rows; x' = H (sigma x) runs in fp64 as butterflies over the index bits,
    // in the lane for bits 0-4 and 6 (positions 32 ks + e) and between lanes
    // l and l ^ 32 for bit 5.  Every partial sum is exact in fp64 for inputs
    // whose exponents span at most 38 binades, so the order of the
    // butterflies does not change the result, rounded once to fp32.
    constexpr int NE = QQ ? D / 2 : 1;
    float qx[NE];
    auto quantize_q_local = [&]() __attribute__((always_inline)) {
        if constexpr (QQ) {
            const int row = l & 31;
            double x[NE];
#pragma unroll
            for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int e0 = 64 * ks + 32 * hi + 8 * cc;   // first element of the chunk
                    u32x4 raw = *reinterpret_cast<const u32x4*>(
                        qs_w + row * D + (((8 * ks + 4 * hi + cc) ^ q_swz(row)) * 8));
                    if (p.q_signs) {
                        // sigma: a sign flip of the bf16 bits where the sign's
                        // own sign bit is set (word k holds elements 2k, 2k+1).
                        const u32x4 s0 = *reinterpret_cast<const u32x4*>(p.q_signs + e0);
                        const u32x4 s1 = *reinterpret_cast<const u32x4*>(p.q_signs + e0 + 4);
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const unsigned a = k < 2 ? s0[2 * k] : s1[2 * k - 4];
                            const unsigned c = k < 2 ? s0[2 * k + 1] : s1[2 * k - 3];
                            raw[k] ^= ((a >> 16) & 0x8000u) | (c & 0x80000000u);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        x[32 * ks + 8 * cc + 2 * k] = (double)__builtin_bit_cast(float, raw[k] << 16);
                        x[32 * ks + 8 * cc + 2 * k + 1] = (double)__builtin_bit_cast(float, raw[k] & 0xFFFF0000u);
                    }
                }
            if (p.q_signs) {
#pragma unroll
                for (int bit = 1; bit < NE; bit <<= 1)
#pragma unroll
                    for (int i = 0; i < NE; ++i)
                        if ((i & bit) == 0) {
                            const double a = x[i], c2 = x[i + bit];
                            x[i] = a + c2;
                            x[i + bit] = a - c2;
                        }
                // Index bit 5 lies between lanes l and l ^ 32.  One exchange
                // of x[i] (upper lanes) with x[i + 4] (lower lanes), local
                // bit 2 of i clear, gives each lane both partners of one
                // index: the lower lanes of i, the upper lanes of i + 4.  The
                // butterfly then leaves y(bit 5 clear) in slot i and y(bit 5
                // set) in slot i + 4 on either half; the codes are exchanged
                // back once encoded (four per word).
#pragma unroll
                for (int i = 0; i < NE; ++i)
                    if ((i & 4) == 0) {
                        const unsigned long long a = __builtin_bit_cast(unsigned long long, x[i]);
                        const unsigned long long c2 = __builtin_bit_cast(unsigned long long, x[i + 4]);
                        const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)c2, false, false);
                        const auto up = __builtin_amdgcn_permlane32_swap((unsigned)(a >> 32), (unsigned)(c2 >> 32),
                                                                         false, false);
                        // [0]: x[i] with its upper lanes from x[i + 4] of the lower lanes;
                        // [1]: x[i + 4] with its lower lanes from x[i] of the upper lanes.
                        const double A = __builtin_bit_cast(double, ((unsigned long long)up[0] << 32) | lo[0]);
                        const double C = __builtin_bit_cast(double, ((unsigned long long)up[1] << 32) | lo[1]);
                        x[i] = A + C;
                        x[i + 4] = A - C;
                    }
            }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                qx[i] = (float)x[i];
                amax = fmaxf(amax, fabsf(qx[i]));
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
            if (l == 0) qmax_w[w] = amax;       // read after the prologue's barrier
        }
    };
    // After the barrier: the block maximum, its scale 2^k (the smallest power
    // of two with max 2^-k <= 448, E4M3's largest finite value) and the codes
    // of x' 2^-k (round to nearest even) as the B operand.
    auto quantize_q_finish = [&]() __attribute__((always_inline)) {
        if constexpr (QQ) {
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < NW; ++i) amax = fmaxf(amax, qmax_w[i]);
            int k = 0;
            if (amax > 0.0f) {
                int e;
                (void)frexpf(amax, &e);     // amax in [2^(e-1), 2^e)
                k = (amax <= ldexpf(0.875f, e)) ? e - 9 : e - 8;
            }
            cq = p.c * ldexpf(1.0f, k);
            auto encode4 = [&](const float* v) __attribute__((always_inline)) {
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[0], -k), ldexpf(v[1], -k), 0, false);
                return __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[2], -k), ldexpf(v[3], -k), lo, true);
            };
#pragma unroll
            for (int ks = 0; ks < KSQ; ++ks) {
                SA f;
#pragma unroll
                for (int d = 0; d < 8; d += 2) {
                    const int we = encode4(qx + 32 * ks + 4 * d);
                    const int wo = encode4(qx + 32 * ks + 4 * d + 4);
                    if (p.q_signs) {
                        // Word d of the upper lanes is held by the lower lanes
                        // (as their word d + 1) and the other way round.
                        const auto r = __builtin_amdgcn_permlane32_swap((unsigned)we, (unsigned)wo, false, false);
                        f[d] = (int)r[0];
                        f[d + 1] = (int)r[1];
                    } else {
                        f[d] = we;
                        f[d + 1] = wo;
                    }
                }
                qf[ks] = f;
            }
        }
    };
    auto read_q = [&]() __attribute__((always_inline)) {
        if constexpr (!FP8) {
            const int row = l & 31;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = *reinterpret_cast<const bf16x8*>(qs_w + row * D + (((2 * ks + hi) ^ q_swz(row)) * 8));
        }
    };
    const int nks = (p.Lk + kFp8KBlock - 1) / kFp8KBlock;
    const float* kscale = FP8 ? p.k_scale + (size_t)(b * p.Hkv + g) * nks : nullptr;
    auto k_scale_of = [&](int t) __attribute__((always_inline)) {   // tile index relative to tb
        return (FP8 && nks > 0) ? kscale[min(tb + t, nks - 1)] : 1.0f;   // no K rows: nothing to read
    };

    // ---- direct HBM -> LDS copies -----------------------------------------
    // Copy i of wavefront w fills LDS chunk positions P = (w*NI + i)*64 + lane of
    // a tile buffer; position P holds chunk (P % CH) ^ swizzle(row) of row P / CH.
    // The per-lane source offsets are fixed; each tile gets its own buffer
    // descriptor (base advanced by the tile, range = the valid rows left), so
    // rows past n arrive as zeros and the per-tile work is scalar.
    uint32_t koff[NIK], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int P = (w * NI + i) * 64 + l;
        const int row = P / CH;
        if (!FP8) koff[i] = (uint32_t)(row * D + (((P % CH) ^ k_swizzle<D>(row)) * 8)) * 2;
        voff[i] = (uint32_t)(row * D + (((P % CH) ^ v_swizzle<D>(row)) * 8)) * 2;
    }
    if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < NIK; ++i) {     // E4M3 rows of D bytes: D / 16 chunks
            const int P = (w * NIK + i) * 64 + l;
            const int row = P / (D / 16);
            koff[i] = (uint32_t)(row * D + (((P % (D / 16)) ^ k8_swizzle<D>(row)) * 16));
        }
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) bf16*)smem);
    auto copy_tile = [&](const bf16* base, int t, int buf, const uint32_t (&offs)[NI]) __attribute__((always_inline)) {
        const int ta = tile_abs(t);         // absolute tile index
        // Valid rows from the tile start; <= 0 past the end (in reverse order,
        // the copies past the last visited tile fetch nothing either).
        const int rows = (REV && t >= ntiles) ? 0 : n - ta * BN;
        const i32x4 d = make_desc(base + kvoff + (size_t)(rows > 0 ? ta : 0) * BN * D,
                                  (uint32_t)(rows > 0 ? rows : 0) * D * 2);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            copy16_to_lds_async(d, offs[i], lds0 + (uint32_t)(buf * TILE + (w * NI + i) * 512) * 2);
    };
    auto copy_k = [&](int t) __attribute__((always_inline)) {
        if constexpr (FP8) {
            const int ta = tb + t;
            const int rows = min(n - ta * BN, BN);   // the tile's rows only (see NIK)
            const i32x4 d = make_desc(p.k8 + kvoff + (size_t)(rows > 0 ? ta : 0) * BN * D,
                                      (uint32_t)(rows > 0 ? rows : 0) * D);
#pragma unroll
            for (int i = 0; i < NIK; ++i)
                copy16_to_lds_async(d, koff[i], lds0 + (uint32_t)((t % NB) * TILE * 2 + (w * NIK + i) * 1024));
        } else {
            copy_tile(p.k, t, t % NB, koff);
        }
    };
    auto copy_v = [&](int t) { copy_tile(p.v, t, NB + t % NB, voff); };

    // ---- per-lane LDS read offsets (constant over the loop) -----------------
    // K (A operand of S^T): row kb*32 + krow, chunk 2*ks + hi.
    const int krow = swap_bits_2_3(l & 31);
    const int kxor = k_swizzle<D>(krow);    // swizzle of rows kb*32 + krow does not depend on kb
    // V (A operand of O^T via the transposing read): row
    // kbase + 8*hi + 4*hh + (l & 15) / 4, column db*32 + 16*((l >> 4) & 1) + 4*(l & 3).
    const int vrow = 8 * hi + ((l & 15) >> 2);
    const int vxor = v_swizzle<D>(vrow);    // rows differ from vrow by multiples of 4
    const int vcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

    // A operand (K rows) of score step ks of key block kb, and the product.
    auto k_operand = [&](const bf16* Ks, int kb, int ks) __attribute__((always_inline)) -> SA {
        if constexpr (FP8) {
            const uint8_t* row = reinterpret_cast<const uint8_t*>(Ks) + (kb * 32 + krow) * D;
            const int x8 = k8_swizzle<D>(krow);   // rows kb*32 + krow share it
            const int c0 = 4 * ks + 2 * hi;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(row + ((c0 ^ x8) * 16));
            const i32x4 up = *reinterpret_cast<const i32x4*>(row + (((c0 + 1) ^ x8) * 16));
            return i32x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
        } else {
            return *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + krow) * D + (((2 * ks + hi) ^ kxor) * 8));
        }
    };
    auto score_mfma = [&](const SA& a, int ks, const f32x16& acc_in) __attribute__((always_inline)) -> f32x16 {
        if constexpr (FP8)
            return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], acc_in, 0, 0, 0, 127, 0, 127);
        else
            return mfma_32x32x16(a, qf[ks], acc_in);
    };

    f32x16 s[KB];                           // S^T of the tile being prepared
    auto score_tile = [&](int t) __attribute__((always_inline)) {
        const bf16* Ks = smem + (t % NB) * TILE;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s[kb] = zero_f32x16();
#pragma unroll
            for (int ks = 0; ks < KSQ; ++ks) s[kb] = score_mfma(k_operand(Ks, kb, ks), ks, s[kb]);
        }
    };

    // ---- online-softmax state ----------------------------------------------
    const float c = p.c;
    float ref = kNegInf;                    // reference r = (running max) * c; -inf while the row is empty
    float ell_e = 0.0f;                     // the row's sum of p (both lanes of the row hold it)
    float ell_r = 0.0f;                     // this lane's half of the normaliser: sum of bf16(p) (split tiles: of p)
    f32x16 acc[DB];                         // O^T accumulator: rows d, column = this lane's query
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();
    // p of the tile whose PV product is next, as fp32 from the vector phase;
    // the matrix phase converts it to the bf16 P^T operand (and sums the
    // rounded values) while its score products run.
    float pe[KB][2][8];
    bf16x8 pbs[KB][2];                      // split tiles: bf16(p), converted in the vector phase
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    bool split = false;                     // this wavefront splits its probabilities (wave-uniform, sticky)
    float ksc_next = k_scale_of(0);         // FP8: s_k of the tile softmax_tile handles next
    // Modifier constants in raw-score units.
    const float mod_a = MOD == kModAlibi ? p.alibi_slopes[h] / p.scale
                      : MOD == kModSoftcap ? p.softcap / p.scale : 0.0f;   // slope, or cap
    const float mod_b = MOD == kModSoftcap ? 2.0f * p.scale * 1.4426950408889634f / p.softcap : 0.0f;

    // Residuals p - bf16(p) of every 16-key chunk of pe to LDS, for the next
    // matrix phase's residual products.  Inside the split loop the rounded
    // halves stay in registers (pbs, `keep`) as that phase's P^T operands,
    // and the tile's normaliser is the fp32 sum of p: its weights
    // bf16(p) + bf16(p - bf16(p)) are within 2^-18 of p, relative.  A tile
    // that enters the split loop (the prologue's, or the one after the
    // switch) keeps the plain tiles' form instead -- its matrix phase converts
    // P^T and sums the rounded values -- and adds its residuals' sum (`sum`),
    // so no split operand stays live through the plain loop.
    auto write_residuals = [&](auto keep, auto sum) __attribute__((always_inline)) -> float {
        float rs[2] = {0.0f, 0.0f};
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
            const float* e = pe[cc / 2][cc % 2];
            const bf16x8 hi8 = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
            if constexpr (decltype(keep)::value) pbs[cc / 2][cc % 2] = hi8;
            float r8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                r8[j] = e[j] - (float)hi8[j];
                if constexpr (decltype(sum)::value) rs[j & 1] += r8[j];
            }
            plo_lds[(w * NCH + cc) * 64 + l] = to_bf16x8(r8[0], r8[1], r8[2], r8[3], r8[4], r8[5], r8[6], r8[7]);
        }
        return rs[0] + rs[1];
    };
    float rs_first = 0.0f;                  // residual sum of the prologue's tile

    // Vector phase for tile t (scores in s): mask where needed, p -> pe and the
    // fp32 row sum, and the rare reference move.  MODE (split probabilities,
    // D = 128): 0 plain; 1 plain, and the wavefront switches to split
    // probabilities from this tile on once the workgroup's count is reached
    // (only before a matrix phase of LDS stage 0, so each form of the tile
    // loop runs whole stage cycles); 2 split; 3 plain, with the residuals
    // written and their sum kept aside (the prologue's tile, whose form is
    // decided after it).
    auto softmax_tile = [&](int t, auto mode) __attribute__((always_inline)) {
        constexpr int MODE = CORR ? decltype(mode)::value : 0;
        const int k0 = tile_abs(t) * BN;
        // The workgroup's split count, read early (used after the exponentials).
        const int flag_seen = MODE == 1 ? split_rows : 0;
        const float ct = FP8 ? cq * ksc_next : c;   // this tile's exponent scale
        if (FP8) ksc_next = k_scale_of(t + 1);
        // ALiBi: |pos_i - pos_j| = |base - K_v| with base = qpos - k0 - 8 hi
        // and K_v = 32 kb + 16 (v / 8) + v % 8.  Where every key of the tile
        // is on one side of every row of the wavefront (sign sgn of
        // pos_i - pos_j), the bias is linear in K_v and goes into the
        // exponent's fma instead (see exponentials); else it is added here.
        const float base = (float)(qrow + off - k0 - 8 * hi);
        const int sgn = MOD != kModAlibi ? 0 : (qw0 + off >= k0 + BN - 1) ? 1 : (k0 > qw0 + 31 + off) ? -1 : 0;
        auto add_alibi = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    s[kb][v] = __builtin_fmaf(-mod_a, fabsf(base - (float)(kb * 32 + 16 * (v >> 3) + (v & 7))), s[kb][v]);
        };
        if constexpr (MOD == kModAlibi) {
            if (sgn == 0) add_alibi();
        } else if constexpr (MOD == kModSoftcap) {
            // s becomes u = 1 / (1 + 2^(s mod_b)); the capped score is
            // mod_a (1 - 2u), whose last fma merges into the exponent's.
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    s[kb][v] = __builtin_amdgcn_rcpf(1.0f + exp2_fast(s[kb][v] * mod_b));
        }
        // A masked element's value: -inf, or for the cap u = +inf (capped score -inf).
        constexpr float kMasked = MOD == kModSoftcap ? kPosInf : kNegInf;
        // Elementwise masks only where some pair of this wavefront's rows and
        // the tile is out: past n, above the diagonal, or (window) at least w
        // positions before the wavefront's last row.
        const bool need = (k0 + BN > n) || (CAUSAL && (k0 + BN - 1 > qw0 + off)) ||
                          (WINDOW && (qw0 + 31 + off - k0 >= p.window));
        if (need) {
            // Element (kb, v) holds key base + idx with idx a compile-time
            // constant, so every condition is one compare of idx against a
            // per-lane limit: key < n and (causal) key <= qpos give
            // idx <= lim; (window) qpos - key < w gives idx >= lo.
            const int qpos = qrow + off;
            const int base = k0 + 8 * hi;
            const int lim = CAUSAL ? min(n - 1, qpos) - base : n - 1 - base;
            const int lo = WINDOW ? qpos - p.window + 1 - base : 0;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int idx = kb * 32 + 16 * (v >> 3) + (v & 7);
                    const bool ok = WINDOW ? (idx <= lim) & (idx >= lo) : idx <= lim;
                    s[kb][v] = ok ? s[kb][v] : kMasked;   // a select, no branch
                }
        }
        // p = 2^(s c - r), the tile's sums and P -> bf16, against the current
        // reference.  Four partial sums of p and two of bf16(p) keep the
        // dependency chains short.
        float se[4];
        bool folded = MOD == kModAlibi && sgn != 0;    // bias still to be applied, in the exponent
        auto exponentials = [&]() __attribute__((always_inline)) {
            const float r = ref == kNegInf ? 0.0f : ref;   // never form -inf - (-inf)
            // Folded ALiBi: s ct - r - a ct sgn (base - K_v) = fma(s, ct, fma(c1, K_v, b0)).
            const float c1 = folded ? (float)sgn * mod_a * ct : 0.0f;
            const float b0 = folded ? __builtin_fmaf(-c1, base, -r) : -r;
            // Soft-cap: mod_a (1 - 2u) ct - r = fma(u, -2 mod_a ct, mod_a ct - r).
            const float sa = MOD == kModSoftcap ? -2.0f * mod_a * ct : ct;
            const float sb = MOD == kModSoftcap ? __builtin_fmaf(mod_a, ct, -r) : b0;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float kv = (float)(kb * 32 + 16 * half + j);
                        const float t = (MOD == kModAlibi) ? __builtin_fmaf(c1, kv, b0) : sb;
                        pe[kb][half][j] = exp2_fast(__builtin_fmaf(s[kb][8 * half + j], sa, t));
                        // The first four terms start the partial sums (p >= 0, so
                        // 0 + p would be p: no add needed).
                        if (kb == 0 && half == 0 && j < 4) se[j] = pe[kb][half][j];
                        else se[j & 3] += pe[kb][half][j];
                    }
        };
        exponentials();
        // The reference holds while the row's tile sum of p is at most
        // 2^kTau, which bounds every single p by 2^kTau; no row max is needed
        // on this path.  An empty-so-far row, a larger sum, or a sum that is
        // not finite moves it: to kTau above the true row max (so the max must
        // rise by about 2 kTau before the next move), with A and l rescaled,
        // and the tile is recomputed.  The move is decided per wavefront, so
        // the headroom keeps it rare even on rows whose max keeps climbing.
        float se_l = (se[0] + se[1]) + (se[2] + se[3]);
        float row_sum = sum_with_partner(se_l);
        const bool move = ref == kNegInf || !(row_sum <= kTauSum);
        if constexpr (MODE == 1)   // counted by all wavefronts at earlier phases
            split = __builtin_amdgcn_readfirstlane(flag_seen) >= kSplitRows;
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(move) != 0, 0)) {
            if constexpr (MOD == kModAlibi) {
                // The row max is of the biased scores: apply the bias here.
                if (folded) add_alibi();
                folded = false;
            }
            float mx;
            if constexpr (MOD == kModSoftcap) {
                // The capped score falls as u rises: its max is at the least u
                // (+inf, a row with no valid key so far, gives -inf).
                float m8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) m8[j] = fminf(fminf(s[0][j], s[0][j + 8]), fminf(s[1][j], s[1][j + 8]));
#pragma unroll
                for (int j = 0; j < 4; ++j) m8[j] = fminf(m8[j], m8[j + 4]);
                const float umin = -max_with_partner(-fminf(fminf(m8[0], m8[1]), fminf(m8[2], m8[3])));
                mx = __builtin_fmaf(-2.0f * mod_a, umin, mod_a);
            } else {
                float m8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) m8[j] = fmaxf(fmaxf(s[0][j], s[0][j + 8]), fmaxf(s[1][j], s[1][j + 8]));
#pragma unroll
                for (int j = 0; j < 4; ++j) m8[j] = fmaxf(m8[j], m8[j + 4]);
                mx = fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3]));
                mx = max_with_partner(mx);
            }
            const bool shift = move && mx != kNegInf;   // a row with no valid key so far keeps -inf
            const float r_new = shift ? mx * ct + kTau : ref;  // kTau of headroom above the max
            const float alpha = shift ? exp2_fast(ref - r_new) : 1.0f;   // 0 from an empty row
            ref = r_new;
            ell_e *= alpha;
            ell_r *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
            exponentials();
            se_l = (se[0] + se[1]) + (se[2] + se[3]);
            row_sum = sum_with_partner(se_l);
            if constexpr (CORR) {
                // After the move the row's largest p is exactly 2^-kTau.  A row
                // is judged once it has seen kJudgeKeys of its keys, or all of
                // them if it has fewer (key order: its keys up to the tile's
                // end so far); a row with a few keys so far is dominated now
                // whatever the rest of its keys.
                const int qpos = qrow + off;
                const int key_hi = min(CAUSAL ? qpos : n - 1, n - 1);
                const int key_lo = WINDOW ? max(qpos - p.window + 1, 0) : 0;
                const int seen = min(key_hi, k0 + BN - 1) - key_lo + 1;
                const bool judged = seen >= min(kJudgeKeys, key_hi - key_lo + 1);
                const bool dominated = shift && judged && 1.0f / kTauSum >= kPeakFrac * (ell_e + row_sum);
                const uint64_t dm = __builtin_amdgcn_ballot_w64(dominated && hi == 0);   // one lane per row
                if (MODE != 2 && dm != 0 && l == 0) atomicAdd(&split_rows, (int)__builtin_popcountll(dm));
            }
        }
        if constexpr (MODE != 0) {
            if (MODE == 3) {
                rs_first = write_residuals(Const<false>{}, Const<true>{});
            } else if (MODE == 2) {
                write_residuals(Const<true>{}, Const<false>{});
                ell_r += se_l;              // the split tile's normaliser: the fp32 sum
            } else if (__builtin_expect(split, 0)) {
                ell_r += write_residuals(Const<false>{}, Const<true>{});
            }
        }
        ell_e += row_sum;
    };

    // Matrix phase M(t) as one software pipeline over its products: the KB*KS
    // score products of tile t+1, then the DB*KB*2 PV products of tile t, each
    // group ordered so that consecutive products go to different accumulators
    // (the two key blocks' S^T, the DB blocks of O^T).
    // Product i is issued right after the LDS read(s) of product i + AHEAD, so
    // every operand is read AHEAD products (~32 cycles each) before its use
    // and only ~AHEAD fragments are live.  A scheduling fence after each step
    // keeps this order.
    // The split form (SPL, a splitting wavefront's phase) follows each PV
    // product by its residual product, with the same V fragment and the same
    // accumulator (a back-to-back accumulation); the residual operand of a
    // 16-key chunk is read from LDS with the chunk's first V fragment.
    auto matrix_phase = [&](auto phase, auto form) __attribute__((always_inline)) {
        constexpr int PH = decltype(phase)::value;      // t % NB
        // FORM 0: plain; 1: split, P^T converted here from pe with its
        // rounded sums (the tile entering the split loop); 2: split, P^T
        // from the vector phase (pbs), normalised by the fp32 sum.
        constexpr int FORM = decltype(form)::value;
        constexpr bool SPL = FORM != 0;
        const bf16* Ks = smem + ((PH + 1) % NB) * TILE;
        const bf16* Vs = smem + (NB + PH) * TILE;
        constexpr int NQ = KB * KSQ;        // score products
        constexpr int NF = DB * KB * 2;     // PV products (one V fragment each)
        constexpr int NOPS = NQ + NF;
        constexpr int AHEAD = 6;
        constexpr int NP = KB * 2;          // bf16x8 operands of P^T (16-key chunks)
        SA kfrag[NQ];                       // score operands
        bf16x8 frag[NOPS];                  // PV operands (entries NQ..)
        bf16x8 plo[NP];                     // residual operands (SPL)
        auto read_op = [&](int i) __attribute__((always_inline)) {
            if (i < NQ) {
                kfrag[i] = k_operand(Ks, i % KB, i / KB);
            } else {
                const int f = i - NQ;
                const int db = f % DB, kb = (f / DB) / 2, half = (f / DB) % 2;
                const int row0 = kb * 32 + half * 16 + vrow;
                const int col = db * 32 + vcol;
                const bf16* base = Vs + row0 * D + (((col >> 3) ^ vxor) * 8) + (col & 7);
                const bf16x4 lo = lds_read_transposed(base);
                const bf16x4 up = lds_read_transposed(base + 4 * D);
#pragma unroll
                for (int e = 0; e < 4; ++e) { frag[i][e] = lo[e]; frag[i][4 + e] = up[e]; }
                if (SPL && db == 0) plo[f / DB] = plo_lds[(w * NP + f / DB) * 64 + l];
            }
        };
        // P -> bf16 operand and the rounded row sum, spread over the score
        // products (which do not need them): conversion q follows score
        // product q NQ / NP (several per product when there are fewer score
        // products than operands, as with E4M3 scores at D = 64); the PV
        // products come after.
        bf16x8 pb[KB][2];
        float sr[2] = {0.0f, 0.0f};
        auto convert_p = [&](int q) __attribute__((always_inline)) {
            const int kb = q / 2, half = q % 2;
            const float* e = pe[kb][half];
            if constexpr (FORM == 2) {
                // A split tile's operand was converted in the vector phase,
                // and its normaliser is its fp32 sum (no rounded sums).
                pb[kb][half] = pbs[kb][half];
            } else {
                const bf16x8 pv = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
                pb[kb][half] = pv;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sr[j & 1] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pv[2 * j], pv[2 * j + 1]}, ones, sr[j & 1], false);
                // Pin the sums here, between the score products: otherwise the
                // compiler sinks them (and a second conversion of P) to the end
                // of the phase.
                asm volatile("" : "+v"(sr[0]), "+v"(sr[1]));
            }
        };
        auto mfma_op = [&](int i) __attribute__((always_inline)) {
            if (i < NQ) {
                const int kb = i % KB, ks = i / KB;
                s[kb] = score_mfma(kfrag[i], ks, ks == 0 ? zero_f32x16() : s[kb]);
#pragma unroll
                for (int q = 0; q < NP; ++q)
                    if (q * NQ / NP == i) convert_p(q);
                if (FORM != 2 && i == NQ - 1) ell_r += sr[0] + sr[1];
            } else {
                const int f = i - NQ;
                const int db = f % DB, kb = (f / DB) / 2, half = (f / DB) % 2;
                acc[db] = mfma_32x32x16(frag[i], pb[kb][half], acc[db]);
                if constexpr (SPL) acc[db] = mfma_32x32x16(frag[i], plo[f / DB], acc[db]);
            }
        };
        if constexpr (SPL) {
            // Side-effect marker: keeps the compiler from merging the two forms
            // of the phase (executing the residual products as selects).
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) read_op(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NOPS; ++i) {
            mfma_op(i);
            if (i + AHEAD < NOPS) read_op(i + AHEAD);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- prologue: K(0..2), V(0..1) resident; S(0) -> P(0) -------------------
    // V(1) waits for the prologue's barrier where its buffer stages Q.
    constexpr bool LATE_V1 = QBF16 && D == 128;
    copy_k(0);
    copy_k(1);
    copy_v(0);
    copy_k(2);
    if (!LATE_V1) copy_v(1);
    // Q and K(0) only: the other tiles stream in while S(0) and P(0) are
    // computed (vmcnt counts in issue order, the Q copies first).
    wait_vector_loads_until<2 * NIK + (LATE_V1 ? 1 : 2) * NI>();
    if constexpr (QBF16) {
        asm volatile("" ::: "memory");      // the staged rows are read only after the wait
        if constexpr (QQ) quantize_q_local();
        else read_q();
    }
    __syncthreads();                        // K(0) visible; every wavefront's Q read from its staging
    if constexpr (QQ) quantize_q_finish();
    if (LATE_V1) copy_v(1);
    score_tile(0);
    softmax_tile(0, Const<3>{});
    wait_vector_loads_until<NIK + NI>();    // K(1) and V(0), the first matrix phase's operands
    __syncthreads();                        // ... visible; K(0) read by every wavefront before M(0) refills its buffer
    if (grp == 1) __syncthreads();          // the second group runs one phase behind

    // One tile: matrix phase M(t), barrier, vector phase V(t), barrier.
    // PH = t % NB is a compile-time constant, so every LDS offset is one.
    // MODE as in softmax_tile; the matrix phase takes the split form in mode 2.
    auto tile_step = [&](int t, auto phase, auto mode, auto form) __attribute__((always_inline)) {
        // ---- matrix phase M(t) ----
        __builtin_amdgcn_s_setprio(1);
        copy_k(t + NB);                     // into the buffer of K(t)
        copy_v(t + NB - 1);                 // into the buffer of V(t - 1)
        // The score product runs for the last tile too (on the zero-filled
        // buffer past the end; the result is not used), which keeps the
        // phase one basic block.
        matrix_phase(phase, form);
        __builtin_amdgcn_s_setprio(0);
        wait_vector_loads_until<NIK + NI>();   // the copies of M(t-1) have landed
        __syncthreads();
        // ---- vector phase V(t) ----
        if (t + 1 < ntiles) softmax_tile(t + 1, mode);
        __syncthreads();
    };
    // Split probabilities: the plain loop runs until this wavefront switches
    // (at the end of a stage cycle), then the split loop runs the rest.  Both
    // take the same barriers per tile, so wavefronts in either loop stay in step.
    int t = 0;
    if constexpr (CORR) {
        // The counts of the prologue's tile are complete: a workgroup whose
        // rows are dominated from the start splits from its first product.
        split = __builtin_amdgcn_readfirstlane(split_rows) >= kSplitRows;
        ell_r += split ? rs_first : 0.0f;
        if (!split) for (; t < ntiles; t += NB) {
            tile_step(t, Const<0>{}, Const<0>{}, Const<0>{});
            if (t + 1 < ntiles) tile_step(t + 1, Const<1>{}, Const<0>{}, Const<0>{});
            if (t + 2 < ntiles) tile_step(t + 2, Const<2>{}, Const<1>{}, Const<0>{});
            if (__builtin_expect(split, 0)) {
                t += NB;
                break;
            }
        }
        // The split loop's first stage cycle: its first matrix phase converts
        // the entering tile's P^T itself (form 1); later ones take the vector
        // phase's operands (form 2).
        if (t < ntiles) {
            tile_step(t, Const<0>{}, Const<2>{}, Const<1>{});
            if (t + 1 < ntiles) tile_step(t + 1, Const<1>{}, Const<2>{}, Const<2>{});
            if (t + 2 < ntiles) tile_step(t + 2, Const<2>{}, Const<2>{}, Const<2>{});
            t += NB;
        }
    }
    for (; t < ntiles; t += NB) {
        constexpr int M = CORR ? 2 : 0;
        tile_step(t, Const<0>{}, Const<M>{}, Const<M>{});
        if (t + 1 < ntiles) tile_step(t + 1, Const<1>{}, Const<M>{}, Const<M>{});
        if (t + 2 < ntiles) tile_step(t + 2, Const<2>{}, Const<M>{}, Const<M>{});
    }
    if (grp == 0) __syncthreads();          // match the second group's extra barrier
    wait_all_vector_loads();                // copies past the last tile (zero-range) drained

    // ---- epilogue: O = A / l_r, LSE = ln 2 * (r + log2 l_e) ------------------
    const float le = ell_e;
    const float lr = sum_with_partner(ell_r);
    const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
    // O goes out through LDS so that each store instruction writes whole rows:
    // a lane's accumulator holds 8-byte pieces of its row spread over the
    // row, so direct stores would touch 32 rows per instruction.  Each
    // wavefront stages its 32 rows in the now idle K/V buffers, row-major with
    // 16-byte chunks XOR-swizzled by the row (q_swz) and, for rows 16-31, the
    // two 8-byte halves of a chunk swapped, so the 32 lanes of one half of a
    // write (one 8-byte piece of each of 32 rows) hit 64 distinct banks.  It
    // then stores 64 / (D / 8) full rows per instruction through a descriptor
    // over its valid rows (the halves swapped back in registers).
    __syncthreads();                        // every wavefront's copies into the buffers have landed
    constexpr int CPR = D / 8;              // 16-byte chunks per row of O
    bf16* ost = smem + w * 32 * D;
    {
        const int r = l & 31;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                bf16x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = (bf16)(acc[db][4 * gq + j] * inv);
                const int chunk = (4 * db + gq) ^ q_swz(r);
                *reinterpret_cast<bf16x4*>(ost + r * D + chunk * 8 + 4 * (hi ^ (r >> 4))) = ov;
            }
    }
    __syncthreads();
    {
        constexpr int RPI = 64 / CPR;       // rows per store instruction
        // The offsets below equal those of the Q copies; a fresh lane index
        // keeps the compiler from holding those through the tile loop.
        int lane = l;
        asm volatile("" : "+v"(lane));
        const int cl = lane % CPR, rl = lane / CPR;
        const int vrows = min(max(Lq - qw0, 0), 32);
        const rsrc_t obuf = make_rsrc(p.o + qoff + (size_t)min(qw0, Lq) * D, (uint32_t)vrows * D * 2);
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int r = i * RPI + rl;     // rows of instruction i all below 16 or all from 16
            bf16x8 v = *reinterpret_cast<const bf16x8*>(ost + r * D + ((cl ^ q_swz(r)) * 8));
            if (i * RPI >= 16) v = __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), obuf,
                                                   (uint32_t)(r * D + cl * 8) * 2, 0, 0);
        }
    }
    if (p.lse && hi == 0 && qrow < Lq)
        p.lse[lse_off + qrow] = le > 0.0f ? (ref + log2_fast(le)) * kLn2 : kNegInf;
}

template <int D>
void launch_prefill_d(bool causal, bool window, const PrefillParams& p, dim3 grid, dim3 block,
                      hipStream_t stream) {
    if (window)      hipLaunchKernelGGL((prefill_kernel<D, true, true>), grid, block, 0, stream, p);
    else if (causal) hipLaunchKernelGGL((prefill_kernel<D, true, false>), grid, block, 0, stream, p);
    else             hipLaunchKernelGGL((prefill_kernel<D, false, false>), grid, block, 0, stream, p);
}

template <int D, bool QQ>
void launch_prefill_fp8_d(bool causal, const PrefillParams& p, dim3 grid, dim3 block, hipStream_t stream) {
    if (causal) hipLaunchKernelGGL((prefill_kernel<D, true, false, true, kModNone, false, QQ>), grid, block, 0, stream, p);
    else        hipLaunchKernelGGL((prefill_kernel<D, false, false, true, kModNone, false, QQ>), grid, block, 0, stream, p);
}

hipError_t launch_prefill_fp8(int D, bool causal, const PrefillParams& p, hipStream_t stream, bool quantize_q) {
    const long long total = (long long)p.B * p.Hq * p.n_qblocks;
    const dim3 grid((unsigned)total), block(512);
    if (D == 64) {
        if (quantize_q) launch_prefill_fp8_d<64, true>(causal, p, grid, block, stream);
        else            launch_prefill_fp8_d<64, false>(causal, p, grid, block, stream);
    } else {
        if (quantize_q) launch_prefill_fp8_d<128, true>(causal, p, grid, block, stream);
        else            launch_prefill_fp8_d<128, false>(causal, p, grid, block, stream);
    }
    return hipGetLastError();
}

template <int D, int MOD>
void launch_prefill_mod_d(bool causal, const PrefillParams& p, dim3 grid, dim3 block, hipStream_t stream) {
    if (causal) hipLaunchKernelGGL((prefill_kernel<D, true, false, false, MOD>), grid, block, 0, stream, p);
    else        hipLaunchKernelGGL((prefill_kernel<D, false, false, false, MOD>), grid, block, 0, stream, p);
}

hipError_t launch_prefill_mod(int D, bool causal, int mod, const PrefillParams& p, hipStream_t stream) {
    const long long total = (long long)p.B * p.Hq * p.n_qblocks;
    const dim3 grid((unsigned)total), block(512);
    if (D == 64) {
        if (mod == kModAlibi) launch_prefill_mod_d<64, kModAlibi>(causal, p, grid, block, stream);
        else                  launch_prefill_mod_d<64, kModSoftcap>(causal, p, grid, block, stream);
    } else {
        if (mod == kModAlibi) launch_prefill_mod_d<128, kModAlibi>(causal, p, grid, block, stream);
        else                  launch_prefill_mod_d<128, kModSoftcap>(causal, p, grid, block, stream);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_varlen(int D, bool causal, const PrefillParams& p, int items, hipStream_t stream) {
    const dim3 grid((unsigned)((long long)items * p.Hq)), block(512);
    if (D == 64) {
        if (causal) hipLaunchKernelGGL((prefill_kernel<64, true, false, false, kModNone, true>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((prefill_kernel<64, false, false, false, kModNone, true>), grid, block, 0, stream, p);
    } else {
        if (causal) hipLaunchKernelGGL((prefill_kernel<128, true, false, false, kModNone, true>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((prefill_kernel<128, false, false, false, kModNone, true>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_prefill(int D, bool causal, const PrefillParams& p, hipStream_t stream) {
    const long long total = (long long)p.B * p.Hq * p.n_qblocks;
    const dim3 grid((unsigned)total), block(512);
    const bool window = causal && p.window > 0;
    if (D == 64) launch_prefill_d<64>(causal, window, p, grid, block, stream);
    else         launch_prefill_d<128>(causal, window, p, grid, block, stream);
    return hipGetLastError();
}

}  // namespace fa
