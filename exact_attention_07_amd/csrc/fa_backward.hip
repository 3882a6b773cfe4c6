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
// Both kernels run workgroups whose wavefronts share 32-row tiles: the
// workgroup streams the tiles through LDS stages with direct HBM -> LDS
// copies (range-checked, so rows past the valid length arrive as zeros),
// issued ahead of their use -- two stages and one tile ahead, or in the
// D = 128 dk/dv kernel three stages and two tiles ahead -- with one barrier
// per tile.
//
// Launch order (FlashAttention-4 summary, "LPT scheduling for imbalanced
// grids"): under a causal mask the last query blocks see the most keys and
// the first key blocks are seen by the most queries, so each kernel numbers
// its workgroups block-major with the longest blocks first, and a workgroup
// that starts late is a short one.  Dispatch deals workgroups to the eight
// XCDs round-robin; the numbering keeps all blocks of one (batch, head) on
// one XCD when the head count is a multiple of eight, so the tiles that its
// blocks re-read are shared in that XCD's L2.
//
// dq kernel: one workgroup per (batch, query head, 128 queries), each
// wavefront owning 32 of them.  Q and G of a wavefront's queries stay in
// registers as B operands; K and V tiles of 32 keys are shared.  Per tile, on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation: S^T = K Q^T and dP^T = V G^T (K and V rows fed
// through the bit-2/3 swap, as in the forward, so that key 16*(v/8) + 8*hi +
// (v%8) sits in accumulator entry v), P^T and dS^T elementwise with one query
// per lane (its LSE and delta in registers), then dQ^T += K^T dS^T with K^T
// from the transposing LDS read and dS^T rounded to bf16 as the B operand.
// The wavefront also forms delta_i = G_i . O_i for its queries (one dot
// product per lane pair) and stores it for the second kernel.
//
// dk/dv kernels: one workgroup per (batch, KV head, 128 keys), each
// wavefront working on 32 of them.  The workgroup visits every query tile of
// every query head that reads this KV head (section 9.2's grouping, so the
// GQA sum happens in registers) and skips tiles no query of which can see its
// keys (causal, window).  Per shared 32-query tile (Q, G, and the rows' LSE
// and delta): S = Q K^T and dP = G V^T with the query rows fed through the
// bit-2/3 swap, which makes the P and dS accumulators, rounded to bf16,
// exactly the A operands of dV += P^T G and dK += dS^T Q; G and Q enter those
// as B operands through the transposing LDS read.  Keys past a sequence's
// valid length get zero gradient.  D = 64 (bwd_dkdv_kernel): four
// wavefronts, each with both accumulators, K and V in LDS.  D = 128
// (bwd_dkdv_split_kernel): eight wavefronts in a dV and a dK role, pipelined
// one tile apart (see there).
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

// 16-byte-chunk XOR swizzle of the backward's LDS tiles, which are read two
// ways: one row per lane (16 lanes: 16 consecutive rows, one chunk column)
// and by the transposing read (32 lanes: 4 consecutive rows, aligned, times 4
// consecutive chunks, aligned).  The first needs the swizzle to be a
// bijection on the row's low bits (bits 1..3 at D = 64, where two rows share
// the 64 banks); the second needs the 4 rows moved to 4 (D = 128) or 2
// (D = 64) different aligned chunk groups, i.e. swizzle bits 2 (and 3) taken
// from the row's low bits.  Both reads are then free of bank conflicts.
template <int D>
__device__ __forceinline__ int bwd_swizzle(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Direct HBM -> LDS copies of a 32-row tile of a [rows, D] bf16 tensor by the
// workgroup's NT threads into a tile buffer laid out row-major with
// bwd_swizzle.  Copy i of wavefront w fills 16-byte chunk position
// P = (w * NI + i) * 64 + lane of the buffer, so each thread reads chunk
// (P % CH) ^ swizzle(row) of row P / CH: the fixed per-lane source offsets
// carry the swizzle and every copy instruction writes 1 KiB of consecutive
// LDS.  Rows past `valid` arrive as zeros and are not fetched.
template <int D, int NT = 256>
struct TileCopy {
    static constexpr int CH = D / 8;
    static constexpr int NI = 32 * CH / NT;
    static_assert(NI >= 1 && (32 * CH) % NT == 0, "a tile must split evenly over the workgroup");
    uint32_t off[NI];
    __device__ __forceinline__ void init(int w, int l) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int P = (w * NI + i) * 64 + l;
            const int row = P / CH;
            off[i] = (uint32_t)(row * D + (((P % CH) ^ bwd_swizzle<D>(row)) * 8)) * 2;
        }
    }
    __device__ __forceinline__ void issue(const bf16* src, int valid, uint32_t lds_buf, int w) const {
        const i32x4 d = make_desc(src, (uint32_t)(valid > 0 ? valid : 0) * D * 2);
#pragma unroll
        for (int i = 0; i < NI; ++i) copy16_to_lds_async(d, off[i], lds_buf + (uint32_t)((w * NI + i) * 64 * 16));
    }
};


// A compile-time step index of an unrolled tile loop.
template <int N>
struct BwdStage { static constexpr int value = N; };

// Products per pipeline step are issued AHEAD steps after their operands'
// LDS reads, with a scheduling fence after every step so the compiler keeps
// that distance (otherwise it places each read right before its product and
// waits for it there).
constexpr int kAhead = 4;

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// Queries base + idx that key `key` may pair with, as a range of idx:
// i < Lq; (causal) key <= i + off; (window) i + off - key < w; none when the
// key is past n.
__device__ __forceinline__ void query_range(int base, int key, int n, int off, const BwdParams& p,
                                            int& lo, int& hi_lim) {
    lo = p.causal ? key - off - base : INT_MIN;
    hi_lim = p.Lq - 1 - base;
    if (p.window > 0) hi_lim = min(hi_lim, key + p.window - 1 - off - base);
    if (key >= n) hi_lim = -1;
}

// A-operand fragment: row `row` of a swizzled tile, 16-byte chunk `chunk`.
template <int D>
__device__ __forceinline__ bf16x8 read_row_chunk(const bf16* tile, int row, int chunk) {
    return *reinterpret_cast<const bf16x8*>(tile + row * D + ((chunk ^ bwd_swizzle<D>(row)) * 8));
}

// Transposed fragment of a swizzled tile: lane l receives column
// col0 + (l % 32) of rows row0 + 8*(l/32) + e, e = 0..7 (the operand layout of
// an MFMA whose k index runs down the tile's rows).  Each lane's two 8-byte
// reads are addressed through the swizzle of their own rows.
template <int D>
__device__ __forceinline__ bf16x8 read_transposed(const bf16* tile, int row0, int col0, int l) {
    const int hi = l >> 5;
    const int r = row0 + 8 * hi + ((l & 15) >> 2);
    const int col = col0 + 16 * ((l >> 4) & 1) + 4 * (l & 3);
    const bf16* a = tile + r * D + (((col >> 3) ^ bwd_swizzle<D>(r)) * 8) + (col & 7);
    const bf16* b = tile + (r + 4) * D + (((col >> 3) ^ bwd_swizzle<D>(r + 4)) * 8) + (col & 7);
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


// Two wavefronts per SIMD: the register budget that keeps every accumulator
// in ordinary VGPRs (no copies through the accumulation registers per tile).
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdParams p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = 32 * D;
    __shared__ __attribute__((aligned(16))) bf16 kt[2 * TILE];
    __shared__ __attribute__((aligned(16))) bf16 vt[2 * TILE];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int hi = l >> 5;
    const int nqb = (p.Lq + 127) / 128;
    const int nbh = p.B * p.Hq;
    int rank, bh;                               // bh = b * Hq + h
    if ((nbh & 7) == 0) {                       // XCD x gets heads [x nbh / 8, (x + 1) nbh / 8)
        const int per = nbh >> 3, slot = blockIdx.x >> 3;
        rank = slot / per;
        bh = (blockIdx.x & 7) * per + (slot - rank * per);
    } else {
        rank = blockIdx.x / nbh;
        bh = blockIdx.x - rank * nbh;
    }
    const int qb = nqb - 1 - rank;              // last query blocks first
    const int h = bh % p.Hq;
    const int b = bh / p.Hq;
    const int g = h / p.r;
    const int n = clamp_len(p.kv_lens, b, p.Lk);
    const int off = n - p.Lq;                   // query i sits at key position i + off
    const int qw0 = qb * 128;                   // first query of the workgroup
    const int qrow = qw0 + 32 * w + (l & 31);
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

    // Keys some query of the workgroup can see: [k_lo, k_hi).
    int k_hi = n, k_lo = 0;
    if (p.causal) k_hi = min(n, max(min(qw0 + 128, p.Lq) + off, 0));
    if (p.window > 0) k_lo = max(qw0 + off - p.window + 1, 0);
    const int t_lo = k_lo / 32;
    const int ntiles = max((k_hi + 31) / 32 - t_lo, 0);

    TileCopy<D> cp;
    cp.init(w, l);
    const uint32_t lds_k = lds_address(kt), lds_v = lds_address(vt);
    auto issue = [&](int j, auto stage) __attribute__((always_inline)) {   // tile j into stage j % 2
        const int k0 = (t_lo + j) * 32;
        constexpr int buf = decltype(stage)::value * TILE * 2;
        cp.issue(p.k + kvoff + (size_t)k0 * D, n - k0, lds_k + buf, w);
        cp.issue(p.v + kvoff + (size_t)k0 * D, n - k0, lds_v + buf, w);
    };

    const int krow = swap_bits_2_3(l & 31);
    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero_f32x16();
    const float c2 = p.c;

    // Tile j runs with j % 2 as a compile-time constant, so every LDS address
    // is a per-lane base plus an immediate offset.
    auto tile = [&](const int j, auto stage) __attribute__((always_inline)) {
        constexpr int stg = decltype(stage)::value;
        wait_all_vector_loads();                // this wavefront's copies of tile j
        __syncthreads();                        // tile j visible; every wavefront is done with tile j - 1
        if (j + 1 < ntiles) issue(j + 1, BwdStage<1 - stg>{});   // into the stage of tile j - 1
        const int k0 = (t_lo + j) * 32;
        const bf16* Ks = kt + stg * TILE;
        const bf16* Vs = vt + stg * TILE;

        // S^T (even steps) and dP^T (odd steps), pipelined over their K and V
        // fragments.
        constexpr int NOP = 2 * KS;
        bf16x8 fr[NOP];
        auto rd = [&](int i) __attribute__((always_inline)) {
            fr[i] = read_row_chunk<D>((i & 1) ? Vs : Ks, krow, 2 * (i / 2) + hi);
        };
        f32x16 s = zero_f32x16(), dp = zero_f32x16();
        // Products at raised priority: of the two wavefronts on a SIMD (from
        // different workgroups), the one with matrix work to issue goes first
        // and the other fills the gaps with its elementwise step.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < kAhead; ++i) rd(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NOP; ++i) {
            if (i & 1) dp = mfma_32x32x16(fr[i], gf[i / 2], dp);
            else       s = mfma_32x32x16(fr[i], qf[i / 2], s);
            if (i + kAhead < NOP) rd(i + kAhead);
            __builtin_amdgcn_sched_barrier(0);
        }
        // K^T fragments of the dQ product, read now so that the elementwise
        // step below covers their latency.
        bf16x8 kT[2 * DB];
#pragma unroll
        for (int f = 0; f < 2 * DB; ++f) kT[f] = read_transposed<D>(Ks, 16 * (f & 1), 32 * (f >> 1), l);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        // Elementwise masks only on tiles where some pair of this
        // wavefront's rows and the tile is out (a wave-uniform test).
        const int qw = qw0 + 32 * w;            // first query of this wavefront
        const bool need = (k0 + 32 > n) || (qw + 32 > p.Lq) ||
                          (p.causal && k0 + 31 > qw + off) ||
                          (p.window > 0 && qw + 31 + off - k0 >= p.window);
        float x[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v] = __builtin_fmaf(s[v], c2, -lse2);
        if (need) {
            // Element v holds key base + idx with idx a compile-time constant:
            // key < n and (causal) key <= qpos give idx <= lim, (window)
            // qpos - key < w gives idx >= lo; a row past Lq has lim = -1.
            const int base = k0 + 8 * hi;
            const int lim = row_ok ? (p.causal ? min(n - 1, qpos) : n - 1) - base : -1;
            if (p.window > 0) {
                const int lo = qpos - p.window + 1 - base;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int idx = 16 * (v >> 3) + (v & 7);
                    x[v] = (idx <= lim) & (idx >= lo) ? x[v] : kNegInf;   // 2^-inf = 0
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int idx = 16 * (v >> 3) + (v & 7);
                    x[v] = idx <= lim ? x[v] : kNegInf;
                }
            }
        }
        float ds[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) ds[v] = exp2_fast(x[v]) * (dp[v] - delta);
        const bf16x8 dsb0 = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
        const bf16x8 dsb1 = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            dq[db] = mfma_32x32x16(kT[2 * db], dsb0, dq[db]);
            dq[db] = mfma_32x32x16(kT[2 * db + 1], dsb1, dq[db]);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    if (ntiles > 0) issue(0, BwdStage<0>{});
    for (int j = 0; j < ntiles; j += 2) {
        tile(j, BwdStage<0>{});
        if (j + 1 < ntiles) tile(j + 1, BwdStage<1>{});
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

// D = 64: four wavefronts, each accumulating both dK and dV of its 32 keys
// (two wavefronts per SIMD fit with every accumulator in ordinary VGPRs).
// D = 128, where dK and dV of 32 keys alone would take 128 registers, runs
// bwd_dkdv_split_kernel below.
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdParams p) {
    static_assert(D == 64, "D = 128 runs bwd_dkdv_split_kernel");
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = 32 * D;
    constexpr int NT = 256;
    __shared__ __attribute__((aligned(16))) bf16 qt[2 * TILE];
    __shared__ __attribute__((aligned(16))) bf16 gt[2 * TILE];
    __shared__ __attribute__((aligned(16))) float stat[2 * 64];   // per stage: L2 [0, 32), delta [32, 64)
    __shared__ __attribute__((aligned(16))) bf16 kvres[4 * 2 * TILE];  // K and V of the four key blocks

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int hi = l >> 5;
    const int kblk = w & 3;                     // this wavefront's 32-key block
    const int nbg = p.B * p.Hkv;
    const int kb = blockIdx.x / nbg;            // first key blocks first
    const int bg = blockIdx.x - kb * nbg;       // b * Hkv + g; on XCD bg % 8 when nbg % 8 == 0
    const int g = bg % p.Hkv;
    const int b = bg / p.Hkv;
    const int n = clamp_len(p.kv_lens, b, p.Lk);
    const int off = n - p.Lq;
    const int kw0 = kb * 128;                   // first key of the workgroup
    const int k0 = kw0 + 32 * kblk;             // first key of this wavefront
    const int key = k0 + (l & 31);              // this lane's key (accumulator column of S, dP)
    const size_t kvoff = (size_t)bg * p.Lk * D;

    f32x16 acc[DB], acc2[DB];                   // dV, dK
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();
#pragma unroll
    for (int db = 0; db < DB; ++db) acc2[db] = zero_f32x16();

    // K and V of each key block (keys past n read as zero) in LDS, read as B
    // operands: lane l takes row l % 32, chunk 2 ks + hi.
    bf16* Kw = kvres + kblk * 2 * TILE;
    bf16* Vw = Kw + TILE;
    {
        const rsrc_t kbuf = make_rsrc(p.k + kvoff, (uint32_t)n * D * 2);
        const rsrc_t vbuf = make_rsrc(p.v + kvoff, (uint32_t)n * D * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint32_t at = (uint32_t)(key * D + ks * 16 + hi * 8) * 2;
            const int row = l & 31, chunk = 2 * ks + hi;
            const int slot = row * D + ((chunk ^ bwd_swizzle<D>(row)) * 8);
            *reinterpret_cast<bf16x8*>(Kw + slot) = load16(kbuf, at);
            *reinterpret_cast<bf16x8*>(Vw + slot) = load16(vbuf, at);
        }
    }

    // Query tiles in which some query can see a key of the workgroup:
    // position >= kw0 (causal), position < kw0 + 127 + window (window); as one
    // flat sequence f = hh * nqt + j over the query heads of this KV head.
    int i_lo = 0, i_hi = p.Lq;
    if (p.causal) i_lo = max(kw0 - off, 0);
    if (p.window > 0) i_hi = min(p.Lq, max(kw0 + 127 + p.window - off, 0));
    const int q_first = (i_lo / 32) * 32;
    const int nqt = (kw0 < n && i_hi > q_first) ? (i_hi - q_first + 31) / 32 : 0;
    const int total = p.r * nqt;

    TileCopy<D, NT> cp;
    cp.init(w, l);
    const uint32_t lds_q = lds_address(qt), lds_g = lds_address(gt);
    float st_next = 0.0f;                       // wavefront 0: L2 (lanes < 32) or delta of a query
    // Tiles are copied and used in order f = 0, 1, 2, ...: tile f is query
    // tile f % nqt of query head f / nqt.  Running counters (scalar adds)
    // stand in for a division per tile on the CU's shared scalar unit.
    const int head_skip = p.Lq - nqt * 32;      // rows from one head's last tile end to the next head's first tile
    int cp_qi = 0;                              // next tile to copy: tile index within its head
    long long cp_row = ((long long)b * p.Hq + g * p.r) * p.Lq + q_first;   // ... and its first row, all heads
    auto issue = [&](auto stage) __attribute__((always_inline)) {   // the next tile into LDS stage `stage`
        const int q0 = q_first + cp_qi * 32;
        constexpr int buf = decltype(stage)::value * TILE * 2;
        cp.issue(p.q + cp_row * D, p.Lq - q0, lds_q + buf, w);
        cp.issue(p.dout + cp_row * D, p.Lq - q0, lds_g + buf, w);
        if (w == 0) {
            const int i = q0 + (l & 31);
            float val = 0.0f;
            if (i < p.Lq) {
                if (l < 32) {
                    const float L = p.lse[cp_row + (l & 31)];
                    val = L == kNegInf ? 0.0f : L * kLog2e;
                } else {
                    val = p.delta[cp_row + (l & 31)];
                }
            }
            st_next = val;
        }
        cp_row += 32;
        if (++cp_qi == nqt) { cp_qi = 0; cp_row += head_skip; }
    };
    int use_qi = 0;                             // tile index within its head of the tile in use

    const int qrow = swap_bits_2_3(l & 31);   // A-operand row of this lane
    const float c2 = p.c;
    // Tile f runs with f % 2 as a compile-time constant, so every LDS address
    // is a per-lane base plus an immediate offset.
    auto tile = [&](const int f, auto stage) __attribute__((always_inline)) {
        constexpr int stg = decltype(stage)::value;
        wait_all_vector_loads();                // this wavefront's copies of tile f
        if (w == 0) stat[stg * 64 + l] = st_next;
        __syncthreads();                        // tile f visible; every wavefront is done with tile f - 1
        if (f + 1 < total) issue(BwdStage<1 - stg>{});   // into the stage of tile f - 1
        const int q0 = q_first + use_qi * 32;
        if (++use_qi == nqt) use_qi = 0;
        if (k0 >= n) return;                    // this wavefront's keys are all past n
        const bf16* Qs = qt + stg * TILE;
        const bf16* Gs = gt + stg * TILE;
        const float* St = stat + stg * 64;

        // Elementwise masks only on tiles where some pair is out (wave-uniform).
        const bool need = (q0 + 32 > p.Lq) || (k0 + 32 > n) || (p.causal && k0 + 31 > q0 + off) ||
                          (p.window > 0 && q0 + 31 + off - k0 >= p.window);
        // One tile: S and dP (interleaved), P, dV += P^T G, dS, dK += dS^T Q.
        {
            constexpr int NOP = 2 * KS;         // S on even steps, dP on odd ones
            bf16x8 fa[NOP], fb[NOP];
            auto rd = [&](int i) __attribute__((always_inline)) {
                const bool is_dp = (i & 1) != 0;
                const int ks = i / 2;
                fa[i] = read_row_chunk<D>(is_dp ? Gs : Qs, qrow, 2 * ks + hi);
                fb[i] = read_row_chunk<D>(is_dp ? Vw : Kw, l & 31, 2 * ks + hi);
            };
            f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
            for (int i = 0; i < kAhead; ++i) rd(i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NOP; ++i) {
                if (i & 1) dp = mfma_32x32x16(fa[i], fb[i], dp);
                else       s = mfma_32x32x16(fa[i], fb[i], s);
                if (i + kAhead < NOP) rd(i + kAhead);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Transposed G (dV) and Q (dK) fragments, read now so that the
            // elementwise step covers their latency.
            bf16x8 gT[2 * DB], qT[2 * DB];
#pragma unroll
            for (int f = 0; f < 2 * DB; ++f) {
                gT[f] = read_transposed<D>(Gs, 16 * (f & 1), 32 * (f >> 1), l);
                qT[f] = read_transposed<D>(Qs, 16 * (f & 1), 32 * (f >> 1), l);
            }
            __builtin_amdgcn_sched_barrier(0);
            // Entry v of this lane holds query q0 + 16*(v/8) + 8*hi + (v%8):
            // its L2 and delta are St[8 hi + (v%8) (+16 for v >= 8)] and
            // St[32 + ...].
            float x[16];
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int qd = 0; qd < 2; ++qd) {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(St + 16 * half + 8 * hi + 4 * qd);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = 8 * half + 4 * qd + e;
                        x[v] = __builtin_fmaf(s[v], c2, -a[e]);
                    }
                }
            if (need) {
                // Element v holds query base + idx (idx a compile-time
                // constant): one range [lo, hi_lim] of idx per lane.
                int lo, hi_lim;
                query_range(q0 + 8 * hi, key, n, off, p, lo, hi_lim);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int idx = 16 * (v >> 3) + (v & 7);
                    x[v] = (idx >= lo) & (idx <= hi_lim) ? x[v] : kNegInf;   // 2^-inf = 0
                }
            }
            float pr[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) pr[v] = exp2_fast(x[v]);
            const bf16x8 pb0 = to_bf16x8(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
            const bf16x8 pb1 = to_bf16x8(pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc[db] = mfma_32x32x16(pb0, gT[2 * db], acc[db]);
                acc[db] = mfma_32x32x16(pb1, gT[2 * db + 1], acc[db]);
            }
            float ds[16];
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int qd = 0; qd < 2; ++qd) {
                    const f32x4 d = *reinterpret_cast<const f32x4*>(St + 32 + 16 * half + 8 * hi + 4 * qd);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = 8 * half + 4 * qd + e;
                        ds[v] = pr[v] * (dp[v] - d[e]);
                    }
                }
            const bf16x8 db0 = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
            const bf16x8 db1 = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc2[db] = mfma_32x32x16(db0, qT[2 * db], acc2[db]);
                acc2[db] = mfma_32x32x16(db1, qT[2 * db + 1], acc2[db]);
            }
        }
    };
    if (total > 0) issue(BwdStage<0>{});
    for (int f = 0; f < total; f += 2) {
        tile(f, BwdStage<0>{});
        if (f + 1 < total) tile(f + 1, BwdStage<1>{});
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
                dkp[db * 32] = (bf16)(acc2[db][v] * p.scale);
                dvp[db * 32] = (bf16)acc[db][v];
            }
        }
    }
}


// D = 128, role-split and pipelined over the query tiles.  Wavefront w owns
// key block w % 4; w < 4 accumulates dV, w >= 4 dK, each with its own B
// operand rows (K or V of its 32 keys) in registers.  The dV wavefront forms
// P one tile ahead and hands it to the dK wavefront through a double buffer
// in LDS, so within a tile the two roles run independently:
//   dV role, tile t:  dV += P(t)^T G(t);  S(t+1) = Q(t+1) K^T;  P(t+1) -> LDS
//   dK role, tile t:  dP(t) = G(t) V^T;  dS = P(t) (dP - delta);  dK += dS^T Q(t)
// and each SIMD (one wavefront of each role) overlaps one role's products
// with the other's vector work.  Q and G tiles stream through three LDS
// stages (tiles t and t+1 are read in step t), copied two steps ahead by the
// dV wavefronts; one workgroup barrier per tile.
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_split_kernel(BwdParams p) {
    constexpr int D = 128;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int TILE = 32 * D;
    constexpr int NSTG = 3;
    __shared__ __attribute__((aligned(16))) bf16 qt[NSTG * TILE];
    __shared__ __attribute__((aligned(16))) bf16 gt[NSTG * TILE];
    __shared__ __attribute__((aligned(16))) float stat[NSTG * 64];   // per stage: L2 [0, 32), delta [32, 64)
    // P of tile t, key block kb, entry chunk c of lane l at (((t % 2) 4 + kb) 4 + c) 64 + l (f32x4).
    __shared__ __attribute__((aligned(16))) float pshare[2 * 4 * 16 * 64];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int hi = l >> 5;
    const int kblk = w & 3;
    const bool role_dv = w < 4;
    const int nbg = p.B * p.Hkv;
    const int kb = blockIdx.x / nbg;            // first key blocks first
    const int bg = blockIdx.x - kb * nbg;       // b * Hkv + g; on XCD bg % 8 when nbg % 8 == 0
    const int g = bg % p.Hkv;
    const int b = bg / p.Hkv;
    const int n = clamp_len(p.kv_lens, b, p.Lk);
    const int off = n - p.Lq;
    const int kw0 = kb * 128;
    const int k0 = kw0 + 32 * kblk;
    const int key = k0 + (l & 31);
    const bool active = k0 < n;                 // some key of this wavefront is valid
    const size_t kvoff = (size_t)bg * p.Lk * D;

    // This wavefront's K (dV role) or V (dK role) rows as B operands: lane l
    // takes key row l % 32, elements 16 ks + 8 hi .. +7 (zeros past n).
    bf16x8 kvf[KS];
    {
        const rsrc_t buf = make_rsrc((role_dv ? p.k : p.v) + kvoff, (uint32_t)n * D * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kvf[ks] = load16(buf, (uint32_t)(key * D + ks * 16 + hi * 8) * 2);
    }
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero_f32x16();

    int i_lo = 0, i_hi = p.Lq;
    if (p.causal) i_lo = max(kw0 - off, 0);
    if (p.window > 0) i_hi = min(p.Lq, max(kw0 + 127 + p.window - off, 0));
    const int q_first = (i_lo / 32) * 32;
    const int nqt = (kw0 < n && i_hi > q_first) ? (i_hi - q_first + 31) / 32 : 0;
    const int total = p.r * nqt;

    // Only the dK wavefronts copy (two 16-byte copies per lane per tile):
    // the dV wavefront's step (its products, then S and P of the next tile)
    // is the longer one, and copies issued by all eight wavefronts right after
    // the barrier queue behind each other.  Wavefront 4 also loads the rows'
    // statistics.
    const bool copier = !role_dv;
    constexpr int kStatWave = 4;
    TileCopy<D, 256> cp;
    cp.init(w & 3, l);
    const uint32_t lds_q = lds_address(qt), lds_g = lds_address(gt);
    float st_next = 0.0f;                       // wavefront 4: L2 (lanes < 32) or delta of a query
    // Tiles are copied, and P formed, in order f = 0, 1, 2, ...: tile f is
    // query tile f % nqt of query head f / nqt.  Running counters give the
    // tile's first query and row index with scalar adds; a division per tile,
    // in every wavefront right after the barrier, kept the CU's scalar unit
    // busy for hundreds of cycles.
    const int head_skip = p.Lq - nqt * 32;      // rows from one head's last tile end to the next head's first tile
    int cp_qi = 0;                              // next tile to copy: tile index within its head
    long long cp_row = ((long long)b * p.Hq + g * p.r) * p.Lq + q_first;   // ... and its first row, all heads
    // Step f of the loop below runs with f % 6 as a compile-time constant
    // (the LDS stage f % 3 and the P buffer f % 2), so every LDS address is a
    // per-lane base plus an immediate offset: no address arithmetic per step.
    auto issue = [&](auto stage) __attribute__((always_inline)) {   // the next tile into LDS stage `stage` (dK role only)
        const int q0 = q_first + cp_qi * 32;
        constexpr int buf = (decltype(stage)::value % NSTG) * TILE * 2;
        cp.issue(p.q + cp_row * D, p.Lq - q0, lds_q + buf, w & 3);
        cp.issue(p.dout + cp_row * D, p.Lq - q0, lds_g + buf, w & 3);
        if (w == kStatWave) {
            const int i = q0 + (l & 31);
            float val = 0.0f;
            if (i < p.Lq) {
                if (l < 32) {
                    const float L = p.lse[cp_row + (l & 31)];
                    val = L == kNegInf ? 0.0f : L * kLog2e;
                } else {
                    val = p.delta[cp_row + (l & 31)];
                }
            }
            st_next = val;
        }
        cp_row += 32;
        if (++cp_qi == nqt) { cp_qi = 0; cp_row += head_skip; }
    };
    int p_qi = 0;                               // dV role: tile index within its head of the next P formed

    const int qrow = swap_bits_2_3(l & 31);   // A-operand row of this lane
    const float c2 = p.c;
    bf16x8 pb0 = zero_bf16x8(), pb1 = zero_bf16x8();   // dV role: P of the current tile, as the A operand

    // A 32 x 32 product over D with A rows from an LDS tile and B from kvf.
    auto product = [&](const bf16* tile) __attribute__((always_inline)) {
        bf16x8 fa[KS];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) fa[i] = read_row_chunk<D>(tile, qrow, 2 * i + hi);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 r = zero_f32x16();
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            r = mfma_32x32x16(fa[i], kvf[i], r);
            if (i + kAhead < KS) fa[i + kAhead] = read_row_chunk<D>(tile, qrow, 2 * (i + kAhead) + hi);
            __builtin_amdgcn_sched_barrier(0);
        }
        return r;
    };
    // dV role: P of tile f (scores of its Q tile against K), masked where
    // needed, handed over through LDS and kept as the bf16 A operand.
    auto form_p = [&](auto stage) __attribute__((always_inline)) {   // P of the tile of step `stage` (mod 6)
        constexpr int stg = decltype(stage)::value % NSTG;
        constexpr int pbf = decltype(stage)::value & 1;
        const int q0 = q_first + p_qi * 32;
        if (++p_qi == nqt) p_qi = 0;
        const f32x16 s = product(qt + stg * TILE);
        const float* St = stat + stg * 64;
        float pr[16];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int qd = 0; qd < 2; ++qd) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(St + 16 * half + 8 * hi + 4 * qd);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 8 * half + 4 * qd + e;
                    pr[v] = __builtin_fmaf(s[v], c2, -a[e]);
                }
            }
        const bool need = (q0 + 32 > p.Lq) || (k0 + 32 > n) || (p.causal && k0 + 31 > q0 + off) ||
                          (p.window > 0 && q0 + 31 + off - k0 >= p.window);
        if (need) {
            int lo, hi_lim;                     // as in the D = 64 kernel
            query_range(q0 + 8 * hi, key, n, off, p, lo, hi_lim);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int idx = 16 * (v >> 3) + (v & 7);
                pr[v] = (idx >= lo) & (idx <= hi_lim) ? pr[v] : kNegInf;   // 2^-inf = 0
            }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) pr[v] = exp2_fast(pr[v]);
        f32x4* pbuf = reinterpret_cast<f32x4*>(pshare) + (pbf * 4 + kblk) * 4 * 64 + l;
#pragma unroll
        for (int c = 0; c < 4; ++c) pbuf[c * 64] = f32x4{pr[4 * c], pr[4 * c + 1], pr[4 * c + 2], pr[4 * c + 3]};
        pb0 = to_bf16x8(pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]);
        pb1 = to_bf16x8(pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]);
    };

    // ---- prologue: tiles 0 and 1 on their way, P(0) ------------------------
    // dV role: G(f)^T fragments of the next dV product, read at the end of
    // the previous step (tile f is visible from step f - 1 on), so their LDS
    // latency passes during the barrier.
    bf16x8 gT[2 * DB];
    auto read_gT = [&](auto stage) __attribute__((always_inline)) {
        const bf16* Gs = gt + (decltype(stage)::value % NSTG) * TILE;
#pragma unroll
        for (int j = 0; j < 2 * DB; ++j) gT[j] = read_transposed<D>(Gs, 16 * (j & 1), 32 * (j >> 1), l);
    };
    if (copier && total > 0) issue(BwdStage<0>{});
    wait_all_vector_loads();                    // tile 0, its statistics, this wavefront's K / V rows
    if (w == kStatWave) stat[l] = st_next;
    if (copier && total > 1) issue(BwdStage<1>{});
    __syncthreads();                            // tile 0 visible
    if (role_dv && active && total > 0) {
        form_p(BwdStage<0>{});
        read_gT(BwdStage<0>{});
    }

    // One step, in the two roles' own loops (so each role's registers are live
    // only in its own loop); both loops take one workgroup barrier per step.
    auto step = [&](const int f, auto stage, auto role) __attribute__((always_inline)) {
        constexpr int S6 = decltype(stage)::value;   // f % 6
        constexpr int stg = S6 % NSTG;
        constexpr int pbf = S6 & 1;
        wait_all_vector_loads();                // this wavefront's copies of tile f + 1
        if (decltype(role)::value == 1 && w == kStatWave && f + 1 < total) stat[((S6 + 1) % NSTG) * 64 + l] = st_next;
        __syncthreads();                        // tile f + 1 and P(f) visible; step f - 1 done everywhere
        if (decltype(role)::value == 1 && f + 2 < total) issue(BwdStage<(S6 + 2) % 6>{});   // into the stage of tile f - 1
        if (!active) return;
        const bf16* Qs = qt + stg * TILE;
        const bf16* Gs = gt + stg * TILE;
        (void)Qs; (void)Gs;
        if constexpr (decltype(role)::value == 0) {
            // dV += P(f)^T G(f), then P(f + 1) and the G(f + 1)^T fragments.
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc[db] = mfma_32x32x16(pb0, gT[2 * db], acc[db]);
                acc[db] = mfma_32x32x16(pb1, gT[2 * db + 1], acc[db]);
            }
            if (f + 1 < total) {
                form_p(BwdStage<(S6 + 1) % 6>{});
                read_gT(BwdStage<(S6 + 1) % 6>{});
            }
        } else {
            // dP(f), dS = P(f) (dP - delta), dK += dS^T Q(f).
            const f32x16 dp = product(Gs);
            bf16x8 qT[2 * DB];
#pragma unroll
            for (int j = 0; j < 2 * DB; ++j) qT[j] = read_transposed<D>(Qs, 16 * (j & 1), 32 * (j >> 1), l);
            const f32x4* pbuf = reinterpret_cast<const f32x4*>(pshare) + (pbf * 4 + kblk) * 4 * 64 + l;
            const float* St = stat + stg * 64;
            float ds[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 pv = pbuf[c * 64];
                const int half = c >> 1, qd = c & 1;
                const f32x4 d = *reinterpret_cast<const f32x4*>(St + 32 + 16 * half + 8 * hi + 4 * qd);
#pragma unroll
                for (int e = 0; e < 4; ++e) ds[4 * c + e] = pv[e] * (dp[4 * c + e] - d[e]);
            }
            const bf16x8 db0 = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
            const bf16x8 db1 = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc[db] = mfma_32x32x16(db0, qT[2 * db], acc[db]);
                acc[db] = mfma_32x32x16(db1, qT[2 * db + 1], acc[db]);
            }
        }
    };
    auto run_role = [&](auto role) __attribute__((always_inline)) {
        for (int f = 0; f < total; f += 6) {
            step(f, BwdStage<0>{}, role);
            if (f + 1 < total) step(f + 1, BwdStage<1>{}, role);
            if (f + 2 < total) step(f + 2, BwdStage<2>{}, role);
            if (f + 3 < total) step(f + 3, BwdStage<3>{}, role);
            if (f + 4 < total) step(f + 4, BwdStage<4>{}, role);
            if (f + 5 < total) step(f + 5, BwdStage<5>{}, role);
        }
    };
    if (role_dv) run_role(BwdStage<0>{});
    else         run_role(BwdStage<1>{});

    // Accumulator entry v of lane l: key k0 + 8*(v/4) + 4*hi + (v%4), column
    // 32*db + (l % 32).  Keys past n hold zeros.
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int kr = k0 + 8 * (v >> 2) + 4 * hi + (v & 3);
        if (kr < p.Lk) {
            bf16* out = (role_dv ? p.dv : p.dk) + kvoff + (size_t)kr * D + (l & 31);
            const float sc = role_dv ? 1.0f : p.scale;
#pragma unroll
            for (int db = 0; db < DB; ++db) out[db * 32] = (bf16)(acc[db][v] * sc);
        }
    }
}

hipError_t launch_backward(int D, const BwdParams& p, hipStream_t stream) {
    const long long nq = (long long)p.B * p.Hq * ((p.Lq + 127) / 128);
    const long long nk = (long long)p.B * p.Hkv * ((p.Lk + 127) / 128);
    if (D == 64) {
        hipLaunchKernelGGL((bwd_dq_kernel<64>), dim3((unsigned)nq), dim3(256), 0, stream, p);
        if (nk > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<64>), dim3((unsigned)nk), dim3(256), 0, stream, p);
    } else {
        hipLaunchKernelGGL((bwd_dq_kernel<128>), dim3((unsigned)nq), dim3(256), 0, stream, p);
        if (nk > 0) hipLaunchKernelGGL(bwd_dkdv_split_kernel, dim3((unsigned)nk), dim3(512), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
