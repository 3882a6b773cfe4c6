// Longest-tile-first order of the sequences of a packed variable-length batch.
//
// FlashAttention-4 summary, "LPT scheduling for imbalanced grids" (its fourth
// point): with variable lengths, the batches are sorted in a preprocessing
// kernel by their longest work tile, and the virtual-to-actual batch map is
// kept for the attention kernel.  Here a work tile is one query block of 256
// rows against its KV tiles of 64 keys.  A sequence's longest tile is its last
// query block, which sees every key with or without the causal rule (its last
// query sits at the sequence's last key position under the bottom-right
// alignment), so its cost is ceil(Lk_b / 64) tiles, and 0 for a sequence with
// no query.
//
// Thread b ranks sequence b among all B by (cost descending, index
// ascending) -- a total order, so the ranks form a permutation -- and sums the
// query blocks of the sequences ranked ahead of it.  It writes map[rank] = b
// and prefix[rank + 1] = that sum + its own query blocks; thread 0 writes
// prefix[0] = 0.  The costs are staged through LDS 256 at a time: O(B^2)
// comparisons spread over B threads, a few microseconds for batches of a few
// thousand sequences.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kScheduleThreads = 256;
constexpr int kQueryBlock = kPrefillRows;
constexpr int kKeyTile = 64;

__device__ __forceinline__ void sequence_cost(const VarlenScheduleParams& p, int b, int& cost, int& blocks) {
    int qs, lq, ks, lk;
    varlen_segment(p.cu_q, b, p.total_q, qs, lq);
    varlen_segment(p.cu_k, b, p.total_k, ks, lk);
    blocks = (lq + kQueryBlock - 1) / kQueryBlock;
    cost = blocks > 0 ? (lk + kKeyTile - 1) / kKeyTile : 0;
}

__global__ void __launch_bounds__(kScheduleThreads) varlen_schedule_kernel(VarlenScheduleParams p) {
    __shared__ int cost_s[kScheduleThreads];
    __shared__ int blocks_s[kScheduleThreads];
    const int t = threadIdx.x;
    const int b = blockIdx.x * kScheduleThreads + t;
    int cost = 0, blocks = 0;
    if (b < p.B) sequence_cost(p, b, cost, blocks);
    int rank = 0, ahead_blocks = 0;
    for (int c0 = 0; c0 < p.B; c0 += kScheduleThreads) {
        int cj = 0, bj = 0;
        if (c0 + t < p.B) sequence_cost(p, c0 + t, cj, bj);
        cost_s[t] = cj;
        blocks_s[t] = bj;
        __syncthreads();
        const int m = min(kScheduleThreads, p.B - c0);
        for (int i = 0; i < m; ++i) {
            const int ci = cost_s[i];
            const bool ahead = ci > cost || (ci == cost && c0 + i < b);
            rank += ahead ? 1 : 0;
            ahead_blocks += ahead ? blocks_s[i] : 0;
        }
        __syncthreads();
    }
    if (b < p.B) {
        p.schedule[rank] = b;
        p.schedule[p.B + 1 + rank] = ahead_blocks + blocks;
    }
    if (b == 0) p.schedule[p.B] = 0;
}

}  // namespace

hipError_t launch_varlen_schedule(const VarlenScheduleParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)((p.B + kScheduleThreads - 1) / kScheduleThreads)), block(kScheduleThreads);
    hipLaunchKernelGGL(varlen_schedule_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
