// Host-side launch parameters shared by the API layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Query rows per prefill workgroup: four wavefronts of 64 rows, each
// workgroup sharing every K/V tile among them.
constexpr int kPrefillRows = 256;

// FP8 (E4M3) operands: one power-of-two scale per kFp8QBlock query rows and
// per kFp8KBlock keys of a head -- the prefill workgroup's query block and
// its KV tile.
constexpr int kFp8QBlock = kPrefillRows;
constexpr int kFp8KBlock = 64;

struct PrefillParams {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    __bf16* o;
    float* lse;            // may be null
    const int* kv_lens;    // may be null
    int B, Hq, Hkv, Lq, Lk;
    int r;                 // query heads per KV head
    int n_qblocks;         // ceil(Lq / kPrefillRows)
    int xcd_units;         // (B * Hkv) / 8 when divisible by 8, else 0
    int xcd_spread;        // 1: every XCD takes balanced pairs of query blocks of all heads (GQA)
    int window;            // causal window width (keys j with 0 <= pos_i - j < window); 0 = none
    float scale;           // softmax scale
    float c;               // scale * log2(e): scores enter exp2 as s * c
    // FP8 instantiation only: E4M3 codes of Q [B, Hq, Lq, D] and K [B, Hkv, Lk, D]
    // with their block scales [B, Hq, ceil(Lq / 256)] and [B, Hkv, ceil(Lk / 64)].
    const uint8_t* q8 = nullptr;
    const uint8_t* k8 = nullptr;
    const float* q_scale = nullptr;
    const float* k_scale = nullptr;
    // FP8 with Q quantized in the kernel: Q in bf16 (q) and the D sign flips
    // of the Hadamard transform (or null for none).
    const float* q_signs = nullptr;
    // Score modifiers (the modifier instantiations only): ALiBi slopes [Hq]
    // and the soft-cap of the scaled scores.
    const float* alibi_slopes = nullptr;
    float softcap = 0.0f;
    // Variable-length batches (the varlen instantiation only): B sequences
    // packed end to end, Lq and Lk then being the packed totals: Q and O
    // [Hq, Lq, D], K and V [Hkv, Lk, D], the LSE [Hq, Lq]; sequence b owns
    // query rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1.
    // schedule [2B + 1]: the sequences in longest-tile-first order, then the
    // running count of their query blocks in that order (B + 1 entries).
    const int* cu_q = nullptr;
    const int* cu_k = nullptr;
    const int* schedule = nullptr;
};

struct VarlenScheduleParams {
    const int* cu_q;       // [B + 1]
    const int* cu_k;       // [B + 1]
    int* schedule;         // [2B + 1]
    int B, total_q, total_k;
};

struct QuantParams {
    const __bf16* x;       // [heads, L, D]
    uint8_t* x8;           // [heads, L, D] E4M3 codes
    float* scales;         // [heads, nblk] powers of two
    const float* signs;    // D values +-1 (Hadamard with sign flips), or null
    int heads, L, block_rows, nblk;
};

struct SplitParams {
    const __bf16* q;
    const __bf16* k;       // contiguous [B, Hkv, Lk, D], or the paged cache [num_pages, Hkv, page_size, D]
    const __bf16* v;
    float* part_o;         // [B * Hq * Lq, num_splits, D] fp32, normalised partial outputs
    float* part_lse;       // [B * Hq * Lq, num_splits] fp32, base-2 log-sum-exp of each partial
    const int* kv_lens;
    int B, Hq, Hkv, Lq, Lk;
    int r;
    int rows;              // r * Lq packed rows per KV head
    int n_groups;          // ceil(rows / 32)
    int num_splits;        // partitions per sequence
    int chunk;             // keys per partition (multiple of 32)
    int causal;
    int window;            // causal window width, 0 = none (implies causal when > 0)
    // Paged cache (used by the paged instantiation only): logical token t of
    // sequence b lives in page page_table[b * max_pages + t / page_size], row
    // t % page_size.  Lk is the capacity max_pages * page_size.
    const int* page_table;
    int max_pages;
    int num_pages;
    int page_size;         // a multiple of 16
    float c;
};

struct CombineParams {
    const float* part_o;
    const float* part_lse;
    __bf16* o;
    float* lse;            // may be null
    const int* kv_lens;
    int B, Hq, Lq, Lk;
    int num_splits;
    int chunk;
};

struct BwdParams {
    const __bf16* q;       // [B, Hq, Lq, D]
    const __bf16* k;       // [B, Hkv, Lk, D]
    const __bf16* v;
    const __bf16* o;       // the forward's output [B, Hq, Lq, D]
    const __bf16* dout;    // dL/dO [B, Hq, Lq, D]
    const float* lse;      // the forward's natural-log LSE [B, Hq, Lq]
    float* delta;          // workspace [B, Hq, Lq]: rowsum(dO * O), written by the dq kernel
    __bf16* dq;            // [B, Hq, Lq, D]
    __bf16* dk;            // [B, Hkv, Lk, D]
    __bf16* dv;
    const int* kv_lens;    // may be null
    int B, Hq, Hkv, Lq, Lk;
    int r;                 // query heads per KV head
    int causal;
    int window;            // causal window width, 0 = none
    float scale;           // softmax scale c
    float c;               // scale * log2(e)
};

// Each launcher enqueues its kernel(s) on `stream` and returns the launch status.
hipError_t launch_prefill(int D, bool causal, const PrefillParams& p, hipStream_t stream);
// The prefill with E4M3 Q and K (D = 128): p.q8, p.k8 and the scales replace p.q and p.k.
hipError_t launch_prefill_fp8(int D, bool causal, const PrefillParams& p, hipStream_t stream,
                              bool quantize_q = false);
hipError_t launch_quantize_fp8(int D, const QuantParams& p, int cus, hipStream_t stream);
// The prefill with a score modifier: mod 1 = ALiBi (p.alibi_slopes), 2 = soft-cap (p.softcap).
hipError_t launch_prefill_mod(int D, bool causal, int mod, const PrefillParams& p, hipStream_t stream);
// Longest-tile-first order of a packed batch's sequences, then the prefill of
// the packed batch over `items` (an upper bound of its query blocks) work items.
hipError_t launch_varlen_schedule(const VarlenScheduleParams& p, hipStream_t stream);
hipError_t launch_prefill_varlen(int D, bool causal, const PrefillParams& p, int items, hipStream_t stream);
hipError_t launch_splitkv(int D, bool paged, const SplitParams& p, hipStream_t stream);
hipError_t launch_combine(int D, const CombineParams& p, hipStream_t stream);
// The dq kernel (which also writes delta) then the dk/dv kernel.
hipError_t launch_backward(int D, const BwdParams& p, hipStream_t stream);

}  // namespace fa
