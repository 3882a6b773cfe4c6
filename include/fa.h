/*
 * fa.h - C ABI of the MI355X (gfx950) FlashAttention forward library (libfa.so).
 *
 * The operation (FlashAttention from Scratch, ryhuang.blog, section 2 "Begin
 * with one attention row"; FlashAttention Cheat Sheet, mxino.github.io,
 * section 1 "The whole operation"): for every batch b, query head h and query
 * row i,
 *
 *     O[b,h,i,:] = sum_j P_ij V[b,g,j,:],  P_ij = softmax_j(scale * Q[b,h,i,:] . K[b,g,j,:] + M_ij)
 *     LSE[b,h,i] = log sum_j exp(scale * Q[b,h,i,:] . K[b,g,j,:] + M_ij)   (natural log)
 *
 * with g = floor(h / (Hq / Hkv)) (grouped-query attention: FlashAttention
 * from Scratch, section 9.2) and M_ij in {0, -inf}.  The only masks are:
 *   - length: key j is valid iff j < n_b, where n_b = kv_lens[b] clamped to
 *     [0, Lk] (or Lk when kv_lens is NULL);
 *   - causal (optional): bottom-right alignment, query i sits at absolute
 *     position n_b - Lq + i and sees keys j <= that position (FlashAttention
 *     from Scratch, section 5, "Rectangular causal masking is a correctness
 *     issue").
 * A row with no allowed key returns O = 0 and LSE = -inf (same page, section
 * 4.4 "Handle the empty state deliberately").
 *
 * The result is computed tile by tile with the online-softmax recurrence
 * (running max, running sum, rescaled accumulator; same page, section 4.1;
 * Cheat Sheet, section 5) so the Lq x Lk score matrix never reaches HBM.
 * Both matrix products run on bf16 MFMA with fp32 accumulation.
 * Range: the results follow the definition while every score
 * scale * q.k (after any modifier) has magnitude below 2^27.  Scores are
 * held in fp32 in base-2 units, and the exponent of each term is formed as
 * one fused multiply-add against a rounded per-row reference; far past that
 * bound the reference's rounding error alone exceeds its headroom and a row
 * may come out as NaN.
 *
 * Memory layout and ownership (all entry points):
 *   q   : bf16, device, contiguous [B, Hq,  Lq, D]
 *   k, v: bf16, device, contiguous [B, Hkv, Lk, D]; Lk is the per-sequence
 *         row capacity (stride); only the first n_b rows of each sequence are
 *         read, rows >= n_b may hold anything (even NaN)
 *   o   : bf16, device, contiguous [B, Hq, Lq, D], written
 *   lse : fp32, device, contiguous [B, Hq, Lq], written; may be NULL
 *   kv_lens : int32, device, [B], or NULL
 *   stream  : a hipStream_t (NULL = the null stream)
 * q, k, v and o must be 16-byte aligned; lse and kv_lens 4-byte aligned.
 * The caller owns every buffer; the library keeps no pointer after return.
 * All work is enqueued on `stream`; the call returns without synchronising and
 * the outputs are valid once the stream has reached that point.
 *
 * Errors: arguments are validated on the host before any HIP call.  A failed
 * validation returns FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED and enqueues
 * nothing.  A HIP failure (launch, allocation) returns FA_ERR_HIP.
 * fa_last_error() describes the most recent failure on the calling thread.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, bad alignment, bad scale, Hq % Hkv != 0 */
    FA_ERR_UNSUPPORTED = 2,  /* valid but not implemented: D not in {64, 128} */
    FA_ERR_HIP = 3           /* a HIP runtime call or a kernel launch failed */
} fa_status;

/*
 * Attention forward.  Returns an fa_status.
 *   B, Hq, Hkv, Lq, D > 0; Lk >= 0; Hq % Hkv == 0; D in {64, 128};
 *   causal: 0 or 1; scale: finite and > 0 (the usual choice is 1/sqrt(D)).
 * Path choice: when Lq == 1 (single-token decode) the split-KV path runs
 * (Flash-Decoding, FlashAttention from Scratch section 9.1): the valid keys
 * of each sequence are cut into partitions, each partition's normalised
 * output and LSE go to a library-held workspace, and a second kernel merges
 * them by their LSEs (section 4.3).  Otherwise one workgroup per (batch,
 * query head, 256-row query block) runs the whole KV loop on chip.
 * The split-KV workspace is allocated by the library on first need per
 * device and grown (synchronously, with a device synchronisation) when a
 * larger one is needed; concurrent split-KV calls on different streams of
 * one device share it and must not overlap.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Lq, int Lk, int D,
           int causal, float scale, const int* kv_lens, void* stream);

/*
 * Same operation, forcing the split-KV path for any Lq with at most
 * num_splits partitions per sequence (num_splits >= 1).  Partition s covers
 * keys [s*C, (s+1)*C) of each sequence, C = 32 * ceil(ceil(Lk/32) / num_splits);
 * partitions past n_b are empty.  Any partition count gives the same exact
 * result (section 4.3); num_splits == 0 behaves exactly like fa_fwd.
 * Query heads that share a KV head are packed, with their query rows, into
 * the 32 columns of one matrix-core tile (section 9.2).
 */
int fa_fwd_splits(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Lq, int Lk, int D,
                  int causal, float scale, const int* kv_lens, void* stream,
                  int num_splits);

/*
 * fa_fwd_splits for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments, path choice and errors as fa_fwd_splits
 * (num_splits = 0: fa_fwd's choice), except that the split-KV workspace is a
 * static device array of fa_noalloc_scratch_bytes() bytes (16 MiB) inside the
 * library instead of a buffer the library allocates: this entry point calls no
 * hipMalloc or hipFree.  A call whose workspace
 * B * Hq * Lq * partitions * (D + 1) * 4 bytes exceeds the scratch returns
 * FA_ERR_INVALID_ARG (fa_last_error names the sizes) and enqueues nothing.
 * The prefill path (Lq > 1 without forced splits) needs no workspace.
 * Every call writes all of the scratch it reads, so nothing must start at
 * zero.  Each GPU holds its own copy of the scratch (looked up once per device
 * on first use), shared by every fa_fwd_noalloc call on that GPU: calls that
 * overlap on one GPU (other streams, other threads) race on it.
 */
int fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Lq, int Lk, int D,
                   int causal, float scale, const int* kv_lens, void* stream,
                   int num_splits);

/* Size in bytes of fa_fwd_noalloc's static split-KV scratch. */
size_t fa_noalloc_scratch_bytes(void);

/*
 * Causal attention restricted to a window (FlashAttention from Scratch,
 * section 12 "Programmable attention", a causal window of width w): query i,
 * at absolute position p_i = n_b - Lq + i, sees key j iff 0 <= p_i - j < w and
 * j < n_b.  (The page's formula is lost in extraction; w is read as the
 * number of keys a row sees once it is at least w positions in.)  window = 0
 * means no window, i.e. plain causal attention, the same as fa_fwd with
 * causal = 1; window < 0 is FA_ERR_INVALID_ARG.  Every other argument, the
 * layout and the path choice are those of fa_fwd_splits (num_splits = 0:
 * decode takes the split-KV path, longer query blocks the prefill kernel).
 * KV tiles wholly outside every row's window are never read; the split-KV
 * partitions cover only the window's span of each sequence.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Lq, int Lk, int D,
                  int window, float scale, const int* kv_lens, void* stream, int num_splits);

/*
 * Attention against a paged KV cache (FlashAttention from Scratch, section
 * 9.3 "Paging changes where keys live"): logical token t of sequence b lives
 * in physical page page_table[b * max_pages + t / page_size], at row
 * t % page_size of that page.  The result is that of fa_fwd over the logical
 * sequence (same masks, bottom-right causal alignment, GQA mapping, optional
 * causal window as in fa_fwd_window, window = 0 for none).
 *   k_cache, v_cache: bf16, device, contiguous [num_pages, Hkv, page_size, D]
 *                     (each page holds page_size consecutive tokens of every
 *                     KV head, one head's rows contiguous), 16-byte aligned;
 *   page_table: int32, device, [B, max_pages], 4-byte aligned; only the
 *               entries of pages that hold one of the first n_b tokens are
 *               read.  An entry outside [0, num_pages) is never dereferenced:
 *               its tokens count as masked (they keep their positions);
 *   kv_lens: int32, device, [B], required; n_b = kv_lens[b] clamped to
 *            [0, max_pages * page_size];
 *   page_size: a positive multiple of 16; max_pages, num_pages > 0;
 *   q, o, lse, scale, causal, D, B, Hq, Hkv, Lq, stream: as in fa_fwd.
 * Every Lq runs on the split-KV kernels (the paged loader lives there); the
 * automatic partition count (num_splits = 0) is fa_fwd's.  The library's
 * split-KV workspace is shared with fa_fwd (same rules).
 */
int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int D,
                 const int* page_table, int max_pages, int num_pages, int page_size,
                 const int* kv_lens, int causal, int window, float scale, void* stream,
                 int num_splits);

/*
 * Backward of the attention forward by recomputation (FlashAttention from
 * Scratch, section 8 "Backward: spend arithmetic to save memory"): given the
 * forward's inputs, its output o and natural-log lse (as written by fa_fwd or
 * fa_fwd_window with the same arguments), and dout = dL/dO, writes
 *     dq = dL/dQ [B, Hq, Lq, D], dk = dL/dK and dv = dL/dV [B, Hkv, Lk, D]
 * (bf16, device, contiguous, 16-byte aligned; every element is written: keys
 * at or past n_b and rows of no allowed pair get zero).  With c = scale:
 * P_ij = exp(c q_i.k_j - lse_i) on allowed pairs, dV = P^T dO, dP = dO V^T,
 * delta_i = dO_i . O_i, dS = P (dP - delta), dQ = c dS K, dK = c dS^T Q; the
 * gradients of a KV head sum over the Hq/Hkv query heads that read it.
 *   q, k, v, o, dout: bf16 device tensors in the layouts of fa_fwd;
 *   lse: fp32 [B, Hq, Lq] (required);
 *   causal, window, scale, kv_lens: the forward's (window = 0: none; a window
 *   needs causal = 1).
 * Two kernels run on `stream`: a query-owned one for dq (which also forms
 * delta into the library workspace, shared with the split-KV path and with
 * the same rules) and a KV-owned one for dk and dv.  No atomics: the result is
 * deterministic.  Errors as for fa_fwd.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int Lq, int Lk, int D,
           int causal, int window, float scale, const int* kv_lens, void* stream);

/*
 * Attention forward with a score modifier (FlashAttention from Scratch,
 * section 12 "Programmable attention": S'_ij = f(S_ij, i, j) before the
 * softmax; FlashAttention 1-4, FlashAttention-4 point 4 names ALiBi and
 * soft-capping).  fa_fwd's operation with S = scale * q.k replaced by
 *     ALiBi     (alibi_slopes != NULL): S - alibi_slopes[h] * |pos_i - pos_j|
 *     soft-cap  (softcap > 0):          softcap * tanh(S / softcap)
 * with the absolute positions of fa_fwd's causal alignment (query i at
 * n_b - Lq + i, key j at j); the masks act after the modifier.  At most one
 * modifier per call; with neither this is fa_fwd.
 *   alibi_slopes: fp32, device, [Hq] (one per query head), 4-byte aligned
 *   softcap: finite, >= 0 (0 = none)
 * Other arguments, layouts and errors as for fa_fwd (no window; every Lq
 * runs the prefill kernel).  FA_ERR_INVALID_ARG also for both modifiers at
 * once or a negative or non-finite softcap.
 */
int fa_fwd_mod(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, float scale,
               const int* kv_lens, const float* alibi_slopes, float softcap, void* stream);

/*
 * FP8 block quantization with optional incoherent processing (FlashAttention
 * from Scratch, section 10.3 "Treat FP8 as a second lesson"; FlashAttention
 * 1-4, FlashAttention-3 point 3: one FP8 scale per tile, and Q and K
 * multiplied by the same random orthogonal matrix -- a Hadamard transform with
 * random sign flips -- before quantizing).  For each of `heads` independent
 * [L, D] row sets of x and each block of `block_rows` consecutive rows:
 *     x'    = H (signs * x) per row when signs != NULL (H: the D x D Sylvester
 *             Hadamard matrix, entries +-1, unnormalised), else x; rounded to fp32
 *     scale = 2^k, the smallest power of two with max|x'| 2^-k <= 448
 *             (1 for an all-zero block)
 *     x8    = E4M3 code of x' / scale, rounded to nearest, ties to even (OCP
 *             FP8 E4M3: largest finite 448, subnormals to 2^-9)
 *   x      : bf16, device, contiguous [heads, L, D], 16-byte aligned
 *   x8     : uint8 E4M3 codes, device, [heads, L, D], 16-byte aligned, written
 *   scales : fp32, device, [heads, ceil(L / block_rows)], written
 *   signs  : fp32, device, D values each +1 or -1, 16-byte aligned, or NULL
 *            for no transform
 * Since H H^T = D I, scores from transformed Q and K are D times the
 * original: divide the softmax scale by D (fa_fwd_fp8 takes it as given).
 * The forward expects Q blocks of 256 rows and K blocks of 64 rows.
 * Errors: FA_ERR_INVALID_ARG (non-positive sizes, NULL or misaligned
 * buffers, a problem too large), FA_ERR_UNSUPPORTED (D not 64 or 128),
 * FA_ERR_HIP.
 */
int fa_quantize_fp8(const void* x, void* x8, float* scales, int heads, int L, int D,
                    int block_rows, const float* signs, void* stream);

/*
 * Attention forward with FP8 scores: fa_fwd's operation with
 *     S_ij = scale * (q8_i * sq) . (k8_j * sk)
 * where q8 and k8 hold E4M3 codes from fa_quantize_fp8, sq the scale of q8's
 * 256-row block and sk the scale of k8's 64-row block.  The score product runs
 * on the gfx950 FP8 matrix instruction with fp32 accumulation; the
 * probabilities and V stay bf16 (the PV product is fa_fwd's).
 *   q8 : uint8 [B, Hq, Lq, D] codes, with q_scales fp32 [B, Hq, ceil(Lq / 256)]
 *   k8 : uint8 [B, Hkv, Lk, D] codes, with k_scales fp32 [B, Hkv, ceil(Lk / 64)]
 *   v, o, lse, kv_lens, causal, stream: as for fa_fwd (no window)
 * D = 64 or 128 (FA_ERR_UNSUPPORTED otherwise); other errors as for fa_fwd.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v, void* o, float* lse,
               const float* q_scales, const float* k_scales,
               int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, float scale,
               const int* kv_lens, void* stream);

/*
 * fa_fwd_fp8 with Q quantized inside the attention kernel (FlashAttention
 * 1-4, FlashAttention-3 point 3; FlashAttention from Scratch, section 10.3):
 * the result is that of
 *     fa_quantize_fp8(q, q8, q_scales, B * Hq, Lq, D, 256, signs, stream);
 *     fa_fwd_fp8(q8, k8, v, o, lse, q_scales, k_scales, ...);
 * bit for bit, without the Q codes or scales reaching memory: each
 * workgroup's query block is exactly one 256-row scale block, so it
 * transforms, scales and encodes its own rows.  K is quantized beforehand
 * (its blocks are shared by many workgroups), with the same signs.  (Both
 * transforms sum in fp64, exactly for rows whose nonzero entries span at
 * most 2^38 in magnitude; the equality is stated for such rows.)
 *   q      : bf16, device, contiguous [B, Hq, Lq, D], 16-byte aligned
 *   signs  : fp32, device, D values +1 or -1 (the transform's sign flips, as
 *            given to fa_quantize_fp8 for K), 16-byte aligned, or NULL for no
 *            transform
 *   k8, k_scales, v, o, lse, kv_lens, causal, scale, stream: as for fa_fwd_fp8
 * D = 64 or 128 (FA_ERR_UNSUPPORTED otherwise); other errors as for fa_fwd_fp8.
 */
int fa_fwd_fp8_q(const void* q, const float* signs, const void* k8, const void* v, void* o, float* lse,
                 const float* k_scales, int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal,
                 float scale, const int* kv_lens, void* stream);

/*
 * Attention over a batch of variable-length sequences packed end to end
 * (FlashAttention from Scratch, section 11.5: variable-length batches are a
 * source of imbalance; section 12: packed sequences must not see each other).
 * Sequence b is fa_fwd's problem on its own rows: query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 against key rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1, Lq_b and Lk_b the differences,
 * with the causal rule bottom-right aligned per sequence (query i of the
 * sequence at key position Lk_b - Lq_b + i) and the GQA head mapping.
 *   q : bf16, device, contiguous [Hq, total_q, D]   (head-major, packed rows)
 *   k, v: bf16, device, contiguous [Hkv, total_k, D]
 *   o : bf16, device, contiguous [Hq, total_q, D], written on every row
 *       that belongs to a sequence
 *   lse : fp32, device, [Hq, total_q], written likewise; may be NULL
 *   cu_seqlens_q, cu_seqlens_k : int32, device, [B + 1], non-decreasing,
 *       from 0 to total_q / total_k.  Offsets are read on the device and
 *       clamped there (to [0, total] and to non-negative lengths), so any
 *       values keep every access inside the tensors; offsets that are not
 *       non-decreasing give undefined (but in-bounds) results.
 *   schedule : int32, device, [2B + 1] from fa_varlen_schedule over the same
 *       offsets, or NULL: then the library computes it first, on `stream`,
 *       into its workspace (allocated and shared as fa_fwd's split-KV
 *       workspace).  Any order of the sequences is accepted in the same
 *       layout (the sequence indices in the order to run them, then 0 and
 *       the running sum of their ceil(Lq_b / 256) query blocks): the result
 *       does not depend on the order, only the time does.  A schedule that
 *       does not match the offsets gives undefined (in-bounds) results.
 *   B in [1, 65536]; total_q, total_k >= 0 (total_q = 0: nothing is
 *   enqueued and the tensor pointers are not checked); Hq, Hkv > 0, Hq % Hkv == 0; D in {64, 128}; causal 0 or 1;
 *   scale finite and > 0.  q, k, v, o 16-byte aligned; lse, the offsets
 *   and the schedule 4-byte aligned.  Errors as for fa_fwd.
 * Work order (FlashAttention-4 summary, "LPT scheduling for imbalanced
 * grids"): the query blocks run sequence by sequence in the schedule's
 * longest-tile-first order, each sequence's last block first.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, const int* schedule,
                  int B, int Hq, int Hkv, int total_q, int total_k, int D,
                  int causal, float scale, void* stream);

/*
 * The longest-tile-first order of a packed batch's sequences (the
 * FlashAttention-4 summary's preprocessing sort for variable lengths, "LPT
 * scheduling for imbalanced grids"), for fa_fwd_varlen; computed on the
 * device, enqueued on `stream`, so it can be computed once per batch layout
 * and reused.  A sequence's cost is ceil(Lk_b / 64), the KV tiles of its
 * longest work tile (its last 256-row query block sees every key), or 0 if
 * Lq_b = 0.  Written: schedule[0 .. B-1] = the sequence indices by cost
 * descending, equal costs by index ascending; schedule[B .. 2B] = 0 followed
 * by the running sum of ceil(Lq_b / 256) in that order.  The order and the
 * blocks do not depend on the causal flag.
 *   cu_seqlens_q, cu_seqlens_k, B, total_q, total_k: as for fa_fwd_varlen;
 *   schedule: int32, device, [fa_varlen_schedule_ints(B)], 4-byte aligned,
 *   owned by the caller.  Errors as for fa_fwd_varlen.
 */
int fa_varlen_schedule(const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int total_q, int total_k,
                       int* schedule, void* stream);
/* Number of int32 entries of a schedule for B sequences (2B + 1; 0 for a B
 * outside [1, 65536]). */
size_t fa_varlen_schedule_ints(int B);

/* Bytes of split-KV workspace fa_fwd would use for this shape (0 when it
 * takes the prefill path, or for invalid sizes). */
size_t fa_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D);

/* Static text for a status code. */
const char* fa_status_string(int status);

/* Text describing the most recent failed call on this thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
