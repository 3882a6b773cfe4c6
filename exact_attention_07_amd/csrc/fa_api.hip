// C ABI of libfa: host-side validation, path choice, workspace and launches.
// The operation and the contract of every entry point are documented in
// include/fa.h.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "fa_internal.h"

// Split-KV scratch of fa_fwd_noalloc: one static array per device (each GPU the
// library runs on holds its own copy until the process ends).  In host code the
// name is only a stand-in; the device address comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// A launch's work-items (workgroups x threads per workgroup) must fit the 32
// bits of the dispatch packet's grid size.
bool grid_fits(long long workgroups, int threads) {
    return workgroups >= 0 && workgroups * threads <= (long long)UINT32_MAX;
}

constexpr int kTileKeys = 32;          // split-KV partitions are multiples of one 32-key tile
constexpr int kMaxDevices = 64;

struct Shape {
    int B, Hq, Hkv, Lq, Lk, D;
};

// Host-only argument checks shared by every entry point.
int validate_shape(const Shape& s) {
    if (s.B <= 0 || s.Hq <= 0 || s.Hkv <= 0 || s.Lq <= 0 || s.D <= 0 || s.Lk < 0)
        return fail(FA_ERR_INVALID_ARG, "sizes must be positive (Lk may be 0): B=%d Hq=%d Hkv=%d Lq=%d Lk=%d D=%d",
                    s.B, s.Hq, s.Hkv, s.Lq, s.Lk, s.D);
    if (s.Hq % s.Hkv != 0)
        return fail(FA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", s.Hq, s.Hkv);
    if (s.D != 64 && s.D != 128)
        return fail(FA_ERR_UNSUPPORTED, "head dimension D=%d is not supported (64 or 128)", s.D);
    const long long qrows = (long long)s.B * s.Hq * s.Lq;
    const long long kvrows = (long long)s.B * s.Hkv * s.Lk;
    // Per-head byte offsets (plus one tile of overshoot) must fit the 32-bit
    // offsets of the buffer loads; row counts must fit 32-bit indices.
    const long long head_bytes_q = ((long long)s.Lq + 256) * s.D * 2;
    const long long head_bytes_k = ((long long)s.Lk + 256) * s.D * 2;
    if (head_bytes_q > UINT32_MAX || head_bytes_k > UINT32_MAX || qrows > INT32_MAX || kvrows > INT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "problem too large for 32-bit per-head offsets");
    return FA_OK;
}

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const Shape& s, int causal, float scale, const int* kv_lens) {
    int st = validate_shape(s);
    if (st != FA_OK) return st;
    if (!q || !o) return fail(FA_ERR_INVALID_ARG, "q and o must not be NULL");
    if (s.Lk > 0 && (!k || !v)) return fail(FA_ERR_INVALID_ARG, "k and v must not be NULL when Lk > 0");
    if (!aligned(q, 16) || !aligned(o, 16) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)))
        return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if ((lse && !aligned(lse, 4)) || (kv_lens && !aligned(kv_lens, 4)))
        return fail(FA_ERR_INVALID_ARG, "lse and kv_lens must be 4-byte aligned");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!std::isfinite(scale) || !(scale > 0.0f))
        return fail(FA_ERR_INVALID_ARG, "scale must be finite and positive");
    return FA_OK;
}

// Optional parts of a call beyond the contiguous fa_fwd arguments.
struct Extra {
    int window = 0;                 // causal window width, 0 = none
    int requested_splits = 0;       // > 0 forces the split-KV path
    bool no_alloc = false;          // split-KV workspace from the static scratch, no allocation
    // paged cache (page_table != nullptr): Lk of the shape is the capacity
    const int* page_table = nullptr;
    int max_pages = 0, num_pages = 0, page_size = 0;
};

// Keys a sequence's rows can see at most: all Lk, or under a window the
// window's span for Lq queries plus the alignment of its start to a tile.
int visible_span(const Shape& s, int window) {
    if (window <= 0) return s.Lk;
    const long long span = (long long)window + s.Lq - 1 + (kTileKeys - 1);
    return span < s.Lk ? (int)span : s.Lk;
}

struct SplitPlan {
    int num_splits;  // partitions per sequence
    int chunk;       // keys per partition
    int n_groups;    // 32-row groups per KV head
};

int cu_count() {
    static int cached = 0;
    if (cached > 0) return cached;
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        cached = n;
    return cached > 0 ? cached : 256;
}

SplitPlan plan_splits(const Shape& s, int requested, int cus, int span) {
    SplitPlan pl;
    const int rows = (s.Hq / s.Hkv) * s.Lq;
    pl.n_groups = (rows + 31) / 32;
    const int tiles = (span + kTileKeys - 1) / kTileKeys;
    int want;
    if (requested > 0) {
        want = requested;
    } else {
        // The split kernel runs two wavefronts per SIMD, 8 per CU.  About 1.5
        // wavefronts per slot fills the GPU even when part of the partitions
        // of ragged sequences are empty, while keeping each wavefront's stream
        // long (its start-up latency is paid once) and the partials few.
        // Partitions stay at least 256 keys long.
        const long long units = (long long)s.B * s.Hkv * pl.n_groups;
        const long long slots = 8LL * cus;
        const long long by_fill = (3 * slots + 2 * units - 1) / (2 * units);
        const long long by_len = (span + 255) / 256;
        want = (int)(by_fill < by_len ? by_fill : by_len);
    }
    if (want > tiles) want = tiles;
    if (want < 1) want = 1;
    const int tiles_per = tiles > 0 ? (tiles + want - 1) / want : 1;
    pl.chunk = tiles_per * kTileKeys;
    pl.num_splits = span > 0 ? (span + pl.chunk - 1) / pl.chunk : 1;
    return pl;
}

size_t split_workspace_bytes(const Shape& s, const SplitPlan& pl) {
    const size_t rows = (size_t)s.B * s.Hq * s.Lq;
    return rows * pl.num_splits * ((size_t)s.D + 1) * sizeof(float);
}

// Workgroup placement of the prefill kernels over the eight XCDs (dispatched
// round-robin).  With grouped-query attention, the query heads of a KV head
// can differ widely in cost (a head whose scores spread widely may switch to
// split probabilities), so instead of whole KV heads per XCD, every XCD takes
// balanced pairs of query blocks (i, n - 1 - i) of all heads; the r query
// heads of a (KV head, block) stay adjacent, so they share K/V tiles in L2.
int xcd_spread(int r, int n_qblocks) { return (r > 1 && n_qblocks % 16 == 0) ? 1 : 0; }

bool use_split_path(const Shape& s, const Extra& x) {
    if (x.requested_splits > 0 || x.page_table) return true;
    return s.Lq == 1;
}

// Library-held split-KV workspace, one per device, grown on demand.
std::mutex g_ws_mutex;
void* g_ws_ptr[kMaxDevices] = {};
size_t g_ws_size[kMaxDevices] = {};

int get_workspace(size_t bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_HIP, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (g_ws_size[dev] < bytes) {
        if (g_ws_ptr[dev]) {
            e = hipDeviceSynchronize();   // earlier launches may still read the old buffer
            if (e != hipSuccess) return fail(FA_ERR_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
            (void)hipFree(g_ws_ptr[dev]);
            g_ws_ptr[dev] = nullptr;
            g_ws_size[dev] = 0;
        }
        void* p = nullptr;
        e = hipMalloc(&p, bytes);
        if (e != hipSuccess) return fail(FA_ERR_HIP, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
        g_ws_ptr[dev] = p;
        g_ws_size[dev] = bytes;
    }
    *out = g_ws_ptr[dev];
    return FA_OK;
}

// Device address of this device's copy of `scratch`, looked up once per device
// (with that device current) and kept; never the host-side name itself.
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_HIP, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

int validate_extra(const Shape& s, int causal, const int* kv_lens, const Extra& x) {
    if (x.requested_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0");
    if (x.window < 0) return fail(FA_ERR_INVALID_ARG, "window must be >= 0");
    if (x.window > 0 && !causal) return fail(FA_ERR_INVALID_ARG, "a window needs causal masking");
    if (x.page_table) {
        if (!kv_lens) return fail(FA_ERR_INVALID_ARG, "a paged cache needs kv_lens");
        if (!aligned(x.page_table, 4)) return fail(FA_ERR_INVALID_ARG, "page_table must be 4-byte aligned");
        if (x.page_size < 16 || x.page_size % 16 != 0)
            return fail(FA_ERR_INVALID_ARG, "page_size (%d) must be a positive multiple of 16", x.page_size);
        if (x.num_pages <= 0 || x.max_pages <= 0)
            return fail(FA_ERR_INVALID_ARG, "num_pages (%d) and max_pages (%d) must be positive",
                        x.num_pages, x.max_pages);
        const long long table = (long long)s.B * x.max_pages;
        const long long pool = (long long)x.num_pages * s.Hkv * x.page_size * s.D;
        if (table > INT32_MAX || pool > (1LL << 46))
            return fail(FA_ERR_INVALID_ARG, "page table or page pool too large");
    }
    return FA_OK;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, const Shape& s,
        int causal, float scale, const int* kv_lens, void* stream_ptr, const Extra& x) {
    int st = validate(q, k, v, o, lse, s, causal, scale, kv_lens);
    if (st != FA_OK) return st;
    st = validate_extra(s, causal, kv_lens, x);
    if (st != FA_OK) return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    const float c = scale * 1.4426950408889634f;  // scale * log2(e)
    const int r = s.Hq / s.Hkv;
    const auto* qb = static_cast<const __bf16*>(q);
    const auto* kb = static_cast<const __bf16*>(k);
    const auto* vb = static_cast<const __bf16*>(v);
    auto* ob = static_cast<__bf16*>(o);

    if (!use_split_path(s, x)) {
        fa::PrefillParams p;
        p.q = qb; p.k = kb; p.v = vb; p.o = ob; p.lse = lse; p.kv_lens = kv_lens;
        p.B = s.B; p.Hq = s.Hq; p.Hkv = s.Hkv; p.Lq = s.Lq; p.Lk = s.Lk;
        p.r = r;
        p.n_qblocks = (s.Lq + fa::kPrefillRows - 1) / fa::kPrefillRows;
        const int units = s.B * s.Hkv;
        p.xcd_units = (units % 8 == 0) ? units / 8 : 0;
        p.xcd_spread = xcd_spread(r, p.n_qblocks);
        p.window = x.window;
        p.scale = scale;
        p.c = c;
        const long long total = (long long)s.B * s.Hq * p.n_qblocks;
        if (!grid_fits(total, 512)) return fail(FA_ERR_INVALID_ARG, "grid too large");
        hipError_t e = fa::launch_prefill(s.D, causal != 0, p, stream);
        if (e != hipSuccess) return fail(FA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
        return FA_OK;
    }

    // The split kernels address the r * Lq query rows that share a KV head
    // through one buffer descriptor with 32-bit byte offsets.
    if ((long long)r * s.Lq * s.D * 2 > (long long)UINT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "split-KV path: (Hq/Hkv) * Lq * D * 2 = %lld bytes exceeds the "
                    "32-bit offsets of one KV head's packed query rows", (long long)r * s.Lq * s.D * 2);
    const SplitPlan pl = plan_splits(s, x.requested_splits, cu_count(), visible_span(s, x.window));
    void* ws = nullptr;
    const size_t ws_bytes = split_workspace_bytes(s, pl);
    if (x.no_alloc) {
        if (ws_bytes > kNoAllocScratchBytes)
            return fail(FA_ERR_INVALID_ARG, "split-KV workspace of %zu bytes (%d partitions) exceeds the "
                        "static scratch of %zu bytes; pass fewer partitions or a smaller problem",
                        ws_bytes, pl.num_splits, kNoAllocScratchBytes);
        st = scratch_address(&ws);
    } else {
        st = get_workspace(ws_bytes, &ws);
    }
    if (st != FA_OK) return st;
    const size_t rows = (size_t)s.B * s.Hq * s.Lq;
    float* part_o = static_cast<float*>(ws);
    float* part_lse = part_o + rows * pl.num_splits * s.D;

    fa::SplitParams sp;
    sp.q = qb; sp.k = kb; sp.v = vb; sp.part_o = part_o; sp.part_lse = part_lse;
    sp.kv_lens = kv_lens;
    sp.B = s.B; sp.Hq = s.Hq; sp.Hkv = s.Hkv; sp.Lq = s.Lq; sp.Lk = s.Lk;
    sp.r = r; sp.rows = r * s.Lq; sp.n_groups = pl.n_groups;
    sp.num_splits = pl.num_splits; sp.chunk = pl.chunk; sp.causal = causal; sp.c = c;
    sp.window = x.window;
    sp.page_table = x.page_table; sp.max_pages = x.max_pages;
    sp.num_pages = x.num_pages; sp.page_size = x.page_size;
    const long long total = (long long)s.B * s.Hkv * pl.n_groups * pl.num_splits;
    if (!grid_fits(total, 64) || !grid_fits(((long long)rows + 3) / 4, 256))
        return fail(FA_ERR_INVALID_ARG, "grid too large");
    hipError_t e = fa::launch_splitkv(s.D, x.page_table != nullptr, sp, stream);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "split-KV launch: %s", hipGetErrorString(e));

    fa::CombineParams cp;
    cp.part_o = part_o; cp.part_lse = part_lse; cp.o = ob; cp.lse = lse; cp.kv_lens = kv_lens;
    cp.B = s.B; cp.Hq = s.Hq; cp.Lq = s.Lq; cp.Lk = s.Lk;
    cp.num_splits = pl.num_splits; cp.chunk = pl.chunk;
    e = fa::launch_combine(s.D, cp, stream);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
    return FA_OK;
}

constexpr int kMaxVarlenBatch = 1 << 16;   // sequences per packed batch (the schedule is O(B^2))

int validate_varlen_offsets(const int* cu_q, const int* cu_k, int B, int total_q, int total_k) {
    if (B <= 0 || B > kMaxVarlenBatch)
        return fail(FA_ERR_INVALID_ARG, "B (%d) must be in [1, %d]", B, kMaxVarlenBatch);
    if (total_q < 0 || total_k < 0)
        return fail(FA_ERR_INVALID_ARG, "total_q (%d) and total_k (%d) must be >= 0", total_q, total_k);
    if (!cu_q || !cu_k) return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must not be NULL");
    if (!aligned(cu_q, 4) || !aligned(cu_k, 4))
        return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be 4-byte aligned");
    return FA_OK;
}

int enqueue_varlen_schedule(const int* cu_q, const int* cu_k, int B, int total_q, int total_k, int* schedule,
                            hipStream_t stream) {
    fa::VarlenScheduleParams sp;
    sp.cu_q = cu_q; sp.cu_k = cu_k; sp.schedule = schedule;
    sp.B = B; sp.total_q = total_q; sp.total_k = total_k;
    hipError_t e = fa::launch_varlen_schedule(sp, stream);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "varlen schedule launch: %s", hipGetErrorString(e));
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Lq, int Lk, int D,
           int causal, float scale, const int* kv_lens, void* stream) {
    g_last_error[0] = '\0';
    return run(q, k, v, o, lse, Shape{B, Hq, Hkv, Lq, Lk, D}, causal, scale, kv_lens, stream, Extra{});
}

int fa_fwd_splits(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Lq, int Lk, int D,
                  int causal, float scale, const int* kv_lens, void* stream,
                  int num_splits) {
    g_last_error[0] = '\0';
    Extra x;
    x.requested_splits = num_splits;
    return run(q, k, v, o, lse, Shape{B, Hq, Hkv, Lq, Lk, D}, causal, scale, kv_lens, stream, x);
}

int fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Lq, int Lk, int D,
                   int causal, float scale, const int* kv_lens, void* stream,
                   int num_splits) {
    g_last_error[0] = '\0';
    Extra x;
    x.requested_splits = num_splits;
    x.no_alloc = true;
    return run(q, k, v, o, lse, Shape{B, Hq, Hkv, Lq, Lk, D}, causal, scale, kv_lens, stream, x);
}

size_t fa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Lq, int Lk, int D,
                  int window, float scale, const int* kv_lens, void* stream, int num_splits) {
    g_last_error[0] = '\0';
    Extra x;
    x.window = window;
    x.requested_splits = num_splits;
    return run(q, k, v, o, lse, Shape{B, Hq, Hkv, Lq, Lk, D}, 1, scale, kv_lens, stream, x);
}

int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int D,
                 const int* page_table, int max_pages, int num_pages, int page_size,
                 const int* kv_lens, int causal, int window, float scale, void* stream,
                 int num_splits) {
    g_last_error[0] = '\0';
    if (max_pages <= 0 || page_size <= 0 || (long long)max_pages * page_size > INT32_MAX / 2)
        return fail(FA_ERR_INVALID_ARG, "max_pages (%d) and page_size (%d) must be positive and "
                    "their product must fit 30 bits", max_pages, page_size);
    if (!page_table) return fail(FA_ERR_INVALID_ARG, "page_table must not be NULL");
    if (!k_cache || !v_cache) return fail(FA_ERR_INVALID_ARG, "k_cache and v_cache must not be NULL");
    Extra x;
    x.window = window;
    x.requested_splits = num_splits;
    x.page_table = page_table;
    x.max_pages = max_pages;
    x.num_pages = num_pages;
    x.page_size = page_size;
    const int capacity = max_pages * page_size;
    return run(q, k_cache, v_cache, o, lse, Shape{B, Hq, Hkv, Lq, capacity, D}, causal, scale,
               kv_lens, stream, x);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int Lq, int Lk, int D,
           int causal, int window, float scale, const int* kv_lens, void* stream) {
    g_last_error[0] = '\0';
    const Shape s{B, Hq, Hkv, Lq, Lk, D};
    int st = validate(q, k, v, dq, nullptr, s, causal, scale, kv_lens);
    if (st != FA_OK) return st;
    if (!o || !dout || !lse || !dk || !dv)
        return fail(FA_ERR_INVALID_ARG, "o, dout, lse, dk and dv must not be NULL");
    if (!aligned(o, 16) || !aligned(dout, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
        return fail(FA_ERR_INVALID_ARG, "o, dout, dk and dv must be 16-byte aligned, lse 4-byte aligned");
    if (window < 0) return fail(FA_ERR_INVALID_ARG, "window must be >= 0");
    if (window > 0 && !causal) return fail(FA_ERR_INVALID_ARG, "a window needs causal masking");
    void* ws = nullptr;
    st = get_workspace((size_t)B * Hq * Lq * sizeof(float), &ws);
    if (st != FA_OK) return st;
    fa::BwdParams p;
    p.q = static_cast<const __bf16*>(q);
    p.k = static_cast<const __bf16*>(k);
    p.v = static_cast<const __bf16*>(v);
    p.o = static_cast<const __bf16*>(o);
    p.dout = static_cast<const __bf16*>(dout);
    p.lse = lse;
    p.delta = static_cast<float*>(ws);
    p.dq = static_cast<__bf16*>(dq);
    p.dk = static_cast<__bf16*>(dk);
    p.dv = static_cast<__bf16*>(dv);
    p.kv_lens = kv_lens;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lq = Lq; p.Lk = Lk;
    p.r = Hq / Hkv;
    p.causal = causal;
    p.window = window;
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    const long long nq = (long long)B * Hq * ((Lq + 31) / 32);
    const long long nk = (long long)B * Hkv * ((Lk + 31) / 32);
    if (!grid_fits(nq, 256) || !grid_fits(nk, 512)) return fail(FA_ERR_INVALID_ARG, "grid too large");
    hipError_t e = fa::launch_backward(D, p, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return FA_OK;
}

int fa_fwd_mod(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, float scale,
               const int* kv_lens, const float* alibi_slopes, float softcap, void* stream) {
    g_last_error[0] = '\0';
    const Shape s{B, Hq, Hkv, Lq, Lk, D};
    int st = validate(q, k, v, o, lse, s, causal, scale, kv_lens);
    if (st != FA_OK) return st;
    if (!(softcap >= 0.0f) || !std::isfinite(softcap))
        return fail(FA_ERR_INVALID_ARG, "softcap must be finite and >= 0");
    if (alibi_slopes && softcap > 0.0f)
        return fail(FA_ERR_INVALID_ARG, "give ALiBi slopes or a soft-cap, not both");
    if (!aligned(alibi_slopes, 4)) return fail(FA_ERR_INVALID_ARG, "alibi_slopes must be 4-byte aligned");
    if (!alibi_slopes && softcap == 0.0f)       // no modifier: the plain forward
        return fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, causal, scale, kv_lens, stream);
    fa::PrefillParams p;
    p.q = static_cast<const __bf16*>(q);
    p.k = static_cast<const __bf16*>(k);
    p.v = static_cast<const __bf16*>(v);
    p.o = static_cast<__bf16*>(o);
    p.lse = lse; p.kv_lens = kv_lens;
    p.q8 = nullptr; p.k8 = nullptr; p.q_scale = nullptr; p.k_scale = nullptr;
    p.alibi_slopes = alibi_slopes;
    p.softcap = softcap;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lq = Lq; p.Lk = Lk;
    p.r = Hq / Hkv;
    p.n_qblocks = (Lq + fa::kPrefillRows - 1) / fa::kPrefillRows;
    const int units = B * Hkv;
    p.xcd_units = (units % 8 == 0) ? units / 8 : 0;
    p.xcd_spread = xcd_spread(Hq / Hkv, p.n_qblocks);
    p.window = 0;
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    const long long total = (long long)B * Hq * p.n_qblocks;
    if (!grid_fits(total, 512)) return fail(FA_ERR_INVALID_ARG, "grid too large");
    hipError_t e = fa::launch_prefill_mod(D, causal != 0, alibi_slopes ? 1 : 2, p,
                                          reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return FA_OK;
}

int fa_quantize_fp8(const void* x, void* x8, float* scales, int heads, int L, int D,
                    int block_rows, const float* signs, void* stream) {
    g_last_error[0] = '\0';
    if (heads <= 0 || L <= 0 || block_rows <= 0)
        return fail(FA_ERR_INVALID_ARG, "heads, L and block_rows must be positive: heads=%d L=%d block_rows=%d",
                    heads, L, block_rows);
    if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension D=%d is not supported (64 or 128)", D);
    if (!x || !x8 || !scales) return fail(FA_ERR_INVALID_ARG, "x, x8 and scales must not be NULL");
    if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(scales, 4) || !aligned(signs, 16))
        return fail(FA_ERR_INVALID_ARG, "x, x8 and signs must be 16-byte aligned, scales 4-byte aligned");
    const long long nblk = (L + (long long)block_rows - 1) / block_rows;
    if ((long long)heads * nblk > INT32_MAX || (long long)L * D > INT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "problem too large");
    fa::QuantParams p;
    p.x = static_cast<const __bf16*>(x);
    p.x8 = static_cast<uint8_t*>(x8);
    p.scales = scales;
    p.signs = signs;
    p.heads = heads; p.L = L; p.block_rows = block_rows; p.nblk = (int)nblk;
    hipError_t e = fa::launch_quantize_fp8(D, p, cu_count(), reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FA_ERR_HIP, "quantize launch: %s", hipGetErrorString(e));
    return FA_OK;
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v, void* o, float* lse,
               const float* q_scales, const float* k_scales,
               int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, float scale,
               const int* kv_lens, void* stream) {
    g_last_error[0] = '\0';
    const Shape s{B, Hq, Hkv, Lq, Lk, D};
    int st = validate(q8, k8, v, o, lse, s, causal, scale, kv_lens);
    if (st != FA_OK) return st;
    if (!q_scales || (Lk > 0 && !k_scales)) return fail(FA_ERR_INVALID_ARG, "q_scales and k_scales must not be NULL");
    if (!aligned(q_scales, 4) || !aligned(k_scales, 4))
        return fail(FA_ERR_INVALID_ARG, "q_scales and k_scales must be 4-byte aligned");
    fa::PrefillParams p;
    p.q = nullptr; p.k = nullptr;
    p.v = static_cast<const __bf16*>(v);
    p.o = static_cast<__bf16*>(o);
    p.lse = lse; p.kv_lens = kv_lens;
    p.q8 = static_cast<const uint8_t*>(q8);
    p.k8 = static_cast<const uint8_t*>(k8);
    p.q_scale = q_scales;
    p.k_scale = k_scales;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lq = Lq; p.Lk = Lk;
    p.r = Hq / Hkv;
    p.n_qblocks = (Lq + fa::kPrefillRows - 1) / fa::kPrefillRows;
    const int units = B * Hkv;
    p.xcd_units = (units % 8 == 0) ? units / 8 : 0;
    p.xcd_spread = xcd_spread(Hq / Hkv, p.n_qblocks);
    p.window = 0;
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    const long long total = (long long)B * Hq * p.n_qblocks;
    if (!grid_fits(total, 512)) return fail(FA_ERR_INVALID_ARG, "grid too large");
    hipError_t e = fa::launch_prefill_fp8(D, causal != 0, p, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FA_ERR_HIP, "fp8 prefill launch: %s", hipGetErrorString(e));
    return FA_OK;
}

int fa_fwd_fp8_q(const void* q, const float* signs, const void* k8, const void* v, void* o, float* lse,
                 const float* k_scales, int B, int Hq, int Hkv, int Lq, int Lk, int D, int causal, float scale,
                 const int* kv_lens, void* stream) {
    g_last_error[0] = '\0';
    const Shape s{B, Hq, Hkv, Lq, Lk, D};
    int st = validate(q, k8, v, o, lse, s, causal, scale, kv_lens);
    if (st != FA_OK) return st;
    if (Lk > 0 && !k_scales) return fail(FA_ERR_INVALID_ARG, "k_scales must not be NULL");
    if (!aligned(k_scales, 4)) return fail(FA_ERR_INVALID_ARG, "k_scales must be 4-byte aligned");
    if (!aligned(signs, 16)) return fail(FA_ERR_INVALID_ARG, "signs must be 16-byte aligned");
    fa::PrefillParams p;
    p.q = static_cast<const __bf16*>(q);
    p.k = nullptr;
    p.v = static_cast<const __bf16*>(v);
    p.o = static_cast<__bf16*>(o);
    p.lse = lse; p.kv_lens = kv_lens;
    p.k8 = static_cast<const uint8_t*>(k8);
    p.k_scale = k_scales;
    p.q_signs = signs;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lq = Lq; p.Lk = Lk;
    p.r = Hq / Hkv;
    p.n_qblocks = (Lq + fa::kPrefillRows - 1) / fa::kPrefillRows;
    const int units = B * Hkv;
    p.xcd_units = (units % 8 == 0) ? units / 8 : 0;
    p.xcd_spread = xcd_spread(Hq / Hkv, p.n_qblocks);
    p.window = 0;
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    const long long total = (long long)B * Hq * p.n_qblocks;
    if (!grid_fits(total, 512)) return fail(FA_ERR_INVALID_ARG, "grid too large");
    hipError_t e = fa::launch_prefill_fp8(D, causal != 0, p, reinterpret_cast<hipStream_t>(stream), true);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "fp8 prefill launch: %s", hipGetErrorString(e));
    return FA_OK;
}

size_t fa_varlen_schedule_ints(int B) {
    return (B > 0 && B <= kMaxVarlenBatch) ? 2 * (size_t)B + 1 : 0;
}

int fa_varlen_schedule(const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int total_q, int total_k,
                       int* schedule, void* stream) {
    g_last_error[0] = '\0';
    int st = validate_varlen_offsets(cu_seqlens_q, cu_seqlens_k, B, total_q, total_k);
    if (st != FA_OK) return st;
    if (!schedule || !aligned(schedule, 4))
        return fail(FA_ERR_INVALID_ARG, "schedule must be a non-NULL, 4-byte aligned array of 2B + 1 ints");
    return enqueue_varlen_schedule(cu_seqlens_q, cu_seqlens_k, B, total_q, total_k, schedule,
                                   reinterpret_cast<hipStream_t>(stream));
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, const int* schedule,
                  int B, int Hq, int Hkv, int total_q, int total_k, int D,
                  int causal, float scale, void* stream) {
    g_last_error[0] = '\0';
    int st = validate_varlen_offsets(cu_seqlens_q, cu_seqlens_k, B, total_q, total_k);
    if (st != FA_OK) return st;
    if (Hq <= 0 || Hkv <= 0)
        return fail(FA_ERR_INVALID_ARG, "Hq (%d) and Hkv (%d) must be positive", Hq, Hkv);
    if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (D != 64 && D != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension D=%d is not supported (64 or 128)", D);
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and positive");
    if (total_q == 0) return FA_OK;         // no query row: nothing to compute or write
    if (!q || !o) return fail(FA_ERR_INVALID_ARG, "q and o must not be NULL");
    if (total_k > 0 && (!k || !v)) return fail(FA_ERR_INVALID_ARG, "k and v must not be NULL when total_k > 0");
    if (!aligned(q, 16) || !aligned(o, 16) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)))
        return fail(FA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if ((lse && !aligned(lse, 4)) || (schedule && !aligned(schedule, 4)))
        return fail(FA_ERR_INVALID_ARG, "lse and schedule must be 4-byte aligned");
    // Per-sequence byte offsets (plus one query block of overshoot) must fit
    // the 32-bit offsets of the buffer loads; packed row counts 32-bit indices.
    if (((long long)total_q + 256) * D * 2 > (long long)UINT32_MAX ||
        ((long long)total_k + 256) * D * 2 > (long long)UINT32_MAX ||
        (long long)Hq * total_q > INT32_MAX || (long long)Hkv * total_k > INT32_MAX)
        return fail(FA_ERR_INVALID_ARG, "packed batch too large for 32-bit offsets");
    // Query blocks of the batch: sum_b ceil(Lq_b / 256) <= (total_q + 255 B) / 256,
    // and never more than total_q (every block holds a row).
    long long items = ((long long)total_q + 255LL * B) / fa::kPrefillRows;
    if (items > total_q) items = total_q;
    if (!grid_fits(items * Hq, 512)) return fail(FA_ERR_INVALID_ARG, "grid too large");
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if (!schedule) {
        void* ws = nullptr;
        st = get_workspace(fa_varlen_schedule_ints(B) * sizeof(int), &ws);
        if (st != FA_OK) return st;
        st = enqueue_varlen_schedule(cu_seqlens_q, cu_seqlens_k, B, total_q, total_k, static_cast<int*>(ws), hs);
        if (st != FA_OK) return st;
        schedule = static_cast<const int*>(ws);
    }
    fa::PrefillParams p;
    p.q = static_cast<const __bf16*>(q);
    p.k = static_cast<const __bf16*>(k);
    p.v = static_cast<const __bf16*>(v);
    p.o = static_cast<__bf16*>(o);
    p.lse = lse; p.kv_lens = nullptr;
    p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k; p.schedule = schedule;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Lq = total_q; p.Lk = total_k;
    p.r = Hq / Hkv;
    p.n_qblocks = 0; p.xcd_units = 0; p.xcd_spread = 0;
    p.window = 0;
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    hipError_t e = fa::launch_prefill_varlen(D, causal != 0, p, (int)items, hs);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "varlen prefill launch: %s", hipGetErrorString(e));
    return FA_OK;
}

size_t fa_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D) {
    const Shape s{B, Hq, Hkv, Lq, Lk, D};
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    const int st = validate_shape(s);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != FA_OK || !use_split_path(s, Extra{})) return 0;
    return split_workspace_bytes(s, plan_splits(s, 0, cu_count(), s.Lk));
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: valid but unsupported configuration";
        case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime or launch failure";
        default: return "unknown fa_status";
    }
}

const char* fa_last_error(void) { return g_last_error; }

}  // extern "C"
