// Device-side building blocks shared by the gfx950 attention kernels.
//
// Register layouts of the bf16 MFMA used here (v_mfma_f32_32x32x16_bf16, one
// wave64, D[32x32] += A[32x16] * B[16x32]):
//   A operand : lane l holds row (l % 32), k = 8 * (l / 32) + e, e = 0..7
//   B operand : lane l holds column (l % 32), k = 8 * (l / 32) + e
//   C / D     : lane l holds column (l % 32), rows 8 * (v / 4) + 4 * (l / 32) + (v % 4),
//               v = 0..15
// Every lane of these layouts is exercised by the parity tests.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417232121458176568f;

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Value held by lane (l ^ 32): v_permlane32_swap exchanges the upper half of
// its first operand with the lower half of its second; with both operands x,
// result[0] is x[l - 32] on the upper lanes and result[1] is x[l + 32] on the
// lower lanes.
__device__ __forceinline__ float lane_xor32(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned lane = __lane_id();
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// Key-row permutation that makes the S^T accumulator of one 32-key block line
// up with the B operand of the PV product: swap bits 2 and 3 of the row.
// Accumulator entry v of lane l then holds key 16*(v/8) + 8*(l/32) + (v%8).
// max(x, x of lane l ^ 32) and x + (x of lane l ^ 32): the two results of the
// swap hold x and its partner, in an order that depends on the half.
__device__ __forceinline__ float max_with_partner(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
    const unsigned u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int swap_bits_2_3(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Sequence b of a packed batch from its cumulative offsets cu[B + 1]: start
// and length, clamped to [0, total] and to a non-negative length, so that
// malformed offsets give empty or shortened sequences, never an access outside
// the packed tensors.
__device__ __forceinline__ void varlen_segment(const int* cu, int b, int total, int& start, int& len) {
    const int s = min(max(cu[b], 0), total);
    const int e = min(max(cu[b + 1], s), total);
    start = s;
    len = e - s;
}

// Buffer resource over [base, base + bytes): a raw buffer load whose 16 bytes
// lie past `bytes` returns zeros (hardware range check), so rows beyond a
// sequence's valid length read as zero without a branch and are never fetched.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 load16(rsrc_t r, uint32_t byte_offset) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}

// The same load marked non-temporal (the nt cache policy): for data read once
// in full lines, so streamed bytes do not displace cached ones.  Only for
// loads whose lines are consumed whole by the instruction itself: a partial
// line is not kept for the next instruction and would be fetched again.
__device__ __forceinline__ bf16x8 load16_stream(rsrc_t r, uint32_t byte_offset) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 2));
}

// s_waitcnt vmcnt(0): wait for every outstanding vector-memory load of this
// wave (expcnt and lgkmcnt left at their maxima).  Issued through the builtin
// so the compiler's own wait-count tracking knows the loads have completed.
__device__ __forceinline__ void wait_all_vector_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Direct HBM -> LDS copy of 16 bytes per lane through a range-checked buffer:
// lane l's bytes land at lds_base + 16 * l (lane-linear), out-of-range bytes
// arrive as zeros.  lds_base must be the same for the whole wavefront.
__device__ __forceinline__ void load16_to_lds(rsrc_t r, uint32_t byte_offset, bf16* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 16, byte_offset, 0, 0, 0);
}

// Buffer descriptor as four scalar dwords, for the inline-assembly copy below:
// base address (wave-uniform), stride 0, range in bytes, raw-buffer format.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_desc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 d;
    d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFF));
    d[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    d[3] = 0x00020000;
    return d;
}

// The same direct HBM -> LDS copy as load16_to_lds, issued from inline assembly
// so the compiler's wait-count tracking does not see it: the caller waits for
// it explicitly (vmcnt) before any wavefront reads the destination.  Without
// this the compiler waits for every outstanding copy before the first LDS read
// that it cannot prove disjoint, which defeats copying tiles several steps ahead.
// M0 (the LDS base of the copy) is saved and restored around it.
__device__ __forceinline__ void copy16_to_lds_async(i32x4 desc, uint32_t byte_offset,
                                                    uint32_t lds_addr) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(byte_offset), "s"(desc), "s"(lds_addr)
        : "memory");
}

// s_waitcnt vmcnt(N) with the other counters left at their maxima (gfx9
// encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vector_loads_until() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives element
// (j % 4) of the 8-byte rows read by lanes 4k + j / 4 of its group, k = 0..3.
// When four consecutive lanes point at four consecutive columns of one row of
// a row-major tile, each lane gets one column of four consecutive rows.
__device__ __forceinline__ bf16x4 lds_read_transposed(const bf16* addr) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<bf16*>(addr)));
    return __builtin_bit_cast(bf16x4, v);
}

// 16-byte-chunk XOR swizzles of K and V tiles in LDS (row-major, D columns).
// K is read one row per lane (16 consecutive lanes: 16 distinct rows, one
// chunk column); V is read by ds_read_b64_tr_b16 (32 lanes: 4 rows x 4
// chunks).  Either way the XOR spreads each batch of lanes over all 64 banks.
// Both depend only on the low bits of the row, so any tile height that is a
// multiple of 16 rows can use them.
template <int D>
__device__ __forceinline__ int k_swizzle(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swizzle(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
    return z;
}

__device__ __forceinline__ f32x16 zero_f32x16() {
    f32x16 z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.0f;
    return z;
}

// Eight fp32 values to bf16, round to nearest even.
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
    bf16x8 r;
    r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
    r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
    return r;
}

}  // namespace fa
