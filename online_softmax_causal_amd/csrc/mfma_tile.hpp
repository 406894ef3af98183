// MFMA operand helpers shared by the attention kernels (gfx950, wave64):
// 16-bit vector types, the 32x32x16 MFMA with its 16-bit packing and pair
// sums, the LDS chunk swizzle, LDS transpose reads, direct global->LDS copies
// and explicit vector-memory waits.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace osc {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

template <bool BF16>
struct Mma;

// kSumRounded: whether the row sum l is taken over the 16-bit P fed to the
// P V product (with v_dot2 on the packed pairs) or over the FP32 P before
// rounding (with FP32 adds).  Both dtypes take the FP32 sum: on gfx950 every
// v_dot2_f32_{f16,bf16} holds the matrix pipe for about 17 cycles, so the dot2
// form costs a sixth of an MFMA per pair, while FP32 adds issue beside the
// MFMAs.  The FP32 sum carries no P rounding error into the LSE.  O =
// sum(p~ v) / sum(p) then differs from the rounded-P ratio by up to the P
// rounding (unit roundoff 2^-11 fp16, 2^-8 bf16) times max|v| when one key
// dominates a row and its P is not exactly 1: 2.4e-3 at |v| = 5 in fp16, and
// 2e-2 in bf16.  Kernels that take an exact tile max make the dominant P
// exactly 1 in bf16 (rescale_slack below); the kernels with a stale
// reference max keep this bound.
template <>
struct Mma<false> {
    static constexpr bool kSumRounded = false;
    __device__ __forceinline__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    // Round-to-nearest-even conversion of two FP32 values into one packed dword.
    __device__ __forceinline__ static unsigned pack(float lo, float hi) {
        f16x2 r;
        r[0] = (_Float16)lo;
        r[1] = (_Float16)hi;
        return __builtin_bit_cast(unsigned, r);
    }
    // acc + lo + hi of one packed dword, accumulated in FP32.
    __device__ __forceinline__ static float sum2(unsigned packed, float acc) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, acc, false);
    }
};

template <>
struct Mma<true> {
    static constexpr bool kSumRounded = false;
    __device__ __forceinline__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static unsigned pack(float lo, float hi) {
        bf16x2 r;
        r[0] = (__bf16)lo;
        r[1] = (__bf16)hi;
        return __builtin_bit_cast(unsigned, r);
    }
    __device__ __forceinline__ static float sum2(unsigned packed, float acc) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
    }
};

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008;
constexpr int kSgDsRead = 0x100;

template <int D>
__device__ __forceinline__ int chunk_swizzle(int r) {
    if constexpr (D == 128)
        return ((r & 3) << 2) | ((r >> 2) & 3);
    else
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Conditional rescaling: the reference max m moves only when a query's
// tile max exceeds it by more than 2^8.  Between moves the exponentials are
// taken against a stale m, so each P element is at most 2^8 (exact in fp16
// and bf16 range); O and l always share the same reference, so O = o/l is
// unchanged.  This skips the rescale of the O accumulator on most tiles.
constexpr float kRescaleSlack = 8.0f;

// The slack the kernels that take an exact tile max use.  With bf16 inputs
// P is rounded to 8 significant bits before P V, while l sums the FP32 P, so
// a row dominated by one key carries that key's rounding (up to 2^-8
// relative) into O.  Moving m to every new maximum makes the largest P of
// the row exactly 1, which rounds exactly; fp16 (2^-11) keeps the slack.
template <bool BF16>
constexpr float rescale_slack() {
    return BF16 ? 0.0f : kRescaleSlack;
}

__device__ __forceinline__ u32x4 tr16_b64x2(const u16* p0, const u16* p1) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
    const auto a = __builtin_bit_cast(unsigned long long, r0);
    const auto b = __builtin_bit_cast(unsigned long long, r1);
    return u32x4{(unsigned)a, (unsigned)(a >> 32), (unsigned)b, (unsigned)(b >> 32)};
}

// Offsets (16-bit elements, relative to an LDS tile of rows of D values in
// the chunk_swizzle layout) of this lane's MFMA A-operand fragments:
//   row_frag_offset: row `row` (lane % 32 of a 32-row block), the 8 values
//     d = 16 ks + 8 (lane / 32) .. + 7 (one 16-wide step of the contraction
//     over d);
//   tr_frag_offset: one of the two ds_read_b64_tr_b16 reads (r = 0, 1) that
//     give the transposed fragment X^T[d = 32 mt + lane % 32][16 rows of a
//     group], the rows in the order of the 32x32 accumulator layout
//     (8 (j / 4) + 4 (lane / 32) + j % 4 for slot j), relative to the group's
//     first row.
template <int D>
__device__ __forceinline__ int row_frag_offset(int row, int ks, int lane) {
    return row * D + (((2 * ks + (lane >> 5)) ^ chunk_swizzle<D>(row)) << 3);
}

template <int D>
__device__ __forceinline__ int tr_frag_offset(int lane, int mt, int r) {
    const int row = 4 * (lane >> 5) + ((lane >> 2) & 3) + 8 * r;
    const int c = 4 * mt + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return row * D + ((c ^ chunk_swizzle<D>(row)) << 3) + 4 * (lane & 1);
}

// Byte offset of an LDS location (what M0 and ds_* addresses use).
__device__ __forceinline__ unsigned lds_offset(const void* p) {
    return (unsigned)(unsigned long long)((const __attribute__((address_space(3))) char*)p);
}

// global_load_lds_dwordx4: each lane copies 16 bytes from gbase + voff to
// LDS address m0 + 16 * lane.  Written as inline assembly so the compiler's
// memory model does not see an LDS store: it would otherwise make every
// later LDS read wait for the copy, which targets a stage that no wave reads
// until the barrier after the matching wait_vmcnt.
__device__ __forceinline__ void copy_to_lds16(const void* gbase, unsigned voff, void* lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_offset(lds_dst)), "v"(voff), "s"(gbase)
                 : "m0");
}

// The 4-byte form: lane i copies 4 bytes from gbase + voff to m0 + 4 * lane.
__device__ __forceinline__ void copy_to_lds4(const void* gbase, unsigned voff, void* lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(lds_offset(lds_dst)), "v"(voff), "s"(gbase)
                 : "m0");
}

// The same copy from a full 64-bit global address per lane (gathers whose
// offsets do not fit 32 bits, e.g. rows of a paged cache).
__device__ __forceinline__ void copy_to_lds16_at(const void* gaddr, void* lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_offset(lds_dst)), "v"(gaddr)
                 : "m0");
}

// The same with the non-temporal hint, for data read exactly once.
__device__ __forceinline__ void copy_to_lds16_at_nt(const void* gaddr, void* lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(lds_offset(lds_dst)), "v"(gaddr)
                 : "m0");
}

// Wait until at most `n` of this wave's vector-memory loads are outstanding
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt are left at their maxima so they
// are not waited on).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt field");
    // vmcnt is split: bits [3:0] hold its low four bits, bits [15:14] the high two.
    __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

}  // namespace osc
