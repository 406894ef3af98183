// Matrix-core ceiling probe (measurement support for bench.py --ceiling; not
// part of the attention library's interface).
//
// Under a sustained MFMA load this part does not hold its nominal 2.4 GHz:
// the firmware lowers the GFX clock to stay within the board power limit and,
// as the work per cycle grows, further (the probe's heavier mixes settle at
// lower clocks while drawing less power).  The rate an MFMA-bound kernel can
// reach therefore depends on the instructions it issues, not only on the
// nominal peak.  This probe measures that rate for four fixed instruction
// mixes, with the same MFMA (v_mfma_f32_32x32x16_f16), the same occupancy
// (one 512-thread workgroup per CU, two waves per SIMD) and the same kind of
// operand data (random fp16) as the attention forward kernel:
//   mix 0  MFMAs only, four independent accumulator chains per wave;
//   mix 1  mix 0 plus one 16-byte-per-lane LDS read per MFMA as its A operand
//          (1 KiB per MFMA per wave: the forward kernel's K/V fragment bytes);
//   mix 2  mix 1 plus, per MFMA, one FMA, one exp2 and one add on a value of
//          another accumulator chain and, every second MFMA, one fp16 pack
//          (the forward kernel's per-score softmax work at D = 128: 32 scores
//          per lane per 32 MFMAs);
//   mix 3  mix 1 plus that work on two values per MFMA and one pack per MFMA
//          (the score density at D = 64: 64 scores per lane per 32 MFMAs);
//   mix 4  mix 2 with one wave per SIMD (256-thread workgroups);
//   mix 5  mix 4 with each LDS fragment feeding two MFMAs (two B operands,
//          as a wave holding two 32-row query blocks would): half the LDS
//          reads per MFMA, the same softmax work per MFMA;
//   mix 6  mix 2's instructions in phases, as a kernel that finishes a
//          tile's products before its softmax orders them: each step's 16
//          MFMAs back to back, then the 16 values of that step's scores (two
//          waves per SIMD).
// bench.py runs each mix back to back while sampling clock and power.
//
// An LDS probe streams fragment reads alone, as the MFMA operands are read:
// 16-byte ds_read_b128 rows, or pairs of 8-byte ds_read_b64_tr_b16 transposed
// reads in the attention kernels' swizzled layout, 1 KiB per wave
// instruction pair or row read, with one or two waves per SIMD.
//
// Two HBM probes give the same kind of reference for the memory-bound paths:
// a streaming read and a streaming copy, both grid-stride with 16-byte
// non-temporal accesses.  Their shapes are the fastest of a sweep over grid
// size, accesses in flight per thread and temporal / non-temporal accesses:
// the read with 4 workgroups per CU and 8 loads in flight per thread (6.6
// TB/s), the copy with 2 workgroups per CU and 4 (5.7 TB/s read + write).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsVec = 6144;  // 96 KiB of 16-byte vectors: one workgroup per CU
constexpr int kMfmaPerIter = 16;

// Threads per workgroup: two waves per SIMD, or one for mixes 4 and 5.
constexpr int threads_of(int mix) { return mix == 4 || mix == 5 ? 256 : 512; }

// One step: 16 MFMAs into accumulator set PH; with MIX >= 1 their A operands
// come from a ring of 4 LDS fragments, each read 4 fragments ahead of its
// use and used by QB consecutive MFMAs (QB = 2 for mix 5, with B operands
// b0 and b1 alternating); with MIX >= 2 the VALU work reads set PH ^ 1,
// written by the previous step (so it never waits on an MFMA in flight, as
// the softmax of a finished tile does not).
template <int MIX, int PH>
__device__ __forceinline__ void ceiling_step(f32x16 (&c)[2][4], f16x8 (&ring)[4], const f16x8& a,
                                             const f16x8& b0, const f16x8& b1,
                                             const f16x8 __attribute__((address_space(3)))* base,
                                             float& sum, float& p0) {
    constexpr int QB = MIX == 5 ? 2 : 1;
#pragma unroll
    for (int m = 0; m < kMfmaPerIter; ++m) {
        const int fi = m / QB;
        const f16x8 av = MIX >= 1 ? ring[fi & 3] : a;
        const f16x8 bv = (QB == 2 && (m & 1)) ? b1 : b0;
        c[PH][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c[PH][m & 3], 0, 0, 0);
        if constexpr (MIX >= 1) {
            if (m % QB == QB - 1) ring[fi & 3] = base[256 * ((fi + 4) & 15)];
        }
        // Values per MFMA: 1 (mixes 2, 4, 5) or 2 (mix 3); a pack per two values.
        constexpr int VPM = MIX == 3 ? 2 : MIX >= 2 ? 1 : 0;
#pragma unroll
        for (int v = 0; v < VPM; ++v) {
            const int x = m * VPM + v;  // < 32: chains 0 and 1 of the other set
            const float p = __builtin_amdgcn_exp2f(fmaf(c[PH ^ 1][x >> 4][x & 15], 1.0e-4f, -0.5f));
            sum += p;
            if (x & 1) {
                f16x2 pk;
                pk[0] = (_Float16)p0;
                pk[1] = (_Float16)p;
                asm volatile("" ::"v"(pk));
            } else {
                p0 = p;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Mix 6: the 16 MFMAs of a step back to back (A operands through the same
// 4-deep LDS ring), then the softmax work on 16 values of the scores those
// MFMAs just produced, with no MFMA beside it.
template <int PH>
__device__ __forceinline__ void phased_step(f32x16 (&c)[2][4], f16x8 (&ring)[4], const f16x8& b0,
                                            const f16x8 __attribute__((address_space(3)))* base,
                                            float& sum, float& p0) {
#pragma unroll
    for (int m = 0; m < kMfmaPerIter; ++m) {
        c[PH][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[m & 3], b0, c[PH][m & 3], 0, 0, 0);
        ring[m & 3] = base[256 * ((m + 4) & 15)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < kMfmaPerIter; ++x) {
        const float p = __builtin_amdgcn_exp2f(fmaf(c[PH][x >> 3][x & 7], 1.0e-4f, -0.5f));
        sum += p;
        if (x & 1) {
            f16x2 pk;
            pk[0] = (_Float16)p0;
            pk[1] = (_Float16)p;
            asm volatile("" ::"v"(pk));
        } else {
            p0 = p;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int MIX>
__global__ void __launch_bounds__(threads_of(MIX), 1)
ceiling_kernel(const f16x8* __restrict__ src, float* __restrict__ out, int pairs) {
    typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
    constexpr int NT = threads_of(MIX);
    __shared__ f16x8 lds[kLdsVec];
    const int tid = threadIdx.x;
    for (int i = tid; i < kLdsVec; i += NT) lds[i] = src[i];
    __syncthreads();
    // Operands from the first 2048 vectors of src (tid < 512).
    const f16x8 a = src[tid];
    const f16x8 b0 = src[512 + tid];
    const f16x8 b1 = src[1536 + tid];
    f32x16 c[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) c[h][j][e] = (float)src[1024 + tid][(e + j + h) & 7];
    float sum = 0.0f, p0 = 0.0f;
    // Lane reads base[256 m], m < 16: vectors below 511 + 3840 < kLdsVec.
    const lds_f16x8* base = (const lds_f16x8*)lds + tid;
    f16x8 ring[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ring[r] = MIX >= 1 ? base[256 * r] : a;
    for (int it = 0; it < pairs; ++it) {
        // Opaque per iteration, so the LDS reads are not hoisted out of the loop.
        asm volatile("" : "+v"(base));
        if constexpr (MIX == 6) {
            phased_step<0>(c, ring, b0, base, sum, p0);
            phased_step<1>(c, ring, b0, base, sum, p0);
        } else {
            ceiling_step<MIX, 0>(c, ring, a, b0, b1, base, sum, p0);
            ceiling_step<MIX, 1>(c, ring, a, b0, b1, base, sum, p0);
        }
    }
    float r = sum;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) r += c[h][j][e];
#pragma unroll
    for (int q = 0; q < 4; ++q) r += (float)ring[q][q];
    out[(int64_t)blockIdx.x * 512 + tid] = r;
}

// LDS read probe: TR = 0 reads 16-byte rows (ds_read_b128, lane l reads
// vector l of a 1 KiB block), TR = 1 reads pairs of transposed 8-byte
// fragments (ds_read_b64_tr_b16) at the attention kernels' V^T fragment
// offsets in a chunk-swizzled 64-row x 128-column tile.  Eight reads are in
// flight per wave; each iteration reads 16 KiB per wave (16 x 1 KiB).
template <int NT, int TR>
__global__ void __launch_bounds__(NT, 1)
lds_read_kernel(const u32x4* __restrict__ src, unsigned* __restrict__ out, int iters) {
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    __shared__ u32x4 lds[kLdsVec];
    const int tid = threadIdx.x;
    for (int i = tid; i < kLdsVec; i += NT) lds[i] = src[i];
    __syncthreads();
    const int lane = tid & 63;
    // TR = 0: vector lane + 64 (16 b) of 1 KiB block b, b < 16.
    const lds_u32x4* rb = (const lds_u32x4*)lds + lane;
    // TR = 1: two 8-byte reads per fragment at the attention kernels' V^T
    // fragment offsets in a 64 x 128 tile of 16-bit values (16-byte chunks
    // XOR-swizzled by row): d block mt, rows 4 (lane / 32) + (lane / 4) % 4
    // + 8 r of a 16-row group; fragment f is d block f / 4 of group f % 4.
    const __attribute__((address_space(3))) short* tl = (const __attribute__((address_space(3))) short*)lds;
    const lds_s16x4* tb[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 4 * (lane >> 5) + ((lane >> 2) & 3) + 8 * r;
            const int c = 4 * mt + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            const int sw = ((row & 3) << 2) | ((row >> 2) & 3);
            tb[mt][r] = (const lds_s16x4*)(tl + row * 128 + ((c ^ sw) << 3) + 4 * (lane & 1));
        }
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (int it = 0; it < iters; ++it) {
        // Opaque per iteration, so the reads are not hoisted out of the loop.
        asm volatile("" : "+v"(rb));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) asm volatile("" : "+v"(tb[mt][0]), "+v"(tb[mt][1]));
        u32x4 x[16];
#pragma unroll
        for (int f = 0; f < 16; ++f) {
            if constexpr (TR == 0) {
                x[f] = rb[64 * f];
            } else {
                const int o = (f & 3) * 16 * 128 / 4;  // 16-row group, in 8-byte units
                const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tb[f >> 2][0] + o));
                const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tb[f >> 2][1] + o));
                const auto lo = __builtin_bit_cast(unsigned long long, a);
                const auto hi = __builtin_bit_cast(unsigned long long, b);
                x[f] = u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)};
            }
        }
#pragma unroll
        for (int f = 0; f < 16; ++f) acc ^= x[f];
    }
    out[(int64_t)blockIdx.x * 512 + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

constexpr int kHbmThreads = 256;

constexpr int kReadInFlight = 8;   // loads per thread per round
constexpr int kCopyInFlight = 4;

// Reads n16 16-byte vectors of src; thread t stores the XOR of what it read.
__global__ void __launch_bounds__(kHbmThreads)
hbm_read_kernel(const u32x4* __restrict__ src, int64_t n16, unsigned* __restrict__ out) {
    constexpr int U = kReadInFlight;
    const int64_t t = (int64_t)blockIdx.x * kHbmThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kHbmThreads;
    u32x4 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = u32x4{0u, 0u, 0u, 0u};
    int64_t i = t;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] ^= __builtin_nontemporal_load(src + i + u * stride);
    }
    for (; i < n16; i += stride) a[0] ^= __builtin_nontemporal_load(src + i);
    unsigned r = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) r ^= a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3];
    out[t] = r;
}

// Copies n16 16-byte vectors from src to dst.
__global__ void __launch_bounds__(kHbmThreads)
hbm_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16) {
    constexpr int U = kCopyInFlight;
    const int64_t t = (int64_t)blockIdx.x * kHbmThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kHbmThreads;
    int64_t i = t;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(a[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// Bytes of fp16 source data the probe reads (random values, caller-filled).
int64_t osc_ceiling_src_bytes() { return (int64_t)kLdsVec * 16; }

// MFMAs one launch of mix `mix` issues per workgroup and iteration (x 32768
// FLOP each); 0 for a mix outside 0 to 6.
int osc_ceiling_mfma_per_wg_iter(int mix) {
    if (mix < 0 || mix > 6) return 0;
    return (threads_of(mix) / 64) * 2 * kMfmaPerIter;
}

// Enqueue one launch of mix `mix` (0 to 6) on `stream`: `grid` workgroups of
// `iters` iterations (of 2 x 16 MFMAs per wave) each.  src: device buffer of
// osc_ceiling_src_bytes() bytes; out: device buffer of grid * 512 floats.
// Returns a hipError_t value (hipErrorInvalidValue for a bad argument,
// nothing enqueued).
int osc_ceiling_launch(int mix, const void* src, float* out, int grid, int iters, hipStream_t stream) {
    if (!src || !out || grid < 1 || iters < 1 || mix < 0 || mix > 6) return (int)hipErrorInvalidValue;
    const f16x8* s = static_cast<const f16x8*>(src);
    void* params[] = {(void*)&s, (void*)&out, (void*)&iters};
    const void* fns[] = {reinterpret_cast<const void*>(&ceiling_kernel<0>),
                         reinterpret_cast<const void*>(&ceiling_kernel<1>),
                         reinterpret_cast<const void*>(&ceiling_kernel<2>),
                         reinterpret_cast<const void*>(&ceiling_kernel<3>),
                         reinterpret_cast<const void*>(&ceiling_kernel<4>),
                         reinterpret_cast<const void*>(&ceiling_kernel<5>),
                         reinterpret_cast<const void*>(&ceiling_kernel<6>)};
    return (int)hipLaunchKernel(fns[mix], dim3((unsigned)grid), dim3(threads_of(mix)), params, 0, stream);
}

// LDS read probe: `grid` workgroups of `waves` waves (4 or 8: one or two per
// SIMD), `iters` iterations of 16 KiB per wave, 16-byte row reads (tr = 0)
// or transposed pairs (tr = 1).  src: device buffer of osc_ceiling_src_bytes()
// bytes; out: grid * 512 unsigned.  Returns a hipError_t value
// (hipErrorInvalidValue for a bad argument, nothing enqueued).
int osc_lds_read_launch(int tr, int waves, const void* src, unsigned* out, int grid, int iters,
                        hipStream_t stream) {
    if (!src || !out || grid < 1 || iters < 1 || (tr != 0 && tr != 1) || (waves != 4 && waves != 8))
        return (int)hipErrorInvalidValue;
    const u32x4* s = static_cast<const u32x4*>(src);
    void* params[] = {(void*)&s, (void*)&out, (void*)&iters};
    const void* fn = tr == 0 ? (waves == 4 ? reinterpret_cast<const void*>(&lds_read_kernel<256, 0>)
                                           : reinterpret_cast<const void*>(&lds_read_kernel<512, 0>))
                             : (waves == 4 ? reinterpret_cast<const void*>(&lds_read_kernel<256, 1>)
                                           : reinterpret_cast<const void*>(&lds_read_kernel<512, 1>));
    return (int)hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64 * waves), params, 0, stream);
}

// Streaming read of `bytes` (a multiple of 16) from src: `grid` workgroups of
// 256 threads; out: device buffer of grid * 256 unsigned.  Returns a
// hipError_t value (hipErrorInvalidValue for a bad argument, nothing
// enqueued).
int osc_hbm_read_launch(const void* src, int64_t bytes, unsigned* out, int grid, hipStream_t stream) {
    if (!src || !out || bytes < 16 || bytes % 16 != 0 || grid < 1) return (int)hipErrorInvalidValue;
    const u32x4* s = static_cast<const u32x4*>(src);
    int64_t n16 = bytes / 16;
    void* params[] = {(void*)&s, (void*)&n16, (void*)&out};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(&hbm_read_kernel), dim3((unsigned)grid),
                                dim3(kHbmThreads), params, 0, stream);
}

// Streaming copy of `bytes` (a multiple of 16) from src to dst (which must not
// overlap): `grid` workgroups of 256 threads.  Returns as osc_hbm_read_launch.
int osc_hbm_copy_launch(const void* src, void* dst, int64_t bytes, int grid, hipStream_t stream) {
    if (!src || !dst || bytes < 16 || bytes % 16 != 0 || grid < 1) return (int)hipErrorInvalidValue;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    int64_t n16 = bytes / 16;
    void* params[] = {(void*)&s, (void*)&d, (void*)&n16};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(&hbm_copy_kernel), dim3((unsigned)grid),
                                dim3(kHbmThreads), params, 0, stream);
}

}  // extern "C"
