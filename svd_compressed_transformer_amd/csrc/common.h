// Shared device helpers and host-side status plumbing for the fsvd library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <algorithm>

#include "../../include/fsvd.h"

namespace fsvd {

typedef uint16_t bf16_t;
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ bf16 <-> fp32

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// round-to-nearest-even fp32 -> bf16 (hardware conversion on gfx950)
__device__ __forceinline__ bf16_t f2bf(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(bf16_t, h);
}
// two values in one v_cvt_pk_bf16_f32 (converted one at a time, the halves take a shift and an or
// more); the same rounding as f2bf
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    typedef float f32x2_c __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_c{lo, hi}, bf16x2_v));
}

// a.x*b.x + a.y*b.y + c on two packed bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a), __builtin_bit_cast(bf16x2_v, b), c,
                                           false);
}

// ------------------------------------------------------------------ cross-lane reductions (DPP)

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// every lane of each 16-lane row receives the sum over its row
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x124>(v);  // row_ror:4
    v += dpp_f<0x128>(v);  // row_ror:8
    return v;
}
// Reduce-scatter over each 16-lane row of V (a power of two) per-lane partials.  Four pairing
// levels, each pairing lanes that hold the same set of values and differ in one lane bit:
// row_mirror (bit 3), row_half_mirror (bit 2), quad_perm xor 2 (bit 1), quad_perm xor 1 (bit 0).
// At a level each lane keeps the half of its values selected by its bit and adds the partner's
// copy of that half; once one value is left, the remaining levels add it across the pair.  On
// return v[0 .. rs16_count<V>()) hold this lane's row sums of values rs16_first<V>(lane) + i.
// The pairs of a level are independent, so the DPP operations pipeline instead of forming V
// serial chains.
template <int V>
__host__ __device__ constexpr int rs16_count() { return V >= 16 ? V / 16 : 1; }
template <int V>
__device__ __forceinline__ int rs16_first(int lane) {
    constexpr int lg = V >= 16 ? 4 : (V >= 8 ? 3 : (V >= 4 ? 2 : (V >= 2 ? 1 : 0)));
    return ((lane & 15) >> (4 - lg)) * rs16_count<V>();
}
template <int CTRL, int BIT, int N>
__device__ __forceinline__ void rs16_level(float* v, int lane) {
    if constexpr (N >= 2) {
        const bool up = (lane >> BIT) & 1;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float lo = v[i], hi = v[i + N / 2];
            const float keep = up ? hi : lo, send = up ? lo : hi;
            v[i] = keep + dpp_f<CTRL>(send);
        }
    } else {
        v[0] += dpp_f<CTRL>(v[0]);
    }
}
template <int V>
__device__ __forceinline__ void row16_reduce_scatter(float (&v)[V], int lane) {
    static_assert((V & (V - 1)) == 0, "power of two");
    constexpr int N1 = V, N2 = V >= 2 ? V / 2 : 1, N3 = V >= 4 ? V / 4 : 1, N4 = V >= 8 ? V / 8 : 1;
    rs16_level<0x140, 3, N1>(v, lane);  // row_mirror
    rs16_level<0x141, 2, N2>(v, lane);  // row_half_mirror
    rs16_level<0x4E, 1, N3>(v, lane);   // quad_perm [2,3,0,1]
    rs16_level<0xB1, 0, N4>(v, lane);   // quad_perm [1,0,3,2]
}
__host__ __device__ constexpr int pow2_ceil(int n) { return n <= 1 ? 1 : 2 * pow2_ceil((n + 1) / 2); }

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x128>(v));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
}

// ------------------------------------------------------------------ activations

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }
// erf by the rational approximation of Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (|error| <= 1.5e-7 in exact arithmetic; about 5e-7 absolute when evaluated in
// fp32 near 0), branch-free: one hardware reciprocal, one exp2 and five FMAs.  Accurate far
// beyond the bf16 rounding that follows every GELU here.
__device__ __forceinline__ float erf_as(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
    float p = fmaf(1.061405429f, t, -1.453152027f);
    p = fmaf(p, t, 1.421413741f);
    p = fmaf(p, t, -0.284496736f);
    p = fmaf(p, t, 0.254829592f);
    p *= t;
    const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);  // e^(-x^2)
    return copysignf(fmaf(-p, e, 1.0f), x);
}
// GELU in its erf form: u/2 * (1 + erf(u / sqrt 2))
__device__ __forceinline__ float gelu_f(float u) { return 0.5f * u * (1.0f + erf_as(u * 0.70710678118654752f)); }

// RoPE angle for pair i at position p: p * base^i with base = theta^(-2/D) (computed once on the
// host in double).  base^i by binary exponentiation in double (i < 64: at most 12 products, a few
// ulp), the angle reduced to revolutions in [0, 1) in double so long positions keep fp32 accuracy;
// sin and cos of the revolutions from v_sin_f32 / v_cos_f32, which take revolutions (error
// <= 1.3e-7 on [0, 1), measured on MI355X against fp64).
__device__ __forceinline__ void rope_cs(int64_t p, int i, double base, float* c, float* s) {
    double inv = 1.0, sq = base;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
        if (i & (1 << bit)) inv *= sq;
        sq *= sq;
    }
    const double rev = (double)p * inv * 0.15915494309189533576888376337251;  // revolutions
    const float fr = (float)(rev - floor(rev));
    *s = __builtin_amdgcn_sinf(fr);
    *c = __builtin_amdgcn_cosf(fr);
}

// ------------------------------------------------------------------ pipeline waits

// s_waitcnt on the vector-memory counter only: vmcnt in bits [3:0] and [15:14], expcnt (bits 6:4)
// and lgkmcnt (bits 11:8) left at their maxima so they do not wait
#define FSVD_VMCNT(n) (0x0F70 | ((n) & 0xF) | ((((n) >> 4) & 3) << 14))
__device__ __forceinline__ void wait_vm(int n) {
    // wait until at most n vector-memory operations of this wave are outstanding (n rounded down)
    if (n >= 24) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(24));
    else if (n >= 16) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(16));
    else if (n >= 12) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(12));
    else if (n >= 8) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(8));
    else if (n >= 6) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(6));
    else __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(0));
}

// Workgroup barrier that waits for this wave's LDS operations only.  __syncthreads() would also
// drain every outstanding global load (vmcnt(0)), i.e. the prefetches of later stages, which is
// exactly what the pipeline must keep in flight; stage arrival is ordered by wait_vm() instead.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unchanged
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// device error word: first int32 of every workspace header
__device__ __forceinline__ void set_dev_error(int* err, int bits) {
    if (err) atomicOr(err, bits);
}

}  // namespace fsvd

// ------------------------------------------------------------------ host-side plumbing

namespace fsvd {
// Workspace header: the device error word (int32 at offset 0), then two sets of counters that
// every call leaves at zero: from kWsSplitCounterOff one per tile of a decode projection whose
// reduction is split over workgroups (at most 128 tiles), from kWsCounterOff one per (sequence, kv
// head) of the decode attention.  Only the kernels that count write them.
constexpr size_t kWsHeader = 4096;
constexpr size_t kWsSplitCounterOff = 64;
constexpr int kWsSplitCounters = 128;
constexpr size_t kWsCounterOff = kWsSplitCounterOff + 4 * kWsSplitCounters;
constexpr int kWsCounters = (int)((kWsHeader - kWsCounterOff) / 4);

void set_error(const char* fmt, ...);
fsvd_status_t fail(fsvd_status_t s, const char* fmt, ...);

inline bool aligned16(const void* p) { return (((uintptr_t)p) & 15u) == 0; }
inline size_t esize(fsvd_dtype_t t) { return t == FSVD_F32 ? 4 : 2; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// status of the last kernel launch
fsvd_status_t check_launch(const char* what);

// Raises kernel fn's dynamic LDS limit to at least `bytes` on the current device. The attribute
// is set once per (kernel, device) and size; safe to call from several host threads.
fsvd_status_t allow_dynamic_lds(const void* fn, size_t bytes, const char* what);
}  // namespace fsvd

#define FSVD_REQUIRE(cond, ...)                                  \
    do {                                                         \
        if (!(cond)) return ::fsvd::fail(FSVD_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)
