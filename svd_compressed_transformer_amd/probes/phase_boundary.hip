// Measurement probe (not part of the library): what a phase boundary of the decode layer-step costs
// as a kernel boundary inside a graph, against a grid barrier inside one persistent kernel.
//
// One layer-step is modelled as 10 dependent phases that stream the byte counts of the Llama-7B
// decode kernels at batch 4 (Q/K/V phase 1 and 2, attention and its merge, O, gate|up and down
// phases 1 and 2) with 16-byte non-temporal loads; every phase first reads the whole 32 KB
// activation the previous phase wrote (as each projection reads its full input vector) and then
// writes its own.  Four copies of the weights rotate, as in the benchmark, so nothing is served from
// the 256 MB Infinity Cache.
//
//   kernels:  one kernel per phase (grid sized like the decode kernels), one graph per layer-step;
//   persist:  one kernel per layer-step, one workgroup per CU, a two-level grid barrier between
//             phases (a counter per XCD, then one global counter; agent-scope relaxed atomics);
//             the activation is exchanged with 16-byte loads and stores carrying the agent-scope
//             bit (sc1, as agent-scope atomics do), so no cache-wide fence is needed;
//   prefetch: persist, with each workgroup issuing the first loads of its next-phase share before
//             it arrives at the barrier.
// The persistent variants stream with 4 loads in flight per thread, then with 16 (one workgroup
// per CU holds fewer loads in flight than the many-workgroup kernels).
//   lds_prefetch: contiguous shares per workgroup, the first 128 KB of the next phase's share
//             prefetched into LDS with global -> LDS loads while the current phase finishes.
//   kernels9: the layer-step with the attention partitions merged inside the attention kernel (the
//             2.2 MB merge phase gone, the attention phase at 512 workgroups); then the same 9
//             phases with every grid at 512, 1024 and 2048 workgroups.
//   kernels9_mall: the 9 phases at the decode grids, each kernel reading 25 / 50 / 100% of the next
//             phase's bytes with ordinary loads after its own stream (into the Infinity Cache).
//   kernels9_pairs: the 9 phases with each projection's two phases in one launch on separate
//             workgroups (pair_kernel), polling with s_sleep 1, 16 and 64 between reads.
// A first argument n runs the variants from n on.
//
// Every activation word encodes (layer-step, phase, slot); each reader counts the words it does not
// find as expected, which the run reports (a stale read would show there).  Every spin is bounded:
// past the limit the kernel sets an error flag and exits, so it always terminates.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include <vector>
#include <algorithm>
#include <cstdlib>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); return 1; } } while (0)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int P = 10;            // phases per layer-step
constexpr int ACT = 8192;        // activation words (32 KB)
constexpr int NL = 4;            // weight copies rotated
constexpr int PF = 8;            // prefetched 16-byte vectors per thread
// phase sizes in MB (Llama-7B decode at batch 4, algorithmic bytes) and the decode kernels' grids
constexpr double MB[P] = {40.26, 40.26, 138.45, 2.2, 13.42, 13.42, 26.84, 72.13, 36.06, 13.42};
constexpr int GRID[P] = {1248, 1536, 4096, 128, 416, 512, 832, 2752, 416, 512};
constexpr int GRID9[P] = {1248, 1536, 512, 0, 416, 512, 832, 2752, 416, 512};  // 0: phase not run

struct Phases {
    const u32x4* w[P];
    long n16[P];
};

__device__ __forceinline__ uint32_t act_word(uint32_t step, int p, int slot) {
    return (step * 16u + (uint32_t)p) * 0x9E3779B1u ^ (uint32_t)slot;
}

// Reads the whole activation of phase p - 1 (16-byte loads) and counts unexpected words.  COHERENT:
// the loads carry the agent-scope bit (sc1), as an agent-scope atomic load does, so they do not
// return a line another XCD's L2 holds stale; otherwise plain loads (a kernel boundary orders them).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}
template <bool COHERENT>
__device__ __forceinline__ void read_act(const uint32_t* act, uint32_t step, int p, unsigned* bad) {
    if (p == 0) return;
    const uint32_t* a = act + (p - 1) * ACT;
    unsigned miss = 0;
    for (int i = threadIdx.x; i < ACT / 4; i += blockDim.x) {
        u32x4 v;
        if (COHERENT) v = __builtin_amdgcn_raw_buffer_load_b128(rsrc(a), i * 16, 0, 16);
        else v = reinterpret_cast<const u32x4*>(a)[i];
        miss += (v.x != act_word(step, p - 1, 4 * i)) + (v.y != act_word(step, p - 1, 4 * i + 1)) +
                (v.z != act_word(step, p - 1, 4 * i + 2)) + (v.w != act_word(step, p - 1, 4 * i + 3));
    }
    if (miss) atomicAdd(bad, miss);
}
template <bool COHERENT>
__device__ __forceinline__ void write_act(uint32_t* act, uint32_t step, int p) {
    uint32_t* out = act + p * ACT;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < ACT / 4; i += gridDim.x * blockDim.x) {
        const u32x4 v = {act_word(step, p, 4 * i), act_word(step, p, 4 * i + 1), act_word(step, p, 4 * i + 2),
                         act_word(step, p, 4 * i + 3)};
        if (COHERENT) __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(out), i * 16, 0, 16);
        else reinterpret_cast<u32x4*>(out)[i] = v;
    }
}

// one phase as its own kernel: activation in (that of phase p - skip - 1), share of the stream,
// activation slice out
__global__ __launch_bounds__(256) void phase_kernel(const u32x4* __restrict__ w, long n16, uint32_t* act, int p,
                                                    uint32_t step, unsigned* bad, uint32_t* sink, int skip = 0) {
    read_act<false>(act, step, p - skip, bad);
    const long stride = (long)gridDim.x * blockDim.x;
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(w + i), b = __builtin_nontemporal_load(w + i + stride);
        const u32x4 c = __builtin_nontemporal_load(w + i + 2 * stride), d = __builtin_nontemporal_load(w + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(w + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x12345678u) sink[blockIdx.x & 63] = acc;  // keeps the loads live
    write_act<false>(act, step, p);
}

// phase_kernel, then a share of the first pn16 vectors of the NEXT phase's bytes read with ordinary
// (allocating) loads after this phase's own stream: the memory-side Infinity Cache holds them when
// the next kernel starts, and this kernel's tail keeps HBM busy.
__global__ __launch_bounds__(256) void phase_mall_kernel(const u32x4* __restrict__ w, long n16, uint32_t* act, int p,
                                                         uint32_t step, unsigned* bad, uint32_t* sink, int skip,
                                                         const u32x4* __restrict__ pw, long pn16) {
    read_act<false>(act, step, p - skip, bad);
    const long stride = (long)gridDim.x * blockDim.x;
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(w + i), b = __builtin_nontemporal_load(w + i + stride);
        const u32x4 c = __builtin_nontemporal_load(w + i + 2 * stride), d = __builtin_nontemporal_load(w + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(w + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    write_act<false>(act, step, p);
    i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < pn16; i += 4 * stride) {
        const u32x4 a = pw[i], b = pw[i + stride], c = pw[i + 2 * stride], d = pw[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < pn16; i += stride) {
        const u32x4 a = pw[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x12345678u) sink[blockIdx.x & 63] = acc;  // keeps the loads live
}

// Two dependent phases in one launch, on separate workgroups: blocks [0, g1) do phase p (read the
// activation the previous kernel wrote, stream their share of w1, write their activation slice with
// agent-scope stores, wait for those stores, count themselves); blocks [g1, g1 + g2) first issue
// every load of their share of w2 (at most PF 16-byte vectors per thread, the whole share at the
// decode kernels' grids), then wait until all g1 blocks have counted, then read phase p's activation
// with agent-scope loads and fold in the prefetched vectors; the last of them resets both counters.
// Lower block indices are dispatched first, so the waiting blocks never hold back a phase-p block;
// the wait is bounded (past spin_limit the error flag is set and the block exits).
template <int SLEEP>
__global__ __launch_bounds__(256) void pair_kernel(const u32x4* __restrict__ w1, long n1, const u32x4* __restrict__ w2,
                                                   long n2, int g1, uint32_t* act, int p, int skip, uint32_t step,
                                                   unsigned* cnt, unsigned* bad, unsigned* err, uint32_t* sink,
                                                   unsigned spin_limit) {
    uint32_t acc = 0;
    const int g2 = gridDim.x - g1;
    if ((int)blockIdx.x < g1) {
        read_act<false>(act, step, p - skip, bad);
        const long stride = (long)g1 * blockDim.x;
        long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
        for (; i + 3 * stride < n1; i += 4 * stride) {
            const u32x4 a = __builtin_nontemporal_load(w1 + i), b = __builtin_nontemporal_load(w1 + i + stride);
            const u32x4 c = __builtin_nontemporal_load(w1 + i + 2 * stride), d = __builtin_nontemporal_load(w1 + i + 3 * stride);
            acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
        }
        for (; i < n1; i += stride) {
            const u32x4 a = __builtin_nontemporal_load(w1 + i);
            acc ^= a.x ^ a.y ^ a.z ^ a.w;
        }
        // this block's slice of the activation: blocks stride over the words as the phase kernels do
        uint32_t* out = act + p * ACT;
        for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < ACT / 4; j += g1 * blockDim.x) {
            const u32x4 v = {act_word(step, p, 4 * j), act_word(step, p, 4 * j + 1), act_word(step, p, 4 * j + 2),
                             act_word(step, p, 4 * j + 3)};
            __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(out), j * 16, 0, 16);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        const int b2 = blockIdx.x - g1;
        const long stride = (long)g2 * blockDim.x;
        const long t0 = (long)b2 * blockDim.x + threadIdx.x;
        u32x4 pf[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) pf[j] = __builtin_nontemporal_load(w2 + std::min(t0 + j * stride, n2 - 1));
        __shared__ int ok;
        if (threadIdx.x == 0) {
            unsigned it = 0;
            ok = 1;
            while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)g1) {
                if (++it > spin_limit) { atomicOr(err, 1u); ok = 0; break; }
                __builtin_amdgcn_s_sleep(SLEEP);
            }
        }
        __syncthreads();
        if (!ok) return;
        read_act<true>(act, step, p + 1, bad);
#pragma unroll
        for (int j = 0; j < PF; ++j)
            if (t0 + j * stride < n2) acc ^= pf[j].x ^ pf[j].y ^ pf[j].z ^ pf[j].w;
        for (long i = t0 + (long)PF * stride; i < n2; i += stride) {
            const u32x4 a = __builtin_nontemporal_load(w2 + i);
            acc ^= a.x ^ a.y ^ a.z ^ a.w;
        }
        uint32_t* out = act + (p + 1) * ACT;
        for (int j = b2 * blockDim.x + threadIdx.x; j < ACT / 4; j += g2 * blockDim.x)
            reinterpret_cast<u32x4*>(out)[j] = u32x4{act_word(step, p + 1, 4 * j), act_word(step, p + 1, 4 * j + 1),
                                                     act_word(step, p + 1, 4 * j + 2), act_word(step, p + 1, 4 * j + 3)};
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add(cnt + 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == (unsigned)g2) {  // every block has passed its wait: reset for the next launch
                __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(cnt + 32, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (acc == 0x12345678u) sink[blockIdx.x & 63] = acc;
}

// two-level barrier number k (k = 1, 2, ...): XCD counter, the last arriver of an XCD bumps the
// global counter; all wait for the global count of k * 8.  Before arriving, each wave waits until its
// activation stores have completed but leaves its last PENDING loads (the prefetch, issued after the
// stores) in flight: s_waitcnt vmcnt(PENDING) and a bare s_barrier, since __syncthreads() would
// drain every outstanding load.
template <int PENDING>
__device__ __forceinline__ bool grid_barrier(unsigned* xcnt, unsigned* gcnt, unsigned k, unsigned per_xcd,
                                             unsigned spin_limit, unsigned* err) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (PENDING & 0xF) | (((PENDING >> 4) & 3) << 14));  // vmcnt(PENDING)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    bool ok = true;
    if (threadIdx.x == 0) {
        const unsigned x = blockIdx.x & 7;
        const unsigned old = __hip_atomic_fetch_add(xcnt + x * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1 == k * per_xcd) __hip_atomic_fetch_add(gcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned it = 0;
        while (__hip_atomic_load(gcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < k * 8u) {
            if (++it > spin_limit) { atomicOr(err, 1u); ok = false; break; }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    return ok && !__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool PREFETCH, int DEPTH>
__global__ __launch_bounds__(256, 1) void persist_kernel(Phases ph, uint32_t* act, uint32_t step, unsigned* xcnt,
                                                         unsigned* gcnt, unsigned kbase, unsigned per_xcd,
                                                         unsigned* bad, unsigned* err, uint32_t* sink,
                                                         unsigned spin_limit) {
    const long stride = (long)gridDim.x * blockDim.x;
    const long t0 = (long)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    u32x4 pf[PF];
    int npf = 0;  // prefetched vectors of the current phase
    for (int p = 0; p < P; ++p) {
        if (p > 0) {
            if (PREFETCH) {  // first PF loads of this phase's share, issued before the barrier;
                             // indexes past the phase re-read its last vector (masked when consumed)
#pragma unroll
                for (int j = 0; j < PF; ++j)
                    pf[j] = __builtin_nontemporal_load(ph.w[p] + std::min(t0 + j * stride, ph.n16[p] - 1));
                npf = PF;
            }
            if (!grid_barrier<PREFETCH ? PF : 0>(xcnt, gcnt, kbase + p, per_xcd, spin_limit, err)) return;
        }
        read_act<true>(act, step, p, bad);
        const u32x4* w = ph.w[p];
        const long n16 = ph.n16[p];
        long i = t0;
        if (PREFETCH && p > 0) {
#pragma unroll
            for (int j = 0; j < PF; ++j)
                if (t0 + j * stride < n16) acc ^= pf[j].x ^ pf[j].y ^ pf[j].z ^ pf[j].w;
            i += (long)npf * stride;
        }
        // one workgroup per CU: DEPTH independent loads per thread in flight to cover the latency
        for (; i + (DEPTH - 1) * stride < n16; i += DEPTH * stride) {
            u32x4 v[DEPTH];
#pragma unroll
            for (int j = 0; j < DEPTH; ++j) v[j] = __builtin_nontemporal_load(w + i + j * stride);
#pragma unroll
            for (int j = 0; j < DEPTH; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
        }
        for (; i < n16; i += stride) {
            const u32x4 a = __builtin_nontemporal_load(w + i);
            acc ^= a.x ^ a.y ^ a.z ^ a.w;
        }
        write_act<true>(act, step, p);
    }
    if (acc == 0x12345678u) sink[blockIdx.x & 63] = acc;
}

// persist, with each workgroup owning a contiguous share of every phase and prefetching the first
// LDSV vectors of its next-phase share straight into LDS (global -> LDS loads, asynchronous) as soon
// as it has consumed the current phase's prefetched part: the next phase's first 128 KB per
// workgroup (32 MB over the chip, whole phases for the small ones) stream in while the current phase
// finishes and the barrier completes.
constexpr int LDSV = 8192;  // 16-byte vectors per workgroup (128 KB)
typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(256, 1) void persist_lds_kernel(Phases ph, uint32_t* act, uint32_t step, unsigned* xcnt,
                                                             unsigned* gcnt, unsigned kbase, unsigned per_xcd,
                                                             unsigned* bad, unsigned* err, uint32_t* sink,
                                                             unsigned spin_limit) {
    extern __shared__ u32x4 lbuf[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long G = gridDim.x, b = blockIdx.x;
    uint32_t acc = 0;
    auto share = [&](int p, long* s0, long* cnt) {
        const long per = (ph.n16[p] + G - 1) / G;
        *s0 = std::min(b * per, ph.n16[p]);
        *cnt = std::min(per, ph.n16[p] - *s0);
    };
    auto prefetch = [&](int p) -> int {
        long s0, cnt;
        share(p, &s0, &cnt);
        const int nv = (int)std::min<long>(cnt, LDSV);
        for (int c = wave; c * 64 < nv; c += 4) {  // wave-uniform 1 KB chunks; past nv re-read the last
            const long vi = std::min(s0 + c * 64 + lane, s0 + nv - 1);
            __builtin_amdgcn_global_load_lds((const void*)(ph.w[p] + vi), (lds_void*)(lbuf + c * 64), 16, 0, 0);
        }
        return nv;
    };
    int nv = prefetch(0);
    for (int p = 0; p < P; ++p) {
        if (p > 0) {
            if (!grid_barrier<0>(xcnt, gcnt, kbase + p, per_xcd, spin_limit, err)) return;
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the prefetch of phase 0 has landed
            __builtin_amdgcn_s_barrier();
        }
        asm volatile("" ::: "memory");
        read_act<true>(act, step, p, bad);
        for (int i = tid; i < nv; i += 256) {
            const u32x4 a = lbuf[i];
            acc ^= a.x ^ a.y ^ a.z ^ a.w;
        }
        long s0, cnt;
        share(p, &s0, &cnt);
        const int cur = nv;
        __syncthreads();  // every wave is done with this phase's LDS part
        if (p + 1 < P) nv = prefetch(p + 1);
        const u32x4* w = ph.w[p] + s0;
        long i = cur + tid;
        for (; i + 3 * 256 < cnt; i += 4 * 256) {
            const u32x4 a0 = __builtin_nontemporal_load(w + i), a1 = __builtin_nontemporal_load(w + i + 256);
            const u32x4 a2 = __builtin_nontemporal_load(w + i + 512), a3 = __builtin_nontemporal_load(w + i + 768);
            acc ^= a0.x ^ a0.y ^ a0.z ^ a0.w ^ a1.x ^ a1.y ^ a1.z ^ a1.w ^ a2.x ^ a2.y ^ a2.z ^ a2.w ^ a3.x ^ a3.y ^ a3.z ^ a3.w;
        }
        for (; i < cnt; i += 256) {
            const u32x4 a0 = __builtin_nontemporal_load(w + i);
            acc ^= a0.x ^ a0.y ^ a0.z ^ a0.w;
        }
        write_act<true>(act, step, p);
    }
    if (acc == 0x12345678u) sink[blockIdx.x & 63] = acc;
}

int main(int argc, char** argv) {
    const int first = argc > 1 ? atoi(argv[1]) : 0;  // first variant to run
    int dev = 0, cus = 0;
    CK(hipGetDevice(&dev));
    CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    int occ0 = 0, occ1 = 0;
    CK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ0, persist_kernel<false, 16>, 256, 0));
    CK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ1, persist_kernel<true, 16>, 256, 0));
    printf("CUs %d, resident persistent blocks per CU %d / %d\n", cus, occ0, occ1);
    if (occ0 < 1 || occ1 < 1 || cus % 8 != 0) return 1;
    const unsigned per_xcd = cus / 8;

    long n16[P], total16 = 0;
    for (int p = 0; p < P; ++p) {
        n16[p] = ((long)(MB[p] * 1e6 / 16) + 4095) / 4096 * 4096;
        total16 += n16[p];
    }
    u32x4* w;
    CK(hipMalloc(&w, (size_t)total16 * NL * 16));
    CK(hipMemset(w, 0x5a, (size_t)total16 * NL * 16));
    uint32_t *act, *sink;
    unsigned *xcnt, *gcnt, *bad, *err;
    CK(hipMalloc(&act, (size_t)P * ACT * 4)); CK(hipMalloc(&sink, 64 * 4));
    unsigned* pcnt;
    CK(hipMalloc(&pcnt, 64 * 4));
    CK(hipMalloc(&xcnt, 8 * 32 * 4)); CK(hipMalloc(&gcnt, 4)); CK(hipMalloc(&bad, 4)); CK(hipMalloc(&err, 4));
    Phases ph[NL];
    for (int l = 0; l < NL; ++l) {
        long off = (long)l * total16;
        for (int p = 0; p < P; ++p) { ph[l].w[p] = w + off; ph[l].n16[p] = n16[p]; off += n16[p]; }
    }
    hipStream_t st; CK(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
    hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
    const int steps = 256;  // layer-steps timed per run (64 per weight copy)
    const double bytes = (double)total16 * 16;

    // kernels: one graph per weight copy, 10 kernels each; the step index is a kernel argument, so
    // each copy's graph is captured with a fixed step and the activation check tolerates reuse by
    // writing before reading within the same graph (phase 0 reads nothing)
    CK(hipFuncSetAttribute((const void*)persist_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDSV * 16));
    constexpr int NV = 16;
    constexpr double MALL_F[3] = {0.25, 0.5, 1.0};  // variants 10-12: fraction of the next phase prefetched
    for (int variant = first; variant < NV; ++variant) {
        std::vector<float> v;
        for (int rep = 0; rep < 5; ++rep) {
            CK(hipMemsetAsync(xcnt, 0, 8 * 32 * 4, st)); CK(hipMemsetAsync(gcnt, 0, 4, st));
            CK(hipMemsetAsync(pcnt, 0, 64 * 4, st));
            CK(hipMemsetAsync(bad, 0, 4, st)); CK(hipMemsetAsync(err, 0, 4, st));
            CK(hipStreamSynchronize(st));
            std::vector<hipGraphExec_t> ge;
            const bool graphs = variant == 0 || variant >= 6;
            if (graphs) {
                for (int l = 0; l < NL; ++l) {
                    hipGraph_t g;
                    CK(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
                    for (int p = 0, skip = 0; p < P; ++p) {
                        if (variant == 0) {
                            phase_kernel<<<GRID[p], 256, 0, st>>>(ph[l].w[p], n16[p], act, p, (uint32_t)l, bad, sink);
                            continue;
                        }
                        if (GRID9[p] == 0) { skip = 1; continue; }
                        if (variant >= 13) {  // phase pairs in one launch each; the attention alone
                            if (p == 2) {
                                phase_kernel<<<GRID9[p], 256, 0, st>>>(ph[l].w[p], n16[p], act, p, (uint32_t)l, bad, sink, 0);
                            } else if (p % 2 == 0) {
                                auto k = variant == 13 ? pair_kernel<1> : variant == 14 ? pair_kernel<16> : pair_kernel<64>;
                                k<<<GRID9[p] + GRID9[p + 1], 256, 0, st>>>(
                                    ph[l].w[p], n16[p], ph[l].w[p + 1], n16[p + 1], GRID9[p], act, p, skip, (uint32_t)l,
                                    pcnt, bad, err, sink, 1u << 20);
                            }
                            skip = 0;
                            continue;
                        }
                        if (variant >= 10) {  // next phase: p + 1 (past the skipped merge), or the next copy's phase 0
                            int q = p + 1;
                            if (q < P && GRID9[q] == 0) ++q;
                            const u32x4* pw = q < P ? ph[l].w[q] : ph[(l + 1) % NL].w[0];
                            const long pn = (long)(MALL_F[variant - 10] * (double)(q < P ? n16[q] : n16[0]));
                            phase_mall_kernel<<<GRID9[p], 256, 0, st>>>(ph[l].w[p], n16[p], act, p, (uint32_t)l, bad,
                                                                        sink, skip, pw, pn);
                            skip = 0;
                            continue;
                        }
                        const int grid = variant == 6 ? GRID9[p] : variant == 7 ? 512 : variant == 8 ? 1024 : 2048;
                        phase_kernel<<<grid, 256, 0, st>>>(ph[l].w[p], n16[p], act, p, (uint32_t)l, bad, sink, skip);
                        skip = 0;
                    }
                    CK(hipStreamEndCapture(st, &g));
                    hipGraphExec_t x;
                    CK(hipGraphInstantiate(&x, g, nullptr, nullptr, 0));
                    CK(hipGraphDestroy(g));
                    ge.push_back(x);
                }
                for (int l = 0; l < NL; ++l) CK(hipGraphLaunch(ge[l], st));  // warm
            }
            CK(hipStreamSynchronize(st));
            CK(hipEventRecord(e0, st));
            for (int s = 0; s < steps; ++s) {
                const int l = s % NL;
                if (graphs) {
                    CK(hipGraphLaunch(ge[l], st));
                } else {
                    const unsigned kbase = (unsigned)s * (P - 1);  // barriers before this step
                    if (variant == 1)
                        persist_kernel<false, 4><<<cus, 256, 0, st>>>(ph[l], act, (uint32_t)s, xcnt, gcnt, kbase,
                                                                      per_xcd, bad, err, sink, 1u << 20);
                    else if (variant == 2)
                        persist_kernel<true, 4><<<cus, 256, 0, st>>>(ph[l], act, (uint32_t)s, xcnt, gcnt, kbase,
                                                                     per_xcd, bad, err, sink, 1u << 20);
                    else if (variant == 3)
                        persist_kernel<false, 16><<<cus, 256, 0, st>>>(ph[l], act, (uint32_t)s, xcnt, gcnt, kbase,
                                                                       per_xcd, bad, err, sink, 1u << 20);
                    else if (variant == 4)
                        persist_kernel<true, 16><<<cus, 256, 0, st>>>(ph[l], act, (uint32_t)s, xcnt, gcnt, kbase,
                                                                      per_xcd, bad, err, sink, 1u << 20);
                    else
                        persist_lds_kernel<<<cus, 256, LDSV * 16, st>>>(ph[l], act, (uint32_t)s, xcnt, gcnt, kbase,
                                                                        per_xcd, bad, err, sink, 1u << 20);
                }
            }
            CK(hipEventRecord(e1, st));
            CK(hipEventSynchronize(e1));
            float ms; CK(hipEventElapsedTime(&ms, e0, e1));
            unsigned hb = 0, he = 0;
            CK(hipMemcpy(&hb, bad, 4, hipMemcpyDeviceToHost)); CK(hipMemcpy(&he, err, 4, hipMemcpyDeviceToHost));
            for (auto& x : ge) CK(hipGraphExecDestroy(x));
            if (he) { printf("spin limit reached (variant %d)\n", variant); return 2; }
            if (hb) printf("variant %d rep %d: %u activation words not as expected\n", variant, rep, hb);
            v.push_back(ms);
        }
        std::sort(v.begin(), v.end());
        const double us = v[2] * 1e3 / steps;
        const char* name[NV] = {"kernels", "persist", "prefetch", "persist_depth16", "prefetch_depth16", "lds_prefetch",
                                "kernels9", "kernels9_grid512", "kernels9_grid1024", "kernels9_grid2048",
                                "kernels9_mall25", "kernels9_mall50", "kernels9_mall100", "kernels9_pairs",
                                "kernels9_pairs_sleep16", "kernels9_pairs_sleep64"};
        const double vb = variant >= 6 ? bytes - (double)n16[3] * 16 : bytes;  // the 9 phases skip the merge's bytes
        printf("{\"variant\": \"%s\", \"us_per_layer_step\": %.2f, \"gbs\": %.1f, \"of_8tbs\": %.3f}\n", name[variant], us,
               vb / (us * 1e-6) / 1e9, vb / (us * 1e-6) / 8e12);
    }
    return 0;
}
