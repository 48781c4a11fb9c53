// Measurement probe (not part of the library): the cost of a grid-wide barrier on this part, the
// primitive a persistent decode-layer kernel (one workgroup per CU, phases separated by barriers
// instead of kernel boundaries) would need.  G workgroups (one per CU, then half and a quarter of
// the CUs) pass 200 barriers on one global counter (agent-scope relaxed atomic add, then polling
// agent-scope loads); mode "fence+atomic" adds the release / acquire fences that make each
// workgroup's stores visible across the XCDs before the next phase reads them.  The per-barrier
// time is (201 barriers - 1 barrier) / 200.  Every spin is bounded: past the limit the kernel sets
// an error flag and exits, so it always terminates.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#include <algorithm>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); return 1; } } while (0)

template <int MODE>
__global__ __launch_bounds__(256) void barrier_kernel(unsigned* count, unsigned* err, int nb, unsigned spin_limit) {
    const unsigned G = gridDim.x;
    for (int b = 0; b < nb; ++b) {
        __syncthreads();
        if (threadIdx.x == 0) {
            if (MODE == 1) __threadfence();  // release: this workgroup's writes visible device-wide
            __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned target = (unsigned)(b + 1) * G;
            unsigned it = 0;
            while (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                if (++it > spin_limit) { atomicOr(err, 1u); break; }
                __builtin_amdgcn_s_sleep(1);
            }
            if (MODE == 1) __threadfence();  // acquire
        }
        __syncthreads();
        if (*(volatile unsigned*)err) return;
    }
}

int main() {
    int dev = 0, cus = 0;
    CK(hipGetDevice(&dev));
    CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    int occ = 0;
    CK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, barrier_kernel<0>, 256, 0));
    printf("CUs %d, resident blocks per CU %d\n", cus, occ);
    if (occ < 1) return 1;
    unsigned *count, *err;
    CK(hipMalloc(&count, 4)); CK(hipMalloc(&err, 4));
    hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
    const int nbs[2] = {1, 201};
    for (int mode = 0; mode < 2; ++mode) {
        for (int G : {cus, cus / 2, cus / 4}) {
            float t[2];
            for (int k = 0; k < 2; ++k) {
                std::vector<float> v;
                for (int rep = 0; rep < 5; ++rep) {
                    CK(hipMemset(count, 0, 4)); CK(hipMemset(err, 0, 4));
                    CK(hipDeviceSynchronize());
                    CK(hipEventRecord(e0, 0));
                    if (mode == 0) barrier_kernel<0><<<G, 256>>>(count, err, nbs[k], 1u << 20);
                    else barrier_kernel<1><<<G, 256>>>(count, err, nbs[k], 1u << 20);
                    CK(hipEventRecord(e1, 0));
                    CK(hipEventSynchronize(e1));
                    float ms; CK(hipEventElapsedTime(&ms, e0, e1));
                    unsigned h = 0; CK(hipMemcpy(&h, err, 4, hipMemcpyDeviceToHost));
                    if (h) { printf("spin limit reached (mode %d G %d)\n", mode, G); return 2; }
                    v.push_back(ms);
                }
                std::sort(v.begin(), v.end());
                t[k] = v[2];
            }
            printf("{\"mode\": \"%s\", \"workgroups\": %d, \"us_per_barrier\": %.3f, \"launch_us\": %.2f}\n",
                   mode ? "fence+atomic" : "atomic", G, (t[1] - t[0]) * 1e3 / 200.0, t[0] * 1e3);
        }
    }
    return 0;
}
