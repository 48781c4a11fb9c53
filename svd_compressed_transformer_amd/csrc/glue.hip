// Small kernels around the projections: the offline factor prepack, BERT-style post-norm
// LayerNorm, the cache-length advance, the RMSNorm preparation of the MFMA (prefill) path and a
// tiled transpose (weight layouts of the Swift-SVD factor production).
#include "kernels.h"

namespace fsvd {

namespace {

// prepack: copy one item (rows x cols, 16-bit or 32-bit elements) into dst rows
// [row0, row0 + rows_pad) x [0, cols_pad), zero-filling the pad area.  One thread per element.
template <typename E>
__global__ void prepack_kernel(E* dst, int64_t ld_dst, int64_t cols_pad, int64_t row0, const E* src, int64_t rows,
                               int64_t cols, int64_t ld_src, int64_t rows_pad, const E* col_scale) {
    const int64_t total = rows_pad * cols_pad;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / cols_pad, c = i - r * cols_pad;
        E v = (r < rows && c < cols) ? src[r * ld_src + c] : E(0);
        if (col_scale != nullptr && c < cols) {
            // column c scaled by col_scale[c] in fp32, rounded to nearest even
            if constexpr (sizeof(E) == 2) {
                v = f2bf(bf2f(v) * bf2f(col_scale[c]));
            } else {
                v = __float_as_uint(__uint_as_float(v) * __uint_as_float(col_scale[c]));
            }
        }
        dst[(row0 + r) * ld_dst + c] = v;
    }
}

// y = LayerNorm(x + res) * g + b over rows of width d; one workgroup per row, fp32 statistics
__global__ __launch_bounds__(256) void layernorm_kernel(const bf16_t* x, const bf16_t* res, const bf16_t* g,
                                                        const bf16_t* bta, float eps, int64_t d, bf16_t* y) {
    const int64_t row = blockIdx.x;
    const bf16_t* xr = x + row * d;
    const bf16_t* rr = res ? res + row * d : nullptr;
    extern __shared__ float buf[];  // d floats
    __shared__ float red[8];
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < d; i += 256) {
        const float v = bf2f(xr[i]) + (rr ? bf2f(rr[i]) : 0.f);
        buf[i] = v;
        s += v;
    }
    s = wave_sum(s);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = s;
    __syncthreads();
    const float mean = (red[0] + red[1] + red[2] + red[3]) / (float)d;
    float q = 0.f;
    for (int64_t i = threadIdx.x; i < d; i += 256) {
        const float dv = buf[i] - mean;
        q += dv * dv;
    }
    q = wave_sum(q);
    if ((threadIdx.x & 63) == 0) red[4 + w] = q;
    __syncthreads();
    const float rstd = 1.0f / sqrtf((red[4] + red[5] + red[6] + red[7]) / (float)d + eps);
    for (int64_t i = threadIdx.x; i < d; i += 256)
        y[row * d + i] = f2bf((buf[i] - mean) * rstd * bf2f(g[i]) + bf2f(bta[i]));
}

// The same LayerNorm with one wave per row (4 rows per workgroup) when d is a multiple of 8 and the
// operands are 16-byte aligned: 16-byte loads and stores, the row (x + res in fp32) held in
// registers, NV 16-byte vectors per lane at most (d <= 512 * NV).  Statistics in two passes over
// the registers, reduced across the wave with DPP and lane reads.
template <int NV>
__global__ __launch_bounds__(256) void layernorm_wave_kernel(const bf16_t* x, const bf16_t* res, const bf16_t* g,
                                                             const bf16_t* bta, float eps, int64_t M, int64_t d,
                                                             bf16_t* y) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;  // whole wave
    const int lane = threadIdx.x & 63;
    const int nv = (int)(d / 8);
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * d);
    const u32x4* rr = res ? reinterpret_cast<const u32x4*>(res + row * d) : nullptr;
    const u32x4* gv = reinterpret_cast<const u32x4*>(g);
    const u32x4* bv = reinterpret_cast<const u32x4*>(bta);
    u32x4 gg[NV], bb[NV];  // loaded with the row: one round trip to memory less before the stores
    float v[NV][8];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
        if (c < nv) {
            gg[i] = gv[c];
            bb[i] = bv[c];
            const u32x4 a = xr[c];
            const uint32_t ea[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[i][2 * e] = bf_lo(ea[e]);
                v[i][2 * e + 1] = bf_hi(ea[e]);
            }
            if (rr) {
                const u32x4 b = rr[c];
                const uint32_t eb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[i][2 * e] += bf_lo(eb[e]);
                    v[i][2 * e + 1] += bf_hi(eb[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) s += v[i][e];
        }
    }
    const float mean = wave_sum(s) / (float)d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (lane + 64 * i < nv)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dv = v[i][e] - mean;
                q += dv * dv;
            }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
    u32x4* yr = reinterpret_cast<u32x4*>(y + row * d);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        if (c < nv) {
            const uint32_t eg[4] = {gg[i].x, gg[i].y, gg[i].z, gg[i].w}, eb[4] = {bb[i].x, bb[i].y, bb[i].z, bb[i].w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack_bf2((v[i][2 * e] - mean) * rstd * bf_lo(eg[e]) + bf_lo(eb[e]),
                                (v[i][2 * e + 1] - mean) * rstd * bf_hi(eg[e]) + bf_hi(eb[e]));
            yr[c] = u32x4{o[0], o[1], o[2], o[3]};
        }
    }
}

__global__ void seqlens_advance_kernel(int32_t* sl, int64_t B, int32_t n) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < B) sl[i] += n;
}

// rstd[m] = 1/sqrt(mean(x^2) + eps); xn[m, :] = bf16(x * w) (w may be null = ones).  One wave per
// row, 16-byte loads when d is a multiple of 8 (rows then start 16-byte aligned), else 2-byte
// loads; the wave's partial sums are reduced with DPP and lane reads.
__device__ __forceinline__ uint32_t mul_bf2(uint32_t a, uint32_t b) {
    return pack_bf2(bf_lo(a) * bf_lo(b), bf_hi(a) * bf_hi(b));
}
__global__ __launch_bounds__(256) void rms_prep_kernel(const bf16_t* x, const bf16_t* w, float eps, int64_t M,
                                                       int64_t d, bf16_t* xn, float* rstd) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;  // whole wave
    const int lane = threadIdx.x & 63;
    const bf16_t* xr = x + row * d;
    float s = 0.f;
    if ((d & 7) == 0) {
        for (int64_t c = lane; c < d / 8; c += 64) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c * 8);
            const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) s += bf_lo(e[i]) * bf_lo(e[i]) + bf_hi(e[i]) * bf_hi(e[i]);
            if (xn) {
                u32x4 o = v;
                if (w) {
                    const u32x4 g = *reinterpret_cast<const u32x4*>(w + c * 8);
                    o = u32x4{mul_bf2(v.x, g.x), mul_bf2(v.y, g.y), mul_bf2(v.z, g.z), mul_bf2(v.w, g.w)};
                }
                *reinterpret_cast<u32x4*>(xn + row * d + c * 8) = o;
            }
        }
    } else {
        for (int64_t i = lane; i < d; i += 64) {
            const float v = bf2f(xr[i]);
            s += v * v;
            if (xn) xn[row * d + i] = w ? f2bf(v * bf2f(w[i])) : xr[i];
        }
    }
    s = wave_sum(s);
    if (lane == 0) rstd[row] = 1.0f / sqrtf(s / (float)d + eps);
}

// out[c, r] = in[r, c]: a 64 x 64 tile passes through LDS so both the reads (along rows of in)
// and the writes (along rows of out) are coalesced.  256 threads, 4 rows per pass.
__global__ __launch_bounds__(256) void transpose_kernel(const bf16_t* __restrict__ in, int64_t rows, int64_t cols,
                                                        int64_t ld_in, bf16_t* __restrict__ out, int64_t ld_out) {
    __shared__ bf16_t t[64][66];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const int64_t r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) t[i][tx] = in[r * ld_in + c];
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int64_t c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows) out[c * ld_out + r] = t[tx][i];
    }
}

// Read stream: every 16-byte vector of [p, p + n16) read once (non-temporal: the bytes pass
// through, nothing is kept in the caches), four independent loads per lane in flight per
// iteration; the XOR of everything read is folded into out[blockIdx.x % 64] so no load is dead.
// Each workgroup reads one contiguous slice of the buffer, 4 KiB per wave-row step with 8 steps in
// flight per thread, through non-temporal loads.  Measured on MI355X over 4 GiB: 6.97 TB/s, against
// 6.09 TB/s for a grid-stride walk of the same loads and 5.5-5.9 TB/s with plain loads.
constexpr int kReadDepth = 8;
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ p, int64_t n16, uint32_t* out) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    uint32_t acc = 0;
    int64_t i = b0 + threadIdx.x;
    for (; i + (kReadDepth - 1) * 256 < b1; i += kReadDepth * 256) {
        u32x4 v[kReadDepth];
#pragma unroll
        for (int d = 0; d < kReadDepth; ++d) v[d] = __builtin_nontemporal_load(p + i + d * 256);
#pragma unroll
        for (int d = 0; d < kReadDepth; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    for (; i < b1; i += 256) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & 63) == 0) atomicXor(out + (blockIdx.x & 63), acc);
}

}  // namespace

fsvd_status_t launch_read_stream(const void* src, size_t bytes, uint32_t* out, hipStream_t st) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 <= 0) return FSVD_OK;
    const int64_t want = (n16 + 255) / 256;
    const int grid = (int)std::min<int64_t>(want, 256 * 4);  // 4 workgroups per CU, one slice each
    read_stream_kernel<<<grid, 256, 0, st>>>((const u32x4*)src, n16, out);
    return check_launch("read_stream");
}

fsvd_status_t launch_prepack(void* dst, int64_t ld_dst, int64_t cols_pad, int64_t row0, const void* src, int64_t rows,
                             int64_t cols, int64_t ld_src, int64_t rows_pad, size_t es, const void* col_scale,
                             hipStream_t st) {
    const int64_t total = rows_pad * cols_pad;
    if (total == 0) return FSVD_OK;
    const int grid = (int)std::min<int64_t>((total + 255) / 256, 65536);
    if (es == 2)
        prepack_kernel<uint16_t><<<grid, 256, 0, st>>>((uint16_t*)dst, ld_dst, cols_pad, row0, (const uint16_t*)src,
                                                        rows, cols, ld_src, rows_pad, (const uint16_t*)col_scale);
    else
        prepack_kernel<uint32_t><<<grid, 256, 0, st>>>((uint32_t*)dst, ld_dst, cols_pad, row0, (const uint32_t*)src,
                                                        rows, cols, ld_src, rows_pad, (const uint32_t*)col_scale);
    return check_launch("prepack");
}

fsvd_status_t launch_layernorm(const bf16_t* x, const bf16_t* res, const bf16_t* g, const bf16_t* b, float eps,
                               int64_t M, int64_t d, bf16_t* y, hipStream_t st) {
    if (M == 0) return FSVD_OK;
    const bool vec = d % 8 == 0 && d <= 512 * 16 && aligned16(x) && (!res || aligned16(res)) && aligned16(g) &&
                     aligned16(b) && aligned16(y);
    if (vec) {
        const unsigned grid = (unsigned)((M + 3) / 4);
        if (d <= 512 * 2) layernorm_wave_kernel<2><<<grid, 256, 0, st>>>(x, res, g, b, eps, M, d, y);
        else if (d <= 512 * 4) layernorm_wave_kernel<4><<<grid, 256, 0, st>>>(x, res, g, b, eps, M, d, y);
        else if (d <= 512 * 8) layernorm_wave_kernel<8><<<grid, 256, 0, st>>>(x, res, g, b, eps, M, d, y);
        else layernorm_wave_kernel<16><<<grid, 256, 0, st>>>(x, res, g, b, eps, M, d, y);
        return check_launch("layernorm");
    }
    layernorm_kernel<<<(unsigned)M, 256, d * sizeof(float), st>>>(x, res, g, b, eps, d, y);
    return check_launch("layernorm");
}

fsvd_status_t launch_seqlens_advance(int32_t* sl, int64_t B, int32_t n, hipStream_t st) {
    seqlens_advance_kernel<<<(unsigned)((B + 63) / 64), 64, 0, st>>>(sl, B, n);
    return check_launch("seqlens_advance");
}

fsvd_status_t launch_transpose(const bf16_t* in, int64_t rows, int64_t cols, int64_t ld_in, bf16_t* out,
                               int64_t ld_out, hipStream_t st) {
    if (rows == 0 || cols == 0) return FSVD_OK;
    if ((rows + 63) / 64 > 65535) return fail(FSVD_ERR_UNSUPPORTED, "transpose: too many rows (%lld)", (long long)rows);
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
    transpose_kernel<<<grid, 256, 0, st>>>(in, rows, cols, ld_in, out, ld_out);
    return check_launch("transpose");
}

fsvd_status_t launch_rms_prep(const bf16_t* x, const bf16_t* w, float eps, int64_t M, int64_t d, bf16_t* xn,
                              float* rstd, hipStream_t st) {
    if (M == 0) return FSVD_OK;
    if ((d & 7) == 0 && (!aligned16(x) || (w && !aligned16(w)) || (xn && !aligned16(xn))))
        return fail(FSVD_ERR_INVALID_ARG, "rms_prep: x, norm weight and output must be 16-byte aligned");
    rms_prep_kernel<<<(unsigned)((M + 3) / 4), 256, 0, st>>>(x, w, eps, M, d, xn, rstd);
    return check_launch("rms_prep");
}

}  // namespace fsvd
