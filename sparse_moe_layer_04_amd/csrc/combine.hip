// Weighted combine, sandwich RMSNorms and the depth-scaled residual of the Beam MoE
// layer on gfx950.
//
// Combine: y_t = sum_j w_{t,j} z_{t,j}, j ascending (expert outputs combined with the
// normalised, scaled router weights; Glonce, "Reflection releases Beam, a 501B open
// MoE model with 1M context", architecture paragraph).
// Sublayer: RMSNorm before and after the block and the residual update
// x <- sqrt((k-1)/k) x + block(x)/sqrt(k) (Glonce, residual paragraph; transformers
// "Beam" model doc, Overview, "Sandwich norms with depth-scaled residuals"); RMSNorm
// scaling in FP32 (model doc, numerics paragraph).
#include "common.hpp"

#include <math.h>

namespace beam {

constexpr int CMB_THREADS = 256;      // fp32 path
constexpr int CMB_MAX_THREADS = 1024;  // bf16 path: one 16-byte chunk per thread up to H = 8192
constexpr int CMB_MAX_K = 32;

__device__ __forceinline__ float block_sum(float v, float* red) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
    __syncthreads();
    return s;
}

// bf16 path: 8 consecutive features per step (16-byte loads), one work-group per token
// sized so that every thread takes one chunk (two per thread measured 5% slower at T = 8192).  With POST the summed row is kept
// in LDS (H floats) for the post-norm pass.
template <bool POST>
__global__ void __launch_bounds__(CMB_MAX_THREADS) combine_bf16_kernel(const uint16_t* __restrict__ y_pair,
                                                                   const float* __restrict__ topk_w, int H, int K,
                                                                   const uint16_t* __restrict__ x,
                                                                   const float* __restrict__ g2, float eps,
                                                                   float coef_x, float coef_y,
                                                                   uint16_t* __restrict__ out,
                                                                   uint16_t* __restrict__ moe_y) {
    extern __shared__ float ys[];
    __shared__ float wk[CMB_MAX_K];
    __shared__ float red[CMB_MAX_THREADS / 64];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    if (tid < K) wk[tid] = topk_w[t * K + tid];
    __syncthreads();
    const int nch = H / 8;
    float ss = 0.f;
    for (int c = tid; c < nch; c += nth) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.f;
        // up to eight expert rows in flight, then added in j order
        for (int j0 = 0; j0 < K; j0 += 8) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (j0 + u < K) v[u] = *(const u32x4*)(y_pair + ((t * K + j0 + u) * H + c * 8));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u < K) {
                    const float wj = wk[j0 + u];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] = fmaf(wj, __uint_as_float(v[u][q] << 16), acc[2 * q]);
                        acc[2 * q + 1] = fmaf(wj, __uint_as_float(v[u][q] & 0xFFFF0000u), acc[2 * q + 1]);
                    }
                }
            }
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        if (POST) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                ys[c * 8 + q] = acc[q];
                ss = fmaf(acc[q], acc[q], ss);
            }
            if (moe_y) *(u32x4*)(moe_y + t * H + c * 8) = o;
        } else {
            *(u32x4*)(out + t * H + c * 8) = o;
        }
    }
    if (!POST) return;
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    for (int c = tid; c < nch; c += nth) {
        const u32x4 xv = *(const u32x4*)(x + t * H + c * 8);
        float o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float xq = q & 1 ? __uint_as_float(xv[q >> 1] & 0xFFFF0000u) : __uint_as_float(xv[q >> 1] << 16);
            const float yh = g2[c * 8 + q] * (ys[c * 8 + q] * r);
            o[q] = fmaf(coef_x, xq, coef_y * yh);
        }
        u32x4 ov;
#pragma unroll
        for (int q = 0; q < 4; ++q) ov[q] = pack_bf16x2(o[2 * q], o[2 * q + 1]);
        *(u32x4*)(out + t * H + c * 8) = ov;
    }
}

// fp32 path: one feature per step, no sublayer.
__global__ void __launch_bounds__(CMB_THREADS) combine_f32_kernel(const float* __restrict__ y_pair,
                                                                  const float* __restrict__ topk_w, int H, int K,
                                                                  float* __restrict__ out) {
    const int64_t t = blockIdx.x;
    for (int h = threadIdx.x; h < H; h += CMB_THREADS) {
        float acc = 0.f;
        for (int j = 0; j < K; ++j) acc = fmaf(topk_w[t * K + j], y_pair[(t * K + j) * H + h], acc);
        out[t * H + h] = acc;
    }
}

hipError_t launch_combine(const void* y_pair, bool bf16, const float* topk_w, int64_t T, int H, int K, const void* x,
                          const float* post_gain, float eps, float residual_k, void* out, void* moe_y,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    int nth = H / 8;  // one 16-byte chunk per thread
    nth = (nth + 63) / 64 * 64;
    nth = nth < 64 ? 64 : (nth > CMB_MAX_THREADS ? CMB_MAX_THREADS : nth);
    if (!bf16) {
        combine_f32_kernel<<<(unsigned)T, CMB_THREADS, 0, s>>>((const float*)y_pair, topk_w, H, K, (float*)out);
    } else if (post_gain == nullptr) {
        combine_bf16_kernel<false><<<(unsigned)T, nth, 0, s>>>(
            (const uint16_t*)y_pair, topk_w, H, K, nullptr, nullptr, 0.f, 0.f, 0.f, (uint16_t*)out, nullptr);
    } else {
        const double k = (double)residual_k;
        const float cx = (float)sqrt((k - 1.0) / k);
        const float cy = (float)(1.0 / sqrt(k));
        combine_bf16_kernel<true><<<(unsigned)T, nth, (size_t)H * sizeof(float), s>>>(
            (const uint16_t*)y_pair, topk_w, H, K, (const uint16_t*)x, post_gain, eps, cx, cy, (uint16_t*)out,
            (uint16_t*)moe_y);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Pre-RMSNorm with pinned rounding: the mean square is summed in fp64 (squares of
// bf16 values are exact in fp64), r = fp32(1/sqrt(ss/H + eps)) is evaluated in fp64
// and rounded once, then u = bf16(fp32(fp32(x*r) * g)).  Every step is correctly
// rounded, so u does not depend on the summation order except in the last fp64 bit
// of ss.
// ---------------------------------------------------------------------------------
__global__ void __launch_bounds__(CMB_MAX_THREADS) rmsnorm_pinned_kernel(const uint16_t* __restrict__ x,
                                                                         const float* __restrict__ gain, float eps,
                                                                         int H, uint16_t* __restrict__ u) {
    __shared__ double red[CMB_MAX_THREADS / 64];
    __shared__ float r_sh;
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    const uint16_t* xr = x + t * H;
    const int nch = H / 8;  // 16-byte chunks (H % 8 == 0 is checked by the caller)
    double ss = 0.0;
    for (int c = tid; c < nch; c += nth) {
        const u32x4 v = *(const u32x4*)(xr + c * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double lo = (double)__uint_as_float(v[q] << 16);
            const double hi = (double)__uint_as_float(v[q] & 0xFFFF0000u);
            ss += lo * lo;
            ss += hi * hi;
        }
    }
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int w = 0; w < nth / 64; ++w) tot += red[w];
        r_sh = (float)(1.0 / sqrt(tot / (double)H + (double)eps));
    }
    __syncthreads();
    const float r = r_sh;
    for (int c = tid; c < nch; c += nth) {
        const u32x4 v = *(const u32x4*)(xr + c * 8);
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a0 = __fmul_rn(__uint_as_float(v[q] << 16), r);
            const float a1 = __fmul_rn(__uint_as_float(v[q] & 0xFFFF0000u), r);
            o[q] = pack_bf16x2(__fmul_rn(a0, gain[c * 8 + 2 * q]), __fmul_rn(a1, gain[c * 8 + 2 * q + 1]));
        }
        *(u32x4*)(u + t * H + c * 8) = o;
    }
}

hipError_t launch_rmsnorm(const uint16_t* x, const float* gain, float eps, int64_t T, int H, uint16_t* u,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    int nth = (H / 8 + 1) / 2;  // two 16-byte chunks per thread
    nth = (nth + 63) / 64 * 64;
    nth = nth < 64 ? 64 : (nth > CMB_MAX_THREADS ? CMB_MAX_THREADS : nth);
    rmsnorm_pinned_kernel<<<(unsigned)T, nth, 0, s>>>(x, gain, eps, H, u);
    return hipGetLastError();
}

}  // namespace beam
