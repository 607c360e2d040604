// Beam router on gfx950: logits, sigmoid scores, group-limited top-k selection.
//
// Routing rule: Glonce, "Reflection releases Beam, a 501B open MoE model with 1M
// context", architecture paragraph (sigmoid scores, 8 groups of 32, keep the best
// 4 groups, top 8 experts, normalised weights scaled by 2.5); transformers "Beam"
// model doc, Overview, "Sparse MoE" (per-expert bias balances load; best
// topk_group of n_group groups; routed_scaling_factor) and the FP32-routing
// sentence of the numerics paragraph.  Readings the pages leave open: a group's
// score is the sum of its two largest biased scores; the bias only selects;
// groups are contiguous; experts outside the kept groups are excluded.
#include "common.hpp"

#include <math.h>

namespace beam {

// ---------------------------------------------------------------------------------
// Logits for bf16 activations.  Each fp32 router weight is split exactly into three
// bf16 parts (hi + mid + lo, by truncation), so every MFMA product x*part is exact
// in fp32.  MFMA sums each 32-term block (lo, mid, then hi parts) in fp32; the
// blocks are summed in fp64 and the logit is rounded once to fp32.
//
// Work-group: 4 waves, 32 tokens x 128 experts; wave w owns experts [32w, 32w+32).
// Operands are read straight from global memory (the matrix is L2-resident).
// ---------------------------------------------------------------------------------
constexpr int RL_TOK = 32;
constexpr int RL_EXP = 128;

__device__ __forceinline__ void split3(float w, float& hi, float& mid, float& lo) {
    hi = __uint_as_float(__float_as_uint(w) & 0xFFFF0000u);
    float r1 = w - hi;
    mid = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
    lo = r1 - mid;  // at most 8 significant bits remain: exact in bf16
}

__device__ __forceinline__ __bf16 as_bf16_trunc(float f) {
    uint16_t b = (uint16_t)(__float_as_uint(f) >> 16);
    return __builtin_bit_cast(__bf16, b);
}

__global__ void __launch_bounds__(256) router_logits_bf16_kernel(const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ wr, int64_t T, int H,
                                                                 int E, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * RL_TOK;
    const int e0 = blockIdx.y * RL_EXP + wave * 32;
    if (e0 >= E) return;  // whole wave idle (uniform)

    const int kq = (lane >> 4) * 8;  // k offset of this lane inside a 32-wide k step
    const uint16_t* arow[2];
    bool aval[2];
    for (int rb = 0; rb < 2; ++rb) {
        int64_t t = t0 + rb * 16 + (lane & 15);
        aval[rb] = t < T;
        arow[rb] = x + (aval[rb] ? t : 0) * (int64_t)H + kq;
    }
    const float* brow[2];
    bool bval[2];
    for (int cb = 0; cb < 2; ++cb) {
        int e = e0 + cb * 16 + (lane & 15);
        bval[cb] = e < E;
        brow[cb] = wr + (int64_t)(bval[cb] ? e : 0) * H + kq;
    }

    f32x4 acc[2][2];
    double acc64[2][2][4];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int q = 0; q < 4; ++q) acc64[i][j][q] = 0.0;
        }

    const int nks = H / 32;
    for (int ks = 0; ks < nks; ++ks) {
        const int k0 = ks * 32;
        bf16x8 a[2];
        for (int rb = 0; rb < 2; ++rb) {
            u32x4 v = aval[rb] ? *(const u32x4*)(arow[rb] + k0) : u32x4{0u, 0u, 0u, 0u};
            a[rb] = __builtin_bit_cast(bf16x8, v);
        }
        for (int cb = 0; cb < 2; ++cb) {
            f32x4 w0 = bval[cb] ? *(const f32x4*)(brow[cb] + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 w1 = bval[cb] ? *(const f32x4*)(brow[cb] + k0 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 bh, bm, bl;
            for (int q = 0; q < 8; ++q) {
                float w = q < 4 ? w0[q] : w1[q - 4];
                float hi, mid, lo;
                split3(w, hi, mid, lo);
                bh[q] = as_bf16_trunc(hi);
                bm[q] = as_bf16_trunc(mid);
                bl[q] = as_bf16_trunc(lo);
            }
            for (int rb = 0; rb < 2; ++rb) {
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], bl, acc[rb][cb], 0, 0, 0);
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], bm, acc[rb][cb], 0, 0, 0);
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], bh, acc[rb][cb], 0, 0, 0);
            }
        }
        // fold each 32-term block into fp64: the matrix-core sum rounds once per
        // instruction, so short fp32 chains keep the logit error near one fp32 ulp
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 2; ++j) {
                for (int q = 0; q < 4; ++q) acc64[i][j][q] += (double)acc[i][j][q];
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
    }
    // C layout of a 16x16 MFMA block: lane holds rows 4*(lane>>4)+q, column lane&15
    for (int rb = 0; rb < 2; ++rb)
        for (int cb = 0; cb < 2; ++cb) {
            int e = e0 + cb * 16 + (lane & 15);
            for (int q = 0; q < 4; ++q) {
                int64_t t = t0 + rb * 16 + 4 * (lane >> 4) + q;
                if (t < T && e < E) logits[t * E + e] = (float)acc64[rb][cb][q];
            }
        }
}

// fp32 activations: one thread per (token, expert), fp64 accumulation.
__global__ void router_logits_f32_kernel(const float* __restrict__ x, const float* __restrict__ wr, int64_t T, int H,
                                         int E, float* __restrict__ logits) {
    int64_t n = T * E;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t t = i / E;
        int e = (int)(i % E);
        double acc = 0.0;
        for (int h = 0; h < H; ++h) acc += (double)x[t * H + h] * (double)wr[(int64_t)e * H + h];
        logits[i] = (float)acc;
    }
}

hipError_t launch_router_logits(const void* x, bool bf16, const float* w_router, int64_t T, int H, int E,
                                float* logits, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (bf16) {
        dim3 grid((unsigned)((T + RL_TOK - 1) / RL_TOK), (unsigned)((E + RL_EXP - 1) / RL_EXP));
        router_logits_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)x, w_router, T, H, E, logits);
    } else {
        int64_t n = T * E;
        unsigned blocks = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
        router_logits_f32_kernel<<<blocks, 256, 0, s>>>((const float*)x, w_router, T, H, E, logits);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Selection: one wave per token.  s = fp32(sigmoid(l)) evaluated in fp64 and rounded
// once; s' = s + b (fp32); group score = sum of the group's two largest s' (fp32);
// keep the topk_group best groups; top_k largest s' among their experts; every
// comparison orders by value, then by lower index.  w = rho * s / sum(s) in fp32,
// summed in choice order.
// ---------------------------------------------------------------------------------
constexpr int SEL_MAX_E = 1024;
constexpr int SEL_MAX_G = 64;
constexpr int SEL_WAVES = 4;

__device__ __forceinline__ bool ranks_before(float va, int a, float vb, int b) {
    return va > vb || (va == vb && a < b);
}

__global__ void __launch_bounds__(SEL_WAVES * 64) router_select_kernel(const float* __restrict__ logits,
                                                                       const float* __restrict__ bias, int64_t T,
                                                                       int E, int n_group, int topk_group,
                                                                       int top_k, float rho,
                                                                       int32_t* __restrict__ idx_out,
                                                                       float* __restrict__ w_out) {
    __shared__ float s_sc[SEL_WAVES][SEL_MAX_E];
    __shared__ float s_sb[SEL_WAVES][SEL_MAX_E];
    __shared__ float s_gs[SEL_WAVES][SEL_MAX_G];
    __shared__ int s_kept[SEL_WAVES][SEL_MAX_G];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * SEL_WAVES + wave;
    const bool active = t < T;
    const int gsize = E / n_group;

    if (active) {
        for (int e = lane; e < E; e += 64) {
            float l = logits[t * E + e];
            float sc = (float)(1.0 / (1.0 + exp(-(double)l)));
            s_sc[wave][e] = sc;
            s_sb[wave][e] = sc + bias[e];
        }
    }
    __syncthreads();
    if (active) {
        for (int g = lane; g < n_group; g += 64) {
            float a1 = -INFINITY, a2 = -INFINITY;
            for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
                float v = s_sb[wave][e];
                if (v > a1) {
                    a2 = a1;
                    a1 = v;
                } else if (v > a2) {
                    a2 = v;
                }
            }
            s_gs[wave][g] = gsize >= 2 ? a1 + a2 : a1;
        }
    }
    __syncthreads();
    if (active) {
        for (int g = lane; g < n_group; g += 64) {
            float v = s_gs[wave][g];
            int rank = 0;
            for (int o = 0; o < n_group; ++o) rank += (o != g && ranks_before(s_gs[wave][o], o, v, g)) ? 1 : 0;
            s_kept[wave][g] = rank < topk_group;
        }
    }
    __syncthreads();
    if (!active) return;

    // lane owns experts lane, lane+64, ...; `taken` marks its chosen ones
    uint32_t taken = 0;
    float ssum = 0.f;
    int my_e = -1;
    float my_s = 0.f;
    for (int j = 0; j < top_k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int q = 0, e = lane; e < E; ++q, e += 64) {
            if (((taken >> q) & 1u) || !s_kept[wave][e / gsize]) continue;
            float v = s_sb[wave][e];
            if (ranks_before(v, e, bv, bi)) {
                bv = v;
                bi = e;
            }
        }
        for (int off = 32; off >= 1; off >>= 1) {
            float ov = __shfl_xor(bv, off);
            int oi = __shfl_xor(bi, off);
            if (ranks_before(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        // non-finite scores compare false everywhere; keep the index in range regardless
        if (bi < 0 || bi >= E) bi = 0;
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        float sc = s_sc[wave][bi];
        ssum += sc;
        if (lane == j) {
            my_e = bi;
            my_s = sc;
        }
    }
    if (lane < top_k) {
        idx_out[t * top_k + lane] = my_e;
        w_out[t * top_k + lane] = rho * my_s / ssum;
    }
}

hipError_t launch_router_select(const float* logits, const float* bias, int64_t T, int E, int n_group,
                                int topk_group, int top_k, float rho, int32_t* idx, float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    unsigned blocks = (unsigned)((T + SEL_WAVES - 1) / SEL_WAVES);
    router_select_kernel<<<blocks, SEL_WAVES * 64, 0, s>>>(logits, bias, T, E, n_group, topk_group, top_k, rho, idx,
                                                          w);
    return hipGetLastError();
}

}  // namespace beam
