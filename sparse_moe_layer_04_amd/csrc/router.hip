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
// in fp32.  MFMA sums each 32-term block (lo, mid, then hi parts) in fp32; the blocks
// are summed in fp64.  The H columns may be split into `nsplit` ranges handled by
// different work-groups (small T needs the parallelism); each writes an fp64 partial
// and the selection kernel adds the partials in split order before rounding the logit
// once to fp32, so the result does not depend on scheduling.
// ---------------------------------------------------------------------------------
constexpr int RL_KUNIT = 64;   // split granularity: klen is a multiple of 64 columns

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

// x [T,H] bf16, wr [E,H] fp32 -> part [nsplit][T][E] fp64 (split s covers columns
// [s*klen, (s+1)*klen), klen a multiple of 32).
//
// A work-group of 4 waves covers TOK = 16*RB tokens x 64*CB experts (RB*CB = 8): wave w
// owns CB 16-expert blocks of all RB token blocks, so each split weight feeds RB MFMAs.
// Each 32-k step is staged through LDS: the four lanes of every quad load 64 contiguous
// bytes of one row of x or W_r.  Loaded straight in the MFMA layout, each quad would
// touch four rows and the L1 would process the loads at a quarter of its rate; x would
// also be fetched by all four waves.  Fragments are read back with an XOR swizzle on
// the 16-byte piece index, so the lanes of every ds_read_b128 / ds_write_b128 phase hit
// distinct banks (for phases of 8 lanes over 128 bytes and of 16 lanes over 256).
__device__ __forceinline__ int rl_x_off(int row, int piece) {   // 4 pieces of 16 B per row
    return row * 64 + ((piece ^ ((row >> 1) & 3) ^ ((row >> 3) & 1)) << 4);
}
__device__ __forceinline__ int rl_w_off(int row, int piece) {   // 8 pieces of 16 B per row
    return row * 128 + ((piece ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

template <int RB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) router_logits_bf16_kernel(const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ wr, int64_t T, int H,
                                                                 int E, int klen, double* __restrict__ part) {
    constexpr int CB = 8 / RB, TOK = 16 * RB, EXP = 64 * CB;
    constexpr int XS = TOK * 64, BUF = XS + EXP * 128;   // bytes of x, then W_r, per step
    constexpr int XP = TOK / 64, WP = 2 * CB;             // 16-byte pieces per thread
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * BUF];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * TOK;
    const int eb = blockIdx.y * EXP;
    const int split = blockIdx.z;

    // global sources of this thread's pieces (rows past T or E repeat the last row)
    const uint16_t* xsrc[XP];
    int xoff[XP], woff[WP];
    const float* wsrc[WP];
    for (int i = 0; i < XP; ++i) {
        const int n = i * 256 + tid, r = n >> 2;
        const int64_t t = t0 + r < T ? t0 + r : T - 1;
        xsrc[i] = x + t * (int64_t)H + split * klen + (n & 3) * 8;
        xoff[i] = rl_x_off(r, n & 3);
    }
    for (int i = 0; i < WP; ++i) {
        const int n = i * 256 + tid, r = n >> 3;
        const int e = eb + r < E ? eb + r : E - 1;
        wsrc[i] = wr + (int64_t)e * H + split * klen + (n & 7) * 4;
        woff[i] = XS + rl_w_off(r, n & 7);
    }
    u32x4 gx[XP];
    f32x4 gw[WP];
    auto gload = [&](int ks) {
        for (int i = 0; i < XP; ++i) gx[i] = *(const u32x4*)(xsrc[i] + ks * 32);
        for (int i = 0; i < WP; ++i) gw[i] = *(const f32x4*)(wsrc[i] + ks * 32);
    };
    auto lstore = [&](int buf) {
        unsigned char* b = lds + buf * BUF;
        for (int i = 0; i < XP; ++i) *(u32x4*)(b + xoff[i]) = gx[i];
        for (int i = 0; i < WP; ++i) *(f32x4*)(b + woff[i]) = gw[i];
    };

    f32x4 acc[RB][CB];
    double acc64[RB][CB][4];
    for (int i = 0; i < RB; ++i)
        for (int j = 0; j < CB; ++j)
            for (int q = 0; q < 4; ++q) acc64[i][j][q] = 0.0;

    const int kg = lane >> 4;   // this lane's 8-k group of the 32-k step
    auto compute = [&](int buf) {
        const unsigned char* b = lds + buf * BUF;
        bf16x8 a[RB];
        for (int rb = 0; rb < RB; ++rb)
            a[rb] = __builtin_bit_cast(bf16x8, *(const u32x4*)(b + rl_x_off(rb * 16 + (lane & 15), kg)));
        for (int i = 0; i < RB; ++i)
            for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int cb = 0; cb < CB; ++cb) {
            const int row = (wave * CB + cb) * 16 + (lane & 15);
            const f32x4 w0 = *(const f32x4*)(b + XS + rl_w_off(row, 2 * kg));
            const f32x4 w1 = *(const f32x4*)(b + XS + rl_w_off(row, 2 * kg + 1));
            bf16x8 bh, bm, bl;
            for (int q = 0; q < 8; ++q) {
                const float w = q < 4 ? w0[q] : w1[q - 4];
                float hi, mid, lo;
                split3(w, hi, mid, lo);
                bh[q] = as_bf16_trunc(hi);
                bm[q] = as_bf16_trunc(mid);
                bl[q] = as_bf16_trunc(lo);
            }
            for (int rb = 0; rb < RB; ++rb) {
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], bl, acc[rb][cb], 0, 0, 0);
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], bm, acc[rb][cb], 0, 0, 0);
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], bh, acc[rb][cb], 0, 0, 0);
            }
        }
        // fold each 32-term block into fp64: the matrix-core sum rounds once per
        // instruction, so short fp32 chains keep the logit error near one fp32 ulp
        for (int i = 0; i < RB; ++i)
            for (int j = 0; j < CB; ++j)
                for (int q = 0; q < 4; ++q) acc64[i][j][q] += (double)acc[i][j][q];
    };

    const int nks = klen / 32;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
        const bool more = ks + 1 < nks;
        if (more) gload(ks + 1);   // in flight while this step's MFMAs run
        compute(ks & 1);
        if (more) lstore((ks + 1) & 1);
        __syncthreads();
    }
    // C layout of a 16x16 MFMA block: lane holds rows 4*(lane>>4)+q, column lane&15
    double* out = part + (int64_t)split * T * E;
    for (int rb = 0; rb < RB; ++rb)
        for (int cb = 0; cb < CB; ++cb) {
            const int e = eb + (wave * CB + cb) * 16 + (lane & 15);
            for (int q = 0; q < 4; ++q) {
                const int64_t t = t0 + rb * 16 + 4 * (lane >> 4) + q;
                if (t < T && e < E) out[t * E + e] = acc64[rb][cb][q];
            }
        }
}

// 128-token tiles from 128 tokens on (half the weight splits per MFMA); smaller batches
// keep 64-token tiles so that fewer MFMA row blocks are padding.
constexpr int64_t RL_WIDE_MIN_T = 128;
static int router_rb(int64_t T) { return T >= RL_WIDE_MIN_T ? 8 : 4; }

int router_splits(int64_t T, int H, int E) {
    const int rb = router_rb(T), tok = 16 * rb, exp = 512 / rb;
    const int64_t tiles = ((T + tok - 1) / tok) * ((E + exp - 1) / exp);
    // up to ~512 work-groups (two per CU), each taking at least two units (four 32-k
    // steps): more splits add fp64 partials that the selection must read back (at T = 300,
    // 49 MB at 80 splits); a target of 1024 or 256 groups measured slower from T = 1000 on
    const int units = H / RL_KUNIT;
    int best = 1;
    for (int d = 1; 2 * d <= units; ++d)
        if (units % d == 0 && tiles * d <= 512) best = d;
    return best;
}

// fp32 activations: one thread per (token, expert), fp64 accumulation.
__global__ void router_logits_f32_kernel(const float* __restrict__ x, const float* __restrict__ wr, int64_t T, int H,
                                         int E, double* __restrict__ part) {
    int64_t n = T * E;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t t = i / E;
        int e = (int)(i % E);
        double acc = 0.0;
        for (int h = 0; h < H; ++h) acc += (double)x[t * H + h] * (double)wr[(int64_t)e * H + h];
        part[i] = acc;
    }
}

hipError_t launch_router_logits(const void* x, bool bf16, const float* w_router, int64_t T, int H, int E,
                                int nsplit, double* part, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (bf16) {
        const int rb = router_rb(T), tok = 16 * rb, exp = 512 / rb;
        dim3 grid((unsigned)((T + tok - 1) / tok), (unsigned)((E + exp - 1) / exp), (unsigned)nsplit);
        if (rb == 8)
            router_logits_bf16_kernel<8><<<grid, 256, 0, s>>>((const uint16_t*)x, w_router, T, H, E, H / nsplit, part);
        else
            router_logits_bf16_kernel<4><<<grid, 256, 0, s>>>((const uint16_t*)x, w_router, T, H, E, H / nsplit, part);
    } else {
        int64_t n = T * E;
        unsigned blocks = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
        router_logits_f32_kernel<<<blocks, 256, 0, s>>>((const float*)x, w_router, T, H, E, part);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Selection.  s = fp32(sigmoid(l)) evaluated in fp64 and rounded once; s' = s + b
// (fp32); group score = sum of the group's two largest s' (fp32); keep the topk_group
// best groups; top_k largest s' among their experts; every comparison orders by value,
// then by lower index.  w = rho * s / sum(s) in fp32, summed in choice order.
// A work-group takes `tpb` tokens (4 for large T, else 1): all 256 threads reduce the
// partial logits, then wave w chooses the experts of token w.
// ---------------------------------------------------------------------------------
constexpr int SEL_MAX_E = 1024;
constexpr int SEL_MAX_G = 64;
constexpr int SEL_THREADS = 256;
constexpr int SEL_MAX_TPB = SEL_THREADS / 64;

__device__ __forceinline__ bool ranks_before(float va, int a, float vb, int b) {
    return va > vb || (va == vb && a < b);
}

// one exchange of a (score, index) argmax between lanes paired by a DPP pattern that
// stays inside each row of 16 lanes
template <int CTRL>
__device__ __forceinline__ void sel_dpp_step(float& bv, int& bi) {
    const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
    const int oi = __builtin_amdgcn_update_dpp(0, bi, CTRL, 0xF, 0xF, false);
    if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
    }
}

__global__ void __launch_bounds__(SEL_THREADS) router_select_kernel(const double* __restrict__ part, int nsplit,
                                                                    const float* __restrict__ bias, int64_t T, int E,
                                                                    int n_group, int topk_group, int top_k,
                                                                    float rho, int tpb, int32_t* __restrict__ idx_out,
                                                                    float* __restrict__ w_out,
                                                                    float* __restrict__ logits_out) {
    __shared__ float s_sc[SEL_MAX_TPB][SEL_MAX_E];
    __shared__ float s_sb[SEL_MAX_TPB][SEL_MAX_E];
    __shared__ float s_gs[SEL_MAX_TPB][SEL_MAX_G];
    __shared__ int s_kept[SEL_MAX_TPB][SEL_MAX_G];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t tb = (int64_t)blockIdx.x * tpb;
    const int ntok = T - tb < tpb ? (int)(T - tb) : tpb;
    const int gsize = E / n_group;
    const int64_t stride = T * E;

    // each logit adds its partials in split order; at least eight loads are in flight:
    // eight splits of one logit when there are many splits, else four logits per thread
    const int nlog = ntok * E;
    auto finish = [&](int i, double l64) {
        const int tt = i / E, e = i - tt * E;
        const float l = (float)l64;
        if (logits_out) logits_out[(tb + tt) * E + e] = l;
        const float sc = (float)(1.0 / (1.0 + exp(-(double)l)));
        s_sc[tt][e] = sc;
        s_sb[tt][e] = sc + bias[e];
    };
    if (nsplit >= 8) {
        for (int i = tid; i < nlog; i += SEL_THREADS) {
            const double* pe = part + tb * E + i;
            double l64 = 0.0;
            int sp = 0;
            for (; sp + 8 <= nsplit; sp += 8) {
                double v[8];
#pragma unroll
                for (int a = 0; a < 8; ++a) v[a] = pe[(int64_t)(sp + a) * stride];
#pragma unroll
                for (int a = 0; a < 8; ++a) l64 += v[a];
            }
            for (; sp < nsplit; ++sp) l64 += pe[(int64_t)sp * stride];
            finish(i, l64);
        }
    } else {
        for (int i0 = tid; i0 < nlog; i0 += 4 * SEL_THREADS) {
            const double* pe[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * SEL_THREADS < nlog ? i0 + u * SEL_THREADS : i0;  // repeats stay in bounds
                pe[u] = part + tb * E + i;
            }
            double l64[4] = {0.0, 0.0, 0.0, 0.0};
            int sp = 0;
            for (; sp + 2 <= nsplit; sp += 2) {
                double v[2][4];
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int u = 0; u < 4; ++u) v[a][u] = pe[u][(int64_t)(sp + a) * stride];
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int u = 0; u < 4; ++u) l64[u] += v[a][u];
            }
            for (; sp < nsplit; ++sp)
#pragma unroll
                for (int u = 0; u < 4; ++u) l64[u] += pe[u][(int64_t)sp * stride];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * SEL_THREADS;
                if (i >= nlog) break;
                finish(i, l64[u]);
            }
        }
    }
    __syncthreads();
    // group scores: the wave of token tt gives each group L lanes (L a power of two, L *
    // n_group <= 64); each lane keeps the two largest biased scores of its slice, and the
    // L lanes merge their pairs (the top two of four values) by butterfly exchange
    {
        const int tt = tid >> 6;
        int lg = 0;
        while ((2 << lg) * n_group <= 64) ++lg;
        const int L = 1 << lg, g = lane >> lg, sub = lane & (L - 1);
        float a1 = -INFINITY, a2 = -INFINITY;
        if (tt < ntok && g < n_group)
            for (int e = g * gsize + sub; e < (g + 1) * gsize; e += L) {
                const float v = s_sb[tt][e];
                if (v > a1) {
                    a2 = a1;
                    a1 = v;
                } else if (v > a2) {
                    a2 = v;
                }
            }
        for (int off = 1; off < L; off <<= 1) {
            const float b1 = __shfl_xor(a1, off), b2 = __shfl_xor(a2, off);
            a2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
            a1 = fmaxf(a1, b1);
        }
        if (tt < ntok && g < n_group && sub == 0) s_gs[tt][g] = gsize >= 2 ? a1 + a2 : a1;
    }
    __syncthreads();
    for (int i = tid; i < ntok * n_group; i += SEL_THREADS) {
        const int tt = i / n_group, g = i - tt * n_group;
        const float v = s_gs[tt][g];
        int rank = 0;
        for (int o = 0; o < n_group; ++o) rank += (o != g && ranks_before(s_gs[tt][o], o, v, g)) ? 1 : 0;
        s_kept[tt][g] = rank < topk_group;
    }
    __syncthreads();
    const int tt = tid >> 6;  // this wave's token
    if (tt >= ntok) return;
    const int64_t t = tb + tt;

    // lane owns experts lane, lane+64, ...; `avail` marks those still available (in a
    // kept group, not yet chosen)
    uint32_t avail = 0;
    for (int q = 0, e = lane; e < E; ++q, e += 64)
        if (s_kept[tt][e / gsize]) avail |= 1u << q;
    float ssum = 0.f;
    int my_e = -1;
    float my_s = 0.f;
    for (int j = 0; j < top_k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int q = 0, e = lane; e < E; ++q, e += 64) {
            if (!((avail >> q) & 1u)) continue;
            const float v = s_sb[tt][e];
            if (ranks_before(v, e, bv, bi)) {
                bv = v;
                bi = e;
            }
        }
        // best of each row of 16 lanes (DPP exchanges), then of the four rows
        sel_dpp_step<0xB1>(bv, bi);    // quad_perm [1,0,3,2]
        sel_dpp_step<0x4E>(bv, bi);    // quad_perm [2,3,0,1]
        sel_dpp_step<0x141>(bv, bi);   // row_half_mirror
        sel_dpp_step<0x140>(bv, bi);   // row_mirror
        {
            float gv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
            int gi = __builtin_amdgcn_readlane(bi, 0);
            for (int r = 16; r < 64; r += 16) {
                const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), r));
                const int oi = __builtin_amdgcn_readlane(bi, r);
                if (ranks_before(ov, oi, gv, gi)) {
                    gv = ov;
                    gi = oi;
                }
            }
            bv = gv;
            bi = gi;
        }
        // non-finite scores compare false everywhere; keep the index in range regardless
        if (bi < 0 || bi >= E) bi = 0;
        if ((bi & 63) == lane) avail &= ~(1u << (bi >> 6));
        const float sc = s_sc[tt][bi];
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

hipError_t launch_router_select(const double* part, int nsplit, const float* bias, int64_t T, int E, int n_group,
                                int topk_group, int top_k, float rho, int32_t* idx, float* w, float* logits_out,
                                hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int tpb = T >= 1024 ? SEL_MAX_TPB : 1;  // small batches: more work-groups for the reduction
    const unsigned blocks = (unsigned)((T + tpb - 1) / tpb);
    router_select_kernel<<<blocks, SEL_THREADS, 0, s>>>(part, nsplit, bias, T, E, n_group, topk_group, top_k, rho, tpb,
                                                       idx, w, logits_out);
    return hipGetLastError();
}

}  // namespace beam
