// Grouped expert GEMMs of the Beam MoE layer on gfx950.
//
// Expert = SwiGLU MLP with intermediate size I (Glonce, "Reflection releases Beam,
// a 501B open MoE model with 1M context", architecture paragraph; transformers
// "Beam" model doc, Overview, "Sparse MoE"); the SwiGLU activation is evaluated in
// FP32 (model doc, numerics paragraph):
//   gate/up:  h[r, :] = silu(u_t W_g[e]^T) * (u_t W_u[e]^T),  silu(a) = a / (1 + e^-a)
//   down:     y_pair[p, :] = h[r, :] W_d[e]^T
// where row r of the expert-sorted pair list holds pair p = t*top_k + j routed to e.
//
// bf16 path: one work-group computes one (tile, column block): up to BM rows of one
// expert times BN weight rows, K swept in steps of BK through LDS with a register
// prefetch of the next step.  Gate/up tiles hold BN/2 gate rows and BN/2 up rows of
// the same output columns, so the SwiGLU epilogue has both operands in registers.
// The gate/up A operand is gathered straight from the token rows (no permuted copy);
// the down epilogue scatters each row to its pair position.
#include "common.hpp"

namespace beam {

constexpr int GBK = 64;    // k per LDS stage
constexpr int GBN = 128;   // weight rows per tile
constexpr int GTHREADS = 256;

// LDS element offset of 16-byte chunk `ch` (0..7) of tile row `row`; the XOR spreads the
// 16 rows read by one MFMA operand load over distinct banks.
__device__ __forceinline__ int lds_off(int row, int ch) { return row * GBK + ((ch ^ (row & 7)) << 3); }

template <int BM, int WM, bool GATED>
__global__ void __launch_bounds__(GTHREADS) moe_gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                                 const uint16_t* __restrict__ B0,
                                                                 const uint16_t* __restrict__ B1, int K, int N,
                                                                 int top_k, const int32_t* __restrict__ sorted_pairs,
                                                                 const TileEntry* __restrict__ tiles,
                                                                 const int32_t* __restrict__ num_tiles,
                                                                 int n_col_blocks, uint16_t* __restrict__ C) {
    constexpr int WN = 4 / WM;
    constexpr int RB = BM / (16 * WM);   // 16-row MFMA blocks per wave
    constexpr int CB = GBN / (16 * WN);  // 16-column MFMA blocks per wave
    constexpr int NOUT = GATED ? GBN / 2 : GBN;
    constexpr int A_CHUNKS = BM * 8;
    constexpr int A_PER_T = (A_CHUNKS + GTHREADS - 1) / GTHREADS;
    constexpr int B_PER_T = GBN * 8 / GTHREADS;
    static_assert(RB >= 1 && CB >= 2 && (CB % 2) == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t As[BM * GBK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[GBN * GBK];

    const int tile_id = (int)(blockIdx.x / n_col_blocks);
    const int cblk = (int)(blockIdx.x % n_col_blocks);
    if (tile_id >= *num_tiles) return;
    const TileEntry te = tiles[tile_id];
    if (te.row_count <= 0) return;
    const int e = te.expert;
    const int n0 = cblk * NOUT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;

    // ---- global -> register -> LDS assignments (16-byte chunks) ----
    const uint16_t* a_src[A_PER_T];
    int a_lds[A_PER_T];
    bool a_ok[A_PER_T], a_in[A_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
        const int c = tid + i * GTHREADS;
        const int row = c >> 3, ch = c & 7;
        a_in[i] = c < A_CHUNKS;
        a_ok[i] = a_in[i] && row < te.row_count;
        int64_t src_row = 0;
        if (a_ok[i]) {
            const int srow = te.row_begin + row;
            src_row = GATED ? (int64_t)(sorted_pairs[srow] / top_k) : (int64_t)srow;
        }
        a_src[i] = A + src_row * K + ch * 8;
        a_lds[i] = lds_off(a_in[i] ? row : 0, ch);
    }
    const uint16_t* b_src[B_PER_T];
    int b_lds[B_PER_T];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
        const int c = tid + i * GTHREADS;
        const int row = c >> 3, ch = c & 7;
        if (GATED) {
            const uint16_t* W = row < GBN / 2 ? B0 : B1;
            b_src[i] = W + ((int64_t)e * N + n0 + (row & (GBN / 2 - 1))) * K + ch * 8;
        } else {
            b_src[i] = B0 + ((int64_t)e * N + n0 + row) * K + ch * 8;
        }
        b_lds[i] = lds_off(row, ch);
    }

    u32x4 ra[A_PER_T], rbv[B_PER_T];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i)
            ra[i] = a_ok[i] ? *(const u32x4*)(a_src[i] + k0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) rbv[i] = *(const u32x4*)(b_src[i] + k0);
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i)
            if (a_in[i]) *(u32x4*)(As + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) *(u32x4*)(Bs + b_lds[i]) = rbv[i];
    };

    f32x4 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wrow0 = wm * RB * 16;
    bool rb_on[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) rb_on[i] = wrow0 + i * 16 < te.row_count;

    int brow[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        if (GATED)
            brow[cb] = (cb < CB / 2) ? wn * (CB / 2) * 16 + cb * 16 : GBN / 2 + wn * (CB / 2) * 16 + (cb - CB / 2) * 16;
        else
            brow[cb] = wn * CB * 16 + cb * 16;
    }

    const int nk = K / GBK;
    gload(0);
    for (int kt = 0; kt < nk; ++kt) {
        lstore();
        __syncthreads();
        if (kt + 1 < nk) gload((kt + 1) * GBK);
        if (rb_on[0]) {
#pragma unroll
            for (int ks = 0; ks < GBK / 32; ++ks) {
                const int ch = ks * 4 + (lane >> 4);
                bf16x8 b[CB];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) b[cb] = *(const bf16x8*)(Bs + lds_off(brow[cb] + (lane & 15), ch));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if (!rb_on[rb]) continue;
                    const bf16x8 a = *(const bf16x8*)(As + lds_off(wrow0 + rb * 16 + (lane & 15), ch));
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[cb], acc[rb][cb], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue (C layout of a 16x16 block: rows 4*(lane>>4)+q, column lane&15) ----
    if (GATED) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int cb = 0; cb < CB / 2; ++cb) {
                const int col = n0 + wn * (CB / 2) * 16 + cb * 16 + (lane & 15);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = wrow0 + rb * 16 + 4 * (lane >> 4) + q;
                    if (m < te.row_count) {
                        const float g = acc[rb][cb][q];
                        const float u = acc[rb][cb + CB / 2][q];
                        const float hv = g / (1.0f + __expf(-g)) * u;
                        C[(int64_t)(te.row_begin + m) * N + col] = f32_to_bf16(hv);
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = wrow0 + rb * 16 + 4 * (lane >> 4) + q;
                if (m < te.row_count) {
                    const int64_t p = sorted_pairs[te.row_begin + m];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const int col = n0 + wn * CB * 16 + cb * 16 + (lane & 15);
                        C[p * N + col] = f32_to_bf16(acc[rb][cb][q]);
                    }
                }
            }
        }
    }
}

int gemm_tile_rows(int64_t P, int E, bool bf16) {
    if (!bf16) return 1 << 30;  // the fp32 path does not use tiles
    const int64_t avg = E > 0 ? P / E : 0;
    if (avg >= 64) return 128;
    if (avg >= 16) return 32;
    return 16;
}

template <int BM, int WM, bool GATED>
static void launch_gemm(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, int K, int N, int top_k,
                        const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                        int64_t max_tile_count, uint16_t* C, hipStream_t s) {
    const int nout = GATED ? GBN / 2 : GBN;
    const int ncb = N / nout;
    const int64_t blocks = max_tile_count * ncb;
    moe_gemm_bf16_kernel<BM, WM, GATED><<<(unsigned)blocks, GTHREADS, 0, s>>>(A, B0, B1, K, N, top_k, sorted_pairs,
                                                                             tiles, num_tiles, ncb, C);
}

hipError_t launch_gate_up(const void* act, bool bf16, const void* w_gate, const void* w_up, int H, int I, int top_k,
                          const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                          int64_t max_tile_count, int tile_rows, void* h, hipStream_t s) {
    if (!bf16 || max_tile_count <= 0) return hipErrorInvalidValue;
    auto A = (const uint16_t*)act;
    auto g = (const uint16_t*)w_gate;
    auto u = (const uint16_t*)w_up;
    auto o = (uint16_t*)h;
    if (tile_rows == 128)
        launch_gemm<128, 2, true>(A, g, u, H, I, top_k, sorted_pairs, tiles, num_tiles, max_tile_count, o, s);
    else if (tile_rows == 32)
        launch_gemm<32, 2, true>(A, g, u, H, I, top_k, sorted_pairs, tiles, num_tiles, max_tile_count, o, s);
    else if (tile_rows == 16)
        launch_gemm<16, 1, true>(A, g, u, H, I, top_k, sorted_pairs, tiles, num_tiles, max_tile_count, o, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_down(const void* h, bool bf16, const void* w_down, int H, int I, const int32_t* sorted_pairs,
                       const TileEntry* tiles, const int32_t* num_tiles, int64_t max_tile_count, int tile_rows,
                       void* y_pair, hipStream_t s) {
    if (!bf16 || max_tile_count <= 0) return hipErrorInvalidValue;
    auto A = (const uint16_t*)h;
    auto w = (const uint16_t*)w_down;
    auto o = (uint16_t*)y_pair;
    if (tile_rows == 128)
        launch_gemm<128, 2, false>(A, w, nullptr, I, H, 0, sorted_pairs, tiles, num_tiles, max_tile_count, o, s);
    else if (tile_rows == 32)
        launch_gemm<32, 2, false>(A, w, nullptr, I, H, 0, sorted_pairs, tiles, num_tiles, max_tile_count, o, s);
    else if (tile_rows == 16)
        launch_gemm<16, 1, false>(A, w, nullptr, I, H, 0, sorted_pairs, tiles, num_tiles, max_tile_count, o, s);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---- fp32 path: one thread per output element, fp32 accumulation -----------------

__global__ void gate_up_f32_kernel(const float* __restrict__ act, const float* __restrict__ wg,
                                   const float* __restrict__ wu, int H, int I, int top_k,
                                   const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ topk_idx,
                                   int64_t P, float* __restrict__ h) {
    const int64_t n = P * I;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / I;
        const int col = (int)(i % I);
        const int p = sorted_pairs[row];
        const int64_t e = topk_idx[p];
        const int64_t t = p / top_k;
        const float* x = act + t * H;
        const float* g = wg + (e * I + col) * H;
        const float* u = wu + (e * I + col) * H;
        float a = 0.f, c = 0.f;
        for (int k = 0; k < H; ++k) {
            a = fmaf(x[k], g[k], a);
            c = fmaf(x[k], u[k], c);
        }
        h[i] = a / (1.0f + expf(-a)) * c;
    }
}

__global__ void down_f32_kernel(const float* __restrict__ h, const float* __restrict__ wd, int H, int I,
                                const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ topk_idx,
                                int64_t P, float* __restrict__ y_pair) {
    const int64_t n = P * H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / H;
        const int col = (int)(i % H);
        const int p = sorted_pairs[row];
        const int64_t e = topk_idx[p];
        const float* hr = h + row * I;
        const float* w = wd + (e * H + col) * I;
        float z = 0.f;
        for (int k = 0; k < I; ++k) z = fmaf(hr[k], w[k], z);
        y_pair[(int64_t)p * H + col] = z;
    }
}

static unsigned grid_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    return (unsigned)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

hipError_t launch_gate_up_f32(const float* act, const float* w_gate, const float* w_up, int H, int I, int top_k,
                              const int32_t* sorted_pairs, const int32_t* topk_idx, int64_t P, float* h,
                              hipStream_t s) {
    if (P > 0)
        gate_up_f32_kernel<<<grid_for(P * I), 256, 0, s>>>(act, w_gate, w_up, H, I, top_k, sorted_pairs, topk_idx, P,
                                                           h);
    return hipGetLastError();
}

hipError_t launch_down_f32(const float* h, const float* w_down, int H, int I, const int32_t* sorted_pairs,
                           const int32_t* topk_idx, int64_t P, float* y_pair, hipStream_t s) {
    if (P > 0) down_f32_kernel<<<grid_for(P * H), 256, 0, s>>>(h, w_down, H, I, sorted_pairs, topk_idx, P, y_pair);
    return hipGetLastError();
}

}  // namespace beam
