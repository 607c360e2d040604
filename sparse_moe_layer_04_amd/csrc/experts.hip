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
// bf16 path (details below): one work-group computes one (tile, column block) on
// MFMA.  Gate/up column blocks hold the gate and the up rows of the same output
// columns, so the SwiGLU epilogue has both operands in registers.  The gate/up A
// operand is gathered straight from the token rows (no permuted copy); the down
// epilogue scatters each row to its pair position.
#include "common.hpp"

#include <type_traits>

namespace beam {

// ---------------------------------------------------------------------------------
// bf16 grouped GEMM on MFMA (16x16x32, fp32 accumulation).
//
// Work item: (tile, column block).  A tile is up to GROWS = 288 consecutive rows of the
// expert-sorted pair list, all routed to one expert (row_count may be smaller; 16-row
// blocks past it are skipped).  A column block is 128 h columns (gate/up: 8 waves x
// (16 gate + 16 up weight rows)) or 256 output columns (down: 8 waves x 32 weight
// rows).  Each wave owns its weight rows: they stream from HBM straight into
// registers, never through LDS.  All waves share the tile's activation rows
// through an LDS double buffer.  K is swept 32 at a time; global loads of both
// operands run 3 steps ahead in a ring of 4 register sets (one VMEM counter orders
// both streams, so they share the prefetch distance).
// ---------------------------------------------------------------------------------
constexpr int GROWS = 288;    // rows per tile: at 8192 tokens almost every expert fits one tile
constexpr int GRB = GROWS / 16;
constexpr int GKS = 32;       // k per step (one MFMA)
constexpr int GWAVES = 8;
constexpr int GTHREADS = GWAVES * 64;
constexpr int GRING = 4;      // register sets: 3 steps in flight + 1 in use

// LDS element offset of 16-byte chunk `ch` (0..3) of activation row `row` (64-byte rows).
// The MFMA operand read (lane -> row lane&15, chunk lane>>4) and the staging write are
// free of bank conflicts on gfx950 with this XOR (measured with the LDS bank-conflict
// counter over candidate layouts).
__device__ __forceinline__ int a_off(int row, int ch) { return row * GKS + ((ch ^ ((row >> 1) & 3)) << 3); }

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-tile context shared by the row-count variants of the main loop.
struct TileCtx {
    const uint16_t* A;    // activations (gate/up: token rows, gathered) or h (down)
    const uint16_t* bp0;  // this lane's first weight row (k offset applied)
    const uint16_t* bp1;  // second weight row block (up rows, or the next 16 down rows)
    int K, nk, top_k;     // reduction length, its 32-wide steps, routes per token
    int row_begin, row_count, ccol, N;
    const int32_t* sorted_pairs;
    uint16_t* C;
};

// Main loop and epilogue for tiles of at most NRB 16-row blocks, with global loads
// RING - 1 steps ahead.  Every load and store is unconditional (clamped addresses), so
// the steady state has no branches and the compiler's memory-counter waits stay exact.
// Only the NRB*16 activation rows the variant reads are loaded: thread t stages chunk
// (t + 512 i) mod (NRB*64), so small tiles reload (cached) chunks instead of branching.
template <bool GATED, int NRB, int RING>
__device__ __forceinline__ void tile_body(const TileCtx& c, uint16_t (*lds)[GROWS * GKS]) {
    constexpr int ACH = NRB * 64;                          // 16-byte activation chunks per step
    constexpr int AL = (ACH + GTHREADS - 1) / GTHREADS;    // activation loads per thread per step
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x;
    const uint16_t* ap[AL];
    int alds[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int q = (tid + i * GTHREADS) % ACH;
        const int row = q >> 2, ch = q & 3;
        const int src = row < c.row_count ? row : 0;  // rows past the tile read row 0 (never stored)
        const int64_t arow = GATED ? (int64_t)(c.sorted_pairs[c.row_begin + src] / c.top_k)
                                   : (int64_t)(c.row_begin + src);
        ap[i] = c.A + arow * c.K + ch * 8;
        alds[i] = a_off(row, ch);
    }

    u32x4 ra[RING][AL], rb[RING][2];
    f32x4 acc[NRB][2];
#pragma unroll
    for (int i = 0; i < NRB; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = c.nk;
    auto load = [&](int kstep, int set) {
        const int k0 = (kstep < nk ? kstep : nk - 1) * GKS;  // past the end: reload the last step
#pragma unroll
        for (int i = 0; i < AL; ++i) ra[set][i] = *(const u32x4*)(ap[i] + k0);
        rb[set][0] = *(const u32x4*)(c.bp0 + k0);
        rb[set][1] = *(const u32x4*)(c.bp1 + k0);
    };
    auto store_a = [&](int set, int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) *(u32x4*)(&lds[buf][alds[i]]) = ra[set][i];
    };
    const int rd_row = lane & 15, rd_ch = lane >> 4;
    auto compute = [&](int set, int buf) {
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, rb[set][0]);
        const bf16x8 b1 = __builtin_bit_cast(bf16x8, rb[set][1]);
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            const bf16x8 a = *(const bf16x8*)(&lds[buf][a_off(r * 16 + rd_row, rd_ch)]);
            acc[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc[r][0], 0, 0, 0);
            acc[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc[r][1], 0, 0, 0);
        }
    };
    // one K step; `j` (= kt % RING) is a compile-time constant in the unrolled loop
    auto step = [&](int kt, auto jc) {
        constexpr int j = decltype(jc)::value;
        load(kt + RING - 1, (j + RING - 1) % RING);
        compute(j, j & 1);
        store_a((j + 1) % RING, (j + 1) & 1);
        lds_barrier();
    };

#pragma unroll
    for (int s = 0; s < RING - 1; ++s) load(s, s);
    store_a(0, 0);
    lds_barrier();
    for (int kt = 0; kt < nk; kt += RING) {  // nk is a multiple of RING
        step(kt, std::integral_constant<int, 0>());
        step(kt + 1, std::integral_constant<int, 1>());
        step(kt + 2, std::integral_constant<int, 2>());
        step(kt + 3, std::integral_constant<int, 3>());
        if constexpr (RING == 8) {
            step(kt + 4, std::integral_constant<int, 4>());
            step(kt + 5, std::integral_constant<int, 5>());
            step(kt + 6, std::integral_constant<int, 6>());
            step(kt + 7, std::integral_constant<int, 7>());
        }
    }

    // ---- epilogue (C layout of a 16x16 block: rows 4*(lane>>4)+q, column lane&15) ----
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = r * 16 + 4 * (lane >> 4) + q;
            if (m >= c.row_count) continue;
            if (GATED) {
                const float g = acc[r][0][q];
                const float u = acc[r][1][q];
                c.C[(int64_t)(c.row_begin + m) * c.N + c.ccol] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
            } else {
                const int64_t p = c.sorted_pairs[c.row_begin + m];
                c.C[p * c.N + c.ccol] = f32_to_bf16(acc[r][0][q]);
                c.C[p * c.N + c.ccol + 16] = f32_to_bf16(acc[r][1][q]);
            }
        }
    }
}

template <bool GATED>
__global__ void __launch_bounds__(GTHREADS) moe_gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                                 const uint16_t* __restrict__ B0,
                                                                 const uint16_t* __restrict__ B1, int K, int N,
                                                                 int top_k, const int32_t* __restrict__ sorted_pairs,
                                                                 const TileEntry* __restrict__ tiles,
                                                                 const int32_t* __restrict__ num_tiles,
                                                                 int n_col_blocks, uint16_t* __restrict__ C) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][GROWS * GKS];

    // XCD-aware order: blocks are dealt round-robin to the 8 XCDs, so give each XCD a
    // contiguous run of work items (the column blocks of one tile share its activation
    // rows in that XCD's L2).
    const int work = *num_tiles * n_col_blocks;
    const int per_xcd = (work + 7) >> 3;
    const int slot = (int)(blockIdx.x >> 3);
    if (slot >= per_xcd) return;
    const int item = (int)(blockIdx.x & 7) * per_xcd + slot;
    if (item >= work) return;
    const TileEntry te = tiles[item / n_col_blocks];
    const int cblk = item % n_col_blocks;
    if (te.row_count <= 0) return;
    const int e = te.expert;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    TileCtx c;
    c.nk = K / GKS;
    c.row_begin = te.row_begin;
    c.row_count = te.row_count;
    c.N = N;
    c.sorted_pairs = sorted_pairs;
    c.C = C;
    // weight rows of this wave (two 16-row MFMA operand blocks)
    int col0;
    if (GATED) {
        col0 = cblk * (GWAVES * 16) + wave * 16;
        const int64_t r = (int64_t)e * N + col0 + (lane & 15);
        c.bp0 = B0 + r * K + (lane >> 4) * 8;
        c.bp1 = B1 + r * K + (lane >> 4) * 8;
    } else {
        col0 = cblk * (GWAVES * 32) + wave * 32;
        const int64_t r = (int64_t)e * N + col0 + (lane & 15);
        c.bp0 = B0 + r * K + (lane >> 4) * 8;
        c.bp1 = c.bp0 + (int64_t)16 * K;
    }
    c.ccol = col0 + (lane & 15);
    c.A = A;
    c.K = K;
    c.top_k = top_k;

    // row-count variants; small tiles are load-latency bound and keep 7 steps in flight
    const int nrb = (te.row_count + 15) >> 4;
    const bool deep = (c.nk & 7) == 0;
    if (nrb > 16)
        tile_body<GATED, 18, 4>(c, lds);
    else if (nrb > 12)
        tile_body<GATED, 16, 4>(c, lds);
    else if (nrb > 8)
        tile_body<GATED, 12, 4>(c, lds);
    else if (nrb > 4)
        tile_body<GATED, 8, 4>(c, lds);
    else if (nrb > 2)
        tile_body<GATED, 4, 4>(c, lds);
    else if (nrb > 1)
        deep ? tile_body<GATED, 2, 8>(c, lds) : tile_body<GATED, 2, 4>(c, lds);
    else
        deep ? tile_body<GATED, 1, 8>(c, lds) : tile_body<GATED, 1, 4>(c, lds);
}

int gemm_tile_rows(int64_t P, int E, bool bf16) {
    (void)P;
    (void)E;
    return bf16 ? GROWS : (1 << 30);  // the fp32 path does not use tiles
}

template <bool GATED>
static void launch_gemm(const uint16_t* A, const uint16_t* B0, const uint16_t* B1, int K, int N, int top_k,
                        const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                        int64_t max_tile_count, uint16_t* C, hipStream_t s) {
    const int ncols = GATED ? GWAVES * 16 : GWAVES * 32;
    const int ncb = N / ncols;
    const int64_t blocks = (max_tile_count * ncb + 7) / 8 * 8;
    moe_gemm_bf16_kernel<GATED><<<(unsigned)blocks, GTHREADS, 0, s>>>(A, B0, B1, K, N, top_k, sorted_pairs, tiles,
                                                                     num_tiles, ncb, C);
}

hipError_t launch_gate_up(const void* act, bool bf16, const void* w_gate, const void* w_up, int H, int I, int top_k,
                          const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                          int64_t max_tile_count, int tile_rows, void* h, hipStream_t s) {
    if (!bf16 || max_tile_count <= 0 || tile_rows != GROWS) return hipErrorInvalidValue;
    launch_gemm<true>((const uint16_t*)act, (const uint16_t*)w_gate, (const uint16_t*)w_up, H, I, top_k, sorted_pairs,
                      tiles, num_tiles, max_tile_count, (uint16_t*)h, s);
    return hipGetLastError();
}

hipError_t launch_down(const void* h, bool bf16, const void* w_down, int H, int I, const int32_t* sorted_pairs,
                       const TileEntry* tiles, const int32_t* num_tiles, int64_t max_tile_count, int tile_rows,
                       void* y_pair, hipStream_t s) {
    if (!bf16 || max_tile_count <= 0 || tile_rows != GROWS) return hipErrorInvalidValue;
    launch_gemm<false>((const uint16_t*)h, (const uint16_t*)w_down, nullptr, I, H, 0, sorted_pairs, tiles, num_tiles,
                       max_tile_count, (uint16_t*)y_pair, s);
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
