// Device helpers and the internal launcher interface of the Beam MoE library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace beam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// One grouped-GEMM tile: `row_count` consecutive rows of the expert-sorted pair list
// starting at `row_begin`, all routed to `expert`.  `group` = (j << 16) | n when the tile is
// tile j of the n (< 32768) tiles of its expert, else 0.
struct TileEntry {
    int32_t expert;
    int32_t row_begin;
    int32_t row_count;
    int32_t group;
};

// Work item -> (tile, column block).  The items of an expert's tiles form one run of
// n_tiles * n_col_blocks items ordered column block first, so the n tiles of an expert that
// needs several read the same weight columns one after the other (from L2 for all but the
// first); an expert of one tile keeps its column blocks in order.
__device__ __forceinline__ void item_tile(const TileEntry* __restrict__ tiles, int item, int n_col_blocks, int& tile,
                                          int& cblk) {
    const int t0 = item / n_col_blocks;
    const int grp = tiles[t0].group;
    const int n = grp & 0xFFFF;
    if (n > 1) {
        const int first = t0 - (grp >> 16);
        const int local = item - first * n_col_blocks;
        cblk = local / n;
        tile = first + local % n;
    } else {
        tile = t0;
        cblk = item - t0 * n_col_blocks;
    }
}

// ---- launchers (each returns hipGetLastError() of its launches) ----------------

hipError_t launch_rmsnorm(const uint16_t* x, const float* gain, float eps, int64_t T, int H, uint16_t* u,
                          hipStream_t s);

// number of H ranges the bf16 router splits its reduction into (1 for fp32)
int router_splits(int64_t T, int H, int E);

// fp64 partial logits part[nsplit][T][E] from activations (bf16 or fp32; fp32 needs
// nsplit == 1) and the fp32 router matrix
hipError_t launch_router_logits(const void* x, bool bf16, const float* w_router, int64_t T, int H, int E,
                                int nsplit, double* part, hipStream_t s);

// sums the partials in split order, rounds the logits to fp32 (written to logits_out
// when non-null) and selects the experts
hipError_t launch_router_select(const double* part, int nsplit, const float* bias, int64_t T, int E, int n_group,
                                int topk_group, int top_k, float rho, int32_t* idx, float* w, float* logits_out,
                                hipStream_t s);

// scratch words the permutation needs for P pairs and E experts
size_t permute_scratch_words(int64_t P, int E);

// stable counting sort of pairs by expert; when tiles != nullptr also the GEMM
// work list with at most `tile_rows` rows per tile (count in *num_tiles)
hipError_t launch_permute(const int32_t* idx, int64_t P, int E, int32_t* scratch, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, TileEntry* tiles, int32_t* num_tiles,
                          int tile_rows, hipStream_t s);

// upper bound on the number of tiles of at most `tile_rows` rows
inline int64_t max_tiles(int64_t P, int E, int tile_rows) { return (P + tile_rows - 1) / tile_rows + E; }

// expert weight storage: bf16, OCP FP8 E4M3 codes, or OCP FP4 E2M1 codes two per byte (the
// last two with one E8M0 scale byte per 32 elements of a row along K)
constexpr int WF_BF16 = 0, WF_E4M3 = 1, WF_E2M1 = 2;

// rows per GEMM tile the forward pass uses for P pairs over E experts with weight format
// wf (it depends on which GEMM kernel takes the batch), and the smallest it ever uses (the
// workspace bounds the tile count with it)
int gemm_tile_rows(int64_t P, int E, int H, int I, bool bf16, int wf);
int gemm_min_tile_rows();
// bits per stored weight
__host__ __device__ constexpr int wbits(int wf) { return wf == WF_BF16 ? 16 : wf == WF_E4M3 ? 8 : 4; }

// h[row, :] = silu(A W_g^T) * (A W_u^T) for the expert-sorted rows (A = gathered token rows)
// (act: T token rows; the activation and h tensors must stay below 4 GiB).  Weights stored
// as `wf`; quantized formats come with s_gate and s_up (bf16: null).
hipError_t launch_gate_up(const void* act, bool bf16, const void* w_gate, const void* w_up, int wf,
                          const uint8_t* s_gate, const uint8_t* s_up, int64_t T, int H, int I, int E, int top_k,
                          const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                          int64_t max_tile_count, int tile_rows, void* h, hipStream_t s);

// y_pair[sorted_pairs[row], :] = h[row, :] W_d^T   (h: P rows of the T tokens' routes; quantized
// weights with s_down)
hipError_t launch_down(const void* h, bool bf16, const void* w_down, int wf, const uint8_t* s_down, int64_t T,
                       int64_t P, int H, int I, int E, const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                       int64_t max_tile_count, int tile_rows, void* y_pair, hipStream_t s);

// fp32 path (no tiles): one thread per output element
hipError_t launch_gate_up_f32(const float* act, const float* w_gate, const float* w_up, int H, int I, int top_k,
                              const int32_t* sorted_pairs, const int32_t* topk_idx, int64_t P, float* h,
                              hipStream_t s);
hipError_t launch_down_f32(const float* h, const float* w_down, int H, int I, const int32_t* sorted_pairs,
                           const int32_t* topk_idx, int64_t P, float* y_pair, hipStream_t s);

// out[t] = sum_j w[t,j] y_pair[t*K + j] (+ post-norm and residual when post_gain != nullptr)
hipError_t launch_combine(const void* y_pair, bool bf16, const float* topk_w, int64_t T, int H, int K,
                          const void* x, const float* post_gain, float eps, float residual_k, void* out, void* moe_y,
                          hipStream_t s);

}  // namespace beam
