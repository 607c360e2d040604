// Token permutation on gfx950: a stable counting sort of (token, choice) pairs by
// expert, plus the grouped-GEMM work list.
//
// Pairs are cut into chunks of PERM_CHUNK.  (1) each chunk counts its experts in LDS;
// (2) one work-group scans the counts per expert over chunks and over experts, giving
// every chunk a base row per expert, the expert offsets and the tile list; (3) one
// wave per chunk walks its pairs in order and ranks equal experts with ballots, so
// rows inside an expert stay in ascending pair order (deterministic output).  A single
// chunk runs the three steps in one work-group.
#include "common.hpp"

namespace beam {

constexpr int PERM_CHUNK = 1024;
constexpr int PERM_MAX_E = 1024;

size_t permute_scratch_words(int64_t P, int E) {
    int64_t chunks = (P + PERM_CHUNK - 1) / PERM_CHUNK;
    if (chunks < 1) chunks = 1;
    return (size_t)(chunks * E);
}

__global__ void __launch_bounds__(256) perm_hist_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                        int32_t* __restrict__ counts) {
    __shared__ int32_t cnt[PERM_MAX_E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * PERM_CHUNK;
    const int64_t p1 = p0 + PERM_CHUNK < P ? p0 + PERM_CHUNK : P;
    for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
        const int e = idx[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scans over experts of the row totals `tot` and the tile counts `ntl` (thread t
// handles expert t; a 1024-thread work-group): inclusive scans inside each wave by shuffles,
// then the totals of the earlier waves.  Writes off and toff, the row total to offsets[E] and
// the tile total to *num_tiles.
__device__ __forceinline__ void perm_expert_scan(int E, const int32_t* tot, const int32_t* ntl, int32_t* off,
                                                 int32_t* toff, int32_t (*wsum)[16], int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ num_tiles) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int32_t a = tid < E ? tot[tid] : 0, b = tid < E ? ntl[tid] : 0;
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t ua = __shfl_up(a, o), ub = __shfl_up(b, o);
        if (lane >= o) {
            a += ua;
            b += ub;
        }
    }
    if (lane == 63) {
        wsum[0][w] = a;
        wsum[1][w] = b;
    }
    __syncthreads();
    int32_t pa = 0, pb = 0;
    for (int v = 0; v < w; ++v) {
        pa += wsum[0][v];
        pb += wsum[1][v];
    }
    if (tid < E) {
        off[tid] = pa + a - tot[tid];
        toff[tid] = pb + b - ntl[tid];
    }
    if (tid == 1023) {  // ids past E add zero
        offsets[E] = pa + a;
        if (num_tiles) *num_tiles = pb + b;
    }
}

// Expert offsets and the balanced tile list (n = ceil(c / tile_rows) tiles per expert, the
// rows split evenly).
__device__ __forceinline__ void perm_write_tiles(int E, const int32_t* tot, const int32_t* ntl, const int32_t* off,
                                                 const int32_t* toff, int32_t* __restrict__ offsets,
                                                 TileEntry* __restrict__ tiles) {
    for (int k = threadIdx.x; k < E; k += blockDim.x) {
        offsets[k] = off[k];
        if (tiles) {
            const int n = ntl[k];
            if (n > 0) {
                const int c = tot[k];
                const int r = (c + n - 1) / n;  // balanced rows per tile, <= tile_rows
                for (int j = 0; j < n; ++j) {
                    TileEntry te;
                    te.expert = k;
                    te.row_begin = off[k] + j * r;
                    te.row_count = (c - j * r) < r ? (c - j * r) : r;
                    te.group = n < 32768 ? (j << 16) | n : 0;
                    tiles[toff[k] + j] = te;
                }
            }
        }
    }
}

// Exclusive scan of v[0..n) into out (a 1024-thread work-group, n <= 1024; out may alias v).
__device__ __forceinline__ void perm_scan_one(int n, const int32_t* v, int32_t* out, int32_t* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int32_t own = tid < n ? v[tid] : 0;
    int32_t a = own;
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(a, o);
        if (lane >= o) a += u;
    }
    if (lane == 63) wsum[w] = a;
    __syncthreads();
    int32_t pa = 0;
    for (int q = 0; q < w; ++q) pa += wsum[q];
    if (tid < n) out[tid] = pa + a - own;
}

// Order of the experts' tiles in the work list (thread t handles expert t).  The GEMM kernels
// hand each of the 8 XCDs a contiguous eighth of the work items, so the list is dealt into 8
// runs of equal cost: experts sorted by the 16-row blocks of their tiles, largest first
// (stable by id; empty experts last), then dealt to the runs in snake order (0..7, 7..0, ...),
// each run taking its experts in that sorted order so that every compute unit starts with
// the largest items.  The sort is a stable counting sort: ballots rank each expert among the
// experts of its wave with the same key, and one scan over the (key, wave) counts in key order
// gives each its place (a loop comparing every expert with every other took 9 us of the scan
// kernel at 256 experts).  At 8192 tokens of the Beam layer (one tile per expert) each XCD gets
// 32 experts of about the same total rows instead of 32 consecutive ones, whose totals
// differed by up to 3%: on one MI355X gate/up took 3.15 instead of 3.26 ms, and the down GEMM
// after it 1.88 instead of 1.85 in either order (the faster gate/up leaves the clock lower
// when down starts), the layer 5.39 instead of 5.44 ms.  pos[t] is expert t's place in the
// list; only the order of the tiles changes, each tile's rows and results stay the same.
__device__ __forceinline__ void perm_deal_order(int E, const int32_t* tot, const int32_t* ntl, int32_t* table,
                                                int32_t* pos, int32_t* wsum) {
    // table: 1024 words of LDS, cell (63 - key) * 16 + wave: the experts of a wave with a key
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int k = -1;
    if (tid < E) {
        const int n = ntl[tid];
        k = 0;
        if (n > 0) {
            const int blocks = ((tot[tid] + n - 1) / n + 15) >> 4;
            k = 1 + (blocks < 62 ? blocks : 62);
        }
    }
    table[tid] = 0;
    __syncthreads();
    // per wave: each expert's rank among the wave's experts with its key (ballots over the
    // keys present), and the count of each key
    int rw = 0;
    if (w * 64 < E) {   // uniform per wave
        unsigned long long todo = __ballot(tid < E);
        while (todo) {
            const int leader = __builtin_ctzll(todo);
            const int kl = __shfl(k, leader);
            const unsigned long long m = __ballot(k == kl);
            if (k == kl) rw = __popcll(m & ((1ull << lane) - 1ull));
            if (lane == leader) table[(63 - kl) * 16 + w] = __popcll(m);
            todo &= ~m;
        }
    }
    __syncthreads();
    // cells in (key descending, wave ascending) order: the scan gives each cell its first rank
    perm_scan_one(1024, table, table, wsum);
    __syncthreads();
    if (tid < E) {
        const int s = table[(63 - k) * 16 + w] + rw;   // rank: larger keys, then equal keys of lower ids
        const int r = s >> 3, wb = s & 7;
        const int bin = (r & 1) ? 7 - wb : wb;
        // experts in the runs before this one: every full round gives each run one, the last
        // partial round (E % 8 experts) gives one to the first E % 8 runs of its direction
        const int full = E >> 3, m = E & 7;
        const bool fwd = (full & 1) == 0;
        int before = bin * full;
        for (int b = 0; b < bin; ++b) before += fwd ? (b < m) : (b >= 8 - m);
        pos[tid] = before + r;
    }
}

// Scan by one work-group of 1024 threads.  Thread t handles expert t % E for chunk
// group t / E (G = 1024 / E groups of consecutive chunks), so the per-expert scan over
// chunks runs in G pieces with coalesced reads of the count rows; the scans over experts
// are prefix sums across the work-group.
__device__ __forceinline__ void perm_scan_body(int32_t* __restrict__ counts, int nchunks, int E,
                                               int32_t* __restrict__ offsets, TileEntry* __restrict__ tiles,
                                               int32_t* __restrict__ num_tiles, int tile_rows) {
    __shared__ int32_t part[1024];  // [group][expert] chunk-range sums, then group bases
    __shared__ int32_t tot[PERM_MAX_E];
    __shared__ int32_t off[PERM_MAX_E];
    __shared__ int32_t ntl[PERM_MAX_E];
    __shared__ int32_t toff[PERM_MAX_E];   // first the sort's (key, wave) table
    __shared__ int32_t pos[PERM_MAX_E];
    __shared__ int32_t ntl_pos[PERM_MAX_E];   // tile counts in work-list order, then their scan
    __shared__ int32_t wsum[2][16];
    const int tid = threadIdx.x;
    const int G = 1024 / E;  // >= 1 since E <= 1024
    const int e = tid % E, g = tid / E;
    const int cpg = (nchunks + G - 1) / G;
    const int c0 = g * cpg, c1 = (g + 1) * cpg < nchunks ? (g + 1) * cpg : nchunks;
    // (1) sum of each chunk range (eight count rows in flight)
    if (g < G) {
        int32_t sum = 0;
        for (int cb = c0; cb < c1; cb += 8) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = cb + u < c1 ? counts[(int64_t)(cb + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        part[g * E + e] = sum;
    }
    __syncthreads();
    // (2) per expert: exclusive scan over the groups and the expert total
    if (tid < E) {
        int32_t run = 0;
        for (int gg = 0; gg < G; ++gg) {
            const int32_t v = part[gg * E + tid];
            part[gg * E + tid] = run;
            run += v;
        }
        tot[tid] = run;
        ntl[tid] = run > 0 ? (run + tile_rows - 1) / tile_rows : 0;
    }
    __syncthreads();
    // (3) the experts' order in the work list (toff is scratch here), then exclusive scans of
    // the row counts over experts and of the tile counts in that order
    perm_deal_order(E, tot, ntl, toff, pos, wsum[0]);
    __syncthreads();
    if (tid < E) ntl_pos[pos[tid]] = ntl[tid];
    __syncthreads();
    perm_expert_scan(E, tot, ntl_pos, off, ntl_pos, wsum, offsets, num_tiles);
    __syncthreads();
    if (tid < E) toff[tid] = ntl_pos[pos[tid]];
    __syncthreads();
    // (4) every chunk's first row per expert: expert offset + earlier chunks' counts
    if (g < G) {
        int32_t run = off[e] + part[g * E + e];
        for (int cb = c0; cb < c1; cb += 8) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = cb + u < c1 ? counts[(int64_t)(cb + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (cb + u < c1) {
                    counts[(int64_t)(cb + u) * E + e] = run;
                    run += v[u];
                }
        }
    }
    // (5) expert offsets and the balanced tile list
    perm_write_tiles(E, tot, ntl, off, toff, offsets, tiles);
}

__global__ void __launch_bounds__(1024) perm_scan_kernel(int32_t* __restrict__ counts, int nchunks, int E,
                                                         int32_t* __restrict__ offsets, TileEntry* __restrict__ tiles,
                                                         int32_t* __restrict__ num_tiles, int tile_rows) {
    perm_scan_body(counts, nchunks, E, offsets, tiles, num_tiles, tile_rows);
}

// The expert ids of a chunk's pairs, 64 per slice: lane l holds pair p0 + 64 s + l of
// slice s (-1 past p1), all loaded before the ranking starts.
constexpr int PERM_SLICES = PERM_CHUNK / 64;
__device__ __forceinline__ void perm_load_ids(const int32_t* __restrict__ idx, int64_t p0, int64_t p1, int lane,
                                              int (&ev)[PERM_SLICES]) {
#pragma unroll
    for (int sl = 0; sl < PERM_SLICES; ++sl) {
        const int64_t p = p0 + sl * 64 + lane;
        ev[sl] = p < p1 ? idx[p] : -1;
    }
}

// One wave places the 64 pairs [pb, pb + 64) whose expert ids the lanes hold in `e` (-1
// past the end): lanes with equal experts are ranked by ballots in pair order, and `next`
// holds each expert's next row.  The caller makes the cursor updates visible (a barrier)
// before the next 64 pairs.
__device__ __forceinline__ void perm_scatter_step(int e, int64_t pb, int E, int ebits, int32_t* next,
                                                  int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
                                                  int lane) {
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t p = pb + lane;
    const bool valid = e >= 0 && e < E;  // out-of-range ids are skipped
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    if (valid) {
        const int rank = __popcll(peers & lt_mask);
        const int32_t dest = next[e] + rank;
        sorted_pairs[dest] = (int32_t)p;
        pair_pos[p] = dest;
        // the highest lane of the peer group advances the expert's cursor
        if ((peers >> lane) == 1ull) next[e] += __popcll(peers);
    }
}

__device__ __forceinline__ int perm_ebits(int E) {
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    return ebits;
}

__global__ void __launch_bounds__(64) perm_scatter_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                          const int32_t* __restrict__ base,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_pos) {
    __shared__ int32_t next[PERM_MAX_E];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) next[e] = base[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    const int ebits = perm_ebits(E);
    const int64_t p0 = (int64_t)blockIdx.x * PERM_CHUNK;
    const int64_t p1 = p0 + PERM_CHUNK < P ? p0 + PERM_CHUNK : P;
    int ev[PERM_SLICES];
    perm_load_ids(idx, p0, p1, lane, ev);
#pragma unroll
    for (int sl = 0; sl < PERM_SLICES; ++sl) {
        if (p0 + sl * 64 >= p1) break;   // uniform
        perm_scatter_step(ev[sl], p0 + sl * 64, E, ebits, next, sorted_pairs, pair_pos, lane);
        __syncthreads();
    }
}

// All pairs in one chunk (1 <= P <= PERM_CHUNK): histogram, scan and scatter in one
// work-group of 1024 threads, saving two dependent launches for decode-sized batches.
// The histogram goes through `counts` (E words of the scratch) so the scan reads it as
// in the multi-chunk path; wave 0 then places the pairs.
__global__ void __launch_bounds__(1024) perm_single_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_pairs,
                                                           int32_t* __restrict__ pair_pos,
                                                           TileEntry* __restrict__ tiles,
                                                           int32_t* __restrict__ num_tiles, int tile_rows) {
    // one chunk: the counts, the scans and the cursors stay in LDS
    __shared__ int32_t cnt[PERM_MAX_E];
    __shared__ int32_t ntl[PERM_MAX_E];
    __shared__ int32_t off[PERM_MAX_E];
    __shared__ int32_t toff[PERM_MAX_E];
    __shared__ int32_t next[PERM_MAX_E];
    __shared__ int32_t wsum[2][16];
    const int tid = threadIdx.x;
    int ev[PERM_SLICES];   // wave 0's ids for the scatter, in flight during the count and scan
    if (tid < 64) perm_load_ids(idx, 0, P, tid, ev);
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    if (tid < P) {
        const int e = idx[tid];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid < E) ntl[tid] = cnt[tid] > 0 ? (cnt[tid] + tile_rows - 1) / tile_rows : 0;
    __syncthreads();
    perm_expert_scan(E, cnt, ntl, off, toff, wsum, offsets, num_tiles);
    __syncthreads();
    if (tid < E) next[tid] = off[tid];
    perm_write_tiles(E, cnt, ntl, off, toff, offsets, tiles);
    __syncthreads();
    const int ebits = perm_ebits(E);
#pragma unroll
    for (int sl = 0; sl < PERM_SLICES; ++sl) {
        if (sl * 64 >= P) break;   // uniform
        if (tid < 64) perm_scatter_step(ev[sl], sl * 64, E, ebits, next, sorted_pairs, pair_pos, tid);
        __syncthreads();
    }
}

hipError_t launch_permute(const int32_t* idx, int64_t P, int E, int32_t* scratch, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, TileEntry* tiles, int32_t* num_tiles,
                          int tile_rows, hipStream_t s) {
    int nchunks = (int)((P + PERM_CHUNK - 1) / PERM_CHUNK);
    if (nchunks == 1) {
        perm_single_kernel<<<1, 1024, 0, s>>>(idx, P, E, offsets, sorted_pairs, pair_pos, tiles, num_tiles,
                                              tile_rows);
        return hipGetLastError();
    }
    if (nchunks > 0) perm_hist_kernel<<<nchunks, 256, 0, s>>>(idx, P, E, scratch);
    perm_scan_kernel<<<1, 1024, 0, s>>>(scratch, nchunks, E, offsets, tiles, num_tiles, tile_rows);
    if (nchunks > 0) perm_scatter_kernel<<<nchunks, 64, 0, s>>>(idx, P, E, scratch, sorted_pairs, pair_pos);
    return hipGetLastError();
}

}  // namespace beam
