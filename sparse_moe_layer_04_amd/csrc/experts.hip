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
// bf16 path (details below): one work-group computes one (tile, column block) on bf16
// MFMA.  Expert weights are bf16, or E4M3 / E2M1 codes with E8M0 block scales that are
// decoded exactly to bf16 in registers (template parameter WF).  Gate/up column blocks
// hold the gate and the up rows of the same output columns, so the SwiGLU epilogue has
// both operands in registers.  The gate/up A operand is gathered straight from the token
// rows (no permuted copy); the down epilogue scatters each row to its pair position.
#include "common.hpp"

#include <type_traits>
#include <utility>

namespace beam {

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>)
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

// ---------------------------------------------------------------------------------
// bf16 grouped GEMM on MFMA (16x16x32, fp32 accumulation).
//
// Work item: (tile, column block).  A tile is up to GROWS = 288 consecutive rows of the
// expert-sorted pair list, all routed to one expert (row_count may be smaller; 16-row
// blocks past it are skipped).  A column block is WAVES x 16 h columns (gate/up: each
// wave 16 gate + 16 up weight rows) or WAVES x 32 output columns (down: 32 weight rows
// per wave).  Each wave owns its weight rows: they stream from HBM straight into
// registers, never through LDS.  All waves share the tile's activation rows
// through an LDS double buffer.  K is swept 32 at a time; global loads of both
// operands run 3 steps ahead in a ring of 4 register sets (one VMEM counter orders
// both streams, so they share the prefetch distance).
// ---------------------------------------------------------------------------------
constexpr int GROWS = 288;    // rows per tile: at 8192 tokens almost every expert fits one tile
constexpr int GKS = 32;       // k per step (one MFMA)

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

// ---- Quantized weights: OCP FP8 E4M3 codes (one byte each) or OCP FP4 E2M1 codes (MXFP4:
// two per byte, the even element in bits 0..3), with one E8M0 scale byte per 32 elements of
// a row along K (the weight is code value * 2^(scale - 127)).  An E4M3 or E2M1 value times a
// power of two is exactly a bf16 value (at most 3 mantissa bits, exponents in range), so the
// weights are decoded exactly to bf16 in registers and the bf16 MFMA path is unchanged. ----
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// factor 2^(s - 127) of an E8M0 scale byte s (1..254)
__device__ __forceinline__ float e8m0_factor(uint32_t s) { return __uint_as_float(s << 23); }

// 8 E4M3 codes (dword lo holds codes 0..3, byte 0 first; hi codes 4..7) times `scale`
__device__ __forceinline__ bf16x8 decode8(uint32_t lo, uint32_t hi, float scale) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 E2M1 codes (dword w, element 0 in bits 0..3, element 7 in bits 28..31) times `scale`
__device__ __forceinline__ bf16x8 decode8_fp4(uint32_t w, float scale) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Per-tile context shared by the row-count variants of the main loop.  Weight pointers
// are byte pointers (2 bytes per bf16 weight, 1 per E4M3 code, 1/2 per E2M1 code).
struct TileCtx {
    const uint16_t* A;    // activations (gate/up: token rows, gathered) or h (down)
    const uint8_t* bp0;   // this lane's first weight row (k offset applied)
    const uint8_t* bp1;   // second weight row block (up rows, or the next 16 down rows)
    const uint8_t* sp0;   // quantized weights: the scale rows of bp0's and bp1's rows
    const uint8_t* sp1;
    int K, nk, top_k;     // reduction length, its 32-wide steps, routes per token
    bool gather;          // activation rows come from token rows via sorted_pairs
    int row_begin, row_count, ccol, N;
    const int32_t* sorted_pairs;
    uint16_t* C;
};

// Activation source row of tile row `row` (rows past the tile read row 0; their results
// are never stored).
__device__ __forceinline__ const uint16_t* act_row(const TileCtx& c, int row) {
    const int src = row < c.row_count ? row : 0;
    const int64_t r = c.gather ? (int64_t)(c.sorted_pairs[c.row_begin + src] / c.top_k) : (int64_t)(c.row_begin + src);
    return c.A + r * c.K;
}

// Main loop for tiles of at most NRB 16-row blocks (tiles of up to 4 blocks take the
// streaming loop below when K is a multiple of its chunk).  Activations go
// through an LDS double buffer: one register set stages step kt+2 while step kt+1 is
// written to LDS and step kt is multiplied; weights stream RING-1 steps ahead.  Within
// a step the loads are issued activations first, then weights, so waiting for the
// staged activations never waits for the newest weight loads.  Every load and store is
// unconditional (clamped addresses): the steady state has no branches and the
// compiler's memory-counter waits stay exact.  Thread t stages chunk (t + THREADS i)
// mod (NRB*64), so smaller variants reload cached chunks instead of branching.
template <bool GATED, int WF, int NRB, int RING, int THREADS>
__device__ __forceinline__ void tile_body(const TileCtx& c, uint16_t (*lds)[GROWS * GKS], f32x4 (&acc)[NRB][2]) {
    constexpr int ACH = NRB * 64;                          // 16-byte activation chunks per step
    constexpr int AL = (ACH + THREADS - 1) / THREADS;      // activation loads per thread per step
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x;
    const uint16_t* ap[AL];
    int alds[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int q = (tid + i * THREADS) % ACH;
        const int row = q >> 2, ch = q & 3;
        ap[i] = act_row(c, row) + ch * 8;
        alds[i] = a_off(row, ch);
    }

    u32x4 sa[AL], rb[RING][2];
    uint32_t rs[RING][2];   // quantized weights: the scale bytes of the step (one 32-k block)
    const int nk = c.nk;
    auto clampk = [&](int kstep) { return (kstep < nk ? kstep : nk - 1) * GKS; };
    auto load_a = [&](int kstep) {
        const int k0 = clampk(kstep);
#pragma unroll
        for (int i = 0; i < AL; ++i) sa[i] = *(const u32x4*)(ap[i] + k0);
    };
    auto load_b = [&](int kstep, int set) {
        const int k0 = clampk(kstep);
        if constexpr (WF == WF_E4M3) {
            const uint2 w0 = *(const uint2*)(c.bp0 + k0);
            const uint2 w1 = *(const uint2*)(c.bp1 + k0);
            rb[set][0] = u32x4{w0.x, w0.y, 0u, 0u};
            rb[set][1] = u32x4{w1.x, w1.y, 0u, 0u};
        } else if constexpr (WF == WF_E2M1) {
            rb[set][0] = u32x4{*(const uint32_t*)(c.bp0 + k0 / 2), 0u, 0u, 0u};
            rb[set][1] = u32x4{*(const uint32_t*)(c.bp1 + k0 / 2), 0u, 0u, 0u};
        }
        if constexpr (WF != WF_BF16) {
            rs[set][0] = c.sp0[k0 / 32];
            rs[set][1] = c.sp1[k0 / 32];
        } else {
            rb[set][0] = *(const u32x4*)(c.bp0 + 2 * k0);
            rb[set][1] = *(const u32x4*)(c.bp1 + 2 * k0);
        }
    };
    auto wfrag = [&](int set, int blk) {
        if constexpr (WF == WF_E4M3)
            return decode8(rb[set][blk][0], rb[set][blk][1], e8m0_factor(rs[set][blk]));
        else if constexpr (WF == WF_E2M1)
            return decode8_fp4(rb[set][blk][0], e8m0_factor(rs[set][blk]));
        else
            return __builtin_bit_cast(bf16x8, rb[set][blk]);
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) *(u32x4*)(&lds[buf][alds[i]]) = sa[i];
    };
    const int rd_row = lane & 15, rd_ch = lane >> 4;
    // fragment reads run LOOKAHEAD row blocks ahead of the MFMAs that use them
    constexpr int LOOKAHEAD = NRB < 4 ? NRB : 4;
    auto compute = [&](int set, int buf) {
        const bf16x8 b0 = wfrag(set, 0);
        const bf16x8 b1 = wfrag(set, 1);
        bf16x8 a[NRB];
#pragma unroll
        for (int r = 0; r < LOOKAHEAD; ++r) a[r] = *(const bf16x8*)(&lds[buf][a_off(r * 16 + rd_row, rd_ch)]);
        __builtin_amdgcn_sched_group_barrier(0x100, LOOKAHEAD, 0);
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            if (r + LOOKAHEAD < NRB) {
                a[r + LOOKAHEAD] = *(const bf16x8*)(&lds[buf][a_off((r + LOOKAHEAD) * 16 + rd_row, rd_ch)]);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            acc[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], b0, acc[r][0], 0, 0, 0);
            acc[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], b1, acc[r][1], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
    };
    // one K step; `j` (= kt % RING) is a compile-time constant in the unrolled loop
    auto step = [&](int kt, auto jc) {
        constexpr int j = decltype(jc)::value;
        // the scheduling barriers keep this issue order (the compiler would otherwise
        // sink the activation loads behind the weight loads and wait on both)
        store_a((j + 1) & 1);                       // activations of step kt+1
        __builtin_amdgcn_sched_barrier(0);
        load_a(kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        load_b(kt + RING - 1, (j + RING - 1) % RING);
        __builtin_amdgcn_sched_barrier(0);
        compute(j, j & 1);
        lds_barrier();
    };

    // prologue in the steady-state issue order (activations, then weights), so the loop
    // head sees the same outstanding loads from either path
    load_a(0);
    store_a(0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < RING - 1; ++s) {
        load_b(s, s);
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
    for (int kt = 0; kt < nk; kt += RING) {  // nk is a multiple of RING
        step(kt, std::integral_constant<int, 0>());
        step(kt + 1, std::integral_constant<int, 1>());
        step(kt + 2, std::integral_constant<int, 2>());
        step(kt + 3, std::integral_constant<int, 3>());
    }
}

// Main loop for tiles of at most NRB <= 4 row blocks (decode-sized), where the weight
// stream is the whole cost.  A step covers one 128-byte line of every weight row (64 k of
// bf16, 128 k of E4M3, 256 k of E2M1; E2M1 at 64-row tiles half a line, 128 k): lane
// (row, g = lane>>4) of a 16-row block loads the 32 bytes at 32*g of its row's line with
// two 16-byte loads (half lines: the 16 bytes at 16*g), so the loads of a step cover whole
// lines of 16 rows; the step's MFMAs take the lane's elements 8 at a time (the activation
// operand uses the same k order).  Weights run RING-1 steps
// ahead.  Activations are staged through LDS in chunks of SKC columns for all rows of the
// tile (one barrier per chunk); the next chunk's global loads are issued a whole chunk
// ahead.  Quantized weights: each wave copies the scale rows of its two blocks (16 rows x
// K/32 bytes each, contiguous in memory) into its own LDS area once per tile with whole-line
// loads, and reads the 16 scale bytes of a row and chunk from there.
constexpr int SKC = 512;            // activation columns per LDS chunk (tiles of 16 rows)
// activation columns per chunk for tiles of NRB row blocks: the same LDS bytes at every size
__host__ __device__ constexpr int stream_chunk(int nrb) { return nrb <= 1 ? 512 : nrb <= 2 ? 256 : 128; }
// bytes of each weight row per step: one 128-byte line; E2M1 at 64-row tiles half a line (a
// whole line is 256 k, more than their 128-column chunks)
__host__ __device__ constexpr int stream_step_bytes(int wf, int nrb) {
    return wf == WF_E2M1 && stream_chunk(nrb) < 256 ? 64 : 128;
}
constexpr int SACT_ELEMS = 2 * 16 * SKC;   // the double-buffered activation chunks
constexpr int SCALE_KMAX = 8192;    // longest K whose scale rows fit the per-wave LDS area
constexpr int SCALE_KMAX_SMALL = 5120;   // the same for the small-tile kernel
__host__ __device__ constexpr int scale_wave_bytes(int kmax) { return 2 * 16 * (kmax / 32); }
constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// LDS element offset of 16-byte chunk `ch` (0..C/8-1) of activation row `row` (C columns per row)
template <int C>
__device__ __forceinline__ int s_off(int row, int ch) { return row * C + ((ch ^ (row & 15)) << 3); }

template <bool GATED, int WF, int NRB, int RING, int THREADS, int SKMAX>
__device__ __forceinline__ void tile_body_stream(const TileCtx& c, uint16_t* lds, f32x4 (&acc)[NRB][2]) {
    constexpr int ROWS = NRB * 16;
    constexpr int SKC = stream_chunk(NRB);
    static_assert(2 * ROWS * SKC <= SACT_ELEMS, "activation chunks fit their LDS area");
    constexpr int ACH = ROWS * SKC / 8;          // 16-byte chunks per activation chunk
    constexpr int AL = ACH / THREADS;            // per thread
    static_assert(AL * THREADS == ACH, "activation chunk split");
    const int lane = threadIdx.x & 63, tid = threadIdx.x;
    constexpr int WB = wbits(WF);
    constexpr int SB = stream_step_bytes(WF, NRB);  // bytes of each weight row per step
    constexpr int SW = SB * 8 / WB;              // k per step
    constexpr int SKS_ = SKC / SW;               // steps per activation chunk
    static_assert(SKS_ >= 1, "a chunk holds at least one step");
    constexpr int U = RING / gcd_c(SKS_, RING);  // chunks per unrolled body: ring slots are static
    const int nk = c.K / SW;                     // steps
    const int nchunk = c.K / SKC;
    // activation staging of this thread
    const uint16_t* ap[AL];
    int alds[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int q = tid + i * THREADS;
        const int row = q / (SKC / 8), ch = q % (SKC / 8);
        ap[i] = act_row(c, row) + ch * 8;
        alds[i] = s_off<SKC>(row, ch);
    }
    u32x4 sa[AL];
    auto load_a = [&](int chunk) {
        const int k0 = (chunk < nchunk ? chunk : nchunk - 1) * SKC;
#pragma unroll
        for (int i = 0; i < AL; ++i) sa[i] = *(const u32x4*)(ap[i] + k0);
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) *(u32x4*)(lds + buf * (ROWS * SKC) + alds[i]) = sa[i];
    };
    // weights: the SB/4 bytes at g*SB/4 of the row's step hold the lane's elements of the
    // step: 16g .. +15 (bf16), 32g .. +31 (E4M3, and E2M1 in half-line steps: one 32-element
    // scale block) or 64g .. +63 (E2M1 in whole-line steps: two blocks); one 16-byte load per
    // 16 bytes
    constexpr int LB = SB / 64;                  // 16-byte loads per block and step
    const uint8_t* b0 = c.bp0 + (lane >> 4) * (SB / 4 - WB);   // bp0 points at element 8g
    const uint8_t* b1 = c.bp1 + (lane >> 4) * (SB / 4 - WB);
    u32x4 rb[RING][4];
    auto load_b = [&](int kstep, int set) {
        const int k0 = (kstep < nk ? kstep : nk - 1) * SB;
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[set][i] = *(const u32x4*)(b0 + k0 + 16 * i);
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[set][2 + i] = *(const u32x4*)(b1 + k0 + 16 * i);
    };
    // Scales of quantized weights: a row's chunk of 512 k has 16 scale bytes (8 and 4 for the
    // 256-k and 128-k chunks of larger tiles).  E4M3: byte 4j + g scales lane group g in step j; E2M1: bytes
    // 8j + 2g and 8j + 2g + 1.  The wave's two blocks' scale rows sit in its LDS area (row r
    // of block b at b*16*K/32 + r*K/32); sc holds the lane's row's bytes of the current chunk.
    constexpr int SCB = SKC / 32;                       // scale bytes per row and chunk
    uint8_t* sarea = reinterpret_cast<uint8_t*>(lds + SACT_ELEMS) + (threadIdx.x >> 6) * scale_wave_bytes(SKMAX);
    uint32_t sc[2][4] = {};
    // the whole scale rows of the wave's blocks, once per tile: loaded into registers first
    // (their latency overlaps the first activation chunk's), then written to the LDS area
    constexpr int SLD = WF == WF_BF16 ? 1 : (SKMAX / 2 + 1023) / 1024;   // 16-byte loads per lane and block
    u32x4 st[2][SLD];
    auto stage_s_load = [&]() {
        if constexpr (WF != WF_BF16) {
            const int nb = c.K >> 1;                        // bytes per block: 16 rows x K/32
            const uint8_t* src[2] = {c.sp0 - (lane & 15) * (c.K >> 5), c.sp1 - (lane & 15) * (c.K >> 5)};
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < SLD; ++i)
                    if (16 * lane + 1024 * i < nb) st[b][i] = *(const u32x4*)(src[b] + 16 * lane + 1024 * i);
        }
    };
    auto stage_s_store = [&]() {
        if constexpr (WF != WF_BF16) {
            const int nb = c.K >> 1;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < SLD; ++i)
                    if (16 * lane + 1024 * i < nb) *(u32x4*)(sarea + b * nb + 16 * lane + 1024 * i) = st[b][i];
        }
    };
    auto fetch_s = [&](int ck) {
        if constexpr (WF != WF_BF16) {
            const int o = (lane & 15) * (c.K >> 5) + ck * SCB;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint8_t* p = sarea + b * (c.K >> 1) + o;
                if constexpr (SCB == 16) {
                    const u32x4 v = *(const u32x4*)p;
                    sc[b][0] = v[0], sc[b][1] = v[1], sc[b][2] = v[2], sc[b][3] = v[3];
                } else if constexpr (SCB == 8) {
                    const uint2 v = *(const uint2*)p;
                    sc[b][0] = v.x, sc[b][1] = v.y;
                } else {
                    sc[b][0] = *(const uint32_t*)p;
                }
            }
        }
    };
    // scale of block h (0, 1) of the lane's elements in step j of the chunk
    auto scale_of = [&](int blk, int j, int h) {
        if constexpr (SW == 128) {   // one block per lane and step: byte 4j + g
            return e8m0_factor((sc[blk][j] >> (8 * (lane >> 4))) & 0xFFu);
        } else {                     // two: bytes 8j + 2g + h
            // lanes 32..63 take the odd word (a bit select: a conditional pick of the two
            // array elements becomes a load at a lane-dependent index from a private array)
            const uint32_t lo = sc[blk][2 * j], hi = sc[blk][2 * j + 1];
            const uint32_t d = lo ^ ((lo ^ hi) & (0u - (uint32_t)((lane >> 5) & 1)));
            return e8m0_factor((d >> (8 * (2 * ((lane >> 4) & 1) + h))) & 0xFFu);
        }
    };
    // step j (0 .. SKS_-1, a compile-time constant in the unrolled loop) of the chunk in `buf`
    auto compute = [&](int j, int set, int buf) {
        const int w = j * (SW / 8);               // 16-byte chunk of the step inside the LDS chunk
        constexpr int NQ = SW / 32;               // MFMAs per block and step
        float s0[2] = {0.f, 0.f}, s1[2] = {0.f, 0.f};
        if constexpr (WF != WF_BF16) {
#pragma unroll
            for (int h = 0; h < SW / 128; ++h) {
                s0[h] = scale_of(0, j, h);
                s1[h] = scale_of(1, j, h);
            }
        }
        // MFMA q of the step takes the lane's elements 8q .. 8q+7: chunk NQ*(lane>>4) + q
        // of the step's window
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            bf16x8 g, u;
            if constexpr (WF == WF_E4M3) {
                const int l = q >> 1, h = q & 1;
                g = decode8(rb[set][l][2 * h], rb[set][l][2 * h + 1], s0[0]);
                u = decode8(rb[set][2 + l][2 * h], rb[set][2 + l][2 * h + 1], s1[0]);
            } else if constexpr (WF == WF_E2M1) {
                const int l = q >> 2;             // elements 32l .. 32l+31: scale block l
                g = decode8_fp4(rb[set][l][q & 3], s0[l]);
                u = decode8_fp4(rb[set][2 + l][q & 3], s1[l]);
            } else {
                g = __builtin_bit_cast(bf16x8, rb[set][q]);
                u = __builtin_bit_cast(bf16x8, rb[set][2 + q]);
            }
#pragma unroll
            for (int r = 0; r < NRB; ++r) {
                const bf16x8 a = *(const bf16x8*)(lds + buf * (ROWS * SKC) +
                                                  s_off<SKC>(r * 16 + (lane & 15), w + NQ * (lane >> 4) + q));
                acc[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, g, acc[r][0], 0, 0, 0);
                acc[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, u, acc[r][1], 0, 0, 0);
            }
        }
    };
    // prologue: chunk 0 into LDS, chunk 1 in flight, weights RING-1 steps ahead (issuing the
    // weights before the scale rows and the activation lookups measured no faster: 8-bit
    // down 2% slower, the others within 0.6%)
    stage_s_load();
    __builtin_amdgcn_sched_barrier(0);
    load_a(0);
    __builtin_amdgcn_sched_barrier(0);
    stage_s_store();
    store_a(0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < RING - 1; ++s) {
        load_b(s, s);
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
    for (int ck0 = 0; ck0 < nchunk; ck0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ck = ck0 + u;
            if (U > 1 && ck >= nchunk) break;
            const int buf = ck & 1;
            fetch_s(ck);
#pragma unroll
            for (int j = 0; j < SKS_; ++j) {
                const int kt = ck * SKS_ + j;
                const int sl = u * SKS_ + j;      // static ring slot
                __builtin_amdgcn_sched_barrier(0);
                load_b(kt + RING - 1, (sl + RING - 1) % RING);
                compute(j, sl % RING, buf);
            }
            // next chunk: stage it into the other buffer (read by no wave since the last
            // barrier), then put the one after it in flight
            __builtin_amdgcn_sched_barrier(0);
            store_a(buf ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            load_a(ck + 2);
            lds_barrier();
        }
    }
}

// Register sets of the stream variant's weight ring (weights run ring-1 steps ahead),
// measured over decode and serving shapes (16..1280 tokens of the Beam layer): bf16 two steps
// ahead (three were 1% slower); E4M3 one step ahead in 16-row tiles and two in larger ones
// (three steps ahead was 4-5% slower from 64 to 512 tokens, 1.5-3% at 768-1024); E2M1 in
// whole-line steps (16 MFMAs per block and step) one step ahead (two measured no faster,
// three spill), in half-line steps three ahead (one or two were 1-4% slower).  A shallower
// ring leaves fewer redundant loads of a row's last line when a work item ends, and issues
// fewer loads at once when one starts.
#ifndef STREAM_RING_BF16
#define STREAM_RING_BF16 3
#endif
#ifndef STREAM_RING_E4M3_1
#define STREAM_RING_E4M3_1 2
#endif
#ifndef STREAM_RING_E4M3_N
#define STREAM_RING_E4M3_N 3
#endif
#ifndef STREAM_RING_E2M1_HALF
#define STREAM_RING_E2M1_HALF 4
#endif
__host__ __device__ constexpr int stream_ring(int wf, int nrb) {
    return wf == WF_E2M1 ? (stream_step_bytes(wf, nrb) == 128 ? 2 : STREAM_RING_E2M1_HALF)
         : wf == WF_E4M3 ? (nrb == 1 ? STREAM_RING_E4M3_1 : STREAM_RING_E4M3_N)
                         : STREAM_RING_BF16;
}

// Runs one tile: main loop variant, then the epilogue.
template <bool GATED, int WF, int NRB, int RING, int THREADS, bool SMALL>
__device__ __forceinline__ void run_tile(const TileCtx& c, uint16_t (*lds)[GROWS * GKS]) {
    const int lane = threadIdx.x & 63;
    f32x4 acc[NRB][2];
#pragma unroll
    for (int i = 0; i < NRB; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the streaming loop takes tiles of up to 64 rows
    constexpr int CHUNK = stream_chunk(NRB);
    if constexpr (SMALL) {
        // the host checks K % 512 == 0 and K <= SCALE_KMAX_SMALL
        tile_body_stream<GATED, WF, NRB, stream_ring(WF, NRB), THREADS, SCALE_KMAX_SMALL>(c, &lds[0][0], acc);
    } else if constexpr (NRB <= 4) {
        if (c.K % CHUNK == 0 && (WF == WF_BF16 || c.K <= SCALE_KMAX))
            tile_body_stream<GATED, WF, NRB, stream_ring(WF, NRB), THREADS, SCALE_KMAX>(c, &lds[0][0], acc);
        else
            tile_body<GATED, WF, NRB, RING, THREADS>(c, lds, acc);
    } else
        tile_body<GATED, WF, NRB, RING, THREADS>(c, lds, acc);

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

// SMALL: every tile has at most 64 rows (at most 64 tokens, so no expert has more) and K is a
// multiple of 512 and at most SCALE_KMAX_SMALL.  Only the stream variant is compiled, with
// 52 KB of LDS and at most 168 registers, so that three work-groups fit on a compute unit.
template <bool GATED, int WF, int WAVES, bool SMALL>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(SMALL ? 3 : 2)))
moe_gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint8_t* __restrict__ B0, const uint8_t* __restrict__ B1,
                     const uint8_t* __restrict__ S0, const uint8_t* __restrict__ S1, int K, int N, int top_k,
                     const int32_t* __restrict__ sorted_pairs, const TileEntry* __restrict__ tiles,
                     const int32_t* __restrict__ num_tiles, int n_col_blocks, uint16_t* __restrict__ C) {
    // the large-tile loop's buffers, or the streaming loop's activation chunks and the
    // waves' scale areas
    constexpr int STREAM_ELEMS = SACT_ELEMS + WAVES * scale_wave_bytes(SMALL ? SCALE_KMAX_SMALL : SCALE_KMAX) / 2;
    constexpr int LDS_ELEMS = SMALL || STREAM_ELEMS > 2 * GROWS * GKS ? STREAM_ELEMS : 2 * GROWS * GKS;
    __shared__ __attribute__((aligned(16))) uint16_t lds_raw[LDS_ELEMS];
    auto lds = reinterpret_cast<uint16_t (*)[GROWS * GKS]>(lds_raw);

    // XCD-aware order: blocks are dealt round-robin to the 8 XCDs, so give each XCD a
    // contiguous run of work items (the column blocks of one tile share its activation
    // rows in that XCD's L2).
    const int work = *num_tiles * n_col_blocks;
    const int per_xcd = (work + 7) >> 3;
    const int slot = (int)(blockIdx.x >> 3);
    if (slot >= per_xcd) return;
    const int item = (int)(blockIdx.x & 7) * per_xcd + slot;
    if (item >= work) return;
    int tile, cblk;
    item_tile(tiles, item, n_col_blocks, tile, cblk);
    const TileEntry te = tiles[tile];
    if (te.row_count <= 0) return;
    const int e = te.expert;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    TileCtx c;
    c.sp0 = c.sp1 = nullptr;
    c.nk = K / GKS;
    c.row_begin = te.row_begin;
    c.row_count = te.row_count;
    c.N = N;
    c.sorted_pairs = sorted_pairs;
    c.C = C;
    // weight rows of this wave (two 16-row MFMA operand blocks); byte pointers
    constexpr int WB = wbits(WF);   // bits per weight
    int col0;
    if (GATED) {
        col0 = cblk * (WAVES * 16) + wave * 16;
        const int64_t r = (int64_t)e * N + col0 + (lane & 15);
        c.bp0 = B0 + (r * K + (lane >> 4) * 8) * WB / 8;
        c.bp1 = B1 + (r * K + (lane >> 4) * 8) * WB / 8;
        if (WF != WF_BF16) {
            c.sp0 = S0 + r * (K / 32);
            c.sp1 = S1 + r * (K / 32);
        }
    } else {
        col0 = cblk * (WAVES * 32) + wave * 32;
        const int64_t r = (int64_t)e * N + col0 + (lane & 15);
        c.bp0 = B0 + (r * K + (lane >> 4) * 8) * WB / 8;
        c.bp1 = c.bp0 + (int64_t)16 * K * WB / 8;
        if (WF != WF_BF16) {
            c.sp0 = S0 + r * (K / 32);
            c.sp1 = c.sp0 + (int64_t)16 * (K / 32);
        }
    }
    c.ccol = col0 + (lane & 15);
    c.A = A;
    c.K = K;
    c.top_k = top_k;
    c.gather = GATED;

    // row-count variants (tiles of up to 4 row blocks stream; larger ones take 32-k steps)
    const int nrb = (te.row_count + 15) >> 4;

    constexpr int TH = WAVES * 64;
    if constexpr (SMALL) {
        // at most 64 tokens: no expert has more than 64 rows
        if (nrb > 2)
            run_tile<GATED, WF, 4, 4, TH, true>(c, lds);
        else if (nrb > 1)
            run_tile<GATED, WF, 2, 4, TH, true>(c, lds);
        else
            run_tile<GATED, WF, 1, 4, TH, true>(c, lds);
    } else {
        if (nrb > 16)
            run_tile<GATED, WF, 18, 4, TH, false>(c, lds);
        else if (nrb > 12)
            run_tile<GATED, WF, 16, 4, TH, false>(c, lds);
        else if (nrb > 8)
            run_tile<GATED, WF, 12, 4, TH, false>(c, lds);
        else if (nrb > 4)
            run_tile<GATED, WF, 8, 4, TH, false>(c, lds);
        else if (nrb > 2)
            run_tile<GATED, WF, 4, 4, TH, false>(c, lds);
        else if (nrb > 1)
            run_tile<GATED, WF, 2, 4, TH, false>(c, lds);
        else
            run_tile<GATED, WF, 1, 4, TH, false>(c, lds);
    }
}

// ---------------------------------------------------------------------------------
// Line-streaming variant for prefill-sized tiles.  Work item and tile are as above (up
// to 288 rows; 128 h columns for gate/up, 256 output columns for down); a work-group
// of WAVES waves gives each wave NB 16-row weight blocks (gate/up: NB/2 gate blocks and
// the up blocks of the same h columns).
//
// K advances 64 per step.  bf16 weights go straight into LDS, whole 128-byte lines of 8
// rows per load (16 bytes per lane), one step ahead, into two slots; each wave reads its
// own rows back as MFMA fragments.  (Loaded into registers in the MFMA operand shape, 16
// rows per load, they would be read as 64-byte half lines, which cost 11% more on the load
// path once the activation stream shares it.)  The even MFMA of a step takes k-chunk g of
// a row (g = lane>>4), the odd one 4+g, and the activation fragments use the same k order.
// 8-bit and 4-bit codes: the lane's 16 contiguous elements per block and step, loaded into
// a ring of RING register sets, RING-1 steps ahead, with their scale byte.  Activations:
// the rows of step kt+1 are written into one of two LDS buffers while step kt is
// multiplied out of the other, and one barrier per step publishes them.  The LDS writes
// and every global load of a step are spread over its MFMA sequence.  Buffer loads with
// 32-bit offsets keep one address register per stream.
// ---------------------------------------------------------------------------------
constexpr int WKS = 64;                    // k per step
// Rows per tile of the line kernel.  With 16- and 8-bit weights a tile holds up to 320 rows:
// at 8192 tokens of the Beam layer every expert (at most ~313 rows there) then fits one tile,
// so no expert's weights are streamed twice and the 256 x 20 work items of a GEMM fill the
// 256 compute units in 20 whole rounds; with 288-row tiles nine experts split into two
// half-full tiles and 5300 items leave the last round 70% full.  4-bit weights keep 288 rows:
// their three-step register ring leaves no room for a 20th row block of accumulators.
constexpr int LROWS = 320;
template <int WF>
__host__ __device__ constexpr int line_rows() { return WF == WF_E2M1 ? GROWS : LROWS; }
// one LDS activation buffer (40 KB at 320 rows)
template <int WF>
constexpr int wbuf_elems() { return line_rows<WF>() * WKS; }
constexpr int BUF_DWORD3 = 0x00020000;     // raw buffer descriptor word 3 on gfx9

// LDS element offset of 16-byte chunk `ch` (0..7) of activation row `row` (128-byte
// rows).  The XOR pattern makes the fragment reads (16 consecutive rows at one chunk per
// 16 lanes) free of bank conflicts on gfx950; it was chosen among candidate patterns with
// the LDS bank-conflict counter (patterns such as row & 7 or (row >> 1) & 7 conflict
// 2-way).  Writes cover whole 128-byte rows, which any in-row permutation keeps intact.
__device__ __forceinline__ int w_swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ int w_off(int row, int ch) { return row * WKS + ((ch ^ w_swz(row)) << 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, BUF_DWORD3);
}

__device__ __forceinline__ u32x4 buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// bf16 rows keep k-chunk c at position kpos(c) = 2c (c < 4) or 2(c-4)+1 of their LDS row (then
// XOR-swizzled by w_swz); kinv is its inverse: the chunk kept at position q
__device__ __forceinline__ int kinv(int q) { return (q & 1) ? 4 + (q >> 1) : q >> 1; }

// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land at dst + 16 l
__device__ __forceinline__ void buf_load_lds(__amdgpu_buffer_rsrc_t r, uint16_t* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// Work-group barrier for LDS written by ds_write only: this wave's LDS writes are complete
// (lgkmcnt), then s_barrier; the memory clobber keeps the compiler from moving LDS accesses
// across it.  Unlike a release fence it does not wait for loads into LDS still in flight
// (the fence turns into vmcnt(0) while any is outstanding), so the weight loads of the next
// step keep flying across it.
__device__ __forceinline__ void lds_write_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


struct LineCtx {
    __amdgpu_buffer_rsrc_t act;   // activation tensor (token rows or h rows)
    __amdgpu_buffer_rsrc_t w0;    // weight blocks [0, NB/2)
    __amdgpu_buffer_rsrc_t w1;    // weight blocks [NB/2, NB)
    __amdgpu_buffer_rsrc_t s0;    // quantized weights: scale rows of the blocks of w0
    __amdgpu_buffer_rsrc_t s1;    //       and of w1
    uint32_t wvoff;               // codes: this lane's byte offset inside a weight block
    uint32_t wdoff[2];            // bf16: this lane's byte offsets for the two 8-row loads into LDS
    uint32_t svoff;               // quantized weights: this lane's byte offset inside a block's scale rows
    int K, top_k, row_begin, row_count;
    bool gather;
    const int32_t* sorted_pairs;
};

// Weight loads of step `kstep` of a work item into slot `set` (steps past the end reload
// the last step, which the cache still holds).  bf16: the block's 16 rows x 128 bytes into
// the wave's LDS slot, two loads of 8 whole lines; E4M3: one 16-byte load of the lane's 16
// elements into the register ring, E2M1 one 8-byte load, and the scale byte of their 32-k
// block.
template <int NB, int RING, int WF>
__device__ __forceinline__ void line_load_b(const LineCtx& c, u32x4 (&rb)[RING][NB][2], uint32_t (&rs)[RING][NB],
                                            uint16_t* const (&wl)[2], int b, int kstep, int set) {
    constexpr int HB = NB / 2;
    constexpr int WB = wbits(WF);
    const int nk = c.K / WKS;
    const int ks = kstep < nk ? kstep : nk - 1;
    const uint32_t so = (uint32_t)(ks * WKS * WB / 8) + (uint32_t)(b % HB) * (uint32_t)(16 * c.K * WB / 8);
    const __amdgpu_buffer_rsrc_t r = b < HB ? c.w0 : c.w1;
    if constexpr (WF == WF_BF16) {
        // whole 128-byte lines of 8 rows per load, into the wave's block b of LDS slot `set`
        (void)rb;
        uint16_t* dst = wl[set] + b * 16 * WKS;
        buf_load_lds(r, dst, c.wdoff[0], so);
        buf_load_lds(r, dst + 8 * WKS, c.wdoff[1], so);
        return;
    }
    if constexpr (WF == WF_E2M1) {
        const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, c.wvoff, so, 0));
        rb[set][b][0] = u32x4{v.x, v.y, 0u, 0u};
    } else {
        rb[set][b][0] = buf_load(r, c.wvoff, so);
    }
    const uint32_t ss = (uint32_t)(ks * (WKS / 32)) + (uint32_t)(b % HB) * (uint32_t)(16 * (c.K / 32));
    rs[set][b] = __builtin_amdgcn_raw_buffer_load_b8(b < HB ? c.s0 : c.s1, c.svoff, ss, 0);
}

// The weights of a work item's first RING-1 steps.
template <int NB, int RING, int WF>
__device__ __forceinline__ void line_prologue_b(const LineCtx& c, u32x4 (&rb)[RING][NB][2], uint32_t (&rs)[RING][NB],
                                                uint16_t* const (&wl)[2]) {
#pragma unroll
    for (int s2 = 0; s2 < RING - 1; ++s2)
#pragma unroll
        for (int b = 0; b < NB; ++b) line_load_b<NB, RING, WF>(c, rb, rs, wl, b, s2, s2);
}

// Main loop of one work item; the caller has issued its first RING-1 weight steps.
template <int WAVES, int NB, int RING, int NRB, int WF>
__device__ __forceinline__ void line_body(const LineCtx& c, uint16_t* lds, u32x4 (&rb)[RING][NB][2],
                                          uint32_t (&rs)[RING][NB], uint16_t* const (&wl)[2],
                                          f32x4 (&acc)[NRB][NB]) {
    constexpr int THREADS = WAVES * 64;
    constexpr int ACH = NRB * 16 * 8;                  // 16-byte activation chunks per step
    constexpr int AL = (ACH + THREADS - 1) / THREADS;
    constexpr int NOPS = 2 * AL + NB;                  // memory operations spread over a step
    constexpr int UNR = RING % 2 ? 2 * RING : RING;    // ring slot and LDS buffer both static
    const int lane = threadIdx.x & 63, tid = threadIdx.x;
    const int nk = c.K / WKS;

    // activation staging: chunk q = tid + THREADS*i (wrapped for partial tiles)
    uint32_t avoff[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int q = (tid + i * THREADS) % ACH;
        const int row = q >> 3, ch = q & 7;
        const int src = row < c.row_count ? row : 0;
        const int64_t r = c.gather ? (int64_t)(c.sorted_pairs[c.row_begin + src] / c.top_k)
                                   : (int64_t)(c.row_begin + src);
        avoff[i] = (uint32_t)((r * c.K + ch * 8) * 2);
    }
    // bf16: k-chunk c of a row is kept at position 2c (c < 4) or 2(c-4)+1 of its LDS row, so
    // the fragments of k-chunks g and 4+g (the lane's weight chunks, below) are read from
    // positions 2g and 2g+1: the read pattern the XOR layout keeps free of bank conflicts
    // (reading positions g and 4+g conflicted in 28% of the LDS cycles)
    auto kpos = [&](int ch) { return WF == WF_BF16 ? (ch < 4 ? 2 * ch : 2 * ch - 7) : ch; };
    auto lds_slot = [&](int i) {
        const int q = (tid + i * THREADS) % ACH;
        return w_off(q >> 3, kpos(q & 7));
    };
    u32x4 sa[AL];
    auto kbytes = [&](int kstep) { return (uint32_t)((kstep < nk ? kstep : nk - 1) * WKS * 2); };
    auto load_a = [&](int i, int kstep) { sa[i] = buf_load(c.act, avoff[i], kbytes(kstep)); };
    auto store_a = [&](int i, int buf) { *(u32x4*)(lds + buf * wbuf_elems<WF>() + lds_slot(i)) = sa[i]; };
    auto load_b = [&](int b, int kstep, int set) { line_load_b<NB, RING, WF>(c, rb, rs, wl, b, kstep, set); };
    // fragment read offsets: row r*16 + (lane & 15), LDS positions 2g and 2g+1 (g = lane >> 4).
    // bf16 weights: the even MFMA takes k-chunk g of the step's 128 bytes, the odd one k-chunk
    // 4+g (each weight load then reads 64 contiguous bytes of 16 rows: one 64-byte request per
    // row), which kpos puts at positions 2g and 2g+1; the 8-bit and 4-bit codes of a lane's 16
    // elements are contiguous, so there the two MFMAs take k-chunks 2g and 2g+1 themselves
    const int fr = lane & 15, g = lane >> 4;
    const int off_e = w_off(fr, 2 * g);
    const int off_o = w_off(fr, 2 * g + 1);
    constexpr int LA = 1;  // fragment lookahead (row blocks); deeper measured no faster

    // memory operations of a step, in issue order: with weights one step ahead (RING = 2)
    // the weight loads of step kt+1 come first (a block each), then alternately the LDS
    // write of activation chunk i of step kt+1 and the load of chunk i of step kt+2; issued
    // early, those weights have about a whole step to arrive (issued after the activation
    // operations they had about half a step: bf16 gate/up 3.66 -> 3.60 ms at 8192 tokens).
    // Waiting for a staged activation chunk still never waits for the newest weight loads:
    // those are younger.  With weights two steps ahead (RING = 3, E2M1) the weight loads
    // stay last (first measured 9% slower for gate/up).
    constexpr bool WEIGHTS_FIRST = RING == 2;
    auto op_kind = [&](int o) { return WEIGHTS_FIRST ? (o < NB ? 2 * AL + o : o - NB) : o; };
    auto mem_op = [&](int o, int kt, int wbuf, int set) {
        o = op_kind(o);
        if (o < 2 * AL) {
            if ((o & 1) == 0)
                store_a(o >> 1, wbuf);
            else
                load_a(o >> 1, kt + 2);
        } else {
            load_b(o - 2 * AL, kt + RING - 1, set);
        }
    };

    auto step = [&](int kt, auto jc) {
        constexpr int j = decltype(jc)::value;          // kt mod UNR
        constexpr int set = j % RING;
        constexpr int nset = (j + RING - 1) % RING;     // ring slot of step kt+RING-1
        const uint16_t* L = lds + (j & 1) * wbuf_elems<WF>();
        const int wbuf = (j + 1) & 1;
        if constexpr (WF == WF_BF16)
            lds_write_barrier();   // bf16 weights of the next step are loading into LDS
        else
            lds_barrier();
        // this step's weight fragments (quantized weights: decoded exactly to bf16)
        bf16x8 wf[NB][2];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if constexpr (WF == WF_E4M3) {
                const float sc = e8m0_factor(rs[set][b]);
                wf[b][0] = decode8(rb[set][b][0][0], rb[set][b][0][1], sc);
                wf[b][1] = decode8(rb[set][b][0][2], rb[set][b][0][3], sc);
            } else if constexpr (WF == WF_E2M1) {
                const float sc = e8m0_factor(rs[set][b]);
                wf[b][0] = decode8_fp4(rb[set][b][0][0], sc);
                wf[b][1] = decode8_fp4(rb[set][b][0][1], sc);
            } else {   // bf16: this wave's rows of LDS slot `set`, read like the activations
                wf[b][0] = *(const bf16x8*)(wl[set] + b * 16 * WKS + off_e);
                wf[b][1] = *(const bf16x8*)(wl[set] + b * 16 * WKS + off_o);
            }
        }
        bf16x8 ae[NRB], ao[NRB];
#pragma unroll
        for (int r = 0; r < LA; ++r) {
            ae[r] = *(const bf16x8*)(L + off_e + r * 16 * WKS);
            ao[r] = *(const bf16x8*)(L + off_o + r * 16 * WKS);
        }
        // (bf16: the weight fragments are LDS reads too)
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA + (WF == WF_BF16 ? 2 * NB : 0), 0);
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            if (r + LA < NRB) {
                ae[r + LA] = *(const bf16x8*)(L + off_e + (r + LA) * 16 * WKS);
                ao[r + LA] = *(const bf16x8*)(L + off_o + (r + LA) * 16 * WKS);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[r][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae[r], wf[b][0], acc[r][b], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
            // this row block's share of the step's memory operations
#pragma unroll
            for (int o = 0; o < NOPS; ++o) {
                if (o >= (r * NOPS) / NRB && o < ((r + 1) * NOPS) / NRB) {
                    mem_op(o, kt, wbuf, nset);
                    const int k = op_kind(o);
                    if (k < 2 * AL && (k & 1) == 0)
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                    else if (k < 2 * AL)
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    else
                        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[r][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao[r], wf[b][1], acc[r][b], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
        }
    };

    // prologue: step 0 in buffer 0, step 1 staged in registers (the weights of the first
    // RING-1 steps are already in flight)
#pragma unroll
    for (int i = 0; i < AL; ++i) load_a(i, 0);
#pragma unroll
    for (int i = 0; i < AL; ++i) store_a(i, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < AL; ++i) load_a(i, 1);
    __builtin_amdgcn_sched_barrier(0);
    int kt = 0;
    for (; kt + UNR <= nk; kt += UNR) {
        static_for<UNR>([&](auto jc) { step(kt + decltype(jc)::value, jc); });
    }
    // remainder: nk is even and nk - kt < UNR <= 6
    if (nk - kt >= 2) {
        step(kt, std::integral_constant<int, 0>());
        step(kt + 1, std::integral_constant<int, 1>());
    }
    if (UNR > 4 && nk - kt >= 4) {
        step(kt + 2, std::integral_constant<int, 2 % UNR>());
        step(kt + 3, std::integral_constant<int, 3 % UNR>());
    }
}

template <bool GATED, int WF, int WAVES, int NB, int RING>
__global__ void __launch_bounds__(WAVES * 64) moe_gemm_line_kernel(
    const uint16_t* __restrict__ A, uint32_t a_bytes, const uint8_t* __restrict__ B0,
    const uint8_t* __restrict__ B1, const uint8_t* __restrict__ S0, const uint8_t* __restrict__ S1, int K, int N,
    int top_k, const int32_t* __restrict__ sorted_pairs, const TileEntry* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int n_col_blocks, uint16_t* __restrict__ C) {
    static_assert(WAVES * NB * 16 == 256 && NB % 2 == 0, "a work-group covers 256 weight rows");
    // the output tile is staged through LDS (rows padded by 16 bytes) once the main loop is
    // done, EPI_RB row blocks at a time (down: half the tile with bf16 weights or 320-row
    // tiles, so that with the bf16 weight slots below everything fits in 160 KB)
    constexpr int EPI_COLS = GATED ? WAVES * (NB / 2) * 16 : WAVES * NB * 16;
    constexpr int EPI_STRIDE = EPI_COLS + 8;
    constexpr int ROWS = line_rows<WF>();
    constexpr int EPI_RB = GATED || (WF != WF_BF16 && ROWS == GROWS) ? ROWS / 16 : ROWS / 32;
    constexpr int WBUF = wbuf_elems<WF>();
    constexpr int LDS_ELEMS = EPI_RB * 16 * EPI_STRIDE > 2 * WBUF ? EPI_RB * 16 * EPI_STRIDE : 2 * WBUF;
    static_assert(2 * (LDS_ELEMS + 2 * (WF == WF_BF16 ? WAVES * NB * 16 * WKS : 8)) <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
    // bf16 weights: two slots (steps of even and odd parity), each wave's 16*NB rows x 128
    // bytes; two arrays, so that a read of one slot waits only for the loads into that slot
    constexpr int WSLOT = WF == WF_BF16 ? WAVES * NB * 16 * WKS : 8;
    __shared__ __attribute__((aligned(16))) uint16_t wlds0[WSLOT];
    __shared__ __attribute__((aligned(16))) uint16_t wlds1[WSLOT];
    constexpr int HB = NB / 2;

    // XCD-aware order (blocks are dealt to the 8 XCDs round-robin): each XCD takes a
    // contiguous run of work items, so the column blocks of one tile share its activation
    // rows in that XCD's L2.
    const int work = *num_tiles * n_col_blocks;
    const int per_xcd = (work + 7) >> 3;
    const int slot = (int)(blockIdx.x >> 3);
    if (slot >= per_xcd) return;
    const int item = (int)(blockIdx.x & 7) * per_xcd + slot;
    if (item >= work) return;
    int tile, cblk;
    item_tile(tiles, item, n_col_blocks, tile, cblk);
    const TileEntry te = tiles[tile];
    if (te.row_count <= 0) return;
    const int64_t e = te.expert;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    LineCtx c;
    c.act = make_rsrc(A, a_bytes);
    c.K = K;
    c.top_k = top_k;
    c.row_begin = te.row_begin;
    c.row_count = te.row_count;
    c.gather = GATED;
    c.sorted_pairs = sorted_pairs;
    constexpr int WB = wbits(WF);   // bits per weight
    // codes: the lane's 16 elements 16g .. 16g+15 of its row (g = lane>>4; E4M3 16 bytes,
    // E2M1 8 bytes); the bf16 weights use wdoff (below)
    c.wvoff = (uint32_t)(WF == WF_BF16 ? ((lane & 15) * K * 2 + (lane >> 4) * 16)
                                       : ((lane & 15) * K + (lane >> 4) * 16) * WB / 8);
    c.svoff = (uint32_t)((lane & 15) * (K / 32) + (lane >> 5));   // scale block of elements 16*(lane>>4)
    // bf16 weights into LDS: load i covers block rows 8i .. 8i+7, lane l lands at position l&7
    // of row 8i + (l>>3) and so loads the k-chunk kept there (the activations' layout)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 8 * i + (lane >> 3);
        c.wdoff[i] = (uint32_t)(row * K * 2 + kinv((lane & 7) ^ w_swz(row)) * 16);
    }
    uint16_t* const wl[2] = {wlds0 + wave * (NB * 16 * WKS), wlds1 + wave * (NB * 16 * WKS)};
    const uint32_t bytes = (uint32_t)((int64_t)HB * 16 * K * WB / 8);
    const uint32_t sbytes = (uint32_t)(HB * 16 * (K / 32));
    int col0;
    int64_t r0, r1;   // first weight rows of the blocks of w0 and w1
    if (GATED) {
        col0 = cblk * (WAVES * HB * 16) + wave * (HB * 16);  // h columns [col0, col0 + 16*HB)
        r0 = r1 = e * N + col0;
        c.w0 = make_rsrc(B0 + r0 * K * WB / 8, bytes);
        c.w1 = make_rsrc(B1 + r1 * K * WB / 8, bytes);
    } else {
        col0 = cblk * (WAVES * NB * 16) + wave * (NB * 16);  // output columns [col0, col0 + 16*NB)
        r0 = e * N + col0;
        r1 = r0 + HB * 16;
        c.w0 = make_rsrc(B0 + r0 * K * WB / 8, bytes);
        c.w1 = make_rsrc(B0 + r1 * K * WB / 8, bytes);
    }
    if (WF != WF_BF16) {
        c.s0 = make_rsrc(S0 + r0 * (K / 32), sbytes);
        c.s1 = make_rsrc((GATED ? S1 : S0) + r1 * (K / 32), sbytes);
    }

    auto run = [&](auto nrbc) {
        constexpr int NRB = decltype(nrbc)::value;
        u32x4 rb[RING][NB][2];
        uint32_t rs[RING][NB];
        line_prologue_b<NB, RING, WF>(c, rb, rs, wl);
        f32x4 acc[NRB][NB];
#pragma unroll
        for (int r = 0; r < NRB; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[r][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        line_body<WAVES, NB, RING, NRB, WF>(c, lds, rb, rs, wl, acc);
        // epilogue: each wave writes its bf16 columns of the tile into LDS (C layout of a
        // 16x16 block: rows 4*(lane>>4)+q, column lane&15), then the work-group stores
        // whole 16-byte chunks of every output row; EPI_RB row blocks at a time.
        // silu(g) = g / (1 + e^-g) with the hardware reciprocal (the result is rounded to bf16).
        const int wcol = col0 - cblk * EPI_COLS;
        static_for<(NRB + EPI_RB - 1) / EPI_RB>([&](auto hc) {
            constexpr int R0 = decltype(hc)::value * EPI_RB;
            constexpr int RN = NRB - R0 < EPI_RB ? NRB - R0 : EPI_RB;   // row blocks of this part
            lds_barrier();  // every wave is done with the LDS it overwrites
#pragma unroll
            for (int r = 0; r < RN; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint16_t* lrow = lds + (r * 16 + 4 * (lane >> 4) + q) * EPI_STRIDE + wcol + (lane & 15);
                    if (GATED) {
#pragma unroll
                        for (int hb = 0; hb < HB; ++hb) {
                            const float gv = acc[R0 + r][hb][q], uv = acc[R0 + r][HB + hb][q];
                            lrow[16 * hb] = f32_to_bf16(gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv);
                        }
                    } else {
#pragma unroll
                        for (int b = 0; b < NB; ++b) lrow[16 * b] = f32_to_bf16(acc[R0 + r][b][q]);
                    }
                }
            lds_barrier();
            constexpr int CPR = EPI_COLS / 8;  // 16-byte chunks per output row
#pragma unroll
            for (int q0 = 0; q0 < RN * 16 * CPR; q0 += WAVES * 64) {
                const int q = q0 + (int)threadIdx.x;
                const int row = q / CPR, ch = q % CPR;
                if (q < RN * 16 * CPR && R0 * 16 + row < c.row_count) {
                    const u32x4 v = *(const u32x4*)(lds + row * EPI_STRIDE + ch * 8);
                    const int trow = c.row_begin + R0 * 16 + row;
                    const int64_t orow = GATED ? (int64_t)trow : (int64_t)c.sorted_pairs[trow];
                    *(u32x4*)(C + orow * N + cblk * EPI_COLS + ch * 8) = v;
                }
            }
        });
    };
    // row-block variants: 13..18 (and 20 for 320-row tiles) cover prefill-sized experts
    // with little padding
    const int nrb = (te.row_count + 15) >> 4;
    if (ROWS > GROWS && nrb > 18)
        run(std::integral_constant<int, ROWS / 16>());
    else if (nrb > 17)
        run(std::integral_constant<int, 18>());
    else if (nrb > 16)
        run(std::integral_constant<int, 17>());
    else if (nrb > 15)
        run(std::integral_constant<int, 16>());
    else if (nrb > 14)
        run(std::integral_constant<int, 15>());
    else if (nrb > 13)
        run(std::integral_constant<int, 14>());
    else if (nrb > 12)
        run(std::integral_constant<int, 13>());
    else if (nrb > 8)
        run(std::integral_constant<int, 12>());
    else if (nrb > 4)
        run(std::integral_constant<int, 8>());
    else if (nrb > 2)
        run(std::integral_constant<int, 4>());
    else
        run(std::integral_constant<int, 2>());
}

// prefill configuration: 8 waves x 2 weight blocks (256 weight rows per work-group),
// weights one step ahead (a deeper ring measured no faster and costs 16 registers)
constexpr int LINE_WAVES = 8;
constexpr int LINE_NB = 2;
constexpr int LINE_RING = 2;
// E2M1 weights (8 bytes per block and step) two steps ahead: 4-6% faster from 48 rows per
// expert through prefill; E4M3 spills with a third register set
#ifndef LINE_RING_Q
#define LINE_RING_Q 3
#endif


// Average rows per expert from which the line-streaming kernel is used.  bf16: below it
// the decode kernel (4-wave work-groups, two per CU) is 1-2% faster; above it the line
// kernel wins, by 25% at 32-48 rows per expert (measured over 16..8192 tokens of the Beam
// layer).  Quantized weights: the line kernel reads them in half or quarter lines, and the
// decode kernel's stream (tiles of up to 64 rows) stays ahead longer: E4M3 up to 36 rows
// per expert (by 25% at 24, 13% at 32; even at 40, the line kernel ahead at 44), E2M1 up to
// 40 (by 42% at 24, 11% at 40; the line kernel ahead at 48).
#ifndef WIDE_MIN_ROWS_PER_EXPERT
#define WIDE_MIN_ROWS_PER_EXPERT 8
#endif
#ifndef WIDE_MIN_ROWS_PER_EXPERT_E4M3
#define WIDE_MIN_ROWS_PER_EXPERT_E4M3 40
#endif
#ifndef WIDE_MIN_ROWS_PER_EXPERT_E2M1
#define WIDE_MIN_ROWS_PER_EXPERT_E2M1 44
#endif
#ifndef DECODE_WAVES
#define DECODE_WAVES 4
#endif
// Work items whose weight rows hold at most this many bytes (10 whole-line steps: 4-bit
// down at I = 2560) take the small-tile kernel at up to 64 tokens: three work-groups per
// compute unit instead of two, so that more of each short item's start-up overlaps the
// others' weight streams (4-bit down at 64 tokens 6% faster; 20-step items, 4-bit gate/up
// and 8-bit down, 3% slower, 40- and 80-step items 3-4% slower).
#ifndef SMALL_MAX_ROW_BYTES
#define SMALL_MAX_ROW_BYTES 1280
#endif

static bool use_line_kernel(int64_t P, int E, int K, int wf) {
    const int wide_min = wf == WF_BF16 ? WIDE_MIN_ROWS_PER_EXPERT
                         : wf == WF_E4M3 ? WIDE_MIN_ROWS_PER_EXPERT_E4M3
                                         : WIDE_MIN_ROWS_PER_EXPERT_E2M1;
    return P >= (int64_t)wide_min * E && K % (2 * WKS) == 0;
}

int gemm_tile_rows(int64_t P, int E, int H, int I, bool bf16, int wf) {
    if (!bf16) return 1 << 30;  // the fp32 path does not use tiles
    // the two GEMMs share one tile list: larger tiles only when the line kernel takes both
    if (use_line_kernel(P, E, H, wf) && use_line_kernel(P, E, I, wf))
        return wf == WF_E4M3 ? line_rows<WF_E4M3>() : wf == WF_E2M1 ? line_rows<WF_E2M1>() : line_rows<WF_BF16>();
    return GROWS;
}

int gemm_min_tile_rows() { return GROWS; }

template <bool GATED, int WF>
static hipError_t launch_gemm(const uint16_t* A, uint64_t a_bytes, const uint8_t* B0, const uint8_t* B1, const uint8_t* S0,
                        const uint8_t* S1, int K, int N, int top_k, int64_t P, int E, int64_t max_rows,
                        const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                        int64_t max_tile_count, uint16_t* C, hipStream_t s) {
    if (use_line_kernel(P, E, K, WF)) {
        const int ncb = N / (GATED ? LINE_WAVES * (LINE_NB / 2) * 16 : LINE_WAVES * LINE_NB * 16);
        const int64_t blocks = (max_tile_count * ncb + 7) / 8 * 8;
        moe_gemm_line_kernel<GATED, WF, LINE_WAVES, LINE_NB, WF == WF_E2M1 ? LINE_RING_Q : LINE_RING><<<(unsigned)blocks, LINE_WAVES * 64, 0, s>>>(
            A, (uint32_t)a_bytes, B0, B1, S0, S1, K, N, top_k, sorted_pairs, tiles, num_tiles, ncb, C);
    } else {
        // decode-sized: 4-wave work-groups (two per compute unit) over half-width column
        // blocks, so one work-group's start and end overlap another's weight stream and
        // the last round of work items is shorter
        constexpr int W = DECODE_WAVES;
        const int ncb = N / (GATED ? W * 16 : W * 32);
        const int64_t blocks = (max_tile_count * ncb + 7) / 8 * 8;
        if (max_rows <= 64 && K % 512 == 0 && K <= SCALE_KMAX_SMALL && (int64_t)K * wbits(WF) / 8 <= SMALL_MAX_ROW_BYTES)
            moe_gemm_bf16_kernel<GATED, WF, W, true><<<(unsigned)blocks, W * 64, 0, s>>>(
                A, B0, B1, S0, S1, K, N, top_k, sorted_pairs, tiles, num_tiles, ncb, C);
        else
            moe_gemm_bf16_kernel<GATED, WF, W, false><<<(unsigned)blocks, W * 64, 0, s>>>(
                A, B0, B1, S0, S1, K, N, top_k, sorted_pairs, tiles, num_tiles, ncb, C);
    }
    return hipGetLastError();
}

hipError_t launch_gate_up(const void* act, bool bf16, const void* w_gate, const void* w_up, int wf,
                          const uint8_t* s_gate, const uint8_t* s_up, int64_t T, int H, int I, int E, int top_k,
                          const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                          int64_t max_tile_count, int tile_rows, void* h, hipStream_t s) {
    if (!bf16 || max_tile_count <= 0 || tile_rows != gemm_tile_rows(T * top_k, E, H, I, true, wf))
        return hipErrorInvalidValue;
    if ((wf != WF_BF16) != (s_gate != nullptr)) return hipErrorInvalidValue;
    const uint16_t* A = (const uint16_t*)act;
    const uint8_t *B0 = (const uint8_t*)w_gate, *B1 = (const uint8_t*)w_up;
    const uint64_t ab = (uint64_t)T * H * 2;
    const int64_t P = T * top_k;
    if (wf == WF_E4M3)
        return launch_gemm<true, WF_E4M3>(A, ab, B0, B1, s_gate, s_up, H, I, top_k, P, E, T, sorted_pairs, tiles,
                                          num_tiles, max_tile_count, (uint16_t*)h, s);
    if (wf == WF_E2M1)
        return launch_gemm<true, WF_E2M1>(A, ab, B0, B1, s_gate, s_up, H, I, top_k, P, E, T, sorted_pairs, tiles,
                                          num_tiles, max_tile_count, (uint16_t*)h, s);
    return launch_gemm<true, WF_BF16>(A, ab, B0, B1, nullptr, nullptr, H, I, top_k, P, E, T, sorted_pairs, tiles,
                                      num_tiles, max_tile_count, (uint16_t*)h, s);
}

hipError_t launch_down(const void* h, bool bf16, const void* w_down, int wf, const uint8_t* s_down, int64_t T,
                       int64_t P, int H, int I, int E, const int32_t* sorted_pairs, const TileEntry* tiles, const int32_t* num_tiles,
                       int64_t max_tile_count, int tile_rows, void* y_pair, hipStream_t s) {
    if (!bf16 || max_tile_count <= 0 || tile_rows != gemm_tile_rows(P, E, H, I, true, wf))
        return hipErrorInvalidValue;
    if ((wf != WF_BF16) != (s_down != nullptr)) return hipErrorInvalidValue;
    const uint16_t* A = (const uint16_t*)h;
    const uint8_t* B0 = (const uint8_t*)w_down;
    const uint64_t ab = (uint64_t)P * I * 2;
    if (wf == WF_E4M3)
        return launch_gemm<false, WF_E4M3>(A, ab, B0, nullptr, s_down, nullptr, I, H, 0, P, E, T, sorted_pairs, tiles,
                                           num_tiles, max_tile_count, (uint16_t*)y_pair, s);
    if (wf == WF_E2M1)
        return launch_gemm<false, WF_E2M1>(A, ab, B0, nullptr, s_down, nullptr, I, H, 0, P, E, T, sorted_pairs, tiles,
                                           num_tiles, max_tile_count, (uint16_t*)y_pair, s);
    return launch_gemm<false, WF_BF16>(A, ab, B0, nullptr, nullptr, nullptr, I, H, 0, P, E, T, sorted_pairs, tiles,
                                       num_tiles, max_tile_count, (uint16_t*)y_pair, s);
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
