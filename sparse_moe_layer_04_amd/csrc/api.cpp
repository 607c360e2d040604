// C ABI of the Beam MoE library: argument validation, workspace layout and the launch
// sequence.  Declarations and the contract of every entry point: include/beam_moe.h.
#include "../../include/beam_moe.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "common.hpp"

namespace {

using beam::TileEntry;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool shape_valid(const beam_moe_shape* s) {
    if (!s) return false;
    if (s->T < 0 || s->H < 1 || s->I < 1 || s->E < 1 || s->E > 1024) return false;
    if (s->n_group < 1 || s->n_group > 64 || s->E % s->n_group != 0) return false;
    const int gsize = s->E / s->n_group;
    if (s->topk_group < 1 || s->topk_group > s->n_group) return false;
    if (s->top_k < 1 || s->top_k > 32 || s->top_k > s->topk_group * gsize) return false;
    if (s->T * (int64_t)s->top_k >= ((int64_t)1 << 31)) return false;
    if (s->dtype != BEAM_F32 && s->dtype != BEAM_BF16) return false;
    if (!isfinite(s->routed_scaling)) return false;
    return true;
}

// bf16 kernels: the router sweeps H in groups of 4 32-wide MFMA steps; the expert GEMMs sweep K in
// 128-wide unrolled groups and cover N in 128 (gate/up) or 256 (down) column blocks.
bool route_supported(const beam_moe_shape* s) { return s->dtype != BEAM_BF16 || s->H % 128 == 0; }
bool shape_supported(const beam_moe_shape* s) {
    if (s->dtype == BEAM_BF16) {
        // the GEMMs address token rows and h rows with 32-bit byte offsets
        const int64_t P = s->T * s->top_k;
        return s->H % 256 == 0 && s->I % 128 == 0 && s->T * (int64_t)s->H * 2 < ((int64_t)1 << 32) &&
               P * (int64_t)s->I * 2 < ((int64_t)1 << 32);
    }
    return true;
}

struct Layout {
    size_t part = 0, idx = 0, w = 0, u = 0, scratch = 0, offsets = 0, sorted = 0, pos = 0, ntiles = 0, tiles = 0,
           h = 0, ypair = 0, total = 0;
    int nsplit = 1;  // router reduction splits
    int64_t max_tiles = 0;
};

Layout make_layout(const beam_moe_shape* s, int op) {
    Layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    const int64_t T = s->T, P = T * s->top_k;
    const size_t elt = s->dtype == BEAM_BF16 ? 2 : 4;
    L.nsplit = s->dtype == BEAM_BF16 ? beam::router_splits(T, s->H, s->E) : 1;
    if (op == BEAM_OP_ROUTE) {
        L.part = take((size_t)L.nsplit * T * s->E * 8);
    } else if (op == BEAM_OP_PERMUTE) {
        L.scratch = take(beam::permute_scratch_words(P, s->E) * 4);
    } else {
        const bool bf16 = s->dtype == BEAM_BF16;
        L.max_tiles = bf16 ? beam::max_tiles(P, s->E, beam::gemm_min_tile_rows()) : 0;
        L.part = take((size_t)L.nsplit * T * s->E * 8);
        L.idx = take((size_t)P * 4);
        L.w = take((size_t)P * 4);
        if (op == BEAM_OP_FORWARD_SUBLAYER) L.u = take((size_t)T * s->H * 2);
        L.scratch = take(beam::permute_scratch_words(P, s->E) * 4);
        L.offsets = take((size_t)(s->E + 1) * 4);
        L.sorted = take((size_t)P * 4);
        L.pos = take((size_t)P * 4);
        L.ntiles = take(4);
        L.tiles = take((size_t)L.max_tiles * sizeof(TileEntry));
        L.h = take((size_t)P * s->I * elt);
        L.ypair = take((size_t)P * s->H * elt);
    }
    L.total = off;
    return L;
}

template <typename Tp>
Tp* at(void* ws, size_t off) {
    return reinterpret_cast<Tp*>(static_cast<char*>(ws) + off);
}

beam_status hip_status(hipError_t e) { return e == hipSuccess ? BEAM_OK : BEAM_ERR_HIP; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int32_t beam_moe_abi_version(void) { return BEAM_MOE_ABI_VERSION; }

const char* beam_status_string(beam_status st) {
    switch (st) {
        case BEAM_OK: return "ok";
        case BEAM_ERR_INVALID_ARG: return "invalid argument";
        case BEAM_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case BEAM_ERR_WORKSPACE: return "workspace missing or too small";
        case BEAM_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

beam_status beam_moe_workspace_size(const beam_moe_shape* shape, int32_t op, size_t* bytes) {
    if (!bytes || !shape_valid(shape) || op < BEAM_OP_ROUTE || op > BEAM_OP_FORWARD_SUBLAYER)
        return BEAM_ERR_INVALID_ARG;
    if (op == BEAM_OP_ROUTE ? !route_supported(shape) : (op != BEAM_OP_PERMUTE && !shape_supported(shape)))
        return BEAM_ERR_UNSUPPORTED;
    if (op == BEAM_OP_FORWARD_SUBLAYER && shape->dtype != BEAM_BF16) return BEAM_ERR_UNSUPPORTED;
    *bytes = make_layout(shape, op).total;
    return BEAM_OK;
}

beam_status beam_moe_rmsnorm(const beam_moe_shape* shape, const void* x, const float* gain, float eps, void* u,
                             void* stream) {
    if (!shape || !x || !gain || !u || shape->T < 0 || shape->H < 1 || !(eps >= 0.f) || !isfinite(eps))
        return BEAM_ERR_INVALID_ARG;
    if (shape->dtype != BEAM_BF16 || shape->H % 8 != 0) return BEAM_ERR_UNSUPPORTED;
    if (x == u || !aligned16(x) || !aligned16(u)) return BEAM_ERR_INVALID_ARG;
    if (shape->T == 0) return BEAM_OK;
    return hip_status(beam::launch_rmsnorm(static_cast<const uint16_t*>(x), gain, eps, shape->T, shape->H,
                                           static_cast<uint16_t*>(u), static_cast<hipStream_t>(stream)));
}

beam_status beam_moe_route(const beam_moe_shape* shape, const void* x, const float* w_router, const float* bias,
                           int32_t* topk_idx, float* topk_w, float* logits_out, void* ws, size_t ws_bytes,
                           void* stream) {
    if (!shape_valid(shape) || !x || !w_router || !bias || !topk_idx || !topk_w) return BEAM_ERR_INVALID_ARG;
    if (!route_supported(shape)) return BEAM_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_router)) return BEAM_ERR_INVALID_ARG;
    if (shape->T == 0) return BEAM_OK;
    const Layout L = make_layout(shape, BEAM_OP_ROUTE);
    if (!ws || ws_bytes < L.total) return BEAM_ERR_WORKSPACE;
    double* part = at<double>(ws, L.part);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = shape->dtype == BEAM_BF16;
    hipError_t e = beam::launch_router_logits(x, bf16, w_router, shape->T, shape->H, shape->E, L.nsplit, part, s);
    if (e != hipSuccess) return BEAM_ERR_HIP;
    return hip_status(beam::launch_router_select(part, L.nsplit, bias, shape->T, shape->E, shape->n_group,
                                                 shape->topk_group, shape->top_k, shape->routed_scaling, topk_idx,
                                                 topk_w, logits_out, s));
}

beam_status beam_moe_permute(const beam_moe_shape* shape, const int32_t* topk_idx, int32_t* offsets,
                             int32_t* sorted_pairs, int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream) {
    if (!shape_valid(shape) || !topk_idx || !offsets || !sorted_pairs || !pair_pos) return BEAM_ERR_INVALID_ARG;
    if (shape->T == 0)  // no pairs: the scan alone writes the all-zero offsets
        return hip_status(beam::launch_permute(topk_idx, 0, shape->E, nullptr, offsets, sorted_pairs, pair_pos,
                                               nullptr, nullptr, 1, static_cast<hipStream_t>(stream)));
    const Layout L = make_layout(shape, BEAM_OP_PERMUTE);
    if (!ws || ws_bytes < L.total) return BEAM_ERR_WORKSPACE;
    const int64_t P = shape->T * shape->top_k;
    return hip_status(beam::launch_permute(topk_idx, P, shape->E, at<int32_t>(ws, L.scratch), offsets, sorted_pairs,
                                           pair_pos, nullptr, nullptr, 1, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// E8M0 block scales of quantized expert weights (all three, or none for bf16/fp32 weights)
// and the storage format of the codes (beam::WF_E4M3 or beam::WF_E2M1)
struct WeightScales {
    const uint8_t* gate;
    const uint8_t* up;
    const uint8_t* down;
    int format;
};

beam_status forward_impl(const beam_moe_shape* shape, const void* x, const float* w_router, const float* bias,
                         const void* w_gate, const void* w_up, const void* w_down, const WeightScales* sc,
                         const beam_sublayer* sub, void* out, int32_t* topk_idx, float* topk_w, void* moe_y, void* ws,
                         size_t ws_bytes, void* const* stage_events, void* stream) {
    if (!shape_valid(shape) || !x || !w_router || !bias || !w_gate || !w_up || !w_down || !out)
        return BEAM_ERR_INVALID_ARG;
    if (sc && (!sc->gate || !sc->up || !sc->down)) return BEAM_ERR_INVALID_ARG;
    if (sc && (!aligned16(sc->gate) || !aligned16(sc->up) || !aligned16(sc->down))) return BEAM_ERR_INVALID_ARG;
    if (sub && (!sub->pre_gain || !sub->post_gain || !(sub->eps > 0.f) || !isfinite(sub->eps) ||
                !(sub->residual_k >= 1.f) || !isfinite(sub->residual_k)))
        return BEAM_ERR_INVALID_ARG;
    if (!shape_supported(shape)) return BEAM_ERR_UNSUPPORTED;
    const bool bf16 = shape->dtype == BEAM_BF16;
    if (sub && !bf16) return BEAM_ERR_UNSUPPORTED;
    if (sc && !bf16) return BEAM_ERR_UNSUPPORTED;
    for (const void* p : {x, (const void*)w_router, w_gate, w_up, w_down, (const void*)out})
        if (!aligned16(p)) return BEAM_ERR_INVALID_ARG;
    if (moe_y && !aligned16(moe_y)) return BEAM_ERR_INVALID_ARG;
    if (stage_events)
        for (int i = 0; i <= BEAM_NUM_STAGES; ++i)
            if (!stage_events[i]) return BEAM_ERR_INVALID_ARG;
    if (shape->T == 0) return BEAM_OK;  // nothing to do: no workspace needed
    const Layout L = make_layout(shape, sub ? BEAM_OP_FORWARD_SUBLAYER : BEAM_OP_FORWARD);
    if (!ws || ws_bytes < L.total) return BEAM_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t T = shape->T, P = T * shape->top_k;
    const int H = shape->H, I = shape->I, E = shape->E, K = shape->top_k;
    auto mark = [&](int stage) -> hipError_t {
        return stage_events ? hipEventRecord(static_cast<hipEvent_t>(stage_events[stage]), s) : hipSuccess;
    };
#define BEAM_TRY(expr)                                  \
    do {                                                \
        if ((expr) != hipSuccess) return BEAM_ERR_HIP; \
    } while (0)

    int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
    float* w = topk_w ? topk_w : at<float>(ws, L.w);
    int32_t* sorted = at<int32_t>(ws, L.sorted);
    int32_t* ntiles = at<int32_t>(ws, L.ntiles);
    TileEntry* tiles = at<TileEntry>(ws, L.tiles);
    const int wf = sc ? sc->format : beam::WF_BF16;
    const int tile_rows = beam::gemm_tile_rows(P, E, H, I, bf16, wf);

    BEAM_TRY(mark(BEAM_STAGE_PRENORM));
    const void* act = x;
    if (sub) {
        uint16_t* u = at<uint16_t>(ws, L.u);
        BEAM_TRY(beam::launch_rmsnorm(static_cast<const uint16_t*>(x), sub->pre_gain, sub->eps, T, H, u, s));
        act = u;
    }
    BEAM_TRY(mark(BEAM_STAGE_ROUTER_LOGITS));
    BEAM_TRY(beam::launch_router_logits(act, bf16, w_router, T, H, E, L.nsplit, at<double>(ws, L.part), s));
    BEAM_TRY(mark(BEAM_STAGE_ROUTER_SELECT));
    BEAM_TRY(beam::launch_router_select(at<double>(ws, L.part), L.nsplit, bias, T, E, shape->n_group,
                                        shape->topk_group, K, shape->routed_scaling, idx, w, nullptr, s));
    BEAM_TRY(mark(BEAM_STAGE_PERMUTE));
    BEAM_TRY(beam::launch_permute(idx, P, E, at<int32_t>(ws, L.scratch), at<int32_t>(ws, L.offsets), sorted,
                                  at<int32_t>(ws, L.pos), bf16 ? tiles : nullptr, bf16 ? ntiles : nullptr,
                                  tile_rows, s));
    BEAM_TRY(mark(BEAM_STAGE_GATE_UP));
    void* h = at<void>(ws, L.h);
    void* ypair = at<void>(ws, L.ypair);
    if (bf16) {
        BEAM_TRY(beam::launch_gate_up(act, true, w_gate, w_up, wf,
                                      sc ? sc->gate : nullptr, sc ? sc->up : nullptr, T, H, I, E, K, sorted, tiles,
                                      ntiles, L.max_tiles, tile_rows, h, s));
    } else {
        BEAM_TRY(beam::launch_gate_up_f32(static_cast<const float*>(act), static_cast<const float*>(w_gate),
                                          static_cast<const float*>(w_up), H, I, K, sorted, idx, P,
                                          static_cast<float*>(h), s));
    }
    BEAM_TRY(mark(BEAM_STAGE_DOWN));
    if (bf16) {
        BEAM_TRY(beam::launch_down(h, true, w_down, wf, sc ? sc->down : nullptr, T, P, H,
                                   I, E, sorted, tiles, ntiles, L.max_tiles, tile_rows, ypair, s));
    } else {
        BEAM_TRY(beam::launch_down_f32(static_cast<const float*>(h), static_cast<const float*>(w_down), H, I, sorted,
                                       idx, P, static_cast<float*>(ypair), s));
    }
    BEAM_TRY(mark(BEAM_STAGE_COMBINE));
    BEAM_TRY(beam::launch_combine(ypair, bf16, w, T, H, K, x, sub ? sub->post_gain : nullptr, sub ? sub->eps : 0.f,
                                  sub ? sub->residual_k : 1.f, out, sub ? moe_y : nullptr, s));
    BEAM_TRY(mark(BEAM_NUM_STAGES));
#undef BEAM_TRY
    return BEAM_OK;
}

}  // namespace

extern "C" {

beam_status beam_moe_forward(const beam_moe_shape* shape, const void* x, const float* w_router, const float* bias,
                             const void* w_gate, const void* w_up, const void* w_down, const beam_sublayer* sub,
                             void* out, int32_t* topk_idx, float* topk_w, void* moe_y, void* ws, size_t ws_bytes,
                             void* const* stage_events, void* stream) {
    return forward_impl(shape, x, w_router, bias, w_gate, w_up, w_down, nullptr, sub, out, topk_idx, topk_w, moe_y,
                        ws, ws_bytes, stage_events, stream);
}

beam_status beam_moe_forward_fp8(const beam_moe_shape* shape, const void* x, const float* w_router, const float* bias,
                                 const uint8_t* w_gate, const uint8_t* w_up, const uint8_t* w_down,
                                 const uint8_t* s_gate, const uint8_t* s_up, const uint8_t* s_down,
                                 const beam_sublayer* sub, void* out, int32_t* topk_idx, float* topk_w, void* moe_y,
                                 void* ws, size_t ws_bytes, void* const* stage_events, void* stream) {
    const WeightScales sc{s_gate, s_up, s_down, beam::WF_E4M3};
    return forward_impl(shape, x, w_router, bias, w_gate, w_up, w_down, &sc, sub, out, topk_idx, topk_w, moe_y, ws,
                        ws_bytes, stage_events, stream);
}

beam_status beam_moe_forward_mxfp4(const beam_moe_shape* shape, const void* x, const float* w_router,
                                   const float* bias, const uint8_t* w_gate, const uint8_t* w_up,
                                   const uint8_t* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                   const uint8_t* s_down, const beam_sublayer* sub, void* out, int32_t* topk_idx,
                                   float* topk_w, void* moe_y, void* ws, size_t ws_bytes, void* const* stage_events,
                                   void* stream) {
    const WeightScales sc{s_gate, s_up, s_down, beam::WF_E2M1};
    return forward_impl(shape, x, w_router, bias, w_gate, w_up, w_down, &sc, sub, out, topk_idx, topk_w, moe_y, ws,
                        ws_bytes, stage_events, stream);
}

}  // extern "C"

// ---- allocation-free forward ------------------------------------------------------------
//
// The workspace of beam_moe_forward_noalloc: a file-scope device array (each GPU that loads
// the library holds its own copy until the process ends).  In host code `scratch` is only a
// stand-in for the symbol; its device address on a GPU comes from hipGetSymbolAddress with
// that GPU current, looked up on the entry point's first call on the GPU and kept per device.
// Nothing in the array has to start at zero: every region of the forward workspace is
// written before it is read within a call.
static __device__ __attribute__((aligned(256))) uint8_t scratch[BEAM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];   // device address of `scratch` per device, nullptr until looked up

// the scratch array's address on the device of `stream` (which must be the current device)
beam_status device_scratch(void* stream, void** addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BEAM_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return BEAM_ERR_HIP;
        if (sdev != dev) return BEAM_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BEAM_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return BEAM_OK;
}

}  // namespace

extern "C" {

beam_status beam_moe_forward_noalloc(const beam_moe_shape* shape, const void* x, const float* w_router,
                                     const float* bias, const void* w_gate, const void* w_up, const void* w_down,
                                     const beam_sublayer* sub, void* out, int32_t* topk_idx, float* topk_w,
                                     void* moe_y, void* const* stage_events, void* stream) {
    if (!shape_valid(shape)) return BEAM_ERR_INVALID_ARG;
    if (!shape_supported(shape)) return BEAM_ERR_UNSUPPORTED;
    if (shape->T == 0)   // no launch, no scratch: argument checks as beam_moe_forward
        return forward_impl(shape, x, w_router, bias, w_gate, w_up, w_down, nullptr, sub, out, topk_idx, topk_w,
                            moe_y, nullptr, 0, stage_events, stream);
    if (make_layout(shape, sub ? BEAM_OP_FORWARD_SUBLAYER : BEAM_OP_FORWARD).total > BEAM_NOALLOC_SCRATCH_BYTES)
        return BEAM_ERR_WORKSPACE;
    void* ws = nullptr;
    const beam_status st = device_scratch(stream, &ws);
    if (st != BEAM_OK) return st;
    return forward_impl(shape, x, w_router, bias, w_gate, w_up, w_down, nullptr, sub, out, topk_idx, topk_w, moe_y,
                        ws, BEAM_NOALLOC_SCRATCH_BYTES, stage_events, stream);
}

}  // extern "C"
