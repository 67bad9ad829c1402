// The C ABI of libmoe_nvfp4: argument validation, workspace sizing and path dispatch.
// Every check here runs on the host before anything is enqueued.
#include <algorithm>

#include "moe_internal.h"

using namespace moe;

namespace moe {
KernelProfile g_profile;
}

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool bank_ok(const moe_bank &b) {
    if (!aligned(b.scale2, 4) || !aligned(b.kpack, 16)) return false;
    if (b.experts != nullptr) return aligned(b.experts, 8);   // base and stride unused
    return b.base != nullptr && aligned(b.base, 16) && b.expert_stride >= 0 &&
           b.expert_stride % 16 == 0;
}

// The three banks of an FFN call: each valid, and gate and up either both with a K-step-packed
// copy or both without (the gate/up GEMM reads both from one form).
bool banks_ok(const moe_bank &gate, const moe_bank &up, const moe_bank &down) {
    return bank_ok(gate) && bank_ok(up) && bank_ok(down) &&
           (gate.kpack == nullptr) == (up.kpack == nullptr);
}

int check_common(int32_t T, int32_t k, int32_t E) {
    if (T < 0 || k < 1 || E < 1 || k > 4096) return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS || (int64_t)T * k > MOE_MAX_PAIRS) return MOE_ESHAPE;
    return MOE_OK;
}

// MOE_PATH_AUTO: the decode path where it measured faster than the GEMM path -- up to 128
// tokens, or up to MOE_AUTO_PAIRS_PER_EXPERT routed pairs per local expert (the decode kernels
// stream an expert's weights once per run of 16 pairs, so their cost grows with the pairs per
// expert, the GEMMs' with the 128-pair M tiles) -- and where its kernels can launch; else the
// GEMM path.
int32_t auto_path(const FfnArgs &a) {
    const int64_t P = (int64_t)a.T * a.k;
    const bool few = a.T <= 128 || P <= (int64_t)MOE_AUTO_PAIRS_PER_EXPERT * a.E;
    return few && decode_supported(a) ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
}

}  // namespace

extern "C" {

size_t moe_route_bucket_ws(int32_t T, int32_t k, int32_t E) {
    if (T < 0 || k < 1 || E < 1) return 0;
    return bucket_ws_bytes(T, k, E);
}

int moe_route_bucket(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t expert_base,
                     int32_t *offsets, int32_t *pair_ids, int32_t *active, int32_t *counts,
                     void *ws, size_t ws_bytes, moe_stream_t stream) {
    int st = check_common(T, k, E);
    if (st != MOE_OK) return st;
    if (!offsets || !active || !counts) return MOE_EINVAL;
    if (T > 0 && (!topk_ids || !pair_ids)) return MOE_EINVAL;
    const size_t need = moe_route_bucket_ws(T, k, E);
    if (ws_bytes < need || (need && !ws)) return MOE_EWS;
    return launch_bucket(topk_ids, T, k, E, expert_base, offsets, pair_ids, active, counts, ws,
                         reinterpret_cast<hipStream_t>(stream));
}

int32_t moe_auto_path(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F) {
    const int st = check_common(T, k, E);
    if (st != MOE_OK) return -st;
    if (H < 64 || F < 64 || H % 64 || F % 64) return -MOE_EINVAL;
    if (H > MOE_MAX_HIDDEN || F > MOE_MAX_FF) return -MOE_ESHAPE;
    const FfnArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, {}, {}, {},
                    T, k, E, H, F, nullptr, nullptr, 0};
    return auto_path(a);
}

size_t moe_ffn_nvfp4_ws(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F) {
    if (T < 0 || k < 1 || E < 1 || H < 1 || F < 1) return 0;
    return std::max(decode_ws_bytes(T, k, E, H, F), prefill_ws_bytes(T, k, E, H, F));
}

int moe_ffn_nvfp4(const uint16_t *x, const float *topk_w, const int32_t *offsets,
                  const int32_t *pair_ids, const int32_t *active, const int32_t *counts,
                  moe_bank gate, moe_bank up, moe_bank down, int32_t T, int32_t k, int32_t E,
                  int32_t H, int32_t F, float *y, int32_t path, void *ws, size_t ws_bytes,
                  moe_stream_t stream) {
    int st = check_common(T, k, E);
    if (st != MOE_OK) return st;
    if (H < 64 || F < 64 || H % 64 || F % 64) return MOE_EINVAL;
    if (H > MOE_MAX_HIDDEN || F > MOE_MAX_FF) return MOE_ESHAPE;
    if (path < MOE_PATH_AUTO || path > MOE_PATH_PREFILL) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !topk_w || !offsets || !pair_ids || !active || !counts || !y || !ws)
        return MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256)) return MOE_EINVAL;
    if (!banks_ok(gate, up, down)) return MOE_EINVAL;
    if (ws_bytes < moe_ffn_nvfp4_ws(T, k, E, H, F)) return MOE_EWS;
    FfnArgs a{x, topk_w, offsets, pair_ids, active, counts, gate, up, down, T, k, E, H, F, y,
              ws, ws_bytes};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (path == MOE_PATH_AUTO) path = auto_path(a);
    return path == MOE_PATH_DECODE ? launch_decode(a, s) : launch_prefill(a, s);
}

namespace {
inline size_t a256(size_t b) { return (b + 255) & ~size_t(255); }
// The fused layer's workspace: the CSR of its fallback path (offsets, pair_ids, active, counts,
// the bucketing's own workspace), then the FFN's.
size_t layer_csr_bytes(int32_t T, int32_t k, int32_t E) {
    const size_t P = (size_t)T * k;
    return a256(4 * ((size_t)E + 1)) + a256(4 * P) + a256(4 * (size_t)E) + 256 +
           a256(bucket_ws_bytes(T, k, E));
}
}  // namespace

size_t moe_layer_nvfp4_ws(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F) {
    if (T < 0 || k < 1 || E < 1 || H < 1 || F < 1) return 0;
    return layer_csr_bytes(T, k, E) + moe_ffn_nvfp4_ws(T, k, E, H, F);
}

int moe_layer_nvfp4(const int32_t *topk_ids, int32_t expert_base, const uint16_t *x,
                    const float *topk_w, moe_bank gate, moe_bank up, moe_bank down, int32_t T,
                    int32_t k, int32_t E, int32_t H, int32_t F, float *y, int32_t path, void *ws,
                    size_t ws_bytes, moe_stream_t stream) {
    int st = check_common(T, k, E);
    if (st != MOE_OK) return st;
    if (H < 64 || F < 64 || H % 64 || F % 64) return MOE_EINVAL;
    if (H > MOE_MAX_HIDDEN || F > MOE_MAX_FF) return MOE_ESHAPE;
    if (path < MOE_PATH_AUTO || path > MOE_PATH_PREFILL) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !x || !topk_w || !y || !ws) return MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256)) return MOE_EINVAL;
    if (!banks_ok(gate, up, down)) return MOE_EINVAL;
    if (ws_bytes < moe_layer_nvfp4_ws(T, k, E, H, F)) return MOE_EWS;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const size_t csr = layer_csr_bytes(T, k, E);
    uint8_t *b = static_cast<uint8_t *>(ws);
    int32_t *offsets = reinterpret_cast<int32_t *>(b);
    int32_t *pair_ids = reinterpret_cast<int32_t *>(b + a256(4 * ((size_t)E + 1)));
    int32_t *active = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(pair_ids) +
                                                  a256(4 * (size_t)T * k));
    int32_t *counts = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(active) +
                                                  a256(4 * (size_t)E));
    void *bws = reinterpret_cast<uint8_t *>(counts) + 256;
    FfnArgs a{x, topk_w, offsets, pair_ids, active, counts, gate, up, down, T, k, E, H, F, y,
              b + csr, ws_bytes - csr};
    if (path == MOE_PATH_AUTO) path = auto_path(a);
    if (path == MOE_PATH_DECODE) {
        // bucketed inside the decode kernels when the routed pairs fit their LDS plan
        FfnArgs f = a;
        f.offsets = f.pair_ids = f.active = f.counts = nullptr;
        f.ids = topk_ids;
        f.expert_base = expert_base;
        if (decode_fused_supported(f)) return launch_decode(f, s);
        if (!decode_supported(a)) return MOE_ESHAPE;
    }
    // otherwise the bucketing kernel first, then the FFN over its CSR
    st = launch_bucket(topk_ids, T, k, E, expert_base, offsets, pair_ids, active, counts, bws, s);
    if (st != MOE_OK) return st;
    return path == MOE_PATH_DECODE ? launch_decode(a, s) : launch_prefill(a, s);
}

int moe_router_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_ids,
                    float *topk_w, moe_stream_t stream) {
    if (T < 0 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_ROUTER_K || (int64_t)T * k > MOE_MAX_PAIRS)
        return MOE_ESHAPE;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w) return MOE_EINVAL;
    return launch_router_topk(logits, T, E, k, topk_ids, topk_w,
                              reinterpret_cast<hipStream_t>(stream));
}

size_t moe_kpack_bytes(int32_t E, int32_t out_f, int32_t in_f) {
    if (E < 1 || out_f < 1 || in_f < kBlockWeights || in_f % kBlockWeights) return 0;
    return (size_t)E * (size_t)kpack_expert_bytes(out_f, in_f);
}

int moe_kpack(moe_bank src, int32_t E, int32_t out_f, int32_t in_f, uint8_t *dst,
              moe_stream_t stream) {
    if (E < 1 || out_f < 1 || in_f < kBlockWeights || in_f % kBlockWeights) return MOE_EINVAL;
    if (!dst || !aligned(dst, 16) || !bank_ok(src)) return MOE_EINVAL;
    if (out_f > MOE_MAX_HIDDEN || in_f > MOE_MAX_HIDDEN || E > MOE_MAX_EXPERTS) return MOE_ESHAPE;
    return launch_kpack(src, E, out_f, in_f, dst, reinterpret_cast<hipStream_t>(stream));
}

int moe_profile_kernel(int32_t kernel_id, void *const *start_events, void *const *stop_events,
                       int32_t n_events) {
    if (kernel_id < MOE_KERNEL_NONE || kernel_id > MOE_KERNEL_ROUTER || n_events < 0)
        return MOE_EINVAL;
    if (kernel_id != MOE_KERNEL_NONE && n_events > 0 && (!start_events || !stop_events))
        return MOE_EINVAL;
    g_profile.kernel = n_events > 0 ? kernel_id : MOE_KERNEL_NONE;
    g_profile.starts = reinterpret_cast<hipEvent_t *>(const_cast<void **>(start_events));
    g_profile.stops = reinterpret_cast<hipEvent_t *>(const_cast<void **>(stop_events));
    g_profile.n = n_events;
    g_profile.next = 0;
    return MOE_OK;
}

int32_t moe_profile_count(void) { return g_profile.next; }

const char *moe_status_str(int status) {
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL";
    case MOE_EWS: return "MOE_EWS";
    case MOE_ESHAPE: return "MOE_ESHAPE";
    case MOE_ELAUNCH: return "MOE_ELAUNCH";
    default: return "MOE_UNKNOWN";
    }
}

}  // extern "C"
