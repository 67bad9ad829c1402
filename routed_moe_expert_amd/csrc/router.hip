// Router step of the routed layer: per token, the top-k expert ids and their softmax weights
// from fp32 router logits, written in the [T, k] layouts that moe_route_bucket and moe_ffn_nvfp4
// take (the pages route k distinct experts per token with softmax weights; the selection order
// and the tie rule are this library's reading, stated in include/moe_nvfp4.h).
//
// One wavefront per token. Lane l holds the logits of experts l, l + 64, l + 128, ... in
// registers (one coalesced pass over the row) and a bit mask of those it still holds. Each of the
// k rounds takes every lane's best remaining (logit, expert) pair and reduces the 64 candidates
// across the wavefront in two DPP passes (VALU lane moves, no LDS round trips): the largest logit,
// then the lowest expert id among the lanes holding it. That is the total order "larger logit
// first, then lower expert id", whose winner is unique, so the selection is deterministic. The
// owning lane drops the winner. Lane j keeps round j's winner; the softmax over the k winners is
// then one exp per lane and a DPP-tree sum (fixed order), and lanes 0..k-1 store slot j.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;                      // four tokens per workgroup
constexpr int kRouterMaxPerLane = MOE_MAX_EXPERTS / 64;  // 32: the live mask is one dword

// DPP lane move (dpp_ctrl CTRL, rows in ROW_MASK; lanes of other rows keep `old`)
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}

// Reductions over the 64 lanes, result in every lane (read from lane 63). The butterfly steps
// swap lanes 1 and 2 apart within quads (0xB1, 0x4E), mirror each half row (0x141) and each row
// (0x140), after which every row holds its own result; broadcasting lane 15 into the next row
// (0x142, rows 1 and 3) and lane 31 into rows 2 and 3 (0x143) leaves the total in row 3.
template <typename Op>
__device__ __forceinline__ int wave_reduce(int v, Op op) {
    v = op(v, dpp<0xB1>(v, v));
    v = op(v, dpp<0x4E>(v, v));
    v = op(v, dpp<0x141>(v, v));
    v = op(v, dpp<0x140>(v, v));
    v = op(v, dpp<0x142, 0xA>(v, v));
    v = op(v, dpp<0x143, 0xC>(v, v));
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_max(float v) {
    return __int_as_float(wave_reduce(__float_as_int(v), [](int a, int b) {
        return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
    }));
}
__device__ __forceinline__ int wave_min(int v) {
    return wave_reduce(v, [](int a, int b) { return min(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
    return __int_as_float(wave_reduce(__float_as_int(v), [](int a, int b) {
        return __float_as_int(__int_as_float(a) + __int_as_float(b));
    }));
}

// PER: logits held per lane, a power of two with 64 PER >= E
template <int PER>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(
    const float *__restrict__ logits, int32_t T, int32_t E, int32_t k, int32_t *__restrict__ ids,
    float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * (kRouterThreads / 64) + (threadIdx.x >> 6);
    if (t >= T) return;   // wave-uniform
    const float *row = logits + t * E;
    float v[PER];
    uint32_t live = 0;   // bit i: expert lane + 64 i exists and is not yet taken
#pragma unroll
    for (int i = 0; i < PER; i++) {   // branch-free: lanes past E re-read the last logit
        const int e = lane + 64 * i;
        v[i] = row[min(e, E - 1)];
        live |= (e < E ? 1u : 0u) << i;
    }
    float mine_v = 0.f, top = 0.f;
    int mine_e = 0;
#pragma unroll 1
    for (int j = 0; j < k; j++) {
        // this lane's best remaining pair (lower i first among equal logits: lower expert id)
        float lv = 0.f;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const bool take = ((live >> i) & 1u) && (bi < 0 || v[i] > lv);
            lv = take ? v[i] : lv;
            bi = take ? i : bi;
        }
        // the wavefront's best: the largest logit (a lane with nothing left offers -inf; logits
        // are finite), then the lowest expert id among the lanes offering it (equal compares
        // treat -0 and +0 alike, as the selection order does)
        const float bv = wave_max(bi >= 0 ? lv : -INFINITY);
        const int be = wave_min(bi >= 0 && lv == bv ? lane + 64 * bi : 0x7fffffff);
        if ((be & 63) == lane) live &= ~(1u << (be >> 6));   // the owner drops the winner
        if (j == 0) top = bv;
        if (lane == j) {
            mine_v = bv;
            mine_e = be;
        }
    }
    // softmax over the k winners: w_j = exp(l_j - l_0) / sum over the winners
    const float ex = lane < k ? expf(mine_v - top) : 0.f;
    const float sum = wave_sum(ex);
    if (lane < k) {
        ids[t * k + lane] = mine_e;
        w[t * k + lane] = ex / sum;
    }
}

}  // namespace

int launch_router_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids,
                       float *w, hipStream_t s) {
    const int per_block = kRouterThreads / 64;
    const int blocks = (T + per_block - 1) / per_block;
    const int per = (E + 63) / 64;
    const dim3 g(blocks), b(kRouterThreads);
    prof_start(MOE_KERNEL_ROUTER, s);
    if (per <= 1) hipLaunchKernelGGL(router_topk_kernel<1>, g, b, 0, s, logits, T, E, k, ids, w);
    else if (per <= 2) hipLaunchKernelGGL(router_topk_kernel<2>, g, b, 0, s, logits, T, E, k, ids, w);
    else if (per <= 4) hipLaunchKernelGGL(router_topk_kernel<4>, g, b, 0, s, logits, T, E, k, ids, w);
    else if (per <= 8) hipLaunchKernelGGL(router_topk_kernel<8>, g, b, 0, s, logits, T, E, k, ids, w);
    else if (per <= 16)
        hipLaunchKernelGGL(router_topk_kernel<16>, g, b, 0, s, logits, T, E, k, ids, w);
    else
        hipLaunchKernelGGL(router_topk_kernel<kRouterMaxPerLane>, g, b, 0, s, logits, T, E, k, ids,
                           w);
    prof_stop(MOE_KERNEL_ROUTER, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
