// Decode path of the routed NVFP4 FFN (few tokens per expert, weight-stream bound).
//
// The union gather (moe_union_probe.rs: read each distinct expert's NVFP4 bytes once per call
// instead of once per routed slot): a workgroup owns one active expert and a tile of its weight
// rows. It stages the tile's NVFP4 bytes and the bf16 rows of every token routed to that expert
// in LDS once, then runs all of those tokens against the tile.
//
//   gu_decode: 8 gate rows + the 8 matching up rows per workgroup; each thread takes one row and
//              every 16th scale group of it, decodes E2M1 pairs to bf16 in registers
//              (v_cvt_scalef32_pk_bf16_fp4, exact), forms 16-weight partial dot products with
//              v_dot2_f32_bf16 against the staged activations, scales each partial by its
//              UE4M3 group scale, and the 16 threads of a row reduce with lane shuffles.
//              The epilogue applies SiLU(g) * u and writes h (fp32) in CSR pair order.
//   dn_decode: 32 down rows per workgroup, h rows staged in LDS as fp32, E2M1 pairs decoded to
//              fp32 (v_cvt_scalef32_pk_f32_fp4), fp32 FMAs; writes the per-pair down output
//              ypair (fp32) in CSR pair order.
//   combine:   y[t] = sum over t's local slots in ascending j of w[t,j] * ypair[pos(t,j)].
//
// Grids are sized from host-known bounds (at most min(E, T*k) active experts); workgroups whose
// active-slot index is at or past n_active exit at once, so nothing reads the device counts on
// the host.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kGuRowsPerSide = 8;      // gate rows (and up rows) per gu workgroup
constexpr int kGuRows = 2 * kGuRowsPerSide;
constexpr int kGuLanesPerRow = kThreads / kGuRows;   // 16
constexpr int kDnRows = 32;            // down rows per dn workgroup
constexpr int kDnLanesPerRow = kThreads / kDnRows;   // 8

// Copy `bytes` (a multiple of 16) from 16-byte aligned global memory into LDS.
__device__ __forceinline__ void stage16(uint8_t *lds, const uint8_t *g, int bytes) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(g);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(lds);
    for (int u = threadIdx.x; u < bytes / 16; u += kThreads) dst[u] = src[u];
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int d = W / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, W);
    return v;
}

// Writes pos[pair_ids[q]] = q for q in [q_lo, q_hi).
__device__ __forceinline__ void write_pos(const int32_t *pair_ids, int32_t *pos, int q_lo, int q_hi) {
    for (int q = q_lo + threadIdx.x; q < q_hi; q += kThreads) pos[pair_ids[q]] = q;
}

template <int MT>
__global__ __launch_bounds__(kThreads) void gu_decode_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_ids, const int32_t *__restrict__ active,
    const int32_t *__restrict__ counts, const uint8_t *__restrict__ gate, int64_t gate_stride,
    const uint8_t *__restrict__ up, int64_t up_stride, int32_t k, int32_t E, int32_t P, int32_t H,
    int32_t F, float *__restrict__ h, int32_t *__restrict__ pos) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int rb = H / kBlockWeights * kBlockBytes;
    uint8_t *wbuf = smem;                                          // [16][rb] NVFP4 rows
    uint16_t *xbuf = reinterpret_cast<uint16_t *>(smem + kGuRows * rb);  // [MT][H] bf16
    float *red = reinterpret_cast<float *>(xbuf + MT * H);         // [16][MT]

    const int a = blockIdx.y;
    if (blockIdx.x == 0 && a == 0) write_pos(pair_ids, pos, offsets[E], P);  // non-local pairs
    if (a >= counts[0]) return;
    const int e = active[a];
    const int q0 = offsets[e], m = offsets[e + 1] - q0;
    if (blockIdx.x == 0) write_pos(pair_ids, pos, q0, q0 + m);

    const int o0 = blockIdx.x * kGuRowsPerSide;
    const int span = kGuRowsPerSide * rb;
    stage16(wbuf, gate + e * gate_stride + (int64_t)o0 * rb, span);
    stage16(wbuf + span, up + e * up_stride + (int64_t)o0 * rb, span);

    const int tid = threadIdx.x;
    const int row = tid / kGuLanesPerRow, sub = tid % kGuLanesPerRow;
    const uint8_t *wrow = wbuf + row * rb;
    const int groups = H / kGroup;

    for (int c0 = 0; c0 < m; c0 += MT) {
        const int mt = min(MT, m - c0);
        if (c0) __syncthreads();  // previous chunk's x and red are no longer read
        for (int i = 0; i < mt; i++) {
            const int t = pair_ids[q0 + c0 + i] / k;
            stage16(reinterpret_cast<uint8_t *>(xbuf + i * H),
                    reinterpret_cast<const uint8_t *>(x + (int64_t)t * H), H * 2);
        }
        __syncthreads();

        float acc[MT];
#pragma unroll
        for (int i = 0; i < MT; i++) acc[i] = 0.f;
        for (int g = sub; g < groups; g += kGuLanesPerRow) {
            const uint8_t *blk = wrow + (g >> 2) * kBlockBytes;
            const float S = ue4m3_to_f32(blk[g & 3]);
            const uint32_t *cw = reinterpret_cast<const uint32_t *>(blk + 4 + 8 * (g & 3));
            const uint32_t c0w = cw[0], c1w = cw[1];
            uint32_t wv[8];
            wv[0] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(c0w));
            wv[1] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(c0w));
            wv[2] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(c0w));
            wv[3] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(c0w));
            wv[4] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(c1w));
            wv[5] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(c1w));
            wv[6] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(c1w));
            wv[7] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(c1w));
#pragma unroll
            for (int i = 0; i < MT; i++) {
                if (i < mt) {
                    const u32x4_t *xr = reinterpret_cast<const u32x4_t *>(xbuf + i * H + g * kGroup);
                    const u32x4_t xa = xr[0], xb = xr[1];
                    float p = 0.f;
                    p = dot2_bf16(wv[0], xa[0], p);
                    p = dot2_bf16(wv[1], xa[1], p);
                    p = dot2_bf16(wv[2], xa[2], p);
                    p = dot2_bf16(wv[3], xa[3], p);
                    p = dot2_bf16(wv[4], xb[0], p);
                    p = dot2_bf16(wv[5], xb[1], p);
                    p = dot2_bf16(wv[6], xb[2], p);
                    p = dot2_bf16(wv[7], xb[3], p);
                    acc[i] = fmaf(S, p, acc[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MT; i++) {
            if (i < mt) {
                const float v = group_sum<kGuLanesPerRow>(acc[i]);
                if (sub == 0) red[row * MT + i] = v;
            }
        }
        __syncthreads();
        if (tid < kGuRowsPerSide * mt) {
            const int oi = tid % kGuRowsPerSide, i = tid / kGuRowsPerSide;
            const float gv = red[oi * MT + i], uv = red[(kGuRowsPerSide + oi) * MT + i];
            h[(int64_t)(q0 + c0 + i) * F + o0 + oi] = silu(gv) * uv;
        }
    }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void dn_decode_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ active,
    const int32_t *__restrict__ counts, const uint8_t *__restrict__ down, int64_t down_stride,
    int32_t H, int32_t F, const float *__restrict__ h, float *__restrict__ ypair) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int rb = F / kBlockWeights * kBlockBytes;
    uint8_t *wbuf = smem;                                        // [32][rb]
    float *hbuf = reinterpret_cast<float *>(smem + kDnRows * rb);  // [MT][F]

    const int a = blockIdx.y;
    if (a >= counts[0]) return;
    const int e = active[a];
    const int q0 = offsets[e], m = offsets[e + 1] - q0;
    const int r0 = blockIdx.x * kDnRows;
    stage16(wbuf, down + e * down_stride + (int64_t)r0 * rb, kDnRows * rb);

    const int tid = threadIdx.x;
    const int row = tid / kDnLanesPerRow, sub = tid % kDnLanesPerRow;
    const uint8_t *wrow = wbuf + row * rb;
    const int groups = F / kGroup;

    for (int c0 = 0; c0 < m; c0 += MT) {
        const int mt = min(MT, m - c0);
        if (c0) __syncthreads();
        stage16(reinterpret_cast<uint8_t *>(hbuf),
                reinterpret_cast<const uint8_t *>(h + (int64_t)(q0 + c0) * F), mt * F * 4);
        __syncthreads();
        float acc[MT];
#pragma unroll
        for (int i = 0; i < MT; i++) acc[i] = 0.f;
        for (int g = sub; g < groups; g += kDnLanesPerRow) {
            const uint8_t *blk = wrow + (g >> 2) * kBlockBytes;
            const float S = ue4m3_to_f32(blk[g & 3]);
            const uint32_t *cw = reinterpret_cast<const uint32_t *>(blk + 4 + 8 * (g & 3));
            const uint32_t c0w = cw[0], c1w = cw[1];
            f32x2_t wv[8];
            wv[0] = e2m1x2_to_f32<0>(c0w);
            wv[1] = e2m1x2_to_f32<1>(c0w);
            wv[2] = e2m1x2_to_f32<2>(c0w);
            wv[3] = e2m1x2_to_f32<3>(c0w);
            wv[4] = e2m1x2_to_f32<0>(c1w);
            wv[5] = e2m1x2_to_f32<1>(c1w);
            wv[6] = e2m1x2_to_f32<2>(c1w);
            wv[7] = e2m1x2_to_f32<3>(c1w);
#pragma unroll
            for (int i = 0; i < MT; i++) {
                if (i < mt) {
                    const f32x4_t *hr = reinterpret_cast<const f32x4_t *>(hbuf + i * F + g * kGroup);
                    float p = 0.f;
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        const f32x4_t hv = hr[v];
                        p = fmaf(wv[2 * v][0], hv[0], p);
                        p = fmaf(wv[2 * v][1], hv[1], p);
                        p = fmaf(wv[2 * v + 1][0], hv[2], p);
                        p = fmaf(wv[2 * v + 1][1], hv[3], p);
                    }
                    acc[i] = fmaf(S, p, acc[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MT; i++) {
            if (i < mt) {
                const float v = group_sum<kDnLanesPerRow>(acc[i]);
                if (sub == 0) ypair[(int64_t)(q0 + c0 + i) * H + r0 + row] = v;
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float *__restrict__ w, const int32_t *__restrict__ pos, const int32_t *__restrict__ offsets,
    int32_t E, const float *__restrict__ ypair, int32_t k, int32_t H, float *__restrict__ y) {
    const int t = blockIdx.y;
    const int r = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (r >= H) return;
    const int n_local = offsets[E];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
        const int p = t * k + j;
        const int q = pos[p];
        if (q < n_local) {
            const float wt = w[p];
            const f32x4_t v = *reinterpret_cast<const f32x4_t *>(ypair + (int64_t)q * H + r);
            acc[0] = fmaf(wt, v[0], acc[0]);
            acc[1] = fmaf(wt, v[1], acc[1]);
            acc[2] = fmaf(wt, v[2], acc[2]);
            acc[3] = fmaf(wt, v[3], acc[3]);
        }
    }
    *reinterpret_cast<f32x4_t *>(y + (int64_t)t * H + r) = acc;
}

constexpr int kMT = 8;

struct DecodeWs {
    int32_t *pos;   // [P]
    float *h;       // [P][F]
    float *ypair;   // [P][H]
};

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

DecodeWs carve(void *ws, int32_t P, int32_t H, int32_t F) {
    uint8_t *b = static_cast<uint8_t *>(ws);
    DecodeWs d;
    d.pos = reinterpret_cast<int32_t *>(b);
    b += align256(sizeof(int32_t) * (size_t)P);
    d.h = reinterpret_cast<float *>(b);
    b += align256(sizeof(float) * (size_t)P * F);
    d.ypair = reinterpret_cast<float *>(b);
    return d;
}

bool set_lds_attr(const void *fn, size_t bytes) {
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) ==
           hipSuccess;
}

}  // namespace

size_t decode_ws_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F) {
    (void)E;
    const size_t P = (size_t)T * k;
    return align256(sizeof(int32_t) * P) + align256(sizeof(float) * P * F) +
           align256(sizeof(float) * P * H);
}

int launch_combine(const float *w, const int32_t *pos, const int32_t *offsets, int32_t E,
                   const float *ypair, int32_t T, int32_t k, int32_t H, float *y, hipStream_t s) {
    dim3 grid((H / 4 + kThreads - 1) / kThreads, T);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, s, w, pos, offsets, E, ypair, k,
                       H, y);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

int launch_decode(const FfnArgs &a, hipStream_t s) {
    const int32_t P = a.T * a.k;
    const DecodeWs d = carve(a.ws, P, a.H, a.F);
    const int max_active = (int)std::min<int64_t>(a.E, P);
    const size_t rbh = (size_t)row_bytes(a.H), rbf = (size_t)row_bytes(a.F);

    const size_t gu_lds = kGuRows * rbh + (size_t)kMT * a.H * 2 + kGuRows * kMT * 4;
    const size_t dn_lds = kDnRows * rbf + (size_t)kMT * a.F * 4;
    if (gu_lds > 160 * 1024 || dn_lds > 160 * 1024) return MOE_ESHAPE;
    static bool attrs = false;
    if (!attrs) {
        if (!set_lds_attr(reinterpret_cast<const void *>(gu_decode_kernel<kMT>), 160 * 1024) ||
            !set_lds_attr(reinterpret_cast<const void *>(dn_decode_kernel<kMT>), 160 * 1024))
            return MOE_ELAUNCH;
        attrs = true;
    }
    hipLaunchKernelGGL(gu_decode_kernel<kMT>, dim3(a.F / kGuRowsPerSide, max_active),
                       dim3(kThreads), gu_lds, s, a.x, a.offsets, a.pair_ids, a.active, a.counts,
                       a.gate.base, a.gate.expert_stride, a.up.base, a.up.expert_stride, a.k, a.E,
                       P, a.H, a.F, d.h, d.pos);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    hipLaunchKernelGGL(dn_decode_kernel<kMT>, dim3(a.H / kDnRows, max_active), dim3(kThreads),
                       dn_lds, s, a.offsets, a.active, a.counts, a.down.base,
                       a.down.expert_stride, a.H, a.F, d.h, d.ypair);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    return launch_combine(a.w, d.pos, a.offsets, a.E, d.ypair, a.T, a.k, a.H, a.y, s);
}

}  // namespace moe
