// Decode path of the routed NVFP4 FFN (few tokens per expert, weight-stream bound).
//
// The union gather (moe_union_probe.rs: read each distinct expert's NVFP4 bytes once per call
// instead of once per routed slot): work items are (active expert, tile of weight rows); each
// item's NVFP4 tile is read from HBM once and run against every token routed to that expert,
// whose rows are staged in LDS once per expert.
//
//   gu_decode: items of 8 gate rows + the 8 matching up rows. Each thread takes one row and
//              every 16th scale group of it, decodes E2M1 pairs to bf16 in registers
//              (v_cvt_scalef32_pk_bf16_fp4, exact), forms 16-weight partial dot products with
//              v_dot2_f32_bf16 against the staged activations, scales each partial by its
//              UE4M3 group scale, and the 16 threads of a row reduce with lane shuffles.
//              The epilogue applies SiLU(g) * u and writes h (fp32) in CSR pair order.
//   dn_decode: items of 64 down rows, h rows staged in LDS as fp32, E2M1 pairs decoded to fp32
//              (v_cvt_scalef32_pk_f32_fp4), fp32 FMAs; writes the per-pair down output ypair
//              (fp32) at row p = t*k + j of its pair.
//   combine:   y[t] = sum over t's local slots in ascending j of w[t,j] * ypair[t*k + j]; the
//              pair -> CSR slot map only says which slots are local.
//
// Both FFN kernels are persistent: a grid of at most two 512-thread workgroups per CU splits the
// (expert, tile) items into contiguous ranges, read from the device CSR (nothing is read back on
// the host). Tiles stream through three LDS buffers with direct-to-LDS loads, two tiles in
// flight while one is computed.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;          // 8 waves: 4 per SIMD with two workgroups per CU
constexpr int kGuO = 8;                // output features per gu item: 8 gate rows + 8 up rows
constexpr int kGuLanes = 32;           // lanes per weight row: wave o holds feature o, its gate
                                       // row in lanes 0..31 and its up row in lanes 32..63
constexpr int kDnRows = 64;            // down rows per dn item
constexpr int kDnLanes = kThreads / kDnRows;         // 8 lanes per down row
constexpr int kNBuf = 3;               // weight tiles in LDS: one computed, two in flight
constexpr int kWgPerCu = 2;
constexpr int kCUs = 256;

// 16 E2M1 codes (two code dwords) -> 8 bf16 pairs, exact.
__device__ __forceinline__ void e2m1x16_to_bf16(uint32_t c0, uint32_t c1, uint32_t (&w)[8]) {
    w[0] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(c0));
    w[1] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(c0));
    w[2] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(c0));
    w[3] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(c0));
    w[4] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<0>(c1));
    w[5] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<1>(c1));
    w[6] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<2>(c1));
    w[7] = __builtin_bit_cast(uint32_t, e2m1x2_to_bf16<3>(c1));
}

__device__ __forceinline__ float dot16(const uint32_t (&w)[8], const u32x4_t &xa, const u32x4_t &xb) {
    float p = 0.f;
    p = dot2_bf16(w[0], xa[0], p);
    p = dot2_bf16(w[1], xa[1], p);
    p = dot2_bf16(w[2], xa[2], p);
    p = dot2_bf16(w[3], xa[3], p);
    p = dot2_bf16(w[4], xb[0], p);
    p = dot2_bf16(w[5], xb[1], p);
    p = dot2_bf16(w[6], xb[2], p);
    p = dot2_bf16(w[7], xb[3], p);
    return p;
}

// One gu item: thread (o, sub) accumulates the gate row and the up row of feature o over scale
// groups sub, sub+32, ... against the mt staged token rows; each x load serves both rows.
// GPL > 0: every lane has exactly GPL groups (H = 512*GPL) and the loop is fully unrolled, so
// all of an item's LDS reads issue before the first wait; GPL = 0: any H, runtime loop.
// One weight row (this lane's) against the mt staged token rows over scale groups sub, sub+32,
// ... GPL > 0: every lane has exactly GPL groups (H = 512*GPL) and the loop is fully unrolled,
// so all of an item's LDS reads issue before the first wait; GPL = 0: any H, runtime loop.
template <int MT, int GPL>
__device__ __forceinline__ void gu_row_dot(const uint8_t *row, const uint16_t *xbuf, int sub,
                                           int H, int mt, float (&acc)[MT]) {
#pragma unroll
    for (int i = 0; i < MT; i++) acc[i] = 0.f;
    auto group = [&](int g) {
        const int boff = (g >> 2) * kBlockBytes, j = g & 3;
        const float S = ue4m3_to_f32(row[boff + j]);
        const uint32_t *c = reinterpret_cast<const uint32_t *>(row + boff + 4 + 8 * j);
        uint32_t w[8];
        e2m1x16_to_bf16(c[0], c[1], w);
#pragma unroll
        for (int i = 0; i < MT; i++) {
            if (i < mt) {
                const u32x4_t *xr = reinterpret_cast<const u32x4_t *>(xbuf + i * H + g * kGroup);
                acc[i] = fmaf(S, dot16(w, xr[0], xr[1]), acc[i]);
            }
        }
    };
    if constexpr (GPL > 0 && MT == 1) {
#pragma unroll
        for (int it = 0; it < GPL; it++) group(sub + it * kGuLanes);
    } else if constexpr (GPL > 0) {   // two token rows: unroll less to stay within 128 VGPRs
#pragma unroll 2
        for (int it = 0; it < GPL; it++) group(sub + it * kGuLanes);
    } else {
        const int groups = H / kGroup;
#pragma nounroll
        for (int g = sub; g < groups; g += kGuLanes) group(g);
    }
}

// One down row (this lane's) against the mt staged fp32 h rows over scale groups sub, sub+8, ...
template <int MT, int GPL>
__device__ __forceinline__ void dn_row_dot(const uint8_t *row, const float *hbuf, int sub, int F,
                                           int mt, float (&acc)[MT]) {
#pragma unroll
    for (int i = 0; i < MT; i++) acc[i] = 0.f;
    auto group = [&](int g) {
        const int boff = (g >> 2) * kBlockBytes, j = g & 3;
        const float S = ue4m3_to_f32(row[boff + j]);
        const uint32_t *c = reinterpret_cast<const uint32_t *>(row + boff + 4 + 8 * j);
        f32x2_t w[8];
        w[0] = e2m1x2_to_f32<0>(c[0]); w[1] = e2m1x2_to_f32<1>(c[0]);
        w[2] = e2m1x2_to_f32<2>(c[0]); w[3] = e2m1x2_to_f32<3>(c[0]);
        w[4] = e2m1x2_to_f32<0>(c[1]); w[5] = e2m1x2_to_f32<1>(c[1]);
        w[6] = e2m1x2_to_f32<2>(c[1]); w[7] = e2m1x2_to_f32<3>(c[1]);
#pragma unroll
        for (int i = 0; i < MT; i++) {
            if (i < mt) {
                const f32x4_t *hr = reinterpret_cast<const f32x4_t *>(hbuf + i * F + g * kGroup);
                float p = 0.f;
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const f32x4_t hv = hr[v];
                    p = fmaf(w[2 * v][0], hv[0], p);
                    p = fmaf(w[2 * v][1], hv[1], p);
                    p = fmaf(w[2 * v + 1][0], hv[2], p);
                    p = fmaf(w[2 * v + 1][1], hv[3], p);
                }
                acc[i] = fmaf(S, p, acc[i]);
            }
        }
    };
    if constexpr (GPL > 0 && MT == 1) {
#pragma unroll
        for (int it = 0; it < GPL; it++) group(sub + it * kDnLanes);
    } else if constexpr (GPL > 0) {   // two fp32 h rows: unroll less to stay within 128 VGPRs
#pragma unroll 2
        for (int it = 0; it < GPL; it++) group(sub + it * kDnLanes);
    } else {
        const int groups = F / kGroup;
#pragma nounroll
        for (int g = sub; g < groups; g += kDnLanes) group(g);
    }
}

// Item range of this workgroup: items are (active expert a, row tile t) in a-major order, split
// into equal contiguous ranges over the grid, so a workgroup mostly stays on one expert and its
// token rows are staged once.
__device__ __forceinline__ void item_range(int total, int &i0, int &i1) {
    const int per = (total + gridDim.x - 1) / gridDim.x;
    i0 = min((int)blockIdx.x * per, total);
    i1 = min(i0 + per, total);
}

// The CSR entries a workgroup needs (its experts, their first CSR slot, pair count and first MT
// pair ids), fetched once into LDS at kernel start: reading them per item would put a chain of
// dependent scalar loads (active -> offsets -> pair_ids), each a round trip to memory the
// previous kernel just wrote, in front of every tile.
constexpr int kMaxMeta = 32;   // experts per workgroup range; grids are sized so this holds
template <int MT>
struct Meta {
    int e[kMaxMeta], q0[kMaxMeta], m[kMaxMeta], pid[kMaxMeta][MT];
};

template <int MT>
__device__ __forceinline__ void load_meta(Meta<MT> &meta, const int32_t *active,
                                          const int32_t *offsets, const int32_t *pair_ids,
                                          int a_first, int na) {
    const int tid = threadIdx.x;
    if (tid < na) {
        const int e = active[a_first + tid];
        const int q0 = offsets[e], m = offsets[e + 1] - q0;
        meta.e[tid] = e;
        meta.q0[tid] = q0;
        meta.m[tid] = m;
#pragma unroll
        for (int j = 0; j < MT; j++) meta.pid[tid][j] = j < m ? pair_ids[q0 + j] : 0;
    }
}

// Gate/up + SiLU * up over the union of active experts. Persistent workgroups stream their
// 16-row NVFP4 tiles through kNBuf LDS buffers with direct-to-LDS loads: two tiles in flight
// while one is computed. Tile i is awaited with "at most the next tile's loads outstanding";
// vector-memory loads complete in issue order, so that wait also covers tile i whatever stores
// were issued in between.
template <int MT, int GPL>
__global__ __launch_bounds__(kThreads, 4) void gu_decode_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_ids, const int32_t *__restrict__ active,
    const int32_t *__restrict__ counts, const uint8_t *__restrict__ gate, int64_t gate_stride,
    const uint8_t *__restrict__ up, int64_t up_stride, int32_t k, int32_t P, int32_t H, int32_t F,
    float *__restrict__ h, int32_t *__restrict__ pos) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int rb = H / kBlockWeights * kBlockBytes;
    const int side = kGuO * rb, tile_bytes = 2 * side;
    uint8_t *wb = smem;                                                     // [kNBuf][16 rows]
    uint16_t *xbuf = reinterpret_cast<uint16_t *>(smem + kNBuf * tile_bytes);  // [MT][H] bf16
    __shared__ Meta<MT> meta;
    const int tid = threadIdx.x;

    const int tiles = F / kGuO;
    int i0, i1;
    item_range(counts[0] * tiles, i0, i1);
    const int o = tid >> 6, lane = tid & 63, sub = lane & 31;
    const int wrow = (lane < 32 ? 0 : side) + o * rb;   // this lane's row within a tile
    const int n_inst = 2 * stage_async_count<kThreads>(side);
    const int a_first = i0 / tiles;

    auto issue_e = [&](int i, int e) {
        const int t = i % tiles;
        uint8_t *dst = wb + ((i - i0) % kNBuf) * tile_bytes;
        stage_async<kThreads>(dst, gate + e * gate_stride + (int64_t)t * side, side);
        stage_async<kThreads>(dst + side, up + e * up_stride + (int64_t)t * side, side);
    };
    auto issue = [&](int i) { issue_e(i, meta.e[i / tiles - a_first]); };
    if (i0 < i1) {
        // the first two tiles go out before the rest of the CSR metadata is fetched
        issue_e(i0, active[i0 / tiles]);
        if (i0 + 1 < i1) issue_e(i0 + 1, active[(i0 + 1) / tiles]);
        load_meta<MT>(meta, active, offsets, pair_ids, a_first,
                      min((i1 - 1) / tiles - a_first + 1, kMaxMeta));
        lds_barrier();
    }
    auto stage_x = [&](int a, int c0, int mt) {   // token rows of CSR pairs c0..c0+mt-1
        for (int j = 0; j < mt; j++) {
            const int p = c0 + j < MT ? meta.pid[a][c0 + j] : pair_ids[meta.q0[a] + c0 + j];
            stage_async<kThreads>(xbuf + j * H, x + (int64_t)(p / k) * H, H * 2);
        }
    };
    auto finish = [&](float (&acc)[MT], int q0, int o0, int mt) {
#pragma unroll
        for (int j = 0; j < MT; j++) {
            if (j < mt) {
                const float v = sum32_dpp(acc[j]);   // gate sum in lanes 16..31, up in 48..63
                const float gv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, v), 31));
                const float uv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, v), 63));
                if (lane == 0) h[(int64_t)(q0 + j) * F + o0 + o] = silu(gv) * uv;
            }
        }
    };

    int cur_a = -1;
    for (int i = i0; i < i1; i++) {
        const int a = i / tiles - a_first, t = i % tiles;
        const int q0 = meta.q0[a], m = meta.m[a];
        const uint8_t *wt = wb + ((i - i0) % kNBuf) * tile_bytes;
        if (a != cur_a && m <= MT) {  // new expert: stage its token rows once xbuf is free
            lds_barrier();
            stage_x(a, 0, m);
            lds_dma_wait();
            cur_a = a;
        } else {
            vm_wait_le(i + 1 < i1 ? n_inst : 0);  // tile i landed; only tile i+1 outstanding
        }
        lds_barrier();   // tile i visible to all; everyone is done with item i-1's buffer
        if (i + 2 < i1) issue(i + 2);
        // one pass when the expert's rows are staged; otherwise token chunks, each restaged
        // (which waits on all loads)
        const bool chunked = m > MT;
        for (int c0 = 0; c0 < m; c0 += MT) {
            const int mt = min(MT, m - c0);
            if (chunked) {
                lds_barrier();
                stage_x(a, c0, mt);
                lds_dma_wait();
                lds_barrier();
            }
            float acc[MT];
            gu_row_dot<MT, GPL>(wt + wrow, xbuf, sub, H, mt, acc);
            finish(acc, q0 + c0, t * kGuO, mt);
        }
        if (chunked) cur_a = -1;
    }
    // pair -> CSR slot map for the combine (not needed before it)
    for (int q = blockIdx.x * kThreads + tid; q < P; q += gridDim.x * kThreads) pos[pair_ids[q]] = q;
}

// Down projection over the union of active experts, same streaming scheme with 64-row tiles;
// the per-pair rows go to ypair at the pair id.
template <int MT, int GPL>
__global__ __launch_bounds__(kThreads, 4) void dn_decode_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ pair_ids,
    const int32_t *__restrict__ active, const int32_t *__restrict__ counts,
    const uint8_t *__restrict__ down, int64_t down_stride, int32_t H, int32_t F,
    const float *__restrict__ h, float *__restrict__ ypair) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int rb = F / kBlockWeights * kBlockBytes;
    const int tile_bytes = kDnRows * rb;
    uint8_t *wb = smem;                                                     // [kNBuf][64 rows]
    float *hbuf = reinterpret_cast<float *>(smem + kNBuf * tile_bytes);     // [MT][F]
    __shared__ Meta<MT> meta;
    const int tid = threadIdx.x;

    const int tiles = H / kDnRows;
    int i0, i1;
    item_range(counts[0] * tiles, i0, i1);
    if (i0 >= i1) return;
    const int a_first = i0 / tiles;
    const int row = tid / kDnLanes, sub = tid % kDnLanes;   // this lane's row of the tile
    const int n_inst = stage_async_count<kThreads>(tile_bytes);

    auto issue_e = [&](int i, int e) {
        stage_async<kThreads>(wb + ((i - i0) % kNBuf) * tile_bytes,
                              down + e * down_stride + (int64_t)(i % tiles) * tile_bytes, tile_bytes);
    };
    auto issue = [&](int i) { issue_e(i, meta.e[i / tiles - a_first]); };
    issue_e(i0, active[i0 / tiles]);
    if (i0 + 1 < i1) issue_e(i0 + 1, active[(i0 + 1) / tiles]);
    load_meta<MT>(meta, active, offsets, pair_ids, a_first,
                  min((i1 - 1) / tiles - a_first + 1, kMaxMeta));
    lds_barrier();
    auto finish = [&](float (&acc)[MT], int a, int c0, int r0, int mt) {
#pragma unroll
        for (int j = 0; j < MT; j++) {
            if (j < mt) {
                const float v = sum8_dpp(acc[j]);
                if (sub == 0) {
                    const int p = c0 + j < MT ? meta.pid[a][c0 + j] : pair_ids[meta.q0[a] + c0 + j];
                    ypair[(int64_t)p * H + r0 + row] = v;
                }
            }
        }
    };

    int cur_a = -1;
    for (int i = i0; i < i1; i++) {
        const int a = i / tiles - a_first, t = i % tiles;
        const int q0 = meta.q0[a], m = meta.m[a];
        const uint8_t *wt = wb + ((i - i0) % kNBuf) * tile_bytes;
        if (a != cur_a && m <= MT) {
            lds_barrier();
            stage_async<kThreads>(hbuf, h + (int64_t)q0 * F, m * F * 4);
            lds_dma_wait();
            cur_a = a;
        } else {
            vm_wait_le(i + 1 < i1 ? n_inst : 0);
        }
        lds_barrier();
        if (i + 2 < i1) issue(i + 2);
        const bool chunked = m > MT;
        for (int c0 = 0; c0 < m; c0 += MT) {
            const int mt = min(MT, m - c0);
            if (chunked) {
                lds_barrier();
                stage_async<kThreads>(hbuf, h + (int64_t)(q0 + c0) * F, mt * F * 4);
                lds_dma_wait();
                lds_barrier();
            }
            float acc[MT];
            dn_row_dot<MT, GPL>(wt + row * rb, hbuf, sub, F, mt, acc);
            finish(acc, a, c0, t * kDnRows, mt);
        }
        if (chunked) cur_a = -1;
    }
}

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float *__restrict__ w, const int32_t *__restrict__ pos, const int32_t *__restrict__ offsets,
    int32_t E, const float *__restrict__ ypair, int32_t k, int32_t H, float *__restrict__ y) {
    constexpr int kJ = 8;  // slots whose loads are issued together
    const int t = blockIdx.y;
    const int r = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (r >= H) return;
    const int n_local = offsets[E];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += kJ) {
        int q[kJ];
        float wt[kJ];
        f32x4_t v[kJ];
#pragma unroll
        for (int u = 0; u < kJ; u++) {
            const int p = t * k + j0 + u;
            const bool in = j0 + u < k;
            q[u] = in ? pos[p] : n_local;
            wt[u] = in ? w[p] : 0.f;
            // rows of non-local slots hold stale data; they are loaded and then skipped
            v[u] = in ? *reinterpret_cast<const f32x4_t *>(ypair + (int64_t)p * H + r)
                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kJ; u++) {   // ascending slot order
            if (q[u] < n_local) {
                acc[0] = fmaf(wt[u], v[u][0], acc[0]);
                acc[1] = fmaf(wt[u], v[u][1], acc[1]);
                acc[2] = fmaf(wt[u], v[u][2], acc[2]);
                acc[3] = fmaf(wt[u], v[u][3], acc[3]);
            }
        }
    }
    *reinterpret_cast<f32x4_t *>(y + (int64_t)t * H + r) = acc;
}

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

// Allow up to 160 KB of LDS per workgroup: the dynamic limit is what the kernel's static LDS
// leaves of it.
bool set_lds_attr(const void *fn, size_t total) {
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, fn) != hipSuccess || fa.sharedSizeBytes > total) return false;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)(total - fa.sharedSizeBytes)) == hipSuccess;
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
    prof_start(MOE_KERNEL_COMBINE, s);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, s, w, pos, offsets, E, ypair, k,
                       H, y);
    prof_stop(MOE_KERNEL_COMBINE, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

template <int MT, int GG, int GD>
int launch_decode_mt(const FfnArgs &a, const DecodeWs &d, hipStream_t s) {
    const int32_t P = a.T * a.k;
    const int max_active = (int)std::min<int64_t>(a.E, P);
    const size_t rbh = (size_t)row_bytes(a.H), rbf = (size_t)row_bytes(a.F);
    const size_t gu_lds = kNBuf * 2 * kGuO * rbh + (size_t)MT * a.H * 2;
    const size_t dn_lds = kNBuf * kDnRows * rbf + (size_t)MT * a.F * 4;
    if (gu_lds + sizeof(Meta<MT>) > 160 * 1024 || dn_lds + sizeof(Meta<MT>) > 160 * 1024)
        return MOE_ESHAPE;
    static bool attrs = false;
    if (!attrs) {
        if (!set_lds_attr(reinterpret_cast<const void *>(gu_decode_kernel<MT, GG>), 160 * 1024) ||
            !set_lds_attr(reinterpret_cast<const void *>(dn_decode_kernel<MT, GD>), 160 * 1024))
            return MOE_ELAUNCH;
        attrs = true;
    }
    const int grid_cap = kWgPerCu * kCUs;
    const int gu_tiles = a.F / kGuO, dn_tiles = a.H / kDnRows;
    const int gu_grid = (int)std::min<int64_t>(grid_cap, (int64_t)max_active * gu_tiles);
    const int dn_grid = (int)std::min<int64_t>(grid_cap, (int64_t)max_active * dn_tiles);
    // experts one workgroup's item range can touch must fit its LDS metadata table
    auto max_experts = [&](int tiles, int grid) {
        const int64_t per = ((int64_t)max_active * tiles + grid - 1) / grid;
        return (per - 1) / tiles + 2;
    };
    if (max_experts(gu_tiles, gu_grid) > kMaxMeta || max_experts(dn_tiles, dn_grid) > kMaxMeta)
        return MOE_ESHAPE;
    prof_start(MOE_KERNEL_GU_DECODE, s);
    hipLaunchKernelGGL((gu_decode_kernel<MT, GG>), dim3(gu_grid), dim3(kThreads), gu_lds, s, a.x,
                       a.offsets, a.pair_ids, a.active, a.counts, a.gate.base,
                       a.gate.expert_stride, a.up.base, a.up.expert_stride, a.k, P, a.H, a.F, d.h,
                       d.pos);
    prof_stop(MOE_KERNEL_GU_DECODE, s);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    prof_start(MOE_KERNEL_DN_DECODE, s);
    hipLaunchKernelGGL((dn_decode_kernel<MT, GD>), dim3(dn_grid), dim3(kThreads), dn_lds, s,
                       a.offsets, a.pair_ids, a.active, a.counts, a.down.base,
                       a.down.expert_stride, a.H, a.F, d.h, d.ypair);
    prof_stop(MOE_KERNEL_DN_DECODE, s);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    return launch_combine(a.w, d.pos, a.offsets, a.E, d.ypair, a.T, a.k, a.H, a.y, s);
}

// Compile-time groups per lane for the common widths (gate/up: H/512 in {5, 8}, down: F/128 in
// {5, 10}), else 0 (runtime loop). Two staged token rows per expert only where the unrolled
// kernels stay within 256 VGPRs (two waves per SIMD); elsewhere one.
template <int GG, int GD>
int launch_decode_shape(const FfnArgs &a, const DecodeWs &d, hipStream_t s) {
    if (a.T >= 2) return launch_decode_mt<2, GG, GD>(a, d, s);
    return launch_decode_mt<1, GG, GD>(a, d, s);
}
template <int GG>
int launch_decode_gd(const FfnArgs &a, const DecodeWs &d, hipStream_t s) {
    switch (a.F % 128 ? 0 : a.F / 128) {
    case 5: return launch_decode_shape<GG, 5>(a, d, s);
    case 10: return launch_decode_shape<GG, 10>(a, d, s);
    default: return launch_decode_shape<GG, 0>(a, d, s);
    }
}

int launch_decode(const FfnArgs &a, hipStream_t s) {
    const DecodeWs d = carve(a.ws, a.T * a.k, a.H, a.F);
    switch (a.H % 512 ? 0 : a.H / 512) {
    case 5: return launch_decode_gd<5>(a, d, s);
    case 8: return launch_decode_gd<8>(a, d, s);
    default: return launch_decode_gd<0>(a, d, s);
    }
}

}  // namespace moe
