// Prefill path of the routed NVFP4 FFN: bf16-MFMA grouped GEMM over expert-first CSR tiles.
//
// moe_sk_repro.rs times a prefill MoE layer as three grouped GEMMs (gate, up, down) over the
// expert buckets, in 128-row M tiles; here gate and up share one kernel so the SiLU(g) * u
// epilogue runs on registers, and down is the second kernel.
//
//   schedule:   M tiles of at most kBM consecutive CSR pairs of one expert, listed from the
//               device CSR (no host read-back); also the pair -> CSR slot map for the combine.
//   gu_prefill: one workgroup per (64 output features, M tile). The MFMA A operand is the
//               weights: 64 gate rows and the 64 matching up rows, staged as raw NVFP4 in LDS
//               (four 36-byte blocks per row at a time) and dequantized once per workgroup into
//               a bf16 LDS tile -- exact, since every E2M1 x UE4M3 product is a bf16 value. The
//               B operand is the tile's token rows of x gathered by CSR pair. v_mfma_f32_16x16x32
//               _bf16 with fp32 accumulation; the epilogue forms h = SiLU(g) * u and stores it as
//               a bf16 pair h_hi + h_lo (h_hi = bf16(h), h_lo = bf16(h - h_hi)), which carries
//               h to about 16 significant bits.
//   dn_prefill: one workgroup per (64 down rows, M tile): dequantized W_d tile times h_hi, plus
//               the same tile times h_lo, into the fp32 per-pair rows ypair (row = pair id).
//   combine:    the decode path's ordered fp32 combine.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;               // pairs per M tile
constexpr int kBK = 64;                // K per MFMA sub-step (one NVFP4 block)
constexpr int kPitch = kBK + 8;        // bf16 elements per LDS tile row (144 bytes)
constexpr int kChunkBlocks = 4;        // NVFP4 blocks per raw staging chunk
constexpr int kRawRow = kChunkBlocks * kBlockBytes;  // 144 bytes
constexpr int kGuO = 64;               // output features per gu tile (gate + up = 128 rows)
constexpr int kGuRows = 2 * kGuO;
constexpr int kDnR = 64;               // down rows per dn tile

typedef __attribute__((ext_vector_type(2))) int32_t i32x2_t;

// ------------------------------------------------------------------------------- schedule

__device__ int scan256(int v, int *wsum, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    lds_barrier();
    int before = 0, tot = 0;
    for (int w = 0; w < kThreads / 64; w++) {
        if (w < wave) before += wsum[w];
        tot += wsum[w];
    }
    *total = tot;
    lds_barrier();
    return before + x - v;
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ pair_ids,
    const int32_t *__restrict__ active, const int32_t *__restrict__ counts, int32_t P,
    int32_t max_tiles, i32x2_t *__restrict__ tiles, int32_t *__restrict__ n_tiles,
    int32_t *__restrict__ pos) {
    for (int q = blockIdx.x * kThreads + threadIdx.x; q < P; q += gridDim.x * kThreads)
        pos[pair_ids[q]] = q;
    if (blockIdx.x != 0) return;
    __shared__ int wsum[kThreads / 64];
    const int n_act = counts[0];
    const int per = (n_act + kThreads - 1) / kThreads;
    const int lo = min((int)threadIdx.x * per, n_act), hi = min(lo + per, n_act);
    int mine = 0;
    for (int a = lo; a < hi; a++) {
        const int e = active[a];
        mine += (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
    }
    int total;
    int off = scan256(mine, wsum, &total);
    for (int a = lo; a < hi; a++) {
        const int e = active[a];
        const int m = offsets[e + 1] - offsets[e];
        for (int m0 = 0; m0 < m; m0 += kBM) {
            if (off < max_tiles) tiles[off] = i32x2_t{e, m0};
            off++;
        }
    }
    if (threadIdx.x == 0) n_tiles[0] = min(total, max_tiles);
}

// ------------------------------------------------------------------------ shared helpers

__device__ __forceinline__ bf16x8_t frag(const uint16_t *tile, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(tile + (row0 + (l & 15)) * kPitch + k0 +
                                                         (l >> 4) * 8);
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Dequantize one 16-weight scale group (scale byte `sb`, 8 code bytes c0,c1) to 16 bf16 and store
// them as two 16-byte LDS writes at dst. Exact: each product is a bf16 value.
__device__ __forceinline__ void dequant_group(uint32_t sb, uint32_t c0, uint32_t c1, uint16_t *dst) {
    const float S = ue4m3_to_f32(sb);
    u32x4_t lo, hi;
    f32x2_t v;
    v = e2m1x2_to_f32<0>(c0); lo[0] = pack_bf16(v[0] * S, v[1] * S);
    v = e2m1x2_to_f32<1>(c0); lo[1] = pack_bf16(v[0] * S, v[1] * S);
    v = e2m1x2_to_f32<2>(c0); lo[2] = pack_bf16(v[0] * S, v[1] * S);
    v = e2m1x2_to_f32<3>(c0); lo[3] = pack_bf16(v[0] * S, v[1] * S);
    v = e2m1x2_to_f32<0>(c1); hi[0] = pack_bf16(v[0] * S, v[1] * S);
    v = e2m1x2_to_f32<1>(c1); hi[1] = pack_bf16(v[0] * S, v[1] * S);
    v = e2m1x2_to_f32<2>(c1); hi[2] = pack_bf16(v[0] * S, v[1] * S);
    v = e2m1x2_to_f32<3>(c1); hi[3] = pack_bf16(v[0] * S, v[1] * S);
    reinterpret_cast<u32x4_t *>(dst)[0] = lo;
    reinterpret_cast<u32x4_t *>(dst)[1] = hi;
}

// ----------------------------------------------------------------------------- gate / up

constexpr int kGuRawUnits = kGuRows * kRawRow / 16;            // 1152 16-byte units per chunk
constexpr int kGuRawPerThread = (kGuRawUnits + kThreads - 1) / kThreads;  // 5
constexpr int kActUnits = kBM * kBK * 2 / 16;                  // 1024 units per sub-step
constexpr int kActPerThread = kActUnits / kThreads;            // 4

__global__ __launch_bounds__(kThreads) void gu_prefill_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_ids, const i32x2_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const uint8_t *__restrict__ gate, int64_t gate_stride,
    const uint8_t *__restrict__ up, int64_t up_stride, int32_t k, int32_t H, int32_t F,
    uint16_t *__restrict__ h_hi, uint16_t *__restrict__ h_lo) {
    __shared__ __attribute__((aligned(16))) uint16_t wbf[kGuRows * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t act[kBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t raw[kGuRows * kRawRow];
    __shared__ int tok[kBM];

    const int ti = blockIdx.y;
    if (ti >= n_tiles[0]) return;
    const i32x2_t tl = tiles[ti];
    const int e = tl[0], m0 = tl[1];
    const int q0 = offsets[e] + m0;
    const int mt = min(kBM, offsets[e + 1] - q0);
    const int o0 = blockIdx.x * kGuO;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rb = H / kBlockWeights * kBlockBytes;

    for (int r = tid; r < kBM; r += kThreads) tok[r] = r < mt ? pair_ids[q0 + r] / k : -1;

    const uint8_t *gsrc = gate + e * gate_stride + (int64_t)o0 * rb;
    const uint8_t *usrc = up + e * up_stride + (int64_t)o0 * rb;

    u32x4_t rawr[kGuRawPerThread];
    auto load_raw = [&](int chunk) {
#pragma unroll
        for (int i = 0; i < kGuRawPerThread; i++) {
            const int u = tid + i * kThreads;
            if (u < kGuRawUnits) {
                const int row = u / 9, part = u % 9;
                const uint8_t *src = (row < kGuO ? gsrc + (int64_t)row * rb
                                                 : usrc + (int64_t)(row - kGuO) * rb) +
                                     chunk * kRawRow + part * 16;
                rawr[i] = *reinterpret_cast<const u32x4_t *>(src);
            }
        }
    };
    auto store_raw = [&]() {
#pragma unroll
        for (int i = 0; i < kGuRawPerThread; i++) {
            const int u = tid + i * kThreads;
            if (u < kGuRawUnits) reinterpret_cast<u32x4_t *>(raw)[u] = rawr[i];
        }
    };
    lds_barrier();  // tok visible
    u32x4_t actr[kActPerThread];
    auto load_act = [&](int sub) {
#pragma unroll
        for (int i = 0; i < kActPerThread; i++) {
            const int u = tid + i * kThreads;
            const int row = u >> 3, part = u & 7;
            const int t = tok[row];
            actr[i] = t >= 0 ? *reinterpret_cast<const u32x4_t *>(x + (int64_t)t * H + sub * kBK + part * 8)
                             : u32x4_t{0, 0, 0, 0};
        }
    };
    auto store_act = [&]() {
#pragma unroll
        for (int i = 0; i < kActPerThread; i++) {
            const int u = tid + i * kThreads;
            const int row = u >> 3, part = u & 7;
            *reinterpret_cast<u32x4_t *>(act + row * kPitch + part * 8) = actr[i];
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int wa = wave & 1, wb = wave >> 1;
    const int nsub = H / kBK;
    load_raw(0);
    load_act(0);
    for (int s = 0; s < nsub; s++) {
        lds_barrier();
        if ((s & 3) == 0) store_raw();
        store_act();
        lds_barrier();
        {   // dequantize block (s & 3) of the chunk: thread -> (row, two scale groups)
            const int row = tid >> 1, half = tid & 1;
            const uint8_t *blk = raw + row * kRawRow + (s & 3) * kBlockBytes;
            const uint32_t *b32 = reinterpret_cast<const uint32_t *>(blk);
            const uint32_t scw = b32[0];
            uint16_t *dst = wbf + row * kPitch + half * 32;
            dequant_group((scw >> (16 * half)) & 0xff, b32[1 + 4 * half], b32[2 + 4 * half], dst);
            dequant_group((scw >> (16 * half + 8)) & 0xff, b32[3 + 4 * half], b32[4 + 4 * half],
                          dst + 16);
        }
        if (s + 1 < nsub) load_act(s + 1);
        if ((s & 3) == 3 && s + 1 < nsub) load_raw((s + 1) >> 2);
        lds_barrier();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8_t af[4], bfr[4];
            af[0] = frag(wbf, 32 * wa, kk);
            af[1] = frag(wbf, 32 * wa + 16, kk);
            af[2] = frag(wbf, kGuO + 32 * wa, kk);
            af[3] = frag(wbf, kGuO + 32 * wa + 16, kk);
#pragma unroll
            for (int b = 0; b < 4; b++) bfr[b] = frag(act, 64 * wb + 16 * b, kk);
#pragma unroll
            for (int a = 0; a < 4; a++)
#pragma unroll
                for (int b = 0; b < 4; b++)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
        }
    }

    // epilogue: lane holds C[4*(lane/16)+v][lane%16] of each 16x16 tile (rows = features,
    // columns = pairs); gate tile a pairs with up tile a+2.
#pragma unroll
    for (int a = 0; a < 2; a++) {
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int col = 64 * wb + 16 * b + (lane & 15);
            if (col < mt) {
                const int o = o0 + 32 * wa + 16 * a + 4 * (lane >> 4);
                uint32_t hi2[2], lo2[2];
#pragma unroll
                for (int v = 0; v < 4; v += 2) {
                    const float h0 = silu(acc[a][b][v]) * acc[a + 2][b][v];
                    const float h1 = silu(acc[a][b][v + 1]) * acc[a + 2][b][v + 1];
                    const __bf16 g0 = (__bf16)h0, g1 = (__bf16)h1;
                    hi2[v / 2] = pack_bf16((float)g0, (float)g1);
                    lo2[v / 2] = pack_bf16(h0 - (float)g0, h1 - (float)g1);
                }
                const int64_t off = (int64_t)(q0 + col) * F + o;
                *reinterpret_cast<i32x2_t *>(h_hi + off) = i32x2_t{(int)hi2[0], (int)hi2[1]};
                *reinterpret_cast<i32x2_t *>(h_lo + off) = i32x2_t{(int)lo2[0], (int)lo2[1]};
            }
        }
    }
}

// ---------------------------------------------------------------------------------- down

constexpr int kDnRawDwords = kDnR * kRawRow / 4;                 // 2304 dwords per full chunk
constexpr int kDnRawPerThread = kDnRawDwords / kThreads;          // 9
constexpr int kDnActPerThread = 2 * kActUnits / kThreads;         // 8 (hi and lo)

__global__ __launch_bounds__(kThreads) void dn_prefill_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ pair_ids,
    const i32x2_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const uint8_t *__restrict__ down, int64_t down_stride,
    int32_t H, int32_t F, const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo,
    float *__restrict__ ypair) {
    __shared__ __attribute__((aligned(16))) uint16_t wbf[kDnR * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t ahi[kBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t alo[kBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t raw[kDnR * kRawRow];
    __shared__ int pid[kBM];

    const int ti = blockIdx.y;
    if (ti >= n_tiles[0]) return;
    const i32x2_t tl = tiles[ti];
    const int e = tl[0], m0 = tl[1];
    const int q0 = offsets[e] + m0;
    const int mt = min(kBM, offsets[e + 1] - q0);
    const int r0 = blockIdx.x * kDnR;
    for (int r = threadIdx.x; r < kBM; r += kThreads) pid[r] = r < mt ? pair_ids[q0 + r] : 0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rb = F / kBlockWeights * kBlockBytes;
    const int nblk = F / kBlockWeights;
    const uint8_t *wsrc = down + e * down_stride + (int64_t)r0 * rb;

    uint32_t rawr[kDnRawPerThread];
    auto load_raw = [&](int chunk) {
        const int cb = min(kChunkBlocks, nblk - chunk * kChunkBlocks);
        const int dw_row = cb * 9;
#pragma unroll
        for (int i = 0; i < kDnRawPerThread; i++) {
            const int u = tid + i * kThreads;
            if (u < kDnR * dw_row) {
                const int row = u / dw_row, d = u % dw_row;
                rawr[i] = *reinterpret_cast<const uint32_t *>(wsrc + (int64_t)row * rb +
                                                              chunk * kRawRow + 4 * d);
            }
        }
    };
    auto store_raw = [&](int chunk) {
        const int cb = min(kChunkBlocks, nblk - chunk * kChunkBlocks);
        const int dw_row = cb * 9;
#pragma unroll
        for (int i = 0; i < kDnRawPerThread; i++) {
            const int u = tid + i * kThreads;
            if (u < kDnR * dw_row) {
                const int row = u / dw_row, d = u % dw_row;
                reinterpret_cast<uint32_t *>(raw + row * kRawRow)[d] = rawr[i];
            }
        }
    };
    u32x4_t actr[kDnActPerThread];
    auto load_act = [&](int sub) {
#pragma unroll
        for (int i = 0; i < kDnActPerThread; i++) {
            const int u = tid + (i >> 1) * kThreads;
            const int row = u >> 3, part = u & 7;
            const uint16_t *src = (i & 1) ? h_lo : h_hi;
            actr[i] = row < mt ? *reinterpret_cast<const u32x4_t *>(src + (int64_t)(q0 + row) * F +
                                                                   sub * kBK + part * 8)
                               : u32x4_t{0, 0, 0, 0};
        }
    };
    auto store_act = [&]() {
#pragma unroll
        for (int i = 0; i < kDnActPerThread; i++) {
            const int u = tid + (i >> 1) * kThreads;
            const int row = u >> 3, part = u & 7;
            *reinterpret_cast<u32x4_t *>(((i & 1) ? alo : ahi) + row * kPitch + part * 8) = actr[i];
        }
    };

    f32x4_t acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int wa = wave & 1, wb = wave >> 1;
    const int nsub = nblk;
    load_raw(0);
    load_act(0);
    for (int s = 0; s < nsub; s++) {
        lds_barrier();
        if ((s & 3) == 0) store_raw(s >> 2);
        store_act();
        lds_barrier();
        {   // dequantize block (s & 3) of the chunk: thread -> (row, scale group)
            const int row = tid >> 2, g = tid & 3;
            const uint8_t *blk = raw + row * kRawRow + (s & 3) * kBlockBytes;
            const uint32_t *b32 = reinterpret_cast<const uint32_t *>(blk);
            dequant_group((b32[0] >> (8 * g)) & 0xff, b32[1 + 2 * g], b32[2 + 2 * g],
                          wbf + row * kPitch + 16 * g);
        }
        if (s + 1 < nsub) load_act(s + 1);
        if ((s & 3) == 3 && s + 1 < nsub) load_raw((s + 1) >> 2);
        lds_barrier();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8_t af[2], bh[4], bl[4];
            af[0] = frag(wbf, 32 * wa, kk);
            af[1] = frag(wbf, 32 * wa + 16, kk);
#pragma unroll
            for (int b = 0; b < 4; b++) {
                bh[b] = frag(ahi, 64 * wb + 16 * b, kk);
                bl[b] = frag(alo, 64 * wb + 16 * b, kk);
            }
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bh[b], acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bl[b], acc[a][b], 0, 0, 0);
                }
        }
    }
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int col = 64 * wb + 16 * b + (lane & 15);
            if (col < mt) {
                const int r = r0 + 32 * wa + 16 * a + 4 * (lane >> 4);
                *reinterpret_cast<f32x4_t *>(ypair + (int64_t)pid[col] * H + r) = acc[a][b];
            }
        }
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct PrefillWs {
    int32_t *pos;
    i32x2_t *tiles;
    int32_t *n_tiles;
    uint16_t *h_hi, *h_lo;
    float *ypair;
};

int max_tiles(int32_t P, int32_t E) { return P / kBM + std::min(E, P) + 1; }

PrefillWs carve(void *ws, int32_t P, int32_t E, int32_t H, int32_t F) {
    uint8_t *b = static_cast<uint8_t *>(ws);
    PrefillWs w;
    w.pos = reinterpret_cast<int32_t *>(b);
    b += align256(sizeof(int32_t) * (size_t)P);
    w.tiles = reinterpret_cast<i32x2_t *>(b);
    b += align256(sizeof(i32x2_t) * (size_t)max_tiles(P, E));
    w.n_tiles = reinterpret_cast<int32_t *>(b);
    b += 256;
    w.h_hi = reinterpret_cast<uint16_t *>(b);
    b += align256(2 * (size_t)P * F);
    w.h_lo = reinterpret_cast<uint16_t *>(b);
    b += align256(2 * (size_t)P * F);
    w.ypair = reinterpret_cast<float *>(b);
    return w;
}

}  // namespace

size_t prefill_ws_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F) {
    const int32_t P = T * k;
    return align256(sizeof(int32_t) * (size_t)P) + align256(sizeof(i32x2_t) * (size_t)max_tiles(P, E)) +
           256 + 2 * align256(2 * (size_t)P * F) + align256(sizeof(float) * (size_t)P * H);
}

int launch_prefill(const FfnArgs &a, hipStream_t s) {
    const int32_t P = a.T * a.k;
    const PrefillWs w = carve(a.ws, P, a.E, a.H, a.F);
    const int mt = max_tiles(P, a.E);
    const int sched_blocks = std::max(1, std::min(256, (P + kThreads - 1) / kThreads));
    prof_start(MOE_KERNEL_SCHEDULE, s);
    hipLaunchKernelGGL(schedule_kernel, dim3(sched_blocks), dim3(kThreads), 0, s, a.offsets,
                       a.pair_ids, a.active, a.counts, P, mt, w.tiles, w.n_tiles, w.pos);
    prof_stop(MOE_KERNEL_SCHEDULE, s);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    if (a.F % kGuO || a.H % kDnR) return MOE_ESHAPE;
    prof_start(MOE_KERNEL_GU_PREFILL, s);
    hipLaunchKernelGGL(gu_prefill_kernel, dim3(a.F / kGuO, mt), dim3(kThreads), 0, s, a.x,
                       a.offsets, a.pair_ids, w.tiles, w.n_tiles, a.gate.base,
                       a.gate.expert_stride, a.up.base, a.up.expert_stride, a.k, a.H, a.F, w.h_hi,
                       w.h_lo);
    prof_stop(MOE_KERNEL_GU_PREFILL, s);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    prof_start(MOE_KERNEL_DN_PREFILL, s);
    hipLaunchKernelGGL(dn_prefill_kernel, dim3(a.H / kDnR, mt), dim3(kThreads), 0, s, a.offsets,
                       a.pair_ids, w.tiles, w.n_tiles, a.down.base, a.down.expert_stride, a.H, a.F, w.h_hi,
                       w.h_lo, w.ypair);
    prof_stop(MOE_KERNEL_DN_PREFILL, s);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    return launch_combine(a.w, w.pos, a.offsets, a.E, w.ypair, a.T, a.k, a.H, a.y, s);
}

}  // namespace moe
