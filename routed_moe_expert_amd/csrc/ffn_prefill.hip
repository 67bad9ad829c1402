// Prefill path of the routed NVFP4 FFN: grouped GEMMs over expert-first CSR tiles on f16 MFMA.
//
// moe_sk_repro.rs times a prefill MoE layer as three grouped GEMMs (gate, up, down) over the
// expert buckets, in 128-row M tiles; here gate and up share one kernel so the SiLU(g) * u
// epilogue runs on registers, and down is the second kernel.
//
//   schedule: M tiles of at most kBM consecutive CSR pairs of one expert, listed from the
//             device CSR (no host read-back); also the pair -> CSR slot map for the combine.
//   xcast:    x to f16 per token row, scaled by a power of two (exact), for the gate/up GEMM.
//   gemm:     one workgroup per (N tile, M tile); gate/up: 8 waves, 512 weight rows, one
//             workgroup per CU (or 4 waves, 256 rows, two per CU where ff is not a multiple of
//             256); down: 4 waves, 256 rows, two workgroups per CU, which
//             fall out of step with each other, so that one computes while the other waits
//             at its barrier or for its loads (down GEMM 5-7% faster than one 8-wave
//             workgroup with three stages). The A operand is the
//             weights, staged raw in LDS one NVFP4 block per row per K step; every wave
//             decodes its own 64 rows straight into f16 MFMA fragments in registers -- exact,
//             since every E2M1 x UE4M3 product is an f16 value. The B operand is the M tile's
//             token rows (x gathered by token for gate/up, the h_hi / h_lo rows of the CSR
//             slots for down) with an XOR swizzle of their 16-byte parts so that fragment reads
//             are free of bank conflicts. From row-major banks gate/up keeps two K steps in
//             flight (three LDS stages), each down workgroup one (two stages); from K-step-packed
//             copies (36 bytes a row in LDS) one more each.
//             MFMA 16x16x32 with fp32 accumulation; a wave owns 64 rows x 128
//             tokens (gate/up) or 64 rows x 64 tokens (down, whose workgroups take half an M
//             tile so that h_hi and h_lo fit the stages) and runs only the steps of 32
//             (gate/up) or 16 (down) token columns that the tile reaches. Each weight row is
//             decoded by one wave only, and each B fragment read from LDS feeds four MFMAs: per
//             K step the LDS reads of a workgroup (the B tile once per wave) stay below what
//             the matrix cores take to consume them, which at 32 rows per wave they did not.
//             Both multiply in f16 (v_mfma_f32_16x16x32_f16: weights decoded to f16 at half
//             the VALU of bf16, which has no packed multiply). Gate/up takes x cast per token
//             (exact, power-of-two scaled) and unscales its sums per token column.
//             Gate/up: rows are the tile's gate rows and the matching up rows; the epilogue forms
//             h = SiLU(g) * u and stores it as an f16 pair, h = 2^s (h_hi + h_lo) with one
//             power-of-two s per (pair, h segment of 256 features, or 128 where ff is not a
//             multiple of 256) bringing their largest |h| into
//             [2^14, 2^15) (about 22 significant bits). Down: the same tile times h_hi plus times
//             h_lo, K segment by K segment: at each new segment the running fp32 sums are
//             rescaled to its exponent (exact), and the epilogue applies the last one; into the
//             fp32 per-pair rows ypair.
//   combine:  the decode path's ordered fp32 combine.
//
// Workgroups are mapped XCD-aware (hardware workgroup b runs on XCD b mod 8): M tile t runs on
// XCD t mod 8, the N tiles of an M tile -- which share its token rows -- back to back there.
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreadsSched = 256;
constexpr int kBM = 128;               // pairs per M tile
constexpr int kCF = kBM / 16;          // token column tiles per M tile
constexpr int kBRow = 64 * 2;          // bytes of one token row per K step (64 f16)
constexpr int kBBytes = kBM * kBRow;   // 16 KB per B operand per stage (128 tokens)
constexpr int kRowsW = 64;            // A rows per wave

// gate/up: 8 waves (256 features per N tile), one workgroup per CU, three LDS stages (two K
// steps in flight), four from K-step-packed copies (DENSE: rows staged at 36 bytes instead of
// 48); or, from packed copies when ff is not a multiple of 256, 4 waves (128 features) with two
// workgroups per CU and three stages, so that no N tile is half empty (ff 640: 5 tiles of 128
// instead of 3 of 256). Down: 4 waves, two workgroups per CU, two stages (one step in flight per
// workgroup while the other workgroup of the CU computes), three from packed copies.
template <bool DOWN, bool DENSE, int WAVES> constexpr int gemm_stages() {
    return DOWN ? (DENSE ? 3 : 2) : (DENSE ? (WAVES == 8 ? 4 : 3) : 3);
}
template <bool DENSE> constexpr int gemm_a_pitch() { return DENSE ? 36 : 48; }
// h is scaled per (pair, segment): a segment is the features of one gate/up N tile
template <int WAVES> constexpr int gate_up_segment() { return kRowsW / 2 * WAVES; }
constexpr int kMaxSeg = 32;           // h scale segments per pair (ff <= 32 segments)

typedef __attribute__((ext_vector_type(2))) int32_t i32x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

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
    for (int w = 0; w < kThreadsSched / 64; w++) {
        if (w < wave) before += wsum[w];
        tot += wsum[w];
    }
    *total = tot;
    lds_barrier();
    return before + x - v;
}

__global__ __launch_bounds__(kThreadsSched) void schedule_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ pair_ids,
    const int32_t *__restrict__ active, const int32_t *__restrict__ counts, int32_t P,
    int32_t max_tiles, i32x2_t *__restrict__ tiles, int32_t *__restrict__ n_tiles,
    int32_t *__restrict__ pos) {
    for (int q = blockIdx.x * kThreadsSched + threadIdx.x; q < P; q += gridDim.x * kThreadsSched)
        pos[pair_ids[q]] = q;
    if (blockIdx.x != 0) return;
    __shared__ int wsum[kThreadsSched / 64];
    const int n_act = counts[0];
    const int per = (n_act + kThreadsSched - 1) / kThreadsSched;
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

// ------------------------------------------------------------------------------ x to f16

constexpr int kCastThreads = 256;

// Token row t of x (bf16) -> f16 scaled by 2^-xs[t], xs[t] chosen so that the row's largest
// magnitude lands in [2^14, 2^15): exact for every value within 2^28 of that maximum (bf16 has 8
// significant bits, f16 11; values further down go subnormal and keep fewer), so the gate/up
// GEMM can run on f16 MFMA and unscale its fp32 sums per token column.
__global__ __launch_bounds__(kCastThreads) void xcast_kernel(const uint16_t *__restrict__ x,
                                                            int32_t H, uint16_t *__restrict__ x16,
                                                            int32_t *__restrict__ xs) {
    __shared__ uint32_t wmax[kCastThreads / 64];
    const int t = blockIdx.x, tid = threadIdx.x;
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + (int64_t)t * H);
    const int n8 = H / 8;   // 8 bf16 per 16-byte part
    // the row is read once: a thread's parts stay in registers (H <= MOE_MAX_HIDDEN)
    constexpr int kParts = MOE_MAX_HIDDEN / 8 / kCastThreads;
    u32x4_t part[kParts];
    uint32_t amax = 0;      // |x| as bf16 bits: ordered like the magnitudes for finite values
#pragma unroll
    for (int u = 0; u < kParts; u++) {
        const int i = tid + u * kCastThreads;
        part[u] = i < n8 ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; j++)
            amax = max(amax, max(part[u][j] & 0x7fffu, (part[u][j] >> 16) & 0x7fffu));
    }
    for (int d = 32; d > 0; d >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, d, 64));
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = wmax[0];
    for (int w = 1; w < kCastThreads / 64; w++) amax = max(amax, wmax[w]);
    const float mx = __uint_as_float(amax << 16);
    int e = 0;
    if (mx > 0.f) (void)frexpf(mx, &e);   // mx = f * 2^e, f in [0.5, 1)
    const int sc = mx > 0.f ? e - 15 : 0;
    const float inv = ldexpf(1.0f, -sc);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(x16 + (int64_t)t * H);
#pragma unroll
    for (int u = 0; u < kParts; u++) {
        const int i = tid + u * kCastThreads;
        if (i >= n8) break;
        const u32x4_t v = part[u];
        u32x4_t o;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const f16x2_t h2 = {(_Float16)(__uint_as_float(v[j] << 16) * inv),
                                (_Float16)(__uint_as_float(v[j] & 0xffff0000u) * inv)};
            o[j] = __builtin_bit_cast(uint32_t, h2);
        }
        dst[i] = o;
    }
    if (tid == 0) xs[t] = sc;
}

// ------------------------------------------------------------------------------- gemm

// 8 E2M1 codes times the group scale -> 8 f16, exact (every E2M1 x UE4M3 product is an f16
// value). The converts scale by 2^8 (their scale operand contributes its exponent only); the
// UE4M3 byte shifted into the f16 exponent and mantissa fields reads as 2^-8 times its value,
// for normal and subnormal bytes alike. Half the VALU of the bf16 route, which has no packed
// multiply.
__device__ __forceinline__ f16x8_t dequant8_f16(uint32_t c, uint32_t scale_byte) {
    const _Float16 s = __builtin_bit_cast(f16x2_t, scale_byte << 7)[0];
    const f16x2_t S = {s, s};
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 0) * S;
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 1) * S;
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 2) * S;
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 3) * S;
    return __builtin_bit_cast(f16x8_t, u32x4_t{__builtin_bit_cast(uint32_t, p0),
                                               __builtin_bit_cast(uint32_t, p1),
                                               __builtin_bit_cast(uint32_t, p2),
                                               __builtin_bit_cast(uint32_t, p3)});
}

// Target builtins stay inside __device__ helpers: used directly in a kernel template they make
// its host-side instantiation fail, and the launch stub goes missing.
__device__ __forceinline__ f32x4_t mfma_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 4, 0, 0);
}
__device__ __forceinline__ void dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 16, 0, 0);
}
// 12 bytes per lane; lane i lands at LDS + 16 i (the last 4 bytes of its slot are untouched)
__device__ __forceinline__ void dma12(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 12, 0, 0);
}

// LDS offset of byte b (0..35) of an NVFP4 block staged as three 12-byte loads in 16-byte slots
__host__ __device__ constexpr int blk_lds(int b) { return 16 * (b / 12) + b % 12; }


// LDS slot (16-byte unit) of part p (8 f16) of token row r of a B stage. The LDS serves a
// 16-byte read for 16 lanes at a time from 64 banks (256 bytes): the 16 lanes of a fragment read
// (rows r .. r + 15, one part) must fall on 16 different 16-byte bank groups, i.e. distinct slots
// mod 16. Rows alternate between the two halves of the 256 bytes (r * 8 mod 16), so the XOR key
// is r / 2: the 8 rows of each parity then take 8 distinct parts' places.
__device__ __forceinline__ int b_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int b_slot(int r, int p) { return r * 8 + (p ^ b_swz(r)); }

// One workgroup: N tile nt of M tile ti (gate/up: 64 weight rows per wave, half gate rows and
// half the matching up rows, over all of the tile's up to 128 pairs; down: 256 rows, the half hf
// of 64 pairs). DOWN = false: gate/up (A rows are the tile's gate rows then its up rows; K = H;
// B = x rows by token); DOWN = true: down (A rows are 256 rows of W_d; K = F; B = h_hi and h_lo
// rows by CSR slot, with their scale exponents per SEGF-feature segment). N tiles may run past
// the matrix: rows beyond it are zero (packed copies) or read the last row (row-major banks), and
// are not stored.
//
// Each K step of 64 stages one NVFP4 block of every A row and the B rows in one of kStages LDS
// stages: kStages - 1 steps are in flight while one is computed, which (at two waves per SIMD and
// up to 64 MFMAs per wave per step) covers the latency of these loads. A row's block arrives by
// three 12-byte direct-to-LDS loads (lane i of a load lands at +16 i, so a row takes 48 bytes of
// LDS), or, with DENSE (from K-step-packed copies, whose K step is one contiguous run per bank),
// by 16-byte loads of the run as it is: 36 bytes a row, in the order the waves read their A
// fragments, which frees LDS for another stage. Each wave issues a fixed number of loads per
// step, so its count of outstanding loads is exact and the waits are partial.
template <bool DOWN, bool DENSE, int WAVES, int SEGF>
__global__ __launch_bounds__(WAVES * 64, WAVES == 8 ? 1 : 2) void gemm_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ hin_hi,
    const uint16_t *__restrict__ hin_lo, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_ids, const i32x2_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, int32_t max_tiles, int32_t n_ntiles,
    const uint8_t *__restrict__ w0, int64_t s0, const uint8_t *const *__restrict__ t0,
    const uint8_t *__restrict__ w1, int64_t s1, const uint8_t *const *__restrict__ t1,
    const uint8_t *__restrict__ kp0, const uint8_t *__restrict__ kp1,
    const float *__restrict__ w0_s2, const float *__restrict__ w1_s2,
    int32_t k, int32_t K, int32_t F, int32_t H, const int32_t *__restrict__ xs,
    uint16_t *__restrict__ h_hi, uint16_t *__restrict__ h_lo, int32_t *__restrict__ hs,
    float *__restrict__ ypair) {
    constexpr int segf = SEGF;   // features per h scale segment
    static_assert(!DOWN || WAVES == 4, "the down GEMM runs 4-wave workgroups");
    constexpr int kThreads = WAVES * 64;
    constexpr int kStages = gemm_stages<DOWN, DENSE, WAVES>();
    constexpr int kWaves = kThreads / 64;
    constexpr int kRows = kRowsW * kWaves;          // A rows per workgroup
    constexpr int kPitch = gemm_a_pitch<DENSE>();   // LDS bytes per A row
    // A load units per step: 12-byte pieces (3 per row), or 16-byte pieces of the two runs
    constexpr int kAUnits = DENSE ? kRows * kBlockBytes / 16 : kRows * 3;
    constexpr int kABytes = kRows * kPitch;
    constexpr int kNB = DOWN ? 2 : 1;               // B operands (h_hi, h_lo) or (x)
    constexpr int kBM2 = DOWN ? kBM / 2 : kBM;      // token columns per workgroup
    constexpr int kCols = kBM2 / 16;
    constexpr int kBBytesW = kBM2 * kBRow;
    constexpr int kStageBytes = kABytes + kNB * kBBytesW;
    constexpr int kBUnits = kBBytesW / 16 / kThreads;    // 16-byte B loads per lane per operand
    constexpr int kALoadsMax = (kAUnits + kThreads - 1) / kThreads;   // 3
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int rowid[kBM2];               // token (gate/up) or CSR slot (down) of each column
    __shared__ int16_t hsc[DOWN ? kBM2 : 1][DOWN ? kMaxSeg : 1];   // down: h scale exponents

    // M tile ti runs on XCD ti mod 8 (hardware workgroup b runs on XCD b mod 8), its N tiles (and
    // halves) in consecutive slots there: they share its token rows in that XCD's L2, and the
    // tiles that exist (the schedule's count is only known on the device) spread evenly over the
    // XCDs whatever the count
    const int nh = DOWN ? 2 : 1;
    const int pos = blockIdx.x >> 3;
    const int ti = (pos / (n_ntiles * nh)) * 8 + (blockIdx.x & 7), rem = pos % (n_ntiles * nh);
    const int nt = rem / nh, hf = rem % nh;
    if (ti >= n_tiles[0]) return;
    const i32x2_t tl = tiles[ti];
    const int e = tl[0], m0 = tl[1] + hf * kBM2;
    const int q0 = offsets[e] + m0;
    const int mt = min(kBM2, offsets[e + 1] - q0);
    if (mt <= 0) return;
    // the expert's second-level scales of bank 0 (gate or down) and bank 1 (up): 1 if none
    const float sc0 = w0_s2 ? w0_s2[e] : 1.f, sc1 = w1_s2 ? w1_s2[e] : 1.f;
    // the expert's first row in bank 0 and bank 1: from a per-expert pointer table, else strided
    const uint8_t *e0 = t0 ? t0[e] : w0 + e * s0;
    const uint8_t *e1 = DOWN ? nullptr : t1 ? t1[e] : w1 + e * s1;
    const int ncol = (mt + 15) >> 4;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int nblk = K / kBlockWeights;
    const int rb = nblk * kBlockBytes;
    const int n_out = DOWN ? H : F;                  // rows (down) or features (gate/up)

    for (int r = tid; r < kBM2; r += kThreads) {
        const int c = r < mt ? r : 0;
        rowid[r] = DOWN ? q0 + c : pair_ids[q0 + c] / k;
    }
    // h scale segments of a pair's row (segf: features per segment, the gate/up N tile's width
    // or half of it)
    const int nseg = (F + segf - 1) / segf;
    if constexpr (DOWN)
        for (int i = tid; i < kBM2 * nseg; i += kThreads) {
            const int r = i / nseg, g = i - r * nseg;
            hsc[r][g] = (int16_t)hs[(int64_t)(q0 + (r < mt ? r : 0)) * nseg + g];
        }
    lds_barrier();

    // A: load i of a wave covers units (i*kWaves + wave)*64 + lane (unit j = u % 3 of row
    // u / 3); loads whose units all lie past kAUnits are skipped by the whole wave. From a
    // K-step-packed copy (kp0, kp1) a bank's N tile lies in one row group, and its K step b is one
    // run of 36-byte blocks (rows past the matrix are zero there); from the row-major bank each
    // row's block sits at the row's start plus 36 b (rows past the matrix read the last).
    constexpr int kTileRows = DOWN ? kRows : kRows / 2;   // rows of one bank in the N tile
    static_assert(kKpackRows % kTileRows == 0 && (DENSE || kTileRows == kKpackRows),
                  "an N tile lies in one packed row group");
    constexpr int kRunUnits = kTileRows * kBlockBytes / 16;   // 16-byte units of one run
    // the dense loads of a wave read one run (a wave-uniform base plus 16 bytes per lane) unless
    // a wave's 64 units straddle the gate and up runs (4-wave gate/up: 288 units per run)
    constexpr bool kUniform = DOWN || kRunUnits % 64 == 0;
    // DENSE reads K-step-packed copies (kp0, kp1), the other form the row-major banks
    const int64_t astep = DENSE ? (int64_t)kKpackRows * kBlockBytes : kBlockBytes;
    const int64_t epack = kpack_expert_bytes(n_out, K);
    const uint8_t *asrc[kALoadsMax];
    int adst[kALoadsMax];   // LDS offset of the wave's load i within a stage
    if constexpr (DENSE) {
        // units u < kRunUnits are the gate run of the step (or down's one run), the rest the up
        // run; a wave's last load past kAUnits repeats its first (same bytes to the same place),
        // so that every wave issues kALoadsMax loads
        static_assert(kAUnits > (kALoadsMax - 1) * kThreads, "");
        const int64_t run = e * epack + (int64_t)(nt * kTileRows / kKpackRows) * nblk * astep +
                            (int64_t)(nt * kTileRows % kKpackRows) * kBlockBytes;
#pragma unroll
        for (int i = 0; i < kALoadsMax; i++) {
            int u0 = (i * kWaves + wave) * 64;
            if (u0 >= kAUnits) u0 = wave * 64;
            adst[i] = u0 * 16;
            const int u = kUniform ? u0 : u0 + lane;
            asrc[i] = DOWN || u < kRunUnits ? kp0 + run + 16 * u
                                            : kp1 + run + 16 * (u - kRunUnits);
        }
    } else
#pragma unroll
    for (int i = 0; i < kALoadsMax; i++) {
        adst[i] = (i * kWaves + wave) * 1024;
        const int u = min((i * kWaves + wave) * 64 + lane, kAUnits - 1);
        const int row = u / 3;
        const int half = DOWN ? kRows : kRows / 2;   // gate/up: gate rows, then the up rows
        const bool second = !DOWN && row >= half;
        const int r = second ? row - half : row;     // row within the bank's N tile
        const uint8_t *base = (second ? e1 : e0) + (int64_t)min(nt * half + r, n_out - 1) * rb;
        asrc[i] = base + 12 * (u % 3);
    }
    static_assert(DENSE || kAUnits == kALoadsMax * kThreads,
                  "every lane issues kALoadsMax A loads");
    // B: lane loads 16-byte units u = (i*kWaves + wave)*64 + lane of each operand, i.e. rows
    // 8 (i*kWaves + wave) .. +7 of the tile. Rows past the tile (r >= mt) load the row of the
    // tile's first pair (rowid clamps them; their columns are never stored), so every wave issues
    // the same kLoads loads at every step and its waits are compile-time counts.
    const uint16_t *bsrc[kNB][kBUnits];
#pragma unroll
    for (int i = 0; i < kBUnits; i++) {
        const int u = (i * kWaves + wave) * 64 + lane;
        const int r = u >> 3, p = (u & 7) ^ b_swz(r);
        const int64_t off = (int64_t)rowid[r] * (DOWN ? F : H) + 8 * p;
        if (DOWN) {
            bsrc[0][i] = hin_hi + off;
            bsrc[kNB - 1][i] = hin_lo + off;
        } else {
            bsrc[0][i] = x + off;
        }
    }
    // load li of step kb into the stage at LDS offset soff (that of step kb mod kStages): the A
    // loads, then the B loads of each operand
    constexpr int kLoads = kALoadsMax + kNB * kBUnits;
    static_assert((kStages - 2) * kLoads <= 15, "waits below encode vmcnt in 4 bits");
    auto issue_one = [&](int kb, int li, int soff) {
        uint8_t *st = smem + soff;
        if (li < kALoadsMax) {
            if constexpr (DENSE && kUniform)
                dma16(asrc[li] + (uint32_t)(16 * lane + kb * astep), st + adst[li]);
            else if constexpr (DENSE)
                dma16(asrc[li] + kb * astep, st + adst[li]);
            else
                dma12(asrc[li] + kb * astep, st + adst[li]);
        } else {
            const int o = (li - kALoadsMax) / kBUnits, i = (li - kALoadsMax) % kBUnits;
            dma16(bsrc[o][i] + kb * 64, st + kABytes + o * kBBytesW + (i * kWaves + wave) * 1024);
        }
    };

    // operands are f16: weights decoded to f16; x cast per token by xcast_kernel (gate/up), h as
    // f16 hi + lo scaled per (pair, 256-feature segment) by the gate/up epilogue (down)
    using BT = f16x8_t;
    constexpr int kAT0 = kRowsW / 16;
    f32x4_t acc[kAT0][kCols];
#pragma unroll
    for (int f = 0; f < kAT0; f++)
#pragma unroll
        for (int c = 0; c < kCols; c++) acc[f][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // this wave's two 16-row A tiles: DOWN: rows 32*wave + 16f; gate/up: gate rows 16*wave
    // (f = 0) and the matching up rows (f = 1)
    // this wave's four 16-row A tiles: DOWN: rows 64 wave + 16 f; gate/up: gate rows
    // 32 wave + 16 f (f = 0, 1) and the matching up rows (f = 2, 3)
    constexpr int kAT = kRowsW / 16;
    int arow[kAT];
#pragma unroll
    for (int f = 0; f < kAT; f++)
        arow[f] = DOWN ? kRowsW * wave + 16 * f
                       : (f >= 2 ? kRows / 2 : 0) + (kRowsW / 2) * wave + 16 * (f & 1);
    // row-major stage: this lane's scale byte and code dwords within a staged block (12-byte
    // loads, 16 apart)
    const int c0_off = blk_lds(4 + 8 * q), c1_off = blk_lds(8 + 8 * q);
    // DENSE: the stage holds packed runs in fragment order; the LDS offsets of this wave's two
    // 32-row slices (gate/up: its gate rows' slice, then its up rows' in the up run; down: its 64
    // rows' two slices)
    int aslice[2];
    aslice[0] = DOWN ? 2 * wave * kSliceBytes : wave * kSliceBytes;
    aslice[1] = DOWN ? (2 * wave + 1) * kSliceBytes : kTileRows * kBlockBytes + wave * kSliceBytes;
    // the codes of a K step read up front (down, 4-wave gate/up) or per sub-step (8-wave gate/up,
    // 6% faster there; up front is 4-5% faster in the other two)
    constexpr bool kCodesFirst = DOWN || WAVES == 4;
    constexpr bool kLoadsFirst = DOWN;   // where a step's refill loads go (below)

    const int nsteps = nblk;
    for (int kb = 0; kb < min(kStages - 1, nsteps); kb++)
#pragma unroll
        for (int li = 0; li < kLoads; li++) issue_one(kb, li, kb * kStageBytes);
    // The K loop for each count of token column tiles a tile can need (gate/up: 2, 4, 6 or 8 of
    // 16 columns; down: 2 or 4), one entered per workgroup: a choice per K step made the compiler
    // copy the gate/up accumulators between the cases' registers, 64 moves a step
    auto k_loop = [&](auto cols) {
        // LDS offset of step kb's stage, stepped without a division (with kb % kStages the
        // compiler spent two VALU adds per LDS address and step)
        int cur = 0;
        for (int kb = 0; kb < nsteps; kb++) {
            if constexpr (DOWN) {
                // a new h segment (its own scale exponent per column): rescale the running sums to
                // it, exactly (powers of two)
                constexpr int seg_steps = segf / kBlockWeights;
                const int g = kb / seg_steps;
                if (g > 0 && kb == g * seg_steps) {
#pragma unroll
                    for (int c = 0; c < kCols; c++) {
                        const int d = hsc[16 * c + n][g - 1] - hsc[16 * c + n][g];
#pragma unroll
                        for (int f = 0; f < kAT0; f++)
#pragma unroll
                            for (int v = 0; v < 4; v++) acc[f][c][v] = ldexpf(acc[f][c][v], d);
                    }
                }
            }
            // step kb landed: at most the loads of the kStages - 2 steps after it still outstanding
            // (s_waitcnt vmcnt(n))
            if (kStages == 4 && kb + 2 < nsteps)
                __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kLoads));
            else if (kStages >= 3 && kb + 1 < nsteps)
                __builtin_amdgcn_s_waitcnt(0x0F70 | kLoads);
            else
                __builtin_amdgcn_s_waitcnt(0x0F70);
            lds_barrier();   // visible to all; the stage of step kb-1 is free
            // step kb + kStages - 1's loads go into that stage: in gate/up one after each of the
            // first kLoads of the step's eight MFMA groups (a wave stalled on a full memory queue
            // then still has MFMAs in flight; measured 3% faster than issuing them together), in
            // down all of them before the step's MFMAs (measured 1-3% faster there)
            const bool refill = kb + kStages - 1 < nsteps;
            const uint8_t *st = smem + cur;
            // the stage of step kb + kStages - 1 (that of step kb - 1)
            const int prev = cur == 0 ? (kStages - 1) * kStageBytes : cur - kStageBytes;
            // One K step in two sub-steps of 32, over the column tiles the tile reaches.
            auto step = [&](auto cols) {
                constexpr int kC = decltype(cols)::value;
                uint32_t sb[kAT], cw[kAT][2];
                if constexpr (DENSE) {
                    // per 32-row slice the scale bytes of its two tiles, and (kCodesFirst) both
                    // tiles' codes, 8 bytes a lane; otherwise the codes are read per sub-step
                    // below. Measured fastest of the combinations of 1- or 2-byte scale reads and
                    // 4- or 8-byte code reads.
                    static_assert(kAT == 4, "two slices of two tiles per wave");
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const uint8_t *sl = st + aslice[j];
                        if constexpr (DOWN) {
                            sb[2 * j] = sl[1024 + 2 * lane];
                            sb[2 * j + 1] = sl[1025 + 2 * lane];
                        } else {
                            const uint32_t two =
                                *reinterpret_cast<const uint16_t *>(sl + 1024 + 2 * lane);
                            sb[2 * j] = two & 0xFF;
                            sb[2 * j + 1] = two >> 8;
                        }
                        if constexpr (kCodesFirst)
#pragma unroll
                            for (int t = 0; t < 2; t++) {
                                const i32x2_t c = *reinterpret_cast<const i32x2_t *>(
                                    sl + 512 * t + 8 * lane);
                                cw[2 * j + t][0] = (uint32_t)c[0];
                                cw[2 * j + t][1] = (uint32_t)c[1];
                            }
                    }
                } else {
#pragma unroll
                    for (int f = 0; f < kAT; f++) {
                        const uint8_t *blk = st + (arow[f] + n) * kPitch;
                        sb[f] = blk[q];
                        cw[f][0] = *reinterpret_cast<const uint32_t *>(blk + c0_off);
                        cw[f][1] = *reinterpret_cast<const uint32_t *>(blk + c1_off);
                    }
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; s2++) {
                    BT bfr[kNB][kC];
#pragma unroll
                    for (int o = 0; o < kNB; o++)
#pragma unroll
                        for (int c = 0; c < kC; c++)
                            bfr[o][c] = *reinterpret_cast<const BT *>(
                                st + kABytes + o * kBBytesW + 16 * b_slot(16 * c + n, 2 * q + s2));
                    // A: lane (n, q) takes scale group q of its row: sub-step s2 = weights
                    // 16q + 8 s2 .. +7
#pragma unroll
                    for (int f = 0; f < kAT; f++) {
                        uint32_t cv;
                        if constexpr (DENSE && !kCodesFirst)
                            cv = *reinterpret_cast<const uint32_t *>(
                                st + aslice[f >> 1] + 512 * (f & 1) + 8 * lane + 4 * s2);
                        else
                            cv = cw[f][s2];
                        const f16x8_t af = dequant8_f16(cv, sb[f]);
#pragma unroll
                        for (int o = 0; o < kNB; o++)
#pragma unroll
                            for (int c = 0; c < kC; c++)
                                acc[f][c] = mfma_f16(af, bfr[o][c], acc[f][c]);
                        const int li = s2 * kAT + f;   // MFMA group index, compile-time
                        if (!kLoadsFirst && li < kLoads && refill) {
                            __builtin_amdgcn_sched_barrier(0);   // keep the load at this point
                            issue_one(kb + kStages - 1, li, prev);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            };
            if (kLoadsFirst && refill)
#pragma unroll
                for (int li = 0; li < kLoads; li++) issue_one(kb + kStages - 1, li, prev);
            step(cols);
            cur = cur == (kStages - 1) * kStageBytes ? 0 : cur + kStageBytes;
        }
    };
    using std::integral_constant;
    if (ncol > 3 * kCols / 4)
        k_loop(integral_constant<int, kCols>{});
    else if (ncol > kCols / 2 && kCols % 4 == 0)
        k_loop(integral_constant<int, 3 * kCols / 4>{});
    else if (ncol > kCols / 4 || kCols % 4 != 0)
        k_loop(integral_constant<int, kCols / 2>{});
    else
        k_loop(integral_constant<int, kCols / 4>{});

    // epilogue: lane holds rows 4q..4q+3 of each 16-row A tile for token column 16c + n
    if (DOWN) {
#pragma unroll
        for (int c = 0; c < kCols; c++) {
            const int col = 16 * c + n;
            if (col < mt) {
                const int64_t prow = (int64_t)pair_ids[q0 + col] * H;
                const int sl = hsc[col][nseg - 1];   // the last segment's scale exponent
#pragma unroll
                for (int f = 0; f < kAT; f++) {
                    const int r = nt * kRows + arow[f] + 4 * q;
                    const f32x4_t y4 = {
                        ldexpf(acc[f][c][0], sl) * sc0, ldexpf(acc[f][c][1], sl) * sc0,
                        ldexpf(acc[f][c][2], sl) * sc0, ldexpf(acc[f][c][3], sl) * sc0};
                    if (r < H) *reinterpret_cast<f32x4_t *>(ypair + prow + r) = y4;
                }
            }
        }
    } else {
        // h = SiLU(g) * u for this lane's 2 x 4 features of each token column (features past ff
        // count as 0), then one power-of-two scale per (pair, this tile's 256 features): the
        // largest |h| over the tile into [2^14, 2^15), so h = 2^s (hi + lo) with hi and lo f16
        // (about 22 significant bits)
        // (h is formed once, into the gate accumulators, whose sums it no longer needs)
        auto hval = [&](int t, int c, int v, int sc) {
            const int o = nt * (kRows / 2) + (kRowsW / 2) * wave + 16 * t + 4 * q + v;
            const float g = ldexpf(acc[t][c][v], sc) * sc0, u = ldexpf(acc[2 + t][c][v], sc) * sc1;
            return o < F ? silu(g) * u : 0.f;
        };
        float *cmax = reinterpret_cast<float *>(smem);   // [kWaves][kBM]: stages are done
#pragma unroll
        for (int c = 0; c < kCols; c++) {
            const int sc = xs[rowid[16 * c + n]];   // the token row's f16 scale exponent
#pragma unroll
            for (int t = 0; t < 2; t++)
#pragma unroll
                for (int v = 0; v < 4; v++) acc[t][c][v] = hval(t, c, v, sc);
        }
        lds_barrier();   // every wave is past its last read of the stages
#pragma unroll
        for (int c = 0; c < kCols; c++) {
            float m = 0.f;
#pragma unroll
            for (int t = 0; t < 2; t++)
#pragma unroll
                for (int v = 0; v < 4; v++) m = fmaxf(m, fabsf(acc[t][c][v]));
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (q == 0) cmax[wave * kBM + 16 * c + n] = m;
        }
        lds_barrier();
        // this wave's h segment: segf / 32 waves (32 features each) per segment, the tile's
        // segments in order (segf is the tile's width, or half of it with the 8-wave kernel
        // when ff is not a multiple of 256)
        constexpr int wps = segf / (kRowsW / 2);
        const int w0 = wave / wps * wps;
        const int seg = nt * (kRows / 2 / segf) + wave / wps;
#pragma unroll
        for (int c = 0; c < kCols; c++) {
            const int col = 16 * c + n;
            float m = 0.f;
            for (int w = w0; w < w0 + wps; w++) m = fmaxf(m, cmax[w * kBM + col]);
            int e = 0;
            if (m > 0.f) (void)frexpf(m, &e);   // m = f * 2^e, f in [0.5, 1)
            const int sh = m > 0.f ? e - 15 : 0;
            if (col >= mt || seg >= nseg) continue;   // (a half tile past ff: no segment)
            if (wave == w0 && q == 0) hs[(int64_t)(q0 + col) * nseg + seg] = sh;
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int o = nt * (kRows / 2) + (kRowsW / 2) * wave + 16 * t + 4 * q;
                if (o >= F) continue;
                uint32_t hi2[2], lo2[2];
#pragma unroll
                for (int v = 0; v < 4; v += 2) {
                    const float h0 = ldexpf(acc[t][c][v], -sh);
                    const float h1 = ldexpf(acc[t][c][v + 1], -sh);
                    const _Float16 a0 = (_Float16)h0, a1 = (_Float16)h1;
                    hi2[v / 2] = __builtin_bit_cast(uint32_t, f16x2_t{a0, a1});
                    lo2[v / 2] = __builtin_bit_cast(
                        uint32_t, f16x2_t{(_Float16)(h0 - (float)a0), (_Float16)(h1 - (float)a1)});
                }
                const int64_t off = (int64_t)(q0 + col) * F + o;
                *reinterpret_cast<i32x2_t *>(h_hi + off) = i32x2_t{(int)hi2[0], (int)hi2[1]};
                *reinterpret_cast<i32x2_t *>(h_lo + off) = i32x2_t{(int)lo2[0], (int)lo2[1]};
            }
        }
    }
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct PrefillWs {
    int32_t *pos;
    i32x2_t *tiles;
    int32_t *n_tiles;
    uint16_t *h_hi, *h_lo;
    int32_t *hs;     // [P][segments] h scale exponents
    float *ypair;
    uint16_t *x16;   // [T][H] x as scaled f16 (in the ypair region: dead before down writes it)
    int32_t *xs;     // [T] its scale exponents
};

int max_tiles(int32_t P, int32_t E) { return P / kBM + std::min(E, P) + 1; }
int h_segments(int32_t F, int32_t segf) { return (F + segf - 1) / segf; }
// the workspace holds the most segments any gate/up form can make
constexpr int kMinSegF = gate_up_segment<4>();

PrefillWs carve(void *ws, int32_t T, int32_t P, int32_t E, int32_t H, int32_t F) {
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
    w.hs = reinterpret_cast<int32_t *>(b);
    b += align256(sizeof(int32_t) * (size_t)P * h_segments(F, kMinSegF));
    w.ypair = reinterpret_cast<float *>(b);
    w.x16 = reinterpret_cast<uint16_t *>(b);   // 2 T H bytes <= 4 P H: P = T k >= T
    w.xs = reinterpret_cast<int32_t *>(b + align256(2 * (size_t)T * H));
    return w;
}

template <bool DOWN, bool DENSE, int WAVES, int SEGF>
int launch_gemm_as(const FfnArgs &a, const PrefillWs &w, int mt, hipStream_t s) {
    constexpr int kThreads = WAVES * 64;
    constexpr int kRows = kRowsW * WAVES;
    // A rows at their pitch; B: 128 rows x 1 operand or 64 x 2
    constexpr size_t lds =
        gemm_stages<DOWN, DENSE, WAVES>() * (kRows * gemm_a_pitch<DENSE>() + kBBytes);
    static bool attr = false;
    if (!attr) {
        const void *fn = reinterpret_cast<const void *>(gemm_kernel<DOWN, DENSE, WAVES, SEGF>);
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
            hipSuccess)
            return MOE_ELAUNCH;
        attr = true;
    }
    const int per_nt = DOWN ? kRows : kRows / 2;
    const int n_out = DOWN ? a.H : a.F;
    const int n_ntiles = (n_out + per_nt - 1) / per_nt;
    const int grid = 8 * ((mt + 7) / 8) * n_ntiles * (DOWN ? 2 : 1);
    const int id = DOWN ? MOE_KERNEL_DN_PREFILL : MOE_KERNEL_GU_PREFILL;
    prof_start(id, s);
    if constexpr (DOWN)
        hipLaunchKernelGGL((gemm_kernel<true, DENSE, WAVES, SEGF>), dim3(grid), dim3(kThreads),
                           lds, s,
                           nullptr, w.h_hi, w.h_lo, a.offsets, a.pair_ids, w.tiles, w.n_tiles, mt,
                           n_ntiles, a.down.base, a.down.expert_stride, a.down.experts, nullptr,
                           (int64_t)0, nullptr, a.down.kpack, nullptr, a.down.scale2, nullptr,
                           a.k, a.F, a.F, a.H, nullptr, nullptr, nullptr, w.hs, w.ypair);
    else
        hipLaunchKernelGGL((gemm_kernel<false, DENSE, WAVES, SEGF>), dim3(grid), dim3(kThreads),
                           lds, s,
                           (const uint16_t *)w.x16, nullptr, nullptr, a.offsets, a.pair_ids,
                           w.tiles, w.n_tiles, mt, n_ntiles, a.gate.base, a.gate.expert_stride,
                           a.gate.experts, a.up.base, a.up.expert_stride, a.up.experts,
                           a.gate.kpack, a.gate.kpack ? a.up.kpack : nullptr, a.gate.scale2,
                           a.up.scale2, a.k, a.H, a.F, a.H, (const int32_t *)w.xs, w.h_hi,
                           w.h_lo, w.hs, nullptr);
    prof_stop(id, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

// h's scale segments: 128 features when ff is not a multiple of 256 (and 32 segments of 128
// hold it), else 256. With 128, the gate/up GEMM from K-step-packed copies runs 4-wave
// workgroups over 128 features, so that no N tile is half empty (ff 640: 5 tiles of 128 instead
// of 3 of 256); from row-major banks it keeps 8 waves over 256 features with one scale per half,
// so that y does not depend on the form. Measured on the skewed ff-640 routing at T = 4096 (one
// box): gate/up 641 -> 498 us, the down GEMM, with twice the segment rescales, 522 -> 565 us.
int h_segment(int32_t F) {
    return F % gate_up_segment<8>() != 0 && h_segments(F, gate_up_segment<4>()) <= kMaxSeg
               ? gate_up_segment<4>()
               : gate_up_segment<8>();
}

}  // namespace

size_t prefill_ws_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F) {
    const int32_t P = T * k;
    return align256(sizeof(int32_t) * (size_t)P) +
           align256(sizeof(i32x2_t) * (size_t)max_tiles(P, E)) +
           256 + 2 * align256(2 * (size_t)P * F) +
           align256(sizeof(int32_t) * (size_t)P * h_segments(F, kMinSegF)) +
           align256(sizeof(float) * (size_t)P * H);
}

int launch_prefill(const FfnArgs &a, hipStream_t s) {
    const int32_t P = a.T * a.k;
    if (h_segments(a.F, gate_up_segment<8>()) > kMaxSeg) return MOE_ESHAPE;
    const PrefillWs w = carve(a.ws, a.T, P, a.E, a.H, a.F);
    const int mt = max_tiles(P, a.E);
    const int sched_blocks = std::max(1, std::min(256, (P + kThreadsSched - 1) / kThreadsSched));
    prof_start(MOE_KERNEL_SCHEDULE, s);
    hipLaunchKernelGGL(schedule_kernel, dim3(sched_blocks), dim3(kThreadsSched), 0, s, a.offsets,
                       a.pair_ids, a.active, a.counts, P, mt, w.tiles, w.n_tiles, w.pos);
    prof_stop(MOE_KERNEL_SCHEDULE, s);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    hipLaunchKernelGGL(xcast_kernel, dim3(a.T), dim3(kCastThreads), 0, s, a.x, a.H, w.x16, w.xs);
    if (hipGetLastError() != hipSuccess) return MOE_ELAUNCH;
    // from K-step-packed copies the GEMMs stage dense rows (DENSE), from row-major banks
    // 48-byte rows
    constexpr int kS4 = gate_up_segment<4>(), kS8 = gate_up_segment<8>();
    int st;
    if (h_segment(a.F) == kS4) {   // segments of 128 features
        st = a.gate.kpack ? launch_gemm_as<false, true, 4, kS4>(a, w, mt, s)
                          : launch_gemm_as<false, false, 8, kS4>(a, w, mt, s);
        if (st != MOE_OK) return st;
        st = a.down.kpack ? launch_gemm_as<true, true, 4, kS4>(a, w, mt, s)
                          : launch_gemm_as<true, false, 4, kS4>(a, w, mt, s);
    } else {
        st = a.gate.kpack ? launch_gemm_as<false, true, 8, kS8>(a, w, mt, s)
                          : launch_gemm_as<false, false, 8, kS8>(a, w, mt, s);
        if (st != MOE_OK) return st;
        st = a.down.kpack ? launch_gemm_as<true, true, 4, kS8>(a, w, mt, s)
                          : launch_gemm_as<true, false, 4, kS8>(a, w, mt, s);
    }
    if (st != MOE_OK) return st;
    return launch_combine(a.w, w.pos, a.offsets + a.E, w.ypair, a.T, a.k, a.H, a.y, s);
}

}  // namespace moe
