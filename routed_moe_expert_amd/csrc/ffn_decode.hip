// Decode path of the routed NVFP4 FFN (few tokens per expert, weight-stream bound).
//
// The union gather (moe_union_probe.rs: read each distinct expert's NVFP4 bytes once per call
// instead of once per routed slot): work items are (virtual expert, tile of weight rows); each
// item's NVFP4 tile is read once and contracted against up to 16 tokens routed to that expert on
// the matrix cores, one MFMA column tile, so the cost of an item does not grow with the expert's
// token count up to 16. A virtual expert is a run of at most 16 of an expert's pairs in CSR
// order: an expert with more tokens (a hot expert, a shared expert) becomes several, whose items
// are dealt out like any others and run side by side on different CUs. The same tile is then
// read once per virtual expert, close together in time (an L2 or last-level-cache hit for all
// but the first), instead of one workgroup reloading its token rows -- behind every tile in
// flight -- per 16-token chunk.
//
//   gu_decode: items of 8 gate rows + the 8 matching up rows = one 16-row MFMA A tile. The
//              four waves split K = hidden into four slices. Each lane decodes the E2M1 codes
//              of one row and one 16-weight scale group to f16 (v_cvt_scalef32_pk_f16_fp4) and
//              multiplies in the UE4M3 group scale (v_pk_mul_f16); both steps are exact, since
//              every E2M1 x UE4M3 product is an f16 value. The B operand is the expert's token
//              rows of x, held in registers as f16 for the whole expert: bf16 -> f16 is exact
//              once each (token, K slice) is scaled by a power of two that brings its largest
//              magnitude into [2^14, 2^15). v_mfma_f32_16x16x32_f16 accumulates in fp32; the
//              slices are unscaled, summed across the waves through LDS, and the epilogue
//              writes h = SiLU(g) * u (fp32) in CSR pair order.
//   dn_decode: items of 16*RT down rows; RT row tiles x (4/RT) K slices of ff over the four
//              waves, the split KS = 4/RT chosen by the kernel once its plan has counted the
//              virtual experts (more slices for a union of a few experts, so that the smaller
//              items reach every workgroup). B is the expert's h rows, scaled per (pair, K
//              slice) and split into f16 hi + lo (about 22 significant bits), two MFMAs per
//              step. Slices are summed through LDS into the per-pair rows ypair (row = pair
//              id).
//   combine:   y[t] = sum over t's local slots in ascending j of w[t,j] * ypair[t*k + j]; the
//              pair -> CSR slot map only says which slots are local.
//
// MFMA operand layout (v_mfma_f32_16x16x32_*): lane l supplies row l%16 of A and column l%16 of
// B, each with 8 consecutive reduction indices of group l/16; it receives rows 4*(l/16)..+3 of
// column l%16 of the result. The reduction order is free, so K step s of NVFP4 block b gives
// lane group q the weights 16q + 8s .. 16q + 8s + 7 of the block: one scale group per lane and
// two steps per block.
//
// Both FFN kernels are persistent: a grid of one or two 256-thread workgroups per CU, read from
// the device CSR (nothing is read back on the host). The (virtual expert, tile) items are dealt
// out in contiguous ranges over per-CU slots: each virtual expert's tiles over a group of slots
// of its own where there are no more of them than slots and that costs at most one item over an
// even cut, else an even cut of the item list; the two workgroups sharing a CU split their
// slot's range unevenly, since the first dispatched runs ahead. Tiles stream through a ring of
// LDS buffers with direct-to-LDS loads (two per workgroup with two workgroups per CU, up to six
// with one). Each wave copies its share of a tile into registers first thing, and the buffer is
// refilled as soon as every wave has done so, so all buffers are in flight while a tile is
// computed.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;          // 4 waves; two workgroups per CU
constexpr int kWaves = kThreads / 64;
constexpr int kCols = 16;              // token columns per MFMA tile
constexpr int kGuO = 8;                // output features per gu item: 8 gate rows + 8 up rows
constexpr int kCUs = 256;
constexpr int kMaxGuBlocks = 16;       // NVFP4 blocks per wave slice: hidden <= 4 * 16 * 64
constexpr int kMaxDnBlocks = 10;       // ... ff <= 4 * 10 * 64
constexpr int64_t kDnSpreadItems = 2048;   // down items (4 per workgroup) below which K splits
constexpr int kRedFloats = kWaves * kCols * 16;      // one set of per-wave 16x16 fp32 partials
constexpr int kRedBytes = 2 * kRedFloats * 4;        // two sets (double-buffered)

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

// 8 E2M1 codes (one code dword, low nibble first) times the group scale -> 8 f16, exact. The
// converts scale by 2^8 (their scale operand contributes its exponent only) and S holds the
// group scale times 2^-8 (scale_f16x2), so the products are the plain E2M1 x UE4M3 values.
__device__ __forceinline__ f16x8_t dequant8(uint32_t c, f16x2_t S) {
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 0) * S;
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 1) * S;
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 2) * S;
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 3) * S;
    return __builtin_bit_cast(f16x8_t, u32x4_t{__builtin_bit_cast(uint32_t, p0),
                                               __builtin_bit_cast(uint32_t, p1),
                                               __builtin_bit_cast(uint32_t, p2),
                                               __builtin_bit_cast(uint32_t, p3)});
}

// UE4M3 scale byte (0x00..0x7E) -> f16 pair holding 2^-8 times its value, exactly: the byte's
// 4 exponent and 3 mantissa bits shifted into the f16 exponent and top mantissa bits read as
// 2^(e-15) (1 + m/8) for e > 0 and as the subnormal m 2^-17 for e = 0, i.e. 2^-8 times the
// UE4M3 values 2^(e-7) (1 + m/8) and m 2^-9. One shift instead of a decode and a conversion.
__device__ __forceinline__ f16x2_t scale_f16x2(uint32_t byte) {
    const _Float16 s = __builtin_bit_cast(f16x2_t, byte << 7)[0];
    return f16x2_t{s, s};
}

__device__ __forceinline__ f32x4_t mfma16(f16x8_t a, f16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One lane's share of a row's K slice in an LDS tile: for each of NB blocks, the UE4M3 scale
// byte of its group q and the group's 16 E2M1 codes (two dwords). All reads are issued before
// any is used, so their LDS latencies overlap instead of adding up block by block.
template <int NB>
struct SliceA {
    uint32_t s[NB];
    uint32_t c[NB][2];
};

// Block j of the slice is block min(j0 + j, jlast) of the row: the clamp only bites for a last
// slice that runs past the row, whose extra blocks meet zero B operands (re-reading a block of
// the row keeps them finite). Whole slices take the unclamped form, with constant offsets.
template <int NB>
__device__ __forceinline__ void read_slice_at(const uint8_t *row, int j0, int jlast, int q,
                                              SliceA<NB> &a) {
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const uint8_t *blk = row + min(j0 + j, jlast) * kBlockBytes;
        a.s[j] = blk[q];
        const uint32_t *c = reinterpret_cast<const uint32_t *>(blk + 4 + 8 * q);
        a.c[j][0] = c[0];
        a.c[j][1] = c[1];
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the code that uses them
}

template <int NB>
__device__ __forceinline__ void read_slice(const uint8_t *row, int j0, int nblk, int q,
                                           SliceA<NB> &a) {
    if (j0 + NB <= nblk)
        read_slice_at<NB>(row + j0 * kBlockBytes, 0, NB - 1, q, a);
    else
        read_slice_at<NB>(row, j0, nblk - 1, q, a);
}

// Max over the four lanes of a column (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float colmax(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

// Power-of-two exponent s such that mx * 2^-s lies in [2^14, 2^15) (0 for mx = 0).
__device__ __forceinline__ int pick_scale(float mx) {
    int e = 0;
    if (mx > 0.f) (void)frexpf(mx, &e);   // mx = f * 2^e, f in [0.5, 1)
    return mx > 0.f ? e - 15 : 0;
}

// B operands of one token column for a K slice of NB blocks starting at blk0: lane (n, q) holds
// x[64 b + 16 q .. +15] of its token for every block b of the slice, as f16 scaled by 2^-s with
// s chosen per (token, slice); returns s. Absent token columns (row == nullptr) and blocks past
// the row give zeros. fetch_x_operands issues the loads, all under one branch (so they issue
// back to back), and convert_x_operands, once they have landed, zeroes the blocks past the row,
// scales and converts in place (same register footprint).
template <int NB>
__device__ __forceinline__ void fetch_x_operands(u32x4_t (&xb)[NB][2], const uint16_t *row,
                                                 int blk0, int nblk, int q) {
#pragma unroll
    for (int j = 0; j < NB; j++) xb[j][0] = xb[j][1] = u32x4_t{0, 0, 0, 0};
    if (row != nullptr) {
#pragma unroll
        for (int j = 0; j < NB; j++) {   // blocks past the row re-read the row's start
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
                blk0 + j < nblk ? row + 64 * (blk0 + j) + 16 * q : row);
            xb[j][0] = src[0];
            xb[j][1] = src[1];
        }
    }
}
template <int NB>
__device__ __forceinline__ int convert_x_operands(u32x4_t (&xb)[NB][2], int blk0, int nblk) {
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const bool in = blk0 + j < nblk;   // wave-uniform
        xb[j][0] = in ? xb[j][0] : u32x4_t{0, 0, 0, 0};
        xb[j][1] = in ? xb[j][1] : u32x4_t{0, 0, 0, 0};
    }
    uint32_t amax = 0;   // |x| as bf16 bits: ordered like the magnitudes for finite values
#pragma unroll
    for (int j = 0; j < NB; j++)
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                amax = max(amax, max(xb[j][h][i] & 0x7fffu, (xb[j][h][i] >> 16) & 0x7fffu));
    const int s = pick_scale(colmax(__uint_as_float(amax << 16)));
    const float inv = ldexpf(1.0f, -s);
#pragma unroll
    for (int j = 0; j < NB; j++)
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t w = xb[j][h][i];
                const f16x2_t v = {(_Float16)(__uint_as_float(w << 16) * inv),
                                   (_Float16)(__uint_as_float(w & 0xffff0000u) * inv)};
                xb[j][h][i] = __builtin_bit_cast(uint32_t, v);
            }
    return s;
}

// B operands of one h column (fp32, CSR row of a pair) for a K slice of ff: hi + lo f16 pairs,
// scaled by 2^-s per (pair, slice); returns s. The fp32 words land in the hi/lo registers
// (hi[j] = values 0..7 of block j, lo[j] = values 8..15) and are converted one block at a time.
// Absent columns and blocks past the row give zeros, as for the token rows of x; the loads
// (fetch_h_operands) and the conversion (convert_h_operands) are split the same way.
template <int NB>
__device__ __forceinline__ void fetch_h_operands(u32x4_t (&hi)[NB][2], u32x4_t (&lo)[NB][2],
                                                 const float *row, int blk0, int nblk, int q) {
#pragma unroll
    for (int j = 0; j < NB; j++)
        hi[j][0] = hi[j][1] = lo[j][0] = lo[j][1] = u32x4_t{0, 0, 0, 0};
    if (row != nullptr) {
#pragma unroll
        for (int j = 0; j < NB; j++) {   // blocks past the row re-read the row's start
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(
                blk0 + j < nblk ? row + 64 * (blk0 + j) + 16 * q : row);
            hi[j][0] = src[0];
            hi[j][1] = src[1];
            lo[j][0] = src[2];
            lo[j][1] = src[3];
        }
    }
}
template <int NB>
__device__ __forceinline__ int convert_h_operands(u32x4_t (&hi)[NB][2], u32x4_t (&lo)[NB][2],
                                                  int blk0, int nblk) {
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < NB; j++)
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float m = fmaxf(fabsf(__uint_as_float(hi[j][h][i])),
                                      fabsf(__uint_as_float(lo[j][h][i])));
                mx = blk0 + j < nblk ? fmaxf(mx, m) : mx;
            }
    const int s = pick_scale(colmax(mx));
    const float inv = ldexpf(1.0f, -s);
#pragma unroll
    for (int j = 0; j < NB; j++) {
        const bool in = blk0 + j < nblk;   // wave-uniform
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[i] = in ? __uint_as_float(hi[j][0][i]) * inv : 0.f;
            v[4 + i] = in ? __uint_as_float(hi[j][1][i]) * inv : 0.f;
            v[8 + i] = in ? __uint_as_float(lo[j][0][i]) * inv : 0.f;
            v[12 + i] = in ? __uint_as_float(lo[j][1][i]) * inv : 0.f;
        }
#pragma unroll
        for (int st = 0; st < 2; st++)      // K step st: values 8 st .. 8 st + 7
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float f0 = v[8 * st + 2 * i], f1 = v[8 * st + 2 * i + 1];
                const _Float16 h0 = (_Float16)f0, h1 = (_Float16)f1;
                hi[j][st][i] = __builtin_bit_cast(uint32_t, f16x2_t{h0, h1});
                lo[j][st][i] = __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)(f0 - (float)h0),
                                                                    (_Float16)(f1 - (float)h1)});
            }
    }
    return s;
}

__device__ __forceinline__ f32x4_t unscale(f32x4_t acc, int s) {
    return f32x4_t{ldexpf(acc[0], s), ldexpf(acc[1], s), ldexpf(acc[2], s), ldexpf(acc[3], s)};
}

// Item range of this workgroup: items are (virtual expert a, row tile t) in a-major order.
//
// Ranges are dealt to "slots": with a grid of two workgroups per CU, hardware places workgroups
// 0..255 one per CU and 256..511 beside them, and under oldest-first issue arbitration the first
// of a CU's two runs ahead (measured on the decode shapes: with equal ranges the second set
// finishes about 19% later than the first). So slot u is the pair (u, u + 256), and its range is
// cut so that the first member takes kLeadNum / kLeadDen of it. Otherwise a slot is a workgroup.
//
// When the slots number at least the virtual experts without costing balance, each one's tiles
// are split over g slots and no workgroup changes expert: its token rows are loaded once, before
// its stream of tiles starts, instead of at an expert change, where the load (vector memory
// completes in issue order) would wait for every tile in flight. Otherwise the items are split
// into equal contiguous ranges.
constexpr int kLeadNum = 23, kLeadDen = 40;   // 57.5%: measured best of 52.5, 55, 57.5 and 60%

__host__ __device__ inline bool paired_grid(int grid) { return grid == 2 * kCUs; }

__device__ __forceinline__ void item_range(int n_active, int tiles, int &i0, int &i1) {
    const int G = gridDim.x, b = blockIdx.x, total = n_active * tiles;
    const bool paired = paired_grid(G);
    const int U = paired ? G / 2 : G, u = paired ? b % U : b;
    const int per = (total + U - 1) / U;
    int lo = min(u * per, total), hi = min(lo + per, total);
    if (n_active > 0 && n_active <= U) {
        const int g = U / n_active, per_g = (tiles + g - 1) / g;
        if (per_g <= per + 1) {
            const int a = u / g, r = u % g;
            lo = hi = 0;
            if (a < n_active) {
                lo = a * tiles + r * tiles / g;
                hi = a * tiles + (r + 1) * tiles / g;
            }
        }
    }
    i0 = lo;
    i1 = hi;
    if (paired) {
        const int cut = lo + ((hi - lo) * kLeadNum + kLeadDen / 2) / kLeadDen;
        if (b < U) i1 = cut;
        else i0 = cut;
    }
}

// Gate/up tile layout in LDS: 16 rows (8 gate, then the 8 matching up rows), one per lane row of
// the MFMA tile, each lane reading its own row. When a row is whole 16-byte chunks (hidden a
// multiple of 256) the rows sit one chunk further apart than their length: for hidden 2560
// (1440-byte rows, 360 dwords: 8 past a multiple of the 32 LDS banks) the same byte of rows n and
// n + 4 would fall in one bank; at a 1456-byte pitch only rows n and n + 8 share one, which halves
// the bank conflicts of the reads. The pad chunk is filled with a copy of the row's first chunk,
// so each direct-to-LDS load still moves 64 whole chunks. Otherwise (hidden a multiple of 64
// only) the 8 gate rows and the 8 up rows are each one contiguous 16-byte aligned run
// (8 rows = 4.5 hidden bytes) and land unpadded, pitch = row length.
__host__ __device__ inline int gu_pitch(int rb) { return rb % 16 == 0 ? rb + 16 : rb; }
constexpr int kMaxTileInst = 10;   // loads per wave for one padded tile (hidden <= 4096)

// Wait for every outstanding vector-memory operation with a real s_waitcnt (the builtin, which
// the compiler's wait insertion understands, unlike an asm statement): registers loaded before
// it are then known to be complete, and their first use after later direct-to-LDS loads does not
// wait for those.
__device__ __forceinline__ void wait_vm_all() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt not waited on
}

__device__ __forceinline__ void dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 16, 0, 0);
}

// The CSR entries a workgroup needs, per virtual expert of its range: the expert, the first CSR
// slot and pair count (at most kCols) of its run of pairs and their pair ids, and for up to two
// banks the expert's first weight rows and second-level weight scales (1 when a bank has none).
constexpr int kMaxMeta = 32;   // virtual experts per workgroup range; grids are sized so this holds
struct Meta {
    int n_active, n_local, n_real;   // n_active: virtual experts; n_real: see plan_ids_a
    int e[kMaxMeta], q0[kMaxMeta], m[kMaxMeta], pid[kMaxMeta][kCols];
    int pbase[kMaxMeta];   // first entry of the run's pairs in the fused plan's pair list
    float s2a[kMaxMeta], s2b[kMaxMeta];
    const uint8_t *pa[kMaxMeta], *pb[kMaxMeta];
};

// Virtual experts of an expert with m pairs: runs of kCols pairs, the last one shorter.
__host__ __device__ inline int n_virtual(int m) { return (m + kCols - 1) / kCols; }

// At most as many virtual experts as pairs, and at most one per active expert plus one per
// kCols further pairs (the count a grid is sized for).
__host__ __device__ inline int max_virtual(int E, int P) {
    const int v = (E < P ? E : P) + P / kCols;
    return v < P ? v : P;
}

// The down kernel's K split, chosen once the number of virtual experts is known (the same rule on
// both plan forms, so they scale h alike and give the same y): from the smallest split the slice
// width allows (ks_min), doubled while the slices average two NVFP4 blocks or more and the items
// (virtual experts x H / (16 RT), RT = 4 / KS row tiles per item) stay under kDnSpreadItems. With
// a union of a few experts the smaller items then spread over every workgroup, and each wave
// loads only its slice of the h rows (with one slice every wave loads all of them). Measured
// down kernel, KS 1 / 2 / 4: 10 experts (tiny decode) 17.1 / 15.5 / 14.7 us; 30 experts 21.1 /
// 20.9 / 25.1 us (layer 45.0 / 43.5 / 48.9 us); 60 experts 25.7 / 28.2 / 38.6 us; E256 T=16
// 46.6 / 55.6 / 83.3 us.
struct DnSplit {
    int ks_min, bf, H;   // ks_min 0: not the down kernel (tiles fixed)
};
__host__ __device__ inline int dn_ks(const DnSplit &d, int n_active) {
    int ks = d.ks_min;
    while (ks < kWaves && 4 * ks <= d.bf &&
           (int64_t)n_active * (d.H / (16 * kWaves)) * ks < kDnSpreadItems)
        ks *= 2;
    return ks;
}
// Row tiles per virtual expert: fixed, or the down kernel's for its split.
__device__ __forceinline__ int plan_tiles(const DnSplit &d, int n_active, int tiles) {
    return d.ks_min ? d.H / (16 * (kWaves / dn_ks(d, n_active))) : tiles;
}

// Expert e's first weight row in a bank: from the bank's per-expert pointer table when it has one,
// else at base + e * stride.
__device__ __forceinline__ const uint8_t *expert_rows(const uint8_t *base, int64_t stride,
                                                      const uint8_t *const *tab, int e) {
    return tab ? tab[e] : base + e * stride;
}

constexpr int kPairCap = 4096;   // pair ids read whole at start up to this many

// LDS scratch of load_plan: the active list, the offsets, (up to kPairCap) the pair ids, scan
// partials and the workgroup's virtual experts (expert, run).
inline size_t plan_scratch_bytes(int E, int P) {
    return 4 * (2 * (size_t)E + 1 + (P <= kPairCap ? P : 0) + 16 + 2 * kMaxMeta);
}

// Exclusive scan of one int per thread over the workgroup; *total gets the sum. wsum: kWaves ints.
__device__ int wg_exclusive_scan(int v, int *wsum, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    lds_barrier();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        const int ws = wsum[w];
        before += w < wave ? ws : 0;
        tot += ws;
    }
    *total = tot;
    lds_barrier();
    return before + x - v;
}

// This workgroup's item range and CSR entries. The counts, the whole active list, the whole
// offsets array and (when short) all pair ids are fetched at once into LDS scratch, so start up
// costs one round trip to memory instead of the chain counts -> active -> offsets -> pair ids.
// The virtual experts are then numbered by a scan of their counts over the active list (each
// thread a contiguous run of it), and each thread enters those of its run that fall in the
// workgroup's range.
__device__ void load_plan(Meta &meta, int32_t *scratch, const int32_t *__restrict__ counts,
                          const int32_t *__restrict__ active, const int32_t *__restrict__ offsets,
                          const int32_t *__restrict__ pair_ids, const uint8_t *wa, int64_t sa,
                          const uint8_t *const *ta, const float *__restrict__ s2a,
                          const uint8_t *wb, int64_t sb, const uint8_t *const *tb,
                          const float *__restrict__ s2b, int E, int P, const DnSplit &sp,
                          int &tiles, int &i0, int &i1, int &a_first) {
    const int tid = threadIdx.x;
    const bool pairs_in_lds = P <= kPairCap;
    int32_t *s_act = scratch, *s_off = scratch + E, *s_pair = scratch + 2 * E + 1;
    int32_t *s_wsum = s_pair + (pairs_in_lds ? P : 0), *s_ve = s_wsum + 16,
            *s_vc = s_ve + kMaxMeta;
    if (tid == 0) meta.n_real = counts[0];
    // scratch[j] for j < total is entry j of active ++ offsets ++ pair_ids; each thread issues
    // all of its loads of a batch before storing any, so the batch costs one memory round trip
    constexpr int kBatch = 8;
    const int total = 2 * E + 1 + (pairs_in_lds ? P : 0);
    for (int base = 0; base < total; base += kBatch * kThreads) {
        int32_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const int j = base + u * kThreads + tid;
            // a pointer select and one unconditional load (past the end: counts, always valid)
            const int32_t *src = j < E       ? active + j
                                 : j <= 2 * E ? offsets + (j - E)
                                 : j < total  ? pair_ids + (j - 2 * E - 1)
                                              : counts;
            v[u] = *src;
        }
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const int j = base + u * kThreads + tid;
            if (j < total) scratch[j] = v[u];
        }
    }
    lds_barrier();
    const int n_act = meta.n_real;
    const int per = (n_act + kThreads - 1) / kThreads;
    const int lo = min(tid * per, n_act), hi = min(lo + per, n_act);
    int mine = 0;
    for (int j = lo; j < hi; j++) {
        const int e = s_act[j];
        mine += n_virtual(s_off[e + 1] - s_off[e]);
    }
    int nv;
    int v = wg_exclusive_scan(mine, s_wsum, &nv);
    tiles = plan_tiles(sp, nv, tiles);
    item_range(nv, tiles, i0, i1);
    a_first = i0 / tiles;
    const int na = i0 < i1 ? min((i1 - 1) / tiles - a_first + 1, kMaxMeta) : 0;
    for (int j = lo; j < hi && v < a_first + na; j++) {
        const int e = s_act[j], nch = n_virtual(s_off[e + 1] - s_off[e]);
        for (int c = max(0, a_first - v); c < nch && v + c < a_first + na; c++) {
            s_ve[v + c - a_first] = e;
            s_vc[v + c - a_first] = c;
        }
        v += nch;
    }
    if (tid == 0) meta.n_active = nv;
    lds_barrier();
    if (tid < na) {
        const int e = s_ve[tid], c = s_vc[tid];
        const int q0 = s_off[e] + c * kCols, m = min(kCols, s_off[e + 1] - q0);
        meta.e[tid] = e;
        meta.q0[tid] = q0;
        meta.m[tid] = m;
        meta.s2a[tid] = s2a ? s2a[e] : 1.f;
        meta.s2b[tid] = s2b ? s2b[e] : 1.f;
        meta.pa[tid] = expert_rows(wa, sa, ta, e);
        meta.pb[tid] = (wb || tb) ? expert_rows(wb, sb, tb, e) : nullptr;
        // a run has m >= 1: entries past m re-read entry m - 1 and are then zeroed
        if (pairs_in_lds) {
#pragma unroll
            for (int j = 0; j < kCols; j++) {
                const int pv = s_pair[q0 + min(j, m - 1)];
                meta.pid[tid][j] = j < m ? pv : 0;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kCols; j++) {
                const int pv = pair_ids[q0 + min(j, m - 1)];
                meta.pid[tid][j] = j < m ? pv : 0;
            }
        }
    }
    lds_barrier();
}

// The fused layer (moe_layer_nvfp4): the decode kernels bucket the routed pairs themselves, in
// each workgroup's LDS, from the routed expert ids -- the same stable expert-first CSR as
// moe_route_bucket (moe_sk_repro.rs, its host bucketing) -- so the layer needs no bucketing
// launch. Up to kIdsMaxPairs pairs and kIdsMaxExperts experts.
constexpr int kIdsMaxPairs = 2048;
constexpr int kIdsMaxExperts = 1024;
constexpr int kIdsPer = kIdsMaxPairs / kThreads;   // routed ids per thread

// LDS of the fused plan. The early part (phase A only) lies in the ring region, which no tile
// has reached yet: counts [E], offsets [E+1], the virtual expert list [max_virtual], scan
// partials. The late part (phase B, while the first tiles stream into the ring) lies after the
// partials and the pair list: keys [P], the workgroup's expert ranks [E], per-wave counts
// [kWaves][kMaxMeta], cursors [kMaxMeta].
inline size_t ids_early_bytes(int E, int P) {
    return 4 * (2 * (size_t)E + 1 + (size_t)max_virtual(E, P) + 16);
}
inline size_t ids_late_bytes(int E, int P) {
    return 4 * ((size_t)P + (size_t)E + (kWaves + 1) * kMaxMeta);
}

struct IdsLds {
    int32_t *cnt, *off, *act, *wsum;   // early
    int32_t *key, *rank, *wc, *cur;    // late
};

__device__ __forceinline__ IdsLds ids_lds(uint8_t *ring, int32_t *late, int E, int P) {
    IdsLds l;
    l.cnt = reinterpret_cast<int32_t *>(ring);
    l.off = l.cnt + E;
    l.act = l.off + E + 1;
    l.wsum = l.act + max_virtual(E, P);
    l.key = late;
    l.rank = l.key + P;
    l.wc = l.rank + E;
    l.cur = l.wc + kWaves * kMaxMeta;
    return l;
}

// Phase A of the plan from the routed ids: load the P ids (one round trip) and histogram the
// local expert of each pair; scan the counts into the CSR offsets and the virtual expert counts
// into the ascending virtual expert list (one scan: both packed in one int, P <= 2^16), entries
// expert | run << 16; take the item range and the virtual experts' entries -- all that
// addressing the weight tiles needs.
// An expert's CSR slots are offsets[e] + the rank of the pair among its pairs, as
// moe_route_bucket lays them out. For phase B, the experts the workgroup's virtual experts belong
// to (its "real" experts, a contiguous run of the active experts, so in ascending order) get
// indices 0 .. n_real - 1 in rank[], and each the first entry of its whole pair list in cur[]
// (pair lists of real experts follow each other; a run's pairs start kCols * run further in).
__device__ void plan_ids_a(Meta &meta, const IdsLds &l, const int32_t *__restrict__ ids,
                           int expert_base, const uint8_t *wa, int64_t sa,
                           const uint8_t *const *ta, const float *__restrict__ s2a,
                           const uint8_t *wb, int64_t sb, const uint8_t *const *tb,
                           const float *__restrict__ s2b, int E, int P, const DnSplit &sp,
                           int &tiles, int &i0, int &i1, int &a_first, int &na) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int key[kIdsPer];
#pragma unroll
    for (int u = 0; u < kIdsPer; u++) {   // one round trip; past P re-read ids[0]
        const int p = u * kThreads + tid;
        key[u] = ids[p < P ? p : 0];
    }
    for (int i = tid; i < E; i += kThreads) l.cnt[i] = 0;
    lds_barrier();
#pragma unroll
    for (int u = 0; u < kIdsPer; u++) {
        const int p = u * kThreads + tid;
        const int64_t e = (int64_t)key[u] - expert_base;
        const int kk = (e >= 0 && e < E) ? (int)e : -1;
        if (p < P) {
            l.key[p] = kk;
            if (kk >= 0) atomicAdd(&l.cnt[kk], 1);
        }
    }
    lds_barrier();
    // each thread a contiguous run of experts; pair counts in the low 16 bits, virtual counts above
    const int per = (E + kThreads - 1) / kThreads;
    const int lo = min(tid * per, E), hi = min(lo + per, E);
    int mine = 0;
    for (int i = lo; i < hi; i++) {
        const int c = l.cnt[i];
        mine += c + (n_virtual(c) << 16);
    }
    int tot;
    const int ex = wg_exclusive_scan(mine, l.wsum, &tot);
    int run = ex & 0xffff, v = ex >> 16;
    for (int i = lo; i < hi; i++) {
        const int c = l.cnt[i];
        l.off[i] = run;
        for (int r = 0; r < n_virtual(c); r++) l.act[v++] = i | r << 16;
        run += c;
    }
    if (tid == 0) {
        l.off[E] = tot & 0xffff;
        meta.n_active = tot >> 16;
        meta.n_local = tot & 0xffff;
    }
    lds_barrier();
    tiles = plan_tiles(sp, tot >> 16, tiles);
    item_range(meta.n_active, tiles, i0, i1);
    a_first = i0 / tiles;
    na = i0 < i1 ? min((i1 - 1) / tiles - a_first + 1, kMaxMeta) : 0;
    if (wave == 0) {
        const int ent = lane < na ? l.act[a_first + lane] : 0;
        const int e = ent & 0xffff, r = ent >> 16;
        const int me = lane < na ? l.cnt[e] : 0;   // pairs of the whole expert
        // a real expert starts at lane 0 and at every run 0
        const bool start = lane < na && (lane == 0 || r == 0);
        const uint64_t sm = __ballot(start);
        const int ri = __popcll(sm & (~0ull >> (63 - lane))) - 1;   // its index
        int x = start ? me : 0;   // inclusive scan over the lanes: lists of the real experts
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane < na) {
            const int first = x - me;   // the real expert's first list entry
            meta.e[lane] = e;
            meta.q0[lane] = l.off[e] + r * kCols;
            meta.m[lane] = min(kCols, me - r * kCols);
            meta.pbase[lane] = first + r * kCols;
            meta.s2a[lane] = s2a ? s2a[e] : 1.f;
            meta.s2b[lane] = s2b ? s2b[e] : 1.f;
            meta.pa[lane] = expert_rows(wa, sa, ta, e);
            meta.pb[lane] = (wb || tb) ? expert_rows(wb, sb, tb, e) : nullptr;
            if (start) {
                l.rank[e] = ri;
                l.cur[ri] = first;
            }
        }
        if (lane == 0) meta.n_real = __popcll(sm);
    }
    lds_barrier();
}

// Phase B: list the pairs of the workgroup's real experts in ascending pair id, expert by
// expert, into plist: per 256-pair step, a pair's rank among its expert's pairs of the step is
// the population of a wave ballot below its lane plus the counts of the waves before it, added
// to the expert's running cursor. The workgroup's real experts are the active experts with ids
// from its first virtual expert's to its last one's.
// With pos != nullptr (gate/up), the workgroup that holds tile 0 of a virtual expert writes the
// pair -> CSR slot map of that run's pairs, and workgroup 0 marks the non-local pairs and writes
// the number of local pairs to *n_local.
__device__ void plan_ids_b(Meta &meta, const IdsLds &l, int32_t *plist, int P, int tiles, int i0,
                           int i1, int a_first, int na, int32_t *__restrict__ pos,
                           int32_t *__restrict__ n_local) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int nr = na > 0 ? meta.n_real : 0;
    const int e_lo = na > 0 ? meta.e[0] : 0, e_hi = na > 0 ? meta.e[na - 1] : -1;
    for (int c0 = 0; c0 < P; c0 += kThreads) {
        const int p = c0 + tid;
        int al = -1;   // the pair's expert among the workgroup's real experts, or -1
        if (p < P) {
            const int kk = l.key[p];
            if (kk >= e_lo && kk <= e_hi) al = l.rank[kk];
        }
        int rank = 0;
        for (int a = 0; a < nr; a++) {
            const uint64_t mk = __ballot(al == a);
            if (al == a) rank = __popcll(mk & below);
            if (lane == 0) l.wc[wave * kMaxMeta + a] = __popcll(mk);
        }
        lds_barrier();
        if (al >= 0) {
            int at = l.cur[al] + rank;
            for (int w = 0; w < wave; w++) at += l.wc[w * kMaxMeta + al];
            plist[at] = p;
        }
        lds_barrier();
        if (tid < nr) {
            int add = 0;
#pragma unroll
            for (int w = 0; w < kWaves; w++) add += l.wc[w * kMaxMeta + tid];
            l.cur[tid] += add;
        }
        lds_barrier();
    }
    if (tid < na) {
        const int m = meta.m[tid], b = meta.pbase[tid];
#pragma unroll
        for (int j = 0; j < kCols; j++) {   // entries past m re-read entry m - 1, then zeroed
            const int v = plist[b + min(j, m - 1)];
            meta.pid[tid][j] = j < m ? v : 0;
        }
    }
    if (pos != nullptr) {
        // pair -> CSR slot: by the holder of each run's tile 0; non-local pairs by workgroup 0
        for (int a = 0; a < na; a++) {
            const int it0 = (a_first + a) * tiles;
            if (it0 < i0 || it0 >= i1) continue;
            const int m = meta.m[a], b = meta.pbase[a], q0 = meta.q0[a];
            for (int j = tid; j < m; j += kThreads) pos[plist[b + j]] = q0 + j;
        }
        if (blockIdx.x == 0) {
            for (int p = tid; p < P; p += kThreads)
                if (l.key[p] < 0) pos[p] = 0x7fffffff;
            if (tid == 0) *n_local = meta.n_local;
        }
    }
    lds_barrier();
}

// Gate/up + SiLU * up over the union of active experts; the four waves split K = hidden. An
// item's first barrier publishes tile i and the previous item's partial tiles (double-buffered);
// once every wave holds its slice of tile i in registers, a second barrier hands the buffer back
// to the stream. One wave (rotating) then sums the previous item's partials while the others
// contract.
// Tile i is awaited with "at most the memory operations issued after it outstanding": vector
// memory operations complete in issue order, so that wait covers tile i and nothing newer.
template <int NB>
__global__ __launch_bounds__(kThreads, 2) void gu_decode_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ pair_ids, const int32_t *__restrict__ active,
    const int32_t *__restrict__ counts, const uint8_t *__restrict__ gate, int64_t gate_stride,
    const uint8_t *const *__restrict__ gate_tab, const uint8_t *__restrict__ up, int64_t up_stride,
    const uint8_t *const *__restrict__ up_tab, const float *__restrict__ gate_s2,
    const float *__restrict__ up_s2, int32_t k, int32_t P, int32_t E, int32_t H, int32_t F,
    int32_t nbuf, int32_t ring_bytes, float *__restrict__ h, int32_t *__restrict__ pos,
    const int32_t *__restrict__ ids, int32_t expert_base, int32_t T, int32_t tokcols,
    int32_t *__restrict__ n_local) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int rb = H / kBlockWeights * kBlockBytes;
    const int side = kGuO * rb;
    const int pitch = gu_pitch(rb), tile_bytes = 2 * kGuO * pitch;
    uint8_t *wb = smem;                                                // [nbuf][16 rows]
    float *red = reinterpret_cast<float *>(smem + ring_bytes);         // [2][wave][col][16 rows]
    __shared__ Meta meta;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;   // A row / B column, and K group
    // K slices of NB blocks; a last slice may run past the row (reads clamp, operands zero)
    const int nblk = H / kBlockWeights, blk0 = wave * NB;
    int tiles = F / kGuO;
    // fused layer: the pair list and the plan's late scratch live in LDS behind the partials;
    // else the pair list is the CSR's
    const bool fused = ids != nullptr;
    int32_t *lds_list = reinterpret_cast<int32_t *>(smem + ring_bytes + kRedBytes);
    const IdsLds il = ids_lds(smem, lds_list + P, E, P);

    // token columns (T <= 16): the B operand is every token's row of x, column n = token n, the
    // same for every expert, so it is loaded now, beside the plan's loads; each expert then keeps
    // the columns of its own pairs' tokens
    u32x4_t xb[NB][2];
    if (tokcols) fetch_x_operands<NB>(xb, n < T ? x + (int64_t)n * H : nullptr, blk0, nblk, q);

    int i0, i1, a_first, na = 0;
    if (fused)
        plan_ids_a(meta, il, ids, expert_base, gate, gate_stride, gate_tab, gate_s2, up,
                   up_stride, up_tab, up_s2, E, P, DnSplit{0, 0, 0}, tiles, i0, i1, a_first, na);
    else
        load_plan(meta, reinterpret_cast<int32_t *>(smem), counts, active, offsets, pair_ids, gate,
                  gate_stride, gate_tab, gate_s2, up, up_stride, up_tab, up_s2, E, P,
                  DnSplit{0, 0, 0}, tiles, i0, i1, a_first);
    // load k of this wave moves LDS chunk p = 64 wave + 256 k + lane of the tile; its source
    // offset within the gate or up rows of the tile (sign bit: up) is the same for every tile.
    // Padded pitch: chunk p is chunk p % cpr of row p / cpr (the last one a copy of chunk 0).
    // Unpadded: chunk p is chunk p of the 8 gate rows' run, then of the 8 up rows' run.
    const bool padded = pitch != rb;
    const int cpr = rb / 16 + 1, half = kGuO * rb / 16;
    const int units = padded ? 2 * kGuO * cpr : 2 * half;
    // (row, chunk) of p stepped along kk without a division: p grows by kThreads per step
    int32_t src_off[kMaxTileInst];
    {
        int p = wave * 64 + lane, r = 0, c = p;
        while (c >= cpr) { c -= cpr; r++; }
#pragma unroll
        for (int kk = 0; kk < kMaxTileInst; kk++) {
            if (padded)
                src_off[kk] = ((r & (kGuO - 1)) * rb + (c == cpr - 1 ? 0 : c) * 16) |
                              (r >= kGuO ? (int32_t)0x80000000 : 0);
            else
                src_off[kk] = p < half ? p * 16 : ((p - half) * 16) | (int32_t)0x80000000;
            p += kThreads;
            c += kThreads;
            while (c >= cpr) { c -= cpr; r++; }
        }
    }
    const int n_inst = stage_async_count<kThreads>(units * 16);
    // stream cursor: the next item to load (expert index, row tile, ring slot)
    int ia = 0, it = i0 - a_first * tiles, is = 0;
    auto issue_next = [&]() {
        uint8_t *dst = wb + is * tile_bytes;
        const uint8_t *gt = meta.pa[ia] + (int64_t)it * side;
        const uint8_t *ut = meta.pb[ia] + (int64_t)it * side;
#pragma unroll
        for (int kk = 0; kk < kMaxTileInst; kk++) {
            const int base = wave * 64 + kk * kThreads;
            if (base < units && base + lane < units) {
                const int32_t o = src_off[kk];
                dma16((o < 0 ? ut : gt) + (o & 0x7fffffff), dst + base * 16);
            }
        }
        asm volatile("" ::: "memory");   // later stores stay behind these loads (ring waits)
        if (++it == tiles) { it = 0; ++ia; }
        if (++is == nbuf) is = 0;
    };

    // reduction of an item by one wave: lane -> (feature f, pair nn of the run). One wave
    // (rotating) takes it while the others go on, which measured faster than a quarter per wave.
    // A pair's column is its place in the run, or with token columns its token.
    // (a_: the item's virtual expert, for its first CSR slot and second-level gate and up scales)
    auto reduce = [&](const float *rp, int a_, int t, int mt) {
        const int q0 = meta.q0[a_];
        const float sg = meta.s2a[a_], su = meta.s2b[a_];
        for (int o = lane; o < kGuO * mt; o += 64) {
            const int f = o & (kGuO - 1), nn = o / kGuO;
            const int col = tokcols ? meta.pid[a_][nn] / k : nn;
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; w++) {
                g += rp[(w * kCols + col) * 16 + f];
                u += rp[(w * kCols + col) * 16 + f + kGuO];
            }
            g *= sg;
            u *= su;
            h[(int64_t)(q0 + nn) * F + t * kGuO + f] = silu(g) * u;
        }
    };

    int xs = 0, cur_a = -1;
    auto fetch_x = [&](int a_) {   // token rows of virtual expert a_
        const uint16_t *row = nullptr;
        if (n < meta.m[a_]) row = x + (int64_t)(meta.pid[a_][n] / k) * H;
        fetch_x_operands<NB>(xb, row, blk0, nblk, q);
        cur_a = a_;
    };
    // Start-up order: the token rows are complete (and the compiler told so by a real wait)
    // before tile 0 is issued, so that their conversion to f16 -- about a thousand VALU
    // instructions per wave -- runs while tile 0 is in flight (after a direct-to-LDS load the
    // compiler would otherwise wait for everything outstanding before the first use of x). With
    // token columns x was loaded beside the plan and the whole ring is issued at once (so that a
    // workgroup's later tiles travel with every workgroup's first); otherwise the token rows come
    // after the fused plan's phase B (pair lists) and the rest of the ring follows.
    if (tokcols) {
        if (i0 < i1) wait_vm_all();   // x landed with the plan's loads
        for (int i = i0; i < min(i0 + nbuf, i1); i++) issue_next();   // the whole ring at once
        if (i0 < i1) xs = convert_x_operands<NB>(xb, blk0, nblk);    // overlaps the ring
        if (fused) plan_ids_b(meta, il, lds_list, P, tiles, i0, i1, a_first, na, pos, n_local);
    } else {
        if (fused) plan_ids_b(meta, il, lds_list, P, tiles, i0, i1, a_first, na, pos, n_local);
        if (i0 < i1) {
            fetch_x(0);
            wait_vm_all();   // the token rows first, so that their conversion overlaps tile 0
            issue_next();
            xs = convert_x_operands<NB>(xb, blk0, nblk);
        }
        for (int i = i0 + 1; i < min(i0 + nbuf, i1); i++) issue_next();   // every buffer in flight
    }

    int p_a = 0, p_t = 0, p_mt = 0;
    int a = 0, t = i0 - a_first * tiles, slot = 0;   // item i: virtual expert, row tile, ring slot
    for (int i = i0; i < i1; i++) {
        const int mt = meta.m[a];
        const uint8_t *wt = wb + slot * tile_bytes + n * pitch;   // this lane's row of the tile
        if (!tokcols && a != cur_a) {   // token rows of this virtual expert
            fetch_x(a);
            xs = convert_x_operands<NB>(xb, blk0, nblk);
        }
        // tile i landed: issued after it are at least the tiles behind it (the reducing wave's h
        // stores are not counted: they only make its wait stricter)
        vm_wait_le(min(nbuf - 1, i1 - 1 - i) * n_inst);
        lds_barrier();   // tile i and the previous item's partials visible to all
        SliceA<NB> sa;
        read_slice<NB>(wt, blk0, nblk, q, sa);
        if (i + nbuf < i1) {
            lds_barrier();   // tile i is in every wave's registers: refill its buffer
            issue_next();
        }
        const int u = i - i0;
        if (u > 0 && wave == (u - 1) % kWaves)
            reduce(red + ((u - 1) & 1) * kRedFloats, p_a, p_t, p_mt);
        // two independent accumulation chains (K steps 0 and 1 of each block) halve the
        // dependent MFMA latency
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const f16x2_t S = scale_f16x2(sa.s[j]);
            acc0 = mfma16(dequant8(sa.c[j][0], S), __builtin_bit_cast(f16x8_t, xb[j][0]), acc0);
            acc1 = mfma16(dequant8(sa.c[j][1], S), __builtin_bit_cast(f16x8_t, xb[j][1]), acc1);
        }
        *reinterpret_cast<f32x4_t *>(red + (u & 1) * kRedFloats + (wave * kCols + n) * 16 +
                                     4 * q) = unscale(acc0 + acc1, xs);
        p_a = a;
        p_t = t;
        p_mt = mt;
        if (++t == tiles) { t = 0; ++a; }
        if (++slot == nbuf) slot = 0;
    }
    if (i1 > i0) {
        const int u = i1 - i0;
        lds_barrier();
        if (wave == (u - 1) % kWaves) reduce(red + ((u - 1) & 1) * kRedFloats, p_a, p_t, p_mt);
    }
    // pair -> CSR slot map for the combine (not needed before it; the fused plan wrote it)
    if (!fused)
        for (int q2 = blockIdx.x * kThreads + tid; q2 < P; q2 += gridDim.x * kThreads)
            pos[pair_ids[q2]] = q2;
}

// Down projection over the union of active experts, same streaming scheme; an item is 16*RT
// down rows, wave w takes row tile w % RT and K slice w / RT of ff. With one K slice (RT = 4,
// ff up to 640) every wave owns whole rows and stores them from registers; otherwise the slices
// are summed through LDS like gate/up, a quarter of the outputs per wave. Either way every wave
// issues at least one store per item, which the ring waits count.
// dn_items is the item loop for K slices of NB blocks (NB = ceil(blocks / KS), one instantiation
// per split the kernel can choose), once the plan has given the workgroup its items [i0, i1) and
// the row tiles per virtual expert.
template <int NB>
__device__ __forceinline__ void dn_items(
    Meta &meta, int (&s_pid)[2][kCols], uint8_t *smem, const IdsLds &il, int32_t *lds_list,
    bool fused, int P, int H, int F, int tiles, int i0, int i1, int a_first, int na, int nbuf,
    int ring_bytes, const float *__restrict__ h, float *__restrict__ ypair) {
    const int rb = F / kBlockWeights * kBlockBytes;
    const int rows = H / tiles, tile_bytes = rows * rb, RT = rows / 16;
    uint8_t *wb = smem;                                                // [nbuf][rows]
    float *red = reinterpret_cast<float *>(smem + ring_bytes);         // [2][wave][col][16 rows]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int rt = wave % RT, ks = wave / RT, KS = kWaves / RT;
    const int nblk = F / kBlockWeights, blk0 = ks * NB;
    const int n_inst = stage_async_count<kThreads>(tile_bytes);
    int ia = 0, it = i0 - a_first * tiles, is = 0;   // stream cursor
    auto issue_next = [&]() {
        stage_async<kThreads>(wb + is * tile_bytes, meta.pa[ia] + (int64_t)it * tile_bytes,
                              tile_bytes);
        asm volatile("" ::: "memory");   // later stores stay behind these loads (ring waits)
        if (++it == tiles) { it = 0; ++ia; }
        if (++is == nbuf) is = 0;
    };
    // output u = (token column u / rows, row u % rows of the item) sums the KS slices of its row
    // tile; wave w takes the quarter u in [w Q, (w + 1) Q), Q = rows mt / 4 >= 4
    // (sd: the expert's second-level down scale)
    auto reduce = [&](const float *rp, const int *pids, int t, int mt, float sd) {
        const int Q = rows * mt / kWaves;
        for (int l = lane; l < Q; l += 64) {
            const int u = wave * Q + l, r = u % rows, nn = u / rows;
            float v = 0.f;
            for (int s2 = 0; s2 < KS; s2++)
                v += rp[((s2 * RT + r / 16) * kCols + nn) * 16 + r % 16];
            ypair[(int64_t)pids[nn] * H + t * rows + r] = v * sd;
        }
    };

    u32x4_t hh[NB][2], hl[NB][2];
    int hs = 0, cur_a = -1;
    int pid_n = 0;   // pair id of token column n of the current virtual expert (its ypair row)
    const float *h_row = nullptr;
    auto locate_h = [&](int a_) {   // h row and pair id of column n of virtual expert a_
        const bool in = n < meta.m[a_];
        h_row = in ? h + (int64_t)(meta.q0[a_] + n) * F : nullptr;
        pid_n = in ? meta.pid[a_][n] : 0;
        cur_a = a_;
    };
    // the h rows of the first item (their CSR slots are known from phase A) are loaded with the
    // first tile, before the rest of the ring; the fused plan's phase B (pair lists, for the
    // output rows) runs while they stream in
    h_row = n < meta.m[0] ? h + (int64_t)(meta.q0[0] + n) * F : nullptr;
    fetch_h_operands<NB>(hh, hl, h_row, blk0, nblk, q);
    issue_next();
    if (fused) plan_ids_b(meta, il, lds_list, P, tiles, i0, i1, a_first, na, nullptr, nullptr);
    locate_h(0);
    hs = convert_h_operands<NB>(hh, hl, blk0, nblk);

    int p_t = 0, p_mt = 0;
    float p_sd = 1.f;
    int a = 0, t = i0 - a_first * tiles, slot = 0, issued = i0 + 1;
    for (int i = i0; i < i1; i++) {
        const int mt = meta.m[a], u = i - i0;
        const float sd = meta.s2a[a];
        const uint8_t *wt = wb + slot * tile_bytes + (rt * 16 + n) * rb;
        // every buffer in flight (the rest of the ring, on the first item; filling it here
        // rather than before the loop keeps the h operands in registers: with a separate loop
        // the register allocator spilled them around it)
        for (; issued < min(i + nbuf, i1); issued++) issue_next();
        if (a != cur_a) {
            locate_h(a);
            fetch_h_operands<NB>(hh, hl, h_row, blk0, nblk, q);
            hs = convert_h_operands<NB>(hh, hl, blk0, nblk);
        }
        // tile i landed: issued after it are the tiles behind it and one store per wave and item
        // (from item 1 on with KS > 1; a lower bound with two stores)
        vm_wait_le(min(nbuf - 1, i1 - 1 - i) * n_inst +
                   (KS == 1 ? min(nbuf, u) : max(0, min(nbuf, u - 1))));
        lds_barrier();
        if (KS > 1 && wave == 0 && lane < kCols) s_pid[u & 1][lane] = pid_n;
        SliceA<NB> sa;
        read_slice<NB>(wt, blk0, nblk, q, sa);
        if (i + nbuf < i1) {
            lds_barrier();   // tile i is in every wave's registers: refill its buffer
            issue_next();
            issued++;
        }
        if (KS > 1 && u > 0)
            reduce(red + ((u - 1) & 1) * kRedFloats, s_pid[(u - 1) & 1], p_t, p_mt, p_sd);
        // hi and lo parts accumulate in two independent chains (half the dependent latency)
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acl = acc;
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const f16x2_t S = scale_f16x2(sa.s[j]);
            const f16x8_t a0 = dequant8(sa.c[j][0], S), a1 = dequant8(sa.c[j][1], S);
            acc = mfma16(a0, __builtin_bit_cast(f16x8_t, hh[j][0]), acc);
            acl = mfma16(a0, __builtin_bit_cast(f16x8_t, hl[j][0]), acl);
            acc = mfma16(a1, __builtin_bit_cast(f16x8_t, hh[j][1]), acc);
            acl = mfma16(a1, __builtin_bit_cast(f16x8_t, hl[j][1]), acl);
        }
        acc = unscale(acc + acl, hs);
        if (KS == 1) {   // whole rows: lane holds rows 4q..4q+3 of token column n
            if (n < mt)
                *reinterpret_cast<f32x4_t *>(ypair + (int64_t)pid_n * H + t * rows + rt * 16 +
                                             4 * q) = acc * sd;
        } else {
            *reinterpret_cast<f32x4_t *>(red + (u & 1) * kRedFloats + (wave * kCols + n) * 16 +
                                         4 * q) = acc;
        }
        p_t = t;
        p_mt = mt;
        p_sd = sd;
        if (++t == tiles) { t = 0; ++a; }
        if (++slot == nbuf) slot = 0;
    }
    if (KS > 1) {
        const int u = i1 - i0;
        lds_barrier();
        reduce(red + ((u - 1) & 1) * kRedFloats, s_pid[(u - 1) & 1], p_t, p_mt, p_sd);
    }
}

template <int NB>
__global__ __launch_bounds__(kThreads, 2) void dn_decode_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ pair_ids,
    const int32_t *__restrict__ active, const int32_t *__restrict__ counts,
    const uint8_t *__restrict__ down, int64_t down_stride,
    const uint8_t *const *__restrict__ down_tab, const float *__restrict__ down_s2,
    int32_t P, int32_t E, int32_t H, int32_t F, int32_t ks_min, int32_t nbuf,
    int32_t ring_bytes,
    const float *__restrict__ h, float *__restrict__ ypair, const int32_t *__restrict__ ids,
    int32_t expert_base) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ Meta meta;
    __shared__ int s_pid[2][kCols];   // pair ids of the token columns of the last two items
    const int nblk = F / kBlockWeights;

    // fused layer: the plan from the routed ids, the pair list and the plan's late scratch in
    // LDS behind the partials
    const bool fused = ids != nullptr;
    int32_t *lds_list = reinterpret_cast<int32_t *>(smem + ring_bytes + kRedBytes);
    const IdsLds il = ids_lds(smem, lds_list + P, E, P);

    // the K split (and with it the row tiles per virtual expert) is the plan's
    const DnSplit sp{ks_min, nblk, H};
    int tiles = 0, i0, i1, a_first, na = 0;
    if (fused)
        plan_ids_a(meta, il, ids, expert_base, down, down_stride, down_tab, down_s2, nullptr, 0,
                   nullptr, nullptr, E, P, sp, tiles, i0, i1, a_first, na);
    else
        load_plan(meta, reinterpret_cast<int32_t *>(smem), counts, active, offsets, pair_ids, down,
                  down_stride, down_tab, down_s2, nullptr, 0, nullptr, nullptr, E, P, sp, tiles,
                  i0, i1, a_first);
    // workgroup-uniform: kept in scalar registers
    tiles = __builtin_amdgcn_readfirstlane(tiles);
    i0 = __builtin_amdgcn_readfirstlane(i0);
    i1 = __builtin_amdgcn_readfirstlane(i1);
    a_first = __builtin_amdgcn_readfirstlane(a_first);
    na = __builtin_amdgcn_readfirstlane(na);
    if (i0 >= i1) return;
    // slice width for the chosen split: NB at ks_min, halved (rounded up) per doubling
    const int KS = kWaves * 16 * tiles / H, nbs = (nblk + KS - 1) / KS;
    constexpr int NB2 = (NB + 1) / 2, NB4 = (NB + 3) / 4;
    if (nbs == NB)
        dn_items<NB>(meta, s_pid, smem, il, lds_list, fused, P, H, F, tiles, i0, i1, a_first, na,
                     nbuf, ring_bytes, h, ypair);
    else if (nbs == NB2)
        dn_items<NB2>(meta, s_pid, smem, il, lds_list, fused, P, H, F, tiles, i0, i1, a_first, na,
                      nbuf, ring_bytes, h, ypair);
    else if (nbs == NB4)
        dn_items<NB4>(meta, s_pid, smem, il, lds_list, fused, P, H, F, tiles, i0, i1, a_first, na,
                      nbuf, ring_bytes, h, ypair);
}

// One thread per 4 consecutive outputs of a token row; the grid's y dimension steps over the
// tokens (it is capped on the host, so any T launches).
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float *__restrict__ w, const int32_t *__restrict__ pos,
    const int32_t *__restrict__ n_local_ptr, const float *__restrict__ ypair, int32_t T, int32_t k,
    int32_t H, float *__restrict__ y) {
    constexpr int kJ = 16;  // slots whose loads are issued together (one round trip for k <= 16)
    const int r = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (r >= H) return;
    const int n_local = *n_local_ptr;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += kJ) {
            int q[kJ];
            float wt[kJ];
            f32x4_t v[kJ];
#pragma unroll
            for (int u = 0; u < kJ; u++) {
                const int64_t p = (int64_t)t * k + j0 + u;
                const bool in = j0 + u < k;
                q[u] = in ? pos[p] : n_local;
                wt[u] = in ? w[p] : 0.f;
                // rows of non-local slots hold stale data; they are loaded and then skipped.
                // Streaming loads and stores: ypair is read once, y written once (measured 1-2%
                // off the prefill layers, whose ypair is hundreds of MB)
                v[u] = in ? __builtin_nontemporal_load(
                                reinterpret_cast<const f32x4_t *>(ypair + p * H + r))
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
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4_t *>(y + (int64_t)t * H + r));
    }
}

struct DecodeWs {
    int32_t *pos;       // [P]
    int32_t *n_local;   // [1] local pairs (fused layer: written by the gate/up kernel)
    float *h;           // [P][F]
    float *ypair;       // [P][H]
};

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

DecodeWs carve(void *ws, int32_t P, int32_t H, int32_t F) {
    uint8_t *b = static_cast<uint8_t *>(ws);
    DecodeWs d;
    d.pos = reinterpret_cast<int32_t *>(b);
    b += align256(sizeof(int32_t) * (size_t)P);
    d.n_local = reinterpret_cast<int32_t *>(b);
    b += 256;
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
    return align256(sizeof(int32_t) * P) + 256 + align256(sizeof(float) * P * F) +
           align256(sizeof(float) * P * H);
}

int launch_combine(const float *w, const int32_t *pos, const int32_t *n_local, const float *ypair,
                   int32_t T, int32_t k, int32_t H, float *y, hipStream_t s) {
    // grid.y is limited to 65535: tokens beyond it are looped over inside the kernel
    dim3 grid((H / 4 + kThreads - 1) / kThreads, std::min<int32_t>(T, 32768));
    prof_start(MOE_KERNEL_COMBINE, s);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, s, w, pos, n_local, ypair, T, k,
                       H, y);
    prof_stop(MOE_KERNEL_COMBINE, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

namespace {

constexpr size_t kLds = 160 * 1024;
constexpr int kMaxBuf = 6;

// Virtual experts that one workgroup's contiguous item range can touch (its range lies within its
// slot's).
int64_t max_experts(int64_t n_items, int64_t tiles, int grid) {
    const int slots = paired_grid(grid) ? grid / 2 : grid;
    const int64_t per = (n_items + slots - 1) / slots;
    return (per - 1) / tiles + 2;
}

// Two workgroups per CU with two tile buffers each when the LDS holds them (both in flight while
// a tile is computed from registers: measured as fast as three, the streaming rate being set
// elsewhere), else two with one buffer each, else one with as many as fit (at most kMaxBuf).
// The ring region also holds the start-up scratch, so it is at least that large; `extra` bytes
// (the fused layer's pair list and late plan scratch) follow the partials. Returns the dynamic
// LDS bytes (0: does not fit).
size_t ring_plan(size_t tile, size_t scratch, size_t extra, int &nbuf, int &ring_bytes,
                 int &wgs) {
    const size_t fixed = kRedBytes + sizeof(Meta) + extra;
    const size_t scr = (scratch + 15) & ~size_t(15);
    if (2 * (std::max(2 * tile, scr) + fixed) <= kLds) {
        nbuf = 2;
        wgs = 2;
    } else if (2 * (std::max(tile, scr) + fixed) <= kLds) {
        // wide tiles (hidden 4096: 37 KB): two workgroups of one buffer each, the tile in flight
        // while the last one is computed from registers, measured 25% faster than one
        // workgroup per CU with four (skewed prefill T=512, gate/up 406 -> 307 us)
        nbuf = 1;
        wgs = 2;
    } else {
        if (kLds < fixed + 2 * tile) return 0;
        nbuf = (int)std::min<size_t>(kMaxBuf, (kLds - fixed) / tile);
        wgs = 1;
    }
    const size_t ring = std::max(nbuf * tile, scr);
    if (ring + fixed > kLds) return 0;
    ring_bytes = (int)ring;
    return ring + kRedBytes + extra;
}

// Everything the two decode launches need, settled on the host before either is enqueued.
struct DecodeCfg {
    int nb_gu, nb_dn, rt, ks_min;
    bool fused, tokcols;
    int gu_nbuf, gu_ring, gu_grid, dn_nbuf, dn_ring, dn_grid;
    size_t gu_lds, dn_lds;
};

// Gate/up: the four waves split hidden into slices of NB = ceil(blocks / 4) NVFP4 blocks.
// Down: the smallest K split KS in {1, 2, 4} with at most kMaxDnBlocks blocks per slice, and
// RT = 4 / KS row tiles per item; H must hold whole items, and two tiles plus the start-up
// scratch must fit in LDS. fused: the plan is built from the routed ids (a.ids).
// That KS is the smallest the down kernel takes; it raises it on the device for a union of few
// experts (dn_ks).
int decode_plan(const FfnArgs &a, bool fused, DecodeCfg &c) {
    const int bh = a.H / kBlockWeights, bf = a.F / kBlockWeights;
    const int32_t P = a.T * a.k;
    const int max_v = max_virtual(a.E, P);   // items: virtual experts x row tiles
    c.nb_gu = (bh + kWaves - 1) / kWaves;
    int ks = 1;
    while (ks < kWaves && (bf + ks - 1) / ks > kMaxDnBlocks) ks *= 2;
    // the split the kernel would take for the most virtual experts the routing can make is the
    // least it can take (dn_ks falls with the count): start there, in the narrowest kernel
    ks = dn_ks(DnSplit{ks, bf, a.H}, max_v);
    c.ks_min = ks;
    c.nb_dn = (bf + ks - 1) / ks;
    c.rt = kWaves / ks;   // the most row tiles per item: the LDS tile size
    if (c.nb_gu > kMaxGuBlocks || c.nb_dn > kMaxDnBlocks || a.H % (16 * c.rt)) return MOE_ESHAPE;
    if (fused && (P > kIdsMaxPairs || a.E > kIdsMaxExperts)) return MOE_ESHAPE;
    c.fused = fused;
    // token columns when most tokens hit each active expert (dense routing, e.g. a shared
    // expert): every workgroup then loads all T token rows, which costs more than it saves when
    // an expert holds only a pair or two (measured: tiny decode, the verify chunk, E256 T=16)
    c.tokcols = a.T <= kCols && 2 * (int64_t)P >= (int64_t)a.T * std::min<int64_t>(a.E, P);
    const size_t scratch = fused ? ids_early_bytes(a.E, P) : plan_scratch_bytes(a.E, P);
    const size_t extra = fused ? sizeof(int32_t) * (size_t)P + ids_late_bytes(a.E, P) : 0;
    int wgs;
    c.gu_lds = ring_plan(2 * kGuO * (size_t)gu_pitch((int)row_bytes(a.H)), scratch, extra,
                         c.gu_nbuf, c.gu_ring, wgs);
    if (!c.gu_lds) return MOE_ESHAPE;
    const int gu_tiles = a.F / kGuO;
    c.gu_grid = (int)std::min<int64_t>(wgs * kCUs, (int64_t)max_v * gu_tiles);
    if (max_experts((int64_t)max_v * gu_tiles, gu_tiles, c.gu_grid) > kMaxMeta)
        return MOE_ESHAPE;
    const int rows = 16 * c.rt;
    c.dn_lds = ring_plan(rows * (size_t)row_bytes(a.F), scratch, extra, c.dn_nbuf, c.dn_ring, wgs);
    if (!c.dn_lds) return MOE_ESHAPE;
    // the kernel splits K from ks_min up to ks_max (one virtual expert): the grid is sized for
    // the finest items, and every split keeps a workgroup's experts within kMaxMeta
    const DnSplit sp{c.ks_min, bf, a.H};
    const int ks_max = dn_ks(sp, 1);
    c.dn_grid = (int)std::min<int64_t>(wgs * kCUs, (int64_t)max_v * (a.H * ks_max / 64));
    for (int kk = c.ks_min; kk <= ks_max; kk *= 2) {
        const int dn_tiles = a.H * kk / 64;
        if (max_experts((int64_t)max_v * dn_tiles, dn_tiles, c.dn_grid) > kMaxMeta)
            return MOE_ESHAPE;
    }
    return MOE_OK;
}

template <int NB>
int launch_gu(const FfnArgs &a, const DecodeWs &d, const DecodeCfg &c, hipStream_t s) {
    auto kern = gu_decode_kernel<NB>;
    static bool attr = false;
    if (!attr) {
        if (!set_lds_attr(reinterpret_cast<const void *>(kern), kLds)) return MOE_ELAUNCH;
        attr = true;
    }
    prof_start(MOE_KERNEL_GU_DECODE, s);
    hipLaunchKernelGGL(kern, dim3(c.gu_grid), dim3(kThreads), c.gu_lds, s, a.x, a.offsets,
                       a.pair_ids, a.active, a.counts, a.gate.base, a.gate.expert_stride,
                       a.gate.experts, a.up.base, a.up.expert_stride, a.up.experts, a.gate.scale2,
                       a.up.scale2, a.k, a.T * a.k, a.E, a.H, a.F, c.gu_nbuf, c.gu_ring, d.h, d.pos,
                       a.ids, a.expert_base, a.T, c.tokcols ? 1 : 0, d.n_local);
    prof_stop(MOE_KERNEL_GU_DECODE, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

template <int NB>
int launch_dn(const FfnArgs &a, const DecodeWs &d, const DecodeCfg &c, hipStream_t s) {
    auto kern = dn_decode_kernel<NB>;
    static bool attr = false;
    if (!attr) {
        if (!set_lds_attr(reinterpret_cast<const void *>(kern), kLds)) return MOE_ELAUNCH;
        attr = true;
    }
    prof_start(MOE_KERNEL_DN_DECODE, s);
    hipLaunchKernelGGL(kern, dim3(c.dn_grid), dim3(kThreads), c.dn_lds, s, a.offsets, a.pair_ids,
                       a.active, a.counts, a.down.base, a.down.expert_stride, a.down.experts,
                       a.down.scale2, a.T * a.k, a.E, a.H, a.F, c.ks_min, c.dn_nbuf, c.dn_ring, d.h,
                       d.ypair, a.ids, a.expert_base);
    prof_stop(MOE_KERNEL_DN_DECODE, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

int run_decode(const FfnArgs &a, const DecodeCfg &c, hipStream_t s) {
    const DecodeWs d = carve(a.ws, a.T * a.k, a.H, a.F);
    int st = MOE_OK;
    switch (c.nb_gu) {
#define MOE_GU(nb) case nb: st = launch_gu<nb>(a, d, c, s); break;
        MOE_GU(1) MOE_GU(2) MOE_GU(3) MOE_GU(4) MOE_GU(5) MOE_GU(6) MOE_GU(7) MOE_GU(8)
        MOE_GU(9) MOE_GU(10) MOE_GU(11) MOE_GU(12) MOE_GU(13) MOE_GU(14) MOE_GU(15) MOE_GU(16)
#undef MOE_GU
    default: return MOE_ESHAPE;
    }
    if (st != MOE_OK) return st;
    switch (c.nb_dn) {
#define MOE_DN(nb) case nb: st = launch_dn<nb>(a, d, c, s); break;
        MOE_DN(1) MOE_DN(2) MOE_DN(3) MOE_DN(4) MOE_DN(5)
        MOE_DN(6) MOE_DN(7) MOE_DN(8) MOE_DN(9) MOE_DN(10)
#undef MOE_DN
    default: return MOE_ESHAPE;
    }
    if (st != MOE_OK) return st;
    return launch_combine(a.w, d.pos, c.fused ? d.n_local : a.offsets + a.E, d.ypair, a.T, a.k,
                          a.H, a.y, s);
}

}  // namespace

bool decode_supported(const FfnArgs &a) {
    DecodeCfg c;
    return decode_plan(a, false, c) == MOE_OK;
}

bool decode_fused_supported(const FfnArgs &a) {
    DecodeCfg c;
    return decode_plan(a, true, c) == MOE_OK;
}

int launch_decode(const FfnArgs &a, hipStream_t s) {
    DecodeCfg c;
    if (int st = decode_plan(a, a.ids != nullptr, c)) return st;
    return run_decode(a, c, s);
}

}  // namespace moe
