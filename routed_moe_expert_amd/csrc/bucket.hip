// Expert-first bucketing of routed (token, expert) pairs into a stable CSR.
//
// Computes what moe_sk_repro.rs's host bucketing computes (pairs pushed into per-expert lists in
// ascending pair id, non-empty lists concatenated in ascending expert id, running-total offsets),
// on the GPU with workgroups of 8 wave64s. Up to kSingleMax pairs, one workgroup does it all:
//   1. LDS histogram of the local expert ids (non-local pairs counted in an extra bucket E);
//   2. workgroup exclusive scans of the counts (offsets, cursors) and of the non-empty flags
//      (the ascending active list);
//   3. a stable scatter in chunks of 512 consecutive pairs. Inside a wave, each lane ORs its bit
//      into a per-wave 64-bit mask kept in LDS for its key; the mask's population below the lane
//      is the lane's rank among equal keys (constant time, however many distinct keys). Across
//      the 8 waves of a chunk the per-wave key counts give each wave its start; the cursors then
//      advance by the chunk's counts.
// More pairs are split into at most kMaxChunks contiguous chunks, one workgroup each, in three
// launches: per-chunk histograms (to the workspace); one workgroup turning them into each
// (chunk, key)'s first position -- an exclusive scan over chunks per key plus the key's offset --
// with the offsets, active list and counts; then per-chunk stable scatters (step 3) from those
// positions. Chunks are in pair order, so the result is the same.
// The result depends only on the ids, so it is bit-exact and run-to-run identical.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kSingleMax = 4096;   // pairs bucketed by one workgroup
constexpr int kMaxChunks = 256;    // workgroups of the chunked form

// Pairs per chunk of the chunked form: a multiple of the 512-pair scatter step, at most
// kMaxChunks chunks.
inline int chunk_pairs(int64_t P) {
    int64_t c = (P + kMaxChunks - 1) / kMaxChunks;
    c = (c + kThreads - 1) / kThreads * kThreads;
    return (int)std::max<int64_t>(c, 4 * kThreads);
}

// Exclusive scan of one int per thread over the workgroup; *total gets the sum.
__device__ int block_exclusive_scan(int v, int *wsum, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    lds_barrier();
    if (wave == 0) {
        int s = lane < kWaves ? wsum[lane] : 0;
#pragma unroll
        for (int d = 1; d < kWaves; d <<= 1) {
            int y = __shfl_up(s, d, 64);
            if (lane >= d) s += y;
        }
        if (lane < kWaves) wsum[lane] = s;
    }
    lds_barrier();
    int before = wave ? wsum[wave - 1] : 0;
    *total = wsum[kWaves - 1];
    lds_barrier();
    return before + x - v;
}

// Bucket of pair p: its local expert, or E when not local.
__device__ __forceinline__ int key_of(const int32_t *ids, int p, int E, int expert_base) {
    const int64_t e = (int64_t)ids[p] - expert_base;
    return (e >= 0 && e < E) ? (int)e : E;
}

// LDS of the scatter: per-wave 64-bit lane masks [kWaves][NB][2] and per-wave key counts
// [kWaves][NB], both zero on entry and on exit.
struct ScatterLds {
    uint32_t *tbl;
    uint8_t *wcnt;
};

__device__ void zero_scatter_lds(ScatterLds sl, int NB) {
    for (int i = threadIdx.x; i < 2 * kWaves * NB; i += kThreads) sl.tbl[i] = 0;
    uint32_t *wcnt32 = reinterpret_cast<uint32_t *>(sl.wcnt);   // kWaves*NB is a multiple of 4
    for (int i = threadIdx.x; i < kWaves * NB / 4; i += kThreads) wcnt32[i] = 0;
}

// One step of the stable scatter: the workgroup's 512 consecutive pairs, thread t holding pair
// p = (first pair) + t with bucket key (-1: no pair). cur[key] holds the next free CSR position of
// each key and is advanced past the step's pairs.
__device__ void scatter_step(int key, int p, int E, int32_t *cur, ScatterLds sl,
                             int32_t *__restrict__ pair_ids) {
    const int NB = E + 1, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t *my_tbl = sl.tbl + 2 * wave * NB;
    if (key >= 0) atomicOr(&my_tbl[2 * key + (lane >> 5)], 1u << (lane & 31));
    // the wave's own LDS operations complete in order; wait for them before reading back
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    int rank = 0, gsize = 0;
    if (key >= 0) {
        const uint64_t m = (uint64_t)my_tbl[2 * key] | ((uint64_t)my_tbl[2 * key + 1] << 32);
        rank = __popcll(m & lanes_below);
        gsize = __popcll(m);
    }
    if (key >= 0 && rank == 0) sl.wcnt[wave * NB + key] = (uint8_t)gsize;
    lds_barrier();
    if (key >= 0) {
        int pos = cur[key] + rank;
        for (int w2 = 0; w2 < wave; w2++) pos += sl.wcnt[w2 * NB + key];
        pair_ids[pos] = p;
    }
    lds_barrier();
    if (key >= 0 && rank == 0) {
        atomicAdd(&cur[key], gsize);
        sl.wcnt[wave * NB + key] = 0;
        my_tbl[2 * key] = 0;
        my_tbl[2 * key + 1] = 0;
    }
    lds_barrier();
}

// Stable scatter of pairs [p0, p1) (cur[] as in scatter_step).
__device__ void scatter_range(const int32_t *__restrict__ ids, int p0, int p1, int E,
                              int expert_base, int32_t *cur, ScatterLds sl,
                              int32_t *__restrict__ pair_ids) {
    for (int c0 = p0; c0 < p1; c0 += kThreads) {
        const int p = c0 + threadIdx.x;
        scatter_step(p < p1 ? key_of(ids, p, E, expert_base) : -1, p, E, cur, sl, pair_ids);
    }
}

// offsets, active list and counts from the per-key totals tot[] (LDS); tot[] is replaced by the
// keys' first positions.
__device__ void write_csr_head(int32_t *tot, int E, int *wsum, int32_t *__restrict__ offsets,
                               int32_t *__restrict__ active, int32_t *__restrict__ counts) {
    const int NB = E + 1, tid = threadIdx.x;
    // each thread owns a contiguous run of buckets
    const int per = (NB + kThreads - 1) / kThreads;
    const int lo = min(tid * per, NB), hi = min(lo + per, NB);
    int my_cnt = 0, my_flags = 0;
    for (int i = lo; i < hi; i++) {
        my_cnt += tot[i];
        my_flags += (i < E && tot[i] > 0);
    }
    int tot_cnt, tot_flags;
    int run = block_exclusive_scan(my_cnt, wsum, &tot_cnt);
    int fl = block_exclusive_scan(my_flags, wsum, &tot_flags);
    for (int i = lo; i < hi; i++) {
        const int c = tot[i];
        offsets[i] = run;  // i == E writes offsets[E] = number of local pairs
        if (i < E && c > 0) active[fl++] = i;
        if (i == E) counts[1] = c;
        tot[i] = run;
        run += c;
    }
    if (tid == 0) counts[0] = tot_flags;
    lds_barrier();
}

// LDS layout shared by the kernels that scatter: counts/cursors [NB], scan scratch [32], then the
// scatter tables.
inline size_t scatter_kernel_lds(int E) {
    const int NB = E + 1;
    return sizeof(int32_t) * (NB + 32) + sizeof(uint32_t) * 2 * kWaves * NB + (size_t)kWaves * NB;
}

__device__ void carve(int E, int32_t *&cnt, int *&wsum, ScatterLds &sl) {
    extern __shared__ __attribute__((aligned(16))) int32_t smem[];
    const int NB = E + 1;
    cnt = smem;
    wsum = cnt + NB;
    sl.tbl = reinterpret_cast<uint32_t *>(wsum + 32);
    sl.wcnt = reinterpret_cast<uint8_t *>(sl.tbl + 2 * kWaves * NB);
}

// One workgroup, all P pairs.
__global__ __launch_bounds__(kThreads) void bucket_kernel(
    const int32_t *__restrict__ ids, int32_t P, int32_t E, int32_t expert_base,
    int32_t *__restrict__ offsets, int32_t *__restrict__ pair_ids, int32_t *__restrict__ active,
    int32_t *__restrict__ counts) {
    int32_t *cnt;
    int *wsum;
    ScatterLds sl;
    carve(E, cnt, wsum, sl);
    const int NB = E + 1;
    // thread t holds the keys of pairs u * 512 + t, all loaded before any is used (one memory
    // round trip; past P the load reads offsets[0], always valid, and the key is -1)
    constexpr int kKeys = kSingleMax / kThreads;
    int key[kKeys];
#pragma unroll
    for (int u = 0; u < kKeys; u++) {
        const int p = u * kThreads + threadIdx.x;
        key[u] = *(p < P ? ids + p : offsets);
    }
#pragma unroll
    for (int u = 0; u < kKeys; u++) {
        const int64_t e = (int64_t)key[u] - expert_base;
        key[u] = u * kThreads + (int)threadIdx.x < P ? ((e >= 0 && e < E) ? (int)e : E) : -1;
    }
    for (int i = threadIdx.x; i < NB; i += kThreads) cnt[i] = 0;
    zero_scatter_lds(sl, NB);
    lds_barrier();
#pragma unroll
    for (int u = 0; u < kKeys; u++)
        if (key[u] >= 0) atomicAdd(&cnt[key[u]], 1);
    lds_barrier();
    write_csr_head(cnt, E, wsum, offsets, active, counts);
#pragma unroll
    for (int u = 0; u < kKeys; u++)
        if (u * kThreads < P) scatter_step(key[u], u * kThreads + threadIdx.x, E, cnt, sl, pair_ids);
}

// Chunked form, step 1: the histogram of chunk blockIdx.x into hist[chunk][NB].
__global__ __launch_bounds__(kThreads) void bucket_hist_kernel(
    const int32_t *__restrict__ ids, int32_t P, int32_t E, int32_t expert_base, int32_t chunk,
    int32_t *__restrict__ hist) {
    extern __shared__ __attribute__((aligned(16))) int32_t smem[];
    const int NB = E + 1;
    int32_t *cnt = smem;
    for (int i = threadIdx.x; i < NB; i += kThreads) cnt[i] = 0;
    lds_barrier();
    const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
    for (int p = p0 + threadIdx.x; p < p1; p += kThreads)
        atomicAdd(&cnt[key_of(ids, p, E, expert_base)], 1);
    lds_barrier();
    for (int i = threadIdx.x; i < NB; i += kThreads) hist[(int64_t)blockIdx.x * NB + i] = cnt[i];
}

// Step 2 (one workgroup): hist[c][key] becomes the first CSR position of chunk c's pairs of that
// key; also offsets, the active list and the counts.
__global__ __launch_bounds__(kThreads) void bucket_scan_kernel(
    int32_t E, int32_t n_chunks, int32_t *__restrict__ hist, int32_t *__restrict__ offsets,
    int32_t *__restrict__ active, int32_t *__restrict__ counts) {
    extern __shared__ __attribute__((aligned(16))) int32_t smem[];
    const int NB = E + 1;
    int32_t *tot = smem;
    int *wsum = tot + NB;
    // the chunks' counts are read kBatch at a time with independent loads (one round trip per
    // batch; read, write and read again one chunk after another, they took a round trip each)
    constexpr int kBatch = 16;
    for (int key = threadIdx.x; key < NB; key += kThreads) {
        int run = 0;
        for (int c0 = 0; c0 < n_chunks; c0 += kBatch) {
#pragma unroll
            for (int u = 0; u < kBatch; u++)
                run += c0 + u < n_chunks ? hist[(int64_t)(c0 + u) * NB + key] : 0;
        }
        tot[key] = run;
    }
    lds_barrier();
    write_csr_head(tot, E, wsum, offsets, active, counts);   // tot[key]: the key's first slot
    // each (chunk, key) count becomes the chunk's first slot for the key
    for (int key = threadIdx.x; key < NB; key += kThreads) {
        int run = tot[key];
        for (int c0 = 0; c0 < n_chunks; c0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; u++)
                v[u] = c0 + u < n_chunks ? hist[(int64_t)(c0 + u) * NB + key] : 0;
#pragma unroll
            for (int u = 0; u < kBatch; u++)
                if (c0 + u < n_chunks) {
                    hist[(int64_t)(c0 + u) * NB + key] = run;
                    run += v[u];
                }
        }
    }
}

// Step 3: the stable scatter of chunk blockIdx.x from its first positions.
__global__ __launch_bounds__(kThreads) void bucket_scatter_kernel(
    const int32_t *__restrict__ ids, int32_t P, int32_t E, int32_t expert_base, int32_t chunk,
    const int32_t *__restrict__ hist, int32_t *__restrict__ pair_ids) {
    int32_t *cur;
    int *wsum;
    ScatterLds sl;
    carve(E, cur, wsum, sl);
    const int NB = E + 1;
    for (int i = threadIdx.x; i < NB; i += kThreads) cur[i] = hist[(int64_t)blockIdx.x * NB + i];
    zero_scatter_lds(sl, NB);
    lds_barrier();
    const int p0 = blockIdx.x * chunk;
    scatter_range(ids, p0, min(P, p0 + chunk), E, expert_base, cur, sl, pair_ids);
}

bool set_max_lds(const void *fn, bool &done) {
    if (!done) {
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) !=
            hipSuccess)
            return false;
        done = true;
    }
    return true;
}

}  // namespace

size_t bucket_ws_bytes(int32_t T, int32_t k, int32_t E) {
    const int64_t P = (int64_t)T * k;
    if (P <= kSingleMax) return 0;
    const int64_t n_chunks = (P + chunk_pairs(P) - 1) / chunk_pairs(P);
    return (size_t)(n_chunks * (E + 1) * 4 + 255) / 256 * 256;
}

int launch_bucket(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t expert_base,
                  int32_t *offsets, int32_t *pair_ids, int32_t *active, int32_t *counts,
                  void *ws, hipStream_t s) {
    const int32_t P = T * k;
    const size_t lds = scatter_kernel_lds(E);
    static bool a0 = false, a1 = false;
    if (!set_max_lds(reinterpret_cast<const void *>(bucket_kernel), a0) ||
        !set_max_lds(reinterpret_cast<const void *>(bucket_scatter_kernel), a1))
        return MOE_ELAUNCH;
    prof_start(MOE_KERNEL_BUCKET, s);
    if (P <= kSingleMax) {
        hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kThreads), lds, s, ids, P, E, expert_base,
                           offsets, pair_ids, active, counts);
    } else {
        const int chunk = chunk_pairs(P), n_chunks = (P + chunk - 1) / chunk;
        int32_t *hist = static_cast<int32_t *>(ws);
        const size_t lds_nb = sizeof(int32_t) * (E + 1 + 32);
        hipLaunchKernelGGL(bucket_hist_kernel, dim3(n_chunks), dim3(kThreads), lds_nb, s, ids, P,
                           E, expert_base, chunk, hist);
        hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(kThreads), lds_nb, s, E, n_chunks,
                           hist, offsets, active, counts);
        hipLaunchKernelGGL(bucket_scatter_kernel, dim3(n_chunks), dim3(kThreads), lds, s, ids, P,
                           E, expert_base, chunk, (const int32_t *)hist, pair_ids);
    }
    prof_stop(MOE_KERNEL_BUCKET, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
