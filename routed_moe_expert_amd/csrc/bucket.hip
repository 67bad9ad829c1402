// Expert-first bucketing of routed (token, expert) pairs into a stable CSR.
//
// Computes what moe_sk_repro.rs's host bucketing computes (pairs pushed into per-expert lists in
// ascending pair id, non-empty lists concatenated in ascending expert id, running-total offsets),
// on the GPU, in one workgroup of 8 wave64s:
//   1. LDS histogram of the local expert ids (non-local pairs counted in an extra bucket E);
//   2. workgroup exclusive scans of the counts (offsets, cursors) and of the non-empty flags
//      (the ascending active list);
//   3. a stable scatter in chunks of 512 consecutive pairs. Inside a wave, each lane ORs its bit
//      into a per-wave 64-bit mask kept in LDS for its key; the mask's population below the lane
//      is the lane's rank among equal keys (constant time, however many distinct keys). Across
//      the 8 waves of a chunk the per-wave key counts give each wave its start; the cursors then
//      advance by the chunk's counts.
// The result depends only on the ids, so it is bit-exact and run-to-run identical.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

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

__global__ __launch_bounds__(kThreads) void bucket_kernel(
    const int32_t *__restrict__ ids, int32_t P, int32_t E, int32_t expert_base,
    int32_t *__restrict__ offsets, int32_t *__restrict__ pair_ids, int32_t *__restrict__ active,
    int32_t *__restrict__ counts) {
    extern __shared__ __attribute__((aligned(16))) int32_t smem[];
    const int NB = E + 1;                    // buckets 0..E-1 local experts, E = not local
    int32_t *cnt = smem;                     // [NB] counts, then cursors
    int32_t *wsum = cnt + NB;                // [32] scan scratch
    uint32_t *tbl = reinterpret_cast<uint32_t *>(wsum + 32);  // [kWaves][NB][2] lane masks
    uint8_t *wcnt = reinterpret_cast<uint8_t *>(tbl + 2 * kWaves * NB);  // [kWaves][NB]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    auto key_of = [&](int p) -> int {
        int64_t e = (int64_t)ids[p] - expert_base;
        return (e >= 0 && e < E) ? (int)e : E;
    };
    const int key0 = tid < P ? key_of(tid) : -1;  // the first chunk's keys stay in registers

    for (int i = tid; i < NB; i += kThreads) cnt[i] = 0;
    for (int i = tid; i < 2 * kWaves * NB; i += kThreads) tbl[i] = 0;
    uint32_t *wcnt32 = reinterpret_cast<uint32_t *>(wcnt);   // kWaves*NB is a multiple of 4
    for (int i = tid; i < kWaves * NB / 4; i += kThreads) wcnt32[i] = 0;
    lds_barrier();

    if (key0 >= 0) atomicAdd(&cnt[key0], 1);
    for (int p = tid + kThreads; p < P; p += kThreads) atomicAdd(&cnt[key_of(p)], 1);
    lds_barrier();

    // each thread owns a contiguous run of buckets
    const int per = (NB + kThreads - 1) / kThreads;
    const int lo = min(tid * per, NB), hi = min(lo + per, NB);
    int my_cnt = 0, my_flags = 0;
    for (int i = lo; i < hi; i++) {
        my_cnt += cnt[i];
        my_flags += (i < E && cnt[i] > 0);
    }
    int tot_cnt, tot_flags;
    int run = block_exclusive_scan(my_cnt, wsum, &tot_cnt);
    int fl = block_exclusive_scan(my_flags, wsum, &tot_flags);
    for (int i = lo; i < hi; i++) {
        int c = cnt[i];
        offsets[i] = run;  // i == E writes offsets[E] = number of local pairs
        if (i < E && c > 0) active[fl++] = i;
        if (i == E) counts[1] = c;
        cnt[i] = run;
        run += c;
    }
    if (tid == 0) counts[0] = tot_flags;
    lds_barrier();

    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t *my_tbl = tbl + 2 * wave * NB;
    for (int p0 = 0; p0 < P; p0 += kThreads) {
        const int p = p0 + tid;
        const int key = p0 == 0 ? key0 : (p < P ? key_of(p) : -1);
        if (key >= 0) atomicOr(&my_tbl[2 * key + (lane >> 5)], 1u << (lane & 31));
        // the wave's own LDS operations complete in order; wait for them before reading back
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        int rank = 0, gsize = 0;
        if (key >= 0) {
            const uint64_t m = (uint64_t)my_tbl[2 * key] | ((uint64_t)my_tbl[2 * key + 1] << 32);
            rank = __popcll(m & lanes_below);
            gsize = __popcll(m);
        }
        if (key >= 0 && rank == 0) wcnt[wave * NB + key] = (uint8_t)gsize;
        lds_barrier();
        if (key >= 0) {
            int pos = cnt[key] + rank;
            for (int w2 = 0; w2 < wave; w2++) pos += wcnt[w2 * NB + key];
            pair_ids[pos] = p;
        }
        lds_barrier();
        if (key >= 0 && rank == 0) {
            atomicAdd(&cnt[key], gsize);
            wcnt[wave * NB + key] = 0;
            my_tbl[2 * key] = 0;
            my_tbl[2 * key + 1] = 0;
        }
        lds_barrier();
    }
}

}  // namespace

int launch_bucket(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t expert_base,
                  int32_t *offsets, int32_t *pair_ids, int32_t *active, int32_t *counts,
                  hipStream_t s) {
    const int32_t P = T * k;
    const int NB = E + 1;
    const size_t lds = sizeof(int32_t) * (NB + 32) + sizeof(uint32_t) * 2 * kWaves * NB +
                       (size_t)kWaves * NB;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(bucket_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
            return MOE_ELAUNCH;
        attr_set = true;
    }
    prof_start(MOE_KERNEL_BUCKET, s);
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kThreads), lds, s, ids, P, E, expert_base,
                       offsets, pair_ids, active, counts);
    prof_stop(MOE_KERNEL_BUCKET, s);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
