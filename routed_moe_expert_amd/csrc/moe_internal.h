// Internal declarations shared by the HIP translation units of libmoe_nvfp4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kBlockWeights = 64;  // NVFP4: weights per block
constexpr int kBlockBytes = 36;    // NVFP4: 4 UE4M3 scale bytes + 32 code bytes

inline int64_t row_bytes(int64_t in_f) { return in_f / kBlockWeights * kBlockBytes; }
// K-step-packed banks (moe_kpack): rows per group, and bytes per expert of the packed copy
constexpr int kKpackRows = MOE_KPACK_ROWS;
constexpr int kSliceBytes = 32 * kBlockBytes;   // one 32-row slice of a packed K-step run
__host__ __device__ inline int64_t kpack_expert_bytes(int64_t out_f, int64_t in_f) {
    return (out_f + kKpackRows - 1) / kKpackRows * (in_f / kBlockWeights) * kKpackRows *
           kBlockBytes;
}

// SiLU(z) = z * sigmoid(z), with the hardware reciprocal (about 1 ulp) in place of a division.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

typedef __attribute__((address_space(3))) void lds_void_t;

// Asynchronous copy of `bytes` (a multiple of 16) from 16-byte aligned global memory into
// 16-byte aligned LDS with the gfx950 direct-to-LDS load (global_load_lds_dwordx4): wave w moves
// 64 consecutive 16-byte units per instruction, lane i landing at the wave's LDS base + 16*i, so
// no VGPRs are used and every load of the workgroup is in flight at once. Completion is awaited
// with vm_wait_le() followed by a workgroup barrier.
template <int kThreads>
__device__ __forceinline__ void stage_async(void *lds, const void *g, int bytes) {
    // the wave index is uniform: as a scalar, each instruction's LDS base is set up in SGPRs
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int units = bytes >> 4;
    const uint8_t *src = static_cast<const uint8_t *>(g);
    uint8_t *dst = static_cast<uint8_t *>(lds);
    for (int base = wave * 64; base < units; base += kThreads) {
        const int u = base + lane;
        if (u < units)
            __builtin_amdgcn_global_load_lds(src + (size_t)u * 16, (lds_void_t *)(dst + base * 16),
                                             16, 0, 0);
    }
}

// Workgroup barrier that orders LDS only: it waits for this wave's LDS (and scalar) operations
// and synchronizes the workgroup, but leaves global loads in flight. __syncthreads() carries a
// fence over global memory, for which the compiler waits for every outstanding vector-memory
// operation, and that would drain the prefetched tiles at each barrier. Kernels using this share
// data between waves through LDS only; data landed by direct-to-LDS loads is awaited first with
// vm_wait_le by every issuing wave.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Number of global_load_lds instructions one wave issues in stage_async for `bytes`.
template <int kThreads>
__device__ __forceinline__ int stage_async_count(int bytes) {
    const int units = bytes >> 4, first = (threadIdx.x >> 6) * 64;
    return units > first ? (units - first + kThreads - 1) / kThreads : 0;
}

// Wait until at most n vector-memory operations of this wave are outstanding (n wave-uniform).
// Vector memory loads complete in issue order, so this waits for everything issued before the n
// most recent ones. The counter holds 6 bits; larger n waits for all.
__device__ __forceinline__ void vm_wait_le(int n) {
    switch (__builtin_amdgcn_readfirstlane(n)) {   // a scalar branch, not per-lane compares
#define MOE_VMW(i) case i: asm volatile("s_waitcnt vmcnt(" #i ")" ::: "memory"); break;
        MOE_VMW(1) MOE_VMW(2) MOE_VMW(3) MOE_VMW(4) MOE_VMW(5) MOE_VMW(6) MOE_VMW(7) MOE_VMW(8)
        MOE_VMW(9) MOE_VMW(10) MOE_VMW(11) MOE_VMW(12) MOE_VMW(13) MOE_VMW(14) MOE_VMW(15)
        MOE_VMW(16) MOE_VMW(17) MOE_VMW(18) MOE_VMW(19) MOE_VMW(20) MOE_VMW(21) MOE_VMW(22)
        MOE_VMW(23) MOE_VMW(24) MOE_VMW(25) MOE_VMW(26) MOE_VMW(27) MOE_VMW(28) MOE_VMW(29)
        MOE_VMW(30) MOE_VMW(31) MOE_VMW(32) MOE_VMW(33) MOE_VMW(34) MOE_VMW(35) MOE_VMW(36)
        MOE_VMW(37) MOE_VMW(38) MOE_VMW(39) MOE_VMW(40) MOE_VMW(41) MOE_VMW(42) MOE_VMW(43)
        MOE_VMW(44) MOE_VMW(45) MOE_VMW(46) MOE_VMW(47) MOE_VMW(48) MOE_VMW(49) MOE_VMW(50)
        MOE_VMW(51) MOE_VMW(52) MOE_VMW(53) MOE_VMW(54) MOE_VMW(55) MOE_VMW(56) MOE_VMW(57)
        MOE_VMW(58) MOE_VMW(59) MOE_VMW(60) MOE_VMW(61) MOE_VMW(62) MOE_VMW(63)
#undef MOE_VMW
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

// ------------------------------------------------------------------- optional kernel timing
struct KernelProfile {
    int kernel = MOE_KERNEL_NONE;
    hipEvent_t *starts = nullptr;
    hipEvent_t *stops = nullptr;
    int n = 0;
    int next = 0;
};
extern KernelProfile g_profile;

inline void prof_start(int id, hipStream_t s) {
    if (g_profile.kernel == id && g_profile.next < g_profile.n)
        (void)hipEventRecord(g_profile.starts[g_profile.next], s);
}
inline void prof_stop(int id, hipStream_t s) {
    if (g_profile.kernel == id && g_profile.next < g_profile.n) {
        (void)hipEventRecord(g_profile.stops[g_profile.next], s);
        g_profile.next++;
    }
}

// ----------------------------------------------------------------------------- host launchers
// Each returns a MOE_* status; arguments have been validated by the ABI layer.

size_t bucket_ws_bytes(int32_t T, int32_t k, int32_t E);
int launch_bucket(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t expert_base,
                  int32_t *offsets, int32_t *pair_ids, int32_t *active, int32_t *counts,
                  void *ws, hipStream_t s);

struct FfnArgs {
    const uint16_t *x;
    const float *w;
    const int32_t *offsets, *pair_ids, *active, *counts;   // the CSR (null in the fused layer)
    moe_bank gate, up, down;
    int32_t T, k, E, H, F;
    float *y;
    void *ws;
    size_t ws_bytes;
    const int32_t *ids = nullptr;   // fused layer: the routed expert ids, bucketed in-kernel
    int32_t expert_base = 0;
};

size_t decode_ws_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F);
size_t prefill_ws_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t F);
bool decode_supported(const FfnArgs &a);         // shape within the decode kernels' limits
bool decode_fused_supported(const FfnArgs &a);   // ... and the in-kernel bucketing's
int launch_decode(const FfnArgs &a, hipStream_t s);
int launch_prefill(const FfnArgs &a, hipStream_t s);

int launch_kpack(const moe_bank &src, int32_t E, int32_t out_f, int32_t in_f, uint8_t *dst,
                 hipStream_t s);

int launch_router_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids,
                       float *w, hipStream_t s);

// y[t] = sum_j w[t,j] * ypair[t*k+j] over local slots; pos[p] >= *n_local means non-local.
int launch_combine(const float *w, const int32_t *pos, const int32_t *n_local, const float *ypair,
                   int32_t T, int32_t k, int32_t H, float *y, hipStream_t s);

}  // namespace moe
