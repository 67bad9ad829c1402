// The K-step-packed copy of a weight bank for the grouped-GEMM path (moe_kpack).
//
// A grouped-GEMM K step stages one 64-wide NVFP4 block of each of the weight tile's rows. In the
// row-major bank those are 36-byte pieces one row length apart, so each 12-byte direct-to-LDS
// load of a step touches a different row; in the packed copy the blocks of one K step of a group
// of kKpackRows rows are one contiguous run, which the same loads read front to back:
//     dst[e][g][b][r][0..35] = block b of row g * kKpackRows + r of expert e (zero past the rows).
// The bytes of each block are unchanged (four UE4M3 scales, then the E2M1 codes), so the packed
// copy is the same NVFP4 data in another order. It is written once, when the weights are loaded.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kPackThreads = 256;
constexpr int kBlockWords = kBlockBytes / 4;   // a block is 9 dwords, 4-byte aligned in a bank

// One dword of the copy per thread and grid step: dword d of expert e's packed rows is word w of
// block b of row r of group g, d = ((g * nb + b) * kKpackRows + r) * 9 + w.
__global__ __launch_bounds__(kPackThreads) void kpack_kernel(
    const uint8_t *__restrict__ base, int64_t stride, const uint8_t *const *__restrict__ tab,
    int32_t out_f, int32_t nb, int64_t words_per_expert, int64_t words,
    uint32_t *__restrict__ dst) {
    const int64_t rb = (int64_t)nb * kBlockBytes;
    for (int64_t d = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; d < words;
         d += (int64_t)gridDim.x * kPackThreads) {
        const int64_t e = d / words_per_expert;
        int64_t rest = d - e * words_per_expert;
        const int w = (int)(rest % kBlockWords);
        rest /= kBlockWords;
        const int r = (int)(rest % kKpackRows);
        rest /= kKpackRows;
        const int b = (int)(rest % nb);
        const int64_t row = rest / nb * kKpackRows + r;
        uint32_t v = 0;
        if (row < out_f) {
            const uint8_t *rows = tab ? tab[e] : base + e * stride;
            v = *reinterpret_cast<const uint32_t *>(rows + row * rb + b * kBlockBytes + 4 * w);
        }
        dst[d] = v;
    }
}

}  // namespace

int launch_kpack(const moe_bank &src, int32_t E, int32_t out_f, int32_t in_f, uint8_t *dst,
                 hipStream_t s) {
    const int32_t nb = in_f / kBlockWeights;
    const int64_t per_e = kpack_expert_bytes(out_f, in_f) / 4;
    const int64_t words = per_e * E;
    const int grid = (int)std::min<int64_t>((words + kPackThreads - 1) / kPackThreads, 16384);
    hipLaunchKernelGGL(kpack_kernel, dim3(grid), dim3(kPackThreads), 0, s, src.base,
                       src.expert_stride, src.experts, out_f, nb, per_e, words,
                       reinterpret_cast<uint32_t *>(dst));
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // namespace moe
