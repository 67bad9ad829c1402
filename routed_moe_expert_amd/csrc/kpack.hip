// The K-step-packed copy of a weight bank for the grouped-GEMM path (moe_kpack).
//
// A grouped-GEMM K step stages one 64-wide NVFP4 block of each of the weight tile's rows. In the
// row-major bank those are 36-byte pieces one row length apart, so each direct-to-LDS load of a
// step touches many rows; in the packed copy the blocks of one K step of a group of kKpackRows
// rows are one contiguous run of kKpackRows * 36 bytes, which 16-byte loads copy into LDS as it
// is. Within a run the bytes are in the order the GEMM's waves read them as MFMA A fragments:
// per slice of 32 rows (kSliceBytes = 1152 bytes), for each of its two 16-row tiles the code
// bytes lane by lane (lane l = n + 16 q holds code bytes 4 + 8 q .. 11 + 8 q of row n of the
// tile: 8 bytes, 512 per tile), then the scale bytes lane by lane (lane l: byte q of row n of
// tile 0, then of tile 1). A wave's reads of its fragments then take consecutive lanes to
// consecutive addresses (no LDS bank conflicts), up to 8 bytes a read. Rows past the bank are
// zero. Every block keeps its 36 bytes (four UE4M3 scales and 32 code bytes), so the
// copy is the same NVFP4 data in another order. It is written once, when the weights are loaded.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kPackThreads = 256;

// One dword of the copy per thread and grid step. Dword w of a run (K step b of row group g):
// slice s = w / 288; within the slice, dwords 0..255 are codes (tile t = r / 128, lane l =
// (r % 128) / 2, half h = r % 2: the dword at 4 + 8 q + 4 h of the block), dwords 256..287 the
// scale bytes (byte i of the slice's scale part: lane i / 2, tile i % 2).
__global__ __launch_bounds__(kPackThreads) void kpack_kernel(
    const uint8_t *__restrict__ base, int64_t stride, const uint8_t *const *__restrict__ tab,
    int32_t out_f, int32_t nb, int64_t words_per_expert, int64_t words,
    uint32_t *__restrict__ dst) {
    constexpr int kRunWords = kKpackRows * kBlockBytes / 4;   // 2304
    constexpr int kSliceWords = kSliceBytes / 4;               // 288
    const int64_t rb = (int64_t)nb * kBlockBytes;
    for (int64_t d = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; d < words;
         d += (int64_t)gridDim.x * kPackThreads) {
        const int64_t e = d / words_per_expert;
        const int64_t rest = d - e * words_per_expert;
        const int64_t run = rest / kRunWords;   // g * nb + b
        const int w = (int)(rest - run * kRunWords);
        const int b = (int)(run % nb);
        const int64_t row0 = run / nb * kKpackRows + w / kSliceWords * 32;   // the slice's row 0
        const int r = w % kSliceWords;
        const uint8_t *rows = tab ? tab[e] : base + e * stride;
        auto block = [&](int64_t row) { return rows + row * rb + b * kBlockBytes; };
        uint32_t v = 0;
        if (r < 256) {   // codes
            const int t = r / 128, l = (r % 128) / 2, h = r % 2;
            const int64_t row = row0 + 16 * t + (l & 15);
            if (row < out_f)
                v = *reinterpret_cast<const uint32_t *>(block(row) + 4 + 8 * (l >> 4) + 4 * h);
        } else {         // scales: bytes 4 (r - 256) .. +3 of the scale part
            for (int j = 0; j < 4; j++) {
                const int i = 4 * (r - 256) + j, l = i / 2, t = i % 2;
                const int64_t row = row0 + 16 * t + (l & 15);
                if (row < out_f) v |= (uint32_t)block(row)[l >> 4] << (8 * j);
            }
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
