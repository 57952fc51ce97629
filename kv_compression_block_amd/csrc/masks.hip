// Explicit masks of "mindspore.ops.nsa_compress_attention" (Parameters:
// optional bool atten_mask and topk_mask of shape (S1, S2)), packed to bits
// before the attention and importance/top-k kernels read them.
//
// One wave covers 64 consecutive columns of one row: each lane loads one
// byte (64 contiguous bytes per wave), and one ballot gives the two 32-bit
// words of kept pairs (bit set iff the byte is zero and the column exists).
// A second pass records per row the span of words that keep anything and
// the number of leading words that keep everything, from which the kernels
// bound the key tiles a workgroup has to visit and find the leading tiles
// that need no mask.
#include "nsa_device.h"

namespace nsa {

constexpr int kPackThreads = 256;

__global__ __launch_bounds__(kPackThreads) void k_pack_mask(MaskPackParams p)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kPackThreads + threadIdx.x) >> 6;
    const int pairs = (p.words + 1) >> 1;           // 64-column groups per row
    const int64_t total = (int64_t)p.rows * pairs;
    if (wave >= total)
        return;                                      // uniform per wave
    const int t = (int)(wave / pairs);
    const int grp = (int)(wave - (int64_t)t * pairs);
    const int64_t col = (int64_t)grp * 64 + lane;
    bool keep = false;
    if (col < p.src_cols)
        keep = p.src[(int64_t)t * p.src_cols + col] == 0;
    const uint64_t bits = __ballot(keep);
    const int w = grp * 2 + (lane >> 5);
    if ((lane & 31) == 0 && w < p.words)
        p.dst[(int64_t)t * p.words + w] = (uint32_t)(lane ? bits >> 32 : bits);
}

// One thread per row: the first and one past the last non-zero word, and
// the number of leading all-ones words.
__global__ __launch_bounds__(kPackThreads) void k_mask_span(MaskPackParams p)
{
    const int t = blockIdx.x * kPackThreads + threadIdx.x;
    if (t >= p.rows)
        return;
    const uint32_t* row = p.dst + (int64_t)t * p.words;
    int lo = p.words, hi = 0, full = 0;
    bool lead = true;
    for (int w = 0; w < p.words; ++w) {
        const uint32_t v = row[w];
        if (v != 0u) {
            lo = min(lo, w);
            hi = w + 1;
        }
        lead = lead && v == 0xFFFFFFFFu;
        full += lead;
    }
    p.span[t] = make_int4(lo, hi, full, 0);
}

hipError_t launch_pack_mask(const MaskPackParams& p, hipStream_t stream)
{
    if (p.rows <= 0 || p.words <= 0)
        return hipSuccess;
    const int64_t waves = (int64_t)p.rows * ((p.words + 1) / 2);
    const int64_t blocks = (waves * 64 + kPackThreads - 1) / kPackThreads;
    if (blocks > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_pack_mask, dim3((unsigned)blocks), dim3(kPackThreads), 0, stream, p);
    if (p.span) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(k_mask_span, dim3((unsigned)((p.rows + kPackThreads - 1) / kPackThreads)),
                           dim3(kPackThreads), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace nsa
