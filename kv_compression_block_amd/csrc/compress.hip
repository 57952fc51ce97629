// Kernel (a): NSA compression ("aclnnNsaCompress", Formula).
//
// y[i, n, :] = sum_{p < l} w[p, n] * x[start + i*d + p, n, :]   per sequence,
// accumulated in float32 in ascending p, rounded once to the element type
// of x and w (bfloat16 or float16, nearest even).
//
// HBM-bound: one thread owns 8 consecutive elements (16 bytes) of one output
// row and walks the l input rows of its window with 16-byte loads, so a wave
// reads whole 64-byte..256-byte row segments.  Overlapping windows (l > d)
// re-read rows through L2, not HBM.  Weights are staged in LDS as float32.
// Grid: x = row-chunk blocks, y = sequence (blocks past a sequence's rows
// exit at once).
#include "nsa_device.h"

namespace nsa {

constexpr int kCompressThreads = 256;
constexpr int kCompressMaxW = 128 * 64;   // l * N floats staged in LDS (32 KB)

template <typename E>
__global__ __launch_bounds__(kCompressThreads) void k_compress(CompressParams p)
{
    __shared__ float wl[kCompressMaxW];
    const int seg = blockIdx.y;
    const int n_out = p.n_out[seg];
    const int nd8 = (p.N * p.D) >> 3;              // 16-byte chunks per row
    const int64_t item0 = (int64_t)blockIdx.x * kCompressThreads;
    if (item0 >= (int64_t)n_out * nd8)
        return;                                    // uniform per block

    const int nw = p.l * p.N;
    for (int k = threadIdx.x; k < nw; k += kCompressThreads) {
        wl[k] = E::widen(p.w[k]);
    }
    __syncthreads();

    const int64_t item = item0 + threadIdx.x;
    if (item >= (int64_t)n_out * nd8)
        return;
    const int i = (int)(item / nd8);
    const int c = (int)(item - (int64_t)i * nd8);
    const int n = (c * 8) / p.D;
    const int64_t row_stride = (int64_t)p.N * p.D;
    const uint16_t* src = p.x + ((int64_t)p.in_off[seg] + (int64_t)i * p.d) * row_stride + c * 8;

    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc[j] = 0.f;
    const float* wcol = wl + n;
#pragma unroll 4
    for (int pp = 0; pp < p.l; ++pp) {
        const u32x4 v = *(const u32x4*)(src + (int64_t)pp * row_stride);
        const float wv = wcol[pp * p.N];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[2 * j] = fmaf(wv, E::lo(v[j]), acc[2 * j]);
            acc[2 * j + 1] = fmaf(wv, E::hi(v[j]), acc[2 * j + 1]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = E::pack2(acc[2 * j], acc[2 * j + 1]);
    *(u32x4*)(p.y + ((int64_t)p.out_off[seg] + i) * row_stride + c * 8) = o;
}

hipError_t launch_compress(int dtype, const CompressParams& p, hipStream_t stream)
{
    if (p.l * p.N > kCompressMaxW)
        return hipErrorInvalidValue;
    dim3 grid(p.max_blocks_x, p.nseg, 1);
    if (dtype == ElemBf16::code)
        hipLaunchKernelGGL(k_compress<ElemBf16>, grid, dim3(kCompressThreads), 0, stream, p);
    else if (dtype == ElemF16::code)
        hipLaunchKernelGGL(k_compress<ElemF16>, grid, dim3(kCompressThreads), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nsa
