// Kernel (a): NSA compression ("aclnnNsaCompress", Formula).
//
// y[i, n, :] = sum_{p < l} w[p, n] * x[start + i*d + p, n, :]   per sequence,
// accumulated in float32 in ascending p, rounded once to the element type
// of x and w (bfloat16 or float16, nearest even).
//
// HBM-bound.  A workgroup owns a run of nw consecutive windows of one
// sequence and one column slab of cs 16-byte chunks of the [N*D] row: it
// copies the run's (nw-1)*d + l input rows of that slab into LDS once
// (every load independent, 16 bytes per lane), then thread (window j,
// chunk c) walks its l rows in LDS.  Each input row is read from global
// memory once per run instead of once per window that contains it; the
// l - d rows two runs share are fetched by both, and the runs of a
// sequence are numbered so that consecutive runs go to the same XCD (the
// dispatcher deals workgroups to the eight XCDs in turn), where the
// second fetch finds them in that XCD's L2.  Weights are staged in LDS as
// float32.  Grid: x = XCD-ordered (run, slab) blocks, y = sequence (blocks
// past a sequence's runs exit at once).
#include "nsa_device.h"

namespace nsa {

constexpr int kCompressThreads = 256;
constexpr int kCompressMaxW = 128 * 64;   // l * N floats staged in LDS (32 KB)
constexpr int kCompressLoads = kCompressStageBytes / 16 / kCompressThreads;   // row-chunk copies per thread

template <typename E>
__global__ __launch_bounds__(kCompressThreads) void k_compress(CompressParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char cmp_smem[];
    u32x4* stage = (u32x4*)cmp_smem;                                   // [rows][cs]
    float* wl = (float*)(cmp_smem + kCompressStageBytes);              // [l][N]
    const int seg = blockIdx.y;
    const int n_out = p.n_out[seg];
    // XCD-ordered numbering: block x runs on XCD x % 8; the blocks of one
    // XCD take consecutive (run, slab) numbers.
    const int xb = blockIdx.x;
    const int u = (xb & 7) * (p.max_blocks_x >> 3) + (xb >> 3);
    const int run = u / p.nslab;
    const int slab = u - run * p.nslab;
    const int w0 = run * p.nw;
    if (w0 >= n_out)
        return;                                    // uniform per block
    const int nwv = min(p.nw, n_out - w0);         // windows of this run
    const int nrows = (nwv - 1) * p.d + p.l;       // input rows they cover
    const int cs_log2 = p.cs_log2;
    const int cs = 1 << cs_log2;
    const int64_t row_stride = (int64_t)p.N * p.D;     // elements
    const uint16_t* src = p.x + ((int64_t)p.in_off[seg] + (int64_t)w0 * p.d) * row_stride + slab * cs * 8;

    // Every copy of the run's rows is issued before the first one is stored.
    u32x4 v[kCompressLoads];
#pragma unroll
    for (int k = 0; k < kCompressLoads; ++k) {
        const int x = threadIdx.x + k * kCompressThreads;
        const int r = x >> cs_log2;
        if (r < nrows)
            v[k] = *(const u32x4*)(src + (int64_t)r * row_stride + (x & (cs - 1)) * 8);
    }
    const int nw = p.l * p.N;
    for (int k = threadIdx.x; k < nw; k += kCompressThreads)
        wl[k] = E::widen(p.w[k]);
#pragma unroll
    for (int k = 0; k < kCompressLoads; ++k) {
        const int x = threadIdx.x + k * kCompressThreads;
        if ((x >> cs_log2) < nrows)
            stage[x] = v[k];
    }
    __syncthreads();

    const int j = threadIdx.x >> cs_log2;          // window of the run
    const int c = threadIdx.x & (cs - 1);          // chunk of the slab
    if (j >= nwv)
        return;
    const int n = ((slab * cs + c) * 8) / p.D;     // the chunk's head
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.f;
    const u32x4* srow = stage + ((j * p.d) << cs_log2) + c;
    const float* wcol = wl + n;
#pragma unroll 4
    for (int pp = 0; pp < p.l; ++pp) {
        const u32x4 x = srow[pp << cs_log2];
        const float wv = wcol[pp * p.N];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = fmaf(wv, E::lo(x[e]), acc[2 * e]);
            acc[2 * e + 1] = fmaf(wv, E::hi(x[e]), acc[2 * e + 1]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = E::pack2(acc[2 * e], acc[2 * e + 1]);
    *(u32x4*)(p.y + ((int64_t)p.out_off[seg] + w0 + j) * row_stride + (slab * cs + c) * 8) = o;
}

// Backward (for training; the derivative of the formula above):
//   dx[start + i*d + p, n, :] += w[p, n] * dy[i, n, :]
//   dw[p, n] += sum_i sum_e dy[i, n, e] * x[start + i*d + p, n, e]
// dx: one thread per 4 consecutive floats of an input row, summing the at
// most ceil(l/d) windows that contain the row in ascending window order
// (rows in no window get 0).  dw: workgroups per (p, n) and chunk of the
// windows, each thread a fixed strided share of the (window, dim) pairs and
// a fixed-shape tree in LDS, then the chunks added in order: no atomics,
// bitwise repeatable.  The chunk sums live in d_input before it is written.
template <typename E>
__global__ __launch_bounds__(kCompressThreads) void k_compress_bwd_dx(CompressBwdParams p)
{
    const int seg = blockIdx.y;
    const int T = p.n_in[seg], n_out = p.n_out[seg];
    const int nd4 = (p.N * p.D) >> 2;
    const int64_t item = (int64_t)blockIdx.x * kCompressThreads + threadIdx.x;
    if (item >= (int64_t)T * nd4)
        return;
    const int r = (int)(item / nd4);
    const int c = (int)(item - (int64_t)r * nd4);
    const int n = (c * 4) / p.D;
    const int i_lo = r - p.l + 1 <= 0 ? 0 : (r - p.l + p.d) / p.d;
    const int i_hi = min(n_out - 1, r / p.d);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = i_lo; i <= i_hi; ++i) {
        const float wv = E::widen(p.w[(r - i * p.d) * p.N + n]);
        const f32x4 g = *(const f32x4*)(p.dy + ((int64_t)p.out_off[seg] + i) * p.N * p.D + c * 4);
        acc[0] = fmaf(wv, g[0], acc[0]);
        acc[1] = fmaf(wv, g[1], acc[1]);
        acc[2] = fmaf(wv, g[2], acc[2]);
        acc[3] = fmaf(wv, g[3], acc[3]);
    }
    *(f32x4*)(p.dx + ((int64_t)p.in_off[seg] + r) * p.N * p.D + c * 4) = acc;
}

// dw, first pass: workgroup (p*N + n, chunk) sums its chunk of the launch's
// windows (flattened over the sequences, ascending) into part[pn * C + chunk];
// with one chunk it writes (or adds to) dw directly.
template <typename E>
__global__ __launch_bounds__(kCompressThreads) void k_compress_bwd_dw(CompressBwdParams p)
{
    __shared__ float red[kCompressThreads];
    const int pn = blockIdx.x;                       // p * N + n
    const int chunk = blockIdx.y, C = gridDim.y;
    const int pp = pn / p.N, n = pn - pp * p.N;
    int64_t wtot = 0;
    for (int s = 0; s < p.nseg; ++s)
        wtot += p.n_out[s];
    const int64_t w_lo = wtot * chunk / C, w_hi = wtot * (chunk + 1) / C;
    float acc = 0.f;
    int64_t wbase = 0;
    for (int s = 0; s < p.nseg; ++s) {
        const int64_t lo = max(w_lo - wbase, (int64_t)0), hi = min(w_hi - wbase, (int64_t)p.n_out[s]);
        wbase += p.n_out[s];
        if (lo >= hi)
            continue;
        const int64_t pairs = (hi - lo) * p.D;
        for (int64_t k = threadIdx.x; k < pairs; k += kCompressThreads) {
            const int64_t i = lo + k / p.D;
            const int e = (int)(k % p.D);
            const float g = p.dy[(((int64_t)p.out_off[s] + i) * p.N + n) * p.D + e];
            const float xv = E::widen(p.x[(((int64_t)p.in_off[s] + i * p.d + pp) * p.N + n) * p.D + e]);
            acc = fmaf(g, xv, acc);
        }
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = kCompressThreads / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h)
            red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (C > 1)
            p.part[(int64_t)pn * C + chunk] = red[0];
        else
            p.dw[pn] = p.accumulate ? p.dw[pn] + red[0] : red[0];
    }
}

// dw, second pass: the chunks' sums in chunk order.
__global__ __launch_bounds__(64) void k_compress_bwd_dw_sum(CompressBwdParams p, int C)
{
    const int pn = blockIdx.x * 64 + threadIdx.x;
    if (pn >= p.l * p.N)
        return;
    float acc = 0.f;
    for (int c = 0; c < C; ++c)
        acc += p.part[(int64_t)pn * C + c];
    p.dw[pn] = p.accumulate ? p.dw[pn] + acc : acc;
}

hipError_t launch_compress_bwd_dw(int dtype, const CompressBwdParams& p, int chunks, hipStream_t stream)
{
    const int C = chunks < 1 ? 1 : chunks;
    dim3 g(p.l * p.N, C, 1);
    if (dtype == ElemBf16::code)
        hipLaunchKernelGGL(k_compress_bwd_dw<ElemBf16>, g, dim3(kCompressThreads), 0, stream, p);
    else if (dtype == ElemF16::code)
        hipLaunchKernelGGL(k_compress_bwd_dw<ElemF16>, g, dim3(kCompressThreads), 0, stream, p);
    else
        return hipErrorInvalidValue;
    if (C > 1)
        hipLaunchKernelGGL(k_compress_bwd_dw_sum, dim3((p.l * p.N + 63) / 64), dim3(64), 0, stream, p, C);
    return hipGetLastError();
}

hipError_t launch_compress_bwd_dx(int dtype, const CompressBwdParams& p, hipStream_t stream)
{
    if (p.max_blocks_x <= 0 || p.nseg <= 0)
        return hipSuccess;
    dim3 gx(p.max_blocks_x, p.nseg, 1);
    if (dtype == ElemBf16::code)
        hipLaunchKernelGGL(k_compress_bwd_dx<ElemBf16>, gx, dim3(kCompressThreads), 0, stream, p);
    else if (dtype == ElemF16::code)
        hipLaunchKernelGGL(k_compress_bwd_dx<ElemF16>, gx, dim3(kCompressThreads), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_compress(int dtype, const CompressParams& p, hipStream_t stream)
{
    const int cs = 1 << p.cs_log2;
    if (p.l * p.N > kCompressMaxW || p.max_blocks_x % 8 != 0 || cs > 16 || p.nw < 1 ||
        p.nw * cs > kCompressThreads || ((p.nw - 1) * p.d + p.l) * cs * 16 > kCompressStageBytes)
        return hipErrorInvalidValue;
    dim3 grid(p.max_blocks_x, p.nseg, 1);
    const size_t lds = kCompressStageBytes + (size_t)p.l * p.N * sizeof(float);
    if (lds > 64 * 1024) {
        auto kern = dtype == ElemBf16::code ? (const void*)k_compress<ElemBf16> : (const void*)k_compress<ElemF16>;
        const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    if (dtype == ElemBf16::code)
        hipLaunchKernelGGL(k_compress<ElemBf16>, grid, dim3(kCompressThreads), lds, stream, p);
    else if (dtype == ElemF16::code)
        hipLaunchKernelGGL(k_compress<ElemF16>, grid, dim3(kCompressThreads), lds, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nsa
