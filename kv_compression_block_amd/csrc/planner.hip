// Planning on the device.
//
// "QuantLightningIndexerMetadata" (README, 功能说明) describes a pre-pass that
// runs before the sparse-attention operator on the device: it takes each
// batch's basic blocks and load (step 1), the totals over all batches (step
// 2) and each core's share of the load with its start and end points (step
// 3), and hands the operator a small int32 metadata array, so that the
// sequence lengths may stay in device memory.  Here the same role is played
// by two pieces of device code:
//
//   * k_meta_table -- one workgroup derives the per-sequence table every
//     kernel of the library reads (offsets, lengths, and each kernel's
//     workgroup ranges: the "basic blocks and load" per batch, scanned into
//     start points) from device prefix sums, checks every relation the host
//     planner checks, and writes a status word next to the table.  Every
//     kernel that reads the table exits at once when the word is not zero.
//
//   * k_list_count / k_list_fill -- work lists built from the table: for a
//     split attention launch every row block of the attention kernel becomes
//     one piece, or ceil(n / C) pieces when it walks n > C key tiles; for the
//     key-side backward every key block becomes ceil(n / qmax) pieces of the
//     n query tiles that see it.  The pieces are numbered in unit order by an
//     exclusive prefix sum over chunks of 256 units (the count kernel writes
//     chunk totals, the fill kernel adds the totals of the chunks before its
//     own).
#include "nsa_device.h"

namespace nsa {

namespace {

constexpr int kPlanThreads = 256;

__device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Exclusive prefix sums of v over the workgroup (Hillis-Steele in LDS);
// returns the sum of all threads' values.
__device__ int64_t block_exclusive_scan(int64_t* sh, int64_t& v)
{
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int64_t add = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += add;
        __syncthreads();
    }
    const int64_t incl = sh[tid];
    const int64_t total = sh[kPlanThreads - 1];
    __syncthreads();
    v = incl - v;
    return total;
}

}  // namespace

__global__ __launch_bounds__(kPlanThreads) void k_meta_table(MetaParams p)
{
    __shared__ int64_t sh[kPlanThreads];
    __shared__ int err_bits;
    const int tid = threadIdx.x;
    if (tid == 0)
        err_bits = 0;
    __syncthreads();
    int64_t ta = 0, tc = 0, ts = 0, tk = 0, tot_s = 0;   // running totals (uniform)
    int my_err = 0;
    for (int base = 0; base < p.B; base += kPlanThreads) {
        const int b = base + tid;
        const bool in = b < p.B;
        int64_t T = 0, Tkv = 0, nc = 0, ns = 0, q0 = 0, kv0 = 0, c0 = 0;
        if (in) {
            q0 = b > 0 ? p.qlen[b - 1] : 0;
            T = p.qlen[b] - q0;
            kv0 = p.kvlen ? (b > 0 ? p.kvlen[b - 1] : 0) : q0;
            Tkv = p.kvlen ? p.kvlen[b] - kv0 : T;
            c0 = b > 0 ? p.cmplen[b - 1] : 0;
            nc = p.cmplen[b] - c0;
            const int64_t s0 = b > 0 ? p.sellen[b - 1] : 0;
            ns = p.sellen[b] - s0;
            if (q0 < 0 || T < 0 || kv0 < 0 || c0 < 0 || s0 < 0)
                my_err |= kMetaErrPrefix;
            else if (Tkv < T)
                my_err |= kMetaErrKvShort;
            else if (nc != (Tkv < p.l ? 0 : (Tkv - p.l) / p.d + 1))
                my_err |= kMetaErrCmpLen;
            else if (ns != ceil_div(Tkv, p.lsel))
                my_err |= kMetaErrSelLen;
            else if (T > p.T_max || nc > p.ncmp_max || ns > p.S_max || Tkv - T > INT32_MAX)
                my_err |= kMetaErrCapacity;
            if (my_err) {   // keep the arithmetic below in range
                T = Tkv = nc = ns = 0;
            }
        }
        int64_t na = in ? ceil_div(T * p.G, p.rows_a) : 0;
        int64_t nt = in ? ceil_div(T * p.GP, p.rows_c) : 0;
        int64_t nsr = in ? ceil_div(T * p.G, p.rows_s) : 0;
        int64_t nk = in ? ceil_div(nc, kBwdKeyBlock) : 0;
        int64_t sv = in ? ns : 0;
        int64_t ea = na * p.N2, ec = nt * p.N2, es = nsr * p.N2, ek = nk * p.N2;
        const int64_t sum_a = block_exclusive_scan(sh, ea);
        const int64_t sum_c = block_exclusive_scan(sh, ec);
        const int64_t sum_s = block_exclusive_scan(sh, es);
        const int64_t sum_k = block_exclusive_scan(sh, ek);
        const int64_t sum_v = block_exclusive_scan(sh, sv);
        if (in) {
            BatchEnt e;
            e.q_off = (int32_t)q0;
            e.T = (int32_t)T;
            e.cmp_off = (int32_t)c0;
            e.n_cmp = (int32_t)nc;
            e.tile_off_a = (int32_t)(ta + ea);
            e.n_rb_a = (int32_t)na;
            e.tile_off_c = (int32_t)(tc + ec);
            e.n_rb_c = (int32_t)nt;
            e.S_sel = (int32_t)ns;
            e.tile_off_s = (int32_t)(ts + es);
            e.n_rb_s = (int32_t)nsr;
            e.tile_off_k = (int32_t)(tk + ek);
            e.pos_off = (int32_t)(Tkv - T);
            e.kv_off = (int32_t)kv0;
            e.pad1 = 0;
            e.pad2 = 0;
            p.table[b] = e;
        }
        ta += sum_a;
        tc += sum_c;
        ts += sum_s;
        tk += sum_k;
        tot_s += sum_v;
    }
    if (my_err)
        atomicOr(&err_bits, my_err);
    __syncthreads();
    if (tid == 0) {
        int e = err_bits;
        const int64_t last_q = p.qlen[p.B - 1], last_c = p.cmplen[p.B - 1];
        if (!e && (last_q != p.T1 || last_c != p.T2 || tot_s != p.S_total || ta != p.tiles_a ||
                   tc != p.tiles_c || ts != p.tiles_s || tk != p.tiles_k ||
                   (p.kvlen && p.kvlen[p.B - 1] != p.Tkv_total)))
            e |= kMetaErrTotals;
        __builtin_nontemporal_store(e, p.status);
    }
}

// ---- work lists cut into pieces ------------------------------------------------
// A unit (a row block of the attention kernel, or a key block of the
// key-side backward) becomes one work item, or several pieces whose partial
// results a combine item adds.  The count kernel writes the totals of each
// chunk of 256 units; the fill kernel adds the totals of the chunks before
// its own, numbers its units' items by an exclusive prefix sum and writes
// them, and checks that the list ends where the host's counts say.
struct UnitSplit {
    int b, g, r, n, pieces;   // sequence, KV head, row or key block, tiles it walks, pieces
    bool split;
};

__device__ __forceinline__ int last_le(const BatchEnt* t, int B, int u, int BatchEnt::*off)
{
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t[mid].*off <= u)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Split attention: row block wg of the unsplit launch walks n key tiles of
// kKeyTileMin entries; pieces of C tiles when n > C.
__device__ __forceinline__ int64_t units_of(const SplitPlanParams& p) { return p.tiles_a; }
__device__ __forceinline__ UnitSplit unit_of(const SplitPlanParams& p, int wg)
{
    UnitSplit r;
    const int b = last_le(p.table, p.B, wg, &BatchEnt::tile_off_a);
    const BatchEnt be = p.table[b];
    const int idx = wg - be.tile_off_a;
    r.b = b;
    r.g = idx % p.N2;
    r.r = be.n_rb_a - 1 - idx / p.N2;
    const int64_t rows = (int64_t)be.T * p.G;
    const int64_t last_row = min((int64_t)(r.r + 1) * p.rows_a, rows) - 1;
    const int t = (int)(last_row / p.G) + be.pos_off;
    const int nv = n_visible(t, p.l, p.d, be.n_cmp);
    r.n = (nv + kKeyTileMin - 1) / kKeyTileMin;
    r.split = r.n > p.C;
    r.pieces = r.split ? (r.n + p.C - 1) / p.C : 1;
    return r;
}
__device__ __forceinline__ void write_unit(const SplitPlanParams& p, const UnitSplit& r, int64_t i0, int64_t c0,
                                           int64_t s0)
{
    if (!r.split) {
        p.items[i0] = SplitItem{r.b, r.g, r.r, 0, r.n, -1, 0, 0};
        return;
    }
    for (int q = 0; q < r.pieces; ++q)
        p.items[i0 + q] = SplitItem{r.b, r.g, r.r, q * p.C, min(p.C, r.n - q * p.C), (int)(s0 + q), 0, 0};
    p.combs[c0] = CombineItem{r.b, r.g, r.r, (int)s0, r.pieces, 0, 0, 0};
}

// Key-side backward: key block kb (kBwdKeyBlock entries) of KV head g is
// seen by the 32-row query tiles from the row of the block's first entry to
// the end of the sequence; ceil(n / qmax) pieces of nearly equal length.
__device__ __forceinline__ int64_t units_of(const BwdPlanParams& p) { return p.tiles_k; }
__device__ __forceinline__ UnitSplit unit_of(const BwdPlanParams& p, int u)
{
    UnitSplit r;
    const int b = last_le(p.table, p.B, u, &BatchEnt::tile_off_k);
    const BatchEnt be = p.table[b];
    const int idx = u - be.tile_off_k;
    r.b = b;
    r.g = idx % p.N2;
    r.r = idx / p.N2;
    const int64_t first = min(max((int64_t)r.r * kBwdKeyBlock * p.d + p.l - 1 - be.pos_off, (int64_t)0),
                              (int64_t)be.T) * p.G;
    r.n = (int)(((int64_t)be.T * p.G - first + 31) / 32);
    r.pieces = r.n > p.qmax ? (r.n + p.qmax - 1) / p.qmax : 1;
    r.split = r.pieces > 1;
    return r;
}
__device__ __forceinline__ void write_unit(const BwdPlanParams& p, const UnitSplit& r, int64_t i0, int64_t c0,
                                           int64_t s0)
{
    if (!r.split) {
        p.items[i0] = BwdItem{r.b, r.g, r.r, 0, r.n, -1, 0, 0};
        return;
    }
    for (int q = 0; q < r.pieces; ++q) {
        const int a = (int)((int64_t)q * r.n / r.pieces), e = (int)((int64_t)(q + 1) * r.n / r.pieces);
        p.items[i0 + q] = BwdItem{r.b, r.g, r.r, a, e - a, (int)(s0 + q), 0, 0};
    }
    p.combs[c0] = CombineItem{r.b, r.g, r.r, (int)s0, r.pieces, 0, 0, 0};
}

template <class P>
__global__ __launch_bounds__(kPlanThreads) void k_list_count(P p)
{
    __shared__ int64_t sh[kPlanThreads];
    if (*p.status != 0)
        return;
    const int u = blockIdx.x * kPlanThreads + threadIdx.x;
    int64_t items = 0, combs = 0, slots = 0;
    if (u < units_of(p)) {
        const UnitSplit r = unit_of(p, u);
        items = r.pieces;
        combs = r.split ? 1 : 0;
        slots = r.split ? r.pieces : 0;
    }
    const int64_t ti = block_exclusive_scan(sh, items);
    const int64_t tcb = block_exclusive_scan(sh, combs);
    const int64_t tsl = block_exclusive_scan(sh, slots);
    if (threadIdx.x == 0)
        p.chunk_tot[blockIdx.x] = make_int4((int)ti, (int)tcb, (int)tsl, 0);
}

template <class P>
__global__ __launch_bounds__(kPlanThreads) void k_list_fill(P p)
{
    __shared__ int64_t sh[kPlanThreads];
    __shared__ int bad;
    if (*p.status != 0)
        return;
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    if (tid == 0)
        bad = 0;
    // Start of this chunk: the totals of the chunks before it.
    int64_t bi = 0, bc = 0, bs = 0;
    for (int c = tid; c < chunk; c += kPlanThreads) {
        const int4 t = p.chunk_tot[c];
        bi += t.x;
        bc += t.y;
        bs += t.z;
    }
    int64_t x = bi;
    bi = block_exclusive_scan(sh, x);   // sum over threads
    x = bc;
    bc = block_exclusive_scan(sh, x);
    x = bs;
    bs = block_exclusive_scan(sh, x);
    const int u = chunk * kPlanThreads + tid;
    UnitSplit r{};
    int64_t items = 0, combs = 0, slots = 0;
    const bool in = u < units_of(p);
    if (in) {
        r = unit_of(p, u);
        items = r.pieces;
        combs = r.split ? 1 : 0;
        slots = r.split ? r.pieces : 0;
    }
    const int64_t ti = block_exclusive_scan(sh, items);
    const int64_t tcb = block_exclusive_scan(sh, combs);
    const int64_t tsl = block_exclusive_scan(sh, slots);
    if (in) {
        const int64_t i0 = bi + items, c0 = bc + combs, s0 = bs + slots;
        if (i0 + r.pieces > p.n_items || (r.split && (c0 >= p.n_combs || s0 + r.pieces > p.n_slots)))
            atomicOr(&bad, 1);
        else
            write_unit(p, r, i0, c0, s0);
    }
    __syncthreads();
    // The last chunk ends the list: its end must be the host's count.
    if (tid == 0 && (bad || (chunk == gridDim.x - 1 &&
                             (bi + ti != p.n_items || bc + tcb != p.n_combs || bs + tsl != p.n_slots))))
        atomicOr(p.status, kMetaErrSplit);
}

template <class P>
static hipError_t launch_list(const P& p, int64_t units, hipStream_t stream)
{
    const int chunks = plan_chunks(units);
    if (chunks <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_list_count<P>, dim3(chunks), dim3(kPlanThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_list_fill<P>, dim3(chunks), dim3(kPlanThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_meta_table(const MetaParams& p, hipStream_t stream)
{
    hipLaunchKernelGGL(k_meta_table, dim3(1), dim3(kPlanThreads), 0, stream, p);
    return hipGetLastError();
}

int plan_chunks(int64_t units) { return (int)((units + kPlanThreads - 1) / kPlanThreads); }

hipError_t launch_split_plan(const SplitPlanParams& p, hipStream_t stream) { return launch_list(p, p.tiles_a, stream); }

hipError_t launch_bwd_plan(const BwdPlanParams& p, hipStream_t stream) { return launch_list(p, p.tiles_k, stream); }

}  // namespace nsa
