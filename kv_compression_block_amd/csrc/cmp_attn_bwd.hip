// Backward of the compressed attention (steps 1-3 of
// "mindspore.ops.nsa_compress_attention"), for training.  The pages give no
// backward formulas; these are the derivatives of the forward with respect
// to the gradient dout of attention_out, using the forward's saved softmax
// max and sum:  P = exp(scale*s - max) / sum over the visible blocks,
//   dP = dout . vc,  Delta = dout . out,  dS = P (dP - Delta),
//   dq = scale * sum_i dS_i kc_i,  dkc_i = scale * sum dS_i q,  dvc_i = sum P_i dout.
// Two kernels, no floating-point atomics (results are bitwise repeatable):
//   * query side (rows = (token, head), as the forward): recomputes P and dS
//     tile by tile and accumulates dq; also leaves each row's exponent bias
//     and Delta in the workspace for the key side;
//   * key side (one 32-entry key tile of one KV head per workgroup): four
//     waves split the query rows that see the tile, each accumulates dkc and
//     dvc for it, and the four partial sums are added in a fixed order.
// Both use bf16 or f16 MFMA 32x32x16 with fp32 accumulation; tiles go
// through LDS by buffer-unit copies of whole rows (16 bytes of padding per
// row) and transposed reads (ds_read_b64_tr_b16) where an operand needs
// the other orientation.
#include <type_traits>

#include "nsa_device.h"

namespace nsa {

namespace {

constexpr float kLog2eB = 1.4426950408889634f;

// Rows of `R` elements (a multiple of 8) padded by 8: copy layout in LDS.
template <int R>
struct PadRows {
    static constexpr int CH = R / 8;                       // 16-byte chunks per row
    static constexpr int S = R + 8;                        // row stride (elements)
    static constexpr int INS = (32 * (CH + 1) + 63) / 64;  // wave copy instructions per 32 rows
    static constexpr int BUF = INS * 512;                  // elements per 32-row buffer
};

// Transposed-read offset (elements) for a 32-row tile with row stride S:
// lane receives column `dim0 + l32` of rows {16kk + 4hf + 0..3, 16kk + 8 + 4hf + 0..3}
// (kk added by the caller as kk * 16 * S): the order a score accumulator
// leaves its rows in.
template <int S>
__device__ __forceinline__ int tr_off(int lane, int dim0)
{
    const int vi = lane & 15, vgrp = (lane >> 4) & 1, hf = lane >> 5;
    const int r0 = 4 * hf + (vi >> 2);
    return r0 * S + dim0 + 16 * vgrp + 4 * (vi & 3);
}

__device__ __forceinline__ u32x4 tr_read(const uint16_t* base, int S)
{
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)base);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * S));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace

// ---- query side: dq -----------------------------------------------------------
template <typename E, int D1, int D2>
__global__ __launch_bounds__(256, 2) void k_cmp_attn_bwd_dq(BwdParams p)
{
    constexpr int KT = 32, W = 4;
    using KR = PadRows<D1>;
    using VR = PadRows<D2>;
    constexpr int NKS = D1 / 16, NDS = D2 / 16, NDB1 = D1 / 32;
    constexpr int KIPW = (KR::INS + W - 1) / W, VIPW = (VR::INS + W - 1) / W;
    __shared__ __attribute__((aligned(16))) uint16_t K0[KR::BUF], K1[KR::BUF];
    __shared__ __attribute__((aligned(16))) uint16_t V0[VR::BUF], V1[VR::BUF];
    if (*p.status != 0)
        return;   // the table failed the planner's checks

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int wg = blockIdx.x;
    const int b = find_batch<true>(p.bt, p.B, wg);
    const BatchEnt be = p.bt[b];
    const int idx = wg - be.tile_off_a;
    const int g = idx % p.N2;
    const int rb = be.n_rb_a - 1 - idx / p.N2;
    const int G = p.G;
    const int rows_total = be.T * G;
    const int row_wg = rb * (32 * W);

    const int r = row_wg + wave * 32 + l32;
    const bool vq = r < rows_total;
    const int tok = r / G;
    const int64_t grow = (int64_t)(be.q_off + tok) * p.N1 + (int64_t)g * G + (r - tok * G);
    const int nvq = vq ? n_visible(tok + be.pos_off, p.l, p.d, be.n_cmp) : 0;
    const int64_t rsrc = vq ? grow : (int64_t)(be.q_off + row_wg / G) * p.N1 + (int64_t)g * G;

    // q, dout and out rows as B operands (lane l32 = row, k-slots 8hf..8hf+7)
    u32x4 qf[NKS], dof[NDS];
    float delta = 0.f;
    {
        const uint16_t* qrow = p.q + rsrc * D1 + hf * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qf[ks] = *(const u32x4*)(qrow + ks * 16) ^ p.qsign;
        const uint16_t* drow = p.dout + rsrc * D2 + hf * 8;
        const uint16_t* orow = p.out + rsrc * D2 + hf * 8;
#pragma unroll
        for (int ks = 0; ks < NDS; ++ks) {
            dof[ks] = *(const u32x4*)(drow + ks * 16);
            const u32x4 ov = *(const u32x4*)(orow + ks * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                delta += E::lo(dof[ks][j]) * E::lo(ov[j]) + E::hi(dof[ks][j]) * E::hi(ov[j]);
        }
        delta = half_sum(delta);
    }
    float bias = INFINITY;              // P = exp2(s*c - bias); +inf: the row sees nothing
    if (vq) {
        const float L = p.ssum[grow * 8];
        if (L > 0.f)
            bias = p.smax[grow * 8] * kLog2eB + __builtin_amdgcn_logf(L);
        if (hf == 0) {
            p.rowstat[grow * 2] = bias;
            p.rowstat[grow * 2 + 1] = delta;
        }
    }

    const int last_row = min(row_wg + 32 * W, rows_total) - 1;
    const int n_kt = (n_visible(last_row / G + be.pos_off, p.l, p.d, be.n_cmp) + KT - 1) / KT;

    // ---- tile copies ---------------------------------------------------------------
    const int64_t kstride = (int64_t)p.N2 * D1, vstride = (int64_t)p.N2 * D2;
    const uint16_t* kbase = p.kc + ((int64_t)be.cmp_off * p.N2 + g) * D1;
    const uint16_t* vbase = p.vc + ((int64_t)be.cmp_off * p.N2 + g) * D2;
    const uint32_t kst_b = (uint32_t)(kstride * 2), vst_b = (uint32_t)(vstride * 2);
    auto tile_bytes = [&](int kt, uint32_t stride_b, int row_bytes) -> uint32_t {
        const int nvalid = min(KT, be.n_cmp - kt * KT);
        return nvalid > 0 ? (uint32_t)(nvalid - 1) * stride_b + (uint32_t)row_bytes : 0u;
    };
    uint32_t kdo[KIPW], vdo[VIPW];
#pragma unroll
    for (int q = 0; q < KIPW; ++q) {
        const int slot = (q * W + wave) * 64 + lane;
        const int rr = slot / (KR::CH + 1), ch = slot % (KR::CH + 1);
        kdo[q] = (ch < KR::CH && rr < KT) ? (uint32_t)rr * kst_b + (uint32_t)ch * 16u : 0x7FFFFFF0u;
    }
#pragma unroll
    for (int q = 0; q < VIPW; ++q) {
        const int slot = (q * W + wave) * 64 + lane;
        const int rr = slot / (VR::CH + 1), ch = slot % (VR::CH + 1);
        vdo[q] = (ch < VR::CH && rr < KT) ? (uint32_t)rr * vst_b + (uint32_t)ch * 16u : 0x7FFFFFF0u;
    }
    auto copy_tile = [&](int kt, uint16_t* kd, uint16_t* vd) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + (int64_t)kt * KT * kstride, tile_bytes(kt, kst_b, D1 * 2));
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + (int64_t)kt * KT * vstride, tile_bytes(kt, vst_b, D2 * 2));
#pragma unroll
        for (int q = 0; q < KIPW; ++q)
            if (q * W + wave < KR::INS)
                copy16_to_lds(kr, kd + (q * W + wave) * 512, kdo[q]);
#pragma unroll
        for (int q = 0; q < VIPW; ++q)
            if (q * W + wave < VR::INS)
                copy16_to_lds(vr, vd + (q * W + wave) * 512, vdo[q]);
    };
    // This wave's copies have landed and (after the barrier) every wave's;
    // every wave is done with the previous tile's LDS reads.
    auto step_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0070);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };

    f32x16 dqa[NDB1];
#pragma unroll
    for (int db = 0; db < NDB1; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x)
            dqa[db][x] = 0.f;
    const float c = p.c;
    int ktr[NDB1];
#pragma unroll
    for (int db = 0; db < NDB1; ++db)
        ktr[db] = tr_off<KR::S>(lane, db * 32);

    auto tile = [&](int kt, const uint16_t* ks_, const uint16_t* vs_) __attribute__((always_inline)) {
        // S^T = K Q^T and dP^T = V dO^T (rows = keys, lane = query row)
        f32x16 s, dp;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            s[x] = 0.f;
            dp[x] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            s = E::mfma(*(const u32x4*)&ks_[l32 * KR::S + ks * 16 + hf * 8], qf[ks], s);
#pragma unroll
        for (int ks = 0; ks < NDS; ++ks)
            dp = E::mfma(*(const u32x4*)&vs_[l32 * VR::S + ks * 16 + hf * 8], dof[ks], dp);
        // key kt*KT + 8*(x/4) + 4*hf + x%4 is visible iff it is below nvq
        const int lim = nvq - kt * KT - 4 * hf;
        u32x4 dsf[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int x = kk * 8 + 2 * q + e;
                    const bool vis = 8 * (x >> 2) + (x & 3) < lim;
                    const float pr = vis ? fast_exp2(fmaf(s[x], c, -bias)) : 0.f;
                    v2[e] = pr * (dp[x] - delta);
                }
                dsf[kk][q] = E::pack2(v2[0], v2[1]);
            }
        }
        // dq^T += K^T dS^T (K^T read transposed from the key tile)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < NDB1; ++db)
                dqa[db] = E::mfma(tr_read(&ks_[ktr[db] + kk * 16 * KR::S], KR::S), dsf[kk], dqa[db]);
    };

    if (n_kt > 0)
        copy_tile(0, K0, V0);
    for (int kt = 0; kt < n_kt; kt += 2) {
        step_barrier();
        if (kt + 1 < n_kt)
            copy_tile(kt + 1, K1, V1);
        tile(kt, K0, V0);
        if (kt + 1 >= n_kt)
            break;
        step_barrier();
        if (kt + 2 < n_kt)
            copy_tile(kt + 2, K0, V0);
        tile(kt + 1, K1, V1);
    }

    // dq = scale * (K^T dS^T)^T: lane l32 holds dims 8*(x/4) + 4*hf + x%4 of
    // each 32-dim block for its row
    if (vq) {
        float* dst = p.dq + grow * D1;
#pragma unroll
        for (int db = 0; db < NDB1; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 v = {dqa[db][4 * r4] * p.scale, dqa[db][4 * r4 + 1] * p.scale,
                           dqa[db][4 * r4 + 2] * p.scale, dqa[db][4 * r4 + 3] * p.scale};
                *(f32x4*)(dst + db * 32 + 8 * r4 + 4 * hf) = v;
            }
    }
}

// ---- key side: dkc, dvc ---------------------------------------------------------
// One workgroup per (sequence, KV head, 32-entry key tile).  Keys and values
// of the tile are B operands held in registers (lane l32 = entry); the query
// rows that see the tile's first entry are split over the four waves in
// 32-row tiles, each copied with its dout rows into the wave's own LDS
// slots.  Per query tile: S = Q K^T and dP = dO V^T (rows = queries in
// registers, lane = key), P and dS from the rows' bias and Delta, then
// dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read transposed.
template <typename E, int D1, int D2>
__global__ __launch_bounds__(256, 1) void k_cmp_attn_bwd_dkv(BwdParams p)
{
    constexpr int W = 4;
    using QR = PadRows<D1>;
    using OR = PadRows<D2>;
    constexpr int NKS = D1 / 16, NDS = D2 / 16, NDB1 = D1 / 32, NDB2 = D2 / 32;
    constexpr int QSZ = QR::BUF, OSZ = OR::BUF;
    // per wave: a query-row tile, a dout-row tile; reused at the end for the
    // cross-wave sum (3 waves x 64 lanes x max(NDB1, NDB2) x 16 floats)
    // Two slots per wave where the LDS allows it (the next tile's copies then
    // overlap this tile's work), else one.
    constexpr int NBUF = (2 * W * (QSZ + OSZ) * 2 <= 150 * 1024) ? 2 : 1;
    constexpr int SMEL = NBUF * W * (QSZ + OSZ);
    static_assert(SMEL * 2 >= 3 * 64 * (NDB1 > NDB2 ? NDB1 : NDB2) * 16 * 4, "reduction space");
    __shared__ __attribute__((aligned(16))) uint16_t SM[SMEL];
    __shared__ __attribute__((aligned(16))) float ST[W * 64];
    if (*p.status != 0)
        return;   // the table failed the planner's checks

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int wg = blockIdx.x;
    int b = 0;
    {
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.bt[mid].tile_off_k <= wg)
                lo = mid;
            else
                hi = mid - 1;
        }
        b = lo;
    }
    const BatchEnt be = p.bt[b];
    const int idx = wg - be.tile_off_k;
    const int g = idx % p.N2;
    const int i0 = (idx / p.N2) * 32;                  // first entry of the tile (local)
    const int G = p.G;
    const int key = i0 + l32;
    const bool kvalid = key < be.n_cmp;

    // keys and values as B operands: lane l32 = entry, k-slots 8hf..8hf+7
    u32x4 kf[NKS], vf[NDS];
    {
        const int64_t krow = ((int64_t)(be.cmp_off + (kvalid ? key : i0)) * p.N2 + g);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            kf[ks] = *(const u32x4*)(p.kc + krow * D1 + ks * 16 + hf * 8);
#pragma unroll
        for (int ks = 0; ks < NDS; ++ks)
            vf[ks] = *(const u32x4*)(p.vc + krow * D2 + ks * 16 + hf * 8);
    }
    // first row (t*G + hh) that sees this lane's entry: the query's
    // position pos_off + t >= key*d + l - 1
    const int key_first_row = (key * p.d + p.l - 1 - be.pos_off) * G;

    // query rows r = t*G + hh seeing the tile's first entry
    const int rows_total = be.T * G;
    const int r_first = min(max(i0 * p.d + p.l - 1 - be.pos_off, 0), be.T) * G;
    const int n_qt = (rows_total - r_first + 31) / 32;

    auto qs_at = [&](int slot) { return SM + (slot * W + wave) * QSZ; };
    auto os_at = [&](int slot) { return SM + NBUF * W * QSZ + (slot * W + wave) * OSZ; };
    float* st = ST + wave * 64;
    // byte offsets inside the sequence's query rows: row r -> ((t*N1 + g*G + hh) * D) * 2
    const uint16_t* qseq = p.q + (int64_t)be.q_off * p.N1 * D1;
    const uint16_t* oseq = p.dout + (int64_t)be.q_off * p.N1 * D2;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qseq, (uint32_t)((int64_t)be.T * p.N1 * D1 * 2));
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(oseq, (uint32_t)((int64_t)be.T * p.N1 * D2 * 2));
    // element row of sequence row rr = t*G + hh: t*N1 + g*G + hh (t = rr / G
    // by a multiply-high with the host's magic number for G)
    auto row_elem = [&](int rr) -> int64_t {
        const int t = (int)(((uint64_t)__umulhi((uint32_t)rr, p.gdiv_m) + (uint32_t)rr) >> p.gdiv_s);
        return (int64_t)t * p.N1 + (int64_t)g * G + (rr - t * G);
    };

    f32x16 dka[NDB1], dva[NDB2];
#pragma unroll
    for (int db = 0; db < NDB1; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x)
            dka[db][x] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB2; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x)
            dva[db][x] = 0.f;
    int qtr[NDB1], otr[NDB2];
#pragma unroll
    for (int db = 0; db < NDB1; ++db)
        qtr[db] = tr_off<QR::S>(lane, db * 32);
#pragma unroll
    for (int db = 0; db < NDB2; ++db)
        otr[db] = tr_off<OR::S>(lane, db * 32);
    const float c = p.c;

    // Tile qt's copies: the rows' bias and Delta into registers (lanes < 32),
    // then the query and dout rows (rows past the sequence load 0).
    float stb = INFINITY, stq = 0.f;
    auto issue = [&](int qt, int slot) __attribute__((always_inline)) {
        const int r0 = r_first + qt * 32;
        if (lane < 32) {
            const bool ok = r0 + lane < rows_total;
            const int64_t grow = ok ? (int64_t)be.q_off * p.N1 + row_elem(r0 + lane) : 0;
            stb = ok ? p.rowstat[grow * 2] : INFINITY;
            stq = ok ? p.rowstat[grow * 2 + 1] : 0.f;
        }
        uint16_t* qd = qs_at(slot);
        uint16_t* od = os_at(slot);
#pragma unroll
        for (int q = 0; q < QR::INS; ++q) {
            const int sl = q * 64 + lane;
            const int rr = sl / (QR::CH + 1), ch = sl % (QR::CH + 1);
            const bool ok = ch < QR::CH && rr < 32 && r0 + rr < rows_total;
            const uint32_t off = ok ? (uint32_t)(row_elem(r0 + rr) * D1 * 2) + (uint32_t)ch * 16u : 0xFFFFFFF0u;
            copy16_to_lds(qrs, qd + q * 512, off);
        }
#pragma unroll
        for (int q = 0; q < OR::INS; ++q) {
            const int sl = q * 64 + lane;
            const int rr = sl / (OR::CH + 1), ch = sl % (OR::CH + 1);
            const bool ok = ch < OR::CH && rr < 32 && r0 + rr < rows_total;
            const uint32_t off = ok ? (uint32_t)(row_elem(r0 + rr) * D2 * 2) + (uint32_t)ch * 16u : 0xFFFFFFF0u;
            copy16_to_lds(ors, od + q * 512, off);
        }
    };

    int slot = 0;
    if (wave < n_qt)
        issue(wave, 0);
    for (int qt = wave; qt < n_qt; qt += W) {
        const int r0 = r_first + qt * 32;
        __builtin_amdgcn_s_waitcnt(0x0070);         // tile qt's copies and loads are done
        __asm__ volatile("" ::: "memory");
        if (lane < 32) {
            st[lane] = stb;
            st[32 + lane] = stq;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint16_t* qs = qs_at(slot);
        const uint16_t* os = os_at(slot);
        if constexpr (NBUF == 2) {
            if (qt + W < n_qt)
                issue(qt + W, slot ^ 1);            // the other slot's tile is done
        }

        // S = Q K^T, dP = dO V^T: rows = queries 8*(x/4) + 4*hf + x%4, lane = entry
        f32x16 s, dp;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            s[x] = 0.f;
            dp[x] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            s = E::mfma(*(const u32x4*)&qs[l32 * QR::S + ks * 16 + hf * 8] ^ p.qsign, kf[ks], s);
#pragma unroll
        for (int ks = 0; ks < NDS; ++ks)
            dp = E::mfma(*(const u32x4*)&os[l32 * OR::S + ks * 16 + hf * 8], vf[ks], dp);
        u32x4 pf[2], dsf[2];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int qr0 = 8 * r4 + 4 * hf;             // first of 4 consecutive rows
            const f32x4 bias4 = *(const f32x4*)&st[qr0];
            const f32x4 del4 = *(const f32x4*)&st[32 + qr0];
            float pv[4], dv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = 4 * r4 + e;
                const bool vis = kvalid && key_first_row <= r0 + qr0 + e;
                const float pr = vis ? fast_exp2(fmaf(s[x], c, -bias4[e])) : 0.f;
                pv[e] = pr;
                dv[e] = pr * (dp[x] - del4[e]);
            }
            const int kk = r4 >> 1, q2 = (r4 & 1) * 2;
            pf[kk][q2] = E::pack2(pv[0], pv[1]);
            pf[kk][q2 + 1] = E::pack2(pv[2], pv[3]);
            dsf[kk][q2] = E::pack2(dv[0], dv[1]);
            dsf[kk][q2 + 1] = E::pack2(dv[2], dv[3]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS (transposed reads of the row tiles)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int db = 0; db < NDB2; ++db)
                dva[db] = E::mfma(tr_read(&os[otr[db] + kk * 16 * OR::S], OR::S), pf[kk], dva[db]);
#pragma unroll
            for (int db = 0; db < NDB1; ++db)   // the true q: dkc = scale * sum dS q
                dka[db] = E::mfma(tr_read(&qs[qtr[db] + kk * 16 * QR::S], QR::S), dsf[kk], dka[db]);
        }
        __asm__ volatile("" ::: "memory");          // later copies stay after these reads
        if constexpr (NBUF == 1) {
            if (qt + W < n_qt)
                issue(qt + W, 0);
        } else {
            slot ^= 1;
        }
    }

    // Fixed-order sum of the four waves' partial sums: waves 1-3 park theirs
    // in LDS, wave 0 adds them in wave order and stores (lane = entry, 4
    // consecutive dims per register quad).
    float* red = (float*)SM;                         // [3][64 lanes][NDB * 16]
    auto reduce_store = [&](auto& acc, auto nb_tag, float* dst_base, int dcols, float mul) __attribute__((always_inline)) {
        constexpr int NB = decltype(nb_tag)::value;
        __syncthreads();
        if (wave > 0) {
#pragma unroll
            for (int db = 0; db < NB; ++db)
#pragma unroll
                for (int x = 0; x < 16; x += 4)
                    *(f32x4*)&red[(((wave - 1) * 64 + lane) * NB + db) * 16 + x] =
                        f32x4{acc[db][x], acc[db][x + 1], acc[db][x + 2], acc[db][x + 3]};
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 0; w < W - 1; ++w)
#pragma unroll
                for (int db = 0; db < NB; ++db)
#pragma unroll
                    for (int x = 0; x < 16; x += 4) {
                        const f32x4 v = *(const f32x4*)&red[((w * 64 + lane) * NB + db) * 16 + x];
                        acc[db][x] += v[0];
                        acc[db][x + 1] += v[1];
                        acc[db][x + 2] += v[2];
                        acc[db][x + 3] += v[3];
                    }
            if (kvalid) {
                float* dst = dst_base + ((int64_t)(be.cmp_off + key) * p.N2 + g) * dcols;
#pragma unroll
                for (int db = 0; db < NB; ++db)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4)
                        *(f32x4*)(dst + db * 32 + 8 * r4 + 4 * hf) =
                            f32x4{acc[db][4 * r4] * mul, acc[db][4 * r4 + 1] * mul,
                                  acc[db][4 * r4 + 2] * mul, acc[db][4 * r4 + 3] * mul};
            }
        }
    };
    reduce_store(dka, std::integral_constant<int, NDB1>{}, p.dkc, D1, p.scale);
    reduce_store(dva, std::integral_constant<int, NDB2>{}, p.dvc, D2, 1.f);
}

#define NSA_BWD_CONFIGS(X) X(64, 64) X(128, 64) X(128, 128) X(192, 64) X(192, 128)

bool attn_bwd_supported(int d1, int d2)
{
#define X(a, b_) if (d1 == a && d2 == b_) return true;
    NSA_BWD_CONFIGS(X)
#undef X
    return false;
}

template <typename E>
static hipError_t launch_bwd_typed(int d1, int d2, const BwdParams& p, int tiles_q, int tiles_k,
                                   hipStream_t stream)
{
#define X(a, b_)                                                                                    \
    if (d1 == a && d2 == b_) {                                                                      \
        if (tiles_q > 0)                                                                            \
            hipLaunchKernelGGL((k_cmp_attn_bwd_dq<E, a, b_>), dim3(tiles_q), dim3(256), 0, stream, p); \
        if (tiles_k > 0)                                                                            \
            hipLaunchKernelGGL((k_cmp_attn_bwd_dkv<E, a, b_>), dim3(tiles_k), dim3(256), 0, stream, p); \
        return hipGetLastError();                                                                   \
    }
    NSA_BWD_CONFIGS(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd(int dtype, int d1, int d2, const BwdParams& p, int tiles_q, int tiles_k,
                           hipStream_t stream)
{
    if (dtype == ElemBf16::code)
        return launch_bwd_typed<ElemBf16>(d1, d2, p, tiles_q, tiles_k, stream);
    if (dtype == ElemF16::code)
        return launch_bwd_typed<ElemF16>(d1, d2, p, tiles_q, tiles_k, stream);
    return hipErrorInvalidValue;
}

}  // namespace nsa
