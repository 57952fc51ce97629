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
//   * key side (a block of 128 compressed entries of one KV head and a
//     range of the query tiles that see it per workgroup, each wave owning
//     32 entries; the query tiles stream through LDS slots shared by the
//     waves): blocks seen by more tiles than an item holds leave partial
//     sums, added in piece order by a combine kernel.
// Both use bf16 or f16 MFMA 32x32x16 with fp32 accumulation; tiles go
// through LDS by buffer-unit copies (16-byte chunks permuted within each
// row so that row reads and transposed reads, ds_read_b64_tr_b16, are both
// free of bank conflicts).
#include <type_traits>

#include "nsa_device.h"

namespace nsa {

namespace {

constexpr float kLog2eB = 1.4426950408889634f;

// A 32-row tile of R elements (R a multiple of 64) in LDS, rows packed,
// the 16-byte chunks of row r permuted by c -> c ^ s(r).  The tile is read
// two ways: whole rows (ds_read_b128, 16 lanes a pass: rows r..r+15 at one
// chunk) and transposed (ds_read_b64_tr_b16, 32 lanes a pass: four rows
// 4m..4m+3 at four chunks 4n..4n+3).  With 64 four-byte banks a pass is
// free of bank conflicts when its 16-byte units fall on distinct positions
// modulo 16; s is chosen so that both passes do:
//   * 16 chunks a row (rows a multiple of 256 bytes): s(r) = 4 (r & 3) +
//     ((r >> 2) & 3), a bijection on r & 15 (row reads), and for the rows
//     4m + i of a transposed read 4 i + (m & 3): bits 2-3 follow i, bits
//     0-1 the chunk;
//   * 8 or 24 chunks a row (rows at 128-byte steps, alternate rows half a
//     bank cycle apart): s(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3) < 8, a
//     bijection on the even and on the odd rows of 16, and for rows 4m + i
//     bit 2 follows i >> 1, bits 0-1 the chunk, the row's parity the rest.
template <int R>
struct SwzRows {
    static_assert(R % 64 == 0, "rows of a multiple of 64 elements");
    static constexpr int CH = R / 8;                  // 16-byte chunks per row
    static constexpr int UNITS = 32 * CH;             // 16-byte units of the tile
    static constexpr int INS = (UNITS + 63) / 64;     // wave copy instructions per tile
    static constexpr int BUF = INS * 512;             // elements per tile buffer
    static constexpr int KK = 16 * R;                 // elements of 16 rows
    __device__ static __forceinline__ int s(int r)
    {
        if constexpr (CH % 16 == 0)
            return ((r & 3) << 2) | ((r >> 2) & 3);
        else
            return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    }
    // element offset of chunk c (8 elements) of row r
    __device__ static __forceinline__ int at(int r, int c) { return (r * CH + (c ^ s(r))) * 8; }
    // Row reads of the A operand of k-step ks (chunk 2 ks + hf of row l32):
    // at(l32, 2 ks + hf) = (lb ^ 16 (ks & M)) + G (ks >> L) with lb =
    // at(l32, hf), since the XOR only moves chunks inside a group of 16 (8)
    // and the row starts on a group boundary of the element offset.
    static constexpr int M = CH % 16 == 0 ? 7 : 3, L = CH % 16 == 0 ? 3 : 2, G = CH % 16 == 0 ? 128 : 64;
    __device__ static __forceinline__ int row_base(int l32, int hf) { return at(l32, hf); }
    __device__ static __forceinline__ int row_at(int lb, int ks) { return (lb ^ (16 * (ks & M))) + G * (ks >> L); }
    // unit P of the buffer holds chunk chunk_of(P) of row P / CH
    __device__ static __forceinline__ int chunk_of(int P) { return (P % CH) ^ s(P / CH); }
    // Transposed read: lane receives column 32 db + l32 of rows {4hf + 0..3}
    // (lo) and {8 + 4hf + 0..3} (hi), + 16 kk rows (added as kk * KK): the
    // order a score accumulator leaves its rows in.  Lane (vi, vgrp, hf)
    // supplies the 8 bytes of row 4hf + vi/4 at dims 32 db + 16 vgrp +
    // 4 (vi%4).  From the block-0 offset tb: block db flips chunk bits 2-3
    // (bit 2 and the group for 8-chunk swizzles), and the row 8 further on
    // has s(r + 8) = s(r) ^ 2, one chunk bit.
    static constexpr int MD = CH % 16 == 0 ? 3 : 1, LD = CH % 16 == 0 ? 2 : 1, GD = CH % 16 == 0 ? 128 : 64;
    __device__ static __forceinline__ int tr_base(int lane)
    {
        const int vi = lane & 15, vgrp = (lane >> 4) & 1, hf = lane >> 5;
        const int r = 4 * hf + (vi >> 2);
        const int dim = 16 * vgrp + 4 * (vi & 3);
        return at(r, dim >> 3) + (dim & 7);
    }
    __device__ static __forceinline__ int tr_lo(int tb, int db) { return (tb ^ (32 * (db & MD))) + GD * (db >> LD); }
    __device__ static __forceinline__ int tr_hi(int tb, int db) { return (tr_lo(tb, db) ^ 16) + 64 * CH; }
};

__device__ __forceinline__ u32x4 tr_read2(const uint16_t* lo_p, const uint16_t* hi_p)
{
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo_p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi_p);
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Buffer-to-LDS copies with the LDS address passed as a plain number: the
// compiler then cannot tie a copy to an LDS object and adds no waits of its
// own before reads of other objects (it would otherwise wait for copies it
// cannot tell apart, several tiles ahead).  The kernels order every copy
// against its reads with their own wait counts and barriers.  16 (or 4)
// bytes per lane land at lds + 16 i (4 i); voff per lane, soff per wave.
__device__ __forceinline__ lds_void* lds_untracked(void* lds)
{
    return (lds_void*)(uintptr_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
}

__device__ __forceinline__ void copy16_to_lds_untracked(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                                        uint32_t soff = 0)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_untracked(lds), 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void copy4_to_lds_untracked(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                                       uint32_t soff = 0)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_untracked(lds), 4, voff, soff, 0, 0);
}

}  // namespace

// ---- query side: dq -----------------------------------------------------------
template <typename E, int D1, int D2>
__global__ __launch_bounds__(256, 2) void k_cmp_attn_bwd_dq(BwdParams p)
{
    constexpr int KT = 32, W = 4;
    using KR = SwzRows<D1>;
    using VR = SwzRows<D2>;
    constexpr int NKS = D1 / 16, NDS = D2 / 16, NDB1 = D1 / 32;
    constexpr int KIPW = (KR::INS + W - 1) / W, VIPW = (VR::INS + W - 1) / W;
    constexpr int KBUF = KIPW * W * 512, VBUF = VIPW * W * 512;   // with the slack of uneven copies
    constexpr int CPW = KIPW + VIPW;                              // copy instructions per wave and tile
    // Three K and three V slots, walked in a fixed order: a tile is copied
    // two tiles ahead of its use.
    __shared__ __attribute__((aligned(16))) uint16_t K0[KBUF], K1[KBUF], K2[KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t V0[VBUF], V1[VBUF], V2[VBUF];
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
        const int unit = (q * W + wave) * 64 + lane;
        kdo[q] = unit < KR::UNITS ? (uint32_t)(unit / KR::CH) * kst_b + (uint32_t)KR::chunk_of(unit) * 16u
                                  : 0x7FFFFFF0u;
    }
#pragma unroll
    for (int q = 0; q < VIPW; ++q) {
        const int unit = (q * W + wave) * 64 + lane;
        vdo[q] = unit < VR::UNITS ? (uint32_t)(unit / VR::CH) * vst_b + (uint32_t)VR::chunk_of(unit) * 16u
                                  : 0x7FFFFFF0u;
    }
    auto copy_tile = [&](int kt, uint16_t* kd, uint16_t* vd) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + (int64_t)kt * KT * kstride, tile_bytes(kt, kst_b, D1 * 2));
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + (int64_t)kt * KT * vstride, tile_bytes(kt, vst_b, D2 * 2));
        // every wave issues CPW copies per tile (slack ones land past the
        // tile in the slot, tiles past the end copy nothing but zeros), so
        // one immediate wait count fits every wave
#pragma unroll
        for (int q = 0; q < KIPW; ++q)
            copy16_to_lds_untracked(kr, kd + (q * W + wave) * 512, kdo[q]);
#pragma unroll
        for (int q = 0; q < VIPW; ++q)
            copy16_to_lds_untracked(vr, vd + (q * W + wave) * 512, vdo[q]);
    };
    // This wave's copies of the tile about to be read have landed (the next
    // tile's may still be in flight) and, after the barrier, every wave's;
    // every wave is done with the slot the next copy overwrites.
    auto step_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt((CPW & 15) | ((CPW >> 4) << 14) | 0x0070);
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
    const int ktb0 = KR::tr_base(lane);

    auto tile = [&](int kt, const uint16_t* ks_, const uint16_t* vs_) __attribute__((always_inline)) {
        // read offsets; with D1 = 192 the bases are made opaque to the
        // compiler so that the per-step offsets are formed here (a few XORs)
        // instead of held in registers, which two workgroups per CU lack
        int klb = KR::row_base(l32, hf), vlb = VR::row_base(l32, hf), ktb = ktb0;
        if constexpr (D1 > 128)
            __asm__ volatile("" : "+v"(klb), "+v"(vlb), "+v"(ktb));
        // S^T = K Q^T and dP^T = V dO^T (rows = keys, lane = query row)
        f32x16 s, dp;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            s[x] = 0.f;
            dp[x] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            s = E::mfma(*(const u32x4*)&ks_[KR::row_at(klb, ks)], qf[ks], s);
#pragma unroll
        for (int ks = 0; ks < NDS; ++ks)
            dp = E::mfma(*(const u32x4*)&vs_[VR::row_at(vlb, ks)], dof[ks], dp);
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
                dqa[db] = E::mfma(tr_read2(&ks_[KR::tr_lo(ktb, db) + kk * KR::KK], &ks_[KR::tr_hi(ktb, db) + kk * KR::KK]),
                                  dsf[kk], dqa[db]);
    };

    if (n_kt > 0) {
        copy_tile(0, K0, V0);
        copy_tile(1, K1, V1);
        for (int kt = 0; kt < n_kt; kt += 3) {
            step_barrier();
            copy_tile(kt + 2, K2, V2);
            tile(kt, K0, V0);
            if (kt + 1 >= n_kt)
                break;
            step_barrier();
            copy_tile(kt + 3, K0, V0);
            tile(kt + 1, K1, V1);
            if (kt + 2 >= n_kt)
                break;
            step_barrier();
            copy_tile(kt + 4, K1, V1);
            tile(kt + 2, K2, V2);
        }
        // the copies past the end land before the workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt(0x0070);
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

// ---- key side: dkc, dvc -----------------------------------------------------------
// One work item per workgroup: a block of kBwdKeyBlock = 128 compressed
// entries (keys) of one KV head and a range of the 32-row query tiles that
// see the block.  Each of the four waves owns 32 keys: K and V are its MFMA
// B operands in registers, dK^T and dV^T its accumulators.  The query tiles
// (rows of q and dout, then each row's exponent bias and Delta) stream
// through NS LDS slots shared by the four waves, copied by the buffer unit
// NS - 1 tiles ahead of their use, so a tile is fetched once for 128 keys
// and its copy latency is covered by NS - 1 steps of work.  Per tile and
// wave: S = Q K^T and dP = dO V^T (rows = queries, lane = key), P and
// dS = P (dP - Delta), then dV^T += dO^T P and dK^T += Q^T dS with the row
// tiles read transposed.  A block seen by more query tiles than an item
// holds is cut into pieces; a piece leaves unscaled dK and dV in its
// partial slot and k_cmp_attn_bwd_combine adds the pieces in order.
template <int D1, int D2>
struct DkvCfg {
    static constexpr int W = 4;
    static constexpr int KB = 32 * W;
    static_assert(KB == kBwdKeyBlock, "key block");
    using QR = SwzRows<D1>;
    using OR = SwzRows<D2>;
    static constexpr int QIW = (QR::INS + W - 1) / W;       // Q copy instructions per wave and tile
    static constexpr int OIW = (OR::INS + W - 1) / W;       // dout copy instructions per wave and tile
    static constexpr int QSZ = QIW * W * 512;               // elements of a slot's Q tile (with slack)
    static constexpr int OSZ = OIW * W * 512;
    static constexpr int SLOT_B = (QSZ + OSZ) * 2 + 64 * 4;  // + 32 rows x (bias, Delta)
    static constexpr int NS = 5;                            // slots: a tile is copied 4 steps ahead
    static_assert(NS * SLOT_B <= 150 * 1024, "slots do not fit in LDS");
    static constexpr int CPW = QIW + OIW + 1;               // copy instructions per wave and tile
    static constexpr int NW = (NS - 2) * CPW;               // copies still in flight when a tile is read
    static_assert(NW < 64, "wait count");
};

template <typename E, int D1, int D2>
__global__ __launch_bounds__(256, 1) void k_cmp_attn_bwd_dkv(BwdParams p)
{
    using C = DkvCfg<D1, D2>;
    using QR = typename C::QR;
    using OR = typename C::OR;
    constexpr int W = C::W;
    constexpr int NKS = D1 / 16, NDS = D2 / 16, NDB1 = D1 / 32, NDB2 = D2 / 32;
    // Five slot objects: the main loop walks them in a fixed order, so the
    // compiler sees that a step's LDS reads and the copies it issues touch
    // different objects and adds no wait of its own for the copies.
    __shared__ __attribute__((aligned(16))) unsigned char SL0[C::SLOT_B], SL1[C::SLOT_B], SL2[C::SLOT_B],
        SL3[C::SLOT_B], SL4[C::SLOT_B];
    if (*p.status != 0)
        return;   // the table failed the planner's checks

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const BwdItem it = p.items[blockIdx.x];
    const BatchEnt be = p.bt[it.b];
    const int g = it.g;
    const int G = p.G;
    const int key0 = it.kb * C::KB + wave * 32;     // the wave's first key (local)
    const int key = key0 + l32;
    const bool kvalid = key < be.n_cmp;
    const bool wave_has_keys = key0 < be.n_cmp;

    // keys and values as B operands: lane l32 = entry, k-slots 8hf..8hf+7
    u32x4 kf[NKS], vf[NDS];
    {
        const int64_t krow = ((int64_t)(be.cmp_off + (kvalid ? key : it.kb * C::KB)) * p.N2 + g);
        // S = (-q) k = q (-k): a negative scale negates the keys here and
        // leaves the query tiles as they are (dK needs the true q)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            kf[ks] = *(const u32x4*)(p.kc + krow * D1 + ks * 16 + hf * 8) ^ p.qsign;
#pragma unroll
        for (int ks = 0; ks < NDS; ++ks)
            vf[ks] = *(const u32x4*)(p.vc + krow * D2 + ks * 16 + hf * 8);
    }
    // query rows r = t*G + hh (local token t at position pos_off + t): the
    // first row that sees this lane's key, the first that sees the wave's
    // first key, and the first that sees the block's first key
    const int key_first_row = (key * p.d + p.l - 1 - be.pos_off) * G;
    const int wave_first_row = (key0 * p.d + p.l - 1 - be.pos_off) * G;
    const int rows_total = be.T * G;
    const int r_first = min(max(it.kb * C::KB * p.d + p.l - 1 - be.pos_off, 0), be.T) * G;

    const uint16_t* qseq = p.q + (int64_t)be.q_off * p.N1 * D1;
    const uint16_t* oseq = p.dout + (int64_t)be.q_off * p.N1 * D2;
    const float* sseq = p.rowstat + (int64_t)be.q_off * p.N1 * 2;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qseq, (uint32_t)((int64_t)be.T * p.N1 * D1 * 2));
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(oseq, (uint32_t)((int64_t)be.T * p.N1 * D2 * 2));
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(sseq, (uint32_t)((int64_t)be.T * p.N1 * 2 * 4));
    // element row of sequence row rr = t*G + hh: t*N1 + g*G + hh (t = rr / G
    // by a multiply-high with the host's magic number for G); the sequence's
    // rows span less than 4 GiB, so 32-bit byte offsets hold
    const uint32_t gG = (uint32_t)(g * G);
    auto row_elem = [&](int rr) -> uint32_t {
        const uint32_t t = (uint32_t)(((uint64_t)__umulhi((uint32_t)rr, p.gdiv_m) + (uint32_t)rr) >> p.gdiv_s);
        return t * (uint32_t)p.N1 + gG + ((uint32_t)rr - t * (uint32_t)G);
    };

    // Copies of tile tt (of the item) into a slot: every wave issues the same
    // number of copy instructions (slack ones land in the slot's slack), so
    // one immediate wait count fits all.  Lane (ins, lane) of a copy
    // instruction always fills row rr, chunk ch of the tile (or a pad or
    // slack position, never read).
    //
    // When G divides 32 or 32 divides G (the common head ratios), the
    // element row of tile row rr is u(r0) + L(rr) with
    //   u(r0) = (r0 / G) * N1 + g*G + r0 % G,  L(rr) = (rr / G) * N1 + rr % G
    // (r0, a multiple of 32 past the first row of a token, never splits a
    // tile across a token boundary when 32 divides G), so each lane's byte
    // offset is a constant and the tile a scalar offset: no vector work per
    // copy.  Rows past the sequence fall past the buffer and land as zeros;
    // tiles past the item load whatever they hold (they are never read).
    // Other ratios take the per-lane division, and rows past the sequence or
    // the item are pointed past the buffer.
    const bool affine = (G % 32 == 0) || (32 % G == 0);
    uint32_t qv[C::QIW], ov[C::OIW], sv;
    auto lane_row = [&](int rr) -> uint32_t { return (uint32_t)((rr / G) * p.N1 + rr % G); };
#pragma unroll
    for (int q = 0; q < C::QIW; ++q) {
        const int unit = (q * W + wave) * 64 + lane;
        qv[q] = unit < QR::UNITS ? lane_row(unit / QR::CH) * (uint32_t)(D1 * 2) + (uint32_t)QR::chunk_of(unit) * 16u : 0u;
    }
#pragma unroll
    for (int q = 0; q < C::OIW; ++q) {
        const int unit = (q * W + wave) * 64 + lane;
        ov[q] = unit < OR::UNITS ? lane_row(unit / OR::CH) * (uint32_t)(D2 * 2) + (uint32_t)OR::chunk_of(unit) * 16u : 0u;
    }
    sv = (lane_row(8 * wave + ((lane & 15) >> 1)) * 2u + (uint32_t)(lane & 1)) * 4u;
    auto issue = [&](int tt, unsigned char* slot) __attribute__((always_inline)) {
        const int r0 = r_first + 32 * (it.qt0 + tt);
        uint16_t* qd = (uint16_t*)slot;
        uint16_t* od = (uint16_t*)slot + C::QSZ;
        float* sd = (float*)(slot + (C::QSZ + C::OSZ) * 2);
        if (affine) {
            const uint32_t t0 = (uint32_t)(((uint64_t)__umulhi((uint32_t)r0, p.gdiv_m) + (uint32_t)r0) >> p.gdiv_s);
            const uint32_t u = t0 * (uint32_t)p.N1 + gG + ((uint32_t)r0 - t0 * (uint32_t)G);
#pragma unroll
            for (int q = 0; q < C::QIW; ++q)
                copy16_to_lds_untracked(qrs, qd + (q * W + wave) * 512, qv[q], u * (uint32_t)(D1 * 2));
#pragma unroll
            for (int q = 0; q < C::OIW; ++q)
                copy16_to_lds_untracked(ors, od + (q * W + wave) * 512, ov[q], u * (uint32_t)(D2 * 2));
            // rows 8*wave .. 8*wave+7: lane i < 16 copies float i%2 (bias,
            // Delta) of row 8*wave + i/2 to sd[16*wave + i]; the other lanes
            // stay inactive (they would land on the other waves' rows)
            if (lane < 16)
                copy4_to_lds_untracked(srs, sd + 16 * wave, sv, u * 8u);
            return;
        }
        const bool live = tt < it.n_qt;
#pragma unroll
        for (int q = 0; q < C::QIW; ++q) {
            const int ins = q * W + wave;
            const int unit = ins * 64 + lane;
            const int rr = min(unit / QR::CH, 31);
            const bool ok = live && unit < QR::UNITS && r0 + rr < rows_total;
            const uint32_t off = row_elem(r0 + rr) * (uint32_t)(D1 * 2) + (uint32_t)QR::chunk_of(unit) * 16u;
            copy16_to_lds_untracked(qrs, qd + ins * 512, ok ? off : 0xFFFFFFF0u);
        }
#pragma unroll
        for (int q = 0; q < C::OIW; ++q) {
            const int ins = q * W + wave;
            const int unit = ins * 64 + lane;
            const int rr = min(unit / OR::CH, 31);
            const bool ok = live && unit < OR::UNITS && r0 + rr < rows_total;
            const uint32_t off = row_elem(r0 + rr) * (uint32_t)(D2 * 2) + (uint32_t)OR::chunk_of(unit) * 16u;
            copy16_to_lds_untracked(ors, od + ins * 512, ok ? off : 0xFFFFFFF0u);
        }
        if (lane < 16) {
            const int rr = 8 * wave + (lane >> 1);
            const bool ok = live && r0 + rr < rows_total;
            const uint32_t off = (row_elem(r0 + rr) * 2u + (uint32_t)(lane & 1)) * 4u;
            copy4_to_lds_untracked(srs, sd + 16 * wave, ok ? off : 0xFFFFFFF0u);
        }
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
    const int qtb0 = QR::tr_base(lane), otb0 = OR::tr_base(lane);
    const float c = p.c;

    // Step tt: wait until tile tt's copies have landed (the NS - 2 later
    // tiles may still be in flight) and this wave's LDS reads of the previous
    // tile are done; after the barrier every wave's copies are visible and
    // every wave is done with the slot the next copy overwrites.
    auto step = [&](int tt, const unsigned char* rd, unsigned char* cp) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt((C::NW & 15) | ((C::NW >> 4) << 14) | 0x0070);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        issue(tt + C::NS - 1, cp);

        const int r0 = r_first + 32 * (it.qt0 + tt);
        if (!wave_has_keys || r0 + 31 < wave_first_row)
            return;                                  // no row of the tile sees a key of this wave
        const uint16_t* qs = (const uint16_t*)rd;
        const uint16_t* os = (const uint16_t*)rd + C::QSZ;
        const float* st = (const float*)(rd + (C::QSZ + C::OSZ) * 2);
        // Four phases, each a run of MFMAs with the vector work that does
        // not depend on them beside it:
        //   1. S = Q K^T (rows = queries 8*(x/4) + 4*hf + x%4, lane = entry);
        //   2. dP = dO V^T, beside P = exp2(S c - bias);
        //   3. dV^T += dO^T P, beside dS = P (dP - Delta);
        //   4. dK^T += Q^T dS.
        // Only the causal test is needed for P: rows past the sequence were
        // copied as zeros (q, dout, bias and Delta), which makes their dS and
        // their dout rows zero, and keys past the block's entries are never
        // stored.  Element x is row r0 + 8*(x/4) + 4*hf + x%4, visible iff
        // that row >= key_first_row.
        f32x16 sc, dp;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            sc[x] = 0.f;
            dp[x] = 0.f;
        }
        const int qlb = QR::row_base(l32, hf), olb = OR::row_base(l32, hf), qtb = qtb0, otb = otb0;
        f32x4 stv[8];   // (bias, Delta) of rows 8*r4 + 4*hf + {0, 1}, then {2, 3}
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            stv[2 * r4] = *(const f32x4*)&st[2 * (8 * r4 + 4 * hf)];
            stv[2 * r4 + 1] = *(const f32x4*)&st[2 * (8 * r4 + 4 * hf) + 4];
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            sc = E::mfma(*(const u32x4*)&qs[QR::row_at(qlb, ks)], kf[ks], sc);
        __builtin_amdgcn_sched_barrier(0);
        const int d0 = r0 + 4 * hf - key_first_row;
        float pv[16];
        u32x4 pf[2], dsf[2];
#pragma unroll
        for (int ks = 0; ks < NDS; ++ks)
            dp = E::mfma(*(const u32x4*)&os[OR::row_at(olb, ks)], vf[ks], dp);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r4 = x >> 2, e = x & 3;
            const float bias = stv[2 * r4 + (e >> 1)][(e & 1) * 2];
            const float pr = fast_exp2(fmaf(sc[x], c, -bias));
            pv[x] = d0 >= -(8 * r4 + e) ? pr : 0.f;
            if (x & 1)
                pf[r4 >> 1][(r4 & 1) * 2 + (e >> 1)] = E::pack2(pv[x - 1], pv[x]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // Phases 3 and 4 as one run of 2*(NDB2 + NDB1) products: dV blocks
        // (kk-major) then dK blocks, each operand read three products ahead
        // of its use; the dS work sits beside the dV products.
        constexpr int NGV = 2 * NDB2, NG = NGV + 2 * NDB1, PF = 3;
        auto g_operand = [&](int m) __attribute__((always_inline)) -> u32x4 {
            if (m < NGV)
                return tr_read2(&os[OR::tr_lo(otb, m % NDB2) + (m / NDB2) * OR::KK],
                                &os[OR::tr_hi(otb, m % NDB2) + (m / NDB2) * OR::KK]);
            const int j = m - NGV;
            return tr_read2(&qs[QR::tr_lo(qtb, j % NDB1) + (j / NDB1) * QR::KK],
                            &qs[QR::tr_hi(qtb, j % NDB1) + (j / NDB1) * QR::KK]);
        };
        u32x4 ga[NG];
#pragma unroll
        for (int m = 0; m < PF; ++m)
            ga[m] = g_operand(m);
#pragma unroll
        for (int m = 0; m < NG; ++m) {
            if (m + PF < NG)
                ga[m + PF] = g_operand(m + PF);
            if (m < NGV) {
                dva[m % NDB2] = E::mfma(ga[m], pf[m / NDB2], dva[m % NDB2]);
#pragma unroll
                for (int x = 1; x < 16; x += 2) {
                    if (((x >> 1) * NGV) / 8 != m)
                        continue;
                    const int r4 = x >> 2, e = x & 3;
                    const f32x4& v = stv[2 * r4 + (e >> 1)];
                    dsf[r4 >> 1][(r4 & 1) * 2 + (e >> 1)] =
                        E::pack2(pv[x - 1] * (dp[x - 1] - v[1]), pv[x] * (dp[x] - v[3]));
                }
            } else {   // the true q: dkc = scale * sum dS q
                const int j = m - NGV;
                dka[j % NDB1] = E::mfma(ga[m], dsf[j / NDB1], dka[j % NDB1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // tile tt lives in slot tt % 5; step tt refills the slot step tt - 1 read
    issue(0, SL0);
    issue(1, SL1);
    issue(2, SL2);
    issue(3, SL3);
    for (int tt = 0; tt < it.n_qt; tt += 5) {
        step(tt, SL0, SL4);
        if (tt + 1 >= it.n_qt)
            break;
        step(tt + 1, SL1, SL0);
        if (tt + 2 >= it.n_qt)
            break;
        step(tt + 2, SL2, SL1);
        if (tt + 3 >= it.n_qt)
            break;
        step(tt + 3, SL3, SL2);
        if (tt + 4 >= it.n_qt)
            break;
        step(tt + 4, SL4, SL3);
    }
    // the copies of the tiles past the end (zeros) land before the
    // workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0x0070);

    // lane = key, 4 consecutive dims per register quad
    auto store = [&](auto& acc, auto nb_tag, float* dst, float mul) __attribute__((always_inline)) {
        constexpr int NB = decltype(nb_tag)::value;
#pragma unroll
        for (int db = 0; db < NB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *(f32x4*)(dst + db * 32 + 8 * r4 + 4 * hf) =
                    f32x4{acc[db][4 * r4] * mul, acc[db][4 * r4 + 1] * mul, acc[db][4 * r4 + 2] * mul,
                          acc[db][4 * r4 + 3] * mul};
    };
    if (it.slot < 0) {
        if (kvalid) {
            const int64_t krow = (int64_t)(be.cmp_off + key) * p.N2 + g;
            store(dka, std::integral_constant<int, NDB1>{}, p.dkc + krow * D1, p.scale);
            store(dva, std::integral_constant<int, NDB2>{}, p.dvc + krow * D2, 1.f);
        }
    } else {
        float* dst = p.part + ((int64_t)it.slot * C::KB + wave * 32 + l32) * (D1 + D2);
        store(dka, std::integral_constant<int, NDB1>{}, dst, 1.f);
        store(dva, std::integral_constant<int, NDB2>{}, dst + D1, 1.f);
    }
}

// Key blocks cut into pieces: per entry and dim, the pieces' partial sums
// added in piece order (bitwise repeatable), dK scaled, then stored.
template <int D1, int D2>
__global__ __launch_bounds__(256) void k_cmp_attn_bwd_combine(BwdParams p)
{
    if (*p.status != 0)
        return;
    const CombineItem it = p.combs[blockIdx.x];
    const BatchEnt be = p.bt[it.b];
    constexpr int DC = D1 + D2;
    constexpr int Q4 = DC / 4;
    const int64_t piece = (int64_t)kBwdKeyBlock * DC;
    for (int u = threadIdx.x; u < kBwdKeyBlock * Q4; u += 256) {
        const int kl = u / Q4, e = (u - kl * Q4) * 4;
        const int key = it.rb * kBwdKeyBlock + kl;
        if (key >= be.n_cmp)
            continue;
        const float* src = p.part + ((int64_t)it.slot0 * kBwdKeyBlock + kl) * DC + e;
        f32x4 acc = *(const f32x4*)src;
        for (int s = 1; s < it.n; ++s) {
            const f32x4 v = *(const f32x4*)(src + s * piece);
            acc[0] += v[0];
            acc[1] += v[1];
            acc[2] += v[2];
            acc[3] += v[3];
        }
        const int64_t krow = (int64_t)(be.cmp_off + key) * p.N2 + it.g;
        if (e < D1)
            *(f32x4*)(p.dkc + krow * D1 + e) = f32x4{acc[0] * p.scale, acc[1] * p.scale, acc[2] * p.scale,
                                                     acc[3] * p.scale};
        else
            *(f32x4*)(p.dvc + krow * D2 + (e - D1)) = acc;
    }
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
static hipError_t launch_bwd_typed(int d1, int d2, const BwdParams& p, int tiles_q, int n_items, int n_combs,
                                   hipStream_t stream)
{
#define X(a, b_)                                                                                      \
    if (d1 == a && d2 == b_) {                                                                        \
        if (tiles_q > 0)                                                                              \
            hipLaunchKernelGGL((k_cmp_attn_bwd_dq<E, a, b_>), dim3(tiles_q), dim3(256), 0, stream, p);   \
        if (n_items > 0)                                                                              \
            hipLaunchKernelGGL((k_cmp_attn_bwd_dkv<E, a, b_>), dim3(n_items), dim3(256), 0, stream, p);  \
        if (n_combs > 0)                                                                              \
            hipLaunchKernelGGL((k_cmp_attn_bwd_combine<a, b_>), dim3(n_combs), dim3(256), 0, stream, p); \
        return hipGetLastError();                                                                     \
    }
    NSA_BWD_CONFIGS(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd(int dtype, int d1, int d2, const BwdParams& p, int tiles_q, int n_items, int n_combs,
                           hipStream_t stream)
{
    if (dtype == ElemBf16::code)
        return launch_bwd_typed<ElemBf16>(d1, d2, p, tiles_q, n_items, n_combs, stream);
    if (dtype == ElemF16::code)
        return launch_bwd_typed<ElemF16>(d1, d2, p, tiles_q, n_items, n_combs, stream);
    return hipErrorInvalidValue;
}

}  // namespace nsa
