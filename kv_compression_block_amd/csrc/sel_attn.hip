// Selected-block attention: the step of Native Sparse Attention that
// consumes topk_indices.  The pages give it only as an interface
// ("lite_boost.ops.rain_fusion_attention": a -1 padded list of KV blocks per
// query, output plus softmax log-sum-exp); the reading implemented here:
// query token t (local position), head h of KV group g attends to the raw
// keys s <= t of its sequence whose select block floor(s / l') is listed in
// topk_indices[t, g, :]; -1, repeats and entries past the sequence's last
// block add nothing; a query with no such key has output 0 and lse -inf.
//
// Design (gfx950, bf16 or f16 MFMA 32x32x16, fp32 accumulate):
//   * A workgroup is two waves, 64 rows of (token, query head of group g):
//     one token for groups of 64, a few for smaller groups.  The heads of a
//     token share its block list, so the workgroup walks the union of its
//     tokens' lists (bit sets built in LDS with LDS atomics) in ascending
//     key order, 32-key tiles, skipping keys past its last token; a row
//     masks the tiles of blocks its own token did not list and its future.
//   * Key and value tiles are copied from global memory into LDS by the
//     buffer unit, whole rows per instruction (keys with 16 bytes of row
//     padding, values with XOR-swizzled chunks read transposed for the P.V
//     operand), two slots each, shared by both waves.  Step i issues the
//     copies of K(i+2) and V(i+1), then the scores of tile i+1 beside the
//     exponentials and P.V of tile i, then the mask and max of tile i+1;
//     one barrier per step (after waiting for the previous step's copies).
//   * S^T = K Q^T (a lane owns one query row), online softmax in base 2
//     with a lazily moved reference max, O^T += V^T P^T.
#include "nsa_device.h"

namespace nsa {

template <int D1, int D2>
struct SelCfg {
    static constexpr int W = kSelRows / 32;      // waves per workgroup
    static constexpr int KT = 32;                // keys per tile
    static constexpr int KS = D1 + 8;            // LDS row stride of K (elements): 16 B pad
    static constexpr int NKS = D1 / 16;          // k-steps of QK^T
    static constexpr int NDB = D2 / 32;          // 32-dim blocks of O^T
    static constexpr int KCH = D1 / 8;           // 16-byte chunks per key row
    static constexpr int VCH = D2 / 8;           // 16-byte chunks per value row
    static constexpr int KINS = (KT * (KCH + 1) + 63) / 64;   // copy instructions per K tile
    static constexpr int KIPW = (KINS + W - 1) / W;           // ... per wave
    static constexpr int KBUF = KINS * 64 * 8;                // elements per K slot
    static constexpr int VINS = KT * VCH / 64;                // copy instructions per V tile
    static constexpr int VIPW = VINS / W;
    static_assert((KT * VCH) % (64 * W) == 0, "value tile copy");
    static_assert(D2 == 64 || D2 == 128, "value swizzle");
};

template <typename E, int D1, int D2>
__global__ __launch_bounds__(kSelRows * 2, 2) void k_sel_attn_fwd(SelParams p)
{
    using C = SelCfg<D1, D2>;
    constexpr int KT = C::KT;
    constexpr int W = C::W;
    // Two K and two V slots, each its own LDS object (the compiler then
    // waits only for copies into the slot a read touches); the block sets
    // follow in dynamic LDS.
    __shared__ __attribute__((aligned(16))) uint16_t K0[C::KBUF], K1[C::KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t V0[KT * D2], V1[KT * D2];
    extern __shared__ __attribute__((aligned(16))) uint32_t sel_bits[];
    if (*p.status != 0)
        return;   // the table failed the planner's checks

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int wg = blockIdx.x;
    // largest b with tile_off_s(b) <= wg
    int b = 0;
    {
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.bt[mid].tile_off_s <= wg)
                lo = mid;
            else
                hi = mid - 1;
        }
        b = lo;
    }
    const BatchEnt be = p.bt[b];
    const int idx = wg - be.tile_off_s;
    const int g = idx % p.N2;
    const int rb = be.n_rb_s - 1 - idx / p.N2;
    const int G = p.G;
    const int rows_total = be.T * G;
    const int row_wg = rb * kSelRows;
    const int row_last = min(row_wg + kSelRows, rows_total) - 1;
    const int t_lo = row_wg / G, t_hi = row_last / G;     // the workgroup's tokens
    const int ntok = t_hi - t_lo + 1;

    // ---- this lane's row -------------------------------------------------------
    const int r = row_wg + wave * 32 + l32;
    const bool vq = r < rows_total;
    const int tok = vq ? r / G : t_lo;
    const int64_t grow = (int64_t)(be.q_off + tok) * p.N1 + (int64_t)g * G + (r - (r / G) * G);
    u32x4 qf[C::NKS];
    {
        const int64_t qsrc = vq ? grow : (int64_t)(be.q_off + t_lo) * p.N1 + (int64_t)g * G;
        const uint16_t* qrow = p.q + qsrc * D1 + hf * 8;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
            qf[ks] = *(const u32x4*)(qrow + ks * 16) ^ p.qsign;
    }

    // ---- block sets: per token, and their union ----------------------------------
    const int sw = p.sw;
    uint32_t* tbits = sel_bits;                  // [ntok][sw]
    uint32_t* ubits = sel_bits + p.tpw * sw;     // [sw]
    for (int x = tid; x < p.tpw * sw + sw; x += 64 * W)
        sel_bits[x] = 0u;
    __syncthreads();
    // Chunked prefill: query t sits at position pos_off + t among the
    // sequence's Tkv = T + pos_off key/value tokens (bottom-right alignment).
    const int pos_hi = t_hi + be.pos_off;
    const int jmax = min(pos_hi / p.lsel, be.S_sel - 1);   // later blocks hold only future keys
    for (int e = tid; e < ntok * p.count; e += 64 * W) {
        const int tt = e / p.count;
        const int j = p.topk[((int64_t)(be.q_off + t_lo + tt) * p.N2 + g) * p.count + (e - tt * p.count)];
        if (j >= 0 && j <= jmax) {
            atomicOr(&tbits[tt * sw + (j >> 5)], 1u << (j & 31));
            atomicOr(&ubits[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();
    const uint32_t uw = lane < sw ? ubits[lane] : 0u;      // lane w holds union word w
    const uint32_t* my_bits = tbits + (tok - t_lo) * sw;

    // First listed block >= jfrom, or -1 (uniform: every wave holds the union).
    auto first_block = [&](int jfrom) -> int {
        if (jfrom > jmax)
            return -1;
        const int wi = jfrom >> 5;
        uint32_t w = lane < wi ? 0u : uw;
        if (lane == wi)
            w &= ~0u << (jfrom & 31);
        const uint64_t nz = __ballot(w != 0u);
        if (nz == 0)
            return -1;
        const int L = (int)__builtin_ctzll(nz);
        const uint32_t wl = (uint32_t)__shfl((int)w, L);
        const int j = __builtin_amdgcn_readfirstlane(L * 32 + (int)__builtin_ctz(wl));
        return j <= jmax ? j : -1;
    };
    // Tiles are (block j, 32-key part u); parts that start past the last
    // token are skipped.  A tile is its first key, -1 for none.
    const int nsub = p.lsel / KT;
    auto next_key0 = [&](int key0) -> int {
        if (key0 < 0)
            return -1;
        const int j = key0 / p.lsel, u = (key0 - j * p.lsel) / KT;
        if (u + 1 < nsub && key0 + KT <= pos_hi)
            return key0 + KT;
        const int jn = first_block(j + 1);
        return jn < 0 ? -1 : jn * p.lsel;
    };

    // ---- tile copies into LDS ----------------------------------------------------
    const int64_t kstride = (int64_t)p.N2 * D1;
    const int64_t vstride = (int64_t)p.N2 * D2;
    const uint16_t* kbase = p.k + ((int64_t)be.kv_off * p.N2 + g) * D1;
    const uint16_t* vbase = p.v + ((int64_t)be.kv_off * p.N2 + g) * D2;
    const int Tkv = be.T + be.pos_off;
    const uint32_t kst_b = (uint32_t)(kstride * 2), vst_b = (uint32_t)(vstride * 2);
    // keys key0 .. key0+31 of the sequence; rows past its end load as zero
    auto tile_bytes = [&](int key0, uint32_t stride_b, int row_bytes) -> uint32_t {
        const int nvalid = min(KT, Tkv - key0);
        return nvalid > 0 ? (uint32_t)(nvalid - 1) * stride_b + (uint32_t)row_bytes : 0u;
    };
    // Global byte offset (inside a tile) each lane copies into LDS slot
    // 64*q + lane of instruction q; padding slots point past any tile.
    uint32_t kdo[C::KIPW], vdo[C::VIPW];
#pragma unroll
    for (int q = 0; q < C::KIPW; ++q) {
        const int slot = (q * W + wave) * 64 + lane;
        const int kr = slot / (C::KCH + 1), ch = slot % (C::KCH + 1);
        kdo[q] = (ch < C::KCH && kr < KT) ? (uint32_t)kr * kst_b + (uint32_t)ch * 16u : 0x7FFFFFF0u;
    }
#pragma unroll
    for (int q = 0; q < C::VIPW; ++q) {
        const int slot = (q * W + wave) * 64 + lane;
        const int vr = slot / C::VCH;
        const int ch = v_swz<D2>(vr, slot % C::VCH);
        vdo[q] = (uint32_t)vr * vst_b + (uint32_t)ch * 16u;
    }
    auto load_k = [&](int key0, uint16_t* dst) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(kbase + (int64_t)key0 * kstride, tile_bytes(key0, kst_b, D1 * 2));
#pragma unroll
        for (int q = 0; q < C::KIPW; ++q)
            if (q < C::KINS / W || q * W + wave < C::KINS)
                copy16_to_lds(rs, dst + (q * W + wave) * 512, kdo[q]);
    };
    auto load_v = [&](int key0, uint16_t* dst) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(vbase + (int64_t)key0 * vstride, tile_bytes(key0, vst_b, D2 * 2));
#pragma unroll
        for (int q = 0; q < C::VIPW; ++q)
            copy16_to_lds(rs, dst + (q * W + wave) * 512, vdo[q]);
    };
    // This wave's copies have landed, and (after the barrier) every wave's;
    // every wave is also done with the previous step's LDS reads.  The copies
    // write LDS behind the compiler's back, hence the explicit wait and the
    // empty asm statements that keep LDS accesses on their side.
    auto step_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0070);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };
    int voff_lane[C::NDB];
    {
        const int vi = lane & 15, vgrp = (lane >> 4) & 1;
        const int r0 = 4 * hf + (vi >> 2);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const int dim = db * 32 + 16 * vgrp + 4 * (vi & 3);
            voff_lane[db] = r0 * D2 + v_swz<D2>(r0, dim >> 3) * 8 + (dim & 7);
        }
    }

    // ---- state -----------------------------------------------------------------
    f32x16 o[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x)
            o[db][x] = 0.f;
    float mref = -INFINITY, mtrue = -INFINITY, lsum = 0.f, nbias = 0.f;
    const float c = p.c;

    auto qk = [&](const uint16_t* kbuf, f32x16& sc) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < 16; ++x)
            sc[x] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            const u32x4 ka = *(const u32x4*)&kbuf[l32 * C::KS + ks * 16 + hf * 8];
            sc = E::mfma(ka, qf[ks], sc);
        }
    };
    // Mask and max of a tile's scores; moves the reference max (rescaling O
    // and the running sum) when a row asks for it, then the exponent bias.
    // Key key0 + 8*(x/4) + 4*hf + x%4 is kept iff its block is listed for
    // this row's token and the key is not in its future.
    auto mask_max = [&](int key0, f32x16& sc) __attribute__((always_inline)) {
        const int j = key0 / p.lsel;
        const bool listed = (my_bits[j >> 5] >> (j & 31)) & 1u;
        const int lim = listed ? tok + be.pos_off - key0 - 4 * hf + 1 : 0;
        if (__ballot(lim < 32) != 0) {
#pragma unroll
            for (int x = 0; x < 16; ++x)
                sc[x] = (8 * (x >> 2) + (x & 3) < lim) ? sc[x] : -INFINITY;
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int x = 0; x < 16; ++x)
            tmax = fmaxf(tmax, sc[x]);
        tmax = half_max(tmax);
        mtrue = fmaxf(mtrue, tmax);
        if (__builtin_expect(__ballot(tmax > mref + p.thr) != 0, 0)) {
            float alpha = 1.f;
            if (tmax > mref + p.thr) {
                alpha = (mref == -INFINITY) ? 0.f : fast_exp2((mref - tmax) * c);
                mref = tmax;
            }
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x)
                    o[db][x] *= alpha;
        }
        nbias = (mref == -INFINITY) ? 0.f : -mref * c;
    };
    auto softmax_pv = [&](f32x16& sc, const uint16_t* vbuf) __attribute__((always_inline)) {
        float ps = 0.f;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            sc[x] = fast_exp2(fmaf(sc[x], c, nbias));
            ps += sc[x];
        }
        lsum += ps;
        u32x4 pf[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pf[kk][q] = E::pack2(sc[kk * 8 + 2 * q], sc[kk * 8 + 2 * q + 1]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                const uint16_t* vb = &vbuf[voff_lane[db] + kk * 16 * D2];
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * D2));
                const u32x4 va = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = E::mfma(va, pf[kk], o[db]);
            }
        }
    };

    // ---- tile pipeline -----------------------------------------------------------
    // Tile i lives in K slot i%2 and V slot i%2.  Step i: barrier (the
    // copies of K(i+1) and V(i) have landed, QK(i) and P.V(i-1) are done
    // everywhere), copies of K(i+2) into K slot i%2 and V(i+1) into V slot
    // (i+1)%2, scores of tile i+1, exponentials and P.V of tile i, mask and
    // max of tile i+1.
    f32x16 scur, snxt;
    int ka = first_block(0);                       // key0 of tiles i, i+1, i+2
    ka = ka < 0 ? -1 : ka * p.lsel;
    int kb = next_key0(ka);
    int kc = next_key0(kb);
    if (ka >= 0) {
        load_k(ka, K0);
        load_v(ka, V0);
        if (kb >= 0)
            load_k(kb, K1);
        step_barrier();
        qk(K0, scur);
        mask_max(ka, scur);
    }
    auto step = [&](uint16_t* k_this, uint16_t* k_other, uint16_t* v_this, uint16_t* v_other) __attribute__((always_inline)) {
        step_barrier();
        if (kc >= 0)
            load_k(kc, k_this);
        if (kb >= 0) {
            load_v(kb, v_other);
            qk(k_other, snxt);
        }
        softmax_pv(scur, v_this);
        if (kb >= 0) {
            mask_max(kb, snxt);
            scur = snxt;
        }
        ka = kb;
        kb = kc;
        kc = next_key0(kc);
    };
    while (ka >= 0) {
        step(K0, K1, V0, V1);
        if (ka < 0)
            break;
        step(K1, K0, V1, V0);
    }

    // ---- outputs -------------------------------------------------------------------
    const float lf = half_sum(lsum);
    const bool empty = (mtrue == -INFINITY);
    const float inv = empty ? 0.f : 1.f / lf;
    if (vq) {
        uint16_t* orow = p.out + grow * D2;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dv = db * 32 + 8 * r4 + 4 * hf;
                u32x2 w2 = {E::pack2(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv),
                            E::pack2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv)};
                *(u32x2*)(orow + dv) = w2;
            }
        }
        if (hf == 0)
            p.lse[grow] = empty ? -INFINITY : mref * p.abs_scale + __builtin_logf(lf);
    }
}

#define NSA_SEL_CONFIGS(X) X(64, 64) X(128, 64) X(128, 128) X(192, 64) X(192, 128)

bool sel_attn_supported(int d1, int d2)
{
#define X(a, b) if (d1 == a && d2 == b) return true;
    NSA_SEL_CONFIGS(X)
#undef X
    return false;
}

size_t sel_attn_lds_bytes(int tpw, int sw) { return (size_t)(tpw + 1) * sw * 4; }

template <typename E>
static hipError_t launch_sel_typed(int d1, int d2, const SelParams& p, int n_tiles, size_t lds,
                                   hipStream_t stream)
{
#define X(a, b)                                                                                    \
    if (d1 == a && d2 == b) {                                                                      \
        hipLaunchKernelGGL((k_sel_attn_fwd<E, a, b>), dim3(n_tiles), dim3(kSelRows * 2), lds, stream, p); \
        return hipGetLastError();                                                                  \
    }
    NSA_SEL_CONFIGS(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_sel_attn(int dtype, int d1, int d2, const SelParams& p, int n_tiles, size_t lds,
                           hipStream_t stream)
{
    if (n_tiles <= 0)
        return hipSuccess;
    if (dtype == ElemBf16::code)
        return launch_sel_typed<ElemBf16>(d1, d2, p, n_tiles, lds, stream);
    if (dtype == ElemF16::code)
        return launch_sel_typed<ElemF16>(d1, d2, p, n_tiles, lds, stream);
    return hipErrorInvalidValue;
}

}  // namespace nsa
