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
//   * Rows are (token, query head of group g), 32 per wave, four independent
//     waves per workgroup: the heads of a token share its block list, so for
//     groups of 32 or more a wave's rows belong to one token; smaller groups
//     put several tokens in a wave, which then walks the union of their
//     lists and masks per row.
//   * A wave first turns its tokens' index lists into per-token bit sets and
//     their union in LDS (LDS atomics), then visits the listed blocks in
//     ascending order in 32-key tiles, skipping keys past its last token.
//   * Keys go straight from global memory into the MFMA A-operand registers
//     (one 16-byte load per lane and k-step, the operand layout is the row
//     layout), two register sets alternating; value tiles are copied into
//     two per-wave LDS slots by the buffer unit and read transposed for the
//     P.V operand (ds_read_b64_tr_b16), as in the compressed attention.
//     Tile i+1 is in flight while tile i is computed.
//   * S^T = K Q^T (a lane owns one query row), online softmax in base 2
//     with a lazily moved reference max, O^T += V^T P^T; the row's mask is
//     one bit per tile (is the block listed for its token) plus the causal
//     limit inside the token's own block.
#include "nsa_device.h"

namespace nsa {

template <int D1, int D2>
struct SelCfg {
    static constexpr int KT = 32;                // keys per tile
    static constexpr int NKS = D1 / 16;          // k-steps of QK^T
    static constexpr int NDB = D2 / 32;          // 32-dim blocks of O^T
    static constexpr int VCH = D2 / 8;           // 16-byte chunks per value row
    static constexpr int VINS = KT * VCH / 64;   // wave copy instructions per value tile
    static constexpr int VSLOT = KT * D2;        // elements per value slot
    static_assert(D2 == 64 || D2 == 128, "value swizzle");
};

constexpr int kSelWaves = 4;

template <typename E, int D1, int D2>
__global__ __launch_bounds__(64 * kSelWaves, 2) void k_sel_attn_fwd(SelParams p)
{
    using C = SelCfg<D1, D2>;
    constexpr int KT = C::KT;
    // Two value slots per wave, each its own LDS object (the compiler then
    // waits only for copies into the slot a read touches); per-wave token
    // bit sets and their union follow in dynamic LDS.
    __shared__ __attribute__((aligned(16))) uint16_t VS0[kSelWaves * C::VSLOT], VS1[kSelWaves * C::VSLOT];
    extern __shared__ __attribute__((aligned(16))) uint32_t sel_bits[];

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
    const int row_w = rb * (32 * kSelWaves) + wave * 32;   // first row of this wave
    if (row_w >= rows_total)
        return;                                             // waves never wait for each other
    const int row_last = min(row_w + 31, rows_total - 1);
    const int t_lo = row_w / G, t_hi = row_last / G;       // this wave's tokens
    const int ntok = t_hi - t_lo + 1;

    // ---- this lane's row -------------------------------------------------------
    const int r = row_w + l32;
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
    uint32_t* tbits = sel_bits + wave * (p.tpw + 1) * sw;   // [ntok][sw]
    uint32_t* ubits = tbits + p.tpw * sw;                    // [sw]
    for (int x = lane; x < (ntok + 1) * sw; x += 64)
        (x < ntok * sw ? tbits[x] : ubits[x - ntok * sw]) = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int jmax = min(t_hi / p.lsel, be.S_sel - 1);      // later blocks hold only future keys
    for (int e = lane; e < ntok * p.count; e += 64) {
        const int tt = e / p.count;
        const int j = p.topk[((int64_t)(be.q_off + t_lo + tt) * p.N2 + g) * p.count + (e - tt * p.count)];
        if (j >= 0 && j <= jmax) {
            atomicOr(&tbits[tt * sw + (j >> 5)], 1u << (j & 31));
            atomicOr(&ubits[j >> 5], 1u << (j & 31));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t uw = lane < sw ? ubits[lane] : 0u;       // lane w holds union word w
    const uint32_t* my_bits = tbits + (tok - t_lo) * sw;

    // First listed block >= jfrom, or -1 (wave-uniform).
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
        const int j = L * 32 + (int)__builtin_ctz(wl);
        return j <= jmax ? j : -1;
    };
    // Tiles: (block j, 32-key part u); parts that start past the last token
    // are skipped.
    const int nsub = p.lsel / KT;
    auto next_tile = [&](int& j, int& u) {
        if (u + 1 < nsub && j * p.lsel + (u + 1) * KT <= t_hi) {
            ++u;
        } else {
            j = first_block(j + 1);
            u = 0;
        }
    };

    // ---- tile loads ----------------------------------------------------------------
    const int64_t kstride = (int64_t)p.N2 * D1;
    const int64_t vstride = (int64_t)p.N2 * D2;
    const uint16_t* kbase = p.k + ((int64_t)be.q_off * p.N2 + g) * D1;
    const uint16_t* vbase = p.v + ((int64_t)be.q_off * p.N2 + g) * D2;
    const uint32_t kst_b = (uint32_t)(kstride * 2), vst_b = (uint32_t)(vstride * 2);
    // keys key0 .. key0+31 of the sequence; rows past its end load as zero
    auto tile_bytes = [&](int key0, uint32_t stride_b, int row_bytes) -> uint32_t {
        const int nvalid = min(KT, be.T - key0);
        return nvalid > 0 ? (uint32_t)(nvalid - 1) * stride_b + (uint32_t)row_bytes : 0u;
    };
    uint32_t vdo[C::VINS];
#pragma unroll
    for (int q = 0; q < C::VINS; ++q) {
        const int slot = q * 64 + lane;
        const int vr = slot / C::VCH;
        const int ch = v_swz<D2>(vr, slot % C::VCH);
        vdo[q] = (uint32_t)vr * vst_b + (uint32_t)ch * 16u;
    }
    auto load_k = [&](int key0, u32x4 (&kr)[C::NKS]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(kbase + (int64_t)key0 * kstride, tile_bytes(key0, kst_b, D1 * 2));
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
            kr[ks] = buffer_load16(rs, (uint32_t)l32 * kst_b + (uint32_t)(ks * 32 + hf * 16));
    };
    auto load_v = [&](int key0, uint16_t* slot) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(vbase + (int64_t)key0 * vstride, tile_bytes(key0, vst_b, D2 * 2));
#pragma unroll
        for (int q = 0; q < C::VINS; ++q)
            copy16_to_lds(rs, slot + q * 512, vdo[q]);
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
    float mref = -INFINITY, mtrue = -INFINITY, lsum = 0.f;
    const float c = p.c;

    // One tile: scores, mask, online softmax, P.V.
    auto tile = [&](int j, int u, const u32x4 (&kr)[C::NKS], const uint16_t* vslot) __attribute__((always_inline)) {
        const int key0 = j * p.lsel + u * KT;
        f32x16 s;
#pragma unroll
        for (int x = 0; x < 16; ++x)
            s[x] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
            s = E::mfma(kr[ks], qf[ks], s);
        // key key0 + 8*(x/4) + 4*hf + x%4 is kept iff block j is listed for
        // this row's token and the key is not in its future
        const bool listed = (my_bits[j >> 5] >> (j & 31)) & 1u;
        const int lim = listed ? tok - key0 - 4 * hf + 1 : 0;
        if (__ballot(lim < 32) != 0) {
#pragma unroll
            for (int x = 0; x < 16; ++x)
                s[x] = (8 * (x >> 2) + (x & 3) < lim) ? s[x] : -INFINITY;
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int x = 0; x < 16; ++x)
            tmax = fmaxf(tmax, s[x]);
        tmax = half_max(tmax);
        mtrue = fmaxf(mtrue, tmax);
        if (__ballot(tmax > mref + p.thr) != 0) {
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
        const float nbias = (mref == -INFINITY) ? 0.f : -mref * c;
        float ps = 0.f;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            s[x] = fast_exp2(fmaf(s[x], c, nbias));
            ps += s[x];
        }
        lsum += ps;
        u32x4 pf[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pf[kk][q] = E::pack2(s[kk * 8 + 2 * q], s[kk * 8 + 2 * q + 1]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                const uint16_t* vb = &vslot[voff_lane[db] + kk * 16 * D2];
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * D2));
                const u32x4 va = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = E::mfma(va, pf[kk], o[db]);
            }
        }
    };

    // ---- tile loop: two register sets and two value slots alternate ---------------
    // Each tile's loads are NLD vector-memory instructions issued together;
    // before a tile is used, the loads issued after it (the next tile's, when
    // there is one) may stay in flight.  The value copies write LDS behind
    // the compiler's back, so these waits, and the fences that keep the
    // copies into a slot after the reads of its previous tile, are explicit.
    constexpr int NLD = C::NKS + C::VINS;
    static_assert(NLD < 64, "vmcnt range");
    auto wait_tile = [&](bool next_in_flight) __attribute__((always_inline)) {
        if (next_in_flight)
            __builtin_amdgcn_s_waitcnt((NLD & 15) | ((NLD >> 4) << 14) | 0x0070);
        else
            __builtin_amdgcn_s_waitcnt(0x0070);
        __asm__ volatile("" ::: "memory");
    };
    uint16_t* vs0 = VS0 + wave * C::VSLOT;
    uint16_t* vs1 = VS1 + wave * C::VSLOT;
    u32x4 ka[C::NKS], kb[C::NKS];
    int j0 = first_block(0), u0 = 0;
    int j1 = j0, u1 = 0;
    if (j0 >= 0) {
        load_k(j0 * p.lsel, ka);
        load_v(j0 * p.lsel, vs0);
        next_tile(j1, u1);
        if (j1 >= 0) {
            load_k(j1 * p.lsel + u1 * KT, kb);
            load_v(j1 * p.lsel + u1 * KT, vs1);
        }
    }
    while (j0 >= 0) {
        wait_tile(j1 >= 0);
        tile(j0, u0, ka, vs0);
        int j2 = j1, u2 = u1;
        if (j1 >= 0)
            next_tile(j2, u2);
        __asm__ volatile("" ::: "memory");
        if (j2 >= 0) {
            load_k(j2 * p.lsel + u2 * KT, ka);
            load_v(j2 * p.lsel + u2 * KT, vs0);
        }
        if (j1 < 0)
            break;
        wait_tile(j2 >= 0);
        tile(j1, u1, kb, vs1);
        j0 = j2;
        u0 = u2;
        j1 = j2;
        u1 = u2;
        if (j0 >= 0)
            next_tile(j1, u1);
        __asm__ volatile("" ::: "memory");
        if (j1 >= 0) {
            load_k(j1 * p.lsel + u1 * KT, kb);
            load_v(j1 * p.lsel + u1 * KT, vs1);
        }
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

size_t sel_attn_lds_bytes(int tpw, int sw) { return (size_t)kSelWaves * (tpw + 1) * sw * 4; }

template <typename E>
static hipError_t launch_sel_typed(int d1, int d2, const SelParams& p, int n_tiles, size_t lds,
                                   hipStream_t stream)
{
#define X(a, b)                                                                                    \
    if (d1 == a && d2 == b) {                                                                      \
        hipLaunchKernelGGL((k_sel_attn_fwd<E, a, b>), dim3(n_tiles), dim3(64 * kSelWaves), lds, stream, p); \
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
