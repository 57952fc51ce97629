// Kernel (b): compressed attention, steps 1-3 of
// "mindspore.ops.nsa_compress_attention" -- scaled QK^T, the causal mask
// over compressed blocks, softmax and P.V -- fused, plus the softmax max and
// sum outputs.
//
// Design (gfx950, bf16 or f16 MFMA 32x32x16, fp32 accumulate; the element
// type E is a template parameter and only changes the MFMA and the packing):
//   * A workgroup is 4 waves; a wave owns QB blocks of 32 query rows of one
//     (sequence, KV head).  A row is (token, query head of the group): the
//     group's heads of a token are adjacent rows, so they share every K/V
//     tile and every mask.  With QB = 1 and KT = 32 a wave of the D1 = D2 =
//     128 kernel stays within 168 registers, so three waves share each SIMD
//     (three workgroups per CU): one wave's softmax VALU work overlaps the
//     others' MFMAs, and one workgroup's prologue/epilogue overlaps the
//     others' main loops.
//   * K and V tiles of KT compressed entries are copied straight from
//     global memory into LDS by the buffer unit (no register staging),
//     through three rotating slots each, so a copy has about one pipeline
//     step to land before anything waits for it.  K rows carry 16 bytes of
//     padding; V rows are stored as they are, with XOR-swizzled 16-byte
//     chunks, and the P.V operand is read transposed (ds_read_b64_tr_b16)
//     in the order the score accumulator leaves P in.
//   * Scores are computed transposed, S^T = K Q^T: a lane owns one query
//     column and 16 keys per 32x32 block, so the row max and sum are
//     in-lane plus one exchange with the lane 32 away.  P^T is then directly
//     the B operand of O^T += V^T P^T: no shuffles between the two MFMAs.
//   * Online softmax in base 2 with the scale folded into one FMA; the
//     running reference max only moves when a tile's max exceeds it by more
//     than 2^8, so the O rescale is rare (and is a real branch).  The true
//     max is tracked apart for the softmax_max output.
//   * Tiles that every row of the workgroup sees in full run a mask-free
//     body; only the last one or two tiles of a workgroup apply the mask.
//   * With an explicit atten_mask (XM) the workgroup visits the key tiles
//     between the first and the last mask word that keeps anything for one
//     of its tokens (per-row spans from the packing pass), all through the
//     masked body, which keeps a score iff its entry exists and its bit is
//     set in the packed mask row of the lane's token; the row's 32-bit word
//     for the next tile is loaded at the start of each step.
#include <type_traits>

#include "nsa_device.h"

namespace nsa {

template <int D1, int D2, int QB, int KT, int W>
struct AttnCfg {
    static constexpr int NT = 64 * W;          // threads per workgroup (W waves)
    static constexpr int ROWS = W * 32 * QB;   // query rows per workgroup
    static constexpr int KS = D1 + 8;          // LDS row stride of K (elements): 16 B pad
    static constexpr int NKB = KT / 32;        // 32-entry blocks per tile
    static constexpr int NKS = D1 / 16;        // k-steps of QK^T
    static constexpr int NDB = D2 / 32;        // 32-row blocks of O^T
    static constexpr int KCH = D1 / 8;         // 16-byte chunks per K row
    static constexpr int VCH = D2 / 8;         // 16-byte chunks per V row
    // Tiles are copied global -> LDS by the buffer unit (16 bytes per lane,
    // 64 consecutive 16-byte LDS slots per wave instruction).  A K row is
    // KCH + 1 slots (the last one is padding, loaded from outside the
    // buffer's range); a V row is VCH slots in a swizzled order.
    static constexpr int KSLOT = KT * (KCH + 1);
    static constexpr int KINS = (KSLOT + 63) / 64;   // wave instructions per K tile
    static constexpr int KIPW = (KINS + W - 1) / W;  // ... per wave
    static constexpr int KBUF = KINS * 64 * 8;       // elements per K buffer (with slack)
    static constexpr int VINS = KT * VCH / 64;       // wave instructions per V tile
    static constexpr int VIPW = VINS / W;
    static_assert(KT % 32 == 0 && (KT * VCH) % (64 * W) == 0, "V tile copy");
    static_assert(D2 == 64 || D2 == 128, "V swizzle");
};


// At least three waves per SIMD for D1 = D2 = 128 (168 registers, a few
// values spilled around the main loop), which the unrolled loop would
// otherwise exceed; two elsewhere.
template <typename E, bool XM, int D1, int D2, int QB, int KT, int W>
__global__ __launch_bounds__(64 * W, (D1 == 128 && D2 == 128) ? 3 : 2) void k_cmp_attn_fwd(AttnParams p)
{
    using C = AttnCfg<D1, D2, QB, KT, W>;
    static_assert(!XM || KT == 32, "one mask word per key tile");
    // Three K and three V slots, each its own LDS object: the compiler then
    // knows which slot every copy and every read touches and inserts no wait
    // for a copy into another slot.
    __shared__ __attribute__((aligned(16))) uint16_t K0[C::KBUF], K1[C::KBUF], K2[C::KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t V0[KT * D2], V1[KT * D2], V2[KT * D2];
    auto kslot = [&](int i) __attribute__((always_inline)) { return i == 0 ? K0 : (i == 1 ? K1 : K2); };
    auto vslot = [&](int i) __attribute__((always_inline)) { return i == 0 ? V0 : (i == 1 ? V1 : V2); };

    if (*p.status != 0)
        return;   // the table failed the planner's checks
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    // ---- workgroup -> (sequence, KV head, row block) -------------------------
    const int wg = blockIdx.x;
    int b, g, rb;
    int split_kt0 = 0, split_nkt = 0, split_slot = -1;   // split launches only
    const bool split = !XM && p.split != nullptr;
    if (split) {
        const SplitItem it = p.split[wg];
        b = it.b;
        g = it.g;
        rb = it.rb;
        split_kt0 = it.kt0;
        split_nkt = it.n_kt;
        split_slot = it.slot;
    } else {
        b = find_batch<true>(p.bt, p.B, wg);
        const int idx = wg - p.bt[b].tile_off_a;
        g = idx % p.N2;
        rb = p.bt[b].n_rb_a - 1 - idx / p.N2;
    }
    const BatchEnt be = p.bt[b];
    const int G = p.G;
    const int rows_total = be.T * G;
    const int row_wg = rb * C::ROWS;

    int nvq[QB];
    int mrow[QB];    // packed atten_mask row of the lane's token (XM)
    bool vq[QB];
    u32x4 qf[QB][C::NKS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int r = row_wg + (wave * QB + qb) * 32 + l32;
        vq[qb] = r < rows_total;
        const int tok = r / G;
        const int hh = r - tok * G;
        nvq[qb] = vq[qb] ? n_visible(tok + be.pos_off, p.l, p.d, be.n_cmp) : 0;
        mrow[qb] = vq[qb] ? tok : 0;
        // Rows past the sequence read the workgroup's first row (always valid);
        // they see no block and are never written.
        const int64_t qsrc = vq[qb] ? (int64_t)(be.q_off + tok) * p.N1 + (int64_t)g * G + hh
                                    : (int64_t)(be.q_off + row_wg / G) * p.N1 + (int64_t)g * G;
        const uint16_t* qrow = p.q + qsrc * D1 + hf * 8;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            u32x4 v = *(const u32x4*)(qrow + ks * 16);
            v ^= p.qsign;
            qf[qb][ks] = v;
        }
    }
    const int last_row = min(row_wg + C::ROWS, rows_total) - 1;
    const int nv_max = XM ? be.n_cmp : n_visible(last_row / G + be.pos_off, p.l, p.d, be.n_cmp);
    const int nv_min = XM ? 0 : n_visible(row_wg / G + be.pos_off, p.l, p.d, be.n_cmp);
    // XM: tiles [kt0, kt0 + n_kt) hold every kept entry of the workgroup's
    // tokens, and the first n_full of them (only when kt0 = 0) are kept
    // whole by every token (wave-uniform: every wave reduces over all of
    // them).  Below, kt counts tiles from kt0.
    int kt0 = 0, n_kt = (nv_max + KT - 1) / KT, n_full = min(nv_min / KT, n_kt);
    if constexpr (XM) {
        int lo = 0x7FFFFFFF, hi = 0, full = 0x7FFFFFFF;
        for (int tt = row_wg / G + lane; tt <= last_row / G; tt += 64) {
            const int4 sp = p.vis_span[tt];
            lo = min(lo, sp.x);
            hi = max(hi, sp.y);
            full = min(full, sp.z);
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            lo = min(lo, __shfl_xor(lo, m));
            hi = max(hi, __shfl_xor(hi, m));
            full = min(full, __shfl_xor(full, m));
        }
        hi = min(hi, n_kt);
        kt0 = __builtin_amdgcn_readfirstlane(lo < hi ? lo : 0);
        n_kt = __builtin_amdgcn_readfirstlane(lo < hi ? hi - lo : 0);
        n_full = __builtin_amdgcn_readfirstlane(lo == 0 ? min(min(full, be.n_cmp / KT), n_kt) : 0);
    } else {
        if (split) {
            // this piece's tiles; those every row sees in full stay unmasked
            n_full = max(0, min(n_full - split_kt0, split_nkt));
            kt0 = split_kt0;
            n_kt = split_nkt;
        }
    }

    // ---- tile staging ----------------------------------------------------------
    const int64_t kv_stride1 = (int64_t)p.N2 * D1;
    const int64_t kv_stride2 = (int64_t)p.N2 * D2;
    const uint16_t* kbase = p.kc + ((int64_t)be.cmp_off * p.N2 + g) * D1;
    const uint16_t* vbase = p.vc + ((int64_t)be.cmp_off * p.N2 + g) * D2;
    const uint32_t kst_b = (uint32_t)(kv_stride1 * 2);
    const uint32_t vst_b = (uint32_t)(kv_stride2 * 2);
    // Global byte offset (inside a tile) that each lane copies into LDS slot
    // 64*q + lane of instruction q.  Padding slots point past any tile range
    // and load zero.
    uint32_t kdo[C::KIPW], vdo[C::VIPW];
#pragma unroll
    for (int j = 0; j < C::KIPW; ++j) {
        const int slot = (j * W + wave) * 64 + lane;
        const int r = slot / (C::KCH + 1), ch = slot % (C::KCH + 1);
        kdo[j] = (ch < C::KCH && r < KT) ? (uint32_t)r * kst_b + (uint32_t)ch * 16u : 0x7FFFFFF0u;
    }
#pragma unroll
    for (int j = 0; j < C::VIPW; ++j) {
        const int slot = (j * W + wave) * 64 + lane;
        const int r = slot / C::VCH;
        const int ch = v_swz<D2>(r, slot % C::VCH);   // the XOR is its own inverse
        vdo[j] = (uint32_t)r * vst_b + (uint32_t)ch * 16u;
    }
    // Each tile's buffer resource starts at its first entry and ends after
    // the sequence's last one, so entries past the end load as zero (they are
    // masked); a tile index at or past the last one gets an empty range.
    auto tile_bytes = [&](int kt, uint32_t stride_b, int row_bytes) -> uint32_t __attribute__((always_inline)) {
        const int nvalid = min(KT, be.n_cmp - kt * KT);
        return nvalid > 0 ? (uint32_t)(nvalid - 1) * stride_b + (uint32_t)row_bytes : 0u;
    };
    auto load_k = [&](int kt, uint16_t* dst) __attribute__((always_inline)) {
        kt += kt0;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + (int64_t)kt * KT * kv_stride1, tile_bytes(kt, kst_b, D1 * 2));
#pragma unroll
        for (int j = 0; j < C::KIPW; ++j)
            if (j < C::KINS / W || j * W + wave < C::KINS)
                copy16_to_lds(kr, dst + (j * W + wave) * 512, kdo[j]);
    };
    auto load_v = [&](int kt, uint16_t* dst) __attribute__((always_inline)) {
        kt += kt0;
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + (int64_t)kt * KT * kv_stride2, tile_bytes(kt, vst_b, D2 * 2));
#pragma unroll
        for (int j = 0; j < C::VIPW; ++j)
            copy16_to_lds(vr, dst + (j * W + wave) * 512, vdo[j]);
    };
    // All copies of this wave have landed in LDS (the barrier that follows
    // makes every wave's copies visible).
    auto copies_done = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(0x0F70); };
    // End of a pipeline step: this wave's LDS reads have returned and its
    // copies issued before the step have landed (only the step's own, at
    // least NCP per wave, may still be in flight); then the workgroup
    // barrier.  The empty asm statements keep the compiler from moving LDS
    // accesses across the barrier.
    constexpr int NCP = C::KINS / W + C::VIPW;
    static_assert(NCP < 64, "vmcnt range");
    auto step_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt((NCP & 15) | ((NCP >> 4) << 14) | 0x0070);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };

    // P.V operand addressing (ds_read_b64_tr_b16): in each 16-lane group,
    // lane i supplies the 8 bytes of row key0 + i/4, dims dimbase + 4*(i%4)
    // and receives V[key0 + 0..3][dimbase + i].  k-slots 0-3 of a lane in
    // half hf are keys 16kk + 4hf + 0..3, k-slots 4-7 keys 16kk + 8 + 4hf +
    // 0..3: the order the score accumulator leaves P in.
    int voff_lane[C::NDB];
    {
        const int vi = lane & 15, vgrp = (lane >> 4) & 1;
        const int r0 = 4 * hf + (vi >> 2);           // row inside a 16-key chunk
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const int dim = db * 32 + 16 * vgrp + 4 * (vi & 3);
            voff_lane[db] = r0 * D2 + v_swz<D2>(r0, dim >> 3) * 8 + (dim & 7);
        }
    }

    // ---- state -------------------------------------------------------------------
    f32x16 o[QB][C::NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o[qb][db][r] = 0.f;
    float mref[QB], mtrue[QB], lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mref[qb] = -INFINITY;
        mtrue[qb] = -INFINITY;
        lsum[qb] = 0.f;
    }
    const float c = p.c;
    f32x16 scur[QB][C::NKB], snxt[QB][C::NKB];
    u32x4 pfr[QB][2 * C::NKB];   // P of the current tile, packed B operands of P.V

    // S^T = K Q^T for tile kt (K in LDS buffer kt & 1) into snxt.
    auto qk = [&](const uint16_t* kbuf) __attribute__((always_inline)) {
        auto& s = snxt;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[qb][kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                const u32x4 ka = *(const u32x4*)&kbuf[(kb * 32 + l32) * C::KS + ks * 16 + hf * 8];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[qb][kb] = E::mfma(ka, qf[qb][ks], s[qb][kb]);
            }
        }
    };

    // Mask and max of tile kt (in snxt); decides whether the reference max
    // must move.  The move itself (and the O rescale) waits for rescale(),
    // after the P.V of the previous tile has been accumulated.
    float tmaxq[QB], nbias[QB];
    bool growq[QB];
    uint32_t mword[QB];   // XM: packed mask word of the next tile to mask
    auto load_mword = [&](const int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            mword[qb] = p.vis[(int64_t)mrow[qb] * p.vis_words + kt0 + kt];
    };
    auto tile_max = [&](const int kt, auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        auto& s = snxt;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if constexpr (MASK && XM) {
                // key kt*KT + 8*(r/4) + 4*hf + r%4 is kept iff it exists and
                // its bit is set; a wave whose rows keep the whole tile skips
                // the selects
                const int lim = be.n_cmp - (kt0 + kt) * KT - 4 * hf;
                const bool part = mword[qb] != 0xFFFFFFFFu || (kt0 + kt + 1) * KT > be.n_cmp;
                if (__ballot(part) != 0) {
                    const uint32_t w = mword[qb] >> (4 * hf);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[qb][0][r] = (8 * (r >> 2) + (r & 3) < lim && ((w >> (8 * (r >> 2) + (r & 3))) & 1u))
                                          ? s[qb][0][r] : -INFINITY;
                }
            } else if constexpr (MASK) {
                // key kt*KT + kb*32 + 8*(r/4) + 4*hf + r%4 is visible iff it is
                // below nvq: compare the compile-time part against one bound
                const int lim = nvq[qb] - (kt0 + kt) * KT - 4 * hf;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[qb][kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3) < lim) ? s[qb][kb][r] : -INFINITY;
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    tmax = fmaxf(tmax, s[qb][kb][r]);
            tmax = half_max(tmax);
            mtrue[qb] = fmaxf(mtrue[qb], tmax);
            tmaxq[qb] = tmax;
            growq[qb] = tmax > mref[qb] + p.thr;
        }
    };
    // Rare: move the reference max where a row asked for it, rescaling O and
    // the running sum; then the exponent bias of the next tile.
    auto rescale = [&]() __attribute__((always_inline)) {
        bool any = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            any |= growq[qb];
        if (__builtin_expect(__ballot(any) != 0, 0)) {
            __asm__ volatile("" ::: "memory");
            // A row whose reference max is still -inf has O = 0 and sum 0
            // (every P so far was 0): nothing to rescale.  Only when some
            // row of the wave moves a finite max is O multiplied (always
            // at a wave's first tile, the one place most rows move).
            bool live = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                live |= growq[qb] && mref[qb] != -INFINITY;
            const bool scale_o = __ballot(live) != 0;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float alpha = 1.f;
                if (growq[qb]) {
                    alpha = (mref[qb] == -INFINITY) ? 0.f : fast_exp2((mref[qb] - tmaxq[qb]) * c);
                    mref[qb] = tmaxq[qb];
                }
                if (scale_o) {
                    lsum[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            o[qb][db][r] *= alpha;
                }
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            nbias[qb] = (mref[qb] == -INFINITY) ? 0.f : -mref[qb] * c;
    };
    // P = exp2(S*c - mref*c) of the current tile, the running sum, and P
    // packed to the element type in the order the P.V MFMAs consume it.  Masked scores
    // are -inf and c > 0, so their exponentials are exactly 0.
    auto softmax_exp = [&](auto mask_tag) __attribute__((always_inline)) {
        (void)mask_tag;
        auto& s = scur;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // the tile's sum starts at its first exponential (the same value
            // as 0 + it: every P is >= +0), saving one add per tile
            float ps;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float sv = s[qb][kb][r];
                    const float pv = fast_exp2(fmaf(sv, c, nbias[qb]));
                    s[qb][kb][r] = pv;
                    ps = (kb == 0 && r == 0) ? pv : ps + pv;
                }
            }
            lsum[qb] += ps;
#pragma unroll
            for (int kk = 0; kk < 2 * C::NKB; ++kk) {
                const int kb = kk >> 1;
                const int r0 = (kk & 1) * 8;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pfr[qb][kk][j] = E::pack2(s[qb][kb][r0 + 2 * j], s[qb][kb][r0 + 2 * j + 1]);
            }
        }
    };

    // O^T += V^T P^T for tile kt (V in LDS buffer kt & 1), 16 keys per MFMA.
    auto pv = [&](const uint16_t* vbuf) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 2 * C::NKB; ++kk) {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                const uint16_t* vb = &vbuf[voff_lane[db] + kk * 16 * D2];
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * D2));
                const u32x4 va = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][db] = E::mfma(va, pfr[qb][kk], o[qb][db]);
            }
        }
    };

    // Software pipeline, one barrier per tile.  On entry to step kt, scur
    // holds S(kt) with its mask applied and nbias is final for it.  The
    // step issues the QK^T MFMAs of tile kt+1 next to the exponentials of
    // tile kt, then the P.V MFMAs of tile kt next to the max of tile kt+1,
    // so both MFMA phases have independent vector work beside them.
    //
    // K and V tiles rotate through three LDS slots each (tile t in slot
    // t % 3).  Step kt reads K(kt+1) and V(kt), and first refills the slots
    // read in step kt-1 with K(kt+3) and V(kt+2): the first barrier that
    // waits for those copies is the one at the end of step kt+1, so each has
    // more than a step to land.  The main loop runs three steps per trip with
    // fixed slot objects, which is what lets the compiler see that the
    // step's reads and copies touch different slots.
    auto step_bufs = [&](const int kt, auto mask_cur, auto mask_next, auto last_tag,
                         uint16_t* k_rd, uint16_t* k_cp, uint16_t* v_rd, uint16_t* v_cp) __attribute__((always_inline)) {
        constexpr bool LAST = decltype(last_tag)::value;
        if constexpr (!LAST) {
            if constexpr (XM && decltype(mask_next)::value)
                load_mword(kt + 1);   // before the copies: waited for without them
            load_k(kt + 3, k_cp);
            load_v(kt + 2, v_cp);
            qk(k_rd);
        }
        softmax_exp(mask_cur);
        pv(v_rd);
        if constexpr (!LAST) {
            tile_max(kt + 1, mask_next);
            rescale();
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
                    scur[qb][kb] = snxt[qb][kb];
            step_barrier();
        }
    };
    // Step with the slots picked at run time (the few steps outside the
    // unrolled loop).
    auto step = [&](const int kt, auto mask_cur, auto mask_next, auto last_tag) __attribute__((always_inline)) {
        const int b0 = kt % 3, b1 = (kt + 1) % 3, b2 = (kt + 2) % 3;
        step_bufs(kt, mask_cur, mask_next, last_tag, kslot(b1), kslot(b0), vslot(b0), vslot(b2));
    };
    // Tiles every row of the workgroup sees in full need no mask; the last
    // tile has no successor to prefetch.
    using F = std::false_type;
    using T = std::true_type;
    if (n_kt > 0) {
        load_k(0, K0);
        load_v(0, V0);
        load_k(1, K1);
        load_k(2, K2);
        load_v(1, V1);
        copies_done();
        __syncthreads();
        if constexpr (XM)
            if (n_full == 0)
                load_mword(0);
        qk(K0);
        if (n_full > 0)
            tile_max(0, F{});
        else
            tile_max(0, T{});
        rescale();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
                scur[qb][kb] = snxt[qb][kb];
        __syncthreads();   // step 0 refills K buffer 0, which qk(0) just read
        int kt = 0;
        // tiles kt and kt+1 both unmasked, three steps per trip
        for (; kt + 3 < min(n_full, n_kt); kt += 3) {
            step_bufs(kt, F{}, F{}, F{}, K1, K0, V0, V2);
            __builtin_amdgcn_sched_barrier(0);
            step_bufs(kt + 1, F{}, F{}, F{}, K2, K1, V1, V0);
            __builtin_amdgcn_sched_barrier(0);
            step_bufs(kt + 2, F{}, F{}, F{}, K0, K2, V2, V1);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (; kt + 1 < min(n_full, n_kt); ++kt)
            step(kt, F{}, F{}, F{});
        // tile kt unmasked, kt+1 masked
        if (kt < n_full && kt + 1 < n_kt) {
            step(kt, F{}, T{}, F{});
            ++kt;
        }
        for (; kt + 1 < n_kt; ++kt)
            step(kt, T{}, T{}, F{});
        if (kt < n_full)
            step(kt, F{}, F{}, T{});
        else
            step(kt, T{}, T{}, T{});
    }

    // ---- epilogue ------------------------------------------------------------------
    // O goes out through LDS so that the global stores are whole 16-byte
    // chunks of consecutive dims, 128 contiguous bytes per output row and
    // pass: a lane's accumulators hold 4-dim pieces of one row.  Outputs are
    // stored non-temporal: nothing in this kernel reads them back, and the
    // L2 is better kept for the K/V tiles.  Every wave
    // is done with the K slots after this barrier; each wave stages its rows
    // in a private part of them, half of D2 per pass.
    // The lane and each row's output index are recomputed here rather than
    // kept live across the key loop (which would cost registers it needs).
    const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int l32_e = lane_e & 31, hf_e = lane_e >> 5;
    if (split && split_slot >= 0) {
        // a piece of a split row block: unnormalised O with the running sum,
        // reference max and true max of each row, for the combine kernel
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int rr = (wave * QB + qb) * 32 + l32_e;
            if (row_wg + rr >= rows_total)
                continue;
            float* dst = p.part + ((int64_t)split_slot * C::ROWS + rr) * (D2 + 4);
            const float lf = half_sum(lsum[qb]);
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *(f32x4*)(dst + db * 32 + 8 * r4 + 4 * hf_e) =
                        f32x4{o[qb][db][4 * r4], o[qb][db][4 * r4 + 1], o[qb][db][4 * r4 + 2], o[qb][db][4 * r4 + 3]};
            if (hf_e == 0)
                *(f32x4*)(dst + D2) = f32x4{lf, mref[qb], mtrue[qb], 0.f};
        }
        return;
    }
    __syncthreads();
    constexpr int HD = D2 / 2;                 // dims per pass
    constexpr int OPITCH = HD + 8;             // staging row pitch (elements), 16 B pad
    constexpr int CPR = HD / 8;                // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPR;              // staged rows per read instruction
    constexpr int WPS = C::KBUF / (32 * OPITCH);   // waves staged per K slot
    static_assert(WPS >= 1 && (W + WPS - 1) / WPS <= 3, "O staging fits the K slots");
    uint16_t* ostg = kslot(wave / WPS) + (wave % WPS) * 32 * OPITCH;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lf = half_sum(lsum[qb]);
        const bool empty = (mtrue[qb] == -INFINITY);
        const float inv = empty ? 0.f : 1.f / lf;
        // The rows this lane stores in both passes, and where they go (null
        // past the sequence): computed once, the two passes share them.
        uint16_t* odst[32 / RPI];
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int r = row_wg + (wave * QB + qb) * 32 + i * RPI + lane_e / CPR;
            const uint32_t tok = (uint32_t)r / (uint32_t)G;
            const int64_t orow = (int64_t)(be.q_off + (int)tok) * p.N1 + (int64_t)g * G + (r - (int)tok * G);
            odst[i] = r < rows_total ? p.out + orow * D2 + (lane_e % CPR) * 8 : nullptr;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int db = h * C::NDB / 2; db < (h + 1) * C::NDB / 2; ++db) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int dv = (db - h * C::NDB / 2) * 32 + 8 * r4 + 4 * hf_e;
                    u32x2 w2 = {E::pack2(o[qb][db][4 * r4 + 0] * inv, o[qb][db][4 * r4 + 1] * inv),
                                E::pack2(o[qb][db][4 * r4 + 2] * inv, o[qb][db][4 * r4 + 3] * inv)};
                    *(u32x2*)&ostg[l32_e * OPITCH + dv] = w2;
                }
            }
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {
                const int rr = i * RPI + lane_e / CPR;          // staged row
                const int ch = lane_e % CPR;
                const u32x4 v = *(const u32x4*)&ostg[rr * OPITCH + ch * 8];
                if (odst[i] != nullptr)
                    __builtin_nontemporal_store(v, (u32x4*)(odst[i] + h * HD));
            }
        }
        const int r = row_wg + (wave * QB + qb) * 32 + l32_e;
        if (r >= rows_total)
            continue;
        const int tok = (int)((uint32_t)r / (uint32_t)G);
        const int64_t grow = (int64_t)(be.q_off + tok) * p.N1 + (int64_t)g * G + (r - tok * G);
        const float smv = empty ? -INFINITY : mtrue[qb] * p.abs_scale;
        const float ssv = empty ? 0.f : lf * fast_exp2((mref[qb] - mtrue[qb]) * c);
        const float val = hf_e == 0 ? smv : ssv;
        float* dst = (hf_e == 0 ? p.smax : p.ssum) + grow * 8;
        f32x4 v4 = {val, val, val, val};
        __builtin_nontemporal_store(v4, (f32x4*)dst);
        __builtin_nontemporal_store(v4, (f32x4*)(dst + 4));
        if (p.bias != nullptr && hf_e == 0)
            p.bias[grow] = row_bias(smv, ssv);
    }
}

// Combine of a split row block: per row, the pieces' partial sums are
// brought to the largest reference max and added in piece order (bitwise
// repeatable); then the outputs as the single-pass epilogue writes them.
// Thread = (row, 4 consecutive dims); 256 threads stride over the block.
template <typename E, int D2, int ROWS>
__global__ __launch_bounds__(256) void k_cmp_attn_combine(AttnParams p, const CombineItem* items)
{
    if (*p.status != 0)
        return;
    const CombineItem it = items[blockIdx.x];
    const BatchEnt be = p.bt[it.b];
    const int G = p.G;
    const int rows_total = be.T * G;
    const float c = p.c;
    for (int u = threadIdx.x; u < ROWS * (D2 / 4); u += 256) {
        const int rr = u / (D2 / 4), d4 = (u % (D2 / 4)) * 4;
        const int r = it.rb * ROWS + rr;
        if (r >= rows_total)
            continue;
        const float* base = p.part + ((int64_t)it.slot0 * ROWS + rr) * (D2 + 4);
        const int64_t piece = (int64_t)ROWS * (D2 + 4);
        float R = -INFINITY, M = -INFINITY;
        for (int s = 0; s < it.n; ++s) {
            const f32x4 st = *(const f32x4*)(base + s * piece + D2);
            R = fmaxf(R, st[1]);
            M = fmaxf(M, st[2]);
        }
        float L = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (R != -INFINITY) {
            for (int s = 0; s < it.n; ++s) {
                const f32x4 st = *(const f32x4*)(base + s * piece + D2);
                if (st[1] == -INFINITY)
                    continue;
                const float w = exp2f((st[1] - R) * c);
                L += st[0] * w;
                const f32x4 ov = *(const f32x4*)(base + s * piece + d4);
                acc[0] += ov[0] * w;
                acc[1] += ov[1] * w;
                acc[2] += ov[2] * w;
                acc[3] += ov[3] * w;
            }
        }
        const bool empty = (M == -INFINITY);
        const float inv = empty ? 0.f : 1.f / L;
        const int tok = r / G;
        const int64_t orow = (int64_t)(be.q_off + tok) * p.N1 + (int64_t)it.g * G + (r - tok * G);
        *(u32x2*)(p.out + orow * D2 + d4) = u32x2{E::pack2(acc[0] * inv, acc[1] * inv),
                                                  E::pack2(acc[2] * inv, acc[3] * inv)};
        if (d4 == 0) {
            const float smv = empty ? -INFINITY : M * p.abs_scale;
            const float ssv = empty ? 0.f : L * exp2f((R - M) * c);
            const f32x4 a = {smv, smv, smv, smv}, bb = {ssv, ssv, ssv, ssv};
            *(f32x4*)(p.smax + orow * 8) = a;
            *(f32x4*)(p.smax + orow * 8 + 4) = a;
            *(f32x4*)(p.ssum + orow * 8) = bb;
            *(f32x4*)(p.ssum + orow * 8 + 4) = bb;
            if (p.bias != nullptr)
                p.bias[orow] = row_bias(smv, ssv);
        }
    }
}

// Launch shape per head-dim pair: query-row blocks per wave (QB), key-tile
// length (KT) and waves per workgroup.  QB = 1 keeps each wave within 256
// registers; KT = 32 keeps the score tiles small enough for three
// workgroups per CU (four for D2 = 64) and the three K and V slots within
// the LDS share of each (52 KB for D1 = D2 = 128).
#define NSA_ATTN_CONFIGS(X)      \
    X(64, 64, 1, 32, 4)          \
    X(128, 64, 1, 32, 4)         \
    X(128, 128, 1, 32, 4)        \
    X(192, 64, 1, 32, 4)         \
    X(192, 128, 1, 32, 4)

bool cmp_attn_supported(int d1, int d2)
{
#define X(a, b, q, k, w) if (d1 == a && d2 == b) return true;
    NSA_ATTN_CONFIGS(X)
#undef X
    return false;
}

int cmp_attn_rows_per_wg(int d1, int d2)
{
#define X(a, b, q, k, w) if (d1 == a && d2 == b) return AttnCfg<a, b, q, k, w>::ROWS;
    NSA_ATTN_CONFIGS(X)
#undef X
    return 0;
}

template <typename E, bool XM>
static hipError_t launch_typed(int d1, int d2, const AttnParams& p, int n_tiles, hipStream_t stream)
{
#define X(a, b, q, k, w)                                                                          \
    if (d1 == a && d2 == b) {                                                                  \
        hipLaunchKernelGGL((k_cmp_attn_fwd<E, XM, a, b, q, k, w>), dim3(n_tiles), dim3(64 * w), 0, stream, p); \
        return hipGetLastError();                                                              \
    }
    NSA_ATTN_CONFIGS(X)
#undef X
    return hipErrorInvalidValue;
}

template <typename E>
static hipError_t launch_combine_typed(int d1, int d2, const AttnParams& p, const CombineItem* items,
                                       int n_items, hipStream_t stream)
{
#define X(a, b, q, k, w)                                                                          \
    if (d1 == a && d2 == b) {                                                                  \
        hipLaunchKernelGGL((k_cmp_attn_combine<E, b, AttnCfg<a, b, q, k, w>::ROWS>), dim3(n_items), dim3(256), 0, \
                           stream, p, items);                                                  \
        return hipGetLastError();                                                              \
    }
    NSA_ATTN_CONFIGS(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(int dtype, int d1, int d2, const AttnParams& p, const CombineItem* items,
                               int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (dtype == ElemBf16::code)
        return launch_combine_typed<ElemBf16>(d1, d2, p, items, n_items, stream);
    if (dtype == ElemF16::code)
        return launch_combine_typed<ElemF16>(d1, d2, p, items, n_items, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_cmp_attn(int dtype, int d1, int d2, const AttnParams& p, int n_tiles,
                           hipStream_t stream)
{
    if (n_tiles <= 0)
        return hipSuccess;
    const bool xm = p.vis != nullptr;
    if (dtype == ElemBf16::code)
        return xm ? launch_typed<ElemBf16, true>(d1, d2, p, n_tiles, stream)
                  : launch_typed<ElemBf16, false>(d1, d2, p, n_tiles, stream);
    if (dtype == ElemF16::code)
        return xm ? launch_typed<ElemF16, true>(d1, d2, p, n_tiles, stream)
                  : launch_typed<ElemF16, false>(d1, d2, p, n_tiles, stream);
    return hipErrorInvalidValue;
}

}  // namespace nsa
