// Kernel (c): importance scores and top-k, steps 4-7 of
// "mindspore.ops.nsa_compress_attention".
//
//   P_slc'[t, g, j] = sum_{h in group g} sum_{m < R} sum_{n < L2} P_cmp^h[R*j - m - n]
//   R = l'/d, L2 = floor(l/d); then the top-k mask (candidates j*l' <= t) and
//   the select_block_count largest scores, ties to the lower j, -1 padded.
//
// P_cmp is recomputed rather than stored: S = Q K^T on MFMA (bf16 or f16 in, fp32
// out) and P = exp2(S * c - bias) with bias = max * log2(e) + log2(sum) from
// the attention kernel's outputs, i.e. already normalised.
//
// Design (gfx950):
//   * Rows are (token, query head) with the group padded to a power of two GP
//     (<= 64), so the GP heads of a token are adjacent rows of one wave.  S is
//     computed un-transposed (rows = heads, columns = compressed entries):
//     the sum over a token's heads is then an in-lane sum of accumulator
//     registers plus, for GP >= 8, one exchange with the lane 32 away.
//   * K tiles (32 entries up to D1 = 128, 64 above) are double buffered in
//     LDS and loaded with range-limited buffer loads one tile ahead; one
//     workgroup barrier per tile.  Everything else a wave touches in LDS (its tokens' rings,
//     importance scores and top-k staging) is private to the wave and needs
//     only wave-level ordering.
//   * The group-summed P of each token goes to an LDS ring indexed by
//     compressed-entry number; after every batch of key tiles (as many as
//     keep the wave's lanes about busy in the stencil, one tile when a wave
//     holds four tokens or more) the select blocks whose whole stencil is
//     available are finished as a fixed-order weighted sum of at most H+1
//     ring entries (the remap written as a stencil over r = m + n with
//     coefficient c(r) = number of (m, n) pairs).  The ring (128-512
//     entries) keeps a batch plus the H entries a later block still needs.
//     Its first four slots are repeated past its end, so a stencil of up
//     to five taps (every workload's: H = R + floor(l/d) - 2 = 4) reads
//     five consecutive slots from one address with immediate offsets.  The
//     (token, block) pairs of a batch are spread over the wave's lanes.
//   * Top-k per (token, KV head) row, wave-local, on the float bits (scores
//     are >= 0, so their bit patterns order like the values).  A radix
//     select over the 64 per-lane maxima (one ballot per bit) gives a lower
//     bound of the k-th largest score; the few candidates at or above it are
//     staged in LDS and each finds its rank by (score desc, index asc)
//     against the others.  When more than 64 reach the bound (heavy ties),
//     a radix select over all candidates finds the k-th largest score and
//     the picks above it plus the lowest-index ties are ranked the same way.
//   * Explicit masks: with an atten_mask (XM) the workgroup visits the key
//     tiles between the first and the last mask word that keeps anything
//     for one of its tokens, all through the masked body, where P is kept
//     iff its entry exists and its bit is set in the packed mask row of its
//     token (the wave's mask words of a
//     tile are loaded before the tile's MFMAs and passed through LDS); a
//     topk_mask replaces the candidate rule j*l' <= t by the packed bits.
//   * Deterministic: every sum has a fixed order; no atomics.
#include <type_traits>

#include "nsa_device.h"

namespace nsa {

// Orders this wave's LDS accesses: a wave's LDS operations execute in order,
// so it is enough to keep the compiler from moving them across this point.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Whether accumulator register r of row half rr is the first, in the order
// (rr, r), whose row (rr * 32 + 8 * (r / 4) + r % 4 in the lower half-wave)
// belongs to its token (rows of one token: 2^log2gp consecutive rows).
constexpr bool first_term(int rr, int r, int log2gp)
{
    const int tw = (rr * 32 + 8 * (r >> 2) + (r & 3)) >> log2gp;
    for (int r2 = 0; r2 < rr * 16 + r; ++r2)
        if (((r2 >> 4) * 32 + 8 * ((r2 & 15) >> 2) + (r2 & 3)) >> log2gp == tw)
            return false;
    return true;
}

// Three waves per SIMD where the registers allow it (D1 = 128 with groups
// of 16 or more), two elsewhere.
template <typename E, bool XM, int D1, int LOG2GP>
__global__ __launch_bounds__(256, (D1 == 128 && LOG2GP >= 4) ? 3 : 2) void k_slc_topk(TopkParams p)
{
    constexpr int GP = 1 << LOG2GP;
    constexpr int TOKW = 64 / GP;           // tokens per wave
    constexpr int KT = topk_key_tile(D1);
    constexpr int NKB = KT / 32;            // 32-entry blocks per key tile
    constexpr int KS = D1 + 8;
    constexpr int NKS = D1 / 16;
    constexpr int KCH = D1 / 8;
    constexpr int KLD = KT * KCH / 256;
    constexpr int RING = topk_ring(LOG2GP);
    constexpr int RINGP = RING + kTopkRingDup;        // ring row: the ring, then its first slots again
    constexpr int HSH = 4 >> LOG2GP;        // token offset of the upper half-wave (GP <= 4)

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    if (*p.status != 0)
        return;   // the table failed the planner's checks
    const int waves = p.waves;
    const int nbuf = p.kbufs;                              // K tile buffers: 2, or 1 if LDS is tight
    uint16_t* Ks = (uint16_t*)smem;                        // [nbuf][KT * KS]
    float* ring = (float*)(smem + nbuf * KT * KS * 2);     // [waves * TOKW][RINGP]
    float* bins = ring + waves * TOKW * RINGP;             // [waves * TOKW][sb]
    uint32_t* stg = (uint32_t*)(bins + waves * TOKW * p.sb);  // [waves][128]

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int nthreads = waves * 64;

    // ---- workgroup -> (sequence, KV head, row block) ---------------------------
    const int wg = blockIdx.x;
    const int b = find_batch<false>(p.bt, p.B, wg);
    const BatchEnt be = p.bt[b];
    const int idx = wg - be.tile_off_c;
    const int g = idx % p.N2;
    const int rb = be.n_rb_c - 1 - idx / p.N2;
    const int G = p.G;
    const int tok_wg = rb * ((waves * 64) >> LOG2GP);
    const int tok_w = tok_wg + wave * TOKW;

    // Q rows as the A operand: lane l32 holds row rr*32 + l32 of its wave.
    // Padding heads and tokens past the sequence read the workgroup's first
    // row; their bias below makes their P zero.
    u32x4 qa[2][NKS];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int pr = rr * 32 + l32;
        const int tok = tok_w + (pr >> LOG2GP);
        const int hh = pr & (GP - 1);
        const bool valid = tok < be.T && hh < G;
        const int64_t row = valid ? (int64_t)(be.q_off + tok) * p.N1 + (int64_t)g * G + hh
                                  : (int64_t)(be.q_off + tok_wg) * p.N1 + (int64_t)g * G;
        const uint16_t* qrow = p.q + row * D1 + hf * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4 v = *(const u32x4*)(qrow + ks * 16);
            v ^= p.qsign;
            qa[rr][ks] = v;
        }
    }
    // Per accumulator register: P = exp2(S*c - bias) is the normalised P_cmp.
    // Rows that are padding, past the sequence, or see no block get +inf.
    // Each lane loads the bias of row `lane` of its wave (one load from the
    // attention pass's compact array, else the two statistics), then every
    // register fetches its row's bias from that lane.
    float bias_lane = INFINITY;
    {
        const int tok = tok_w + (lane >> LOG2GP);
        const int hh = lane & (GP - 1);
        if (tok < be.T && hh < G) {
            const int64_t row = (int64_t)(be.q_off + tok) * p.N1 + (int64_t)g * G + hh;
            bias_lane = p.bias != nullptr ? p.bias[row] : row_bias(p.smax[row * 8], p.ssum[row * 8]);
        }
    }
    float bias[2][16];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            bias[rr][r] = __shfl(bias_lane, rr * 32 + 8 * (r >> 2) + 4 * hf + (r & 3));

    const int tok_last = min(tok_wg + ((waves * 64) >> LOG2GP), be.T) - 1;
    const int nv_max = XM ? be.n_cmp : n_visible(tok_last + be.pos_off, p.l, p.d, be.n_cmp);
    const int nv_min = XM ? 0 : n_visible(tok_wg + be.pos_off, p.l, p.d, be.n_cmp);
    const int n_kt = (nv_max + KT - 1) / KT;
    // Key tiles [kt_begin, kt_end).  XM: the tiles that hold a kept entry of
    // one of the workgroup's tokens (wave-uniform: every wave reduces over
    // all of them); entries before kt_begin are zero for every token.
    // The first n_full tiles are seen whole by every token (XM: kept whole
    // by every token's mask row, only when kt_begin = 0) and need no mask.
    int kt_begin = 0, kt_end = n_kt, n_full = min(nv_min / KT, n_kt);
    if constexpr (XM) {
        int lo = 0x7FFFFFFF, hi = 0, full = 0x7FFFFFFF;
        for (int tt = tok_wg + lane; tt <= tok_last; tt += 64) {
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
        const int tlo = lo / NKB;
        const int thi = min((hi + NKB - 1) / NKB, n_kt);
        kt_begin = __builtin_amdgcn_readfirstlane(tlo < thi ? tlo : 0);
        kt_end = __builtin_amdgcn_readfirstlane(tlo < thi ? thi : 0);
        n_full = __builtin_amdgcn_readfirstlane(
            (tlo < thi && tlo == 0) ? min(min(full / NKB, be.n_cmp / KT), kt_end) : 0);
    }

    float* my_ring = ring + wave * TOKW * RINGP;
    float* my_bins = bins + wave * TOKW * p.sb;
    uint32_t* my_stg = stg + wave * 128;     // XM mask words in the key loop; top-k staging after it
    for (int x = lane; x < TOKW * RINGP; x += 64)
        my_ring[x] = 0.f;
    // The stencil runs once per batch of nbt key tiles: enough tiles that the
    // (token, block) pairs they finish fill most of the wave's lanes, few
    // enough that the ring still holds the batch plus the stencil's reach.
    // Stencil lanes: lane -> (token tw_l, block slot jj_l) with nbt * nj_slots
    // (nj_slots = ceil(KT / R)) slots per token, tpp tokens per pass.
    const int nbt = max(1, min(64 / (TOKW * p.nj_slots), (RING - 16) / KT));
    const int nj_bat = nbt * p.nj_slots;
    const int tw_l = lane / nj_bat;
    const int jj_l = lane - tw_l * nj_bat;
    const int tpp = max(1, 64 / nj_bat);
    int bat_n = 0;   // tiles of the current batch so far

    // ---- K tile staging ------------------------------------------------------------
    const int64_t kstride = (int64_t)p.N2 * D1;
    const uint16_t* kbase = p.kc + ((int64_t)be.cmp_off * p.N2 + g) * D1;
    const uint32_t kst_b = (uint32_t)(kstride * 2);
    // Each tile's buffer resource starts at its first entry and ends after the
    // sequence's last one: entries past the end load as zero (they are masked).
    auto tile_rsrc = [&](int kt) {
        const int key0 = kt * KT;
        const int nvalid = min(KT, be.n_cmp - key0);
        return make_rsrc(kbase + (int64_t)key0 * kstride, (uint32_t)(nvalid - 1) * kst_b + D1 * 2);
    };
    auto chunk_off = [&](int cidx) { return (uint32_t)(cidx / KCH) * kst_b + (uint32_t)(cidx % KCH) * 16u; };
    auto ks_at = [&](int buf, int cidx) -> u32x4* {
        return (u32x4*)&Ks[buf * KT * KS + (cidx / KCH) * KS + (cidx % KCH) * 8];
    };
    const bool full_wg = (nthreads == 256);
    u32x4 kreg[KLD];
    auto load_tile = [&](int kt) {
        const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kt);
#pragma unroll
        for (int i = 0; i < KLD; ++i)
            kreg[i] = buffer_load16(kr, chunk_off(tid + 256 * i));
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KLD; ++i)
            *ks_at(buf, tid + 256 * i) = kreg[i];
    };
    // A workgroup narrower than 256 threads loads and stores in several passes.
    auto stage_tile = [&](int kt, int buf) {
        const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kt);
        for (int cidx = tid; cidx < KT * KCH; cidx += nthreads)
            *ks_at(buf, cidx) = buffer_load16(kr, chunk_off(cidx));
    };

    const float c = p.c;
    const int R = p.R;
    const int H = p.H;
    float cf[8];                          // remap coefficients, kept in registers
#pragma unroll
    for (int r = 0; r < 8; ++r)
        cf[r] = p.coef[r];
    // Importance score of select block j from a token's ring: the remap
    // stencil sum over r = 0..H of coef(r) * P[R*j - r], ascending r, with the
    // entries at or past `limit` taken as 0.  Up to H = 7 the ring reads are
    // independent and go out together.
    // Up to five taps (H <= 4): slots w[4 - r] hold P[R*j - r]; the read
    // never passes the ring row's end (its first slots are repeated there).
    // Taps past H have coefficient 0 and add nothing, so the sum equals the
    // general one below bit for bit.
    auto stencil5 = [&](const float* rg, int j) __attribute__((always_inline)) {
        const float* w = rg + ((R * j - kTopkRingDup) & (RING - 1));
        float v = 0.f;
        v = fmaf(cf[0], w[4], v);
        v = fmaf(cf[1], w[3], v);
        v = fmaf(cf[2], w[2], v);
        v = fmaf(cf[3], w[1], v);
        v = fmaf(cf[4], w[0], v);
        return v;
    };
    const bool short_stencil = H < kTopkRingDup + 1;
    // Longer stencils inside the key loop (rare): a plain loop, so that
    // nothing of it is computed ahead of the branch that skips it.
    auto stencil_long = [&](const float* rg, int j) __attribute__((always_inline)) {
        float v = 0.f;
        for (int r = 0; r <= H; ++r)
            v = fmaf(p.coef[r], rg[(R * j - r) & (RING - 1)], v);
        return v;
    };
    auto stencil = [&](const float* rg, int j, int limit) __attribute__((always_inline)) {
        float v = 0.f;
        if (H < 8) {
            float e[8];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                e[r] = rg[(R * j - r) & (RING - 1)];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (r <= H)
                    v = fmaf(cf[r], (R * j - r < limit) ? e[r] : 0.f, v);
        } else {
            for (int r = 0; r <= H; ++r) {
                const int k = R * j - r;
                v = fmaf(p.coef[r], (k < limit) ? rg[k & (RING - 1)] : 0.f, v);
            }
        }
        return v;
    };

    if (kt_end > kt_begin) {
        if (full_wg) {
            load_tile(kt_begin);
            store_tile(0);
        } else {
            stage_tile(kt_begin, 0);
        }
    }
    // Select blocks whose stencil lies wholly before kt_begin score 0.
    {
        const int jz = min((kt_begin * KT + R - 1) / R, be.S_sel);
        for (int j = lane; j < jz; j += 64)
            for (int tw = 0; tw < TOKW; ++tw)
                my_bins[tw * p.sb + j] = 0.f;
    }
    __syncthreads();

    auto key_tile = [&](const int kt, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int buf = (nbuf == 2) ? ((kt - kt_begin) & 1) : 0;
        // XM: lane i < TOKW * NKB fetches the mask word of token i / NKB for
        // 32-entry block i % NKB of this tile (issued before the K loads, so
        // waiting for it does not wait for them).
        constexpr int MWPL = (TOKW * NKB + 63) / 64;   // mask words per lane
        uint32_t mw_lane[MWPL];
        if constexpr (XM && MASK) {
#pragma unroll
            for (int m = 0; m < MWPL; ++m) {
                const int i = lane + 64 * m;
                const int word = kt * NKB + i % NKB;   // past the row: entries >= n_cmp
                mw_lane[m] = 0;
                if (i < TOKW * NKB && word < p.vis_words) {
                    const int tok = min(tok_w + i / NKB, be.T - 1);
                    mw_lane[m] = p.vis[(int64_t)tok * p.vis_words + word];
                }
            }
        }
        if (full_wg && kt + 1 < kt_end)
            load_tile(kt + 1);

        f32x16 s[2][NKB];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[rr][kb][r] = 0.f;
        const uint16_t* kt_lds = Ks + buf * KT * KS;
        // Raised wave priority while the MFMAs issue: a wave that reaches its
        // MFMAs gets them into the matrix pipe ahead of the other waves'
        // vector work, which then fills the MFMA shadow.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 kf = *(const u32x4*)&kt_lds[(kb * 32 + l32) * KS + ks * 16 + hf * 8];
#pragma unroll
                for (int rr = 0; rr < 2; ++rr)
                    s[rr][kb] = E::mfma(qa[rr][ks], kf, s[rr][kb]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        if constexpr (XM && MASK) {
#pragma unroll
            for (int m = 0; m < MWPL; ++m)
                if (lane + 64 * m < TOKW * NKB)
                    my_stg[lane + 64 * m] = mw_lane[m];
            wave_lds_sync();
        }

        // P, masked on the last tiles, summed over the heads of each token.
        // A token's sum starts at its first term (the same value as 0 + it:
        // every P is >= +0); every token of the wave has at least one term.
        float acc[TOKW][NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int key = kt * KT + kb * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pv = fast_exp2(fmaf(s[rr][kb][r], c, -bias[rr][r]));
                    if constexpr (MASK && !XM && GP < 8) {
                        const int pr = rr * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                        const int tok = tok_w + (pr >> LOG2GP);
                        // visible iff key*d + l - 1 <= the token's position
                        pv = (key * p.d + p.l - 1 <= tok + be.pos_off) ? pv : 0.f;
                    }
                    const int tw = (rr * 32 + 8 * (r >> 2) + (r & 3)) >> LOG2GP;
                    if (first_term(rr, r, LOG2GP))
                        acc[tw][kb] = pv;
                    else
                        acc[tw][kb] += pv;
                }
            }
        }
        if constexpr (MASK && !XM && GP >= 8) {
            // Groups of 8 or more: the heads summed in acc[tw][kb] are rows
            // of token tok_w + tw in both half-waves, so the visibility rule
            // applies to the sum (invisible entries' exponentials, however
            // large, are dropped by the select).
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int key = kt * KT + kb * 32 + l32;
#pragma unroll
                for (int tw = 0; tw < TOKW; ++tw)
                    acc[tw][kb] = (key * p.d + p.l - 1 <= tok_w + tw + be.pos_off) ? acc[tw][kb] : 0.f;
            }
        }
        if constexpr (MASK && XM) {
            // The heads summed in acc[tw][kb] share one token (tw, plus
            // hf * HSH for groups below 8) and one key, so the mask applies
            // to the sum: kept iff the entry exists and its bit is set.
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bool in = kt * KT + kb * 32 + l32 < be.n_cmp;
#pragma unroll
                for (int tw = 0; tw < TOKW; ++tw) {
                    if ((tw & HSH) == 0) {
                        const uint32_t w = my_stg[(tw + hf * HSH) * NKB + kb];
                        acc[tw][kb] = (in && ((w >> l32) & 1u)) ? acc[tw][kb] : 0.f;
                    }
                }
            }
        }
#pragma unroll
        for (int tw = 0; tw < TOKW; ++tw) {
            if constexpr (GP >= 8) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const float v = half_sum(acc[tw][kb]);
                    const int ri = (kt * KT + kb * 32 + l32) & (RING - 1);
                    if (hf == 0) {
                        my_ring[tw * RINGP + ri] = v;
                        if (ri < kTopkRingDup)
                            my_ring[tw * RINGP + RING + ri] = v;
                    }
                }
            } else {
                if ((tw & HSH) == 0) {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const int ri = (kt * KT + kb * 32 + l32) & (RING - 1);
                        float* rg = my_ring + (tw + hf * HSH) * RINGP;
                        rg[ri] = acc[tw][kb];
                        if (ri < kTopkRingDup)
                            rg[RING + ri] = acc[tw][kb];
                    }
                }
            }
        }
        wave_lds_sync();

        // At the end of a batch of nbt tiles (and after the last tile): the
        // select blocks j whose stencil top R*j lies in the batch's keys (at
        // most nbt * nj_slots of them per token), one (token, block) pair
        // per lane.
        if (++bat_n == nbt || kt + 1 == kt_end) {
            const int key0 = (kt + 1 - bat_n) * KT;   // the batch's first key
            bat_n = 0;
            const int jlo = (key0 + R - 1) / R;
            const int nj = min(((kt + 1) * KT + R - 1) / R, be.S_sel) - jlo;
            for (int tw0 = 0; tw0 < TOKW; tw0 += tpp) {
                const int tw = tw0 + tw_l;
                if (tw_l < tpp && tw < TOKW && jj_l < nj) {
                    const int j = jlo + jj_l;
                    const float* rg = my_ring + tw * RINGP;
                    my_bins[tw * p.sb + j] = __builtin_expect(short_stencil, 1) ? stencil5(rg, j) : stencil_long(rg, j);
                }
            }
            wave_lds_sync();
        }

        if (kt + 1 < kt_end) {
            if (nbuf == 1)
                __syncthreads();   // single buffer: every wave is done reading it
            if (full_wg)
                store_tile(nbuf == 2 ? (buf ^ 1) : 0);
            else
                stage_tile(kt + 1, nbuf == 2 ? (buf ^ 1) : 0);
        }
        __syncthreads();
    };

    // Tiles every row of the workgroup sees in full need no mask.
    int kt = kt_begin;
    for (; kt < n_full; ++kt)
        key_tile(kt, std::false_type{});
    for (; kt < kt_end; ++kt)
        key_tile(kt, std::true_type{});

    // Select blocks past the last tile: only entries < keys_done can be
    // non-zero.  Without the debug output only the blocks the wave's tokens
    // may pick (j * l' <= t) are needed.
    {
        const int keys_done = kt_end * KT;
        const int jlo = (keys_done + R - 1) / R;
        const int j_end = (p.pslc || p.cand) ? be.S_sel : min(be.S_sel, (tok_w + TOKW - 1 + be.pos_off) / p.lsel + 1);
        for (int j = jlo + lane; j < j_end; j += 64)
            for (int tw = 0; tw < TOKW; ++tw)
                my_bins[tw * p.sb + j] = stencil(my_ring + tw * RINGP, j, keys_done);
    }
    wave_lds_sync();

    // ---- top-k per (token, KV head), wave-local ----------------------------------
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int tw = 0; tw < TOKW; ++tw) {
        const int tok = tok_w + tw;
        if (tok >= be.T)
            break;                           // wave-uniform
        const float* brow = my_bins + tw * p.sb;
        const int64_t tg = (int64_t)be.q_off + tok;
        if (p.pslc) {
            float* dst = p.pslc + (tg * p.N2 + g) * p.s_stride;
            for (int j = lane; j < p.s_stride; j += 64)
                dst[j] = (j < be.S_sel) ? brow[j] : 0.f;
        }
        // Candidates: j with j*l' <= t (a prefix of the select blocks), or
        // the set bits of the token's packed topk_mask row.  Bit i of cm:
        // block lane + 64 i is a candidate.
        const int range = p.cand ? be.S_sel : min((tok + be.pos_off) / p.lsel + 1, be.S_sel);
        const int nch = (range + 63) >> 6;    // 64-block chunks of this row
        uint32_t cm = 0;
        int nvalid = 0;                       // number of candidates
        if (p.cand) {
            const uint32_t* crow = p.cand + (int64_t)tok * p.cand_words;
#pragma unroll
            for (int i = 0; i < kTopkMaxNpl; ++i) {
                if (i < nch) {
                    const int j = lane + 64 * i;
                    const bool c_i = j < range && ((crow[j >> 5] >> (j & 31)) & 1u);
                    cm |= (uint32_t)c_i << i;
                    nvalid += __popcll(__ballot(c_i));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kTopkMaxNpl; ++i)
                cm |= (uint32_t)(lane + 64 * i < range) << i;
            nvalid = range;
        }
        const int kk = min(p.count, nvalid);
        // Candidates as float bits; non-candidates hold 0 and never reach a
        // threshold >= 1 below.
        uint32_t key[kTopkMaxNpl];
#pragma unroll
        for (int i = 0; i < kTopkMaxNpl; ++i) {
            const int j = lane + 64 * i;
            key[i] = (i < nch && ((cm >> i) & 1u)) ? __float_as_uint(brow[j]) : 0u;
        }
        int32_t* trow = p.topk + (tg * p.N2 + g) * p.count;
        // Lower bound first: the kk-th largest of the per-lane maxima.  The
        // kk lanes at or above it hold kk distinct scores >= it, so every
        // score of the top kk is >= it too; usually only a few dozen
        // candidates reach it.  With at most 64 candidates the bound stays 0
        // and all of them are ranked.
        uint32_t tau0 = 0;
        if (nvalid > 64) {
            uint32_t lmax = 0;
#pragma unroll
            for (int i = 0; i < kTopkMaxNpl; ++i)
                if (i < nch)
                    lmax = max(lmax, key[i]);
            for (int bit = 30; bit >= 0; --bit) {
                const uint32_t cand = tau0 | (1u << bit);
                const int cnt = __popcll(__ballot(lmax >= cand));
                if (cnt >= kk) {
                    tau0 = cand;
                    if (cnt == kk)
                        break;
                }
            }
        }
        int ncand = 0;
#pragma unroll
        for (int i = 0; i < kTopkMaxNpl; ++i)
            if (i < nch)
                ncand += __popcll(__ballot(((cm >> i) & 1u) && key[i] >= tau0));
        if (ncand <= 64) {
            // Stage the candidates as 64-bit keys (score bits << 32 | ~index):
            // they order like (score desc, index asc), all distinct, and the
            // zeros that pad the staging to a multiple of 8 rank below every
            // candidate.  Each candidate's rank is the number of larger keys;
            // the first kk ranks are the picks.
            uint64_t* stg64 = (uint64_t*)my_stg;
            int pos = 0;
#pragma unroll
            for (int i = 0; i < kTopkMaxNpl; ++i) {
                if (i < nch) {
                    const bool sel = ((cm >> i) & 1u) && key[i] >= tau0;
                    const uint64_t bs = __ballot(sel);
                    if (sel) {
                        const int at = pos + __popcll(bs & lt_mask);
                        stg64[at] = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(lane + 64 * i);
                    }
                    pos += __popcll(bs);
                }
            }
            const int nc8 = (ncand + 7) & ~7;
            if (lane >= ncand && lane < nc8)
                stg64[lane] = 0;
            wave_lds_sync();
            if (lane < ncand) {
                const uint64_t mu = stg64[lane];
                int rank = 0;
                for (int q = 0; q < nc8; q += 8) {
                    u64x2 o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = *(const u64x2*)&stg64[q + 2 * e];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        rank += (int)(o[e][0] > mu) + (int)(o[e][1] > mu);
                }
                if (rank < kk)
                    trow[rank] = (int32_t)~(uint32_t)mu;
            }
            if (lane >= kk && lane < p.count)
                trow[lane] = -1;
        } else {
            // Radix select, most significant bit first: tau grows while at least
            // kk keys stay >= tau.  Once exactly kk keys are >= tau they are the
            // kk largest and the search stops; otherwise tau ends as the kk-th
            // largest bit pattern.
            uint32_t tau = 0;
            if (nvalid > kk) {
                for (int bit = 30; bit >= 0; --bit) {
                    const uint32_t cand = tau | (1u << bit);
                    int cnt = 0;
#pragma unroll
                    for (int i = 0; i < kTopkMaxNpl; ++i)
                        if (i < nch)
                            cnt += __popcll(__ballot(key[i] >= cand));
                    if (cnt >= kk) {
                        tau = cand;
                        if (cnt == kk)
                            break;
                    }
                }
            }
            // Everything above tau, then the lowest-index candidates equal to tau.
            int n_gt = 0;
#pragma unroll
            for (int i = 0; i < kTopkMaxNpl; ++i)
                if (i < nch)
                    n_gt += __popcll(__ballot(key[i] > tau));
            const int need_eq = kk - n_gt;
            int pos_gt = 0, pos_eq = 0;
#pragma unroll
            for (int i = 0; i < kTopkMaxNpl; ++i) {
                if (i < nch) {
                    const bool cand_i = (cm >> i) & 1u;
                    const bool gt = cand_i && key[i] > tau;
                    const bool eq = cand_i && key[i] == tau;
                    const uint64_t bg = __ballot(gt);
                    const uint64_t beq = __ballot(eq);
                    const int rg = __popcll(bg & lt_mask);
                    const int re = __popcll(beq & lt_mask);
                    if (gt) {
                        my_stg[pos_gt + rg] = key[i];
                        my_stg[32 + pos_gt + rg] = (uint32_t)(lane + 64 * i);
                    }
                    if (eq && pos_eq + re < need_eq) {
                        my_stg[n_gt + pos_eq + re] = key[i];
                        my_stg[32 + n_gt + pos_eq + re] = (uint32_t)(lane + 64 * i);
                    }
                    pos_gt += __popcll(bg);
                    pos_eq += __popcll(beq);
                }
            }
            wave_lds_sync();
            // Order: score descending, index ascending.  Each pick counts the picks
            // that precede it and writes itself at that rank; unused slots get -1.
            if (lane < kk) {
                const uint32_t mk = my_stg[lane];
                const uint32_t mi = my_stg[32 + lane];
                int rank = 0;
                for (int q = 0; q < kk; q += 4) {
                    const u32x4 ok = *(const u32x4*)&my_stg[q];
                    const u32x4 oi = *(const u32x4*)&my_stg[32 + q];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        rank += (q + e < kk) && (ok[e] > mk || (ok[e] == mk && oi[e] < mi));
                }
                trow[rank] = (int32_t)mi;
            } else if (lane < p.count) {
                trow[lane] = -1;
            }
        }
        wave_lds_sync();   // the staging area is reused by the next token
    }
}

template <typename E, bool XM, int D1, int LOG2GP>
static hipError_t launch_t(const TopkParams& p, int n_tiles, size_t lds, hipStream_t stream)
{
    auto kern = k_slc_topk<E, XM, D1, LOG2GP>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(kern, dim3(n_tiles), dim3(p.waves * 64), lds, stream, p);
    return hipGetLastError();
}

template <typename E, bool XM, int D1>
static hipError_t launch_d(int log2gp, const TopkParams& p, int n_tiles, size_t lds, hipStream_t stream)
{
    switch (log2gp) {
    case 0: return launch_t<E, XM, D1, 0>(p, n_tiles, lds, stream);
    case 1: return launch_t<E, XM, D1, 1>(p, n_tiles, lds, stream);
    case 2: return launch_t<E, XM, D1, 2>(p, n_tiles, lds, stream);
    case 3: return launch_t<E, XM, D1, 3>(p, n_tiles, lds, stream);
    case 4: return launch_t<E, XM, D1, 4>(p, n_tiles, lds, stream);
    case 5: return launch_t<E, XM, D1, 5>(p, n_tiles, lds, stream);
    case 6: return launch_t<E, XM, D1, 6>(p, n_tiles, lds, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename E, bool XM>
static hipError_t launch_e(int d1, int log2gp, const TopkParams& p, int n_tiles, size_t lds,
                           hipStream_t stream)
{
    if (d1 == 64) return launch_d<E, XM, 64>(log2gp, p, n_tiles, lds, stream);
    if (d1 == 128) return launch_d<E, XM, 128>(log2gp, p, n_tiles, lds, stream);
    if (d1 == 192) return launch_d<E, XM, 192>(log2gp, p, n_tiles, lds, stream);
    return hipErrorInvalidValue;
}

int topk_log2_gp(int G)
{
    int lg = 0;
    while ((1 << lg) < G)
        ++lg;
    return lg <= 6 ? lg : -1;
}

size_t topk_lds_bytes(int d1, int log2gp, int waves, int sb, int kbufs)
{
    const size_t tokw = (size_t)(64 >> log2gp);
    return (size_t)kbufs * topk_key_tile(d1) * (d1 + 8) * 2 + (size_t)waves * tokw * (topk_ring(log2gp) + kTopkRingDup) * 4 +
           (size_t)waves * tokw * sb * 4 + (size_t)waves * 128 * 4;
}

bool slc_topk_supported(int d1) { return d1 == 64 || d1 == 128 || d1 == 192; }

hipError_t launch_slc_topk(int dtype, int d1, int log2gp, const TopkParams& p, int n_tiles,
                           size_t lds, hipStream_t stream)
{
    if (n_tiles <= 0)
        return hipSuccess;
    const bool xm = p.vis != nullptr;
    if (dtype == ElemBf16::code)
        return xm ? launch_e<ElemBf16, true>(d1, log2gp, p, n_tiles, lds, stream)
                  : launch_e<ElemBf16, false>(d1, log2gp, p, n_tiles, lds, stream);
    if (dtype == ElemF16::code)
        return xm ? launch_e<ElemF16, true>(d1, log2gp, p, n_tiles, lds, stream)
                  : launch_e<ElemF16, false>(d1, log2gp, p, n_tiles, lds, stream);
    return hipErrorInvalidValue;
}

}  // namespace nsa
