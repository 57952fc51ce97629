// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
// Nothing here is part of the public interface (include/nsa_cmp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

// Per-sequence extents and launch-tile ranges, uploaded into the workspace.
// Tiles of one kernel are numbered sequence by sequence; inside a sequence
// they run from the last row block (largest causal cost) to the first, and
// the KV heads of a row block are adjacent.
struct BatchEnt {
    int32_t q_off;      // first query token of the sequence (global)
    int32_t T;          // query tokens of the sequence
    int32_t cmp_off;    // first compressed entry of the sequence (global)
    int32_t n_cmp;      // compressed entries of the sequence
    int32_t tile_off_a; // first tile of the attention kernel
    int32_t n_rb_a;     // row blocks of the attention kernel (per KV head)
    int32_t tile_off_c; // first tile of the importance/top-k kernel
    int32_t n_rb_c;     // row blocks of the importance/top-k kernel
    int32_t S_sel;      // select blocks of the sequence, ceil(T / l')
    int32_t tile_off_s; // first workgroup of the selected-block attention kernel
    int32_t n_rb_s;     // row blocks of the selected-block attention kernel (per KV head)
    int32_t tile_off_k; // first key block (kBwdKeyBlock entries, per KV head) of the key-side backward
    int32_t pos_off;    // KV tokens before the first query token (chunked prefill; 0 otherwise)
    int32_t kv_off;     // first raw key/value token of the sequence (global; == q_off unless chunked)
    int32_t pad1, pad2;
};
static_assert(sizeof(BatchEnt) == 64, "BatchEnt layout");

// The table of B sequences is followed in the workspace by one more entry
// whose first word is the status: 0 when the table is valid.  The host
// planner uploads it as 0; the device planner writes the outcome of its
// checks (kMetaErr* bits).  Kernels reading the table return at once, before
// any other memory access, when it is not 0.
constexpr int kMetaErrPrefix = 1;     // a prefix sum decreases (or is negative)
constexpr int kMetaErrKvShort = 2;    // fewer key/value tokens than queries in a sequence
constexpr int kMetaErrCmpLen = 4;     // compressed length != floor((Tkv - l)/d) + 1
constexpr int kMetaErrSelLen = 8;     // select length != ceil(Tkv / l')
constexpr int kMetaErrCapacity = 16;  // a sequence exceeds the plan's longest / largest counts
constexpr int kMetaErrTotals = 32;    // totals or launch sizes differ from the plan's
constexpr int kMetaErrSplit = 64;     // a work list (split attention, key-side backward) differs from the host's counts

// ---- planning on the device ----------------------------------------------------
struct MetaParams {
    const int64_t* qlen;     // [B] prefix sums of query tokens, device
    const int64_t* kvlen;    // NULL or [B] prefix sums of key/value tokens
    const int64_t* cmplen;   // [B] prefix sums of compressed entries
    const int64_t* sellen;   // [B] prefix sums of select blocks
    struct BatchEnt* table;  // [B] out
    int* status;             // out: 0 or kMetaErr* bits
    int B, l, d, lsel, N2, G, GP;
    int rows_a, rows_c, rows_s;        // rows per workgroup: attention, top-k (padded group), selected-block attention
    int64_t T_max, ncmp_max, S_max;    // the plan's largest sequence, compressed and select counts
    int64_t T1, T2, Tkv_total, S_total, tiles_a, tiles_c, tiles_s, tiles_k;   // the plan's totals
};
hipError_t launch_meta_table(const MetaParams& p, hipStream_t stream);

// ---- compression kernel ---------------------------------------------------
constexpr int kCompressMaxSeg = 128;   // sequences per launch (more -> several launches)

// Compression: a workgroup owns a run of nw consecutive windows of one
// sequence and one column slab (cs 16-byte chunks) of the [N*D] row, and
// stages the run's input rows in LDS (at most kCompressStageBytes).
constexpr int kCompressStageBytes = 64 * 1024;

struct CompressParams {
    const uint16_t* x;   // [T, N, D]
    const uint16_t* w;   // [l, N]
    uint16_t* y;         // [T2, N, D]
    int N, D, l, d;
    int nseg;
    int max_blocks_x;    // grid x: a multiple of 8 covering (runs x slabs) of the longest sequence
    int cs_log2;         // log2 of the 16-byte chunks per column slab
    int nslab;           // column slabs per row: N*D/8 / cs
    int nw;              // windows per run
    int in_off[kCompressMaxSeg];   // first input token of each sequence
    int out_off[kCompressMaxSeg];  // first output entry of each sequence
    int n_out[kCompressMaxSeg];    // output entries of each sequence
};

// dtype: 0 = bfloat16, 1 = float16 (the public enum's values).
hipError_t launch_compress(int dtype, const CompressParams& p, hipStream_t stream);

// Backward of the compression for up to kCompressMaxSeg sequences per launch.
struct CompressBwdParams {
    const uint16_t* x;    // [T, N, D]
    const uint16_t* w;    // [l, N]
    const float* dy;      // [T2, N, D]
    float* dx;            // [T, N, D]
    float* dw;            // [l, N]
    int N, D, l, d;
    int nseg;
    int max_blocks_x;     // dx kernel: blocks of 256 threads covering the longest sequence
    int accumulate;       // dw kernel: add to dw (a later launch of one call) instead of writing
    float* part;          // dw chunk sums (scratch: the start of dx, before dx is written)
    int in_off[kCompressMaxSeg];
    int out_off[kCompressMaxSeg];
    int n_in[kCompressMaxSeg];     // tokens of each sequence
    int n_out[kCompressMaxSeg];    // windows of each sequence
};
hipError_t launch_compress_bwd_dw(int dtype, const CompressBwdParams& p, int chunks, hipStream_t stream);
hipError_t launch_compress_bwd_dx(int dtype, const CompressBwdParams& p, hipStream_t stream);

// ---- explicit masks ---------------------------------------------------------
// A [rows, cols] byte matrix (non-zero = masked out) becomes a bit matrix of
// kept pairs: word w of row t holds columns 32w .. 32w+31, bit k set iff
// column 32w + k < cols and its byte is zero.
struct MaskPackParams {
    const uint8_t* src;   // [src_rows, src_cols] bytes
    int64_t src_cols;
    uint32_t* dst;        // [rows, words]
    int rows, words;
    int4* span;           // NULL, or [rows]: (first word with a kept pair, last such word + 1,
                          // number of leading words that keep all 32 pairs, 0);
                          // (words, 0, 0, 0) for a row that keeps nothing
};
hipError_t launch_pack_mask(const MaskPackParams& p, hipStream_t stream);

// ---- attention kernels ------------------------------------------------------
// One workgroup of a split attention launch: row block rb of (sequence b,
// KV head g), key tiles [kt0, kt0 + n_kt).  slot < 0: the row block is not
// split and the workgroup writes the outputs; else its partial slot.
struct SplitItem {
    int32_t b, g, rb, kt0, n_kt, slot, pad0, pad1;
};

struct AttnParams {
    const uint16_t* q;    // [T1, N1, D1]
    const uint16_t* kc;   // [T2, N2, D1]
    const uint16_t* vc;   // [T2, N2, D2]
    uint16_t* out;        // [T1, N1, D2]
    float* smax;          // [T1, N1, 8]
    float* ssum;          // [T1, N1, 8]
    float* bias;          // NULL or [T1, N1]: row_bias(max, sum) of every row, for the importance pass
    const BatchEnt* bt;   // [B], device
    const int* status;    // the table's status word (a kernel returns at once when it is not 0)
    int B, N1, N2, G;
    int l, d;
    float c;              // |scale| * log2(e): raw score -> base-2 exponent
    float abs_scale;      // |scale|: raw score -> natural-unit score
    float thr;            // running-max slack before rescaling, raw-score units
    uint32_t qsign;       // 0x80008000 when scale < 0 (q negated), else 0
    const uint32_t* vis;  // NULL (positional rule) or packed atten_mask [T_max, vis_words]
    const int4* vis_span; // per row of vis: span of words with a kept pair, leading full words
    int vis_words;
    // Split key ranges (positional rule only): NULL, or one item per
    // workgroup; pieces with slot >= 0 leave partial sums in `part`.
    const SplitItem* split;
    float* part;          // [slots][rows per workgroup][D2 + 4]: O, then (L, R, M)
};

// One row block whose pieces occupy partial slots [slot0, slot0 + n).
struct CombineItem {
    int32_t b, g, rb, slot0, n, pad0, pad1, pad2;
};

// Work list of a split launch, built on the device from the table.
struct SplitPlanParams {
    const BatchEnt* table;   // [B]
    int* status;             // the table's status word (set on a count mismatch)
    int4* chunk_tot;         // [chunks]: items, combine items, slots of each 256 row blocks
    SplitItem* items;        // [n_items]
    CombineItem* combs;      // [n_combs]
    int B, N2, G, l, d, rows_a, C, tiles_a;
    int64_t n_items, n_combs, n_slots;   // the host's counts for this plan and C
};
int plan_chunks(int64_t units);   // chunk totals a work-list build needs (int4 each)
hipError_t launch_split_plan(const SplitPlanParams& p, hipStream_t stream);
hipError_t launch_attn_combine(int dtype, int d1, int d2, const AttnParams& p, const CombineItem* items,
                               int n_items, hipStream_t stream);

// Compressed entries per key tile of the importance/top-k kernel: 32 keeps
// its registers within three waves per SIMD up to D1 = 128; D1 = 192 stays
// at two waves either way and prefers the longer tile.
constexpr int topk_key_tile(int d1) { return d1 > 128 ? 64 : 32; }
constexpr int kKeyTileMin = 32;

hipError_t launch_cmp_attn(int dtype, int d1, int d2, const AttnParams& p, int n_tiles,
                           hipStream_t stream);
bool cmp_attn_supported(int d1, int d2);
int cmp_attn_rows_per_wg(int d1, int d2);   // query rows per attention workgroup

struct TopkParams {
    const uint16_t* q;    // [T1, N1, D1]
    const uint16_t* kc;   // [T2, N2, D1]
    const float* smax;    // [T1, N1, 8]
    const float* ssum;    // [T1, N1, 8]
    const float* bias;    // NULL (derive from smax, ssum) or [T1, N1] as the attention pass wrote it
    int32_t* topk;        // [T1, N2, count]
    float* pslc;          // NULL or [T1, N2, s_stride]
    const BatchEnt* bt;   // [B], device
    const int* status;    // the table's status word
    int B, N1, N2, G;
    int l, d, lsel, count;
    int R, H;             // R = l'/d; H = largest remap offset = R + floor(l/d) - 2
    float coef[16];       // remap coefficient of P_cmp[R*j - r], r = 0..H
    float c;              // |scale| * log2(e)
    uint32_t qsign;
    int s_stride;         // row stride of pslc (max select blocks)
    int sb;               // LDS row length of the importance scores (multiple of 64)
    int nj_slots;         // ceil(key tile / R): select blocks a key tile can finish per token
    int npl;              // candidates per lane in top-k, sb / 64
    int waves;            // waves per workgroup
    int kbufs;            // K tile buffers in LDS (2 = double buffered)
    const uint32_t* vis;  // NULL (positional rule) or packed atten_mask [T_max, vis_words]
    const int4* vis_span; // per row of vis: span of words with a kept pair, leading full words
    int vis_words;
    const uint32_t* cand; // NULL (positional rule) or packed topk_mask [T_max, cand_words]
    int cand_words;
};

// ---- selected-block attention ------------------------------------------------
struct SelParams {
    const uint16_t* q;      // [T1, N1, D1]
    const uint16_t* k;      // [T1, N2, D1] raw keys
    const uint16_t* v;      // [T1, N2, D2] raw values
    const int32_t* topk;    // [T1, N2, count]
    uint16_t* out;          // [T1, N1, D2]
    float* lse;             // [T1, N1]
    const BatchEnt* bt;     // [B], device (tile_off_s / n_rb_s: kSelRows rows per workgroup)
    const int* status;      // the table's status word
    int B, N1, N2, G;
    int lsel, count;
    float c;                // |scale| * log2(e)
    float abs_scale;
    float thr;              // running-max slack before rescaling, raw-score units
    uint32_t qsign;
    int sw;                 // 32-bit words per block set, ceil(max select blocks / 32)
    int tpw;                // block sets per workgroup (tokens its rows can span)
};

constexpr int kSelRows = 64;                  // (token, head) rows per workgroup
bool sel_attn_supported(int d1, int d2);
size_t sel_attn_lds_bytes(int tpw, int sw);   // dynamic LDS per workgroup
hipError_t launch_sel_attn(int dtype, int d1, int d2, const SelParams& p, int n_tiles, size_t lds,
                           hipStream_t stream);

// ---- backward of the compressed attention -------------------------------------
constexpr int kBwdKeyBlock = 128;     // compressed entries per key-side work item (4 waves x 32)

// One key-side work item: key block kb (entries kBwdKeyBlock*kb ...) of KV
// head g of sequence b, query tiles [qt0, qt0 + n_qt) of the 32-row tiles
// that see the block; slot < 0: the block's only item (writes dK, dV),
// else its partial slot.
struct BwdItem {
    int32_t b, g, kb, qt0, n_qt, slot, pad0, pad1;
};

struct BwdParams {
    const uint16_t* q;     // [T1, N1, D1]
    const uint16_t* kc;    // [T2, N2, D1]
    const uint16_t* vc;    // [T2, N2, D2]
    const uint16_t* out;   // [T1, N1, D2] forward attention_out
    const uint16_t* dout;  // [T1, N1, D2] gradient of attention_out
    const float* smax;     // [T1, N1, 8] forward softmax_max
    const float* ssum;     // [T1, N1, 8] forward softmax_sum
    float* dq;             // [T1, N1, D1]
    float* dkc;            // [T2, N2, D1]
    float* dvc;            // [T2, N2, D2]
    float* rowstat;        // workspace [T1 * N1][2]: exponent bias and Delta = dout . out per row
    const BatchEnt* bt;    // [B], device
    const int* status;     // the table's status word
    int B, N1, N2, G;
    int l, d;
    float c;               // |scale| * log2(e)
    float scale;           // signed scale
    uint32_t qsign;        // 0x80008000 when scale < 0 (q negated), else 0
    uint32_t gdiv_m, gdiv_s;   // n / G = (umulhi(n, m) + n) >> s for 0 <= n < 2^31
    const BwdItem* items;  // key-side work items
    const CombineItem* combs;   // key blocks cut into pieces (rb = key block), added in piece order
    float* part;           // [slots][kBwdKeyBlock][D1 + D2]: unscaled partial dK, dV
};

// Key-side work list, built on the device from the table: every key block
// becomes ceil(n_qt / qmax) items (at least one).
struct BwdPlanParams {
    const BatchEnt* table;   // [B]
    int* status;             // the table's status word (set on a count mismatch)
    int4* chunk_tot;         // [chunks]: items, combine items, slots of each 256 key blocks
    BwdItem* items;          // [n_items]
    CombineItem* combs;      // [n_combs]
    int B, N2, G, l, d, qmax, tiles_k;
    int64_t n_items, n_combs, n_slots;   // the host's counts
};
hipError_t launch_bwd_plan(const BwdPlanParams& p, hipStream_t stream);

bool attn_bwd_supported(int d1, int d2);
hipError_t launch_attn_bwd(int dtype, int d1, int d2, const BwdParams& p, int tiles_q, int n_items,
                           int n_combs, hipStream_t stream);

constexpr int kTopkRing = 128;         // smallest per-token ring of group-summed P (floats)
// Ring length for 64 / 2^log2gp tokens per wave: the stencil pass runs once
// per batch of key tiles, sized so that the wave's lanes are about all busy,
// and the ring keeps a batch plus the stencil's reach (at most 15 entries).
constexpr int topk_ring(int log2gp) { return log2gp >= 6 ? 4 * kTopkRing : (log2gp == 5 ? 2 * kTopkRing : kTopkRing); }
constexpr int kTopkRingDup = 4;        // ring slots repeated past its end (stencils of <= 5 taps)
constexpr int kTopkMaxNpl = 16;        // at most 1024 select blocks per sequence

int topk_log2_gp(int G);               // log2 of the padded group size, -1 if G > 64
size_t topk_lds_bytes(int d1, int log2gp, int waves, int sb, int kbufs);
hipError_t launch_slc_topk(int dtype, int d1, int log2gp, const TopkParams& p, int n_tiles,
                           size_t lds, hipStream_t stream);
bool slc_topk_supported(int d1);

}  // namespace nsa
