// C ABI of the library (include/nsa_cmp.h): argument validation, extent
// derivation, launch planning and launches.  The library allocates no device
// memory; an attention call copies a small per-sequence table into the
// caller's workspace (or, with a device-planned plan, finds it there, written
// by nsa_compress_attention_metadata) and launches its kernels on the
// caller's stream.  Plans are never written after they are made.
#include "nsa_cmp.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "nsa_internal.h"

namespace {

thread_local std::string g_last_error;

nsa_status fail(nsa_status s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

nsa_status ok()
{
    g_last_error.clear();
    return NSA_OK;
}

bool mult16(int64_t v) { return v > 0 && v % 16 == 0; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t n_cmp_of(int64_t T, int64_t l, int64_t d) { return T < l ? 0 : (T - l) / d + 1; }

// Validates host prefix sums; fills per-sequence lengths.
nsa_status read_prefix(const int64_t* prefix, int64_t batch, const char* name,
                       std::vector<int64_t>& lens)
{
    if (!prefix)
        return fail(NSA_ERR_NULLPTR, "%s is NULL", name);
    lens.resize((size_t)batch);
    int64_t prev = 0;
    for (int64_t b = 0; b < batch; ++b) {
        if (prefix[b] < prev)
            return fail(NSA_ERR_SHAPE, "%s must be non-decreasing prefix sums from 0 (entry %lld = %lld after %lld)",
                        name, (long long)b, (long long)prefix[b], (long long)prev);
        lens[(size_t)b] = prefix[b] - prev;
        prev = prefix[b];
    }
    if (prev > INT32_MAX)
        return fail(NSA_ERR_UNSUPPORTED, "%s total %lld exceeds 2^31-1", name, (long long)prev);
    return NSA_OK;
}

nsa_status check_dtype(int dtype)
{
    if (dtype == NSA_DTYPE_BF16 || dtype == NSA_DTYPE_FP16)
        return NSA_OK;
    return fail(NSA_ERR_DTYPE, "unknown dtype code %d", dtype);
}

}  // namespace

struct nsa_plan_s {
    int64_t B, N1, N2, D1, D2, l, d, lsel, count;
    int dtype;   // element type of q, k, v and attention_out (nsa_dtype)
    float scale;
    int64_t T1, T2, S_total, S_max;
    int64_t T_max, ncmp_max;          // longest sequence, most compressed entries
    int64_t vis_words, cand_words;    // packed mask row lengths (32-bit words)
    size_t ws_masked_bytes;           // workspace of the calls that take masks
    size_t ws_bwd_bytes;              // workspace of the backward call
    int64_t tiles_k;                  // key blocks of the key-side backward (all KV heads)
    int64_t bwd_qmax;                 // query tiles per key-side work item, at most
    int64_t bwd_items, bwd_combs, bwd_slots;   // the key-side work list's counts
    int log2gp, topk_waves, topk_kbufs, sb;
    size_t topk_lds;
    int64_t tiles_a, tiles_c, tiles_s;
    size_t ws_bytes;                  // the table, then the per-row bias array (the headline calls' workspace)
    size_t table_bytes;               // the table and its status entry, rounded up to 256 bytes
    size_t bias_off;                  // byte offset of the [T1, N1] float32 bias array the forward writes
    // B entries, then one zero entry whose first word is the status word
    // (kernels exit at once when it is not 0; the upload keeps it 0)
    std::vector<nsa::BatchEnt> table;
    int64_t T_kv;             // key/value tokens of all sequences (== T1 unless chunked)
    bool chunked = false;     // some sequence has key/value tokens before its first query
    bool device_meta = false; // execute calls read the table the device planner wrote
    int rows_c = 0;           // rows per workgroup of the top-k kernel
};

extern "C" {

int64_t nsa_compress_out_len(int64_t seq_len, int64_t l, int64_t d)
{
    if (l < 1 || d < 1 || seq_len < 0)
        return -1;
    return n_cmp_of(seq_len, l, d);
}

const char* nsa_status_string(nsa_status s)
{
    switch (s) {
    case NSA_OK: return "NSA_OK";
    case NSA_ERR_NULLPTR: return "NSA_ERR_NULLPTR";
    case NSA_ERR_DTYPE: return "NSA_ERR_DTYPE";
    case NSA_ERR_SHAPE: return "NSA_ERR_SHAPE";
    case NSA_ERR_CONSTRAINT: return "NSA_ERR_CONSTRAINT";
    case NSA_ERR_WORKSPACE: return "NSA_ERR_WORKSPACE";
    case NSA_ERR_UNSUPPORTED: return "NSA_ERR_UNSUPPORTED";
    case NSA_ERR_HIP: return "NSA_ERR_HIP";
    }
    return "NSA_ERR_UNKNOWN";
}

const char* nsa_last_error(void) { return g_last_error.c_str(); }

nsa_status nsa_compress(const void* input, const void* weight, const int64_t* act_seq_len,
                        int64_t batch, int64_t total_tokens, int64_t num_heads, int64_t head_dim,
                        int64_t l, int64_t d, nsa_dtype dtype, void* output,
                        int64_t output_tokens, void* stream)
{
    if (!input || !weight || !act_seq_len)
        return fail(NSA_ERR_NULLPTR, "input, weight and act_seq_len must not be NULL");
    nsa_status st = check_dtype((int)dtype);
    if (st != NSA_OK)
        return st;
    if (batch < 1)
        return fail(NSA_ERR_SHAPE, "act_seq_len must not be empty (batch = %lld)", (long long)batch);
    if (num_heads < 1)
        return fail(NSA_ERR_SHAPE, "num_heads must be >= 1");
    if (!mult16(head_dim) || head_dim > 256)
        return fail(NSA_ERR_CONSTRAINT, "head_dim must be a multiple of 16 and <= 256 (got %lld)", (long long)head_dim);
    if (!mult16(l) || l > 128)
        return fail(NSA_ERR_CONSTRAINT, "compress_block_size must be a multiple of 16 in [16, 128] (got %lld)", (long long)l);
    if (!mult16(d) || d > l)
        return fail(NSA_ERR_CONSTRAINT, "compress_stride must be a multiple of 16 with 16 <= d <= compress_block_size (got %lld)", (long long)d);
    if (l * num_heads > 128 * 64)
        return fail(NSA_ERR_UNSUPPORTED, "compress_block_size * num_heads must be <= 8192");
    std::vector<int64_t> lens;
    st = read_prefix(act_seq_len, batch, "act_seq_len", lens);
    if (st != NSA_OK)
        return st;
    if (act_seq_len[batch - 1] != total_tokens)
        return fail(NSA_ERR_SHAPE, "last prefix sum %lld != total_tokens %lld",
                    (long long)act_seq_len[batch - 1], (long long)total_tokens);
    int64_t T2 = 0;
    for (int64_t T : lens)
        T2 += n_cmp_of(T, l, d);
    if (T2 != output_tokens)
        return fail(NSA_ERR_SHAPE, "output_tokens %lld != sum of compressed lengths %lld",
                    (long long)output_tokens, (long long)T2);
    if (T2 > 0 && !output)
        return fail(NSA_ERR_NULLPTR, "output must not be NULL");
    if (!aligned(input, 16) || (output && !aligned(output, 16)) || !aligned(weight, 2))
        return fail(NSA_ERR_CONSTRAINT, "input/output must be 16-byte aligned");
    if (T2 == 0)
        return ok();

    const int64_t nd8 = num_heads * head_dim / 8;
    nsa::CompressParams p;
    std::memset(&p, 0, sizeof p);
    p.x = (const uint16_t*)input;
    p.w = (const uint16_t*)weight;
    p.y = (uint16_t*)output;
    p.N = (int)num_heads;
    p.D = (int)head_dim;
    p.l = (int)l;
    p.d = (int)d;
    // Column slab: the largest power of two <= 16 chunks that divides the
    // row's chunks; a run: as many windows as the staged rows and the
    // workgroup's threads allow.
    p.cs_log2 = 0;
    while (p.cs_log2 < 4 && nd8 % (2 << p.cs_log2) == 0)
        ++p.cs_log2;
    const int64_t cs = 1 << p.cs_log2;
    p.nslab = (int)(nd8 / cs);
    const int64_t stage_rows = nsa::kCompressStageBytes / 16 / cs;
    p.nw = (int)std::min<int64_t>((stage_rows - l) / d + 1, 256 / cs);
    int64_t in_off = 0, out_off = 0;
    size_t b = 0;
    while (b < lens.size()) {
        p.nseg = 0;
        int64_t max_items = 0;
        while (b < lens.size() && p.nseg < nsa::kCompressMaxSeg) {
            const int64_t n = n_cmp_of(lens[b], l, d);
            if (n > 0) {
                p.in_off[p.nseg] = (int)in_off;
                p.out_off[p.nseg] = (int)out_off;
                p.n_out[p.nseg] = (int)n;
                const int64_t blocks = (n + p.nw - 1) / p.nw * p.nslab;
                if (blocks > max_items)
                    max_items = blocks;
                ++p.nseg;
            }
            in_off += lens[b];
            out_off += n;
            ++b;
        }
        if (p.nseg == 0)
            continue;
        if (max_items > (int64_t)INT32_MAX - 8)
            return fail(NSA_ERR_CONSTRAINT, "sequence too long for one compression launch");
        p.max_blocks_x = (int)((max_items + 7) / 8 * 8);
        hipError_t e = nsa::launch_compress((int)dtype, p, (hipStream_t)stream);
        if (e != hipSuccess)
            return fail(NSA_ERR_HIP, "compress launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

// Query tiles (32 rows t*G + hh) that see key block kb of a sequence: from
// the row of the block's first entry to the end of the sequence.
static int64_t bwd_tiles_of(const nsa::BatchEnt& e, int64_t kb, int64_t G, int64_t l, int64_t d)
{
    const int64_t first = std::min<int64_t>(std::max<int64_t>(kb * nsa::kBwdKeyBlock * d + l - 1 - e.pos_off, 0), e.T) * G;
    return ((int64_t)e.T * G - first + 31) / 32;
}

// Key-side backward work list: every key block (per KV head) is cut into
// ceil(n / qmax) pieces of its n query tiles, qmax chosen so that the list
// holds about 2048 items (eight per compute unit) however long the sequences
// are, and no fewer than 16 tiles per item.  The list is built on the device
// (launch_bwd_plan); these counts size the workspace and the launches.
static void bwd_counts(nsa_plan_s* plan)
{
    const int64_t G = plan->N1 / plan->N2;
    int64_t total = 0;
    for (int64_t b = 0; b < plan->B; ++b) {
        const nsa::BatchEnt& e = plan->table[(size_t)b];
        const int64_t nkb = (e.n_cmp + nsa::kBwdKeyBlock - 1) / nsa::kBwdKeyBlock;
        for (int64_t kb = 0; kb < nkb; ++kb)
            total += bwd_tiles_of(e, kb, G, plan->l, plan->d);
    }
    total *= plan->N2;
    const int64_t qmax = std::max<int64_t>(16, (total + 2047) / 2048);
    int64_t items = 0, combs = 0, slots = 0;
    for (int64_t b = 0; b < plan->B; ++b) {
        const nsa::BatchEnt& e = plan->table[(size_t)b];
        const int64_t nkb = (e.n_cmp + nsa::kBwdKeyBlock - 1) / nsa::kBwdKeyBlock;
        for (int64_t kb = 0; kb < nkb; ++kb) {
            const int64_t n = bwd_tiles_of(e, kb, G, plan->l, plan->d);
            const int64_t pieces = n > qmax ? (n + qmax - 1) / qmax : 1;
            items += pieces;
            if (pieces > 1) {
                combs += 1;
                slots += pieces;
            }
        }
    }
    plan->bwd_qmax = qmax;
    plan->bwd_items = items * plan->N2;
    plan->bwd_combs = combs * plan->N2;
    plan->bwd_slots = slots * plan->N2;
}

// Backward workspace after the table: each row's exponent bias and Delta,
// the work-list build's chunk totals, the work list, its combine items, and
// the partial dK, dV of the pieces.
struct BwdLayout {
    size_t rowstat_off, chunk_off, items_off, combs_off, part_off, bytes;
};

static BwdLayout bwd_layout(const nsa_plan_s* plan)
{
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    BwdLayout k;
    k.rowstat_off = plan->ws_bytes;
    k.chunk_off = k.rowstat_off + up((size_t)plan->T1 * (size_t)plan->N1 * 8);
    k.items_off = k.chunk_off + up((size_t)nsa::plan_chunks(plan->tiles_k) * sizeof(int4));
    k.combs_off = k.items_off + up((size_t)plan->bwd_items * sizeof(nsa::BwdItem));
    k.part_off = k.combs_off + up((size_t)plan->bwd_combs * sizeof(nsa::CombineItem));
    k.bytes = k.part_off + (size_t)plan->bwd_slots * nsa::kBwdKeyBlock * (size_t)(plan->D1 + plan->D2) * 4;
    return k;
}

static nsa_status make_plan(
    int64_t batch, const int64_t* act_seq_qlen, const int64_t* act_seq_kvlen, const int64_t* act_cmp_seq_kvlen,
    const int64_t* act_sel_seq_kvlen, int64_t head_num, int64_t kv_head_num, int64_t d1,
    int64_t d2, float scale_value, int64_t l, int64_t d, int64_t lsel, int64_t count,
    nsa_dtype dtype, size_t* workspace_bytes, nsa_plan* plan_out)
{
    if (plan_out)
        *plan_out = nullptr;
    if (!workspace_bytes || !plan_out)
        return fail(NSA_ERR_NULLPTR, "workspace_bytes and plan_out must not be NULL");
    nsa_status st = check_dtype((int)dtype);
    if (st != NSA_OK)
        return st;
    if (batch < 1)
        return fail(NSA_ERR_SHAPE, "the prefix-sum lists must not be empty (batch = %lld)", (long long)batch);
    // Parameter constraints of the compressed-attention operator.
    if (!mult16(l) || l > 128)
        return fail(NSA_ERR_CONSTRAINT, "compress_block_size must be a multiple of 16 in [16, 128] (got %lld)", (long long)l);
    if (!mult16(d) || d > 64)
        return fail(NSA_ERR_CONSTRAINT, "compress_stride must be a multiple of 16 in [16, 64] (got %lld)", (long long)d);
    if (!mult16(lsel) || lsel > 128)
        return fail(NSA_ERR_CONSTRAINT, "select_block_size must be a multiple of 16 in [16, 128] (got %lld)", (long long)lsel);
    if (count < 1 || count > 32)
        return fail(NSA_ERR_CONSTRAINT, "select_block_count must be in [1, 32] (got %lld)", (long long)count);
    if (l < d)
        return fail(NSA_ERR_CONSTRAINT, "compress_block_size (%lld) must be >= compress_stride (%lld)", (long long)l, (long long)d);
    if (lsel < l)
        return fail(NSA_ERR_CONSTRAINT, "select_block_size (%lld) must be >= compress_block_size (%lld)", (long long)lsel, (long long)l);
    if (lsel % d != 0)
        return fail(NSA_ERR_CONSTRAINT, "select_block_size (%lld) must be a multiple of compress_stride (%lld)", (long long)lsel, (long long)d);
    if (!mult16(d1) || !mult16(d2))
        return fail(NSA_ERR_CONSTRAINT, "head dims must be positive multiples of 16 (D1 = %lld, D2 = %lld)", (long long)d1, (long long)d2);
    if (d1 < d2)
        return fail(NSA_ERR_CONSTRAINT, "D1 (%lld) must be >= D2 (%lld)", (long long)d1, (long long)d2);
    if (kv_head_num < 1 || head_num < kv_head_num || head_num % kv_head_num != 0)
        return fail(NSA_ERR_CONSTRAINT, "need N1 >= N2 >= 1 and N1 %% N2 == 0 (N1 = %lld, N2 = %lld)", (long long)head_num, (long long)kv_head_num);
    if (!std::isfinite(scale_value))
        return fail(NSA_ERR_CONSTRAINT, "scale_value must be finite");

    std::vector<int64_t> qlen, kvlen, clen, slen;
    if ((st = read_prefix(act_seq_qlen, batch, "actual_seq_qlen", qlen)) != NSA_OK) return st;
    if (act_seq_kvlen) {
        if ((st = read_prefix(act_seq_kvlen, batch, "actual_seq_kvlen", kvlen)) != NSA_OK) return st;
    } else {
        kvlen = qlen;
    }
    if ((st = read_prefix(act_cmp_seq_kvlen, batch, "actual_cmp_seq_kvlen", clen)) != NSA_OK) return st;
    if ((st = read_prefix(act_sel_seq_kvlen, batch, "actual_sel_seq_kvlen", slen)) != NSA_OK) return st;
    int64_t S_max = 0;
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t T = kvlen[(size_t)b];
        if (T < qlen[(size_t)b])
            return fail(NSA_ERR_SHAPE, "sequence %lld: %lld query tokens but only %lld key/value tokens",
                        (long long)b, (long long)qlen[(size_t)b], (long long)T);
        const int64_t nc = n_cmp_of(T, l, d);
        const int64_t ns = (T + lsel - 1) / lsel;
        if (clen[(size_t)b] != nc)
            return fail(NSA_ERR_SHAPE, "sequence %lld: compressed length %lld != floor((%lld - l)/d) + 1 = %lld",
                        (long long)b, (long long)clen[(size_t)b], (long long)T, (long long)nc);
        if (slen[(size_t)b] != ns)
            return fail(NSA_ERR_SHAPE, "sequence %lld: select length %lld != ceil(%lld / l') = %lld",
                        (long long)b, (long long)slen[(size_t)b], (long long)T, (long long)ns);
        if (ns > S_max)
            S_max = ns;
    }

    // What this build implements.
    if (!nsa::cmp_attn_supported((int)d1, (int)d2) || !nsa::slc_topk_supported((int)d1))
        return fail(NSA_ERR_UNSUPPORTED, "head dims (D1, D2) = (%lld, %lld) are not built; built: D1 in {64,128,192}, D2 in {64,128}, D2 <= D1",
                    (long long)d1, (long long)d2);
    const int64_t G = head_num / kv_head_num;
    const int log2gp = nsa::topk_log2_gp((int)G);
    if (log2gp < 0)
        return fail(NSA_ERR_UNSUPPORTED, "N1/N2 = %lld > 64 query heads per KV head is not built", (long long)G);
    if (S_max > 64 * nsa::kTopkMaxNpl)
        return fail(NSA_ERR_UNSUPPORTED, "%lld select blocks in one sequence; at most %d are built",
                    (long long)S_max, 64 * nsa::kTopkMaxNpl);
    const int R = (int)(lsel / d);
    const int H = R + (int)(l / d) - 2;
    if (H + 1 > 16 || H >= nsa::kKeyTileMin)
        return fail(NSA_ERR_UNSUPPORTED, "remap stencil of %d taps is not built", H + 1);
    const int sb = (int)(((S_max + 63) / 64) * 64 > 0 ? ((S_max + 63) / 64) * 64 : 64);
    // Largest workgroup whose LDS lets two workgroups share a CU; K double
    // buffered when that still fits.
    int waves = 4, kbufs = 2;
    size_t lds = nsa::topk_lds_bytes((int)d1, log2gp, waves, sb, kbufs);
    while (lds > 80 * 1024 && (waves > 1 || kbufs > 1)) {
        if (kbufs == 2)
            kbufs = 1;
        else {
            waves >>= 1;
            kbufs = 2;
        }
        lds = nsa::topk_lds_bytes((int)d1, log2gp, waves, sb, kbufs);
    }
    if (lds > 160 * 1024)
        return fail(NSA_ERR_UNSUPPORTED, "importance scores of %lld select blocks x %d tokens do not fit in LDS",
                    (long long)S_max, 64 >> log2gp);

    nsa_plan_s* plan = new (std::nothrow) nsa_plan_s();
    if (!plan)
        return fail(NSA_ERR_WORKSPACE, "out of host memory");
    plan->B = batch;
    plan->N1 = head_num;
    plan->N2 = kv_head_num;
    plan->D1 = d1;
    plan->D2 = d2;
    plan->l = l;
    plan->d = d;
    plan->lsel = lsel;
    plan->count = count;
    plan->scale = scale_value;
    plan->dtype = (int)dtype;
    plan->S_max = S_max;
    plan->log2gp = log2gp;
    plan->topk_waves = waves;
    plan->topk_kbufs = kbufs;
    plan->sb = sb;
    plan->topk_lds = lds;
    plan->table.assign((size_t)batch + 1, nsa::BatchEnt{});
    int64_t q_off = 0, kv_off = 0, c_off = 0, ta = 0, tc = 0, ts = 0, tk = 0, S_total = 0, T_max = 0, ncmp_max = 0;
    const int64_t rows_c = (int64_t)waves * 64;
    const int64_t rows_a = nsa::cmp_attn_rows_per_wg((int)d1, (int)d2);
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t T = qlen[(size_t)b];
        nsa::BatchEnt& e = plan->table[(size_t)b];
        std::memset(&e, 0, sizeof e);
        e.q_off = (int32_t)q_off;
        e.T = (int32_t)T;
        e.pos_off = (int32_t)(kvlen[(size_t)b] - T);
        e.kv_off = (int32_t)kv_off;
        kv_off += kvlen[(size_t)b];
        if (e.pos_off > 0)
            plan->chunked = true;
        e.cmp_off = (int32_t)c_off;
        e.n_cmp = (int32_t)clen[(size_t)b];
        e.n_rb_a = (int32_t)((T * G + rows_a - 1) / rows_a);
        e.tile_off_a = (int32_t)ta;
        e.n_rb_c = (int32_t)((T * (1 << log2gp) + rows_c - 1) / rows_c);
        e.tile_off_c = (int32_t)tc;
        e.S_sel = (int32_t)slen[(size_t)b];
        e.n_rb_s = (int32_t)((T * G + nsa::kSelRows - 1) / nsa::kSelRows);
        e.tile_off_s = (int32_t)ts;
        ts += (int64_t)e.n_rb_s * kv_head_num;
        e.tile_off_k = (int32_t)tk;
        tk += (clen[(size_t)b] + nsa::kBwdKeyBlock - 1) / nsa::kBwdKeyBlock * kv_head_num;
        ta += (int64_t)e.n_rb_a * kv_head_num;
        tc += (int64_t)e.n_rb_c * kv_head_num;
        q_off += T;
        c_off += clen[(size_t)b];
        S_total += slen[(size_t)b];
        T_max = std::max(T_max, T);
        ncmp_max = std::max(ncmp_max, clen[(size_t)b]);
    }
    if (ta > INT32_MAX || tc > INT32_MAX || ts > INT32_MAX || tk > INT32_MAX || kv_off > INT32_MAX ||
        q_off * head_num * 8 > ((int64_t)1 << 62)) {
        delete plan;
        return fail(NSA_ERR_UNSUPPORTED, "problem too large for one launch");
    }
    plan->T1 = q_off;
    plan->T_kv = kv_off;
    plan->rows_c = (int)rows_c;
    plan->T2 = c_off;
    plan->S_total = S_total;
    plan->tiles_a = ta;
    plan->tiles_c = tc;
    plan->tiles_s = ts;
    plan->tiles_k = tk;
    plan->table_bytes = ((size_t)(batch + 1) * sizeof(nsa::BatchEnt) + 255) / 256 * 256;
    plan->bias_off = plan->table_bytes;
    plan->ws_bytes = plan->bias_off + ((size_t)q_off * (size_t)head_num * 4 + 255) / 256 * 256;
    plan->T_max = T_max;
    plan->ncmp_max = ncmp_max;
    plan->vis_words = std::max<int64_t>(1, (ncmp_max + 31) / 32);
    plan->cand_words = std::max<int64_t>(1, (S_max + 31) / 32);
    const size_t vis_bytes = ((size_t)T_max * (size_t)plan->vis_words * 4 + 255) / 256 * 256;
    const size_t cand_bytes = ((size_t)T_max * (size_t)plan->cand_words * 4 + 255) / 256 * 256;
    const size_t span_bytes = ((size_t)T_max * 16 + 255) / 256 * 256;
    plan->ws_masked_bytes = plan->ws_bytes + vis_bytes + cand_bytes + span_bytes;
    bwd_counts(plan);
    if (plan->bwd_items > INT32_MAX || plan->bwd_slots > INT32_MAX) {
        delete plan;
        return fail(NSA_ERR_UNSUPPORTED, "problem too large for one launch");
    }
    plan->ws_bwd_bytes = bwd_layout(plan).bytes;
    *workspace_bytes = plan->ws_bytes;
    *plan_out = plan;
    return ok();
}

nsa_status nsa_compress_attention_get_workspace(
    int64_t batch, const int64_t* act_seq_qlen, const int64_t* act_cmp_seq_kvlen,
    const int64_t* act_sel_seq_kvlen, int64_t head_num, int64_t kv_head_num, int64_t d1,
    int64_t d2, float scale_value, int64_t l, int64_t d, int64_t lsel, int64_t count,
    nsa_dtype dtype, size_t* workspace_bytes, nsa_plan* plan_out)
{
    return make_plan(batch, act_seq_qlen, nullptr, act_cmp_seq_kvlen, act_sel_seq_kvlen, head_num, kv_head_num,
                     d1, d2, scale_value, l, d, lsel, count, dtype, workspace_bytes, plan_out);
}

nsa_status nsa_compress_attention_get_workspace_kv(
    int64_t batch, const int64_t* act_seq_qlen, const int64_t* act_seq_kvlen,
    const int64_t* act_cmp_seq_kvlen, const int64_t* act_sel_seq_kvlen, int64_t head_num,
    int64_t kv_head_num, int64_t d1, int64_t d2, float scale_value, int64_t l, int64_t d,
    int64_t lsel, int64_t count, nsa_dtype dtype, size_t* workspace_bytes, nsa_plan* plan_out)
{
    if (!act_seq_kvlen) {
        if (plan_out)
            *plan_out = nullptr;
        return fail(NSA_ERR_NULLPTR, "actual_seq_kvlen must not be NULL");
    }
    return make_plan(batch, act_seq_qlen, act_seq_kvlen, act_cmp_seq_kvlen, act_sel_seq_kvlen, head_num,
                     kv_head_num, d1, d2, scale_value, l, d, lsel, count, dtype, workspace_bytes, plan_out);
}

nsa_status nsa_plan_get_info(nsa_plan plan, nsa_plan_info* info)
{
    if (!plan || !info)
        return fail(NSA_ERR_NULLPTR, "plan and info must not be NULL");
    info->batch = plan->B;
    info->total_q_tokens = plan->T1;
    info->total_cmp_tokens = plan->T2;
    info->total_sel_blocks = plan->S_total;
    info->max_sel_blocks = plan->S_max;
    info->head_num = plan->N1;
    info->kv_head_num = plan->N2;
    info->d1 = plan->D1;
    info->d2 = plan->D2;
    info->select_block_count = plan->count;
    info->workspace_bytes = plan->ws_bytes;
    info->dtype = plan->dtype;
    info->masked_workspace_bytes = plan->ws_masked_bytes;
    info->backward_workspace_bytes = plan->ws_bwd_bytes;
    info->total_kv_tokens = plan->T_kv;
    info->device_metadata = plan->device_meta ? 1 : 0;
    info->status_offset = plan->B * (int64_t)sizeof(nsa::BatchEnt);
    return ok();
}

void nsa_plan_destroy(nsa_plan plan) { delete plan; }

nsa_status nsa_compress_attention_device_plan(nsa_plan plan, nsa_plan* device_plan)
{
    if (device_plan)
        *device_plan = nullptr;
    if (!plan || !device_plan)
        return fail(NSA_ERR_NULLPTR, "plan and device_plan must not be NULL");
    nsa_plan_s* p = new (std::nothrow) nsa_plan_s(*plan);
    if (!p)
        return fail(NSA_ERR_WORKSPACE, "out of host memory");
    p->device_meta = true;
    *device_plan = p;
    return ok();
}

nsa_status nsa_compress_attention_metadata(nsa_plan device_plan, const int64_t* act_seq_qlen,
                                           const int64_t* act_seq_kvlen, const int64_t* act_cmp_seq_kvlen,
                                           const int64_t* act_sel_seq_kvlen, void* workspace,
                                           size_t workspace_bytes, void* stream)
{
    nsa_plan plan = device_plan;
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (!plan->device_meta)
        return fail(NSA_ERR_CONSTRAINT, "the plan does not read its metadata from the workspace; derive one "
                    "with nsa_compress_attention_device_plan");
    if (!act_seq_qlen || !act_cmp_seq_kvlen || !act_sel_seq_kvlen)
        return fail(NSA_ERR_NULLPTR, "the device prefix sums of query, compressed and select lengths must not be NULL");
    if (!workspace || workspace_bytes < plan->ws_bytes)
        return fail(NSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, plan->ws_bytes);
    if (!aligned(workspace, 16) || !aligned(act_seq_qlen, 8) || !aligned(act_cmp_seq_kvlen, 8) ||
        !aligned(act_sel_seq_kvlen, 8) || (act_seq_kvlen && !aligned(act_seq_kvlen, 8)))
        return fail(NSA_ERR_CONSTRAINT, "workspace must be 16-byte and the prefix sums 8-byte aligned");
    nsa::MetaParams m;
    std::memset(&m, 0, sizeof m);
    m.qlen = act_seq_qlen;
    m.kvlen = act_seq_kvlen;
    m.cmplen = act_cmp_seq_kvlen;
    m.sellen = act_sel_seq_kvlen;
    m.table = (nsa::BatchEnt*)workspace;
    m.status = (int*)((char*)workspace + plan->B * (int64_t)sizeof(nsa::BatchEnt));
    m.B = (int)plan->B;
    m.l = (int)plan->l;
    m.d = (int)plan->d;
    m.lsel = (int)plan->lsel;
    m.N2 = (int)plan->N2;
    m.G = (int)(plan->N1 / plan->N2);
    m.GP = 1 << plan->log2gp;
    m.rows_a = nsa::cmp_attn_rows_per_wg((int)plan->D1, (int)plan->D2);
    m.rows_c = plan->rows_c;
    m.rows_s = nsa::kSelRows;
    m.T_max = plan->T_max;
    m.ncmp_max = plan->ncmp_max;
    m.S_max = plan->S_max;
    m.T1 = plan->T1;
    m.T2 = plan->T2;
    m.Tkv_total = plan->T_kv;
    m.S_total = plan->S_total;
    m.tiles_a = plan->tiles_a;
    m.tiles_c = plan->tiles_c;
    m.tiles_s = plan->tiles_s;
    m.tiles_k = plan->tiles_k;
    hipError_t e = nsa::launch_meta_table(m, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "metadata launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

// `need`: the workspace bytes the call reads and writes (default: the plan's
// workspace size).
nsa_status check_exec(nsa_plan plan, void* workspace, size_t workspace_bytes,
                      std::initializer_list<const void*> a16, std::initializer_list<const void*> a4,
                      size_t need = SIZE_MAX)
{
    if (need == SIZE_MAX)
        need = plan->ws_bytes;
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(NSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
    for (const void* ptr : a16)
        if (ptr && !aligned(ptr, 16))
            return fail(NSA_ERR_CONSTRAINT, "tensors and workspace must be 16-byte aligned");
    for (const void* ptr : a4)
        if (ptr && !aligned(ptr, 4))
            return fail(NSA_ERR_CONSTRAINT, "topk_indices and p_slc_debug must be 4-byte aligned");
    return NSA_OK;
}

// The table (and its zero status word) into the workspace, unless the plan
// is device-planned: then nsa_compress_attention_metadata wrote both there.
nsa_status upload_table(nsa_plan plan, void* workspace, hipStream_t s)
{
    if (plan->device_meta)
        return NSA_OK;
    hipError_t e = hipMemcpyAsync(workspace, plan->table.data(), plan->table.size() * sizeof(nsa::BatchEnt),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "workspace upload failed: %s", hipGetErrorString(e));
    return NSA_OK;
}

const int* status_word(nsa_plan plan, const void* workspace)
{
    return (const int*)((const char*)workspace + plan->B * (int64_t)sizeof(nsa::BatchEnt));
}

// The [T1, N1] array of per-row biases (base-2 log-normalisers) that every
// forward call writes into its workspace and the importance pass may read
// instead of the two [T1, N1, 8] statistics.
float* ws_bias(nsa_plan plan, void* workspace) { return (float*)((char*)workspace + plan->bias_off); }

// Where the importance pass takes its row statistics from: softmax_max and
// softmax_sum when both are given, the bias array the forward call left in
// the workspace when both are NULL.
nsa_status select_stats(nsa_plan plan, const float* softmax_max, const float* softmax_sum, void* workspace,
                        const float** bias)
{
    *bias = nullptr;
    if ((softmax_max == nullptr) != (softmax_sum == nullptr))
        return fail(NSA_ERR_NULLPTR, "softmax_max and softmax_sum must both be given, or both be NULL "
                    "(then the forward call's statistics in the workspace are read)");
    if (softmax_max == nullptr)
        *bias = ws_bias(plan, workspace);
    return NSA_OK;
}

float exp2_scale(const nsa_plan_s* plan) { return std::fabs(plan->scale) * 1.4426950408889634f; }

// Magic numbers for division by G (round-up method): s = ceil(log2 G),
// m = floor(2^32 (2^s - G) / G) + 1; then n / G = (umulhi(n, m) + n) >> s
// for 0 <= n < 2^31.
void g_magic(int G, uint32_t* m, uint32_t* s)
{
    uint32_t sh = 0;
    while (((uint64_t)1 << sh) < (uint64_t)G)
        ++sh;
    *s = sh;
    *m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << sh) - (uint64_t)G)) / (uint64_t)G + 1);
}
uint32_t q_sign(const nsa_plan_s* plan) { return plan->scale < 0.f ? 0x80008000u : 0u; }

nsa::AttnParams fwd_params(nsa_plan plan, const void* query, const void* key, const void* value,
                           void* attention_out, float* softmax_max, float* softmax_sum, void* workspace,
                           bool write_bias = true)
{
    const float abs_scale = std::fabs(plan->scale);
    const float c = exp2_scale(plan);
    nsa::AttnParams a;
    std::memset(&a, 0, sizeof a);
    a.q = (const uint16_t*)query;
    a.kc = (const uint16_t*)key;
    a.vc = (const uint16_t*)value;
    a.out = (uint16_t*)attention_out;
    a.smax = softmax_max;
    a.ssum = softmax_sum;
    a.bias = write_bias ? ws_bias(plan, workspace) : nullptr;
    a.bt = (const nsa::BatchEnt*)workspace;
    a.status = status_word(plan, workspace);
    a.B = (int)plan->B;
    a.N1 = (int)plan->N1;
    a.N2 = (int)plan->N2;
    a.G = (int)(plan->N1 / plan->N2);
    a.l = (int)plan->l;
    a.d = (int)plan->d;
    // A positive exponent scale keeps exp2(-inf * c) = 0 for masked scores
    // (a zero scale makes every score 0: any tiny c gives the same P = 1).
    a.c = std::fmax(c, 1e-30f);
    a.abs_scale = abs_scale;
    // the running max moves only when a score beats it by more than 8 in base 2
    a.thr = std::fmin(8.0f / a.c, 3.0e38f);
    a.qsign = q_sign(plan);
    a.vis_words = (int)plan->vis_words;
    return a;
}

nsa_status launch_fwd(nsa_plan plan, const void* query, const void* key, const void* value,
                      void* attention_out, float* softmax_max, float* softmax_sum, void* workspace,
                      hipStream_t s, const uint32_t* vis = nullptr, const int4* vis_span = nullptr,
                      bool write_bias = true)
{
    nsa::AttnParams a = fwd_params(plan, query, key, value, attention_out, softmax_max, softmax_sum, workspace,
                                   write_bias);
    a.vis = vis;
    a.vis_span = vis_span;
    hipError_t e = nsa::launch_cmp_attn(plan->dtype, (int)plan->D1, (int)plan->D2, a, (int)plan->tiles_a, s);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
    return NSA_OK;
}

// Counts of a split attention launch with pieces of at most C key tiles:
// the attention kernel's row blocks in its own order (per sequence and KV
// head, costliest first); a row block with n > C key tiles becomes
// ceil(n / C) pieces, each with a partial slot, plus one combine item.  The
// list itself is built on the device from the table (launch_split_plan);
// these host counts size the workspace and the launches, and
// the device checks its list against them.
struct SplitCounts {
    int64_t items = 0, combs = 0, slots = 0;
    size_t chunk_off = 0, items_off = 0, combs_off = 0, part_off = 0, bytes = 0;
};

SplitCounts split_counts(const nsa_plan_s* plan, int64_t C)
{
    constexpr int KT = nsa::kKeyTileMin;   // key tile of the attention kernel
    const int64_t rows_a = nsa::cmp_attn_rows_per_wg((int)plan->D1, (int)plan->D2);
    const int64_t G = plan->N1 / plan->N2;
    SplitCounts k;
    for (int64_t b = 0; b < plan->B; ++b) {
        const nsa::BatchEnt& e = plan->table[(size_t)b];
        for (int64_t rb = 0; rb < e.n_rb_a; ++rb) {
            const int64_t last_row = std::min<int64_t>((rb + 1) * rows_a, (int64_t)e.T * G) - 1;
            const int64_t t = last_row / G + e.pos_off;
            const int64_t nv = t < plan->l - 1 ? 0 : std::min<int64_t>((t - plan->l + 1) / plan->d + 1, e.n_cmp);
            const int64_t n_kt = (nv + KT - 1) / KT;
            const int64_t pieces = n_kt > C ? (n_kt + C - 1) / C : 1;
            k.items += pieces * plan->N2;
            if (n_kt > C) {
                k.combs += plan->N2;
                k.slots += pieces * plan->N2;
            }
        }
    }
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    k.chunk_off = plan->ws_bytes;
    k.items_off = k.chunk_off + up((size_t)nsa::plan_chunks(plan->tiles_a) * sizeof(int4));
    k.combs_off = k.items_off + up((size_t)k.items * sizeof(nsa::SplitItem));
    k.part_off = k.combs_off + up((size_t)k.combs * sizeof(nsa::CombineItem));
    k.bytes = k.part_off + (size_t)k.slots * (size_t)rows_a * (size_t)(plan->D2 + 4) * 4;
    return k;
}

nsa_status launch_select(nsa_plan plan, const void* query, const void* key, const float* softmax_max,
                         const float* softmax_sum, const float* bias, int32_t* topk_indices, float* p_slc_debug,
                         void* workspace, hipStream_t s, const uint32_t* vis = nullptr,
                         const int4* vis_span = nullptr, const uint32_t* cand = nullptr)
{
    nsa::TopkParams t;
    std::memset(&t, 0, sizeof t);
    t.q = (const uint16_t*)query;
    t.kc = (const uint16_t*)key;
    t.smax = softmax_max;
    t.ssum = softmax_sum;
    t.bias = bias;
    t.topk = topk_indices;
    t.pslc = p_slc_debug;
    t.bt = (const nsa::BatchEnt*)workspace;
    t.status = status_word(plan, workspace);
    t.B = (int)plan->B;
    t.N1 = (int)plan->N1;
    t.N2 = (int)plan->N2;
    t.G = (int)(plan->N1 / plan->N2);
    t.l = (int)plan->l;
    t.d = (int)plan->d;
    t.lsel = (int)plan->lsel;
    t.count = (int)plan->count;
    t.R = (int)(plan->lsel / plan->d);
    const int L2 = (int)(plan->l / plan->d);
    t.H = t.R + L2 - 2;
    // P_slc[j] = sum_m sum_n P[R*j - m - n]: entry R*j - r is counted once per
    // pair (m, n) with m + n = r, 0 <= m < R, 0 <= n < L2.
    for (int r = 0; r <= t.H; ++r) {
        int cnt = 0;
        for (int m = 0; m < t.R; ++m)
            if (r - m >= 0 && r - m < L2)
                ++cnt;
        t.coef[r] = (float)cnt;
    }
    t.c = exp2_scale(plan);
    t.qsign = q_sign(plan);
    t.s_stride = (int)plan->S_max;
    t.sb = plan->sb;
    t.nj_slots = (nsa::topk_key_tile((int)plan->D1) + t.R - 1) / t.R;
    t.npl = plan->sb / 64;
    t.waves = plan->topk_waves;
    t.kbufs = plan->topk_kbufs;
    t.vis = vis;
    t.vis_span = vis_span;
    t.vis_words = (int)plan->vis_words;
    t.cand = cand;
    t.cand_words = (int)plan->cand_words;
    hipError_t e = nsa::launch_slc_topk(plan->dtype, (int)plan->D1, plan->log2gp, t, (int)plan->tiles_c, plan->topk_lds, s);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "top-k launch failed: %s", hipGetErrorString(e));
    return NSA_OK;
}

// Validates the masks a call uses and packs them into the workspace after
// the sequence table: *vis / *cand point at the packed rows, or stay NULL
// where the positional rule applies.
nsa_status prepare_masks(nsa_plan plan, const nsa_masks* masks, bool use_atten, bool use_topk,
                         void* workspace, size_t workspace_bytes, hipStream_t s,
                         const uint32_t** vis, const int4** vis_span, const uint32_t** cand)
{
    *vis = nullptr;
    *vis_span = nullptr;
    *cand = nullptr;
    if (!masks)
        return NSA_OK;
    const bool a = use_atten && masks->atten_mask;
    const bool t = use_topk && masks->topk_mask;
    if (a && (masks->atten_rows < plan->T_max || masks->atten_cols < plan->ncmp_max))
        return fail(NSA_ERR_SHAPE, "atten_mask is [%lld, %lld]; it needs at least [%lld, %lld] "
                    "(longest sequence, most compressed entries)", (long long)masks->atten_rows,
                    (long long)masks->atten_cols, (long long)plan->T_max, (long long)plan->ncmp_max);
    if (t && (masks->topk_rows < plan->T_max || masks->topk_cols < plan->S_max))
        return fail(NSA_ERR_SHAPE, "topk_mask is [%lld, %lld]; it needs at least [%lld, %lld] "
                    "(longest sequence, most select blocks)", (long long)masks->topk_rows,
                    (long long)masks->topk_cols, (long long)plan->T_max, (long long)plan->S_max);
    if (!a && !t)
        return NSA_OK;
    if (workspace_bytes < plan->ws_masked_bytes)
        return fail(NSA_ERR_WORKSPACE, "calls with masks need %zu workspace bytes, %zu given",
                    plan->ws_masked_bytes, workspace_bytes);
    uint32_t* vis_ws = (uint32_t*)((char*)workspace + plan->ws_bytes);
    uint32_t* cand_ws = vis_ws + ((size_t)plan->T_max * (size_t)plan->vis_words * 4 + 255) / 256 * 64;
    int4* span_ws = (int4*)(cand_ws + ((size_t)plan->T_max * (size_t)plan->cand_words * 4 + 255) / 256 * 64);
    if (a) {
        nsa::MaskPackParams mp{(const uint8_t*)masks->atten_mask, masks->atten_cols, vis_ws,
                               (int)plan->T_max, (int)plan->vis_words, span_ws};
        hipError_t e = nsa::launch_pack_mask(mp, s);
        if (e != hipSuccess)
            return fail(NSA_ERR_HIP, "mask packing failed: %s", hipGetErrorString(e));
        *vis = vis_ws;
        *vis_span = span_ws;
    }
    if (t) {
        nsa::MaskPackParams mp{(const uint8_t*)masks->topk_mask, masks->topk_cols, cand_ws,
                               (int)plan->T_max, (int)plan->cand_words, nullptr};
        hipError_t e = nsa::launch_pack_mask(mp, s);
        if (e != hipSuccess)
            return fail(NSA_ERR_HIP, "mask packing failed: %s", hipGetErrorString(e));
        *cand = cand_ws;
    }
    return NSA_OK;
}

}  // namespace

extern "C" {

nsa_status nsa_compress_attention_fwd(nsa_plan plan, const void* query, const void* key,
                                      const void* value, void* attention_out, float* softmax_max,
                                      float* softmax_sum, void* workspace, size_t workspace_bytes,
                                      void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->T1 > 0 && (!query || !attention_out || !softmax_max || !softmax_sum))
        return fail(NSA_ERR_NULLPTR, "query and the three outputs must not be NULL");
    if (plan->T2 > 0 && (!key || !value))
        return fail(NSA_ERR_NULLPTR, "key and value must not be NULL");
    nsa_status st = check_exec(plan, workspace, workspace_bytes,
                               {query, key, value, attention_out, softmax_max, softmax_sum, workspace}, {});
    if (st != NSA_OK || plan->T1 == 0)
        return st == NSA_OK ? ok() : st;
    hipStream_t s = (hipStream_t)stream;
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    if ((st = launch_fwd(plan, query, key, value, attention_out, softmax_max, softmax_sum, workspace, s)) != NSA_OK)
        return st;
    return ok();
}

nsa_status nsa_compress_attention_split_workspace(nsa_plan plan, int64_t key_tiles_per_piece,
                                                  size_t* workspace_bytes)
{
    if (!plan || !workspace_bytes)
        return fail(NSA_ERR_NULLPTR, "plan and workspace_bytes must not be NULL");
    if (key_tiles_per_piece < 1 || key_tiles_per_piece > (1 << 20))
        return fail(NSA_ERR_CONSTRAINT, "key_tiles_per_piece must be in [1, 2^20], got %lld",
                    (long long)key_tiles_per_piece);
    const SplitCounts k = split_counts(plan, key_tiles_per_piece);
    if (k.items > INT32_MAX || k.slots > INT32_MAX)
        return fail(NSA_ERR_UNSUPPORTED, "problem too large for one launch");
    *workspace_bytes = k.bytes;
    return ok();
}

nsa_status nsa_compress_attention_fwd_split(nsa_plan plan, const void* query, const void* key,
                                            const void* value, void* attention_out, float* softmax_max,
                                            float* softmax_sum, int64_t key_tiles_per_piece,
                                            void* workspace, size_t workspace_bytes, void* stream)
{
    size_t need = 0;
    nsa_status st = nsa_compress_attention_split_workspace(plan, key_tiles_per_piece, &need);
    if (st != NSA_OK)
        return st;
    if (plan->T1 > 0 && (!query || !attention_out || !softmax_max || !softmax_sum))
        return fail(NSA_ERR_NULLPTR, "query and the three outputs must not be NULL");
    if (plan->T2 > 0 && (!key || !value))
        return fail(NSA_ERR_NULLPTR, "key and value must not be NULL");
    if (workspace_bytes < need || !workspace)
        return fail(NSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
    if ((st = check_exec(plan, workspace, workspace_bytes,
                         {query, key, value, attention_out, softmax_max, softmax_sum, workspace}, {})) != NSA_OK)
        return st;
    if (plan->T1 == 0)
        return ok();
    const SplitCounts k = split_counts(plan, key_tiles_per_piece);
    hipStream_t s = (hipStream_t)stream;
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    char* ws = (char*)workspace;
    nsa::SplitPlanParams sp;
    std::memset(&sp, 0, sizeof sp);
    sp.table = (const nsa::BatchEnt*)workspace;
    sp.status = (int*)status_word(plan, workspace);
    sp.chunk_tot = (int4*)(ws + k.chunk_off);
    sp.items = (nsa::SplitItem*)(ws + k.items_off);
    sp.combs = (nsa::CombineItem*)(ws + k.combs_off);
    sp.B = (int)plan->B;
    sp.N2 = (int)plan->N2;
    sp.G = (int)(plan->N1 / plan->N2);
    sp.l = (int)plan->l;
    sp.d = (int)plan->d;
    sp.rows_a = nsa::cmp_attn_rows_per_wg((int)plan->D1, (int)plan->D2);
    sp.C = (int)key_tiles_per_piece;
    sp.tiles_a = (int)plan->tiles_a;
    sp.n_items = k.items;
    sp.n_combs = k.combs;
    sp.n_slots = k.slots;
    hipError_t e = nsa::launch_split_plan(sp, s);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "split work list launch failed: %s", hipGetErrorString(e));
    nsa::AttnParams a = fwd_params(plan, query, key, value, attention_out, softmax_max, softmax_sum, workspace);
    a.split = sp.items;
    a.part = (float*)(ws + k.part_off);
    e = nsa::launch_cmp_attn(plan->dtype, (int)plan->D1, (int)plan->D2, a, (int)k.items, s);
    if (e == hipSuccess)
        e = nsa::launch_attn_combine(plan->dtype, (int)plan->D1, (int)plan->D2, a, sp.combs, (int)k.combs, s);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "split attention launch failed: %s", hipGetErrorString(e));
    return ok();
}

nsa_status nsa_compress_attention_select(nsa_plan plan, const void* query, const void* key,
                                         const float* softmax_max, const float* softmax_sum,
                                         int32_t* topk_indices, float* p_slc_debug,
                                         void* workspace, size_t workspace_bytes, void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->T1 > 0 && (!query || !topk_indices))
        return fail(NSA_ERR_NULLPTR, "query and topk_indices must not be NULL");
    if (plan->T2 > 0 && !key)
        return fail(NSA_ERR_NULLPTR, "key must not be NULL");
    nsa_status st = check_exec(plan, workspace, workspace_bytes, {query, key, softmax_max, softmax_sum, workspace},
                               {topk_indices, p_slc_debug});
    if (st != NSA_OK || plan->T1 == 0)
        return st == NSA_OK ? ok() : st;
    const float* bias = nullptr;
    if ((st = select_stats(plan, softmax_max, softmax_sum, workspace, &bias)) != NSA_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    if ((st = launch_select(plan, query, key, softmax_max, softmax_sum, bias, topk_indices, p_slc_debug, workspace,
                            s)) != NSA_OK)
        return st;
    return ok();
}

nsa_status nsa_compress_attention(nsa_plan plan, const void* query, const void* key,
                                  const void* value, void* attention_out, int32_t* topk_indices,
                                  float* softmax_max, float* softmax_sum, float* p_slc_debug,
                                  void* workspace, size_t workspace_bytes, void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->T1 > 0 && (!query || !attention_out || !topk_indices || !softmax_max || !softmax_sum))
        return fail(NSA_ERR_NULLPTR, "query and the four outputs must not be NULL");
    if (plan->T2 > 0 && (!key || !value))
        return fail(NSA_ERR_NULLPTR, "key and value must not be NULL");
    nsa_status st = check_exec(plan, workspace, workspace_bytes,
                               {query, key, value, attention_out, softmax_max, softmax_sum, workspace},
                               {topk_indices, p_slc_debug});
    if (st != NSA_OK || plan->T1 == 0)
        return st == NSA_OK ? ok() : st;
    hipStream_t s = (hipStream_t)stream;
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    if ((st = launch_fwd(plan, query, key, value, attention_out, softmax_max, softmax_sum, workspace, s)) != NSA_OK)
        return st;
    if ((st = launch_select(plan, query, key, softmax_max, softmax_sum, ws_bias(plan, workspace), topk_indices,
                            p_slc_debug, workspace, s)) != NSA_OK)
        return st;
    return ok();
}

}  // extern "C"

// ---- the entry point that allocates nothing -----------------------------------
// Its scratch (the per-sequence table, the only device memory beyond inputs
// and outputs that the two kernels of nsa_compress_attention read) is a
// file-scope device array.  Host code never passes the array's name to a
// kernel or a copy: each device's own address comes from
// hipGetSymbolAddress, resolved once per device with that device current.
namespace {

constexpr int kNoAllocMaxBatch = 1024;   // sequences the scratch table holds (64 KiB)
constexpr int kMaxDevices = 64;

// The table of up to 1024 sequences, then the entry that carries its status
// word, rounded up to 256 bytes (the size a plan's table occupies).
__device__ __align__(256) nsa::BatchEnt scratch[kNoAllocMaxBatch + 4];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The scratch address on the current device (NULL with the detail set on failure).
nsa_status scratch_on_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(NSA_ERR_UNSUPPORTED, "device %d: at most %d devices are supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(NSA_ERR_HIP, "hipGetSymbolAddress of the scratch table failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return NSA_OK;
}

}  // namespace

extern "C" {

nsa_status nsa_compress_attention_noalloc(nsa_plan plan, const void* query, const void* key,
                                          const void* value, void* attention_out, int32_t* topk_indices,
                                          float* softmax_max, float* softmax_sum, float* p_slc_debug,
                                          void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->device_meta)
        return fail(NSA_ERR_CONSTRAINT, "a device-planned plan reads its table from a workspace; the "
                    "no-allocation entry point takes a plan from nsa_compress_attention_get_workspace(_kv)");
    if (plan->B > kNoAllocMaxBatch)
        return fail(NSA_ERR_UNSUPPORTED, "the no-allocation entry point holds at most %d sequences in its static "
                    "scratch (plan has %lld); use nsa_compress_attention with a workspace", kNoAllocMaxBatch,
                    (long long)plan->B);
    if (plan->T1 > 0 && (!query || !attention_out || !topk_indices || !softmax_max || !softmax_sum))
        return fail(NSA_ERR_NULLPTR, "query and the four outputs must not be NULL");
    if (plan->T2 > 0 && (!key || !value))
        return fail(NSA_ERR_NULLPTR, "key and value must not be NULL");
    void* ws = nullptr;
    nsa_status st = scratch_on_current_device(&ws);
    if (st != NSA_OK)
        return st;
    const size_t ws_bytes = sizeof(nsa::BatchEnt) * (kNoAllocMaxBatch + 4);
    if ((st = check_exec(plan, ws, ws_bytes, {query, key, value, attention_out, softmax_max, softmax_sum},
                         {topk_indices, p_slc_debug}, plan->table_bytes)) != NSA_OK)
        return st;
    if (plan->T1 == 0)
        return ok();
    hipStream_t s = (hipStream_t)stream;
    if ((st = upload_table(plan, ws, s)) != NSA_OK)
        return st;
    // The scratch holds the table only: the importance pass reads the row
    // statistics from softmax_max / softmax_sum.
    if ((st = launch_fwd(plan, query, key, value, attention_out, softmax_max, softmax_sum, ws, s, nullptr, nullptr,
                         false)) != NSA_OK)
        return st;
    if ((st = launch_select(plan, query, key, softmax_max, softmax_sum, nullptr, topk_indices, p_slc_debug, ws,
                            s)) != NSA_OK)
        return st;
    return ok();
}

nsa_status nsa_compress_attention_fwd_masked(nsa_plan plan, const void* query, const void* key,
                                             const void* value, const nsa_masks* masks,
                                             void* attention_out, float* softmax_max,
                                             float* softmax_sum, void* workspace,
                                             size_t workspace_bytes, void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->T1 > 0 && (!query || !attention_out || !softmax_max || !softmax_sum))
        return fail(NSA_ERR_NULLPTR, "query and the three outputs must not be NULL");
    if (plan->T2 > 0 && (!key || !value))
        return fail(NSA_ERR_NULLPTR, "key and value must not be NULL");
    nsa_status st = check_exec(plan, workspace, workspace_bytes,
                               {query, key, value, attention_out, softmax_max, softmax_sum, workspace}, {});
    if (st != NSA_OK || plan->T1 == 0)
        return st == NSA_OK ? ok() : st;
    hipStream_t s = (hipStream_t)stream;
    const uint32_t *vis = nullptr, *cand = nullptr;
    const int4* span = nullptr;
    if ((st = prepare_masks(plan, masks, true, false, workspace, workspace_bytes, s, &vis, &span, &cand)) != NSA_OK)
        return st;
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    if ((st = launch_fwd(plan, query, key, value, attention_out, softmax_max, softmax_sum, workspace, s,
                         vis, span)) != NSA_OK)
        return st;
    return ok();
}

nsa_status nsa_compress_attention_select_masked(nsa_plan plan, const void* query, const void* key,
                                                const nsa_masks* masks, const float* softmax_max,
                                                const float* softmax_sum, int32_t* topk_indices,
                                                float* p_slc_debug, void* workspace,
                                                size_t workspace_bytes, void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->T1 > 0 && (!query || !topk_indices))
        return fail(NSA_ERR_NULLPTR, "query and topk_indices must not be NULL");
    if (plan->T2 > 0 && !key)
        return fail(NSA_ERR_NULLPTR, "key must not be NULL");
    nsa_status st = check_exec(plan, workspace, workspace_bytes, {query, key, softmax_max, softmax_sum, workspace},
                               {topk_indices, p_slc_debug});
    if (st != NSA_OK || plan->T1 == 0)
        return st == NSA_OK ? ok() : st;
    const float* bias = nullptr;
    if ((st = select_stats(plan, softmax_max, softmax_sum, workspace, &bias)) != NSA_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const uint32_t *vis = nullptr, *cand = nullptr;
    const int4* span = nullptr;
    if ((st = prepare_masks(plan, masks, true, true, workspace, workspace_bytes, s, &vis, &span, &cand)) != NSA_OK)
        return st;
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    if ((st = launch_select(plan, query, key, softmax_max, softmax_sum, bias, topk_indices, p_slc_debug, workspace,
                            s, vis, span, cand)) != NSA_OK)
        return st;
    return ok();
}

nsa_status nsa_compress_attention_masked(nsa_plan plan, const void* query, const void* key,
                                         const void* value, const nsa_masks* masks,
                                         void* attention_out, int32_t* topk_indices,
                                         float* softmax_max, float* softmax_sum, float* p_slc_debug,
                                         void* workspace, size_t workspace_bytes, void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->T1 > 0 && (!query || !attention_out || !topk_indices || !softmax_max || !softmax_sum))
        return fail(NSA_ERR_NULLPTR, "query and the four outputs must not be NULL");
    if (plan->T2 > 0 && (!key || !value))
        return fail(NSA_ERR_NULLPTR, "key and value must not be NULL");
    nsa_status st = check_exec(plan, workspace, workspace_bytes,
                               {query, key, value, attention_out, softmax_max, softmax_sum, workspace},
                               {topk_indices, p_slc_debug});
    if (st != NSA_OK || plan->T1 == 0)
        return st == NSA_OK ? ok() : st;
    hipStream_t s = (hipStream_t)stream;
    const uint32_t *vis = nullptr, *cand = nullptr;
    const int4* span = nullptr;
    if ((st = prepare_masks(plan, masks, true, true, workspace, workspace_bytes, s, &vis, &span, &cand)) != NSA_OK)
        return st;
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    if ((st = launch_fwd(plan, query, key, value, attention_out, softmax_max, softmax_sum, workspace, s,
                         vis, span)) != NSA_OK)
        return st;
    if ((st = launch_select(plan, query, key, softmax_max, softmax_sum, ws_bias(plan, workspace), topk_indices,
                            p_slc_debug, workspace, s, vis, span, cand)) != NSA_OK)
        return st;
    return ok();
}

nsa_status nsa_select_attention(nsa_plan plan, const void* query, const void* key, const void* value,
                                const int32_t* topk_indices, void* attention_out, float* softmax_lse,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->T1 > 0 && (!query || !key || !value || !topk_indices || !attention_out || !softmax_lse))
        return fail(NSA_ERR_NULLPTR, "query, key, value, topk_indices and the outputs must not be NULL");
    if (plan->lsel % 32 != 0)
        return fail(NSA_ERR_UNSUPPORTED, "selected-block attention needs select_block_size %% 32 == 0 (got %lld)",
                    (long long)plan->lsel);
    if (!nsa::sel_attn_supported((int)plan->D1, (int)plan->D2))
        return fail(NSA_ERR_UNSUPPORTED, "head dims (%lld, %lld) are not built for selected-block attention",
                    (long long)plan->D1, (long long)plan->D2);
    nsa_status st = check_exec(plan, workspace, workspace_bytes, {query, key, value, attention_out, workspace},
                               {topk_indices, softmax_lse});
    if (st != NSA_OK || plan->T1 == 0)
        return st == NSA_OK ? ok() : st;
    hipStream_t s = (hipStream_t)stream;
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    nsa::SelParams a;
    std::memset(&a, 0, sizeof a);
    a.q = (const uint16_t*)query;
    a.k = (const uint16_t*)key;
    a.v = (const uint16_t*)value;
    a.topk = topk_indices;
    a.out = (uint16_t*)attention_out;
    a.lse = softmax_lse;
    a.bt = (const nsa::BatchEnt*)workspace;
    a.status = status_word(plan, workspace);
    a.B = (int)plan->B;
    a.N1 = (int)plan->N1;
    a.N2 = (int)plan->N2;
    a.G = (int)(plan->N1 / plan->N2);
    a.lsel = (int)plan->lsel;
    a.count = (int)plan->count;
    a.c = std::fmax(exp2_scale(plan), 1e-30f);
    a.abs_scale = std::fabs(plan->scale);
    a.thr = std::fmin(8.0f / a.c, 3.0e38f);
    a.qsign = q_sign(plan);
    a.sw = (int)std::max<int64_t>(1, (plan->S_max + 31) / 32);
    a.tpw = (nsa::kSelRows - 1) / a.G + 2;
    const size_t lds = nsa::sel_attn_lds_bytes(a.tpw, a.sw);
    hipError_t e = nsa::launch_sel_attn(plan->dtype, (int)plan->D1, (int)plan->D2, a, (int)plan->tiles_s, lds, s);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "selected-block attention launch failed: %s", hipGetErrorString(e));
    return ok();
}

nsa_status nsa_compress_attention_backward(nsa_plan plan, const void* query, const void* key,
                                          const void* value, const void* attention_out,
                                          const void* d_attention_out, const float* softmax_max,
                                          const float* softmax_sum, float* d_query, float* d_key,
                                          float* d_value, void* workspace, size_t workspace_bytes,
                                          void* stream)
{
    if (!plan)
        return fail(NSA_ERR_NULLPTR, "plan is NULL");
    if (plan->T1 > 0 && (!query || !attention_out || !d_attention_out || !softmax_max || !softmax_sum || !d_query))
        return fail(NSA_ERR_NULLPTR, "query, attention_out, its gradient, the softmax statistics and d_query must not be NULL");
    if (plan->T2 > 0 && (!key || !value || !d_key || !d_value))
        return fail(NSA_ERR_NULLPTR, "key, value, d_key and d_value must not be NULL");
    if (!nsa::attn_bwd_supported((int)plan->D1, (int)plan->D2))
        return fail(NSA_ERR_UNSUPPORTED, "head dims (%lld, %lld) are not built for the backward",
                    (long long)plan->D1, (long long)plan->D2);
    for (int64_t b = 0; b < plan->B; ++b)
        if ((int64_t)plan->table[(size_t)b].T * plan->N1 * std::max(plan->D1, plan->D2) * 2 >= ((int64_t)1 << 32) - 64)
            return fail(NSA_ERR_UNSUPPORTED, "a sequence's query rows exceed 4 GiB; the backward addresses "
                        "them with 32-bit offsets");
    if (workspace_bytes < plan->ws_bwd_bytes || !workspace)
        return fail(NSA_ERR_WORKSPACE, "the backward needs %zu workspace bytes, %zu given", plan->ws_bwd_bytes,
                    workspace_bytes);
    nsa_status st = check_exec(plan, workspace, workspace_bytes,
                               {query, key, value, attention_out, d_attention_out, softmax_max, softmax_sum,
                                d_query, d_key, d_value, workspace}, {});
    if (st != NSA_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    if (plan->T1 == 0)
        return ok();
    if ((st = upload_table(plan, workspace, s)) != NSA_OK)
        return st;
    nsa::BwdParams a;
    std::memset(&a, 0, sizeof a);
    a.q = (const uint16_t*)query;
    a.kc = (const uint16_t*)key;
    a.vc = (const uint16_t*)value;
    a.out = (const uint16_t*)attention_out;
    a.dout = (const uint16_t*)d_attention_out;
    a.smax = softmax_max;
    a.ssum = softmax_sum;
    a.dq = d_query;
    a.dkc = d_key;
    a.dvc = d_value;
    const BwdLayout lay = bwd_layout(plan);
    a.rowstat = (float*)((char*)workspace + lay.rowstat_off);
    a.items = (const nsa::BwdItem*)((char*)workspace + lay.items_off);
    a.combs = (const nsa::CombineItem*)((char*)workspace + lay.combs_off);
    a.part = (float*)((char*)workspace + lay.part_off);
    a.bt = (const nsa::BatchEnt*)workspace;
    a.status = status_word(plan, workspace);
    a.B = (int)plan->B;
    a.N1 = (int)plan->N1;
    a.N2 = (int)plan->N2;
    a.G = (int)(plan->N1 / plan->N2);
    a.l = (int)plan->l;
    a.d = (int)plan->d;
    a.c = std::fmax(exp2_scale(plan), 1e-30f);
    a.scale = plan->scale;
    a.qsign = q_sign(plan);
    g_magic(a.G, &a.gdiv_m, &a.gdiv_s);
    nsa::BwdPlanParams bp;
    std::memset(&bp, 0, sizeof bp);
    bp.table = a.bt;
    bp.status = (int*)a.status;
    bp.chunk_tot = (int4*)((char*)workspace + lay.chunk_off);
    bp.items = (nsa::BwdItem*)a.items;
    bp.combs = (nsa::CombineItem*)a.combs;
    bp.B = a.B;
    bp.N2 = a.N2;
    bp.G = a.G;
    bp.l = a.l;
    bp.d = a.d;
    bp.qmax = (int)plan->bwd_qmax;
    bp.tiles_k = (int)plan->tiles_k;
    bp.n_items = plan->bwd_items;
    bp.n_combs = plan->bwd_combs;
    bp.n_slots = plan->bwd_slots;
    hipError_t e = nsa::launch_bwd_plan(bp, s);
    if (e == hipSuccess)
        e = nsa::launch_attn_bwd(plan->dtype, (int)plan->D1, (int)plan->D2, a, (int)plan->tiles_a,
                                 (int)plan->bwd_items, (int)plan->bwd_combs, s);
    if (e != hipSuccess)
        return fail(NSA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

nsa_status nsa_compress_backward(const void* input, const void* weight, const float* d_output,
                                 const int64_t* act_seq_len, int64_t batch, int64_t total_tokens,
                                 int64_t num_heads, int64_t head_dim, int64_t l, int64_t d,
                                 nsa_dtype dtype, int64_t output_tokens, float* d_input,
                                 float* d_weight, void* stream)
{
    if (!input || !weight || !act_seq_len || !d_input || !d_weight)
        return fail(NSA_ERR_NULLPTR, "input, weight, act_seq_len, d_input and d_weight must not be NULL");
    nsa_status st = check_dtype((int)dtype);
    if (st != NSA_OK)
        return st;
    if (batch < 1)
        return fail(NSA_ERR_SHAPE, "act_seq_len must not be empty (batch = %lld)", (long long)batch);
    if (num_heads < 1)
        return fail(NSA_ERR_SHAPE, "num_heads must be >= 1");
    if (!mult16(head_dim) || head_dim > 256)
        return fail(NSA_ERR_CONSTRAINT, "head_dim must be a multiple of 16 and <= 256 (got %lld)", (long long)head_dim);
    if (!mult16(l) || l > 128)
        return fail(NSA_ERR_CONSTRAINT, "compress_block_size must be a multiple of 16 in [16, 128] (got %lld)", (long long)l);
    if (!mult16(d) || d > l)
        return fail(NSA_ERR_CONSTRAINT, "compress_stride must be a multiple of 16 with 16 <= d <= compress_block_size (got %lld)", (long long)d);
    std::vector<int64_t> lens;
    if ((st = read_prefix(act_seq_len, batch, "act_seq_len", lens)) != NSA_OK)
        return st;
    if (act_seq_len[batch - 1] != total_tokens)
        return fail(NSA_ERR_SHAPE, "last prefix sum %lld != total_tokens %lld",
                    (long long)act_seq_len[batch - 1], (long long)total_tokens);
    int64_t T2 = 0;
    for (int64_t T : lens)
        T2 += n_cmp_of(T, l, d);
    if (T2 != output_tokens)
        return fail(NSA_ERR_SHAPE, "output_tokens %lld != sum of compressed lengths %lld",
                    (long long)output_tokens, (long long)T2);
    if (T2 > 0 && !d_output)
        return fail(NSA_ERR_NULLPTR, "d_output must not be NULL");
    if (!aligned(input, 16) || !aligned(d_input, 16) || (d_output && !aligned(d_output, 16)) ||
        !aligned(weight, 2) || !aligned(d_weight, 4))
        return fail(NSA_ERR_CONSTRAINT, "input, d_output and d_input must be 16-byte aligned");
    nsa::CompressBwdParams p;
    std::memset(&p, 0, sizeof p);
    p.x = (const uint16_t*)input;
    p.w = (const uint16_t*)weight;
    p.dy = d_output;
    p.dx = d_input;
    p.dw = d_weight;
    p.N = (int)num_heads;
    p.D = (int)head_dim;
    p.l = (int)l;
    p.d = (int)d;
    const int64_t nd4 = num_heads * head_dim / 4;
    // Weight gradient first (all launches), its chunk sums parked in d_input;
    // then d_input itself.  Chunks: enough workgroups to fill the chip, as
    // many as d_input can hold.
    const int64_t room = total_tokens * head_dim / l;          // chunk sums per (p, n) d_input holds
    const int chunks = (int)std::max<int64_t>(1, std::min<int64_t>({64, room, (1024 + l * num_heads - 1) / (l * num_heads)}));
    for (int pass = 0; pass < 2; ++pass) {
        int64_t in_off = 0, out_off = 0;
        size_t b = 0;
        bool first = true;
        while (b < lens.size() || first) {
            p.nseg = 0;
            int64_t max_items = 0;
            while (b < lens.size() && p.nseg < nsa::kCompressMaxSeg) {
                const int64_t n = n_cmp_of(lens[b], l, d);
                if (lens[b] > 0) {
                    p.in_off[p.nseg] = (int)in_off;
                    p.out_off[p.nseg] = (int)out_off;
                    p.n_in[p.nseg] = (int)lens[b];
                    p.n_out[p.nseg] = (int)n;
                    max_items = std::max(max_items, lens[b] * nd4);
                    ++p.nseg;
                }
                in_off += lens[b];
                out_off += n;
                ++b;
            }
            if (p.nseg == 0 && !first)
                continue;
            p.max_blocks_x = (int)((max_items + 255) / 256);
            p.accumulate = first ? 0 : 1;
            p.part = d_input;
            first = false;
            hipError_t e = pass == 0 ? nsa::launch_compress_bwd_dw((int)dtype, p, chunks, (hipStream_t)stream)
                                     : nsa::launch_compress_bwd_dx((int)dtype, p, (hipStream_t)stream);
            if (e != hipSuccess)
                return fail(NSA_ERR_HIP, "compress backward launch failed: %s", hipGetErrorString(e));
        }
    }
    return ok();
}

}  // extern "C"
