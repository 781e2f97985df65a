// C ABI of the Prefix Sliding library: argument validation, cache layout,
// launch planning.  Every device step runs in the library's own HIP kernels;
// nothing here touches tensor data on the host.
#include <math.h>
#include <new>
#include <string.h>

#include "ps_internal.h"

namespace {

constexpr size_t kAlign = 256;
// Largest position any call accepts: positions and position + length stay
// far from int64 overflow.
constexpr int64_t kMaxPos = (int64_t)1 << 62;
constexpr float kLog2e = 1.4426950408889634f;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool desc_ok(const ps_cache_desc* d) {
    if (!d) return false;
    if (d->n_layers < 1 || d->max_seqs < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1) return false;
    if (d->n_q_heads % d->n_kv_heads != 0) return false;
    if (d->prefix_cap < 0 || d->window < 1 || d->prefix_blocks < 0) return false;
    if (d->page_size == 0) return d->n_pages == 0;
    // paged layout: a power of two >= 128 dividing prefix_cap and W, at most
    // 256 pages per sequence, and no prefix blocks
    const int pg = d->page_size;
    if (pg < 128 || (pg & (pg - 1)) != 0 || d->prefix_cap % pg != 0 || d->window % pg != 0) return false;
    if (d->n_pages < 1 || d->prefix_blocks != 0) return false;
    return (int64_t)d->prefix_cap / pg + d->window / pg <= 256;
}

bool desc_supported(const ps_cache_desc* d) {
    if (d->head_dim != 64 && d->head_dim != 128) return false;
    if (d->dtype != PS_BF16 && d->dtype != PS_F32) return false;
    const int g = d->n_q_heads / d->n_kv_heads;
    return g >= 1 && g <= 8;  // GQA groups of the Qwen2.5 / Qwen3 / Llama families
}

// Buffer layout: K prefix pools of every layer, K window pools, V prefix
// pools, V window pools, then the decode workspace.
struct Layout {
    size_t elem, pre_layer_bytes, win_layer_bytes, pre_bytes, win_bytes, ws_o_bytes, ws_ml_bytes, ticket_bytes,
        flag_bytes, next_pos_bytes, total;
    int64_t rows_per_head;
    int32_t prefix_blocks, s_max;
};

Layout layout_of(const ps_cache_desc* d) {
    Layout l{};
    l.elem = d->dtype == PS_BF16 ? 2 : 4;
    l.rows_per_head = (int64_t)d->prefix_cap + d->window;
    if (d->page_size > 0) {  // paged: one page pool per layer (the "prefix" pool), no window pool
        l.prefix_blocks = 0;
        l.pre_layer_bytes = align_up((size_t)d->n_pages * d->n_kv_heads * d->page_size * d->head_dim * l.elem);
        l.win_layer_bytes = 0;
    } else {
        l.prefix_blocks = d->prefix_blocks > 0 ? d->prefix_blocks : d->max_seqs;
        l.pre_layer_bytes = align_up((size_t)l.prefix_blocks * d->n_kv_heads * d->prefix_cap * d->head_dim * l.elem);
        l.win_layer_bytes = align_up((size_t)d->max_seqs * d->n_kv_heads * d->window * d->head_dim * l.elem);
    }
    l.pre_bytes = l.pre_layer_bytes * (size_t)d->n_layers;
    l.win_bytes = l.win_layer_bytes * (size_t)d->n_layers;
    l.s_max = (int32_t)((l.rows_per_head + ps::kMinSplitRows - 1) / ps::kMinSplitRows);
    l.ws_o_bytes = align_up((size_t)d->max_seqs * d->n_q_heads * l.s_max * d->head_dim * 4);
    l.ws_ml_bytes = align_up((size_t)d->max_seqs * d->n_q_heads * l.s_max * 2 * 4);
    l.ticket_bytes = align_up((size_t)d->max_seqs * d->n_kv_heads * ps::kTicketStride * 4);
    l.flag_bytes = kAlign;
    l.next_pos_bytes = align_up((size_t)d->n_layers * d->max_seqs * 8);
    l.total = 2 * (l.pre_bytes + l.win_bytes) + l.ws_o_bytes + l.ws_ml_bytes + l.ticket_bytes + l.flag_bytes +
              l.next_pos_bytes;
    return l;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PS_OK : PS_ERR_HIP; }

// Without prefix_rows a sequence's prefix block is its row, which needs one
// prefix block per row.
bool batch_ok(const ps_cache* c, const ps_seq_batch* b) {
    if (!b || b->n < 1 || b->n > c->desc.max_seqs || !b->rows || !b->prefix_len || !b->pos) return false;
    if (c->page_size) return b->page_table != nullptr;  // paged: the page table names every slot's page
    if (b->page_table) return false;
    return b->prefix_rows || c->prefix_blocks == c->desc.max_seqs;
}

ps::CacheLayer cache_layer(const ps_cache* c, int32_t layer, const ps_seq_batch* b) {
    ps::CacheLayer v{};
    v.kpre = c->k_pre + (size_t)layer * c->pre_layer_bytes;
    v.vpre = c->v_pre + (size_t)layer * c->pre_layer_bytes;
    v.kwin = c->k_win + (size_t)layer * c->win_layer_bytes;
    v.vwin = c->v_win + (size_t)layer * c->win_layer_bytes;
    v.hkv = c->desc.n_kv_heads;
    v.pcap = c->desc.prefix_cap;
    v.window = c->desc.window;
    v.rows = b->rows;
    v.prows = b->prefix_rows ? b->prefix_rows : b->rows;
    v.v_off = c->v_pre - c->k_pre;  // == v_win - k_win (see ps_cache_create)
    v.guard = c->checks ? c->check_flags : nullptr;
    if (c->page_size) {  // one page pool serves prefix and window slots
        v.kwin = v.kpre;
        v.vwin = v.vpre;
        v.pages = b->page_table;
        v.pages_per_seq = c->pages_per_seq;
        v.page_shift = c->page_shift;
    }
    return v;
}

// Debug checks of a call's per-sequence arguments, enqueued before its kernels.
int run_checks(const ps_cache* c, int32_t layer, const int32_t* rows, const int32_t* prows, const int32_t* plen,
               const int64_t* pos, int64_t plen_scalar, int64_t pos_scalar, int32_t n, int32_t n_new, int32_t mode,
               void* stream, const int32_t* pages = nullptr) {
    ps::CheckParams p{};
    p.pages = pages;
    p.pages_per_seq = c->pages_per_seq;
    p.n_pages = c->n_pages;
    p.rows = rows;
    p.prows = prows;
    p.plen = plen;
    p.pos = pos;
    p.plen_scalar = plen_scalar;
    p.pos_scalar = pos_scalar;
    p.n = n;
    p.n_new = n_new;
    p.mode = mode;
    p.max_seqs = c->desc.max_seqs;
    p.prefix_blocks = c->prefix_blocks;
    p.pcap = c->desc.prefix_cap;
    p.next_pos = c->next_pos + (size_t)layer * c->desc.max_seqs;
    p.flags = c->check_flags;
    return hip_status(ps::launch_check(p, (hipStream_t)stream));
}

int batch_checks(const ps_cache* c, int32_t layer, const ps_seq_batch* b, int32_t n_new, int32_t mode, void* stream) {
    if (!c->checks) return PS_OK;
    return run_checks(c, layer, b->rows, b->prefix_rows, b->prefix_len, b->pos, 0, 0, b->n, n_new, mode, stream,
                      b->page_table);
}

// Rows per decode split.  A decode launch is short (tens of MB at batch 1),
// so the split count per (sequence, kv head) also sets the length of the
// merge the last split performs: take the largest split whose launch still
// has at least 160 workgroups (5/8 of the 256 CUs), else the smallest valid
// one.  At batch 1 with 4196 rows per kv head and 8 kv heads that is 192
// rows (176 workgroups): measured 1.7% faster per launch than 256 rows (136
// workgroups), 160 rows (216) 0.6% faster, 128 rows (272, more than the CUs)
// 25% slower.
int auto_decode_rows(const ps_cache* c, int n_seqs) {
    const int r = ps::decode_rows_per_load(c->desc.dtype, c->desc.head_dim);
    const int cand[] = {64 * r, 48 * r, 32 * r, 16 * r, 8 * r, 4 * r};
    int smallest = 0;
    for (int rows : cand) {
        if (!ps::decode_rows_valid(c->desc.dtype, c->desc.head_dim, rows)) continue;
        smallest = rows;
        const int64_t splits = (c->rows_per_head + rows - 1) / rows;
        if ((int64_t)n_seqs * c->desc.n_kv_heads * splits >= 160) return rows;
    }
    return smallest;
}

bool decode_rows_ok(const ps_cache* c, int rows) {
    return ps::decode_rows_valid(c->desc.dtype, c->desc.head_dim, rows);
}

int decode_common(ps_cache* c, int32_t layer, const ps_seq_batch* batch, const void* q, const void* knew,
                  const void* vnew, void* out, float* lse, float scale, void* stream) {
    if (!c || !batch_ok(c, batch) || !q || !out) return PS_ERR_INVALID;
    if (layer < 0 || layer >= c->desc.n_layers) return PS_ERR_INVALID;
    if (!isfinite(scale)) return PS_ERR_INVALID;
    ps::DecodeParams p{};
    p.c = cache_layer(c, layer, batch);
    p.hq = c->desc.n_q_heads;
    p.rows_per_head = c->rows_per_head;
    p.plen = batch->prefix_len;
    p.pos = batch->pos;
    p.q = q;
    p.out = out;
    p.lse = lse;
    p.scale_log2 = scale * kLog2e;
    p.knew = knew;
    p.vnew = vnew;
    p.ws_o = c->ws_o;
    p.ws_ml = c->ws_ml;
    p.tickets = c->tickets;
    p.s_max = c->s_max;
    p.n_seqs = batch->n;
    const int st = batch_checks(c, layer, batch, knew ? 1 : 0, knew ? ps::kCheckAppend : ps::kCheckQuery, stream);
    if (st != PS_OK) return st;
    const int group = c->desc.n_q_heads / c->desc.n_kv_heads;
    if (c->page_size) {
        // paged layout: the vector kernel with 8 waves and 8 rows per lane
        const int rows = 64 * ps::decode_rows_per_load(c->desc.dtype, c->desc.head_dim);
        if (c->trace || (c->decode_rows != 0 && c->decode_rows != rows)) return PS_ERR_UNSUPPORTED;
        p.stream_nt = ps::decode_grid(rows, p) >= 1024;
        return hip_status(ps::launch_decode(c->desc.dtype, c->desc.head_dim, group, rows, p, (hipStream_t)stream));
    }
    if (c->trace) {
        // traced launches: the 192- or 256-row split kernel with phase timestamps
        const int rows = c->decode_rows > 0 ? c->decode_rows : auto_decode_rows(c, batch->n);
        if (c->desc.dtype != PS_BF16 || c->desc.head_dim != 128 || (group != 1 && group != 2 && group != 4) ||
            (rows != 192 && rows != 256))
            return PS_ERR_UNSUPPORTED;
        if (ps::decode_grid(rows, p) > c->trace_max_wg) return PS_ERR_UNSUPPORTED;
        const int64_t slot = c->trace_calls++ % c->trace_launches;
        p.trace = c->trace + (size_t)slot * c->trace_max_wg * ps::kDecodeTracePoints;
        return hip_status(ps::launch_decode_traced(group, rows, p, (hipStream_t)stream));
    }
    if (c->decode_rows == 0 && c->desc.dtype == PS_BF16 && c->desc.head_dim == 128 && group >= 5) {
        // five or more heads per kv head: the matrix-core kernel (its own
        // split size; measured faster from G = 5 on, 2% slower at G = 4)
        const int64_t n_wg = (int64_t)batch->n * c->desc.n_kv_heads *
                             ((c->rows_per_head + ps::kDecodeMfmaRows - 1) / ps::kDecodeMfmaRows);
        p.stream_nt = n_wg >= 1024;
        return hip_status(ps::launch_decode_mfma(p, (hipStream_t)stream));
    }
    const int rows = c->decode_rows > 0 ? c->decode_rows : auto_decode_rows(c, batch->n);
    // several workgroups per CU: the kernel marks its K/V loads non-temporal
    const int64_t n_wg = (int64_t)batch->n * c->desc.n_kv_heads * ((c->rows_per_head + rows - 1) / rows);
    p.stream_nt = n_wg >= 1024;
    return hip_status(ps::launch_decode(c->desc.dtype, c->desc.head_dim, group, rows, p, (hipStream_t)stream));
}

// Trainer backward: validation, then Delta, dK/dV and dQ on `stream`.  With
// own_delta the Delta rows go to the library's own device array (the
// allocation-free entry point) and args->delta must be NULL.
int bwd_common(const ps_prefill_bwd_args* a, bool own_delta, void* stream) {
    if (!a) return PS_ERR_INVALID;
    if (own_delta && a->delta) return PS_ERR_INVALID;
    if (a->batch < 1 || a->seq_len < 0 || a->start_pos < 0 || a->prefix_len < 0 || a->window < 1)
        return PS_ERR_INVALID;
    if (!isfinite(a->scale) || !(a->scale > 0.f)) return PS_ERR_INVALID;
    const int hq = a->n_q_heads, hkv = a->n_kv_heads, d = a->head_dim;
    if (hq < 1 || hkv < 1 || hq % hkv != 0) return PS_ERR_INVALID;
    if (a->dtype != PS_BF16 || d != 128) return PS_ERR_UNSUPPORTED;
    const int group = hq / hkv;
    if (group < 1 || group > 8) return PS_ERR_UNSUPPORTED;
    if (a->start_pos > kMaxPos - a->seq_len) return PS_ERR_UNSUPPORTED;
    // positions in the chunk's frame (ps::pos_frame: counted from the chunk
    // start) are 32-bit in the kernels
    const ps::PosFrame fr = ps::pos_frame(a->start_pos, a->seq_len, a->prefix_len, a->window, true);
    // byte offsets of rows inside one sequence (plus one 64-row sub-tile past
    // its end) are 32-bit in the kernels
    if (((int64_t)a->seq_len + 64) * hq * d * 2 >= ((int64_t)1 << 31)) return PS_ERR_UNSUPPORTED;
    if (own_delta && (int64_t)a->batch * a->seq_len * hq > PS_BWD_NOALLOC_MAX_ROWS) return PS_ERR_CAPACITY;
    if (a->seq_len == 0) return PS_OK;
    if (!a->q || !a->k || !a->v || !a->out || !a->lse || !a->dout || !a->dq || !a->dk || !a->dv ||
        (!own_delta && !a->delta))
        return PS_ERR_INVALID;
    float* delta = own_delta ? ps::static_delta() : a->delta;
    if (!delta) return PS_ERR_HIP;
    ps::BwdParams p{};
    const int64_t T = a->seq_len;
    ps::KeyRun& r = p.f.runs[0];
    r.k = a->k;
    r.v = a->v;
    r.seq_stride = T * hkv * d;
    r.head_stride = d;
    r.row_stride = (int64_t)hkv * d;
    r.pos0 = a->start_pos - fr.shift;
    r.n = T;
    r.rows = nullptr;
    p.f.n_runs = 1;
    p.f.batch = a->batch;
    p.f.seq_len = a->seq_len;
    p.f.hq = hq;
    p.f.hkv = hkv;
    p.f.start_pos = a->start_pos - fr.shift;
    p.f.P = fr.P;
    p.f.W = fr.W;
    p.f.q = a->q;
    p.f.out = const_cast<void*>(a->out);
    p.f.lse = nullptr;
    p.f.scale_log2 = a->scale * kLog2e;
    p.dout = a->dout;
    p.lse = a->lse;
    p.delta_out = delta;
    p.delta = delta;
    p.dq = a->dq;
    p.dk = a->dk;
    p.dv = a->dv;
    p.k = a->k;
    p.v = a->v;
    p.scale = a->scale;
    const ps::DsBand band = ps::ds_band(a->batch, T, hq, group, fr.P, fr.W);
    if (a->ds_work && band.bytes > 0) {
        if (a->ds_work_bytes < band.bytes) return PS_ERR_CAPACITY;
        p.ds = static_cast<char*>(a->ds_work);
        p.ds_nrb = (int32_t)band.nrb;
        p.ds_npre = (int32_t)band.npre;
        p.ds_nwin = (int32_t)band.nwin;
        p.ds_nband = (int32_t)band.nband;
    }
    return hip_status(ps::launch_prefill_bwd(group, p, (hipStream_t)stream));
}

}  // namespace

extern "C" {

size_t ps_cache_bytes(const ps_cache_desc* desc) {
    if (!desc_ok(desc) || !desc_supported(desc)) return 0;
    return layout_of(desc).total;
}

int ps_cache_create(const ps_cache_desc* desc, void* dev_mem, size_t bytes, void* stream, ps_cache** out) {
    if (!out) return PS_ERR_INVALID;
    *out = nullptr;
    if (!desc_ok(desc) || !dev_mem) return PS_ERR_INVALID;
    if (!desc_supported(desc)) return PS_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(dev_mem) % kAlign != 0) return PS_ERR_INVALID;
    const Layout l = layout_of(desc);
    if (bytes < l.total) return PS_ERR_CAPACITY;
    ps_cache* c = new (std::nothrow) ps_cache;
    if (!c) return PS_ERR_INVALID;
    c->desc = *desc;
    c->base = static_cast<char*>(dev_mem);
    c->bytes = bytes;
    c->elem_bytes = l.elem;
    c->rows_per_head = l.rows_per_head;
    c->prefix_blocks = l.prefix_blocks;
    c->page_size = desc->page_size;
    c->n_pages = desc->n_pages;
    c->page_shift = 0;
    while (c->page_size && (1 << c->page_shift) < c->page_size) ++c->page_shift;
    c->pages_per_seq = c->page_size ? desc->prefix_cap / c->page_size + desc->window / c->page_size : 0;
    c->pre_layer_bytes = l.pre_layer_bytes;
    c->win_layer_bytes = l.win_layer_bytes;
    // K pools, then V pools in the same order: a V slot lies at one fixed
    // distance from its K slot in both pools, which lets a kernel address V
    // from K with one add
    c->k_pre = c->base;
    c->k_win = c->k_pre + l.pre_bytes;
    c->v_pre = c->k_win + l.win_bytes;
    c->v_win = c->v_pre + l.pre_bytes;
    // (paged: win_bytes is 0, and the kernels address window slots in the
    // page pool, see cache_layer)
    char* ws = c->v_win + l.win_bytes;
    c->ws_o = reinterpret_cast<float*>(ws);
    c->ws_ml = reinterpret_cast<float*>(ws + l.ws_o_bytes);
    c->tickets = reinterpret_cast<uint32_t*>(ws + l.ws_o_bytes + l.ws_ml_bytes);
    c->check_flags = reinterpret_cast<uint32_t*>(ws + l.ws_o_bytes + l.ws_ml_bytes + l.ticket_bytes);
    c->next_pos = reinterpret_cast<int64_t*>(ws + l.ws_o_bytes + l.ws_ml_bytes + l.ticket_bytes + l.flag_bytes);
    c->s_max = l.s_max;
    c->decode_rows = 0;
    c->checks = 0;
    hipError_t e = ps::launch_fill_u32(c->tickets, (size_t)desc->max_seqs * desc->n_kv_heads * ps::kTicketStride, 0u,
                                       (hipStream_t)stream);
    if (e == hipSuccess) e = ps::launch_fill_u32(c->check_flags, kAlign / 4, 0u, (hipStream_t)stream);
    if (e == hipSuccess)  // -1 in every next position: nothing appended yet
        e = ps::launch_fill_u32(reinterpret_cast<uint32_t*>(c->next_pos), (size_t)desc->n_layers * desc->max_seqs * 2,
                                0xFFFFFFFFu, (hipStream_t)stream);
    if (e != hipSuccess) {
        delete c;
        return PS_ERR_HIP;
    }
    *out = c;
    return PS_OK;
}

int ps_cache_destroy(ps_cache* cache) {
    delete cache;
    return PS_OK;
}

int ps_cache_pages(const ps_cache* c, int32_t layer, void** k_pages, void** v_pages) {
    if (!c || !k_pages || !v_pages || layer < 0 || layer >= c->desc.n_layers) return PS_ERR_INVALID;
    if (!c->page_size) return PS_ERR_UNSUPPORTED;
    *k_pages = c->k_pre + (size_t)layer * c->pre_layer_bytes;
    *v_pages = c->v_pre + (size_t)layer * c->pre_layer_bytes;
    return PS_OK;
}

int ps_cache_blocks(const ps_cache* c, int32_t layer, void** k_prefix, void** v_prefix, void** k_window,
                    void** v_window) {
    if (!c || !k_prefix || !v_prefix || !k_window || !v_window || layer < 0 || layer >= c->desc.n_layers)
        return PS_ERR_INVALID;
    if (c->page_size) return PS_ERR_UNSUPPORTED;
    *k_prefix = c->k_pre + (size_t)layer * c->pre_layer_bytes;
    *v_prefix = c->v_pre + (size_t)layer * c->pre_layer_bytes;
    *k_window = c->k_win + (size_t)layer * c->win_layer_bytes;
    *v_window = c->v_win + (size_t)layer * c->win_layer_bytes;
    return PS_OK;
}

int ps_cache_set_checks(ps_cache* c, int32_t on) {
    if (!c) return PS_ERR_INVALID;
    c->checks = on != 0;
    return PS_OK;
}

int ps_cache_check_flags(ps_cache* c, uint32_t* flags, int32_t clear, void* stream) {
    if (!c || !flags) return PS_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(flags, c->check_flags, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return PS_ERR_HIP;
    if (clear && ps::launch_fill_u32(c->check_flags, 1, 0u, s) != hipSuccess) return PS_ERR_HIP;
    return hip_status(hipStreamSynchronize(s));
}

int ps_cache_set_decode_split(ps_cache* c, int32_t rows_per_split) {
    if (!c || rows_per_split < 0) return PS_ERR_INVALID;
    if (rows_per_split != 0 && !decode_rows_ok(c, rows_per_split)) return PS_ERR_UNSUPPORTED;
    c->decode_rows = rows_per_split;
    return PS_OK;
}

int ps_cache_set_decode_trace(ps_cache* c, uint64_t* dev_buf, int32_t n_launches, int32_t max_wg) {
    if (!c) return PS_ERR_INVALID;
    if (dev_buf && (n_launches < 1 || max_wg < 1)) return PS_ERR_INVALID;
    c->trace = dev_buf;
    c->trace_launches = dev_buf ? n_launches : 0;
    c->trace_max_wg = dev_buf ? max_wg : 0;
    c->trace_calls = 0;
    return PS_OK;
}

int ps_kv_append_evict(ps_cache* c, int32_t layer, const ps_seq_batch* batch, int32_t n_new, const void* k_new,
                       const void* v_new, void* stream) {
    if (!c || !batch_ok(c, batch) || n_new < 0) return PS_ERR_INVALID;
    if (layer < 0 || layer >= c->desc.n_layers) return PS_ERR_INVALID;
    if (n_new == 0) return PS_OK;
    if (!k_new || !v_new) return PS_ERR_INVALID;
    const int st = batch_checks(c, layer, batch, n_new, ps::kCheckAppend, stream);
    if (st != PS_OK) return st;
    ps::AppendParams p{};
    p.c = cache_layer(c, layer, batch);
    p.plen = batch->prefix_len;
    p.pos = batch->pos;
    p.n_seqs = batch->n;
    p.n_new = n_new;
    p.knew = k_new;
    p.vnew = v_new;
    return hip_status(ps::launch_append(c->desc.dtype, c->desc.head_dim, p, (hipStream_t)stream));
}

int ps_kv_append_rope(ps_cache* c, int32_t layer, const ps_seq_batch* batch, int32_t n_new, const void* k_new,
                      const void* v_new, float rope_base, void* stream) {
    if (!c || !batch_ok(c, batch) || n_new < 0) return PS_ERR_INVALID;
    if (layer < 0 || layer >= c->desc.n_layers) return PS_ERR_INVALID;
    if (!isfinite(rope_base) || !(rope_base > 1.f)) return PS_ERR_INVALID;
    if (n_new == 0) return PS_OK;
    if (!k_new || !v_new) return PS_ERR_INVALID;
    const int st = batch_checks(c, layer, batch, n_new, ps::kCheckAppend, stream);
    if (st != PS_OK) return st;
    ps::AppendParams p{};
    p.c = cache_layer(c, layer, batch);
    p.plen = batch->prefix_len;
    p.pos = batch->pos;
    p.n_seqs = batch->n;
    p.n_new = n_new;
    p.knew = k_new;
    p.vnew = v_new;
    ps::RopeFreqs f{};
    const int d = c->desc.head_dim;
    for (int e = 0; e < d / 2; ++e) f.inv_freq[e] = pow((double)rope_base, -2.0 * e / (double)d);
    return hip_status(ps::launch_append_rope(c->desc.dtype, d, p, f, (hipStream_t)stream));
}

int ps_kv_rerotate(ps_cache* c, int32_t layer, const ps_seq_batch* batch, int64_t delta, float rope_base,
                   void* stream) {
    if (!c || !batch_ok(c, batch)) return PS_ERR_INVALID;
    if (layer < 0 || layer >= c->desc.n_layers) return PS_ERR_INVALID;
    if (!isfinite(rope_base) || !(rope_base > 1.f)) return PS_ERR_INVALID;
    if (delta == 0) return PS_OK;
    const int st = batch_checks(c, layer, batch, 0, ps::kCheckNext, stream);
    if (st != PS_OK) return st;
    ps::RerotateParams p{};
    p.c = cache_layer(c, layer, batch);
    p.plen = batch->prefix_len;
    p.pos = batch->pos;
    p.n_seqs = batch->n;
    const int d = c->desc.head_dim;
    for (int e = 0; e < d / 2; ++e) {
        const double t = (double)delta * pow((double)rope_base, -2.0 * e / (double)d);
        p.cs[e] = (float)cos(t);
        p.sn[e] = (float)sin(t);
    }
    return hip_status(ps::launch_rerotate(c->desc.dtype, c->desc.head_dim, p, (hipStream_t)stream));
}

int ps_decode_attn(ps_cache* c, int32_t layer, const ps_seq_batch* batch, const void* q, void* out, float* lse,
                   float scale, void* stream) {
    return decode_common(c, layer, batch, q, nullptr, nullptr, out, lse, scale, stream);
}

int ps_decode_step(ps_cache* c, int32_t layer, const ps_seq_batch* batch, const void* q, const void* k_new,
                   const void* v_new, void* out, float* lse, float scale, void* stream) {
    if (!k_new || !v_new) return PS_ERR_INVALID;
    return decode_common(c, layer, batch, q, k_new, v_new, out, lse, scale, stream);
}

int ps_prefill_attn(const ps_prefill_args* a, void* stream) {
    if (!a) return PS_ERR_INVALID;
    if (a->batch < 1 || a->seq_len < 0 || a->start_pos < 0 || a->prefix_len < 0 || a->window < 1)
        return PS_ERR_INVALID;
    if (!isfinite(a->scale) || !(a->scale > 0.f)) return PS_ERR_INVALID;
    if (a->prefix_lens && !a->starts) return PS_ERR_INVALID;
    if (!a->cache && a->page_table) return PS_ERR_INVALID;
    if (a->start_pos > kMaxPos - a->seq_len) return PS_ERR_UNSUPPORTED;
    int hq = a->n_q_heads, hkv = a->n_kv_heads, d = a->head_dim, dtype = a->dtype;
    const ps_cache* c = a->cache;
    if (c) {
        if (a->layer < 0 || a->layer >= c->desc.n_layers || a->batch > c->desc.max_seqs || !a->rows)
            return PS_ERR_INVALID;
        if (hq != c->desc.n_q_heads || hkv != c->desc.n_kv_heads || d != c->desc.head_dim ||
            dtype != c->desc.dtype)
            return PS_ERR_INVALID;
        if (a->window != c->desc.window || a->prefix_len > c->desc.prefix_cap) return PS_ERR_INVALID;
        if (c->page_size) {
            if (!a->page_table) return PS_ERR_INVALID;
        } else {
            if (a->page_table) return PS_ERR_INVALID;
            if (!a->prefix_rows && c->prefix_blocks != c->desc.max_seqs) return PS_ERR_INVALID;
        }
    }
    if (hq < 1 || hkv < 1 || hq % hkv != 0) return PS_ERR_INVALID;
    if (dtype != PS_BF16 && dtype != PS_F32) return PS_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return PS_ERR_UNSUPPORTED;
    const int group = hq / hkv;
    if (a->seq_len == 0) return PS_OK;
    if (!a->q || !a->k || !a->v || !a->out) return PS_ERR_INVALID;

    ps::PrefillParams p{};
    const int64_t P = a->prefix_len, W = a->window, S = a->start_pos, T = a->seq_len;
    const bool ragged = a->starts != nullptr;
    // The kernels work on positions moved into the chunk's frame
    // (ps::pos_frame), in 32 bits: every position there is below T (trainer
    // mode) or min(S, P + W) + T (cache mode, P <= prefix_cap).  Ragged
    // chunks are moved on the device.
    const ps::PosFrame fr = ps::pos_frame(S, T, P, W, c == nullptr);
    const int64_t lim = (int64_t)1 << 31;
    if (ragged) {
        if (c && (int64_t)c->desc.prefix_cap + W + T >= lim) return PS_ERR_UNSUPPORTED;
    } else if (S - fr.shift + T >= lim) {
        return PS_ERR_UNSUPPORTED;
    }
    int nr = 0;
    if (c) {
        ps::PrefillCache& pc = p.cache;
        pc.kpre = c->k_pre + (size_t)a->layer * c->pre_layer_bytes;
        pc.vpre = c->v_pre + (size_t)a->layer * c->pre_layer_bytes;
        pc.kwin = c->k_win + (size_t)a->layer * c->win_layer_bytes;
        pc.vwin = c->v_win + (size_t)a->layer * c->win_layer_bytes;
        pc.pcap = c->desc.prefix_cap;
        pc.window = c->desc.window;
        pc.hkv = hkv;
        pc.head_dim = d;
        pc.elem_bytes = (int32_t)c->elem_bytes;
        pc.rows = a->rows;
        pc.prows = a->prefix_rows ? a->prefix_rows : a->rows;
        if (c->page_size) {
            pc.kwin = pc.kpre;
            pc.vwin = pc.vpre;
            pc.pages = a->page_table;
            pc.pages_per_seq = c->pages_per_seq;
            pc.page_shift = c->page_shift;
        }
        p.cache_mode = 1;
        // uniform chunks: the cached runs are the same for every sequence
        if (!ragged) nr = ps::cache_key_runs(pc, S, P, p.runs);
        if (c->checks) {
            const int st = run_checks(c, a->layer, a->rows, a->prefix_rows, ragged ? a->prefix_lens : nullptr,
                                      a->starts, P, S, a->batch, a->seq_len, ps::kCheckNext, stream, a->page_table);
            if (st != PS_OK) return st;
            p.guard = c->check_flags;
        }
    }
    {
        ps::KeyRun& r = p.runs[nr++];
        r.k = a->k;
        r.v = a->v;
        r.seq_stride = T * hkv * d;
        r.head_stride = d;
        r.row_stride = (int64_t)hkv * d;
        r.pos0 = S;
        r.n = T;
        r.rows = nullptr;
    }
    p.n_runs = nr;
    p.batch = a->batch;
    p.seq_len = a->seq_len;
    p.hq = hq;
    p.hkv = hkv;
    if (ragged) {  // each sequence's frame is taken on the device
        p.start_pos = S;
        p.P = P;
        p.W = W;
    } else {
        ps::frame_runs(fr, p.runs, nr);
        p.start_pos = S - fr.shift;
        p.P = fr.P;
        p.W = fr.W;
    }
    p.q = a->q;
    p.out = a->out;
    p.lse = a->lse;
    p.scale_log2 = a->scale * kLog2e;
    p.starts = a->starts;
    p.plens = ragged ? a->prefix_lens : nullptr;
    p.trace = reinterpret_cast<unsigned long long*>(a->trace);
    return hip_status(ps::launch_prefill(dtype, d, group, p, (hipStream_t)stream));
}

int ps_prefill_attn_bwd(const ps_prefill_bwd_args* a, void* stream) { return bwd_common(a, false, stream); }

int ps_prefill_attn_bwd_noalloc(const ps_prefill_bwd_args* a, void* stream) { return bwd_common(a, true, stream); }

int ps_prefill_bwd_ds_bytes(const ps_prefill_bwd_args* a, int64_t* bytes) {
    if (!a || !bytes) return PS_ERR_INVALID;
    if (a->batch < 1 || a->seq_len < 0 || a->start_pos < 0 || a->prefix_len < 0 || a->window < 1 ||
        a->n_q_heads < 1 || a->n_kv_heads < 1 || a->n_q_heads % a->n_kv_heads != 0)
        return PS_ERR_INVALID;
    if (a->start_pos > kMaxPos - a->seq_len) return PS_ERR_UNSUPPORTED;
    const ps::PosFrame fr = ps::pos_frame(a->start_pos, a->seq_len, a->prefix_len, a->window, true);
    const int group = a->n_q_heads / a->n_kv_heads;
    *bytes = a->seq_len == 0 ? 0 : ps::ds_band(a->batch, a->seq_len, a->n_q_heads, group, fr.P, fr.W).bytes;
    return PS_OK;
}

int ps_tile_class(int64_t i0, int64_t i1, int64_t j0, int64_t j1, int64_t P, int64_t W) {
    if (i1 < i0 || j1 < j0 || P < 0 || W < 1) return -1;
    return ps::tile_class(i0, i1, j0, j1, P, W);
}

const char* ps_status_str(int s) {
    switch (s) {
        case PS_OK: return "ok";
        case PS_ERR_INVALID: return "invalid argument";
        case PS_ERR_UNSUPPORTED: return "unsupported configuration";
        case PS_ERR_CAPACITY: return "buffer too small";
        case PS_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* ps_version(void) { return "0.1.0"; }

}  // extern "C"
