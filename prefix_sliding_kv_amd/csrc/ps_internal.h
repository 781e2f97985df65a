// Internal declarations shared by the library's host code and kernels.
// Not part of the C ABI (see include/ps.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ps.h"

// Host handle behind the opaque ps_cache.
struct ps_cache {
    ps_cache_desc desc;
    char* base = nullptr;        // caller's device buffer
    size_t bytes = 0;
    size_t elem_bytes = 0;       // 2 (bf16) or 4 (f32)
    int64_t rows_per_head = 0;   // prefix_cap + window: the most keys one sequence can hold
    int32_t prefix_blocks = 0;   // prefix pool size (blocks); paged layout: 0
    int32_t page_size = 0;       // paged layout: slots per page (power of two >= 128), else 0
    int32_t page_shift = 0;      // log2(page_size)
    int32_t pages_per_seq = 0;   // paged layout: prefix_cap / page_size + window / page_size
    int32_t n_pages = 0;         // paged layout: pages in the pool of each layer
    size_t pre_layer_bytes = 0;  // bytes of one layer's K (or V) prefix pool
    size_t win_layer_bytes = 0;  // bytes of one layer's K (or V) window pool
    char* k_pre = nullptr;       // [L][prefix_blocks][Hkv][Pcap][d]; paged: page pool [L][n_pages][Hkv][page][d]
    char* v_pre = nullptr;
    char* k_win = nullptr;       // [L][max_seqs][Hkv][W][d]
    char* v_win = nullptr;
    float* ws_o = nullptr;       // [max_seqs][Hq][s_max][d]  unnormalised partial outputs
    float* ws_ml = nullptr;      // [max_seqs][Hq][s_max][2]  (running max in log2 units, sum)
    uint32_t* tickets = nullptr; // [max_seqs][Hkv] arrival counters, one per 256-byte line (self-resetting)
    int32_t s_max = 0;           // split slots per (seq, q head) in the workspace
    int32_t decode_rows = 0;     // requested rows per split, 0 = automatic
    uint32_t* check_flags = nullptr;  // debug checks: sticky violation bits (own 256-byte line)
    int64_t* next_pos = nullptr;      // debug checks: [L][max_seqs] next position of each row, -1 unknown
    int32_t checks = 0;               // debug checks on
    uint64_t* trace = nullptr;        // decode phase trace buffer (device), or null: tracing off
    int32_t trace_launches = 0;       // launch slots in the trace buffer
    int32_t trace_max_wg = 0;         // workgroups per launch slot
    int64_t trace_calls = 0;          // decode calls traced so far (selects the slot)
};

namespace ps {

constexpr int kMinSplitRows = 16;  // smallest rows-per-split the workspace is sized for
constexpr int kTicketStride = 64;  // u32 words between arrival counters: one counter per 256-byte line

// A layer of the cache as the kernels address it.  Block layout: prefix
// block b, kv head g starts at kpre + (b * hkv + g) * pcap rows; window block
// r, kv head g at kwin + (r * hkv + g) * window rows.  Paged layout (pages
// non-null): kpre == kwin is the page pool [n_pages][hkv][page][d]; entry j
// of a sequence's page table row is the page holding its prefix slots
// [j page, (j + 1) page) for j < pcap / page, and its ring slots
// [(j - pcap / page) page, ...) after that.
struct CacheLayer {
    void* kpre;
    void* vpre;
    void* kwin;
    void* vwin;
    int32_t hkv;
    int32_t pcap, window;
    const int32_t* rows;   // window block of each sequence (paged: the sequence's slot for the checks)
    const int32_t* prows;  // prefix block of each sequence of the batch (block layout)
    int64_t v_off;         // bytes from a K slot to its V slot: vpre - kpre == vwin - kwin
    const uint32_t* guard; // checks on: the cache's flag word; a kernel does nothing while it is set
    const int32_t* pages;  // paged layout: page table [n][pages_per_seq], else null
    int32_t pages_per_seq;
    int32_t page_shift;    // log2(page size)
};

// Row index (in rows of d elements, from kpre / vpre) of prefix slot s of
// sequence b, kv head g.
__host__ __device__ inline int64_t prefix_row(const CacheLayer& c, int b, int g, int64_t s) {
    if (c.pages) {
        const int64_t page = c.pages[(int64_t)b * c.pages_per_seq + (s >> c.page_shift)];
        return ((page * c.hkv + g) << c.page_shift) + (s & ((1 << c.page_shift) - 1));
    }
    return ((int64_t)c.prows[b] * c.hkv + g) * c.pcap + s;
}
// Row index (from kwin / vwin) of ring slot r of sequence b, kv head g.
__host__ __device__ inline int64_t ring_row(const CacheLayer& c, int b, int g, int64_t r) {
    if (c.pages) {
        const int64_t page =
            c.pages[(int64_t)b * c.pages_per_seq + (c.pcap >> c.page_shift) + (r >> c.page_shift)];
        return ((page * c.hkv + g) << c.page_shift) + (r & ((1 << c.page_shift) - 1));
    }
    return ((int64_t)c.rows[b] * c.hkv + g) * c.window + r;
}

// Device-side checks of a call's per-sequence arguments (debug mode of a
// cache).  One workgroup: every violation is OR-ed into *flags (bits of
// ps_check_flag); when the word is still clear afterwards, an appending call
// advances next_pos[row] to the position after its last token.
enum CheckMode : int32_t {
    kCheckNone = 0,     // ranges only
    kCheckAppend = 1,   // pos = the row's next position; the call appends n_new tokens
    kCheckNext = 2,     // pos = the row's next position; nothing appended
    kCheckQuery = 3     // pos = the row's last appended position
};
struct CheckParams {
    const int32_t* rows;
    const int32_t* prows;  // or null: rows
    const int32_t* plen;   // or null: plen_scalar
    const int64_t* pos;    // or null: pos_scalar
    int64_t plen_scalar, pos_scalar;
    int32_t n, n_new, mode;
    int32_t max_seqs, prefix_blocks, pcap;
    int64_t* next_pos;     // [max_seqs] of the layer; -1 = nothing appended yet
    uint32_t* flags;
    const int32_t* pages;  // paged layout: page table [n][pages_per_seq], else null
    int32_t pages_per_seq, n_pages;
};
hipError_t launch_check(const CheckParams& p, hipStream_t stream);


// Visibility of key position j to query position i (prefix + window, causal).
__host__ __device__ inline bool visible(int64_t i, int64_t j, int64_t P, int64_t W) {
    return j <= i && (j < P || j > i - W);
}

// Tile classes of the prefill kernel.
enum TileClass : int { kSkip = 0, kFull = 1, kMasked = 2 };

// Closed-form class of query positions [i0, i1] against key positions [j0, j1]:
//   SKIP   iff j0 > i1, or every key is a non-prefix key older than the window
//          of the earliest query (j0 >= P and j1 <= i0 - W);
//   FULL   iff every key is causal for the earliest query (j1 <= i0) and every
//          non-prefix key is inside the window of the latest query
//          (j1 < P or max(j0, P) > i1 - W);
//   MASKED otherwise.
__host__ __device__ inline int tile_class(int64_t i0, int64_t i1, int64_t j0, int64_t j1, int64_t P,
                                          int64_t W) {
    if (j0 > i1 || (j0 >= P && j1 <= i0 - W)) return kSkip;
    const int64_t lo = j0 > P ? j0 : P;
    if (j1 <= i0 && (j1 < P || lo > i1 - W)) return kFull;
    return kMasked;
}

// ------------------------------------------------------------ decode
struct DecodeParams {
    CacheLayer c;
    int32_t hq;
    int64_t rows_per_head; // pcap + window: the most keys a sequence can hold
    const int32_t* plen;
    const int64_t* pos;
    const void* q;
    void* out;
    float* lse;
    float scale_log2;      // scale * log2(e)
    const void* knew;      // fused append: [n][Hkv][d]; nullptr for attention only
    const void* vnew;
    float* ws_o;
    float* ws_ml;
    uint32_t* tickets;
    int32_t s_max;
    int32_t n_seqs;
    int32_t stream_nt;     // nonzero: K/V loads carry the non-temporal hint
    uint64_t* trace;       // non-null: phase timestamps, kDecodeTracePoints per workgroup
};
// Phase timestamps of a traced decode launch (s_memrealtime, 100 MHz), per
// workgroup: entry, sequence metadata in, K rows in and scored, V rows summed,
// waves combined, partial stored and acknowledged, arrival counted, merge
// done (0 unless the workgroup merged).
constexpr int kDecodeTracePoints = 8;

// Workgroups of a decode launch with rows_per_split rows per split.
int64_t decode_grid(int rows_per_split, const DecodeParams& p);
// Traced decode (p.trace set): bf16, head_dim 128, GQA 1, 2 or 4, splits of
// 192 or 256 rows, no non-temporal hint; other shapes return hipErrorNotSupported.
hipError_t launch_decode_traced(int group, int rows_per_split, const DecodeParams& p, hipStream_t stream);
// Launch decode attention; rows_per_split chosen by the caller (host).
hipError_t launch_decode(int dtype, int head_dim, int group, int rows_per_split,
                         const DecodeParams& p, hipStream_t stream);
// Decode on the matrix cores: bf16, head_dim 128, GQA groups 4..8, splits of
// kDecodeMfmaRows key rows.
constexpr int kDecodeMfmaRows = 256;
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);
// Rows one wave covers per 16-byte load instruction for (dtype, head_dim).
int decode_rows_per_load(int dtype, int head_dim);
// Split sizes the decode kernel is built for: with r = decode_rows_per_load,
// 4r, 8r, 16r, 32r, 64r and 128r, each >= 16.
bool decode_rows_valid(int dtype, int head_dim, int rows);

// ------------------------------------------------------------ append
struct AppendParams {
    CacheLayer c;
    const int32_t* plen;
    const int64_t* pos;
    int32_t n_seqs, n_new;
    const void* knew;      // [n][n_new][Hkv][d]
    const void* vnew;
};
hipError_t launch_append(int dtype, int head_dim, const AppendParams& p, hipStream_t stream);
// Append with the rotary encoding of the new keys fused in (keys arrive unrotated).
struct RopeFreqs {
    double inv_freq[64];   // base^(-2e/d), e < d/2, computed on the host
};
hipError_t launch_append_rope(int dtype, int head_dim, const AppendParams& p, const RopeFreqs& f,
                              hipStream_t stream);

// Reset-PE re-rotation of the window keys of a batch by delta positions.
struct RerotateParams {
    CacheLayer c;          // only the window pool is touched
    const int32_t* plen;
    const int64_t* pos;    // window = tokens [max(P, pos - W), pos)
    int32_t n_seqs;
    float cs[64], sn[64];  // cos, sin of the turn of pair e (e < d/2), from the host in double
};
hipError_t launch_rerotate(int dtype, int head_dim, const RerotateParams& p, hipStream_t stream);

// Zero-fill of a u32 array with a kernel (safe inside captured graphs).
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t stream);

// ------------------------------------------------------------ prefill
// A run of keys with contiguous positions and contiguous storage.
struct KeyRun {
    const void* k;         // row 0 of the run for (seq 0, kv head 0)
    const void* v;
    int64_t seq_stride;    // elements between sequences
    int64_t head_stride;   // elements between kv heads
    int64_t row_stride;    // elements between consecutive rows
    int64_t pos0;          // position of row 0
    int64_t n;             // rows in the run
    const int32_t* rows;   // if non-null: sequence b uses cache row rows[b] (seq_stride applies to it)
    // Paged runs (pages non-null): k, v are the page pool; row r of the run
    // is slot first_slot + r of a region whose page j is table entry
    // page_col + j of the sequence's row in `pages`, and is found at row
    // (page * hkv + g) * page + slot % page of the pool.  A paged run never
    // crosses a page boundary inside a 128-row tile (the ring run is split at
    // its first page boundary).
    const int32_t* pages;
    int32_t pages_per_seq, page_col, page_shift;
    int64_t first_slot;
};

constexpr int kMaxRuns = 5;

// One layer's cache pools as a chunk reads them.
struct PrefillCache {
    const char* kpre;      // prefix pool: [prefix_blocks][hkv][pcap][d] (paged: the page pool)
    const char* vpre;
    const char* kwin;      // window pool: [max_seqs][hkv][window][d] (paged: the page pool)
    const char* vwin;
    int64_t pcap, window;
    int32_t hkv, head_dim, elem_bytes;
    const int32_t* rows;   // window block of each sequence
    const int32_t* prows;  // prefix block of each sequence
    const int32_t* pages;  // paged layout: page table [B][pages_per_seq], else null
    int32_t pages_per_seq, page_shift;
};

__host__ __device__ inline void set_cache_run(KeyRun& r, const char* kpool, const char* vpool, int64_t block_rows,
                                              const int32_t* blocks, const PrefillCache& c, int64_t first_slot,
                                              int64_t pos0, int64_t n, int32_t page_col) {
    const int64_t d = c.head_dim;
    r.pos0 = pos0;
    r.n = n;
    r.row_stride = d;
    r.first_slot = first_slot;
    if (c.pages) {
        r.k = kpool;
        r.v = vpool;
        r.seq_stride = 0;
        r.head_stride = d << c.page_shift;
        r.rows = nullptr;
        r.pages = c.pages;
        r.pages_per_seq = c.pages_per_seq;
        r.page_col = page_col;
        r.page_shift = c.page_shift;
        return;
    }
    r.k = kpool + first_slot * d * c.elem_bytes;
    r.v = vpool + first_slot * d * c.elem_bytes;
    r.seq_stride = (int64_t)c.hkv * block_rows * d;
    r.head_stride = block_rows * d;
    r.rows = blocks;
    r.pages = nullptr;
    r.pages_per_seq = r.page_col = r.page_shift = 0;
}

// Runs of the cached keys a chunk starting at position S (prefix length P)
// reads: the prefix slots [0, min(S, P)), then the ring slots of positions
// [max(P, S - W), S) as one or two runs (split where the ring wraps); in the
// paged layout the first ring run is also split at its first page boundary,
// so that every run's 128-row tiles lie inside single pages.  Returns the
// number of runs written (0 to 4).
__host__ __device__ inline int cache_key_runs(const PrefillCache& c, int64_t S, int64_t P, KeyRun* runs) {
    int nr = 0;
    const int64_t W = c.window;
    const int64_t n_pre = S < P ? S : P;
    const int32_t ring_col = c.pages ? (int32_t)(c.pcap >> c.page_shift) : 0;
    if (n_pre > 0) set_cache_run(runs[nr++], c.kpre, c.vpre, c.pcap, c.prows, c, 0, 0, n_pre, 0);
    if (S > P) {
        const int64_t first = S - W > P ? S - W : P;  // oldest position the ring still holds
        const int64_t cnt = S - first;
        const int64_t slot = (first - P) % W;
        int64_t n_a = slot + cnt <= W ? cnt : W - slot;
        int64_t head = 0;  // paged: slots of the first run before its first page boundary
        if (c.pages) {
            const int64_t pg = (int64_t)1 << c.page_shift;
            const int64_t to_boundary = (pg - (slot & (pg - 1))) & (pg - 1);
            head = to_boundary < n_a ? to_boundary : 0;
        }
        if (head > 0) {
            set_cache_run(runs[nr++], c.kwin, c.vwin, W, c.rows, c, slot, first, head, ring_col);
            set_cache_run(runs[nr++], c.kwin, c.vwin, W, c.rows, c, slot + head, first + head, n_a - head, ring_col);
        } else {
            set_cache_run(runs[nr++], c.kwin, c.vwin, W, c.rows, c, slot, first, n_a, ring_col);
        }
        if (n_a < cnt) set_cache_run(runs[nr++], c.kwin, c.vwin, W, c.rows, c, 0, first + n_a, cnt - n_a, ring_col);
    }
    return nr;
}

struct PrefillParams {
    KeyRun runs[kMaxRuns];
    int32_t n_runs;
    int32_t batch, seq_len, hq, hkv;
    int64_t start_pos, P, W;
    const void* q;         // [B][T][Hq][d]
    void* out;
    float* lse;
    float scale_log2;
    // Ragged chunks: when `starts` is set, sequence b's chunk starts at
    // starts[b] (its prefix length is plens[b], or P when plens is null);
    // runs[0] is then the chunk run alone (its pos0 is replaced by starts[b])
    // and, in cache mode, the cached runs come from cache_key_runs(cache).
    const int64_t* starts;
    const int32_t* plens;
    int32_t cache_mode;
    PrefillCache cache;
    const uint32_t* guard;  // checks on: the cache's flag word; the kernel does nothing while it is set
    unsigned long long* trace;  // phase trace [2][8] (bf16 MFMA kernel only), or null
};

// Positions enter the visibility rule only through j < P and i - W < j <= i,
// so a chunk of queries at [S, S + T) gets the same decisions from smaller
// numbers (its "frame"):
//   * trainer mode (the chunk's own keys only): every position is counted
//     from S, P becomes P - S clamped to [0, T] and W is clamped to T
//     (a window longer than the chunk already holds every earlier key);
//   * cache mode (keys are the retained ones, all in [0, S + T)): P and W
//     beyond S + T decide nothing and are clamped to it, and when the chunk
//     starts more than P + W tokens in, every position >= P moves down by
//     S - W - P; differences between those positions are kept, every moved
//     key stays at or above P, and each prefix key stays visible to every
//     query, as it was.
// Afterwards every position is below T (trainer) or min(S, P + W) + T
// (cache), so a kernel may handle a chunk's positions in 32 bits at any
// trace length.
struct PosFrame {
    int64_t P, W;
    int64_t shift;     // subtracted from every position >= move_from
    int64_t move_from;
};
__host__ __device__ inline PosFrame pos_frame(int64_t S, int64_t T, int64_t P, int64_t W, bool chunk_only) {
    PosFrame f;
    if (chunk_only) {
        const int64_t p = P - S;
        f.P = p < 0 ? 0 : (p > T ? T : p);
        f.W = W < T ? W : T;
        f.shift = S;
        f.move_from = 0;
        return f;
    }
    const int64_t end = S + T;
    f.P = P < end ? P : end;
    f.W = W < end ? W : end;
    const int64_t sh = S - f.W - f.P;
    f.shift = sh > 0 ? sh : 0;
    f.move_from = f.P;
    return f;
}
// Move the runs' positions into the frame.
__host__ __device__ inline void frame_runs(const PosFrame& f, KeyRun* runs, int n) {
    for (int r = 0; r < n; ++r)
        if (runs[r].pos0 >= f.move_from) runs[r].pos0 -= f.shift;
}

// Key runs of sequence b, with positions in the frame f of its chunk start S
// and prefix length P (S and P as the caller gave them: the ring slots follow
// from those).  Uniform chunks arrive with runs and positions the host
// already moved (their frame on the device is then the identity).
__device__ inline int seq_key_runs(const PrefillParams& p, int b, int64_t S, int64_t P, const PosFrame& f,
                                   KeyRun* out) {
    if (!p.starts) {
        for (int r = 0; r < p.n_runs; ++r) out[r] = p.runs[r];
        return p.n_runs;
    }
    const int nr = p.cache_mode ? cache_key_runs(p.cache, S, P, out) : 0;
    out[nr] = p.runs[0];
    out[nr].pos0 = S;
    frame_runs(f, out, nr + 1);
    return nr + 1;
}
hipError_t launch_prefill(int dtype, int head_dim, int group, const PrefillParams& p,
                          hipStream_t stream);

// Trainer-side backward (bf16, head_dim 128): Delta, dK/dV, then dQ on one stream.
struct BwdParams {
    PrefillParams f;       // trainer-mode walk: one key run (the chunk); f.q = Q, f.out = forward O
    const void* dout;      // [B][T][Hq][d]
    const float* lse;      // [B][T][Hq] natural log, from the forward
    float* delta_out;      // [B][T][Hq] fp32 workspace: rowsum(dO * O), written first
    const float* delta;    // the same buffer, read by the dQ and dK/dV kernels
    void* dq;              // [B][T][Hq][d]
    void* dk;              // [B][T][Hkv][d]
    void* dv;
    const void* k;         // [B][T][Hkv][d]
    const void* v;
    float scale;
    // Stored dS (DsBand): null, or the band the dK/dV kernel writes and the
    // dQ kernel reads instead of recomputing S and dP
    char* ds;
    int32_t ds_nrb, ds_npre, ds_nwin, ds_nband;
};

// The band of stored dS tiles.  For every (sequence, query head, block rb of
// 32 chunk positions) the blocks of 32 keys its rows can see are the prefix
// blocks 0 .. npre-1 and the window blocks rb-nwin+1 .. rb; a key block kb
// sits in slot kb when kb < npre, else in slot npre + kb - rb + nwin - 1.
// Each slot holds a 32 x 32 tile of bf16 dS (query row x key) as the dK/dV
// kernel holds it: two 1 KB halves of 16 rows, each 64 lanes x 16 bytes,
// lane 32h + key holding rows 16 st + 4h + 0..3 and 16 st + 8 + 4h + 0..3
// of half st.  P and W are in the chunk's frame (positions counted from the
// chunk start, P <= T, W <= T).
// The dK/dV kernel addresses one kv head's part (its `group` query heads)
// with 32-bit offsets, so the band is used only while that part stays below
// 2^31 bytes, and only for groups of up to 4 query heads: on the 8-head
// layout a 16-byte piece of dS spans two heads and takes two stores, which
// cost the dK/dV kernel more than the dQ kernel saves (bytes = 0 otherwise).
struct DsBand {
    int64_t nrb, npre, nwin, nband, bytes;
};
inline DsBand ds_band(int64_t batch, int64_t T, int64_t hq, int64_t group, int64_t P, int64_t W) {
    DsBand d{};
    d.nrb = (T + 31) / 32;
    d.npre = (P + 31) / 32;
    const int64_t nw0 = (W - 1 + 31) / 32;  // window blocks below the row block
    d.nwin = nw0 + 1 < d.nrb ? nw0 + 1 : d.nrb;
    d.nband = d.npre + d.nwin;
    const bool fits = group <= 4 && group * d.nrb * d.nband * 2048 < ((int64_t)1 << 31);
    d.bytes = fits ? batch * hq * d.nrb * d.nband * 2048 : 0;
    return d;
}
hipError_t launch_prefill_bwd(int group, const BwdParams& p, hipStream_t stream);
// The allocation-free backward's Delta rows: a device array of
// PS_BWD_NOALLOC_MAX_ROWS floats the library owns (one copy per GPU, kept
// until the process ends).  Returns this device's copy, its address taken
// once per device, or nullptr if that fails.
float* static_delta();

}  // namespace ps
