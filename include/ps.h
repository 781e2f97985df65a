/*
 * ps.h -- C ABI of the Prefix Sliding attention library (libprefix_sliding.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * Prefix Sliding keeps, for every query, the pinned task prefix (the first P
 * tokens of the sequence) plus the most recent W tokens; every token in
 * between leaves the KV cache for good (njhaofan.com article on Prefix
 * Sliding, section "PrefixSliding如何丢掉中间Token？"; agihunt.info summary
 * "Prefix Sliding for efficient test-time scaling", paragraphs on the two kept
 * slices and the 4,196-token memory cap).  Key j is visible to query i iff
 *
 *     j <= i  and  (j < P  or  j > i - W).
 *
 * Position IDs keep climbing (Continue PE, agihunt.info summary, paragraph on
 * position encodings): keys are stored already rotated at their own position
 * and are never re-encoded, so evicting a token never touches another.
 *
 * Conventions shared by every entry point
 *  - Memory: the caller owns all device memory and every stream.  The library
 *    allocates nothing on the device, ever; a cache handle owns only a small
 *    host struct.  Pointers documented "device" must be device-accessible
 *    (hipMalloc / torch CUDA tensors); "host" pointers are read before return.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  All device work is enqueued on it and the call returns without
 *    waiting; outputs are valid once the stream reaches that point.
 *  - Errors: every function validates its host-visible arguments before any
 *    device work and returns a ps_status; nothing is enqueued on error.  A
 *    failed launch is reported as PS_ERR_HIP.  No C++ exception crosses the
 *    ABI.  Device-resident arguments (positions, prefix lengths, cache rows)
 *    are not read by the host; their preconditions are listed per call and
 *    are the caller's responsibility.
 *  - Concurrency: calls that use the same cache must be ordered (one stream, or
 *    streams joined by events): decode calls share one split-K workspace
 *    inside the cache buffer.
 *  - dtypes: PS_BF16 (the production path; fp32 accumulation) and PS_F32 (a
 *    debug path computing in fp32 throughout).  head_dim is 64 or 128.
 *  - Layouts are row-major C arrays; the last index is contiguous.
 */
#ifndef PREFIX_SLIDING_PS_H
#define PREFIX_SLIDING_PS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PS_OK = 0,
    PS_ERR_INVALID = 1,      /* bad argument (NULL pointer, out-of-range index, size) */
    PS_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim, dtype, GQA ratio) */
    PS_ERR_CAPACITY = 3,     /* buffer too small for the described cache */
    PS_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} ps_status;

typedef enum { PS_BF16 = 0, PS_F32 = 1 } ps_dtype;

/* Static shape of a cache.  One cache holds every layer of up to max_seqs
 * sequences as two pools of blocks: PREFIX blocks of prefix_cap slots and
 * WINDOW blocks of W slots (a ring), per (layer, block, kv head) -- the
 * two-block cache of the papers.ananclaw.com explainer, section "核心方法"
 * (PREFIX block kept read-only after prefill, WINDOW block of the last W
 * tokens, middle evicted).  A sequence uses one window block (its row) and
 * one prefix block, which several sequences may share: rollouts of the same
 * prompt keep one copy of the pinned prefix (the explainer notes the policy
 * is orthogonal to paged memory management and can be combined with it).
 * A sequence's size is bounded by P + W tokens no matter how long the trace
 * grows (njhaofan.com, same section as above).
 *
 * Paged layout (page_size > 0): the explainer's remark that the policy sits
 * on top of paged memory management and combines with it (papers.ananclaw.com,
 * section "对工程落地的启发"), taken literally.  Each layer then holds one pool
 * of n_pages pages of page_size slots per kv head, and every sequence names
 * its pages in a page table: entry j < prefix_cap / page_size is the page of
 * its prefix slots [j * page_size, (j + 1) * page_size), entry
 * prefix_cap / page_size + j the page of its window (ring) slots
 * [j * page_size, (j + 1) * page_size).  Pages are allocated and shared by
 * the caller (ps_block_pool counts references): sequences whose prompts
 * begin with the same page_size-aligned run of tokens may point at the same
 * prefix pages for it, and each keeps private pages for the rest of its
 * prefix and for its window.  page_size is a power of two >= 128 (the
 * prefill kernels' key tile) that divides prefix_cap and W, and a sequence
 * has at most 256 pages (prefix_cap + W <= 256 * page_size). */
typedef struct {
    int32_t n_layers;       /* >= 1 */
    int32_t max_seqs;       /* >= 1: window blocks (sequence rows) */
    int32_t n_q_heads;      /* Hq >= 1, n_kv_heads times 1 to 8 (the GQA group) */
    int32_t n_kv_heads;     /* Hkv >= 1 */
    int32_t head_dim;       /* d: 64 or 128 */
    int32_t prefix_cap;     /* largest prefix length P any sequence may use, >= 0 */
    int32_t window;         /* W >= 1 */
    int32_t dtype;          /* ps_dtype of K, V, queries and outputs */
    int32_t prefix_blocks;  /* prefix blocks, >= 0; 0 means max_seqs (one per row); 0 when paged */
    int32_t page_size;      /* 0: block layout; else slots per page of the paged layout */
    int32_t n_pages;        /* paged layout: pages in each layer's pool (>= 1), else 0 */
} ps_cache_desc;

typedef struct ps_cache ps_cache; /* opaque host handle */

/* A batch of sequences for append / decode.  All arrays are DEVICE arrays of
 * length n.  Preconditions (not checked): rows are distinct values in
 * [0, max_seqs); prefix_rows values in [0, prefix_blocks); 0 <= prefix_len[b]
 * <= prefix_cap; pos[b] >= 0.  Sequences that share a prefix block have the
 * same prefix_len; its rows are appended once (by any one of them) and only
 * read afterwards.  Paged layout: page_table is required and prefix_rows
 * unused; rows still name each sequence's slot in [0, max_seqs) (the debug
 * checks follow positions per slot); every table entry lies in [0, n_pages);
 * a page shared by several sequences holds the same prefix tokens for each,
 * is appended once and only read afterwards; pages of different sequences'
 * windows are distinct. */
typedef struct {
    int32_t n;                  /* number of sequences in the call, 1..max_seqs */
    const int32_t* rows;        /* device: window block (cache row) of each sequence */
    const int32_t* prefix_len;  /* device: P of each sequence */
    const int64_t* pos;         /* device: position of the first new token /
                                   of the query (see each call) */
    const int32_t* prefix_rows; /* device: prefix block of each sequence, or NULL:
                                   prefix block = rows[b] (requires prefix_blocks
                                   == max_seqs) */
    const int32_t* page_table;  /* device [n][prefix_cap / page_size + W / page_size]:
                                   paged layout only (else NULL) */
} ps_seq_batch;

/* Bytes of device memory a cache with this shape needs (K and V for every
 * layer, plus the decode split-K workspace).  0 if the descriptor is invalid. */
size_t ps_cache_bytes(const ps_cache_desc* desc);

/* Carve `dev_mem` (device, >= ps_cache_bytes(desc) bytes, 256-byte aligned,
 * owned by the caller and kept alive until ps_cache_destroy) into the cache
 * regions, clear the workspace counters with a kernel on `stream`, and return
 * a handle in *out.  K/V slots are NOT cleared: a slot is read only after the
 * position it holds was appended.
 * Errors: PS_ERR_INVALID (NULL, bad shape, misaligned), PS_ERR_UNSUPPORTED
 * (head_dim or dtype), PS_ERR_CAPACITY (bytes too small), PS_ERR_HIP. */
int ps_cache_create(const ps_cache_desc* desc, void* dev_mem, size_t bytes, void* stream,
                    ps_cache** out);

/* Free the host handle.  The device buffer stays the caller's.  NULL is a no-op. */
int ps_cache_destroy(ps_cache* cache);

/* Device addresses of layer `layer`'s K and V page pools in the paged layout:
 * [n_pages][n_kv_heads][page_size][head_dim] (cache dtype); slot s of a page
 * holds the prefix or ring slot the page table assigns it.  Errors:
 * PS_ERR_INVALID (NULL, layer out of range), PS_ERR_UNSUPPORTED (block
 * layout). */
int ps_cache_pages(const ps_cache* cache, int32_t layer, void** k_pages, void** v_pages);

/* Device addresses of layer `layer`'s K and V pools.  Layouts (cache dtype):
 *   prefix pools  [prefix_blocks][n_kv_heads][prefix_cap][head_dim]
 *   window pools  [max_seqs][n_kv_heads][window][head_dim]
 * Slot s of a prefix block holds prefix position s; slot r of a window block
 * holds the token at the position p >= P with (p - P) mod W == r that was
 * appended last.  For inspection and snapshot / restore (a plain device copy
 * of the whole buffer restores a cache).  Errors: PS_ERR_INVALID,
 * PS_ERR_UNSUPPORTED (paged layout: see ps_cache_pages). */
int ps_cache_blocks(const ps_cache* cache, int32_t layer, void** k_prefix, void** v_prefix,
                    void** k_window, void** v_window);

/* Debug checks of the device-resident arguments (off by default).  While
 * they are on, every call on the cache (append, decode, rerotate, cache-mode
 * prefill) first runs a one-workgroup check kernel on the same stream, which
 * ORs a bit per violated precondition into a flag word kept in the cache
 * buffer; every kernel of the call, and of any later call, does nothing while
 * the word is set, so a bad batch never touches the cache.  The word stays set
 * until ps_cache_check_flags clears it.  Positions are followed per (layer,
 * row): an append must start where the row's last append ended (or at 0,
 * which starts a new sequence in the row), a decode query must sit at the
 * last appended position (ps_decode_attn) or at the next one
 * (ps_decode_step), and a cache-mode chunk must start at the next one. */
enum ps_check_flag {
    PS_CHECK_ROW = 1u << 0,            /* a window block (row) outside [0, max_seqs) */
    PS_CHECK_DUPLICATE_ROW = 1u << 1,  /* two sequences of one call on the same row */
    PS_CHECK_PREFIX_BLOCK = 1u << 2,   /* a prefix block outside [0, prefix_blocks) */
    PS_CHECK_PREFIX_LEN = 1u << 3,     /* a prefix length outside [0, prefix_cap] */
    PS_CHECK_POSITION = 1u << 4,       /* a position below 0, or one whose call
                                          reaches past 2^62 */
    PS_CHECK_SEQUENCE = 1u << 5,       /* a position that does not continue its row */
    PS_CHECK_SHARED_PREFIX = 1u << 6,  /* one prefix block with two prefix lengths */
    PS_CHECK_PAGE = 1u << 7            /* a page table entry outside [0, n_pages) */
};

/* Turn the checks on (on != 0) or off.  Errors: PS_ERR_INVALID (NULL). */
int ps_cache_set_checks(ps_cache* cache, int32_t on);

/* Wait for `stream`, then return the flag word in *flags (host) and, if clear
 * != 0, reset it to 0 (with a kernel on `stream`, waited for).  Errors:
 * PS_ERR_INVALID (NULL), PS_ERR_HIP. */
int ps_cache_check_flags(ps_cache* cache, uint32_t* flags, int32_t clear, void* stream);

/* Split-K granularity of decode: rows (keys) handled per workgroup.  0 picks
 * automatically (default: the largest size whose launch has at least 160
 * workgroups); otherwise one of 16, 32, 64, 128, 192, 256, 512 for bf16
 * head_dim 128 and fp32 head_dim 64 (the same sizes times 2 for bf16
 * head_dim 64; 16, 32, 64, 96, 128, 256 for fp32 head_dim 128).  Errors: PS_ERR_INVALID (NULL, negative),
 * PS_ERR_UNSUPPORTED (a size the kernel is not built for). */
int ps_cache_set_decode_split(ps_cache* cache, int32_t rows_per_split);

/* Decode phase trace, a profiling aid (off by default).  With dev_buf
 * non-NULL every later decode call on the cache (ps_decode_attn,
 * ps_decode_step) runs the same decode kernel, at its split size and
 * without the non-temporal hint, with thread 0 of each workgroup writing
 * s_memrealtime stamps (100 MHz) at eight points: entry, sequence metadata
 * in, K rows in and scored, V rows summed, waves combined, partial stored and
 * acknowledged, arrival counted, merge done (the last point is 0 for a
 * workgroup that did not merge).  The k-th traced call (counted from this
 * call) writes slot k mod n_launches of dev_buf, a device array
 * [n_launches][max_wg][8] of uint64 the caller owns; a captured graph keeps
 * the slot each call had at capture.  The stamps observe the kernel and skip
 * none of its work; the waits they need cost a little time.  NULL turns the
 * trace off.  While it is on, decode calls return PS_ERR_UNSUPPORTED for
 * shapes other than bf16, head_dim 128, GQA 1, 2 or 4 with a split of 192
 * or 256 rows (set, or chosen automatically), or a launch of more than
 * max_wg workgroups.
 * Errors: PS_ERR_INVALID (NULL cache; n_launches or max_wg < 1 with a
 * buffer). */
int ps_cache_set_decode_trace(ps_cache* cache, uint64_t* dev_buf, int32_t n_launches, int32_t max_wg);

/* Append n_new consecutive tokens per sequence to layer `layer`: token t of
 * sequence b has position pos[b] + t.  A position p < P goes to slot p of the
 * sequence's prefix block; p >= P goes to slot (p - P) mod W of its window
 * block, overwriting the token at p - W, which
 * is exactly the token that falls out of the window (positional eviction:
 * njhaofan.com section above; papers.ananclaw.com "被丢弃的中间区").  When more
 * than W ring-bound tokens arrive in one call only the last W are written, so
 * the resulting cache is bit-identical to n_new single-token appends.
 *   k_new, v_new: device [n][n_new][n_kv_heads][head_dim], pre-rotated keys.
 * Preconditions: positions of a sequence are appended in increasing order and
 * a decode/prefill query at position i sees the cache as left by appending
 * every position < i (Continue PE: nothing is ever re-encoded); the debug
 * checks (ps_cache_set_checks) verify them on the device.
 * Errors: PS_ERR_INVALID, PS_ERR_HIP. */
int ps_kv_append_evict(ps_cache* cache, int32_t layer, const ps_seq_batch* batch,
                       int32_t n_new, const void* k_new, const void* v_new, void* stream);

/* One decode query per sequence at position i = pos[b], which must already be
 * appended: GQA attention over the visible keys of i, which are exactly the
 * retained slots (prefix-block slots [0, min(P, i+1)) and the window-block
 * slots of positions (i - W, i]).  Query head h reads kv head
 * floor(h * Hkv / Hq).
 *   q:   device [n][n_q_heads][head_dim]
 *   out: device [n][n_q_heads][head_dim]  (cache dtype; normalised output)
 *   lse: device [n][n_q_heads] float, natural-log log-sum-exp of the scaled
 *        scores, or NULL
 *   scale: multiplier of q.k (1/sqrt(head_dim) for standard attention)
 * Split-K over the keys with a log-sum-exp combine done by the last finishing
 * workgroup of each (sequence, kv head).  Errors: PS_ERR_INVALID, PS_ERR_HIP. */
int ps_decode_attn(ps_cache* cache, int32_t layer, const ps_seq_batch* batch, const void* q,
                   void* out, float* lse, float scale, void* stream);

/* Fused decode step: append the token at position pos[b] (k_new, v_new: device
 * [n][n_kv_heads][head_dim]) and attend from it in one launch.  Same cache
 * state and same result as ps_kv_append_evict(n_new = 1) followed by
 * ps_decode_attn.  Errors: PS_ERR_INVALID, PS_ERR_HIP. */
int ps_decode_step(ps_cache* cache, int32_t layer, const ps_seq_batch* batch, const void* q,
                   const void* k_new, const void* v_new, void* out, float* lse, float scale,
                   void* stream);

/* ps_kv_append_evict with the rotary position encoding of the new keys fused
 * in: k_new arrives unrotated and each key is turned at its own position
 * (Continue PE -- position IDs keep climbing, so a key is encoded once, on
 * its way into the cache, and never again: agihunt.info summary, paragraph on
 * position encodings).  The half-split pair (x_e, x_{e+d/2}), e < d/2, turns
 * by pos * rope_base^(-2e/d); the angle is formed in double precision and
 * reduced before its fp32 sine and cosine are taken, the turn runs in fp32
 * with one rounding to the cache type.  V rows are copied unchanged.  Slots,
 * eviction, layouts and errors as ps_kv_append_evict, plus PS_ERR_INVALID for
 * rope_base <= 1 or not finite. */
int ps_kv_append_rope(ps_cache* cache, int32_t layer, const ps_seq_batch* batch, int32_t n_new,
                      const void* k_new, const void* v_new, float rope_base, void* stream);

/* Reset PE support: turn the rotary encoding of every key the window holds
 * by delta positions, in place.  Under Reset PE the retained tokens are given
 * new positions and their rotary-encoded keys are recomputed (agihunt.info
 * summary, paragraph on position encodings; njhaofan.com article, passage
 * comparing ContinuePE and ResetPE, which the pages reject as the costlier
 * option).  Rotary encoding turns each half-split pair (x_e, x_{e+d/2}),
 * e < d/2, by pos * rope_base^(-2e/d); turns compose, so a key stored rotated
 * at position p becomes the key rotated at p + delta.  For sequence s the
 * window is the ring rows holding the tokens [max(P_s, pos_s - W), pos_s)
 * (the cache as left by appending every token < pos_s; batch->pos is read as
 * that bound, batch->prefix_len as P_s).  Prefix rows and V rows are not
 * touched.  The turn is computed from double-precision sines and cosines and
 * applied in fp32 with one rounding per call, so repeated calls on a bf16
 * cache accumulate rounding like any in-place update.
 *
 * Errors: PS_ERR_INVALID (NULL cache or batch, layer out of range, rope_base
 * <= 1 or not finite, n outside [1, max_seqs]), PS_ERR_HIP. */
int ps_kv_rerotate(ps_cache* cache, int32_t layer, const ps_seq_batch* batch, int64_t delta, float rope_base,
                   void* stream);

/* Chunked prefill (cache != NULL) or trainer-side forward (cache == NULL).
 *
 * Every sequence of the batch has the same prefix length P and its chunk
 * occupies positions start_pos .. start_pos + seq_len - 1, unless `starts` is
 * given (ragged chunks of a continuous batch): then sequence b's chunk starts
 * at starts[b] and its prefix length is prefix_lens[b] (or P when
 * prefix_lens is NULL).  Device-side preconditions of ragged chunks (not
 * checked): 0 <= starts[b] <= 2^62 - seq_len, 0 <= prefix_lens[b] (<=
 * prefix_cap in cache mode).  Positions may take any value up to 2^62 (the
 * chunk of a trace of any length): the kernels handle a chunk's positions in
 * 32 bits in a frame of its own (counted from the chunk start in trainer
 * mode; positions past the prefix moved down together in cache mode), which
 * changes no visibility decision.  Query i of the chunk attends to the visible
 * keys among
 *   - the cached prefix rows [0, min(P, start_pos))          (cache mode)
 *   - the cached ring rows holding positions
 *     [max(P, start_pos - W), start_pos)                      (cache mode)
 *   - the chunk's own keys start_pos .. i.
 * Cache mode reads the cache as left by appending every position < start_pos
 * and does NOT append the chunk: commit it afterwards with
 * ps_kv_append_evict(n_new = seq_len).  Trainer mode sees only the chunk
 * (start_pos is normally 0: the prefix is the first P tokens of the slice,
 * and the trainer receives the last 4W tokens of a rollout -- njhaofan.com
 * section "无需训练最高提速3倍，RL扩展到10万Token"; agihunt.info, paragraph on
 * truncated backprop).
 *
 * Key tiles wholly outside prefix and window are skipped without a load, tiles
 * entirely visible run unmasked, and only tiles that straddle the boundary
 * apply an elementwise mask (the two-level filtering of the pages' Hopper
 * kernel: agihunt.info paragraph on the FlashAttention kernel; njhaofan.com
 * section "PrefixSliding如何丢掉中间Token？").  bf16 uses MFMA for Q.K^T and P.V. */
typedef struct {
    ps_cache* cache;        /* NULL: trainer mode */
    int32_t layer;          /* cache mode only */
    int32_t batch;          /* B >= 1 (<= max_seqs in cache mode) */
    int32_t seq_len;        /* T >= 0 tokens per sequence (0: nothing to do) */
    int32_t n_q_heads;      /* trainer mode; must match the cache in cache mode */
    int32_t n_kv_heads;     /* trainer mode; must match the cache in cache mode */
    int32_t head_dim;       /* trainer mode; must match the cache in cache mode */
    int32_t dtype;          /* trainer mode; must match the cache in cache mode */
    int64_t start_pos;      /* position of chunk token 0, >= 0 */
    int64_t prefix_len;     /* P >= 0 (<= prefix_cap in cache mode) */
    int64_t window;         /* W >= 1 (must equal the cache's W in cache mode) */
    const int32_t* rows;    /* device [B] window blocks (cache mode), else NULL */
    const void* q;          /* device [B][T][n_q_heads][head_dim] */
    const void* k;          /* device [B][T][n_kv_heads][head_dim] */
    const void* v;          /* device [B][T][n_kv_heads][head_dim] */
    void* out;              /* device [B][T][n_q_heads][head_dim] */
    float* lse;             /* device [B][T][n_q_heads] natural log, or NULL */
    float scale;            /* multiplier of q.k, > 0 */
    const int32_t* prefix_rows; /* device [B] prefix blocks (cache mode), or NULL:
                                   prefix block = rows[b] (requires prefix_blocks
                                   == max_seqs) */
    const int64_t* starts;      /* device [B] chunk start of each sequence (ragged
                                   chunks), or NULL: start_pos for every sequence */
    const int32_t* prefix_lens; /* device [B] prefix length of each sequence, or
                                   NULL: prefix_len; only together with starts */
    const int32_t* page_table;  /* paged cache: device [B][pages per sequence] page
                                   table (see ps_seq_batch), else NULL */
    uint64_t* trace;            /* NULL, or a phase trace (a profiling aid): a
                                   device array [2][8] of uint64 the caller owns
                                   and clears; see below */
} ps_prefill_args;

/* Prefill phase trace.  With args->trace non-NULL a call that runs on the
 * MFMA kernel (bf16, head_dim 128) runs a copy of it that reads the shader
 * clock (s_memtime) around each phase of its tile loop and adds, per wave,
 * the cycles spent into trace[grp][k], grp 0 for waves 0-3 (they stage the
 * key tiles), 1 for waves 4-7:
 *   k = 0 scores (S^T = K Q^T), 1 mask and row maximum, 2 exponentials and
 *   P.V, 3 wait for the next tile's loads, 4 barrier, 5 issuing the next
 *   tile's loads, 6 tiles processed, 7 cycles from kernel entry to the end
 *   of the tile loop.
 * The traced copy computes the same results (bit for bit); the clock reads
 * and their waits cost a little time.  Other shapes ignore the field. */

/* bf16 with head_dim 128 and a GQA group of 1 to 8 runs on the MFMA kernel
 * (groups 3 and 5-7 on the layout of the next power of two, the missing
 * heads' rows idle); every other supported shape (bf16 head_dim 64, groups
 * above 8, fp32) runs on a plain kernel with fp32 arithmetic: same results
 * within the dtype's tolerance, far slower.
 * Errors of ps_prefill_attn: PS_ERR_INVALID (NULL or inconsistent arguments,
 * scale <= 0 or not finite), PS_ERR_UNSUPPORTED (head_dim other than 64 or
 * 128, a dtype other than bf16 / fp32, start_pos + seq_len above 2^62, and
 * -- the kernels' 32-bit frame -- in cache mode prefix_cap + W + seq_len
 * >= 2^31 for ragged chunks, min(start_pos, P + W) + seq_len >= 2^31 for
 * uniform ones),
 * PS_ERR_HIP. */

int ps_prefill_attn(const ps_prefill_args* args, void* stream);

/* Trainer-side backward of ps_prefill_attn in trainer mode (cache == NULL):
 * the gradients dq, dk, dv of the masked attention given the upstream
 * gradient dout.  The trainer backpropagates through the last windows of a
 * rollout (agihunt.info summary, paragraph on RL; njhaofan.com article,
 * passage on truncated backpropagation); the pages give no formula, this is
 * the derivative of the forward: with P the softmax over the visible keys,
 * Delta_i = sum_d dout[i][d] out[i][d] and dS = P (dout V^T - Delta),
 *   dq = scale dS K,   dk = scale dS^T Q,   dv = P^T dout,
 * summed over the query heads of each kv head for dk and dv.  Visibility,
 * positions and tile skipping are those of the forward.
 *
 * Layouts as in ps_prefill_attn trainer mode: q, out, dout, dq
 * [B][T][n_q_heads][head_dim]; k, v, dk, dv [B][T][n_kv_heads][head_dim];
 * lse [B][T][n_q_heads] natural log, as written by the forward of the same
 * q, k, v (P is rebuilt from it); delta [B][T][n_q_heads] fp32 is a
 * caller-owned workspace the call overwrites.  Every pointer is device memory
 * the caller owns; dq, dk and dv are overwritten (no accumulation into them).
 * bf16 only, head_dim 128, GQA group 1 to 8.  Stream-ordered: Delta, then
 * dk/dv, then dq, on the given stream.
 *
 * Stored dS (optional): with ds_work non-NULL the dk/dv pass also writes dS
 * (bf16, per query head) into that caller-owned device workspace, and dq is
 * taken from it (dq = scale dS K) instead of rebuilding S and dP a second
 * time: two of the seven products of the backward go away for HBM traffic of
 * twice the workspace.  The workspace holds, for each (sequence, query head,
 * block of 32 positions), the 32 x 32 tiles of the key blocks those rows can
 * see: ps_prefill_bwd_ds_bytes gives its size, about
 * batch * n_q_heads * seq_len * (min(window, seq_len) + min(P', seq_len) + 64) * 2
 * bytes with P' the prefix keys inside the chunk.  dk and dv are the same
 * either way, and dq is formed from the same bf16 dS in the same order.  The
 * workspace's contents on return are unspecified; nothing needs clearing
 * before a call.  With ds_work NULL
 * (ds_work_bytes ignored), or when ps_prefill_bwd_ds_bytes gives 0 (GQA
 * groups of more than 4 query heads, where storing costs more than it saves,
 * or one kv head's share of the workspace would reach 2^31 bytes), S and dP
 * are rebuilt and ds_work is not touched.
 *
 * Errors: PS_ERR_INVALID (NULL pointer, batch < 1, seq_len < 0, start_pos < 0,
 * prefix_len < 0, window < 1, n_q_heads not a multiple of n_kv_heads, scale
 * <= 0 or not finite), PS_ERR_UNSUPPORTED (dtype other than bf16, head_dim
 * other than 128, another GQA group, start_pos + seq_len above 2^62),
 * PS_ERR_CAPACITY (ds_work non-NULL with ds_work_bytes below
 * ps_prefill_bwd_ds_bytes), PS_ERR_HIP. */
typedef struct {
    int32_t batch;          /* B >= 1 */
    int32_t seq_len;        /* T >= 0 (0: nothing to do) */
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;       /* 128 */
    int32_t dtype;          /* PS_BF16 */
    int64_t start_pos;      /* position of token 0, >= 0 */
    int64_t prefix_len;     /* P >= 0 */
    int64_t window;         /* W >= 1 */
    const void* q;
    const void* k;
    const void* v;
    const void* out;        /* forward output */
    const float* lse;       /* forward log-sum-exp */
    const void* dout;       /* gradient of out */
    void* dq;
    void* dk;
    void* dv;
    float* delta;           /* workspace [B][T][n_q_heads] fp32 */
    float scale;            /* the forward's multiplier of q.k, > 0 */
    void* ds_work;          /* optional stored-dS workspace (device), or NULL */
    int64_t ds_work_bytes;  /* its size in bytes */
} ps_prefill_bwd_args;

int ps_prefill_attn_bwd(const ps_prefill_bwd_args* args, void* stream);

/* Bytes of the stored-dS workspace ps_prefill_attn_bwd takes for these
 * arguments (only batch, seq_len, n_q_heads, n_kv_heads, start_pos,
 * prefix_len and window are read; no device call), written to *bytes: 0 when
 * seq_len is 0 or the stored-dS path does not apply (then ds_work is unused).
 * Errors: PS_ERR_INVALID (args or bytes NULL, batch < 1, seq_len < 0,
 * start_pos < 0, prefix_len < 0, window < 1, n_q_heads or n_kv_heads < 1,
 * n_q_heads not a multiple of n_kv_heads), PS_ERR_UNSUPPORTED
 * (start_pos + seq_len above 2^62). */
int ps_prefill_bwd_ds_bytes(const ps_prefill_bwd_args* args, int64_t* bytes);

/* The same trainer backward for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation): identical arguments and results, except that args->delta must
 * be NULL -- the Delta rows go to a device array the library owns, of
 * PS_BWD_NOALLOC_MAX_ROWS fp32 rows (16 MiB), one per GPU, held until the
 * process ends.  The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks up that
 * device's copy of the array.  Every call on one GPU shares the array, and
 * each call overwrites the rows it uses before reading them, so nothing
 * carries over from an earlier call; calls that overlap on one GPU (streams
 * not ordered with each other) race on it.
 * Errors: those of ps_prefill_attn_bwd, PS_ERR_INVALID for a non-NULL delta,
 * PS_ERR_CAPACITY when batch * seq_len * n_q_heads exceeds
 * PS_BWD_NOALLOC_MAX_ROWS, PS_ERR_HIP when the array cannot be found. */
#define PS_BWD_NOALLOC_MAX_ROWS 4194304
int ps_prefill_attn_bwd_noalloc(const ps_prefill_bwd_args* args, void* stream);

/* Host-side pool of block indices with reference counts: the bookkeeping of
 * the block table.  A serving loop keeps one pool for window blocks (cache
 * rows, size max_seqs) and one for prefix blocks (size prefix_blocks); a
 * sequence takes a window block of its own and a prefix block that rollouts
 * of the same prompt share, each holding one reference (the PREFIX block is
 * read-only once prefilled, papers.ananclaw.com explainer, section
 * "核心方法"; the policy combines with paged memory management, same page,
 * section "工程启发").  A block returns to the free list when its last
 * reference is released; the cache bytes are not touched.  Blocks are handed
 * out lowest index first.  A pool is plain host memory, not thread-safe:
 * callers that share one across threads serialise the calls.  Errors:
 * PS_ERR_INVALID (NULL, index out of range, releasing or retaining a free
 * block), PS_ERR_CAPACITY (no free block). */
typedef struct ps_block_pool ps_block_pool;
int ps_block_pool_create(int32_t n_blocks, ps_block_pool** out);   /* n_blocks >= 1 */
int ps_block_pool_destroy(ps_block_pool* pool);                     /* NULL is a no-op */
int ps_block_alloc(ps_block_pool* pool, int32_t* block);            /* one reference */
int ps_block_retain(ps_block_pool* pool, int32_t block);            /* one more reference */
int ps_block_release(ps_block_pool* pool, int32_t block);           /* one less; freed at zero */
int ps_block_refcount(const ps_block_pool* pool, int32_t block, int32_t* count);
int ps_block_free_count(const ps_block_pool* pool, int32_t* count);

/* Class of a (query tile, key tile) pair, query positions [i0, i1] and key
 * positions [j0, j1] (both non-empty, contiguous): 0 SKIP (no visible pair),
 * 1 FULL (every pair visible), 2 MASKED.  The same closed form the prefill
 * kernel uses on the device; exported for host-side planning and tests.
 * Returns -1 for an empty range, P < 0 or W < 1. */
int ps_tile_class(int64_t i0, int64_t i1, int64_t j0, int64_t j1, int64_t P, int64_t W);

/* Static description of a status code. */
const char* ps_status_str(int status);

/* Library version, e.g. "0.1.0". */
const char* ps_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PREFIX_SLIDING_PS_H */
