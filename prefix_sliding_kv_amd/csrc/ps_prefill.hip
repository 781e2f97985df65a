// Chunked-prefill / trainer-side forward for Prefix Sliding on gfx950.
//
// Query i sees key j iff j <= i and (j < P or j > i - W).  Keys come in at
// most four runs of contiguous positions and contiguous storage: the cached
// prefix, the two halves of the ring (split where it wraps), and the chunk's
// own keys.  For a query tile with positions [i0, i1] only two intervals of a
// run can hold visible keys: positions below min(P, i1+1), and positions in
// (i0 - W, i1].  Key tiles outside both are never visited (SKIP costs
// nothing); a visited tile is FULL when every (query, key) pair is visible and
// runs without any mask, and MASKED otherwise, where the rule is applied per
// element.  This is the two-level filtering the pages describe for their
// Hopper FlashAttention kernel (agihunt.info summary, paragraph on the
// FlashAttention kernel; njhaofan.com article, section
// "PrefixSliding如何丢掉中间Token？"), rebuilt for CDNA4.
//
// bf16 path (head_dim 128): a workgroup of 8 waves owns 256 query rows, the
// G heads of one GQA group stacked over 256/G positions, so every K/V tile
// staged in LDS serves all heads that share it.  Per 128-key tile each wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (a lane then holds 16
// scores of a single query per 32-key block, so the online softmax needs one
// cross-lane step), and O^T += V^T P^T with the same instruction, reading the
// V^T operand from the row-major V tile with the transposing LDS read
// (ds_read_b64_tr_b16); the exponentials of each 16-key step are made right
// before its MFMAs.  K and V tiles go from global memory straight into two
// LDS stages (buffer_load ... lds), the next tile loading while the current
// one is computed, one barrier per tile.  The tile walk is kept in scalar
// registers and touches LDS only at range boundaries.  GQA groups 3 and 5-7
// run on the 4- and 8-head layouts with the missing heads' rows idle.  Plain
// path: one thread per query row with 64-key tiles, the same walk and
// classification, fp32 arithmetic; it serves fp32 inputs and the bf16 shapes
// the MFMA kernel is not built for (head_dim 64, GQA groups above 8).
//
// Trainer backward (bf16, head_dim 128): Delta = rowsum(dO * O); dK/dV with
// one workgroup per 256-key block walking the query sub-tiles that see it;
// dQ either in the forward's layout, rebuilding S and dP, or -- with the
// caller's stored-dS workspace -- from the dS the dK/dV kernel stored.
#include <mutex>

#include "ps_internal.h"

namespace ps {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2eF = 1.4426950408889634f;
constexpr int kBN = 64;  // keys per tile of the plain kernel

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

struct alignas(16) Vec16 {
    uint32_t w[4];
};
struct alignas(8) Vec8 {
    uint32_t w[2];
};

// Ranges of key tiles of one run that may hold keys visible to queries [i0, i1].
struct TileWalk {
    int n_ranges;
    int run[2 * kMaxRuns];
    int begin[2 * kMaxRuns];
    int end[2 * kMaxRuns];
};

// Geometry of one key run resolved for one (sequence, kv head): the address
// of its row 0, the byte stride between rows, its first position and length.
// Kept in LDS so the tile loop reads it with a dynamic index instead of
// holding every run of the kernel arguments in scalar registers.
struct RunView {
    const char* k;
    const char* v;
    int64_t pos0;
    int n;
    int row_bytes;
    // paged runs: page_shift >= 0; row r is slot first_slot + r of the
    // region whose pages are table entries page_col, page_col + 1, ...
    int page_shift, page_col, first_slot, page_rows;
};

// Pages a sequence's page table may hold (the host enforces it); the bf16
// and plain kernels keep the sequence's table row in LDS.
constexpr int kMaxPagesPerSeq = 256;

// Fill a run view for sequence b, kv head g (element size esz).
__device__ inline void make_view(RunView& v, const KeyRun& run, int b, int g, int hkv, int esz) {
    if (run.pages) {
        const int64_t head_el = (int64_t)g * run.head_stride;
        v.k = static_cast<const char*>(run.k) + head_el * esz;
        v.v = static_cast<const char*>(run.v) + head_el * esz;
        v.page_shift = run.page_shift;
        v.page_col = run.page_col;
        v.first_slot = (int)run.first_slot;
        v.page_rows = hkv << run.page_shift;
    } else {
        const int64_t seq = run.rows ? (int64_t)run.rows[b] : (int64_t)b;
        const int64_t base_el = seq * run.seq_stride + (int64_t)g * run.head_stride;
        v.k = static_cast<const char*>(run.k) + base_el * esz;
        v.v = static_cast<const char*>(run.v) + base_el * esz;
        v.page_shift = -1;
        v.page_col = v.first_slot = v.page_rows = 0;
    }
    v.pos0 = run.pos0;
    v.n = (int)run.n;
    v.row_bytes = (int)(run.row_stride * esz);
}

// Byte offset from a view's base of rows [row0, row0 + n) of its run, which
// lie inside one page when the run is paged (table: the sequence's page
// table row in LDS).
__device__ inline int64_t view_row_offset(int shift, int page_col, int first_slot, int page_rows, int rs,
                                          const int32_t* table, int row0) {
    if (shift < 0) return (int64_t)row0 * rs;
    const int slot = first_slot + row0;
    const int64_t page = table[page_col + (slot >> shift)];
    return (page * page_rows + (slot & ((1 << shift) - 1))) * (int64_t)rs;
}

__device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

// v_exp_f32 without the denormal-range fix-up of exp2f: results below 2^-126
// flush to zero, which is below the rounding error of any softmax row sum
// (every row has a term equal to 1 at its running reference).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int TILE>
__device__ inline void plan_walk(const KeyRun* runs, int n_runs, int64_t P, int64_t W, int64_t i0, int64_t i1,
                                 TileWalk& w) {
    w.n_ranges = 0;
    for (int r = 0; r < n_runs; ++r) {
        const KeyRun& run = runs[r];
        const int64_t n = run.n;
        if (n <= 0) continue;
        // prefix part: positions < min(P, i1 + 1)
        const int64_t hiA = clamp64((P < i1 + 1 ? P : i1 + 1) - run.pos0, 0, n);
        // window part: positions in [i0 - W + 1, i1]
        const int64_t loB = clamp64(i0 - W + 1 - run.pos0, 0, n);
        const int64_t hiB = clamp64(i1 + 1 - run.pos0, 0, n);
        const int endA = (int)((hiA + TILE - 1) / TILE);
        int begB = (int)(loB / TILE);
        const int endB = hiB > loB ? (int)((hiB + TILE - 1) / TILE) : 0;
        if (endA > 0) {
            w.run[w.n_ranges] = r;
            w.begin[w.n_ranges] = 0;
            w.end[w.n_ranges] = endA;
            ++w.n_ranges;
        }
        if (begB < endA) begB = endA;
        if (endB > begB) {
            w.run[w.n_ranges] = r;
            w.begin[w.n_ranges] = begB;
            w.end[w.n_ranges] = endB;
            ++w.n_ranges;
        }
    }
}

// ----------------------------------------------------------------- bf16 MFMA
constexpr int kXcds = 8;

// Bijection from the dispatch-order id to a work index such that the ids an
// XCD receives (id % 8 == x) map to one contiguous block of work indices.
__device__ inline int xcd_remap(int id, int n) {
    const int q = n / kXcds, r = n % kXcds;
    const int x = id % kXcds, slot = id / kXcds;
    return x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

constexpr int kWaves = 8;                // waves per workgroup (2 per SIMD, one workgroup per CU)
constexpr int kThreads = kWaves * 64;
constexpr int kBNB = 128;                // keys per tile of the bf16 kernel
constexpr int kStages = 2;               // LDS ring of key tiles
constexpr int kRowBytes = 128 * 2;       // one K or V row (head_dim 128, bf16)
constexpr int kTileBytes = kBNB * kRowBytes;
constexpr int kStageBytes = 2 * kTileBytes;  // K tile then V tile

// Both tiles are row-major (row = key, 256 bytes = all 64 LDS banks once)
// with 16-byte chunks xor-swizzled by row so that the operand reads hit every
// bank once per cycle:
//  K: chunk c of row r at c ^ (r & 15): a 16-byte read serves 16 lanes per
//     cycle, 16 consecutive rows at the same logical chunk;
//  V: chunk c of row r at c ^ 4(r & 3): an 8-byte transposing read serves 32
//     lanes per cycle, rows 4h .. 4h + 3 at logical chunks 4m .. 4m + 3, and
//     4(r & 3) spreads those 16 chunks over 16 distinct bank quads.  (With
//     c ^ 2(r & 3) the two 16-lane halves land on the same 32 banks: a 2-way
//     conflict on every V^T read.)
__device__ inline int k_chunk_swz(int row) { return row & 15; }
__device__ inline int v_chunk_swz(int row) { return 4 * (row & 3); }

// 32-bit LDS address of a pointer into shared memory.
__device__ inline uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Buffer resource (V#) over [base, base + bytes), as four uniform words:
// loads at offsets past the end return zero, so partial tiles need no
// per-lane checks.
__device__ inline i32x4 rsrc_words(const void* base, int bytes) {
    i32x4 r;
    r[0] = (int)(uint32_t)(uintptr_t)base;
    r[1] = (int)(((uintptr_t)base >> 32) & 0xFFFF);
    r[2] = bytes;
    r[3] = 0x00020000;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
    return r;
}

// Direct-to-LDS loads written as asm: 16 (or 4) bytes per lane from
// rsrc + voff land at LDS address m0 + 16 (4) * lane.  The compiler does not
// see them, so it does not make every later LDS read wait for them (with the
// builtin it waits for all loads in flight before the first read of any
// buffer); the kernels order them against the reads of their buffer
// themselves (vmcnt before the barrier that hands the buffer over).  The
// hardware counter is in order, so the compiler's own vmcnt waits only wait
// longer for the loads it does not see.
__device__ inline void dma16_asm(i32x4 rsrc, int voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ inline void dma4_asm(i32x4 rsrc, int voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Bits [lo, hi) of a 32-bit word, with lo and hi clamped to [0, 32].
__device__ inline uint32_t range_bits(int lo, int hi) {
    lo = lo < 0 ? 0 : (lo > 32 ? 32 : lo);
    hi = hi < 0 ? 0 : (hi > 32 ? 32 : hi);
    if (hi <= lo) return 0u;
    return (uint32_t)((((uint64_t)1 << hi) - 1) ^ (((uint64_t)1 << lo) - 1));
}

__device__ inline int uniform_int(int x) { return __builtin_amdgcn_readfirstlane(x); }
// A uniform read of device memory the kernel does not write, through the
// scalar data cache (s_load).
template <typename V>
__device__ inline V scalar_load(const V* ptr) {
    return *reinterpret_cast<const __attribute__((address_space(4))) V*>(reinterpret_cast<uintptr_t>(ptr));
}
__device__ inline const char* uniform_ptr(const char* p) {
    const uint64_t u = (uint64_t)p;
    return (const char*)(((uint64_t)(uint32_t)uniform_int((int)(u >> 32)) << 32) | (uint32_t)uniform_int((int)(uint32_t)u));
}
__device__ inline int64_t uniform_i64(int64_t x) {
    const uint64_t u = (uint64_t)x;
    return (int64_t)(((uint64_t)(uint32_t)uniform_int((int)(u >> 32)) << 32) | (uint32_t)uniform_int((int)(uint32_t)u));
}

// Workgroup barrier between key tiles.  Each wave has already waited for its
// own direct-to-LDS loads of the next tile (vmcnt) and for its LDS reads of
// the current one (their results are consumed), so a bare s_barrier orders
// everything that matters; __syncthreads would add a release fence that
// waits for every direct-to-LDS load still in flight, prefetches included.
__device__ inline void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Workgroup barrier for data in LDS: every wave's LDS operations (and scalar
// loads) have completed; vector memory loads still in flight stay in flight
// (__syncthreads would wait for those as well).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A position in the tile walk: range r, tile t of its run, end of the range,
// and the run's geometry.  Everything is uniform across a wave and lives in
// scalar registers; the walk and run tables in LDS are read only when the
// cursor enters a new range.
struct Cursor {
    int r, t, end;
    const char* k;
    const char* v;
    int64_t pos0;
    int n, rs;
    int shift, page_col, first_slot, page_rows;  // paged runs (shift >= 0)
};

__device__ inline void cursor_enter(Cursor& c, int r, const TileWalk& w, const RunView* views) {
    c.r = r;
    c.t = uniform_int(w.begin[r]);
    c.end = uniform_int(w.end[r]);
    const RunView& v = views[uniform_int(w.run[r])];
    c.k = uniform_ptr(v.k);
    c.v = uniform_ptr(v.v);
    c.pos0 = uniform_i64(v.pos0);
    c.n = uniform_int(v.n);
    c.rs = uniform_int(v.row_bytes);
    c.shift = uniform_int(v.page_shift);
    c.page_col = uniform_int(v.page_col);
    c.first_slot = uniform_int(v.first_slot);
    c.page_rows = uniform_int(v.page_rows);
}

// Step to the next tile; returns true when the cursor entered a new range.
__device__ inline bool cursor_next(Cursor& c, int n_ranges, const TileWalk& w, const RunView* views) {
    if (++c.t < c.end || c.r + 1 >= n_ranges) return false;
    cursor_enter(c, c.r + 1, w, views);
    return true;
}

// Per-lane byte offsets, within a tile, of this lane's 16-byte pieces of the
// direct-to-LDS loads.  Only waves 0-3 stage tiles (eight K and eight V
// instructions per wave and tile; wave w fills rows 32w .. 32w + 31): issuing
// these loads stalls a wave for a while, and waves 4-7, which share the SIMDs
// with 0-3, keep the MFMA pipes busy meanwhile.  The offsets depend on the
// run's row stride only.
constexpr int kLoadWaves = 4;
constexpr int kLoadsPerWave = kBNB / kLoadWaves / 4;  // 4-row instructions per loading wave for K (and for V)
struct LaneOffsets {
    int k[kLoadsPerWave], v[kLoadsPerWave];
};
__device__ inline void lane_offsets(LaneOffsets& o, int rs, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int row = (kBNB / kLoadWaves) * (wave & (kLoadWaves - 1)) + 4 * i + (lane >> 4);
        o.k[i] = row * rs + (((lane & 15) ^ k_chunk_swz(row)) << 4);
        o.v[i] = row * rs + (((lane & 15) ^ v_chunk_swz(row)) << 4);
    }
}

// Stage the cursor's tile: K and V go straight from global memory into LDS
// (buffer_load ... lds: 16 bytes per lane, landing at LDS base + lane * 16;
// each lane loads the global chunk that belongs at its swizzled position).
// The buffer resources cover only the run's rows of this tile, so rows past
// the run's end read as zero (those keys are masked; zero V rows add nothing).
__device__ inline void load_tile_bf16(const Cursor& c, const LaneOffsets& lo, int wave, char* stage,
                                      const int32_t* table) {
    const int row0 = c.t * kBNB;
    const int nrows = c.n - row0 < kBNB ? c.n - row0 : kBNB;
    const int64_t off =
        c.shift < 0 ? (int64_t)row0 * c.rs
                    : uniform_i64(view_row_offset(c.shift, c.page_col, c.first_slot, c.page_rows, c.rs, table, row0));
    if (wave >= kLoadWaves) return;
    const i32x4 kr = rsrc_words(c.k + off, nrows * c.rs);
    const i32x4 vr = rsrc_words(c.v + off, nrows * c.rs);
    const uint32_t sb = lds_addr(stage);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int r4 = (kBNB / kLoadWaves) * wave + 4 * i;  // first of the 4 rows this instruction fills
        dma16_asm(kr, lo.k[i], sb + r4 * kRowBytes);
        dma16_asm(vr, lo.v[i], sb + kTileBytes + r4 * kRowBytes);
    }
}
constexpr int kLoadsPerTile = 2 * kLoadsPerWave;  // vector memory instructions per thread per staged tile

__device__ inline bf16x8 as_bf16x8(const Vec16& v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
    // hardware round-to-nearest-even conversion (v_cvt_pk_bf16_f32)
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 r = {(__bf16)a, (__bf16)b};
    uint32_t u;
    __builtin_memcpy(&u, &r, 4);
    return u;
}

// Sum of the 8 bf16 values of a packed P operand, in fp32 (v_dot2 with ones):
// the row sum then matches the bf16 P the P.V product uses.
__device__ inline float sum_bf16x8(const Vec16& v) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bf16x2 x;
        __builtin_memcpy(&x, &v.w[i], 4);
        acc = __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
    }
    return acc;
}

// V^T operands of k-step ST (keys 16 ST .. 16 ST + 15) for the four dim
// blocks, from the row-major V tile.  ds_read_b64_tr_b16 works on 16-lane
// groups: group lane k reads 4 bf16 at its own address and lane i of the
// group receives element i % 4 from each of group lanes i / 4, 4 + i / 4,
// 8 + i / 4 and 12 + i / 4.  Group lane k reads key row base + k / 4 at
// dims 32m + 16(q % 2) + 4(k % 4) (q = lane / 16), so lane i ends up with one
// head dim (32m + lane % 32) of four consecutive keys; the reads at rows
// +0 and +8 fill the two halves of the 8-key operand.  vaddr[m] already holds
// the swizzled LDS address of row 4h + k / 4 (h = lane / 32) for dim block m;
// the k-step and half become immediate offsets.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline void read_vt(int st, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, Vec16 (&va)[4]) {
    const uint32_t ad[4] = {a0, a1, a2, a3};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)(ad[m] + st * 16 * kRowBytes));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)(ad[m] + st * 16 * kRowBytes + 8 * kRowBytes));
        __builtin_memcpy(&va[m].w[0], &lo, 8);
        __builtin_memcpy(&va[m].w[2], &hi, 8);
    }
}

// tile_class for positions below 2^31, in 32-bit arithmetic: P and W at most
// 2^31 - 1 and i0 >= 0 keep i0 - W and i1 - W in range.
__device__ inline int tile_class32(int i0, int i1, int j0, int j1, int P, int W) {
    if (j0 > i1 || (j0 >= P && j1 <= i0 - W)) return kSkip;
    const int lo = j0 > P ? j0 : P;
    if (j1 <= i0 && (j1 < P || lo > i1 - W)) return kFull;
    return kMasked;
}

// One workgroup of 8 waves per CU owns 256 query rows: the G heads of a GQA
// group stacked over 256/G positions; wave w owns rows 32w .. 32w + 31, so
// every key tile staged in LDS serves all heads of the group.
// TRACE: the same kernel reading the shader clock around each phase of the
// tile loop (the prefill phase trace of ps.h); the results are identical.
template <int G, bool TRACE = false>
__global__ void __launch_bounds__(kThreads, 1) prefill_bf16_kernel(PrefillParams p) {
    constexpr int D = 128;
    constexpr int QP = 32 * kWaves / G;  // positions per query tile
    extern __shared__ __attribute__((aligned(16))) char smem[];
    if (p.guard && *p.guard) return;  // checks on and a check failed
    // phase cycle sums of this wave (TRACE only): scores, mask + maximum,
    // P.V, load wait, barrier, load issue
    uint32_t tr_acc[6] = {0, 0, 0, 0, 0, 0};
    uint64_t tr_last = 0, tr_entry = 0;
    auto tr_mark = [&](int k) __attribute__((always_inline)) {
        if constexpr (TRACE) {
            const uint64_t t = __builtin_amdgcn_s_memtime();
            if (k >= 0) tr_acc[k] += (uint32_t)(t - tr_last);
            tr_last = t;
        }
    };
    if constexpr (TRACE) {
        tr_mark(-1);
        tr_entry = tr_last;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    // Workgroups are dealt to the 8 XCDs round-robin by linear id; give each
    // XCD a contiguous run of (sequence, kv head, q tile) work so the
    // workgroups sharing an L2 walk neighbouring q tiles of the same head,
    // whose key windows overlap almost entirely.
    const int n_qt = (p.seq_len + QP - 1) / QP;
    const int work = xcd_remap((int)blockIdx.x, n_qt * p.hkv * p.batch);
    const int qt = work % n_qt, g = (work / n_qt) % p.hkv, b = work / (n_qt * p.hkv);

    // Chunk start and prefix length of this sequence, in the frame of its
    // chunk (pos_frame; the host moved uniform chunks already): there every
    // position is below 2^31 (the host checks the bound), so positions are
    // handled in 32 bits.
    // (scalar loads: a pending vector load read under a condition would make
    // the compiler wait for every vector load, the query loads included, at
    // its first use past the planning barriers)
    const int64_t S_abs = p.starts ? scalar_load(p.starts + b) : p.start_pos;
    const int64_t P_abs = p.plens ? (int64_t)scalar_load(p.plens + b) : p.P;
    const PosFrame fr = p.starts ? pos_frame(S_abs, p.seq_len, P_abs, p.W, !p.cache_mode)
                                 : PosFrame{P_abs, p.W, 0, 0};
    const int64_t S = S_abs - fr.shift, Pb = fr.P;
    const int t0 = qt * QP;                    // first chunk row of the tile
    const int t_last = (t0 + QP < p.seq_len ? t0 + QP : p.seq_len) - 1;
    const int i0 = (int)S + t0;
    const int i1 = (int)S + t_last;
    const int P32 = (int)Pb;
    const int w32 = (int)fr.W;
    const float c = p.scale_log2;                              // > 0 (checked on the host)

    // this lane's query: stacked row 32*wave + col.  G is the layout's head
    // count; a group of fewer heads (3 on the 4-head layout, 5 to 7 on the
    // 8-head one) leaves the rows of the missing heads idle.
    const int qrow = 32 * wave + col;
    const int greal = p.hq / p.hkv;
    const int hh = qrow / QP;
    const int head = g * greal + (hh < greal ? hh : 0);
    const int my_t = t0 + qrow % QP;
    const bool q_ok = my_t < p.seq_len && hh < greal;
    const int my_i = (int)S + my_t;

    // The walk over the key tiles is planned by thread 0 from the key runs in
    // LDS.  Uniform chunks copy the runs from the kernel arguments, each wave
    // 16 words with scalar loads (thread 0 copying them field by field takes
    // several microseconds of dependent loads); ragged chunks build each
    // sequence's runs on thread 0.  Scalar loads and LDS count in lgkmcnt,
    // and the barriers around the planning wait for that counter only, so
    // the query loads below stay in flight through the planning.
    __shared__ TileWalk walk;
    __shared__ RunView views[kMaxRuns];
    __shared__ KeyRun s_runs[kMaxRuns];
    __shared__ int32_t s_table[kMaxPagesPerSeq];  // paged layout: the sequence's page table row
    static_assert(sizeof(KeyRun) % 4 == 0 && kMaxRuns * sizeof(KeyRun) / 4 <= 16 * kWaves, "16 words per wave");
    const int run_words = p.starts ? 0 : p.n_runs * (int)(sizeof(KeyRun) / 4);
    uint32_t run_word = 0;  // word 16 * wave + lane of the run table (lanes 0-15)
    {
        // uniform indexes: the words stay inside the kernel argument block
        // (the run table is followed by more arguments)
        static_assert(16 * kWaves * 4 <= sizeof(PrefillParams) - offsetof(PrefillParams, runs),
                      "every wave's 16 words lie inside the parameter block");
        const uint32_t* src = reinterpret_cast<const uint32_t*>(p.runs) + 16 * wave;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t wd = src[j];
            run_word = lane == j ? wd : run_word;
        }
    }

    Vec16 qreg[8];
    {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) +
                             (((int64_t)b * p.seq_len + (q_ok ? my_t : 0)) * p.hq + head) * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qreg[ks] = q_ok ? *reinterpret_cast<const Vec16*>(qp + 8 * h + 16 * ks) : Vec16{{0, 0, 0, 0}};
    }

    if (lane < 16 && 16 * wave + lane < run_words) reinterpret_cast<uint32_t*>(s_runs)[16 * wave + lane] = run_word;
    if (p.cache_mode && p.cache.pages)
        for (int j = tid; j < p.cache.pages_per_seq; j += kThreads)
            s_table[j] = p.cache.pages[(int64_t)b * p.cache.pages_per_seq + j];
    lds_barrier();
    if (tid == 0) {
        const int n_runs = p.starts ? seq_key_runs(p, b, S_abs, P_abs, fr, s_runs) : p.n_runs;
        plan_walk<kBNB>(s_runs, n_runs, Pb, fr.W, (int64_t)i0, (int64_t)i1, walk);
        for (int r = 0; r < n_runs; ++r) make_view(views[r], s_runs[r], b, g, p.hkv, 2);
    }
    lds_barrier();
    int total = 0;
    for (int r = 0; r < walk.n_ranges; ++r) total += walk.end[r] - walk.begin[r];

    // per-lane LDS offsets of the transposing V reads (row 4h + k/4 of the
    // 16-lane group, dims 32m + 16(q%2) + 4(k%4)); rows differing by a
    // multiple of 4 share the swizzle, so the k-step and half add constants
    uint32_t vt_off[4];
    {
        const int q = lane >> 4, gp = lane & 15;
        const int row = 4 * h + (gp >> 2);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int dim = 32 * m + 16 * (q & 1) + 4 * (gp & 3);
            vt_off[m] = row * kRowBytes + ((((dim >> 3) ^ v_chunk_swz(row)) << 4) | ((dim & 7) << 1));
        }
    }

    f32x16 o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[m][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // Tile pipeline: two LDS stages of one 128-key tile each.  While tile f is
    // computed, tile f + 1 is resident or in flight.  At the end of iteration
    // f every wave waits until its own loads of tile f + 1 landed and meets
    // the others at the barrier; the stage of tile f is then free and
    // receives tile f + 2.  Two cursors walk the tiles: one for the tile being
    // computed, one for the next tile to stage.
    Cursor cc, pc;
    LaneOffsets lo;
    if (total > 0) {
        cursor_enter(cc, 0, walk, views);
        cursor_enter(pc, 0, walk, views);
        lane_offsets(lo, pc.rs, lane, wave);
    }
    auto stage_next = [&](char* stage) {
        load_tile_bf16(pc, lo, wave, stage, s_table);
        if (cursor_next(pc, walk.n_ranges, walk, views)) lane_offsets(lo, pc.rs, lane, wave);
    };
    static_assert(kStages == 2 && kLoadsPerTile == 16, "vmcnt immediates assume 2 stages of 16 loads");

    // prologue: tile 0 in flight beside the query loads; both have landed
    // before tile 1 is issued.  (The query registers are waited for here, once:
    // left to the compiler, that wait would sit at their first use inside the
    // tile loop and drain the tile prefetch on every iteration.)
    if (total > 0) stage_next(smem);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qreg[ks].w[0]), "v"(qreg[ks].w[3]));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (total > 1) stage_next(smem + kStageBytes);
    tile_barrier();

    constexpr int kMB = kBNB / 32;  // 32-key score blocks per tile
    constexpr int kST = kBNB / 16;  // 16-key k-steps of P.V per tile
    tr_mark(-1);
    for (int f = 0; f < total; ++f) {
        const int row0 = cc.t * kBNB;
        const int nrows = cc.n - row0 < kBNB ? cc.n - row0 : kBNB;
        const int j0 = (int)cc.pos0 + row0;
        const int j1 = j0 + nrows - 1;
        const int cls = nrows < kBNB ? kMasked : tile_class32(i0, i1, j0, j1, P32, w32);
        const char* ks_lds = smem + (f & 1) * kStageBytes;
        __builtin_amdgcn_sched_barrier(0);

        // S^T = K Q^T (raw scores, unscaled), one 32-key block per accumulator,
        // in two halves of two interleaved blocks.  The mask and the running
        // maximum of the first half need none of the second half's products,
        // so they are written inside the same basic block as its MFMAs (one
        // copy of that block per tile kind) and go out between them, while the
        // matrix core is busy, instead of after the last product (0.5% on both
        // prefill shapes, bit-identical).  Four one-block chains, each block's
        // maximum beside the next block's products, were 2% slower: a chain of
        // dependent products stalls the matrix core.
        //
        // Elementwise mask, straddling tiles only.  For this lane's query the
        // visible keys of the tile (tile-relative index kr) form at most two
        // intervals: [0, min(pj, hic + 1)) -- the prefix -- and
        // [max(relw + 1, 0), hic + 1) -- the window -- with rel = i - j0,
        // relw = rel - W, pj = P - j0, hic = min(rel, nrows - 1).  They become
        // one 32-bit bitmap per 32-key block, and each score is kept or set to
        // -inf with a bit extract and a bitfield select (no per-element compares).
        f32x16 s[kMB];
        float tmax = -INFINITY;
        {
            const f32x16 zero = {};
            const int pj = P32 - j0;
            const int rel = my_i - j0;
            const int hic = rel < nrows - 1 ? rel : nrows - 1;
            const int a_hi = pj < hic + 1 ? pj : hic + 1;
            const int b_lo = rel - w32 + 1 > 0 ? rel - w32 + 1 : 0;
            auto mask_block = [&](int mb) __attribute__((always_inline)) {
                const uint32_t bits = range_bits(0, a_hi - 32 * mb) | range_bits(b_lo - 32 * mb, hic + 1 - 32 * mb);
                const uint32_t bits_h = bits >> (4 * h);  // this lane half's keys start at bit 4h
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t km = (uint32_t)__builtin_amdgcn_sbfe((int)bits_h, 8 * (r >> 2) + (r & 3), 1);
                    s[mb][r] = __uint_as_float((km & __float_as_uint(s[mb][r])) | (~km & 0xFF800000u));
                }
            };
            auto max_block = [&](int mb) __attribute__((always_inline)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[mb][r]);
            };
            auto qk_pair = [&](int half) __attribute__((always_inline)) {
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int mb = 2 * half; mb < 2 * half + 2; ++mb) {
                        const int krow = 32 * mb + col;
                        const Vec16 ka = *reinterpret_cast<const Vec16*>(ks_lds + krow * kRowBytes + (((2 * kk + h) ^ k_chunk_swz(krow)) << 4));
                        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qreg[kk]),
                                                                         kk == 0 ? zero : s[mb], 0, 0, 0);
                    }
            };
            qk_pair(0);
            if (cls == kMasked) {
                qk_pair(1);
                mask_block(0);
                mask_block(1);
                max_block(0);
                max_block(1);
                __builtin_amdgcn_sched_barrier(0);
                tr_mark(0);
                mask_block(2);
                mask_block(3);
            } else {
                qk_pair(1);
                max_block(0);
                max_block(1);
                __builtin_amdgcn_sched_barrier(0);
                tr_mark(0);
            }
            max_block(2);
            max_block(3);
        }
        // online softmax in raw-score units: the reference first
        {
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            // The exponent reference only moves when some row's maximum
            // exceeds it by more than 8 (log2 units): until then terms stay
            // below 2^8, and since l and O share the reference the result is
            // the same.
            if (__any(tmax * c > m_run * c + 8.f)) {
                const float m_new = fmaxf(m_run, tmax);
                const float alpha = fast_exp2(m_run == -INFINITY ? -INFINITY : (m_run - m_new) * c);
                l_run *= alpha;
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[m][r] *= alpha;
                m_run = m_new;
            }
        }
        const float mc = m_run == -INFINITY ? 0.f : m_run * c;
        __builtin_amdgcn_sched_barrier(0);
        tr_mark(1);

        // O^T += V^T P^T, k-step by k-step.  P^T of k-step st (keys 16 st ..
        // 16 st + 15, exp2((s - m) * c) packed to bf16) is made right before
        // its four MFMAs, so the exponentials of one k-step run beside the
        // MFMAs of the previous one.  The A operand (V^T: row = head dim, 8
        // keys in the order of P's k-step) comes from the row-major V tile with
        // two transposing reads per dim block (see read_vt).
        {
            const uint32_t vb = lds_addr(ks_lds + kTileBytes);
#pragma unroll
            for (int st = 0; st < kST; ++st) {
                const int mb = st >> 1, base = 8 * (st & 1);
                Vec16 pb;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    pb.w[w] = pack_bf16x2(fast_exp2(fmaf(s[mb][base + 2 * w], c, -mc)),
                                          fast_exp2(fmaf(s[mb][base + 2 * w + 1], c, -mc)));
                l_run += sum_bf16x8(pb);
                Vec16 va[4];
                read_vt(st, vb + vt_off[0], vb + vt_off[1], vb + vt_off[2], vb + vt_off[3], va);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    o[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[m]), as_bf16x8(pb), o[m], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        tr_mark(2);

        // tile f + 1 must have landed before anyone reads it; then the stage
        // of tile f takes tile f + 2
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        tr_mark(3);
        tile_barrier();
        tr_mark(4);
        if (f + kStages < total) stage_next(smem + (f & 1) * kStageBytes);
        cursor_next(cc, walk.n_ranges, walk, views);
        tr_mark(5);
    }
    if constexpr (TRACE) {
        if (lane == 0 && p.trace) {
            unsigned long long* tr = p.trace + 8 * (wave >= kLoadWaves ? 1 : 0);
#pragma unroll
            for (int k = 0; k < 6; ++k) atomicAdd(tr + k, (unsigned long long)tr_acc[k]);
            atomicAdd(tr + 6, (unsigned long long)total);
            atomicAdd(tr + 7, (unsigned long long)(__builtin_amdgcn_s_memtime() - tr_entry));
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (!q_ok) return;
    const float inv = 1.f / l_tot;
    uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + (((int64_t)b * p.seq_len + my_t) * p.hq + head) * D;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            Vec8 w;
            w.w[0] = pack_bf16x2(o[m][4 * cc] * inv, o[m][4 * cc + 1] * inv);
            w.w[1] = pack_bf16x2(o[m][4 * cc + 2] * inv, o[m][4 * cc + 3] * inv);
            *reinterpret_cast<Vec8*>(op + 32 * m + 8 * cc + 4 * h) = w;
        }
    if (p.lse && h == 0) p.lse[((int64_t)b * p.seq_len + my_t) * p.hq + head] = (m_run * c + log2f(l_tot)) * kLn2;
}

// Stacked-row layout of a GQA group: the kernels are built for 1, 2, 4 and
// 8 heads per kv head; 3 runs on the 4-head layout and 5 to 7 on the 8-head
// one, the missing heads' rows idle.
inline int layout_group(int group) { return group <= 2 ? group : (group <= 4 ? 4 : 8); }

// Whether the dynamic-LDS limit of kernel slot `slot` was raised on the
// current device (a host call made once per kernel and device).
constexpr int kMaxDevices = 64;
inline bool* lds_flag(int slot) {
    static bool flags[kMaxDevices][16] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    return &flags[dev][slot];
}

// Delta rows of the allocation-free backward.  Each GPU holds its own copy of
// this array at its own address.  On the host the name is only a stand-in
// (passing it to a kernel would hand the kernel a host address), so host
// code uses the device address hipGetSymbolAddress returns, taken once per
// device with that device current.
static __device__ __align__(256) float scratch[PS_BWD_NOALLOC_MAX_ROWS];

// ----------------------------------------------------------------- plain path
// One thread per query row of a 64-position tile of one q head; K/V tiles in
// LDS as fp32; two passes per tile (scores for the tile maximum, then the
// weighted sum).  T is the storage type: float, or uint16_t holding bf16 bits
// (widened exactly; the output rounded to nearest even).
__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ inline void store_as(float* p, float v) { *p = v; }
__device__ inline void store_as(uint16_t* p, float v) {
    const __bf16 b = (__bf16)v;
    __builtin_memcpy(p, &b, 2);
}

template <typename T, int D>
__global__ void __launch_bounds__(64) prefill_plain_kernel(PrefillParams p) {
    constexpr int BR = 32;  // rows staged per LDS fill (two fills per 64-key tile)
    __shared__ float ks[BR][D];
    __shared__ float vs[BR][D];
    __shared__ TileWalk walk;
    if (p.guard && *p.guard) return;  // checks on and a check failed
    const int tid = threadIdx.x;
    const int qt = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
    const int group = p.hq / p.hkv;
    const int g = head / group;
    const int64_t S_abs = p.starts ? p.starts[b] : p.start_pos;
    const int64_t P_abs = p.plens ? (int64_t)p.plens[b] : p.P;
    const PosFrame fr = p.starts ? pos_frame(S_abs, p.seq_len, P_abs, p.W, !p.cache_mode)
                                 : PosFrame{P_abs, p.W, 0, 0};
    const int64_t S = S_abs - fr.shift, Pb = fr.P, Wb = fr.W;
    const int64_t t0 = (int64_t)qt * 64;
    const int64_t t_last = (t0 + 64 < p.seq_len ? t0 + 64 : p.seq_len) - 1;
    const int64_t i0 = S + t0, i1 = S + t_last;
    const int64_t my_t = t0 + tid;
    const bool q_ok = my_t < p.seq_len;
    const int64_t my_i = S + my_t;

    float q[D], o[D];
    const T* qp = reinterpret_cast<const T*>(p.q) + (((int64_t)b * p.seq_len + (q_ok ? my_t : 0)) * p.hq + head) * D;
    for (int e = 0; e < D; ++e) {
        q[e] = q_ok ? to_f32(qp[e]) * p.scale_log2 : 0.f;
        o[e] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;

    __shared__ KeyRun s_runs[kMaxRuns];
    if (tid == 0) plan_walk<kBN>(s_runs, seq_key_runs(p, b, S_abs, P_abs, fr, s_runs), Pb, Wb, i0, i1, walk);
    __syncthreads();
    for (int rr = 0; rr < walk.n_ranges; ++rr) {
        const KeyRun& run = s_runs[walk.run[rr]];
        const int64_t seq = run.rows ? (int64_t)run.rows[b] : (int64_t)b;
        const int64_t base_el = run.pages ? (int64_t)g * run.head_stride : seq * run.seq_stride + (int64_t)g * run.head_stride;
        const T* kb = reinterpret_cast<const T*>(run.k) + base_el;
        const T* vb = reinterpret_cast<const T*>(run.v) + base_el;
        for (int tile = walk.begin[rr]; tile < walk.end[rr]; ++tile) {
            const int64_t row0 = (int64_t)tile * kBN;
            const int64_t nrows = run.n - row0 < kBN ? run.n - row0 : kBN;
            // first row of the tile: a paged run's 64-row tile lies in one page
            int64_t tile_el = row0 * run.row_stride;
            if (run.pages) {
                const int64_t slot = run.first_slot + row0;
                const int64_t page = run.pages[(int64_t)b * run.pages_per_seq + run.page_col + (slot >> run.page_shift)];
                tile_el = ((page * p.hkv) << run.page_shift) * run.row_stride +
                          (slot & (((int64_t)1 << run.page_shift) - 1)) * run.row_stride;
            }
            const T* kt = kb + tile_el;
            const T* vt = vb + tile_el;
            const int64_t j0 = run.pos0 + row0;
            const int cls = nrows < kBN ? kMasked : tile_class(i0, i1, j0, j0 + nrows - 1, Pb, Wb);
            if (cls == kSkip) continue;
            for (int pass = 0; pass < 2; ++pass) {
                float tmax = -INFINITY;
                for (int half = 0; half < kBN / BR; ++half) {
                    __syncthreads();
                    for (int idx = tid; idx < BR * D; idx += 64) {
                        const int r = idx / D, e = idx % D;
                        const int64_t row = half * BR + r;
                        const bool ok = row < nrows;
                        ks[r][e] = ok ? to_f32(kt[row * run.row_stride + e]) : 0.f;
                        vs[r][e] = ok ? to_f32(vt[row * run.row_stride + e]) : 0.f;
                    }
                    __syncthreads();
                    for (int r = 0; r < BR; ++r) {
                        const int64_t row = half * BR + r;
                        float acc = 0.f;
                        for (int e = 0; e < D; ++e) acc = fmaf(q[e], ks[r][e], acc);
                        if (cls == kMasked && (row >= nrows || !visible(my_i, j0 + row, Pb, Wb))) acc = -INFINITY;
                        if (pass == 0) {
                            tmax = fmaxf(tmax, acc);
                        } else {
                            const float w = exp2f(acc - (m_run == -INFINITY ? 0.f : m_run));
                            l_run += w;
                            for (int e = 0; e < D; ++e) o[e] = fmaf(w, vs[r][e], o[e]);
                        }
                    }
                }
                if (pass == 0) {
                    const float m_new = fmaxf(m_run, tmax);
                    const float alpha = exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
                    m_run = m_new;
                    l_run *= alpha;
                    for (int e = 0; e < D; ++e) o[e] *= alpha;
                }
            }
        }
    }
    if (!q_ok) return;
    T* op = reinterpret_cast<T*>(p.out) + (((int64_t)b * p.seq_len + my_t) * p.hq + head) * D;
    for (int e = 0; e < D; ++e) store_as(op + e, o[e] / l_run);
    if (p.lse) p.lse[((int64_t)b * p.seq_len + my_t) * p.hq + head] = (m_run + log2f(l_run)) * kLn2;
}

// ================================================================ backward
// Trainer-side backward of the masked attention (the gradient of the forward
// above; the agihunt.info summary, paragraph on RL, and the njhaofan.com
// article, passage on truncated backpropagation, describe the trainer that
// backpropagates through it).  With P = softmax over the visible keys,
// Delta_i = rowsum(dO_i * O_i) and dS = P * (dP - Delta), dP = dO V^T:
//   dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO.
// Three kernels: Delta (a row reduction), dQ (per query tile over its key
// tiles, the forward's walk and staging) and dK/dV (per key block over the
// query tiles that see it).  P is rebuilt from the forward's log-sum-exp, so
// no running maximum is needed.  Tile classification is the forward's: SKIP
// pairs cost nothing, FULL pairs run unmasked, MASKED pairs mask per element.

// Delta[row] = sum_d dO[row][d] * O[row][d] over rows of 128 bf16; 16 lanes
// per row, 8 elements per lane.
__global__ void __launch_bounds__(256) bwd_delta_kernel(const uint16_t* out, const uint16_t* dout, float* delta,
                                                        int64_t rows) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid >> 4;
    const int part = (int)(gid & 15);
    float acc = 0.f;
    if (row < rows) {
        const Vec16 a = *reinterpret_cast<const Vec16*>(out + row * 128 + part * 8);
        const Vec16 b = *reinterpret_cast<const Vec16*>(dout + row * 128 + part * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc = fmaf(__uint_as_float(a.w[w] << 16), __uint_as_float(b.w[w] << 16), acc);
            acc = fmaf(__uint_as_float(a.w[w] & 0xFFFF0000u), __uint_as_float(b.w[w] & 0xFFFF0000u), acc);
        }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 16);
    if (row < rows && part == 0) delta[row] = acc;
}

// Tiles the backward reads both as rows (16-byte operand reads: 16 lanes
// read one chunk of 16 consecutive rows) and transposed (ds_read_b64_tr_b16:
// 16 lanes read chunks c and c + 1 of 4 consecutive rows, c even) swizzle
// chunk c of row r to c ^ b_chunk_swz(r), the two 2-bit halves of r & 15
// swapped: a bijection on every 16 rows (row reads hit 16 distinct chunks),
// whose upper three bits take 4 distinct values over 4 consecutive rows
// (transposing reads hit 8 distinct chunks).  Both are conflict-free.
__device__ inline int b_chunk_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Per-lane byte offsets of the transposing operand reads from such a tile:
// the same lane pattern as read_vt (row 4h + k/4 of the 16-lane group, dims
// 32m + 16(q%2) + 4(k%4)), for the two 8-row halves of a 16-row step; the
// step itself adds 16 rows, which keeps row & 15.
__device__ inline void kswz_tr_offsets(int lane, uint32_t (&off)[2][4]) {
    const int h = lane >> 5, q = lane >> 4, gp = lane & 15;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int row = 8 * half + 4 * h + (gp >> 2);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int dim = 32 * m + 16 * (q & 1) + 4 * (gp & 3);
            off[half][m] = row * kRowBytes + ((((dim >> 3) ^ b_chunk_swz(row)) << 4) | ((dim & 7) << 1));
        }
    }
}
// Transposed operands of 16-row step ST (rows 16 ST .. 16 ST + 15) for the
// four dim blocks, from a tile at LDS address base with the b_chunk_swz swizzle.
__device__ inline void read_t_kswz(int st, uint32_t base, const uint32_t (&off)[2][4], Vec16 (&va)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(uintptr_t)(base + off[0][m] + st * 16 * kRowBytes));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(uintptr_t)(base + off[1][m] + st * 16 * kRowBytes));
        __builtin_memcpy(&va[m].w[0], &lo, 8);
        __builtin_memcpy(&va[m].w[2], &hi, 8);
    }
}


// Per-lane byte offsets of the dQ kernel's tile loads (waves 0-3, rows 32w ..
// 32w + 31), chunks placed with b_chunk_swz.
__device__ inline void lane_offsets_bwd(LaneOffsets& o, int rs, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int row = (kBNB / kLoadWaves) * (wave & (kLoadWaves - 1)) + 4 * i + (lane >> 4);
        o.k[i] = o.v[i] = row * rs + (((lane & 15) ^ b_chunk_swz(row)) << 4);
    }
}

// Stage the cursor's tile for the dQ kernel: K and V rows both with
// b_chunk_swz (K is read as rows for S^T and transposed for dQ; V as rows
// for dP^T).
__device__ inline void load_tile_bwd(const Cursor& c, const LaneOffsets& lo, int wave, char* stage) {
    const int row0 = c.t * kBNB;
    const int nrows = c.n - row0 < kBNB ? c.n - row0 : kBNB;
    const int64_t off = (int64_t)row0 * c.rs;
    if (wave >= kLoadWaves) return;
    const i32x4 kr = rsrc_words(c.k + off, nrows * c.rs);
    const i32x4 vr = rsrc_words(c.v + off, nrows * c.rs);
    const uint32_t sb = lds_addr(stage);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int r4 = (kBNB / kLoadWaves) * wave + 4 * i;
        dma16_asm(kr, lo.k[i], sb + r4 * kRowBytes);
        dma16_asm(vr, lo.k[i], sb + kTileBytes + r4 * kRowBytes);
    }
}

// dQ: the forward's workgroup layout (8 waves, 256 stacked query rows, 128-key
// tiles in a 2-stage ring).  Per tile and 64-key half: S^T = K Q^T and
// dP^T = V dO^T (both with the key rows as the A operand), dS^T in registers,
// then dQ^T += K^T dS^T with K^T from transposing reads.
template <int G>
__global__ void __launch_bounds__(kThreads, 1) bwd_dq_kernel(BwdParams bp) {
    constexpr int D = 128;
    constexpr int QP = 32 * kWaves / G;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const PrefillParams& p = bp.f;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int n_qt = (p.seq_len + QP - 1) / QP;
    const int work = xcd_remap((int)blockIdx.x, n_qt * p.hkv * p.batch);
    const int qt = work % n_qt, g = (work / n_qt) % p.hkv, b = work / (n_qt * p.hkv);

    const int t0 = qt * QP;
    const int t_last = (t0 + QP < p.seq_len ? t0 + QP : p.seq_len) - 1;
    const int i0 = (int)p.start_pos + t0;
    const int i1 = (int)p.start_pos + t_last;
    const int P32 = p.P > 0x7FFFFFFF ? 0x7FFFFFFF : (int)p.P;
    const int w32 = p.W > 0x7FFFFFFF ? 0x7FFFFFFF : (int)p.W;
    const float c = p.scale_log2;

    const int qrow = 32 * wave + col;
    const int greal = p.hq / p.hkv;  // heads of the group (<= G; missing heads' rows idle)
    const int hh = qrow / QP;
    const int head = g * greal + (hh < greal ? hh : 0);
    const int my_t = t0 + qrow % QP;
    const bool q_ok = my_t < p.seq_len && hh < greal;
    const int my_i = (int)p.start_pos + my_t;
    const int64_t row_el = ((int64_t)b * p.seq_len + (q_ok ? my_t : 0)) * p.hq + head;
    Vec16 qreg[8], dreg[8];
    {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + row_el * D;
        const uint16_t* dp = reinterpret_cast<const uint16_t*>(bp.dout) + row_el * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qreg[ks] = q_ok ? *reinterpret_cast<const Vec16*>(qp + 8 * h + 16 * ks) : Vec16{{0, 0, 0, 0}};
            dreg[ks] = q_ok ? *reinterpret_cast<const Vec16*>(dp + 8 * h + 16 * ks) : Vec16{{0, 0, 0, 0}};
        }
    }
    // P = exp2(s c - lse log2 e); rows past the chunk get P = 0
    const float lse2 = q_ok ? bp.lse[row_el] * kLog2eF : INFINITY;
    const float dlt = q_ok ? bp.delta[row_el] : 0.f;
    // the compiler cannot see the asm tile loads: make these loads complete
    // here rather than at their first use inside the tile loop
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qreg[ks].w[0]), "v"(dreg[ks].w[0]));
    asm volatile("" ::"v"(lse2), "v"(dlt));

    __shared__ TileWalk walk;
    __shared__ RunView views[kMaxRuns];
    if (tid == 0) {
        plan_walk<kBNB>(p.runs, p.n_runs, p.P, p.W, (int64_t)i0, (int64_t)i1, walk);
        for (int r = 0; r < p.n_runs; ++r) make_view(views[r], p.runs[r], b, g, p.hkv, 2);
    }
    __syncthreads();
    int total = 0;
    for (int r = 0; r < walk.n_ranges; ++r) total += walk.end[r] - walk.begin[r];

    uint32_t kt_off[2][4];
    kswz_tr_offsets(lane, kt_off);

    f32x16 dq[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[m][r] = 0.f;

    Cursor cc, pc;
    LaneOffsets lo;
    if (total > 0) {
        cursor_enter(cc, 0, walk, views);
        cursor_enter(pc, 0, walk, views);
        lane_offsets_bwd(lo, pc.rs, lane, wave);
    }
    auto stage_next = [&](char* stage) {
        load_tile_bwd(pc, lo, wave, stage);
        if (cursor_next(pc, walk.n_ranges, walk, views)) lane_offsets_bwd(lo, pc.rs, lane, wave);
    };
    if (total > 0) stage_next(smem);
    if (total > 1) {
        stage_next(smem + kStageBytes);
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    tile_barrier();

    for (int f = 0; f < total; ++f) {
        const int row0 = cc.t * kBNB;
        const int nrows = cc.n - row0 < kBNB ? cc.n - row0 : kBNB;
        const int j0 = (int)cc.pos0 + row0;
        const int j1 = j0 + nrows - 1;
        const int cls = nrows < kBNB ? kMasked : tile_class32(i0, i1, j0, j1, P32, w32);
        const char* ks_lds = smem + (f & 1) * kStageBytes;
        const char* vs_lds = ks_lds + kTileBytes;
        const uint32_t kb = lds_addr(ks_lds);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f32x16 s[2], dp[2];
            const f32x16 zero = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    const int krow = 32 * (2 * half + mm) + col;
                    const int off = krow * kRowBytes + (((2 * kk + h) ^ b_chunk_swz(krow)) << 4);
                    const Vec16 ka = *reinterpret_cast<const Vec16*>(ks_lds + off);
                    const Vec16 va = *reinterpret_cast<const Vec16*>(vs_lds + off);
                    s[mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qreg[kk]),
                                                                     kk == 0 ? zero : s[mm], 0, 0, 0);
                    dp[mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(dreg[kk]),
                                                                      kk == 0 ? zero : dp[mm], 0, 0, 0);
                }
            if (cls == kMasked) {
                const int pj = P32 - j0;
                const int rel = my_i - j0;
                const int hic = rel < nrows - 1 ? rel : nrows - 1;
                const int a_hi = pj < hic + 1 ? pj : hic + 1;
                const int b_lo = rel - w32 + 1 > 0 ? rel - w32 + 1 : 0;
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    const int mb = 2 * half + mm;
                    const uint32_t bits = range_bits(0, a_hi - 32 * mb) | range_bits(b_lo - 32 * mb, hic + 1 - 32 * mb);
                    const uint32_t bits_h = bits >> (4 * h);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const uint32_t km = (uint32_t)__builtin_amdgcn_sbfe((int)bits_h, 8 * (r >> 2) + (r & 3), 1);
                        s[mm][r] = __uint_as_float((km & __float_as_uint(s[mm][r])) | (~km & 0xFF800000u));
                    }
                }
            }
            // dS^T = P^T (dP^T - Delta), packed to bf16 per 16-key step, and
            // dQ^T += K^T dS^T
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) {
                const int mm = sl >> 1, base = 8 * (sl & 1);
                Vec16 ds;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int r0 = base + 2 * w;
                    const float p0 = fast_exp2(fmaf(s[mm][r0], c, -lse2));
                    const float p1 = fast_exp2(fmaf(s[mm][r0 + 1], c, -lse2));
                    ds.w[w] = pack_bf16x2(p0 * (dp[mm][r0] - dlt), p1 * (dp[mm][r0 + 1] - dlt));
                }
                Vec16 ka[4];
                read_t_kswz(4 * half + sl, kb, kt_off, ka);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    dq[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[m]), as_bf16x8(ds), dq[m], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        tile_barrier();
        if (f + kStages < total) stage_next(smem + (f & 1) * kStageBytes);
        cursor_next(cc, walk.n_ranges, walk, views);
    }

    if (!q_ok) return;
    uint16_t* op = reinterpret_cast<uint16_t*>(bp.dq) + row_el * D;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int cc4 = 0; cc4 < 4; ++cc4) {
            Vec8 w;
            w.w[0] = pack_bf16x2(dq[m][4 * cc4] * bp.scale, dq[m][4 * cc4 + 1] * bp.scale);
            w.w[1] = pack_bf16x2(dq[m][4 * cc4 + 2] * bp.scale, dq[m][4 * cc4 + 3] * bp.scale);
            *reinterpret_cast<Vec8*>(op + 32 * m + 8 * cc4 + 4 * h) = w;
        }
}

// The lane index taken afresh (mbcnt in asm): the compiler cannot equate it
// with an earlier one, so values derived from it are not kept live across
// the caller's loop.
__device__ inline int lane_now() {
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    return lane;
}

// One 32 x 32 tile of bf16 dS from the key-on-the-lane layout the dK/dV
// kernel stores (v[st]: rows 16 st + 4h + 0..3 in words 0-1 and
// 16 st + 8 + 4h + 0..3 in words 2-3, the lane's key) to the query row on the
// lane, through 2 KB of the wave's own LDS at tb: one 64-byte row per key,
// the lane's 16 bytes of step st at 16-byte slot (2 st + h) ^ ((key >> 2) & 3)
// (one 128-bit write per step).  The transposing reads give lane (row j,
// half h) keys 16 st + 4h + 0..3 and 16 st + 8 + 4h + 0..3, the order of the
// K^T operands read_t_kswz gives; the slot swizzle keeps both the writes and
// the reads free of bank conflicts.
__device__ inline void ds_transpose(uint32_t tba, const Vec16 (&v)[2], Vec16 (&out)[2]) {
    const int lane = lane_now();
    const int h = lane >> 5, col = lane & 31, q = lane >> 4, gp = lane & 15;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        i32x4 w;
        __builtin_memcpy(&w, &v[st], 16);
        *reinterpret_cast<__attribute__((address_space(3))) i32x4*>(
            (uintptr_t)(tba + col * 64 + (((2 * st + h) ^ ((col >> 2) & 3)) << 4))) = w;
    }
    // lane (q, gp) fetches rows 16 (q & 1) + 4 (gp & 3) .. + 3 of key
    // 16 st + 8 hf + 4 (q >> 1) + (gp >> 2): the 8-byte half (gp >> 1) & 1 of
    // the slot written for step q & 1 by the lane half gp & 1
    const int slot_r = 2 * (q & 1) + (gp & 1), part_r = (gp >> 1) & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int key = 16 * st + 8 * hf + 4 * h + (gp >> 2);
            const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
                uintptr_t)(tba + key * 64 + ((slot_r ^ ((key >> 2) & 3)) << 4) + (part_r << 3)));
            __builtin_memcpy(&out[st].w[2 * hf], &r, 8);
        }
}
constexpr int kDsXpose = 2048;  // LDS bytes of one tile transpose

// Stage the cursor's K tile alone (b_chunk_swz, read transposed by the dQ
// kernel that takes dS from the band).
__device__ inline void load_tile_k(const Cursor& c, const LaneOffsets& lo, int wave, char* stage) {
    const int row0 = c.t * kBNB;
    const int nrows = c.n - row0 < kBNB ? c.n - row0 : kBNB;
    if (wave >= kLoadWaves) return;
    const i32x4 kr = rsrc_words(c.k + (int64_t)row0 * c.rs, nrows * c.rs);
    const uint32_t sb = lds_addr(stage);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
        dma16_asm(kr, lo.k[i], sb + ((kBNB / kLoadWaves) * wave + 4 * i) * kRowBytes);
}

// dQ from the stored dS band: dQ^T += K^T dS^T over the key tiles of the
// walk, the forward's workgroup layout (8 waves, 256 stacked query rows;
// wave w's 32 rows are one head's 32 positions, one row block of the band).
// K tiles go through a 2-stage LDS ring (read transposed); each wave loads
// its dS tiles from the band straight into registers, two tiles in flight,
// and turns them to the query row on the lane through its own LDS
// (ds_transpose, one 2 KB buffer per key block of the tile, after the K
// ring).  Blocks of 32 keys the wave's rows cannot see are skipped; on
// blocks that straddle the rule the invisible pairs are zeroed (the band
// holds only what the dK/dV kernel stored: its skipped halves are never
// written).
template <int G>
__global__ void __launch_bounds__(kThreads, 1) bwd_dq_ds_kernel(BwdParams bp) {
    constexpr int D = 128;
    constexpr int QP = 32 * kWaves / G;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const PrefillParams& p = bp.f;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int n_qt = (p.seq_len + QP - 1) / QP;
    const int work = xcd_remap((int)blockIdx.x, n_qt * p.hkv * p.batch);
    const int qt = work % n_qt, g = (work / n_qt) % p.hkv, b = work / (n_qt * p.hkv);

    const int S0 = (int)p.start_pos;
    const int t0 = qt * QP;
    const int t_last = (t0 + QP < p.seq_len ? t0 + QP : p.seq_len) - 1;
    const int i0 = S0 + t0, i1 = S0 + t_last;
    const int P32 = p.P > 0x7FFFFFFF ? 0x7FFFFFFF : (int)p.P;
    const int w32 = p.W > 0x7FFFFFFF ? 0x7FFFFFFF : (int)p.W;

    const int greal = p.hq / p.hkv;
    const int hh = 32 * wave / QP;             // the wave's head of the group
    const int tw = t0 + (32 * wave) % QP;      // its first position (chunk row)
    const bool w_ok = hh < greal && tw < p.seq_len;
    const int head = g * greal + (hh < greal ? hh : 0);
    const int wi0 = S0 + tw, wi1 = wi0 + 31;   // its positions (rows past the chunk included)
    const int rb = tw >> 5;
    const int my_i = wi0 + col;
    // the wave's row block of the band (waves without rows read slot 0 of the
    // band's first block: every tile loads all its operands, so that no load
    // is conditional and the compiler never waits for one before its use)
    const char* dsb = bp.ds + (w_ok ? (((int64_t)b * p.hq + head) * bp.ds_nrb + rb) * bp.ds_nband * 2048 : 0) +
                      lane * 16;

    __shared__ TileWalk walk;
    __shared__ RunView views[kMaxRuns];
    if (tid == 0) {
        plan_walk<kBNB>(p.runs, p.n_runs, p.P, p.W, (int64_t)i0, (int64_t)i1, walk);
        for (int r = 0; r < p.n_runs; ++r) make_view(views[r], p.runs[r], b, g, p.hkv, 2);
    }
    __syncthreads();
    int total = 0;
    for (int r = 0; r < walk.n_ranges; ++r) total += walk.end[r] - walk.begin[r];

    uint32_t kt_off[2][4];
    kswz_tr_offsets(lane, kt_off);
    f32x16 dq[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[m][r] = 0.f;

    // class of the wave's rows against key block mb of the cursor's tile
    auto block_class = [&](const Cursor& c, int mb, int& jb0, int& nb) __attribute__((always_inline)) {
        const int row0 = c.t * kBNB;
        const int nrows = c.n - row0 < kBNB ? c.n - row0 : kBNB;
        jb0 = (int)c.pos0 + row0 + 32 * mb;
        nb = nrows - 32 * mb < 32 ? nrows - 32 * mb : 32;
        if (!w_ok || nb <= 0) return (int)kSkip;
        return tile_class32(wi0, wi1, jb0, jb0 + nb - 1, P32, w32);
    };
    auto load_ds = [&](const Cursor& c, Vec16 (&buf)[4][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            int jb0, nb;
            const bool skip = block_class(c, mb, jb0, nb) == kSkip;  // then slot 0, never used
            const int kb = (jb0 - S0) >> 5;
            const int slot = skip ? 0 : kb < bp.ds_npre ? kb : bp.ds_npre + kb - rb + bp.ds_nwin - 1;
            const char* src = dsb + (int64_t)slot * 2048;
            buf[mb][0] = *reinterpret_cast<const Vec16*>(src);
            buf[mb][1] = *reinterpret_cast<const Vec16*>(src + 1024);
        }
    };
    const uint32_t xpose = lds_addr(smem + kStages * kTileBytes) + wave * 4 * kDsXpose;
    auto compute = [&](const Cursor& c, const char* kstage, Vec16 (&raw)[4][2]) __attribute__((always_inline)) {
        const uint32_t kb_lds = lds_addr(kstage);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            int jb0, nb;
            const int cls = block_class(c, mb, jb0, nb);
            if (cls == kSkip) continue;
            Vec16 ds[2];  // the block's dS, query row on the lane
            ds_transpose(xpose + mb * kDsXpose, raw[mb], ds);
            if (cls == kMasked) {
                // visible keys of the lane's row among the block's nb keys
                const int rel = my_i - jb0;
                const int hic = rel < nb - 1 ? rel : nb - 1;
                const int a_hi = P32 - jb0 < hic + 1 ? P32 - jb0 : hic + 1;
                const int b_lo = rel - w32 + 1 > 0 ? rel - w32 + 1 : 0;
                const uint32_t bits = range_bits(0, a_hi) | range_bits(b_lo, hic + 1);
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd) {
                        const int k0 = 16 * st + 8 * (wd >> 1) + 4 * h + 2 * (wd & 1);
                        const uint32_t m2 = bits >> k0;
                        const uint32_t keep = ((m2 & 1u) ? 0x0000FFFFu : 0u) | ((m2 & 2u) ? 0xFFFF0000u : 0u);
                        ds[st].w[wd] &= keep;
                    }
            }
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                Vec16 ka[4];
                read_t_kswz(2 * mb + st, kb_lds, kt_off, ka);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    dq[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[m]), as_bf16x8(ds[st]), dq[m], 0, 0, 0);
            }
        }
    };
    // the compiler cannot see the asm tile loads: after the explicit wait,
    // a use of the next tile's dS registers settles its own wait for them
    // there, not at their first use in the next tile
    auto settle = [&](Vec16 (&buf)[4][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) asm volatile("" ::"v"(buf[mb][0].w[0]), "v"(buf[mb][1].w[0]));
    };

    Cursor cc, pc;
    LaneOffsets lo;
    if (total > 0) {
        cursor_enter(cc, 0, walk, views);
        cursor_enter(pc, 0, walk, views);
        lane_offsets_bwd(lo, pc.rs, lane, wave);
    }
    Vec16 bufa[4][2], bufb[4][2];
    auto stage_next = [&](char* stage, Vec16 (&buf)[4][2]) __attribute__((always_inline)) {
        load_tile_k(pc, lo, wave, stage);
        load_ds(pc, buf);
        if (cursor_next(pc, walk.n_ranges, walk, views)) lane_offsets_bwd(lo, pc.rs, lane, wave);
    };
    if (total > 0) stage_next(smem, bufa);
    if (total > 1) stage_next(smem + kTileBytes, bufb);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    settle(bufa);
    settle(bufb);
    tile_barrier();

    // tile f: compute from stage f & 1, wait for tile f + 1, then stage tile
    // f + 2 into the freed stage and registers
    auto step = [&](int f, Vec16 (&cur)[4][2], Vec16 (&nxt)[4][2]) __attribute__((always_inline)) {
        compute(cc, smem + (f & 1) * kTileBytes, cur);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        settle(nxt);
        tile_barrier();
        if (f + kStages < total) stage_next(smem + (f & 1) * kTileBytes, cur);
        cursor_next(cc, walk.n_ranges, walk, views);
    };
    // (both steps unconditional inside the loop: on every path into an
    // iteration the registers it computes from are settled)
    int f = 0;
    for (; f + 1 < total; f += 2) {
        step(f, bufa, bufb);
        step(f + 1, bufb, bufa);
    }
    if (f < total) step(f, bufa, bufb);

    const int my_t = tw + col;
    if (!w_ok || my_t >= p.seq_len) return;
    const int64_t row_el = ((int64_t)b * p.seq_len + my_t) * p.hq + head;
    uint16_t* op = reinterpret_cast<uint16_t*>(bp.dq) + row_el * D;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int cc4 = 0; cc4 < 4; ++cc4) {
            Vec8 w;
            w.w[0] = pack_bf16x2(dq[m][4 * cc4] * bp.scale, dq[m][4 * cc4 + 1] * bp.scale);
            w.w[1] = pack_bf16x2(dq[m][4 * cc4 + 2] * bp.scale, dq[m][4 * cc4 + 3] * bp.scale);
            *reinterpret_cast<Vec8*>(op + 32 * m + 8 * cc4 + 4 * h) = w;
        }
}

// dK / dV: one workgroup of 8 waves per (sequence, kv head, block of 256
// keys).  Wave w owns keys 32w .. 32w + 31 of the block: their K rows stay in
// registers (B operand of S = Q K^T), their dK^T and dV^T accumulate in
// registers; the block's V rows sit in LDS (B operand of dP = dO V^T).  The
// query positions that can see the block are walked in sub-tiles of 64
// stacked rows (the G heads of the group over 64/G positions); Q, dO, lse and
// Delta of a sub-tile are staged into one of two LDS buffers while the other
// is computed.  Per sub-tile each wave runs its two 32-row halves: S, P, dP,
// dS with the key on the lane and the query on the register, then
// dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T from transposing reads.
constexpr int kKB = 256;                                  // keys per block
constexpr int kSubRows = 64;                              // stacked query rows per sub-tile
constexpr int kSubRowBytes = kSubRows * kRowBytes;        // 16 KB of Q (or dO) rows
constexpr int kSubStage = 2 * kSubRowBytes + 2 * kSubRows * 4;  // Q, dO, lse, Delta
constexpr int kVBlock = kKB * kRowBytes;                  // 64 KB
constexpr size_t kDkdvLds = (size_t)kVBlock + 2 * kSubStage;

// dS of one 32-row half of a dK/dV sub-tile into the dS band (DsBand), as the
// dK/dV kernel holds it: key on the lane, sb[st] = rows 16 st + 4h + 0..3
// (words 0-1) and 16 st + 8 + 4h + 0..3 (words 2-3) of the half's stacked
// rows.  Those 16 rows are one head's (G <= 4: 16 or more positions per
// head in a sub-tile), so each st is one 16-byte store into the lane's own
// slot of the 1 KB half-tile that holds their positions.  Rows of a piece
// past the chunk or of missing heads get an offset past the resource (dsr:
// this sequence and kv head's part of the band), which the hardware drops,
// so the stores need no branch.  Non-temporal: the band is read once, by
// the dQ kernel, after this kernel has ended (measured 1.5% faster than
// plain stores).
template <int G>
__device__ inline void store_ds_native(const BwdParams& bp, const Vec16 (&sb)[2], i32x4 dsr, int greal, int ts,
                                       int half, int kb) {
    static_assert(G <= 4, "stored dS covers groups of up to 4 heads");
    constexpr int QS = kSubRows / G;
    const int lane = lane_now(), h = lane >> 5;
    const int rb = uniform_int((ts + (G == 1 ? 32 * half : 0)) >> 5);
    const int slot = kb < bp.ds_npre ? kb : bp.ds_npre + kb - rb + bp.ds_nwin - 1;
    const int tile0 = rb * bp.ds_nband + slot;  // tile index within one head's band
    // The piece starts at stacked row r = 32 half + 16 st + 4h: its head
    // r / QS does not depend on h (QS is a multiple of 16), its position is
    // ts + (r - 4h) % QS + 4h.
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int rr = 32 * half + 16 * st;  // the piece's row without the 4h
        const int hh = rr / QS;
        const int tu = uniform_int(ts + rr % QS);  // its position without the 4h
        const int base = uniform_int((hh * bp.ds_nrb * bp.ds_nband + tile0) * 2048 + ((tu & 31) >> 4) * 1024);
        const int voff = tu + 4 * h < bp.f.seq_len && hh < greal ? base + lane * 16 : (int)0x80000000u;
        i32x4 d;
        __builtin_memcpy(&d, &sb[st], 16);
        asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen nt" ::"v"(d), "v"(voff), "s"(dsr) : "memory");
    }
}

// DS: also store each half's dS into the band the dQ kernel reads.
template <int G, bool DS = false>
__global__ void __launch_bounds__(kThreads, 1) bwd_dkdv_kernel(BwdParams bp) {
    constexpr int D = 128;
    constexpr int QS = kSubRows / G;  // positions per sub-tile
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const PrefillParams& p = bp.f;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int T = p.seq_len, hq = p.hq, hkv = p.hkv;
    // heads of the group; with fewer than G the rows of the missing heads
    // load a real head's data and are masked out of P
    const int greal = hq / hkv;
    const bool padded = greal < G;
    const int n_kb = (T + kKB - 1) / kKB;
    const int S0 = (int)p.start_pos;
    const int P32 = p.P > 0x7FFFFFFF ? 0x7FFFFFFF : (int)p.P;
    // Key blocks holding prefix keys are seen by every later query, so they
    // take the longest: they get the first workgroup ids (dispatched first),
    // padded to a multiple of the XCD count; the other blocks follow, dealt
    // to the XCDs in contiguous runs of (sequence, kv head, block).
    int kb, g, b;
    {
        const int n_bg = hkv * p.batch;
        const int pre_pos = P32 - S0;  // prefix positions inside the chunk
        const int kb_pre = pre_pos <= 0 ? 0 : ((pre_pos < T ? pre_pos : T) + kKB - 1) / kKB;
        const int n_pre = kb_pre * n_bg;
        const int n_pre_pad = (n_pre + kXcds - 1) / kXcds * kXcds;
        const int id = (int)blockIdx.x;
        if (id < n_pre_pad) {
            if (id >= n_pre) return;
            kb = id % kb_pre;
            g = (id / kb_pre) % hkv;
            b = id / (kb_pre * hkv);
        } else {
            const int n_rest_kb = n_kb - kb_pre;
            const int work = xcd_remap(id - n_pre_pad, n_rest_kb * n_bg);
            kb = kb_pre + work % n_rest_kb;
            g = (work / n_rest_kb) % hkv;
            b = work / (n_rest_kb * hkv);
        }
    }
    const int w32 = p.W > 0x7FFFFFFF ? 0x7FFFFFFF : (int)p.W;
    const float c = p.scale_log2;

    const int kt0 = kb * kKB;                          // first key (chunk row) of the block
    const int nk = T - kt0 < kKB ? T - kt0 : kKB;
    const int wk0 = kt0 + 32 * wave;                   // this wave's first key
    const int wk_n = T - wk0 < 32 ? (T - wk0 > 0 ? T - wk0 : 0) : 32;
    const int jw0 = S0 + wk0, jw1 = jw0 + wk_n - 1;

    // K rows of this wave's keys (lane: key col, dims 16 kk + 8h .. + 7)
    Vec16 kreg[8];
    {
        const bool ok = col < wk_n;
        const uint16_t* kp = reinterpret_cast<const uint16_t*>(bp.k) +
                             (((int64_t)b * T + (ok ? wk0 + col : 0)) * hkv + g) * D;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            kreg[kk] = ok ? *reinterpret_cast<const Vec16*>(kp + 8 * h + 16 * kk) : Vec16{{0, 0, 0, 0}};
    }

    char* vblk = smem;
    char* stage0 = smem + kVBlock;
    // V rows of the block into LDS (K swizzle); rows past the chunk read as zero
    {
        const int rs = hkv * D * 2;
        const i32x4 vr = rsrc_words(static_cast<const char*>(bp.v) + (((int64_t)b * T + kt0) * hkv + g) * D * 2,
                                    nk * rs);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 32 * wave + 4 * i + (lane >> 4);
            dma16_asm(vr, row * rs + (((lane & 15) ^ b_chunk_swz(row)) << 4),
                      lds_addr(vblk) + (32 * wave + 4 * i) * kRowBytes);
        }
    }

    // query positions (chunk-relative) that can see a key of the block
    const int t_lo = kt0;
    const int64_t t_hi_w = (int64_t)kt0 + nk - 1 + w32 - 1;  // last query of the block's window
    const int t_hi = (S0 + kt0 < P32 || t_hi_w >= T - 1) ? T - 1 : (int)t_hi_w;
    const int s_first = t_lo / QS, s_last = t_hi / QS;
    const int n_sub = s_last - s_first + 1;

    // staging of sub-tile n: stacked row r = head offset r / QS, position
    // t = (s_first + n) QS + r % QS; wave w stages rows 8w .. 8w + 7 of Q and
    // dO; waves 0 and 1 stage the 64 lse and Delta values
    const int64_t qseq = (int64_t)b * T * hq;  // row index of (b, t = 0, head 0)
    const i32x4 qr = rsrc_words(static_cast<const char*>(p.q) + qseq * D * 2, T * hq * D * 2);
    const i32x4 dr = rsrc_words(static_cast<const char*>(bp.dout) + qseq * D * 2, T * hq * D * 2);
    const i32x4 xr = rsrc_words(wave == 0 ? (const void*)(bp.lse + qseq) : (const void*)(bp.delta + qseq), T * hq * 4);
    auto stage_sub = [&](int n, char* st) {
        const int ts = (s_first + n) * QS;
        const uint32_t sb = lds_addr(st);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = 8 * wave + 4 * i + (lane >> 4);
            const int t = ts + row % QS, head = g * greal + (row / QS < greal ? row / QS : 0);
            const int off = (t * hq + head) * D * 2 + (((lane & 15) ^ b_chunk_swz(row)) << 4);
            dma16_asm(qr, off, sb + (8 * wave + 4 * i) * kRowBytes);
            dma16_asm(dr, off, sb + kSubRowBytes + (8 * wave + 4 * i) * kRowBytes);
        }
        if (wave < 2) {
            const int t = ts + lane % QS, head = g * greal + (lane / QS < greal ? lane / QS : 0);
            dma4_asm(xr, (t * hq + head) * 4, sb + 2 * kSubRowBytes + wave * kSubRows * 4);
        }
    };
    if (n_sub > 0) stage_sub(0, stage0);
    if (n_sub > 1) {
        stage_sub(1, stage0 + kSubStage);
        if (wave < 2) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) asm volatile("" ::"v"(kreg[kk].w[0]));
    tile_barrier();

    uint32_t tr_off[2][4];
    kswz_tr_offsets(lane, tr_off);
    f32x16 dkacc[4], dvacc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkacc[m][r] = dvacc[m][r] = 0.f;

    // DS: this (sequence, kv head)'s part of the dS band as a buffer resource
    // (its size is below 2^31: the host uses the band only then)
    i32x4 dsr = {0, 0, 0, 0};
    if constexpr (DS)
        dsr = rsrc_words(bp.ds + ((int64_t)b * hq + g * greal) * bp.ds_nrb * bp.ds_nband * 2048,
                         greal * bp.ds_nrb * bp.ds_nband * 2048);
    for (int n = 0; n < n_sub; ++n) {
        const char* st = stage0 + (n & 1) * kSubStage;
        const char* qs = st;
        const char* ds_ = st + kSubRowBytes;
        const float* lse_s = reinterpret_cast<const float*>(st + 2 * kSubRowBytes);
        const float* dlt_s = lse_s + kSubRows;
        const int ts = (s_first + n) * QS;
        if (wk_n > 0) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                // positions of this half's 32 stacked rows
                const int iw0 = S0 + ts + (G == 1 ? 32 * half : 0);
                const int iw1 = iw0 + (QS < 32 ? QS : 32) - 1;
                const int cls = tile_class32(iw0, iw1, jw0, jw1, P32, w32);
                if (cls == kSkip) continue;
                const int qrow = 32 * half + col;
                const int vrow = 32 * wave + col;
                // S = Q K^T; register r holds query row 8(r/4) + 4h + r%4 of the
                // half, the lane's key col
                f32x16 s = {};
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const Vec16 qa = *reinterpret_cast<const Vec16*>(
                        qs + qrow * kRowBytes + (((2 * kk + h) ^ b_chunk_swz(qrow)) << 4));
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa), as_bf16x8(kreg[kk]), s, 0, 0, 0);
                }
                // P from the forward's log-sum-exp (fp32, kept for dS) and its bf16 operand
                const int my_j = jw0 + col;
                float pf[16];
                Vec16 pb[2], sb[2];
                // lse and Delta of the lane's rows come four at a time: rows
                // 8a + 4h .. 8a + 4h + 3 of the half (registers 4a .. 4a + 3) are
                // one 16-byte read, the same address for the 32 lanes of a half
                float4 l4;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qr_ = 32 * half + 8 * (r >> 2) + 4 * h + (r & 3);
                    if ((r & 3) == 0) l4 = *reinterpret_cast<const float4*>(lse_s + qr_);
                    const float lse_v = (r & 3) == 0 ? l4.x : (r & 3) == 1 ? l4.y : (r & 3) == 2 ? l4.z : l4.w;
                    float sv = s[r];
                    if (cls == kMasked || padded) {
                        const int i = S0 + ts + qr_ % QS;
                        const bool vis = my_j <= i && (my_j < P32 || my_j > i - w32) && col < wk_n &&
                                         qr_ / QS < greal;
                        sv = vis ? sv : -INFINITY;
                    }
                    pf[r] = fast_exp2(fmaf(sv, c, -lse_v * kLog2eF));
                }
#pragma unroll
                for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
                    for (int w = 0; w < 4; ++w) pb[st2].w[w] = pack_bf16x2(pf[8 * st2 + 2 * w], pf[8 * st2 + 2 * w + 1]);
                // dP = dO V^T, then dS = P (dP - Delta)
                f32x16 dp = {};
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const Vec16 da = *reinterpret_cast<const Vec16*>(
                        ds_ + qrow * kRowBytes + (((2 * kk + h) ^ b_chunk_swz(qrow)) << 4));
                    const Vec16 vb = *reinterpret_cast<const Vec16*>(
                        vblk + vrow * kRowBytes + (((2 * kk + h) ^ b_chunk_swz(vrow)) << 4));
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(da), as_bf16x8(vb), dp, 0, 0, 0);
                }
                float4 d4;
#pragma unroll
                for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        float dv2[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int r = 8 * st2 + 2 * w + e;
                            if ((r & 3) == 0) d4 = *reinterpret_cast<const float4*>(dlt_s + 32 * half + 8 * (r >> 2) + 4 * h);
                            const float dl = (r & 3) == 0 ? d4.x : (r & 3) == 1 ? d4.y : (r & 3) == 2 ? d4.z : d4.w;
                            dv2[e] = pf[r] * (dp[r] - dl);
                        }
                        sb[st2].w[w] = pack_bf16x2(dv2[0], dv2[1]);
                    }
                if constexpr (DS) store_ds_native<G>(bp, sb, dsr, greal, ts, half, kt0 / 32 + wave);
                const uint32_t qb_ = lds_addr(qs) + 32 * half * kRowBytes;
                const uint32_t db_ = lds_addr(ds_) + 32 * half * kRowBytes;
#pragma unroll
                for (int st2 = 0; st2 < 2; ++st2) {
                    Vec16 ta[4];
                    read_t_kswz(st2, db_, tr_off, ta);
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        dvacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ta[m]), as_bf16x8(pb[st2]), dvacc[m], 0, 0, 0);
                    read_t_kswz(st2, qb_, tr_off, ta);
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        dkacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ta[m]), as_bf16x8(sb[st2]), dkacc[m], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // (the dS stores count here too: a wait that let the last half's
        // stores stay in flight, vmcnt(2), measured no faster, and it would
        // rest on loads and stores completing in order)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        tile_barrier();
        if (n + 2 < n_sub) stage_sub(n + 2, stage0 + (n & 1) * kSubStage);
    }

    // The lane index is taken afresh here (mbcnt in asm, which the compiler
    // cannot equate with the one above): otherwise it keeps the lane-derived
    // values live across the loop and spills them at 256 VGPRs.
    int lane_e;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
    const int col_e = lane_e & 31, h_e = lane_e >> 5;
    if (col_e >= wk_n) return;
    const int64_t kel = (((int64_t)b * T + wk0 + col_e) * hkv + g) * D;
    uint16_t* dkp = reinterpret_cast<uint16_t*>(bp.dk) + kel;
    uint16_t* dvp = reinterpret_cast<uint16_t*>(bp.dv) + kel;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int cc4 = 0; cc4 < 4; ++cc4) {
            Vec8 wk, wv;
            wk.w[0] = pack_bf16x2(dkacc[m][4 * cc4] * bp.scale, dkacc[m][4 * cc4 + 1] * bp.scale);
            wk.w[1] = pack_bf16x2(dkacc[m][4 * cc4 + 2] * bp.scale, dkacc[m][4 * cc4 + 3] * bp.scale);
            wv.w[0] = pack_bf16x2(dvacc[m][4 * cc4], dvacc[m][4 * cc4 + 1]);
            wv.w[1] = pack_bf16x2(dvacc[m][4 * cc4 + 2], dvacc[m][4 * cc4 + 3]);
            *reinterpret_cast<Vec8*>(dkp + 32 * m + 8 * cc4 + 4 * h_e) = wk;
            *reinterpret_cast<Vec8*>(dvp + 32 * m + 8 * cc4 + 4 * h_e) = wv;
        }
}

}  // namespace

hipError_t launch_prefill(int dtype, int head_dim, int group, const PrefillParams& p, hipStream_t stream) {
    if (p.seq_len == 0) return hipSuccess;
    if (dtype == PS_BF16 && head_dim == 128 && group >= 1 && group <= 8) {
        group = layout_group(group);
        const int qp = 32 * kWaves / group;
        dim3 grid((unsigned)(((p.seq_len + qp - 1) / qp) * p.hkv * p.batch));
        const size_t lds = (size_t)kStages * kStageBytes;
        // the traced copy (phase trace) is a kernel of its own, with its own
        // LDS-limit flag
        const bool traced = p.trace != nullptr;
        const void* fn = nullptr;
        switch (group) {
            case 1: fn = traced ? (const void*)prefill_bf16_kernel<1, true> : (const void*)prefill_bf16_kernel<1>; break;
            case 2: fn = traced ? (const void*)prefill_bf16_kernel<2, true> : (const void*)prefill_bf16_kernel<2>; break;
            case 4: fn = traced ? (const void*)prefill_bf16_kernel<4, true> : (const void*)prefill_bf16_kernel<4>; break;
            case 8: fn = traced ? (const void*)prefill_bf16_kernel<8, true> : (const void*)prefill_bf16_kernel<8>; break;
            default: return hipErrorInvalidValue;
        }
        // raise the dynamic LDS limit once per kernel and device (a host call, not per launch)
        const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : 3;
        bool* set = lds_flag(traced ? 8 + gi : gi);
        if (!set || !*set) {
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            if (set) *set = true;
        }
        if (traced) {
            switch (group) {
                case 1: hipLaunchKernelGGL((prefill_bf16_kernel<1, true>), grid, dim3(kThreads), lds, stream, p); break;
                case 2: hipLaunchKernelGGL((prefill_bf16_kernel<2, true>), grid, dim3(kThreads), lds, stream, p); break;
                case 4: hipLaunchKernelGGL((prefill_bf16_kernel<4, true>), grid, dim3(kThreads), lds, stream, p); break;
                case 8: hipLaunchKernelGGL((prefill_bf16_kernel<8, true>), grid, dim3(kThreads), lds, stream, p); break;
            }
        } else {
            switch (group) {
                case 1: hipLaunchKernelGGL(prefill_bf16_kernel<1>, grid, dim3(kThreads), lds, stream, p); break;
                case 2: hipLaunchKernelGGL(prefill_bf16_kernel<2>, grid, dim3(kThreads), lds, stream, p); break;
                case 4: hipLaunchKernelGGL(prefill_bf16_kernel<4>, grid, dim3(kThreads), lds, stream, p); break;
                case 8: hipLaunchKernelGGL(prefill_bf16_kernel<8>, grid, dim3(kThreads), lds, stream, p); break;
            }
        }
        return hipGetLastError();
    }
    dim3 grid((unsigned)((p.seq_len + 63) / 64), (unsigned)p.hq, (unsigned)p.batch);
    if (dtype == PS_BF16 && head_dim == 64)
        hipLaunchKernelGGL((prefill_plain_kernel<uint16_t, 64>), grid, dim3(64), 0, stream, p);
    else if (dtype == PS_BF16 && head_dim == 128)
        hipLaunchKernelGGL((prefill_plain_kernel<uint16_t, 128>), grid, dim3(64), 0, stream, p);
    else if (head_dim == 64)
        hipLaunchKernelGGL((prefill_plain_kernel<float, 64>), grid, dim3(64), 0, stream, p);
    else if (head_dim == 128)
        hipLaunchKernelGGL((prefill_plain_kernel<float, 128>), grid, dim3(64), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

float* static_delta() {
    static std::mutex mu;
    static float* ptr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
        ptr[dev] = static_cast<float*>(addr);
    }
    return ptr[dev];
}

hipError_t launch_prefill_bwd(int group, const BwdParams& p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.f.batch * p.f.seq_len * p.f.hq;
    if (rows == 0) return hipSuccess;
    if (group < 1 || group > 8) return hipErrorInvalidValue;
    group = layout_group(group);
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(p.f.out), static_cast<const uint16_t*>(p.dout), p.delta_out, rows);
    const int qp = 32 * kWaves / group;
    const dim3 grid_q((unsigned)(((p.f.seq_len + qp - 1) / qp) * p.f.hkv * p.f.batch));
    // dK/dV grid: blocks holding prefix keys first (padded to a multiple of 8)
    const int64_t n_kb = (p.f.seq_len + kKB - 1) / kKB;
    const int64_t pre_pos = p.f.P - p.f.start_pos;
    const int64_t kb_pre = pre_pos <= 0 ? 0 : ((pre_pos < p.f.seq_len ? pre_pos : p.f.seq_len) + kKB - 1) / kKB;
    const int64_t n_bg = (int64_t)p.f.hkv * p.f.batch;
    const int64_t n_pre_pad = (kb_pre * n_bg + kXcds - 1) / kXcds * kXcds;
    const dim3 grid_k((unsigned)(n_pre_pad + (n_kb - kb_pre) * n_bg));
    const size_t lds_q = (size_t)kStages * kStageBytes;
    const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : 3;
    if (p.ds) {
        // dS stored by the dK/dV kernel, dQ from it (no second S and dP)
        const size_t lds_qd = (size_t)kStages * kTileBytes + (size_t)kWaves * 4 * kDsXpose;
        const void* fqd = nullptr;
        const void* fkd = nullptr;
        switch (group) {
            case 1: fqd = (const void*)bwd_dq_ds_kernel<1>; fkd = (const void*)bwd_dkdv_kernel<1, true>; break;
            case 2: fqd = (const void*)bwd_dq_ds_kernel<2>; fkd = (const void*)bwd_dkdv_kernel<2, true>; break;
            case 4: fqd = (const void*)bwd_dq_ds_kernel<4>; fkd = (const void*)bwd_dkdv_kernel<4, true>; break;
            default: return hipErrorInvalidValue;  // (the host uses the band for groups up to 4 only)
        }
        bool* set_d = lds_flag(12 + gi);
        if (!set_d || !*set_d) {
            hipError_t e = hipFuncSetAttribute(fqd, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_qd);
            if (e != hipSuccess) return e;
            e = hipFuncSetAttribute(fkd, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDkdvLds);
            if (e != hipSuccess) return e;
            if (set_d) *set_d = true;
        }
        switch (group) {
            case 1: hipLaunchKernelGGL((bwd_dkdv_kernel<1, true>), grid_k, dim3(kThreads), kDkdvLds, stream, p);
                    hipLaunchKernelGGL(bwd_dq_ds_kernel<1>, grid_q, dim3(kThreads), lds_qd, stream, p); break;
            case 2: hipLaunchKernelGGL((bwd_dkdv_kernel<2, true>), grid_k, dim3(kThreads), kDkdvLds, stream, p);
                    hipLaunchKernelGGL(bwd_dq_ds_kernel<2>, grid_q, dim3(kThreads), lds_qd, stream, p); break;
            case 4: hipLaunchKernelGGL((bwd_dkdv_kernel<4, true>), grid_k, dim3(kThreads), kDkdvLds, stream, p);
                    hipLaunchKernelGGL(bwd_dq_ds_kernel<4>, grid_q, dim3(kThreads), lds_qd, stream, p); break;
        }
        return hipGetLastError();
    }
    const void* fq = nullptr;
    const void* fk = nullptr;
    switch (group) {
        case 1: fq = (const void*)bwd_dq_kernel<1>; fk = (const void*)bwd_dkdv_kernel<1>; break;
        case 2: fq = (const void*)bwd_dq_kernel<2>; fk = (const void*)bwd_dkdv_kernel<2>; break;
        case 4: fq = (const void*)bwd_dq_kernel<4>; fk = (const void*)bwd_dkdv_kernel<4>; break;
        case 8: fq = (const void*)bwd_dq_kernel<8>; fk = (const void*)bwd_dkdv_kernel<8>; break;
        default: return hipErrorInvalidValue;
    }
    bool* set = lds_flag(4 + gi);
    if (!set || !*set) {
        hipError_t e = hipFuncSetAttribute(fq, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_q);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(fk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDkdvLds);
        if (e != hipSuccess) return e;
        if (set) *set = true;
    }
    // dK/dV first: its prefix blocks are the longest workgroups of the two
    // launches (measured 1.3% faster than dQ first; running the two on two
    // streams gained nothing)
    switch (group) {
        case 1: hipLaunchKernelGGL(bwd_dkdv_kernel<1>, grid_k, dim3(kThreads), kDkdvLds, stream, p);
                hipLaunchKernelGGL(bwd_dq_kernel<1>, grid_q, dim3(kThreads), lds_q, stream, p); break;
        case 2: hipLaunchKernelGGL(bwd_dkdv_kernel<2>, grid_k, dim3(kThreads), kDkdvLds, stream, p);
                hipLaunchKernelGGL(bwd_dq_kernel<2>, grid_q, dim3(kThreads), lds_q, stream, p); break;
        case 4: hipLaunchKernelGGL(bwd_dkdv_kernel<4>, grid_k, dim3(kThreads), kDkdvLds, stream, p);
                hipLaunchKernelGGL(bwd_dq_kernel<4>, grid_q, dim3(kThreads), lds_q, stream, p); break;
        case 8: hipLaunchKernelGGL(bwd_dkdv_kernel<8>, grid_k, dim3(kThreads), kDkdvLds, stream, p);
                hipLaunchKernelGGL(bwd_dq_kernel<8>, grid_q, dim3(kThreads), lds_q, stream, p); break;
    }
    return hipGetLastError();
}

}  // namespace ps
