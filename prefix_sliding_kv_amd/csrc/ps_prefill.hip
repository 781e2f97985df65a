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
// bf16 path (head_dim 128): a workgroup of 4 waves owns 128 query rows, the G
// heads of one GQA group stacked over 128/G positions, so every K/V tile
// staged in LDS serves all heads that share it.  Per 64-key tile each wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (a lane then holds 16
// scores of a single query, so the online softmax needs one cross-lane step),
// and O^T += V^T P^T with the same instruction, reading V from a transposed
// LDS copy written while staging.  The next tile's global loads are issued
// before the current tile's math (register prefetch, two LDS buffers, one
// barrier per tile).  fp32 path: a plain debug kernel with the same tile
// walk and classification.
#include "ps_internal.h"

namespace ps {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBN = 64;  // keys per tile

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
};

__device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

// v_exp_f32 without the denormal-range fix-up of exp2f: results below 2^-126
// flush to zero, which is below the rounding error of any softmax row sum
// (every row has a term equal to 1 at its running reference).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline void plan_walk(const PrefillParams& p, int64_t i0, int64_t i1, TileWalk& w) {
    w.n_ranges = 0;
    for (int r = 0; r < p.n_runs; ++r) {
        const KeyRun& run = p.runs[r];
        const int64_t n = run.n;
        if (n <= 0) continue;
        // prefix part: positions < min(P, i1 + 1)
        const int64_t hiA = clamp64((p.P < i1 + 1 ? p.P : i1 + 1) - run.pos0, 0, n);
        // window part: positions in [i0 - W + 1, i1]
        const int64_t loB = clamp64(i0 - p.W + 1 - run.pos0, 0, n);
        const int64_t hiB = clamp64(i1 + 1 - run.pos0, 0, n);
        const int endA = (int)((hiA + kBN - 1) / kBN);
        int begB = (int)(loB / kBN);
        const int endB = hiB > loB ? (int)((hiB + kBN - 1) / kBN) : 0;
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

constexpr int kKStride = 128 * 2;       // bytes per K row in LDS; 16-byte chunks xor-swizzled by row & 15
constexpr int kVStride = kBN * 2;       // bytes per transposed V row (one head dimension), unpadded
constexpr int kKBytes = kBN * kKStride;
constexpr int kVBytes = 128 * kVStride;
constexpr int kStageBytes = kKBytes + kVBytes;

// Transposed V layout.  Row = head dimension, 64 keys of 2 bytes.  Keys are
// stored in the order the P.V MFMA consumes them: the 8 keys lane half h
// needs for k-step st (keys 16st + 8a + 4h + c, a, c in {0,1},{0..3}) sit in
// columns 16st + 8h + 4a + c, i.e. key bits 2 and 3 swapped, so one 16-byte
// read fetches them.  The 16-byte chunk of a row is xor-swizzled by
// ((row >> 3) ^ row) & 7 so that both the staging writes and the operand
// reads hit all LDS banks once.
__device__ inline int vt_chunk_swz(int row) { return ((row >> 3) ^ row) & 7; }
__device__ inline int swap01(int x) { return (x & ~3) | ((x & 1) << 1) | ((x >> 1) & 1); }
// staging thread -> (dim group 0..15, key group 0..15) for V
__device__ inline int v_dim_group(int t) { return (t & 7) | (((t >> 4) & 1) << 3); }
__device__ inline int v_key_group(int t) { return (((t >> 3) & 1) << 1) | ((t >> 5) & 1) | ((t >> 6) << 2); }

__device__ inline int k_chunk_swz(int row) { return row & 15; }

// Bits [lo, hi) of a 32-bit word, with lo and hi clamped to [0, 32].
__device__ inline uint32_t range_bits(int lo, int hi) {
    lo = lo < 0 ? 0 : (lo > 32 ? 32 : lo);
    hi = hi < 0 ? 0 : (hi > 32 ? 32 : hi);
    if (hi <= lo) return 0u;
    return (uint32_t)((((uint64_t)1 << hi) - 1) ^ (((uint64_t)1 << lo) - 1));
}

struct TileRegs {
    Vec16 v[4];
};

// Buffer resource (V#) over [base, base + bytes): loads at offsets past the
// end return zero, so partial tiles need no per-lane checks.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Stage one 64-key tile: K goes straight from global memory into LDS
// (buffer_load ... lds, 16 bytes per lane at LDS base + lane * 16; each lane
// picks the global chunk that belongs at its swizzled LDS position), V is
// loaded to registers for the transposed store.  Both use a buffer resource
// limited to the run's rows, so rows past the end read as zero (those keys are
// masked out of the softmax; their zero V rows contribute nothing).
__device__ inline void load_tile_bf16(const RunView& run, int tile, int tid, char* stage, TileRegs& t) {
    const int row0 = tile * kBN;
    const int rs = run.row_bytes;
    const int nrows = run.n - row0 < kBN ? run.n - row0 : kBN;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(run.k + (int64_t)row0 * rs, nrows * rs);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(run.v + (int64_t)row0 * rs, nrows * rs);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * i + (lane >> 4);
        const int chunk = (lane & 15) ^ k_chunk_swz(row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (__attribute__((address_space(3))) void*)(stage + (16 * wave + 4 * i) * kKStride), 16,
            row * rs + chunk * 16, 0, 0, 0);
    }
    const int vpiece = v_dim_group(tid), vrow = 4 * v_key_group(tid);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vr, (vrow + i) * rs + vpiece * 16, 0, 0);
        __builtin_memcpy(&t.v[i], &x, 16);
    }
}

__device__ inline void store_tile_bf16(char* stage, int tid, const TileRegs& t) {
    char* vs = stage + kKBytes;
    // transpose: this thread holds keys 4kg..4kg+3 of dims 8dg..8dg+7
    const int dg = v_dim_group(tid);
    const int col = 4 * swap01(v_key_group(tid));  // permuted key column of the 4 keys
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        Vec8 o;
        o.w[0] = __builtin_amdgcn_perm(t.v[1].w[w], t.v[0].w[w], sel);
        o.w[1] = __builtin_amdgcn_perm(t.v[3].w[w], t.v[2].w[w], sel);
        const int row = 8 * dg + e;
        *reinterpret_cast<Vec8*>(vs + row * kVStride + (((col >> 3) ^ vt_chunk_swz(row)) << 4) + (col & 7) * 2) = o;
    }
}

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

// Scheduling recipe for a region with N LDS operand reads each feeding QB
// MFMAs: issue 4 reads, then alternate one MFMA group with one read, then the
// remaining MFMAs, so four reads are always in flight ahead of their use.
template <int N, int QB>
__device__ inline void pipeline_reads_and_mfma() {
    constexpr int kAhead = 4;
#pragma unroll
    for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
#pragma unroll
    for (int i = 0; i < N - kAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
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

// A workgroup of 4 waves owns 128*QB query rows: the G heads of a GQA group
// stacked over 128*QB/G positions.  Each wave owns QB blocks of 32 rows, so
// every K or V operand it reads from LDS feeds QB MFMAs; K and V operands of
// a 32-key block are read into registers before the MFMAs that use them.
template <int G, int QB>
__global__ void __launch_bounds__(256, QB == 1 ? 2 : 1) prefill_bf16_kernel(PrefillParams p) {
    constexpr int D = 128;
    constexpr int QP = 128 * QB / G;  // positions per query tile
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, col = lane & 31;
    // Workgroups are dealt to the 8 XCDs round-robin by linear id; give each
    // XCD a contiguous run of (sequence, kv head, q tile) work so the
    // workgroups sharing an L2 walk neighbouring q tiles of the same head,
    // whose key windows overlap almost entirely.
    const int n_qt = (p.seq_len + QP - 1) / QP;
    const int work = xcd_remap((int)blockIdx.x, n_qt * p.hkv * p.batch);
    const int qt = work % n_qt, g = (work / n_qt) % p.hkv, b = work / (n_qt * p.hkv);

    const int64_t t0 = (int64_t)qt * QP;       // first chunk row of the tile
    const int64_t t_last = (t0 + QP < p.seq_len ? t0 + QP : p.seq_len) - 1;
    const int64_t i0 = p.start_pos + t0;
    const int64_t i1 = p.start_pos + t_last;
    const float c = p.scale_log2;                              // > 0 (checked on the host)
    const int w32 = p.W > (1 << 30) ? (1 << 30) : (int)p.W;    // a window beyond every position is the same

    // this lane's query in each block: stacked row 32*(QB*wave + qb) + col
    int head[QB];
    int64_t my_t[QB], my_i[QB];
    bool q_ok[QB];
    Vec16 qreg[QB][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = 32 * (QB * wave + qb) + col;
        head[qb] = g * G + row / QP;
        my_t[qb] = t0 + row % QP;
        q_ok[qb] = my_t[qb] < p.seq_len;
        my_i[qb] = p.start_pos + my_t[qb];
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) +
                             (((int64_t)b * p.seq_len + (q_ok[qb] ? my_t[qb] : 0)) * p.hq + head[qb]) * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qreg[qb][ks] = q_ok[qb] ? *reinterpret_cast<const Vec16*>(qp + 8 * h + 16 * ks) : Vec16{{0, 0, 0, 0}};
    }

    __shared__ TileWalk walk;
    __shared__ RunView views[kMaxRuns];
    if (tid == 0) {
        plan_walk(p, i0, i1, walk);
        for (int r = 0; r < p.n_runs; ++r) {
            const KeyRun& run = p.runs[r];
            const int64_t seq = run.rows ? (int64_t)run.rows[b] : (int64_t)b;
            const int64_t base_el = seq * run.seq_stride + (int64_t)g * run.head_stride;
            views[r].k = static_cast<const char*>(run.k) + base_el * 2;
            views[r].v = static_cast<const char*>(run.v) + base_el * 2;
            views[r].pos0 = run.pos0;
            views[r].n = (int)run.n;
            views[r].row_bytes = (int)(run.row_stride * 2);
        }
    }
    __syncthreads();
    int total = 0;
    for (int r = 0; r < walk.n_ranges; ++r) total += walk.end[r] - walk.begin[r];

    f32x16 o[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][m][r] = 0.f;
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
    }

    int cr = 0, ct = walk.n_ranges ? walk.begin[0] : 0;  // cursor (range, tile)
    TileRegs regs;
    if (total > 0) {
        load_tile_bf16(views[walk.run[0]], ct, tid, smem, regs);
        store_tile_bf16(smem, tid, regs);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // direct-to-LDS K loads landed
    __syncthreads();

    for (int f = 0; f < total; ++f) {
        const int run_idx = walk.run[cr];
        const int tile = ct;
        // advance the cursor and prefetch the next tile
        if (++ct >= walk.end[cr]) {
            ++cr;
            if (cr < walk.n_ranges) ct = walk.begin[cr];
        }
        const bool has_next = f + 1 < total;
        if (has_next) load_tile_bf16(views[walk.run[cr]], ct, tid, smem + ((f + 1) & 1) * kStageBytes, regs);

        const int row0 = tile * kBN;
        const int run_n = views[run_idx].n;
        const int nrows = run_n - row0 < kBN ? run_n - row0 : kBN;
        const int64_t j0 = views[run_idx].pos0 + row0;
        const int64_t j1 = j0 + nrows - 1;
        const int cls = nrows < kBN ? kMasked : tile_class(i0, i1, j0, j1, p.P, p.W);

        const char* stage = smem + (f & 1) * kStageBytes;
        const char* ks_lds = stage;
        const char* vs_lds = stage + kKBytes;
        __builtin_amdgcn_sched_barrier(0);

        // S^T = K Q^T (raw scores, unscaled).  The 16 K operands of the tile
        // are read from LDS once and feed QB MFMAs each; the schedule keeps
        // four reads in flight ahead of the MFMAs.
        f32x16 s[QB][2];
        {
            Vec16 ka[2][8];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int krow = 32 * mb + col;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
                    ka[mb][kk] = *reinterpret_cast<const Vec16*>(ks_lds + krow * kKStride + (((2 * kk + h) ^ k_chunk_swz(krow)) << 4));
            }
            const f32x16 zero = {};
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        s[qb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[mb][kk]), as_bf16x8(qreg[qb][kk]),
                                                                            kk == 0 ? zero : s[qb][mb], 0, 0, 0);
            pipeline_reads_and_mfma<16, QB>();
        }
        __builtin_amdgcn_sched_barrier(0);
        // Elementwise mask, straddling tiles only.  For this lane's query the
        // visible keys of the tile (tile-relative index kr) form at most two
        // intervals: [0, min(pj, hic + 1)) -- the prefix -- and
        // [max(relw + 1, 0), hic + 1) -- the window -- with rel = i - j0,
        // relw = rel - W, pj = P - j0, hic = min(rel, nrows - 1).  They become
        // one 32-bit bitmap per 32-key block, and each score is kept or set to
        // -inf with a bit extract and a bitfield select (no per-element compares).
        if (cls == kMasked) {
            const int64_t pj64 = p.P - j0;
            const int pj = pj64 > (1 << 30) ? (1 << 30) : (pj64 < -(1 << 30) ? -(1 << 30) : (int)pj64);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int rel = (int)(my_i[qb] - j0);
                const int hic = rel < nrows - 1 ? rel : nrows - 1;
                const int a_hi = pj < hic + 1 ? pj : hic + 1;
                const int b_lo = rel - w32 + 1 > 0 ? rel - w32 + 1 : 0;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const uint32_t bits = range_bits(0, a_hi - 32 * mb) | range_bits(b_lo - 32 * mb, hic + 1 - 32 * mb);
                    const uint32_t bits_h = bits >> (4 * h);  // this lane half's keys start at bit 4h
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int keep = __builtin_amdgcn_sbfe((int)bits_h, 8 * (r >> 2) + (r & 3), 1);  // 0 or -1
                        const uint32_t km = (uint32_t)keep;
                        s[qb][mb][r] = __uint_as_float((km & __float_as_uint(s[qb][mb][r])) | (~km & 0xFF800000u));
                    }
                }
            }
        }
        // online softmax in raw-score units; exp2((s - m) * c) as one FMA + exp
        Vec16 pb[QB][4];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float tmax = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[qb][mb][r]);
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            // The exponent reference only moves when some row's maximum
            // exceeds it by more than 8 (log2 units): until then terms stay
            // below 2^8, and since l and O share the reference the result is
            // the same.
            if (__any(tmax * c > m_run[qb] * c + 8.f)) {
                const float m_new = fmaxf(m_run[qb], tmax);
                const float alpha = m_run[qb] == -INFINITY ? 0.f : fast_exp2((m_run[qb] - m_new) * c);
                l_run[qb] *= alpha;
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[qb][m][r] *= alpha;
                m_run[qb] = m_new;
            }
            const float mc = m_run[qb] == -INFINITY ? 0.f : m_run[qb] * c;
            // P^T as B operand: k-step st covers keys 16 st .. 16 st + 15
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int mb = st >> 1, base = 8 * (st & 1);
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    pb[qb][st].w[w] = pack_bf16x2(fast_exp2(fmaf(s[qb][mb][base + 2 * w], c, -mc)),
                                                  fast_exp2(fmaf(s[qb][mb][base + 2 * w + 1], c, -mc)));
                l_run[qb] += sum_bf16x8(pb[qb][st]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // O^T += V^T P^T: the 16 V operands are read once and feed QB MFMAs
        // each, with the same read-ahead schedule.
        {
            Vec16 va[4][4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int dim = 32 * m + col;
                const char* vrow = vs_lds + dim * kVStride;
                const int swz = vt_chunk_swz(dim);
#pragma unroll
                for (int st = 0; st < 4; ++st) va[m][st] = *reinterpret_cast<const Vec16*>(vrow + (((2 * st + h) ^ swz) << 4));
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o[qb][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[m][st]), as_bf16x8(pb[qb][st]),
                                                                           o[qb][m], 0, 0, 0);
            pipeline_reads_and_mfma<16, QB>();
        }
        __builtin_amdgcn_sched_barrier(0);

        if (has_next) store_tile_bf16(smem + ((f + 1) & 1) * kStageBytes, tid, regs);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // direct-to-LDS K loads landed
        __syncthreads();
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
        if (!q_ok[qb]) continue;
        const float inv = 1.f / l_tot;
        uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + (((int64_t)b * p.seq_len + my_t[qb]) * p.hq + head[qb]) * D;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                Vec8 w;
                w.w[0] = pack_bf16x2(o[qb][m][4 * cc] * inv, o[qb][m][4 * cc + 1] * inv);
                w.w[1] = pack_bf16x2(o[qb][m][4 * cc + 2] * inv, o[qb][m][4 * cc + 3] * inv);
                *reinterpret_cast<Vec8*>(op + 32 * m + 8 * cc + 4 * h) = w;
            }
        if (p.lse && h == 0)
            p.lse[((int64_t)b * p.seq_len + my_t[qb]) * p.hq + head[qb]] = (m_run[qb] * c + log2f(l_tot)) * kLn2;
    }
}

// ----------------------------------------------------------------- fp32 debug
// One thread per query row of a 64-position tile of one q head; K/V tiles in
// LDS; two passes per tile (scores for the tile maximum, then the weighted sum).
template <int D>
__global__ void __launch_bounds__(64) prefill_f32_kernel(PrefillParams p) {
    constexpr int BR = 32;  // rows staged per LDS fill (two fills per 64-key tile)
    __shared__ float ks[BR][D];
    __shared__ float vs[BR][D];
    __shared__ TileWalk walk;
    const int tid = threadIdx.x;
    const int qt = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
    const int group = p.hq / p.hkv;
    const int g = head / group;
    const int64_t t0 = (int64_t)qt * 64;
    const int64_t t_last = (t0 + 64 < p.seq_len ? t0 + 64 : p.seq_len) - 1;
    const int64_t i0 = p.start_pos + t0, i1 = p.start_pos + t_last;
    const int64_t my_t = t0 + tid;
    const bool q_ok = my_t < p.seq_len;
    const int64_t my_i = p.start_pos + my_t;

    float q[D], o[D];
    const float* qp = reinterpret_cast<const float*>(p.q) + (((int64_t)b * p.seq_len + (q_ok ? my_t : 0)) * p.hq + head) * D;
    for (int e = 0; e < D; ++e) {
        q[e] = q_ok ? qp[e] * p.scale_log2 : 0.f;
        o[e] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;

    if (tid == 0) plan_walk(p, i0, i1, walk);
    __syncthreads();
    for (int rr = 0; rr < walk.n_ranges; ++rr) {
        const KeyRun& run = p.runs[walk.run[rr]];
        const int64_t seq = run.rows ? (int64_t)run.rows[b] : (int64_t)b;
        const float* kb = reinterpret_cast<const float*>(run.k) + seq * run.seq_stride + (int64_t)g * run.head_stride;
        const float* vb = reinterpret_cast<const float*>(run.v) + seq * run.seq_stride + (int64_t)g * run.head_stride;
        for (int tile = walk.begin[rr]; tile < walk.end[rr]; ++tile) {
            const int64_t row0 = (int64_t)tile * kBN;
            const int64_t nrows = run.n - row0 < kBN ? run.n - row0 : kBN;
            const int64_t j0 = run.pos0 + row0;
            const int cls = nrows < kBN ? kMasked : tile_class(i0, i1, j0, j0 + nrows - 1, p.P, p.W);
            if (cls == kSkip) continue;
            for (int pass = 0; pass < 2; ++pass) {
                float tmax = -INFINITY;
                for (int half = 0; half < kBN / BR; ++half) {
                    __syncthreads();
                    for (int idx = tid; idx < BR * D; idx += 64) {
                        const int r = idx / D, e = idx % D;
                        const int64_t row = half * BR + r;
                        const bool ok = row < nrows;
                        ks[r][e] = ok ? kb[(row0 + row) * run.row_stride + e] : 0.f;
                        vs[r][e] = ok ? vb[(row0 + row) * run.row_stride + e] : 0.f;
                    }
                    __syncthreads();
                    for (int r = 0; r < BR; ++r) {
                        const int64_t row = half * BR + r;
                        float acc = 0.f;
                        for (int e = 0; e < D; ++e) acc = fmaf(q[e], ks[r][e], acc);
                        if (cls == kMasked && (row >= nrows || !visible(my_i, j0 + row, p.P, p.W))) acc = -INFINITY;
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
    float* op = reinterpret_cast<float*>(p.out) + (((int64_t)b * p.seq_len + my_t) * p.hq + head) * D;
    for (int e = 0; e < D; ++e) op[e] = o[e] / l_run;
    if (p.lse) p.lse[((int64_t)b * p.seq_len + my_t) * p.hq + head] = (m_run + log2f(l_run)) * kLn2;
}

}  // namespace

hipError_t launch_prefill(int dtype, int head_dim, int group, const PrefillParams& p, hipStream_t stream) {
    if (p.seq_len == 0) return hipSuccess;
    if (dtype == PS_BF16) {
        if (head_dim != 128) return hipErrorInvalidValue;
        constexpr int QB = 1;
        const int qp = 128 * QB / group;
        dim3 grid((unsigned)(((p.seq_len + qp - 1) / qp) * p.hkv * p.batch));
        const size_t lds = 2 * kStageBytes;
        const void* fn = nullptr;
        switch (group) {
            case 1: fn = (const void*)prefill_bf16_kernel<1, QB>; break;
            case 2: fn = (const void*)prefill_bf16_kernel<2, QB>; break;
            case 4: fn = (const void*)prefill_bf16_kernel<4, QB>; break;
            case 8: fn = (const void*)prefill_bf16_kernel<8, QB>; break;
            default: return hipErrorInvalidValue;
        }
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        switch (group) {
            case 1: hipLaunchKernelGGL((prefill_bf16_kernel<1, QB>), grid, dim3(256), lds, stream, p); break;
            case 2: hipLaunchKernelGGL((prefill_bf16_kernel<2, QB>), grid, dim3(256), lds, stream, p); break;
            case 4: hipLaunchKernelGGL((prefill_bf16_kernel<4, QB>), grid, dim3(256), lds, stream, p); break;
            case 8: hipLaunchKernelGGL((prefill_bf16_kernel<8, QB>), grid, dim3(256), lds, stream, p); break;
        }
        return hipGetLastError();
    }
    dim3 grid((unsigned)((p.seq_len + 63) / 64), (unsigned)p.hq, (unsigned)p.batch);
    if (head_dim == 64)
        hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(64), 0, stream, p);
    else if (head_dim == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(64), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ps
