// Decode attention for Prefix Sliding on gfx950.
//
// One query per sequence.  The keys a decode query at position i may see are
// the prefix positions [0, min(P, i+1)) and the window positions (i-W, i]
// (njhaofan.com article, section "PrefixSliding如何丢掉中间Token？"; agihunt.info
// summary, paragraph on the two kept slices).  Those are exactly the rows the
// cache retains, so no elementwise mask is needed: the kernel streams the
// prefix rows and the filled ring rows of each (sequence, kv head), in any
// order, because softmax does not depend on key order.
//
// This is memory-bound work (2 * Hkv * d * (P+W) * sizeof(bf16) bytes per
// layer and token against a few flops per byte), so the design is about HBM
// streaming, not matrix cores:
//   * one workgroup per (split, kv head, sequence); a split owns R consecutive key rows
//     and issues every 16-byte K and V load of its rows before doing any math,
//     so each CU keeps tens of KB in flight;
//   * a K row of d elements is read by LPR = d*sizeof(T)/16 adjacent lanes
//     (one fully coalesced 16-byte load each); the q.k partial sums are
//     combined with DPP row rotations inside each 16-lane row;
//   * the G query heads of a GQA group share every K/V load;
//   * each split writes an unnormalised partial (m, l, o[d]) per query head;
//     the last split to finish (atomic arrival counter, self-resetting) merges
//     them with the log-sum-exp rule and writes the output, so a layer is one
//     launch;
//   * the fused variant also writes the new token's K/V row into its slot and
//     serves that row from the input instead of the cache.
#include "ps_internal.h"

namespace ps {
namespace {

constexpr float kLn2 = 0.6931471805599453f;

struct alignas(16) Vec16 {
    uint32_t w[4];
};

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {  // bfloat16 storage
    static constexpr int kPerVec = 8;
    __device__ static inline void unpack(const Vec16& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v.w[i] << 16);
            f[2 * i + 1] = __uint_as_float(v.w[i] & 0xFFFF0000u);
        }
    }
    // 8-element dot product: packed bf16 pairs, products exact, fp32 sums
    __device__ static inline float dot(const Vec16& a, const Vec16& b) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x2 x, y;
            __builtin_memcpy(&x, &a.w[i], 4);
            __builtin_memcpy(&y, &b.w[i], 4);
            acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
        }
        return acc;
    }
    __device__ static inline uint16_t from_float(float x) {
        // round to nearest even; NaN stays NaN
        uint32_t u = __float_as_uint(x);
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
        u += 0x7FFFu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
};
template <>
struct Elem<float> {
    static constexpr int kPerVec = 4;
    __device__ static inline void unpack(const Vec16& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v.w[i]);
    }
    __device__ static inline float dot(const Vec16& a, const Vec16& b) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(a.w[i]), __uint_as_float(b.w[i]), acc);
        return acc;
    }
    __device__ static inline float from_float(float x) { return x; }
};

template <int CTRL>
__device__ inline float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR adjacent lanes; every lane of a group gets the total.
template <int LPR>
__device__ inline float group_sum(float x) {
    if constexpr (LPR == 16) {
        // row_ror:n rotates within each 16-lane row (DPP control 0x120 + n)
        x += dpp_f<0x128>(x);
        x += dpp_f<0x124>(x);
        x += dpp_f<0x122>(x);
        x += dpp_f<0x121>(x);
        return x;
    } else {
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
        return x;
    }
}

__device__ inline Vec16 load16(const void* p) { return *reinterpret_cast<const Vec16*>(p); }
// The same load, optionally with the non-temporal hint (data read once, not
// worth keeping in the caches).
template <bool NT>
__device__ inline Vec16 load16_stream(const void* p) {
    if constexpr (NT) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        Vec16 r;
        r.w[0] = x[0];
        r.w[1] = x[1];
        r.w[2] = x[2];
        r.w[3] = x[3];
        return r;
    } else {
        return load16(p);
    }
}

// Split partials cross workgroups that may sit on different XCDs (separate
// L2s): they are written and read with agent-scope atomic accesses, which
// the hardware keeps coherent across the device without cache maintenance.
__device__ inline void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// v_exp_f32 without the denormal-range fix-up of exp2f.  Every argument here
// is a score minus a maximum over a set that contains it (so <= 0), and a
// result below 2^-126 is far below the rounding error of a sum that holds a
// term equal to 1.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the row groups of a wave: lanes that hold the same slice
// (lane % LPR) of different key rows.  Lane pairs l, l ^ 8 inside a 16-lane
// row meet through a DPP rotation; l, l ^ 16 and l, l ^ 32 through the
// permlane swaps, which leave the value of each lane and of its partner in
// the two results, in an order that depends on the lane, so a symmetric op
// of the pair gives the same answer on both lanes.
template <int LPR>
__device__ inline float rowgroup_sum(float x) {
    if constexpr (LPR <= 8) x += dpp_f<0x128>(x);
    if constexpr (LPR <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (LPR <= 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}
template <int LPR>
__device__ inline float rowgroup_max(float x) {
    if constexpr (LPR <= 8) x = fmaxf(x, dpp_f<0x128>(x));
    if constexpr (LPR <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (LPR <= 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return x;
}

// A wave-uniform address in scalar registers, for scalar loads written in asm
// (an address the compiler happened to form in vector registers would not
// assemble there).
template <typename P>
__device__ inline P* sgpr_ptr(P* ptr) {
    const uint64_t a = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// Phase timestamp of a traced launch (thread 0 of each workgroup).
__device__ inline void trace_mark(const DecodeParams& p, int point) {
    p.trace[(size_t)blockIdx.x * kDecodeTracePoints + point] = __builtin_amdgcn_s_memrealtime();
}

// PAGED: the paged cache layout.  The split rows are then fixed logical rows
// of the sequence -- [0, pcap) its prefix slots, [pcap, pcap + W) its ring
// slots, valid while filled -- so the page of a row is table entry
// row / page, known before the sequence metadata arrives; a wave's rows
// (U * RPW consecutive rows, at most 128) lie in one page.
template <typename T, int D, int G, int NW, int U, bool NTL, bool TRACE = false, bool PAGED = false>
__global__ void __launch_bounds__(NW * 64) decode_kernel(DecodeParams p) {
    constexpr int NT = NW * 64;
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int LPR = D / VEC;          // lanes per key row
    constexpr int RPW = 64 / LPR;         // rows per wave per load instruction
    constexpr int R = NW * RPW * U;       // rows per split
    constexpr int PAIRS = G * D;          // (head, dim) outputs of a group
    static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row must map onto a wave");

    // per-wave partials; maxima, sums and weights with the wave index
    // innermost so a reader takes them with 16-byte LDS reads
    __shared__ __attribute__((aligned(16))) float s_m[G][NW];
    __shared__ __attribute__((aligned(16))) float s_l[G][NW];
    __shared__ __attribute__((aligned(16))) float s_w[G][NW];
    __shared__ float s_ref[G];
    __shared__ float s_o[NW][G * D];
    __shared__ int s_last;

    // 1-D grid, group (sequence, kv head) fastest: the workgroups of one
    // group share blockIdx % 8 whenever the group count is a multiple of 8, so
    // the hardware's round-robin deal puts them on one XCD (one L2); measured
    // 3% faster at batch 1 than the (split, kv head, sequence) grid.
    if constexpr (TRACE) {
        if (threadIdx.x == 0) {
            trace_mark(p, 0);
            p.trace[(size_t)blockIdx.x * kDecodeTracePoints + 7] = 0;
        }
    }
    const int n_groups = p.n_seqs * p.c.hkv;
    // (the divisions run through the vector unit: readfirstlane keeps the
    // results, and every address made from them, in scalar registers)
    const int group = __builtin_amdgcn_readfirstlane((int)blockIdx.x % n_groups);
    const int split = __builtin_amdgcn_readfirstlane((int)blockIdx.x / n_groups);
    const int g = __builtin_amdgcn_readfirstlane(group % p.c.hkv), b = __builtin_amdgcn_readfirstlane(group / p.c.hkv);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address arithmetic
    const int sub = lane % LPR, rg = lane / LPR;

    // paged: the page of this wave's rows (independent of the metadata)
    const int64_t wave_row0 = (int64_t)split * R + (int64_t)wave * U * RPW;
    // (a wave wholly past the last row reads entry 0; its loads are masked off)
    const int64_t wave_page =
        PAGED ? (int64_t)p.c.pages[(int64_t)b * p.c.pages_per_seq +
                                   (wave_row0 < p.rows_per_head ? (wave_row0 >> p.c.page_shift) : 0)]
              : 0;
    // Metadata first: prefix length, position, the sequence's blocks and the
    // debug-check flag word (when checks are off any readable word stands in
    // and its value is ignored) are five scalar loads issued back to back
    // and waited for once.  Left to the compiler they were spaced by a
    // round trip each, which put about a microsecond before the first K load.
    const uint32_t* guard_p = p.c.guard ? p.c.guard : reinterpret_cast<const uint32_t*>(p.plen);
    int32_t P32, crow32, prow32;
    int64_t i;
    uint32_t guard_v;
    asm volatile(
        "s_load_dword %0, %5, 0x0\n\t"
        "s_load_dwordx2 %1, %6, 0x0\n\t"
        "s_load_dword %2, %7, 0x0\n\t"
        "s_load_dword %3, %8, 0x0\n\t"
        "s_load_dword %4, %9, 0x0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(P32), "=&s"(i), "=&s"(crow32), "=&s"(prow32), "=&s"(guard_v)
        : "s"(sgpr_ptr(p.plen + b)), "s"(sgpr_ptr(p.pos + b)), "s"(sgpr_ptr(p.c.rows + b)),
          "s"(sgpr_ptr(p.c.prows + b)), "s"(sgpr_ptr(guard_p))
        : "memory");
    const int64_t P = P32;
    const int64_t crow = PAGED ? 0 : crow32, prow = PAGED ? 0 : prow32;
    Vec16 qraw[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
        qraw[hh] = load16(reinterpret_cast<const T*>(p.q) + ((int64_t)b * p.hq + g * G + hh) * D + sub * VEC);

    const int64_t n_pre = i + 1 < P ? i + 1 : P;
    int64_t n_ring = i - P + 1;
    n_ring = n_ring < 0 ? 0 : (n_ring > p.c.window ? (int64_t)p.c.window : n_ring);
    const int64_t n = n_pre + n_ring;
    const int nsplit = PAGED ? (int)((p.rows_per_head + R - 1) / R) : (int)((n + R - 1) / R);
    if (split >= nsplit) return;
    if (p.c.guard && guard_v) return;  // checks on and a check failed
    if constexpr (TRACE) {
        if (tid == 0) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            trace_mark(p, 1);
        }
    }

    // Key row r of the sequence: r < n_pre is slot r of its prefix block,
    // else slot r - n_pre of its window block.  The choice is one select of a
    // base per row: r's byte offset goes on the prefix block's base or on the
    // window block's base moved back by n_pre rows.  A V row lies v_off bytes
    // after its K row in both pools.
    constexpr int64_t kRowBytes = (int64_t)D * sizeof(T);
    const int64_t pre_off = (prow * p.c.hkv + g) * p.c.pcap;
    const int64_t win_off = (crow * p.c.hkv + g) * p.c.window;
    const char* kpre_a = static_cast<const char*>(p.c.kpre) + pre_off * kRowBytes;
    const char* kwin_a = static_cast<const char*>(p.c.kwin) + (win_off - n_pre) * kRowBytes;
    const int64_t v_off = p.c.v_off;
    const bool fused = p.knew != nullptr;
    int64_t new_r = i;  // key row of the new token
    if (fused && i >= P) {
        const int64_t off = i - P;
        new_r = (PAGED ? (int64_t)p.c.pcap : n_pre) +
                (off < 0x7FFFFFFF ? (int64_t)((uint32_t)off % (uint32_t)p.c.window) : off % p.c.window);
    }
    // paged: the new token's page, for the commit below
    const int64_t new_page =
        PAGED && fused && split == 0 && tid < LPR ? (int64_t)p.c.pages[(int64_t)b * p.c.pages_per_seq + (new_r >> p.c.page_shift)]
                                                  : 0;
    const int64_t page_mask = PAGED ? ((int64_t)1 << p.c.page_shift) - 1 : 0;
    // paged row r -> byte address of its K row
    auto paged_k = [&](int64_t page, int64_t r) -> const char* {
        return static_cast<const char*>(p.c.kpre) + (((page * p.c.hkv + g) << p.c.page_shift) + (r & page_mask)) * kRowBytes;
    };
    // paged: this lane's rows r0 + (wave U + u) RPW + rg all lie in the wave's
    // page, at a constant stride from the first
    const char* lane_k = PAGED ? paged_k(wave_page, wave_row0 + rg) : nullptr;
    const T* knew_row = fused ? reinterpret_cast<const T*>(p.knew) + ((int64_t)b * p.c.hkv + g) * D : nullptr;
    const T* vnew_row = fused ? reinterpret_cast<const T*>(p.vnew) + ((int64_t)b * p.c.hkv + g) * D : nullptr;

    // This lane's K loads, then its V loads.  Rows past the end are clamped
    // to the last valid row (a harmless in-bounds read, no branch) and masked
    // out of the softmax below.  (The compiler issues the V loads after the
    // scores; pinning them before the scores with a scheduling barrier, so
    // that K and V share one round trip, measured 1.5% slower at batch 1.)
    const int64_t r0 = (int64_t)split * R;
    Vec16 kr[U], vr[U];
    const T* vps[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t r = r0 + (int64_t)(wave * U + u) * RPW + rg;
        const char* ka;
        if constexpr (PAGED) {
            // Every row is loaded (its page is a pool page, so the read is in
            // bounds); an unfilled slot may hold anything, so its score is
            // replaced by -inf and its V row by zeros below.
            valid[u] = r < p.c.pcap ? r < n_pre : (r - p.c.pcap < n_ring);
            ka = lane_k + (int64_t)u * RPW * kRowBytes;
        } else {
            valid[u] = r < n;
            r = valid[u] ? r : n - 1;
            ka = (r < n_pre ? kpre_a : kwin_a) + r * kRowBytes;
        }
        const bool is_new = fused && r == new_r;
        const T* kp = is_new ? knew_row : reinterpret_cast<const T*>(ka);
        vps[u] = is_new ? vnew_row : reinterpret_cast<const T*>(ka + v_off);
        kr[u] = load16_stream<NTL>(kp + sub * VEC);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) vr[u] = load16_stream<NTL>(vps[u] + sub * VEC);

    // Scores (log2 units): q.k over this lane's slice, summed over the row's
    // lanes, then scaled.
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s[u][hh] = Elem<T>::dot(qraw[hh], kr[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float t = group_sum<LPR>(s[u][hh]) * p.scale_log2;
            s[u][hh] = valid[u] ? t : -INFINITY;
        }

    if constexpr (TRACE) {
        if (tid == 0) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            trace_mark(p, 2);
        }
    }
    // The split that owns the new token's slot also commits it to the cache
    // (after the loads above, so no wait on them is forced here).
    if (fused && split == 0 && tid < LPR) {
        const char* ka = PAGED ? paged_k(new_page, new_r) : (new_r < n_pre ? kpre_a : kwin_a) + new_r * kRowBytes;
        T* kd = const_cast<T*>(reinterpret_cast<const T*>(ka)) + tid * VEC;
        T* vd = const_cast<T*>(reinterpret_cast<const T*>(ka + v_off)) + tid * VEC;
        *reinterpret_cast<Vec16*>(kd) = load16(knew_row + tid * VEC);
        *reinterpret_cast<Vec16*>(vd) = load16(vnew_row + tid * VEC);
    }

    // Softmax per wave: each head's reference is the wave's maximum score
    // (row groups meet through lane swaps), so a wave finishes its rows as
    // soon as they are in, without waiting for the rest of the workgroup.
    // Row-group partials then add without rescaling; the waves are combined
    // through LDS with one weight per (head, wave).  A wave whose rows all
    // lie past the end has reference -inf and weight 0.
    float mw[G], lg[G], og[G][VEC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        float m = s[0][hh];
#pragma unroll
        for (int u = 1; u < U; ++u) m = fmaxf(m, s[u][hh]);
        mw[hh] = rowgroup_max<LPR>(m);
        lg[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) og[hh][e] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float vf[VEC];
        if constexpr (PAGED) {
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) vr[u].w[w4] = valid[u] ? vr[u].w[w4] : 0u;
        }
        Elem<T>::unpack(vr[u], vf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float w = valid[u] ? fast_exp2(s[u][hh] - mw[hh]) : 0.f;
            lg[hh] += w;
#pragma unroll
            for (int e = 0; e < VEC; ++e) og[hh][e] = fmaf(w, vf[e], og[hh][e]);
        }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        lg[hh] = rowgroup_sum<LPR>(lg[hh]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) og[hh][e] = rowgroup_sum<LPR>(og[hh][e]);
    }
    if constexpr (TRACE) {
        if (tid == 0) trace_mark(p, 3);
    }
    if (rg == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) s_o[wave][hh * D + sub * VEC + e] = og[hh][e];
            if (sub == 0) {
                s_m[hh][wave] = mw[hh];
                s_l[hh][wave] = lg[hh];
            }
        }
    }
    __syncthreads();
    // weight of each (head, wave) against the split's maximum
    if (tid < G * NW) {
        const int hh = tid / NW, k = tid % NW;
        float M = -INFINITY;
#pragma unroll
        for (int j = 0; j < NW; j += 4) {
            const float4 x = *reinterpret_cast<const float4*>(&s_m[hh][j]);
            M = fmaxf(fmaxf(M, fmaxf(x.x, x.y)), fmaxf(x.z, x.w));
        }
        const float mk = s_m[hh][k];
        s_w[hh][k] = mk == -INFINITY ? 0.f : fast_exp2(mk - M);
        if (k == 0) s_ref[hh] = M;  // finite: every split holds at least one valid row
    }
    __syncthreads();

    if constexpr (TRACE) {
        if (tid == 0) trace_mark(p, 4);
    }
    const int64_t ws_head0 = (int64_t)b * p.hq + g * G;
    for (int idx = tid; idx < PAIRS; idx += NT) {
        const int hh = idx / D, dim = idx % D;
        float O = 0.f, L = 0.f;
#pragma unroll
        for (int k = 0; k < NW; k += 4) {
            const float4 w = *reinterpret_cast<const float4*>(&s_w[hh][k]);
            const float4 l = *reinterpret_cast<const float4*>(&s_l[hh][k]);
            L = fmaf(w.x, l.x, fmaf(w.y, l.y, fmaf(w.z, l.z, fmaf(w.w, l.w, L))));
            O = fmaf(w.x, s_o[k][idx], fmaf(w.y, s_o[k + 1][idx], fmaf(w.z, s_o[k + 2][idx], fmaf(w.w, s_o[k + 3][idx], O))));
        }
        const float M = s_ref[hh];
        if (nsplit == 1) {
            T* o = reinterpret_cast<T*>(p.out) + (ws_head0 + hh) * D + dim;
            *o = Elem<T>::from_float(O / L);
            if (p.lse && dim == 0) p.lse[ws_head0 + hh] = (M + log2f(L)) * kLn2;
        } else {
            const int64_t slot = (ws_head0 + hh) * p.s_max + split;
            store_coherent(p.ws_o + slot * D + dim, O);
            if (dim == 0) {
                store_coherent(p.ws_ml + slot * 2, M);
                store_coherent(p.ws_ml + slot * 2 + 1, L);
            }
        }
    }
    if (nsplit == 1) return;

    // Arrival counter: the last split of this (sequence, kv head) merges.
    // The partials travel through agent-coherent stores and loads, so the
    // only ordering needed is "every store of this workgroup has completed
    // before the counter moves": each wave waits for its stores to be
    // acknowledged (stores count in vmcnt on CDNA), then the barrier.  A
    // device-scope fence would instead write back and invalidate the XCD's
    // whole L2 for every workgroup.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (TRACE) {
        if (tid == 0) trace_mark(p, 5);
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t* t = p.tickets + ((int64_t)b * p.c.hkv + g) * kTicketStride;
        const uint32_t prev = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(nsplit - 1));
        if (s_last) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if constexpr (TRACE) {
        if (tid == 0) trace_mark(p, 6);
    }
    if (!s_last) return;

    // Merge the splits.  Thread t owns output (head, dim) = t % PAIRS and the
    // splits part, part + PARTS, ... (part = t / PAIRS); it requests (m, l, o)
    // of a whole batch of its splits before using any, so a batch costs one
    // round trip.  The PARTS partial results meet in LDS.
    constexpr int PARTS = NT >= PAIRS ? NT / PAIRS : 1;
    constexpr int kBatch = 16;
    __shared__ float red[PARTS > 1 ? PARTS * 3 * PAIRS : 1];  // [PARTS][3][PAIRS]
    // (threads past PARTS * PAIRS, when PAIRS does not divide the workgroup,
    // take no part)
    const int part = NT >= PAIRS ? tid / PAIRS : 0;
    for (int pair = (NT >= PAIRS ? tid % PAIRS : tid); part < PARTS && pair < PAIRS;
         pair += (NT >= PAIRS ? PAIRS : NT)) {
        const int hh = pair / D, dim = pair % D;
        const float* oh = p.ws_o + ((ws_head0 + hh) * p.s_max) * D + dim;
        const float* mlh = p.ws_ml + ((ws_head0 + hh) * p.s_max) * 2;
        float M = -INFINITY, L = 0.f, O = 0.f;
        for (int s0 = part; s0 < nsplit; s0 += kBatch * PARTS) {
            float bm[kBatch], bl[kBatch], bo[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                // part is uniform across a wave, so this branch is too: no
                // load is issued for a split past the end
                const int sidx = s0 + j * PARTS;
                if (sidx < nsplit) {
                    bm[j] = load_coherent(mlh + 2 * sidx);
                    bl[j] = load_coherent(mlh + 2 * sidx + 1);
                    bo[j] = load_coherent(oh + (int64_t)sidx * D);
                } else {
                    bm[j] = -INFINITY;
                    bl[j] = 0.f;
                    bo[j] = 0.f;
                }
            }
            float bM = M;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) bM = fmaxf(bM, bm[j]);
            const float a = M == -INFINITY ? 0.f : fast_exp2(M - bM);
            L *= a;
            O *= a;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const float w = bm[j] == -INFINITY ? 0.f : fast_exp2(bm[j] - bM);
                L = fmaf(w, bl[j], L);
                O = fmaf(w, bo[j], O);
            }
            M = bM;
        }
        if constexpr (PARTS > 1) {
            red[(part * 3 + 0) * PAIRS + pair] = M;
            red[(part * 3 + 1) * PAIRS + pair] = L;
            red[(part * 3 + 2) * PAIRS + pair] = O;
        }
        if constexpr (PARTS == 1) {
            T* o = reinterpret_cast<T*>(p.out) + (ws_head0 + hh) * D + dim;
            *o = Elem<T>::from_float(O / L);
            if (p.lse && dim == 0) p.lse[ws_head0 + hh] = (M + log2f(L)) * kLn2;
        }
    }
    if constexpr (PARTS > 1) {
        __syncthreads();
        if (tid < PAIRS) {
            const int pair = tid, hh = pair / D, dim = pair % D;
            float M = -INFINITY;
#pragma unroll
            for (int k = 0; k < PARTS; ++k) M = fmaxf(M, red[(k * 3) * PAIRS + pair]);
            float L = 0.f, O = 0.f;
#pragma unroll
            for (int k = 0; k < PARTS; ++k) {
                const float mk = red[(k * 3) * PAIRS + pair];
                const float w = mk == -INFINITY ? 0.f : fast_exp2(mk - M);
                L = fmaf(w, red[(k * 3 + 1) * PAIRS + pair], L);
                O = fmaf(w, red[(k * 3 + 2) * PAIRS + pair], O);
            }
            T* o = reinterpret_cast<T*>(p.out) + (ws_head0 + hh) * D + dim;
            *o = Elem<T>::from_float(O / L);
            if (p.lse && dim == 0) p.lse[ws_head0 + hh] = (M + log2f(L)) * kLn2;
        }
    }
    if constexpr (TRACE) {
        __syncthreads();
        if (tid == 0) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            trace_mark(p, 7);
        }
    }
}

// ------------------------------------------------------------ MFMA decode
// bf16, head_dim 128, GQA groups of 5 to 8 heads (4 also works; the host
// sends 4 to the vector kernel, which is 2% faster there).  With many heads per kv
// head the vector work per key row (one dot product and eight multiply-adds
// of the V sum per head) outgrows the streaming, so the products run on the
// matrix cores: per 16-key block S^T = K Q^T with v_mfma_f32_16x16x32_bf16
// (the key rows are the A operand, loaded straight from global memory; the
// group's heads are the 16 columns, missing heads zero), then
// O^T += V^T P^T with v_mfma_f32_16x16x16_bf16, V^T coming from transposing
// LDS reads (ds_read_b64_tr_b16) of the wave's own V rows.  The lane layout
// of S^T (lane: key 4 (lane / 16) + r, head lane % 16) is exactly the P^T
// operand of the second product.  Splits of 256 key rows, 4 waves of 64
// rows; the split combine and the last-arriver merge follow decode_kernel.
constexpr int kMfWaves = 4;
constexpr int kMfKeysPerWave = 64;
constexpr int kMfRows = kMfWaves * kMfKeysPerWave;  // rows per split
static_assert(kMfRows == kDecodeMfmaRows, "split size shared with the host");

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef short mf_s16x4 __attribute__((ext_vector_type(4)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));

__device__ inline mf_bf16x8 mf_as_bf16x8(const Vec16& v) {
    mf_bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}
__device__ inline uint32_t mf_pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 r = {(__bf16)a, (__bf16)b};
    uint32_t u;
    __builtin_memcpy(&u, &r, 4);
    return u;
}
// chunk c (16 bytes) of V row r sits at chunk c ^ 2 (r & 3): the four rows a
// 16-lane transposing read touches then hit different banks
__device__ inline int mf_v_swz(int row) { return 2 * (row & 3); }

template <bool NTL>
__global__ void __launch_bounds__(kMfWaves * 64) decode_mfma_kernel(DecodeParams p) {
    constexpr int D = 128;
    constexpr int NT = kMfWaves * 64;
    constexpr int RB = D * 2;  // bytes per row
    __shared__ __attribute__((aligned(16))) char s_v[kMfWaves][kMfKeysPerWave * RB];
    __shared__ __attribute__((aligned(16))) float s_o[kMfWaves][16 * D];
    __shared__ float s_m[kMfWaves][16], s_l[kMfWaves][16], s_w[kMfWaves][16];
    __shared__ float s_ref[16];
    __shared__ int s_last;
    if (p.c.guard && *p.c.guard) return;  // checks on and a check failed

    const int n_groups = p.n_seqs * p.c.hkv;
    const int group = (int)blockIdx.x % n_groups, split = (int)blockIdx.x / n_groups;
    const int g = group % p.c.hkv, b = group / p.c.hkv;
    const int G = p.hq / p.c.hkv;  // heads of the group, 4..8 (host-checked)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kl = lane & 15, kq = lane >> 4;

    const int64_t P = p.plen[b];
    const int64_t i = p.pos[b];
    const int64_t crow = p.c.rows[b], prow = p.c.prows[b];
    const int64_t n_pre = i + 1 < P ? i + 1 : P;
    int64_t n_ring = i - P + 1;
    n_ring = n_ring < 0 ? 0 : (n_ring > p.c.window ? (int64_t)p.c.window : n_ring);
    const int64_t n = n_pre + n_ring;
    const int nsplit = (int)((n + kMfRows - 1) / kMfRows);
    if (split >= nsplit) return;

    // key row r: slot r of the prefix block below n_pre, else slot r - n_pre
    // of the window block; V lies v_off bytes after K (as in decode_kernel)
    constexpr int64_t kRowBytes = RB;
    const int64_t pre_off = (prow * p.c.hkv + g) * p.c.pcap;
    const int64_t win_off = (crow * p.c.hkv + g) * p.c.window;
    const char* kpre_a = static_cast<const char*>(p.c.kpre) + pre_off * kRowBytes;
    const char* kwin_a = static_cast<const char*>(p.c.kwin) + (win_off - n_pre) * kRowBytes;
    const int64_t v_off = p.c.v_off;
    const bool fused = p.knew != nullptr;
    int64_t new_r = i;
    if (fused && i >= P) {
        const int64_t off = i - P;
        new_r = n_pre + (off < 0x7FFFFFFF ? (int64_t)((uint32_t)off % (uint32_t)p.c.window) : off % p.c.window);
    }
    const char* knew_row = fused ? static_cast<const char*>(p.knew) + ((int64_t)b * p.c.hkv + g) * kRowBytes : nullptr;
    const char* vnew_row = fused ? static_cast<const char*>(p.vnew) + ((int64_t)b * p.c.hkv + g) * kRowBytes : nullptr;
    auto k_row = [&](int64_t r) -> const char* {
        if (fused && r == new_r) return knew_row;
        return (r < n_pre ? kpre_a : kwin_a) + r * kRowBytes;
    };
    auto v_row = [&](int64_t r) -> const char* {
        if (fused && r == new_r) return vnew_row;
        return (r < n_pre ? kpre_a : kwin_a) + r * kRowBytes + v_off;
    };

    // Q^T operand: head kl, dims 32 ks + 8 kq .. + 7 (zero for missing heads)
    Vec16 qb[4];
    {
        const bool hok = kl < G;
        const char* qp = static_cast<const char*>(p.q) + (((int64_t)b * p.hq + g * G + (hok ? kl : 0)) * D) * 2;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb[ks] = hok ? load16(qp + (32 * ks + 8 * kq) * 2) : Vec16{{0, 0, 0, 0}};
    }
    // K operand rows of this wave (key 16 kb + kl, dims 32 ks + 8 kq ..) and
    // its V rows (row 4 j + kq, 16-byte chunk kl), every load issued first;
    // rows past the end are clamped to the last valid row and masked below
    const int64_t r0w = (int64_t)split * kMfRows + (int64_t)wave * kMfKeysPerWave;
    Vec16 ka[4][4], vv[16];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        int64_t r = r0w + 16 * kb + kl;
        r = r < n ? r : n - 1;
        const char* kp = k_row(r);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = load16_stream<NTL>(kp + (32 * ks + 8 * kq) * 2);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        int64_t r = r0w + 4 * j + kq;
        r = r < n ? r : n - 1;
        vv[j] = load16_stream<NTL>(v_row(r) + kl * 16);
    }

    mf_f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        s[kb] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mf_as_bf16x8(ka[kb][ks]), mf_as_bf16x8(qb[ks]), s[kb], 0, 0, 0);
    }

    // the commit of the new token by split 0 (after the loads above)
    if (fused && split == 0 && tid < 16) {
        char* kd = const_cast<char*>((new_r < n_pre ? kpre_a : kwin_a) + new_r * kRowBytes) + tid * 16;
        *reinterpret_cast<Vec16*>(kd) = load16(knew_row + tid * 16);
        *reinterpret_cast<Vec16*>(kd + v_off) = load16(vnew_row + tid * 16);
    }

    // V rows into this wave's LDS region (read back only by this wave)
    char* vl = s_v[wave];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int row = 4 * j + kq;
        *reinterpret_cast<Vec16*>(vl + row * RB + ((kl ^ mf_v_swz(row)) << 4)) = vv[j];
    }

    // scores (log2 units) of keys 16 kb + 4 kq + r for head kl; the wave's
    // maximum per head over the four lanes that hold that head
    float sc[4][4];
    float mw = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool valid = r0w + 16 * kb + 4 * kq + r < n;
            sc[kb][r] = valid ? s[kb][r] * p.scale_log2 : -INFINITY;
            mw = fmaxf(mw, sc[kb][r]);
        }
    mw = fmaxf(mw, __shfl_xor(mw, 16, 64));
    mw = fmaxf(mw, __shfl_xor(mw, 32, 64));
    float lw = 0.f;
    mf_s16x4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pr[r] = mw == -INFINITY ? 0.f : fast_exp2(sc[kb][r] - mw);
            lw += pr[r];
        }
        const uint32_t lo = mf_pack_bf16x2(pr[0], pr[1]), hi = mf_pack_bf16x2(pr[2], pr[3]);
        __builtin_memcpy(&pb[kb], &lo, 4);
        __builtin_memcpy(reinterpret_cast<char*>(&pb[kb]) + 4, &hi, 4);
    }
    lw += __shfl_xor(lw, 16, 64);
    lw += __shfl_xor(lw, 32, 64);

    // O^T += V^T P^T: lane i of 16-lane group kq gets dims 16 mb + i of keys
    // 16 kb + 4 kq + j (j = 0..3): group lane L reads 4 dims of key
    // 16 kb + 4 kq + L / 4 at dims 16 mb + 4 (L % 4)
    mf_f32x4 o[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) o[mb] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t vbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)vl;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int row = 16 * kb + 4 * kq + (kl >> 2);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int byte = 32 * mb + 8 * (kl & 3);  // within the row, before the swizzle
            const uint32_t addr = vbase + row * RB + ((((byte >> 4) ^ mf_v_swz(row)) << 4) | (byte & 15));
            const mf_s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) mf_s16x4*)(uintptr_t)addr);
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[kb], o[mb], 0, 0, 0);
        }
    }

    // combine the waves: lane holds O^T[dim 16 mb + 4 kq + r][head kl]
    if (kl < G) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_o[wave][kl * D + 16 * mb + 4 * kq + r] = o[mb][r];
        if (kq == 0) {
            s_m[wave][kl] = mw;
            s_l[wave][kl] = lw;
        }
    }
    __syncthreads();
    if (tid < 16 && tid < G) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kMfWaves; ++w) M = fmaxf(M, s_m[w][tid]);
#pragma unroll
        for (int w = 0; w < kMfWaves; ++w) s_w[w][tid] = s_m[w][tid] == -INFINITY ? 0.f : fast_exp2(s_m[w][tid] - M);
        s_ref[tid] = M;  // finite: every split holds at least one valid row
    }
    __syncthreads();

    const int64_t ws_head0 = (int64_t)b * p.hq + g * G;
    const int pairs = G * D;
    for (int idx = tid; idx < pairs; idx += NT) {
        const int hh = idx / D, dim = idx % D;
        float O = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < kMfWaves; ++w) {
            O = fmaf(s_w[w][hh], s_o[w][hh * D + dim], O);
            L = fmaf(s_w[w][hh], s_l[w][hh], L);
        }
        const float M = s_ref[hh];
        if (nsplit == 1) {
            uint16_t* op = static_cast<uint16_t*>(p.out) + (ws_head0 + hh) * D + dim;
            *op = Elem<uint16_t>::from_float(O / L);
            if (p.lse && dim == 0) p.lse[ws_head0 + hh] = (M + log2f(L)) * kLn2;
        } else {
            const int64_t slot = (ws_head0 + hh) * p.s_max + split;
            store_coherent(p.ws_o + slot * D + dim, O);
            if (dim == 0) {
                store_coherent(p.ws_ml + slot * 2, M);
                store_coherent(p.ws_ml + slot * 2 + 1, L);
            }
        }
    }
    if (nsplit == 1) return;

    // arrival counter and merge by the last split (as in decode_kernel)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        uint32_t* t = p.tickets + ((int64_t)b * p.c.hkv + g) * kTicketStride;
        const uint32_t prev = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(nsplit - 1));
        if (s_last) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;

    // Merge: every load is issued before any is used, so the merge costs one
    // round trip per batch of kMergeBatch splits.  (m, l) of each (head,
    // split) are read once, by one thread each, and turned into weights in
    // LDS (reusing s_o); thread t combines outputs t, t + NT, ... (at most
    // kMfPairsPerThread of them) from its own o loads.
    constexpr int kMergeBatch = 32;
    constexpr int kMfPairsPerThread = 8 * D / NT;  // groups of up to 8 heads (the cache's limit)
    float* s_ml = &s_o[0][0];                    // [G][kMergeBatch] (m, then weight), [G][kMergeBatch] l
    float* s_wt = s_ml;
    float* s_ll = s_ml + 16 * kMergeBatch;
    __shared__ float s_M[16], s_L[16];
    if (tid < G) {
        s_M[tid] = -INFINITY;
        s_L[tid] = 0.f;
    }
    float accO[kMfPairsPerThread];
#pragma unroll
    for (int k = 0; k < kMfPairsPerThread; ++k) accO[k] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += kMergeBatch) {
        const int nb = nsplit - s0 < kMergeBatch ? nsplit - s0 : kMergeBatch;
        float bo[kMfPairsPerThread][kMergeBatch];
        // Unconditional loads (split and pair indices clamped into range; the
        // extra ones get weight 0 or are not written), so the compiler emits
        // them back to back instead of one branch and one wait each.
#pragma unroll
        for (int k = 0; k < kMfPairsPerThread; ++k) {
            const int pair = tid + k * NT < pairs ? tid + k * NT : pairs - 1;
            const int hh = pair / D, dim = pair % D;
            const float* oh = p.ws_o + ((ws_head0 + hh) * p.s_max + s0) * D + dim;
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) bo[k][j] = load_coherent(oh + (int64_t)(j < nb ? j : nb - 1) * D);
        }
        for (int e = tid; e < G * kMergeBatch; e += NT) {
            const int hh = e / kMergeBatch, j = e % kMergeBatch;
            const float* mlh = p.ws_ml + ((ws_head0 + hh) * p.s_max + s0 + (j < nb ? j : nb - 1)) * 2;
            const float m = load_coherent(mlh), l = load_coherent(mlh + 1);
            s_ml[e] = j < nb ? m : -INFINITY;
            s_ll[e] = j < nb ? l : 0.f;
        }
        __syncthreads();
        if (tid < G) {
            // new running maximum of the head, rescale of what came before,
            // and the weights of this batch relative to it
            float bM = s_M[tid];
            for (int j = 0; j < nb; ++j) bM = fmaxf(bM, s_ml[tid * kMergeBatch + j]);
            const float a = s_M[tid] == -INFINITY ? 0.f : fast_exp2(s_M[tid] - bM);
            float L = s_L[tid] * a;
            for (int j = 0; j < kMergeBatch; ++j) {
                const float m = s_ml[tid * kMergeBatch + j];
                const float w = m == -INFINITY ? 0.f : fast_exp2(m - bM);
                s_wt[tid * kMergeBatch + j] = w;
                L = fmaf(w, s_ll[tid * kMergeBatch + j], L);
            }
            s_ll[tid * kMergeBatch] = a;  // the rescale factor of earlier batches, read below
            s_M[tid] = bM;
            s_L[tid] = L;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMfPairsPerThread; ++k) {
            const int pair = tid + k * NT < pairs ? tid + k * NT : pairs - 1;
            const int hh = pair / D;
            float O = accO[k] * s_ll[hh * kMergeBatch];
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) O = fmaf(s_wt[hh * kMergeBatch + j], bo[k][j], O);
            accO[k] = O;
        }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < kMfPairsPerThread; ++k) {
        const int pair = tid + k * NT;
        if (pair < pairs) {
            const int hh = pair / D, dim = pair % D;
            uint16_t* op = static_cast<uint16_t*>(p.out) + (ws_head0 + hh) * D + dim;
            *op = Elem<uint16_t>::from_float(accO[k] / s_L[hh]);
            if (p.lse && dim == 0) p.lse[ws_head0 + hh] = (s_M[hh] + log2f(s_L[hh])) * kLn2;
        }
    }
}

template <typename T, int D, int G, int NW, int U, bool NTL = false>
hipError_t launch_one(const DecodeParams& p, hipStream_t stream) {
    constexpr int R = NW * (64 / (D / Elem<T>::kPerVec)) * U;
    const int64_t n_wg = ((p.rows_per_head + R - 1) / R) * (int64_t)p.c.hkv * p.n_seqs;
    if (n_wg > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (p.trace) return hipErrorNotSupported;  // traced launches: see launch_decode_traced
    if (p.c.pages) {  // paged layout: built for the 8-wave, 8-rows-per-lane split only
        if constexpr (NW == 8 && U == 8)
            hipLaunchKernelGGL((decode_kernel<T, D, G, NW, U, NTL, false, true>), dim3((unsigned)n_wg), dim3(NW * 64),
                               0, stream, p);
        else
            return hipErrorNotSupported;
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_kernel<T, D, G, NW, U, NTL>), dim3((unsigned)n_wg), dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
}

// rows_per_split = NW * RPW * U: four waves for the two smallest sizes,
// sixteen for 16 RPW and 128 RPW, eight (longer per-lane row chains, a
// cheaper combine across waves) for 32 RPW, 48 RPW and 64 RPW.
template <typename T, int D, int G>
hipError_t dispatch_rows(int rows, const DecodeParams& p, hipStream_t stream) {
    constexpr int RPW = 64 / (D / Elem<T>::kPerVec);
    const int r4 = 4 * RPW, r16 = 16 * RPW;
    if (rows == r4) return launch_one<T, D, G, 4, 1>(p, stream);
    if (rows == 2 * r4) return launch_one<T, D, G, 4, 2>(p, stream);
    if (rows == r16) return launch_one<T, D, G, 16, 1>(p, stream);
    if (rows == 2 * r16) return launch_one<T, D, G, 8, 4>(p, stream);
    if (rows == 3 * r16) return launch_one<T, D, G, 8, 6>(p, stream);
    if (rows == 4 * r16) {
        // many workgroups (several per CU) stream far more than the caches
        // hold: mark the K/V loads non-temporal (a single sequence's few
        // workgroups are latency-bound and measured faster without the hint)
        if (p.stream_nt) return launch_one<T, D, G, 8, 8, true>(p, stream);
        return launch_one<T, D, G, 8, 8>(p, stream);
    }
    if (rows == 8 * r16) return launch_one<T, D, G, 16, 8>(p, stream);
    return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t dispatch_g(int group, int rows, const DecodeParams& p, hipStream_t stream) {
    switch (group) {
        case 1: return dispatch_rows<T, D, 1>(rows, p, stream);
        case 2: return dispatch_rows<T, D, 2>(rows, p, stream);
        case 3: return dispatch_rows<T, D, 3>(rows, p, stream);
        case 4: return dispatch_rows<T, D, 4>(rows, p, stream);
        case 5: return dispatch_rows<T, D, 5>(rows, p, stream);
        case 6: return dispatch_rows<T, D, 6>(rows, p, stream);
        case 7: return dispatch_rows<T, D, 7>(rows, p, stream);
        case 8: return dispatch_rows<T, D, 8>(rows, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int decode_rows_per_load(int dtype, int head_dim) {
    const int vec = dtype == PS_BF16 ? 8 : 4;
    return 64 / (head_dim / vec);  // rows one wave covers per load instruction
}

bool decode_rows_valid(int dtype, int head_dim, int rows) {
    const int rpw = decode_rows_per_load(dtype, head_dim);
    const int r4 = 4 * rpw, r16 = 16 * rpw;
    if (rows < kMinSplitRows) return false;
    return rows == r4 || rows == 2 * r4 || rows == r16 || rows == 2 * r16 || rows == 3 * r16 || rows == 4 * r16 ||
           rows == 8 * r16;
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
    const int64_t n_wg = ((p.rows_per_head + kMfRows - 1) / kMfRows) * (int64_t)p.c.hkv * p.n_seqs;
    if (n_wg > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (p.stream_nt)
        hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3((unsigned)n_wg), dim3(kMfWaves * 64), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_mfma_kernel<false>, dim3((unsigned)n_wg), dim3(kMfWaves * 64), 0, stream, p);
    return hipGetLastError();
}

int64_t decode_grid(int rows_per_split, const DecodeParams& p) {
    return ((p.rows_per_head + rows_per_split - 1) / rows_per_split) * (int64_t)p.c.hkv * p.n_seqs;
}

template <int U>
hipError_t launch_traced_u(int group, const DecodeParams& p, hipStream_t stream) {
    const int64_t n_wg = decode_grid(8 * 4 * U, p);
    const dim3 grid((unsigned)n_wg), block(512);
    switch (group) {
        case 1: hipLaunchKernelGGL((decode_kernel<uint16_t, 128, 1, 8, U, false, true>), grid, block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL((decode_kernel<uint16_t, 128, 2, 8, U, false, true>), grid, block, 0, stream, p); break;
        case 4: hipLaunchKernelGGL((decode_kernel<uint16_t, 128, 4, 8, U, false, true>), grid, block, 0, stream, p); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

hipError_t launch_decode_traced(int group, int rows_per_split, const DecodeParams& p, hipStream_t stream) {
    if (rows_per_split == 256) return launch_traced_u<8>(group, p, stream);
    if (rows_per_split == 192) return launch_traced_u<6>(group, p, stream);
    return hipErrorNotSupported;
}

hipError_t launch_decode(int dtype, int head_dim, int group, int rows_per_split, const DecodeParams& p,
                         hipStream_t stream) {
    if (!decode_rows_valid(dtype, head_dim, rows_per_split)) return hipErrorInvalidValue;
    if (dtype == PS_BF16) {
        if (head_dim == 128) return dispatch_g<uint16_t, 128>(group, rows_per_split, p, stream);
        if (head_dim == 64) return dispatch_g<uint16_t, 64>(group, rows_per_split, p, stream);
    } else {
        if (head_dim == 128) return dispatch_g<float, 128>(group, rows_per_split, p, stream);
        if (head_dim == 64) return dispatch_g<float, 64>(group, rows_per_split, p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ps
