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
//   * grid = (split, kv head, sequence); a split owns R consecutive key rows
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

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
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

template <typename T, int D, int G, int U>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecodeParams p) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int LPR = D / VEC;          // lanes per key row
    constexpr int RPW = 64 / LPR;         // rows per wave per load instruction
    constexpr int NG = kWaves * RPW;      // row groups per workgroup
    constexpr int R = NG * U;             // rows per split
    static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row must map onto a wave");

    __shared__ float s_m[NG][G];
    __shared__ float s_l[NG][G];
    __shared__ float s_o[NG][G][D];
    __shared__ int s_last;

    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane % LPR, rg = lane / LPR;
    const int gi = wave * RPW + rg;

    const int64_t P = p.plen[b];
    const int64_t i = p.pos[b];
    const int64_t n_pre = i + 1 < P ? i + 1 : P;
    int64_t n_ring = i - P + 1;
    n_ring = n_ring < 0 ? 0 : (n_ring > p.window ? (int64_t)p.window : n_ring);
    const int64_t n = n_pre + n_ring;
    const int nsplit = (int)((n + R - 1) / R);
    if (split >= nsplit) return;

    const int64_t head_off = ((int64_t)p.rows[b] * p.hkv + g) * p.rows_per_head;
    const T* kbase = reinterpret_cast<const T*>(p.kc) + head_off * D;
    const T* vbase = reinterpret_cast<const T*>(p.vc) + head_off * D;
    const bool fused = p.knew != nullptr;
    const int64_t new_phys = i < P ? i : p.pcap + (i - P) % p.window;
    const T* knew_row = fused ? reinterpret_cast<const T*>(p.knew) + ((int64_t)b * p.hkv + g) * D : nullptr;
    const T* vnew_row = fused ? reinterpret_cast<const T*>(p.vnew) + ((int64_t)b * p.hkv + g) * D : nullptr;

    // Issue every K/V load of this lane's rows first.
    const int64_t r0 = (int64_t)split * R;
    Vec16 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t r = r0 + (int64_t)(wave * U + u) * RPW + rg;
        valid[u] = r < n;
        const int64_t phys = r < n_pre ? r : p.pcap + (r - n_pre);
        const T* kp = kbase + phys * D;
        const T* vp = vbase + phys * D;
        if (fused && phys == new_phys) {
            kp = knew_row;
            vp = vnew_row;
        }
        if (valid[u]) {
            kr[u] = load16(kp + sub * VEC);
            vr[u] = load16(vp + sub * VEC);
        } else {
            kr[u] = Vec16{{0, 0, 0, 0}};
            vr[u] = Vec16{{0, 0, 0, 0}};
        }
    }

    // Queries of the GQA group (pre-multiplied by scale * log2 e).
    float qf[G][VEC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        const T* qp = reinterpret_cast<const T*>(p.q) + ((int64_t)b * p.hq + g * G + hh) * D + sub * VEC;
        Elem<T>::unpack(load16(qp), qf[hh]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) qf[hh][e] *= p.scale_log2;
    }

    // The split that owns the new token's slot also commits it to the cache.
    if (fused && split == 0 && tid < LPR) {
        T* kd = const_cast<T*>(kbase) + new_phys * D + tid * VEC;
        T* vd = const_cast<T*>(vbase) + new_phys * D + tid * VEC;
        *reinterpret_cast<Vec16*>(kd) = load16(knew_row + tid * VEC);
        *reinterpret_cast<Vec16*>(vd) = load16(vnew_row + tid * VEC);
    }

    // Scores (log2 units).
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float kf[VEC];
        Elem<T>::unpack(kr[u], kf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc = fmaf(qf[hh][e], kf[e], acc);
            acc = group_sum<LPR>(acc);
            s[u][hh] = valid[u] ? acc : -INFINITY;
        }
    }

    // Softmax over this row group's rows and weighted sum of values.
    float mg[G], lg[G], og[G][VEC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) m = fmaxf(m, s[u][hh]);
        mg[hh] = m;
        lg[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) og[hh][e] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float vf[VEC];
        Elem<T>::unpack(vr[u], vf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float w = valid[u] ? exp2f(s[u][hh] - mg[hh]) : 0.f;
            lg[hh] += w;
#pragma unroll
            for (int e = 0; e < VEC; ++e) og[hh][e] = fmaf(w, vf[e], og[hh][e]);
        }
    }

    // Merge the NG row groups of the workgroup through LDS.
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) s_o[gi][hh][sub * VEC + e] = og[hh][e];
        if (sub == 0) {
            s_m[gi][hh] = mg[hh];
            s_l[gi][hh] = lg[hh];
        }
    }
    __syncthreads();

    const int64_t ws_head0 = (int64_t)b * p.hq + g * G;
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int hh = idx / D, dim = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NG; ++k) M = fmaxf(M, s_m[k][hh]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const float w = s_m[k][hh] == -INFINITY ? 0.f : exp2f(s_m[k][hh] - M);
            L = fmaf(w, s_l[k][hh], L);
            O = fmaf(w, s_o[k][hh][dim], O);
        }
        if (nsplit == 1) {
            T* o = reinterpret_cast<T*>(p.out) + (ws_head0 + hh) * D + dim;
            *o = Elem<T>::from_float(O / L);
            if (p.lse && dim == 0) p.lse[ws_head0 + hh] = (M + log2f(L)) * kLn2;
        } else {
            const int64_t slot = (ws_head0 + hh) * p.s_max + split;
            p.ws_o[slot * D + dim] = O;
            if (dim == 0) {
                p.ws_ml[slot * 2] = M;
                p.ws_ml[slot * 2 + 1] = L;
            }
        }
    }
    if (nsplit == 1) return;

    // Arrival counter: the last split of this (sequence, kv head) merges.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        uint32_t* t = p.tickets + (int64_t)b * p.hkv + g;
        const uint32_t prev = __hip_atomic_fetch_add(t, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(nsplit - 1));
        if (s_last) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // Stage (m, l) of every split in LDS (reuse s_o: nsplit * G * 2 floats).
    float* ml = &s_o[0][0][0];
    constexpr int kMlCap = NG * G * D;
    const bool staged = nsplit * G * 2 <= kMlCap;
    if (staged) {
        for (int idx = tid; idx < nsplit * G * 2; idx += kThreads) {
            const int hh = idx / (nsplit * 2), rem = idx % (nsplit * 2);
            ml[idx] = p.ws_ml[((ws_head0 + hh) * p.s_max) * 2 + rem];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int hh = idx / D, dim = idx % D;
        const float* mlh = staged ? ml + hh * nsplit * 2 : p.ws_ml + ((ws_head0 + hh) * p.s_max) * 2;
        float M = -INFINITY;
        for (int sidx = 0; sidx < nsplit; ++sidx) M = fmaxf(M, mlh[2 * sidx]);
        float L = 0.f, O = 0.f;
        const float* oh = p.ws_o + ((ws_head0 + hh) * p.s_max) * D + dim;
        for (int sidx = 0; sidx < nsplit; ++sidx) {
            const float w = exp2f(mlh[2 * sidx] - M);
            L = fmaf(w, mlh[2 * sidx + 1], L);
            O = fmaf(w, oh[(int64_t)sidx * D], O);
        }
        T* o = reinterpret_cast<T*>(p.out) + (ws_head0 + hh) * D + dim;
        *o = Elem<T>::from_float(O / L);
        if (p.lse && dim == 0) p.lse[ws_head0 + hh] = (M + log2f(L)) * kLn2;
    }
}

template <typename T, int D, int G>
hipError_t dispatch_u(int u, const DecodeParams& p, hipStream_t stream) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int R1 = kWaves * (64 / (D / VEC));
    dim3 block(kThreads);
    const int rows = (int)p.rows_per_head;
    auto grid_for = [&](int R) { return dim3((unsigned)((rows + R - 1) / R), (unsigned)p.hkv, (unsigned)p.n_seqs); };
    switch (u) {
        case 1: hipLaunchKernelGGL((decode_kernel<T, D, G, 1>), grid_for(R1), block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL((decode_kernel<T, D, G, 2>), grid_for(2 * R1), block, 0, stream, p); break;
        case 4: hipLaunchKernelGGL((decode_kernel<T, D, G, 4>), grid_for(4 * R1), block, 0, stream, p); break;
        case 8: hipLaunchKernelGGL((decode_kernel<T, D, G, 8>), grid_for(8 * R1), block, 0, stream, p); break;
        case 16: hipLaunchKernelGGL((decode_kernel<T, D, G, 16>), grid_for(16 * R1), block, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_g(int group, int u, const DecodeParams& p, hipStream_t stream) {
    switch (group) {
        case 1: return dispatch_u<T, D, 1>(u, p, stream);
        case 2: return dispatch_u<T, D, 2>(u, p, stream);
        case 4: return dispatch_u<T, D, 4>(u, p, stream);
        case 8: return dispatch_u<T, D, 8>(u, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int decode_rows_per_load(int dtype, int head_dim) {
    const int vec = dtype == PS_BF16 ? 8 : 4;
    return kWaves * (64 / (head_dim / vec));
}

hipError_t launch_decode(int dtype, int head_dim, int group, int rows_per_split, const DecodeParams& p,
                         hipStream_t stream) {
    const int r1 = decode_rows_per_load(dtype, head_dim);
    if (rows_per_split % r1 != 0) return hipErrorInvalidValue;
    const int u = rows_per_split / r1;
    if (dtype == PS_BF16) {
        if (head_dim == 128) return dispatch_g<uint16_t, 128>(group, u, p, stream);
        if (head_dim == 64) return dispatch_g<uint16_t, 64>(group, u, p, stream);
    } else {
        if (head_dim == 128) return dispatch_g<float, 128>(group, u, p, stream);
        if (head_dim == 64) return dispatch_g<float, 64>(group, u, p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ps
