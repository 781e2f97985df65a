// Append / evict for the two-region Prefix Sliding cache.
//
// A token at position p of a sequence with prefix length P lands in prefix row
// p when p < P and in ring row (p - P) mod W otherwise.  The ring write
// overwrites the token at p - W, which is the one that leaves the window when
// p arrives: eviction is positional and moves no data (njhaofan.com article,
// section "PrefixSliding如何丢掉中间Token？"; papers.ananclaw.com explainer,
// section "核心方法", "被丢弃的中间区").  When a call brings more than W
// ring-bound tokens, only the last W of them are written, which leaves the
// same bytes as appending the tokens one at a time.
//
// Pure copy work: one thread moves one 16-byte piece of a K row and the same
// piece of the V row; consecutive threads cover consecutive pieces, so both
// the reads and the writes are coalesced.
#include "ps_internal.h"

#include <hip/hip_bf16.h>

namespace ps {
namespace {

struct alignas(16) Vec16 {
    uint32_t w[4];
};

__global__ void __launch_bounds__(256) append_kernel(AppendParams p, int pieces_per_row) {
    if (p.c.guard && *p.c.guard) return;
    const int64_t total = (int64_t)p.n_seqs * p.n_new * p.c.hkv * pieces_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t row_bytes = (int64_t)pieces_per_row * 16;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int piece = (int)(idx % pieces_per_row);
        int64_t rest = idx / pieces_per_row;
        const int g = (int)(rest % p.c.hkv);
        rest /= p.c.hkv;
        const int t = (int)(rest % p.n_new);
        const int b = (int)(rest / p.n_new);

        const int64_t P = p.plen[b];
        const int64_t pos = p.pos[b] + t;
        const int64_t last = p.pos[b] + p.n_new - 1;
        char* kd;
        char* vd;
        if (pos < P) {  // prefix slot pos
            const int64_t row = prefix_row(p.c, b, g, pos);
            kd = static_cast<char*>(p.c.kpre) + row * row_bytes;
            vd = static_cast<char*>(p.c.vpre) + row * row_bytes;
        } else {        // ring slot (pos - P) mod W
            if (pos <= last - p.c.window) continue;  // overwritten later in this same call
            const int64_t row = ring_row(p.c, b, g, (pos - P) % p.c.window);
            kd = static_cast<char*>(p.c.kwin) + row * row_bytes;
            vd = static_cast<char*>(p.c.vwin) + row * row_bytes;
        }
        const int64_t src = ((((int64_t)b * p.n_new + t) * p.c.hkv + g) * row_bytes) + piece * 16;
        *reinterpret_cast<Vec16*>(kd + piece * 16) = *reinterpret_cast<const Vec16*>(static_cast<const char*>(p.knew) + src);
        *reinterpret_cast<Vec16*>(vd + piece * 16) = *reinterpret_cast<const Vec16*>(static_cast<const char*>(p.vnew) + src);
    }
}

// Append with the rotary encoding fused in: the new keys arrive unrotated and
// each is turned at its own position (Continue PE: the position of a token
// never changes, so its key is encoded once, on the way into the cache --
// agihunt.info summary, paragraph on position encodings).  The half-split
// pair (x_e, x_{e+d/2}) turns by pos * base^(-2e/d): the angle is formed in
// double precision from the host's frequency table, reduced to [-pi, pi],
// and its sine and cosine taken in fp32; the turn runs in fp32 with one
// rounding.  One thread owns 8 pairs of one row (16 bytes of each half of K,
// and the same bytes of V); slots as in append_kernel.
template <typename T, int D>
__global__ void __launch_bounds__(256) append_rope_kernel(AppendParams p, RopeFreqs f) {
    if (p.c.guard && *p.c.guard) return;
    constexpr int LPR = D / 16;
    const int64_t total = (int64_t)p.n_seqs * p.n_new * p.c.hkv * LPR;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int j = (int)(idx % LPR);
        int64_t rest = idx / LPR;
        const int g = (int)(rest % p.c.hkv);
        rest /= p.c.hkv;
        const int t = (int)(rest % p.n_new);
        const int b = (int)(rest / p.n_new);

        const int64_t P = p.plen[b];
        const int64_t pos = p.pos[b] + t;
        const int64_t last = p.pos[b] + p.n_new - 1;
        T* kd;
        T* vd;
        if (pos < P) {
            const int64_t row = prefix_row(p.c, b, g, pos);
            kd = static_cast<T*>(p.c.kpre) + row * D;
            vd = static_cast<T*>(p.c.vpre) + row * D;
        } else {
            if (pos <= last - p.c.window) continue;  // overwritten later in this same call
            const int64_t row = ring_row(p.c, b, g, (pos - P) % p.c.window);
            kd = static_cast<T*>(p.c.kwin) + row * D;
            vd = static_cast<T*>(p.c.vwin) + row * D;
        }
        const int64_t src = (((int64_t)b * p.n_new + t) * p.c.hkv + g) * D;
        const T* ks = static_cast<const T*>(p.knew) + src;
        const T* vs = static_cast<const T*>(p.vnew) + src;
        T a[8], c[8];
        __builtin_memcpy(a, ks + 8 * j, sizeof(a));
        __builtin_memcpy(c, ks + 8 * j + D / 2, sizeof(c));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double th = (double)pos * f.inv_freq[8 * j + i];
            const float r = (float)(th - 6.283185307179586 * rint(th * 0.15915494309189535));
            float sn, cs;
            sincosf(r, &sn, &cs);
            const float x0 = (float)a[i], x1 = (float)c[i];
            a[i] = (T)(x0 * cs - x1 * sn);
            c[i] = (T)(x0 * sn + x1 * cs);
        }
        __builtin_memcpy(kd + 8 * j, a, sizeof(a));
        __builtin_memcpy(kd + 8 * j + D / 2, c, sizeof(c));
        T va[8], vc[8];
        __builtin_memcpy(va, vs + 8 * j, sizeof(va));
        __builtin_memcpy(vc, vs + 8 * j + D / 2, sizeof(vc));
        __builtin_memcpy(vd + 8 * j, va, sizeof(va));
        __builtin_memcpy(vd + 8 * j + D / 2, vc, sizeof(vc));
    }
}

// Re-rotation of the window's keys by a position change (Reset PE: retained
// tokens are given new positions and their rotary-encoded keys recomputed --
// agihunt.info summary, paragraph on position encodings; njhaofan.com
// article, the passage comparing ContinuePE and ResetPE).  Rotary encoding
// turns the half-split pair (x_e, x_{e+d/2}) by pos * base^(-2e/d); rotations
// compose, so a key stored rotated at p becomes the key rotated at p + delta
// by one more turn of delta * base^(-2e/d).  The host computes the d/2
// cosines and sines in double precision; one lane owns the pair chunks
// e = 8j .. 8j + 7 and their partners (j = lane % (d/16)) and turns them in
// fp32 with one rounding to the cache type.  Memory-bound: every window key
// row is read and written once; V rows and prefix rows are not touched.
template <typename T, int D>
__global__ void __launch_bounds__(256) rerotate_kernel(RerotateParams p) {
    if (p.c.guard && *p.c.guard) return;
    constexpr int LPR = D / 16;          // lanes per row (each: 8 pairs)
    constexpr int RPW = 256 / LPR;       // rows per workgroup pass
    const int j = threadIdx.x % LPR;
    const int rsub = threadIdx.x / LPR;
    const int g = blockIdx.y, b = blockIdx.z;
    const int64_t P = p.plen[b];
    const int64_t pos = p.pos[b];
    const int64_t lo = pos - p.c.window > P ? pos - p.c.window : P;
    const int64_t count = pos - lo;      // window tokens [lo, pos)
    if ((int64_t)blockIdx.x * RPW >= count) return;
    float cs[8], sn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        cs[i] = p.cs[8 * j + i];
        sn[i] = p.sn[8 * j + i];
    }
    for (int64_t k = (int64_t)blockIdx.x * RPW + rsub; k < count; k += (int64_t)gridDim.x * RPW) {
        const int64_t t = lo + k;
        const int64_t slot = (t - P) % p.c.window;
        T* row = static_cast<T*>(p.c.kwin) + ring_row(p.c, b, g, slot) * D;
        T a[8], c[8];
        __builtin_memcpy(a, row + 8 * j, sizeof(a));
        __builtin_memcpy(c, row + 8 * j + D / 2, sizeof(c));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x0 = (float)a[i], x1 = (float)c[i];
            a[i] = (T)(x0 * cs[i] - x1 * sn[i]);
            c[i] = (T)(x0 * sn[i] + x1 * cs[i]);
        }
        __builtin_memcpy(row + 8 * j, a, sizeof(a));
        __builtin_memcpy(row + 8 * j + D / 2, c, sizeof(c));
    }
}

// One workgroup checks every sequence of a call (pairs of sequences for the
// duplicate-row and shared-prefix rules), then, if no check anywhere has
// failed, moves the rows' next positions past an append.
__global__ void __launch_bounds__(256) check_kernel(CheckParams p) {
    for (int b = threadIdx.x; b < p.n; b += blockDim.x) {
        const int32_t row = p.rows[b];
        const int32_t pr = p.prows ? p.prows[b] : row;
        const int64_t P = p.plen ? (int64_t)p.plen[b] : p.plen_scalar;
        const int64_t pos = p.pos ? p.pos[b] : p.pos_scalar;
        uint32_t f = 0;
        const bool row_ok = row >= 0 && row < p.max_seqs;
        if (!row_ok) f |= PS_CHECK_ROW;
        if (!p.pages && (pr < 0 || pr >= p.prefix_blocks)) f |= PS_CHECK_PREFIX_BLOCK;
        if (P < 0 || P > p.pcap) f |= PS_CHECK_PREFIX_LEN;
        // positions run up to 2^62 (far from int64 overflow of pos + length)
        if (pos < 0 || pos > ((int64_t)1 << 62) - p.n_new) f |= PS_CHECK_POSITION;
        if (p.pages)  // paged layout: every page the sequence may touch lies in the pool
            for (int j = 0; j < p.pages_per_seq; ++j) {
                const int32_t pg = p.pages[(int64_t)b * p.pages_per_seq + j];
                if (pg < 0 || pg >= p.n_pages) f |= PS_CHECK_PAGE;
            }
        for (int o = 0; o < b; ++o) {
            const int32_t orow = p.rows[o];
            if (orow == row) f |= PS_CHECK_DUPLICATE_ROW;
            const int32_t opr = p.prows ? p.prows[o] : orow;
            const int64_t oP = p.plen ? (int64_t)p.plen[o] : p.plen_scalar;
            if (!p.pages && opr == pr && oP != P) f |= PS_CHECK_SHARED_PREFIX;
        }
        if (row_ok && p.mode != kCheckNone) {
            const int64_t nx = p.next_pos[row];
            const int64_t want = p.mode == kCheckQuery ? nx - 1 : nx;
            // position 0 starts a new sequence in the row
            if (nx >= 0 && pos != 0 && pos != want) f |= PS_CHECK_SEQUENCE;
        }
        if (f) atomicOr(p.flags, f);
    }
    __syncthreads();
    if (p.mode != kCheckAppend) return;
    if (__hip_atomic_load(p.flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
    for (int b = threadIdx.x; b < p.n; b += blockDim.x) {
        const int64_t pos = p.pos ? p.pos[b] : p.pos_scalar;
        p.next_pos[p.rows[b]] = pos + p.n_new;
    }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t value) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = value;
}

}  // namespace

hipError_t launch_append(int dtype, int head_dim, const AppendParams& p, hipStream_t stream) {
    const int elem = dtype == PS_BF16 ? 2 : 4;
    const int pieces = head_dim * elem / 16;
    const int64_t total = (int64_t)p.n_seqs * p.n_new * p.c.hkv * pieces;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, pieces);
    return hipGetLastError();
}

hipError_t launch_check(const CheckParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(check_kernel, dim3(1), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, value);
    return hipGetLastError();
}

hipError_t launch_rerotate(int dtype, int head_dim, const RerotateParams& p, hipStream_t stream) {
    // one pass of 256 threads covers 256 / (d / 16) rows; the grid covers the
    // whole window of the longest possible sequence
    const int rpw = 256 / (head_dim / 16);
    const dim3 grid((unsigned)((p.c.window + rpw - 1) / rpw), (unsigned)p.c.hkv, (unsigned)p.n_seqs);
    if (dtype == PS_BF16) {
        if (head_dim == 128) hipLaunchKernelGGL((rerotate_kernel<__hip_bfloat16, 128>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((rerotate_kernel<__hip_bfloat16, 64>), grid, dim3(256), 0, stream, p);
    } else {
        if (head_dim == 128) hipLaunchKernelGGL((rerotate_kernel<float, 128>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((rerotate_kernel<float, 64>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_append_rope(int dtype, int head_dim, const AppendParams& p, const RopeFreqs& f,
                              hipStream_t stream) {
    const int64_t total = (int64_t)p.n_seqs * p.n_new * p.c.hkv * (head_dim / 16);
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const dim3 grid((unsigned)blocks);
    if (dtype == PS_BF16) {
        if (head_dim == 128) hipLaunchKernelGGL((append_rope_kernel<__hip_bfloat16, 128>), grid, dim3(256), 0, stream, p, f);
        else hipLaunchKernelGGL((append_rope_kernel<__hip_bfloat16, 64>), grid, dim3(256), 0, stream, p, f);
    } else {
        if (head_dim == 128) hipLaunchKernelGGL((append_rope_kernel<float, 128>), grid, dim3(256), 0, stream, p, f);
        else hipLaunchKernelGGL((append_rope_kernel<float, 64>), grid, dim3(256), 0, stream, p, f);
    }
    return hipGetLastError();
}

}  // namespace ps
