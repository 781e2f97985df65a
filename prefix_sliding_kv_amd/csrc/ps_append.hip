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

namespace ps {
namespace {

struct alignas(16) Vec16 {
    uint32_t w[4];
};

__global__ void __launch_bounds__(256) append_kernel(AppendParams p, int pieces_per_row) {
    const int64_t total = (int64_t)p.n_seqs * p.n_new * p.hkv * pieces_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t row_bytes = (int64_t)pieces_per_row * 16;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int piece = (int)(idx % pieces_per_row);
        int64_t rest = idx / pieces_per_row;
        const int g = (int)(rest % p.hkv);
        rest /= p.hkv;
        const int t = (int)(rest % p.n_new);
        const int b = (int)(rest / p.n_new);

        const int64_t P = p.plen[b];
        const int64_t pos = p.pos[b] + t;
        const int64_t last = p.pos[b] + p.n_new - 1;
        int64_t phys;
        if (pos < P) {
            phys = pos;
        } else {
            if (pos <= last - p.window) continue;  // overwritten later in this same call
            phys = p.pcap + (pos - P) % p.window;
        }
        const int64_t src = ((((int64_t)b * p.n_new + t) * p.hkv + g) * row_bytes) + piece * 16;
        const int64_t dst = ((((int64_t)p.rows[b] * p.hkv + g) * p.rows_per_head + phys) * row_bytes) + piece * 16;
        *reinterpret_cast<Vec16*>(static_cast<char*>(p.kc) + dst) =
            *reinterpret_cast<const Vec16*>(static_cast<const char*>(p.knew) + src);
        *reinterpret_cast<Vec16*>(static_cast<char*>(p.vc) + dst) =
            *reinterpret_cast<const Vec16*>(static_cast<const char*>(p.vnew) + src);
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
    const int64_t total = (int64_t)p.n_seqs * p.n_new * p.hkv * pieces;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, pieces);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, value);
    return hipGetLastError();
}

}  // namespace ps
