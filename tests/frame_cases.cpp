// Prints the position frame (ps::pos_frame in the library's internal header)
// of each "S T P W chunk_only" line read from stdin as "P W shift move_from".
// Built with the host compiler by tests/test_abi_host.py; no GPU code.
#include <cstdio>

#include "../prefix_sliding_kv_amd/csrc/ps_internal.h"

int main() {
    long long S, T, P, W;
    int chunk_only;
    while (std::scanf("%lld %lld %lld %lld %d", &S, &T, &P, &W, &chunk_only) == 5) {
        const ps::PosFrame f = ps::pos_frame(S, T, P, W, chunk_only != 0);
        std::printf("%lld %lld %lld %lld\n", (long long)f.P, (long long)f.W, (long long)f.shift,
                    (long long)f.move_from);
    }
    return 0;
}
