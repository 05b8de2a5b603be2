// Reference Philox4x32-10 stream from PyTorch's header-only engine
// (ATen/core/PhiloxRNGEngine.h), used to pin the oracle's Philox.
// stdin: lines "seed subsequence offset"; stdout: the first four 32-bit
// outputs of philox_engine(seed, subsequence, offset), in hex.
#include <ATen/core/PhiloxRNGEngine.h>

#include <cinttypes>
#include <cstdio>

int main()
{
    unsigned long long seed, sub, off;
    while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
        at::philox_engine e(seed, sub, off);
        const uint32_t a = e(), b = e(), c = e(), d = e();
        std::printf("%08" PRIx32 " %08" PRIx32 " %08" PRIx32 " %08" PRIx32 "\n", a, b, c, d);
    }
    return 0;
}
