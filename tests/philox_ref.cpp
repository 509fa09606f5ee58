// Independent Philox4x32-10 streams for the oracle's (seed, element) mapping:
// key = seed, counter = (i >> 2, 0, 0) as a 128-bit integer, output word i & 3.
// Built by the tests against either rocRAND's or PyTorch's header-only engine.
// Reads "seed index" pairs from stdin, prints one hex word per pair.
#include <cstdint>
#include <cstdio>
#ifdef USE_ROCRAND
#include <rocrand/rocrand_philox4x32_10.h>
#else
#include <ATen/core/PhiloxRNGEngine.h>
#endif

int main() {
    unsigned long long seed, index;
    while (std::scanf("%llu %llu", &seed, &index) == 2) {
#ifdef USE_ROCRAND
        // offset counts 32-bit outputs: counter = offset / 4, word = offset % 4
        rocrand_device::philox4x32_10_engine eng(seed, 0, index);
        unsigned int u = eng();
#else
        // offset counts 128-bit blocks; each call returns the next word of the block
        at::philox_engine eng(seed, 0, index >> 2);
        uint32_t u = 0;
        for (unsigned k = 0; k <= (index & 3); ++k) u = eng();
#endif
        std::printf("%08x\n", u);
    }
    return 0;
}
