// Drives the library's host-side plan construction (onebit_plan_host_tables) over
// random and adversarial chunk / tensor tables, for a build whose host pass has
// -fsanitize=address,undefined: empty chunks, chunks of every length around the
// 2048-element tile and the 32-element word, unaligned starts, masked runs that
// start, end or cover whole tiles, adjacent masked tensors, a million one-element
// chunks, and invalid tables (decreasing offsets, a tensor table that does not end
// at n, keep flags without a tensor table).  Each table is queried twice: sizes,
// then contents into exactly sized buffers, whose invariants are checked (tiles
// cover the chunks in order, words per chunk, masked intervals sorted and disjoint).
// No device is touched.  Prints "ok" and exits 0 when every check holds.  Test
// infrastructure only.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

extern "C" int onebit_plan_host_tables(const int64_t *chunk_offsets, int64_t n_chunks, const int64_t *tensor_offsets,
                                       const uint8_t *tensor_keep, int64_t n_tensors, int64_t *n_tiles,
                                       int64_t *n_words, int64_t *out_tiles, int64_t *n_mask_iv,
                                       int64_t *out_mask_iv);

// plan.hip is built alone; its plan-creation path (never called here) takes these
// from the compression kernels' file.
namespace onebit {
int32_t resident_capacity(int) { return 1; }
int32_t onepass_depth() { return 3; }
}  // namespace onebit

static int failures = 0;

static void check(bool ok, const char *what, int64_t a = 0) {
    if (!ok) {
        std::fprintf(stderr, "check failed: %s (%lld)\n", what, (long long)a);
        ++failures;
    }
}

static void run(const std::vector<int64_t> &co, const std::vector<int64_t> &to, const std::vector<uint8_t> &keep) {
    const int64_t nc = (int64_t)co.size() - 1, nt = to.empty() ? 0 : (int64_t)to.size() - 1;
    int64_t tiles = -1, words = -1, niv = -1;
    int st = onebit_plan_host_tables(co.data(), nc, to.empty() ? nullptr : to.data(),
                                     keep.empty() ? nullptr : keep.data(), nt, &tiles, &words, nullptr, &niv, nullptr);
    check(st == 0, "valid table accepted", st);
    if (st != 0) return;
    std::vector<int64_t> t((size_t)(6 * tiles)), iv((size_t)(2 * niv));
    st = onebit_plan_host_tables(co.data(), nc, to.empty() ? nullptr : to.data(), keep.empty() ? nullptr : keep.data(),
                                 nt, nullptr, nullptr, t.data(), nullptr, iv.data());
    check(st == 0, "second query", st);
    int64_t k = 0, word = 0;
    for (int64_t j = 0; j < nc; ++j) {
        const int64_t len = co[j + 1] - co[j], ntile = len > 0 ? (len + 2047) / 2048 : 1;
        for (int64_t q = 0; q < ntile; ++q, ++k) {
            const int64_t *r = &t[(size_t)(6 * k)];
            check(r[0] == co[j] + 2048 * q, "tile start", k);
            check(r[1] == word + 64 * q, "tile first word", k);
            check(r[2] == (len > 0 ? std::min<int64_t>(2048, len - 2048 * q) : 0), "tile length", k);
            check(r[3] == j, "tile chunk", k);
            check(r[4] == -1 || (r[4] >= 0 && r[4] <= r[5] && r[5] <= niv), "tile mask range", k);
        }
        word += (len + 31) / 32;
    }
    check(k == tiles, "tile count", tiles);
    check(word == words, "word count", words);
    for (int64_t i = 0; i < niv; ++i) {
        check(iv[(size_t)(2 * i)] < iv[(size_t)(2 * i + 1)], "interval non-empty", i);
        if (i > 0) check(iv[(size_t)(2 * i - 1)] < iv[(size_t)(2 * i)], "intervals sorted, disjoint, merged", i);
    }
}

static void expect_invalid(const std::vector<int64_t> &co, const std::vector<int64_t> &to,
                           const std::vector<uint8_t> &keep, const char *what) {
    int64_t tiles = 0, words = 0, niv = 0;
    const int st = onebit_plan_host_tables(co.data(), (int64_t)co.size() - 1, to.empty() ? nullptr : to.data(),
                                           keep.empty() ? nullptr : keep.data(), to.empty() ? 0 : (int64_t)to.size() - 1,
                                           &tiles, &words, nullptr, &niv, nullptr);
    check(st != 0, what);
}

int main() {
    std::mt19937_64 rng(12345);
    // every chunk length around the tile and word boundaries, aligned and unaligned starts
    for (int64_t len : {0, 1, 31, 32, 33, 2047, 2048, 2049, 4095, 4096, 4097, 6145}) {
        for (int64_t pre : {0, 1, 3, 4}) {
            std::vector<int64_t> co = {0, pre, pre + len, pre + len + 5};
            run(co, {}, {});
            std::vector<int64_t> to = {0, pre + len / 2, pre + len + 5};
            run(co, to, {1, 0});
            run(co, to, {0, 0});
        }
    }
    // random tables with masks
    for (int it = 0; it < 300; ++it) {
        const int nc = 1 + (int)(rng() % 40);
        std::vector<int64_t> co = {0};
        for (int j = 0; j < nc; ++j) co.push_back(co.back() + (int64_t)(rng() % 3 == 0 ? rng() % 9000 : rng() % 70));
        const int64_t n = co.back();
        std::vector<int64_t> to = {0};
        while (to.back() < n) to.push_back(std::min<int64_t>(n, to.back() + (int64_t)(rng() % 5000)));
        if (to.size() == 1) to.push_back(n);
        std::vector<uint8_t> keep(to.size() - 1);
        for (auto &b : keep) b = (uint8_t)(rng() % 3 != 0);
        run(co, to, keep);
        run(co, {}, {});
    }
    // a million one-element chunks
    std::vector<int64_t> many(1000001);
    for (size_t i = 0; i < many.size(); ++i) many[i] = (int64_t)i;
    run(many, {}, {});
    // invalid tables
    expect_invalid({0, 5, 3}, {}, {}, "decreasing chunk offsets");
    expect_invalid({1, 5}, {}, {}, "chunk table not starting at 0");
    expect_invalid({0, 5}, {0, 4}, {1}, "tensor table not ending at n");
    expect_invalid({0, 5}, {}, {1}, "keep flags without a tensor table");
    if (failures) {
        std::fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
