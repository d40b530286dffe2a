// Randomised driver of the library's host-only logic (test infrastructure only), built together with
// split_weight_expert_amd/csrc/host.cpp by a plain C++ compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).  It needs no GPU and no HIP runtime.
//
// What it drives, with valid and invalid arguments:
//   * dwdp_prefetch_plan: fixed-size slices issued round-robin over the sources (DWDP paper summary
//     §4.3.2).  Checked: every byte of every source is covered exactly once, slices never exceed the
//     chunk size, slice c of every source precedes slice c+1 of any, overlapping destinations and a
//     zero chunk are rejected, and a too-small output array is never overrun;
//   * dwdp_fill_expert_table: the per-expert pointer table over separate buffers (§4.2), against the
//     record layout of dwdp_expert_record_bytes / _offsets (parts 256-byte aligned, disjoint, inside
//     the record), with out-of-range buffers, negative slots and misaligned buffers rejected;
//   * dwdp_workspace_bytes: monotone in T, 0 for invalid arguments, large enough for A.
// Exit status 0 when every check holds; the sanitizers abort on any memory or UB error.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/dwdp.h"

static int g_fail = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            std::fprintf(stderr, "CHECK failed (%s:%d) %s: ", __FILE__, __LINE__, #cond); \
            std::fprintf(stderr, __VA_ARGS__);            \
            std::fprintf(stderr, "\n");                   \
            if (++g_fail > 20) std::exit(1);              \
        }                                                 \
    } while (0)

static void fuzz_plan(std::mt19937_64& rng, int iters) {
    for (int it = 0; it < iters; ++it) {
        const int n = 1 + (int)(rng() % 8);
        std::vector<dwdp_copy_src> src(n);
        size_t off = rng() % 64;
        std::vector<size_t> sizes(n);
        for (int s = 0; s < n; ++s) {
            const int kind = (int)(rng() % 4);
            sizes[s] = kind == 0 ? 0 : kind == 1 ? rng() % 64 : rng() % 20000;
            src[s].src = reinterpret_cast<const void*>((uintptr_t)0x1000 * (s + 1));
            src[s].dst_offset = off;
            src[s].bytes = sizes[s];
            off += sizes[s] + rng() % 3;
        }
        const int ck = (int)(rng() % 5);
        const size_t chunk = ck == 0 ? 1 + rng() % 16 : ck == 1 ? SIZE_MAX - rng() % 4 : ck == 2 ? ((size_t)1 << 40)
                                                                                       : 1 + rng() % 5000;
        size_t count = 0;
        int rc = dwdp_prefetch_plan(src.data(), n, chunk, nullptr, 0, &count);
        CHECK(rc == DWDP_OK, "valid plan rejected: %s", dwdp_last_error());
        if (rc != DWDP_OK) continue;
        size_t expect = 0;
        for (size_t b : sizes) expect += b == 0 ? 0 : (b - 1) / chunk + 1;
        CHECK(count == expect, "slice count %zu, expected %zu", count, expect);
        // a short output array: only max_chunks entries may be written
        const size_t cap = count == 0 ? 0 : rng() % (count + 1);
        std::vector<dwdp_chunk> part(cap + 1);
        std::memset(&part[cap], 0xAB, sizeof(dwdp_chunk));
        size_t again = 0;
        rc = dwdp_prefetch_plan(src.data(), n, chunk, cap ? part.data() : nullptr, cap, &again);
        CHECK(rc == DWDP_OK && again == count, "second call");
        const unsigned char* sentinel = reinterpret_cast<const unsigned char*>(&part[cap]);
        for (size_t i = 0; i < sizeof(dwdp_chunk); ++i) CHECK(sentinel[i] == 0xAB, "entry past max_chunks written");
        std::vector<dwdp_chunk> plan(count);
        rc = dwdp_prefetch_plan(src.data(), n, chunk, plan.data(), count, &again);
        CHECK(rc == DWDP_OK, "full plan");
        // coverage: per source, slices tile [0, bytes) in order; round-robin across sources
        std::vector<size_t> next(n, 0);
        std::vector<size_t> round_of(n, 0);
        size_t prev_round = 0;
        for (size_t i = 0; i < count; ++i) {
            const dwdp_chunk& c = plan[i];
            CHECK(c.source >= 0 && c.source < n, "source %d", c.source);
            if (c.source < 0 || c.source >= n) break;
            const int s = c.source;
            CHECK(c.src_offset == next[s], "slice of source %d starts at %zu, expected %zu", s, c.src_offset, next[s]);
            CHECK(c.bytes >= 1 && c.bytes <= chunk, "slice size %zu", c.bytes);
            CHECK(c.dst_offset == src[s].dst_offset + c.src_offset, "dst offset");
            CHECK(c.src_offset + c.bytes <= sizes[s], "slice past the source");
            const size_t r = c.src_offset / chunk;
            CHECK(r >= prev_round, "round %zu after round %zu", r, prev_round);
            prev_round = r;
            next[s] += c.bytes;
        }
        for (int s = 0; s < n; ++s) CHECK(next[s] == sizes[s], "source %d covered %zu of %zu", s, next[s], sizes[s]);
        // an overlap anywhere is rejected
        if (n >= 2 && sizes[0] > 0 && sizes[1] > 0) {
            std::vector<dwdp_copy_src> bad = src;
            bad[1].dst_offset = bad[0].dst_offset + sizes[0] - 1;
            CHECK(dwdp_prefetch_plan(bad.data(), n, chunk, nullptr, 0, &again) == DWDP_ERR_INVALID_ARG, "overlap");
        }
        CHECK(dwdp_prefetch_plan(src.data(), n, 0, nullptr, 0, &again) == DWDP_ERR_INVALID_ARG, "zero chunk");
        CHECK(dwdp_prefetch_plan(src.data(), 0, chunk, nullptr, 0, &again) == DWDP_ERR_INVALID_ARG, "no sources");
        CHECK(dwdp_prefetch_plan(nullptr, n, chunk, nullptr, 0, &again) == DWDP_ERR_INVALID_ARG, "null sources");
    }
    // a destination range that wraps the address space
    dwdp_copy_src wrap{reinterpret_cast<const void*>((uintptr_t)0x1000), SIZE_MAX - 10, 100};
    size_t cnt = 0;
    CHECK(dwdp_prefetch_plan(&wrap, 1, 16, nullptr, 0, &cnt) == DWDP_ERR_INVALID_ARG, "wrapping destination");
}

static void fuzz_table(std::mt19937_64& rng, int iters) {
    const int dts[3] = {DWDP_F32, DWDP_BF16, DWDP_FP8_E4M3};
    for (int it = 0; it < iters; ++it) {
        const int dt = dts[rng() % 3];
        const int H = 128 * (1 + (int)(rng() % 64)), I = 128 * (1 + (int)(rng() % 32));
        const size_t rec = dwdp_expert_record_bytes(H, I, dt);
        size_t o_w2 = 0, o_s13 = 0, o_s2 = 0;
        CHECK(dwdp_expert_record_offsets(H, I, dt, &o_w2, &o_s13, &o_s2) == DWDP_OK, "offsets");
        const size_t eb = dt == DWDP_F32 ? 4 : dt == DWDP_BF16 ? 2 : 1;
        CHECK(o_w2 % 256 == 0 && o_w2 >= (size_t)2 * I * H * eb, "W2 offset %zu", o_w2);
        CHECK(o_s13 >= o_w2 + (size_t)H * I * eb && o_s13 % 256 == 0, "S13 offset");
        if (dt == DWDP_FP8_E4M3) {
            CHECK(o_s2 >= o_s13 + (size_t)(2 * I / 128) * (H / 128) * 4 && o_s2 % 256 == 0, "S2 offset");
            CHECK(rec >= o_s2 + (size_t)(H / 128) * (I / 128) * 4, "record size");
        } else {
            CHECK(rec >= o_w2 + (size_t)H * I * eb, "record size");
        }
        CHECK(rec % 256 == 0, "record size %zu not 256-aligned", rec);
        const int nb = 1 + (int)(rng() % 4), G = 1 + (int)(rng() % 300);
        std::vector<void*> bufs(nb);
        for (int b = 0; b < nb; ++b) bufs[b] = reinterpret_cast<void*>((uintptr_t)(b + 1) << 40);
        std::vector<int32_t> bo(G), so(G);
        for (int g = 0; g < G; ++g) {
            bo[g] = (int32_t)(rng() % nb);
            so[g] = (int32_t)(rng() % 512);
        }
        std::vector<dwdp_expert_ptrs> out(G + 1);
        std::memset(&out[G], 0xCD, sizeof(dwdp_expert_ptrs));
        CHECK(dwdp_fill_expert_table(bufs.data(), nb, bo.data(), so.data(), G, H, I, dt, out.data()) == DWDP_OK,
              "table: %s", dwdp_last_error());
        for (int g = 0; g < G; ++g) {
            const uintptr_t r = (uintptr_t)bufs[bo[g]] + (uintptr_t)so[g] * rec;
            CHECK((uintptr_t)out[g].w13 == r && (uintptr_t)out[g].w2 == r + o_w2, "group %d", g);
            if (dt == DWDP_FP8_E4M3)
                CHECK((uintptr_t)out[g].s13 == r + o_s13 && (uintptr_t)out[g].s2 == r + o_s2, "scales %d", g);
            else
                CHECK(out[g].s13 == nullptr && out[g].s2 == nullptr, "scales must be NULL");
        }
        const unsigned char* sentinel = reinterpret_cast<const unsigned char*>(&out[G]);
        for (size_t i = 0; i < sizeof(dwdp_expert_ptrs); ++i) CHECK(sentinel[i] == 0xCD, "entry past n_groups written");
        // invalid placements
        std::vector<int32_t> bad = bo;
        bad[rng() % G] = nb;
        CHECK(dwdp_fill_expert_table(bufs.data(), nb, bad.data(), so.data(), G, H, I, dt, out.data()) ==
                  DWDP_ERR_INVALID_ARG, "buffer out of range");
        bad = so;
        bad[rng() % G] = -1;
        CHECK(dwdp_fill_expert_table(bufs.data(), nb, bo.data(), bad.data(), G, H, I, dt, out.data()) ==
                  DWDP_ERR_INVALID_ARG, "negative slot");
        std::vector<void*> odd = bufs;
        odd[0] = reinterpret_cast<void*>((uintptr_t)odd[0] + 4);
        std::vector<int32_t> zero(G, 0);
        CHECK(dwdp_fill_expert_table(odd.data(), nb, zero.data(), so.data(), G, H, I, dt, out.data()) ==
                  DWDP_ERR_INVALID_ARG, "misaligned buffer");
    }
    CHECK(dwdp_expert_record_bytes(0, 128, DWDP_BF16) == 0 && dwdp_expert_record_bytes(128, 128, 9) == 0, "invalid");
}

static void fuzz_workspace(std::mt19937_64& rng, int iters) {
    const int dts[3] = {DWDP_F32, DWDP_BF16, DWDP_FP8_E4M3};
    for (int it = 0; it < iters; ++it) {
        const int dt = dts[rng() % 3];
        const int64_t T = (int64_t)(rng() % 40000);
        const int k = 1 + (int)(rng() % 16), E = k + (int)(rng() % 300), S = (int)(rng() % 2);
        const int H = 256 * (1 + (int)(rng() % 32)), I = 128 * (1 + (int)(rng() % 32));
        const size_t a = dwdp_workspace_bytes(DWDP_OP_GROUPED_FFN, T, k, E, H, I, dt, S);
        const size_t b = dwdp_workspace_bytes(DWDP_OP_GROUPED_FFN, T + 1 + (int64_t)(rng() % 100), k, E, H, I, dt, S);
        const size_t eb = dt == DWDP_F32 ? 4 : dt == DWDP_BF16 ? 2 : 1;
        const int64_t rows = T * k + S * T;
        CHECK(a >= (size_t)rows * I * eb + (size_t)(E + S + 1) * 4, "FFN workspace %zu for %lld rows", a, (long long)rows);
        CHECK(b >= a && a % 256 == 0, "FFN workspace not monotone");
        const size_t p = dwdp_workspace_bytes(DWDP_OP_PERMUTE, T, k, E, H, I, dt, S);
        CHECK(p >= (size_t)E * 4 && p % 256 == 0, "permute workspace %zu", p);
        CHECK(dwdp_workspace_bytes(DWDP_OP_GROUPED_FFN, -1, k, E, H, I, dt, S) == 0, "negative T");
        CHECK(dwdp_workspace_bytes(DWDP_OP_GROUPED_FFN, T, 0, E, H, I, dt, S) == 0, "k = 0");
        CHECK(dwdp_workspace_bytes(DWDP_OP_GROUPED_FFN, T, k, E, H, I, dt, 2) == 0, "shared = 2");
        CHECK(dwdp_workspace_bytes(7, T, k, E, H, I, dt, S) == 0, "unknown op");
        CHECK(dwdp_workspace_bytes(DWDP_OP_GROUPED_FFN, T, k, E, H, I, 9, S) == 0, "unknown dtype");
    }
}

int main(int argc, char** argv) {
    const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
    const int iters = argc > 2 ? std::atoi(argv[2]) : 2000;
    std::mt19937_64 rng(seed);
    fuzz_plan(rng, iters);
    fuzz_table(rng, iters / 4);
    fuzz_workspace(rng, iters);
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("host logic ok (seed %llu, %d iterations)\n", (unsigned long long)seed, iters);
    return 0;
}
