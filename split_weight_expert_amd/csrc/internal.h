// Declarations shared between the library's translation units (not part of the ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <vector>

#include "../../include/dwdp.h"

namespace dwdp {

constexpr int kMaxCopySources = 64;
// Kernels with one workgroup per row or token launch at most this many workgroups and walk the rest
// (a launch holds fewer than 2^32 work-items).
constexpr int64_t kMaxRowGrid = 1 << 20;
// Work-items one launch may hold.
constexpr int64_t kMaxLaunchItems = ((int64_t)1 << 32) - 1;
constexpr int kBmMin = 32;             // smallest expert-GEMM tile height (sizes the m-tile tables)
constexpr size_t kMTileBytes = 16;     // one entry of an m-tile table
constexpr int kPermuteWaves = 16;      // waves per count / scatter workgroup of the permutation (E > kHistMaxE)
// Permutation by chunk histograms (E <= kHistMaxE): the T*k entries are cut into chunks of
// hist_chunk(N) consecutive entries, one wave each, so that there are at most kHistMaxChunks of them.
constexpr int kHistMaxE = 4096;
constexpr int64_t kHistMaxChunks = 1024;
inline int64_t hist_chunk(int64_t N) {
    const int64_t per = (N + kHistMaxChunks - 1) / kHistMaxChunks;
    const int64_t c = (per + 63) / 64 * 64;
    return c < 1024 ? 1024 : c;
}
inline int64_t hist_chunks(int64_t N) { return (N + hist_chunk(N) - 1) / hist_chunk(N); }

// Grouped-FFN workspace: A [rows, I] in the activation type (+ its fp8 scales [rows, I/128]), the
// m-tile prefix [G+1], two m-tile tables and the two expert-GEMM launches' tile tickets (int32 each),
// each part 256-byte aligned; the tables are sized for the smallest tile height, so any tile choice
// fits.
struct FfnWs {
    size_t a, a_scale, pre, mt, mt_by_size, tickets, total;
};
FfnWs ffn_ws_layout(int64_t rows, int groups, int I, int dtype);

size_t elem_bytes(int dtype);
void record_layout(int H, int I, int w_dtype, size_t* w2, size_t* s13, size_t* s2, size_t* total);
// Slices of a source of `bytes` bytes cut into `chunk`-byte pieces (no sum that could wrap).
size_t n_slices(size_t bytes, size_t chunk);
std::vector<dwdp_chunk> make_plan(const dwdp_copy_src* srcs, int n_src, size_t chunk);
int check_sources(const dwdp_copy_src* srcs, int n_src, size_t chunk);

size_t permute_ws_bytes(int64_t T, int k, int E);
size_t ffn_ws_bytes(int64_t rows, int groups, int H, int I, int dtype);

}  // namespace dwdp
