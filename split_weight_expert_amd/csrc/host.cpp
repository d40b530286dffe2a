// Host-side parts of the C ABI: error state, workspace sizing, the expert
// record layout and pointer table (the split-weight "TensorList" of the DWDP
// paper summary, §4.2), and the round-robin slice plan of the prefetch (§4.3.2).
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "errors.h"
#include "internal.h"

namespace dwdp {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t elem_bytes(int dtype) {
    switch (dtype) {
        case DWDP_F32: return 4;
        case DWDP_BF16: return 2;
        case DWDP_FP8_E4M3: return 1;
        default: return 0;
    }
}

void record_layout(int H, int I, int w_dtype, size_t* w2, size_t* s13, size_t* s2, size_t* total) {
    size_t eb = elem_bytes(w_dtype);
    size_t n13 = (size_t)2 * I * H, n2 = (size_t)H * I;
    size_t o_w2 = align256(n13 * eb);
    size_t end = o_w2 + align256(n2 * eb);
    size_t o_s13 = end, o_s2 = end;
    if (w_dtype == DWDP_FP8_E4M3) {
        size_t ns13 = (size_t)(2 * I / kFp8Group) * (H / kFp8Group);
        size_t ns2 = (size_t)(H / kFp8Group) * (I / kFp8Group);
        o_s13 = end;
        o_s2 = o_s13 + align256(ns13 * 4);
        end = o_s2 + align256(ns2 * 4);
    }
    *w2 = o_w2;
    *s13 = o_s13;
    *s2 = o_s2;
    *total = end;
}

FfnWs ffn_ws_layout(int64_t rows, int groups, int I, int dtype) {
    FfnWs w{};
    const size_t ea = elem_bytes(dtype);
    const int64_t maxm = (rows + kBmMin - 1) / kBmMin + groups;
    size_t off = 0;
    w.a = off;
    off += align256((size_t)rows * I * ea);
    w.a_scale = off;
    if (dtype == DWDP_FP8_E4M3) off += align256((size_t)rows * (I / kFp8Group) * 4);
    w.pre = off;
    off += align256((size_t)(groups + 1) * 4);
    w.mt = off;
    off += align256((size_t)maxm * kMTileBytes);
    w.mt_by_size = off;
    off += align256((size_t)maxm * kMTileBytes);
    w.tickets = off;
    off += align256(2 * sizeof(int32_t));
    w.total = off;
    return w;
}

size_t ffn_ws_bytes(int64_t rows, int groups, int H, int I, int dtype) {
    (void)H;
    if (elem_bytes(dtype) == 0) return 0;
    return ffn_ws_layout(rows, groups, I, dtype).total;
}

size_t permute_ws_bytes(int64_t T, int k, int E) {
    if (E <= kHistMaxE) return align256((size_t)hist_chunks(T * k) * (size_t)E * 4);   // [chunks][E]
    return align256((size_t)E * kPermuteWaves * 4 * 2);
}

size_t n_slices(size_t bytes, size_t chunk) { return bytes == 0 ? 0 : (bytes - 1) / chunk + 1; }

std::vector<dwdp_chunk> make_plan(const dwdp_copy_src* srcs, int n_src, size_t chunk) {
    std::vector<dwdp_chunk> plan;
    size_t most = 0;
    for (int s = 0; s < n_src; ++s) most = std::max(most, n_slices(srcs[s].bytes, chunk));
    for (size_t c = 0; c < most; ++c) {
        for (int s = 0; s < n_src; ++s) {
            size_t n = n_slices(srcs[s].bytes, chunk);
            if (c >= n) continue;
            dwdp_chunk ch{};
            ch.source = s;
            ch.src_offset = c * chunk;
            ch.dst_offset = srcs[s].dst_offset + c * chunk;
            ch.bytes = std::min(chunk, srcs[s].bytes - c * chunk);
            plan.push_back(ch);
        }
    }
    return plan;
}

int check_sources(const dwdp_copy_src* srcs, int n_src, size_t chunk) {
    if (srcs == nullptr) return fail(DWDP_ERR_INVALID_ARG, "prefetch: srcs is NULL");
    if (n_src < 1 || n_src > kMaxCopySources)
        return fail(DWDP_ERR_INVALID_ARG, "prefetch: n_src must be in [1, 64]");
    if (chunk == 0) return fail(DWDP_ERR_INVALID_ARG, "prefetch: chunk_bytes is 0");
    std::vector<std::pair<size_t, size_t>> ranges;
    for (int s = 0; s < n_src; ++s) {
        if (srcs[s].bytes == 0) continue;
        if (srcs[s].src == nullptr) return fail(DWDP_ERR_INVALID_ARG, "prefetch: a source pointer is NULL");
        if (srcs[s].dst_offset + srcs[s].bytes < srcs[s].dst_offset)
            return fail(DWDP_ERR_INVALID_ARG, "prefetch: destination range overflows");
        ranges.emplace_back(srcs[s].dst_offset, srcs[s].dst_offset + srcs[s].bytes);
    }
    std::sort(ranges.begin(), ranges.end());
    for (size_t i = 1; i < ranges.size(); ++i)
        if (ranges[i].first < ranges[i - 1].second)
            return fail(DWDP_ERR_INVALID_ARG, "prefetch: destination ranges overlap");
    return DWDP_OK;
}

}  // namespace dwdp

using namespace dwdp;

extern "C" {

const char* dwdp_last_error(void) { return g_last_error.c_str(); }

// The compile-time kernel options this build was made with are listed after the architecture.
#define DWDP_STR2(x) #x
#define DWDP_STR(x) DWDP_STR2(x)
const char* dwdp_version(void) {
    return "dwdp-mi355x 0.2 (gfx950)"
#ifdef DWDP_FP8_BM256
           " fp8-bm256"
#endif
#ifdef DWDP_MSUPER_BF16
           " msuper-bf16=" DWDP_STR(DWDP_MSUPER_BF16)
#endif
#ifdef DWDP_MSUPER_FP8
           " msuper-fp8=" DWDP_STR(DWDP_MSUPER_FP8)
#endif
#ifdef DWDP_MSUPER_FP8_GEMM2
           " msuper-fp8-gemm2=" DWDP_STR(DWDP_MSUPER_FP8_GEMM2)
#endif
#ifdef DWDP_MSUPER_BALANCED
           " msuper-balanced=" DWDP_STR(DWDP_MSUPER_BALANCED)
#endif
#ifdef DWDP_SPARSE_ROWS
           " sparse-rows=" DWDP_STR(DWDP_SPARSE_ROWS)
#endif
#ifdef DWDP_BALANCED_MTILES
           " balanced-mtiles=" DWDP_STR(DWDP_BALANCED_MTILES)
#endif
#ifdef DWDP_WEIGHT_CPOL
           " weight-cpol=" DWDP_STR(DWDP_WEIGHT_CPOL)
#endif
#ifdef DWDP_STREAM_WEIGHT_CPOL
           " stream-weight-cpol=" DWDP_STR(DWDP_STREAM_WEIGHT_CPOL)
#endif
#ifdef DWDP_YPERM_NT
           " yperm-nt=" DWDP_STR(DWDP_YPERM_NT)
#endif
#ifdef DWDP_CLUSTER_GEMM1_LOG2
           " cluster-gemm1-log2=" DWDP_STR(DWDP_CLUSTER_GEMM1_LOG2)
#endif
#ifdef DWDP_CLUSTER_GEMM2_LOG2
           " cluster-gemm2-log2=" DWDP_STR(DWDP_CLUSTER_GEMM2_LOG2)
#endif
#ifdef DWDP_TICKET_TILES
           " ticket-tiles=" DWDP_STR(DWDP_TICKET_TILES)
#endif
#ifdef DWDP_TILE_TRACE
           " tile-trace=" DWDP_STR(DWDP_TILE_TRACE)
#endif
#ifdef DWDP_MFMA_E8M0
           " mfma-e8m0=" DWDP_STR(DWDP_MFMA_E8M0)
#endif
#ifdef DWDP_FP8_GEMM2_BM256
           " fp8-gemm2-bm256=" DWDP_STR(DWDP_FP8_GEMM2_BM256)
#endif
#ifdef DWDP_SILU_RCP
           " silu-rcp=" DWDP_STR(DWDP_SILU_RCP)
#endif
#ifdef DWDP_ROUTER_DMA
           " router-dma=" DWDP_STR(DWDP_ROUTER_DMA)
#endif
#ifdef DWDP_ROUTER_SPLITK_TILE
           " router-splitk-tile=" DWDP_STR(DWDP_ROUTER_SPLITK_TILE)
#endif
#ifdef DWDP_COMBINE_NT
           " combine-nt=" DWDP_STR(DWDP_COMBINE_NT)
#endif
#ifdef DWDP_ACT_CPOL
           " act-cpol=" DWDP_STR(DWDP_ACT_CPOL)
#endif
        ;
}

size_t dwdp_expert_record_bytes(int H, int I, int w_dtype) {
    if (H <= 0 || I <= 0 || elem_bytes(w_dtype) == 0) return 0;
    size_t a, b, c, t;
    record_layout(H, I, w_dtype, &a, &b, &c, &t);
    return t;
}

int dwdp_expert_record_offsets(int H, int I, int w_dtype, size_t* off_w2, size_t* off_s13, size_t* off_s2) {
    clear_error();
    DWDP_REQUIRE(H > 0 && I > 0, "H and I must be positive");
    DWDP_REQUIRE(elem_bytes(w_dtype) != 0, "unknown w_dtype");
    DWDP_REQUIRE(off_w2 && off_s13 && off_s2, "null output pointer");
    size_t t;
    record_layout(H, I, w_dtype, off_w2, off_s13, off_s2, &t);
    return DWDP_OK;
}

int dwdp_fill_expert_table(void* const* buffers, int n_buffers, const int32_t* buf_of, const int32_t* slot_of,
                           int n_groups, int H, int I, int w_dtype, dwdp_expert_ptrs* out) {
    clear_error();
    DWDP_REQUIRE(buffers && buf_of && slot_of && out, "null pointer argument");
    DWDP_REQUIRE(n_buffers > 0 && n_groups > 0, "n_buffers and n_groups must be positive");
    DWDP_REQUIRE(H > 0 && I > 0 && elem_bytes(w_dtype) != 0, "bad H, I or w_dtype");
    if (w_dtype == DWDP_FP8_E4M3) DWDP_REQUIRE(H % kFp8Group == 0 && I % kFp8Group == 0, "fp8 needs H, I % 128 == 0");
    size_t o_w2, o_s13, o_s2, rec;
    record_layout(H, I, w_dtype, &o_w2, &o_s13, &o_s2, &rec);
    for (int g = 0; g < n_groups; ++g) {
        DWDP_REQUIRE(buf_of[g] >= 0 && buf_of[g] < n_buffers, "buf_of entry out of range");
        DWDP_REQUIRE(slot_of[g] >= 0, "negative slot");
        const char* base = static_cast<const char*>(buffers[buf_of[g]]);
        DWDP_REQUIRE(base != nullptr, "a buffer pointer is NULL");
        DWDP_REQUIRE(aligned16(base), "buffers must be 16-byte aligned");
        const char* r = base + (size_t)slot_of[g] * rec;
        out[g].w13 = r;
        out[g].w2 = r + o_w2;
        out[g].s13 = w_dtype == DWDP_FP8_E4M3 ? reinterpret_cast<const float*>(r + o_s13) : nullptr;
        out[g].s2 = w_dtype == DWDP_FP8_E4M3 ? reinterpret_cast<const float*>(r + o_s2) : nullptr;
    }
    return DWDP_OK;
}

int dwdp_prefetch_plan(const dwdp_copy_src* srcs, int n_src, size_t chunk_bytes, dwdp_chunk* out,
                       size_t max_chunks, size_t* n_chunks) {
    clear_error();
    int rc = check_sources(srcs, n_src, chunk_bytes);
    if (rc != DWDP_OK) return rc;
    DWDP_REQUIRE(n_chunks != nullptr, "n_chunks is NULL");
    std::vector<dwdp_chunk> plan = make_plan(srcs, n_src, chunk_bytes);
    *n_chunks = plan.size();
    if (out != nullptr) std::memcpy(out, plan.data(), std::min(max_chunks, plan.size()) * sizeof(dwdp_chunk));
    return DWDP_OK;
}

size_t dwdp_workspace_bytes(int op, int64_t T, int k, int E, int H, int I, int dtype, int shared) {
    if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1 || (shared != 0 && shared != 1)) return 0;
    if (op == DWDP_OP_PERMUTE) return permute_ws_bytes(T, k, E);
    if (op == DWDP_OP_GROUPED_FFN) {
        int64_t rows = T * k + shared * T;
        return ffn_ws_bytes(rows, E + shared, H, I, dtype);
    }
    return 0;
}

}  // extern "C"
