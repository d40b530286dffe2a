// Declarations shared between the library's translation units (not part of the ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <vector>

#include "../../include/dwdp.h"

namespace dwdp {

constexpr int kMaxCopySources = 64;

size_t elem_bytes(int dtype);
void record_layout(int H, int I, int w_dtype, size_t* w2, size_t* s13, size_t* s2, size_t* total);
std::vector<dwdp_chunk> make_plan(const dwdp_copy_src* srcs, int n_src, size_t chunk);
int check_sources(const dwdp_copy_src* srcs, int n_src, size_t chunk);

size_t permute_ws_bytes(int64_t T, int k, int E);
size_t ffn_ws_bytes(int64_t rows, int groups, int H, int I, int dtype);

}  // namespace dwdp
