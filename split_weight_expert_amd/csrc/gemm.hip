// Grouped expert GEMMs of the MoE block and the router GEMM, for gfx950.
//
// The split-weight grouped GEMM of the DWDP paper summary (§4.2) reads each
// expert's weights wherever they sit -- the resident partition or a prefetch
// slot -- through a per-group pointer table, instead of first merging the
// buffers with a device-to-device copy.  Here that table is an array of
// dwdp_expert_ptrs in device memory, read once per workgroup tile.
//
// Structure
//   * A tile schedule is built on the device from the group row offsets (no
//     host round trip): every group is cut into BM-row m-tiles, and two tables
//     list them in group order and in group-size order (schedule_kernel).
//   * Tiles reach the 8 XCDs in clusters of consecutive tiles dealt
//     round-robin (decode_tile), so tiles that share a weight or activation
//     slab run together on one XCD's L2.
//   * bf16 / fp8 (gemm_frag_kernel): weights are stored fragment-major, every
//     operand goes global -> LDS by DMA into a multi-stage ring, and the
//     MFMAs are v_mfma_f32_32x32x16_bf16 or the unscaled fp8 form of
//     v_mfma_f32_32x32x64_f8f6f4 (with a per-128-K fold of the fp32 block
//     scales).  GEMM1's
//     tile holds the gate and up rows of the same output columns, so SwiGLU
//     (and for fp8 the re-quantisation of A) happens in the epilogue.
//     GEMM1 reads its activation rows either from the permuted rows or from
//     the token rows through perm_src.
//   * f32 (small shapes only): LDS-tiled FMA kernel with the same schedule.
//   * Router (bf16): router_dma_kernel (up to 512 tiles: operands by DMA into
//     a four-slot LDS ring) or router_mfma_kernel (two-stage, register-staged).
#include <algorithm>
#include <mutex>

#include <type_traits>

#include "common.h"
#include "internal.h"

// Tile trace (a diagnostic): built with -DDWDP_TILE_TRACE=1, every workgroup of gemm_frag_kernel stores
// one dwdp_tile_record -- its tile, its XCD and the real-time counter at its start and end -- at its
// index in a fixed device array, which dwdp_diag_tile_trace_clear / _read zero and read.  The default
// build compiles none of it.
#ifndef DWDP_TILE_TRACE
#define DWDP_TILE_TRACE 0
#endif
// E8M0 block-scale code passed to the fp8 MFMA builtin.  The block scales of this path are fp32 and are
// applied in the fold, so the MFMA itself must not scale: with code 0 the compiler emits the unscaled
// v_mfma_f32_32x32x64_f8f6f4 (8 bytes shorter than the scaled form; 16K fp8 block 0.5% faster), with 127
// (2^0) the scaled form with unit scales.  Both give the same products.
#ifndef DWDP_FP8_GEMM2_BM256
#define DWDP_FP8_GEMM2_BM256 1
#endif
#ifndef DWDP_ROUTER_DMA
#define DWDP_ROUTER_DMA 1
#endif
#ifndef DWDP_MFMA_E8M0
#define DWDP_MFMA_E8M0 0
#endif

namespace dwdp {

#if DWDP_TILE_TRACE
constexpr int kTraceRecords = 1 << 17;
static __device__ dwdp_tile_record tile_trace[kTraceRecords];
#endif

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Kind { kGemm1 = 0, kGemm2 = 1, kRouter = 2 };

struct MTile {
    int32_t g;    // group
    int32_t m0;   // index of the group's first m-tile
    int32_t mc;   // the group's m-tile count
    int32_t h;    // rows per m-tile of the group (the last one may hold fewer)
};
static_assert(sizeof(MTile) == kMTileBytes, "the workspace layout sizes the m-tile tables");

struct GemmParams {
    const uint8_t* a;               // activation rows [rows, K]
    const float* a_scale;           // fp8: [a_nrows, K/128]
    const int32_t* a_rows;          // GEMM1: activation row of permuted row r (token mode), or null
    int64_t a_nrows;                // rows of a
    const dwdp_expert_ptrs* table;  // GEMM1 / GEMM2: per-group weights
    const uint8_t* b_single;        // router: weight [N, K]
    const float* bias;              // router: bias [N] or null
    const int32_t* offsets;         // [G+1]
    const int32_t* mprefix;         // [G+1]; mprefix[G] = number of m-tiles
    const MTile* mtiles;            // one entry per m-tile
    int64_t rows;                   // router: T
    int G;
    int N;                          // GEMM1: I (A columns); GEMM2: H; router: E
    int K;
    int NT;                         // n-tiles
    int msuper;                     // largest m super-block (m-tiles that run n-tile by n-tile together)
    int I;                          // GEMM1: first up row inside W13
    uint8_t* out;
    float* out_scale;               // GEMM1 fp8: A scales [rows, I/128]
    int32_t* ticket;                // expert GEMMs: tile ticket counter (tiles drawn in schedule order), or
                                    // null (tile fixed by the workgroup index, clusters dealt over the XCDs)
};

struct Tile {
    int g;
    int nt;
    int64_t row0;
    int nrows;
    int mc;       // m-tiles of the group (1: the tile is the only reader of its weight slab)
#if DWDP_TILE_TRACE
    int lin;      // position in the schedule
#endif
};

// Row of the activation matrix that holds permuted row prow: itself, or its token (clamped).
__device__ __forceinline__ int64_t act_row(const GemmParams& p, int64_t prow) {
    if (p.a_rows == nullptr) return prow;
    const int64_t r = p.a_rows[prow];
    return r < 0 ? 0 : (r >= p.a_nrows ? p.a_nrows - 1 : r);
}

// Tiles reach the XCDs in clusters: workgroup b runs on XCD b % 8, and XCD x takes clusters x, x+8,
// x+16, ... of 2^cl consecutive tiles, in order.  Consecutive tiles share operands (below), so a
// cluster's reuse stays inside one XCD's L2, while the round-robin over clusters spreads heavy and
// light groups evenly over the eight XCDs.  kCluster (32) is the largest cluster; the launch grid is a
// whole number of rounds of 8 of them.  GEMM1 deals clusters of 32 tiles, GEMM2 of 16 (its tiles are
// a quarter as long; measured 1.8% faster at 8K bf16 tokens, while GEMM1 is 1% slower with 16).
constexpr int kCluster = 32;
#ifndef DWDP_CLUSTER_GEMM1_LOG2
#define DWDP_CLUSTER_GEMM1_LOG2 5
#endif
#ifndef DWDP_CLUSTER_GEMM2_LOG2
#define DWDP_CLUSTER_GEMM2_LOG2 4
#endif
static_assert(DWDP_CLUSTER_GEMM1_LOG2 >= 0 && DWDP_CLUSTER_GEMM1_LOG2 <= 5 && DWDP_CLUSTER_GEMM2_LOG2 >= 0 &&
                  DWDP_CLUSTER_GEMM2_LOG2 <= 5, "clusters of 1 .. kCluster tiles");
// Inside a group, m-tiles are taken in super-blocks of up to p.msuper: the tiles of a super-block run
// n-tile by n-tile with the m-tiles innermost, so a window of 32 running tiles reads about msuper
// activation slabs and 32 / msuper weight slabs instead of 32 of one kind.
#ifndef DWDP_MSUPER_BF16
#define DWDP_MSUPER_BF16 4
#endif
#ifndef DWDP_MSUPER_FP8
#define DWDP_MSUPER_FP8 4
#endif
#ifndef DWDP_MSUPER_FP8_GEMM2
#define DWDP_MSUPER_FP8_GEMM2 8
#endif
#ifndef DWDP_MSUPER_BALANCED
#define DWDP_MSUPER_BALANCED 0
#endif

// Schedule position of this workgroup's tile: workgroup b runs on XCD b % 8, and XCD x takes
// clusters x, x+8, ... of 2^cl consecutive positions.
__device__ __forceinline__ int dealt_lin(int cl) {
    const int bid = blockIdx.x;
    const int slot = bid / kNumXcd;
    return (((slot >> cl) * kNumXcd + bid % kNumXcd) << cl) + (slot & ((1 << cl) - 1));
}

template <int BM, int KIND>
__device__ __forceinline__ bool decode_tile(const GemmParams& p, Tile& t, int lin) {
    int total;
    int mt_router = 0;
    if (KIND == kRouter) {
        mt_router = (int)((p.rows + BM - 1) / BM);
        total = mt_router * p.NT;
    } else {
        total = p.mprefix[p.G] * p.NT;
    }
    if (lin >= total) return false;
#if DWDP_TILE_TRACE
    t.lin = lin;
#endif
    if (KIND == kRouter) {
        const int mi = lin % mt_router;
        t.g = 0;
        t.nt = lin / mt_router;
        t.row0 = (int64_t)mi * BM;
        t.nrows = (int)min((int64_t)BM, p.rows - t.row0);
        t.mc = 1;
        return true;
    }
    const MTile m = p.mtiles[lin / p.NT];
    int rem = lin - m.m0 * p.NT;               // tile index inside the group
    int ms, mfirst;
    if (DWDP_MSUPER_BALANCED) {
        // the group's m-tiles in ceil(mc / msuper) super-blocks of nearly equal size (the first `extra`
        // ones a tile larger)
        const int nsb = (m.mc + p.msuper - 1) / p.msuper, base = m.mc / nsb, extra = m.mc % nsb;
        const int big = (base + 1) * p.NT;
        if (rem < extra * big) {
            const int sb = rem / big;
            ms = base + 1;
            mfirst = sb * (base + 1);
            rem -= sb * big;
        } else {
            const int r2 = rem - extra * big, sb = r2 / (base * p.NT);
            ms = base;
            mfirst = extra * (base + 1) + sb * base;
            rem = r2 - sb * base * p.NT;
        }
    } else {
        const int sb = rem / (p.msuper * p.NT);     // m super-block
        ms = min(p.msuper, m.mc - sb * p.msuper);
        mfirst = sb * p.msuper;
        rem -= sb * p.msuper * p.NT;
    }
    t.g = m.g;
    t.nt = rem / ms;
    const int mi = mfirst + rem % ms;
    const int r0 = p.offsets[m.g], r1 = p.offsets[m.g + 1];
    t.row0 = (int64_t)r0 + (int64_t)mi * m.h;
    t.nrows = min(m.h, r1 - (int)t.row0);
    t.mc = m.mc;
    return true;
}

template <int BM, int KIND>
__device__ __forceinline__ bool decode_tile(const GemmParams& p, Tile& t) {
    return decode_tile<BM, KIND>(p, t, dealt_lin(5));
}

// ------------------------------------------------------------------------------ schedule
// One workgroup: m-tile counts per group, their exclusive scan, and two m-tile tables over the same
// tiles: `mtiles` in group order and `mtiles_by_size` with the groups taken by row count, largest
// first (ties: lower group first; group order when G > kSortGroups).  bf16 GEMM1 walks the second:
// tiles of similar length then share clusters, run in step and reuse each other's operands in L2.
// GEMM2 was slower that way and keeps group order.
constexpr int kSortGroups = 4096;
#ifndef DWDP_SPARSE_ROWS
#define DWDP_SPARSE_ROWS 0
#endif
#ifndef DWDP_BALANCED_MTILES
#define DWDP_BALANCED_MTILES 0
#endif
// 32-row tiles draw their schedule position from a ticket counter (0: dealt over the XCDs like the rest)
#ifndef DWDP_TICKET_TILES
#define DWDP_TICKET_TILES 1
#endif

template <int BM>
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ offsets, int G,
                                                        int32_t* __restrict__ mprefix, MTile* __restrict__ mtiles,
                                                        MTile* __restrict__ mtiles_by_size,
                                                        int32_t* __restrict__ tickets) {
    if (tickets != nullptr && threadIdx.x < 2) tickets[threadIdx.x] = 0;   // both launches' ticket counters
    __shared__ int wave_sum[16];
    __shared__ int carry_s;
    __shared__ int order_s[kSortGroups];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool sorted = G <= kSortGroups;
    if (sorted && DWDP_SPARSE_ROWS == 0) {
        // every thread compares its groups with all G: the row counts are read from LDS (one broadcast
        // per h), not G times from global memory
        __shared__ int rows_s[kSortGroups];
        for (int g = tid; g < G; g += 1024) rows_s[g] = offsets[g + 1] - offsets[g];
        __syncthreads();
        for (int g = tid; g < G; g += 1024) {
            const int n = rows_s[g];
            int rank = 0;
            for (int h = 0; h < G; ++h) {
                const int m = rows_s[h];
                rank += (m > n) || (m == n && h < g);
            }
            order_s[rank] = g;
        }
    } else if (sorted) {
        // Sparse groups (1 .. DWDP_SPARSE_ROWS rows) stream their weights with little compute; spread
        // them evenly between the dense groups (each class by size, largest first), so that their weight
        // streaming runs beside the dense groups' MFMA work instead of after it.  Dense group d of D sits
        // at key 2 d S, sparse group s of S at (2 s + 1) D.
        __shared__ int crank_s[kSortGroups];
        __shared__ int nsparse_s;
        if (tid == 0) nsparse_s = 0;
        __syncthreads();
        auto is_sparse = [&](int n) { return n > 0 && n <= DWDP_SPARSE_ROWS; };
        for (int g = tid; g < G; g += 1024) {
            const int n = offsets[g + 1] - offsets[g];
            const bool sp = is_sparse(n);
            int rank = 0;
            for (int h = 0; h < G; ++h) {
                const int m = offsets[h + 1] - offsets[h];
                rank += is_sparse(m) == sp && ((m > n) || (m == n && h < g));
            }
            crank_s[g] = rank;
            if (sp) atomicAdd(&nsparse_s, 1);
        }
        __syncthreads();
        const int64_t S = nsparse_s, D = G - nsparse_s;
        // with one class empty the keys are the class ranks themselves
        auto key_of = [&](int r, bool sp) -> int64_t {
            if (S == 0 || D == 0) return r;
            return sp ? (2 * (int64_t)r + 1) * D : 2 * (int64_t)r * S;
        };
        for (int g = tid; g < G; g += 1024) {
            const bool sp = is_sparse(offsets[g + 1] - offsets[g]);
            const int64_t key = key_of(crank_s[g], sp);
            int rank = 0;
            for (int h = 0; h < G; ++h) {
                const bool hs = is_sparse(offsets[h + 1] - offsets[h]);
                const int64_t kh = key_of(crank_s[h], hs);
                rank += kh < key || (kh == key && !hs && sp);
            }
            order_s[rank] = g;
        }
    }
    for (int pass = 0; pass < 2; ++pass) {
    MTile* table = pass == 0 ? mtiles : mtiles_by_size;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < G; base += 1024) {
        const int g = (pass == 1 && sorted && base + tid < G) ? order_s[base + tid] : base + tid;
        int c = 0;
        if (g < G) {
            const int n = offsets[g + 1] - offsets[g];
            c = n > 0 ? (n + BM - 1) / BM : 0;
        }
        int incl = c;
        for (int d = 1; d < 64; d <<= 1) {
            int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        if (lane == 63) wave_sum[wave] = incl;
        __syncthreads();
        int before = carry_s;
        for (int w = 0; w < wave; ++w) before += wave_sum[w];
        const int excl = before + incl - c;
        if (g < G) {
            if (pass == 0) mprefix[g] = excl;
            // m-tile height: BM, or with DWDP_BALANCED_MTILES the group's rows split evenly over its c
            // m-tiles (in whole 32-row blocks), so that its tiles take about the same time
            int h = BM;
            if (DWDP_BALANCED_MTILES && c > 1) {
                const int n = offsets[g + 1] - offsets[g];
                h = ((n + c - 1) / c + 31) / 32 * 32;
            }
            for (int m = 0; m < c; ++m) table[excl + m] = MTile{g, excl, c, h};
        }
        __syncthreads();
        if (tid == 0) {
            int s = 0;
            for (int w = 0; w < 16; ++w) s += wave_sum[w];
            carry_s += s;
        }
        __syncthreads();
    }
    if (pass == 0 && tid == 0) mprefix[G] = carry_s;
    }
}

// SwiGLU of one gate / up pair, silu(g) * u = g / (1 + e^-g) * u, with the hardware reciprocal (1 ulp)
// in place of the correctly rounded division (about ten instructions): the epilogue runs on VALU while
// the compute unit's matrix cores idle, and this one cut GEMM1 by 0.5-1% (DWDP_SILU_RCP=0 restores it).
#ifndef DWDP_SILU_RCP
#define DWDP_SILU_RCP 1
#endif
__device__ __forceinline__ float silu_mul(float g, float u) {
#if DWDP_SILU_RCP
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
#else
    return g / (1.0f + __expf(-g)) * u;
#endif
}

// ------------------------------------------------------------------------------ router kernel
// logits [T, E] = x [T, H] * w_router[E, H]^T + bias, bf16 inputs and fp32 accumulation.  BM x BN tile,
// WM x WN waves, 128 bytes (64 bf16) of K per step through a two-stage register-staged LDS buffer; rows
// of both operands are swizzled in LDS (chunk c of row r at c ^ (r & 7)).
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void router_mfma_kernel(GemmParams p) {
    constexpr int NTHR = WM * WN * 64;
    constexpr int ROWB = 128, KSTEP = 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MI = TM / 32, NJ = TN / 32;
    constexpr int AC = BM * 8 / NTHR, BC = BN * 8 / NTHR;
    static_assert(AC >= 1 && BC >= 1 && BM * 8 % NTHR == 0 && BN * 8 % NTHR == 0, "tile / thread mismatch");

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * ROWB];

    Tile t;
    if (!decode_tile<BM, kRouter>(p, t)) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, hi = lane >> 5;
    const size_t ldk = (size_t)p.K * 2;
    const int KT = p.K / KSTEP;

    const uint8_t* ga[AC];
    int la[AC];
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int lin = tid + i * NTHR, r = lin >> 3, c = lin & 7;
        const int rr = min(r, t.nrows - 1);
        ga[i] = p.a + (size_t)(t.row0 + rr) * ldk + c * 16;
        la[i] = r * ROWB + ((c ^ (r & 7)) << 4);
    }
    const uint8_t* gb[BC];
    int lb[BC];
#pragma unroll
    for (int i = 0; i < BC; ++i) {
        const int lin = tid + i * NTHR, r = lin >> 3, c = lin & 7;
        gb[i] = p.b_single + (size_t)min(t.nt * BN + r, p.N - 1) * ldk + c * 16;
        lb[i] = r * ROWB + ((c ^ (r & 7)) << 4);
    }

    bool m_act[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) m_act[i] = wm * TM + i * 32 < t.nrows;

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    u32x4 ra[AC], rb[BC];
    auto gload = [&](int kt) {
        const size_t off = (size_t)kt * ROWB;
#pragma unroll
        for (int i = 0; i < AC; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ga[i] + off);
#pragma unroll
        for (int i = 0; i < BC; ++i) rb[i] = *reinterpret_cast<const u32x4*>(gb[i] + off);
    };
    auto sstore = [&](int st) {
#pragma unroll
        for (int i = 0; i < AC; ++i) *reinterpret_cast<u32x4*>(&sA[st][la[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < BC; ++i) *reinterpret_cast<u32x4*>(&sB[st][lb[i]]) = rb[i];
    };
    auto lds16 = [&](const uint8_t* s, int row, int chunk) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(&s[row * ROWB + ((chunk ^ (row & 7)) << 4)]);
    };
    auto row_of = [&](int i, int r) -> int { return wm * TM + i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3); };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const uint8_t* A = sA[cur];
        const uint8_t* B = sB[cur];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ch = s * 2 + hi;
            bf16x8 af[MI], bf[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) af[i] = __builtin_bit_cast(bf16x8, lds16(A, wm * TM + i * 32 + l32, ch));
#pragma unroll
            for (int j = 0; j < NJ; ++j) bf[j] = __builtin_bit_cast(bf16x8, lds16(B, wn * TN + j * 32 + l32, ch));
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (!m_act[i]) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < KT) sstore(cur ^ 1);
        __syncthreads();
    }

    float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int col = t.nt * BN + wn * TN + j * 32 + l32;
        if (col >= p.N) continue;
        const float b = p.bias ? p.bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = row_of(i, r);
                if (m < t.nrows) out[(size_t)(t.row0 + m) * p.N + col] = acc[i][j][r] + b;
            }
    }
}

// ------------------------------------------------------------------------------ fragment kernel
// The expert GEMMs.  One workgroup per CU computes a BM x 256 tile of one group.  The 256 output
// columns are four column groups of 64 (two 32-wide n-blocks each); each column group is one wave
// holding all BM rows (bf16), or two waves holding 64 rows each (fp8 at BM = 128).  A short tail tile
// runs a variant that touches only its active 32-row m-blocks.
//   * Weights are stored fragment-major (dwdp_pack_weights): the 32 x 16 bf16 (or 32 x 64 fp8)
//     operand of one MFMA is 1 KB (2 KB) of contiguous memory in lane order.
//   * Every operand goes from global memory straight into an NS-stage LDS ring with
//     global_load_lds_dwordx4 (no register staging): per K step the stage holds ROWB bytes of each
//     active row, the weight fragments of all four column groups and, for fp8, the row scales.
//     Each wave issues its own share and waits only for its own oldest batch (vmcnt; vector loads
//     complete in order); one barrier per step orders the ring.
//   * bf16 keeps P = NS - 2 steps in flight and issues the next batch before the step's closing LDS
//     wait; its LDS reads are interleaved one by one with the MFMAs.  fp8 keeps P = NS - 1.
//   * Activation rows are swizzled in LDS (aslot) so that the 16 lanes one ds_read_b128 cycle
//     serves hit 16 distinct 16-byte slots of the 256-byte bank window.
//   * Cache policy of the operand loads (compile-time options, 0 = default): DWDP_WEIGHT_CPOL for the
//     weight fragments and DWDP_ACT_CPOL for the activation rows, as the instruction's cache-policy
//     bits (2 = non-temporal: the lines are streamed, not kept for reuse).
#ifndef DWDP_WEIGHT_CPOL
#define DWDP_WEIGHT_CPOL 0
#endif
#ifndef DWDP_ACT_CPOL
#define DWDP_ACT_CPOL 0
#endif
// Weight loads of a tile whose group has a single m-tile are the only reads of those lines: they use
// DWDP_STREAM_WEIGHT_CPOL (default 2, non-temporal), which streams HBM about 13% faster than the default
// policy with this kernel's loads (7.0 against 6.2 TB/s).  Slabs that several m-tiles share keep
// DWDP_WEIGHT_CPOL, so that the tiles after the first find them in L2.
// GEMM2 writes y_perm with non-temporal stores (DWDP_YPERM_NT, default 1): the combine reads it once.
#ifndef DWDP_YPERM_NT
#define DWDP_YPERM_NT 1
#endif
#ifndef DWDP_STREAM_WEIGHT_CPOL
#define DWDP_STREAM_WEIGHT_CPOL 2
#endif
constexpr int kStreamWeightCpol = DWDP_STREAM_WEIGHT_CPOL;
template <int CPOL = 0>
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, CPOL);
#endif
}

__device__ __forceinline__ void dma4(const uint8_t* g, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
#endif
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void ordered_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Everything a tile needs once it is decoded.
struct TileCtx {
    Tile t;
    int KT;                 // K steps
    const uint8_t* wb[2];   // this wave's two n-block fragment streams (+ lane * 16)
    int nblk[2];
    const float* wscale;
};

// ROWB: bytes of one activation row per K step (64 or 128).  Weight fragments are 1 KB per 16 bf16
// (or per 64 fp8 / 2 halves) K columns, so a step moves ROWB / 32 fragment-KB per n-block.
//
// Waves: four column groups of 64 output columns each.  Tiles up to 128 rows (bf16) have one wave
// per column group holding all BM rows.  bf16 tiles of 256 rows and fp8 tiles of 128 rows have two
// waves per column group, one per half of the rows (two waves per SIMD): the SIMD switches to the
// other wave while one waits on LDS or the barrier, and for fp8 one wave's fp32 scale fold runs
// while the other's MFMAs do.
// 256-row fp8 tiles (compile-time option DWDP_FP8_BM256) take 64-byte K steps: a 128-byte step of 256
// rows leaves room for only two ring slots
constexpr int rowb_of(int BM, bool FP8) { return FP8 ? (BM >= 256 ? 64 : 128) : (BM == 32 ? 128 : 64); }

template <int BM, int ROWB, bool FP8>
struct FragCfg {
    static constexpr int NW = (FP8 ? BM >= 128 : BM >= 256) ? 8 : 4;   // waves
    static constexpr int RH = NW / 4;                         // row parts (waves per column group)
    static constexpr int MI = BM / 32, MIW = MI / RH, NJ = 2; // m-blocks per tile / per wave
    static constexpr int CH = ROWB / 16;                      // 16-byte chunks per activation row
    static constexpr int BF = ROWB / 32;                      // weight KB per n-block per step
    static constexpr int RPI = 1024 / ROWB;                   // activation rows per DMA instruction
    static constexpr int BI = NJ * BF;                        // weight KB per column group per step
    static constexpr int BIW = BI / RH;                       // weight DMA instructions per wave per step
    static constexpr int ABYTES = BM * ROWB;
    static constexpr int BBYTES = 4 * BI * 1024;
    // fp8: a step's slot also holds the row scales of its K block.  Each wave loads those of RW rows
    // with one 64-lane DMA instruction into a 64-float slice of its own (lanes past RW repeat the
    // last row), so row R's scale sits at float (R / RW) * SSTRIDE + R % RW.  Slices are SSTRIDE = 80
    // floats apart: the 32 rows one read serves span two slices, and the 16-float shift puts them
    // on different LDS banks (at 64 floats apart the two halves collide).
    static constexpr int RW = BM / NW;
    static constexpr int SSTRIDE = 80;                        // floats between waves' scale slices
    static constexpr int STAGE = ABYTES + BBYTES + (FP8 ? NW * SSTRIDE * 4 : 0);
    // fp8, outside the ring: the weight block scales of each wave's n-blocks (K / 128 <= 64), read
    // once per tile
    static constexpr int BSC = FP8 ? NW * NJ * 64 : 0;        // floats
    static constexpr int EXTRA = BSC * 4;
    static constexpr int FIT = (163840 - EXTRA) / STAGE;
    static constexpr int NS = FIT < 8 ? FIT : 8;              // ring slots
    // bf16 reuses a slot one step after its last read (P = NS - 2), so the DMA can be issued before
    // the step's closing LDS wait; fp8 reuses it right after the barrier (P = NS - 1)
    static constexpr int P = FP8 ? NS - 1 : NS - 2;           // steps in flight ahead of the MFMAs
    static_assert(BM % 32 == 0 && (ROWB == 64 || ROWB == 128), "tile shape");
    static_assert(P >= 1, "ring too shallow");
    static_assert(BI % RH == 0 && MI % RH == 0, "waves split the tile evenly");
};

// activation rows a tile with MA active m-blocks loads (a whole number of DMA instructions per wave)
template <int ROWB, int MA, int NW>
constexpr int loaded_rows() {
    constexpr int unit = NW * (1024 / ROWB);
    return ((MA * 32 + unit - 1) / unit) * unit;
}

// Chunk c of activation row r is stored at slot c ^ f(r) so that ds_read_b128 of 16 consecutive rows
// (the 16 lanes one LDS cycle serves) hits 16 distinct 16-byte slots of the 256-byte bank window.
template <int ROWB>
__device__ __forceinline__ int aslot(int row, int chunk) {
    return ROWB == 128 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 2) & 3);
}

// Router (bf16) with its operands moved by DMA: the router_mfma_kernel tile (64 x 64, 4 waves of 32 x 32,
// K steps of 64 columns) with global_load_lds into an NS-slot LDS ring and P = NS - 1 steps in flight,
// so a workgroup keeps three 16 KB steps of loads outstanding without staging them in registers.  Wave w
// fills the 1 KB blocks 2w and 2w+1 of the step's A rows and of its B rows: lane l of block b carries
// row 8b + l/8 into LDS slot l % 8, which holds that row's 16-byte chunk aslot(row, l % 8).  Slot
// (kt + P) % NS is the one step kt - 1 read, so step kt + P is issued after step kt's barrier.
template <int NS>
__global__ __launch_bounds__(256) void router_dma_kernel(GemmParams p) {
    constexpr int BM = 64, BN = 64, ROWB = 128, ABYTES = BM * ROWB, STAGE = (BM + BN) * ROWB;
    constexpr int P = NS - 1;
    static_assert(NS >= 2 && NS <= 4, "ring depth (the waits below cover up to 3 steps in flight)");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * STAGE];

    Tile t;
    if (!decode_tile<BM, kRouter>(p, t)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, hi = lane >> 5;
    const size_t ldk = (size_t)p.K * 2;
    const int KT = p.K / 64;

    const uint8_t* ga[2];
    const uint8_t* gb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = (2 * wave + q) * 8 + lane / 8;
        const int c = aslot<ROWB>(r, lane & 7);
        ga[q] = p.a + (size_t)(t.row0 + min(r, t.nrows - 1)) * ldk + c * 16;
        gb[q] = p.b_single + (size_t)min(t.nt * BN + r, p.N - 1) * ldk + c * 16;
    }
    auto issue = [&](int kt) {
        uint8_t* st = ring + (kt % NS) * STAGE;
        const size_t off = (size_t)kt * ROWB;
#pragma unroll
        for (int q = 0; q < 2; ++q) dma16(ga[q] + off, st + (2 * wave + q) * 1024);
#pragma unroll
        for (int q = 0; q < 2; ++q) dma16(gb[q] + off, st + ABYTES + (2 * wave + q) * 1024);
    };
    auto frag = [&](const uint8_t* S, int row, int chunk) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(S + row * ROWB + (aslot<ROWB>(row, chunk) << 4)));
    };

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const bool active = wm * 32 < t.nrows;
    for (int k = 0; k < P && k < KT; ++k) issue(k);
    for (int kt = 0; kt < KT; ++kt) {
        // this wave's DMAs of step kt have landed once at most those of the later issued steps are out
        const int later = min(P - 1, KT - 1 - kt);
        if (later >= 2) wait_vmcnt<8>();
        else if (later == 1) wait_vmcnt<4>();
        else wait_vmcnt<0>();
        ordered_barrier();                     // every wave's step kt landed; step kt-1's slot is free
        if (kt + P < KT) issue(kt + P);
        const uint8_t* A = ring + (kt % NS) * STAGE;
        const uint8_t* B = A + ABYTES;
        if (active) {
            bf16x8 af[4], bf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                af[s] = frag(A, wm * 32 + l32, 2 * s + hi);
                bf[s] = frag(B, wn * 32 + l32, 2 * s + hi);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], bf[s], acc, 0, 0, 0);
        }
        // the fragments are in registers before any wave passes the next barrier
        __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0), vmcnt and expcnt not waited on
    }

    float* out = reinterpret_cast<float*>(p.out);
    const int col = t.nt * BN + wn * 32 + l32;
    if (col < p.N) {
        const float b = p.bias ? p.bias[col] : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = wm * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            if (m < t.nrows) out[(size_t)(t.row0 + m) * p.N + col] = acc[r] + b;
        }
    }
}

// Main loop and epilogue of one tile with MA active 32-row m-blocks, of which this wave multiplies
// MWV (compile-time: the loop body is straight-line code; only the LDS ring is waited on, and only
// here, with vmcnt).  Every wave loads its share of the MA blocks' rows whatever its MWV, and a wave
// with MWV == 0 only loads and keeps the barriers.
template <int BM, int ROWB, int MA, int MWV, int KIND, bool FP8, int WPOL>
__device__ __forceinline__ void frag_tile(const GemmParams& p, const TileCtx& c, uint8_t* smem,
                                          const float* s_bscale) {
    using C = FragCfg<BM, ROWB, FP8>;
    constexpr int NS = C::NS, P = C::P, NJ = C::NJ, CH = C::CH, BF = C::BF, STAGE = C::STAGE;
    constexpr int BI = C::BI, BIW = C::BIW, ABYTES = C::ABYTES, BBYTES = C::BBYTES;
    constexpr int RPI = C::RPI, NW = C::NW, MIW = C::MIW;
    // only the rows of the MA active m-blocks are loaded: each wave DMAs an equal share of them
    constexpr int AI = loaded_rows<ROWB, MA, NW>() / NW / RPI;
    constexpr int AS = FP8 ? 1 : 0;                    // row-scale DMA instructions per step
    constexpr int PER = AI + BIW + AS;
    constexpr bool active = MWV > 0;
    constexpr int MW = active ? MWV : 1;               // accumulator blocks (one unused when idle)
    static_assert(AI >= 1 && loaded_rows<ROWB, MA, NW>() <= BM, "activation rows must split evenly over the waves");
    static_assert(MWV >= 0 && MWV <= MIW, "a wave holds at most its part's m-blocks");
    static_assert(PER * P < 64, "vmcnt budget");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = wave & 3, rh = C::RH == 1 ? 0 : wave >> 2;   // column group, row part
    const int rbase = rh * MIW * 32;                   // first tile row of this wave's part
    const int l32 = lane & 31, hi = lane >> 5;
    const Tile& t = c.t;
    const int KT = c.KT;
    const size_t lda = (size_t)p.K * (FP8 ? 1 : 2);

    // fp8: this wave's RW rows of the step's row scales (lanes RW.. idle)
    [[maybe_unused]] const float* gs = nullptr;
    if constexpr (FP8)
        gs = p.a_scale + (size_t)act_row(p, t.row0 + min(wave * C::RW + min(lane, C::RW - 1), t.nrows - 1)) * (p.K / kFp8Group);
    const uint8_t* ga[AI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int r = (wave * AI + i) * RPI + lane / CH;
        ga[i] = p.a + (size_t)act_row(p, t.row0 + min(r, t.nrows - 1)) * lda + aslot<ROWB>(r, lane % CH) * 16;
    }
    // this wave's share of its column group's weight fragments: BIW of the group's NJ * BF per step
    const uint8_t* gb[BIW];
    int lb[BIW];
#pragma unroll
    for (int q = 0; q < BIW; ++q) {
        const int idx = rh * BIW + q;                  // = j * BF + v
        gb[q] = (idx < BF ? c.wb[0] : c.wb[1]) + (idx % BF) * 1024;
        lb[q] = ABYTES + (cg * BI + idx) * 1024;
    }

    f32x16 acc[MW][NJ];
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    [[maybe_unused]] auto scale_dma = [&](int kt, uint8_t* st) {
        dma4(reinterpret_cast<const uint8_t*>(gs + kt * ROWB / kFp8Group), st + ABYTES + BBYTES + wave * C::SSTRIDE * 4);
    };
    auto issue = [&](int kt, int buf) {
        uint8_t* st = smem + buf * STAGE;
#pragma unroll
        for (int i = 0; i < AI; ++i) dma16<DWDP_ACT_CPOL>(ga[i] + (size_t)kt * ROWB, st + (wave * AI + i) * 1024);
#pragma unroll
        for (int q = 0; q < BIW; ++q) dma16<WPOL>(gb[q] + (size_t)kt * BF * 1024, st + lb[q]);
        if constexpr (FP8) scale_dma(kt, st);
    };
    // DMA instructions q0 .. q1-1 of a step's PER (activation rows, weight fragments, row scales)
    auto issue_part = [&](int kt, int buf, int q0, int q1) {
        uint8_t* st = smem + buf * STAGE;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (q < q0 || q >= q1) continue;
            if (q < AI) dma16<DWDP_ACT_CPOL>(ga[q] + (size_t)kt * ROWB, st + (wave * AI + q) * 1024);
            else if (q < AI + BIW) dma16<WPOL>(gb[q - AI] + (size_t)kt * BF * 1024, st + lb[q - AI]);
            else if constexpr (FP8) scale_dma(kt, st);
        }
    };
    auto a_frag = [&](const uint8_t* A, int i, int chunk) -> u32x4 {
        const int row = rbase + i * 32 + l32;
        return *reinterpret_cast<const u32x4*>(A + row * ROWB + (aslot<ROWB>(row, chunk) << 4));
    };
    auto b_frag = [&](const uint8_t* B, int j, int v) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(B + (cg * BI + j * BF + v) * 1024 + lane * 16);
    };
    // fp8 step: per m-block, the two 64-wide halves of the 128-wide K block go through the unscaled
    // fp8 MFMA into a fresh partial sum, which is folded into the accumulator with the row scale
    // times the weight block's scale.
    // fp8 step kt; the DMA of step ikt into slot ibuf (when iss) is spread over its MFMA blocks, so a
    // wave never waits for the memory pipe to accept its whole batch before its first MFMA
    // fp8 with 64-byte K steps (256-row tiles): the accumulator is kept in units of the current K block's
    // scale product c = (row scale) * (weight block scale), so the MFMAs accumulate straight into it.  At
    // the first half of each 128-wide K block it is multiplied by c_previous / c_current, and after the
    // last block by c_last: the sum of c_kb * P_kb without a separate partial sum per block.
    [[maybe_unused]] float cprev[MW][NJ];
    if constexpr (FP8 && ROWB == 64) {
#pragma unroll
        for (int i = 0; i < MW; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) cprev[i][j] = 1.0f;
    }
    auto compute = [&](int kt, int buf, int ikt, int ibuf, bool iss) {
        const uint8_t* A = smem + buf * STAGE;
        const uint8_t* B = A + ABYTES;
        if constexpr (FP8 && ROWB == 64) {
            if (!active) {
                if (iss) issue(ikt, ibuf);
                return;
            }
            const bool first = (kt & 1) == 0;              // first 64-wide half of a 128-wide K block
            i32x8 bf[NJ], af[MW];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const u32x4 b0 = b_frag(B, j, 0), b1 = b_frag(B, j, 1);
                bf[j] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                              (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
            }
#pragma unroll
            for (int i = 0; i < MW; ++i) {
                const u32x4 lo = a_frag(A, i, hi * 2), up = a_frag(A, i, hi * 2 + 1);
                af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2],
                              (int)up[3]};
            }
            float rs[MW][NJ];
            if (first) {
                const float* sa_lds = reinterpret_cast<const float*>(B + BBYTES);
                const int kb = kt / 2;
#pragma unroll
                for (int i = 0; i < MW; ++i) {
                    const int R = rbase + i * 32 + l32;
                    const float sa = sa_lds[(R / C::RW) * C::SSTRIDE + R % C::RW];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const float c = sa * s_bscale[(wave * NJ + j) * 64 + kb];
                        rs[i][j] = cprev[i][j] * __builtin_amdgcn_rcpf(c);     // c > 0: scales are amax/448 or 1
                        cprev[i][j] = c;
                    }
                }
            }
            constexpr int NB = MW * NJ, QB = (PER + NB - 1) / NB;   // DMA instructions per block
            auto rescale = [&](int b) {
                const int i = b / NJ, j = b % NJ;
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] *= rs[i][j];
            };
            auto mfma = [&](int b) {
                const int i = b / NJ, j = b % NJ;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af[i], acc[i][j], 0, 0, 0,
                                                                            DWDP_MFMA_E8M0, 0, DWDP_MFMA_E8M0);
            };
            if (first) {
                // block b's rescale runs under block b-1's MFMA
                rescale(0);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    mfma(b);
                    if (iss) issue_part(ikt, ibuf, b * QB, (b + 1) * QB);
                    if (b + 1 < NB) rescale(b + 1);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // block b's MFMA
                    __builtin_amdgcn_sched_group_barrier(0x020, QB, 0);   // part of the next DMA batch
                    if (b + 1 < NB) __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);   // block b+1's rescale
                }
            } else {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    mfma(b);
                    if (iss) issue_part(ikt, ibuf, b * QB, (b + 1) * QB);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, QB, 0);
                }
            }
        } else if constexpr (FP8) {
            if (!active) {
                if (iss) issue(ikt, ibuf);
                return;
            }
            const float* sa_lds = reinterpret_cast<const float*>(B + BBYTES);   // this K block's row scales
            float sb[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) sb[j] = s_bscale[(wave * NJ + j) * 64 + kt * ROWB / kFp8Group];
            constexpr int SH = ROWB / 64;                  // 64-wide K halves per step
            i32x8 bf[NJ][SH];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int s = 0; s < SH; ++s) {
                    const u32x4 b0 = b_frag(B, j, 2 * s), b1 = b_frag(B, j, 2 * s + 1);
                    bf[j][s] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                                     (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
                }
            // fp8 blocks are computed transposed (weights as the MFMA's first operand): a lane then
            // holds one row (token) of the block and 16 of its columns, all inside one 32-row weight
            // n-block, so the fold's scale is a single product per lane and block.
            i32x8 af[MW][SH];
            float sa[MW];
#pragma unroll
            for (int i = 0; i < MW; ++i) {
#pragma unroll
                for (int s = 0; s < SH; ++s) {
                    const u32x4 lo = a_frag(A, i, s * 4 + hi * 2), up = a_frag(A, i, s * 4 + hi * 2 + 1);
                    af[i][s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1],
                                     (int)up[2], (int)up[3]};
                }
                const int R = rbase + i * 32 + l32;
                sa[i] = sa_lds[(R / C::RW) * C::SSTRIDE + R % C::RW];
            }
            // The fold of an output block needs its MFMAs' result, so block b's fold is issued after
            // block b+1's MFMAs: the VALU folds while the matrix core multiplies.
            f32x16 part[2];
            auto fold = [&](int b) {
                const int i = b / NJ, j = b % NJ;
                const float c = sa[i] * sb[j];
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] += part[b & 1][r] * c;
            };
            auto mfma = [&](int b) {
                const int i = b / NJ, j = b % NJ;
#pragma unroll
                for (int r = 0; r < 16; ++r) part[b & 1][r] = 0.0f;
#pragma unroll
                for (int s = 0; s < SH; ++s)
                    part[b & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j][s], af[i][s], part[b & 1], 0, 0,
                                                                                  0, DWDP_MFMA_E8M0, 0,
                                                                                  DWDP_MFMA_E8M0);
            };
            constexpr int NB = MW * NJ, QB = (PER + NB - 1) / NB;   // DMA instructions per block
            constexpr int NF = 17;                                  // VALU per fold
            mfma(0);
            if (iss) issue_part(ikt, ibuf, 0, QB);
            __builtin_amdgcn_sched_group_barrier(0x008, SH, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, QB, 0);
#pragma unroll
            for (int b = 1; b < NB; ++b) {
                mfma(b);
                if (iss) issue_part(ikt, ibuf, b * QB, (b + 1) * QB);
                fold(b - 1);
                __builtin_amdgcn_sched_group_barrier(0x008, SH, 0);   // block b's MFMAs
                __builtin_amdgcn_sched_group_barrier(0x020, QB, 0);   // part of the next DMA batch
                __builtin_amdgcn_sched_group_barrier(0x002, NF, 0);   // block b-1's fold
            }
            fold(NB - 1);
        }
    };

    if constexpr (!FP8) {
        // bf16: fragments of the next sub-step are read from LDS while the MFMAs of the current one
        // run; the last sub-step of a step first crosses the barrier into the next step's slot.
        constexpr int S = ROWB / 32;
        struct Frags {
            bf16x8 a[MW];
            bf16x8 b[NJ];
        };
        Frags F[2];
        auto load = [&](Frags& f, int buf, int sub) {
            if (!active) return;
            const uint8_t* A = smem + buf * STAGE;
            const uint8_t* B = A + ABYTES;
#pragma unroll
            for (int j = 0; j < NJ; ++j) f.b[j] = __builtin_bit_cast(bf16x8, b_frag(B, j, sub));
#pragma unroll
            for (int i = 0; i < MW; ++i) f.a[i] = __builtin_bit_cast(bf16x8, a_frag(A, i, sub * 2 + hi));
        };
        auto mma = [&](const Frags& f) {
            if (!active) return;
#pragma unroll
            for (int i = 0; i < MW; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
        };
        // End of step kt (ring slot u) into step kt + 1.  Batch kt + 1 + P goes to the slot of step
        // kt - 1, which every wave stopped reading before the previous barrier; issuing it here, just
        // before the LDS wait, keeps the compiler's ds_read counting exact after the barrier.
        auto cross = [&](int kt, int u, bool steady) {
            __builtin_amdgcn_sched_barrier(0);   // keep the DMA (it rewrites M0) out of the MFMA region
            __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
            // batch kt + 1 must have landed: the batches after it are kt+2 .. min(KT-1, kt+1+P)
            if (steady) {
                wait_vmcnt<P * PER>();
            } else {
                const int after = min(KT - 2 - kt, P);
                if (after >= P) wait_vmcnt<P * PER>();
                else if (P >= 2 && after == P - 1) wait_vmcnt<(P >= 2 ? P - 1 : 0) * PER>();
                else if (P >= 3 && after == P - 2) wait_vmcnt<(P >= 3 ? P - 2 : 0) * PER>();
                else wait_vmcnt<0>();
            }
            ordered_barrier();
            load(F[0], (u + 1) % NS, 0);
        };
        // Interleave the next fragments' ds_reads one by one between this sub-step's MFMAs: the LDS
        // counter is 4 bits, so a batch of reads issued ahead of still-pending ones would force a
        // full drain (lgkmcnt(0)) before the first MFMA.
        constexpr int NL = MW + NJ, NM = MW * NJ, PERL = (NM + NL - 1) / NL;
        auto interleave = [&]() {
#pragma unroll
            for (int q = 0; q < NL; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, PERL, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
            }
        };
        // with the DMA of batch kt + 1 + P spread over the first sub-step's MFMAs
        auto interleave_dma = [&]() {
#pragma unroll
            for (int q = 0; q < NL; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, PERL, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
                if (q < PER) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // DMA
            }
        };
        auto step = [&](int kt, int u, bool steady) {
#pragma unroll
            for (int sub = 0; sub < S; ++sub) {
                if (sub + 1 < S) load(F[(sub + 1) & 1], u, sub + 1);
                else if (steady || kt + 1 < KT) cross(kt, u, steady);
                const bool dma = sub == 0 && (steady || kt + 1 + P < KT);
                if (dma) issue(kt + 1 + P, (u + 1 + P) % NS);
                mma(F[sub & 1]);
                if (sub == 0) interleave_dma();
                else interleave();
            }
        };
        // prologue: batches 0 .. P into slots 0 .. P
#pragma unroll
        for (int u = 0; u <= P; ++u)
            if (u < KT) issue(u, u);
        if (KT > P) wait_vmcnt<P * PER>();               // batch 0 landed (1 .. P may be in flight)
        else wait_vmcnt<0>();
        ordered_barrier();
        load(F[0], 0, 0);
        int k0 = 0;
        for (; k0 + NS + P < KT; k0 += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u) step(k0 + u, u, true);
        }
#pragma unroll
        for (int u = 0; u < NS + P; ++u)
            if (k0 + u < KT) step(k0 + u, u % NS, false);
    } else {
        // prologue: batches 0 .. P-1
#pragma unroll
        for (int u = 0; u < P; ++u)
            if (u < KT) issue(u, u);
        // steady state: every step of the group can issue step + P
        int k0 = 0;
        for (; k0 + NS + P - 1 < KT; k0 += NS) {
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                wait_vmcnt<(P - 1) * PER>();
                ordered_barrier();
                compute(k0 + u, u, k0 + u + P, (u + P) % NS, true);
            }
        }
        // drain: at most NS + P - 1 steps, exact waits
#pragma unroll
        for (int u = 0; u < NS + P - 1; ++u) {
            const int kt = k0 + u;
            if (kt < KT) {
                if constexpr (P >= 2) {
                    if (kt + P - 1 < KT) wait_vmcnt<(P - 1) * PER>();
                    else if (kt + P - 2 < KT) wait_vmcnt<((P >= 3 ? P - 2 : 0)) * PER>();
                    else wait_vmcnt<0>();
                } else {
                    wait_vmcnt<0>();
                }
                ordered_barrier();
                compute(kt, u % NS, kt + P, (u + P) % NS, kt + P < KT);
            }
        }
    }

    // ---------------------------------------------------------------- epilogue
    if constexpr (FP8 && ROWB == 64) {
        if (active) {
#pragma unroll
            for (int i = 0; i < MW; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] *= cprev[i][j];
        }
    }
    if constexpr (KIND == kGemm1) {
        if constexpr (!FP8) {
            // Blocks are transposed (lane l32 holds row rbase + 32 i + l32, element r holds A column
            // cg * 32 + (r >> 2) * 8 + hi * 4 + (r & 3)): A's bf16 rows go through LDS and leave in
            // 16-byte pieces.
            ordered_barrier();                                   // every wave is done with the ring
            uint8_t* stg = smem;                                 // [BM][256 B], chunks c at c ^ (row & 15)
            if (active) {
#pragma unroll
                for (int i = 0; i < MW; ++i) {
                    const int m = rbase + i * 32 + l32;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint32_t w[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            w[h] = bf16x2(silu_mul(acc[i][0][4 * q + 2 * h], acc[i][1][4 * q + 2 * h]),
                                          silu_mul(acc[i][0][4 * q + 2 * h + 1], acc[i][1][4 * q + 2 * h + 1]));
                        const int byte = (cg * 32 + q * 8 + hi * 4) * 2;
                        uint32_t* d = reinterpret_cast<uint32_t*>(stg + m * 256 + (((byte >> 4) ^ (m & 15)) << 4) + (byte & 15));
                        d[0] = w[0];
                        d[1] = w[1];
                    }
                }
            }
            __syncthreads();
            uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
            for (int q = threadIdx.x; q < BM * 16; q += NW * 64) {
                const int row = q >> 4, c = q & 15;
                if (row < t.nrows)
                    *reinterpret_cast<u32x4*>(out + (size_t)(t.row0 + row) * p.N + t.nt * 128 + c * 8) =
                        *reinterpret_cast<const u32x4*>(stg + row * 256 + ((c ^ (row & 15)) << 4));
            }
        } else {
            // Blocks are transposed: lane l32 holds row rbase + 32 i + l32 and element r holds A column
            // cg * 32 + (r >> 2) * 8 + hi * 4 + (r & 3).  The tile's 128 A columns are exactly one
            // quantisation group: the row's amax over its 4 column groups meets in LDS, then the codes
            // go through LDS so that every row leaves as 128 contiguous bytes.
            ordered_barrier();                                   // every wave is done with the ring
            float* red = reinterpret_cast<float*>(smem);         // [4][BM]
            uint8_t* codes = smem + 4 * BM * 4;                  // [BM][128], 16-byte chunks c at c ^ (row & 7)
            float av[MW][16];
            if (active) {
#pragma unroll
                for (int i = 0; i < MW; ++i) {
                    float m = 0.0f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        av[i][r] = silu_mul(acc[i][0][r], acc[i][1][r]);
                        m = fmaxf(m, fabsf(av[i][r]));
                    }
                    m = fmaxf(m, __shfl_xor(m, 32));
                    if (hi == 0) red[cg * BM + rbase + i * 32 + l32] = m;
                }
            }
            __syncthreads();
            if (active) {
                const int IB = p.N / kFp8Group;
#pragma unroll
                for (int i = 0; i < MW; ++i) {
                    const int m = rbase + i * 32 + l32;
                    const float amax = fmaxf(fmaxf(red[m], red[BM + m]), fmaxf(red[2 * BM + m], red[3 * BM + m]));
                    const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
                    // A / scale as A * (1 / scale): one division a row instead of one a value (16K fp8
                    // GEMM1 1.2% faster).  The product is within an ulp of the quotient, far inside the
                    // window in which A's fp32 accumulation order already moves codes.
                    const float rs = 1.0f / sc;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t w = e4m3x4(av[i][4 * q] * rs, av[i][4 * q + 1] * rs, av[i][4 * q + 2] * rs,
                                                  av[i][4 * q + 3] * rs);
                        const int byte = cg * 32 + q * 8 + hi * 4;
                        *reinterpret_cast<uint32_t*>(codes + m * 128 + (((byte >> 4) ^ (m & 7)) << 4) + (byte & 15)) = w;
                    }
                    if (cg == 0 && hi == 0 && m < t.nrows) p.out_scale[(size_t)(t.row0 + m) * IB + t.nt] = sc;
                }
            }
            __syncthreads();
            for (int q = threadIdx.x; q < BM * 8; q += NW * 64) {
                const int row = q >> 3, c = q & 7;
                if (row < t.nrows)
                    *reinterpret_cast<u32x4*>(p.out + (size_t)(t.row0 + row) * p.N + t.nt * 128 + c * 16) =
                        *reinterpret_cast<const u32x4*>(codes + row * 128 + ((c ^ (row & 7)) << 4));
            }
        }
    } else {
        // Blocks are transposed (lane l32 holds a row, element r holds column (r >> 2) * 8 + hi * 4 +
        // (r & 3) of n-block j): the tile's bf16 rows go through LDS and leave in 16-byte pieces.
        ordered_barrier();                                       // every wave is done with the ring
        uint8_t* stg = smem;                                     // [BM][512 B], chunks c at c ^ (row & 31)
        if (active) {
#pragma unroll
            for (int i = 0; i < MW; ++i) {
                const int m = rbase + i * 32 + l32;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t w0 = bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                        const uint32_t w1 = bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                        const int byte = (cg * 64 + j * 32 + q * 8 + hi * 4) * 2;
                        uint32_t* d = reinterpret_cast<uint32_t*>(stg + m * 512 + (((byte >> 4) ^ (m & 31)) << 4) + (byte & 15));
                        d[0] = w0;
                        d[1] = w1;
                    }
            }
        }
        __syncthreads();
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
        for (int q = threadIdx.x; q < BM * 32; q += NW * 64) {
            const int row = q >> 5, c = q & 31;
            if (row < t.nrows) {
                u32x4* dst = reinterpret_cast<u32x4*>(out + (size_t)(t.row0 + row) * p.N + t.nt * 256 + c * 8);
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * 512 + ((c ^ (row & 31)) << 4));
                // y_perm is read once, by the combine, and is larger than the caches: stream it out
                if constexpr (DWDP_YPERM_NT) __builtin_nontemporal_store(v, dst);
                else *dst = v;
            }
        }
    }
}

template <int BM, int KIND, bool FP8>
__global__ __launch_bounds__((FragCfg<BM, rowb_of(BM, FP8), FP8>::NW * 64), 1) void gemm_frag_kernel(GemmParams p) {
    constexpr int ROWB = rowb_of(BM, FP8);
    using C = FragCfg<BM, ROWB, FP8>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::NS * C::STAGE + C::EXTRA];
    float* s_bscale = reinterpret_cast<float*>(smem + C::NS * C::STAGE);   // fp8 only

    TileCtx c;
    int lin;
    if (p.ticket != nullptr) {
        // Tiles in schedule order to whichever workgroup asks first, on any XCD (used where tiles share
        // next to nothing: 32-row tiles of small groups, which only stream weights).  Every workgroup
        // draws exactly one ticket, so the draw of ticket gridDim.x - 1 is the launch's last: that
        // workgroup resets the counter for the next launch.  The ticket passes through the ring's first
        // word, which is rewritten only after the second barrier.
        int* s_ticket = reinterpret_cast<int*>(smem);
        if (threadIdx.x == 0) {
            const int tk = atomicAdd(p.ticket, 1);
            if (tk == (int)gridDim.x - 1) atomicExch(p.ticket, 0);
            *s_ticket = tk;
        }
        __syncthreads();
        lin = *s_ticket;
        __syncthreads();
    } else {
        lin = dealt_lin(KIND == kGemm1 ? DWDP_CLUSTER_GEMM1_LOG2 : DWDP_CLUSTER_GEMM2_LOG2);
    }
    if (!decode_tile<BM, KIND>(p, c.t, lin)) return;
#if DWDP_TILE_TRACE
    const uint64_t trace_t0 = __builtin_amdgcn_s_memrealtime();
#endif
    // Above the default wave priority, so that the GEMM's waves win the arbitration on a CU that also
    // hosts waves of another kernel (the layer-ahead prefetch copy); alone it makes no difference.
    __builtin_amdgcn_s_setprio(2);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    c.KT = p.K / (FP8 ? ROWB : ROWB / 2);
    const uint8_t* wbase;
    if (KIND == kGemm1) {
        wbase = static_cast<const uint8_t*>(p.table[c.t.g].w13);
        c.wscale = p.table[c.t.g].s13;
    } else {
        wbase = static_cast<const uint8_t*>(p.table[c.t.g].w2);
        c.wscale = p.table[c.t.g].s2;
    }
    // fragment-major weights: 4 KB per 32-row n-block per 128 bytes of K
    const size_t nblk_bytes = (size_t)p.K * (FP8 ? 1 : 2) * 32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int cg = wave & 3;
        c.nblk[j] = KIND == kGemm1 ? (j == 0 ? 0 : p.I / 32) + c.t.nt * 4 + cg : c.t.nt * 8 + cg * 2 + j;
        c.wb[j] = wbase + (size_t)c.nblk[j] * nblk_bytes + lane * 16;
    }
    if constexpr (FP8) {
        const int KB = p.K / kFp8Group;
        for (int q = lane; q < 2 * KB; q += 64) {
            const int j = q / KB, kb = q % KB;
            s_bscale[(wave * 2 + j) * 64 + kb] = c.wscale[(size_t)(c.nblk[j] * 32 / kFp8Group) * KB + kb];
        }
        __syncthreads();
    }
    // active 32-row m-blocks
    const int ma = (c.t.nrows + 31) / 32;
    auto dispatch = [&](auto pol) __attribute__((always_inline)) {
        constexpr int WPOL = decltype(pol)::value;
        if constexpr (C::NW == 4) {
            if constexpr (C::MI == 1) {
                frag_tile<BM, ROWB, 1, 1, KIND, FP8, WPOL>(p, c, smem, s_bscale);
            } else if constexpr (C::MI == 2) {
                if (ma <= 1) frag_tile<BM, ROWB, 1, 1, KIND, FP8, WPOL>(p, c, smem, s_bscale);
                else frag_tile<BM, ROWB, 2, 2, KIND, FP8, WPOL>(p, c, smem, s_bscale);
            } else {
                static_assert(C::MI == 4, "4-wave tiles hold at most 128 rows");
                if (ma <= 1) frag_tile<BM, ROWB, 1, 1, KIND, FP8, WPOL>(p, c, smem, s_bscale);
                else if (ma == 2) frag_tile<BM, ROWB, 2, 2, KIND, FP8, WPOL>(p, c, smem, s_bscale);
                else if (ma == 3) frag_tile<BM, ROWB, 3, 3, KIND, FP8, WPOL>(p, c, smem, s_bscale);
                else frag_tile<BM, ROWB, 4, 4, KIND, FP8, WPOL>(p, c, smem, s_bscale);
            }
        } else {
            // two row parts of MIW m-blocks: the first part takes the first active blocks; a part without
            // active rows runs the load-only variant (the same loads as the active part's)
            constexpr int MIW = C::MIW;
            const int rh = wave >> 2;
            auto run = [&](auto tag) {
                constexpr int MA = decltype(tag)::value;
                constexpr int W0 = MA < MIW ? MA : MIW, W1 = MA > MIW ? MA - MIW : 0;
                if (rh == 0) frag_tile<BM, ROWB, MA, W0, KIND, FP8, WPOL>(p, c, smem, s_bscale);
                else if constexpr (W1 > 0) frag_tile<BM, ROWB, MA, W1, KIND, FP8, WPOL>(p, c, smem, s_bscale);
                else frag_tile<BM, ROWB, MIW, 0, KIND, FP8, WPOL>(p, c, smem, s_bscale);
            };
            if constexpr (MIW == 4) {
                if (ma <= 1) run(std::integral_constant<int, 1>{});
                else if (ma == 2) run(std::integral_constant<int, 2>{});
                else if (ma <= 4) run(std::integral_constant<int, 4>{});
                else if (ma <= 6) run(std::integral_constant<int, 6>{});
                else run(std::integral_constant<int, 8>{});
            } else {
                static_assert(MIW == 2, "8-wave tiles are 128 (fp8) or 256 (bf16) rows");
                if (ma <= 1) run(std::integral_constant<int, 1>{});
                else if (ma == 2) run(std::integral_constant<int, 2>{});
                else if (ma == 3) run(std::integral_constant<int, 3>{});
                else run(std::integral_constant<int, 4>{});
            }
        }
    };
    // A group with one m-tile reads each weight slab exactly once: stream it (kStreamWeightCpol)
    if constexpr (kStreamWeightCpol == DWDP_WEIGHT_CPOL) {
        dispatch(std::integral_constant<int, DWDP_WEIGHT_CPOL>{});
    } else {
        if (c.t.mc == 1) dispatch(std::integral_constant<int, kStreamWeightCpol>{});
        else dispatch(std::integral_constant<int, DWDP_WEIGHT_CPOL>{});
    }
#if DWDP_TILE_TRACE
    __syncthreads();                                   // every wave has finished the tile
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kTraceRecords) {
        dwdp_tile_record r;
        r.t_start = trace_t0;
        r.t_end = __builtin_amdgcn_s_memrealtime();
        r.order = c.t.lin;
        r.group = c.t.g;
        r.first_row = (int32_t)c.t.row0;
        r.rows = c.t.nrows;
        r.n_tile = c.t.nt;
        r.group_m_tiles = c.t.mc;
        r.xcd = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xF);   // hardware register XCC_ID, bits 3:0
        r.hw_id = (int)((__builtin_amdgcn_s_getreg((31 << 11) | 4) >> 8) & 0xFF);   // HW_ID bits 15:8
        tile_trace[blockIdx.x] = r;
    }
#endif
}

// ------------------------------------------------------------------------------ weight packing
// Fragment-major layout of a weight matrix W [N, K] (N % 32 == 0):
//   bf16 (K % 64 == 0): fragment (nb, kb) = rows 32nb..32nb+31, columns 16kb..16kb+15, 1 KB in
//     lane order -- lane l holds row 32nb + l%32, columns 16kb + 8(l/32) .. +7 -- stored at
//     byte (nb * K/16 + kb) * 1024.
//   fp8 (K % 128 == 0): fragment (nb, kb) = rows 32nb.., columns 64kb..64kb+63, 2 KB: lane l holds
//     row 32nb + l%32, columns 64kb + 32(l/32) .. +31; bytes h*16..h*16+15 of that slice sit at
//     byte (nb * K/64 + kb) * 2048 + h * 1024 + l * 16.
// Both give 4 KB per 32-row block per 128-byte K step, read as four 1 KB lane-ordered loads.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ w, int64_t N, int64_t K, int fp8,
                                                   uint8_t* __restrict__ out) {
    const int64_t nchunks = N * K * (fp8 ? 1 : 2) / 16;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nchunks; q += stride) {
        int64_t row, col;
        if (!fp8) {
            const int64_t frag = q >> 6, l = q & 63, per = K / 16;
            row = (frag / per) * 32 + (l & 31);
            col = (frag % per) * 16 + (l >> 5) * 8;
            *reinterpret_cast<uint4*>(out + q * 16) = *reinterpret_cast<const uint4*>(w + (row * K + col) * 2);
        } else {
            const int64_t frag = q >> 7, h = (q >> 6) & 1, l = q & 63, per = K / 64;
            row = (frag / per) * 32 + (l & 31);
            col = (frag % per) * 64 + (l >> 5) * 32 + h * 16;
            *reinterpret_cast<uint4*>(out + q * 16) = *reinterpret_cast<const uint4*>(w + row * K + col);
        }
    }
}

// ------------------------------------------------------------------------------ f32 kernel
// 64 x 64 tile, 256 threads, 4 x 4 outputs per thread, K step 16.  Exact-ish
// fp32 math (expf, IEEE division) for the small fp32 workload.
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float sA[BK][BM + 4];
    __shared__ float sB[BK][BN + 4];
    Tile t;
    if (!decode_tile<BM, KIND>(p, t)) return;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const float* A = reinterpret_cast<const float*>(p.a);
    const float* W;
    if (KIND == kGemm1) W = static_cast<const float*>(p.table[t.g].w13);
    else if (KIND == kGemm2) W = static_cast<const float*>(p.table[t.g].w2);
    else W = reinterpret_cast<const float*>(p.b_single);
    auto w_row = [&](int r) -> int {
        if (KIND == kGemm1) {
            const int n0 = t.nt * (BN / 2);
            return r < BN / 2 ? n0 + r : p.I + n0 + (r - BN / 2);
        }
        return min(t.nt * BN + r, p.N - 1);
    };
    // my B tile rows: GEMM1 pairs gate rows tx*2,+1 with up rows 32+tx*2,+1; others tx*4..+3
    int brow[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) brow[c] = KIND == kGemm1 ? (c < 2 ? tx * 2 + c : 32 + tx * 2 + (c - 2)) : tx * 4 + c;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lin = tid + i * 256, r = lin >> 4, kk = lin & 15;
            const int rr = min(r, t.nrows - 1);
            sA[kk][r] = A[(size_t)act_row(p, t.row0 + rr) * p.K + k0 + kk];
            sB[kk][r] = W[(size_t)w_row(r) * p.K + k0 + kk];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
            for (int c = 0; c < 4; ++c) b[c] = sB[kk][brow[c]];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(a[i], b[c], acc[i][c]);
        }
        __syncthreads();
    }
    float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = ty * 4 + i;
        if (m >= t.nrows) continue;
        const size_t orow = (size_t)(t.row0 + m) * p.N;
        if (KIND == kGemm1) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float g = acc[i][c], u = acc[i][c + 2];
                out[orow + t.nt * (BN / 2) + tx * 2 + c] = g / (1.0f + expf(-g)) * u;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int col = t.nt * BN + tx * 4 + c;
                if (col < p.N) out[orow + col] = acc[i][c] + ((KIND == kRouter && p.bias) ? p.bias[col] : 0.0f);
            }
        }
    }
}

// ------------------------------------------------------------------------------ configs
// Expert GEMMs (bf16, fp8): gemm_frag_kernel, BM x 256 tiles with BM = 32, 64, 128 or 256 (fp8: at
// most 128) picked from the mean rows per group (decode batches give groups of a few rows).
// f32: 64 x 64 FMA tiles.
// Router (bf16): router_dma_kernel or router_mfma_kernel, 64 x 64 tiles.
constexpr int kBnDma = 256;
constexpr int kBmF32 = 64, kBnF32 = 64;
constexpr int kBmRouter = 64, kBnRouter = 64;

int choose_bm(int dtype, int64_t rows, int groups) {
    if (dtype == DWDP_F32) return kBmF32;
    const int64_t mean = rows / groups;
    const int bm = mean >= 192 ? 256 : mean >= 96 ? 128 : mean >= 40 ? 64 : 32;
#ifdef DWDP_FP8_BM256
    return bm;
#else
    // fp8 stays at 128 rows by default: 256-row fp8 tiles (64-byte K steps, the accumulator rescaled at
    // every 128-wide K block) measured GEMM1 5.96 vs 5.60 ms and GEMM2 3.43 vs 3.49 ms at 16K tokens
    return dtype == DWDP_FP8_E4M3 && bm > 128 ? 128 : bm;
#endif
}

template <int BM>
void launch_schedule(const int32_t* offsets, int G, int32_t* pre, MTile* mt, MTile* mt_by_size, int32_t* tickets,
                     hipStream_t st) {
    hipLaunchKernelGGL(schedule_kernel<BM>, dim3(1), dim3(1024), 0, st, offsets, G, pre, mt, mt_by_size, tickets);
}

// decode_tile deals clusters of kCluster tiles round-robin over the 8 XCDs, so the launch holds whole
// rounds of 8 clusters: round the tile bound up to a multiple of 8 * kCluster (the surplus exits).
int64_t xcd_grid(int64_t tiles) {
    constexpr int64_t q = (int64_t)kNumXcd * kCluster;
    return (tiles + q - 1) / q * q;
}

template <int BM, int BN, int WM, int WN>
void launch_router(const GemmParams& p, int64_t tiles, hipStream_t st) {
    static_assert(BM == 64 && BN == 64 && WM == 2 && WN == 2, "the DMA router has one tile shape");
    // Up to two tiles per compute unit the DMA form is faster (its 64 KB ring leaves room for two
    // workgroups per unit, each with three steps in flight); larger batches need more workgroups per unit
    // at once, which the register-staged kernel's 32 KB allow.
    if (DWDP_ROUTER_DMA && tiles <= 2 * 256) {
        hipLaunchKernelGGL(router_dma_kernel<4>, dim3((unsigned)xcd_grid(tiles)), dim3(256), 0, st, p);
    } else {
        hipLaunchKernelGGL((router_mfma_kernel<BM, BN, WM, WN>), dim3((unsigned)xcd_grid(tiles)), dim3(WM * WN * 64),
                           0, st, p);
    }
}

template <int KIND>
void launch_f32(const GemmParams& p, int64_t tiles, hipStream_t st) {
    hipLaunchKernelGGL(gemm_f32_kernel<KIND>, dim3((unsigned)xcd_grid(tiles)), dim3(256), 0, st, p);
}

template <int BM, int KIND, bool FP8>
void launch_dma(const GemmParams& p, int64_t tiles, hipStream_t st) {
    constexpr int threads = FragCfg<BM, rowb_of(BM, FP8), FP8>::NW * 64;
    hipLaunchKernelGGL((gemm_frag_kernel<BM, KIND, FP8>), dim3((unsigned)xcd_grid(tiles)), dim3(threads), 0, st, p);
}

// g2_wide (fp8, 128-row GEMM1 tiles): GEMM2 runs 256-row tiles, whose schedule replaces GEMM1's in the
// same tables once GEMM1 is done (so a GEMM2-only call builds it too); maxm_wide bounds their m-tiles.
template <int BM>
void launch_ffn(bool g1, bool g2, bool fp8_path, bool g2_wide, const int32_t* offsets, int G, const GemmParams& p1,
                const GemmParams& p2, MTile* mt_group, MTile* mt_size, int64_t maxm, int64_t maxm_wide,
                hipStream_t st) {
    if (g1) launch_schedule<BM>(offsets, G, const_cast<int32_t*>(p1.mprefix), mt_group, mt_size, p1.ticket, st);
#ifdef DWDP_FP8_BM256
    constexpr bool fp8_tiles = true;
#else
    constexpr bool fp8_tiles = BM <= 128;
#endif
    if constexpr (fp8_tiles) {
        if (fp8_path) {
            if (g1) launch_dma<BM, kGemm1, true>(p1, maxm * p1.NT, st);
            if (g2) {
                if constexpr (BM == 128) {
                    if (g2_wide) {
                        launch_schedule<256>(offsets, G, const_cast<int32_t*>(p2.mprefix), mt_group, mt_size, nullptr,
                                             st);
                        launch_dma<256, kGemm2, true>(p2, maxm_wide * p2.NT, st);
                        return;
                    }
                }
                launch_dma<BM, kGemm2, true>(p2, maxm * p2.NT, st);
            }
            return;
        }
    }
    {
        if (g1) launch_dma<BM, kGemm1, false>(p1, maxm * p1.NT, st);
        if (g2) launch_dma<BM, kGemm2, false>(p2, maxm * p2.NT, st);
    }
}

}  // namespace

// Router GEMM: logits [T, E] = x [T, H] * w_router^T + bias.
int router_gemm(const void* x, const void* w, int dtype, const float* bias, int64_t T, int H, int E, float* logits,
                hipStream_t st) {
    GemmParams p{};
    p.a = static_cast<const uint8_t*>(x);
    p.b_single = static_cast<const uint8_t*>(w);
    p.bias = bias;
    p.rows = T;
    p.G = 1;
    p.N = E;
    p.K = H;
    p.out = reinterpret_cast<uint8_t*>(logits);
    if (dtype == DWDP_BF16) {
        p.NT = (E + kBnRouter - 1) / kBnRouter;
        const int64_t grid = ((T + kBmRouter - 1) / kBmRouter) * p.NT;
        DWDP_REQUIRE(xcd_grid(grid) * 256 <= kMaxLaunchItems, "T too large for one router launch");
        launch_router<kBmRouter, kBnRouter, 2, 2>(p, grid, st);
    } else {
        p.NT = (E + kBnF32 - 1) / kBnF32;
        const int64_t grid = ((T + kBmF32 - 1) / kBmF32) * p.NT;
        DWDP_REQUIRE(xcd_grid(grid) * 256 <= kMaxLaunchItems, "T too large for one router launch");
        launch_f32<kRouter>(p, grid, st);
    }
    DWDP_LAUNCHED();
    return DWDP_OK;
}

}  // namespace dwdp

using namespace dwdp;

namespace {

// The grouped FFN.  a_rows == nullptr: GEMM1's activation row r is x row r (x holds the permuted
// rows); otherwise it is x row a_rows[r] (x holds the x_rows token rows).
int grouped_ffn(int stage, const dwdp_expert_ptrs* table, int n_groups, const int32_t* offsets, const int32_t* a_rows,
                const void* x, const float* x_scale, int64_t x_rows, int64_t rows, int H, int I, int w_dtype,
                void* y_perm, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    DWDP_REQUIRE(stage >= 0 && stage <= 2, "stage must be 0, 1 or 2");
    DWDP_REQUIRE(w_dtype == DWDP_F32 || w_dtype == DWDP_BF16 || w_dtype == DWDP_FP8_E4M3, "unknown w_dtype");
    DWDP_REQUIRE(n_groups >= 1 && n_groups <= (1 << 20), "n_groups out of range");
    DWDP_REQUIRE(rows >= 0 && rows < (int64_t)1 << 31, "rows out of range");
    DWDP_REQUIRE(H > 0 && I > 0, "H and I must be positive");
    if (w_dtype == DWDP_F32) {
        DWDP_REQUIRE(H % 64 == 0 && I % 32 == 0 && H % 16 == 0 && I % 16 == 0, "f32 path needs H % 64 == 0, I % 32 == 0");
    } else {
        DWDP_REQUIRE(H % 256 == 0 && I % 128 == 0, "bf16/fp8 paths need H % 256 == 0 and I % 128 == 0");
        if (w_dtype == DWDP_FP8_E4M3) DWDP_REQUIRE(H <= 8192 && I <= 8192, "fp8 path needs H, I <= 8192");
    }
    if (rows == 0) return DWDP_OK;
    DWDP_REQUIRE(table && offsets && x && ws && (y_perm || stage == 1), "null pointer argument");
    DWDP_REQUIRE(aligned16(table) && aligned16(x) && aligned16(y_perm) && aligned16(ws),
                 "pointers must be 16-byte aligned");
    DWDP_REQUIRE(x_rows >= 1 && x_rows < ((int64_t)1 << 31), "x_rows out of range");
    if (w_dtype == DWDP_FP8_E4M3)
        DWDP_REQUIRE(x_scale != nullptr && aligned16(x_scale), "fp8 needs the activation scales, 16-byte aligned");
    FfnWs L = ffn_ws_layout(rows, n_groups, I, w_dtype);
    if (ws_bytes < L.total)
        return fail(DWDP_ERR_WORKSPACE, "dwdp_moe_grouped_ffn: workspace too small (need " + std::to_string(L.total) + ")");
    hipStream_t st = as_stream(stream);
    uint8_t* base = static_cast<uint8_t*>(ws);
    const int bm = choose_bm(w_dtype, rows, n_groups);
    const int64_t maxm = (rows + bm - 1) / bm + n_groups;

    GemmParams p1{};
    p1.a = static_cast<const uint8_t*>(x);
    p1.a_scale = x_scale;
    p1.a_rows = a_rows;
    p1.a_nrows = x_rows;
    p1.table = table;
    p1.offsets = offsets;
    p1.mprefix = reinterpret_cast<int32_t*>(base + L.pre);
    // GEMM1 walks the groups by size (bf16: measured ~1.5% faster at 8K tokens).  GEMM2 keeps group
    // order for bf16 (slower by size) and walks by size otherwise.  The order moves no result bit.
    MTile* mt_group = reinterpret_cast<MTile*>(base + L.mt);
    MTile* mt_size = reinterpret_cast<MTile*>(base + L.mt_by_size);
    p1.mtiles = mt_size;
    p1.G = n_groups;
    p1.N = I;
    p1.K = H;
    p1.I = I;
    p1.NT = w_dtype == DWDP_F32 ? I / (kBnF32 / 2) : I / (kBnDma / 2);
    p1.msuper = w_dtype == DWDP_FP8_E4M3 ? DWDP_MSUPER_FP8 : DWDP_MSUPER_BF16;
    p1.out = base + L.a;
    p1.out_scale = reinterpret_cast<float*>(base + L.a_scale);

    GemmParams p2 = p1;
    p2.mtiles = w_dtype == DWDP_BF16 ? mt_group : mt_size;
    p2.a = base + L.a;
    p2.a_scale = reinterpret_cast<const float*>(base + L.a_scale);
    p2.a_rows = nullptr;
    p2.a_nrows = rows;
    p2.N = H;
    p2.K = I;
    p2.NT = w_dtype == DWDP_F32 ? H / kBnF32 : H / kBnDma;
    p2.out = static_cast<uint8_t*>(y_perm);
    p2.out_scale = nullptr;
    // fp8 GEMM2 takes super-blocks of 8 m-tiles (16K fp8 GEMM2 3.41-3.42 ms against 3.44-3.46 with 4;
    // bf16 GEMM2 was not faster with 1, 2 or 8)
    if (w_dtype == DWDP_FP8_E4M3) p2.msuper = DWDP_MSUPER_FP8_GEMM2;
    // 32-row tiles (a few rows per group, as in decode) share next to nothing: they draw tickets, so
    // that every XCD keeps taking tiles until none are left.  The schedule kernel zeroes both counters
    // (p2.ticket = p1.ticket + 1), and each launch's last draw resets its own.
    if (DWDP_TICKET_TILES && w_dtype != DWDP_F32 && bm == 32) {
        p1.ticket = reinterpret_cast<int32_t*>(base + L.tickets);
        p2.ticket = p1.ticket + 1;
    }
    // every expert-GEMM launch holds at most 512 work-items per workgroup
    DWDP_REQUIRE(xcd_grid(maxm * std::max(p1.NT, p2.NT)) * 512 <= kMaxLaunchItems, "problem too large for one launch");

    const bool g1 = stage != 2, g2 = stage != 1;
    if (w_dtype == DWDP_F32) {
        if (g1) launch_schedule<kBmF32>(offsets, n_groups, const_cast<int32_t*>(p1.mprefix), mt_group, mt_size, nullptr,
                                        st);
        if (g1) launch_f32<kGemm1>(p1, maxm * p1.NT, st);
        if (g2) launch_f32<kGemm2>(p2, maxm * p2.NT, st);
    } else {
        const bool fp8 = w_dtype == DWDP_FP8_E4M3;
        // fp8 GEMM2 in 256-row tiles where the groups average 192 rows or more (the bf16 rule): half the
        // weight re-reads of 128-row tiles; GEMM1 stays at 128 rows (its per-block rescale made 256-row
        // tiles slower there)
        const bool g2_wide = DWDP_FP8_GEMM2_BM256 && fp8 && bm == 128 && rows / n_groups >= 192;
        const int64_t maxm_wide = (rows + 255) / 256 + n_groups;
        if (bm == 256)
            launch_ffn<256>(g1, g2, fp8, false, offsets, n_groups, p1, p2, mt_group, mt_size, maxm, maxm, st);
        else if (bm == 128)
            launch_ffn<128>(g1, g2, fp8, g2_wide, offsets, n_groups, p1, p2, mt_group, mt_size, maxm, maxm_wide, st);
        else if (bm == 64)
            launch_ffn<64>(g1, g2, fp8, false, offsets, n_groups, p1, p2, mt_group, mt_size, maxm, maxm, st);
        else launch_ffn<32>(g1, g2, fp8, false, offsets, n_groups, p1, p2, mt_group, mt_size, maxm, maxm, st);
    }
    DWDP_LAUNCHED();
    return DWDP_OK;
}

}  // namespace

extern "C" int dwdp_moe_grouped_ffn_stage(int stage, const dwdp_expert_ptrs* table, int n_groups,
                                          const int32_t* offsets, const void* x_perm, const float* x_perm_scale,
                                          int64_t rows, int H, int I, int w_dtype, void* y_perm, void* ws,
                                          size_t ws_bytes, void* stream) {
    return grouped_ffn(stage, table, n_groups, offsets, nullptr, x_perm, x_perm_scale, rows > 0 ? rows : 1, rows, H, I,
                       w_dtype, y_perm, ws, ws_bytes, stream);
}

extern "C" int dwdp_moe_grouped_ffn_tokens(int stage, const dwdp_expert_ptrs* table, int n_groups,
                                           const int32_t* offsets, const int32_t* perm_src, const void* x,
                                           const float* x_scale, int64_t T, int64_t rows, int H, int I, int w_dtype,
                                           void* y_perm, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    DWDP_REQUIRE(rows == 0 || perm_src != nullptr, "perm_src is NULL");
    DWDP_REQUIRE(rows == 0 || T >= 1, "T must be positive");
    return grouped_ffn(stage, table, n_groups, offsets, perm_src, x, x_scale, T, rows, H, I, w_dtype, y_perm, ws,
                       ws_bytes, stream);
}

// ------------------------------------------------------------------------------ no-allocation variant
// The grouped FFN's workspace (A, its fp8 scales and the tile schedule) in a fixed device array of the
// library, for callers that cannot allocate.  In host code `scratch` names a host-side stand-in, not
// the device array: its device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed on.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
    int dev = -1;
    DWDP_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(DWDP_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        DWDP_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (p == nullptr) return fail(DWDP_ERR_HIP, "hipGetSymbolAddress returned a null address for the scratch array");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DWDP_OK;
}

}  // namespace

extern "C" size_t dwdp_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" int dwdp_moe_grouped_ffn_tokens_static(int stage, const dwdp_expert_ptrs* table, int n_groups,
                                                  const int32_t* offsets, const int32_t* perm_src, const void* x,
                                                  const float* x_scale, int64_t T, int64_t rows, int H, int I,
                                                  int w_dtype, void* y_perm, void* stream) {
    clear_error();
    DWDP_REQUIRE(rows >= 0 && n_groups >= 1 && I > 0, "bad rows, n_groups or I");
    DWDP_REQUIRE(w_dtype == DWDP_F32 || w_dtype == DWDP_BF16 || w_dtype == DWDP_FP8_E4M3, "unknown w_dtype");
    const size_t need = ffn_ws_layout(rows, n_groups, I, w_dtype).total;
    if (need > kStaticScratchBytes)
        return fail(DWDP_ERR_WORKSPACE, "dwdp_moe_grouped_ffn_tokens_static: the workspace of " + std::to_string(rows) +
                                            " rows needs " + std::to_string(need) + " bytes, more than the " +
                                            std::to_string(kStaticScratchBytes) + "-byte static scratch");
    if (rows == 0) return DWDP_OK;
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != DWDP_OK) return rc;
    return dwdp_moe_grouped_ffn_tokens(stage, table, n_groups, offsets, perm_src, x, x_scale, T, rows, H, I, w_dtype,
                                       y_perm, ws, kStaticScratchBytes, stream);
}

extern "C" int dwdp_moe_grouped_ffn(const dwdp_expert_ptrs* table, int n_groups, const int32_t* offsets,
                                    const void* x_perm, const float* x_perm_scale, int64_t rows, int H, int I,
                                    int w_dtype, void* y_perm, void* ws, size_t ws_bytes, void* stream) {
    return dwdp_moe_grouped_ffn_stage(0, table, n_groups, offsets, x_perm, x_perm_scale, rows, H, I, w_dtype, y_perm,
                                      ws, ws_bytes, stream);
}

#if DWDP_TILE_TRACE
namespace {
__global__ __launch_bounds__(256) void zero_trace_kernel(uint4* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = uint4{0, 0, 0, 0};
}
}  // namespace
#endif

extern "C" int dwdp_diag_tile_trace_clear(void* stream) {
    clear_error();
#if DWDP_TILE_TRACE
    void* p = nullptr;
    DWDP_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(tile_trace)));
    static_assert(sizeof(tile_trace) % 16 == 0, "whole 16-byte words");
    const int64_t n = (int64_t)(sizeof(tile_trace) / 16);
    hipLaunchKernelGGL(zero_trace_kernel, dim3(1024), dim3(256), 0, as_stream(stream), static_cast<uint4*>(p), n);
    DWDP_LAUNCHED();
    return DWDP_OK;
#else
    (void)stream;
    return fail(DWDP_ERR_UNSUPPORTED, "dwdp_diag_tile_trace_clear: the library was built without -DDWDP_TILE_TRACE=1");
#endif
}

extern "C" int dwdp_diag_tile_trace_read(dwdp_tile_record* out, size_t max_records, size_t* n_records) {
    clear_error();
    DWDP_REQUIRE(out != nullptr && n_records != nullptr, "null pointer argument");
#if DWDP_TILE_TRACE
    void* p = nullptr;
    DWDP_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(tile_trace)));
    const size_t n = std::min(max_records, (size_t)kTraceRecords);
    DWDP_HIP(hipDeviceSynchronize());
    DWDP_HIP(hipMemcpy(out, p, n * sizeof(dwdp_tile_record), hipMemcpyDeviceToHost));
    *n_records = n;
    return DWDP_OK;
#else
    (void)max_records;
    return fail(DWDP_ERR_UNSUPPORTED, "dwdp_diag_tile_trace_read: the library was built without -DDWDP_TILE_TRACE=1");
#endif
}

extern "C" int dwdp_pack_weights(const void* w, int64_t N, int64_t K, int dtype, void* out, void* stream) {
    clear_error();
    DWDP_REQUIRE(dtype == DWDP_BF16 || dtype == DWDP_FP8_E4M3, "dtype must be DWDP_BF16 or DWDP_FP8_E4M3");
    DWDP_REQUIRE(N > 0 && K > 0 && N % 32 == 0, "N must be a positive multiple of 32");
    DWDP_REQUIRE(K % (dtype == DWDP_BF16 ? 64 : 128) == 0, "K must be a multiple of 64 (bf16) or 128 (fp8)");
    DWDP_REQUIRE(w && out && w != out, "w and out must be distinct non-null pointers");
    DWDP_REQUIRE(aligned16(w) && aligned16(out), "w and out must be 16-byte aligned");
    const int64_t chunks = N * K * (dtype == DWDP_BF16 ? 2 : 1) / 16;
    const int64_t grid = std::min<int64_t>((chunks + 255) / 256, 65536);
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(256), 0, as_stream(stream),
                       static_cast<const uint8_t*>(w), N, K, dtype == DWDP_FP8_E4M3 ? 1 : 0, static_cast<uint8_t*>(out));
    DWDP_LAUNCHED();
    return DWDP_OK;
}
