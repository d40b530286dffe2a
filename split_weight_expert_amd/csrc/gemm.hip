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
//     host round trip): every group is cut into BM-row m-tiles; tile `lin`
//     of the (group, n-tile, m-tile) order -- m fastest, so the m-tiles that
//     share one weight tile run back to back -- is found from lin / NT.
//   * Workgroup ids are remapped so that each of the 8 XCDs (one 4 MB L2
//     each) walks one contiguous stretch of that order: the m-tiles sharing a
//     weight tile and the n-tiles sharing an activation tile are resident in
//     the same L2 at the same time, so HBM sees each weight byte about once.
//   * bf16 / fp8: both operands are K-contiguous; 128-byte row slices are
//     staged through LDS (XOR-swizzled 16-byte chunks, double buffered,
//     global loads for step k+1 in flight during the MFMAs of step k) and fed
//     to v_mfma_f32_32x32x16_bf16 or v_mfma_scale_f32_32x32x64_f8f6f4 (unit
//     scales).  fp8 keeps a per-128-K partial sum and folds it into the fp32
//     accumulator with (row scale x block scale).
//   * GEMM1's weight tile holds the gate rows and the up rows of the same
//     output columns, so SwiGLU is applied in registers in the epilogue.
//   * f32 (small shapes only): LDS-tiled FMA kernel with the same schedule.
#include "common.h"
#include "internal.h"

namespace dwdp {
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
    int32_t pad;
};

struct GemmParams {
    const uint8_t* a;               // activation rows [rows, K]
    const float* a_scale;           // fp8: [rows, K/128]
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
    int I;                          // GEMM1: first up row inside W13
    uint8_t* out;
    float* out_scale;               // GEMM1 fp8: A scales [rows, I/128]
};

struct Tile {
    int g;
    int nt;
    int64_t row0;
    int nrows;
};

template <int BM, int KIND>
__device__ __forceinline__ bool decode_tile(const GemmParams& p, Tile& t) {
    int total;
    int mt_router = 0;
    if (KIND == kRouter) {
        mt_router = (int)((p.rows + BM - 1) / BM);
        total = mt_router * p.NT;
    } else {
        total = p.mprefix[p.G] * p.NT;
    }
    const int per = (total + kNumXcd - 1) / kNumXcd;
    const int bid = blockIdx.x;
    const int slot = bid / kNumXcd;
    if (slot >= per) return false;
    const int lin = (bid % kNumXcd) * per + slot;
    if (lin >= total) return false;
    if (KIND == kRouter) {
        const int mi = lin % mt_router;
        t.g = 0;
        t.nt = lin / mt_router;
        t.row0 = (int64_t)mi * BM;
        t.nrows = (int)min((int64_t)BM, p.rows - t.row0);
        return true;
    }
    const MTile m = p.mtiles[lin / p.NT];
    const int rem = lin - m.m0 * p.NT;
    t.g = m.g;
    t.nt = rem / m.mc;
    const int mi = rem - t.nt * m.mc;
    const int r0 = p.offsets[m.g], r1 = p.offsets[m.g + 1];
    t.row0 = (int64_t)r0 + (int64_t)mi * BM;
    t.nrows = min(BM, r1 - (int)t.row0);
    return true;
}

// ------------------------------------------------------------------------------ schedule
// One workgroup: m-tile counts per group, their exclusive scan, and the m-tile table.
template <int BM>
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ offsets, int G,
                                                        int32_t* __restrict__ mprefix, MTile* __restrict__ mtiles) {
    __shared__ int wave_sum[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < G; base += 1024) {
        const int g = base + tid;
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
            mprefix[g] = excl;
            for (int m = 0; m < c; ++m) mtiles[excl + m] = MTile{g, excl, c, 0};
        }
        __syncthreads();
        if (tid == 0) {
            int s = 0;
            for (int w = 0; w < 16; ++w) s += wave_sum[w];
            carry_s += s;
        }
        __syncthreads();
    }
    if (tid == 0) mprefix[G] = carry_s;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ------------------------------------------------------------------------------ MFMA kernel
// BM x BN tile, WM x WN waves, 128 bytes of K per step (64 bf16 or 128 fp8 elements).
template <int BM, int BN, int WM, int WN, int KIND, bool FP8>
__global__ __launch_bounds__(WM * WN * 64) void gemm_mfma_kernel(GemmParams p) {
    constexpr int NTHR = WM * WN * 64;
    constexpr int ROWB = 128;
    constexpr int KSTEP = FP8 ? 128 : 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MI = TM / 32, NJ = TN / 32;
    constexpr int AC = BM * 8 / NTHR, BC = BN * 8 / NTHR;
    static_assert(AC >= 1 && BC >= 1 && BM * 8 % NTHR == 0 && BN * 8 % NTHR == 0, "tile / thread mismatch");
    static_assert(KIND != kGemm1 || NJ % 2 == 0, "GEMM1 waves hold gate and up blocks in pairs");

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * ROWB];

    Tile t;
    if (!decode_tile<BM, KIND>(p, t)) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, hi = lane >> 5;

    const uint8_t* wbase;
    const float* wscale = nullptr;
    if (KIND == kGemm1) {
        wbase = static_cast<const uint8_t*>(p.table[t.g].w13);
        wscale = p.table[t.g].s13;
    } else if (KIND == kGemm2) {
        wbase = static_cast<const uint8_t*>(p.table[t.g].w2);
        wscale = p.table[t.g].s2;
    } else {
        wbase = p.b_single;
    }
    const size_t ldk = (size_t)p.K * (FP8 ? 1 : 2);
    const int KT = p.K / KSTEP;

    // weight row held by tile row r
    auto w_row = [&](int r) -> int {
        if (KIND == kGemm1) {
            constexpr int half = BN / 2;
            const int n0 = t.nt * half;
            return r < half ? n0 + r : p.I + n0 + (r - half);
        }
        return min(t.nt * BN + r, p.N - 1);
    };
    // tile row of the first row of the wave's n-block j
    auto b_block_row = [&](int j) -> int {
        if (KIND == kGemm1) {
            constexpr int CW = BN / 2 / WN;
            return j < NJ / 2 ? wn * CW + j * 32 : BN / 2 + wn * CW + (j - NJ / 2) * 32;
        }
        return wn * TN + j * 32;
    };

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
        gb[i] = wbase + (size_t)w_row(r) * ldk + c * 16;
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

    // fp8: per-row activation scales of this lane's accumulator rows
    auto row_of = [&](int i, int r) -> int { return wm * TM + i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3); };

    gload(0);
    sstore(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const uint8_t* A = sA[cur];
        const uint8_t* B = sB[cur];
        if constexpr (!FP8) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ch = s * 2 + hi;
                bf16x8 af[MI], bf[NJ];
#pragma unroll
                for (int i = 0; i < MI; ++i) af[i] = __builtin_bit_cast(bf16x8, lds16(A, wm * TM + i * 32 + l32, ch));
#pragma unroll
                for (int j = 0; j < NJ; ++j) bf[j] = __builtin_bit_cast(bf16x8, lds16(B, b_block_row(j) + l32, ch));
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (!m_act[i]) continue;
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
                }
            }
        } else {
            f32x16 part[MI][NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ch = s * 4 + hi * 2;
                i32x8 af[MI], bf[NJ];
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const int row = wm * TM + i * 32 + l32;
                    const u32x4 lo = lds16(A, row, ch), up = lds16(A, row, ch + 1);
                    af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
                }
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int row = b_block_row(j) + l32;
                    const u32x4 lo = lds16(B, row, ch), up = lds16(B, row, ch + 1);
                    bf[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
                }
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (!m_act[i]) continue;
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], part[i][j], 0, 0, 0, 127,
                                                                                     0, 127);
                }
            }
            // fold this 128-wide K block: acc += part * (row scale * block scale)
            const int KB = p.K / kFp8Group;
            float sb[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) sb[j] = wscale[(size_t)(w_row(b_block_row(j)) / kFp8Group) * KB + kt];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (!m_act[i]) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = min(row_of(i, r), t.nrows - 1);
                    const float sa = p.a_scale[(size_t)(t.row0 + rr) * KB + kt];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[i][j][r] += part[i][j][r] * (sa * sb[j]);
                }
            }
        }
        if (kt + 1 < KT) sstore(cur ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    if constexpr (KIND == kGemm1) {
        constexpr int CW = BN / 2 / WN;          // A columns per wave
        const int colA = t.nt * (BN / 2) + wn * CW;
        if constexpr (!FP8) {
            uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int jb = 0; jb < NJ / 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = row_of(i, r);
                        if (m < t.nrows) {
                            const float a = silu_mul(acc[i][jb][r], acc[i][jb + NJ / 2][r]);
                            out[(size_t)(t.row0 + m) * p.N + colA + jb * 32 + l32] = f32_to_bf16(a);
                        }
                    }
        } else {
            // A is quantised per row and 128-column group; the tile spans exactly one group.
            static_assert(!FP8 || KIND != kGemm1 || BN / 2 == kFp8Group, "fp8 GEMM1 tile must cover one A group");
            __shared__ float red[WN][BM];
            float av[MI][NJ / 2][16];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int jb = 0; jb < NJ / 2; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) av[i][jb][r] = silu_mul(acc[i][jb][r], acc[i][jb + NJ / 2][r]);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float m = 0.0f;
#pragma unroll
                    for (int jb = 0; jb < NJ / 2; ++jb) m = fmaxf(m, fabsf(av[i][jb][r]));
#pragma unroll
                    for (int d = 16; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
                    if (l32 == 0) red[wn][row_of(i, r)] = m;
                }
            __syncthreads();
            uint8_t* out = p.out;
            const int IB = p.N / kFp8Group;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = row_of(i, r);
                    float amax = 0.0f;
#pragma unroll
                    for (int w = 0; w < WN; ++w) amax = fmaxf(amax, red[w][m]);
                    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
                    if (m < t.nrows) {
#pragma unroll
                        for (int jb = 0; jb < NJ / 2; ++jb)
                            out[(size_t)(t.row0 + m) * p.N + colA + jb * 32 + l32] = f32_to_e4m3(av[i][jb][r] / s);
                        if (wn == 0 && l32 == 0) p.out_scale[(size_t)(t.row0 + m) * IB + t.nt] = s;
                    }
                }
        }
    } else if constexpr (KIND == kGemm2) {
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = row_of(i, r);
                    if (m < t.nrows)
                        out[(size_t)(t.row0 + m) * p.N + t.nt * BN + wn * TN + j * 32 + l32] = f32_to_bf16(acc[i][j][r]);
                }
    } else {
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
}

// ------------------------------------------------------------------------------ LDS-DMA kernel
// The expert GEMMs.  One workgroup of 4 waves per CU computes a BM x 256 tile; the waves split the
// 256 weight rows (64 each) and share all BM activation rows, so a short tail tile skips whole
// 32-row m-blocks in every wave.  Operand slices of 128 bytes per row go straight from global
// memory into a 3-stage LDS ring (global_load_lds_dwordx4: no register staging), two K steps
// ahead of the MFMAs; each wave waits only for its own oldest stage (vmcnt) and one barrier per
// step orders the ring.  XOR-swizzled 16-byte chunks keep the ds_read_b128 fragment reads
// conflict-free.
// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at lds + 16 * l
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
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

template <int BM, int KIND, bool FP8>
__global__ __launch_bounds__(256, 1) void gemm_dma_kernel(GemmParams p) {
    constexpr int BN = 256, NW = 4, S = 3, ROWB = 128;
    constexpr int MI = BM / 32, NJ = 2;
    constexpr int AI = BM / 8 / NW, BI = BN / 8 / NW, PER = AI + BI;
    constexpr int STAGE = (BM + BN) * ROWB;
    static_assert(AI >= 1 && BM % 32 == 0, "BM must be 32, 64 or 128");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

    Tile t;
    if (!decode_tile<BM, KIND>(p, t)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    const uint8_t* wbase;
    const float* wscale;
    if (KIND == kGemm1) {
        wbase = static_cast<const uint8_t*>(p.table[t.g].w13);
        wscale = p.table[t.g].s13;
    } else {
        wbase = static_cast<const uint8_t*>(p.table[t.g].w2);
        wscale = p.table[t.g].s2;
    }
    const size_t ldk = (size_t)p.K * (FP8 ? 1 : 2);
    const int KT = p.K / (FP8 ? 128 : 64);

    auto w_row = [&](int r) -> int {
        if (KIND == kGemm1) return r < BN / 2 ? t.nt * (BN / 2) + r : p.I + t.nt * (BN / 2) + (r - BN / 2);
        return t.nt * BN + r;
    };
    // tile row of the first row of this wave's n-block j (GEMM1: j = 0 gate, j = 1 up)
    auto b_block_row = [&](int j) -> int { return KIND == kGemm1 ? j * (BN / 2) + wave * 32 : wave * 64 + j * 32; };
    auto row_of = [&](int i, int r) -> int { return i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3); };

    // lane l of a load instruction fills LDS row (l/8) position (l%8) of an 8-row group; it fetches the
    // logical chunk that the swizzle puts there
    const uint8_t* ga[AI];
    const uint8_t* gb[BI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int r = (wave * AI + i) * 8 + (lane >> 3), c = (lane & 7) ^ (r & 7);
        ga[i] = p.a + (size_t)(t.row0 + min(r, t.nrows - 1)) * ldk + c * 16;
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int r = (wave * BI + i) * 8 + (lane >> 3), c = (lane & 7) ^ (r & 7);
        gb[i] = wbase + (size_t)w_row(r) * ldk + c * 16;
    }
    auto issue = [&](int kt) {
        uint8_t* st = smem + (kt % S) * STAGE;
        const size_t off = (size_t)kt * ROWB;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            dma16(ga[i] + off, st + (wave * AI + i) * 8 * ROWB);
#pragma unroll
        for (int i = 0; i < BI; ++i)
            dma16(gb[i] + off, st + BM * ROWB + (wave * BI + i) * 8 * ROWB);
    };
    auto lds16 = [&](const uint8_t* base, int row, int chunk) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(base + row * ROWB + ((chunk ^ (row & 7)) << 4));
    };

    bool m_act[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) m_act[i] = i * 32 < t.nrows;

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    issue(0);
    if (KT > 1) issue(1);
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) wait_vmcnt<PER>();
        else wait_vmcnt<0>();
        ordered_barrier();
        // fp8 scales of this K block, loaded before the next DMA batch so that waiting for them does
        // not wait for that batch too (vector memory loads complete in order)
        [[maybe_unused]] float sb[NJ], sa[FP8 ? MI : 1][16];
        if constexpr (FP8) {
            const int KB = p.K / kFp8Group;
#pragma unroll
            for (int j = 0; j < NJ; ++j) sb[j] = wscale[(size_t)(w_row(b_block_row(j)) / kFp8Group) * KB + kt];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sa[i][r] = m_act[i] ? p.a_scale[(size_t)(t.row0 + min(row_of(i, r), t.nrows - 1)) * KB + kt] : 0.0f;
        }
        if (kt + 2 < KT) issue(kt + 2);
        const uint8_t* A = smem + (kt % S) * STAGE;
        const uint8_t* B = A + BM * ROWB;
        if constexpr (!FP8) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ch = s * 2 + hi;
                bf16x8 af[MI], bf[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) bf[j] = __builtin_bit_cast(bf16x8, lds16(B, b_block_row(j) + l32, ch));
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    if (m_act[i]) af[i] = __builtin_bit_cast(bf16x8, lds16(A, i * 32 + l32, ch));
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (!m_act[i]) continue;
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
                }
            }
        } else {
            f32x16 part[MI][NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) part[i][j][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ch = s * 4 + hi * 2;
                i32x8 af[MI], bf[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int row = b_block_row(j) + l32;
                    const u32x4 lo = lds16(B, row, ch), up = lds16(B, row, ch + 1);
                    bf[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2],
                                  (int)up[3]};
                }
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (!m_act[i]) continue;
                    const u32x4 lo = lds16(A, i * 32 + l32, ch), up = lds16(A, i * 32 + l32, ch + 1);
                    af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2],
                                  (int)up[3]};
                }
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    if (!m_act[i]) continue;
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], part[i][j], 0, 0, 0,
                                                                                     127, 0, 127);
                }
            }
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (!m_act[i]) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[i][j][r] += part[i][j][r] * (sa[i][r] * sb[j]);
            }
        }
    }

    // ---------------------------------------------------------------- epilogue
    if constexpr (KIND == kGemm1) {
        const int col = t.nt * (BN / 2) + wave * 32 + l32;     // A column of this lane
        if constexpr (!FP8) {
            uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = row_of(i, r);
                    if (m < t.nrows) out[(size_t)(t.row0 + m) * p.N + col] = f32_to_bf16(silu_mul(acc[i][0][r], acc[i][1][r]));
                }
        } else {
            // the tile's 128 A columns are exactly one quantisation group: amax over the 4 waves
            ordered_barrier();                                   // the ring is free: reuse it for the reduction
            float* red = reinterpret_cast<float*>(smem);         // [NW][BM]
            float av[MI][16];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    av[i][r] = silu_mul(acc[i][0][r], acc[i][1][r]);
                    float m = fabsf(av[i][r]);
#pragma unroll
                    for (int d = 16; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
                    if (l32 == 0) red[wave * BM + row_of(i, r)] = m;
                }
            __syncthreads();
            const int IB = p.N / kFp8Group;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = row_of(i, r);
                    const float amax = fmaxf(fmaxf(red[m], red[BM + m]), fmaxf(red[2 * BM + m], red[3 * BM + m]));
                    const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
                    if (m < t.nrows) {
                        p.out[(size_t)(t.row0 + m) * p.N + col] = f32_to_e4m3(av[i][r] / sc);
                        if (wave == 0 && l32 == 0) p.out_scale[(size_t)(t.row0 + m) * IB + t.nt] = sc;
                    }
                }
        }
    } else {
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = row_of(i, r);
                    if (m < t.nrows)
                        out[(size_t)(t.row0 + m) * p.N + t.nt * BN + wave * 64 + j * 32 + l32] = f32_to_bf16(acc[i][j][r]);
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
            sA[kk][r] = A[(size_t)(t.row0 + rr) * p.K + k0 + kk];
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
// Expert GEMMs (bf16, fp8): gemm_dma_kernel, BM x 256 tiles with BM = 32, 64 or 128 picked from the
// mean rows per group (decode batches give groups of a few rows).  f32: 64 x 64 FMA tiles.
// Router (bf16): gemm_mfma_kernel, 64 x 64 tiles.
constexpr int kBnDma = 256;
constexpr int kBmF32 = 64, kBnF32 = 64;
constexpr int kBmRouter = 64, kBnRouter = 64;
constexpr int kBmMin = 32;

int choose_bm(int dtype, int64_t rows, int groups) {
    if (dtype == DWDP_F32) return kBmF32;
    const int64_t mean = rows / groups;
    const int bm = mean >= 96 ? 128 : mean >= 40 ? 64 : 32;
    return dtype == DWDP_FP8_E4M3 ? (bm > 64 ? 64 : bm) : bm;   // fp8 keeps a partial sum: 64 rows max
}

size_t a256(size_t v) { return (v + 255) & ~size_t(255); }

struct FfnWs {
    size_t a, a_scale, pre, mt, total;
};

// Workspace: A [rows, I] (+ fp8 scales), the m-tile prefix [G+1] and the m-tile table, sized for
// the smallest BM so that any choice fits.
FfnWs ffn_ws_layout(int64_t rows, int groups, int I, int dtype) {
    FfnWs w{};
    const size_t ea = dtype == DWDP_F32 ? 4 : dtype == DWDP_BF16 ? 2 : 1;
    const int64_t maxm = (rows + kBmMin - 1) / kBmMin + groups;
    size_t off = 0;
    w.a = off;
    off += a256((size_t)rows * I * ea);
    w.a_scale = off;
    if (dtype == DWDP_FP8_E4M3) off += a256((size_t)rows * (I / kFp8Group) * 4);
    w.pre = off;
    off += a256((size_t)(groups + 1) * 4);
    w.mt = off;
    off += a256((size_t)maxm * sizeof(MTile));
    w.total = off;
    return w;
}

template <int BM>
void launch_schedule(const int32_t* offsets, int G, int32_t* pre, MTile* mt, hipStream_t st) {
    hipLaunchKernelGGL(schedule_kernel<BM>, dim3(1), dim3(1024), 0, st, offsets, G, pre, mt);
}

// decode_tile gives XCD x the slots x, x+8, x+16, ... of a stretch of ceil(total/8) tiles, so the
// launch must hold whole rounds of 8 workgroups: round the tile bound up to a multiple of 8.
int64_t xcd_grid(int64_t tiles) { return (tiles + kNumXcd - 1) / kNumXcd * kNumXcd; }

template <int BM, int BN, int WM, int WN, int KIND, bool FP8>
void launch_mfma(const GemmParams& p, int64_t tiles, hipStream_t st) {
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, KIND, FP8>), dim3((unsigned)xcd_grid(tiles)),
                       dim3(WM * WN * 64), 0, st, p);
}

template <int KIND>
void launch_f32(const GemmParams& p, int64_t tiles, hipStream_t st) {
    hipLaunchKernelGGL(gemm_f32_kernel<KIND>, dim3((unsigned)xcd_grid(tiles)), dim3(256), 0, st, p);
}

template <int BM, int KIND, bool FP8>
void launch_dma(const GemmParams& p, int64_t tiles, hipStream_t st) {
    hipLaunchKernelGGL((gemm_dma_kernel<BM, KIND, FP8>), dim3((unsigned)xcd_grid(tiles)), dim3(256), 0, st, p);
}

template <int BM>
void launch_ffn(bool g1, bool g2, bool fp8_path, const int32_t* offsets, int G, const GemmParams& p1,
                const GemmParams& p2, int64_t maxm, hipStream_t st) {
    if (g1) launch_schedule<BM>(offsets, G, const_cast<int32_t*>(p1.mprefix), const_cast<MTile*>(p1.mtiles), st);
    if constexpr (BM <= 64) {
        if (fp8_path) {
            if (g1) launch_dma<BM, kGemm1, true>(p1, maxm * p1.NT, st);
            if (g2) launch_dma<BM, kGemm2, true>(p2, maxm * p2.NT, st);
            return;
        }
    }
    {
        if (g1) launch_dma<BM, kGemm1, false>(p1, maxm * p1.NT, st);
        if (g2) launch_dma<BM, kGemm2, false>(p2, maxm * p2.NT, st);
    }
}

}  // namespace

size_t ffn_ws_bytes(int64_t rows, int groups, int H, int I, int dtype) {
    (void)H;
    if (dtype != DWDP_F32 && dtype != DWDP_BF16 && dtype != DWDP_FP8_E4M3) return 0;
    return ffn_ws_layout(rows, groups, I, dtype).total;
}

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
        launch_mfma<kBmRouter, kBnRouter, 2, 2, kRouter, false>(p, grid, st);
    } else {
        p.NT = (E + kBnF32 - 1) / kBnF32;
        const int64_t grid = ((T + kBmF32 - 1) / kBmF32) * p.NT;
        launch_f32<kRouter>(p, grid, st);
    }
    DWDP_LAUNCHED();
    return DWDP_OK;
}

}  // namespace dwdp

using namespace dwdp;

extern "C" int dwdp_moe_grouped_ffn_stage(int stage, const dwdp_expert_ptrs* table, int n_groups,
                                          const int32_t* offsets, const void* x_perm, const float* x_perm_scale,
                                          int64_t rows, int H, int I, int w_dtype, void* y_perm, void* ws,
                                          size_t ws_bytes, void* stream) {
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
    }
    if (rows == 0) return DWDP_OK;
    DWDP_REQUIRE(table && offsets && x_perm && ws && (y_perm || stage == 1), "null pointer argument");
    DWDP_REQUIRE(aligned16(table) && aligned16(x_perm) && aligned16(y_perm) && aligned16(ws),
                 "pointers must be 16-byte aligned");
    if (w_dtype == DWDP_FP8_E4M3) DWDP_REQUIRE(x_perm_scale != nullptr, "fp8 needs x_perm_scale");
    FfnWs L = ffn_ws_layout(rows, n_groups, I, w_dtype);
    if (ws_bytes < L.total)
        return fail(DWDP_ERR_WORKSPACE, "dwdp_moe_grouped_ffn: workspace too small (need " + std::to_string(L.total) + ")");
    hipStream_t st = as_stream(stream);
    uint8_t* base = static_cast<uint8_t*>(ws);
    const int bm = choose_bm(w_dtype, rows, n_groups);
    const int64_t maxm = (rows + bm - 1) / bm + n_groups;

    GemmParams p1{};
    p1.a = static_cast<const uint8_t*>(x_perm);
    p1.a_scale = x_perm_scale;
    p1.table = table;
    p1.offsets = offsets;
    p1.mprefix = reinterpret_cast<int32_t*>(base + L.pre);
    p1.mtiles = reinterpret_cast<MTile*>(base + L.mt);
    p1.G = n_groups;
    p1.N = I;
    p1.K = H;
    p1.I = I;
    p1.NT = w_dtype == DWDP_F32 ? I / (kBnF32 / 2) : I / (kBnDma / 2);
    p1.out = base + L.a;
    p1.out_scale = reinterpret_cast<float*>(base + L.a_scale);

    GemmParams p2 = p1;
    p2.a = base + L.a;
    p2.a_scale = reinterpret_cast<const float*>(base + L.a_scale);
    p2.N = H;
    p2.K = I;
    p2.NT = w_dtype == DWDP_F32 ? H / kBnF32 : H / kBnDma;
    p2.out = static_cast<uint8_t*>(y_perm);
    p2.out_scale = nullptr;
    DWDP_REQUIRE(maxm * p1.NT < ((int64_t)1 << 31) && maxm * p2.NT < ((int64_t)1 << 31),
                 "problem too large for one launch");

    const bool g1 = stage != 2, g2 = stage != 1;
    if (w_dtype == DWDP_F32) {
        if (g1) launch_schedule<kBmF32>(offsets, n_groups, const_cast<int32_t*>(p1.mprefix), const_cast<MTile*>(p1.mtiles), st);
        if (g1) launch_f32<kGemm1>(p1, maxm * p1.NT, st);
        if (g2) launch_f32<kGemm2>(p2, maxm * p2.NT, st);
    } else {
        const bool fp8 = w_dtype == DWDP_FP8_E4M3;
        if (bm == 128 && !fp8) launch_ffn<128>(g1, g2, false, offsets, n_groups, p1, p2, maxm, st);
        else if (bm == 64) launch_ffn<64>(g1, g2, fp8, offsets, n_groups, p1, p2, maxm, st);
        else launch_ffn<32>(g1, g2, fp8, offsets, n_groups, p1, p2, maxm, st);
    }
    DWDP_LAUNCHED();
    return DWDP_OK;
}

extern "C" int dwdp_moe_grouped_ffn(const dwdp_expert_ptrs* table, int n_groups, const int32_t* offsets,
                                    const void* x_perm, const float* x_perm_scale, int64_t rows, int H, int I,
                                    int w_dtype, void* y_perm, void* ws, size_t ws_bytes, void* stream) {
    return dwdp_moe_grouped_ffn_stage(0, table, n_groups, offsets, x_perm, x_perm_scale, rows, H, I, w_dtype, y_perm,
                                      ws, ws_bytes, stream);
}
