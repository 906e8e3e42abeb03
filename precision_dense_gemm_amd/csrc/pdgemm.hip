// pdgemm.hip -- multi-precision dense GEMM kernels for gfx950 (MI355X) and the
// C ABI declared in include/pdgemm.h.
//
// C = A * B with A row-major (M x K), B column-major (K x N) and C row-major,
// in FP16 -> fp32, INT8 -> int32 and packed signed INT4 -> int32.
//
// The method is the tiled matrix-unit GEMM of "Hand-Written PTX Tensor-Core
// GEMM Kernels: A Multi-Precision Study on NVIDIA L4": a block tile of C per
// workgroup, a loop over K tiles that are staged from global memory into
// double-buffered shared memory while the previous tile feeds the matrix
// units (Section II-B, Listing 1), fragments read from shared memory into
// registers (Listing 2), and the matrix multiply-accumulate itself
// (Section II-A).  Its design targets the L4; this file keeps the structure
// and re-derives every choice for CDNA4:
//
//  * Matrix units: v_mfma_f32_32x32x16_f16 and v_mfma_i32_32x32x32_i8.  Both
//    consume, per lane, 16 contiguous bytes of one row of A and of one column
//    of B (32 rows x 32 bytes of K per instruction), so FP16, INT8 and
//    unpacked INT4 share one LDS geometry: a K tile is 128 bytes per row.
//  * INT4: gfx950 has no signed 4-bit MFMA (the paper's m16n8k64.s4 path,
//    Listing 2, has no equivalent here).  Each packed dword w is split in
//    registers, on its way from global memory to LDS, into two int8 planes:
//    (w << 4) & 0xF0F0F0F0 holds 16*a for the even k and w & 0xF0F0F0F0 holds
//    16*a for the odd k, each as a signed byte.  A and B are split the same
//    way, so the planes pair k with k; every product is 256*a*b and the int32
//    sum is exactly 256*C (no overflow while 16384*K < 2^31, K <= 131071).
//    The epilogue shifts right by 8, which is exact.
//  * Staging: 16-byte global loads, coalesced along K (A rows and B columns
//    are both K-contiguous: the paper's "non-transposed B", Section IV-D),
//    into registers and then LDS, two LDS stages.  The 16-byte chunks of each
//    128-byte LDS row are XOR-swizzled by the row index so that the fragment
//    reads of consecutive rows fall in different banks (the paper pads shared
//    rows for the same reason on its first page's coalescing discussion; a
//    swizzle keeps rows dense).
//  * Tiles: a workgroup of 4 waves computes a BM x BN block of C, each wave a
//    WM x WN sub-block made of (WM/32) x (WN/32) MFMA tiles held in
//    accumulator registers for the whole K loop.
//  * Scheduling over 8 XCDs: workgroups are dispatched round-robin over the
//    XCDs, so the block id is remapped to give each XCD a contiguous range of
//    tiles, and tiles are ordered in bands of GM block rows so that the
//    workgroups resident on one XCD share A and B panels in its L2.
//  * Ragged edges: rows of A / columns of B past M / N are clamped to the
//    last valid one (their results are discarded); the last K tile loads
//    only bytes below K and zero-fills the rest, so no access leaves the
//    operands' valid extents.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "pdgemm.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef int intx4_t __attribute__((ext_vector_type(4)));
typedef int intx16_t __attribute__((ext_vector_type(16)));

constexpr int kF16 = PDGEMM_PREC_F16;
constexpr int kI8 = PDGEMM_PREC_I8;
constexpr int kI4 = PDGEMM_PREC_I4;

constexpr int kRowBytes = 128;   // LDS bytes per tile row per K tile
constexpr int kChunks = kRowBytes / 16;
constexpr int kWave = 64;

template <int P> struct Prec;
template <> struct Prec<kF16> {
    using Out = float;
    using Acc = floatx16_t;
    static constexpr int kGlobalRowBytes = 128;  // global bytes per row per K tile
    static constexpr int kElemsPerTile = 64;     // K elements per K tile
};
template <> struct Prec<kI8> {
    using Out = int32_t;
    using Acc = intx16_t;
    static constexpr int kGlobalRowBytes = 128;
    static constexpr int kElemsPerTile = 128;
};
template <> struct Prec<kI4> {
    using Out = int32_t;
    using Acc = intx16_t;
    static constexpr int kGlobalRowBytes = 64;
    static constexpr int kElemsPerTile = 128;
};

// Physical 16-byte chunk of logical chunk c in LDS row r.
__device__ __forceinline__ int swz(int c, int r) { return c ^ (r & 7); }

__device__ __forceinline__ uint4 load16(const uint8_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// The chunk [cb, cb + 16) of a row whose first `valid` bytes are data; bytes
// at or past `valid` read as zero and are never touched.
__device__ __forceinline__ uint4 load16_tail(const uint8_t *row, int cb, int valid) {
    if (cb + 16 <= valid) return load16(row + cb);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (cb >= valid) return v;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int b = 0; b < 16; ++b)
        if (cb + b < valid) w[b >> 2] |= (uint32_t)row[cb + b] << (8 * (b & 3));
    v.x = w[0];
    v.y = w[1];
    v.z = w[2];
    v.w = w[3];
    return v;
}

template <int P>
__device__ __forceinline__ typename Prec<P>::Acc mfma(const uint4 &a, const uint4 &b,
                                                      const typename Prec<P>::Acc &c) {
    if constexpr (P == kF16) {
        half8_t av, bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, &b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
    } else {
        intx4_t av, bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, &b, 16);
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, c, 0, 0, 0);
    }
}

// The two signed-byte planes of 16 packed INT4 bytes (see the file header).
__device__ __forceinline__ void split_s4(const uint4 &w, uint4 &even, uint4 &odd) {
    const uint32_t m = 0xF0F0F0F0u;
    even.x = (w.x << 4) & m;
    even.y = (w.y << 4) & m;
    even.z = (w.z << 4) & m;
    even.w = (w.w << 4) & m;
    odd.x = w.x & m;
    odd.y = w.y & m;
    odd.z = w.z & m;
    odd.w = w.w & m;
}

struct Args {
    const uint8_t *A;
    const uint8_t *B;
    void *C;
    int64_t lda_bytes;
    int64_t ldb_bytes;
    int64_t ldc;
    int M, N, K;
    int tiles_m, tiles_n;
};

template <int P, int BM, int BN, int WM, int WN, int GM>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave) void gemm_kernel(Args args) {
    using Acc = typename Prec<P>::Acc;
    using Out = typename Prec<P>::Out;
    constexpr int kWavesN = BN / WN;
    constexpr int kThreads = (BM / WM) * kWavesN * kWave;
    constexpr int kGRow = Prec<P>::kGlobalRowBytes;
    constexpr int kGChunks = kGRow / 16;                 // global chunks per row per K tile
    constexpr int kLoadsA = BM * kGChunks / kThreads;    // chunks per thread per K tile
    constexpr int kLoadsB = BN * kGChunks / kThreads;
    constexpr int FM = WM / 32;
    constexpr int FN = WN / 32;
    static_assert(BM * kGChunks % kThreads == 0 && BN * kGChunks % kThreads == 0, "tile/threads");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");

    __shared__ uint4 sA[2][BM][kChunks];
    __shared__ uint4 sB[2][BN][kChunks];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int M = args.M, N = args.N, K = args.K;

    // ---- block id -> tile, XCD-aware and banded by GM block rows ----
    int tile_m, tile_n;
    {
        const int nb = gridDim.x;
        const int bid = blockIdx.x;
        const int q = nb >> 3, r = nb & 7;
        const int xcd = bid & 7, loc = bid >> 3;
        const int id = (xcd < r) ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
        const int band = id / (GM * args.tiles_n);
        const int first_m = band * GM;
        const int rows = min(args.tiles_m - first_m, GM);
        const int in_band = id - band * GM * args.tiles_n;
        tile_m = first_m + in_band % rows;
        tile_n = in_band / rows;
    }
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    // ---- global staging assignment: chunk q of the tile -> (row, chunk) ----
    const uint8_t *a_rows[kLoadsA];
    const uint8_t *b_rows[kLoadsB];
    int a_r[kLoadsA], a_c[kLoadsA], b_r[kLoadsB], b_c[kLoadsB];
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
        const int q = tid + i * kThreads;
        a_r[i] = q / kGChunks;
        a_c[i] = q % kGChunks;
        const int gr = min(m0 + a_r[i], M - 1);
        a_rows[i] = args.A + (int64_t)gr * args.lda_bytes;
    }
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) {
        const int q = tid + i * kThreads;
        b_r[i] = q / kGChunks;
        b_c[i] = q % kGChunks;
        const int gr = min(n0 + b_r[i], N - 1);
        b_rows[i] = args.B + (int64_t)gr * args.ldb_bytes;
    }
    // valid bytes per row: f16 2K, i8 K, i4 K/2
    const int valid = (P == kF16) ? 2 * K : (P == kI8 ? K : K / 2);
    const int n_tiles = (K + Prec<P>::kElemsPerTile - 1) / Prec<P>::kElemsPerTile;

    uint4 ra[kLoadsA], rb[kLoadsB];

    auto load_tile = [&](int t) {
        const int kb = t * kGRow;
        if (kb + kGRow <= valid) {
#pragma unroll
            for (int i = 0; i < kLoadsA; ++i) ra[i] = load16(a_rows[i] + kb + a_c[i] * 16);
#pragma unroll
            for (int i = 0; i < kLoadsB; ++i) rb[i] = load16(b_rows[i] + kb + b_c[i] * 16);
        } else {
#pragma unroll
            for (int i = 0; i < kLoadsA; ++i) ra[i] = load16_tail(a_rows[i], kb + a_c[i] * 16, valid);
#pragma unroll
            for (int i = 0; i < kLoadsB; ++i) rb[i] = load16_tail(b_rows[i], kb + b_c[i] * 16, valid);
        }
    };

    auto store_tile = [&](int buf) {
        if constexpr (P == kI4) {
#pragma unroll
            for (int i = 0; i < kLoadsA; ++i) {
                uint4 e, o;
                split_s4(ra[i], e, o);
                sA[buf][a_r[i]][swz(2 * a_c[i], a_r[i])] = e;
                sA[buf][a_r[i]][swz(2 * a_c[i] + 1, a_r[i])] = o;
            }
#pragma unroll
            for (int i = 0; i < kLoadsB; ++i) {
                uint4 e, o;
                split_s4(rb[i], e, o);
                sB[buf][b_r[i]][swz(2 * b_c[i], b_r[i])] = e;
                sB[buf][b_r[i]][swz(2 * b_c[i] + 1, b_r[i])] = o;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kLoadsA; ++i) sA[buf][a_r[i]][swz(a_c[i], a_r[i])] = ra[i];
#pragma unroll
            for (int i = 0; i < kLoadsB; ++i) sB[buf][b_r[i]][swz(b_c[i], b_r[i])] = rb[i];
        }
    };

    // ---- accumulators ----
    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    const int wm0 = (wave / kWavesN) * WM;   // wave's first row in the block tile
    const int wn0 = (wave % kWavesN) * WN;
    const int frow = lane & 31;              // fragment row (A) / column (B) of this lane
    const int fhalf = lane >> 5;             // which 16-byte half of a 32-byte K step

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < n_tiles;
        if (more) load_tile(t + 1);

#pragma unroll
        for (int s = 0; s < kChunks / 2; ++s) {
            const int ch = swz(2 * s + fhalf, frow);
            uint4 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = sA[cur][wm0 + i * 32 + frow][ch];
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[j] = sB[cur][wn0 + j * 32 + frow][ch];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma<P>(af[i], bf[j], acc[i][j]);
        }

        if (more) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: 32x32 MFMA result layout -> row-major C ----
    // Register e of lane l holds row 8*(e/4) + 4*(l/32) + e%4, column l%32.
    Out *C = reinterpret_cast<Out *>(args.C);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn0 + j * 32 + frow;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm0 + i * 32 + 8 * (e >> 2) + 4 * fhalf + (e & 3);
                if (row < M && col < N) {
                    Out v;
                    if constexpr (P == kI4)
                        v = acc[i][j][e] >> 8;
                    else
                        v = acc[i][j][e];
                    C[(int64_t)row * args.ldc + col] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host side

struct Config {
    int bm, bn, wm, wn, gm;
};

constexpr Config kConfigs[] = {
    {256, 256, 128, 128, 4},  // 0: large shapes
    {128, 128, 64, 64, 8},    // 1: medium
    {64, 64, 32, 32, 8},      // 2: small
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

template <int P, int C>
const void *kernel_for() {
    constexpr Config c = kConfigs[C];
    return reinterpret_cast<const void *>(&gemm_kernel<P, c.bm, c.bn, c.wm, c.wn, c.gm>);
}

template <int P>
const void *kernel_ptr(int cfg) {
    switch (cfg) {
    case 0: return kernel_for<P, 0>();
    case 1: return kernel_for<P, 1>();
    case 2: return kernel_for<P, 2>();
    default: return nullptr;
    }
}

int elem_bits(int prec) { return prec == kF16 ? 16 : (prec == kI8 ? 8 : 4); }

bool sync_check_enabled() {
    static const bool on = [] {
        const char *e = getenv("PDGEMM_SYNC_CHECK");
        return e && strcmp(e, "1") == 0;
    }();
    return on;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int pick(int prec, int64_t M, int64_t N, int64_t K) {
    (void)prec;
    (void)K;
    // the largest tile that still gives every CU (256) at least one workgroup
    for (int c = 0; c < kNumConfigs; ++c)
        if (cdiv(M, kConfigs[c].bm) * cdiv(N, kConfigs[c].bn) >= 256) return c;
    return kNumConfigs - 1;
}

int validate(int prec, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
             const void *B, int64_t ldb, const void *C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return PDGEMM_EINVAL_DIM;
    if (M > INT32_MAX || N > INT32_MAX || K > (int64_t(1) << 30)) return PDGEMM_EINVAL_DIM;
    if (prec == kI4 && K > PDGEMM_I4_MAX_K) return PDGEMM_EINVAL_DIM;
    if (lda < K || ldb < K || ldc < N) return PDGEMM_EINVAL_LD;
    if (prec == kI4 && ((K & 1) || (lda & 1) || (ldb & 1))) return PDGEMM_EINVAL_I4;
    if (M == 0 || N == 0) return PDGEMM_OK;
    if (!C || (K > 0 && (!A || !B))) return PDGEMM_ENULL;
    const int64_t lda_bytes = lda * elem_bits(prec) / 8;
    const int64_t ldb_bytes = ldb * elem_bits(prec) / 8;
    if ((lda_bytes & 15) || (ldb_bytes & 15)) return PDGEMM_EALIGN;
    if (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || ((uintptr_t)C & 3)) return PDGEMM_EALIGN;
    return PDGEMM_OK;
}

int launch(int prec, int cfg, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
           const void *B, int64_t ldb, void *C, int64_t ldc, void *stream) {
    if (prec < 0 || prec > 2 || cfg < 0 || cfg >= kNumConfigs) return PDGEMM_EINVAL_CFG;
    int rc = validate(prec, M, N, K, A, lda, B, ldb, C, ldc);
    if (rc != PDGEMM_OK) return rc;
    if (M == 0 || N == 0) return PDGEMM_OK;

    const Config &c = kConfigs[cfg];
    Args args;
    // With K = 0 no operand byte is read; point at C so the clamped row
    // addresses the kernel forms are well-defined.
    args.A = K > 0 ? static_cast<const uint8_t *>(A) : static_cast<const uint8_t *>(C);
    args.B = K > 0 ? static_cast<const uint8_t *>(B) : static_cast<const uint8_t *>(C);
    args.C = C;
    args.lda_bytes = lda * elem_bits(prec) / 8;
    args.ldb_bytes = ldb * elem_bits(prec) / 8;
    args.ldc = ldc;
    args.M = (int)M;
    args.N = (int)N;
    args.K = (int)K;
    args.tiles_m = (int)cdiv(M, c.bm);
    args.tiles_n = (int)cdiv(N, c.bn);
    const int64_t blocks = (int64_t)args.tiles_m * args.tiles_n;
    if (blocks > INT32_MAX) return PDGEMM_EINVAL_DIM;

    const void *fn = prec == kF16 ? kernel_ptr<kF16>(cfg)
                     : prec == kI8 ? kernel_ptr<kI8>(cfg)
                                   : kernel_ptr<kI4>(cfg);
    const int threads = (c.bm / c.wm) * (c.bn / c.wn) * kWave;
    void *kargs[] = {&args};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(threads), kargs, 0, s);
    if (e != hipSuccess) return (int)e;
    if (sync_check_enabled()) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return (int)e;
    }
    return PDGEMM_OK;
}

}  // namespace

extern "C" {

int gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
             const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream) {
    return launch(kF16, pick(kF16, M, N, K), M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_i8(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
            const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    return launch(kI8, pick(kI8, M, N, K), M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_i4(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
            const uint8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    return launch(kI4, pick(kI4, M, N, K), M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int pdgemm_gemm_cfg(int prec, int cfg, int64_t M, int64_t N, int64_t K, const void *A,
                    int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
                    void *stream) {
    return launch(prec, cfg, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int pdgemm_num_configs(void) { return kNumConfigs; }

int pdgemm_pick_config(int prec, int64_t M, int64_t N, int64_t K) {
    if (prec < 0 || prec > 2) return -1;
    return pick(prec, M, N, K);
}

int pdgemm_config_info(int cfg, int *block_m, int *block_n, int *wave_m, int *wave_n,
                       int *threads) {
    if (cfg < 0 || cfg >= kNumConfigs) return PDGEMM_EINVAL_CFG;
    const Config &c = kConfigs[cfg];
    if (block_m) *block_m = c.bm;
    if (block_n) *block_n = c.bn;
    if (wave_m) *wave_m = c.wm;
    if (wave_n) *wave_n = c.wn;
    if (threads) *threads = (c.bm / c.wm) * (c.bn / c.wn) * kWave;
    return PDGEMM_OK;
}

const char *pdgemm_strerror(int code) {
    switch (code) {
    case PDGEMM_OK: return "success";
    case PDGEMM_EINVAL_DIM: return "invalid dimension (negative, too large, or INT4 K above 131071)";
    case PDGEMM_EINVAL_LD: return "leading dimension smaller than the row length";
    case PDGEMM_ENULL: return "null pointer for an operand with nonzero extent";
    case PDGEMM_EINVAL_I4: return "INT4 K, lda and ldb must be even";
    case PDGEMM_EALIGN: return "A and B must be 16-byte aligned with rows spanning a multiple of 16 bytes; C 4-byte aligned";
    case PDGEMM_EINVAL_CFG: return "unknown precision or tile configuration";
    default: return code > 0 ? hipGetErrorString((hipError_t)code) : "unknown error";
    }
}

int pdgemm_version(void) { return 100; }

}  // extern "C"
