// pdgemm.hip -- multi-precision dense GEMM kernels for gfx950 (MI355X) and the
// C ABI declared in include/pdgemm.h.
//
// C = A * B with A row-major (M x K), B column-major or row-major (K x N) and
// C row-major, in FP16 -> fp32, INT8 -> int32 and packed signed INT4 -> int32,
// optionally followed (integer paths) by a dequantizing epilogue.
//
// The method is the tiled matrix-unit GEMM of "Hand-Written PTX Tensor-Core
// GEMM Kernels: A Multi-Precision Study on NVIDIA L4": a block tile of C per
// workgroup, a loop over K tiles that are staged from global memory into
// shared memory while earlier tiles feed the matrix units (Section II-B,
// Listing 1), fragments read from shared memory into registers (Listing 2),
// and the matrix multiply-accumulate itself (Section II-A).  Its design
// targets the L4; this file keeps the structure and re-derives every choice
// for CDNA4:
//
//  * Matrix units: v_mfma_f32_32x32x16_f16 and v_mfma_i32_32x32x32_i8.  Both
//    take, per lane, 16 contiguous bytes of K of one row of A and of one
//    column of B, so FP16, INT8 and packed INT4 share one LDS geometry: a K
//    tile is 64 bytes of K per row of A (32 f16, 64 int8, 128 int4 values).
//    The FP16 and INT8 tiles of 128 rows and more without K split run
//    v_mfma_f32_16x16x32_f16 and v_mfma_i32_16x16x64_i8 instead (the same 16
//    bytes per lane, fewer register accesses per MAC: see gemm_mf16_kernel).
//  * INT4: gfx950 has no signed 4-bit MFMA (the paper's m16n8k64.s4 path,
//    Listing 2, has no equivalent here).  INT4 stays packed in LDS; after a
//    fragment read each packed dword w is split in registers into two int8
//    planes: (w << 4) & 0xF0F0F0F0 holds 16*a for the even k and
//    w & 0xF0F0F0F0 holds 16*a for the odd k, each as a signed byte.  A and B
//    are split the same way, so the planes pair k with k; every product is
//    256*a*b and the int32 sum is exactly 256*C (no overflow while
//    16384*K < 2^31, K <= 131071).  The epilogue shifts right by 8 (exact).
//  * Staging: buffer_load_dwordx4 ... lds, a direct global -> LDS copy in
//    16-byte chunks.  A stage holds 128 bytes of K per row (per wave, with a
//    K split), so that every DMA instruction requests whole 128-byte lines
//    (the L2 returns whole lines: staging 64-byte pieces of them doubles the
//    L2 -> CU traffic), two or three stages deep; the 32 x 32 K-split tile
//    stages 64 bytes per row and wave, four stages deep.  The 16-byte chunks
//    of each LDS row are
//    XOR-swizzled by the row index so that fragment reads are free of bank
//    conflicts (the paper pads shared rows for the same purpose; a swizzle
//    keeps rows dense).
//  * B layouts: K-contiguous (column-major, the paper's "non-transposed B"
//    that its Section IV-D ablation finds fastest) is staged like A.
//    N-contiguous (row-major, the "transposed B" of the same ablation) is
//    staged as K rows of the tile and read with gfx950's transposing LDS reads
//    (ds_read_b64_tr_b16 / _b8 / _b4), which hand each lane K-contiguous
//    values of its own column: the same fragments, no transposition pass.
//  * Tiles: a workgroup of 4 or 8 waves computes a BM x BN block of C, each
//    wave a WM x WN sub-block made of (WM/32) x (WN/32) MFMA tiles held in
//    accumulator registers for the whole K loop.
//  * Scheduling over 8 XCDs: workgroups are dispatched round-robin over the
//    XCDs, so the block id is remapped to give each XCD a contiguous range of
//    tiles, and tiles are ordered in bands of GM block rows so that the
//    workgroups resident on one XCD share A and B panels in its L2.
//  * C is stored non-temporally: at N = 8192 its 268 MB would otherwise push
//    the A and B panels out of the 256 MB MALL between rounds of tiles.
//  * Ragged edges: rows of A (and columns of a column-major B) past M / N are
//    clamped to the last valid one, and the columns of a row-major B past N
//    are read from its padding; their results are discarded.  The buffer
//    range of each K tile ends at the last 16-byte chunk that holds valid
//    data, so the hardware zero-fills everything beyond it, and the last K
//    tile's fragments are masked below K.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "pdgemm.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef int intx2_t __attribute__((ext_vector_type(2)));
typedef int intx4_t __attribute__((ext_vector_type(4)));
typedef int intx16_t __attribute__((ext_vector_type(16)));

constexpr int kF16 = PDGEMM_PREC_F16;
constexpr int kI8 = PDGEMM_PREC_I8;
constexpr int kI4 = PDGEMM_PREC_I4;

constexpr int kRowBytes = 64;    // bytes of K per row per K tile (global and LDS)
constexpr int kChunks = kRowBytes / 16;
constexpr int kStages = 4;       // LDS stages: a K tile is fetched four tiles ahead
constexpr int kWave = 64;

template <int P> struct Prec;
template <> struct Prec<kF16> {
    using Out = float;
    using Acc = floatx16_t;
};
template <> struct Prec<kI8> {
    using Out = int32_t;
    using Acc = intx16_t;
};
template <> struct Prec<kI4> {
    using Out = int32_t;
    using Acc = intx16_t;
};
// INT4 run as e2m3 values on the FP6 matrix cores (an internal id: the
// entry points take INT4 and return int32): exact integer sums in fp32
constexpr int kF6 = 3;
template <> struct Prec<kF6> {
    using Out = int32_t;
    using Acc = floatx16_t;
};

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

// LDS position of logical 16-byte chunk c (0..3) of stage row r (64 bytes) is
// c ^ swizzle(r).  A fragment read has the 16 lanes of a quarter-wave on 16
// consecutive rows at the same logical chunk.  With 64 four-byte banks, row
// r's position p covers banks 16*(r%4) + 4p .. +3, so those 16 lanes are
// conflict-free iff the pairs (r%4, p) are all distinct; with 32 banks, iff
// any 8 consecutive rows have distinct pairs (r%2, p).
// ((r >> 1) & 3) ^ ((r >> 3) & 1) satisfies both.
__device__ __forceinline__ int swizzle(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// The same for rows of 128 bytes (eight chunks), where row r's position p
// covers banks 32*(r%2) + 4p .. +3 of 64: the 16 lanes of a quarter-wave
// are conflict-free iff the pairs (r%2, p) are all distinct, and with 32
// banks iff any 8 consecutive rows have distinct p.  (r & 7) ^ ((r >> 3) & 1)
// satisfies both.
__device__ __forceinline__ int swizzle8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ floatx16_t mfma_f16(const uint4 &a, const uint4 &b, const floatx16_t &c) {
    half8_t av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
}

__device__ __forceinline__ intx16_t mfma_i8(const uint4 &a, const uint4 &b, const intx16_t &c) {
    intx4_t av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, c, 0, 0, 0);
}

// The two signed-byte planes of 16 packed INT4 bytes (see the file header):
// `even` holds 16*a for the even k, `odd` 16*a for the odd k.  With kWide the
// even plane is shifted as two 64-bit values, one VALU instruction for two
// dwords: the nibble carried across a dword boundary lands in a low-nibble
// position, which the mask clears.  (Written in C++, the compiler narrows
// such a shift back to two 32-bit ones, since the carried bits are dead.)
// The whole-line kernels gain 2-5% on INT4 from it; the 64-byte-stage kernel
// was 3-8% slower, so it keeps the 32-bit form.
template <bool kWide>
__device__ __forceinline__ void split_s4(const uint4 &w, uint4 &even, uint4 &odd) {
    const uint32_t m = 0xF0F0F0F0u;
    if constexpr (kWide) {
        uint64_t lo = (uint64_t(w.y) << 32) | w.x;
        uint64_t hi = (uint64_t(w.w) << 32) | w.z;
        asm("v_lshlrev_b64 %0, 4, %1" : "=v"(lo) : "v"(lo));
        asm("v_lshlrev_b64 %0, 4, %1" : "=v"(hi) : "v"(hi));
        even.x = uint32_t(lo) & m;
        even.y = uint32_t(lo >> 32) & m;
        even.z = uint32_t(hi) & m;
        even.w = uint32_t(hi >> 32) & m;
    } else {
        even.x = (w.x << 4) & m;
        even.y = (w.y << 4) & m;
        even.z = (w.z << 4) & m;
        even.w = (w.w << 4) & m;
    }
    odd.x = w.x & m;
    odd.y = w.y & m;
    odd.z = w.z & m;
    odd.w = w.w & m;
}

struct Args {
    const uint8_t *A;
    const uint8_t *B;
    void *C;
    const float *scale_a;  // dequantizing epilogue only: one scale per row of A
    const float *scale_b;  // ... and per column of B
    int64_t lda_bytes;
    int64_t ldb_bytes;
    int64_t ldc;
    int M, N, K;
    int tiles_m, tiles_n;
    int kslice;   // K split across workgroups (epilogue kAtomicAdd): K values per split, else 0
};

// Epilogues: the int32 / fp32 sums as they are, or (integer paths) the
// dequantized ((float)sum * scale_a[i]) * scale_b[j] as fp32 or binary16.
constexpr int kRaw = 0;
constexpr int kDequantF32 = 1;
constexpr int kDequantF16 = 2;
// (K split across workgroups) the sums of one range of K added atomically
// into C, which the host has zeroed
constexpr int kAtomicAdd = 3;
constexpr bool is_dequant(int e) { return e == kDequantF32 || e == kDequantF16; }

template <int P, int E> struct OutOf { using type = typename Prec<P>::Out; };
template <int P> struct OutOf<P, kDequantF32> { using type = float; };
template <int P> struct OutOf<P, kDequantF16> { using type = _Float16; };

// B layouts: K-contiguous (column-major) or N-contiguous (row-major).
constexpr int kBCol = 0;
constexpr int kBRow = 1;

// Row-major B in LDS.  A stage holds the tile's kKRows rows of B (the K
// values of one 64-byte K tile: 32, 64 or 128 rows), each BN values wide
// (kCpr 16-byte chunks).  A transposing read hands each lane R consecutive
// rows of one column: the 16 lanes of a group read R rows (f16 4, i8 8,
// i4 16) and Q = 16/R chunks of each, so a half-wave covers 16 chunk
// positions.  Position p of row r holds logical chunk p ^ bswizzle(r);
// bswizzle(r) = Q * ((r / V) % (min(kCpr, 16) / Q)) with V = max(1, 16/kCpr)
// makes the 16 positions of a half-wave fall in 16 different 16-byte bank
// groups (64 banks), so the reads are conflict-free.
template <int P> struct RowB {
    static constexpr int kKRows = P == kF16 ? 32 : (P == kI8 ? 64 : 128);  // rows per K tile
    static constexpr int kR = P == kF16 ? 4 : (P == kI8 ? 8 : 16);         // rows per read
    static constexpr int kQ = 16 / kR;                                      // chunks per row per read
    static constexpr int kElemPerChunk = P == kF16 ? 8 : (P == kI8 ? 16 : 32);
};

template <int P, int BN>
__device__ __forceinline__ int bswizzle(int r) {
    constexpr int cpr = BN / RowB<P>::kElemPerChunk;
    constexpr int v = cpr >= 16 ? 1 : 16 / cpr;
    constexpr int span = (cpr < 16 ? cpr : 16) / RowB<P>::kQ;
    return RowB<P>::kQ * ((r / v) % span);
}

// Block id -> tile (tile_m, tile_n).  Workgroups are dispatched round-robin
// over the 8 XCDs, so the block id is remapped to give each XCD a contiguous
// range of tiles, and tiles are ordered in bands of GM block rows (column by
// column within a band), so that the workgroups resident on one XCD share A
// and B panels in its L2.
//
// With kWindows and band 4 (the 256-row tiles, and every tile of the 16 x 16
// MFMA kernel) and a grid of whole 16 x 16 windows of tiles, the order is by
// window instead: window w takes block ids 256 w .. 256 w + 255, one round of
// the 256 CUs at one workgroup each; in it XCD x
// runs the 4 x 8 tiles at block row x % 4, block column x / 4 (column by
// column), and the windows are taken row by row in serpentine order.  Each
// XCD still shares 4 panels of A and 8 of B in its L2, but a round reads 16
// panels of A and 16 of B from memory instead of all of A's and a quarter of
// B's, and each window shares one side with the one before, which the MALL
// still holds when the GEMM starts cold (8192^3 FP16 and INT8 in a sweep of
// other GEMMs: 2-4% faster; the same back to back).
template <int GM, bool kWindows = true>
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int &tile_m, int &tile_n) {
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    if constexpr (kWindows && GM == 4) {
        if (((tiles_m | tiles_n) & 15) == 0) {
            const int x = bid & 7, loc = bid >> 3;
            const int w = loc >> 5, k = loc & 31;   // window; this XCD's k-th tile in it
            const int wcols = tiles_n >> 4;
            const int wm = w / wcols, wi = w - wm * wcols;
            const int wn = (wm & 1) ? wcols - 1 - wi : wi;
            tile_m = wm * 16 + (x & 3) * 4 + (k & 3);
            tile_n = wn * 16 + (x >> 2) * 8 + (k >> 2);
            return;
        }
    }
    const int q = nb >> 3, r = nb & 7;
    const int xcd = bid & 7, loc = bid >> 3;
    const int id = (xcd < r) ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
    const int band = id / (GM * tiles_n);
    const int first_m = band * GM;
    const int rows = min(tiles_m - first_m, GM);
    const int in_band = id - band * GM * tiles_n;
    tile_m = first_m + in_band % rows;
    tile_n = in_band / rows;
}

// Epilogue of a tile without K split: the accumulators of a wave's WM x WN
// sub-block (FM x FN MFMA blocks of 32 x 32) stored to row-major C, converted
// per precision (INT4 planes: the exact >> 8; INT4 on the FP6 cores: the
// integer-valued fp32 sum to int32) and, with a dequantizing epilogue, scaled.
// Register e of lane l in MFMA block (i, j) holds row
// i*32 + 8*(e/4) + 4*(l/32) + e%4 and column j*32 + l%32 of the wave's
// tile.  Row offsets are wave-uniform (scalar registers); each lane adds
// one 32-bit offset, so a store costs no vector address arithmetic.
template <int P, int E, int BM, int BN, int FM, int FN, typename AccT>
__device__ __forceinline__ void store_tile(void *C, int64_t ldc, int M, int N, AccT (&acc)[FM][FN], int m0, int n0,
                                           int wm0, int wn0, int lane, const float *lds_scale) {
    using Out = typename OutOf<P, E>::type;
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    char *const wave_c = reinterpret_cast<char *>(C) +
                         ((int64_t)(m0 + wm0) * ldc + n0 + wn0) * (int64_t)sizeof(Out);
    const int64_t row_bytes = ldc * (int64_t)sizeof(Out);
    const uint32_t lane_off = (uint32_t)(4 * fhalf * row_bytes) + frow * (uint32_t)sizeof(Out);
    const bool interior = m0 + BM <= M && n0 + BN <= N;
    const int rows_left = M - (m0 + wm0) - 4 * fhalf;  // rows this lane may write: r < rows_left
    const int cols_left = N - (n0 + wn0) - frow;        // columns: j*32 < cols_left

    // this lane's scales: 4 consecutive rows per quarter of a 32-row
    // block (one 16-byte LDS read each), one column per column block
    float sb[!is_dequant(E) ? 1 : FN];
    if constexpr (is_dequant(E)) {
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j] = lds_scale[BM + wn0 + j * 32 + frow];
    }
    auto store_all = [&](auto &&keep) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            float4 sa[!is_dequant(E) ? 1 : 4];
            if constexpr (is_dequant(E)) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sa[q] = *reinterpret_cast<const float4 *>(&lds_scale[wm0 + i * 32 + 8 * q + 4 * fhalf]);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = i * 32 + 8 * (e >> 2) + (e & 3);   // wave-uniform part of the row
                char *const row_c = wave_c + r * row_bytes;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    Out v;
                    if constexpr (is_dequant(E)) {
                        // ((float)sum * scale_a) * scale_b, rounded once per step
                        // (on the FP6 cores the sum already is that binary32 value)
                        float c;
                        if constexpr (P == kF6)
                            c = acc[i][j][e];
                        else
                            c = (float)(P == kI4 ? acc[i][j][e] >> 8 : acc[i][j][e]);
                        const float4 a4 = sa[e >> 2];
                        c = c * ((e & 3) == 0 ? a4.x : (e & 3) == 1 ? a4.y : (e & 3) == 2 ? a4.z : a4.w);
                        c = c * sb[j];
                        // The binary16 result is the binary32 product rounded
                        // again.  The backend would otherwise fold product and
                        // narrowing into one mixed-precision FMA, which rounds
                        // once (and turns -0 into +0): the empty asm makes the
                        // binary32 value opaque to it.
                        if constexpr (E == kDequantF16) asm("" : "+v"(c));
                        v = (Out)c;
                    } else if constexpr (P == kI4) {
                        v = acc[i][j][e] >> 8;
                    } else if constexpr (P == kF6) {
                        v = (int32_t)acc[i][j][e];   // an integer below 2^24 in magnitude: exact
                    } else {
                        v = acc[i][j][e];
                    }
                    // non-temporal: C is not read again here, and
                    // streaming it past the MALL keeps A and B there
                    // for the later rounds of tiles
                    if (keep(r, j)) {
                        Out *const dst = reinterpret_cast<Out *>(row_c + lane_off + j * 32 * (int)sizeof(Out));
                        if constexpr (E == kAtomicAdd)
                            __hip_atomic_fetch_add(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        else
                            __builtin_nontemporal_store(v, dst);
                    }
                }
                // dequantized values are converted one row at a time
                if constexpr (is_dequant(E)) __builtin_amdgcn_sched_barrier(0);
            }
            // one row block at a time keeps accumulator reads from piling up
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (is_dequant(E)) {
        // one path: with two, more of the accumulators are copied out of
        // the accumulation registers ahead of the branch
        store_all([&](int r, int j) { return interior || (r < rows_left && j * 32 < cols_left); });
    } else if (interior) {
        store_all([](int, int) { return true; });
    } else {
        store_all([&](int r, int j) { return r < rows_left && j * 32 < cols_left; });
    }
}

// One workgroup computes a BM x BN block of C with (BM/WM) x (BN/WN) waves
// (times KS with a K split, whose waves share the block).
//
// K is consumed in K tiles of 64 bytes per row (32 f16, 64 int8 or 128
// packed int4 values); a k-step is 32 of those bytes.  A k-step reads one
// 16-byte fragment per lane for each of a wave's WM/32 row blocks of A and
// WN/32 column blocks of B (row = lane%32, 16-byte half = lane/32) and
// issues the MFMAs on them; fragments are read one k-step ahead.
//
// Whole-line staging (LS > 0, every tile but the 32 x 32 K-split one): a
// stage holds two K tiles, 128 bytes per row (with a K split: per row of
// each wave's own slice) in eight 16-byte chunks, logical chunk c of row r at
// position c ^ swizzle8(r); BM rows of A, then BN rows of B (a row-major B
// part holds the 2 * kKRows rows of B of the two K tiles as flat chunks,
// each row of B a whole number of lines).  Each DMA instruction of a wave
// writes 1 KB = 8 whole rows, lane l landing in row l/8 at position l%8, so
// each instruction reads whole 128-byte lines.  Stage s is fetched LS
// stages before it is consumed, four k-steps per stage; the one barrier of
// a stage comes after its last fragments are in registers, once this wave's
// DMA of stage s+1 has landed (stages s+2 .. s+LS-1 stay in flight), and a
// K-split wave, which reads only its own slice, needs no barrier.
//
// 64-byte staging (LS = 0, the 32 x 32 K-split tile): kStages stages, each
// with one 64-byte slice of KS x 64 bytes of K per row and wave; each DMA
// instruction of a wave writes 1 KB = 16 rows of its slice, lane l landing
// in row l/4 at position l%4 (logical chunk c of row r at position
// c ^ swizzle(r)).  Tile t lives in stage t % kStages and is fetched
// kStages tiles before it is consumed, two k-steps per tile; each wave
// waits only for its own DMA of tile t+1 (tiles t+2 .. t+kStages-1 stay in
// flight).  (The same path serves tiles without K split, with the stage
// rows spread over the waves and a barrier per tile.)
template <int P, int BM, int BN, int WM, int WN, int GM, int E, int BR, int KS, int LS>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * KS * kWave) void gemm_kernel(Args args) {
    // The body uses gfx950-only types (buffer resources), which the host
    // pass cannot type-check; the host pass only needs the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    using Acc = typename Prec<P>::Acc;
    using Out = typename OutOf<P, E>::type;
    static_assert(!is_dequant(E) || P != kF16, "the dequantizing epilogues are for the integer paths");
    static_assert(E != kAtomicAdd || KS == 1, "a K split across workgroups adds whole tiles");
    using RB = RowB<P>;
    constexpr int kCpr = BN / RB::kElemPerChunk;   // row-major B: 16-byte chunks per row of B
    static_assert(BR == kBCol || (kCpr >= 1 && (kCpr & (kCpr - 1)) == 0), "row-major B tile width");
    // KS > 1 splits K over the waves: each of the KS waves computes the whole
    // BM x BN tile over its own 64-byte quarter (KS = 4) of every K tile,
    // from its own slice of each stage, and the partial tiles are summed
    // through LDS in wave order at the end.
    constexpr int kWavesN = BN / WN;
    constexpr int NT = (BM / WM) * kWavesN;  // waves tiling the block
    constexpr int NW = NT * KS;              // waves in the workgroup
    constexpr int kSub = BM + BN;            // LDS rows of one K slice of a stage
    constexpr int kRows = KS * kSub;         // LDS rows per stage
    constexpr int kDma = KS > 1 ? kSub / 16 : kRows / 16 / NW;  // 1 KB DMA instructions per wave per stage
    constexpr int kDmaA = KS > 1 ? BM / 16 : BM / 16 / NW;      // ... of which fill A rows
    constexpr int kTileBytes = kRowBytes * KS;                  // bytes of K per row per K tile
    constexpr int FM = WM / 32;
    constexpr int FN = WN / 32;
    static_assert(KS > 1 || ((BM / 16) % NW == 0 && (BN / 16) % NW == 0), "stage rows must split evenly over waves");
    static_assert(KS == 1 || (NT == 1 && 16 % KS == 0), "the K-split variant computes the whole block tile per wave");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(kStages == 4, "the main loop is unrolled for four stages");
    static_assert((kStages - 2) * kDma <= 63, "vmcnt holds at most 63 outstanding loads");
    // whole-line staging: 8 rows of 128 bytes per DMA instruction (with a K
    // split, each wave stages its own 128-byte slice of every row)
    constexpr bool kLine = LS > 0;
    constexpr int kDmaL = KS > 1 ? kSub / 8 : kRows / 8 / NW;   // DMA instructions per wave per stage
    constexpr int kDmaLA = KS > 1 ? BM / 8 : BM / 8 / NW;       // ... of which fill A rows
    static_assert(!kLine || (KS > 1 ? BM % 8 == 0 && BN % 8 == 0 : BM % (8 * NW) == 0 && BN % (8 * NW) == 0),
                  "stage rows must split evenly over waves");
    static_assert(!kLine || BR == kBCol || 2 * RB::kKRows * kCpr == 8 * BN, "row-major B part of a whole-line stage");
    static_assert(!kLine || (LS == 2 || LS == 3), "the whole-line loop is unrolled for two or three stages");
    static_assert(!kLine || (LS - 1) * kDmaL <= 63, "vmcnt holds at most 63 outstanding loads");

    // The stages are separate objects so that the compiler can tell a DMA
    // into one from fragment reads of another (no false waits).  Only one of
    // the two sets is used.
    __shared__ uint4 lds0[kLine ? 1 : kRows][kChunks];
    __shared__ uint4 lds1[kLine ? 1 : kRows][kChunks];
    __shared__ uint4 lds2[kLine ? 1 : kRows][kChunks];
    __shared__ uint4 lds3[kLine ? 1 : kRows][kChunks];
    __shared__ uint4 ln0[kLine ? kRows : 1][2 * kChunks];
    __shared__ uint4 ln1[kLine ? kRows : 1][2 * kChunks];
    __shared__ uint4 ln2[kLine && LS > 2 ? kRows : 1][2 * kChunks];
    using Stage = uint4[kRows][kChunks];
    using LStage = uint4[kLine ? kRows : 1][2 * kChunks];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int slice = KS > 1 ? wave : 0;     // this wave's K slice
    const int twave = KS > 1 ? 0 : wave;     // this wave's place in the block tile
    const int M = args.M, N = args.N;
    // K split across workgroups: blockIdx.y picks the range of K this
    // workgroup sums (a whole number of stages in, so alignments hold)
    const int k_first = E == kAtomicAdd ? (int)blockIdx.y * args.kslice : 0;
    const int K = E == kAtomicAdd ? min(args.K - k_first, args.kslice) : args.K;
    const int64_t k_first_bytes = (int64_t)k_first * (P == kF16 ? 2 : 1) / (P == kI4 ? 2 : 1);
    const uint8_t *const op_a = args.A + k_first_bytes;
    const uint8_t *const op_b = args.B + (BR == kBRow ? (int64_t)k_first * args.ldb_bytes : k_first_bytes);

    // ---- block id -> tile, XCD-aware and banded by GM block rows ----
    int tile_m, tile_n;
    tile_of<GM>(args.tiles_m, args.tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    // ---- stage geometry ----
    // Each lane has one 32-bit offset per DMA instruction: its row (clamped to
    // the last valid row of A or B) times the leading dimension, plus its
    // chunk (and, with a K split, its wave's 64-byte slice).  K tile t is
    // addressed by a buffer resource based t * kTileBytes bytes further on
    // (row-major B: t * kKRows rows), whose range ends at the last 16-byte
    // chunk that holds data
    // of the last valid row: the hardware returns zeros for offsets outside
    // it without touching memory, so no DMA reads past an operand.  A range
    // of zero turns a stage past the last K tile into a no-op.
    const int valid = (P == kF16) ? 2 * K : (P == kI8 ? K : K / 2);  // data bytes per row
    const int n_tiles = (valid + kTileBytes - 1) / kTileBytes;
    const int valid16 = (valid + 15) & ~15;
    const uint8_t *a_base = op_a + (int64_t)m0 * args.lda_bytes;
    const int a_end = (int)((min(BM, M - m0) - 1) * args.lda_bytes) + valid16;
    // column-major B: like A, BN rows of K.  Row-major B: the tile's columns
    // start n0 values into every row of B; the range ends at the last chunk
    // of row K-1 that holds a column below N, so rows past K read as zeros.
    const int64_t b_col_bytes = (int64_t)n0 * (P == kF16 ? 2 : 1) / (P == kI4 ? 2 : 1);
    const uint8_t *b_base = op_b + (BR == kBRow ? b_col_bytes : (int64_t)n0 * args.ldb_bytes);
    // bytes of the last row of B that hold columns n0 .. N-1 (INT4: an odd
    // count of columns ends inside a byte, which still counts)
    const int64_t b_row_valid = ((int64_t)min(BN, N - n0) * (P == kF16 ? 16 : (P == kI8 ? 8 : 4)) + 7) / 8;
    const int64_t b_end = BR == kBRow ? (int64_t)(K - 1) * args.ldb_bytes + ((b_row_valid + 15) & ~int64_t(15))
                                      : (int64_t)(min(BN, N - n0) - 1) * args.ldb_bytes + valid16;
    // row-major B: a K tile is KS slices of kKRows rows of B.  A wave's
    // slice is addressed from a base of its own (its first row of B), so
    // that a lane's 32-bit offset spans at most kKRows rows (at most 512 MiB
    // with rows of 4 MiB) whatever the slice.
    const int64_t b_tile_bytes = BR == kBRow ? (int64_t)KS * RB::kKRows * args.ldb_bytes : kTileBytes;
    const int64_t b_slice_rows = BR == kBRow ? (int64_t)slice * RB::kKRows * args.ldb_bytes : 0;
    const int lrow = lane >> 2;              // row within the 16-row group
    const int lpos = lane & 3;               // LDS position written by this lane
    uint32_t voff[kDma];
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
        // row within the stage (KS > 1: within this wave's slice, which
        // starts a multiple of 16 rows in, so the swizzle is the same)
        const int cr = KS > 1 ? j * 16 + lrow : (j * NW + wave) * 16 + lrow;
        const int lchunk = lpos ^ swizzle(cr);       // logical chunk this lane fetches
        const int kofs = slice * kRowBytes;          // this wave's bytes of the K tile
        if (j < kDmaA) {
            voff[j] = (uint32_t)((min(m0 + cr, M - 1) - m0) * args.lda_bytes) + lchunk * 16 + kofs;
        } else if (BR == kBCol) {
            voff[j] = (uint32_t)((min(n0 + cr - BM, N - 1) - n0) * args.ldb_bytes) + lchunk * 16 + kofs;
        } else {
            // flat chunk f of the B part: row f / kCpr, position f % kCpr
            // (K split: of this wave's slice, kKRows rows further on per slice)
            const int f = (cr - BM) * kChunks + lpos;
            const int krow = f / kCpr;
            const int gchunk = (f % kCpr) ^ bswizzle<P, BN>(krow);
            voff[j] = (uint32_t)(krow * args.ldb_bytes) + gchunk * 16;
        }
    }

    auto stage = [&](int t, Stage &buf) __attribute__((always_inline)) {
        const int kb = t * kTileBytes;
        const bool live = t < n_tiles;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a_base + kb), (short)0, live ? a_end - kb : 0, kRsrcWord3);
        const int64_t bt = (int64_t)t * b_tile_bytes + b_slice_rows;
        // a row-major slice spans kKRows rows of B; the range never exceeds
        // it (nor 2^31 - 1: every offset a lane forms is below that), and is
        // zero for a slice that starts past row K - 1
        const int b_range = !live ? 0
                            : BR == kBRow ? (int)max(min(min(b_end - bt, (int64_t)RB::kKRows * args.ldb_bytes),
                                                         (int64_t)INT32_MAX), (int64_t)0)
                                          : (int)(b_end - bt);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(b_base + bt), (short)0, b_range, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < kDma; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(j < kDmaA ? ra : rb,
                                                     LDS_PTR(&buf[KS > 1 ? slice * kSub + j * 16
                                                                          : (j * NW + wave) * 16][0]),
                                                     16, voff[j], 0, 0, 0);
    };

    const int wm0 = (twave / kWavesN) * WM;  // wave's first row / column in the block tile
    const int wn0 = (twave % kWavesN) * WN;
    const int srow = slice * kSub;           // first LDS row of this wave's K slice
    const int frow = lane & 31;              // fragment row (A) / column (B) of this lane
    const int fhalf = lane >> 5;             // which 16-byte half of a 32-byte k-step

    // Row-major B: lane i of a 16-lane group points its transposing read at
    // row kb + i / Q, bytes 8 * (i % Q) of its Q chunks, and receives the R
    // values of column (group base + i) in rows kb .. kb + R - 1; two reads
    // make one 16-byte fragment.  Per lane constants:
    const int tr_i = lane & 15;
    const int tr_row = tr_i / RB::kQ;                 // row within a read
    const int tr_byte = 8 * (tr_i % RB::kQ);          // byte within the lane's chunks
    const int tr_col_bytes = (16 * ((lane >> 4) & 1)) * (P == kF16 ? 2 : 1) / (P == kI4 ? 2 : 1);
    // (bpart: the B part of a stage; s: the k-step within it)
    auto read_b_rm = [&](const char *bpart, int s, int j) __attribute__((always_inline)) {
        // bytes of K per k-step are 32: 16 f16, 32 int8 or 64 int4 rows, half per lane half
        constexpr int kStepRows = RB::kKRows / 2;
        const int col_bytes = ((wn0 + j * 32) * (P == kF16 ? 2 : 1) / (P == kI4 ? 2 : 1)) + tr_col_bytes + tr_byte;
        uint32_t w[4];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int krow = s * kStepRows + fhalf * (kStepRows / 2) + r * RB::kR + tr_row;
            const int pos = (col_bytes >> 4) ^ bswizzle<P, BN>(krow);
            const char *p = bpart + (krow * kCpr + pos) * 16 + (col_bytes & 15);
            if constexpr (P == kF16) {
                typedef short v4s __attribute__((ext_vector_type(4)));
                const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s *)(p));
                __builtin_memcpy(&w[2 * r], &v, 8);
            } else if constexpr (P == kI8) {
                const intx2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) intx2_t *)(p));
                __builtin_memcpy(&w[2 * r], &v, 8);
            } else {
                const intx2_t v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                    (__attribute__((address_space(3))) intx2_t *)(p));
                __builtin_memcpy(&w[2 * r], &v, 8);
            }
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    };
    auto read_b_rowmajor = [&](const Stage &buf, int s, int j) __attribute__((always_inline)) {
        return read_b_rm(reinterpret_cast<const char *>(&buf[srow + BM][0]), s, j);
    };

    auto read_frags = [&](const Stage &buf, int s, uint4 (&fa)[FM], uint4 (&fb)[FN]) __attribute__((always_inline)) {
        const int ch = (2 * s + fhalf) ^ swizzle(frow);  // fragment rows start at multiples of 32
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = buf[srow + wm0 + i * 32 + frow][ch];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (BR == kBCol)
                fb[j] = buf[srow + BM + wn0 + j * 32 + frow][ch];
            else
                fb[j] = read_b_rowmajor(buf, s, j);
        }
    };

    // Zero the bytes of this lane's fragments of K tile t, k-step s, that lie
    // at or beyond K (the last tile may be partial; what DMA left there is
    // either zeros or bytes of the row's padding).
    auto mask_frags = [&](int t, int s, uint4 (&fa)[FM], uint4 (&fb)[FN]) __attribute__((always_inline)) {
        const int nb = valid - (t * kTileBytes + slice * kRowBytes + (2 * s + fhalf) * 16);
        uint32_t m[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int r = nb - 4 * d;
            m[d] = r >= 4 ? 0xFFFFFFFFu : (r <= 0 ? 0u : (1u << (8 * r)) - 1u);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            fa[i].x &= m[0];
            fa[i].y &= m[1];
            fa[i].z &= m[2];
            fa[i].w &= m[3];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            fb[j].x &= m[0];
            fb[j].y &= m[1];
            fb[j].z &= m[2];
            fb[j].w &= m[3];
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    auto mma = [&](const uint4 (&fa)[FM], const uint4 (&fb)[FN]) __attribute__((always_inline)) {
        if constexpr (P == kF16) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_f16(fa[i], fb[j], acc[i][j]);
        } else if constexpr (P == kI8) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_i8(fa[i], fb[j], acc[i][j]);
        } else {
            // planes of all B fragments, then one A fragment at a time; the
            // even and odd products of one accumulator are FN MFMAs apart
            uint4 eb[FN], ob[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) split_s4<kLine>(fb[j], eb[j], ob[j]);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                uint4 ea, oa;
                split_s4<kLine>(fa[i], ea, oa);
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_i8(ea, eb[j], acc[i][j]);
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_i8(oa, ob[j], acc[i][j]);
            }
        }
    };

    uint4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];

    // Issue order of a k-step: its MFMAs with the next fragment reads (and,
    // after the barrier, the DMA of a later tile) slotted one by one between
    // them, so that no burst of memory instructions holds up MFMA issue.
    constexpr int kMfma = FM * FN * (P == kI4 ? 2 : 1);   // MFMAs per k-step
    constexpr int kReads = FM + FN * (BR == kBRow ? 2 : 1);   // LDS reads per k-step
    // VALU per k-step: the INT4 plane split (12 per fragment in the 32-bit
    // form, 10 in the 64-bit one; the slots are sized for 12 in both, as
    // timed) and the row-major B read addresses (about 3 per read)
    constexpr int kValuWork = (P == kI4 ? 12 * (FM + FN) : 0) + (BR == kBRow ? 6 * FN : 0);
    constexpr int kValu = (kValuWork + kMfma - 1) / kMfma;
    // (whole-line staging issues a stage's DMA after its last barrier,
    // several per MFMA when there are more DMAs than MFMAs)
    auto interleave = [&](auto dma_count) __attribute__((always_inline)) {
        constexpr int dma = decltype(dma_count)::value;
        constexpr int per = kLine && dma > kMfma ? (dma + kMfma - 1) / kMfma : 1;
#pragma unroll
        for (int i = 0; i < kMfma; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // 1 MFMA
            if (i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
            if (i * per < dma) __builtin_amdgcn_sched_group_barrier(0x020, per, 0);  // VMEM (DMA)
            if (kValu) __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU (planes)
        }
    };
    using NoDma = std::integral_constant<int, 0>;

    // K tile t (not the last) from stage `cur`, whose first fragments are in
    // fa0/fb0; refills `cur` with tile t+kStages (a no-op past the last tile)
    // and reads tile t+1's first fragments from `next`.
    auto tile = [&](Stage &cur, const Stage &next, int t) __attribute__((always_inline)) {
        read_frags(cur, 1, fa1, fb1);
        mma(fa0, fb0);
        interleave(NoDma{});
        // this wave's DMA of tile t+1 has landed (only tiles t+2 .. t+3 may
        // still be in flight) and its reads of `cur` are done; after the
        // barrier the same holds for every wave
        // (KS > 1: every wave reads only its own slice, so its own waits suffice)
        if constexpr (KS > 1)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((kStages - 2) * kDma) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((kStages - 2) * kDma) : "memory");
        stage(t + kStages, cur);
        read_frags(next, 0, fa0, fb0);
        mma(fa1, fb1);
        interleave(std::integral_constant<int, kDma>{});
        __builtin_amdgcn_sched_barrier(0);
    };

    // the last K tile, with the bytes at or beyond K masked off
    auto last_tile = [&](const Stage &cur, int t) __attribute__((always_inline)) {
        mask_frags(t, 0, fa0, fb0);
        read_frags(cur, 1, fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        mma(fa0, fb0);
        mask_frags(t, 1, fa1, fb1);
        mma(fa1, fb1);
    };

    // Dequantizing epilogue: the block tile's row scales (BM entries) and
    // column scales (BN entries) are staged in LDS once; rows and columns
    // past the edge take the last valid scale (their results are not
    // stored).  The loads are issued before the first DMAs and written to
    // LDS after them; the first barrier makes them visible.
    constexpr int kThreads = NW * kWave;
    constexpr int kScaleLoads = !is_dequant(E) ? 0 : (BM + BN + kThreads - 1) / kThreads;
    __shared__ __align__(16) float lds_scale[!is_dequant(E) ? 1 : BM + BN];
    float scale_v[kScaleLoads + 1];
#pragma unroll
    for (int x = 0; x < kScaleLoads; ++x) {
        const int idx = tid + x * kThreads;
        if (idx < BM + BN)
            scale_v[x] = idx < BM ? args.scale_a[min(m0 + idx, M - 1)] : args.scale_b[min(n0 + idx - BM, N - 1)];
    }

    if constexpr (kLine) {
        // ---- whole-line staging ----
        constexpr int kLineBytes = 2 * kRowBytes;         // bytes of K per row and wave slice
        constexpr int kStageK = KS * kLineBytes;           // bytes of K per row per stage
        const int n_st = (valid + kStageK - 1) / kStageK;  // stages of two K tiles
        // lane offsets: instruction j of this wave fills stage rows
        // (j*NW + wave)*8 .. +7 (K split: rows j*8 .. +7 of its own slice);
        // lane l fetches logical chunk (l%8) ^ swizzle8(row) of row (l/8),
        // rows clamped as above.  Row-major B: the B part of a stage (of a
        // slice) holds the 2 * kKRows rows of B of its two K tiles as flat
        // 16-byte chunks (as in a 64-byte stage), so lane l of a B
        // instruction fills flat chunk f = l of its 1 KB.
        const int kofs = slice * kLineBytes;               // this wave's bytes of a stage's K
        uint32_t voffl[kDmaL];
#pragma unroll
        for (int j = 0; j < kDmaL; ++j) {
            const int blk = KS > 1 ? j : j * NW + wave;    // 1 KB block of the stage (slice)
            const int cr = blk * 8 + (lane >> 3);
            const int lchunk = (lane & 7) ^ swizzle8(cr);
            if (j < kDmaLA) {
                voffl[j] = (uint32_t)((min(m0 + cr, M - 1) - m0) * args.lda_bytes) + lchunk * 16 + kofs;
            } else if constexpr (BR == kBCol) {
                voffl[j] = (uint32_t)((min(n0 + cr - BM, N - 1) - n0) * args.ldb_bytes) + lchunk * 16 + kofs;
            } else {
                const int f = (blk - BM / 8) * 64 + lane;
                const int krow = f / kCpr;
                const int gchunk = (f % kCpr) ^ bswizzle<P, BN>(krow);
                voffl[j] = (uint32_t)(krow * args.ldb_bytes) + gchunk * 16;
            }
        }
        // row-major B: a stage spans KS * 2 * kKRows rows of B, a wave's
        // slice 2 * kKRows of them, from a base of its own (as above)
        const int64_t b_stage_bytes = BR == kBRow ? (int64_t)KS * 2 * RB::kKRows * args.ldb_bytes : kStageK;
        const int64_t b_slice_bytes = (int64_t)2 * RB::kKRows * args.ldb_bytes;
        auto stage_l = [&](int st, LStage &buf) __attribute__((always_inline)) {
            const int kb = st * kStageK;
            const bool live = st < n_st;
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a_base + kb), (short)0, live ? a_end - kb : 0, kRsrcWord3);
            const int64_t bt = (int64_t)st * b_stage_bytes + (BR == kBRow ? slice * b_slice_bytes : 0);
            const int b_range = !live ? 0
                                : BR == kBRow ? (int)max(min(min(b_end - bt, b_slice_bytes), (int64_t)INT32_MAX),
                                                         (int64_t)0)
                                              : (int)(b_end - bt);
            const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(b_base + bt), (short)0, b_range, kRsrcWord3);
#pragma unroll
            for (int j = 0; j < kDmaL; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(j < kDmaLA ? ra : rb,
                                                         LDS_PTR(&buf[KS > 1 ? srow + j * 8 : (j * NW + wave) * 8][0]),
                                                         16, voffl[j], 0, 0, 0);
        };
        // fragments of k-step q (0..3) of a stage: logical chunk 2q + half
        auto read_l = [&](const LStage &buf, int q, uint4 (&fa)[FM], uint4 (&fb)[FN]) __attribute__((always_inline)) {
            const int ch = (2 * q + fhalf) ^ swizzle8(frow);   // fragment rows start at multiples of 32
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = buf[srow + wm0 + i * 32 + frow][ch];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (BR == kBCol)
                    fb[j] = buf[srow + BM + wn0 + j * 32 + frow][ch];
                else
                    fb[j] = read_b_rm(reinterpret_cast<const char *>(&buf[srow + BM][0]), q, j);
            }
        };
        // zero the bytes of k-step q of stage st at or beyond K
        auto mask_l = [&](int st, int q, uint4 (&fa)[FM], uint4 (&fb)[FN]) __attribute__((always_inline)) {
            const int nb = valid - (st * kStageK + kofs + (2 * q + fhalf) * 16);
            uint32_t m[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int r = nb - 4 * d;
                m[d] = r >= 4 ? 0xFFFFFFFFu : (r <= 0 ? 0u : (1u << (8 * r)) - 1u);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                fa[i].x &= m[0];
                fa[i].y &= m[1];
                fa[i].z &= m[2];
                fa[i].w &= m[3];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                fb[j].x &= m[0];
                fb[j].y &= m[1];
                fb[j].z &= m[2];
                fb[j].w &= m[3];
            }
        };
        // stage st (not the last) from `cur`, whose first fragments are in
        // fa0/fb0; refills `cur` with stage st+LS and reads the first
        // fragments of stage st+1 from `nxt`
        auto full_stage = [&](LStage &cur, const LStage &nxt, int st) __attribute__((always_inline)) {
            read_l(cur, 1, fa1, fb1);
            mma(fa0, fb0);
            interleave(NoDma{});
            read_l(cur, 2, fa0, fb0);
            mma(fa1, fb1);
            interleave(NoDma{});
            read_l(cur, 3, fa1, fb1);
            mma(fa0, fb0);
            interleave(NoDma{});
            // this wave's DMA of stage st+1 has landed and its reads of `cur`
            // are done; after the barrier the same holds for every wave
            // (K split: every wave reads only its own slice)
            if constexpr (KS > 1)
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((LS - 2) * kDmaL) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((LS - 2) * kDmaL) : "memory");
            stage_l(st + LS, cur);
            read_l(nxt, 0, fa0, fb0);
            mma(fa1, fb1);
            interleave(std::integral_constant<int, kDmaL>{});
            __builtin_amdgcn_sched_barrier(0);
        };
        // the last stage, with the bytes at or beyond K masked off
        auto last_stage = [&](const LStage &cur, int st) __attribute__((always_inline)) {
            read_l(cur, 1, fa1, fb1);
            mask_l(st, 0, fa0, fb0);
            mma(fa0, fb0);
            read_l(cur, 2, fa0, fb0);
            mask_l(st, 1, fa1, fb1);
            mma(fa1, fb1);
            read_l(cur, 3, fa1, fb1);
            mask_l(st, 2, fa0, fb0);
            mma(fa0, fb0);
            mask_l(st, 3, fa1, fb1);
            mma(fa1, fb1);
        };
        if (n_st > 0) {
            stage_l(0, ln0);
            stage_l(1, ln1);
            if constexpr (LS > 2) stage_l(2, ln2);
#pragma unroll
            for (int x = 0; x < kScaleLoads; ++x)
                if (tid + x * kThreads < BM + BN) lds_scale[tid + x * kThreads] = scale_v[x];
            if constexpr (KS > 1)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"((LS - 1) * kDmaL) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((LS - 1) * kDmaL) : "memory");
            read_l(ln0, 0, fa0, fb0);
            int st = 0;
            if constexpr (LS == 2) {
                for (; st + 2 < n_st; st += 2) {
                    full_stage(ln0, ln1, st);
                    full_stage(ln1, ln0, st + 1);
                }
                if (st + 1 < n_st) full_stage(ln0, ln1, st++);
                last_stage((st & 1) ? ln1 : ln0, st);
            } else {
                for (; st + 3 < n_st; st += 3) {
                    full_stage(ln0, ln1, st);
                    full_stage(ln1, ln2, st + 1);
                    full_stage(ln2, ln0, st + 2);
                }
                // 1 to 3 stages remain, the first of them in ln0
                if (st + 1 < n_st) {
                    full_stage(ln0, ln1, st++);
                    if (st + 1 < n_st) full_stage(ln1, ln2, st++);
                }
                const int r = st % 3;
                last_stage(r == 0 ? ln0 : r == 1 ? ln1 : ln2, st);
            }
            // no DMA may still be writing this workgroup's LDS when it exits
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else if constexpr (is_dequant(E)) {
            // K == 0: no main loop, so stage the scales here
#pragma unroll
            for (int x = 0; x < kScaleLoads; ++x)
                if (tid + x * kThreads < BM + BN) lds_scale[tid + x * kThreads] = scale_v[x];
            __syncthreads();
        }
    } else {
        if (n_tiles > 0) {
            stage(0, lds0);
            stage(1, lds1);
            stage(2, lds2);
            stage(3, lds3);
    #pragma unroll
            for (int x = 0; x < kScaleLoads; ++x)
                if (tid + x * kThreads < BM + BN) lds_scale[tid + x * kThreads] = scale_v[x];
            if constexpr (KS > 1)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kStages - 1) * kDma) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((kStages - 1) * kDma) : "memory");
            read_frags(lds0, 0, fa0, fb0);
            int t = 0;
            for (; t + kStages < n_tiles; t += kStages) {
                tile(lds0, lds1, t);
                tile(lds1, lds2, t + 1);
                tile(lds2, lds3, t + 2);
                tile(lds3, lds0, t + 3);
            }
            // 1 to 4 tiles remain, the first of them in lds0
            if (t + 1 < n_tiles) {
                tile(lds0, lds1, t++);
                if (t + 1 < n_tiles) {
                    tile(lds1, lds2, t++);
                    if (t + 1 < n_tiles) tile(lds2, lds3, t++);
                }
            }
            const int last = t & 3;
            last_tile(last == 0 ? lds0 : last == 1 ? lds1 : last == 2 ? lds2 : lds3, t);
            // no DMA may still be writing this workgroup's LDS when it exits
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else if constexpr (is_dequant(E)) {
            // K == 0: no main loop, so stage the scales here
    #pragma unroll
            for (int x = 0; x < kScaleLoads; ++x)
                if (tid + x * kThreads < BM + BN) lds_scale[tid + x * kThreads] = scale_v[x];
            __syncthreads();
        }

    }

    // ---- K-split epilogue: sum the partial tiles, then store ----
    // Stage 0 is free once every wave has drained its own DMAs.  One 32 x 32
    // MFMA block at a time, each wave writes its 16 accumulators per lane
    // there; wave w then sums registers kPer*w .. kPer*w + kPer-1 over the KS
    // partials in wave order (a fixed order, so fp32 results do not vary
    // between runs) and stores them: with KS = 4 that is rows 8w .. 8w+7 of
    // the block.
    if constexpr (KS > 1) {
        using Sc = typename Prec<P>::Out;    // the sums (int32 or fp32)
        constexpr int kPer = 16 / KS;
        constexpr size_t kStage0Bytes = kLine ? sizeof(ln0) : sizeof(lds0);
        static_assert(kStage0Bytes >= KS * 16 * kWave * sizeof(Sc), "partials of a block fit in one stage");
        Sc *const part = kLine ? reinterpret_cast<Sc *>(&ln0[0][0]) : reinterpret_cast<Sc *>(&lds0[0][0]);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                __syncthreads();   // stage 0 free: main loop, or the previous block, done
#pragma unroll
                for (int e = 0; e < 16; ++e) part[(wave * 16 + e) * kWave + lane] = acc[i][j][e];
                __syncthreads();
                const int rows_left = M - m0 - i * 32 - 4 * fhalf;
                const bool col_ok = j * 32 + frow < N - n0;
                char *const c_lane = reinterpret_cast<char *>(args.C) +
                                     ((int64_t)(m0 + i * 32 + 4 * fhalf) * args.ldc + n0 + j * 32 + frow) *
                                         (int64_t)sizeof(Out);
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    const int e = wave * kPer + u;
                    Sc v = part[e * kWave + lane];
#pragma unroll
                    for (int w = 1; w < KS; ++w) v += part[(w * 16 + e) * kWave + lane];
                    if constexpr (P == kI4) v >>= 8;
                    const int r = 8 * (e >> 2) + (e & 3);   // row in the block, less 4*(l/32)
                    Out o;
                    if constexpr (is_dequant(E)) {
                        // ((float)sum * scale_a) * scale_b, one rounding per step,
                        // then (binary16 output) narrowed as a separate step
                        float c = (float)v;
                        c = c * lds_scale[i * 32 + r + 4 * fhalf];
                        c = c * lds_scale[BM + j * 32 + frow];
                        if constexpr (E == kDequantF16) asm("" : "+v"(c));
                        o = (Out)c;
                    } else {
                        o = v;
                    }
                    if (col_ok && r < rows_left)
                        *reinterpret_cast<Out *>(c_lane + (int64_t)r * args.ldc * (int64_t)sizeof(Out)) = o;
                }
            }
        }
    }

    // ---- epilogue: 32x32 MFMA result layout -> row-major C ----
    if constexpr (KS == 1)
        store_tile<P, E, BM, BN, FM, FN>(args.C, args.ldc, M, N, acc, m0, n0, wm0, wn0, lane, lds_scale);
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// INT4 on the FP6 matrix cores
//
// gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies 6-bit e2m3 values
// (1 sign, 2 exponent bits of bias 1, 3 mantissa bits) at about twice the
// rate of the INT8 MFMA.  Every INT4 value v in [-8, 7] is exact in e2m3 as
// v / 8: |v| = 0..7 are the subnormals m / 8 (exponent 0, mantissa m) and
// |v| = 8 is 1.0 (exponent 1, mantissa 0), so the 6-bit code of v / 8 is
// sign << 5 | |v|.  Each operand carries the block scale 2^3 (E8M0 code
// 130), so an MFMA adds the exact integer products a * b, and the fp32
// accumulators hold exact integers: |C| <= 64 K < 2^24 for K <= 131071.
// One MFMA covers 64 values of K per output, where the INT8 path needs two
// (one per nibble plane), and the main loop holds no unpacking.
//
// The cost is the format: 32 values take 24 bytes (six registers) per lane,
// and turning nibbles into 6-bit codes takes about three VALU operations per
// value.  Done per fragment in the main loop, that would cost more than the
// MFMAs, because every operand row is read by many workgroups.  So a
// pre-pass (f6_pack_kernel) converts each operand once into a workspace
// "image", and the GEMM (gemm_f6_kernel) stages the image with straight
// 1 KB DMA copies.
//
// Image layout.  Rows (of A, or columns of B) come in groups of 32 and K in
// blocks of 128 values; unit (g, b) of an operand is 3072 bytes at offset
// (g * nkb + b) * 3072, nkb = ceil(K / 128).  A unit holds, for each row r
// of the group and each k-step s (64 values) and lane half h (32 values,
// as the MFMA takes them: lane (row, h) holds k = 64 s + 32 h + e), the six
// code words of those 32 values: words 0-3 ("main", 16 bytes) and words 4-5
// ("tail", 8 bytes).
//   main part, bytes 0 .. 2047:    row r at 64 r, logical chunk c = 2 s + h
//                                  at 16-byte position c ^ swizzle(r)
//   tail part, bytes 2048 .. 3071: row r at 2048 + 32 r, logical slot
//                                  c = 2 s + h at 8-byte position
//                                  c ^ tswizzle(r)
// A GEMM stage is one K block: the units of the tile's row groups, copied
// as they are into LDS (main parts as 64-byte rows, tail parts as 32-byte
// rows).  Rows past M (N) and values past K are zero codes in the image, so
// the GEMM needs no masking; groups past the image read as zeros through the
// buffer range.  Within the 32 values of a fragment the pre-pass orders the
// codes as its SWAR arithmetic leaves them (the even k of each dword, then
// the odd ones); A and B use the same order, so the MFMA still pairs equal k.

// 8-byte tail slot positions: the 32 lanes of a half-wave read 32 rows at
// one logical slot; with 64 banks, row r at position p covers banks
// 8 (r % 8) + 2 p .. + 1, so rows r and r + 8 j must differ in p.
__device__ __forceinline__ int tswizzle(int r) { return (r >> 3) & 3; }

// four 6-bit codes, one per byte (bits 0-5), packed into bits 0 .. 23
__device__ __forceinline__ uint32_t pack4_codes(uint32_t x) {
    const uint32_t z = (x & 0x00FF00FFu) | ((x & 0xFF00FF00u) >> 2);   // codes at bits 0, 6, 16, 22
    return (z & 0xFFFu) | ((z >> 4) & 0xFFF000u);                        // ... at 0, 6, 12, 18
}

// 8 two's complement nibbles -> the e2m3 codes of their values / 8: those of
// the even nibbles in lo (bits 0 .. 23), of the odd ones in hi.
__device__ __forceinline__ void s4_to_e2m3(uint32_t w, uint32_t &lo, uint32_t &hi) {
    const uint32_t t = w & 0x88888888u;      // sign bits
    const uint32_t s1 = t >> 3;              // 1 in each negative nibble
    const uint32_t neg = (t << 1) - s1;      // 0xF in each negative nibble (no carries across)
    const uint32_t mag = (w ^ neg) + s1;     // |v| per nibble, 0 .. 8 (16 - n for a negative n)
    const uint32_t e = (mag & 0x0F0F0F0Fu) | ((t << 2) & 0x20202020u);          // sign to bit 5
    const uint32_t o = ((mag >> 4) & 0x0F0F0F0Fu) | ((t >> 2) & 0x20202020u);
    lo = pack4_codes(e);
    hi = pack4_codes(o);
}

// 32 packed INT4 values (16 bytes) -> their six code words (192 bits: eight
// 24-bit groups of four codes, dense)
__device__ __forceinline__ void fragment_to_e2m3(const uint4 &w, uint4 &main, uint2 &tail) {
    uint32_t p[8];
    s4_to_e2m3(w.x, p[0], p[1]);
    s4_to_e2m3(w.y, p[2], p[3]);
    s4_to_e2m3(w.z, p[4], p[5]);
    s4_to_e2m3(w.w, p[6], p[7]);
    main.x = p[0] | (p[1] << 24);
    main.y = (p[1] >> 8) | (p[2] << 16);
    main.z = (p[2] >> 16) | (p[3] << 8);
    main.w = p[4] | (p[5] << 24);
    tail.x = (p[5] >> 8) | (p[6] << 16);
    tail.y = (p[6] >> 16) | (p[7] << 8);
}

constexpr int kF6Block = 128;    // K values per image unit and per GEMM stage
constexpr int kF6Unit = 3072;    // bytes per unit: 32 rows x (64 main + 32 tail)
constexpr int kF6Main = 2048;    // bytes of the main part of a unit
constexpr int kF6Scale = 130;    // E8M0 block scale 2^3 (bias 127)

// One operand of the pre-pass.
struct F6Operand {
    const uint8_t *src;   // packed INT4
    uint8_t *img;         // the image
    int64_t ld_bytes;     // row stride of src
    int rows;             // rows of the image (M for A, N for B)
    int groups;           // ceil(rows / 32)
    int rowmajor;         // B only: src is K x N packed along N (row-major B)
};

struct F6PackArgs {
    F6Operand op[2];      // A, B
    int K, nkb;
    int blocks_a;         // workgroups of A; the rest convert B
};

// The pre-pass: one wave per unit (four per workgroup), lane (r, h) = (lane
// % 32, lane / 32) converting the 2 x 32 values of row r, half h of the
// unit's two k-steps.  K-contiguous rows (A, column-major B) are read as
// 16-byte chunks; a row-major B tile (128 rows of K x 32 columns) is first
// copied to LDS and each lane gathers its column from there.
__global__ __launch_bounds__(256) void f6_pack_kernel(F6PackArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ uint8_t tile_s[4][kF6Block][16];   // row-major B: K rows x 32 nibbles, per wave
    const int which = blockIdx.x < args.blocks_a ? 0 : 1;
    const F6Operand &op = args.op[which];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)(blockIdx.x - (which ? args.blocks_a : 0)) * 4 + wave;
    if (unit >= (int64_t)op.groups * args.nkb) return;
    const int g = (int)(unit / args.nkb);
    const int b = (int)(unit - (int64_t)g * args.nkb);
    const int r = lane & 31, h = lane >> 5;
    const int K = args.K;
    uint8_t *const dst = op.img + unit * kF6Unit;
    uint4 w[2];
    if (!op.rowmajor) {
        const int row = g * 32 + r;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int k0 = b * kF6Block + s * 64 + h * 32;   // first value of the fragment
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row < op.rows && k0 < K) {
                v = *reinterpret_cast<const uint4 *>(op.src + (int64_t)row * op.ld_bytes + k0 / 2);
                const int nb = (K - k0) / 2;   // valid bytes (K is even)
                if (nb < 16) {
                    uint32_t m[4];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int q = nb - 4 * d;
                        m[d] = q >= 4 ? 0xFFFFFFFFu : (q <= 0 ? 0u : (1u << (8 * q)) - 1u);
                    }
                    v.x &= m[0];
                    v.y &= m[1];
                    v.z &= m[2];
                    v.w &= m[3];
                }
            }
            w[s] = v;
        }
    } else {
        // 128 rows of K (b * 128 ..) x 32 columns (g * 32 ..) = 16 bytes per row;
        // lane l copies rows l and l + 64 (zeros past K), nibbles past N zeroed
        const int cbyte = g * 16;
        const int valid_nib = min(op.rows - g * 32, 32);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int kr = lane + 64 * x;
            const int k = b * kF6Block + kr;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (k < K) {
                v = *reinterpret_cast<const uint4 *>(op.src + (int64_t)k * op.ld_bytes + cbyte);
                if (valid_nib < 32) {
                    uint32_t m[4];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int q = valid_nib - 8 * d;   // valid nibbles in this dword
                        m[d] = q >= 8 ? 0xFFFFFFFFu : (q <= 0 ? 0u : (1u << (4 * q)) - 1u);
                    }
                    v.x &= m[0];
                    v.y &= m[1];
                    v.z &= m[2];
                    v.w &= m[3];
                }
            }
            *reinterpret_cast<uint4 *>(&tile_s[wave][kr][0]) = v;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        // column r: nibble r % 2 of byte r / 2 of each row; fragment s holds
        // rows 64 s + 32 h .. + 31, two per byte, the lower row in the low nibble
        const int sh = 4 * (r & 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint32_t d[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t acc = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kr = s * 64 + h * 32 + q * 8 + e;
                    acc |= (uint32_t)((tile_s[wave][kr][r >> 1] >> sh) & 0xF) << (4 * e);
                }
                d[q] = acc;
            }
            w[s] = make_uint4(d[0], d[1], d[2], d[3]);
        }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        uint4 m;
        uint2 t;
        fragment_to_e2m3(w[s], m, t);
        const int c = 2 * s + h;
        *reinterpret_cast<uint4 *>(dst + r * 64 + 16 * (c ^ swizzle(r))) = m;
        *reinterpret_cast<uint2 *>(dst + kF6Main + r * 32 + 8 * (c ^ tswizzle(r))) = t;
    }
#endif
}

struct F6Args {
    const uint8_t *A;     // images
    const uint8_t *B;
    void *C;
    const float *scale_a;
    const float *scale_b;
    int64_t a_bytes;      // image sizes
    int64_t b_bytes;
    int64_t ldc;
    int M, N, nkb;
    int tiles_m, tiles_n;
};

// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// An FP6 fragment: the six code words of a lane.  The MFMA builtin takes
// eight registers per operand and reads the first six for e2m3.
typedef int intx6_t __attribute__((ext_vector_type(6)));
typedef int intx8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx16_t mfma_f6(const intx6_t &a, const intx6_t &b, const floatx16_t &c) {
    const intx8_t a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, 4, 5, -1, -1);
    const intx8_t b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, -1, -1);
    // formats 2, 2: e2m3 for both operands; block scales 2^3 each
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 2, 2, 0, kF6Scale, 0, kF6Scale);
}

// The GEMM on the images: a BM x BN block of C per workgroup of
// (BM/WM) x (BN/WN) waves, each wave a WM x WN sub-block of 32 x 32 MFMA
// blocks.  Three LDS stages, each one K block (two k-steps) of the tile's
// A and B units; stage st is fetched three stages before it is consumed,
// one barrier per stage, after this wave's DMA of stage st+1 has landed.
// Launch bounds: two waves per SIMD (8-wave tiles, or two 4-wave workgroups
// per CU), except for the 128 x 128 wave tile, whose 256 accumulators take a
// SIMD's registers for one wave.
template <int BM, int BN, int WM, int WN, int GM, int E, int LA>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave, WM * WN >= 128 * 128 ? 1 : 2) void
gemm_f6_kernel(F6Args args) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NW = (BM / WM) * (BN / WN);
    constexpr int kWavesN = BN / WN;
    constexpr int FM = WM / 32;
    constexpr int FN = WN / 32;
    constexpr int kRows = BM + BN;             // LDS rows of a stage (main: 64 B, tail: 32 B)
    constexpr int kUnitsA = BM / 32;
    constexpr int kDma = 3 * (kRows / 32) / NW;  // 1 KB copies per wave per stage
    static_assert(3 * (kRows / 32) % NW == 0, "a stage's copies must split evenly over the waves");
    static_assert(kDma <= 31, "vmcnt holds at most 63 outstanding loads");
    static_assert(LA >= 1 && LA <= FM, "A fragments are read 1 .. FM row blocks ahead");
    using Stage = uint4[kRows][4];
    using Tail = uint2[kRows][4];
    __shared__ uint4 mn0[kRows][4], mn1[kRows][4], mn2[kRows][4];
    __shared__ uint2 tl0[kRows][4], tl1[kRows][4], tl2[kRows][4];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int M = args.M, N = args.N, nkb = args.nkb;

    // band order: the operands are the images the pre-pass has just written,
    // still in the MALL, and the window order measured 1% slower here
    int tile_m, tile_n;
    tile_of<GM, false>(args.tiles_m, args.tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    // copy j of this wave: unit u = x / 3 of the stage, part x % 3 (main
    // rows 0-15, main rows 16-31, tail); the stage's buffer resources start
    // at the tile's first unit of K block st, lane offsets add the unit's
    // group (nkb units apart), the part and the lane's 16 bytes
    const int64_t unit_stride = (int64_t)nkb * kF6Unit;
    const int64_t a_first = (int64_t)tile_m * kUnitsA * unit_stride;
    const int64_t b_first = (int64_t)tile_n * (BN / 32) * unit_stride;
    uint32_t voff[kDma];
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
        const int x = j * NW + wave;
        const int u = x / 3, part = x % 3;
        const int gl = u < kUnitsA ? u : u - kUnitsA;
        voff[j] = (uint32_t)(gl * unit_stride) + part * 1024 + lane * 16;
    }
    // bytes of each image from the tile's first unit on (capped: every
    // offset a lane forms stays far below 2^31)
    const int a_rem =
        __builtin_amdgcn_readfirstlane((int)max(min(args.a_bytes - a_first, (int64_t)INT32_MAX), (int64_t)0));
    const int b_rem =
        __builtin_amdgcn_readfirstlane((int)max(min(args.b_bytes - b_first, (int64_t)INT32_MAX), (int64_t)0));
    auto stage = [&](int st, Stage &mn, Tail &tl) __attribute__((always_inline)) {
        const bool live = st < nkb;
        const int64_t ao = a_first + (int64_t)st * kF6Unit;
        const int64_t bo = b_first + (int64_t)st * kF6Unit;
        const int a_range = live ? max(a_rem - st * kF6Unit, 0) : 0;
        const int b_range = live ? max(b_rem - st * kF6Unit, 0) : 0;
        const __amdgpu_buffer_rsrc_t ra =
            __builtin_amdgcn_make_buffer_rsrc((void *)(args.A + ao), (short)0, a_range, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rb =
            __builtin_amdgcn_make_buffer_rsrc((void *)(args.B + bo), (short)0, b_range, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < kDma; ++j) {
            const int x = j * NW + wave;
            const int u = x / 3, part = x % 3;
            void *dst = part < 2 ? (void *)&mn[u * 32 + part * 16][0] : (void *)&tl[u * 32][0];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(u < kUnitsA ? ra : rb, LDS_PTR(dst), 16, voff[j], 0, 0, 0);
        }
    };

    const int wm0 = (wave / kWavesN) * WM;
    const int wn0 = (wave % kWavesN) * WN;
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    auto frag = [&](const Stage &mn, const Tail &tl, int row, int pm, int pt) __attribute__((always_inline)) {
        const uint4 m = mn[row][pm];
        // volatile keeps the tail reads apart: merged in pairs (ds_read2), their
        // registers would have to be copied next to each fragment's main words
        typedef unsigned int uintx2_t __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) const volatile uintx2_t lds_tail_t;
        const uintx2_t t = *(lds_tail_t *)(&tl[row][pt]);
        intx6_t f;
        f[0] = (int)m.x;
        f[1] = (int)m.y;
        f[2] = (int)m.z;
        f[3] = (int)m.w;
        f[4] = (int)t[0];
        f[5] = (int)t[1];
        return f;
    };
    // fragment of LDS row `row` (A: wm0 + 32 i + frow; B: BM + wn0 + 32 j +
    // frow) for k-step s: logical chunk / slot 2 s + half
    auto frag_at = [&](const Stage &mn, const Tail &tl, int row, int s) __attribute__((always_inline)) {
        const int c = 2 * s + fhalf;
        return frag(mn, tl, row, c ^ swizzle(frow), c ^ tswizzle(frow));   // rows start at multiples of 32
    };

    floatx16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Fragments in registers: the B fragments of the current k-step, and A
    // one row block ahead (the INT8 kernels read a whole k-step ahead; here
    // a fragment takes six registers, and that would not fit two waves per
    // SIMD).  Row block i of k-step s reads A row block i+1; the last one
    // reads the next k-step's B fragments and A row block 0, from the next
    // stage after the stage barrier (kind 1) or not at all (kind 2).
    intx6_t faq[LA], fb[FN];
    auto kstep = [&](Stage &mn, Tail &tl, int s, const Stage &nmn, const Tail &ntl, int ns, auto kind_c, int st)
        __attribute__((always_inline)) {
        constexpr int kind = decltype(kind_c)::value;
        intx6_t fbn[FN];
        static_for<FM>([&](auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            constexpr int t = i + LA;                  // the row block this step reads:
            constexpr bool here = t < FM;              // of this k-step,
            constexpr bool next = !here && kind != 2;  // or row t - FM of the next one
            intx6_t fan;
            if constexpr (here) {
                fan = frag_at(mn, tl, wm0 + t * 32 + frow, s);
            } else if constexpr (next) {
                if constexpr (t == FM) {
                    if constexpr (kind == 1) {
                        // this wave's copies of stage st+1 have landed and its
                        // reads of this stage are done; after the barrier the
                        // same holds for every wave, and this stage's buffer
                        // is free for stage st+3
                        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDma) : "memory");
                        stage(st + 3, mn, tl);
                    }
#pragma unroll
                    for (int j = 0; j < FN; ++j) fbn[j] = frag_at(nmn, ntl, BM + wn0 + j * 32 + frow, ns);
                }
                fan = frag_at(nmn, ntl, wm0 + (t - FM) * 32 + frow, ns);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma_f6(faq[0], fb[j], acc[i][j]);
            // this step's reads (and copies), then its MFMAs, in this order
            constexpr int reads = here ? 2 : (next ? (t == FM ? 2 * (FN + 1) : 2) : 0);
            if constexpr (reads > 0) __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);
            if constexpr (next && t == FM && kind == 1) __builtin_amdgcn_sched_group_barrier(0x020, kDma, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q + 1 < LA; ++q) faq[q] = faq[q + 1];
            if constexpr (here || next) faq[LA - 1] = fan;
            if constexpr (i + 1 == FM && kind != 2) {
#pragma unroll
                for (int j = 0; j < FN; ++j) fb[j] = fbn[j];
            }
        });
    };
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    // stage st (not the last) from (mn, tl), whose k-step 0 fragments are in
    // registers; refills it with stage st+3 and reads k-step 0 of the next
    auto full_stage = [&](Stage &mn, Tail &tl, const Stage &nmn, const Tail &ntl, int st)
        __attribute__((always_inline)) {
        kstep(mn, tl, 0, mn, tl, 1, K0{}, st);
        kstep(mn, tl, 1, nmn, ntl, 0, K1{}, st);
    };
    auto last_stage = [&](Stage &mn, Tail &tl) __attribute__((always_inline)) {
        kstep(mn, tl, 0, mn, tl, 1, K0{}, 0);
        kstep(mn, tl, 1, mn, tl, 0, K2{}, 0);
    };

    // dequantizing epilogue: the tile's scales staged in LDS (see gemm_kernel)
    constexpr int kThreads = NW * kWave;
    constexpr int kScaleLoads = !is_dequant(E) ? 0 : (BM + BN + kThreads - 1) / kThreads;
    __shared__ __align__(16) float lds_scale[!is_dequant(E) ? 1 : BM + BN];
    float scale_v[kScaleLoads + 1];
#pragma unroll
    for (int x = 0; x < kScaleLoads; ++x) {
        const int idx = tid + x * kThreads;
        if (idx < BM + BN)
            scale_v[x] = idx < BM ? args.scale_a[min(m0 + idx, M - 1)] : args.scale_b[min(n0 + idx - BM, N - 1)];
    }

    if (nkb > 0) {
        // nkb is a multiple of 3 (the images are padded with zero blocks), so
        // every stage's buffer is fixed at compile time and the K loop has
        // one copy of each step
        stage(0, mn0, tl0);
        stage(1, mn1, tl1);
        stage(2, mn2, tl2);
#pragma unroll
        for (int x = 0; x < kScaleLoads; ++x)
            if (tid + x * kThreads < BM + BN) lds_scale[tid + x * kThreads] = scale_v[x];
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kDma) : "memory");
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[j] = frag_at(mn0, tl0, BM + wn0 + j * 32 + frow, 0);
#pragma unroll
        for (int q = 0; q < LA; ++q) faq[q] = frag_at(mn0, tl0, wm0 + q * 32 + frow, 0);
        int st = 0;
        for (; st + 3 < nkb; st += 3) {
            full_stage(mn0, tl0, mn1, tl1, st);
            full_stage(mn1, tl1, mn2, tl2, st + 1);
            full_stage(mn2, tl2, mn0, tl0, st + 2);
        }
        full_stage(mn0, tl0, mn1, tl1, st);
        full_stage(mn1, tl1, mn2, tl2, st + 1);
        last_stage(mn2, tl2);
        // no DMA may still be writing this workgroup's LDS when it exits
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else if constexpr (is_dequant(E)) {
#pragma unroll
        for (int x = 0; x < kScaleLoads; ++x)
            if (tid + x * kThreads < BM + BN) lds_scale[tid + x * kThreads] = scale_v[x];
        __syncthreads();
    }

    store_tile<kF6, E, BM, BN, FM, FN>(args.C, args.ldc, M, N, acc, m0, n0, wm0, wn0, lane, lds_scale);
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// The 256 x 256 FP16 and INT8 tile on 16 x 16 MFMAs
//
// At the large shapes the board runs at its power limit, so a GEMM's time
// follows its energy.  v_mfma_f32_32x32x16_f16 (v_mfma_i32_32x32x32_i8) reads
// 8 operand registers and reads and writes 16 accumulator registers per 16384
// MACs; v_mfma_f32_16x16x32_f16 (v_mfma_i32_16x16x64_i8) reads 8 operand
// registers and reads and writes 4 accumulator registers per 8192 MACs, a
// fifth fewer register accesses per MAC for the same LDS traffic and the
// same number of MFMA cycles.  Configuration 0 (256 x 256, 8 waves of
// 128 x 64, two whole-line stages) runs this kernel for FP16 and INT8 with
// either B layout and for the INT8 dequantizing epilogues (column-major B),
// and so do configuration 4 (256 x 128, 8 waves of 64 x 64, three stages)
// and the 128 x 128 tiles 1 and 7 (8 waves of 32 x 64, two or three
// stages; at one round of tiles, e.g. 2048^3, 9-13% faster than 4 waves of
// 64 x 64 on 32 x 32 MFMAs); configuration 10 keeps the 32 x 32 form of 0
// for comparison.  FP16 results are bit-identical to those of the 32 x 32
// form.  The other tiles and INT4 keep the 32 x 32 form.
//
// The stage geometry is that of the whole-line kernel: stages of 128 bytes
// of K per row (two or three), BM rows of A then BN
// of B, each DMA instruction writing 8 whole rows, with chunk c of row r at
// position c ^ swizzle16(r).  The MFMA takes 16 bytes of K per lane: lane l
// of a 16-row block holds row l % 16 and bytes 16 (l / 16) .. + 15 of a
// 64-byte k-step (8 f16 or 16 int8 values; logical chunks 4 q .. 4 q + 3 of
// stage k-step q = 0, 1), and the lanes of a 16-lane phase of the LDS read 8
// consecutive rows at two logical chunks, the pattern swizzle16 keeps free
// of bank conflicts.  A wave's 128 x 64 block is 8 x 4 MFMA blocks (128
// accumulator registers; a 64 x 64 block 4 x 4, 64; a 32 x 64 block 2 x 4,
// 32); its A fragments are held
// in halves of its row blocks, so that the fragments of the next half k-step
// fit beside the current ones and the accumulators within the 256 registers
// of two waves per SIMD.  Result of block (i, j), register e of lane l: row
// 16 i + 4 (l / 16) + e, column 16 j + l % 16.
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// LDS position of logical chunk c of 128-byte stage row r in this kernel:
// c ^ swizzle16(r).  ds_read_b128 serves a wave in four phases of 16 lanes,
// lanes 8p .. 8p+7 with lanes 32+8p .. 32+8p+7 (the rocprofv3 bank-conflict
// counter reads 4 extra cycles per read of this kernel with swizzle8 and none
// for the 32 x 32 reads, as that grouping predicts).  Here a phase reads 8
// consecutive rows at logical chunk c and the same rows at c ^ 2; a 128-byte
// row r at position p covers the 16-byte bank group 8 (r % 2) + p of 16, so
// the phase is conflict-free iff, among its rows of each parity,
// swizzle16(r) differs outside bit 1.  Bits: 0 = r0 ^ r1, 1 = r3, 2 = r2;
// every 16 consecutive rows of one parity also take 8 distinct values, so a
// read of 16 rows at one chunk is conflict-free too.
__device__ __forceinline__ int swizzle16(int r) { return ((r ^ (r >> 1)) & 1) | ((r >> 2) & 2) | (r & 4); }

// Row-major B in this kernel: a stage's B part holds its rows of B (64 for
// FP16, 128 for INT8: the K values of 128 bytes of A) as BN columns, kCpr
// 16-byte chunks each (FP16 32 or 16, INT8 16 or 8 for BN = 256 or 128),
// logical chunk c of B row r at position c ^ bswizzle16(r).  A transposing
// read gives each 16-lane group g of a k-step the kR rows (FP16 4, INT8 8)
// starting at row 2 kR g + kR t of its 16 columns (1 chunk of INT8, 2 of
// FP16), so one read touches 16 (row, chunk) pairs of two groups; they fall
// in distinct bank groups when the swizzle separates the rows of one read
// and the groups g of either pairing, (0, 1) with (2, 3) or (0, 2) with
// (1, 3) (the bit g0 ^ g1).  With 16 or 32 chunks a row, position p of row
// r is bank group p % 16 whatever r; with 8 (INT8, BN = 128) it is
// 8 (r % 2) + p, so there the parity of the row separates half the pairs
// and the swizzle needs one bit less.
template <int P, int BN>
__device__ __forceinline__ int bswizzle16(int r) {
    if constexpr (P == kF16)
        return 2 * ((r & 3) | ((((r >> 3) ^ (r >> 4)) & 1) << 2));
    else if constexpr (BN == 256)
        return (r & 7) | ((((r >> 4) ^ (r >> 5)) & 1) << 3);
    else
        return ((r >> 1) & 3) | ((((r >> 4) ^ (r >> 5)) & 1) << 2);
}

__device__ __forceinline__ floatx4_t mfma16_f16(const uint4 &a, const uint4 &b, const floatx4_t &c) {
    half8_t av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
}

__device__ __forceinline__ intx4_t mfma16_i8(const uint4 &a, const uint4 &b, const intx4_t &c) {
    intx4_t av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
}

template <int P, int E, int BR, int BM, int BN, int WM, int WN, int LS>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave) void gemm_mf16_kernel(Args args) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int GM = 4;
    constexpr int NW = (BM / WM) * (BN / WN);   // 8 waves
    constexpr int kWavesN = BN / WN;
    constexpr int kRows = BM + BN;              // LDS rows per stage
    constexpr int kDmaL = kRows / 8 / NW;       // 1 KB DMA instructions per wave per stage
    constexpr int kDmaLA = BM / 8 / NW;         // ... of which fill A rows
    constexpr int kStageK = 2 * kRowBytes;      // bytes of K per row per stage
    constexpr int FM = WM / 16, FN = WN / 16;   // MFMA blocks of a wave
    constexpr int FH = FM / 2;                  // A fragments per half k-step
    static_assert(NW == 8 && BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "8 waves; stage rows split evenly");
    static_assert(FN == 4 && FM % 2 == 0, "two column pairs per wave for the stores");
    static_assert(LS == 2 || LS == 3, "two or three stages");
    static_assert((LS - 1) * kDmaL <= 63, "vmcnt holds at most 63 outstanding loads");
    __shared__ uint4 ln0[kRows][2 * kChunks];
    __shared__ uint4 ln1[kRows][2 * kChunks];
    __shared__ uint4 ln2[LS > 2 ? kRows : 1][2 * kChunks];
    using LStage = uint4[kRows][2 * kChunks];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int M = args.M, N = args.N, K = args.K;
    int tile_m, tile_n;
    tile_of<GM>(args.tiles_m, args.tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    // operand rows past M (N) are clamped to the last valid one; the buffer
    // range of a stage ends at the last 16-byte chunk of the last valid row
    // that holds data, and is zero for a stage past K (as in gemm_kernel)
    static_assert(P == kF16 || P == kI8, "FP16 or INT8");
    static_assert(E == kRaw || (P == kI8 && is_dequant(E) && BR == kBCol), "plain, or INT8 dequantized");
    using RB = RowB<P>;
    constexpr int kEs = P == kF16 ? 2 : 1;                  // bytes per element
    constexpr int kCpr = BN * kEs / 16;                     // row-major B: chunks per row of B
    static_assert(BR == kBCol || 2 * RB::kKRows * kCpr == 8 * BN, "row-major B part of a stage");
    constexpr bool kDeq = is_dequant(E);
    // Dequantizing epilogue: the block's 256 row and 256 column scales, one
    // per thread, loaded now, written to LDS after the first DMAs and
    // published by the first barrier (rows and columns past the edge take the
    // last valid scale; their results are not stored)
    __shared__ __align__(16) float lds_scale[kDeq ? BM + BN : 1];
    float scale_v = 0.0f;
    if constexpr (kDeq) {
        static_assert(BM + BN <= NW * kWave, "one scale per thread at most");
        if (tid < BM + BN)
            scale_v = tid < BM ? args.scale_a[min(m0 + tid, M - 1)] : args.scale_b[min(n0 + tid - BM, N - 1)];
    }
    const int valid = P == kF16 ? 2 * K : K;        // data bytes per row
    const int valid16 = (valid + 15) & ~15;
    const int n_st = (valid + kStageK - 1) / kStageK;
    const uint8_t *const a_base = args.A + (int64_t)m0 * args.lda_bytes;
    const int a_end = (int)((min(BM, M - m0) - 1) * args.lda_bytes) + valid16;
    // column-major B: like A, BN rows of K.  Row-major B: the tile's columns
    // start n0 values into every row of B; the range ends at the last chunk
    // of row K-1 that holds a column below N, so rows past K read as zeros,
    // and a stage's resource starts at its first row of B (a lane's offset
    // spans at most 2 kKRows rows: 512 MiB with rows of 4 MiB)
    const uint8_t *const b_base = args.B + (BR == kBRow ? (int64_t)n0 * kEs : (int64_t)n0 * args.ldb_bytes);
    const int64_t b_end = BR == kBRow
                              ? (int64_t)(K - 1) * args.ldb_bytes + (((int64_t)min(BN, N - n0) * kEs + 15) & ~int64_t(15))
                              : (int64_t)(min(BN, N - n0) - 1) * args.ldb_bytes + valid16;
    const int64_t b_stage_bytes = BR == kBRow ? (int64_t)2 * RB::kKRows * args.ldb_bytes : kStageK;
    // DMA instruction j of this wave fills stage rows (j*NW + wave)*8 .. +7;
    // lane l fetches logical chunk (l%8) ^ swizzle16(row) of row l/8.
    // Row-major B: lane l of a B instruction fills flat chunk f of the B
    // part: row f / kCpr of B, position f % kCpr
    uint32_t voffl[kDmaL];
#pragma unroll
    for (int j = 0; j < kDmaL; ++j) {
        const int cr = (j * NW + wave) * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ swizzle16(cr);
        if (j < kDmaLA) {
            voffl[j] = (uint32_t)((min(m0 + cr, M - 1) - m0) * args.lda_bytes) + lchunk * 16;
        } else if constexpr (BR == kBCol) {
            voffl[j] = (uint32_t)((min(n0 + cr - BM, N - 1) - n0) * args.ldb_bytes) + lchunk * 16;
        } else {
            const int f = ((j * NW + wave) - BM / 8) * 64 + lane;
            const int krow = f / kCpr;
            const int gchunk = (f % kCpr) ^ bswizzle16<P, BN>(krow);
            voffl[j] = (uint32_t)(krow * args.ldb_bytes) + gchunk * 16;
        }
    }
    auto stage_l = [&](int st, LStage &buf) __attribute__((always_inline)) {
        const int kb = st * kStageK;
        const bool live = st < n_st;
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a_base + kb), (short)0, live ? a_end - kb : 0, kRsrcWord3);
        const int64_t bt = (int64_t)st * b_stage_bytes;
        const int b_range = !live ? 0
                            : BR == kBRow ? (int)max(min(min(b_end - bt, b_stage_bytes), (int64_t)INT32_MAX), (int64_t)0)
                                          : (int)(b_end - bt);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(b_base + bt), (short)0, b_range, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < kDmaL; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(j < kDmaLA ? ra : rb, LDS_PTR(&buf[(j * NW + wave) * 8][0]),
                                                     16, voffl[j], 0, 0, 0);
    };

    const int wm0 = (wave / kWavesN) * WM;   // wave's first row / column in the block tile
    const int wn0 = (wave % kWavesN) * WN;
    const int frow = lane & 15;              // fragment row (A) / column (B) of this lane
    const int fq = lane >> 4;                // which 16-byte quarter of a 64-byte k-step
    // fragment rows start at multiples of 16, so the swizzle of row frow applies
    // A fragments of k-step q for row blocks hi*FH .. hi*FH + FH-1
    auto read_a = [&](const LStage &buf, int q, int hi, uint4 (&fa)[FH]) __attribute__((always_inline)) {
        const int ch = (4 * q + fq) ^ swizzle16(frow);
#pragma unroll
        for (int i = 0; i < FH; ++i) fa[i] = buf[wm0 + (hi * FH + i) * 16 + frow][ch];
    };
    // Row-major B: lane i of a 16-lane group points its transposing read at
    // row i / kQ of the read, bytes 8 (i % kQ) of the group's columns, and
    // receives the kR values of column i; two reads make the 16 bytes of K the
    // MFMA takes (group g: values 2 kR g .. 2 kR g + 2 kR - 1 of the k-step)
    // The swizzle of a lane's rows depends only on the row within a read and
    // on the group (q and t move the row by multiples of 2 kR that leave
    // bswizzle16 unchanged), so a lane's byte offset is fixed per column
    // block and q and t add constants.
    const int tr_i = lane & 15;
    const int tr_row = tr_i / RB::kQ;
    const int tr_byte = 8 * (tr_i % RB::kQ);
    uint32_t b_off[BR == kBRow ? FN : 1];
    if constexpr (BR == kBRow) {
        const int krow0 = fq * (2 * RB::kR) + tr_row;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col_bytes = (wn0 + j * 16) * kEs + tr_byte;
            const int pos = (col_bytes >> 4) ^ bswizzle16<P, BN>(krow0);
            b_off[j] = (uint32_t)((krow0 * kCpr + pos) * 16 + (col_bytes & 15));
        }
    }
    auto read_b = [&](const LStage &buf, int q, uint4 (&fb)[FN]) __attribute__((always_inline)) {
        if constexpr (BR == kBCol) {
            const int ch = (4 * q + fq) ^ swizzle16(frow);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = buf[BM + wn0 + j * 16 + frow][ch];
        } else {
            const char *const bpart = reinterpret_cast<const char *>(&buf[BM][0]);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                uint32_t w[4];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const char *const ptr = bpart + b_off[j] + (q * RB::kKRows + t * RB::kR) * kCpr * 16;
                    if constexpr (P == kF16) {
                        typedef short v4s __attribute__((ext_vector_type(4)));
                        const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) v4s *)(ptr));
                        __builtin_memcpy(&w[2 * t], &v, 8);
                    } else {
                        const intx2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (__attribute__((address_space(3))) intx2_t *)(ptr));
                        __builtin_memcpy(&w[2 * t], &v, 8);
                    }
                }
                fb[j] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    };
    // zero the bytes of this lane's fragments of k-step q of stage st at or beyond K
    auto mask = [&](int st, int q, uint4 *f, int n) __attribute__((always_inline)) {
        const int nb = valid - (st * kStageK + (4 * q + fq) * 16);
        uint32_t m[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int r = nb - 4 * d;
            m[d] = r >= 4 ? 0xFFFFFFFFu : (r <= 0 ? 0u : (1u << (8 * r)) - 1u);
        }
#pragma unroll
        for (int i = 0; i < n; ++i) {
            f[i].x &= m[0];
            f[i].y &= m[1];
            f[i].z &= m[2];
            f[i].w &= m[3];
        }
    };

    using Acc4 = typename std::conditional<P == kF16, floatx4_t, intx4_t>::type;
    Acc4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0;
    auto mma_half = [&](int hi, const uint4 (&fa)[FH], const uint4 (&fb)[FN]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FH; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (P == kF16)
                    acc[hi * FH + i][j] = mfma16_f16(fa[i], fb[j], acc[hi * FH + i][j]);
                else
                    acc[hi * FH + i][j] = mfma16_i8(fa[i], fb[j], acc[hi * FH + i][j]);
            }
    };
    // issue order of a half k-step: its MFMAs with the next fragment reads
    // (and, after the stage barrier, the DMA of a later stage) slotted one by
    // one between them
    constexpr int kMfma = FH * FN;
    auto interleave = [&](auto reads_c, auto dma_c) __attribute__((always_inline)) {
        constexpr int reads = decltype(reads_c)::value;
        constexpr int dma = decltype(dma_c)::value;
        constexpr int rper = (reads + kMfma - 1) / kMfma;   // LDS reads per MFMA slot (row-major B
                                                            // on 64 x 64 waves: two in some)
        static_assert(dma <= kMfma, "one DMA per MFMA slot at most");
#pragma unroll
        for (int i = 0; i < kMfma; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                            // 1 MFMA
            if (i * rper < reads) __builtin_amdgcn_sched_group_barrier(0x100, rper, 0);  // LDS reads
            if (i < dma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);              // 1 DMA
        }
    };
    using kNone = std::integral_constant<int, 0>;
    using kHalfA = std::integral_constant<int, FH>;
    using kHalfAB = std::integral_constant<int, FH + FN * (BR == kBRow ? 2 : 1)>;
    using kStageDma = std::integral_constant<int, kDmaL>;

    // A fragments of the lower (fL) and upper (fU) row blocks; B fragments of
    // the even (fbA) and odd (fbB) k-step of a stage
    uint4 fL[FH], fU[FH], fbA[FN], fbB[FN];
    // stage st (not the last) from `cur`, whose k-step 0 lower half is in
    // fL / fbA; refills `cur` with stage st+LS and reads the first fragments
    // of stage st+1 from `nxt`
    auto full_stage = [&](LStage &cur, const LStage &nxt, int st) __attribute__((always_inline)) {
        read_a(cur, 0, 1, fU);
        mma_half(0, fL, fbA);
        interleave(kHalfA{}, kNone{});
        read_a(cur, 1, 0, fL);
        read_b(cur, 1, fbB);
        mma_half(1, fU, fbA);
        interleave(kHalfAB{}, kNone{});
        read_a(cur, 1, 1, fU);
        mma_half(0, fL, fbB);
        interleave(kHalfA{}, kNone{});
        // this wave's DMA of stage st+1 has landed (stages st+2 .. st+LS-1
        // may still be in flight) and its reads of `cur` are done; after the
        // barrier the same holds for every wave
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((LS - 2) * kDmaL) : "memory");
        stage_l(st + LS, cur);
        read_a(nxt, 0, 0, fL);
        read_b(nxt, 0, fbA);
        mma_half(1, fU, fbB);
        interleave(kHalfAB{}, kStageDma{});
        __builtin_amdgcn_sched_barrier(0);
    };
    // the last stage, with the bytes at or beyond K masked off
    auto last_stage = [&](const LStage &cur, int st) __attribute__((always_inline)) {
        read_a(cur, 0, 1, fU);
        mask(st, 0, fL, FH);
        mask(st, 0, fbA, FN);
        mask(st, 0, fU, FH);
        mma_half(0, fL, fbA);
        mma_half(1, fU, fbA);
        read_a(cur, 1, 0, fL);
        read_b(cur, 1, fbB);
        read_a(cur, 1, 1, fU);
        mask(st, 1, fL, FH);
        mask(st, 1, fbB, FN);
        mask(st, 1, fU, FH);
        mma_half(0, fL, fbB);
        mma_half(1, fU, fbB);
    };
    if (n_st > 0) {
        stage_l(0, ln0);
        stage_l(1, ln1);
        if constexpr (LS > 2) stage_l(2, ln2);
        if constexpr (kDeq)
            if (tid < BM + BN) lds_scale[tid] = scale_v;
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((LS - 1) * kDmaL) : "memory");
        read_a(ln0, 0, 0, fL);
        read_b(ln0, 0, fbA);
        int st = 0;
        if constexpr (LS == 2) {
            for (; st + 2 < n_st; st += 2) {
                full_stage(ln0, ln1, st);
                full_stage(ln1, ln0, st + 1);
            }
            if (st + 1 < n_st) full_stage(ln0, ln1, st++);
            last_stage((st & 1) ? ln1 : ln0, st);
        } else {
            for (; st + 3 < n_st; st += 3) {
                full_stage(ln0, ln1, st);
                full_stage(ln1, ln2, st + 1);
                full_stage(ln2, ln0, st + 2);
            }
            // 1 to 3 stages remain, the first of them in ln0
            if (st + 1 < n_st) {
                full_stage(ln0, ln1, st++);
                if (st + 1 < n_st) full_stage(ln1, ln2, st++);
            }
            const int r = st % 3;
            last_stage(r == 0 ? ln0 : r == 1 ? ln1 : ln2, st);
        }
        // no DMA may still be writing this workgroup's LDS when it exits
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else if constexpr (kDeq) {
        // K == 0: no main loop, so stage the scales here
        if (tid < BM + BN) lds_scale[tid] = scale_v;
        __syncthreads();
    }

    // ---- epilogue: 16 x 16 MFMA result layout -> row-major C, non-temporal ----
    // In block (i, j) lane l holds column l % 16 of rows 4 (l / 16) + e, so a
    // store straight from it writes 64-byte pieces of lines.  v_permlane16_swap
    // exchanges the odd 16-lane rows of block 2h's register e with the even
    // 16-lane rows of block 2h+1's; then lanes 0-31 of the first hold columns
    // 32h .. 32h+31 of row e and lanes 32-63 those of row 8 + e, the second
    // rows 4 + e and 12 + e: every 32-bit store writes two whole 128-byte
    // pieces.  A binary16 C takes one more exchange, v_permlane32_swap of the
    // h = 0 and h = 1 results (upper 32 lanes of the first with the lower 32 of
    // the second), after which a register holds columns 0 .. 63 of one row.
    using Out = typename OutOf<P, E>::type;
    constexpr int kOut = (int)sizeof(Out);
    const int half = lane >> 5;
    const int hcol = lane & 31;
    char *const wave_c = reinterpret_cast<char *>(args.C) + ((int64_t)(m0 + wm0) * args.ldc + n0 + wn0) * kOut;
    const int64_t row_bytes = args.ldc * kOut;
    const bool interior = m0 + BM <= M && n0 + BN <= N;
    // this lane's row scales of block row i: rows 16 i + 8 half + 0..3 (x) and + 4..7 (y);
    // column scales: columns 32 h + hcol
    float sb[FN / 2];
    if constexpr (kDeq) {
#pragma unroll
        for (int h = 0; h < FN / 2; ++h) sb[h] = lds_scale[BM + wn0 + 32 * h + hcol];
    }
    // ((float)sum * scale_a) * scale_b, rounded once per step; a binary16 C
    // rounds that binary32 value again (the empty asm keeps the backend from
    // fusing the product and the narrowing into one rounding)
    auto dequant = [&](uint32_t bits, float sa, float sbv) __attribute__((always_inline)) {
        float c = (float)(int32_t)bits;
        c = c * sa;
        c = c * sbv;
        if constexpr (E == kDequantF16) asm("" : "+v"(c));
        return c;
    };
    if constexpr (E != kDequantF16) {
        const uint32_t lane_off = (uint32_t)(8 * half * row_bytes) + hcol * (uint32_t)kOut;
        const int rows_left = M - (m0 + wm0) - 8 * half;   // rows this lane may write: r < rows_left
        const int cols_left = N - (n0 + wn0) - hcol;       // columns: 32 h < cols_left
        auto store_all = [&](auto &&keep) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                float4 sa0, sa1;
                if constexpr (kDeq) {
                    sa0 = *reinterpret_cast<const float4 *>(&lds_scale[wm0 + 16 * i + 8 * half]);
                    sa1 = *reinterpret_cast<const float4 *>(&lds_scale[wm0 + 16 * i + 8 * half + 4]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = i * 16 + e;   // wave-uniform part of the row
#pragma unroll
                    for (int h = 0; h < FN / 2; ++h) {
                        // (the elements are copied out first: a bit cast of a
                        // vector element in place reads element 0 with this compiler)
                        const auto lo = acc[i][2 * h][e], hi = acc[i][2 * h + 1][e];
                        const auto xy = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, lo),
                                                                         __builtin_bit_cast(uint32_t, hi), false, false);
                        uint32_t v0 = xy[0], v1 = xy[1];
                        if constexpr (kDeq) {
                            const float e0 = e == 0 ? sa0.x : e == 1 ? sa0.y : e == 2 ? sa0.z : sa0.w;
                            const float e1 = e == 0 ? sa1.x : e == 1 ? sa1.y : e == 2 ? sa1.z : sa1.w;
                            v0 = __builtin_bit_cast(uint32_t, dequant(v0, e0, sb[h]));
                            v1 = __builtin_bit_cast(uint32_t, dequant(v1, e1, sb[h]));
                        }
                        if (keep(r, h))
                            __builtin_nontemporal_store(v0, reinterpret_cast<uint32_t *>(
                                                                wave_c + r * row_bytes + lane_off + h * 128));
                        if (keep(r + 4, h))
                            __builtin_nontemporal_store(v1, reinterpret_cast<uint32_t *>(
                                                                wave_c + (r + 4) * row_bytes + lane_off + h * 128));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (interior)
            store_all([](int, int) { return true; });
        else
            store_all([&](int r, int h) { return r < rows_left && h * 32 < cols_left; });
    } else {
        static_assert(FN == 4, "two column halves per store");
        // after both exchanges lane l holds column l of a row: 128 bytes per store
        const uint32_t lane_off = (uint32_t)(lane * kOut);
        const int rows_left = M - (m0 + wm0);
        const int cols_left = N - (n0 + wn0) - lane;
        auto store_all = [&](auto &&keep) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const float4 sa0 = *reinterpret_cast<const float4 *>(&lds_scale[wm0 + 16 * i + 8 * half]);
                const float4 sa1 = *reinterpret_cast<const float4 *>(&lds_scale[wm0 + 16 * i + 8 * half + 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = i * 16 + e;
                    const float e0 = e == 0 ? sa0.x : e == 1 ? sa0.y : e == 2 ? sa0.z : sa0.w;
                    const float e1 = e == 0 ? sa1.x : e == 1 ? sa1.y : e == 2 ? sa1.z : sa1.w;
                    uint32_t hv[2][2];   // [rows r (+8) | rows r + 4 (+8)][h]: binary16 bits in the low half
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const auto lo = acc[i][2 * h][e], hi = acc[i][2 * h + 1][e];
                        const auto xy = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, lo),
                                                                         __builtin_bit_cast(uint32_t, hi), false, false);
                        const _Float16 f0 = (_Float16)dequant(xy[0], e0, sb[h]);
                        const _Float16 f1 = (_Float16)dequant(xy[1], e1, sb[h]);
                        hv[0][h] = __builtin_bit_cast(uint16_t, f0);
                        hv[1][h] = __builtin_bit_cast(uint16_t, f1);
                    }
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(hv[k][0], hv[k][1], false, false);
                        const int rr = r + 4 * k;   // sw[0]: row rr, sw[1]: row rr + 8; column = lane
                        if (keep(rr))
                            __builtin_nontemporal_store((uint16_t)sw[0], reinterpret_cast<uint16_t *>(
                                                                             wave_c + rr * row_bytes + lane_off));
                        if (keep(rr + 8))
                            __builtin_nontemporal_store((uint16_t)sw[1], reinterpret_cast<uint16_t *>(
                                                                             wave_c + (rr + 8) * row_bytes + lane_off));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (interior)
            store_all([](int) { return true; });
        else
            store_all([&](int rr) { return rr < rows_left && 0 < cols_left; });
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// host side

// ls: whole-line stages, or 0 for four 64-byte stages.  Only the 32 x 32
// K-split tile keeps 64-byte stages: at M = 16 and 512^3, where it runs, whole
// lines were no faster (their 4-wave 512-byte K tiles make few, deep stages),
// while the 64 x 32 K-split tile gained 10-18% from them (FP16 and INT8).
// 256 x 256 fits two 64 KB stages; 128 x 128 keeps two so that two
// workgroups share a CU, except in 7, which takes three for products of at
// most one tile per CU (where a CU holds one workgroup anyway); the others
// take three.  The 256-row and 128 x 128 tiles run 8 waves, two per SIMD
// for each workgroup, so that one wave's fragment reads, INT4 unpacking and
// barrier wait overlap the other's MFMAs (their accumulators then live in
// VGPRs).  128 x 128 with 8 waves of 32 x 64 on 16 x 16 MFMAs (FP16, INT8)
// beat 4 waves of 64 x 64 on 32 x 32 ones by 2-13%; for INT4 on 32 x 32
// MFMAs the 8 waves gained 2-14% on three stages (7) and lost 1-3% on two
// (1) at 10240 x 2048 x 4096 and 4096^3, and one geometry serves both.
struct Config {
    int bm, bn, wm, wn, gm, ks, ls;
};

constexpr Config kConfigs[] = {
    {256, 256, 128, 64, 4, 1, 2},   // 0: large shapes (8 waves; FP16 and INT8 on 16 x 16 MFMAs)
    {128, 128, 32, 64, 8, 1, 2},    // 1: medium (8 waves)
    {64, 64, 32, 32, 8, 1, 3},      // 2: small
    {32, 32, 32, 32, 8, 4, 0},      // 3: few tiles (small M or N): K split over 4 waves
    {256, 128, 64, 64, 4, 1, 3},    // 4: between 0 and 1 (e.g. M = 1024 of a wide product; 8 waves)
    {128, 64, 64, 32, 8, 1, 3},     // 5: between 1 and 2 (e.g. M = 256)
    {64, 32, 64, 32, 8, 4, 3},      // 6: K split over 4 waves, 64 rows (e.g. M = 64 of a wide product)
    {128, 128, 32, 64, 8, 1, 3},    // 7: 1 with three stages, for at most one round of tiles
    {256, 256, 128, 128, 4, 1, 2},  // 8: 0 with 4 waves of 128 x 128 (never picked: kept to compare)
    {64, 64, 64, 64, 8, 4, 2},      // 9: 2 with K split over 4 waves, for one round of tiles and long K
    {256, 256, 128, 64, 4, 1, 2},   // 10: 0 on 32 x 32 MFMAs for FP16 and INT8 too (never picked: kept to compare)
};

// Tiles without K split, largest first: the order in which pick() tries them.
constexpr int kPickOrder[] = {0, 4, 1, 5, 2};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

template <int P, int C, int E, int BR>
const void *kernel_for() {
    constexpr Config c = kConfigs[C];
    return reinterpret_cast<const void *>(&gemm_kernel<P, c.bm, c.bn, c.wm, c.wn, c.gm, E, BR, c.ks, c.ls>);
}

template <int P, int C, int E, int BR>
const void *mf16_for() {
    constexpr Config c = kConfigs[C];
    static_assert(c.ks == 1, "no K split inside the workgroup");
    return reinterpret_cast<const void *>(&gemm_mf16_kernel<P, E, BR, c.bm, c.bn, c.wm, c.wn, c.ls>);
}

template <int P, int E, int BR>
const void *kernel_ptr(int cfg) {
    switch (cfg) {
    case 0:
        // FP16 and INT8, either B layout (INT8 with column-major B also
        // dequantized): the same tile on 16 x 16 MFMAs
        if constexpr ((P == kF16 || P == kI8) && (E == kRaw || (P == kI8 && is_dequant(E) && BR == kBCol)))
            return mf16_for<P, 0, E, BR>();
        else
            return kernel_for<P, 0, E, BR>();
    case 1:
        // 128 x 128 (8 waves of 32 x 64), two or three stages: as 4
        if constexpr ((P == kF16 || P == kI8) && (E == kRaw || (P == kI8 && BR == kBCol)))
            return mf16_for<P, 1, E, BR>();
        else
            return kernel_for<P, 1, E, BR>();
    case 2: return kernel_for<P, 2, E, BR>();
    case 3: return kernel_for<P, 3, E, BR>();
    case 4:
        // 256 x 128: FP16 and INT8 with either B layout, INT8 dequantized
        // (column-major B), on 16 x 16 MFMAs too
        if constexpr ((P == kF16 || P == kI8) && (E == kRaw || (P == kI8 && BR == kBCol)))
            return mf16_for<P, 4, E, BR>();
        else
            return kernel_for<P, 4, E, BR>();
    case 5: return kernel_for<P, 5, E, BR>();
    case 6: return kernel_for<P, 6, E, BR>();
    case 7:
        if constexpr ((P == kF16 || P == kI8) && (E == kRaw || (P == kI8 && BR == kBCol)))
            return mf16_for<P, 7, E, BR>();
        else
            return kernel_for<P, 7, E, BR>();
    case 8: return kernel_for<P, 8, E, BR>();
    case 9: return kernel_for<P, 9, E, BR>();
    case 10: return kernel_for<P, 10, E, BR>();
    default: return nullptr;
    }
}

// Instantiated: every precision with either B layout; the dequantizing
// epilogues with column-major B.
const void *kernel_ptr(int prec, int cfg, int epi, int br) {
    if (br == kBRow) {
        if (epi != kRaw) return nullptr;
        switch (prec) {
        case kF16: return kernel_ptr<kF16, kRaw, kBRow>(cfg);
        case kI8: return kernel_ptr<kI8, kRaw, kBRow>(cfg);
        case kI4: return kernel_ptr<kI4, kRaw, kBRow>(cfg);
        default: return nullptr;
        }
    }
    switch (prec * 3 + epi) {
    case kF16 * 3 + kRaw: return kernel_ptr<kF16, kRaw, kBCol>(cfg);
    case kI8 * 3 + kRaw: return kernel_ptr<kI8, kRaw, kBCol>(cfg);
    case kI8 * 3 + kDequantF32: return kernel_ptr<kI8, kDequantF32, kBCol>(cfg);
    case kI8 * 3 + kDequantF16: return kernel_ptr<kI8, kDequantF16, kBCol>(cfg);
    case kI4 * 3 + kRaw: return kernel_ptr<kI4, kRaw, kBCol>(cfg);
    case kI4 * 3 + kDequantF32: return kernel_ptr<kI4, kDequantF32, kBCol>(cfg);
    case kI4 * 3 + kDequantF16: return kernel_ptr<kI4, kDequantF16, kBCol>(cfg);
    default: return nullptr;
    }
}

constexpr int64_t kMaxRowBytes = int64_t(1) << 22;  // 4 MiB: a 256-row tile spans at most 1 GiB

int elem_bits(int prec) { return prec == kF16 ? 16 : (prec == kI8 ? 8 : 4); }

bool sync_check_enabled() {
    static const bool on = [] {
        const char *e = getenv("PDGEMM_SYNC_CHECK");
        return e && strcmp(e, "1") == 0;
    }();
    return on;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Steady throughput of each tile without K split, in TFLOP/s (FP16) or TOP/s
// (INT8, INT4): back-to-back timings (HIP graphs of about 25 ms, medians of
// three alternated rounds, one GPU) on a product that gives every one of
// them whole rounds of workgroups (M = K = 8192, N = 6144); only the ratios
// within a row matter.  0 = not a candidate (the K-split tiles, 7,
// which stands in for 1, 9, which stands in for 2, 8, the 4-wave form of 0,
// slower than 0 at N = 8192, and 10, 0 on 32 x 32 MFMAs).
constexpr int kTileRate[3][kNumConfigs] = {
    {1463, 1167, 728, 0, 1319, 766, 0, 0, 0, 0, 0},    // FP16
    {2771, 2254, 1372, 0, 2566, 1667, 0, 0, 0, 0, 0},  // INT8
    {2947, 2462, 1950, 0, 2625, 2086, 0, 0, 0, 0, 0},  // INT4
};

// When the 64 x 64 tile fills the chip (at least one workgroup per CU), a
// time model chooses among the tiles that give more than half of the CUs
// one: the busiest CU sets the time, so a product of T tiles takes T / 256
// rounds, each of which costs the tile's area over its throughput.  A
// partial last round costs 0.35 + 0.65 * (its fill) of a full one: the fewer
// CUs run, the higher their clock and the more L2 and HBM bandwidth each
// gets.  (A tile that busies exactly half of the CUs lost to a full round
// of a smaller one wherever it was timed, e.g. 128 x 128 against 128 x 64 at
// 256 x 8192 x 8192 by 1-13%, most with row-major B.)  The cheapest tile
// wins, the larger one on a tie.  (E.g. 144 tiles of
// 256 x 256 rather than 576 of 128 x 128 at 3072^3; for FP16 and INT8, 768
// of 256 x 128 rather than 384 of 256 x 256 at 8192 x 3072 x 8192.)  The
// partial-round rule was fitted to 69 shapes from 1024^3 to 12288 x 4096 x
// 4096 in three precisions on two GPUs, the rates measured again after the
// 16 x 16 MFMA kernels: over 78 shapes (M = 256-512 x 8192 x 8192 added)
// 0.09% slower than the fastest tile on average, at most 2.5% (FP16 256 x
// 8192 x 8192, a near tie there).  When
// even the 64 x 64 tile leaves CUs idle (small M or N), a K-split tile puts
// 4 waves on each of up to 4 times as many tiles.  128 x 128 with at most
// one tile per CU takes configuration 7.
int pick(int prec, int64_t M, int64_t N, int64_t K) {
    auto tiles = [&](int c) { return cdiv(M, kConfigs[c].bm) * cdiv(N, kConfigs[c].bn); };
    if (tiles(2) >= 256) {
        int best = -1;
        double best_cost = 0;
        for (int c : kPickOrder) {
            const int64_t t = tiles(c);
            if (kTileRate[prec][c] == 0 || t <= 128) continue;
            const double partial = double(t % 256) / 256;
            const double rounds = double(t / 256) + (partial > 0 ? 0.35 + 0.65 * partial : 0.0);
            const double cost = rounds * kConfigs[c].bm * kConfigs[c].bn / kTileRate[prec][c];
            if (best < 0 || cost < best_cost) {
                best = c;
                best_cost = cost;
            }
        }
        // the 64 x 64 tile is always a candidate here.  At most one 128 x 128
        // tile per CU: the three-stage variant (7), as a CU holds one anyway
        if (best == 1 && tiles(1) <= 256) return 7;
        // One round of 64 x 64 tiles over a long K (e.g. 128 x 8192 x 8192):
        // four waves on K slices of each tile, with no stage barrier, beat
        // four waves on its quarters by 8-23% when a row of K values is a
        // whole number of 128-byte lines; at K <= 4096, or with rows that end
        // inside a line, the reduction of the partial tiles costs more.
        const int64_t k_bytes = prec == kF16 ? 2 * K : (prec == kI8 ? K : K / 2);
        if (best == 2 && tiles(2) <= 288 && K >= 8192 && k_bytes % 128 == 0) return 9;
        return best;
    }
    // K split: 64 x 32 when more than 32 rows still fill the chip (each B
    // panel is then staged once rather than once per 32 rows), else 32 x 32
    if (M > 32 && cdiv(M, 64) * cdiv(N, 32) >= 256) return 6;
    return 3;
}

// K split across workgroups.  Where even 64 x 64 tiles leave CUs idle
// (pick() settles on a K-split tile) and K is long, each CU runs one long
// row of K; splitting K over S grid rows of workgroups that add into a
// zeroed C multiplies the workgroups by S.  Row-major B gains most, as its
// K-split tiles read 32-64 bytes of each row of B, while the 64-row tiles
// read whole 128-byte lines.  The tile is 64 x 64 (128 x 64 for integers
// past 64 rows of A) and S the largest of 2, 4, 8 with at most 256
// workgroups; taken for integers when each range still holds 2048 values of
// K (column-major B: only for at most 32 tiles and 4096 values, as its
// K-split tiles already read whole lines), for FP16 (two ranges only: see
// launch_splitk) with row-major B, at most 128 tiles and K >= 16384.
// Measured at M = 8-512, N = 512-16384, K = 2048-65536: 1.2-1.3x at
// M <= 64 x 8192 x 8192 (row-major B, integers), up to 3x at 64 x 2048 x
// 32768; where the rule declines (K <= 4096, or the chip filled), the split
// lost up to 2x to the zero pass and the atomic adds.
int pick_splits(int prec, int br, int64_t M, int64_t N, int64_t K, int *cfg) {
    const int base = pick(prec, M, N, K);
    *cfg = base;
    if (base != 3 && base != 6) return 1;
    const int tile = (prec != kF16 && M > 64) ? 5 : 2;
    const int64_t t = cdiv(M, kConfigs[tile].bm) * cdiv(N, kConfigs[tile].bn);
    int s = 1;
    if (prec == kF16) {
        if (br == kBRow && t <= 128 && K >= 16384) s = 2;
    } else {
        while (s < 8 && t * s * 2 <= 256) s *= 2;
        const int64_t min_range = br == kBRow ? 2048 : 4096;
        if ((br == kBCol && t > 32) || K / s < min_range) s = 1;
    }
    if (s > 1) *cfg = tile;
    return s;
}

int validate(int prec, int epi, int br, int64_t M, int64_t N, int64_t K, const void *A,
             int64_t lda, const void *B, int64_t ldb, const void *C, int64_t ldc,
             const float *scale_a, const float *scale_b) {
    if (M < 0 || N < 0 || K < 0) return PDGEMM_EINVAL_DIM;
    if (M > INT32_MAX || N > INT32_MAX || K > (int64_t(1) << 30)) return PDGEMM_EINVAL_DIM;
    if (prec == kI4 && K > PDGEMM_I4_MAX_K) return PDGEMM_EINVAL_DIM;
    // a row of B holds K values (column-major) or N values (row-major)
    if (lda < K || ldb < (br == kBRow ? N : K) || ldc < N) return PDGEMM_EINVAL_LD;
    if (prec == kI4 && ((K & 1) || (lda & 1) || (ldb & 1))) return PDGEMM_EINVAL_I4;
    if (M == 0 || N == 0) return PDGEMM_OK;
    if (!C || (K > 0 && (!A || !B))) return PDGEMM_ENULL;
    if (epi != kRaw && (!scale_a || !scale_b)) return PDGEMM_ENULL;
    // operand tiles are addressed with 32-bit offsets from the tile's first
    // row; the limit is checked in elements, before any byte count is formed
    const int64_t c_size = epi == kDequantF16 ? 2 : 4;
    const int64_t max_ld = kMaxRowBytes * 8 / elem_bits(prec);
    if (lda > max_ld || ldb > max_ld || ldc > kMaxRowBytes / c_size) return PDGEMM_EINVAL_LD;
    const int64_t lda_bytes = lda * elem_bits(prec) / 8;
    const int64_t ldb_bytes = ldb * elem_bits(prec) / 8;
    if ((lda_bytes & 15) || (ldb_bytes & 15)) return PDGEMM_EALIGN;
    if (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || ((uintptr_t)C & (c_size - 1))) return PDGEMM_EALIGN;
    if (epi != kRaw && (((uintptr_t)scale_a & 3) || ((uintptr_t)scale_b & 3))) return PDGEMM_EALIGN;
    return PDGEMM_OK;
}

int launch(int prec, int cfg, int epi, int br, int64_t M, int64_t N, int64_t K, const void *A,
           int64_t lda, const void *B, int64_t ldb, const float *scale_a, const float *scale_b,
           void *C, int64_t ldc, void *stream) {
    if (prec < 0 || prec > 2 || cfg < 0 || cfg >= kNumConfigs) return PDGEMM_EINVAL_CFG;
    if (epi != kRaw && prec == kF16) return PDGEMM_EINVAL_CFG;
    const void *fn = kernel_ptr(prec, cfg, epi, br);   // null: no such kernel (dequantizing row-major B)
    if (!fn) return PDGEMM_EINVAL_CFG;
    int rc = validate(prec, epi, br, M, N, K, A, lda, B, ldb, C, ldc, scale_a, scale_b);
    if (rc != PDGEMM_OK) return rc;
    if (M == 0 || N == 0) return PDGEMM_OK;

    const Config &c = kConfigs[cfg];
    Args args;
    // With K = 0 no operand byte is read; point at C so the clamped row
    // addresses the kernel forms are well-defined.
    args.A = K > 0 ? static_cast<const uint8_t *>(A) : static_cast<const uint8_t *>(C);
    args.B = K > 0 ? static_cast<const uint8_t *>(B) : static_cast<const uint8_t *>(C);
    args.C = C;
    args.scale_a = scale_a;
    args.scale_b = scale_b;
    args.lda_bytes = lda * elem_bits(prec) / 8;
    args.ldb_bytes = ldb * elem_bits(prec) / 8;
    args.ldc = ldc;
    args.M = (int)M;
    args.N = (int)N;
    args.K = (int)K;
    args.tiles_m = (int)cdiv(M, c.bm);
    args.tiles_n = (int)cdiv(N, c.bn);
    args.kslice = 0;
    const int64_t blocks = (int64_t)args.tiles_m * args.tiles_n;
    const int threads = (c.bm / c.wm) * (c.bn / c.wn) * c.ks * kWave;
    // a launch counts its work-items in 32 bits
    if (blocks * threads > (int64_t)UINT32_MAX) return PDGEMM_EINVAL_DIM;

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

// zeroes the M x N block of a 32-bit C (row stride ldc): a workgroup clears
// 1024 columns (four coalesced passes of 256) of every gridDim.y-th row
__global__ __launch_bounds__(256) void zero_rows_kernel(int32_t *C, int64_t ldc, int M, int N) {
    const int c0 = blockIdx.x * 1024 + threadIdx.x;
    for (int64_t r = blockIdx.y; r < M; r += gridDim.y) {
        int32_t *const row = C + r * ldc;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (c0 + 256 * j < N) row[c0 + 256 * j] = 0;
    }
}

// Tiles a K split across workgroups runs on: 64 x 64 and 128 x 64 (the
// atomic epilogue needs a tile without an in-workgroup K split)
template <int P, int BR>
const void *splitk_kernel_ptr(int cfg) {
    switch (cfg) {
    case 2: return kernel_for<P, 2, kAtomicAdd, BR>();
    case 5: return kernel_for<P, 5, kAtomicAdd, BR>();
    default: return nullptr;
    }
}

const void *splitk_kernel_ptr(int prec, int cfg, int br) {
    switch (prec * 2 + (br == kBRow)) {
    case kF16 * 2: return splitk_kernel_ptr<kF16, kBCol>(cfg);
    case kF16 * 2 + 1: return splitk_kernel_ptr<kF16, kBRow>(cfg);
    case kI8 * 2: return splitk_kernel_ptr<kI8, kBCol>(cfg);
    case kI8 * 2 + 1: return splitk_kernel_ptr<kI8, kBRow>(cfg);
    case kI4 * 2: return splitk_kernel_ptr<kI4, kBCol>(cfg);
    case kI4 * 2 + 1: return splitk_kernel_ptr<kI4, kBRow>(cfg);
    default: return nullptr;
    }
}

// A GEMM with K split over `splits` ranges of whole stages, each range a
// grid row of workgroups adding its partial tile into C, which is zeroed
// first.  Integer sums are exact in any order, so the result is the plain
// GEMM's.  FP16 takes at most two ranges: 0 + x + y and 0 + y + x round
// alike (binary32 addition commutes), so the result does not depend on
// which range lands first, though it may differ from the one-range sum in
// its last bits.
int launch_splitk(int prec, int cfg, int br, int splits, int64_t M, int64_t N, int64_t K, const void *A,
                  int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc, void *stream) {
    if (cfg < 0 || cfg >= kNumConfigs || splits < 1) return PDGEMM_EINVAL_CFG;
    const void *fn = splitk_kernel_ptr(prec, cfg, br);
    if (!fn) return PDGEMM_EINVAL_CFG;
    int rc = validate(prec, kRaw, br, M, N, K, A, lda, B, ldb, C, ldc, nullptr, nullptr);
    if (rc != PDGEMM_OK) return rc;
    if (M == 0 || N == 0) return PDGEMM_OK;
    if (K == 0 || splits == 1) return launch(prec, cfg, kRaw, br, M, N, K, A, lda, B, ldb, nullptr, nullptr, C, ldc,
                                             stream);
    const Config &c = kConfigs[cfg];
    const int64_t stage_k = 128 * 8 / elem_bits(prec);            // values of K in a 128-byte stage
    const int64_t kslice = cdiv(cdiv(K, splits), stage_k) * stage_k;
    const int64_t ranges = cdiv(K, kslice);
    if (prec == kF16 && ranges > 2) return PDGEMM_EINVAL_CFG;   // x + y = y + x, but (x + y) + z != x + (y + z)
    Args args;
    args.A = static_cast<const uint8_t *>(A);
    args.B = static_cast<const uint8_t *>(B);
    args.C = C;
    args.scale_a = nullptr;
    args.scale_b = nullptr;
    args.lda_bytes = lda * elem_bits(prec) / 8;
    args.ldb_bytes = ldb * elem_bits(prec) / 8;
    args.ldc = ldc;
    args.M = (int)M;
    args.N = (int)N;
    args.K = (int)K;
    args.tiles_m = (int)cdiv(M, c.bm);
    args.tiles_n = (int)cdiv(N, c.bn);
    args.kslice = (int)kslice;
    const int64_t blocks = (int64_t)args.tiles_m * args.tiles_n;
    const int threads = (c.bm / c.wm) * (c.bn / c.wn) * c.ks * kWave;
    if (blocks * threads > (int64_t)UINT32_MAX || ranges > 65535) return PDGEMM_EINVAL_DIM;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *zargs[] = {&C, &ldc, &args.M, &args.N};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&zero_rows_kernel),
                                   dim3((unsigned)cdiv(N, 1024), (unsigned)std::min<int64_t>(M, 1024)), dim3(256), zargs, 0, s);
    if (e != hipSuccess) return (int)e;
    void *kargs[] = {&args};
    e = hipLaunchKernel(fn, dim3((unsigned)blocks, (unsigned)ranges), dim3(threads), kargs, 0, s);
    if (e != hipSuccess) return (int)e;
    if (sync_check_enabled()) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return (int)e;
    }
    return PDGEMM_OK;
}

// The GEMM (raw sums) as the entry points without a configuration run it:
// the picked tile, with K split across workgroups where pick_splits() asks.
int launch_raw(int prec, int br, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
               int64_t ldb, void *C, int64_t ldc, void *stream) {
    int cfg = 0;
    const int splits = pick_splits(prec, br, M, N, K, &cfg);
    if (splits > 1) return launch_splitk(prec, cfg, br, splits, M, N, K, A, lda, B, ldb, C, ldc, stream);
    return launch(prec, cfg, kRaw, br, M, N, K, A, lda, B, ldb, nullptr, nullptr, C, ldc, stream);
}

// ---- INT4 on the FP6 cores: tiles, workspace, launch ----

// 0: 256 x 256 with 8 waves of 128 x 64; 1: 128 x 128 with 4 waves of
// 64 x 64.  Three stages of 48 KB (24 KB for 128 x 128, so two workgroups
// share a CU).  A 256 x 256 tile of 4 waves of 128 x 128 (half the LDS reads
// per MFMA) measured 10% slower at N = 8192 and is not kept.
// (the last field: how many row blocks ahead the A fragments are read; one
// measured fastest, 2-4 were 2-7% slower at N = 8192)
struct F6Config {
    int bm, bn, wm, wn, gm, la;
};
constexpr F6Config kF6Configs[] = {
    {256, 256, 128, 64, 4, 1},
    {128, 128, 64, 64, 8, 1},
};
constexpr int kNumF6Configs = sizeof(kF6Configs) / sizeof(kF6Configs[0]);

template <int C, int E>
const void *f6_kernel_for() {
    constexpr F6Config c = kF6Configs[C];
    return reinterpret_cast<const void *>(&gemm_f6_kernel<c.bm, c.bn, c.wm, c.wn, c.gm, E, c.la>);
}

template <int E>
const void *f6_kernel_ptr(int cfg) {
    switch (cfg) {
    case 0: return f6_kernel_for<0, E>();
    case 1: return f6_kernel_for<1, E>();
    default: return nullptr;
    }
}

const void *f6_kernel_ptr(int cfg, int epi) {
    switch (epi) {
    case kRaw: return f6_kernel_ptr<kRaw>(cfg);
    case kDequantF32: return f6_kernel_ptr<kDequantF32>(cfg);
    case kDequantF16: return f6_kernel_ptr<kDequantF16>(cfg);
    default: return nullptr;
    }
}

// K blocks of an image: ceil(K / 128), padded with zero blocks to a multiple
// of the GEMM's three LDS stages
int64_t f6_blocks(int64_t K) { return cdiv(cdiv(K, kF6Block), 3) * 3; }

// image of an operand with `rows` rows of K values: 32-row groups x 128-value
// blocks of 3072 bytes
int64_t f6_image_bytes(int64_t rows, int64_t K) { return cdiv(rows, 32) * f6_blocks(K) * kF6Unit; }

// the workspace: A's image, then B's at the next multiple of 256 bytes
int64_t f6_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    return cdiv(f6_image_bytes(M, K), 256) * 256 + f6_image_bytes(N, K);
}

// The FP6 tile for a shape, or -1 where the INT8-MFMA kernels are the
// faster choice.  Back-to-back times, FP6 path (pre-pass included) vs INT8
// MFMA: 8192^3 304 vs 371 us, 4096^3 56.6 vs 61.3 us (256 x 256), but
// 2048^3 21.4 vs 13.7 us (128 x 128): with one round of tiles or fewer, the
// pre-pass and its launch do not pay.
int pick_f6(int64_t M, int64_t N, int64_t K) {
    if (M == 0 || N == 0 || K < 1024) return -1;
    if (cdiv(M, 256) * cdiv(N, 256) >= 192) return 0;
    return -1;
}

// The FP6 GEMM's arguments for two images of K values (A's M rows, B's N).
F6Args f6_gemm_args(int cfg, int64_t M, int64_t N, int64_t K, const uint8_t *img_a, const uint8_t *img_b,
                    const float *scale_a, const float *scale_b, void *C, int64_t ldc) {
    const F6Config &c = kF6Configs[cfg];
    F6Args args;
    args.A = img_a;
    args.B = img_b;
    args.C = C;
    args.scale_a = scale_a;
    args.scale_b = scale_b;
    args.a_bytes = f6_image_bytes(M, K);
    args.b_bytes = f6_image_bytes(N, K);
    args.ldc = ldc;
    args.M = (int)M;
    args.N = (int)N;
    args.nkb = (int)f6_blocks(K);
    args.tiles_m = (int)cdiv(M, c.bm);
    args.tiles_n = (int)cdiv(N, c.bn);
    return args;
}

int64_t f6_threads(int cfg) {
    const F6Config &c = kF6Configs[cfg];
    return (c.bm / c.wm) * (c.bn / c.wn) * kWave;
}

// pre-pass workgroups for one operand (four 32-row x 128-value units each)
int64_t f6_pack_blocks(int64_t rows, int64_t K) { return cdiv(cdiv(rows, 32) * f6_blocks(K), 4); }

int launch_f6(int cfg, int epi, int br, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
              const void *B, int64_t ldb, const float *scale_a, const float *scale_b, void *C, int64_t ldc,
              void *ws, int64_t ws_bytes, void *stream) {
    if (cfg < 0 || cfg >= kNumF6Configs) return PDGEMM_EINVAL_CFG;
    int rc = validate(kI4, epi, br, M, N, K, A, lda, B, ldb, C, ldc, scale_a, scale_b);
    if (rc != PDGEMM_OK) return rc;
    if (M == 0 || N == 0) return PDGEMM_OK;
    if (K == 0)   // nothing to convert: the K = 0 result of the INT8-MFMA kernels
        return launch(kI4, pick(kI4, M, N, K), epi, br, M, N, K, A, lda, B, ldb, scale_a, scale_b, C, ldc,
                      stream);
    if (ws_bytes < 0) return PDGEMM_EWORKSPACE;
    if (!ws) return PDGEMM_ENULL;
    if (((uintptr_t)ws & 15) || ws_bytes < f6_workspace_bytes(M, N, K)) return PDGEMM_EWORKSPACE;

    const int64_t a_img = f6_image_bytes(M, K);
    uint8_t *const img_a = static_cast<uint8_t *>(ws);
    uint8_t *const img_b = img_a + cdiv(a_img, 256) * 256;

    F6PackArgs pk;
    pk.op[0] = {static_cast<const uint8_t *>(A), img_a, lda / 2, (int)M, (int)cdiv(M, 32), 0};
    pk.op[1] = {static_cast<const uint8_t *>(B), img_b, ldb / 2, (int)N, (int)cdiv(N, 32), br == kBRow};
    pk.K = (int)K;
    pk.nkb = (int)f6_blocks(K);
    const int64_t blocks_a = f6_pack_blocks(M, K);
    const int64_t blocks_b = f6_pack_blocks(N, K);
    pk.blocks_a = (int)blocks_a;
    F6Args args = f6_gemm_args(cfg, M, N, K, img_a, img_b, scale_a, scale_b, C, ldc);
    const int64_t blocks = (int64_t)args.tiles_m * args.tiles_n;
    const int64_t threads = f6_threads(cfg);
    // launches count their work-items in 32 bits
    if (blocks * threads > (int64_t)UINT32_MAX || (blocks_a + blocks_b) * 256 > (int64_t)UINT32_MAX)
        return PDGEMM_EINVAL_DIM;

    hipStream_t s = static_cast<hipStream_t>(stream);
    void *pargs[] = {&pk};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&f6_pack_kernel),
                                   dim3((unsigned)(blocks_a + blocks_b)), dim3(256), pargs, 0, s);
    if (e != hipSuccess) return (int)e;
    void *gargs[] = {&args};
    e = hipLaunchKernel(f6_kernel_ptr(cfg, epi), dim3((unsigned)blocks), dim3((unsigned)threads), gargs, 0, s);
    if (e != hipSuccess) return (int)e;
    if (sync_check_enabled()) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return (int)e;
    }
    return PDGEMM_OK;
}

// One operand into its FP6 image: `rows` rows of K values packed along K
// (A, or a column-major B given as its N rows), or (rowmajor) the K x rows
// row-major B packed along its rows.  The same checks, in the same order,
// as the GEMM's for that operand, then the image's.
int pack_f6(int64_t rows, int64_t K, const void *src, int64_t ld, int rowmajor, void *img, int64_t img_bytes,
            void *stream) {
    if (rows < 0 || K < 0) return PDGEMM_EINVAL_DIM;
    if (rows > INT32_MAX || K > PDGEMM_I4_MAX_K) return PDGEMM_EINVAL_DIM;
    if (ld < (rowmajor ? rows : K)) return PDGEMM_EINVAL_LD;
    if ((K & 1) || (ld & 1)) return PDGEMM_EINVAL_I4;
    if (img_bytes < 0) return PDGEMM_EWORKSPACE;
    if (rows == 0 || K == 0) return PDGEMM_OK;   // an empty image
    if (!src || !img) return PDGEMM_ENULL;
    if (ld > kMaxRowBytes * 2) return PDGEMM_EINVAL_LD;
    if (((ld / 2) & 15) || ((uintptr_t)src & 15)) return PDGEMM_EALIGN;
    if (((uintptr_t)img & 15) || img_bytes < f6_image_bytes(rows, K)) return PDGEMM_EWORKSPACE;
    const int64_t blocks = f6_pack_blocks(rows, K);
    if (blocks * 256 > (int64_t)UINT32_MAX) return PDGEMM_EINVAL_DIM;
    F6PackArgs pk;
    pk.op[0] = {static_cast<const uint8_t *>(src), static_cast<uint8_t *>(img), ld / 2, (int)rows,
                (int)cdiv(rows, 32), rowmajor ? 1 : 0};
    pk.op[1] = pk.op[0];   // unused: every workgroup converts op[0]
    pk.K = (int)K;
    pk.nkb = (int)f6_blocks(K);
    pk.blocks_a = (int)blocks;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *pargs[] = {&pk};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&f6_pack_kernel), dim3((unsigned)blocks),
                                   dim3(256), pargs, 0, s);
    if (e != hipSuccess) return (int)e;
    if (sync_check_enabled()) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return (int)e;
    }
    return PDGEMM_OK;
}

// The FP6 tile for a GEMM whose B image is given: no B pre-pass to pay for,
// so the FP6 cores win down to one round of 128 x 128 tiles; 256 x 256 where
// it gives most CUs a tile.  (M x 8192 x 8192: M = 2048 75.8 us on 256 x 256
// against 89.0 on 128 x 128; M = 1024 45.6 against 60.0.)
int pick_f6_packed(int64_t M, int64_t N) { return cdiv(M, 256) * cdiv(N, 256) >= 192 ? 0 : 1; }

// A GEMM with B given as its FP6 image (packed with the same K): A is
// converted into the workspace, then the GEMM runs on the two images.
int launch_f6_packed_b(int cfg, int epi, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                       const void *img_b, int64_t img_b_bytes, const float *scale_a, const float *scale_b,
                       void *C, int64_t ldc, void *ws, int64_t ws_bytes, void *stream) {
    if (cfg < -1 || cfg >= kNumF6Configs) return PDGEMM_EINVAL_CFG;
    if (M < 0 || N < 0 || K < 0) return PDGEMM_EINVAL_DIM;
    if (M > INT32_MAX || N > INT32_MAX || K > PDGEMM_I4_MAX_K) return PDGEMM_EINVAL_DIM;
    if (lda < K || ldc < N) return PDGEMM_EINVAL_LD;
    if ((K & 1) || (lda & 1)) return PDGEMM_EINVAL_I4;
    if (ws_bytes < 0 || img_b_bytes < 0) return PDGEMM_EWORKSPACE;
    if (M == 0 || N == 0) return PDGEMM_OK;
    if (!C || (K > 0 && (!A || !img_b || !ws))) return PDGEMM_ENULL;
    if (epi != kRaw && (!scale_a || !scale_b)) return PDGEMM_ENULL;
    const int64_t c_size = epi == kDequantF16 ? 2 : 4;
    if (lda > kMaxRowBytes * 2 || ldc > kMaxRowBytes / c_size) return PDGEMM_EINVAL_LD;
    if (((lda / 2) & 15) || ((uintptr_t)A & 15) || ((uintptr_t)C & (c_size - 1))) return PDGEMM_EALIGN;
    if (epi != kRaw && (((uintptr_t)scale_a & 3) || ((uintptr_t)scale_b & 3))) return PDGEMM_EALIGN;
    if (K > 0 && (((uintptr_t)img_b & 15) || img_b_bytes < f6_image_bytes(N, K) || ((uintptr_t)ws & 15) ||
                  ws_bytes < f6_image_bytes(M, K)))
        return PDGEMM_EWORKSPACE;
    if (cfg < 0) cfg = pick_f6_packed(M, N);
    F6Args args = f6_gemm_args(cfg, M, N, K, static_cast<const uint8_t *>(ws),
                               static_cast<const uint8_t *>(img_b), scale_a, scale_b, C, ldc);
    const int64_t blocks = (int64_t)args.tiles_m * args.tiles_n;
    const int64_t threads = f6_threads(cfg);
    if (blocks * threads > (int64_t)UINT32_MAX || f6_pack_blocks(M, K) * 256 > (int64_t)UINT32_MAX)
        return PDGEMM_EINVAL_DIM;
    if (K > 0) {
        const int rc = pack_f6(M, K, A, lda, 0, ws, ws_bytes, stream);
        if (rc != PDGEMM_OK) return rc;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *gargs[] = {&args};
    hipError_t e = hipLaunchKernel(f6_kernel_ptr(cfg, epi), dim3((unsigned)blocks), dim3((unsigned)threads),
                                   gargs, 0, s);
    if (e != hipSuccess) return (int)e;
    if (sync_check_enabled()) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return (int)e;
    }
    return PDGEMM_OK;
}

// the workspace entry points: the FP6 path where it is picked, else the
// INT8-MFMA kernels (which need no workspace)
int launch_i4_ws(int epi, int br, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                 int64_t ldb, const float *scale_a, const float *scale_b, void *C, int64_t ldc, void *ws,
                 int64_t ws_bytes, void *stream) {
    const int f = pick_f6(M, N, K);
    if (f < 0)
        return epi == kRaw ? launch_raw(kI4, br, M, N, K, A, lda, B, ldb, C, ldc, stream)
                           : launch(kI4, pick(kI4, M, N, K), epi, br, M, N, K, A, lda, B, ldb, scale_a, scale_b, C,
                                    ldc, stream);
    return launch_f6(f, epi, br, M, N, K, A, lda, B, ldb, scale_a, scale_b, C, ldc, ws, ws_bytes, stream);
}

// ---- the allocation-free INT4 entry point ----
//
// gemm_i4_noalloc serves callers that cannot allocate (code under graph
// capture, serving loops, harnesses that forbid it): its workspace is a
// fixed file-scope device array, one copy per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel (in host code
// it is a stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kScratchBytes = int64_t(128) << 20;   // 128 MiB: enough for 8192^3
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// This device's copy of `scratch` (its address), looked up on first use.
int scratch_for(void *stream, void **out) {
    int dev = 0;
    hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;   // beyond the address table
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return (int)e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return (int)e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return (int)e;
        if (e2 != hipSuccess) return (int)e2;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PDGEMM_OK;
}

}  // namespace

extern "C" {

int gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
             const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream) {
    return launch_raw(kF16, kBCol, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_i8(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
            const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    return launch_raw(kI8, kBCol, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_i4(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
            const uint8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    return launch_raw(kI4, kBCol, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_i8_dequant(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                    const int8_t *B, int64_t ldb, const float *scale_a, const float *scale_b,
                    void *C, int64_t ldc, int out_f16, void *stream) {
    return launch(kI8, pick(kI8, M, N, K), out_f16 ? kDequantF16 : kDequantF32, kBCol, M, N, K, A, lda, B,
                  ldb, scale_a, scale_b, C, ldc, stream);
}

int gemm_i4_dequant(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                    const uint8_t *B, int64_t ldb, const float *scale_a, const float *scale_b,
                    void *C, int64_t ldc, int out_f16, void *stream) {
    return launch(kI4, pick(kI4, M, N, K), out_f16 ? kDequantF16 : kDequantF32, kBCol, M, N, K, A, lda, B,
                  ldb, scale_a, scale_b, C, ldc, stream);
}

int pdgemm_gemm_cfg(int prec, int cfg, int64_t M, int64_t N, int64_t K, const void *A,
                    int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
                    void *stream) {
    return launch(prec, cfg, kRaw, kBCol, M, N, K, A, lda, B, ldb, nullptr, nullptr, C, ldc, stream);
}

int pdgemm_dequant_cfg(int prec, int cfg, int64_t M, int64_t N, int64_t K, const void *A,
                       int64_t lda, const void *B, int64_t ldb, const float *scale_a,
                       const float *scale_b, void *C, int64_t ldc, int out_f16, void *stream) {
    if (prec == kF16) return PDGEMM_EINVAL_CFG;
    return launch(prec, cfg, out_f16 ? kDequantF16 : kDequantF32, kBCol, M, N, K, A, lda, B, ldb, scale_a,
                  scale_b, C, ldc, stream);
}

int gemm_f16_rowb(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                  const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream) {
    return launch_raw(kF16, kBRow, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_i8_rowb(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                 const int8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    return launch_raw(kI8, kBRow, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int gemm_i4_rowb(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                 const uint8_t *B, int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    return launch_raw(kI4, kBRow, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int pdgemm_gemm_rowb_cfg(int prec, int cfg, int64_t M, int64_t N, int64_t K, const void *A,
                         int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
                         void *stream) {
    return launch(prec, cfg, kRaw, kBRow, M, N, K, A, lda, B, ldb, nullptr, nullptr, C, ldc,
                  stream);
}

int64_t pdgemm_i4_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || pick_f6(M, N, K) < 0) return 0;
    return f6_workspace_bytes(M, N, K);
}

int pdgemm_i4_f6_pick(int64_t M, int64_t N, int64_t K) { return pick_f6(M, N, K); }

int pdgemm_i4_f6_num_configs(void) { return kNumF6Configs; }

int64_t pdgemm_i4_f6_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return f6_workspace_bytes(M, N, K);
}

int gemm_i4_ws(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
               int32_t *C, int64_t ldc, void *workspace, int64_t workspace_bytes, void *stream) {
    return launch_i4_ws(kRaw, kBCol, M, N, K, A, lda, B, ldb, nullptr, nullptr, C, ldc, workspace,
                        workspace_bytes, stream);
}

int gemm_i4_rowb_ws(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B,
                    int64_t ldb, int32_t *C, int64_t ldc, void *workspace, int64_t workspace_bytes,
                    void *stream) {
    return launch_i4_ws(kRaw, kBRow, M, N, K, A, lda, B, ldb, nullptr, nullptr, C, ldc, workspace,
                        workspace_bytes, stream);
}

int gemm_i4_dequant_ws(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B,
                       int64_t ldb, const float *scale_a, const float *scale_b, void *C, int64_t ldc,
                       int out_f16, void *workspace, int64_t workspace_bytes, void *stream) {
    return launch_i4_ws(out_f16 ? kDequantF16 : kDequantF32, kBCol, M, N, K, A, lda, B, ldb, scale_a, scale_b,
                        C, ldc, workspace, workspace_bytes, stream);
}

int pdgemm_i4_f6_cfg(int cfg, int b_rowmajor, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                     const void *B, int64_t ldb, const float *scale_a, const float *scale_b, void *C,
                     int64_t ldc, int out_f16, void *workspace, int64_t workspace_bytes, void *stream) {
    const int epi = (scale_a || scale_b) ? (out_f16 ? kDequantF16 : kDequantF32) : kRaw;
    return launch_f6(cfg, epi, b_rowmajor ? kBRow : kBCol, M, N, K, A, lda, B, ldb, scale_a, scale_b, C, ldc,
                     workspace, workspace_bytes, stream);
}

int gemm_i4_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B,
                    int64_t ldb, int32_t *C, int64_t ldc, void *stream) {
    // shapes the INT8-MFMA kernels take need no workspace
    if (pick_f6(M, N, K) < 0) return launch_raw(kI4, kBCol, M, N, K, A, lda, B, ldb, C, ldc, stream);
    const int rc = validate(kI4, kRaw, kBCol, M, N, K, A, lda, B, ldb, C, ldc, nullptr, nullptr);
    if (rc != PDGEMM_OK) return rc;
    if (f6_workspace_bytes(M, N, K) > kScratchBytes) return PDGEMM_EWORKSPACE;
    void *ws = nullptr;
    const int e = scratch_for(stream, &ws);
    if (e != PDGEMM_OK) return e;
    return launch_f6(pick_f6(M, N, K), kRaw, kBCol, M, N, K, A, lda, B, ldb, nullptr, nullptr, C, ldc, ws,
                     kScratchBytes, stream);
}

int64_t pdgemm_i4_noalloc_max_bytes(void) { return kScratchBytes; }

int pdgemm_gemm_splitk_cfg(int prec, int cfg, int b_rowmajor, int splits, int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
                           void *stream) {
    return launch_splitk(prec, cfg, b_rowmajor ? kBRow : kBCol, splits, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int64_t pdgemm_i4_f6_image_bytes(int64_t rows, int64_t K) {
    if (rows < 0 || K < 0) return 0;
    return f6_image_bytes(rows, K);
}

int pdgemm_i4_f6_pack(int64_t rows, int64_t K, const uint8_t *src, int64_t ld, int src_rowmajor, void *image,
                      int64_t image_bytes, void *stream) {
    return pack_f6(rows, K, src, ld, src_rowmajor, image, image_bytes, stream);
}

int gemm_i4_packed_b(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const void *image_b,
                     int64_t image_b_bytes, int32_t *C, int64_t ldc, void *workspace, int64_t workspace_bytes,
                     void *stream) {
    return launch_f6_packed_b(-1, kRaw, M, N, K, A, lda, image_b, image_b_bytes, nullptr, nullptr, C, ldc,
                              workspace, workspace_bytes, stream);
}

int gemm_i4_dequant_packed_b(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                             const void *image_b, int64_t image_b_bytes, const float *scale_a,
                             const float *scale_b, void *C, int64_t ldc, int out_f16, void *workspace,
                             int64_t workspace_bytes, void *stream) {
    return launch_f6_packed_b(-1, out_f16 ? kDequantF16 : kDequantF32, M, N, K, A, lda, image_b, image_b_bytes,
                              scale_a, scale_b, C, ldc, workspace, workspace_bytes, stream);
}

int pdgemm_i4_packed_b_cfg(int cfg, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                           const void *image_b, int64_t image_b_bytes, const float *scale_a,
                           const float *scale_b, void *C, int64_t ldc, int out_f16, void *workspace,
                           int64_t workspace_bytes, void *stream) {
    if (cfg < 0) return PDGEMM_EINVAL_CFG;
    const int epi = (scale_a || scale_b) ? (out_f16 ? kDequantF16 : kDequantF32) : kRaw;
    return launch_f6_packed_b(cfg, epi, M, N, K, A, lda, image_b, image_b_bytes, scale_a, scale_b, C, ldc,
                              workspace, workspace_bytes, stream);
}

int pdgemm_num_configs(void) { return kNumConfigs; }

int pdgemm_pick_config(int prec, int64_t M, int64_t N, int64_t K) {
    if (prec < 0 || prec > 2) return -1;
    return pick(prec, M, N, K);
}

int pdgemm_pick_splits(int prec, int b_rowmajor, int64_t M, int64_t N, int64_t K, int *cfg) {
    int c = -1;
    const int s = (prec < 0 || prec > 2) ? -1 : pick_splits(prec, b_rowmajor ? kBRow : kBCol, M, N, K, &c);
    if (cfg) *cfg = c;
    return s;
}

int pdgemm_config_info(int cfg, int *block_m, int *block_n, int *wave_m, int *wave_n,
                       int *threads) {
    if (cfg < 0 || cfg >= kNumConfigs) return PDGEMM_EINVAL_CFG;
    const Config &c = kConfigs[cfg];
    if (block_m) *block_m = c.bm;
    if (block_n) *block_n = c.bn;
    if (wave_m) *wave_m = c.wm;
    if (wave_n) *wave_n = c.wn;
    if (threads) *threads = (c.bm / c.wm) * (c.bn / c.wn) * c.ks * kWave;
    return PDGEMM_OK;
}

const char *pdgemm_strerror(int code) {
    switch (code) {
    case PDGEMM_OK: return "success";
    case PDGEMM_EINVAL_DIM: return "invalid dimension (negative, too large, or INT4 K above 131071)";
    case PDGEMM_EINVAL_LD: return "leading dimension smaller than the row length, or a row above 4 MiB";
    case PDGEMM_ENULL: return "null pointer for an operand with nonzero extent";
    case PDGEMM_EINVAL_I4: return "INT4 K, lda and ldb must be even";
    case PDGEMM_EALIGN: return "A and B must be 16-byte aligned, A and B rows must span a multiple of 16 bytes, C and the scales must be element-aligned";
    case PDGEMM_EINVAL_CFG: return "unknown precision or tile configuration, or a dequantizing epilogue for FP16";
    case PDGEMM_EWORKSPACE:
        return "workspace or FP6 image smaller than the entry point needs, of negative size, or not 16-byte "
               "aligned";
    default: return code > 0 ? hipGetErrorString((hipError_t)code) : "unknown error";
    }
}

int pdgemm_version(void) { return 200; }

}  // extern "C"
