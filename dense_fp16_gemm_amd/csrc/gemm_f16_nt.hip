// Dense fp16 NT GEMM for MI355X (gfx950): C[M,N] = fp16_rne(A[M,K] * B[N,K]^T),
// fp32 accumulation (Tilus tutorial "Hopper matmul": page "2. Multi-Stage
// Software Pipelining", The Full Kernel; page "6. Register Reallocation,
// Multicast, and a Persistent Kernel", opening paragraphs).
//
// One kernel template, every workgroup doing every job (the pages' V2 shape,
// which suits CDNA's in-order waves sharing one barrier), plus a general
// kernel for the arguments the template's loads cannot take (per operand
// layout):
//
//  * persistent tile loop: grid = min(tiles, CUs); workgroup wg walks slots
//    wg, wg + grid, ... through the grouped, XCD-aware order of
//    tile_schedule.h (page 4 "Tile Rasterization", page 6 "Persistent Tile
//    Loop");
//  * LDS ring of STAGES K-slices (page 2 "Software Pipelining", "Multi-Stage
//    Shared Memory"), filled by gfx950 direct-to-LDS buffer loads
//    (buffer_load_dwordx4 ... lds: 16 bytes per lane straight into LDS, no
//    VGPR staging).  A DMA instruction writes 64 x 16 B contiguously, so the
//    XOR swizzle that keeps the MFMA fragment reads free of bank conflicts is
//    applied on the global side: the lane that fills physical 16-byte chunk p
//    of row r fetches logical chunk p ^ swz(r).  With two stages the refill
//    of slice kt + 2 starts right after the barrier of slice kt's last step
//    (the "early refill"), and a refill inside K carries its K offset in the
//    instruction's scalar offset;
//  * stage bookkeeping without mbarriers: "full" = s_waitcnt vmcnt(n) on the
//    wave's own DMA queue + s_barrier; "empty" = s_waitcnt lgkmcnt(0) before
//    that same barrier, so one barrier per K-slice serves both roles (page 3
//    "Producer-Consumer Barriers" describe the two roles); with two stages
//    the loop runs two slices per trip so stage offsets are compile-time
//    constants (page 2 "Loop Unrolling and Stage Indices");
//  * v_mfma_f32_32x32x16_f16 (builtin) or v_mfma_f32_16x16x32_f16 (inline
//    assembly with accumulators bound to AGPRs) with fp32 accumulators; the
//    output tile is split over a WM x WN grid of waves that share A rows and
//    B rows through LDS (page 4 "Two Consumer Warp Groups"); fragments for
//    the next K step are read while the current step's MFMAs run (the lesson
//    of the pages' V5: never let the matrix pipe drain);
//  * epilogue: round-to-nearest-even fp32 -> fp16 (v_cvt_f16_f32 under the
//    default MODE), staged through a free ring stage for 16-byte row stores
//    at any 2-byte alignment (page 6 "Shared-Memory Epilogue"), or stored
//    straight from the MFMA layout; masked M/N tails.  The staged stores are
//    non-temporal, keeping C out of L2 and the shared A and B strips in it,
//    and after an interior tile the next tile's first wait leaves them in
//    flight (vmcnt counts stores too).
//
// Operand roles: the MFMA's first operand (rows of its result block) takes
// rows of the B tile and the second operand (columns) rows of the A tile, so
// the result block is C^T and each lane ends up holding 4 consecutive N
// columns of one M row -- ready for packed fp16 stores.
//
// Tails: the buffer resource of a tile starts at its first row and covers
// exactly its valid rows, so rows beyond M (or N) read as zero; a 16-byte
// chunk beyond K is given an offset past the resource, which also reads as
// zero (the template needs K a multiple of 8, so chunks never straddle K;
// other K, and A or B not 16-byte aligned, go to the general kernel).
//
// Beyond the pages' NT form, the same template covers
//  * the other operand layouts (B stored [K, N], A stored [K, M]): such a
//    tile keeps its memory layout in LDS and its fragments are read with the
//    transposing LDS read, so each element's K order, and every result bit,
//    stays that of the NT form (see kn_swizzle);
//  * a split over K for tile counts that leave most CUs idle: a second
//    instance of each configuration runs (range, tile) work units that store
//    fp32 partials (non-temporally when they exceed the L2s), and
//    splitk_reduce_kernel sums them in range order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <mutex>
#include <type_traits>
#include <vector>
#include <stddef.h>
#include <stdint.h>

#include "gemm_f16_nt.h"
#include "tile_schedule.h"

namespace gemm_f16 {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes at any 2-byte alignment (the target's unaligned-access mode)
typedef _Float16 half8_u_t __attribute__((ext_vector_type(8), aligned(2)));
typedef _Float16 half4_u_t __attribute__((ext_vector_type(4), aligned(2)));
typedef float f32x4_u_t __attribute__((ext_vector_type(4), aligned(4)));

template <int N>
struct AccVec;
template <>
struct AccVec<16> { typedef f32x16_t type; };
template <>
struct AccVec<4> { typedef f32x4_t type; };

constexpr uint32_t OOB_OFFSET = 0x80000000u;  // past every resource: reads 0
constexpr int64_t MAX_K = int64_t(1) << 21;   // keeps BM * K * 2 < 2^31
constexpr int LDS_LIMIT = 160 * 1024;  // gfx950 LDS per workgroup
constexpr int DEFAULT_XCDS = 8;        // MI355X: 8 XCDs x 32 CUs
constexpr int DMA_BYTES = 64 * 16;     // one direct-to-LDS instruction: 64 lanes x 16 B

// XOR applied to the 16-byte chunk index of LDS tile row r (rows are BK * 2
// bytes = CHUNKS chunks), chosen per fragment shape so that the lanes the LDS
// serves together hit distinct banks.
//
// 32x32x16 fragments: 32 lanes read rows r0 .. r0 + 31 (r0 a multiple of 32)
// at one logical chunk.  The swizzle depends on r mod 32 only and makes any 8
// consecutive rows of such a read cover 128 distinct bytes of bank space and
// any 16 consecutive rows 256 distinct bytes, i.e. conflict-free whether a
// ds_read_b128 is served 8 or 16 lanes at a time from 32 or 64 banks.
//   8 chunks (128 B rows): row parity picks the 128-byte half of a 256-byte
//   bank line, so the chunk XOR must differ across 8 consecutive rows and
//   across the 8 even (odd) rows of 16: (r & 7) ^ ((r >> 3) & 3).
//   4 chunks (64 B rows): r mod 4 picks the 64-byte quarter; the XOR must
//   differ across the 4 rows of one quarter within 16 rows and across the
//   even (odd) rows of 8: ((r >> 1) & 3) ^ ((r >> 3) & 1).
//   16 chunks (256 B rows): every row starts on the same bank, so the XOR
//   must differ across any 16 consecutive rows: r & 15.
//
// 16x16x32 fragments (128 B rows only): lane l reads row l % 16 at logical
// chunk c + l / 16, so four lanes share each row.  With the 32x32 swizzle
// these reads cost twice the LDS cycles of a contiguous read (the hardware
// counter put half of all LDS cycles in bank conflicts).  The pattern that
// avoids this was found by measurement, not derived: all 4096 swizzles
// linear in the bits of r mod 16 were timed as 16x16 fragment reads at both
// K steps and both 16-row parities, and this one (one of 392 that read as
// fast as a contiguous 1 KB) was chosen:
//   bit 0 = r1, bit 1 = r2, bit 2 = r0 ^ r3.
template <int CHUNKS, int MI = 32>
__host__ __device__ constexpr int chunk_swizzle(int r)
{
    if (MI == 16)
        return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2);
    if (CHUNKS == 16) return r & 15;
    return CHUNKS == 8 ? ((r & 7) ^ ((r >> 3) & 3)) : (((r >> 1) & 3) ^ ((r >> 3) & 1));
}

// B stored [K, N] (N contiguous): its LDS tile keeps that layout, one row of
// BN halves per k, and the MFMA fragments are read with the transposing LDS
// read (ds_read_b64_tr_b16).  Within each group of 16 lanes that read takes
// the 8-byte pieces the 16 lanes address as a 16 x 4 block and returns to lane
// j element j % 4 of the pieces of lanes j / 4, j / 4 + 4, j / 4 + 8 and
// j / 4 + 12 (measured).  Lane i addressing row k0 + i / 4 at columns
// n0 + 4 (i % 4) .. + 3 therefore gets column n0 + j at rows k0 .. k0 + 3:
// four consecutive k of one n, the 16x16x32 operand layout; two reads make
// the lane's eight.  One read touches 16 rows (4 per lane group, groups 8
// rows apart) at 32 bytes each; rows of 256 or 512 bytes start on the same
// bank, so each row's 16-byte chunks are XORed with an even value that spreads
// those 16 rows over 8 distinct 32-byte windows (two rows per window, the
// minimum for 512 bytes):
//   chunk ^ 2 ((k & 3) | ((k >> 3) & 1) << 2)
// Rows of 128 bytes (a 64-wide tile) alternate between the two halves of the
// 256-byte bank window, so only the four even (odd) rows of each half-wave's
// eight need distinct 32-byte windows within their half, from k's bits 1 and
// 3 (for the second read, 4 rows on, as well):
//   chunk ^ 2 (((k >> 1) & 1) | ((k >> 3) & 1) << 1)
template <int ROW_BYTES>
__host__ __device__ constexpr int kn_swizzle(int k)
{
    static_assert(ROW_BYTES == 128 || ROW_BYTES == 256 || ROW_BYTES == 512, "[K, X] tile rows");
    if (ROW_BYTES == 128) return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1));
    return 2 * ((k & 3) | (((k >> 3) & 1) << 2));
}

// MI_ picks the MFMA: 32 -> v_mfma_f32_32x32x16_f16 (16 accumulators per lane
// per block), 16 -> v_mfma_f32_16x16x32_f16 (4 per block: half the
// accumulator register traffic per flop).
// DX_ (two stages only): how many of a slice's DMA instructions are issued
// early, during the last step of the slice two before it, right after the
// barrier that frees their stage; the rest go out during the slice before.
// ADB_: double-buffer the A fragments as well as the B fragments.
// BL_: B's layout in memory: 0 = [N, K] (K contiguous, the pages' NT form),
// 1 = [K, N] (N contiguous: C = A B with B row-major).
// AL_: A's layout: 0 = [M, K] (K contiguous), 1 = [K, M] (M contiguous:
// C = A^T B or A^T B^T with A row-major [K, M]).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int MI_ = 32,
          int DSTEPS_ = 0, int DX_ = 0, int ADB_ = 0, int BL_ = 0, int AL_ = 0>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = STAGES_;
    static constexpr int BL = BL_, AL = AL_;
    static constexpr int MI = MI_;               // MFMA block edge (M and N)
    static constexpr int MK = 512 / MI;          // K per MFMA: 16 or 32
    static constexpr int ACC_N = MI * MI / 64;   // accumulators per lane per block
    // steps of a slice that carry refill DMA (0: every step with 3+ stages,
    // the first half with 2)
    static constexpr int DSTEPS = DSTEPS_;
    static constexpr int DX = DX_;
    static constexpr bool ADB = ADB_ != 0;
    typedef typename AccVec<ACC_N>::type Acc;
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = 64 * WAVES;
    // one workgroup per CU (the LDS ring takes most of the 160 KB)
    static constexpr int WAVES_PER_SIMD = WAVES <= 4 ? 1 : WAVES / 4;
    static constexpr int TM = BM / WM;           // wave tile rows (M)
    static constexpr int TN = BN / WN;           // wave tile columns (N)
    static constexpr int FM = TM / MI;           // MFMA blocks per wave along M
    static constexpr int FN = TN / MI;           // ... along N
    static constexpr int KK = BK / MK;           // MFMA K steps per K-slice
    static constexpr int ROW_BYTES = BK * 2;     // one LDS tile row
    static constexpr int CHUNKS = BK / 8;        // 16-byte chunks per row
    static constexpr int DMA_ROWS = DMA_BYTES / ROW_BYTES;   // rows per DMA instruction
    static constexpr int A_BYTES = BM * ROW_BYTES;
    static constexpr int B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    // the A tile in LDS: BM rows of BK halves (AL 0) or BK rows of BM halves
    // (AL 1); DMA instructions per wave per stage
    static constexpr int A_ROW_BYTES = AL ? BM * 2 : ROW_BYTES;
    static constexpr int A_CHUNKS = A_ROW_BYTES / 16;
    static constexpr int A_DMA_ROWS = DMA_BYTES / A_ROW_BYTES;
    static constexpr int A_LOADS = (AL ? BK : BM) / A_DMA_ROWS / WAVES;
    static constexpr int A_RB = WAVES * A_DMA_ROWS;
    static constexpr int A_NB = (16 / (A_RB < 16 ? A_RB : 16)) < A_LOADS
                                    ? (16 / (A_RB < 16 ? A_RB : 16)) : A_LOADS;
    // the B tile in LDS: BN rows of BK halves (BL 0, like A) or BK rows of
    // BN halves (BL 1)
    static constexpr int B_ROW_BYTES = BL ? BN * 2 : ROW_BYTES;
    static constexpr int B_CHUNKS = B_ROW_BYTES / 16;
    static constexpr int B_DMA_ROWS = DMA_BYTES / B_ROW_BYTES;
    static constexpr int B_LOADS = (BL ? BK : BN) / B_DMA_ROWS / WAVES;
    // [K, N] B: instruction ip covers rows ip * B_RB + ...; kn_swizzle repeats
    // every 16 rows, so lane offsets repeat every B_NB instructions and the
    // rest is a multiple of 16 rows, carried in the scalar offset
    static constexpr int B_RB = WAVES * B_DMA_ROWS;
    static constexpr int B_NB = (16 / (B_RB < 16 ? B_RB : 16)) < B_LOADS
                                    ? (16 / (B_RB < 16 ? B_RB : 16)) : B_LOADS;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    // K-contiguous parts in the fused early refill (Step with FUSED): a
    // wave's DMA instructions fill consecutive 1 KB LDS blocks in groups of
    // DMA_G (dma_block), so a group shares one M0 value and the instruction's
    // immediate offset, which moves the LDS and the global address alike,
    // steps through it; DMA_G divides the instruction count of every
    // K-contiguous part (1, the plain interleaving, elsewhere)
    static constexpr int A_KL = AL ? 4 : A_LOADS;
    static constexpr int B_KL = BL ? 4 : B_LOADS;
    static constexpr bool FUSED_REFILL = STAGES_ == 2 && DX_ == A_LOADS + B_LOADS && MI_ == 16;
    static constexpr int DMA_G = !FUSED_REFILL ? 1
                                 : (A_KL % 4 == 0 && B_KL % 4 == 0) ? 4
                                 : (A_KL % 2 == 0 && B_KL % 2 == 0) ? 2 : 1;
    // the LDS-staged epilogue writes one block row of every wave (WM * MI tile
    // rows of BN halves, rows padded by 16 bytes) into one ring stage
    static constexpr bool STAGED_OK = WM * MI * (BN * 2 + 16) <= STAGE_BYTES;
    // Double-buffered staging for tiles wholly inside M x N: two buffers of
    // EPI_RB block rows each, in the free stage and, where the ring already
    // takes more than half of the LDS (one workgroup per CU), the LDS past
    // the ring (EPI_EXTRA more bytes); 0 where two buffers of one block row
    // do not fit.
    static constexpr int EPI_BROW = WM * MI * (BN * 2 + 16);
    static constexpr int EPI_AVAIL = STAGE_BYTES + (2 * LDS_BYTES > LDS_LIMIT ? LDS_LIMIT - LDS_BYTES : 0);
    static constexpr int EPI_RB = EPI_AVAIL / (2 * EPI_BROW) < FM ? EPI_AVAIL / (2 * EPI_BROW) : FM;
    static constexpr int EPI_EXTRA = EPI_RB > 0 && 2 * EPI_RB * EPI_BROW > STAGE_BYTES
                                         ? 2 * EPI_RB * EPI_BROW - STAGE_BYTES : 0;
    static_assert(BK == 32 || BK == 64 || BK == 128, "BK is 32, 64 or 128");
    static_assert(KK % 2 == 0, "fragment double buffer alternates within a slice");
    static_assert(MI == 32 || MI == 16, "MFMA is 32x32x16 or 16x16x32");
    static_assert(MI == 32 || CHUNKS == 8, "16x16x32 fragments need 128-byte rows");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32-row blocks");
    // No configuration has a single wave row.  Trial instances with WM = 1
    // and 32 x 32 x 16 MFMAs (32 x 64 and 32 x 128 tiles, K 128 per stage)
    // returned wrong results, for a cause not found (one with 16 x 16 x 32
    // MFMAs was correct), so the template accepts none.
    static_assert(WM >= 2, "at least two wave rows");
    static_assert((AL ? BK % (A_DMA_ROWS * WAVES) : BM % (DMA_ROWS * WAVES)) == 0 &&
                      (BL ? BK % (B_DMA_ROWS * WAVES) : BN % (DMA_ROWS * WAVES)) == 0,
                  "every wave issues the same number of DMA instructions");
    static_assert(BL == 0 || (MI == 16 && (BN == 64 || BN == 128 || BN == 256) && BK % 32 == 0),
                  "[K, N] B: 16x16x32 fragments, 128-, 256- or 512-byte rows");
    static_assert(AL == 0 || (MI == 16 && (BM == 64 || BM == 128 || BM == 256) && BK % 32 == 0),
                  "[K, M] A: 16x16x32 fragments, 128-, 256- or 512-byte rows");
    static_assert(STAGES >= 2, "need at least a double buffer");
    static_assert(LDS_BYTES <= LDS_LIMIT, "LDS ring exceeds 160 KB");
    static_assert((STAGES - 1) * LOADS <= 63, "vmcnt counts at most 63 loads");
    static_assert(DX == 0 || (STAGES == 2 && DX <= LOADS), "early refill needs exactly two stages");
    // the 16x16x32 MFMAs are hand-issued (see Step): an accumulator must not
    // feed the MFMA right after the one that wrote it
    static_assert(MI == 32 || FM * FN >= 4, "16x16 blocks per wave");
};

struct Params {
    const uint16_t *A;
    const uint16_t *B;
    uint16_t *C;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n, tiles;
    int32_t swizzle, grid, xcds;
    int32_t staged;  // 1: stage C through LDS for row-contiguous stores
    // Split over K: work unit u (after the XCD order) is tile u % (tiles_m *
    // tiles_n) over K range [s * k_split, min((s + 1) * k_split, K)), s = u /
    // (tiles_m * tiles_n); `tiles` counts the units.  With splits > 1 each
    // unit stores its fp32 partial sums to W + s * split_stride (an M x N
    // row-major matrix) instead of writing C.
    int32_t splits, k_split;
    int64_t split_stride;
    float *W;
    int32_t nt_w;   // store the partials non-temporally (they exceed the L2s)
};

// Buffer resource (V#) for raw byte addressing of `bytes` bytes at `base`:
// stride 0, gfx9 data-format word; offsets >= bytes read as zero.
__device__ __forceinline__ i32x4_t make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(a & 0xffffffffu));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((a >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(bytes));
    r.w = 0x00020000;
    return r;
}

// One direct-to-LDS load: lane l copies 16 bytes from rsrc + voff into LDS
// byte address lds + 16 * l.  M0 carries the wave-uniform LDS base; the
// s_nop covers the M0-write -> LDS-DMA hazard, which the compiler cannot see
// inside an asm statement.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t lds)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// All of this wave's LDS reads have returned, then workgroup barrier.  The
// "memory" clobber also stops the compiler moving LDS reads across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Coordinates and buffer resources of one output tile.
struct Tile {
    int32_t m0, n0;
    int32_t split, klen;                 // K split index and the unit's K length
    i32x4_t rsrc_a, rsrc_b;              // buffer resources for the DMA asm
};

// SPLIT: the kernel instance for K split into ranges (see Params); the
// unsplit instance carries none of that arithmetic.
template <class CF, bool SPLIT>
__device__ __forceinline__ Tile make_tile(const Params &p, int32_t slot, uint32_t row_pitch)
{
    int32_t tile_m, tile_n;
    const int32_t unit = slot_to_linear(slot, p.grid, p.tiles, p.xcds);
    Tile t;
    int32_t k0 = 0;
    if constexpr (SPLIT) {
        const int32_t tiles_mn = p.tiles_m * p.tiles_n;
        t.split = static_cast<int32_t>(static_cast<uint32_t>(unit) / static_cast<uint32_t>(tiles_mn));
        grouped_tile(unit - t.split * tiles_mn, p.tiles_m, p.tiles_n, p.swizzle, tile_m, tile_n);
        k0 = t.split * p.k_split;
        t.klen = min(p.k_split, p.K - k0);
    } else {
        t.split = 0;
        grouped_tile(unit, p.tiles_m, p.tiles_n, p.swizzle, tile_m, tile_n);
        // opaque, as the unit's K length is in the split instance: the lane
        // masks of the K-tail checks (dma_one) are then computed per tile,
        // not hoisted out of the tile loop to hold scalar registers
        // throughout the kernel
        t.klen = p.K;
        asm volatile("" : "+s"(t.klen));
    }
    t.m0 = tile_m * CF::BM;
    t.n0 = tile_n * CF::BN;
    // the resource starts at the unit's first column and covers exactly the
    // tile's valid rows: rows past M (N) read 0; columns past the unit's K
    // range are never addressed (they get an out-of-range offset)
    const int32_t rows_a = min(CF::BM, p.M - t.m0);
    const int32_t rows_b = min(CF::BN, p.N - t.n0);
    if constexpr (CF::AL == 0) {
        t.rsrc_a = make_rsrc(p.A + static_cast<int64_t>(t.m0) * p.K + k0,
                             static_cast<uint32_t>(rows_a) * row_pitch);
    } else {
        // [K, M]: rows are k, as for a [K, N] B (the host keeps K M 2 below 2^31)
        t.rsrc_a = make_rsrc(p.A + static_cast<int64_t>(k0) * p.M + t.m0,
                             static_cast<uint32_t>(t.klen) * static_cast<uint32_t>(p.M) * 2u -
                                 static_cast<uint32_t>(t.m0) * 2u);
    }
    if constexpr (CF::BL == 0) {
        t.rsrc_b = make_rsrc(p.B + static_cast<int64_t>(t.n0) * p.K + k0,
                             static_cast<uint32_t>(rows_b) * row_pitch);
    } else {
        // [K, N]: rows are k.  The resource starts at (k0, n0) and spans the
        // unit's rows; columns past N get out-of-range offsets per lane
        // (the host keeps K N 2 below 2^32)
        t.rsrc_b = make_rsrc(p.B + static_cast<int64_t>(k0) * p.N + t.n0,
                             static_cast<uint32_t>(t.klen) * static_cast<uint32_t>(p.N) * 2u -
                                 static_cast<uint32_t>(t.n0) * 2u);
    }
    return t;
}

// kn_swizzle of the A (IS_A) or B tile when that operand is stored k-outermost
template <class CF, bool IS_A>
__device__ __forceinline__ int kn_swizzle_of(int r)
{
    if constexpr (IS_A ? CF::AL == 1 : CF::BL == 1)
        return kn_swizzle<IS_A ? CF::A_ROW_BYTES : CF::B_ROW_BYTES>(r);
    else
        return 0;
}

// The LDS block (DMA_ROWS rows, 1 KB) that DMA instruction ip of a
// K-contiguous part fills for wave `wave`: groups of DMA_G consecutive
// blocks per wave, the groups of the waves interleaved (with DMA_G = 1,
// instruction ip of every wave in turn).  Parts stored k-outermost keep
// ip * WAVES + wave.
template <class CF>
__host__ __device__ constexpr int dma_block(int ip, int wave)
{
    return (ip / CF::DMA_G) * (CF::DMA_G * CF::WAVES) + wave * CF::DMA_G + ip % CF::DMA_G;
}

// This wave's base LDS addresses for its DMA blocks: `kc` for the parts
// stored K-contiguous (block dma_block(ip, wave) = wave * DMA_G + a constant),
// `kn` for the parts stored k-outermost (block ip * WAVES + wave).  Every M0
// value is one of these plus a constant.  The empty asm makes both opaque to
// the optimiser, so each M0 value is computed from them where it is used: the
// compiler cannot fold the wave's offset into a per-instruction constant and
// hoist one scalar register per DMA instruction out of the tile loop, which
// would hold them across the whole kernel.  Made once per tile (and again
// for the next tile's prefill), it costs one scalar add per distinct M0.
struct DmaLds {
    uint32_t kc, kn;
};

template <class CF>
__device__ __forceinline__ DmaLds dma_lds(uint32_t lds0, int wave)
{
    // the inputs are made opaque, so the wave's offsets are recomputed here
    // too rather than held from the kernel's start
    asm volatile("" : "+s"(lds0), "+s"(wave));
    return DmaLds{lds0 + static_cast<uint32_t>(wave * CF::DMA_G) * DMA_BYTES,
                  lds0 + static_cast<uint32_t>(wave) * DMA_BYTES};
}

// One of this wave's DMA instructions for K-slice `kt` of tile `t`, into ring
// stage `stage`.  Instruction i fills rows R = (i' * WAVES + wave) * DMA_ROWS
// .. R + DMA_ROWS - 1 of the A tile (i < A_LOADS, i' = i) or of the B tile
// (i' = i - A_LOADS); lane l writes physical chunk l % CHUNKS of row
// R + l / CHUNKS, so it fetches logical chunk (l % CHUNKS) ^ swz(row).  A
// chunk at or past K gets an offset beyond the resource and lands as zeros.
template <class CF>
__device__ __forceinline__ void dma_one(const Params &p, const Tile &t, int stage, int kt, int i,
                                        const DmaLds &lb, int wave, int lane, uint32_t row_pitch)
{
    const uint32_t k0 = static_cast<uint32_t>(kt) * CF::BK;
    const bool is_a = i < CF::A_LOADS;
    const int rblk = (is_a ? i : i - CF::A_LOADS) * CF::WAVES + wave;
    if ((is_a && CF::AL == 1) || (!is_a && CF::BL == 1)) {
        // row k0 + r of a [K, M] / [K, N] tile: lane l fetches logical chunk
        // (l % chunks) ^ kn_swizzle(r) of it (8 columns), zero past K, M or N
        const int dma_rows = is_a ? CF::A_DMA_ROWS : CF::B_DMA_ROWS;
        const int chunks = is_a ? CF::A_CHUNKS : CF::B_CHUNKS;
        const int32_t x0 = is_a ? t.m0 : t.n0, xn = is_a ? p.M : p.N;
        const int r = rblk * dma_rows + lane / chunks;
        const int chunk = (lane % chunks) ^ (is_a ? kn_swizzle_of<CF, true>(r)
                                                  : kn_swizzle_of<CF, false>(r));
        const uint32_t ld = static_cast<uint32_t>(xn) * 2u;
        uint32_t v = (k0 + r) * ld + chunk * 16;
        if (k0 + r >= static_cast<uint32_t>(t.klen) || x0 + chunk * 8 >= xn) v = OOB_OFFSET;
        dma16(is_a ? t.rsrc_a : t.rsrc_b, v,
              lb.kn + stage * CF::STAGE_BYTES + (is_a ? 0 : CF::A_BYTES) +
                  (rblk - wave) * DMA_BYTES);
        return;
    }
    const int kb = dma_block<CF>(is_a ? i : i - CF::A_LOADS, wave);
    const int row = kb * CF::DMA_ROWS + lane / CF::CHUNKS;
    const int chunk = (lane % CF::CHUNKS) ^ chunk_swizzle<CF::CHUNKS, CF::MI>(row);
    uint32_t v = static_cast<uint32_t>(row) * row_pitch + chunk * 16 + k0 * 2;
    if (k0 + chunk * 8 >= static_cast<uint32_t>(t.klen)) v = OOB_OFFSET;
    dma16(is_a ? t.rsrc_a : t.rsrc_b, v,
          lb.kc + stage * CF::STAGE_BYTES + (is_a ? 0 : CF::A_BYTES) +
              (kb - wave * CF::DMA_G) * DMA_BYTES);
}

// Fast form of dma_one for a slice that lies wholly inside K: the lane's
// row offset `voff` (from dma_lane_offset, fixed for the whole kernel) goes in
// the VGPR operand and the slice's K offset in the scalar offset, so issuing
// it takes no vector ALU work.  Rows past M or N still start past the
// resource's range on their own, so they read zeros as before.
// (ip: the instruction's index within the A part or within the B part; both
// parts use the same row pattern)
template <class CF>
__device__ __forceinline__ uint32_t dma_lane_offset(int ip, int wave, int lane, uint32_t row_pitch)
{
    const int row = dma_block<CF>(ip, wave) * CF::DMA_ROWS + lane / CF::CHUNKS;
    const int chunk = (lane % CF::CHUNKS) ^ chunk_swizzle<CF::CHUNKS, CF::MI>(row);
    return static_cast<uint32_t>(row) * row_pitch + chunk * 16;
}

// The same for the [K, N] B tile: fixed per tile (its columns past N get an
// out-of-range offset), with the slice's row offset k0 N 2 in the scalar
// offset.
template <class CF, bool IS_A>
__device__ __forceinline__ uint32_t dma_lane_offset_kn(int ip, int wave, int lane, int32_t x0,
                                                       int32_t xn)
{
    constexpr int DMA_ROWS_X = IS_A ? CF::A_DMA_ROWS : CF::B_DMA_ROWS;
    constexpr int CHUNKS_X = IS_A ? CF::A_CHUNKS : CF::B_CHUNKS;
    const int r = (ip * CF::WAVES + wave) * DMA_ROWS_X + lane / CHUNKS_X;
    const int chunk = (lane % CHUNKS_X) ^ kn_swizzle<CHUNKS_X * 16>(r);
    if (x0 + chunk * 8 >= xn) return OOB_OFFSET;
    return static_cast<uint32_t>(r) * static_cast<uint32_t>(xn) * 2u + chunk * 16;
}

template <class CF>
__device__ __forceinline__ void dma_full(const Tile &t, uint32_t voff, uint32_t koff, int stage,
                                         int i, const DmaLds &lb)
{
    const bool is_a = i < CF::A_LOADS;
    const int ip = is_a ? i : i - CF::A_LOADS;
    const bool kn = is_a ? CF::AL == 1 : CF::BL == 1;
    // the block less the wave's own part, which the base carries
    const int rblk = kn ? ip * CF::WAVES : dma_block<CF>(ip, 0);
    const uint32_t lds = (kn ? lb.kn : lb.kc) + stage * CF::STAGE_BYTES + (is_a ? 0 : CF::A_BYTES) +
                         rblk * DMA_BYTES;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(is_a ? t.rsrc_a : t.rsrc_b), "s"(koff), "{m0}"(lds));
}

// The operands of one fast-form DMA instruction, for issue fused with an
// MFMA (Step with FUSED): lane offset, buffer resource, scalar offset and the
// LDS address that goes in M0.
struct DmaOp {
    uint32_t voff;
    i32x4_t rsrc;
    uint32_t soff;
    uint32_t m0;
    int imm;   // the instruction's immediate offset: 0, 1024, 2048 or 3072
};

template <class CF>
__device__ __forceinline__ DmaOp dma_full_op(const Tile &t, uint32_t voff, uint32_t koff, int stage,
                                             int i, const DmaLds &lb)
{
    // For a K-contiguous part, `voff` is the lane's offset already lowered
    // by the group position's immediate offset (see the kernel), so the
    // global address and the bounds check (lane offset + immediate) are
    // those of the plain form, while the LDS address steps through the
    // group from one M0 value.
    const bool is_a = i < CF::A_LOADS;
    const int ip = is_a ? i : i - CF::A_LOADS;
    const bool kn = is_a ? CF::AL == 1 : CF::BL == 1;
    const int rblk = kn ? ip * CF::WAVES : dma_block<CF>(ip, 0);
    const int j = kn ? 0 : ip % CF::DMA_G;
    return DmaOp{voff, is_a ? t.rsrc_a : t.rsrc_b, koff,
                 (kn ? lb.kn : lb.kc) + stage * CF::STAGE_BYTES + (is_a ? 0 : CF::A_BYTES) +
                     (rblk - j) * DMA_BYTES,
                 j * DMA_BYTES};
}

// All DMA instructions of one slice, back to back (prefill only).
template <class CF>
__device__ __forceinline__ void dma_slice(const Params &p, const Tile &t, int stage, int kt,
                                          const DmaLds &lb, int wave, int lane, uint32_t row_pitch)
{
#pragma unroll
    for (int i = 0; i < CF::LOADS; ++i) dma_one<CF>(p, t, stage, kt, i, lb, wave, lane, row_pitch);
}

// Work of one MFMA K step, in a fixed issue order.  The wave owns one SIMD's
// matrix pipe, so its instruction stream must keep an MFMA issuing back to
// back.  The FM x FN blocks run in boustrophedon order, row by row (column by
// column when A is double-buffered), so each MFMA shares an operand with the
// previous one, and other work rides between the
// MFMAs, each item after a fixed MFMA:
//   * the next step's B fragments (double-buffered) over the first half of
//     the step, so they have the second half to return;
//   * the next step's A fragment i right after the last MFMA of row i, the
//     earliest point its register is free (single-buffered), or, when A is
//     double-buffered, over the first half of the step like B;
//   * NLD global DMA instructions over the whole step, so the vector-memory
//     queue drains between them instead of stalling the wave.  FUSED (16x16
//     MFMAs, ld(w) returning a DmaOp): the M0 write, the MFMA and the DMA go
//     out as one statement, so the MFMA is the wait state the M0 write needs
//     before an LDS DMA and no s_nop takes an issue slot of the wave.
// sched_barrier(0) after each MFMA group keeps the compiler from regrouping.
//
// The 16x16x32 MFMA goes through inline assembly with its accumulator bound
// to the AGPR file ("a"): a wave's 128x128 block needs all 256 AGPRs, and
// with the builtin the register allocator splits the accumulators between
// the two files and spills.  The compiler then cannot see these MFMAs, so the
// kernel supplies the wait states the ISA requires around them itself: after
// the accumulators are zeroed (VALU write, then MFMA reads them) and before
// they are read back (MFMA write, then VALU read); see the kernel body.
template <class CF, int NLD, bool FUSED = false, bool ZERO = false>
struct Step {
    template <class RdA, class RdB, class Ld>
    __device__ __forceinline__ static void run(typename CF::Acc (&acc)[CF::FM][CF::FN],
                                               const half8_t (&af)[CF::FM],
                                               const half8_t (&bf)[CF::FN], RdA rda, RdB rdb,
                                               Ld ld)
    {
        constexpr int NM = CF::FM * CF::FN;
        constexpr int RSPAN = NM / 2 > 0 ? NM / 2 : 1;
#pragma unroll
        for (int t = 0; t < NM; ++t) {
            // with A double-buffered the blocks run column by column instead
            // (the B operand then stays fixed for FM MFMAs; measured slightly
            // faster); otherwise row by row, which frees A fragment i early
            const int i = CF::ADB ? ((t / CF::FM) & 1 ? CF::FM - 1 - t % CF::FM : t % CF::FM)
                                  : t / CF::FN;
            const int j = CF::ADB ? t / CF::FM
                                  : ((i & 1) ? CF::FN - 1 - t % CF::FN : t % CF::FN);
            // the DMA instruction of this slot, if any (one at most: NLD <= NM)
            int dw = -1;
#pragma unroll
            for (int w = 0; w < NLD; ++w)
                if ((w * NM) / (NLD > 0 ? NLD : 1) == t) dw = w;   // no DMA: no trip
            static_assert(!ZERO || (!FUSED && CF::MI == 16), "zero start: hand-issued MFMAs, no fused DMA");
            if constexpr (FUSED) {
                static_assert(CF::MI == 16 && NLD <= NM, "fused DMA: hand-issued MFMAs, one DMA per slot");
                if (dw >= 0) {
                    const DmaOp op = ld(dw);
                    // M0 is an operand, so a group's later DMAs reuse the
                    // value already there; the immediate offset is a literal
                    // of the instruction, one statement per value
#define GEMM_F16_FUSED_DMA(IMM)                                                          \
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0\n\t"                           \
                 "buffer_load_dwordx4 %3, %4, %6 offen offset:" #IMM " lds"              \
                 : "+a"(acc[i][j])                                                       \
                 : "v"(bf[j]), "v"(af[i]), "v"(op.voff), "s"(op.rsrc), "{m0}"(op.m0),      \
                   "s"(op.soff))
                    switch (op.imm) {
                    case 1024: GEMM_F16_FUSED_DMA(1024); break;
                    case 2048: GEMM_F16_FUSED_DMA(2048); break;
                    case 3072: GEMM_F16_FUSED_DMA(3072); break;
                    default: GEMM_F16_FUSED_DMA(0); break;
                    }
#undef GEMM_F16_FUSED_DMA
                } else {
                    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                                 : "+a"(acc[i][j]) : "v"(bf[j]), "v"(af[i]));
                }
            } else if constexpr (CF::MI == 32) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
            } else if constexpr (ZERO) {
                // a tile's first step: the accumulator input is the constant 0
                asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0"
                             : "=a"(acc[i][j]) : "v"(bf[j]), "v"(af[i]));
            } else {
                asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                             : "+a"(acc[i][j]) : "v"(bf[j]), "v"(af[i]));
            }
#pragma unroll
            for (int w = 0; w < CF::FN; ++w)
                if ((w * RSPAN) / CF::FN == t) rdb(w);
            if constexpr (CF::ADB) {
#pragma unroll
                for (int w = 0; w < CF::FM; ++w)
                    if ((w * RSPAN) / CF::FM == t) rda(w);
            } else {
                if (t % CF::FN == CF::FN - 1) rda(i);
            }
            if constexpr (NLD > 0 && !FUSED) {
                if (dw >= 0) ld(dw);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// For the hand-issued 16x16x32 MFMAs: an empty volatile statement that
// "redefines" an accumulator in the AGPR file.  Volatile statements keep their
// order, so every read of the accumulator after it comes after the wait states
// the kernel issues once the last MFMA is out, and reads of one block are not
// hoisted ahead of the stores of the block before.
template <class CF>
__device__ __forceinline__ void acc_fence(typename CF::Acc &a)
{
    if constexpr (CF::MI == 16) asm volatile("" : "+a"(a));
}

// Epilogue: RNE to fp16 and masked stores.  The MFMA's first operand holds B
// rows, so a result block is a block of C^T: lane l holds, for block (i, j),
// C[m][n .. n+3] with m = l % MI and, per group g of four accumulators,
//   32x32: n = 8 g + 4 (l / 32)  (g = 0..3),   16x16: n = 4 (l / 16).
template <class CF>
__device__ __forceinline__ void store_tile(const Params &p, const Tile &t,
                                           typename CF::Acc (&acc)[CF::FM][CF::FN],
                                           int wave_m, int wave_n, int lane)
{
    const int lrow = lane % CF::MI;
    const int lq = lane / CF::MI;
#pragma unroll
    for (int i = 0; i < CF::FM; ++i) {
        const int32_t m = t.m0 + wave_m * CF::TM + i * CF::MI + lrow;
        if (m < p.M) {
            uint16_t *crow = p.C + static_cast<int64_t>(m) * p.N;
#pragma unroll
            for (int j = 0; j < CF::FN; ++j) {
                acc_fence<CF>(acc[i][j]);
#pragma unroll
                for (int g = 0; g < CF::ACC_N / 4; ++g) {
                    const int32_t n = t.n0 + wave_n * CF::TN + j * CF::MI +
                                      (CF::MI == 32 ? g * 8 + lq * 4 : lq * 4);
                    f32x4_t v;
                    v.x = acc[i][j][4 * g + 0];
                    v.y = acc[i][j][4 * g + 1];
                    v.z = acc[i][j][4 * g + 2];
                    v.w = acc[i][j][4 * g + 3];
                    const half4_t h = __builtin_convertvector(v, half4_t);
                    if (n + 3 < p.N) {
                        __builtin_memcpy(crow + n, &h, 8);   // any 2-byte alignment
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N) reinterpret_cast<_Float16 *>(crow)[n + e] = h[e];
                    }
                }
            }
        }
    }
}

// Split over K: the unit's fp32 partial sums, in the layout of store_tile, to
// its M x N slice of the workspace (16-byte stores, masked at M and N).
template <class CF>
__device__ __forceinline__ void store_tile_f32(const Params &p, const Tile &t,
                                               typename CF::Acc (&acc)[CF::FM][CF::FN],
                                               int wave_m, int wave_n, int lane)
{
    float *ws = p.W + t.split * p.split_stride;
    const int lrow = lane % CF::MI;
    const int lq = lane / CF::MI;
#pragma unroll
    for (int i = 0; i < CF::FM; ++i) {
        const int32_t m = t.m0 + wave_m * CF::TM + i * CF::MI + lrow;
        if (m < p.M) {
            float *wrow = ws + static_cast<int64_t>(m) * p.N;
#pragma unroll
            for (int j = 0; j < CF::FN; ++j) {
                acc_fence<CF>(acc[i][j]);
#pragma unroll
                for (int g = 0; g < CF::ACC_N / 4; ++g) {
                    const int32_t n = t.n0 + wave_n * CF::TN + j * CF::MI +
                                      (CF::MI == 32 ? g * 8 + lq * 4 : lq * 4);
                    f32x4_t v;
                    v.x = acc[i][j][4 * g + 0];
                    v.y = acc[i][j][4 * g + 1];
                    v.z = acc[i][j][4 * g + 2];
                    v.w = acc[i][j][4 * g + 3];
                    if (n + 3 < p.N) {
                        // rows are 4-byte aligned.  Partials larger than the
                        // L2s are stored non-temporally, so they do not evict
                        // the A and B strips; smaller ones stay in L2 for the
                        // reduction.
                        if (p.nt_w)
                            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_u_t *>(wrow + n));
                        else
                            __builtin_memcpy(wrow + n, &v, 16);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N) wrow[n + e] = v[e];
                    }
                }
            }
        }
    }
}

// Store instructions each wave issues, at least, in the staged epilogue of a
// tile wholly inside M x N: one 16-byte segment per item with every lane
// live, counting only the item rounds in which every thread has an item.
template <class CF>
constexpr int staged_stores()
{
    constexpr int ITEMS_R = CF::WM * CF::MI * (CF::BN / 8);
    return CF::FM * (ITEMS_R / CF::THREADS);
}

// Epilogue staged through LDS (the stage the next tile's prefill leaves
// free).  Block rows of every wave -- WM * MI tile rows each -- are written to
// LDS as fp16, as many as the stage holds per round, rows padded by 16 bytes
// so that the 32 rows one write instruction touches fall in distinct banks;
// after a barrier every thread stores 16-byte row segments, a wave covering
// 512 consecutive columns.  A barrier ends each round before the buffer is
// reused.  A tile wholly inside M x N (the common case, known for the whole
// workgroup) takes a path with no per-item checks, and where two buffers fit
// (Cfg::EPI_RB) its rounds alternate between them, so that one round's
// read-back and stores overlap the next round's conversions.  Other tiles
// check every item against M and N.
template <class CF>
__device__ __forceinline__ void store_tile_staged(const Params &p, const Tile &t,
                                                  typename CF::Acc (&acc)[CF::FM][CF::FN],
                                                  int wave_m, int wave_n, int lane, uint8_t *smem)
{
    constexpr int PITCH = CF::BN * 2 + 16;     // bytes per staged row
    constexpr int CROWS = CF::WM * CF::MI;     // tile rows per block row
    constexpr int BROW = CROWS * PITCH;        // bytes per staged block row
    static_assert(CF::STAGED_OK, "staged block row fits one stage");
    static_assert(CF::EPI_BROW == BROW, "staged block row size");
    // block rows per round: as many as one stage holds
    constexpr int R = CF::STAGE_BYTES / BROW < CF::FM ? CF::STAGE_BYTES / BROW : CF::FM;
    static_assert(R >= 1, "one block row per round at least");
    uint8_t *buf = smem + (CF::STAGES - 1) * CF::STAGE_BYTES;
    // the thread's indices, opaque to the optimiser: the per-thread offsets
    // derived from them are computed here for each tile, not hoisted to the
    // kernel's start where they would hold registers through the K loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid), "+v"(lane));
    const int lrow = lane % CF::MI;
    const int lq = lane / CF::MI;
    constexpr int SEGS = CF::BN / 8;           // 8-column segments per row
    constexpr int ITEMS_R = CROWS * SEGS;      // items (16-byte segments) per block row
    constexpr int NI = (ITEMS_R + CF::THREADS - 1) / CF::THREADS;   // per thread
    const bool interior = t.m0 + CF::BM <= p.M && t.n0 + CF::BN <= p.N;
    // block row i of the wave's accumulators, converted to fp16, into staged
    // block row r of buffer b
    auto write_row = [&](uint8_t *b, int r, int i) {
        const int srow = wave_m * CF::MI + lrow;   // staged row of this lane
        // one block row at a time: its accumulators are read out after the
        // previous row's writes
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < CF::FN; ++j) {
            // the block, copied into VGPRs by an empty volatile statement: the
            // copy comes after the wait states that follow the last
            // hand-issued MFMA (see the kernel), and the compiler keeps the
            // AGPRs where the MFMAs left them
            typename CF::Acc av;
            if constexpr (CF::MI == 16)
                asm volatile("" : "=v"(av) : "0"(acc[i][j]));
            else
                av = acc[i][j];
#pragma unroll
            for (int g = 0; g < CF::ACC_N / 4; ++g) {
                const int ncol = wave_n * CF::TN + j * CF::MI + (CF::MI == 32 ? g * 8 + lq * 4 : lq * 4);
                f32x4_t v;
                v.x = av[4 * g + 0];
                v.y = av[4 * g + 1];
                v.z = av[4 * g + 2];
                v.w = av[4 * g + 3];
                *reinterpret_cast<half4_t *>(b + r * BROW + srow * PITCH + ncol * 2) =
                    __builtin_convertvector(v, half4_t);
            }
        }
    };
    if constexpr (CF::EPI_RB > 0) {
        if (interior) {
            // Rounds of RB block rows alternate between two buffers, so the
            // read-back of round q (its LDS reads first, their latency under
            // the conversions) and its stores share one barrier interval
            // with the conversion of round q + 1.  Buffer q % 2 is written
            // again only after the barrier that follows its reads.
            constexpr int RB = CF::EPI_RB;
            constexpr int NR = (CF::FM + RB - 1) / RB;
            half8_t h[RB][NI];
#pragma unroll
            for (int r = 0; r < RB; ++r) write_row(buf, r, r);
            lds_barrier();
#pragma unroll
            for (int q = 0; q < NR; ++q) {
                uint8_t *bq = buf + (q & 1) * RB * BROW;
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    if (q * RB + r >= CF::FM) break;
#pragma unroll
                    for (int it = 0; it < NI; ++it) {
                        const int cr = it * CF::THREADS + tid;
                        if (ITEMS_R % CF::THREADS != 0 && cr >= ITEMS_R) continue;
                        h[r][it] = *reinterpret_cast<const half8_t *>(bq + r * BROW + (cr / SEGS) * PITCH +
                                                                      (cr % SEGS) * 16);
                    }
                }
                if (q + 1 < NR) {
                    uint8_t *bn = buf + ((q + 1) & 1) * RB * BROW;
#pragma unroll
                    for (int r = 0; r < RB; ++r)
                        if ((q + 1) * RB + r < CF::FM) write_row(bn, r, (q + 1) * RB + r);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    if (q * RB + r >= CF::FM) break;
#pragma unroll
                    for (int it = 0; it < NI; ++it) {
                        const int cr = it * CF::THREADS + tid;
                        if (ITEMS_R % CF::THREADS != 0 && cr >= ITEMS_R) continue;
                        const int sr = cr / SEGS;
                        const int32_t m = t.m0 + (sr / CF::MI) * CF::TM + (q * RB + r) * CF::MI + sr % CF::MI;
                        const int32_t n = t.n0 + (cr % SEGS) * 8;
                        _Float16 *dst = reinterpret_cast<_Float16 *>(p.C) + static_cast<int64_t>(m) * p.N + n;
                        // non-temporal: C is written once, and left out of
                        // L2 it does not evict the A and B strips the XCD's
                        // tiles share
                        __builtin_nontemporal_store(h[r][it], reinterpret_cast<half8_u_t *>(dst));
                    }
                }
                lds_barrier();
            }
            return;
        }
    }
#pragma unroll
    for (int i0 = 0; i0 < CF::FM; i0 += R) {
        const int nr = CF::FM - i0 < R ? CF::FM - i0 : R;   // block rows this round
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < nr) write_row(buf, r, i0 + r);
        lds_barrier();
        // item cr of block row r: staged row sr = cr / SEGS, segment sc
        auto row_of = [&](int r, int sr) {
            return t.m0 + (sr / CF::MI) * CF::TM + (i0 + r) * CF::MI + sr % CF::MI;
        };
        if (interior) {
            // per block row: its NI reads back to back, then its NI stores
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r >= nr) break;
                half8_t h[NI];
#pragma unroll
                for (int it = 0; it < NI; ++it) {
                    const int cr = it * CF::THREADS + tid;
                    if (ITEMS_R % CF::THREADS != 0 && cr >= ITEMS_R) continue;
                    h[it] = *reinterpret_cast<const half8_t *>(buf + r * BROW + (cr / SEGS) * PITCH +
                                                               (cr % SEGS) * 16);
                }
#pragma unroll
                for (int it = 0; it < NI; ++it) {
                    const int cr = it * CF::THREADS + tid;
                    if (ITEMS_R % CF::THREADS != 0 && cr >= ITEMS_R) continue;
                    const int32_t m = row_of(r, cr / SEGS);
                    const int32_t n = t.n0 + (cr % SEGS) * 8;
                    _Float16 *dst = reinterpret_cast<_Float16 *>(p.C) + static_cast<int64_t>(m) * p.N + n;
                    // non-temporal: C is written once, and left out of L2 it
                    // does not evict the A and B strips the XCD's tiles share
                    __builtin_nontemporal_store(h[it], reinterpret_cast<half8_u_t *>(dst));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // 16 bytes per lane at any 2-byte alignment: the 2-byte-aligned
            // vector type still gives one 16-byte store, which the target's
            // unaligned-access mode allows; only the segment crossing N is
            // stored element by element.  One block row's items at a time (a
            // scheduling barrier between them keeps only those in registers)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r >= nr) break;
#pragma unroll
                for (int it = 0; it < NI; ++it) {
                    const int cr = it * CF::THREADS + tid;
                    if (cr >= ITEMS_R) continue;
                    const int sr = cr / SEGS, sc = cr % SEGS;
                    const int32_t m = row_of(r, sr);
                    const int32_t n = t.n0 + sc * 8;
                    if (m >= p.M || n >= p.N) continue;
                    const half8_t h =
                        *reinterpret_cast<const half8_t *>(buf + r * BROW + sr * PITCH + sc * 16);
                    _Float16 *dst = reinterpret_cast<_Float16 *>(p.C) + static_cast<int64_t>(m) * p.N + n;
                    if (n + 8 <= p.N) {
                        __builtin_nontemporal_store(h, reinterpret_cast<half8_u_t *>(dst));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (n + e < p.N) dst[e] = h[e];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lds_barrier();
    }
}

// Per-wave constants.
template <class CF>
struct WaveCtx {
    int lane, wave, wave_m, wave_n;
    uint32_t row_pitch, a_frag_base, b_frag_base;
    // Fragment lane l reads row l % MI of an MI-row block, logical chunk
    // kk * (MK / 8) + l / MI (8 consecutive k), physically XOR-swizzled.  The
    // swizzle depends on the row mod 32, so a 16-row block at an odd multiple
    // of 16 (parity 1) sees a different pattern.
    uint32_t frag_off[2][CF::KK];
    // [K, N] B: the lane's byte offset in the B tile for the first
    // transposing read of step 0 of fragment 0 (row 8 (l / 16) + (l % 16) / 4,
    // columns 4 (l % 4) of the wave's block).  Fragment j's 16 columns sit 2 j
    // chunks on, in chunk bits the swizzle XOR shares but the wave's and the
    // lane's own bits do not, so its offset is btr0 ^ 32 j.  Later steps and
    // the second read (4 rows on) keep the row's swizzle: constant offsets.
    uint32_t btr0;
    // [K, M] A: the same, for block i of the wave's rows (atr0 ^ 32 i)
    uint32_t atr0;

    __device__ __forceinline__ WaveCtx(const Params &p)
    {
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        wave_m = wave / CF::WN;
        wave_n = wave - wave_m * CF::WN;
        row_pitch = static_cast<uint32_t>(p.K) * 2u;
        const int lrow = lane % CF::MI;
        const int lq = lane / CF::MI;
#pragma unroll
        for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int kk = 0; kk < CF::KK; ++kk) {
                const int row32 = par * 16 + lrow;
                const int chunk = kk * (CF::MK / 8) + lq;
                frag_off[par][kk] = lrow * CF::ROW_BYTES +
                                    ((chunk ^ chunk_swizzle<CF::CHUNKS, CF::MI>(CF::MI == 16 ? row32 : lrow)) * 16);
            }
        a_frag_base = wave_m * CF::TM * CF::ROW_BYTES;
        b_frag_base = CF::A_BYTES + wave_n * CF::TN * CF::ROW_BYTES;
        btr0 = 0;
        atr0 = 0;
        // the fragment XOR 32 j (j < TN / 16) touches chunk bits below
        // log2(TN / 8); the wave's offset, a multiple of TN / 8 chunks, lies
        // above them when TN is a power of two
        // the fragment XOR (bits 5..8) and the offsets added to the bases
        // before it (multiples of 512) never share a bit
        static_assert(CF::STAGE_BYTES % 512 == 0 && CF::A_BYTES % 512 == 0 &&
                          32 * CF::FN <= 512 && 32 * CF::FM <= 512,
                      "stage and tile offsets clear of the fragment XOR");
        if constexpr (CF::BL == 1) {
            static_assert(CF::TN >= 32 && (CF::TN & (CF::TN - 1)) == 0,
                          "wave column offset clear of the XOR bits");
            const int r = 8 * (lane / 16) + (lane % 16) / 4;
            const int n = wave_n * CF::TN + 4 * (lane % 4);
            btr0 = r * CF::B_ROW_BYTES + (((n / 8) ^ kn_swizzle<CF::B_ROW_BYTES>(r)) * 16) +
                   (n % 8) * 2;
        }
        if constexpr (CF::AL == 1) {
            static_assert(CF::TM >= 32 && (CF::TM & (CF::TM - 1)) == 0,
                          "wave row offset clear of the XOR bits");
            const int r = 8 * (lane / 16) + (lane % 16) / 4;
            const int m = wave_m * CF::TM + 4 * (lane % 4);
            atr0 = r * CF::A_ROW_BYTES + (((m / 8) ^ kn_swizzle<CF::A_ROW_BYTES>(r)) * 16) +
                   (m % 8) * 2;
        }
    }
};

// One transposing LDS read (see kn_swizzle): four 16-bit elements.
__device__ __forceinline__ half4_t lds_read_tr16(const uint8_t *p)
{
    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4_t lds_s4_t;
    const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t *)(p));
    return __builtin_bit_cast(half4_t, v);
}

template <class CF>
__device__ __forceinline__ void zero_acc(typename CF::Acc (&acc)[CF::FM][CF::FN])
{
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
        for (int j = 0; j < CF::FN; ++j)
#pragma unroll
            for (int e = 0; e < CF::ACC_N; ++e) acc[i][j][e] = 0.0f;
}

// ---------------------------------------------------------------------------
// Kernel, direct-to-LDS fill
// ---------------------------------------------------------------------------
// The kernel's arguments, read afresh from the kernarg segment (Params is the
// kernel's only argument and sits at its start).  The empty asm makes every
// call a new pointer value, so the scalar loads of the fields used after it
// are issued there: no field is held in a scalar register from the kernel's
// start to its last use across every tile.
__device__ __forceinline__ const Params &kernel_args()
{
    auto q = __builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(q));
    return *(const Params *)q;
}

template <class CF, bool SPLIT>
__global__ __launch_bounds__(CF::THREADS)
__attribute__((amdgpu_waves_per_eu(CF::WAVES_PER_SIMD, CF::WAVES_PER_SIMD)))
void gemm_f16_nt_kernel(Params p)
{
    // the ring, then the staged epilogue's second buffer where it needs more
    __shared__ __attribute__((aligned(1024))) uint8_t smem[CF::LDS_BYTES + (SPLIT ? 0 : CF::EPI_EXTRA)];
    constexpr int S = CF::STAGES;
    constexpr int KK = CF::KK;
    constexpr int L = CF::LOADS;
    // The refill of slice kt + S - 1 streams over slice kt.  With 3+ stages it
    // spreads over every step; with 2 the refilled slice is the very next one,
    // so it must land before the barrier that ends slice kt: it goes into the
    // first half of the slice's steps, leaving the rest for its latency.
    static_assert(S >= 2, "double buffer at least");
    static_assert(S >= 3 || KK >= 2, "two stages need a slice of 2+ steps");
    constexpr int DSTEPS = CF::DSTEPS > 0 ? CF::DSTEPS : (S >= 3 ? KK : KK / 2);
    static_assert(DSTEPS <= KK && (S >= 3 || DSTEPS < KK), "refill steps");
    // With DX > 0 (two stages), DX instructions of the refill of slice kt + 2
    // go out during the last step of slice kt, right after the barrier that
    // frees its stage; the remaining LY during slice kt + 1 as above.
    constexpr int DX = CF::DX;
    constexpr int LY = L - DX;
    constexpr int DPS = (LY + DSTEPS - 1) / DSTEPS;  // DMA instructions per such step (the last may have fewer)
    // outstanding DMA allowed when slice kt + 1 must have landed at the end of
    // slice kt: slices kt+2 .. kt+S-2 and the parts of kt+S-1 issued so far
    // (none of which is slice kt + 1 when S >= 3; with S = 2 it is).
    constexpr int ISSUED_BEFORE_BARRIER = (KK - 1) * DPS < L ? (KK - 1) * DPS : L;
    constexpr int VM_STEADY = S >= 3 ? (S - 3) * L + ISSUED_BEFORE_BARRIER : 0;
    static_assert((S - 1) * L <= 63 && VM_STEADY <= 63, "vmcnt counts at most 63 loads");

    const WaveCtx<CF> w(p);
    // With two stages and the whole refill issued early, the refill of a
    // slice wholly inside K takes the fast form (dma_full).
    constexpr bool FAST_DMA = S == 2 && DX == L;
    // fast-form lane offsets: one kernel-wide set for the K-contiguous
    // operands (both parts use the same row pattern); an operand stored
    // [K, M] / [K, N] has its own, set per tile
    constexpr int NA_K = CF::AL ? 0 : CF::A_LOADS, NB_K = CF::BL ? 0 : CF::B_LOADS;
    constexpr int NVOFF = !FAST_DMA ? 1 : (NA_K > NB_K ? NA_K : (NB_K > 0 ? NB_K : 1));
    uint32_t dvoff[NVOFF];
    // In the fused early refill (16x16 MFMAs) a K-contiguous part's DMA at
    // group position j carries the immediate offset 1024 j: its lane offset is
    // lowered by as much (never below zero: the row of position j lies at
    // least 8 j rows in, 8 j x 2K >= 1024 j bytes, and the fused refill runs
    // only for K >= 192).
#pragma unroll
    for (int i = 0; i < NVOFF; ++i)
        dvoff[i] = dma_lane_offset<CF>(i, w.wave, w.lane, w.row_pitch) -
                   (FAST_DMA && CF::MI == 16 ? static_cast<uint32_t>(i % CF::DMA_G) * DMA_BYTES : 0u);
    uint32_t dvoffa[FAST_DMA && CF::AL ? CF::A_NB : 1];
    uint32_t dvoffb[FAST_DMA && CF::BL ? CF::B_NB : 1];
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));

    half8_t af[CF::ADB ? 2 : 1][CF::FM], bf[2][CF::FN];
    // the lane's fragment read offsets in the A and B tiles of a stage, one
    // register each, so every read of the loop is that register plus an
    // immediate offset
    uint32_t fra[2][KK], frb[2][KK];
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            fra[par][kk] = w.frag_off[par][kk] + w.a_frag_base;
            frb[par][kk] = w.frag_off[par][kk] + w.b_frag_base;
        }
    // A fragment i / B fragment j of step kk of `stage`, into buffer `buf`
    auto read_a = [&](int buf, int stage, int kk, int i) {
        if constexpr (CF::AL == 0) {
            af[buf][i] = *reinterpret_cast<const half8_t *>(smem + stage * CF::STAGE_BYTES +
                                                        fra[i & 1][kk] + i * CF::MI * CF::ROW_BYTES);
        } else {
            // the stage's offset joins the base before the XOR (see read_b)
            uint32_t off;
            asm volatile("v_xor_b32 %0, %2, %1"
                         : "=v"(off)
                         : "v"(w.atr0 + static_cast<uint32_t>(stage) * CF::STAGE_BYTES), "n"(32 * i));
            const uint8_t *q = smem + off + kk * 32 * CF::A_ROW_BYTES;
            const half4_t lo = lds_read_tr16(q);
            const half4_t hi = lds_read_tr16(q + 4 * CF::A_ROW_BYTES);
            af[buf][i] = half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    auto read_b = [&](int buf, int stage, int kk, int j) {
        if constexpr (CF::BL == 0) {
            bf[buf][j] = *reinterpret_cast<const half8_t *>(smem + stage * CF::STAGE_BYTES +
                                                             frb[j & 1][kk] + j * CF::MI * CF::ROW_BYTES);
        } else {
            // the XOR is issued at the read (an asm the compiler cannot hoist):
            // hoisted, the FN offsets would each hold a register for the
            // whole loop.  The stage's and the A tile's offsets (multiples of
            // 1 KB) join the base before the XOR, which touches bits 5..8
            // only: (x + c) ^ 32 j = (x ^ 32 j) + c.  The XOR result then
            // addresses the reads directly (the K step's offset fits their
            // immediate), with no vector add after the asm -- which the
            // compiler would separate from it by a wait state, not knowing
            // what the asm computes.
            uint32_t off;
            asm volatile("v_xor_b32 %0, %2, %1"
                         : "=v"(off)
                         : "v"(w.btr0 + CF::A_BYTES + static_cast<uint32_t>(stage) * CF::STAGE_BYTES),
                           "n"(32 * j));
            const uint8_t *q = smem + off + kk * 32 * CF::B_ROW_BYTES;
            const half4_t lo = lds_read_tr16(q);
            const half4_t hi = lds_read_tr16(q + 4 * CF::B_ROW_BYTES);
            bf[buf][j] = half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    auto none = [](int) {};

    int32_t slot = blockIdx.x;
    if (slot >= p.tiles) return;
    Tile cur = make_tile<CF, SPLIT>(p, slot, w.row_pitch);
    // the previous tile was an interior one whose C went out through the
    // staged epilogue (see the first wait of a tile)
    bool prev_interior = false;
    // Prefill: slices 0 .. S-2 into stages 0 .. S-2; stage S-1 is refilled
    // while slice 0 is computed.  Issued even when K has fewer slices (those
    // move no data), so every wait below counts the same instructions.
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
        dma_slice<CF>(p, cur, s, s, dma_lds<CF>(lds0, w.wave), w.wave, w.lane, w.row_pitch);

    while (true) {
        const Params pt = kernel_args();
        const uint32_t lda = static_cast<uint32_t>(pt.M) * 2u;   // [K, M] A row pitch
        const uint32_t ldb = static_cast<uint32_t>(pt.N) * 2u;   // [K, N] B row pitch
        const int KT = (cur.klen + CF::BK - 1) / CF::BK;   // slices of this unit
        // this tile's DMA base addresses (see DmaLds), made opaque again at
        // every slice below
        DmaLds lt = dma_lds<CF>(lds0, w.wave);
        if constexpr (FAST_DMA && CF::AL == 1) {
#pragma unroll
            for (int i = 0; i < CF::A_NB; ++i)
                dvoffa[i] = dma_lane_offset_kn<CF, true>(i, w.wave, w.lane, cur.m0, pt.M);
        }
        if constexpr (FAST_DMA && CF::BL == 1) {
#pragma unroll
            for (int i = 0; i < CF::B_NB; ++i)
                dvoffb[i] = dma_lane_offset_kn<CF, false>(i, w.wave, w.lane, cur.n0, pt.N);
        }
        // slices whose early refill (slice kt + 2) lies wholly inside K
        const int kt_fast = FAST_DMA ? min(max(cur.klen / CF::BK - 2, 0), KT) : 0;
        // With hand-issued MFMAs and two such slices, the tile's first K
        // step takes 0 as its accumulator input, so nothing is zeroed here.
        constexpr bool CAN_ZERO_START = FAST_DMA && CF::MI == 16;
        const bool zero_start = CAN_ZERO_START && kt_fast >= 2;
        typename CF::Acc acc[CF::FM][CF::FN];
        if (!zero_start) zero_acc<CF>(acc);
        if (CF::MI == 16 && !zero_start) {
            // the zeros are in the AGPRs before the wait states that separate
            // their (VALU) writes from the first MFMA reading them
#pragma unroll
            for (int i = 0; i < CF::FM; ++i)
#pragma unroll
                for (int j = 0; j < CF::FN; ++j) acc_fence<CF>(acc[i][j]);
            asm volatile("s_nop 4");
        }
        if (KT > 0) {
            // early part of slice 1, into stage 1: free, since the previous
            // tile's epilogue ended with a barrier.  Issued before the wait for
            // slice 0, which (vmcnt also counting stores) drains that
            // epilogue's C stores as well: its latency overlaps theirs.
            if constexpr (DX > 0) {
#pragma unroll
                for (int d = 0; d < DX; ++d)
                    dma_one<CF>(pt, cur, 1, 1, d, lt, w.wave, w.lane, w.row_pitch);
            }
            // slice 0 landed (slices 1 .. S-2, and slice 1's early part, may
            // still be in flight).  After the staged epilogue of an interior
            // tile, the C stores it issued (at least staged_stores<CF>() per
            // wave, all younger than the prefill; vmcnt counts stores) stay in
            // flight too: C drains behind this tile's MFMAs.
            if constexpr (CF::STAGED_OK && !SPLIT) {
                static_assert((S - 2) * L + DX + staged_stores<CF>() <= 63, "vmcnt holds at most 63");
                if (__builtin_amdgcn_readfirstlane(prev_interior ? 1 : 0))
                    wait_vmcnt<(S - 2) * L + DX + staged_stores<CF>()>();
                else
                    wait_vmcnt<(S - 2) * L + DX>();
            } else {
                wait_vmcnt<(S - 2) * L + DX>();
            }
            lds_barrier();
#pragma unroll
            for (int i = 0; i < CF::FM; ++i) read_a(0, 0, 0, i);
#pragma unroll
            for (int j = 0; j < CF::FN; ++j) read_b(0, 0, 0, j);
        }

        // One branch-free loop over the slices.  Slice kt streams in the refill
        // of slice kt + S - 1 (into the stage freed before slice kt); past the
        // end of K those refills carry out-of-range offsets, so they move no
        // data and only write zeros into stages this tile no longer reads.
        // Their accounting is therefore identical to the real ones.
        int rd = 0;        // stage holding slice kt
        int pst = S - 1;   // stage receiving slice kt + S - 1, freed before slice kt
        auto slice = [&](int kt, auto fast, auto zero) {
            constexpr bool FAST = decltype(fast)::value;
            constexpr bool ZERO = decltype(zero)::value;
            // M0 values are computed from the bases where they are written
            // (one scalar add into M0 each), not held in a scalar register
            // per value across the loop
            asm volatile("" : "+s"(lt.kc), "+s"(lt.kn));
            const int rd_next = rd + 1 == S ? 0 : rd + 1;
            const int pkt = kt + S - 1;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                auto dma = [&](int d) {
                    if (kk * DPS + d < LY)
                        dma_one<CF>(pt, cur, pst, pkt, DX + kk * DPS + d, lt, w.wave, w.lane,
                                    w.row_pitch);
                };
                // early part of slice kt + 2, into stage rd, which the barrier
                // of this slice's last step has just freed
                auto dma_early = [&](int d) {
                    if constexpr (FAST) {
                        const uint32_t kslice = static_cast<uint32_t>(kt + 2) * CF::BK;
                        if (d < CF::A_LOADS) {
                            if constexpr (CF::AL == 1)
                                dma_full<CF>(cur, dvoffa[d % CF::A_NB],
                                             (kslice + static_cast<uint32_t>(d / CF::A_NB) *
                                                           CF::A_NB * CF::A_RB) * lda,
                                             rd, d, lt);
                            else
                                dma_full<CF>(cur, dvoff[d], kslice * 2, rd, d, lt);
                        } else {
                            const int db = d - CF::A_LOADS;
                            if constexpr (CF::BL == 1)
                                dma_full<CF>(cur, dvoffb[db % CF::B_NB],
                                             (kslice + static_cast<uint32_t>(db / CF::B_NB) *
                                                           CF::B_NB * CF::B_RB) * ldb,
                                             rd, d, lt);
                            else
                                dma_full<CF>(cur, dvoff[db], kslice * 2, rd, d, lt);
                        }
                    } else
                        dma_one<CF>(pt, cur, rd, kt + 2, d, lt, w.wave, w.lane, w.row_pitch);
                };
                // the same DMA as operands, for issue fused with an MFMA
                auto dma_early_op = [&](int d) -> DmaOp {
                    const uint32_t kslice = static_cast<uint32_t>(kt + 2) * CF::BK;
                    if (d < CF::A_LOADS) {
                        if constexpr (CF::AL == 1)
                            return dma_full_op<CF>(cur, dvoffa[d % CF::A_NB],
                                                   (kslice + static_cast<uint32_t>(d / CF::A_NB) *
                                                                 CF::A_NB * CF::A_RB) * lda,
                                                   rd, d, lt);
                        else
                            return dma_full_op<CF>(cur, dvoff[d], kslice * 2, rd, d, lt);
                    } else {
                        const int db = d - CF::A_LOADS;
                        if constexpr (CF::BL == 1)
                            return dma_full_op<CF>(cur, dvoffb[db % CF::B_NB],
                                                   (kslice + static_cast<uint32_t>(db / CF::B_NB) *
                                                                 CF::B_NB * CF::B_RB) * ldb,
                                                   rd, d, lt);
                        else
                            return dma_full_op<CF>(cur, dvoff[db], kslice * 2, rd, d, lt);
                    }
                };
                if (kk + 1 < KK) {
                    auto ra = [&](int i) { read_a(CF::ADB ? (kk + 1) & 1 : 0, rd, kk + 1, i); };
                    auto rb = [&](int j) { read_b((kk + 1) & 1, rd, kk + 1, j); };
                    if (ZERO && kk == 0)
                        Step<CF, 0, false, ZERO>::run(acc, af[CF::ADB ? kk & 1 : 0], bf[kk & 1], ra, rb, none);
                    else if (kk < DSTEPS)
                        Step<CF, DPS>::run(acc, af[CF::ADB ? kk & 1 : 0], bf[kk & 1], ra, rb, dma);
                    else
                        Step<CF, 0>::run(acc, af[CF::ADB ? kk & 1 : 0], bf[kk & 1], ra, rb, none);
                } else {
                    // End of the slice (the last step's B fragments are in
                    // registers; its A fragments were all read before any
                    // of them is overwritten).  "full": slice kt + 1 has
                    // landed for this wave, and after the barrier for every
                    // wave; "empty": every wave has read all of stage rd,
                    // which receives slice kt + S during the next slice.
                    // After the last slice the reads below fetch unused data
                    // (in bounds).
                    wait_vmcnt<VM_STEADY>();
                    lds_barrier();
                    auto ra = [&](int i) { read_a(0, rd_next, 0, i); };
                    auto rb = [&](int j) { read_b(0, rd_next, 0, j); };
                    if constexpr (DX > 0 && FAST && CF::MI == 16)
                        Step<CF, DX, true>::run(acc, af[CF::ADB ? kk & 1 : 0], bf[kk & 1], ra, rb,
                                                dma_early_op);
                    else if constexpr (DX > 0)
                        Step<CF, DX>::run(acc, af[CF::ADB ? kk & 1 : 0], bf[kk & 1], ra, rb, dma_early);
                    else if (kk < DSTEPS)
                        Step<CF, DPS>::run(acc, af[CF::ADB ? kk & 1 : 0], bf[kk & 1], ra, rb, dma);
                    else
                        Step<CF, 0>::run(acc, af[CF::ADB ? kk & 1 : 0], bf[kk & 1], ra, rb, none);
                }
            }
            pst = rd;
            rd = rd_next;
        };
        // slices whose early refill lies wholly inside K, then the rest
        int kt = 0;
        if constexpr (FAST_DMA) {
            // two slices per trip (FAST_DMA implies two stages), so the ring
            // stage of each is a compile-time constant: LDS addresses and M0
            // values become loop-invariant registers.  The first trip is
            // separate where the tile starts with the zero-input step.
            if constexpr (CAN_ZERO_START) {
                if (zero_start) {
                    rd = 0;
                    pst = 1;
                    slice(0, std::true_type{}, std::true_type{});
                    rd = 1;
                    pst = 0;
                    slice(1, std::true_type{}, std::false_type{});
                    kt = 2;
                }
            }
            for (; kt + 1 < kt_fast; kt += 2) {
                rd = 0;
                pst = 1;
                slice(kt, std::true_type{}, std::false_type{});
                rd = 1;
                pst = 0;
                slice(kt + 1, std::true_type{}, std::false_type{});
            }
        }
        for (; kt < kt_fast; ++kt) slice(kt, std::true_type{}, std::false_type{});
        for (; kt < KT; ++kt) slice(kt, std::false_type{}, std::false_type{});

        // Wait states between the last hand-issued MFMA writing an accumulator
        // and the first VALU read of it: 24, more than the ISA asks for after
        // any MFMA, whatever its pass count.
        if constexpr (CF::MI == 16) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
        // no accumulator read is scheduled ahead of those wait states
        __builtin_amdgcn_sched_barrier(0);
        // Every wave is done with the ring (and every DMA has landed): the next
        // tile's prefill may start, and it flies while this tile is stored.
        wait_vmcnt<0>();
        lds_barrier();
        const Params pe = kernel_args();
        const int32_t next = slot + pe.grid;
        Tile nxt;
        if (next < pe.tiles) {
            nxt = make_tile<CF, SPLIT>(pe, next, w.row_pitch);
#pragma unroll
            for (int s = 0; s < S - 1; ++s)
                dma_slice<CF>(pe, nxt, s, s, dma_lds<CF>(lds0, w.wave), w.wave, w.lane, w.row_pitch);
        }
        const Params pc = kernel_args();
        if constexpr (SPLIT) {
            store_tile_f32<CF>(pc, cur, acc, w.wave_m, w.wave_n, w.lane);
        } else if constexpr (CF::STAGED_OK) {
            if (pc.staged)
                store_tile_staged<CF>(pc, cur, acc, w.wave_m, w.wave_n, w.lane, smem);
            else
                store_tile<CF>(pc, cur, acc, w.wave_m, w.wave_n, w.lane);
            prev_interior = pc.staged && cur.m0 + CF::BM <= pc.M && cur.n0 + CF::BN <= pc.N;
        } else {
            store_tile<CF>(pc, cur, acc, w.wave_m, w.wave_n, w.lane);
        }
        if (next >= pc.tiles) break;
        slot = next;
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// Kernel, producer and consumer waves
// ---------------------------------------------------------------------------
// The pages' later kernels give the loads to a producer warp and the MMAs to
// consumer warp groups (page "3. Warp Specialization", Why a Separate
// Producer Warp and Producer-Consumer Barriers; page "4. Pipeline Abstraction
// and Two Consumer Warp Groups", Pipeline Abstraction).  Here WAVES consumer
// waves compute the tile as the kernel above does, and as many producer
// waves only issue the direct-to-LDS DMA, so a DMA instruction that waits for
// the texture addresser never holds up an MFMA stream.  Waves w and
// w + WAVES share a SIMD: two waves per SIMD, so every wave has at most 256
// registers, and a consumer's wave tile is held to 128 accumulators (a
// 256 x 128 tile over four waves).  CDNA has no per-role register split, so
// the producers get 256 registers too.
//
// Ring of three stages, one s_barrier per K-slice taken by every wave as
// both handshakes.  Before barrier g
//   * every producer has issued slice g + 2 (into the stage that slice g - 1
//     held, freed by barrier g - 1) and waited (vmcnt) until its part of
//     slice g + 1 has landed: after the barrier slice g + 1 is "full";
//   * every consumer has all fragments of slice g in registers (lgkmcnt):
//     after the barrier its stage is "empty".
// A consumer takes barrier g before the last K step of slice g, whose
// fragments are already in registers, so its MFMAs cover the barrier and the
// reads of slice g + 1.  The producers run two slices ahead through the
// workgroup's whole tile sequence, so the next tile's first slices load
// while this tile's epilogue stores C (straight from the MFMA layout: every
// stage is in use by then).  SPLIT: the same over (K range, tile) work units
// (see Params), each storing fp32 partials; units may differ in K length, and
// both roles count every unit's slices alike.
__device__ __forceinline__ void wg_barrier()
{
    asm volatile("s_barrier" : : : "memory");
}

// K slices of the work unit in persistent slot `slot`
template <class CF, bool SPLIT>
__device__ __forceinline__ int unit_slices(const Params &p, int32_t slot)
{
    int32_t klen = p.K;
    if constexpr (SPLIT) {
        const int32_t split = static_cast<int32_t>(
            static_cast<uint32_t>(slot_to_linear(slot, p.grid, p.tiles, p.xcds)) /
            static_cast<uint32_t>(p.tiles_m * p.tiles_n));
        klen = min(p.k_split, p.K - split * p.k_split);
    }
    return (klen + CF::BK - 1) / CF::BK;
}

template <class CF, bool SPLIT>
__global__ __launch_bounds__(2 * CF::THREADS)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_f16_nt_pc_kernel(Params p)
{
    static_assert(CF::STAGES == 3 && CF::MI == 16 && CF::ADB && CF::KK == 2 && CF::DX == 0 &&
                      CF::AL == 0 && CF::BL == 0,
                  "three stages, 16x16x32 MFMAs with both fragments double-buffered, two K "
                  "steps per slice, NT operands");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[CF::LDS_BYTES];
    constexpr int L = CF::LOADS;   // DMA instructions per producer wave per slice
    const int32_t wg = blockIdx.x;
    if (wg >= p.tiles) return;
    const int KT = (p.K + CF::BK - 1) / CF::BK;   // 0 only for K = 0 (never split)
    const uint32_t row_pitch = static_cast<uint32_t>(p.K) * 2u;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    if (wave >= CF::WAVES) {
        // ---- producer: slices in the workgroup's tile order, two ahead ----
        if (KT == 0) return;   // nothing to load; the consumers store zeros
        const int pw = wave - CF::WAVES;
        const int lane = threadIdx.x & 63;
        constexpr int NV = CF::A_LOADS > CF::B_LOADS ? CF::A_LOADS : CF::B_LOADS;
        uint32_t dvoff[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) dvoff[i] = dma_lane_offset<CF>(i, pw, lane, row_pitch);
        const DmaLds plb = dma_lds<CF>(lds0, pw);
        int32_t cslot = wg;   // the next slice to issue: unit cslot, slice ckt
        int ckt = 0;
        Tile ct = make_tile<CF, SPLIT>(p, cslot, row_pitch);
        int ckts = (ct.klen + CF::BK - 1) / CF::BK;
        auto issue = [&](int stage) {
            if ((ckt + 1) * CF::BK <= ct.klen) {
                // wholly inside K: the K offset rides in the scalar offset
                const uint32_t koff = static_cast<uint32_t>(ckt) * CF::BK * 2u;
#pragma unroll
                for (int i = 0; i < L; ++i)
                    dma_full<CF>(ct, dvoff[i < CF::A_LOADS ? i : i - CF::A_LOADS], koff, stage, i,
                                 plb);
            } else {
#pragma unroll
                for (int i = 0; i < L; ++i)
                    dma_one<CF>(p, ct, stage, ckt, i, plb, pw, lane, row_pitch);
            }
            if (++ckt == ckts) {
                ckt = 0;
                cslot += p.grid;
                if (cslot < p.tiles) {
                    ct = make_tile<CF, SPLIT>(p, cslot, row_pitch);
                    ckts = (ct.klen + CF::BK - 1) / CF::BK;
                }
            }
        };
        issue(0);
        if (cslot < p.tiles) {
            issue(1);
            wait_vmcnt<L>();   // slice 0 landed
        } else {
            wait_vmcnt<0>();
        }
        wg_barrier();
        int ps = 2;   // stage of the next slice issued
        for (int32_t slot = wg; slot < p.tiles; slot += p.grid) {
            const int kts = unit_slices<CF, SPLIT>(p, slot);
            for (int kt = 0; kt < kts; ++kt) {
                if (cslot < p.tiles) {
                    issue(ps);
                    ps = ps == 2 ? 0 : ps + 1;
                    wait_vmcnt<L>();   // the slice after the consumers' current one landed
                } else {
                    wait_vmcnt<0>();
                }
                wg_barrier();
            }
        }
        return;
    }

    // ---- consumer ----
    const WaveCtx<CF> w(p);
    half8_t af[2][CF::FM], bf[2][CF::FN];
    auto read_a = [&](int buf, int stage, int kk, int i) {
        af[buf][i] = *reinterpret_cast<const half8_t *>(smem + stage * CF::STAGE_BYTES +
                                                        w.frag_off[i & 1][kk] + w.a_frag_base +
                                                        i * CF::MI * CF::ROW_BYTES);
    };
    auto read_b = [&](int buf, int stage, int kk, int j) {
        bf[buf][j] = *reinterpret_cast<const half8_t *>(smem + stage * CF::STAGE_BYTES +
                                                        w.frag_off[j & 1][kk] + w.b_frag_base +
                                                        j * CF::MI * CF::ROW_BYTES);
    };
    auto none = [](int) {};
    if (KT > 0) {
        lds_barrier();   // slice 0 is full
#pragma unroll
        for (int i = 0; i < CF::FM; ++i) read_a(0, 0, 0, i);
#pragma unroll
        for (int j = 0; j < CF::FN; ++j) read_b(0, 0, 0, j);
    }
    int cs = 0;   // stage of the consumers' current slice
    for (int32_t slot = wg; slot < p.tiles; slot += p.grid) {
        typename CF::Acc acc[CF::FM][CF::FN];
        zero_acc<CF>(acc);
        // the zeros are in the AGPRs before the wait states that separate
        // their (VALU) writes from the first MFMA reading them
#pragma unroll
        for (int i = 0; i < CF::FM; ++i)
#pragma unroll
            for (int j = 0; j < CF::FN; ++j) acc_fence<CF>(acc[i][j]);
        asm volatile("s_nop 4");
        const int kts = KT > 0 ? unit_slices<CF, SPLIT>(p, slot) : 0;
        for (int kt = 0; kt < kts; ++kt) {
            const int ns = cs == 2 ? 0 : cs + 1;
            // step 0 of slice kt, reading step 1's fragments
            auto ra1 = [&](int i) { read_a(1, cs, 1, i); };
            auto rb1 = [&](int j) { read_b(1, cs, 1, j); };
            Step<CF, 0>::run(acc, af[0], bf[0], ra1, rb1, none);
            // this slice's stage is read; the next slice has landed
            lds_barrier();
            // step 1, reading step 0's fragments of the next slice (after the
            // workgroup's last slice: stale data, never used)
            auto ra0 = [&](int i) { read_a(0, ns, 0, i); };
            auto rb0 = [&](int j) { read_b(0, ns, 0, j); };
            Step<CF, 0>::run(acc, af[1], bf[1], ra0, rb0, none);
            cs = ns;
        }
        // 24 wait states between the last MFMA and the first read of its
        // accumulators (as in the kernel above)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
        const Tile t = make_tile<CF, SPLIT>(p, slot, w.row_pitch);
        if constexpr (SPLIT)
            store_tile_f32<CF>(p, t, acc, w.wave_m, w.wave_n, w.lane);
        else
            store_tile<CF>(p, t, acc, w.wave_m, w.wave_n, w.lane);
    }
}

// ---------------------------------------------------------------------------
// Kernel, B streamed through registers (few rows of A)
// ---------------------------------------------------------------------------
// With a handful of A rows each B element is used a handful of times, and the
// GEMM is a stream of B from HBM.  The LDS ring then limits it: what a CU
// keeps in flight is what its stages hold, and for M = 1 most of each stage
// is zero rows of the A tile.  Here one wave owns a 16 x 16 output tile (16
// rows of A and 16 rows of B) and loads both fragments of every K step
// straight from global memory in the MFMA's operand layout: lane l
// reads 16 bytes of row l % 16 at k = 32 s + 8 (l / 16), so one load covers
// 64 bytes of each of 16 rows.  Blocks of D steps are double-buffered: the
// next block's loads fly while this block's MFMAs run.
//
// The MFMA is the 16 x 16 x 32 one of the other configurations, stepping K
// in the same ascending 32-wide steps into one fp32 accumulator per element
// from +0, so every result bit equals theirs.  Chunks past K load as zeros
// (K is a multiple of 8, so a chunk never straddles K); lanes past M or N
// read row 0, whose products land only in outputs that are not stored.  A
// persistent loop walks the tiles row-major (t = blockIdx.x + i gridDim.x)
// for any grid; any M is computed, though only a few rows of A use it well.
//
// SPLIT: unit t is tile t mod (tiles_m tiles_n) over K range [s k_split,
// min((s + 1) k_split, K)), s = t / (tiles_m tiles_n), and its fp32 sums go
// to partial s of W (an M x N row-major matrix) for the reduction kernel.
// k_split is a multiple of 32, so every range starts on a step and each
// unit's steps are those of a GEMM of K = its range length.
template <int D, bool SPLIT>
__global__ __launch_bounds__(64) void gemm_f16_nt_stream_kernel(Params p)
{
    const int lane = threadIdx.x;
    const int r = lane & 15;    // operand row: B row n0 + r, A row m0 + r
    const int kq = lane >> 4;   // which 8-element chunk of the 32-wide K step
    const int32_t M = p.M, N = p.N, K = p.K;   // K: the operands' row length
    const int32_t tiles_mn = p.tiles_m * p.tiles_n;
    const half8_t zero = {};
    for (int32_t t = blockIdx.x; t < p.tiles; t += gridDim.x) {
        int32_t u = t, sp = 0, k0 = 0, klen = K;
        if constexpr (SPLIT) {
            sp = t / tiles_mn;
            u = t - sp * tiles_mn;
            k0 = sp * p.k_split;
            klen = min(p.k_split, K - k0);
        }
        const int steps = (klen + 31) / 32;
        const int blocks = (klen / 32) / D;   // blocks of D steps whose chunks all lie in range
        const int32_t tm = u / p.tiles_n;
        const int32_t tn = u - tm * p.tiles_n;
        const int32_t m = tm * 16 + r, n = tn * 16 + r;
        const bool a_ok = m < M, b_ok = n < N;
        const uint16_t *arow = p.A + static_cast<int64_t>(a_ok ? m : 0) * K + k0 + kq * 8;
        const uint16_t *brow = p.B + static_cast<int64_t>(b_ok ? n : 0) * K + k0 + kq * 8;
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        // whole blocks, double-buffered: block j + 1's loads are in flight
        // while block j's MFMAs (one accumulator, so a dependent chain) run
        half8_t af[2][D], bf[2][D];
        // Unconditional loads (a lane past M or N reads row 0 instead): a
        // load under a branch would make the compiler's vmcnt bookkeeping
        // wait for the other buffer's loads as well.  Row m of A only feeds
        // output column m and row n of B output row n, so those lanes only
        // produce outputs that are never stored.
        auto load = [&](int buf, int j) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                bf[buf][d] = *reinterpret_cast<const half8_t *>(brow + (j * D + d) * 32);
                af[buf][d] = *reinterpret_cast<const half8_t *>(arow + (j * D + d) * 32);
            }
        };
        auto mma = [&](int buf) {
#pragma unroll
            for (int d = 0; d < D; ++d)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[buf][d], af[buf][d], acc, 0, 0, 0);
        };
        // Every load inside is unconditional, so the compiler's waits on a
        // buffer's loads leave the other buffer's in flight (a load that
        // might be skipped would make them wait for everything).  The
        // scheduling barriers keep each block's loads together ahead of the
        // other block's MFMAs: left to itself the compiler spreads them
        // through the MFMA chain, and waits inside the chain then drain the
        // queue to a few loads.  The last trip's prefetch repeats the last
        // block where there is no next one.
        if (blocks > 0) {
            load(0, 0);
            int j = 0;
            for (; j + 2 <= blocks; j += 2) {
                load(1, j + 1);
                __builtin_amdgcn_sched_barrier(0);
                mma(0);
                __builtin_amdgcn_sched_barrier(0);
                load(0, j + 2 < blocks ? j + 2 : blocks - 1);
                __builtin_amdgcn_sched_barrier(0);
                mma(1);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (j < blocks) mma(0);
        }
        // the remaining steps, up to and past K: chunks at or past K are zeros
        for (int s0 = blocks * D; s0 < steps; s0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int s = s0 + d;
                const bool in = s < steps && s * 32 + kq * 8 < klen;
                bf[0][d] = in ? *reinterpret_cast<const half8_t *>(brow + s * 32) : zero;
                af[0][d] = in ? *reinterpret_cast<const half8_t *>(arow + s * 32) : zero;
            }
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (s0 + d < steps)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[0][d], af[0][d], acc, 0, 0, 0);
        }
        // lane l holds C[m0 + l % 16][n0 + 4 (l / 16) + 0..3]
        if (SPLIT && a_ok) {
            const int32_t c0 = tn * 16 + kq * 4;
            float *wrow = p.W + sp * p.split_stride + static_cast<int64_t>(m) * N;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c0 + e < N) wrow[c0 + e] = acc[e];
        } else if (a_ok) {
            const int32_t c0 = tn * 16 + kq * 4;
            uint16_t *crow = p.C + static_cast<int64_t>(m) * N;
            const half4_t h = __builtin_convertvector(acc, half4_t);
            if (c0 + 3 < N) {
                __builtin_memcpy(crow + c0, &h, 8);   // any 2-byte alignment
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < N) reinterpret_cast<_Float16 *>(crow)[c0 + e] = h[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Split-K reduction
// ---------------------------------------------------------------------------
// C = fp16_rne(W_0 + W_1 + ... + W_{splits-1}), summed in fp32 in split order,
// so the result is deterministic.  The partials are M x N row-major and so is
// C, so both are walked as flat arrays: four elements per thread and step
// (each partial starts 256-byte aligned, so the fp32 loads are 16-byte
// aligned), then the last M N mod 4 elements one by one.
template <bool NT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ W,
                                                            int32_t splits, int64_t stride,
                                                            int64_t count, uint16_t *__restrict__ C)
{
    const int64_t nvec = count / 4;
    const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; v < nvec;
         v += step) {
        // every partial is read once: non-temporally when they exceed the L2s
        auto ld = [&](const float *q) {
            if constexpr (NT)
                return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(q));
            else
                return *reinterpret_cast<const f32x4_t *>(q);
        };
        f32x4_t sum = ld(W + 4 * v);
        for (int32_t s = 1; s < splits; ++s) sum += ld(W + s * stride + 4 * v);
        const half4_t h = __builtin_convertvector(sum, half4_t);
        __builtin_memcpy(C + 4 * v, &h, 8);   // C is only 2-byte aligned
    }
    for (int64_t e = 4 * nvec + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
         e < count; e += step) {
        float sum = W[e];
        for (int32_t s = 1; s < splits; ++s) sum += W[s * stride + e];
        reinterpret_cast<_Float16 *>(C)[e] = static_cast<_Float16>(sum);
    }
}

// ---------------------------------------------------------------------------
// General kernel: any K and A, B at any 2-byte alignment
// ---------------------------------------------------------------------------
// The direct-to-LDS path needs every 16-byte chunk of a row 16-byte aligned
// (K a multiple of 8, A and B 16-byte aligned) and 32-bit buffer offsets
// (K <= 2^21).  This path drops all three: each thread loads its 16-byte
// chunks of the next slice into registers with plain global loads (at any
// 2-byte alignment; element by element for the chunk that crosses K, zeros
// for rows past M or N) and writes them to a double-buffered LDS tile in the
// same swizzled layout, while the waves compute the current slice.  One
// barrier per slice: it publishes the slice just written and frees the one
// just read.  32x32x16 MFMAs in the same K order as every other
// configuration, so results are identical to theirs.
template <class CF>
__device__ __forceinline__ half8_t load_chunk(const uint16_t *base, int32_t rows_valid, int row,
                                              int64_t K, int64_t k)
{
    half8_t v = {};
    if (row < rows_valid && k < K) {
        const _Float16 *src = reinterpret_cast<const _Float16 *>(base) + row * K + k;
        if (k + 8 <= K) {
            __builtin_memcpy(&v, src, 16);   // one 16-byte load at any 2-byte alignment
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (k + e < K) v[e] = src[e];
        }
    }
    return v;
}

// Eight consecutive rows at one k of an operand stored with k outermost
// ([K, M] or [K, N], row pitch ld; base is the tile's first row): one 16-byte
// run of the stored row at any 2-byte alignment, element by element for the
// run that crosses the valid rows, zeros past them or past K.
__device__ __forceinline__ half8_t load_run_kn(const uint16_t *base, int32_t rows_valid, int row0,
                                               int64_t ld, int64_t K, int64_t k)
{
    half8_t v = {};
    if (k < K && row0 < rows_valid) {
        const _Float16 *src = reinterpret_cast<const _Float16 *>(base) + k * ld + row0;
        if (row0 + 8 <= rows_valid) {
            __builtin_memcpy(&v, src, 16);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (row0 + e < rows_valid) v[e] = src[e];
        }
    }
    return v;
}

// Position of run c of a k-outermost operand's slice (rows x BK): runs come
// in groups of 64, 8 row-runs by 8 k, so one wave's loads cover 8 k of 128
// contiguous bytes each.
template <class CF, int ROWS>
__device__ __forceinline__ void run_pos_kn(int c, int &row0, int &kl)
{
    constexpr int XG = ROWS / 64;   // groups of 8 runs along the rows
    static_assert(ROWS % 64 == 0 && CF::BK % 8 == 0, "whole 8 x 8 groups of runs");
    const int g = c / 64, l = c % 64;
    row0 = ((g % XG) * 8 + l % 8) * 8;
    kl = (g / XG) * 8 + l / 8;
}

// LA, LB: A stored [K, M] / B stored [K, N] (see Cfg's AL and BL); the LDS
// tiles keep the [rows][K] layout either way, so only the loads differ.
// Three workgroups per CU for NT; two when an operand is stored k-outermost,
// whose chunks take eight 2-byte loads with their own addresses (at three,
// the register budget would spill them).
template <int LA, int LB>
constexpr int any_kernel_per_cu() { return LA || LB ? 2 : 3; }

template <class CF, int LA, int LB>
__global__ __launch_bounds__(CF::THREADS)
__attribute__((amdgpu_waves_per_eu(any_kernel_per_cu<LA, LB>())))
void gemm_f16_nt_any_kernel(Params p)
{
    static_assert(CF::MI == 32 && CF::STAGES == 2, "general path: 32x32x16 MFMAs, 2 buffers");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[CF::LDS_BYTES];
    constexpr int KK = CF::KK;
    constexpr int A_CH = CF::BM * CF::CHUNKS / CF::THREADS;   // chunks per thread per slice
    constexpr int B_CH = CF::BN * CF::CHUNKS / CF::THREADS;
    static_assert(A_CH * CF::THREADS == CF::BM * CF::CHUNKS &&
                  B_CH * CF::THREADS == CF::BN * CF::CHUNKS, "whole chunks per thread");
    const WaveCtx<CF> w(p);
    const int tid = threadIdx.x;
    const int64_t K = p.K;
    const int KT = static_cast<int>((K + CF::BK - 1) / CF::BK);
    half8_t ra[A_CH], rb[B_CH];
    half8_t af[CF::FM], bf[CF::FN];

    int32_t slot = blockIdx.x;
    if (slot >= p.tiles) return;
    while (true) {
        int32_t tile_m, tile_n;
        grouped_tile(slot_to_linear(slot, p.grid, p.tiles, p.xcds), p.tiles_m, p.tiles_n,
                     p.swizzle, tile_m, tile_n);
        Tile t;
        t.m0 = tile_m * CF::BM;
        t.n0 = tile_n * CF::BN;
        const int32_t rows_a = min(CF::BM, p.M - t.m0), rows_b = min(CF::BN, p.N - t.n0);
        // a tile's first row (K-contiguous) or first column ([K, M] / [K, N])
        const uint16_t *a0 = p.A + (LA ? static_cast<int64_t>(t.m0) : static_cast<int64_t>(t.m0) * K);
        const uint16_t *b0 = p.B + (LB ? static_cast<int64_t>(t.n0) : static_cast<int64_t>(t.n0) * K);
        // chunk c of a slice: K-contiguous operands walk a row's chunks with
        // consecutive threads; k-outermost ones load 8-row runs along their
        // stored rows (run_pos_kn), both coalesced
        // one operand's runs of slice kt into registers
        auto load_op = [&](half8_t *r, int n_ch, const uint16_t *base, int32_t rows_valid,
                           auto rows_c, auto kn_c, int64_t ld, int kt) {
            constexpr int ROWS = decltype(rows_c)::value;
            constexpr bool KN = decltype(kn_c)::value;
#pragma unroll
            for (int q = 0; q < n_ch; ++q) {
                const int c = q * CF::THREADS + tid;
                if constexpr (KN) {
                    int row0, kl;
                    run_pos_kn<CF, ROWS>(c, row0, kl);
                    r[q] = load_run_kn(base, rows_valid, row0, ld, K,
                                       static_cast<int64_t>(kt) * CF::BK + kl);
                } else {
                    r[q] = load_chunk<CF>(base, rows_valid, c / CF::CHUNKS, K,
                                          static_cast<int64_t>(kt) * CF::BK + (c % CF::CHUNKS) * 8);
                }
            }
        };
        // ... and from registers into a stage's [rows][K] swizzled tile: a
        // K-contiguous chunk is one 16-byte write, a k-outermost run eight
        // 2-byte writes down its rows
        auto store_op = [&](const half8_t *r, int n_ch, uint8_t *tile, auto rows_c, auto kn_c) {
            constexpr int ROWS = decltype(rows_c)::value;
            constexpr bool KN = decltype(kn_c)::value;
#pragma unroll
            for (int q = 0; q < n_ch; ++q) {
                const int c = q * CF::THREADS + tid;
                if constexpr (KN) {
                    int row0, kl;
                    run_pos_kn<CF, ROWS>(c, row0, kl);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = row0 + e;
                        const int phys = (kl / 8) ^ chunk_swizzle<CF::CHUNKS, CF::MI>(row);
                        *reinterpret_cast<_Float16 *>(tile + row * CF::ROW_BYTES + phys * 16 +
                                                      (kl % 8) * 2) = r[q][e];
                    }
                } else {
                    const int row = c / CF::CHUNKS;
                    const int phys = (c % CF::CHUNKS) ^ chunk_swizzle<CF::CHUNKS, CF::MI>(row);
                    *reinterpret_cast<half8_t *>(tile + row * CF::ROW_BYTES + phys * 16) = r[q];
                }
            }
        };
        using BMc = std::integral_constant<int, CF::BM>;
        using BNc = std::integral_constant<int, CF::BN>;
        using LAc = std::integral_constant<bool, LA != 0>;
        using LBc = std::integral_constant<bool, LB != 0>;
        auto load = [&](int kt) {
            load_op(ra, A_CH, a0, rows_a, BMc{}, LAc{}, p.M, kt);
            load_op(rb, B_CH, b0, rows_b, BNc{}, LBc{}, p.N, kt);
        };
        auto store = [&](int stage) {
            store_op(ra, A_CH, smem + stage * CF::STAGE_BYTES, BMc{}, LAc{});
            store_op(rb, B_CH, smem + stage * CF::STAGE_BYTES + CF::A_BYTES, BNc{}, LBc{});
        };

        typename CF::Acc acc[CF::FM][CF::FN];
        zero_acc<CF>(acc);
        if (KT > 0) {
            load(0);
            store(0);
        }
        lds_barrier();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT) load(kt + 1);     // in flight during this slice's MFMAs
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int i = 0; i < CF::FM; ++i)
                    af[i] = *reinterpret_cast<const half8_t *>(
                        smem + cur * CF::STAGE_BYTES + w.frag_off[0][kk] + w.a_frag_base +
                        i * CF::MI * CF::ROW_BYTES);
#pragma unroll
                for (int j = 0; j < CF::FN; ++j)
                    bf[j] = *reinterpret_cast<const half8_t *>(
                        smem + cur * CF::STAGE_BYTES + w.frag_off[0][kk] + w.b_frag_base +
                        j * CF::MI * CF::ROW_BYTES);
#pragma unroll
                for (int i = 0; i < CF::FM; ++i)
#pragma unroll
                    for (int j = 0; j < CF::FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j],
                                                                          0, 0, 0);
            }
            if (kt + 1 < KT) store(cur ^ 1);
            lds_barrier();
        }
        store_tile<CF>(p, t, acc, w.wave_m, w.wave_n, w.lane);
        slot += p.grid;
        if (slot >= p.tiles) break;
    }
}

// ---------------------------------------------------------------------------
// Kernel table
// ---------------------------------------------------------------------------
struct KernelEntry {
    const void *fn;
    const void *fn_split;   // the instance for K split into ranges (NT configurations)
    int32_t block_m, block_n, block_k, waves, stages, lds_bytes, threads;
    int32_t default_swizzle;
    float rel_rate;   // relative MFMA rate per tile area, for the plan cost model
    float split_rate; // fraction of one CU's dense fp16 peak, fitted to measured times; split planner
    int32_t staged_ok;
    int32_t general;  // the general kernel: any K, A and B at any 2-byte alignment
    int32_t per_cu;   // workgroups resident per CU (the persistent grid's multiple of the CUs)
    int32_t layout;   // operand layouts: 0 NT, 1 NN, 2 TT, 3 TN (2 * A's + B's, see Cfg)
};

template <class CF>
const void *split_instance()
{
    return reinterpret_cast<const void *>(&gemm_f16_nt_kernel<CF, true>);
}

template <class CF>
KernelEntry entry(int swizzle, float rate, float split_rate)
{
    // LDS of the unsplit instance: the ring and the staged epilogue's second
    // buffer (the split instance has the ring only)
    return KernelEntry{reinterpret_cast<const void *>(&gemm_f16_nt_kernel<CF, false>),
                       split_instance<CF>(), CF::BM, CF::BN, CF::BK, CF::WAVES, CF::STAGES,
                       CF::LDS_BYTES + CF::EPI_EXTRA, CF::THREADS,
                       swizzle, rate, split_rate, CF::STAGED_OK ? 1 : 0, 0, 1, 2 * CF::AL + CF::BL};
}

// The producer/consumer kernel: twice the waves of CF (consumers and
// producers), no staged epilogue.
template <class CF>
KernelEntry entry_pc(int swizzle, float rate, float split_rate)
{
    return KernelEntry{reinterpret_cast<const void *>(&gemm_f16_nt_pc_kernel<CF, false>),
                       reinterpret_cast<const void *>(&gemm_f16_nt_pc_kernel<CF, true>),
                       CF::BM, CF::BN, CF::BK, 2 * CF::WAVES, CF::STAGES, CF::LDS_BYTES,
                       2 * CF::THREADS, swizzle, rate, split_rate, 0, 0, 1, 0};
}

// The register-streaming kernel: 16 x 16 tiles, K 32 per MFMA step, no LDS
// ring (stages and LDS 0), one wave per workgroup.
template <int D>
KernelEntry entry_stream(float rate)
{
    return KernelEntry{reinterpret_cast<const void *>(&gemm_f16_nt_stream_kernel<D, false>),
                       reinterpret_cast<const void *>(&gemm_f16_nt_stream_kernel<D, true>),
                       16, 16, 32, 1, 0, 0, 64, 1, rate, 0.0f, 0, 0, 8, 0};
}

template <class CF, int LA = 0, int LB = 0>
KernelEntry entry_general(int swizzle)
{
    return KernelEntry{reinterpret_cast<const void *>(&gemm_f16_nt_any_kernel<CF, LA, LB>),
                       nullptr, CF::BM, CF::BN, CF::BK, CF::WAVES, CF::STAGES, CF::LDS_BYTES,
                       CF::THREADS, swizzle, 0.0f, 0.0f, 0, 1, any_kernel_per_cu<LA, LB>(),
                       2 * LA + LB};
}

static const KernelEntry kKernels[] = {
    entry<Cfg<256, 256, 32, 2, 2, 4>>(8, 0.00f, 0.749f),   // 0: 4 waves of 128x128, 4 stages of K 32
    entry<Cfg<256, 256, 32, 2, 2, 5>>(8, 0.00f, 0.742f),   // 1: the same, 5 stages
    entry<Cfg<256, 128, 64, 2, 2, 3>>(8, 0.85f, 0.700f),   // 2: 4 waves of 128x64, 3 stages of K 64
    entry<Cfg<256, 128, 32, 2, 2, 6>>(8, 0.00f, 0.551f),   // 3: the same tile, 6 stages of K 32
    entry<Cfg<128, 128, 64, 2, 2, 4>>(8, 0.75f, 0.547f),   // 4: 4 waves of 64x64, 4 stages
    entry<Cfg<128, 64, 64, 2, 1, 6>>(8, 0.60f, 0.286f),    // 5: 2 waves of 64x64, 6 stages
    entry<Cfg<256, 256, 32, 2, 4, 4>>(8, 0.00f, 0.747f),   // 6: 8 waves of 128x64, 4 stages of K 32
    entry<Cfg<256, 256, 32, 4, 2, 4>>(8, 0.00f, 0.747f),   // 7: 8 waves of 64x128, 4 stages of K 32
    entry<Cfg<256, 256, 32, 2, 4, 5>>(8, 0.00f, 0.742f),   // 8: 8 waves of 128x64, 5 stages of K 32
    entry<Cfg<256, 256, 64, 2, 2, 2>>(8, 1.00f, 0.721f),   // 9: 4 waves of 128x128, 2 stages of K 64
    entry<Cfg<256, 256, 64, 2, 4, 2>>(8, 0.00f, 0.713f),   // 10: 8 waves of 128x64, 2 stages of K 64
    // 11: as 9 with 16x16x32 MFMAs, the whole refill issued early, A double-buffered
    entry<Cfg<256, 256, 64, 2, 2, 2, 16, 0, 16, 1>>(8, 1.06f, 0.828f),
    entry<Cfg<256, 128, 64, 2, 2, 3, 16>>(8, 0.00f, 0.675f),   // 12: as 2 with 16x16x32 MFMAs
    entry<Cfg<192, 256, 64, 2, 2, 2>>(8, 0.80f, 0.628f),   // 13: 4 waves of 96x128, 2 stages of K 64
    entry<Cfg<256, 192, 64, 2, 2, 2>>(8, 0.82f, 0.628f),   // 14: 4 waves of 128x96, 2 stages of K 64
    entry<Cfg<192, 256, 32, 2, 2, 5>>(8, 0.00f, 0.672f),   // 15: 4 waves of 96x128, 5 stages of K 32
    entry<Cfg<256, 192, 32, 2, 2, 5>>(8, 0.00f, 0.697f),   // 16: 4 waves of 128x96, 5 stages of K 32
    // 17-20: the scheme of 11 on smaller tiles
    entry<Cfg<256, 192, 64, 2, 2, 2, 16, 0, 14, 1>>(8, 0.94f, 0.769f),   // 17: 4 waves of 128x96
    entry<Cfg<192, 256, 64, 2, 2, 2, 16, 0, 14, 1>>(8, 0.97f, 0.759f),   // 18: 4 waves of 96x128
    entry<Cfg<256, 128, 64, 2, 2, 2, 16, 0, 12, 1>>(8, 0.00f, 0.575f),   // 19: 4 waves of 128x64
    entry<Cfg<128, 128, 64, 2, 2, 2, 16, 0, 8, 1>>(8, 0.00f, 0.389f),    // 20: 4 waves of 64x64
    // 21: 4 waves of 32x64.  For a small M the two tile rows that share a B
    // strip run together on one XCD, and B, the operand streamed from HBM,
    // holds two thirds of every stage (a 128x64 tile gives it one third).
    entry<Cfg<64, 128, 64, 2, 2, 6>>(8, 0.65f, 0.349f),
    // 22: 21 with K 128 per stage (256-byte rows): twice the contiguous bytes
    // per row and DMA instruction, which the HBM stream of B prefers
    entry<Cfg<64, 128, 128, 2, 2, 3>>(8, 0.66f, 0.369f),
    // 23: 4 waves of 32x32, five stages of K 128: more tiles for a small M
    // whose 64x128 tiles would leave CUs idle (M <= 256, N of a few thousand)
    entry<Cfg<64, 64, 128, 2, 2, 5>>(8, 0.62f, 0.259f),
    // 24-29: B stored [K, N] (gemm_f16_nn), the schemes of 11 and 18-21 with
    // transposing fragment reads of B
    entry<Cfg<256, 256, 64, 2, 2, 2, 16, 0, 16, 0, 1>>(8, 1.06f, 0.781f),   // 24: as 11, A single-buffered
    entry<Cfg<192, 256, 64, 2, 2, 2, 16, 0, 14, 1, 1>>(8, 0.97f, 0.740f),   // 25: as 18
    entry<Cfg<256, 128, 64, 2, 2, 2, 16, 0, 12, 1, 1>>(8, 0.85f, 0.584f),   // 26: as 19
    entry<Cfg<128, 128, 64, 2, 2, 2, 16, 0, 8, 1, 1>>(8, 0.75f, 0.391f),    // 27: as 20
    entry<Cfg<64, 128, 64, 2, 2, 2, 16, 0, 6, 1, 1>>(8, 0.62f, 0.225f),     // 28: 4 waves of 32x64
    // 29: 28 with 6 stages, the refill spread over each slice: more of B in
    // flight for a small M (the streamed operand)
    entry<Cfg<64, 128, 64, 2, 2, 6, 16, 0, 0, 0, 1>>(8, 0.58f, 0.261f),
    // 30-32: A stored [K, M] and B [N, K] (gemm_f16_tt); 33-35: A [K, M] and
    // B [K, N] (gemm_f16_tn): transposing fragment reads for A as well
    entry<Cfg<256, 256, 64, 2, 2, 2, 16, 0, 16, 0, 0, 1>>(8, 1.06f, 0.778f),   // 30
    entry<Cfg<256, 128, 64, 2, 2, 2, 16, 0, 12, 1, 0, 1>>(8, 0.85f, 0.573f),   // 31
    entry<Cfg<128, 128, 64, 2, 2, 2, 16, 0, 8, 1, 0, 1>>(8, 0.75f, 0.395f),    // 32
    entry<Cfg<256, 256, 64, 2, 2, 2, 16, 0, 16, 0, 1, 1>>(8, 1.06f, 0.735f),   // 33
    entry<Cfg<256, 128, 64, 2, 2, 2, 16, 0, 12, 1, 1, 1>>(8, 0.85f, 0.579f),   // 34
    entry<Cfg<128, 128, 64, 2, 2, 2, 16, 0, 8, 1, 1, 1>>(8, 0.75f, 0.396f),    // 35
    // 36-37: TT with a 64-wide B side (B [N, K] takes any multiple of 32
    // rows; A [K, M] needs 128): 4 waves of 64x32, twice the tiles of 32 for
    // a small M.  36 keeps 6 stages with the refill spread over each slice,
    // as 29 does for NN; 37 is the two-stage early-refill scheme.
    entry<Cfg<128, 64, 64, 2, 2, 6, 16, 0, 0, 0, 0, 1>>(8, 0.56f, 0.266f),     // 36
    entry<Cfg<128, 64, 64, 2, 2, 2, 16, 0, 6, 1, 0, 1>>(8, 0.00f, 0.228f),     // 37
    // 38-41: 64-wide tiles on a k-outermost side (128-byte LDS rows), 6
    // stages with the refill spread over each slice, for a small M or N:
    // 38 NN 128x64 (B [K, N]), 39 TT 64x128 (A [K, M]), 40 TN 64x128, 41 TN
    // 128x64.  Against the same-area tile of the other orientation
    // (29, 36, 40), unsplit and timed by the autotuner over 14-16 shapes
    // each, 38 was about 14% faster than 29, 39 18% faster than 36 and 41 2%
    // faster than 40; the rates of 29, 36 and 40 say so.
    entry<Cfg<128, 64, 64, 2, 2, 6, 16, 0, 0, 0, 1, 0>>(8, 0.66f, 0.294f),     // 38
    entry<Cfg<64, 128, 64, 2, 2, 6, 16, 0, 0, 0, 0, 1>>(8, 0.66f, 0.317f),     // 39
    entry<Cfg<64, 128, 64, 2, 2, 6, 16, 0, 0, 0, 1, 1>>(8, 0.645f, 0.229f),    // 40
    entry<Cfg<128, 64, 64, 2, 2, 6, 16, 0, 0, 0, 1, 1>>(8, 0.66f, 0.228f),     // 41
    // 42: 256x128x64, three stages, four consumer waves of 128x64 (16x16x32
    // MFMAs, both fragments double-buffered) and four producer waves that
    // only issue the DMA (gemm_f16_nt_pc_kernel).  Faster than 2 and 19, the
    // same tile with every wave loading, on every shape measured (8192^3:
    // 814 against 937 and 857 us), so it takes 2's place in both planners
    // (split_rate: 2's scaled by the unsplit gain at 2048 x 4096 x 8192, 1.11)
    entry_pc<Cfg<256, 128, 64, 2, 2, 3, 16, 0, 0, 1>>(8, 0.87f, 0.754f),
    // 43: B streamed through registers for a few rows of A (planned for M <=
    // 16: see choose_config_planned)
    entry_stream<12>(0.0f),
    // 44-46: the general kernel for NN, TT and TN (loads along the operand's
    // contiguous dimension), for arguments the direct-to-LDS kernels of those
    // layouts cannot take
    entry_general<Cfg<128, 128, 32, 2, 2, 2>, 0, 1>(8),
    entry_general<Cfg<128, 128, 32, 2, 2, 2>, 1, 0>(8),
    entry_general<Cfg<128, 128, 32, 2, 2, 2>, 1, 1>(8),
    // 47: the general kernel, 4 waves of 64x64, two register-staged buffers of
    // K 32; planned only when the direct-to-LDS path cannot run
    entry_general<Cfg<128, 128, 32, 2, 2, 2>>(8),
};
constexpr int kNumKernels = sizeof(kKernels) / sizeof(kKernels[0]);
constexpr int kGeneralConfig = kNumKernels - 1;

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static bool overlaps(const void *p, int64_t pbytes, const void *q, int64_t qbytes)
{
    if (pbytes <= 0 || qbytes <= 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + static_cast<uintptr_t>(qbytes) && b < a + static_cast<uintptr_t>(pbytes);
}

static int validate(int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C)
{
    if (M < 0 || N < 0 || K < 0) return GEMM_F16_INVALID_ARG;
    // every dimension below 2^31 first: the byte counts below then stay
    // below 2^63
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return GEMM_F16_UNSUPPORTED;
    const int64_t a_bytes = M * K * 2, b_bytes = N * K * 2, c_bytes = M * N * 2;
    if ((a_bytes > 0 && !A) || (b_bytes > 0 && !B) || (c_bytes > 0 && !C))
        return GEMM_F16_INVALID_ARG;
    if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes))
        return GEMM_F16_INVALID_ARG;
    // fp16 elements: every matrix at least 2-byte aligned
    if ((a_bytes > 0 && reinterpret_cast<uintptr_t>(A) % 2 != 0) ||
        (b_bytes > 0 && reinterpret_cast<uintptr_t>(B) % 2 != 0) ||
        (c_bytes > 0 && reinterpret_cast<uintptr_t>(C) % 2 != 0))
        return GEMM_F16_UNSUPPORTED;
    // the smallest tile (64 x 64) must leave the tile count within int32
    if (cdiv(M, 64) * cdiv(N, 64) > INT32_MAX) return GEMM_F16_UNSUPPORTED;
    return GEMM_F16_OK;
}

// Whether the direct-to-LDS configurations can run these arguments: K a
// multiple of 8 and at most 2^21, A and B 16-byte aligned.  Otherwise only
// the general kernel can.
static bool needs_general(int64_t K, const void *A, const void *B, bool check_pointers)
{
    if (K % 8 != 0 || K > MAX_K) return true;
    if (!check_pointers) return false;
    return reinterpret_cast<uintptr_t>(A) % 16 != 0 || reinterpret_cast<uintptr_t>(B) % 16 != 0;
}

static void fill_info(int id, gemm_f16_nt_plan_t *out)
{
    const KernelEntry &e = kKernels[id];
    *out = gemm_f16_nt_plan_t{};
    out->config_id = id;
    out->block_m = e.block_m;
    out->block_n = e.block_n;
    out->block_k = e.block_k;
    out->waves = e.waves;
    out->stages = e.stages;
    out->swizzle = e.default_swizzle;
    out->lds_bytes = e.lds_bytes;
    out->xcds = DEFAULT_XCDS;
    out->a_layout = e.layout >> 1;
    out->b_layout = e.layout & 1;
}

// Epilogue policy: stage C through LDS whenever the configuration has room
// for it (row-contiguous stores measured faster than direct stores from the
// MFMA layout for aligned and unaligned C alike).
static int32_t choose_epilogue(int id) { return kKernels[id].staged_ok ? 1 : 0; }

static void make_plan(int id, int64_t M, int64_t N, int32_t num_cus, int32_t swizzle,
                      int32_t grid, gemm_f16_nt_plan_t *out)
{
    fill_info(id, out);
    out->epilogue = choose_epilogue(id);
    out->tiles_m = static_cast<int32_t>(cdiv(M, out->block_m));
    out->tiles_n = static_cast<int32_t>(cdiv(N, out->block_n));
    out->tiles = static_cast<int64_t>(out->tiles_m) * out->tiles_n;
    if (swizzle > 0) out->swizzle = swizzle;
    if (out->swizzle > out->tiles_n) out->swizzle = out->tiles_n > 0 ? out->tiles_n : 1;
    const int64_t cap = grid > 0 ? grid : (num_cus > 0 ? int64_t(num_cus) * kKernels[id].per_cu : 1);
    out->grid = static_cast<int32_t>(out->tiles < cap ? out->tiles : cap);
}

static double split_cost(int id, int64_t M, int64_t N, int64_t K, int32_t splits, int32_t cus,
                         int64_t *splits_eff);

// Cost model: rounds of the persistent grid times the time one tile takes,
// which scales with its area over the configuration's relative MFMA rate.
// Entries with rel_rate 0 are compiled for sweeps but never planned.  Between
// tiles of equal cost, one whose long side lies along the longer of M and N
// is preferred (1%): its strip of the larger operand, the one streamed from
// HBM, then fills most of each LDS stage.
//
// This rule sees no K.  When K is long and the tiles are small, their
// operand traffic (which grows as the tile shrinks) decides instead: at
// 1536 x 1536 x 16384 the rule's 64 x 64 tiles took 1.78 times as long as
// 128 x 128 ones, at 2048 x 3072 x 4096 its 64 x 128 tiles 1.54 times as long
// as the 256 x 128 producer/consumer tile.  So the plan is then checked
// against the fitted time model of the split planner (split_cost, one range),
// which counts K and the operand bytes, and the model's unsplit pick replaces
// the rule's when it predicts a gain above kModelMargin.  Below that the rule
// stands: against measured times the model errs by up to about 11% on fully
// occupied shapes (8192 x 5120 x 8192: it prefers the 256 x 128 tile by 8%,
// the 256 x 256 one measures 2.5% faster).  Timed on one MI355X over square
// and oblong shapes from 256 to 8192 in all four layouts, the plans this
// check changes ran at 0.64 of the rule's time (geometric mean, none
// slower), while the model's picks below the margin were no better than the
// rule's.
static int choose_config_search(int64_t M, int64_t N, int64_t K, int32_t num_cus, int32_t layout)
{
    constexpr double kModelMargin = 1.15;
    int best = -1;
    double best_cost = 0.0;
    for (int id = 0; id < kNumKernels; ++id) {
        const KernelEntry &e = kKernels[id];
        if (e.rel_rate <= 0.0f || e.layout != layout) continue;
        const int64_t tiles = cdiv(M, e.block_m) * cdiv(N, e.block_n);
        const int64_t rounds = cdiv(tiles, num_cus > 0 ? num_cus : 1);
        const bool along = (N > M && e.block_n > e.block_m) || (M > N && e.block_m > e.block_n);
        const double cost = static_cast<double>(rounds) * e.block_m * e.block_n / e.rel_rate *
                            (along ? 0.99 : 1.0);
        if (best < 0 || cost < best_cost) {
            best = id;
            best_cost = cost;
        }
    }
    if (best < 0 || K <= 0) return best;
    int64_t eff = 1;
    const double rule_time = split_cost(best, M, N, K, 1, num_cus, &eff);
    int alt = best;
    double alt_time = rule_time;
    for (int id = 0; id < kNumKernels; ++id) {
        const KernelEntry &e = kKernels[id];
        if (e.rel_rate <= 0.0f || e.layout != layout || e.general) continue;
        const double t = split_cost(id, M, N, K, 1, num_cus, &eff);
        if (t < alt_time) {
            alt = id;
            alt_time = t;
        }
    }
    return rule_time > kModelMargin * alt_time ? alt : best;
}

// The register-streaming configuration (no LDS ring) and when the plain plan
// takes it: NT, at most kStreamMaxM rows of A, and a plan whose tiles would
// fill at most a quarter of the CUs; or at most kStreamHalfM rows, K up to
// kStreamHalfK and tiles on at most half the CUs.  Timed on one MI355X in
// captured graphs against the plan it replaces (M = 1 / 4 / 8 / 16): 4096 x
// 4096 7.6 / 8.6 / 8.9 / 10.6 us against 15.6-15.8; N = 4096, K = 14336
// 19.2 / - / 22.9 / - us against 45.4; N = 8192 (M = 1 / 4 / 8), K = 2048
// 7.1 / 7.8 / 8.4 against 9.7-9.8 and K = 4096 13.4 / 14.2 / 15.4 against
// 15.8-16.0.  With more tiles, more rows or a longer K the tile kernels keep
// up (N = 8192, K = 16384, M = 4: 56.9 against 51.8; N = 14336 at K = 4096
// they are faster).  Up to kStreamRoundM rows it still wins where its 16 x 16
// tiles fit in one round of the CUs and the tile plan fills at most a
// quarter: B is then read once per 16 rows of A, but the reads after the
// first hit the L2s (the tile rows run together), and the grid has more
// waves than the tile plan's (M = 17 / 32 / 64 at N = 1024, K = 8192: 16.6 /
// 16.5 / 16.5 us against 27.4-27.5; M = 32 at N = 2048, K = 4096: 10.2
// against 15.8).  With more tiles B's reads are too many (M = 48, N = 2048,
// K = 4096: 17.7 against 15.8).
constexpr int64_t kStreamMaxM = 16;
constexpr int64_t kStreamHalfM = 8;
constexpr int64_t kStreamHalfK = 8192;
constexpr int64_t kStreamRoundM = 64;

static int stream_config()
{
    static const int id = [] {
        for (int i = 0; i < kNumKernels; ++i)
            if (kKernels[i].stages == 0) return i;
        return -1;
    }();
    return id;
}

static int choose_config_planned(int64_t M, int64_t N, int64_t K, int32_t num_cus, int32_t layout)
{
    const int id = choose_config_search(M, N, K, num_cus, layout);
    const int st = stream_config();
    if (layout != 0 || st < 0 || id < 0 || K <= 0) return id;
    // the kernel's loads and tiles treat A and B alike, so a few columns of
    // B (A streamed) count as a few rows of A
    const int64_t few = M < N ? M : N;
    const int64_t tiles = cdiv(M, kKernels[id].block_m) * cdiv(N, kKernels[id].block_n);
    if ((few <= kStreamMaxM && tiles * 4 <= num_cus) ||
        (few <= kStreamHalfM && K <= kStreamHalfK && tiles * 2 <= num_cus) ||
        (few <= kStreamRoundM && tiles * 4 <= num_cus &&
         cdiv(M, kKernels[st].block_m) * cdiv(N, kKernels[st].block_n) <= num_cus))
        return st;
    return id;
}

// choose_config_planned behind a per-thread cache of the last few decisions
// (the search prices every configuration of the layout), so a caller that
// repeats a shape pays for it once.
static int choose_config(int64_t M, int64_t N, int64_t K, int32_t num_cus, int32_t layout = 0)
{
    struct Choice {
        int64_t M = -1, N = -1, K = -1;
        int32_t cus = 0, layout = 0;
        int id = -1;
    };
    static thread_local Choice cache[4];
    static thread_local int next = 0;
    for (const Choice &c : cache)
        if (c.id >= 0 && c.M == M && c.N == N && c.K == K && c.cus == num_cus && c.layout == layout)
            return c.id;
    const int id = choose_config_planned(M, N, K, num_cus, layout);
    cache[next] = Choice{M, N, K, num_cus, layout, id};
    next = (next + 1) % 4;
    return id;
}

struct DeviceInfo {
    std::once_flag once;
    int32_t cus = 0;
    hipError_t err = hipSuccess;
};
constexpr int kMaxDevices = 64;
static DeviceInfo g_devices[kMaxDevices];

static int current_cus(int32_t *cus)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMM_F16_LAUNCH_FAILED;
    DeviceInfo &d = g_devices[dev];
    std::call_once(d.once, [&] {
        int v = 0;
        d.err = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        d.cus = v;
    });
    if (d.err != hipSuccess || d.cus <= 0) return GEMM_F16_LAUNCH_FAILED;
    *cus = d.cus;
    return GEMM_F16_OK;
}

// ---------------------------------------------------------------------------
// Split over K (for tile counts that leave most CUs idle)
// ---------------------------------------------------------------------------
constexpr int32_t kMaxSplits = 64;
constexpr int64_t kMinSplitK = 512;   // K per unit the planner goes down to

// Partials of more bytes than the L2s hold together (8 XCDs of 4 MB) are
// written and read back non-temporally: they would only evict the GEMM's
// A and B strips.  Smaller ones stay in L2 for the reduction (measured both
// ways: 1024 x 1024 x 65536, 64 MB of partials, +22% non-temporal; 256 x 256
// x 65536, 4 MB, -14%).
static bool nt_partials(int64_t splits, int64_t M, int64_t N)
{
    return splits * M * N * 4 > (int64_t(32) << 20);
}

// fp32 elements between the partials of consecutive splits: M N rounded up to
// 64, so each partial starts 256-byte aligned when the workspace does
static int64_t split_stride(int64_t M, int64_t N) { return cdiv(M * N, 64) * 64; }

// K per unit when K is split `splits` ways for configuration `id`: a multiple
// of its K slice, so every unit but the last covers whole slices.  The
// effective split count is then cdiv(K, k_split) <= splits.
static int64_t split_k_len(int id, int64_t K, int32_t splits)
{
    const int64_t bk = kKernels[id].block_k;
    return cdiv(cdiv(K, splits), bk) * bk;
}

// Estimated time of configuration `id` with K split `splits` ways, a model
// fitted to measured times of every configuration and split count on 28
// shapes per layout (under-filled grids, long and short K; one MI355X; the
// tables and the fit are in planner_fit/, beside this directory):
//   compute  rounds of the persistent grid x (one unit's MFMA work at the
//            configuration's split_rate of a CU's dense fp16 peak + a fixed
//            cost per unit)
//   operands A and B read once from HBM, at a bandwidth that falls with the
//            fraction of CUs the units occupy
//   time     the larger of the two plus a tenth of the smaller (they overlap
//            almost entirely), a fixed launch cost and C written to HBM
//   split    when K is actually split, the fp32 partials written and read
//            back, the fp16 result written, and the reduction launch.
static double split_cost(int id, int64_t M, int64_t N, int64_t K, int32_t splits, int32_t cus,
                         int64_t *splits_eff)
{
    constexpr double kCuPeak = 2.5e15 / 256;   // dense fp16 flop/s of one CU
    constexpr double kUnitSec = 2.3e-07;      // per unit: pipeline fill and epilogue
    constexpr double kLaunchSec = 3.59e-06;     // per launch
    constexpr double kHbmBytesPerSec = 4.08e+12;
    static constexpr double kActiveExp = 0.351;      // bandwidth ~ (fraction of CUs busy)^kActiveExp
    constexpr double kOverlap = 0.1;
    constexpr double kReduceBytesPerSec = 4.95e+12;
    constexpr double kReduceSec = 3.34e-06;
    const KernelEntry &e = kKernels[id];
    if (cus <= 0) cus = 1;
    const int64_t ks = split_k_len(id, K, splits);
    const int64_t eff = cdiv(K, ks);
    const int64_t units = cdiv(M, e.block_m) * cdiv(N, e.block_n) * eff;
    const double rounds = static_cast<double>(cdiv(units, cus));
    const double rate = e.split_rate > 0.0f ? e.split_rate : 0.01;
    const double compute =
        rounds * (e.block_m * e.block_n * static_cast<double>(eff > 1 ? ks : K) * 2.0 /
                      (rate * kCuPeak) + kUnitSec);
    // (fraction of CUs busy)^kActiveExp, tabulated in steps of 1/1024
    static const std::array<float, 1025> busy_pow = [] {
        std::array<float, 1025> t{};
        for (int i = 0; i <= 1024; ++i)
            t[i] = static_cast<float>(std::pow(std::max(i, 1) / 1024.0, kActiveExp));
        return t;
    }();
    const double busy = units < cus ? busy_pow[units * 1024 / cus] : 1.0;
    const double operands =
        static_cast<double>(M + N) * static_cast<double>(K) * 2.0 / (kHbmBytesPerSec * busy);
    const double mn = static_cast<double>(M) * static_cast<double>(N);
    double t = std::max(compute, operands) + kOverlap * std::min(compute, operands) + kLaunchSec +
               mn * 2.0 / kHbmBytesPerSec;
    if (eff > 1) t += (2.0 * eff * mn * 4.0 + mn * 2.0) / kReduceBytesPerSec + kReduceSec;
    *splits_eff = eff;
    return t;
}

// Whether configuration `id` takes part in the split-K planner's search:
// only configurations the plain planner may choose (rel_rate > 0; the others
// are compiled for sweeps and tests), and of those with one layout and tile,
// only the one with the highest split_rate (split_cost sees nothing else of
// a configuration but the rounding of K to its slices).  Keeps the search to
// a few hundred cost evaluations per call.
static bool split_candidate(int id)
{
    static const std::array<bool, kNumKernels> flags = [] {
        std::array<bool, kNumKernels> f{};
        auto plannable = [](const KernelEntry &e) {
            return e.split_rate > 0.0f && e.rel_rate > 0.0f && !e.general;
        };
        for (int i = 0; i < kNumKernels; ++i) {
            const KernelEntry &e = kKernels[i];
            f[i] = plannable(e);
            for (int j = 0; j < kNumKernels && f[i]; ++j) {
                const KernelEntry &o = kKernels[j];
                if (j != i && plannable(o) && o.layout == e.layout && o.block_m == e.block_m &&
                    o.block_n == e.block_n &&
                    (o.split_rate > e.split_rate || (o.split_rate == e.split_rate && j < i)))
                    f[i] = false;
            }
        }
        return f;
    }();
    return flags[id];
}

// The split planner's choice for a register-streaming plan, which its cost
// model has no rate for ("few" is the smaller of M and N: the kernel treats
// A and B alike).  One CU keeps only so many loads in flight, so where the
// 16 x 16 tiles occupy few CUs only a split over K adds bandwidth: S ranges
// of K per tile, S the largest power of two with tiles S <= CUs, S <=
// kStreamMaxSplits and K / S >= kStreamMinSplitK (only for few <=
// kStreamMaxM).  The plan is kept where it beat the model's split of a tile
// configuration: grids of at most a quarter of the CUs with few <=
// kStreamMaxM; K <= kStreamKeepK; few <= kStreamFewM with K <=
// kStreamFewAnyK, or K <= kStreamFewMK and at most one tile per CU; or K <=
// kStreamShortK with few <=
// kStreamHalfM or at most a quarter of the CUs.  Elsewhere (more tiles and a
// long K) the model's split stands.  Timed on one MI355X in captured graphs
// over M in {1, 4, 8, 16}, N from 256 to 4096 and K from 2048 to 32768 (80
// shapes): 0.85 of the model's split's time (geometric mean; 1 x 256 x 32768
// 9.6 against 20.8 us, 1 x 4096 x 4096 7.5 against 9.8), none more than 3%
// slower; the short-K clause, over 70 random shapes with few <= 64 and K
// from 2056 to 4096, changed 20 plans, to 0.72 of the time (3467 x 5 x 3856
// 6.5 against 13.2 us), none slower; the few <= kStreamFewM clause up to K =
// kStreamFewAnyK, over 36 shapes with 1, 3 or 4 rows or columns, the other
// side 4500-10000 and K = 4200 or 5000, to 0.72 (7500 x 1 x 4200 12.1
// against 22.4 us), none slower (at K = 6144 it lost up to 1.26 times).
constexpr int32_t kStreamMaxSplits = 16;
constexpr int64_t kStreamMinSplitK = 2048;
constexpr int64_t kStreamKeepK = 2048;
constexpr int64_t kStreamFewM = 4;
constexpr int64_t kStreamFewMK = 8192;
constexpr int64_t kStreamFewAnyK = 5120;
constexpr int64_t kStreamShortK = 4096;

static bool stream_split(int64_t M, int64_t N, int64_t K, int32_t cus, int32_t *splits_out)
{
    const int64_t tiles = cdiv(M, 16) * cdiv(N, 16);
    const int64_t c = cus > 0 ? cus : 1;
    const int64_t few = M < N ? M : N;   // rows of A or columns of B
    const bool short_k = K <= kStreamShortK && (few <= kStreamHalfM || tiles * 4 <= c);
    const bool few_k =
        few <= kStreamFewM && (K <= kStreamFewAnyK || (K <= kStreamFewMK && tiles <= c));
    if (!((few <= kStreamMaxM && tiles * 4 <= c) || K <= kStreamKeepK || few_k || short_k))
        return false;
    int32_t s = 1;
    while (few <= kStreamMaxM && s * 2 <= kStreamMaxSplits && tiles * s * 2 <= c &&
           K / (s * 2) >= kStreamMinSplitK)
        s *= 2;
    *splits_out = s > 1 ? static_cast<int32_t>(cdiv(K, split_k_len(stream_config(), K, s))) : 1;
    return true;
}

// Configuration and effective split count for the split-K entry points
// (K > 0, direct-to-LDS arguments).  config_id >= 0 fixes the configuration;
// splits > 0 fixes the requested count, and splits == 1 (or no split chosen)
// means exactly the plain entry point's plan.  Otherwise the cheapest by
// split_cost among the plain plan and the layout's split candidates split at
// least two ways (K per unit at least kMinSplitK, at most 4 rounds of units).
static void choose_split_search(int64_t M, int64_t N, int64_t K, int32_t cus, int32_t config_id,
                                int32_t splits, int *id_out, int32_t *splits_out, int32_t layout)
{
    const int plain = config_id >= 0 ? config_id : choose_config(M, N, K, cus, layout);
    if (splits <= 0 && config_id < 0 && plain == stream_config() &&
        stream_split(M, N, K, cus, splits_out)) {
        *id_out = plain;
        return;
    }
    double best = 0.0;
    int best_id = -1;
    int64_t best_eff = 1;
    auto consider = [&](int id, int32_t sp) {
        int64_t eff = 1;
        const double c = split_cost(id, M, N, K, sp, cus, &eff);
        if (best_id < 0 || c < best) {
            best = c;
            best_id = id;
            best_eff = eff;
        }
    };
    if (splits == 1) {
        *id_out = plain;
        *splits_out = 1;
        return;
    }
    if (splits <= 0) consider(plain, 1);
    for (int id = 0; id < kNumKernels; ++id) {
        if (config_id >= 0 ? id != config_id
                           : (!split_candidate(id) || kKernels[id].layout != layout))
            continue;
        const int32_t s_lo = splits > 0 ? splits : 2;
        const int32_t s_hi = splits > 0 ? splits : kMaxSplits;
        const int64_t tiles = cdiv(M, kKernels[id].block_m) * cdiv(N, kKernels[id].block_n);
        for (int32_t sp = s_lo; sp <= s_hi; ++sp) {
            if (splits <= 0 && cdiv(K, sp) < kMinSplitK) break;
            // beyond 4 rounds of the grid more ranges only add partials
            if (splits <= 0 && tiles * sp > 4 * int64_t(cus > 0 ? cus : 1)) break;
            if (splits <= 0 && cdiv(K, split_k_len(id, K, sp)) <= 1) continue;
            consider(id, sp);
        }
    }
    *id_out = best_id;
    *splits_out = static_cast<int32_t>(best_eff);
    if (best_eff <= 1 && splits <= 0) *id_out = plain;
}

// choose_split_search behind a per-thread cache of the last few decisions, so
// a caller that repeats a shape does not pay for the search on every call.
static void choose_split(int64_t M, int64_t N, int64_t K, int32_t cus, int32_t config_id,
                         int32_t splits, int *id_out, int32_t *splits_out, int32_t layout = 0)
{
    struct Choice {
        int64_t M = -1, N = -1, K = -1;
        int32_t cus = 0, config_id = 0, splits = 0, layout = 0;
        int id = -1;
        int32_t eff = 1;
    };
    static thread_local Choice cache[4];
    static thread_local int next = 0;
    for (const Choice &c : cache) {
        if (c.id >= 0 && c.M == M && c.N == N && c.K == K && c.cus == cus &&
            c.config_id == config_id && c.splits == splits && c.layout == layout) {
            *id_out = c.id;
            *splits_out = c.eff;
            return;
        }
    }
    choose_split_search(M, N, K, cus, config_id, splits, id_out, splits_out, layout);
    Choice &c = cache[next];
    next = (next + 1) % 4;
    c.M = M;
    c.N = N;
    c.K = K;
    c.cus = cus;
    c.config_id = config_id;
    c.splits = splits;
    c.layout = layout;
    c.id = *id_out;
    c.eff = *splits_out;
}

static int launch(const gemm_f16_nt_plan_t &plan, int64_t M, int64_t N, int64_t K,
                  const void *A, const void *B, void *C, hipStream_t stream,
                  int32_t splits = 1, int64_t k_split = 0, float *W = nullptr)
{
    Params p;
    p.A = static_cast<const uint16_t *>(A);
    p.B = static_cast<const uint16_t *>(B);
    p.C = static_cast<uint16_t *>(C);
    p.M = static_cast<int32_t>(M);
    p.N = static_cast<int32_t>(N);
    p.K = static_cast<int32_t>(K);
    p.tiles_m = plan.tiles_m;
    p.tiles_n = plan.tiles_n;
    p.tiles = static_cast<int32_t>(plan.tiles);
    p.swizzle = plan.swizzle;
    p.grid = plan.grid;
    p.xcds = plan.xcds;
    p.staged = plan.epilogue;
    p.splits = splits;
    p.k_split = static_cast<int32_t>(splits > 1 ? k_split : K);
    p.split_stride = splits > 1 ? split_stride(M, N) : 0;
    p.W = W;
    p.nt_w = splits > 1 && nt_partials(splits, M, N) ? 1 : 0;
    if (splits > 1) p.tiles = static_cast<int32_t>(plan.tiles * splits);
    const KernelEntry &e = kKernels[plan.config_id];
    void *args[] = {&p};
    // the launch's own status only: the thread's sticky error state (which may
    // hold an unrelated earlier error) is neither read nor cleared
    const void *fn = splits > 1 ? e.fn_split : e.fn;
    if (!fn) return GEMM_F16_UNSUPPORTED;
    const hipError_t err = hipLaunchKernel(fn, dim3(plan.grid), dim3(e.threads), args, 0, stream);
    return err == hipSuccess ? GEMM_F16_OK : GEMM_F16_LAUNCH_FAILED;
}

static int run(int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C,
               hipStream_t stream, int32_t config_id, int32_t swizzle, int32_t grid,
               int32_t epilogue)
{
    const int v = validate(M, N, K, A, B, C);
    if (v != GEMM_F16_OK) return v;
    if (config_id >= kNumKernels || (config_id >= 0 && kKernels[config_id].layout != 0))
        return GEMM_F16_INVALID_ARG;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    const bool general = needs_general(K, A, B, K > 0);
    if (general && config_id >= 0 && !kKernels[config_id].general) return GEMM_F16_UNSUPPORTED;
    int32_t cus = 0;
    const int s = current_cus(&cus);
    if (s != GEMM_F16_OK) return s;
    const int id = config_id >= 0 ? config_id
                                  : (general ? kGeneralConfig : choose_config(M, N, K, cus));
    gemm_f16_nt_plan_t plan;
    make_plan(id, M, N, cus, swizzle, grid, &plan);
    if (epilogue < 0) {
        plan.epilogue = choose_epilogue(id);
    } else {
        if (epilogue > 1 || (epilogue == 1 && !kKernels[id].staged_ok)) return GEMM_F16_UNSUPPORTED;
        plan.epilogue = epilogue;
    }
    return launch(plan, M, N, K, A, B, C, stream);
}

// Layouts other than NT (layout = 2 * A's + B's: 1 NN, 2 TT, 3 TN): only the
// direct-to-LDS kernels of that layout take them.  Each operand's rows must
// be 16-byte aligned: a K-contiguous operand needs K a multiple of 8 and at
// most 2^21 (as on the NT path), an M- or N-contiguous one M or N a multiple
// of 8 and its K rows within 2^31 bytes of offsets; A and B 16-byte aligned.
static bool layout_supported(int32_t layout, int64_t M, int64_t N, int64_t K, const void *A,
                             const void *B, bool check_pointers)
{
    const bool a_kn = (layout >> 1) & 1, b_kn = layout & 1;
    if (K > MAX_K) return false;
    if (a_kn ? (M % 8 != 0 || K * M * 2 > INT32_MAX) : K % 8 != 0) return false;
    if (b_kn ? (N % 8 != 0 || K * N * 2 > INT32_MAX) : K % 8 != 0) return false;
    if (!check_pointers) return true;
    return reinterpret_cast<uintptr_t>(A) % 16 == 0 && reinterpret_cast<uintptr_t>(B) % 16 == 0;
}

// The general kernel of a layout (any sizes, any 2-byte alignment).
static int general_config(int32_t layout)
{
    for (int id = 0; id < kNumKernels; ++id)
        if (kKernels[id].general && kKernels[id].layout == layout) return id;
    return kGeneralConfig;
}

static int run_layout(int32_t layout, int64_t M, int64_t N, int64_t K, const void *A,
                      const void *B, void *C, hipStream_t stream, int32_t config_id,
                      int32_t swizzle, int32_t grid, int32_t epilogue)
{
    const int v = validate(M, N, K, A, B, C);   // A and B hold M K and K N elements either way
    if (v != GEMM_F16_OK) return v;
    if (config_id >= kNumKernels || (config_id >= 0 && kKernels[config_id].layout != layout))
        return GEMM_F16_INVALID_ARG;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    if (K == 0) return run(M, N, 0, A, B, C, stream, -1, 0, 0, -1);   // the empty sum
    // arguments the direct-to-LDS kernels of the layout cannot take run its
    // general kernel
    const bool fast = layout_supported(layout, M, N, K, A, B, true);
    if (!fast && config_id >= 0 && !kKernels[config_id].general) return GEMM_F16_UNSUPPORTED;
    int32_t cus = 0;
    const int s = current_cus(&cus);
    if (s != GEMM_F16_OK) return s;
    const int id = config_id >= 0 ? config_id
                                  : (fast ? choose_config(M, N, K, cus, layout) : general_config(layout));
    gemm_f16_nt_plan_t plan;
    make_plan(id, M, N, cus, swizzle, grid, &plan);
    if (epilogue < 0) {
        plan.epilogue = choose_epilogue(id);
    } else {
        if (epilogue > 1 || (epilogue == 1 && !kKernels[id].staged_ok)) return GEMM_F16_UNSUPPORTED;
        plan.epilogue = epilogue;
    }
    return launch(plan, M, N, K, A, B, C, stream);
}

static int plan_layout(int32_t layout, int64_t M, int64_t N, int64_t K, int32_t num_cus,
                       gemm_f16_nt_plan_t *plan)
{
    if (!plan || M < 0 || N < 0 || K < 0 || num_cus <= 0) return GEMM_F16_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || cdiv(M, 64) * cdiv(N, 64) > INT32_MAX)
        return GEMM_F16_UNSUPPORTED;
    if (K == 0) return gemm_f16_nt_plan(M, N, K, num_cus, plan);
    const int id = layout_supported(layout, M, N, K, nullptr, nullptr, false)
                       ? choose_config(M, N, K, num_cus, layout) : general_config(layout);
    make_plan(id, M, N, num_cus, 0, 0, plan);
    return GEMM_F16_OK;
}

// fixed_scratch: the workspace is the library's own fixed-size scratch array
// (gemm_f16_nt_splitk_noalloc), so a plan that needs more of it than it
// holds is reported as GEMM_F16_SCRATCH_LIMIT rather than as a bad argument.
static int run_splitk(int32_t layout, int64_t M, int64_t N, int64_t K, const void *A,
                      const void *B, void *C, int32_t splits, void *workspace,
                      int64_t workspace_bytes, hipStream_t stream, int32_t config_id,
                      bool fixed_scratch = false)
{
    const int v = validate(M, N, K, A, B, C);
    if (v != GEMM_F16_OK) return v;
    if (config_id >= kNumKernels || (config_id >= 0 && kKernels[config_id].layout != layout) ||
        splits > kMaxSplits || workspace_bytes < 0)
        return GEMM_F16_INVALID_ARG;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    if (K == 0) return run(M, N, 0, A, B, C, stream, -1, 0, 0, -1);   // the empty sum
    if (layout == 0) {
        // arguments only the general kernel takes: no split
        if (needs_general(K, A, B, true) || (config_id >= 0 && kKernels[config_id].general))
            return run(M, N, K, A, B, C, stream, config_id, 0, 0, -1);
    } else if (!layout_supported(layout, M, N, K, A, B, true) ||
               (config_id >= 0 && kKernels[config_id].general)) {
        // the layout's general kernel, without a split
        return run_layout(layout, M, N, K, A, B, C, stream, config_id, 0, 0, -1);
    }
    int32_t cus = 0;
    const int s = current_cus(&cus);
    if (s != GEMM_F16_OK) return s;
    int id = -1;
    int32_t eff = 1;
    choose_split(M, N, K, cus, config_id, splits, &id, &eff, layout);
    if (eff <= 1)
        return layout == 0 ? run(M, N, K, A, B, C, stream, id, 0, 0, -1)
                           : run_layout(layout, M, N, K, A, B, C, stream, id, 0, 0, -1);
    gemm_f16_nt_plan_t plan;
    make_plan(id, M, N, cus, 0, 0, &plan);
    if (plan.tiles * eff > INT32_MAX) return GEMM_F16_UNSUPPORTED;
    const int64_t stride = split_stride(M, N);
    const int64_t need = eff * stride * 4;
    if (!workspace || workspace_bytes < need)
        return fixed_scratch ? GEMM_F16_SCRATCH_LIMIT : GEMM_F16_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return GEMM_F16_UNSUPPORTED;
    if (overlaps(workspace, need, A, M * K * 2) || overlaps(workspace, need, B, N * K * 2) ||
        overlaps(workspace, need, C, M * N * 2))
        return GEMM_F16_INVALID_ARG;
    const int64_t units = plan.tiles * eff;
    const int64_t cap = int64_t(cus) * kKernels[id].per_cu;
    plan.grid = static_cast<int32_t>(units < cap ? units : cap);
    plan.epilogue = 0;
    float *W = static_cast<float *>(workspace);
    const int l = launch(plan, M, N, K, A, B, C, stream, eff, split_k_len(id, K, eff), W);
    if (l != GEMM_F16_OK) return l;
    const int64_t count = M * N;
    const int64_t blocks = cdiv(cdiv(count, 4), 256);
    const int64_t rgrid = blocks < int64_t(cus) * 8 ? (blocks > 0 ? blocks : 1) : int64_t(cus) * 8;
    int64_t stride_arg = stride;
    int64_t count_arg = count;
    int32_t splits_arg = eff;
    const float *w_arg = W;
    uint16_t *c_arg = static_cast<uint16_t *>(C);
    void *args[] = {&w_arg, &splits_arg, &stride_arg, &count_arg, &c_arg};
    const void *reduce = nt_partials(eff, M, N)
                             ? reinterpret_cast<const void *>(&splitk_reduce_kernel<true>)
                             : reinterpret_cast<const void *>(&splitk_reduce_kernel<false>);
    const hipError_t err = hipLaunchKernel(reduce,
                                           dim3(static_cast<uint32_t>(rgrid)), dim3(256), args, 0,
                                           stream);
    return err == hipSuccess ? GEMM_F16_OK : GEMM_F16_LAUNCH_FAILED;
}

// ---------------------------------------------------------------------------
// Split over K without allocation: the fp32 partials in a fixed array
// ---------------------------------------------------------------------------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid it), the partials of
// gemm_f16_nt_splitk_noalloc live in this file-scope device array.  Each GPU
// the library runs on holds its own copy, at its own address, for as long as
// the process lives.  In host code `scratch` names a host-side stand-in, not
// device memory: kernels get the device address that hipGetSymbolAddress
// returns for the current device, fetched once per device.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

struct ScratchInfo {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
static ScratchInfo g_scratch[kMaxDevices];

// The current device's copy of `scratch` (with that device current).
static int scratch_address(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMM_F16_LAUNCH_FAILED;
    ScratchInfo &d = g_scratch[dev];
    std::call_once(d.once, [&] {
        void *q = nullptr;
        d.err = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        d.ptr = q;
    });
    if (d.err != hipSuccess || !d.ptr) return GEMM_F16_LAUNCH_FAILED;
    *out = d.ptr;
    return GEMM_F16_OK;
}

// ---------------------------------------------------------------------------
// Autotuning: every configuration of a layout, with and without a split over K
// ---------------------------------------------------------------------------
// Requested split counts tried per configuration; each maps to an effective
// count (ranges of whole K slices) and repeated effective counts are dropped.
constexpr int32_t kTuneSplits[] = {2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
constexpr int64_t kTuneMinSplitK = 256;   // K per range the tuner goes down to
constexpr int64_t kStreamTuneMaxM = 64;   // M up to which the streaming kernel is tried

// The (configuration, split) pairs the tuner times for these arguments, in
// configuration order, each configuration's unsplit run first.  Splits are
// tried only while the unsplit grid would fill fewer than 4 rounds, up to 16
// rounds of units, and only where their partials fit `workspace_bytes`
// (*needed: the largest workspace any split candidate would use).  `fast`:
// the arguments suit the layout's direct-to-LDS configurations; otherwise
// only its general kernel is a candidate.
static void tune_candidates(int32_t layout, int64_t M, int64_t N, int64_t K, int32_t cus,
                            bool fast, int64_t workspace_bytes,
                            std::vector<gemm_f16_tune_entry_t> &out, int64_t *needed)
{
    out.clear();
    *needed = 0;
    const int64_t stride_bytes = split_stride(M, N) * 4;
    for (int id = 0; id < kNumKernels; ++id) {
        const KernelEntry &e = kKernels[id];
        if (e.layout != layout || (!fast && !e.general)) continue;
        // the register-streaming kernel re-reads B for every 16 rows of A
        if (e.stages == 0 && M > kStreamTuneMaxM) continue;
        out.push_back(gemm_f16_tune_entry_t{id, 1, GEMM_F16_OK, -1.0f});
        if (e.general || !e.fn_split || K <= 0) continue;
        const int64_t tiles = cdiv(M, e.block_m) * cdiv(N, e.block_n);
        if (tiles >= 4 * int64_t(cus)) continue;
        int64_t last = 1;
        for (int32_t sp : kTuneSplits) {
            if (cdiv(K, sp) < kTuneMinSplitK) break;
            const int64_t eff = cdiv(K, split_k_len(id, K, sp));
            if (eff <= last) continue;
            last = eff;
            if (tiles * eff > 16 * int64_t(cus) || tiles * eff > INT32_MAX) break;
            const int64_t bytes = eff * stride_bytes;
            if (bytes > *needed) *needed = bytes;
            if (bytes <= workspace_bytes)
                out.push_back(gemm_f16_tune_entry_t{id, static_cast<int32_t>(eff), GEMM_F16_OK, -1.0f});
        }
    }
}

static bool fast_arguments(int32_t layout, int64_t M, int64_t N, int64_t K, const void *A,
                           const void *B, bool check_pointers)
{
    return layout == 0 ? !needs_general(K, A, B, check_pointers)
                       : layout_supported(layout, M, N, K, A, B, check_pointers);
}

// Times each candidate on the caller's buffers: one untimed call, then
// `iters` back-to-back calls between two events on `stream`.  Candidates that
// report GEMM_F16_UNSUPPORTED are recorded and skipped; any other failure
// ends the search with that status.  The fastest is run once more at the end
// so that C holds its result.
static int autotune(int32_t layout, int64_t M, int64_t N, int64_t K, const void *A,
                    const void *B, void *C, void *workspace, int64_t workspace_bytes,
                    int32_t iters, hipStream_t stream, gemm_f16_tune_entry_t *best,
                    gemm_f16_tune_entry_t *entries, int32_t max_entries, int32_t *n_entries)
{
    if (layout < 0 || layout > 3 || !best || iters < 1 || iters > 10000 || max_entries < 0 ||
        (max_entries > 0 && !entries) || workspace_bytes < 0 || (workspace_bytes > 0 && !workspace))
        return GEMM_F16_INVALID_ARG;
    const int v = validate(M, N, K, A, B, C);
    if (v != GEMM_F16_OK) return v;
    *best = gemm_f16_tune_entry_t{-1, 1, GEMM_F16_OK, 0.0f};
    if (n_entries) *n_entries = 0;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    if (K == 0) return run(M, N, 0, A, B, C, stream, -1, 0, 0, -1);   // nothing to choose
    int32_t cus = 0;
    const int s = current_cus(&cus);
    if (s != GEMM_F16_OK) return s;
    std::vector<gemm_f16_tune_entry_t> cand;
    int64_t needed = 0;
    tune_candidates(layout, M, N, K, cus, fast_arguments(layout, M, N, K, A, B, true),
                    workspace_bytes, cand, &needed);
    hipEvent_t ev[2] = {nullptr, nullptr};
    if (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess) {
        if (ev[0]) (void)hipEventDestroy(ev[0]);
        return GEMM_F16_LAUNCH_FAILED;
    }
    int status = GEMM_F16_OK;
    int best_i = -1;
    // The clock ramps up over the first ~50 ms of sustained work after idle:
    // run the first candidate that long before anything is timed, so that
    // the first candidates are not ranked on a cold clock.
    if (!cand.empty()) {
        float warm = 0.0f;
        for (int batch = 0; batch < 1000 && warm < 50.0f && status == GEMM_F16_OK; ++batch) {
            if (hipEventRecord(ev[0], stream) != hipSuccess) status = GEMM_F16_LAUNCH_FAILED;
            for (int32_t it = 0; it < iters && status == GEMM_F16_OK; ++it) {
                const int st = run_splitk(layout, M, N, K, A, B, C, cand[0].splits, workspace,
                                          workspace_bytes, stream, cand[0].config_id);
                if (st != GEMM_F16_OK) {
                    // the first candidate cannot run these arguments: no warm-up
                    if (st != GEMM_F16_UNSUPPORTED) status = st;
                    batch = 1000;
                    break;
                }
            }
            float ms = 0.0f;
            if (status == GEMM_F16_OK && batch < 1000 &&
                (hipEventRecord(ev[1], stream) != hipSuccess ||
                 hipEventSynchronize(ev[1]) != hipSuccess ||
                 hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess))
                status = GEMM_F16_LAUNCH_FAILED;
            warm += ms;
        }
    }
    for (size_t i = 0; i < cand.size() && status == GEMM_F16_OK; ++i) {
        gemm_f16_tune_entry_t &c = cand[i];
        auto call = [&] {
            return run_splitk(layout, M, N, K, A, B, C, c.splits, workspace, workspace_bytes,
                              stream, c.config_id);
        };
        c.status = call();
        if (c.status == GEMM_F16_OK && hipEventRecord(ev[0], stream) != hipSuccess)
            c.status = GEMM_F16_LAUNCH_FAILED;
        for (int32_t it = 0; it < iters && c.status == GEMM_F16_OK; ++it) c.status = call();
        if (c.status == GEMM_F16_OK) {
            float ms = 0.0f;
            if (hipEventRecord(ev[1], stream) != hipSuccess || hipEventSynchronize(ev[1]) != hipSuccess ||
                hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess)
                c.status = GEMM_F16_LAUNCH_FAILED;
            c.ms = ms / iters;
        }
        if (c.status == GEMM_F16_OK) {
            if (best_i < 0 || c.ms < cand[best_i].ms) best_i = static_cast<int>(i);
        } else if (c.status != GEMM_F16_UNSUPPORTED) {
            status = c.status;
        }
    }
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    const size_t n = cand.size() < size_t(max_entries) ? cand.size() : size_t(max_entries);
    for (size_t i = 0; i < n; ++i) entries[i] = cand[i];
    if (n_entries) *n_entries = static_cast<int32_t>(cand.size());
    if (status != GEMM_F16_OK) return status;
    if (best_i < 0) return GEMM_F16_UNSUPPORTED;
    *best = cand[best_i];
    return run_splitk(layout, M, N, K, A, B, C, best->splits, workspace, workspace_bytes, stream,
                      best->config_id);
}

}  // namespace gemm_f16

using namespace gemm_f16;

extern "C" int gemm_f16_nt(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                           void *C, hipStream_t stream)
{
    return run(M, N, K, A, B, C, stream, -1, 0, 0, -1);
}

extern "C" int gemm_f16_nt_with_config(int64_t M, int64_t N, int64_t K, const void *A,
                                       const void *B, void *C, hipStream_t stream,
                                       int32_t config_id, int32_t swizzle, int32_t grid,
                                       int32_t epilogue)
{
    return run(M, N, K, A, B, C, stream, config_id < 0 ? -1 : config_id, swizzle, grid,
               epilogue);
}

extern "C" const char *gemm_f16_nt_status_string(int status)
{
    switch (status) {
    case GEMM_F16_OK: return "ok";
    case GEMM_F16_INVALID_ARG: return "invalid argument";
    case GEMM_F16_UNSUPPORTED: return "unsupported argument";
    case GEMM_F16_LAUNCH_FAILED: return "HIP launch failed";
    case GEMM_F16_SCRATCH_LIMIT:
        return "the planned split-K partials exceed the no-allocation scratch (64 MiB)";
    default: return "unknown status";
    }
}

extern "C" int gemm_f16_nt_validate(int64_t M, int64_t N, int64_t K, const void *A,
                                    const void *B, const void *C)
{
    return validate(M, N, K, A, B, C);
}

extern "C" int gemm_f16_nt_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                                gemm_f16_nt_plan_t *plan)
{
    if (!plan || M < 0 || N < 0 || K < 0 || num_cus <= 0) return GEMM_F16_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || cdiv(M, 64) * cdiv(N, 64) > INT32_MAX)
        return GEMM_F16_UNSUPPORTED;
    const int id = needs_general(K, nullptr, nullptr, false) ? kGeneralConfig
                                                              : choose_config(M, N, K, num_cus);
    make_plan(id, M, N, num_cus, 0, 0, plan);
    return GEMM_F16_OK;
}

extern "C" int gemm_f16_nn(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                           void *C, hipStream_t stream)
{
    return run_layout(1, M, N, K, A, B, C, stream, -1, 0, 0, -1);
}

extern "C" int gemm_f16_nn_with_config(int64_t M, int64_t N, int64_t K, const void *A,
                                       const void *B, void *C, hipStream_t stream,
                                       int32_t config_id, int32_t swizzle, int32_t grid,
                                       int32_t epilogue)
{
    return run_layout(1, M, N, K, A, B, C, stream, config_id < 0 ? -1 : config_id, swizzle,
                      grid, epilogue);
}

extern "C" int gemm_f16_nn_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                                gemm_f16_nt_plan_t *plan)
{
    return plan_layout(1, M, N, K, num_cus, plan);
}

extern "C" int gemm_f16_tt(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                           void *C, hipStream_t stream)
{
    return run_layout(2, M, N, K, A, B, C, stream, -1, 0, 0, -1);
}

extern "C" int gemm_f16_tt_with_config(int64_t M, int64_t N, int64_t K, const void *A,
                                       const void *B, void *C, hipStream_t stream,
                                       int32_t config_id, int32_t swizzle, int32_t grid,
                                       int32_t epilogue)
{
    return run_layout(2, M, N, K, A, B, C, stream, config_id < 0 ? -1 : config_id, swizzle,
                      grid, epilogue);
}

extern "C" int gemm_f16_tt_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                                gemm_f16_nt_plan_t *plan)
{
    return plan_layout(2, M, N, K, num_cus, plan);
}

extern "C" int gemm_f16_tn(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                           void *C, hipStream_t stream)
{
    return run_layout(3, M, N, K, A, B, C, stream, -1, 0, 0, -1);
}

extern "C" int gemm_f16_tn_with_config(int64_t M, int64_t N, int64_t K, const void *A,
                                       const void *B, void *C, hipStream_t stream,
                                       int32_t config_id, int32_t swizzle, int32_t grid,
                                       int32_t epilogue)
{
    return run_layout(3, M, N, K, A, B, C, stream, config_id < 0 ? -1 : config_id, swizzle,
                      grid, epilogue);
}

extern "C" int gemm_f16_tn_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                                gemm_f16_nt_plan_t *plan)
{
    return plan_layout(3, M, N, K, num_cus, plan);
}

static int splitk_plan(int32_t layout, int64_t M, int64_t N, int64_t K, int32_t num_cus,
                       int32_t splits, gemm_f16_nt_plan_t *plan, int32_t *splits_out,
                       int64_t *workspace_bytes)
{
    if (!plan || !splits_out || !workspace_bytes || M < 0 || N < 0 || K < 0 || num_cus <= 0 ||
        splits > kMaxSplits)
        return GEMM_F16_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || cdiv(M, 64) * cdiv(N, 64) > INT32_MAX)
        return GEMM_F16_UNSUPPORTED;
    *splits_out = 1;
    *workspace_bytes = 0;
    if (K == 0 || M == 0 || N == 0) return gemm_f16_nt_plan(M, N, K, num_cus, plan);
    if (layout == 0 && needs_general(K, nullptr, nullptr, false))
        return gemm_f16_nt_plan(M, N, K, num_cus, plan);
    if (layout != 0 && !layout_supported(layout, M, N, K, nullptr, nullptr, false))
        return plan_layout(layout, M, N, K, num_cus, plan);   // the general kernel, no split
    int id = -1;
    int32_t eff = 1;
    choose_split(M, N, K, num_cus, -1, splits, &id, &eff, layout);
    make_plan(id, M, N, num_cus, 0, 0, plan);
    if (eff > 1) {
        if (plan->tiles * eff > INT32_MAX) return GEMM_F16_UNSUPPORTED;
        const int64_t units = plan->tiles * eff;
        const int64_t cap = int64_t(num_cus) * kKernels[id].per_cu;
        plan->grid = static_cast<int32_t>(units < cap ? units : cap);
        plan->epilogue = 0;
        *splits_out = eff;
        *workspace_bytes = eff * split_stride(M, N) * 4;
    }
    return GEMM_F16_OK;
}

extern "C" int gemm_f16_device_cus(int32_t *cus)
{
    if (!cus) return GEMM_F16_INVALID_ARG;
    return current_cus(cus);
}

extern "C" int gemm_f16_splitk_workspace_bytes(int64_t M, int64_t N, int32_t splits,
                                               int64_t *workspace_bytes)
{
    if (!workspace_bytes || M < 0 || N < 0 || splits < 0 || splits > kMaxSplits)
        return GEMM_F16_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX) return GEMM_F16_UNSUPPORTED;
    *workspace_bytes = splits > 1 ? int64_t(splits) * split_stride(M, N) * 4 : 0;
    return GEMM_F16_OK;
}

extern "C" int gemm_f16_nt_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                                       int32_t splits, gemm_f16_nt_plan_t *plan,
                                       int32_t *splits_out, int64_t *workspace_bytes)
{
    return splitk_plan(0, M, N, K, num_cus, splits, plan, splits_out, workspace_bytes);
}

extern "C" int gemm_f16_nt_splitk(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                                  void *C, int32_t splits, void *workspace,
                                  int64_t workspace_bytes, hipStream_t stream)
{
    return run_splitk(0, M, N, K, A, B, C, splits, workspace, workspace_bytes, stream, -1);
}

extern "C" int gemm_f16_nt_splitk_with_config(int64_t M, int64_t N, int64_t K, const void *A,
                                              const void *B, void *C, int32_t splits,
                                              void *workspace, int64_t workspace_bytes,
                                              hipStream_t stream, int32_t config_id)
{
    return run_splitk(0, M, N, K, A, B, C, splits, workspace, workspace_bytes, stream,
                      config_id < 0 ? -1 : config_id);
}

extern "C" int gemm_f16_nt_splitk_noalloc(int64_t M, int64_t N, int64_t K, const void *A,
                                          const void *B, void *C, int32_t splits,
                                          hipStream_t stream)
{
    // argument errors first, before the device is touched
    const int v = validate(M, N, K, A, B, C);
    if (v != GEMM_F16_OK) return v;
    if (splits > kMaxSplits) return GEMM_F16_INVALID_ARG;
    void *ws = nullptr;
    const int s = scratch_address(&ws);
    if (s != GEMM_F16_OK) return s;
    return run_splitk(0, M, N, K, A, B, C, splits, ws, kScratchBytes, stream, -1, true);
}

extern "C" int gemm_f16_nn_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                                       int32_t splits, gemm_f16_nt_plan_t *plan,
                                       int32_t *splits_out, int64_t *workspace_bytes)
{
    return splitk_plan(1, M, N, K, num_cus, splits, plan, splits_out, workspace_bytes);
}

extern "C" int gemm_f16_nn_splitk(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                                  void *C, int32_t splits, void *workspace,
                                  int64_t workspace_bytes, hipStream_t stream)
{
    return run_splitk(1, M, N, K, A, B, C, splits, workspace, workspace_bytes, stream, -1);
}

extern "C" int gemm_f16_nn_splitk_with_config(int64_t M, int64_t N, int64_t K, const void *A,
                                              const void *B, void *C, int32_t splits,
                                              void *workspace, int64_t workspace_bytes,
                                              hipStream_t stream, int32_t config_id)
{
    return run_splitk(1, M, N, K, A, B, C, splits, workspace, workspace_bytes, stream,
                      config_id < 0 ? -1 : config_id);
}

extern "C" int gemm_f16_tt_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                                       int32_t splits, gemm_f16_nt_plan_t *plan,
                                       int32_t *splits_out, int64_t *workspace_bytes)
{
    return splitk_plan(2, M, N, K, num_cus, splits, plan, splits_out, workspace_bytes);
}

extern "C" int gemm_f16_tt_splitk(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                                  void *C, int32_t splits, void *workspace,
                                  int64_t workspace_bytes, hipStream_t stream)
{
    return run_splitk(2, M, N, K, A, B, C, splits, workspace, workspace_bytes, stream, -1);
}

extern "C" int gemm_f16_tt_splitk_with_config(int64_t M, int64_t N, int64_t K, const void *A,
                                              const void *B, void *C, int32_t splits,
                                              void *workspace, int64_t workspace_bytes,
                                              hipStream_t stream, int32_t config_id)
{
    return run_splitk(2, M, N, K, A, B, C, splits, workspace, workspace_bytes, stream,
                      config_id < 0 ? -1 : config_id);
}

extern "C" int gemm_f16_tn_splitk_plan(int64_t M, int64_t N, int64_t K, int32_t num_cus,
                                       int32_t splits, gemm_f16_nt_plan_t *plan,
                                       int32_t *splits_out, int64_t *workspace_bytes)
{
    return splitk_plan(3, M, N, K, num_cus, splits, plan, splits_out, workspace_bytes);
}

extern "C" int gemm_f16_tn_splitk(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                                  void *C, int32_t splits, void *workspace,
                                  int64_t workspace_bytes, hipStream_t stream)
{
    return run_splitk(3, M, N, K, A, B, C, splits, workspace, workspace_bytes, stream, -1);
}

extern "C" int gemm_f16_tn_splitk_with_config(int64_t M, int64_t N, int64_t K, const void *A,
                                              const void *B, void *C, int32_t splits,
                                              void *workspace, int64_t workspace_bytes,
                                              hipStream_t stream, int32_t config_id)
{
    return run_splitk(3, M, N, K, A, B, C, splits, workspace, workspace_bytes, stream,
                      config_id < 0 ? -1 : config_id);
}

extern "C" int gemm_f16_nt_num_configs(void) { return kNumKernels; }

extern "C" int gemm_f16_nt_config_info(int32_t config_id, gemm_f16_nt_plan_t *info)
{
    if (!info || config_id < 0 || config_id >= kNumKernels) return GEMM_F16_INVALID_ARG;
    fill_info(config_id, info);
    return GEMM_F16_OK;
}

extern "C" int gemm_f16_nt_tile_of_slot(const gemm_f16_nt_plan_t *plan, int64_t slot,
                                        int32_t *tile_m, int32_t *tile_n)
{
    if (!plan || !tile_m || !tile_n || slot < 0 || slot >= plan->tiles || plan->grid <= 0 ||
        plan->swizzle <= 0)
        return GEMM_F16_INVALID_ARG;
    int32_t tm, tn;
    grouped_tile(slot_to_linear(static_cast<int32_t>(slot), plan->grid,
                                static_cast<int32_t>(plan->tiles), plan->xcds),
                 plan->tiles_m, plan->tiles_n, plan->swizzle, tm, tn);
    *tile_m = tm;
    *tile_n = tn;
    return GEMM_F16_OK;
}

extern "C" int gemm_f16_autotune_candidates(int32_t layout, int64_t M, int64_t N, int64_t K,
                                            int32_t num_cus, int32_t aligned,
                                            int64_t workspace_bytes,
                                            gemm_f16_tune_entry_t *entries, int32_t max_entries,
                                            int32_t *n_entries, int64_t *workspace_needed)
{
    if (layout < 0 || layout > 3 || M < 0 || N < 0 || K < 0 || num_cus <= 0 ||
        workspace_bytes < 0 || max_entries < 0 || (max_entries > 0 && !entries) || !n_entries ||
        !workspace_needed)
        return GEMM_F16_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || cdiv(M, 64) * cdiv(N, 64) > INT32_MAX)
        return GEMM_F16_UNSUPPORTED;
    *n_entries = 0;
    *workspace_needed = 0;
    if (M == 0 || N == 0 || K == 0) return GEMM_F16_OK;
    std::vector<gemm_f16_tune_entry_t> cand;
    const bool fast = fast_arguments(layout, M, N, K, nullptr, nullptr, false) && aligned;
    tune_candidates(layout, M, N, K, num_cus, fast, workspace_bytes, cand, workspace_needed);
    const size_t n = cand.size() < size_t(max_entries) ? cand.size() : size_t(max_entries);
    for (size_t i = 0; i < n; ++i) entries[i] = cand[i];
    *n_entries = static_cast<int32_t>(cand.size());
    return GEMM_F16_OK;
}

extern "C" int gemm_f16_autotune(int32_t layout, int64_t M, int64_t N, int64_t K, const void *A,
                                 const void *B, void *C, void *workspace,
                                 int64_t workspace_bytes, int32_t iters, hipStream_t stream,
                                 gemm_f16_tune_entry_t *best, gemm_f16_tune_entry_t *entries,
                                 int32_t max_entries, int32_t *n_entries)
{
    return autotune(layout, M, N, K, A, B, C, workspace, workspace_bytes, iters, stream, best,
                    entries, max_entries, n_entries);
}
