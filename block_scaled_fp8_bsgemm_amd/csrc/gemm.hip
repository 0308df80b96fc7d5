// gemm.hip -- block-scale fp8 GEMM with a destination-major band epilogue
// for gfx950 (MI355X).
//
// Computes C = A * B^T for A [M,K] e4m3 with one fp32 scale per 1x128 block
// and B [N,K] e4m3 with one fp32 scale per 128x128 block, accumulating in
// fp32 and writing bf16 ("MORI GEMM + All-Reduce Benchmark", "Running the
// benchmark", --quant blockscale; sglang PR 40757, "What").  Each 128-deep K
// block of a 16x16 output sub-tile is one v_mfma_f32_16x16x128_f8f6f4 into a
// zeroed fp32 temporary; its result is folded into the running accumulator
// with one fma by the block's combined scale a_scale[m,kb] * b_scale[n/128,kb],
// K blocks in ascending order.  The epilogue writes each output row straight
// into its destination's row band (sglang PR 40757, "What": the GEMM writes
// each destination's row band as its own unit).
//
// Tiling (one workgroup = 8 waves = 512 lanes, one 256x256 output tile):
//  - per K block the A tile [256 x 128 B] and B tile [256 x 128 B] are staged
//    in LDS, double buffered (2 x 64 KiB); rows are placed in even / odd
//    128-byte slots and 16-byte chunks XOR-swizzled (swz) so that every MFMA
//    operand read is served without bank conflicts;
//  - global loads use buffer descriptors that end where the matrix ends, so
//    rows past M (a ragged last tile) read as zero without any branch;
//  - waves form a 2 (M) x 4 (N) grid of 128 x 64 wave tiles (8 x 4 MFMA
//    sub-tiles, 128 fp32 accumulator registers per lane);
//  - the MFMA takes the B fragment as its first operand, so each lane ends up
//    holding 4 consecutive output columns of one output row: one combined
//    scale per lane per sub-tile row;
//  - the K block's a_scale values of the tile's 256 rows and its b_scale
//    values are DMA'd into LDS with the operands; each wave forms its rows'
//    combined scales a_scale * b_scale in registers;
//  - at the end each wave stores its 128 x 64 bf16 sub-tile straight from
//    the accumulators as whole 128-byte row segments of the destination
//    band, eight rows per instruction (B's rows are staged in an order that
//    makes this possible; non-temporal stores in the blockscale kernels);
//  - workgroup -> tile mapping is XCD-aware: workgroups are dealt to the 8
//    XCDs round-robin, so each XCD is given a contiguous run of tiles, ordered
//    in groups of 4 M-tiles so that concurrently running tiles share A and B
//    panels in that XCD's L2 (its 32 concurrent tiles span 4 M-tiles x 8
//    N-tiles; measured faster than 8 x 4, 2 x 16 or 1 x 32).
//
// When K / 128 is even (the benchmark's K = 2048) and each operand stays
// under 2^31 bytes, the blockscale and mxfp8 GEMMs run as persistent kernels
// instead: one workgroup per CU walks several tiles, so the workgroup launch
// is not paid per tile, a tile's last K block already loads the next tile's
// first, and a finished tile's stores drain under the next tile's first K
// block (in the blockscale one, half of them go out between its MFMAs).
// Results are bit-identical to the tile kernels'.
//
// A second blockscale kernel reads B in a prepacked form (the same bytes in the
// MFMA's operand order, written once by bprepack_kernel) straight into
// registers instead of staging it in LDS; its results are bit-identical.
//
// The same tile kernel is also built for the mxfp8 variant (sglang PR 43480,
// "What" and "Not in this PR": e4m3 operands with one E8M0 scale byte per
// 1x32 block of A's and B's rows): there the scales are applied by the scaled
// MFMA v_mfma_scale_f32_16x16x128_f8f6f4 itself, the MFMAs accumulate
// directly, and the stage's scale piece carries the tile rows' scale bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "codec.hpp"
#include "launch.hpp"

namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int NTHREADS = 512;
constexpr int WM = 128, WN = 64;        // wave tile
constexpr int TM = WM / 16, TN = WN / 16;
constexpr int GROUP_M = 4;
constexpr int NUM_XCD = 8;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct GemmArgs {
    const uint8_t *A;
    const void *sa;         // blockscale: fp32 [M, K/128]; mxfp8: E8M0 bytes [M, K/32]
    const uint8_t *B;
    const void *sb;         // blockscale: fp32 [N/128, K/128]; mxfp8: E8M0 bytes [N, K/32]
    uint16_t *C;
    int64_t M, N, K;
    int64_t band_rows, band_stride;
    int KB;                 // K / 128
    int NB;                 // N / 128
    int tiles_m, tiles_n;
};

// The two pipeline stages are distinct LDS objects so that the compiler can
// tell a DMA into one stage from reads of the other and does not serialise
// them with a wait.
__shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * BK];
__shared__ __attribute__((aligned(1024))) uint8_t sA1[BM * BK];
__shared__ __attribute__((aligned(1024))) uint8_t sB0[BN * BK];
__shared__ __attribute__((aligned(1024))) uint8_t sB1[BN * BK];
// scales per stage, one dword per entry: blockscale: [0, 256) a_scale of the
// tile's rows (in the order of sa_row); [256, 512) four 64-entry slots filled by waves 4..7 with
// b_scale, of which entries 256 and 257 (the tile's two 128-column blocks) are
// read.  mxfp8: [0, 256) the K block's 4 E8M0 bytes of each A row, [256, 512)
// those of each B row.
constexpr int SCALES = BM + 256;
__shared__ __attribute__((aligned(1024))) float sS0[SCALES];
__shared__ __attribute__((aligned(1024))) float sS1[SCALES];

template <int ST> __device__ __forceinline__ uint8_t *stA() { return ST ? sA1 : sA0; }
template <int ST> __device__ __forceinline__ uint8_t *stB() { return ST ? sB1 : sB0; }
template <int ST> __device__ __forceinline__ float *stS() { return ST ? sS1 : sS0; }


// Byte offset of 16-byte chunk `c` (0..7) of tile row `r` inside a staged
// [rows x 128 B] operand tile.  An MFMA fragment read (ds_read_b128) has each
// 16-lane quarter read one chunk of 16 consecutive rows.  Within every 16-row
// group, rows 0-7 go to the even 128-byte slots and rows 8-15 to the odd
// ones, and chunks are XOR-swizzled by the row's low three bits: lanes 0-7 of
// a quarter then read banks 0-31 and lanes 8-15 banks 32-63, each half
// without conflicts, each lane from a different slot row.  Measured, this
// reads at the LDS's full rate; the plain row-major XOR swizzle, which also
// puts the 16 lanes in 64 distinct banks, reads at about half of it.
__device__ __forceinline__ int lds_slot(int r) { return (r & ~15) | ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return lds_slot(r) * 128 + ((c ^ (r & 7)) << 4); }

// B's rows are staged in a permuted order so that the epilogue can store C
// straight from the accumulators.  Each wave's 64 output columns are four
// 16-column MFMA sub-tiles j, and the MFMA leaves lane l with 4 consecutive
// columns 4 (l/16) .. +4 of its sub-tile.  If sub-tile j's fragment row r is
// B row brow_j(r) = 32 (j/2) + 8 (r/4) + 4 (j%2) + r%4 of the wave's 64, then
// lane l's columns of sub-tiles 0 and 1 are the 8 consecutive columns
// 8 (l/16) .. +8 and those of sub-tiles 2 and 3 the 8 at 32 + 8 (l/16): two
// 16-byte stores per lane and row group.  brow_of(R) applies this to LDS row
// R = 64 w + 16 j + r of the staged B tile; it is a permutation within each
// 64-row group, so each wave's columns still lie in one 128-column b_scale
// block.
__device__ __forceinline__ int brow_of(int R) {
    const int j = (R >> 4) & 3, r = R & 15;
    return (R & ~63) + 32 * (j >> 1) + 8 * (r >> 2) + 4 * (j & 1) + (r & 3);
}

// Every descriptor here is workgroup-uniform; readfirstlane says so to the
// compiler, which otherwise may keep one in VGPRs and wrap each load through
// it in a loop over distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    int32_t n = bytes > 0x7FFFFFFFll ? 0x7FFFFFFF : (bytes > 0 ? (int32_t)bytes : 0);
    const uint64_t b = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    n = __builtin_amdgcn_readfirstlane(n);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, n,
                                             0x00020000);
}

// A tile's operand descriptors: its row panels of A and B, and its scales.
struct Panels {
    __amdgpu_buffer_rsrc_t rA, rB, rS;   // rS: a_scale (waves 0..3) or b_scale (4..7)
};

struct Loader {
    Panels P;                            // the current tile's
    __amdgpu_buffer_rsrc_t rZ;           // zero-size: every load through it reads nothing
    int poff;    // prepacked B: this lane's byte offset in its wave's first fragment
    int pstep;   // prepacked B: bytes from one 16-row group to the next (K/128 * 2 KiB)
    int voff;    // this lane's byte offset of its chunk in the A row panel (even slots i)
    int voff1;   // the same for odd slots i (the lane's chunk with bit 2 flipped)
    int voffB;   // the same two for the B panel, whose rows are fetched in the
    int voffB1;  //   permuted order of brow_of (see there)
    int k4;      // 4 rows of a panel, in bytes
    int soff;    // this lane's byte offset of its scale (a_scale row, or b_scale block)
    int ldsq;    // byte offset of this wave's first 1 KiB LDS slot
    int sdst;    // byte offset of this wave's 256-byte scale slot
};

// A tile's byte offsets in A, in B and in this wave's scales, or the change
// of them from one tile to another (persistent kernels).
struct TileOff {
    int a, b, s;
};

// One DMA instruction of a stage load: pieces 0..7 are the A and B slots
// i = piece / 2 (A for even pieces, B for odd), piece 8 the scales.  A block
// past the end (valid == false) goes through the zero-size descriptor: the
// loads touch no memory and the stage is not read again.  d moves the
// lanes' offsets to another tile of the same whole-matrix descriptors.
template <int ST, int PIECE>
__device__ __forceinline__ void dma_piece(const Loader &L, const Panels &P, int kb, bool valid,
                                          const TileOff &d = TileOff{0, 0, 0}) {
    const int koff = kb * BK;
    if (PIECE < 8) {
        const int i = PIECE >> 1;
        const int q = L.ldsq + i * 1024;
        if (PIECE & 1) {
            // B: slot i's global rows are those of slot 0 plus 0, 8, 4, 12
            const int vo = ((i & 1) ? L.voffB1 : L.voffB) + (2 * (i & 1) + (i >> 1)) * L.k4 + d.b;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(valid ? P.rB : L.rZ, (lds_void *)(stB<ST>() + q),
                                                     16, vo, koff, 0, 0);
        } else {
            // A: slot i's rows are those of slot 0 plus 0, 4, 16, 20 (see load_stage)
            const int vo = ((i & 1) ? L.voff1 : L.voff) + (4 * (i >> 1) + (i & 1)) * L.k4 + d.a;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(valid ? P.rA : L.rZ, (lds_void *)(stA<ST>() + q),
                                                     16, vo, koff, 0, 0);
        }
    } else {
        // blockscale: waves 0..3 fetch a_scale of rows 64w..64w+63, waves
        // 4..7 b_scale of the column blocks from the tile's first one on;
        // mxfp8: waves 0..3 fetch the 4 scale bytes of the K block for A rows
        // 64w.., waves 4..7 for B rows 64(w-4)..  Each wave fills its own
        // 256-byte slot; no branch: every wave issues exactly one.
        __builtin_amdgcn_raw_ptr_buffer_load_lds(valid ? P.rS : L.rZ,
                                                 (lds_void *)((uint8_t *)stS<ST>() + L.sdst), 4,
                                                 L.soff + d.s, kb * 4, 0, 0);
    }
}

// DMA the K block kb of the A and B panels and of the scales into stage ST.
// One buffer_load ... lds writes 64 lanes x 16 B = 1 KiB of LDS in lane order:
// eight 128-byte row slots, lane l on slot l/8 at physical chunk l%8.  Wave w's
// slot i (0..3) covers LDS slots 32w + 8i .. 32w + 8i + 7, which hold tile rows
// 32w + {0, 4, 16, 20}[i] + (l/16) + 8 * ((l/8) % 2) (lds_slot inverted), so
// every instruction still fetches eight whole 128-byte row segments; the lane
// fetches logical chunk (l%8) ^ (row & 7) of its row, which realises the
// swizzle.  B's LDS row R holds the tile's B row brow_of(R) (a permutation
// within each 64-row group), so slot i of wave w fetches B rows 32w + {0, 8,
// 4, 12}[i] + (l/16) + 16 * ((l/8) % 2).
template <int ST>
__device__ __forceinline__ void load_stage(const Loader &L, int kb, bool valid = true) {
    dma_piece<ST, 0>(L, L.P, kb, valid); dma_piece<ST, 1>(L, L.P, kb, valid);
    dma_piece<ST, 2>(L, L.P, kb, valid); dma_piece<ST, 3>(L, L.P, kb, valid);
    dma_piece<ST, 4>(L, L.P, kb, valid); dma_piece<ST, 5>(L, L.P, kb, valid);
    dma_piece<ST, 6>(L, L.P, kb, valid); dma_piece<ST, 7>(L, L.P, kb, valid);
    dma_piece<ST, 8>(L, L.P, kb, valid);
}

// One MFMA operand fragment: lane l's 32 bytes of a 16-row fragment are row
// r's 16-byte chunks g and g + 4 (g = l / 16), i.e. K [16g, 16g+16) and
// [64+16g, 64+16g+16) of the 128-deep block.  The 16x16x128 fp8 MFMA adds its
// products into the fp32 result in 16-slot passes taken from the bytes 0-15
// of lane groups 0..3 first, then from their bytes 16-31 (measured on the
// device, with and without scales); with this placement the passes cover K
// in ascending order, 16 at a time.  The scaled MFMA takes the lane's scale
// byte for K group g, which this placement also satisfies.
__device__ __forceinline__ v8i lds_frag(const uint8_t *st, int r, int g) {
    const u32x4 lo = *(const u32x4 *)(st + swz(r, g));
    const u32x4 hi = *(const u32x4 *)(st + swz(r, g + 4));
    return (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ void fold4(v4f &acc, const v4f &p, float s) {
#pragma unroll
    for (int e = 0; e < 4; e++) acc[e] = __builtin_fmaf(p[e], s, acc[e]);
}

// A workgroup barrier that leaves vector memory operations in flight:
// __syncthreads() also fences global memory, which makes the compiler wait
// for every outstanding store before it.  The caller waits for what the
// barrier must cover (its DMA) with its own s_waitcnt; the LDS reads issued
// before are waited for here, and the empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_lds_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_dma_and_sync() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMAs have landed
    __syncthreads();                     // ... and every other wave's; LDS reads are done
}

// The scales of one K block for this wave's rows: a_scale of its 8 row
// groups (lane row m = 16 i + lane % 16 of the wave tile) and b_scale of its
// column block; their products are the combined scales s[i].
struct RawScales {
    float sa[TM];
    float sb;
};

// The a_scale slots hold the tile's 256 rows so that a lane's 8 values
// (row 128 wm + 16 i + frow, i = 0..7; q = 16 wm + frow) are two 16-byte
// pieces, i = 0..3 at slot 4 q and i = 4..7 at slot 128 + 4 q: two reads
// instead of eight, and consecutive lanes read consecutive 16-byte pieces
// (no bank conflicts).  Slot p holds row sa_row(p).
__device__ __forceinline__ int sa_row(int p) {
    const int q = (p >> 2) & 31, i = ((p >> 7) << 2) | (p & 3);
    return (q >> 4) * WM + i * 16 + (q & 15);
}

// The mxfp8 scale slots (4 bytes each: a row's scale bytes of the K block)
// hold the tile's 256 A rows, then its 256 B rows, so that the 8 A rows of a
// lane (row 128 wm + 16 i + frow, i = 0..7) sit in 8 consecutive slots, and
// so do its 4 B rows (the B rows of LDS rows 64 wn + 16 j + frow, j = 0..3):
// three 16-byte reads instead of twelve byte reads.  Slot p (waves 0..3 fill
// 0..255, waves 4..7 256..511) holds tile row mx_scale_row(p) of A or B.
__device__ __forceinline__ int mx_scale_row(int p) {
    if (p < BM) return (p & 128) | ((p & 7) << 4) | ((p >> 3) & 15);
    const int q = p - BM;
    return brow_of((q & ~63) | ((q & 3) << 4) | ((q >> 2) & 15));
}

template <int ST>
__device__ __forceinline__ void read_scales(RawScales &r, int wm, int wn, int frow) {
    const float *sc = stS<ST>();
    // this wave's 64 columns lie inside one 128-column b_scale block
    r.sb = sc[BM + (wn >> 1)];   // wave 4's slot: entries BM, BM+1
    typedef float v4s __attribute__((ext_vector_type(4)));
    const v4s *q = (const v4s *)sc + (wm * 16 + frow);
    const v4s lo = q[0], hi = q[32];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        r.sa[i] = lo[i];
        r.sa[4 + i] = hi[i];
    }
}

__device__ __forceinline__ void combine_scales(float (&s)[TM], const RawScales &r) {
#pragma unroll
    for (int i = 0; i < TM; i++) s[i] = r.sa[i] * r.sb;
}

// The first fragments of the K block in stage ST, in the order the first
// MFMAs use them (A row group 0, then B column groups 0..3), then the scales.
template <int ST>
__device__ __forceinline__ void read_head(v8i &a, v8i (&bf)[TN], float (&s)[TM], int wm, int wn,
                                          int frow, int fc) {
    a = lds_frag(stA<ST>(), wm * WM + frow, fc);
#pragma unroll
    for (int j = 0; j < TN; j++) bf[j] = lds_frag(stB<ST>(), wn * WN + j * 16 + frow, fc);
    RawScales r;
    read_scales<ST>(r, wm, wn, frow);
    combine_scales(s, r);
}

// ---- mxfp8 --------------------------------------------------------------
// The scaled MFMA takes lane l's 32 bytes of a 16-row fragment as the K
// values [16g, 16g+16) and [64+16g, 64+16g+16) of row l%16 (g = l/16), the
// placement lds_frag gives, and lane l's scale byte as the E8M0 scale of that
// row's 32-wide block g: byte g of the row's 4 scale bytes for the K block.
// The scale bytes are held four to a register: byte i % 4 of a[i / 4] for A
// row group i, byte j of b for B column group j.  The scaled MFMA's op_sel
// picks the byte (mx_mfma), so a wave holds 3 registers of scales, not 12.
struct MxScales {
    int a[TM / 4];   // A rows of the wave's 8 row groups
    int b;           // B rows of its 4 column groups
};

// byte g of each of the four dwords of v, packed (byte i from dword i)
__device__ __forceinline__ int byte_g4(const u32x4 &v, int g) {
    // v_perm selects bytes of {hi, lo}: selector byte k in 0..7 picks that
    // byte, 0x0C gives 0
    const uint32_t s01 = 0x0C0C0400u + (uint32_t)g * 0x0101u;            // bytes g, 4 + g
    const uint32_t s23 = 0x04000C0Cu + (uint32_t)g * 0x01010000u;        // bytes 2, 3
    const uint32_t t01 = __builtin_amdgcn_perm(v[1], v[0], s01);
    const uint32_t t23 = __builtin_amdgcn_perm(v[3], v[2], s23);
    return (int)(t01 | t23);
}

template <int ST>
__device__ __forceinline__ void read_mx_scales(MxScales &x, int wm, int wn, int frow, int g) {
    // the slots of the lane's 8 A rows and of its 4 B rows are contiguous
    // (mx_scale_row): 32 and 16 bytes, each dword a row's 4 group bytes
    const uint8_t *sc = (const uint8_t *)stS<ST>();
    const u32x4 a0 = *(const u32x4 *)(sc + (wm * WM + frow * 8) * 4);
    const u32x4 a1 = *(const u32x4 *)(sc + (wm * WM + frow * 8) * 4 + 16);
    const u32x4 b = *(const u32x4 *)(sc + (BM + wn * WN + frow * 4) * 4);
    x.a[0] = byte_g4(a0, g);
    x.a[1] = byte_g4(a1, g);
    x.b = byte_g4(b, g);
}

// The scaled MFMA of A row group i and B column group j (both compile-time
// after unrolling), each scale byte selected by op_sel.
template <int OB>
__device__ __forceinline__ v4f mx_mfma_j(const v8i &b, const v8i &a, const v4f &c, int sb, int sa, int i) {
    switch (i & 3) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, OB, sb, 0, sa);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, OB, sb, 1, sa);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, OB, sb, 2, sa);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, OB, sb, 3, sa);
    }
}
__device__ __forceinline__ v4f mx_mfma(const v8i &b, const v8i &a, const v4f &c, const MxScales &x, int i,
                                       int j) {
    const int sa = x.a[i >> 2];
    switch (j) {
    case 0: return mx_mfma_j<0>(b, a, c, x.b, sa, i);
    case 1: return mx_mfma_j<1>(b, a, c, x.b, sa, i);
    case 2: return mx_mfma_j<2>(b, a, c, x.b, sa, i);
    default: return mx_mfma_j<3>(b, a, c, x.b, sa, i);
    }
}

template <int ST>
__device__ __forceinline__ void read_head_mx(v8i &a, v8i (&bf)[TN], MxScales &x, int wm, int wn,
                                             int frow, int g) {
    a = lds_frag(stA<ST>(), wm * WM + frow, g);
#pragma unroll
    for (int j = 0; j < TN; j++) bf[j] = lds_frag(stB<ST>(), wn * WN + j * 16 + frow, g);
    read_mx_scales<ST>(x, wm, wn, frow, g);
}

// DMA of block kb + 1 into stage ST ^ 1 during the first nine MFMAs of block
// kb (see kblock); dma_block takes the block, its validity and the tile's
// panels explicitly.
template <int ST>
__device__ __forceinline__ void dma_block(const Loader &L, const Panels &P, int k, int kload, bool v,
                                          const TileOff &d = TileOff{0, 0, 0}) {
    if (k < 9) {
        if (k == 0) dma_piece<ST ^ 1, 8>(L, P, kload, v, d);
        if (k == 1) dma_piece<ST ^ 1, 0>(L, P, kload, v, d);
        if (k == 2) dma_piece<ST ^ 1, 1>(L, P, kload, v, d);
        if (k == 3) dma_piece<ST ^ 1, 2>(L, P, kload, v, d);
        if (k == 4) dma_piece<ST ^ 1, 3>(L, P, kload, v, d);
        if (k == 5) dma_piece<ST ^ 1, 4>(L, P, kload, v, d);
        if (k == 6) dma_piece<ST ^ 1, 5>(L, P, kload, v, d);
        if (k == 7) dma_piece<ST ^ 1, 6>(L, P, kload, v, d);
        if (k == 8) dma_piece<ST ^ 1, 7>(L, P, kload, v, d);
    }
}

// One mxfp8 K block from stage ST: the same schedule as the blockscale kblock
// below (A fragments one row group ahead, barrier after row group 6, the next
// block's head read between the MFMAs of row group 7, its DMA of block kload
// (moved by d to another tile) during the first nine MFMAs), but the block
// scales are applied inside the MFMA and each MFMA accumulates straight into
// its accumulator: no fold.
template <int ST>
__device__ __forceinline__ void kblock_mx(v4f (&acc)[TM][TN], v8i &a, v8i (&bf)[TN], MxScales &x,
                                          const Loader &L, int kload, bool vload, int wm, int wn,
                                          int frow, int g, const TileOff &d = TileOff{0, 0, 0}) {
    const uint8_t *as = stA<ST>();
    v8i an = a;
    v8i a_next = a;
    MxScales xn;
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const v8i af = an;
        if (i + 1 < TM) an = lds_frag(as, wm * WM + (i + 1) * 16 + frow, g);
        if (i == TM - 1) {
            wait_dma_and_sync();
            a_next = lds_frag(stA<ST ^ 1>(), wm * WM + frow, g);
            read_mx_scales<ST ^ 1>(xn, wm, wn, frow, g);
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int k = i * TN + j;
            acc[i][j] = mx_mfma(bf[j], af, acc[i][j], x, i, j);
            if (i == TM - 1) bf[j] = lds_frag(stB<ST ^ 1>(), wn * WN + j * 16 + frow, g);
            dma_block<ST>(L, L.P, k, kload, vload, d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    x = xn;
    a = a_next;
}

// ---- blockscale with prepacked B -----------------------------------------
// The prepacked weight holds, for each 16-row group of B and K block, the
// 2 KiB the MFMA takes as its B operand, in lane order and split in two
// 1 KiB halves: half h, lane l = 16 g + r: bytes [16 g + 64 h, 16 g + 64 h + 16)
// of the 128-byte K segment of the group's fragment row r, which is B row
// brow_of(16 nt + r) (the order the LDS-staged kernels stage B in).  A wave loads its fragment j of block kb
// straight into registers with two fully coalesced 1 KiB loads; B needs no
// LDS and no DMA.  A block past the end loads through the zero-size
// descriptor.
template <int H>
__device__ __forceinline__ void load_bp_half(const Loader &L, v8i &f, int j, int kb, bool valid) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(valid ? L.P.rB : L.rZ, L.poff + H * 1024,
                                                          j * L.pstep + kb * 2048, 0);
#pragma unroll
    for (int e = 0; e < 4; e++) f[4 * H + e] = (int)v[e];
}

// The loads of block kb + 1 during the first MFMAs of block kb: the B
// fragments into the registers block kb - 1 used, the A slots and scales by
// DMA into the other stage (unread since the previous block's barrier).
template <int ST>
__device__ __forceinline__ void load_next_pb(const Loader &L, v8i (&bn)[TN], int k, int kb,
                                             int KB) {
    const bool v = kb + 1 < KB;
    if (k < 8) {
        if (k & 1) load_bp_half<1>(L, bn[k >> 1], k >> 1, kb + 1, v);
        else load_bp_half<0>(L, bn[k >> 1], k >> 1, kb + 1, v);
    }
    if (k == 0) dma_piece<ST ^ 1, 8>(L, L.P, kb + 1, v);
    if (k == 1) dma_piece<ST ^ 1, 0>(L, L.P, kb + 1, v);
    if (k == 2) dma_piece<ST ^ 1, 2>(L, L.P, kb + 1, v);
    if (k == 3) dma_piece<ST ^ 1, 4>(L, L.P, kb + 1, v);
    if (k == 4) dma_piece<ST ^ 1, 6>(L, L.P, kb + 1, v);
}

// The first K block of a tile: A slots and scales by DMA into stage ST, the
// B fragments into b; then the head reads (A row group 0, the scales).
template <int ST>
__device__ __forceinline__ void load_first_pb(const Loader &L, v8i (&b)[TN]) {
    dma_piece<ST, 8>(L, L.P, 0, true);
    dma_piece<ST, 0>(L, L.P, 0, true); dma_piece<ST, 2>(L, L.P, 0, true);
    dma_piece<ST, 4>(L, L.P, 0, true); dma_piece<ST, 6>(L, L.P, 0, true);
#pragma unroll
    for (int j = 0; j < TN; j++) {
        load_bp_half<0>(L, b[j], j, 0, true);
        load_bp_half<1>(L, b[j], j, 0, true);
    }
}

template <int ST>
__device__ __forceinline__ void read_head_pb(v8i &a, float (&s)[TM], int wm, int wn, int frow,
                                             int fc) {
    a = lds_frag(stA<ST>(), wm * WM + frow, fc);
    RawScales r;
    read_scales<ST>(r, wm, wn, frow);
    combine_scales(s, r);
}

// One K block as kblock below, with the B fragments of this block in bc and
// those of the next block loaded into bn.
template <int ST>
__device__ __forceinline__ void kblock_pb(v4f (&acc)[TM][TN], v4f (&p)[4], float &s_tail, v8i &a,
                                          const v8i (&bc)[TN], v8i (&bn)[TN], float (&s)[TM],
                                          const Loader &L, int kb, int KB, int wm, int wn,
                                          int frow, int fc) {
    const uint8_t *as = stA<ST>();
    v8i an = a;
    v8i a_next = a;
    RawScales rn;
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const v8i af = an;
        if (i + 1 < TM) an = lds_frag(as, wm * WM + (i + 1) * 16 + frow, fc);
        if (i == TM - 1) {
            wait_dma_and_sync();
            a_next = lds_frag(stA<ST ^ 1>(), wm * WM + frow, fc);
            read_scales<ST ^ 1>(rn, wm, wn, frow);
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int k = i * TN + j;
            p[k & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bc[j], af, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            if (k >= 3) {
                const int kp = k - 3;
                fold4(acc[kp / TN][kp % TN], p[kp & 3], s[kp / TN]);
            } else {
                fold4(acc[TM - 1][k + 1], p[(k + 1) & 3], s_tail);
            }
            load_next_pb<ST>(L, bn, k, kb, KB);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    s_tail = s[TM - 1];
    combine_scales(s, rn);
    a = a_next;
}

// One K block from stage ST: 8 x 4 MFMAs per wave, each into a zeroed
// temporary p[k % 4] that is folded into its accumulator (one fma per
// element, by the row's combined scale) three MFMAs later, when it is
// certainly complete.  The fold pipeline runs on across K blocks: the last
// three products of a block are folded during the first MFMAs of the next,
// with that block's row-group-7 scale s_tail.
//
// The next K block kb + 1 goes to the other stage, which nobody reads after
// the previous block's barrier: its DMA is issued one instruction after each
// of nine consecutive MFMAs from MFMA SHIFT on (0 or DMA_SHIFT, see
// gemm_persistent).  After row group 6 (every fragment of this
// stage is then in registers) each wave waits for its DMA and the waves meet
// at a barrier; the reads of block kb + 1's first fragments and scales then go
// out between the MFMAs of row group 7, so that its MFMAs find them landed.
// The block loaded is block kload of the panels P, moved by d to another
// tile: the persistent kernel's last block of a tile loads the next tile's
// block 0, whose head it then reads.  After the last tile the DMA goes
// nowhere and those reads fetch unused values.
template <int ST, int SHIFT = 0>
__device__ __forceinline__ void kblock(v4f (&acc)[TM][TN], v4f (&p)[4], float &s_tail, v8i &a,
                                       v8i (&bf)[TN], float (&s)[TM], const Loader &L,
                                       const Panels &P, int kload, bool vload, int wm, int wn,
                                       int frow, int fc, const TileOff &d = TileOff{0, 0, 0}) {
    const uint8_t *as = stA<ST>();
    v8i an = a;
    v8i a_next = a;
    RawScales rn;
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const v8i af = an;
        if (i + 1 < TM) an = lds_frag(as, wm * WM + (i + 1) * 16 + frow, fc);
        if (i == TM - 1) {
            wait_dma_and_sync();
            a_next = lds_frag(stA<ST ^ 1>(), wm * WM + frow, fc);
            read_scales<ST ^ 1>(rn, wm, wn, frow);
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int k = i * TN + j;
            p[k & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bf[j], af, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            if (k >= 3) {
                const int kp = k - 3;
                fold4(acc[kp / TN][kp % TN], p[kp & 3], s[kp / TN]);
            } else {
                // products 29, 30, 31 of the previous block: row group 7
                fold4(acc[TM - 1][k + 1], p[(k + 1) & 3], s_tail);
            }
            if (i == TM - 1) {
                bf[j] = lds_frag(stB<ST ^ 1>(), wn * WN + j * 16 + frow, fc);
            }
            // the DMA of the next block (kload, normally kb + 1) into the
            // other stage (unread since the previous block's barrier), one
            // instruction after each of nine consecutive MFMAs from MFMA
            // SHIFT on, away from the head reads of row group 7
            if (k >= SHIFT) dma_block<ST>(L, P, k - SHIFT, kload, vload, d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    s_tail = s[TM - 1];
    combine_scales(s, rn);
    a = a_next;
}

constexpr int MODE_BS = 0, MODE_PB = 1, MODE_MX = 2;

// Workgroup (or, in the persistent kernel, virtual workgroup) b -> tile,
// XCD-aware and grouped: b runs on XCD b % 8, which is given the contiguous
// run of tiles [x * per_xcd, (x + 1) * per_xcd), ordered in groups of GROUP_M
// M-tiles.  False for the padding workgroups past the last tile.
__device__ __forceinline__ bool tile_of(const GemmArgs &g, int b, int64_t &m0, int64_t &n0) {
    const int T = g.tiles_m * g.tiles_n;
    const int per_xcd = (T + NUM_XCD - 1) / NUM_XCD;
    if (b >= per_xcd * NUM_XCD) return false;
    const int t = (b % NUM_XCD) * per_xcd + b / NUM_XCD;
    if (t >= T) return false;
    const int group = t / (GROUP_M * g.tiles_n);
    const int first_m = group * GROUP_M;
    const int gm = min(GROUP_M, g.tiles_m - first_m);
    const int local = t - group * GROUP_M * g.tiles_n;
    m0 = (int64_t)(first_m + local % gm) * BM;
    n0 = (int64_t)(local / gm) * BN;
    return true;
}

// The tile-dependent part of the loader in the tile kernels: descriptors of
// the tile's row panels and scales, zero past the end of the matrices.
template <int MODE>
__device__ __forceinline__ Panels panels_of(const GemmArgs &g, int64_t m0, int64_t n0, int wave) {
    const int64_t K = g.K;
    Panels P;
    P.rA = make_rsrc(g.A + m0 * K, (g.M - m0) * K);
    if (MODE == MODE_PB)
        P.rB = make_rsrc(g.B + (n0 / 16) * ((int64_t)g.KB * 2048), (g.N - n0) * K);
    else
        P.rB = make_rsrc(g.B + n0 * K, (g.N - n0) * K);
    if (MODE == MODE_MX) {
        const int KQ = (int)(K / 32);   // mxfp8 scale bytes per row
        P.rS = wave < 4 ? make_rsrc((const uint8_t *)g.sa + m0 * KQ, (g.M - m0) * KQ)
                        : make_rsrc((const uint8_t *)g.sb + n0 * KQ, (g.N - n0) * KQ);
    } else {
        const int nb0 = (int)(n0 / 128);
        P.rS = wave < 4 ? make_rsrc((const float *)g.sa + m0 * g.KB, (g.M - m0) * g.KB * 4)
                        : make_rsrc((const float *)g.sb + (int64_t)nb0 * g.KB,
                                    (int64_t)(g.NB - nb0) * g.KB * 4);
    }
    return P;
}

// The lane-dependent part, the same for every tile.
template <int MODE>
__device__ __forceinline__ void init_loader(Loader &L, const GemmArgs &g, int wave, int lane) {
    const int K = (int)g.K;
    L.rZ = make_rsrc(g.A, 0);
    L.ldsq = wave * 4096;
    if (MODE == MODE_PB) {
        L.pstep = g.KB * 2048;
        L.poff = (wave & 3) * TN * L.pstep + lane * 16;
    }
    // slot 0's row and chunk of this lane (see load_stage); the odd slots'
    // rows are 4 further on, so their row & 7 has bit 2 set
    const int row = wave * 32 + (lane >> 4) + 8 * ((lane >> 3) & 1);
    const int chunk = (lane & 7) ^ (lane >> 4);
    L.voff = row * K + chunk * 16;
    L.voff1 = L.voff ^ 64;
    const int rowB = wave * 32 + (lane >> 4) + 16 * ((lane >> 3) & 1);   // = brow_of(LDS row)
    L.voffB = rowB * K + chunk * 16;
    L.voffB1 = L.voffB ^ 64;
    L.k4 = 4 * K;
    // blockscale: waves 0..3 fetch a_scale in the slot order of sa_row;
    // mxfp8: each row's 4 scale bytes in the slot order of mx_scale_row
    L.soff = MODE == MODE_MX ? mx_scale_row(wave * 64 + lane) * (K / 32)
                             : (wave < 4 ? sa_row(wave * 64 + lane) : lane) * g.KB * 4;
    L.sdst = wave * 256;
}

// The persistent kernels' descriptors cover whole matrices (each
// under 2^31 bytes, which the host checks), and a tile is a byte offset in
// the lanes' offsets: range-checked like them, so rows past the end still
// read zeros, and a tile change needs no new descriptor.
template <int MODE>
__device__ __forceinline__ Panels whole_panels(const GemmArgs &g, int wave) {
    Panels P;
    P.rA = make_rsrc(g.A, g.M * g.K);
    P.rB = make_rsrc(g.B, g.N * g.K);
    if (MODE == MODE_MX)
        P.rS = wave < 4 ? make_rsrc(g.sa, g.M * (g.K / 32)) : make_rsrc(g.sb, g.N * (g.K / 32));
    else
        P.rS = wave < 4 ? make_rsrc(g.sa, g.M * g.KB * 4) : make_rsrc(g.sb, (int64_t)g.NB * g.KB * 4);
    return P;
}

// Tile (m0, n0)'s offsets for whole_panels: A's and B's row panels, and the
// scales this wave fetches (a_scale rows for waves 0..3, b_scale column
// blocks for 4..7).
template <int MODE>
__device__ __forceinline__ TileOff tile_off(const GemmArgs &g, int64_t m0, int64_t n0, int wave) {
    TileOff t;
    t.a = (int)(m0 * g.K);
    t.b = (int)(n0 * g.K);
    if (MODE == MODE_MX)
        t.s = (int)((wave < 4 ? m0 : n0) * (g.K / 32));
    else
        t.s = wave < 4 ? (int)(m0 * g.KB * 4) : (int)((n0 / 128) * g.KB * 4);
    return t;
}

__device__ __forceinline__ void shift_loader(Loader &L, const TileOff &d) {
    L.voff += d.a;
    L.voff1 += d.a;
    L.voffB += d.b;
    L.voffB1 += d.b;
    L.soff += d.s;
}

// Where the epilogue's stores go.  Row m0 + ml of a tile lies in band
// d0 + (r0 + ml) / band_rows at row (r0 + ml) % band_rows, with d0, r0 those
// of the tile's first row (rows < 2^31): one division per tile.  With bands
// of at least 256 rows a tile crosses at most one band boundary, at tile row
// mlb: rows before it are at element off0 + ml * N of C, rows from it on at
// off1 + ml * N, so each stored row costs a compare, a select and an add.
struct BandOut {
    int64_t off0, off1, lane_off, n;
    uint32_t br, d0, r0;
    int mlb, rows, ml0;
    bool col_ok;
};
__device__ __forceinline__ BandOut band_out(const GemmArgs &g, int64_t m0, int64_t n, int ml0) {
    BandOut o;
    o.n = n;
    o.ml0 = ml0;
    o.br = (uint32_t)g.band_rows;
    o.d0 = __builtin_amdgcn_readfirstlane((uint32_t)m0 / o.br);
    o.r0 = (uint32_t)m0 - o.d0 * o.br;
    o.rows = (int)(g.M - m0 < BM ? g.M - m0 : BM);   // tile rows inside M
    o.col_ok = n < g.N;
    o.lane_off = (int64_t)ml0 * g.N + n;
    o.off0 = (int64_t)o.d0 * g.band_stride + (int64_t)o.r0 * g.N;
    o.off1 = (int64_t)(o.d0 + 1) * g.band_stride - (int64_t)(o.br - o.r0) * g.N;
    o.mlb = o.br - o.r0 < (uint32_t)BM ? (int)(o.br - o.r0) : BM;
    return o;
}
template <int MODE>
__device__ __forceinline__ void store_piece(uint16_t *dst, u32x4 v) {
    // C is written once.  Inside the wo_b step, storing it non-temporally
    // made both the blockscale GEMM and the fused reduce that follows it
    // faster (step 338 -> 331 us); the mxfp8 GEMM, measured on its own,
    // was slower with it (162 -> 167 us) and keeps ordinary stores.
    if constexpr (MODE == MODE_MX) *(u32x4 *)dst = v;
    else __builtin_nontemporal_store(v, (u32x4 *)dst);
}

// Store one 16-byte piece of tile row ml = o.ml0 + dml (dml a constant) at
// column o.n + dn.
template <int MODE>
__device__ __forceinline__ void band_store(const GemmArgs &g, const BandOut &o, int dml, int dn, u32x4 v) {
    const int ml = o.ml0 + dml;
    if (ml >= o.rows || !o.col_ok) return;
    uint16_t *dst;
    if (o.br >= BM) {
        dst = g.C + ((ml < o.mlb ? o.off0 : o.off1) + o.lane_off + (int64_t)dml * g.N + dn);
    } else {
        const uint32_t rr = o.r0 + (uint32_t)ml;
        dst = g.C + ((int64_t)(o.d0 + rr / o.br) * g.band_stride + (int64_t)(rr % o.br) * g.N + o.n + dn);
    }
    store_piece<MODE>(dst, v);
}

// The epilogue: each wave's 128 x 64 bf16 sub-tile goes from the accumulators
// straight to the destination band, without LDS.  With B's rows staged in the
// order of brow_of, lane l = r + 16 g (r < 16) holds for row group i the 8
// consecutive columns 8 g .. +8 ("piece" g of the row's 8 16-byte pieces) of
// tile row 16 i + r in sub-tiles 0 and 1 (lo), and piece 4 + g in sub-tiles 2
// and 3 (hi).  Lanes l and l ^ 8 (rows r and r ^ 8) trade their hi pieces
// with one DPP row rotation by 8; then the lanes with r < 8 hold pieces g and
// 4 + g of row r and the lanes with r >= 8 pieces 4 + g and g of row r - 8
// (the X store), and likewise for rows r + 8 (the Y store).  Each store
// instruction so writes 8 whole 128-byte row segments, which measured faster
// than 16 half rows.  A wave's columns are either all inside N or all past it
// (N % 128 == 0).
__device__ __forceinline__ u32x4 swap_rows8(u32x4 v) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; e++)   // row_ror:8 within each 16-lane row: lane l reads lane l ^ 8
        r[e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[e], 0x128, 0xF, 0xF, false);
    return r;
}

// The pieces lane l stores for row group i: x for tile row 16 i + (l % 8) at
// column piece px, y for tile row 16 i + 8 + (l % 8) at piece px +- 4.
__device__ __forceinline__ void tile_pieces(const v4f (&acc)[TM][TN], int i, bool up, u32x4 &x, u32x4 &y) {
    const u32x4 lo = {pack_bf16x2(acc[i][0][0], acc[i][0][1]), pack_bf16x2(acc[i][0][2], acc[i][0][3]),
                      pack_bf16x2(acc[i][1][0], acc[i][1][1]), pack_bf16x2(acc[i][1][2], acc[i][1][3])};
    const u32x4 hi = swap_rows8(
        (u32x4){pack_bf16x2(acc[i][2][0], acc[i][2][1]), pack_bf16x2(acc[i][2][2], acc[i][2][3]),
                pack_bf16x2(acc[i][3][0], acc[i][3][1]), pack_bf16x2(acc[i][3][2], acc[i][3][3])});
#pragma unroll
    for (int e = 0; e < 4; e++) {
        x[e] = up ? hi[e] : lo[e];
        y[e] = up ? lo[e] : hi[e];
    }
}

// Whether every row and column of the tile is inside the matrix and the
// bands are contiguous (C is then plain row-major [M, N]): the epilogue of
// such a tile takes the fast path of store_tile, and every lane issues all
// 2 * TM of its stores.
__device__ __forceinline__ bool tile_is_plain(const GemmArgs &g, int64_t m0, int64_t n0) {
    return m0 + BM <= g.M && n0 + BN <= g.N && g.band_stride == g.band_rows * g.N;
}

template <int MODE>
__device__ __forceinline__ void store_tile(const v4f (&acc)[TM][TN], const GemmArgs &g, int64_t m0,
                                           int64_t n0, int wave, int lane) {
    // opaque to the compiler, so that the addresses below are formed here
    // rather than hoisted out of a tile loop and kept live across it
    asm volatile("" : "+v"(lane));
    const int wm = wave >> 2, wn = wave & 3;
    const bool up = (lane >> 3) & 1;                 // r >= 8
    const int px = (lane >> 4) + (up ? 4 : 0);       // piece of the X store
    const int dny = up ? -32 : 32;                   // the Y store's piece, in columns from X's
    if (tile_is_plain(g, m0, n0)) {
        // row-major C, no bounds: a uniform base per row group and one
        // 32-bit lane offset (the tile spans 256 rows of N <= 2^22 elements)
        const uint32_t lx = (uint32_t)((wm * WM + (lane & 7)) * g.N + wn * WN + px * 8);
        const uint32_t ly = lx + (uint32_t)(8 * g.N + dny);
        uint16_t *base = g.C + m0 * g.N + n0;
#pragma unroll
        for (int i = 0; i < TM; i++) {
            u32x4 x, y;
            tile_pieces(acc, i, up, x, y);
            uint16_t *bi = base + (int64_t)i * 16 * g.N;
            store_piece<MODE>(bi + lx, x);
            store_piece<MODE>(bi + ly, y);
        }
        return;
    }
    const BandOut o = band_out(g, m0, n0 + wn * WN + px * 8, wm * WM + (lane & 7));
#pragma unroll
    for (int i = 0; i < TM; i++) {
        u32x4 x, y;
        tile_pieces(acc, i, up, x, y);
        band_store<MODE>(g, o, i * 16, 0, x);
        band_store<MODE>(g, o, i * 16 + 8, dny, y);
    }
}

// One 256x256 output tile.  MODE_BS: blockscale operands, A and B staged in
// LDS; MODE_PB: blockscale with the prepacked B loaded into registers;
// MODE_MX: mxfp8 operands (E8M0 scales per 1x32 block, applied by the scaled
// MFMA).
template <int MODE>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g) {
    int64_t m0, n0;
    if (!tile_of(g, blockIdx.x, m0, n0)) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep in SGPRs
    const int wm = wave >> 2, wn = wave & 3;
    const int KB = g.KB;
    constexpr bool MX = MODE == MODE_MX;

    Loader L;
    init_loader<MODE>(L, g, wave, lane);
    L.P = panels_of<MODE>(g, m0, n0, wave);

    const int frow = lane & 15;
    const int fc = lane >> 4;   // the lane group: K chunks fc and fc + 4
    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    if constexpr (MODE == MODE_PB) {
        // stage 1 runs with the B registers bA, stage 0 with bB
        v8i a, bA[TN], bB[TN];
        float s[TM];
        if (KB & 1) {
            load_first_pb<0>(L, bB);
            wait_dma_and_sync();
            read_head_pb<0>(a, s, wm, wn, frow, fc);
        } else {
            load_first_pb<1>(L, bA);
            wait_dma_and_sync();
            read_head_pb<1>(a, s, wm, wn, frow, fc);
        }
        v4f p[4];
#pragma unroll
        for (int q = 0; q < 4; q++) p[q] = (v4f){0.f, 0.f, 0.f, 0.f};
        float s_tail = 0.f;
        int kb = 0;
        if (KB & 1) {
            kblock_pb<0>(acc, p, s_tail, a, bB, bA, s, L, 0, KB, wm, wn, frow, fc);
            kb = 1;
        }
        for (; kb < KB; kb += 2) {
            kblock_pb<1>(acc, p, s_tail, a, bA, bB, s, L, kb, KB, wm, wn, frow, fc);
            kblock_pb<0>(acc, p, s_tail, a, bB, bA, s, L, kb + 1, KB, wm, wn, frow, fc);
        }
#pragma unroll
        for (int j = 1; j < TN; j++) fold4(acc[TM - 1][j], p[(TM * TN - TN + j) & 3], s_tail);
    } else if constexpr (MX) {
        const int gq = lane >> 4;
        v8i a, bf[TN];
        MxScales x;
        if (KB & 1) {
            load_stage<0>(L, 0);
            wait_dma_and_sync();
            read_head_mx<0>(a, bf, x, wm, wn, frow, gq);
        } else {
            load_stage<1>(L, 0);
            wait_dma_and_sync();
            read_head_mx<1>(a, bf, x, wm, wn, frow, gq);
        }
        int kb = 0;
        if (KB & 1) {
            kblock_mx<0>(acc, a, bf, x, L, 1, 1 < KB, wm, wn, frow, gq);
            kb = 1;
        }
        for (; kb < KB; kb += 2) {
            kblock_mx<1>(acc, a, bf, x, L, kb + 1, kb + 1 < KB, wm, wn, frow, gq);
            kblock_mx<0>(acc, a, bf, x, L, kb + 2, kb + 2 < KB, wm, wn, frow, gq);
        }
    } else {

    // K block kb sits in stage (kb + KB + 1) % 2, so that the blocks after
    // an odd first one come in (stage 1, stage 0) pairs.  The first block is
    // loaded and read before the loop; each block then starts the DMA of the
    // next one (see kblock).
    v8i a, bf[TN];
    float s[TM];
    if (KB & 1) {
        load_stage<0>(L, 0);
        wait_dma_and_sync();
        read_head<0>(a, bf, s, wm, wn, frow, fc);
    } else {
        load_stage<1>(L, 0);
        wait_dma_and_sync();
        read_head<1>(a, bf, s, wm, wn, frow, fc);
    }

    // nothing pending before the first block: its first three folds add 0 * 0
    v4f p[4];
#pragma unroll
    for (int q = 0; q < 4; q++) p[q] = (v4f){0.f, 0.f, 0.f, 0.f};
    float s_tail = 0.f;

    int kb = 0;
    if (KB & 1) {
        kblock<0>(acc, p, s_tail, a, bf, s, L, L.P, 1, 1 < KB, wm, wn, frow, fc);
        kb = 1;
    }
    for (; kb < KB; kb += 2) {
        kblock<1>(acc, p, s_tail, a, bf, s, L, L.P, kb + 1, kb + 1 < KB, wm, wn, frow, fc);
        kblock<0>(acc, p, s_tail, a, bf, s, L, L.P, kb + 2, kb + 2 < KB, wm, wn, frow, fc);
    }
#pragma unroll
    for (int j = 1; j < TN; j++) fold4(acc[TM - 1][j], p[(TM * TN - TN + j) & 3], s_tail);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the last (empty) DMA is retired

    store_tile<MODE>(acc, g, m0, n0, wave, lane);
}

// A plain tile's epilogue is split in two, so that neither end of a tile
// boundary waits idle.  Its row groups 0 .. TAIL_RG - 1 are stored at the end
// of the tile (in gemm_persistent, after the K loop), behind the next tile's
// first DMA and while it lands; the rest go out inside the next tile's first
// K block (kblock_first).  TAIL_RG = 4 measured 1-2 % faster than 0, 2, 6 or
// 8.
constexpr int TAIL_RG = 4;

// The lane's two store offsets in a row group of a plain tile, in elements
// (see store_tile), and its half.
struct PlainOffsets {
    uint32_t lx, ly;
    bool up;
};
__device__ __forceinline__ PlainOffsets plain_offsets(int64_t N, int wm, int wn, int lane) {
    asm volatile("" : "+v"(lane));   // formed here, per tile, not hoisted
    PlainOffsets o;
    o.up = (lane >> 3) & 1;
    const int px = (lane >> 4) + (o.up ? 4 : 0);
    o.lx = (uint32_t)((wm * WM + (lane & 7)) * N + wn * WN + px * 8);
    o.ly = o.lx + (uint32_t)(8 * N + (o.up ? -32 : 32));
    return o;
}

// Row group i of a plain tile (i a constant once the caller's loop is
// unrolled), stored non-temporally through rC (a descriptor of C from the
// tile's first element on), or through the zero-size descriptor, which
// stores nothing but issues the same two instructions.
__device__ __forceinline__ void plain_store_rg(const v4f (&acc)[TM][TN], int i, __amdgpu_buffer_rsrc_t rC,
                                               int64_t N, const PlainOffsets &o) {
    u32x4 x, y;
    tile_pieces(acc, i, o.up, x, y);
    const uint32_t ri = (uint32_t)(i * 16 * N);   // the row group's first element
    __builtin_amdgcn_raw_buffer_store_b128(x, rC, 2 * (ri + o.lx), 0, 2);   // 2: nt
    __builtin_amdgcn_raw_buffer_store_b128(y, rC, 2 * (ri + o.ly), 0, 2);
}

// The first K block of every tile in the persistent blockscale kernel.  It
// carries no products over from a previous block, and the first fold of each
// sub-tile, three MFMAs after its MFMA as in kblock, sets the accumulator to
// fma(p, s, +0), which is what folding into a zeroed accumulator gives; the
// last three sub-tiles, whose first fold is the next block's, are zeroed
// here.  So the accumulators may still hold the previous tile when the block
// starts: if that tile was a plain one (see tile_is_plain), the stores of
// its row group i >= TAIL_RG go out here, just before MFMA 4 i, the last
// reads of those accumulators, and drain while the new tile's MFMAs run.  rC
// is a descriptor of the previous tile's part of C from its first element
// on (row-major C: contiguous bands), or the zero-size one when there is
// nothing to store: the stores are always issued, so that every wave runs
// the same instructions and the vector memory count below is exact.  The
// DMA of block 1 goes out after MFMAs 0..8 as in kblock, before the stores of
// row groups 4..6, so at the barrier before row group 7 this wave's DMA has
// landed once at most those 6 stores are outstanding (vector memory
// operations retire in issue order).
template <int ST>
__device__ __forceinline__ void kblock_first(v4f (&acc)[TM][TN], v4f (&p)[4], float &s_tail, v8i &a,
                                             v8i (&bf)[TN], float (&s)[TM], const Loader &L,
                                             const Panels &P, int kload, bool vload, int wm, int wn,
                                             int frow, int fc, __amdgpu_buffer_rsrc_t rC,
                                             int64_t N, const PlainOffsets &o) {
    static_assert(TAIL_RG >= 3 && TAIL_RG <= 6, "the wait below counts the stores of row groups TAIL_RG..6");
    const uint8_t *as = stA<ST>();
    v8i an = a;
    v8i a_next = a;
    RawScales rn;
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const v8i af = an;
        if (i + 1 < TM) an = lds_frag(as, wm * WM + (i + 1) * 16 + frow, fc);
        if (i == TM - 1) {
            // vmcnt(2 * (7 - TAIL_RG)): the stores of row groups TAIL_RG..6 may remain
            __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (7 - TAIL_RG)));
            barrier_lds_only();
            a_next = lds_frag(stA<ST ^ 1>(), wm * WM + frow, fc);
            read_scales<ST ^ 1>(rn, wm, wn, frow);
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int k = i * TN + j;
            if (j == 0 && i >= TAIL_RG) plain_store_rg(acc, i, rC, N, o);
            if (j == 0 && i == TM - 1) {
                // products 29..31 are first folded by the next block, which
                // adds them (fma into the accumulator): start those at zero
#pragma unroll
                for (int jj = 1; jj < TN; jj++) acc[i][jj] = (v4f){0.f, 0.f, 0.f, 0.f};
            }
            p[k & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bf[j], af, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            if (k >= 3) {
                const int kp = k - 3;
#pragma unroll
                for (int e = 0; e < 4; e++)
                    acc[kp / TN][kp % TN][e] = __builtin_fmaf(p[kp & 3][e], s[kp / TN], 0.0f);
            }
            if (i == TM - 1) {
                bf[j] = lds_frag(stB<ST ^ 1>(), wn * WN + j * 16 + frow, fc);
            }
            dma_block<ST>(L, P, k, kload, vload);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    s_tail = s[TM - 1];
    combine_scales(s, rn);
    a = a_next;
}

// ---- persistent kernels (K / 128 even; blockscale and mxfp8) ----
// One workgroup per CU walks the tiles of virtual workgroups b, b + G,
// b + 2G, ... (G = grid size, a multiple of 8, so every tile stays on the XCD
// the non-persistent mapping gives it).  The K blocks of successive tiles form
// one stream; block 0 of every tile sits in stage 1, its last block in stage
// 0.  The descriptors cover whole matrices, so the last K block of a tile
// DMAs the next tile's block 0 (its lanes' offsets moved by dn) as any block
// DMAs its successor, and reads its head.  (Switching descriptors inside the
// K loop instead made the compiler spill hundreds of VGPRs.)  Blockscale: a
// plain tile then stores half of its row groups at once and the other half
// inside the next tile's first K block (kblock_first), between its MFMAs.
// mxfp8: a plain tile stores all of them at once, and they drain under the
// next tile's first K block.  The last tile and tiles that are not plain
// store everything at once.
// The blockscale kernel runs one copy of this body per row half of the wave
// grid (WMC = wm, a compile-time constant: each wave executes straight-line
// code with its row offsets folded), and the second half issues its K
// blocks' DMA DMA_SHIFT MFMAs later than the first, so that the two waves of
// a SIMD do not stall on DMA issue at the same time (together ≈ 3 % faster,
// bit-identical; a shift of 8 was slower).  WMC = -1: one body, wm at run
// time (mxfp8).
constexpr int DMA_SHIFT = 4;

template <int MODE, int WMC>
__device__ __forceinline__ void gemm_persistent(const GemmArgs &g) {
    constexpr int DSH = WMC == 1 ? DMA_SHIFT : 0;
    constexpr bool MX = MODE == MODE_MX;
    int vb = blockIdx.x;
    int64_t m0, n0;
    if (!tile_of(g, vb, m0, n0)) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep in SGPRs
    const int wm = WMC >= 0 ? WMC : wave >> 2;
    const int wn = wave & 3;
    const int KB = g.KB;   // even, at least 2
    const int frow = lane & 15;
    const int fc = lane >> 4;   // the lane group: K chunks fc and fc + 4

    Loader L;
    init_loader<MODE>(L, g, wave, lane);
    L.P = whole_panels<MODE>(g, wave);
    shift_loader(L, tile_off<MODE>(g, m0, n0, wave));

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    // block 0 of every tile sits in stage 1 (K / 128 even)
    const int gq = lane >> 4;   // mxfp8: the lane's 32-wide K group
    v8i a, bf[TN];
    float s[TM];
    MxScales x;
    load_stage<1>(L, 0);
    wait_dma_and_sync();
    if constexpr (MX) read_head_mx<1>(a, bf, x, wm, wn, frow, gq);
    else read_head<1>(a, bf, s, wm, wn, frow, fc);

    v4f p[4];
#pragma unroll
    for (int q = 0; q < 4; q++) p[q] = (v4f){0.f, 0.f, 0.f, 0.f};
    float s_tail = 0.f;

    // The kernel's only argument, read in place from the kernarg segment
    // where each tile needs it (scalar loads), rather than held in SGPRs
    // across the K loop.
    typedef const __attribute__((address_space(4))) GemmArgs *KArgs;
    const KArgs gp = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
    auto args = [gp]() {
        KArgs q = gp;
        asm volatile("" : "+s"(q));
        return *(const GemmArgs *)q;
    };
    // blockscale: whether the accumulators hold the previous tile, whose
    // stores then go out inside this tile's first K block (kblock_first), and
    // that tile's origin
    bool pend = false;
    int64_t pm0 = 0, pn0 = 0;
    // the tile after this one and the move of the loader's offsets from
    // this tile to it (zero if there is none); found at the tile boundary,
    // so that only three offsets stay live across the K loop
    int64_t m0n = 0, n0n = 0;
    bool has_next = false;
    TileOff dn = {0, 0, 0};
    auto find_next = [&]() {
        const GemmArgs gt = args();
        has_next = __builtin_amdgcn_readfirstlane((int)tile_of(gt, vb + (int)gridDim.x, m0n, n0n));
        dn = TileOff{0, 0, 0};
        if (has_next) {
            const TileOff tn = tile_off<MODE>(gt, m0n, n0n, wave), tc = tile_off<MODE>(gt, m0, n0, wave);
            dn.a = __builtin_amdgcn_readfirstlane(tn.a - tc.a);
            dn.b = __builtin_amdgcn_readfirstlane(tn.b - tc.b);
            dn.s = __builtin_amdgcn_readfirstlane(tn.s - tc.s);
        }
    };
    find_next();
    for (;;) {
        if constexpr (MX) {
            const TileOff d0 = {0, 0, 0};
            for (int kb = 0; kb < KB; kb += 2) {
                kblock_mx<1>(acc, a, bf, x, L, kb + 1, true, wm, wn, frow, gq);
                kblock_mx<0>(acc, a, bf, x, L, kb + 2 < KB ? kb + 2 : 0, kb + 2 < KB || has_next, wm, wn,
                             frow, gq, kb + 2 < KB ? d0 : dn);
            }
            shift_loader(L, dn);
        } else {
            {
                const GemmArgs gt = args();
                const PlainOffsets o = plain_offsets(gt.N, wm, wn, lane);
                const __amdgpu_buffer_rsrc_t rC =
                    pend ? make_rsrc(gt.C + pm0 * gt.N + pn0, (gt.M - pm0) * gt.N * 2) : L.rZ;
                kblock_first<1>(acc, p, s_tail, a, bf, s, L, L.P, 1, true, wm, wn, frow, fc, rC,
                                gt.N, o);
            }
            // The last block (always in stage 0) DMAs the next tile's block
            // 0 into stage 1, as any block DMAs its successor, and its head
            // reads fetch that block's first fragments and scales.
            const TileOff d0 = {0, 0, 0};
            kblock<0, DSH>(acc, p, s_tail, a, bf, s, L, L.P, 2 < KB ? 2 : 0, 2 < KB || has_next, wm, wn,
                           frow, fc, 2 < KB ? d0 : dn);
            for (int kb = 2; kb < KB; kb += 2) {
                kblock<1, DSH>(acc, p, s_tail, a, bf, s, L, L.P, kb + 1, true, wm, wn, frow, fc);
                kblock<0, DSH>(acc, p, s_tail, a, bf, s, L, L.P, kb + 2 < KB ? kb + 2 : 0,
                               kb + 2 < KB || has_next, wm, wn, frow, fc, kb + 2 < KB ? d0 : dn);
            }
            shift_loader(L, dn);
        }
        if constexpr (!MX) {
            // the last three products of the tile (kblock_first carries none)
#pragma unroll
            for (int j = 1; j < TN; j++) fold4(acc[TM - 1][j], p[(TM * TN - TN + j) & 3], s_tail);
        }

        if constexpr (MX) {
            // The last tile and tiles that are not plain store here; a plain
            // one stores its 2 * TM pieces per lane (other tiles issue the
            // same instructions through the zero-size descriptor, so that
            // every path issues the same vector memory operations), and they
            // drain under the next tile's first K block, whose block 0 and
            // head are already in.
            const bool plain = tile_is_plain(args(), m0, n0);
            if (!has_next || !plain) store_tile<MODE>(acc, args(), m0, n0, wave, lane);
            if (!has_next) break;
            {
                const GemmArgs gt = args();
                const PlainOffsets o = plain_offsets(gt.N, wm, wn, lane);
                const __amdgpu_buffer_rsrc_t rT =
                    plain ? make_rsrc(gt.C + m0 * gt.N + n0, (gt.M - m0) * gt.N * 2) : L.rZ;
#pragma unroll
                for (int i = 0; i < TM; i++) plain_store_rg(acc, i, rT, gt.N, o);
            }
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
        } else {
            // The last tile and tiles that are not plain store here.  A
            // plain tile stores its row groups 0 .. TAIL_RG - 1 here and the
            // rest inside the next tile's first K block.  Every path issues
            // those 2 * TAIL_RG stores (other tiles through the zero-size
            // descriptor), so that the vector memory count of the next
            // tile's first block is exact.  The next tile's block 0 and its
            // head are already in (the last K block loaded them).
            const bool plain = tile_is_plain(args(), m0, n0);
            if (!has_next || !plain) store_tile<MODE>(acc, args(), m0, n0, wave, lane);
            if (!has_next) break;
            {
                const GemmArgs gt = args();
                const PlainOffsets o = plain_offsets(gt.N, wm, wn, lane);
                const __amdgpu_buffer_rsrc_t rT =
                    plain ? make_rsrc(gt.C + m0 * gt.N + n0, (gt.M - m0) * gt.N * 2) : L.rZ;
#pragma unroll
                for (int i = 0; i < TAIL_RG; i++) plain_store_rg(acc, i, rT, gt.N, o);
            }
            pend = plain;
            pm0 = m0;
            pn0 = n0;
        }
        vb += (int)gridDim.x;
        m0 = m0n;
        n0 = n0n;
        find_next();
    }
}

__global__ void __launch_bounds__(NTHREADS) bsgemm_persistent_kernel(GemmArgs g) {
    // wm = wave / 4 = threadIdx.x / 256, the same for every lane of a wave
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 8)) gemm_persistent<MODE_BS, 1>(g);
    else gemm_persistent<MODE_BS, 0>(g);
}
__global__ void __launch_bounds__(NTHREADS) mxgemm_persistent_kernel(GemmArgs g) {
    gemm_persistent<MODE_MX, -1>(g);
}

__global__ void __launch_bounds__(NTHREADS) bsgemm_tile_kernel(GemmArgs g) { gemm_tile<MODE_BS>(g); }

__global__ void __launch_bounds__(NTHREADS) bsgemm_pb_tile_kernel(GemmArgs g) { gemm_tile<MODE_PB>(g); }

__global__ void __launch_bounds__(NTHREADS) mxgemm_tile_kernel(GemmArgs g) { gemm_tile<MODE_MX>(g); }

// B [N, K] -> the prepacked layout [N/16][K/128][2][64][16 B]: unit u of the
// output (16 bytes) is half h, lane l = 16 g + r of 16-row group nt and K
// block kb, and holds bytes [16 g + 64 h, +16) of row brow_of(16 nt + r)'s K
// block kb (the two halves of lane l are the chunks lds_frag gives it; the
// rows are those the LDS-staged kernel places in the same fragment slot).
// One lane per output unit: the writes are contiguous, the reads 16-byte
// aligned gathers.
__global__ void __launch_bounds__(256)
bprepack_kernel(const u32x4 *__restrict__ B, u32x4 *__restrict__ Bp, int64_t units, int64_t K) {
    const int64_t KB = K / 128;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * 256) {
        const int l = (int)(u & 63);
        const int h = (int)((u >> 6) & 1);
        const int64_t blk = u >> 7;          // nt * KB + kb
        const int64_t nt = blk / KB, kb = blk - nt * KB;
        const int64_t row = (nt & ~(int64_t)3) * 16 + brow_of((int)((nt & 3) * 16 + (l & 15)));
        const int64_t col = kb * 128 + 16 * (l >> 4) + 64 * h;
        Bp[u] = B[(row * K + col) >> 4];
    }
}

}  // namespace

static GemmArgs gemm_args(const uint8_t *A, const void *sa, const uint8_t *B, const void *sb,
                          uint16_t *C, int64_t M, int64_t N, int64_t K, int64_t band_rows,
                          int64_t band_stride) {
    GemmArgs g;
    g.A = A; g.sa = sa; g.B = B; g.sb = sb; g.C = C;
    g.M = M; g.N = N; g.K = K;
    g.band_rows = band_rows; g.band_stride = band_stride;
    g.KB = (int)(K / 128);
    g.NB = (int)(N / 128);
    g.tiles_m = (int)((M + BM - 1) / BM);
    g.tiles_n = (int)((N + BN - 1) / BN);
    return g;
}

static int gemm_grid(const GemmArgs &g) {
    const int T = g.tiles_m * g.tiles_n;
    return ((T + NUM_XCD - 1) / NUM_XCD) * NUM_XCD;
}

// CUs of the device a stream belongs to, asked once per device and kept
// (an atomic per device: concurrent first calls store the same value).
static std::atomic<int> g_cus[64];

static int stream_cus(hipStream_t stream) {
    hipDevice_t dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < NUM_XCD)
            cus = 256;
        g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// The persistent kernels' grid: one workgroup per CU of the stream's device,
// a multiple of 8 so that the XCD of each tile is the one the non-persistent
// launch gives it.
static int persistent_grid(const GemmArgs &g, hipStream_t stream) {
    const int grid = gemm_grid(g), per = stream_cus(stream) / NUM_XCD * NUM_XCD;
    return grid < per ? grid : per;
}

int bs_launch_gemm(const uint8_t *A, const float *sa, const uint8_t *B, const float *sb,
                   uint16_t *C, int64_t M, int64_t N, int64_t K, int64_t band_rows,
                   int64_t band_stride, hipStream_t stream) {
    const GemmArgs g = gemm_args(A, sa, B, sb, C, M, N, K, band_rows, band_stride);
    // The persistent kernel addresses each operand through one descriptor
    // with 31-bit lane offsets, the rows of a ragged last tile included.
    const int64_t lim = 0x7FFFFFFF;
    if (g.KB % 2 == 0 && (M + BM) * K <= lim && (N + BN) * K <= lim)
        return bs_enqueue(bsgemm_persistent_kernel, dim3(persistent_grid(g, stream)), dim3(NTHREADS),
                          stream, g);
    return bs_enqueue(bsgemm_tile_kernel, dim3(gemm_grid(g)), dim3(NTHREADS), stream, g);
}

int bs_launch_gemm_pb(const uint8_t *A, const float *sa, const uint8_t *Bp, const float *sb,
                      uint16_t *C, int64_t M, int64_t N, int64_t K, int64_t band_rows,
                      int64_t band_stride, hipStream_t stream) {
    const GemmArgs g = gemm_args(A, sa, Bp, sb, C, M, N, K, band_rows, band_stride);
    return bs_enqueue(bsgemm_pb_tile_kernel, dim3(gemm_grid(g)), dim3(NTHREADS), stream, g);
}

int bs_launch_bprepack(const uint8_t *B, uint8_t *Bp, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t units = N * K / 16;
    int64_t blocks = (units + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return bs_enqueue(bprepack_kernel, dim3((unsigned)blocks), dim3(256), stream, (const u32x4 *)B,
                      (u32x4 *)Bp, units, K);
}

int bs_launch_mxgemm(const uint8_t *A, const uint8_t *sa, const uint8_t *B, const uint8_t *sb,
                     uint16_t *C, int64_t M, int64_t N, int64_t K, int64_t band_rows,
                     int64_t band_stride, hipStream_t stream) {
    const GemmArgs g = gemm_args(A, sa, B, sb, C, M, N, K, band_rows, band_stride);
    const int64_t lim = 0x7FFFFFFF;   // as for the blockscale kernel
    if (g.KB % 2 == 0 && (M + BM) * K <= lim && (N + BN) * K <= lim)
        return bs_enqueue(mxgemm_persistent_kernel, dim3(persistent_grid(g, stream)), dim3(NTHREADS),
                          stream, g);
    return bs_enqueue(mxgemm_tile_kernel, dim3(gemm_grid(g)), dim3(NTHREADS), stream, g);
}
