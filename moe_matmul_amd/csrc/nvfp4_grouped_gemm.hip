// NVFP4 block-scaled grouped GEMM for gfx950 (MI355X).
//
// C_g[m, n] = sum_k (a[m,k] * sfa[m,k/16]) * (b[n,k] * sfb[n,k/16]), fp32
// accumulation, fp16 output (the contraction of the block-scaled MMA in
// submissions 506336 / 385043 / 499344, kernelindex.com "kernelbot nvfp4 group
// gemm"; layouts as in the header).
//
// Design (gfx950 first, not a translation of the pages' Blackwell kernels):
//  * Persistent grid of one 256-thread workgroup per compute unit. Workgroup
//    b gets a virtual index that gives each of the 8 XCDs a contiguous run of
//    indices. Whole tiles: virtual index v takes tiles v, v + grid, ...
//    Stream-K: v takes an equal share of all (tile, 128-K stage) units. The
//    group of a tile is found by binary search over the per-group tile prefix
//    sum (the scheduler of submission 506336 keeps the same prefix); inside a
//    group, tiles run down columns of 8-tile-wide super-columns.
//  * Packed FP4 operand tiles and their scale atoms go straight from global
//    memory to LDS (buffer_load ... lds), four stages deep, streamed across
//    tile boundaries. Each 64-byte row slab has its four 16-byte chunks XOR
//    swizzled so that the 128-bit reads of a wave are bank-conflict free.
//  * Scales are read from the tiled layout in LDS: the 16-byte chunk (r % 32)
//    of a 512-byte atom holds rows r, r+32, r+64, r+96 for four 16-blocks,
//    exactly the rows one lane feeds to a 32x32 MFMA.
//  * Exact dequantisation to f16 in registers: v_cvt_scalef32_pk_f16_fp4 with
//    scale 1.0 (E2M1 values are exact in f16), then one v_pk_mul_f16 by the
//    E4M3 scale (converted exactly with v_cvt_scalef32_pk_f16_fp8). |a*s| has
//    at most 6 significant bits, so the product is exact in f16, and the f16
//    MFMA products are exact in fp32. (The scaled conversion only applies the
//    exponent of its f32 scale, so the E4M3 mantissa needs the separate
//    multiply.)
//  * v_mfma_f32_32x32x16_f16 with B as the first operand, so each lane ends up
//    holding four consecutive columns of one output row. A wave skips the
//    LDS reads, dequantisation and MFMAs of its 32-row blocks that lie wholly
//    past m (ragged M of the expert groups); in a tile with a single row
//    block below m the four waves sit side by side along n instead.
//  * Inside each 64-K group the K order fed to the MFMA is permuted so that a
//    lane reads 32 consecutive FP4 codes (16 bytes) of its row: lane half h
//    takes K elements [32h, 32h+32) in four steps of 8. A and B use the same
//    permutation, so the sum is unchanged; each step of 8 lies inside one
//    16-block, so one scale covers it.
//  * Epilogue: fp32 -> fp16 (RNE) fused; a lane-half swap gives each lane 8
//    consecutive columns, stored as 16 bytes, masked to m and n.
//    Tiles split by stream-K store fp32 partials, and their contributors fold
//    them in the same kernel along a fixed binary tree (the second to arrive
//    at a node adds; no workgroup waits for another), so results do not
//    depend on timing.
//  * Scales that are all zero or powers of two (an MX-compatible special case
//    of the pages' MX/NV FP4 block-scaled MMA) have their own mainloop: the
//    packed codes go to v_mfma_scale_f32_32x32x64_f8f6f4 as E2M1 with E8M0
//    scales, one 16-block per 32-K lane slice, without dequantisation.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "nvfp4_grouped_gemm.h"

// Stream-K partials of nvfp4_grouped_gemm_scratch (see scratch_address).
static __device__ __align__(256) uint8_t scratch[NVFP4_SCRATCH_BYTES];

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int N>
using ScaleVec = uint32_t __attribute__((ext_vector_type(N)));

constexpr int kMaxGroups = NVFP4_MAX_GROUPS;
constexpr int kThreads = 256;
constexpr int kBK = 128;          // K elements per pipeline stage
constexpr int kRowBytes = kBK / 2; // packed bytes per row per stage
constexpr int kAtomBytes = 512;    // one 128-row x 64-K scale atom
constexpr int kBufferWord3 = 0x00020000;  // gfx9 buffer resource word 3 (raw, 32-bit data)
constexpr int kXcds = 8;                  // accelerator complex dies: workgroups go round-robin over them
constexpr int kRasterWidth = 8;           // n-tiles per raster super-column

// A work class is a run of tile rows of one group: [tm0, tm0 + tiles_m). The
// host splits a group whose last tile row is mostly past m into its full rows
// and that lighter last row, and orders the classes by cost per tile, heaviest
// first, so that the whole-tile walk below hands out big tiles first.
constexpr int kMaxClasses = 2 * kMaxGroups;
constexpr int kMaxSplitGrid = 512;  // stream-K workgroups (unit ranges passed by value)
// stream-K fold tree levels (contributors of one tile <= kMaxSplitGrid = 2^(kFoldLevels - 1))
constexpr int kFoldLevels = 10;
static_assert(kMaxSplitGrid <= (1 << (kFoldLevels - 1)), "fold tree depth");

struct ClassArgs {
  const uint8_t* a;  // the group's tensors and sizes
  const uint8_t* b;
  uint16_t* c;
  const uint8_t* sfa;
  const uint8_t* sfb;
  int32_t m, n, k, l;
  int32_t tiles_m, tiles_n;  // tile rows of the class, tile columns of the group
  int32_t nk;                // 128-K stages per tile
  int32_t tm0;               // first tile row of the class within its group
};

struct KernelArgs {
  ClassArgs cls[kMaxClasses];
  int32_t tile_prefix[kMaxClasses + 1];  // first tile of class c (tiles numbered class by class)
  int32_t unit_prefix[kMaxClasses + 1];  // first (tile, stage) unit of class c
  int32_t num_classes;
  int32_t split;        // 0: whole tiles strided over the grid; 1: stream-K over units
  int32_t grid;         // workgroups of the main kernel
  // split: tiles [0, whole_tiles) - whole rounds of `grid` tiles - are dealt
  // out whole first (as without split), the units of the rest by range
  int32_t whole_tiles;
  float* partials;      // split: two fp32 tile-sized slots per workgroup
  // split: workgroup w takes units [wg_unit[w], wg_unit[w + 1]) of the tiles
  // from whole_tiles on (a range may be empty); the host sizes the ranges so
  // that every workgroup's modelled cost, its whole tiles included, comes out
  // equal (a stage of a tile that is mostly past m costs less than a full one).
  int32_t wg_unit[kMaxSplitGrid + 1];
  // power-of-two-scale kernels: set to 1 when a used scale is not zero or a
  // positive power of two
  int32_t* status;
};
static_assert(sizeof(KernelArgs) <= 4096, "kernel arguments must fit the kernarg segment");

// 8 FP4 codes (one dword) -> 8 f16 values a * s, exact.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, _Float16 s) {
  const f16x2 ss = {s, s};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Swizzle of the four 16-byte chunks of a 64-byte row slab: chunk c of row r is
// stored at c ^ swz(r). Sixteen consecutive rows read at the same logical chunk
// then land on sixteen distinct 16-byte bank groups of a 256-byte bank window,
// and any eight consecutive rows on eight distinct groups of a 128-byte window.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Byte offset of chunk c of row r inside a staged operand tile.
__device__ __forceinline__ int lds_off(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Raw buffer resource (4 SGPRs): 48-bit base, stride 0, num_records bytes;
// offsets at or past num_records read 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int32_t num_bytes) {
  // 32-bit counts (every operand is validated below 2^31 bytes): scalar
  // arithmetic, where 64-bit compares would go to the vector unit
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{(int32_t)(uint32_t)b, (int32_t)((uint32_t)(b >> 32) & 0xFFFFu), max(num_bytes, 0), kBufferWord3};
}

// 16 bytes per lane from global (buffer, bounds-checked) straight into LDS at
// lds_block + 16 * lane (M0 holds the wave's LDS base). Issued as inline asm so
// the compiler does not treat it as an LDS write it must wait for: the kernel
// tracks these loads itself with exact vmcnt waits. The LDS base is an M0
// input operand, so the compiler sets M0 itself and knows what it holds.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t lds_block, int voffset) {
  // the resource and the LDS address are wave-uniform (the caller passes rsrc
  // through readfirstlane); say so, so they stay in SGPRs
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(lds_block);
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voffset), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

// The waits are emitted with the builtin (not as asm text) so that the
// compiler's own wait insertion knows the counters are clear afterwards; the
// empty asm keeps memory accesses from moving across the wait.
// Workgroup barrier without the compiler's release fence (which would wait for
// every outstanding load): LDS reads of this wave are complete, then s_barrier.
__device__ __forceinline__ void block_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt left at their maximum, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int enc = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(enc);
}

// Instruction-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002;
constexpr int kSchedMFMA = 0x008;
constexpr int kSchedDSRead = 0x100;

// Everything a workgroup needs about one output tile (wave-uniform values).
struct TileCtx {
  const uint8_t* a_tile;   // first byte of the tile's A rows
  const uint8_t* b_tile;
  int32_t a_rem, b_rem;    // bytes from the tile base to the end of the operand (< 2^31)
  const uint8_t* sf_row;   // this wave's scale atom row (nullptr: none)
  int32_t sf_rem;
  uint16_t* c;             // C of the tile's batch
  int M, N, kbytes, nk, row0, col0;
  // Tiles narrower than a 128-row scale atom (64 rows or columns) use half of
  // it: the word offset (0 or 2) inside each 16-byte atom chunk of their first
  // row (A: bits 0-3, B: bits 4-7; 0 for tiles of 128 or more).
  int sub_words;
  // k % 64 == 32: the last 64-K scale atom is half used; its 16-blocks 2 and
  // 3 (bytes 2 and 3 of every 4-byte row word) are padding and may hold
  // anything. kpad_group is the 64-K group of the last stage that holds that
  // atom (0 or 1), -1 when k % 64 == 0.
  int kpad_group;
};

// A run of 128-K stages [s0, s1) of one tile, processed by one workgroup.
struct Segment {
  int tile, s0, s1;
  int64_t u;  // stream-K: first work unit of the segment; whole tiles: the round
  bool valid;
  bool sk;    // a stream-K segment (of a unit range)
};

__device__ __forceinline__ int search_prefix(const int32_t* prefix, int count, int64_t x) {
  int lo = 0, hi = count - 1;  // last entry whose prefix is <= x
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Where a kernel finds its work: the by-value argument block (up to eight
// groups, split into cost-ordered classes by the host) - whole tiles, or with
// SPLIT whole rounds and stream-K (separate instantiations, so that the
// whole-tile kernels carry none of the stream-K code and its registers) ...
template <bool SPLIT>
struct KernargSrc {
  static constexpr bool kCanSplit = SPLIT;
  const KernelArgs& args;
  __device__ __forceinline__ int grid() const { return args.grid; }
  __device__ __forceinline__ bool split() const { return SPLIT && args.split != 0; }
  __device__ __forceinline__ int total_tiles() const { return args.tile_prefix[args.num_classes]; }
  __device__ __forceinline__ int class_of_tile(int tile) const {
    return search_prefix(args.tile_prefix, args.num_classes, tile);
  }
  __device__ __forceinline__ int tile_prefix(int c) const { return args.tile_prefix[c]; }
  __device__ __forceinline__ const ClassArgs& cls(int c) const { return args.cls[c]; }
  __device__ __forceinline__ int nk(int c) const { return args.cls[c].nk; }
  // The first tile's lookup is a chain of dependent scalar loads (grid and
  // class count, the binary search over the tile prefix, then the class);
  // each would miss the scalar cache in turn. One load per 64-byte line of
  // the class table, the prefixes and the counts, all issued at once at the
  // start, puts those lines in the cache for the price of about one miss.
  // The 21 loads read inside the argument block. Their values are not used:
  // every load writes the same register, and the block waits for all of them
  // before it ends.
  __device__ __forceinline__ void prefetch() const {
    static_assert(offsetof(KernelArgs, whole_tiles) + 4 <= 21 * 64, "the lines below cover the counts");
    const KernelArgs* p = &args;
    uint32_t x;
    asm volatile(
        "s_load_dword %0, %1, 0x0\n s_load_dword %0, %1, 0x40\n s_load_dword %0, %1, 0x80\n"
        "s_load_dword %0, %1, 0xc0\n s_load_dword %0, %1, 0x100\n s_load_dword %0, %1, 0x140\n"
        "s_load_dword %0, %1, 0x180\n s_load_dword %0, %1, 0x1c0\n s_load_dword %0, %1, 0x200\n"
        "s_load_dword %0, %1, 0x240\n s_load_dword %0, %1, 0x280\n s_load_dword %0, %1, 0x2c0\n"
        "s_load_dword %0, %1, 0x300\n s_load_dword %0, %1, 0x340\n"
        "s_waitcnt lgkmcnt(7)\n"  // (at most 15 in flight: the counter has four bits)
        "s_load_dword %0, %1, 0x380\n"
        "s_load_dword %0, %1, 0x3c0\n s_load_dword %0, %1, 0x400\n s_load_dword %0, %1, 0x440\n"
        "s_load_dword %0, %1, 0x480\n s_load_dword %0, %1, 0x4c0\n s_load_dword %0, %1, 0x500\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(x)
        : "s"(p));
  }
};

// ... or group tables in device memory. There the kernel makes the classes
// itself, heaviest first as far as the row count goes: with R = BM / 64
// (32-row blocks per wave in a full tile row), class b * G + g holds the tile
// rows of group g in which a wave computes R - b blocks - the full rows for
// b = 0, the last row for the b its row count gives (none if that row is
// full). Tiles are numbered class by class: the full rows of all groups, then
// the last rows, the least light first. Whole tiles only. The tile prefix over
// the classes is built in LDS (build_device_prefix).
constexpr int kMaxDeviceGroups = NVFP4_MAX_DEVICE_GROUPS;
constexpr int kMaxRowClasses = 4;  // R for the 256-row tiles
constexpr int kMaxDeviceClasses = kMaxRowClasses * kMaxDeviceGroups;
static_assert(kMaxDeviceClasses == 32 * 64, "two-level ballot search over 64 lanes");

struct DeviceGroupArgs {
  const int32_t* sizes;  // [G][4] (m, n, k, l)
  const uint64_t* abc;   // [G][3] addresses of A, B, C
  const uint64_t* sf;    // [G][2] addresses of SFA, SFB
  int32_t* status;       // nullptr, or: number of rejected groups
  int32_t num_groups;
  int32_t grid;
};

// The tables do not change while the kernel runs: reading them through the
// constant address space lets the wave-uniform reads be scalar loads.
template <class T>
__device__ __forceinline__ T load_const(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// Class of the last tile row of a group with m > 0 rows: BM / 64 minus the
// 32-row blocks a wave computes there (0: a full row).
template <int BM>
__host__ __device__ inline int last_row_class(int64_t m) {
  const int64_t rows = m - ((m + BM - 1) / BM - 1) * BM;  // 1 .. BM
  const int64_t amb = ((rows + 31) / 32 + 1) / 2;
  return BM / 64 - (int)amb;
}

template <int BM, int BN>
struct DeviceSrc {
  static constexpr bool kCanSplit = false;
  static constexpr int R = BM / 64;
  static_assert(R >= 1 && R <= kMaxRowClasses, "row classes");
  const DeviceGroupArgs& args;
  const int32_t* prefix;  // LDS: first tile of class c for c = 0 .. R G (prefix[R G] = all tiles)
  __device__ __forceinline__ void prefetch() const {}  // (the classes are in LDS by then)
  __device__ __forceinline__ int grid() const { return args.grid; }
  __device__ __forceinline__ bool split() const { return false; }
  __device__ __forceinline__ int total_tiles() const {
    return __builtin_amdgcn_readfirstlane(prefix[R * args.num_groups]);
  }
  __device__ __forceinline__ int tile_prefix(int c) const { return __builtin_amdgcn_readfirstlane(prefix[c]); }
  // Last class whose first tile is <= tile (the prefix does not decrease, so
  // the entries at or below `tile` are a leading run): one ballot over every
  // 32nd entry, one over the 32 entries of the block it finds. Called with
  // all 64 lanes of the wave active.
  __device__ __forceinline__ int class_of_tile(int tile) const {
    const int nc = R * args.num_groups;
    const int lane = (int)(threadIdx.x & 63);
    const int i0 = lane * 32;
    const bool c0 = i0 < nc && prefix[i0] <= tile;
    const int blk = __popcll(__ballot(c0)) - 1;
    const int i1 = blk * 32 + (lane & 31);
    const bool c1 = lane < 32 && i1 < nc && prefix[i1] <= tile;
    return blk * 32 + __popcll(__ballot(c1)) - 1;
  }
  __device__ __forceinline__ ClassArgs cls(int c) const {
    const int G = args.num_groups;
    const int b = c / G, g = c - b * G;
    ClassArgs r;
    r.m = load_const(args.sizes, 4 * g + 0);
    r.n = load_const(args.sizes, 4 * g + 1);
    r.k = load_const(args.sizes, 4 * g + 2);
    r.l = load_const(args.sizes, 4 * g + 3);
    r.a = reinterpret_cast<const uint8_t*>(load_const(args.abc, 3 * g + 0));
    r.b = reinterpret_cast<const uint8_t*>(load_const(args.abc, 3 * g + 1));
    r.c = reinterpret_cast<uint16_t*>(load_const(args.abc, 3 * g + 2));
    r.sfa = reinterpret_cast<const uint8_t*>(load_const(args.sf, 2 * g + 0));
    r.sfb = reinterpret_cast<const uint8_t*>(load_const(args.sf, 2 * g + 1));
    const int tiles_m = (r.m + BM - 1) / BM;
    const int full = tiles_m - (last_row_class<BM>(r.m) > 0 ? 1 : 0);
    r.tiles_m = b == 0 ? full : tiles_m - full;  // a class with tiles is never empty here
    r.tm0 = b == 0 ? 0 : full;
    r.tiles_n = (r.n + BN - 1) / BN;
    r.nk = (r.k + kBK - 1) / kBK;
    return r;
  }
  __device__ __forceinline__ int nk(int c) const {
    const int g = c % args.num_groups;
    return (load_const(args.sizes, 4 * g + 2) + kBK - 1) / kBK;
  }
};

// KPAD: the instantiation that can meet a k % 64 == 32 group (a tile's last
// stage then needs its scales patched, a check per stage in the mainloop);
// calls without such groups use the one without. MX: the mainloop for scales
// that are all zero or positive powers of two (FP4 MFMA with E8M0 scales, no
// dequantisation).
template <int BM, int BN, int WM, int WN, int NS, class Src, bool KPAD = false, bool MX = false, bool KS2R_ALL = false>
struct GemmKernel {
  static constexpr int MB = WM / 32;
  static constexpr int NB = WN / 32;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int WAVES_M = BM / WM;
  static_assert(WAVES_M == 2, "row-block interleave assumes two wave rows");
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = BN * kRowBytes;
  // Scale atom rows staged per operand: a 64-row (column) tile stages the
  // whole 128-row atom it lies in and uses half of it.
  static constexpr int A_ATOMS = BM >= 128 ? BM / 128 : 1;
  static constexpr int B_ATOMS = BN >= 128 ? BN / 128 : 1;
  static constexpr bool kSubAtomA = BM < 128, kSubAtomB = BN < 128;
  static_assert((BM % 128 == 0 || BM == 64) && (BN % 128 == 0 || BN == 64), "tile shape");
  static constexpr int SF_ATOMS = A_ATOMS + B_ATOMS;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SF_ATOMS * 1024;
  static constexpr int A_INSTR = A_BYTES / 1024 / 4;  // 1 KiB direct loads per wave per stage
  static constexpr int B_INSTR = B_BYTES / 1024 / 4;
  static constexpr int TILE_FLOATS = BM * BN;
  static_assert((BM / WM) * (BN / WN) == kThreads / 64, "four waves per workgroup");
  static_assert(WM <= 128 && WN <= 128 && 128 % WM == 0 && 128 % WN == 0 && WM >= 32 && WN >= 32,
                "wave tile inside one scale atom");
  static_assert(A_INSTR >= 1 && B_INSTR >= 1 && SF_ATOMS <= 4, "tile shape");
  // Direct loads every wave issues per stage: its A and B rows and one scale
  // atom row (waves past the last atom row load nothing into a 1 KiB dummy).
  static constexpr int L = A_INSTR + B_INSTR + 1;
  // Stores every wave issues in an unmasked epilogue (one 16-byte store per
  // lane per run pair of each 32x32 block), all unconditional.
  static constexpr int S = MB * NB * 2;
  static_assert((NS - 1) * L + S < 64, "vmcnt range (counted waits across the epilogue's stores)");
  static constexpr int DUMMY_OFF = NS * STAGE_BYTES;
  static constexpr int FLAG_OFF = DUMMY_OFF + 1024;  // stream-K: a tile's arrival count, shared by the waves
  // Whole-tile f16 kernels that split K over the waves (mainloop_ks) and add
  // the partials through 16 LDS slots of 64 lanes x 8 floats after the
  // stages: the 256x128 ones (light tiles; with KS2R_ALL every tile, fuller
  // ones as 128x128 wave tiles), and the 128x256 ones with KS2R_ALL (every
  // tile). With KS2R_ALL the accumulators are 4 x 4 blocks, else as in the
  // two-by-two layout.
  static constexpr bool kKS256x128 = BM == 256 && BN == 128 && WM == 128 && WN == 64;
  static constexpr bool kKS128x256 = BM == 128 && BN == 256 && WM == 64 && WN == 128;
  static constexpr bool kKS128x128 = BM == 128 && BN == 128 && WM == 64 && WN == 64;
  static constexpr bool kKS = !Src::kCanSplit && !MX && (kKS256x128 || ((kKS128x256 || kKS128x128) && KS2R_ALL));
  static constexpr int EX_OFF = FLAG_OFF + 16;
  static constexpr int EX_BYTES = kKS ? 16 * 2048 : 0;
  static constexpr bool kKS2R = kKS && KS2R_ALL;
  static constexpr int ACC_M = kKS ? 4 : MB, ACC_N = kKS2R ? 4 : NB;
  static constexpr int NCB = BN / 32;       // column blocks of a tile
  static constexpr int CPW = NCB / 4;       // column blocks each wave stores after a K split
  static constexpr int LDS_BYTES = NS * STAGE_BYTES + 1024 + 16 + EX_BYTES;
  static_assert(NS >= 3 && NS <= 4 && LDS_BYTES <= 160 * 1024, "LDS stages");
  static_assert((NS - 2) * L < 64, "vmcnt range");

  // Packed FP4 of one 64-K half stage for this lane (one 16-byte chunk per 32-row
  // block) and the lane's two E4M3 scales per block.
  struct Raw {
    u32x4 a[MB];
    u32x4 b[NB];
    u32x4 sa[(MB + 1) / 2];  // whole scale chunks; this wave's words are picked at conversion
    uint32_t sb[NB];
  };
  struct Scales {
    f16x2 a[MB];
    f16x2 b[NB];
  };
  struct Frags {
    f16x8 a[MB];
    f16x8 b[NB];
  };

  const Src src;
  uint8_t* smem;
  mutable int sub_words = 0;  // TileCtx::sub_words of the segment being computed
  int wave, wm, wn, h, lr, lane;
  int vwg;  // this workgroup's virtual index
  // Row blocks are interleaved over the two wave rows: 32-row block i of wave
  // row wm is block b = 2 i + wm of the tile (rows 32 b .. 32 b + 31), so a
  // ragged M tail leaves both wave rows about the same number of blocks.
  __device__ __forceinline__ static constexpr int row_block(int wm_, int i) { return i * WAVES_M + wm_; }
  // Per-lane byte offsets inside a stage of the lane's first A and B chunk for
  // half kk, and of its 16-byte scale chunks. A row's swizzle depends only on
  // its bits 1..3, so A block i adds exactly i * 64 * kRowBytes and B block j
  // adds j * 32 * kRowBytes. Block b's scales sit in atom b / 4, word b % 4 of
  // the lane's chunk, so this wave's block i is word 2 (i & 1) + wm of the
  // chunk of atom i / 2 (whole chunks are read: 16-byte lane strides are
  // bank-conflict free, 4-byte reads at that stride are not).
  int a_base[2], b_base[2], sa_base, sb_base;
  // v_perm_b32 selector that moves this lane's two A scale bytes (16-blocks
  // 2h, 2h+1) of the word of wave row wm (the second source holds the word of
  // row 0, the first that of row 1) into the low half of the result.
  uint32_t sa_sel;

  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2). The virtual index gives each XCD a contiguous run of indices, hence of
  // tiles (or units), which the raster below turns into compact 2-D blocks.
  __device__ __forceinline__ int virtual_wg(int b) const {
    const int P = src.grid(), q = P / kXcds, r = P % kXcds, x = b % kXcds;
    return x * q + (x < r ? x : r) + b / kXcds;
  }

  __device__ __forceinline__ GemmKernel(const Src& s, uint8_t* sm) : src(s), smem(sm) {
    s.prefetch();
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    wm = wave / WAVES_N;
    wn = wave % WAVES_N;
    h = lane >> 5;
    lr = lane & 31;
    vwg = blockIdx.x < (unsigned)s.grid() ? virtual_wg(blockIdx.x) : 0;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      a_base[kk] = lds_off(row_block(wm, 0) * 32 + lr, kk * 2 + h);
      b_base[kk] = A_BYTES + lds_off(wn * WN + lr, kk * 2 + h);
    }
    sa_base = A_BYTES + B_BYTES + lr * 16;
    sb_base = A_BYTES + B_BYTES + (A_ATOMS + ((wn * WN) >> 7)) * 1024 + lr * 16 + (((wn * WN) & 127) >> 5) * 4;
    sa_sel = (uint32_t)(wm * 4 + 2 * h) | ((uint32_t)(wm * 4 + 2 * h + 1) << 8) | 0x0C0C0000u;
  }

  // ---------------- work decomposition ----------------
  // Tiles are numbered class by class (the persistent scheduler of submission
  // 506336 numbers them group by group; here a group may be two classes, and
  // heavier classes come first). A unit is one 128-K stage of one tile; units
  // are numbered tile by tile.
  __device__ __forceinline__ int class_of_tile(int tile) const { return src.class_of_tile(tile); }
  __device__ __forceinline__ int total_tiles() const { return src.total_tiles(); }
  // stream-K only (the by-value argument block)
  __device__ __forceinline__ int64_t unit_begin(int wg) const { return src.args.wg_unit[wg]; }
  // the workgroup whose unit range holds unit u
  __device__ __forceinline__ int owner_of_unit(int64_t u) const {
    int lo = 0, hi = src.args.grid - 1;  // last workgroup whose range starts at or before u
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (src.args.wg_unit[mid] <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  __device__ __forceinline__ int tile_of_unit(int64_t u, int* stage) const {
    const KernelArgs& args = src.args;
    const int g = search_prefix(args.unit_prefix, args.num_classes, u);
    const int nk = args.cls[g].nk;
    const int local = (int)(u - args.unit_prefix[g]);
    *stage = local % nk;
    return args.tile_prefix[g] + local / nk;
  }

  __device__ __forceinline__ void locate(Segment& s, int64_t u, int64_t u_end) const {
    s.u = u;
    s.sk = true;
    s.valid = u < u_end;
    if (!s.valid) return;
    int stage;
    s.tile = tile_of_unit(u, &stage);
    const int nk = src.nk(class_of_tile(s.tile));
    s.s0 = stage;
    s.s1 = (int)min((int64_t)nk, stage + (u_end - u));
  }

  __device__ __forceinline__ void first_segment(Segment& s) const {
    s.sk = false;
    if constexpr (Src::kCanSplit) {
      if (src.split() && src.args.whole_tiles == 0) {
        locate(s, unit_begin(vwg), unit_begin(vwg + 1));
        return;
      }
    }
    s.u = 0;
    s.tile = vwg;
    s.valid = s.tile < total_tiles();
    s.s0 = 0;
    s.s1 = s.valid ? src.nk(class_of_tile(s.tile)) : 0;
  }

  __device__ __forceinline__ void next_segment(Segment& s) const {
    if constexpr (Src::kCanSplit) {
      if (s.sk) {
        locate(s, s.u + (s.s1 - s.s0), unit_begin(vwg + 1));
        return;
      }
      // after the whole rounds, this workgroup's unit range
      if (src.split() && (int)s.u + 1 >= src.args.whole_tiles / src.grid()) {
        locate(s, unit_begin(vwg), unit_begin(vwg + 1));
        return;
      }
    }
    {
      // Round r hands tiles [r grid, (r + 1) grid) out forwards when r is
      // even and backwards when r is odd: tiles come heaviest first, so the
      // workgroups that drew the lightest tiles of one round draw the
      // heaviest of the next.
      const int r = (int)++s.u;
      const int P = src.grid();
      s.tile = r * P + ((r & 1) ? P - 1 - vwg : vwg);
      s.valid = s.tile < total_tiles();
      s.s0 = 0;
      s.s1 = s.valid ? src.nk(class_of_tile(s.tile)) : 0;
    }
  }

  __device__ __forceinline__ TileCtx setup(int tile) const {
    const int gi = class_of_tile(tile);
    const ClassArgs& G = src.cls(gi);
    const int M = G.m, N = G.n, K = G.k;
    const int tiles_m = G.tiles_m;
    const int per_l = tiles_m * G.tiles_n;
    const int rest = tile - src.tile_prefix(gi);
    const int li = rest / per_l;
    const int r2 = rest - li * per_l;
    // Raster inside the group: super-columns of kRasterWidth n-tiles, taken
    // left to right; inside one, rows of up to kRasterWidth tiles, top to
    // bottom. Consecutive tiles then share A rows and B columns: 32 of them
    // (one XCD's share of a 256-workgroup wave) span 4 A and 8 B panels.
    const int tiles_n = G.tiles_n;
    const int sc = r2 / (tiles_m * kRasterWidth);
    const int in_sc = r2 - sc * tiles_m * kRasterWidth;
    const int width = min(kRasterWidth, tiles_n - sc * kRasterWidth);
    const int tm = G.tm0 + in_sc / width;
    const int tn = sc * kRasterWidth + in_sc % width;
    const int kbytes = K >> 1;
    const int Kt = (K + 63) >> 6;  // scale atoms along K (the last may be half used)
    const int Mt = (M + 127) >> 7;
    const int Nt = (N + 127) >> 7;
    TileCtx t;
    t.M = M;
    t.N = N;
    t.kbytes = kbytes;
    t.nk = G.nk;
    t.kpad_group = (K & 63) ? (K >> 6) & 1 : -1;
    t.row0 = tm * BM;
    t.col0 = tn * BN;
    t.a_tile = G.a + ((size_t)li * M + (size_t)tm * BM) * kbytes;
    t.b_tile = G.b + ((size_t)li * N + (size_t)tn * BN) * kbytes;
    t.a_rem = (M - tm * BM) * kbytes;
    t.b_rem = (N - tn * BN) * kbytes;
    t.c = G.c + (size_t)li * M * N;
    t.sf_row = nullptr;
    t.sf_rem = 0;
    if (wave < A_ATOMS) {
      const int atom = (tm * BM >> 7) + wave;
      t.sf_row = G.sfa + ((size_t)li * Mt + atom) * Kt * kAtomBytes;
      t.sf_rem = atom < Mt ? Kt * kAtomBytes : 0;
    } else if (wave < SF_ATOMS) {
      const int atom = (tn * BN >> 7) + (wave - A_ATOMS);
      t.sf_row = G.sfb + ((size_t)li * Nt + atom) * Kt * kAtomBytes;
      t.sf_rem = atom < Nt ? Kt * kAtomBytes : 0;
    }
    t.sub_words = (kSubAtomA ? ((tm * BM) & 127) >> 5 : 0) | (kSubAtomB ? (((tn * BN) & 127) >> 5) << 4 : 0);
    return t;
  }

  // ---------------- operand staging ----------------
  // Direct loads of stage kt (A, B and the scale atoms) into LDS buffer buf.


  // The loader walks the workgroup's segments ahead of the compute. Global stage
  // X (counted over all segments) lives in LDS buffer X % NS.
  struct Loader {
    Segment seg;
    TileCtx ctx;
    int stage;   // next stage of seg to issue
    int issued;  // stages issued so far
  };

  __device__ __forceinline__ void loader_skip_empty(Loader& ld) const {
    while (ld.seg.valid && ld.seg.s0 == ld.seg.s1) next_segment(ld.seg);  // k = 0 tiles load nothing
    if (ld.seg.valid) {
      ld.ctx = setup(ld.seg.tile);
      ld.stage = ld.seg.s0;
    }
  }

  __device__ __forceinline__ void loader_init(Loader& ld) const {
    first_segment(ld.seg);
    ld.issued = 0;
    loader_skip_empty(ld);
  }

  // Resources and LDS targets of one stage's direct loads; the loads are
  // issued one by one (dma<U>) between the MFMAs of the next half stage.
  struct StageIssue {
    i32x4 ra, rb, rs;  // A, B and scale resources (0 bytes: the loads write zeros)
    uint32_t st;       // LDS address of the stage buffer
    uint32_t sdst;     // LDS address of this wave's scale atom row (or the dummy)
    int voff;          // lane offset of its 16 bytes inside a 1 KiB A or B load
    int ustride;       // bytes between a wave's consecutive A or B loads (64 rows)
  };

  __device__ __forceinline__ static i32x4 uniform(i32x4 r) {
    return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                 __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
  }

  // The loads of the loader's next stage into buffer issued % NS. With no
  // stage left they read 0 bytes and write zeros into that buffer, which
  // every wave has finished reading (it held stage issued - NS).
  __device__ __forceinline__ StageIssue prep_issue(const Loader& ld) const {
    const TileCtx& t = ld.ctx;
    StageIssue si;
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    si.st = lds0 + ((uint32_t)ld.issued % NS) * STAGE_BYTES;
    // Lane -> (row, chunk) of its 16 bytes in a 1 KiB direct load: 16 rows of 64
    // bytes; the physical chunk is lane & 3, the global chunk undoes the swizzle.
    si.voff = (wave * 16 + (lane >> 2)) * t.kbytes + (((lane & 3) ^ swz(lane >> 2)) << 4);
    si.ustride = 64 * t.kbytes;
    // the K offset goes into the resource base, so the range check also
    // zero-fills past the end of the last row
    const bool live = ld.seg.valid;
    const int kb0 = ld.stage * kRowBytes;
    si.ra = uniform(make_rsrc(t.a_tile + kb0, live ? t.a_rem - kb0 : 0));
    si.rb = uniform(make_rsrc(t.b_tile + kb0, live ? t.b_rem - kb0 : 0));
    // two 64-K groups (1 KiB) of this wave's atom row; groups past k read 0
    const int q0 = ld.stage * 2 * kAtomBytes;
    const bool has_sf = wave < SF_ATOMS;
    si.rs = uniform(make_rsrc(t.sf_row + q0, live && has_sf ? t.sf_rem - q0 : 0));
    si.sdst = has_sf ? si.st + A_BYTES + B_BYTES + wave * 1024 : lds0 + DUMMY_OFF;
    return si;
  }

  template <int U>
  __device__ __forceinline__ void dma(const StageIssue& si) const {
    if constexpr (U < A_INSTR) {
      load_lds16(si.ra, si.st + (U * 4 + wave) * 1024, si.voff + U * si.ustride);
    } else if constexpr (U < A_INSTR + B_INSTR) {
      constexpr int V = U - A_INSTR;
      load_lds16(si.rb, si.st + A_BYTES + (V * 4 + wave) * 1024, si.voff + V * si.ustride);
    } else {
      load_lds16(si.rs, si.sdst, lane * 16);
    }
  }

  template <int U0, int U1>
  __device__ __forceinline__ void dma_range(const StageIssue& si) const {
    if constexpr (U0 < U1) {
      dma<U0>(si);
      dma_range<U0 + 1, U1>(si);
    }
  }

  // After a stage was issued: the loader moves to its next stage.
  __device__ __forceinline__ void advance(Loader& ld) const {
    ++ld.issued;
    if (ld.seg.valid && ++ld.stage == ld.seg.s1) {
      next_segment(ld.seg);
      loader_skip_empty(ld);
    }
  }

  __device__ __forceinline__ void issue_all(Loader& ld) const {
    const StageIssue si = prep_issue(ld);
    dma_range<0, L>(si);
    advance(ld);
  }

  // ---------------- dequantisation and MFMA ----------------
  // The compute below is instantiated for AMB = number of this wave's 32-row
  // blocks that hold rows below m (0 .. MB): blocks past m cost no LDS reads,
  // no dequantisation and no MFMAs. A wave with AMB = 0 still issues its share
  // of the loads and joins every barrier.

  // Per-lane LDS offsets of a wave's operands: its first A and B chunk for
  // each half, its B scale words, and the selector of its A scale bytes.
  // The normal layout is the wave's (wm, wn) tile; the wide one (tiles of one
  // row block, see mainloop_rows) gives each wave row block 0 and a quarter
  // of the tile's columns.
  struct Bases {
    int a[2], b[2], sb;
    uint32_t sel;
  };
  __device__ __forceinline__ Bases normal_bases() const {
    return Bases{{a_base[0], a_base[1]}, {b_base[0], b_base[1]}, sb_base, sa_sel};
  }
  static constexpr int WIDE_COLS = BN / 4;
  static constexpr int NBW = WIDE_COLS / 32;  // block columns of a wave in the wide layout
  __device__ __forceinline__ Bases wide_bases() const {
    Bases b;
    const int c0 = wave * WIDE_COLS;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      b.a[kk] = lds_off(lr, kk * 2 + h);
      b.b[kk] = A_BYTES + lds_off(c0 + lr, kk * 2 + h);
    }
    b.sb = A_BYTES + B_BYTES + (A_ATOMS + (c0 >> 7)) * 1024 + lr * 16 + ((c0 & 127) >> 5) * 4;
    b.sel = (uint32_t)(2 * h) | ((uint32_t)(2 * h + 1) << 8) | 0x0C0C0000u;
    return b;
  }

  // ds_reads of one half stage (kk) from LDS buffer buf (NBX block columns).
  template <int AMB, int NBX = NB>
  __device__ __forceinline__ void read_half(Raw& r, int buf, int kk, const Bases& bs) const {
    if (AMB == 0) return;
    const uint8_t* St = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < AMB; ++i)
      r.a[i] = *reinterpret_cast<const u32x4*>(St + bs.a[kk] + i * WAVES_M * 32 * kRowBytes);
#pragma unroll
    for (int j = 0; j < NBX; ++j)
      r.b[j] = *reinterpret_cast<const u32x4*>(St + bs.b[kk] + j * 32 * kRowBytes);
    const int sbo = kSubAtomB ? 4 * (sub_words >> 4) : 0;
    const ScaleVec<NBX> sb = *reinterpret_cast<const ScaleVec<NBX>*>(St + bs.sb + kk * 512 + sbo);
#pragma unroll
    for (int a = 0; a < (AMB + 1) / 2; ++a)
      r.sa[a] = *reinterpret_cast<const u32x4*>(St + sa_base + a * 1024 + kk * 512);
#pragma unroll
    for (int j = 0; j < NBX; ++j) r.sb[j] = sb[j];
  }
  template <int AMB>
  __device__ __forceinline__ void read_half(Raw& r, int buf, int kk) const {
    read_half<AMB, NB>(r, buf, kk, normal_bases());
  }

  // The word of the lane's A scale chunk that holds wave block i's scales,
  // with this lane's two bytes (16-blocks 2h, 2h+1) in the low half: block
  // b = 2 i + wm sits in word b % 4 of atom b / 4, shifted by the tile's
  // sub-atom offset for 64-row tiles.
  __device__ __forceinline__ uint32_t a_scale_word(const Raw& r, int i, uint32_t sel) const {
    const u32x4& c = r.sa[i >> 1];
    if constexpr (kSubAtomA) {
      const bool upper = (sub_words & 15) != 0;  // rows 64..127 of the atom: words 2 and 3
      return __builtin_amdgcn_perm(upper ? c[3] : c[1], upper ? c[2] : c[0], sel);
    }
    return __builtin_amdgcn_perm(c[2 * (i & 1) + 1], c[2 * (i & 1)], sel);
  }
  __device__ __forceinline__ uint32_t a_scale_word(const Raw& r, int i) const { return a_scale_word(r, i, sa_sel); }

  // The lane's two E4M3 scales (16-blocks 2h, 2h+1 of the half) -> f16, exactly.
  template <int AMB, int NBX = NB>
  __device__ __forceinline__ void convert_scales(Scales& s, const Raw& r, uint32_t sel) const {
    if (AMB == 0) return;
    const int hshift = h * 16;
#pragma unroll
    for (int i = 0; i < AMB; ++i) {
      const uint32_t w = a_scale_word(r, i, sel);
      s.a[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    }
#pragma unroll
    for (int j = 0; j < NBX; ++j) s.b[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sb[j] >> hshift, 1.0f, false);
  }

  // Operand fragments of substep S (K elements 8S..8S+7 of the lane's 32).
  template <int S, int AMB, int NBX = NB>
  __device__ __forceinline__ void dequant(Frags& f, const Raw& r, const Scales& s) const {
    if (AMB == 0) return;
#pragma unroll
    for (int i = 0; i < AMB; ++i) f.a[i] = dequant8(r.a[i][S], s.a[i][S >> 1]);
#pragma unroll
    for (int j = 0; j < NBX; ++j) f.b[j] = dequant8(r.b[j][S], s.b[j][S >> 1]);
  }

  template <int AMB, int NBX = NB>
  __device__ __forceinline__ static void mfmas(f32x16 (&acc)[ACC_M][ACC_N], const Frags& f) {
#pragma unroll
    for (int i = 0; i < AMB; ++i)
#pragma unroll
      for (int j = 0; j < NBX; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  }

  // Keeps the fragments and scales of the next substep computed before this
  // point: without it the compiler sinks their conversion past the barrier,
  // next to their first use, where it cannot overlap any MFMA.
  template <int AMB, int NBX = NB>
  __device__ __forceinline__ static void pin(const Frags& f, const Scales& s) {
#pragma unroll
    for (int i = 0; i < AMB; ++i) asm volatile("" ::"v"(f.a[i]), "v"(s.a[i]));
#pragma unroll
    for (int j = 0; j < (AMB ? NBX : 0); ++j) asm volatile("" ::"v"(f.b[j]), "v"(s.b[j]));
  }

  // One substep, in a scheduling region of its own: the MFMAs of `use`
  // interleaved with the dequantisation of the next substep into `fill`
  // (8 VALU per pair of fragments: 4 VALU per MFMA for 128x128 wave tiles).
  // With CONVERT, the next half's scales are converted here as well.
  // Direct loads U0 .. U1-1 of the next stage go first, in a region of their
  // own, so each step hands the memory pipeline a few loads while its MFMAs
  // run (issued all at once, a stage's loads stall every wave behind the
  // address unit).
  template <int NEXT_S, bool CONVERT, int AMB, int U0 = 0, int U1 = 0, int NBX = NB>
  __device__ __forceinline__ void step(f32x16 (&acc)[ACC_M][ACC_N], const Frags& use, Frags& fill, const Raw& src,
                                       Scales& ssrc, uint32_t sel, const StageIssue* si = nullptr) const {
    if constexpr (U0 < U1) {
      dma_range<U0, U1>(*si);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (AMB == 0) return;
    constexpr int VALU = (AMB + NBX) * 8 + (CONVERT ? 2 * (AMB + NBX) : 0);
    constexpr int PER = (VALU + AMB * NBX - 1) / (AMB * NBX > 0 ? AMB * NBX : 1);
    if (CONVERT) convert_scales<AMB, NBX>(ssrc, src, sel);
    dequant<NEXT_S, AMB, NBX>(fill, src, ssrc);
    mfmas<AMB, NBX>(acc, use);
#pragma unroll
    for (int q = 0; q < AMB * NBX; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVALU, PER, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Zeroes the padding 16-blocks of a half-used last scale atom (bytes 2 and
  // 3 of each of its 128 row words) in this wave's atom row of the stage in
  // LDS buffer buf: after this wave's loads of the stage have landed, before
  // the barrier after which every wave reads it. The A and B bytes past k in
  // that stage (the next row's codes, or zeros past the end) are finite, so
  // with zero scales they add exactly nothing.
  __device__ __forceinline__ void zero_half_atom(uint32_t buf, int group) const {
    if (wave >= SF_ATOMS) return;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2* w = reinterpret_cast<u32x2*>(smem + buf * STAGE_BYTES + A_BYTES + B_BYTES + wave * 1024 +
                                        group * kAtomBytes) + lane;
    *w = *w & 0x0000FFFFu;
  }

  // What a segment's mainloop may assume about the vector-memory operations
  // in flight when it starts (vmcnt counts loads and stores, retired in issue
  // order): kPendPrologue - only the NS stages the prologue issued; kPendStores
  // - stages g0 .. g0 + NS - 1, then exactly S epilogue stores (the previous
  // segment ran at least NS stages, so it issued all of them, and ended in an
  // unmasked epilogue); kPendUnknown - anything (wait for all).
  static constexpr int kPendPrologue = 0, kPendStores = 1, kPendUnknown = 2;
  // Only the 128x128-wave-tile kernels overlap the epilogue's stores with the
  // next tile: their epilogue is the longest (all compute units write 128 KiB
  // at once), and in the smaller kernels the extra branch in the loop body
  // measured slower (256x128 tiles, workload 2: +2%).
  static constexpr bool kOverlapStores = MB * NB == 16;

  // Wait until stage g0 of a segment has landed, given `pend`.
  __device__ __forceinline__ static void wait_first_stage(int pend) {
    if (pend == kPendPrologue) wait_vmem<(NS - 1) * L>();
    else if (pend == kPendStores) wait_vmem<(NS - 1) * L + S>();
    else wait_vmem_all();
  }

  // The mid-stage wait of iteration kt (stage g0 + kt + 1 must have landed).
  // The stages after it are exactly NS - 2; with kPendStores the epilogue's S
  // stores sit between them for the first NS - 1 iterations, so they need not
  // have drained: the next tile's MFMAs run while they do.
  __device__ __forceinline__ static void wait_next_stage(int pend, int kt) {
    if constexpr (kOverlapStores) {
      if (pend == kPendStores && kt < NS - 1) {
        wait_vmem<(NS - 2) * L + S>();
        return;
      }
    }
    wait_vmem<(NS - 2) * L>();
  }

  // n stages of one segment, whose first stage is global stage g0. Every
  // iteration issues exactly one stage (L loads per wave), so on entry stages
  // up to g0 + NS - 1 are issued, and at the mid-stage wait of stage g the
  // stages after g + 1 are exactly NS - 2 (plus the epilogue's stores, see
  // wait_next_stage). With KPAD, global stage kpad_g (or none, -1) is a
  // tile's last stage with a half-used scale atom in 64-K group kpad_grp.
  template <int AMB, int NBX = NB>
  __device__ __forceinline__ void mainloop(f32x16 (&acc)[ACC_M][ACC_N], int n, int g0, Loader& ld, int kpad_g,
                                           int kpad_grp, int pend, const Bases& bs) const {
    // split of a stage's L loads over the four steps of a half stage
    constexpr int U1 = (L + 3) / 4, U2 = U1 + (L - U1 + 2) / 3, U3 = U2 + (L - U2 + 1) / 2;
    Raw r0, r1;
    Scales s0, s1;
    Frags f0, f1;
    wait_first_stage(pend);
    if (KPAD && g0 == kpad_g) zero_half_atom((uint32_t)g0 % NS, kpad_grp);
    block_sync();
    read_half<AMB, NBX>(r0, (uint32_t)g0 % NS, 0, bs);
    convert_scales<AMB, NBX>(s0, r0, bs.sel);
    dequant<0, AMB, NBX>(f0, r0, s0);
    for (int kt = 0; kt < n; ++kt) {
      const int g = g0 + kt;
      // ---- first half (K 0..63 of the stage): raw data in r0 ----
      read_half<AMB, NBX>(r1, (uint32_t)g % NS, 1, bs);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, AMB + NBX + 1 + (AMB + 1) / 2, 0);
      step<1, false, AMB, 0, 0, NBX>(acc, f0, f1, r0, s0, bs.sel);
      step<2, false, AMB, 0, 0, NBX>(acc, f1, f0, r0, s0, bs.sel);
      step<3, false, AMB, 0, 0, NBX>(acc, f0, f1, r0, s0, bs.sel);
      step<0, true, AMB, 0, 0, NBX>(acc, f1, f0, r1, s1, bs.sel);
      pin<AMB, NBX>(f0, s1);
      // ---- second half: raw data in r1. Stage g+1 must have landed before its
      // first half is read; every wave is done with stage g's buffer here, so
      // stage g + NS can take it.
      wait_next_stage(pend, kt);
      if (KPAD && g + 1 == kpad_g) zero_half_atom((uint32_t)(g + 1) % NS, kpad_grp);
      block_sync();
      const StageIssue si = prep_issue(ld);
      read_half<AMB, NBX>(r0, (uint32_t)(g + 1) % NS, 0, bs);  // unused after the last stage
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, AMB + NBX + 1 + (AMB + 1) / 2, 0);
      step<1, false, AMB, 0, U1, NBX>(acc, f0, f1, r1, s1, bs.sel, &si);
      step<2, false, AMB, U1, U2, NBX>(acc, f1, f0, r1, s1, bs.sel, &si);
      step<3, false, AMB, U2, U3, NBX>(acc, f0, f1, r1, s1, bs.sel, &si);
      step<0, true, AMB, U3, L, NBX>(acc, f1, f0, r0, s0, bs.sel, &si);
      pin<AMB, NBX>(f0, s0);
      advance(ld);
    }
  }

  // ---------------- the 256x128 whole-tile kernels: the waves split K ----------------
  // In the two-by-two layout each wave dequantises its 4 A and 2 B fragments
  // for every 16-K substep: 6 VALU per MFMA, and light tiles dequantise every
  // B fragment twice for few rows. Here the four waves split the K range of
  // every stage instead, in one of three modes by the tile's row blocks below
  // m (r):
  //  * KS4 (r <= 2; r <= 4 with 4 x 4 accumulator blocks): wave w takes
  //    substeps 2 (w % 2), 2 (w % 2) + 1 of half w / 2 of every stage, for
  //    all r row blocks and all 4 column blocks;
  //  * KS2C (r = 3, 4 with 4 x 2 accumulator blocks): wave w takes half
  //    w % 2 of every stage, for all r row blocks and the 2 column blocks
  //    2 (w / 2), 2 (w / 2) + 1;
  //  * KS2R (r >= 5, only in the kernels that split every tile, KS2R_ALL;
  //    the others keep the two-by-two layout there): wave w takes half w % 2
  //    of every stage, for row blocks w / 2, w / 2 + 2, ... (as in the
  //    two-by-two layout) and all 4 column blocks: 128x128 wave tiles, 4 VALU
  //    per MFMA.
  // Per stage a wave dequantises 80-256 VALU where the two-by-two layout
  // needs 128-384, for the same MFMAs. At the end of the tile the partials of
  // each 32x32 block are added through LDS, in the order of their K parts, so
  // results are deterministic (and differ from the other layouts' in the last
  // bits only). The wave's partial of row block i, column block j is
  // acc_at(acc, i, j).
  enum { KS4 = 0, KS2C = 1, KS2R = 2 };
  template <int MODE>
  struct KsShape {
    static constexpr int KS = MODE == KS4 ? 4 : 2;
    static constexpr int P = 8 / KS;                          // substeps per stage per wave
    static constexpr int NBK = MODE == KS2C ? NCB / 2 : NCB;  // column blocks per wave
  };
  __device__ __forceinline__ bool ks_tile(const TileCtx& t) const { return kKS && (kKS2R || t.M - t.row0 <= 128); }
  // Block (i, j) of a wave's partials (NBK column blocks): when a row block's
  // NBK blocks do not fit a row of the accumulator array, block (i, j) is
  // element i NBK + j of it in row-major order (KS4 with 4 x 2 accumulators:
  // acc[2 i][0..1], acc[2 i + 1][0..1]).
  template <int NBK>
  __device__ __forceinline__ static f32x16& acc_at(f32x16 (&acc)[ACC_M][ACC_N], int i, int j) {
    if constexpr (NBK <= ACC_N) return acc[i][j];
    else return acc[(i * NBK + j) / ACC_N][(i * NBK + j) % ACC_N];
  }
  template <int NBK>
  __device__ __forceinline__ static const f32x16& acc_at(const f32x16 (&acc)[ACC_M][ACC_N], int i, int j) {
    if constexpr (NBK <= ACC_N) return acc[i][j];
    else return acc[(i * NBK + j) / ACC_N][(i * NBK + j) % ACC_N];
  }
  __device__ __forceinline__ int ks_rows(const TileCtx& t) const {
    const int rows = t.M - t.row0;
    return rows >= BM ? BM / 32 : (rows + 31) >> 5;
  }

  // A wave's operands for its P substeps of a stage: P dwords of each of its
  // R A chunks and NBK B chunks, and the scale words.
  template <int R, int NBK, int P>
  struct KsRaw {
    typedef uint32_t chunk __attribute__((ext_vector_type(P)));
    chunk a[R];
    chunk b[NBK];
    uint32_t sa[R];
    uint32_t sb[NBK];
  };
  template <int R, int NBK>
  struct KsScales {
    f16x2 a[R];
    f16x2 b[NBK];
  };
  template <int R, int NBK>
  struct KsFrags {
    f16x8 a[R];
    f16x8 b[NBK];
  };
  // Per-lane LDS offsets of a wave's first A and B chunk (8 bytes into the
  // chunk for the second substep pair of KS4), of its A scale chunk(s) and B
  // scale words inside a stage; the shift that brings the lane's scale bytes
  // (two 16-blocks, or KS4's one) to the bottom of a word; and, for KS2R, the
  // wave's word in each A scale chunk (row blocks rpart + 2i sit in atom
  // i / 2, word rpart + 2 (i % 2)).
  struct KsBases {
    int a, b, sa, sb, shift, rpart;
  };
  template <int MODE>
  __device__ __forceinline__ KsBases ks_bases() const {
    constexpr int KS = KsShape<MODE>::KS;
    const int kpart = wave % KS, npart = wave / KS;
    const int kk = KS == 2 ? kpart : kpart >> 1;
    const int sub = KS == 4 ? (kpart & 1) : 0;
    const int c0 = MODE == KS2C ? npart * (BN / 2) : 0;
    const int r0 = MODE == KS2R ? npart * 32 : 0;
    KsBases b;
    b.a = lds_off(r0 + lr, kk * 2 + h) + sub * 8;
    b.b = A_BYTES + lds_off(c0 + lr, kk * 2 + h) + sub * 8;
    b.sa = A_BYTES + B_BYTES + lr * 16 + kk * 512;
    b.sb = A_BYTES + B_BYTES + (A_ATOMS + (c0 >> 7)) * 1024 + lr * 16 + ((c0 & 127) >> 5) * 4 + kk * 512;
    b.shift = h * 16 + sub * 8;
    b.rpart = MODE == KS2R ? npart : 0;
    return b;
  }
  template <int MODE, int R, int NBK, int P>
  __device__ __forceinline__ void ks_read(KsRaw<R, NBK, P>& r, int buf, const KsBases& bs) const {
    typedef typename KsRaw<R, NBK, P>::chunk chunk;
    constexpr int AS = MODE == KS2R ? 64 : 32;  // rows between the wave's A blocks
    const uint8_t* St = smem + buf * STAGE_BYTES;
    if constexpr (kKsScalesFirst) ks_read_scales<MODE>(r, St, bs);
#pragma unroll
    for (int i = 0; i < R; ++i) r.a[i] = *reinterpret_cast<const chunk*>(St + bs.a + i * AS * kRowBytes);
#pragma unroll
    for (int j = 0; j < NBK; ++j) r.b[j] = *reinterpret_cast<const chunk*>(St + bs.b + j * 32 * kRowBytes);
    if constexpr (!kKsScalesFirst) ks_read_scales<MODE>(r, St, bs);
  }
  // The scale words of ks_read. The 128x128 kernels read them before the
  // operand chunks: they are converted before the first fragment is
  // dequantised and LDS reads complete in issue order, so the conversion
  // then waits for them alone (2-3% faster on long-K MoE shapes). The
  // 256x128 kernels measured up to 4% slower that way, the 128x256 ones
  // within +-1.5%: they read them last.
  static constexpr bool kKsScalesFirst = BM == 128 && BN == 128;
  template <int MODE, int R, int NBK, int P>
  __device__ __forceinline__ void ks_read_scales(KsRaw<R, NBK, P>& r, const uint8_t* St, const KsBases& bs) const {
    if constexpr (MODE == KS2R) {
#pragma unroll
      for (int a = 0; a < (R + 1) / 2; ++a) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(St + bs.sa + a * 1024);
        r.sa[2 * a] = bs.rpart ? c[1] : c[0];
        if (2 * a + 1 < R) r.sa[2 * a + 1] = bs.rpart ? c[3] : c[2];
      }
    } else {
      const u32x4 c = *reinterpret_cast<const u32x4*>(St + bs.sa);
#pragma unroll
      for (int i = 0; i < R; ++i) r.sa[i] = c[i];
    }
    // (at most four words per 128-column scale atom; the next atom row is 1 KiB on)
    constexpr int NW = NBK < 4 ? NBK : 4;
#pragma unroll
    for (int a = 0; a < NBK / NW; ++a) {
      const ScaleVec<NW> cb = *reinterpret_cast<const ScaleVec<NW>*>(St + bs.sb + a * 1024);
#pragma unroll
      for (int j = 0; j < NW; ++j) r.sb[a * NW + j] = cb[j];
    }
  }
  template <int R, int NBK, int P>
  __device__ __forceinline__ static void ks_convert(KsScales<R, NBK>& s, const KsRaw<R, NBK, P>& r, int shift) {
#pragma unroll
    for (int i = 0; i < R; ++i) s.a[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sa[i] >> shift, 1.0f, false);
#pragma unroll
    for (int j = 0; j < NBK; ++j) s.b[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sb[j] >> shift, 1.0f, false);
  }
  // Substep PS of the wave's P: dword PS of each chunk, under the scale of its
  // 16-block (P = 2: the wave's one 16-block).
  template <int PS, int R, int NBK, int P>
  __device__ __forceinline__ static void ks_dequant(KsFrags<R, NBK>& f, const KsRaw<R, NBK, P>& r,
                                                    const KsScales<R, NBK>& s) {
    constexpr int SI = P == 4 ? (PS >> 1) : 0;
#pragma unroll
    for (int i = 0; i < R; ++i) f.a[i] = dequant8(r.a[i][PS], s.a[i][SI]);
#pragma unroll
    for (int j = 0; j < NBK; ++j) f.b[j] = dequant8(r.b[j][PS], s.b[j][SI]);
  }
  template <int R, int NBK>
  __device__ __forceinline__ static void ks_mfmas(f32x16 (&acc)[ACC_M][ACC_N], const KsFrags<R, NBK>& f) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < NBK; ++j) {
        f32x16& c = acc_at<NBK>(acc, i, j);
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], c, 0, 0, 0);
      }
  }
  template <int R, int NBK>
  __device__ __forceinline__ static void ks_pin(const KsFrags<R, NBK>& f, const KsScales<R, NBK>& s) {
#pragma unroll
    for (int i = 0; i < R; ++i) asm volatile("" ::"v"(f.a[i]), "v"(s.a[i]));
#pragma unroll
    for (int j = 0; j < NBK; ++j) asm volatile("" ::"v"(f.b[j]), "v"(s.b[j]));
  }
  // One substep (as step): the MFMAs of `use` with the dequantisation of the
  // wave's substep NEXT of `src` into `fill` (and, with CONVERT, first the
  // conversion of src's scales), after direct loads U0 .. U1-1.
  template <int NEXT, bool CONVERT, int U0, int U1, int R, int NBK, int P>
  __device__ __forceinline__ void ks_step(f32x16 (&acc)[ACC_M][ACC_N], const KsFrags<R, NBK>& use,
                                          KsFrags<R, NBK>& fill, const KsRaw<R, NBK, P>& src, KsScales<R, NBK>& ssrc,
                                          int shift, const StageIssue* si) const {
    if constexpr (U0 < U1) {
      dma_range<U0, U1>(*si);
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int VALU = (R + NBK) * 8 + (CONVERT ? 2 * (R + NBK) : 0);
    constexpr int PER = (VALU + R * NBK - 1) / (R * NBK);
    if (CONVERT) ks_convert(ssrc, src, shift);
    ks_dequant<NEXT>(fill, src, ssrc);
    ks_mfmas(acc, use);
#pragma unroll
    for (int q = 0; q < R * NBK; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVALU, PER, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // Stage g of a segment (iteration kt) from the raw operands r, whose
  // substep 0 is dequantised in f0. All but the last of the wave's substeps
  // run before the mid-stage barrier, so r is free by then and takes stage
  // g + 1 (no second register set, no copies); the last substep's MFMAs then
  // cover the reads, the stage's direct loads and stage g + 1's first
  // dequantisation into f0. The same waits, barrier and loads per stage as
  // mainloop.
  template <int MODE, int R, int NBK, int P>
  __device__ __forceinline__ void ks_stage(f32x16 (&acc)[ACC_M][ACC_N], KsRaw<R, NBK, P>& r, KsScales<R, NBK>& s,
                                           KsFrags<R, NBK>& f0, KsFrags<R, NBK>& f1, const KsBases& bs, int g, int kt,
                                           Loader& ld, int kpad_g, int kpad_grp, int pend) const {
    if constexpr (P == 4) {
      ks_step<1, false, 0, 0>(acc, f0, f1, r, s, bs.shift, nullptr);
      ks_step<2, false, 0, 0>(acc, f1, f0, r, s, bs.shift, nullptr);
      ks_step<3, false, 0, 0>(acc, f0, f1, r, s, bs.shift, nullptr);
    } else {
      ks_step<1, false, 0, 0>(acc, f0, f1, r, s, bs.shift, nullptr);
    }
    ks_pin(f1, s);
    wait_next_stage(pend, kt);
    if (KPAD && g + 1 == kpad_g) zero_half_atom((uint32_t)(g + 1) % NS, kpad_grp);
    block_sync();
    const StageIssue si = prep_issue(ld);
    ks_read<MODE>(r, (uint32_t)(g + 1) % NS, bs);  // unused after the last stage
    if constexpr (kKsScalesFirst) {  // the scale reads, then the operand chunks
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, (NBK + 3) / 4 + (MODE == KS2R ? (R + 1) / 2 : 1), 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, R + NBK, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead,
                                           R + NBK + (NBK + 3) / 4 + (MODE == KS2R ? (R + 1) / 2 : 1), 0);
    }
    ks_step<0, true, 0, L>(acc, f1, f0, r, s, bs.shift, &si);
    ks_pin(f0, s);
    advance(ld);
  }
  // n stages of a segment in mode MODE, R (1 .. 4) row blocks for this wave.
  template <int MODE, int R>
  __device__ __forceinline__ void mainloop_ks(f32x16 (&acc)[ACC_M][ACC_N], int n, int g0, Loader& ld, int kpad_g,
                                              int kpad_grp, int pend) const {
    constexpr int NBK = KsShape<MODE>::NBK, P = KsShape<MODE>::P;
    static_assert(NBK <= ACC_N ? R <= ACC_M : R * NBK <= ACC_M * ACC_N, "partials fit the accumulators");
    const KsBases bs = ks_bases<MODE>();
    KsRaw<R, NBK, P> r;
    KsScales<R, NBK> s;
    KsFrags<R, NBK> f0, f1;
    wait_first_stage(pend);
    if (KPAD && g0 == kpad_g) zero_half_atom((uint32_t)g0 % NS, kpad_grp);
    block_sync();
    ks_read<MODE>(r, (uint32_t)g0 % NS, bs);
    ks_convert(s, r, bs.shift);
    ks_dequant<0>(f0, r, s);
    for (int kt = 0; kt < n; ++kt) ks_stage<MODE>(acc, r, s, f0, f1, bs, g0 + kt, kt, ld, kpad_g, kpad_grp, pend);
  }
  // KS4 when its R x NCB partial blocks fit the accumulators, else KS2C.
  template <int R>
  static constexpr int ks_light_mode() { return R * NCB <= ACC_M * ACC_N ? KS4 : KS2C; }
  template <int R>
  __device__ __forceinline__ void ks_mode34(f32x16 (&acc)[ACC_M][ACC_N], int n, int g0, Loader& ld, int kpad_g,
                                            int kpad_grp, int pend) const {
    mainloop_ks<ks_light_mode<R>(), R>(acc, n, g0, ld, kpad_g, kpad_grp, pend);
  }
  // Mode and this wave's row blocks for a tile with r row blocks below m.
  __device__ __forceinline__ void mainloop_ks_rows(f32x16 (&acc)[ACC_M][ACC_N], int r, int n, int g0, Loader& ld,
                                                   int kpad_g, int kpad_grp, int pend) const {
    switch (r) {
      case 1: ks_mode34<1>(acc, n, g0, ld, kpad_g, kpad_grp, pend); return;
      case 2: ks_mode34<2>(acc, n, g0, ld, kpad_g, kpad_grp, pend); return;
      // (with 4 x 4 accumulator blocks KS4 holds up to four row blocks: a
      // quarter of the substeps costs (r + 4) 16 VALU per stage, one half
      // (r + 2) 32)
      case 3: ks_mode34<3>(acc, n, g0, ld, kpad_g, kpad_grp, pend); return;
      case 4: ks_mode34<4>(acc, n, g0, ld, kpad_g, kpad_grp, pend); return;
      default: break;
    }
    if constexpr (kKS2R && BM == 256) {
      switch ((r - wave / 2 + 1) >> 1) {  // KS2R: row blocks w / 2, w / 2 + 2, ... below m
        case 2: mainloop_ks<KS2R, 2>(acc, n, g0, ld, kpad_g, kpad_grp, pend); return;
        case 3: mainloop_ks<KS2R, 3>(acc, n, g0, ld, kpad_g, kpad_grp, pend); return;
        default: mainloop_ks<KS2R, 4>(acc, n, g0, ld, kpad_g, kpad_grp, pend); return;
      }
    }
  }

  // The end of a tile in modes KS4 and KS2C: wave o stores column blocks
  // CPW o .. CPW o + CPW - 1. For each row block i, each of its column blocks
  // q and each half p of the lane's 16 accumulator elements (one 16-column
  // store run pair), every wave writes its partials of the blocks in that
  // position into LDS slot (o, kp) - o the wave that stores the block, kp
  // the writer's K part - and after a barrier each wave adds the KS partials
  // of its own block in K-part order and stores them. Two barriers per round;
  // the slots lie past the stages (which already hold the next tile's loads).
  template <int MODE, int R>
  __device__ __forceinline__ void epilogue_ks(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t) const {
    constexpr int KS = KsShape<MODE>::KS, NBK = KsShape<MODE>::NBK;
    const int kpart = wave % KS, npart = wave / KS;
    const int base = MODE == KS2C ? npart * NBK : 0;  // the wave's first column block (a multiple of CPW)
    int lro = lr, h8 = h * 8;
    asm volatile("" : "+v"(lro), "+v"(h8));
    const int col0 = t.col0 + wave * CPW * 32;
    typedef __attribute__((address_space(1))) uint16_t gu16;
    gu16* crow = (gu16*)t.c + (size_t)(t.row0 + lro) * t.N + col0 + h8;
    // slot (o, kp): 2 x 64 lanes x 16 bytes at EX_OFF + (o * 4 + kp) * 2048
    f32x4* wr = reinterpret_cast<f32x4*>(smem + EX_OFF) + ((base / CPW) * 4 + kpart) * 128 + lane;
    const f32x4* rd = reinterpret_cast<const f32x4*>(smem + EX_OFF) + wave * 4 * 128 + lane;
#pragma unroll
    for (int i = 0; i < R; ++i) {
#pragma unroll
      for (int q = 0; q < CPW; ++q) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          // local column block j is block (base + j) % CPW of wave (base + j) / CPW
#pragma unroll
          for (int j = q; j < NBK; j += CPW) {
            wr[(j / CPW) * 4 * 128] = acc_quad(acc_at<NBK>(acc, i, j), 8 * p);
            wr[(j / CPW) * 4 * 128 + 64] = acc_quad(acc_at<NBK>(acc, i, j), 8 * p + 4);
          }
          block_sync();
          f32x4 sum0 = rd[0], sum1 = rd[64];
#pragma unroll
          for (int kp = 1; kp < KS; ++kp) {
            sum0 += rd[kp * 128];
            sum1 += rd[kp * 128 + 64];
          }
          const int cu = q * 32 + 16 * p;
          store_run(sum0, sum1, crow + (size_t)i * 32 * t.N + cu,
                    lro < t.M - t.row0 - i * 32 && h8 < t.N - col0 - cu);
          block_sync();  // the slots are rewritten next round
        }
      }
    }
  }
  // The end of a KS2R tile: the waves of K parts 0 and 1 with the same row
  // blocks pair up; wave kp stores column blocks 2 kp, 2 kp + 1 of them. Per
  // round (one row block of the wave, four for every wave, so the barriers
  // match) each wave writes its partials of its partner's two column blocks
  // (2 halves each) into the partner's four slots, and adds the partner's
  // into its own in K-part order.
  template <int R>
  __device__ __forceinline__ void epilogue_ks2r(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t) const {
    const int kpart = wave & 1, rpart = wave >> 1;
    int lro = lr, h8 = h * 8;
    asm volatile("" : "+v"(lro), "+v"(h8));
    const int col0 = t.col0 + kpart * 64;
    typedef __attribute__((address_space(1))) uint16_t gu16;
    gu16* crow = (gu16*)t.c + (size_t)(t.row0 + rpart * 32 + lro) * t.N + col0 + h8;
    f32x4* wr = reinterpret_cast<f32x4*>(smem + EX_OFF) + (wave ^ 1) * 4 * 128 + lane;
    const f32x4* rd = reinterpret_cast<const f32x4*>(smem + EX_OFF) + wave * 4 * 128 + lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < R) {
        // slot q = jl * 2 + p of the partner: its column block 2 (1 - kpart) + jl, half p
#pragma unroll
        for (int jl = 0; jl < 2; ++jl)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            // (values, not a reference, are selected: a reference picked at
            // run time would put the accumulators in memory)
            const f32x4 q0 = kpart ? acc_quad(acc[i][jl], 8 * p) : acc_quad(acc[i][2 + jl], 8 * p);
            const f32x4 q1 = kpart ? acc_quad(acc[i][jl], 8 * p + 4) : acc_quad(acc[i][2 + jl], 8 * p + 4);
            wr[(jl * 2 + p) * 128] = q0;
            wr[(jl * 2 + p) * 128 + 64] = q1;
          }
      }
      block_sync();
      if (i < R) {
        const int rb = rpart + 2 * i;
#pragma unroll
        for (int jl = 0; jl < 2; ++jl)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const f32x4 o0 = rd[(jl * 2 + p) * 128], o1 = rd[(jl * 2 + p) * 128 + 64];
            const f32x4 m0 = kpart ? acc_quad(acc[i][2 + jl], 8 * p) : acc_quad(acc[i][jl], 8 * p);
            const f32x4 m1 = kpart ? acc_quad(acc[i][2 + jl], 8 * p + 4) : acc_quad(acc[i][jl], 8 * p + 4);
            // K part 0's partial first
            const f32x4 sum0 = kpart ? o0 + m0 : m0 + o0, sum1 = kpart ? o1 + m1 : m1 + o1;
            const int cu = jl * 32 + 16 * p;
            store_run(sum0, sum1, crow + (size_t)i * 64 * t.N + cu,
                      lro < t.M - t.row0 - rb * 32 && h8 < t.N - col0 - cu);
          }
      }
      block_sync();
    }
  }
  __device__ __forceinline__ static f32x4 acc_quad(const f32x16& c, int e) {
    return f32x4{acc_read(c[e]), acc_read(c[e + 1]), acc_read(c[e + 2]), acc_read(c[e + 3])};
  }
  // One lane's run pair of a block row (elements 8p .. 8p + 7 as two quads)
  // to 8 consecutive fp16 columns, as in epilogue_impl.
  __device__ __forceinline__ static void store_run(const f32x4& q0, const f32x4& q1,
                                                   __attribute__((address_space(1))) uint16_t* dst, bool ok) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(pack_f16(q0[0], q0[1]), pack_f16(q1[0], q1[1]), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pack_f16(q0[2], q0[3]), pack_f16(q1[2], q1[3]), false, false);
    if (ok) {
      const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
      *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(dst) = v;
    }
  }
  __device__ __forceinline__ void epilogue_ks_rows(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t) const {
    const int r = ks_rows(t);
    switch (r) {
      case 1: epilogue_ks<ks_light_mode<1>(), 1>(acc, t); return;
      case 2: epilogue_ks<ks_light_mode<2>(), 2>(acc, t); return;
      case 3: epilogue_ks<ks_light_mode<3>(), 3>(acc, t); return;
      case 4: epilogue_ks<ks_light_mode<4>(), 4>(acc, t); return;
      default: break;
    }
    if constexpr (kKS2R && BM == 256) {
      switch ((r - wave / 2 + 1) >> 1) {
        case 2: epilogue_ks2r<2>(acc, t); return;
        case 3: epilogue_ks2r<3>(acc, t); return;
        default: epilogue_ks2r<4>(acc, t); return;
      }
    }
  }

  // ---------------- power-of-two scales: FP4 MFMA with E8M0 scales ----------------
  // v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands: lane l of an operand
  // holds 32 codes (four dwords, low nibble first) of row l % 32 at K
  // 32 (l / 32) .. +31 of the instruction, and one E8M0 scale for all 32 of
  // them (checked on the MI355X); the result has the layout of the f16 MFMA.
  // A lane's 16-byte chunk of a half stage spans two 16-blocks (2h, 2h+1),
  // each with its own scale, so a block pair (i, j) takes two passes: pass p
  // feeds the B chunk whole and the A chunk with only 16-block 2h + p (zeros
  // in the other 16 K), with that 16-block's scales. An E4M3 scale that is
  // a positive power of two is an E8M0 scale exactly, so every product is
  // exact as in the f16 path. A zero scale becomes 2^-127: with a zero on
  // both sides (the padding past k) the products vanish below fp32's range;
  // with one zero side they stay below 2^-100, so they change no fp16 result
  // (the other terms are multiples of 2^-20), except that an exact zero sum
  // may come out as -0.
  struct MxScales {
    uint32_t a[MB];  // bytes 1 and 3: E8M0 of 16-blocks 2h and 2h+1 of the lane's row
    uint32_t b[NB];
  };

  // E4M3 scales in bytes 0 and 1 of w -> two bf16 (exact), shifted left by
  // one bit: bytes 1 and 3 are then the bf16 exponent fields, the E8M0 codes
  // of zero and of positive powers of two. The bf16 bits are OR-ed into
  // `seen`; a sign or mantissa bit there marks a scale outside that set.
  __device__ __forceinline__ static uint32_t e8m0_pair(uint32_t w, uint32_t& seen) {
    const uint32_t x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    seen |= x;
    return x << 1;
  }

  template <int AMB>
  __device__ __forceinline__ void mx_scales(MxScales& s, const Raw& r, uint32_t& seen) const {
    const int hshift = h * 16;
#pragma unroll
    for (int i = 0; i < AMB; ++i) s.a[i] = e8m0_pair(a_scale_word(r, i), seen);
#pragma unroll
    for (int j = 0; j < NB; ++j) s.b[j] = e8m0_pair(r.sb[j] >> hshift, seen);
  }

  // Operands of a half stage's first pass, prepared during the half before:
  // the A operands (the chunk's first 16-block, zeros above) and the scales.
  struct MxOps {
    u32x4 t[MB];
    MxScales s;
  };

  // Each A operand goes through an empty asm: built straight from the loaded
  // chunk, the compiler reassembles its dwords byte by byte.
  template <int AMB>
  __device__ __forceinline__ static void mx_pass0_operands(u32x4 (&t)[MB], const Raw& r) {
#pragma unroll
    for (int i = 0; i < AMB; ++i) {
      t[i] = u32x4{r.a[i][0], r.a[i][1], 0u, 0u};
      asm volatile("" : "+v"(t[i]));
    }
  }
  // ... and zeros, then the second 16-block (in the chunk's own registers).
  template <int AMB>
  __device__ __forceinline__ static void mx_pass1_operands(u32x4 (&t)[MB], const Raw& r) {
#pragma unroll
    for (int i = 0; i < AMB; ++i) {
      t[i] = u32x4{0u, 0u, r.a[i][2], r.a[i][3]};
      asm volatile("" : "+v"(t[i]));
    }
  }

  // One quarter of a half stage: pass P over block columns [J0, J1) with A
  // operands ta, after direct loads U0 .. U1-1 of the next stage (in a region
  // of their own, as in the f16 steps); the VALU work `work` emits (VALU
  // instructions, about) is spread between the MFMAs.
  template <int P, int J0, int J1, int AMB, int U0, int U1, int VALU, class Work>
  __device__ __forceinline__ void mx_sub(f32x16 (&acc)[ACC_M][ACC_N], const u32x4 (&ta)[MB], const Raw& r,
                                         const MxScales& s, const StageIssue* si, Work&& work) const {
    if constexpr (U0 < U1) {
      dma_range<U0, U1>(*si);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (AMB == 0) return;
    work();
#pragma unroll
    for (int i = 0; i < AMB; ++i) {
      const i32x8 a = {(int)ta[i][0], (int)ta[i][1], (int)ta[i][2], (int)ta[i][3], 0, 0, 0, 0};
#pragma unroll
      for (int j = J0; j < J1; ++j) {
        const i32x8 b = {(int)r.b[j][0], (int)r.b[j][1], (int)r.b[j][2], (int)r.b[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[i][j], 4, 4, 2 * P + 1, (int)s.b[j],
                                                                    2 * P + 1, (int)s.a[i]);
      }
    }
    constexpr int N = AMB * (J1 - J0);
    constexpr int PER = (VALU + N - 1) / (N > 0 ? N : 1);
#pragma unroll
    for (int q = 0; q < N; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      if constexpr (PER > 0) __builtin_amdgcn_sched_group_barrier(kSchedVALU, PER, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // One half stage on `cur` with its prepared operands `o`, in four quarters
  // (the second pass starts after AMB * NB independent MFMAs), with the next
  // stage's L direct loads spread over the quarters when ISSUE. Meanwhile the
  // next half's operands `no` are prepared from `nxt` (whose LDS reads were
  // issued before this half), so that after the barrier its MFMAs start at
  // once.
  template <int AMB, bool ISSUE>
  __device__ __forceinline__ void mx_half(f32x16 (&acc)[ACC_M][ACC_N], const Raw& cur, const MxOps& o, const Raw& nxt,
                                          MxOps& no, uint32_t& seen, const StageIssue* si) const {
    constexpr int U1 = ISSUE ? (L + 3) / 4 : 0, U2 = ISSUE ? U1 + (L - U1 + 2) / 3 : 0;
    constexpr int U3 = ISSUE ? U2 + (L - U2 + 1) / 2 : 0, U4 = ISSUE ? L : 0;
    constexpr int JH = NB / 2;
    u32x4 t1[MB];
    mx_sub<0, 0, JH, AMB, 0, U1, 2 * AMB>(acc, o.t, cur, o.s, si, [&] { mx_pass1_operands<AMB>(t1, cur); });
    mx_sub<0, JH, NB, AMB, U1, U2, 4 * (AMB + NB)>(acc, o.t, cur, o.s, si,
                                                   [&] { if (AMB > 0) mx_scales<AMB>(no.s, nxt, seen); });
    mx_sub<1, 0, JH, AMB, U2, U3, 3 * AMB>(acc, t1, cur, o.s, si, [&] { mx_pass0_operands<AMB>(no.t, nxt); });
    mx_sub<1, JH, NB, AMB, U3, U4, 0>(acc, t1, cur, o.s, si, [] {});
    // The next operands and this half's MFMAs stay before what follows (the
    // barrier): sunk past it, they would keep two halves' chunks live at once
    // and delay the next MFMAs.
#pragma unroll
    for (int i = 0; i < AMB; ++i) asm volatile("" ::"v"(no.t[i]), "v"(no.s.a[i]));
#pragma unroll
    for (int j = 0; j < (AMB ? NB : 0); ++j) asm volatile("" ::"v"(no.s.b[j]));
#pragma unroll
    for (int i = 0; i < AMB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) asm volatile("" : "+a"(acc[i][j]));
  }

  // The MX counterpart of mainloop: the same stages, waits, barriers and
  // direct loads; a half stage's raw chunks feed the MFMAs directly.
  template <int AMB>
  __device__ __forceinline__ void mainloop_mx(f32x16 (&acc)[ACC_M][ACC_N], int n, int g0, Loader& ld, int kpad_g,
                                              int kpad_grp, uint32_t& seen, int pend) const {
    static_assert(NB % 2 == 0 || NB == 1, "two block-column parts per pass (one: the first part is empty)");
    Raw r0, r1;
    MxOps o0, o1;
    // The loader's sizes are used here, so that any reload of them from the
    // spill area (after the epilogue, where register pressure peaks) comes
    // before the wait below; a reload first waited for inside the loop costs
    // a wait for every direct load in flight at each stage.
    asm volatile("" : "+v"(ld.ctx.a_rem), "+v"(ld.ctx.b_rem), "+v"(ld.ctx.sf_rem), "+v"(ld.ctx.kbytes));
    wait_first_stage(pend);
    if (KPAD && g0 == kpad_g) zero_half_atom((uint32_t)g0 % NS, kpad_grp);
    block_sync();
    read_half<AMB>(r0, (uint32_t)g0 % NS, 0);
    if (AMB > 0) mx_scales<AMB>(o0.s, r0, seen);
    mx_pass0_operands<AMB>(o0.t, r0);
    for (int kt = 0; kt < n; ++kt) {
      const int g = g0 + kt;
      read_half<AMB>(r1, (uint32_t)g % NS, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, AMB + NB + 1 + (AMB + 1) / 2, 0);
      mx_half<AMB, false>(acc, r0, o0, r1, o1, seen, nullptr);
      wait_next_stage(pend, kt);
      if (KPAD && g + 1 == kpad_g) zero_half_atom((uint32_t)(g + 1) % NS, kpad_grp);
      block_sync();
      const StageIssue si = prep_issue(ld);
      read_half<AMB>(r0, (uint32_t)(g + 1) % NS, 0);  // unused after the last stage
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, AMB + NB + 1 + (AMB + 1) / 2, 0);
      mx_half<AMB, true>(acc, r1, o1, r0, o0, seen, &si);
      advance(ld);
    }
  }

  // This wave's 32-row blocks that hold rows below m (0 .. MB).
  __device__ __forceinline__ int active_blocks(const TileCtx& t) const {
    const int rows = t.M - t.row0;
    const int nb = rows <= 0 ? 0 : (rows + 31) >> 5;  // row blocks of the tile below m
    return nb <= wm ? 0 : min(MB, (nb - wm + 1) >> 1);
  }

  __device__ __forceinline__ void mainloop_rows_mx(f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t, int n, int g0,
                                                   Loader& ld, int kpad_g, uint32_t& seen, int pend) const {
    switch (active_blocks(t)) {
      case 0: mainloop_mx<0>(acc, n, g0, ld, kpad_g, t.kpad_group, seen, pend); break;
      case 1: mainloop_mx<(MB >= 1 ? 1 : MB)>(acc, n, g0, ld, kpad_g, t.kpad_group, seen, pend); break;
      case 2: mainloop_mx<(MB >= 2 ? 2 : MB)>(acc, n, g0, ld, kpad_g, t.kpad_group, seen, pend); break;
      case 3: mainloop_mx<(MB >= 3 ? 3 : MB)>(acc, n, g0, ld, kpad_g, t.kpad_group, seen, pend); break;
      default: mainloop_mx<MB>(acc, n, g0, ld, kpad_g, t.kpad_group, seen, pend); break;
    }
  }

  // After a segment's mainloop (so that nothing of it is live in the
  // epilogue): whether any scale this wave converted (the rows of its active
  // 32-row blocks, so also the padding rows of a scale tensor's last atom
  // that share a block with rows below m or n) was not zero or a positive
  // power of two. One register for all of it: a per-block account of which
  // rows count would cost the hot loop eight. Any wave that saw one stores 1.
  __device__ __forceinline__ void mx_report(uint32_t seen) const {
    if (__builtin_amdgcn_ballot_w64((seen & 0x807F807Fu) != 0) != 0 && lane == 0) *src.args.status = 1;
  }

  // Dispatch on this wave's active 32-row blocks (rows below m).
  __device__ __forceinline__ void mainloop_rows(f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t, int n, int g0,
                                                Loader& ld, int kpad_g, int pend) const {
    static_assert(MB <= 4, "active-block dispatch covers MB <= 4");
    if constexpr (kKS2R) {
      mainloop_ks_rows(acc, ks_rows(t), n, g0, ld, kpad_g, t.kpad_group, pend);
    } else if (kKS && ks_tile(t)) {
      if constexpr (kKS) mainloop_ks_rows(acc, ks_rows(t), n, g0, ld, kpad_g, t.kpad_group, pend);
    } else {
      if constexpr (kWide) {
        if (wide(t)) {
          mainloop<1, NBW>(acc, n, g0, ld, kpad_g, t.kpad_group, pend, wide_bases());
          return;
        }
      }
      const Bases bs = normal_bases();
      switch (active_blocks(t)) {
        case 0: mainloop<0>(acc, n, g0, ld, kpad_g, t.kpad_group, pend, bs); break;
        case 1: mainloop<(MB >= 1 ? 1 : MB)>(acc, n, g0, ld, kpad_g, t.kpad_group, pend, bs); break;
        case 2: mainloop<(MB >= 2 ? 2 : MB)>(acc, n, g0, ld, kpad_g, t.kpad_group, pend, bs); break;
        case 3: mainloop<(MB >= 3 ? 3 : MB)>(acc, n, g0, ld, kpad_g, t.kpad_group, pend, bs); break;
        default: mainloop<MB>(acc, n, g0, ld, kpad_g, t.kpad_group, pend, bs); break;
      }
    }
  }

  // Tiles with at most 32 rows below m (a light group's only tile, or the
  // last of a ragged one) leave one wave row idle in the (wm, wn) layout:
  // there the four waves instead sit side by side along n, each on row
  // block 0 and a quarter of the columns (NBW blocks), so that all of them
  // do MFMAs. Whole-tile f16 kernels only (the stream-K fold and the MX
  // mainloop keep the wave-tile layout of their accumulators).
  static constexpr bool kWide = !Src::kCanSplit && !MX && NBW >= 1 && !kKS;
  __device__ __forceinline__ bool wide(const TileCtx& t) const { return kWide && t.M - t.row0 <= 32; }

  // ---------------- output ----------------
  // fp32 -> fp16 (RNE), 16-byte stores masked to m and n. A lane holds runs
  // of 4 consecutive columns of its row (e * 8 + h * 4 .. +3 of each 32-column
  // block); swapping runs between the two lane halves (v_permlane32_swap) gives
  // each lane 8 consecutive columns, so a store instruction writes 32
  // contiguous bytes per row instead of two 16-byte pieces.
  __device__ __forceinline__ static uint32_t pack_f16(float lo, float hi) {
    const f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }

  // 128x128 wave tiles: the accumulators take all 256 AGPRs, and left to
  // itself the compiler copies every one of them to VGPRs right after the
  // mainloop, which do not hold them all, and spills; they are kept in AGPRs
  // (pin_acc) and each element is read where the epilogue needs it. Smaller
  // wave tiles fit in VGPRs and are left to the compiler.
  static constexpr bool kAccInAgprs = ACC_M * ACC_N == 16;
  __device__ __forceinline__ static float acc_read(float x) {
    if constexpr (!kAccInAgprs) return x;
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
    return v;
  }
  __device__ __forceinline__ static void pin_acc(f32x16 (&acc)[ACC_M][ACC_N]) {
    if constexpr (kAccInAgprs) {
#pragma unroll
      for (int i = 0; i < ACC_M; ++i)
#pragma unroll
        for (int j = 0; j < ACC_N; ++j) asm volatile("" : "+a"(acc[i][j]));
    }
  }

  // Returns true for an unmasked epilogue: every wave then issued exactly S
  // stores (see kPendStores).
  __device__ __forceinline__ bool epilogue(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t) const {
    if constexpr (kKS2R) {
      epilogue_ks_rows(acc, t);
      return false;
    } else if (kKS && ks_tile(t)) {
      if constexpr (kKS) epilogue_ks_rows(acc, t);
      return false;
    } else {
      if constexpr (kWide) {
        if (wide(t)) {
          epilogue_wide(acc, t);
          return false;
        }
      }
      // Tiles wholly inside m and n (all but the edges) store without masks,
      // i.e. without an exec-mask branch around every store.
      if (t.row0 + BM <= t.M && t.col0 + BN <= t.N) {
        epilogue_impl<false>(acc, t);
        return true;
      }
      epilogue_impl<true>(acc, t);
      return false;
    }
  }

  // The wide layout's output: block j of a wave is columns
  // wave * WIDE_COLS + 32 j .. +31 of the tile's first 32 rows.
  __device__ __forceinline__ void epilogue_wide(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t) const {
    int lro = lr, h8 = h * 8;
    asm volatile("" : "+v"(lro), "+v"(h8));
    const int col0 = t.col0 + wave * WIDE_COLS;
    typedef __attribute__((address_space(1))) uint16_t gu16;
    gu16* crow = (gu16*)t.c + (size_t)(t.row0 + lro) * t.N + col0 + h8;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = acc_read(acc[0][j][8 * p + e]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(pack_f16(a[0], a[1]), pack_f16(a[4], a[5]), false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(pack_f16(a[2], a[3]), pack_f16(a[6], a[7]), false, false);
        const int cu = j * 32 + 2 * p * 8;
        if (lro < t.M - t.row0 && h8 < t.N - col0 - cu) {
          const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
          *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(crow + cu) = v;
        }
      }
    }
  }

  template <bool MASKED>
  __device__ __forceinline__ void epilogue_impl(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t) const {
    // The lane's row and column offsets are formed here, per tile, from a copy
    // the compiler cannot see through: left to itself it hoists one offset per
    // block out of the tile loop and spills them, and each reload between
    // stores then waits for every store before it.
    int lro = lr, h8 = h * 8;
    asm volatile("" : "+v"(lro), "+v"(h8));
    const int col0 = t.col0 + wn * WN;
    // global (not flat) stores: they count in vmcnt only, not in the lgkmcnt
    // the barriers wait for
    typedef __attribute__((address_space(1))) uint16_t gu16;
    gu16* clane = (gu16*)t.c + (size_t)(t.row0 + lro) * t.N + col0 + h8;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int rb = row_block(wm, i) * 32;
      gu16* crow = clane + (size_t)rb * t.N;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          // runs 2p (kept by lanes h = 0) and 2p + 1 (kept by lanes h = 1)
          float a[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = acc_read(acc[i][j][8 * p + e]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(pack_f16(a[0], a[1]), pack_f16(a[4], a[5]), false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pack_f16(a[2], a[3]), pack_f16(a[6], a[7]), false, false);
          const int cu = j * 32 + 2 * p * 8;  // uniform part of the column
          // n % 8 == 0: an 8-column chunk is all in or all out
          if (!MASKED || (lro < t.M - t.row0 - rb && h8 < t.N - col0 - cu)) {
            const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
            *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(crow + cu) = v;
          }
        }
      }
    }
  }


  // ---------------- stream-K: partials and the fold ----------------
  // Workgroup wg owns two fp32 tile-sized slots: slot 0 for the segment that
  // starts its range, slot 1 for its last. Accumulator element e of block
  // (i, j) of a lane is float ((((wave * MB + i) * NB + j) * 16 + e) * 64 + lane)
  // of the slot, so that the 64 lanes' accesses to one element are 256
  // contiguous bytes; only the wave's active row blocks are written. After
  // the slots: arrival counters, kFoldLevels per slot, zero between calls.
  __device__ __forceinline__ int partial_index(int i, int j) const {
    return (((wave * MB + i) * NB + j) * 16) * 64 + lane;
  }
  // Partials are stored and loaded element by element as relaxed atomics of
  // device scope (global_store/global_load with cache-policy bit SC1): such
  // stores write through the XCD's L2, and such loads read what they wrote,
  // from any XCD (the L2s of the XCDs are not coherent with each other).
  __device__ __forceinline__ float* slot_ptr(int wg, int slot) const {
    return src.args.partials + ((size_t)wg * 2 + slot) * TILE_FLOATS;
  }
  __device__ __forceinline__ int32_t* arrivals(int wg, int slot, int level) const {
    uint8_t* p = reinterpret_cast<uint8_t*>(src.args.partials) + (size_t)src.args.grid * 2 * (TILE_FLOATS * 4);
    return reinterpret_cast<int32_t*>(p) + ((wg * 2 + slot) * kFoldLevels + level);
  }

  // The contributors of a split tile are the workgroups in [c_first, c_last]
  // with non-empty ranges (ranges are empty only after whole rounds), ranked
  // in workgroup order, which is K order. Contributor c's partial of the tile
  // is in its slot 0 if its range starts inside the tile (or at its first
  // unit u_first), else in slot 1.
  __device__ __forceinline__ bool has_units(int c) const { return unit_begin(c + 1) > unit_begin(c); }
  __device__ __forceinline__ int contributor(int c_first, int c_last, int rank) const {
    if (src.args.whole_tiles == 0) return c_first + rank;
    for (int c = c_first; c < c_last; ++c)
      if (has_units(c) && rank-- == 0) return c;
    return c_last;
  }
  __device__ __forceinline__ int slot_of(int c, int64_t u_first) const { return unit_begin(c) >= u_first ? 0 : 1; }

  // This workgroup computed stages [s0, s1) of a tile, not all of it: the
  // tile's C contributors fold their partials along a fixed binary tree over
  // their ranks. Node (L, j) covers ranks [j 2^L, (j + 1) 2^L); its sum is
  // (left child) + (right child) and sits in the slot of its first rank.
  // Each contributor stores its partial (device-scope stores) and waits until
  // they have completed; then, level by level, one thread adds one to the
  // counter of its node (device-scope atomic, skipped where the node has no
  // right child). The first to arrive stops there; the second loads both
  // children (its own from registers at the first level), adds them, and
  // either stores the sum to the node's slot and goes on up, or - at the
  // root - rounds to fp16 and stores C. The order of every addition is fixed
  // by the tree, so the result does not depend on timing, and no workgroup
  // ever waits for another. Each node's counter is cleared by its folder.
  // Returns true when this workgroup stored the tile's C.
  __device__ __forceinline__ bool publish_partial(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t,
                                                  const Segment& seg) const {
    const int amb = active_blocks(t);
    float* mine = slot_ptr(vwg, seg.u == unit_begin(vwg) ? 0 : 1);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i >= amb) break;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        float x[16];
        acc_block(acc, i, j, x);
        store_block(mine, i, j, x);
      }
    }
    wait_vmem_all();  // this wave's partial is visible at device scope
    const int64_t u_first = seg.u - seg.s0;  // the tile's first unit
    const int c_first = owner_of_unit(u_first);
    const int c_last = owner_of_unit(u_first + t.nk - 1);
    int count = c_last - c_first + 1, me = vwg - c_first;
    if (src.args.whole_tiles != 0) {
      count = me = 0;
      for (int c = c_first; c <= c_last; ++c) {
        me += c < vwg && has_units(c);
        count += has_units(c);
      }
    }
    const bool masked = !(t.row0 + BM <= t.M && t.col0 + BN <= t.N);
    int32_t* flag = reinterpret_cast<int32_t*>(smem + FLAG_OFF);
    for (int level = 1; (1 << (level - 1)) < count; ++level) {
      const int left = (me >> level) << level, right = left + (1 << (level - 1));  // first ranks of the children
      if (right >= count) continue;  // no right child: the node's sum is the left child's, in the same slot
      const int wl = contributor(c_first, c_last, left), wr = contributor(c_first, c_last, right);
      const int sl = slot_of(wl, u_first), sr = slot_of(wr, u_first);
      block_sync();  // every wave's stores (partial, or the sum of the level below) have completed
      if (threadIdx.x == 0)
        *flag = __hip_atomic_fetch_add(arrivals(wl, sl, level), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      block_sync();
      if (__builtin_amdgcn_readfirstlane(*flag) == 0) return false;  // the other child's folder goes on
      const bool root = (1 << level) >= count;
      // at the first level this workgroup's own child is its partial, still in registers
      const int own = level == 1 ? (me == left ? 0 : 1) : -1;
      if (root && masked) fold_node<true, true>(acc, t, amb, own, wl, sl, wr, sr);
      else if (root) fold_node<true, false>(acc, t, amb, own, wl, sl, wr, sr);
      else fold_node<false, false>(acc, t, amb, own, wl, sl, wr, sr);
      if (threadIdx.x == 0) __hip_atomic_store(arrivals(wl, sl, level), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (root) return true;
      wait_vmem_all();  // the node's sum is visible at device scope
    }
    return false;  // (not reached: the root always has a right child)
  }

  // The lane's 16 floats of block (i, j) of a partial slot, and of the
  // accumulators.
  __device__ __forceinline__ void load_block(const float* p, int i, int j, float (&x)[16]) const {
    const float* b = p + partial_index(i, j);
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = __hip_atomic_load(b + e * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ void store_block(float* p, int i, int j, const float (&x)[16]) const {
    float* b = p + partial_index(i, j);
#pragma unroll
    for (int e = 0; e < 16; ++e) __hip_atomic_store(b + e * 64, x[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ static void acc_block(const f32x16 (&acc)[ACC_M][ACC_N], int i, int j, float (&x)[16]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = acc_read(acc[i][j][e]);
  }

  // Node sum = left child + right child, two blocks of a row block at a
  // time: each child's values are loaded (device-scope; own = 0 or 1 takes
  // that child from the accumulators instead), then added; at the root the
  // sum is rounded and stored to C, elsewhere it is stored (device-scope) to
  // the left child's slot, whose values were just read.
  template <bool ROOT, bool MASKED>
  __device__ __forceinline__ void fold_node(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t, int amb, int own, int wl,
                                            int sl, int wr, int sr) const {
    int lro = lr, h8 = h * 8;
    asm volatile("" : "+v"(lro), "+v"(h8));
    float* pl = slot_ptr(wl, sl);
    const float* pr = slot_ptr(wr, sr);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i >= amb) break;
      fold_blocks<ROOT, MASKED, 0>(acc, t, i, own, pl, pr, lro, h8);
      if constexpr (NB > 2) fold_blocks<ROOT, MASKED, 2>(acc, t, i, own, pl, pr, lro, h8);
    }
  }

  template <bool ROOT, bool MASKED, int J0>
  __device__ __forceinline__ void fold_blocks(const f32x16 (&acc)[ACC_M][ACC_N], const TileCtx& t, int i, int own, float* pl,
                                              const float* pr, int lro, int h8) const {
    constexpr int JB = NB < 2 ? NB : 2;
    float sum[JB][16], y[JB][16];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      if (own == 0) acc_block(acc, i, J0 + j, sum[j]);
      else load_block(pl, i, J0 + j, sum[j]);
      if (own == 1) acc_block(acc, i, J0 + j, y[j]);
      else load_block(pr, i, J0 + j, y[j]);
    }
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[j][e] += y[j][e];
    if constexpr (ROOT) {
#pragma unroll
      for (int j = 0; j < JB; ++j) store_block_c<MASKED>(sum[j], t, i, J0 + j, lro, h8);
    } else {
#pragma unroll
      for (int j = 0; j < JB; ++j) store_block(pl, i, J0 + j, sum[j]);
    }
  }

  // C stores of block (i, j) of this wave from the lane's 16 floats (the
  // layout of the accumulators), as in epilogue_impl.
  template <bool MASKED>
  __device__ __forceinline__ void store_block_c(const float (&a)[16], const TileCtx& t, int i, int j, int lro,
                                                int h8) const {
    const int col0 = t.col0 + wn * WN;
    typedef __attribute__((address_space(1))) uint16_t gu16;
    const int rb = row_block(wm, i) * 32;
    gu16* crow = (gu16*)t.c + (size_t)(t.row0 + rb + lro) * t.N + col0 + h8;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const auto s0 = __builtin_amdgcn_permlane32_swap(pack_f16(a[8 * p + 0], a[8 * p + 1]),
                                                       pack_f16(a[8 * p + 4], a[8 * p + 5]), false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(pack_f16(a[8 * p + 2], a[8 * p + 3]),
                                                       pack_f16(a[8 * p + 6], a[8 * p + 7]), false, false);
      const int cu = j * 32 + 2 * p * 8;
      if (!MASKED || (lro < t.M - t.row0 - rb && h8 < t.N - col0 - cu)) {
        const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
        *reinterpret_cast<__attribute__((address_space(1))) u32x4*>(crow + cu) = w;
      }
    }
  }

  // Stream-K leaves the tiles of k = 0 groups (no units) to a strided pass.
  __device__ __forceinline__ void zero_k_tiles() const {
    f32x16 zero[ACC_M][ACC_N];
#pragma unroll
    for (int i = 0; i < ACC_M; ++i)
#pragma unroll
      for (int j = 0; j < ACC_N; ++j) zero[i][j] = f32x16{};
    const KernelArgs& args = src.args;
    for (int gi = 0; gi < args.num_classes; ++gi) {
      if (args.cls[gi].nk != 0) continue;
      for (int tile = args.tile_prefix[gi] + vwg; tile < args.tile_prefix[gi + 1]; tile += args.grid)
        if (tile >= args.whole_tiles) epilogue(zero, setup(tile));  // (earlier ones were dealt out whole)
    }
  }

  __device__ __forceinline__ void run() const {
    Loader ld;
    loader_init(ld);
    for (int b = 0; b < NS; ++b) issue_all(ld);  // every buffer is free
    Segment seg;
    first_segment(seg);
    int g0 = 0;
    int pend = kPendPrologue;
    while (seg.valid) {
      const TileCtx t = setup(seg.tile);
      const int n = seg.s1 - seg.s0;
      sub_words = t.sub_words;
      f32x16 acc[ACC_M][ACC_N];
#pragma unroll
      for (int i = 0; i < ACC_M; ++i)
#pragma unroll
        for (int j = 0; j < ACC_N; ++j) acc[i][j] = f32x16{};
      // the tile's last stage, if this segment ends the tile and its last
      // scale atom is half used
      const int kpad_g = KPAD && t.kpad_group >= 0 && seg.s1 == t.nk ? g0 + n - 1 : -1;
      if constexpr (MX) {
        uint32_t seen = 0;  // bf16 bits of every scale converted
        if (n > 0) mainloop_rows_mx(acc, t, n, g0, ld, kpad_g, seen, pend);
        mx_report(seen);
      } else {
        if (n > 0) mainloop_rows(acc, t, n, g0, ld, kpad_g, pend);
      }
      pin_acc(acc);  // (128x128 wave tiles) in AGPRs until the epilogue reads them
      bool unmasked = false;
      if constexpr (Src::kCanSplit) {
        if (seg.s0 == 0 && seg.s1 == t.nk) unmasked = epilogue(acc, t);
        else publish_partial(acc, t, seg);
      } else {
        unmasked = epilogue(acc, t);  // whole tiles only
      }
      // the next segment's first NS stages were all issued by this mainloop,
      // after any earlier stores, iff it ran at least NS stages
      pend = (kOverlapStores && unmasked && n >= NS) ? kPendStores : kPendUnknown;
      g0 += n;
      next_segment(seg);
    }
    if constexpr (Src::kCanSplit) {
      if (src.split()) zero_k_tiles();
    }
    wait_vmem_all();  // no direct load may still be writing LDS when the workgroup ends
  }
};

// The kernels' single argument, read in place from the kernarg segment (where
// it starts at offset 0). Binding the by-value parameter to a reference makes
// the compiler keep a private copy of it once the argument has many readers;
// reads through this pointer stay uniform constant loads.
__device__ __forceinline__ const KernelArgs& kernel_args() {
  return *(const KernelArgs*)__builtin_amdgcn_kernarg_segment_ptr();
}

// Stage layout in LDS (bytes): [A: BM rows x 64][B: BN rows x 64]
// [scale atoms: (BM + BN) / 128 atom rows x 2 k-groups x 512]; A and B rows are
// swizzled by lds_off, the scale atoms are stored as in global memory.
template <int BM, int BN, int WM, int WN, int NS, bool KPAD, bool MX = false, bool SPLIT = false, bool KS2R_ALL = false>
__global__ __launch_bounds__(kThreads, 1) void nvfp4_grouped_gemm_kernel(KernelArgs) {
  using K = GemmKernel<BM, BN, WM, WN, NS, KernargSrc<SPLIT>, KPAD, MX, KS2R_ALL>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[K::LDS_BYTES];
  const K k(KernargSrc<SPLIT>{kernel_args()}, smem);
  k.run();
}

// Tiles of one group of the device tables with BM x BN tiles, or -1 if the
// group breaks a rule of the host-side validation (or has more than 2^20 tiles
// of 128x128, which keeps the tile count of all groups within 2^30).
__host__ __device__ inline bool bad_ptr(uint64_t p) { return p == 0 || (p & 15) != 0; }

template <int BM, int BN>
__host__ __device__ int64_t device_group_tiles(const int32_t* sz, const uint64_t* ptr) {
  const int64_t m = sz[0], n = sz[1], k = sz[2], l = sz[3];
  if (m < 0 || n < 0 || k < 0 || l < 1 || k % 32 != 0 || n % 8 != 0) return -1;
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (k > (int64_t(1) << 22) || m > (int64_t(1) << 30) || n > (int64_t(1) << 30)) return -1;
  if (m * (k / 2) > lim / l || n * (k / 2) > lim / l) return -1;
  if ((m + 127) / 128 * 128 * (k / 16) > lim / l || (n + 127) / 128 * 128 * (k / 16) > lim / l) return -1;
  if (m * n > (int64_t(1) << 40) / l) return -1;
  if (m == 0 || n == 0) return 0;
  if (bad_ptr(ptr[2])) return -1;  // C
  if (k > 0 && (bad_ptr(ptr[0]) || bad_ptr(ptr[1]) || bad_ptr(ptr[3]) || bad_ptr(ptr[4]))) return -1;
  if ((m + 127) / 128 * ((n + 127) / 128) * l > (int64_t(1) << 20)) return -1;
  return (m + BM - 1) / BM * ((n + BN - 1) / BN) * l;
}

// prefix[c] = first tile of class c (see DeviceSrc), prefix[R G] = all tiles;
// rejected groups own no tiles. Each thread takes G / 256 consecutive groups;
// wave scans and the four wave totals give the offsets. Workgroup 0 stores the
// number of rejected groups. Ends with a barrier.
template <int BM, int BN>
__device__ void build_device_prefix(const DeviceGroupArgs& a, int32_t* prefix, int32_t* wave_sums) {
  constexpr int PER = kMaxDeviceGroups / kThreads;
  constexpr int WAVES = kThreads / 64;
  constexpr int R = BM / 64;
  constexpr int V = R + 1;  // tiles per row class, then rejected groups
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.num_groups;
  // every table read first (one round trip), then the checks
  int32_t sz[PER][4];
  uint64_t ptr[PER][5];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = min(tid * PER + q, G - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) sz[q][i] = a.sizes[4 * g + i];
#pragma unroll
    for (int i = 0; i < 3; ++i) ptr[q][i] = a.abc[3 * g + i];
#pragma unroll
    for (int i = 0; i < 2; ++i) ptr[q][3 + i] = a.sf[2 * g + i];
  }
  int32_t full[PER], last[PER], last_cls[PER];
  int32_t v[V] = {};
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    const int64_t x = g < G ? device_group_tiles<BM, BN>(sz[q], ptr[q]) : 0;
    last_cls[q] = x > 0 ? last_row_class<BM>(sz[q][0]) : 0;
    const int64_t row = x > 0 ? (int64_t)((sz[q][1] + BN - 1) / BN) * sz[q][3] : 0;  // tiles of one tile row
    last[q] = last_cls[q] > 0 ? (int32_t)row : 0;
    full[q] = x > 0 ? (int32_t)(x - last[q]) : 0;
    v[0] += full[q];
#pragma unroll
    for (int b = 1; b < R; ++b) v[b] += last_cls[q] == b ? last[q] : 0;
    v[R] += x < 0 ? 1 : 0;
  }
  int incl[V];
#pragma unroll
  for (int j = 0; j < V; ++j) incl[j] = v[j];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int y = __shfl_up(incl[j], d);
      if (lane >= d) incl[j] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < V; ++j) wave_sums[j * WAVES + wave] = incl[j];
  }
  __syncthreads();
  int before[V] = {}, total[V] = {};
#pragma unroll
  for (int w = 0; w < WAVES; ++w)
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int x = wave_sums[j * WAVES + w];
      before[j] += w < wave ? x : 0;
      total[j] += x;
    }
  // run[b]: first tile of this thread's first group in class b
  int run[R];
  int base = 0;
#pragma unroll
  for (int b = 0; b < R; ++b) {
    run[b] = base + before[b] + incl[b] - v[b];
    base += total[b];
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
#pragma unroll
    for (int b = 0; b < R; ++b) {
      if (g < G) prefix[b * G + g] = run[b];
      run[b] += b == 0 ? full[q] : (last_cls[q] == b ? last[q] : 0);
    }
  }
  if (tid == 0) prefix[R * G] = base;
  // (a wave-uniform test outside the one-thread branch: a test on the
  // workgroup id inside it would make the id look lane-dependent below)
  if (blockIdx.x == 0 && a.status != nullptr) {
    if (tid == 0) *a.status = total[R];
  }
  __syncthreads();
}

template <int BM, int BN, int WM, int WN, int NS>
__global__ __launch_bounds__(kThreads, 1) void nvfp4_grouped_gemm_device_kernel(DeviceGroupArgs) {
  using Src = DeviceSrc<BM, BN>;
  using K = GemmKernel<BM, BN, WM, WN, NS, Src, true>;  // the tables may hold any k
  static_assert(K::LDS_BYTES + 4 * (kMaxDeviceClasses + 1 + (kMaxRowClasses + 1) * kThreads / 64) <= 160 * 1024,
                "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[K::LDS_BYTES];
  __shared__ int32_t prefix[kMaxDeviceClasses + 1];
  __shared__ int32_t wave_sums[(kMaxRowClasses + 1) * kThreads / 64];
  const DeviceGroupArgs& args = *(const DeviceGroupArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  build_device_prefix<BM, BN>(args, prefix, wave_sums);
  const K k(Src{args, prefix}, smem);
  k.run();
}

// Clears the stream-K arrival counters before a split launch: a kernel rather than a memset, so that a captured graph
// replays it correctly. The fold also leaves them zero.
__global__ __launch_bounds__(kThreads) void nvfp4_clear_arrivals_kernel(int32_t* p, int n) {
  for (int i = (int)threadIdx.x; i < n; i += kThreads) p[i] = 0;
}

// ---------------------------------------------------------------------------
// Host side: tile configurations, planning, workspace
// ---------------------------------------------------------------------------

struct TileConfig {
  int bm, bn, wm, wn;
  // [stream-K][power-of-two scales][some group with k % 64 == 32]
  void (*kernel[2][2][2])(KernelArgs);
  void (*device_kernel)(DeviceGroupArgs);
  int64_t (*device_tiles)(const int32_t*, const uint64_t*);  // the device kernel's per-group check
  // The same computation with a three-stage LDS pipeline (any k; [stream-K]),
  // for verification: each LDS buffer is then rewritten one stage sooner after
  // its last reads, so a missing wait or barrier shows up as a difference.
  void (*kernel_ns3[2])(KernelArgs);
  // 256x128 and 128x256 only (else null): whole-tile f16 kernels that put
  // every tile in a K-split mode ([some group with k % 64 == 32]), and their
  // three-stage counterpart; for calls whose groups all have long K (see
  // kKS2RMinStages).
  void (*kernel_ks2r[2])(KernelArgs);
  void (*kernel_ks2r_ns3)(KernelArgs);
};

constexpr int kStages = 4;  // LDS pipeline depth (4 x 36 KiB for 256x256 tiles)

#define NVFP4_KERNEL(bm, bn, wm, wn, kpad, mx, split) nvfp4_grouped_gemm_kernel<bm, bn, wm, wn, kStages, kpad, mx, split>
// The end-of-tile exchange of a K-split tile moves 128 KiB through LDS: on
// short tiles it costs more than the split saves (a 16-stage workload on
// 256x128 tiles measured 62 -> 66 us with every tile split, 56-stage ones
// gain 2-3%), so calls take the all-split kernels only when every group with
// work has at least this many 128-K stages.
constexpr int kKS2RMinStages = 32;
#define NVFP4_TILE_CONFIG(bm, bn, wm, wn)                                                                       \
  { bm, bn, wm, wn,                                                                                         \
    {{{NVFP4_KERNEL(bm, bn, wm, wn, false, false, false), NVFP4_KERNEL(bm, bn, wm, wn, true, false, false)},   \
      {NVFP4_KERNEL(bm, bn, wm, wn, false, true, false), NVFP4_KERNEL(bm, bn, wm, wn, true, true, false)}},    \
     {{NVFP4_KERNEL(bm, bn, wm, wn, false, false, true), NVFP4_KERNEL(bm, bn, wm, wn, true, false, true)},     \
      {NVFP4_KERNEL(bm, bn, wm, wn, false, true, true), NVFP4_KERNEL(bm, bn, wm, wn, true, true, true)}}},     \
    nvfp4_grouped_gemm_device_kernel<bm, bn, wm, wn, kStages>, device_group_tiles<bm, bn>,                     \
    {nvfp4_grouped_gemm_kernel<bm, bn, wm, wn, 3, true, false, false>,                                       \
     nvfp4_grouped_gemm_kernel<bm, bn, wm, wn, 3, true, false, true>},                                       \
    {nullptr, nullptr}, nullptr }
#define NVFP4_TILE_CONFIG_KS2R(bm, bn, wm, wn)                                                                  \
  { bm, bn, wm, wn,                                                                                         \
    {{{NVFP4_KERNEL(bm, bn, wm, wn, false, false, false), NVFP4_KERNEL(bm, bn, wm, wn, true, false, false)},   \
      {NVFP4_KERNEL(bm, bn, wm, wn, false, true, false), NVFP4_KERNEL(bm, bn, wm, wn, true, true, false)}},    \
     {{NVFP4_KERNEL(bm, bn, wm, wn, false, false, true), NVFP4_KERNEL(bm, bn, wm, wn, true, false, true)},     \
      {NVFP4_KERNEL(bm, bn, wm, wn, false, true, true), NVFP4_KERNEL(bm, bn, wm, wn, true, true, true)}}},     \
    nvfp4_grouped_gemm_device_kernel<bm, bn, wm, wn, kStages>, device_group_tiles<bm, bn>,                     \
    {nvfp4_grouped_gemm_kernel<bm, bn, wm, wn, 3, true, false, false>,                                       \
     nvfp4_grouped_gemm_kernel<bm, bn, wm, wn, 3, true, false, true>},                                       \
    {nvfp4_grouped_gemm_kernel<bm, bn, wm, wn, kStages, false, false, false, true>,                          \
     nvfp4_grouped_gemm_kernel<bm, bn, wm, wn, kStages, true, false, false, true>},                          \
    nvfp4_grouped_gemm_kernel<bm, bn, wm, wn, 3, true, false, false, true> }
const TileConfig kConfigs[] = {
    NVFP4_TILE_CONFIG(256, 256, 128, 128),
    NVFP4_TILE_CONFIG_KS2R(128, 256, 64, 128),
    NVFP4_TILE_CONFIG_KS2R(256, 128, 128, 64),
    NVFP4_TILE_CONFIG_KS2R(128, 128, 64, 64),
    NVFP4_TILE_CONFIG(64, 64, 32, 32),
};
#undef NVFP4_TILE_CONFIG
#undef NVFP4_KERNEL
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
// 256x256 tiles for the device-table entry point: the largest wave tiles
// dequantise least per MFMA, and a many-group launch has tiles enough to
// fill the grid (120 groups of 40-400 x 4096 x 7168: 1.83 ms against 2.08 ms
// with 256x128 tiles)
constexpr int kDefaultDeviceConfig = 0;

thread_local int t_last_hip_error = 0;

std::atomic<int> g_cu_cache[64];

int device_cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { t_last_hip_error = (int)e; return NVFP4_ERR_HIP; }
  if (dev >= 0 && dev < 64) {
    const int cached = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (cached > 0) { *out = cached; return NVFP4_OK; }
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) { t_last_hip_error = (int)e; return NVFP4_ERR_HIP; }
  if (dev >= 0 && dev < 64) g_cu_cache[dev].store(cus, std::memory_order_relaxed);
  *out = cus;
  return NVFP4_OK;
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// How one call is carried out.
struct Plan {
  int cfg;        // tile configuration
  int split;      // 0: whole tiles strided over the grid, 1: stream-K
  int rounds;     // stream-K: whole rounds of `grid` tiles before the unit ranges
  int grid;       // persistent workgroups
  int64_t tiles;  // output tiles
  int64_t units;  // (tile, 128-K stage) units
  size_t ws_bytes;  // workspace the plan needs (0 without stream-K)
  double cost;    // modelled makespan
};

int64_t group_tiles(const int32_t* ps, int g, int cfg) {
  const int32_t m = ps[4 * g + 0], n = ps[4 * g + 1], l = ps[4 * g + 3];
  if (m == 0 || n == 0) return 0;
  return ceil_div64(m, kConfigs[cfg].bm) * ceil_div64(n, kConfigs[cfg].bn) * l;
}

int group_stages(const int32_t* ps, int g) { return (int)ceil_div64(ps[4 * g + 2], kBK); }

// Whether a whole-tile call of the general entry points on configuration cfg
// runs the kernels that split K over the waves in every tile: cfg has them,
// and every group with work (m, n and k > 0) has at least kKS2RMinStages
// 128-K stages.
bool splits_k_everywhere(const int32_t* ps, int G, int cfg) {
  if (kConfigs[cfg].kernel_ks2r[0] == nullptr) return false;
  for (int g = 0; g < G; ++g)
    if (ps[4 * g + 0] > 0 && ps[4 * g + 1] > 0 && ps[4 * g + 2] > 0 && group_stages(ps, g) < kKS2RMinStages)
      return false;
  return true;
}

// Largest number of 32-row blocks a wave computes in a tile with `rows` rows
// below m (row blocks alternate between the two wave rows).
int max_active_blocks(int64_t rows, int bm) {
  const int64_t nb = std::min<int64_t>(rows, bm) <= 0 ? 0 : (std::min<int64_t>(rows, bm) + 31) / 32;
  return (int)((nb + 1) / 2);
}

// Share of a full stage's time that a tile stage with `amb` of `mb` active
// blocks per wave takes: the loads, barrier and B dequantisation do not shrink
// with m.
double stage_fraction(int amb, int mb) {
  const double fixed = 0.25;
  return fixed + (1.0 - fixed) * (double)amb / (double)mb;
}

struct WorkClass {
  int g;          // group
  int tm0;        // first tile row
  int tiles_m;    // tile rows
  int64_t tiles;  // tiles_m * tiles_n * l
  int nk;         // stages per tile
  double cost;    // modelled time per tile, in full tile-stages
  double fill;    // share of a full tile's row blocks that hold rows below m (sizes its stream-K partial)
};

double tile_overhead_stages() { return 1.5; }  // epilogue and pipeline fill per tile

// The work classes of a call for tile configuration cfg, heaviest per tile
// first (stable: groups keep their order among equals). Returns the count.
int build_classes(const int32_t* ps, int G, int cfg, WorkClass* out);

// Modelled stream-K costs, in full tile-stages of the configuration, for a
// partial of fill f (its share of a full tile's row blocks): storing it
// (device-scope stores, then a wait for them) and folding a tile with C
// contributors along the fold tree (the root's folder goes through
// ceil(log2 C) levels, each but the first loading two children and storing
// a sum). Fitted to per-workgroup timestamps on 256x256 and 256x128 tiles
// (256x256, f = 1: ~6 us to store, ~8 us more to fold with C = 2, against a
// ~2.2 us stage). The one-workgroup kernel that clears the counters first is
// counted in 128x128 tile-stage units.
double partial_store_stages(double f) { return 1.0 + 1.7 * f; }
double fold_stages(double f, int contributors) {
  int levels = 0;
  while ((1 << levels) < contributors) ++levels;
  return (0.3 + 3.3 * f) * (1.0 + 1.3 * (levels - 1));
}
constexpr double kClearKernelUnits = 4.0;

// Stream-K after `rounds` whole rounds: the first rounds * grid tiles (in
// class order) are dealt out whole by the kernel's snake walk; the units of
// the remaining tiles are cut into ranges[w] .. ranges[w + 1] for workgroup
// w (contiguous in workgroup order, possibly empty) so that every
// workgroup's whole tiles plus units (a unit of class c costs
// cls[c].cost / nk) come out equal: the remaining cost is water-filled over
// the whole-tile loads. The partials' stores and folds are left out of the
// cuts (which contributor folds depends on timing: cutting around a
// predicted folder measured worse) and added to the returned makespan
// estimate, in full tile-stages: a range's first segment may be the tail of
// a tile begun by an earlier workgroup (it stores a partial), and its last
// the head of a tile that later workgroups finish, whose fold it usually
// does. Needs 1 <= grid <= kMaxSplitGrid and rounds * grid <= tiles.
double hybrid_ranges(const WorkClass* cls, int nc, int grid, int rounds, int32_t* ranges) {
  double load[kMaxSplitGrid], over[kMaxSplitGrid];
  for (int w = 0; w < grid; ++w) load[w] = over[w] = 0.0;
  int64_t unit_at[kMaxClasses + 1], tile_at[kMaxClasses + 1];
  unit_at[0] = 0;
  tile_at[0] = 0;
  for (int c = 0; c < nc; ++c) {
    unit_at[c + 1] = unit_at[c] + cls[c].tiles * cls[c].nk;
    tile_at[c + 1] = tile_at[c] + cls[c].tiles;
  }
  // the whole rounds, as the kernel walks them
  const int64_t whole = (int64_t)rounds * grid;
  int64_t u0 = 0;  // first unit after the whole tiles
  for (int c = 0; c < nc; ++c) {
    const int64_t n = std::min(cls[c].tiles, std::max<int64_t>(whole - tile_at[c], 0));
    for (int64_t i = 0; i < n; ++i) {
      const int64_t t = tile_at[c] + i, r = t / grid, pos = t % grid;
      load[(r & 1) ? grid - 1 - pos : pos] += cls[c].cost;
    }
    u0 += n * cls[c].nk;
  }
  const int64_t units = unit_at[nc];
  auto cost_to = [&](int64_t u) {  // cost of units [u0, u)
    double x = 0.0;
    for (int c = 0; c < nc; ++c) {
      const int64_t lo = std::max(unit_at[c], u0), hi = std::min(unit_at[c + 1], u);
      if (hi > lo) x += (double)(hi - lo) * cls[c].cost / cls[c].nk;
    }
    return x;
  };
  auto unit_of_cost = [&](double target) {  // inverse of cost_to, to the nearest unit
    double x = 0.0;
    for (int c = 0; c < nc; ++c) {
      const int64_t lo = std::max(unit_at[c], u0), hi = unit_at[c + 1];
      if (hi <= lo) continue;
      const double per = cls[c].cost / cls[c].nk, span = (double)(hi - lo) * per;
      if (x + span >= target) return lo + (int64_t)std::llround((target - x) / per);
      x += span;
    }
    return units;
  };
  auto locate_unit = [&](int64_t u, int* c, int* stage) {
    int k = 0;
    while (k < nc - 1 && unit_at[k + 1] <= u) ++k;
    *c = k;
    const int64_t local = u - unit_at[k];
    *stage = (int)(local % cls[k].nk);
    return tile_at[k] + local / cls[k].nk;
  };
  const double total = cost_to(units);
  {
    // water level: the sum over w of max(0, level - load[w]) is total. After
    // whole rounds a workgroup gets at least about a quarter of a tile's
    // stages or nothing: slivers of a few units would spread one tile over
    // many workgroups, whose partials then pass through a deep fold tree
    // (measured: 14 one-unit ranges of one tile, folds of up to 45 us).
    int order[kMaxSplitGrid];
    for (int w = 0; w < grid; ++w) order[w] = w;
    std::stable_sort(order, order + grid, [&](int x, int y) { return load[x] < load[y]; });
    const int64_t sk_tiles = tile_at[nc] - whole;
    const double min_amount =
        rounds == 0 || units == u0 ? 0.0
                                   : total / (double)(units - u0) *
                                         std::max<double>(2.0, std::floor((double)(units - u0) / sk_tiles / 4.0));
    // the k lowest-loaded workgroups share the rest: k as large as the level
    // allows (each of them below it) and, after whole rounds, as leaves the
    // k-th at least min_amount
    double level = 0.0, acc = 0.0;
    int k = 0;
    for (int i = 1; i <= grid; ++i) {
      acc += load[order[i - 1]];
      const double lv = (total + acc) / i;
      if (i > 1 && (lv < load[order[i - 1]] || lv - load[order[i - 1]] < min_amount)) break;
      level = lv;
      k = i;
    }
    double amount[kMaxSplitGrid];
    for (int w = 0; w < grid; ++w) amount[w] = 0.0;
    for (int r = 0; r < k; ++r) amount[order[r]] = std::max(0.0, level - load[order[r]]);
    ranges[0] = (int32_t)u0;
    double target = 0.0;
    for (int w = 1; w < grid; ++w) {
      target += amount[w - 1];
      // without whole rounds every workgroup gets at least one unit (grid <= units)
      const int64_t lo = ranges[w - 1] + (rounds == 0 ? 1 : 0), hi = units - (rounds == 0 ? grid - w : 0);
      ranges[w] = (int32_t)std::min<int64_t>(std::max<int64_t>(unit_of_cost(target), lo), hi);
    }
    ranges[grid] = (int32_t)units;
    // the partials of these cuts
    for (int w = 0; w < grid; ++w) {
      over[w] = 0.0;
      const int64_t a = ranges[w], b = ranges[w + 1];
      if (b <= a) continue;
      int ca, cb, sa, sb;
      const int64_t ta = locate_unit(a, &ca, &sa), tb = locate_unit(b - 1, &cb, &sb);
      const bool tail = sa > 0, head = sb + 1 < cls[cb].nk;  // first segment begun earlier; last unfinished
      if (tail) over[w] += partial_store_stages(cls[ca].fill);
      if (head && !(tail && ta == tb)) {
        // contributors of tile tb: this one and the later non-empty ranges that start inside it
        const int64_t end = b - 1 - sb + cls[cb].nk;
        int contributors = 1;
        for (int v = w + 1; v < grid && ranges[v] < end; ++v) contributors += ranges[v + 1] > ranges[v];
        over[w] += partial_store_stages(cls[cb].fill) + fold_stages(cls[cb].fill, contributors);
      }
    }
  }
  double worst = 0.0;
  for (int w = 0; w < grid; ++w)
    worst = std::max(worst, load[w] + over[w] + cost_to(ranges[w + 1]) - cost_to(ranges[w]));
  return worst;
}

int build_classes(const int32_t* ps, int G, int cfg, WorkClass* out) {
  const TileConfig& tc = kConfigs[cfg];
  const int mb = tc.wm / 32;
  int n = 0;
  for (int g = 0; g < G; ++g) {
    const int64_t m = ps[4 * g + 0], nn = ps[4 * g + 1], l = ps[4 * g + 3];
    if (m == 0 || nn == 0) continue;
    const int tiles_m = (int)ceil_div64(m, tc.bm);
    const int64_t tiles_n = ceil_div64(nn, tc.bn);
    const int nk = group_stages(ps, g);
    const int tail_amb = max_active_blocks(m - (int64_t)(tiles_m - 1) * tc.bm, tc.bm);
    const bool split_tail = tiles_m > 1 && tail_amb < mb;
    const int body_rows = split_tail ? tiles_m - 1 : tiles_m;
    const int body_amb = tiles_m == 1 ? tail_amb : mb;  // a one-row group is all tail
    out[n++] = WorkClass{g, 0, body_rows, body_rows * tiles_n * l, nk,
                         nk * stage_fraction(body_amb, mb) + tile_overhead_stages(), (double)body_amb / mb};
    if (split_tail)
      out[n++] = WorkClass{g, tiles_m - 1, 1, tiles_n * l, nk, nk * stage_fraction(tail_amb, mb) + tile_overhead_stages(),
                           (double)tail_amb / mb};
  }
  std::stable_sort(out, out + n, [](const WorkClass& x, const WorkClass& y) { return x.cost > y.cost; });
  return n;
}

// Stream-K workspace: two fp32 tile slots per workgroup, then the fold
// tree's arrival counters, kFoldLevels int32 per slot (padded to 256 bytes).
size_t partial_bytes_for(int cfg, int grid) { return (size_t)grid * 2 * kConfigs[cfg].bm * kConfigs[cfg].bn * 4; }
int counter_count(int grid) { return grid * 2 * kFoldLevels; }
size_t workspace_bytes_for(int cfg, int grid) {
  return partial_bytes_for(cfg, grid) + ((size_t)counter_count(grid) * 4 + 255) / 256 * 256;
}

// Cost model, in units of one 128x128 tile-stage of MFMA work. Smaller wave
// tiles dequantise more per MFMA; a tile costs a fixed prologue/epilogue on top
// of its stages; a stream-K plan adds its partial stores and folds and the
// kernel that clears its counters (plan_for).
double tile_unit(int cfg) {
  const TileConfig& tc = kConfigs[cfg];
  const double size = (double)tc.bm * tc.bn / (128.0 * 128.0);
  double eff = 1.0 + 0.35 * ((128.0 / tc.wm + 128.0 / tc.wn) / 2.0 - 1.0);
  // 32x32 wave tiles dequantise 16 VALU per MFMA (64x64: 8): a stage costs
  // about what the VALU takes, half a 64x64-wave stage for a quarter of the
  // MFMA work
  if (tc.wm < 64 && tc.wn < 64) eff = 2.4;
  return size * eff;
}

Plan plan_for(const int32_t* ps, int G, int cus, int cfg, int split) {
  Plan p{};
  p.cfg = cfg;
  p.split = split;
  const double unit = tile_unit(cfg);
  const double tile_overhead = tile_overhead_stages();
  int64_t tiles = 0, units = 0;
  for (int g = 0; g < G; ++g) {
    tiles += group_tiles(ps, g, cfg);
    units += group_tiles(ps, g, cfg) * group_stages(ps, g);
  }
  p.tiles = tiles;
  p.units = units;
  if (!split) {
    p.grid = (int)(tiles < cus ? tiles : cus);
    // the kernel's walk: rounds of `grid` tiles, heaviest class first,
    // alternately forwards and backwards over the workgroups
    static thread_local double load[1024];
    const int ns = p.grid < 1024 ? (p.grid > 0 ? p.grid : 1) : 1024;
    for (int s = 0; s < ns; ++s) load[s] = 0.0;
    WorkClass cls[kMaxClasses];
    const int nc = build_classes(ps, G, cfg, cls);
    int64_t t = 0;
    for (int c = 0; c < nc; ++c)
      for (int64_t i = 0; i < cls[c].tiles; ++i, ++t) {
        const int64_t r = t / ns, pos = t % ns;
        load[(r & 1) ? ns - 1 - pos : pos] += unit * cls[c].cost;
      }
    double mx = 0.0;
    for (int s = 0; s < ns; ++s) mx = load[s] > mx ? load[s] : mx;
    p.cost = mx;
    p.ws_bytes = 0;
  } else {
    const int cap = cus < kMaxSplitGrid ? cus : kMaxSplitGrid;
    p.grid = (int)(units < cap ? units : cap);
    WorkClass cls[kMaxClasses];
    const int nc = build_classes(ps, G, cfg, cls);
    int32_t ranges[kMaxSplitGrid + 1];
    // whole rounds first (up to four), then the water-filled unit ranges
    // (no units, e.g. every group empty or of k = 0: nothing to plan)
    const int64_t max_rounds = p.grid > 0 ? std::min<int64_t>(tiles / p.grid, 4) : -1;
    double best = 0.0;
    p.rounds = 0;
    for (int r = 0; r <= max_rounds; ++r) {
      const double m = hybrid_ranges(cls, nc, p.grid, r, ranges);
      if (r == 0 || m < best) {
        best = m;
        p.rounds = r;
      }
    }
    p.cost = unit * best + kClearKernelUnits;
    p.ws_bytes = workspace_bytes_for(cfg, p.grid);
  }
  return p;
}

// Picks the cheapest (config, mode): the best whole-tile plan, unless the best
// stream-K plan is modelled at least 15% cheaper (measured on the workloads:
// stream-K only pays when whole tiles would leave most compute units idle for
// long, e.g. few tiles with a long K). Stream-K plans whose workspace exceeds
// ws_cap are not candidates. Forced values are honoured.
Plan choose_plan(const int32_t* ps, int G, int cus, int force_cfg, int force_split, size_t ws_cap) {
  Plan best[2] = {};
  bool have[2] = {false, false};
  for (int c = 0; c < kNumConfigs; ++c) {
    if (force_cfg >= 0 && c != force_cfg) continue;
    for (int sp = 0; sp < 2; ++sp) {
      if (force_split >= 0 && sp != force_split) continue;
      const Plan p = plan_for(ps, G, cus, c, sp);
      if (sp == 1 && (p.units == 0 || p.ws_bytes > ws_cap)) continue;  // nothing to split, or no room
      if (!have[sp] || p.cost < best[sp].cost) {
        best[sp] = p;
        have[sp] = true;
      }
    }
  }
  if (have[1] && (!have[0] || best[1].cost < 0.85 * best[0].cost)) return best[1];
  if (have[0]) return best[0];
  return plan_for(ps, G, cus, force_cfg >= 0 ? force_cfg : 0, 0);
}

// The plan depends only on the sizes, the compute-unit count and the forced
// choices, and choosing it (every configuration and mode modelled) costs
// 10-25 us of host time for the larger calls; callers repeat the same sizes
// with other buffers, so each thread keeps its last few plans.
struct PlanKey {
  int G, cus, cfg, split;
  size_t ws_cap;
  int32_t sizes[4 * kMaxGroups];
  bool operator==(const PlanKey& o) const {
    return G == o.G && cus == o.cus && cfg == o.cfg && split == o.split && ws_cap == o.ws_cap &&
           std::memcmp(sizes, o.sizes, sizeof(int32_t) * 4 * G) == 0;
  }
};

Plan cached_plan(const int32_t* ps, int G, int cus, int force_cfg, int force_split, size_t ws_cap) {
  constexpr int kSlots = 8;
  static thread_local PlanKey keys[kSlots];
  static thread_local Plan plans[kSlots];
  static thread_local int used = 0, next = 0;
  PlanKey k{};
  k.G = G;
  k.cus = cus;
  k.cfg = force_cfg;
  k.split = force_split;
  k.ws_cap = ws_cap;
  std::memcpy(k.sizes, ps, sizeof(int32_t) * 4 * G);
  for (int i = 0; i < used; ++i)
    if (keys[i] == k) return plans[i];
  const Plan p = choose_plan(ps, G, cus, force_cfg, force_split, ws_cap);
  keys[next] = k;
  plans[next] = p;
  next = (next + 1) % kSlots;
  used = used < kSlots ? used + 1 : kSlots;
  return p;
}

bool aligned16(uint64_t p) { return (p & 15u) == 0; }

// The stream-K partials of nvfp4_grouped_gemm_scratch, for callers that
// cannot allocate: a fixed device array (each device that runs the library
// holds its own copy until the process ends). Kernels take its address as
// found by hipGetSymbolAddress (the name itself is a host-side stand-in),
// looked up once per device.
constexpr size_t kScratchBytes = NVFP4_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { t_last_hip_error = (int)e; return NVFP4_ERR_HIP; }
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_INVALID;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy (the device is current)
      if (e != hipSuccess || p == nullptr) { t_last_hip_error = (int)e; return NVFP4_ERR_HIP; }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return NVFP4_OK;
}

int launch(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, void* stream, const Plan& plan,
           void* workspace, int32_t* mx_status, int stages) {
  const TileConfig& tc = kConfigs[plan.cfg];
  KernelArgs args;
  std::memset(&args, 0, sizeof(args));
  WorkClass cls[kMaxClasses];
  const int nc = build_classes(ps, G, plan.cfg, cls);
  int64_t tiles = 0, units = 0;
  for (int c = 0; c < nc; ++c) {
    const int g = cls[c].g;
    ClassArgs& ca = args.cls[c];
    ca.m = ps[4 * g + 0];
    ca.n = ps[4 * g + 1];
    ca.k = ps[4 * g + 2];
    ca.l = ps[4 * g + 3];
    ca.a = reinterpret_cast<const uint8_t*>(abc[3 * g + 0]);
    ca.b = reinterpret_cast<const uint8_t*>(abc[3 * g + 1]);
    ca.c = reinterpret_cast<uint16_t*>(abc[3 * g + 2]);
    ca.sfa = reinterpret_cast<const uint8_t*>(sf[2 * g + 0]);
    ca.sfb = reinterpret_cast<const uint8_t*>(sf[2 * g + 1]);
    ca.tiles_m = cls[c].tiles_m;
    ca.tiles_n = (int32_t)ceil_div64(ca.n, tc.bn);
    ca.nk = cls[c].nk;
    ca.tm0 = cls[c].tm0;
    args.tile_prefix[c] = (int32_t)tiles;
    args.unit_prefix[c] = (int32_t)units;
    tiles += cls[c].tiles;
    units += cls[c].tiles * ca.nk;
  }
  for (int c = nc; c <= kMaxClasses; ++c) {
    args.tile_prefix[c] = (int32_t)tiles;
    args.unit_prefix[c] = (int32_t)units;
  }
  args.num_classes = nc > 0 ? nc : 1;
  args.split = plan.split;
  args.grid = plan.grid;
  args.status = mx_status;
  if (plan.split) {
    args.partials = reinterpret_cast<float*>(workspace);
    args.whole_tiles = plan.rounds * plan.grid;
    hybrid_ranges(cls, nc, plan.grid, plan.rounds, args.wg_unit);
  }
  if (tiles == 0 || plan.grid == 0) return NVFP4_OK;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  bool kpad = false;
  for (int g = 0; g < G; ++g) kpad = kpad || (ps[4 * g + 2] % 64 != 0);
  void (*kernel)(KernelArgs) = tc.kernel[plan.split ? 1 : 0][mx_status ? 1 : 0][kpad ? 1 : 0];
  const bool all_long = !plan.split && mx_status == nullptr && splits_k_everywhere(ps, G, plan.cfg);
  if (all_long) kernel = tc.kernel_ks2r[kpad ? 1 : 0];
  if (stages == 3) kernel = all_long ? tc.kernel_ks2r_ns3 : tc.kernel_ns3[plan.split ? 1 : 0];
  if (plan.split) {
    int32_t* counters = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) +
                                                   partial_bytes_for(plan.cfg, plan.grid));
    hipLaunchKernelGGL(nvfp4_clear_arrivals_kernel, dim3(1), dim3(kThreads), 0, st, counters, counter_count(plan.grid));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) { t_last_hip_error = (int)e; return NVFP4_ERR_HIP; }
  }
  hipLaunchKernelGGL(kernel, dim3(plan.grid), dim3(kThreads), 0, st, args);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) { t_last_hip_error = (int)e; return NVFP4_ERR_HIP; }
  return NVFP4_OK;
}

int sizes_ok(const int32_t* ps, int G) {
  if (G < 1 || G > kMaxGroups || ps == nullptr) return NVFP4_ERR_INVALID;
  int64_t tiles = 0, units = 0;
  for (int g = 0; g < G; ++g) {
    const int64_t m = ps[4 * g + 0], n = ps[4 * g + 1], k = ps[4 * g + 2], l = ps[4 * g + 3];
    if (m < 0 || n < 0 || k < 0 || l < 1) return NVFP4_ERR_INVALID;
    if (k % 32 != 0 || n % 8 != 0) return NVFP4_ERR_INVALID;
    // The kernel addresses A, B and the scale tensors with 32-bit buffer
    // offsets: each must stay below 2^31 bytes, and k below 2^22.
    // (x > lim / l stands for x * l > lim without overflowing)
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (k > (int64_t(1) << 22) || m > (int64_t(1) << 30) || n > (int64_t(1) << 30)) return NVFP4_ERR_INVALID;
    if (m * (k / 2) > lim / l || n * (k / 2) > lim / l || ceil_div64(m, 128) * 128 * (k / 16) > lim / l ||
        ceil_div64(n, 128) * 128 * (k / 16) > lim / l || m * n > (int64_t(1) << 40) / l)
      return NVFP4_ERR_INVALID;
    if (m == 0 || n == 0) continue;
    // tile and unit counts (of the smallest tile) stay within int32
    tiles += ceil_div64(m, 128) * ceil_div64(n, 128) * l;
    units += ceil_div64(m, 128) * ceil_div64(n, 128) * l * ceil_div64(k, kBK);
    if (tiles > (int64_t(1) << 30) || units > (int64_t(1) << 30)) return NVFP4_ERR_INVALID;
  }
  return NVFP4_OK;
}

// mx_status: non-null selects the power-of-two-scale kernels, which report
// there. Stream-K needs a workspace: without one (or with one too small for
// every stream-K plan) the call runs whole tiles, unless stream-K is forced.
int run_call(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, void* stream, int cfg, int split,
             void* workspace, size_t ws_bytes, int32_t* mx_status = nullptr, int stages = kStages) {
  const int rc = nvfp4_grouped_gemm_validate(ps, abc, sf, G);
  if (rc != NVFP4_OK) return rc;
  if (cfg < -1 || cfg >= kNumConfigs || split < -1 || split > 1) return NVFP4_ERR_CONFIG;
  int cus = 0;
  const int crc = device_cu_count(&cus);
  if (crc != NVFP4_OK) return crc;
  const size_t cap = workspace != nullptr ? ws_bytes : 0;
  // forced stream-K is planned without the cap, so that a plan with no room is an error
  const Plan plan = cached_plan(ps, G, cus, cfg, split, split == 1 ? SIZE_MAX : cap);
  if (plan.split && plan.ws_bytes > cap) return NVFP4_ERR_WORKSPACE;
  return launch(ps, abc, sf, G, stream, plan, workspace, mx_status, stages);
}

}  // namespace

extern "C" {

int nvfp4_grouped_gemm_validate(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G) {
  const int src = sizes_ok(ps, G);
  if (src != NVFP4_OK) return src;
  if (abc == nullptr || sf == nullptr) return NVFP4_ERR_INVALID;
  for (int g = 0; g < G; ++g) {
    const int64_t m = ps[4 * g + 0], n = ps[4 * g + 1], k = ps[4 * g + 2];
    if (m == 0 || n == 0) continue;
    const uint64_t a = abc[3 * g + 0], b = abc[3 * g + 1], c = abc[3 * g + 2];
    const uint64_t sa = sf[2 * g + 0], sb = sf[2 * g + 1];
    if (c == 0) return NVFP4_ERR_INVALID;
    if (!aligned16(c)) return NVFP4_ERR_MISALIGNED;
    if (k > 0) {
      if (a == 0 || b == 0 || sa == 0 || sb == 0) return NVFP4_ERR_INVALID;
      if (!aligned16(a) || !aligned16(b) || !aligned16(sa) || !aligned16(sb)) return NVFP4_ERR_MISALIGNED;
    }
  }
  return NVFP4_OK;
}

int nvfp4_grouped_gemm_device(const int32_t* d_ps, const uint64_t* d_abc, const uint64_t* d_sf, int G,
                              int tile_config, int32_t* d_status, void* stream) {
  if (G < 1 || G > kMaxDeviceGroups || d_ps == nullptr || d_abc == nullptr || d_sf == nullptr)
    return NVFP4_ERR_INVALID;
  if (!aligned16(reinterpret_cast<uint64_t>(d_ps)) || !aligned16(reinterpret_cast<uint64_t>(d_abc)) ||
      !aligned16(reinterpret_cast<uint64_t>(d_sf)) || (reinterpret_cast<uint64_t>(d_status) & 3u) != 0)
    return NVFP4_ERR_MISALIGNED;
  if (tile_config < -1 || tile_config >= kNumConfigs) return NVFP4_ERR_CONFIG;
  const int cfg = tile_config < 0 ? kDefaultDeviceConfig : tile_config;
  int cus = 0;
  const int crc = device_cu_count(&cus);
  if (crc != NVFP4_OK) return crc;
  const DeviceGroupArgs args{d_ps, d_abc, d_sf, d_status, G, cus};
  hipLaunchKernelGGL(kConfigs[cfg].device_kernel, dim3(cus), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), args);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) { t_last_hip_error = (int)e; return NVFP4_ERR_HIP; }
  return NVFP4_OK;
}

int64_t nvfp4_device_group_tiles(const int32_t* size, const uint64_t* ptrs, int tile_config) {
  if (size == nullptr || ptrs == nullptr || tile_config < -1 || tile_config >= kNumConfigs) return -1;
  return kConfigs[tile_config < 0 ? kDefaultDeviceConfig : tile_config].device_tiles(size, ptrs);
}

int nvfp4_num_tile_configs(void) { return kNumConfigs; }

int nvfp4_tile_config_info(int cfg, int* bm, int* bn, int* bk, int* threads) {
  if (cfg < 0 || cfg >= kNumConfigs) return NVFP4_ERR_CONFIG;
  if (bm) *bm = kConfigs[cfg].bm;
  if (bn) *bn = kConfigs[cfg].bn;
  if (bk) *bk = kBK;
  if (threads) *threads = kThreads;
  return NVFP4_OK;
}

int nvfp4_select_tile_config(const int32_t* ps, int G, int num_cus) {
  if (sizes_ok(ps, G) != NVFP4_OK || num_cus < 1) return NVFP4_ERR_INVALID;
  return choose_plan(ps, G, num_cus, -1, -1, SIZE_MAX).cfg;
}

int nvfp4_splits_k_over_waves(const int32_t* ps, int G, int num_cus, int cfg, int split) {
  if (sizes_ok(ps, G) != NVFP4_OK || num_cus < 1) return NVFP4_ERR_INVALID;
  if (cfg < -1 || cfg >= kNumConfigs || split < -1 || split > 1) return NVFP4_ERR_CONFIG;
  const Plan p = cached_plan(ps, G, num_cus, cfg, split, SIZE_MAX);
  return !p.split && splits_k_everywhere(ps, G, p.cfg) ? 1 : 0;
}

int nvfp4_launch_geometry(const int32_t* ps, int G, int num_cus, int cfg, int split, int64_t* total_tiles,
                          int* grid, int* split_used, size_t* workspace_bytes) {
  if (sizes_ok(ps, G) != NVFP4_OK || num_cus < 1) return NVFP4_ERR_INVALID;
  if (cfg < -1 || cfg >= kNumConfigs || split < -1 || split > 1) return NVFP4_ERR_CONFIG;
  const Plan p = cached_plan(ps, G, num_cus, cfg, split, SIZE_MAX);
  if (total_tiles) *total_tiles = p.tiles;
  if (grid) *grid = p.grid;
  if (split_used) *split_used = p.split;
  if (workspace_bytes) *workspace_bytes = p.ws_bytes;
  return p.cfg;
}

int nvfp4_split_plan(const int32_t* ps, int G, int num_cus, int cfg, int32_t* whole_tiles, int32_t* unit_ranges,
                     int max_ranges) {
  if (sizes_ok(ps, G) != NVFP4_OK || num_cus < 1) return NVFP4_ERR_INVALID;
  if (cfg < -1 || cfg >= kNumConfigs) return NVFP4_ERR_CONFIG;
  const Plan p = cached_plan(ps, G, num_cus, cfg, 1, SIZE_MAX);
  if (!p.split) return NVFP4_ERR_INVALID;  // nothing to split (no units)
  if (whole_tiles) *whole_tiles = p.rounds * p.grid;
  if (unit_ranges && max_ranges >= p.grid + 1) {
    WorkClass cls[kMaxClasses];
    const int nc = build_classes(ps, G, p.cfg, cls);
    hybrid_ranges(cls, nc, p.grid, p.rounds, unit_ranges);
  }
  return p.grid;
}

size_t nvfp4_workspace_bytes(const int32_t* ps, int G, int num_cus) {
  if (sizes_ok(ps, G) != NVFP4_OK || num_cus < 1) return 0;
  // enough for any plan the library may pick on this many compute units
  size_t need = 0;
  for (int c = 0; c < kNumConfigs; ++c) {
    const Plan p = plan_for(ps, G, num_cus, c, 1);
    need = p.ws_bytes > need ? p.ws_bytes : need;
  }
  return need;
}

int nvfp4_grouped_gemm_config(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, void* stream,
                              int cfg) {
  return run_call(ps, abc, sf, G, stream, cfg, -1, nullptr, 0);
}

int nvfp4_grouped_gemm(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, void* stream) {
  return run_call(ps, abc, sf, G, stream, -1, -1, nullptr, 0);
}

int nvfp4_grouped_gemm_ex(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, void* workspace,
                          size_t workspace_bytes, int tile_config, int split_mode, void* stream) {
  if (workspace != nullptr && (reinterpret_cast<uint64_t>(workspace) & 255u) != 0) return NVFP4_ERR_MISALIGNED;
  return run_call(ps, abc, sf, G, stream, tile_config, split_mode, workspace, workspace_bytes);
}

int nvfp4_grouped_gemm_stages(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, void* workspace,
                              size_t workspace_bytes, int tile_config, int split_mode, int stages, void* stream) {
  if (stages != 3 && stages != kStages) return NVFP4_ERR_CONFIG;
  if (workspace != nullptr && (reinterpret_cast<uint64_t>(workspace) & 255u) != 0) return NVFP4_ERR_MISALIGNED;
  return run_call(ps, abc, sf, G, stream, tile_config, split_mode, workspace, workspace_bytes, nullptr, stages);
}

int nvfp4_grouped_gemm_scratch(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, int tile_config,
                               int split_mode, void* stream) {
  // the host checks run first, so a rejected call makes no HIP call at all
  const int rc = nvfp4_grouped_gemm_validate(ps, abc, sf, G);
  if (rc != NVFP4_OK) return rc;
  if (tile_config < -1 || tile_config >= kNumConfigs || split_mode < -1 || split_mode > 1) return NVFP4_ERR_CONFIG;
  void* ws = nullptr;
  const int src = scratch_address(&ws);
  if (src != NVFP4_OK) return src;
  return run_call(ps, abc, sf, G, stream, tile_config, split_mode, ws, kScratchBytes);
}

int nvfp4_grouped_gemm_pow2(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, int32_t* d_status,
                            void* workspace, size_t workspace_bytes, int tile_config, int split_mode, void* stream) {
  if (d_status == nullptr) return NVFP4_ERR_INVALID;
  if ((reinterpret_cast<uint64_t>(d_status) & 3u) != 0) return NVFP4_ERR_MISALIGNED;
  if (workspace != nullptr && (reinterpret_cast<uint64_t>(workspace) & 255u) != 0) return NVFP4_ERR_MISALIGNED;
  return run_call(ps, abc, sf, G, stream, tile_config, split_mode, workspace, workspace_bytes, d_status);
}

size_t nvfp4_sf_bytes(int rows, int k, int l) {
  if (rows < 0 || k < 0 || l < 0) return 0;
  return (size_t)ceil_div64(rows, 128) * 128 * (size_t)ceil_div64(k, 64) * 4 * (size_t)l;
}

int nvfp4_last_hip_error(void) { return t_last_hip_error; }

const char* nvfp4_error_string(int code) {
  switch (code) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID: return "invalid argument (group count, sizes, divisibility or null pointer)";
    case NVFP4_ERR_MISALIGNED: return "pointer not aligned (16 bytes; 256 for a workspace)";
    case NVFP4_ERR_HIP: return "HIP runtime error (see nvfp4_last_hip_error)";
    case NVFP4_ERR_CONFIG: return "unknown tile configuration or split mode";
    case NVFP4_ERR_WORKSPACE: return "stream-K requested without a large enough workspace (or scratch)";
    default: return "unknown error code";
  }
}

}  // extern "C"
