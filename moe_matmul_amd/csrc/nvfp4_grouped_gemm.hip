// NVFP4 block-scaled grouped GEMM for gfx950 (MI355X).
//
// C_g[m, n] = sum_k (a[m,k] * sfa[m,k/16]) * (b[n,k] * sfb[n,k/16]), fp32
// accumulation, fp16 output (the contraction of the block-scaled MMA in
// submissions 506336 / 385043 / 499344, kernelindex.com "kernelbot nvfp4 group
// gemm"; layouts as in the header).
//
// Design (gfx950 first, not a translation of the pages' Blackwell kernels):
//  * Persistent grid of one 256-thread workgroup per compute unit. A workgroup
//    walks output tiles t = blockIdx.x, blockIdx.x + gridDim.x, ...; the group
//    of a tile is found by binary search over the per-group tile prefix sum
//    (the scheduler of submission 506336 keeps the same prefix), and tiles are
//    rastered M-fastest inside a group.
//  * Packed FP4 operand tiles are staged through two LDS buffers with 128-bit
//    loads. Each 64-byte row slab is stored with its four 16-byte chunks XOR
//    swizzled by (row >> 1) & 3, so the 128-bit reads of eight consecutive rows
//    touch all 32 banks.
//  * Scales come straight from the tiled layout into VGPRs: the 16-byte chunk
//    (r % 32) of a 512-byte atom holds rows r, r+32, r+64, r+96 for four
//    16-blocks, exactly the rows one lane feeds to a 32x32 MFMA.
//  * Exact dequantisation to f16 in registers: v_cvt_scalef32_pk_f16_fp4 with
//    scale 1.0 (E2M1 values are exact in f16), then one v_pk_mul_f16 by the
//    E4M3 scale (converted exactly with v_cvt_scalef32_pk_f16_fp8). |a*s| has
//    at most 6 significant bits, so the product is exact in f16, and the f16
//    MFMA products are exact in fp32. (The scaled conversion only applies the
//    exponent of its f32 scale, so the E4M3 mantissa needs the separate
//    multiply.)
//  * v_mfma_f32_32x32x16_f16 with B as the first operand, so each lane ends up
//    holding four consecutive columns of one output row.
//  * Inside each 64-K group the K order fed to the MFMA is permuted so that a
//    lane reads 32 consecutive FP4 codes (16 bytes) of its row: lane half h
//    takes K elements [32h, 32h+32) in four steps of 8. A and B use the same
//    permutation, so the sum is unchanged; each step of 8 lies inside one
//    16-block, so one scale covers it.
//  * Epilogue: fp32 -> fp16 (RNE) fused, 8-byte stores masked to m and n.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "nvfp4_grouped_gemm.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int N>
using ScaleVec = uint32_t __attribute__((ext_vector_type(N)));

constexpr int kMaxGroups = NVFP4_MAX_GROUPS;
constexpr int kThreads = 256;
constexpr int kBK = 128;          // K elements per pipeline stage
constexpr int kRowBytes = kBK / 2; // packed bytes per row per stage
constexpr int kAtomBytes = 512;    // one 128-row x 64-K scale atom
constexpr int kBufferWord3 = 0x00020000;  // gfx9 buffer resource word 3 (raw, 32-bit data)

struct GroupArgs {
  const uint8_t* a;
  const uint8_t* b;
  uint16_t* c;
  const uint8_t* sfa;
  const uint8_t* sfb;
  int32_t m, n, k, l;
  int32_t tiles_m, tiles_n;
  int32_t pad0, pad1;
};

struct KernelArgs {
  GroupArgs g[kMaxGroups];
  int32_t prefix[kMaxGroups + 1];  // prefix[g] = first tile of group g
  int32_t num_groups;
};

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

// Raw buffer resource (4 SGPRs): 48-bit base, stride 0, num_records bytes;
// offsets at or past num_records read 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int64_t num_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const int n = num_bytes <= 0 ? 0 : (num_bytes >= 0x7fffffff ? 0x7fffffff : (int)num_bytes);
  return i32x4{(int32_t)(uint32_t)b, (int32_t)((uint32_t)(b >> 32) & 0xFFFFu), n, kBufferWord3};
}

// 16 bytes per lane from global (buffer, bounds-checked) straight into LDS at
// lds_block + 16 * lane (M0 holds the wave's LDS base). Issued as inline asm so
// the compiler does not treat it as an LDS write it must wait for: the kernel
// tracks these loads itself with exact vmcnt waits.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint8_t* lds_block, int voffset) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_block));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc) : "memory", "m0");
}

// Workgroup barrier without the compiler's release fence (which would wait for
// every outstanding load): LDS reads of this wave are complete, then s_barrier.
__device__ __forceinline__ void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
  int64_t a_rem, b_rem;    // bytes from the tile base to the end of the operand
  const uint8_t* sf_row;   // this wave's scale atom row (nullptr: none)
  int64_t sf_rem;
  uint16_t* c;             // C of the tile's batch
  int M, N, kbytes, nk, row0, col0;
};

template <int BM, int BN, int WM, int WN, int NS>
struct GemmKernel {
  static constexpr int MB = WM / 32;
  static constexpr int NB = WN / 32;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = BN * kRowBytes;
  static constexpr int SF_ATOMS = (BM + BN) / 128;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SF_ATOMS * 1024;
  static constexpr int A_INSTR = A_BYTES / 1024 / 4;  // 1 KiB direct loads per wave per stage
  static constexpr int B_INSTR = B_BYTES / 1024 / 4;
  static_assert((BM / WM) * (BN / WN) == kThreads / 64, "four waves per workgroup");
  static_assert(WM <= 128 && WN <= 128 && 128 % WM == 0 && 128 % WN == 0, "wave tile inside one scale atom");
  static_assert(A_INSTR >= 1 && B_INSTR >= 1 && SF_ATOMS <= 4, "tile shape");
  static_assert(NS >= 2 && NS <= 4 && NS * STAGE_BYTES <= 160 * 1024, "LDS stages");
  // direct loads one wave issues per stage (without / with a scale atom row)
  static constexpr int L0 = A_INSTR + B_INSTR;
  static constexpr int L1 = A_INSTR + B_INSTR + 1;

  // Packed FP4 of one 64-K half stage for this lane (one 16-byte chunk per 32-row
  // block) and the lane's two E4M3 scales per block.
  struct Raw {
    u32x4 a[MB];
    u32x4 b[NB];
    uint32_t sa[MB];
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

  uint8_t* smem;
  int wave, wm, wn, h, lr, lane;

  __device__ __forceinline__ TileCtx setup(const KernelArgs& args, int tile) const {
    int lo = 0, hi = args.num_groups - 1;
    while (lo < hi) {  // group of the tile: binary search over the tile prefix sum
      const int mid = (lo + hi + 1) >> 1;
      if (args.prefix[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const GroupArgs& G = args.g[lo];
    const int M = G.m, N = G.n, K = G.k;
    const int tiles_m = G.tiles_m;
    const int per_l = tiles_m * G.tiles_n;
    const int rest = tile - args.prefix[lo];
    const int li = rest / per_l;
    const int r2 = rest - li * per_l;
    const int tm = r2 % tiles_m;  // M-fastest raster inside the group
    const int tn = r2 / tiles_m;
    const int kbytes = K >> 1;
    const int Kt = K >> 6;
    const int Mt = (M + 127) >> 7;
    const int Nt = (N + 127) >> 7;
    TileCtx t;
    t.M = M;
    t.N = N;
    t.kbytes = kbytes;
    t.nk = (K + kBK - 1) / kBK;
    t.row0 = tm * BM;
    t.col0 = tn * BN;
    t.a_tile = G.a + ((size_t)li * M + (size_t)tm * BM) * kbytes;
    t.b_tile = G.b + ((size_t)li * N + (size_t)tn * BN) * kbytes;
    t.a_rem = (int64_t)(M - tm * BM) * kbytes;
    t.b_rem = (int64_t)(N - tn * BN) * kbytes;
    t.c = G.c + (size_t)li * M * N;
    t.sf_row = nullptr;
    t.sf_rem = 0;
    if (wave < BM / 128) {
      const int atom = tm * (BM / 128) + wave;
      t.sf_row = G.sfa + ((size_t)li * Mt + atom) * Kt * kAtomBytes;
      t.sf_rem = atom < Mt ? (int64_t)Kt * kAtomBytes : 0;
    } else if (wave < SF_ATOMS) {
      const int atom = tn * (BN / 128) + (wave - BM / 128);
      t.sf_row = G.sfb + ((size_t)li * Nt + atom) * Kt * kAtomBytes;
      t.sf_rem = atom < Nt ? (int64_t)Kt * kAtomBytes : 0;
    }
    return t;
  }

  // Direct loads of stage kt (A, B and the scale atoms) into LDS buffer buf.
  __device__ __forceinline__ void issue_stage(const TileCtx& t, int kt, int buf) const {
    uint8_t* st = smem + buf * STAGE_BYTES;
    // Lane -> (row, chunk) of its 16 bytes in a 1 KiB direct load: 16 rows of 64
    // bytes; the physical chunk is lane & 3, the global chunk undoes the swizzle.
    const int voff = (wave * 16 + (lane >> 2)) * t.kbytes + (((lane & 3) ^ swz(lane >> 2)) << 4);
    // the K offset goes into the resource base, so the range check also
    // zero-fills past the end of the last row
    const int64_t kb0 = (int64_t)kt * kRowBytes;
    const i32x4 ra = make_rsrc(t.a_tile + kb0, t.a_rem - kb0);
    const i32x4 rb = make_rsrc(t.b_tile + kb0, t.b_rem - kb0);
#pragma unroll
    for (int u = 0; u < A_INSTR; ++u) load_lds16(ra, st + (u * 4 + wave) * 1024, voff + u * 64 * t.kbytes);
#pragma unroll
    for (int u = 0; u < B_INSTR; ++u)
      load_lds16(rb, st + A_BYTES + (u * 4 + wave) * 1024, voff + u * 64 * t.kbytes);
    if (wave < SF_ATOMS) {
      // two 64-K groups (1 KiB) of this atom row; groups past k read 0
      const int64_t q0 = (int64_t)kt * 2 * kAtomBytes;
      load_lds16(make_rsrc(t.sf_row + q0, t.sf_rem - q0), st + A_BYTES + B_BYTES + wave * 1024, lane * 16);
    }
  }

  // ds_reads of one half stage (kk) from LDS buffer buf.
  __device__ __forceinline__ void read_half(Raw& r, int buf, int kk) const {
    const uint8_t* As = smem + buf * STAGE_BYTES;
    const uint8_t* Bs = As + A_BYTES;
    const uint8_t* Ss = Bs + B_BYTES;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      r.a[i] = *reinterpret_cast<const u32x4*>(As + lds_off(wm * WM + i * 32 + lr, kk * 2 + h));
#pragma unroll
    for (int j = 0; j < NB; ++j)
      r.b[j] = *reinterpret_cast<const u32x4*>(Bs + lds_off(wn * WN + j * 32 + lr, kk * 2 + h));
    const ScaleVec<MB> sa = *reinterpret_cast<const ScaleVec<MB>*>(
        Ss + ((wm * WM) >> 7) * 1024 + kk * 512 + lr * 16 + (((wm * WM) & 127) >> 5) * 4);
    const ScaleVec<NB> sb = *reinterpret_cast<const ScaleVec<NB>*>(
        Ss + (BM / 128 + ((wn * WN) >> 7)) * 1024 + kk * 512 + lr * 16 + (((wn * WN) & 127) >> 5) * 4);
#pragma unroll
    for (int i = 0; i < MB; ++i) r.sa[i] = sa[i];
#pragma unroll
    for (int j = 0; j < NB; ++j) r.sb[j] = sb[j];
  }

  // The lane's two E4M3 scales (16-blocks 2h, 2h+1 of the half) -> f16, exactly.
  __device__ __forceinline__ void convert_scales(Scales& s, const Raw& r) const {
    const int hshift = h * 16;
#pragma unroll
    for (int i = 0; i < MB; ++i) s.a[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sa[i] >> hshift, 1.0f, false);
#pragma unroll
    for (int j = 0; j < NB; ++j) s.b[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.sb[j] >> hshift, 1.0f, false);
  }

  // Operand fragments of substep S (K elements 8S..8S+7 of the lane's 32).
  template <int S>
  __device__ __forceinline__ void dequant(Frags& f, const Raw& r, const Scales& s) const {
#pragma unroll
    for (int i = 0; i < MB; ++i) f.a[i] = dequant8(r.a[i][S], s.a[i][S >> 1]);
#pragma unroll
    for (int j = 0; j < NB; ++j) f.b[j] = dequant8(r.b[j][S], s.b[j][S >> 1]);
  }

  __device__ __forceinline__ static void mfmas(f32x16 (&acc)[MB][NB], const Frags& f) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  }

  // One substep, in a scheduling region of its own: the MFMAs of `use`
  // interleaved with the dequantisation of the next substep into `fill`
  // (8 VALU per pair of fragments: VALU_PER_MFMA = 4 for 128x128 wave tiles).
  // With CONVERT, the next half's scales are converted here as well.
  template <int NEXT_S, bool CONVERT>
  __device__ __forceinline__ void step(f32x16 (&acc)[MB][NB], const Frags& use, Frags& fill, const Raw& src,
                                       Scales& ssrc) const {
    constexpr int VALU = (MB + NB) * 8 + (CONVERT ? 2 * (MB + NB) : 0);
    constexpr int PER = (VALU + MB * NB - 1) / (MB * NB);
    if (CONVERT) convert_scales(ssrc, src);
    dequant<NEXT_S>(fill, src, ssrc);
    mfmas(acc, use);
#pragma unroll
    for (int q = 0; q < MB * NB; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVALU, PER, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- the stage stream ----
  // The stages of a workgroup's tiles form one sequence; global stage X lives in
  // LDS buffer X % NS. Loads run up to NS stages ahead and may run into the next
  // tile (never further). `issued` is the next global stage to issue.
  struct Stream {
    int issued;  // next global stage to issue
    int g0;      // first global stage of the current tile
    int end;     // one past the last issuable stage (end of the next tile)
  };

  __device__ __forceinline__ void issue_global(Stream& q, const TileCtx& t, const TileCtx& tn) const {
    const int x = q.issued++;
    if (x < q.g0 + t.nk) issue_stage(t, x - q.g0, x % NS);
    else issue_stage(tn, x - q.g0 - t.nk, x % NS);
  }

  // Wait until at most `stages` stages of this wave's loads are outstanding.
  __device__ __forceinline__ void wait_stages(int stages) const {
    const int n = stages * (wave < SF_ATOMS ? L1 : L0);
    switch (n) {
      case L0: wait_vmem<L0>(); break;
      case L1: wait_vmem<L1>(); break;
      case 2 * L0: wait_vmem<2 * L0>(); break;
      case 2 * L1: wait_vmem<2 * L1>(); break;
      default: wait_vmem<0>(); break;
    }
  }

  // One tile. On entry the stream holds this tile's first stages (issued earlier).
  __device__ __forceinline__ void mainloop(f32x16 (&acc)[MB][NB], const TileCtx& t, const TileCtx& tn,
                                           Stream& q) const {
    Raw r0, r1;
    Scales s0, s1;
    Frags f0, f1;
    wait_vmem_all();  // stage g0 landed (and the last tile's C stores are done)
    block_sync();
    // top up: every buffer of a stage before g0 is free now
    while (q.issued < q.end && q.issued < q.g0 + NS) issue_global(q, t, tn);
    read_half(r0, q.g0 % NS, 0);
    convert_scales(s0, r0);
    dequant<0>(f0, r0, s0);
    for (int kt = 0; kt < t.nk; ++kt) {
      const int g = q.g0 + kt;
      // ---- first half (K 0..63 of the stage): raw data in r0 ----
      read_half(r1, g % NS, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, MB + NB + 2, 0);
      step<1, false>(acc, f0, f1, r0, s0);
      step<2, false>(acc, f1, f0, r0, s0);
      step<3, false>(acc, f0, f1, r0, s0);
      step<0, true>(acc, f1, f0, r1, s1);
      // ---- second half: raw data in r1. Stage g+1 must have landed before its
      // first half is read; every wave is done with stage g's buffer here, so
      // stage g + NS can take it.
      if (kt + 1 < t.nk) {
        const int after = q.issued - (g + 2);  // stages issued after g+1
        wait_stages(after < 0 ? 0 : after);
      }
      block_sync();
      if (q.issued < q.end && q.issued <= g + NS) issue_global(q, t, tn);
      read_half(r0, (g + 1) % NS, 0);  // unused after the last stage
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, MB + NB + 2, 0);
      step<1, false>(acc, f0, f1, r1, s1);
      step<2, false>(acc, f1, f0, r1, s1);
      step<3, false>(acc, f0, f1, r1, s1);
      step<0, true>(acc, f1, f0, r0, s0);
    }
  }

  // fp32 -> fp16 (RNE), 8-byte stores masked to m and n.
  __device__ __forceinline__ void epilogue(const f32x16 (&acc)[MB][NB], const TileCtx& t) const {
    const int row0 = t.row0 + wm * WM;
    const int col0 = t.col0 + wn * WN;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int row = row0 + i * 32 + lr;
      if (row < t.M) {
        uint16_t* crow = t.c + (size_t)row * t.N;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = col0 + j * 32 + e * 8 + h * 4;
            if (col < t.N) {
              const f16x4 v = {(_Float16)acc[i][j][e * 4 + 0], (_Float16)acc[i][j][e * 4 + 1],
                               (_Float16)acc[i][j][e * 4 + 2], (_Float16)acc[i][j][e * 4 + 3]};
              *reinterpret_cast<f16x4*>(crow + col) = v;
            }
          }
        }
      }
    }
  }
};

// Stage layout in LDS (bytes): [A: BM rows x 64][B: BN rows x 64]
// [scale atoms: (BM + BN) / 128 atom rows x 2 k-groups x 512]; A and B rows are
// swizzled by lds_off, the scale atoms are stored as in global memory.
template <int BM, int BN, int WM, int WN, int NS>
__global__ __launch_bounds__(kThreads, 1) void nvfp4_grouped_gemm_kernel(KernelArgs args) {
  using K = GemmKernel<BM, BN, WM, WN, NS>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * K::STAGE_BYTES];
  K k;
  k.smem = smem;
  const int tid = threadIdx.x;
  k.lane = tid & 63;
  k.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  k.wm = k.wave / K::WAVES_N;
  k.wn = k.wave % K::WAVES_N;
  k.h = k.lane >> 5;
  k.lr = k.lane & 31;
  const int total = args.prefix[args.num_groups];

  int tile = blockIdx.x;
  if (tile >= total) return;
  TileCtx t = k.setup(args, tile);
  int next = tile + gridDim.x;
  TileCtx tn = next < total ? k.setup(args, next) : t;
  typename K::Stream q;
  q.issued = 0;
  q.g0 = 0;
  q.end = t.nk + (next < total ? tn.nk : 0);
  while (q.issued < q.end && q.issued < NS) k.issue_global(q, t, tn);  // all buffers are free
  while (true) {
    f32x16 acc[K::MB][K::NB];
#pragma unroll
    for (int i = 0; i < K::MB; ++i)
#pragma unroll
      for (int j = 0; j < K::NB; ++j) acc[i][j] = f32x16{};
    if (t.nk > 0) k.mainloop(acc, t, tn, q);
    k.epilogue(acc, t);
    if (next >= total) break;
    // advance: the next tile becomes current, the one after it joins the stream
    q.g0 += t.nk;
    tile = next;
    t = tn;
    next = tile + gridDim.x;
    if (next < total) tn = k.setup(args, next);
    q.end = q.g0 + t.nk + (next < total ? tn.nk : 0);
  }
}

// ---------------------------------------------------------------------------
// Tile configurations
// ---------------------------------------------------------------------------

struct TileConfig {
  int bm, bn, wm, wn;
  void (*kernel)(KernelArgs);
};

constexpr int kStages = 4;  // LDS pipeline depth (4 x 36 KiB for 256x256 tiles)

const TileConfig kConfigs[] = {
    {256, 256, 128, 128, nvfp4_grouped_gemm_kernel<256, 256, 128, 128, kStages>},
    {128, 256, 64, 128, nvfp4_grouped_gemm_kernel<128, 256, 64, 128, kStages>},
    {256, 128, 128, 64, nvfp4_grouped_gemm_kernel<256, 128, 128, 64, kStages>},
    {128, 128, 64, 64, nvfp4_grouped_gemm_kernel<128, 128, 64, 64, kStages>},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

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

int64_t tiles_of(const int32_t* ps, int g, int cfg) {
  const int32_t m = ps[4 * g + 0], n = ps[4 * g + 1], l = ps[4 * g + 3];
  if (m == 0 || n == 0) return 0;
  return ceil_div64(m, kConfigs[cfg].bm) * ceil_div64(n, kConfigs[cfg].bn) * l;
}

// Makespan estimate (in units of 128x128x64 MFMA work) of strided assignment of
// the tiles to `slots` persistent workgroups, plus a per-tile overhead and a
// penalty for the smaller wave tiles' extra dequantisation work.
double estimate_cost(const int32_t* ps, int G, int slots, int cfg) {
  const TileConfig& tc = kConfigs[cfg];
  const double unit = (double)tc.bm * tc.bn / (128.0 * 128.0);
  // dequant work per MFMA grows with 1/wm + 1/wn; 128x128 wave tiles are the reference
  const double eff = 1.0 + 0.35 * ((128.0 / tc.wm + 128.0 / tc.wn) / 2.0 - 1.0);
  double load[1024];
  const int ns = slots < 1024 ? slots : 1024;
  for (int s = 0; s < ns; ++s) load[s] = 0.0;
  int64_t t = 0;
  for (int g = 0; g < G; ++g) {
    const int64_t nt = tiles_of(ps, g, cfg);
    const double work = unit * eff * (ps[4 * g + 2] / 64.0 + 4.0);
    for (int64_t i = 0; i < nt; ++i, ++t) load[t % ns] += work;
  }
  double mx = 0.0;
  for (int s = 0; s < ns; ++s) mx = load[s] > mx ? load[s] : mx;
  return mx;
}

int select_config(const int32_t* ps, int G, int cus) {
  int best = 0;
  double best_cost = 0.0;
  for (int c = 0; c < kNumConfigs; ++c) {
    const double cost = estimate_cost(ps, G, cus, c);
    if (c == 0 || cost < best_cost) { best = c; best_cost = cost; }
  }
  return best;
}

bool aligned16(uint64_t p) { return (p & 15u) == 0; }

}  // namespace

extern "C" {

int nvfp4_grouped_gemm_validate(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G) {
  if (G < 1 || G > kMaxGroups || ps == nullptr || abc == nullptr || sf == nullptr) return NVFP4_ERR_INVALID;
  int64_t total = 0;
  for (int g = 0; g < G; ++g) {
    const int64_t m = ps[4 * g + 0], n = ps[4 * g + 1], k = ps[4 * g + 2], l = ps[4 * g + 3];
    if (m < 0 || n < 0 || k < 0 || l < 1) return NVFP4_ERR_INVALID;
    if (k % 64 != 0 || n % 8 != 0) return NVFP4_ERR_INVALID;
    // The kernel addresses A, B and the scale tensors with 32-bit buffer
    // offsets: each must stay below 2^31 bytes, and k below 2^22.
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (k > (int64_t(1) << 22) || m * (k / 2) * l > lim || n * (k / 2) * l > lim ||
        ceil_div64(m, 128) * 128 * (k / 16) * l > lim || ceil_div64(n, 128) * 128 * (k / 16) * l > lim ||
        m > (int64_t(1) << 30) || n > (int64_t(1) << 30) || m * n * l > (int64_t(1) << 40))
      return NVFP4_ERR_INVALID;
    if (m == 0 || n == 0) continue;
    total += ceil_div64(m, 128) * ceil_div64(n, 128) * l;
    if (total > (int64_t(1) << 30)) return NVFP4_ERR_INVALID;
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
  if (G < 1 || G > kMaxGroups || ps == nullptr || num_cus < 1) return NVFP4_ERR_INVALID;
  return select_config(ps, G, num_cus);
}

int nvfp4_launch_geometry(const int32_t* ps, int G, int num_cus, int cfg, int64_t* total_tiles, int* grid) {
  if (G < 1 || G > kMaxGroups || ps == nullptr || num_cus < 1) return NVFP4_ERR_INVALID;
  if (cfg < -1 || cfg >= kNumConfigs) return NVFP4_ERR_CONFIG;
  if (cfg < 0) cfg = select_config(ps, G, num_cus);
  int64_t total = 0;
  for (int g = 0; g < G; ++g) total += tiles_of(ps, g, cfg);
  if (total_tiles) *total_tiles = total;
  if (grid) *grid = (int)(total < num_cus ? total : num_cus);
  return cfg;
}

int nvfp4_grouped_gemm_config(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G,
                              void* stream, int cfg) {
  const int rc = nvfp4_grouped_gemm_validate(ps, abc, sf, G);
  if (rc != NVFP4_OK) return rc;
  if (cfg < -1 || cfg >= kNumConfigs) return NVFP4_ERR_CONFIG;
  int cus = 0;
  const int crc = device_cu_count(&cus);
  if (crc != NVFP4_OK) return crc;
  if (cfg < 0) cfg = select_config(ps, G, cus);
  const TileConfig& tc = kConfigs[cfg];

  KernelArgs args;
  std::memset(&args, 0, sizeof(args));
  int64_t total = 0;
  for (int g = 0; g < G; ++g) {
    GroupArgs& ga = args.g[g];
    ga.m = ps[4 * g + 0];
    ga.n = ps[4 * g + 1];
    ga.k = ps[4 * g + 2];
    ga.l = ps[4 * g + 3];
    ga.a = reinterpret_cast<const uint8_t*>(abc[3 * g + 0]);
    ga.b = reinterpret_cast<const uint8_t*>(abc[3 * g + 1]);
    ga.c = reinterpret_cast<uint16_t*>(abc[3 * g + 2]);
    ga.sfa = reinterpret_cast<const uint8_t*>(sf[2 * g + 0]);
    ga.sfb = reinterpret_cast<const uint8_t*>(sf[2 * g + 1]);
    ga.tiles_m = (int32_t)ceil_div64(ga.m, tc.bm);
    ga.tiles_n = (int32_t)ceil_div64(ga.n, tc.bn);
    args.prefix[g] = (int32_t)total;
    total += tiles_of(ps, g, cfg);
  }
  for (int g = G; g <= kMaxGroups; ++g) args.prefix[g] = (int32_t)total;
  args.num_groups = G;
  if (total == 0) return NVFP4_OK;

  const int grid = (int)(total < cus ? total : cus);
  hipLaunchKernelGGL(tc.kernel, dim3(grid), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream), args);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) { t_last_hip_error = (int)e; return NVFP4_ERR_HIP; }
  return NVFP4_OK;
}

int nvfp4_grouped_gemm(const int32_t* ps, const uint64_t* abc, const uint64_t* sf, int G, void* stream) {
  return nvfp4_grouped_gemm_config(ps, abc, sf, G, stream, -1);
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
    case NVFP4_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case NVFP4_ERR_HIP: return "HIP runtime error (see nvfp4_last_hip_error)";
    case NVFP4_ERR_CONFIG: return "unknown tile configuration";
    default: return "unknown error code";
  }
}

}  // extern "C"
