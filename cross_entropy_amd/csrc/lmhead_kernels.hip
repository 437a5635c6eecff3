// lmhead_kernels.hip -- gfx950 (CDNA4) kernels of the fused LM-head
// log-prob / entropy head.
//
// Method (google/tunix pull request #2913, the fused sharded log-prob head;
// SkyRL issue "[tx] support long sequence", "4. Chunked LM Head"):
//   forward : one pass over each tile of logits z = h W^T keeps, per token,
//             a running max, the exp-sum and the exp-weighted sum of z, and
//             picks the target logit by index compare (a one-hot select);
//             vocabulary splits are merged by log-sum-exp.
//   backward: the logits are recomputed tile by tile, their cotangent dz is
//             formed in one elementwise pass and rounded to bf16, and both
//             gradient matmuls (dh = dz W, dW = dz^T h) read that one dz.
//
// Every contraction runs on one MFMA tile core: a 256 x 256 output tile per
// 256-thread workgroup (4 wave64s as 2 x 2, each owning 128 x 128, its 256
// f32 accumulators in AGPRs), v_mfma_f32_16x16x32_bf16. One wave per SIMD
// halves the LDS fragment traffic per MFMA against two waves of 128 x 64,
// and the short 16x16 MFMA keeps accumulator traffic through the register
// file low; the wave hides its own latencies through the order in which it
// issues work (see mma_tile). K is staged through two 64-wide LDS slices
// filled by direct-to-LDS loads (global_load_lds_dwordx4), so no VGPRs hold
// staged data. Slice rows are 128 bytes with a 16-byte-chunk XOR swizzle,
// which keeps the fragment reads free of bank conflicts. An A operand stored
// MN-contiguous (W and the cotangent in the backward) is staged as it lies
// and read with transposed LDS reads; the hidden states enter the dW GEMM
// through a transposed copy.
//
// MFMA 16x16x32 register layout used throughout (wave64): lane l supplies
// row (l % 16) of A and column (l % 16) of B with the 8 K values
// 8*(l/16) .. 8*(l/16)+7; result register r of lane l holds
// D[4*(l/16) + r][l % 16].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lmhead_internal.h"

namespace lmh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                    // 4 waves
constexpr int kTile = 256;                       // output tile edge
constexpr int kBK = 64;                          // K per LDS slice
constexpr int kRowBytes = kBK * 2;               // 128 B per staged row
constexpr int kOpBytes = kTile * kRowBytes;      // 32 KB per operand slice
constexpr int kStageBytes = 2 * kOpBytes;        // A + B
constexpr int kRingBytes = 2 * kStageBytes;      // two slices in flight
constexpr int kLdsBytes = kRingBytes + 1024;     // + a 1 KB scratch row (see mma_tile)
constexpr int kNB = 8;                           // 16-wide MFMA blocks per wave edge

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegBig = -1.0e30f;              // "minus infinity" that keeps 0 * x finite

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_mul_legacy_f32: a product that is +0 when either factor is 0, whatever
// the other holds (inf and NaN included); IEEE otherwise.
extern "C" __device__ float lmh_fmul_legacy(float, float) __asm("llvm.amdgcn.fmul.legacy");

// NaN-propagating max (v_maximum3_f32 on gfx950): a NaN logit must reach the
// statistics, where fmaxf would drop it.
__device__ __forceinline__ float nan_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);   // round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}

// Workgroup id -> virtual id such that each XCD (workgroups are dealt to the
// 8 XCDs round-robin) runs a contiguous range of virtual ids; neighbouring
// tiles then share that XCD's L2. grid is a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  const int per = grid >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// Virtual id -> (tile_m, tile_n), walking groups of `group` M-tiles
// column by column, so 32 concurrent workgroups cover a compact patch.
__device__ __forceinline__ void raster(int vid, int n_m, int n_n, int group, int& tm, int& tn) {
  const int per_group = group * n_n;
  const int g = vid / per_group;
  const int first = g * group;
  const int gsz = min(group, n_m - first);
  const int in = vid - g * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

// Wave index as a scalar, so the per-wave LDS and address arithmetic stays
// on the scalar unit.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Pin a 4-register accumulator block in AGPRs up to this point: the
// epilogue's reads of it then become copies right here, instead of one bulk
// copy of all 256 accumulators into VGPRs at the end of the loop.
__device__ __forceinline__ void pin_acc(f32x4& a) { asm volatile("" : "+a"(a)); }

// ---------------------------------------------------------------------------
// Staging. An operand of the core: a K-contiguous operand holds element
// (row, k) at base[row * ld + k], rows at or past `rows` are read as row
// rows-1 (their results are discarded or masked by the epilogues), so every
// load stays in bounds; an MN-contiguous operand holds element (m, k) at
// base[k * ld + m], columns m at or past `rows` (a multiple of 8) are read
// as one of the last 8, and its slice at K offset tail_k (if any) is read
// from `tail` (64 rows of stride ld) instead: a slice that would run past
// the end of the matrix. Byte offsets within a tile stay below 2^32 (the
// host bounds ld).
struct Operand {
  const uint16_t* base;
  int64_t ld;
  int rows;
  const uint16_t* tail = nullptr;
  int tail_k = -1;
};

// XOR applied to the 16-byte chunk index of staged row r (8 chunks per row):
// 8 consecutive rows read at one logical chunk hit 8 distinct 16-byte bank
// groups of the 128-byte bank line.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

// MN-contiguous slice rows (64 K-rows of 256 m, 512 bytes each): chunk XOR by
// 2 * (k % 4), so the 4 K-rows one 16-lane group of a transposed read visits
// land on distinct bank groups, and by 8 for K-rows with bit 3 set, so the
// two 16-lane groups served together (32 lanes x 8 bytes per pass over the 64
// banks), 8 K-rows apart, fall on opposite halves of the bank line. Without
// the second term every transposed read took two extra cycles (measured:
// SQ_LDS_BANK_CONFLICT, two per read).
__device__ __forceinline__ int swz_mn(int k) { return (2 * (k & 3)) ^ (8 * ((k >> 3) & 1)); }

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One direct-to-LDS load: 64 lanes x 16 B land at m0 + 16 * lane; lane l
// reads 16 bytes at sbase + voff(l) (scalar base, 32-bit per-lane offset).
// Issued as inline asm so the compiler does not add a vmcnt(0) in front of
// every LDS read of the ring; completion is awaited explicitly (wait_vm)
// before the barrier that publishes a slice.
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds_wave_base)
               : "memory");
}

// s_waitcnt vmcnt(n) leaving expcnt / lgkmcnt alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Per-lane byte offsets of a wave's 8 loads of one operand slice. Load q of
// wave w fills 1 KB of the slice at byte 8 KB * w + 1 KB * q:
//  K-contiguous: rows 64 w + 8 q .. +7; lane l fills physical chunk l % 8
//    of row 64 w + 8 q + l / 8 with the logical chunk the swizzle puts there;
//  MN-contiguous: K-rows 16 w + 2 q, +1; lane l fills physical chunk l % 32
//    of K-row 16 w + 2 q + l / 32 likewise (chunks past `rows` clamped).
struct LoadOffs {
  uint32_t o[8];
};

template <bool MN>
__device__ __forceinline__ LoadOffs load_offsets(const Operand& op) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  LoadOffs d;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if (MN) {
      const int r = wave * 16 + 2 * q + (lane >> 5);
      const int c = min((lane & 31) ^ swz_mn(r), ((op.rows + 7) >> 3) - 1);
      d.o[q] = (uint32_t)((int64_t)r * op.ld * 2) + (uint32_t)(c * 16);
    } else {
      const int r = wave * 64 + 8 * q + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const int rr = min(r, op.rows - 1);
      d.o[q] = (uint32_t)((int64_t)rr * op.ld * 2) + (uint32_t)(c * 16);
    }
  }
  return d;
}

// Scalar base of a slice load, in SGPRs: operand op's slice at K offset k0
// (`own`), or that of the same-shaped operand starting at `base`.
template <bool MN>
__device__ __forceinline__ const void* slice_base(const Operand& op, const uint16_t* base, int k0, bool own) {
  const char* b = reinterpret_cast<const char*>(base) + 2 * (MN ? (int64_t)k0 * op.ld : (int64_t)k0);
  if (MN && own && k0 == op.tail_k) b = reinterpret_cast<const char*>(op.tail);
  const uint64_t bu = reinterpret_cast<uint64_t>(b);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)bu);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane j
// receives element (j & 3) of the 8-byte reads of lanes (j >> 2) + 4q,
// q = 0..3. Pointing lane s of the group at K-row k + (s >> 2), columns
// m + 4 (s & 3) .. +3 therefore hands lane j the 4 consecutive K values
// (k .. k+3) of column m + j.
__device__ __forceinline__ short4v ds_read_tr(const char* p) {
  typedef __attribute__((address_space(3))) short4v* lds_s4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(const __attribute__((address_space(3))) char*)p);
}

// ---------------------------------------------------------------------------
// The tile core: acc[i][j] (wave block i of 16 A-rows, j of 16 B-rows)
// = sum over k < K of A[row][k] * B[row][k]; K a multiple of 64. With A_MN the
// A operand is MN-contiguous and its fragments are assembled with two
// transposed reads each.
//
// A slice is 2 steps of 32 K; a step is 64 MFMAs (8 x 8 blocks, i-major:
// A fragment i serves MFMAs 8 i .. 8 i + 7, B fragment j every eighth).
// Schedule, in 16-cycle MFMA slots:
//  * B fragments are double buffered: those of step s + 1 are read one every
//    4 MFMAs in the first half of step s. A fragments are single buffered:
//    fragment i of step s + 1 is read right after its last MFMA of step s,
//    57 MFMAs ahead of its first use (this frees 32 VGPRs);
//  * the loads of slice k + 2 go into the LDS slot slice k frees, spread
//    evenly over the first SPAN of the 128 slots after the barrier that frees
//    it: a burst of loads stalls the wave's issue, and with one wave per SIMD
//    nothing else feeds the matrix pipe meanwhile, while loads issued late may
//    not have landed by the next barrier (measured best: 96 for the forward's
//    chained walk, 64 for the backward's single tiles);
//  * that barrier, which also publishes slice k + 1, sits halfway through the
//    last step of slice k; the reads of slice k + 1's first step follow it.
// The loop body runs from that barrier to the next, so its back edge falls
// where every pending LDS read was issued long before. Every iteration runs
// the same code: where no slice k + 2 exists its loads go to the scratch row
// (and are awaited like the others by the next iteration), so there is no
// branch (and no merge of 256 accumulator registers) in the loop. The last
// iteration, outside the loop, issues loads only for a chained next tile.
//
// Chaining tiles (the forward's walk over vocabulary tiles): `pipe` holds the
// LDS slot of the tile's first slice and how many of its slices the previous
// tile already issued; with `chain` the loads run on into the next tile, whose
// operands have the same shapes as this tile's (ld, rows, K) and start at
// nA_base and nB_base, so it starts on data that landed during this tile's
// epilogue. Ends with a barrier unless chained, so LDS may be reused.
struct Pipe {
  int slot = 0;     // LDS slot (0 or 1) of the first slice
  int staged = 0;   // slices of this tile already issued (slice 0 then also published)
};

template <bool A_MN, int SPAN>
__device__ __forceinline__ void mma_tile(const Operand& A, const Operand& B, int K, char* lds,
                                         f32x4 (&acc)[kNB][kNB], Pipe& pipe, const uint16_t* nA_base,
                                         const uint16_t* nB_base, bool chain) {
  constexpr int NM = kNB * kNB;            // MFMAs per step
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const uint32_t base = lds_offset(lds);
  const uint32_t scratch_row = base + kRingBytes;
  const int nk = K / kBK;
  const int p0 = pipe.slot;
  // K-contiguous fragment reads: row (l % 16) of a 16-row block, chunk
  // 4 ks + l / 16 of the 8 per row
  const int rowsel = lane & 15;
  const int kq = lane >> 4;
  const int sw = swz(rowsel);
  const int a_off = (wm * 128 + rowsel) * kRowBytes;
  const int b_off = kOpBytes + (wn * 128 + rowsel) * kRowBytes;
  // transposed reads: lane s of group g points at K-row 8 g + s / 4 (+ 4 for
  // the upper half) and columns 4 (s % 4) .. +3 of the 16-column block
  const int t_row = 8 * kq + (rowsel >> 2);
  const int t_x = swz_mn(t_row);                        // same for the upper half
  const int t_chunk = wm * 16 + ((rowsel & 3) >> 1);    // + 2 i
  const int t_byte = 8 * (rowsel & 1);
  const LoadOffs la = load_offsets<A_MN>(A), lb = load_offsets<false>(B);
  const uint32_t wave_off = (uint32_t)wave_id() * 8192;   // this wave's 8 KB of an operand slice

  bf16x8 fa[kNB], fb[2][kNB];
  short8v ft[kNB];   // A_MN: the two transposed halves of each A fragment
  auto cur_of = [&](int slice) { return lds + ((p0 + slice) & 1) * kStageBytes; };
  auto rd_a = [&](int slice, int ks, int i, int h) {   // h: transposed half (A_MN) or -1 for both
    const char* cur = cur_of(slice);
    if (A_MN) {
      auto half = [&](int hh) {
        const char* p = cur + (ks * 32 + 4 * hh + t_row) * (kTile * 2) + (((t_chunk + 2 * i) ^ t_x) << 4) + t_byte;
        const short4v v = ds_read_tr(p);
        if (hh == 0) ft[i].s0123 = v; else ft[i].s4567 = v;
      };
      if (h <= 0) half(0);
      if (h != 0) half(1);
    } else {
      const int co = (((ks * 4) + kq) ^ sw) * 16;
      fa[i] = *reinterpret_cast<const bf16x8*>(cur + a_off + i * 16 * kRowBytes + co);
    }
  };
  auto rd_b = [&](int slice, int ks, int set, int j) {
    const int co = (((ks * 4) + kq) ^ sw) * 16;
    fb[set][j] = *reinterpret_cast<const bf16x8*>(cur_of(slice) + b_off + j * 16 * kRowBytes + co);
  };
  // MFMA q of a step; the tile's first step starts every block from zero (an
  // inline-constant accumulator operand, so the 256 AGPRs need no clearing)
  auto mf = [&](int set, int q, bool first = false) {
    const int i = q / kNB, j = q % kNB;
    const bf16x8 a = A_MN ? __builtin_bit_cast(bf16x8, ft[i]) : fa[i];
    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fb[set][j], first ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[i][j],
                                                      0, 0, 0);
  };
  // reads after MFMA q of a full step (step ks_next - 1 of `slice`): B of the
  // next step early, A fragment i right after its last use
  auto step_reads = [&](int slice, int ks_next, int q) {
    if (q < 4 * kNB && (q & 3) == 0) rd_b(slice, ks_next, ks_next & 1, q / 4);
    if ((q & 7) == 7) rd_a(slice, ks_next, q / 8, -1);
  };
  // reads after MFMA q (32..63) of the last step of a slice: slice + 1's first
  // step; A fragment i is free after MFMA 8 i + 7 (A_MN halves one slot apart,
  // both after MFMA 63 for the last)
  auto tail_reads = [&](int slice, int q) {
    if (q < 32 + 2 * kNB && (q & 1) == 0) rd_b(slice, 0, 0, (q - 32) / 2);
    if (q >= 48 && q < 62) {
      const int i = (q - 48) / 2;
      if (A_MN) rd_a(slice, 0, i, (q - 48) & 1);
      else if ((q & 1) == 0) rd_a(slice, 0, i, -1);
    }
    if (q == 63) rd_a(slice, 0, kNB - 1, -1);
  };

  // stream slice g of this tile (g >= nk: the next tile's slice g - nk)
  auto exists = [&](int g) { return g < nk || (chain && g - nk < nk); };
  auto load_slice = [&](int g) {
    const uint32_t st = __builtin_amdgcn_readfirstlane(base + ((p0 + g) & 1) * kStageBytes + wave_off);
    const bool own = g < nk;
    const int k0 = (own ? g : g - nk) * kBK;
    const void* ba = slice_base<A_MN>(A, own ? A.base : nA_base, k0, own);
    const void* bb = slice_base<false>(B, own ? B.base : nB_base, k0, own);
#pragma unroll
    for (int q = 0; q < 8; ++q) dma16(la.o[q], ba, st + q * 1024);
#pragma unroll
    for (int q = 0; q < 8; ++q) dma16(lb.o[q], bb, st + kOpBytes + q * 1024);
  };

  // prologue: slices 0 and 1 in flight, slice 0 published, its first reads
  if (pipe.staged == 0) load_slice(0);
  const bool pro1 = pipe.staged < 2 && exists(1);
  if (pro1) load_slice(1);
  if (pipe.staged == 0) {
    if (pro1) wait_vm<16>(); else wait_vm<0>();
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < kNB; ++j) rd_b(0, 0, 0, j);
#pragma unroll
  for (int i = 0; i < kNB; ++i) rd_a(0, 0, i, -1);

  // loads of stream slice k + 2 (into the slot of slice k, or the scratch row),
  // every address part but the per-lane offsets in SGPRs
  struct Issue {
    const void* ba;
    const void* bb;
    uint32_t sta, stb, step;   // LDS targets of load 0 and the step between loads
    bool scratch;
  };
  // The plan of iteration k is scalar work (~20 to 40 SALU instructions).
  // Issued in one piece it would stall the matrix pipe (one wave per SIMD
  // issues one instruction per 4 cycles, so only 3 fit beside each 16-cycle
  // MFMA); it is therefore computed in four pieces at four MFMA slots of the
  // previous iteration (plan_piece(n), n = 0..3), where no loads are issued.
  bool pl_own = false, pl_next = false;
  int pl_k0 = 0;
  auto plan_piece = [&](int k, int n, Issue& is) {
    if (n == 0) {
      const int g2 = k + 2;
      pl_own = g2 < nk;
      pl_next = !pl_own && chain && (g2 - nk) < nk;
      pl_k0 = pl_own ? g2 * kBK : (pl_next ? (g2 - nk) * kBK : 0);
    } else if (n == 1) {
      is.ba = slice_base<A_MN>(A, pl_next ? nA_base : A.base, pl_k0, !pl_next);
    } else if (n == 2) {
      is.bb = slice_base<false>(B, pl_next ? nB_base : B.base, pl_k0, !pl_next);
    } else {
      is.scratch = !(pl_own || pl_next);
      const uint32_t st = base + ((p0 + k) & 1) * kStageBytes + wave_off;
      is.sta = __builtin_amdgcn_readfirstlane(is.scratch ? scratch_row : st);
      is.stb = __builtin_amdgcn_readfirstlane(is.scratch ? scratch_row : st + kOpBytes);
      is.step = is.scratch ? 0u : 1024u;
    }
  };
  // MFMA slots (of the 32 in the first half of a step's second MFMA pass)
  // that carry the pieces
  auto plan_at = [&](int k, int q, Issue& is) {
    if (q >= 4 && q <= 16 && (q & 3) == 0) plan_piece(k, q / 4 - 1, is);
  };
  auto load = [&](const Issue& is, int d) {
    if (d < 8) dma16(la.o[d], is.ba, is.sta + d * is.step);
    else dma16(lb.o[d - 8], is.bb, is.stb + (d - 8) * is.step);
  };
  // the 16 loads over 16 <= `slots` <= 128 slots: load d follows slot d * slots / 16
  auto loads_at = [&](const Issue& is, int t, int slots) {
    const int d = (t * 16 + slots - 1) / slots;
    if (d < 16 && (d * slots) / 16 == t) load(is, d);
  };

  // head of slice 0: its first step and the first half of its second
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int q = 0; q < NM; ++q) {
    mf(0, q, true);
    step_reads(0, 1, q);
    __builtin_amdgcn_sched_barrier(0);
  }
  Issue is;   // the plan of the coming iteration
#pragma unroll
  for (int q = 0; q < NM / 2; ++q) {
    mf(1, q);
    plan_at(0, q, is);
    __builtin_amdgcn_sched_barrier(0);
  }
  // iteration k: publish slice k + 1, finish slice k, then the head of k + 1
  // (and the plan of iteration k + 1)
  auto iter = [&](int k, auto last_c) {
    constexpr bool last = decltype(last_c)::value;
    wait_vm<0>();          // slice k + 1 (this wave's part) has landed
    __syncthreads();       // ... everybody's; and every wave has issued its reads of slice k
#pragma unroll
    for (int t = 0; t < NM / 2; ++t) {
      mf(1, NM / 2 + t);
      if (!last) tail_reads(k + 1, NM / 2 + t);
      // the last iteration loads only for a chained next tile (that tile
      // awaits them): nothing may still be landing in LDS when the workgroup
      // ends (its LDS then belongs to the next workgroup on the CU)
      if (!last) loads_at(is, t, SPAN);
      else if (!is.scratch) loads_at(is, t, NM / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!last) {
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        mf(0, q);
        step_reads(k + 1, 1, q);
        loads_at(is, NM / 2 + q, SPAN);
        __builtin_amdgcn_sched_barrier(0);
      }
      Issue nxt;
#pragma unroll
      for (int q = 0; q < NM / 2; ++q) {
        mf(1, q);
        loads_at(is, NM / 2 + NM + q, SPAN);
        plan_at(k + 1, q, nxt);
        __builtin_amdgcn_sched_barrier(0);
      }
      is = nxt;
    }
  };
  for (int k = 0; k < nk - 1; ++k) iter(k, std::false_type{});
  iter(nk - 1, std::true_type{});
  __builtin_amdgcn_s_setprio(0);
  pipe.slot = (p0 + nk) & 1;
  pipe.staged = chain ? (nk >= 2 ? 2 : 1) : 0;
  if (!chain) __syncthreads();
  __builtin_amdgcn_sched_barrier(0);   // the epilogue's accumulator reads stay after the loop
}

// Row (within the wave's 128) held by register r of block i.
__device__ __forceinline__ int acc_row(int i, int r, int lane) { return i * 16 + 4 * (lane >> 4) + r; }

// Running statistics of one token over the vocabulary rows seen so far, in
// base-2 units: m2 = max z * log2(e), s1 = sum 2^(z log2e - m2),
// s2 = sum 2^(z log2e - m2) (z log2e - m2), zt = target logit (0 if unseen).
struct Stats {
  float m2, s1, s2, zt;
};

__device__ __forceinline__ Stats merge_stats(Stats a, Stats b) {
  const float m = nan_max(a.m2, b.m2);
  const float da = a.m2 - m;
  const float db = b.m2 - m;
  const float ea = fast_exp2(da);
  const float eb = fast_exp2(db);
  Stats o;
  o.m2 = m;
  o.s1 = ea * a.s1 + eb * b.s1;
  o.s2 = ea * (a.s2 + da * a.s1) + eb * (b.s2 + db * b.s1);
  o.zt = a.zt + b.zt;
  return o;
}

// ---------------------------------------------------------------------------
// Forward tile kernel. Workgroup (token tile tt, split s) walks vocabulary
// tiles s, s + S, s + 2S, ... for its 256 tokens (A = W rows = vocabulary,
// B = hidden rows = tokens) and writes one partial Stats per token and split.
// sc = log2(e) / T scores the tempered logits z / T in base 2; the target
// logit is kept untempered (the merge scales it). W holds the V vocabulary
// rows from global id voff on (a vocabulary shard; voff = 0 for the whole
// table): a target is picked here only when it falls inside that range.
// Lane l of wave (wm, wn) holds tokens wn * 128 + 16 j + l % 16 (j = 0..7)
// and, of each, 32 vocabulary rows of the wave's 128.
__global__ __launch_bounds__(kThreads) void fwd_stats_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ targets, int N, int H, int V, int voff, int S, int n_tt, int n_vt,
    float sc, float4* __restrict__ part, int64_t part_ld) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int vid = xcd_remap(blockIdx.x, gridDim.x);
  if (vid >= n_tt * S) return;
  const int tt = vid / S;
  const int s = vid - tt * S;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int tok0 = tt * kTile;

  int tgt[kNB];
  Stats st[kNB];
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const int tok = tok0 + wn * 128 + j * 16 + (lane & 15);
    const int t = tok < N ? targets[tok] : -1;
    tgt[j] = (t >= voff && t - voff < V) ? t - voff : -1;   // local row, or no hit
    st[j].m2 = kNegBig;
    st[j].s1 = 0.0f;
    st[j].s2 = 0.0f;
    st[j].zt = 0.0f;
  }

  const Operand ob{hidden + (int64_t)tok0 * H, H, min(kTile, N - tok0)};
  Pipe pipe;
  for (int vt = s; vt < n_vt; vt += S) {
    const int v0 = vt * kTile;
    const Operand oa{W + (int64_t)v0 * H, H, min(kTile, V - v0)};
    // one call site (a runtime chain flag): two inlined copies of the core
    // would merge 256 accumulator registers. Chained only into a tile of the
    // same shape (the next one is not the ragged last tile, or both are).
    const int v1 = v0 + S * kTile;
    const bool more = vt + S < n_vt && min(kTile, V - v1) == oa.rows;
    f32x4 acc[kNB][kNB];
    mma_tile<false, 96>(oa, ob, H, lds, acc, pipe, W + (int64_t)(more ? v1 : v0) * H, ob.base, more);

    const int vrow0 = v0 + wm * 128;
    // ragged last tile: rows past V take no part. Their logits are set to
    // kNegBig so they never win the max (unless the wave has no row left),
    // and their exponentials are zeroed outright: scaled by sc < 1 the
    // rounding error of kNegBig * sc alone would overflow exp2.
    const bool ragged = vrow0 + 128 > V;
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      float z[kNB][4];
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        pin_acc(acc[i][j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) z[i][r] = acc[i][j][r];
      }
      if (ragged) {
#pragma unroll
        for (int i = 0; i < kNB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) z[i][r] = (vrow0 + acc_row(i, r, lane) < V) ? z[i][r] : kNegBig;
      }
      // target logit: one-hot select, only in waves whose rows hold a target
      const int tr = tgt[j] - vrow0;
      const bool hit = (tr >= 0) && (tr < 128);
      if (__any(hit)) {
        float zt = st[j].zt;
#pragma unroll
        for (int i = 0; i < kNB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) zt = (acc_row(i, r, lane) == tr) ? z[i][r] : zt;
        st[j].zt = zt;
      }
      float mx = z[0][0];
#pragma unroll
      for (int i = 0; i < kNB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = nan_max(mx, z[i][r]);
      const float mnew = nan_max(st[j].m2, mx * sc);   // sc > 0: max commutes with the scaling
      const float dm = st[j].m2 - mnew;
      const float alpha = fast_exp2(dm);
      float s1 = alpha * st[j].s1;
      float s2 = alpha * (st[j].s2 + dm * st[j].s1);
      if (!ragged) {
#pragma unroll
        for (int i = 0; i < kNB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float d = fmaf(z[i][r], sc, -mnew);
            const float e = fast_exp2(d);
            s1 += e;
            s2 = fmaf(e, d, s2);
          }
      } else {
#pragma unroll
        for (int i = 0; i < kNB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool live = vrow0 + acc_row(i, r, lane) < V;
            const float d = live ? fmaf(z[i][r], sc, -mnew) : 0.0f;
            const float e = live ? fast_exp2(d) : 0.0f;
            s1 += e;
            s2 = fmaf(e, d, s2);
          }
      }
      st[j].m2 = mnew;
      st[j].s1 = s1;
      st[j].s2 = s2;
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // lanes l, l ^ 16, l ^ 32, l ^ 48 hold other rows of the same tokens:
  // merge in a fixed order (the lower lane group's record first)
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1) {
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      Stats o;
      o.m2 = __shfl_xor(st[j].m2, x);
      o.s1 = __shfl_xor(st[j].s1, x);
      o.s2 = __shfl_xor(st[j].s2, x);
      o.zt = __shfl_xor(st[j].zt, x);
      st[j] = (lane & x) == 0 ? merge_stats(st[j], o) : merge_stats(o, st[j]);
    }
  }
  // waves wm = 0 and wm = 1 hold the two vocabulary halves of the same tokens
  float4* xch = reinterpret_cast<float4*>(lds);
  if (wm == 1 && lane < 16) {
#pragma unroll
    for (int j = 0; j < kNB; ++j)
      xch[(wn * kNB + j) * 16 + lane] = make_float4(st[j].m2, st[j].s1, st[j].s2, st[j].zt);
  }
  __syncthreads();
  if (wm == 0 && lane < 16) {
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      const float4 q = xch[(wn * kNB + j) * 16 + lane];
      const Stats o{q.x, q.y, q.z, q.w};
      const Stats m = merge_stats(st[j], o);
      const int tok = tok0 + wn * 128 + j * 16 + lane;
      if (tok < N) part[(int64_t)s * part_ld + tok] = make_float4(m.m2, m.s1, m.s2, m.zt);
    }
  }
}

// Split merge: per token, the S partial records in order, by log-sum-exp
// (vocabulary splits of one launch, or vocabulary shards). invT = 1 / T
// tempers the target logit; Vtot bounds the valid target ids. With `rec`
// the merged record itself is written (a shard's partial) instead.
__global__ __launch_bounds__(256) void fwd_merge_kernel(
    const float4* __restrict__ part, int64_t part_ld, int S, const int32_t* __restrict__ targets,
    int N, int Vtot, float invT, float* __restrict__ logp, float* __restrict__ entropy,
    float* __restrict__ lse, float4* __restrict__ rec) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  float4 q = part[i];
  Stats a{q.x, q.y, q.z, q.w};
  for (int s = 1; s < S; ++s) {
    q = part[(int64_t)s * part_ld + i];
    a = merge_stats(a, Stats{q.x, q.y, q.z, q.w});
  }
  if (rec != nullptr) {
    rec[i] = make_float4(a.m2, a.s1, a.s2, a.zt);
    return;
  }
  const int t = targets[i];
  const bool valid = (t >= 0) && (t < Vtot);
  const float l2s = log2f(a.s1);
  // lse = m + ln(sum e^(z-m)); a +inf logit (and no NaN) leaves m = +inf and
  // s1 = NaN (inf - inf): the log-sum-exp is +inf
  const float l = a.m2 == INFINITY ? INFINITY : kLn2 * (a.m2 + l2s);
  const float h = kLn2 * (l2s - a.s2 / a.s1);        // lse - sum p z
  logp[i] = valid ? a.zt * invT - l : 0.0f;
  lse[i] = valid ? l : 0.0f;
  if (entropy != nullptr) entropy[i] = valid ? h : 0.0f;
}

// ---------------------------------------------------------------------------
// Backward. The token x vocabulary plane is cut into blocks; each block's
// cotangent is held as one bf16 buffer dz[token - t0][vocab - v0] and read
// by both gradient GEMMs (the dW GEMM as its MN-contiguous operand). Launch
// j of the backward carries the dh / dW tiles of block j - 1 (reading dz
// buffer (j - 1) % 2) and the cotangent tiles of block j (writing buffer
// j % 2): the short cotangent tiles fill the tail of the long GEMM tiles,
// and stream order makes every buffer's writes precede its reads.

// Cotangent tile: recompute a 256 x 256 logits tile of block
// [t0, t0 + Ct) x [v0, v0 + Vb) and write the untempered logits' cotangent
//   dz = (g_l (onehot - p) - g_e p (log p + entropy)) / T,
//   p = 2^(z sc - lse log2e),  sc = log2(e) / T,
// as bf16. Tokens past the block, masked tokens and vocabulary past the block
// are written as 0, so the gradient GEMMs can run over the padded block.
// Staging of one wave's 16 tokens x 128 vocabulary rows of dz in LDS: a
// token's 256 bytes plus 16 of padding, so that neither the 8-byte column
// writes nor the 16-byte row reads collide in a bank.
constexpr int kZStageRow = 256 + 16;
constexpr int kZStageBytes = 16 * kZStageRow;
static_assert(4 * kZStageBytes <= kRingBytes, "staging fits in the slice ring");

__device__ __forceinline__ void dz_tile(const BwdStep& s, int vid, char* lds) {
  int vt, tt;
  raster(vid, s.z_nvt, s.z_ntt, 4, vt, tt);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int t0 = s.z_t0, Ct = s.z_Ct, v0 = s.z_v0, Vb = s.z_Vb, H = s.H, Vtot = s.Vtot;
  const int tl0 = tt * kTile;   // token offset in the block
  const int vl0 = vt * kTile;   // vocabulary offset in the block

  // per-token inputs, loaded before the K loop so their latency hides behind
  // it; indices are clamped so every load is unconditional (a conditional load
  // per value costs a full memory round trip each)
  int t_in[kNB];
  float l_in[kNB], e_in[kNB], gl_in[kNB], ge_in[kNB];
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const int tl = tl0 + wn * 128 + j * 16 + (lane & 15);
    const int tok = t0 + min(tl, Ct - 1);
    t_in[j] = s.targets[tok];
    if (tl >= Ct) t_in[j] = -1;
    l_in[j] = s.lse[tok];
    e_in[j] = s.entropy != nullptr ? s.entropy[tok] : 0.0f;
    gl_in[j] = s.g_logp != nullptr ? s.g_logp[tok] : 0.0f;
    ge_in[j] = s.g_ent != nullptr ? s.g_ent[tok] : 0.0f;
  }

  const Operand oa{s.W + (int64_t)(v0 + vl0) * H, H, min(kTile, Vb - vl0)};
  const Operand ob{s.hidden + (int64_t)(t0 + tl0) * H, H, min(kTile, Ct - tl0)};
  f32x4 acc[kNB][kNB];
  Pipe pipe;
  mma_tile<false, 64>(oa, ob, H, lds, acc, pipe, oa.base, ob.base, false);
  // the ring is free once every wave is past its last fragment read: each
  // wave stages its bf16 columns there and stores whole row segments (in
  // register layout a store instruction would cover 16 rows x 32 bytes)
  __syncthreads();
  char* stage = lds + wave * kZStageBytes;

  const int vw0 = vl0 + wm * 128;   // block-local vocabulary row of this wave
  const bool ragged = (vw0 + 128 > Vb);
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const int t = t_in[j];
    const bool live = (t >= 0) && (t < Vtot);
    // masked tokens: every input is replaced (selected, never multiplied), so
    // whatever their rows hold cannot reach dz
    const float L = live ? l_in[j] : 0.0f;
    const float Hn = live ? e_in[j] : 0.0f;
    const float ga = live ? gl_in[j] : 0.0f;
    const float gb = live ? ge_in[j] : 0.0f;
    const float nlseL = -L * kLog2e;
    // dz = p * (c1 * d + c0) (+ g_l / T at the target), d = log2 p. The
    // entropy term enters only for a nonzero entropy cotangent (selected, so
    // a NaN entropy under g_ent = 0 stays out), and an entry of probability
    // 0 gets no probability term (the legacy product: 0 * -inf and 0 * NaN
    // give 0 there, a -inf logit or a row whose lse is +inf)
    const float c0 = -(ga + (gb != 0.0f ? gb * Hn : 0.0f)) * s.invT;
    const float c1 = -(gb * kLn2) * s.invT;
    const float gl = ga * s.invT;
    // target row relative to this wave's rows (a target of another shard or
    // block lands outside [0, 128) or on rows the ragged mask zeroes)
    const int tr = live ? (t - s.voff - v0 - vw0) : -1;
    const bool hit_any = __any(tr >= 0 && tr < 128);
    const bool any_dead = __any(!live);
    const int tl = tl0 + wn * 128 + j * 16;   // first of the 16 tokens
    // the three corrections apply to few columns (a target among the
    // wave's 128 rows for some of its 16 tokens: ~1% of columns at a large
    // vocabulary; masked tokens; the ragged last tile): they get a path of
    // their own, so the common one is three arithmetic operations and one
    // exp per element (4.4 VALU instructions with the bf16 packing and the
    // addresses; as selects on every element they took 13)
    auto column = [&](auto special_c) {
      constexpr bool special = decltype(special_c)::value;
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        pin_acc(acc[i][j]);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float d = fmaf(acc[i][j][r], s.sc, nlseL);
          const float p = fast_exp2(d);
          float x = lmh_fmul_legacy(p, fmaf(c1, d, c0));
          if (special) {
            x = (acc_row(i, r, lane) == tr) ? x + gl : x;
            x = live ? x : 0.0f;
            x = (vw0 + acc_row(i, r, lane) < Vb) ? x : 0.0f;
          }
          v[r] = x;
        }
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(stage + (lane & 15) * kZStageRow + 2 * acc_row(i, 0, lane)) = w;
      }
    };
    if (hit_any || any_dead || ragged) column(std::true_type{});
    else column(std::false_type{});
    // 4 tokens' 256-byte rows per store, 16 bytes a lane
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = 4 * q + (lane >> 4);
      const uint4 x = *reinterpret_cast<const uint4*>(stage + t * kZStageRow + 16 * (lane & 15));
      *reinterpret_cast<uint4*>(s.z_dz + (int64_t)(tl + t) * s.ld_dz + vw0 + 8 * (lane & 15)) = x;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Write one wave's 128 x 128 accumulator block of a gradient tile: element
// (row, col) of out, row = r_base + acc_row(i, r, lane), col = c_base + 16 j
// + lane % 16; rows at or past `rows` and columns at or past `cols` are
// skipped. With `add` the block is added to what out holds. With `targets`,
// row m belongs to token t_base + m and masked tokens' rows are stored as 0,
// or left unchanged when adding. The read-modify-write is batched per 16-row
// block: its loads (and target ids) are all in flight before the first add;
// one load-add-store per element would wait out the whole memory latency for
// each.
__device__ __forceinline__ void write_acc(float* __restrict__ out, int64_t ld, int r_base, int rows,
                                          int c_base, int cols, bool add, const int32_t* __restrict__ targets,
                                          int t_base, int Vtot, f32x4 (&acc)[kNB][kNB]) {
  const int lane = threadIdx.x & 63;
  bool col_ok[kNB];
  int col[kNB];   // clamped into range, so every load below is unconditional
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const int c = c_base + j * 16 + (lane & 15);
    col_ok[j] = c < cols;
    col[j] = col_ok[j] ? c : cols - 1;
  }
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    float old[4][kNB];
    bool row_ok[4], live[4];
    int row[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = r_base + acc_row(i, r, lane);
      row_ok[r] = m < rows;
      row[r] = row_ok[r] ? m : rows - 1;
      live[r] = true;
    }
    if (targets != nullptr) {
      int t[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = targets[t_base + row[r]];
#pragma unroll
      for (int r = 0; r < 4; ++r) live[r] = (t[r] >= 0) && (t[r] < Vtot);
    }
    if (add) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < kNB; ++j) old[r][j] = out[(int64_t)row[r] * ld + col[j]];
    }
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      pin_acc(acc[i][j]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!(row_ok[r] && col_ok[j])) continue;
        float* p = out + (int64_t)row[r] * ld + col[j];
        if (add) {
          if (live[r]) *p = old[r][j] + acc[i][j][r];
        } else {
          *p = live[r] ? acc[i][j][r] : 0.0f;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The bf16-gradient backward's writers: the same tile layouts as write_acc
// (dW, row-major) and write_acc_t (dh, transposed), reading the values to add
// to from o.src (nothing, a float32 accumulator or a bf16 gradient, widened)
// and writing the sum to o.dst (a float32 accumulator, or a bf16 gradient,
// rounded to nearest even once). Both descriptors point at row 0 of the
// block; rows have stride ld.
__device__ __forceinline__ float widen_bf16(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t round_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ void write_acc_g(const GradOut& o, int64_t ld, int r_base, int rows, int c_base,
                                            int cols, f32x4 (&acc)[kNB][kNB]) {
  const int lane = threadIdx.x & 63;
  const float* sf = static_cast<const float*>(o.src);
  const uint16_t* sb = static_cast<const uint16_t*>(o.src);
  float* df = static_cast<float*>(o.dst);
  uint16_t* db = static_cast<uint16_t*>(o.dst);
  bool col_ok[kNB];
  int col[kNB];
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const int c = c_base + j * 16 + (lane & 15);
    col_ok[j] = c < cols;
    col[j] = col_ok[j] ? c : cols - 1;
  }
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    float old[4][kNB];
    bool row_ok[4];
    int row[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = r_base + acc_row(i, r, lane);
      row_ok[r] = m < rows;
      row[r] = row_ok[r] ? m : rows - 1;
    }
    if (o.src_kind == kSrcF32) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < kNB; ++j) old[r][j] = sf[(int64_t)row[r] * ld + col[j]];
    } else if (o.src_kind == kSrcBf16) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < kNB; ++j) old[r][j] = widen_bf16(sb[(int64_t)row[r] * ld + col[j]]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < kNB; ++j) old[r][j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      pin_acc(acc[i][j]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!(row_ok[r] && col_ok[j])) continue;
        const float v = old[r][j] + acc[i][j][r];
        const int64_t at = (int64_t)row[r] * ld + col[j];
        if (o.dst_bf16) db[at] = round_bf16(v);
        else df[at] = v;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ void write_acc_tg(const GradOut& o, int64_t ld, int r_base, int rows, int c_base,
                                             int cols, bool dead_zero, const int32_t* __restrict__ targets,
                                             int t_base, int Vtot, f32x4 (&acc)[kNB][kNB]) {
  const int lane = threadIdx.x & 63;
  int col[kNB], tgt[kNB];
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const int c = c_base + j * 16 + (lane & 15);
    col[j] = c < cols ? c : cols - 1;
    tgt[j] = targets[t_base + col[j]];
    if (c >= cols) tgt[j] = -2;   // not stored
  }
  const int r0 = (r_base < rows ? r_base : 0) + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const bool in = tgt[j] != -2;
    const bool live = (tgt[j] >= 0) && (tgt[j] < Vtot);
    const int64_t base = (int64_t)col[j] * ld + r0;
    f32x4 old[kNB];
    if (o.src_kind == kSrcF32) {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(o.src) + base);
#pragma unroll
      for (int i = 0; i < kNB; ++i) old[i] = p[r_base + 16 * i < rows ? 4 * i : 0];
    } else if (o.src_kind == kSrcBf16) {
      const uint2* p = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(o.src) + base);
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        const uint2 w = p[r_base + 16 * i < rows ? 4 * i : 0];
        old[i] = f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
      }
    } else {
#pragma unroll
      for (int i = 0; i < kNB; ++i) old[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      pin_acc(acc[i][j]);
      if (!(r_base + 16 * i < rows) || !in) continue;
      if (!live && !dead_zero) continue;
      const f32x4 v = live ? old[i] + acc[i][j] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (o.dst_bf16) {
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        reinterpret_cast<uint2*>(static_cast<uint16_t*>(o.dst) + base)[4 * i] = w;
      } else {
        reinterpret_cast<f32x4*>(static_cast<float*>(o.dst) + base)[4 * i] = v;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// dW tile: dW[v0 + m][n] (+)= sum_k dz[k][m] ht[n][t0 + k] over the block's
// tokens (A = dz read MN-contiguous, B = hidden^T with masked tokens zeroed).
// BF16: the bf16-gradient backward's writer (s.o_dW).
template <bool BF16>
__device__ __forceinline__ void dw_tile(const BwdStep& s, int vid, char* lds) {
  int mt, hb;
  raster(vid, s.n_dw / s.n_ht, s.n_ht, 4, mt, hb);
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int m0 = mt * kTile;
  const int h0 = hb * kTile;
  const int H = s.H;
  const Operand oa{s.g_dz + m0, s.ld_dz, kTile};
  const Operand ob{s.ht + (int64_t)h0 * s.ld_ht + s.g_t0, s.ld_ht, kTile};
  f32x4 acc[kNB][kNB];
  Pipe pipe;
  mma_tile<true, 64>(oa, ob, (s.g_Ct + kBK - 1) / kBK * kBK, lds, acc, pipe, oa.base, ob.base, false);
  if constexpr (BF16) {
    write_acc_g(s.o_dW, H, m0 + wm * 128, s.g_Vb, h0 + wn * 128, H, acc);
  } else {
    write_acc(s.dW + (int64_t)s.g_v0 * H, H, m0 + wm * 128, s.g_Vb, h0 + wn * 128, H, s.g_acc_dW != 0,
              nullptr, 0, 0, acc);
  }
}

// Write one wave's 128 x 128 accumulator block transposed: element (row,
// col) goes to out[col][row], row = r_base + acc_row(i, r, lane) (the 4
// registers of a block are 4 consecutive rows: one 16-byte access), col =
// c_base + 16 j + lane % 16. Rows at or past `rows` (a multiple of 16) and
// columns at or past `cols` are skipped. With `add` the block is added to
// what out holds. Column c belongs to token t_base + c: masked tokens'
// columns are stored as 0, or left unchanged when adding. Batched per
// column: one 64-bit address, 8 accesses at fixed offsets from it.
__device__ __forceinline__ void write_acc_t(float* __restrict__ out, int64_t ld, int r_base, int rows,
                                            int c_base, int cols, bool add, const int32_t* __restrict__ targets,
                                            int t_base, int Vtot, f32x4 (&acc)[kNB][kNB]) {
  const int lane = threadIdx.x & 63;
  int col[kNB], tgt[kNB];
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const int c = c_base + j * 16 + (lane & 15);
    col[j] = c < cols ? c : cols - 1;   // clamped, so the loads below are unconditional
    tgt[j] = targets[t_base + col[j]];
    if (c >= cols) tgt[j] = -2;         // not stored
  }
  // a wave with no row in range points its (unused) loads at row 0; the
  // loads of blocks past `rows` reread block 0 (a select, not a branch: a
  // branch per load makes the compiler copy the accumulators out)
  const int r0 = (r_base < rows ? r_base : 0) + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const bool in = tgt[j] != -2;
    const bool live = (tgt[j] >= 0) && (tgt[j] < Vtot);
    f32x4* p = reinterpret_cast<f32x4*>(out + (int64_t)col[j] * ld + r0);
    f32x4 old[kNB];
    if (add) {
#pragma unroll
      for (int i = 0; i < kNB; ++i) old[i] = p[r_base + 16 * i < rows ? 4 * i : 0];
    }
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      pin_acc(acc[i][j]);
      if (!(r_base + 16 * i < rows) || !in) continue;
      if (add) {
        if (live) p[4 * i] = old[i] + acc[i][j];
      } else {
        p[4 * i] = live ? acc[i][j] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// dh tile, computed transposed: dh[t0 + m][n] (+)= sum_k W[v0 + k][n] dz[m][k]
// over the block's vocabulary (A = W as it lies, MN-contiguous, B = the
// cotangent rows); masked token rows are written as 0 (left alone when
// adding). W's rows past V in the block's last slice are read from the
// zero-padded copy of its last rows. BF16: the bf16-gradient backward's
// writer (s.o_dh).
template <bool BF16>
__device__ __forceinline__ void dh_tile(const BwdStep& s, int vid, char* lds) {
  int mt, hb;
  raster(vid, s.n_dh / s.n_ht, s.n_ht, 4, mt, hb);
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int m0 = mt * kTile;
  const int h0 = hb * kTile;
  const int H = s.H;
  const int tail_k = s.W_tail != nullptr ? s.v_tail - s.g_v0 : -1;
  const Operand oa{s.W + (int64_t)s.g_v0 * H + h0, H, min(kTile, H - h0),
                   s.W_tail != nullptr ? s.W_tail + h0 : nullptr, tail_k};
  const Operand ob{s.g_dz + (int64_t)m0 * s.ld_dz, s.ld_dz, kTile};
  f32x4 acc[kNB][kNB];
  Pipe pipe;
  mma_tile<true, 64>(oa, ob, (s.g_Vb + kBK - 1) / kBK * kBK, lds, acc, pipe, oa.base, ob.base, false);
  if constexpr (BF16) {
    write_acc_tg(s.o_dh, H, h0 + wm * 128, H, m0 + wn * 128, s.g_Ct, s.dh_dead_zero != 0, s.targets, s.g_t0,
                 s.Vtot, acc);
  } else {
    write_acc_t(s.dh + (int64_t)s.g_t0 * H, H, h0 + wm * 128, H, m0 + wn * 128, s.g_Ct, s.g_acc_dh != 0,
                s.targets, s.g_t0, s.Vtot, acc);
  }
}

// One backward launch: each XCD (workgroups are dealt to the 8 XCDs
// round-robin) takes an equal share of the gradient tiles: its eighth of the
// dW tiles and of the dh tiles (the kind with the longer K first), so the
// long tiles start first everywhere. (Cutting the concatenated gradient-tile
// list into eight ranges instead piles all dh tiles onto the last XCDs, which
// doubles their share of the work when the two kinds' K differ.) The
// cotangent tiles follow and fill the tail. Each cotangent workgroup takes
// one tile off an atomic counter: from its XCD's own eighth first
// (neighbouring tiles share operand panels in its L2), and once that is used
// up from the other XCDs' eighths, so an XCD that runs ahead takes work from
// one that lags instead of idling (the XCDs' speeds differ by a few percent).
// Each XCD gets kStealSlots workgroups beyond its own eighth for that; a
// workgroup that finds every counter used up exits. Which workgroup computes
// a tile does not change its result.
constexpr int kStealSlots = 32;   // one round of the XCD's 32 CUs

__device__ __forceinline__ int z_share_lo(int x, int n_z) { return x * n_z / 8; }

template <bool BF16>
__device__ __forceinline__ void bwd_step(const BwdStep& s, char* lds, int& z_tile) {
  const int xcd = blockIdx.x & 7;
  const int loc = blockIdx.x >> 3;
  const int n_z = s.z_ntt * s.z_nvt;
  const int dw_lo = xcd * s.n_dw / 8;
  const int dw_cnt = (xcd + 1) * s.n_dw / 8 - dw_lo;
  const int dh_lo = xcd * s.n_dh / 8;
  const int dh_cnt = (xcd + 1) * s.n_dh / 8 - dh_lo;
  const bool dh_first = s.g_Vb > s.g_Ct;   // dh tiles run K = Vb, dW tiles K = Ct
  const int first_cnt = dh_first ? dh_cnt : dw_cnt;
  const int g_cnt = dw_cnt + dh_cnt;
  if (loc < g_cnt) {
    const bool is_dh = (loc < first_cnt) == dh_first;
    if (is_dh) {
      dh_tile<BF16>(s, dh_lo + (dh_first ? loc : loc - dw_cnt), lds);
    } else {
      dw_tile<BF16>(s, dw_lo + (dh_first ? loc - dh_cnt : loc), lds);
    }
    return;
  }
  if (n_z == 0) return;
  if (threadIdx.x == 0) {
    int t = -1;
    for (int p = 0; p < 8 && t < 0; ++p) {
      const int x = (xcd + p) & 7;
      const int lo = z_share_lo(x, n_z);
      const int cnt = z_share_lo(x + 1, n_z) - lo;
      if (cnt == 0) continue;
      const int i = __hip_atomic_fetch_add(s.z_ctr + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (i < cnt) t = lo + i;
    }
    z_tile = t;
  }
  __syncthreads();
  const int tile = z_tile;
  if (tile >= 0) dz_tile(s, tile, lds);
}

__global__ __launch_bounds__(kThreads) void bwd_step_kernel(const BwdStep s) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  __shared__ int z_tile;
  bwd_step<false>(s, lds, z_tile);
}

// The same launch writing bf16 gradients through float32 accumulators.
__global__ __launch_bounds__(kThreads) void bwd_step_bf16_kernel(const BwdStep s) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  __shared__ int z_tile;
  bwd_step<true>(s, lds, z_tile);
}

// Transposed bf16 copy: out[c][r] = in[r][c] for r < R and c < C, 0 for the
// padding r in [R, R_pad) and c in [C, C_pad); with `tgt`, rows whose target
// id lies outside [0, V) are 0 too (masked tokens never reach the dW GEMM,
// whatever their hidden row holds: the select happens here, once).
// Grid: (R_pad / 64, C_pad / 64), 256 threads; 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, int R, int C, const int32_t* __restrict__ tgt,
    int V, uint16_t* __restrict__ out, int64_t ld_out) {
  __shared__ uint32_t t[64][33];   // 64 rows x 64 bf16 (as 32 words) + 1 word pad
  const int r0 = blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  {
    const int rl = tid >> 2;          // 0..63
    const int cq = (tid & 3) * 16;    // 16 columns each
    const int r = r0 + rl;
    bool ok = (r < R) && (c0 + cq < C);
    if (ok && tgt != nullptr) {
      const int tv = tgt[r];
      ok = (tv >= 0) && (tv < V);
    }
    uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = make_uint4(0u, 0u, 0u, 0u);
    if (ok) {
      const uint4* src = reinterpret_cast<const uint4*>(in + (int64_t)r * ld_in + c0 + cq);
      v0 = src[0];
      v1 = src[1];
    }
    uint32_t* d = &t[rl][cq >> 1];
    d[0] = v0.x; d[1] = v0.y; d[2] = v0.z; d[3] = v0.w;
    d[4] = v1.x; d[5] = v1.y; d[6] = v1.z; d[7] = v1.w;
  }
  __syncthreads();
  {
    const int cl = tid >> 2;          // output row (input column) 0..63
    const int rq = (tid & 3) * 16;    // 16 input rows each
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = t[rq + 2 * e][cl >> 1];
      const uint32_t b = t[rq + 2 * e + 1][cl >> 1];
      const uint32_t lo = (cl & 1) ? (a >> 16) : (a & 0xFFFFu);
      const uint32_t hi = (cl & 1) ? (b >> 16) : (b & 0xFFFFu);
      w[e] = lo | (hi << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(out + (int64_t)(c0 + cl) * ld_out + r0 + rq);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// Row copy with zero padding: out[r][c] = in[r][c] for r < R, 0 for
// R <= r < R_pad (c < C, C % 8 == 0; both of row stride C). One 16-byte
// chunk per thread.
__global__ __launch_bounds__(256) void pad_rows_kernel(const uint16_t* __restrict__ in, int R, int C,
                                                       int R_pad, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = C / 8;
  if (i >= (int64_t)R_pad * cpr) return;
  const int r = (int)(i / cpr);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (r < R) v = reinterpret_cast<const uint4*>(in)[i];
  reinterpret_cast<uint4*>(out)[i] = v;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t k = i; k < n; k += stride) p[k] = 0.0f;
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after argument checks).

static inline unsigned round8(long long x) { return (unsigned)((x + 7) / 8 * 8); }

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const long long wg = (long long)a.n_tt * a.S;
  const double N = (double)a.N, H = (double)a.H, V = (double)a.V;
  trace_begin(stream);
  hipLaunchKernelGGL(fwd_stats_kernel, dim3(round8(wg)), dim3(kThreads), 0, stream, a.hidden, a.W,
                     a.targets, (int)a.N, (int)a.H, (int)a.V, (int)a.voff, a.S, a.n_tt, a.n_vt, a.sc,
                     reinterpret_cast<float4*>(a.part), a.part_ld);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_end(kFwdStats, stream, 2.0 * N * H * V, 2.0 * (N + V) * H + 4.0 * N + 16.0 * a.S * N);
  trace_begin(stream);
  hipLaunchKernelGGL(fwd_merge_kernel, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(a.part), a.part_ld, a.S, a.targets, (int)a.N,
                     (int)a.Vtot, a.invT, a.logp, a.entropy, a.lse, reinterpret_cast<float4*>(a.rec));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_end(kFwdMerge, stream, 0.0, 16.0 * a.S * N + 16.0 * N);
  return hipSuccess;
}

hipError_t launch_merge(const float* partials, int P, int64_t N, const int32_t* targets, int64_t Vtot,
                        float invT, float* logp, float* entropy, float* lse, hipStream_t stream) {
  trace_begin(stream);
  hipLaunchKernelGGL(fwd_merge_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(partials), N, P, targets, (int)N, (int)Vtot, invT,
                     logp, entropy, lse, nullptr);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_end(kFwdMerge, stream, 0.0, 16.0 * P * (double)N + 16.0 * (double)N);
  return hipSuccess;
}

template <bool BF16>
static hipError_t launch_bwd(const BwdStep& st, hipStream_t stream) {
  const int n_z = st.z_ntt * st.z_nvt;
  int per = 0;
  for (int x = 0; x < 8; ++x)
    per = max(per, ((x + 1) * st.n_dw / 8 - x * st.n_dw / 8) + ((x + 1) * st.n_dh / 8 - x * st.n_dh / 8) +
                       ((x + 1) * n_z / 8 - x * n_z / 8) + (n_z > 0 ? kStealSlots : 0));
  if (per == 0) return hipSuccess;
  const int n_g = st.n_dw + st.n_dh;
  const double H = (double)st.H;
  const double gc = (double)st.g_Ct, gv = (double)st.g_Vb;
  const double zc = (double)st.z_Ct, zv = (double)st.z_Vb;
  trace_begin(stream);
  if (BF16) hipLaunchKernelGGL(bwd_step_bf16_kernel, dim3(8 * per), dim3(kThreads), 0, stream, st);
  else hipLaunchKernelGGL(bwd_step_kernel, dim3(8 * per), dim3(kThreads), 0, stream, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // algorithmic (credited) work: 2 Ct Vb H for each of the dh and dW GEMMs;
  // the recomputed logits (2 Ct' Vb' H more) are executed but not counted.
  // Bytes: the dz block written once and read once, operand panels, f32 outputs
  const double fl = n_g ? 4.0 * gc * gv * H : 0.0;
  const double by = (n_g ? 2.0 * gc * gv + 2.0 * (gc + gv) * H +
                               4.0 * H * (gc * (1 + st.g_acc_dh) + gv * (1 + st.g_acc_dW)) : 0.0) +
                    (n_z ? 2.0 * zc * zv + 2.0 * (zc + zv) * H + 20.0 * zc : 0.0);
  trace_end(BF16 ? kBwdStepBf16 : kBwdStep, stream, fl, by);
  return hipSuccess;
}

hipError_t launch_bwd_step(const BwdStep& st, hipStream_t stream) { return launch_bwd<false>(st, stream); }
hipError_t launch_bwd_step_bf16(const BwdStep& st, hipStream_t stream) { return launch_bwd<true>(st, stream); }

hipError_t launch_transpose(const uint16_t* in, int64_t ld_in, int64_t R, int64_t C, int64_t R_pad,
                            int64_t C_pad, const int32_t* tgt, int64_t V, uint16_t* out,
                            int64_t ld_out, hipStream_t stream) {
  trace_begin(stream);
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)(R_pad / 64), (unsigned)(C_pad / 64)), dim3(256),
                     0, stream, in, ld_in, (int)R, (int)C, tgt, (int)V, out, ld_out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_end(kTranspose, stream, 0.0, 2.0 * (double)R * C + 2.0 * (double)R_pad * C_pad);
  return hipSuccess;
}

hipError_t launch_pad_rows(const uint16_t* in, int64_t R, int64_t C, int64_t R_pad, uint16_t* out,
                           hipStream_t stream) {
  const long long n = R_pad * (C / 8);
  if (n <= 0) return hipSuccess;
  trace_begin(stream);
  hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, in, (int)R,
                     (int)C, (int)R_pad, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_end(kPadRows, stream, 0.0, 2.0 * (double)R * C + 2.0 * (double)R_pad * C);
  return hipSuccess;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  trace_begin(stream);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_end(kFill, stream, 0.0, 4.0 * (double)n);
  return hipSuccess;
}

}  // namespace lmh
