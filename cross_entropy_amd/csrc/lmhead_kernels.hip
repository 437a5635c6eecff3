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
// 512-thread workgroup (8 wave64s as 2 x 4, each owning 128 x 64),
// v_mfma_f32_32x32x16_bf16, with both operands K-contiguous. K is staged
// through two 64-wide LDS slices filled by direct-to-LDS loads
// (global_load_lds_dwordx4): the next slice lands while the current one is
// consumed and no VGPRs hold staged data. Slice rows are 128 bytes with a
// 16-byte-chunk XOR swizzle, which keeps the MFMA fragment reads free of
// bank conflicts. The MFMA block of each slice runs at raised wave priority
// so the two waves sharing a SIMD keep its matrix pipe fed. Operands that are stored MN-contiguous (W and hidden in
// the backward) are given to the core through transposed copies.
//
// MFMA 32x32x16 register layout used throughout (wave64): lane l supplies
// row (l % 32) of A and column (l % 32) of B with the 8 K values
// 8*(l/32) .. 8*(l/32)+7; result register r of lane l holds
// D[8*(r/4) + 4*(l/32) + (r%4)][l % 32].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lmhead_internal.h"

namespace lmh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kTile = 256;                       // output tile edge
constexpr int kBK = 64;                          // K per LDS slice
constexpr int kStages = 2;                       // slices in the ring
constexpr int kRowBytes = kBK * 2;               // 128 B per staged row
constexpr int kRowsPerDma = 1024 / kRowBytes;    // rows one wave-wide DMA fills
constexpr int kOpBytes = kTile * kRowBytes;      // 16 KB per operand slice
constexpr int kStageBytes = 2 * kOpBytes;        // A + B
constexpr int kLdsBytes = kStages * kStageBytes; // 128 KB of the 160 KB per CU

constexpr int kTPitch = kTile * 2 + 16;          // staged transposed cotangent row (bytes)
constexpr int kDzLdsBytes = kTile * kTPitch > kLdsBytes ? kTile * kTPitch : kLdsBytes;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegBig = -1.0e30f;              // "minus infinity" that keeps 0 * x finite

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// NaN-propagating max (v_maximum3_f32 on gfx950): a NaN logit must reach the
// statistics, where fmaxf would drop it.
__device__ __forceinline__ float nan_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);   // round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFFu);
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

// ---------------------------------------------------------------------------
// Staging. A K-contiguous operand: element (row, k) at base[row * ld + k];
// rows at or past `rows` read row rows-1 instead (their results are
// discarded or masked by the epilogues), so every load stays in bounds.
struct Operand {
  const uint16_t* base;
  int64_t ld;
  int rows;
};

// XOR applied to the 16-byte chunk index of staged row r (8 chunks per row):
// any 16 consecutive rows read at one logical chunk hit 16 distinct 16-byte
// bank groups of the 256-byte bank line.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One direct-to-LDS load: 64 lanes x 16 B land at m0 + 16 * lane; lane l
// reads 16 bytes at sbase + voff(l) (scalar base, 32-bit per-lane offset,
// so a wave's loads cost one VGPR each). Issued as inline asm so the
// compiler does not add a vmcnt(0) in front of every LDS read of the ring;
// completion is awaited explicitly (wait_vm) before the barrier that
// publishes a slice.
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

// Stage rows [0, 256) x K [k0, k0 + 64) of one operand. Each wave loads 32
// rows as 4 x 8 rows of 8 chunks; lane l fills physical chunk l % 8 of row
// l / 8 with the logical chunk that the swizzle puts there. Byte offsets
// from op.base stay below 2^32: a tile spans 256 rows.
__device__ __forceinline__ void stage(const Operand& op, int k0, uint32_t lds_op) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const char* b = reinterpret_cast<const char*>(op.base) + 2 * (int64_t)k0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = wave * 32 + q * kRowsPerDma;
    const int r = r0 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    const int rr = min(r, op.rows - 1);
    const uint32_t off = (uint32_t)((int64_t)rr * op.ld * 2) + (uint32_t)(c * 16);
    dma16(off, b, __builtin_amdgcn_readfirstlane(lds_op + r0 * kRowBytes));
  }
}

// Stage K-rows [k0, k0 + 64) x M [0, 256) of an MN-contiguous operand:
// element (m, k) at base[k * ld + m]. The slice holds 64 rows of 256 m
// (512 B each); 16-byte chunks are XOR-swizzled by 4 * (k % 4) so the
// transposed fragment reads below hit distinct bank groups. Each wave-wide
// DMA fills two rows.
__device__ __forceinline__ void stage_mn(const Operand& op, int k0, uint32_t lds_op) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const char* b = reinterpret_cast<const char*>(op.base + (int64_t)k0 * op.ld);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = wave * 8 + q * 2;
    const int r = r0 + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (r & 3));
    const uint32_t off = (uint32_t)((int64_t)r * op.ld * 2) + (uint32_t)(c * 16);
    dma16(off, b, __builtin_amdgcn_readfirstlane(lds_op + r0 * (kTile * 2)));
  }
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v* lds_s4;

// LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane j
// receives element (j & 3) of the 8-byte reads of lanes (j >> 2) + 4q,
// q = 0..3. Pointing lane s of the group at row k + (s >> 2), columns
// m + 4 (s & 3) .. +3 therefore hands lane j the 4 consecutive K values
// (k .. k+3) of column m + j.
__device__ __forceinline__ short4v ds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s4)(const __attribute__((address_space(3))) char*)p);
}

// Scheduling pins. NM MFMAs of one 16-deep step with the NR LDS reads of the
// next step spread between them, front-loaded: after MFMA q come
// ceil((q+1) NR / NM) - ceil(q NR / NM) reads. The compiler's own order
// issues the reads late and waits on them at once, which exposes the LDS
// latency to the matrix pipe several times per slice.
template <int NM, int NR, int Q>
struct Pin {
  static __device__ __forceinline__ void run() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    constexpr int n = ((Q + 1) * NR + NM - 1) / NM - (Q * NR + NM - 1) / NM;
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);   // n LDS reads
    Pin<NM, NR, Q + 1>::run();
  }
};
template <int NM, int NR>
struct Pin<NM, NR, NM> {
  static __device__ __forceinline__ void run() {}
};

// The tile core: acc[i][j] (wave sub-block i of 32 A-rows, j of 32 B-rows)
// = sum over k < K of A[row][k] * B[row][k]. K is a multiple of 64. With
// A_MN the A operand is MN-contiguous (see stage_mn) and its fragments are
// assembled with transposed LDS reads. Ends with a barrier, so LDS may be
// reused as soon as it returns.
//
// Schedule of one 64-deep slice k (4 steps of 16): the fragments of step
// s + 1 are read into the other register set between the 8 MFMAs of step s
// (pinned, in the order the MFMAs consume them); the loads of slice k + 1
// are issued at the start of steps 0 (A) and 1 (B); the barrier that
// publishes slice k + 1 sits halfway through the MFMAs of the last step, and
// the first fragments of slice k + 1 are read right after it, between the
// remaining MFMAs, so the matrix pipe never restarts from an empty register
// set. The last slice is peeled off so the steady-state body has no branch.
//
// Chaining tiles (the forward's walk over vocabulary tiles): `pipe` holds the
// LDS slot of the tile's first slice and whether that slice was already
// issued; with `next` the last slice issues the first slice of the next tile
// (same operand shapes) into the free slot, so the next tile starts on data
// that landed during this tile's epilogue.
struct Pipe {
  int slot = 0;         // LDS slot (0 or 1) of the first slice
  bool staged = false;  // its loads were issued by the previous tile
};

template <bool A_MN>
__device__ __forceinline__ void mma_tile(const Operand& A, const Operand& B, int K, char* lds,
                                         f32x16 (&acc)[4][2], Pipe& pipe,
                                         const Operand* nextA = nullptr, const Operand* nextB = nullptr) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const uint32_t base = lds_offset(lds);
  const int nk = K / kBK;
  const int sw = swz(lane & 31);
  const int a_off = (wm * 128 + (lane & 31)) * kRowBytes;
  const int b_off = kOpBytes + (wn * 64 + (lane & 31)) * kRowBytes;
  // transposed A reads: lane group gq = lane / 16 covers columns
  // 16 * (gq & 1) .. +15 of a 32-column sub-block and K rows 8 * (gq >> 1) ..
  const int gq = lane >> 4;
  const int sl = lane & 15;
  const int t_row = 8 * (gq >> 1) + (sl >> 2);             // + 16 ks (+ 4 for the upper half)
  const int t_chunk = wm * 16 + 2 * (gq & 1) + ((sl & 3) >> 1);   // + 4 i, before the swizzle
  const int t_byte = 8 * (sl & 1);

  bf16x8 fa[2][4], fb[2][2];
  auto read_a = [&](const char* cur, int ks, int co, int buf, int i) {
    if (A_MN) {
      const int row = ks * 16 + t_row;          // row & 3 == (row + 4) & 3
      const int x = row & 3;
      const char* p = cur + row * (kTile * 2) + ((t_chunk | ((i ^ x) << 2)) << 4) + t_byte;
      const short4v lo = ds_read_tr(p);
      const short4v hi = ds_read_tr(p + 4 * (kTile * 2));
      const short4v v8[2] = {lo, hi};
      fa[buf][i] = __builtin_bit_cast(bf16x8, v8);
    } else {
      fa[buf][i] = *reinterpret_cast<const bf16x8*>(cur + a_off + i * 32 * kRowBytes + co);
    }
  };
  auto read_b = [&](const char* cur, int co, int buf, int j) {
    fb[buf][j] = *reinterpret_cast<const bf16x8*>(cur + b_off + j * 32 * kRowBytes + co);
  };
  // in the order the MFMAs (i-major) consume them
  const int p0 = pipe.slot;
  auto read_frags = [&](int slice, int ks, int buf) {
    const char* cur = lds + ((p0 + slice) & 1) * kStageBytes;
    const int co = (((ks * 2) + (lane >> 5)) ^ sw) * 16;
    read_a(cur, ks, co, buf, 0);
    read_b(cur, co, buf, 0);
    read_b(cur, co, buf, 1);
#pragma unroll
    for (int i = 1; i < 4; ++i) read_a(cur, ks, co, buf, i);
  };
  auto mfma = [&](int buf, int lo, int hi) {
#pragma unroll
    for (int q = lo; q < hi; ++q) {
      const int i = q >> 1, j = q & 1;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
    }
  };
  constexpr int kReads = A_MN ? 10 : 6;   // LDS read instructions per step

  if (!pipe.staged) {
    const uint32_t first = base + p0 * kStageBytes;
    if (A_MN) stage_mn(A, 0, first); else stage(A, 0, first);
    stage(B, 0, first + kOpBytes);
  }
  wait_vm<0>();
  __syncthreads();
  read_frags(0, 0, 0);

  constexpr int kSteps = kBK / 16;
  constexpr int kLast = (kSteps - 1) & 1;   // register set of the last step
  const bool chain = nextA != nullptr;
  auto slice = [&](int kt, bool more) {
    const uint32_t nxt = base + ((p0 + kt + 1) & 1) * kStageBytes;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < kSteps - 1; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      // the other slot was freed by the barrier of the previous slice
      if (more && ks == 0) {
        if (A_MN) stage_mn(A, (kt + 1) * kBK, nxt); else stage(A, (kt + 1) * kBK, nxt);
      }
      if (more && ks == 1) stage(B, (kt + 1) * kBK, nxt + kOpBytes);
      if (!more && chain && ks == 0) {
        if (A_MN) stage_mn(*nextA, 0, nxt); else stage(*nextA, 0, nxt);
      }
      if (!more && chain && ks == 1) stage(*nextB, 0, nxt + kOpBytes);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(kt, ks + 1, (ks + 1) & 1);
      mfma(ks & 1, 0, 8);
      Pin<8, kReads, 0>::run();
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma(kLast, 0, 4);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      // this wave's loads of slice kt + 1 are done; the barrier publishes
      // everybody's and certifies that slice kt has been read by all waves
      wait_vm<0>();
      __syncthreads();
      read_frags(kt + 1, 0, kLast ^ 1);
    }
    __builtin_amdgcn_s_setprio(1);
    mfma(kLast, 4, 8);
    if (more) Pin<4, kReads, 0>::run();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  for (int kt = 0; kt < nk - 1; ++kt) slice(kt, true);
  slice(nk - 1, false);
  pipe.slot = (p0 + nk) & 1;
  pipe.staged = chain;
  __syncthreads();
}

// Row (within the wave's 128 rows) held by register r of sub-block i.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

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

  int tgt[2];
  Stats st[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tok = tok0 + wn * 64 + j * 32 + (lane & 31);
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
    f32x16 acc[4][2];
    if (vt + S < n_vt) {
      const int v1 = v0 + S * kTile;
      const Operand na{W + (int64_t)v1 * H, H, min(kTile, V - v1)};
      mma_tile<false>(oa, ob, H, lds, acc, pipe, &na, &ob);
    } else {
      mma_tile<false>(oa, ob, H, lds, acc, pipe);
    }

    const int vrow0 = v0 + wm * 128;
    // ragged last tile: rows past V take no part. Their logits are set to
    // kNegBig so they never win the max (unless the wave has no row left),
    // and their exponentials are zeroed outright: scaled by sc < 1 the
    // rounding error of kNegBig * sc alone would overflow exp2.
    const bool ragged = vrow0 + 128 > V;
    if (ragged) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool live = vrow0 + acc_row(i, r, lane) < V;
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j][r] = live ? acc[i][j][r] : kNegBig;
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // target logit: one-hot select, only in waves whose rows hold a target
      const int tr = tgt[j] - vrow0;
      const bool hit = (tr >= 0) && (tr < 128);
      if (__any(hit)) {
        float zt = st[j].zt;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) zt = (acc_row(i, r, lane) == tr) ? acc[i][j][r] : zt;
        st[j].zt = zt;
      }
      float mx = acc[0][j][0];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = nan_max(mx, acc[i][j][r]);
      const float mnew = nan_max(st[j].m2, mx * sc);   // sc > 0: max commutes with the scaling
      const float dm = st[j].m2 - mnew;
      const float alpha = fast_exp2(dm);
      float s1 = alpha * st[j].s1;
      float s2 = alpha * (st[j].s2 + dm * st[j].s1);
      if (!ragged) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float d = fmaf(acc[i][j][r], sc, -mnew);
            const float e = fast_exp2(d);
            s1 += e;
            s2 = fmaf(e, d, s2);
          }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool live = vrow0 + acc_row(i, r, lane) < V;
            const float d = live ? fmaf(acc[i][j][r], sc, -mnew) : 0.0f;
            const float e = live ? fast_exp2(d) : 0.0f;
            s1 += e;
            s2 = fmaf(e, d, s2);
          }
      }
      st[j].m2 = mnew;
      st[j].s1 = s1;
      st[j].s2 = s2;
    }
  }

  // lanes l and l+32 hold other rows of the same tokens
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    Stats o;
    o.m2 = __shfl_xor(st[j].m2, 32);
    o.s1 = __shfl_xor(st[j].s1, 32);
    o.s2 = __shfl_xor(st[j].s2, 32);
    o.zt = __shfl_xor(st[j].zt, 32);
    st[j] = (lane < 32) ? merge_stats(st[j], o) : merge_stats(o, st[j]);
  }
  // waves wm = 0 and wm = 1 hold the two vocabulary halves of the same tokens
  float4* xch = reinterpret_cast<float4*>(lds);
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      xch[(wn * 2 + j) * 32 + lane] = make_float4(st[j].m2, st[j].s1, st[j].s2, st[j].zt);
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 q = xch[(wn * 2 + j) * 32 + lane];
      const Stats o{q.x, q.y, q.z, q.w};
      const Stats m = merge_stats(st[j], o);
      const int tok = tok0 + wn * 64 + j * 32 + lane;
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
// by both gradient GEMMs (the dW GEMM through transposed LDS reads). Launch
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
  int t_in[2];
  float l_in[2], e_in[2], gl_in[2], ge_in[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tl = tl0 + wn * 64 + j * 32 + (lane & 31);
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
  f32x16 acc[4][2];
  Pipe pipe;
  mma_tile<false>(oa, ob, H, lds, acc, pipe);

  float nlseL[2], c0[2], c1[2], gl[2];
  int tr[2];
  bool live[2];
  const int vw0 = vl0 + wm * 128;   // block-local vocabulary row of this wave
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t_in[j];
    live[j] = (t >= 0) && (t < Vtot);
    // masked tokens: every input is replaced (selected, never multiplied), so
    // whatever their rows hold cannot reach dz
    const float L = live[j] ? l_in[j] : 0.0f;
    const float Hn = live[j] ? e_in[j] : 0.0f;
    const float ga = live[j] ? gl_in[j] : 0.0f;
    const float gb = live[j] ? ge_in[j] : 0.0f;
    nlseL[j] = -L * kLog2e;
    // dz = p * (c1 * d + c0) (+ g_l / T at the target), d = log2 p
    c0[j] = -(ga + gb * Hn) * s.invT;
    c1[j] = -(gb * kLn2) * s.invT;
    gl[j] = ga * s.invT;
    // target row relative to this wave's rows (a target of another shard or
    // block lands outside [0, 128) or on rows the ragged mask zeroes)
    tr[j] = live[j] ? (t - s.voff - v0 - vw0) : -1;
  }
  const bool any_dead = __any(!live[0] || !live[1]);
  const bool ragged = (vw0 + 128 > Vb);

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tl = tl0 + wn * 64 + j * 32 + (lane & 31);
    const bool hit_any = __any(tr[j] >= 0 && tr[j] < 128);
    uint16_t* row = s.z_dz + (int64_t)tl * s.ld_dz + vw0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = g * 4 + q;
          const float d = fmaf(acc[i][j][r], s.sc, nlseL[j]);
          const float p = fast_exp2(d);
          float x = p * fmaf(c1[j], d, c0[j]);
          if (hit_any) x = (acc_row(i, r, lane) == tr[j]) ? x + gl[j] : x;
          if (any_dead) x = live[j] ? x : 0.0f;
          if (ragged) x = (vw0 + acc_row(i, r, lane) < Vb) ? x : 0.0f;
          v[q] = x;
        }
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(row + i * 32 + 8 * g + 4 * (lane >> 5)) = w;
      }
  }
}

// Writes a wave's 128 x 64 accumulator block into a float32 matrix (row
// r_base + acc_row(i, r, lane), column c_base + 32 j + lane % 32; rows at or
// past `rows` and columns at or past `cols` are skipped), storing or adding.
// Rows whose target is masked (`targets` given, id outside [0, Vtot)) are
// stored as 0, or left unchanged when adding. The read-modify-write is
// batched per 32-row sub-block: its loads (and target ids) are all in flight
// before the first add; one load-add-store per element would wait out the
// whole memory latency 128 times per lane.
__device__ __forceinline__ void write_acc(float* __restrict__ out, int64_t ld, int r_base, int rows,
                                          int c_base, int cols, bool add, const int32_t* __restrict__ targets,
                                          int t_base, int Vtot, const f32x16 (&acc)[4][2]) {
  const int lane = threadIdx.x & 63;
  bool col_ok[2];
  int col[2];   // clamped into range, so every load below is unconditional
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = c_base + j * 32 + (lane & 31);
    col_ok[j] = c < cols;
    col[j] = col_ok[j] ? c : cols - 1;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float old[16][2];
    bool row_ok[16], live[16];
    int row[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = r_base + acc_row(i, r, lane);
      row_ok[r] = m < rows;
      row[r] = row_ok[r] ? m : rows - 1;
      live[r] = true;
    }
    if (targets != nullptr) {
      int t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = targets[t_base + row[r]];
#pragma unroll
      for (int r = 0; r < 16; ++r) live[r] = (t[r] >= 0) && (t[r] < Vtot);
    }
    if (add) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int j = 0; j < 2; ++j) old[r][j] = out[(int64_t)row[r] * ld + col[j]];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!(row_ok[r] && col_ok[j])) continue;
        float* p = out + (int64_t)row[r] * ld + col[j];
        if (add) {
          if (live[r]) *p = old[r][j] + acc[i][j][r];
        } else {
          *p = live[r] ? acc[i][j][r] : 0.0f;
        }
      }
    }
  }
}

// dW tile: dW[v0 + m][n] (+)= sum_k dz[k][m] ht[n][t0 + k] over the block's
// tokens (A = dz read MN-contiguous, B = hidden^T with masked tokens zeroed).
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
  f32x16 acc[4][2];
  Pipe pipe;
  mma_tile<true>(oa, ob, (s.g_Ct + kBK - 1) / kBK * kBK, lds, acc, pipe);
  write_acc(s.dW + (int64_t)s.g_v0 * H, H, m0 + wm * 128, s.g_Vb, h0 + wn * 64, H, s.g_acc_dW != 0,
            nullptr, 0, 0, acc);
}

// dh tile: dh[t0 + m][n] (+)= sum_k dz[m][k] Wt[n][v0 + k] over the block's
// vocabulary; masked token rows are written as 0 (left alone when adding).
__device__ __forceinline__ void dh_tile(const BwdStep& s, int vid, char* lds) {
  int mt, hb;
  raster(vid, s.n_dh / s.n_ht, s.n_ht, 4, mt, hb);
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int m0 = mt * kTile;
  const int h0 = hb * kTile;
  const int H = s.H;
  const Operand oa{s.g_dz + (int64_t)m0 * s.ld_dz, s.ld_dz, kTile};
  const Operand ob{s.Wt + (int64_t)h0 * s.ld_wt + s.g_v0, s.ld_wt, kTile};
  f32x16 acc[4][2];
  Pipe pipe;
  mma_tile<false>(oa, ob, (s.g_Vb + kBK - 1) / kBK * kBK, lds, acc, pipe);
  write_acc(s.dh + (int64_t)s.g_t0 * H, H, m0 + wm * 128, s.g_Ct, h0 + wn * 64, H, s.g_acc_dh != 0,
            s.targets, s.g_t0, s.Vtot, acc);
}

// One backward launch: each XCD (workgroups are dealt to the 8 XCDs
// round-robin) takes an equal share of each kind of tile: its eighth of the
// dW tiles and of the dh tiles (the kind with the longer K first), then its
// eighth of the cotangent tiles, so the long tiles start first everywhere and
// the short ones fill the tail. (Cutting the concatenated gradient-tile list
// into eight ranges instead piles all dh tiles onto the last XCDs, which
// doubles their share of the work when the two kinds' K differ.)
__global__ __launch_bounds__(kThreads) void bwd_step_kernel(const BwdStep s) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int xcd = blockIdx.x & 7;
  const int loc = blockIdx.x >> 3;
  const int n_z = s.z_ntt * s.z_nvt;
  const int dw_lo = xcd * s.n_dw / 8;
  const int dw_cnt = (xcd + 1) * s.n_dw / 8 - dw_lo;
  const int dh_lo = xcd * s.n_dh / 8;
  const int dh_cnt = (xcd + 1) * s.n_dh / 8 - dh_lo;
  const int z_lo = xcd * n_z / 8;
  const int z_cnt = (xcd + 1) * n_z / 8 - z_lo;
  const bool dh_first = s.g_Vb > s.g_Ct;   // dh tiles run K = Vb, dW tiles K = Ct
  const int first_cnt = dh_first ? dh_cnt : dw_cnt;
  const int g_cnt = dw_cnt + dh_cnt;
  if (loc < g_cnt) {
    const bool is_dh = (loc < first_cnt) == dh_first;
    if (is_dh) {
      dh_tile(s, dh_lo + (dh_first ? loc : loc - dw_cnt), lds);
    } else {
      dw_tile(s, dw_lo + (dh_first ? loc - dh_cnt : loc), lds);
    }
  } else if (loc - g_cnt < z_cnt) {
    dz_tile(s, z_lo + loc - g_cnt, lds);
  }
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

hipError_t launch_bwd_step(const BwdStep& st, hipStream_t stream) {
  const int n_g = st.n_dw + st.n_dh;
  const int n_z = st.z_ntt * st.z_nvt;
  int per = 0;
  for (int x = 0; x < 8; ++x)
    per = max(per, ((x + 1) * st.n_dw / 8 - x * st.n_dw / 8) + ((x + 1) * st.n_dh / 8 - x * st.n_dh / 8) +
                       ((x + 1) * n_z / 8 - x * n_z / 8));
  if (per == 0) return hipSuccess;
  const double H = (double)st.H;
  const double gc = (double)st.g_Ct, gv = (double)st.g_Vb;
  const double zc = (double)st.z_Ct, zv = (double)st.z_Vb;
  trace_begin(stream);
  hipLaunchKernelGGL(bwd_step_kernel, dim3(8 * per), dim3(kThreads), 0, stream, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // algorithmic work: 2 Ct Vb H per GEMM (dh, dW, and the recomputed logits);
  // bytes: the dz block written once and read once, operand panels, f32 outputs
  const double fl = (n_g ? 4.0 * gc * gv * H : 0.0) + (n_z ? 2.0 * zc * zv * H : 0.0);
  const double by = (n_g ? 2.0 * gc * gv + 2.0 * (gc + gv) * H +
                               4.0 * H * (gc * (1 + st.g_acc_dh) + gv * (1 + st.g_acc_dW)) : 0.0) +
                    (n_z ? 2.0 * zc * zv + 2.0 * (zc + zv) * H + 20.0 * zc : 0.0);
  trace_end(kBwdStep, stream, fl, by);
  return hipSuccess;
}

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
