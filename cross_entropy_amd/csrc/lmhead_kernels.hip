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
// 512-thread workgroup (8 wave64s as 2 x 4, each owning 128 x 64), K staged
// through LDS in double-buffered 64-deep slices, v_mfma_f32_32x32x16_bf16.
// Operands are either K-contiguous (loaded with 16-byte vector loads) or
// MN-contiguous (loaded as 8 x 4 blocks and transposed in registers with
// byte permutes before the LDS write), so no operand is ever copied into a
// transposed buffer.
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
constexpr int kTile = 256;                 // BM = BN
constexpr int kBK = 64;                    // K slice per LDS stage
constexpr int kRowBytes = kBK * 2 + 16;    // 128 data bytes + 16 pad: conflict-free 16 B reads
constexpr int kTileBytes = kTile * kRowBytes;
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kLdsBytes = 2 * kStageBytes; // 147,456 B of the 160 KB per CU

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegBig = -1.0e30f;        // "minus infinity" that keeps 0 * x finite

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// ---------------------------------------------------------------------------
// Operand loaders. Each stages one [256 rows x 64 K] slice into LDS as
// rows of 64 K values (128 B) padded to kRowBytes.

// K-contiguous operand: element (row, k) at base[row * ld + k].
struct LoadK {
  const uint16_t* base;
  int64_t ld;
  int rows;          // rows of this tile that exist; others load as 0
  uint4 r[4];

  __device__ __forceinline__ void load(int k0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + kThreads * j;
      const int row = idx >> 3;
      const int ch = idx & 7;
      if (row < rows) {
        r[j] = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + k0 + ch * 8);
      } else {
        r[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + kThreads * j;
      const int row = idx >> 3;
      const int ch = idx & 7;
      *reinterpret_cast<uint4*>(lds + row * kRowBytes + ch * 16) = r[j];
    }
  }
};

// MN-contiguous operand: element (row, k) at base[k * ld + row]. Each thread
// loads 8 K-rows x 4 columns (8-byte loads) and transposes them in registers
// into 4 rows of 8 consecutive K values. K-rows at or beyond k_valid load as
// 0; with `tgt` set, K-rows whose target id lies outside [0, V) load as 0 too
// (masked tokens: their hidden rows never reach a product, whatever they hold).
struct LoadMN {
  const uint16_t* base;
  int64_t ld;
  int k_valid;
  int cols;          // columns (rows of the staged tile) that exist, multiple of 4
  const int32_t* tgt;
  int V;
  uint2 r[8];

  __device__ __forceinline__ void load(int k0) {
    const int tid = threadIdx.x;
    const int kg = tid & 7;
    const int cg = tid >> 3;
    const bool col_ok = cg * 4 < cols;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int k = k0 + kg * 8 + q;
      bool ok = col_ok && (k < k_valid);
      if (tgt != nullptr && ok) {
        const int t = tgt[k];
        ok = (t >= 0) && (t < V);
      }
      if (ok) {
        r[q] = *reinterpret_cast<const uint2*>(base + (int64_t)k * ld + cg * 4);
      } else {
        r[q] = make_uint2(0u, 0u);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int tid = threadIdx.x;
    const int kg = tid & 7;
    const int cg = tid >> 3;
    // column c of the 8 x 4 block: word w packs K-rows 2w (low) and 2w+1 (high)
    uint4 o0, o1, o2, o3;
    o0.x = __builtin_amdgcn_perm(r[1].x, r[0].x, 0x05040100u);
    o0.y = __builtin_amdgcn_perm(r[3].x, r[2].x, 0x05040100u);
    o0.z = __builtin_amdgcn_perm(r[5].x, r[4].x, 0x05040100u);
    o0.w = __builtin_amdgcn_perm(r[7].x, r[6].x, 0x05040100u);
    o1.x = __builtin_amdgcn_perm(r[1].x, r[0].x, 0x07060302u);
    o1.y = __builtin_amdgcn_perm(r[3].x, r[2].x, 0x07060302u);
    o1.z = __builtin_amdgcn_perm(r[5].x, r[4].x, 0x07060302u);
    o1.w = __builtin_amdgcn_perm(r[7].x, r[6].x, 0x07060302u);
    o2.x = __builtin_amdgcn_perm(r[1].y, r[0].y, 0x05040100u);
    o2.y = __builtin_amdgcn_perm(r[3].y, r[2].y, 0x05040100u);
    o2.z = __builtin_amdgcn_perm(r[5].y, r[4].y, 0x05040100u);
    o2.w = __builtin_amdgcn_perm(r[7].y, r[6].y, 0x05040100u);
    o3.x = __builtin_amdgcn_perm(r[1].y, r[0].y, 0x07060302u);
    o3.y = __builtin_amdgcn_perm(r[3].y, r[2].y, 0x07060302u);
    o3.z = __builtin_amdgcn_perm(r[5].y, r[4].y, 0x07060302u);
    o3.w = __builtin_amdgcn_perm(r[7].y, r[6].y, 0x07060302u);
    char* p = lds + (cg * 4) * kRowBytes + kg * 16;
    *reinterpret_cast<uint4*>(p) = o0;
    *reinterpret_cast<uint4*>(p + kRowBytes) = o1;
    *reinterpret_cast<uint4*>(p + 2 * kRowBytes) = o2;
    *reinterpret_cast<uint4*>(p + 3 * kRowBytes) = o3;
  }
};

// ---------------------------------------------------------------------------
// The tile core: acc[i][j] (wave sub-block i of 32 A-rows, j of 32 B-rows)
// = sum over k < K of A[row][k] * B[col][k]. K is a multiple of 64.
// Ends with a barrier, so LDS may be reused right after it returns.
template <class LA, class LB>
__device__ __forceinline__ void mma_tile(LA& la, LB& lb, int K, char* lds, f32x16 (&acc)[4][2]) {
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

  const int nk = K / kBK;
  la.load(0);
  lb.load(0);
  la.store(lds);
  lb.store(lds + kTileBytes);
  __syncthreads();

  const int a_off = (wm * 128 + (lane & 31)) * kRowBytes + (lane >> 5) * 16;
  const int b_off = kTileBytes + (wn * 64 + (lane & 31)) * kRowBytes + (lane >> 5) * 16;

  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = lds + (kt & 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load((kt + 1) * kBK);
      lb.load((kt + 1) * kBK);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(cur + a_off + i * 32 * kRowBytes + ks * 32);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(cur + b_off + j * 32 * kRowBytes + ks * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      char* nxt = lds + ((kt + 1) & 1) * kStageBytes;
      la.store(nxt);
      lb.store(nxt + kTileBytes);
    }
    __syncthreads();
  }
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
  const float m = fmaxf(a.m2, b.m2);
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
__global__ __launch_bounds__(kThreads) void fwd_stats_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ targets, int N, int H, int V, int S, int n_tt, int n_vt,
    float4* __restrict__ part, int64_t part_ld) {
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
    tgt[j] = tok < N ? targets[tok] : -1;
    st[j].m2 = kNegBig;
    st[j].s1 = 0.0f;
    st[j].s2 = 0.0f;
    st[j].zt = 0.0f;
  }

  LoadK lb{hidden + (int64_t)tok0 * H, H, min(kTile, N - tok0)};
  for (int vt = s; vt < n_vt; vt += S) {
    const int v0 = vt * kTile;
    LoadK la{W + (int64_t)v0 * H, H, min(kTile, V - v0)};
    f32x16 acc[4][2];
    mma_tile(la, lb, H, lds, acc);

    const int vrow0 = v0 + wm * 128;
    if (vrow0 + 128 > V) {   // ragged last tile: rows past V take no part
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
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
      const float mnew = fmaxf(st[j].m2, mx * kLog2e);
      const float dm = st[j].m2 - mnew;
      const float alpha = fast_exp2(dm);
      float s1 = alpha * st[j].s1;
      float s2 = alpha * (st[j].s2 + dm * st[j].s1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float d = fmaf(acc[i][j][r], kLog2e, -mnew);
          const float e = fast_exp2(d);
          s1 += e;
          s2 = fmaf(e, d, s2);
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

// Split merge: per token, the S partials in split order, by log-sum-exp.
__global__ __launch_bounds__(256) void fwd_merge_kernel(
    const float4* __restrict__ part, int64_t part_ld, int S, const int32_t* __restrict__ targets,
    int N, int V, float* __restrict__ logp, float* __restrict__ entropy, float* __restrict__ lse) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  float4 q = part[i];
  Stats a{q.x, q.y, q.z, q.w};
  for (int s = 1; s < S; ++s) {
    q = part[(int64_t)s * part_ld + i];
    a = merge_stats(a, Stats{q.x, q.y, q.z, q.w});
  }
  const int t = targets[i];
  const bool valid = (t >= 0) && (t < V);
  const float l2s = log2f(a.s1);
  const float l = kLn2 * (a.m2 + l2s);               // lse = m + ln(sum e^(z-m))
  const float h = kLn2 * (l2s - a.s2 / a.s1);        // lse - sum p z
  logp[i] = valid ? a.zt - l : 0.0f;
  lse[i] = valid ? l : 0.0f;
  if (entropy != nullptr) entropy[i] = valid ? h : 0.0f;
}

// ---------------------------------------------------------------------------
// Backward, step 1: recompute a logits tile of the block [t0, t0+Ct) x
// [v0, v0+Vb) and write its cotangent
//   dz = g_l (onehot - p) - g_e p (log p + entropy),  p = 2^(z log2e - lse log2e)
// as bf16 into the block buffer dz[token - t0][vocab - v0] (row stride ld).
// Rows/columns outside the block, masked tokens and vocabulary past V are
// written as 0, so the gradient GEMMs can run over the padded block.
__global__ __launch_bounds__(kThreads) void bwd_dz_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ targets, int V, int H,
    const float* __restrict__ lse, const float* __restrict__ entropy,
    const float* __restrict__ g_logp, const float* __restrict__ g_ent,
    int t0, int Ct, int v0, int Vb, int n_tt, int n_vt,
    uint16_t* __restrict__ dz, int64_t ld) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int vid = xcd_remap(blockIdx.x, gridDim.x);
  if (vid >= n_tt * n_vt) return;
  int vt, tt;
  raster(vid, n_vt, n_tt, 4, vt, tt);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int tl0 = tt * kTile;   // token offset in the block
  const int vl0 = vt * kTile;   // vocabulary offset in the block

  LoadK la{W + (int64_t)(v0 + vl0) * H, H, min(kTile, Vb - vl0)};
  LoadK lb{hidden + (int64_t)(t0 + tl0) * H, H, min(kTile, Ct - tl0)};
  f32x16 acc[4][2];
  mma_tile(la, lb, H, lds, acc);

  float nlseL[2], c0[2], c1[2], gl[2];
  int tr[2];
  bool live[2];
  const int vw0 = vl0 + wm * 128;   // block-local vocabulary row of this wave
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tl = tl0 + wn * 64 + j * 32 + (lane & 31);
    const int tok = t0 + tl;
    int t = -1;
    if (tl < Ct) t = targets[tok];
    live[j] = (t >= 0) && (t < V);
    const float L = live[j] ? lse[tok] : 0.0f;
    const float Hn = (live[j] && entropy != nullptr) ? entropy[tok] : 0.0f;
    const float a = (live[j] && g_logp != nullptr) ? g_logp[tok] : 0.0f;
    const float b = (live[j] && g_ent != nullptr) ? g_ent[tok] : 0.0f;
    nlseL[j] = -L * kLog2e;
    c0[j] = -(a + b * Hn);       // dz = p * (c1 * d + c0) - ... with d = log2 p
    c1[j] = -(b * kLn2);
    gl[j] = a;
    tr[j] = live[j] ? (t - v0 - vw0) : -1;
  }
  const bool any_dead = __any(!live[0] || !live[1]);
  const bool ragged = (vw0 + 128 > Vb);

  uint16_t* out = dz + vw0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tl = tl0 + wn * 64 + j * 32 + (lane & 31);
    const bool hit_any = __any(tr[j] >= 0 && tr[j] < 128);
    uint16_t* row = out + (int64_t)tl * ld;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = g * 4 + q;
          const float d = fmaf(acc[i][j][r], kLog2e, nlseL[j]);
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

// ---------------------------------------------------------------------------
// Backward, step 2: both gradient GEMMs of one block in one launch.
//   dW tiles (first, the longer ones): dW[v0 + m][n] (+)= sum_k dz[k][m] h[t0 + k][n]
//   dh tiles: dh[t0 + m][n] (+)= sum_k dz[m][k] W[v0 + k][n]
// `acc_dW` / `acc_dh` select accumulate-into (later blocks) or overwrite
// (first block of the fixed block order), which keeps the sums deterministic.
__global__ __launch_bounds__(kThreads) void bwd_grad_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ targets, int N, int H, int V,
    int t0, int Ct, int v0, int Vb, const uint16_t* __restrict__ dz, int64_t ld,
    int n_ht, int n_dw, int n_dh, float* __restrict__ dh, float* __restrict__ dW,
    int acc_dh, int acc_dW) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int vid = xcd_remap(blockIdx.x, gridDim.x);
  if (vid >= n_dw + n_dh) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  f32x16 acc[4][2];

  if (vid < n_dw) {
    int mt, ht;
    raster(vid, n_dw / n_ht, n_ht, 4, mt, ht);
    const int m0 = mt * kTile;
    const int h0 = ht * kTile;
    LoadMN la{dz + m0, ld, Ct, kTile, nullptr, V};
    LoadMN lb{hidden + (int64_t)t0 * H + h0, H, Ct, min(kTile, H - h0), targets + t0, V};
    const int K = (Ct + kBK - 1) / kBK * kBK;
    mma_tile(la, lb, K, lds, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 128 + acc_row(i, r, lane);
        if (m >= Vb) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = h0 + wn * 64 + j * 32 + (lane & 31);
          if (n < H) {
            float* p = dW + (int64_t)(v0 + m) * H + n;
            *p = acc_dW ? (*p + acc[i][j][r]) : acc[i][j][r];
          }
        }
      }
  } else {
    int mt, ht;
    raster(vid - n_dw, n_dh / n_ht, n_ht, 4, mt, ht);
    const int m0 = mt * kTile;
    const int h0 = ht * kTile;
    LoadK la{dz + (int64_t)m0 * ld, ld, kTile};
    LoadMN lb{W + (int64_t)v0 * H + h0, H, Vb, min(kTile, H - h0), nullptr, V};
    const int K = (Vb + kBK - 1) / kBK * kBK;
    mma_tile(la, lb, K, lds, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 128 + acc_row(i, r, lane);
        if (m >= Ct) continue;
        const int tok = t0 + m;
        const int t = targets[tok];
        const bool live = (t >= 0) && (t < V);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = h0 + wn * 64 + j * 32 + (lane & 31);
          if (n < H) {
            float* p = dh + (int64_t)tok * H + n;
            const float v = live ? acc[i][j][r] : 0.0f;
            *p = acc_dh ? (*p + v) : v;
          }
        }
      }
  }
  (void)N;
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
  hipLaunchKernelGGL(fwd_stats_kernel, dim3(round8(wg)), dim3(kThreads), 0, stream, a.hidden, a.W,
                     a.targets, (int)a.N, (int)a.H, (int)a.V, a.S, a.n_tt, a.n_vt,
                     reinterpret_cast<float4*>(a.part), a.part_ld);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_merge_kernel, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(a.part), a.part_ld, a.S, a.targets, (int)a.N,
                     (int)a.V, a.logp, a.entropy, a.lse);
  return hipGetLastError();
}

hipError_t launch_bwd_block(const BwdArgs& a, const BwdBlock& b, hipStream_t stream) {
  const int n_tt = (int)((b.Ct + kTile - 1) / kTile);
  const int n_vt = (int)((b.Vb + kTile - 1) / kTile);
  hipLaunchKernelGGL(bwd_dz_kernel, dim3(round8((long long)n_tt * n_vt)), dim3(kThreads), 0, stream,
                     a.hidden, a.W, a.targets, (int)a.V, (int)a.H, a.lse, a.entropy, a.g_logp,
                     a.g_ent, (int)b.t0, (int)b.Ct, (int)b.v0, (int)b.Vb, n_tt, n_vt, a.dz, a.ld_dz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_ht = (int)((a.H + kTile - 1) / kTile);
  const int n_dw = n_vt * n_ht;
  const int n_dh = n_tt * n_ht;
  hipLaunchKernelGGL(bwd_grad_kernel, dim3(round8((long long)n_dw + n_dh)), dim3(kThreads), 0,
                     stream, a.hidden, a.W, a.targets, (int)a.N, (int)a.H, (int)a.V, (int)b.t0,
                     (int)b.Ct, (int)b.v0, (int)b.Vb, a.dz, a.ld_dz, n_ht, n_dw, n_dh, a.dh, a.dW,
                     b.acc_dh, b.acc_dW);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace lmh
