// lmhead_internal.h -- launch descriptors shared by the C ABI (lmhead_api.hip)
// and the kernels (lmhead_kernels.hip). Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lmh {

constexpr int kTileRows = 256;   // output tile edge of every MMA kernel
constexpr int kNumCUs = 256;     // MI355X: 8 XCDs x 32 CUs

// Forward: token tiles x vocabulary splits of the tile kernel, then the merge.
struct FwdPlan {
  int n_tt = 0;          // token tiles of 256
  int n_vt = 0;          // vocabulary tiles of 256
  int S = 0;             // vocabulary splits (partials per token)
  int64_t part_ld = 0;   // tokens per split row of the partials array
  size_t bytes = 0;      // workspace bytes (partials)
};

// Row stride (elements) for a bf16 operand of the backward GEMMs holding rows
// of at least x elements: a multiple of 64 elements (128 bytes) whose
// quotient by 64 is odd. 256-row tiles of rows strided by a large power of
// two crowd onto few memory channels (measured: such tiles run ~20% slower).
inline int64_t spread_ld(int64_t x) { return (((x + 63) / 64) | 1) * 64; }

// Backward: the token x vocabulary plane is cut into blocks of at most
// Ct x Vb; each block's cotangent is one bf16 buffer dz [Ct][ld_dz], double
// buffered (4 bytes per element in all, like one float32 block, the stride
// padding included). The workspace also holds hidden^T [H_pad][ld_ht]
// (masked tokens zeroed) and W's last V % 64 rows zero-padded to 64 rows
// [64][H] (the dh GEMM's last vocabulary slice).
struct BwdPlan {
  int64_t Ct = 0, Vb = 0;      // block edges (tokens, vocabulary), multiples of 256
  int64_t n_tb = 0, n_vb = 0;  // blocks along tokens and vocabulary
  int64_t N_pad = 0, V_pad = 0, H_pad = 0;
  int64_t ld_dz = 0, ld_ht = 0;                   // row strides (spread_ld)
  size_t off_dz1 = 0, off_ht = 0, off_tail = 0;   // byte offsets in the workspace
  size_t off_ctr = 0;          // 8 int32 cotangent-tile counters per launch (n_tb * n_vb + 1 launches)
  size_t bytes = 0;            // total
  // bf16-gradient backward: float32 accumulators of the gradients across
  // blocks. With vocab_outer (N <= V) the blocks run vocabulary-major: dh
  // accumulates in acc_dh [N_pad][H] over the whole call and each vocabulary
  // block's dW in acc_dW [Vb][H]; otherwise token-major: dW in acc_dW
  // [V_pad][H] over the call and each token block's dh in acc_dh [Ct][H].
  bool vocab_outer = false;
  size_t off_acc_dh = 0, off_acc_dW = 0;
  size_t bytes_bf16 = 0;       // total with the accumulators
};

FwdPlan plan_forward(int64_t N, int64_t H, int64_t V);
BwdPlan plan_backward(int64_t N, int64_t H, int64_t V, int64_t chunk_size);

struct FwdArgs {
  const uint16_t* hidden;
  const uint16_t* W;
  const int32_t* targets;
  int64_t N, H, V;
  int S, n_tt, n_vt;
  int64_t voff;   // global id of W's first row (vocabulary shard), 0 for the whole table
  int64_t Vtot;   // valid target ids are [0, Vtot)
  float sc;       // log2(e) / T
  float invT;     // 1 / T
  void* part;
  int64_t part_ld;
  float* logp;
  float* entropy;
  float* lse;
  float* rec;     // shard partial records [N][4] instead of logp/entropy/lse, or NULL
};

// Where a gradient tile of the bf16-gradient backward reads and writes.
enum SrcKind { kSrcNone = 0, kSrcF32 = 1, kSrcBf16 = 2 };
struct GradOut {
  const void* src = nullptr;
  int src_kind = kSrcNone;
  void* dst = nullptr;
  int dst_bf16 = 0;
};

// One backward launch: the gradient tiles of one block (n_dw + n_dh tiles,
// none if 0) and the cotangent tiles of the next (z_ntt * z_nvt, none if 0).
struct BwdStep {
  const uint16_t* hidden;
  const uint16_t* W;
  const int32_t* targets;
  int N, H, V;     // V: rows of W (the shard's vocabulary)
  int voff, Vtot;  // global id of W's first row; valid target ids are [0, Vtot)
  const float* lse;
  const float* entropy;
  const float* g_logp;
  const float* g_ent;
  float sc;     // log2(e) / T
  float invT;   // 1 / T
  const uint16_t* ht;   // hidden^T [H_pad][N_pad], masked tokens zeroed
  int64_t ld_ht;
  const uint16_t* W_tail;   // W rows v_tail .. V-1 padded with zero rows to 64, or NULL if V % 64 == 0
  int v_tail;               // V rounded down to a multiple of 64
  float* dh;
  float* dW;
  int64_t ld_dz;        // row stride of both dz buffers
  // gradient part
  const uint16_t* g_dz;
  int g_t0, g_Ct, g_v0, g_Vb, g_acc_dh, g_acc_dW;
  int n_dw, n_dh, n_ht;
  // cotangent part
  uint16_t* z_dz;
  int* z_ctr;   // this launch's 8 per-XCD tile counters (zero before the launch)
  int z_t0, z_Ct, z_v0, z_Vb, z_ntt, z_nvt;
  // bf16-gradient backward only (bwd_step_bf16_kernel): per gradient, where
  // this block's tiles read the values they add to (none, a float32
  // accumulator or the caller's bf16 gradient) and where they write the sum
  // (a float32 accumulator, or the caller's bf16 gradient, rounded once),
  // both pointing at the block's first row (row stride H). Masked tokens'
  // dh rows are stored as 0 when dh_dead_zero, else left as they are.
  GradOut o_dh, o_dW;
  int dh_dead_zero;
};

// Kernel ids of the tracing facility (lmhead_trace.hip).
enum KernelId { kFwdStats = 0, kFwdMerge, kBwdStep, kTranspose, kFill, kPadRows, kBwdStepBf16, kNumKernels };
void trace_begin(hipStream_t stream);
void trace_end(int kernel, hipStream_t stream, double flops, double bytes);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// merge of P shard records [P][N] (float4 each) into logp / entropy / lse
hipError_t launch_merge(const float* partials, int P, int64_t N, const int32_t* targets, int64_t Vtot,
                        float invT, float* logp, float* entropy, float* lse, hipStream_t stream);
hipError_t launch_bwd_step(const BwdStep& st, hipStream_t stream);
hipError_t launch_bwd_step_bf16(const BwdStep& st, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
hipError_t launch_pad_rows(const uint16_t* in, int64_t R, int64_t C, int64_t R_pad, uint16_t* out,
                           hipStream_t stream);
hipError_t launch_transpose(const uint16_t* in, int64_t ld_in, int64_t R, int64_t C, int64_t R_pad,
                            int64_t C_pad, const int32_t* tgt, int64_t V, uint16_t* out,
                            int64_t ld_out, hipStream_t stream);

}  // namespace lmh
