// lmhead_api.hip -- the C ABI declared in include/lmhead_logps.h: argument
// checks, work planning and launches on the caller's stream.
//
// Planning follows the chunked head of the pages (SkyRL issue "[tx] support
// long sequence", "4. Chunked LM Head"; google/tunix pull request #2876,
// the chunk loop over flattened tokens):
//  * The forward holds no [tokens, vocab] transient. It runs one tile kernel
//    over all tokens, with the vocabulary cut into S splits so that the
//    launch fills the 256 CUs; S partial (max, exp-sum, exp-weighted sum,
//    target logit) records per token are merged by log-sum-exp.
//  * The backward holds the logits' cotangent as bf16 blocks of Ct tokens x
//    Vb vocabulary entries, double buffered so that the cotangent of the next
//    block is formed while the gradient GEMMs of the current one run (one
//    launch per block). chunk_size bounds the block: the two buffers, 4 bytes
//    per element, stay within one float32 [chunk_size, V] tensor, the
//    transient the pages' chunked head holds per chunk. Within that bound the
//    block shape is chosen to cut the dh / dW accumulation traffic and launch
//    count. The workspace also holds a bf16 transpose of the hidden states
//    (input-sized; the dW GEMM's K-contiguous operand) and W's last V % 64
//    rows padded to 64 (the dh GEMM reads W as it lies, 64 rows at a time).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/lmhead_logps.h"
#include "lmhead_internal.h"

namespace lmh {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

FwdPlan plan_forward(int64_t N, int64_t H, int64_t V) {
  (void)H;
  FwdPlan p;
  p.n_tt = (int)lmh::ceil_div(N, kTileRows);
  p.n_vt = (int)lmh::ceil_div(V, kTileRows);
  const int s_max = (int)std::min<int64_t>(p.n_vt, 128);
  // makespan in tile-steps: rounds of resident workgroups x tiles per split
  auto cost = [&](int S) {
    return ceil_div((int64_t)p.n_tt * S, kNumCUs) * ceil_div(p.n_vt, S);
  };
  int64_t best = INT64_MAX;
  for (int S = 1; S <= s_max; ++S) best = std::min(best, cost(S));
  // among near-best split counts, prefer S near 6: an XCD's 32 concurrent
  // workgroups then cover ~5 token tiles x 6 vocabulary tiles, which share
  // the W and hidden tiles in its L2 about evenly (measured at N = 65536,
  // V = 151936: S = 5 or 6 beat 8 by 2%, 3 and 9 match 8, 2 and 16 lose 3%)
  int pick = 1;
  double pick_dist = 1e30;
  for (int S = 1; S <= s_max; ++S) {
    if ((double)cost(S) > 1.03 * (double)best) continue;
    const double dist = std::fabs(std::log2((double)S / 6.0));
    if (dist < pick_dist) {
      pick_dist = dist;
      pick = S;
    }
  }
  p.S = std::max(1, pick);
  p.part_ld = round_up(std::max<int64_t>(N, 1), 64);
  p.bytes = (size_t)round_up((int64_t)p.S * p.part_ld * 16, 256);
  return p;
}

BwdPlan plan_backward(int64_t N, int64_t H, int64_t V, int64_t chunk_size) {
  const int64_t T = kTileRows;
  N = std::max<int64_t>(N, 1);
  // elements of one dz buffer, stride padding included (two bf16 buffers, 4
  // bytes per element in all): at most chunk_size * V, and at least one
  // 256 x 256 tile.
  const double budget = std::max<double>((double)chunk_size * (double)V, (double)(T * spread_ld(T)));
  const int64_t n_pad = round_up(N, T);
  const int64_t v_pad = round_up(V, T);
  // model: the MFMA work is fixed; what the block shape changes is the f32
  // accumulation traffic of dh (one pass per vocabulary block) and dW (one
  // pass per token block), and the number of launches.
  const double hbm = 5.0e12;
  const double launch = 20e-6;
  BwdPlan best;
  double best_t = 1e300;
  for (int64_t ct = T; ct <= n_pad; ct += T) {
    // spread_ld(vb) = vb + 64 for vb a multiple of 256
    int64_t vb = ((int64_t)(budget / (double)ct) - 64) / T * T;
    vb = std::min(vb, v_pad);
    if (vb < T) break;
    const int64_t n_tb = ceil_div(N, ct);
    const int64_t n_vb = ceil_div(V, vb);
    const int64_t c2 = round_up(ceil_div(N, n_tb), T);   // even out the blocks
    const int64_t v2 = round_up(ceil_div(V, n_vb), T);
    const double traffic = (8.0 * N * H * n_vb + 8.0 * V * H * n_tb) / hbm;
    const double t = (double)(n_tb * n_vb + 1) * launch + traffic;
    if (t < best_t) {
      best_t = t;
      best.Ct = c2;
      best.Vb = v2;
      best.n_tb = n_tb;
      best.n_vb = n_vb;
    }
  }
  best.N_pad = round_up(N, T);
  best.V_pad = round_up(V, T);
  best.H_pad = round_up(H, T);
  best.ld_dz = spread_ld(best.Vb);
  best.ld_ht = spread_ld(best.N_pad);
  const size_t one = (size_t)round_up(best.Ct * best.ld_dz * 2, 256);
  best.off_dz1 = one;
  best.off_ht = 2 * one;
  best.off_tail = best.off_ht + (size_t)round_up(best.H_pad * best.ld_ht * 2, 256);
  best.off_ctr = best.off_tail + (size_t)round_up(64 * H * 2, 256);
  best.bytes = best.off_ctr + (size_t)round_up((best.n_tb * best.n_vb + 1) * 8 * 4, 256);
  // the bf16-gradient backward keeps the larger gradient per block and the
  // smaller one whole in float32
  best.vocab_outer = N <= V;
  const int64_t whole = best.vocab_outer ? best.N_pad : best.V_pad;
  const int64_t part = best.vocab_outer ? best.Vb : best.Ct;
  const size_t acc_whole = (size_t)round_up(whole * H * 4, 256);
  const size_t acc_part = (size_t)round_up(part * H * 4, 256);
  best.off_acc_dh = best.bytes;
  best.off_acc_dW = best.bytes + (best.vocab_outer ? acc_whole : acc_part);
  best.bytes_bf16 = best.bytes + acc_whole + acc_part;
  return best;
}

}  // namespace lmh

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return LMH_OK;
}

int check_shape(int64_t N, int64_t H, int64_t V, int64_t chunk_size) {
  if (N < 0 || N >= (int64_t(1) << 31))
    return fail(LMH_ERR_SHAPE, "N must be in [0, 2^31), got %lld", (long long)N);
  if (H <= 0 || H >= (int64_t(1) << 20))
    return fail(LMH_ERR_SHAPE, "H must be in (0, 2^20), got %lld", (long long)H);
  if (V <= 0 || V >= (int64_t(1) << 31))
    return fail(LMH_ERR_SHAPE, "V must be in (0, 2^31), got %lld", (long long)V);
  if (chunk_size <= 0) return fail(LMH_ERR_CHUNK, "chunk_size must be > 0, got %lld", (long long)chunk_size);
  if (H % 64 != 0) return fail(LMH_ERR_UNSUPPORTED, "H must be a multiple of 64, got %lld", (long long)H);
  return LMH_OK;
}

// The backward's GEMMs read 256-row tiles of the cotangent block and of the
// transposed hidden states (row strides up to V_pad and N_pad elements)
// through 32-bit byte offsets from the tile's base: 256 * stride * 2 bytes
// must stay below 2^32.
int check_backward_size(int64_t N, int64_t V) {
  const int64_t lim = int64_t(1) << 23;
  if (lmh::round_up(std::max<int64_t>(N, 1), lmh::kTileRows) >= lim || lmh::round_up(V, lmh::kTileRows) >= lim)
    return fail(LMH_ERR_UNSUPPORTED, "bwd: N (%lld) and V (%lld) rounded up to 256 must stay below 2^23",
                (long long)N, (long long)V);
  return LMH_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Base-2 scale of the tempered logits and the reciprocal temperature; at
// T = 1 these are log2(e) and 1 exactly, so the untempered entry points give
// the same bits as the tempered ones at T = 1.
float temper_scale(float temperature) { return (float)(1.4426950408889634 / (double)temperature); }
float inv_temperature(float temperature) { return (float)(1.0 / (double)temperature); }

int check_temperature(float temperature) {
  if (!(std::isfinite(temperature) && temperature > 0.0f))
    return fail(LMH_ERR_ARGS, "temperature must be finite and > 0, got %g", (double)temperature);
  if (!std::isfinite(temper_scale(temperature)) || !std::isfinite(inv_temperature(temperature)))
    return fail(LMH_ERR_ARGS, "temperature %g is too small: 1 / temperature overflows float32",
                (double)temperature);
  return LMH_OK;
}

}  // namespace

extern "C" {

const char* lmhead_logps_last_error(void) { return g_last_error.c_str(); }

const char* lmhead_logps_version(void) { return "lmhead_logps 0.1.0 (gfx950)"; }

int lmhead_logps_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t chunk_size,
                                 int with_backward, size_t* bytes_out) {
  if (bytes_out == nullptr) return fail(LMH_ERR_NULL, "bytes_out is NULL");
  const int rc = check_shape(N, H, V, chunk_size);
  if (rc != LMH_OK) return rc;
  if (with_backward) {
    const int rb = check_backward_size(N, V);
    if (rb != LMH_OK) return rb;
  }
  if (with_backward < 0 || with_backward > LMH_WS_BWD_BF16)
    return fail(LMH_ERR_ARGS, "with_backward must be 0, 1 or 2, got %d", with_backward);
  size_t b = lmh::plan_forward(N, H, V).bytes;
  if (with_backward) {
    const lmh::BwdPlan p = lmh::plan_backward(N, H, V, chunk_size);
    b = std::max(b, with_backward == LMH_WS_BWD_BF16 ? p.bytes_bf16 : p.bytes);
  }
  *bytes_out = b;
  return ok();
}

}  // extern "C"

namespace {

// Shard ranges: W holds rows [voff, voff + V) of a vocabulary of Vtot ids.
int check_shard(int64_t V, int64_t voff, int64_t Vtot) {
  if (voff < 0 || Vtot <= 0 || Vtot >= (int64_t(1) << 31) || voff > Vtot - V)
    return fail(LMH_ERR_SHAPE, "shard rows [%lld, %lld) must lie in a vocabulary [0, %lld) with 0 < %lld < 2^31",
                (long long)voff, (long long)(voff + V), (long long)Vtot, (long long)Vtot);
  return LMH_OK;
}

// The forward of W's rows [voff, voff + V); writes logp/entropy/lse, or with
// `rec` the merged partial record of this vocabulary range.
int fwd_impl(const char* who, const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
             int64_t N, int64_t H, int64_t V, int64_t voff, int64_t Vtot, int64_t chunk_size,
             float temperature, float* logp, float* entropy, float* lse, float* rec,
             void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(N, H, V, chunk_size);
  if (rc != LMH_OK) return rc;
  rc = check_shard(V, voff, Vtot);
  if (rc != LMH_OK) return rc;
  rc = check_temperature(temperature);
  if (rc != LMH_OK) return rc;
  if (N == 0) return ok();
  if (rec == nullptr) {
    if (!hidden || !W || !targets || !logp || !lse || !workspace)
      return fail(LMH_ERR_NULL, "%s: hidden, W, targets, logp, lse and workspace must be non-NULL", who);
    if (!aligned(hidden, 16) || !aligned(W, 16) || !aligned(workspace, 16) || !aligned(targets, 4) ||
        !aligned(logp, 4) || !aligned(lse, 4) || (entropy && !aligned(entropy, 4)))
      return fail(LMH_ERR_UNSUPPORTED, "%s: hidden, W and workspace need 16-byte alignment", who);
  } else {
    if (!hidden || !W || !targets || !workspace)
      return fail(LMH_ERR_NULL, "%s: hidden, W, targets, partial and workspace must be non-NULL", who);
    if (!aligned(hidden, 16) || !aligned(W, 16) || !aligned(workspace, 16) || !aligned(targets, 4) ||
        !aligned(rec, 16))
      return fail(LMH_ERR_UNSUPPORTED, "%s: hidden, W, partial and workspace need 16-byte alignment", who);
  }
  const lmh::FwdPlan p = lmh::plan_forward(N, H, V);
  if (workspace_bytes < p.bytes)
    return fail(LMH_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes, p.bytes);
  lmh::FwdArgs a{hidden, W, targets, N, H, V, p.S, p.n_tt, p.n_vt, voff, Vtot,
                 temper_scale(temperature), inv_temperature(temperature), workspace, p.part_ld,
                 logp, entropy, lse, rec};
  const hipError_t e = lmh::launch_fwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LMH_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int lmhead_logps_fwd_temp(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                          int64_t N, int64_t H, int64_t V, int64_t chunk_size, float temperature,
                          float* logp, float* entropy, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return fwd_impl("fwd", hidden, W, targets, N, H, V, 0, V, chunk_size, temperature, logp, entropy, lse,
                  nullptr, workspace, workspace_bytes, stream);
}

int lmhead_logps_fwd_shard(const uint16_t* hidden, const uint16_t* W_shard, const int32_t* targets,
                           int64_t N, int64_t H, int64_t V_shard, int64_t vocab_offset, int64_t V_total,
                           int64_t chunk_size, float temperature, float* partial, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (partial == nullptr && N > 0) return fail(LMH_ERR_NULL, "fwd_shard: partial must be non-NULL");
  return fwd_impl("fwd_shard", hidden, W_shard, targets, N, H, V_shard, vocab_offset, V_total, chunk_size,
                  temperature, nullptr, nullptr, nullptr, partial, workspace, workspace_bytes, stream);
}

int lmhead_logps_merge_shards(const float* partials, int64_t P, const int32_t* targets, int64_t N,
                              int64_t V_total, float temperature, float* logp, float* entropy,
                              float* lse, void* stream) {
  if (N < 0 || N >= (int64_t(1) << 31))
    return fail(LMH_ERR_SHAPE, "merge_shards: N must be in [0, 2^31), got %lld", (long long)N);
  if (P <= 0 || P > 65536) return fail(LMH_ERR_SHAPE, "merge_shards: P must be in [1, 65536], got %lld", (long long)P);
  if (V_total <= 0 || V_total >= (int64_t(1) << 31))
    return fail(LMH_ERR_SHAPE, "merge_shards: V_total must be in (0, 2^31), got %lld", (long long)V_total);
  int rc = check_temperature(temperature);
  if (rc != LMH_OK) return rc;
  if (N == 0) return ok();
  if (!partials || !targets || !logp || !lse)
    return fail(LMH_ERR_NULL, "merge_shards: partials, targets, logp and lse must be non-NULL");
  if (!aligned(partials, 16) || !aligned(targets, 4) || !aligned(logp, 4) || !aligned(lse, 4) ||
      (entropy && !aligned(entropy, 4)))
    return fail(LMH_ERR_UNSUPPORTED, "merge_shards: partials need 16-byte alignment");
  const hipError_t e = lmh::launch_merge(partials, (int)P, N, targets, V_total, inv_temperature(temperature),
                                         logp, entropy, lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LMH_ERR_HIP, "merge_shards: launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// Scratch of the allocation-free forward (lmhead_logps_fwd_noalloc): the
// vocabulary-split partial records, in a fixed device array that every GPU
// the library runs on holds until the process ends. Host code never passes
// the array's name to a kernel (on the host it only stands in for the
// symbol): it passes the device address hipGetSymbolAddress returns, looked
// up once per device.
static __device__ __align__(256) char scratch[LMH_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The address of `scratch` on the device the work runs on: the stream's
// device (the current device for the NULL stream). Looked up once per device,
// with that device current; the caller's current device is restored.
int scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(LMH_ERR_HIP, "fwd_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess)
      return fail(LMH_ERR_HIP, "fwd_noalloc: hipStreamGetDevice failed: %s", hipGetErrorString(e));
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LMH_ERR_UNSUPPORTED, "fwd_noalloc: device %d is beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(LMH_ERR_HIP, "fwd_noalloc: hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || p == nullptr)
      return fail(LMH_ERR_HIP, "fwd_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    if (back != hipSuccess)
      return fail(LMH_ERR_HIP, "fwd_noalloc: restoring device %d failed: %s", cur, hipGetErrorString(back));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LMH_OK;
}

}  // namespace

extern "C" {

int lmhead_logps_fwd_noalloc(const uint16_t* hidden, const uint16_t* W, const int32_t* targets, int64_t N,
                             int64_t H, int64_t V, int64_t chunk_size, float temperature, float* logp,
                             float* entropy, float* lse, void* stream) {
  int rc = check_shape(N, H, V, chunk_size);
  if (rc != LMH_OK) return rc;
  rc = check_temperature(temperature);
  if (rc != LMH_OK) return rc;
  if (N == 0) return ok();
  const size_t need = lmh::plan_forward(N, H, V).bytes;
  if (need > (size_t)LMH_NOALLOC_SCRATCH_BYTES)
    return fail(LMH_ERR_WORKSPACE,
                "fwd_noalloc: N = %lld needs %zu bytes of scratch, beyond the fixed %zu (use lmhead_logps_fwd_temp "
                "with a workspace)",
                (long long)N, need, (size_t)LMH_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  rc = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (rc != LMH_OK) return rc;
  return fwd_impl("fwd_noalloc", hidden, W, targets, N, H, V, 0, V, chunk_size, temperature, logp, entropy, lse,
                  nullptr, ws, (size_t)LMH_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

namespace {

// The backward of W's rows [voff, voff + V) of a vocabulary of Vtot ids.
// dh / dW are float32 (bf16_out false) or bf16 gradients (bf16_out true).
int bwd_impl(const char* who, const uint16_t* hidden, const uint16_t* W, const int32_t* targets, int64_t N,
             int64_t H, int64_t V, int64_t voff, int64_t Vtot, int64_t chunk_size, float temperature,
             const float* lse, const float* entropy, const float* g_logp, const float* g_ent, void* dh,
             void* dW, unsigned flags, bool bf16_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(N, H, V, chunk_size);
  if (rc != LMH_OK) return rc;
  rc = check_shard(V, voff, Vtot);
  if (rc != LMH_OK) return rc;
  rc = check_temperature(temperature);
  if (rc != LMH_OK) return rc;
  if (flags & ~(unsigned)(LMH_BWD_ACCUMULATE_DH | LMH_BWD_ACCUMULATE_DW))
    return fail(LMH_ERR_ARGS, "%s: unknown flags 0x%x", who, flags);
  const bool acc_dh = (flags & LMH_BWD_ACCUMULATE_DH) != 0;
  const bool acc_dW = (flags & LMH_BWD_ACCUMULATE_DW) != 0;
  if (g_ent != nullptr && entropy == nullptr)
    return fail(LMH_ERR_ARGS, "%s: g_ent given without the forward's entropy", who);
  if (!dW) return fail(LMH_ERR_NULL, "%s: dW must be non-NULL", who);
  if (!aligned(dW, bf16_out ? 16 : 4))
    return fail(LMH_ERR_UNSUPPORTED, "%s: dW needs %d-byte alignment", who, bf16_out ? 16 : 4);
  rc = check_backward_size(N, V);
  if (rc != LMH_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) {
    if (acc_dW) return ok();   // nothing to add
    // bf16 zeros are 32-bit zeros two at a time (V * H is even: H % 64 == 0)
    const hipError_t e = lmh::launch_fill_zero(static_cast<float*>(dW), bf16_out ? V * H / 2 : V * H, s);
    if (e != hipSuccess) return fail(LMH_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return ok();
  }
  if (!hidden || !W || !targets || !lse || !dh || !workspace)
    return fail(LMH_ERR_NULL, "%s: hidden, W, targets, lse, dh, dW and workspace must be non-NULL", who);
  if (!aligned(hidden, 16) || !aligned(W, 16) || !aligned(workspace, 16) || !aligned(dh, 16))
    return fail(LMH_ERR_UNSUPPORTED, "%s: hidden, W, dh and workspace need 16-byte alignment", who);
  const lmh::BwdPlan p = lmh::plan_backward(N, H, V, chunk_size);
  const size_t need = bf16_out ? p.bytes_bf16 : p.bytes;
  if (workspace_bytes < need)
    return fail(LMH_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes, need);
  char* ws = static_cast<char*>(workspace);
  uint16_t* dzbuf[2] = {reinterpret_cast<uint16_t*>(ws), reinterpret_cast<uint16_t*>(ws + p.off_dz1)};
  uint16_t* ht = reinterpret_cast<uint16_t*>(ws + p.off_ht);
  uint16_t* W_tail = reinterpret_cast<uint16_t*>(ws + p.off_tail);
  int* ctr = reinterpret_cast<int*>(ws + p.off_ctr);
  float* acc_h = reinterpret_cast<float*>(ws + p.off_acc_dh);
  float* acc_w = reinterpret_cast<float*>(ws + p.off_acc_dW);
  const int64_t v_tail = V / 64 * 64;
  const int64_t nb = p.n_tb * p.n_vb;
  // the cotangent-tile counters start at zero (a fill kernel, not a memset:
  // the call may be captured into a graph)
  hipError_t te = lmh::launch_fill_zero(reinterpret_cast<float*>(ctr), (nb + 1) * 8, s);
  if (te == hipSuccess)
    te = lmh::launch_transpose(hidden, H, N, H, p.N_pad, p.H_pad, targets, Vtot, ht, p.ld_ht, s);
  if (te == hipSuccess && v_tail < V) te = lmh::launch_pad_rows(W + v_tail * H, V - v_tail, H, 64, W_tail, s);
  if (te != hipSuccess) return fail(LMH_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(te));

  lmh::BwdStep st{};
  st.hidden = hidden;
  st.W = W;
  st.targets = targets;
  st.N = (int)N;
  st.H = (int)H;
  st.V = (int)V;
  st.voff = (int)voff;
  st.Vtot = (int)Vtot;
  st.lse = lse;
  st.entropy = entropy;
  st.g_logp = g_logp;
  st.g_ent = g_ent;
  st.sc = temper_scale(temperature);
  st.invT = inv_temperature(temperature);
  st.ht = ht;
  st.ld_ht = p.ld_ht;
  st.W_tail = v_tail < V ? W_tail : nullptr;
  st.v_tail = (int)v_tail;
  st.dh = bf16_out ? nullptr : static_cast<float*>(dh);
  st.dW = bf16_out ? nullptr : static_cast<float*>(dW);
  st.ld_dz = p.ld_dz;
  st.n_ht = (int)lmh::ceil_div(H, lmh::kTileRows);
  // blocks in a fixed order: token blocks outer (vocabulary blocks inner),
  // except for bf16 gradients with N <= V, which run vocabulary blocks outer
  // so that each vocabulary block's dW is complete (and rounded) before the
  // next starts. Launch j forms block j's cotangent and runs block j-1's GEMMs.
  const bool vocab_major = bf16_out && p.vocab_outer;
  auto block_of = [&](int64_t j, int64_t& tb, int64_t& vb) {
    if (vocab_major) {
      vb = j / p.n_tb;
      tb = j % p.n_tb;
    } else {
      tb = j / p.n_vb;
      vb = j % p.n_vb;
    }
  };
  uint16_t* dh16 = static_cast<uint16_t*>(dh);
  uint16_t* dW16 = static_cast<uint16_t*>(dW);
  for (int64_t j = 0; j <= nb; ++j) {
    st.z_ctr = ctr + j * 8;
    if (j >= 1) {
      int64_t tb, vb;
      block_of(j - 1, tb, vb);
      st.g_dz = dzbuf[(j - 1) & 1];
      st.g_t0 = (int)(tb * p.Ct);
      st.g_Ct = (int)std::min(p.Ct, N - tb * p.Ct);
      st.g_v0 = (int)(vb * p.Vb);
      st.g_Vb = (int)std::min(p.Vb, V - vb * p.Vb);
      st.g_acc_dh = vb > 0 || acc_dh;
      st.g_acc_dW = tb > 0 || acc_dW;
      st.n_dw = (int)(lmh::ceil_div(st.g_Vb, lmh::kTileRows) * st.n_ht);
      st.n_dh = (int)(lmh::ceil_div(st.g_Ct, lmh::kTileRows) * st.n_ht);
      if (bf16_out) {
        // each gradient sums its blocks in order (dW over token blocks, dh
        // over vocabulary blocks) in a float32 accumulator; its first block
        // starts from nothing (or the caller's bf16 values when adding) and
        // its last writes the caller's bf16 gradient
        const int64_t t0 = tb * p.Ct, v0 = vb * p.Vb;
        uint16_t* w_out = dW16 + v0 * H;
        float* w_acc = p.vocab_outer ? acc_w : acc_w + v0 * H;
        st.o_dW.src_kind = tb == 0 ? (acc_dW ? lmh::kSrcBf16 : lmh::kSrcNone) : lmh::kSrcF32;
        st.o_dW.src = tb == 0 ? static_cast<const void*>(w_out) : static_cast<const void*>(w_acc);
        st.o_dW.dst_bf16 = tb == p.n_tb - 1;
        st.o_dW.dst = st.o_dW.dst_bf16 ? static_cast<void*>(w_out) : static_cast<void*>(w_acc);
        uint16_t* h_out = dh16 + t0 * H;
        float* h_acc = p.vocab_outer ? acc_h + t0 * H : acc_h;
        st.o_dh.src_kind = vb == 0 ? (acc_dh ? lmh::kSrcBf16 : lmh::kSrcNone) : lmh::kSrcF32;
        st.o_dh.src = vb == 0 ? static_cast<const void*>(h_out) : static_cast<const void*>(h_acc);
        st.o_dh.dst_bf16 = vb == p.n_vb - 1;
        st.o_dh.dst = st.o_dh.dst_bf16 ? static_cast<void*>(h_out) : static_cast<void*>(h_acc);
        st.dh_dead_zero = st.o_dh.dst_bf16 && !acc_dh;
      }
    } else {
      st.g_dz = nullptr;
      st.n_dw = st.n_dh = 0;
    }
    if (j < nb) {
      int64_t tb, vb;
      block_of(j, tb, vb);
      st.z_dz = dzbuf[j & 1];
      st.z_t0 = (int)(tb * p.Ct);
      st.z_Ct = (int)std::min(p.Ct, N - tb * p.Ct);
      st.z_v0 = (int)(vb * p.Vb);
      st.z_Vb = (int)std::min(p.Vb, V - vb * p.Vb);
      st.z_ntt = (int)lmh::ceil_div(st.z_Ct, lmh::kTileRows);
      st.z_nvt = (int)lmh::ceil_div(st.z_Vb, lmh::kTileRows);
    } else {
      st.z_dz = nullptr;
      st.z_ntt = st.z_nvt = 0;
    }
    const hipError_t e = bf16_out ? lmh::launch_bwd_step_bf16(st, s) : lmh::launch_bwd_step(st, s);
    if (e != hipSuccess) return fail(LMH_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

int lmhead_logps_bwd_ex(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                        int64_t N, int64_t H, int64_t V, int64_t chunk_size, float temperature,
                        const float* lse, const float* entropy, const float* g_logp,
                        const float* g_ent, float* dh, float* dW, unsigned flags, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return bwd_impl("bwd", hidden, W, targets, N, H, V, 0, V, chunk_size, temperature, lse, entropy, g_logp, g_ent,
                  dh, dW, flags, false, workspace, workspace_bytes, stream);
}

int lmhead_logps_bwd_bf16(const uint16_t* hidden, const uint16_t* W, const int32_t* targets, int64_t N,
                          int64_t H, int64_t V, int64_t chunk_size, float temperature, const float* lse,
                          const float* entropy, const float* g_logp, const float* g_ent, uint16_t* dh,
                          uint16_t* dW, unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl("bwd_bf16", hidden, W, targets, N, H, V, 0, V, chunk_size, temperature, lse, entropy, g_logp,
                  g_ent, dh, dW, flags, true, workspace, workspace_bytes, stream);
}

int lmhead_logps_bwd_shard(const uint16_t* hidden, const uint16_t* W_shard, const int32_t* targets,
                           int64_t N, int64_t H, int64_t V_shard, int64_t vocab_offset, int64_t V_total,
                           int64_t chunk_size, float temperature, const float* lse, const float* entropy,
                           const float* g_logp, const float* g_ent, float* dh, float* dW_shard,
                           unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl("bwd_shard", hidden, W_shard, targets, N, H, V_shard, vocab_offset, V_total, chunk_size,
                  temperature, lse, entropy, g_logp, g_ent, dh, dW_shard, flags, false, workspace, workspace_bytes,
                  stream);
}

int lmhead_logps_fwd(const uint16_t* hidden, const uint16_t* W, const int32_t* targets, int64_t N,
                     int64_t H, int64_t V, int64_t chunk_size, float* logp, float* entropy,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return lmhead_logps_fwd_temp(hidden, W, targets, N, H, V, chunk_size, 1.0f, logp, entropy, lse,
                               workspace, workspace_bytes, stream);
}

int lmhead_logps_bwd_temp(const uint16_t* hidden, const uint16_t* W, const int32_t* targets,
                          int64_t N, int64_t H, int64_t V, int64_t chunk_size, float temperature,
                          const float* lse, const float* entropy, const float* g_logp,
                          const float* g_ent, float* dh, float* dW, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return lmhead_logps_bwd_ex(hidden, W, targets, N, H, V, chunk_size, temperature, lse, entropy,
                             g_logp, g_ent, dh, dW, 0u, workspace, workspace_bytes, stream);
}

int lmhead_logps_bwd(const uint16_t* hidden, const uint16_t* W, const int32_t* targets, int64_t N,
                     int64_t H, int64_t V, int64_t chunk_size, const float* lse,
                     const float* entropy, const float* g_logp, const float* g_ent, float* dh,
                     float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  return lmhead_logps_bwd_ex(hidden, W, targets, N, H, V, chunk_size, 1.0f, lse, entropy, g_logp,
                             g_ent, dh, dW, 0u, workspace, workspace_bytes, stream);
}

}  // extern "C"
