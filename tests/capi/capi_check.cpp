// capi_check.cpp -- a caller of the C ABI with no Python and no PyTorch: it
// allocates device memory with hipMalloc, runs lmhead_logps_fwd and
// lmhead_logps_bwd on a stream of its own, and writes the outputs back.
// tests/test_gpu_capi.py runs it as a child process and compares its outputs
// with the fp64 oracle.
//
//   capi_check <dir>
// reads  <dir>/dims.txt ("N H V chunk_size"), hidden.bin (bf16 bits [N,H]),
//        W.bin (bf16 bits [V,H]), targets.bin (int32 [N]), g_logp.bin and
//        g_ent.bin (f32 [N]);
// writes logp.bin, entropy.bin, lse.bin (f32 [N]), dh.bin (f32 [N,H]),
//        dW.bin (f32 [V,H]).
// Exit status 0 on success; on a failing call it prints the library's
// message and exits with 1.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../include/lmhead_logps.h"

namespace {

template <class T>
std::vector<T> read_file(const std::string& path, size_t count) {
  std::vector<T> v(count);
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f || std::fread(v.data(), sizeof(T), count, f) != count) {
    std::fprintf(stderr, "cannot read %zu values from %s\n", count, path.c_str());
    std::exit(1);
  }
  std::fclose(f);
  return v;
}

template <class T>
void write_file(const std::string& path, const std::vector<T>& v) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) {
    std::fprintf(stderr, "cannot write %s\n", path.c_str());
    std::exit(1);
  }
  std::fclose(f);
}

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

void lmh_check(int rc, const char* what) {
  if (rc != LMH_OK) {
    std::fprintf(stderr, "%s: status %d: %s\n", what, rc, lmhead_logps_last_error());
    std::exit(1);
  }
}

template <class T>
T* to_device(const std::vector<T>& v) {
  T* p = nullptr;
  hip_check(hipMalloc(&p, v.size() * sizeof(T) + 16), "hipMalloc");
  hip_check(hipMemcpy(p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy H2D");
  return p;
}

template <class T>
T* device_array(size_t count) {
  T* p = nullptr;
  hip_check(hipMalloc(&p, count * sizeof(T) + 16), "hipMalloc");
  return p;
}

template <class T>
std::vector<T> to_host(const T* p, size_t count) {
  std::vector<T> v(count);
  hip_check(hipMemcpy(v.data(), p, count * sizeof(T), hipMemcpyDeviceToHost), "hipMemcpy D2H");
  return v;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s <dir>\n", argv[0]);
    return 2;
  }
  const std::string dir = argv[1];
  long long N = 0, H = 0, V = 0, C = 0;
  {
    FILE* f = std::fopen((dir + "/dims.txt").c_str(), "r");
    if (!f || std::fscanf(f, "%lld %lld %lld %lld", &N, &H, &V, &C) != 4) {
      std::fprintf(stderr, "cannot read dims.txt\n");
      return 1;
    }
    std::fclose(f);
  }
  std::printf("capi_check: %s, N=%lld H=%lld V=%lld chunk=%lld\n", lmhead_logps_version(), N, H, V, C);
  const auto hidden = read_file<uint16_t>(dir + "/hidden.bin", (size_t)(N * H));
  const auto W = read_file<uint16_t>(dir + "/W.bin", (size_t)(V * H));
  const auto targets = read_file<int32_t>(dir + "/targets.bin", (size_t)N);
  const auto g_logp = read_file<float>(dir + "/g_logp.bin", (size_t)N);
  const auto g_ent = read_file<float>(dir + "/g_ent.bin", (size_t)N);

  hipStream_t stream = nullptr;
  hip_check(hipStreamCreate(&stream), "hipStreamCreate");
  uint16_t* d_hidden = to_device(hidden);
  uint16_t* d_W = to_device(W);
  int32_t* d_t = to_device(targets);
  float* d_gl = to_device(g_logp);
  float* d_ge = to_device(g_ent);
  float* d_logp = device_array<float>((size_t)N);
  float* d_ent = device_array<float>((size_t)N);
  float* d_lse = device_array<float>((size_t)N);
  float* d_dh = device_array<float>((size_t)(N * H));
  float* d_dW = device_array<float>((size_t)(V * H));
  size_t ws_bytes = 0;
  lmh_check(lmhead_logps_workspace_bytes(N, H, V, C, LMH_WS_BWD, &ws_bytes), "lmhead_logps_workspace_bytes");
  void* ws = nullptr;
  hip_check(hipMalloc(&ws, ws_bytes + 16), "hipMalloc workspace");

  lmh_check(lmhead_logps_fwd(d_hidden, d_W, d_t, N, H, V, C, d_logp, d_ent, d_lse, ws, ws_bytes, stream),
            "lmhead_logps_fwd");
  lmh_check(lmhead_logps_bwd(d_hidden, d_W, d_t, N, H, V, C, d_lse, d_ent, d_gl, d_ge, d_dh, d_dW, ws, ws_bytes,
                             stream),
            "lmhead_logps_bwd");
  hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize");

  write_file(dir + "/logp.bin", to_host(d_logp, (size_t)N));
  write_file(dir + "/entropy.bin", to_host(d_ent, (size_t)N));
  write_file(dir + "/lse.bin", to_host(d_lse, (size_t)N));
  write_file(dir + "/dh.bin", to_host(d_dh, (size_t)(N * H)));
  write_file(dir + "/dW.bin", to_host(d_dW, (size_t)(V * H)));
  for (void* p : {(void*)d_hidden, (void*)d_W, (void*)d_t, (void*)d_gl, (void*)d_ge, (void*)d_logp, (void*)d_ent,
                  (void*)d_lse, (void*)d_dh, (void*)d_dW, ws})
    hip_check(hipFree(p), "hipFree");
  hip_check(hipStreamDestroy(stream), "hipStreamDestroy");
  std::printf("capi_check: ok\n");
  return 0;
}
