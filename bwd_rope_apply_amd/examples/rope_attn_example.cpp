// A plain C++ caller of the C ABI (include/rope_attn.h), with no Python or
// torch: reads one problem from a binary file, runs the forward and the
// backward on the default HIP device, writes the outputs.
//
//   rope_attn_example IN OUT
//
// IN:  int32 B, H, N, D, causal; float64 base; then Q, K, V, dO as bfloat16
//      bit patterns (uint16, [B][H][N][D] each) and alpha (float32 [D/2]).
// OUT: O [B][H][N][D], LSE [B][H][N], dQ, dK, dV [B][H][N][D], dalpha [D/2],
//      all float32, in that order.
// Exit status 0 on success; otherwise a message on stderr.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "rope_attn.h"

namespace {

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

template <class T>
bool read_n(std::FILE* f, T* p, size_t n) { return std::fread(p, sizeof(T), n, f) == n; }

template <class T>
bool write_n(std::FILE* f, const T* p, size_t n) { return std::fwrite(p, sizeof(T), n, f) == n; }

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  std::FILE* in = std::fopen(argv[1], "rb");
  if (!in) {
    std::fprintf(stderr, "cannot open %s\n", argv[1]);
    return 2;
  }
  int32_t hdr[5];
  double base = 0.0;
  if (!read_n(in, hdr, 5) || !read_n(in, &base, 1)) {
    std::fprintf(stderr, "short header\n");
    return 2;
  }
  const int B = hdr[0], H = hdr[1], N = hdr[2], D = hdr[3], causal = hdr[4];
  if (B < 1 || H < 1 || N < 1 || (D != 64 && D != 128)) {
    std::fprintf(stderr, "bad shape\n");
    return 2;
  }
  const size_t n = (size_t)B * H * N * D, nr = (size_t)B * H * N;
  std::vector<uint16_t> host_in[4];
  for (auto& h : host_in) {
    h.resize(n);
    if (!read_n(in, h.data(), n)) {
      std::fprintf(stderr, "short tensor\n");
      return 2;
    }
  }
  std::vector<float> alpha(D / 2);
  if (!read_n(in, alpha.data(), alpha.size())) {
    std::fprintf(stderr, "short alpha\n");
    return 2;
  }
  std::fclose(in);

  // device buffers: inputs, outputs, one workspace for both passes
  void* dev_in[4];
  float *o, *lse, *dq, *dk, *dv, *da, *a;
  void* ws;
  const size_t ws_bytes = rope_attn_bwd_workspace_bytes(B, H, N, D, ROPE_ATTN_BF16, causal);
  if (ws_bytes == 0) {
    std::fprintf(stderr, "rejected shape\n");
    return 2;
  }
  bool ok = true;
  for (int i = 0; i < 4 && ok; ++i) ok = hip_ok(hipMalloc(&dev_in[i], n * 2), "hipMalloc");
  ok = ok && hip_ok(hipMalloc(&o, n * 4), "hipMalloc") && hip_ok(hipMalloc(&lse, nr * 4), "hipMalloc") &&
       hip_ok(hipMalloc(&dq, n * 4), "hipMalloc") && hip_ok(hipMalloc(&dk, n * 4), "hipMalloc") &&
       hip_ok(hipMalloc(&dv, n * 4), "hipMalloc") && hip_ok(hipMalloc(&da, D / 2 * 4), "hipMalloc") &&
       hip_ok(hipMalloc(&a, D / 2 * 4), "hipMalloc") && hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc");
  for (int i = 0; i < 4 && ok; ++i)
    ok = hip_ok(hipMemcpy(dev_in[i], host_in[i].data(), n * 2, hipMemcpyHostToDevice), "hipMemcpy");
  ok = ok && hip_ok(hipMemcpy(a, alpha.data(), D / 2 * 4, hipMemcpyHostToDevice), "hipMemcpy");
  if (!ok) return 1;

  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
  int st = rope_attn_fwd(dev_in[0], dev_in[1], dev_in[2], o, lse, B, H, N, D, ROPE_ATTN_BF16, base, a,
                         causal, ws, ws_bytes, stream);
  if (st != ROPE_ATTN_OK) {
    std::fprintf(stderr, "rope_attn_fwd: %s\n", rope_attn_status_string(st));
    return 1;
  }
  // the backward reuses the forward's prepared planes in the same workspace
  const unsigned bwd_stages = (ROPE_ATTN_STAGE_ALL & ~ROPE_ATTN_STAGE_PREP) | ROPE_ATTN_STAGE_PREP_GRAD;
  st = rope_attn_bwd_stages(bwd_stages, dev_in[0], dev_in[1], dev_in[2], o, dev_in[3], lse, dq, dk, dv, da,
                            B, H, N, D, ROPE_ATTN_BF16, base, a, causal, ws, ws_bytes, stream);
  if (st != ROPE_ATTN_OK) {
    std::fprintf(stderr, "rope_attn_bwd_stages: %s\n", rope_attn_status_string(st));
    return 1;
  }
  if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;

  std::vector<float> host(n);
  std::FILE* out = std::fopen(argv[2], "wb");
  if (!out) {
    std::fprintf(stderr, "cannot open %s\n", argv[2]);
    return 2;
  }
  const struct { float* p; size_t count; } outs[] = {{o, n}, {lse, nr}, {dq, n}, {dk, n}, {dv, n}, {da, (size_t)D / 2}};
  for (const auto& t : outs) {
    if (!hip_ok(hipMemcpy(host.data(), t.p, t.count * 4, hipMemcpyDeviceToHost), "hipMemcpy") ||
        !write_n(out, host.data(), t.count)) {
      std::fclose(out);
      return 1;
    }
  }
  std::fclose(out);
  hipStreamDestroy(stream);
  for (void* p : dev_in) hipFree(p);
  for (void* p : {(void*)o, (void*)lse, (void*)dq, (void*)dk, (void*)dv, (void*)da, (void*)a, ws}) hipFree(p);
  return 0;
}
