// abi_client.cpp — a caller of libkdkl.so through its C ABI alone
// (include/kd_fused_kl.h) and HIP's runtime API: no Python, no torch.
//
// Reads a problem from a binary file, runs the forward and backward passes of
// the fused top-K KL loss in float32, and writes the results to a binary file.
// With a third argument "one-pass" it makes the single kd_fused_kl_fwd_bwd
// call instead; the output file has the same layout.
//
//   abi_client <in.bin> <out.bin> [one-pass]
//
// in.bin:  int64 N, d, V, K, chunk; then float H[N*d], float W[V*d],
//          int32 idx[N*K], float logp[N*K], float grad
// out.bin: float loss_sum, loss_tok[N], lse[N], dH[N*d], dW[V*d]
//
// Exit status: 0 on success, 1 on a bad file, 2 on a library or HIP error
// (the status is printed).
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "kd_fused_kl.h"

namespace {

bool read_all(FILE* f, void* p, size_t n) { return std::fread(p, 1, n, f) == n; }

#define HIP_OK(x)                                                                 \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      return 2;                                                                   \
    }                                                                             \
  } while (0)

#define KD_OK_OR_FAIL(x)                                                          \
  do {                                                                            \
    int s_ = (x);                                                                 \
    if (s_ != KD_OK) {                                                            \
      std::fprintf(stderr, "%s failed: %s\n", #x, kd_status_str(s_));             \
      return 2;                                                                   \
    }                                                                             \
  } while (0)

}  // namespace

int main(int argc, char** argv) {
  const bool one_pass = argc == 4 && std::string(argv[3]) == "one-pass";
  if (argc != 3 && !one_pass) {
    std::fprintf(stderr, "usage: %s in.bin out.bin [one-pass]\n", argv[0]);
    return 1;
  }
  FILE* in = std::fopen(argv[1], "rb");
  if (!in) return 1;
  int64_t hdr[5];
  if (!read_all(in, hdr, sizeof(hdr))) return 1;
  const int64_t N = hdr[0], d = hdr[1], V = hdr[2], K = hdr[3], chunk = hdr[4];
  if (N < 0 || d <= 0 || V <= 0 || K <= 0 || chunk <= 0) return 1;
  std::vector<float> H(N * d), W(V * d), logp(N * K), loss_tok(N), lse(N), dH(N * d), dW(V * d);
  std::vector<int32_t> idx(N * K);
  float grad = 0.f, loss = 0.f;
  if (!read_all(in, H.data(), H.size() * 4) || !read_all(in, W.data(), W.size() * 4) ||
      !read_all(in, idx.data(), idx.size() * 4) || !read_all(in, logp.data(), logp.size() * 4) ||
      !read_all(in, &grad, 4))
    return 1;
  std::fclose(in);

  const size_t ws_f = kd_fused_kl_workspace_bytes(KD_PASS_FWD, N, d, V, K, chunk, KD_F32);
  const size_t ws_b = kd_fused_kl_workspace_bytes(KD_PASS_BWD, N, d, V, K, chunk, KD_F32);
  const size_t ws_o = kd_fused_kl_workspace_bytes(KD_PASS_FWD_BWD, N, d, V, K, chunk, KD_F32);
  if (ws_f == 0 || ws_b == 0 || ws_o == 0) {
    std::fprintf(stderr, "sizes rejected\n");
    return 2;
  }
  size_t ws_n = ws_f > ws_b ? ws_f : ws_b;
  if (ws_o > ws_n) ws_n = ws_o;
  void *dH_in, *dW_in, *d_idx, *d_logp, *d_tok, *d_lse, *d_loss, *d_grad, *d_dH, *d_dW, *ws;
  HIP_OK(hipMalloc(&dH_in, H.size() * 4));
  HIP_OK(hipMalloc(&dW_in, W.size() * 4));
  HIP_OK(hipMalloc(&d_idx, idx.size() * 4));
  HIP_OK(hipMalloc(&d_logp, logp.size() * 4));
  HIP_OK(hipMalloc(&d_tok, N * 4 + 4));
  HIP_OK(hipMalloc(&d_lse, N * 4 + 4));
  HIP_OK(hipMalloc(&d_loss, 4));
  HIP_OK(hipMalloc(&d_grad, 4));
  HIP_OK(hipMalloc(&d_dH, dH.size() * 4 + 4));
  HIP_OK(hipMalloc(&d_dW, dW.size() * 4));
  HIP_OK(hipMalloc(&ws, ws_n));
  HIP_OK(hipMemcpy(dH_in, H.data(), H.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dW_in, W.data(), W.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_idx, idx.data(), idx.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_logp, logp.data(), logp.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_grad, &grad, 4, hipMemcpyHostToDevice));

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  if (one_pass) {
    KD_OK_OR_FAIL(kd_fused_kl_fwd_bwd(
        dH_in, dW_in, KD_F32, static_cast<const int32_t*>(d_idx), static_cast<const float*>(d_logp),
        nullptr, KD_REDUCE_SUM, N, d, V, K, chunk, static_cast<const float*>(d_grad),
        static_cast<float*>(d_tok), static_cast<float*>(d_lse), static_cast<float*>(d_loss), d_dH,
        static_cast<float*>(d_dW), 0, ws, ws_o, s));
  } else {
    KD_OK_OR_FAIL(kd_fused_kl_fwd(dH_in, dW_in, KD_F32, static_cast<const int32_t*>(d_idx),
                                  static_cast<const float*>(d_logp), N, d, V, K, chunk,
                                  static_cast<float*>(d_tok), static_cast<float*>(d_lse),
                                  static_cast<float*>(d_loss), ws, ws_f, s));
    KD_OK_OR_FAIL(kd_fused_kl_bwd(dH_in, dW_in, KD_F32, static_cast<const int32_t*>(d_idx),
                                  static_cast<const float*>(d_logp),
                                  static_cast<const float*>(d_lse), N, d, V, K, chunk,
                                  static_cast<const float*>(d_grad), d_dH,
                                  static_cast<float*>(d_dW), 0, ws, ws_b, s));
  }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(&loss, d_loss, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(loss_tok.data(), d_tok, N * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse.data(), d_lse, N * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dH.data(), d_dH, dH.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dW.data(), d_dW, dW.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipStreamDestroy(s));
  for (void* p : {dH_in, dW_in, d_idx, d_logp, d_tok, d_lse, d_loss, d_grad, d_dH, d_dW, ws})
    HIP_OK(hipFree(p));

  FILE* out = std::fopen(argv[2], "wb");
  if (!out) return 1;
  std::fwrite(&loss, 4, 1, out);
  std::fwrite(loss_tok.data(), 4, N, out);
  std::fwrite(lse.data(), 4, N, out);
  std::fwrite(dH.data(), 4, dH.size(), out);
  std::fwrite(dW.data(), 4, dW.size(), out);
  std::fclose(out);
  std::printf("abi_client (%s): N=%lld d=%lld V=%lld K=%lld chunk=%lld loss=%.6f\n",
              one_pass ? "one-pass" : "two-pass", (long long)N, (long long)d, (long long)V,
              (long long)K, (long long)chunk, loss);
  return 0;
}
