// Decode latency through the C ABI from native code: times back-to-back
// rmsnorm_fwd calls (bf16 x, residual, weight and output) on one stream with
// HIP events, against rn_launch_empty launched the same way, with no Python
// in the loop.  Prints one JSON object.
//
//   rn_decode_latency ROWS HIDDEN PLUS_ONE [CALLS]
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <chrono>

#include "rmsnorm_rows.h"

namespace {

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

// Host-only cost of the selector and argument checks (no HIP call).
double query_ns(int64_t rows, int64_t hidden, uint32_t flags, int calls) {
  rn_launch_config cfg;
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < calls; ++i) rmsnorm_query_config(rows, hidden, flags, 1, 256, &cfg);
  const auto t1 = std::chrono::steady_clock::now();
  return std::chrono::duration<double, std::nano>(t1 - t0).count() / calls;
}

// Average device time per call of `call` over `calls` back-to-back calls (HIP
// events), and in *host_us the host time to enqueue them.
template <class F>
double us_per_call(F&& call, int calls, hipStream_t s, double* host_us) {
  for (int i = 0; i < 100; ++i)
    if (!call()) return -1.0;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "hipEventCreate") || !ok(hipEventCreate(&b), "hipEventCreate")) return -1.0;
  if (!ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return -1.0;
  ok(hipEventRecord(a, s), "hipEventRecord");
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < calls; ++i)
    if (!call()) return -1.0;
  const auto t1 = std::chrono::steady_clock::now();
  *host_us = std::chrono::duration<double, std::micro>(t1 - t0).count() / calls;
  ok(hipEventRecord(b, s), "hipEventRecord");
  if (!ok(hipEventSynchronize(b), "hipEventSynchronize")) return -1.0;
  float ms = 0.f;
  ok(hipEventElapsedTime(&ms, a, b), "hipEventElapsedTime");
  hipEventDestroy(a);
  hipEventDestroy(b);
  return 1000.0 * ms / calls;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 4) {
    fprintf(stderr, "usage: %s ROWS HIDDEN PLUS_ONE [CALLS]\n", argv[0]);
    return 2;
  }
  const int64_t rows = atoll(argv[1]);
  const int64_t hidden = atoll(argv[2]);
  const int plus_one = atoi(argv[3]);
  const int calls = argc > 4 ? atoi(argv[4]) : 2000;
  if (rows < 1 || hidden < 1 || calls < 1 || rows * hidden > (int64_t)1 << 28) {
    fprintf(stderr, "bad sizes\n");
    return 2;
  }
  const size_t n = static_cast<size_t>(rows * hidden);
  void *x, *res, *w, *out, *res_out;
  if (!ok(hipMalloc(&x, 2 * n), "hipMalloc") || !ok(hipMalloc(&res, 2 * n), "hipMalloc") ||
      !ok(hipMalloc(&w, 2 * hidden), "hipMalloc") || !ok(hipMalloc(&out, 2 * n), "hipMalloc") ||
      !ok(hipMalloc(&res_out, 2 * n), "hipMalloc"))
    return 1;
  // bf16 1.0 for x and the weight, 0.5 for the residual: finite, nonzero rows
  if (!ok(hipMemsetD16(x, 0x3F80, n), "hipMemsetD16") || !ok(hipMemsetD16(res, 0x3F00, n), "hipMemsetD16") ||
      !ok(hipMemsetD16(w, 0x3F80, hidden), "hipMemsetD16") || !ok(hipDeviceSynchronize(), "hipDeviceSynchronize"))
    return 1;
  hipStream_t s;
  if (!ok(hipStreamCreate(&s), "hipStreamCreate")) return 1;
  const uint32_t flags = RN_MAKE_FLAGS(RN_DTYPE_BF16, RN_DTYPE_BF16, RN_DTYPE_BF16, RN_DTYPE_BF16, plus_one != 0);
  rn_status last = RN_OK;
  auto norm = [&]() {
    last = rmsnorm_fwd(x, res, w, out, res_out, nullptr, rows, hidden, 1e-6f, flags, s);
    return last == RN_OK;
  };
  auto empty = [&]() {
    last = rn_launch_empty(s);
    return last == RN_OK;
  };
  double h_norm = 0, h_empty = 0;
  const double t_norm = us_per_call(norm, calls, s, &h_norm);
  const double t_empty = us_per_call(empty, calls, s, &h_empty);
  const double q_ns = query_ns(rows, hidden, flags, calls);
  if (t_norm < 0 || t_empty < 0) {
    fprintf(stderr, "call failed: %s %s\n", rn_status_string(last), rn_last_error());
    return 1;
  }
  printf("{\"rows\": %lld, \"hidden\": %lld, \"plus_one\": %d, \"calls\": %d, \"us_per_call\": %.3f, "
         "\"empty_us_per_call\": %.3f, \"ratio\": %.3f, \"host_enqueue_us\": %.3f, "
         "\"empty_host_enqueue_us\": %.3f, \"select_and_check_ns\": %.1f}\n",
         (long long)rows, (long long)hidden, plus_one, calls, t_norm, t_empty, t_norm / t_empty, h_norm, h_empty, q_ns);
  hipStreamDestroy(s);
  hipFree(x);
  hipFree(res);
  hipFree(w);
  hipFree(out);
  hipFree(res_out);
  return 0;
}
