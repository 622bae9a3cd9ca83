// C ABI entry points: argument checks, selector, kernel lookup, launch.
//
// Order inside every entry point: flags and sizes, then pointers and
// alignment -- all on the host, before any HIP call -- and only then the
// per-device compute-unit count (cached) and the asynchronous launch.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <atomic>

#include "rn_internal.h"

namespace rn {
const char* last_error();

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];  // 0 = not queried yet

rn_status device_cus(int* num_cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RN_ERR_HIP, "device index %d out of range", dev);
  int n = g_num_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n < 1)
      return fail(RN_ERR_HIP, "hipDeviceGetAttribute(compute units): %s", hipGetErrorString(e));
    g_num_cus[dev].store(n, std::memory_order_relaxed);
  }
  *num_cus = n;
  return RN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Storage bits of an output element.
int out_bits(int dt) { return dt == kBF16 ? 16 : dt == kF32 ? 32 : dt == kFP8 ? 8 : 4; }

const void* pick_row_kernel(const RowKey& k) {
  const void* (*const pickers[])(const RowKey&) = {
      pick_row_kernel_bf16_bf16,    pick_row_kernel_bf16_f32,     pick_row_kernel_bf16_fp8_row,
      pick_row_kernel_bf16_fp8_g128, pick_row_kernel_bf16_fp8_mx, pick_row_kernel_bf16_fp4_mx,
      pick_row_kernel_bf16_fp4_nv,  pick_row_kernel_f32_bf16,     pick_row_kernel_f32_f32,
      pick_row_kernel_f32_fp8_row,  pick_row_kernel_f32_fp8_g128, pick_row_kernel_f32_fp8_mx,
      pick_row_kernel_f32_fp4_mx,   pick_row_kernel_f32_fp4_nv};
  for (auto p : pickers) {
    const void* f = p(k);
    if (f) return f;
  }
  return nullptr;
}

// Pointers that come with a quantized output: out_scale (required), out_amax
// (optional) and the NVFP4 tensor scale (required for RN_SCALE_NV16, else NULL).
rn_status check_quant_ptrs(int out, int qs, const void* out_scale, const float* out_amax,
                           const float* tensor_scale, bool rows_nonzero) {
  const bool quant = out == kFP8 || out == kFP4;
  if (!quant && (out_scale != nullptr || out_amax != nullptr))
    return fail(RN_ERR_INVALID_ARG, "out_scale / out_amax are only for fp8 / fp4 output");
  if ((qs == kQNv16) != (tensor_scale != nullptr))
    return fail(RN_ERR_INVALID_ARG, qs == kQNv16 ? "NVFP4 scales (RN_SCALE_NV16) need tensor_scale"
                                                   : "tensor_scale is only for NVFP4 scales (RN_SCALE_NV16)");
  if (!rows_nonzero) return RN_OK;
  if (quant && out_scale == nullptr) return fail(RN_ERR_INVALID_ARG, "quantized output needs out_scale");
  const bool byte_scales = qs == kQMx32 || qs == kQNv16;
  if ((out_scale && !byte_scales && !aligned(out_scale, 4)) || (out_amax && !aligned(out_amax, 4)) ||
      (tensor_scale && !aligned(tensor_scale, 4)))
    return fail(RN_ERR_MISALIGNED, "float32 scales, out_amax and tensor_scale must be 4-byte aligned");
  return RN_OK;
}

rn_status launch(const void* fn, int64_t grid, int block, void* args, void* stream) {
  void* argv[] = {args};
  hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(block),
                                 args ? argv : nullptr, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RN_ERR_HIP, "hipLaunchKernel: %s", hipGetErrorString(e));
  return RN_OK;
}

// Partial-input form (rmsnorm_fwd_partials*): the sizes and flags checks of
// the rows kernel, then those of the partials (count, row length).
rn_status check_parts_key(int32_t num_parts, int64_t hidden, RowKey* key) {
  if (num_parts < 1 || num_parts > kMaxParts)
    return fail(RN_ERR_INVALID_ARG, "num_partials must be in 1..%d (got %d)", kMaxParts, num_parts);
  const int64_t vec = key->x == kBF16 ? 8 : 4;
  const int64_t cap = static_cast<int64_t>(64) * kMaxWavesPerRow * kMaxPartsVecsPerLane * vec;
  if (num_parts > 1 && hidden > cap)
    return fail(RN_ERR_UNSUPPORTED, "hidden (%lld) above the largest row of the partial-input kernels (%lld)",
                (long long)hidden, (long long)cap);
  key->kp = num_parts == 1 ? 1 : parts_slots(num_parts);
  return RN_OK;
}

// parts_form: x is the sum of parts[0 .. num_parts) (x itself is unused);
// otherwise the single-input form.
rn_status rows_entry(bool parts_form, const void* x, const void* const* parts, int32_t num_parts,
                     const void* residual, const void* weight, void* out, void* residual_out, void* out_scale,
                     float* out_amax, const float* tensor_scale, int64_t rows, int64_t hidden, float eps,
                     uint32_t flags, const rn_launch_config* explicit_cfg, void* stream) {
  clear_error();
  RowKey key;
  rn_status st = check_row_shape(rows, hidden, flags, residual != nullptr, &key);
  if (st != RN_OK) return st;
  if (parts_form) {
    st = check_parts_key(num_parts, hidden, &key);
    if (st != RN_OK) return st;
  }
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return fail(RN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  st = check_quant_ptrs(key.out, key.qs, out_scale, out_amax, tensor_scale, false);
  if (st != RN_OK) return st;
  if (rows == 0) return RN_OK;
  if (parts_form) {
    if (parts == nullptr) return fail(RN_ERR_INVALID_ARG, "partials must not be NULL");
    for (int32_t k = 0; k < num_parts; ++k) {
      if (parts[k] == nullptr) return fail(RN_ERR_INVALID_ARG, "partials[%d] is NULL", k);
      if (!aligned(parts[k], 16))
        return fail(RN_ERR_MISALIGNED, "partials[%d] = %p is not 16-byte aligned", k, parts[k]);
      if (residual_out != nullptr && parts[k] == residual_out)
        return fail(RN_ERR_INVALID_ARG, "residual_out must not be one of the partials");
    }
    x = parts[0];
  }
  if (x == nullptr || weight == nullptr || out == nullptr)
    return fail(RN_ERR_INVALID_ARG, "x, weight and out must not be NULL");
  if ((residual == nullptr) != (residual_out == nullptr))
    return fail(RN_ERR_INVALID_ARG, "residual and residual_out must both be given or both be NULL");
  if (residual_out != nullptr && residual_out == out)
    return fail(RN_ERR_INVALID_ARG, "out and residual_out must be different buffers");
  // In place (out over x or over a partial) only with equal element widths:
  // otherwise row r of out covers other rows of the input, which other
  // workgroups may still be reading.
  if (out_bits(key.out) != (key.x == kBF16 ? 16 : 32)) {
    bool aliased = !parts_form && out == x;
    for (int32_t k = 0; parts_form && k < num_parts; ++k) aliased |= out == parts[k];
    if (aliased)
      return fail(RN_ERR_INVALID_ARG, "out may equal x (or a partial) only when both have the same element width");
  }
  const void* ptrs16[] = {x, residual, weight, out, residual_out};
  for (const void* p : ptrs16)
    if (p != nullptr && !aligned(p, 16)) return fail(RN_ERR_MISALIGNED, "tensor pointer %p is not 16-byte aligned", p);
  st = check_quant_ptrs(key.out, key.qs, out_scale, out_amax, tensor_scale, true);
  if (st != RN_OK) return st;

  rn_launch_config cfg;
  if (explicit_cfg != nullptr) {
    st = check_row_config(rows, hidden, key, explicit_cfg, &cfg);
  } else {
    int cus = 0;
    st = device_cus(&cus);
    if (st != RN_OK) return st;
    st = select_row_config(rows, hidden, key, cus, &cfg);
  }
  if (st != RN_OK) return st;
  key.nv = cfg.vecs_per_lane;
  const void* fn = pick_row_kernel(key);
  if (fn == nullptr) return fail(RN_ERR_UNSUPPORTED, "no kernel built for this dtype combination");

  RowArgs a;
  a.x = x;
  a.res = residual;
  a.w = weight;
  a.out = out;
  a.res_out = residual_out;
  a.scale = out_scale;
  a.amax = out_amax;
  a.tscale = tensor_scale;
  a.rows = rows;
  a.hidden = static_cast<int32_t>(hidden);
  a.eps = eps;
  for (int k = 0; k < kMaxParts; ++k) a.parts[k] = parts_form && k < num_parts ? parts[k] : nullptr;
  a.num_parts = parts_form ? num_parts : 1;
  return launch(fn, cfg.grid, cfg.block_threads, &a, stream);
}

rn_status heads_entry(const void* q, const void* k, const void* q_weight, const void* k_weight,
                      void* q_out, void* k_out, int64_t tokens, int32_t num_q_heads,
                      int32_t num_k_heads, int32_t head_dim, int64_t q_token_stride,
                      int64_t k_token_stride, float eps, uint32_t flags,
                      const rn_launch_config* explicit_cfg, void* stream) {
  clear_error();
  HeadKey key;
  rn_status st = check_head_shape(tokens, num_q_heads, num_k_heads, head_dim, flags, &key);
  if (st != RN_OK) return st;
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return fail(RN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const int64_t qrow = (int64_t)num_q_heads * head_dim;
  const int64_t krow = (int64_t)num_k_heads * head_dim;
  if (q_token_stride == 0) q_token_stride = qrow;
  if (k_token_stride == 0) k_token_stride = krow;
  if (q_token_stride < qrow || q_token_stride < 0)
    return fail(RN_ERR_INVALID_ARG, "q_token_stride (%lld) < num_q_heads * head_dim", (long long)q_token_stride);
  if (num_k_heads > 0 && k_token_stride < krow)
    return fail(RN_ERR_INVALID_ARG, "k_token_stride (%lld) < num_k_heads * head_dim", (long long)k_token_stride);
  if (tokens == 0) return RN_OK;
  if (q == nullptr || q_weight == nullptr || q_out == nullptr)
    return fail(RN_ERR_INVALID_ARG, "q, q_weight and q_out must not be NULL");
  const bool has_k = num_k_heads > 0;
  if (has_k != (k != nullptr) || has_k != (k_weight != nullptr) || has_k != (k_out != nullptr))
    return fail(RN_ERR_INVALID_ARG, "k, k_weight and k_out must be given iff num_k_heads > 0");
  const void* ptrs16[] = {q, k, q_weight, k_weight, q_out, k_out};
  for (const void* p : ptrs16)
    if (p != nullptr && !aligned(p, 16)) return fail(RN_ERR_MISALIGNED, "tensor pointer %p is not 16-byte aligned", p);
  const int eb = key.t == kBF16 ? 2 : 4;
  if ((q_token_stride * eb) % 16 != 0 || (has_k && (k_token_stride * eb) % 16 != 0))
    return fail(RN_ERR_MISALIGNED, "token strides must be multiples of 16 bytes");

  rn_launch_config cfg;
  if (explicit_cfg != nullptr) {
    st = check_head_config(tokens, num_q_heads, num_k_heads, key, explicit_cfg, &cfg);
  } else {
    int cus = 0;
    st = device_cus(&cus);
    if (st != RN_OK) return st;
    st = select_head_config(tokens, num_q_heads, num_k_heads, key, cus, &cfg);
  }
  if (st != RN_OK) return st;
  key.rpl = cfg.rows_per_lane;
  const void* fn = pick_head_kernel(key);
  if (fn == nullptr) return fail(RN_ERR_UNSUPPORTED, "no qknorm kernel built for this combination");

  HeadArgs a;
  a.q = q;
  a.k = k;
  a.qw = q_weight;
  a.kw = k_weight;
  a.q_out = q_out;
  a.k_out = k_out;
  a.q_stride = q_token_stride;
  a.k_stride = k_token_stride;
  a.num_q_heads = num_q_heads;
  a.num_heads = num_q_heads + num_k_heads;
  a.total_rows = static_cast<int32_t>(tokens * (num_q_heads + num_k_heads));
  a.eps = eps;
  return launch(fn, cfg.grid, cfg.block_threads, &a, stream);
}

rn_status act_entry(const void* x, void* out, void* out_scale, float* out_amax, const float* tensor_scale,
                    int64_t rows, int64_t d, uint32_t flags, const rn_launch_config* explicit_cfg, void* stream) {
  clear_error();
  ActKey key;
  rn_status st = check_act_shape(rows, d, flags, &key);
  if (st != RN_OK) return st;
  st = check_quant_ptrs(key.out, key.qs, out_scale, out_amax, tensor_scale, false);
  if (st != RN_OK) return st;
  if (rows == 0) return RN_OK;
  if (x == nullptr || out == nullptr) return fail(RN_ERR_INVALID_ARG, "x and out must not be NULL");
  if (!aligned(x, 16) || !aligned(out, 16)) return fail(RN_ERR_MISALIGNED, "x and out must be 16-byte aligned");
  st = check_quant_ptrs(key.out, key.qs, out_scale, out_amax, tensor_scale, true);
  if (st != RN_OK) return st;

  rn_launch_config cfg;
  if (explicit_cfg != nullptr) {
    RowKey rk{};
    rk.x = key.x;
    rk.kp = 1;
    st = check_row_config(rows, d, rk, explicit_cfg, &cfg);
  } else {
    int cus = 0;
    st = device_cus(&cus);
    if (st != RN_OK) return st;
    st = select_act_config(rows, d, key, cus, &cfg);
  }
  if (st != RN_OK) return st;
  key.nv = cfg.vecs_per_lane;
  const void* fn = pick_act_kernel(key);
  if (fn == nullptr) return fail(RN_ERR_UNSUPPORTED, "no silu_mul kernel built for this combination");
  ActArgs a;
  a.x = x;
  a.out = out;
  a.scale = out_scale;
  a.amax = out_amax;
  a.tscale = tensor_scale;
  a.rows = rows;
  a.d = static_cast<int32_t>(d);
  return launch(fn, cfg.grid, cfg.block_threads, &a, stream);
}

}  // namespace
}  // namespace rn

using namespace rn;

extern "C" {

rn_status rmsnorm_fwd(const void* x, const void* residual, const void* weight, void* out,
                      void* residual_out, void* out_scale, int64_t rows, int64_t hidden, float eps,
                      uint32_t flags, void* stream) {
  return rows_entry(false, x, nullptr, 0, residual, weight, out, residual_out, out_scale, nullptr, nullptr, rows,
                    hidden, eps, flags, nullptr, stream);
}

rn_status rmsnorm_fwd_ex(const void* x, const void* residual, const void* weight, void* out,
                         void* residual_out, void* out_scale, float* out_amax, const float* tensor_scale,
                         int64_t rows, int64_t hidden, float eps, uint32_t flags, void* stream) {
  return rows_entry(false, x, nullptr, 0, residual, weight, out, residual_out, out_scale, out_amax, tensor_scale,
                    rows, hidden, eps, flags, nullptr, stream);
}

rn_status rmsnorm_fwd_call(const rn_rmsnorm_call* c) {
  if (c == nullptr) {
    clear_error();
    return fail(RN_ERR_INVALID_ARG, "call record is NULL");
  }
  return rows_entry(false, c->x, nullptr, 0, c->residual, c->weight, c->out, c->residual_out, c->out_scale,
                    c->out_amax, c->tensor_scale, c->rows, c->hidden, c->eps, c->flags, nullptr, c->stream);
}

rn_status rmsnorm_fwd_config(const void* x, const void* residual, const void* weight, void* out,
                             void* residual_out, void* out_scale, float* out_amax,
                             const float* tensor_scale, int64_t rows, int64_t hidden, float eps,
                             uint32_t flags, const rn_launch_config* cfg, void* stream) {
  if (cfg == nullptr) {
    clear_error();
    return fail(RN_ERR_INVALID_ARG, "launch config is NULL");
  }
  return rows_entry(false, x, nullptr, 0, residual, weight, out, residual_out, out_scale, out_amax, tensor_scale,
                    rows, hidden, eps, flags, cfg, stream);
}

rn_status rmsnorm_fwd_partials(const void* const* partials, int32_t num_partials, const void* residual,
                               const void* weight, void* out, void* residual_out, void* out_scale,
                               float* out_amax, const float* tensor_scale, int64_t rows, int64_t hidden, float eps,
                               uint32_t flags, void* stream) {
  return rows_entry(true, nullptr, partials, num_partials, residual, weight, out, residual_out, out_scale, out_amax,
                    tensor_scale, rows, hidden, eps, flags, nullptr, stream);
}

rn_status rmsnorm_fwd_partials_config(const void* const* partials, int32_t num_partials, const void* residual,
                                      const void* weight, void* out, void* residual_out, void* out_scale,
                                      float* out_amax, const float* tensor_scale, int64_t rows, int64_t hidden,
                                      float eps, uint32_t flags, const rn_launch_config* cfg, void* stream) {
  if (cfg == nullptr) {
    clear_error();
    return fail(RN_ERR_INVALID_ARG, "launch config is NULL");
  }
  return rows_entry(true, nullptr, partials, num_partials, residual, weight, out, residual_out, out_scale, out_amax,
                    tensor_scale, rows, hidden, eps, flags, cfg, stream);
}

rn_status qknorm_fwd(const void* q, const void* k, const void* q_weight, const void* k_weight,
                     void* q_out, void* k_out, int64_t tokens, int32_t num_q_heads,
                     int32_t num_k_heads, int32_t head_dim, int64_t q_token_stride,
                     int64_t k_token_stride, float eps, uint32_t flags, void* stream) {
  return heads_entry(q, k, q_weight, k_weight, q_out, k_out, tokens, num_q_heads, num_k_heads, head_dim,
                     q_token_stride, k_token_stride, eps, flags, nullptr, stream);
}

rn_status qknorm_fwd_config(const void* q, const void* k, const void* q_weight, const void* k_weight,
                            void* q_out, void* k_out, int64_t tokens, int32_t num_q_heads,
                            int32_t num_k_heads, int32_t head_dim, int64_t q_token_stride,
                            int64_t k_token_stride, float eps, uint32_t flags,
                            const rn_launch_config* cfg, void* stream) {
  if (cfg == nullptr) {
    clear_error();
    return fail(RN_ERR_INVALID_ARG, "launch config is NULL");
  }
  return heads_entry(q, k, q_weight, k_weight, q_out, k_out, tokens, num_q_heads, num_k_heads, head_dim,
                     q_token_stride, k_token_stride, eps, flags, cfg, stream);
}

rn_status rmsnorm_query_config(int64_t rows, int64_t hidden, uint32_t flags, int32_t has_residual,
                               int32_t num_cus, rn_launch_config* cfg) {
  clear_error();
  if (cfg == nullptr) return fail(RN_ERR_INVALID_ARG, "cfg is NULL");
  RowKey key;
  rn_status st = check_row_shape(rows, hidden, flags, has_residual != 0, &key);
  if (st != RN_OK) return st;
  int cus = num_cus;
  if (cus <= 0) {
    st = device_cus(&cus);
    if (st != RN_OK) return st;
  }
  return select_row_config(rows > 0 ? rows : 1, hidden, key, cus, cfg);
}

rn_status rmsnorm_partials_query_config(int64_t rows, int64_t hidden, int32_t num_partials, uint32_t flags,
                                        int32_t has_residual, int32_t num_cus, rn_launch_config* cfg) {
  clear_error();
  if (cfg == nullptr) return fail(RN_ERR_INVALID_ARG, "cfg is NULL");
  RowKey key;
  rn_status st = check_row_shape(rows, hidden, flags, has_residual != 0, &key);
  if (st != RN_OK) return st;
  st = check_parts_key(num_partials, hidden, &key);
  if (st != RN_OK) return st;
  int cus = num_cus;
  if (cus <= 0) {
    st = device_cus(&cus);
    if (st != RN_OK) return st;
  }
  return select_row_config(rows > 0 ? rows : 1, hidden, key, cus, cfg);
}

rn_status qknorm_query_config(int64_t tokens, int32_t num_q_heads, int32_t num_k_heads,
                              int32_t head_dim, uint32_t flags, int32_t num_cus,
                              rn_launch_config* cfg) {
  clear_error();
  if (cfg == nullptr) return fail(RN_ERR_INVALID_ARG, "cfg is NULL");
  HeadKey key;
  rn_status st = check_head_shape(tokens, num_q_heads, num_k_heads, head_dim, flags, &key);
  if (st != RN_OK) return st;
  int cus = num_cus;
  if (cus <= 0) {
    st = device_cus(&cus);
    if (st != RN_OK) return st;
  }
  return select_head_config(tokens > 0 ? tokens : 1, num_q_heads, num_k_heads, key, cus, cfg);
}

rn_status silu_mul_fwd(const void* x, void* out, void* out_scale, float* out_amax, const float* tensor_scale,
                       int64_t rows, int64_t d, uint32_t flags, void* stream) {
  return act_entry(x, out, out_scale, out_amax, tensor_scale, rows, d, flags, nullptr, stream);
}

rn_status silu_mul_fwd_config(const void* x, void* out, void* out_scale, float* out_amax,
                              const float* tensor_scale, int64_t rows, int64_t d, uint32_t flags,
                              const rn_launch_config* cfg, void* stream) {
  if (cfg == nullptr) {
    clear_error();
    return fail(RN_ERR_INVALID_ARG, "launch config is NULL");
  }
  return act_entry(x, out, out_scale, out_amax, tensor_scale, rows, d, flags, cfg, stream);
}

rn_status silu_mul_query_config(int64_t rows, int64_t d, uint32_t flags, int32_t num_cus,
                                rn_launch_config* cfg) {
  clear_error();
  if (cfg == nullptr) return fail(RN_ERR_INVALID_ARG, "cfg is NULL");
  ActKey key;
  rn_status st = check_act_shape(rows, d, flags, &key);
  if (st != RN_OK) return st;
  int cus = num_cus;
  if (cus <= 0) {
    st = device_cus(&cus);
    if (st != RN_OK) return st;
  }
  return select_act_config(rows > 0 ? rows : 1, d, key, cus, cfg);
}

rn_status rn_launch_empty(void* stream) {
  clear_error();
  return launch(empty_kernel_address(), 1, 64, nullptr, stream);
}

rn_status rn_launch_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  clear_error();
  if (bytes < 0 || bytes % 16 != 0) return fail(RN_ERR_INVALID_ARG, "bytes (%lld) must be a multiple of 16 and >= 0", (long long)bytes);
  if (bytes == 0) return RN_OK;
  if (src == nullptr || dst == nullptr) return fail(RN_ERR_INVALID_ARG, "src and dst must not be NULL");
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + static_cast<uintptr_t>(bytes) && d0 < s0 + static_cast<uintptr_t>(bytes))
    return fail(RN_ERR_INVALID_ARG, "src and dst overlap");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(RN_ERR_MISALIGNED, "src and dst must be 16-byte aligned");
  constexpr int64_t kTile = static_cast<int64_t>(kCopyThreads) * 16;
  const int64_t grid = (bytes + kTile - 1) / kTile;
  if (grid > 0x7FFFFFFF) return fail(RN_ERR_UNSUPPORTED, "copy of %lld bytes is too large", (long long)bytes);
  struct {
    const void* src;
    void* dst;
    int64_t bytes;
  } a = {src, dst, bytes};
  void* argv[] = {&a.src, &a.dst, &a.bytes};
  hipError_t e = hipLaunchKernel(copy_kernel_address(), dim3(static_cast<unsigned>(grid)), dim3(kCopyThreads), argv, 0,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RN_ERR_HIP, "hipLaunchKernel: %s", hipGetErrorString(e));
  return RN_OK;
}

const char* rn_status_string(rn_status status) {
  switch (status) {
    case RN_OK: return "RN_OK: success";
    case RN_ERR_INVALID_ARG: return "RN_ERR_INVALID_ARG: invalid argument";
    case RN_ERR_UNSUPPORTED: return "RN_ERR_UNSUPPORTED: combination or size not built";
    case RN_ERR_MISALIGNED: return "RN_ERR_MISALIGNED: pointer or stride not 16-byte aligned";
    case RN_ERR_HIP: return "RN_ERR_HIP: HIP runtime error";
    default: return "unknown rn_status";
  }
}

const char* rn_last_error(void) { return last_error(); }

int32_t rn_abi_version(void) { return RN_ABI_VERSION; }

}  // extern "C"
