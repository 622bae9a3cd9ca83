// SiLU-and-mul (SwiGLU) over rows: out[r, i] = silu(x[r, i]) * x[r, d + i].
//
// The MLP's gated activation ("Tile-Level Activation Overlap for Efficient LLM
// Inference": the SwiGLU step combines the gate and up projections; "CuTeDSL
// at Perplexity", section "Inference at Perplexity": activation kernels in the
// same kernel library).  Each row of x holds the gate projection in its first
// half and the up projection in its second half (a merged gate/up GEMM
// output).  silu(g) = g * sigmoid(g), evaluated in float32 as
// g * (e / (1 + e)) for g < 0 and g / (1 + e) otherwise, with e = exp(-|g|),
// for float32 outputs, and through an offset exponent with the hardware exp2
// and reciprocal for the narrower outputs (see silu_mul_f32).
//
// Same machinery as the rows kernel: one workgroup of W wave64s per row, each
// lane holding NV steps of one 16-byte chunk of the gate and the matching
// chunk of the up half, buffer resources sized to each half row (ragged ends
// read zeros and write nothing), nontemporal loads and stores.  Outputs:
// bf16 / f32, or quantized (fp8 e4m3fn with a per-row, per-128 or MX scale;
// fp4 e2m1 with an MX or NVFP4 scale).  Only the per-row scale needs a reduction across
// the row (DPP + readlane, then LDS across waves); every other output is local
// to a lane or to a lane group.

#include "device_common.h"

namespace rn {
namespace {

constexpr int act_bits(int dt) { return dt == kBF16 ? 16 : dt == kF32 ? 32 : dt == kFP8 ? 8 : 4; }
constexpr int act_max(int a, int b) { return a > b ? a : b; }

// silu(g) * u in float32.
//
// ACCURATE (float32 outputs): e = exp(-|g|) with the library expf, then
// g / (1 + e) for g >= 0 and g e / (1 + e) otherwise, through an IEEE
// division: a few float32 ulps, and no intermediate overflows.
//
// Otherwise (bf16 / fp8 / fp4 outputs, whose rounding step is 2^-8 relative
// or coarser): silu(g) u = g u / (1 + exp(-g)) evaluated as
//     t = 2^(-g log2(e) - 64) = exp(-g) 2^-64,
//     silu(g) u = (g u) * (rcp(t + 2^-64) * 2^-64),
// with the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32).  The 2^-64
// offset keeps t finite for -132 < g, where the plain form's exp(-g)
// overflows from g < -88.  The factor in parentheses is 1 / (1 + exp(-g)):
// in [1/2, 1) for g >= 0, so g u is never scaled up; for g < -87.3 it falls
// into float32's subnormal range (fewer bits) and below g = -103 to zero,
// where the true result is a normal number only if |u| exceeds about 1e35.
// The argument's rounding near 64 costs about 2^-17 relative, far below those
// formats' steps, in 7 instructions per element without compare or select.
template <bool ACCURATE>
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  if constexpr (ACCURATE) {
    const float e = expf(-__builtin_fabsf(g));  // in (0, 1]
    const float r = 1.0f / (1.0f + e);
    return (g * (g >= 0.f ? r : e * r)) * u;
  } else {
    const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(g, -1.4426950408889634f, -64.0f));
    return (g * u) * (__builtin_amdgcn_rcpf(t + 0x1p-64f) * 0x1p-64f);
  }
}

template <int XD, int OD, int QS, int NV>
__global__ __launch_bounds__(max_threads_for_nv(NV)) void silu_mul_kernel(const ActArgs a) {
  constexpr int XB = act_bits(XD) / 8;
  constexpr int VEC = 16 / XB;
  constexpr bool QUANT = OD == kFP8 || OD == kFP4;
  constexpr int OBITS = act_bits(OD);
  constexpr int SUB = act_max(XB, act_max(OBITS / 8, 1)) / XB;  // chunks per step (1 or 2)
  constexpr int U = VEC / SUB;                                   // elements per chunk
  constexpr int XW = U * XB / 4;
  constexpr int OCB = U * OBITS / 8;
  constexpr int OW = words_for<OD, U>();
  constexpr int QG = scale_group<QS>();
  constexpr bool ROW_MAX = QUANT && QS == kQRow;
  static_assert(SUB == 1 || SUB == 2, "chunking");
  static_assert(QS == kQRow || QUANT, "scale groups only for quantized outputs");
  static_assert(OD != kFP4 || QS == kQMx32 || QS == kQNv16, "fp4 output is MX- or NVFP4-scaled");
  static_assert(QS != kQNv16 || OD == kFP4, "NVFP4 scales are for fp4 output");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  __shared__ float red[2][kMaxWavesPerRow];
  int parity = 0;

  const char* __restrict__ xp = static_cast<const char*>(a.x);
  char* __restrict__ op = static_cast<char*>(a.out);
  const uint32_t d = static_cast<uint32_t>(a.d);
  const uint32_t groups = d / (QG ? QG : d);  // scales per row
  constexpr int SCALE_BYTES = QS == kQMx32 || QS == kQNv16 ? 1 : 4;
  float tscale = 0.f;  // NVFP4's tensor scale, one uniform load
  if constexpr (QS == kQNv16) tscale = *a.tscale;

  auto elem_of = [&](int s, int c) -> uint32_t {
    return static_cast<uint32_t>((((s * nw + wave) * SUB + c) * 64 + lane) * U);
  };

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const char* xrow = xp + row * 2 * static_cast<int64_t>(d) * XB;
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(xrow, d * XB);
    const __amdgpu_buffer_rsrc_t ur = make_rsrc(xrow + static_cast<int64_t>(d) * XB, d * XB);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(op + row * static_cast<int64_t>(d) * OBITS / 8, d * OBITS / 8);

    uint32_t gw[NV][SUB][XW], uw[NV][SUB][XW];
#pragma unroll
    for (int s = 0; s < NV; ++s) {
#pragma unroll
      for (int c = 0; c < SUB; ++c) {
        const uint32_t e = elem_of(s, c);
        buffer_load_words<XW * 4, true>(gr, e * XB, gw[s][c]);
        buffer_load_words<XW * 4, true>(ur, e * XB, uw[s][c]);
      }
    }

    float y[NV][SUB][U];
    float mx = 0.f;
#pragma unroll
    for (int s = 0; s < NV; ++s) {
#pragma unroll
      for (int c = 0; c < SUB; ++c) {
        float g[U], u[U];
        unpack<XD, U>(gw[s][c], g);
        unpack<XD, U>(uw[s][c], u);
#pragma unroll
        for (int i = 0; i < U; ++i) {
          y[s][c][i] = silu_mul_f32<OD == kF32>(g[i], u[i]);
          if constexpr (ROW_MAX) mx = __builtin_fmaxf(mx, __builtin_fabsf(y[s][c][i]));
        }
      }
    }

    float qmul = 0.f;
    if constexpr (ROW_MAX) {
      mx = group_reduce<64, OpMax>(mx);
      if (nw > 1) {
        if (lane == 0) red[parity][wave] = mx;
        __syncthreads();
        mx = 0.f;
        for (int i = 0; i < nw; ++i) mx = __builtin_fmaxf(mx, red[parity][i]);
        parity ^= 1;
      }
      qmul = mx > 0.f ? 448.0f / mx : 0.f;
    }
    __amdgpu_buffer_rsrc_t sr, ar;
    if constexpr (QUANT && QS != kQRow) {
      char* sbase = static_cast<char*>(a.scale) + row * groups * SCALE_BYTES;
      sr = make_rsrc(sbase, groups * SCALE_BYTES);
      ar = make_rsrc(a.amax != nullptr ? reinterpret_cast<char*>(a.amax) + row * groups * 4 : sbase,
                     a.amax != nullptr ? groups * 4 : 0);
    }
#pragma unroll
    for (int s = 0; s < NV; ++s) {
#pragma unroll
      for (int c = 0; c < SUB; ++c) {
        float q[U];
        if constexpr (ROW_MAX) {
#pragma unroll
          for (int i = 0; i < U; ++i) q[i] = y[s][c][i] * qmul;
        } else if constexpr (QUANT) {
          quantize_group_chunk<OD, QS, U>(y[s][c], 1.0f, lane, elem_of(s, c) / QG, sr, ar, a.amax != nullptr, q,
                                          tscale);
        } else {
#pragma unroll
          for (int i = 0; i < U; ++i) q[i] = y[s][c][i];
        }
        uint32_t ow[OW];
        pack<OD, U>(q, ow);
        buffer_store_words<OCB>(orr, elem_of(s, c) * OBITS / 8, ow);
      }
    }
    if constexpr (ROW_MAX) {
      if (threadIdx.x == 0) {
        static_cast<float*>(a.scale)[row] = mx / 448.0f;  // IEEE float32 division
        if (a.amax != nullptr) a.amax[row] = mx;
      }
    }
  }
}

template <int XD, int OD, int QS>
const void* pick_act_nv(int nv) {
  switch (nv) {
    case 1: return reinterpret_cast<const void*>(&silu_mul_kernel<XD, OD, QS, 1>);
    case 2: return reinterpret_cast<const void*>(&silu_mul_kernel<XD, OD, QS, 2>);
    case 4: return reinterpret_cast<const void*>(&silu_mul_kernel<XD, OD, QS, 4>);
    case 8: return reinterpret_cast<const void*>(&silu_mul_kernel<XD, OD, QS, 8>);
    default: return nullptr;
  }
}

template <int XD>
const void* pick_act_out(const ActKey& k) {
  if (k.out == kBF16 && k.qs == kQRow) return pick_act_nv<XD, kBF16, kQRow>(k.nv);
  if (k.out == kF32 && k.qs == kQRow) return pick_act_nv<XD, kF32, kQRow>(k.nv);
  if (k.out == kFP8 && k.qs == kQRow) return pick_act_nv<XD, kFP8, kQRow>(k.nv);
  if (k.out == kFP8 && k.qs == kQGroup128) return pick_act_nv<XD, kFP8, kQGroup128>(k.nv);
  if (k.out == kFP8 && k.qs == kQMx32) return pick_act_nv<XD, kFP8, kQMx32>(k.nv);
  if (k.out == kFP4 && k.qs == kQMx32) return pick_act_nv<XD, kFP4, kQMx32>(k.nv);
  if (k.out == kFP4 && k.qs == kQNv16) return pick_act_nv<XD, kFP4, kQNv16>(k.nv);
  return nullptr;
}

}  // namespace

const void* pick_act_kernel(const ActKey& k) {
  if (k.x == kBF16) return pick_act_out<kBF16>(k);
  if (k.x == kF32) return pick_act_out<kF32>(k);
  return nullptr;
}

}  // namespace rn
