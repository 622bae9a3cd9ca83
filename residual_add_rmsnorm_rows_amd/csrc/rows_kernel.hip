// Fused residual add + RMSNorm over rows: one workgroup of W wave64s per row.
//
// Computes, for each row (definition from the _qk_norm_kernel listing in the
// "QK Norm" section of "CuTeDSL at Perplexity", extended with a residual add
// and an fp8 output whose readings are stated in include/rmsnorm_rows.h):
//   h   = round_res(x + residual)         (or h = x without a residual)
//   inv = rsqrt(sum(h^2) / H + eps)       (float32 accumulation)
//   y   = (w + b) * (h * inv)             -> out (bf16 / f32), or
//   fp8: p = (w + b) * h, amax = max|p| * inv, y = p * inv,
//        code = e4m3fn(y * (448 / amax)), scale = amax / 448
//
// Layout of one row across the workgroup: the row is H / VEC lane vectors of
// 16 bytes of x (VEC = 8 bf16 or 4 f32).  Vector v = (s * W + wave) * 64 + lane
// belongs to lane `lane` of wave `wave` at step s < NV, so every load and
// store instruction of a wave touches 64 consecutive vectors (1 KiB of x).
// All loads of a row are issued before any arithmetic, the row then lives in
// registers: each input byte is read once and each output byte written once.
//
// Reduction: per-lane partial sum -> DPP inside each 16-lane row -> readlane
// of the four row totals (uniform) -> with W > 1, one float per wave through
// LDS and a single barrier (the LDS slots alternate between consecutive rows
// of a workgroup, so the next row's writes cannot race the current reads).
// With W == 1 there is no LDS traffic and no barrier (the decode shape).
//
// This file is compiled once per (x dtype, out dtype) pair, selected by
// RN_TU_X / RN_TU_OUT / RN_TU_NAME, so the variants build in parallel.

#include "device_common.h"

#ifndef RN_TU_X
#error "RN_TU_X (x dtype) must be defined"
#endif
#ifndef RN_TU_OUT
#error "RN_TU_OUT (out dtype) must be defined"
#endif

#define RN_CAT2(a, b) a##b
#define RN_CAT(a, b) RN_CAT2(a, b)

namespace rn {
namespace {

constexpr int storage_bytes(int dt) { return dt == kBF16 ? 2 : dt == kFP8 ? 1 : 4; }

template <int XD, int RD, int WD, int OD, int BIAS, int NV>
__global__ __launch_bounds__(max_threads_for_nv(NV)) void rows_kernel(const RowArgs a) {
  constexpr int XB = storage_bytes(XD);
  constexpr int VEC = 16 / XB;
  constexpr bool HAS_RES = RD != kNone;
  constexpr bool FP8 = OD == kFP8;
  constexpr int RB = storage_bytes(RD);
  constexpr int WB = storage_bytes(WD);
  constexpr int OB = storage_bytes(OD);
  constexpr int RW = VEC * RB / 4;        // dwords of residual per lane vector
  constexpr int WW = VEC * WB / 4;        // dwords of weight per lane vector
  constexpr int OW = (VEC * OB + 3) / 4;  // dwords of output per lane vector

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  __shared__ float red[2][kMaxWavesPerRow][2];
  int parity = 0;

  const char* __restrict__ xp = static_cast<const char*>(a.x);
  const char* __restrict__ rp = static_cast<const char*>(a.res);
  const char* __restrict__ wp = static_cast<const char*>(a.w);
  char* __restrict__ op = static_cast<char*>(a.out);
  char* __restrict__ rop = static_cast<char*>(a.res_out);

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t row_elem = row * a.hidden;

    // 1. Issue every load of this lane's share of the row.
    uint32_t xw[NV][4];
    uint32_t rw[NV][HAS_RES ? RW : 1];
    uint32_t ww[NV][WW];
    bool ok[NV];
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int v = (s * nw + wave) * 64 + lane;
      ok[s] = v < a.nvec;
      if (ok[s]) {
        const int64_t e = row_elem + static_cast<int64_t>(v) * VEC;
        load_words<16>(xp + e * XB, xw[s]);
        if constexpr (HAS_RES) load_words<RW * 4>(rp + e * RB, rw[s]);
        load_words<WW * 4>(wp + static_cast<int64_t>(v) * VEC * WB, ww[s]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xw[s][i] = 0;
#pragma unroll
        for (int i = 0; i < (HAS_RES ? RW : 1); ++i) rw[s][i] = 0;
#pragma unroll
        for (int i = 0; i < WW; ++i) ww[s][i] = 0;
      }
    }

    // 2. Residual add (rounded once to the residual dtype and written back),
    //    local sum of squares of the rounded value; fp8 also takes the
    //    weighted products and their local max magnitude.
    float h[NV][VEC];
    float ss = 0.f;
    float mx = 0.f;
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      float xf[VEC];
      unpack<XD, VEC>(xw[s], xf);
      if constexpr (HAS_RES) {
        float rf[VEC], sum[VEC];
        unpack<RD, VEC>(rw[s], rf);
#pragma unroll
        for (int i = 0; i < VEC; ++i) sum[i] = xf[i] + rf[i];
        uint32_t hw[RW];
        pack<RD, VEC>(sum, hw);
        unpack<RD, VEC>(hw, h[s]);
        if (ok[s]) {
          const int64_t e = row_elem + static_cast<int64_t>((s * nw + wave) * 64 + lane) * VEC;
          store_words<RW * 4>(rop + e * RB, hw);
        }
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) h[s][i] = xf[i];
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) ss += h[s][i] * h[s][i];
      if constexpr (FP8) {
        float wf[VEC];
        unpack<WD, VEC>(ww[s], wf);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          if constexpr (BIAS) wf[i] += 1.0f;
          h[s][i] = wf[i] * h[s][i];
          mx = __builtin_fmaxf(mx, __builtin_fabsf(h[s][i]));
        }
      }
    }

    // 3. Row reduction: DPP + readlane inside the wave, LDS across waves.
    ss = group_reduce<64, OpSum>(ss);
    if constexpr (FP8) mx = group_reduce<64, OpMax>(mx);
    if (nw > 1) {
      if (lane == 0) {
        red[parity][wave][0] = ss;
        red[parity][wave][1] = mx;
      }
      __syncthreads();
      ss = 0.f;
      mx = 0.f;
      for (int i = 0; i < nw; ++i) {
        ss += red[parity][i][0];
        if constexpr (FP8) mx = __builtin_fmaxf(mx, red[parity][i][1]);
      }
      parity ^= 1;
    }
    const float inv = rsqrtf(ss / static_cast<float>(a.hidden) + a.eps);

    // 4. Scale and store.
    float amax = 0.f, qmul = 0.f;
    if constexpr (FP8) {
      amax = mx * inv;  // == max |p * inv|: multiplying by inv > 0 is monotone
      qmul = amax > 0.f ? 448.0f / amax : 0.f;
    }
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      float y[VEC];
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) y[i] = (h[s][i] * inv) * qmul;
      } else {
        float wf[VEC];
        unpack<WD, VEC>(ww[s], wf);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          if constexpr (BIAS) wf[i] += 1.0f;
          y[i] = wf[i] * (h[s][i] * inv);
        }
      }
      uint32_t ow[OW];
      pack<OD, VEC>(y, ow);
      if (ok[s]) {
        const int64_t e = row_elem + static_cast<int64_t>((s * nw + wave) * 64 + lane) * VEC;
        store_words<OW * 4>(op + e * OB, ow);
      }
    }
    if constexpr (FP8) {
      if (threadIdx.x == 0) {
        a.scale[row] = amax / 448.0f;  // IEEE float32 division
        if (a.amax != nullptr) a.amax[row] = amax;
      }
    }
  }
}

template <int XD, int RD, int WD, int OD, int BIAS>
const void* pick_nv(int nv) {
  switch (nv) {
    case 1: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, BIAS, 1>);
    case 2: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, BIAS, 2>);
    case 4: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, BIAS, 4>);
    case 8: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, BIAS, 8>);
    default: return nullptr;
  }
}

template <int XD, int RD, int OD>
const void* pick_weight(const RowKey& k) {
  if (k.w == kBF16) return k.bias ? pick_nv<XD, RD, kBF16, OD, 1>(k.nv) : pick_nv<XD, RD, kBF16, OD, 0>(k.nv);
  if (k.w == kF32) return k.bias ? pick_nv<XD, RD, kF32, OD, 1>(k.nv) : pick_nv<XD, RD, kF32, OD, 0>(k.nv);
  return nullptr;
}

}  // namespace

// Built combinations for this (x, out) pair: residual none, f32, or the x
// dtype; weight bf16 or f32; both weight forms; 1, 2, 4 or 8 vectors per lane.
const void* RN_CAT(pick_row_kernel_, RN_TU_NAME)(const RowKey& k) {
  if (k.x != RN_TU_X || k.out != RN_TU_OUT) return nullptr;
  switch (k.res) {
    case kNone: return pick_weight<RN_TU_X, kNone, RN_TU_OUT>(k);
    case kF32: return pick_weight<RN_TU_X, kF32, RN_TU_OUT>(k);
    case kBF16:
      if constexpr (RN_TU_X == kBF16) return pick_weight<kBF16, kBF16, RN_TU_OUT>(k);
      return nullptr;
    default: return nullptr;
  }
}

}  // namespace rn
