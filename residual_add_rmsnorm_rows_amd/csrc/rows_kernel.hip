// Fused residual add + RMSNorm over rows: one workgroup of W wave64s per row.
//
// Computes, for each row (definition from the _qk_norm_kernel listing in the
// "QK Norm" section of "CuTeDSL at Perplexity", extended with a residual add
// and an fp8 output whose readings are stated in include/rmsnorm_rows.h):
//   h   = round_res(x + residual)         (or h = x without a residual)
//         for the variants that sum K partial inputs (KP slots, K <= KP):
//         h = round_res(p_0 + ... + p_{K-1} + residual), the exact sum of all
//         the terms rounded once (float32 without a residual)
//   inv = rsqrt(sum(h^2) / H + eps)       (float32 accumulation)
//   y   = (w + b) * (h * inv)             -> out (bf16 / f32), or
//   fp8: p = (w + b) * h, amax = max|p| * inv, y = p * inv,
//        code = e4m3fn(y * (448 / amax)), scale = amax / 448
//   (with b = 1, (w + 1) t is evaluated as the fused multiply-add w t + t:
//   one rounding)
//
// Layout of one row across the workgroup: each lane holds NV steps of VEC
// elements, VEC = 16 bytes of x (8 bf16 or 4 f32).  Step s of lane `lane` in
// wave `wave` is split into SUB chunks of U = VEC / SUB contiguous elements;
// chunk c covers row elements [u * U, u * U + U) with
//     u = ((s * W + wave) * SUB + c) * 64 + lane,
// so every load and store instruction of a wave touches one contiguous run of
// 64 * U elements of each tensor.  SUB is 1 when every tensor has the width of
// x; with bf16 x and a 32-bit residual, weight or output it is 2, which keeps
// the 32-bit tensors at 16 bytes per lane per instruction (one whole 1 KiB run)
// instead of two interleaved half-runs, whose nontemporal stores would reach
// HBM as partial lines.  All loads of a row are issued before any arithmetic
// and the row then lives in registers: each input byte is read once and each
// output byte written once.  Every tensor row is addressed through a buffer
// resource sized to the row, so chunks past the row end (a ragged hidden size)
// read zeros and write nothing, without a branch.
//
// Reduction: per-lane partial sum -> DPP inside each 16-lane row -> readlane
// of the four row totals (uniform) -> with W > 1, one float per wave through
// LDS and a single barrier (the LDS slots alternate between consecutive rows
// of a workgroup, so the next row's writes cannot race the current reads).
// With W == 1 there is no LDS traffic and no barrier (the decode shape).
//
// Quantized outputs (fp8 e4m3fn, fp4 e2m1) carry scales at one of four
// granularities ("Blackwell support" names MXFP8/MXFP4/NVFP4 and FP8
// block-wise scaling; the formats follow the OCP FP8 and MX specifications):
//   per row      scale = amax / 448, codes = e4m3fn(y * 448 / amax);
//   per 128      the same per group of 128 consecutive elements;
//   MX per 32    E8M0 scale 2^e with e = floor(log2 amax) - emax (8 for e4m3,
//                2 for e2m1), codes = encode(y * 2^-e), saturating;
//   NVFP4 / 16   E4M3FN scale s_b = e4m3fn(amax / (6 s_t)) with the caller's
//                float32 tensor scale s_t, codes = e2m1(y / (s_b s_t)).
//
// This file is compiled once per (x dtype, out dtype, scale scheme), selected
// by RN_TU_X / RN_TU_OUT / RN_TU_QS / RN_TU_NAME, so the variants build in
// parallel.

#include "device_common.h"

#ifndef RN_TU_X
#error "RN_TU_X (x dtype) must be defined"
#endif
#ifndef RN_TU_OUT
#error "RN_TU_OUT (out dtype) must be defined"
#endif

#ifndef RN_TU_QS
#define RN_TU_QS kQRow
#endif

#define RN_CAT2(a, b) a##b
#define RN_CAT(a, b) RN_CAT2(a, b)

namespace rn {
namespace {

constexpr int storage_bits(int dt) {
  return dt == kBF16 ? 16 : dt == kF32 ? 32 : dt == kFP8 ? 8 : dt == kFP4 ? 4 : 32;
}

constexpr int max_of(int a, int b) { return a > b ? a : b; }

// At one vector per lane a row takes up to 16 waves, and two such workgroups
// per CU need 8 waves per SIMD.  Every variant fits that in VGPRs, but some,
// left alone, take more SGPRs than 8 waves allow (a buffer resource per
// partial-input slot, the scale and amax resources of the block-scaled
// outputs, next to the kernel arguments) and then run one workgroup per CU:
// on MI355X the block-scaled outputs with a float32 residual at 16 x 1 ran
// 11% slower that way.  Asking for 8 waves moves the excess into VGPR lanes.
constexpr int min_waves_per_eu(int nv) { return nv == 1 ? 8 : 1; }

template <int XD, int RD, int WD, int OD, int QS, int BIAS, int NV, int KP>
__global__ __launch_bounds__(max_threads_for_nv(NV))
__attribute__((amdgpu_waves_per_eu(min_waves_per_eu(NV)))) void rows_kernel(const RowArgs a) {
  constexpr int XB = storage_bits(XD) / 8;
  constexpr int VEC = 16 / XB;
  constexpr bool HAS_RES = RD != kNone;
  constexpr bool QUANT = OD == kFP8 || OD == kFP4;
  constexpr int RB = storage_bits(RD) / 8;
  constexpr int WB = storage_bits(WD) / 8;
  constexpr int OBITS = storage_bits(OD);
  constexpr int WIDEST = max_of(max_of(XB, HAS_RES ? RB : 1), max_of(WB, max_of(OBITS / 8, 1)));
  constexpr int SUB = WIDEST / XB;          // chunks per step (1 or 2)
  constexpr int U = VEC / SUB;              // elements per chunk
  constexpr int XW = U * XB / 4;            // dwords of x per chunk
  constexpr int RW = U * RB / 4;            // dwords of residual per chunk
  constexpr int WW = U * WB / 4;            // dwords of weight per chunk
  constexpr int OCB = U * OBITS / 8;        // output bytes per chunk
  constexpr int OW = words_for<OD, U>();    // dwords holding one output chunk
  constexpr int QG = scale_group<QS>();      // elements per scale (0: one per row)
  static_assert(SUB == 1 || SUB == 2, "chunking");
  static_assert(!QUANT || QS == kQRow || (QG % U == 0 && (64 * U) % QG == 0), "scale groups");
  static_assert(QS == kQRow || QUANT, "scale groups only for quantized outputs");
  static_assert(OD != kFP4 || QS == kQMx32 || QS == kQNv16, "fp4 output is MX- or NVFP4-scaled");
  static_assert(QS != kQNv16 || OD == kFP4, "NVFP4 scales are for fp4 output");
  static_assert(KP == 1 || (KP <= kMaxParts && NV <= kMaxPartsVecsPerLane), "partial-input slots");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  __shared__ float red[2][kMaxWavesPerRow][2];
  int parity = 0;

  const char* __restrict__ xp = static_cast<const char*>(a.x);
  const char* __restrict__ rp = static_cast<const char*>(a.res);
  char* __restrict__ op = static_cast<char*>(a.out);
  char* __restrict__ rop = static_cast<char*>(a.res_out);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, static_cast<uint32_t>(a.hidden) * WB);
  const uint32_t groups = static_cast<uint32_t>(a.hidden) / (QG ? QG : a.hidden);  // scales per row
  constexpr int SCALE_BYTES = QS == kQMx32 || QS == kQNv16 ? 1 : 4;
  float tscale = 0.f;  // NVFP4's tensor scale, one uniform load
  if constexpr (QS == kQNv16) tscale = *a.tscale;

  // Element offset of chunk (s, c) of this lane from the row start:
  // (((s * W + wave) * SUB + c) * 64 + lane) * U.  Chunks past the row end
  // fall outside the row's buffer resources.  The partial-input kernels write
  // it as the lane's offset of chunk (0, 0) plus a per-chunk term, so that the
  // chunk term of step 0 is a constant folded into the instructions' immediate
  // offsets instead of one offset register per chunk and tensor (those
  // kernels are the ones short of registers).  They also rebuild the lane
  // offset before the output stage (le below), so that the store and scale
  // offsets are derived there instead of being held across the whole row.
  const uint32_t lane_elem = static_cast<uint32_t>((wave * SUB * 64 + lane) * U);
  uint32_t le = lane_elem;
  auto elem_of = [&](int s, int c) -> uint32_t {
    if constexpr (KP > 1) return le + static_cast<uint32_t>((s * nw * SUB + c) * 64 * U);
    return static_cast<uint32_t>((((s * nw + wave) * SUB + c) * 64 + lane) * U);
  };

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t row_elem = row * a.hidden;
    // x, or partial-input slot k; a slot past num_parts gets an empty
    // resource (its loads return zeros without touching memory)
    auto x_rsrc = [&](int k) -> __amdgpu_buffer_rsrc_t {
      if constexpr (KP == 1) {
        return make_rsrc(xp + row_elem * XB, static_cast<uint32_t>(a.hidden) * XB);
      } else {
        const bool used = k < a.num_parts;
        const char* pk = static_cast<const char*>(a.parts[used ? k : 0]);
        return make_rsrc(pk + row_elem * XB, used ? static_cast<uint32_t>(a.hidden) * XB : 0u);
      }
    };
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rp + row_elem * RB, static_cast<uint32_t>(a.hidden) * RB);
    const __amdgpu_buffer_rsrc_t orr =
        make_rsrc(op + row_elem * OBITS / 8, static_cast<uint32_t>(a.hidden) * OBITS / 8);
    const __amdgpu_buffer_rsrc_t ror = make_rsrc(rop + row_elem * RB, static_cast<uint32_t>(a.hidden) * RB);

    // 1. Issue every load of this lane's share of the row.  Partial inputs
    //    go slot by slot, so that one slot's resource is live at a time.
    uint32_t xw[NV][SUB][KP][XW];
    uint32_t rw[NV][SUB][HAS_RES ? RW : 1];
    uint32_t ww[NV][SUB][WW];
    // The partial-input kernels load the weight after the first chunk's sums
    // (it is a cache hit, first needed for the weighted products or the
    // scaling): before them the loaded partials hold most of their registers.
    // The loads go ahead of the first residual store, because the vector
    // memory counter retires in issue order: a weight load issued after the
    // stores could only be waited for together with them.
    constexpr bool LATE_W = KP > 1;
    if constexpr (KP > 1) {
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const __amdgpu_buffer_rsrc_t pr = x_rsrc(k);
#pragma unroll
        for (int s = 0; s < NV; ++s) {
#pragma unroll
          for (int c = 0; c < SUB; ++c) buffer_load_words<XW * 4, true>(pr, elem_of(s, c) * XB, xw[s][c][k]);
        }
      }
      // An unused slot loads zeros (an empty resource); its elements become
      // -0, the identity of IEEE addition (x + -0 == x for every x, signed
      // zeros included), so that the sums add every slot without a branch.
      // The host launches a KP-slot kernel only for more than KP / 2
      // partials, so the slots below that are always in use.
      constexpr uint32_t kNegZeros = XD == kBF16 ? 0x80008000u : 0x80000000u;
#pragma unroll
      for (int k = KP / 2 + 1; k < KP; ++k) {
        const uint32_t neg = k < a.num_parts ? 0u : kNegZeros;
#pragma unroll
        for (int s = 0; s < NV; ++s) {
#pragma unroll
          for (int c = 0; c < SUB; ++c) {
#pragma unroll
            for (int j = 0; j < XW; ++j) xw[s][c][k][j] |= neg;
          }
        }
      }
    }
    const __amdgpu_buffer_rsrc_t xr = x_rsrc(0);
#pragma unroll
    for (int s = 0; s < NV; ++s) {
#pragma unroll
      for (int c = 0; c < SUB; ++c) {
        const uint32_t e = elem_of(s, c);
        if constexpr (KP == 1) buffer_load_words<XW * 4, true>(xr, e * XB, xw[s][c][0]);
        if constexpr (HAS_RES) buffer_load_words<RW * 4, true>(rr, e * RB, rw[s][c]);
        if constexpr (!LATE_W) buffer_load_words<WW * 4, false>(wr, e * WB, ww[s][c]);
      }
    }

    // 2. Residual add (rounded once to the residual dtype and written back),
    //    local sum of squares of the rounded value; quantized outputs also
    //    take the weighted products p = (w + b) * h (and, with one scale per
    //    row, their local max magnitude).
    float h[NV][SUB][U];
    float ss = 0.f;
    float mx = 0.f;

#pragma unroll
    for (int s = 0; s < NV; ++s) {
#pragma unroll
      for (int c = 0; c < SUB; ++c) {
        if constexpr (KP > 1) {
          // Partial inputs: the exact sum of the partials (and the residual),
          // rounded once -- to the residual dtype, or to float32 without a
          // residual.  Every slot is added, the unused ones as -0 (see the
          // loads).  One element at a time, so that a single accumulator is
          // live and each slot's words die as they are used.
          float hr[U];
#pragma unroll
          for (int i = 0; i < U; ++i) {
            ExactSum acc;
            acc.init(element<XD>(xw[s][c][0], i));
            constexpr int LAST = HAS_RES ? KP : KP - 1;  // slots added before the last term
#pragma unroll
            for (int k = 1; k < LAST; ++k) acc.add(element<XD>(xw[s][c][k], i));
            if constexpr (HAS_RES) {
              // bf16: rounded to odd here, to nearest even by the pack below
              hr[i] = add_last_and_round<RD == kBF16>(acc, element<RD>(rw[s][c], i));
            } else {
              hr[i] = add_last_and_round<false>(acc, element<XD>(xw[s][c][KP - 1], i));
            }
          }
          if (s == 0 && c == 0) {
#pragma unroll
            for (int s2 = 0; s2 < NV; ++s2) {
#pragma unroll
              for (int c2 = 0; c2 < SUB; ++c2) buffer_load_words<WW * 4, false>(wr, elem_of(s2, c2) * WB, ww[s2][c2]);
            }
          }
          if constexpr (HAS_RES) {
            uint32_t hw[RW];
            pack<RD, U>(hr, hw);
            unpack<RD, U>(hw, h[s][c]);
            buffer_store_words<RW * 4>(ror, elem_of(s, c) * RB, hw);
          } else {
#pragma unroll
            for (int i = 0; i < U; ++i) h[s][c][i] = hr[i];
          }
        } else if constexpr (HAS_RES) {
          float xf[U], rf[U], sum[U];
          unpack<XD, U>(xw[s][c][0], xf);
          unpack<RD, U>(rw[s][c], rf);
#pragma unroll
          for (int i = 0; i < U; ++i) sum[i] = xf[i] + rf[i];
          uint32_t hw[RW];
          pack<RD, U>(sum, hw);
          unpack<RD, U>(hw, h[s][c]);
          buffer_store_words<RW * 4>(ror, elem_of(s, c) * RB, hw);
        } else {
          unpack<XD, U>(xw[s][c][0], h[s][c]);
        }
#pragma unroll
        for (int i = 0; i < U; ++i) ss += h[s][c][i] * h[s][c][i];
        if constexpr (QUANT && !LATE_W) {
          float wf[U];
          unpack<WD, U>(ww[s][c], wf);
#pragma unroll
          for (int i = 0; i < U; ++i) {
            // (1 + w) h as one fused multiply-add w h + h: a single rounding
            h[s][c][i] = BIAS ? __builtin_fmaf(wf[i], h[s][c][i], h[s][c][i]) : wf[i] * h[s][c][i];
            if constexpr (QS == kQRow) mx = __builtin_fmaxf(mx, __builtin_fabsf(h[s][c][i]));
          }
        }
      }
    }

    if constexpr (LATE_W) {
      if constexpr (QUANT) {
#pragma unroll
        for (int s = 0; s < NV; ++s) {
#pragma unroll
          for (int c = 0; c < SUB; ++c) {
            float wf[U];
            unpack<WD, U>(ww[s][c], wf);
#pragma unroll
            for (int i = 0; i < U; ++i) {
              h[s][c][i] = BIAS ? __builtin_fmaf(wf[i], h[s][c][i], h[s][c][i]) : wf[i] * h[s][c][i];
              if constexpr (QS == kQRow) mx = __builtin_fmaxf(mx, __builtin_fabsf(h[s][c][i]));
            }
          }
        }
      }
    }

    // 3. Row reduction: DPP + readlane inside the wave, LDS across waves.
    constexpr bool ROW_MAX = QUANT && QS == kQRow;
    ss = group_reduce<64, OpSum>(ss);
    if constexpr (ROW_MAX) mx = group_reduce<64, OpMax>(mx);
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
        if constexpr (ROW_MAX) mx = __builtin_fmaxf(mx, red[parity][i][1]);
      }
      parity ^= 1;
    }
    const float inv = rsqrtf(ss / static_cast<float>(a.hidden) + a.eps);

    // 4. Scale and store.  Scale groups (per 128, 32 or 16 elements) are GL
    //    neighbouring lanes of one chunk: their max is a DPP group reduction,
    //    and the group's first lane stores its scale (and amax).
    if constexpr (KP > 1) {
      // an empty asm that hides le's value from the optimizer: offsets
      // derived from it below stay here instead of being hoisted out of the
      // row loop (where they would occupy VGPRs through the loads)
      le = lane_elem;
      asm volatile("" : "+v"(le));
    }
    float amax = 0.f, qmul = 0.f;
    if constexpr (ROW_MAX) {
      amax = mx * inv;  // == max |p * inv|: multiplying by inv > 0 is monotone
      qmul = amax > 0.f ? 448.0f / amax : 0.f;
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
        float y[U];
        if constexpr (QUANT && QS == kQRow) {
#pragma unroll
          for (int i = 0; i < U; ++i) y[i] = (h[s][c][i] * inv) * qmul;
        } else if constexpr (QUANT) {
          quantize_group_chunk<OD, QS, U>(h[s][c], inv, lane, elem_of(s, c) / QG, sr, ar, a.amax != nullptr, y,
                                          tscale);
        } else {
          float wf[U];
          unpack<WD, U>(ww[s][c], wf);
#pragma unroll
          for (int i = 0; i < U; ++i) {
            const float t = h[s][c][i] * inv;
            y[i] = BIAS ? __builtin_fmaf(wf[i], t, t) : wf[i] * t;  // (1 + w) t, one rounding
          }
        }
        uint32_t ow[OW];
        pack<OD, U>(y, ow);
        buffer_store_words<OCB>(orr, elem_of(s, c) * OBITS / 8, ow);
      }
    }
    if constexpr (ROW_MAX) {
      if (threadIdx.x == 0) {
        static_cast<float*>(a.scale)[row] = amax / 448.0f;  // IEEE float32 division
        if (a.amax != nullptr) a.amax[row] = amax;
      }
    }
  }
}

template <int XD, int RD, int WD, int OD, int QS, int BIAS, int NV>
const void* pick_kp(int kp) {
  switch (kp) {
    case 2: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, QS, BIAS, NV, 2>);
    case 4: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, QS, BIAS, NV, 4>);
    case 8: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, QS, BIAS, NV, 8>);
    default: return nullptr;
  }
}

template <int XD, int RD, int WD, int OD, int QS, int BIAS>
const void* pick_nv(int nv, int kp) {
  if (kp == 1) {
    switch (nv) {
      case 1: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, QS, BIAS, 1, 1>);
      case 2: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, QS, BIAS, 2, 1>);
      case 4: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, QS, BIAS, 4, 1>);
      case 8: return reinterpret_cast<const void*>(&rows_kernel<XD, RD, WD, OD, QS, BIAS, 8, 1>);
      default: return nullptr;
    }
  }
  // partial inputs: every output type and scale scheme, 1 or 2 vectors per lane
  if (nv == 1) return pick_kp<XD, RD, WD, OD, QS, BIAS, 1>(kp);
  if (nv == 2) return pick_kp<XD, RD, WD, OD, QS, BIAS, 2>(kp);
  return nullptr;
}

template <int XD, int RD, int OD, int QS>
const void* pick_weight(const RowKey& k) {
  if (k.w == kBF16)
    return k.bias ? pick_nv<XD, RD, kBF16, OD, QS, 1>(k.nv, k.kp) : pick_nv<XD, RD, kBF16, OD, QS, 0>(k.nv, k.kp);
  if (k.w == kF32)
    return k.bias ? pick_nv<XD, RD, kF32, OD, QS, 1>(k.nv, k.kp) : pick_nv<XD, RD, kF32, OD, QS, 0>(k.nv, k.kp);
  return nullptr;
}

}  // namespace

// Built combinations for this (x, out, scale scheme): residual none, f32, or
// the x dtype; weight bf16 or f32; both weight forms; 1, 2, 4 or 8 vectors
// per lane; and the partial-input variants: 2, 4 or 8 slots at 1 or 2
// vectors per lane.
const void* RN_CAT(pick_row_kernel_, RN_TU_NAME)(const RowKey& k) {
  if (k.x != RN_TU_X || k.out != RN_TU_OUT || k.qs != RN_TU_QS) return nullptr;
  switch (k.res) {
    case kNone: return pick_weight<RN_TU_X, kNone, RN_TU_OUT, RN_TU_QS>(k);
    case kF32: return pick_weight<RN_TU_X, kF32, RN_TU_OUT, RN_TU_QS>(k);
    case kBF16:
      if constexpr (RN_TU_X == kBF16) return pick_weight<kBF16, kBF16, RN_TU_OUT, RN_TU_QS>(k);
      return nullptr;
    default: return nullptr;
  }
}

}  // namespace rn
