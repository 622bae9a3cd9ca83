// Per-head RMSNorm of Q and K ("CuTeDSL at Perplexity", section "QK Norm").
//
// Every (token, head) pair is a row of head_dim elements; rows are numbered
// token-major with the Q heads of a token first and then its K heads, as in
// the page's kernel.  A head is spread over G = head_dim / VEC lanes (each
// lane holds one 16-byte vector: 8 bf16 or 4 f32), so a wave64 holds 64 / G
// heads side by side and its sum-of-squares reduction never leaves a group of
// G lanes (DPP inside 16-lane rows, ds_swizzle for 32, readlane for 64).
//
// MI355X mapping (differs from the page's one-head-per-thread-group launch):
// each lane group normalizes RPL heads, with all RPL loads issued before the
// first reduction, to keep enough bytes in flight per lane; a wave covers the
// 64 / G * RPL consecutive rows [first, first + 64 / G * RPL), so each load
// instruction reads 64 consecutive vectors when the heads are contiguous.
// Rows past the end are masked (the page's kernel needs an exact grid).
// Weights: every lane loads its slice of the Q and K weights once.  Heads are
// loaded without the nontemporal hint: on MI355X this kernel measured 6.07
// TB/s with plain loads and 5.25 TB/s with the hint (4096 x 32 x 128 bf16).

#include "device_common.h"

namespace rn {
namespace {

constexpr int storage_bytes(int dt) { return dt == kBF16 ? 2 : 4; }

template <int TD, int WD, int BIAS, int D, int RPL>
__global__ __launch_bounds__(kHeadBlockThreads) void heads_kernel(const HeadArgs a) {
  constexpr int TB = storage_bytes(TD);
  constexpr int WB = storage_bytes(WD);
  constexpr int VEC = 16 / TB;
  constexpr int G = D / VEC;    // lanes per head
  constexpr int GPW = 64 / G;   // heads side by side in a wave
  constexpr int WW = VEC * WB / 4;
  static_assert(G >= 8 && G <= 64, "lanes per head");

  const int lane = threadIdx.x & 63;
  const int gl = lane % G;
  const int grp = lane / G;
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t first = wave_id * (GPW * RPL);

  uint32_t qw[WW], kw[WW];
  load_words<WW * 4>(static_cast<const char*>(a.qw) + gl * VEC * WB, qw);
  if (a.kw != nullptr) {
    load_words<WW * 4>(static_cast<const char*>(a.kw) + gl * VEC * WB, kw);
  } else {
#pragma unroll
    for (int i = 0; i < WW; ++i) kw[i] = 0;
  }

  uint32_t xw[RPL][4];
  int64_t off[RPL];  // element offset of this lane's vector inside q or k
  bool ok[RPL], isq[RPL];
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    const int64_t row = first + j * GPW + grp;
    ok[j] = row < a.total_rows;
    isq[j] = true;
    off[j] = 0;
    if (ok[j]) {
      const uint32_t r = static_cast<uint32_t>(row);
      const uint32_t token = r / static_cast<uint32_t>(a.num_heads);
      const int hoff = static_cast<int>(r - token * static_cast<uint32_t>(a.num_heads));
      isq[j] = hoff < a.num_q_heads;
      off[j] = isq[j] ? token * a.q_stride + static_cast<int64_t>(hoff) * D + gl * VEC
                      : token * a.k_stride + static_cast<int64_t>(hoff - a.num_q_heads) * D + gl * VEC;
      const char* src = static_cast<const char*>(isq[j] ? a.q : a.k);
      load_words<16>(src + off[j] * TB, xw[j]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) xw[j][i] = 0;
    }
  }

#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    float x[VEC];
    unpack<TD, VEC>(xw[j], x);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) ss += x[i] * x[i];
    ss = group_reduce<G, OpSum>(ss);
    const float inv = rsqrtf(ss / static_cast<float>(D) + a.eps);
    float wf[VEC];
    if (isq[j]) {
      unpack<WD, VEC>(qw, wf);
    } else {
      unpack<WD, VEC>(kw, wf);
    }
    float y[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float t = x[i] * inv;
      y[i] = BIAS ? __builtin_fmaf(wf[i], t, t) : wf[i] * t;  // (1 + w) t, one rounding
    }
    uint32_t ow[4];
    pack<TD, VEC>(y, ow);
    if (ok[j]) {
      char* dst = static_cast<char*>(isq[j] ? a.q_out : a.k_out);
      store_words<16>(dst + off[j] * TB, ow);
    }
  }
}

template <int TD, int WD, int BIAS, int D>
const void* pick_rpl(int rpl) {
  switch (rpl) {
    case 1: return reinterpret_cast<const void*>(&heads_kernel<TD, WD, BIAS, D, 1>);
    case 2: return reinterpret_cast<const void*>(&heads_kernel<TD, WD, BIAS, D, 2>);
    case 4: return reinterpret_cast<const void*>(&heads_kernel<TD, WD, BIAS, D, 4>);
    default: return nullptr;
  }
}

template <int TD, int WD, int BIAS>
const void* pick_dim(const HeadKey& k) {
  switch (k.head_dim) {
    case 64: return pick_rpl<TD, WD, BIAS, 64>(k.rpl);
    case 128: return pick_rpl<TD, WD, BIAS, 128>(k.rpl);
    case 256: return pick_rpl<TD, WD, BIAS, 256>(k.rpl);
    default: return nullptr;
  }
}

template <int TD, int WD>
const void* pick_bias(const HeadKey& k) {
  return k.bias ? pick_dim<TD, WD, 1>(k) : pick_dim<TD, WD, 0>(k);
}

}  // namespace

const void* pick_head_kernel(const HeadKey& k) {
  if (k.t == kBF16 && k.w == kBF16) return pick_bias<kBF16, kBF16>(k);
  if (k.t == kBF16 && k.w == kF32) return pick_bias<kBF16, kF32>(k);
  if (k.t == kF32 && k.w == kBF16) return pick_bias<kF32, kBF16>(k);
  if (k.t == kF32 && k.w == kF32) return pick_bias<kF32, kF32>(k);
  return nullptr;
}

}  // namespace rn
