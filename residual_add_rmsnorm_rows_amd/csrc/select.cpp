// Host-side argument checks and launch-configuration selector.
//
// Plain C++ with no HIP dependency: everything here runs before the first
// HIP call of an entry point, so it is testable on a machine without a GPU.
//
// Selector rules (the page's "Prefill & decode specialization" section picks
// a per-thread vector giving 128-bit loads, then the number of warps, then a
// decode variant with one warp per block when there are fewer warps than SMs;
// this is the MI355X version of that idea, tuned by measurement):
//   * vec = 16 bytes of x per lane (8 bf16 or 4 f32): global_load_dwordx4;
//   * decode shape (rows <= compute units): the data is small and the call is
//     latency bound, so a row is spread over as many waves as give each lane a
//     single vector (up to 16 waves; longer rows take 2, 4 or 8 vectors per
//     lane).  Measured on MI355X for 256 x 4096 bf16: 8 waves x 1 vector per
//     lane take 2.7 us per call against 4.5 us for one wave x 8 vectors;
//   * prefill shape: W waves share a row so that each lane holds
//     `prefill_vecs_per_lane` vectors (2), with W in 1..16; the variant with
//     the fewest idle lanes wins among equal choices;
//   * grid = rows (a workgroup per row; MI355X's dispatcher refills CUs as
//     workgroups finish, so no persistent loop is needed).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "rn_internal.h"

namespace rn {

namespace {
thread_local char g_err[512];
}  // namespace

rn_status fail(rn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = '\0'; }

const char* last_error() { return g_err; }

static const char* dt_name(int dt) {
  switch (dt) {
    case kBF16: return "bf16";
    case kF32: return "f32";
    case kFP8: return "fp8_e4m3fn";
    default: return "invalid";
  }
}

rn_status check_row_shape(int64_t rows, int64_t hidden, uint32_t flags, bool has_residual,
                          RowKey* key) {
  if (rows < 0) return fail(RN_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  if (hidden < 1) return fail(RN_ERR_INVALID_ARG, "hidden must be >= 1 (got %lld)", (long long)hidden);
  if (flags & ~RN_FLAGS_KNOWN_MASK)
    return fail(RN_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags & ~RN_FLAGS_KNOWN_MASK);
  const int x = (flags >> RN_FLAGS_X_SHIFT) & 3;
  const int r = (flags >> RN_FLAGS_RES_SHIFT) & 3;
  const int w = (flags >> RN_FLAGS_W_SHIFT) & 3;
  const int o = (flags >> RN_FLAGS_OUT_SHIFT) & 3;
  if (x == 3 || w == 3 || o == 3 || (has_residual && r == 3))
    return fail(RN_ERR_INVALID_ARG, "dtype code 3 is not a dtype (flags 0x%x)", flags);
  if (x == kFP8) return fail(RN_ERR_UNSUPPORTED, "x must be bf16 or f32");
  if (w == kFP8) return fail(RN_ERR_UNSUPPORTED, "weight must be bf16 or f32");
  int res = kNone;
  if (has_residual) {
    if (r == kFP8) return fail(RN_ERR_UNSUPPORTED, "residual must be bf16 or f32");
    if (r != x && r != kF32)
      return fail(RN_ERR_UNSUPPORTED, "residual dtype %s with x dtype %s is not built (residual is "
                  "the x dtype or f32)", dt_name(r), dt_name(x));
    res = r;
  }
  const int vec = 16 / (x == kBF16 ? 2 : 4);
  if (hidden % vec != 0)
    return fail(RN_ERR_UNSUPPORTED, "hidden (%lld) must be a multiple of %d for %s x (16-byte lane "
                "vectors)", (long long)hidden, vec, dt_name(x));
  const int64_t max_vecs = (int64_t)64 * kMaxVecsPerLane * (max_threads_for_nv(kMaxVecsPerLane) / 64);
  const int64_t max_vecs2 = (int64_t)64 * 4 * kMaxWavesPerRow;
  const int64_t cap = (max_vecs > max_vecs2 ? max_vecs : max_vecs2) * vec;
  if (hidden > cap)
    return fail(RN_ERR_UNSUPPORTED, "hidden (%lld) above the largest row held in registers (%lld "
                "for %s x)", (long long)hidden, (long long)cap, dt_name(x));
  key->x = x;
  key->res = res;
  key->w = w;
  key->out = o;
  key->bias = (flags & RN_FLAG_WEIGHT_PLUS_ONE) ? 1 : 0;
  key->nv = 0;
  return RN_OK;
}

static void fill_rows_cfg(int vec, int waves, int nv, int64_t rows, int64_t grid,
                          rn_launch_config* cfg) {
  memset(cfg, 0, sizeof(*cfg));
  cfg->kernel = RN_KERNEL_ROWS;
  cfg->vec = vec;
  cfg->waves_per_row = waves;
  cfg->vecs_per_lane = nv;
  cfg->lanes_per_row = 64 * waves;
  cfg->rows_per_lane = 1;
  cfg->block_threads = 64 * waves;
  cfg->grid = grid < rows ? grid : rows;
  if (cfg->grid < 1) cfg->grid = 1;
}

static bool rows_variant_ok(int waves, int nv, int64_t nvec) {
  if (waves < 1 || waves > kMaxWavesPerRow) return false;
  if (nv != 1 && nv != 2 && nv != 4 && nv != 8) return false;
  if (64 * waves > max_threads_for_nv(nv)) return false;
  return (int64_t)64 * waves * nv >= nvec;
}

// Smallest built vecs-per-lane that covers nvec with `waves` waves (0: none).
static int fit_nv(int waves, int64_t nvec) {
  const int choices[4] = {1, 2, 4, 8};
  for (int nv : choices)
    if (rows_variant_ok(waves, nv, nvec)) return nv;
  return 0;
}

static const int kPrefillVecsPerLane = 2;
static const int64_t kMaxGrid = 0x7FFFFFFF;

rn_status select_row_config(int64_t rows, int64_t hidden, const RowKey& key, int num_cus,
                            rn_launch_config* cfg) {
  if (num_cus < 1) return fail(RN_ERR_INVALID_ARG, "num_cus must be >= 1");
  const int vec = 16 / (key.x == kBF16 ? 2 : 4);
  const int64_t nvec = hidden / vec;
  int waves = 0, nv = 0;
  if (rows <= num_cus) {
    // decode: the fewest vectors per lane, then the fewest waves giving that
    const int choices[4] = {1, 2, 4, 8};
    for (int f : choices) {
      const int64_t w = (nvec + 64 * f - 1) / (64 * f);
      if (rows_variant_ok(static_cast<int>(w < 1 ? 1 : w), f, nvec)) {
        waves = static_cast<int>(w < 1 ? 1 : w);
        nv = f;
        break;
      }
    }
  } else {
    // prefill: about kPrefillVecsPerLane vectors per lane; among the waves
    // counts around that target, take the one with the fewest idle lanes.
    int64_t target = (nvec + 64 * kPrefillVecsPerLane - 1) / (64 * kPrefillVecsPerLane);
    if (target < 1) target = 1;
    if (target > kMaxWavesPerRow) target = kMaxWavesPerRow;
    int64_t best_idle = -1;
    for (int w = 1; w <= kMaxWavesPerRow; ++w) {
      if (w < target / 2 || w > 2 * target) continue;
      const int f = fit_nv(w, nvec);
      if (!f) continue;
      const int64_t idle = (int64_t)64 * w * f - nvec;
      // fewer idle lanes first, then closest to the target waves count
      const int64_t dist = w > target ? w - target : target - w;
      const int64_t score = idle * 64 + dist;
      if (best_idle < 0 || score < best_idle) {
        best_idle = score;
        waves = w;
        nv = f;
      }
    }
    if (!nv) {
      for (int w = 1; w <= kMaxWavesPerRow && !nv; ++w) {
        const int f = fit_nv(w, nvec);
        if (f) { waves = w; nv = f; }
      }
    }
  }
  if (!nv) return fail(RN_ERR_UNSUPPORTED, "no rows-kernel variant holds %lld lane vectors", (long long)nvec);
  fill_rows_cfg(vec, waves, nv, rows, rows < kMaxGrid ? rows : kMaxGrid, cfg);
  return RN_OK;
}

rn_status check_row_config(int64_t rows, int64_t hidden, const RowKey& key,
                           const rn_launch_config* in, rn_launch_config* out) {
  if (in == nullptr) return fail(RN_ERR_INVALID_ARG, "launch config is NULL");
  if (in->kernel != RN_KERNEL_ROWS) return fail(RN_ERR_INVALID_ARG, "config kernel must be RN_KERNEL_ROWS");
  const int vec = 16 / (key.x == kBF16 ? 2 : 4);
  const int64_t nvec = hidden / vec;
  if (!rows_variant_ok(in->waves_per_row, in->vecs_per_lane, nvec))
    return fail(RN_ERR_INVALID_ARG, "config waves_per_row=%d vecs_per_lane=%d does not cover %lld "
                "lane vectors or is not built", in->waves_per_row, in->vecs_per_lane, (long long)nvec);
  if (in->grid < 1 || in->grid > kMaxGrid || (rows > 0 && in->grid > rows))
    return fail(RN_ERR_INVALID_ARG, "config grid %lld outside [1, rows]", (long long)in->grid);
  fill_rows_cfg(vec, in->waves_per_row, in->vecs_per_lane, rows > 0 ? rows : 1, in->grid, out);
  return RN_OK;
}

rn_status check_head_shape(int64_t tokens, int32_t nq, int32_t nk, int32_t head_dim,
                           uint32_t flags, HeadKey* key) {
  if (tokens < 0) return fail(RN_ERR_INVALID_ARG, "tokens must be >= 0");
  if (nq < 1) return fail(RN_ERR_INVALID_ARG, "num_q_heads must be >= 1");
  if (nk < 0) return fail(RN_ERR_INVALID_ARG, "num_k_heads must be >= 0");
  const uint32_t allowed = (3u << RN_FLAGS_X_SHIFT) | (3u << RN_FLAGS_W_SHIFT) | RN_FLAG_WEIGHT_PLUS_ONE;
  if (flags & ~allowed) return fail(RN_ERR_INVALID_ARG, "qknorm flags 0x%x use bits other than x, w, plus-one", flags);
  const int t = (flags >> RN_FLAGS_X_SHIFT) & 3;
  const int w = (flags >> RN_FLAGS_W_SHIFT) & 3;
  if (t == 3 || w == 3) return fail(RN_ERR_INVALID_ARG, "dtype code 3 is not a dtype");
  if (t == kFP8 || w == kFP8) return fail(RN_ERR_UNSUPPORTED, "qknorm tensors and weights are bf16 or f32");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(RN_ERR_UNSUPPORTED, "head_dim %d not built (64, 128, 256)", head_dim);
  const int64_t heads = (int64_t)nq + nk;
  if (tokens > 0 && tokens * heads >= ((int64_t)1 << 31))
    return fail(RN_ERR_UNSUPPORTED, "tokens * heads must be < 2^31");
  key->t = t;
  key->w = w;
  key->bias = (flags & RN_FLAG_WEIGHT_PLUS_ONE) ? 1 : 0;
  key->head_dim = head_dim;
  key->rpl = 0;
  return RN_OK;
}

rn_status select_head_config(int64_t tokens, int32_t nq, int32_t nk, const HeadKey& key,
                             int num_cus, rn_launch_config* cfg) {
  if (num_cus < 1) return fail(RN_ERR_INVALID_ARG, "num_cus must be >= 1");
  const int vec = 16 / (key.t == kBF16 ? 2 : 4);
  const int lanes = key.head_dim / vec;
  const int per_wave = 64 / lanes;
  const int64_t rows = tokens * ((int64_t)nq + nk);
  const int waves_per_block = kHeadBlockThreads / 64;
  // Several heads per lane group keep more loads in flight per lane; with few
  // heads, one head per group spreads the work over more compute units.
  int rpl = 2;
  const int64_t waves2 = (rows + per_wave * 2 - 1) / (per_wave * 2);
  if (waves2 < (int64_t)num_cus * waves_per_block * 2) rpl = 1;
  const int64_t waves = (rows + (int64_t)per_wave * rpl - 1) / ((int64_t)per_wave * rpl);
  memset(cfg, 0, sizeof(*cfg));
  cfg->kernel = RN_KERNEL_HEADS;
  cfg->vec = vec;
  cfg->waves_per_row = 1;
  cfg->vecs_per_lane = 1;
  cfg->lanes_per_row = lanes;
  cfg->rows_per_lane = rpl;
  cfg->block_threads = kHeadBlockThreads;
  cfg->grid = (waves + waves_per_block - 1) / waves_per_block;
  if (cfg->grid < 1) cfg->grid = 1;
  return RN_OK;
}

}  // namespace rn
