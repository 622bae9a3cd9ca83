// Host-side argument checks and launch-configuration selector.
//
// Plain C++ with no HIP dependency: everything here runs before the first
// HIP call of an entry point, so it is testable on a machine without a GPU.
//
// Selector rules (the page's "Prefill & decode specialization" section picks
// a per-thread vector giving 128-bit loads, then the number of warps, then a
// decode variant with one warp per block when there are fewer warps than SMs;
// this is the MI355X version of that idea, tuned by measurement and keyed on
// the token count as well as the row width and dtypes):
//   * vec = 16 bytes of x per lane (8 bf16 or 4 f32), one 16-byte buffer load;
//   * decode (rows <= compute units), norm kernels: the call is latency bound.
//     A row of at most 128 lane vectors stays in one wave (one or two vectors
//     per lane: no LDS and no barrier); a longer row is spread over at most 8
//     waves with the fewest vectors per lane that cover it.  Measured on
//     MI355X (graph launches, 1-256 rows): 1024 wide, 1 wave x 2 vectors beat
//     2 x 1 by 3-5%; 4096 wide, 8 x 1 took 2.7 us per call against 3.1 us for
//     one wave x 8 vectors; 8192 wide, 8 x 2 beat 16 x 1 by 5-8%.  SwiGLU
//     decode keeps the exact fit (see select_act_config);
//   * mid-size (compute units < rows <= 16 x compute units: chunked prefill,
//     large decode batches): a table per rows-per-CU bucket (kTunedMid,
//     kTunedActMid), falling back to the prefill tables;
//   * prefill: for the dtype classes and hidden sizes that were measured
//     (2048..16384 wide rows), the fastest variant of an interleaved sweep
//     from a table (kTuned; kTunedAct for SwiGLU); otherwise the exact fit
//     with the fewest vectors per lane, except for rows without a residual
//     (2 or 4 vectors per lane, by output width) and quantized outputs with
//     a residual of the x dtype (2 vectors per lane past 8 waves).  (With a residual and a
//     16/32-bit output, one extra partly idle wave often measured 0.5-2%
//     faster than the exact fit; with fp8 output or no residual the same
//     extra wave measured up to 25% slower, so the exact fit is the default);
//   * grid = rows (a workgroup per row; MI355X's dispatcher refills CUs as
//     workgroups finish, and persistent grids measured 1-7% slower).
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
    case kFP4: return "fp4_e2m1";
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
  const int o_code = (flags >> RN_FLAGS_OUT_SHIFT) & 3;
  const int qs = (flags >> RN_FLAGS_SCALE_SHIFT) & 3;
  if (x == 3 || w == 3 || (has_residual && r == 3))
    return fail(RN_ERR_INVALID_ARG, "dtype code 3 is not an input dtype (flags 0x%x)", flags);
  if (x == kFP8) return fail(RN_ERR_UNSUPPORTED, "x must be bf16 or f32");
  if (w == kFP8) return fail(RN_ERR_UNSUPPORTED, "weight must be bf16 or f32");
  const int o = o_code == 3 ? kFP4 : o_code;
  const bool quant = o == kFP8 || o == kFP4;
  if (!quant && qs != kQRow)
    return fail(RN_ERR_INVALID_ARG, "a scale granularity needs an fp8 or fp4 output");
  if (o == kFP4 && qs != kQMx32 && qs != kQNv16)
    return fail(RN_ERR_UNSUPPORTED, "fp4 e2m1 output takes MX (RN_SCALE_MX32) or NVFP4 (RN_SCALE_NV16) scales");
  if (qs == kQNv16 && o != kFP4)
    return fail(RN_ERR_UNSUPPORTED, "NVFP4 scales (RN_SCALE_NV16) are for fp4 e2m1 output only");
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
  if (qs == kQGroup128 && hidden % 128 != 0)
    return fail(RN_ERR_UNSUPPORTED, "hidden (%lld) must be a multiple of 128 for per-128 scales",
                (long long)hidden);
  if (qs == kQMx32 && hidden % 32 != 0)
    return fail(RN_ERR_UNSUPPORTED, "hidden (%lld) must be a multiple of 32 for MX scales", (long long)hidden);
  if (qs == kQNv16 && hidden % 16 != 0)
    return fail(RN_ERR_UNSUPPORTED, "hidden (%lld) must be a multiple of 16 for NVFP4 scales",
                (long long)hidden);
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
  key->qs = qs;
  key->bias = (flags & RN_FLAG_WEIGHT_PLUS_ONE) ? 1 : 0;
  key->nv = 0;
  key->kp = 1;
  return RN_OK;
}

int parts_slots(int num_parts) { return num_parts <= 2 ? 2 : num_parts <= 4 ? 4 : 8; }

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

static bool rows_variant_ok(int waves, int nv, int64_t nvec, int kp) {
  if (waves < 1 || waves > kMaxWavesPerRow) return false;
  if (nv != 1 && nv != 2 && nv != 4 && nv != 8) return false;
  if (kp > 1 && nv > kMaxPartsVecsPerLane) return false;
  if (64 * waves > max_threads_for_nv(nv)) return false;
  return (int64_t)64 * waves * nv >= nvec;
}

static const int64_t kMaxGrid = 0x7FFFFFFF;

// Fastest (waves, vectors per lane) measured on MI355X for prefill-sized row
// counts with a bf16 weight, where they beat the shape the rules below give.
// Every entry was re-timed against that shape in one interleaved run (five
// repetitions, median; the geometric mean of the times at 1.2 GB and 0.4 GB
// of traffic per call) and is kept where it won by at least 2% -- the box-to-
// box spread.  The shapes of the benchmark's own workloads were also timed
// at those workloads' sizes (nine interleaved repetitions) and are kept
// where they won there by at least 1%, that A/B's resolution: 4 x 4 for the
// 16384 x 8192 prefill with an f32 residual (+2.9%; earlier A/Bs +0.5% to
// +1.05%; 16 x 1 is within 0.8% of it at 2-16 rows per CU), and 8 x 2 for
// the 8192 x 7168 fp8 prefill (+1.45%: 8 waves fill a CU's 32 wave slots in
// 4 workgroups; the exact fit's 7 leave 4 idle).  The re-timing removed 31
// of 45 entries (17 chose the rules' own shape, 4 were slower than it, 10
// were within 2%); the 4 x 4 entry is new.
// Key: x dtype, residual dtype (kNone: no residual), whether the output is
// quantized (fp8 / fp4), hidden size.
struct Tuned {
  int x, res;
  bool fp8;
  int hidden;
  int waves, nv;
};
static const Tuned kTuned[] = {
    {kBF16, kF32, false, 5120, 11, 1}, {kBF16, kF32, false, 7168, 16, 1}, {kBF16, kF32, false, 8192, 4, 4},
    {kBF16, kF32, false, 12288, 16, 2},
    {kBF16, kBF16, false, 7168, 9, 2}, {kBF16, kBF16, true, 6144, 8, 2}, {kBF16, kBF16, true, 7168, 8, 2},
    {kBF16, kF32, true, 7168, 16, 1},
    {kBF16, kF32, true, 16384, 8, 4}, {kBF16, kNone, false, 2048, 3, 2}, {kBF16, kNone, false, 4096, 5, 2},
    {kBF16, kNone, false, 12288, 8, 4}, {kBF16, kNone, false, 16384, 8, 4}, {kF32, kF32, false, 4096, 9, 2},
    {kF32, kF32, false, 5120, 16, 2},
};

// Mid-size calls (more rows than compute units, at most 16 per CU: chunked
// prefill, large decode batches): fastest (waves, vectors per lane) measured
// on MI355X at 2, 4, 8 and 16 rows per CU.  Fewer waves holding more vectors
// per lane win here: with at most 16 rows per CU the whole grid is resident
// at once, and each lane keeps more loads in flight.  Every entry was
// re-timed at 3/4 of its bucket's largest row count against the shape the
// selector gives without it (kTuned's, else the rules'), in HIP graphs (GPU
// time; these calls take 3-40 us, where eager launches would time the
// launch path), scored by the geometric mean of a cache-warm call (one
// buffer set) and a cold one (buffers rotated past the 256 MB Infinity
// Cache), five interleaved repetitions; kept where it won by at least 2%
// (55 of 80; most by 4-28%).  Key as kTuned, plus cu_mult: the entry serves
// rows in ((cu_mult / 2) * CUs, cu_mult * CUs].
struct TunedMid {
  int x, res;
  bool fp8;
  int hidden;
  int cu_mult;
  int waves, nv;
};
static const TunedMid kTunedMid[] = {
    {kBF16, kBF16, false, 2048, 8, 1, 4}, {kBF16, kBF16, false, 4096, 4, 1, 8}, {kBF16, kBF16, false, 4096, 8, 1, 8},
    {kBF16, kBF16, false, 5120, 4, 2, 8}, {kBF16, kBF16, false, 5120, 8, 8, 2}, {kBF16, kBF16, false, 7168, 4, 2, 8},
    {kBF16, kBF16, false, 8192, 2, 8, 2}, {kBF16, kBF16, false, 8192, 4, 2, 8}, {kBF16, kBF16, false, 8192, 8, 2, 8},
    {kBF16, kBF16, false, 12288, 4, 3, 8}, {kBF16, kBF16, false, 16384, 4, 4, 8}, {kBF16, kF32, false, 2048, 4, 1, 4},
    {kBF16, kF32, false, 2048, 8, 1, 4}, {kBF16, kF32, false, 4096, 4, 1, 8}, {kBF16, kF32, false, 5120, 4, 2, 8},
    {kBF16, kF32, false, 7168, 4, 2, 8}, {kBF16, kF32, false, 12288, 2, 3, 8}, {kBF16, kBF16, true, 5120, 8, 8, 2},
    {kBF16, kBF16, true, 16384, 2, 4, 8}, {kBF16, kF32, true, 2048, 4, 1, 4}, {kBF16, kF32, true, 2048, 8, 1, 4},
    {kBF16, kF32, true, 4096, 4, 2, 4}, {kBF16, kF32, true, 4096, 8, 1, 8}, {kBF16, kF32, true, 5120, 4, 2, 8},
    {kBF16, kF32, true, 7168, 4, 2, 8}, {kBF16, kF32, true, 8192, 2, 4, 4}, {kBF16, kF32, true, 8192, 4, 2, 8},
    {kBF16, kNone, false, 2048, 2, 1, 4}, {kBF16, kNone, false, 2048, 4, 1, 4}, {kBF16, kNone, false, 2048, 8, 2, 2},
    {kBF16, kNone, false, 2048, 16, 1, 4}, {kBF16, kNone, false, 4096, 2, 8, 1}, {kBF16, kNone, false, 4096, 4, 1, 8},
    {kBF16, kNone, false, 4096, 8, 1, 8}, {kBF16, kNone, false, 5120, 2, 3, 4}, {kBF16, kNone, false, 5120, 8, 3, 4},
    {kBF16, kNone, false, 7168, 4, 2, 8}, {kBF16, kNone, false, 8192, 2, 4, 4}, {kBF16, kNone, false, 8192, 4, 2, 8},
    {kBF16, kNone, false, 8192, 8, 2, 8}, {kBF16, kNone, false, 12288, 2, 3, 8}, {kBF16, kNone, false, 12288, 4, 3, 8},
    {kBF16, kNone, false, 16384, 2, 4, 8}, {kF32, kF32, false, 2048, 2, 1, 8}, {kF32, kF32, false, 2048, 4, 1, 8},
    {kF32, kF32, false, 2048, 8, 1, 8}, {kF32, kF32, false, 4096, 2, 2, 8}, {kF32, kF32, false, 4096, 4, 2, 8},
    {kF32, kF32, false, 4096, 8, 2, 8}, {kF32, kF32, false, 5120, 2, 3, 8}, {kF32, kF32, false, 5120, 4, 5, 4},
    {kF32, kF32, false, 7168, 2, 4, 8}, {kF32, kF32, false, 7168, 4, 4, 8}, {kF32, kF32, false, 8192, 2, 4, 8},
    {kF32, kF32, false, 8192, 4, 4, 8},
};

// SwiGLU (bf16 x): fastest (waves, vectors per lane) measured on MI355X,
// re-timed like kTuned against the exact fit and kept where it won by at
// least 2% (15 of 21; fp4 outputs by 4-9%), plus, as for kTuned, the
// benchmark workload's 14336-wide shapes, which won at its own size
// (8192 tokens): 13 x 4 for bf16 out (+1.1%), 9 x 4 for fp8 (+1.9%).
// Output class: 0 bf16 / f32, 1 fp8 (measured with MX scales), 2 fp4
// (measured with NVFP4 scales).
struct TunedAct {
  int out_class;
  int d;
  int waves, nv;
};
static const TunedAct kTunedAct[] = {
    {0, 14336, 13, 4}, {1, 14336, 9, 4},
    {0, 4096, 9, 1}, {0, 8192, 12, 2}, {0, 11008, 14, 2}, {0, 18944, 14, 4}, {0, 28672, 16, 4},
    {1, 13824, 9, 4}, {2, 8192, 8, 2}, {2, 11008, 6, 4}, {2, 13824, 4, 8}, {2, 14336, 4, 8},
    {0, 6144, 13, 1}, {0, 27648, 16, 4}, {2, 5632, 4, 4}, {2, 8960, 5, 4}, {2, 9728, 6, 4},
};

// SwiGLU mid-size calls (CUs < rows <= 16 x CUs), re-timed and kept as
// kTunedMid (27 of 33, against kTunedAct's shape or the exact fit).
struct TunedActMid {
  int out_class;
  int d;
  int cu_mult;
  int waves, nv;
};
static const TunedActMid kTunedActMid[] = {
    {0, 4096, 8, 1, 8}, {0, 8192, 2, 8, 2}, {0, 8192, 4, 2, 8}, {0, 8192, 8, 8, 2},
    {0, 11008, 4, 6, 4}, {0, 13824, 4, 16, 2}, {0, 13824, 8, 16, 2}, {0, 14336, 4, 16, 2},
    {0, 14336, 8, 16, 2}, {0, 18944, 2, 12, 4}, {1, 11008, 4, 6, 4}, {1, 13824, 2, 16, 2},
    {1, 13824, 4, 8, 4}, {1, 13824, 8, 8, 4}, {1, 13824, 16, 8, 4}, {1, 14336, 4, 8, 4},
    {1, 18944, 2, 12, 4}, {1, 18944, 4, 12, 4}, {2, 8192, 2, 16, 1}, {2, 11008, 2, 12, 2},
    {2, 13824, 2, 15, 2}, {2, 13824, 4, 7, 4}, {2, 13824, 8, 8, 4}, {2, 13824, 16, 8, 4},
    {2, 14336, 2, 16, 2}, {2, 14336, 4, 7, 4}, {2, 14336, 8, 8, 4},
};

// Launch shape for rows of `hidden` elements: the tabulated (waves, nv) when
// given (tw > 0) and valid for a prefill-sized call; for a decode-sized call
// with `compact_decode`, the decode rule above; else the exact fit with the
// fewest vectors per lane.
static rn_status select_rows_shape(int64_t rows, int64_t hidden, const RowKey& key, int num_cus, int tw,
                                   int tnv, bool compact_decode, rn_launch_config* cfg) {
  if (num_cus < 1) return fail(RN_ERR_INVALID_ARG, "num_cus must be >= 1");
  const int vec = 16 / (key.x == kBF16 ? 2 : 4);
  const int64_t nvec = hidden / vec;
  const int choices[4] = {1, 2, 4, 8};
  int waves = 0, nv = 0;
  if (rows > num_cus && tw > 0 && rows_variant_ok(tw, tnv, nvec, key.kp)) {
    waves = tw;
    nv = tnv;
  }
  // decode (rows <= CUs, latency bound): one wave for rows of at most 128
  // vectors, else at most 8 waves with the fewest vectors per lane
  if (!nv && rows <= num_cus && compact_decode) {
    for (int f : choices) {
      const int64_t w = nvec <= 128 ? 1 : (nvec + 64 * f - 1) / (64 * f) < 8 ? (nvec + 64 * f - 1) / (64 * f) : 8;
      if (rows_variant_ok(static_cast<int>(w), f, nvec, key.kp)) {
        waves = static_cast<int>(w);
        nv = f;
        break;
      }
    }
  }
  // untabulated prefill shapes: the fewest vectors per lane, then the fewest
  // waves that cover the row
  for (int f : choices) {
    if (nv) break;
    int64_t w = (nvec + 64 * f - 1) / (64 * f);
    if (w < 1) w = 1;
    if (w <= kMaxWavesPerRow && rows_variant_ok(static_cast<int>(w), f, nvec, key.kp)) {
      waves = static_cast<int>(w);
      nv = f;
    }
  }
  if (!nv) return fail(RN_ERR_UNSUPPORTED, "no rows-kernel variant holds %lld lane vectors", (long long)nvec);
  fill_rows_cfg(vec, waves, nv, rows, rows < kMaxGrid ? rows : kMaxGrid, cfg);
  return RN_OK;
}

// Partial-input kernels (KP > 1, exact sums).  A sweep of every shape of up
// to 16 waves and 1-2 vectors per lane on MI355X (2, 4 and 8 bf16 partials;
// f32 or bf16 residual; bf16, per-row fp8 and MXFP4 outputs; 2048-16384 wide;
// 8-1024 rows and ~0.6 GB prefill calls; 150 cases) found the exact fit at
// one vector per lane best or within 3% in most cases, and no table needed:
//   * the exact fit at one vector per lane (two past 16 waves), at every
//     row count -- the exact sums give a lane more arithmetic than the
//     single-input kernel, so decode rows spread over up to 16 waves (16 x 1
//     beat 8 x 2 by 6-13% at 8 and 64 rows x 8192 with 4-8 partials);
//   * a fit of 9-15 waves, not a multiple of 4, with more than 2 rows per
//     CU: 8 waves x 2 vectors, which hold the row too.
// Against each case's best shape: geometric mean 1.003, worst 1.047 (the
// replaced table and rules: 1.026 and 1.225).  Every output type takes the
// same rule since the one-vector kernels all fit two 16-wave workgroups per
// CU (a second sweep: 6144-8192 wide, 384 rows to ~0.6 GB calls).
static rn_status select_parts_shape(int64_t rows, int64_t hidden, const RowKey& key, int num_cus,
                                    rn_launch_config* cfg) {
  if (num_cus < 1) return fail(RN_ERR_INVALID_ARG, "num_cus must be >= 1");
  const int vec = 16 / (key.x == kBF16 ? 2 : 4);
  const int64_t nvec = hidden / vec;
  int64_t w = (nvec + 63) / 64;
  int nv = 1;
  if (w > kMaxWavesPerRow) {
    w = (nvec + 127) / 128;
    nv = 2;
  }
  if (w > kMaxWavesPerRow)
    return fail(RN_ERR_UNSUPPORTED, "no partial-input variant holds %lld lane vectors", (long long)nvec);
  // One vector per lane over 9-15 waves, the count not a multiple of 4, past
  // 2 rows per CU: 8 x 2, which holds the row too (nvec <= 1024).  Measured
  // on MI355X with 2-8 partials and bf16, fp8 per-128 and MXFP4 outputs:
  // 14 x 1 ran up to 14% behind 8 x 2 there, while 12 x 1 and 16 x 1 ran
  // level with it or ahead (to 9%), and every exact fit was level or ahead
  // at up to 2 rows per CU.
  if (nv == 1 && w > 8 && w % 4 != 0 && rows > 2 * static_cast<int64_t>(num_cus)) {
    w = 8;
    nv = 2;
  }
  fill_rows_cfg(vec, static_cast<int>(w), nv, rows, rows < kMaxGrid ? rows : kMaxGrid, cfg);
  return RN_OK;
}

rn_status select_row_config(int64_t rows, int64_t hidden, const RowKey& key, int num_cus,
                            rn_launch_config* cfg) {
  if (key.kp > 1) return select_parts_shape(rows, hidden, key, num_cus, cfg);
  int tw = 0, tnv = 0;
  const bool quant = key.out == kFP8 || key.out == kFP4;
  // the tables were measured with a bf16 weight and a single x input
  if (key.w == kBF16 && key.kp == 1 && num_cus >= 1 && rows > num_cus) {
    int bucket = 0;  // rows per CU, rounded up to 2, 4, 8 or 16; 0 above that
    for (int b = 2; b <= 16; b *= 2) {
      if (rows <= static_cast<int64_t>(b) * num_cus) {
        bucket = b;
        break;
      }
    }
    for (const TunedMid& t : kTunedMid) {
      if (bucket && t.x == key.x && t.res == key.res && t.fp8 == quant && t.hidden == hidden && t.cu_mult == bucket) {
        tw = t.waves;
        tnv = t.nv;
        break;
      }
    }
    for (const Tuned& t : kTuned) {
      if (tw == 0 && t.x == key.x && t.res == key.res && t.fp8 == quant && t.hidden == hidden) {
        tw = t.waves;
        tnv = t.nv;
        break;
      }
    }
  }
  // Untabulated shapes whose exact fit at one vector per lane runs many
  // short waves take more vectors per lane and the fewest waves instead; the
  // fewer bytes one lane vector streams, the more vectors pay:
  //   * no residual, output narrower than x (fp8 / fp4, or f32 x to bf16):
  //     4 vectors per lane;
  //   * no residual, output as wide as x: 2 vectors per lane;
  //   * a quantized output with a residual of the x dtype, past 8 waves:
  //     2 vectors per lane;
  //   * with an f32 weight, a bf16 residual and bf16 output, past 8 waves:
  //     4 vectors per lane.
  // Swept at 1536-8192 wide with a bf16 weight: 1.26-1.70x for bf16 rows to
  // fp8 without a residual, 1.09-1.50x for f32 rows without one, 2-31% for
  // bf16 rows to bf16 without one, 6-14% (bf16) and 4-14% (f32) for the
  // quantized outputs; within 2.5% of each size's best shape (2.7% once).  With an f32
  // weight (2048-8192 wide): 1.10-1.58x, 1.02-1.27x and 1.04-1.16x for the
  // first three bf16 classes past the sizes the rule starts at, and 3-8% for
  // the last.  A wider output (bf16 x to f32 out without a residual)
  // measured 2-3% slower this way and keeps the exact fit, as do the other
  // classes (within 2% of their best).
  if (tw == 0 && key.kp == 1 && num_cus >= 1 && rows > num_cus) {
    const int64_t nvec = hidden / (key.x == kBF16 ? 8 : 4);
    const int xb = key.x == kBF16 ? 2 : 4;
    const int ob = key.out == kBF16 ? 2 : key.out == kF32 ? 4 : 1;
    int nv_rule = 0;
    if (key.res == kNone && nvec > 2 * 64) {
      if (quant || ob < xb) {
        nv_rule = 4;
      } else if (ob == xb) {
        nv_rule = 2;
      }
    } else if (key.res == key.x && quant && nvec > 8 * 64) {
      nv_rule = 2;
    } else if (key.w == kF32 && key.x == kBF16 && key.res == kBF16 && key.out == kBF16 && nvec > 8 * 64) {
      nv_rule = 4;
    }
    if (nv_rule) {
      const int64_t w = (nvec + 64 * nv_rule - 1) / (64 * nv_rule);
      if (w <= kMaxWavesPerRow && 64 * w <= max_threads_for_nv(nv_rule)) {
        tw = static_cast<int>(w);
        tnv = nv_rule;
      }
    }
  }
  return select_rows_shape(rows, hidden, key, num_cus, tw, tnv, true, cfg);
}

rn_status check_row_config(int64_t rows, int64_t hidden, const RowKey& key,
                           const rn_launch_config* in, rn_launch_config* out) {
  if (in == nullptr) return fail(RN_ERR_INVALID_ARG, "launch config is NULL");
  if (in->kernel != RN_KERNEL_ROWS) return fail(RN_ERR_INVALID_ARG, "config kernel must be RN_KERNEL_ROWS");
  const int vec = 16 / (key.x == kBF16 ? 2 : 4);
  const int64_t nvec = hidden / vec;
  if (!rows_variant_ok(in->waves_per_row, in->vecs_per_lane, nvec, key.kp))
    return fail(RN_ERR_INVALID_ARG, "config waves_per_row=%d vecs_per_lane=%d does not cover %lld "
                "lane vectors or is not built", in->waves_per_row, in->vecs_per_lane, (long long)nvec);
  if (in->grid < 1 || in->grid > kMaxGrid || (rows > 0 && in->grid > rows))
    return fail(RN_ERR_INVALID_ARG, "config grid %lld outside [1, rows]", (long long)in->grid);
  fill_rows_cfg(vec, in->waves_per_row, in->vecs_per_lane, rows > 0 ? rows : 1, in->grid, out);
  return RN_OK;
}

rn_status check_act_shape(int64_t rows, int64_t d, uint32_t flags, ActKey* key) {
  if (rows < 0) return fail(RN_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  if (d < 1) return fail(RN_ERR_INVALID_ARG, "d must be >= 1 (got %lld)", (long long)d);
  const uint32_t allowed = (3u << RN_FLAGS_X_SHIFT) | (3u << RN_FLAGS_OUT_SHIFT) | (3u << RN_FLAGS_SCALE_SHIFT);
  if (flags & ~allowed)
    return fail(RN_ERR_INVALID_ARG, "silu_mul flags 0x%x use bits other than x, out and scale", flags);
  // the output checks are those of the rows kernel (no residual, bf16 weight)
  RowKey rk;
  rn_status st = check_row_shape(rows, d, flags, false, &rk);
  if (st != RN_OK) return st;
  key->x = rk.x;
  key->out = rk.out;
  key->qs = rk.qs;
  key->nv = 0;
  return RN_OK;
}

rn_status select_act_config(int64_t rows, int64_t d, const ActKey& key, int num_cus, rn_launch_config* cfg) {
  RowKey rk;
  rk.x = key.x;
  rk.res = kNone;
  rk.w = kBF16;
  rk.out = key.out;
  rk.qs = key.qs;
  rk.bias = 0;
  rk.nv = 0;
  rk.kp = 1;
  int tw = 0, tnv = 0;
  if (key.x == kBF16 && num_cus >= 1 && rows > num_cus) {
    const int cls = key.out == kFP8 ? 1 : key.out == kFP4 ? 2 : 0;
    int bucket = 0;  // rows per CU, rounded up to 2, 4, 8 or 16; 0 above that
    for (int b = 2; b <= 16; b *= 2) {
      if (rows <= static_cast<int64_t>(b) * num_cus) {
        bucket = b;
        break;
      }
    }
    for (const TunedActMid& t : kTunedActMid) {
      if (bucket && t.out_class == cls && t.d == d && t.cu_mult == bucket) {
        tw = t.waves;
        tnv = t.nv;
        break;
      }
    }
    for (const TunedAct& t : kTunedAct) {
      if (tw == 0 && t.out_class == cls && t.d == d) {
        tw = t.waves;
        tnv = t.nv;
        break;
      }
    }
  }
  // SwiGLU decode keeps the exact fit: its rows load two tensors, and for
  // 11008 / 14336 wide rows at 1-64 tokens 11-16 waves x 2 vectors measured
  // 6-16% faster than the rows kernel's 8-wave cap
  return select_rows_shape(rows, d, rk, num_cus, tw, tnv, false, cfg);
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

static void fill_head_cfg(int64_t rows, int vec, int lanes, int rpl, int block,
                          rn_launch_config* cfg) {
  const int per_wave = 64 / lanes;
  const int64_t waves = (rows + (int64_t)per_wave * rpl - 1) / ((int64_t)per_wave * rpl);
  const int waves_per_block = block / 64;
  memset(cfg, 0, sizeof(*cfg));
  cfg->kernel = RN_KERNEL_HEADS;
  cfg->vec = vec;
  cfg->waves_per_row = 1;
  cfg->vecs_per_lane = 1;
  cfg->lanes_per_row = lanes;
  cfg->rows_per_lane = rpl;
  cfg->block_threads = block;
  cfg->grid = (waves + waves_per_block - 1) / waves_per_block;
  if (cfg->grid < 1) cfg->grid = 1;
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
  fill_head_cfg(rows, vec, lanes, rpl, kHeadBlockThreads, cfg);
  return RN_OK;
}

rn_status check_head_config(int64_t tokens, int32_t nq, int32_t nk, const HeadKey& key,
                            const rn_launch_config* in, rn_launch_config* out) {
  if (in == nullptr) return fail(RN_ERR_INVALID_ARG, "launch config is NULL");
  if (in->kernel != RN_KERNEL_HEADS) return fail(RN_ERR_INVALID_ARG, "config kernel must be RN_KERNEL_HEADS");
  if (in->rows_per_lane != 1 && in->rows_per_lane != 2 && in->rows_per_lane != 4)
    return fail(RN_ERR_INVALID_ARG, "config rows_per_lane must be 1, 2 or 4");
  if (in->block_threads != 64 && in->block_threads != 128 && in->block_threads != 256)
    return fail(RN_ERR_INVALID_ARG, "config block_threads must be 64, 128 or 256");
  const int vec = 16 / (key.t == kBF16 ? 2 : 4);
  const int64_t rows = tokens * ((int64_t)nq + nk);
  fill_head_cfg(rows > 0 ? rows : 1, vec, key.head_dim / vec, in->rows_per_lane, in->block_threads, out);
  return RN_OK;
}

}  // namespace rn
