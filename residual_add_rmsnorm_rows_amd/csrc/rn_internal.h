// Internal declarations shared by the host-side selector, the C ABI and the
// kernel translation units.  Plain C++ (no HIP headers) so that the selector
// builds and runs on any host.
#pragma once

#include <stdint.h>

#include "rmsnorm_rows.h"

namespace rn {

// kFP4 is OCP fp4 e2m1 (outputs only, two codes per byte); kNone marks an
// absent residual.
enum DType : int { kBF16 = 0, kF32 = 1, kFP8 = 2, kNone = 3, kFP4 = 4 };

// Scale granularity of a quantized (fp8 / fp4) output.
enum QScheme : int {
  kQRow = 0,       // one float32 scale amax / 448 per row (fp8)
  kQGroup128 = 1,  // one float32 scale amax / 448 per 128 consecutive elements (fp8)
  kQMx32 = 2,      // OCP MX: one E8M0 scale per 32 consecutive elements (fp8 e4m3 or fp4 e2m1)
  kQNv16 = 3,      // NVFP4: one E4M3FN scale per 16 elements and a float32 tensor scale (fp4 e2m1)
};

// Partial inputs a rows-kernel launch can sum in front of the residual add.
constexpr int kMaxParts = 8;

// Kernel arguments of the rows kernel, passed by value as the only argument.
struct RowArgs {
  const void* x;
  const void* res;       // nullptr: no residual add
  const void* w;
  void* out;
  void* res_out;         // nullptr iff res is nullptr
  void* scale;           // quantized output only: float32 per row / per group, or E8M0 per block
  float* amax;           // quantized output only, may be nullptr: float32 amax per scale
  const float* tscale;   // NVFP4 only: the float32 tensor scale (one value, device memory)
  int64_t rows;
  int32_t hidden;        // elements per row
  float eps;
  // Kernels built for partial inputs (KP > 1) read x as the sum of
  // parts[0 .. num_parts) instead of x; the other slots are ignored.
  const void* parts[kMaxParts];
  int32_t num_parts;
};

// Kernel arguments of the per-head kernel.
struct HeadArgs {
  const void* q;
  const void* k;
  const void* qw;
  const void* kw;
  void* q_out;
  void* k_out;
  int64_t q_stride;      // elements between tokens
  int64_t k_stride;
  int32_t num_q_heads;
  int32_t num_heads;     // num_q_heads + num_k_heads
  int32_t total_rows;    // tokens * num_heads
  float eps;
};

// Kernel arguments of the SiLU-and-mul kernel.
struct ActArgs {
  const void* x;         // [rows, 2 d]: gate in [0, d), up in [d, 2 d)
  void* out;             // [rows, d]
  void* scale;           // quantized output only
  float* amax;           // quantized output only, may be nullptr
  const float* tscale;   // NVFP4 only: the float32 tensor scale
  int64_t rows;
  int32_t d;
};

// Everything the launcher needs to pick a compiled kernel.
struct RowKey {
  int x, res, w, out;  // res == kNone: no residual
  int qs;              // QScheme (kQRow unless the output is quantized)
  int bias;            // 0 or 1
  int nv;              // vectors per lane: 1, 2, 4, 8
  int kp;              // partial-input slots: 1 = x itself; 2, 4 or 8 = a sum of up to that many
};

struct ActKey {
  int x, out, qs;
  int nv;
};

struct HeadKey {
  int t, w;            // q/k dtype, weight dtype
  int bias;
  int head_dim;        // 64, 128, 256
  int rpl;             // heads per lane group: 1, 2, 4
};

// --- selector / validation (select.cpp, host only) -------------------------

// Thread-local message for rn_last_error(); returns `st` for convenience.
rn_status fail(rn_status st, const char* fmt, ...);
void clear_error();

// Checks flags/sizes (not pointers) of an rmsnorm call and fills key.{x,res,w,out,bias}.
rn_status check_row_shape(int64_t rows, int64_t hidden, uint32_t flags, bool has_residual,
                          RowKey* key);
// Selector: launch configuration for rows x hidden on num_cus compute units
// (key.kp > 1: the kernels that sum partial inputs, see kMaxPartsVecsPerLane).
rn_status select_row_config(int64_t rows, int64_t hidden, const RowKey& key, int num_cus,
                            rn_launch_config* cfg);
// Partial-input slots of the smallest kernel that sums num_parts inputs (2, 4 or 8).
int parts_slots(int num_parts);
// Checks an explicit configuration and fills the derived fields.
rn_status check_row_config(int64_t rows, int64_t hidden, const RowKey& key,
                           const rn_launch_config* in, rn_launch_config* out);

// SiLU-and-mul: flags (x dtype, out dtype, scale scheme) and sizes.
rn_status check_act_shape(int64_t rows, int64_t d, uint32_t flags, ActKey* key);
// Selector for the SiLU-and-mul kernel (same launch shapes as the rows kernel).
rn_status select_act_config(int64_t rows, int64_t d, const ActKey& key, int num_cus, rn_launch_config* cfg);

rn_status check_head_shape(int64_t tokens, int32_t nq, int32_t nk, int32_t head_dim,
                           uint32_t flags, HeadKey* key);
rn_status select_head_config(int64_t tokens, int32_t nq, int32_t nk, const HeadKey& key,
                             int num_cus, rn_launch_config* cfg);
// Checks an explicit per-head configuration (rows_per_lane, block_threads) and
// derives the grid.
rn_status check_head_config(int64_t tokens, int32_t nq, int32_t nk, const HeadKey& key,
                            const rn_launch_config* in, rn_launch_config* out);

constexpr int kMaxWavesPerRow = 16;
constexpr int kMaxVecsPerLane = 8;
constexpr int kHeadBlockThreads = 256;
constexpr int kCopyThreads = 512;  // reference copy: one 16-byte vector per lane, 8 KiB per workgroup

// Largest workgroup a rows-kernel variant is compiled for: holding 8 vectors
// per lane needs more than the 128 VGPRs a 1024-thread workgroup leaves each
// lane, so that variant is built for at most 8 waves (256 VGPRs per lane).
constexpr int max_threads_for_nv(int nv) { return nv >= 8 ? 512 : 1024; }

// Kernels that sum partial inputs keep every slot's loads in flight, so they
// are built for at most 2 vectors per lane (rows of up to 2048 lane vectors).
constexpr int kMaxPartsVecsPerLane = 2;

}  // namespace rn

// --- kernel pickers (defined in the kernel translation units) ----------------
// Each returns the address of the compiled kernel for `key`, or nullptr when
// that combination is not built.
namespace rn {
// rows_kernel.hip, compiled once per (x dtype, out dtype, scale scheme)
const void* pick_row_kernel_bf16_bf16(const RowKey& key);
const void* pick_row_kernel_bf16_f32(const RowKey& key);
const void* pick_row_kernel_bf16_fp8_row(const RowKey& key);
const void* pick_row_kernel_bf16_fp8_g128(const RowKey& key);
const void* pick_row_kernel_bf16_fp8_mx(const RowKey& key);
const void* pick_row_kernel_bf16_fp4_mx(const RowKey& key);
const void* pick_row_kernel_bf16_fp4_nv(const RowKey& key);
const void* pick_row_kernel_f32_bf16(const RowKey& key);
const void* pick_row_kernel_f32_f32(const RowKey& key);
const void* pick_row_kernel_f32_fp8_row(const RowKey& key);
const void* pick_row_kernel_f32_fp8_g128(const RowKey& key);
const void* pick_row_kernel_f32_fp8_mx(const RowKey& key);
const void* pick_row_kernel_f32_fp4_mx(const RowKey& key);
const void* pick_row_kernel_f32_fp4_nv(const RowKey& key);
// heads_kernel.hip
const void* pick_head_kernel(const HeadKey& key);
// act_kernel.hip
const void* pick_act_kernel(const ActKey& key);
// reference_kernels.hip
const void* empty_kernel_address();
const void* copy_kernel_address();
}  // namespace rn
