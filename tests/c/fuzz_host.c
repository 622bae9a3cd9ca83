/* Randomized host-side calls of the C ABI (C99), meant to run under
 * AddressSanitizer and UBSan: the configuration queries and the argument checks
 * of the rows (also through the call record), partial-input, SwiGLU and
 * per-head entry points, with random sizes, flags, counts and explicit
 * configurations.  Every pointer is a fake, never-dereferenced address.  No
 * call can reach a kernel launch: every explicit configuration has
 * grid = rows + 1 and every call record a residual without residual_out,
 * which the checks reject (and rows == 0 returns before launching), so this
 * is safe on a machine with a GPU and needs none.  Checks that every configuration the queries accept
 * covers the row.  Exit status 0 on success. */
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include "rmsnorm_rows.h"
static uint64_t s = 88172645463325252ull;  /* xorshift64 state */
static uint64_t rnd(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }
int main(void) {
  rn_launch_config cfg;
  long counts[5] = {0};
  for (int i = 0; i < 200000; ++i) {
    int64_t rows = (int64_t)(rnd() % 70000) - 5;
    int64_t hidden = (int64_t)(rnd() % 40000) - 5;
    if (rnd() % 4 == 0) hidden = (hidden / 16) * 16;
    uint32_t flags = (uint32_t)(rnd() & 0xFFF);
    int32_t cus = (int32_t)(rnd() % 300) + 1;
    rn_status st = rmsnorm_query_config(rows, hidden, flags, (int32_t)(rnd() & 1), cus, &cfg);
    counts[st]++;
    if (st == RN_OK) {
      if ((int64_t)64 * cfg.waves_per_row * cfg.vecs_per_lane * cfg.vec < hidden) { printf("coverage bug %lld %lld\n", (long long)rows, (long long)hidden); return 1; }
      if (cfg.block_threads > (cfg.vecs_per_lane == 8 ? 512 : 1024)) { printf("threads bug\n"); return 1; }
    }
    st = silu_mul_query_config(rows, hidden, flags & 0x6C3u, cus, &cfg);
    if (st == RN_OK && (int64_t)64 * cfg.waves_per_row * cfg.vecs_per_lane * cfg.vec < hidden) { printf("act coverage bug\n"); return 1; }
    int32_t nq = (int32_t)(rnd() % 70) - 2, nk = (int32_t)(rnd() % 20) - 2, D = (int32_t)(rnd() % 300);
    if (rnd() % 2) D = 64 << (rnd() % 3);
    st = qknorm_query_config(rows, nq, nk, D, flags & 0x133u, cus, &cfg);
    /* explicit configuration with fake pointers: grid = rows + 1 is always rejected */
    rn_launch_config c = {0, 0, (int32_t)(rnd() % 20) - 2, 1 << (rnd() % 5), 0, 0, 0, 0, rows + 1};
    rmsnorm_fwd_config((void*)0x1000, NULL, (void*)0x1000, (void*)0x2000, NULL, NULL, NULL, NULL, rows, hidden, 1e-6f,
                       flags, &c, NULL);
    /* the call record: a residual without residual_out is always rejected (rows == 0 returns first) */
    rn_rmsnorm_call rec = {(void*)0x1000, (void*)0x3000, (void*)0x1000, (void*)0x2000, NULL, NULL, NULL, NULL,
                           rows, hidden, 1e-6f, flags, NULL};
    if (rmsnorm_fwd_call(&rec) == RN_OK && rows != 0) { printf("call record bug\n"); return 1; }
    if (rmsnorm_fwd_call(NULL) != RN_ERR_INVALID_ARG) { printf("call record NULL bug\n"); return 1; }
    /* partial inputs: random counts (including out of range), explicit configs, queries */
    const void* parts[9] = {(void*)0x10000, (void*)0x20000, (void*)0x30000, (void*)0x40000, (void*)0x50000,
                            (void*)0x60000, (void*)0x70000, (void*)0x80000, (void*)0x90000};
    int32_t np = (int32_t)(rnd() % 12) - 2;
    st = rmsnorm_partials_query_config(rows, hidden, np, flags, (int32_t)(rnd() & 1), cus, &cfg);
    if (st == RN_OK && ((int64_t)64 * cfg.waves_per_row * cfg.vecs_per_lane * cfg.vec < hidden ||
                        (np > 1 && cfg.vecs_per_lane > 2))) { printf("partials cfg bug\n"); return 1; }
    rmsnorm_fwd_partials_config(np > 9 || np < 0 ? NULL : parts, np, NULL, (void*)0x1000, (void*)0x2000, NULL, NULL,
                                NULL, NULL, rows, hidden, 1e-6f, flags, &c, NULL);
  }
  printf("fuzz ok: %ld ok, %ld invalid, %ld unsupported, %ld misaligned, %ld hip\n", counts[0], counts[1], counts[2], counts[3], counts[4]);
  return 0;
}
