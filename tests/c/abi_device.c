/* A plain C99 client of the C ABI on the device, with no Python and no
 * torch: rank buffers from hipMalloc, hbmc_allreduce / hbmc_reduce_scatter on
 * the null stream, results compared with exact integer references computed
 * here (wrapping int32 sum, int8 max).  Prints one line per case and "ok" at
 * the end; exits non-zero on the first mismatch or error. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hbmcoll.h"

#define MAXP 16

static uint64_t lcg(uint64_t* s) {
  *s = *s * 6364136223846793005ull + 1442695040888963407ull;
  return *s >> 33;
}

/* One AllReduce (or the ring's reduce-scatter: only each rank's own segment
 * checked) of P rank buffers of L elements; returns 0 when exact. */
static int run_case(int P, hbmc_algo_t algo, hbmc_coll_t coll, hbmc_dtype_t dtype, hbmc_op_t op, size_t L,
                    hbmc_exec_t form) {
  const size_t e = dtype == HBMC_INT32 ? 4 : 1;
  void* host[MAXP];
  void* dev[MAXP];
  uint64_t seed = 12345u + (uint64_t)P * 7u + L;
  hbmc_comm_t comm = NULL;
  hbmc_exec_t chosen = HBMC_EXEC_STEPS;
  int bad = 0;
  if (hbmc_comm_create(P, algo, 0, 0, 0, &comm) != HBMC_OK) return 1;
  if (hbmc_comm_set_exec_mode(comm, form) != HBMC_OK) return 1;
  if (hbmc_exec_choice(comm, coll, 0, L, dtype, 0, 0, &chosen) != HBMC_OK) return 1;
  for (int r = 0; r < P; ++r) {
    host[r] = malloc(L * e);
    for (size_t i = 0; i < L; ++i) {
      const int64_t v = (int64_t)(lcg(&seed) % 2001u) - 1000;
      if (dtype == HBMC_INT32) ((int32_t*)host[r])[i] = (int32_t)(v * 997);
      else ((int8_t*)host[r])[i] = (int8_t)(v % 128);
    }
    if (hipMalloc(&dev[r], L * e) != hipSuccess || hipMemcpy(dev[r], host[r], L * e, hipMemcpyHostToDevice) != hipSuccess)
      return 1;
  }
  hbmc_status_t st = coll == HBMC_COLL_ALLREDUCE ? hbmc_allreduce(comm, dev, L, dtype, op, NULL)
                                                 : hbmc_reduce_scatter(comm, dev, L, dtype, op, NULL);
  if (st != HBMC_OK || hipDeviceSynchronize() != hipSuccess) {
    printf("error: status %d\n", (int)st);
    return 1;
  }
  /* the exact reference */
  const size_t q = (L + (size_t)P - 1) / (size_t)P;  /* the ceiling split of the ring */
  for (int r = 0; r < P && !bad; ++r) {
    unsigned char* got = malloc(L * e);
    if (hipMemcpy(got, dev[r], L * e, hipMemcpyDeviceToHost) != hipSuccess) return 1;
    size_t lo = 0, hi = L;
    if (coll == HBMC_COLL_REDUCE_SCATTER) {
      lo = (size_t)r * q < L ? (size_t)r * q : L;
      hi = lo + q < L ? lo + q : L;
    }
    for (size_t i = lo; i < hi && !bad; ++i) {
      if (dtype == HBMC_INT32) {
        uint32_t acc = 0;
        for (int s = 0; s < P; ++s) acc += (uint32_t)((int32_t*)host[s])[i];
        if (((uint32_t*)got)[i] != acc) bad = 1;
      } else {
        int8_t m = -128;
        for (int s = 0; s < P; ++s)
          if (((int8_t*)host[s])[i] > m) m = ((int8_t*)host[s])[i];
        if (((int8_t*)got)[i] != m) bad = 1;
      }
      if (bad) printf("mismatch: rank %d element %zu\n", r, i);
    }
    free(got);
  }
  printf("case P=%d algo=%d coll=%d dtype=%d L=%zu form=%d -> %s\n", P, (int)algo, (int)coll, (int)dtype, L,
         (int)chosen, bad ? "MISMATCH" : "exact");
  for (int r = 0; r < P; ++r) {
    (void)hipFree(dev[r]);
    free(host[r]);
  }
  if (hbmc_comm_destroy(comm) != HBMC_OK) return 1;
  return bad;
}

int main(void) {
  int fail = 0;
  fail |= run_case(8, HBMC_ALGO_RING, HBMC_COLL_ALLREDUCE, HBMC_INT32, HBMC_SUM, 100003, HBMC_EXEC_AUTO);
  fail |= run_case(8, HBMC_ALGO_RING, HBMC_COLL_ALLREDUCE, HBMC_INT32, HBMC_SUM, 100003, HBMC_EXEC_STEPS);
  fail |= run_case(5, HBMC_ALGO_RHD, HBMC_COLL_ALLREDUCE, HBMC_INT8, HBMC_MAX, 4099, HBMC_EXEC_AUTO);
  fail |= run_case(16, HBMC_ALGO_RHD, HBMC_COLL_ALLREDUCE, HBMC_INT32, HBMC_SUM, (size_t)3 << 20, HBMC_EXEC_AUTO);
  fail |= run_case(6, HBMC_ALGO_RING, HBMC_COLL_REDUCE_SCATTER, HBMC_INT32, HBMC_SUM, 77777, HBMC_EXEC_AUTO);
  fail |= run_case(7, HBMC_ALGO_RING, HBMC_COLL_ALLREDUCE, HBMC_INT8, HBMC_MAX, 5001, HBMC_EXEC_FLOW);
  printf(fail ? "failed\n" : "ok\n");
  return fail;
}
