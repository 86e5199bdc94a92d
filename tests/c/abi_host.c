/* A plain C99 client of the C ABI (host-only calls, no device needed):
 * it must compile against include/hbmcoll.h as C and link against the
 * library.  Prints one line per fact; tests/test_c_abi.py compares them
 * with the Python binding's view of the same calls. */
#include <stdio.h>
#include <string.h>

#include "hbmcoll.h"

static int report(const char* what, hbmc_status_t st) {
  if (st != HBMC_OK) {
    printf("error %s %d %s\n", what, (int)st, hbmc_status_string(st));
    return 1;
  }
  return 0;
}

int main(void) {
  hbmc_comm_t ring = NULL, rhd = NULL, bad = NULL;
  int nsteps = 0, nitems = 0;
  uint64_t hbm = 0, recv = 0, bytes = 0;
  hbmc_exec_t mode = HBMC_EXEC_AUTO;
  if (report("create ring", hbmc_comm_create(8, HBMC_ALGO_RING, 0, 0, 0, &ring))) return 1;
  if (report("create rhd", hbmc_comm_create(5, HBMC_ALGO_RHD, 0, 0, 0, &rhd))) return 1;

  if (report("plan_info", hbmc_plan_info(ring, HBMC_COLL_ALLREDUCE, 0, (size_t)1 << 20, HBMC_FP32, &nsteps, &hbm, &recv)))
    return 1;
  printf("ring8 allreduce steps %d hbm %llu recv %llu\n", nsteps, (unsigned long long)hbm, (unsigned long long)recv);
  if (report("plan_info rhd", hbmc_plan_info(rhd, HBMC_COLL_ALLREDUCE, 0, 4096, HBMC_BF16, &nsteps, &hbm, NULL)))
    return 1;
  printf("rhd5 allreduce steps %d hbm %llu\n", nsteps, (unsigned long long)hbm);
  if (report("step_info", hbmc_plan_step_info(ring, HBMC_COLL_REDUCE_SCATTER, 0, 1000, HBMC_INT32, 0, &nitems, &hbm)))
    return 1;
  printf("ring8 reduce_scatter step0 items %d hbm %llu\n", nitems, (unsigned long long)hbm);

  if (report("exec_choice", hbmc_exec_choice(ring, HBMC_COLL_ALLREDUCE, 0, 4096, HBMC_FP16, 0, 0, &mode))) return 1;
  printf("ring8 allreduce 4096 fp16 form %d\n", (int)mode);
  if (report("exec_bytes", hbmc_exec_bytes(ring, HBMC_COLL_ALLREDUCE, 0, 4096, HBMC_FP16, 0, 0, HBMC_EXEC_REGS, &bytes)))
    return 1;
  printf("ring8 allreduce 4096 fp16 regs bytes %llu\n", (unsigned long long)bytes);

  /* argument checks come back as status codes */
  printf("create P=0 -> %d\n", (int)hbmc_comm_create(0, HBMC_ALGO_RING, 0, 0, 0, &bad));
  printf("pipeline S*M != P -> %d\n", (int)hbmc_comm_create(8, HBMC_ALGO_PIPELINE, 3, 2, 0, &bad));
  printf("set_exec_mode 99 -> %d\n", (int)hbmc_comm_set_exec_mode(ring, (hbmc_exec_t)99));
  printf("allreduce null bufs -> %d\n",
         (int)hbmc_allreduce(ring, NULL, 16, HBMC_FP32, HBMC_SUM, NULL));
  printf("status 1 %s\n", hbmc_status_string(HBMC_ERR_INVALID_ARG));

  if (report("destroy", hbmc_comm_destroy(ring)) || report("destroy", hbmc_comm_destroy(rhd))) return 1;
  printf("done\n");
  return 0;
}
