/*
 * A C99 consumer of libvcoll's C ABI, with no Python and no torch: the
 * 4-device worked example of "Networks and Collective Communication"
 * (section 4.1; device d holds [10d, 10d+1, 10d+2, 10d+3]) through the ring
 * all-reduce, reduce-scatter and all-gather, and the ring ledger through the
 * two-call convention. Prints "OK" and exits 0 when every check holds.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "vcoll.h"

#define P 4
#define N 4

static int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

static int check(vcoll_status s, const char* what) {
  if (s != VCOLL_OK) {
    fprintf(stderr, "%s: %s\n", what, vcoll_status_str(s));
    return 1;
  }
  return 0;
}

int main(void) {
  float host[P][N], out[P][N], rs_host[P];
  void* send[P];
  void* recv[P];
  void* rs[P];
  void* ag[P];
  int r, i, bad = 0;
  if (vcoll_abi_version() != VCOLL_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", vcoll_abi_version(), VCOLL_ABI_VERSION);
    return 1;
  }
  for (r = 0; r < P; ++r) {
    for (i = 0; i < N; ++i) host[r][i] = (float)(10 * r + i);
    if (check_hip(hipMalloc(&send[r], sizeof(host[r])), "hipMalloc") ||
        check_hip(hipMalloc(&recv[r], sizeof(host[r])), "hipMalloc") ||
        check_hip(hipMalloc(&rs[r], sizeof(float)), "hipMalloc") ||
        check_hip(hipMalloc(&ag[r], sizeof(host[r])), "hipMalloc") ||
        check_hip(hipMemcpy(send[r], host[r], sizeof(host[r]), hipMemcpyHostToDevice), "hipMemcpy"))
      return 1;
  }
  if (check(vcoll_allreduce(VCOLL_RING, P, N, VCOLL_F32, (const void* const*)send, recv, NULL), "allreduce") ||
      check(vcoll_reduce_scatter(VCOLL_RING, P, N, VCOLL_F32, (const void* const*)send, rs, NULL), "reduce_scatter") ||
      check(vcoll_all_gather(VCOLL_RING, P, 1, VCOLL_F32, (const void* const*)rs, ag, NULL), "all_gather") ||
      check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize"))
    return 1;
  for (r = 0; r < P; ++r) {
    if (check_hip(hipMemcpy(out[r], recv[r], sizeof(out[r]), hipMemcpyDeviceToHost), "hipMemcpy") ||
        check_hip(hipMemcpy(&rs_host[r], rs[r], sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy"))
      return 1;
    for (i = 0; i < N; ++i)
      if (out[r][i] != (float)(60 + 4 * i)) {
        fprintf(stderr, "all-reduce rank %d element %d: %g\n", r, i, out[r][i]);
        bad = 1;
      }
    if (rs_host[r] != (float)(60 + 4 * r)) {
      fprintf(stderr, "reduce-scatter rank %d: %g\n", r, rs_host[r]);
      bad = 1;
    }
    if (check_hip(hipMemcpy(out[r], ag[r], sizeof(out[r]), hipMemcpyDeviceToHost), "hipMemcpy")) return 1;
    for (i = 0; i < N; ++i)
      if (out[r][i] != (float)(60 + 4 * i)) {
        fprintf(stderr, "all-gather of the reduce-scatter, rank %d element %d: %g\n", r, i, out[r][i]);
        bad = 1;
      }
  }
  {
    int64_t n_msgs = 0, sent[P], got[P];
    int32_t steps = 0;
    vcoll_msg* msgs;
    if (check(vcoll_ledger(VCOLL_OP_ALLREDUCE, VCOLL_RING, P, N, VCOLL_F32, NULL, 0, NULL, 0, &n_msgs, NULL, NULL,
                           NULL), "ledger size"))
      return 1;
    msgs = (vcoll_msg*)malloc(sizeof(vcoll_msg) * (size_t)n_msgs);
    if (!msgs ||
        check(vcoll_ledger(VCOLL_OP_ALLREDUCE, VCOLL_RING, P, N, VCOLL_F32, NULL, 0, msgs, n_msgs, &n_msgs, sent, got,
                           &steps), "ledger"))
      return 1;
    /* 2(p-1) steps, p messages each, one 4-byte element per message */
    if (n_msgs != 2 * (P - 1) * P || steps != 2 * (P - 1)) {
      fprintf(stderr, "ledger: %lld messages, %d steps\n", (long long)n_msgs, (int)steps);
      bad = 1;
    }
    for (r = 0; r < P; ++r)
      if (sent[r] != 2 * (P - 1) * 4 || got[r] != 2 * (P - 1) * 4) {
        fprintf(stderr, "ledger rank %d: sent %lld received %lld\n", r, (long long)sent[r], (long long)got[r]);
        bad = 1;
      }
    free(msgs);
  }
  for (r = 0; r < P; ++r) {
    hipFree(send[r]);
    hipFree(recv[r]);
    hipFree(rs[r]);
    hipFree(ag[r]);
  }
  if (bad) return 1;
  printf("OK\n");
  return 0;
}
