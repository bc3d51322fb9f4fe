// ddtree_validate_inputs: a debug check of the index arrays a verify step is
// marshalled from.
//
// The marshalling mistakes it looks for are the ones "The 30-Column Mask:
// Debugging a Structural Marshaling Mismatch in Custom MLA Verification
// Attention" describes (sections "The Fix: Building Combined Indices" and
// "Mistakes and Incorrect Assumptions"): a KV index list that holds only the
// prefix slots while the mask expects prefix + tree columns, per-request
// offsets that do not line up, and slot ids outside the pool; plus offsets
// derived from the wrong length ("The Mask Bug That Changed Everything ...",
// section "The Context: A Cascade of Infrastructure and Algorithm
// Challenges") and parent links that do not point to an earlier node of the
// same tree.
//
// Three small launches: clear the report, check (grid-stride loops, one
// atomic count and one atomic minimum per violated check), then turn "no
// violation" minima into -1.  Every read is bounded by the host sizes, so
// the check itself cannot read out of bounds on the inputs it diagnoses.
#include <climits>

#include "common.h"

namespace {

enum Check { QO_INDPTR = 0, KV_INDPTR, KV_LEN, KV_INDEX, PARENT, NCHECK };
static_assert(NCHECK == DDTREE_NUM_CHECKS, "report layout");

__global__ void clear_kernel(int32_t* report) {
  const int k = threadIdx.x;
  if (k < NCHECK) {
    report[2 * k] = 0;
    report[2 * k + 1] = INT_MAX;
  }
}

__global__ void finish_kernel(int32_t* report) {
  const int k = threadIdx.x;
  if (k < NCHECK && report[2 * k + 1] == INT_MAX) report[2 * k + 1] = -1;
}

__device__ inline void flag(int32_t* report, int check, long long where) {
  atomicAdd(&report[2 * check], 1);
  atomicMin(&report[2 * check + 1], (int32_t)min(where, (long long)INT_MAX - 1));
}

// blockIdx.y = 0: per-request checks (qo / kv offsets, lengths) and the KV
// index range; blockIdx.y = 1 + r (r < bs): the parents of request r
__global__ __launch_bounds__(256) void check_kernel(int bs, const int32_t* __restrict__ qo,
                                                    int total_q, const int32_t* __restrict__ kvp,
                                                    const int32_t* __restrict__ kvi,
                                                    long long n_kvi, long long num_slots,
                                                    const int32_t* __restrict__ prefix_lens,
                                                    const int32_t* __restrict__ parents,
                                                    int32_t* report) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.y == 0) {
    for (long long r = tid; r < bs; r += stride) {
      const int q0 = qo[r], q1 = qo[r + 1], k0 = kvp[r], k1 = kvp[r + 1];
      if (q0 < 0 || q1 < q0 || q1 > total_q) flag(report, QO_INDPTR, r);
      if (k0 < 0 || k1 < k0 || k1 > n_kvi) flag(report, KV_INDPTR, r);
      const long long Q = (long long)q1 - q0, N = (long long)k1 - k0;
      if (N < Q || (prefix_lens && N != (long long)prefix_lens[r] + Q)) flag(report, KV_LEN, r);
    }
    for (long long j = tid; j < n_kvi; j += stride) {
      const int32_t s = kvi[j];
      if (s < 0 || s >= num_slots) flag(report, KV_INDEX, j);
    }
    return;
  }
  if (!parents) return;
  const int r = blockIdx.y - 1;
  // the request's node range, clamped to the array: a bad qo_indptr is
  // reported above and never makes this loop read outside [0, total_q)
  const int q0 = min(max(qo[r], 0), total_q);
  const int q1 = min(max(qo[r + 1], q0), total_q);
  for (long long c = tid; c < q1 - q0; c += stride) {
    const int p = parents[q0 + c];
    const bool ok = c == 0 ? p == -1 : (p >= 0 && p < c);
    if (!ok) flag(report, PARENT, q0 + c);
  }
}

}  // namespace

extern "C" int ddtree_validate_inputs(int bs, const int32_t* qo_indptr, int total_q,
                                      const int32_t* kv_indptr, const int32_t* kv_indices,
                                      int64_t num_kv_indices, int64_t num_slots,
                                      const int32_t* prefix_lens, const int32_t* node_parents,
                                      int32_t* report, void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(report, DDTREE_EINVAL, "validate_inputs: null report");
  DDTREE_REQUIRE(bs >= 0 && total_q >= 0 && num_kv_indices >= 0 && num_slots >= 0,
                 DDTREE_EINVAL, "validate_inputs: negative size");
  DDTREE_REQUIRE(bs == 0 || (qo_indptr && kv_indptr), DDTREE_EINVAL,
                 "validate_inputs: null indptr");
  DDTREE_REQUIRE(num_kv_indices == 0 || kv_indices, DDTREE_EINVAL,
                 "validate_inputs: null kv_indices");
  DDTREE_REQUIRE(bs < 65535, DDTREE_EUNSUPPORTED, "validate_inputs: bs above 65534");
  hipStream_t s = ddtree::as_stream(stream);
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(64), 0, s, report);
  int rc = ddtree::check_launch("validate_inputs");
  if (rc != DDTREE_OK) return rc;
  if (bs > 0) {
    const long long work = num_kv_indices > bs ? num_kv_indices : bs;
    const unsigned gx = (unsigned)min((work + 255) / 256, 1024LL);
    const unsigned gy = 1 + (node_parents ? (unsigned)bs : 0u);
    hipLaunchKernelGGL(check_kernel, dim3(gx, gy), dim3(256), 0, s, bs, qo_indptr, total_q,
                       kv_indptr, kv_indices, (long long)num_kv_indices, (long long)num_slots,
                       prefix_lens, node_parents, report);
    rc = ddtree::check_launch("validate_inputs");
    if (rc != DDTREE_OK) return rc;
  }
  hipLaunchKernelGGL(finish_kernel, dim3(1), dim3(64), 0, s, report);
  return ddtree::check_launch("validate_inputs");
}
