// ddtree_accept: greedy root walk along the target argmax, one wavefront per
// request.  Each step the lanes look among the request's nodes for a child of
// the current node whose token equals the target's prediction there, and the
// smallest such index wins ("The DDTree CUDA Graph Fix ...", section "The
// DDTree Architecture: Confirming Multiple-Path Evaluation"): for trees of up
// to 128 nodes over registers loaded once (two ballots a step), for larger
// ones by a scan of memory and a wave minimum.
// The walk ends when no child matches or after depth_max + 1 path nodes; the
// bonus is the prediction at the last accepted node ("The Oracle Drafter
// ...", sections "The Engine Interface Design" and "Reasoning About Cache
// Positions and Token Indices").
#include <climits>

#include "common.h"

namespace {

__global__ __launch_bounds__(64) void accept_kernel(
    const int32_t* __restrict__ tok, const int32_t* __restrict__ par,
    const int32_t* __restrict__ qo, const int32_t* __restrict__ pred, int D,
    int32_t* __restrict__ acc_nodes, int32_t* __restrict__ acc_len,
    int32_t* __restrict__ commit, int32_t* __restrict__ bonus) {
  extern __shared__ int path[];  // [D + 1]
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int base = qo[r];
  const int Q = qo[r + 1] - base;
  const size_t row = (size_t)r * (D + 1);
  if (Q < 1) {
    for (int k = lane; k <= D; k += 64) {
      acc_nodes[row + k] = -1;
      commit[row + k] = -1;
    }
    if (lane == 0) {
      acc_len[r] = 0;
      bonus[r] = -1;
    }
    return;
  }
  int cur = 0, len = 1;
  if (lane == 0) path[0] = 0;
  if (Q <= 128) {
    // Small trees: parents, tokens and predictions are read once into
    // registers (node j in lane j & 63, slot j >> 6), so each step is two
    // ballots instead of a round trip to memory.
    int p[2], t[2], pr[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = lane + 64 * q;
      const bool in = j < Q;
      p[q] = in ? par[base + j] : -2;
      t[q] = in ? tok[base + j] : 0;
      pr[q] = in ? pred[base + j] : 0;
    }
    auto at = [&](const int* v, int j) {  // node j's value, j wave-uniform
      return __builtin_amdgcn_readlane(j < 64 ? v[0] : v[1], j & 63);
    };
    while (len < D + 1) {
      const int want = at(pr, cur);
      // children of cur carrying the predicted token; the root is no child
      const uint64_t m0 = __ballot(lane > 0 && p[0] == cur && t[0] == want);
      const uint64_t m1 = __ballot(p[1] == cur && t[1] == want);
      if (!m0 && !m1) break;
      cur = m0 ? __ffsll((long long)m0) - 1 : 64 + __ffsll((long long)m1) - 1;
      if (lane == 0) path[len] = cur;
      ++len;
    }
  } else {
    while (len < D + 1) {
      const int t = pred[base + cur];
      int found = INT_MAX;
      for (int j = 1 + lane; j < Q; j += 64) {
        if (par[base + j] == cur && tok[base + j] == t) {
          found = j;
          break;  // smallest matching index of this lane's stride
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) found = min(found, __shfl_xor(found, off));
      if (found == INT_MAX) break;
      cur = found;
      if (lane == 0) path[len] = cur;
      ++len;
    }
  }
  __syncthreads();
  const int b = pred[base + cur];
  for (int k = lane; k <= D; k += 64) {
    acc_nodes[row + k] = k < len ? path[k] : -1;
    int c = -1;
    if (k < len - 1) c = tok[base + path[k + 1]];
    else if (k == len - 1) c = b;
    commit[row + k] = c;
  }
  if (lane == 0) {
    acc_len[r] = len;
    bonus[r] = b;
  }
}

}  // namespace

extern "C" int ddtree_accept(const int32_t* node_tokens, const int32_t* node_parents,
                             const int32_t* qo_indptr, const int32_t* target_predict, int bs,
                             int depth_max, int32_t* accepted_nodes, int32_t* accept_len,
                             int32_t* commit_tokens, int32_t* bonus_tokens, void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "accept: bs must be >= 0");
  DDTREE_REQUIRE(depth_max >= 0, DDTREE_EINVAL, "accept: depth_max must be >= 0");
  DDTREE_REQUIRE(depth_max <= 4096, DDTREE_EUNSUPPORTED, "accept: depth_max above 4096");
  if (bs == 0) return DDTREE_OK;
  DDTREE_REQUIRE(node_tokens && node_parents && qo_indptr && target_predict && accepted_nodes &&
                     accept_len && commit_tokens && bonus_tokens,
                 DDTREE_EINVAL, "accept: null pointer");
  hipLaunchKernelGGL(accept_kernel, dim3(bs), dim3(64), (depth_max + 1) * sizeof(int),
                     ddtree::as_stream(stream), node_tokens, node_parents, qo_indptr,
                     target_predict, depth_max, accepted_nodes, accept_len, commit_tokens,
                     bonus_tokens);
  return ddtree::check_launch("accept");
}
