// ddtree_build_tree: best-first draft-tree growth, one wavefront per request.
//
// The candidate frontier (nodes offered but not yet taken) lives in LDS as a
// structure of arrays.  Each step every lane scans a strided slice of the
// frontier for its best entry, a 6-step butterfly over the 64 lanes picks the
// overall best, and lane 0 appends it to the tree and offers its best child
// and its next-ranked sibling ("The DDTree CUDA Graph Fix: Unlocking
// Speculative Decoding at 109 tok/s on PCIe Blackwell", section "The DDTree
// Architecture: Confirming Multiple-Path Evaluation").  After k steps the
// frontier holds at most k + 1 entries, so max_budget + 2 slots suffice.
//
// The request's per-depth log-probs and token ids are staged in LDS first:
// the loop is a serial chain of budget steps, and a global load inside it
// would add a full memory latency to every step.
//
// Order: higher fp32 score first, then smaller depth, then the
// lexicographically smaller rank path.  Rank paths are packed big-endian in
// 64 bits (rank_bits per depth), so equal-depth paths compare as integers.
#include <climits>

#include "common.h"

namespace {

struct Cand {
  float score;
  int depth;
  uint64_t code;
  int idx;  // frontier slot, -1 = none
};

__device__ inline bool better(const Cand& a, const Cand& b) {
  if (a.idx < 0) return false;
  if (b.idx < 0) return true;
  if (a.score != b.score) return a.score > b.score;
  if (a.depth != b.depth) return a.depth < b.depth;
  return a.code < b.code;
}

__global__ __launch_bounds__(64) void build_tree_kernel(
    const float* __restrict__ lp, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ roots, const int32_t* __restrict__ qo, int D, int K,
    int max_budget, int rank_bits, int32_t* __restrict__ tok, int32_t* __restrict__ par,
    int32_t* __restrict__ dep, float* __restrict__ sc) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int cap = max_budget + 2;
  uint64_t* f_code = reinterpret_cast<uint64_t*>(smem);
  float* f_score = reinterpret_cast<float*>(f_code + cap);
  float* f_pscore = f_score + cap;
  int* f_depth = reinterpret_cast<int*>(f_pscore + cap);
  int* f_rank = f_depth + cap;
  int* f_parent = f_rank + cap;
  float* s_lp = reinterpret_cast<float*>(f_parent + cap);  // [D * K]
  int32_t* s_id = reinterpret_cast<int32_t*>(s_lp + D * K);  // [D * K]
  __shared__ int n_front;

  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int base = qo[r];
  const int Q = qo[r + 1] - base;
  if (Q < 1) return;
  const int B = min(Q - 1, max_budget);
  if (B > 0) {
    const float* lpg = lp + (size_t)r * D * K;
    const int32_t* idg = ids + (size_t)r * D * K;
    for (int i = lane; i < D * K; i += 64) {
      s_lp[i] = lpg[i];
      s_id[i] = idg[i];
    }
  }
  __syncthreads();
  const float* lpr = s_lp;
  const int32_t* idr = s_id;

  for (int i = B + 1 + lane; i < Q; i += 64) {  // budget beyond max_budget
    tok[base + i] = -1;
    par[base + i] = -1;
    dep[base + i] = -1;
    if (sc) sc[base + i] = 0.f;
  }
  if (lane == 0) {
    tok[base] = roots[r];
    par[base] = -1;
    dep[base] = 0;
    if (sc) sc[base] = 0.f;
    n_front = 0;
    if (B > 0) {  // the root's best child
      f_score[0] = __fadd_rn(0.f, lpr[0]);
      f_pscore[0] = 0.f;
      f_depth[0] = 1;
      f_rank[0] = 0;
      f_parent[0] = 0;
      f_code[0] = 0;
      n_front = 1;
    }
  }
  __syncthreads();

  for (int k = 1; k <= B; ++k) {
    const int n = n_front;
    Cand best{0.f, 0, 0, -1};
    for (int e = lane; e < n; e += 64) {
      Cand c{f_score[e], f_depth[e], f_code[e], e};
      if (better(c, best)) best = c;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      Cand o;
      o.score = __shfl_xor(best.score, off);
      o.depth = __shfl_xor(best.depth, off);
      uint32_t lo = __shfl_xor((uint32_t)best.code, off);
      uint32_t hi = __shfl_xor((uint32_t)(best.code >> 32), off);
      o.code = ((uint64_t)hi << 32) | lo;
      o.idx = __shfl_xor(best.idx, off);
      if (better(o, best) || (o.idx >= 0 && best.idx >= 0 && !better(best, o) && o.idx < best.idx))
        best = o;
    }
    if (lane == 0) {
      const int e = best.idx;
      if (e < 0) {  // empty frontier: only reachable if preconditions are broken
        for (int i = k; i <= B; ++i) {
          tok[base + i] = -1;
          par[base + i] = -1;
          dep[base + i] = -1;
          if (sc) sc[base + i] = 0.f;
        }
        n_front = 0;
      } else {
        const float s = f_score[e], ps = f_pscore[e];
        const int d = f_depth[e], rk = f_rank[e], p = f_parent[e];
        const uint64_t code = f_code[e];
        tok[base + k] = idr[(d - 1) * K + rk];
        par[base + k] = p;
        dep[base + k] = d;
        if (sc) sc[base + k] = s;
        // remove entry e (the last entry moves into its slot)
        int m = n - 1;
        f_score[e] = f_score[m];
        f_pscore[e] = f_pscore[m];
        f_depth[e] = f_depth[m];
        f_rank[e] = f_rank[m];
        f_parent[e] = f_parent[m];
        f_code[e] = f_code[m];
        if (d < D) {  // best child of the new node
          f_score[m] = __fadd_rn(s, lpr[d * K]);
          f_pscore[m] = s;
          f_depth[m] = d + 1;
          f_rank[m] = 0;
          f_parent[m] = k;
          f_code[m] = code << rank_bits;
          ++m;
        }
        if (rk + 1 < K) {  // next-ranked sibling under the same parent
          f_score[m] = __fadd_rn(ps, lpr[(d - 1) * K + rk + 1]);
          f_pscore[m] = ps;
          f_depth[m] = d;
          f_rank[m] = rk + 1;
          f_parent[m] = p;
          f_code[m] = code + 1;
          ++m;
        }
        n_front = min(m, cap);
      }
    }
    __syncthreads();
    if (n_front == 0) break;
  }
}

}  // namespace

extern "C" int ddtree_build_tree(const float* topk_logprobs, const int32_t* topk_ids,
                                 const int32_t* root_tokens, const int32_t* qo_indptr, int bs,
                                 int depth_max, int topk, int max_budget, int32_t* node_tokens,
                                 int32_t* node_parents, int32_t* node_depths, float* node_scores,
                                 void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "build_tree: bs must be >= 0 (got %d)", bs);
  DDTREE_REQUIRE(max_budget >= 0, DDTREE_EINVAL, "build_tree: max_budget must be >= 0");
  if (bs == 0) return DDTREE_OK;
  DDTREE_REQUIRE(root_tokens && qo_indptr && node_tokens && node_parents && node_depths,
                 DDTREE_EINVAL, "build_tree: null required pointer");
  if (max_budget > 0) {
    DDTREE_REQUIRE(topk_logprobs && topk_ids, DDTREE_EINVAL, "build_tree: null top-k input");
    DDTREE_REQUIRE(depth_max >= 1 && topk >= 1, DDTREE_EINVAL,
                   "build_tree: depth_max and topk must be >= 1 for a non-empty tree");
    // reachable = sum_{d=1..D} K^d, saturating
    long long reach = 0, pw = 1;
    for (int d = 1; d <= depth_max && reach < (long long)max_budget; ++d) {
      pw = (pw > (1LL << 40) / topk) ? (1LL << 40) : pw * topk;
      reach += pw;
    }
    DDTREE_REQUIRE((long long)max_budget <= reach, DDTREE_EINVAL,
                   "build_tree: max_budget %d exceeds the %lld reachable rank paths", max_budget,
                   reach);
  }
  int rank_bits = 1;
  while ((1 << rank_bits) < topk) ++rank_bits;
  DDTREE_REQUIRE(max_budget == 0 || (long long)depth_max * rank_bits <= 64, DDTREE_EUNSUPPORTED,
                 "build_tree: depth_max * ceil(log2(topk)) = %lld exceeds 64 bits",
                 (long long)depth_max * rank_bits);
  DDTREE_REQUIRE(max_budget <= 2048, DDTREE_EUNSUPPORTED,
                 "build_tree: max_budget %d above the supported 2048", max_budget);
  DDTREE_REQUIRE(max_budget == 0 || (long long)depth_max * topk <= 8192, DDTREE_EUNSUPPORTED,
                 "build_tree: depth_max * topk = %lld above the supported 8192",
                 (long long)depth_max * topk);
  const size_t staged = max_budget > 0 ? (size_t)depth_max * topk * 8 : 0;  // log-probs + ids
  const size_t lds = (size_t)(max_budget + 2) * (8 + 4 * 5) + staged;
  hipLaunchKernelGGL(build_tree_kernel, dim3(bs), dim3(64), lds, ddtree::as_stream(stream),
                     topk_logprobs, topk_ids, root_tokens, qo_indptr, depth_max, topk, max_budget,
                     rank_bits, node_tokens, node_parents, node_depths, node_scores);
  return ddtree::check_launch("build_tree");
}
