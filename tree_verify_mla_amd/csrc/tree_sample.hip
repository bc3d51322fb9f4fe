// ddtree_tree_sample: stochastic (temperature) acceptance along the tree.
//
// With temperature the tree is walked by tree-structured rejection sampling
// against the target's filtered distribution at every node, the draft being
// the tree's own tokens ("The DDTree CUDA Graph Fix ...", section
// "Temperature Support: Already Working for Linear, Planned for DDTree").
// The rule is the speculative-sampling one for a draft that puts all its
// mass on its token: at node cur the residual starts as the target row with
// mass R; the children are tried in node order; child c with token t is
// accepted iff coin[c] * R < res[t], otherwise R -= res[t] and res[t] = 0;
// the walk stops when no child is accepted or after depth_max + 1 nodes,
// and the bonus is drawn from the residual at the last node by inverse CDF
// at bonus_u * R.
//
// The comparisons decide integers, so every sum has one fixed order (fp32):
// a row is cut into NT contiguous blocks of ceil(V / NT) tokens (thread b
// owns block b); a block's mass is its tokens summed one by one, the row's
// mass the block masses summed one by one, and the running mass at token j
// the masses of the blocks before j's block summed one by one plus j's
// block's tokens up to j.  Inverse CDF: the first block b whose running
// mass plus its own exceeds the threshold, then the first token of b whose
// running mass does; if rounding leaves the threshold unreached in that
// block, its last token with mass; if no block reaches it, the row's last
// token with mass.
//
// One workgroup per request; its threads sum the row blocks, thread 0 takes
// the decisions.
#include "common.h"

namespace {

constexpr int NT = 256;       // threads = row blocks
constexpr int MAX_REJ = 1024; // rejected tokens remembered at one node

__global__ __launch_bounds__(NT) void tree_sample_kernel(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ qo, const float* __restrict__ probs,
    const float* __restrict__ coins, const float* __restrict__ bonus_u, int D, int V,
    int32_t* __restrict__ acc_nodes, int32_t* __restrict__ acc_len,
    int32_t* __restrict__ commit, int32_t* __restrict__ bonus_out) {
  __shared__ float s_mass[NT];
  __shared__ int s_last[NT];
  __shared__ int s_rej[MAX_REJ];
  __shared__ int s_nrej, s_cur, s_next, s_block, s_tok;  // written by thread 0 only
  __shared__ float s_run, s_thr;
  const int r = blockIdx.x, t = threadIdx.x;
  const int a = qo[r], Q = qo[r + 1] - a;
  int32_t* nodes_r = acc_nodes + (size_t)r * (D + 1);
  int32_t* commit_r = commit + (size_t)r * (D + 1);
  for (int i = t; i <= D; i += NT) {
    nodes_r[i] = -1;
    commit_r[i] = -1;
  }
  if (Q < 1) {
    if (t == 0) {
      acc_len[r] = 0;
      bonus_out[r] = -1;
    }
    return;
  }
  const int per = (V + NT - 1) / NT;
  const int lo = min(V, t * per), hi = min(V, lo + per);
  // residual value of token j at the current node
  auto res_of = [&](const float* row, int j) {
    float v = row[j];
    for (int k = 0; k < s_nrej; ++k)
      if (s_rej[k] == j) v = 0.f;
    return v;
  };
  // this thread's block mass of the current residual row, and its last
  // token with mass
  auto block_mass = [&](const float* row) {
    float m = 0.f;
    int last = -1;
    for (int j = lo; j < hi; ++j) {
      const float v = res_of(row, j);
      m = m + v;
      if (v > 0.f) last = j;
    }
    s_mass[t] = m;
    s_last[t] = last;
  };

  int cur = 0, n = 1;  // current node, path length (thread 0's; s_cur for all)
  if (t == 0) {
    s_nrej = 0;
    s_cur = 0;
    nodes_r[0] = 0;
  }
  __syncthreads();
  while (true) {
    const float* row = probs + (size_t)(a + s_cur) * V;
    block_mass(row);
    __syncthreads();
    if (t == 0) {
      float R = 0.f;
      for (int b = 0; b < NT; ++b) R = R + s_mass[b];
      int next = -1;
      if (n < D + 1) {
        for (int c = 1; c < Q; ++c) {
          if (parents[a + c] != cur) continue;
          const int tok = tokens[a + c];
          const float pt = (tok >= 0 && tok < V) ? res_of(row, tok) : 0.f;
          if (coins[a + c] * R < pt) {
            next = c;
            break;
          }
          R = R - pt;
          if (s_nrej < MAX_REJ) s_rej[s_nrej++] = tok;
        }
      }
      s_next = next;
      s_thr = bonus_u[r] * R;
    }
    __syncthreads();
    const int next = s_next;
    if (next < 0) break;
    __syncthreads();  // everyone has read s_next
    if (t == 0) {
      nodes_r[n] = next;
      commit_r[n - 1] = tokens[a + next];
      ++n;
      cur = next;
      s_cur = next;
      s_nrej = 0;
    }
    __syncthreads();
  }

  // bonus: inverse CDF of the residual at the last node (block masses are
  // those of the residual after the last rejections)
  const float* row = probs + (size_t)(a + s_cur) * V;
  block_mass(row);
  __syncthreads();
  if (t == 0) {
    const float thr = s_thr;
    float run = 0.f;
    int blk = -1;
    for (int b = 0; b < NT; ++b) {
      if (run + s_mass[b] > thr) {
        blk = b;
        break;
      }
      run = run + s_mass[b];
    }
    s_block = blk;
    s_run = run;
    if (blk < 0) {  // the row's last token with mass
      int last = -1;
      for (int b = 0; b < NT; ++b) last = s_last[b] >= 0 ? s_last[b] : last;
      s_tok = last;
    }
  }
  __syncthreads();
  if (t == s_block) {
    float acc = s_run;
    int tok = -1;
    for (int j = lo; j < hi; ++j) {
      const float v = res_of(row, j);
      acc = acc + v;
      if (acc > s_thr) {
        tok = j;
        break;
      }
    }
    s_tok = tok >= 0 ? tok : s_last[t];
  }
  __syncthreads();
  if (t == 0) {
    const int bonus = s_tok;
    commit_r[n - 1] = bonus;
    acc_len[r] = n;
    bonus_out[r] = bonus;
  }
}

}  // namespace

extern "C" int ddtree_tree_sample(const int32_t* node_tokens, const int32_t* node_parents,
                                  const int32_t* qo_indptr, const float* target_probs,
                                  const float* coins, const float* bonus_uniforms, int bs,
                                  int depth_max, int vocab, int32_t* accepted_nodes,
                                  int32_t* accept_len, int32_t* commit_tokens,
                                  int32_t* bonus_tokens, void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "tree_sample: bs must be >= 0");
  if (bs == 0) return DDTREE_OK;
  DDTREE_REQUIRE(node_tokens && node_parents && qo_indptr && target_probs && coins &&
                     bonus_uniforms && accepted_nodes && accept_len && commit_tokens &&
                     bonus_tokens,
                 DDTREE_EINVAL, "tree_sample: null required pointer");
  DDTREE_REQUIRE(depth_max >= 0, DDTREE_EINVAL, "tree_sample: depth_max must be >= 0");
  DDTREE_REQUIRE(vocab >= 1, DDTREE_EINVAL, "tree_sample: vocab must be >= 1");
  hipLaunchKernelGGL(tree_sample_kernel, dim3(bs), dim3(NT), 0, ddtree::as_stream(stream),
                     node_tokens, node_parents, qo_indptr, target_probs, coins, bonus_uniforms,
                     depth_max, vocab, accepted_nodes, accept_len, commit_tokens, bonus_tokens);
  return ddtree::check_launch("tree_sample");
}
