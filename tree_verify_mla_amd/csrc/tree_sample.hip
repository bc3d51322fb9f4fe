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
// at bonus_u times the residual's mass.  A token without mass is never
// accepted and never drawn.
//
// The comparisons decide integers; fp32 with one fixed order for every sum,
// so the kernel's own results do not depend on timing:
// a row is cut into NB contiguous blocks of ceil(V / NB) tokens; a block's
// mass is its tokens summed one by one, the row's mass the block masses
// summed one by one, and the running mass at token j the masses of the
// blocks before j's block summed one by one plus j's block's tokens up to
// j.  Inverse CDF: the first block b whose running mass plus its own exceeds
// the threshold, then the first token of b whose running mass does; if
// rounding leaves the threshold unreached in that block, its last token with
// mass; if no block reaches it, the row's last token with mass.
//
// Two kernels.  block_mass_kernel sums every block of every node's row (the
// whole [total_q, V] tensor read once, coalesced: tiles of 64 blocks x 64
// tokens are staged through LDS and one lane keeps each block's sequential
// sum) into the workspace.  walk_kernel (one workgroup per request) then
// takes the decisions from those masses and the children's probabilities,
// and for the bonus re-sums only the blocks that hold rejected tokens and
// scans the one block the threshold falls in.
#include <mutex>
#include <vector>

#include "common.h"

namespace {

constexpr int NB = 256;        // blocks per row
constexpr int GB = 64;         // blocks per block_mass workgroup
constexpr int KT = 64;         // tokens per block per tile
constexpr int WT = 256;        // walk threads
constexpr int MAXQ = 4096;     // nodes per request the walk tries
constexpr int MAX_REJ = 1024;  // rejected tokens remembered at one node
constexpr int STAGE = 8192;    // floats of one staged block (limits ceil(V / NB))

// ---------------------------------------------------------------------------
// block masses: bm[row][b] = sequential sum of block b, bl[row][b] = its last
// token with mass (-1 if none)
__global__ __launch_bounds__(256) void block_mass_kernel(const float* __restrict__ probs, int V,
                                                         int per, float* __restrict__ bm,
                                                         int* __restrict__ bl) {
  __shared__ __align__(16) float tile[GB][KT + 4];  // rows 16-byte aligned; 16 lanes cover the banks
  const int row = blockIdx.x, b0 = blockIdx.y * GB;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float* src = probs + (size_t)row * V;
  static_assert(256 % KT == 0 && GB * KT % 256 == 0, "tile shape");
  constexpr int PER_T = GB * KT / 256;  // values each thread loads per tile
  constexpr int BSTEP = 256 / KT;       // blocks one pass of the workgroup covers
  const int kk = t % KT, bb = t / KT;   // this thread's token and block in the tile
  float v[PER_T];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int b = b0 + bb + BSTEP * i, k = k0 + kk;
      const int tok = b * per + k;
      v[i] = (k < per && tok < V) ? src[tok] : 0.f;
    }
  };
  float acc = 0.f;
  int last = -1;
  load(0);
  for (int k0 = 0; k0 < per; k0 += KT) {
    __syncthreads();  // the previous tile has been summed
#pragma unroll
    for (int i = 0; i < PER_T; ++i) tile[bb + BSTEP * i][kk] = v[i];
    __syncthreads();
    if (k0 + KT < per) load(k0 + KT);  // in flight while the tile is summed
    if (w == 0) {  // the tile's padding past the block is zero: adding it is exact
      const int base = (b0 + lane) * per + k0;
      const float4* tr = reinterpret_cast<const float4*>(&tile[lane][0]);
#pragma unroll
      for (int q = 0; q < KT / 4; ++q) {
        const float4 x = tr[q];
        acc = acc + x.x;
        last = x.x > 0.f ? base + 4 * q : last;
        acc = acc + x.y;
        last = x.y > 0.f ? base + 4 * q + 1 : last;
        acc = acc + x.z;
        last = x.z > 0.f ? base + 4 * q + 2 : last;
        acc = acc + x.w;
        last = x.w > 0.f ? base + 4 * q + 3 : last;
      }
    }
  }
  if (w == 0) {
    bm[(size_t)row * NB + b0 + lane] = acc;
    bl[(size_t)row * NB + b0 + lane] = last;
  }
}

// ---------------------------------------------------------------------------
__device__ inline float rl(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// sequential fp32 sum of n (multiple of 4) LDS values, in order
__device__ inline float seq_sum4(const float* p, int n) {
  float s = 0.f;
#pragma unroll 8
  for (int k = 0; k < n; k += 4) {
    const float4 v = *reinterpret_cast<const float4*>(p + k);
    s = s + v.x;
    s = s + v.y;
    s = s + v.z;
    s = s + v.w;
  }
  return s;
}

__global__ __launch_bounds__(WT) void walk_kernel(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ qo, const float* __restrict__ probs,
    const float* __restrict__ coins, const float* __restrict__ bonus_u, int total_q, int D, int V,
    int per, const float* __restrict__ bm, const int* __restrict__ bl,
    int32_t* __restrict__ acc_nodes, int32_t* __restrict__ acc_len, int32_t* __restrict__ commit,
    int32_t* __restrict__ bonus_out) {
  __shared__ __align__(16) float s_bm[NB];
  __shared__ int s_bl[NB];
  __shared__ int s_par[MAXQ], s_tok[MAXQ];
  __shared__ float s_coin[MAXQ], s_pc[MAXQ];
  __shared__ int s_rej[MAX_REJ];
  __shared__ __align__(16) float s_stage[STAGE];
  __shared__ int s_aff[NB], s_group[NB];
  // written by one thread between barriers
  __shared__ int s_nrej, s_cur, s_next, s_ngroup, s_block, s_first, s_tokout;
  __shared__ float s_R, s_run;

  const int r = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int a = min(max(qo[r], 0), total_q);
  const int Q = min(max(min(qo[r + 1], total_q) - a, 0), MAXQ);
  int32_t* nodes_r = acc_nodes + (size_t)r * (D + 1);
  int32_t* commit_r = commit + (size_t)r * (D + 1);
  for (int i = t; i <= D; i += WT) {
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
  for (int c = t; c < Q; c += WT) {
    s_par[c] = parents[a + c];
    s_tok[c] = tokens[a + c];
    s_coin[c] = coins[a + c];
  }
  int n = 1;  // path length (wave 0's)
  if (t == 0) {
    s_nrej = 0;
    s_cur = 0;
    nodes_r[0] = 0;
  }
  __syncthreads();

  // walk: per node, everyone fetches the row's block masses and the
  // children's probabilities; wave 0 decides, every lane holding the same
  // values
  while (true) {
    const int cur = s_cur;
    const size_t row = (size_t)(a + cur);
    s_bm[t] = bm[row * NB + t];
    s_bl[t] = bl[row * NB + t];
    for (int c = 1 + t; c < Q; c += WT) {
      if (s_par[c] == cur) {
        const int tok = s_tok[c];
        float p = (tok >= 0 && tok < V) ? probs[row * V + tok] : 0.f;
        // when c is tried every earlier sibling has been rejected, so an
        // earlier sibling with the same token has zeroed it
        for (int c2 = 1; c2 < c; ++c2)
          if (s_par[c2] == cur && s_tok[c2] == tok) p = 0.f;
        s_pc[c] = p;
      }
    }
    __syncthreads();
    if (t < 64) {
      float R = seq_sum4(s_bm, NB);
      int next = -1, nrej = s_nrej;
      if (n < D + 1) {
        for (int base = 1; base < Q && next < 0; base += 64) {
          const int c = base + lane;
          const bool kid = c < Q && s_par[c] == cur;
          const float pc = kid ? s_pc[c] : 0.f, cn = kid ? s_coin[c] : 0.f;
          const int tk = kid ? s_tok[c] : -1;
          unsigned long long m = __ballot(kid);
          while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            const float pt = rl(pc, j);
            // a token without mass is never accepted (coin * R >= 0 in exact
            // arithmetic), nor is a running mass that rounding took below
            // zero allowed to accept one
            if (pt > 0.f && rl(cn, j) * R < pt) {
              next = base + j;
              break;
            }
            R = fmaxf(R - pt, 0.f);
            const int tok = __builtin_amdgcn_readlane(tk, j);
            if (tok >= 0 && tok < V && nrej < MAX_REJ) {
              if (lane == 0) s_rej[nrej] = tok;
              ++nrej;
            }
          }
        }
      }
      if (lane == 0) {
        s_R = R;
        s_next = next;
        s_nrej = nrej;
        if (next >= 0) {
          nodes_r[n] = next;
          commit_r[n - 1] = s_tok[next];
          s_cur = next;
          s_nrej = 0;
        }
      }
      if (next >= 0) ++n;
    }
    __syncthreads();
    if (s_next < 0) break;  // s_next is next written after the following barrier
  }

  // bonus at the last node (s_bm, s_bl hold its row; s_rej its rejections):
  // re-sum the blocks that hold rejected tokens with those tokens zeroed
  const int cur = s_cur;
  const float* src = probs + (size_t)(a + cur) * V;
  const int nrej = s_nrej;
  s_aff[t] = 0;
  if (t == 0) s_ngroup = 0;
  __syncthreads();
  for (int k = t; k < nrej; k += WT) s_aff[s_rej[k] / per] = 1;
  __syncthreads();
  if (s_aff[t]) {  // the order of the list does not matter
    s_group[atomicAdd(&s_ngroup, 1)] = t;
    s_bl[t] = -1;
  }
  __syncthreads();
  const int naff = s_ngroup;
  const int per4 = (per + 3) & ~3;  // staged stride, zero padded
  const int G = STAGE / per4;       // blocks staged at once (>= 1)
  for (int g0 = 0; g0 < naff; g0 += G) {
    const int ng = min(G, naff - g0);
    for (int i = t; i < ng * per4; i += WT) {
      const int k = i % per4, tok = s_group[g0 + i / per4] * per + k;
      s_stage[i] = (k < per && tok < V) ? src[tok] : 0.f;
    }
    __syncthreads();
    for (int k = t; k < nrej; k += WT) {
      const int tok = s_rej[k];
      for (int j = 0; j < ng; ++j)
        if (s_group[g0 + j] == tok / per) s_stage[j * per4 + tok % per] = 0.f;
    }
    __syncthreads();
    for (int i = t; i < ng * per4; i += WT)
      if (s_stage[i] > 0.f) {
        const int b = s_group[g0 + i / per4];
        atomicMax(&s_bl[b], b * per + i % per4);
      }
    if (t < ng) s_bm[s_group[g0 + t]] = seq_sum4(s_stage + t * per4, per4);
    __syncthreads();
  }

  // the block the threshold falls in: wave 0 forms the running masses in
  // order (lane l keeps those of blocks 4l .. 4l+3); the threshold is the
  // uniform times the residual's mass in the same order (its last running
  // mass); then the first block whose running mass plus its own exceeds it
  if (t < 64) {
    float run = 0.f, mine[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int q = 0; q < NB / 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(s_bm + 4 * q);
      const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (q == lane) mine[e] = run;
        run = run + x[e];
      }
    }
    const float thr = bonus_u[r] * run;
    int k = -1;
#pragma unroll
    for (int e = 3; e >= 0; --e)
      if (mine[e] + s_bm[4 * lane + e] > thr) k = e;
    const unsigned long long m = __ballot(k >= 0);
    if (lane == 0) {
      s_R = thr;
      s_block = -1;
    }
    if (m) {
      const int l0 = __builtin_ctzll(m);
      if (lane == l0) {
        s_block = 4 * l0 + k;
        s_run = mine[k];
      }
    } else if (lane == 0) {  // the row's last token with mass
      int last = -1;
      for (int b = 0; b < NB; ++b) last = s_bl[b] >= 0 ? s_bl[b] : last;
      s_tokout = last;
    }
    if (lane == 0) s_first = INT_MAX;
  }
  __syncthreads();
  const int blk = s_block;
  if (blk >= 0) {
    for (int i = t; i < per4; i += WT) {
      const int tok = blk * per + i;
      s_stage[i] = (i < per && tok < V) ? src[tok] : 0.f;
    }
    __syncthreads();
    for (int k = t; k < nrej; k += WT) {
      const int tok = s_rej[k];
      if (tok / per == blk) s_stage[tok % per] = 0.f;
    }
    __syncthreads();
    // running masses inside the block, in order, in place
    if (t == 0) {
      float acc = s_run;
#pragma unroll 4
      for (int k = 0; k < per4; k += 4) {
        float4 v = *reinterpret_cast<const float4*>(s_stage + k);
        acc = acc + v.x;
        v.x = acc;
        acc = acc + v.y;
        v.y = acc;
        acc = acc + v.z;
        v.z = acc;
        acc = acc + v.w;
        v.w = acc;
        *reinterpret_cast<float4*>(s_stage + k) = v;
      }
    }
    __syncthreads();
    const float thr = s_R;
    for (int k = t; k < per; k += WT)
      if (s_stage[k] > thr) {
        atomicMin(&s_first, k);
        break;
      }
    __syncthreads();
    if (t == 0) s_tokout = s_first < per ? blk * per + s_first : s_bl[blk];
  }
  if (t == 0) {
    const int bonus = s_tokout;
    commit_r[n - 1] = bonus;
    acc_len[r] = n;
    bonus_out[r] = bonus;
  }
}

// The launches of one call, the block masses in bm / bl.
int launch_sample(const int32_t* node_tokens, const int32_t* node_parents,
                  const int32_t* qo_indptr, const float* target_probs, const float* coins,
                  const float* bonus_uniforms, int bs, int total_q, int depth_max, int vocab,
                  int32_t* accepted_nodes, int32_t* accept_len, int32_t* commit_tokens,
                  int32_t* bonus_tokens, float* bm, int* bl, hipStream_t s) {
  const int per = (vocab + NB - 1) / NB;
  if (total_q > 0) {
    hipLaunchKernelGGL(block_mass_kernel, dim3(total_q, NB / GB), dim3(256), 0, s, target_probs,
                       vocab, per, bm, bl);
    const int rc = ddtree::check_launch("tree_sample");
    if (rc != DDTREE_OK) return rc;
  }
  hipLaunchKernelGGL(walk_kernel, dim3(bs), dim3(WT), 0, s, node_tokens, node_parents, qo_indptr,
                     target_probs, coins, bonus_uniforms, total_q, depth_max, vocab, per, bm, bl,
                     accepted_nodes, accept_len, commit_tokens, bonus_tokens);
  return ddtree::check_launch("tree_sample");
}

// Host checks shared by both entry points (everything but the workspace).
int check_args(const char* fn, const int32_t* node_tokens, const int32_t* node_parents,
               const int32_t* qo_indptr, const float* target_probs, const float* coins,
               const float* bonus_uniforms, int bs, int total_q, int depth_max, int vocab,
               int32_t* accepted_nodes, int32_t* accept_len, int32_t* commit_tokens,
               int32_t* bonus_tokens) {
  DDTREE_REQUIRE(node_tokens && node_parents && qo_indptr && target_probs && coins &&
                     bonus_uniforms && accepted_nodes && accept_len && commit_tokens &&
                     bonus_tokens,
                 DDTREE_EINVAL, "%s: null required pointer", fn);
  DDTREE_REQUIRE(total_q >= 0, DDTREE_EINVAL, "%s: total_q must be >= 0", fn);
  DDTREE_REQUIRE(depth_max >= 0, DDTREE_EINVAL, "%s: depth_max must be >= 0", fn);
  DDTREE_REQUIRE(vocab >= 1, DDTREE_EINVAL, "%s: vocab must be >= 1", fn);
  DDTREE_REQUIRE((long long)vocab <= (long long)NB * STAGE, DDTREE_EUNSUPPORTED,
                 "%s: vocab %d above the supported %d", fn, vocab, NB * STAGE);
  return DDTREE_OK;
}

// Scratch of the allocation-free entry point: the block masses (floats) and
// last-token indices (ints) of up to NOALLOC_MAX_Q rows.  Every call on a
// device uses that device's copy; the kernels overwrite every entry they
// read, so nothing needs clearing.
constexpr int NOALLOC_MAX_Q = 4096;
constexpr size_t NOALLOC_BYTES = (size_t)NOALLOC_MAX_Q * NB * (sizeof(float) + sizeof(int));
__device__ __align__(256) char scratch[NOALLOC_BYTES];

// The device address of the current device's scratch, looked up once per
// device with that device current (host code never uses the array's name as
// an address).
int scratch_ptr(char** out) {
  static std::mutex mu;
  static std::vector<char*> ptrs;
  int dev = 0;
  DDTREE_REQUIRE(hipGetDevice(&dev) == hipSuccess && dev >= 0, DDTREE_EHIP,
                 "tree_sample_noalloc: no current device");
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    DDTREE_REQUIRE(e == hipSuccess && p, DDTREE_EHIP,
                   "tree_sample_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
    ptrs[dev] = static_cast<char*>(p);
  }
  *out = ptrs[dev];
  return DDTREE_OK;
}

}  // namespace

extern "C" size_t ddtree_tree_sample_workspace_size(int total_q) {
  return total_q > 0 ? (size_t)total_q * NB * (sizeof(float) + sizeof(int)) : 0;
}

extern "C" int ddtree_tree_sample(const int32_t* node_tokens, const int32_t* node_parents,
                                  const int32_t* qo_indptr, const float* target_probs,
                                  const float* coins, const float* bonus_uniforms, int bs,
                                  int total_q, int depth_max, int vocab, int32_t* accepted_nodes,
                                  int32_t* accept_len, int32_t* commit_tokens,
                                  int32_t* bonus_tokens, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "tree_sample: bs must be >= 0");
  if (bs == 0) return DDTREE_OK;
  int rc = check_args("tree_sample", node_tokens, node_parents, qo_indptr, target_probs, coins,
                      bonus_uniforms, bs, total_q, depth_max, vocab, accepted_nodes, accept_len,
                      commit_tokens, bonus_tokens);
  if (rc != DDTREE_OK) return rc;
  const size_t need = ddtree_tree_sample_workspace_size(total_q);
  DDTREE_REQUIRE(need == 0 || (workspace && workspace_bytes >= need), DDTREE_EWORKSPACE,
                 "tree_sample: workspace of %zu bytes needed (got %zu)", need,
                 workspace ? workspace_bytes : (size_t)0);
  float* bm = static_cast<float*>(workspace);
  int* bl = reinterpret_cast<int*>(static_cast<char*>(workspace) + (size_t)total_q * NB * sizeof(float));
  return launch_sample(node_tokens, node_parents, qo_indptr, target_probs, coins, bonus_uniforms,
                       bs, total_q, depth_max, vocab, accepted_nodes, accept_len, commit_tokens,
                       bonus_tokens, bm, bl, ddtree::as_stream(stream));
}

extern "C" int ddtree_tree_sample_noalloc(const int32_t* node_tokens, const int32_t* node_parents,
                                          const int32_t* qo_indptr, const float* target_probs,
                                          const float* coins, const float* bonus_uniforms, int bs,
                                          int total_q, int depth_max, int vocab,
                                          int32_t* accepted_nodes, int32_t* accept_len,
                                          int32_t* commit_tokens, int32_t* bonus_tokens,
                                          void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "tree_sample_noalloc: bs must be >= 0");
  if (bs == 0) return DDTREE_OK;
  int rc = check_args("tree_sample_noalloc", node_tokens, node_parents, qo_indptr, target_probs,
                      coins, bonus_uniforms, bs, total_q, depth_max, vocab, accepted_nodes,
                      accept_len, commit_tokens, bonus_tokens);
  if (rc != DDTREE_OK) return rc;
  DDTREE_REQUIRE(total_q <= NOALLOC_MAX_Q, DDTREE_EUNSUPPORTED,
                 "tree_sample_noalloc: total_q %d above the built-in scratch's %d rows", total_q,
                 NOALLOC_MAX_Q);
  char* base = nullptr;
  rc = scratch_ptr(&base);
  if (rc != DDTREE_OK) return rc;
  float* bm = reinterpret_cast<float*>(base);
  int* bl = reinterpret_cast<int*>(base + (size_t)NOALLOC_MAX_Q * NB * sizeof(float));
  return launch_sample(node_tokens, node_parents, qo_indptr, target_probs, coins, bonus_uniforms,
                       bs, total_q, depth_max, vocab, accepted_nodes, accept_len, commit_tokens,
                       bonus_tokens, bm, bl, ddtree::as_stream(stream));
}
