// ddtree_commit_kv: the accepted path enters the request's KV cache.
//
// The verify forward appended every tree node's latent after the request's
// prefix; after acceptance only the accepted nodes, root included and in path
// order, stay, in the positions right after the prefix, so the cache grows by
// accept_len and the bonus token is not cached ("The Architecture of a
// Speculative Decoding Engine ...", sections "The First Attempt: Temporary
// Buffers and Post-Verify Compaction", "The Off-by-One Labyrinth" and "The
// Final Resolution: A Concrete Trace").
//
// Workgroup (r, c): request r, prefix chunk c of CH slot ids.  Every
// workgroup copies its chunk of the prefix list; chunk 0 also writes the
// accepted entries and, in the move form, copies the accepted latent rows.
//
// Move form.  Path node i (node id n_i, n_0 = 0, strictly increasing along
// the path) goes to node slot i <= n_i.  A batch of rows is read completely
// before any row of it is written: a destination slot may be the source of
// an earlier path entry (n_j = i for j < i), never of a later one (n_j >= j),
// so batches taken in path order never read a row that was already replaced.
#include "common.h"

namespace {

constexpr int CT = 256;       // threads per workgroup
constexpr int CH = CT * 32;   // prefix slot ids per workgroup
constexpr int RB = 8;         // rows per move batch
constexpr int LATENT = 576;

struct Req {
  int kv0, P, Q, a;
};

// geometry of request r, clamped so that disagreeing device data stays in
// bounds: Q <= kv length, a in [0, min(Q, D + 1)]
__device__ inline Req request(const int32_t* kvp, const int32_t* qo, const int32_t* acc_len,
                              int r, int D) {
  Req q;
  q.kv0 = kvp[r];
  const int L = max(kvp[r + 1] - q.kv0, 0);
  q.Q = min(max(qo[r + 1] - qo[r], 0), L);
  q.P = L - q.Q;
  q.a = min(max(acc_len[r], 0), min(q.Q, D + 1));
  return q;
}

__global__ __launch_bounds__(CT) void commit_kv_kernel(
    const int32_t* __restrict__ kvp, const int32_t* __restrict__ kvi,
    const int32_t* __restrict__ qo, const int32_t* __restrict__ acc_nodes,
    const int32_t* __restrict__ acc_len, int bs, int D, int32_t* __restrict__ new_kvp,
    int32_t* __restrict__ new_kvi, long long new_cap, char* __restrict__ pool,
    long long num_slots, int row_bytes) {
  __shared__ long long part[CT / 64];
  const int r = blockIdx.x, c = blockIdx.y;
  const int t = threadIdx.x;
  const Req q = request(kvp, qo, acc_len, r, D);

  // start of request r's new list: the new lengths of the requests before it
  long long s = 0;
  for (int k = t; k < r; k += CT) {
    const Req o = request(kvp, qo, acc_len, k, D);
    s += o.P + o.a;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if ((t & 63) == 0) part[t >> 6] = s;
  __syncthreads();
  const long long off = part[0] + part[1] + part[2] + part[3];

  // the prefix slot ids of chunk c
  const int j0 = c * CH, j1 = min(q.P, j0 + CH);
  for (int j = j0 + t; j < j1; j += CT)
    if (off + j < new_cap) new_kvi[off + j] = kvi[q.kv0 + j];
  if (c != 0) return;

  if (t == 0) {
    new_kvp[r] = (int32_t)off;
    if (r == bs - 1) new_kvp[bs] = (int32_t)(off + q.P + q.a);
  }
  const int32_t* path = acc_nodes + (size_t)r * (D + 1);
  const int32_t* nodes = kvi + q.kv0 + q.P;  // node slots in node order
  auto node_of = [&](int i) { return min(max(path[i], 0), q.Q - 1); };
  for (int i = t; i < q.a; i += CT) {
    const long long dst = off + q.P + i;
    if (dst < new_cap) new_kvi[dst] = pool ? nodes[i] : nodes[node_of(i)];
  }
  if (!pool || q.a <= 1) return;

  // move form: row of node n_i -> node slot i, batches of RB rows
  const int cpr = row_bytes / 16;  // 16-byte chunks per row
  const long long smax = num_slots - 1;
  auto slot = [&](int node) { return min(max((long long)nodes[node], 0LL), smax); };
  for (int b0 = 1; b0 < q.a; b0 += RB) {
    const int nrow = min(RB, q.a - b0);
    const int n = nrow * cpr;
    constexpr int PER = (RB * LATENT * 4 / 16 + CT - 1) / CT;  // chunks per thread (fp32 rows)
    uint4 v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = t + k * CT;
      if (idx < n) {
        const int i = b0 + idx / cpr, ch = idx % cpr;
        v[k] = *reinterpret_cast<const uint4*>(pool + slot(node_of(i)) * row_bytes + ch * 16);
      }
    }
    // every row of the batch has been read (by every thread) before any is written
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = t + k * CT;
      if (idx < n) {
        const int i = b0 + idx / cpr, ch = idx % cpr;
        *reinterpret_cast<uint4*>(pool + slot(i) * row_bytes + ch * 16) = v[k];
      }
    }
  }
}

}  // namespace

extern "C" int ddtree_commit_kv(const int32_t* kv_indptr, const int32_t* kv_indices,
                                const int32_t* qo_indptr, const int32_t* accepted_nodes,
                                const int32_t* accept_len, int bs, int depth_max, int max_kv_len,
                                int32_t* new_kv_indptr, int32_t* new_kv_indices,
                                long long new_kv_capacity, void* kv_pool, long long num_slots,
                                int dtype, void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "commit_kv: bs must be >= 0 (got %d)", bs);
  if (bs == 0) return DDTREE_OK;
  DDTREE_REQUIRE(kv_indptr && kv_indices && qo_indptr && accepted_nodes && accept_len &&
                     new_kv_indptr && new_kv_indices,
                 DDTREE_EINVAL, "commit_kv: null required pointer");
  DDTREE_REQUIRE(depth_max >= 0, DDTREE_EINVAL, "commit_kv: depth_max must be >= 0");
  DDTREE_REQUIRE(max_kv_len >= 1, DDTREE_EINVAL, "commit_kv: max_kv_len must be >= 1");
  DDTREE_REQUIRE(new_kv_capacity >= 0, DDTREE_EINVAL, "commit_kv: new_kv_capacity must be >= 0");
  int row_bytes = 0;
  if (kv_pool) {
    DDTREE_REQUIRE(dtype == DDTREE_F32 || dtype == DDTREE_BF16, DDTREE_EINVAL,
                   "commit_kv: unknown dtype %d", dtype);
    DDTREE_REQUIRE(num_slots >= 1, DDTREE_EINVAL, "commit_kv: num_slots must be >= 1");
    row_bytes = LATENT * (dtype == DDTREE_F32 ? 4 : 2);
  }
  const long long nch = ((long long)max_kv_len + CH - 1) / CH;
  DDTREE_REQUIRE(nch <= 65535, DDTREE_EUNSUPPORTED, "commit_kv: max_kv_len %d too large",
                 max_kv_len);
  hipLaunchKernelGGL(commit_kv_kernel, dim3(bs, (unsigned)nch), dim3(CT), 0, ddtree::as_stream(stream),
                     kv_indptr, kv_indices, qo_indptr, accepted_nodes, accept_len, bs, depth_max,
                     new_kv_indptr, new_kv_indices, (long long)new_kv_capacity,
                     static_cast<char*>(kv_pool), num_slots, row_bytes);
  return ddtree::check_launch("commit_kv");
}
