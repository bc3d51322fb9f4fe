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
// Two candidates never share a rank path, so the order is total.
//
// Budgets up to 126 run build_tree_reg_kernel: the frontier lives in
// registers, two entries per lane, and a step is one wave-wide max of a
// 32-bit score key (DPP inside each 16-lane row, then the four row results
// in scalar registers), a ballot, and per-lane selects that put the taken
// entry's best child in its slot and append its sibling.  Exact score ties fall to
// a rarely taken exact tie-break on depth and rank path.  Larger budgets run
// build_tree_kernel, which keeps the frontier in LDS.
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


// ---------------------------------------------------------------------------
// Register frontier (budget <= REG_MAX_BUDGET)
// ---------------------------------------------------------------------------
constexpr int REG_MAX_BUDGET = 126;  // frontier slots <= budget + 1 <= 127 < 2 x 64

// value of lane src_lane (uniform) of x
__device__ inline uint32_t lane_val(uint32_t x, int src_lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, src_lane);
}

// wave-wide maximum (MAX) or minimum of x, uniform result
template <bool MAX>
__device__ inline uint32_t wave_ext(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  // the operation's identity as the DPP fill value lets the move fold into it
  constexpr int ID = MAX ? 0 : -1;
  // inside each 16-lane row: swap neighbours, pairs, then mirror halves
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)x, 0xB1, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)x, 0x4E, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)x, 0x141, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)x, 0x140, 0xF, 0xF, false));
  return op(op(lane_val(x, 0), lane_val(x, 16)), op(lane_val(x, 32), lane_val(x, 48)));
}

// order-preserving map of an fp32 score to uint32 (larger score -> larger key)
__device__ inline uint32_t score_key(float f) {
  const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One frontier entry.  meta packs depth (7 bits), rank (13 bits) and parent
// node (11 bits) -- depth_max * rank_bits <= 64, depth_max * topk <= 8192
// and the budget <= 126 bound them -- plus a valid bit.
struct Slot {
  float score, pscore;
  uint32_t meta, code_lo, code_hi;
};
__device__ inline uint32_t pack_meta(int depth, int rank, int parent) {
  return 0x80000000u | ((uint32_t)parent << 20) | ((uint32_t)rank << 7) | (uint32_t)depth;
}
__device__ inline int meta_depth(uint32_t m) { return (int)(m & 0x7f); }
__device__ inline int meta_rank(uint32_t m) { return (int)((m >> 7) & 0x1fff); }
__device__ inline int meta_parent(uint32_t m) { return (int)((m >> 20) & 0x7ff); }

__device__ inline Slot bcast(const Slot& x, int lane) {
  Slot r;
  r.score = __uint_as_float(lane_val(__float_as_uint(x.score), lane));
  r.pscore = __uint_as_float(lane_val(__float_as_uint(x.pscore), lane));
  r.meta = lane_val(x.meta, lane);
  r.code_lo = lane_val(x.code_lo, lane);
  r.code_hi = lane_val(x.code_hi, lane);
  return r;
}

__device__ inline Slot pick(bool c, const Slot& a, const Slot& b) {
  Slot r;
  r.score = c ? a.score : b.score;
  r.pscore = c ? a.pscore : b.pscore;
  r.meta = c ? a.meta : b.meta;
  r.code_lo = c ? a.code_lo : b.code_lo;
  r.code_hi = c ? a.code_hi : b.code_hi;
  return r;
}

// Top-k tables of up to TAB_REGS * 64 entries are also held in registers,
// entry i in lane i & 63, register i >> 6, and read with readlane (a few
// cycles instead of an LDS round trip).
constexpr int TAB_REGS = 4;

template <bool REG_TAB>
__global__ __launch_bounds__(64) void build_tree_reg_kernel(
    const float* __restrict__ lp, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ roots, const int32_t* __restrict__ qo, int D, int K,
    int max_budget, int rank_bits, int32_t* __restrict__ tok, int32_t* __restrict__ par,
    int32_t* __restrict__ dep, float* __restrict__ sc) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* s_lp = reinterpret_cast<float*>(smem);               // [D * K]
  int32_t* s_id = reinterpret_cast<int32_t*>(s_lp + D * K);   // [D * K]

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
  }
  if (B <= 0) return;

  // Entry e lives in lane e & 63, slot e >> 6.  A taken entry's slot is
  // reused by its best child; its sibling is appended at n, so n <= k + 1.
  // A slot whose entry left no successor stays invalid (meta 0).
  Slot f[2];
  // entry i of the tables (uniform i); named registers, not an array, so
  // that the uniform selection stays in registers
  uint32_t lp0 = 0, lp1 = 0, lp2 = 0, lp3 = 0, id0 = 0, id1 = 0, id2 = 0, id3 = 0;
  static_assert(TAB_REGS == 4, "four table registers per lane");
  if constexpr (REG_TAB) {
    auto ld = [&](int j, uint32_t& l, uint32_t& t) {
      const int i = lane + 64 * j;
      l = i < D * K ? __float_as_uint(s_lp[i]) : 0u;
      t = i < D * K ? (uint32_t)s_id[i] : 0u;
    };
    ld(0, lp0, id0);
    ld(1, lp1, id1);
    ld(2, lp2, id2);
    ld(3, lp3, id3);
  }
  auto table = [&](uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3, int i) {
    const int j = i >> 6;  // uniform
    const uint32_t v = j == 0 ? t0 : (j == 1 ? t1 : (j == 2 ? t2 : t3));
    return lane_val(v, i & 63);
  };
  auto lp_at = [&](int i) {
    if constexpr (REG_TAB) return __uint_as_float(table(lp0, lp1, lp2, lp3, i));
    else return s_lp[i];
  };
  auto id_at = [&](int i) {
    if constexpr (REG_TAB) return (int32_t)table(id0, id1, id2, id3, i);
    else return s_id[i];
  };

  const Slot none{0.f, 0.f, 0u, 0u, 0u};
  f[0] = none;
  f[1] = none;
  if (lane == 0) {  // the root's best child
    f[0].score = __fadd_rn(0.f, s_lp[0]);
    f[0].meta = pack_meta(1, 0, 0);
  }
  int n = 1;
  for (int k = 1; k <= B; ++k) {
    // 1. the best entry: largest score key, ties resolved exactly
    uint32_t key[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t kq = score_key(f[q].score);
      key[q] = f[q].meta ? kq : 0u;
    }
    const uint32_t kmax = wave_ext<true>(max(key[0], key[1]));
    if (kmax == 0u) {  // empty frontier: only reachable if preconditions are broken
      for (int i = k + lane; i <= B; i += 64) {
        tok[base + i] = -1;
        par[base + i] = -1;
        dep[base + i] = -1;
        if (sc) sc[base + i] = 0.f;
      }
      break;
    }
    uint64_t hit0 = __ballot(key[0] == kmax);
    uint64_t hit1 = __ballot(key[1] == kmax);
    if (__popcll(hit0) + __popcll(hit1) > 1) {  // rare: equal scores
      bool t0 = (hit0 >> lane) & 1, t1 = (hit1 >> lane) & 1;
      const uint32_t d0 = f[0].meta & 0x7f, d1 = f[1].meta & 0x7f;
      const uint32_t dmin = wave_ext<false>(min(t0 ? d0 : ~0u, t1 ? d1 : ~0u));
      t0 = t0 && d0 == dmin;
      t1 = t1 && d1 == dmin;
      const uint32_t hmin = wave_ext<false>(min(t0 ? f[0].code_hi : ~0u, t1 ? f[1].code_hi : ~0u));
      t0 = t0 && f[0].code_hi == hmin;
      t1 = t1 && f[1].code_hi == hmin;
      const uint32_t lmin = wave_ext<false>(min(t0 ? f[0].code_lo : ~0u, t1 ? f[1].code_lo : ~0u));
      t0 = t0 && f[0].code_lo == lmin;
      t1 = t1 && f[1].code_lo == lmin;
      hit0 = __ballot(t0);
      hit1 = __ballot(t1);
    }
    const int e = hit0 ? __ffsll((unsigned long long)hit0) - 1
                       : 64 + __ffsll((unsigned long long)hit1) - 1;
    const Slot w = bcast(e < 64 ? f[0] : f[1], e & 63);
    const int d = meta_depth(w.meta), rk = meta_rank(w.meta), p = meta_parent(w.meta);

    // 2. the three table values this step needs, read together (clamped
    //    indices; a value is used only when its candidate exists)
    const bool has_child = d < D, has_sib = rk + 1 < K;
    const int32_t t_id = id_at((d - 1) * K + rk);
    const float lp_child = lp_at(min(d, D - 1) * K);
    const float lp_sib = lp_at((d - 1) * K + min(rk + 1, K - 1));

    // 3. the new node
    if (lane == 0) {
      tok[base + k] = t_id;
      par[base + k] = p;
      dep[base + k] = d;
      if (sc) sc[base + k] = w.score;
    }

    // 4. successors: the best child takes slot e, the sibling slot n (or e)
    const uint64_t code = ((uint64_t)w.code_hi << 32) | w.code_lo;
    const uint64_t cc = code << rank_bits, cs = code + 1;
    const Slot child{__fadd_rn(w.score, lp_child), w.score, pack_meta(d + 1, 0, k),
                     (uint32_t)cc, (uint32_t)(cc >> 32)};
    const Slot sib{__fadd_rn(w.pscore, lp_sib), w.pscore, pack_meta(d, rk + 1, p), (uint32_t)cs,
                   (uint32_t)(cs >> 32)};
    const Slot at_e = has_child ? child : (has_sib ? sib : none);
    const int pos_sib = has_child && has_sib ? n : -1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = lane + 64 * q;
      f[q] = pick(idx == e, at_e, f[q]);
      f[q] = pick(idx == pos_sib, sib, f[q]);
    }
    n += pos_sib >= 0 ? 1 : 0;
  }
}


// ---------------------------------------------------------------------------
// Lean builder (budget <= LEAN_MAX_BUDGET, depth_max * topk <= 64 * TAB)
// ---------------------------------------------------------------------------
// At pop k the frontier holds at most k entries, so budgets up to 64 need
// one entry per lane.  A pop reads the taken entry with readlane and
// rewrites only the lanes that change (its slot, and the appended sibling):
// one select per field, where two frontier entries per lane cost twice the
// selects and twice the reduction inputs.  Each entry keeps its score's
// order key, formed once when the entry is written.  The node records (token,
// parent, depth, score) stay in registers too -- node i in lane i & 63,
// slot i >> 6 -- and go to memory once at the end, as does the optional
// visibility: node k's ancestor-or-self bitset is its parent's plus bit k,
// formed when k is taken (parents are taken before their children), so the
// bitsets and positions of ddtree_compile_visibility come out of the same
// launch.
constexpr int LEAN_MAX_BUDGET = 64;
constexpr int LEAN_SLOTS = 2;   // node records per lane: up to 128 nodes in registers
constexpr int LEAN_WORDS = 4;   // bitset words per node record (128 nodes)

// reg with lane lane_idx (uniform) set to v (uniform): one compare, shared by
// the fields written to one lane, and one select each
__device__ inline uint32_t wl(uint32_t reg, int lane_idx, uint32_t v) {
  return (int)threadIdx.x == lane_idx ? v : reg;
}

template <int TAB, bool VIS>
__global__ __launch_bounds__(64) void build_lean_kernel(
    const float* __restrict__ lp, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ roots, const int32_t* __restrict__ qo, int D, int K,
    int max_budget, int rank_bits, int32_t* __restrict__ tok, int32_t* __restrict__ par,
    int32_t* __restrict__ dep, float* __restrict__ sc, const int32_t* __restrict__ prefix, int W,
    uint32_t* __restrict__ bits, int64_t* __restrict__ positions) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int base = qo[r];
  const int Q = qo[r + 1] - base;
  if (Q < 1) return;
  const int B = min(Q - 1, max_budget);
  const int DK = D * K;
  // the request's tables: entry i in lane i & 63, register i >> 6
  uint32_t tl[TAB], ti[TAB];
#pragma unroll
  for (int j = 0; j < TAB; ++j) {
    const int i = lane + 64 * j;
    const bool in = B > 0 && i < DK;
    tl[j] = in ? __float_as_uint(lp[(size_t)r * DK + i]) : 0u;
    ti[j] = in ? (uint32_t)ids[(size_t)r * DK + i] : 0u;
  }
  const int32_t root_tok = roots[r];
  auto tab = [&](const uint32_t* t, int i) {  // entry i (uniform)
    uint32_t v = t[0];
#pragma unroll
    for (int j = 1; j < TAB; ++j) v = (i >> 6) == j ? t[j] : v;
    return lane_val(v, i & 63);
  };

  // node records: every node starts as "not in the tree" (token, parent and
  // depth -1, score 0, only its own bit), the root as itself
  int32_t n_tok[LEAN_SLOTS], n_par[LEAN_SLOTS], n_dep[LEAN_SLOTS];
  uint32_t n_sc[LEAN_SLOTS], n_vis[LEAN_SLOTS][LEAN_WORDS];
#pragma unroll
  for (int q = 0; q < LEAN_SLOTS; ++q) {
    const int i = lane + 64 * q;
    const bool root = i == 0;
    n_tok[q] = root ? root_tok : -1;
    n_par[q] = -1;
    n_dep[q] = root ? 0 : -1;
    n_sc[q] = 0u;
#pragma unroll
    for (int w = 0; w < LEAN_WORDS; ++w) n_vis[q][w] = (i >> 5) == w ? 1u << (i & 31) : 0u;
  }

  // the frontier: one entry per lane, with its score's order key (0 = empty)
  uint32_t fk = 0u, fs = 0u, fp = 0u, fm = 0u, flo = 0u, fhi = 0u;
  if (B > 0 && lane == 0) {  // the root's best child
    const float s0 = __fadd_rn(0.f, __uint_as_float(tl[0]));
    fk = score_key(s0);
    fs = __float_as_uint(s0);
    fm = pack_meta(1, 0, 0);
  }
  int n = 1;
  for (int k = 1; k <= B; ++k) {
    // 1. the best entry: largest score key, ties resolved exactly
    const uint32_t key = fk;
    const uint32_t kmax = wave_ext<true>(key);
    if (kmax == 0u) break;  // empty frontier: only reachable if preconditions are broken
    uint64_t hit = __ballot(key == kmax);
    if (__popcll(hit) > 1) {  // rare: equal scores
      bool tt = (hit >> lane) & 1;
      const uint32_t dmin = wave_ext<false>(tt ? (fm & 0x7f) : ~0u);
      tt = tt && (fm & 0x7f) == dmin;
      const uint32_t hmin = wave_ext<false>(tt ? fhi : ~0u);
      tt = tt && fhi == hmin;
      const uint32_t lmin = wave_ext<false>(tt ? flo : ~0u);
      tt = tt && flo == lmin;
      hit = __ballot(tt);
    }
    const int e = __ffsll((unsigned long long)hit) - 1;
    const float w_score = __uint_as_float(lane_val(fs, e));
    const float w_ps = __uint_as_float(lane_val(fp, e));
    const uint32_t w_meta = lane_val(fm, e);
    const uint64_t code = ((uint64_t)lane_val(fhi, e) << 32) | lane_val(flo, e);
    const int d = meta_depth(w_meta), rk = meta_rank(w_meta), p = meta_parent(w_meta);

    // 2. node k (its record in lane k & 63, slot k >> 6)
    const int32_t t_id = (int32_t)tab(ti, (d - 1) * K + rk);
    const int kl = k & 63, ks = k >> 6;
#pragma unroll
    for (int q = 0; q < LEAN_SLOTS; ++q) {
      if (q != ks) continue;
      n_tok[q] = (int32_t)wl((uint32_t)n_tok[q], kl, (uint32_t)t_id);
      n_par[q] = (int32_t)wl((uint32_t)n_par[q], kl, (uint32_t)p);
      n_dep[q] = (int32_t)wl((uint32_t)n_dep[q], kl, (uint32_t)d);
      n_sc[q] = wl(n_sc[q], kl, __float_as_uint(w_score));
    }
    if (k == B) break;  // no further pop reads the frontier

    // 3. successors: the best child takes slot e, the sibling slot n (or e)
    const bool has_child = d < D, has_sib = rk + 1 < K;
    const float lp_child = __uint_as_float(tab(tl, min(d, D - 1) * K));
    const float lp_sib = __uint_as_float(tab(tl, (d - 1) * K + min(rk + 1, K - 1)));
    const uint64_t cc = code << rank_bits, cs = code + 1;
    const float c_f = __fadd_rn(w_score, lp_child), s_f = __fadd_rn(w_ps, lp_sib);
    const uint32_t c_s = __float_as_uint(c_f), s_s = __float_as_uint(s_f);
    const uint32_t c_k = score_key(c_f), s_k = score_key(s_f);
    const uint32_t c_m = pack_meta(d + 1, 0, k), s_m = pack_meta(d, rk + 1, p);
    if (has_child) {
      fk = wl(fk, e, c_k);
      fs = wl(fs, e, c_s);
      fp = wl(fp, e, __float_as_uint(w_score));
      fm = wl(fm, e, c_m);
      flo = wl(flo, e, (uint32_t)cc);
      fhi = wl(fhi, e, (uint32_t)(cc >> 32));
    }
    if (has_sib) {
      const int at = has_child ? n : e;  // n <= k < B <= 64
      fk = wl(fk, at, s_k);
      fs = wl(fs, at, s_s);
      fp = wl(fp, at, __float_as_uint(w_ps));
      fm = wl(fm, at, s_m);
      flo = wl(flo, at, (uint32_t)cs);
      fhi = wl(fhi, at, (uint32_t)(cs >> 32));
      n += has_child ? 1 : 0;
    }
    if (!has_child && !has_sib) fk = wl(fk, e, 0u);
  }

  // 4. each node's ancestor-or-self bits: walk up the parent records (at
  //    most depth_max steps; every node of the wave walks at once)
  if constexpr (VIS) {
#pragma unroll
    for (int q = 0; q < LEAN_SLOTS; ++q) {
      int j = n_par[q] < lane + 64 * q ? n_par[q] : -1;
      for (int step = 0; step < D && __ballot(j >= 0); ++step) {
        if (j >= 0) {
#pragma unroll
          for (int w = 0; w < LEAN_WORDS; ++w)
            if ((j >> 5) == w) n_vis[q][w] |= 1u << (j & 31);
        }
        // the parent of j: its record in lane j & 63, slot j >> 6
        const int src = j >= 0 ? (j & 63) : lane;
        const int p0 = __shfl(n_par[0], src), p1 = __shfl(n_par[LEAN_SLOTS - 1], src);
        const int pj = j < 0 ? -1 : ((j >> 6) == 0 ? p0 : p1);
        j = pj < j ? pj : -1;  // parents precede their children
      }
    }
  }

  // 5. the records (and bitsets, positions) to memory, one store per lane
  const int64_t P = VIS && positions ? (int64_t)max(prefix[r], 0) : 0;
#pragma unroll
  for (int q = 0; q < LEAN_SLOTS; ++q) {
    const int i = lane + 64 * q;
    if (i >= Q) break;
    tok[base + i] = n_tok[q];
    par[base + i] = n_par[q];
    dep[base + i] = n_dep[q];
    if (sc) sc[base + i] = __uint_as_float(n_sc[q]);
    if constexpr (VIS) {
      for (int w = 0; w < W; ++w) bits[(size_t)(base + i) * W + w] = w < LEAN_WORDS ? n_vis[q][w] : 0u;
      if (positions) positions[base + i] = P + n_dep[q];
    }
  }
  // nodes past the records (only when the device data exceeds the host bounds)
  for (int i = 64 * LEAN_SLOTS + lane; i < Q; i += 64) {
    tok[base + i] = -1;
    par[base + i] = -1;
    dep[base + i] = -1;
    if (sc) sc[base + i] = 0.f;
    if constexpr (VIS) {
      for (int w = 0; w < W; ++w) bits[(size_t)(base + i) * W + w] = (i >> 5) == w ? 1u << (i & 31) : 0u;
      if (positions) positions[base + i] = P - 1;
    }
  }
}
}  // namespace

namespace {

// Host checks of ddtree_build_tree's arguments; fills rank_bits.
int check_build(const char* fn, const float* topk_logprobs, const int32_t* topk_ids,
                const int32_t* root_tokens, const int32_t* qo_indptr, int bs, int depth_max,
                int topk, int max_budget, int32_t* node_tokens, int32_t* node_parents,
                int32_t* node_depths, int& rank_bits) {
  DDTREE_REQUIRE(root_tokens && qo_indptr && node_tokens && node_parents && node_depths,
                 DDTREE_EINVAL, "%s: null required pointer", fn);
  if (max_budget > 0) {
    DDTREE_REQUIRE(topk_logprobs && topk_ids, DDTREE_EINVAL, "%s: null top-k input", fn);
    DDTREE_REQUIRE(depth_max >= 1 && topk >= 1, DDTREE_EINVAL,
                   "%s: depth_max and topk must be >= 1 for a non-empty tree", fn);
    // reachable = sum_{d=1..D} K^d, saturating
    long long reach = 0, pw = 1;
    for (int d = 1; d <= depth_max && reach < (long long)max_budget; ++d) {
      pw = (pw > (1LL << 40) / topk) ? (1LL << 40) : pw * topk;
      reach += pw;
    }
    DDTREE_REQUIRE((long long)max_budget <= reach, DDTREE_EINVAL,
                   "%s: max_budget %d exceeds the %lld reachable rank paths", fn, max_budget,
                   reach);
  }
  rank_bits = 1;
  while ((1 << rank_bits) < topk) ++rank_bits;
  DDTREE_REQUIRE(max_budget == 0 || (long long)depth_max * rank_bits <= 64, DDTREE_EUNSUPPORTED,
                 "%s: depth_max * ceil(log2(topk)) = %lld exceeds 64 bits", fn,
                 (long long)depth_max * rank_bits);
  DDTREE_REQUIRE(max_budget <= 2048, DDTREE_EUNSUPPORTED,
                 "%s: max_budget %d above the supported 2048", fn, max_budget);
  DDTREE_REQUIRE(max_budget == 0 || (long long)depth_max * topk <= 8192, DDTREE_EUNSUPPORTED,
                 "%s: depth_max * topk = %lld above the supported 8192", fn,
                 (long long)depth_max * topk);
  return DDTREE_OK;
}

// registers per lane the lean builder needs for the top-k tables (0: not lean)
int lean_tab(int depth_max, int topk, int max_budget) {
  if (max_budget > LEAN_MAX_BUDGET || depth_max > 127) return 0;
  const long long dk = max_budget > 0 ? (long long)depth_max * topk : 1;
  return dk <= 64 ? 1 : (dk <= 128 ? 2 : (dk <= 256 ? 4 : 0));
}

template <bool VIS>
void launch_lean(int tab, int bs, hipStream_t s, const float* lp, const int32_t* ids,
                 const int32_t* roots, const int32_t* qo, int D, int K, int max_budget,
                 int rank_bits, int32_t* tok, int32_t* par, int32_t* dep, float* sc,
                 const int32_t* prefix, int W, uint32_t* bits, int64_t* positions) {
  auto k = tab == 1 ? build_lean_kernel<1, VIS> : (tab == 2 ? build_lean_kernel<2, VIS> : build_lean_kernel<4, VIS>);
  hipLaunchKernelGGL(k, dim3(bs), dim3(64), 0, s, lp, ids, roots, qo, D, K, max_budget, rank_bits,
                     tok, par, dep, sc, prefix, W, bits, positions);
}

// The tree-building launch of ddtree_build_tree (arguments already checked).
int launch_build(const float* topk_logprobs, const int32_t* topk_ids, const int32_t* root_tokens,
                 const int32_t* qo_indptr, int bs, int depth_max, int topk, int max_budget,
                 int rank_bits, int32_t* node_tokens, int32_t* node_parents, int32_t* node_depths,
                 float* node_scores, hipStream_t s) {
  const int tab = lean_tab(depth_max, topk, max_budget);
  if (tab) {
    launch_lean<false>(tab, bs, s, topk_logprobs, topk_ids, root_tokens, qo_indptr, depth_max,
                       topk, max_budget, rank_bits, node_tokens, node_parents, node_depths,
                       node_scores, nullptr, 0, nullptr, nullptr);
    return ddtree::check_launch("build_tree");
  }
  const size_t staged = max_budget > 0 ? (size_t)depth_max * topk * 8 : 0;  // log-probs + ids
  if (max_budget <= REG_MAX_BUDGET) {
    if ((long long)depth_max * topk <= TAB_REGS * 64)
      hipLaunchKernelGGL(build_tree_reg_kernel<true>, dim3(bs), dim3(64), staged, s, topk_logprobs,
                         topk_ids, root_tokens, qo_indptr, depth_max, topk, max_budget, rank_bits,
                         node_tokens, node_parents, node_depths, node_scores);
    else
      hipLaunchKernelGGL(build_tree_reg_kernel<false>, dim3(bs), dim3(64), staged, s, topk_logprobs,
                         topk_ids, root_tokens, qo_indptr, depth_max, topk, max_budget, rank_bits,
                         node_tokens, node_parents, node_depths, node_scores);
  } else {
    const size_t lds = (size_t)(max_budget + 2) * (8 + 4 * 5) + staged;
    hipLaunchKernelGGL(build_tree_kernel, dim3(bs), dim3(64), lds, s, topk_logprobs, topk_ids,
                       root_tokens, qo_indptr, depth_max, topk, max_budget, rank_bits, node_tokens,
                       node_parents, node_depths, node_scores);
  }
  return ddtree::check_launch("build_tree");
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
  int rank_bits = 1;
  int rc = check_build("build_tree", topk_logprobs, topk_ids, root_tokens, qo_indptr, bs, depth_max,
                       topk, max_budget, node_tokens, node_parents, node_depths, rank_bits);
  if (rc != DDTREE_OK) return rc;
  return launch_build(topk_logprobs, topk_ids, root_tokens, qo_indptr, bs, depth_max, topk,
                      max_budget, rank_bits, node_tokens, node_parents, node_depths, node_scores,
                      ddtree::as_stream(stream));
}

// defined in visibility.hip
int ddtree_visibility_launch(const int32_t* node_parents, const int32_t* node_depths,
                             const int32_t* qo_indptr, const int32_t* prefix_lens, int bs,
                             int max_q_len, int words_per_row, uint32_t* vis_bits,
                             int64_t* positions, hipStream_t s);

extern "C" int ddtree_build_tree_visibility(
    const float* topk_logprobs, const int32_t* topk_ids, const int32_t* root_tokens,
    const int32_t* qo_indptr, const int32_t* prefix_lens, int bs, int depth_max, int topk,
    int max_budget, int max_q_len, int words_per_row, int32_t* node_tokens,
    int32_t* node_parents, int32_t* node_depths, float* node_scores, uint32_t* vis_bits,
    int64_t* positions, void* stream) {
  ddtree::clear_error();
  const char* fn = "build_tree_visibility";
  DDTREE_REQUIRE(bs >= 0, DDTREE_EINVAL, "%s: bs must be >= 0 (got %d)", fn, bs);
  DDTREE_REQUIRE(max_budget >= 0, DDTREE_EINVAL, "%s: max_budget must be >= 0", fn);
  if (bs == 0) return DDTREE_OK;
  int rank_bits = 1;
  int rc = check_build(fn, topk_logprobs, topk_ids, root_tokens, qo_indptr, bs, depth_max, topk,
                       max_budget, node_tokens, node_parents, node_depths, rank_bits);
  if (rc != DDTREE_OK) return rc;
  DDTREE_REQUIRE(max_q_len >= 1, DDTREE_EINVAL, "%s: max_q_len must be >= 1", fn);
  DDTREE_REQUIRE(vis_bits, DDTREE_EINVAL, "%s: null vis_bits", fn);
  DDTREE_REQUIRE(!positions || prefix_lens, DDTREE_EINVAL, "%s: positions need prefix_lens", fn);
  DDTREE_REQUIRE((long long)words_per_row * 32 >= max_q_len, DDTREE_EINVAL,
                 "%s: words_per_row %d < ceil(max_q_len/32) for max_q_len %d", fn, words_per_row,
                 max_q_len);
  hipStream_t s = ddtree::as_stream(stream);
  const int tab = lean_tab(depth_max, topk, max_budget);
  if (tab && max_q_len <= 64 * LEAN_SLOTS) {
    launch_lean<true>(tab, bs, s, topk_logprobs, topk_ids, root_tokens, qo_indptr, depth_max, topk,
                      max_budget, rank_bits, node_tokens, node_parents, node_depths, node_scores,
                      prefix_lens, words_per_row, vis_bits, positions);
    return ddtree::check_launch(fn);
  }
  rc = launch_build(topk_logprobs, topk_ids, root_tokens, qo_indptr, bs, depth_max, topk,
                    max_budget, rank_bits, node_tokens, node_parents, node_depths, node_scores, s);
  if (rc != DDTREE_OK) return rc;
  return ddtree_visibility_launch(node_parents, node_depths, qo_indptr, prefix_lens, bs, max_q_len,
                                  words_per_row, vis_bits, positions, s);
}
