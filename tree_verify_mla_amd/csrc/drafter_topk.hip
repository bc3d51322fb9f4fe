// ddtree_drafter_topk: per-depth top-k log-probabilities of the drafter's
// logits -- the builder's input ("The DDTree CUDA Graph Fix ...", section
// "The DDTree Architecture: Confirming Multiple-Path Evaluation": from each
// depth position's hidden state the vocabulary head gives the top-k
// candidate tokens with their log-probabilities).
//
// The log-probability of token j of a row is x_j - lse, lse = log sum_i e^x_i
// over the whole vocabulary; the top k are the k largest, equal values in
// ascending token id.  lse is one constant per row, so the order is the order
// of the logits themselves, and only the k values need the subtraction.
//
// Two kernels, in the shape of a vocabulary split across ranks:
// * chunk_kernel: workgroup (row, chunk) reads CHUNK consecutive logits of
//   its row once (32 per thread, kept in registers) and writes the chunk's
//   max m_c, its sum s_c of e^(x - m_c), and its k best (value, id), best
//   first (32-bit order keys, the smallest id among equal keys): each wave
//   ranks its logits at or above a threshold that at least k of them reach
//   (rounds of an argmax over its entries where equal or -inf logits leave
//   no useful threshold), and each wave's list is then placed by counting
//   the entries of the other three lists before each of its entries;
//   (a row of one chunk -- vocabularies up to CHUNK -- is final there:
//   the chunk writes x - lse and the ids itself and no merge runs);
// * merge_kernel: one wavefront per row folds the chunks' (m_c, s_c) into
//   M = max m_c and S = sum_c s_c e^(m_c - M), lse = M + log S, and takes
//   the row's k best out of the chunks' candidates (the j-th best of a row
//   is among the j best of its chunk), writing x - lse and the ids.
// Everything is fp32; exponentials and the log are the hardware's.
#include <climits>
#include <type_traits>

#include "common.h"

namespace {

constexpr int CT = 256;            // threads per chunk workgroup
constexpr int EPT = 32;            // logits per thread
constexpr int CHUNK = CT * EPT;    // logits per chunk
constexpr int KMAX = 32;           // largest k
constexpr float LOG2E = 1.44269504088896340736f;
constexpr int MERGE_PER_LANE = 16; // chunk candidates per lane in the merge (C * k <= 1024)
constexpr int STAGE = 64;          // a wave's logits at or above its threshold, staged in LDS

// order-preserving map of a finite fp32 to uint32 (larger value -> larger key)
__device__ inline uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.f);  // -0 + 0 = +0: -0 ties with +0
  // negative: all bits flipped; otherwise the sign bit set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
// its inverse (key 0x80000000u gives +0)
__device__ inline float funkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// element e (0 <= e < CHUNK) of the chunk sits in thread t, register j:
//   VEC (16-byte loads of W = 16 / sizeof(T) elements): e = W t + W CT (j / W) + j % W
//   scalar loads:                                      e = t + CT j
template <typename T, bool VEC>
__device__ inline int elem_of(int t, int j) {
  if constexpr (VEC) {
    constexpr int W = 16 / (int)sizeof(T);
    return W * t + W * CT * (j / W) + j % W;
  } else {
    return t + CT * j;
  }
}

// the same with a runtime register index (arithmetic only)
template <typename T, bool VEC>
__device__ inline int elem_of_rt(int t, int j) {
  if constexpr (VEC) {
    constexpr int W = 16 / (int)sizeof(T);
    return W * t + W * CT * (j / W) + j % W;
  } else {
    return t + CT * j;
  }
}

// wave-wide maximum (MAX) or minimum of x, uniform result: DPP inside each
// 16-lane row (swap neighbours, pairs, then mirror halves and rows), then
// the four row results through scalar registers
template <bool MAX>
__device__ inline uint32_t wave_ext(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  // the operation's identity as the DPP fill value lets the move fold into it
  constexpr int ID = MAX ? 0 : -1;
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)x, 0xB1, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)x, 0x4E, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)x, 0x141, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(ID, (int)x, 0x140, 0xF, 0xF, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return op(op(r0, r1), op(r2, r3));
}

// Whether this lane holds the wave's best (key, id): the largest key, then
// the smallest id among the lanes that hold it (ids are unique).  The id
// reduction runs only when several lanes hold the largest key.  gk: the
// wave's largest key.
__device__ inline bool wave_owner(uint32_t key, uint32_t id, uint32_t& gk) {
  gk = wave_ext<true>(key);
  uint64_t hold = __ballot(key == gk);
  if (__popcll(hold) > 1) {
    const uint32_t gid = wave_ext<false>(key == gk ? id : 0xffffffffu);
    hold = __ballot(key == gk && id == gid);
  }
  return (hold >> (threadIdx.x & 63)) & 1ull;
}

// (m, s) <- (m, s) + (m2, s2): a pair is a max and a sum of e^(x - max); a
// max of -inf carries no mass
__device__ inline void lse_add(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float a = m == -INFINITY ? 0.f : s * __expf(m - M);
  const float b = m2 == -INFINITY ? 0.f : s2 * __expf(m2 - M);
  m = M;
  s = a + b;
}

// the wave's (m, s) in every lane: inside each 16-lane row by DPP (both
// partners of a step form the same sum), then the four rows in order
__device__ inline void wave_lse(float& m, float& s) {
  auto step = [&](auto ctrl) {
    const float m2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), ctrl.value, 0xF, 0xF, false));
    const float s2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), ctrl.value, 0xF, 0xF, false));
    lse_add(m, s, m2, s2);
  };
  step(std::integral_constant<int, 0xB1>{});
  step(std::integral_constant<int, 0x4E>{});
  step(std::integral_constant<int, 0x141>{});
  step(std::integral_constant<int, 0x140>{});
  float r_m[4], r_s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r_m[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16 * i));
    r_s[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 16 * i));
  }
  lse_add(r_m[0], r_s[0], r_m[1], r_s[1]);
  lse_add(r_m[2], r_s[2], r_m[3], r_s[3]);
  lse_add(r_m[0], r_s[0], r_m[2], r_s[2]);
  m = r_m[0];
  s = r_s[0];
}

template <typename T>
__device__ inline float to_f32(T x) {
  if constexpr (sizeof(T) == 2) return (float)x;
  else return x;
}

// Workgroup (row, c).  FULL: the chunk holds CHUNK logits (every chunk but
// a row's last), so no element needs a bounds check.
template <typename T, bool VEC, bool FULL>
__device__ __forceinline__ void chunk_body(const T* __restrict__ logits, int vocab, int C, int k,
                                           float* __restrict__ ws_ms, float* __restrict__ ws_val,
                                           int32_t* __restrict__ ws_id, float* __restrict__ out_val,
                                           int32_t* __restrict__ out_id, int row, int c,
                                           float* red_m, float* red_s, uint2 (*cand)[KMAX],
                                           uint2 (*stage)[STAGE]) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const long long c0 = (long long)c * CHUNK;          // first element of the chunk in its row
  const int n = FULL ? CHUNK : (int)min((long long)CHUNK, vocab - c0);  // elements of the chunk
  const T* src = logits + (size_t)row * vocab + c0;

  float x[EPT];
  if constexpr (VEC) {
    constexpr int W = 16 / (int)sizeof(T);
    typedef __attribute__((__vector_size__(16))) char v16;
#pragma unroll
    for (int q = 0; q < EPT / W; ++q) {
      const int e = W * t + W * CT * q;
      if (FULL || e + W <= n) {
        const v16 raw = *reinterpret_cast<const v16*>(src + e);
        const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int i = 0; i < W; ++i) x[W * q + i] = to_f32(vals[i]);
      } else {
#pragma unroll
        for (int i = 0; i < W; ++i) x[W * q + i] = e + i < n ? to_f32(src[e + i]) : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = t + CT * j;
      x[j] = FULL || e < n ? to_f32(src[e]) : -INFINITY;
    }
  }
  uint32_t live = 0;  // bit j: register j holds an element of the chunk still in play
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if (FULL || elem_of<T, VEC>(t, j) < n) live |= 1u << j;

  // The chunk's max m and sum s of e^(x - m): each lane's own (max, sum)
  // first, then the wave's and the workgroup's by the pairwise rule
  // (m, s) + (m', s') = (M, s e^(m - M) + s' e^(m' - M)), M = max(m, m'), so
  // the workgroup meets at one barrier only.  Elements with nothing in them
  // (a masked tail of the vocabulary) give max -inf and sum 0, which the
  // merge skips; their reference is 0, so e^(-inf - 0) = 0.
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPT; ++j) m = fmaxf(m, x[j]);
  const float lane_max = m;
  // e^(x - m) as 2^(x log2 e - m log2 e): one fused multiply-add per element
  const float mref = (m == -INFINITY ? 0.f : m) * LOG2E;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if ((live >> j) & 1u) s += __builtin_amdgcn_exp2f(__fmaf_rn(x[j], LOG2E, -mref));
  wave_lse(m, s);
  if (lane == 0) {
    red_m[wave] = m;
    red_s[wave] = s;
  }
  const size_t slot = (size_t)row * C + c;

  // The chunk's k best (the largest value, then the smallest id), in two
  // steps with one barrier between them.  Keys are 32-bit order keys; 0
  // means nothing (every float's key is larger).
  // 1. each wave takes its own k best, cand[wave][0 .. k-1].
  //    Threshold form: the k-th largest of the lanes' maxima, tau, is at most
  //    the wave's k-th largest logit (each of those k lanes holds a logit
  //    >= tau), so the wave's k best are among its logits >= tau -- with
  //    distinct values, little more than k of them.  tau comes from rounds
  //    of a wave maximum over the lanes' maxima (the lanes holding a round's
  //    maximum leave together, so equal maxima count once each); the logits
  //    >= tau go to LDS, and each takes the place its rank among them gives
  //    (the number of staged entries before it in the order).  The form
  //    needs tau > -inf (a logit >= tau is then real: masked elements hold
  //    -inf) and at most STAGE logits >= tau; a wave where either fails (a
  //    run of equal or -inf logits) takes the general form below.
  const uint32_t key_ninf = fkey(-INFINITY);
  bool general = false;
  {
    uint32_t cur = fkey(lane_max), tk = 0u;
    int got = 0;  // lanes whose maximum is >= tk
    while (got < k) {
      const uint32_t gk = wave_ext<true>(cur);
      if (gk <= key_ninf) break;
      got += (int)__popcll(__ballot(cur == gk));
      cur = cur == gk ? 0u : cur;
      tk = gk;
    }
    general = got < k;
    if (!general) {
      const float tau = funkey(tk);
      int nw = 0;  // logits >= tau so far (wave-uniform)
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const bool pass = x[j] >= tau;
        const uint64_t b = __ballot(pass);
        if (b != 0ull) {
          const int pos = nw + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
          if (pass && pos < STAGE)
            stage[wave][pos] = make_uint2(fkey(x[j]), (uint32_t)(c0 + elem_of<T, VEC>(t, j)));
          nw += (int)__popcll(b);
        }
      }
      general = nw > STAGE;
      if (!general) {
        uint32_t mk = 0u, mid = 0xffffffffu;
        if (lane < nw) {
          const uint2 v = stage[wave][lane];
          mk = v.x, mid = v.y;
        }
        int rank = 0;
#pragma unroll 4
        for (int i = 0; i < nw; ++i) {
          const uint2 v = stage[wave][i];  // the same entry in every lane
          rank += (int)((v.x > mk) | ((v.x == mk) & (v.y < mid)));
        }
        if (lane < nw && rank < k) cand[wave][rank] = make_uint2(mk, mid);
      }
    }
  }
  // General form: a lane keeps its two best entries (its registers hold ids
  // in ascending order, so of equal keys the first is the smaller id); a
  // round is the wave maximum of the lanes' first keys, then the smallest id
  // among the lanes that hold it, and the owner moves its second entry up.
  // A lane that has given up both looks again, for the best entries after
  // the last one it gave up in (key descending, id ascending) order -- rare,
  // and only that lane's wave waits for it.
  // The keys take the logits' place (a key gives its logit back), which
  // keeps the kernel within the registers of six waves per SIMD.
  if (general) {
    uint32_t key[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) key[j] = ((live >> j) & 1u) ? fkey(x[j]) : 0u;
    // the two best entries after (bk, bj) in the order; bk = ~0u: from the top
    auto best_two = [&](uint32_t lk, int lj, uint32_t& k1, int& j1, uint32_t& k2, int& j2) {
      k1 = 0u, j1 = 0, k2 = 0u, j2 = 0;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        // bitwise, not short-circuit: no branches around the comparisons
        const bool after = (key[j] < lk) | ((key[j] == lk) & (j > lj));
        const uint32_t kj = after ? key[j] : 0u;
        const bool first = kj > k1, second = !first && kj > k2;
        k2 = first ? k1 : (second ? kj : k2);
        j2 = first ? j1 : (second ? j : j2);
        k1 = first ? kj : k1;
        j1 = first ? j : j1;
      }
    };
    uint32_t k1, k2;
    int j1, j2;
    best_two(0xffffffffu, -1, k1, j1, k2, j2);
    for (int r = 0; r < k; ++r) {
      const uint32_t myid = k1 ? (uint32_t)(c0 + elem_of_rt<T, VEC>(t, j1)) : 0xffffffffu;
      uint32_t wk;
      const bool owner = wave_owner(k1, myid, wk);
      if (wk == 0u) {  // fewer than k logits in the wave
        if (lane == 0) cand[wave][r] = make_uint2(0u, 0xffffffffu - (uint32_t)(wave * KMAX + r));
      } else if (owner) {
        cand[wave][r] = make_uint2(wk, myid);
        if (k2 != 0u) {
          k1 = k2, j1 = j2, k2 = 0u;
        } else {
          best_two(k1, j1, k1, j1, k2, j2);
        }
      }
    }
  }
  __syncthreads();
  // the workgroup's (max, sum), waves in order (every wave forms it)
  float mc = red_m[0], sc = red_s[0];
  lse_add(mc, sc, red_m[1], red_s[1]);
  lse_add(mc, sc, red_m[2], red_s[2]);
  lse_add(mc, sc, red_m[3], red_s[3]);
  if (t == 0 && C > 1) {
    ws_ms[2 * slot] = mc;
    ws_ms[2 * slot + 1] = sc;
  }
  // A row of one chunk needs no merge: its log-sum-exp is the chunk's (the
  // merge's fold of a single (max, sum) returns it exactly), and the chunk's
  // k best, best first, are the row's.
  const bool whole_row = C == 1;
  const float lse = mc + __logf(sc);
  // 2. each wave places its own list's entries: the chunk-wide place of
  //    entry p of a wave's list is p plus the number of entries of the other
  //    three lists before it in the order (each list is sorted, so places
  //    0 .. k-1 are each taken once); entries placed at k or later drop out.
  //    Entries standing for nothing (key 0, distinct ids above every token
  //    id) come after every real one.
  if (lane < k) {
    const uint2 me = cand[wave][lane];
    int place = lane;
#pragma unroll
    for (int d = 1; d < CT / 64; ++d) {
      const int w2 = (wave + d) & (CT / 64 - 1);
#pragma unroll 4
      for (int q = 0; q < k; ++q) {
        const uint2 v = cand[w2][q];  // the same entry in every lane
        place += (int)((v.x > me.x) | ((v.x == me.x) & (v.y < me.y)));
      }
    }
    if (place < k) {
      if (whole_row) {
        out_val[(size_t)row * k + place] = funkey(me.x) - lse;
        out_id[(size_t)row * k + place] = (int32_t)me.y;
      } else if (me.x == 0u) {
        ws_val[slot * k + place] = -INFINITY;
        ws_id[slot * k + place] = INT_MAX;
      } else {
        ws_val[slot * k + place] = funkey(me.x);
        ws_id[slot * k + place] = (int32_t)me.y;
      }
    }
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(CT) void chunk_kernel(const T* __restrict__ logits, int vocab, int C,
                                                   int k, float* __restrict__ ws_ms,
                                                   float* __restrict__ ws_val,
                                                   int32_t* __restrict__ ws_id,
                                                   float* __restrict__ out_val,
                                                   int32_t* __restrict__ out_id) {
  __shared__ float red_m[CT / 64], red_s[CT / 64];
  __shared__ uint2 cand[CT / 64][KMAX];  // each wave's k best: (key, id)
  __shared__ uint2 stage[CT / 64][STAGE];  // each wave's logits at or above its threshold
  const int row = blockIdx.x / C, c = blockIdx.x % C;
  if ((long long)(c + 1) * CHUNK <= vocab)
    chunk_body<T, VEC, true>(logits, vocab, C, k, ws_ms, ws_val, ws_id, out_val, out_id, row, c, red_m,
                             red_s, cand, stage);
  else
    chunk_body<T, VEC, false>(logits, vocab, C, k, ws_ms, ws_val, ws_id, out_val, out_id, row, c, red_m,
                              red_s, cand, stage);
}

__global__ __launch_bounds__(64) void merge_kernel(int C, int k, const float* __restrict__ ws_ms,
                                                   const float* __restrict__ ws_val,
                                                   const int32_t* __restrict__ ws_id,
                                                   float* __restrict__ out_val,
                                                   int32_t* __restrict__ out_id) {
  const int row = blockIdx.x, lane = threadIdx.x;
  // the chunks' candidates, MERGE_PER_LANE per lane (candidate i in lane
  // i % 64); k rounds as in the chunks: each lane keeps its two best (the
  // larger key, then the smaller id), a round takes the wave maximum key and
  // then the smallest id holding it, and the owner moves its second up (or,
  // having given up both, looks again after the last one)
  const int nc = C * k;
  const float* cv = ws_val + (size_t)row * nc;
  const int32_t* ci = ws_id + (size_t)row * nc;
  uint32_t key[MERGE_PER_LANE], id[MERGE_PER_LANE];
  float val[MERGE_PER_LANE];
#pragma unroll
  for (int q = 0; q < MERGE_PER_LANE; ++q) {
    const int i = lane + 64 * q;
    const bool in = i < nc;
    const int32_t cid = in ? ci[i] : INT_MAX;  // both loads issued together:
    const float cvv = in ? cv[i] : 0.f;        // neither waits for the other
    const bool real = cid != INT_MAX;
    val[q] = cvv;
    key[q] = real ? fkey(cvv) : 0u;
    id[q] = real ? (uint32_t)cid : 0xffffffffu;
  }
  // (the candidates' loads above are issued first: the two sets are
  // independent, so the wave waits for memory once)
  const float* ms = ws_ms + (size_t)row * C * 2;
  // the row's (M, S) from the chunks' (m_c, s_c) by the pairwise rule, 64
  // chunks at a time in a fixed order (chunks without mass, max -inf, add
  // nothing; the row needs at least one finite logit)
  float M = -INFINITY, S = 0.f;
  for (int c0 = 0; c0 < C; c0 += 64) {
    const int c = c0 + lane;
    float mb = c < C ? ms[2 * c] : -INFINITY;
    float sb = c < C && mb != -INFINITY ? ms[2 * c + 1] : 0.f;
    wave_lse(mb, sb);
    lse_add(M, S, mb, sb);
  }
  const float lse = M + __logf(S);

  if (C <= 64) {
    // Each chunk wrote its candidates best first, so the row's k best are a
    // merge of C sorted lists: lane c follows chunk c's list, and a round
    // takes the best head (the largest key, then the smallest id) and moves
    // the winner's head along -- one LDS read, where the general path below
    // may rescan a lane's candidates.
    __shared__ uint32_t s_key[64 * MERGE_PER_LANE], s_id[64 * MERGE_PER_LANE];
    __shared__ float s_val[64 * MERGE_PER_LANE];
#pragma unroll
    for (int q = 0; q < MERGE_PER_LANE; ++q) {
      const int i = lane + 64 * q;
      if (i < nc) {
        s_key[i] = key[q];
        s_id[i] = id[q];
        s_val[i] = val[q];
      }
    }
    __syncthreads();
    const int base = lane * k;
    int pos = 0;
    uint32_t hk = lane < C ? s_key[base] : 0u, hid = lane < C ? s_id[base] : 0xffffffffu;
    float hv = lane < C ? s_val[base] : 0.f;
    for (int r = 0; r < k; ++r) {
      uint32_t gk;
      const bool owner = wave_owner(hk, hid, gk);
      if (gk != 0u && owner) {
        out_val[(size_t)row * k + r] = hv - lse;
        out_id[(size_t)row * k + r] = (int32_t)hid;
        ++pos;
        hk = pos < k ? s_key[base + pos] : 0u;
        hid = pos < k ? s_id[base + pos] : 0xffffffffu;
        hv = pos < k ? s_val[base + pos] : 0.f;
      }
    }
    return;
  }

  // a lane's two best candidates after (lk, lid) in (key descending, id
  // ascending) order; lk = ~0u: from the top (ids are unique)
  auto best_two = [&](uint32_t lk, uint32_t lid, uint32_t& k1, uint32_t& i1, float& v1,
                      uint32_t& k2, uint32_t& i2, float& v2) {
    k1 = 0u, i1 = 0xffffffffu, v1 = 0.f, k2 = 0u, i2 = 0xffffffffu, v2 = 0.f;
#pragma unroll
    for (int q = 0; q < MERGE_PER_LANE; ++q) {
      const bool after = key[q] < lk || (key[q] == lk && id[q] > lid);
      const uint32_t kq = after ? key[q] : 0u;
      const bool first = kq != 0u && (kq > k1 || (kq == k1 && id[q] < i1));
      const bool second = !first && kq != 0u && (kq > k2 || (kq == k2 && id[q] < i2));
      k2 = first ? k1 : (second ? kq : k2);
      i2 = first ? i1 : (second ? id[q] : i2);
      v2 = first ? v1 : (second ? val[q] : v2);
      k1 = first ? kq : k1;
      i1 = first ? id[q] : i1;
      v1 = first ? val[q] : v1;
    }
  };
  uint32_t k1, i1, k2, i2;
  float v1, v2;
  best_two(0xffffffffu, 0u, k1, i1, v1, k2, i2, v2);
  for (int r = 0; r < k; ++r) {
    uint32_t gk;
    const bool owner = wave_owner(k1, i1, gk);
    if (gk != 0u && owner) {
      out_val[(size_t)row * k + r] = v1 - lse;
      out_id[(size_t)row * k + r] = (int32_t)i1;
      if (k2 != 0u) {
        k1 = k2, i1 = i2, v1 = v2, k2 = 0u;
      } else {
        best_two(k1, i1, k1, i1, v1, k2, i2, v2);
      }
    }
  }
}

}  // namespace

extern "C" size_t ddtree_drafter_topk_workspace_size(int rows, int vocab, int topk) {
  if (rows <= 0 || vocab <= 0 || topk < 1) return 0;
  const long long C = ((long long)vocab + CHUNK - 1) / CHUNK;
  return (size_t)((long long)rows * C * (2 + 2 * topk) * 4);
}

extern "C" int ddtree_drafter_topk(const void* logits, int dtype, int rows, int vocab, int topk,
                                   float* topk_logprobs, int32_t* topk_ids, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  ddtree::clear_error();
  DDTREE_REQUIRE(rows >= 0, DDTREE_EINVAL, "drafter_topk: rows must be >= 0");
  if (rows == 0) return DDTREE_OK;
  DDTREE_REQUIRE(logits && topk_logprobs && topk_ids, DDTREE_EINVAL,
                 "drafter_topk: null required pointer");
  DDTREE_REQUIRE(dtype == DDTREE_F32 || dtype == DDTREE_BF16, DDTREE_EINVAL,
                 "drafter_topk: unknown dtype %d", dtype);
  DDTREE_REQUIRE(vocab >= 1 && topk >= 1 && topk <= vocab, DDTREE_EINVAL,
                 "drafter_topk: need 1 <= topk <= vocab (topk %d, vocab %d)", topk, vocab);
  DDTREE_REQUIRE(topk <= KMAX, DDTREE_EUNSUPPORTED, "drafter_topk: topk %d above %d", topk, KMAX);
  const long long C = ((long long)vocab + CHUNK - 1) / CHUNK;
  DDTREE_REQUIRE(C * topk <= 64LL * MERGE_PER_LANE, DDTREE_EUNSUPPORTED,
                 "drafter_topk: vocab %d with topk %d exceeds %d chunk candidates", vocab, topk,
                 64 * MERGE_PER_LANE);
  DDTREE_REQUIRE((long long)rows * C < (1LL << 31), DDTREE_EUNSUPPORTED,
                 "drafter_topk: grid too large");
  const size_t need = ddtree_drafter_topk_workspace_size(rows, vocab, topk);
  DDTREE_REQUIRE(workspace && workspace_bytes >= need, DDTREE_EWORKSPACE,
                 "drafter_topk: workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  float* ws_ms = static_cast<float*>(workspace);
  float* ws_val = ws_ms + (size_t)rows * C * 2;
  int32_t* ws_id = reinterpret_cast<int32_t*>(ws_val + (size_t)rows * C * topk);
  hipStream_t s = ddtree::as_stream(stream);
  const dim3 grid((unsigned)(rows * C));
  const bool aligned = ((uintptr_t)logits & 15) == 0;
  if (dtype == DDTREE_F32) {
    const float* x = static_cast<const float*>(logits);
    if (aligned && vocab % 4 == 0)
      hipLaunchKernelGGL((chunk_kernel<float, true>), grid, dim3(CT), 0, s, x, vocab, (int)C, topk,
                         ws_ms, ws_val, ws_id, topk_logprobs, topk_ids);
    else
      hipLaunchKernelGGL((chunk_kernel<float, false>), grid, dim3(CT), 0, s, x, vocab, (int)C, topk,
                         ws_ms, ws_val, ws_id, topk_logprobs, topk_ids);
  } else {
    const __bf16* x = static_cast<const __bf16*>(logits);
    if (aligned && vocab % 8 == 0)
      hipLaunchKernelGGL((chunk_kernel<__bf16, true>), grid, dim3(CT), 0, s, x, vocab, (int)C,
                         topk, ws_ms, ws_val, ws_id, topk_logprobs, topk_ids);
    else
      hipLaunchKernelGGL((chunk_kernel<__bf16, false>), grid, dim3(CT), 0, s, x, vocab, (int)C,
                         topk, ws_ms, ws_val, ws_id, topk_logprobs, topk_ids);
  }
  int rc = ddtree::check_launch("drafter_topk(chunks)");
  if (rc != DDTREE_OK || C == 1) return rc;  // rows of one chunk are final already
  hipLaunchKernelGGL(merge_kernel, dim3(rows), dim3(64), 0, s, (int)C, topk, ws_ms, ws_val, ws_id,
                     topk_logprobs, topk_ids);
  return ddtree::check_launch("drafter_topk(merge)");
}
