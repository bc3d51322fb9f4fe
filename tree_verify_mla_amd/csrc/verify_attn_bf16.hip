// bf16 verify attention on gfx950 matrix cores.
//
// Workgroup = NW wavefronts = one tile of 16*NW query rows of one request.
// Waves pair up: both waves of pair g own the same 32 query rows; wave half
// h contracts latent features [288h, 288h+288) of the score and produces
// output features [256h, 256h+256).  The tile walks its KV columns in
// blocks of 32; each block is gathered once from the slot pool into LDS and
// shared by all rows -- the prefix is read once for every tree node and head
// ("The DDTree CUDA Graph Fix ...", section "The DDTree Architecture:
// Confirming Multiple-Path Evaluation").
//
// Per block and wave pair (32 rows x 32 columns):
//   partial S^T[32 col x 32 row] = K[32 x 288] . Q^T[288 x 32]   18 x mfma_f32_32x32x16_bf16
//     A = latent rows from LDS (ds_read_b128), B = the wave's half of the
//     queries, kept in registers for the whole tile.  With columns as the
//     MFMA row index each lane's accumulator holds ONE query row, so the
//     row max is one cross-half exchange and the output rescale is one
//     multiplier per lane.  The two halves are summed through LDS.
//   mask: prefix columns always visible; column P + j visible iff bit j of
//     the row's ancestor bitset is set (tail blocks only).
//   online softmax in base 2 (identical in both waves); P^T rounded to bf16.
//   O^T[256 x 32 row] += V^T[256 x 32 col] . P^T                16 x mfma_f32_32x32x16_bf16
//     A = c_kv columns read transposed from LDS with ds_read_b64_tr_b16,
//     B = P^T straight from the score accumulator: the columns' order inside
//     the k dimension is permuted to match the accumulator layout, so P
//     never moves between lanes.
// Splitting the pair this way keeps each LDS byte feeding 32 rows while a
// wave needs only 72 VGPRs of queries and 128 accumulators of output.
//
// Block buffer layout.  A block is 32 latent rows x 72 chunks of 16 bytes,
// stored as 36 groups of 1 KB: group 2m + h holds chunks 4m .. 4m+3 of rows
// 16h .. 16h+15, and 16-byte position 4u + v of the group holds chunk
// 4m + ((v - (u >> 2)) & 3) of row 16h + u.
// * gather: one global_load_lds_dwordx4 fills one group (lane = position).
//   Each 4-lane quad reads one 64-byte span of one row (a quarter of the
//   lanes' cache lines, coalesced), and wave w fetches rows 16 (w & 1) + l/4,
//   features [288 (w >> 1), +288) of them: one pool address per lane and
//   block, the 64-byte steps in the instruction's immediate offset.
// * score fragment (k-step j, lane l: row l & 31, chunk 2j + (l >> 5)): two
//   base addresses (j even / odd) plus an immediate 2 KB * (j >> 1).
// * transposed value fragments (4 rows x 16 features per 16 lanes): two
//   base addresses plus immediates.
// gfx950 LDS has 64 four-byte banks; a b128 read is serviced 16 lanes at a
// time, a b64 (and the transposing b64) read 32 lanes at a time.  The
// rotation by (u >> 2) puts the lanes of each phase of both patterns on 16
// distinct 16-byte positions mod 256 bytes, so neither has bank conflicts.
//
// Pipeline: four block buffers, two blocks in flight.  Iteration b holds the
// partial scores of block b; it starts the gather of block b+3, completes
// S(b) with the partner's half and runs its softmax under the 18 score
// MFMAs of block b+1, then runs the 16 value MFMAs of block b with the rest
// of the exponentials underneath and hands S(b+1)'s half to the partner.
#include "attn_common.h"
#include "common.h"

namespace ddtree {
namespace attn {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short __attribute__((ext_vector_type(4))) i16x4_t;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int ROWB = LATENT * 2;   // 1152 bytes per latent row
constexpr int BUFB = KB * ROWB;    // 36864 bytes per block buffer
constexpr int LOADS = BUFB / 1024; // 36 one-KB groups per block
constexpr int NBUF = 4;            // block buffers: two blocks in flight
constexpr int XCH = 64 * 64;       // bytes per wave of score-exchange space (64 lanes x 16 f32)
constexpr int KS_HALF = 18;        // k-steps of 16 features per half of the 576-wide score
constexpr int FB_HALF = 8;         // 32-feature output blocks per half of the 512 outputs
constexpr float LN2 = 0.693147180559945309f;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14)
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14); }
constexpr int WAIT_LGKM0 = 0xF | (7 << 4) | (0 << 8) | (3 << 14);


// Workgroup barrier that waits only for this wave's LDS traffic, leaving the
// global->LDS gathers of later blocks in flight (__syncthreads() would wait
// for every outstanding memory operation).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
__device__ inline long long uni64(long long x) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(x & 0xffffffffLL));
  const int hi = __builtin_amdgcn_readfirstlane((int)(x >> 32));
  return ((long long)hi << 32) | (unsigned int)lo;
}

// Every lane computed the same request geometry from the same loads; saying
// so lets the compiler keep it in scalar registers and branch on it.
__device__ inline Geom uniform(Geom g) {
  g.q0 = uni(g.q0); g.Q = uni(g.Q); g.kv0 = uni(g.kv0); g.N = uni(g.N);
  g.P = uni(g.P); g.R = uni(g.R); g.T = uni(g.T); g.NB = uni(g.NB);
  return g;
}

__device__ inline bf16x8_t lds_read_b128(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(p);
}

__device__ inline bf16x4_t lds_read_tr(const lds_char* p) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4_t*>(const_cast<lds_char*>(p)));
  return __builtin_bit_cast(bf16x4_t, v);
}

__device__ inline float other_half(float x) {
  // value of lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(Params p) {
  constexpr int MT = 16 * NW;
  static_assert(MT == MT_BF16, "tile rows must match the schedule");
  static_assert(NW == 4, "the block layout splits the gather over 2 x 2 waves");
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * BUFB + NW * XCH];
  lds_char* lds = (lds_char*)smem;  // generic -> LDS address space
  lds_char* xch = lds + NBUF * BUFB;

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int pair = wave >> 1, half = wave & 1;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q);
  const char* __restrict__ poolb = static_cast<const char*>(p.pool);
  const int xmine = wave * XCH + lane * 16;
  const int xpart = (wave ^ 1) * XCH + lane * 16;

  // ---- lane constants of the buffer layout (header comment) ----
  // score fragments: k-step 18 * half + k at kofs[k & 1] + 2048 * (k >> 1)
  // (row l32 = 16 (l32 >> 4) + u, chunk 2 k-step + hl)
  int kofs0, kofs1;
  {
    const int u = l32 & 15;
    const int kb = KS_HALF * 1024 * half + 1024 * (l32 >> 4) + 64 * u;
    kofs0 = kb + 16 * ((hl + (u >> 2)) & 3);
    kofs1 = kb + 16 * ((2 + hl + (u >> 2)) & 3);
  }
  // value fragments of output block fb, column half k2, row quad t at
  // vofs[t] + 2048 * fb + 1024 * k2: in 16-lane group g, lane c supplies block
  // row 16 k2 + 8 t + 4 (l >> 5) + (c >> 2), features 16 (g & 1) + 4 (c & 3) .. +3
  int vofs0, vofs1;
  {
    const int g16 = lane >> 4, cq = lane & 15;
    const int cp = 2 * (g16 & 1) + ((cq & 3) >> 1);  // chunk inside the group's 4
    const int vb = 16 * 1024 * half + 64 * (4 * hl + (cq >> 2)) + 8 * (cq & 1);
    vofs0 = vb + 16 * ((cp + hl) & 3);
    vofs1 = vb + 512 + 16 * ((cp + 2 + hl) & 3);
  }
  // gather: the block row this lane fetches and its byte offset in the row
  const int grow = 16 * half + (lane >> 2);
  const int gofs = 16 * (((lane & 3) - (lane >> 4)) & 3) + 576 * (wave >> 1);

  // ---- schedule ----
  // Persistent: G workgroups take equal contiguous ranges of the unit list.
  // Workgroup w runs on XCD w % 8 (hardware round-robin), so ranges are
  // handed out by "virtual" id v = (w % 8) * (G / 8) + w / 8: the 32
  // workgroups of one XCD share a contiguous stretch of work -- for the
  // 64-head batch exactly one request -- and re-read its KV blocks from that
  // XCD's L2 instead of the last-level cache.
  long long U = 0, Ge = 1, u0 = 0, u1 = 0, v = blockIdx.x;
  if (p.S == 0) {
    U = uni64(units_before(p.bs, p.qo, p.kvp, p.H, MT));
    if (U <= 0) return;
    Ge = effective_groups(U, gridDim.x);
    if (blockIdx.x >= Ge) return;
    if (Ge == gridDim.x && (Ge & 7) == 0) v = (blockIdx.x & 7) * (Ge >> 3) + (blockIdx.x >> 3);
    u0 = range_begin(v, U, Ge);
    u1 = range_begin(v + 1, U, Ge);
  }

  // A range is a run of segments, each inside one tile.  Only the first can
  // start mid-tile; it runs last, so every workgroup sweeps its tiles' KV
  // blocks from block 0 onward in step with the rest of its XCD.
  long long cursor = 0;  // next unit among the segments after the first
  bool first_done = false;
  if (p.S == 0) {
    int r0;
    long long start0;
    locate(u0, p.qo, p.kvp, p.bs, p.H, MT, r0, start0);
    r0 = uni(r0);
    if (r0 >= p.bs) return;
    start0 = uni64(start0);
    const Geom g0 = uniform(geom(p.qo, p.kvp, r0, p.H, MT));
    cursor = start0 + min(((u0 - start0) / g0.NB + 1) * g0.NB, u1 - start0);
  }
  int seg_no = 0;
  const int nslot_m1 = (int)min(p.num_slots - 1, (long long)0x7fffffff);
  while (true) {
    int r, t, b_begin, b_end;
    long long slot = -1;
    Geom g;
    if (p.S == 0) {
      long long useg;
      if (cursor < u1) {
        useg = cursor;
      } else if (!first_done) {
        useg = u0;
        first_done = true;
      } else {
        break;
      }
      long long start;
      locate(useg, p.qo, p.kvp, p.bs, p.H, MT, r, start);
      r = uni(r);
      if (r >= p.bs) break;
      start = uni64(start);
      g = uniform(geom(p.qo, p.kvp, r, p.H, MT));
      const long long local = useg - start;
      t = uni((int)(local / g.NB));
      b_begin = uni((int)(local % g.NB));
      const long long seg_end = min((long long)(t + 1) * g.NB, u1 - start);
      b_end = uni((int)(seg_end - (long long)t * g.NB));
      if (!(b_begin == 0 && b_end == g.NB)) slot = 2 * v + (useg == u0 ? 0 : 1);
      if (useg != u0) cursor = start + seg_end;
    } else {
      if (seg_no > 0) break;
      const int S = p.S;
      const int s = blockIdx.x % S;
      t = (blockIdx.x / S) % p.T_max;
      r = blockIdx.x / (S * p.T_max);
      if (r >= p.bs) break;
      g = uniform(geom(p.qo, p.kvp, r, p.H, MT));
      if (t >= g.T) break;
      b_begin = uni((int)((long long)s * g.NB / S));
      b_end = uni((int)((long long)(s + 1) * g.NB / S));
      if (S > 1) slot = ((long long)r * p.T_max + t) * S + s;
    }
    ++seg_no;

    // ---- this pair's 32 query rows; this wave's half of their features ----
    const int rho = t * MT + pair * 32 + l32;
    const bool row_ok = rho < g.R;
    // A pair whose 32 rows all lie past the tile's end still runs the whole
    // pipeline (on zero queries) so that every wave follows one straight-line
    // path; the epilogue writes only rows < R.
    const int node = row_ok ? rho / p.H : g.Q - 1;
    bf16x8_t qf[KS_HALF];
    {
      const __bf16* qrow =
          qg + ((size_t)g.q0 * p.H + (row_ok ? rho : 0)) * LATENT + 8 * hl + 16 * KS_HALF * half;
#pragma unroll
      for (int k = 0; k < KS_HALF; ++k) {
        bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * k);
        if (!row_ok) x = bf16x8_t{};
        qf[k] = x;
      }
    }
    // The row's ancestor bitset words, read once per segment: a global load
    // inside the block loop would have to wait behind the in-flight gathers.
    // Rows of up to 128 tree nodes keep all words in registers.
    const uint32_t* vrow = p.vis + (size_t)(g.q0 + node) * p.W;
    uint32_t vw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) vw[k] = k < p.W ? vrow[k] : 0u;

    f32x16_t o[FB_HALF];
#pragma unroll
    for (int fb = 0; fb < FB_HALF; ++fb) o[fb] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;
    const float c = p.scale_log2;

    // slot of the block row this lane gathers in block b (a register load,
    // issued one block ahead of its use)
    const int32_t* kvi = p.kvi + g.kv0;
    auto load_idx = [&](int b) { return kvi[min(b * KB + grow, g.N - 1)]; };
    // this wave's share of the gather of block b: groups j = wave, wave + NW, ...
    // Load i fills group 2 (9 (wave >> 1) + i) + (wave & 1) of buffer dst from row
    // offset gofs + 64 i.  The immediate offset applies to the pool address and
    // the LDS address alike, so the LDS base (M0) is given as target - 64 i.
    const int wofs = 18432 * (wave >> 1) + 1024 * (wave & 1);
    auto gather_src = [&](int sid) {
      // The index is opaque here so that the clamp below (and with it the
      // wait for the index load) cannot be hoisted to the load itself.
      asm volatile("" : "+v"(sid));
      sid = min(max(sid, 0), nslot_m1);
      return poolb + (long long)sid * ROWB + gofs;
    };
    auto gather_one = [&](lds_char* dst, const char* src, auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_global_load_lds(
          src, reinterpret_cast<__attribute__((address_space(3))) void*>(dst + wofs + 1984 * i), 16,
          64 * i, 0);
    };
    auto issue_data = [&](lds_char* dst, int sid) {
      const char* src = gather_src(sid);
      static_for<0, LOADS / NW>([&](auto ic) { gather_one(dst, src, ic); });
    };
    constexpr int LPW = LOADS / NW;  // gather loads per wave per block
    constexpr int KDEPTH = 4;        // score fragments read ahead
    constexpr int VDEPTH = 2;        // value MFMAs whose fragments are read ahead

    // ------------------------------------------------------------------
    // Prologue: gather blocks b0 .. b0+2, compute this wave's half of S(b0),
    // hand it to the partner, and read the first score fragments of b0+1.
    // ------------------------------------------------------------------
    __syncthreads();  // the previous segment is done with all buffers
    f32x16_t s_mine = f32x16_t{};  // this wave's half of the scores of the current block
    bf16x8_t kpre[KDEPTH];         // first score fragments of the next block
#pragma unroll
    for (int k = 0; k < KDEPTH; ++k) kpre[k] = bf16x8_t{};
    int idx_cur = 0;               // slot for the gather of block b+3
    if (b_begin < b_end) {
      const int b0 = b_begin;
      // The pipeline is straight-line: blocks past the segment's end are
      // "gathered" too (a valid row, into a buffer nobody reads), so every
      // wait below is one fixed count that the compiler can account for.
      const int i0 = load_idx(b0);
      const int i1 = load_idx(b0 + 1);
      const int i2 = load_idx(b0 + 2);
      idx_cur = load_idx(b0 + 3);
      issue_data(lds + (b0 % NBUF) * BUFB, i0);
      issue_data(lds + ((b0 + 1) % NBUF) * BUFB, i1);
      issue_data(lds + ((b0 + 2) % NBUF) * BUFB, i2);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(LPW));  // blocks b0, b0+1 have landed
      __builtin_amdgcn_s_barrier();
      {
        const lds_char* kb0 = lds + (b0 % NBUF) * BUFB + kofs0;
        const lds_char* kb1 = lds + (b0 % NBUF) * BUFB + kofs1;
        f32x16_t sp = f32x16_t{};
#pragma unroll
        for (int k = 0; k < KS_HALF; ++k)
          sp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_read_b128((k & 1 ? kb1 : kb0) + 2048 * (k >> 1)), qf[k], sp, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f32x4 x = {sp[4 * k], sp[4 * k + 1], sp[4 * k + 2], sp[4 * k + 3]};
          *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(xch + xmine + k * 1024) = x;
        }
        s_mine = sp;
        const lds_char* nb0 = lds + ((b0 + 1) % NBUF) * BUFB + kofs0;
        const lds_char* nb1 = lds + ((b0 + 1) % NBUF) * BUFB + kofs1;
#pragma unroll
        for (int k = 0; k < KDEPTH; ++k) kpre[k] = lds_read_b128((k & 1 ? nb1 : nb0) + 2048 * (k >> 1));
      }
      lds_barrier();
    }

    // ------------------------------------------------------------------
    // Iteration b.  Entry: blocks b, b+1 resident, b+2 in flight; this
    // wave's half of S(b) in s_mine, the partner's in the exchange buffer;
    // the first KDEPTH score fragments of block b+1 in kpre.
    // Each MFMA below is one scheduling step (sched_barrier on both sides),
    // with a hand-placed share of the other work underneath it.
    // ------------------------------------------------------------------
    // The four buffers an iteration touches are distinct, and the body says
    // so with restrict pointers: that lets the compiler see that the
    // transposing reads of block b cannot alias the gather into block b+3, so
    // it does not wait for that gather before them.
    //   dmab: block b+3 (gather target; held block b-1, whose last reader
    //         finished before the previous barrier)
    //   vbuf: block b (values)   kbuf: block b+1 (scores; stale if none)
    //   nbuf: block b+2 (first score fragments of the next iteration)
    auto body = [&](int b, auto tail_tag, f32x16_t& s_cur, f32x16_t& sp,
                    lds_char* __restrict__ dmab, const lds_char* __restrict__ vbuf,
                    const lds_char* __restrict__ kbuf, const lds_char* __restrict__ nbuf,
                    lds_char* __restrict__ xb) {
      constexpr bool TAIL = decltype(tail_tag)::value;
      // 1. gather of block b+3 (past the end: a valid row into a free
      //    buffer), then the slot of block b+4.  The gather is spread over
      //    the score MFMAs below so the address unit drains between loads.
      //    Its address is formed
      //    before the next index load, so no wait can cover that load.
      const char* gsrc = gather_src(idx_cur);
      const int idx_next = load_idx(b + 4);

      bf16x8_t pk0, pk1, vf[2 * FB_HALF];
      float psum = 0.f, m_use = 0.f, mb = 0.f;
      bool move = false;
      f32x16_t s;
      const lds_char* vb0 = vbuf + vofs0;
      const lds_char* vb1 = vbuf + vofs1;
      auto vread = [&](int i) {  // value MFMA i: output block i & 7, column half i >> 3
        const int off = 2048 * (i & 7) + 1024 * (i >> 3);
        const bf16x4_t lo = lds_read_tr(vb0 + off);
        const bf16x4_t hi = lds_read_tr(vb1 + off);
        return (bf16x8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      auto expo = [&](int x) {  // weight of score x under the current reference
        const float e = __builtin_amdgcn_exp2f(fmaf(s[x], c, -m_use));
        psum += e;
        return e;
      };
      {
        // 2. phase A: the 18 score MFMAs of block b+1.  Underneath: S(b) =
        //    own half + partner's half, mask, block max, reference check,
        //    weights of the lane's first 8 columns.
        f32x4 xp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          xp[k] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
              xb + xpart + k * 1024);
        const lds_char* kb0 = kbuf + kofs0;
        const lds_char* kb1 = kbuf + kofs1;
        bf16x8_t kf[KS_HALF];
#pragma unroll
        for (int k = 0; k < KDEPTH; ++k) kf[k] = kpre[k];
        float mx0 = 0.f;
        sp = f32x16_t{};
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, KS_HALF>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          if constexpr (k % 2 == 1 && k / 2 < LPW)
            gather_one(dmab, gsrc, std::integral_constant<int, k / 2>{});
          if (k + KDEPTH < KS_HALF)
            kf[k + KDEPTH] =
                lds_read_b128(((k + KDEPTH) & 1 ? kb1 : kb0) + 2048 * ((k + KDEPTH) >> 1));
          sp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qf[k], sp, 0, 0, 0);
          if (k >= 1 && k <= 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * (k - 1) + e] = s_cur[4 * (k - 1) + e] + xp[k - 1][e];
          }
          if (TAIL && k == 5) {
            // mask: one 32-bit word, bit c = column cb + c visible
            const int cb = b * KB;
            const int jbase = cb - g.P;  // tree index of the block's column 0
            uint32_t m32;
            if (jbase >= 0) {
              const int w0 = jbase >> 5, sh = jbase & 31;
              uint32_t lo, hi;
              if (p.W <= 4) {
                lo = w0 == 0 ? vw[0] : (w0 == 1 ? vw[1] : (w0 == 2 ? vw[2] : vw[3]));
                hi = w0 == 0 ? vw[1] : (w0 == 1 ? vw[2] : (w0 == 2 ? vw[3] : 0u));
              } else {  // trees of more than 128 nodes
                lo = w0 < p.W ? vrow[w0] : 0u;
                hi = w0 + 1 < p.W ? vrow[w0 + 1] : 0u;
              }
              m32 = sh == 0 ? lo : (lo >> sh) | (hi << (32 - sh));
            } else {  // prefix columns 0 .. -jbase-1, then tree nodes 0, 1, ...
              const int np = -jbase;
              m32 = (0xffffffffu >> (32 - np)) | (vw[0] << np);
            }
            const int ncol = g.N - cb;  // columns of the block that exist
            if (ncol < 32) m32 &= (1u << ncol) - 1u;
            // lane l holds columns 8 (x >> 2) + 4 (l >> 5) + (x & 3)
            const uint32_t mine = m32 >> (4 * hl);
#pragma unroll
            for (int x = 0; x < 16; ++x)
              if (!((mine >> (8 * (x >> 2) + (x & 3))) & 1u)) s[x] = -INFINITY;
          }
          if (k == 6)
            mx0 = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                        fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
          if (k == 7) {
            const float mx1 = fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                                    fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15])));
            mb = fmaxf(mx0, mx1);
          }
          if (k == 8) {
            mb = fmaxf(mb, other_half(mb)) * c;  // c > 0
            // Online softmax reference in base 2, moved lazily: m_run
            // changes only when the block max exceeds it by RESCALE_SLACK
            // (log2 units), so the accumulator rescale is rare and weights
            // stay below 2^RESCALE_SLACK.  O and l share the reference, so
            // the result is exact.
            constexpr float RESCALE_SLACK = 8.f;
            move = mb > m_run + RESCALE_SLACK;  // also true while m_run is -inf
            m_use = m_run == -INFINITY ? 0.f : m_run;  // all columns masked so far
          }
          if (k >= 9 && k <= 16) {
            const int x = k - 9;
            pk0[x] = (__bf16)expo(x);
          }
          __builtin_amdgcn_sched_barrier(0);
        });

        // 3. rare: the reference moves -- rescale O and l, redo the weights
        if (__ballot(move) != 0) {  // wave-uniform
          const float m_new = move ? mb : m_run;
          // rows that keep their reference get exactly 1 (also when it is still -inf)
          const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
          // The accumulators live in AGPRs; pinning them there on both sides
          // of the multiply keeps the compiler from moving all 128 of them
          // into VGPRs for the rest of the loop.
#pragma unroll
          for (int fb = 0; fb < FB_HALF; ++fb) {
            f32x16_t t = o[fb];
            asm volatile("" : "+a"(t));
            t *= alpha;
            asm volatile("" : "+a"(t));
            o[fb] = t;
          }
          m_run = m_new;
          m_use = m_run == -INFINITY ? 0.f : m_run;
          psum = 0.f;
#pragma unroll
          for (int x = 0; x < 8; ++x) pk0[x] = (__bf16)expo(x);
        }
        // first value fragments of block b (resident since two steps ago)
#pragma unroll
        for (int i = 0; i < VDEPTH; ++i) vf[i] = vread(i);
      }

      // 4. block b+2 has landed (only block b+3's gather may still run) and
      //    everyone has read the exchange buffer before it is rewritten
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(LPW));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);

      {
        // 5. phase B: O^T[half] += V^T[half] P^T for block b, column half 0
        //    first.  Underneath: the weights of the lane's last 8 columns,
        //    the hand-off of S(b+1)'s half, the first score fragments of b+2.
        const lds_char* nb0 = nbuf + kofs0;
        const lds_char* nb1 = nbuf + kofs1;
#pragma unroll
        for (int i = 0; i < 2 * FB_HALF; ++i) {
          if (i + VDEPTH < 2 * FB_HALF) vf[i + VDEPTH] = vread(i + VDEPTH);
          o[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], i < 8 ? pk0 : pk1, o[i & 7], 0,
                                                              0, 0);
          if (i < 8) pk1[i] = (__bf16)expo(8 + i);
          if (i >= 8 && i < 12) {
            const int k = i - 8;
            f32x4 x = {sp[4 * k], sp[4 * k + 1], sp[4 * k + 2], sp[4 * k + 3]};
            *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(xb + xmine + k * 1024) = x;
          }
          if (i >= 2 * FB_HALF - KDEPTH) {
            const int k = i - (2 * FB_HALF - KDEPTH);
            kpre[k] = lds_read_b128((k & 1 ? nb1 : nb0) + 2048 * (k >> 1));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        l_run += psum;
      }

      // 6. the hand-off is visible
      lds_barrier();
      idx_cur = idx_next;
    };
    auto step = [&](int b, auto tail_tag, f32x16_t& s_cur, f32x16_t& sp) {
      body(b, tail_tag, s_cur, sp, lds + ((b + 3) % NBUF) * BUFB, lds + (b % NBUF) * BUFB,
           lds + ((b + 1) % NBUF) * BUFB, lds + ((b + 2) % NBUF) * BUFB, xch);
    };

    // Blocks that lie wholly inside the prefix need no mask.  The prefix
    // loop is unrolled by two so the two score registers swap roles instead
    // of being copied every block.
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    const int b_mask = max(b_begin, min(b_end, g.P / KB));
    f32x16_t s_alt = f32x16_t{};
    int b = b_begin;
    for (; b + 1 < b_mask; b += 2) {
      step(b, NoMask{}, s_mine, s_alt);
      step(b + 1, NoMask{}, s_alt, s_mine);
    }
    if (b < b_mask) {
      step(b, NoMask{}, s_mine, s_alt);
      s_mine = s_alt;
      ++b;
    }
    for (; b < b_end; ++b) {
      step(b, Mask{}, s_mine, s_alt);
      s_mine = s_alt;
    }

    // ---- write this segment (rows of the pair, features of the half) ----
    const float l_tot = l_run + other_half(l_run);
    if (row_ok && (slot >= 0 || b_begin < b_end)) {  // empty split segments still report m=-inf, l=0
      const size_t orow = (size_t)g.q0 * p.H + rho;
      const int fo = 256 * half + 4 * hl;
      if (slot < 0) {
        const float inv = 1.f / l_tot;
        __bf16* out = static_cast<__bf16*>(p.out) + orow * DV + fo;
#pragma unroll
        for (int fb = 0; fb < FB_HALF; ++fb) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            bf16x4_t v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[fb][4 * gq + e] * inv);
            *reinterpret_cast<bf16x4_t*>(out + 32 * fb + 8 * gq) = v4;
          }
        }
        if (half == 0 && hl == 0 && p.lse) p.lse[orow] = (m_run + log2f(l_tot)) * LN2;
      } else {
        float* base = p.ws + slot * slot_floats(MT);
        const int trow = pair * 32 + l32;
        float* ob = base + (size_t)trow * DV + fo;
#pragma unroll
        for (int fb = 0; fb < FB_HALF; ++fb) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            float4 v4 = make_float4(o[fb][4 * gq], o[fb][4 * gq + 1], o[fb][4 * gq + 2],
                                    o[fb][4 * gq + 3]);
            *reinterpret_cast<float4*>(ob + 32 * fb + 8 * gq) = v4;
          }
        }
        if (half == 0 && hl == 0) {
          base[(size_t)MT * DV + trow] = m_run;
          base[(size_t)MT * DV + MT + trow] = l_tot;
        }
      }
    }
  }
}

}  // namespace

int launch_bf16(const Params& p, int grid, hipStream_t s) {
  constexpr int NW = MT_BF16 / 16;
  hipLaunchKernelGGL(attn_bf16_kernel<NW>, dim3(grid), dim3(NW * 64), 0, s, p);
  return check_launch("verify_attn(bf16)");
}

}  // namespace attn
}  // namespace ddtree
