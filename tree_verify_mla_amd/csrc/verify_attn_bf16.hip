// bf16 verify attention on gfx950 matrix cores.
//
// Workgroup = NW = 4 wavefronts = one tile of 64 query rows of one request.
// The tile walks its KV columns in blocks of 32; each block is gathered once
// from the slot pool into LDS and shared by all rows -- the prefix is read
// once for every tree node and head ("The DDTree CUDA Graph Fix ...",
// section "The DDTree Architecture: Confirming Multiple-Path Evaluation").
//
// Scores: waves pair up; pair g owns rows 32g .. 32g+31 and wave half h
// contracts latent features [288h, 288h+288):
//   partial S^T[32 col x 32 row] = K[32 x 288] . Q^T[288 x 32]   18 x mfma_f32_32x32x16_bf16
//     A = latent rows from LDS (ds_read_b128), B = the wave's half of the
//     queries, kept in registers for the whole tile.  With columns as the
//     MFMA row index each lane's accumulator holds ONE query row, so the
//     row max is one cross-half exchange and the output rescale is one
//     multiplier per lane.  Half 1 hands its partial to half 0 through LDS.
//   mask: prefix columns always visible; column P + j visible iff bit j of
//     the row's ancestor bitset is set (tail blocks only).
//   online softmax in base 2 (by half 0); P^T rounded to bf16 and
//     published in LDS in the accumulator's own lane layout (the columns'
//     order inside the k dimension is permuted to match it).
// Values: wave w produces output features [128w, 128w+128) for all 64 rows:
//   O^T[128 x 64 row] += V^T[128 x 32 col] . P^T[32 col x 64 row]   16 x mfma_f32_32x32x16_bf16
//     A = c_kv columns read transposed from LDS with ds_read_b64_tr_b16,
//     each fragment serving both row groups; B = P^T from LDS.
// Each LDS byte of a block thus feeds 64 rows of values and 32 rows of each
// score half, while a wave keeps 72 VGPRs of queries and 128 accumulators.
//
// Block buffer layout.  A block is 32 latent rows x 72 chunks of 16 bytes,
// stored as 36 groups of 1 KB: group 2m + h holds chunks 4m .. 4m+3 of rows
// 16h .. 16h+15, and 16-byte position 4u + v of the group holds chunk
// 4m + ((v - (u >> 2)) & 3) of row 16h + u.
// * gather: one buffer_load_dwordx4 ... lds fills one group (lane =
//   position).  Each 4-lane quad reads one 64-byte span of one row (a
//   quarter of the lanes' cache lines, coalesced), and wave w fetches rows
//   16 (w & 1) + l/4, features [288 (w >> 1), +288) of them: one pool offset
//   per lane and block, the 64-byte steps in the instruction's immediate.
// * score fragment (k-step j, lane l: row l & 31, chunk 2j + (l >> 5)): two
//   base addresses (j even / odd) plus an immediate 2 KB * (j >> 1).
// * transposed value fragments (4 rows x 16 features per 16 lanes): two
//   base addresses plus immediates.
// gfx950 LDS has 64 four-byte banks; a b128 read is serviced 16 lanes at a
// time, a b64 (and the transposing b64) read 32 lanes at a time.  The
// rotation by (u >> 2) puts the lanes of each phase of both patterns on 16
// distinct 16-byte positions mod 256 bytes, so neither has bank conflicts.
//
// Pipeline: four block buffers, two blocks in flight, two barriers per
// block.  Iteration b starts the gather of block b+3 and runs the 18 score
// MFMAs of block b+1 (half 0 weighs columns 8-15 of block b underneath),
// then the 16 value MFMAs of block b (half 0 runs the first part of the
// softmax of block b+1 underneath).  The loop is compiled once per half.
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
constexpr int XCH = 64 * 64;       // bytes per pair of score-exchange space (64 lanes x 16 f32)
constexpr int PBYTES = 4 * 1024;   // P^T of a block: 2 row groups x 2 column halves x 1 KB
constexpr int ABYTES = 64 * 4;     // one rescale factor per tile row
constexpr int KS_HALF = 18;        // k-steps of 16 features per half of the 576-wide score
constexpr int FB_WAVE = 4;         // 32-feature output blocks per wave (128 of the 512 outputs)
constexpr float LN2 = 0.693147180559945309f;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14)
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14); }
constexpr int WAIT_LGKM0 = 0xF | (7 << 4) | (0 << 8) | (3 << 14);


// Workgroup barrier after an explicit wait (an s_waitcnt immediate).  The
// empty asm statements with a memory clobber keep the compiler from moving
// any memory access across the barrier (the barrier builtin alone does not
// order memory for the optimiser); they emit nothing.
template <int WAITCNT>
__device__ inline void barrier_after() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(WAITCNT);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that waits only for this wave's LDS traffic, leaving the
// global->LDS gathers of later blocks in flight (__syncthreads() would wait
// for every outstanding memory operation).
__device__ inline void lds_barrier() { barrier_after<WAIT_LGKM0>(); }

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

// BUF: the pool is addressed through a buffer resource (32-bit offsets,
// pools under 4 GiB).  The gathers are then buffer_load ... lds, which the
// compiler's wait-count tracking keeps apart from LDS reads, so the LDS
// reads of fragments wait only for themselves.  With global_load_lds (the
// form for larger pools) every LDS read waits for all outstanding LDS
// traffic.
template <int NW, bool BUF>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(Params p) {
  // The body uses buffer-resource builtins that exist only for the device;
  // the host pass needs nothing but the kernel's symbol.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int MT = 16 * NW;
  static_assert(MT == MT_BF16, "tile rows must match the schedule");
  static_assert(NW == 4, "the block layout splits the gather over 2 x 2 waves");
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * BUFB + 2 * XCH + PBYTES + ABYTES];
  lds_char* lds = (lds_char*)smem;       // generic -> LDS address space
  lds_char* xch = lds + NBUF * BUFB;     // score halves: one slot per pair
  lds_char* pbuf = xch + 2 * XCH;        // P^T fragments of both pairs
  lds_char* abuf = pbuf + PBYTES;        // rescale factors of both pairs' rows

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int pair = wave >> 1, half = wave & 1;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q);
  const char* __restrict__ poolb = static_cast<const char*>(p.pool);
  const __amdgpu_buffer_rsrc_t pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.pool), 0, (int)(unsigned)min((long long)p.num_slots * ROWB, 0xffffffffLL),
      0x00020000);  // gfx9 raw buffer: untyped, no swizzle
  const int xofs = pair * XCH + lane * 16;  // the pair's exchange slot, this lane's 16 bytes per KB
  const int pofs = lane * 16;               // P^T fragment (row group rg, column half k2) at 1 KB (2 rg + k2)

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
  // value fragments of the wave's output block fb, column half k2, row quad t
  // at vofs[t] + 2048 * fb + 1024 * k2: in 16-lane group g, lane c supplies
  // block row 16 k2 + 8 t + 4 (l >> 5) + (c >> 2), features
  // 128 wave + 32 fb + 16 (g & 1) + 4 (c & 3) .. +3
  int vofs0, vofs1;
  {
    const int g16 = lane >> 4, cq = lane & 15;
    const int cp = 2 * (g16 & 1) + ((cq & 3) >> 1);  // chunk inside the group's 4
    const int vb = 8 * 1024 * wave + 64 * (4 * hl + (cq >> 2)) + 8 * (cq & 1);
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

    // O^T of the wave's 128 output features for all 64 rows of the tile
    f32x16_t o[2][FB_WAVE];  // [row group][32-feature block]
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int fb = 0; fb < FB_WAVE; ++fb) o[rg][fb] = f32x16_t{};
    // softmax reference of the pair's rows (kept by half 0; half 1's copy
    // is unused)
    float m_run = -INFINITY;
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
      if constexpr (BUF)
        return (int)((unsigned)sid * ROWB + gofs);  // byte offset in the pool
      else
        return poolb + (long long)sid * ROWB + gofs;
    };
    auto gather_one = [&](lds_char* dst, auto src, auto ic) {
      constexpr int i = decltype(ic)::value;
      auto* d = reinterpret_cast<__attribute__((address_space(3))) void*>(dst + wofs + 1984 * i);
      if constexpr (BUF)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pool_rsrc, d, 16, src, 0, 64 * i, 0);
      else
        __builtin_amdgcn_global_load_lds(src, d, 16, 64 * i, 0);
    };
    auto issue_data = [&](lds_char* dst, int sid) {
      const auto src = gather_src(sid);
      static_for<0, LOADS / NW>([&](auto ic) { gather_one(dst, src, ic); });
    };
    constexpr int LPW = LOADS / NW;  // gather loads per wave per block
    constexpr int KDEPTH = 4;        // score fragments read ahead
    constexpr int VDEPTH = 3;        // value fragments read ahead

    // visibility of block blk's 32 columns to this lane's row (bit c =
    // column blk * KB + c); nothing past the segment is visible
    auto mask_word = [&](int blk) -> uint32_t {
      const int cb = blk * KB;
      const int ncol = g.N - cb;  // columns of the block that exist
      if (blk >= b_end || ncol <= 0) return 0u;
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
      } else if (jbase <= -KB) {  // prefix columns only
        m32 = 0xffffffffu;
      } else {  // prefix columns 0 .. -jbase-1, then tree nodes 0, 1, ...
        const int np = -jbase;
        m32 = (0xffffffffu >> (32 - np)) | (vw[0] << np);
      }
      if (ncol < 32) m32 &= (1u << ncol) - 1u;
      return m32;
    };

    // ------------------------------------------------------------------
    // Softmax of one block, run by half 0 of each pair in stages that each
    // sit under one MFMA.
    //   under the value MFMAs of the previous block: add the partner's half
    //     of the scores, mask, take the block max, move the reference, weigh
    //     the lane's columns 0-7 (P^T k-half 0) and publish them with the
    //     rows' rescale factor; keep columns 8-15 as exponents;
    //   under the score MFMAs of the next block: weigh columns 8-15 and
    //     publish P^T k-half 1.
    // Half 1 only hands its partial scores over; the block loop is compiled
    // once per half.
    // ------------------------------------------------------------------
    f32x16_t s;
    f32x4 xp[4], th[2];
    float mb = 0.f, mu = 0.f, psum0 = 0.f, psum1 = 0.f, alpha = 1.f;
    float l_run = 0.f;  // row sum of the lane's 16 columns (half 0)
    bf16x8_t pk0, pk1;
    auto sm_read = [&](const lds_char* xb) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        xp[k] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(xb + xofs +
                                                                                 k * 1024);
    };
    auto sm_add = [&](const f32x16_t& sp, int q) {  // columns of accumulator quarters 2q, 2q+1
#pragma unroll
      for (int k = 2 * q; k < 2 * q + 2; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * k + e] = sp[4 * k + e] + xp[k][e];
    };
    auto sm_mask = [&](int blk) {
      // lane l holds columns 8 (x >> 2) + 4 (l >> 5) + (x & 3)
      const uint32_t mine = mask_word(blk) >> (4 * hl);
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (!((mine >> (8 * (x >> 2) + (x & 3))) & 1u)) s[x] = -INFINITY;
    };
    auto sm_max = [&]() {
      const float mx0 = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                              fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      const float mx1 = fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                              fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15])));
      mb = fmaxf(mx0, mx1);
    };
    auto sm_ref = [&]() {
      mb = fmaxf(mb, other_half(mb)) * c;  // c > 0
      // Online softmax reference in base 2, moved lazily: m_run changes only
      // when the block max exceeds it by RESCALE_SLACK (log2 units), so the
      // accumulator rescale is rare and weights stay below 2^RESCALE_SLACK.
      // O and l share the reference, so the result is exact.
      constexpr float RESCALE_SLACK = 8.f;
      const bool move = mb > m_run + RESCALE_SLACK;  // also true while m_run is -inf
      const float m_new = move ? mb : m_run;
      // rows that keep their reference get exactly 1 (also when it is still -inf)
      alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      mu = m_run == -INFINITY ? 0.f : m_run;  // all columns masked so far
      psum0 = 0.f;
    };
    auto sm_defer = [&]() {  // columns 8-15 as exponents, weighed one phase later
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) th[k][e] = fmaf(s[8 + 4 * k + e], c, -mu);
      psum1 = 0.f;
    };
    auto sm_exp0 = [&](int x) {  // weight of column x (0-7) under the reference
      const float e = __builtin_amdgcn_exp2f(fmaf(s[x], c, -mu));
      psum0 += e;
      pk0[x] = (__bf16)e;
    };
    auto sm_publish0 = [&](lds_char* pb, lds_char* ab) {
      *reinterpret_cast<__attribute__((address_space(3))) bf16x8_t*>(pb + 2 * pair * 1024 + pofs) =
          pk0;
      if (hl == 0)
        reinterpret_cast<__attribute__((address_space(3))) float*>(ab)[pair * 32 + l32] = alpha;
      l_run += psum0;
    };
    auto sm_exp1 = [&](int j) {  // weight of column 8 + j
      const float e = __builtin_amdgcn_exp2f(th[j >> 2][j & 3]);
      psum1 += e;
      pk1[j] = (__bf16)e;
    };
    auto sm_publish1 = [&](lds_char* pb) {
      *reinterpret_cast<__attribute__((address_space(3))) bf16x8_t*>(
          pb + (2 * pair + 1) * 1024 + pofs) = pk1;
      l_run += psum1;
    };
    auto score_mfmas = [&](const lds_char* kbuf, bf16x8_t* kf, auto&& under) {
      // S^T partial of one block (this wave's 288 features); under(k) runs
      // beneath step k
      const lds_char* kb0 = kbuf + kofs0;
      const lds_char* kb1 = kbuf + kofs1;
      f32x16_t acc = f32x16_t{};
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, KS_HALF>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        under(kc);
        if (k + KDEPTH < KS_HALF)
          kf[k + KDEPTH] =
              lds_read_b128(((k + KDEPTH) & 1 ? kb1 : kb0) + 2048 * ((k + KDEPTH) >> 1));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qf[k], acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      return acc;
    };
    auto hand_off = [&](const f32x16_t& sp, lds_char* xb) {  // half 1 -> half 0
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f32x4 x = {sp[4 * k], sp[4 * k + 1], sp[4 * k + 2], sp[4 * k + 3]};
        *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(xb + xofs + k * 1024) = x;
      }
    };

    // ------------------------------------------------------------------
    // Prologue: gather blocks b0 .. b0+2, the scores and softmax of b0
    // (P(b0) published), and the first score fragments of b0+1.
    // ------------------------------------------------------------------
    __syncthreads();  // the previous segment is done with all buffers
    bf16x8_t kpre[KDEPTH];  // first score fragments of the next block
#pragma unroll
    for (int k = 0; k < KDEPTH; ++k) kpre[k] = bf16x8_t{};
    int idx_cur = 0;        // slot for the gather of block b+3
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
      barrier_after<waitcnt_vm_lgkm0(LPW)>();  // blocks b0, b0+1 have landed
      bf16x8_t kf[KS_HALF];
      {
        const lds_char* kb0 = lds + (b0 % NBUF) * BUFB + kofs0;
        const lds_char* kb1 = lds + (b0 % NBUF) * BUFB + kofs1;
#pragma unroll
        for (int k = 0; k < KDEPTH; ++k) kf[k] = lds_read_b128((k & 1 ? kb1 : kb0) + 2048 * (k >> 1));
      }
      const f32x16_t sp = score_mfmas(lds + (b0 % NBUF) * BUFB, kf, [](auto) {});
      if (half == 1) hand_off(sp, xch);
      {
        const lds_char* nb0 = lds + ((b0 + 1) % NBUF) * BUFB + kofs0;
        const lds_char* nb1 = lds + ((b0 + 1) % NBUF) * BUFB + kofs1;
#pragma unroll
        for (int k = 0; k < KDEPTH; ++k) kpre[k] = lds_read_b128((k & 1 ? nb1 : nb0) + 2048 * (k >> 1));
      }
      lds_barrier();
      if (half == 0) {
        sm_read(xch);
        sm_add(sp, 0);
        sm_add(sp, 1);
        sm_mask(b0);
        sm_max();
        sm_ref();
        sm_defer();
#pragma unroll
        for (int x = 0; x < 8; ++x) sm_exp0(x);
        sm_publish0(pbuf, abuf);
      }
      lds_barrier();
    }

    // ------------------------------------------------------------------
    // Iteration b.  Entry: blocks b, b+1 resident, b+2 in flight; P^T k-half
    // 0 of block b and the factors that bring O to its reference published,
    // half 0 holding the exponents of columns 8-15 of block b; the first
    // KDEPTH score fragments of block b+1 in kpre.
    //   phase A: 18 score MFMAs of block b+1 (the gather of block b+3
    //            spread underneath); half 0 weighs columns 8-15 of block b
    //            and publishes P^T k-half 1; rare rescale of O; half 1 hands
    //            its half of S(b+1) to half 0.
    //   phase B: 16 value MFMAs of block b (each value fragment serves both
    //            row groups; k-half 0 first, so k-half 1's fragments, read
    //            after the barrier, arrive in time); underneath, half 0's
    //            part of the softmax of block b+1; first score fragments of
    //            block b+2.
    // Each MFMA is one scheduling step (sched_barrier on both sides).
    // ------------------------------------------------------------------
    // The buffers an iteration touches are distinct, and the body says so
    // with restrict pointers: that lets the compiler see that the
    // transposing reads of block b cannot alias the gather into block b+3,
    // so it does not wait for that gather before them.
    //   dmab: block b+3 (gather target; held block b-1, whose last reader
    //         finished before the previous barrier)
    //   vbuf: block b (values)   kbuf: block b+1 (scores; stale if none)
    //   nbuf: block b+2 (first score fragments of the next iteration)
    // The exchange slot, P^T and rescale regions (xb, pb, ab) carry data
    // between waves and must not be restrict: the compiler would assume no
    // other wave writes them and reuse values loaded before a barrier.
    auto body = [&](int b, auto mask_tag, auto half_tag, lds_char* __restrict__ dmab,
                    const lds_char* __restrict__ vbuf, const lds_char* __restrict__ kbuf,
                    const lds_char* __restrict__ nbuf, lds_char* xb, lds_char* pb,
                    lds_char* ab) {
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr int H = decltype(half_tag)::value;  // == half
      // gather of block b+3 (past the end: a valid row into a free buffer),
      // then the slot of block b+4.  The gather's address is formed before
      // the next index load, so no wait can cover that load.
      const auto gsrc = gather_src(idx_cur);
      const int idx_next = load_idx(b + 4);

      // ---- phase A ----
      bf16x8_t pf[2][2];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) pf[rg][0] = lds_read_b128(pb + 2 * rg * 1024 + pofs);
      const float a0 = reinterpret_cast<const __attribute__((address_space(3))) float*>(ab)[l32];
      const float a1 = reinterpret_cast<const __attribute__((address_space(3))) float*>(ab)[32 + l32];
      bf16x8_t kf[KS_HALF];
#pragma unroll
      for (int k = 0; k < KDEPTH; ++k) kf[k] = kpre[k];
      const f32x16_t sp = score_mfmas(kbuf, kf, [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k % 2 == 1 && k / 2 < LPW)
          gather_one(dmab, gsrc, std::integral_constant<int, k / 2>{});
        if constexpr (H == 0 && k >= 2 && k < 10) sm_exp1(k - 2);
        if constexpr (H == 0 && k == 10) sm_publish1(pb);
      });
      // rare: some row's reference moved with block b -- bring O along first
      if (__ballot(a0 != 1.f || a1 != 1.f) != 0) {  // wave-uniform
        // The accumulators live in AGPRs; pinning them there on both sides
        // of the multiply keeps the compiler from moving all of them into
        // VGPRs for the rest of the loop.
#pragma unroll
        for (int fb = 0; fb < FB_WAVE; ++fb) {
          f32x16_t t0 = o[0][fb], t1 = o[1][fb];
          asm volatile("" : "+a"(t0), "+a"(t1));
          t0 *= a0;
          t1 *= a1;
          asm volatile("" : "+a"(t0), "+a"(t1));
          o[0][fb] = t0;
          o[1][fb] = t1;
        }
      }
      const lds_char* vb0 = vbuf + vofs0;
      const lds_char* vb1 = vbuf + vofs1;
      auto vread = [&](int f) {  // value fragment f: output block f & 3, column half f >> 2
        const int off = 2048 * (f & 3) + 1024 * (f >> 2);
        const bf16x4_t lo = lds_read_tr(vb0 + off);
        const bf16x4_t hi = lds_read_tr(vb1 + off);
        return (bf16x8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8_t vf[2 * FB_WAVE];
#pragma unroll
      for (int f = 0; f < VDEPTH; ++f) vf[f] = vread(f);
      if constexpr (H == 1) hand_off(sp, xb);

      // block b+2 has landed (only block b+3's gather may still run); S(b+1)'s
      // half and P^T k-half 1 of block b are visible, and k-half 0 has been
      // read by everyone
      barrier_after<waitcnt_vm_lgkm0(LPW)>();

      // ---- phase B ----
      const lds_char* nb0 = nbuf + kofs0;
      const lds_char* nb1 = nbuf + kofs1;
      static_for<0, 4 * FB_WAVE>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int f = i >> 1, rg = i & 1, fb = f & 3, k2 = f >> 2;
        if constexpr (rg == 0 && f + VDEPTH < 2 * FB_WAVE) vf[f + VDEPTH] = vread(f + VDEPTH);
        o[rg][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[f], pf[rg][k2], o[rg][fb], 0, 0, 0);
        if constexpr (i == 0) {
#pragma unroll
          for (int r = 0; r < 2; ++r) pf[r][1] = lds_read_b128(pb + (2 * r + 1) * 1024 + pofs);
        }
        if constexpr (H == 0) {
          if constexpr (i == 0) sm_read(xb);
          if constexpr (i == 2) sm_add(sp, 0);
          if constexpr (i == 3) {
            sm_add(sp, 1);
            if constexpr (MASK) sm_mask(b + 1);
          }
          if constexpr (i == 4) sm_max();
          if constexpr (i == 5) sm_ref();
          if constexpr (i == 6) sm_defer();
          if constexpr (i >= 7 && i < 11) {
            sm_exp0(2 * (i - 7));
            sm_exp0(2 * (i - 7) + 1);
          }
          if constexpr (i == 11) sm_publish0(pb, ab);
        }
        if constexpr (i >= 4 * FB_WAVE - KDEPTH) {
          constexpr int k = i - (4 * FB_WAVE - KDEPTH);
          kpre[k] = lds_read_b128((k & 1 ? nb1 : nb0) + 2048 * (k >> 1));
        }
        __builtin_amdgcn_sched_barrier(0);
      });

      // P^T k-half 0 of block b+1 is visible; everyone is done with block b
      // and P^T k-half 1 of block b
      lds_barrier();
      idx_cur = idx_next;
    };
    auto step = [&](int b, auto mask_tag, auto half_tag) {
      body(b, mask_tag, half_tag, lds + ((b + 3) % NBUF) * BUFB, lds + (b % NBUF) * BUFB,
           lds + ((b + 1) % NBUF) * BUFB, lds + ((b + 2) % NBUF) * BUFB, xch, pbuf, abuf);
    };

    // Iterations whose next block lies wholly inside the prefix need no mask;
    // the others (and the last, whose next block is past the segment) do.
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    // The loops are compiled once per half (wave-uniform dispatch).
    const int b_full = min(b_end, g.P / KB);
    auto run_blocks = [&](auto half_tag) {
      int b = b_begin;
      for (; b + 1 < b_full; ++b) step(b, NoMask{}, half_tag);
      for (; b < b_end; ++b) step(b, Mask{}, half_tag);
    };
    if (half == 0)
      run_blocks(std::integral_constant<int, 0>{});
    else
      run_blocks(std::integral_constant<int, 1>{});

    // ---- segment statistics of both pairs' rows, then the output ----
    // m and l of each pair's rows come from its half 0
    const float l_tot = l_run + other_half(l_run);
    auto* stat = reinterpret_cast<__attribute__((address_space(3))) float*>(xch);
    if (half == 0 && hl == 0) {
      stat[pair * 32 + l32] = m_run;
      stat[MT + pair * 32 + l32] = l_tot;
    }
    lds_barrier();
    const int fo = 128 * wave + 4 * hl;
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int trow = rg * 32 + l32;
      const int rho_o = t * MT + trow;
      const float m_row = stat[trow], l_row = stat[MT + trow];
      if (rho_o < g.R && (slot >= 0 || b_begin < b_end)) {  // empty split segments report m=-inf, l=0
        const size_t orow = (size_t)g.q0 * p.H + rho_o;
        if (slot < 0) {
          const float inv = 1.f / l_row;
          __bf16* out = static_cast<__bf16*>(p.out) + orow * DV + fo;
#pragma unroll
          for (int fb = 0; fb < FB_WAVE; ++fb) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              bf16x4_t v4;
#pragma unroll
              for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[rg][fb][4 * gq + e] * inv);
              *reinterpret_cast<bf16x4_t*>(out + 32 * fb + 8 * gq) = v4;
            }
          }
          if (wave == 0 && hl == 0 && p.lse) p.lse[orow] = (m_row + log2f(l_row)) * LN2;
        } else {
          float* base = p.ws + slot * slot_floats(MT);
          float* ob = base + (size_t)trow * DV + fo;
#pragma unroll
          for (int fb = 0; fb < FB_WAVE; ++fb) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              float4 v4 = make_float4(o[rg][fb][4 * gq], o[rg][fb][4 * gq + 1],
                                      o[rg][fb][4 * gq + 2], o[rg][fb][4 * gq + 3]);
              *reinterpret_cast<float4*>(ob + 32 * fb + 8 * gq) = v4;
            }
          }
          if (wave == 0 && hl == 0) {
            base[(size_t)MT * DV + trow] = m_row;
            base[(size_t)MT * DV + MT + trow] = l_row;
          }
        }
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace

int launch_bf16(const Params& p, int grid, hipStream_t s) {
  constexpr int NW = MT_BF16 / 16;
  if (p.num_slots * (long long)ROWB <= 0xffffffffLL)
    hipLaunchKernelGGL((attn_bf16_kernel<NW, true>), dim3(grid), dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<NW, false>), dim3(grid), dim3(NW * 64), 0, s, p);
  return check_launch("verify_attn(bf16)");
}

}  // namespace attn
}  // namespace ddtree
