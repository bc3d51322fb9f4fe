// bf16 verify attention for problems too small to fill the device with
// 128-row tiles: few heads and requests, as on one tensor-parallel shard
// ("The 30-Column Mask ...", section "TP8 Sharding": 8 heads per rank).
//
// There the 128-row kernel runs few, long workgroups: each loads a 147 KB
// query tile and stores a 128 KB partial, so splitting the KV range finer
// costs more than it gains.  Here a workgroup holds 32 query rows (36 KB of
// queries, a 32 KB partial) and the split is fixed by the host:
//
// Workgroup (r, t, s) = 4 wavefronts = tile t (32 rows) of request r, KV
// blocks [s NB / S, (s+1) NB / S) (S splits, part s on XCD s % 8).  The
// range is taken in steps of up to four 32-column blocks.  In a step, wave w
//   * gathers its block into its own LDS buffer and forms
//     S^T[32 col x 32 row] = K . Q^T over the 576 latents (36 MFMAs
//     32x32x16, the queries held in AGPRs: the B operand of every step);
//   * after the four waves have put their block maxima in LDS, moves each
//     row's softmax reference (the same decision in every wave), turns its
//     scores into bf16 weights P^T and puts them in LDS;
//   * accumulates output features 128w .. 128w+127 of all 32 rows over the
//     step's blocks: O^T[128 x 32] += V^T[128 x 32 col] . P^T[32 col x 32]
//     per block (8 MFMAs, V^T read transposed from the block's buffer).
// A step costs three workgroup barriers and leaves its buffers free for the
// next step's gathers.  At the end the waves add their row sums; with one
// part per tile (S = 1) the workgroup writes the bf16 output and lse, else a
// partial that merge_narrow_kernel folds by log-sum-exp ("The 30-Column Mask
// ...", section "The Context: Building a Custom Verify Attention Kernel":
// KV-split flash decoding with a partial reduction).
//
// The queries are staged through buffer 3 (a block's layout, so their
// fragments are read like score fragments); so the first step takes three
// blocks and wave 3 gathers its first block (the part's fourth) while that
// step runs.
#include "attn_common.h"
#include "attn_device.h"
#include "common.h"

namespace ddtree {
namespace attn {

namespace {

using namespace dev;

constexpr int NW = 4;                       // waves = blocks per step
constexpr int MTN = MT_NARROW;              // 32 rows per tile
constexpr int PBUF_N = NW * BUFB;           // P^T of a step: [block][k-step] x 1 KB
constexpr int RED_N = PBUF_N + NW * 2048;   // block maxima [wave][32] f32
constexpr int LSUM_N = RED_N + NW * 32 * 4; // row sums [wave][32] f32
constexpr int LDS_N = LSUM_N + NW * 32 * 4;
static_assert(LDS_N <= 160 * 1024, "LDS budget");
constexpr float RESCALE_SLACK = 8.f;  // log2 units the block max may exceed the reference
constexpr int KDN = 6;  // score fragments read ahead

template <bool BUF>
__global__ __launch_bounds__(NW * 64) void attn_narrow_kernel(Params p_all) {
#if defined(__HIP_DEVICE_COMPILE__)
  const Params p = at_layer(p_all);
  __shared__ __attribute__((aligned(1024))) char smem[LDS_N];
  lds_char* lds = (lds_char*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  // Workgroup i runs on XCD i % 8 (hardware round-robin); XCD x takes the
  // parts s = x, x + 8, ... of every tile, so the tiles of one request read
  // each KV block through one XCD's L2 instead of all eight
  const int S = p.S;
  const int x = blockIdx.x & 7;
  const int k8 = blockIdx.x >> 3;
  const int tiles = p.bs * p.T_max;
  const int s = x + 8 * (k8 / tiles);
  const int r = (k8 % tiles) / p.T_max;
  const int t = (k8 % tiles) % p.T_max;
  if (s >= S) return;
  const Geom g = uniform(geom(p.qo, p.kvp, r, p.H, MTN));
  if (t >= g.T) return;
  const int b0 = uni((int)((long long)s * g.NB / S));
  const int b1 = uni((int)((long long)(s + 1) * g.NB / S));
  if (b0 >= b1) {
    // an empty part (NB < S): its rows saw no column (m = -inf), so the
    // merge needs no geometry to skip it
    if (threadIdx.x < 4 * MTN)
      p.ws[(((long long)r * p.T_max + t) * S + s) * slot_floats_narrow() + MTN * DV / 2 + 4 * threadIdx.x] =
          -INFINITY;
    return;
  }

  const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q);
  const char* __restrict__ poolb = static_cast<const char*>(p.pool);
  const __amdgpu_buffer_rsrc_t pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.pool), 0, (int)(unsigned)min((long long)p.num_slots * ROWB, 0xffffffffLL),
      0x00020000);  // gfx9 raw buffer: untyped, no swizzle

  int kofs0, kofs1, vofs0, vofs1;
  score_offsets(lane, kofs0, kofs1);
  value_offsets(lane, wave, vofs0, vofs1);
  const int gofs = gather_row_offset(lane);
  lds_char* const pbuf = lds + PBUF_N;
  lds_char* const red = lds + RED_N;
  lds_char* const lsum = lds + LSUM_N;
  lds_char* const own = lds + wave * BUFB;  // this wave's block buffer

  // ---- the tile's rows ----
  const int rho = t * MTN + l32;
  const bool row_ok = rho < g.R;
  // rows past the request's end run on its last row's data; only live rows
  // are stored
  const int node = row_ok ? rho / p.H : g.Q - 1;
  const uint32_t* vrow = p.vis + (size_t)(g.q0 + node) * p.W;
  uint32_t vw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) vw[k] = vrow[min(k, p.W - 1)];

  // slots of the two block rows this lane gathers (rows lane / 4 and
  // 16 + lane / 4), clamped to the request's last column: blocks past the
  // range or the request gather valid rows that the mask hides
  const int32_t* kvi = p.kvi + g.kv0;
  const int nslot_m1 = (int)min(p.num_slots - 1, (long long)0x7fffffff);
  auto load_idx = [&](int blk, int h) {
    return kvi[min(max(blk * KB + 16 * h + (lane >> 2), 0), g.N - 1)];
  };
  auto gather = [&](lds_char* dst, int sid0, int sid1) {
    asm volatile("" : "+v"(sid0), "+v"(sid1));  // the clamp below waits for the index loads here
    const int sids[2] = {min(max(sid0, 0), nslot_m1), min(max(sid1, 0), nslot_m1)};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int base = uni((int)(size_t)dst + 1024 * h);
      if constexpr (BUF) {
        const int src = (int)((unsigned)sids[h] * ROWB + gofs);
        static_for<0, 18>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              pool_rsrc, (__attribute__((address_space(3))) void*)(size_t)(base + 1984 * i), 16, src, 0,
              64 * i, 0);
        });
      } else {
        const char* src = poolb + (long long)sids[h] * ROWB + gofs;
        static_for<0, 18>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(size_t)(base + 1984 * i),
                                           16, 64 * i, 0);
        });
      }
    }
  };

  // ---- block order ----
  // The range's blocks b0 + q, q = 0 .. n-1, are taken in order of q.  Step 0
  // gives q = 0, 1, 2 to waves 0, 1, 2 (wave 3's buffer first stages the
  // queries); step k >= 1 gives q = 4k - 1 to wave 3 and q = 4k + w to waves
  // w < 3, so wave 3 gathers its first block while step 0 runs.  A wave whose
  // q is past the range gathers nothing and skips its scores, and every
  // wave's value product skips that block.
  // Position q holds block b0 + (q + rot) % n: the tiles of one part start
  // at different blocks (rot = 3 t mod n), so a block one tile takes in a
  // later step was already brought into the XCD's L2 by another tile's first
  // step.
  const int n = b1 - b0;
  const int nsteps = n <= 3 ? 1 : 1 + (n - 3 + NW - 1) / NW;
  const int rot = (3 * t) % n;
  auto pos_of = [](int k, int w) { return NW * k + (w == 3 ? -1 : w); };
  auto block_at = [&](int q) { return b0 + (q + rot) % n; };  // q >= 0
  auto live = [&](int k, int w) {
    const int q = pos_of(k, w);
    return q >= 0 && q < n;
  };

  // ---- prologue: slots of the first blocks, the queries through buffer 3 ----
  const int b_first = block_at(wave == 3 ? 3 : wave);
  int i0 = load_idx(b_first, 0), i1 = load_idx(b_first, 1);
  // The slots and the ancestor words are taken before the queries' loads go
  // out: the compiler waits for every outstanding load at a load's first use,
  // and the first gathers would otherwise queue behind the queries.
#pragma unroll
  for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(vw[k]));
  asm volatile("" : "+v"(i0), "+v"(i1));
  {
    // wave w stages groups 2 (9 (w >> 1) + i) + (w & 1), i < 9, of the query
    // tile (tile row 16 (w & 1) + lane / 4; rows past the request: its last)
    const int qr = t * MTN + 16 * (wave & 1) + (lane >> 2);
    const char* src = reinterpret_cast<const char*>(qg) +
                      ((long long)g.q0 * p.H + min(qr, g.R - 1)) * ROWB + gofs + 576 * (wave >> 1);
    asm volatile("" : "+v"(src));
    const int base = uni((int)(size_t)(lds + 3 * BUFB) + 18432 * (wave >> 1) + 1024 * (wave & 1));
    static_for<0, 9>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(size_t)(base + 1984 * i),
                                       16, 64 * i, 0);
    });
  }
  __builtin_amdgcn_sched_barrier(0);
  const bool gather0 = wave < 3 && live(0, wave);
  if (gather0) gather(own, i0, i1);
  __builtin_amdgcn_sched_barrier(0);
  // the query tile has landed for every wave (waves 0-2 may still gather)
  if (gather0) {
    barrier_after<waitcnt_imm(36, 0)>();
  } else {
    barrier_after<waitcnt_imm(0, 0)>();
  }
  // B operand of k-step j: features 16 j + 8 hl .. +7 of row l32.  Held in
  // AGPRs (matrix-core operands may come from either file), which leaves the
  // VGPRs to the fragments read ahead in the loops below.
  // (all reads issued before the first pin, which waits for its operand)
  bf16x8_t qf[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) qf[k] = lds_ld<bf16x8_t>(lds + 3 * BUFB + (k & 1 ? kofs1 : kofs0) + 2048 * (k >> 1));
#pragma unroll
  for (int k = 0; k < KS; ++k) asm volatile("" : "+a"(qf[k]));
  barrier_after<waitcnt_imm(VM_ANY, 0)>();  // buffer 3 is free
  if (wave == 3 && live(1, 3)) gather(own, i0, i1);
  __builtin_amdgcn_sched_barrier(0);

  f32x16_t o[4];  // O^T: features 128 wave + 32 fb .. +31 of row l32
#pragma unroll
  for (int fb = 0; fb < 4; ++fb) o[fb] = f32x16_t{};
  const float c = p.scale_log2;
  float m_run = -INFINITY;  // the row's reference, the same in every wave
  float l_run = 0.f;        // this wave's columns' share of the row sum

  for (int k = 0; k < nsteps; ++k) {
    const bool mine = live(k, wave);
    const int blk = block_at(max(pos_of(k, wave), 0));
    if (mine && k > 0 && !(wave == 3 && k == 1)) gather(own, i0, i1);
    __builtin_amdgcn_sched_barrier(0);
    // slots of the next step's block (past the range: clamped, unused)
    const int b_next = block_at(pos_of(k + 1, wave));
    i0 = load_idx(b_next, 0);
    i1 = load_idx(b_next, 1);
    // this wave's block has landed: every load but the two slot loads just
    // issued (cold reads, left in flight) is done.  The gathers write LDS
    // behind the compiler's back: no LDS read may move above this wait.
    __builtin_amdgcn_sched_barrier(0);
    if (mine) __builtin_amdgcn_s_waitcnt(waitcnt_imm(2, 15));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // scores of the 32 rows against this wave's block, the fragments read
    // KDN steps ahead; lane (l32, hl) holds columns 8 (x >> 2) + 4 hl + (x & 3)
    // of row l32
    f32x16_t sc = f32x16_t{};
    float mb = -INFINITY;
    if (mine) {
      bf16x8_t kf[KS];
      auto kread = [&](int j) { return lds_ld<bf16x8_t>(own + (j & 1 ? kofs1 : kofs0) + 2048 * (j >> 1)); };
      static_for<0, KDN>([&](auto jc) { kf[jc] = kread(jc); });
      static_for<0, KS>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (j + KDN < KS) kf[j + KDN] = kread(j + KDN);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf[j], sc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      const uint32_t vis = mask_word(blk, b1, g, p.W, vw, vrow) >> (4 * hl);
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (!((vis >> (8 * (x >> 2) + (x & 3))) & 1u)) sc[x] = -INFINITY;
      mb = max3(max3(sc[0], sc[1], sc[2]), max3(sc[3], sc[4], sc[5]), max3(sc[6], sc[7], sc[8]));
      mb = max3(max3(sc[9], sc[10], sc[11]), max3(sc[12], sc[13], sc[14]), max3(sc[15], mb, mb));
    }
    mb = fmaxf(mb, other_half(mb));
    if (hl == 0) lds_st(red + 128 * wave + 4 * l32, mb);
    barrier_after<waitcnt_imm(VM_ANY, 0)>();

    // the step's maximum of each row, the reference (moved only when the
    // maximum exceeds it by RESCALE_SLACK, so rescales are rare and weights
    // stay below 2^RESCALE_SLACK; O and l share it, so the result is exact)
    const float m4 = max3(lds_ld<float>(red + 4 * l32), lds_ld<float>(red + 128 + 4 * l32),
                          fmaxf(lds_ld<float>(red + 256 + 4 * l32), lds_ld<float>(red + 384 + 4 * l32))) *
                     c;  // c > 0
    const float m_new = m4 > m_run + RESCALE_SLACK ? m4 : m_run;  // also moves from -inf
    const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    if (mine) {
      const float mu = m_run == -INFINITY ? 0.f : m_run;
      uint32_t pw[8];
#pragma unroll
      for (int x = 0; x < 16; x += 2) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[x], c, -mu));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[x + 1], c, -mu));
        l_run += e0 + e1;
        const bf16x2_t two = {(__bf16)e0, (__bf16)e1};
        pw[x >> 1] = __builtin_bit_cast(uint32_t, two);
      }
      // P^T in the B-operand layout of the value product: k-step 0 holds
      // columns x = 0..7 of the lane, k-step 1 x = 8..15
      lds_st(pbuf + 2048 * wave + 16 * lane, __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0], pw[1], pw[2], pw[3]}));
      lds_st(pbuf + 2048 * wave + 1024 + 16 * lane,
             __builtin_bit_cast(bf16x8_t, u32x4_t{pw[4], pw[5], pw[6], pw[7]}));
    }
    if (alpha != 1.f) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) o[fb] *= alpha;
    }
    barrier_after<waitcnt_imm(VM_ANY, 0)>();

    // values: this wave's 128 features over the step's live blocks, in order
    // of q (step 0: waves 0, 1, 2; later steps: 3, 0, 1, 2 -- a prefix of
    // that order is live); per block both P^T fragments and all eight value
    // fragments are read before its 8 MFMAs
    const int nlive = k == 0 ? min(n, 3) : min(max(n - pos_of(k, 3), 0), NW);
    for (int i = 0; i < nlive; ++i) {
      const int sb = k == 0 ? i : (i + 3) & 3;
      const lds_char* vb = lds + sb * BUFB;
      bf16x8_t pf[2], vf[8];
      pf[0] = lds_ld<bf16x8_t>(pbuf + 2048 * sb + 16 * lane);
      pf[1] = lds_ld<bf16x8_t>(pbuf + 2048 * sb + 1024 + 16 * lane);
      static_for<0, 8>([&](auto jc) {
        constexpr int j = decltype(jc)::value;  // k-step j >> 2, feature block j & 3
        const int off = 1024 * (j >> 2) + 2048 * (j & 3);
        const bf16x4_t lo = lds_read_tr(vb + vofs0 + off);
        const bf16x4_t hi = lds_read_tr(vb + vofs1 + off);
        vf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      });
      static_for<0, 8>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], pf[j >> 2], o[j & 3], 0, 0, 0);
      });
    }
    // every wave is done with the buffers, P^T and the maxima
    barrier_after<waitcnt_imm(VM_ANY, 0)>();
  }

  // ---- the rows' sums, then the output or the partial ----
  const float l_row = l_run + other_half(l_run);
  if (hl == 0) lds_st(lsum + 128 * wave + 4 * l32, l_row);
  barrier_after<waitcnt_imm(0, 0)>();
  const float L = lds_ld<float>(lsum + 4 * l32) + lds_ld<float>(lsum + 128 + 4 * l32) +
                  lds_ld<float>(lsum + 256 + 4 * l32) + lds_ld<float>(lsum + 384 + 4 * l32);
  const float M = m_run;
  if (S == 1) {
    // the whole tile: bf16 O / l, staged in this wave's block buffer (rows
    // of 256 bytes padded by 16) and written as row segments
    constexpr int STR = 256 + 16;
    const float inv = 1.f / L;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[fb][4 * gq + e] * inv);
        lds_st(own + l32 * STR + 2 * (32 * fb + 8 * gq + 4 * hl), v4);
      }
    __bf16* out = static_cast<__bf16*>(p.out) + ((size_t)g.q0 * p.H + t * MTN) * DV + 128 * wave + 8 * (lane & 15);
#pragma unroll
    for (int i = 0; i < MTN / 4; ++i) {
      const int trow = 4 * i + (lane >> 4);
      const bf16x8_t v = lds_ld<bf16x8_t>(own + trow * STR + 16 * (lane & 15));
      if (t * MTN + trow < g.R) *reinterpret_cast<bf16x8_t*>(out + (size_t)trow * DV) = v;
    }
    if (p.lse && wave == 0 && hl == 0 && row_ok)
      p.lse[(size_t)g.q0 * p.H + rho] = (M + log2f(L)) * LN2;
    return;
  }
  // The partial (stored non-temporally: nothing on this XCD reads it again,
  // and fewer dirty lines are left to write back when the kernel ends): O / l of every row (a weighted mean of the c_kv rows the
  // range saw) in fp16 after a power-of-two scale per row and feature quarter
  // that brings its largest magnitude into [2^14, 2^15), in the
  // accumulators' lane layout -- store (fb, gp) of wave w writes 1 KB at half
  // offset ((4 w + fb) 2 + gp) 512, lane l's 16 bytes holding features
  // 128 w + 32 fb + 16 gp + 4 (l >> 5) .. +3 and the same + 8 of row l & 31 --
  // then per feature quarter and row {m, l, inverse scale, 0} in fp32 (one
  // 16-byte load per part in the merge).  A row that saw no column (l = 0,
  // m = -inf) stores zeros; the merge skips it.
  float* base = p.ws + (((long long)r * p.T_max + t) * S + s) * slot_floats_narrow();
  float* stats = base + MTN * DV / 2;
  _Float16* ob = reinterpret_cast<_Float16*>(base) + (size_t)wave * (4 * 2 * 512) + 8 * lane;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float mx = 0.f;
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(o[fb][e]));
  mx = fmaxf(mx, other_half(mx)) * inv;
  int ex = 0;
  (void)frexpf(mx, &ex);  // mx < 2^ex (ex = 0 for mx = 0)
  ex = min(max(ex, -100), 100);
  const float f = inv * ldexpf(1.f, 15 - ex);
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      f16x8_t v8;
#pragma unroll
      for (int e = 0; e < 8; ++e) v8[e] = (_Float16)(o[fb][8 * gp + e] * f);
      __builtin_nontemporal_store(v8, reinterpret_cast<f16x8_t*>(ob + (fb * 2 + gp) * 512));
    }
  if (hl == 0)
    __builtin_nontemporal_store(f32x4_t{M, L, ldexpf(1.f, ex - 15), 0.f}, reinterpret_cast<f32x4_t*>(stats + 4 * (wave * MTN + l32)));
#endif  // __HIP_DEVICE_COMPILE__
}

// Merge of the narrow kernel's partials: one workgroup of NMW waves per
// (request, tile, run of 1 KB).  Wave h folds its share of the S parts in
// order by log-sum-exp (part j enters with the weight l_j 2^(m_j - M), its
// values times their inverse scale), lane l holding row l & 31's eight
// features of the run; wave 0 then folds the other waves' states in wave
// order.  A wave keeps few loads in flight, so spreading the parts over
// four waves shortens the round trip (one wave per run: 24.3 us for the
// 8-head shard call, two: 23.4, four: 22.8, eight: 23.2).  The slots' places
// do not depend on the request's offsets, so their loads and the offsets'
// go out together.
constexpr int NMW = 4;  // merge waves per run
template <int NM_BATCH>  // parts whose loads are in flight together, per wave
__global__ __launch_bounds__(NMW * 64) void merge_narrow_kernel(Params p_all) {
  const Params p = at_layer(p_all);
  const int run = blockIdx.x & 31, tile = blockIdx.x >> 5;
  const int r = tile / p.T_max, t = tile % p.T_max;
  if (r >= p.bs) return;
  const int lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
  const int half = threadIdx.x >> 6;  // wave h folds parts [h S2, min(S, (h + 1) S2))
  const int S2 = (p.S + NMW - 1) / NMW;
  const int j_lo = min(half * S2, p.S), j_hi = min(p.S, j_lo + S2);
  const int w = run >> 3;  // feature quarter of the run
  const long long sf = slot_floats_narrow();
  const float* slot0 = p.ws + ((long long)r * p.T_max + t) * p.S * sf;
  float M = -INFINITY, L = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  f32x4_t st[NM_BATCH];  // {m, l, inverse scale, 0} of the lane's row and quarter
  f16x8_t x[NM_BATCH];
  // Two loads per part (a wave keeps at most 63 in flight).  No load is
  // conditional (a branch around a load makes the compiler wait for every
  // load before it): parts past the wave's last reread it, unused.
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int j = 0; j < NM_BATCH; ++j) {
      const float* base = slot0 + (long long)min(j0 + j, j_hi - 1) * sf;
      st[j] = *reinterpret_cast<const f32x4_t*>(base + MT_NARROW * DV / 2 + 4 * (w * MT_NARROW + l32));
      x[j] = *reinterpret_cast<const f16x8_t*>(reinterpret_cast<const _Float16*>(base) + run * 512 + 8 * lane);
    }
  };
  // fold (m, l, the lane's eight values times their weight) into the state by
  // log-sum-exp: the part enters with the weight l 2^(m - M)
  auto fold = [&](float mj, float lj, float scale, const float* y) {
    if (mj == -INFINITY) return;  // the row saw no column in this part (or none at all)
    const float Mn = fmaxf(M, mj);
    const float a = M == -INFINITY ? 0.f : exp2f(M - Mn);
    const float wj = lj * exp2f(mj - Mn);
    const float wv = wj * scale;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a + y[e] * wv;
    L = L * a + wj;
    M = Mn;
  };
  auto fold_batch = [&](int j0) {
#pragma unroll
    for (int j = 0; j < NM_BATCH; ++j) {
      if (j0 + j >= j_hi) continue;
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (float)x[j][e];
      fold(st[j][0], st[j][1], st[j][2], y);
    }
  };
  load_batch(min(j_lo, p.S - 1));
  // the request's offsets are read after the first parts' loads are issued
  // (nothing moves across this statement), so both are in flight together
  asm volatile("" ::: "memory");
  const Geom g = geom(p.qo, p.kvp, r, p.H, MT_NARROW);
  fold_batch(j_lo);
  for (int j0 = j_lo + NM_BATCH; j0 < j_hi; j0 += NM_BATCH) {
    load_batch(j0);
    fold_batch(j0);
  }
  // waves 1 .. NMW-1 hand their (M, L, values) to wave 0, which folds them
  // in wave order (values weighted relative to the wave's M: divided by its
  // L they are the weighted mean a part carries)
  __shared__ float hand[NMW][64][10];
  hand[half][lane][0] = M;
  hand[half][lane][1] = L;
#pragma unroll
  for (int e = 0; e < 8; ++e) hand[half][lane][2 + e] = acc[e];
  __syncthreads();
  if (half != 0) return;
#pragma unroll
  for (int h = 1; h < NMW; ++h)
    fold(hand[h][lane][0], hand[h][lane][1], hand[h][lane][1] > 0.f ? 1.f / hand[h][lane][1] : 0.f,
         &hand[h][lane][2]);
  // a tile past the request's end, or a row past it (its slots were never
  // written)
  if (t >= g.T || t * MT_NARROW + l32 >= g.R) return;
  const float inv = 1.f / L;
  // run (fb, gp) of quarter w: features 128 w + 32 fb + 16 gp + 4 hl .. +3 and + 8
  const int fb = (run >> 1) & 3, gp = run & 1;
  __bf16* out = static_cast<__bf16*>(p.out) + ((size_t)g.q0 * p.H + t * MT_NARROW + l32) * DV + 128 * w +
                32 * fb + 16 * gp + 4 * hl;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    bf16x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[4 * h2 + e] * inv);
    *reinterpret_cast<bf16x4_t*>(out + 8 * h2) = v;
  }
  if (p.lse && run == 0 && hl == 0) p.lse[(size_t)g.q0 * p.H + t * MT_NARROW + l32] = (M + log2f(L)) * LN2;
}

}  // namespace

int launch_narrow(const Params& p, hipStream_t s) {
  // eight XCD columns of ceil(S / 8) parts x every tile
  const unsigned grid = (unsigned)(8LL * ((p.S + 7) / 8) * p.bs * p.T_max);
  if (p.num_slots * (long long)ROWB <= 0xffffffffLL)
    hipLaunchKernelGGL((attn_narrow_kernel<true>), dim3(grid, p.L), dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((attn_narrow_kernel<false>), dim3(grid, p.L), dim3(NW * 64), 0, s, p);
  int rc = check_launch("verify_attn(narrow)");
  if (rc != DDTREE_OK || p.S == 1) return rc;
  const dim3 mgrid((unsigned)((long long)p.bs * p.T_max * 32), p.L);
  if (p.S <= 8)
    hipLaunchKernelGGL(merge_narrow_kernel<2>, mgrid, dim3(NMW * 64), 0, s, p);
  else
    hipLaunchKernelGGL(merge_narrow_kernel<6>, mgrid, dim3(NMW * 64), 0, s, p);
  return check_launch("verify_attn(narrow merge)");
}

}  // namespace attn
}  // namespace ddtree
