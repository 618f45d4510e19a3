// Fused flash-style attention over the quantized workspace.  Three kernels:
// attn_fp8_kernel (FP8 Q/K codes, asynchronous LDS ring; optionally
// quantizing Q itself from bf16), attn_mx_kernel (MXFP4 Q/K codes, scores on
// the scaled MFMA in its FP4 format, same ring and schedule) and
// attn_fp4_kernel (FP4 Q/K codes with fp32 scales per 16 channels, scores
// from f16 hi parts plus FP8 hi/lo corrections).  What follows describes the
// structure all share; the FP4 kernel's workgroups differ (8 waves in two
// groups, one workgroup per CU, described at that kernel).
//
// Work split: each wave owns 32 consecutive queries of one (b,h) and walks
// all keys in steps of 64, in ascending order (the online-softmax step of the
// method).  In the FP8 and MXFP4 kernels a workgroup is 4 waves = 128 queries
// and two workgroups share a CU, so each SIMD runs two waves whose MFMA and
// softmax phases interleave.
//
// Per 64-key step t a wave computes
//   S^T (64 keys x 32 queries) = K_tile . Q^T      (MFMA, keys on rows)
// so that each lane owns one query column: the row max, the exponentials and
// the row sum stay in-lane, with one exchange between lanes l and l^32 for
// the max.  The probabilities, quantized to FP8 as E4M3(448 p), are packed
// straight from the S^T accumulator into the B operand of
//   O^T (128 channels x 32 queries) += V_tile^T . P^T   (FP8 MFMA)
// The accumulator holds its 16 keys per lane in a fixed order; the V tiles
// are stored by the quantize step in that same key order, so no shuffle is
// needed.
//
// Pipeline: step t issues the score MFMAs of step t+1 and the value MFMAs of
// step t-1 while the VALU runs the softmax of step t, so the matrix cores
// work beside the softmax in one instruction stream.  The accumulator
// recursion is the online-softmax one delayed by a step: step t first
// rescales O^T by alpha(t-1), then accumulates V(t-1)^T P(t-1)^T.  Tiles are
// 8 KB with a 16-byte-chunk XOR swizzle under which the 128-bit operand reads
// show no LDS bank conflicts (SQ_LDS_BANK_CONFLICT = 0 on the Kontext shape).
//
// Numerics: scores are exact FP8 dot products accumulated in fp32 by the
// MFMA; one per-step constant c = tau*log2(e)*sQ*sK >= 0 (tau*log2(e) in
// MXFP4 mode, where the MFMA applies the scales) turns them into base-2
// logits; p*448 = exp2(s*c - m + log2 448); the running max m is taken over
// the exact per-step maxima; the rescale exp2(m_old - m_new) is skipped when
// no lane's maximum moved (then it is exactly 1).
#include <atomic>
#include <type_traits>

#include "qsdpa_device.h"
#include "qsdpa_launch.h"

namespace qsdpa {

constexpr int WAVES = 4;
constexpr int QW = 32;              // queries per wave
constexpr int QT = QW * WAVES;      // queries per workgroup
constexpr int FP4_WAVES = 8, FP4_T = 64 * FP4_WAVES;   // FP4 kernel: two groups of four waves
constexpr int KTILE = KSTEP * D;    // bytes of an FP8 K tile / V^T tile

// LDS byte offset of 16-byte chunk c of row `row` in an FP8 K tile (128-B rows).
__device__ __forceinline__ int k_off(int row, int c) { return row * 128 + ((c ^ ((row ^ (row >> 3)) & 7)) << 4); }
// ... of a V^T tile (64-B channel rows, 4 chunks).
__device__ __forceinline__ int v_off(int d, int c) { return d * 64 + ((c ^ ((d >> 2) & 3)) << 4); }

__device__ __forceinline__ v8i lds_v8i(const uint8_t* p0, const uint8_t* p1) {
  const u32x4 a = *(const u32x4*)p0, b = *(const u32x4*)p1;
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// IEEE-754 maximum (v_maximum3_f32).  On the finite scores of the softmax it
// gives the same value as fmaxf, whose maxnum semantics make the compiler
// quiet each operand that is not known canonical (an MFMA result, a lane swap,
// the running max) with an extra v_max_f32 x, x, x.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// max / sum of a value over the lane pair (l, l^32): one v_permlane32_swap
// exchanges the two halves of the wave.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// A register whose value does not matter (the first of two half-word FP8
// conversions into a dword overwrites only its low half; the second fills the
// high half), so no instruction is spent initialising it.
__device__ __forceinline__ int undef_int() {
  int x;
  asm volatile("" : "=v"(x));
  return x;
}

// Issue priority by dispatch round.  Workgroups start in id order as slots
// free up, `slots` at a time (two per CU), and a SIMD's arbiter favours its
// older wave: the younger of two only takes the cycles the older leaves
// idle.  Near the end of the grid that makes the last workgroups, which start
// beside an older one and carry the most remaining work, crawl until their
// partner finishes and then run alone.  With s_setprio 3 for the last round
// and 1 for the one before (the best of the level patterns measured), the
// later workgroup leads instead: Kontext FP8 attention 2.3 % faster, MXFP4
// 2.5 %.
__device__ __forceinline__ void set_round_priority(int slots) {
  const int round = (int)blockIdx.x / slots, last = ((int)gridDim.x - 1) / slots;
  if (round == last) __builtin_amdgcn_s_setprio(3);
  else if (round == last - 1) __builtin_amdgcn_s_setprio(1);
}

// Maps the hardware workgroup id so that each XCD (ids are dealt round-robin
// over the 8 XCDs) receives one contiguous range of logical workgroups:
// consecutive query tiles of a head then share one L2.
__device__ __forceinline__ int xcd_remap(int hw, int n) {
  const int xcd = hw & 7, slot = hw >> 3;
  const int q = n >> 3, rem = n & 7;
  return xcd * q + min(xcd, rem) + slot;
}


// ---------------------------------------------------------------------------
// Pieces shared by the kernels
// ---------------------------------------------------------------------------

// Online softmax of one 64-key step for the 32 raw scores a lane holds (two
// 16-value accumulator blocks, overwritten by the weights).  c turns a raw
// score into a base-2 logit.  Returns the FP8 weights E4M3(448 p) packed in
// B-operand order (slot j = kb*16 + i); updates the running max m and the sum
// l of the unquantized p; alpha = exp2(m_old - m_new), exactly 1 when the max
// did not move.  FULL = false masks keys at or past N (the last step).
template <bool FULL>
__device__ __forceinline__ v8i softmax_step(v16f* s, float c, float& m, float& l, float& alpha,
                                            int key0, int N, int g) {
  float m_new;
  if constexpr (FULL) {
    float m0 = vmax(vmax(s[0][0], s[0][1]), s[0][2]);
    float m1 = vmax(vmax(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) {
      m0 = vmax(vmax(m0, s[0][i]), s[0][i + 1]);
      m1 = vmax(vmax(m1, s[1][i]), s[1][i + 1]);
    }
    const float mx = pair_max(vmax(vmax(m0, s[0][15]), vmax(m1, s[1][15])));
    m_new = vmax(m, c * mx);
    const float b = LOG2_448 - m_new;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, b));
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        s[kb][i] = key < N ? s[kb][i] * c : -INFINITY;
        mx = vmax(mx, s[kb][i]);
      }
    m_new = vmax(m, pair_max(mx));
    const float b = LOG2_448 - m_new;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(s[kb][i] + b);
  }
  v8i pb;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int kb = w >> 2, i0 = 4 * (w & 3);
    const int x = cvt_e4m3x2<false>(s[kb][i0], s[kb][i0 + 1], undef_int());
    pb[w] = cvt_e4m3x2<true>(s[kb][i0 + 2], s[kb][i0 + 3], x);
  }
  // row sum of the unquantized p (four independent chains)
  float ps[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
  for (int i = 4; i < 16; ++i) ps[i & 3] += s[0][i];
#pragma unroll
  for (int i = 0; i < 16; ++i) ps[i & 3] += s[1][i];
  const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  alpha = m_new != m ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
  l = alpha * l + psum;
  // materialize l here: otherwise the compiler defers the row sums of
  // several unrolled steps to the end of the loop body, keeping their p
  // values live and issuing the adds as one burst with no MFMA beside them
  asm volatile("" : "+v"(l));
  m = m_new;
  return pb;
}

// O^T *= alpha, skipped when alpha is exactly 1 in every lane
__device__ __forceinline__ void rescale_o(v16f* o, float alpha) {
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
  }
}

// O^T += V^T . P^T for the V^T tile at vbuf (channel rows db*32 + r)
__device__ __forceinline__ void value_mfma(v16f* o, const v8i& pb, const uint8_t* vbuf, int voff0, int voff1) {
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const v8i a = lds_v8i(vbuf + db * 2048 + voff0, vbuf + db * 2048 + voff1);
    o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o[db], 0, 0, 0, 127, 0, 127);
  }
}

// O = acc * sV / (448 l) as bf16 for query q (one lane pair holds it):
// each lane stores 16 runs of 4 channels (8 bytes).
__device__ __forceinline__ void store_out(const v16f* o, float l, uint16_t* __restrict__ out,
                                          const float* __restrict__ vsc, size_t row, bool valid, int g) {
  const float inv_l = 1.f / pair_sum(l);
  if (!valid) return;
  uint16_t* orow = out + row * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = db * 32 + 8 * rg + 4 * g;
      const uint32_t b0 = f32_to_bf16(o[db][4 * rg + 0] * (vsc[d0 + 0] * inv_l));
      const uint32_t b1 = f32_to_bf16(o[db][4 * rg + 1] * (vsc[d0 + 1] * inv_l));
      const uint32_t b2 = f32_to_bf16(o[db][4 * rg + 2] * (vsc[d0 + 2] * inv_l));
      const uint32_t b3 = f32_to_bf16(o[db][4 * rg + 3] * (vsc[d0 + 3] * inv_l));
      *(u32x2*)(orow + d0) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
    }
}

// ---------------------------------------------------------------------------
// FP8 kernel.  K and V^T tiles go from HBM/L2 straight into LDS
// (global_load_lds_dwordx4: no registers, no LDS store instructions) through
// a ring of 4 stages, issued 3 steps before they are read:
//   step t reads K(t+1) (scores of step t+1) and V(t-1) (values of step t-1)
//   and issues the loads of K(t+4) and V(t+2).
// Each wave issues 4 such loads per step, so at the end of step t a wave waits
// until at most 8 of its loads are outstanding (those of steps t-1 and t),
// which means K(t+2) and V(t) have landed (given the prologue's issue order,
// ring_prologue), then joins the barrier.  The barrier is a plain s_barrier:
// the only loads in flight across it are these ring loads, which target
// stages no wave reads before the wait that covers them.
// ---------------------------------------------------------------------------
constexpr int NSTAGE = 4;

// One 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4): lane i
// reads gbase + voff and the wave writes 64 x 16 contiguous bytes at LDS byte
// address lds.  Written as one asm statement (M0 set and load issued together)
// so that no compiler-inserted wait lands between the ring loads; the
// instruction has no VGPR result, and completion is awaited explicitly with
// s_waitcnt vmcnt before the barrier that publishes the stage.  Every global
// load in the loop is one of these, so the explicit vmcnt counts are exact.
__device__ __forceinline__ void ring_copy16(const uint8_t* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// LDS byte address of p, made a wave-uniform (scalar) value for M0
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p);
}

#ifdef QSDPA_RING_STRESS
// Race-detection build of the library (libqsdpa_stress.so): at each point
// where the tile ring hands stages between waves, every wave sleeps for a
// pseudo-random 0, 64, 128, 256 or 448 cycles, drawn per (workgroup, wave,
// step, site).  Waves then reach the ring's waits and barriers in orders the
// normal build rarely produces; with every wait in place the output stays
// bit-identical to the normal build's, which a GPU test checks.
__device__ __forceinline__ void ring_stress(int t, int site) {
  uint32_t h = (uint32_t)blockIdx.x * 0x9E3779B1u +
               (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 0x85EBCA77u +
               (uint32_t)t * 0xC2B2AE3Du + (uint32_t)site * 0x27D4EB2Fu;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  switch (h & 7u) {
    case 1: __builtin_amdgcn_s_sleep(1); break;
    case 2: __builtin_amdgcn_s_sleep(2); break;
    case 3: __builtin_amdgcn_s_sleep(4); break;
    case 4: __builtin_amdgcn_s_sleep(7); break;
    default: break;
  }
}
#else
__device__ __forceinline__ void ring_stress(int, int) {}
#endif

// The ring's start: K(0), K(1), K(2), V(0), K(3), V(1), in that order, so
// that after K(0) and K(1) the copies go out as K(j+2), V(j) pairs: K(0)
// K(1) | K(2) V(0) | K(3) V(1) | K(4) V(2) | ...  (K(t+4) and V(t+2) issued
// by step t).  A wave then has 2t + 8 copy groups (2 copies each) issued by
// the end of step t, and a wait for at most 8 outstanding copies means the
// first 2t + 4 groups landed, the last two of them K(t+2) and V(t): the
// operands of step t+1.  Tiles past the last one repeat it.
template <class RK, class RV>
__device__ __forceinline__ void ring_prologue(RK ring_k, RV ring_v, int Tm1) {
  ring_stress(-1, 0);
  ring_k(0, 0);
  ring_k(min(1, Tm1), 1);
  ring_k(min(2, Tm1), 2);
  ring_v(0, 0);
  ring_k(min(3, Tm1), 3);
  ring_v(min(1, Tm1), 1);
}

// After the prologue's score reads of K(0): every wave's LDS reads have
// returned before any wave passes, so step 0 may refill K stage 0.
__device__ __forceinline__ void ring_release() {
  ring_stress(-1, 1);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void ring_barrier_wait8(int t) {
  ring_stress(t, 3);
  // s_waitcnt vmcnt(8) lgkmcnt(0): ring copies of the last two steps may stay
  // in flight; every LDS read of this wave has returned before the barrier,
  // so a stage can be refilled right after it
  __builtin_amdgcn_s_waitcnt(0x0070 | 8);
  asm volatile("s_barrier" ::: "memory");
}

// FUSE_Q: Q comes as bf16 (qx) and this kernel computes its block scale and
// codes in the prologue, with the operations of the quantize pass (same
// block, same IEEE divisions, products and conversions), so the result is
// bit-identical to quantizing Q first; qc and qs are then not read.
template <bool FUSE_Q>
__global__ __launch_bounds__(256, 2) void attn_fp8_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qs, const uint16_t* __restrict__ qx,
    const uint8_t* __restrict__ kc, const float* __restrict__ ks, const uint8_t* __restrict__ vc,
    const float* __restrict__ vs, uint16_t* __restrict__ out, int N, int n_pad, int block_q,
    int q_scale_count, int k_scale_count, float tau_log2e, int tiles_per_bh, int prio_slots,
    double* __restrict__ vc_err) {
  set_round_priority(prio_slots);
  // ring: stages 0..3 of K tiles, then stages 0..3 of V^T tiles
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * NSTAGE * KTILE];
  auto lds_k = [&](int S) -> uint8_t* { return ring + S * KTILE; };
  auto lds_v = [&](int S) -> uint8_t* { return ring + (NSTAGE + S) * KTILE; };
  // LDS byte address of the ring and this wave's 2 KB slice of a stage, as scalars
  const uint32_t ring_lds = lds_addr(ring);
  const uint32_t wave_lds = ring_lds + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 2048u;

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / tiles_per_bh, tile = wg - bh * tiles_per_bh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int q0 = tile * QT + wave * QW;
  const int T = (N + KSTEP - 1) / KSTEP;

  v8i qb8[2];
  float qscale = 0.f;
  auto load_q = [&]() {
    if constexpr (FUSE_Q) {
      // this lane's 64 channels of query q0 + r: 64h + 32g .. 64h + 32g + 31
      float x[2][32];
      float amax = 0.f;
      const int q = q0 + r;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4 w = {0u, 0u, 0u, 0u};
          if (q < N) w = *(const u32x4*)(qx + ((size_t)bh * N + q) * D + 64 * h + 32 * g + 8 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[h][8 * j + 2 * e] = bf16_lo(w[e]);
            x[h][8 * j + 2 * e + 1] = bf16_hi(w[e]);
          }
        }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[h][i]));
      // the scale block: all 4 waves (block_q = 128) or this wave pair (64)
      __shared__ float qred[4];
      amax = wave_max(amax);
      if (lane == 0) qred[wave] = amax;
      __syncthreads();
      amax = block_q == 128 ? fmaxf(fmaxf(qred[0], qred[1]), fmaxf(qred[2], qred[3]))
                            : fmaxf(qred[wave & 2], qred[(wave & 2) + 1]);
      const float inv0 = FP8_MAX / amax;   // not finite: amax = 0 or below FP8_MAX / FLT_MAX
      const bool live = inv0 < INFINITY;
      const float inv = live ? inv0 : 0.f;
      qscale = live ? amax / FP8_MAX : 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int lo = cvt_e4m3x2<false>(clamp448(x[h][4 * j] * inv), clamp448(x[h][4 * j + 1] * inv), 0);
          qb8[h][j] = cvt_e4m3x2<true>(clamp448(x[h][4 * j + 2] * inv), clamp448(x[h][4 * j + 3] * inv), lo);
        }
      if (vc_err) {
        // the token's own quantization error sum_d (x_d - code_d * s)^2 for the
        // selective correction: each difference is exact in fp64, the squares
        // summed in fp64 over this lane's 64 channels, then over the lane pair
        const double s = (double)qscale;
        double e = 0.0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const auto c01 = __builtin_amdgcn_cvt_pk_f32_fp8(qb8[h][j], false);
            const auto c23 = __builtin_amdgcn_cvt_pk_f32_fp8(qb8[h][j], true);
            const double d0 = (double)x[h][4 * j] - (double)c01[0] * s;
            const double d1 = (double)x[h][4 * j + 1] - (double)c01[1] * s;
            const double d2 = (double)x[h][4 * j + 2] - (double)c23[0] * s;
            const double d3 = (double)x[h][4 * j + 3] - (double)c23[1] * s;
            e = __builtin_fma(d0, d0, e);
            e = __builtin_fma(d1, d1, e);
            e = __builtin_fma(d2, d2, e);
            e = __builtin_fma(d3, d3, e);
          }
        // after the swap, element 0 holds the value of lane l & 31 and element
        // 1 that of lane l | 32 (the g = 0 and g = 1 halves of the token)
        const uint64_t eb = (uint64_t)__double_as_longlong(e);
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)eb, (uint32_t)eb, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(eb >> 32), (uint32_t)(eb >> 32), false, false);
        const double e0 = __longlong_as_double((long long)(((uint64_t)hi[0]) << 32 | lo[0]));
        const double e1 = __longlong_as_double((long long)(((uint64_t)hi[1]) << 32 | lo[1]));
        if (g == 0 && q < N) vc_err[(size_t)bh * n_pad + q] = e0 + e1;
      }
    } else {
      const uint8_t* qrow = qc + ((size_t)bh * n_pad + q0 + r) * D;
#pragma unroll
      for (int h = 0; h < 2; ++h) qb8[h] = lds_v8i(qrow + 64 * h + 32 * g, qrow + 64 * h + 32 * g + 16);
      qscale = qs[(size_t)bh * q_scale_count + q0 / block_q];
    }
  };
  if constexpr (!FUSE_Q) load_q();
  float cscale = tau_log2e * qscale;   // FUSE_Q: set once Q is quantized in the prologue
  const uint8_t* kbase = kc + (size_t)bh * n_pad * D;
  const float* ksc = ks + (size_t)bh * k_scale_count;
  const uint8_t* vbase = vc + (size_t)bh * n_pad * D;

  // K operand chunks (row kb*32 + r, chunk 4h + 2g + i): the swizzle of row
  // kb*32 + r is that of row r with bit 2 flipped by kb, so
  // offset(kb, h, i) = kb * 4096 + offset(0, h ^ kb, i).
  int koff0[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 2; ++i) koff0[h][i] = k_off(r, 4 * h + 2 * g + i);
  const int voff0 = v_off(r, 2 * g), voff1 = v_off(r, 2 * g + 1);

  // Ring loads: wave w's instruction i fills LDS chunks (2w+i)*64 + lane of a
  // stage; each lane fetches the global chunk the swizzle puts there.
  uint32_t kg[2], vg[2];   // unsigned: lets the loads use an SGPR base + 32-bit offset
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int P = (2 * wave + i) * 64 + lane;
    const int row = P >> 3, pc = P & 7;
    kg[i] = (uint32_t)(row * 128 + ((pc ^ ((row ^ (row >> 3)) & 7)) << 4));
    const int d = P >> 2, pv = P & 3;
    vg[i] = (uint32_t)(d * 64 + ((pv ^ ((d >> 2) & 3)) << 4));
  }
  auto ring_k = [&](int t, int S) {
    const uint8_t* tp = kbase + (size_t)t * KTILE;
#pragma unroll
    for (int i = 0; i < 2; ++i) ring_copy16(tp, kg[i], wave_lds + S * KTILE + i * 1024);
  };
  auto ring_v = [&](int t, int S) {
    const uint8_t* tp = vbase + (size_t)t * KTILE;
#pragma unroll
    for (int i = 0; i < 2; ++i) ring_copy16(tp, vg[i], wave_lds + (NSTAGE + S) * KTILE + i * 1024);
  };

  // a00 is the operand of the first MFMA (kb = 0, h = 0), read by the caller
  // ahead of the rescale so that its LDS latency is hidden
  auto k_first = [&](const uint8_t* kbuf) { return lds_v8i(kbuf + koff0[0][0], kbuf + koff0[0][1]); };
  auto scores = [&](const uint8_t* kbuf, v16f* s, const v8i& a00) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = v16f{};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v8i a = (kb == 0 && h == 0)
                          ? a00
                          : lds_v8i(kbuf + kb * 4096 + koff0[h ^ kb][0], kbuf + kb * 4096 + koff0[h ^ kb][1]);
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qb8[h], s[kb], 0, 0, 0, 127, 0, 127);
      }
    }
  };
  v16f o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v16f{};
  float m = -INFINITY, l = 0.f;

  // K-block scale of the step whose softmax runs next.  Each step loads the
  // next one just before its barrier wait, which covers the scalar load; a
  // load next to the LDS reads would make their waits include it.
  float kscn = ksc[0];
  auto softmax = [&](int t, v16f* s, auto full_t, float& alpha) -> v8i {
    return softmax_step<decltype(full_t)::value>(s, cscale * kscn, m, l, alpha, t * KSTEP, N, g);
  };
  auto rescale = [&](float alpha) { rescale_o(o, alpha); };
  auto pv = [&](const v8i& pb, const uint8_t* vbuf) { value_mfma(o, pb, vbuf, voff0, voff1); };

  // prologue: K(0..3) and V(0), V(1) in flight; V(-1) (stage 3) is zero.
  // The Q operand and scale loads complete first, so that from here on the
  // only vector-memory loads in flight are ring copies.  FUSE_Q issues the
  // ring copies first and then loads and quantizes Q, so that both memory
  // latencies overlap: its Q loads are younger than the copies, and loads
  // complete in order, so the waits the compiler puts before using Q also
  // cover the copies.
  const int Tm1 = T - 1;
  if constexpr (!FUSE_Q) __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0)
  ring_prologue(ring_k, ring_v, Tm1);
  if constexpr (FUSE_Q) {
    load_q();
    cscale = tau_log2e * qscale;
  }
  *(u32x4*)(lds_v(3) + tid * 16) = u32x4{0u, 0u, 0u, 0u};
  *(u32x4*)(lds_v(3) + tid * 16 + 4096) = u32x4{0u, 0u, 0u, 0u};
  // K(0), K(1) landed (at most K(2), V(0), K(3), V(1) outstanding)
  __builtin_amdgcn_s_waitcnt(0x0070 | 8);
  asm volatile("s_barrier" ::: "memory");
  v16f sa[2], sb[2];
  scores(lds_k(0), sa, k_first(lds_k(0)));
  // every wave has read K(0) before step 0 refills its stage
  ring_release();
  v8i pb_prev = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  float alpha_prev = 1.f;

  // steps 0 .. T-2 (full)
  // Instruction order of a step: the 8 MFMAs (4 scores, 4 values) spread
  // over the ~150 VALU instructions of the softmax, 19 after each, and the
  // two LDS reads of each MFMA operand issued right after the MFMA before it.
  auto step = [&](int t, v16f* s_cur, v16f* s_next, auto st) {
    constexpr int S = decltype(st)::value;   // t % 4
    const v8i a00 = k_first(lds_k((S + 1) & 3));
    rescale(alpha_prev);
    ring_stress(t, 2);
    ring_k(min(t + 4, Tm1), S);
    ring_v(min(t + 2, Tm1), (S + 2) & 3);
    scores(lds_k((S + 1) & 3), s_next, a00);
    pv(pb_prev, lds_v((S + 3) & 3));
    pb_prev = softmax(t, s_cur, std::true_type{}, alpha_prev);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
      if (i < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x402, 19, 0);         // VALU
    }
    kscn = ksc[t + 1];
    ring_barrier_wait8(t);
  };
  int t = 0;
  for (; t + 4 < T; t += 4) {
    step(t, sa, sb, std::integral_constant<int, 0>{});
    step(t + 1, sb, sa, std::integral_constant<int, 1>{});
    step(t + 2, sa, sb, std::integral_constant<int, 2>{});
    step(t + 3, sb, sa, std::integral_constant<int, 3>{});
  }
  // remaining full steps t .. T-2 (at most 3; t is a multiple of 4 here, so
  // the ring stage is t & 3 computed at run time), then the last step T-1
  auto step_dyn = [&](int tt, v16f* s_cur, v16f* s_next) {
    const int S = tt & 3;
    const v8i a00 = k_first(lds_k((S + 1) & 3));
    rescale(alpha_prev);
    ring_stress(tt, 2);
    ring_k(min(tt + 4, Tm1), S);
    ring_v(min(tt + 2, Tm1), (S + 2) & 3);
    scores(lds_k((S + 1) & 3), s_next, a00);
    pv(pb_prev, lds_v((S + 3) & 3));
    pb_prev = softmax(tt, s_cur, std::true_type{}, alpha_prev);
    kscn = ksc[tt + 1];
    ring_barrier_wait8(tt);
  };
  auto last = [&](int tl, v16f* s_cur) {
    const int S = tl & 3;
    rescale(alpha_prev);
    pv(pb_prev, lds_v((S + 3) & 3));
    float alpha;
    const v8i pb = (tl + 1) * KSTEP <= N ? softmax(tl, s_cur, std::true_type{}, alpha)
                                         : softmax(tl, s_cur, std::false_type{}, alpha);
    // V(tl) is in stage S (issued at step tl-2 or in the prologue): wait for every ring copy
    ring_stress(tl, 4);
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("s_barrier" ::: "memory");
    rescale(alpha);
    pv(pb, lds_v(S));
  };
  for (; t + 2 < T; t += 2) {
    step_dyn(t, sa, sb);
    step_dyn(t + 1, sb, sa);
  }
  if (t + 1 < T) {
    step_dyn(t, sa, sb);
    last(t + 1, sb);
  } else {
    last(t, sa);
  }

  const int q = q0 + r;
  store_out(o, l, out, vs + (size_t)bh * D, (size_t)bh * N + q, q < N, g);
}

// ---------------------------------------------------------------------------
// MXFP4 kernel: the FP8 kernel's work split, tile ring, step schedule,
// softmax and value product, with the scores on the scaled MFMA in its FP4
// format.  Q and K arrive as E2M1 codes with one E8M0 scale per 32 channels,
// and the MFMA applies those scales per lane (one byte per row or column and
// 32-channel block), so the scores come out in real units and the softmax
// constant is tau * log2(e) alone.  A K stage holds the tile's 4 KB of codes
// (rows of 64 B; 16-byte chunk c of key row r stored at chunk
// c ^ ((r >> 2) & 3), as in a V^T tile) and, per wave, a 1 KB copy of the tile's 256 scale
// bytes (four replicas): each wave copies its own, so every wave issues the
// same 4 copies per step and the ring's waits are those of the FP8 kernel.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kmx_off(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }

// score MFMA with FP4 A (K) and B (Q) operands: OA / OB select the scale byte
template <int OA, int OB>
__device__ __forceinline__ v16f mx_mfma(const v8i& a, const v8i& b, const v16f& c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, OA, (int)sa, OB, (int)sb);
}
__device__ __forceinline__ v8i lds_v4i(const uint8_t* p) {
  const u32x4 a = *(const u32x4*)p;
  return v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
}

// FUSE_Q: Q arrives as bf16 (qx) and each lane quantizes its own two 32-channel
// blocks in the prologue, with the quantize pass's operations, so the result
// is bit-identical to reading the pass's codes (qc, qs).
template <bool FUSE_Q>
__global__ __launch_bounds__(256, 2) void attn_mx_kernel(
    const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs, const uint16_t* __restrict__ qx,
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks, const uint8_t* __restrict__ vc,
    const float* __restrict__ vs, uint16_t* __restrict__ out, int N, int n_pad, float tau_log2e,
    int tiles_per_bh, int prio_slots) {
  set_round_priority(prio_slots);
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * NSTAGE * KTILE];
  auto lds_k = [&](int S) -> uint8_t* { return ring + S * KTILE; };
  auto lds_v = [&](int S) -> uint8_t* { return ring + (NSTAGE + S) * KTILE; };
  const uint32_t ring_lds = lds_addr(ring);
  const uint32_t wave_u = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wave_lds = ring_lds + wave_u * 2048u;

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / tiles_per_bh, tile = wg - bh * tiles_per_bh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int q0 = tile * QT + wave * QW;
  const int T = (N + KSTEP - 1) / KSTEP;

  // Q operand: channels 64h + 32g .. +31 (scale block 2h + g) of query q0 + r
  // as 16 bytes of codes per half h; the two scale bytes in bytes 0 and 1 of
  // qscale
  v8i qb[2];
  uint32_t qscale = 0u;
  auto load_q = [&]() {
    if constexpr (FUSE_Q) {
      const int q = q0 + r;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float x[32];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4 w = {0u, 0u, 0u, 0u};
          if (q < N) w = *(const u32x4*)(qx + ((size_t)bh * N + q) * D + 64 * h + 32 * g + 8 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[8 * j + 2 * e] = bf16_lo(w[e]);
            x[8 * j + 2 * e + 1] = bf16_hi(w[e]);
          }
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
        const uint32_t byte = amax > 0.f ? mx_scale_byte(amax) : 0u;
        const float inv = mx_inv_scale(byte);
        int words[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) words[j] = amax > 0.f ? (int)e2m1_word8(x + 8 * j, inv) : 0;
        qb[h] = v8i{words[0], words[1], words[2], words[3], 0, 0, 0, 0};
        qscale |= byte << (8 * h);
      }
    } else {
      const size_t qrow = (size_t)bh * n_pad + q0 + r;
#pragma unroll
      for (int h = 0; h < 2; ++h) qb[h] = lds_v4i(qc + qrow * 64 + 32 * h + 16 * g);
      qscale = (uint32_t)qs[qrow * 4 + g] | ((uint32_t)qs[qrow * 4 + 2 + g] << 8);
    }
  };
  if constexpr (!FUSE_Q) load_q();
  const uint8_t* kbase = kc + (size_t)bh * n_pad * 64;
  const uint8_t* ksbase = ks + (size_t)bh * (n_pad / KSTEP) * 256;
  const uint8_t* vbase = vc + (size_t)bh * n_pad * D;

  // K operand of (kb, h): row kb*32 + r, chunk 2h + g; the swizzle depends on r only
  int koff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) koff[h] = kmx_off(r, 2 * h + g);
  const int voff0 = v_off(r, 2 * g), voff1 = v_off(r, 2 * g + 1);

  // Ring copies.  K codes: wave w fills LDS chunks w*64 + lane of the stage
  // with the global chunk the swizzle puts there; scale bytes: lane l reads
  // bytes 16*(l & 15) .. +15 of the tile's 256, into the wave's own 1 KB.
  uint32_t kg, sg, vg[2];
  {
    const int P = wave * 64 + lane, row = P >> 2, pc = P & 3;
    kg = (uint32_t)(row * 64 + ((pc ^ ((row >> 2) & 3)) << 4));
    sg = (uint32_t)((lane & 15) * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int Pv = (2 * wave + i) * 64 + lane;
      const int d = Pv >> 2, pv = Pv & 3;
      vg[i] = (uint32_t)(d * 64 + ((pv ^ ((d >> 2) & 3)) << 4));
    }
  }
  auto ring_k = [&](int t, int S) {
    ring_copy16(kbase + (size_t)t * 4096, kg, ring_lds + (uint32_t)S * KTILE + wave_u * 1024u);
    ring_copy16(ksbase + (size_t)t * 256, sg, ring_lds + (uint32_t)S * KTILE + 4096u + wave_u * 1024u);
  };
  auto ring_v = [&](int t, int S) {
    const uint8_t* tp = vbase + (size_t)t * KTILE;
#pragma unroll
    for (int i = 0; i < 2; ++i) ring_copy16(tp, vg[i], wave_lds + (NSTAGE + S) * KTILE + i * 1024);
  };

  // the first score operand and the scale bytes, read by the caller ahead of
  // the rescale: byte 2*kb + h of ksw scales K operand (kb, h)
  auto k_first = [&](const uint8_t* kbuf) { return lds_v4i(kbuf + koff[0]); };
  auto k_scales = [&](const uint8_t* kbuf) { return *(const uint32_t*)(kbuf + 4096 + wave * 1024 + lane * 4); };
  auto scores = [&](const uint8_t* kbuf, v16f* s, const v8i& a00, uint32_t ksw) {
    s[0] = mx_mfma<0, 0>(a00, qb[0], v16f{}, ksw, qscale);
    s[0] = mx_mfma<1, 1>(lds_v4i(kbuf + koff[1]), qb[1], s[0], ksw, qscale);
    s[1] = mx_mfma<2, 0>(lds_v4i(kbuf + 2048 + koff[0]), qb[0], v16f{}, ksw, qscale);
    s[1] = mx_mfma<3, 1>(lds_v4i(kbuf + 2048 + koff[1]), qb[1], s[1], ksw, qscale);
  };
  v16f o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v16f{};
  float m = -INFINITY, l = 0.f;
  auto softmax = [&](int t, v16f* s, auto full_t, float& alpha) -> v8i {
    return softmax_step<decltype(full_t)::value>(s, tau_log2e, m, l, alpha, t * KSTEP, N, g);
  };
  auto rescale = [&](float alpha) { rescale_o(o, alpha); };
  auto pv = [&](const v8i& pb, const uint8_t* vbuf) { value_mfma(o, pb, vbuf, voff0, voff1); };

  // prologue as in the FP8 kernel (FUSE_Q: Q loaded after the ring copies)
  const int Tm1 = T - 1;
  if constexpr (!FUSE_Q) __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0)
  ring_prologue(ring_k, ring_v, Tm1);
  if constexpr (FUSE_Q) load_q();
  *(u32x4*)(lds_v(3) + tid * 16) = u32x4{0u, 0u, 0u, 0u};
  *(u32x4*)(lds_v(3) + tid * 16 + 4096) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_s_waitcnt(0x0070 | 8);
  asm volatile("s_barrier" ::: "memory");
  v16f sa[2], sb[2];
  scores(lds_k(0), sa, k_first(lds_k(0)), k_scales(lds_k(0)));
  ring_release();
  v8i pb_prev = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  float alpha_prev = 1.f;

  auto step = [&](int t, v16f* s_cur, v16f* s_next, auto st) {
    constexpr int S = decltype(st)::value;   // t % 4
    const v8i a00 = k_first(lds_k((S + 1) & 3));
    const uint32_t ksw = k_scales(lds_k((S + 1) & 3));
    rescale(alpha_prev);
    ring_stress(t, 2);
    ring_k(min(t + 4, Tm1), S);
    ring_v(min(t + 2, Tm1), (S + 2) & 3);
    scores(lds_k((S + 1) & 3), s_next, a00, ksw);
    pv(pb_prev, lds_v((S + 3) & 3));
    pb_prev = softmax(t, s_cur, std::true_type{}, alpha_prev);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x402, 22, 0);   // VALU
    }
    ring_barrier_wait8(t);
  };
  int t = 0;
  for (; t + 4 < T; t += 4) {
    step(t, sa, sb, std::integral_constant<int, 0>{});
    step(t + 1, sb, sa, std::integral_constant<int, 1>{});
    step(t + 2, sa, sb, std::integral_constant<int, 2>{});
    step(t + 3, sb, sa, std::integral_constant<int, 3>{});
  }
  auto step_dyn = [&](int tt, v16f* s_cur, v16f* s_next) {
    const int S = tt & 3;
    const v8i a00 = k_first(lds_k((S + 1) & 3));
    const uint32_t ksw = k_scales(lds_k((S + 1) & 3));
    rescale(alpha_prev);
    ring_stress(tt, 2);
    ring_k(min(tt + 4, Tm1), S);
    ring_v(min(tt + 2, Tm1), (S + 2) & 3);
    scores(lds_k((S + 1) & 3), s_next, a00, ksw);
    pv(pb_prev, lds_v((S + 3) & 3));
    pb_prev = softmax(tt, s_cur, std::true_type{}, alpha_prev);
    ring_barrier_wait8(tt);
  };
  auto last = [&](int tl, v16f* s_cur) {
    const int S = tl & 3;
    rescale(alpha_prev);
    pv(pb_prev, lds_v((S + 3) & 3));
    float alpha;
    const v8i pb = (tl + 1) * KSTEP <= N ? softmax(tl, s_cur, std::true_type{}, alpha)
                                         : softmax(tl, s_cur, std::false_type{}, alpha);
    ring_stress(tl, 4);
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("s_barrier" ::: "memory");
    rescale(alpha);
    pv(pb, lds_v(S));
  };
  for (; t + 2 < T; t += 2) {
    step_dyn(t, sa, sb);
    step_dyn(t + 1, sb, sa);
  }
  if (t + 1 < T) {
    step_dyn(t, sa, sb);
    last(t + 1, sb);
  } else {
    last(t, sa);
  }

  const int q = q0 + r;
  store_out(o, l, out, vs + (size_t)bh * D, (size_t)bh * N + q, q < N, g);
}

// ---------------------------------------------------------------------------
// FP4 kernel: Q and K arrive as E2M1 codes with an fp32 scale per 16
// channels.  Q is dequantized once into registers, and K comes in the tiles
// the quantize pass expanded.  With x' = code * scale * 2^-E, hi = f16(x')
// and lo = x' - hi (exact in fp32, at most 2^-11 |x'|), a score is
//   sum hi_q hi_k             one f16 MFMA per 16-channel chunk (its
//                             products are exact and it keeps 24 bits below
//                             the largest)
// + sum (hi_q lo_k + lo_q hi_k)   one FP8 MFMA per 32 channels, on E4M3
//                             copies hi8 = E4M3(hi 2^-6) and lo8 = E4M3(lo 2^5)
//                             concatenated along the contraction, its E8M0
//                             scale 2^1 undoing the powers of two;
// the FP8 roundings move each correction by at most 2^-4 of itself, so a
// score is good to about 2^-15 of its terms.  Before the split, a query row
// is scaled by 2^-EQ and a K tile by 2^-EK (fp4_norm_exp), which keeps every
// f16 and E4M3 value in range; the softmax constant tau * log2(e) *
// 2^(EQ + EK) of the lane and step takes both back.  P and V stay FP8.
// The tiles reach LDS as in the FP8 kernel, by asynchronous copies
// (global_load_lds_dwordx4), through a ring of 2 stages of 32 KB K + 8 KB V^T
// (80 KB).  The Q operands take 64 registers, so a wave has one scores
// buffer: its softmax and its MFMAs alternate.  A workgroup is 8 waves, 256
// queries, one per CU: two groups of four waves, the second running one
// half-step behind the first, so that the two waves of each SIMD alternate
// between softmax and MFMAs; the eight waves share each K/V tile, which
// halves the tile copies per query against two 4-wave workgroups per CU.
// ---------------------------------------------------------------------------
// FUSE_Q: Q arrives as bf16 (qx), and each lane makes the codes and fp32
// scales of the 8 sixteen-channel groups of its query with the quantize
// pass's operations (block maximum, IEEE divisions 6/amax and amax/6, fp32
// product, clamp, E2M1 conversion), so the result is bit-identical to reading
// the pass's codes (qc, qs).  Both lanes of a query make all 8 groups.
template <bool FUSE_Q>
__global__ __launch_bounds__(FP4_T, 1) void attn_fp4_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qs, const uint16_t* __restrict__ qx,
    const uint8_t* __restrict__ kx, const int* __restrict__ kexp, const uint8_t* __restrict__ vc,
    const float* __restrict__ vs, uint16_t* __restrict__ out, int N, int n_pad, float tau_log2e,
    int tiles_per_bh) {
  // ring: stages 0, 1 of expanded K tiles (f16 hi, then E4M3 corrections), then stages 0, 1
  // of V^T tiles: 80 KB
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * (KXTILE + KTILE)];
  auto lds_k = [&](int S) -> uint8_t* { return ring + S * KXTILE; };
  auto lds_v = [&](int S) -> uint8_t* { return ring + 2 * KXTILE + S * KTILE; };
  const uint32_t ring_lds = lds_addr(ring);
  const uint32_t wave_u = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / tiles_per_bh, tile = wg - bh * tiles_per_bh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int q0 = tile * (FP4_WAVES * QW) + wave * QW;
  const bool grp_b = wave >= FP4_WAVES / 2;   // the group one slot behind
  const int T = (N + KSTEP - 1) / KSTEP;

  // Q operands of query q0 + r, scaled by 2^-EQ of the query row (both lanes
  // of the row read all 8 scales; the softmax constant of the lane takes 2^EQ
  // back):
  //   qhi[c]: hi of channels 16c + 8g .. 16c + 8g + 7 (f16 MFMA, chunk c);
  //   qx8[p]: the 32 FP8 bytes hi8 (channels 16c .. 16c + 15) then lo8 (same
  //           channels) of chunk c = 2p + g, matching the K correction chunks
  //           lo8, hi8 of that chunk in the FP8 MFMA of channels 32p .. 32p + 31.
  v8h qhi[8];
  v8i qx8[4];
  float cq;
  {
    const size_t qrow = (size_t)bh * n_pad + q0 + r;
    // scale and the two code words (channels 16c .. 16c + 7, then + 8 .. + 15) of each group
    float sc[8], smax = 0.f;
    uint32_t cw[8][2];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (FUSE_Q) {
        const int q = q0 + r;
        u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
        if (q < N) {
          const u32x4* src = (const u32x4*)(qx + ((size_t)bh * N + q) * D + 16 * c);
          w0 = src[0];
          w1 = src[1];
        }
        float val[16];
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          val[2 * j] = bf16_lo(w0[j]);
          val[2 * j + 1] = bf16_hi(w0[j]);
          val[8 + 2 * j] = bf16_lo(w1[j]);
          val[8 + 2 * j + 1] = bf16_hi(w1[j]);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(val[j]));
        const float inv = FP4_MAX / amax;   // +inf for amax = 0 or below FP4_MAX / FLT_MAX: zero codes
        const bool live = inv < INFINITY;
        sc[c] = live ? amax / FP4_MAX : 0.f;
        cw[c][0] = live ? e2m1_word8(val, inv) : 0u;
        cw[c][1] = live ? e2m1_word8(val + 8, inv) : 0u;
      } else {
        // rows at or past n_pad (the second half of a head's last query tile) read as zero
        u32x2 w = {0u, 0u};
        sc[c] = 0.f;
        if (q0 + r < n_pad) {
          sc[c] = qs[qrow * 8 + c];
          w = *(const u32x2*)(qc + qrow * 64 + 8 * c);
        }
        cw[c][0] = w[0];
        cw[c][1] = w[1];
      }
      smax = fmaxf(smax, sc[c]);
    }
    const int EQ = fp4_norm_exp(smax);
    cq = ldexpf(tau_log2e, EQ);
    auto scaled = [&](uint32_t code, float scale) {
      float x = e2m1_value(code) * scale;
      asm volatile("" : "+v"(x));
      return ldexpf(x, -EQ);
    };
    // lane-dependent choices as bit selects (an indexed pick would put the
    // arrays in scratch memory)
    const uint32_t gm = 0u - (uint32_t)g;
    auto pick = [&](uint32_t a, uint32_t b) { return a ^ ((a ^ b) & gm); };   // g ? b : a
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t w = pick(cw[c][0], cw[c][1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qhi[c][e] = (_Float16)scaled((w >> (4 * e)) & 15u, sc[c]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // chunk c = 2p + g
      const u32x2 w = {pick(cw[2 * p][0], cw[2 * p + 1][0]), pick(cw[2 * p][1], cw[2 * p + 1][1])};
      const float scale = __uint_as_float(pick(__float_as_uint(sc[2 * p]), __float_as_uint(sc[2 * p + 1])));
      float h8[16], l8[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = scaled((w[e >> 3] >> (4 * (e & 7))) & 15u, scale);
        const float h = (float)(_Float16)x;
        h8[e] = h * 0.015625f;
        l8[e] = (x - h) * 32.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qx8[p][j] = cvt_e4m3x2<true>(h8[4 * j + 2], h8[4 * j + 3], cvt_e4m3x2<false>(h8[4 * j], h8[4 * j + 1], 0));
        qx8[p][4 + j] = cvt_e4m3x2<true>(l8[4 * j + 2], l8[4 * j + 3], cvt_e4m3x2<false>(l8[4 * j], l8[4 * j + 1], 0));
      }
    }
  }
  const uint8_t* kxbase = kx + (size_t)bh * (n_pad / KSTEP) * KXTILE;
  const int* kebase = kexp + (size_t)bh * (n_pad / KSTEP);
  const uint8_t* vbase = vc + (size_t)bh * n_pad * D;
  const int voff0 = v_off(r, 2 * g), voff1 = v_off(r, 2 * g + 1);

  // Ring copies.  An expanded K tile is already in LDS order: wave w copies
  // its 1 KB pieces 4w .. 4w+3 unchanged.  V^T tiles as in the FP8 kernel:
  // wave w fills LDS chunks w*64 + lane of a stage with the global chunk the
  // swizzle puts there.
  const uint32_t kgl = (uint32_t)lane * 16u;
  uint32_t vg;
  {
    const int P = wave * 64 + lane;
    const int d = P >> 2, pv = P & 3;
    vg = (uint32_t)(d * 64 + ((pv ^ ((d >> 2) & 3)) << 4));
  }
  auto ring_k = [&](int t, int S) {
    const uint8_t* tp = kxbase + (size_t)t * KXTILE + wave_u * 4096u;
    const uint32_t dst = ring_lds + (uint32_t)S * KXTILE + wave_u * 4096u;
#pragma unroll
    for (int i = 0; i < 4; ++i) ring_copy16(tp + i * 1024, kgl, dst + i * 1024);
  };
  auto ring_v = [&](int t, int S) {
    const uint8_t* tp = vbase + (size_t)t * KTILE;
    ring_copy16(tp, vg, ring_lds + 2 * KXTILE + (uint32_t)S * KTILE + wave_u * 1024u);
  };

  // scores of a 64-key tile: the chains of keys 0..31 and 32..63 interleaved;
  // per 32 channels two f16 hi.hi MFMAs and one FP8 correction MFMA, whose
  // lane operand is correction chunks 4p + 2g (lo8) and 4p + 2g + 1 (hi8) of
  // its key row against qx8[p] (hi8, lo8): lo_k hi_q + hi_k lo_q, times the
  // E8M0 scale 2^1 (byte 128) that undoes 2^5 * 2^-6
  auto scores = [&](const uint8_t* kbuf, v16f* s) {
    s[0] = v16f{};
    s[1] = v16f{};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * p + h;
        v8h ah[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ah[kb] = *(const v8h*)(kbuf + kh_off(kb * 32 + r, 2 * c + g));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[kb], qhi[c], s[kb], 0, 0, 0);
      }
      v8i ax[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        ax[kb] = lds_v8i(kbuf + KXTILE / 2 + kh_off(kb * 32 + r, 4 * p + 2 * g),
                         kbuf + KXTILE / 2 + kh_off(kb * 32 + r, 4 * p + 2 * g + 1));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ax[kb], qx8[p], s[kb], 0, 0, 0, 128, 0, 127);
    }
  };

  v16f o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v16f{};
  float m = -INFINITY, l = 0.f;

  // Prologue: K(0), K(1), V(0) land (after the Q loads, so that from here on
  // the only vector-memory loads in flight are ring copies), then group A
  // makes the scores of step 0.
  const int Tm1 = T - 1;
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0)
  ring_k(0, 0);
  if (T > 1) ring_k(1, 1);
  ring_v(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0070);
  asm volatile("s_barrier" ::: "memory");
  v16f s[2];
  v8i pb = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  float alpha;
  int ken = kebase[0];
  if (!grp_b) scores(lds_k(0), s);
  ring_stress(-1, 1);
  auto softmax = [&](int t) {
    const float c = ldexpf(cq, ken);
    pb = (t + 1) * KSTEP <= N ? softmax_step<true>(s, c, m, l, alpha, t * KSTEP, N, g)
                              : softmax_step<false>(s, c, m, l, alpha, t * KSTEP, N, g);
    rescale_o(o, alpha);
  };

  // Slots, each closed by a barrier of all eight waves.  Group A (waves 0-3)
  // runs the softmax of step t in slot 2t and the MFMAs of step t (values of
  // t, scores of t+1) in slot 2t+1; group B (waves 4-7, one per SIMD beside
  // a wave of group A) runs the same sequence one slot later, so that each
  // SIMD overlaps one wave's softmax with the other's MFMAs.
  // K(t) is read in slots 2t-1 (A) and 2t (B), V(t) in slots 2t+1 (A) and
  // 2t+2 (B).  Slot 2t+1 copies K(t+2) over K(t) and V(t+1) over V(t-1); the
  // copies are waited for at the end of slot 2t+2, before the barrier that
  // precedes their first reader.
  for (int t = 0; t < T; ++t) {
    const int S = t & 1;
    // slot 2t: A softmax of step t; B values of step t-1 and scores of step t
    if (!grp_b) {
      softmax(t);
    } else {
      if (t > 0) value_mfma(o, pb, lds_v(S ^ 1), voff0, voff1);
      scores(lds_k(S), s);
      ken = kebase[t];
    }
    ring_stress(t, 2);
    __builtin_amdgcn_s_waitcnt(0x0070);   // the copies of slot 2t-1 landed, LDS reads done
    asm volatile("s_barrier" ::: "memory");
    // slot 2t+1: A values of step t and scores of step t+1; B softmax of step t
    if (t + 2 <= Tm1) ring_k(t + 2, S);
    if (t + 1 <= Tm1) ring_v(t + 1, S ^ 1);
    if (!grp_b) {
      value_mfma(o, pb, lds_v(S), voff0, voff1);
      if (t + 1 < T) {
        scores(lds_k(S ^ 1), s);
        ken = kebase[t + 1];
      }
    } else {
      softmax(t);
    }
    ring_stress(t, 3);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): LDS reads done (the copies keep flying)
    asm volatile("s_barrier" ::: "memory");
  }
  // slot 2T: B values of step T-1
  if (grp_b) value_mfma(o, pb, lds_v(Tm1 & 1), voff0, voff1);

  const int q = q0 + r;
  store_out(o, l, out, vs + (size_t)bh * D, (size_t)bh * N + q, q < N, g);
}

// Compute units of the current device, read once per device (an immutable
// property); 256 if the query fails.
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

void launch_attention(const LaunchArgs& a, hipStream_t s) {
  const int BH = a.batch * a.heads;
  const int slots = 2 * device_cus();   // two workgroups of each attention kernel per CU
  const int tiles = a.n_pad / QT;
  const float tl = a.softmax_scale * LOG2E;
  if (a.mx) {
    auto kern = a.fuse_q ? attn_mx_kernel<true> : attn_mx_kernel<false>;
    kern<<<BH * tiles, 256, 0, s>>>(a.q_codes, (const uint8_t*)a.q_scales, (const uint16_t*)a.q, a.k_codes,
                                    (const uint8_t*)a.k_scales, a.v_codes, a.v_scales, (uint16_t*)a.o, a.seq_len,
                                    a.n_pad, tl, tiles, slots);
  } else if (a.fp4) {
    const int ktiles = a.n_pad / KSTEP, tiles4 = (a.n_pad + FP4_WAVES * QW - 1) / (FP4_WAVES * QW);
    auto kern = a.fuse_q ? attn_fp4_kernel<true> : attn_fp4_kernel<false>;
    kern<<<BH * tiles4, FP4_T, 0, s>>>(a.q_codes, a.q_scales, (const uint16_t*)a.q, a.k_expanded,
                                       (const int*)(a.k_expanded + (size_t)BH * ktiles * KXTILE), a.v_codes,
                                       a.v_scales, (uint16_t*)a.o, a.seq_len, a.n_pad, tl, tiles4);
  } else {
    auto kern = a.fuse_q ? attn_fp8_kernel<true> : attn_fp8_kernel<false>;
    kern<<<BH * tiles, 256, 0, s>>>(a.q_codes, a.q_scales, (const uint16_t*)a.q, a.k_codes, a.k_scales,
                                    a.v_codes, a.v_scales, (uint16_t*)a.o, a.seq_len, a.n_pad, a.block_q,
                                    a.q_scale_count, a.k_scale_count, tl, tiles, slots, a.vc_err);
  }
}

}  // namespace qsdpa
