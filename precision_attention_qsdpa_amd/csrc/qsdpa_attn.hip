// Fused flash-style attention over the quantized workspace.
//
// Work split: one workgroup = 4 waves = 128 consecutive queries of one (b,h);
// each wave owns 32 queries and walks all keys in steps of 64, in ascending
// order (the online-softmax step of the method).  Two workgroups share a CU,
// so each SIMD runs two waves whose MFMA and softmax phases interleave.
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
// Pipeline: the score MFMAs of step t+1 are issued before the softmax of
// step t, so the matrix cores work while the VALU runs the softmax.  K tiles
// are therefore staged in LDS one step ahead of V tiles: during step t the
// LDS holds K(t+1) and V(t) while the registers bring in K(t+2) and V(t+1)
// (two LDS buffers each, one barrier per step).  Tiles are 8 KB with a
// 16-byte-chunk XOR swizzle that keeps both the 128-bit stores and the
// 128-bit operand reads free of bank conflicts.
//
// Numerics: scores are exact integer-valued FP8 dot products accumulated in
// fp32 by the MFMA; one per-step constant c = tau*log2(e)*sQ*sK turns them
// into base-2 logits; p*448 = exp2(s*c - m + log2 448); the running max m is
// taken over the exact per-step maxima; the rescale exp2(m_old - m_new) is
// skipped when no lane's maximum moved (then it is exactly 1).
#include <type_traits>

#include "qsdpa_device.h"
#include "qsdpa_launch.h"

namespace qsdpa {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int WAVES = 4;
constexpr int QW = 32;              // queries per wave
constexpr int QT = QW * WAVES;      // queries per workgroup
constexpr int KTILE = KSTEP * D;    // bytes of an FP8 K tile / V^T tile

// LDS byte offset of 16-byte chunk c of row `row` in an FP8 K tile (128-B rows).
__device__ __forceinline__ int k_off(int row, int c) { return row * 128 + ((c ^ ((row ^ (row >> 3)) & 7)) << 4); }
// ... of an f16 K tile (256-B rows, 16 chunks).
__device__ __forceinline__ int kh_off(int row, int c) { return row * 256 + ((c ^ (row & 15)) << 4); }
// ... of a V^T tile (64-B channel rows, 4 chunks).
__device__ __forceinline__ int v_off(int d, int c) { return d * 64 + ((c ^ (((d >> 1) ^ (d >> 3)) & 3)) << 4); }

__device__ __forceinline__ v8i lds_v8i(const uint8_t* p0, const uint8_t* p1) {
  const u32x4 a = *(const u32x4*)p0, b = *(const u32x4*)p1;
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// max / sum of a value over the lane pair (l, l^32): one v_permlane32_swap
// exchanges the two halves of the wave.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e ? (float)((2u + m) << (e - 1u)) * 0.5f : (float)m * 0.5f;
  return (c & 8u) ? -mag : mag;
}

// Maps the hardware workgroup id so that each XCD (ids are dealt round-robin
// over the 8 XCDs) receives one contiguous range of logical workgroups:
// consecutive query tiles of a head then share one L2.
__device__ __forceinline__ int xcd_remap(int hw, int n) {
  const int xcd = hw & 7, slot = hw >> 3;
  const int q = n >> 3, rem = n & 7;
  return xcd * q + min(xcd, rem) + slot;
}

template <bool FP4>
__global__ __launch_bounds__(256, FP4 ? 1 : 2) void attn_kernel(
    const uint8_t* __restrict__ qc, const float* __restrict__ qs, const uint8_t* __restrict__ kc,
    const float* __restrict__ ks, const uint8_t* __restrict__ vc, const float* __restrict__ vs,
    uint16_t* __restrict__ out, int N, int n_pad, int block_q, int q_scale_count,
    int k_scale_count, float tau_log2e, int tiles_per_bh) {
  // K tile in LDS: FP8 codes, or in FP4 mode the dequantized values as an
  // f16 pair hi + lo (hi = f16(x), lo = f16(x - hi)), which carries x to about
  // 2^-22 relative so the scores keep fp32-level accuracy.
  constexpr int KBYTES = FP4 ? 4 * KTILE : KTILE;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][KTILE];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / tiles_per_bh, tile = wg - bh * tiles_per_bh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int q0 = tile * QT + wave * QW;
  const int T = (N + KSTEP - 1) / KSTEP;

  // ---- Q operand (B side of S^T), held in registers for the whole kernel.
  v8i qb8[2];
  v8h qhi[8], qlo[8];
  float cscale;   // base-2 logit per unit of the raw MFMA score
  if constexpr (!FP4) {
    const uint8_t* qrow = qc + ((size_t)bh * n_pad + q0 + r) * D;
#pragma unroll
    for (int h = 0; h < 2; ++h) qb8[h] = lds_v8i(qrow + 64 * h + 32 * g, qrow + 64 * h + 32 * g + 16);
    cscale = tau_log2e * qs[(size_t)bh * q_scale_count + q0 / block_q];
  } else {
    const size_t qrow = (size_t)bh * n_pad + q0 + r;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t w = *(const uint32_t*)(qc + qrow * 64 + 8 * c + 4 * g);
      const float s = qs[qrow * 8 + c];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e2m1_value((w >> (4 * e)) & 15u) * s;
        qhi[c][e] = (_Float16)x;
        qlo[c][e] = (_Float16)(x - (float)qhi[c][e]);
      }
    }
    cscale = tau_log2e;
  }

  const uint8_t* kbase = FP4 ? kc + (size_t)bh * n_pad * 64 : kc + (size_t)bh * n_pad * D;
  const float* ksc = FP4 ? ks + (size_t)bh * n_pad * 8 : ks + (size_t)bh * k_scale_count;
  const uint8_t* vbase = vc + (size_t)bh * n_pad * D;

  // ---- per-lane LDS offsets, computed once
  // K operand chunks of this lane: row kb*32 + r, chunks 4h + 2g + i.
  int koff[2][2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 2; ++i) koff[kb][h][i] = k_off(kb * 32 + r, 4 * h + 2 * g + i);
  // V operand chunks: channel row db*32 + r (the swizzle does not depend on db).
  const int voff0 = v_off(r, 2 * g), voff1 = v_off(r, 2 * g + 1);
  // staging stores of this thread: chunks tid and tid + 256
  const int kst0 = k_off(tid >> 3, tid & 7), kst1 = k_off((tid + 256) >> 3, tid & 7);
  const int vst0 = v_off(tid >> 2, tid & 3), vst1 = v_off((tid + 256) >> 2, tid & 3);

  // ---- tile staging: global -> registers -> LDS
  u32x4 kreg[2], vreg[2];
  uint32_t kcode[2][2];
  float kscl[2];
  auto load_k = [&](int t) {
    if constexpr (!FP4) {
      const uint8_t* tp = kbase + (size_t)t * KTILE;
      kreg[0] = *(const u32x4*)(tp + tid * 16);
      kreg[1] = *(const u32x4*)(tp + tid * 16 + 4096);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ci = tid + 256 * i;
        const int key = ci >> 3, grp = ci & 7;
        const u32x2 w = *(const u32x2*)(kbase + ((size_t)t * KSTEP + key) * 64 + grp * 8);
        kcode[i][0] = w[0];
        kcode[i][1] = w[1];
        kscl[i] = ksc[((size_t)t * KSTEP + key) * 8 + grp];
      }
    }
  };
  auto load_v = [&](int t) {
    const uint8_t* tp = vbase + (size_t)t * KTILE;
    vreg[0] = *(const u32x4*)(tp + tid * 16);
    vreg[1] = *(const u32x4*)(tp + tid * 16 + 4096);
  };
  auto store_k = [&](uint8_t* kbuf) {
    if constexpr (!FP4) {
      *(u32x4*)(kbuf + kst0) = kreg[0];
      *(u32x4*)(kbuf + kst1) = kreg[1];
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ci = tid + 256 * i;
        const int key = ci >> 3, grp = ci & 7;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          v8h hv, lv;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = e2m1_value((kcode[i][half] >> (4 * e)) & 15u) * kscl[i];
            hv[e] = (_Float16)x;
            lv[e] = (_Float16)(x - (float)hv[e]);
          }
          *(v8h*)(kbuf + kh_off(key, 2 * grp + half)) = hv;
          *(v8h*)(kbuf + 2 * KTILE + kh_off(key, 2 * grp + half)) = lv;
        }
      }
    }
  };
  auto store_v = [&](uint8_t* vbuf) {
    *(u32x4*)(vbuf + vst0) = vreg[0];
    *(u32x4*)(vbuf + vst1) = vreg[1];
  };

  // ---- S^T = K . Q^T for the two 32-key blocks of a step, from a K buffer
  auto scores = [&](const uint8_t* kbuf, v16f* s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = v16f{};
      if constexpr (!FP4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v8i a = lds_v8i(kbuf + koff[kb][h][0], kbuf + koff[kb][h][1]);
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qb8[h], s[kb], 0, 0, 0, 127, 0, 127);
        }
      } else {
        const int row = kb * 32 + r;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const v8h ah = *(const v8h*)(kbuf + kh_off(row, 2 * c + g));
          const v8h al = *(const v8h*)(kbuf + 2 * KTILE + kh_off(row, 2 * c + g));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qhi[c], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qhi[c], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qlo[c], s[kb], 0, 0, 0);
        }
      }
    }
  };

  v16f o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v16f{};
  float m = -INFINITY, l = 0.f;

  // ---- online softmax of one step on scores s (step t): returns the packed
  // FP8 weights and the rescale factor; updates m and l.
  auto softmax = [&](int t, v16f* s, auto full_t, float& alpha) -> v8i {
    constexpr bool full = decltype(full_t)::value;
    const float c = FP4 ? cscale : cscale * ksc[t];
    float m_new;
    if constexpr (full) {
      // max over the 32 raw scores of this lane (two independent chains)
      float m0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
      float m1 = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) {
        m0 = fmaxf(fmaxf(m0, s[0][i]), s[0][i + 1]);
        m1 = fmaxf(fmaxf(m1, s[1][i]), s[1][i + 1]);
      }
      const float mx = pair_max(fmaxf(fmaxf(m0, s[0][15]), fmaxf(m1, s[1][15])));
      m_new = fmaxf(m, c * mx);
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
          const int key = t * KSTEP + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          s[kb][i] = key < N ? s[kb][i] * c : -INFINITY;
          mx = fmaxf(mx, s[kb][i]);
        }
      m_new = fmaxf(m, pair_max(mx));
      const float b = LOG2_448 - m_new;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(s[kb][i] + b);
    }
    // P -> FP8, packed in the B-operand order (slot j = kb*16 + i)
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
    m = m_new;
    return pb;
  };
  // O^T *= alpha, skipped when alpha is exactly 1 in every lane
  auto rescale = [&](float alpha) {
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
  };
  // O^T += V^T . P^T for the V tile in vbuf
  auto pv = [&](const v8i& pb, const uint8_t* vbuf) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const v8i a = lds_v8i(vbuf + db * 2048 + voff0, vbuf + db * 2048 + voff1);
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o[db], 0, 0, 0, 127, 0, 127);
    }
  };

  // ---- Pipeline.  Step t issues the score MFMAs of step t+1 and the value
  // MFMAs of step t-1 while the VALU runs the softmax of step t, so the
  // matrix cores and the VALU work side by side in one instruction stream.
  // During step t the LDS holds K(t+1) and V(t-1); the registers bring in
  // K(t+2) and V(t), stored at the end of the step (two buffers each).
  // Order on O^T: step t first rescales by alpha(t-1), then accumulates
  // PV(t-1), which is the online-softmax recursion delayed by one step.
  load_k(0);
  store_k(lds_k[0]);
  if (T > 1) {
    load_k(1);
    store_k(lds_k[1]);
  }
  // V buffer 1 is read by the (zero-weight) value product of step -1
  *(u32x4*)(lds_v[1] + vst0) = u32x4{0u, 0u, 0u, 0u};
  *(u32x4*)(lds_v[1] + vst1) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  v16f sa[2], sb[2];
  scores(lds_k[0], sa);
  v8i pb_prev = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  float alpha_prev = 1.f;

  // steps 0 .. T-2 are full 64-key steps (only the last step can be short)
  auto step = [&](int t, v16f* s_cur, v16f* s_next, auto par) {
    constexpr int P = decltype(par)::value;   // t & 1
    rescale(alpha_prev);
    load_k(min(t + 2, T - 1));
    load_v(t);
    scores(lds_k[P ^ 1], s_next);
    pv(pb_prev, lds_v[P ^ 1]);
    pb_prev = softmax(t, s_cur, std::true_type{}, alpha_prev);
    if constexpr (!FP4) {
      // interleave: each MFMA followed by a slice of the softmax VALU work
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 16, 0);
      }
    }
    store_k(lds_k[P]);
    store_v(lds_v[P]);
    __syncthreads();
  };
  int t = 0;
  for (; t + 2 < T; t += 2) {
    step(t, sa, sb, std::integral_constant<int, 0>{});
    step(t + 1, sb, sa, std::integral_constant<int, 1>{});
  }
  // last one or two steps
  auto last = [&](int tl, v16f* s_cur, auto par) {
    constexpr int P = decltype(par)::value;
    rescale(alpha_prev);
    load_v(tl);
    pv(pb_prev, lds_v[P ^ 1]);
    float alpha;
    const v8i pb = (tl + 1) * KSTEP <= N ? softmax(tl, s_cur, std::true_type{}, alpha)
                                         : softmax(tl, s_cur, std::false_type{}, alpha);
    store_v(lds_v[P]);
    __syncthreads();
    rescale(alpha);
    pv(pb, lds_v[P]);
  };
  if (t + 1 < T) {           // two steps left: t (full) and t+1 (last)
    step(t, sa, sb, std::integral_constant<int, 0>{});
    last(t + 1, sb, std::integral_constant<int, 1>{});
  } else {                   // one step left: t (last)
    last(t, sa, std::integral_constant<int, 0>{});
  }

  // ---- epilogue: O = acc * sV / (448 l), bf16, 4 channels (8 bytes) per store
  const float ltot = pair_sum(l);
  const float inv_l = 1.f / ltot;
  const int q = q0 + r;
  if (q < N) {
    uint16_t* orow = out + ((size_t)bh * N + q) * D;
    const float* vsc = vs + (size_t)bh * D;
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
}

void launch_attention(const LaunchArgs& a, hipStream_t s) {
  const int BH = a.batch * a.heads;
  const int tiles = a.n_pad / QT;
  const float tl = a.softmax_scale * LOG2E;
  if (a.fp4) {
    attn_kernel<true><<<BH * tiles, 256, 0, s>>>(a.q_codes, a.q_scales, a.k_codes, a.k_scales, a.v_codes,
                                                  a.v_scales, (uint16_t*)a.o, a.seq_len, a.n_pad, a.block_q,
                                                  a.q_scale_count, a.k_scale_count, tl, tiles);
  } else {
    attn_kernel<false><<<BH * tiles, 256, 0, s>>>(a.q_codes, a.q_scales, a.k_codes, a.k_scales, a.v_codes,
                                                   a.v_scales, (uint16_t*)a.o, a.seq_len, a.n_pad, a.block_q,
                                                   a.q_scale_count, a.k_scale_count, tl, tiles);
  }
}

}  // namespace qsdpa
