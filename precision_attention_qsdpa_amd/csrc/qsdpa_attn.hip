// Fused flash-style attention over the quantized workspace.
//
// Work split: one workgroup = 4 waves = 128 consecutive queries of one (b,h);
// each wave owns 32 queries and walks all keys in steps of 64, in ascending
// order (the online-softmax step of the method).  Two workgroups share a CU,
// so each SIMD runs two waves whose MFMA and softmax phases interleave.
//
// Per 64-key step a wave computes
//   S^T (64 keys x 32 queries) = K_tile . Q^T      (MFMA, keys on rows)
// so that each lane owns one query column: the row max, the exponentials and
// the row sum stay in-lane, with one exchange between lanes l and l^32 for
// the max.  The probabilities, quantized to FP8 as E4M3(448 p), are packed
// straight from the S^T accumulator into the B operand of
//   O^T (128 channels x 32 queries) += V_tile^T . P^T   (FP8 MFMA)
// The accumulator holds its 16 keys per lane in a fixed order; the V tiles
// are stored by the quantize step in that same key order, so no shuffle is
// needed.  K and V^T tiles (8 KB each) are double-buffered in LDS with a
// 16-byte-chunk XOR swizzle; the next tile's global loads are in flight
// while the current one is consumed.
//
// Numerics: scores are exact integer-valued FP8 dot products accumulated in
// fp32 by the MFMA; one per-step constant c = tau*log2(e)*sQ*sK turns them
// into base-2 logits; p*448 = exp2(s*c - m + log2 448); the running max m is
// taken over the exact per-step maxima; the rescale exp2(m_old - m_new) is
// skipped when no lane's maximum moved (then it is exactly 1).
#include "qsdpa_device.h"
#include "qsdpa_launch.h"

namespace qsdpa {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int WAVES = 4;
constexpr int QW = 32;              // queries per wave
constexpr int QT = QW * WAVES;      // queries per workgroup
constexpr int KTILE = KSTEP * D;    // bytes of an FP8 K tile / V^T tile

// LDS byte offset of 16-byte chunk c of row `row` in an FP8 K tile (128 B rows).
__device__ __forceinline__ int k_off(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }
// ... of an f16 K tile (256 B rows, 16 chunks).
__device__ __forceinline__ int kh_off(int row, int c) { return row * 256 + ((c ^ (row & 7)) << 4); }
// ... of a V^T tile (64 B channel rows, 4 chunks).
__device__ __forceinline__ int v_off(int d, int c) { return d * 64 + ((c ^ ((d >> 1) & 3)) << 4); }

__device__ __forceinline__ v8i lds_v8i(const uint8_t* p0, const uint8_t* p1) {
  const u32x4 a = *(const u32x4*)p0, b = *(const u32x4*)p1;
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
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
    for (int h = 0; h < 2; ++h) {
      const u32x4 a = *(const u32x4*)(qrow + 64 * h + 32 * g);
      const u32x4 b = *(const u32x4*)(qrow + 64 * h + 32 * g + 16);
      qb8[h][0] = a[0]; qb8[h][1] = a[1]; qb8[h][2] = a[2]; qb8[h][3] = a[3];
      qb8[h][4] = b[0]; qb8[h][5] = b[1]; qb8[h][6] = b[2]; qb8[h][7] = b[3];
    }
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

  // ---- tile staging: global -> registers -> LDS
  u32x4 kreg[2], vreg[2];
  uint32_t kcode[2][2];
  float kscl[2];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = tid + 256 * i;
      vreg[i] = *(const u32x4*)(vbase + (size_t)t * KTILE + ci * 16);
      if constexpr (!FP4) {
        kreg[i] = *(const u32x4*)(kbase + (size_t)t * KTILE + ci * 16);
      } else {
        const int key = ci >> 3, grp = ci & 7;
        const u32x2 w = *(const u32x2*)(kbase + ((size_t)t * KSTEP + key) * 64 + grp * 8);
        kcode[i][0] = w[0];
        kcode[i][1] = w[1];
        kscl[i] = ksc[((size_t)t * KSTEP + key) * 8 + grp];
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = tid + 256 * i;
      *(u32x4*)(lds_v[buf] + v_off(ci >> 2, ci & 3)) = vreg[i];
      if constexpr (!FP4) {
        *(u32x4*)(lds_k[buf] + k_off(ci >> 3, ci & 7)) = kreg[i];
      } else {
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
          *(v8h*)(lds_k[buf] + kh_off(key, 2 * grp + half)) = hv;
          *(v8h*)(lds_k[buf] + 2 * KTILE + kh_off(key, 2 * grp + half)) = lv;
        }
      }
    }
  };

  v16f o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v16f{};
  float m = -INFINITY, l = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    if (t + 1 < T) load_tile(t + 1);

    // ---- S^T = K . Q^T for the two 32-key blocks of the step
    v16f s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = v16f{};
      const int row = kb * 32 + r;
      if constexpr (!FP4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v8i a = lds_v8i(lds_k[buf] + k_off(row, 4 * h + 2 * g), lds_k[buf] + k_off(row, 4 * h + 2 * g + 1));
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qb8[h], s[kb], 0, 0, 0, 127, 0, 127);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const v8h ah = *(const v8h*)(lds_k[buf] + kh_off(row, 2 * c + g));
          const v8h al = *(const v8h*)(lds_k[buf] + 2 * KTILE + kh_off(row, 2 * c + g));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qhi[c], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qhi[c], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qlo[c], s[kb], 0, 0, 0);
        }
      }
    }

    // ---- online softmax (base 2), lane = one query, 32 of the step's keys
    const float c = FP4 ? cscale : cscale * ksc[t];
    float m_new;
    float p[32];
    const bool tail = (t + 1) * KSTEP > N;
    if (!tail) {
      float mx = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_new = fmaxf(m, c * mx);
      const float b = LOG2_448 - m_new;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) p[kb * 16 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, b));
    } else {
      float sc[32];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t * KSTEP + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          sc[kb * 16 + i] = key < N ? s[kb][i] * c : -INFINITY;
          mx = fmaxf(mx, sc[kb * 16 + i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_new = fmaxf(m, mx);
      const float b = LOG2_448 - m_new;
#pragma unroll
      for (int i = 0; i < 32; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] + b);
    }
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) psum += p[i];
    const bool moved = m_new != m;
    const float alpha = moved ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
    l = alpha * l + psum;
    if (__any(moved)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    m = m_new;

    // ---- P -> FP8, packed in the B-operand order (slot j = kb*16 + i)
    v8i pb;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      int x = cvt_e4m3x2<false>(p[4 * w], p[4 * w + 1], 0);
      x = cvt_e4m3x2<true>(p[4 * w + 2], p[4 * w + 3], x);
      pb[w] = x;
    }

    // ---- O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + r;
      const v8i a = lds_v8i(lds_v[buf] + v_off(d, 2 * g), lds_v[buf] + v_off(d, 2 * g + 1));
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, o[db], 0, 0, 0, 127, 0, 127);
    }

    if (t + 1 < T) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc * sV / (448 l), bf16, 4 channels (8 bytes) per store
  const float ltot = l + __shfl_xor(l, 32);
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
