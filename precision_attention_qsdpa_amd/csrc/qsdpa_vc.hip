// Selective correction of the FP8 path (VC-Attention-style): per (b,h) the
// k = ceil(rho N) query tokens whose own FP8 quantization error is largest
// are recomputed as unquantized softmax attention of the bf16 inputs, and
// their rows of O are overwritten.  The errors come from the FP8 attention
// kernel's prologue (vc_err).  Three kernels:
//   vc_select_kernel   per (b,h): the k largest errors, ties to the lower
//                      index, as ascending row indices (radix select on the
//                      fp64 bit patterns, which order like the values for
//                      errors >= 0);
//   vc_partial_kernel  per (b,h, 32 selected rows, key range): flash
//                      attention of the selected rows over the range, bf16
//                      MFMA with fp32 accumulation, fp32 softmax in base 2,
//                      P rounded to bf16 for the value product; writes the
//                      range's (max, sum, accumulators);
//   vc_combine_kernel  per (b,h, selected row): merges the ranges and writes
//                      the bf16 row of O.
#include "qsdpa_device.h"
#include "qsdpa_launch.h"

namespace qsdpa {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Selection.  grid = BH, block = 256.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void vc_select_kernel(const double* __restrict__ err, int32_t* __restrict__ sel,
                                                         int N, int n_pad, int count, int count_pad) {
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t* key = (const uint64_t*)(err + (size_t)bh * n_pad);
  __shared__ uint32_t hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  __shared__ int wsum[2][4];
  __shared__ int s_last;
  // the k-th largest key T, one byte per pass from the top; need = how many
  // keys equal to T are taken (the rest of the k are the keys above T)
  uint64_t prefix = 0, mask = 0;
  int need = count;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += 256) {
      const uint64_t u = key[i];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0, d = 255;
      for (; d > 0; --d) {
        if (above + (int)hist[d] >= need) break;
        above += (int)hist[d];
      }
      s_prefix = prefix | ((uint64_t)d << shift);
      s_need = need - above;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= (uint64_t)0xff << shift;
    __syncthreads();
  }
  // rows in ascending order: every key above T, and the first `need` keys
  // equal to T; positions from block-wide prefix counts, chunk by chunk
  int taken = 0, ties = 0;
  for (int base = 0; base < N; base += 256) {
    const int i = base + tid;
    const uint64_t u = i < N ? key[i] : 0;
    const bool gt = i < N && u > prefix, eq = i < N && u == prefix;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint64_t beq = __ballot(eq);
    const int eq_before_w = __popcll(beq & below);
    if (lane == 0) wsum[0][wave] = __popcll(beq);
    __syncthreads();
    int eq_before = ties + eq_before_w;
    for (int w = 0; w < wave; ++w) eq_before += wsum[0][w];
    const bool take = gt || (eq && eq_before < need);
    const uint64_t btk = __ballot(take);
    const int tk_before_w = __popcll(btk & below);
    if (lane == 0) wsum[1][wave] = __popcll(btk);
    __syncthreads();
    int pos = taken + tk_before_w;
    for (int w = 0; w < wave; ++w) pos += wsum[1][w];
    if (take) {
      sel[(size_t)bh * count_pad + pos] = i;
      if (pos == count - 1) s_last = i;
    }
    for (int w = 0; w < 4; ++w) {
      ties += wsum[0][w];
      taken += wsum[1][w];
    }
    __syncthreads();
  }
  // padding entries repeat the last selected row (their results are not used)
  for (int j = count + tid; j < count_pad; j += 256) sel[(size_t)bh * count_pad + j] = s_last;
}

// ---------------------------------------------------------------------------
// Recomputation over one key range.  grid = BH * (count_pad / 32) * chunks,
// block = 64 (one wave): 32 selected rows, keys [c * chunk_keys, ...).
// Scores S^T (32 keys x 32 rows) = K . Q^T on v_mfma_f32_32x32x16_bf16 (8
// over D = 128); lane l holds row l % 32 and keys 4g + (i % 4) + 8 (i / 4)
// (g = l / 32, i = 0..15) of each 32-key step.  The value product
// O^T (128 x 32) += V^T . P^T takes P's bf16 values straight from those
// registers: MFMA m (keys 16m .. 16m + 15) reads a lane's values 8m .. 8m + 7,
// which are keys 16m + 8 (e / 4) + 4g + (e % 4), e = 0..7, so each lane loads
// the matching 8 V values of its channel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void vc_partial_kernel(const uint16_t* __restrict__ qx, const uint16_t* __restrict__ kx,
                                                         const uint16_t* __restrict__ vx,
                                                         const int32_t* __restrict__ sel, float* __restrict__ part,
                                                         int N, int count_pad, int chunks, int chunk_keys,
                                                         float tau_log2e) {
  const int qgroups = count_pad / 32;
  const int c = blockIdx.x % chunks, rest = blockIdx.x / chunks;
  const int qg = rest % qgroups, bh = rest / qgroups;
  const int lane = threadIdx.x, g = lane >> 5, r = lane & 31;
  const int row = sel[(size_t)bh * count_pad + 32 * qg + r];
  const uint16_t* kb = kx + (size_t)bh * N * D;
  const uint16_t* vb = vx + (size_t)bh * N * D;
  // Q^T operand of chunk cc: channels 16cc + 8g .. + 7 of the row
  v8bf qop[8];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    const u32x4 w = *(const u32x4*)(qx + ((size_t)bh * N + row) * D + 16 * cc + 8 * g);
    qop[cc] = __builtin_bit_cast(v8bf, w);
  }
  v16f o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v16f{};
  float m = -INFINITY, lsum = 0.f;
  const int j_begin = c * chunk_keys, j_end = min(N, j_begin + chunk_keys);
  for (int j0 = j_begin; j0 < j_end; j0 += 32) {
    // scores
    v16f s = v16f{};
    const int kr = j0 + r;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (kr < j_end) w = *(const u32x4*)(kb + (size_t)kr * D + 16 * cc + 8 * g);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, w), qop[cc], s, 0, 0, 0);
    }
    // online softmax of the 16 keys this lane holds (base 2, fp32)
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = j0 + 4 * g + (i & 3) + 8 * (i >> 2);
      s[i] = key < j_end ? s[i] * tau_log2e : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
      ps += s[i];
    }
    lsum = alpha * lsum + ps;
    m = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    // values
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      v8bf pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[8 * mm + e];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + r;
        v8bf va;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = j0 + 16 * mm + 8 * (e >> 2) + 4 * g + (e & 3);
          const uint16_t bits = key < j_end ? vb[(size_t)key * D + d] : (uint16_t)0;
          va[e] = __builtin_bit_cast(__bf16, bits);
        }
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
      }
    }
  }
  // the pair (l, l ^ 32) holds the row's two halves of the sum
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  // O^T column r: channels 32 db + 4g + 8j + (0..3) in registers 4j .. 4j + 3
  float* dst = part + (((size_t)bh * count_pad + 32 * qg + r) * chunks + c) * VC_PART;
  if (g == 0) {
    dst[0] = m;
    dst[1] = lsum;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(float4*)(dst + 4 + 32 * db + 8 * j + 4 * g) =
          make_float4(o[db][4 * j], o[db][4 * j + 1], o[db][4 * j + 2], o[db][4 * j + 3]);
}

// ---------------------------------------------------------------------------
// Combine.  grid = BH * count, block = 128 (one channel each).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void vc_combine_kernel(const int32_t* __restrict__ sel, const float* __restrict__ part,
                                                          uint16_t* __restrict__ out, int N, int count, int count_pad,
                                                          int chunks) {
  const int bh = blockIdx.x / count, j = blockIdx.x % count, d = threadIdx.x;
  const float* src = part + ((size_t)bh * count_pad + j) * chunks * VC_PART;
  float M = -INFINITY;
  for (int c = 0; c < chunks; ++c) M = fmaxf(M, src[c * VC_PART]);
  float L = 0.f, acc = 0.f;
  for (int c = 0; c < chunks; ++c) {
    const float w = __builtin_amdgcn_exp2f(src[c * VC_PART] - M);
    L += w * src[c * VC_PART + 1];
    acc += w * src[c * VC_PART + 4 + d];
  }
  const int row = sel[(size_t)bh * count_pad + j];
  out[((size_t)bh * N + row) * D + d] = (uint16_t)f32_to_bf16(acc / L);
}

void launch_vc(const VcArgs& a, hipStream_t s) {
  const int BH = a.batch * a.heads;
  vc_select_kernel<<<BH, 256, 0, s>>>(a.err, a.sel, a.seq_len, a.n_pad, a.count, a.count_pad);
  vc_partial_kernel<<<BH * (a.count_pad / 32) * a.chunks, 64, 0, s>>>(
      (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.sel, a.part, a.seq_len, a.count_pad,
      a.chunks, a.chunk_keys, a.softmax_scale * LOG2E);
  vc_combine_kernel<<<BH * a.count, 128, 0, s>>>(a.sel, a.part, (uint16_t*)a.o, a.seq_len, a.count, a.count_pad,
                                                a.chunks);
}

}  // namespace qsdpa
