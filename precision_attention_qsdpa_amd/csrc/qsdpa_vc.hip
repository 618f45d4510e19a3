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
// Selection.  grid = BH, block = VC_SEL threads.  Thread tid owns a
// contiguous run of at most VC_RUN of the head's errors: runs in thread order
// are the errors in index order.  The runs are held in registers when
// N <= VC_SEL VC_RUN, and read from global memory in each pass for longer
// sequences.
// ---------------------------------------------------------------------------
constexpr int VC_SEL = 1024, VC_SEL_WAVES = VC_SEL / 64, VC_RUN = 16;

// Inclusive prefix sum of v over the VC_SEL threads of the block (tid order).
__device__ __forceinline__ int block_scan(int v, int* wtot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += wtot[w];
  __syncthreads();
  return v;
}

template <bool IN_REGS>
__global__ __launch_bounds__(VC_SEL) void vc_select_kernel(const double* __restrict__ err, int32_t* __restrict__ sel,
                                                         int N, int n_pad, int count, int count_pad) {
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t* gkey = (const uint64_t*)(err + (size_t)bh * n_pad);
  __shared__ int hist[256];
  __shared__ int wtot[VC_SEL_WAVES];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  __shared__ int wsum[VC_SEL_WAVES];
  __shared__ int s_last;
  __shared__ int s_done;
  const int per = (N + VC_SEL - 1) / VC_SEL, i0 = min(N, tid * per), n_run = min(N, i0 + per) - i0;
  uint64_t kr[IN_REGS ? VC_RUN : 1];
  if constexpr (IN_REGS) {
#pragma unroll
    for (int u = 0; u < VC_RUN; ++u) kr[u] = u < n_run ? gkey[i0 + u] : 0;
  }
  // f(u, key) for the run's keys in order
  auto visit = [&](auto f) {
    if constexpr (IN_REGS) {
#pragma unroll
      for (int u = 0; u < VC_RUN; ++u)
        if (u < n_run) f(u, kr[u]);
    } else {
      for (int u = 0; u < n_run; ++u) f(u, gkey[i0 + u]);
    }
  };
  // the k-th largest key T, one byte per pass from the top; need = how many
  // keys equal to T are taken (the rest of the k are the keys above T).  The
  // passes stop early once every key under the bytes found so far is taken:
  // T is then that prefix (mask covers its bytes), and the comparisons below
  // are on the masked keys.
  uint64_t prefix = 0, mask = 0;
  int need = count;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    // one atomic per run of equal digits: the first passes see one digit in
    // most keys (the errors share their top exponent bits)
    int cur = -1, cnt = 0;
    visit([&](int, uint64_t u) {
      if ((u & mask) == prefix) {
        const int dg = (int)((u >> shift) & 0xffu);
        if (dg != cur) {
          if (cnt) atomicAdd(&hist[cur], cnt);
          cur = dg;
          cnt = 0;
        }
        ++cnt;
      }
    });
    if (cnt) atomicAdd(&hist[cur], cnt);
    __syncthreads();
    // thread t < 256 takes digit 255 - t: cum = keys with this digit or a
    // larger one
    const int h = tid < 256 ? hist[255 - tid] : 0;
    const int cum = block_scan(h, wtot);
    const uint64_t b = __ballot(tid < 256 && cum >= need);
    if (lane == 0) wsum[wave] = b ? (int)__builtin_ctzll(b) : 64;
    __syncthreads();
    int first = VC_SEL;
    for (int w = VC_SEL_WAVES - 1; w >= 0; --w)
      if (wsum[w] < 64) first = 64 * w + wsum[w];
    if (tid == first) {
      s_prefix = prefix | ((uint64_t)(255 - tid) << shift);
      s_need = need - (cum - h);
      s_done = need - (cum - h) == h;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= (uint64_t)0xff << shift;
    if (s_done) break;   // uniform: every thread reads the same word after the barrier
  }
  // rows in ascending order: every key above T, and the first `need` keys
  // equal to T; each run's place from block-wide prefix counts
  int gt_c = 0, eq_c = 0;
  visit([&](int, uint64_t u) {
    gt_c += (u & mask) > prefix;
    eq_c += (u & mask) == prefix;
  });
  const int eq_before = block_scan(eq_c, wtot) - eq_c;
  const int take_c = gt_c + min(eq_c, max(0, need - eq_before));
  int pos = block_scan(take_c, wtot) - take_c;
  int eq_seen = eq_before;
  visit([&](int u, uint64_t x) {
    bool take = (x & mask) > prefix;
    if ((x & mask) == prefix) take = eq_seen++ < need;
    if (take) {
      sel[(size_t)bh * count_pad + pos] = i0 + u;
      if (pos == count - 1) s_last = i0 + u;
      ++pos;
    }
  });
  __syncthreads();
  // padding entries repeat the last selected row (their results are not used)
  for (int j = count + tid; j < count_pad; j += VC_SEL) sel[(size_t)bh * count_pad + j] = s_last;
}

// ---------------------------------------------------------------------------
// Recomputation over one key range.  grid = BH * qblocks * chunks, block =
// 64 * VC_WAVES: wave w takes the 32 selected rows of row group
// VC_WAVES * qb + w (if it exists) over keys [c * chunk_keys, ...), and the
// waves share each 32-key step's K tile and V^T tile, staged once in LDS.
// Scores S^T (32 keys x 32 rows) = K . Q^T on v_mfma_f32_32x32x16_bf16 (8
// over D = 128); lane l holds row l % 32 and keys 4g + (i % 4) + 8 (i / 4)
// (g = l / 32, i = 0..15) of the step.  The value product O^T (128 x 32) +=
// V^T . P^T takes P's bf16 values straight from those registers: MFMA mm
// (k = 16 mm .. 16 mm + 15) reads a lane's values 8 mm .. 8 mm + 7, so the V^T
// tile stores key j at k index kappa(j) = 16 (j / 16) + 8 g + e, the place
// of the register that holds it.
// ---------------------------------------------------------------------------
constexpr int VC_WAVES = 2;

__global__ __launch_bounds__(64 * VC_WAVES) void vc_partial_kernel(
    const uint16_t* __restrict__ qx, const uint16_t* __restrict__ kx, const uint16_t* __restrict__ vx,
    const int32_t* __restrict__ sel, float* __restrict__ part, int N, int count, int count_pad, int chunks,
    int chunk_keys, float tau_log2e) {
  const int qgroups = count_pad / 32, qblocks = (qgroups + VC_WAVES - 1) / VC_WAVES;
  const int c = blockIdx.x % chunks, rest = blockIdx.x / chunks;
  const int qb = rest % qblocks, bh = rest / qblocks;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int qg = VC_WAVES * qb + wave;
  const bool active = qg < qgroups;
  const uint16_t* kb = kx + (size_t)bh * N * D;
  const uint16_t* vb = vx + (size_t)bh * N * D;
  // two stages of the K tile (32 key rows of 256 B, 16-byte chunk c of row j
  // at c ^ (j & 15)) and the V^T tile (128 channel rows of 64 B in kappa
  // order, chunk c of row d at c ^ ((d >> 2) & 3))
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][32 * 256];
  __shared__ __attribute__((aligned(16))) uint8_t vt[2][D * 64];
  auto kt_off = [](int j, int ch) { return j * 256 + ((ch ^ (j & 15)) << 4); };
  auto vt_off = [](int d, int ch) { return d * 64 + ((ch ^ ((d >> 2) & 3)) << 4); };
  auto kappa = [](int j) { return 16 * (j >> 4) + 8 * ((j >> 2) & 1) + 4 * ((j >> 3) & 1) + (j & 3); };

  const int row = active ? sel[(size_t)bh * count_pad + 32 * qg + r] : 0;
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

  // a step's tiles are 512 sixteen-byte pieces each; thread tid loads pieces
  // tid + 64 VC_WAVES u (key p / 16, channels 8 (p % 16) .. + 7); keys at or
  // past the range end read as 0
  constexpr int PER = 512 / (64 * VC_WAVES);
  u32x4 kin[PER], vin[PER];
  auto load = [&](int j0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int p = tid + 64 * VC_WAVES * u, key = j0 + (p >> 4);
      kin[u] = vin[u] = u32x4{0u, 0u, 0u, 0u};
      if (key < j_end) {
        kin[u] = *(const u32x4*)(kb + (size_t)key * D + 8 * (p & 15));
        vin[u] = *(const u32x4*)(vb + (size_t)key * D + 8 * (p & 15));
      }
    }
  };
  auto store = [&](int S) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int p = tid + 64 * VC_WAVES * u, j = p >> 4, cg = p & 15;
      *(u32x4*)(kt[S] + kt_off(j, cg)) = kin[u];
      const int kp = kappa(j);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t x = (uint16_t)(vin[u][e >> 1] >> (16 * (e & 1)));
        *(uint16_t*)(vt[S] + vt_off(8 * cg + e, kp >> 3) + 2 * (kp & 7)) = x;
      }
    }
  };
  auto compute = [&](int j0, int S) {
    // scores: K operand of chunk cc is row r, channels 16cc + 8g .. + 7
    v16f s = v16f{};
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const u32x4 w = *(const u32x4*)(kt[S] + kt_off(r, 2 * cc + g));
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
    // values: A operand (channel 32 db + r, k 16 mm + 8 g .. + 7)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      v8bf pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[8 * mm + e];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x4 w = *(const u32x4*)(vt[S] + vt_off(32 * db + r, 2 * mm + g));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, w), pb, o[db], 0, 0, 0);
      }
    }
  };
  // the next step's tiles load while this one computes; the barrier after
  // each store hands the stage over (every wave has finished reading the
  // stage the next store refills)
  load(j_begin);
  store(0);
  __syncthreads();
  int S = 0;
  for (int j0 = j_begin; j0 < j_end; j0 += 32) {
    const bool more = j0 + 32 < j_end;
    if (more) load(j0 + 32);
    if (active) compute(j0, S);
    if (more) store(S ^ 1);
    __syncthreads();
    S ^= 1;
  }
  if (!active) return;
  // the pair (l, l ^ 32) holds the row's two halves of the sum
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  // padding rows (repeats of the last selected row) are not combined
  if (32 * qg + r >= count) return;
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
// Combine.  grid = BH * count, block = 64 (one wave per corrected row): lane
// l takes channels 8 (l % 16) .. + 7 of the ranges c = l / 16, l / 16 + 4,
// ..., merges them online (running max, rescaled sum and accumulators), and
// the four lanes of a channel group merge their results through shuffles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void vc_combine_kernel(const int32_t* __restrict__ sel, const float* __restrict__ part,
                                                         uint16_t* __restrict__ out, int N, int count, int count_pad,
                                                         int chunks) {
  const int bh = blockIdx.x / count, j = blockIdx.x % count, lane = threadIdx.x, cl = lane >> 4, cg = lane & 15;
  const float* src = part + ((size_t)bh * count_pad + j) * chunks * VC_PART;
  float M = -INFINITY, L = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int c = cl; c < chunks; c += 4) {
    const float* p = src + (size_t)c * VC_PART;
    const float mc = p[0], lc = p[1];
    const float4 x0 = *(const float4*)(p + 4 + 8 * cg), x1 = *(const float4*)(p + 8 + 8 * cg);
    const float Mn = fmaxf(M, mc);
    const float a = __builtin_amdgcn_exp2f(M - Mn), w = __builtin_amdgcn_exp2f(mc - Mn);
    L = a * L + w * lc;
    acc[0] = a * acc[0] + w * x0.x;
    acc[1] = a * acc[1] + w * x0.y;
    acc[2] = a * acc[2] + w * x0.z;
    acc[3] = a * acc[3] + w * x0.w;
    acc[4] = a * acc[4] + w * x1.x;
    acc[5] = a * acc[5] + w * x1.y;
    acc[6] = a * acc[6] + w * x1.z;
    acc[7] = a * acc[7] + w * x1.w;
    M = Mn;
  }
  // merge the four chunk lanes of each channel group (lanes cg, cg + 16, cg + 32, cg + 48)
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    const float Mo = __shfl_xor(M, o), Lo = __shfl_xor(L, o);
    const float Mn = fmaxf(M, Mo);
    // a lane with no ranges has M = -inf; exp2(-inf - Mn) = 0 drops it
    const float a = Mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    const float b = Mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mo - Mn);
    L = a * L + b * Lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = a * acc[e] + b * __shfl_xor(acc[e], o);
    M = Mn;
  }
  if (cl == 0) {
    const int row = sel[(size_t)bh * count_pad + j];
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = f32_to_bf16(acc[2 * e] / L) | (uint32_t)f32_to_bf16(acc[2 * e + 1] / L) << 16;
    *(u32x4*)(out + ((size_t)bh * N + row) * D + 8 * cg) = w;
  }
}

void launch_vc(const VcArgs& a, hipStream_t s) {
  const int BH = a.batch * a.heads;
  auto select = a.seq_len <= VC_SEL * VC_RUN ? vc_select_kernel<true> : vc_select_kernel<false>;
  select<<<BH, VC_SEL, 0, s>>>(a.err, a.sel, a.seq_len, a.n_pad, a.count, a.count_pad);
  const int qblocks = (a.count_pad / 32 + VC_WAVES - 1) / VC_WAVES;
  vc_partial_kernel<<<BH * qblocks * a.chunks, 64 * VC_WAVES, 0, s>>>(
      (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.sel, a.part, a.seq_len, a.count,
      a.count_pad, a.chunks, a.chunk_keys, a.softmax_scale * LOG2E);
  vc_combine_kernel<<<BH * a.count, 64, 0, s>>>(a.sel, a.part, (uint16_t*)a.o, a.seq_len, a.count, a.count_pad,
                                               a.chunks);
}

}  // namespace qsdpa
