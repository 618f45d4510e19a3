// Statistics and quantize kernels: channel mean of K and max |V| (fp64 /
// fp32), K smoothing, per-block FP8, per-16-channel FP4 or per-32-channel
// MXFP4 (E8M0 scale) codes of Q and K, per-channel FP8 codes of V written as
// key-tiles in the order the attention kernel's value product consumes them,
// and in FP4 mode K expanded once per head into the attention kernel's f16
// hi and E4M3 correction tiles.
//
// All of these kernels are bound by HBM traffic; they read bf16 rows with
// 16-byte loads, 16 threads per 256-byte token row.
//
// Every fp32 operation that decides a code (K - mu, F / amax, amax / F,
// x * inv) is a single correctly rounded IEEE operation, so the codes and
// scales are bit-identical to a plain CPU evaluation of the same steps.
#include "qsdpa_device.h"
#include "qsdpa_launch.h"

#pragma clang fp contract(off)

namespace qsdpa {

// The passes that re-read K and V after the statistics pass (which walks the
// (b,h) pairs in order) take them last-first: the pairs the statistics pass
// read last are then re-read first, while they are still in the caches
// (2048x2048: the quantize pass 5 % faster; Kontext's K and V fit either way).
__device__ __forceinline__ int last_first(int y) { return (int)gridDim.y - 1 - y; }

// ---------------------------------------------------------------------------
// Channel statistics, pass 1: per (b,h, token range of STATS_ROWS tokens)
// partial fp64 sums of K, fp32 maxima of |V|, and the range of K's
// magnitudes: the largest |K| and the smallest nonzero |K|, as bf16 bits
// (max in the high half of a word, min - 1 in the low half; 0xffff when the
// range has no nonzero K).  The magnitudes are tracked two channels at a
// time with packed 16-bit integer operations: bf16 magnitudes order like
// their bit patterns, and min - 1 wraps a zero to 0xffff.
// grid = (splits, BH), block = 256: thread = (row lane 0..15, 8 channels).
// ---------------------------------------------------------------------------
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void stats_partial_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int splits,
    double* __restrict__ psum, float* __restrict__ pmax, uint32_t* __restrict__ prange) {
  const int split = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, cg = tid & 15, rl = tid >> 4;
  const size_t base = (size_t)bh * N * D + cg * 8;
  const int n0 = split * STATS_ROWS, n1 = min(N, n0 + STATS_ROWS);
  double s[8];
  float m[8];
  u16x2 kmx[4], kmn[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) { s[j] = 0.0; m[j] = 0.f; }
#pragma unroll
  for (int j = 0; j < 4; ++j) { kmx[j] = u16x2{0, 0}; kmn[j] = u16x2{0xffff, 0xffff}; }
  for (int n = n0 + rl; n < n1; n += 16) {
    const u32x4 kk = *(const u32x4*)(k + base + (size_t)n * D);
    const u32x4 vv = *(const u32x4*)(v + base + (size_t)n * D);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[2 * j] += (double)bf16_lo(kk[j]);
      s[2 * j + 1] += (double)bf16_hi(kk[j]);
      m[2 * j] = fmaxf(m[2 * j], fabsf(bf16_lo(vv[j])));
      m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf(bf16_hi(vv[j])));
      const u16x2 mag = __builtin_bit_cast(u16x2, kk[j] & 0x7fff7fffu);
      kmx[j] = __builtin_elementwise_max(kmx[j], mag);
      kmn[j] = __builtin_elementwise_min(kmn[j], mag - u16x2{1, 1});
    }
  }
  __shared__ double lsum[16][D];
  __shared__ float lmax[16][D];
  __shared__ uint32_t lrange[16][D];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lsum[rl][cg * 8 + j] = s[j];
    lmax[rl][cg * 8 + j] = m[j];
    lrange[rl][cg * 8 + j] = (uint32_t)kmx[j >> 1][j & 1] << 16 | kmn[j >> 1][j & 1];
  }
  __syncthreads();
  if (tid < D) {
    double t = 0.0;
    float mm = 0.f;
    uint32_t hi = 0, lo = 0xffff;
    for (int r = 0; r < 16; ++r) {
      t += lsum[r][tid];
      mm = fmaxf(mm, lmax[r][tid]);
      hi = max(hi, lrange[r][tid] >> 16);
      lo = min(lo, lrange[r][tid] & 0xffffu);
    }
    const size_t at = ((size_t)bh * splits + split) * D + tid;
    psum[at] = t;
    pmax[at] = mm;
    prange[at] = hi << 16 | lo;
  }
}

// The exact sum of one channel of K over the tokens of a (b,h), rounded once
// to fp64 (nearest, ties to even), for channels whose values span too many
// binades for fp64 partial sums to be exact.  Every bf16 value is an integer
// M < 256 times 2^(p - 133), p = max(exponent field, 1) - 1 in 0..253, so the
// sum is an integer times 2^-133 below 2^(254 + 8 + 22): each thread adds
// +-M << (p % 32) into the int64 digit p / 32 (8 digits of 32 bits with
// headroom), the block adds the digits, and one thread carries them into
// 32-bit limbs of a two's complement integer and rounds its magnitude's top
// 53 bits with the bits below.  N <= 2^22 keeps every digit sum below 2^62.
// Called by all threads of a 128-thread block; returns the sum to all.
__device__ double exact_channel_sum(const uint16_t* __restrict__ kcol, int N, long long (*part)[128],
                                    long long* tot, uint32_t* limb, double* result) {
  const int tid = threadIdx.x;
  long long acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0;
  for (int n = tid; n < N; n += 128) {
    const uint32_t h = kcol[(size_t)n * D];
    const uint32_t f = (h >> 7) & 0xffu, man = h & 0x7fu;
    const long long M = (long long)(f ? (man | 0x80u) : man);
    const int p = (int)max(f, 1u) - 1;
    const long long t = M << (p & 31);
    const long long st = (h & 0x8000u) ? -t : t;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += (p >> 5) == j ? st : 0;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[j][tid] = acc[j];
  __syncthreads();
  if (tid < 8) {
    long long x = 0;
    for (int i = 0; i < 128; ++i) x += part[tid][i];
    tot[tid] = x;
  }
  __syncthreads();
  if (tid == 0) {
    // carry into 10 limbs of 32 bits (two's complement), then the magnitude
    long long c = 0;
    for (int j = 0; j < 8; ++j) {
      const long long x = tot[j] + c;
      limb[j] = (uint32_t)x;
      c = x >> 32;   // arithmetic: floor division by 2^32
    }
    limb[8] = (uint32_t)c;
    limb[9] = (uint32_t)(c >> 32);
    const bool neg = (int32_t)limb[9] < 0;
    if (neg) {
      uint32_t carry = 1;
      for (int j = 0; j < 10; ++j) {
        const uint64_t x = (uint64_t)(~limb[j]) + carry;
        limb[j] = (uint32_t)x;
        carry = (uint32_t)(x >> 32);
      }
    }
    auto bit = [&](int i) -> uint64_t { return (limb[i >> 5] >> (i & 31)) & 1u; };
    int top = -1;
    for (int i = 319; i >= 0 && top < 0; --i)
      if (bit(i)) top = i;
    double r = 0.0;
    if (top >= 0) {
      const int lo = max(top - 52, 0);
      uint64_t mant = 0;
      for (int i = top; i >= lo; --i) mant = mant << 1 | bit(i);
      if (lo > 0) {
        uint64_t sticky = 0;
        for (int i = 0; i < lo - 1; ++i) sticky |= bit(i);
        if (bit(lo - 1) && (sticky || (mant & 1u))) ++mant;   // at most 2^53: exact in fp64
      }
      r = ldexp((double)mant, lo - 133);
      if (neg) r = -r;
    }
    *result = r;
  }
  __syncthreads();
  const double r = *result;
  __syncthreads();   // the shared buffers are reused by the next call
  return r;
}

// Pass 2: per (b,h), combine the ranges: mu = fp32(fp64 sum / N),
// vmax = max, sV = fp32(vmax / 448).  grid = BH, block = 128 (one channel each).
// The partial sums are fetched eight at a time (independent loads) and added
// in range order.  That sum is exact, in any order, when every value is a
// multiple of the smallest nonzero one's unit in the last place and N times
// the largest stays within 53 bits of it: with exponent fields e_hi of the
// largest and e_lo (at least 1) of the smallest, e_hi - e_lo + ceil(log2 N)
// <= 45.  A channel beyond that (and with a finite sum) is summed again by
// exact_channel_sum from K itself.
__global__ __launch_bounds__(128) void stats_final_kernel(
    const double* __restrict__ psum, const float* __restrict__ pmax, const uint32_t* __restrict__ prange,
    const uint16_t* __restrict__ k, int N, int splits, float* __restrict__ mu, float* __restrict__ vamax,
    float* __restrict__ vscale) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const double* ps = psum + (size_t)bh * splits * D + d;
  const float* pm = pmax + (size_t)bh * splits * D + d;
  const uint32_t* pr = prange + (size_t)bh * splits * D + d;
  double t = 0.0;
  float mm = 0.f;
  uint32_t hi = 0, lo = 0xffff;
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
    double x[8];
    float y[8];
    uint32_t z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { x[i] = ps[(s + i) * D]; y[i] = pm[(s + i) * D]; z[i] = pr[(s + i) * D]; }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      t += x[i];
      mm = fmaxf(mm, y[i]);
      hi = max(hi, z[i] >> 16);
      lo = min(lo, z[i] & 0xffffu);
    }
  }
  for (; s < splits; ++s) {
    t += ps[s * D];
    mm = fmaxf(mm, pm[s * D]);
    hi = max(hi, pr[s * D] >> 16);
    lo = min(lo, pr[s * D] & 0xffffu);
  }
  const int log2n = N > 1 ? 32 - __clz(N - 1) : 0;
  const int e_hi = (int)(hi >> 7), e_lo = max((int)((lo + 1) >> 7), 1);
  const bool inexact = lo != 0xffffu && e_hi - e_lo + log2n > 45 && isfinite(t);
  __shared__ int redo[D];
  redo[d] = inexact;
  if (__syncthreads_or(inexact)) {
    __shared__ long long part[8][128];
    __shared__ long long tot[8];
    __shared__ uint32_t limb[10];
    __shared__ double result;
    for (int c = 0; c < D; ++c) {
      if (!redo[c]) continue;   // uniform: every thread reads the same word
      const double x = exact_channel_sum(k + (size_t)bh * N * D + c, N, part, tot, limb, &result);
      if (d == c) t = x;
    }
  }
  mu[bh * D + d] = (float)(t / (double)N);
  vamax[bh * D + d] = mm;
  vscale[bh * D + d] = FP8_MAX / mm < INFINITY ? mm / FP8_MAX : 0.f;
}

// ---------------------------------------------------------------------------
// FP8 codes of one token block of Q (mu == nullptr) or of smoothed K.
// block = 256 threads: thread = (row lane rl, channel group cg of 8); rows
// rl, rl+16, ... of the block.  Rows at or past N get zero codes.
// ---------------------------------------------------------------------------
template <int BLK>
__device__ __forceinline__ void fp8_block(const uint16_t* __restrict__ x, const float* __restrict__ mu,
                                          uint8_t* __restrict__ codes, float* __restrict__ scales,
                                          int N, int n_pad, int bh, int blk, float* red) {
  constexpr int RPT = BLK / 16;
  const int tid = threadIdx.x, cg = tid & 15, rl = tid >> 4;
  const int n0 = blk * BLK;
  float val[RPT][8];
  float mloc[8];
  if (mu) {
#pragma unroll
    for (int j = 0; j < 8; ++j) mloc[j] = mu[bh * D + cg * 8 + j];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int n = n0 + rl + 16 * i;
    if (n < N) {
      const u32x4 w = *(const u32x4*)(x + ((size_t)bh * N + n) * D + cg * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) { val[i][2 * j] = bf16_lo(w[j]); val[i][2 * j + 1] = bf16_hi(w[j]); }
      if (mu) {
#pragma unroll
        for (int j = 0; j < 8; ++j) val[i][j] = val[i][j] - mloc[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(val[i][j]));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) val[i][j] = 0.f;
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // the block gets codes when its fp32 inverse scale is finite: not for
  // amax = 0, nor for amax below FP8_MAX / FLT_MAX, where it overflows
  const float inv = FP8_MAX / amax;
  const bool live = inv < INFINITY;
  if (tid == 0) scales[blk] = live ? amax / FP8_MAX : 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int n = n0 + rl + 16 * i;
    u32x2 out = {0u, 0u};
    if (live && n < N) {
      int lo = cvt_e4m3x2<false>(clamp448(val[i][0] * inv), clamp448(val[i][1] * inv), 0);
      lo = cvt_e4m3x2<true>(clamp448(val[i][2] * inv), clamp448(val[i][3] * inv), lo);
      int hi = cvt_e4m3x2<false>(clamp448(val[i][4] * inv), clamp448(val[i][5] * inv), 0);
      hi = cvt_e4m3x2<true>(clamp448(val[i][6] * inv), clamp448(val[i][7] * inv), hi);
      out[0] = (uint32_t)lo;
      out[1] = (uint32_t)hi;
    }
    *(u32x2*)(codes + ((size_t)bh * n_pad + n) * D + cg * 8) = out;
  }
}

// ---------------------------------------------------------------------------
// FP4 codes: one thread per (token, 16-channel group).  grid = (n_pad/32, BH, 2)
// (z = 0: Q, z = 1: smoothed K; first_z = 1 and grid z = 1 when the attention
// kernel quantizes Q itself), block = 256 = 32 tokens x 8 groups.
// Codes [BH][n_pad][64] (even channel in the low nibble), scales [BH][n_pad][8].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_qk_fp4_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ mu,
    uint8_t* __restrict__ qc, float* __restrict__ qs, uint8_t* __restrict__ kc,
    float* __restrict__ ks, int N, int n_pad, int first_z) {
  const int bh = last_first(blockIdx.y);
  const bool is_k = blockIdx.z + first_z == 1;
  const uint16_t* x = is_k ? k : q;
  uint8_t* codes = is_k ? kc : qc;
  float* scales = is_k ? ks : qs;
  const int tid = threadIdx.x, grp = tid & 7;
  const int n = blockIdx.x * 32 + (tid >> 3);
  float val[16];
  float amax = 0.f;
  if (n < N) {
    const u32x4* src = (const u32x4*)(x + ((size_t)bh * N + n) * D + grp * 16);
    const u32x4 w0 = src[0], w1 = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      val[2 * j] = bf16_lo(w0[j]);
      val[2 * j + 1] = bf16_hi(w0[j]);
      val[8 + 2 * j] = bf16_lo(w1[j]);
      val[8 + 2 * j + 1] = bf16_hi(w1[j]);
    }
    if (is_k) {
#pragma unroll
      for (int j = 0; j < 16; ++j) val[j] = val[j] - mu[bh * D + grp * 16 + j];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(val[j]));
  }
  u32x2 out = {0u, 0u};
  float scale = 0.f;
  const float inv = FP4_MAX / amax;   // +inf for amax = 0 or below FP4_MAX / FLT_MAX: zero codes
  if (inv < INFINITY) {
    scale = amax / FP4_MAX;
    out[0] = e2m1_word8(val, inv);
    out[1] = e2m1_word8(val + 8, inv);
  }
  *(u32x2*)(codes + ((size_t)bh * n_pad + n) * (D / 2) + grp * 8) = out;
  scales[((size_t)bh * n_pad + n) * 8 + grp] = scale;
}

// ---------------------------------------------------------------------------
// V codes, written as 64-key tiles [128 channels][64 keys] in the key order of
// the value product's B operand: byte p of a channel row holds key
// 32*kb + 8*(r>>2) + 4*g + (r&3) with g = p>>5, kb = (p>>4)&1, r = p&15.
// grid = (n_pad/64, BH), block = 256.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int vtile_pos(int key) {
  const int kb = key >> 5, w = key & 31;
  const int r = ((w >> 3) << 2) | (w & 3);
  const int g = (w >> 2) & 1;
  return 32 * g + 16 * kb + r;
}

// One 64-key V tile.  Thread = (token group tg of 4 consecutive keys, channel
// group cg of 8): the 4 keys of a group sit in 4 consecutive bytes of a
// channel row (keys 4m..4m+3 map to bytes p..p+3), so each thread writes one
// 32-bit word per channel.  The LDS copy of the tile uses 72-byte rows, which
// keeps those word writes free of bank conflicts; it is then copied out as the
// 8 KB tile.  Keys at or past N and channels with no finite inverse scale
// (vmax = 0, or below FP8_MAX / FLT_MAX) get zero codes.
constexpr int VROW = 72;

__device__ __forceinline__ void quant_v_tile(const uint16_t* __restrict__ v, const float* __restrict__ vamax,
                                             uint8_t* __restrict__ vc, int N, int n_pad, int bh, int t,
                                             uint8_t* tile) {
  const int tid = threadIdx.x, tg = tid & 15, cg = tid >> 4;
  float inv[8];
  bool nz[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = vamax[bh * D + cg * 8 + j];
    inv[j] = FP8_MAX / a;   // +inf for a = 0 or below FP8_MAX / FLT_MAX: zero codes
    nz[j] = inv[j] < INFINITY;
    inv[j] = nz[j] ? inv[j] : 0.f;
  }
  float val[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = t * KSTEP + 4 * tg + i;
    if (n < N) {
      const u32x4 w = *(const u32x4*)(v + ((size_t)bh * N + n) * D + cg * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) { val[i][2 * j] = bf16_lo(w[j]); val[i][2 * j + 1] = bf16_hi(w[j]); }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) val[i][j] = 0.f;
    }
  }
  const int pos = vtile_pos(4 * tg);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int wd = cvt_e4m3x2<false>(clamp448(val[0][j] * inv[j]), clamp448(val[1][j] * inv[j]), 0);
    wd = cvt_e4m3x2<true>(clamp448(val[2][j] * inv[j]), clamp448(val[3][j] * inv[j]), wd);
    *(uint32_t*)(tile + (cg * 8 + j) * VROW + pos) = nz[j] ? (uint32_t)wd : 0u;
  }
  __syncthreads();
  u32x4* dst = (u32x4*)(vc + ((size_t)bh * (n_pad / KSTEP) + t) * (D * KSTEP));
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ci = tid + 256 * i;
    const int d = ci >> 2, c = ci & 3;
    const u32x2 a = *(const u32x2*)(tile + d * VROW + c * 16);
    const u32x2 b = *(const u32x2*)(tile + d * VROW + c * 16 + 8);
    dst[ci] = u32x4{a[0], a[1], b[0], b[1]};
  }
}

// All codes in one launch: grid = (q_blocks + k_blocks + n_pad/64, BH); the
// first q_blocks blocks quantize Q (block_q tokens each), the next k_blocks
// smoothed K (64 tokens each), the rest V (one 64-key tile each).
template <int BQ>
__global__ __launch_bounds__(256) void quant_fp8_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ mu, const float* __restrict__ vamax, uint8_t* __restrict__ qc,
    float* __restrict__ qs, uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc,
    int N, int n_pad, int first_block) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * VROW];
  const int bh = last_first(blockIdx.y);
  const int qb = n_pad / BQ, kb = n_pad / KSTEP;
  const int b = blockIdx.x + first_block;   // first_block = qb: skip the Q blocks
  if (b < qb) {
    fp8_block<BQ>(q, nullptr, qc, qs + (size_t)bh * qb, N, n_pad, bh, b, red);
  } else if (b < qb + kb) {
    fp8_block<KSTEP>(k, mu, kc, ks + (size_t)bh * kb, N, n_pad, bh, b - qb, red);
  } else {
    quant_v_tile(v, vamax, vc, N, n_pad, bh, b - qb - kb, tile);
  }
}

// V codes alone (FP4 mode, where Q and K take the per-group kernel).
__global__ __launch_bounds__(256) void quant_v_kernel(const uint16_t* __restrict__ v,
                                                      const float* __restrict__ vamax,
                                                      uint8_t* __restrict__ vc, int N, int n_pad) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * VROW];
  quant_v_tile(v, vamax, vc, N, n_pad, last_first(blockIdx.y), blockIdx.x, tile);
}

// ---------------------------------------------------------------------------
// MXFP4 codes of 64 tokens of Q (mu == nullptr) or of smoothed K.  Thread =
// (row lane rl, 8-channel group cg): rows rl, rl+16, rl+32, rl+48, one 16-byte
// load each; the 4 lanes of a 32-channel block (consecutive lanes) combine
// their maxima with two xor shuffles.  The shared scale is 2**(byte - 127)
// with byte = floor(log2 amax) - 2 + 127, which for a normal fp32 amax is its
// exponent field minus 2 (0 below that or for a zero block); x / 2**(byte-127)
// is one exact fp32 multiply by the power of two 2**(127 - byte), and the code
// is E2M1 of it, saturated at 6.  Codes [BH][n_pad][64] (even channel in the
// low nibble).  Q scale bytes [BH][n_pad][4]; K scale bytes in the score
// MFMA's lane order: per 64-key tile t, byte 2*kb + h of entry 32*g + r
// belongs to key 64t + 32kb + r and channel block 2h + g.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mx_block(const uint16_t* __restrict__ x, const float* __restrict__ mu,
                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, bool lane_order,
                                         int N, int n_pad, int bh, int blk) {
  const int tid = threadIdx.x, cg = tid & 15, rl = tid >> 4;
  float mloc[8];
  if (mu) {
#pragma unroll
    for (int j = 0; j < 8; ++j) mloc[j] = mu[bh * D + cg * 8 + j];
  }
  float val[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = blk * KSTEP + rl + 16 * i;
    if (n < N) {
      const u32x4 w = *(const u32x4*)(x + ((size_t)bh * N + n) * D + cg * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) { val[i][2 * j] = bf16_lo(w[j]); val[i][2 * j + 1] = bf16_hi(w[j]); }
      if (mu) {
#pragma unroll
        for (int j = 0; j < 8; ++j) val[i][j] = val[i][j] - mloc[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) val[i][j] = 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = blk * KSTEP + rl + 16 * i;
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(val[i][j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    uint32_t word = 0, byte = 0;
    if (amax > 0.f) {
      byte = mx_scale_byte(amax);
      const float inv = mx_inv_scale(byte);
      word = e2m1_word8(val[i], inv);
    }
    *(uint32_t*)(codes + ((size_t)bh * n_pad + n) * (D / 2) + cg * 4) = word;
    if ((cg & 3) == 0) {
      const int b = cg >> 2;
      if (lane_order) {
        const int t = n >> 6, kk = n & 63, kb = kk >> 5, r = kk & 31, h = b >> 1, g = b & 1;
        scales[((size_t)bh * (n_pad / KSTEP) + t) * 256 + (32 * g + r) * 4 + 2 * kb + h] = (uint8_t)byte;
      } else {
        scales[((size_t)bh * n_pad + n) * 4 + b] = (uint8_t)byte;
      }
    }
  }
}

// MXFP4 mode: Q blocks, then K blocks, then V tiles, 64 tokens each, in one
// grid = (3 * n_pad/64, BH); first_block = n_pad/64 skips the Q blocks.
__global__ __launch_bounds__(256) void quant_mx_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ mu, const float* __restrict__ vamax, uint8_t* __restrict__ qc,
    uint8_t* __restrict__ qs, uint8_t* __restrict__ kc, uint8_t* __restrict__ ks, uint8_t* __restrict__ vc,
    int N, int n_pad, int first_block) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * VROW];
  const int bh = last_first(blockIdx.y), nb = n_pad / KSTEP;
  const int b = blockIdx.x + first_block;
  if (b < nb) {
    mx_block(q, nullptr, qc, qs, false, N, n_pad, bh, b);
  } else if (b < 2 * nb) {
    mx_block(k, mu, kc, ks, true, N, n_pad, bh, b - nb);
  } else {
    quant_v_tile(v, vamax, vc, N, n_pad, bh, b - 2 * nb, tile);
  }
}

// ---------------------------------------------------------------------------
// FP4 mode: K expanded once per head for the attention kernel's score MFMAs.
// Each element x = code * scale, times the tile's power of two 2^-E
// (fp4_norm_exp of the tile's largest scale), gives
//   hi = f16(x')                      (f16 hi.hi MFMA operand)
//   lo8 = E4M3((x' - hi) * 2^5)       (FP8 correction operands: x' - hi is
//   hi8 = E4M3(hi * 2^-6)              exact in fp32, the powers of two keep
//                                      both below 448)
// all rounded to nearest even, written as 32 KB per 64-key tile in the LDS
// order the attention kernel reads, so that it can copy tiles into LDS
// unchanged: the 16 KB f16 hi tile, then the 16 KB correction tile whose
// 16-byte chunk 2c + i of a key row holds lo8 (i = 0) or hi8 (i = 1) of the
// 16 channels 16c .. 16c + 15 (both tiles with the kh_off chunk swizzle); E
// goes to kexp[tile].  grid = (n_pad/64, BH), block = 256; a thread expands
// 4 of the tile's 64 x 16 chunks of 8 channels.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void expand_k_fp4_kernel(const uint8_t* __restrict__ kc,
                                                           const float* __restrict__ ks,
                                                           uint8_t* __restrict__ kx, int* __restrict__ kexp,
                                                           int n_pad) {
  __shared__ float wmax[4];
  const int tile = blockIdx.x, bh = blockIdx.y, tiles = n_pad / KSTEP;
  uint8_t* dst = kx + ((size_t)bh * tiles + tile) * KXTILE;
  uint32_t w[4];
  float s[4], smax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int key = idx >> 4, c = idx & 15;
    const size_t row = (size_t)bh * n_pad + (size_t)tile * KSTEP + key;
    w[i] = *(const uint32_t*)(kc + row * (D / 2) + 4 * c);
    s[i] = ks[row * 8 + (c >> 1)];
    smax = fmaxf(smax, s[i]);
  }
  smax = wave_max(smax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = smax;
  __syncthreads();
  const int E = fp4_norm_exp(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
  if (threadIdx.x == 0) kexp[(size_t)bh * tiles + tile] = E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int key = idx >> 4, c8 = idx & 15;
    v8h hv;
    float lo[8], h8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // x rounded to fp32 first (no fused multiply-convert), then scaled
      // exactly; the scalings by 2^5 and 2^-6 are exact too
      float x = e2m1_value((w[i] >> (4 * e)) & 15u) * s[i];
      asm volatile("" : "+v"(x));
      x = ldexpf(x, -E);
      hv[e] = (_Float16)x;
      lo[e] = (x - (float)hv[e]) * 32.f;
      h8[e] = (float)hv[e] * 0.015625f;
    }
    u32x2 lw, hw;
    lw[0] = (uint32_t)cvt_e4m3x2<true>(lo[2], lo[3], cvt_e4m3x2<false>(lo[0], lo[1], 0));
    lw[1] = (uint32_t)cvt_e4m3x2<true>(lo[6], lo[7], cvt_e4m3x2<false>(lo[4], lo[5], 0));
    hw[0] = (uint32_t)cvt_e4m3x2<true>(h8[2], h8[3], cvt_e4m3x2<false>(h8[0], h8[1], 0));
    hw[1] = (uint32_t)cvt_e4m3x2<true>(h8[6], h8[7], cvt_e4m3x2<false>(h8[4], h8[5], 0));
    // 8-channel chunk c8 is half (c8 & 1) of 16-channel chunk c8 >> 1
    const int half = (c8 & 1) * 8, c16 = c8 >> 1;
    *(v8h*)(dst + kh_off(key, c8)) = hv;
    *(u32x2*)(dst + KXTILE / 2 + kh_off(key, 2 * c16) + half) = lw;
    *(u32x2*)(dst + KXTILE / 2 + kh_off(key, 2 * c16 + 1) + half) = hw;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
void launch_quantize(const LaunchArgs& a, hipStream_t s) {
  const int BH = a.batch * a.heads;
  stats_partial_kernel<<<dim3(a.stats_splits, BH), 256, 0, s>>>(
      (const uint16_t*)a.k, (const uint16_t*)a.v, a.seq_len, a.stats_splits, (double*)a.stats_sum,
      (float*)a.stats_max, (uint32_t*)a.stats_range);
  stats_final_kernel<<<BH, 128, 0, s>>>((const double*)a.stats_sum, (const float*)a.stats_max,
                                        (const uint32_t*)a.stats_range, (const uint16_t*)a.k, a.seq_len,
                                        a.stats_splits, a.k_mean, a.v_amax, a.v_scales);
  const int vtiles = a.n_pad / KSTEP;
  if (a.mx) {
    // Q blocks skipped when the attention kernel quantizes Q
    const int first = a.fuse_q ? vtiles : 0;
    quant_mx_kernel<<<dim3(3 * vtiles - first, BH), 256, 0, s>>>(
        (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.k_mean, a.v_amax, a.q_codes,
        (uint8_t*)a.q_scales, a.k_codes, (uint8_t*)a.k_scales, a.v_codes, a.seq_len, a.n_pad, first);
  } else if (a.fp4) {
    // the Q groups are skipped when the attention kernel quantizes Q
    const int first_z = a.fuse_q ? 1 : 0;
    quant_qk_fp4_kernel<<<dim3(a.n_pad / 32, BH, 2 - first_z), 256, 0, s>>>(
        (const uint16_t*)a.q, (const uint16_t*)a.k, a.k_mean, a.q_codes, a.q_scales, a.k_codes,
        a.k_scales, a.seq_len, a.n_pad, first_z);
    expand_k_fp4_kernel<<<dim3(vtiles, BH), 256, 0, s>>>(a.k_codes, a.k_scales, a.k_expanded,
                                                        (int*)(a.k_expanded + (size_t)BH * vtiles * KXTILE), a.n_pad);
    quant_v_kernel<<<dim3(vtiles, BH), 256, 0, s>>>((const uint16_t*)a.v, a.v_amax, a.v_codes, a.seq_len,
                                                   a.n_pad);
  } else {
    // Q blocks first (skipped when the attention kernel quantizes Q), then K blocks and V tiles
    const int qblocks = a.n_pad / a.block_q, first = a.fuse_q ? qblocks : 0;
    const dim3 grid(qblocks + a.n_pad / KSTEP + vtiles - first, BH);
    auto kern = a.block_q == 128 ? quant_fp8_kernel<128> : quant_fp8_kernel<64>;
    kern<<<grid, 256, 0, s>>>((const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.k_mean,
                              a.v_amax, a.q_codes, a.q_scales, a.k_codes, a.k_scales, a.v_codes, a.seq_len,
                              a.n_pad, first);
  }
}

}  // namespace qsdpa
