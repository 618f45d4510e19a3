// Internal interface between the C ABI (argument checking, workspace layout)
// and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsdpa {

constexpr int STATS_ROWS = 256;  // tokens per range of the statistics pass

struct LaunchArgs {
  int batch, heads, seq_len, n_pad;
  int block_q;
  bool fp4;   // 16-channel FP4 with fp32 scales
  bool mx;    // MXFP4: 32-channel blocks with E8M0 scales
  bool fuse_q;   // FP8, MXFP4: the attention kernel quantizes Q (the quantize pass skips it)
  float softmax_scale;
  int stats_splits;
  int q_scale_count, k_scale_count;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  uint8_t* q_codes;
  float* q_scales;
  uint8_t* k_codes;
  float* k_scales;
  float* k_mean;
  uint8_t* v_codes;
  float* v_scales;
  float* v_amax;
  uint8_t* k_expanded;   // FP4 mode: K as f16 hi + E4M3 correction tiles
  void* stats_sum;
  void* stats_max;
};

void launch_quantize(const LaunchArgs& a, hipStream_t s);
void launch_attention(const LaunchArgs& a, hipStream_t s);

}  // namespace qsdpa
