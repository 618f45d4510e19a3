// Internal interface between the C ABI (argument checking, workspace layout)
// and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsdpa.h"

namespace qsdpa {

constexpr int STATS_ROWS = 256;  // tokens per range of the statistics pass

struct LaunchArgs {
  int batch, heads, seq_len, n_pad;
  int block_q;
  bool fp4;   // 16-channel FP4 with fp32 scales
  bool mx;    // MXFP4: 32-channel blocks with E8M0 scales
  bool fuse_q;   // the attention kernel quantizes Q from bf16 (the quantize pass skips it)
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
  void* stats_range;
  double* vc_err = nullptr;   // FP8 with FUSE_Q: per-token Q quantization error (selective correction)
};

// Selective correction (FP8): which rows of each (b,h) are recomputed, and
// how the recomputation is split.
struct VcArgs {
  int batch, heads, seq_len, n_pad;
  int count, count_pad;   // k = ceil(rho N) rows per (b,h), and k rounded up to 32
  int chunks, chunk_keys; // key ranges of the split recomputation
  float softmax_scale;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const double* err;      // [BH][n_pad]
  int32_t* sel;           // [BH][count_pad]
  float* part;            // [BH][count_pad][chunks][VC_PART]
};
constexpr int VC_PART = 132;   // floats per partial row: m, l, 2 spare, 128 accumulators

void launch_vc(const VcArgs& a, hipStream_t s);

void launch_quantize(const LaunchArgs& a, hipStream_t s);
void launch_attention(const LaunchArgs& a, hipStream_t s);

// qsdpa_forward on a caller-chosen workspace (argument checks, launches,
// status); shared by qsdpa_forward and the entry point on the static scratch.
int forward_impl(const qsdpa_params* p, const void* q, const void* k, const void* v, void* o, void* workspace,
                 size_t ws_bytes, void* stream);

}  // namespace qsdpa
