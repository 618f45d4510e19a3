// C ABI of the quantized attention library: argument checking, workspace
// layout and dispatch.  Everything up to the first launch is plain host code
// that makes no HIP call, so an invalid call returns before any work is
// enqueued (and can be exercised on a machine without a GPU).
#include "../../include/qsdpa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "qsdpa_launch.h"

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_params(const qsdpa_params* p) {
  if (!p) return QSDPA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 1) return QSDPA_ERR_INVALID_ARG;
  if (p->head_dim != QSDPA_HEAD_DIM) return QSDPA_ERR_UNSUPPORTED;
  if (p->seq_len > QSDPA_MAX_SEQ_LEN) return QSDPA_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)p->batch * p->heads;
  if (bh > QSDPA_MAX_BH) return QSDPA_ERR_UNSUPPORTED;  // grid y / flattened grid limits
  const int64_t n_pad = ((int64_t)p->seq_len + 127) / 128 * 128;
  if (bh * n_pad * QSDPA_HEAD_DIM > QSDPA_MAX_ELEMS) return QSDPA_ERR_INVALID_ARG;
  if (!(p->softmax_scale > 0.f) || !std::isfinite(p->softmax_scale)) return QSDPA_ERR_INVALID_ARG;
  if (p->qk_format == QSDPA_QK_FP8_E4M3) {
    if (p->block_q != 64 && p->block_q != 128) return QSDPA_ERR_UNSUPPORTED;
    if (p->block_k != 64) return QSDPA_ERR_UNSUPPORTED;
  } else if (p->qk_format == QSDPA_QK_FP4_E2M1) {
    if (p->fp4_group != 16) return QSDPA_ERR_UNSUPPORTED;
  } else if (p->qk_format != QSDPA_QK_MXFP4_E2M1) {
    return QSDPA_ERR_UNSUPPORTED;
  }
  return QSDPA_OK;
}

void make_layout(const qsdpa_params* p, qsdpa_layout* L) {
  std::memset(L, 0, sizeof(*L));
  const uint64_t bh = (uint64_t)p->batch * p->heads;
  const int n_pad = (p->seq_len + 127) / 128 * 128;
  const bool fp4 = p->qk_format == QSDPA_QK_FP4_E2M1;
  const bool mx = p->qk_format == QSDPA_QK_MXFP4_E2M1;
  L->n_pad = n_pad;
  L->code_row_bytes = fp4 || mx ? 64 : 128;
  L->q_scale_count = fp4 ? n_pad * 8 : mx ? n_pad * 4 : n_pad / p->block_q;
  L->k_scale_count = fp4 ? n_pad * 8 : mx ? n_pad * 4 : n_pad / 64;
  const uint64_t scale_bytes = mx ? 1 : 4;   // E8M0 bytes or fp32
  L->stats_splits = (p->seq_len + qsdpa::STATS_ROWS - 1) / qsdpa::STATS_ROWS;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { const uint64_t at = off; off = align_up(off + bytes); return at; };
  L->q_codes = take(bh * n_pad * L->code_row_bytes);
  L->k_codes = take(bh * n_pad * L->code_row_bytes);
  L->v_codes = take(bh * n_pad * QSDPA_HEAD_DIM);
  L->q_scales = take(bh * L->q_scale_count * scale_bytes);
  L->k_scales = take(bh * L->k_scale_count * scale_bytes);
  L->k_mean = take(bh * QSDPA_HEAD_DIM * 4);
  L->v_scales = take(bh * QSDPA_HEAD_DIM * 4);
  L->v_amax = take(bh * QSDPA_HEAD_DIM * 4);
  L->stats = take(bh * L->stats_splits * QSDPA_HEAD_DIM * (8 + 4 + 4));
  L->k_expanded = take(fp4 ? bh * n_pad * QSDPA_HEAD_DIM * 4 + bh * (n_pad / 64) * 4 : 0);
  L->total = off;
}

// Selective correction: rows per (b,h), their split, and the extra
// workspace sections after the base layout.
int vc_plan(const qsdpa_params* p, float rho, const qsdpa_layout& L, qsdpa_vc_layout* v) {
  if (p->qk_format != QSDPA_QK_FP8_E4M3) return QSDPA_ERR_UNSUPPORTED;
  if (!(rho > 0.f) || !(rho <= 1.f)) return QSDPA_ERR_INVALID_ARG;
  std::memset(v, 0, sizeof(*v));
  const int N = p->seq_len;
  const uint64_t bh = (uint64_t)p->batch * p->heads;
  const double want = std::ceil((double)rho * N - 1e-9);
  v->count = (int32_t)std::min<double>(N, std::max(1.0, want));
  v->count_pad = (v->count + 31) / 32 * 32;
  // about 2048 waves in the recomputation, each over whole 32-key steps
  const uint64_t groups = bh * (uint64_t)(v->count_pad / 32);
  const int by_waves = (int)std::max<uint64_t>(1, (2048 + groups - 1) / groups);
  const int chunks = std::min(by_waves, (N + 31) / 32);
  v->chunk_keys = ((N + chunks - 1) / chunks + 31) / 32 * 32;
  v->chunks = (N + v->chunk_keys - 1) / v->chunk_keys;
  uint64_t off = L.total;
  auto take = [&](uint64_t bytes) { const uint64_t at = off; off = align_up(off + bytes); return at; };
  v->token_error = take(bh * L.n_pad * 8);
  v->selected = take(bh * v->count_pad * 4);
  v->partials = take(bh * v->count_pad * (uint64_t)v->chunks * qsdpa::VC_PART * 4);
  v->total = off;
  return QSDPA_OK;
}

bool aligned(const void* ptr, uint64_t a) { return ((uintptr_t)ptr % a) == 0; }

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

qsdpa::LaunchArgs make_args(const qsdpa_params* p, const qsdpa_layout& L, const void* q, const void* k,
                            const void* v, void* o, const void* ws) {
  uint8_t* w = (uint8_t*)ws;
  qsdpa::LaunchArgs a;
  a.batch = p->batch;
  a.heads = p->heads;
  a.seq_len = p->seq_len;
  a.n_pad = L.n_pad;
  a.block_q = p->block_q;
  a.fp4 = p->qk_format == QSDPA_QK_FP4_E2M1;
  a.mx = p->qk_format == QSDPA_QK_MXFP4_E2M1;
  a.fuse_q = false;
  a.softmax_scale = p->softmax_scale;
  a.stats_splits = L.stats_splits;
  a.q_scale_count = L.q_scale_count;
  a.k_scale_count = L.k_scale_count;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.q_codes = w + L.q_codes;
  a.q_scales = (float*)(w + L.q_scales);
  a.k_codes = w + L.k_codes;
  a.k_scales = (float*)(w + L.k_scales);
  a.k_mean = (float*)(w + L.k_mean);
  a.v_codes = w + L.v_codes;
  a.v_scales = (float*)(w + L.v_scales);
  a.v_amax = (float*)(w + L.v_amax);
  a.k_expanded = w + L.k_expanded;
  a.stats_sum = w + L.stats;
  const uint64_t partials = (uint64_t)p->batch * p->heads * L.stats_splits * QSDPA_HEAD_DIM;
  a.stats_max = w + L.stats + partials * 8;
  a.stats_range = w + L.stats + partials * 12;
  return a;
}

int check_buffers(const qsdpa_params* p, const qsdpa_layout& L, const void* q, const void* k, const void* v,
                  const void* o, const void* ws, size_t ws_bytes, bool need_qkv, bool need_o) {
  if (!ws) return QSDPA_ERR_INVALID_ARG;
  if (need_qkv && (!q || !k || !v)) return QSDPA_ERR_INVALID_ARG;
  if (need_o && !o) return QSDPA_ERR_INVALID_ARG;
  if (!aligned(ws, kAlign)) return QSDPA_ERR_ALIGNMENT;
  if (need_qkv && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))) return QSDPA_ERR_ALIGNMENT;
  if (need_o && !aligned(o, 16)) return QSDPA_ERR_ALIGNMENT;
  if (ws_bytes < L.total) return QSDPA_ERR_WORKSPACE_TOO_SMALL;
  const uint64_t tbytes = (uint64_t)p->batch * p->heads * p->seq_len * QSDPA_HEAD_DIM * 2;
  if (need_o) {
    if (overlaps(o, tbytes, ws, L.total)) return QSDPA_ERR_ALIAS;
    if (need_qkv && (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) ||
                     overlaps(o, tbytes, v, tbytes)))
      return QSDPA_ERR_ALIAS;
  }
  if (need_qkv && (overlaps(q, tbytes, ws, L.total) || overlaps(k, tbytes, ws, L.total) ||
                   overlaps(v, tbytes, ws, L.total)))
    return QSDPA_ERR_ALIAS;
  return QSDPA_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? QSDPA_OK : QSDPA_ERR_HIP; }

}  // namespace

extern "C" {

int qsdpa_abi_version(void) { return QSDPA_ABI_VERSION; }

const char* qsdpa_status_string(int status) {
  switch (status) {
    case QSDPA_OK: return "ok";
    case QSDPA_ERR_INVALID_ARG: return "invalid argument";
    case QSDPA_ERR_UNSUPPORTED: return "unsupported configuration";
    case QSDPA_ERR_ALIGNMENT: return "misaligned pointer";
    case QSDPA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QSDPA_ERR_ALIAS: return "output overlaps an input or the workspace";
    case QSDPA_ERR_HIP: return "HIP launch failure";
    case QSDPA_ERR_SCRATCH_TOO_SMALL: return "the problem needs more workspace than the static scratch buffer holds";
    default: return "unknown status";
  }
}

int qsdpa_validate_params(const qsdpa_params* p) { return check_params(p); }

size_t qsdpa_workspace_bytes(const qsdpa_params* p) {
  if (check_params(p) != QSDPA_OK) return 0;
  qsdpa_layout L;
  make_layout(p, &L);
  return (size_t)L.total;
}

int qsdpa_workspace_layout(const qsdpa_params* p, qsdpa_layout* out) {
  const int st = check_params(p);
  if (st != QSDPA_OK) return st;
  if (!out) return QSDPA_ERR_INVALID_ARG;
  make_layout(p, out);
  return QSDPA_OK;
}

int qsdpa_quantize(const qsdpa_params* p, const void* q, const void* k, const void* v, void* workspace,
                   size_t ws_bytes, void* stream) {
  int st = check_params(p);
  if (st != QSDPA_OK) return st;
  qsdpa_layout L;
  make_layout(p, &L);
  st = check_buffers(p, L, q, k, v, nullptr, workspace, ws_bytes, true, false);
  if (st != QSDPA_OK) return st;
  (void)hipGetLastError();
  qsdpa::launch_quantize(make_args(p, L, q, k, v, nullptr, workspace), (hipStream_t)stream);
  return launch_status();
}

int qsdpa_attention(const qsdpa_params* p, const void* workspace, size_t ws_bytes, void* o, void* stream) {
  int st = check_params(p);
  if (st != QSDPA_OK) return st;
  qsdpa_layout L;
  make_layout(p, &L);
  st = check_buffers(p, L, nullptr, nullptr, nullptr, o, workspace, ws_bytes, false, true);
  if (st != QSDPA_OK) return st;
  (void)hipGetLastError();
  qsdpa::launch_attention(make_args(p, L, nullptr, nullptr, nullptr, o, workspace), (hipStream_t)stream);
  return launch_status();
}

int qsdpa_forward(const qsdpa_params* p, const void* q, const void* k, const void* v, void* o, void* workspace,
                  size_t ws_bytes, void* stream) {
  return qsdpa::forward_impl(p, q, k, v, o, workspace, ws_bytes, stream);
}

int qsdpa_vc_workspace_layout(const qsdpa_params* p, float rho, qsdpa_vc_layout* out) {
  int st = check_params(p);
  if (st != QSDPA_OK) return st;
  if (!out) return QSDPA_ERR_INVALID_ARG;
  qsdpa_layout L;
  make_layout(p, &L);
  return vc_plan(p, rho, L, out);
}

size_t qsdpa_vc_workspace_bytes(const qsdpa_params* p, float rho) {
  qsdpa_vc_layout V;
  return qsdpa_vc_workspace_layout(p, rho, &V) == QSDPA_OK ? (size_t)V.total : 0;
}

int qsdpa_forward_vc(const qsdpa_params* p, float rho, const void* q, const void* k, const void* v, void* o,
                     void* workspace, size_t ws_bytes, void* stream) {
  int st = check_params(p);
  if (st != QSDPA_OK) return st;
  qsdpa_layout L;
  make_layout(p, &L);
  qsdpa_vc_layout V;
  st = vc_plan(p, rho, L, &V);
  if (st != QSDPA_OK) return st;
  st = check_buffers(p, L, q, k, v, o, workspace, ws_bytes, true, true);
  if (st != QSDPA_OK) return st;
  if (ws_bytes < V.total) return QSDPA_ERR_WORKSPACE_TOO_SMALL;
  const uint64_t tbytes = (uint64_t)p->batch * p->heads * p->seq_len * QSDPA_HEAD_DIM * 2;
  if (overlaps(o, tbytes, workspace, V.total) || overlaps(q, tbytes, workspace, V.total) ||
      overlaps(k, tbytes, workspace, V.total) || overlaps(v, tbytes, workspace, V.total))
    return QSDPA_ERR_ALIAS;
  (void)hipGetLastError();
  uint8_t* w = (uint8_t*)workspace;
  qsdpa::LaunchArgs a = make_args(p, L, q, k, v, o, workspace);
  a.fuse_q = true;
  a.vc_err = (double*)(w + V.token_error);
  qsdpa::launch_quantize(a, (hipStream_t)stream);
  if (launch_status() != QSDPA_OK) return QSDPA_ERR_HIP;
  qsdpa::launch_attention(a, (hipStream_t)stream);
  if (launch_status() != QSDPA_OK) return QSDPA_ERR_HIP;
  qsdpa::VcArgs c;
  c.batch = p->batch;
  c.heads = p->heads;
  c.seq_len = p->seq_len;
  c.n_pad = L.n_pad;
  c.count = V.count;
  c.count_pad = V.count_pad;
  c.chunks = V.chunks;
  c.chunk_keys = V.chunk_keys;
  c.softmax_scale = p->softmax_scale;
  c.q = q;
  c.k = k;
  c.v = v;
  c.o = o;
  c.err = (const double*)(w + V.token_error);
  c.sel = (int32_t*)(w + V.selected);
  c.part = (float*)(w + V.partials);
  qsdpa::launch_vc(c, (hipStream_t)stream);
  return launch_status();
}

int qsdpa_attention_bf16q(const qsdpa_params* p, const void* q, const void* workspace, size_t ws_bytes, void* o,
                          void* stream) {
  int st = check_params(p);
  if (st != QSDPA_OK) return st;
  qsdpa_layout L;
  make_layout(p, &L);
  st = check_buffers(p, L, nullptr, nullptr, nullptr, o, workspace, ws_bytes, false, true);
  if (st != QSDPA_OK) return st;
  if (!q) return QSDPA_ERR_INVALID_ARG;
  if (!aligned(q, 16)) return QSDPA_ERR_ALIGNMENT;
  const uint64_t tbytes = (uint64_t)p->batch * p->heads * p->seq_len * QSDPA_HEAD_DIM * 2;
  if (overlaps(o, tbytes, q, tbytes) || overlaps(q, tbytes, workspace, L.total)) return QSDPA_ERR_ALIAS;
  (void)hipGetLastError();
  qsdpa::LaunchArgs a = make_args(p, L, q, nullptr, nullptr, o, workspace);
  a.fuse_q = true;
  qsdpa::launch_attention(a, (hipStream_t)stream);
  return launch_status();
}

}  // extern "C"

namespace qsdpa {

int forward_impl(const qsdpa_params* p, const void* q, const void* k, const void* v, void* o, void* workspace,
                 size_t ws_bytes, void* stream) {
  int st = check_params(p);
  if (st != QSDPA_OK) return st;
  qsdpa_layout L;
  make_layout(p, &L);
  st = check_buffers(p, L, q, k, v, o, workspace, ws_bytes, true, true);
  if (st != QSDPA_OK) return st;
  (void)hipGetLastError();
  qsdpa::LaunchArgs a = make_args(p, L, q, k, v, o, workspace);
  // Q is quantized inside the attention kernel, bit-identically
  a.fuse_q = true;
  qsdpa::launch_quantize(a, (hipStream_t)stream);
  if (launch_status() != QSDPA_OK) return QSDPA_ERR_HIP;
  qsdpa::launch_attention(a, (hipStream_t)stream);
  return launch_status();
}

}  // namespace qsdpa
