/*
 * qsdpa.h - C ABI of quantized scaled-dot-product attention for MI355X (gfx950).
 *
 * The operation.  Attention softmax(tau * Q K^T) V over one joint token
 * sequence per (batch, head) - text tokens, then image tokens, then (for
 * Kontext edits) context-image tokens, with no mask - computed with FP8 or
 * FP4 operands.  The pages describe quantizing the SDPA of the FLUX
 * transformer as the core of the work, with FP8 and FP4 schemes that differ
 * only in the precision of the query/key side while attention itself stays
 * FP8 (NVIDIA RTX AI optimiert FLUX.1 fuer Bilddaten mit niedriger
 * Genauigkeit, hyper.ai/de; NVIDIA RTX AI, 저정밀 양자화로 FLUX.1 Kontext 최적화,
 * hyper.ai/kr); Kontext concatenates the input-image tokens to the output-image
 * tokens (same articles).  They print no formula; the steps below are the
 * reading this library implements:
 *
 *   1. per (b,h,d): mu = fp32(fp64(sum_n K) / N), the exact sum rounded once
 *      to fp64 (for every finite input), vmax = max_n |V|;
 *   2. Ks = fp32(K - mu) (K smoothing: softmax is unchanged by it);
 *   3. FP8 mode: Q per block of block_q tokens, Ks per block of block_k
 *      tokens, scale s = fp32(amax/448), code = E4M3(fp32(x * fp32(448/amax)));
 *      FP4 mode: per token and 16 consecutive channels, s = fp32(amax/6),
 *      code = E2M1(fp32(x * fp32(6/amax))); an all-zero block has s = 0 and
 *      zero codes, and so does a block whose inverse fp32(F/amax) overflows
 *      (0 < amax < F/FLT_MAX: below about 1.3e-36 for FP8, 1.8e-38 for FP4).
 *      E4M3/E2M1 round to nearest even and saturate;
 *   4. V per channel: sV = fp32(vmax/448), code = E4M3(fp32(V * fp32(448/vmax)))
 *      (zero scale and codes for a channel as in 3);
 *   5. scores S = tau * dequant(Q) . dequant(K);
 *   6. online softmax over steps of 64 keys in ascending order:
 *      m = running max, p = exp(S - m), P = E4M3(448 p) fed to an FP8 P.V
 *      product, l = sum of the unquantized p, accumulators rescaled by
 *      exp(m_old - m_new);
 *   7. O = bf16_rne(acc * sV / (448 l)).
 *
 * Conventions for every entry point:
 *   - Q, K, V, O are device pointers to contiguous bf16 [B, H, N, 128]
 *     tensors owned by the caller; the workspace is a caller-owned device
 *     buffer of at least qsdpa_workspace_bytes() bytes.
 *   - Device pointers must be 16-byte aligned, the workspace 256-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; the library never allocates, frees or
 *     synchronizes, and keeps no state between calls (thread-safe).  The one
 *     exception is qsdpa_forward_noalloc: its static scratch array is shared by
 *     every call on a GPU (see there).
 *   - Every argument is validated before the first launch: a negative status
 *     means nothing was enqueued (except QSDPA_ERR_HIP, which reports a failed
 *     launch).  Nothing throws across the ABI.  Inputs must be finite.
 */
#ifndef QSDPA_H
#define QSDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSDPA_ABI_VERSION 7
#define QSDPA_HEAD_DIM 128

/* Status codes (return values). */
#define QSDPA_OK 0
#define QSDPA_ERR_INVALID_ARG (-1)         /* null pointer, size <= 0 or overflowing, bad scale */
#define QSDPA_ERR_UNSUPPORTED (-2)         /* head_dim != 128, block sizes, format, group size */
#define QSDPA_ERR_ALIGNMENT (-3)           /* a pointer is not 16 B (workspace: 256 B) aligned */
#define QSDPA_ERR_WORKSPACE_TOO_SMALL (-4) /* ws_bytes < qsdpa_workspace_bytes() */
#define QSDPA_ERR_ALIAS (-5)               /* O overlaps an input or the workspace */
#define QSDPA_ERR_HIP (-6)                 /* a kernel launch failed */
#define QSDPA_ERR_SCRATCH_TOO_SMALL (-7)   /* qsdpa_forward_noalloc: workspace > QSDPA_SCRATCH_BYTES */

/* Size limits, checked before any launch.  N above QSDPA_MAX_SEQ_LEN or
 * B*H above QSDPA_MAX_BH give QSDPA_ERR_UNSUPPORTED; B*H*round_up(N, 128)*128
 * above QSDPA_MAX_ELEMS (elements of one padded tensor) gives
 * QSDPA_ERR_INVALID_ARG. */
#define QSDPA_MAX_SEQ_LEN (1 << 22)
#define QSDPA_MAX_BH 65535
#define QSDPA_MAX_ELEMS (1LL << 36)

/* Size of the static scratch array of qsdpa_forward_noalloc (96 MiB per GPU):
 * enough for the Kontext workload [1, 24, 8704, 128] in FP8 and MXFP4 mode. */
#define QSDPA_SCRATCH_BYTES (96u << 20)

/* Q/K precision.  P and V are FP8 E4M3 in every mode.
 * MXFP4 (beyond the pages' FP4): E2M1 codes with one shared E8M0 (power of
 * two) scale per 32 consecutive channels, as in the OCP Microscaling Formats
 * specification v1.0; the shared exponent is floor(log2 amax) - 2, biased by
 * 127 and clamped to [0, 254] (0 for an all-zero block), and the codes are
 * E2M1(x / 2**(byte - 127)), nearest even, saturating at 6.  block_q, block_k
 * and fp4_group are ignored in this mode. */
#define QSDPA_QK_FP8_E4M3 0
#define QSDPA_QK_FP4_E2M1 1
#define QSDPA_QK_MXFP4_E2M1 2

typedef struct qsdpa_params {
  int32_t batch;         /* B >= 1, B*H <= QSDPA_MAX_BH */
  int32_t heads;         /* H >= 1 */
  int32_t seq_len;       /* 1 <= N <= QSDPA_MAX_SEQ_LEN (any value: tails are handled) */
  int32_t head_dim;      /* must be 128 */
  int32_t block_q;       /* FP8 mode: Q tokens per scale, 64 or 128 (ignored in the FP4 modes) */
  int32_t block_k;       /* FP8 mode: K tokens per scale, must be 64 (ignored in the FP4 modes) */
  int32_t qk_format;     /* QSDPA_QK_FP8_E4M3, QSDPA_QK_FP4_E2M1 or QSDPA_QK_MXFP4_E2M1 */
  int32_t fp4_group;     /* FP4 mode: channels per scale, must be 16 (ignored otherwise) */
  float softmax_scale;   /* tau > 0 and finite, normally 1/sqrt(128) */
} qsdpa_params;

/*
 * Byte offsets of the workspace sections (filled by qsdpa_workspace_layout).
 * N is padded to n_pad = round_up(N, 128); padded tokens hold zero codes.
 * BH = B*H, (b,h) index bh = b*H + h.
 *   q_codes, k_codes: uint8 [BH][n_pad][code_row_bytes]; FP8: one E4M3 code
 *                     per channel; FP4, MXFP4: two E2M1 codes per byte, the
 *                     even channel in the low nibble.
 *   q_scales:         fp32 [BH][q_scale_count]; FP8: per block_q tokens
 *                     (q_scale_count = n_pad/block_q, blocks past N are 0);
 *                     FP4: [BH][n_pad][8], one per 16 channels.
 *                     MXFP4: uint8 E8M0 bytes [BH][n_pad][4], one per 32
 *                     channels (q_scale_count = n_pad * 4).
 *   k_scales:         as q_scales with block_k.  MXFP4: uint8 E8M0 bytes
 *                     [BH][n_pad/64][64][4] in the lane order of the score
 *                     MFMA: for the 64-key tile t, byte 2*kb + h of entry
 *                     32*g + r is the scale of key 64t + 32kb + r, channels
 *                     64h + 32g .. 64h + 32g + 31 (k_scale_count = n_pad * 4).
 *   k_mean:           fp32 [BH][128] (mu).
 *   v_codes:          uint8 [BH][n_pad/64][128][64]: for each 64-key tile,
 *                     channel-major rows of 64 codes in a fixed key order:
 *                     byte p of a row holds key 32*kb + 8*(r>>2) + 4*g + (r&3)
 *                     with g = p>>5, kb = (p>>4)&1, r = p&15.
 *   v_scales:         fp32 [BH][128] (sV).
 *   v_amax:           fp32 [BH][128] (vmax).
 *   stats:            scratch for the statistics pass, per token range of
 *                     256 and channel: fp64 sums of K, fp32 maxima of |V|,
 *                     and the largest and smallest nonzero |K| (bf16 bits).
 *   k_expanded:       FP4 mode only (0 bytes in other modes): every K
 *                     element x = code * scale (one fp32 product) times
 *                     2^-E of its 64-key tile, x', as hi = f16(x') and the
 *                     E4M3 bytes lo8 = E4M3(fp32(x' - hi) * 2^5) and
 *                     hi8 = E4M3(hi * 2^-6), all rounded to nearest even.
 *                     Per tile 32 KB: the hi tile f16 [64 keys][128], its
 *                     8-channel chunk c of a key row stored at chunk
 *                     position c ^ (key & 15); then the correction tile
 *                     u8 [64 keys][16 chunks][16], whose chunk 2c + i holds
 *                     lo8 (i = 0) or hi8 (i = 1) of channels 16c .. 16c + 15
 *                     and is stored at position (2c + i) ^ (key & 15).
 *                     [BH][n_pad/64] such tiles, then int32 E [BH][n_pad/64]:
 *                     E = e - 138, e the biased exponent field of the
 *                     largest K scale of the tile, so |x'| < 24576 and
 *                     none of the three overflows.
 */
typedef struct qsdpa_layout {
  uint64_t q_codes, q_scales, k_codes, k_scales, k_mean, v_codes, v_scales, v_amax, stats;
  uint64_t k_expanded;
  uint64_t total;          /* bytes needed (= qsdpa_workspace_bytes) */
  int32_t n_pad;
  int32_t code_row_bytes;  /* 128 (FP8) or 64 (FP4) */
  int32_t q_scale_count;   /* per (b,h) */
  int32_t k_scale_count;   /* per (b,h) */
  int32_t stats_splits;    /* token ranges of the statistics pass */
  int32_t reserved[3];
} qsdpa_layout;

/* ABI version (QSDPA_ABI_VERSION of the built library). */
int qsdpa_abi_version(void);

/* Human-readable text of a status code (static storage, never NULL). */
const char* qsdpa_status_string(int status);

/* Validate parameters (host only, no GPU call).  Returns a status. */
int qsdpa_validate_params(const qsdpa_params* p);

/* Workspace bytes for p, or 0 if p is invalid.  No GPU call. */
size_t qsdpa_workspace_bytes(const qsdpa_params* p);

/* Fill *out with the workspace layout for p.  No GPU call.  Returns a status. */
int qsdpa_workspace_layout(const qsdpa_params* p, qsdpa_layout* out);

/*
 * Steps 1-4: channel statistics, K smoothing and the Q/K/V codes and scales,
 * written into the workspace (layout above).  q, k, v: bf16 [B,H,N,128].
 * In FP4 mode it also writes k_expanded from the K codes and scales.
 * (The quantization of the SDPA inputs, FP8 or FP4 for the query/key side:
 * hyper.ai/de, the paragraph on GEMM and SDPA quantization and the
 * SageAttention series; hyper.ai/kr, the paragraph on SDPA quantization.)
 */
int qsdpa_quantize(const qsdpa_params* p, const void* q, const void* k, const void* v,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * Steps 5-7 on a workspace filled by qsdpa_quantize with the same params:
 * writes O bf16 [B,H,N,128].  (The attention itself kept in FP8: hyper.ai/de,
 * the paragraph on Table 1; hyper.ai/kr, the paragraph on FP4 against FP8.)
 */
int qsdpa_attention(const qsdpa_params* p, const void* workspace, size_t ws_bytes, void* o,
                    void* stream);

/*
 * Steps 5-7 with Q given as bf16 [B,H,N,128]: the attention kernel quantizes
 * Q itself (step 3 for Q, with the quantize pass's blocks and operations, so
 * O is bit-identical to qsdpa_attention after qsdpa_quantize), on the K and V
 * codes, scales and statistics of a workspace that qsdpa_quantize or
 * qsdpa_forward filled with the same params and the same K and V.  The
 * workspace's q_codes and q_scales sections are neither read nor written.
 * This is the attention kernel of qsdpa_forward on its own (for example to
 * attend several query sets to keys and values quantized once).
 */
int qsdpa_attention_bf16q(const qsdpa_params* p, const void* q, const void* workspace, size_t ws_bytes,
                          void* o, void* stream);

/*
 * qsdpa_quantize followed by qsdpa_attention on the same stream: O is
 * bit-identical to the two calls.  (The quantized SDPA in place of the
 * transformer's BF16 SDPA: hyper.ai/de and hyper.ai/kr, as above.)  The attention kernel quantizes Q itself
 * (as qsdpa_attention_bf16q), so the q_codes and q_scales sections of the
 * workspace are not written by this call.
 */
int qsdpa_forward(const qsdpa_params* p, const void* q, const void* k, const void* v, void* o,
                  void* workspace, size_t ws_bytes, void* stream);

/*
 * Selective correction of the FP8 path (VC-Attention-style).  The VisualGen
 * article (FLUX 3 Image Klein Base, devotd.net, section on why the results
 * differ) names VC-Attention FP8 with rho = 0.005 as FP8 attention that
 * corrects only the tokens with a large error.  Reading implemented here:
 * per (b,h), the k = ceil(rho N) query tokens whose own FP8 quantization
 * error sum_d (q_d - code_d * s)^2 is largest (ties to the lower index) get
 * the unquantized softmax attention of the bf16 inputs (bf16 matrix-core
 * products with fp32 accumulation and an fp32 softmax) in place of their FP8
 * row of O; every other row is qsdpa_forward's, bit for bit.
 *
 * The workspace holds qsdpa_forward's sections followed by these (byte
 * offsets from the workspace start):
 *   token_error: fp64 [BH][n_pad], each token's error (rows < N);
 *   selected:    int32 [BH][count_pad], the corrected rows in ascending
 *                order (the first `count` entries are meaningful);
 *   partials:    fp32 scratch of the recomputation, split into `chunks`
 *                ranges of `chunk_keys` keys.
 * FP8 mode only (QSDPA_ERR_UNSUPPORTED otherwise); rho in (0, 1].
 */
typedef struct qsdpa_vc_layout {
  uint64_t token_error, selected, partials;
  uint64_t total;        /* workspace bytes needed (= qsdpa_vc_workspace_bytes) */
  int32_t count;         /* k = ceil(rho N), at least 1, at most N */
  int32_t count_pad;     /* k rounded up to 32 */
  int32_t chunks, chunk_keys;
} qsdpa_vc_layout;

/* Workspace bytes of qsdpa_forward_vc for (p, rho), or 0 if invalid.  No GPU call. */
size_t qsdpa_vc_workspace_bytes(const qsdpa_params* p, float rho);

/* Fill *out with the layout for (p, rho).  No GPU call.  Returns a status. */
int qsdpa_vc_workspace_layout(const qsdpa_params* p, float rho, qsdpa_vc_layout* out);

/* qsdpa_forward with the selective correction: buffers as for qsdpa_forward,
 * the workspace at least qsdpa_vc_workspace_bytes(p, rho). */
int qsdpa_forward_vc(const qsdpa_params* p, float rho, const void* q, const void* k, const void* v, void* o,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * qsdpa_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and result, bit for bit, with the workspace taken
 * from a static device array of QSDPA_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends.  No allocation of any kind.
 * q, k, v, o as for qsdpa_forward, on the current device.
 *   - Returns QSDPA_ERR_SCRATCH_TOO_SMALL (nothing enqueued) when
 *     qsdpa_workspace_bytes(p) exceeds QSDPA_SCRATCH_BYTES.
 *   - Every call on one GPU shares that GPU's array: calls whose work may
 *     overlap on one GPU (two streams, or two threads) race on it and must be
 *     serialized by the caller.  The array keeps the last call's contents;
 *     no call depends on them.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress); QSDPA_ERR_HIP if that fails.
 */
int qsdpa_forward_noalloc(const qsdpa_params* p, const void* q, const void* k, const void* v, void* o,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSDPA_H */
