/*
 * duolm_debug.h -- test-support entry points of the DuoLM ranker library.
 *
 * These expose single stages of the forward pass so that a test can compare
 * each kernel with an independent CPU computation of the same stage, and a
 * plain copy kernel used to calibrate hardware byte counters.  They are not
 * needed for scoring.  Same return and error conventions as duolm.h.
 */
#ifndef DUOLM_DEBUG_H
#define DUOLM_DEBUG_H

#include <stdint.h>

#include "duolm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stages inside one decoder layer, in execution order. */
typedef enum {
  DUOLM_STAGE_ATTN_NORM = 0, /* buffer: a = RMSNorm(x) bf16 [T, d] */
  DUOLM_STAGE_QKV = 1,       /* buffer: x W_qkv^T bf16 [T, (H + 2 H_kv) hd], q | k | v */
  DUOLM_STAGE_QK_ROPE = 2,   /* same buffer after per-head q/k RMSNorm and rotary embedding */
  DUOLM_STAGE_ATTN = 3,      /* buffer: attention output bf16 [T, H hd] */
  DUOLM_STAGE_ATTN_RESID = 4,/* buffer: residual stream fp32 [T, d] after x += o W_o^T */
  DUOLM_STAGE_MLP_NORM = 5,  /* buffer: b = RMSNorm(x) bf16 [T, d] */
  DUOLM_STAGE_SWIGLU = 6,    /* buffer: silu(b W_g^T) * (b W_u^T) bf16 [T, F] */
  DUOLM_STAGE_LAYER_OUT = 7, /* buffer: residual stream fp32 [T, d] after the MLP */
  DUOLM_STAGE_EMBED = 8      /* layer 0 only: residual stream fp32 [T, d] right after the gather */
} duolm_stage;

/*
 * Runs the embedding gather, layers 0 .. layer-1 in full, then layer `layer`
 * up to and including `stage`, for one batch, and copies the stage's buffer
 * (first T rows, row-major, the dtype listed above) into host_out.  Rows are
 * packed as the scoring call packs them: MIS mode [prefix_i, cands_i] per
 * request; independent mode [prefix_i, cand_ij] per (request, candidate).
 * layer == n_layers with stage DUOLM_STAGE_LAYER_OUT copies the final
 * residual stream.  The batch must fit one launch.  nbytes must equal the
 * buffer size; otherwise EINVAL.
 */
int duolm_debug_forward(duolm_ranker* r, const duolm_request* reqs, int32_t n_req, int32_t mode, int32_t layer,
                        int32_t stage, void* host_out, uint64_t nbytes);

/* Epilogues of the MFMA GEMM kernel. */
typedef enum {
  DUOLM_EPI_STORE_BF16 = 0, /* C bf16 [M, N] = A W^T */
  DUOLM_EPI_RESID_F32 = 1,  /* C fp32 [M, N] += A W^T */
  DUOLM_EPI_SWIGLU = 2      /* W rows interleaved in 32-row blocks (gate block p, up block p, ...);
                               C bf16 [M, N/2] = silu(gate) * up */
} duolm_epilogue;

/*
 * C = epilogue(A W^T) on device pointers with the library's bf16 MFMA GEMM.
 * A bf16 [M, K] row-major, W bf16 [N, K] row-major (nn.Linear layout).
 * Needs N % 64 == 0 and K % 64 == 0.  stream: hipStream_t or NULL.
 */
int duolm_debug_gemm(int32_t epilogue, const uint16_t* d_A, const uint16_t* d_W, void* d_C, int32_t M,
                     int32_t N, int32_t K, void* stream);

/* Plain device-to-device copy kernel (nbytes % 16 == 0), for byte-counter calibration. */
int duolm_copy_device(void* d_dst, const void* d_src, uint64_t nbytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DUOLM_DEBUG_H */
