/*
 * gpt_debug.h -- single-kernel entry points of libgpt.so for component
 * parity tests.  Not part of the forward-pass API; same conventions as
 * gpt.h (caller-owned device memory, asynchronous, validated on the host).
 */
#ifndef GPT_BLOCK_FWD_GPT_DEBUG_H
#define GPT_BLOCK_FWD_GPT_DEBUG_H

#include <stdint.h>
#include "gpt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogues of gpt_debug_gemm. */
enum { GPT_EPI_BF16 = 0, GPT_EPI_RELU2_BF16 = 1, GPT_EPI_RESID = 2, GPT_EPI_F32 = 3 };

/*
 * C = A W^T with A bf16 [M, K], W bf16 [N, K] (the projections of the
 * decoder block, [microgpt "Core architecture"] linear layers), fp32
 * accumulation, then the epilogue: store bf16, ReLU^2 then bf16
 * ([nanochat-launch tricks]), add into fp32 C (residual), or store fp32.
 * M <= 64 runs the decode-row kernel, larger M the tiled kernel.
 * ksplit: 1, or (M <= 64 and GPT_EPI_F32 only) 2 .. 16 and at most K / 64:
 * the k range is split over ksplit workgroups per column tile and C then
 * holds ksplit fp32 slabs [ksplit, M, N] of partial products whose sum is
 * A W^T (the form the decode step's consumers read).
 * Needs K % 64 == 0, N % 128 == 0, 16-byte aligned pointers.
 * Errors: GPT_ERR_ARG for NULL pointers, bad shapes, epilogue or ksplit.
 */
gpt_status gpt_debug_gemm(const void *A, const void *W, int32_t M, int32_t N, int32_t K, void *C,
                          int32_t epi, int32_t ksplit, gpt_stream_t stream);

/*
 * Causal MQA attention of packed sequences ([nanochat-forum]: multi-query
 * attention): q bf16 [total, H*128], k bf16 [total, 128], vt bf16
 * [128, ldvt] holding V transposed: position i of sequence b at column
 * cu_pad[b] + (i with bits 2 and 3 swapped), where cu_pad[b] = sum over
 * earlier sequences of their length rounded up to 64 (ldvt >= cu_pad[n_seqs],
 * multiple of 64).  The swap puts each lane's eight keys of the attention
 * MFMA in one 16-byte run; it is the layout the forward pass itself writes.
 * o bf16 [total, H*128].
 * cu_seqlens is a host array [n_seqs + 1]; cu_dev is a device int32 buffer
 * of 2*(n_seqs + 1) entries the call fills with cu_seqlens and cu_pad.
 * qk_norm != 0 promises QK-normalised q and k (RMS <= 1 per head, as the
 * forward pass leaves them): the softmax then runs against a fixed bound on
 * the scores instead of a running maximum; with qk_norm == 0 any q and k.
 */
gpt_status gpt_debug_attn_prefill(const void *q, const void *k, const void *vt, int64_t ldvt,
                                  const int32_t *cu_seqlens, int32_t n_seqs, int32_t n_head, int32_t qk_norm,
                                  int32_t *cu_dev, void *o, gpt_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif
