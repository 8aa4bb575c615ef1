/*
 * gpt_profile.h -- optional per-kernel-class timing of libgpt.so.
 *
 * Not part of the method: a measurement aid.  When a class is enabled, the
 * library records a pair of HIP events on the launch stream around every
 * kernel launch of that class and notes the launch's algorithmic work
 * (floating-point operations and the bytes the operation must move at
 * least once: operands read, results written).  Reading synchronises on the
 * recorded events.  Disabled classes add no work.  Not thread-safe.
 */
#ifndef GPT_BLOCK_FWD_GPT_PROFILE_H
#define GPT_BLOCK_FWD_GPT_PROFILE_H

#include <stdint.h>
#include "gpt.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT_PROF_GEMM = 0,        /* prefill block GEMMs: QKV, O, MLP up, MLP down */
  GPT_PROF_LMHEAD = 1,      /* LM-head GEMM (prefill and decode) */
  GPT_PROF_ATTN = 2,        /* prefill causal attention */
  GPT_PROF_DECODE_ATTN = 3, /* decode split-KV attention + combine */
  GPT_PROF_SKINNY = 4,      /* decode block GEMMs (M = sequences) */
  GPT_PROF_NORM = 5,        /* RMSNorm, RoPE/QK-norm scatter, embedding */
  GPT_PROF_SOFTMAX = 6,     /* vocabulary softmax / LSE and token selection */
  GPT_PROF_OPTIM = 7,       /* optimiser update (Adam) */
  GPT_PROF_BWD_GEMM = 8,    /* loss backward: GEMMs (weight and input gradients, recomputed projections) */
  GPT_PROF_BWD_ATTN = 9,    /* loss backward: attention */
  GPT_PROF_BWD_OTHER = 10,  /* loss backward: transposes, norms, activations, RoPE, logits, embeddings */
  GPT_PROF_NCLASSES = 11
} gpt_prof_class;

/* Enable timing for the classes whose bit (1 << class) is set in mask; 0
 * disables.  Clears every accumulated record. */
gpt_status gpt_profile_enable(uint32_t mask);

/* Change which classes are timed without clearing the records, so that a
 * long run can be sampled (for instance every eighth decode step) and the
 * number of HIP events stays bounded. */
gpt_status gpt_profile_mask(uint32_t mask);

/* Totals since the last enable for one class: summed kernel time in
 * milliseconds, number of launches, algorithmic flops and bytes. */
gpt_status gpt_profile_read(int32_t cls, double *ms, int64_t *launches, double *flops,
                            double *bytes);

/* The launch with index i (0-based, in launch order) among those of class
 * cls recorded since the last enable: its kernel time in milliseconds and
 * its algorithmic flops and bytes, so that launches of different shapes can
 * be told apart.  NULL outputs are skipped.  GPT_ERR_ARG for a bad class, or
 * when fewer than i + 1 launches of the class are recorded. */
gpt_status gpt_profile_read_launch(int32_t cls, int64_t i, double *ms, double *flops, double *bytes);

#ifdef __cplusplus
}
#endif
#endif
