// Shared device-side types and helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define DEV __device__ __forceinline__

// Round-to-nearest-even conversion (gfx950 v_cvt_pk_bf16_f32).
DEV bf16 f2bf(float x) { return (bf16)x; }
DEV float bf2f(bf16 x) { return (float)x; }

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 2^x on the hardware exponential unit (v_exp_f32); exp(x) = 2^(x log2 e).
DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// Row metadata shared by the prefill kernels: for packed row m, its
// sequence, its 0-based position and its column in the per-sequence padded
// transposed-V buffer.
struct RowInfo {
  const int *seq;
  const int *pos;
  const int *vcol;
};

// Paged KV cache addressing (see include/gpt.h for the layout).
struct PagedKV {
  char *base;             // start of layer 0's pages
  const int *table;       // [n_seqs][pages_per_seq]
  int *lens;              // [n_seqs]
  long long layer_stride; // bytes per layer
  long long page_stride;  // bytes per page (K half + V half)
  long long half_bytes;   // bytes of the K half
  int pages_per_seq;
  int page_size;
};
