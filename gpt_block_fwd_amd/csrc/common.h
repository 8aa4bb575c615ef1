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

// ---------------------------------------------------------------- exchange between workgroups
// Within one kernel, values that one workgroup hands to another (split-K
// partials, the rows a last-arriving workgroup normalises, per-page attention
// partials) are written and read with relaxed agent-scope atomic accesses,
// which compile to sc1 loads and stores.  Each XCD has its own L2, and for
// ordinary device memory the eight are not kept coherent with one another;
// sc1 accesses are coherent across them by themselves.  Publishing therefore
// only needs the workgroup's own stores to have completed before its arrival
// is counted.  An acquire-release counter atomic would instead write back and
// invalidate the whole L2 of the XCD at every arrival, which costs tens of
// microseconds per launch.
DEV void xst(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV float xld(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Four consecutive floats, 16-byte aligned, as two 8-byte accesses.
DEV void xst4(float *p, f32x4 v) {
  unsigned long long *q = (unsigned long long *)p;
  const unsigned long long lo = (unsigned long long)__float_as_uint(v[0]) |
                                ((unsigned long long)__float_as_uint(v[1]) << 32);
  const unsigned long long hi = (unsigned long long)__float_as_uint(v[2]) |
                                ((unsigned long long)__float_as_uint(v[3]) << 32);
  __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV f32x4 xld4(const float *p) {
  unsigned long long *q = (unsigned long long *)const_cast<float *>(p);
  const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (f32x4){__uint_as_float((unsigned)lo), __uint_as_float((unsigned)(lo >> 32)),
                 __uint_as_float((unsigned)hi), __uint_as_float((unsigned)(hi >> 32))};
}
// Wait until this wave's stores have completed (and keep the compiler from
// moving memory accesses across the wait).
DEV void stores_done() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Count one arrival on *ctr (called by one lane, after every wave of the
// workgroup has passed stores_done and a barrier); returns the count before.
DEV unsigned arrive(unsigned *ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Row metadata shared by the prefill kernels: for packed row m, its
// sequence, its 0-based position and its column in the per-sequence padded
// transposed-V buffer.
struct RowInfo {
  const int *seq;
  const int *pos;
  const int *vcol;
};

// Column of cached position p (0 .. 63) in a page's transposed V rows.
// Within each 32-position half, position 16 a + 4 q + b (a < 2, q < 4,
// b < 4) sits at column 8 q + 4 a + b: the order in which the decode
// kernel's MFMA takes keys (k slot 8 q + j <-> key 16 (j / 4) + 4 q + j % 4),
// so one 16-byte load yields a lane's eight keys.
DEV int vslot(int p) { return (p & 32) | (((p >> 2) & 3) << 3) | (((p >> 4) & 1) << 2) | (p & 3); }

// Column of sequence position p (from the sequence's first column) in the
// prefill V^T buffer: bits 2 and 3 of p swapped, so within each 16-position
// group, position 8 a + 4 q + b (a, q < 2, b < 4) sits at column 8 q + 4 a + b.
// That is the order in which the prefill attention's 32x32x16 MFMA takes
// keys (k slot 8 q + j <-> key 8 (j / 4) + 4 q + j % 4 of the group), so one
// 16-byte load yields a lane's eight keys.  The map is its own inverse.
DEV int vperm16(int p) { return (p & ~15) | (((p >> 2) & 1) << 3) | (((p >> 3) & 1) << 2) | (p & 3); }

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
