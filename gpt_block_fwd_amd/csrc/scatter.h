// Per-row device helpers of the bf16 path, each run by one 64-lane wave:
// RoPE + QK-norm + bf16 scatter of one 128-wide head slot, and RMSNorm of
// one fp32 row into bf16.
#pragma once
#include "kernels.h"

// Lane l owns the rotary pair (l, l + 64) of head slot j, values (x0, x1)
// of the fp32 q|k|v projections.  Query and key slots: half-split rotation
// by the angle of the row's position (table factors c, s), then a weightless
// RMSNorm over the head (sum of squares reduced across the wave).  V slots
// are left as they are.
DEV void rope_norm_pair(const ScatterArgs &a, float &x0, float &x1, float c, float s, int j) {
  if (j >= a.H + a.Hkv) return;
  if (a.cos) {
    const float r0 = x0 * c - x1 * s, r1 = x0 * s + x1 * c;
    x0 = r0;
    x1 = r1;
  }
  if (a.qk_norm) {
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float rs = 1.0f / sqrtf(ss * (1.0f / 128.0f) + a.eps);
    x0 *= rs;
    x1 *= rs;
  }
}

// The bf16 pair (y0, y1) of K slot (j < H + Hkv) or V slot j of position p
// into the paged cache (page index `page` of the sequence's block table).
DEV void cache_store_pair(const ScatterArgs &a, bf16 y0, bf16 y1, int p, int page, int j, int lane) {
  const bool is_v = j >= a.H + a.Hkv;
  const int g = is_v ? j - a.H - a.Hkv : j - a.H;
  const int kvd = a.Hkv * 128;
  const PagedKV &kv = a.kv;
  const int slot = p % kv.page_size;
  char *pg = kv.base + (long long)a.layer * kv.layer_stride + (long long)page * kv.page_stride;
  if (!is_v) {
    bf16 *k = (bf16 *)pg + (long long)slot * kvd + g * 128;
    k[lane] = y0;
    k[lane + 64] = y1;
  } else {
    bf16 *vt = (bf16 *)(pg + kv.half_bytes);
    vt[(long long)(g * 128 + lane) * kv.page_size + vslot(slot)] = y0;
    vt[(long long)(g * 128 + lane + 64) * kv.page_size + vslot(slot)] = y1;
  }
}

// The pair (l, l + 64) of slot values at u in each partial slab of a split
// GEMM (nslab <= 1: one slab), loaded, then summed in slab order.
struct SlabPair {
  float v[kMaxRowSplit][2];
};
DEV void slab_load(const ScatterArgs &a, const float *u, int lane, SlabPair &t) {
  // 32-bit offsets (the slabs of at most 64 rows are far below 2^31 / 16
  // floats): a scalar slab offset plus the lane, no 64-bit address math
  const int st = (int)a.slab;
#pragma unroll
  for (int k = 0; k < kMaxRowSplit; ++k)
    if (k == 0 || k < a.nslab) {
      t.v[k][0] = u[k * st + lane];
      t.v[k][1] = u[k * st + lane + 64];
    }
}
DEV void slab_sum(const ScatterArgs &a, const SlabPair &t, float &x0, float &x1) {
  x0 = t.v[0][0];
  x1 = t.v[0][1];
#pragma unroll
  for (int k = 1; k < kMaxRowSplit; ++k)
    if (k < a.nslab) {
      x0 += t.v[k][0];
      x1 += t.v[k][1];
    }
}
DEV void slab_pair(const ScatterArgs &a, const float *u, int lane, float &x0, float &x1) {
  SlabPair t;
  slab_load(a, u, lane, t);
  slab_sum(a, t, x0, x1);
}

// RoPE + QK-norm of head slot j of row m, then bf16 stores to q_out /
// k_out / vt_out and the paged cache.  V slots are only rounded and stored
// (V^T layout).
DEV void rope_norm_scatter_vals(const ScatterArgs &a, float x0, float x1, float c, float s, int p, int page,
                                int m, int j, int lane) {
  rope_norm_pair(a, x0, x1, c, s, j);
  const bool is_v = j >= a.H + a.Hkv;
  const bf16 y0 = f2bf(x0), y1 = f2bf(x1);
  if (j < a.H) {
    bf16 *q = (bf16 *)a.q_out + (long long)m * a.H * 128 + j * 128;
    q[lane] = y0;
    q[lane + 64] = y1;
    return;
  }
  const int g = is_v ? j - a.H - a.Hkv : j - a.H;
  const int kvd = a.Hkv * 128;
  if (!is_v) {
    if (a.k_out) {
      bf16 *k = (bf16 *)a.k_out + (long long)m * kvd + g * 128;
      k[lane] = y0;
      k[lane + 64] = y1;
    }
  } else if (a.vt_out) {
    bf16 *vt = (bf16 *)a.vt_out;
    const long long col = a.vcol ? a.vcol[m] : m;
    vt[(long long)(g * 128 + lane) * a.ldvt + col] = y0;
    vt[(long long)(g * 128 + lane + 64) * a.ldvt + col] = y1;
  }
  if (a.use_cache) cache_store_pair(a, y0, y1, p, page, j, lane);
}

DEV int scatter_page(const ScatterArgs &a, int m, int p) {
  if (!a.use_cache) return 0;
  const int b = a.seq ? a.seq[m] : m;
  return a.kv.table[b * a.kv.pages_per_seq + p / a.kv.page_size];
}

// One row, values read from u (written by an earlier kernel), summed over
// the partial slabs of a split GEMM.
DEV void rope_norm_scatter_row(const ScatterArgs &a, const float *u, int m, int j, int lane) {
  float x0, x1;
  slab_pair(a, u, lane, x0, x1);
  const int p = a.pos[m];
  float c = 0.f, s = 0.f;
  if (a.cos && j < a.H + a.Hkv) {
    c = a.cos[p * 64 + lane];
    s = a.sin[p * 64 + lane];
  }
  rope_norm_scatter_vals(a, x0, x1, c, s, p, scatter_page(a, m, p), m, j, lane);
}

// Weightless RMSNorm of one fp32 row of width d into bf16, by one wave.
DEV void rmsnorm_row_bf16(const float *xr, bf16 *yr, int d, float eps, int lane) {
  float ss = 0.f;
  for (int c = lane * 4; c < d; c += 256) {
    const f32x4 v = *(const f32x4 *)(xr + c);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = lane * 4; c < d; c += 256) {
    const f32x4 v = *(const f32x4 *)(xr + c);
    bf16x4 o = {f2bf(v[0] * rs), f2bf(v[1] * rs), f2bf(v[2] * rs), f2bf(v[3] * rs)};
    *(bf16x4 *)(yr + c) = o;
  }
}
