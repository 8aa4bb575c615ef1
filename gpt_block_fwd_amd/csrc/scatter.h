// RoPE + QK-norm + bf16 scatter of one 128-wide head slot of one row, for
// one 64-lane wave.  Shared by the standalone scatter kernel and by the
// fused decode QKV GEMM.
#pragma once
#include "kernels.h"

// Lane l owns the rotary pair (l, l + 64) of head slot j of row m of the fp32
// q|k|v projections `u`: half-split rotation by the tabled angle of the row's
// position, then a weightless RMSNorm over the head (sum of squares reduced
// across the wave), then bf16 stores to q_out / k_out / vt_out and the paged
// cache.  V slots are only rounded and stored (V^T layout).
DEV void rope_norm_scatter_row(const ScatterArgs &a, const float *u, int m, int j, int lane) {
  float x0 = u[lane], x1 = u[lane + 64];
  const int p = a.pos[m];
  const int b = a.seq ? a.seq[m] : m;
  const bool is_v = j >= a.H + a.Hkv;
  if (!is_v) {
    if (a.cos) {
      const float c = a.cos[p * 64 + lane], s = a.sin[p * 64 + lane];
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
  if (a.use_cache) {
    const PagedKV &kv = a.kv;
    const int page = kv.table[b * kv.pages_per_seq + p / kv.page_size];
    const int slot = p % kv.page_size;
    char *pg = kv.base + (long long)a.layer * kv.layer_stride + (long long)page * kv.page_stride;
    if (!is_v) {
      bf16 *k = (bf16 *)pg + (long long)slot * kvd + g * 128;
      k[lane] = y0;
      k[lane + 64] = y1;
    } else {
      bf16 *vt = (bf16 *)(pg + kv.half_bytes);
      vt[(long long)(g * 128 + lane) * kv.page_size + slot] = y0;
      vt[(long long)(g * 128 + lane + 64) * kv.page_size + slot] = y1;
    }
  }
}

// Weightless RMSNorm of one fp32 row of width d into bf16, by one wave.
DEV void rmsnorm_row_bf16(const float *xr, bf16 *yr, int d, float eps, int lane) {
  float ss = 0.f;
  for (int c = lane * 4; c < d; c += 256) {
    const float4 v = *(const float4 *)(xr + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = lane * 4; c < d; c += 256) {
    const float4 v = *(const float4 *)(xr + c);
    bf16x4 o = {f2bf(v.x * rs), f2bf(v.y * rs), f2bf(v.z * rs), f2bf(v.w * rs)};
    *(bf16x4 *)(yr + c) = o;
  }
}
