// RoPE + QK-norm + bf16 scatter of one 128-wide head slot of one row, for
// one 64-lane wave.  Shared by the standalone scatter kernel and by the
// fused decode QKV GEMM.
#pragma once
#include "kernels.h"

// Lane l owns the rotary pair (l, l + 64) of head slot j of row m, values
// (x0, x1) of the fp32 q|k|v projections: half-split rotation by the angle
// of the row's position p (table factors c, s), then a weightless RMSNorm
// over the head (sum of squares reduced across the wave), then bf16 stores
// to q_out / k_out / vt_out and the paged cache (page index `page` of the
// sequence's block table).  V slots are only rounded and stored (V^T layout).
DEV void rope_norm_scatter_vals(const ScatterArgs &a, float x0, float x1, float c, float s, int p, int page,
                                int m, int j, int lane) {
  const bool is_v = j >= a.H + a.Hkv;
  if (!is_v) {
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

DEV int scatter_page(const ScatterArgs &a, int m, int p) {
  if (!a.use_cache) return 0;
  const int b = a.seq ? a.seq[m] : m;
  return a.kv.table[b * a.kv.pages_per_seq + p / a.kv.page_size];
}

// One row, values read from u (written by an earlier kernel).
DEV void rope_norm_scatter_row(const ScatterArgs &a, const float *u, int m, int j, int lane) {
  const float x0 = u[lane], x1 = u[lane + 64];
  const int p = a.pos[m];
  float c = 0.f, s = 0.f;
  if (a.cos && j < a.H + a.Hkv) {
    c = a.cos[p * 64 + lane];
    s = a.sin[p * 64 + lane];
  }
  rope_norm_scatter_vals(a, x0, x1, c, s, p, scatter_page(a, m, p), m, j, lane);
}

// Rows r0, r0 + rstep, ... < M of head slot j, values at U + r * ldu
// written by other workgroups of the same kernel.  Four rows at a time, the
// loads of every row are issued together, in two dependent rounds (values
// and positions, then table factors and pages), before any row is finished.
DEV void rope_norm_scatter_rows_xwg(const ScatterArgs &a, const float *U, int ldu, int M, int j, int r0,
                                    int rstep, int lane) {
  constexpr int R = 4;
  for (; r0 < M; r0 += R * rstep) {
    float x0[R], x1[R], c[R], s[R];
  int p[R], page[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = r0 + i * rstep;
    if (r < M) {
      x0[i] = xld(U + (long long)r * ldu + lane);
      x1[i] = xld(U + (long long)r * ldu + lane + 64);
      p[i] = a.pos[r];
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = r0 + i * rstep;
    c[i] = s[i] = 0.f;
    page[i] = 0;
    if (r < M) {
      if (a.cos && j < a.H + a.Hkv) {
        c[i] = a.cos[p[i] * 64 + lane];
        s[i] = a.sin[p[i] * 64 + lane];
      }
      if (j >= a.H) page[i] = scatter_page(a, r, p[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = r0 + i * rstep;
    if (r < M) rope_norm_scatter_vals(a, x0[i], x1[i], c[i], s[i], p[i], page[i], r, j, lane);
  }
  }
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

// The same normalisation for rows r0, r0 + rstep, ... < M of X (row stride
// ldx, written by other workgroups of the same kernel) into Y (row stride
// ldy), by one wave.  CPL = ceil(d / 256) four-float chunks per lane and
// row; the loads of R rows are all issued before the first is reduced.
// The per-lane order of the sum of squares is that of rmsnorm_row_bf16.
template <int CPL>
DEV void rmsnorm_rows_xwg(const float *X, int ldx, bf16 *Y, int ldy, int M, int d, float eps, int r0,
                          int rstep, int lane) {
  constexpr int R = CPL >= 12 ? 1 : 12 / CPL;
  for (int rb = r0; rb < M; rb += R * rstep) {
    f32x4 v[R][CPL];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int r = rb + i * rstep, col = (c * 64 + lane) * 4;
        v[i][c] = (r < M && col < d) ? xld4(X + (long long)r * ldx + col) : (f32x4){};
      }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) ss += v[i][c][0] * v[i][c][0] + v[i][c][1] * v[i][c][1] +
                                          v[i][c][2] * v[i][c][2] + v[i][c][3] * v[i][c][3];
      ss = wave_sum(ss);
      const float rs = 1.0f / sqrtf(ss / (float)d + eps);
      const int r = rb + i * rstep;
      if (r >= M) continue;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int col = (c * 64 + lane) * 4;
        if (col < d) {
          bf16x4 o = {f2bf(v[i][c][0] * rs), f2bf(v[i][c][1] * rs), f2bf(v[i][c][2] * rs), f2bf(v[i][c][3] * rs)};
          *(bf16x4 *)(Y + (long long)r * ldy + col) = o;
        }
      }
    }
  }
}
