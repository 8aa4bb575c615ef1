// Kernels of the loss backward: the gradient of the mean next-token
// cross-entropy with respect to every weight.  The matrix products run on
// the forward's GEMM kernels (fed with transposed bf16 or fp32 copies made
// here); this file holds the elementwise, normalisation, attention and
// scatter steps between them.  Every kernel computes in fp32.
#include <algorithm>

#include "kernels.h"

namespace {

template <typename T>
DEV float ld(const T *p) {
  if constexpr (std::is_same<T, bf16>::value) return bf2f(*p);
  else return *p;
}
template <typename T>
DEV T cvt(float x) {
  if constexpr (std::is_same<T, bf16>::value) return f2bf(x);
  else return x;
}

// ---------------------------------------------------------------- transpose
// dst[c][r] = src[r][c] for r < R, c < C; columns R .. Rp of dst are zero.
// 64x64 tiles through LDS (padded rows: no bank conflicts on the column
// reads).
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void transpose_kernel(const TI *src, long long lds, int R, int C, TO *dst,
                                                        long long ldd, int Rp) {
  __shared__ float t[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < R && c < C) ? ld(src + (long long)r * lds + c) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) dst[(long long)c * ldd + r] = cvt<TO>(t[tx][i]);
  }
}

// The same into bf16 through a 64 x 64 LDS tile with 16-byte global
// accesses both ways (C % 64 == 0; lds, ldd, Rp multiples of 8; 16-byte
// aligned bases).  Reads: 8 lanes cover one source row's 64 columns.
// Writes: 8 lanes cover one destination row's 64 entries, 8 rows per wave
// instruction, so every store instruction writes whole 128-byte lines.
// RELU2: the source is the MLP pre-activation z, the value moved relu(z)^2.
template <typename TI, bool RELU2 = false>
__global__ __launch_bounds__(256) void transpose16_kernel(const TI *src, long long lds, int R, int C, bf16 *dst,
                                                          long long ldd, int Rp) {
  constexpr int P = 66;  // row pitch in bf16
  __shared__ bf16 t[64 * P];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + 256 * k, row = i >> 3, ch = i & 7, r = r0 + row;
    float v[8];
    if (r < R) {
      const TI *p = src + (long long)r * lds + c0 + 8 * ch;
      if constexpr (std::is_same<TI, bf16>::value) {
        const bf16x8 x = *(const bf16x8 *)p;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf2f(x[e]);
      } else {
        const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = a[e];
          v[4 + e] = b[e];
        }
      }
      if constexpr (RELU2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float q = fmaxf(v[e], 0.f);
          v[e] = q * q;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) t[row * P + 8 * ch + e] = f2bf(v[e]);
  }
  __syncthreads();
  const int rc = tid & 7, r = r0 + 8 * rc;  // destination entries r .. r + 7
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int col = (tid >> 3) + 32 * k;      // destination row c0 + col
    if (r >= Rp) continue;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = t[(8 * rc + e) * P + col];
    *(bf16x8 *)(dst + (long long)(c0 + col) * ldd + r) = o;
  }
}

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void cast_kernel(const TI *src, TO *dst, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    dst[i] = cvt<TO>(ld(src + i));
}

// ---------------------------------------------------------------- RMSNorm backward
// y = x / r, r = sqrt(mean(x^2) + eps): dx += (dy - y mean(dy y)) / r.
// One wave per row.
__global__ __launch_bounds__(256) void rms_bwd_kernel(const float *x, const float *dy, float *dx, bf16 *dxb, int M,
                                                      int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  const float *xr = x + (long long)row * d, *gr = dy + (long long)row * d;
  float ss = 0.f, sg = 0.f;
  for (int c = lane; c < d; c += 64) {
    const float v = xr[c];
    ss += v * v;
    sg += gr[c] * v;
  }
  ss = wave_sum(ss);
  sg = wave_sum(sg);
  const float r = sqrtf(ss / d + eps), inv = 1.0f / r;
  // mean(dy y) = sum(dy x) / (d r)
  const float m = sg * inv / d;
  float *o = dx + (long long)row * d;
  bf16 *ob = dxb ? dxb + (long long)row * d : nullptr;
  for (int c = lane; c < d; c += 64) {
    const float v = o[c] + (gr[c] - xr[c] * inv * m) * inv;
    o[c] = v;
    if (ob) ob[c] = f2bf(v);
  }
}

// The same with 16-byte accesses, the row held in registers between the two
// passes: lane l takes floats 256 c + 4 l .. +3 of each 256-float chunk c
// (NC chunks, d <= 256 NC, d % 4 == 0).
template <int NC>
__global__ __launch_bounds__(256) void rms_bwd4_kernel(const float *x, const float *dy, float *dx, bf16 *dxb,
                                                       int M, int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  const long long base = (long long)row * d;
  f32x4 xv[NC], gv[NC];
  float ss = 0.f, sg = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = 256 * c + 4 * lane;
    if (i < d) {
      xv[c] = *(const f32x4 *)(x + base + i);
      gv[c] = *(const f32x4 *)(dy + base + i);
    } else {
      xv[c] = (f32x4){};
      gv[c] = (f32x4){};
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss += xv[c][e] * xv[c][e];
      sg += gv[c][e] * xv[c][e];
    }
  }
  ss = wave_sum(ss);
  sg = wave_sum(sg);
  const float r = sqrtf(ss / d + eps), inv = 1.0f / r;
  const float m = sg * inv / d;  // mean(dy y)
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = 256 * c + 4 * lane;
    if (i >= d) continue;
    f32x4 v = *(const f32x4 *)(dx + base + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += (gv[c][e] - xv[c][e] * inv * m) * inv;
    *(f32x4 *)(dx + base + i) = v;
    if (dxb) *(bf16x4 *)(dxb + base + i) = (bf16x4){f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])};
  }
}

// ---------------------------------------------------------------- MLP activation
// u = act(z) and dz = du act'(z): ReLU^2 (2 max(z, 0)) or ReLU ([z > 0]).
template <typename T>
__global__ __launch_bounds__(256) void act_bwd_kernel(const float *z, const float *du, T *u, T *dz, long long n,
                                                      int relu2) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const float r = fmaxf(z[i], 0.f);
    if (u) u[i] = cvt<T>(relu2 ? r * r : r);
    if (dz) dz[i] = cvt<T>(relu2 ? 2.f * r * du[i] : (z[i] > 0.f ? du[i] : 0.f));
  }
}

// ---------------------------------------------------------------- RoPE + QK-norm backward
// One wave per (row, slot): slots 0 .. H-1 query heads, H .. H+Hkv-1 key
// heads, then value heads.  pre: the projection output [M][(H+2Hkv) dh]
// (fp32).  For q and k the forward was u = R pre (RoPE), y = u / rms(u);
// here du = (dy - y mean(dy y)) / rms, dpre = R^T du.  v passes through.
template <typename T>
__global__ __launch_bounds__(256) void qkv_bwd_kernel(QkvBwdArgs a, T *dqkv) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int slots = a.H + 2 * a.Hkv;
  if (item >= a.M * slots) return;
  const int m = item / slots, j = item - m * slots;
  const int dh = a.dh, half = dh / 2, nq = a.H * dh;
  const float *pre = a.pre + (long long)m * slots * dh + j * dh;
  T *out = dqkv + (long long)m * slots * dh + j * dh;
  const float *dy;
  if (j < a.H) dy = a.dq + (long long)m * nq + j * dh;
  else if (j < a.H + a.Hkv) dy = a.dk + (long long)m * a.Hkv * dh + (j - a.H) * dh;
  else dy = a.dv + (long long)m * a.Hkv * dh + (j - a.H - a.Hkv) * dh;
  if (j >= a.H + a.Hkv) {
    for (int c = lane; c < dh; c += 64) out[c] = cvt<T>(dy[c]);
    return;
  }
  const int p = a.pos[m];
  // lane handles pair i = lane (dims i and i + dh/2), dh <= 128
  const bool has = lane < half;
  float u0 = 0.f, u1 = 0.f, c = 1.f, s = 0.f;
  if (has) {
    const float x0 = pre[lane], x1 = pre[lane + half];
    if (a.cos) {
      c = a.cos[(long long)p * half + lane];
      s = a.sin[(long long)p * half + lane];
    }
    u0 = x0 * c - x1 * s;
    u1 = x0 * s + x1 * c;
  }
  float g0 = has ? dy[lane] : 0.f, g1 = has ? dy[lane + half] : 0.f;
  if (a.qk_norm) {
    const float ss = wave_sum(u0 * u0 + u1 * u1);
    const float r = sqrtf(ss / dh + a.eps), inv = 1.0f / r;
    const float sg = wave_sum(g0 * u0 + g1 * u1);  // sum(dy u)
    const float mdy = sg * inv / dh;               // mean(dy y)
    g0 = (g0 - u0 * inv * mdy) * inv;
    g1 = (g1 - u1 * inv * mdy) * inv;
  }
  if (has) {
    out[lane] = cvt<T>(g0 * c + g1 * s);
    out[lane + half] = cvt<T>(-g0 * s + g1 * c);
  }
}

// ---------------------------------------------------------------- attention backward
// 16 lanes per item, each lane 8 of the head's dims (dh <= 128).
DEV float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

// Row-parallel: item = (row m, query head h); 4 items per wave.  Pass 1:
// the row's log-sum-exp over its visible keys; pass 2: P, dP = dO . v,
// dS = P (dP - D) with D = dO . O, and dq = scale sum_j dS_j k_j.  Writes
// dq, and the row's lse and D for the key-parallel kernel.
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_rows_kernel(AttnBwdArgs a) {
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const long long item = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  if (item >= (long long)a.M * a.H) return;
  const int m = (int)(item / a.H), h = (int)(item - (long long)m * a.H);
  const int dh = a.dh, g = h * a.Hkv / a.H, kvd = a.Hkv * dh;
  const int p = a.pos[m], r0 = m - p;
  const T *q = (const T *)a.q + (long long)m * a.H * dh + h * dh;
  const T *o = (const T *)a.o + (long long)m * a.H * dh + h * dh;
  const float *gO = a.dout + (long long)m * a.H * dh + h * dh;
  float qr[8], dor[8], dq[8];
  float D = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = l16 + 16 * i;
    qr[i] = c < dh ? ld(q + c) : 0.f;
    dor[i] = c < dh ? gO[c] : 0.f;
    D += c < dh ? dor[i] * ld(o + c) : 0.f;
    dq[i] = 0.f;
  }
  D = sum16(D);
  const float scale = 1.0f / sqrtf((float)dh);
  float mx = -INFINITY, l = 0.f;
  for (int j = 0; j <= p; ++j) {
    const T *k = (const T *)a.k + (long long)(r0 + j) * kvd + g * dh;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = l16 + 16 * i;
      if (c < dh) s += qr[i] * ld(k + c);
    }
    s = sum16(s) * scale;
    const float mn = fmaxf(mx, s);
    l = l * expf(mx - mn) + expf(s - mn);
    mx = mn;
  }
  const float lse = mx + logf(l);
  for (int j = 0; j <= p; ++j) {
    const T *k = (const T *)a.k + (long long)(r0 + j) * kvd + g * dh;
    const float *v = a.v + (long long)(r0 + j) * a.ldv + g * dh;
    float s = 0.f, dp = 0.f;
    float kr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = l16 + 16 * i;
      kr[i] = c < dh ? ld(k + c) : 0.f;
      float vv = c < dh ? v[c] : 0.f;
      if (a.v_bf16) vv = bf2f(f2bf(vv));
      s += qr[i] * kr[i];
      dp += dor[i] * vv;
    }
    s = sum16(s) * scale;
    dp = sum16(dp);
    const float P = expf(s - lse);
    const float ds = P * (dp - D) * scale;
#pragma unroll
    for (int i = 0; i < 8; ++i) dq[i] += ds * kr[i];
  }
  float *dqo = a.dq + (long long)m * a.H * dh + h * dh;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = l16 + 16 * i;
    if (c < dh) dqo[c] = dq[i];
  }
  if (l16 == 0) {
    a.lse[(long long)m * a.H + h] = lse;
    a.dsum[(long long)m * a.H + h] = D;
  }
}

// Key-parallel: item = (key row j, K/V head g); 4 items per wave.  For every
// query head of the group and every row r >= j of the sequence:
// dk += scale dS q_r, dv += P dO_r.
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_keys_kernel(AttnBwdArgs a) {
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const long long item = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  if (item >= (long long)a.M * a.Hkv) return;
  const int j = (int)(item / a.Hkv), g = (int)(item - (long long)j * a.Hkv);
  const int dh = a.dh, kvd = a.Hkv * dh, G = a.H / a.Hkv;
  const int end = a.cu[a.seq[j] + 1];  // the sequence's rows end before this one
  const T *k = (const T *)a.k + (long long)j * kvd + g * dh;
  const float *v = a.v + (long long)j * a.ldv + g * dh;
  float kr[8], vr[8], dk[8], dv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = l16 + 16 * i;
    kr[i] = c < dh ? ld(k + c) : 0.f;
    float vv = c < dh ? v[c] : 0.f;
    if (a.v_bf16) vv = bf2f(f2bf(vv));
    vr[i] = vv;
    dk[i] = dv[i] = 0.f;
  }
  const float scale = 1.0f / sqrtf((float)dh);
  for (int hh = g * G; hh < g * G + G; ++hh) {
    for (int r = j; r < end; ++r) {
      const T *q = (const T *)a.q + (long long)r * a.H * dh + hh * dh;
      const float *gO = a.dout + (long long)r * a.H * dh + hh * dh;
      float qr[8], dor[8], s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = l16 + 16 * i;
        qr[i] = c < dh ? ld(q + c) : 0.f;
        dor[i] = c < dh ? gO[c] : 0.f;
        s += qr[i] * kr[i];
        dp += dor[i] * vr[i];
      }
      s = sum16(s) * scale;
      dp = sum16(dp);
      const float P = expf(s - a.lse[(long long)r * a.H + hh]);
      const float ds = P * (dp - a.dsum[(long long)r * a.H + hh]) * scale;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dk[i] += ds * qr[i];
        dv[i] += P * dor[i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = l16 + 16 * i;
    if (c < dh) {
      a.dk[(long long)j * kvd + g * dh + c] = dk[i];
      a.dv[(long long)j * kvd + g * dh + c] = dv[i];
    }
  }
}

// dst[m][c] = bf16(src[m lds + c]), c < C
__global__ __launch_bounds__(256) void cast_rows_kernel(const float *src, long long lds, int M, int C, bf16 *dst) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)M * C) return;
  const int m = (int)(i / C), c = (int)(i - (long long)m * C);
  dst[i] = f2bf(src[(long long)m * lds + c]);
}

// ---------------------------------------------------------------- cross-entropy gradient
// dlogits[r][v] = (exp(logits[r][v] - lse[r]) - [v == t_r]) / count for rows
// with a target in [0, V) (count read from the device), 0 otherwise.
template <typename T>
__global__ __launch_bounds__(256) void dlogits_kernel(const float *logits, const float *lse, const int *targets,
                                                      const int *count, int V, T *dl) {
  const int r = blockIdx.x;
  const int t = targets[r];
  const bool ok = t >= 0 && t < V;
  const float inv = 1.0f / (float)max(*count, 1), l = lse[r];
  const float *row = logits + (long long)r * V;
  T *out = dl + (long long)r * V;
  for (int v = threadIdx.x; v < V; v += 256) {
    const float gd = ok ? (expf(row[v] - l) - (v == t ? 1.f : 0.f)) * inv : 0.f;
    out[v] = cvt<T>(gd);
  }
}

// Softmax gradient of the LM head from bf16 logits, in both layouts the
// backward's GEMMs take: dl[m][v] = (exp(z[m][v] - lse[m]) - [v == t_m]) /
// count (zero for rows without a target) row-major [M][V], and transposed
// [V][ldt] with columns M .. Rp - 1 zero.  A workgroup takes 64 rows and
// kDlCols columns in 64 x 64 tiles: a thread reads 8 consecutive logits of
// one row (8 lanes per 128-byte line) and writes its 8 gradients straight
// back; each tile passes through LDS for the transposed copy, whose stores
// also cover whole lines (8 lanes per destination row).  The rows' lse,
// target and validity are loaded once per workgroup.
constexpr int kDlCols = 256;
__global__ __launch_bounds__(256) void dlogits_t_kernel(const bf16 *z, const float *lse, const int *targets,
                                                        const int *count, int M, int V, bf16 *dl, bf16 *dlt,
                                                        long long ldt, int Rp) {
  constexpr int P = 66;  // row pitch in bf16
  __shared__ bf16 t[64 * P];
  const int r0 = blockIdx.y * 64, tid = threadIdx.x;
  const float inv = 1.0f / (float)max(*count, 1);
  // this thread's two source rows
  int tg[2];
  float l2[2];  // lse in the base-2 domain
  bool ok[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = r0 + ((tid + 256 * k) >> 3);
    tg[k] = r < M ? targets[r] : -1;
    ok[k] = r < M && tg[k] >= 0 && tg[k] < V;
    l2[k] = r < M ? lse[r] * kLog2e : 0.f;
  }
  const int rc = tid & 7, rd = r0 + 8 * rc;  // destination entries rd .. rd + 7
  for (int c0 = blockIdx.x * kDlCols; c0 < min(V, (int)(blockIdx.x + 1) * kDlCols); c0 += 64) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + 256 * k, row = i >> 3, ch = i & 7, r = r0 + row;
      bf16x8 o;
      if (r < M) {
        const long long off = (long long)r * V + c0 + 8 * ch;
        const bf16x8 x = *(const bf16x8 *)(z + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = c0 + 8 * ch + e;
          // exp(z - lse) = 2^(z log2 e - lse log2 e)
          o[e] = f2bf(ok[k] ? (fast_exp2(bf2f(x[e]) * kLog2e - l2[k]) - (v == tg[k] ? 1.f : 0.f)) * inv : 0.f);
        }
        *(bf16x8 *)(dl + off) = o;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) t[row * P + 8 * ch + e] = o[e];
    }
    __syncthreads();
    if (rd < Rp) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int col = (tid >> 3) + 32 * k;  // destination row c0 + col
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = t[(8 * rc + e) * P + col];
        *(bf16x8 *)(dlt + (long long)(c0 + col) * ldt + rd) = w;
      }
    }
    __syncthreads();  // the tile is read before the next one overwrites it
  }
}

// ---------------------------------------------------------------- embedding backward
// dwte[tokens[m]] += dx[m] (and dwpe[pos[m]] += dx[m]): one thread per
// element, fp32 atomics (several rows may share a token).
__global__ __launch_bounds__(256) void embed_bwd_kernel(const int *tokens, const int *pos, const float *dx,
                                                        float *dwte, float *dwpe, int M, int d) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)M * d) return;
  const int m = (int)(i / d), c = (int)(i - (long long)m * d);
  atomicAdd(dwte + (long long)tokens[m] * d + c, dx[i]);
  if (dwpe) atomicAdd(dwpe + (long long)pos[m] * d + c, dx[i]);
}

__global__ __launch_bounds__(256) void count_targets_kernel(const int *targets, int M, int V, int *count) {
  __shared__ int s[256];
  int c = 0;
  for (int r = threadIdx.x; r < M; r += 256) c += (targets[r] >= 0 && targets[r] < V);
  s[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *count = s[0];
}

unsigned grid_for(long long n) { return (unsigned)std::max(1LL, std::min((n + 255) / 256, 8192LL)); }

}  // namespace

template <typename TI, typename TO>
void launch_transpose(const TI *src, long long lds, int R, int C, TO *dst, long long ldd, int Rp, hipStream_t s) {
  if (R <= 0 || C <= 0) return;
  const dim3 grid((C + 63) / 64, (std::max(R, Rp) + 63) / 64);
  if constexpr (std::is_same<TO, bf16>::value) {
    if (C % 64 == 0 && ldd % 8 == 0 && Rp % 8 == 0 && lds % 8 == 0 &&
        (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      transpose16_kernel<TI><<<grid, 256, 0, s>>>(src, lds, R, C, dst, ldd, Rp);
      return;
    }
  }
  transpose_kernel<TI, TO><<<grid, 256, 0, s>>>(src, lds, R, C, dst, ldd, Rp);
}
template void launch_transpose<float, bf16>(const float *, long long, int, int, bf16 *, long long, int, hipStream_t);
template void launch_transpose<bf16, bf16>(const bf16 *, long long, int, int, bf16 *, long long, int, hipStream_t);
template void launch_transpose<float, float>(const float *, long long, int, int, float *, long long, int, hipStream_t);

void launch_transpose_relu2(const float *z, long long lds, int R, int C, bf16 *dst, long long ldd, int Rp,
                            hipStream_t s) {
  if (R <= 0 || C <= 0) return;
  const dim3 grid((C + 63) / 64, (std::max(R, Rp) + 63) / 64);
  transpose16_kernel<float, true><<<grid, 256, 0, s>>>(z, lds, R, C, dst, ldd, Rp);
}

template <typename TI, typename TO>
void launch_cast(const TI *src, TO *dst, long long n, hipStream_t s) {
  if (n > 0) cast_kernel<TI, TO><<<grid_for(n), 256, 0, s>>>(src, dst, n);
}
template void launch_cast<float, bf16>(const float *, bf16 *, long long, hipStream_t);
template void launch_cast<float, float>(const float *, float *, long long, hipStream_t);

void launch_rms_bwd(const float *x, const float *dy, float *dx, bf16 *dxb, int M, int d, float eps, hipStream_t s) {
  if (M <= 0) return;
  const unsigned grid = (unsigned)((M + 3) / 4);
  if (d % 4 == 0 && d <= 2048) {
    switch ((d + 255) / 256) {
      case 1: rms_bwd4_kernel<1><<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps); return;
      case 2: rms_bwd4_kernel<2><<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps); return;
      case 3: rms_bwd4_kernel<3><<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps); return;
      case 4: rms_bwd4_kernel<4><<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps); return;
      case 5: rms_bwd4_kernel<5><<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps); return;
      case 6: rms_bwd4_kernel<6><<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps); return;
      case 7: rms_bwd4_kernel<7><<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps); return;
      default: rms_bwd4_kernel<8><<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps); return;
    }
  }
  rms_bwd_kernel<<<grid, 256, 0, s>>>(x, dy, dx, dxb, M, d, eps);
}

template <typename T>
void launch_act_bwd(const float *z, const float *du, T *u, T *dz, long long n, int relu2, hipStream_t s) {
  if (n > 0) act_bwd_kernel<T><<<grid_for(n), 256, 0, s>>>(z, du, u, dz, n, relu2);
}
template void launch_act_bwd<bf16>(const float *, const float *, bf16 *, bf16 *, long long, int, hipStream_t);
template void launch_act_bwd<float>(const float *, const float *, float *, float *, long long, int, hipStream_t);

template <typename T>
void launch_qkv_bwd(const QkvBwdArgs &a, T *dqkv, hipStream_t s) {
  const long long items = (long long)a.M * (a.H + 2 * a.Hkv);
  if (items > 0) qkv_bwd_kernel<T><<<(unsigned)((items + 3) / 4), 256, 0, s>>>(a, dqkv);
}
template void launch_qkv_bwd<bf16>(const QkvBwdArgs &, bf16 *, hipStream_t);
template void launch_qkv_bwd<float>(const QkvBwdArgs &, float *, hipStream_t);

template <typename T>
void launch_attn_bwd(const AttnBwdArgs &a, hipStream_t s) {
  const long long rows = (long long)a.M * a.H, keys = (long long)a.M * a.Hkv;
  if (rows > 0) attn_bwd_rows_kernel<T><<<(unsigned)((rows + 15) / 16), 256, 0, s>>>(a);
  if (keys > 0) attn_bwd_keys_kernel<T><<<(unsigned)((keys + 15) / 16), 256, 0, s>>>(a);
}

void launch_cast_rows(const float *src, long long lds, int M, int C, bf16 *dst, hipStream_t s) {
  const long long n = (long long)M * C;
  if (n > 0) cast_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src, lds, M, C, dst);
}
template void launch_attn_bwd<float>(const AttnBwdArgs &, hipStream_t);

template <typename T>
void launch_dlogits(const float *logits, const float *lse, const int *targets, const int *count, int rows, int V,
                    T *dl, hipStream_t s) {
  if (rows > 0) dlogits_kernel<T><<<rows, 256, 0, s>>>(logits, lse, targets, count, V, dl);
}
template void launch_dlogits<bf16>(const float *, const float *, const int *, const int *, int, int, bf16 *,
                                   hipStream_t);
template void launch_dlogits<float>(const float *, const float *, const int *, const int *, int, int, float *,
                                    hipStream_t);

void launch_dlogits_t(const bf16 *logits, const float *lse, const int *targets, const int *count, int rows, int V,
                      bf16 *dl, bf16 *dlt, long long ldt, int Rp, hipStream_t s) {
  if (rows <= 0) return;
  dlogits_t_kernel<<<dim3((V + kDlCols - 1) / kDlCols, Rp / 64), 256, 0, s>>>(logits, lse, targets, count, rows, V,
                                                                              dl, dlt, ldt, Rp);
}

void launch_embed_bwd(const int *tokens, const int *pos, const float *dx, float *dwte, float *dwpe, int M, int d,
                      hipStream_t s) {
  const long long n = (long long)M * d;
  if (n > 0) embed_bwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(tokens, pos, dx, dwte, dwpe, M, d);
}

void launch_count_targets(const int *targets, int M, int V, int *count, hipStream_t s) {
  count_targets_kernel<<<1, 256, 0, s>>>(targets, M, V, count);
}
