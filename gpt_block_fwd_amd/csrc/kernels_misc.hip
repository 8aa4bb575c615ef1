// Row-wise and element-wise kernels of the decoder-block forward for gfx950:
// row metadata, embedding gather, weightless RMSNorm, RoPE + QK-norm +
// K/V scatter, vocabulary softmax / log-sum-exp, token selection, and the
// fp32 small-model GEMM and attention.
#include "scatter.h"

// ---------------------------------------------------------------- row info

__global__ void rowinfo_kernel(const int *cu, const int *cu_pad, int n_seqs, int M, int *seq,
                               int *pos, int *vcol) {
  int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  int lo = 0, hi = n_seqs - 1;  // last b with cu[b] <= m
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= m) lo = mid; else hi = mid - 1;
  }
  seq[m] = lo;
  int p = m - cu[lo];
  pos[m] = p;
  if (vcol) vcol[m] = cu_pad[lo] + vperm16(p);
}

void launch_rowinfo(const int *cu, const int *cu_pad, int n_seqs, int M, int *seq, int *pos,
                    int *vcol, hipStream_t s) {
  rowinfo_kernel<<<(M + 255) / 256, 256, 0, s>>>(cu, cu_pad, n_seqs, M, seq, pos, vcol);
}

// ---------------------------------------------------------------- embedding
// Token embedding (plus learned position embedding on the small path) into
// the fp32 residual stream.

__global__ void embed_bf16_kernel(const int *tok, const bf16 *wte, float *x, int M, int d) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // 8 elements each
  long long total = (long long)M * d / 8;
  if (i >= total) return;
  long long m = i * 8 / d;
  int c = (int)(i * 8 - m * d);
  const bf16x8 v = *(const bf16x8 *)(wte + (long long)tok[m] * d + c);
  float4 a = make_float4(bf2f(v[0]), bf2f(v[1]), bf2f(v[2]), bf2f(v[3]));
  float4 b = make_float4(bf2f(v[4]), bf2f(v[5]), bf2f(v[6]), bf2f(v[7]));
  float4 *dst = (float4 *)(x + m * d + c);
  dst[0] = a;
  dst[1] = b;
}

// The step's decode-attention work list (one workgroup): the chunks that
// hold positions, in order of sequence then chunk.  A wave-wide inclusive
// scan of the chunk counts, plus the waves before it, gives each sequence its
// first entry.
DEV void decode_map_block(const DecodeMapArgs &a) {
  __shared__ int wsum[4];
  const PagedKV &kv = a.kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int run = 0;  // entries of the sequences before this pass
  for (int base = 0; base < a.n; base += 256) {
    const int b = base + tid;
    const int len = b < a.n ? kv.lens[b] + 1 : 0;
    const int pages = (len + 63) / 64;
    // at most max_chunks per sequence, the list's room per sequence (the
    // host picks chunk_pages so that none has more, from its copy of the
    // lengths; the bound keeps the list in its buffer should the copies
    // ever disagree)
    const int nc = min((pages + a.chunk_pages - 1) / a.chunk_pages, a.max_chunks);
    int inc = nc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int before = run;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int first = before + inc - nc;
    for (int c = 0; c < nc; ++c) {
      int *e = a.map + kDecodeMapStride * (first + c);
      e[0] = b;
      e[1] = c;
      e[2] = len;
      e[3] = 0;
#pragma unroll
      for (int w = 0; w < 8; ++w)
        e[4 + w] = kv.table[(long long)b * kv.pages_per_seq + min(c * a.chunk_pages + w, kv.pages_per_seq - 1)];
    }
    run += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();  // wsum is rewritten by the next pass
  }
}

// Decode rows: x = WTE[token] (fp32), h = rms(x) (bf16), one wave per row.
// Block 0 also clears the completion counters the fused kernels of the step
// use (they reset what they use, so this only matters for a fresh workspace),
// and one more workgroup after the rows' writes the step's work list.
__global__ __launch_bounds__(256) void embed_norm_bf16_kernel(const int *tok, const bf16 *wte, float *x,
                                                              bf16 *h, int M, int d, float eps,
                                                              unsigned *ctr, int nctr, DecodeMapArgs dm) {
  if (blockIdx.x == gridDim.x - 1 && dm.map) {
    decode_map_block(dm);
    return;
  }
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nctr; i += blockDim.x) ctr[i] = 0u;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + wave;
  if (m >= M) return;
  const bf16 *er = wte + (long long)tok[m] * d;
  float *xr = x + (long long)m * d;
  for (int c = lane * 8; c < d; c += 512) {
    const bf16x8 v = *(const bf16x8 *)(er + c);
    *(float4 *)(xr + c) = make_float4(bf2f(v[0]), bf2f(v[1]), bf2f(v[2]), bf2f(v[3]));
    *(float4 *)(xr + c + 4) = make_float4(bf2f(v[4]), bf2f(v[5]), bf2f(v[6]), bf2f(v[7]));
  }
  rmsnorm_row_bf16(xr, h + (long long)m * d, d, eps, lane);
}

void launch_embed_norm_bf16(const int *tok, const bf16 *wte, float *x, bf16 *h, int M, int d,
                            float eps, unsigned *ctr, int nctr, const DecodeMapArgs &dm, hipStream_t s) {
  const int blocks = (M + 3) / 4 + (dm.map && dm.n > 0 ? 1 : 0);
  embed_norm_bf16_kernel<<<blocks, 256, 0, s>>>(tok, wte, x, h, M, d, eps, ctr, nctr, dm);
}

// One workgroup per row; d <= 2048, so a thread holds at most two
// four-float chunks (columns 4 t and 4 t + 1024).  All slab loads of both
// chunks are issued before the first add; the sum runs x + slab 0 + slab 1
// + ... in that order.
__global__ __launch_bounds__(256) void resid_norm_bf16_kernel(const float *part, int nslab, long long slab,
                                                              float *x, bf16 *h, int M, int d, float eps) {
  __shared__ float red[4];
  const int m = blockIdx.x, t = threadIdx.x;
  float *xr = x + (long long)m * d;
  const float *pr = part + (long long)m * d;
  f32x4 v[2], p[2][kMaxRowSplit];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int col = 4 * (t + 256 * i);
    if (col < d) {
      v[i] = *(const f32x4 *)(xr + col);
#pragma unroll
      for (int k = 0; k < kMaxRowSplit; ++k)
        if (k < nslab) p[i][k] = *(const f32x4 *)(pr + k * slab + col);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int col = 4 * (t + 256 * i);
    if (col < d) {
#pragma unroll
      for (int k = 0; k < kMaxRowSplit; ++k)
        if (k < nslab) v[i] += p[i][k];
      *(f32x4 *)(xr + col) = v[i];
      ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
  }
  ss = wave_sum(ss);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float rs = 1.0f / sqrtf(ss / (float)d + eps);
  bf16 *hr = h + (long long)m * d;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int col = 4 * (t + 256 * i);
    if (col < d) {
      bf16x4 o = {f2bf(v[i][0] * rs), f2bf(v[i][1] * rs), f2bf(v[i][2] * rs), f2bf(v[i][3] * rs)};
      *(bf16x4 *)(hr + col) = o;
    }
  }
}

void launch_resid_norm_bf16(const float *part, int nslab, long long slab, float *x, bf16 *h, int M, int d,
                            float eps, hipStream_t s) {
  resid_norm_bf16_kernel<<<M, 256, 0, s>>>(part, nslab, slab, x, h, M, d, eps);
}

void launch_embed_bf16(const int *tok, const bf16 *wte, float *x, int M, int d, hipStream_t s) {
  long long total = (long long)M * d / 8;
  embed_bf16_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(tok, wte, x, M, d);
}

__global__ void embed_f32_kernel(const int *tok, const float *wte, const float *wpe,
                                 const int *pos, float *x, int M, int d) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)M * d) return;
  long long m = i / d;
  int c = (int)(i - m * d);
  float v = wte[(long long)tok[m] * d + c];
  if (wpe) v += wpe[(long long)pos[m] * d + c];
  x[i] = v;
}

void launch_embed_f32(const int *tok, const float *wte, const float *wpe, const int *pos, float *x,
                      int M, int d, hipStream_t s) {
  long long total = (long long)M * d;
  embed_f32_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(tok, wte, wpe, pos, x, M, d);
}

// ---------------------------------------------------------------- RMSNorm
// y = x / sqrt(mean(x^2) + eps), no gain.  One 64-lane wave per row, fp32
// sum of squares reduced across the wave.  `rows` optionally selects source
// rows (the last position of each sequence).

// NC > 0: the row (d <= 256 NC) is loaded into registers with every load in
// flight at once and written from there; NC == 0: any d, two passes.
template <typename TO, int NC>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *x, TO *y, const int *rows,
                                                      int M, int d, float eps) {
  int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int r = blockIdx.x * 4 + wave;
  if (r >= M) return;
  long long src = rows ? rows[r] : r;
  const float *xr = x + src * d;
  TO *yr = y + (long long)r * d;
  auto put = [&](int c, f32x4 v, float rs) {
    if constexpr (sizeof(TO) == 2) {
      bf16x4 o = {f2bf(v[0] * rs), f2bf(v[1] * rs), f2bf(v[2] * rs), f2bf(v[3] * rs)};
      *(bf16x4 *)(yr + c) = o;
    } else {
      *(f32x4 *)(yr + c) = (f32x4){v[0] * rs, v[1] * rs, v[2] * rs, v[3] * rs};
    }
  };
  float ss = 0.f;
  if constexpr (NC > 0) {
    f32x4 v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (lane * 4 + 256 * i < d) v[i] = *(const f32x4 *)(xr + lane * 4 + 256 * i);
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (lane * 4 + 256 * i < d) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (lane * 4 + 256 * i < d) put(lane * 4 + 256 * i, v[i], rs);
  } else {
    for (int c = lane * 4; c < d; c += 256) {
      const f32x4 v = *(const f32x4 *)(xr + c);
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane * 4; c < d; c += 256) put(c, *(const f32x4 *)(xr + c), rs);
  }
}

void launch_rmsnorm_bf16(const float *x, bf16 *y, const int *rows, int M, int d, float eps,
                         hipStream_t s) {
  if (d <= 2048) rmsnorm_kernel<bf16, 8><<<(M + 3) / 4, 256, 0, s>>>(x, y, rows, M, d, eps);
  else rmsnorm_kernel<bf16, 0><<<(M + 3) / 4, 256, 0, s>>>(x, y, rows, M, d, eps);
}
void launch_rmsnorm_f32(const float *x, float *y, const int *rows, int M, int d, float eps,
                        hipStream_t s) {
  if (d <= 2048) rmsnorm_kernel<float, 8><<<(M + 3) / 4, 256, 0, s>>>(x, y, rows, M, d, eps);
  else rmsnorm_kernel<float, 0><<<(M + 3) / 4, 256, 0, s>>>(x, y, rows, M, d, eps);
}

// ---------------------------------------------------------------- RoPE + QK-norm + scatter
// One wave per (row, head slot) of a 128-wide head.  Lane l owns the rotary
// pair (l, l + 64): half-split rotation by the tabled angle, then a
// weightless RMSNorm over the head (sum of squares reduced across the wave).

__global__ __launch_bounds__(256) void rope_norm_scatter_bf16_kernel(ScatterArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slots = a.H + 2 * a.Hkv;
  const long long item = (long long)blockIdx.x * 4 + wave;
  if (item >= (long long)a.M * slots) return;
  const int m = (int)(item / slots), j = (int)(item - (long long)m * slots);
  rope_norm_scatter_row(a, a.qkv + (long long)m * slots * 128 + j * 128, m, j, lane);
}

void launch_rope_norm_scatter_bf16(const ScatterArgs &a, hipStream_t s) {
  long long items = (long long)a.M * (a.H + 2 * a.Hkv);
  rope_norm_scatter_bf16_kernel<<<(unsigned)((items + 3) / 4), 256, 0, s>>>(a);
}

// fp32 small path: one thread per (row, head slot), any even head_dim <= 64.
__global__ void qkv_scatter_f32_kernel(ScatterArgs a) {
  int slots = a.H + 2 * a.Hkv;
  long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (long long)a.M * slots) return;
  int m = (int)(item / slots), j = (int)(item - (long long)m * slots);
  int dh = a.head_dim, half = dh / 2;
  const float *u = a.qkv + (long long)m * slots * dh + j * dh;
  float y[64];
  for (int i = 0; i < dh; ++i) y[i] = u[i];
  int p = a.pos[m];
  int b = a.seq ? a.seq[m] : m;
  bool is_v = j >= a.H + a.Hkv;
  if (!is_v) {
    if (a.cos) {
      for (int i = 0; i < half; ++i) {
        float c = a.cos[p * half + i], s = a.sin[p * half + i];
        float r0 = y[i] * c - y[i + half] * s, r1 = y[i] * s + y[i + half] * c;
        y[i] = r0;
        y[i + half] = r1;
      }
    }
    if (a.qk_norm) {
      float ss = 0.f;
      for (int i = 0; i < dh; ++i) ss += y[i] * y[i];
      float rs = 1.0f / sqrtf(ss / (float)dh + a.eps);
      for (int i = 0; i < dh; ++i) y[i] *= rs;
    }
  }
  int kvd = a.Hkv * dh;
  float *dst = nullptr;
  if (j < a.H) {
    dst = (float *)a.q_out + (long long)m * a.H * dh + j * dh;
  } else if (!is_v) {
    if (a.k_out) dst = (float *)a.k_out + (long long)m * kvd + (j - a.H) * dh;
  } else {
    if (a.vt_out) dst = (float *)a.vt_out + (long long)m * kvd + (j - a.H - a.Hkv) * dh;
  }
  if (dst)
    for (int i = 0; i < dh; ++i) dst[i] = y[i];
  if (a.use_cache && j >= a.H) {
    const PagedKV &kv = a.kv;
    int g = is_v ? j - a.H - a.Hkv : j - a.H;
    int page = kv.table[b * kv.pages_per_seq + p / kv.page_size];
    int slot = p % kv.page_size;
    char *pg = kv.base + (long long)a.layer * kv.layer_stride + (long long)page * kv.page_stride;
    float *c = (float *)(pg + (is_v ? kv.half_bytes : 0)) + (long long)slot * kvd + g * dh;
    for (int i = 0; i < dh; ++i) c[i] = y[i];
  }
}

void launch_qkv_scatter_f32(const ScatterArgs &a, hipStream_t s) {
  long long items = (long long)a.M * (a.H + 2 * a.Hkv);
  qkv_scatter_f32_kernel<<<(unsigned)((items + 127) / 128), 128, 0, s>>>(a);
}

// ---------------------------------------------------------------- softmax / LSE
// One 256-thread workgroup per row: running (max, sum of exp) per thread,
// merged across the workgroup; lse = max + log(sum).  Optionally a second
// pass writes p = exp(logit - lse).

DEV void ms_merge(float &m, float &s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * fast_exp2((m - mn) * kLog2e) + s2 * fast_exp2((m2 - mn) * kLog2e);
  m = mn;
}

__global__ __launch_bounds__(256) void softmax_lse_kernel(const float *logits, int V, float *lse,
                                                          float *probs) {
  __shared__ float sm[4], ss[4];
  const float *row = logits + (long long)blockIdx.x * V;
  float m = -INFINITY, s = 0.f;
  for (int i = threadIdx.x; i < V; i += 256) {
    float x = row[i];
    if (x > m) {
      s = s * fast_exp2((m - x) * kLog2e) + 1.f;
      m = x;
    } else {
      s += fast_exp2((x - m) * kLog2e);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
  int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[w] = m;
    ss[w] = s;
  }
  __syncthreads();
  m = sm[0];
  s = ss[0];
  for (int i = 1; i < 4; ++i) ms_merge(m, s, sm[i], ss[i]);
  float l = m + logf(s);
  if (threadIdx.x == 0 && lse) lse[blockIdx.x] = l;
  if (probs) {
    float *pr = probs + (long long)blockIdx.x * V;
    for (int i = threadIdx.x; i < V; i += 256) pr[i] = fast_exp2((row[i] - l) * kLog2e);
  }
}

void launch_softmax_lse(const float *logits, int rows, int V, float *lse, float *probs,
                        hipStream_t s) {
  if (rows <= 0) return;
  softmax_lse_kernel<<<rows, 256, 0, s>>>(logits, V, lse, probs);
}

// lse of each row from per-block partials (max_k, sum_k) written by the
// LM-head GEMM epilogue: lse = M + log(sum_k sum_k * exp(max_k - M)).  One
// wave per row.  With `probs`, one 256-thread workgroup per row then writes
// p = exp(logit - lse).

__global__ __launch_bounds__(256) void lse_combine_kernel(const float *part, int nparts, int rows,
                                                          float *lse) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= rows) return;
  const float2 *pp = (const float2 *)part + (long long)r * nparts;
  float m = -INFINITY, s = 0.f;
  for (int i = lane; i < nparts; i += 64) {
    float2 v = pp[i];
    ms_merge(m, s, v.x, v.y);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
  if (lane == 0) lse[r] = m + logf(s);
}

__global__ __launch_bounds__(256) void probs_kernel(const float *logits, const float *lse, int V,
                                                    float *probs) {
  const float l = lse[blockIdx.x];
  const float4 *row = (const float4 *)(logits + (long long)blockIdx.x * V);
  float4 *pr = (float4 *)(probs + (long long)blockIdx.x * V);
  for (int i = threadIdx.x; i < V / 4; i += 256) {
    float4 x = row[i];
    pr[i] = make_float4(fast_exp2((x.x - l) * kLog2e), fast_exp2((x.y - l) * kLog2e),
                        fast_exp2((x.z - l) * kLog2e), fast_exp2((x.w - l) * kLog2e));
  }
}

void launch_lse_combine(const float *part, int nparts, int rows, float *lse, const float *logits,
                        int V, float *probs, hipStream_t s) {
  if (rows <= 0) return;
  lse_combine_kernel<<<(rows + 3) / 4, 256, 0, s>>>(part, nparts, rows, lse);
  if (probs) probs_kernel<<<rows, 256, 0, s>>>(logits, lse, V, probs);
}

// ---------------------------------------------------------------- cross-entropy
// Next-token cross-entropy of row r: lse[r] - logit[r][t], t = targets[r];
// a target outside [0, V) marks a row with no next token (loss 0).

// From the LM-head loss epilogue: one wave per row merges the row's (max,
// sum exp) partials as lse_combine_kernel does and subtracts the target
// logit the epilogue kept.
__global__ __launch_bounds__(256) void ce_parts_kernel(const float *part, int nparts, const float *tgt,
                                                       const int *targets, int V, int rows, float *loss,
                                                       float *lse) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= rows) return;
  const float2 *pp = (const float2 *)part + (long long)r * nparts;
  float m = -INFINITY, s = 0.f;
  for (int i = lane; i < nparts; i += 64) {
    float2 v = pp[i];
    ms_merge(m, s, v.x, v.y);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
  if (lane == 0) {
    const float l = m + logf(s);
    const int t = targets[r];
    loss[r] = (t >= 0 && t < V) ? l - tgt[r] : 0.f;
    if (lse) lse[r] = l;
  }
}

__global__ __launch_bounds__(256) void ce_logits_kernel(const float *logits, const float *lse,
                                                        const int *targets, int V, int rows, float *loss) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int t = targets[r];
  loss[r] = (t >= 0 && t < V) ? lse[r] - logits[(long long)r * V + t] : 0.f;
}

// One workgroup: thread i sums rows i, i + 1024, ... in fp64, then a fixed
// tree over the threads, so the mean does not depend on scheduling.
__global__ __launch_bounds__(1024) void mean_loss_kernel(const float *loss, const int *targets, int V,
                                                         int rows, float *mean) {
  __shared__ double ssum[1024];
  __shared__ int scnt[1024];
  double acc = 0.0;
  int cnt = 0;
  for (int r = threadIdx.x; r < rows; r += 1024) {
    const int t = targets[r];
    if (t >= 0 && t < V) {
      acc += (double)loss[r];
      ++cnt;
    }
  }
  ssum[threadIdx.x] = acc;
  scnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      ssum[threadIdx.x] += ssum[threadIdx.x + w];
      scnt[threadIdx.x] += scnt[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = scnt[0] ? (float)(ssum[0] / scnt[0]) : 0.f;
}

void launch_ce_from_parts(const float *part, int nparts, const float *tgt, const int *targets, int V,
                          int rows, float *loss, float *lse, hipStream_t s) {
  if (rows <= 0) return;
  ce_parts_kernel<<<(rows + 3) / 4, 256, 0, s>>>(part, nparts, tgt, targets, V, rows, loss, lse);
}

void launch_ce_from_logits(const float *logits, const float *lse, const int *targets, int V, int rows,
                           float *loss, hipStream_t s) {
  if (rows <= 0) return;
  ce_logits_kernel<<<(rows + 255) / 256, 256, 0, s>>>(logits, lse, targets, V, rows, loss);
}

void launch_mean_loss(const float *loss, const int *targets, int V, int rows, float *mean, hipStream_t s) {
  mean_loss_kernel<<<1, 1024, 0, s>>>(loss, targets, V, rows, mean);
}

// ---------------------------------------------------------------- greedy
// Argmax per row; among equal maxima the lowest index wins.  Two phases so
// that a few rows still spread over many CUs: phase 1 reduces chunks of
// kArgChunk columns (grid rows x chunks), phase 2 merges a row's chunks.

constexpr int kArgChunk = 2048;

DEV void arg_merge(float &best, int &bi, float v2, int i2) {
  if (v2 > best || (v2 == best && i2 < bi)) {
    best = v2;
    bi = i2;
  }
}

// Partials are (float bits of the value, index) pairs of ints, so the index
// never passes through a float register (small integers are denormals).
__global__ __launch_bounds__(256) void argmax_partial_kernel(const float *logits, int V,
                                                             int2 *part) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int row = blockIdx.y, chunk = blockIdx.x;
  const float *r = logits + (long long)row * V;
  const int i0 = chunk * kArgChunk, i1 = min(V, i0 + kArgChunk);
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = i0 + threadIdx.x; i < i1; i += 256) {
    const float x = r[i];
    if (x > best) {  // indices visited in increasing order: keep the first
      best = x;
      bi = i;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) arg_merge(best, bi, __shfl_xor(best, o, 64), __shfl_xor(bi, o, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = best;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k) arg_merge(best, bi, sv[k], si[k]);
    part[(long long)row * gridDim.x + chunk] = make_int2(__float_as_int(best), bi);
  }
}

__global__ __launch_bounds__(256) void argmax_final_kernel(const int2 *part, int nchunks,
                                                           int rows, int *out, int *lens) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int c = lane; c < nchunks; c += 64) {
    const int2 v = part[(long long)row * nchunks + c];
    arg_merge(best, bi, __int_as_float(v.x), v.y);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) arg_merge(best, bi, __shfl_xor(best, o, 64), __shfl_xor(bi, o, 64));
  if (lane == 0) {
    out[row] = bi == 0x7fffffff ? 0 : bi;
    if (lens) lens[row] += 1;  // decode: the step's position is now cached
  }
}

// Single-pass variant without scratch: one workgroup per row.
__global__ __launch_bounds__(256) void argmax_rows_kernel(const float *logits, int V, int *out) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const float *r = logits + (long long)blockIdx.x * V;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < V; i += 256) {
    const float x = r[i];
    if (x > best) {
      best = x;
      bi = i;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) arg_merge(best, bi, __shfl_xor(best, o, 64), __shfl_xor(bi, o, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = best;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k) arg_merge(best, bi, sv[k], si[k]);
    out[blockIdx.x] = bi == 0x7fffffff ? 0 : bi;
  }
}

void launch_argmax_rows(const float *logits, int rows, int V, int *out, hipStream_t s) {
  if (rows > 0) argmax_rows_kernel<<<rows, 256, 0, s>>>(logits, V, out);
}

int argmax_scratch_floats(int rows, int V) { return 2 * rows * ((V + kArgChunk - 1) / kArgChunk); }

void launch_argmax(const float *logits, int rows, int V, int *out, float *scratch, int *lens,
                   hipStream_t s) {
  if (rows <= 0) return;
  const int nchunks = (V + kArgChunk - 1) / kArgChunk;
  argmax_partial_kernel<<<dim3(nchunks, rows), 256, 0, s>>>(logits, V, (int2 *)scratch);
  argmax_final_kernel<<<(rows + 3) / 4, 256, 0, s>>>((const int2 *)scratch, nchunks, rows, out, lens);
}

// ---------------------------------------------------------------- sampling
// Inverse-CDF temperature sampling, one 1024-thread workgroup per row:
// weights e_i = 2^((x_i - max) log2(e) / T); the token is the first i whose
// cumulative weight exceeds u * total.  The row is walked in super-tiles of
// 8192 entries; thread t owns entries 8t .. 8t + 8 of each (32 contiguous
// bytes, so a wave's loads are contiguous).  The row max, then each
// super-tile's total (per-wave sums added in wave order); the total weight
// is the sum of the super-tile totals in order.  The first super-tile whose
// running total passes the target holds the crossing, and samp_claim finds
// the thread and the entry inside it.  If rounding leaves the target at or
// above the total, the last entry of positive weight is taken.

constexpr int kSampThreads = 1024, kSampPer = 8, kSampTile = kSampThreads * kSampPer;

DEV void samp_load(const float *row, int V, int base, int t, float (&x)[kSampPer]) {
  const int i0 = base + kSampPer * t;
  if (i0 + kSampPer <= V && (V & 3) == 0) {
    const f32x4 lo = *(const f32x4 *)(row + i0), hi = *(const f32x4 *)(row + i0 + 4);
    x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
    x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
  } else {
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) x[j] = i0 + j < V ? row[i0 + j] : -INFINITY;
  }
}

// The crossing inside the super-tile that holds it.  Called by every thread
// of the workgroup (it has a barrier) with the same `run` (weight of the
// super-tiles before this one) and `target`; `wtot` holds the super-tile's
// 16 wave totals, and the super-tile's total is their sum in wave order from
// zero -- the same sum that chose this super-tile.  Thread t claims the half-open
// range [lo_t, lo_{t+1}) of the running weight, where lo_t is its wave's
// start (run plus the earlier waves' totals, summed in wave order) plus the
// exclusive scan of the wave's thread sums, and the last thread's range ends
// at run plus the super-tile total.  Each boundary is one value computed once
// and handed to both neighbours, so the ranges tile [run, run + total)
// exactly: a target inside it is claimed by at least one thread, whatever the
// rounding.  The claiming thread walks its 8 entries from lo_t to the first
// whose running weight passes the target; if rounding leaves none, it takes
// the last entry of positive weight at or before its own entries in this
// super-tile.  Where rounding makes ranges overlap, the lowest index wins.
DEV void samp_claim(const float (&e)[kSampPer], float mine, const float *wtot, float run, float target,
                    int idx0, int *s_pick, int *s_wlast) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  float before = 0.f;
  for (int k = 0; k < w; ++k) before += wtot[k];
  const float base_w = run + before, base_n = run + (before + wtot[w]);
  float incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  float excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.f;
  const float lo = base_w + excl;
  float hi = __shfl_down(lo, 1, 64);
  if (lane == 63) hi = base_n;
  // last positive entry at or before this thread's, within the super-tile
  int lastp = -1;
#pragma unroll
  for (int j = 0; j < kSampPer; ++j)
    if (e[j] > 0.f) lastp = idx0 + j;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(lastp, o, 64);
    if (lane >= o) lastp = max(lastp, v);
  }
  if (lane == 63) s_wlast[w] = lastp;
  __syncthreads();
  for (int k = 0; k < w; ++k) lastp = max(lastp, s_wlast[k]);
  if (lo <= target && target < hi) {
    float cum = lo;
    int pick = -1;
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) {
      cum += e[j];
      if (pick < 0 && cum > target) pick = idx0 + j;
    }
    if (pick < 0) pick = lastp;
    if (pick >= 0) atomicMin(s_pick, pick);
  }
}

constexpr int kNoPick = 0x7fffffff;

// Rows longer than the register-resident kernel takes: three passes over
// the row (max; per-super-tile totals; the super-tile holding the crossing),
// the per-super-tile totals formed identically in the last two.
__global__ __launch_bounds__(kSampThreads) void sample_kernel(const float *logits, int V, float inv_t,
                                                              const float *uniforms, int *out, int *lens) {
  constexpr int NW = kSampThreads / 64;
  __shared__ float red[NW];
  __shared__ int s_wlast[NW];
  __shared__ int s_pick, s_last;
  const float *row = logits + (long long)blockIdx.x * V;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  float x[kSampPer];
  // pass 1: max
  float m = -INFINITY;
  for (int base = 0; base < V; base += kSampTile) {
    samp_load(row, V, base, t, x);
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) m = fmaxf(m, x[j]);
  }
  m = wave_max(m);
  if (lane == 0) red[w] = m;
  if (t == 0) {
    s_pick = kNoPick;
    s_last = -1;
  }
  __syncthreads();
  m = red[0];
  for (int k = 1; k < NW; ++k) m = fmaxf(m, red[k]);
  const float sc = inv_t * kLog2e;
  // weights of this thread's entries of super-tile `base`, their sum, and
  // the super-tile's wave totals in red (ends with a barrier)
  auto tile = [&](int base, float (&e)[kSampPer], float &mine) {
    samp_load(row, V, base, t, x);
    mine = 0.f;
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) {
      e[j] = fast_exp2((x[j] - m) * sc);
      mine += e[j];
    }
    const float v = wave_sum(mine);
    __syncthreads();  // every thread is done reading red
    if (lane == 0) red[w] = v;
    __syncthreads();
  };
  // pass 2: the total, as the sum of the super-tile totals in order
  float total = 0.f;
  int last = -1;
  for (int base = 0; base < V; base += kSampTile) {
    float e[kSampPer], mine;
    tile(base, e, mine);
#pragma unroll
    for (int j = 0; j < kSampPer; ++j)
      if (e[j] > 0.f) last = base + kSampPer * t + j;
    float T = 0.f;
    for (int k = 0; k < NW; ++k) T += red[k];
    total += T;
  }
  const float target = uniforms[blockIdx.x] * total;
  // pass 3: the first super-tile whose running total passes the target
  float run = 0.f;
  for (int base = 0; base < V; base += kSampTile) {
    float e[kSampPer], mine;
    tile(base, e, mine);
    float T = 0.f;
    for (int k = 0; k < NW; ++k) T += red[k];
    if (run + T > target) {  // the same in every thread
      samp_claim(e, mine, red, run, target, base + kSampPer * t, &s_pick, s_wlast);
      break;
    }
    run += T;
  }
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  if (t == 0) {
    out[blockIdx.x] = s_pick != kNoPick ? s_pick : (s_last >= 0 ? s_last : 0);
    if (lens) lens[blockIdx.x] += 1;  // decode: the step's position is now cached
  }
}

// The same choice with the row read once: for V <= NS super-tiles the
// thread keeps its NS x 8 entries in registers.  The weights of every
// super-tile are summed per wave; the total is the sum of the super-tile
// totals in order, and the super-tile holding the crossing is the first
// whose running total passes the target.  The last entry of positive weight
// stands in where rounding leaves no crossing.
template <int NS>
__global__ __launch_bounds__(kSampThreads) void sample_reg_kernel(const float *logits, int V, float inv_t,
                                                                  const float *uniforms, int *out, int *lens) {
  constexpr int NW = kSampThreads / 64;
  __shared__ float red[NS][NW];
  __shared__ float red_m[NW];
  __shared__ int s_wlast[NW];
  __shared__ int s_pick, s_last;
  const float *row = logits + (long long)blockIdx.x * V;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  float x[NS][kSampPer];
#pragma unroll
  for (int st = 0; st < NS; ++st) samp_load(row, V, st * kSampTile, t, x[st]);
  float m = -INFINITY;
#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) m = fmaxf(m, x[st][j]);
  m = wave_max(m);
  if (lane == 0) red_m[w] = m;
  if (t == 0) {
    s_pick = kNoPick;
    s_last = -1;
  }
  __syncthreads();
  m = red_m[0];
  for (int k = 1; k < NW; ++k) m = fmaxf(m, red_m[k]);
  const float sc = inv_t * kLog2e;
  float ts[NS];
  int last = -1;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    ts[st] = 0.f;
#pragma unroll
    for (int j = 0; j < kSampPer; ++j) {
      x[st][j] = fast_exp2((x[st][j] - m) * sc);
      ts[st] += x[st][j];
      if (x[st][j] > 0.f) last = st * kSampTile + kSampPer * t + j;
    }
    const float v = wave_sum(ts[st]);
    if (lane == 0) red[st][w] = v;
  }
  __syncthreads();
  float T[NS], total = 0.f;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    T[st] = 0.f;
    for (int k = 0; k < NW; ++k) T[st] += red[st][k];
    total += T[st];
  }
  const float target = uniforms[blockIdx.x] * total;
  // the super-tile holding the crossing (the same for every thread)
  int sx = -1;
  float run = 0.f;
#pragma unroll
  for (int st = 0; st < NS; ++st)
    if (sx < 0) {
      if (run + T[st] > target) sx = st;
      else run += T[st];
    }
  if (sx >= 0) {
    float e[kSampPer], mine = 0.f;
#pragma unroll
    for (int st = 0; st < NS; ++st)
      if (st == sx) {
#pragma unroll
        for (int j = 0; j < kSampPer; ++j) e[j] = x[st][j];
        mine = ts[st];
      }
    samp_claim(e, mine, red[sx], run, target, sx * kSampTile + kSampPer * t, &s_pick, s_wlast);
  }
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  if (t == 0) {
    out[blockIdx.x] = s_pick != kNoPick ? s_pick : (s_last >= 0 ? s_last : 0);
    if (lens) lens[blockIdx.x] += 1;  // decode: the step's position is now cached
  }
}

void launch_sample(const float *logits, int rows, int V, float temperature, const float *u,
                   int *out, int *lens, hipStream_t s) {
  if (rows <= 0) return;
  const float it = 1.0f / temperature;
  switch ((V + kSampTile - 1) / kSampTile) {
    case 1: sample_reg_kernel<1><<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
    case 2: sample_reg_kernel<2><<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
    case 3: sample_reg_kernel<3><<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
    case 4: sample_reg_kernel<4><<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
    case 5: sample_reg_kernel<5><<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
    case 6: sample_reg_kernel<6><<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
    case 7: sample_reg_kernel<7><<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
    case 8: sample_reg_kernel<8><<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
    default: sample_kernel<<<rows, kSampThreads, 0, s>>>(logits, V, it, u, out, lens); return;
  }
}

// ---------------------------------------------------------------- KV lengths

__global__ void lens_set_kernel(int *lens, const int *cu, int n) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < n) lens[b] = cu[b + 1] - cu[b];
}
__global__ void lens_inc_kernel(int *lens, int n) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < n) lens[b] += 1;
}
void launch_lens_set(int *lens, const int *cu, int n, hipStream_t s) {
  lens_set_kernel<<<(n + 255) / 256, 256, 0, s>>>(lens, cu, n);
}
void launch_lens_inc(int *lens, int n, hipStream_t s) {
  lens_inc_kernel<<<(n + 255) / 256, 256, 0, s>>>(lens, n);
}

__global__ void gather_rows_bf16_kernel(const bf16 *src, bf16 *dst, const int *rows, int d) {
  const bf16 *s = src + (long long)rows[blockIdx.x] * d;
  bf16 *o = dst + (long long)blockIdx.x * d;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) *(bf16x8 *)(o + c) = *(const bf16x8 *)(s + c);
}
void launch_gather_rows_bf16(const bf16 *src, bf16 *dst, const int *rows, int n, int d,
                             hipStream_t s) {
  if (n > 0) gather_rows_bf16_kernel<<<n, 64, 0, s>>>(src, dst, rows, d);
}

// ---------------------------------------------------------------- fp32 small path

__global__ void gemm_f32_kernel(GemmArgs g) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)g.M * g.N) return;
  int m = (int)(i / g.N), n = (int)(i - (long long)m * g.N);
  const float *w;
  if (n < g.n1) w = (const float *)g.W0 + (long long)n * g.ldw;
  else if (n < g.n2) w = (const float *)g.W1 + (long long)(n - g.n1) * g.ldw;
  else w = (const float *)g.W2 + (long long)(n - g.n2) * g.ldw;
  const float *a = (const float *)g.A + (long long)m * g.lda;
  float acc = 0.f;
  for (int k = 0; k < g.K; ++k) acc = fmaf(a[k], w[k], acc);
  float *c = (float *)g.C + (long long)m * g.ldc + n;
  if (g.epi == EPI_RESID) *c = (g.rin ? g.rin[(long long)m * g.ldc + n] : *c) + acc;
  else if (g.epi == EPI_RELU_F32) *c = fmaxf(acc, 0.f);
  else if (g.epi == EPI_RELU2_BF16) { float r = fmaxf(acc, 0.f); *c = r * r; }  // fp32 output here
  else *c = acc;
}

void launch_gemm_f32(const GemmArgs &g, hipStream_t s) {
  long long total = (long long)g.M * g.N;
  if (total > 0) gemm_f32_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(g);
}

// Causal attention, one thread per (row, head), online softmax in fp32.
__global__ void attn_prefill_f32_kernel(AttnF32Args a) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)a.M * a.H) return;
  int m = (int)(i / a.H), h = (int)(i - (long long)m * a.H);
  int g = h * a.Hkv / a.H, dh = a.dh, kvd = a.Hkv * dh;
  int p = a.pos[m];
  int r0 = m - p;
  const float *q = a.q + (long long)m * a.H * dh + h * dh;
  float acc[64];
  for (int c = 0; c < dh; ++c) acc[c] = 0.f;
  float mx = -INFINITY, l = 0.f, scale = 1.0f / sqrtf((float)dh);
  for (int j = 0; j <= p; ++j) {
    const float *k = a.k + (long long)(r0 + j) * kvd + g * dh;
    const float *v = a.v + (long long)(r0 + j) * kvd + g * dh;
    float s = 0.f;
    for (int c = 0; c < dh; ++c) s = fmaf(q[c], k[c], s);
    s *= scale;
    float mn = fmaxf(mx, s);
    float alpha = expf(mx - mn), e = expf(s - mn);
    l = l * alpha + e;
    for (int c = 0; c < dh; ++c) acc[c] = acc[c] * alpha + e * v[c];
    mx = mn;
  }
  float *o = a.o + (long long)m * a.H * dh + h * dh;
  for (int c = 0; c < dh; ++c) o[c] = acc[c] / l;
}

void launch_attn_prefill_f32(const AttnF32Args &a, hipStream_t s) {
  long long total = (long long)a.M * a.H;
  if (total > 0) attn_prefill_f32_kernel<<<(unsigned)((total + 127) / 128), 128, 0, s>>>(a);
}

// Decode: row b is sequence b at position lens[b]; keys 0..lens[b] from the
// fp32 paged cache.
__global__ void attn_decode_f32_kernel(AttnF32Args a) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)a.M * a.H) return;
  int b = (int)(i / a.H), h = (int)(i - (long long)b * a.H);
  int g = h * a.Hkv / a.H, dh = a.dh, kvd = a.Hkv * dh;
  const PagedKV &kv = a.kv;
  int p = kv.lens[b];
  const float *q = a.q + (long long)b * a.H * dh + h * dh;
  float acc[64];
  for (int c = 0; c < dh; ++c) acc[c] = 0.f;
  float mx = -INFINITY, l = 0.f, scale = 1.0f / sqrtf((float)dh);
  const char *lay = kv.base + (long long)a.layer * kv.layer_stride;
  for (int j = 0; j <= p; ++j) {
    int page = kv.table[b * kv.pages_per_seq + j / kv.page_size];
    const char *pg = lay + (long long)page * kv.page_stride;
    int slot = j % kv.page_size;
    const float *k = (const float *)pg + (long long)slot * kvd + g * dh;
    const float *v = (const float *)(pg + kv.half_bytes) + (long long)slot * kvd + g * dh;
    float s = 0.f;
    for (int c = 0; c < dh; ++c) s = fmaf(q[c], k[c], s);
    s *= scale;
    float mn = fmaxf(mx, s);
    float alpha = expf(mx - mn), e = expf(s - mn);
    l = l * alpha + e;
    for (int c = 0; c < dh; ++c) acc[c] = acc[c] * alpha + e * v[c];
    mx = mn;
  }
  float *o = a.o + (long long)b * a.H * dh + h * dh;
  for (int c = 0; c < dh; ++c) o[c] = acc[c] / l;
}

void launch_attn_decode_f32(const AttnF32Args &a, hipStream_t s) {
  long long total = (long long)a.M * a.H;
  if (total > 0) attn_decode_f32_kernel<<<(unsigned)((total + 127) / 128), 128, 0, s>>>(a);
}
