// C-ABI layer of libgpt.so: argument validation, workspace layout, the
// paged KV-cache handle and the prefill / decode drivers that enqueue the
// gfx950 kernels.  No device memory is allocated here; every device buffer
// belongs to the caller.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gpt.h"
#include "../../include/gpt_profile.h"
#include "../../include/gpt_debug.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

gpt_status fail(gpt_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

gpt_status hip_check(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GPT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GPT_OK;
}

constexpr int kMaxPrefillSeqs = 512;

// Decode-attention chunking for one step, from the host mirror of the cached
// lengths: a sequence of P pages (its positions and the new one) splits into
// ceil(P / chunk) chunks of `chunk` pages, one workgroup each (one per CU,
// for the LDS).  The smallest chunk that keeps the busy workgroups within
// the 256 CUs spreads the pages most evenly.  Chunks of up to 4 pages run on
// four waves, 5 to 8 on eight waves in one round, 9 to 16 on eight waves in
// two.  Chunks of at least ceil(longest / partial-buffer splits) pages fit
// the partial buffers.
void decode_chunking(const int *lens, int n, int n_kv_head, int splits_alloc, int *chunk_pages, int *splits,
                     int *work) {
  int pmax = 1;
  for (int b = 0; b < n; ++b) pmax = std::max(pmax, (lens[b] + 1 + 63) / 64);
  int chunk = std::max(1, (pmax + splits_alloc - 1) / splits_alloc);
  long long wgs = 0;
  for (;; ++chunk) {
    wgs = 0;
    for (int b = 0; b < n; ++b) wgs += ((lens[b] + 1 + 63) / 64 + chunk - 1) / chunk;
    if (wgs * n_kv_head <= 256 || chunk == 16) break;
  }
  *chunk_pages = chunk;
  *splits = (pmax + chunk - 1) / chunk;
  *work = (int)wgs;
}
constexpr int kCounters = 4096;  // decode-attention chunk counters (one per sequence and K/V head)
constexpr int kPage = 64;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ------------------------------------------------------------------ profiler

struct ProfRec {
  int cls;
  hipEvent_t a, b;
  double flops, bytes;
};
struct Profiler {
  uint32_t mask = 0;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    hipEventCreate(&e);
    return e;
  }
  void reset() {
    for (auto &r : recs) {
      pool.push_back(r.a);
      pool.push_back(r.b);
    }
    recs.clear();
  }
} g_prof;

// Brackets one launch with events when its class is enabled.
struct Timed {
  int cls;
  hipStream_t s;
  hipEvent_t a = nullptr;
  double flops, bytes;
  Timed(int c, hipStream_t st, double f, double by) : cls(c), s(st), flops(f), bytes(by) {
    if (g_prof.mask & (1u << cls)) {
      a = g_prof.get();
      hipEventRecord(a, s);
    }
  }
  ~Timed() {
    if (!a) return;
    hipEvent_t b = g_prof.get();
    hipEventRecord(b, s);
    g_prof.recs.push_back({cls, a, b, flops, bytes});
  }
};

// ------------------------------------------------------------------ config

gpt_status check_config(const gpt_config *c) {
  if (!c) return fail(GPT_ERR_ARG, "config is NULL");
  if (c->vocab <= 0 || c->n_layer <= 0 || c->d_model <= 0 || c->n_head <= 0 ||
      c->n_kv_head <= 0 || c->head_dim <= 0 || c->d_ff <= 0 || c->max_seq <= 0)
    return fail(GPT_ERR_ARG, "config sizes must be positive");
  if (c->n_head % c->n_kv_head) return fail(GPT_ERR_ARG, "n_head must be a multiple of n_kv_head");
  if (c->pos_kind != GPT_POS_LEARNED && c->pos_kind != GPT_POS_ROPE)
    return fail(GPT_ERR_ARG, "pos_kind must be 0 or 1");
  if (c->act != GPT_ACT_RELU && c->act != GPT_ACT_RELU2) return fail(GPT_ERR_ARG, "act must be 0 or 1");
  if (c->qk_norm != 0 && c->qk_norm != 1) return fail(GPT_ERR_ARG, "qk_norm must be 0 or 1");
  if (c->dtype != GPT_DTYPE_F32 && c->dtype != GPT_DTYPE_BF16) return fail(GPT_ERR_ARG, "dtype must be 0 or 1");
  if (!(c->norm_eps >= 0.f)) return fail(GPT_ERR_ARG, "norm_eps must be >= 0");
  if (c->pos_kind == GPT_POS_ROPE && !(c->rope_base > 0.f)) return fail(GPT_ERR_ARG, "rope_base must be > 0");
  if (c->pos_kind == GPT_POS_ROPE && (c->head_dim & 1)) return fail(GPT_ERR_ARG, "RoPE needs an even head_dim");
  if (c->dtype == GPT_DTYPE_BF16) {
    if (c->head_dim != 128) return fail(GPT_ERR_UNSUPPORTED, "bf16 path needs head_dim 128");
    if (c->n_head > 16) return fail(GPT_ERR_UNSUPPORTED, "bf16 path supports at most 16 query heads");
    if (c->pos_kind != GPT_POS_ROPE) return fail(GPT_ERR_UNSUPPORTED, "bf16 path uses rotary positions");
    if (c->act != GPT_ACT_RELU2) return fail(GPT_ERR_UNSUPPORTED, "bf16 path uses the ReLU^2 MLP");
    if (c->d_model % 128 || c->d_ff % 128 || c->vocab % 128)
      return fail(GPT_ERR_UNSUPPORTED, "bf16 path needs d_model, d_ff, vocab multiples of 128");
    // weight rows are addressed with 32-bit element offsets
    if ((long long)c->vocab * c->d_model >= (1LL << 31) || (long long)c->d_ff * c->d_model >= (1LL << 31))
      return fail(GPT_ERR_UNSUPPORTED, "bf16 path needs vocab x d_model and d_ff x d_model below 2^31");
  } else {
    if (c->head_dim > 64) return fail(GPT_ERR_UNSUPPORTED, "fp32 path needs head_dim <= 64");
    if (c->d_model % 4 || c->d_model > 4096) return fail(GPT_ERR_UNSUPPORTED, "fp32 path needs d_model % 4 == 0, <= 4096");
  }
  if (c->d_model != c->n_head * c->head_dim && c->dtype == GPT_DTYPE_BF16)
    return fail(GPT_ERR_UNSUPPORTED, "bf16 path needs d_model == n_head * head_dim");
  return GPT_OK;
}

// ------------------------------------------------------------------ workspace

struct Bufs {
  int *cu, *cu_pad, *lastrows, *seq, *pos, *vcol;
  float *x, *qkv, *lse_tmp, *opart, *mlpart, *dlogits, *lpart, *sel;
  float *tgt;      // target logits of the fused cross-entropy [M]
  float *llogits;  // logits for the cross-entropy where the LM head cannot fuse it
  float *slabs;   // partial products of split decode-row GEMMs
  unsigned *ctr;  // completion counters of decode attention
  int *dmap;      // decode-attention work list: [nseq * max_splits][kDecodeMapStride]
  void *h, *q, *k, *vt, *o, *u;
  long long ldvt;
  int max_splits;
};

long long b_ldvt(long long M, long long nseq) { return ((M + kPage * nseq) + 63) / 64 * 64; }

size_t carve(const gpt_config *c, long long M, long long nseq, char *base, Bufs *b) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char * {
    off = align256(off);
    char *p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  const long long d = c->d_model, H = c->n_head, Hkv = c->n_kv_head, dh = c->head_dim;
  const size_t es = c->dtype == GPT_DTYPE_BF16 ? 2 : 4;
  Bufs t{};
  t.cu = (int *)take((nseq + 1) * 4);
  t.cu_pad = (int *)take((nseq + 1) * 4);
  t.lastrows = (int *)take(nseq * 4);
  t.seq = (int *)take(M * 4);
  t.pos = (int *)take(M * 4);
  t.vcol = (int *)take(M * 4);
  t.x = (float *)take(M * d * 4);
  t.h = take(M * d * es);
  t.qkv = (float *)take(M * (H + 2 * Hkv) * dh * 4);
  t.q = take(M * H * dh * es);
  t.k = take(M * Hkv * dh * es);
  t.ldvt = b_ldvt(M, nseq);
  if (c->dtype == GPT_DTYPE_BF16) t.vt = take(Hkv * dh * t.ldvt * es);
  else t.vt = take(M * Hkv * dh * es);
  t.o = take(M * H * dh * es);
  t.u = take(M * (long long)c->d_ff * es);
  t.lse_tmp = (float *)take(M * 4);
  t.max_splits = (c->max_seq + 64 * kDecodeMinChunkPages - 1) / (64 * kDecodeMinChunkPages);
  t.opart = (float *)take(nseq * t.max_splits * H * dh * 4);
  t.mlpart = (float *)take(nseq * t.max_splits * H * 2 * 4);
  t.dmap = (int *)take(nseq * t.max_splits * kDecodeMapStride * 4);
  t.dlogits = (float *)take(nseq * (long long)c->vocab * 4);
  t.ctr = (unsigned *)take((size_t)kCounters * 4);
  t.slabs = (float *)take((size_t)kMaxRowSplit * std::min(M, 64LL) * std::max(d, (H + 2 * Hkv) * dh) * 4);
  t.sel = (float *)take((size_t)argmax_scratch_floats((int)nseq, c->vocab) * 4);
  t.lpart = (float *)take(M * (long long)((c->vocab + kLogitsPartCols - 1) / kLogitsPartCols) * 2 * 4);
  t.tgt = (float *)take(M * 4);
  // fp32 models and bf16 prefills of at most 64 rows compute the loss from
  // materialised logits (sized by min(M, 64) for bf16, so the total grows
  // with M)
  t.llogits = (float *)take((c->dtype == GPT_DTYPE_BF16 ? std::min(M, 64LL) : M) * (long long)c->vocab * 4);
  if (b) *b = t;
  return align256(off);
}

// Extra buffers of the loss backward, carved after the forward's.
struct TrainBufs {
  float *xs;        // [2L + 1][M][d] residual stream at each layer's input and middle, then the last
  float *logits;    // [M][V] fp32, or bf16 where the LM head fuses the softmax partials
  void *dl;         // [M][V] gradient of the logits (model dtype)
  void *trA, *trB;  // transposed operands of the weight-gradient GEMMs, rows of Mp
  void *wT;         // a transposed weight
  float *dx, *dh;   // [M][d] gradient of the residual stream; gradient of a norm's output
  void *dxb;        // [M][d] dx in the model dtype
  float *z, *du;    // [M][F]
  void *u, *dz;     // [M][F] model dtype
  float *dO, *dq, *dk, *dv, *lse, *dsum;
  void *dqkv;       // [M][(H + 2Hkv) dh] model dtype
  void *vb;         // [M][Hkv dh] bf16 V rows for the attention backward
  void *dob;        // [M][H dh] bf16 dO
  void *kt, *qt, *dot;  // transposed K, Q, dO (bf16, [dims][ldvt], V^T column order)
  float *dkp, *dvp; // [H][M][dh] per-query-head partial dK, dV
  float *ksl;       // k-split slabs of the weight-gradient GEMMs
  int *count;
  int Mp;
  // bf16: each layer's forward activations, kept for the backward: the
  // normed inputs h and h2, q, k, V^T, the attention output o and its
  // per-row base-2 log-sum-exp, and u = act(W1 h2).  Layer l's copy of a
  // buffer starts l times its size in.
  void *hl, *h2l, *ql, *kl, *vtl, *ol, *ul;
  float *lsel;
};

size_t carve_train(const gpt_config *c, long long M, long long nseq, char *base, Bufs *b, TrainBufs *tb) {
  size_t off = carve(c, M, nseq, base, b);
  auto take = [&](size_t bytes) -> char * {
    off = align256(off);
    char *p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  const long long d = c->d_model, H = c->n_head, Hkv = c->n_kv_head, dh = c->head_dim, F = c->d_ff, V = c->vocab;
  const long long L = c->n_layer, qkv_n = (H + 2 * Hkv) * dh;
  const size_t es = c->dtype == GPT_DTYPE_BF16 ? 2 : 4;
  TrainBufs t{};
  t.Mp = (int)((M + 63) / 64 * 64);
  const long long Mp = t.Mp;
  t.xs = (float *)take((2 * L + 1) * M * d * 4);
  // bf16 steps of more than 64 rows store bf16 logits; smaller ones fp32
  t.logits = (float *)take(c->dtype == GPT_DTYPE_BF16 ? std::max(M * V * 2, std::min(M, 64LL) * V * 4) : M * V * 4);
  t.dl = take(M * V * es);
  t.trA = take(std::max({V, F, qkv_n, d, H * dh}) * Mp * es);
  t.trB = take(std::max({d, F, H * dh}) * Mp * es);
  t.wT = take(std::max({V * d, F * d, qkv_n * d, H * dh * d}) * es);
  t.dx = (float *)take(M * d * 4);
  t.dh = (float *)take(M * d * 4);
  t.dxb = take(M * d * es);
  t.z = (float *)take(M * F * 4);
  t.du = (float *)take(M * F * 4);
  t.u = take(M * F * es);
  t.dz = take(M * F * es);
  t.dO = (float *)take(M * H * dh * 4);
  t.dq = (float *)take(M * H * dh * 4);
  t.dk = (float *)take(M * Hkv * dh * 4);
  t.dv = (float *)take(M * Hkv * dh * 4);
  t.lse = (float *)take(M * H * 4);
  t.dsum = (float *)take(M * H * 4);
  t.dqkv = take(M * qkv_n * es);
  t.vb = take(M * Hkv * dh * 2);
  if (c->dtype == GPT_DTYPE_BF16) {
    t.dob = take(M * H * dh * 2);
    t.kt = take(Hkv * dh * b_ldvt(M, nseq) * 2);
    t.qt = take(H * dh * b_ldvt(M, nseq) * 2);
    t.dot = take(H * dh * b_ldvt(M, nseq) * 2);
    t.dkp = (float *)take(H * M * dh * 4);
    t.dvp = (float *)take(H * M * dh * 4);
  }
  {
    // the weight-gradient GEMMs: [out][in] over K = Mp rows
    const long long shapes[6][2] = {{V, d}, {d, F}, {F, d}, {d, H * dh}, {H * dh, d}, {Hkv * dh, d}};
    long long most = 0;
    if (c->dtype == GPT_DTYPE_BF16)
      for (auto &sh : shapes) {
        const int ks = gemm_splitk_ways((int)sh[0], (int)sh[1], (int)Mp);
        if (ks > 1) most = std::max(most, ks * sh[0] * sh[1]);
      }
    t.ksl = (float *)take(most * 4);
  }
  t.count = (int *)take(4);
  if (c->dtype == GPT_DTYPE_BF16) {
    t.hl = take(L * M * d * 2);
    t.h2l = take(L * M * d * 2);
    t.ql = take(L * M * H * dh * 2);
    t.kl = take(L * M * Hkv * dh * 2);
    t.vtl = take(L * Hkv * dh * b_ldvt(M, nseq) * 2);
    t.ol = take(L * M * H * dh * 2);
    t.ul = take(L * M * F * 2);
    t.lsel = (float *)take(L * M * H * 4);
  }
  if (tb) *tb = t;
  return align256(off);
}

// ------------------------------------------------------------------ weights

gpt_status check_weights(const gpt_config *c, const gpt_weights *w) {
  if (!w) return fail(GPT_ERR_ARG, "weights is NULL");
  if (!w->wte || !w->lm_head) return fail(GPT_ERR_ARG, "wte and lm_head are required");
  if (c->pos_kind == GPT_POS_LEARNED && !w->wpe) return fail(GPT_ERR_ARG, "wpe is required for learned positions");
  if (!w->wq || !w->wk || !w->wv || !w->wo || !w->w1 || !w->w2)
    return fail(GPT_ERR_ARG, "per-layer weight arrays are required");
  const void *all[3] = {w->wte, w->lm_head, w->wpe};
  for (const void *p : all)
    if (p && !aligned16(p)) return fail(GPT_ERR_ARG, "weights must be 16-byte aligned");
  for (int l = 0; l < c->n_layer; ++l) {
    const void *lp[6] = {w->wq[l], w->wk[l], w->wv[l], w->wo[l], w->w1[l], w->w2[l]};
    for (const void *p : lp) {
      if (!p) return fail(GPT_ERR_ARG, "layer %d has a NULL weight", l);
      if (!aligned16(p)) return fail(GPT_ERR_ARG, "layer %d weight not 16-byte aligned", l);
    }
  }
  return GPT_OK;
}

// ------------------------------------------------------------------ prefill metadata

struct PrefillMeta {
  int n;
  int cu[kMaxPrefillSeqs + 1];
};

// One workgroup: device copies of cu_seqlens, the 64-padded offsets of the
// transposed-V columns, each sequence's last row; clears the counters.
__global__ void prefill_meta_kernel(PrefillMeta m, int *cu, int *cu_pad, int *lastrows,
                                    unsigned *ctr, int nctr) {
  if (ctr)
    for (int i = threadIdx.x; i < nctr; i += blockDim.x) ctr[i] = 0u;
  for (int i = threadIdx.x; i <= m.n; i += blockDim.x) cu[i] = m.cu[i];
  if (lastrows)
    for (int i = threadIdx.x; i < m.n; i += blockDim.x) lastrows[i] = m.cu[i + 1] - 1;
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < m.n; ++i) {
      cu_pad[i] = acc;
      acc += (m.cu[i + 1] - m.cu[i] + 63) / 64 * 64;
    }
    cu_pad[m.n] = acc;
  }
}

GemmArgs gemm(const void *A, long long lda, const void *W, int M, int N, int K, void *C, long long ldc,
              int epi) {
  GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.W0 = g.W1 = g.W2 = W;
  g.n1 = g.n2 = N;
  g.ldw = K;
  g.M = M;
  g.N = N;
  g.K = K;
  g.C = C;
  g.ldc = ldc;
  g.epi = epi;
  return g;
}

void run_gemm(const gpt_config *c, const GemmArgs &g, int cls, hipStream_t s) {
  const double es = c->dtype == GPT_DTYPE_BF16 ? 2.0 : 4.0;
  double out_b = g.epi == EPI_RESID ? 8.0
                 : g.epi == EPI_DRELU2 ? 4.0 + es  // reads z, writes dz
                 : (g.epi == EPI_BF16 || g.epi == EPI_RELU2_BF16 || g.epi == EPI_QKV || g.epi == EPI_LOGITS_BF16)
                     ? es
                     : 4.0;
  bool rows = c->dtype == GPT_DTYPE_BF16 && g.M <= 64;
  Timed t(rows && cls == GPT_PROF_GEMM ? GPT_PROF_SKINNY : cls, s, 2.0 * g.M * g.N * g.K,
          es * ((double)g.M * g.K + (double)g.N * g.K) + out_b * g.M * g.N);
  if (c->dtype == GPT_DTYPE_F32) launch_gemm_f32(g, s);
  else if (rows) launch_gemm_bf16_rows(g, 1, 0, s);
  else launch_gemm_bf16(g, s);
}

// Decode-row GEMM (bf16, M <= 64) with its k range split ks ways into fp32
// slabs `slab` floats apart (EPI_F32); bytes counted are the algorithmic
// ones (operands and one fp32 output).
void run_gemm_rows(const GemmArgs &g, int ks, long long slab, int cls, hipStream_t s) {
  Timed t(cls == GPT_PROF_GEMM ? GPT_PROF_SKINNY : cls, s, 2.0 * g.M * g.N * g.K,
          2.0 * ((double)g.M * g.K + (double)g.N * g.K) + 4.0 * g.M * g.N);
  launch_gemm_bf16_rows(g, ks, slab, s);
}

PagedKV paged_view(const gpt_kv_cache *kv);

}  // namespace

// ------------------------------------------------------------------ KV cache handle

struct gpt_kv_cache {
  gpt_config cfg;
  int n_seqs, capacity, page_size, pps;
  char *buf;
  size_t bytes, table_off, lens_off;
  long long layer_stride, page_stride, half_bytes;
  std::vector<int> lens;
};

namespace {
PagedKV paged_view(const gpt_kv_cache *kv) {
  PagedKV p{};
  p.base = kv->buf;
  p.table = (const int *)(kv->buf + kv->table_off);
  p.lens = (int *)(kv->buf + kv->lens_off);
  p.layer_stride = kv->layer_stride;
  p.page_stride = kv->page_stride;
  p.half_bytes = kv->half_bytes;
  p.pages_per_seq = kv->pps;
  p.page_size = kv->page_size;
  return p;
}
}  // namespace

extern "C" {

const char *gpt_last_error(void) { return g_err.c_str(); }

gpt_status rope_tables(int32_t max_seq, int32_t head_dim, float base, float *cos_out, float *sin_out,
                       gpt_stream_t stream) {
  if (max_seq <= 0) return fail(GPT_ERR_ARG, "max_seq must be positive");
  if (head_dim <= 0 || (head_dim & 1)) return fail(GPT_ERR_ARG, "head_dim must be positive and even");
  if (!(base > 0.f)) return fail(GPT_ERR_ARG, "base must be positive");
  if (!cos_out || !sin_out) return fail(GPT_ERR_ARG, "outputs are NULL");
  const int half = head_dim / 2;
  std::vector<float> cs((size_t)max_seq * half), sn((size_t)max_seq * half);
  for (int i = 0; i < half; ++i) {
    const double inv_freq = std::pow((double)base, -2.0 * i / head_dim);
    for (int t = 0; t < max_seq; ++t) {
      const double ang = (double)t * inv_freq;
      cs[(size_t)t * half + i] = (float)std::cos(ang);
      sn[(size_t)t * half + i] = (float)std::sin(ang);
    }
  }
  hipStream_t s = (hipStream_t)stream;
  const size_t bytes = cs.size() * sizeof(float);
  if (hipMemcpyAsync(cos_out, cs.data(), bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(sin_out, sn.data(), bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return hip_check("rope_tables copy");
  return GPT_OK;
}

gpt_status kv_cache_alloc(const gpt_config *c, int32_t n_seqs, int32_t capacity_per_seq, int32_t page_size,
                          void *device_buf, size_t *bytes_inout, gpt_kv_cache **out) {
  gpt_status st = check_config(c);
  if (st) return st;
  if (!bytes_inout) return fail(GPT_ERR_ARG, "bytes_inout is NULL");
  if (n_seqs <= 0 || capacity_per_seq <= 0) return fail(GPT_ERR_ARG, "n_seqs and capacity must be positive");
  if (capacity_per_seq > c->max_seq) return fail(GPT_ERR_ARG, "capacity exceeds max_seq");
  if (c->dtype == GPT_DTYPE_BF16 && capacity_per_seq > kDecodeMaxPositions)
    return fail(GPT_ERR_UNSUPPORTED, "bf16 decode supports at most %d cached positions per sequence",
                kDecodeMaxPositions);
  if (page_size != kPage) return fail(GPT_ERR_UNSUPPORTED, "page_size must be 64");
  const long long pps = (capacity_per_seq + page_size - 1) / page_size;
  const long long n_pages = pps * n_seqs;
  const long long es = c->dtype == GPT_DTYPE_BF16 ? 2 : 4;
  const long long half = (long long)page_size * c->n_kv_head * c->head_dim * es;
  const long long layer_stride = n_pages * 2 * half;
  const size_t table_off = align256((size_t)(layer_stride * c->n_layer));
  const size_t lens_off = align256(table_off + (size_t)n_pages * 4);
  const size_t need = align256(lens_off + (size_t)n_seqs * 4);
  if (!device_buf) {
    *bytes_inout = need;
    return GPT_OK;
  }
  if (!out) return fail(GPT_ERR_ARG, "out is NULL");
  if (*bytes_inout < need) return fail(GPT_ERR_ARG, "buffer too small: %zu < %zu bytes", *bytes_inout, need);
  if (reinterpret_cast<uintptr_t>(device_buf) & 255) return fail(GPT_ERR_ARG, "buffer must be 256-byte aligned");
  std::vector<int> table(n_pages);
  for (long long i = 0; i < n_pages; ++i) table[i] = (int)i;
  char *buf = (char *)device_buf;
  if (hipMemcpy(buf + table_off, table.data(), table.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(buf + lens_off, 0, (size_t)n_seqs * 4) != hipSuccess)
    return hip_check("kv_cache_alloc init");
  gpt_kv_cache *kv = new gpt_kv_cache();
  kv->cfg = *c;
  kv->n_seqs = n_seqs;
  kv->capacity = capacity_per_seq;
  kv->page_size = page_size;
  kv->pps = (int)pps;
  kv->buf = buf;
  kv->bytes = *bytes_inout;
  kv->table_off = table_off;
  kv->lens_off = lens_off;
  kv->layer_stride = layer_stride;
  kv->page_stride = 2 * half;
  kv->half_bytes = half;
  kv->lens.assign(n_seqs, 0);
  *out = kv;
  return GPT_OK;
}

gpt_status kv_cache_free(gpt_kv_cache *kv) {
  if (!kv) return fail(GPT_ERR_ARG, "kv is NULL");
  delete kv;
  return GPT_OK;
}

gpt_status kv_cache_lengths(const gpt_kv_cache *kv, int32_t *lens_out) {
  if (!kv || !lens_out) return fail(GPT_ERR_ARG, "NULL argument");
  std::copy(kv->lens.begin(), kv->lens.end(), lens_out);
  return GPT_OK;
}

size_t gpt_workspace_bytes(const gpt_config *c, int32_t max_tokens, int32_t max_seqs) {
  if (check_config(c) != GPT_OK || max_tokens <= 0 || max_seqs <= 0) return 0;
  return carve(c, max_tokens, max_seqs, nullptr, nullptr);
}

}  // extern "C"

namespace {

// ------------------------------------------------------------------ forward layers
// What a prefill forward's layers need: the model, the rotary tables, the
// carved buffers (the residual stream is bf->x), the cache view and the
// stream.
struct Fwd {
  const gpt_config *c;
  const gpt_weights *w;
  const float *cos, *sin;
  Bufs *bf;
  PagedKV pv;
  bool use_cache;
  int M, n_seqs, max_len;
  double attn_flops;
  hipStream_t s;
  float *lse2;  // bf16 attention: each row's base-2 log-sum-exp, or NULL
  float *x_out; // residual GEMMs write bf->x + f(bf->x) here instead of in place, or NULL
};

Fwd make_fwd(const gpt_config *c, const gpt_weights *w, const float *rope_cos, const float *rope_sin, Bufs *bf,
             PagedKV pv, bool use_cache, int M, int n_seqs, const int32_t *cu_seqlens, hipStream_t s) {
  Fwd f{};
  f.c = c;
  f.w = w;
  f.cos = c->pos_kind == GPT_POS_ROPE ? rope_cos : nullptr;
  f.sin = c->pos_kind == GPT_POS_ROPE ? rope_sin : nullptr;
  f.bf = bf;
  f.pv = pv;
  f.use_cache = use_cache;
  f.M = M;
  f.n_seqs = n_seqs;
  for (int b = 0; b < n_seqs; ++b) {
    const double L = cu_seqlens[b + 1] - cu_seqlens[b];
    f.max_len = std::max(f.max_len, cu_seqlens[b + 1] - cu_seqlens[b]);
    f.attn_flops += 4.0 * c->n_head * c->head_dim * L * (L + 1) / 2;
  }
  f.s = s;
  return f;
}

// h = RMSNorm(x) (bf16 or fp32 per the model dtype)
void fwd_norm(const Fwd &f, const float *x, void *h) {
  const gpt_config *c = f.c;
  const bool bf16p = c->dtype == GPT_DTYPE_BF16;
  Timed t(GPT_PROF_NORM, f.s, 0, (double)f.M * c->d_model * (4 + (bf16p ? 2 : 4)));
  if (bf16p) launch_rmsnorm_bf16(x, (bf16 *)h, nullptr, f.M, c->d_model, c->norm_eps, f.s);
  else launch_rmsnorm_f32(x, (float *)h, nullptr, f.M, c->d_model, c->norm_eps, f.s);
}

// q, k, v of layer l from h = bf->h: q -> bf->q, k -> bf->k, v -> bf->vt
// (transposed for bf16), after RoPE and QK-norm, and into the cache when
// there is one.  fused: in the GEMM's epilogue; otherwise the fp32
// projection goes to bf->qkv first and a scatter kernel finishes.
void fwd_qkv(const Fwd &f, int l, bool fused) {
  const gpt_config *c = f.c;
  Bufs &bf = *f.bf;
  const bool bf16p = c->dtype == GPT_DTYPE_BF16;
  const int d = c->d_model, H = c->n_head, Hkv = c->n_kv_head, dh = c->head_dim;
  const int qkv_n = (H + 2 * Hkv) * dh, M = f.M;
  GemmArgs g = gemm(bf.h, d, f.w->wq[l], M, qkv_n, d, bf.qkv, qkv_n, fused ? EPI_QKV : EPI_F32);
  g.W1 = f.w->wk[l];
  g.W2 = f.w->wv[l];
  g.n1 = H * dh;
  g.n2 = (H + Hkv) * dh;
  if (fused) {
    QkvEpi &e = g.qkv;
    e.seq = bf.seq;
    e.pos = bf.pos;
    e.vcol = bf.vcol;
    e.cos = f.cos;
    e.sin = f.sin;
    e.eps = c->norm_eps;
    e.qk_norm = c->qk_norm;
    e.H = H;
    e.Hkv = Hkv;
    e.q_out = (bf16 *)bf.q;
    e.k_out = (bf16 *)bf.k;
    e.vt_out = (bf16 *)bf.vt;
    e.ldvt = bf.ldvt;
    e.kv = f.pv;
    e.layer = l;
    e.use_cache = f.use_cache;
  }
  run_gemm(c, g, GPT_PROF_GEMM, f.s);
  if (fused) return;
  ScatterArgs sa{};
  sa.qkv = bf.qkv;
  sa.M = M;
  sa.H = H;
  sa.Hkv = Hkv;
  sa.seq = bf.seq;
  sa.pos = bf.pos;
  sa.vcol = bf.vcol;
  sa.cos = f.cos;
  sa.sin = f.sin;
  sa.qk_norm = c->qk_norm;
  sa.eps = c->norm_eps;
  sa.q_out = bf.q;
  sa.k_out = bf.k;
  sa.vt_out = bf.vt;
  sa.ldvt = bf.ldvt;
  sa.kv = f.pv;
  sa.layer = l;
  sa.use_cache = f.use_cache;
  sa.head_dim = dh;
  Timed t(GPT_PROF_NORM, f.s, 0, (double)M * qkv_n * 4 + (double)M * qkv_n * (bf16p ? 2 : 4));
  if (bf16p) launch_rope_norm_scatter_bf16(sa, f.s);
  else launch_qkv_scatter_f32(sa, f.s);
}

// o = causal attention of bf->q against bf->k, bf->vt
void fwd_attention(const Fwd &f) {
  const gpt_config *c = f.c;
  Bufs &bf = *f.bf;
  const bool bf16p = c->dtype == GPT_DTYPE_BF16;
  const int H = c->n_head, Hkv = c->n_kv_head, dh = c->head_dim;
  Timed t(GPT_PROF_ATTN, f.s, f.attn_flops, (double)f.M * (H + 2 * Hkv + H) * dh * (bf16p ? 2 : 4));
  if (bf16p) {
    AttnPrefillArgs aa{};
    aa.q = (const bf16 *)bf.q;
    aa.k = (const bf16 *)bf.k;
    aa.vt = (const bf16 *)bf.vt;
    aa.ldvt = bf.ldvt;
    aa.cu = bf.cu;
    aa.cu_pad = bf.cu_pad;
    aa.H = H;
    aa.Hkv = Hkv;
    aa.qk_norm = c->qk_norm;
    aa.n_seqs = f.n_seqs;
    aa.max_wg = (f.max_len * (H / Hkv) + kAttnPrefillRows - 1) / kAttnPrefillRows;
    aa.o = (bf16 *)bf.o;
    aa.lse2 = f.lse2;
    launch_attn_prefill_bf16(aa, f.s);
  } else {
    AttnF32Args aa{};
    aa.q = (const float *)bf.q;
    aa.k = (const float *)bf.k;
    aa.v = (const float *)bf.vt;
    aa.seq = bf.seq;
    aa.pos = bf.pos;
    aa.M = f.M;
    aa.H = H;
    aa.Hkv = Hkv;
    aa.dh = dh;
    aa.o = (float *)bf.o;
    launch_attn_prefill_f32(aa, f.s);
  }
}

// x += Wo Attn(q, k, v) with q, k, v from RMSNorm(x): the first half of layer l
void fwd_attn_half(const Fwd &f, int l) {
  const gpt_config *c = f.c;
  Bufs &bf = *f.bf;
  const int d = c->d_model, H = c->n_head, dh = c->head_dim;
  fwd_norm(f, bf.x, bf.h);
  fwd_qkv(f, l, c->dtype == GPT_DTYPE_BF16 && f.M > 64);
  fwd_attention(f);
  GemmArgs g = gemm(bf.o, H * dh, f.w->wo[l], f.M, d, H * dh, f.x_out ? f.x_out : bf.x, d, EPI_RESID);
  if (f.x_out) g.rin = bf.x;
  run_gemm(c, g, GPT_PROF_GEMM, f.s);
}

// x += W2 act(W1 RMSNorm(x)): the second half of layer l
void fwd_mlp_half(const Fwd &f, int l) {
  const gpt_config *c = f.c;
  Bufs &bf = *f.bf;
  const bool bf16p = c->dtype == GPT_DTYPE_BF16;
  const int d = c->d_model, F = c->d_ff, M = f.M;
  fwd_norm(f, bf.x, bf.h);
  run_gemm(c, gemm(bf.h, d, f.w->w1[l], M, F, d, bf.u, F,
                   bf16p ? EPI_RELU2_BF16 : (c->act == GPT_ACT_RELU ? EPI_RELU_F32 : EPI_RELU2_BF16)),
           GPT_PROF_GEMM, f.s);
  GemmArgs g = gemm(bf.u, F, f.w->w2[l], M, d, F, f.x_out ? f.x_out : bf.x, d, EPI_RESID);
  if (f.x_out) g.rin = bf.x;
  run_gemm(c, g, GPT_PROF_GEMM, f.s);
}

// Prefill forward.  Logits mode (targets == NULL): logits of `logits_rows`
// rows, optional lse and probs.  Loss mode: every row's cross-entropy
// against targets into loss (optional lse, mean); logits is unused.
gpt_status prefill_impl(const gpt_config *c, const gpt_weights *w, const float *rope_cos, const float *rope_sin,
                        const int32_t *tokens, const int32_t *cu_seqlens, int32_t n_seqs, gpt_kv_cache *kv,
                        int32_t logits_rows, float *logits, float *lse, float *probs, const int32_t *targets,
                        float *loss, float *mean, void *workspace, size_t workspace_bytes, gpt_stream_t stream) {
  gpt_status st = check_config(c);
  if (st) return st;
  if ((st = check_weights(c, w))) return st;
  const bool loss_mode = targets != nullptr;
  if (!tokens || !cu_seqlens || !workspace || (loss_mode ? !loss : !logits))
    return fail(GPT_ERR_ARG, "NULL required pointer");
  if (n_seqs <= 0) return fail(GPT_ERR_ARG, "n_seqs must be positive");
  if (n_seqs > kMaxPrefillSeqs) return fail(GPT_ERR_UNSUPPORTED, "at most %d sequences per prefill", kMaxPrefillSeqs);
  if (logits_rows != GPT_ROWS_ALL && logits_rows != GPT_ROWS_LAST) return fail(GPT_ERR_ARG, "bad logits_rows");
  if (c->pos_kind == GPT_POS_ROPE && (!rope_cos || !rope_sin)) return fail(GPT_ERR_ARG, "RoPE tables required");
  if (cu_seqlens[0] != 0) return fail(GPT_ERR_ARG, "cu_seqlens[0] must be 0");
  for (int b = 0; b < n_seqs; ++b) {
    const int len = cu_seqlens[b + 1] - cu_seqlens[b];
    if (len <= 0) return fail(GPT_ERR_ARG, "sequence %d is empty or cu_seqlens decreases", b);
    if (len > c->max_seq) return fail(GPT_ERR_ARG, "sequence %d longer than max_seq", b);
  }
  const int M = cu_seqlens[n_seqs];
  {
    // the tiled GEMM and the row kernels address an activation operand with
    // 32-bit element offsets (row x width)
    const long long widest = std::max({(long long)c->d_model, (long long)c->d_ff,
                                       (long long)c->n_head * c->head_dim});
    if (widest * M >= (1LL << 31))
      return fail(GPT_ERR_UNSUPPORTED, "%d rows x %lld columns exceed the 32-bit operand offsets", M, widest);
  }
  if (kv) {
    if (kv->n_seqs != n_seqs) return fail(GPT_ERR_ARG, "n_seqs %d != kv cache's %d", n_seqs, kv->n_seqs);
    if (kv->cfg.n_layer != c->n_layer || kv->cfg.dtype != c->dtype || kv->cfg.n_kv_head != c->n_kv_head ||
        kv->cfg.head_dim != c->head_dim)
      return fail(GPT_ERR_ARG, "kv cache was made for another config");
    for (int b = 0; b < n_seqs; ++b)
      if (cu_seqlens[b + 1] - cu_seqlens[b] > kv->capacity)
        return fail(GPT_ERR_CAPACITY, "sequence %d exceeds the cache capacity %d", b, kv->capacity);
  }
  const size_t need = carve(c, M, n_seqs, nullptr, nullptr);
  if (workspace_bytes < need) return fail(GPT_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(GPT_ERR_ARG, "workspace must be 256-byte aligned");
  if (!loss_mode && (!aligned16(logits) || (probs && !aligned16(probs))))
    return fail(GPT_ERR_ARG, "logits/probs must be 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  hipGetLastError();  // clear any stale error from unrelated work
  Bufs bf;
  carve(c, M, n_seqs, (char *)workspace, &bf);
  const bool bf16p = c->dtype == GPT_DTYPE_BF16;
  const int d = c->d_model, H = c->n_head, Hkv = c->n_kv_head, dh = c->head_dim, F = c->d_ff, V = c->vocab;
  const int qkv_n = (H + 2 * Hkv) * dh;
  const int rows = logits_rows == GPT_ROWS_ALL ? M : n_seqs;

  PrefillMeta meta;
  meta.n = n_seqs;
  for (int b = 0; b <= n_seqs; ++b) meta.cu[b] = cu_seqlens[b];
  {
    Timed t(GPT_PROF_NORM, s, 0, 0);
    prefill_meta_kernel<<<1, 256, 0, s>>>(meta, bf.cu, bf.cu_pad, bf.lastrows, bf.ctr, kCounters);
    launch_rowinfo(bf.cu, bf.cu_pad, n_seqs, M, bf.seq, bf.pos, bf.vcol, s);
  }
  PagedKV pv{};
  if (kv) pv = paged_view(kv);
  {
    Timed t(GPT_PROF_NORM, s, 0, (double)M * d * (4 + (bf16p ? 2 : 4)));
    if (bf16p) launch_embed_bf16(tokens, (const bf16 *)w->wte, bf.x, M, d, s);
    else launch_embed_f32(tokens, (const float *)w->wte, (const float *)w->wpe, bf.pos, bf.x, M, d, s);
  }
  Fwd fw = make_fwd(c, w, rope_cos, rope_sin, &bf, pv, kv != nullptr, M, n_seqs, cu_seqlens, s);
  for (int l = 0; l < c->n_layer; ++l) {
    fwd_attn_half(fw, l);
    fwd_mlp_half(fw, l);
  }
  {
    Timed t(GPT_PROF_NORM, s, 0, (double)rows * d * (4 + (bf16p ? 2 : 4)));
    const int *sel = logits_rows == GPT_ROWS_ALL ? nullptr : bf.lastrows;
    if (bf16p) launch_rmsnorm_bf16(bf.x, (bf16 *)bf.h, sel, rows, d, c->norm_eps, s);
    else launch_rmsnorm_f32(bf.x, (float *)bf.h, sel, rows, d, c->norm_eps, s);
  }
  if (loss_mode) {
    // next-token cross-entropy of every row without materialising the
    // logits when the LM head runs on the large-M kernel
    if (bf16p && rows > 64) {
      GemmArgs lg = gemm(bf.h, d, w->lm_head, rows, V, d, nullptr, V, EPI_LOSS);
      lg.part = bf.lpart;
      lg.targets = targets;
      lg.tgt = bf.tgt;
      {
        Timed t(GPT_PROF_LMHEAD, s, 2.0 * rows * V * d,
                2.0 * ((double)rows * d + (double)V * d) + (double)rows * (V / kLogitsPartCols) * 8);
        launch_gemm_bf16(lg, s);
      }
      Timed t(GPT_PROF_SOFTMAX, s, 0, (double)rows * (V / kLogitsPartCols) * 8 + (double)rows * 12);
      launch_ce_from_parts(bf.lpart, V / kLogitsPartCols, bf.tgt, targets, V, rows, loss, lse, s);
    } else {
      run_gemm(c, gemm(bf.h, d, w->lm_head, rows, V, d, bf.llogits, V, EPI_F32), GPT_PROF_LMHEAD, s);
      Timed t(GPT_PROF_SOFTMAX, s, 0, (double)rows * V * 4 + (double)rows * 12);
      launch_softmax_lse(bf.llogits, rows, V, lse ? lse : bf.lse_tmp, nullptr, s);
      launch_ce_from_logits(bf.llogits, lse ? lse : bf.lse_tmp, targets, V, rows, loss, s);
    }
    if (mean) launch_mean_loss(loss, targets, V, rows, mean, s);
    if (kv) launch_lens_set(pv.lens, bf.cu, n_seqs, s);
    if ((st = hip_check("gpt_prefill_loss launch"))) return st;
    if (kv)
      for (int b = 0; b < n_seqs; ++b) kv->lens[b] = cu_seqlens[b + 1] - cu_seqlens[b];
    return GPT_OK;
  }
  const bool want_lse = lse || probs;
  const bool fused_lse = want_lse && bf16p && rows > 64;
  GemmArgs lg = gemm(bf.h, d, w->lm_head, rows, V, d, logits, V, fused_lse ? EPI_LOGITS : EPI_F32);
  lg.part = bf.lpart;
  run_gemm(c, lg, GPT_PROF_LMHEAD, s);
  if (fused_lse) {
    Timed t(GPT_PROF_SOFTMAX, s, 0, (double)rows * (V / kLogitsPartCols) * 8 + (probs ? (double)rows * V * 8 : 0.0));
    launch_lse_combine(bf.lpart, V / kLogitsPartCols, rows, lse ? lse : bf.lse_tmp, logits, V, probs, s);
  } else if (want_lse) {
    Timed t(GPT_PROF_SOFTMAX, s, 0, (double)rows * V * 4 * (probs ? 3 : 1));
    launch_softmax_lse(logits, rows, V, lse ? lse : bf.lse_tmp, probs, s);
  }
  if (kv) launch_lens_set(pv.lens, bf.cu, n_seqs, s);
  if ((st = hip_check("gpt_prefill launch"))) return st;
  if (kv)
    for (int b = 0; b < n_seqs; ++b) kv->lens[b] = cu_seqlens[b + 1] - cu_seqlens[b];
  return GPT_OK;
}
// dst[c][r] = src[r][c] in the model dtype
void tr_md(const gpt_config *c, const void *src, long long lds, int R, int C, void *dst, long long ldd, int Rp,
           hipStream_t s) {
  if (c->dtype == GPT_DTYPE_BF16)
    launch_transpose<bf16, bf16>((const bf16 *)src, lds, R, C, (bf16 *)dst, ldd, Rp, s);
  else launch_transpose<float, float>((const float *)src, lds, R, C, (float *)dst, ldd, Rp, s);
}

// Mean next-token loss and its gradient for every weight.  Forward: the
// prefill's layers, keeping the residual stream at each layer's input and
// middle, then the materialised logits.  Backward: everything else is
// recomputed per layer from the kept residual stream.  Linear layers
// y = X W^T take dX = dY W and dW = dY^T X, both on the forward's GEMM
// kernels with transposed copies of W, dY and X.
gpt_status loss_grads_impl(const gpt_config *c, const gpt_weights *w, const float *rope_cos, const float *rope_sin,
                           const int32_t *tokens, const int32_t *targets, const int32_t *cu_seqlens, int32_t n_seqs,
                           const gpt_grads *gr, float *loss, float *mean, void *workspace, size_t workspace_bytes,
                           gpt_stream_t stream) {
  gpt_status st = check_config(c);
  if (st) return st;
  if ((st = check_weights(c, w))) return st;
  if (!tokens || !targets || !cu_seqlens || !gr || !loss || !workspace) return fail(GPT_ERR_ARG, "NULL required pointer");
  if (!gr->wte || !gr->lm_head || !gr->wq || !gr->wk || !gr->wv || !gr->wo || !gr->w1 || !gr->w2)
    return fail(GPT_ERR_ARG, "NULL gradient pointer");
  if (c->pos_kind == GPT_POS_LEARNED && !gr->wpe) return fail(GPT_ERR_ARG, "wpe gradient required");
  for (int l = 0; l < c->n_layer; ++l)
    if (!gr->wq[l] || !gr->wk[l] || !gr->wv[l] || !gr->wo[l] || !gr->w1[l] || !gr->w2[l])
      return fail(GPT_ERR_ARG, "layer %d gradient pointer is NULL", l);
  if (n_seqs <= 0) return fail(GPT_ERR_ARG, "n_seqs must be positive");
  if (n_seqs > kMaxPrefillSeqs) return fail(GPT_ERR_UNSUPPORTED, "at most %d sequences", kMaxPrefillSeqs);
  if (c->pos_kind == GPT_POS_ROPE && (!rope_cos || !rope_sin)) return fail(GPT_ERR_ARG, "RoPE tables required");
  if (c->head_dim > 128) return fail(GPT_ERR_UNSUPPORTED, "head_dim above 128");
  if (cu_seqlens[0] != 0) return fail(GPT_ERR_ARG, "cu_seqlens[0] must be 0");
  for (int b = 0; b < n_seqs; ++b) {
    const int len = cu_seqlens[b + 1] - cu_seqlens[b];
    if (len <= 0) return fail(GPT_ERR_ARG, "sequence %d is empty or cu_seqlens decreases", b);
    if (len > c->max_seq) return fail(GPT_ERR_ARG, "sequence %d longer than max_seq", b);
  }
  const int M = cu_seqlens[n_seqs];
  {
    // the GEMM kernels address an operand with 32-bit element offsets
    const long long Mp = (M + 63) / 64 * 64;
    const long long widest = std::max({(long long)c->vocab, (long long)c->d_ff,
                                       (long long)(c->n_head + 2 * c->n_kv_head) * c->head_dim});
    if (widest * Mp >= (1LL << 31))
      return fail(GPT_ERR_UNSUPPORTED, "%d rows x %lld columns exceed the backward's 32-bit operand offsets", M,
                  widest);
  }
  const size_t need = carve_train(c, M, n_seqs, nullptr, nullptr, nullptr);
  if (workspace_bytes < need) return fail(GPT_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(GPT_ERR_ARG, "workspace must be 256-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  hipGetLastError();
  Bufs bf;
  TrainBufs tb;
  carve_train(c, M, n_seqs, (char *)workspace, &bf, &tb);
  const bool bf16p = c->dtype == GPT_DTYPE_BF16;
  const int d = c->d_model, H = c->n_head, Hkv = c->n_kv_head, dh = c->head_dim, F = c->d_ff, V = c->vocab;
  const int L = c->n_layer, qkv_n = (H + 2 * Hkv) * dh, Mp = tb.Mp;
  const size_t es = bf16p ? 2 : 4;
  auto xs = [&](int i) { return tb.xs + (long long)i * M * d; };
  // C[M][N] = A[M][K] B[N][K]^T into fp32
  auto mm = [&](const void *A, long long lda, const void *B, long long ldb, int m, int n, int k, float *C,
                long long ldc) {
    GemmArgs g = gemm(A, lda, B, m, n, k, C, ldc, EPI_F32);
    g.ldw = ldb;
    run_gemm(c, g, GPT_PROF_BWD_GEMM, s);
  };
  // weight gradient dW[m][n] = sum over the Mp rows of A^T[m][.] B^T[n][.]: k split where the
  // [m][n] tiling alone leaves CUs idle
  auto mmw = [&](const void *A, const void *Bt, int m, int n, float *C) {
    if (!bf16p) {
      mm(A, Mp, Bt, Mp, m, n, Mp, C, n);
      return;
    }
    GemmArgs g = gemm(A, Mp, Bt, m, n, Mp, C, n, EPI_F32);
    Timed t(GPT_PROF_BWD_GEMM, s, 2.0 * m * n * Mp, 2.0 * ((double)m + n) * Mp + 4.0 * m * n);
    launch_gemm_bf16_splitk(g, gemm_splitk_ways(m, n, Mp), tb.ksl, s);
  };
  // dx in the model dtype: the bf16 copy the RMSNorm backward keeps, or dx itself
  auto dxA0 = [&]() -> const void * { return bf16p ? tb.dxb : (const void *)tb.dx; };
  // dx += the RMSNorm backward; bf16 models also get dx in bf16 (tb.dxb),
  // the A operand of the next input-gradient GEMM
  auto rms_bwd = [&](const float *x, const float *dy) {
    Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)M * d * (16 + (bf16p ? 2 : 0)));
    launch_rms_bwd(x, dy, tb.dx, bf16p ? (bf16 *)tb.dxb : nullptr, M, d, c->norm_eps, s);
  };

  // ---- forward, keeping the residual stream
  PrefillMeta meta;
  meta.n = n_seqs;
  for (int b = 0; b <= n_seqs; ++b) meta.cu[b] = cu_seqlens[b];
  {
    Timed t(GPT_PROF_NORM, s, 0, 0);
    prefill_meta_kernel<<<1, 256, 0, s>>>(meta, bf.cu, bf.cu_pad, bf.lastrows, bf.ctr, kCounters);
    launch_rowinfo(bf.cu, bf.cu_pad, n_seqs, M, bf.seq, bf.pos, bf.vcol, s);
  }
  // The residual stream lives in the kept buffers: the embedding writes
  // xs(0), and each half-layer's residual GEMM writes xs(i + 1) = xs(i) + f.
  bf.x = xs(0);
  {
    Timed t(GPT_PROF_NORM, s, 0, (double)M * d * (4 + es));
    if (bf16p) launch_embed_bf16(tokens, (const bf16 *)w->wte, bf.x, M, d, s);
    else launch_embed_f32(tokens, (const float *)w->wte, (const float *)w->wpe, bf.pos, bf.x, M, d, s);
  }
  Fwd fw = make_fwd(c, w, rope_cos, rope_sin, &bf, PagedKV{}, false, M, n_seqs, cu_seqlens, s);
  // bf16 prefills on the large-M kernels keep every layer's activations
  // (tb.hl ...) and the backward recomputes only the QKV projection; the
  // others keep the residual stream alone and recompute each layer.
  const bool keep = bf16p && M > 64;
  const Bufs bf0 = bf;
  auto layer_ptr = [&](void *base, long long elems, size_t esz, int l) -> void * {
    return (char *)base + (size_t)l * elems * esz;
  };
  auto h_l = [&](int l) { return layer_ptr(tb.hl, (long long)M * d, 2, l); };
  auto h2_l = [&](int l) { return layer_ptr(tb.h2l, (long long)M * d, 2, l); };
  auto q_l = [&](int l) { return layer_ptr(tb.ql, (long long)M * H * dh, 2, l); };
  auto k_l = [&](int l) { return layer_ptr(tb.kl, (long long)M * Hkv * dh, 2, l); };
  auto vt_l = [&](int l) { return layer_ptr(tb.vtl, (long long)Hkv * dh * bf.ldvt, 2, l); };
  auto o_l = [&](int l) { return layer_ptr(tb.ol, (long long)M * H * dh, 2, l); };
  auto u_l = [&](int l) { return layer_ptr(tb.ul, (long long)M * F, 2, l); };
  auto lse_l = [&](int l) { return (float *)layer_ptr(tb.lsel, (long long)M * H, 4, l); };
  for (int l = 0; l < L; ++l) {
    if (keep) {
      bf.h = h_l(l);
      bf.q = q_l(l);
      bf.k = k_l(l);
      bf.vt = vt_l(l);
      bf.o = o_l(l);
      fw.lse2 = lse_l(l);
    }
    fw.x_out = xs(2 * l + 1);
    fwd_attn_half(fw, l);
    bf.x = xs(2 * l + 1);
    if (keep) {
      bf.h = h2_l(l);
      bf.u = u_l(l);
    }
    fw.x_out = xs(2 * l + 2);
    fwd_mlp_half(fw, l);
    bf.x = xs(2 * l + 2);
  }
  bf = bf0;
  fw.lse2 = nullptr;
  fw.x_out = nullptr;
  fwd_norm(fw, xs(2 * L), bf.h);  // hf
  // Large M in bf16: the LM head stores the logits in bf16 (the precision
  // the softmax gradient is rounded to anyway) with the softmax partials and
  // each row's fp32 target logit, from which the loss comes; the gradient
  // kernel then writes dl and its transpose in one pass.
  const bool fused_lse = bf16p && M > 64;
  {
    GemmArgs lg = gemm(bf.h, d, w->lm_head, M, V, d, tb.logits, V, fused_lse ? EPI_LOGITS_BF16 : EPI_F32);
    lg.part = bf.lpart;
    lg.targets = targets;
    lg.tgt = bf.tgt;
    run_gemm(c, lg, GPT_PROF_LMHEAD, s);
    if (fused_lse) {
      Timed t(GPT_PROF_SOFTMAX, s, 0, (double)M * (V / kLogitsPartCols) * 8 + (double)M * 12);
      launch_ce_from_parts(bf.lpart, V / kLogitsPartCols, bf.tgt, targets, V, M, loss, bf.lse_tmp, s);
    } else {
      Timed t(GPT_PROF_SOFTMAX, s, 0, (double)M * V * 4);
      launch_softmax_lse(tb.logits, M, V, bf.lse_tmp, nullptr, s);
      launch_ce_from_logits(tb.logits, bf.lse_tmp, targets, V, M, loss, s);
    }
    if (mean) launch_mean_loss(loss, targets, V, M, mean, s);
    launch_count_targets(targets, M, V, tb.count, s);
  }

  // ---- LM head and final norm
  if (fused_lse) {
    Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)M * V * 2 * es + (double)V * Mp * es);
    launch_dlogits_t((const bf16 *)tb.logits, bf.lse_tmp, targets, tb.count, M, V, (bf16 *)tb.dl,
                     (bf16 *)tb.trA, Mp, Mp, s);  // dl and dl^T [V][Mp]
  } else {
    Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)M * V * (4 + es));
    if (bf16p) launch_dlogits<bf16>(tb.logits, bf.lse_tmp, targets, tb.count, M, V, (bf16 *)tb.dl, s);
    else launch_dlogits<float>(tb.logits, bf.lse_tmp, targets, tb.count, M, V, (float *)tb.dl, s);
  }
  {
    Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)((fused_lse ? 0 : M * (long long)V) + (long long)M * d + (long long)V * d) * 2 * es);
    if (!fused_lse) tr_md(c, tb.dl, V, M, V, tb.trA, Mp, Mp, s);  // dl^T [V][Mp]
    tr_md(c, bf.h, d, M, d, tb.trB, Mp, Mp, s);     // hf^T [d][Mp]
    tr_md(c, w->lm_head, d, V, d, tb.wT, V, V, s);  // W_lm^T [d][V]
  }
  mmw(tb.trA, tb.trB, V, d, gr->lm_head);               // dW_lm = dl^T hf
  mm(tb.dl, V, tb.wT, V, M, d, V, tb.dh, d);              // dhf = dl W_lm
  hipMemsetAsync(tb.dx, 0, (size_t)M * d * 4, s);
  rms_bwd(xs(2 * L), tb.dh);
  if (bf16p) {  // columns outside the sequences stay zero for every layer
    hipMemsetAsync(tb.kt, 0, (size_t)Hkv * dh * bf.ldvt * 2, s);
    hipMemsetAsync(tb.qt, 0, (size_t)H * dh * bf.ldvt * 2, s);
    hipMemsetAsync(tb.dot, 0, (size_t)H * dh * bf.ldvt * 2, s);
  }

  for (int l = L - 1; l >= 0; --l) {
    const float *xl = xs(2 * l), *xm = xs(2 * l + 1);
    // ---- MLP: x = xm + W2 act(W1 rms(xm))
    if (keep) {
      bf.h = h2_l(l);                                             // h2 kept
    } else {
      fwd_norm(fw, xm, bf.h);                                     // h2
      mm(bf.h, d, w->w1[l], d, M, F, d, tb.z, F);                 // z
    }
    {
      Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)M * F * ((keep ? 2 : 4) + es) + (double)M * d * (4 + es) +
                                            (double)d * F * 2 * es);
      if (keep) {
        tr_md(c, u_l(l), F, M, F, tb.trB, Mp, Mp, s);           // u^T [F][Mp]
      } else if (bf16p) {
        launch_transpose_relu2(tb.z, F, M, F, (bf16 *)tb.trB, Mp, Mp, s);  // u^T [F][Mp] from z
      } else {
        launch_act_bwd<float>(tb.z, nullptr, (float *)tb.u, nullptr, (long long)M * F, c->act, s);
        tr_md(c, tb.u, F, M, F, tb.trB, Mp, Mp, s);              // u^T [F][Mp]
      }
      tr_md(c, dxA0(), d, M, d, tb.trA, Mp, Mp, s);              // dx^T [d][Mp]
      tr_md(c, w->w2[l], F, d, F, tb.wT, d, d, s);               // W2^T [F][d]
    }
    mmw(tb.trA, tb.trB, d, F, gr->w2[l]);                         // dW2 = dx^T u
    const void *dxA = bf16p ? tb.dxb : (const void *)tb.dx;
    // the large-M GEMM applies the ReLU^2 backward in its epilogue:
    // dz = (dx W2) * 2 sqrt(u) with the kept u; otherwise du = dx W2, then a
    // pass over the recomputed z
    const bool fused_dact = keep;
    if (fused_dact) {
      GemmArgs g = gemm(dxA, d, tb.wT, M, F, d, tb.dz, F, EPI_DRELU2);
      g.aux = (const bf16 *)u_l(l);
      run_gemm(c, g, GPT_PROF_BWD_GEMM, s);
    } else {
      mm(dxA, d, tb.wT, d, M, F, d, tb.du, F);
    }
    {
      Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)M * F * 2 * es + (double)M * d * 2 * es + (double)d * F * 2 * es +
                                            (fused_dact ? 0.0 : (double)M * F * (8 + es)));
      if (!fused_dact) {
        if (bf16p) launch_act_bwd<bf16>(tb.z, tb.du, nullptr, (bf16 *)tb.dz, (long long)M * F, c->act, s);
        else launch_act_bwd<float>(tb.z, tb.du, nullptr, (float *)tb.dz, (long long)M * F, c->act, s);
      }
      tr_md(c, tb.dz, F, M, F, tb.trA, Mp, Mp, s);               // dz^T [F][Mp]
      tr_md(c, bf.h, d, M, d, tb.trB, Mp, Mp, s);                // h2^T [d][Mp]
      tr_md(c, w->w1[l], d, F, d, tb.wT, F, F, s);               // W1^T [d][F]
    }
    mmw(tb.trA, tb.trB, F, d, gr->w1[l]);                         // dW1 = dz^T h2
    mm(tb.dz, F, tb.wT, F, M, d, F, tb.dh, d);                    // dh2 = dz W1
    rms_bwd(xm, tb.dh);

    // ---- attention: xm = xl + Wo Attn(q, k, v)
    float *lse_cur = tb.lse;
    if (keep) {
      // h, q, k, V^T, o and lse2 kept; the fp32 projection (pre) recomputed
      bf.h = h_l(l);
      bf.q = q_l(l);
      bf.k = k_l(l);
      bf.vt = vt_l(l);
      bf.o = o_l(l);
      lse_cur = lse_l(l);
      GemmArgs g = gemm(bf.h, d, w->wq[l], M, qkv_n, d, bf.qkv, qkv_n, EPI_F32);
      g.W1 = w->wk[l];
      g.W2 = w->wv[l];
      g.n1 = H * dh;
      g.n2 = (H + Hkv) * dh;
      run_gemm(c, g, GPT_PROF_BWD_GEMM, s);                       // pre -> bf.qkv
    } else {
      fwd_norm(fw, xl, bf.h);                                     // h
      fwd_qkv(fw, l, false);                                      // pre -> bf.qkv; q, k, vt
      fw.lse2 = bf16p ? tb.lse : nullptr;
      fwd_attention(fw);                                          // o (and lse2)
      fw.lse2 = nullptr;
    }
    {
      Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)M * d * (4 + es) + (double)M * H * dh * 2 * es +
                                            (double)d * H * dh * 2 * es);
      tr_md(c, dxA0(), d, M, d, tb.trA, Mp, Mp, s);              // dx^T
      tr_md(c, bf.o, H * dh, M, H * dh, tb.trB, Mp, Mp, s);      // o^T [H dh][Mp]
      tr_md(c, w->wo[l], H * dh, d, H * dh, tb.wT, d, d, s);     // Wo^T [H dh][d]
    }
    mmw(tb.trA, tb.trB, d, H * dh, gr->wo[l]);                    // dWo = dx^T o
    mm(dxA, d, tb.wT, d, M, H * dh, d, tb.dO, H * dh);            // dO = dx Wo
    {
      Timed t(GPT_PROF_BWD_ATTN, s, 2.5 * fw.attn_flops, (double)M * (3 * H + 4 * Hkv) * dh * 4);
      if (bf16p) {
        // V as bf16 rows (the values the forward's attention read), dO in
        // bf16, and K, Q, dO transposed in the V^T column order
        launch_cast_rows(bf.qkv + (H + Hkv) * dh, qkv_n, M, Hkv * dh, (bf16 *)tb.vb, s);
        launch_cast<float, bf16>(tb.dO, (bf16 *)tb.dob, (long long)M * H * dh, s);
        launch_transpose_cols((const bf16 *)bf.k, Hkv * dh, M, Hkv * dh, bf.vcol, (bf16 *)tb.kt, bf.ldvt, s);
        launch_transpose_cols((const bf16 *)bf.q, H * dh, M, H * dh, bf.vcol, (bf16 *)tb.qt, bf.ldvt, s);
        launch_transpose_cols((const bf16 *)tb.dob, H * dh, M, H * dh, bf.vcol, (bf16 *)tb.dot, bf.ldvt, s);
        AttnBwdMfmaArgs mb{};
        mb.q = (const bf16 *)bf.q;
        mb.k = (const bf16 *)bf.k;
        mb.vb = (const bf16 *)tb.vb;
        mb.dob = (const bf16 *)tb.dob;
        mb.kt = (const bf16 *)tb.kt;
        mb.qt = (const bf16 *)tb.qt;
        mb.dot = (const bf16 *)tb.dot;
        mb.ldt = bf.ldvt;
        mb.lse2 = lse_cur;
        mb.dsum = tb.dsum;
        mb.cu = bf.cu;
        mb.cu_pad = bf.cu_pad;
        mb.n_seqs = n_seqs;
        mb.max_len = fw.max_len;
        mb.max_wg = (fw.max_len * (H / Hkv) + 255) / 256;  // 256-row blocks of the dq pass
        mb.M = M;
        mb.H = H;
        mb.Hkv = Hkv;
        mb.dq = tb.dq;
        mb.dkp = tb.dkp;
        mb.dvp = tb.dvp;
        launch_attn_bwd_mfma(mb, tb.dO, (const bf16 *)bf.o, tb.dk, tb.dv, s);
      } else {
        AttnBwdArgs ab{};
        ab.q = bf.q;
        ab.k = bf.k;
        ab.o = bf.o;
        ab.v = bf.qkv + (H + Hkv) * dh;
        ab.ldv = qkv_n;
        ab.v_bf16 = bf16p;
        ab.dout = tb.dO;
        ab.pos = bf.pos;
        ab.seq = bf.seq;
        ab.cu = bf.cu;
        ab.M = M;
        ab.H = H;
        ab.Hkv = Hkv;
        ab.dh = dh;
        ab.dq = tb.dq;
        ab.dk = tb.dk;
        ab.dv = tb.dv;
        ab.lse = tb.lse;
        ab.dsum = tb.dsum;
        launch_attn_bwd<float>(ab, s);
      }
    }
    {
      QkvBwdArgs qa{};
      qa.pre = bf.qkv;
      qa.dq = tb.dq;
      qa.dk = tb.dk;
      qa.dv = tb.dv;
      qa.pos = bf.pos;
      qa.cos = fw.cos;
      qa.sin = fw.sin;
      qa.M = M;
      qa.H = H;
      qa.Hkv = Hkv;
      qa.dh = dh;
      qa.qk_norm = c->qk_norm;
      qa.eps = c->norm_eps;
      Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)M * qkv_n * (8 + 3 * es) + (double)M * d * 2 * es +
                                            (double)qkv_n * d * 2 * es);
      if (bf16p) launch_qkv_bwd<bf16>(qa, (bf16 *)tb.dqkv, s);
      else launch_qkv_bwd<float>(qa, (float *)tb.dqkv, s);
      tr_md(c, tb.dqkv, qkv_n, M, qkv_n, tb.trA, Mp, Mp, s);     // dqkv^T [qkv_n][Mp]
      tr_md(c, bf.h, d, M, d, tb.trB, Mp, Mp, s);                // h^T [d][Mp]
      // [Wq; Wk; Wv]^T [d][qkv_n]
      tr_md(c, w->wq[l], d, H * dh, d, tb.wT, qkv_n, H * dh, s);
      tr_md(c, w->wk[l], d, Hkv * dh, d, (char *)tb.wT + (size_t)H * dh * es, qkv_n, Hkv * dh, s);
      tr_md(c, w->wv[l], d, Hkv * dh, d, (char *)tb.wT + (size_t)(H + Hkv) * dh * es, qkv_n, Hkv * dh, s);
    }
    mmw(tb.trA, tb.trB, H * dh, d, gr->wq[l]);
    mmw((char *)tb.trA + (size_t)H * dh * Mp * es, tb.trB, Hkv * dh, d, gr->wk[l]);
    mmw((char *)tb.trA + (size_t)(H + Hkv) * dh * Mp * es, tb.trB, Hkv * dh, d, gr->wv[l]);
    mm(tb.dqkv, qkv_n, tb.wT, qkv_n, M, d, qkv_n, tb.dh, d);       // dh = dqkv [Wq; Wk; Wv]
    rms_bwd(xl, tb.dh);
  }
  bf = bf0;
  // ---- embeddings
  {
    Timed t(GPT_PROF_BWD_OTHER, s, 0, (double)M * d * 12);
    hipMemsetAsync(gr->wte, 0, (size_t)V * d * 4, s);
    if (c->pos_kind == GPT_POS_LEARNED) hipMemsetAsync(gr->wpe, 0, (size_t)c->max_seq * d * 4, s);
    launch_embed_bwd(tokens, bf.pos, tb.dx, gr->wte, c->pos_kind == GPT_POS_LEARNED ? gr->wpe : nullptr, M, d, s);
  }
  return hip_check("gpt_loss_grads launch");
}

}  // namespace

extern "C" {

size_t gpt_train_workspace_bytes(const gpt_config *c, int32_t max_tokens, int32_t max_seqs) {
  if (check_config(c) != GPT_OK || max_tokens <= 0 || max_seqs <= 0) return 0;
  return carve_train(c, max_tokens, max_seqs, nullptr, nullptr, nullptr);
}

gpt_status gpt_loss_grads(const gpt_config *c, const gpt_weights *w, const float *rope_cos, const float *rope_sin,
                          const int32_t *tokens, const int32_t *targets, const int32_t *cu_seqlens, int32_t n_seqs,
                          const gpt_grads *grads, float *loss, float *mean, void *workspace,
                          size_t workspace_bytes, gpt_stream_t stream) {
  return loss_grads_impl(c, w, rope_cos, rope_sin, tokens, targets, cu_seqlens, n_seqs, grads, loss, mean,
                         workspace, workspace_bytes, stream);
}

gpt_status gpt_prefill(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                       const float *rope_sin, const int32_t *tokens, const int32_t *cu_seqlens,
                       int32_t n_seqs, gpt_kv_cache *kv, int32_t logits_rows, float *logits, float *lse,
                       float *probs, void *workspace, size_t workspace_bytes, gpt_stream_t stream) {
  return prefill_impl(c, w, rope_cos, rope_sin, tokens, cu_seqlens, n_seqs, kv, logits_rows, logits, lse, probs,
                      nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
}

gpt_status gpt_prefill_loss(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                            const float *rope_sin, const int32_t *tokens, const int32_t *targets,
                            const int32_t *cu_seqlens, int32_t n_seqs, gpt_kv_cache *kv, float *loss,
                            float *lse, float *mean, void *workspace, size_t workspace_bytes,
                            gpt_stream_t stream) {
  if (!targets) return fail(GPT_ERR_ARG, "NULL required pointer");
  return prefill_impl(c, w, rope_cos, rope_sin, tokens, cu_seqlens, n_seqs, kv, GPT_ROWS_ALL, nullptr, lse,
                      nullptr, targets, loss, mean, workspace, workspace_bytes, stream);
}

gpt_status gpt_decode_step(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                           const float *rope_sin, gpt_kv_cache *kv, const int32_t *tokens_in,
                           float temperature, const float *uniforms, int32_t *tokens_out, float *logits,
                           void *workspace, size_t workspace_bytes, gpt_stream_t stream) {
  gpt_status st = check_config(c);
  if (st) return st;
  if ((st = check_weights(c, w))) return st;
  if (!kv || !tokens_in || !tokens_out || !workspace) return fail(GPT_ERR_ARG, "NULL required pointer");
  if (temperature > 0.f && !uniforms) return fail(GPT_ERR_ARG, "uniforms are required when temperature > 0");
  if (!(temperature == temperature)) return fail(GPT_ERR_ARG, "temperature is NaN");
  if (c->pos_kind == GPT_POS_ROPE && (!rope_cos || !rope_sin)) return fail(GPT_ERR_ARG, "RoPE tables required");
  if (kv->cfg.n_layer != c->n_layer || kv->cfg.dtype != c->dtype || kv->cfg.n_kv_head != c->n_kv_head ||
      kv->cfg.head_dim != c->head_dim)
    return fail(GPT_ERR_ARG, "kv cache was made for another config");
  const int n = kv->n_seqs;
  if ((long long)n * c->n_kv_head > kCounters)
    return fail(GPT_ERR_UNSUPPORTED, "at most %d sequences x K/V heads per decode step", kCounters);
  for (int b = 0; b < n; ++b)
    if (kv->lens[b] + 1 > kv->capacity)
      return fail(GPT_ERR_CAPACITY, "sequence %d: length %d + 1 exceeds capacity %d", b, kv->lens[b], kv->capacity);
  const size_t need = carve(c, n, n, nullptr, nullptr);
  if (workspace_bytes < need) return fail(GPT_ERR_ARG, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(GPT_ERR_ARG, "workspace must be 256-byte aligned");
  if (logits && !aligned16(logits)) return fail(GPT_ERR_ARG, "logits must be 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  hipGetLastError();
  Bufs bf;
  carve(c, n, n, (char *)workspace, &bf);
  const bool bf16p = c->dtype == GPT_DTYPE_BF16;
  const int d = c->d_model, H = c->n_head, Hkv = c->n_kv_head, dh = c->head_dim, F = c->d_ff, V = c->vocab;
  const int qkv_n = (H + 2 * Hkv) * dh;
  PagedKV pv = paged_view(kv);
  float *lg = logits ? logits : bf.dlogits;
  double kv_bytes = 0;
  for (int b = 0; b < n; ++b) kv_bytes += (double)(kv->lens[b] + 1) * 2 * Hkv * dh * (bf16p ? 2 : 4);
  ScatterArgs sa{};
  sa.qkv = bf.qkv;
  sa.M = n;
  sa.H = H;
  sa.Hkv = Hkv;
  sa.seq = nullptr;
  sa.pos = pv.lens;
  sa.cos = c->pos_kind == GPT_POS_ROPE ? rope_cos : nullptr;
  sa.sin = c->pos_kind == GPT_POS_ROPE ? rope_sin : nullptr;
  sa.qk_norm = c->qk_norm;
  sa.eps = c->norm_eps;
  sa.q_out = bf.q;
  sa.kv = pv;
  sa.use_cache = 1;
  sa.head_dim = dh;
  const double att_flops = 4.0 * H * dh * (kv_bytes / (2.0 * Hkv * dh * (bf16p ? 2 : 4)));
  const double att_bytes = kv_bytes + (double)n * H * dh * 2 * (bf16p ? 2 : 4);

  if (bf16p) {
    // Per layer: QKV projection (k split into fp32 slabs) -> attention, which
    // sums the slabs, applies RoPE and QK-norm and appends k, v to the cache
    // -> O projection (slabs) -> residual + RMSNorm -> W1 + ReLU^2 -> W2
    // (slabs) -> residual + RMSNorm.
    // Above 64 rows the large-M GEMMs write x and the norms run on their own.
    const bool rows = n <= 64;
    // decode-attention chunks of this step (the lengths are the same for
    // every layer): chosen on the host, listed on the device once
    int chunk_pages = 0, splits = 0, work = 0;
    decode_chunking(kv->lens.data(), n, Hkv, bf.max_splits, &chunk_pages, &splits, &work);
    {
      DecodeMapArgs dm{pv, n, chunk_pages, bf.max_splits, bf.dmap};
      Timed t(GPT_PROF_NORM, s, 0, (double)n * d * 8);
      launch_embed_norm_bf16(tokens_in, (const bf16 *)w->wte, bf.x, (bf16 *)bf.h, n, d, c->norm_eps,
                             bf.ctr, kCounters, dm, s);
    }
    // x += A W^T, then h = RMSNorm(x)
    auto proj_resid_norm = [&](const void *A, int K, const void *Wt) {
      if (rows) {
        const int ks = gemm_rows_ksplit(d, K);
        run_gemm_rows(gemm(A, K, Wt, n, d, K, bf.slabs, d, EPI_F32), ks, (long long)n * d, GPT_PROF_GEMM, s);
        Timed t(GPT_PROF_NORM, s, 0, (double)n * d * (4.0 * ks + 10.0));
        launch_resid_norm_bf16(bf.slabs, ks, (long long)n * d, bf.x, (bf16 *)bf.h, n, d, c->norm_eps, s);
      } else {
        run_gemm(c, gemm(A, K, Wt, n, d, K, bf.x, d, EPI_RESID), GPT_PROF_GEMM, s);
        Timed t(GPT_PROF_NORM, s, 0, (double)n * d * 6);
        launch_rmsnorm_bf16(bf.x, (bf16 *)bf.h, nullptr, n, d, c->norm_eps, s);
      }
    };
    for (int l = 0; l < c->n_layer; ++l) {
      ScatterArgs sl = sa;
      sl.layer = l;
      if (rows) {
        const int ks = gemm_rows_ksplit(qkv_n, d);
        GemmArgs g = gemm(bf.h, d, w->wq[l], n, qkv_n, d, bf.slabs, qkv_n, EPI_F32);
        g.W1 = w->wk[l];
        g.W2 = w->wv[l];
        g.n1 = H * dh;
        g.n2 = (H + Hkv) * dh;
        run_gemm_rows(g, ks, (long long)n * qkv_n, GPT_PROF_GEMM, s);
        sl.qkv = bf.slabs;
        sl.nslab = ks;
        sl.slab = (long long)n * qkv_n;
      } else {
        GemmArgs g = gemm(bf.h, d, w->wq[l], n, qkv_n, d, bf.qkv, qkv_n, EPI_F32);
        g.W1 = w->wk[l];
        g.W2 = w->wv[l];
        g.n1 = H * dh;
        g.n2 = (H + Hkv) * dh;
        run_gemm(c, g, GPT_PROF_GEMM, s);
      }
      {
        Timed t(GPT_PROF_DECODE_ATTN, s, att_flops, att_bytes);
        AttnDecodeArgs aa{};
        aa.in = sl;
        aa.n = n;
        aa.chunk_pages = chunk_pages;
        aa.max_splits = splits;
        aa.work = work;
        aa.map = bf.dmap;
        aa.o_part = bf.opart;
        aa.ml_part = bf.mlpart;
        aa.o = (bf16 *)bf.o;
        aa.ctr = bf.ctr;
        launch_attn_decode_bf16(aa, s);
      }
      proj_resid_norm(bf.o, H * dh, w->wo[l]);
      run_gemm(c, gemm(bf.h, d, w->w1[l], n, F, d, bf.u, F, EPI_RELU2_BF16), GPT_PROF_GEMM, s);
      proj_resid_norm(bf.u, F, w->w2[l]);
    }
  } else {
    {
      Timed t(GPT_PROF_NORM, s, 0, (double)n * d * 8);
      launch_embed_f32(tokens_in, (const float *)w->wte, (const float *)w->wpe, pv.lens, bf.x, n, d, s);
    }
    for (int l = 0; l < c->n_layer; ++l) {
      launch_rmsnorm_f32(bf.x, (float *)bf.h, nullptr, n, d, c->norm_eps, s);
      GemmArgs g = gemm(bf.h, d, w->wq[l], n, qkv_n, d, bf.qkv, qkv_n, EPI_F32);
      g.W1 = w->wk[l];
      g.W2 = w->wv[l];
      g.n1 = H * dh;
      g.n2 = (H + Hkv) * dh;
      run_gemm(c, g, GPT_PROF_GEMM, s);
      ScatterArgs sl = sa;
      sl.layer = l;
      launch_qkv_scatter_f32(sl, s);
      {
        Timed t(GPT_PROF_DECODE_ATTN, s, att_flops, att_bytes);
        AttnF32Args aa{};
        aa.q = (const float *)bf.q;
        aa.M = n;
        aa.H = H;
        aa.Hkv = Hkv;
        aa.dh = dh;
        aa.kv = pv;
        aa.layer = l;
        aa.o = (float *)bf.o;
        launch_attn_decode_f32(aa, s);
      }
      run_gemm(c, gemm(bf.o, H * dh, w->wo[l], n, d, H * dh, bf.x, d, EPI_RESID), GPT_PROF_GEMM, s);
      launch_rmsnorm_f32(bf.x, (float *)bf.h, nullptr, n, d, c->norm_eps, s);
      run_gemm(c, gemm(bf.h, d, w->w1[l], n, F, d, bf.u, F, c->act == GPT_ACT_RELU ? EPI_RELU_F32 : EPI_RELU2_BF16),
               GPT_PROF_GEMM, s);
      run_gemm(c, gemm(bf.u, F, w->w2[l], n, d, F, bf.x, d, EPI_RESID), GPT_PROF_GEMM, s);
    }
    launch_rmsnorm_f32(bf.x, (float *)bf.h, nullptr, n, d, c->norm_eps, s);
  }
  // h holds the final RMSNorm of x here
  run_gemm(c, gemm(bf.h, d, w->lm_head, n, V, d, lg, V, EPI_F32), GPT_PROF_LMHEAD, s);
  {
    Timed t(GPT_PROF_SOFTMAX, s, 0, (double)n * V * 4);
    if (temperature > 0.f) launch_sample(lg, n, V, temperature, uniforms, tokens_out, pv.lens, s);
    else launch_argmax(lg, n, V, tokens_out, bf.sel, pv.lens, s);
  }
  if ((st = hip_check("gpt_decode_step launch"))) return st;
  for (int b = 0; b < n; ++b) kv->lens[b] += 1;
  return GPT_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation decode
// The scratch of gpt_decode_step_noalloc.  In host code `scratch` names a
// host-side stand-in, not device memory: only the per-device address from
// hipGetSymbolAddress is ever handed to kernels or copies.
static __device__ __align__(256) char scratch[GPT_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;  // per device id, looked up once

gpt_status scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(GPT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GPT_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GPT_OK;
}
}  // namespace

extern "C" {

gpt_status gpt_decode_step_noalloc(const gpt_config *c, const gpt_weights *w, const float *rope_cos,
                                   const float *rope_sin, gpt_kv_cache *kv, const int32_t *tokens_in,
                                   float temperature, const float *uniforms, int32_t *tokens_out,
                                   float *logits, gpt_stream_t stream) {
  gpt_status st = check_config(c);
  if (st) return st;
  if (!kv) return fail(GPT_ERR_ARG, "NULL required pointer");
  const size_t need = carve(c, kv->n_seqs, kv->n_seqs, nullptr, nullptr);
  if (need > GPT_NOALLOC_SCRATCH_BYTES)
    return fail(GPT_ERR_CAPACITY, "a decode step of %d sequences needs %zu bytes of scratch, more than the %zu "
                "the no-allocation entry point holds", kv->n_seqs, need, (size_t)GPT_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if ((st = scratch_on_current_device(&ws))) return st;
  const uint32_t mask = g_prof.mask;  // timing events would be created on demand: none here
  g_prof.mask = 0;
  st = gpt_decode_step(c, w, rope_cos, rope_sin, kv, tokens_in, temperature, uniforms, tokens_out, logits, ws,
                       GPT_NOALLOC_SCRATCH_BYTES, stream);
  g_prof.mask = mask;
  return st;
}

gpt_status gpt_select_tokens(const float *logits, int32_t rows, int32_t vocab, float temperature,
                             const float *uniforms, int32_t *tokens_out, gpt_stream_t stream) {
  if (!logits || !tokens_out) return fail(GPT_ERR_ARG, "NULL required pointer");
  if (rows <= 0 || vocab <= 0) return fail(GPT_ERR_ARG, "rows and vocab must be positive");
  if (temperature > 0.f && !uniforms) return fail(GPT_ERR_ARG, "uniforms are required when temperature > 0");
  if (!(temperature == temperature)) return fail(GPT_ERR_ARG, "temperature is NaN");
  hipStream_t s = (hipStream_t)stream;
  hipGetLastError();
  {
    Timed t(GPT_PROF_SOFTMAX, s, 0, (double)rows * vocab * 4);
    if (temperature > 0.f) launch_sample(logits, rows, vocab, temperature, uniforms, tokens_out, nullptr, s);
    else launch_argmax_rows(logits, rows, vocab, tokens_out, s);
  }
  return hip_check("gpt_select_tokens launch");
}

gpt_status gpt_adam_step(float *param, const float *grad, float *m, float *v, void *param_bf16, int64_t n,
                         int32_t step, float lr, float beta1, float beta2, float eps, gpt_stream_t stream) {
  if (!param || !grad || !m || !v) return fail(GPT_ERR_ARG, "NULL required pointer");
  if (n < 0) return fail(GPT_ERR_ARG, "n must be >= 0");
  if (step < 1) return fail(GPT_ERR_ARG, "step must be >= 1");
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
    return fail(GPT_ERR_ARG, "betas must lie in [0, 1)");
  if (!(eps >= 0.f)) return fail(GPT_ERR_ARG, "eps must be >= 0");
  if (!std::isfinite(lr)) return fail(GPT_ERR_ARG, "lr must be finite");
  if (!aligned16(param) || !aligned16(grad) || !aligned16(m) || !aligned16(v))
    return fail(GPT_ERR_ARG, "param, grad, m, v must be 16-byte aligned");
  if (param_bf16 && (reinterpret_cast<uintptr_t>(param_bf16) & 7))
    return fail(GPT_ERR_ARG, "param_bf16 must be 8-byte aligned");
  if (n == 0) return GPT_OK;
  AdamHyper h;
  h.lr = lr;
  h.beta1 = beta1;
  h.beta2 = beta2;
  h.one_minus_beta1 = (float)(1.0 - (double)beta1);
  h.one_minus_beta2 = (float)(1.0 - (double)beta2);
  h.eps = eps;
  h.corr1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)step)));
  h.corr2 = (float)(1.0 / (1.0 - std::pow((double)beta2, (double)step)));
  hipStream_t s = (hipStream_t)stream;
  hipGetLastError();
  {
    Timed t(GPT_PROF_OPTIM, s, 0, (double)n * (28 + (param_bf16 ? 2 : 0)));
    launch_adam(param, grad, m, v, (bf16 *)param_bf16, (long long)n, h, s);
  }
  return hip_check("gpt_adam_step launch");
}

gpt_status gpt_debug_gemm(const void *A, const void *W, int32_t M, int32_t N, int32_t K, void *C,
                          int32_t epi, int32_t ksplit, gpt_stream_t stream) {
  if (!A || !W || !C) return fail(GPT_ERR_ARG, "NULL pointer");
  if (M <= 0 || N <= 0 || K <= 0 || K % 64 || N % 128) return fail(GPT_ERR_ARG, "bad GEMM shape");
  if (epi < 0 || epi > 3) return fail(GPT_ERR_ARG, "bad epilogue");
  if (ksplit < 1 || ksplit > kMaxRowSplit || ksplit > K / 64) return fail(GPT_ERR_ARG, "bad ksplit");
  if (ksplit > 1 && (M > 64 || epi != EPI_F32))
    return fail(GPT_ERR_ARG, "ksplit > 1 needs M <= 64 and the fp32 epilogue");
  if (!aligned16(A) || !aligned16(W) || !aligned16(C)) return fail(GPT_ERR_ARG, "pointers must be 16-byte aligned");
  hipGetLastError();
  const GemmArgs g = gemm(A, K, W, M, N, K, C, N, epi);
  if (ksplit > 1) {
    run_gemm_rows(g, ksplit, (long long)M * N, GPT_PROF_GEMM, (hipStream_t)stream);
  } else {
    gpt_config c{};
    c.dtype = GPT_DTYPE_BF16;
    run_gemm(&c, g, GPT_PROF_GEMM, (hipStream_t)stream);
  }
  return hip_check("gpt_debug_gemm");
}

gpt_status gpt_debug_attn_prefill(const void *q, const void *k, const void *vt, int64_t ldvt,
                                  const int32_t *cu_seqlens, int32_t n_seqs, int32_t n_head, int32_t qk_norm,
                                  int32_t *cu_dev, void *o, gpt_stream_t stream) {
  if (!q || !k || !vt || !cu_seqlens || !cu_dev || !o) return fail(GPT_ERR_ARG, "NULL pointer");
  if (n_seqs <= 0 || n_seqs > kMaxPrefillSeqs || n_head <= 0 || n_head > 16) return fail(GPT_ERR_ARG, "bad sizes");
  if (cu_seqlens[0] != 0) return fail(GPT_ERR_ARG, "cu_seqlens[0] must be 0");
  long long pad = 0;
  int max_len = 0;
  for (int b = 0; b < n_seqs; ++b) {
    int len = cu_seqlens[b + 1] - cu_seqlens[b];
    if (len <= 0) return fail(GPT_ERR_ARG, "empty sequence");
    pad += (len + 63) / 64 * 64;
    max_len = std::max(max_len, len);
  }
  if (ldvt < pad || ldvt % 64) return fail(GPT_ERR_ARG, "ldvt too small or not a multiple of 64");
  hipStream_t s = (hipStream_t)stream;
  hipGetLastError();
  PrefillMeta meta;
  meta.n = n_seqs;
  for (int b = 0; b <= n_seqs; ++b) meta.cu[b] = cu_seqlens[b];
  prefill_meta_kernel<<<1, 256, 0, s>>>(meta, cu_dev, cu_dev + n_seqs + 1, nullptr, nullptr, 0);
  AttnPrefillArgs aa{};
  aa.q = (const bf16 *)q;
  aa.k = (const bf16 *)k;
  aa.vt = (const bf16 *)vt;
  aa.ldvt = ldvt;
  aa.cu = cu_dev;
  aa.cu_pad = cu_dev + n_seqs + 1;
  aa.n_seqs = n_seqs;
  aa.max_wg = (max_len * n_head + kAttnPrefillRows - 1) / kAttnPrefillRows;
  aa.H = n_head;
  aa.Hkv = 1;
  aa.qk_norm = qk_norm != 0;
  aa.o = (bf16 *)o;
  launch_attn_prefill_bf16(aa, s);
  return hip_check("gpt_debug_attn_prefill");
}

gpt_status gpt_profile_enable(uint32_t mask) {
  g_prof.reset();
  g_prof.mask = mask;
  return GPT_OK;
}

gpt_status gpt_profile_mask(uint32_t mask) {
  g_prof.mask = mask;
  return GPT_OK;
}

gpt_status gpt_profile_read(int32_t cls, double *ms, int64_t *launches, double *flops, double *bytes) {
  if (cls < 0 || cls >= GPT_PROF_NCLASSES) return fail(GPT_ERR_ARG, "bad class");
  double tot = 0, fl = 0, by = 0;
  int64_t n = 0;
  for (auto &r : g_prof.recs) {
    if (r.cls != cls) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return hip_check("profile sync");
    float t = 0;
    hipEventElapsedTime(&t, r.a, r.b);
    tot += t;
    fl += r.flops;
    by += r.bytes;
    ++n;
  }
  if (ms) *ms = tot;
  if (launches) *launches = n;
  if (flops) *flops = fl;
  if (bytes) *bytes = by;
  return GPT_OK;
}

gpt_status gpt_profile_read_launch(int32_t cls, int64_t i, double *ms, double *flops, double *bytes) {
  if (cls < 0 || cls >= GPT_PROF_NCLASSES) return fail(GPT_ERR_ARG, "bad class");
  if (i < 0) return fail(GPT_ERR_ARG, "negative launch index");
  int64_t n = 0;
  for (auto &r : g_prof.recs) {
    if (r.cls != cls || n++ != i) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return hip_check("profile sync");
    float t = 0;
    hipEventElapsedTime(&t, r.a, r.b);
    if (ms) *ms = t;
    if (flops) *flops = r.flops;
    if (bytes) *bytes = r.bytes;
    return GPT_OK;
  }
  return fail(GPT_ERR_ARG, "launch %lld of class %d not recorded (%lld are)", (long long)i, (int)cls, (long long)n);
}

}  // extern "C"
