// Host-side launchers of the gfx950 kernels.  Every launcher enqueues on the
// given stream and does no validation: the C-ABI layer (api.cpp) checks
// shapes before calling them.
#pragma once
#include "common.h"

// ------------------------------------------------------------ small kernels
void launch_rowinfo(const int *cu, const int *cu_pad, int n_seqs, int M, int *seq, int *pos,
                    int *vcol, hipStream_t s);
void launch_embed_bf16(const int *tok, const bf16 *wte, float *x, int M, int d, hipStream_t s);
// The chunks of one decode step that hold positions, in order of sequence
// then chunk: map[kDecodeMapStride i ..] = {sequence, chunk, lens[sequence] + 1,
// 0, the block-table entries of the chunk's pages 0 .. 7 (clamped to the
// table's row)}; the list
// has sum over sequences of min(ceil(pages / chunk_pages), max_chunks)
// entries, and map holds room for n max_chunks of them.
struct DecodeMapArgs {
  PagedKV kv;
  int n, chunk_pages, max_chunks;
  int *map;  // null: no list
};
// Decode rows: x = WTE[tok], h = RMSNorm(x) (bf16), the completion counters
// cleared, and (dm.map set) the step's decode-attention work list written by
// one more workgroup.
void launch_embed_norm_bf16(const int *tok, const bf16 *wte, float *x, bf16 *h, int M, int d,
                            float eps, unsigned *ctr, int nctr, const DecodeMapArgs &dm, hipStream_t s);
void launch_embed_f32(const int *tok, const float *wte, const float *wpe, const int *pos, float *x,
                      int M, int d, hipStream_t s);
void launch_rmsnorm_bf16(const float *x, bf16 *y, const int *rows, int M, int d, float eps,
                         hipStream_t s);
void launch_rmsnorm_f32(const float *x, float *y, const int *rows, int M, int d, float eps,
                        hipStream_t s);
// Residual add of a split GEMM's partial slabs, then RMSNorm: for every row,
// x += part[0] + part[1] + ... (nslab slabs `slab` floats apart, in order)
// and h = bf16(rmsnorm(x)).  d <= 2048.
void launch_resid_norm_bf16(const float *part, int nslab, long long slab, float *x, bf16 *h, int M, int d,
                            float eps, hipStream_t s);

// RoPE + QK-norm of the fp32 q/k head vectors of `qkv` ([M][(H+2Hkv)*128]),
// then bf16 scatter: q -> q_out [M][H*128]; k -> k_out [M][Hkv*128] and/or
// the paged cache; v -> vt_out [Hkv*128][ldvt] at column vcol[m] and/or the
// cache.  seq == NULL means row m is sequence m (decode).
struct ScatterArgs {
  const float *qkv;
  int nslab;       // qkv holds nslab fp32 partial slabs (k ranges of a split GEMM) ...
  long long slab;  // ... `slab` floats apart, summed in order; nslab <= 1: one slab
  int M, H, Hkv;
  const int *seq, *pos, *vcol;
  const float *cos, *sin;  // [max_seq][64] or NULL (no RoPE)
  int qk_norm;
  float eps;
  void *q_out, *k_out, *vt_out;  // bf16 (or fp32 on the small path)
  long long ldvt;
  PagedKV kv;
  int layer;
  int use_cache;
  int head_dim;  // small path only
};
void launch_rope_norm_scatter_bf16(const ScatterArgs &a, hipStream_t s);
void launch_qkv_scatter_f32(const ScatterArgs &a, hipStream_t s);

void launch_softmax_lse(const float *logits, int rows, int V, float *lse, float *probs,
                        hipStream_t s);
// lse[r] from the LM-head epilogue's per-block partials; then optional probs.
void launch_lse_combine(const float *part, int nparts, int rows, float *lse, const float *logits,
                        int V, float *probs, hipStream_t s);
// Next-token cross-entropy per row, loss[r] = lse[r] - logit of targets[r]
// (0 for a target outside [0, V)).  From the EPI_LOSS partials and target
// logits (part, tgt), lse optional:
void launch_ce_from_parts(const float *part, int nparts, const float *tgt, const int *targets, int V,
                          int rows, float *loss, float *lse, hipStream_t s);
// ... or from materialised logits and their lse:
void launch_ce_from_logits(const float *logits, const float *lse, const int *targets, int V, int rows,
                           float *loss, hipStream_t s);
// mean[0] = sum of loss[r] over rows with a target in [0, V) / their number
// (0 if none), summed in a fixed order by one workgroup.
void launch_mean_loss(const float *loss, const int *targets, int V, int rows, float *mean, hipStream_t s);
// scratch: argmax_scratch_floats(rows, V) floats of device memory
// lens (optional): decode lengths, incremented once the token is chosen
void launch_argmax(const float *logits, int rows, int V, int *out, float *scratch, int *lens,
                   hipStream_t s);
int argmax_scratch_floats(int rows, int V);
void launch_argmax_rows(const float *logits, int rows, int V, int *out, hipStream_t s);
void launch_sample(const float *logits, int rows, int V, float temperature, const float *u,
                   int *out, int *lens, hipStream_t s);
void launch_lens_set(int *lens, const int *cu, int n, hipStream_t s);
void launch_lens_inc(int *lens, int n, hipStream_t s);
void launch_gather_rows_bf16(const bf16 *src, bf16 *dst, const int *rows, int n, int d,
                             hipStream_t s);

// ------------------------------------------------------------ Adam
// m = beta1 m + (1 - beta1) g; v = beta2 v + (1 - beta2) g^2;
// p -= lr (m corr1) / (sqrt(v corr2) + eps), corr = 1 / (1 - beta^step).
struct AdamHyper {
  float lr, beta1, one_minus_beta1, beta2, one_minus_beta2, eps, corr1, corr2;
};
// p, g, m, v: fp32 [n], 16-byte aligned; pb (nullable): bf16 [n], 8-byte aligned
void launch_adam(float *p, const float *g, float *m, float *v, bf16 *pb, long long n, const AdamHyper &h,
                 hipStream_t s);

// ------------------------------------------------------------ loss backward
// dst[c][r] = src[r][c] (r < R, c < C), zero for R <= r < Rp.
template <typename TI, typename TO>
void launch_transpose(const TI *src, long long lds, int R, int C, TO *dst, long long ldd, int Rp, hipStream_t s);
template <typename TI, typename TO>
void launch_cast(const TI *src, TO *dst, long long n, hipStream_t s);
// dx[m] += the gradient through y = x / sqrt(mean(x^2) + eps), given dy;
// dxb (nullable) receives the updated dx in bf16
void launch_rms_bwd(const float *x, const float *dy, float *dx, bf16 *dxb, int M, int d, float eps, hipStream_t s);
// u = act(z) and dz = du act'(z) (either may be NULL)
template <typename T>
void launch_act_bwd(const float *z, const float *du, T *u, T *dz, long long n, int relu2, hipStream_t s);
// dst[c][r] = bf16(relu(z[r][c])^2) (r < R, zero for R <= r < Rp): the
// transposed MLP activation straight from its fp32 pre-activation
// (C % 64 == 0; lds, ldd, Rp multiples of 8)
void launch_transpose_relu2(const float *z, long long lds, int R, int C, bf16 *dst, long long ldd, int Rp,
                            hipStream_t s);
struct QkvBwdArgs {
  const float *pre;             // [M][(H + 2Hkv) dh] projection output before RoPE / QK-norm
  const float *dq, *dk, *dv;    // [M][H dh], [M][Hkv dh] x 2: gradients of the attention inputs
  const int *pos;
  const float *cos, *sin;       // [max_seq][dh/2] or NULL (no RoPE)
  int M, H, Hkv, dh, qk_norm;
  float eps;
};
template <typename T>
void launch_qkv_bwd(const QkvBwdArgs &a, T *dqkv, hipStream_t s);
// Attention backward on the vector ALUs (any head width up to 128; the
// fp32 small-model path).
struct AttnBwdArgs {
  const void *q, *k, *o;  // [M][H dh], [M][Hkv dh], [M][H dh] in the model dtype
  const float *v;         // rows of ldv floats; v_bf16: rounded to bf16 as the forward used them
  long long ldv;
  int v_bf16;
  const float *dout;      // [M][H dh] gradient of the attention output
  const int *pos, *seq, *cu;
  int M, H, Hkv, dh;
  float *dq, *dk, *dv;    // [M][H dh], [M][Hkv dh] x 2
  float *lse, *dsum;      // [M][H] scratch
};
template <typename T>
void launch_attn_bwd(const AttnBwdArgs &a, hipStream_t s);
// dst[m][c] = bf16(src[m lds + c]) for c < C
void launch_cast_rows(const float *src, long long lds, int M, int C, bf16 *dst, hipStream_t s);
// From bf16 logits [rows][V]: dl [rows][V] and its transpose dlt [V][ldt]
// (columns rows .. Rp - 1 zero); V % 64 == 0, Rp % 64 == 0, ldt % 8 == 0.
void launch_dlogits_t(const bf16 *logits, const float *lse, const int *targets, const int *count, int rows, int V,
                      bf16 *dl, bf16 *dlt, long long ldt, int Rp, hipStream_t s);
template <typename T>
void launch_dlogits(const float *logits, const float *lse, const int *targets, const int *count, int rows, int V,
                    T *dl, hipStream_t s);
void launch_embed_bwd(const int *tokens, const int *pos, const float *dx, float *dwte, float *dwpe, int M, int d,
                      hipStream_t s);
void launch_count_targets(const int *targets, int M, int V, int *count, hipStream_t s);

// ------------------------------------------------------------ GEMMs
enum Epi {
  EPI_BF16 = 0,
  EPI_RELU2_BF16 = 1,
  EPI_RESID = 2,
  EPI_F32 = 3,
  EPI_RELU_F32 = 4,
  EPI_LOGITS = 5,  // fp32 store + per-row (max, sum exp) over each kLogitsPartCols columns
  EPI_QKV = 6,     // RoPE + QK-norm + bf16 scatter of q / k / v^T (+ paged cache)
  EPI_LOSS = 7,    // EPI_LOGITS' partials and each row's target logit; C is not written
  EPI_DRELU2 = 8,  // bf16 C = acc * 2 sqrt(u), u = aux[m][n] = max(z, 0)^2 (bf16, row stride ldc): ReLU^2 backward
  EPI_LOGITS_BF16 = 9  // EPI_LOSS' partials and target logit, and C = the logits in bf16
};

// Extra operands of the EPI_QKV epilogue (column block = one 128-wide head).
struct QkvEpi {
  const int *seq, *pos, *vcol;
  const float *cos, *sin;  // [max_seq][64]
  float eps;
  int qk_norm, H, Hkv;
  bf16 *q_out, *k_out, *vt_out;
  long long ldvt;
  PagedKV kv;
  int layer, use_cache;
};

// C[m][n] = sum_k A[m][k] * W[n][k]; W rows come from up to three segments
// ([0,n1) from W0, [n1,n2) from W1, [n2,N) from W2) so separate Q/K/V
// weights feed one GEMM without a copy.
struct GemmArgs {
  const void *A;
  long long lda;
  const void *W0, *W1, *W2;
  int n1, n2;
  long long ldw;
  int M, N, K;
  void *C;
  long long ldc;
  int epi;
  float *part;  // EPI_LOGITS, EPI_LOSS, EPI_LOGITS_BF16: [M][N/kLogitsPartCols][2] partial (max, sum exp)
  const bf16 *aux;     // EPI_DRELU2: the activation u = max(z, 0)^2
  const float *rin;    // EPI_RESID: C = rin + A W^T (same layout as C); NULL: C += A W^T
  const int *targets;  // EPI_LOSS, EPI_LOGITS_BF16: [M] target column of each row (any value)
  float *tgt;          // EPI_LOSS, EPI_LOGITS_BF16: [M] C[m][targets[m]] (fp32), where targets[m] is in [0, N)
  QkvEpi qkv;   // EPI_QKV
  // k split of the large-M kernel (EPI_F32 only): grid row kz multiplies the
  // kz-th K-long slice of every row of A and W (rows lda / ldw apart) into
  // C + kz * slab
  long long slab;
};
void launch_gemm_bf16(const GemmArgs &g, hipStream_t s);         // MFMA, large M
// C (fp32, ldc = N) = A W^T with the k range split ks ways into slabs
// [ks][M][N] (ks * M * N floats of scratch), then summed in order: for
// long-K products whose M x N tiling leaves CUs idle.  K % (64 ks) == 0.
void launch_gemm_bf16_splitk(const GemmArgs &g, int ks, float *slabs, hipStream_t s);
// ks for launch_gemm_bf16_splitk: about 256 tiles, at least 8 k-tiles per slice
int gemm_splitk_ways(int M, int N, int K);
// Decode-row GEMM (M <= 64, N % 64 == 0, K % 64 == 0).  With ks > 1 the k
// range is split over ks workgroups per column tile and range kz writes its
// fp32 partial product to C + kz * slab (EPI_F32 only); the consumer sums
// the slabs in order.
void launch_gemm_bf16_rows(const GemmArgs &g, int ks, long long slab, hipStream_t s);
constexpr int kMaxRowSplit = 16;
int gemm_rows_ksplit(int N, int K);  // k ranges for a decode-row GEMM whose consumer sums slabs
void launch_gemm_f32(const GemmArgs &g, hipStream_t s);          // small fp32 path

// ------------------------------------------------------------ attention
// Prefill-attention workgroup: kAttnPrefillRows rows over kAttnPrefillWaves
// waves (32 or 64 rows per wave).  256 rows: each staged K/V tile serves
// that many (128 rows measured 10% slower at depth 12).
constexpr int kAttnPrefillWaves = 8;
constexpr int kAttnPrefillRows = 256;
struct AttnPrefillArgs {
  const bf16 *q;   // [M][H*128]
  const bf16 *k;   // [M][Hkv*128]
  const bf16 *vt;  // [Hkv*128][ldvt]
  long long ldvt;
  const int *cu, *cu_pad;
  // grid: (sequence, kAttnPrefillRows-row block counted from the end, K/V
  // head); a K/V head's rows are its H/Hkv query heads at every position
  int n_seqs, max_wg;
  int H, Hkv;
  int qk_norm;  // q and k are QK-normalised (RMS <= 1 per head): fixed softmax reference
  bf16 *o;  // [M][H*128]
  float *lse2;  // [M][H] or NULL: each row's base-2 log-sum-exp of log2(e) q.k / sqrt(128)
};
// MFMA attention backward (bf16, head width 128).  The transposed operands
// kt, qt, dot have the V^T layout: [dims][ldt], a row's column at
// cu_pad[seq] + vperm16(position), zero elsewhere.
struct AttnBwdMfmaArgs {
  const bf16 *q, *k, *vb, *dob;   // [M][H 128], [M][Hkv 128] x 2, [M][H 128] (dO in bf16)
  const bf16 *kt, *qt, *dot;      // [Hkv 128][ldt], [H 128][ldt] x 2
  long long ldt;
  const float *lse2;              // [M][H] from the forward
  float *dsum;                    // [M][H] D = dO . O (written by the launcher)
  const int *cu, *cu_pad;
  int n_seqs, max_wg, max_len;    // max_wg: 256-row blocks (dq pass) of the longest sequence's rows
  int M, H, Hkv;
  float *dq;                      // [M][H 128]
  float *dkp, *dvp;               // [H][M][128] per-query-head partials
};
void launch_attn_bwd_mfma(const AttnBwdMfmaArgs &a, const float *dout, const bf16 *o, float *dk, float *dv,
                          hipStream_t s);
// dst[c][vcol[m]] = src[m][c] (C % 64 == 0, 16-byte aligned rows)
void launch_transpose_cols(const bf16 *src, long long lds, int M, int C, const int *vcol, bf16 *dst, long long ldt,
                           hipStream_t s);
void launch_attn_prefill_bf16(const AttnPrefillArgs &a, hipStream_t s);

struct AttnDecodeArgs {
  // The new position of each sequence b: its q|k|v projection row b (fp32,
  // in.nslab partial slabs, H + 2 slots of 128), the RoPE tables and QK-norm
  // setting, the paged cache, the layer and H.  The kernel builds q, appends
  // k and v at position lens[b] and attends over positions 0 .. lens[b].
  ScatterArgs in;
  int n;
  int max_splits;   // chunks per sequence in the partial buffers' layout
  int chunk_pages;  // cached pages per chunk: 1 .. 16
  int work;         // chunks that hold positions: the grid's x extent
  const int *map;   // [work][kDecodeMapStride], the step's work list (DecodeMapArgs)
  float *o_part;  // [n][max_splits][H][128], one split per chunk
  float *ml_part; // [n][max_splits][H][2]
  bf16 *o;        // [n][H*128]
  unsigned *ctr;  // [n] chunk-completion counters, zero before first use
};
void launch_attn_decode_bf16(const AttnDecodeArgs &a, hipStream_t s);

struct AttnF32Args {
  const float *q, *k, *v;  // prefill: [M][H*dh], [M][Hkv*dh]
  const int *seq, *pos;
  int M, H, Hkv, dh;
  PagedKV kv;  // decode
  int layer;
  float *o;
};
void launch_attn_prefill_f32(const AttnF32Args &a, hipStream_t s);
void launch_attn_decode_f32(const AttnF32Args &a, hipStream_t s);

constexpr int kDecodeMapStride = 16;                 // ints per decode work-list entry (8 pages)
constexpr int kDecodeMinChunkPages = 2;              // smallest chunk the partial buffers are sized for
constexpr int kDecodeMaxPositions = 16384;           // longest cached sequence the bf16 decode accepts
constexpr int kLogitsPartCols = 64;  // columns per LM-head softmax partial (one wave's width)
