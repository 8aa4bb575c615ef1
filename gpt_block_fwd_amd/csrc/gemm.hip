// bf16 MFMA GEMMs for gfx950: C[m][n] = sum_k A[m][k] W[n][k] (both operands
// K-contiguous), fp32 accumulation, fused epilogues (bf16 store, ReLU^2 ->
// bf16, fp32 residual add, fp32 store).
//
// Large-M kernel: 256-thread workgroups (4 waves in 2x2), BM x BN x 64 tiles
// staged through double-buffered LDS with a 16-byte XOR swizzle, one
// v_mfma_f32_32x32x16_bf16 per 32x32 block and 16-deep k substep.  The MFMA
// A operand is the weight tile and the B operand the activation tile, so a
// lane's accumulator holds one activation row and runs of 4 consecutive
// output columns (vector stores in the epilogue).  Workgroup ids are remapped
// so consecutive tiles share an XCD (8 XCDs, round-robin dispatch) and
// grouped 8 tile-rows at a time for L2 reuse.
//
// Skinny kernel (decode, M <= 64): one workgroup per 16 output columns, the
// K range split across 8 waves, v_mfma_f32_16x16x32_bf16 fed straight from
// global memory, partial sums reduced through LDS.
#include "kernels.h"

namespace {

constexpr int BK = 64;

DEV int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

DEV const bf16 *wrow(const GemmArgs &g, int n) {
  if (n < g.n1) return (const bf16 *)g.W0 + (long long)n * g.ldw;
  if (n < g.n2) return (const bf16 *)g.W1 + (long long)(n - g.n1) * g.ldw;
  return (const bf16 *)g.W2 + (long long)(n - g.n2) * g.ldw;
}

// Store 4 consecutive outputs of row m starting at column n.
template <int EPI>
DEV void epi_store4(const GemmArgs &g, int m, int n, float v0, float v1, float v2, float v3) {
  if constexpr (EPI == EPI_BF16 || EPI == EPI_RELU2_BF16) {
    if constexpr (EPI == EPI_RELU2_BF16) {
      v0 = fmaxf(v0, 0.f); v0 *= v0;
      v1 = fmaxf(v1, 0.f); v1 *= v1;
      v2 = fmaxf(v2, 0.f); v2 *= v2;
      v3 = fmaxf(v3, 0.f); v3 *= v3;
    }
    bf16x4 o = {f2bf(v0), f2bf(v1), f2bf(v2), f2bf(v3)};
    *(bf16x4 *)((bf16 *)g.C + (long long)m * g.ldc + n) = o;
  } else if constexpr (EPI == EPI_RESID) {
    float4 *p = (float4 *)((float *)g.C + (long long)m * g.ldc + n);
    float4 x = *p;
    x.x += v0; x.y += v1; x.z += v2; x.w += v3;
    *p = x;
  } else {
    *(float4 *)((float *)g.C + (long long)m * g.ldc + n) = make_float4(v0, v1, v2, v3);
  }
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LA = BM / 32, LB = BN / 32;
  __shared__ bf16 sa[2][BM * BK];
  __shared__ bf16 sb[2][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;

  // XCD-aware remap: the hardware hands workgroup ids to the 8 XCDs round
  // robin; give each XCD a contiguous range of logical tiles.
  int pid = blockIdx.x;
  {
    const int xcd = pid & 7, idx = pid >> 3;
    const int per_lo = ntiles >> 3, rem = ntiles & 7;
    pid = xcd < rem ? xcd * (per_lo + 1) + idx : rem * (per_lo + 1) + (xcd - rem) * per_lo + idx;
  }
  constexpr int GROUP_M = 8;
  const int group_size = GROUP_M * tiles_n;
  const int first_m = (pid / group_size) * GROUP_M;
  const int gsize_m = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (pid % group_size) % gsize_m;
  const int tn = (pid % group_size) / gsize_m;
  const int m0 = tm * BM, n0 = tn * BN;

  // Global loads: thread t moves 16 bytes of row (t/8 + 32 i), chunk t%8.
  // Row groups of 32 never straddle a weight segment (segment boundaries
  // are multiples of 128), so each group's base pointer is wave-uniform and
  // only a 32-bit offset lives in a lane register.
  const int lrow = tid >> 3, lchunk = tid & 7;
  const bf16 *abase = (const bf16 *)g.A;
  int aoff[LA];
  const bf16 *bbase[LB];
  int boff[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    int r = min(m0 + lrow + 32 * i, g.M - 1);
    aoff[i] = r * (int)g.lda + lchunk * 8;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int nb = min(n0 + 32 * i, g.N - 32);
    const bf16 *base;
    int first;
    if (nb < g.n1) { base = (const bf16 *)g.W0; first = 0; }
    else if (nb < g.n2) { base = (const bf16 *)g.W1; first = g.n1; }
    else { base = (const bf16 *)g.W2; first = g.n2; }
    bbase[i] = base;
    boff[i] = (nb - first + lrow) * (int)g.ldw + lchunk * 8;
  }
  bf16x8 ra[LA], rb[LB];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *(const bf16x8 *)(abase + aoff[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = *(const bf16x8 *)(bbase[i] + boff[i] + kt * BK);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *(bf16x8 *)&sa[buf][swz(lrow + 32 * i, lchunk)] = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *(bf16x8 *)&sb[buf][swz(lrow + 32 * i, lchunk)] = rb[i];
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = (f32x16){};

  const int KT = g.K / BK;
  const int c32 = lane & 31, hi = lane >> 5;
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int j = 0; j < TM; ++j) fa[j] = *(const bf16x8 *)&sa[buf][swz(wm * WM + 32 * j + c32, 2 * s + hi)];
#pragma unroll
      for (int i = 0; i < TN; ++i) fb[i] = *(const bf16x8 *)&sb[buf][swz(wn * WN + 32 * i + c32, 2 * s + hi)];
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[i], fa[j], acc[i][j], 0, 0, 0);
    }
  };
  // Double-buffered main loop: the next stage's global loads are in flight
  // while the current stage feeds the MFMAs; one barrier per stage.
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT - 1; ++kt) {
    gload(kt + 1);
    compute(kt & 1);
    sstore((kt + 1) & 1);
    __syncthreads();
  }
  compute((KT - 1) & 1);
  // A wave whose 128 columns lie beyond N computed on clamped rows; drop it.
  const bool active = (n0 + wn * WN) < g.N;
  if (!active) return;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wm * WM + 32 * j + c32;
      if (m >= g.M) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = n0 + wn * WN + 32 * i + 8 * c + 4 * hi;
        epi_store4<EPI>(g, m, n, acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2],
                        acc[i][j][4 * c + 3]);
      }
    }
}

// ------------------------------------------------------------------ skinny

constexpr int SK_WAVES = 8;

template <int EPI, int MB>
__global__ __launch_bounds__(64 * SK_WAVES) void gemm_skinny_kernel(GemmArgs g) {
  __shared__ f32x4 red[SK_WAVES][MB][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const bf16 *w = wrow(g, n0 + l16) + 8 * q4;
  const bf16 *x[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int m = min(mb * 16 + l16, g.M - 1);
    x[mb] = (const bf16 *)g.A + (long long)m * g.lda + 8 * q4;
  }
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (f32x4){};
  const int steps = g.K / 32;
  int st = wave;
  // four k-steps per round so that several weight loads are in flight
  for (; st + 3 * SK_WAVES < steps; st += 4 * SK_WAVES) {
    bf16x8 wf[4], xf[4][MB];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = (st + u * SK_WAVES) * 32;
      wf[u] = *(const bf16x8 *)(w + k);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xf[u][mb] = *(const bf16x8 *)(x[mb] + k);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], xf[u][mb], acc[mb], 0, 0, 0);
  }
  for (; st < steps; st += SK_WAVES) {
    const int k = st * 32;
    bf16x8 wf = *(const bf16x8 *)(w + k);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      bf16x8 xf = *(const bf16x8 *)(x[mb] + k);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf, acc[mb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  if (wave >= MB) return;
  const int mb = wave;
  f32x4 s = red[0][mb][lane];
#pragma unroll
  for (int k = 1; k < SK_WAVES; ++k) s += red[k][mb][lane];
  const int m = mb * 16 + l16;
  if (m >= g.M) return;
  epi_store4<EPI>(g, m, n0 + 4 * q4, s[0], s[1], s[2], s[3]);
}

template <int EPI>
void launch_big(const GemmArgs &g, hipStream_t s) {
  constexpr int BM = 256, BN = 256;
  int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  gemm_bf16_kernel<BM, BN, EPI><<<tiles, 256, 0, s>>>(g);
}

template <int EPI>
void launch_sk(const GemmArgs &g, hipStream_t s) {
  int blocks = g.N / 16;
  int mb = (g.M + 15) / 16;
  switch (mb) {
    case 1: gemm_skinny_kernel<EPI, 1><<<blocks, 64 * SK_WAVES, 0, s>>>(g); break;
    case 2: gemm_skinny_kernel<EPI, 2><<<blocks, 64 * SK_WAVES, 0, s>>>(g); break;
    case 3: gemm_skinny_kernel<EPI, 3><<<blocks, 64 * SK_WAVES, 0, s>>>(g); break;
    default: gemm_skinny_kernel<EPI, 4><<<blocks, 64 * SK_WAVES, 0, s>>>(g); break;
  }
}

}  // namespace

void launch_gemm_bf16(const GemmArgs &g, hipStream_t s) {
  if (g.M <= 0) return;
  switch (g.epi) {
    case EPI_BF16: launch_big<EPI_BF16>(g, s); break;
    case EPI_RELU2_BF16: launch_big<EPI_RELU2_BF16>(g, s); break;
    case EPI_RESID: launch_big<EPI_RESID>(g, s); break;
    default: launch_big<EPI_F32>(g, s); break;
  }
}

void launch_gemm_bf16_skinny(const GemmArgs &g, hipStream_t s) {
  if (g.M <= 0) return;
  switch (g.epi) {
    case EPI_BF16: launch_sk<EPI_BF16>(g, s); break;
    case EPI_RELU2_BF16: launch_sk<EPI_RELU2_BF16>(g, s); break;
    case EPI_RESID: launch_sk<EPI_RESID>(g, s); break;
    default: launch_sk<EPI_F32>(g, s); break;
  }
}
