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
#include <type_traits>

#include "scatter.h"

namespace {

constexpr int BK = 64;

// LDS tile [rows][64 bf16]: 16-byte chunk c of row r is stored in slot
// c ^ ((r / 2) % 8), so the 16 rows one ds_read_b128 phase touches (lanes
// 0-15 of a fragment read) land in 16 distinct 16-byte bank groups.
DEV int swz_key(int row) { return (row >> 1) & 7; }
DEV int swz(int row, int chunk) { return row * BK + ((chunk ^ swz_key(row)) << 3); }

DEV const bf16 *wrow(const GemmArgs &g, int n) {
  if (n < g.n1) return (const bf16 *)g.W0 + (long long)n * g.ldw;
  if (n < g.n2) return (const bf16 *)g.W1 + (long long)(n - g.n1) * g.ldw;
  return (const bf16 *)g.W2 + (long long)(n - g.n2) * g.ldw;
}

// Store 4 consecutive outputs of row m starting at column n.  XWG: fp32
// results are read back by another workgroup of the same kernel.
template <int EPI, bool XWG = false>
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
    float *p = (float *)g.C + (long long)m * g.ldc + n;
    f32x4 x = *(const f32x4 *)p;
    x[0] += v0; x[1] += v1; x[2] += v2; x[3] += v3;
    if constexpr (XWG) xst4(p, x);
    else *(f32x4 *)p = x;
  } else {
    float *p = (float *)g.C + (long long)m * g.ldc + n;
    if constexpr (XWG) xst4(p, (f32x4){v0, v1, v2, v3});
    else *(f32x4 *)p = (f32x4){v0, v1, v2, v3};
  }
}

// QKV epilogue.  The wave's 128 columns are one head: a query head, the K
// head or the V head.  Lane (c32, hi) holds, for row m, the columns
// 32 i + 8 c + 4 hi + e (i, c, e < 4), so the rotary partners (p, p + 64) are
// acc[i] and acc[i + 2] of the same lane.  q and k are rotated by the tabled
// angle of their position, then divided by their RMS over the head (the
// partner lane l ^ 32 holds the other 64 columns), and stored as bf16; v is
// stored transposed for the attention kernels.
template <int TM>
DEV void epi_qkv(const GemmArgs &g, f32x16 (&acc)[4][TM], int mw0, int nw0, int c32, int hi) {
  const QkvEpi &e = g.qkv;
  const int head = nw0 / 128;
  const bool is_q = head < e.H, is_k = !is_q && head < e.H + e.Hkv;
  const int kvh = is_q ? 0 : (is_k ? head - e.H : head - e.H - e.Hkv);
  const int kvd = e.Hkv * 128;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    __builtin_amdgcn_sched_barrier(0);  // one row block at a time (register pressure)
    const int m = mw0 + 32 * j + c32;
    const int mm = min(m, g.M - 1);
    const int p = e.pos[mm];
    if (!(is_q || is_k)) {
      // V: transposed store v^T[dim][column of the row]
      if (m < g.M) {
        const long long col = e.vcol ? e.vcol[m] : m;
        bf16 *cv = nullptr;
        int slot = 0;
        if (e.use_cache) {
          const int b = e.seq ? e.seq[m] : m;
          const int page = e.kv.table[b * e.kv.pages_per_seq + p / e.kv.page_size];
          slot = p % e.kv.page_size;
          cv = (bf16 *)(e.kv.base + (long long)e.layer * e.kv.layer_stride +
                        (long long)page * e.kv.page_stride + e.kv.half_bytes);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int dim = kvh * 128 + 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bf16 y = f2bf(acc[i][j][r]);
            if (e.vt_out) e.vt_out[(long long)dim * e.ldvt + col] = y;
            if (cv) cv[(long long)dim * e.kv.page_size + slot] = y;
          }
      }
      continue;
    }
    if (e.cos) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int pi = 32 * i + 8 * c + 4 * hi;
          const float4 cs = *(const float4 *)(e.cos + (long long)p * 64 + pi);
          const float4 sn = *(const float4 *)(e.sin + (long long)p * 64 + pi);
          const float cc[4] = {cs.x, cs.y, cs.z, cs.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float a = acc[i][j][4 * c + q], b = acc[i + 2][j][4 * c + q];
            acc[i][j][4 * c + q] = a * cc[q] - b * ss[q];
            acc[i + 2][j][4 * c + q] = a * ss[q] + b * cc[q];
          }
        }
    }
    float rs = 1.0f;
    if (e.qk_norm) {
      float ssum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) ssum += acc[i][j][r] * acc[i][j][r];
      ssum += __shfl_xor(ssum, 32, 64);
      rs = 1.0f / sqrtf(ssum * (1.0f / 128.0f) + e.eps);
    }
    if (m >= g.M) continue;
    bf16 *dst = is_q ? e.q_out + (long long)m * e.H * 128 + head * 128
                     : (e.k_out ? e.k_out + (long long)m * kvd + kvh * 128 : nullptr);
    bf16 *ck = nullptr;
    if (is_k && e.use_cache) {
      const int b = e.seq ? e.seq[m] : m;
      const int page = e.kv.table[b * e.kv.pages_per_seq + p / e.kv.page_size];
      ck = (bf16 *)(e.kv.base + (long long)e.layer * e.kv.layer_stride + (long long)page * e.kv.page_stride) +
           (long long)(p % e.kv.page_size) * kvd + kvh * 128;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = 32 * i + 8 * c + 4 * hi;
        bf16x4 o = {f2bf(acc[i][j][4 * c] * rs), f2bf(acc[i][j][4 * c + 1] * rs),
                    f2bf(acc[i][j][4 * c + 2] * rs), f2bf(acc[i][j][4 * c + 3] * rs)};
        if (dst) *(bf16x4 *)(dst + col) = o;
        if (ck) *(bf16x4 *)(ck + col) = o;
      }
  }
}

#define GLOBAL_PTR(p) ((const void __attribute__((address_space(1))) *)(p))
#define LDS_PTR(p) ((void __attribute__((address_space(3))) *)(p))

// NWN waves along N and 2 along M: NWN = 2 gives 4 waves (one per SIMD)
// with 128x128 wave tiles; NWN = 4 gives 8 waves (two per SIMD) with
// 128x64 wave tiles, so one wave's LDS and DMA traffic overlaps the other's
// MFMAs.
template <int BM, int BN, int NWN, int EPI>
__global__ __launch_bounds__(128 * NWN) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NW = 2 * NWN;
  constexpr int WM = BM / 2, WN = BN / NWN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int PA = BM / 8 / NW, PB = BN / 8 / NW;  // 1 KB direct-to-LDS loads per wave per k-tile
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

  // Direct global->LDS loads (global_load_lds_dwordx4): one instruction of a
  // wave fills 1 KB of LDS = 8 rows of 64 bf16, lane i landing at row i/8,
  // 16-byte slot i%8.  The slot holds logical k-chunk (i%8) ^ swz_key(row),
  // so the lane loads that chunk: the XOR swizzle costs nothing.  Instruction p of
  // wave w covers rows (4p + w)*8 .. +8; 8-row groups never straddle a
  // weight segment (segment boundaries are multiples of 128), so the row
  // base is wave-uniform and a lane keeps a 32-bit offset.  Instruction p of
  // wave w covers rows (NW p + w)*8 .. +8.
  const int lr = lane >> 3;
  int aoff[PA], boff[PB];
  const bf16 *bbase[PB];
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const int lrow = (NW * p + wave) * 8 + lr;  // row within the tile
    const int r = min(m0 + lrow, g.M - 1);
    aoff[p] = r * (int)g.lda + (((lane & 7) ^ swz_key(lrow)) << 3);
  }
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const int nb = min(n0 + (NW * p + wave) * 8, g.N - 8);
    const bf16 *base;
    int first;
    if (nb < g.n1) { base = (const bf16 *)g.W0; first = 0; }
    else if (nb < g.n2) { base = (const bf16 *)g.W1; first = g.n1; }
    else { base = (const bf16 *)g.W2; first = g.n2; }
    bbase[p] = base;
    const int lrow = (NW * p + wave) * 8 + lr;
    boff[p] = (nb - first + lr) * (int)g.ldw + (((lane & 7) ^ swz_key(lrow)) << 3);
  }
  const bf16 *abase = (const bf16 *)g.A;
  auto dma = [&](int kt, int buf) {
#pragma unroll
    for (int p = 0; p < PA; ++p)
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(abase + aoff[p] + kt * BK),
                                       LDS_PTR(&sa[buf][(NW * p + wave) * 8 * BK]), 16, 0, 0);
#pragma unroll
    for (int p = 0; p < PB; ++p)
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(bbase[p] + boff[p] + kt * BK),
                                       LDS_PTR(&sb[buf][(NW * p + wave) * 8 * BK]), 16, 0, 0);
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = (f32x16){};

  const int KT = g.K / BK;
  const int c32 = lane & 31, hi = lane >> 5;
  // MFMA operand fragments, double-buffered across the 16-deep k substeps
  bf16x8 fa[2][TM], fb[2][TN];
  auto lfrag = [&](int f, int buf, int s) {
#pragma unroll
    for (int j = 0; j < TM; ++j) fa[f][j] = *(const bf16x8 *)&sa[buf][swz(wm * WM + 32 * j + c32, 2 * s + hi)];
#pragma unroll
    for (int i = 0; i < TN; ++i) fb[f][i] = *(const bf16x8 *)&sb[buf][swz(wn * WN + 32 * i + c32, 2 * s + hi)];
  };
  auto mfmas = [&](int f) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][i], fa[f][j], acc[i][j], 0, 0, 0);
  };
  auto interleave = [&]() {  // MFMA / LDS-read pairs, then the remaining MFMAs
#pragma unroll
    for (int q = 0; q < TM + TN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - TM - TN, 0);
  };

  // Main loop over k-tiles.  LDS buffer kt&1 holds k-tile kt; the DMA of
  // k-tile kt+1 into the other buffer is issued first and overlaps the four
  // MFMA substeps of k-tile kt.  Fragments of substep s+1 are read while the
  // MFMAs of substep s run.  The single barrier of a k-tile sits after
  // substep 2: by then every wave has read all of buffer kt&1 and (after its
  // vmcnt wait) landed its share of k-tile kt+1, so substep 3's MFMAs overlap
  // the first fragment reads of k-tile kt+1.
  dma(0, 0);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  lfrag(0, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) dma(kt + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    lfrag(1, buf, 1);
    mfmas(0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    lfrag(0, buf, 2);
    mfmas(1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    lfrag(1, buf, 3);
    mfmas(0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (more) lfrag(0, buf ^ 1, 0);
    mfmas(1);
    if (more) interleave();
    __builtin_amdgcn_sched_barrier(0);
  }
  // A wave whose columns lie beyond N computed on clamped rows; drop it.
  const bool active = (n0 + wn * WN) < g.N;
  if (!active) return;
  const int nw0 = n0 + wn * WN;  // first column of this wave (multiple of WN)
  if constexpr (EPI == EPI_QKV) {
    static_assert(WN == 128, "the QKV epilogue needs one head per wave");
    epi_qkv<TM>(g, acc, m0 + wm * WM, nw0, c32, hi);
    return;
  } else {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wm * WM + 32 * j + c32;
      const bool ok = m < g.M;
      if constexpr (EPI == EPI_LOGITS) {
        // partial softmax statistics of this row over the wave's WN columns
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        float se = 0.f;
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) se += fast_exp2((acc[i][j][r] - mx) * kLog2e);
        se += __shfl_xor(se, 32, 64);
        if (ok && hi == 0) {
          float *pp = g.part + ((long long)m * (g.N / WN) + nw0 / WN) * 2;
          *(float2 *)pp = make_float2(mx, se);
        }
      }
      if (!ok) continue;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int n = nw0 + 32 * i + 8 * c + 4 * hi;
          epi_store4<EPI == EPI_LOGITS ? EPI_F32 : EPI>(g, m, n, acc[i][j][4 * c], acc[i][j][4 * c + 1],
                                                        acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]);
        }
    }
  }
}

// ------------------------------------------------------------------ skinny

constexpr int SK_KSTEP = 128;  // k granularity of a split (four steps of 32)

// The fusions of SkinnyFuse are done by the last workgroup to finish: what
// the others hand over is stored and loaded with sc1 accesses, and arrival
// is counted only after the workgroup's stores have completed.  Called by
// every thread; the answer is broadcast through *flag.
DEV bool last_arrival(unsigned *ctr, unsigned total, int *flag) {
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) *flag = arrive(ctr) == total - 1;
  __syncthreads();
  return *flag;
}

// Workgroup (nb, kz): output columns nb*16 .. +16 for all M <= 16 MB rows,
// k range kz*KS .. +KS (KS = K without a split).  Its NW waves share that
// range: wave w takes the k-steps of 32 at w, w + NW, ..., UNR loads in
// flight before their MFMAs, and the waves' sums meet in LDS.  Lane l of an
// MFMA holds weight row n0 + l%16 and activation row 16 mb + l%16, k
// elements 8 (l/16) .. +8 of the step.
template <int EPI, int MB, int NW>
__global__ __launch_bounds__(64 * NW, 4) void gemm_skinny_kernel(GemmArgs g, int ksplit, SkinnyFuse f) {
  constexpr int UNR = MB <= 2 ? 8 : 4;
  __shared__ f32x4 red[NW][MB][64];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int n0 = blockIdx.x * 16, kz = blockIdx.y;
  const int KS = g.K / ksplit;
  const int kbeg = kz * KS;
  const bf16 *w = wrow(g, n0 + l16) + 8 * q4 + kbeg;
  const bf16 *x[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int m = min(mb * 16 + l16, g.M - 1);
    x[mb] = (const bf16 *)g.A + (long long)m * g.lda + 8 * q4 + kbeg;
  }
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (f32x4){};
  const int steps = KS / 32;
  for (int st = wave; st < steps; st += UNR * NW) {
    bf16x8 wf[UNR], xf[UNR][MB];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (st + u * NW < steps) {  // wave-uniform
        const int k = (st + u * NW) * 32;
        wf[u] = *(const bf16x8 *)(w + k);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[u][mb] = *(const bf16x8 *)(x[mb] + k);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (st + u * NW < steps)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[u], xf[u][mb], acc[mb], 0, 0, 0);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  // wave mb < MB owns rows mb*16 + l16, columns n0 + 4 q4 .. +4
  const int m = wave * 16 + l16;
  const bool own = wave < MB && m < g.M;
  f32x4 sum = {};
  if (wave < MB) {
    sum = red[0][wave][lane];
#pragma unroll
    for (int k = 1; k < NW; ++k) sum += red[k][wave][lane];
  }
  if (ksplit > 1) {
    if (own) xst4(f.part + ((long long)kz * g.M + m) * g.N + n0 + 4 * q4, sum);
    if (!last_arrival(&f.tile_ctr[blockIdx.x], (unsigned)ksplit, &s_last)) return;
    if (tid == 0) f.tile_ctr[blockIdx.x] = 0u;
    if (own) {
      sum = xld4(f.part + (long long)m * g.N + n0 + 4 * q4);
      for (int k = 1; k < ksplit; ++k) sum += xld4(f.part + ((long long)k * g.M + m) * g.N + n0 + 4 * q4);
    }
  }
  if (f.mode == SK_PLAIN) {
    if (own) epi_store4<EPI>(g, m, n0 + 4 * q4, sum[0], sum[1], sum[2], sum[3]);
    return;
  }
  if (own) epi_store4<EPI, true>(g, m, n0 + 4 * q4, sum[0], sum[1], sum[2], sum[3]);
  // group completion: the whole GEMM (SK_NORM) or one 128-wide head slot (SK_QKV)
  const int gid = f.mode == SK_QKV ? n0 / 128 : 0;
  const unsigned total = f.mode == SK_QKV ? 8u : gridDim.x;
  if (!last_arrival(&f.grp_ctr[gid], total, &s_last)) return;
  if (tid == 0) f.grp_ctr[gid] = 0u;
  const float *C = (const float *)g.C;
  if (f.mode == SK_QKV) {
    rope_norm_scatter_rows_xwg(f.sc, C + gid * 128, g.ldc, g.M, gid, wave, NW, lane);
    return;
  }
  switch ((g.N + 255) / 256) {
#define NORM_CASE(k) \
  case k: rmsnorm_rows_xwg<k>(C, g.ldc, f.norm_out, g.N, g.M, g.N, f.eps, wave, NW, lane); break;
    NORM_CASE(1) NORM_CASE(2) NORM_CASE(3) NORM_CASE(4) NORM_CASE(5) NORM_CASE(6) NORM_CASE(7) NORM_CASE(8)
#undef NORM_CASE
    default: break;  // unreachable: the bf16 path has d_model = n_head * 128 <= 2048
  }
}

// Number of k splits across workgroups (only when a split scratch is given):
// the largest divisor of K / 128 that keeps the grid at or below 1024
// workgroups.
int skinny_ksplit(int N, int K) {
  const int units = K / SK_KSTEP, nb = N / 16;
  int best = 1;
  for (int d = 1; d <= units; ++d)
    if (units % d == 0 && nb * d <= 1024) best = d;
  return best;
}

// Waves per workgroup: many column blocks (the LM head) keep four; few
// blocks with a long k range take eight or sixteen so that the range is
// covered by more loads in flight instead of a split across workgroups.
int skinny_waves(int N, int K, int ks) {
  const int nb = N / 16, steps = K / ks / 32;
  if (nb >= 512 || steps < 16) return 4;
  return steps < 48 ? 8 : 16;
}

template <int EPI, int MB>
void launch_sk_mb(const GemmArgs &g, const SkinnyFuse &f, int ks, int nw, hipStream_t s) {
  const dim3 grid(g.N / 16, ks);
  switch (nw) {
    case 4: gemm_skinny_kernel<EPI, MB, 4><<<grid, 256, 0, s>>>(g, ks, f); break;
    case 8: gemm_skinny_kernel<EPI, MB, 8><<<grid, 512, 0, s>>>(g, ks, f); break;
    default: gemm_skinny_kernel<EPI, MB, 16><<<grid, 1024, 0, s>>>(g, ks, f); break;
  }
}

template <int EPI>
void launch_sk(const GemmArgs &g, const SkinnyFuse &f, hipStream_t s) {
  const int ks = f.part ? skinny_ksplit(g.N, g.K) : 1;
  const int nw = skinny_waves(g.N, g.K, ks);
  switch ((g.M + 15) / 16) {
    case 1: launch_sk_mb<EPI, 1>(g, f, ks, nw, s); break;
    case 2: launch_sk_mb<EPI, 2>(g, f, ks, nw, s); break;
    case 3: launch_sk_mb<EPI, 3>(g, f, ks, nw, s); break;
    default: launch_sk_mb<EPI, 4>(g, f, ks, nw, s); break;
  }
}

template <int EPI>
void launch_big(const GemmArgs &g, hipStream_t s) {
  constexpr int BM = 256, BN = 256;
  // the QKV epilogue needs a whole 128-wide head per wave
  constexpr int NWN = EPI == EPI_QKV ? 2 : 4;
  static_assert(EPI != EPI_LOGITS || BN / NWN == kLogitsPartCols, "partial width");
  int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  gemm_bf16_kernel<BM, BN, NWN, EPI><<<tiles, 128 * NWN, 0, s>>>(g);
}

}  // namespace

void launch_gemm_bf16(const GemmArgs &g, hipStream_t s) {
  if (g.M <= 0) return;
  switch (g.epi) {
    case EPI_BF16: launch_big<EPI_BF16>(g, s); break;
    case EPI_RELU2_BF16: launch_big<EPI_RELU2_BF16>(g, s); break;
    case EPI_RESID: launch_big<EPI_RESID>(g, s); break;
    case EPI_LOGITS: launch_big<EPI_LOGITS>(g, s); break;
    case EPI_QKV: launch_big<EPI_QKV>(g, s); break;
    default: launch_big<EPI_F32>(g, s); break;
  }
}

void launch_gemm_bf16_skinny(const GemmArgs &g, const SkinnyFuse &f, hipStream_t s) {
  if (g.M <= 0) return;
  switch (g.epi) {
    case EPI_BF16: launch_sk<EPI_BF16>(g, f, s); break;
    case EPI_RELU2_BF16: launch_sk<EPI_RELU2_BF16>(g, f, s); break;
    case EPI_RESID: launch_sk<EPI_RESID>(g, f, s); break;
    default: launch_sk<EPI_F32>(g, f, s); break;
  }
}
