// bf16 MFMA GEMMs for gfx950: C[m][n] = sum_k A[m][k] W[n][k] (both operands
// K-contiguous), fp32 accumulation, fused epilogues (bf16 store, ReLU^2 ->
// bf16, fp32 residual add, fp32 store).
//
// Large-M kernel: 256x256x64 tiles staged through double-buffered LDS by
// direct-to-LDS loads with a 16-byte XOR swizzle, one
// v_mfma_f32_32x32x16_bf16 per 32x32 block and 16-deep k substep; eight waves
// in two groups that alternate load and compute phases.  The MFMA
// A operand is the weight tile and the B operand the activation tile, so a
// lane's accumulator holds one activation row and runs of 4 consecutive
// output columns (vector stores in the epilogue).  Workgroup ids are remapped
// so consecutive tiles share an XCD (8 XCDs, round-robin dispatch) and
// grouped 8 tile-rows at a time for L2 reuse.
//
// Decode-row kernel (M <= 64): one workgroup per 64 output columns (and k
// range, when k is split), weight and activation chunks staged through a
// multi-stage LDS ring by whole-line direct-to-LDS loads, then
// v_mfma_f32_16x16x32_bf16 from LDS.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

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
  } else if constexpr (EPI == EPI_DRELU2) {
    // d/dz max(z, 0)^2 = 2 max(z, 0) = 2 sqrt(u)
    const bf16x4 u = *(const bf16x4 *)(g.aux + (long long)m * g.ldc + n);
    bf16x4 o = {f2bf(v0 * 2.f * sqrtf(bf2f(u[0]))), f2bf(v1 * 2.f * sqrtf(bf2f(u[1]))),
                f2bf(v2 * 2.f * sqrtf(bf2f(u[2]))), f2bf(v3 * 2.f * sqrtf(bf2f(u[3])))};
    *(bf16x4 *)((bf16 *)g.C + (long long)m * g.ldc + n) = o;
  } else if constexpr (EPI == EPI_RESID) {
    float *p = (float *)g.C + (long long)m * g.ldc + n;
    f32x4 x = *(const f32x4 *)(g.rin ? g.rin + (long long)m * g.ldc + n : p);
    x[0] += v0; x[1] += v1; x[2] += v2; x[3] += v3;
    *(f32x4 *)p = x;
  } else {
    *(f32x4 *)((float *)g.C + (long long)m * g.ldc + n) = (f32x4){v0, v1, v2, v3};
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
          slot = vslot(p % e.kv.page_size);
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

// Tile origin of this workgroup.  XCD-aware remap: the hardware hands
// workgroup ids to the 8 XCDs round robin; give each XCD a contiguous range
// of logical tiles, then group 8 tile-rows at a time for L2 reuse.
template <int BM, int BN>
DEV void tile_origin(const GemmArgs &g, int &m0, int &n0) {
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
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
  m0 = tm * BM;
  n0 = tn * BN;
}

// Epilogue of a WM x WN wave tile (TM x TN blocks of 32x32) whose first
// row is m0 + wm WM and first column n0 + wn WN.
template <int TM, int TN, int WM, int WN, int EPI>
DEV void tile_epilogue(const GemmArgs &g, f32x16 (&acc)[TN][TM], int m0, int n0, int wm, int wn, int c32,
                       int hi) {
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


// Epilogue of gemm_pp_kernel's 128x64 wave tiles through LDS (the operand
// buffers are free once the main loop is done).  In the accumulator layout a
// store instruction covers 32 rows x 32 bytes; here each wave writes one
// 32-row block at a time into its own LDS area and reads it back so that 16
// lanes cover 64 consecutive columns of one row: every store instruction
// then writes whole 128-byte lines (bf16: 128-byte halves of 256-byte rows),
// and a residual add reads whole lines.  The area's row pitch of 68 floats
// keeps both the block writes and the row reads free of bank conflicts.
constexpr int kStagePitch = 68;
template <int TM, int TN, int WM, int WN, int EPI>
DEV void tile_epilogue_staged(const GemmArgs &g, f32x16 (&acc)[TN][TM], int m0, int n0, int wm, int wn,
                              int c32, int hi, int lane, float *stg) {
  static_assert((WN == 64 || WN == 96) && EPI != EPI_QKV, "staged epilogue: 64- or 96-column wave tiles");
  const bool active = (n0 + wn * WN) < g.N;
  if (!active) return;
  const int nw0 = n0 + wn * WN;
  if constexpr (EPI == EPI_LOGITS || EPI == EPI_LOSS || EPI == EPI_LOGITS_BF16) {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wm * WM + 32 * j + c32;
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
      if (m < g.M && hi == 0) {
        float *pp = g.part + ((long long)m * (g.N / WN) + nw0 / WN) * 2;
        *(float2 *)pp = make_float2(mx, se);
      }
    }
  }
  if constexpr (EPI == EPI_LOSS) {
    // no logits leave the chip: only each row's target logit, read back from
    // the staged 32-row block by the lane that owns the row
    static_assert(WN == 64, "one partial block per wave");
#pragma unroll
    for (int j = 0; j < TM; ++j) {
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *(f32x4 *)&stg[c32 * kStagePitch + 32 * i + 8 * c + 4 * hi] =
              (f32x4){acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]};
      const int m = m0 + wm * WM + 32 * j + c32;
      if (hi == 0 && m < g.M) {
        const int col = g.targets[m] - nw0;
        if (col >= 0 && col < WN) g.tgt[m] = stg[c32 * kStagePitch + col];
      }
    }
    return;
  }
  constexpr int EPS = EPI == EPI_LOGITS ? EPI_F32 : EPI;
  static_assert(EPI != EPI_LOGITS_BF16 || WN == 64, "one partial block per wave");
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    // EPI_LOGITS_BF16: the lane that owns row mrow keeps its target logit
    // (fp32, from the staged block) when the target falls in this wave tile
    const int mrow = m0 + wm * WM + 32 * j + c32;
    int tcol = -1;
    if constexpr (EPI == EPI_LOGITS_BF16)
      if (hi == 0 && mrow < g.M) tcol = g.targets[mrow] - nw0;
    // columns 0-63 of the wave tile, then (96-wide tiles) columns 64-95
#pragma unroll
    for (int i0 = 0; i0 < TN; i0 += 2) {
      const int ni = TN - i0 >= 2 ? 2 : 1;   // 32-column blocks in this pass
      const int lpr = 8 * ni;                // lanes per 32 ni-column row
      const int rr = lane / lpr, cc = 4 * (lane % lpr);
#pragma unroll
      for (int i = 0; i < ni; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *(f32x4 *)&stg[c32 * kStagePitch + 32 * i + 8 * c + 4 * hi] =
              (f32x4){acc[i0 + i][j][4 * c], acc[i0 + i][j][4 * c + 1], acc[i0 + i][j][4 * c + 2],
                      acc[i0 + i][j][4 * c + 3]};
      if constexpr (EPI == EPI_LOGITS_BF16)
        if (tcol >= 32 * i0 && tcol < 32 * (i0 + ni)) g.tgt[mrow] = stg[c32 * kStagePitch + tcol - 32 * i0];
#pragma unroll
      for (int q = 0; q < 4 * ni; ++q) {
        const int r = (64 / lpr) * q + rr;
        const f32x4 v = *(const f32x4 *)&stg[r * kStagePitch + cc];
        const int m = m0 + wm * WM + 32 * j + r;
        const int n = nw0 + 32 * i0 + cc;
        if (m >= g.M) continue;
        if constexpr (EPI == EPI_LOGITS) {
          // nothing in this pass reads the logits again: non-temporal stores
          // keep them from displacing the operands in L2 (10% on the LM head)
          __builtin_nontemporal_store(v, (f32x4 *)((float *)g.C + (long long)m * g.ldc + n));
        } else if constexpr (EPI == EPI_LOGITS_BF16) {
          const bf16x4 o = {f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])};
          __builtin_nontemporal_store(o, (bf16x4 *)((bf16 *)g.C + (long long)m * g.ldc + n));
        } else {
          epi_store4<EPS>(g, m, n, v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

// Eight waves in two groups of four (one wave per SIMD each); group q owns
// rows 128 q .. 128 q + 127 of the 256x256 tile, wave w of a group columns
// 64 w .. 64 w + 63 (for QKV: rows 64 (w / 2) .. and columns 128 (w % 2) ..
// of the group's half).  The groups alternate between a load phase (the LDS ->
// register reads of two 16-deep substeps) and a compute phase (their 16
// MFMAs), group 1 one phase behind group 0, so each SIMD's matrix core runs
// one group's compute phase while the other group loads.  Every phase ends
// at a workgroup barrier, and a load phase's reads have completed before it.
// Each group streams half of every k-tile into LDS by DMA.  Both issue their
// half of k-tile t+1 in their first load phase of k-tile t, after its reads
// (the target buffer was last read two phases earlier), and both wait for it
// three phases later: group 0 after its last compute phase of k-tile t,
// group 1 before the barrier that ends its last load phase.
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs g) {
  if constexpr (EPI == EPI_F32) {
    if (gridDim.y > 1) {  // k split: this grid row's slice of K and its output slab
      const long long k0 = (long long)blockIdx.y * g.K;
      g.A = (const bf16 *)g.A + k0;
      g.W0 = (const bf16 *)g.W0 + k0;
      g.W1 = (const bf16 *)g.W1 + k0;
      g.W2 = (const bf16 *)g.W2 + k0;
      g.C = (float *)g.C + blockIdx.y * g.slab;
    }
  }
  // The QKV epilogue needs a whole 128-wide head per wave, and 192-column
  // tiles split into 96-column wave tiles: there the four waves of a group
  // split its 128 rows in two and the columns in two (64x128 or 64x96 wave
  // tiles); otherwise 128x64.
  constexpr bool WIDE = EPI == EPI_QKV || BN == 192;
  constexpr int NW = 8, WM = WIDE ? BM / 4 : BM / 2, WN = WIDE ? BN / 2 : BN / 4;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int PA = BM / 8 / NW, PB = BN / 8 / NW;  // 1 KB direct-to-LDS loads per wave per k-tile
  // One LDS object per buffer, so the compiler can tell a DMA into one
  // buffer from reads of the other and adds no wait for it.
  __shared__ bf16 sa0[BM * BK], sa1[BM * BK];
  __shared__ bf16 sb0[BN * BK], sb1[BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wm = WIDE ? 2 * grp + ((wave >> 1) & 1) : grp, wn = WIDE ? wave & 1 : wave & 3;
  int m0, n0;
  tile_origin<BM, BN>(g, m0, n0);

  // Direct global->LDS loads (global_load_lds_dwordx4): one instruction of a
  // wave fills 1 KB of LDS = 8 rows of 64 bf16, lane i landing at row i/8,
  // 16-byte slot i%8.  The slot holds logical k-chunk (i%8) ^ swz_key(row),
  // so the lane loads that chunk: the XOR swizzle costs nothing.
  // Instruction p of wave w fills rows (8 p + w) * 8 .. +8 of the tile;
  // 8-row groups never straddle a weight segment (segment boundaries are
  // multiples of 128), so the row base is wave-uniform and a lane keeps a
  // 32-bit offset.
  const int lr = lane >> 3;
  int aoff[PA], boff[PB];
  const bf16 *bbase[PB];
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const int lrow = (NW * p + wave) * 8 + lr;
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
  auto dma = [&](int kt, bf16 *As, bf16 *Bs) {
#pragma unroll
    for (int p = 0; p < PA; ++p)
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(abase + aoff[p] + kt * BK),
                                       LDS_PTR(&As[(NW * p + wave) * 8 * BK]), 16, 0, 0);
#pragma unroll
    for (int p = 0; p < PB; ++p)
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(bbase[p] + boff[p] + kt * BK),
                                       LDS_PTR(&Bs[(NW * p + wave) * 8 * BK]), 16, 0, 0);
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = (f32x16){};

  const int KT = g.K / BK;
  const int c32 = lane & 31, hi = lane >> 5;
  bf16x8 fa[2][TM], fb[2][TN];
  auto lfrag = [&](int f, const bf16 *As, const bf16 *Bs, int s) {
#pragma unroll
    for (int j = 0; j < TM; ++j) fa[f][j] = *(const bf16x8 *)&As[swz(wm * WM + 32 * j + c32, 2 * s + hi)];
#pragma unroll
    for (int i = 0; i < TN; ++i) fb[f][i] = *(const bf16x8 *)&Bs[swz(wn * WN + 32 * i + c32, 2 * s + hi)];
  };
  auto compute = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f][i], fa[f][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto bar = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Waits the compiler sees (a vmcnt(0) in inline asm would leave its own
  // tracking of the DMA in flight): vmcnt(0), and lgkmcnt(0).
  auto wait_dma = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };
  auto wait_lds = [&]() { __builtin_amdgcn_s_waitcnt(0xC07F); };
  // Where the compiler cannot tell which group runs, it adds a vmcnt(0)
  // before a load phase; both groups have waited for their DMA by then.
  auto ktile = [&](int kt, const bf16 *As, const bf16 *Bs, bf16 *nAs, bf16 *nBs) {
    lfrag(0, As, Bs, 0);
    lfrag(1, As, Bs, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < KT) dma(kt + 1, nAs, nBs);
    wait_lds();
    bar();
    compute();
    bar();
    lfrag(0, As, Bs, 2);
    lfrag(1, As, Bs, 3);
    wait_lds();
    if (grp == 1) wait_dma();
    bar();
    compute();
    if (grp == 0) wait_dma();
    // group 1's last compute phase ends the kernel's barriers
    if (!(grp == 1 && kt == KT - 1)) bar();
  };
  dma(0, sa0, sb0);
  wait_dma();
  bar();
  if (grp == 1) bar();
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    ktile(kt, sa0, sb0, sa1, sb1);
    ktile(kt + 1, sa1, sb1, sa0, sb0);
  }
  if (kt < KT) ktile(kt, sa0, sb0, sa1, sb1);
  // Staging areas: 32 x 68 floats per wave, two waves per 32 KB buffer.  A
  // group reaches its epilogue only after both groups' last LDS reads
  // (group 0 after the barrier that ends group 1's last load phase), and no
  // DMA is in flight by then.
  static_assert(2 * 32 * kStagePitch * 4 <= BM * BK * 2 && 2 * 32 * kStagePitch * 4 <= BN * BK * 2,
                "staging area");
  if constexpr (EPI == EPI_QKV) {
    tile_epilogue<TM, TN, WM, WN, EPI>(g, acc, m0, n0, wm, wn, c32, hi);
  } else {
    bf16 *const sbuf = wave < 2 ? sa0 : wave < 4 ? sa1 : wave < 6 ? sb0 : sb1;
    float *stg = (float *)sbuf + (wave & 1) * 32 * kStagePitch;
    tile_epilogue_staged<TM, TN, WM, WN, EPI>(g, acc, m0, n0, wm, wn, c32, hi, lane, stg);
  }
}

// ------------------------------------------------------------------ decode rows

template <int N>
DEV void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most min(ahead, MAXA) chunks of NI loads each are in flight.
template <int NI, int MAXA>
DEV void wait_ahead(int ahead) {
  if constexpr (MAXA == 0) {
    wait_vm<0>();
  } else {
    if (ahead >= MAXA) wait_vm<MAXA * NI>();
    else wait_ahead<NI, MAXA - 1>(ahead);
  }
}

// Decode-row kernel (M <= 64): one workgroup of 4 waves per BNR output
// columns (64 or 32) and k range kz of ks.  The k range streams in chunks of
// 64 through an S-stage LDS ring holding the BNR weight rows and the
// activation rows (padded to an even number of 16-row blocks), each chunk
// filled by direct-to-LDS loads that read whole 128-byte lines: a wave
// instruction covers 8 rows x 128 B.  Every wave issues the same number NI
// of those per chunk, so "chunk c has landed" is a fixed vmcnt.  BNR = 64:
// wave w multiplies weight rows 16w .. +16 (output columns) by all
// activation rows for both 32-deep k substeps of a chunk.  BNR = 32 (twice
// the workgroups, for grids that would leave CUs idle): wave w takes column
// block w % 2 and substep w / 2, and the two substep halves are added
// through LDS at the end.  v_mfma_f32_16x16x32_bf16: lane l holds weight row
// l%16 / activation row 16 mb + l%16, k elements 8 (l/16) .. +8 of the step.
template <int EPI, int MB, int BNR>
__global__ __launch_bounds__(256) void gemm_rows_kernel(GemmArgs g, int ks, long long slab) {
  constexpr int MBE = (MB + 1) & ~1;      // activation 16-row blocks loaded
  constexpr int ROWS = BNR + 16 * MBE;    // LDS tile rows: weights, then activations
  static_assert((ROWS / 8) % 4 == 0, "DMA instructions must split evenly over the waves");
  constexpr int NI = (ROWS / 8) / 4;      // DMA instructions per wave per chunk
  // Stages: a 72 KB ring, so two workgroups fit on a CU.  A 144 KB ring
  // (one workgroup per CU) was slower on every decode shape, also for grids
  // of fewer workgroups than CUs.
  constexpr int S = 73728 / (ROWS * BK * 2);
  static_assert(S >= 3 && (S - 2) * NI < 64, "ring depth");
  __shared__ bf16 lds[S][ROWS * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int n0 = blockIdx.x * BNR, kz = blockIdx.y;
  const int nck = g.K / BK;
  const int c0 = (int)((long long)kz * nck / ks), c1 = (int)((long long)(kz + 1) * nck / ks);
  const int nch = c1 - c0;

  // DMA slot j of this wave fills tile rows 8 (w + 4 j) .. +8; lane i lands
  // in row i/8, 16-byte slot i%8, which holds logical chunk (i%8) ^ key.
  const bf16 *src[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int slot = wave + 4 * j;
    const int r = 8 * slot + (lane >> 3);
    const int lc = (lane & 7) ^ swz_key(r);
    if (r < BNR) src[j] = wrow(g, n0 + r) + lc * 8 + c0 * BK;
    else src[j] = (const bf16 *)g.A + (long long)min(r - BNR, g.M - 1) * g.lda + lc * 8 + c0 * BK;
  }
  auto dma = [&](int c, int st) {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(src[j] + c * BK), LDS_PTR(&lds[st][8 * (wave + 4 * j) * BK]),
                                       16, 0, 0);
  };

  constexpr int NSUB = BNR == 64 ? 2 : 1;          // k substeps per chunk for this wave
  const int cb = BNR == 64 ? wave : (wave & 1);    // 16-column block of this wave
  const int sub0 = BNR == 64 ? 0 : (wave >> 1);    // first k substep of this wave
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = (f32x4){};
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < nch) dma(j, j);
  for (int c = 0; c < nch; ++c) {
    wait_ahead<NI, S - 2>(nch - 1 - c);  // chunks still allowed in flight after chunk c
    // Chunk c is in LDS and every wave is done with chunk c - 1's stage (its
    // MFMAs consumed those reads).  A bare s_barrier: __syncthreads() would
    // add a workgroup fence, and with it a wait for every load in flight.
    asm volatile("s_barrier" ::: "memory");
    if (c + S - 1 < nch) dma(c + S - 1, (c + S - 1) % S);
    const bf16 *t = lds[c % S];
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      const int ksub = sub0 + i;
      const bf16x8 wf = *(const bf16x8 *)&t[swz(16 * cb + l16, 4 * ksub + q4)];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 xf = *(const bf16x8 *)&t[swz(BNR + 16 * mb + l16, 4 * ksub + q4)];
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf, acc[mb], 0, 0, 0);
      }
    }
  }
  if constexpr (BNR == 32) {
    // add the second substep's partial sums (waves 2, 3) into waves 0, 1
    f32x4 *red = (f32x4 *)&lds[0][0];  // [2 column blocks][MB][64 lanes]
    __syncthreads();                    // every wave is done reading the ring
    if (wave >= 2)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) red[(cb * MB + mb) * 64 + lane] = acc[mb];
    __syncthreads();
    if (wave >= 2) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] += red[(cb * MB + mb) * 64 + lane];
  }
  // lane holds output columns n0 + 16 cb + 4 q4 .. +4 of row 16 mb + l16
  GemmArgs go = g;
  if (ks > 1) go.C = (float *)g.C + kz * slab;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = 16 * mb + l16;
    if (m < g.M) epi_store4<EPI>(go, m, n0 + 16 * cb + 4 * q4, acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
  }
}

template <int EPI, int BNR>
void launch_rows_d(const GemmArgs &g, int ks, long long slab, hipStream_t s) {
  const dim3 grid(g.N / BNR, ks);
  switch ((g.M + 15) / 16) {
    case 1: gemm_rows_kernel<EPI, 1, BNR><<<grid, 256, 0, s>>>(g, ks, slab); break;
    case 2: gemm_rows_kernel<EPI, 2, BNR><<<grid, 256, 0, s>>>(g, ks, slab); break;
    case 3: gemm_rows_kernel<EPI, 3, BNR><<<grid, 256, 0, s>>>(g, ks, slab); break;
    default: gemm_rows_kernel<EPI, 4, BNR><<<grid, 256, 0, s>>>(g, ks, slab); break;
  }
}

template <int EPI>
void launch_rows(const GemmArgs &g, int ks, long long slab, hipStream_t s) {
  // 256 CUs.  Fewer than 128 tiles of 64 columns: halve the tiles.
  const long long t64 = (long long)(g.N / 64) * ks;
  if (t64 < 128) launch_rows_d<EPI, 32>(g, ks, slab, s);
  else launch_rows_d<EPI, 64>(g, ks, slab, s);
}

template <int EPI>
void launch_big(const GemmArgs &g, hipStream_t s) {
  constexpr int BM = 256;
  static_assert((EPI != EPI_LOGITS && EPI != EPI_LOSS && EPI != EPI_LOGITS_BF16) || 256 / 4 == kLogitsPartCols,
                "partial width");
  const int tm = (g.M + BM - 1) / BM;
  const int t256 = tm * ((g.N + 255) / 256);
  if constexpr (EPI == EPI_RESID || EPI == EPI_F32) {
    // 192-column tiles when N splits into them and they take fewer
    // column-rounds over the 256 CUs (d = 768: 256 tiles instead of 192)
    const int t192 = tm * (g.N / 192);
    if (g.N % 192 == 0 && (long long)((t192 + 255) / 256) * 192 < (long long)((t256 + 255) / 256) * 256) {
      gemm_pp_kernel<BM, 192, EPI><<<t192, 512, 0, s>>>(g);
      return;
    }
  }
  gemm_pp_kernel<BM, 256, EPI><<<t256, 512, 0, s>>>(g);
}

// C[i] = sum over z of slabs[z][i], z in order
__global__ __launch_bounds__(256) void slab_sum_kernel(const float *slabs, int ks, long long n, float *C) {
  const long long i4 = (long long)blockIdx.x * 256 + threadIdx.x;
  if (4 * i4 >= n) return;
  f32x4 acc = ((const f32x4 *)slabs)[i4];
  for (int z = 1; z < ks; ++z) acc += ((const f32x4 *)(slabs + (long long)z * n))[i4];
  ((f32x4 *)C)[i4] = acc;
}

}  // namespace

int gemm_splitk_ways(int M, int N, int K) {
  const int tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int ks = (256 + tiles - 1) / tiles;
  ks = std::min(ks, K / (8 * BK));
  while (ks > 1 && K % (ks * BK)) --ks;
  return std::max(ks, 1);
}

void launch_gemm_bf16_splitk(const GemmArgs &g, int ks, float *slabs, hipStream_t s) {
  if (g.M <= 0) return;
  if (ks <= 1) {
    launch_gemm_bf16(g, s);
    return;
  }
  GemmArgs p = g;
  p.epi = EPI_F32;
  p.K = g.K / ks;
  p.C = slabs;
  p.ldc = g.N;
  p.slab = (long long)g.M * g.N;
  const int tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256);
  gemm_pp_kernel<256, 256, EPI_F32><<<dim3(tiles, ks), 512, 0, s>>>(p);
  const long long n = (long long)g.M * g.N;
  slab_sum_kernel<<<(unsigned)((n / 4 + 255) / 256), 256, 0, s>>>(slabs, ks, n, (float *)g.C);
}

void launch_gemm_bf16(const GemmArgs &g, hipStream_t s) {
  if (g.M <= 0) return;
  switch (g.epi) {
    case EPI_BF16: launch_big<EPI_BF16>(g, s); break;
    case EPI_RELU2_BF16: launch_big<EPI_RELU2_BF16>(g, s); break;
    case EPI_RESID: launch_big<EPI_RESID>(g, s); break;
    case EPI_LOGITS: launch_big<EPI_LOGITS>(g, s); break;
    case EPI_LOSS: launch_big<EPI_LOSS>(g, s); break;
    case EPI_LOGITS_BF16: launch_big<EPI_LOGITS_BF16>(g, s); break;
    case EPI_DRELU2: launch_big<EPI_DRELU2>(g, s); break;
    case EPI_QKV: launch_big<EPI_QKV>(g, s); break;
    default: launch_big<EPI_F32>(g, s); break;
  }
}

void launch_gemm_bf16_rows(const GemmArgs &g, int ks, long long slab, hipStream_t s) {
  if (g.M <= 0) return;
  switch (g.epi) {
    case EPI_BF16: launch_rows<EPI_BF16>(g, ks, slab, s); break;
    case EPI_RELU2_BF16: launch_rows<EPI_RELU2_BF16>(g, ks, slab, s); break;
    case EPI_RESID: launch_rows<EPI_RESID>(g, ks, slab, s); break;
    default: launch_rows<EPI_F32>(g, ks, slab, s); break;
  }
}

// About 224 workgroups of 64 columns (timed on the decode shapes: 200 to
// 250 beat both one per CU and the 320 to 400 of two per CU, since each
// range re-reads the activation rows and adds a slab for the consumer to
// sum), at least two 64-deep chunks per k range, at most kMaxRowSplit
// ranges.
int gemm_rows_ksplit(int N, int K) {
  const int tiles = N / 64, chunks = K / BK;
  int ks = (224 + tiles / 2) / tiles;
  ks = std::min(ks, chunks / 2);
  ks = std::min(ks, kMaxRowSplit);
  return std::max(ks, 1);
}
