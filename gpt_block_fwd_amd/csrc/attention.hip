// Causal multi-query attention for gfx950 (one K/V head shared by all query
// heads, head width 128, bf16 operands, fp32 softmax and accumulation).
//
// Prefill: the H query heads of a sequence are flattened into rows
// r = position * H + head, which is exactly the memory order of q.  Row r
// sees keys 0 .. r / H.  A workgroup owns kAttnPrefillRows consecutive rows
// (32 per wave); every 64-key K tile and transposed V tile is staged once in
// LDS and serves all of them, so the single K/V head is read once per
// workgroup rather than once per query head.  Scores are formed transposed,
// S^T = K Q^T, so each lane's accumulators hold one row and its softmax
// statistics stay lane-local (one cross-lane exchange per 32 keys); the
// exponentiated scores are already laid out as the B operand of
// O^T = V^T P^T.  Softmax in the base-2 domain, against a fixed reference
// when q and k are QK-normalised, else online.
//
// Decode: one workgroup per chunk of cached pages of a sequence (and K/V
// head).  Chunks of up to 4 pages: 4 waves, each staging a 64-position page
// of K and V^T in LDS with whole-line direct-to-LDS loads; 5 to 16 pages: 8
// waves, each staging its page's K in LDS and loading its V^T fragments into
// registers, in one or two rounds.  Pages are scored with
// v_mfma_f32_16x16x32_bf16, the (<= 16) query heads as the N side.  The last
// chunk of a sequence to finish merges the chunks (log-sum-exp).
#include "kernels.h"
#include "scatter.h"

#define GLOBAL_PTR(p) ((const void __attribute__((address_space(1))) *)(p))
#define LDS_PTR(p) ((void __attribute__((address_space(3))) *)(p))

namespace {

constexpr int DH = 128;
constexpr int KT = 64;  // keys per tile
constexpr float kLazy = 8.0f;  // log2 headroom of the lazy softmax reference
// With QK-norm, q and k have RMS <= 1 per head, so |q.k| <= 128 (1 + 2^-9)^2
// after bf16 rounding and a scaled score |q.k| log2(e) / sqrt(128) stays
// below 16.4: a fixed reference of 16.5 keeps every 2^(score - ref) in
// (2^-33, 1), far from fp32 overflow and underflow.
constexpr float kScoreBound = 16.5f;

// K tile [64 keys][128 dims]: 16-byte chunk c of key r at slot c ^ (r % 16),
// so the 16 keys of a fragment read's lane group hit 16 distinct bank groups.
DEV int kidx(int key, int chunk) { return key * DH + ((chunk ^ (key & 15)) << 3); }
// V^T tile [128 dims][64 stored key columns] (keys in the vperm16 order of
// the V^T buffer): 16-byte chunk c of dim r at slot c ^ ((r / 2) % 8), so a
// fragment read's 16 lanes (dims of both parities) hit 16 distinct bank
// groups.  Both swizzles move whole 16-byte chunks, so direct-to-LDS loads
// can apply them by choosing each lane's source.
DEV int vidx(int dim, int col) { return dim * KT + ((((col >> 3) ^ ((dim >> 1) & 7))) << 3) + (col & 7); }

// NWV waves per workgroup, 32 RB rows each.  FIXREF: q and k are QK-normalised,
// so the softmax runs against the fixed reference kScoreBound (no running
// max, no rescale of the output accumulators).
template <int NWV, int RB, bool FIXREF>
__global__ __launch_bounds__(64 * NWV) void attn_prefill_kernel(AttnPrefillArgs a) {
  constexpr int NT = 64 * NWV, ROWS = 32 * RB * NWV;
  constexpr int SP = 4 * 4 / NWV;  // 16-byte staging loads per thread for each of K and V^T
  // One LDS object per buffer, so the compiler can tell the DMA into one
  // buffer from reads of the other and adds no wait for it.
  __shared__ bf16 sk0[KT * DH], sk1[KT * DH];
  __shared__ bf16 sv0[DH * KT], sv1[DH * KT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  // blockIdx.y counts row blocks from the last one, so the blocks that see
  // the most keys are dispatched first.
  const int b = blockIdx.x, R0 = (a.max_wg - 1 - (int)blockIdx.y) * ROWS;
  // K/V head gk serves the G query heads gk G .. gk G + G - 1; the rows of
  // this grid plane are (position, head of the group) pairs, r = t G + hg.
  const int H = a.H, G = a.H / a.Hkv, gk = blockIdx.z;
  const int kvw = a.Hkv * DH;  // K row width
  const int tok0 = a.cu[b], len = a.cu[b + 1] - tok0;
  const long long col0 = a.cu_pad[b];
  const int rows_total = len * G;
  if (R0 >= rows_total) return;
  const int Rw = R0 + 32 * RB * wave;

  // Q fragments (B operand of S^T = K Q^T): row r, dims 16 s + 8 g .. +8.
  int prow[RB];
  bf16x8 qf[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    int r = min(Rw + 32 * rb + c32, rows_total - 1);
    prow[rb] = r / G;
    const bf16 *qp = a.q + ((long long)(tok0 + prow[rb]) * H + gk * G + (r - prow[rb] * G)) * DH + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[rb][s] = *(const bf16x8 *)(qp + 16 * s);
  }
  const int last_row = min(R0 + ROWS - 1, rows_total - 1);
  const int n_kt = (last_row / G) / KT + 1;
  const int pw_max = Rw < rows_total ? min(Rw + 32 * RB - 1, rows_total - 1) / G : -1;
  const int pw_min = Rw / G;

  // Direct-to-LDS staging: a tile is 16 KB of K (4 keys x 256 B per wave
  // instruction) and 16 KB of V^T (8 dims x 128 B per instruction); wave w
  // issues instructions j = w, w + NWV, ...  Lane i fills 16-byte slot i of
  // the instruction's kilobyte and so loads the logical chunk that slot
  // holds.  Keys past the sequence are clamped to its last key (they are
  // masked); V^T columns past it are zeroed once the tile has landed.
  constexpr int DJ = 16 / NWV;  // instructions per wave for each of K and V^T
  auto dma = [&](int kt, bf16 *sk, bf16 *sv) {
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj) {
      const int j = wave + NWV * jj;
      const int key = 4 * j + (lane >> 4), pc = lane & 15;
      const int gkey = min(kt * KT + key, len - 1);
      __builtin_amdgcn_global_load_lds(
          GLOBAL_PTR(a.k + (long long)(tok0 + gkey) * kvw + gk * DH + ((pc ^ (key & 15)) << 3)),
          LDS_PTR(&sk[j * 512]), 16, 0, 0);
    }
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj) {
      const int j = wave + NWV * jj;
      const int dim = 8 * j + (lane >> 3), pc = lane & 7;
      __builtin_amdgcn_global_load_lds(
          GLOBAL_PTR(a.vt + (long long)(gk * DH + dim) * a.ldvt + col0 + kt * KT + ((pc ^ ((dim >> 1) & 7)) << 3)),
          LDS_PTR(&sv[j * 512]), 16, 0, 0);
    }
  };
  // After a tile has landed (and a barrier): zero its V^T columns past the
  // sequence; the caller puts another barrier before the tile is read.
  auto zero_tail = [&](int kt, bf16 *sv) {
    const int valid = len - kt * KT;  // 1 .. 63 here
    for (int i = tid; i < DH * KT; i += NT) {
      const int dim = i / KT, key = i % KT;
      if (key >= valid) sv[vidx(dim, vperm16(key))] = (bf16)0.f;
    }
  };

  f32x16 oacc[4][RB];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) oacc[d][rb] = (f32x16){};
  float mrow[RB], lrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mrow[rb] = -INFINITY;
    lrow[rb] = 0.f;
  }
  const float sc = kLog2e / sqrtf((float)DH);

  auto tile = [&](int kt, const bf16 *sk, const bf16 *sv) {
    if (kt * KT > pw_max) return;  // every key of the tile is in this wave's future
    f32x16 sacc[2][RB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[kb][rb] = (f32x16){};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 kf = *(const bf16x8 *)&sk[kidx(32 * kb + c32, 2 * s + g)];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[kb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[rb][s], sacc[kb][rb], 0, 0, 0);
      }
    }
    // Online softmax in the base-2 domain with a lazy reference: a row's
    // reference max moves (and its output and sum are rescaled) only when a
    // tile's max exceeds it by more than kLazy, so the probabilities formed
    // against it stay below 2^kLazy and most tiles skip the rescale.
    // Causal masking is needed only on tiles that reach past the wave's
    // first row position (a wave-uniform test).
    const bool need_mask = kt * KT + KT - 1 > pw_min;
    if constexpr (FIXREF) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              int key = kt * KT + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
              if (key > prow[rb]) sacc[kb][rb][r] = -INFINITY;
            }
        }
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float p = fast_exp2(__builtin_fmaf(sacc[kb][rb][r], sc, -kScoreBound));
            sacc[kb][rb][r] = p;
            rs += p;
          }
        rs += __shfl_xor(rs, 32, 64);
        lrow[rb] += rs;
      }
    } else
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int key = kt * KT + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key > prow[rb]) sacc[kb][rb][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][rb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sc;  // scaled tile max of the row
      if (mx > mrow[rb] + kLazy) {
        const float alpha = fast_exp2(mrow[rb] - mx);
        lrow[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) oacc[d][rb] *= alpha;
        mrow[rb] = mx;
      }
      const float mref = mrow[rb];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(sacc[kb][rb][r], sc, -mref));
          sacc[kb][rb][r] = p;
          rs += p;
        }
      rs += __shfl_xor(rs, 32, 64);
      lrow[rb] += rs;
    }
    // O^T += V^T P^T, 16 keys per MFMA; k slot 8g+j <-> key 16h + 8(j/4) + 4g + j%4
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1, h = st & 1;
      bf16x8 pf[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[rb][j] = f2bf(sacc[kb][rb][8 * h + j]);
      // the lane's eight keys are stored columns 32 kb + 16 h + 8 g .. +8
      const int col = 32 * kb + 16 * h + 8 * g;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int dim = 32 * d + c32;
        const bf16x8 vf = *(const bf16x8 *)&sv[vidx(dim, col)];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          oacc[d][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[rb], oacc[d][rb], 0, 0, 0);
      }
    }
  };

  auto land = [&](int kt, bf16 *sv) {  // wait for tile kt's loads (all waves)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt * KT + KT > len) {
      zero_tail(kt, sv);
      __syncthreads();
    }
  };
  // tile kt computes from one buffer while tile kt + 1 streams into the other
  auto step = [&](int kt, bf16 *sk, bf16 *sv, bf16 *nsk, bf16 *nsv) {
    dma(kt + 1, nsk, nsv);
    __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the tile's MFMAs
    tile(kt, sk, sv);
    land(kt + 1, nsv);
  };
  dma(0, sk0, sv0);
  land(0, sv0);
  int kt = 0;
  for (; kt + 2 < n_kt; kt += 2) {
    step(kt, sk0, sv0, sk1, sv1);
    step(kt + 1, sk1, sv1, sk0, sv0);
  }
  if (kt + 1 < n_kt) {
    step(kt, sk0, sv0, sk1, sv1);
    tile(kt + 1, sk1, sv1);
  } else {
    tile(kt, sk0, sv0);
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = Rw + 32 * rb + c32;
    if (r >= rows_total) continue;
    const float inv = 1.0f / lrow[rb];
    const int t = r / G;
    if (a.lse2 && g == 0)  // base-2 log-sum-exp of the row's scaled scores
      a.lse2[(long long)(tok0 + t) * H + gk * G + (r - t * G)] = (FIXREF ? kScoreBound : mrow[rb]) + log2f(lrow[rb]);
    bf16 *op = a.o + ((long long)(tok0 + t) * H + gk * G + (r - t * G)) * DH + 4 * g;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x4 o = {f2bf(oacc[d][rb][4 * c] * inv), f2bf(oacc[d][rb][4 * c + 1] * inv),
                    f2bf(oacc[d][rb][4 * c + 2] * inv), f2bf(oacc[d][rb][4 * c + 3] * inv)};
        *(bf16x4 *)(op + 32 * d + 8 * c) = o;
      }
  }
}

// ------------------------------------------------------------------ backward
// Attention backward on MFMA (bf16 operands, fp32 accumulation), two passes
// that recompute the probabilities P = 2^(s sc - lse2) from the forward's
// base-2 row log-sum-exp:
//   dq pass, row-parallel like the forward: S^T = K Q^T and dP^T = V dO^T
//     per 64-key tile, dS = P (dP - D), dQ^T += K^T dS^T;
//   dk/dv pass, key-parallel with the roles of rows and keys swapped: the
//     workgroup's keys and their V rows are the fragments, 64-position tiles
//     of Q, dO, Q^T and dO^T stream through LDS, dV^T += dO^T P,
//     dK^T += Q^T dS, per query head (a fixed-order sum merges the heads of
//     a K/V group).
// D = dO . O per row.  The transposed operands K^T, Q^T, dO^T are stored like
// the forward's V^T (columns in vperm16 order, zero padding), so P and dS
// feed the MFMA exactly as P does in the forward.

// 64 rows x 128 bf16 of a row tile into the kidx layout: 16 instructions of 1 KB
// (4 rows each), row i of the tile read from base + min(i0 + i, last) * stride.
DEV void dma_rows(bf16 *dst, const bf16 *base, long long stride, int i0, int last, int wave, int nwv, int lane) {
  for (int j = wave; j < 16; j += nwv) {
    const int row = 4 * j + (lane >> 4), pc = lane & 15;
    const int src = min(i0 + row, last);
    __builtin_amdgcn_global_load_lds(GLOBAL_PTR(base + (long long)src * stride + ((pc ^ (row & 15)) << 3)),
                                     LDS_PTR(&dst[j * 512]), 16, 0, 0);
  }
}
// 128 dims x 64 stored columns of a transposed operand into the vidx layout.
DEV void dma_cols(bf16 *dst, const bf16 *base, long long ld, long long col0, int wave, int nwv, int lane) {
  for (int j = wave; j < 16; j += nwv) {
    const int dim = 8 * j + (lane >> 3), pc = lane & 7;
    __builtin_amdgcn_global_load_lds(GLOBAL_PTR(base + (long long)dim * ld + col0 + ((pc ^ ((dim >> 1) & 7)) << 3)),
                                     LDS_PTR(&dst[j * 512]), 16, 0, 0);
  }
}

// Eight waves of 32 rows: two waves per SIMD, so one wave's softmax-gradient
// arithmetic overlaps the other's MFMAs (with four, one wave per SIMD, the
// pass took 140 us per depth-12 layer against 100).
__global__ __launch_bounds__(512) void attn_bwd_dq_kernel(AttnBwdMfmaArgs a) {
  constexpr int NWV = 8, ROWS = 32 * NWV;
  // two buffers of (K rows, V rows, K^T), one LDS object each: the next
  // tile's DMA needs no wait before this tile's reads
  __shared__ bf16 sk0[KT * DH], sv0[KT * DH], skt0[DH * KT];
  __shared__ bf16 sk1[KT * DH], sv1[KT * DH], skt1[DH * KT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  const int b = blockIdx.x, R0 = (a.max_wg - 1 - (int)blockIdx.y) * ROWS;
  const int H = a.H, G = a.H / a.Hkv, gk = blockIdx.z, kvd = a.Hkv * DH;
  const int tok0 = a.cu[b], len = a.cu[b + 1] - tok0;
  const long long col0 = a.cu_pad[b];
  const int rows_total = len * G;
  if (R0 >= rows_total) return;
  const int Rw = R0 + 32 * wave;
  const int r = min(Rw + c32, rows_total - 1);
  const int prow = r / G, hq = gk * G + (r - prow * G);
  const long long qrow = ((long long)(tok0 + prow) * H + hq) * DH;
  bf16x8 qf[8], dof[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qf[s] = *(const bf16x8 *)(a.q + qrow + 16 * s + 8 * g);
    dof[s] = *(const bf16x8 *)(a.dob + qrow + 16 * s + 8 * g);
  }
  const float lse2 = a.lse2[(long long)(tok0 + prow) * H + hq];
  const float D = a.dsum[(long long)(tok0 + prow) * H + hq];
  const int last_row = min(R0 + ROWS - 1, rows_total - 1);
  const int n_kt = (last_row / G) / KT + 1;
  const int pw_max = Rw < rows_total ? min(Rw + 31, rows_total - 1) / G : -1;
  const float sc = kLog2e / sqrtf((float)DH);
  f32x16 dq[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dq[d] = (f32x16){};
  const bf16 *kbase = a.k + (long long)tok0 * kvd + gk * DH;
  const bf16 *vbase = a.vb + (long long)tok0 * kvd + gk * DH;
  const bf16 *ktbase = a.kt + (long long)gk * DH * a.ldt;
  auto dma = [&](int kt, bf16 *sk, bf16 *sv, bf16 *skt) {
    dma_rows(sk, kbase, kvd, kt * KT, len - 1, wave, NWV, lane);
    dma_rows(sv, vbase, kvd, kt * KT, len - 1, wave, NWV, lane);
    dma_cols(skt, ktbase, a.ldt, col0 + kt * KT, wave, NWV, lane);
  };
  auto tile = [&](int kt, const bf16 *sk, const bf16 *sv, const bf16 *skt) {
    if (kt * KT > pw_max) return;
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = (f32x16){};
      dpacc[kb] = (f32x16){};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf = *(const bf16x8 *)&sk[kidx(32 * kb + c32, 2 * s + g)];
        const bf16x8 vf = *(const bf16x8 *)&sv[kidx(32 * kb + c32, 2 * s + g)];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kb], 0, 0, 0);
        dpacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[s], dpacc[kb], 0, 0, 0);
      }
    }
    // dS = P (dP - D), P = 2^(s sc - lse2) on visible keys
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kt * KT + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
        const float p = key > prow ? 0.f : fast_exp2(__builtin_fmaf(sacc[kb][e], sc, -lse2));
        sacc[kb][e] = p * (dpacc[kb][e] - D);
      }
    // dQ^T += K^T dS^T, 16 keys per MFMA (k slot 8g+j <-> key 16h + 8(j/4) + 4g + j%4)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1, h = st & 1;
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = f2bf(sacc[kb][8 * h + j]);
      const int col = 32 * kb + 16 * h + 8 * g;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 ktf = *(const bf16x8 *)&skt[vidx(32 * d + c32, col)];
        dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktf, pf, dq[d], 0, 0, 0);
      }
    }
  };
  auto land = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  // tile kt computes from one buffer while tile kt + 1 streams into the other
  auto step = [&](int kt, const bf16 *sk, const bf16 *sv, const bf16 *skt, bf16 *nk, bf16 *nv, bf16 *nkt) {
    if (kt + 1 < n_kt) dma(kt + 1, nk, nv, nkt);
    __builtin_amdgcn_sched_barrier(0);
    tile(kt, sk, sv, skt);
    land();
  };
  dma(0, sk0, sv0, skt0);
  land();
  int kt = 0;
  for (; kt + 1 < n_kt; kt += 2) {
    step(kt, sk0, sv0, skt0, sk1, sv1, skt1);
    step(kt + 1, sk1, sv1, skt1, sk0, sv0, skt0);
  }
  if (kt < n_kt) step(kt, sk0, sv0, skt0, sk1, sv1, skt1);
  if (Rw + c32 >= rows_total) return;
  const float scale = 1.0f / sqrtf((float)DH);
  float *op = a.dq + qrow + 4 * g;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *(f32x4 *)(op + 32 * d + 8 * c) = (f32x4){dq[d][4 * c] * scale, dq[d][4 * c + 1] * scale,
                                                 dq[d][4 * c + 2] * scale, dq[d][4 * c + 3] * scale};
}

__global__ __launch_bounds__(256) void attn_bwd_dkv_kernel(AttnBwdMfmaArgs a) {
  constexpr int NWV = 4, KEYS = 32 * NWV;
  // two buffers of (Q rows, dO rows, Q^T, dO^T, lse2, D), one LDS object each
  __shared__ bf16 sq0[KT * DH], sdo0[KT * DH], sqt0[DH * KT], sdot0[DH * KT];
  __shared__ bf16 sq1[KT * DH], sdo1[KT * DH], sqt1[DH * KT], sdot1[DH * KT];
  __shared__ __attribute__((aligned(16))) float sl0[KT], sd0[KT], sl1[KT], sd1[KT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c32 = lane & 31, g = lane >> 5;
  // grid (query head, sequence, key block): the key blocks that see the
  // most rows (the first ones) are dispatched first for every head
  const int hq = blockIdx.x, b = blockIdx.y, K0 = blockIdx.z * KEYS;
  const int H = a.H, gk = hq * a.Hkv / a.H, kvd = a.Hkv * DH;
  const int tok0 = a.cu[b], len = a.cu[b + 1] - tok0;
  const long long col0 = a.cu_pad[b];
  if (K0 >= len) return;
  const int kw = K0 + 32 * wave;                 // this wave's first key
  const int key = min(kw + c32, len - 1);
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    kf[s] = *(const bf16x8 *)(a.k + (long long)(tok0 + key) * kvd + gk * DH + 16 * s + 8 * g);
    vf[s] = *(const bf16x8 *)(a.vb + (long long)(tok0 + key) * kvd + gk * DH + 16 * s + 8 * g);
  }
  const float sc = kLog2e / sqrtf((float)DH);
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dk[d] = dv[d] = (f32x16){};
  const bf16 *qbase = a.q + (long long)tok0 * H * DH + hq * DH;
  const bf16 *obase = a.dob + (long long)tok0 * H * DH + hq * DH;
  const bf16 *qtb = a.qt + (long long)hq * DH * a.ldt, *otb = a.dot + (long long)hq * DH * a.ldt;
  const int t0 = K0 / KT, t_end = (len - 1) / KT;
  // per-position lse2 and D of a tile: global loads into registers, stored
  // to LDS after the previous tile's reads
  float nl = 0.f, nd = 0.f;
  auto fetch_ld = [&](int tt) {
    if (tid < KT) {
      const int pos = min(tt * KT + tid, len - 1);
      nl = a.lse2[(long long)(tok0 + pos) * H + hq];
      nd = a.dsum[(long long)(tok0 + pos) * H + hq];
    }
  };
  auto put_ld = [&](float *sl, float *sd) {
    if (tid < KT) {
      sl[tid] = nl;
      sd[tid] = nd;
    }
  };
  auto dma = [&](int tt, bf16 *sq, bf16 *sdo, bf16 *sqt, bf16 *sdot) {
    dma_rows(sq, qbase, (long long)H * DH, tt * KT, len - 1, wave, NWV, lane);
    dma_rows(sdo, obase, (long long)H * DH, tt * KT, len - 1, wave, NWV, lane);
    dma_cols(sqt, qtb, a.ldt, col0 + tt * KT, wave, NWV, lane);
    dma_cols(sdot, otb, a.ldt, col0 + tt * KT, wave, NWV, lane);
  };
  // The wave's u-th load of tile tt (u < 16): instruction j = wave + 4 (u % 4)
  // of Q, dO, Q^T, dO^T in turn, as dma() issues them.
  static_assert(NWV == 4, "four loads of each operand per wave");
  auto dma1 = [&](int u, int tt, bf16 *sq, bf16 *sdo, bf16 *sqt, bf16 *sdot) {
    const int j = wave + NWV * (u & 3), op = u >> 2;
    if (op < 2) {
      const int row = 4 * j + (lane >> 4), pc = lane & 15;
      const int src = min(tt * KT + row, len - 1);
      const bf16 *base = op == 0 ? qbase : obase;
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(base + (long long)src * H * DH + ((pc ^ (row & 15)) << 3)),
                                       LDS_PTR(&(op == 0 ? sq : sdo)[j * 512]), 16, 0, 0);
    } else {
      const int dim = 8 * j + (lane >> 3), pc = lane & 7;
      const bf16 *base = op == 2 ? qtb : otb;
      __builtin_amdgcn_global_load_lds(
          GLOBAL_PTR(base + (long long)dim * a.ldt + col0 + tt * KT + ((pc ^ ((dim >> 1) & 7)) << 3)),
          LDS_PTR(&(op == 2 ? sqt : sdot)[j * 512]), 16, 0, 0);
    }
  };
  // One tile; load(u), u < 16, issues the wave's loads of the next tile.  With
  // one wave per SIMD, a burst of load instructions at the start of a tile
  // (each blocks the wave until the CU accepts it) would leave the matrix core
  // idle, so they go one after each pair of S^T / dP^T MFMAs.
  auto tile = [&](int tt, const bf16 *sq, const bf16 *sdo, const bf16 *sqt, const bf16 *sdot, const float *sl,
                  const float *sd, auto load) {
    // the tile reaches this wave's keys (positions >= key), and the wave has keys
    if (!(tt * KT + KT - 1 >= kw && kw < len)) {
#pragma unroll
      for (int u = 0; u < 16; ++u) load(u);
      return;
    }
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      sacc[pb] = (f32x16){};
      dpacc[pb] = (f32x16){};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 qa = *(const bf16x8 *)&sq[kidx(32 * pb + c32, 2 * s + g)];
        const bf16x8 oa = *(const bf16x8 *)&sdo[kidx(32 * pb + c32, 2 * s + g)];
        sacc[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[s], sacc[pb], 0, 0, 0);
        dpacc[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[s], dpacc[pb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load(8 * pb + s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // lane (key, g): positions 32 pb + 8 (e/4) + 4 g + e%4 of the tile; the
    // four positions of one e/4 are adjacent, so lse2 and D come 16 bytes
    // at a time
    f32x16 pp[2];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pl0 = 32 * pb + 8 * q + 4 * g;
        const f32x4 l4 = *(const f32x4 *)&sl[pl0], d4 = *(const f32x4 *)&sd[pl0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * q + i, pos = tt * KT + pl0 + i;
          const bool vis = pos >= kw + c32 && pos < len;
          const float p = vis ? fast_exp2(__builtin_fmaf(sacc[pb][e], sc, -l4[i])) : 0.f;
          pp[pb][e] = p;
          sacc[pb][e] = p * (dpacc[pb][e] - d4[i]);
        }
      }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int pb = st >> 1, h = st & 1;
      bf16x8 pf, sf;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pf[j] = f2bf(pp[pb][8 * h + j]);
        sf[j] = f2bf(sacc[pb][8 * h + j]);
      }
      const int col = 32 * pb + 16 * h + 8 * g;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 ota = *(const bf16x8 *)&sdot[vidx(32 * d + c32, col)];
        const bf16x8 qta = *(const bf16x8 *)&sqt[vidx(32 * d + c32, col)];
        dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ota, pf, dv[d], 0, 0, 0);
        dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, sf, dk[d], 0, 0, 0);
      }
    }
  };
  auto land = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto step = [&](int tt, const bf16 *sq, const bf16 *sdo, const bf16 *sqt, const bf16 *sdot, const float *sl,
                  const float *sd, bf16 *nq, bf16 *ndo, bf16 *nqt, bf16 *ndot, float *nsl, float *nsd) {
    const bool more = tt + 1 <= t_end;
    if (more) fetch_ld(tt + 1);
    __builtin_amdgcn_sched_barrier(0);
    tile(tt, sq, sdo, sqt, sdot, sl, sd, [&](int u) {
      if (more) dma1(u, tt + 1, nq, ndo, nqt, ndot);
    });
    if (more) put_ld(nsl, nsd);
    land();
  };
  dma(t0, sq0, sdo0, sqt0, sdot0);
  fetch_ld(t0);
  put_ld(sl0, sd0);
  land();
  int tt = t0;
  for (; tt + 1 <= t_end; tt += 2) {
    step(tt, sq0, sdo0, sqt0, sdot0, sl0, sd0, sq1, sdo1, sqt1, sdot1, sl1, sd1);
    step(tt + 1, sq1, sdo1, sqt1, sdot1, sl1, sd1, sq0, sdo0, sqt0, sdot0, sl0, sd0);
  }
  if (tt <= t_end) step(tt, sq0, sdo0, sqt0, sdot0, sl0, sd0, sq1, sdo1, sqt1, sdot1, sl1, sd1);
  if (kw + c32 >= len) return;
  const float scale = 1.0f / sqrtf((float)DH);
  const long long orow = ((long long)hq * a.M + tok0 + kw + c32) * DH + 4 * g;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      *(f32x4 *)(a.dkp + orow + 32 * d + 8 * c) = (f32x4){dk[d][4 * c] * scale, dk[d][4 * c + 1] * scale,
                                                          dk[d][4 * c + 2] * scale, dk[d][4 * c + 3] * scale};
      *(f32x4 *)(a.dvp + orow + 32 * d + 8 * c) =
          (f32x4){dv[d][4 * c], dv[d][4 * c + 1], dv[d][4 * c + 2], dv[d][4 * c + 3]};
    }
}

// D[m][h] = dO[m][h] . O[m][h] (fp32 dO, bf16 O); 16 lanes per (row, head)
__global__ __launch_bounds__(256) void attn_bwd_dsum_kernel(const float *dout, const bf16 *o, int M, int H,
                                                            float *dsum) {
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const long long item = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  if (item >= (long long)M * H) return;
  const float *dp = dout + item * DH + 8 * l16;
  const bf16x8 ov = *(const bf16x8 *)(o + item * DH + 8 * l16);
  const f32x4 d0 = *(const f32x4 *)dp, d1 = *(const f32x4 *)(dp + 4);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) sum += d0[i] * bf2f(ov[i]) + d1[i] * bf2f(ov[4 + i]);
  sum += __shfl_xor(sum, 1, 64);
  sum += __shfl_xor(sum, 2, 64);
  sum += __shfl_xor(sum, 4, 64);
  sum += __shfl_xor(sum, 8, 64);
  if (l16 == 0) dsum[item] = sum;
}

// dst[c][vcol[m]] = src[m][c] (bf16): the V^T-like layout of a row operand.
// 64 x 64 tiles through LDS: 16-byte reads along rows; the writes of a
// wave cover 64 consecutive rows, whose columns vcol[m] are consecutive up
// to the vperm16 order within 16.  C % 64 == 0.
__global__ __launch_bounds__(256) void transpose_cols_kernel(const bf16 *src, long long lds, int M, const int *vcol,
                                                             bf16 *dst, long long ldt) {
  constexpr int P = 66;
  __shared__ bf16 t[64 * P];
  const int m0 = blockIdx.y * 64, c0 = blockIdx.x * 64, tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + 256 * k, row = i >> 3, ch = i & 7, m = m0 + row;
    if (m < M) {
      const bf16x8 x = *(const bf16x8 *)(src + (long long)m * lds + c0 + 8 * ch);
#pragma unroll
      for (int e = 0; e < 8; ++e) t[row * P + 8 * ch + e] = x[e];
    }
  }
  __syncthreads();
  const int row = tid & 63, m = m0 + row;
  if (m >= M) return;
  const long long col = vcol[m];
  for (int c = tid >> 6; c < 64; c += 4) dst[(long long)(c0 + c) * ldt + col] = t[row * P + c];
}

// dk[m][g dh + d] = sum over the group's query heads h of dkp[h][m][d] (in order)
__global__ __launch_bounds__(256) void sum_heads_kernel(const float *part, int M, int H, int Hkv, float *out) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long n = (long long)M * Hkv * DH;
  if (i >= n) return;
  const int m = (int)(i / (Hkv * DH)), gd = (int)(i - (long long)m * Hkv * DH), gg = gd / DH, d = gd - gg * DH;
  const int G = H / Hkv;
  float acc = 0.f;
  for (int h = gg * G; h < gg * G + G; ++h) acc += part[((long long)h * M + m) * DH + d];
  out[i] = acc;
}

// ------------------------------------------------------------------ decode

// Page staging in LDS.  K [64 keys][128 dims]: 16-byte chunk c of key r at
// slot c ^ (r % 16), so the 16 keys of a fragment read hit 16 bank groups.
// V^T [128 dims][64 keys]: 16-byte chunk c of dim r at slot c ^ ((r / 2) % 8);
// fragments read it in 8-byte units.
DEV int kdx(int key, int chunk) { return key * DH + ((chunk ^ (key & 15)) << 3); }
DEV int vdx(int dim, int unit) { return dim * 64 + (((unit >> 1) ^ ((dim >> 1) & 7)) << 3) + ((unit & 1) << 2); }

// A wave-uniform int through the scalar cache.  Block-table entries read
// this way do not occupy the vector-memory counter, so waiting for them does
// not also wait for the slab loads in flight.
DEV int sload(const int *p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// The query of the new position: every workgroup builds its group's query
// heads into LDS (sum of the split-GEMM slabs, RoPE, QK-norm, bf16), head slots spread
// over the half-waves of all its waves.  The chunk holding the new position
// also builds its k and v, stores them to the cache for later steps, and the
// wave whose page holds that position patches them into its copy of the page
// (which it may have read before or after the store).
//
// One workgroup per chunk of a.chunk_pages pages of one sequence and K/V
// head (grid z).  Wave w takes pages w, w + NP, ... of the chunk (at most R
// rounds) and scores
// their 64 cached positions for all query heads that share the K/V head at
// once (the H / Hkv heads of its group; under MQA every head).  "Heads" below
// are the group's.  Each page (K and V^T, 32 KB) is copied into the wave's
// LDS area with direct-to-LDS loads that read whole 128-byte lines, and the
// MFMA fragments are read from there (128 KB of LDS for 4 waves, one
// workgroup per CU); the next round's page is staged as soon as this round's
// fragments are in registers.  Online softmax over the rounds.  The pages of
// a chunk are merged in LDS by log-sum-exp, and the chunk's unnormalised
// output with its (max, sum) per head goes to the partial buffers.  The last
// chunk of the sequence to finish merges all chunks and writes o.
template <int NP, int R>
__global__ __launch_bounds__(64 * NP) void attn_decode_kernel(AttnDecodeArgs a) {
  constexpr int NT = 64 * NP;
  // VREG: eight waves, each staging only its K page in LDS and loading its
  // V^T fragments straight into registers (128 KB of LDS holds eight K pages
  // but only four K + V^T pairs), so a chunk of up to 8 pages lands in one
  // round.
  constexpr bool VREG = NP == 8;
  static_assert(NP == 4 || NP == 8, "four waves (K and V^T staged) or eight (K staged)");
  const int CH = 64 * a.chunk_pages;  // cached positions per chunk (at most 64 NP R)
  // per wave a K page (and, four waves, a V^T page); the wave's partial
  // output (16 heads x 128 fp32) later reuses the first 8 KB
  constexpr int WAVE_BYTES = (VREG ? 1 : 2) * 64 * DH * 2;
  constexpr int QS = DH + 8;  // q row pitch: the 16 heads of a fragment read start on different banks
  __shared__ __attribute__((aligned(16))) char smem[NP * WAVE_BYTES];
  __shared__ float ml_s[NP][16][2];  // per-page (max, sum) per head
  __shared__ __attribute__((aligned(16))) bf16 q_s[16 * QS];
  __shared__ __attribute__((aligned(16))) bf16 kv_s[2 * DH];  // the new position's k and v
  auto wave_area = [&](int w) { return smem + w * WAVE_BYTES; };
  __shared__ unsigned s_prev;
  // wave index as a scalar, so per-wave addresses and the block-table
  // lookups are scalar and only the slab and page loads use the vector
  // memory counter
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hl = lane & 15, q4 = lane >> 4;
  // this workgroup's chunk from the step's work list (consecutive workgroups
  // go to different XCDs, so the chunks spread evenly over them)
  const int *wk = a.map + kDecodeMapStride * blockIdx.x;
  const int b = wk[0], chunk = wk[1];
  if (b >= a.n) return;  // only a list out of step with the lengths holds one
  const ScatterArgs &in = a.in;
  const PagedKV &kv = in.kv;
  // K/V head gk and its G query heads hq0 .. hq0 + G - 1
  const int Hall = in.H, Hkv = in.Hkv, G = Hall / Hkv, gk = blockIdx.z, hq0 = gk * G;
  const int kvd = Hkv * DH;  // row width of a K page
  const int len = wk[2];  // positions 0 .. lens[b], the last one new
  // The work list also holds this wave's first page (the block-table entry
  // clamped to the table's row; one past the chunk is not used), so the page
  // copy starts after one round trip.
  const int page0 = wk[4 + wave];
  const int pn = len - 1;
  const int c0 = chunk * CH;
  const int cend = min(c0 + CH, len);             // end of this chunk's positions
  const int H = G;
  const int kpos0 = c0 + wave * 64;               // this wave's first page
  const int nw = min(NP, (cend - c0 + 63) / 64);  // waves with a page
  const bool owner = pn < c0 + CH;                // the chunk holds the new position
  const int nslot = H + (owner ? 2 : 0);
  // Slots are built by half-waves: lane li of half hw holds dims 4 li ..
  // 4 li + 3 of one slot, so each slab costs one 16-byte load per lane for
  // two slots.  Half-wave hh = 2 wave + hw builds slots hh, hh + 2 NP, ...
  // Slot j < H: query head hq0 + j into q_s.  j = H: k, j = H + 1: v of K/V
  // head gk at the new position, into kv_s and the cache.  The slab loads
  // follow the page loads: the compiler waits for every load in flight
  // before the slabs are summed, so issuing them first would only delay the
  // page loads.
  const int li = lane & 31, hw = lane >> 5, hh = 2 * wave + hw;
  const float *u = in.qkv + (long long)b * (Hall + 2 * Hkv) * DH;
  const int st = (int)in.slab;  // slabs of at most 64 rows: far below 2^31 floats
  f32x4 t[kMaxRowSplit];
  auto load_slot = [&](int j) {
    // slab column of the slot: query head hq0 + j, K head gk, V head gk
    const int col = j < H ? hq0 + j : (j == H ? Hall + gk : Hall + Hkv + gk);
    const float *uj = u + col * DH + 4 * li;
#pragma unroll
    for (int k = 0; k < kMaxRowSplit; ++k)
      if (k == 0 || k < in.nslab) t[k] = *(const f32x4 *)(uj + k * st);
  };
  f32x4 c4 = {}, s4 = {};
  if (in.cos && hh < nslot) {
    c4 = *(const f32x4 *)(in.cos + pn * 64 + 4 * (li & 15));
    s4 = *(const f32x4 *)(in.sin + pn * 64 + 4 * (li & 15));
  }
  bf16 *Ks = (bf16 *)wave_area(wave), *Vs = Ks + 64 * DH;
  // cache page `page` of this layer
  auto page_ptr = [&](int page) {
    return (const char *)kv.base + (long long)in.layer * kv.layer_stride + (long long)page * kv.page_stride;
  };
  // 32 wave instructions of 1 KB: K as 4 keys x 256 B each, V^T as 8 dims x
  // 128 B each; lane i fills slot i of the instruction's kilobyte and so
  // loads the logical chunk that slot holds.
  auto stage_page = [&](int page) {
    const char *pg = page_ptr(page);
    const bf16 *K = (const bf16 *)pg + gk * DH;                      // rows of kvd
    const bf16 *Vt = (const bf16 *)(pg + kv.half_bytes) + gk * DH * 64;  // [128][64]
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = 4 * j + (lane >> 4), pc = lane & 15;
      __builtin_amdgcn_global_load_lds(GLOBAL_PTR(K + key * kvd + ((pc ^ (key & 15)) << 3)),
                                       LDS_PTR(Ks + j * 512), 16, 0, 0);
    }
    if constexpr (!VREG)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int dim = 8 * j + (lane >> 3), pc = lane & 7;
        __builtin_amdgcn_global_load_lds(GLOBAL_PTR(Vt + dim * 64 + ((pc ^ ((dim >> 1) & 7)) << 3)),
                                         LDS_PTR(Vs + j * 512), 16, 0, 0);
      }
  };
  // VREG: the V^T fragments of a page straight from the cache, in the layout
  // the four-wave kernel reads them from LDS: dims 16 d + hl, the eight
  // stored key columns 8 (4 h + q4) .. +8 (two sets for two rounds)
  bf16x8 vreg[VREG && R > 1 ? 2 : 1][8][2];
  auto load_v = [&](int page, bf16x8 (&vr)[8][2]) __attribute__((always_inline)) {
    const bf16 *Vt = (const bf16 *)(page_ptr(page) + kv.half_bytes) + gk * DH * 64;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int h = 0; h < 2; ++h) vr[d][h] = *(const bf16x8 *)(Vt + (16 * d + hl) * 64 + 8 * (4 * h + q4));
  };
  if (kpos0 < cend) {
    stage_page(page0);
    if constexpr (VREG) load_v(page0, vreg[0]);
  }
  {
    // Query heads and k: half-split rotation (dim i pairs with i + 64, held
    // by lane li ^ 16), then a weightless RMSNorm over the head.
    const int npage = owner ? sload(kv.table + b * kv.pages_per_seq + pn / kv.page_size) : 0;
    char *npg = kv.base + (long long)in.layer * kv.layer_stride + (long long)npage * kv.page_stride;
    const int nsl = pn % kv.page_size;
    for (int j = hh; j < nslot; j += 2 * NP) {
      load_slot(j);
      f32x4 x = t[0];
#pragma unroll
      for (int k = 1; k < kMaxRowSplit; ++k)
        if (k < in.nslab) x += t[k];
      if (j < H + 1) {
        if (in.cos) {
          f32x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = __shfl_xor(x[e], 16, 64);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = li < 16 ? x[e] * c4[e] - y[e] * s4[e] : y[e] * s4[e] + x[e] * c4[e];
        }
        if (in.qk_norm) {
          float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) ss += __shfl_xor(ss, o, 64);
          const float rs = 1.0f / sqrtf(ss * (1.0f / 128.0f) + in.eps);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] *= rs;
        }
      }
      const bf16x4 y4 = {f2bf(x[0]), f2bf(x[1]), f2bf(x[2]), f2bf(x[3])};
      if (j < H) {
        *(bf16x4 *)&q_s[j * QS + 4 * li] = y4;
      } else {
        *(bf16x4 *)&kv_s[(j - H) * DH + 4 * li] = y4;
        if (j == H) {
          *(bf16x4 *)((bf16 *)npg + nsl * kvd + gk * DH + 4 * li) = y4;
        } else {
          bf16 *vt = (bf16 *)(npg + kv.half_bytes);
#pragma unroll
          for (int e = 0; e < 4; ++e) vt[(gk * DH + 4 * li + e) * kv.page_size + vslot(nsl)] = y4[e];
        }
      }
    }
  }
  // q_s and kv_s complete (a bare barrier: the page loads stay in flight)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (kpos0 < cend) {
    bf16x8 qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (hl < H) qf[s] = *(const bf16x8 *)&q_s[hl * QS + 32 * s + 8 * q4];
      else qf[s] = (bf16x8){};
    }
    // Round r: page w + r NP of the chunk.  The next round's page is staged
    // into the same LDS area once this round's fragments are in registers,
    // so it lands while this round computes.  Online softmax over the
    // rounds: running max mx, sum rs and O^T.
    float mx = -INFINITY, rs = 0.f;
    f32x4 oacc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) oacc[d] = (f32x4){};
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int kp = kpos0 + r * NP * 64;
      if (kp >= cend) break;
      const int nkey = pn - kp;  // the new position's slot in this page, if it holds it
      const bool pw = nkey >= 0 && nkey < 64;
      bf16x8 kf[4][4];
      // V^T: dims 16 d + hl, the eight keys of k slots 8 q4 .. of half h
      // (four waves: read from LDS below)
      bf16x8 (&vf)[8][2] = vreg[VREG && R > 1 ? (r & 1) : 0];
      {
        // this round's page has landed (each wave reads only its own area)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (pw) {
          Ks[kdx(nkey, lane >> 3) + (lane & 7)] = kv_s[lane];
          Ks[kdx(nkey, (lane + 64) >> 3) + (lane & 7)] = kv_s[lane + 64];
          const int cc = vslot(nkey);
          if constexpr (VREG) {
            // the stored column cc is element cc % 8 of vf[.][cc / 32] in the
            // lanes of q4 = (cc / 8) % 4
            if (q4 == ((cc >> 3) & 3)) {
              const int hn = cc >> 5, jn = cc & 7;
#pragma unroll
              for (int d = 0; d < 8; ++d) {
                const bf16 v = kv_s[DH + 16 * d + hl];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                  for (int j = 0; j < 8; ++j)
                    if (h == hn && j == jn) vf[d][h][j] = v;
              }
            }
          } else {
            Vs[vdx(lane, cc >> 2) + (cc & 3)] = kv_s[DH + lane];
            Vs[vdx(lane + 64, cc >> 2) + (cc & 3)] = kv_s[DH + lane + 64];
          }
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int s = 0; s < 4; ++s) kf[kb][s] = *(const bf16x8 *)&Ks[kdx(16 * kb + hl, 4 * s + q4)];
        if constexpr (!VREG)
#pragma unroll
          for (int d = 0; d < 8; ++d)
#pragma unroll
            for (int h = 0; h < 2; ++h) vf[d][h] = *(const bf16x8 *)&Vs[vdx(16 * d + hl, 2 * (4 * h + q4))];
        if (r + 1 < R && kp + NP * 64 < cend) {
          // the fragment reads (and the patch) have completed: the area is free
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          const int npg = sload(kv.table + b * kv.pages_per_seq + (kp + NP * 64) / kv.page_size);
          stage_page(npg);
          if constexpr (VREG) load_v(npg, vreg[(r + 1) & 1]);
        }
      }
      // S^T[key][head] = K Q^T: lane holds head hl, keys 16 kb + 4 q4 + r
      f32x4 sacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sacc[kb] = (f32x4){};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][s], qf[s], sacc[kb], 0, 0, 0);
      }
      const float sc = kLog2e / sqrtf((float)DH);
      float pm = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kp + 16 * kb + 4 * q4 + e;
          const float v = key < len ? sacc[kb][e] * sc : -INFINITY;
          sacc[kb][e] = v;
          pm = fmaxf(pm, v);
        }
      pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
      pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
      const float mn = fmaxf(mx, pm);
      const float scale = fast_exp2(mx - mn);  // 0 in the first round (mx = -inf)
      mx = mn;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(sacc[kb][e] - mn);
          sacc[kb][e] = p;
          ps += p;
        }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      rs = rs * scale + ps;
#pragma unroll
      for (int d = 0; d < 8; ++d) oacc[d] *= scale;
      // positions past the end hold stale data: zero them so 0 * garbage cannot appear
      if (kp + 64 > len) {
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (kp + 32 * h + 16 * (j >> 2) + 4 * q4 + (j & 3) >= len) vf[d][h][j] = (bf16)0.f;
      }
      // O^T += V^T P^T; k slot 8 q4 + j <-> key 32 h + 16 (j/4) + 4 q4 + j%4
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[e] = f2bf(sacc[2 * h][e]);
          pf[4 + e] = f2bf(sacc[2 * h + 1][e]);
        }
#pragma unroll
        for (int d = 0; d < 8; ++d) oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d][h], pf, oacc[d], 0, 0, 0);
      }
    }
    if (hl < H) {
      // lane holds head hl, dims 16 d + 4 q4 + r; the partial overwrites
      // this wave's K staging area, whose reads the MFMAs above have
      // consumed
      float *o_w = (float *)wave_area(wave);
#pragma unroll
      for (int d = 0; d < 8; ++d) *(f32x4 *)&o_w[hl * DH + 16 * d + 4 * q4] = oacc[d];
      if (q4 == 0) {
        ml_s[wave][hl][0] = mx;
        ml_s[wave][hl][1] = rs;
      }
    }
  }
  __syncthreads();
  const int S = (len + CH - 1) / CH;   // chunks of this sequence
  const long long obase = (((long long)b * a.max_splits + chunk) * Hall + hq0) * DH;
  // Merge the pages: each thread takes 4 consecutive dims of one head.
  for (int i4 = tid; i4 < H * DH / 4; i4 += NT) {
    const int idx = 4 * i4, h = idx >> 7;
    float M = ml_s[0][h][0];
    for (int w = 1; w < nw; ++w) M = fmaxf(M, ml_s[w][h][0]);
    float L = 0.f;
    f32x4 O = {};
    for (int w = 0; w < nw; ++w) {
      const float f = fast_exp2(ml_s[w][h][0] - M);
      L += f * ml_s[w][h][1];
      O += f * *(const f32x4 *)((const float *)wave_area(w) + idx);
    }
    if (S == 1) {
      *(bf16x4 *)&a.o[((long long)b * Hall + hq0) * DH + idx] =
          (bf16x4){f2bf(O[0] / L), f2bf(O[1] / L), f2bf(O[2] / L), f2bf(O[3] / L)};
    } else {
      xst4(a.o_part + obase + idx, O);
      if ((idx & (DH - 1)) == 0) {
        float *ml = a.ml_part + (((long long)b * a.max_splits + chunk) * Hall + hq0 + h) * 2;
        xst(ml, M);
        xst(ml + 1, L);
      }
    }
  }
  if (S == 1) return;
  // Publish the chunk: its partials travel through sc1 stores and loads and
  // it is counted once they have completed.  The counter resets itself for
  // the next layer.
  stores_done();
  __syncthreads();
  if (tid == 0) s_prev = arrive(&a.ctr[b * Hkv + gk]);
  __syncthreads();
  if (s_prev != (unsigned)(S - 1)) return;
  if (tid == 0) a.ctr[b * Hkv + gk] = 0u;
  // Final merge over the S chunks, 4 dims of one head per thread: the
  // (max, sum) and partial output of up to 8 chunks are loaded at once, then
  // folded into a running (max, sum, output).
  const float *ob = a.o_part + ((long long)b * a.max_splits * Hall + hq0) * DH;
  const float *mb = a.ml_part + ((long long)b * a.max_splits * Hall + hq0) * 2;
  for (int i4 = tid; i4 < H * DH / 4; i4 += NT) {
    const int idx = 4 * i4, h = idx >> 7;
    float M = -INFINITY, L = 0.f;
    f32x4 O = {};
    for (int cg = 0; cg < S; cg += 8) {
      float m[8], l[8];
      f32x4 v[8];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        if (cg + cc < S) {
          const long long c = cg + cc;
          m[cc] = xld(mb + (c * Hall + h) * 2);
          l[cc] = xld(mb + (c * Hall + h) * 2 + 1);
          v[cc] = xld4(ob + c * Hall * DH + idx);
        }
      float Mg = M;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        if (cg + cc < S) Mg = fmaxf(Mg, m[cc]);
      const float r = fast_exp2(M - Mg);  // 0 on the first group (M = -inf)
      L *= r;
      O *= r;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        if (cg + cc < S) {
          const float f = fast_exp2(m[cc] - Mg);
          L += f * l[cc];
          O += f * v[cc];
        }
      M = Mg;
    }
    *(bf16x4 *)&a.o[((long long)b * Hall + hq0) * DH + idx] =
        (bf16x4){f2bf(O[0] / L), f2bf(O[1] / L), f2bf(O[2] / L), f2bf(O[3] / L)};
  }
}

}  // namespace

void launch_attn_prefill_bf16(const AttnPrefillArgs &a, hipStream_t s) {
  if (a.n_seqs <= 0 || a.max_wg <= 0) return;
  const dim3 grid(a.n_seqs, a.max_wg, a.Hkv);
  constexpr int NWV = kAttnPrefillWaves, RB = kAttnPrefillRows / (32 * kAttnPrefillWaves);
  if (a.qk_norm) attn_prefill_kernel<NWV, RB, true><<<grid, 64 * NWV, 0, s>>>(a);
  else attn_prefill_kernel<NWV, RB, false><<<grid, 64 * NWV, 0, s>>>(a);
}

void launch_attn_bwd_mfma(const AttnBwdMfmaArgs &a, const float *dout, const bf16 *o, float *dk, float *dv,
                          hipStream_t s) {
  if (a.n_seqs <= 0 || a.M <= 0) return;
  const long long items = (long long)a.M * a.H;
  attn_bwd_dsum_kernel<<<(unsigned)((items + 15) / 16), 256, 0, s>>>(dout, o, a.M, a.H, a.dsum);
  attn_bwd_dq_kernel<<<dim3(a.n_seqs, a.max_wg, a.Hkv), 512, 0, s>>>(a);
  attn_bwd_dkv_kernel<<<dim3(a.H, a.n_seqs, (a.max_len + 127) / 128), 256, 0, s>>>(a);
  const long long n = (long long)a.M * a.Hkv * DH;
  sum_heads_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.dkp, a.M, a.H, a.Hkv, dk);
  sum_heads_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.dvp, a.M, a.H, a.Hkv, dv);
}

void launch_transpose_cols(const bf16 *src, long long lds, int M, int C, const int *vcol, bf16 *dst, long long ldt,
                           hipStream_t s) {
  if (M <= 0 || C <= 0) return;
  transpose_cols_kernel<<<dim3(C / 64, (M + 63) / 64), 256, 0, s>>>(src, lds, M, vcol, dst, ldt);
}

// One workgroup: each thread takes sequences t, t + 256, ...; a block-wide
// exclusive scan of their chunk counts gives each sequence's first entry.
void launch_attn_decode_bf16(const AttnDecodeArgs &a, hipStream_t s) {
  if (a.n <= 0 || a.work <= 0) return;
  // a.chunk_pages pages per workgroup: up to 4 on four waves, 5 to 8 on
  // eight (one round), 9 to 16 on eight in two rounds
  const dim3 grid(a.work, 1, a.in.Hkv);
  if (a.chunk_pages <= 4) attn_decode_kernel<4, 1><<<grid, 256, 0, s>>>(a);
  else if (a.chunk_pages <= 8) attn_decode_kernel<8, 1><<<grid, 512, 0, s>>>(a);
  else attn_decode_kernel<8, 2><<<grid, 512, 0, s>>>(a);
}
