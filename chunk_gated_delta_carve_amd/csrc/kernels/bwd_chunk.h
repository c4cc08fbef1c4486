// Chunk-parallel backward pass without a content projection (bf16 inputs,
// d_k = d_v = 64). Without a projection the chunk length L only decides which
// tokens d_mean_out reaches, so the work is cut into 64-token blocks whatever
// L is; "chunk" below means such a block. One workgroup per (batch, head,
// chunk) forms every gradient of the chunk's tokens at once, from the state S
// at the chunk start (written by the forward pair), the state gradient dS_L
// at the chunk end and the chunk's inputs, as 16x16 products on the matrix
// cores.
// The state gradients come from a chain over chunks run by the forward's own
// state pass (carve_state_kernel with checkpoints) on images that
// carve_bwd_image_kernel derives from the forward pair's: the adjoint of
// S <- S M + C, O = Q_eff S^T + O_loc is
//   dS_start = dS_end M^T + dO^T Q_eff,
// which is the state pass's S^T <- M^T S^T + C^T with M^T replaced by M and
// C^T by (dO^T Q_eff)^T, walked from the last chunk to the first.
//
// The pages train the layer but give no backward pass (gist.science technical
// summaries, §2 and §3); the forward these derivatives belong to is the WY
// block form of the key-axis recurrence (§2.1 erase gate, §2.2 write gate,
// §2.3 key-axis decay). Inside a chunk, with G_i the inclusive cumulative
// log-decay (G_{-1} = 0), E(a, b) = e^{a - b} per key channel, and
// u_i = w_i v_i - S_{i-1} D_i (b_i k_i) (the rows of Delta):
//   A_ij = sum_c b_i k_i k_j E(G_i, G_j),  P_ij = sum_c q_i k_j E(G_{i-1}, G_j)   (j < i)
//   Delta = (I + A)^{-1} (W V - Kb S^T),   Kb_i = b_i k_i e^{G_i}
// The gradient du_i = dS_i k_i of every u_i solves the transposed system
//   dU = (I + A)^{-T} (P^T dO + Kdec dS_L^T),   Kdec_i = k_i e^{G_L - G_i},
// and with Z_ij = do_i . u_j and N_ij = du_i . u_j:
//   dq_i = e^{G_{i-1}} (dO S)_i + sum_{j<i} Z_ij k_j E(G_{i-1}, G_j)
//   x_i  = e^{G_i} (dU S)_i + sum_{j<i} N_ij k_j E(G_i, G_j)          (x_i = X_i^T du_i, X_i = S_{i-1} D_i)
//   dk_i = e^{G_L - G_i} (Delta dS_L)_i + sum_{j>i} Z_ji q_j E(G_{j-1}, G_i)
//          - sum_{j>i} N_ji b_j k_j E(G_j, G_i) - b_i x_i
//   db_i = -k_i x_i,  dv_i = w_i du_i,  dw_i = v_i . du_i.
// The decay gradient needs no per-token state: H_i = diag(S_i^T dS_i) obeys
// H_{i-1} = H_i + phi_i with phi_i = q_i dq_i - k_i dk_i + 2 b_i db_i, and
// dg_i = H_{i-1} - q_i dq_i, so
//   dg_i = H_L + sum_{j>=i} phi_j - q_i dq_i,
//   H_L  = e^{G_L} diag(S^T dS_L) + sum_i Kdec_i (Delta dS_L)_i.
// Chunk 0 also returns d_state_in = dS_L diag(e^{G_L}) + dO^T Qd - dU^T Kb,
// Qd_i = q_i e^{G_{i-1}}.
//
// Decay factors use the 16-row sub-blocks of the forward (Gs_I: G before
// sub-block I, Ge_I: G at its end): for sub-blocks I > J,
// E(G_a, G_j) = E(G_a, Gs_I) E(Gs_I, Ge_J) E(Ge_J, G_j), every factor <= 1;
// the middle factor scales a reduction index (Grams) or an output column
// (token sums). Diagonal sub-blocks use E(Gs_I, Ge_I) <= 2^kSpanLimit2 on
// top; a sub-block whose decay is steeper takes its diagonal terms pairwise,
// from the raw inputs (slow, exact).
//
// Work split: eight waves, two per 16-row block I: both form the 16x16 tiles
// that feed rows 16I..16I+15, and each takes half of the d output columns.
// LDS holds the bf16 operands (BKl_i = b_i k_i E(G_i, Gs_I), Ql_i = q_i E(G_{i-1}, Gs_I),
// Kr_j = k_j E(Ge_J, G_j), W V, dO, S, dS_L, Delta and dU), G in fp32 and
// the factor tables.
#pragma once

#include "block.h"
#include "bwd.h"

namespace carve {

template <int D>
struct ChunkBwdLayout {
  static_assert(D == 64, "the chunk-parallel backward is built for d = 64");
  static constexpr int L = 64, LD = 72, GLD = 68;                // bf16 / fp32 row strides
  static constexpr int NWV = 8, NT = 64 * NWV;                    // two waves per 16-row block
  static constexpr int MB = L * LD * 2;                           // one bf16 [64][LD] matrix
  static constexpr int oBKl = 0, oQl = MB, oKr = 2 * MB, oWV = 3 * MB, odO = 4 * MB, oS = 5 * MB,
                       odS = 6 * MB, oDel = 7 * MB;
  static constexpr int oG = 8 * MB;                               // fp32 [L][GLD]: G in log2 units
  static constexpr int oGs = oG + L * GLD * 4;                    // fp32 [4][D]
  static constexpr int oGe = oGs + 4 * D * 4;                     // fp32 [4][D]
  static constexpr int oMid = oGe + 4 * D * 4;                    // fp32 [4][4][D]
  static constexpr int oDec = oMid + 16 * D * 4;                  // fp32 [4][D]: 2^{G_L - Ge_I}
  static constexpr int oEg = oDec + 4 * D * 4;                    // fp32 [4][D]: 2^{Gs_I}
  static constexpr int oAd = oEg + 4 * D * 4;                     // fp32 [4][16][16]: diagonal tiles of A
  static constexpr int oTd = oAd + 4 * 256 * 4;                   // fp32 [4][16][16]: their inverses
  static constexpr int oRed = oTd + 4 * 256 * 4;                  // fp32 [20][D]: column partial sums
  static constexpr int oScr = oRed + 20 * D * 4;                  // bf16 [NWV][4][16][16]
  static constexpr int oDw = oScr + NWV * 4 * 256 * 2;            // fp32 [NWV][16]: dw partials
  static constexpr int oFlag = oDw + NWV * 16 * 4;                // int [4]: steep sub-blocks
  static constexpr int oVec = oFlag + 16;                         // fp32 [5][64]: the content schedule's vectors
  static constexpr int oU = oVec + 5 * 64 * 4;                    // bf16 U_down [r][D], U_up [D][r] (r <= 64)
  static constexpr int bytes = oU + 2 * 64 * D * 2;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// What one chunk's gradients are formed from, and what else they return.
struct ChunkIO {
  const float* S0;    // fp32 [dv][dk] state at the chunk start
  const float* dSL;   // fp32 [dv][dk] state gradient at the chunk end (nullptr: zeros)
  const float* z;     // content bias of the chunk's erase gate [dk] (nullptr: none)
  const float* dml;   // per value channel, added to the output gradients of tokens >= dml_from (nullptr: none)
  int dml_from;
  float* dS0;         // the state gradient at the chunk start [dv][dk] (nullptr: not formed)
  float* dz;          // LDS [dk]: the chunk's sum of dbx over its tokens (nullptr: not formed)
  // with q, k normalisation (kNorm): every token's inverse norms of q and k
  // (2 t, 2 t + 1), and where the fp32 gradients of the normalised q and k
  // go ([t][dk]) for carve_bwd_norm_kernel
  const float* nrm;
  float* dqh;
  float* dkh;
};

// kLogits: g holds raw decay logits a (g = -softplus(a)); dg is then the
// gradient of a, dg_g (-sigmoid(a)). kNorm: q and k are used over their L2
// norms, and dq, dk are left as gradients of the normalised q and k. Called
// by all threads of a 512-thread workgroup; ends with the gradient stores
// (no barrier after).
template <int D, bool kLogits, bool kNorm>
__device__ __forceinline__ void chunk_body(const BwdArgs& a, unsigned char* smem, const int bh, const int ch,
                                           const ChunkIO& io) {
  using LY = ChunkBwdLayout<D>;
  constexpr int L = LY::L, LD = LY::LD, GLD = LY::GLD, NT = LY::NT;
  static_assert(NT == 512, "eight waves: two per 16-row block, two column tiles each");
  constexpr size_t DD = (size_t)D * D;
  typedef bf16x4 b4;
  typedef Mma16<bf16> MB;
  typedef Mma16<float> MF;
  bf16* BKl = reinterpret_cast<bf16*>(smem + LY::oBKl);
  bf16* Ql = reinterpret_cast<bf16*>(smem + LY::oQl);
  bf16* Kr = reinterpret_cast<bf16*>(smem + LY::oKr);
  bf16* WV = reinterpret_cast<bf16*>(smem + LY::oWV);
  bf16* dU = WV;                                                  // W V is dead once R is formed
  bf16* dO = reinterpret_cast<bf16*>(smem + LY::odO);
  bf16* Sm = reinterpret_cast<bf16*>(smem + LY::oS);
  bf16* dSm = reinterpret_cast<bf16*>(smem + LY::odS);
  bf16* Del = reinterpret_cast<bf16*>(smem + LY::oDel);
  float* Gf = reinterpret_cast<float*>(smem + LY::oG);
  float* Gs = reinterpret_cast<float*>(smem + LY::oGs);
  float* Ge = reinterpret_cast<float*>(smem + LY::oGe);
  float* Mid = reinterpret_cast<float*>(smem + LY::oMid);
  float* Dec = reinterpret_cast<float*>(smem + LY::oDec);
  float* Eg = reinterpret_cast<float*>(smem + LY::oEg);
  float* Ad = reinterpret_cast<float*>(smem + LY::oAd);
  float* Td = reinterpret_cast<float*>(smem + LY::oTd);
  float* Red = reinterpret_cast<float*>(smem + LY::oRed);
  bf16* Scr = reinterpret_cast<bf16*>(smem + LY::oScr);
  float* Dwp = reinterpret_cast<float*>(smem + LY::oDw);
  int* Flag = reinterpret_cast<int*>(smem + LY::oFlag);

  // wave w: rows 16 I .. 16 I + 15 (I = w / 2) of every L x d result, column
  // tiles 2 hc and 2 hc + 1 (hc = w % 2). The thread index is read through an
  // empty asm statement so that a caller's chunk loop cannot hoist the
  // per-lane addresses derived from it (they would hold registers across
  // the whole loop).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, w = wave_id(), I = w >> 1, hc = w & 1;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int T = a.T, H = a.H, bi = bh / H, h = bh % H;
  const int t0 = ch * L, n = min(L, T - t0);
  const float* Sg = io.S0;
  const float* dSg = io.dSL;
  auto zb = [&](int cc) { return io.z ? io.z[cc] : 0.f; };     // content bias of key channel cc
  // inverse norms of q (0) and k (1) of chunk row `row` (1 without kNorm)
  auto nrm = [&](int row, int which) { return kNorm ? io.nrm[2 * (size_t)(t0 + row) + which] : 1.f; };
  const bf16* Q = static_cast<const bf16*>(a.q);
  const bf16* K = static_cast<const bf16*>(a.k);
  const bf16* V = static_cast<const bf16*>(a.v);
  const bf16* Gin = static_cast<const bf16*>(a.g);
  const bf16* BX = static_cast<const bf16*>(a.bx);
  const bf16* W = static_cast<const bf16*>(a.w);
  const bf16* DOg = static_cast<const bf16*>(a.d_o);
  auto tok = [&](int t) { return ((size_t)bi * T + t) * H + h; };

  // ------------------------------------------------------------------ staging
  // thread (row r, channels cs .. cs + 7) for the token inputs; rows past
  // the chunk's tokens stay zero (they add nothing to any sum)
  const int r = tid >> 3, cs = (tid & 7) * 8;
  const bool rv = r < n;
  bf16x8 xq, xk, xbx;
  {
    bf16x8 xv, xg, xdo;
    float wr = 0.f;
    if (rv) {
      const size_t o = tok(t0 + r) * D + cs;
      xq = *reinterpret_cast<const bf16x8*>(Q + o);
      xk = *reinterpret_cast<const bf16x8*>(K + o);
      xv = *reinterpret_cast<const bf16x8*>(V + o);
      xg = *reinterpret_cast<const bf16x8*>(Gin + o);
      xbx = *reinterpret_cast<const bf16x8*>(BX + o);
      xdo = *reinterpret_cast<const bf16x8*>(DOg + o);
      wr = to_f32(W[tok(t0 + r)]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xq[i] = xk[i] = xv[i] = xg[i] = xbx[i] = xdo[i] = (bf16)0.f;
    }
    // S and dS_L: thread (channel cc, rows 8 s .. 8 s + 7), every load issued
    // before any store; the partial column sums of S .* dS_L on the side
    const int cc = tid & 63, s = tid >> 6;
    float sv[8], dv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sv[j] = Sg[(size_t)(8 * s + j) * D + cc];
      dv[j] = dSg ? dSg[(size_t)(8 * s + j) * D + cc] : 0.f;
    }
    // output gradients from the chunk mean (d_mean_out / n on the last
    // L-token chunk's tokens; with a projection, the next chunk's gate too)
    const bool lastc = io.dml && t0 + r >= io.dml_from;
    bf16x8 pwv, pdo;
    f32x4 gg[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pwv[i] = (bf16)(wr * to_f32(xv[i]));
      const float dml = lastc && rv ? io.dml[cs + i] : 0.f;
      pdo[i] = (bf16)(to_f32(xdo[i]) + dml);
      gg[i >> 2][i & 3] = rv ? decay_log2<kLogits>(to_f32(xg[i])) : 0.f;   // padding rows do not decay
    }
    *reinterpret_cast<bf16x8*>(WV + r * LD + cs) = pwv;
    *reinterpret_cast<bf16x8*>(dO + r * LD + cs) = pdo;
    *reinterpret_cast<f32x4*>(Gf + r * GLD + cs) = gg[0];
    *reinterpret_cast<f32x4*>(Gf + r * GLD + cs + 4) = gg[1];
    float hs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hs += sv[j] * dv[j];
      Sm[(8 * s + j) * LD + cc] = (bf16)sv[j];
      dSm[(8 * s + j) * LD + cc] = (bf16)dv[j];
    }
    Red[s * D + cc] = hs;                                         // rows 0 .. 7: S .* dS_L partials
  }
  lds_barrier();
  {
    // G: inclusive prefix over the chunk's rows, by (channel, 16-row
    // segment) in the first four waves
    const int cc = tid & 63, s = tid >> 6;
    float gv[16], run = 0.f;
    if (s < 4) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        run += Gf[(16 * s + j) * GLD + cc];
        gv[j] = run;
      }
      Red[(8 + s) * D + cc] = run;
    }
    lds_barrier();
    if (s < 4) {
      float off = 0.f;
      for (int s2 = 0; s2 < s; ++s2) off += Red[(8 + s2) * D + cc];
#pragma unroll
      for (int j = 0; j < 16; ++j) Gf[(16 * s + j) * GLD + cc] = gv[j] + off;
      Gs[s * D + cc] = off;
      Ge[s * D + cc] = off + run;
      const bool steep = -run > kSpanLimit2;
      const bool any = __builtin_amdgcn_ballot_w64(steep) != 0;
      if (lane == 0) Flag[s] = any ? 1 : 0;
    }
  }
  lds_barrier();
  // factor tables: Mid[I][J] = 2^{Gs_I - Ge_J} (J < I), Mid[I][I] = 2^{Gs_I - Ge_I},
  // Dec[I] = 2^{G_L - Ge_I}, Eg[I] = 2^{Gs_I}
  for (int idx = tid; idx < 16 * D; idx += NT) {
    const int i1 = idx / (4 * D), j1 = (idx / D) & 3, cc = idx % D;
    if (j1 <= i1) Mid[idx] = fast_exp2(Gs[i1 * D + cc] - Ge[j1 * D + cc]);
  }
  if (tid < 4 * D) {
    const int i1 = tid / D, cc = tid % D;
    Dec[tid] = fast_exp2(Ge[3 * D + cc] - Ge[i1 * D + cc]);
    Eg[tid] = fast_exp2(Gs[i1 * D + cc]);
  }
  {
    // decayed operands of the thread's row
    const int I0 = r >> 4;
    const float* gr = Gf + r * GLD;
    const float* grm = (r & 15) ? Gf + (r - 1) * GLD : Gs + I0 * D;
    bf16x8 pb, pq, pk;
    const float nq = rv ? nrm(r, 0) : 0.f, nk = rv ? nrm(r, 1) : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = cs + i;
      const float G0 = gr[cc], gs = Gs[I0 * D + cc], ge = Ge[I0 * D + cc];
      const float kv = to_f32(xk[i]) * nk;
      pb[i] = (bf16)(sigmoid_f(to_f32(xbx[i]) + zb(cc)) * kv * fast_exp2(G0 - gs));
      pq[i] = (bf16)(to_f32(xq[i]) * nq * fast_exp2(grm[cc] - gs));
      pk[i] = (bf16)(kv * fast_exp2(ge - G0));
    }
    *reinterpret_cast<bf16x8*>(BKl + r * LD + cs) = pb;
    *reinterpret_cast<bf16x8*>(Ql + r * LD + cs) = pq;
    *reinterpret_cast<bf16x8*>(Kr + r * LD + cs) = pk;
  }
  lds_barrier();

  // ------------------------------------------------------------- fragments
  // A operand: row r0 + c16, reduction indices k0 + 4 g4 .. + 3 of a
  // row-major [row][k] matrix (also the B operand of a product against the
  // rows of a second matrix, B[k][n] = Y[n][k]).
  auto ldA = [&](const bf16* m, int r0, int k0) -> b4 {
    return *reinterpret_cast<const b4*>(m + (r0 + c16) * LD + k0 + 4 * g4);
  };
  // B operand from a row-major [k][n] matrix: B[k0 + 4 g4 + p][n0 + c16]
  auto ldBc = [&](const bf16* m, int k0, int n0) -> b4 {
    const bf16* p = m + (k0 + 4 * g4) * LD + n0 + c16;
    return b4{p[0], p[LD], p[2 * LD], p[3 * LD]};
  };
  auto scl = [](b4 x, float f) -> b4 {
    return b4{(bf16)(to_f32(x[0]) * f), (bf16)(to_f32(x[1]) * f), (bf16)(to_f32(x[2]) * f), (bf16)(to_f32(x[3]) * f)};
  };
  // 16x32 operand of a 16x16x32 product: row r0 + c16, reduction indices
  // k0 + 8 g4 .. + 7 (one 16-byte read), optionally times sc[k] and a sign
  typedef Mma<bf16> M32;
  auto ld8 = [&](const bf16* m, int r0, int k0) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(m + (r0 + c16) * LD + k0 + 8 * g4);
  };
  auto ld8s = [&](const bf16* m, int r0, int k0, const float* sc, float sign) -> bf16x8 {
    const bf16x8 x = ld8(m, r0, k0);
    const f32x4 f0 = *reinterpret_cast<const f32x4*>(sc + k0 + 8 * g4);
    const f32x4 f1 = *reinterpret_cast<const f32x4*>(sc + k0 + 8 * g4 + 4);
    bf16x8 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = (bf16)(sign * to_f32(x[i]) * f0[i]);
      y[4 + i] = (bf16)(sign * to_f32(x[4 + i]) * f1[i]);
    }
    return y;
  };
  // 16x16 tile C[row][col] = sum over the 64 columns of X[rx + row] . Y[ry + col]
  auto gram = [&](const bf16* X, int rx, const bf16* Y, int ry) -> f32x4 {
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < 64; k0 += 32) acc = M32::mma(ld8(X, rx, k0), ld8(Y, ry, k0), acc);
    return acc;
  };
  auto grams = [&](const bf16* X, int rx, const float* sx, const bf16* Y, int ry) -> f32x4 {
    f32x4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < 64; k0 += 32) acc = M32::mma(ld8s(X, rx, k0, sx, 1.f), ld8(Y, ry, k0), acc);
    return acc;
  };
  auto rnd = [](f32x4 x) { return MB::round(x); };
  const bool steep = Flag[I] != 0;
  // raw inputs of the pairwise path (steep sub-blocks only)
  // q (X = Q) or k (X = K) of a chunk row, over its norm with kNorm
  auto raw = [&](const bf16* X, int row, int cc) {
    return row < n ? to_f32(X[tok(t0 + row) * D + cc]) * nrm(row, X == K ? 1 : 0) : 0.f;
  };
  auto raw_bk = [&](int row, int cc) {
    return row < n ? sigmoid_f(to_f32(BX[tok(t0 + row) * D + cc]) + zb(cc)) * to_f32(K[tok(t0 + row) * D + cc]) *
                         nrm(row, 1)
                   : 0.f;
  };
  auto gprev = [&](int row, int cc) { return (row & 15) ? Gf[(row - 1) * GLD + cc] : Gs[(row >> 4) * D + cc]; };

  // ------------------------------------------------- Grams, R and the right side
  const int r0 = 16 * I;
  // aF[J] (J < I): C[j][i] = A[i][j]; aB[J] (J > I): C[j][i] = A[j][i]
  // (both waves of a block form them)
  f32x4 aF[4], aB[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    aF[J] = aB[J] = zero4();
    if (J < I) aF[J] = grams(Kr, 16 * J, Mid + (I * 4 + J) * D, BKl, r0);
    if (J > I) aB[J] = grams(BKl, 16 * J, Mid + (J * 4 + I) * D, Kr, r0);
  }
  if (hc == 0) {
    // diagonal tile of A: C[i][j], j < i
    f32x4 ad;
    if (!steep) {
      ad = grams(BKl, r0, Mid + I * 5 * D, Kr, r0);
    } else {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = r0 + 4 * g4 + ii, j = r0 + c16;
        float acc = 0.f;
        if (j < i)
          for (int cc = 0; cc < D; ++cc)
            acc += raw_bk(i, cc) * raw(K, j, cc) * fast_exp2(Gf[i * GLD + cc] - Gf[j * GLD + cc]);
        ad[ii] = acc;
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) Ad[I * 256 + (4 * g4 + ii) * 16 + c16] = c16 < 4 * g4 + ii ? ad[ii] : 0.f;
  }
  // Y = P^T dO + Kdec dS_L^T  (rows i of block I, this wave's columns e)
  f32x4 y[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) y[q] = zero4();
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J < I) continue;
    f32x4 p;                                                      // C[j][i] = P[j][i]
    if (J > I) {
      p = grams(Ql, 16 * J, Mid + (J * 4 + I) * D, Kr, r0);
    } else {
      if (!steep) {
        p = grams(Ql, r0, Mid + I * 5 * D, Kr, r0);
      } else {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int j = r0 + 4 * g4 + ii, i = r0 + c16;
          float acc = 0.f;
          if (j > i)
            for (int cc = 0; cc < D; ++cc)
              acc += raw(Q, j, cc) * raw(K, i, cc) * fast_exp2(gprev(j, cc) - Gf[i * GLD + cc]);
          p[ii] = acc;
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (!(4 * g4 + ii > c16)) p[ii] = 0.f;
    }
    const b4 pa = rnd(p);
#pragma unroll
    for (int q = 0; q < 2; ++q) y[q] = MB::mma(pa, ldBc(dO, 16 * J, 16 * (2 * hc + q)), y[q]);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int k0 = 0; k0 < 64; k0 += 32)
      y[q] = M32::mma(ld8s(Kr, r0, k0, Dec + I * D, 1.f), ld8(dSm, 16 * (2 * hc + q), k0), y[q]);
  // R = W V - Kb S^T
  f32x4 R[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = 2 * hc + q;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) R[q][ii] = to_f32(WV[(r0 + 4 * g4 + ii) * LD + 16 * nt + c16]);
#pragma unroll
    for (int k0 = 0; k0 < 64; k0 += 32)
      R[q] = M32::mma(ld8s(BKl, r0, k0, Eg + I * D, -1.f), ld8(Sm, 16 * nt, k0), R[q]);
  }
  lds_barrier();
  if (hc == 0) {
    // Td_I = (I + A_II)^{-1}: lane c16 walks column c16 down the rows
    const float* A_ = Ad + I * 256;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = i == c16 ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < i; ++k) v -= A_[i * 16 + k] * t[k];
      t[i] = v;
    }
    if (lane < 16)
#pragma unroll
      for (int i = 0; i < 16; ++i) Td[I * 256 + i * 16 + c16] = t[i];
  }
  lds_barrier();

  // ------------------------------------------ Delta = (I + A)^{-1} R, by blocks
  f32x4 acc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) acc[q] = zero4();
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    if (I == rr) {
      const f32x4 ta = *reinterpret_cast<const f32x4*>(Td + rr * 256 + c16 * 16 + 4 * g4);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4 dl = MF::mma(ta, R[q] - acc[q], zero4());
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) Del[(16 * rr + 4 * g4 + ii) * LD + 16 * (2 * hc + q) + c16] = (bf16)dl[ii];
      }
    }
    lds_barrier();
    if (I > rr) {
      const b4 af = rnd(aF[rr]);
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q] = MB::mma(af, ldBc(Del, 16 * rr, 16 * (2 * hc + q)), acc[q]);
    }
  }

  // ------------------------------------------ dU = (I + A)^{-T} Y, by blocks
  f32x4 du[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    acc[q] = zero4();
    du[q] = zero4();
  }
#pragma unroll
  for (int rr = 3; rr >= 0; --rr) {
    if (I == rr) {
      const float* tdb = Td + rr * 256 + 4 * g4 * 16 + c16;
      const f32x4 ta = {tdb[0], tdb[16], tdb[32], tdb[48]};     // (Td^T)[c16][4 g4 + p]
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        du[q] = MF::mma(ta, y[q] - acc[q], zero4());
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) dU[(16 * rr + 4 * g4 + ii) * LD + 16 * (2 * hc + q) + c16] = (bf16)du[q][ii];
      }
    }
    lds_barrier();
    if (I < rr) {
      const b4 ab = rnd(aB[rr]);
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q] = MB::mma(ab, ldBc(dU, 16 * rr, 16 * (2 * hc + q)), acc[q]);
    }
  }

  // ------------------------------------------------------------ token sums
  // raw inputs of the lane's output elements (rows 16 I + 4 g4 + ii,
  // columns 16 nt + c16), loaded now so they land during the products
  bf16 pq[2][4], pk[2][4], pbx[2][4], pv[2][4], pg[2][4];
  float pw[4], pnq[4], pnk[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int i = r0 + 4 * g4 + ii;
    const bool ok = i < n;
    const size_t ro = tok(t0 + min(i, n - 1)) * D;
    pw[ii] = ok ? to_f32(W[tok(t0 + min(i, n - 1))]) : 0.f;
    pnq[ii] = ok ? nrm(i, 0) : 0.f;
    pnk[ii] = ok ? nrm(i, 1) : 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const size_t o = ro + 16 * (2 * hc + q) + c16;
      pq[q][ii] = ok ? Q[o] : (bf16)0.f;
      pk[q][ii] = ok ? K[o] : (bf16)0.f;
      pbx[q][ii] = ok ? BX[o] : (bf16)0.f;
      pv[q][ii] = ok ? V[o] : (bf16)0.f;
      pg[q][ii] = kLogits && ok ? Gin[o] : (bf16)0.f;
    }
  }
  // qa, xa: sums over j < i (left factor applied at the end); ka: sums over
  // j > i; qx, xx, kx: exact diagonal terms of steep sub-blocks
  f32x4 qa[2], xa[2], ka[2], qx[2], xx[2], kx[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) qa[q] = xa[q] = ka[q] = qx[q] = xx[q] = kx[q] = zero4();
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J < I) {
      const b4 zt = rnd(gram(Del, 16 * J, dO, r0));              // C[j][i] = Z[i][j]
      const b4 nt_ = rnd(gram(Del, 16 * J, dU, r0));             // C[j][i] = N[i][j]
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int nt = 2 * hc + q;
        const b4 kb = ldBc(Kr, 16 * J, 16 * nt);
        const float m = Mid[(I * 4 + J) * D + 16 * nt + c16];
        qa[q] += m * MB::mma(zt, kb, zero4());
        xa[q] += m * MB::mma(nt_, kb, zero4());
      }
    } else if (J > I) {
      const b4 z = rnd(gram(dO, 16 * J, Del, r0));               // C[j][i] = Z[j][i]
      const b4 nn = rnd(-gram(dU, 16 * J, Del, r0));             // C[j][i] = -N[j][i]
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int nt = 2 * hc + q;
        const float m = Mid[(J * 4 + I) * D + 16 * nt + c16];
        ka[q] += m * MB::mma(z, ldBc(Ql, 16 * J, 16 * nt), MB::mma(nn, ldBc(BKl, 16 * J, 16 * nt), zero4()));
      }
    } else {
      f32x4 zt = gram(Del, r0, dO, r0), nt_ = gram(Del, r0, dU, r0);
      f32x4 z = gram(dO, r0, Del, r0), nn = gram(dU, r0, Del, r0);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int jr = 4 * g4 + ii;                              // C row: j; column: i = c16
        if (!(jr < c16)) zt[ii] = nt_[ii] = 0.f;
        if (!(jr > c16)) z[ii] = nn[ii] = 0.f;
      }
      if (!steep) {
        const b4 zb = rnd(zt), nb = rnd(nt_), z2 = rnd(z), n2 = rnd(-nn);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int nt = 2 * hc + q;
          const b4 kb = ldBc(Kr, r0, 16 * nt);
          const float m = Mid[I * 5 * D + 16 * nt + c16];
          qa[q] += m * MB::mma(zb, kb, zero4());
          xa[q] += m * MB::mma(nb, kb, zero4());
          ka[q] += m * MB::mma(z2, ldBc(Ql, r0, 16 * nt), MB::mma(n2, ldBc(BKl, r0, 16 * nt), zero4()));
        }
      } else {
        // the four diagonal tiles (bf16, as the factorised path rounds them)
        // to this wave's scratch, then each output element's terms pairwise
        bf16* sc = Scr + w * 1024;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int o = (4 * g4 + ii) * 16 + c16;
          sc[o] = (bf16)zt[ii];
          sc[256 + o] = (bf16)nt_[ii];
          sc[512 + o] = (bf16)z[ii];
          sc[768 + o] = (bf16)nn[ii];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int cc = 16 * (2 * hc + q) + c16;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int il = 4 * g4 + ii, i = r0 + il;
            const float gi = Gf[i * GLD + cc], gim = gprev(i, cc);
            float sq = 0.f, sx = 0.f, sk = 0.f;
            for (int jl = 0; jl < 16; ++jl) {
              const int j = r0 + jl;
              if (jl < il) {
                const float kj = raw(K, j, cc), gj = Gf[j * GLD + cc];
                sq += to_f32(sc[jl * 16 + il]) * kj * fast_exp2(gim - gj);
                sx += to_f32(sc[256 + jl * 16 + il]) * kj * fast_exp2(gi - gj);
              } else if (jl > il) {
                sk += to_f32(sc[512 + jl * 16 + il]) * raw(Q, j, cc) * fast_exp2(gprev(j, cc) - gi) -
                      to_f32(sc[768 + jl * 16 + il]) * raw_bk(j, cc) * fast_exp2(Gf[j * GLD + cc] - gi);
              }
            }
            qx[q][ii] = sq;
            xx[q][ii] = sx;
            kx[q][ii] = sk;
          }
        }
      }
    }
  }

  // -------------------------------------------------------- assembly
  bf16* dq_o = static_cast<bf16*>(a.dq);
  bf16* dk_o = static_cast<bf16*>(a.dk);
  bf16* dv_o = static_cast<bf16*>(a.dv);
  bf16* dg_o = static_cast<bf16*>(a.dg);
  bf16* dbx_o = static_cast<bf16*>(a.dbx);
  bf16* dw_o = static_cast<bf16*>(a.dw);
  f32x4 sfx[2];                                  // within-lane suffix of phi minus q dq
  float tot[2], hlc[2], dzc[2], dwp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = 2 * hc + q;
    f32x4 dOS = zero4(), dUS = zero4(), DdS = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const b4 sb = ldBc(Sm, 16 * ks, 16 * nt);
      dOS = MB::mma(ldA(dO, r0, 16 * ks), sb, dOS);
      dUS = MB::mma(ldA(dU, r0, 16 * ks), sb, dUS);
      DdS = MB::mma(ldA(Del, r0, 16 * ks), ldBc(dSm, 16 * ks, 16 * nt), DdS);
    }
    const int cc = 16 * nt + c16;
    const float gs = Gs[I * D + cc], ge = Ge[I * D + cc], gl = Ge[3 * D + cc], zc = zb(cc);
    f32x4 phi, qdq;
    float hl = 0.f, dzs = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = r0 + 4 * g4 + ii;
      const float gi = Gf[i * GLD + cc], gim = gprev(i, cc);
      const float qv = to_f32(pq[q][ii]) * pnq[ii], kv = to_f32(pk[q][ii]) * pnk[ii];
      const float bv = sigmoid_f(to_f32(pbx[q][ii]) + zc);
      const float ed = fast_exp2(gl - gi);
      const float dq = fast_exp2(gim - gs) * qa[q][ii] + qx[q][ii] + fast_exp2(gim) * dOS[ii];
      const float xd = fast_exp2(gi - gs) * xa[q][ii] + xx[q][ii] + fast_exp2(gi) * dUS[ii];
      const float dk = ed * DdS[ii] + fast_exp2(ge - gi) * ka[q][ii] + kx[q][ii] - bv * xd;
      const float db = -kv * xd;
      phi[ii] = qv * dq - kv * dk + 2.f * bv * db;
      qdq[ii] = qv * dq;
      hl += kv * ed * DdS[ii];
      const float dvv = pw[ii] * du[q][ii];
      dwp[ii] += to_f32(pv[q][ii]) * du[q][ii];
      const float dbxv = db * bv * (1.f - bv);
      if (i < n) {
        const size_t o = tok(t0 + i) * D + cc;
        if constexpr (kNorm) {
          io.dqh[(size_t)(t0 + i) * D + cc] = dq;
          io.dkh[(size_t)(t0 + i) * D + cc] = dk;
        } else {
          dq_o[o] = (bf16)dq;
          dk_o[o] = (bf16)dk;
        }
        dbx_o[o] = (bf16)dbxv;
        dv_o[o] = (bf16)dvv;
        dzs += dbxv;
      }
    }
    // suffix sums of phi over the lane's rows, minus q dq
    const float s3 = phi[3], s2 = phi[2] + s3, s1 = phi[1] + s2, s0 = phi[0] + s1;
    sfx[q] = f32x4{s0 - qdq[0], s1 - qdq[1], s2 - qdq[2], s3 - qdq[3]};
    tot[q] = s0;
    hlc[q] = hl;
    dzc[q] = dzs;
  }
  // dw: this wave's half of each row's sum over the 64 value columns
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const float sm = sum_row16(dwp[ii]);
    if (c16 == ii) Dwp[w * 16 + 4 * g4 + ii] = sm;
  }
  // phi suffixes over the lane groups of the wave, and wave totals
  float sg[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = 2 * hc + q;
    const float t1 = __shfl(tot[q], c16 + 16), t2 = __shfl(tot[q], c16 + 32), t3 = __shfl(tot[q], c16 + 48);
    const float t0v = __shfl(tot[q], c16);
    sg[q] = (g4 < 1 ? t1 : 0.f) + (g4 < 2 ? t2 : 0.f) + (g4 < 3 ? t3 : 0.f);
    const float hw = sum_groups(hlc[q]);
    const float zw = io.dz ? sum_groups(dzc[q]) : 0.f;
    if (g4 == 0) {
      Red[(8 + I) * D + 16 * nt + c16] = t0v + t1 + t2 + t3;
      Red[(12 + I) * D + 16 * nt + c16] = hw;
      Red[(16 + I) * D + 16 * nt + c16] = zw;
    }
  }
  lds_barrier();
  if (io.dz && tid < D)
    io.dz[tid] = Red[16 * D + tid] + Red[17 * D + tid] + Red[18 * D + tid] + Red[19 * D + tid];
  if (hc == 0 && lane < 16) {
    const int i = r0 + lane;
    if (i < n) dw_o[tok(t0 + i)] = (bf16)(Dwp[w * 16 + lane] + Dwp[(w + 1) * 16 + lane]);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int cc = 16 * (2 * hc + q) + c16;
    float hsum = 0.f, hl = 0.f, sw = 0.f;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) hsum += Red[s8 * D + cc];
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      hl += Red[(12 + w4) * D + cc];
      if (w4 > I) sw += Red[(8 + w4) * D + cc];
    }
    const float HL = fast_exp2(Ge[3 * D + cc]) * hsum + hl;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = r0 + 4 * g4 + ii;
      float dgv = HL + sw + sg[q] + sfx[q][ii];
      if (kLogits) dgv *= -sigmoid_f(to_f32(pg[q][ii]));
      if (i < n) dg_o[tok(t0 + i) * D + cc] = (bf16)dgv;
    }
  }

  // ------------------------------------------- the state gradient at the chunk start
  if (io.dS0) {
    // rows e = 16 I + 4 g4 + ii, columns c = 16 nt + c16
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int nt = 2 * hc + q;
      f32x4 s1 = zero4(), s2 = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float eg = Eg[ks * D + 16 * nt + c16];
        s1 = MB::mma(ldBc(dO, 16 * ks, r0), scl(ldBc(Ql, 16 * ks, 16 * nt), eg), s1);
        s2 = MB::mma(ldBc(dU, 16 * ks, r0), scl(ldBc(BKl, 16 * ks, 16 * nt), eg), s2);
      }
      const int cc = 16 * nt + c16;
      const float el = fast_exp2(Ge[3 * D + cc]);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int e = r0 + 4 * g4 + ii;
        const float dsl = dSg ? dSg[(size_t)e * D + cc] : 0.f;
        io.dS0[(size_t)e * D + cc] = dsl * el + s1[ii] - s2[ii];
      }
    }
  }
}

// Without a projection: one workgroup per (batch, head, chunk), all at once.
template <int D, bool kLogits, bool kNorm>
__global__ void __launch_bounds__(512) carve_bwd_chunk_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nc = (a.T + 63) / 64;
  const int ch = blockIdx.x % nc, bh = blockIdx.x / nc;
  const BwdWs lay(D, a.T, 64, 0, kNorm, true, true);
  float* wsb = a.ws + (size_t)bh * lay.total;
  ChunkIO io;
  io.S0 = wsb + lay.ckpt + (size_t)ch * D * D;
  io.dSL = wsb + lay.dsck + (size_t)(nc - 1 - ch) * D * D;      // the chain runs from the last chunk
  io.z = nullptr;
  io.dml = wsb + lay.dmo;                                       // d_mean_out / n, left by the image kernel
  io.dml_from = (a.T - 1) / a.L * a.L;                          // first token of the last L-token chunk
  io.dS0 = ch == 0 && a.d_state_in ? a.d_state_in + (size_t)bh * D * D : nullptr;
  io.dz = nullptr;
  io.nrm = wsb + lay.nrm;
  io.dqh = wsb + lay.dqh;
  io.dkh = wsb + lay.dkh;
  // no gradient reaches the incoming mean without a projection
  if (ch == 0 && a.d_mean_in && threadIdx.x < D) a.d_mean_in[(size_t)bh * D + threadIdx.x] = 0.f;
  chunk_body<D, kLogits, kNorm>(a, smem, bh, ch, io);
}

// With a content projection (d = 64, 64-token chunks): chunk c's erase gate
// reads the mean of chunk c - 1's outputs, so the chunks are walked from the
// last, one workgroup per (batch, head). chunk_body forms each chunk's
// gradients and the state gradient at its start (carried to the previous
// chunk in fp32 through the workspace); then the gate's gradient
//   dz = sum over the chunk of dbx,  y = U_down m_{c-1},  dy = U_up^T dz,
//   dU_up += dz y^T,  dU_down += dy m_{c-1}^T,  dm_{c-1} = U_down^T dy
// adds dm_{c-1} / 64 to every output gradient of chunk c - 1 (nothing with
// detached means) and leaves the factor gradients of this (batch, head) in
// the workspace for carve_bwd_ub_kernel. The chunk-start states, gate biases
// and gate means come from the checkpointing chunk-serial forward.
template <int D, bool kLogits>
__global__ void __launch_bounds__(512) carve_bwd_chunk_serial_kernel(BwdArgs a) {
  using LY = ChunkBwdLayout<D>;
  constexpr size_t DD = (size_t)D * D;
  extern __shared__ __align__(16) unsigned char smem[];
  float* vec = reinterpret_cast<float*>(smem + LY::oVec);
  float* dzs = vec;                      // the chunk's dz
  float* dml = vec + 64;                 // per value channel, added to the chunk's output gradients
  float* ms = vec + 128;                 // m_{c-1}
  float* ys = vec + 192;                 // U_down m_{c-1}
  float* dys = vec + 256;                // U_up^T dz
  bf16* Uds = reinterpret_cast<bf16*>(smem + LY::oU);
  bf16* Uus = Uds + 64 * D;
  const int tid = threadIdx.x, bh = blockIdx.x, h = bh % a.H, T = a.T, rank = a.rank;
  const int nc = (T + 63) / 64;
  const BwdWs lay(D, T, 64, rank, false, true, true);
  float* wsb = a.ws + (size_t)bh * lay.total;
  float* carry = wsb + lay.dsck;
  const bf16* Ud = static_cast<const bf16*>(a.ub_down) + (size_t)h * rank * D;   // [rank][D]
  const bf16* Uu = static_cast<const bf16*>(a.ub_up) + (size_t)h * D * rank;     // [D][rank]
  for (int i = tid; i < rank * D; i += LY::NT) {
    Uds[i] = Ud[i];
    Uus[i] = Uu[i];
    wsb[lay.dud + i] = 0.f;              // this (batch, head)'s factor gradients, each element
    wsb[lay.duu + i] = 0.f;              // cleared and later updated by the same thread
  }
  const int tl0 = (nc - 1) * 64;
  if (tid < D) dml[tid] = a.d_mean_out ? a.d_mean_out[(size_t)bh * D + tid] / (float)(T - tl0) : 0.f;
  __syncthreads();
  for (int ch = nc - 1; ch >= 0; --ch) {
    ChunkIO io;
    io.S0 = wsb + lay.ckpt + (size_t)ch * DD;
    io.dSL = ch == nc - 1 ? (a.d_state_out ? a.d_state_out + (size_t)bh * DD : nullptr) : carry;
    io.z = wsb + lay.z + (size_t)ch * D;
    io.dml = dml;
    io.dml_from = 64 * ch;
    io.dS0 = ch > 0 ? carry : (a.d_state_in ? a.d_state_in + (size_t)bh * DD : nullptr);
    io.dz = dzs;
    io.nrm = nullptr;
    io.dqh = io.dkh = nullptr;
    chunk_body<D, kLogits, false>(a, smem, bh, ch, io);
    __syncthreads();                     // the carried gradient and dz are complete
    if (tid < D) ms[tid] = wsb[lay.m + (size_t)ch * D + tid];
    __syncthreads();
    if (tid < rank) {
      float y = 0.f, dy = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) {
        y += to_f32(Uds[tid * D + e]) * ms[e];
        dy += to_f32(Uus[e * rank + tid]) * dzs[e];
      }
      ys[tid] = y;
      dys[tid] = dy;
    }
    __syncthreads();
    for (int i = tid; i < rank * D; i += LY::NT) {
      wsb[lay.dud + i] += dys[i / D] * ms[i % D];          // dU_down[r][e]
      wsb[lay.duu + i] += dzs[i / rank] * ys[i % rank];    // dU_up[d][r]
    }
    if (tid < D) {
      float dm = 0.f;
      for (int r = 0; r < rank; ++r) dm += to_f32(Uds[r * D + tid]) * dys[r];
      if (a.detach) dm = 0.f;
      if (ch > 0) dml[tid] = dm * (1.f / 64.f);
      else if (a.d_mean_in) a.d_mean_in[(size_t)bh * D + tid] = dm;
    }
    __syncthreads();
  }
}

// Backward images of the chunk-parallel schedule, in place of the forward
// pair's: chunk c's goes to image slot nc - 1 - c (one workgroup per pair of
// chunks c, nc - 1 - c, which swap slots), so that the checkpointing state
// pass, reading the slots in order, walks the chunks from the last:
//   Mt slot: A operands of M (rows d, k = d'), i.e. the forward's M^T units
//            transposed (gathered element by element through LDS);
//   Ct slot: C tiles of F^T = (dO^T Q_eff)^T (rows d, columns e), per value
//            slice and paired as the forward's C^T tiles, with the dO of the
//            last L-token chunk's tokens carrying d_mean_out / n.
// The Q_eff and O_loc slots keep the forward's contents (the state pass
// forms an output from them into a scratch buffer, unused). The workgroup
// that holds the last 64-token chunk also leaves each row's share of
// d_mean_out in the workspace for carve_bwd_chunk_kernel.
template <int D>
__global__ void __launch_bounds__(256) carve_bwd_image_kernel(BwdArgs a, unsigned char* imgs) {
  using LY = BlockLayout<bf16, D, D, 64>;
  static_assert(D == 64 && LY::NU == 2 && LY::TD == 4 && LY::NB == 4, "d = 64 images of 64-token blocks");
  constexpr int NU = LY::NU, TD = LY::TD, LDO = 72;
  constexpr int MTB = D * D * 2;                                  // bytes of the Mt units (Q_eff follows)
  static_assert(LY::wMt == 0 && LY::wQe == MTB, "Mt and Q_eff units are contiguous");
  typedef bf16x4 b4;
  typedef bf16x8 b8;
  __shared__ __align__(16) unsigned char sm[2][2 * MTB];          // Mt and Q_eff units of each chunk
  __shared__ __align__(16) bf16 sdo[2][64 * LDO];                 // dO of each chunk [t][e]
  const int T = a.T, H = a.H, nc = (T + 63) / 64, np = (nc + 1) / 2;
  const int pr = blockIdx.x % np, bh = blockIdx.x / np, bi = bh / H, h = bh % H;
  const int cA = pr, cB = nc - 1 - pr, nch = cA == cB ? 1 : 2;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), c16 = lane & 15, g4 = lane >> 4;
  unsigned char* base = imgs + (size_t)bh * nc * LY::wBytes;
  const BwdWs lay(D, T, 64, 0, a.norm != 0, true, true);
  float* wsb = a.ws + (size_t)bh * lay.total;
  const bf16* DOg = static_cast<const bf16*>(a.d_o);
  const int tl0 = (T - 1) / a.L * a.L;                           // first token of the last L-token chunk
  for (int x = 0; x < nch; ++x) {
    const int c = x ? cB : cA, t0 = 64 * c, n = min(64, T - t0);
    const uint4* src = reinterpret_cast<const uint4*>(base + (size_t)c * LY::wBytes);
#pragma unroll
    for (int i = 0; i < 2 * MTB / 16 / 256; ++i) reinterpret_cast<uint4*>(sm[x])[tid + 256 * i] = src[tid + 256 * i];
    const int r = tid >> 2, cs = (tid & 3) * 16;
    b8 v[2];
    if (r < n) {
      const size_t o = (((size_t)bi * T + t0 + r) * H + h) * D + cs;
      v[0] = *reinterpret_cast<const b8*>(DOg + o);
      v[1] = *reinterpret_cast<const b8*>(DOg + o + 8);
      if (t0 + r >= tl0 && a.d_mean_out) {
        const float inv = 1.f / (float)(T - tl0);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          v[j >> 3][j & 7] = (bf16)(to_f32(v[j >> 3][j & 7]) + a.d_mean_out[(size_t)bh * D + cs + j] * inv);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j >> 3][j & 7] = (bf16)0.f;
    }
    *reinterpret_cast<b8*>(&sdo[x][r * LDO + cs]) = v[0];
    *reinterpret_cast<b8*>(&sdo[x][r * LDO + cs + 8]) = v[1];
    if (c == nc - 1 && tid < D)
      wsb[lay.dmo + tid] = a.d_mean_out ? a.d_mean_out[(size_t)bh * D + tid] / (float)(T - tl0) : 0.f;
  }
  lds_barrier();
  // element (row r, column col) of a forward unit block (Mt or Q_eff):
  // unit (r / 16, col / 32), lane 16 ((col % 16) / 4) + r % 16, half (col / 16) % 2, element col % 4
  auto at = [](const unsigned char* units, int r, int col) {
    const int off = (((r >> 4) * NU + (col >> 5)) * 64 + 16 * ((col & 15) >> 2) + (r & 15)) * 16 +
                    ((col >> 4) & 1) * 8 + (col & 3) * 2;
    return *reinterpret_cast<const bf16*>(units + off);
  };
  for (int x = 0; x < nch; ++x) {
    const int c = x ? cB : cA;
    unsigned char* dst = base + (size_t)(nc - 1 - c) * LY::wBytes;
    // Mb units (D = w, u): lane (g4, c16) holds M[d = 16 D + c16][k], k = 32 u + 4 g4 + i and
    // 32 u + 16 + 4 g4 + i, with M[d][k] = Mt[k][d]
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      b8 m;
      const int d = 16 * w + c16;
#pragma unroll
      for (int j = 0; j < 8; ++j) m[j] = at(sm[x], 32 * u + 16 * (j >> 2) + 4 * g4 + (j & 3), d);
      *reinterpret_cast<b8*>(dst + LY::wMt + ((w * NU + u) * 64 + lane) * 16) = m;
    }
    // F^T tiles (rows d, columns e) = sum_t Q_eff[t][d] dO[t][e]: this wave
    // takes the row tiles 2 a, 2 a + 1 of value slices 2 b, 2 b + 1
    const int ta = w & 1, sb = w >> 1;
    f32x4 f[2][2];
#pragma unroll
    for (int dd = 0; dd < 2; ++dd)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) f[dd][ss] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      b4 qa[2], db[2];
#pragma unroll
      for (int dd = 0; dd < 2; ++dd) {
        const int d = 16 * (2 * ta + dd) + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) qa[dd][i] = at(sm[x] + MTB, 16 * ks + 4 * g4 + i, d);
      }
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const bf16* p = &sdo[x][(16 * ks + 4 * g4) * LDO + 16 * (2 * sb + ss) + c16];
        db[ss] = b4{p[0], p[LDO], p[2 * LDO], p[3 * LDO]};
      }
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) f[dd][ss] = Mma16<bf16>::mma(qa[dd], db[ss], f[dd][ss]);
    }
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const int slice = 2 * sb + ss;
      b8 pv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = (bf16)f[0][ss][i];
        pv[4 + i] = (bf16)f[1][ss][i];
      }
      *reinterpret_cast<b8*>(dst + LY::wCt + ((slice * (TD / 2) + ta) * 64 + lane) * 16) = pv;
    }
  }
}

}  // namespace carve
