// Per-block operations of the CARVE WY chunk solver, shared by every kernel.
//
// A block is BL consecutive tokens (BL in {16, 32, 64}) of one (batch, head).
// With S the state at the block start, G_r the inclusive cumulative log-decay
// inside the block (G_{-1} = 0), b_r = sigmoid(bx_r + z) and z = U_b m_{c-1}
// (gist.science technical summary, §2.1 "Content-Aware Erase via Output
// Reuse"; §2.2 scalar write gate; §2.3 key-axis decay):
//   A_rj  = sum_d b_r k_r k_j e^{G_r - G_j}          (j < r)
//   P_rj  = sum_d q_r k_j e^{G_{r-1} - G_j}          (j < r)
//   T     = (I + A)^{-1}
//   W     = T (b k e^{G_r}),   U = T (w v)
//   Delta = U - W S^T
//   O     = (q e^{G_{r-1}}) S^T + P Delta           (o_t = S_{t-1} q_t)
//   S    <- S diag(e^{G_BL}) + Delta^T (k e^{G_BL - G_j})
// This is exact algebra for the token recurrence S <- S D (I - (b k) k^T) +
// w v k^T; one triangular system per block exists because every gate acts on
// the key axis (Theorem 11, §3 of the same summary).
//
// Exponent safety: the Grams use 16-row sub-blocks. For sub-blocks I > J the
// factor e^{G_r - G_j} is split as e^{G_r - Gs_I} e^{Gs_I - Ge_J} e^{Ge_J - G_j}
// (Gs_I: G just before sub-block I; Ge_J: G at the end of sub-block J), every
// factor <= 1. Diagonal sub-blocks use e^{G_r - Gs_I} e^{Gs_I - G_j}, safe while
// the decay inside one sub-block stays below kSpanLimit2 (log2 units); steeper
// blocks are rebuilt pairwise.
//
// LDS rows are padded by 16 bytes so that the 16 lanes of an MFMA fragment,
// which read 16 consecutive rows, fall into different banks.
#pragma once
#include "common.h"

namespace carve {

struct FwdArgs {
  const void* q; const void* k; const void* v; const void* g; const void* bx; const void* w;
  const void* ub_down; const void* ub_up;
  const float* state_in; const float* mean_in;
  void* o; float* state_out; float* mean_out;
  void* ws;
  int B, H, T, L, rank;
};

constexpr float kSpanLimit2 = 96.0f;   // max decay (log2 units) inside a 16-row sub-block

template <typename E, int DK, int DV, int BL>
struct BlockLayout {
  static_assert(DK % 32 == 0 && DV % 16 == 0 && DK == DV, "head widths");
  static_assert(BL == 16 || BL == 32 || BL == 64, "block length");
  static constexpr int NW = DV / 16;                 // one wave per 16 value channels
  static constexpr int NT = NW * 64;
  static constexpr int NB = BL / 16;
  static constexpr int KP = BL < 32 ? 32 : BL;       // padded token-reduction width
  static_assert(NT >= DK * NB, "one thread per (key column, sub-block) in the gate pass");
  static constexpr int ES = sizeof(E);
  static constexpr int PE = 16 / ES;                 // 16-byte row padding, in elements
  static constexpr int LD = DK + PE;                 // pitch of [.][DK] tiles
  static constexpr int LK = KP + PE;                 // pitch of [.][KP] tiles
  static constexpr int LV = DV + PE;                 // pitch of the value tile
  static constexpr int LA = BL + 4;                  // pitch of A (fp32)
  static constexpr int LTD = 16 + 4;                 // pitch of the diagonal inverses (fp32)
  static constexpr int NFAR = NB > 2 ? (NB - 1) * (NB - 2) / 2 : 1;   // sub-block pairs J < I-1

  // LDS byte offsets. Small arrays first, then tiles; the chunk-parallel
  // kernel stops at intra_bytes, the chunk-serial kernel also keeps the
  // state-pass operands Qd, KdT, P, W.
  static constexpr int oGb = 0;                              // [NB+1][DK] f32 (log2 units)
  static constexpr int oSeg = oGb + (NB + 1) * DK * 4;       // [NB][DK] f32
  static constexpr int oEgl = oSeg + NB * DK * 4;            // [DK] f32 e^{G_BL}
  static constexpr int oEGs = oEgl + DK * 4;                 // [NB][DK] f32 e^{Gs_I}
  static constexpr int oWg = oEGs + NB * DK * 4;             // [KP] f32 write gate (zero padded)
  static constexpr int oZ = oWg + KP * 4;                    // [DK] f32
  static constexpr int oM = oZ + DK * 4;                     // [DV] f32
  static constexpr int oY = oM + DV * 4;                     // [64] f32
  static constexpr int oFlag = oY + 64 * 4;                  // int
  static constexpr int oFd = oFlag + 16;                     // [NB][DK] f32 e^{Gs_J - Ge_J}
  static constexpr int oFf = oFd + NB * DK * 4;              // [NFAR][DK] f32 e^{Gs_I - Ge_J}
  static constexpr int oOnes = oFf + NFAR * DK * 4;          // [DK] f32 all ones
  static constexpr int oKx = oOnes + DK * 4;                 // [BL][LD] E
  static constexpr int oQx = oKx + BL * LD * ES;             // [BL][LD] E   (then A, fp32)
  static constexpr int oKy = oQx + BL * LD * ES;             // [BL][LD] E
  static constexpr int oV = oKy + BL * LD * ES;              // [KP][LV] E   (then U; rows >= BL stay 0)
  static constexpr int oTd = oV + KP * LV * ES;              // [NB][16][LTD] f32
  static constexpr int intra_bytes = oTd + NB * 16 * LTD * 4;
  static constexpr int oQd = intra_bytes;                    // [BL][LD] E
  static constexpr int oKdT = oQd + BL * LD * ES;            // [DK][LK] E
  static constexpr int oP = oKdT + DK * LK * ES;             // [BL][LK] E
  static constexpr int oW = oP + BL * LK * ES;               // [BL][LD] E
  static constexpr int serial_bytes = oW + BL * LD * ES;
  static_assert(2 * BL * LD * ES >= BL * LA * 4, "A fits in the Qx/Ky region");
  static_assert(serial_bytes <= 160 * 1024, "LDS budget");
  static_assert(oKx % 16 == 0 && oV % 16 == 0 && oTd % 16 == 0, "tile alignment");

  // dense image of one block's state-pass operands (workspace)
  static constexpr int wW = 0;                               // [BL][DK] E
  static constexpr int wQd = wW + BL * DK * ES;              // [BL][DK] E
  static constexpr int wP = wQd + BL * DK * ES;              // [BL][KP] E
  static constexpr int wKdT = wP + BL * KP * ES;             // [DK][KP] E
  static constexpr int wU = wKdT + DK * KP * ES;             // [BL][DV] E
  static constexpr int wEgl = wU + BL * DV * ES;             // [DK] f32
  static constexpr int wBytes = wEgl + DK * 4;
  static_assert(wBytes % 16 == 0, "16-byte copies");
  // padded staging copy of the image in LDS (state pass)
  static constexpr int sW = 0;                               // [BL][LD]
  static constexpr int sQd = sW + BL * LD * ES;              // [BL][LD]
  static constexpr int sP = sQd + BL * LD * ES;              // [BL][LK]
  static constexpr int sKdT = sP + BL * LK * ES;             // [DK][LK]
  static constexpr int sU = sKdT + DK * LK * ES;             // [BL][DV] (dense)
  static constexpr int sEgl = sU + BL * DV * ES;             // [DK] f32
  static constexpr int sBytes = sEgl + DK * 4;

  // LDS offset (relative to a staging buffer) of the 16-byte chunk c of the image
  __device__ __forceinline__ static int stage_offset(int c) {
    const int b = 16 * c;
    if (b < wQd) return sW + (b / (DK * ES)) * LD * ES + b % (DK * ES);
    if (b < wP) { const int x = b - wQd; return sQd + (x / (DK * ES)) * LD * ES + x % (DK * ES); }
    if (b < wKdT) { const int x = b - wP; return sP + (x / (KP * ES)) * LK * ES + x % (KP * ES); }
    if (b < wU) { const int x = b - wKdT; return sKdT + (x / (KP * ES)) * LK * ES + x % (KP * ES); }
    return sU + (b - wU);                    // U and Egl are copied densely
  }
};

template <typename E>
__device__ __forceinline__ float ldg(const E* p, size_t i) { return to_f32(p[i]); }

// multiply fragment slot values by per-k factors (natural map)
template <typename M> struct FragScale;
template <> struct FragScale<bf16> {
  __device__ __forceinline__ static bf16x8 apply(bf16x8 a, const float* fac, int k0) {
    const int g = lane_id() >> 4;
    const f32x4* f = reinterpret_cast<const f32x4*>(fac + k0 + 8 * g);
    const f32x4 f0 = f[0], f1 = f[1];
    return bf16x8{(bf16)((float)a[0] * f0[0]), (bf16)((float)a[1] * f0[1]),
                  (bf16)((float)a[2] * f0[2]), (bf16)((float)a[3] * f0[3]),
                  (bf16)((float)a[4] * f1[0]), (bf16)((float)a[5] * f1[1]),
                  (bf16)((float)a[6] * f1[2]), (bf16)((float)a[7] * f1[3])};
  }
};
template <> struct FragScale<float> {
  __device__ __forceinline__ static float apply(float a, const float* fac, int k0) {
    return a * fac[k0 + (lane_id() >> 4)];
  }
};

// Token rows of one (batch, head) in the [B, T, H, d] layout.
template <typename E>
struct Rows {
  const E* Q; const E* K; const E* V; const E* G; const E* BX; const E* W;
  int T, H, bidx, h;
  __device__ __forceinline__ size_t row(int t) const { return (size_t)(bidx * T + t) * H + h; }
};

// Where the state-pass operands of a block go: LDS (chunk-serial kernel) or
// the dense workspace image (chunk-parallel kernel).
template <typename E>
struct Sink {
  E* Qd; int ldQd;      // [BL][.]
  E* KdT; int ldKdT;    // [DK][.]
  E* P; int ldP;        // [BL][.]
  E* W; int ldW;        // [BL][.]
};

template <typename E, int DK, int DV, int BL>
struct Block {
  using LY = BlockLayout<E, DK, DV, BL>;
  using MM = Mma<E>;
  using Frag = typename MM::frag;
  static constexpr int NW = LY::NW, NT = LY::NT, NB = LY::NB, KP = LY::KP, KS = MM::KS;
  static constexpr int LD = LY::LD, LK = LY::LK, LV = LY::LV, LA = LY::LA, LTD = LY::LTD;

  struct Smem {
    unsigned char* base;
    E *Kx, *Qx, *Ky, *V, *Qd, *KdT, *P, *W;
    float *A, *Td, *Gb, *Seg, *Egl, *EGs, *Wg, *Z, *M, *Y, *Fd, *Ff, *Ones;
    int* Flag;
  };

  __device__ static Smem carve(unsigned char* smem) {
    Smem s;
    s.base = smem;
    s.Kx = reinterpret_cast<E*>(smem + LY::oKx);
    s.Qx = reinterpret_cast<E*>(smem + LY::oQx);
    s.A = reinterpret_cast<float*>(smem + LY::oQx);    // A reuses Qx/Ky after the Grams
    s.Ky = reinterpret_cast<E*>(smem + LY::oKy);
    s.V = reinterpret_cast<E*>(smem + LY::oV);
    s.Td = reinterpret_cast<float*>(smem + LY::oTd);
    s.Qd = reinterpret_cast<E*>(smem + LY::oQd);
    s.KdT = reinterpret_cast<E*>(smem + LY::oKdT);
    s.P = reinterpret_cast<E*>(smem + LY::oP);
    s.W = reinterpret_cast<E*>(smem + LY::oW);
    s.Gb = reinterpret_cast<float*>(smem + LY::oGb);
    s.Seg = reinterpret_cast<float*>(smem + LY::oSeg);
    s.Egl = reinterpret_cast<float*>(smem + LY::oEgl);
    s.EGs = reinterpret_cast<float*>(smem + LY::oEGs);
    s.Wg = reinterpret_cast<float*>(smem + LY::oWg);
    s.Z = reinterpret_cast<float*>(smem + LY::oZ);
    s.M = reinterpret_cast<float*>(smem + LY::oM);
    s.Y = reinterpret_cast<float*>(smem + LY::oY);
    s.Flag = reinterpret_cast<int*>(smem + LY::oFlag);
    s.Fd = reinterpret_cast<float*>(smem + LY::oFd);
    s.Ff = reinterpret_cast<float*>(smem + LY::oFf);
    s.Ones = reinterpret_cast<float*>(smem + LY::oOnes);
    return s;
  }

  __device__ static Sink<E> lds_sink(const Smem& s) { return Sink<E>{s.Qd, LD, s.KdT, LK, s.P, LK, s.W, LD}; }
  __device__ static Sink<E> image_sink(unsigned char* img) {
    return Sink<E>{reinterpret_cast<E*>(img + LY::wQd), DK, reinterpret_cast<E*>(img + LY::wKdT), KP,
                   reinterpret_cast<E*>(img + LY::wP), KP, reinterpret_cast<E*>(img + LY::wW), DK};
  }

  __device__ static void zero_lds(unsigned char* smem, int bytes) {
    for (int i = threadIdx.x; i < bytes / 4; i += NT) reinterpret_cast<float*>(smem)[i] = 0.f;
  }

  // -------------------------------------------------------------- gate pass
  // Loads tokens [t0, t0 + nvalid) and builds every decay-scaled operand.
  // Thread (gd, gs) owns key column gd of 16-row sub-block gs. Rows past
  // nvalid read as zeros (k = q = v = w = g = 0), which leaves the state
  // untouched. Returns true if a sub-block's decay is too steep for the
  // factorised diagonal Grams. Ends with a barrier.
  __device__ static bool gate_pass(const Smem& s, const Rows<E>& src, int t0, int nvalid, const Sink<E>& out) {
    const int tid = threadIdx.x;
    const int gs = wave_id() * 64 / DK, gd = tid % DK;
    if (tid == 0) s.Flag[0] = 0;
    for (int d = tid; d < DK; d += NT) s.Ones[d] = 1.f;
    float gv[16], kv[16], qv[16], bv[16];
    if (gs < NB) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * gs + i;
        const int rc = min(r, nvalid - 1);           // clamped row: loads stay in bounds
        const size_t off = src.row(t0 + rc) * DK + gd;
        const float keep = r < nvalid ? 1.f : 0.f;
        gv[i] = keep * ldg(src.G, off);
        kv[i] = keep * ldg(src.K, off);
        qv[i] = keep * ldg(src.Q, off);
        bv[i] = ldg(src.BX, off);
      }
    }
    // values: 16-byte row chunks into the padded V tile
    {
      constexpr int CPR = DV * LY::ES / 16;          // chunks per row
      constexpr int NCH = BL * CPR;
      constexpr int PER = (NCH + NT - 1) / NT;
      f32x4 vc[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int c = tid + j * NT;
        if (c < NCH) {
          const int r = c / CPR, cc = c % CPR;
          const int rc = min(r, nvalid - 1);
          vc[j] = *reinterpret_cast<const f32x4*>(src.V + src.row(t0 + rc) * DV + cc * (16 / LY::ES));
          if (r >= nvalid) vc[j] = zero4();
        }
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int c = tid + j * NT;
        if (c < NCH) {
          const int r = c / CPR, cc = c % CPR;
          *reinterpret_cast<f32x4*>(s.V + r * LV + cc * (16 / LY::ES)) = vc[j];
        }
      }
    }
    for (int r = tid; r < BL; r += NT) {
      const int rc = min(r, nvalid - 1);
      const float ww = ldg(src.W, src.row(t0 + rc));
      s.Wg[r] = r < nvalid ? ww : 0.f;
    }
    float run = 0.f;
    if (gs < NB) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        run += gv[i] * kLog2e;
        gv[i] = run;                                 // local inclusive G, log2 units
      }
      s.Seg[gs * DK + gd] = run;
    }
    __syncthreads();
    if (gs < NB) {
      float base = 0.f, total = 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float t = s.Seg[j * DK + gd];
        if (j < gs) base += t;
        total += t;
      }
      const float Gs = base;                         // G before this sub-block
      const float Ge = base + run;                   // G at its last row
      const float eGs = fast_exp2(Gs);
      s.Gb[gs * DK + gd] = Gs;
      s.EGs[gs * DK + gd] = eGs;
      if (gs == NB - 1) {
        s.Gb[NB * DK + gd] = total;
        s.Egl[gd] = fast_exp2(total);
      }
      if (Gs - Ge > kSpanLimit2) atomicOr(s.Flag, 1);
      // Gram scaling factors of this column: diagonal sub-block gs, and the
      // pairs (I, gs) with I > gs + 1
      s.Fd[gs * DK + gd] = fast_exp2(Gs - Ge);
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        if (I > gs + 1) {
          float gsI = 0.f;                           // G before sub-block I
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (j < I) gsI += s.Seg[j * DK + gd];
          s.Ff[((I - 2) * (I - 1) / 2 + gs) * DK + gd] = fast_exp2(gsI - Ge);
        }
      }
      const float eTail = fast_exp2(total - Ge);
      const float z = s.Z[gd];
      float eprev = 1.f;                             // e^{G_{r-1} - Gs}
      E kd[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * gs + i;
        const float Gr = base + gv[i];
        const float bb = sigmoid_f(bv[i] + z);
        const float e1 = fast_exp2(Gr - Gs);         // <= 1
        const float en = fast_exp2(Ge - Gr);         // <= 1
        s.Kx[r * LD + gd] = from_f32<E>(bb * kv[i] * e1);
        s.Qx[r * LD + gd] = from_f32<E>(qv[i] * eprev);
        s.Ky[r * LD + gd] = from_f32<E>(kv[i] * en);
        out.Qd[r * out.ldQd + gd] = from_f32<E>(qv[i] * eprev * eGs);
        kd[i] = from_f32<E>(kv[i] * en * eTail);
        eprev = e1;
      }
      // Kdec transposed: this thread's 16 rows are 16 consecutive elements
      E* kdt = out.KdT + gd * out.ldKdT + 16 * gs;
#pragma unroll
      for (int c = 0; c < 16 * LY::ES / 16; ++c)
        *reinterpret_cast<f32x4*>(kdt + c * (16 / LY::ES)) = *reinterpret_cast<const f32x4*>(kd + c * (16 / LY::ES));
    }
    __syncthreads();
    return s.Flag[0] != 0;
  }

  // -------------------------------------------------------------- Grams A, P
  // A (fp32) lands over the Qx/Ky region once every wave is done with them.
  // Ends with a barrier.
  __device__ static void grams(const Smem& s, const Rows<E>& src, int t0, int nvalid, bool fallback,
                               const Sink<E>& out) {
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int gq = lane >> 4, cc = lane & 15;
    constexpr int TPW = (NB * NB + NW - 1) / NW;     // tiles per wave
    f32x4 accA[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      accA[k] = zero4();
      const int tile = wave + k * NW;
      if (tile >= NB * NB) continue;
      const int I = tile / NB, J = tile % NB;
      if (J > I) {                                   // above the diagonal: P is zero
#pragma unroll
        for (int i = 0; i < 4; ++i) out.P[(16 * I + 4 * gq + i) * out.ldP + 16 * J + cc] = from_f32<E>(0.f);
        continue;
      }
      const bool diag = (I == J), far = (J < I - 1);
      // left factor e^{Gs_I - Ge_J} for far pairs, right factor e^{Gs_J - Ge_J}
      // on the diagonal; other tiles multiply by ones (no branches)
      const float* fl = far ? s.Ff + ((I - 2) * (I - 1) / 2 + J) * DK : s.Ones;
      const float* fr = diag ? s.Fd + J * DK : s.Ones;
      f32x4 acP = zero4();
      Frag ka[DK / KS], qa[DK / KS], kb[DK / KS];
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) {
        ka[p] = MM::ld_nat(s.Kx, LD, 16 * I + cc, p * KS);
        qa[p] = MM::ld_nat(s.Qx, LD, 16 * I + cc, p * KS);
        kb[p] = MM::ld_nat(s.Ky, LD, 16 * J + cc, p * KS);
      }
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) {
        const Frag a = FragScale<E>::apply(ka[p], fl, p * KS);
        const Frag aq = FragScale<E>::apply(qa[p], fl, p * KS);
        const Frag b = FragScale<E>::apply(kb[p], fr, p * KS);
        accA[k] = MM::mma(a, b, accA[k]);
        acP = MM::mma(aq, b, acP);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * I + 4 * gq + i, j = 16 * J + cc;
        const bool keep = !diag || (j < r);
        accA[k][i] = keep ? accA[k][i] : 0.f;
        out.P[r * out.ldP + j] = from_f32<E>(keep ? acP[i] : 0.f);
      }
    }
    // padding columns of P (only when BL < KP)
    if constexpr (BL < KP)
      for (int idx = tid; idx < BL * (KP - BL); idx += NT)
        out.P[(idx / (KP - BL)) * out.ldP + BL + idx % (KP - BL)] = from_f32<E>(0.f);
    __syncthreads();                                 // Qx/Ky are free now
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int tile = wave + k * NW;
      if (tile >= NB * NB) continue;
      const int I = tile / NB, J = tile % NB;
      if (J > I) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) s.A[(16 * I + 4 * gq + i) * LA + 16 * J + cc] = accA[k][i];
    }
    __syncthreads();
    if (fallback) {
      grams_pairwise(s, src, t0, nvalid, out);
      __syncthreads();
    }
  }

  // Diagonal sub-blocks rebuilt pairwise, straight from the raw gates in
  // global memory: used only for decays too steep for the factorised form.
  // Slow but exact; needs no LDS scratch.
  __device__ static void grams_pairwise(const Smem& s, const Rows<E>& src, int t0, int nvalid,
                                        const Sink<E>& out) {
    for (int item = threadIdx.x; item < NB * 120; item += NT) {
      const int I = item / 120;
      int p = item % 120, ri = 1;
      while (p >= ri) { p -= ri; ++ri; }
      const int ji = p;
      const int r = 16 * I + ri, j = 16 * I + ji;
      float sa = 0.f, sp = 0.f;
      if (r < nvalid) {
        const size_t rowr = src.row(t0 + r) * DK, rowj = src.row(t0 + j) * DK;
        for (int d = 0; d < DK; ++d) {
          float dg = 0.f;                          // G_{r-1} - G_j, log2 units
          for (int t = j + 1; t < r; ++t) dg += ldg(src.G, src.row(t0 + t) * DK + d) * kLog2e;
          const float gr = ldg(src.G, rowr + d) * kLog2e;
          const float kj = ldg(src.K, rowj + d);
          const float br = sigmoid_f(ldg(src.BX, rowr + d) + s.Z[d]);
          sa += br * ldg(src.K, rowr + d) * kj * fast_exp2(dg + gr);
          sp += ldg(src.Q, rowr + d) * kj * fast_exp2(dg);
        }
      }
      s.A[r * LA + j] = sa;
      out.P[r * out.ldP + j] = from_f32<E>(sp);
    }
  }

  // -------------------------------------------------------------- (I + A_II)^{-1}
  // Diagonal 16x16 blocks by forward substitution in fp32. Wave 0, lane
  // (block ib = gq, column c = cc) keeps its whole column in registers.
  // Ends with a barrier.
  __device__ static void inverse_diag(const Smem& s) {
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int ib = lane >> 4, c = lane & 15;
    if (wave == 0 && ib < NB) {
      const float* Ablk = s.A + (16 * ib) * LA + 16 * ib;
      float t[16];
      float cur[16], nxt[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) *reinterpret_cast<f32x4*>(cur + 4 * q4) = *reinterpret_cast<const f32x4*>(Ablk + LA + 4 * q4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r >= 1 && r + 1 < 16) {                    // fetch row r+1 while row r is reduced
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            if (4 * q4 < r + 1) *reinterpret_cast<f32x4*>(nxt + 4 * q4) = *reinterpret_cast<const f32x4*>(Ablk + (r + 1) * LA + 4 * q4);
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < r; ++j) acc += cur[j] * t[j];
        t[r] = (r == c) ? 1.f : ((r > c) ? -acc : 0.f);
        if (r >= 1 && r + 1 < 16) {
#pragma unroll
          for (int j = 0; j < 16; ++j) cur[j] = nxt[j];
        }
      }
      float* Tb = s.Td + ib * 16 * LTD;
#pragma unroll
      for (int r = 0; r < 16; ++r) Tb[r * LTD + c] = t[r];
    }
    __syncthreads();
  }

  // -------------------------------------------------------------- [W | U] = (I + A)^{-1} [Kb | w V]
  // Blocked forward substitution over 16-row sub-blocks:
  //   X_I = T_II (R_I - sum_{J<I} A_IJ X_J),  R = [b k e^{G} | w v],
  // with T_II the diagonal inverses. Wave w solves the two 16-column tiles
  // 2w, 2w+1 of [W | U] (DK + DV = 32 NW columns) independently, keeping its
  // X_J tiles in registers. W goes to the sink, U (rounded to E) overwrites
  // the value tile in place. Ends with a barrier.
  __device__ static void solve(const Smem& s, const Sink<E>& out) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
    // operands that do not depend on the recursion, loaded up front:
    // right-hand sides R (C layout), A_IJ rows and T_II rows (fp32)
    // both column tiles of a wave lie on the same side of [W | U]
    const bool isW = 2 * wave < DK / 16;
    const int col0 = 32 * wave - (isW ? 0 : DK) + cc;
    f32x4 R[NB][2];
    if (isW) {
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * gq + i, c = col0 + 16 * t;
            R[I][t][i] = to_f32(s.Kx[r * LD + c]) * s.EGs[I * DK + c];   // b k e^{G_r}
          }
    } else {
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * gq + i, c = col0 + 16 * t;
            R[I][t][i] = s.Wg[r] * to_f32(s.V[r * LV + c]);              // w v
          }
    }
    f32x4 Arow[NB > 1 ? NB * (NB - 1) / 2 : 1], Trow[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      Trow[I] = *reinterpret_cast<const f32x4*>(s.Td + I * 16 * LTD + cc * LTD + 4 * gq);
#pragma unroll
      for (int J = 0; J < I; ++J)
        Arow[I * (I - 1) / 2 + J] = *reinterpret_cast<const f32x4*>(s.A + (16 * I + cc) * LA + 16 * J + 4 * gq);
    }
    f32x4 X[NB][2];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 acc[2] = {R[I][0], R[I][1]};
#pragma unroll
      for (int J = 0; J < I; ++J)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = Mma16<E>::mma_a_cB(Arow[I * (I - 1) / 2 + J], X[J][t], acc[t], -1.f);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 x = Mma16<E>::mma_a_cB(Trow[I], acc[t], zero4(), 1.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = to_f32(from_f32<E>(x[i]));
        X[I][t] = x;
      }
    }
    if (isW) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            out.W[(16 * I + 4 * gq + i) * out.ldW + col0 + 16 * t] = from_f32<E>(X[I][t][i]);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s.V[(16 * I + 4 * gq + i) * LV + col0 + 16 * t] = from_f32<E>(X[I][t][i]);
    }
    __syncthreads();
  }

  // U tiles of this wave's 16 value channels, from the value tile after solve()
  __device__ static void load_u(const Smem& s, f32x4 (&U)[NB]) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) U[rt][i] = to_f32(s.V[(16 * rt + 4 * gq + i) * LV + 16 * wave + cc]);
  }

  // -------------------------------------------------------------- state and output
  // Per wave (its 16 value channels): Delta = U - W S^T, O = Qd S^T + P Delta,
  // S^T <- diag(e^{G_BL}) S^T + Kdec^T Delta. Operand tiles: W, Qd [BL][LD];
  // P [BL][LK]; KdT [DK][LK]; Egl [DK].
  __device__ static void state_step(const E* W, const E* Qd, const E* P, const E* KdT, const float* Egl,
                                    const f32x4 (&U)[NB], f32x4 (&St)[DK / 16], f32x4 (&Ot)[NB]) {
    const int lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
    constexpr int NDT = KP / 16;                     // Delta tiles incl. padding
    f32x4 D[NDT];
#pragma unroll
    for (int rt = 0; rt < NDT; ++rt) D[rt] = zero4();
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      f32x4 ws = zero4();
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) ws = MM::mma(MM::ld_cp(W, LD, 16 * rt + cc, p), MM::from_c(St, p), ws);
      D[rt] = U[rt] - ws;
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) acc = MM::mma(MM::ld_cp(Qd, LD, 16 * rt + cc, p), MM::from_c(St, p), acc);
#pragma unroll
      for (int p = 0; p < MM::steps(BL); ++p)
        if (p < MM::steps(16 * (rt + 1))) acc = MM::mma(MM::ld_cp(P, LK, 16 * rt + cc, p), MM::from_c(D, p), acc);
      Ot[rt] = acc;
    }
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = St[dt][i] * Egl[16 * dt + 4 * gq + i];
#pragma unroll
      for (int p = 0; p < MM::steps(BL); ++p) acc = MM::mma(MM::ld_cp(KdT, LK, 16 * dt + cc, p), MM::from_c(D, p), acc);
      St[dt] = acc;
    }
  }

  // load/store S^T C tiles of this wave from/to a [B,H,DV,DK] fp32 tensor
  __device__ static void load_state(const float* S, int bh, f32x4 (&St)[DK / 16]) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      if (S) St[dt] = *reinterpret_cast<const f32x4*>(S + ((size_t)bh * DV + 16 * wave + cc) * DK + 16 * dt + 4 * gq);
      else St[dt] = zero4();
    }
  }
  __device__ static void store_state(float* S, int bh, const f32x4 (&St)[DK / 16]) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
      *reinterpret_cast<f32x4*>(S + ((size_t)bh * DV + 16 * wave + cc) * DK + 16 * dt + 4 * gq) = St[dt];
  }
};

}  // namespace carve
