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
  static_assert(DK % 32 == 0 && DV % 16 == 0, "head widths");
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
  static constexpr int LT = KP + 4;                  // pitch of T (fp32)
  static constexpr int LA = BL + 4;                  // pitch of A (fp32)

  // LDS byte offsets. Small arrays first, then tiles; the chunk-parallel
  // kernel stops after A, the chunk-serial kernel also keeps Qd, KdT, P.
  static constexpr int oGb = 0;                              // [NB+1][DK] f32 (log2 units)
  static constexpr int oSeg = oGb + (NB + 1) * DK * 4;       // [NB][DK] f32
  static constexpr int oEgl = oSeg + NB * DK * 4;            // [DK] f32
  static constexpr int oWg = oEgl + DK * 4;                  // [KP] f32 write gate (zero padded)
  static constexpr int oZ = oWg + KP * 4;                    // [DK] f32
  static constexpr int oM = oZ + DK * 4;                     // [DV] f32
  static constexpr int oY = oM + DV * 4;                     // [64] f32
  static constexpr int oFlag = oY + 64 * 4;                  // int
  static constexpr int oKx = oFlag + 16;                     // [BL][LD] E   (serial: later W)
  static constexpr int oQx = oKx + BL * LD * ES;             // [BL][LD] E   (later T, fp32)
  static constexpr int oKy = oQx + BL * LD * ES;             // [BL][LD] E
  static constexpr int oKbT = oKy + BL * LD * ES;            // [DK][LK] E
  static constexpr int oV = oKbT + DK * LK * ES;             // [KP][LV] E (rows >= BL stay 0)
  static constexpr int oA = oV + KP * LV * ES;               // [BL][LA] f32
  static constexpr int intra_bytes = oA + BL * LA * 4;
  static constexpr int oQd = intra_bytes;                    // [BL][LD] E
  static constexpr int oKdT = oQd + BL * LD * ES;            // [DK][LK] E
  static constexpr int oP = oKdT + DK * LK * ES;             // [BL][LK] E
  static constexpr int serial_bytes = oP + BL * LK * ES;
  static_assert(2 * BL * LD * ES >= BL * LT * 4, "T fits in the Qx/Ky region");
  static_assert(BL * LD * ES >= NB * 256 * 2 * 4, "fallback accumulators fit in Kx");
  static_assert(serial_bytes <= 160 * 1024, "LDS budget");
  static_assert(oKx % 16 == 0, "tile alignment");

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
  static constexpr int LD = LY::LD, LK = LY::LK, LV = LY::LV, LT = LY::LT, LA = LY::LA;

  struct Smem {
    unsigned char* base;
    E *Kx, *Qx, *Ky, *KbT, *V, *Qd, *KdT, *P, *W;
    float *T, *A, *Gb, *Seg, *Egl, *Wg, *Z, *M, *Y;
    int* Flag;
  };

  __device__ static Smem carve(unsigned char* smem) {
    Smem s;
    s.base = smem;
    s.Kx = reinterpret_cast<E*>(smem + LY::oKx);
    s.W = s.Kx;                                        // chunk-serial: W reuses Kx
    s.Qx = reinterpret_cast<E*>(smem + LY::oQx);
    s.T = reinterpret_cast<float*>(smem + LY::oQx);    // T reuses Qx/Ky after the Grams
    s.Ky = reinterpret_cast<E*>(smem + LY::oKy);
    s.KbT = reinterpret_cast<E*>(smem + LY::oKbT);
    s.V = reinterpret_cast<E*>(smem + LY::oV);
    s.A = reinterpret_cast<float*>(smem + LY::oA);
    s.Qd = reinterpret_cast<E*>(smem + LY::oQd);
    s.KdT = reinterpret_cast<E*>(smem + LY::oKdT);
    s.P = reinterpret_cast<E*>(smem + LY::oP);
    s.Gb = reinterpret_cast<float*>(smem + LY::oGb);
    s.Seg = reinterpret_cast<float*>(smem + LY::oSeg);
    s.Egl = reinterpret_cast<float*>(smem + LY::oEgl);
    s.Wg = reinterpret_cast<float*>(smem + LY::oWg);
    s.Z = reinterpret_cast<float*>(smem + LY::oZ);
    s.M = reinterpret_cast<float*>(smem + LY::oM);
    s.Y = reinterpret_cast<float*>(smem + LY::oY);
    s.Flag = reinterpret_cast<int*>(smem + LY::oFlag);
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
    const int gs = tid / DK, gd = tid % DK;
    if (tid == 0) s.Flag[0] = 0;
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
      f32x4 vc[(NCH + NT - 1) / NT];
#pragma unroll
      for (int j = 0; j < (NCH + NT - 1) / NT; ++j) {
        const int c = threadIdx.x + j * NT;
        if (c < NCH) {
          const int r = c / CPR, cc = c % CPR;
          const int rc = min(r, nvalid - 1);
          vc[j] = *reinterpret_cast<const f32x4*>(src.V + src.row(t0 + rc) * DV + cc * (16 / LY::ES));
          if (r >= nvalid) vc[j] = zero4();
        }
      }
#pragma unroll
      for (int j = 0; j < (NCH + NT - 1) / NT; ++j) {
        const int c = threadIdx.x + j * NT;
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
      s.Gb[gs * DK + gd] = Gs;
      if (gs == NB - 1) {
        s.Gb[NB * DK + gd] = total;
        s.Egl[gd] = fast_exp2(total);
      }
      if (Gs - Ge > kSpanLimit2) atomicOr(s.Flag, 1);
      const float eGs = fast_exp2(Gs);
      const float eTail = fast_exp2(total - Ge);
      const float z = s.Z[gd];
      float eprev = 1.f;                             // e^{G_{r-1} - Gs}
      E kb[16], kd[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * gs + i;
        const float Gr = base + gv[i];
        const float bb = sigmoid_f(bv[i] + z);
        const float e1 = fast_exp2(Gr - Gs);         // <= 1
        const float en = fast_exp2(Ge - Gr);         // <= 1
        const float bk = bb * kv[i];
        s.Kx[r * LD + gd] = from_f32<E>(bk * e1);
        s.Qx[r * LD + gd] = from_f32<E>(qv[i] * eprev);
        s.Ky[r * LD + gd] = from_f32<E>(kv[i] * en);
        out.Qd[r * out.ldQd + gd] = from_f32<E>(qv[i] * eprev * eGs);
        kb[i] = from_f32<E>(bk * e1 * eGs);
        kd[i] = from_f32<E>(kv[i] * en * eTail);
        eprev = e1;
      }
      // transposed tiles: this thread's 16 rows are 16 consecutive elements
      E* kbt = s.KbT + gd * LK + 16 * gs;
      E* kdt = out.KdT + gd * out.ldKdT + 16 * gs;
#pragma unroll
      for (int c = 0; c < 16 * LY::ES / 16; ++c) {
        *reinterpret_cast<f32x4*>(kbt + c * (16 / LY::ES)) = *reinterpret_cast<const f32x4*>(kb + c * (16 / LY::ES));
        *reinterpret_cast<f32x4*>(kdt + c * (16 / LY::ES)) = *reinterpret_cast<const f32x4*>(kd + c * (16 / LY::ES));
      }
    }
    __syncthreads();
    return s.Flag[0] != 0;
  }

  // -------------------------------------------------------------- Grams A, P
  __device__ static void grams(const Smem& s, const Rows<E>& src, int t0, int nvalid, bool fallback,
                               const Sink<E>& out) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gq = lane >> 4, cc = lane & 15;
    constexpr int NPAIR = NB * (NB + 1) / 2;
    for (int pr = wave; pr < NPAIR; pr += NW) {
      int I = 0, J = pr;
      while (J > I) { J -= I + 1; ++I; }
      const bool diag = (I == J);
      f32x4 accA = zero4(), accP = zero4();
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) {
        Frag ka = MM::ld_nat(s.Kx, LD, 16 * I + cc, p * KS);
        Frag qa = MM::ld_nat(s.Qx, LD, 16 * I + cc, p * KS);
        Frag kb = MM::ld_nat(s.Ky, LD, 16 * J + cc, p * KS);
        if constexpr (KS == 32) {
#pragma unroll
          for (int sl = 0; sl < 8; ++sl) {
            const int kk = p * KS + 8 * gq + sl;
            if (J < I - 1) {                          // left factor e^{Gs_I - Ge_J}
              const float f = fast_exp2(s.Gb[I * DK + kk] - s.Gb[(J + 1) * DK + kk]);
              ka[sl] = (bf16)((float)ka[sl] * f);
              qa[sl] = (bf16)((float)qa[sl] * f);
            }
            if (diag)                                 // right factor e^{Gs_J - Ge_J}
              kb[sl] = (bf16)((float)kb[sl] * fast_exp2(s.Gb[J * DK + kk] - s.Gb[(J + 1) * DK + kk]));
          }
        } else {
          const int kk = p * KS + gq;
          if (J < I - 1) {
            const float f = fast_exp2(s.Gb[I * DK + kk] - s.Gb[(J + 1) * DK + kk]);
            ka = ka * f;
            qa = qa * f;
          }
          if (diag) kb = kb * fast_exp2(s.Gb[J * DK + kk] - s.Gb[(J + 1) * DK + kk]);
        }
        accA = MM::mma(ka, kb, accA);
        accP = MM::mma(qa, kb, accP);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * I + 4 * gq + i, j = 16 * J + cc;
        const bool keep = !diag || (j < r);
        s.A[r * LA + j] = keep ? accA[i] : 0.f;
        out.P[r * out.ldP + j] = from_f32<E>(keep ? accP[i] : 0.f);
      }
    }
    // P blocks above the diagonal and the padding columns are zero
    for (int idx = tid; idx < BL * KP; idx += NT) {
      const int r = idx / KP, j = idx % KP;
      if (j >= 16 * (r / 16 + 1)) out.P[r * out.ldP + j] = from_f32<E>(0.f);
    }
    __syncthreads();
    if (fallback) grams_pairwise(s, src, t0, nvalid, out);
  }

  // Diagonal sub-blocks rebuilt pairwise from the raw gates: only for decays
  // too steep for the factorised form; slow but exact.
  __device__ static void grams_pairwise(const Smem& s, const Rows<E>& src, int t0, int nvalid,
                                        const Sink<E>& out) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int gs = tid / DK, gd = tid % DK;
    float* accA = reinterpret_cast<float*>(s.base + LY::oKx);       // [NB][16][16]
    float* accP = accA + NB * 256;
    for (int i = tid; i < NB * 512; i += NT) accA[i] = 0.f;
    __syncthreads();
    if (gs < NB) {
      const float z = s.Z[gd];
      auto off_of = [&](int r) { return src.row(t0 + r) * DK + gd; };
      float* Gloc = reinterpret_cast<float*>(s.base + LY::oQx) + gd;  // dead Qx region
      float run = 0.f;
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * gs + i;
        run += (r < nvalid) ? ldg(src.G, off_of(r)) * kLog2e : 0.f;
        Gloc[(16 * gs + i) * DK] = run;
      }
      for (int ri = 1; ri < 16; ++ri) {
        const int r = 16 * gs + ri;
        float kr = 0.f, qr = 0.f, br = 0.f;
        if (r < nvalid) {
          kr = ldg(src.K, off_of(r));
          qr = ldg(src.Q, off_of(r));
          br = sigmoid_f(ldg(src.BX, off_of(r)) + z);
        }
        for (int ji = 0; ji < ri; ++ji) {
          const int j = 16 * gs + ji;
          const float kj = (j < nvalid) ? ldg(src.K, off_of(j)) : 0.f;
          const float Gr = Gloc[(16 * gs + ri) * DK], Gj = Gloc[(16 * gs + ji) * DK];
          const float Gp = Gloc[(16 * gs + ri - 1) * DK];
          float ca = br * kr * kj * fast_exp2(Gr - Gj);
          float cp = qr * kj * fast_exp2(Gp - Gj);
          for (int off = 32; off >= 1; off >>= 1) {
            ca += __shfl_xor(ca, off);
            cp += __shfl_xor(cp, off);
          }
          if (lane == 0) {
            atomicAdd(&accA[gs * 256 + ri * 16 + ji], ca);
            atomicAdd(&accP[gs * 256 + ri * 16 + ji], cp);
          }
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < NB * 256; i += NT) {
      const int sb = i / 256, ri = (i / 16) % 16, ji = i % 16;
      const int r = 16 * sb + ri, j = 16 * sb + ji;
      s.A[r * LA + j] = (ji < ri) ? accA[i] : 0.f;
      out.P[r * out.ldP + j] = from_f32<E>((ji < ri) ? accP[i] : 0.f);
    }
    __syncthreads();
  }

  // -------------------------------------------------------------- T = (I + A)^{-1}
  __device__ static void inverse(const Smem& s) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gq = lane >> 4, cc = lane & 15;
    // diagonal 16x16 blocks by forward substitution (fp32): wave 0, lane
    // (block ib = gq, column c = cc) keeps its whole column in registers
    if (wave == 0) {
      const int ib = gq, c = cc;
      if (ib < NB) {
        const float* Ablk = s.A + (16 * ib) * LA + 16 * ib;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < r; ++j) acc += Ablk[r * LA + j] * t[j];
          t[r] = (r == c) ? 1.f : ((r > c) ? -acc : 0.f);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s.T[(16 * ib + r) * LT + 16 * ib + c] = t[r];
      }
    }
    // zero every row block right of its diagonal block (upper blocks, padding)
    for (int idx = tid; idx < BL * KP; idx += NT) {
      const int r = idx / KP, j = idx % KP;
      if (j >= 16 * (r / 16 + 1)) s.T[r * LT + j] = 0.f;
    }
    __syncthreads();
    // off-diagonal blocks: wave J walks its block column downwards,
    // T_IJ = -T_II sum_{J<=K<I} A_IK T_KJ, keeping T_KJ as C tiles
    if (NB > 1 && wave < NB - 1) {
      const int J = wave;
      f32x4 Tc[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) Tc[I] = zero4();
#pragma unroll
      for (int I = 0; I < NB; ++I)
        if (I == J)
#pragma unroll
          for (int i = 0; i < 4; ++i) Tc[I][i] = s.T[(16 * J + 4 * gq + i) * LT + 16 * J + cc];
#pragma unroll
      for (int I = 1; I < NB; ++I) {
        if (I <= J) continue;
        f32x4 X = zero4();
#pragma unroll
        for (int Kb = 0; Kb < NB; ++Kb)
          if (Kb >= J && Kb < I) X = Mma16<E>::mma_rowA_cB(s.A, LA, 16 * I + cc, 16 * Kb, Tc[Kb], X, 1.f);
        Tc[I] = Mma16<E>::mma_rowA_cB(s.T, LT, 16 * I + cc, 16 * I, X, zero4(), -1.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) s.T[(16 * I + 4 * gq + i) * LT + 16 * J + cc] = Tc[I][i];
      }
    }
    __syncthreads();
  }

  // -------------------------------------------------------------- W = T (b k e^{G})
  // Ends with a barrier.
  __device__ static void build_w(const Smem& s, const Sink<E>& out) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gq = lane >> 4, cc = lane & 15;
    constexpr int NTILE = NB * (DK / 16);
    for (int tt = wave; tt < NTILE; tt += NW) {
      const int I = tt / (DK / 16), dt = tt % (DK / 16);
      f32x4 acc = zero4();
      const int nst = MM::steps(16 * (I + 1));
      for (int p = 0; p < nst; ++p)
        acc = MM::mma(MM::ld_nat(s.T, LT, 16 * I + cc, p * KS), MM::ld_nat(s.KbT, LK, 16 * dt + cc, p * KS), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) out.W[(16 * I + 4 * gq + i) * out.ldW + 16 * dt + cc] = from_f32<E>(acc[i]);
    }
    __syncthreads();
  }

  // -------------------------------------------------------------- U = T diag(w) V
  // Per wave, channels [16 wave, 16 wave + 16); values rounded to E so every
  // schedule feeds the state pass identical operands. The value operand is
  // gathered from the row-major V tile with the c-pair map.
  __device__ static void build_u(const Smem& s, f32x4 (&U)[NB]) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
    const int e0 = 16 * wave;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      f32x4 u = zero4();
#pragma unroll
      for (int p = 0; p < MM::steps(BL); ++p) {
        if (p >= MM::steps(16 * (rt + 1))) break;
        Frag ta, vb;
        if constexpr (KS == 32) {
          const float* tr = s.T + (16 * rt + cc) * LT + 32 * p + 4 * gq;
          const f32x4 t0 = *reinterpret_cast<const f32x4*>(tr);
          const f32x4 t1 = *reinterpret_cast<const f32x4*>(tr + 16);
          const float* wg = s.Wg + 32 * p + 4 * gq;
          const f32x4 w0 = *reinterpret_cast<const f32x4*>(wg);
          const f32x4 w1 = *reinterpret_cast<const f32x4*>(wg + 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ta[i] = (bf16)(t0[i] * w0[i]);
            ta[4 + i] = (bf16)(t1[i] * w1[i]);
            vb[i] = s.V[(32 * p + 4 * gq + i) * LV + e0 + cc];
            vb[4 + i] = s.V[(32 * p + 16 + 4 * gq + i) * LV + e0 + cc];
          }
        } else {
          const int k = 16 * (p >> 2) + 4 * gq + (p & 3);
          ta = s.T[(16 * rt + cc) * LT + k] * s.Wg[k];
          vb = s.V[k * LV + e0 + cc];
        }
        u = MM::mma(ta, vb, u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = to_f32(from_f32<E>(u[i]));
      U[rt] = u;
    }
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
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      if (S) St[dt] = *reinterpret_cast<const f32x4*>(S + ((size_t)bh * DV + 16 * wave + cc) * DK + 16 * dt + 4 * gq);
      else St[dt] = zero4();
    }
  }
  __device__ static void store_state(float* S, int bh, const f32x4 (&St)[DK / 16]) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
      *reinterpret_cast<f32x4*>(S + ((size_t)bh * DV + 16 * wave + cc) * DK + 16 * dt + 4 * gq) = St[dt];
  }
};

}  // namespace carve
