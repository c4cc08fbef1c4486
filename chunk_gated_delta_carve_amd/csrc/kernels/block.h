// Per-block operations of the CARVE WY chunk solver, shared by every kernel.
//
// A block is BL consecutive tokens (BL in {16, 32, 64}) of one (batch, head).
// With S the state at the block start, G_r the inclusive cumulative log-decay
// inside the block (G_{-1} = 0), b_r = sigmoid(bx_r + z) and z = U_b m_{c-1}
// (gist.science technical summary, §2.1 "Content-Aware Erase via Output
// Reuse"; §2.2 scalar write gate; §2.3 key-axis decay, whose activation
// g = -softplus(a) of raw logits a the kLogits variants apply as they read g):
//   A_rj  = sum_d b_r k_r k_j e^{G_r - G_j}          (j < r)
//   P_rj  = sum_d q_r k_j e^{G_{r-1} - G_j}          (j < r)
//   [W | U] = (I + A)^{-1} [b k e^{G_r} | w v]       (WY form)
//   Delta = U - W S^T
//   O     = (q e^{G_{r-1}}) S^T + P Delta           (o_t = S_{t-1} q_t)
//   S    <- S diag(e^{G_BL}) + Delta^T Kdec,  Kdec_j = k_j e^{G_BL - G_j}
// This is exact algebra for the token recurrence S <- S D (I - (b k) k^T) +
// w v k^T; one triangular system per block exists because every gate acts on
// the key axis (Theorem 11, §3 of the same summary).
//
// The state pass only needs the block's affine map S <- S M + C and the
// output map O = Qe S^T + Ol, with
//   M  = diag(e^{G_BL}) - W^T Kdec    C  = U^T Kdec
//   Qe = Qd - P W                     Ol = P U          (Qd_r = q_r e^{G_{r-1}})
// so each block hands M^T, C^T, Qe and Ol to the state pass.
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
#include <type_traits>

#include "common.h"

namespace carve {

struct FwdArgs {
  const void* q; const void* k; const void* v; const void* g; const void* bx; const void* w;
  const void* ub_down; const void* ub_up;
  const float* state_in; const float* mean_in;
  void* o; float* state_out; float* mean_out;
  void* ws;
  int B, H, T, L, rank;
  // the state pass's checkpointing variant only: fp32 state [dv][dk] at the
  // start of every (1 << ckpt_shift)-th block, the k-th at
  // ckpt + bh ckpt_bh + k dv dk
  float* ckpt; size_t ckpt_bh; int ckpt_shift;
  // the chunk-serial kernel's checkpointing variant: at every chunk start c
  // also the gate's bias z [dk] at ckpt + bh ckpt_bh + ckpt_z + c dk and the
  // mean it was formed from, m_{c-1} [dv], at ... + ckpt_m + c dv
  size_t ckpt_z, ckpt_m;
};

constexpr float kSpanLimit2 = 96.0f;   // max decay (log2 units) inside a 16-row sub-block

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// WV is the number of waves of a workgroup that runs the per-block stages;
// by default one per 16-channel value slice. With more waves than slices,
// every stage splits its work further (the chunk-parallel intra kernel does
// that to shorten the latency of one block).
template <typename E, int DK, int DV, int BL, int WV = DV / 16>
struct BlockLayout {
  static_assert(DK % 32 == 0 && DV % 16 == 0 && DK == DV, "head widths");
  static_assert(BL == 16 || BL == 32 || BL == 64, "block length");
  static constexpr int NW = DV / 16;                 // 16-channel value slices
  static constexpr int NWV = WV;                     // waves
  static constexpr int NT = NWV * 64;
  static constexpr int PARTS = NWV / NW;             // waves per value slice in the affine stage
  static_assert(NWV % NW == 0, "whole value slices per wave group");
  static constexpr int NB = BL / 16;
  static constexpr int KP = BL < 32 ? 32 : BL;       // padded token-reduction width
  // Gate pass: a lane holds RPL consecutive rows of 4 key channels; a wave
  // covers one segment of SR = 4 RPL rows and 64 channels; a 16-row sub-block
  // has SPS segments (NSEG in the block).
  static constexpr int RPL = BL * DK / (4 * NT) < 1 ? 1 : (BL * DK / (4 * NT) > 4 ? 4 : BL * DK / (4 * NT));
  static constexpr int SR = 4 * RPL;
  static constexpr int SPS = 16 / SR;
  static constexpr int NSEG = BL / SR;
  static_assert(BL * DK == 4 * RPL * NT || NSEG * (DK / 64) <= NWV, "gate pass lanes");
  static_assert(NSEG * (DK / 64) <= NWV, "one wave per gate segment");
  static constexpr int ES = sizeof(E);
  static constexpr int PE = 16 / ES;                 // 16-byte row padding, in elements
  static constexpr int LD = DK + PE;                 // pitch of [.][DK] tiles
  static constexpr int LK = KP + PE;                 // pitch of [.][KP] tiles
  static constexpr int LV = DV + PE;                 // pitch of [.][DV] tiles
  static constexpr int LA = BL + 4;                  // pitch of A (fp32)
  static constexpr int LAE = LA * 4 / ES;            // the same rows as E: off-diagonal tiles of -A
  static constexpr int LTD = 16 + PE;                // pitch of the diagonal inverses (E)
  static constexpr int NFAR = NB > 2 ? (NB - 1) * (NB - 2) / 2 : 1;   // sub-block pairs J < I-1

  // ---- LDS. Persistent small arrays, then regions whose contents change
  // once their first occupant is dead:
  //   RB: Seg, Fd, Ff (gate pass -> Grams), then Td (inverse -> solve)
  //   R1: Kx (gate -> solve), then Wt = W^T (solve -> affine)
  //   R2: Qx, Ky (gate -> Grams), then A (Grams -> solve), then Qd, P (-> affine)
  //   R3: V (gate -> solve), then Ut = U^T (solve -> affine)
  //   R4: KdT = Kdec^T (gate -> affine)
  // The chunk-serial kernel also keeps Mt and Qe (C^T and Ol stay in the
  // registers of the wave that owns their value channels).
  static constexpr int oEgl = 0;                             // [DK] f32 e^{G_BL}
  static constexpr int oEGs = oEgl + DK * 4;                 // [NB][DK] f32 e^{Gs_I}
  static constexpr int oWg = oEGs + NB * DK * 4;             // [KP] f32 write gate (zero padded)
  static constexpr int oZ = oWg + KP * 4;                    // [DK] f32
  static constexpr int oM = oZ + DK * 4;                     // [DV] f32
  static constexpr int oY = oM + DV * 4;                     // [64] f32
  static constexpr int oFlag = oY + 64 * 4;                  // int
  static constexpr int oRB = oFlag + 16;
  static constexpr int oSeg = oRB;                           // [NSEG][DK] f32
  static constexpr int oFd = oSeg + NSEG * DK * 4;           // [NB][DK] f32 e^{Gs_J - Ge_J}
  static constexpr int oFf = oFd + NB * DK * 4;              // [NFAR][DK] f32 e^{Gs_I - Ge_J}
  static constexpr int oTd = oRB;                            // [NB][16][LTD] E
  static constexpr int szRB = cmax((NSEG + NB + NFAR) * DK * 4, NB * 16 * LTD * ES);
  static constexpr int oR1 = oRB + (szRB + 15) / 16 * 16;
  static constexpr int szR1 = cmax(BL * LD * ES, DK * LK * ES);
  static constexpr int oR2 = oR1 + szR1;
  static constexpr int szR2 = cmax(cmax(2 * BL * LD * ES, BL * LA * 4), BL * LD * ES + BL * LK * ES);
  static constexpr int oR3 = oR2 + szR2;
  static constexpr int szR3 = cmax(KP * LV * ES, DV * LK * ES);
  static constexpr int oR4 = oR3 + szR3;
  static constexpr int intra_bytes = oR4 + DK * LK * ES;
  static constexpr int oKx = oR1, oWt = oR1;
  static constexpr int oQx = oR2, oKy = oR2 + BL * LD * ES, oA = oR2;
  static constexpr int oQd = oR2, oP = oR2 + BL * LD * ES;
  static constexpr int oV = oR3, oUt = oR3;                  // V is [KP][LV] (rows >= BL stay 0)
  static constexpr int oKdT = oR4;
  // Mt and Qe as fragment units (see below), chunk-serial kernel only
  static constexpr int TD = DK / 16;
  static constexpr int NU = DK * ES / 64;                    // units per 16-row tile along d
  static constexpr int oMt = intra_bytes;                    // [TD][NU][64] units
  static constexpr int oQe = oMt + DK * DK * ES;             // [NB][NU][64] units
  // chunk-serial kernel with PARTS > 1 waves per value slice: the S operand
  // fragments of every slice, double-buffered by block parity, and the
  // parts' sums for the chunk mean
  static constexpr int NFR = DK / (ES == 2 ? 32 : 4);         // operand fragments of S along d
  static constexpr int FRB = ES == 2 ? 16 : 4;                // bytes per lane of one fragment
  static constexpr int oXc = oQe + BL * DK * ES;             // [2][NW][NFR][64] fragments
  static constexpr int szXc = PARTS > 1 ? 2 * NW * NFR * 64 * FRB : 0;
  static constexpr int oMp = oXc + szXc;                     // [PARTS][DV] f32
  static constexpr int oYp = oMp + (PARTS > 1 ? PARTS * DV * 4 : 0);   // [64][NWV] f32 partial sums of U_down m
  // Lean chunk-serial blocks (bf16, d = 64, 64-token blocks, eight waves):
  // the triangular system's operands in areas of their own
  static constexpr bool kLean = ES == 2 && DK == 64 && DV == 64 && BL == 64 && NWV == 8;
  static constexpr int oLP = oYp + 64 * NWV * 4;             // [BL][LK] E: P
  static constexpr int oLQd = oLP + BL * LK * ES;            // [BL][LD] E: Q_dec
  static constexpr int oLAn = oLQd + BL * LD * ES;           // [BL][LK] E: -A_IJ, J < I
  static constexpr int oLTd = oLAn + BL * LK * ES;           // [NB][16][LTD] E: T_II
  static constexpr int oLCx = oLTd + NB * 16 * LTD * ES;     // [NW][TD/2 + NB/2][64] 8-byte C tiles
  static constexpr int oLXm = oLCx + NW * (TD / 2 + NB / 2) * 64 * 8;   // [NW][64] f32x4 mean partials
  static constexpr int lean_bytes = oLXm + NW * 64 * 16;
  static constexpr int serial_bytes = kLean ? lean_bytes : oYp + 64 * NWV * 4;
  static_assert(serial_bytes <= 160 * 1024, "LDS budget");
  static_assert(oR1 % 16 == 0 && oR2 % 16 == 0 && oR3 % 16 == 0 && oR4 % 16 == 0 && oMt % 16 == 0, "alignment");
  static_assert(oLP % 16 == 0 && oLQd % 16 == 0 && oLAn % 16 == 0 && oLTd % 16 == 0 && oLCx % 16 == 0 &&
                oLXm % 16 == 0, "alignment");
  static_assert(NB * 256 * 4 <= DK * LK * ES, "pairwise scratch fits in R4");

  // ---- image of one block's state-pass operands (workspace), every part in
  // the order in which a wave holds it, so each lane's share is contiguous:
  //   Mt units [TD][NU][64 lanes][16 B]: A operands of M^T (rows d', k = d)
  //   Qe units [NB][NU][64 lanes][16 B]: B operands of Qe^T (k = d, cols t)
  //   Ct  [NW][TD/2][64 lanes][2][4] E: C tiles of C^T (rows d', cols e)
  //       per 16-channel value slice, two tiles side by side per lane
  //   Olt [NW][NB/2][64 lanes][2][4] E: C tiles of Ol^T (rows e, cols t),
  //       per slice, paired the same way
  static constexpr int wMt = 0;
  static constexpr int wQe = wMt + DK * DK * ES;
  static constexpr int wCt = wQe + BL * DK * ES;
  static constexpr int wOl = wCt + NW * TD * 256 * ES;
  static constexpr int wBytes = wOl + NW * NB * 256 * ES;
  static_assert(wBytes % 16 == 0, "16-byte units");
  static_assert(TD % 2 == 0 && (BL < 32 || NB % 2 == 0), "C tiles pair up");
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

// Where affine() puts a block's shared affine maps, as fragment units (LDS of
// the chunk-serial kernel). C^T and Ol^T stay in the registers of the waves
// that own their value channels. (The chunk-parallel intra kernel writes all
// four straight to its workspace image instead: image_from_x.)
template <typename E>
struct Sink {
  typename Mma<E>::unit* Mt;   // [TD][NU][64]
  typename Mma<E>::unit* Qe;   // [NB][NU][64]
};

template <typename E, int DK, int DV, int BL, int WV = DV / 16>
struct Block {
  using LY = BlockLayout<E, DK, DV, BL, WV>;
  using MM = Mma<E>;
  using Frag = typename MM::frag;
  using Unit = typename MM::unit;
  typedef E e4 __attribute__((ext_vector_type(4)));
  static constexpr int NW = LY::NW, NWV = LY::NWV, NT = LY::NT, NB = LY::NB, KP = LY::KP, KS = MM::KS;
  static constexpr int PARTS = LY::PARTS, CTP = LY::TD / PARTS, OLP = NB / PARTS;   // affine tiles per wave
  static constexpr int TD = LY::TD, NU = LY::NU, SPU = MM::SPU, UT = MM::UT;
  static constexpr int LD = LY::LD, LK = LY::LK, LV = LY::LV, LA = LY::LA, LAE = LY::LAE, LTD = LY::LTD;
  // Lower-triangular 16x16 tiles (I, J), J <= I, of the Grams, dealt to the
  // waves in the order: diagonal tiles, adjacent pairs (I = J + 1), then the
  // far pairs by growing distance. Tile t goes to wave t mod NWV as its
  // (t / NWV)-th tile; the kinds are spread evenly that way.
  static constexpr int NTILE = NB * (NB + 1) / 2;
  static constexpr int TPW = (NTILE + NWV - 1) / NWV;      // Gram tiles per wave
  __device__ __forceinline__ static bool gram_tile(int wave, int k, int& I, int& J) {
    int t = wave + k * NWV;
    if (t >= NTILE) return false;
    if (t < NB) { I = J = t; return true; }
    t -= NB;
    for (int dist = 1; dist < NB; ++dist) {
      if (t < NB - dist) { J = t; I = t + dist; return true; }
      t -= NB - dist;
    }
    return false;
  }

  struct Smem {
    unsigned char* base;
    E *Kx, *Qx, *Ky, *V, *Td, *Wt, *Ut, *Qd, *P, *KdT, *Mt, *Qe, *An;
    float *A, *Seg, *Egl, *EGs, *Wg, *Z, *M, *Y, *Fd, *Ff;
    int* Flag;
  };

  __device__ static Smem carve(unsigned char* smem) {
    Smem s;
    s.base = smem;
    auto e = [&](int o) { return reinterpret_cast<E*>(smem + o); };
    auto f = [&](int o) { return reinterpret_cast<float*>(smem + o); };
    s.Kx = e(LY::oKx); s.Qx = e(LY::oQx); s.Ky = e(LY::oKy); s.V = e(LY::oV); s.Td = e(LY::oTd);
    s.Wt = e(LY::oWt); s.Ut = e(LY::oUt); s.Qd = e(LY::oQd); s.P = e(LY::oP); s.KdT = e(LY::oKdT);
    s.Mt = e(LY::oMt); s.Qe = e(LY::oQe); s.An = e(LY::oA);
    s.A = f(LY::oA); s.Seg = f(LY::oSeg); s.Egl = f(LY::oEgl); s.EGs = f(LY::oEGs);
    s.Wg = f(LY::oWg); s.Z = f(LY::oZ); s.M = f(LY::oM); s.Y = f(LY::oY); s.Fd = f(LY::oFd);
    s.Ff = f(LY::oFf);
    s.Flag = reinterpret_cast<int*>(smem + LY::oFlag);
    return s;
  }

  __device__ static Sink<E> lds_sink(const Smem& s) {
    return Sink<E>{reinterpret_cast<Unit*>(s.Mt), reinterpret_cast<Unit*>(s.Qe)};
  }
  // two C tiles of a lane side by side, as the image holds C^T and Ol^T
  // (16 bytes per lane for bf16)
  typedef E e8 __attribute__((ext_vector_type(8)));
  __device__ static e8 pair(f32x4 x, f32x4 y) {
    return e8{from_f32<E>(x[0]), from_f32<E>(x[1]), from_f32<E>(x[2]), from_f32<E>(x[3]),
              from_f32<E>(y[0]), from_f32<E>(y[1]), from_f32<E>(y[2]), from_f32<E>(y[3])};
  }

  __device__ static void zero_lds(unsigned char* smem, int bytes) {
    for (int i = threadIdx.x; i < bytes / 4; i += NT) reinterpret_cast<float*>(smem)[i] = 0.f;
  }

  // -------------------------------------------------------------- gate pass
  // Thread roles: wave w covers gate segment seg = w / (DK/64) (SR = 4 RPL
  // consecutive rows; SPS segments per 16-row sub-block) and key channels
  // 64 (w mod DK/64) .. +63; lane (qr = l / 16, dq = l % 16) holds rows
  // r0 .. r0 + RPL - 1 (r0 = SR seg + RPL qr) of channels d0 .. d0 + 3
  // (d0 = 64 (w mod DK/64) + 4 dq). Each row segment of a lane is one 8-byte
  // (bf16) or 16-byte (fp32) load.
  static constexpr int RPL = LY::RPL, SR = LY::SR, SPS = LY::SPS, NSEG = LY::NSEG;
  struct GateCoord {
    int seg, gs, r0, d0, qr;
    __device__ GateCoord() {
      const int wave = wave_id(), lane = threadIdx.x & 63;
      seg = wave / (DK / 64);
      gs = seg / SPS;
      qr = lane >> 4;
      r0 = SR * seg + RPL * qr;
      d0 = (wave % (DK / 64)) * 64 + 4 * (lane & 15);
    }
    __device__ bool active() const { return seg < NSEG; }
  };

  // Raw token inputs of one block for this thread, straight from global
  // memory. Loading is split from the gate arithmetic so a kernel can fetch
  // the next block while it works on the current one. Rows past nvalid are
  // clamped to the last valid row here and masked in gate_pass.
  struct Raw {
    static constexpr int CPR = DV * LY::ES / 16;         // 16-byte chunks per value row
    static constexpr int NCH = BL * CPR;
    static constexpr int VPER = (NCH + NT - 1) / NT;
    e4 q[RPL], k[RPL], g[RPL], bx[RPL];
    // with q, k normalisation at d_k = 128: this lane's rows at the channels
    // 64 away (held by the partner wave), so each row's norm is one 16-lane sum
    e4 qo[DK == 128 ? RPL : 1], ko[DK == 128 ? RPL : 1];
    f32x4 v[VPER];
    E w;
    // Addresses are a block-uniform base per tensor plus a 32-bit per-lane
    // byte offset (rows of a block lie within 64 H d elements; the host
    // keeps that below 2^32 bytes), shared by the four [., d_k] tensors.
    template <bool kNorm = false>
    __device__ void load(const Rows<E>& src, int t0, int nvalid) {
      const GateCoord gc;
      const int tid = threadIdx.x;
      const size_t r0 = src.row(t0);                       // uniform
      const uint32_t hk = (uint32_t)src.H * DK, hv = (uint32_t)src.H * DV;
      auto at = [](const E* base, uint32_t bytes) {
        return reinterpret_cast<const unsigned char*>(base) + bytes;
      };
      if (gc.active()) {
        const E *Qb = src.Q + r0 * DK, *Kb = src.K + r0 * DK, *Gb = src.G + r0 * DK, *Bb = src.BX + r0 * DK;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
          const uint32_t off = ((uint32_t)min(gc.r0 + i, nvalid - 1) * hk + gc.d0) * (uint32_t)sizeof(E);
          // read once: streaming (non-temporal) loads, so that they do not
          // push the workspace images out of the caches (with d_k = 128 and
          // normalisation the partner wave reads q, k rows a second time)
          if constexpr (kNorm && DK == 128) {
            q[i] = *reinterpret_cast<const e4*>(at(Qb, off));
            k[i] = *reinterpret_cast<const e4*>(at(Kb, off));
          } else {
            q[i] = __builtin_nontemporal_load(reinterpret_cast<const e4*>(at(Qb, off)));
            k[i] = __builtin_nontemporal_load(reinterpret_cast<const e4*>(at(Kb, off)));
          }
          g[i] = __builtin_nontemporal_load(reinterpret_cast<const e4*>(at(Gb, off)));
          bx[i] = __builtin_nontemporal_load(reinterpret_cast<const e4*>(at(Bb, off)));
          if constexpr (kNorm && DK == 128) {
            const uint32_t offo = ((uint32_t)min(gc.r0 + i, nvalid - 1) * hk + (gc.d0 ^ 64)) * (uint32_t)sizeof(E);
            qo[i] = *reinterpret_cast<const e4*>(at(Qb, offo));
            ko[i] = *reinterpret_cast<const e4*>(at(Kb, offo));
          }
        }
      }
      const E* Vb = src.V + r0 * DV;
#pragma unroll
      for (int j = 0; j < VPER; ++j) {
        const int c = tid + j * NT;
        if (c < NCH) {
          const int r = c / CPR, cc = c % CPR;
          const uint32_t off = ((uint32_t)min(r, nvalid - 1) * hv + cc * (16 / LY::ES)) * (uint32_t)sizeof(E);
          v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(at(Vb, off)));
        }
      }
      if (tid < BL) w = __builtin_nontemporal_load(src.W + r0 + (size_t)min(tid, nvalid - 1) * src.H);
    }
  };

  // Builds every decay-scaled operand of the block from the raw inputs.
  // G is the inclusive cumulative log-decay (log2 units): within a lane over
  // its RPL rows, then across the 4 row quarters of the segment with lane
  // shuffles, then across segments through LDS. Rows past nvalid act as
  // k = q = v = w = g = 0, which leaves the state untouched. qd (Qd values,
  // element 4i + j = row r0 + i, channel d0 + j) stays in registers until
  // the Qx/Ky region is free again. Returns true if a sub-block's decay is too
  // steep for the factorised diagonal Grams. Ends with a barrier.
  // kContent: the erase logits carry the content bias z from s.Z; without a
  // content projection z = 0 and s.Z is not read here. kLogits: the decay
  // input holds raw logits a and g = -softplus(a). kNorm: q and k are used
  // per token divided by their L2 norms over d_k (max(|x|, 1e-12)).
  template <bool kContent = true, bool kLogits = false, bool kNorm = false>
  __device__ static bool gate_pass(const Smem& s, const Raw& raw, int nvalid, E (&qd)[16]) {
    const GateCoord gc;
    const int tid = threadIdx.x;
    const int sg = gc.seg, gs = gc.gs, r0 = gc.r0, d0 = gc.d0, qr = gc.qr;
    if (tid == 0) s.Flag[0] = 0;
#pragma unroll
    for (int j = 0; j < Raw::VPER; ++j) {
      const int c = tid + j * NT;
      if (c < Raw::NCH) {
        const int r = c / Raw::CPR, cc = c % Raw::CPR;
        *reinterpret_cast<f32x4*>(s.V + r * LV + cc * (16 / LY::ES)) = r < nvalid ? raw.v[j] : zero4();
      }
    }
    if (tid < BL) s.Wg[tid] = tid < nvalid ? to_f32(raw.w) : 0.f;
    float pre[RPL][4];                               // [row i][channel j]
    f32x4 excl = zero4();
    // k, q, g of this lane's rows; in a ragged last block the rows past
    // nvalid are zeroed here (the block-uniform branch skips this otherwise)
    e4 rk[RPL], rq[RPL], rg[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) { rk[i] = raw.k[i]; rq[i] = raw.q[i]; rg[i] = raw.g[i]; }
    if (nvalid < BL) {
#pragma unroll
      for (int i = 0; i < RPL; ++i)
        if (r0 + i >= nvalid) { rk[i] = e4{}; rq[i] = e4{}; rg[i] = e4{}; }
    }
    float ik[RPL], iq[RPL];                          // inverse norms of this lane's k, q rows
    if constexpr (kNorm) {
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float kv = to_f32(raw.k[i][j]), qv = to_f32(raw.q[i][j]);
          sk += kv * kv;
          sq += qv * qv;
          if constexpr (DK == 128) {
            const float ko = to_f32(raw.ko[i][j]), qo = to_f32(raw.qo[i][j]);
            sk += ko * ko;
            sq += qo * qo;
          }
        }
        ik[i] = inv_norm(sum_row16(sk));
        iq[i] = inv_norm(sum_row16(sq));
      }
    }
    if (gc.active()) {
      f32x4 run = zero4();
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // log-decay in log2 units; a zeroed logit is not a zero decay, so
          // with logits the padding rows are masked after the activation
          if constexpr (kLogits) run[j] += r0 + i < nvalid ? decay_log2<true>(to_f32(rg[i][j])) : 0.f;
          else run[j] += to_f32(rg[i][j]) * kLog2e;
          pre[i][j] = run[j];
        }
      }
      // exclusive prefix over the row quarters (lanes dq, dq + 16, dq + 32,
      // dq + 48) with cross-row lane swaps: the 16-lane swap gives each odd
      // row the total of the row below it and each row its pair's total; the
      // 32-lane swap gives rows 2 and 3 the total of rows 0 and 1
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned v = __float_as_uint(run[j]);
        const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        const float even = __uint_as_float(p16[0]), odd = __uint_as_float(p16[1]);
        const unsigned pair = __float_as_uint(even + odd);
        const float low = __uint_as_float(__builtin_amdgcn_permlane32_swap(pair, pair, false, false)[0]);
        excl[j] = qr == 0 ? 0.f : qr == 1 ? even : qr == 2 ? low : even + low;
      }
#pragma unroll
      for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) pre[i][j] += excl[j];   // G_r - G before the segment
      if (qr == 3)
        *reinterpret_cast<f32x4*>(s.Seg + sg * DK + d0) =
            f32x4{pre[RPL - 1][0], pre[RPL - 1][1], pre[RPL - 1][2], pre[RPL - 1][3]};
    }
    __syncthreads();
    if (gc.active()) {
      // Segment totals -> sub-block sums sb_I (segments added in order from
      // zero) -> prefix P_I = sb_0 + ... + sb_{I-1}, the log-decay before
      // sub-block I. Gs = P_gs, Ge = P_{gs+1} (so Ge of one sub-block is
      // exactly Gs of the next), total = P_NB. offs: the segments of this
      // sub-block before this one, added in the same order as sb, so the
      // last row of the sub-block reproduces sb_gs exactly.
      f32x4 sb[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        sb[I] = *reinterpret_cast<const f32x4*>(s.Seg + (I * SPS) * DK + d0);
#pragma unroll
        for (int t = 1; t < SPS; ++t) sb[I] += *reinterpret_cast<const f32x4*>(s.Seg + (I * SPS + t) * DK + d0);
      }
      f32x4 offs = zero4();
      if constexpr (SPS > 1) {
        const int first = gs * SPS;                  // wave-uniform
#pragma unroll
        for (int t = 0; t < SPS - 1; ++t)
          if (first + t < sg) offs += *reinterpret_cast<const f32x4*>(s.Seg + (first + t) * DK + d0);
      }
      // P_I for I <= NB; Gs/Ge picked by the wave-uniform gs
      f32x4 P[NB + 1];
      P[0] = zero4();
      P[1] = sb[0];
#pragma unroll
      for (int I = 1; I < NB; ++I) P[I + 1] = P[I] + sb[I];
      f32x4 Gs = P[0], seg = sb[0];
#pragma unroll
      for (int I = 1; I < NB; ++I)
        if (gs == I) { Gs = P[I]; seg = sb[I]; }
      const f32x4 Ge = Gs + seg;                     // = P[gs + 1], the same sum
      const f32x4 total = P[NB];
#pragma unroll
      for (int i = 0; i < RPL; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) pre[i][j] = offs[j] + pre[i][j];   // G_r - Gs
      f32x4 eGs, eTail;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        eGs[j] = fast_exp2(Gs[j]);
        eTail[j] = fast_exp2(total[j] - Ge[j]);
      }
      if (qr == 0 && sg == gs * SPS) {
        // per (sub-block, channel) tables: the first lane row of the sub-block
        *reinterpret_cast<f32x4*>(s.EGs + gs * DK + d0) = eGs;
        if (gs == NB - 1) {
          f32x4 egl;
#pragma unroll
          for (int j = 0; j < 4; ++j) egl[j] = fast_exp2(total[j]);
          *reinterpret_cast<f32x4*>(s.Egl + d0) = egl;
        }
        bool steep = false;
        f32x4 fd;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          steep |= Gs[j] - Ge[j] > kSpanLimit2;
          fd[j] = fast_exp2(Gs[j] - Ge[j]);
        }
        if (steep) atomicOr(s.Flag, 1);
        // Gram scaling factors: diagonal sub-block gs, and the pairs (I, gs)
        // with I > gs + 1
        *reinterpret_cast<f32x4*>(s.Fd + gs * DK + d0) = fd;
#pragma unroll
        for (int I = 2; I < NB; ++I) {
          if (I > gs + 1) {
            f32x4 ff;
#pragma unroll
            for (int j = 0; j < 4; ++j) ff[j] = fast_exp2(P[I][j] - Ge[j]);
            *reinterpret_cast<f32x4*>(s.Ff + ((I - 2) * (I - 1) / 2 + gs) * DK + d0) = ff;
          }
        }
      }
      const f32x4 z = kContent ? *reinterpret_cast<const f32x4*>(s.Z + d0) : zero4();
      float eprev[4];                                // e^{G_{r-1} - Gs}
#pragma unroll
      for (int j = 0; j < 4; ++j) eprev[j] = fast_exp2(offs[j] + excl[j]);
      E kd[4][RPL];                                  // [channel j][row i]
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        e4 kx, qx, ky;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float kvij = to_f32(rk[i][j]), qvij = to_f32(rq[i][j]);
          if constexpr (kNorm) {
            kvij *= ik[i];
            qvij *= iq[i];
          }
          const float bb = sigmoid_f(kContent ? to_f32(raw.bx[i][j]) + z[j] : to_f32(raw.bx[i][j]));
          const float e1 = fast_exp2(pre[i][j]);                     // e^{G_r - Gs} <= 1
          const float en = fast_exp2(seg[j] - pre[i][j]);            // e^{Ge - G_r} <= 1
          kx[j] = from_f32<E>(bb * kvij * e1);
          qx[j] = from_f32<E>(qvij * eprev[j]);
          ky[j] = from_f32<E>(kvij * en);
          qd[4 * i + j] = from_f32<E>(qvij * eprev[j] * eGs[j]);
          kd[j][i] = from_f32<E>(kvij * en * eTail[j]);
          eprev[j] = e1;
        }
        const int r = r0 + i;
        *reinterpret_cast<e4*>(s.Kx + r * LD + d0) = kx;
        *reinterpret_cast<e4*>(s.Qx + r * LD + d0) = qx;
        *reinterpret_cast<e4*>(s.Ky + r * LD + d0) = ky;
      }
      // Kdec transposed: RPL consecutive rows of each channel
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        E* dst = s.KdT + (d0 + j) * LK + r0;
        if constexpr (RPL == 4) {
          *reinterpret_cast<e4*>(dst) = e4{kd[j][0], kd[j][1], kd[j][2], kd[j][3]};
        } else if constexpr (RPL == 2) {
          typedef E e2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<e2*>(dst) = e2{kd[j][0], kd[j][1]};
        } else {
          dst[0] = kd[j][0];
        }
      }
    }
    __syncthreads();
    return s.Flag[0] != 0;
  }

  // -------------------------------------------------------------- Grams A, P
  // A (fp32) lands over the Qx/Ky region once every wave is done with them;
  // the P tiles of this wave stay in registers (Pt) until solve() frees the
  // region again. Ends with a barrier.
  template <bool kLogits = false, bool kNorm = false>
  __device__ static void grams(const Smem& s, const Rows<E>& src, int t0, int nvalid, bool fallback,
                               f32x4 (&Pt)[TPW]) {
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int gq = lane >> 4, cc = lane & 15;
    f32x4 accA[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      accA[k] = zero4();
      Pt[k] = zero4();
      int I, J;
      if (!gram_tile(wave, k, I, J)) continue;
      const bool diag = (I == J), far = (J < I - 1);
      Frag ka[DK / KS], qa[DK / KS], kb[DK / KS];
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) {
        ka[p] = MM::ld_nat(s.Kx, LD, 16 * I + cc, p * KS);
        qa[p] = MM::ld_nat(s.Qx, LD, 16 * I + cc, p * KS);
        kb[p] = MM::ld_nat(s.Ky, LD, 16 * J + cc, p * KS);
      }
      // The per-channel factor of a tile multiplies the shared right operand:
      // e^{Gs_I - Ge_J} for far pairs, e^{Gs_J - Ge_J} on the diagonal;
      // adjacent pairs need none. The tile kind is the same for the whole
      // wave, so these are scalar branches.
      if (far || diag) {
        const float* fr = far ? s.Ff + ((I - 2) * (I - 1) / 2 + J) * DK : s.Fd + J * DK;
#pragma unroll
        for (int p = 0; p < DK / KS; ++p) kb[p] = FragScale<E>::apply(kb[p], fr, p * KS);
      }
      f32x4 acP = zero4();
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) {
        accA[k] = MM::mma(ka[p], kb[p], accA[k]);
        acP = MM::mma(qa[p], kb[p], acP);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * I + 4 * gq + i, j = 16 * J + cc;
        const bool keep = !diag || (j < r);
        accA[k][i] = keep ? accA[k][i] : 0.f;
        Pt[k][i] = keep ? to_f32(from_f32<E>(acP[i])) : 0.f;
      }
    }
    __syncthreads();                                 // Qx/Ky are free now
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int I, J;
      if (!gram_tile(wave, k, I, J)) continue;
      if (I == J) {
        // diagonal tiles are stored transposed (column c of the block is row
        // c in memory), as the inverse walks them by column
        *reinterpret_cast<f32x4*>(s.A + (16 * I + cc) * LA + 16 * J + 4 * gq) = accA[k];
      } else {
        // -A_IJ in operand precision, row r at the start of the fp32 row r:
        // for J < I it ends before the fp32 diagonal tile of the same rows
#pragma unroll
        for (int i = 0; i < 4; ++i) s.An[(16 * I + 4 * gq + i) * LAE + 16 * J + cc] = from_f32<E>(-accA[k][i]);
      }
    }
    __syncthreads();
    if (fallback) {
      grams_pairwise<kLogits, kNorm>(s, src, t0, nvalid, Pt);
      __syncthreads();
    }
  }

  // Diagonal sub-blocks rebuilt pairwise, straight from the raw gates in
  // global memory: used only for decays too steep for the factorised form.
  // Slow but exact. A entries go to LDS; the P entries reach the Pt registers
  // of the wave that owns the tile through a scratch area in R4 (KdT is
  // parked in registers meanwhile).
  template <bool kLogits = false, bool kNorm = false>
  __device__ static void grams_pairwise(const Smem& s, const Rows<E>& src, int t0, int nvalid,
                                        f32x4 (&Pt)[TPW]) {
    float* pdiag = reinterpret_cast<float*>(s.base + LY::oR4);    // scratch: [NB][16][16]
    constexpr int KCH = DK * LK * LY::ES / 16;
    constexpr int KPER = (KCH + NT - 1) / NT;
    f32x4 keep[KPER];
#pragma unroll
    for (int j = 0; j < KPER; ++j) {
      const int c = threadIdx.x + j * NT;
      if (c < KCH) keep[j] = reinterpret_cast<const f32x4*>(s.KdT)[c];
    }
    __syncthreads();
    for (int item = threadIdx.x; item < NB * 120; item += NT) {
      const int I = item / 120;
      int p = item % 120, ri = 1;
      while (p >= ri) { p -= ri; ++ri; }
      const int ji = p;
      const int r = 16 * I + ri, j = 16 * I + ji;
      float sa = 0.f, sp = 0.f, nkr = 0.f, nkj = 0.f, nqr = 0.f;   // squared norms (kNorm)
      if (r < nvalid) {
        const size_t rowr = src.row(t0 + r) * DK, rowj = src.row(t0 + j) * DK;
        for (int d = 0; d < DK; ++d) {
          float dg = 0.f;                          // G_{r-1} - G_j, log2 units
          for (int t = j + 1; t < r; ++t) dg += decay_log2<kLogits>(ldg(src.G, src.row(t0 + t) * DK + d));
          const float gr = decay_log2<kLogits>(ldg(src.G, rowr + d));
          const float kj = ldg(src.K, rowj + d);
          const float br = sigmoid_f(ldg(src.BX, rowr + d) + s.Z[d]);
          const float kr = ldg(src.K, rowr + d), qr = ldg(src.Q, rowr + d);
          sa += br * kr * kj * fast_exp2(dg + gr);
          sp += qr * kj * fast_exp2(dg);
          if constexpr (kNorm) {
            nkr += kr * kr;
            nkj += kj * kj;
            nqr += qr * qr;
          }
        }
        if constexpr (kNorm) {
          sa *= inv_norm(nkr) * inv_norm(nkj);
          sp *= inv_norm(nqr) * inv_norm(nkj);
        }
      }
      s.A[(16 * I + ji) * LA + 16 * I + ri] = sa;   // diagonal blocks are stored transposed
      pdiag[I * 256 + ri * 16 + ji] = to_f32(from_f32<E>(sp));
    }
    __syncthreads();
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int I, J;
      if (!gram_tile(wave, k, I, J) || I != J) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ri = 4 * gq + i;
        Pt[k][i] = (cc < ri) ? pdiag[I * 256 + ri * 16 + cc] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPER; ++j) {
      const int c = threadIdx.x + j * NT;
      if (c < KCH) reinterpret_cast<f32x4*>(s.KdT)[c] = keep[j];
    }
  }

  // -------------------------------------------------------------- (I + A_II)^{-1}
  // Diagonal 16x16 blocks, one per wave, as a product of four factors on the
  // matrix cores: with P = -A_II strictly lower triangular (P^16 = 0),
  //   (I + A_II)^{-1} = sum_k P^k = (I + P)(I + P^2)(I + P^4)(I + P^8),
  // three squarings and three products in fp32 (16x16x4 steps, so the
  // result is the fp32 inverse up to rounding), stored as E. The instruction
  // takes its left operand by rows, so a product X Y needs X in the
  // transposed layout (lane (g, c) holds row c, columns 4g..4g+3) and Y in the
  // C layout (rows 4g..4g+3 of column c): (X Y)_C = mma(X_T, Y_C), and
  // (X Y)_T = (Y^T X^T)_C = mma(Y_C, X_T). The powers of P are formed in both
  // layouts, the running product R only in the transposed one, which is also
  // the row-major order in which the solve reads the inverse. The diagonal
  // blocks of A are stored transposed (column c of the block is row c in
  // memory). Ends with a barrier.
  __device__ static void inverse_diag(const Smem& s) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
    if (wave < NB) {
      using M16 = Mma16<float>;
      const float* At = s.A + (16 * wave) * LA + 16 * wave;   // At[r * LA + i] = A_II[i][r]
      f32x4 Pc = *reinterpret_cast<const f32x4*>(At + cc * LA + 4 * gq), Pt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Pc[i] = -Pc[i];
        Pt[i] = -At[(4 * gq + i) * LA + cc];
      }
      f32x4 Rt = Pt;                                   // R = I + P
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * gq + i == cc) Rt[i] += 1.f;
      const f32x4 P2c = M16::mma(Pt, Pc, zero4()), P2t = M16::mma(Pc, Pt, zero4());
      Rt += M16::mma(P2c, Rt, zero4());                // R <- R (I + P^2)
      const f32x4 P4c = M16::mma(P2t, P2c, zero4()), P4t = M16::mma(P2c, P2t, zero4());
      Rt += M16::mma(P4c, Rt, zero4());                // R <- R (I + P^4)
      const f32x4 P8c = M16::mma(P4t, P4c, zero4());
      Rt += M16::mma(P8c, Rt, zero4());                // R <- R (I + P^8)
      *reinterpret_cast<e4*>(s.Td + wave * 16 * LTD + cc * LTD + 4 * gq) =
          e4{from_f32<E>(Rt[0]), from_f32<E>(Rt[1]), from_f32<E>(Rt[2]), from_f32<E>(Rt[3])};
    }
    __syncthreads();
  }

  // -------------------------------------------------------------- [W | U] = (I + A)^{-1} [Kb | w V]
  // Blocked forward substitution over 16-row sub-blocks:
  //   X_I = T_II (R_I - sum_{J<I} A_IJ X_J),  R = [b k e^{G} | w v],
  // with T_II the diagonal inverses. Wave w solves the CTW 16-column tiles
  // CTW w .. CTW w + CTW - 1 of [W | U], keeping its X_J tiles in
  // registers. Once every operand is in registers the Qx/Ky/A region takes
  // Qd (from the gate-pass registers) and P (from the Gram registers).
  // kImage = false: the results go transposed (W^T over Kx, U^T over V) for
  // affine(); ends with a barrier. kImage = true (the chunk-parallel intra
  // kernel): after a barrier the block's affine maps are formed at once from
  // the X tiles in registers and written to the image at img (see
  // image_from_x); no W^T / U^T round trip through LDS, and no final barrier.
  static constexpr int CTW = (DK + DV) / 16 / NWV;         // [W | U] column tiles per wave
  static_assert(CTW >= 1 && CTW * NWV * 16 == DK + DV && (DK / 16) % CTW == 0, "solve tiles");
  template <bool kImage = false>
  __device__ static void solve(const Smem& s, const E (&qd)[16], const f32x4 (&Pt)[TPW],
                               unsigned char* img = nullptr) {
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int gq = lane >> 4, cc = lane & 15;
    // all column tiles of a wave lie on the same side of [W | U]
    const bool isW = CTW * wave < DK / 16;
    const int col0 = 16 * CTW * wave - (isW ? 0 : DK) + cc;
    f32x4 R[NB][CTW];
    if (isW) {
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int t = 0; t < CTW; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * gq + i, c = col0 + 16 * t;
            R[I][t][i] = to_f32(s.Kx[r * LD + c]) * s.EGs[I * DK + c];   // b k e^{G_r}
          }
    } else {
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int t = 0; t < CTW; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * gq + i, c = col0 + 16 * t;
            R[I][t][i] = s.Wg[r] * to_f32(s.V[r * LV + c]);              // w v
          }
    }
    using M16 = Mma16<E>;
    e4 Arow[NB > 1 ? NB * (NB - 1) / 2 : 1], Trow[NB];   // A operands: -A_IJ, T_II
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      Trow[I] = *reinterpret_cast<const e4*>(s.Td + I * 16 * LTD + cc * LTD + 4 * gq);
#pragma unroll
      for (int J = 0; J < I; ++J)
        Arow[I * (I - 1) / 2 + J] = *reinterpret_cast<const e4*>(s.An + (16 * I + cc) * LAE + 16 * J + 4 * gq);
    }
    __syncthreads();                                 // Kx, A, V, Td fully read
    // Qd and P into the Qx/Ky/A region
    {
      const GateCoord gc;
      if (gc.active())
#pragma unroll
        for (int i = 0; i < RPL; ++i)
          *reinterpret_cast<e4*>(s.Qd + (gc.r0 + i) * LD + gc.d0) = e4{qd[4 * i], qd[4 * i + 1], qd[4 * i + 2], qd[4 * i + 3]};
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        int I, J;
        if (!gram_tile(wave, k, I, J)) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) s.P[(16 * I + 4 * gq + i) * LK + 16 * J + cc] = from_f32<E>(Pt[k][i]);
      }
      // tiles above the diagonal are read as zeros by the affine products
      constexpr int CPT = 16 * LY::ES;               // 16-byte chunks per 16x16 tile
      for (int c = tid; c < NB * (NB - 1) / 2 * CPT; c += NT) {
        int u = c / CPT, I = 0;
        while (u >= NB - 1 - I) { u -= NB - 1 - I; ++I; }
        const int J = I + 1 + u, row = (c % CPT) / LY::ES, part = c % LY::ES;
        *reinterpret_cast<f32x4*>(s.P + (16 * I + row) * LK + 16 * J + part * (16 / LY::ES)) = zero4();
      }
      if constexpr (BL < KP)                         // padding columns of P
        for (int idx = tid; idx < BL * (KP - BL); idx += NT)
          s.P[(idx / (KP - BL)) * LK + BL + idx % (KP - BL)] = from_f32<E>(0.f);
    }
    e4 X[NB][CTW];                                  // [W | U] tiles, operand precision
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 acc[CTW];
#pragma unroll
      for (int t = 0; t < CTW; ++t) acc[t] = R[I][t];
#pragma unroll
      for (int J = 0; J < I; ++J)
#pragma unroll
        for (int t = 0; t < CTW; ++t) acc[t] = M16::mma(Arow[I * (I - 1) / 2 + J], X[J][t], acc[t]);
#pragma unroll
      for (int t = 0; t < CTW; ++t) X[I][t] = M16::round(M16::mma(Trow[I], M16::round(acc[t]), zero4()));
    }
    if constexpr (kImage) {
      __syncthreads();                               // P, Qd and KdT are complete
      image_from_x(s, X, isW, col0 - cc, img);
      return;
    }
    // transposed stores: lane holds rows 4gq..4gq+3 of column col -> 4 consecutive
    E* dst = isW ? s.Wt : s.Ut;
#pragma unroll
    for (int t = 0; t < CTW; ++t) {
      E* rowp = dst + (col0 + 16 * t) * LK;
#pragma unroll
      for (int I = 0; I < NB; ++I)
        *reinterpret_cast<e4*>(rowp + 16 * I + 4 * gq) = X[I][t];
      if constexpr (BL < KP)
        for (int j = BL + 4 * gq; j < KP; j += 16)
#pragma unroll
          for (int i = 0; i < 4; ++i) rowp[j + i] = from_f32<E>(0.f);
    }
    __syncthreads();
  }

  // -------------------------------------------------------------- affine maps from X
  // The block's affine maps from the [W | U] column tiles x0 .. x0 + 16 CTW
  // of this wave, held as C tiles X[I][t] (rows j = 16 I + 4g + i, column
  // x0 + 16 t + c), with every product taking X as one operand and K_dec^T,
  // P or Q_dec from LDS as the other:
  //   W tiles (x = k):  M[k][d] = e^{G_BL}[d] [k = d] - sum_j W[j][k] Kdec[j][d]
  //                     Qe[r][k] = Qd[r][k] - sum_j P[r][j] W[j][k]
  //     With X^T as the A operand, lane (g, c) gets k = x + 4g + i against
  //     d = 16 D + c (or r = 16 R + c): one half of an image unit of M^T (or
  //     Q_eff), written as an 8-byte store.
  //   U tiles (x = e, one value slice each):
  //                     C^T[d][e] = sum_j Kdec[j][d] U[j][e]   (K_dec^T as A, X as B)
  //                     Ol^T[e][r] = sum_j U[j][e] P[r][j]      (X^T as A, P^T as B)
  //     C tiles, written in the image's pairs.
  // P is strictly lower triangular: row block R takes j < 16 (R + 1) only.
  __device__ static void image_from_x(const Smem& s, const e4 (&X)[NB][CTW], bool isW, int x0,
                                      unsigned char* img) {
    using M16 = Mma16<E>;
    static_assert(sizeof(E) == 2 && KP == BL, "bf16 images of full 32- or 64-token blocks");
    const int lane = threadIdx.x & 63, gq = lane >> 4, cc = lane & 15;
    // B (or A) operand rows from LDS: 4 values j = 16 I + 4g .. + 3 of row `row`
    auto rd = [&](const E* base, int pitch, int row, int I) {
      return *reinterpret_cast<const e4*>(base + row * pitch + 16 * I + 4 * gq);
    };
    if (isW) {
#pragma unroll
      for (int t = 0; t < CTW; ++t) {
        const int kt = x0 / 16 + t, u = kt / 2, half = kt % 2;
#pragma unroll
        for (int D = 0; D < TD; ++D) {
          f32x4 acc = zero4();
#pragma unroll
          for (int I = 0; I < NB; ++I) acc = M16::mma(X[I][t], rd(s.KdT, LK, 16 * D + cc, I), acc);
          const float eg = s.Egl[16 * D + cc];
          e4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] = from_f32<E>((16 * kt + 4 * gq + i == 16 * D + cc ? eg : 0.f) - acc[i]);
          *reinterpret_cast<e4*>(img + LY::wMt + ((D * NU + u) * 64 + lane) * 16 + half * 8) = v;
        }
#pragma unroll
        for (int R = 0; R < NB; ++R) {
          f32x4 acc = zero4();
#pragma unroll
          for (int I = 0; I <= R; ++I) acc = M16::mma(X[I][t], rd(s.P, LK, 16 * R + cc, I), acc);
          const e4 q = *reinterpret_cast<const e4*>(s.Qd + (16 * R + cc) * LD + 16 * kt + 4 * gq);
          e4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = from_f32<E>(to_f32(q[i]) - acc[i]);
          *reinterpret_cast<e4*>(img + LY::wQe + ((R * NU + u) * 64 + lane) * 16 + half * 8) = v;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < CTW; ++t) {
        const int slice = x0 / 16 + t;
        f32x4 Ct[TD], Ol[NB];
#pragma unroll
        for (int D = 0; D < TD; ++D) {
          Ct[D] = zero4();
#pragma unroll
          for (int I = 0; I < NB; ++I) Ct[D] = M16::mma(rd(s.KdT, LK, 16 * D + cc, I), X[I][t], Ct[D]);
        }
#pragma unroll
        for (int R = 0; R < NB; ++R) {
          Ol[R] = zero4();
#pragma unroll
          for (int I = 0; I <= R; ++I) Ol[R] = M16::mma(X[I][t], rd(s.P, LK, 16 * R + cc, I), Ol[R]);
        }
        e8* ct = reinterpret_cast<e8*>(img + LY::wCt) + slice * (TD / 2) * 64 + lane;
        e8* ol = reinterpret_cast<e8*>(img + LY::wOl) + slice * (NB / 2) * 64 + lane;
#pragma unroll
        for (int a = 0; a < TD / 2; ++a) ct[a * 64] = pair(Ct[2 * a], Ct[2 * a + 1]);
#pragma unroll
        for (int a = 0; a < NB / 2; ++a) ol[a * 64] = pair(Ol[2 * a], Ol[2 * a + 1]);
      }
    }
  }

  // -------------------------------------------------------------- affine maps
  //   Mt[d'][d] = e^{G_BL}[d] [d = d'] - sum_j Kdec[j][d'] W[j][d]
  //   Qe[r][d]  = Qd[r][d] - sum_j P[r][j] W[j][d]
  //   Ct[d'][e] = sum_j Kdec[j][d'] U[j][e]
  //   Olt[e][r] = sum_j P[r][j] U[j][e]
  // Every product reads rows of two tiles whose columns run over j (natural
  // map); values are rounded to E. Mt and Qe are computed transposed (C rows
  // over d), so a lane's C values of UT adjacent tiles are exactly one
  // operand unit over d: they go to the sink as 16-byte stores, spread over
  // the waves. Wave w computes the Ct and Olt tiles of value slice
  // w mod NW, channels [16 slice, 16 slice + 16) (part w / NW of them when
  // several waves share a slice), and keeps them in registers (CtR, OltR).
  // Ends with a barrier.
  __device__ static void affine(const Smem& s, const Sink<E>& out, f32x4 (&CtR)[CTP], f32x4 (&OltR)[OLP]) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
    auto product = [&](const E* left, int a, const E* right, int b, int nst) {
      f32x4 acc = zero4();
      for (int p = 0; p < nst; ++p)
        acc = MM::mma(MM::ld_nat(left, LK, 16 * a + cc, p * KS), MM::ld_nat(right, LK, 16 * b + cc, p * KS), acc);
      return acc;
    };
    // units of Mt (rows d' = 16a + c) and then of Qe (rows r = 16a + c), dealt
    // to the waves in turn
    auto unit_job = [&](auto isM, int x) {
      const int a = x / NU, u = x % NU, r = 16 * a + cc;
      // the diagonal of Mt: element (r, d = r) of tile b = a sits in lane
      // (g, c) with c = 4g + i
      const float eg = isM ? s.Egl[r] : 0.f;
      f32x4 t[UT];
#pragma unroll
      for (int j = 0; j < UT; ++j) {
        const int b = UT * u + j;                     // 16-wide slice of d
        // P is lower-triangular: row block a needs j < 16 (a + 1) only
        const f32x4 acc = isM ? product(s.Wt, b, s.KdT, a, MM::steps(KP))
                              : product(s.Wt, b, s.P, a, MM::steps(16 * (a + 1)));
        const e4 qd4 = isM ? e4{} : *reinterpret_cast<const e4*>(s.Qd + r * LD + 16 * b + 4 * gq);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          t[j][i] = isM ? (b == a && cc == 4 * gq + i ? eg : 0.f) - acc[i] : to_f32(qd4[i]) - acc[i];
      }
      if constexpr (decltype(isM)::value) out.Mt[x * 64 + lane] = MM::pack(t);
      else out.Qe[x * 64 + lane] = MM::pack(t);
    };
    constexpr int NMJ = TD * NU;
    for (int x = wave; x < NMJ; x += NWV) unit_job(std::true_type{}, x);
    for (int x = ((wave - NMJ) % NWV + NWV) % NWV; x < NB * NU; x += NWV) unit_job(std::false_type{}, x);
    // Ct and Olt of this wave's value channels (part `part` of the tiles of
    // slice `slice` when several waves share a slice)
    const int slice = wave % NW, part = wave / NW;
#pragma unroll
    for (int j = 0; j < CTP; ++j) {
      f32x4 acc = product(s.KdT, part * CTP + j, s.Ut, slice, MM::steps(KP));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = to_f32(from_f32<E>(acc[i]));
      CtR[j] = acc;
    }
#pragma unroll
    for (int j = 0; j < OLP; ++j) {
      const int a = part * OLP + j;
      f32x4 acc = product(s.Ut, slice, s.P, a, MM::steps(16 * (a + 1)));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = to_f32(from_f32<E>(acc[i]));
      OltR[j] = acc;
    }
    __syncthreads();
  }

  // -------------------------------------------------------------- lean blocks
  // The chunk-serial kernel at d = 64 with 64-token bf16 blocks has LDS to
  // spare, so the operands of the triangular system get areas of their own
  // and the stage sequence loses three barriers and a round trip:
  //   - P, -A_IJ and Q_dec do not wait for the gate operands to die;
  //   - the wave that computes a diagonal Gram tile forms its inverse
  //     T_II = (I + A_II)^{-1} at once from its registers (the transposed
  //     copy of -A_II comes from a product with the identity, which is
  //     exact), as inverse_diag does from LDS;
  //   - the affine maps come from the solve's registers as in the
  //     chunk-parallel intra kernel (image_from_x): M^T and Qe units go to
  //     the kernel's LDS sink, and the U waves keep the C^T and Ol^T tiles of
  //     their value slice, handing half of them to the other wave of the
  //     slice through Cx.
  // Blocks whose decay is too steep for the factorised Grams take the
  // general stages instead.
  struct Lean {
    E* P; E* Qd; E* An; E* Td; e4* Cx;
  };
  __device__ static Lean lean(unsigned char* smem) {
    return Lean{reinterpret_cast<E*>(smem + LY::oLP), reinterpret_cast<E*>(smem + LY::oLQd),
                reinterpret_cast<E*>(smem + LY::oLAn), reinterpret_cast<E*>(smem + LY::oLTd),
                reinterpret_cast<e4*>(smem + LY::oLCx)};
  }
  // Q_dec rows of this thread from the gate-pass registers
  __device__ static void lean_qd(const Lean& ln, const E (&qd)[16]) {
    const GateCoord gc;
    if (gc.active())
#pragma unroll
      for (int i = 0; i < RPL; ++i)
        *reinterpret_cast<e4*>(ln.Qd + (gc.r0 + i) * LD + gc.d0) = e4{qd[4 * i], qd[4 * i + 1], qd[4 * i + 2], qd[4 * i + 3]};
  }
  // Grams A and P (factorised form only) and the diagonal inverses. Ends
  // with a barrier.
  __device__ static void grams_lean(const Smem& s, const Lean& ln) {
    static_assert(LY::kLean, "lean blocks only");
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int I, J;
      if (!gram_tile(wave, k, I, J)) continue;
      const bool diag = (I == J), far = (J < I - 1);
      Frag ka[DK / KS], qa[DK / KS], kb[DK / KS];
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) {
        ka[p] = MM::ld_nat(s.Kx, LD, 16 * I + cc, p * KS);
        qa[p] = MM::ld_nat(s.Qx, LD, 16 * I + cc, p * KS);
        kb[p] = MM::ld_nat(s.Ky, LD, 16 * J + cc, p * KS);
      }
      if (far || diag) {
        const float* fr = far ? s.Ff + ((I - 2) * (I - 1) / 2 + J) * DK : s.Fd + J * DK;
#pragma unroll
        for (int p = 0; p < DK / KS; ++p) kb[p] = FragScale<E>::apply(kb[p], fr, p * KS);
      }
      f32x4 accA = zero4(), acP = zero4();
#pragma unroll
      for (int p = 0; p < DK / KS; ++p) {
        accA = MM::mma(ka[p], kb[p], accA);
        acP = MM::mma(qa[p], kb[p], acP);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * I + 4 * gq + i, j = 16 * J + cc;
        const bool keep = !diag || (j < r);
        accA[i] = keep ? accA[i] : 0.f;
        ln.P[r * LK + j] = from_f32<E>(keep ? acP[i] : 0.f);
      }
      if (diag) {
        // (I + P)(I + P^2)(I + P^4)(I + P^8) with P = -A_II, as in inverse_diag
        using M16 = Mma16<float>;
        f32x4 Pc, Id;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Pc[i] = -accA[i];
          Id[i] = 4 * gq + i == cc ? 1.f : 0.f;
        }
        const f32x4 Pt = M16::mma(Pc, Id, zero4());   // (P^T I)_C: P in the transposed layout
        f32x4 Rt = Pt;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * gq + i == cc) Rt[i] += 1.f;
        const f32x4 P2c = M16::mma(Pt, Pc, zero4()), P2t = M16::mma(Pc, Pt, zero4());
        Rt += M16::mma(P2c, Rt, zero4());
        const f32x4 P4c = M16::mma(P2t, P2c, zero4()), P4t = M16::mma(P2c, P2t, zero4());
        Rt += M16::mma(P4c, Rt, zero4());
        const f32x4 P8c = M16::mma(P4t, P4c, zero4());
        Rt += M16::mma(P8c, Rt, zero4());
        *reinterpret_cast<e4*>(ln.Td + I * 16 * LTD + cc * LTD + 4 * gq) =
            e4{from_f32<E>(Rt[0]), from_f32<E>(Rt[1]), from_f32<E>(Rt[2]), from_f32<E>(Rt[3])};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) ln.An[(16 * I + 4 * gq + i) * LK + 16 * J + cc] = from_f32<E>(-accA[i]);
      }
    }
    __syncthreads();
  }
  // [W | U] by blocked forward substitution (as in solve) into registers, then
  // the affine maps from them. W waves write M^T and Qe units to the sink;
  // U waves return the C^T and Ol^T tiles of this wave's part of its value
  // slice (rounded to E) in CtR, OltR and hand the other part's to Cx. Ends
  // with a barrier, after which the waves of part 0 read theirs from Cx.
  __device__ static void solve_affine_lean(const Smem& s, const Lean& ln, f32x4 (&CtR)[CTP], f32x4 (&OltR)[OLP]) {
    static_assert(LY::kLean && CTW == 1 && PARTS == 2 && CTP * 2 == TD && OLP * 2 == NB, "lean blocks only");
    using M16 = Mma16<E>;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
    const bool isW = wave < DK / 16;
    const int col0 = 16 * wave - (isW ? 0 : DK) + cc;
    f32x4 R[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * I + 4 * gq + i;
        R[I][i] = isW ? to_f32(s.Kx[r * LD + col0]) * s.EGs[I * DK + col0]     // b k e^{G_r}
                      : s.Wg[r] * to_f32(s.V[r * LV + col0]);                  // w v
      }
    e4 X[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 acc = R[I];
#pragma unroll
      for (int J = 0; J < I; ++J)
        acc = M16::mma(*reinterpret_cast<const e4*>(ln.An + (16 * I + cc) * LK + 16 * J + 4 * gq), X[J], acc);
      const e4 T = *reinterpret_cast<const e4*>(ln.Td + I * 16 * LTD + cc * LTD + 4 * gq);
      X[I] = M16::round(M16::mma(T, M16::round(acc), zero4()));
    }
    auto rd = [&](const E* base, int pitch, int row, int I) {
      return *reinterpret_cast<const e4*>(base + row * pitch + 16 * I + 4 * gq);
    };
    if (isW) {
      // M^T (rows d = 16 D + c) and Qe (rows r = 16 R + c) against k = 16 kt + 4g + i:
      // one half of a sink unit each
      unsigned char* sink = reinterpret_cast<unsigned char*>(s.Mt);
      const int kt = wave, u = kt / 2, half = kt % 2;
#pragma unroll
      for (int D = 0; D < TD; ++D) {
        f32x4 acc = zero4();
#pragma unroll
        for (int I = 0; I < NB; ++I) acc = M16::mma(X[I], rd(s.KdT, LK, 16 * D + cc, I), acc);
        const float eg = s.Egl[16 * D + cc];
        e4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = from_f32<E>((16 * kt + 4 * gq + i == 16 * D + cc ? eg : 0.f) - acc[i]);
        *reinterpret_cast<e4*>(sink + LY::wMt + ((D * NU + u) * 64 + lane) * 16 + half * 8) = v;
      }
#pragma unroll
      for (int Rb = 0; Rb < NB; ++Rb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int I = 0; I <= Rb; ++I) acc = M16::mma(X[I], rd(ln.P, LK, 16 * Rb + cc, I), acc);
        const e4 q = *reinterpret_cast<const e4*>(ln.Qd + (16 * Rb + cc) * LD + 16 * kt + 4 * gq);
        e4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = from_f32<E>(to_f32(q[i]) - acc[i]);
        *reinterpret_cast<e4*>(sink + LY::wQe + ((Rb * NU + u) * 64 + lane) * 16 + half * 8) = v;
      }
    } else {
      const int slice = wave - DK / 16;               // = wave % NW: this wave is part 1 of its slice
      e4* cx = ln.Cx + slice * (CTP + OLP) * 64 + lane;
#pragma unroll
      for (int D = 0; D < TD; ++D) {
        f32x4 acc = zero4();
#pragma unroll
        for (int I = 0; I < NB; ++I) acc = M16::mma(rd(s.KdT, LK, 16 * D + cc, I), X[I], acc);
        const e4 v = M16::round(acc);
        if (D < CTP) cx[D * 64] = v;
        else
#pragma unroll
          for (int i = 0; i < 4; ++i) CtR[D - CTP][i] = to_f32(v[i]);
      }
#pragma unroll
      for (int Rb = 0; Rb < NB; ++Rb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int I = 0; I <= Rb; ++I) acc = M16::mma(X[I], rd(ln.P, LK, 16 * Rb + cc, I), acc);
        const e4 v = M16::round(acc);
        if (Rb < OLP) cx[(CTP + Rb) * 64] = v;
        else
#pragma unroll
          for (int i = 0; i < 4; ++i) OltR[Rb - OLP][i] = to_f32(v[i]);
      }
    }
    __syncthreads();
    if (isW) {
      const e4* cx = ln.Cx + wave * (CTP + OLP) * 64 + lane;   // part 0 of slice `wave`
#pragma unroll
      for (int t = 0; t < CTP; ++t) {
        const e4 v = cx[t * 64];
#pragma unroll
        for (int i = 0; i < 4; ++i) CtR[t][i] = to_f32(v[i]);
      }
#pragma unroll
      for (int j = 0; j < OLP; ++j) {
        const e4 v = cx[(CTP + j) * 64];
#pragma unroll
        for (int i = 0; i < 4; ++i) OltR[j][i] = to_f32(v[i]);
      }
    }
  }

  // -------------------------------------------------------------- state and output
  // One wave, 16 value channels, S^T held as C tiles (rows d, cols e):
  //   O^T = S Qe^T + Ol^T      (S at the block start; tile rt holds tokens
  //                             16 rt .. 16 rt + 15 as columns)
  //   S^T <- Mt S^T + Ct
  // The S fragments serve as the A operand of the first product and the B
  // operand of the second. mt(dt, u) and qe(rt, u) return operand units.
  // the S operand fragments (bf16 or fp32) of the current state
  __device__ static void state_frags(const f32x4 (&St)[TD], Frag (&sf)[DK / KS]) {
#pragma unroll
    for (int p = 0; p < DK / KS; ++p) sf[p] = MM::from_c(St, p);
  }
  // O^T = S Qe^T + Ol^T from the fragments of S at the block start
  // (reduction steps outermost, so consecutive instructions write different
  // tiles and never wait for each other's results)
  template <typename QeF>
  __device__ static void state_out(QeF qe, const f32x4 (&Olt)[NB], const Frag (&sf)[DK / KS], f32x4 (&Ot)[NB]) {
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) Ot[rt] = Olt[rt];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int j = 0; j < SPU; ++j)
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) Ot[rt] = MM::mma(sf[u * SPU + j], MM::step(qe(rt, u), j), Ot[rt]);
  }
  // S^T <- Mt S^T + Ct
  template <typename MtF>
  __device__ static void state_chain(MtF mt, const f32x4 (&Ct)[TD], const Frag (&sf)[DK / KS], f32x4 (&St)[TD]) {
    f32x4 acc[TD];
#pragma unroll
    for (int dt = 0; dt < TD; ++dt) acc[dt] = Ct[dt];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int j = 0; j < SPU; ++j)
#pragma unroll
        for (int dt = 0; dt < TD; ++dt) acc[dt] = MM::mma(MM::step(mt(dt, u), j), sf[u * SPU + j], acc[dt]);
#pragma unroll
    for (int dt = 0; dt < TD; ++dt) St[dt] = acc[dt];
  }

  // load/store the S^T C tiles of value slice `ws` from/to a [B,H,DV,DK] fp32 tensor
  __device__ static void load_state(const float* S, int bh, int ws, f32x4 (&St)[TD]) {
    const int lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int dt = 0; dt < TD; ++dt) {
      if (S) St[dt] = *reinterpret_cast<const f32x4*>(S + ((size_t)bh * DV + 16 * ws + cc) * DK + 16 * dt + 4 * gq);
      else St[dt] = zero4();
    }
  }
  __device__ static void store_state(float* S, int bh, int ws, const f32x4 (&St)[TD]) {
    const int lane = threadIdx.x & 63;
    const int gq = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int dt = 0; dt < TD; ++dt)
      *reinterpret_cast<f32x4*>(S + ((size_t)bh * DV + 16 * ws + cc) * DK + 16 * dt + 4 * gq) = St[dt];
  }
};

}  // namespace carve
