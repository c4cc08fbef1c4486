// Chunk-serial CARVE forward kernel: one workgroup per (batch, head).
//
// The workgroup walks the sequence in blocks of BL tokens (BL <= L, BL | L)
// and applies the WY form of the token recurrence to each block. With
// S the state at the block start, G_r the inclusive cumulative log-decay
// inside the block (G_{-1} = 0), b_r = sigmoid(bx_r + z) and
// U_b m_{c-1} = z (gist.science summary §2.1):
//   A_rj  = sum_d b_r k_r k_j e^{G_r - G_j}          (j < r)
//   P_rj  = sum_d q_r k_j e^{G_{r-1} - G_j}          (j < r)
//   T     = (I + A)^{-1}
//   W     = T (b k e^{G_r}),   U = T (w v)
//   Delta = U - W S^T
//   O     = (q e^{G_{r-1}}) S^T + P Delta           (o_t = S_{t-1} q_t)
//   S    <- S diag(e^{G_BL}) + Delta^T (k e^{G_BL - G_j})
// This is exact algebra for the recurrence S <- S D (I - (b k) k^T) + w v k^T;
// the single triangular system per block exists because every gate acts on
// the key axis (Theorem 11 in §3 of the same summary).
//
// Work split: wave w owns value channels [16w, 16w+16), i.e. 16 rows of S,
// which it keeps in registers as fp32 MFMA accumulators of S^T for the whole
// sequence. The shared per-block quantities (gates, Grams, T, W) are built
// cooperatively in LDS.
//
// Exponent safety: the Grams use 16-row sub-blocks. For a pair of sub-blocks
// (I > J) the factor e^{G_r - G_j} is split as
//   e^{G_r - Gs_I} * e^{Gs_I - Ge_J} * e^{Ge_J - G_j}
// (Gs_I: G just before sub-block I; Ge_J: G at the end of sub-block J), each
// factor <= 1. Diagonal sub-blocks use e^{G_r - Gs_I} * e^{Gs_I - G_j}, which
// is safe while the decay inside one sub-block stays below kSpanLimit2 (in
// log2 units); beyond that the diagonal entries are rebuilt pairwise.
#pragma once
#include "common.h"

namespace carve {

struct FwdArgs {
  const void* q; const void* k; const void* v; const void* g; const void* bx; const void* w;
  const void* ub_down; const void* ub_up;
  const float* state_in; const float* mean_in;
  void* o; float* state_out; float* mean_out;
  int B, H, T, L, rank;
};

constexpr float kSpanLimit2 = 96.0f;   // max decay (log2 units) inside a 16-row sub-block

template <typename E, int DK, int DV, int BL>
struct SerialLayout {
  static_assert(DK % 32 == 0 && DV % 16 == 0, "head widths");
  static_assert(BL == 16 || BL == 32 || BL == 64, "block length");
  static constexpr int NW = DV / 16;
  static constexpr int NT = NW * 64;
  static constexpr int NB = BL / 16;
  static constexpr int KP = BL < 32 ? 32 : BL;     // padded token-reduction width
  static_assert(NT >= DK * NB, "one thread per (key column, sub-block) in the gate pass");
  static constexpr int ES = sizeof(E);
  // byte offsets
  static constexpr int oKx = 0;                              // [BL][DK] E   (later W)
  static constexpr int oQx = oKx + BL * DK * ES;             // [BL][DK] E   (later T fp32)
  static constexpr int oKy = oQx + BL * DK * ES;             // [BL][DK] E
  static constexpr int oKbT = oKy + BL * DK * ES;            // [DK][KP] E
  static constexpr int oVt = oKbT + DK * KP * ES;            // [DV][KP] E
  static constexpr int oQd = oVt + DV * KP * ES;             // [BL][DK] E
  static constexpr int oKdT = oQd + BL * DK * ES;            // [DK][KP] E
  static constexpr int oP = oKdT + DK * KP * ES;             // [BL][KP] E
  static constexpr int oA = oP + BL * KP * ES;               // [BL][BL] f32
  static constexpr int oGb = oA + BL * BL * 4;               // [NB+1][DK] f32 (log2 units)
  static constexpr int oSeg = oGb + (NB + 1) * DK * 4;       // [NB][DK] f32
  static constexpr int oEgl = oSeg + NB * DK * 4;            // [DK] f32
  static constexpr int oWg = oEgl + DK * 4;                  // [KP] f32 write gate (zero padded)
  static constexpr int oZ = oWg + KP * 4;                    // [DK] f32
  static constexpr int oM = oZ + DK * 4;                     // [DV] f32
  static constexpr int oY = oM + DV * 4;                     // [64] f32
  static constexpr int oFlag = oY + 64 * 4;                  // int
  static constexpr int bytes = oFlag + 16;
  static_assert(2 * BL * DK * ES >= BL * KP * 4, "T fits in the Qx/Ky region");
  static_assert(BL * DK * ES >= NB * 256 * 2 * 4, "fallback accumulators fit in Kx");
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <typename E>
__device__ __forceinline__ float ldg(const E* p, size_t i) { return to_f32(p[i]); }

// multiply fragment slot values by per-k factors (natural map, k0 + KS-slot)
template <typename M> struct FragScale;
template <> struct FragScale<bf16> {
  __device__ __forceinline__ static bf16x8 apply(bf16x8 a, const float* fac, int k0) {
    const int g = lane_id() >> 4;
    const f32x4* f = reinterpret_cast<const f32x4*>(fac + k0 + 8 * g);
    f32x4 f0 = f[0], f1 = f[1];
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

template <typename E, int DK, int DV, int BL>
__global__ void __launch_bounds__((SerialLayout<E, DK, DV, BL>::NT))
carve_chunk_serial_kernel(FwdArgs a) {
  using LY = SerialLayout<E, DK, DV, BL>;
  using MM = Mma<E>;
  using Frag = typename MM::frag;
  constexpr int NW = LY::NW, NT = LY::NT, NB = LY::NB, KP = LY::KP;
  constexpr int KS = MM::KS;

  extern __shared__ __align__(16) unsigned char smem[];
  E* sKx = reinterpret_cast<E*>(smem + LY::oKx);
  E* sW = sKx;                                   // alias after the Grams
  E* sQx = reinterpret_cast<E*>(smem + LY::oQx);
  float* sT = reinterpret_cast<float*>(smem + LY::oQx);   // alias after the Grams
  E* sKy = reinterpret_cast<E*>(smem + LY::oKy);
  E* sKbT = reinterpret_cast<E*>(smem + LY::oKbT);
  E* sVt = reinterpret_cast<E*>(smem + LY::oVt);
  E* sQd = reinterpret_cast<E*>(smem + LY::oQd);
  E* sKdT = reinterpret_cast<E*>(smem + LY::oKdT);
  E* sP = reinterpret_cast<E*>(smem + LY::oP);
  float* sA = reinterpret_cast<float*>(smem + LY::oA);
  float* sGb = reinterpret_cast<float*>(smem + LY::oGb);
  float* sSeg = reinterpret_cast<float*>(smem + LY::oSeg);
  float* sEgl = reinterpret_cast<float*>(smem + LY::oEgl);
  float* sWg = reinterpret_cast<float*>(smem + LY::oWg);
  float* sZ = reinterpret_cast<float*>(smem + LY::oZ);
  float* sM = reinterpret_cast<float*>(smem + LY::oM);
  float* sY = reinterpret_cast<float*>(smem + LY::oY);
  int* sFlag = reinterpret_cast<int*>(smem + LY::oFlag);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int gq = lane >> 4;      // row group within a C tile
  const int cc = lane & 15;      // column within a C tile
  const int bh = blockIdx.x;
  const int bidx = bh / a.H, h = bh % a.H;
  const int T = a.T, H = a.H, L = a.L;

  const E* __restrict__ Q = static_cast<const E*>(a.q);
  const E* __restrict__ K = static_cast<const E*>(a.k);
  const E* __restrict__ V = static_cast<const E*>(a.v);
  const E* __restrict__ Gl = static_cast<const E*>(a.g);
  const E* __restrict__ BX = static_cast<const E*>(a.bx);
  const E* __restrict__ Wt = static_cast<const E*>(a.w);
  E* __restrict__ O = static_cast<E*>(a.o);
  const E* Ud = static_cast<const E*>(a.ub_down);
  const E* Uu = static_cast<const E*>(a.ub_up);
  const int rank = a.rank;

  // zero all LDS once: padded columns and never-written blocks stay zero
  for (int i = tid; i < LY::bytes / 4; i += NT) reinterpret_cast<float*>(smem)[i] = 0.f;

  // state: wave owns S rows e0..e0+15, kept as S^T C tiles (rows = key dim)
  const int e0 = 16 * wave;
  f32x4 St[DK / 16];
#pragma unroll
  for (int dt = 0; dt < DK / 16; ++dt) {
    if (a.state_in) {
      const float* s = a.state_in + ((size_t)bh * DV + e0 + cc) * DK + 16 * dt + 4 * gq;
      St[dt] = *reinterpret_cast<const f32x4*>(s);
    } else {
      St[dt] = zero4();
    }
  }
  __syncthreads();
  // the mean that gates chunk 0
  for (int e = tid; e < DV; e += NT) sM[e] = a.mean_in ? a.mean_in[(size_t)bh * DV + e] : 0.f;
  __syncthreads();

  auto content_bias = [&]() {
    // z = U_up (U_down m) into sZ; all threads call
    if (rank > 0) {
      for (int r = tid; r < rank; r += NT) {
        float y = 0.f;
        for (int e = 0; e < DV; ++e) y += ldg(Ud, ((size_t)h * rank + r) * DV + e) * sM[e];
        sY[r] = y;
      }
      __syncthreads();
      for (int d = tid; d < DK; d += NT) {
        float z = 0.f;
        for (int r = 0; r < rank; ++r) z += ldg(Uu, ((size_t)h * DK + d) * rank + r) * sY[r];
        sZ[d] = z;
      }
    }
    __syncthreads();
  };
  content_bias();

  float m_part = 0.f;                   // this lane's running column sum of O
  const int nblk = (T + BL - 1) / BL;
  const int gs = tid / DK;              // gate pass: sub-block of this thread
  const int gd = tid % DK;              //            key column of this thread

  for (int blk = 0; blk < nblk; ++blk) {
    const int t0 = blk * BL;
    const int nvalid = min(BL, T - t0);
    const int chunk = t0 / L;
    const bool chunk_end = ((t0 + BL) % L == 0) || (t0 + BL >= T);

    // ------------------------------------------------------------ gate pass
    if (tid == 0) sFlag[0] = 0;
    float Greg[16];                     // local inclusive G (log2 units), 16 rows
    if (gs < NB) {
      float run = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * gs + i;
        float gv = 0.f;
        if (r < nvalid) gv = ldg(Gl, ((size_t)(bidx * T + t0 + r) * H + h) * DK + gd);
        run += gv * kLog2e;
        Greg[i] = run;
      }
      sSeg[gs * DK + gd] = run;
    }
    // write gate and transposed values
    for (int idx = tid; idx < BL * DV; idx += NT) {
      const int r = idx / DV, e = idx % DV;
      float vv = 0.f;
      if (r < nvalid) vv = ldg(V, ((size_t)(bidx * T + t0 + r) * H + h) * DV + e);
      sVt[e * KP + r] = from_f32<E>(vv);
    }
    for (int r = tid; r < BL; r += NT)
      sWg[r] = (r < nvalid) ? ldg(Wt, (size_t)(bidx * T + t0 + r) * H + h) : 0.f;
    __syncthreads();
    if (gs < NB) {
      float base = 0.f, total = 0.f;
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        const float t = sSeg[s * DK + gd];
        if (s < gs) base += t;
        total += t;
      }
      const float Gs = base;                         // G before this sub-block
      const float Ge = base + Greg[15];              // G at its last row
      sGb[gs * DK + gd] = Gs;
      if (gs == NB - 1) {
        sGb[NB * DK + gd] = total;
        sEgl[gd] = fast_exp2(total);
      }
      if (Gs - Ge > kSpanLimit2) atomicOr(sFlag, 1);
      const float eGs = fast_exp2(Gs);
      const float eTail = fast_exp2(total - Ge);
      const float z = sZ[gd];
      float eprev = 1.f;                             // e^{G_{r-1} - Gs}
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * gs + i;
        float kk = 0.f, qq = 0.f, bxv = 0.f;
        if (r < nvalid) {
          const size_t off = ((size_t)(bidx * T + t0 + r) * H + h) * DK + gd;
          kk = ldg(K, off);
          qq = ldg(Q, off);
          bxv = ldg(BX, off);
        }
        const float Gr = base + Greg[i];
        const float bb = sigmoid_f(bxv + z);
        const float e1 = fast_exp2(Gr - Gs);         // <= 1
        const float en = fast_exp2(Ge - Gr);         // <= 1
        const float bk = bb * kk;
        sKx[r * DK + gd] = from_f32<E>(bk * e1);
        sQx[r * DK + gd] = from_f32<E>(qq * eprev);
        sKy[r * DK + gd] = from_f32<E>(kk * en);
        sKbT[gd * KP + r] = from_f32<E>(bk * e1 * eGs);
        sQd[r * DK + gd] = from_f32<E>(qq * eprev * eGs);
        sKdT[gd * KP + r] = from_f32<E>(kk * en * eTail);
        eprev = e1;
      }
    }
    __syncthreads();
    const bool fallback = sFlag[0] != 0;

    // ------------------------------------------------------------ Grams A, P
    {
      constexpr int NPAIR = NB * (NB + 1) / 2;
      for (int pr = wave; pr < NPAIR; pr += NW) {
        int I = 0, J = pr;
        while (J > I) { J -= I + 1; ++I; }
        f32x4 accA = zero4(), accP = zero4();
        const bool diag = (I == J);
        // per-k factors: left operand e^{Gs_I - Ge_J} (J < I-1); diagonal right
        // operand e^{Gs_J - Ge_J}
#pragma unroll
        for (int p = 0; p < DK / KS; ++p) {
          Frag ka = MM::ld_nat(sKx, DK, 16 * I + cc, p * KS);
          Frag qa = MM::ld_nat(sQx, DK, 16 * I + cc, p * KS);
          Frag kb = MM::ld_nat(sKy, DK, 16 * J + cc, p * KS);
          if (J < I - 1) {
            // scale left operands by 2^{Gb[I] - Gb[J+1]}
            float f[KS < 8 ? 1 : 8];
            const int g = lane_id() >> 4;
            constexpr int NSL = (KS == 32) ? 8 : 1;
#pragma unroll
            for (int s = 0; s < NSL; ++s) {
              const int kk = p * KS + (KS == 32 ? 8 * g + s : g);
              f[s] = fast_exp2(sGb[I * DK + kk] - sGb[(J + 1) * DK + kk]);
            }
            if constexpr (KS == 32) {
#pragma unroll
              for (int s = 0; s < 8; ++s) {
                ka[s] = (bf16)((float)ka[s] * f[s]);
                qa[s] = (bf16)((float)qa[s] * f[s]);
              }
            } else {
              ka = ka * f[0];
              qa = qa * f[0];
            }
          }
          if (diag) {
            const int g = lane_id() >> 4;
            if constexpr (KS == 32) {
#pragma unroll
              for (int s = 0; s < 8; ++s) {
                const int kk = p * KS + 8 * g + s;
                kb[s] = (bf16)((float)kb[s] * fast_exp2(sGb[J * DK + kk] - sGb[(J + 1) * DK + kk]));
              }
            } else {
              const int kk = p * KS + g;
              kb = kb * fast_exp2(sGb[J * DK + kk] - sGb[(J + 1) * DK + kk]);
            }
          }
          accA = MM::mma(ka, kb, accA);
          accP = MM::mma(qa, kb, accP);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * I + 4 * gq + i, j = 16 * J + cc;
          const bool keep = !diag || (j < r);
          sA[r * BL + j] = keep ? accA[i] : 0.f;
          sP[r * KP + j] = from_f32<E>(keep ? accP[i] : 0.f);
        }
      }
    }
    __syncthreads();

    if (fallback) {
      // Rebuild the diagonal sub-blocks pairwise from the raw gates (only for
      // decays too steep for the factorised form; slow but exact).
      float* accA = reinterpret_cast<float*>(smem + LY::oKx);         // [NB][16][16]
      float* accP = accA + NB * 256;
      for (int i = tid; i < NB * 512; i += NT) accA[i] = 0.f;
      __syncthreads();
      if (gs < NB) {
        const float z = sZ[gd];
        auto off_of = [&](int r) { return ((size_t)(bidx * T + t0 + r) * H + h) * DK + gd; };
        // local inclusive G (log2 units) of this column, kept in the dead Qx region
        float* Gloc = reinterpret_cast<float*>(smem + LY::oQx) + gd;
        float run = 0.f;
        for (int i = 0; i < 16; ++i) {
          const int r = 16 * gs + i;
          run += (r < nvalid) ? ldg(Gl, off_of(r)) * kLog2e : 0.f;
          Gloc[(16 * gs + i) * DK] = run;
        }
        for (int ri = 1; ri < 16; ++ri) {
          const int r = 16 * gs + ri;
          float kr = 0.f, qr = 0.f, br = 0.f;
          if (r < nvalid) {
            kr = ldg(K, off_of(r));
            qr = ldg(Q, off_of(r));
            br = sigmoid_f(ldg(BX, off_of(r)) + z);
          }
          for (int ji = 0; ji < ri; ++ji) {
            const int j = 16 * gs + ji;
            const float kj = (j < nvalid) ? ldg(K, off_of(j)) : 0.f;
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
        const int s = i / 256, ri = (i / 16) % 16, ji = i % 16;
        const int r = 16 * s + ri, j = 16 * s + ji;
        sA[r * BL + j] = (ji < ri) ? accA[i] : 0.f;
        sP[r * KP + j] = from_f32<E>((ji < ri) ? accP[i] : 0.f);
      }
      __syncthreads();
    }

    // ------------------------------------------------ T = (I + A)^{-1}
    // diagonal 16x16 blocks by forward substitution (fp32); lane = c + 16 q
    if (wave < NB) {
      const int I = wave;
      const int c = cc, qd = gq;
      float tcol[4] = {0.f, 0.f, 0.f, 0.f};          // T[4jj + qd][c] within the block
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float part = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * jj + qd;
          if (j < r) part += sA[(16 * I + r) * BL + 16 * I + j] * tcol[jj];
        }
        part = sum_groups(part);
        const float val = (r == c) ? 1.f : ((r > c) ? -part : 0.f);
        if ((r & 3) == qd) tcol[r >> 2] = val;
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sT[(16 * I + 4 * jj + qd) * KP + 16 * I + c] = tcol[jj];
      // zero this row block right of the diagonal block (upper blocks, padding)
      for (int idx = lane; idx < 16 * KP; idx += 64) {
        const int rr = idx / KP, j = idx % KP;
        if (j >= 16 * (I + 1)) sT[(16 * I + rr) * KP + j] = 0.f;
      }
    }
    __syncthreads();
    // off-diagonal blocks: wave J walks its block column downwards
    if (NB > 1 && wave < NB - 1) {
      const int J = wave;
      f32x4 Tc[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) Tc[I] = zero4();
#pragma unroll
      for (int I = 0; I < NB; ++I)
        if (I == J)
#pragma unroll
          for (int i = 0; i < 4; ++i) Tc[I][i] = sT[(16 * J + 4 * gq + i) * KP + 16 * J + cc];
#pragma unroll
      for (int I = 1; I < NB; ++I) {
        if (I <= J) continue;
        f32x4 X = zero4();
#pragma unroll
        for (int Kb = 0; Kb < NB; ++Kb)
          if (Kb >= J && Kb < I) X = Mma16<E>::mma_rowA_cB(sA, BL, 16 * I + cc, 16 * Kb, Tc[Kb], X, 1.f);
        Tc[I] = Mma16<E>::mma_rowA_cB(sT, KP, 16 * I + cc, 16 * I, X, zero4(), -1.f);
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(16 * I + 4 * gq + i) * KP + 16 * J + cc] = Tc[I][i];
      }
    }
    __syncthreads();

    // ------------------------------------------------ W = T (b k e^{G})
    {
      constexpr int NTILE = NB * (DK / 16);
      for (int tt = wave; tt < NTILE; tt += NW) {
        const int I = tt / (DK / 16), dt = tt % (DK / 16);
        f32x4 acc = zero4();
        const int nst = MM::steps(16 * (I + 1));
        for (int p = 0; p < nst; ++p)
          acc = MM::mma(MM::ld_nat(sT, KP, 16 * I + cc, p * KS), MM::ld_nat(sKbT, KP, 16 * dt + cc, p * KS), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) sW[(16 * I + 4 * gq + i) * DK + 16 * dt + cc] = from_f32<E>(acc[i]);
      }
    }
    __syncthreads();

    // ------------------------------------------------ per-wave state and output
    {
      constexpr int NDT = KP / 16;                   // Delta tiles incl. padding
      f32x4 D[NDT];
#pragma unroll
      for (int rt = 0; rt < NDT; ++rt) D[rt] = zero4();
      // U = (T diag(w)) V for this wave's channels, then Delta = U - W S^T
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        f32x4 u = zero4();
        constexpr int MAXST = MM::steps(BL);
#pragma unroll
        for (int p = 0; p < MAXST; ++p) {
          if (p >= MM::steps(16 * (rt + 1))) break;
          Frag ta = MM::ld_nat(sT, KP, 16 * rt + cc, p * KS);
          ta = FragScale<E>::apply(ta, sWg, p * KS);
          u = MM::mma(ta, MM::ld_nat(sVt, KP, e0 + cc, p * KS), u);
        }
        f32x4 ws = zero4();
#pragma unroll
        for (int p = 0; p < DK / KS; ++p) ws = MM::mma(MM::ld_cp(sW, DK, 16 * rt + cc, p), MM::from_c(St, p), ws);
        D[rt] = u - ws;
      }
      // O = Qdec S^T + P Delta
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int p = 0; p < DK / KS; ++p) acc = MM::mma(MM::ld_cp(sQd, DK, 16 * rt + cc, p), MM::from_c(St, p), acc);
#pragma unroll
        for (int p = 0; p < MM::steps(BL); ++p)
          if (p < MM::steps(16 * (rt + 1))) acc = MM::mma(MM::ld_cp(sP, KP, 16 * rt + cc, p), MM::from_c(D, p), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * gq + i;
          m_part += acc[i];
          if (r < nvalid) O[((size_t)(bidx * T + t0 + r) * H + h) * DV + e0 + cc] = from_f32<E>(acc[i]);
        }
      }
      // S^T <- diag(e^{G_BL}) S^T + Kdec^T Delta
#pragma unroll
      for (int dt = 0; dt < DK / 16; ++dt) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = St[dt][i] * sEgl[16 * dt + 4 * gq + i];
#pragma unroll
        for (int p = 0; p < MM::steps(BL); ++p) acc = MM::mma(MM::ld_cp(sKdT, KP, 16 * dt + cc, p), MM::from_c(D, p), acc);
        St[dt] = acc;
      }
    }
    __syncthreads();

    if (chunk_end) {
      const int count = min(L, T - chunk * L);
      const float tot = sum_groups(m_part);
      if (gq == 0) sM[e0 + cc] = tot / (float)count;
      m_part = 0.f;
      __syncthreads();
      if (t0 + BL < T) content_bias();
    }
  }

  // ------------------------------------------------ outputs
  if (a.state_out) {
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      float* s = a.state_out + ((size_t)bh * DV + e0 + cc) * DK + 16 * dt + 4 * gq;
      *reinterpret_cast<f32x4*>(s) = St[dt];
    }
  }
  if (a.mean_out)
    for (int e = tid; e < DV; e += NT) a.mean_out[(size_t)bh * DV + e] = sM[e];
}

}  // namespace carve
