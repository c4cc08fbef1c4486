// CARVE forward kernels for gfx950, all built from the per-block operations
// in block.h.
//
//   carve_chunk_serial_kernel  one workgroup per (batch, head) walks the
//       sequence block by block. Needed whenever the content projection U_b
//       is present: the erase gate of chunk c depends on the mean output of
//       chunk c-1, so every stage of a block waits for the previous block.
//   carve_intra_kernel + carve_state_kernel  used when U_b is absent: the
//       gates no longer depend on earlier outputs, so gate prep, the Grams,
//       the triangular inverse and W/U run for all blocks at once (one
//       workgroup per block); each block's state-pass operands go to a
//       workspace, and a per-(batch, head) kernel then runs only the serial
//       state update and the output.
// Both schedules compute the same per-block quantities and round the same
// intermediates to the input type. The chunk-parallel pair forms the affine
// maps with other products (from the solve's registers) and splits stages
// over the waves differently, so some fp32 sums run in another order: the two
// schedules agree to rounding, not bit for bit.
#pragma once
#include "block.h"

namespace carve {

// Largest rank of the content projection (checked on the host).
constexpr int kMaxRank = 64;

// Waves of a chunk-serial workgroup: eight at d_k = 64 with blocks of 32 or
// 64 tokens (two waves then share each 16-channel value slice of the state,
// each holding half of its key-channel tiles), else one per value slice.
template <int DK, int BL>
constexpr int serial_waves() { return DK == 64 && BL >= 32 ? 8 : DK / 16; }

// kLogits: the decay input g holds raw decay logits a, and the log-decay is
// -softplus(a), formed where g is read. kNorm: q and k are divided per token
// by their L2 norms over d_k where they are read. kCkpt: at every chunk start
// the state, the gate's bias z and the mean m_{c-1} behind it are stored for
// the backward pass (a.ckpt, a.ckpt_z, a.ckpt_m).
template <typename E, int DK, int DV, int BL, bool kLogits, bool kNorm, bool kCkpt = false>
__global__ void __launch_bounds__((BlockLayout<E, DK, DV, BL, serial_waves<DK, BL>()>::NT))
carve_chunk_serial_kernel(FwdArgs a) {
  using B = Block<E, DK, DV, BL, serial_waves<DK, BL>()>;
  using LY = typename B::LY;
  using MM = Mma<E>;
  using Frag = typename B::Frag;
  constexpr int NT = LY::NT, NB = LY::NB, TD = LY::TD, NU = LY::NU, NW = LY::NW, SPU = MM::SPU;
  constexpr int PARTS = LY::PARTS, TDP = TD / PARTS, NBP = NB / PARTS;   // state / output tiles per wave
  constexpr int NF = LY::NFR, NFP = NF / PARTS;                         // S fragments, per wave
  static_assert(TDP * PARTS == TD && NBP * PARTS == NB && NFP * PARTS == NF && NBP >= 1, "tile parts");
  extern __shared__ __align__(16) unsigned char smem[];
  const auto s = B::carve(smem);

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int gq = lane >> 4, cc = lane & 15;
  // value slice of this wave and its part: state tiles [TDP part, TDP (part + 1)),
  // output tiles [NBP part, NBP (part + 1))
  const int slice = wave % NW, part = wave / NW;
  const int bh = blockIdx.x;
  Rows<E> src{static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v),
              static_cast<const E*>(a.g), static_cast<const E*>(a.bx), static_cast<const E*>(a.w),
              a.T, a.H, bh / a.H, bh % a.H};
  const int h = src.h;
  const int T = a.T, L = a.L, rank = a.rank;
  E* __restrict__ O = static_cast<E*>(a.o);
  const E* Ud = static_cast<const E*>(a.ub_down);
  const E* Uu = static_cast<const E*>(a.ub_up);
  const int e0 = 16 * slice;
  Frag* xc = reinterpret_cast<Frag*>(smem + LY::oXc);        // [2][NW][NF][64]
  float* Mp = reinterpret_cast<float*>(smem + LY::oMp);      // [PARTS][DV]

  B::zero_lds(smem, LY::serial_bytes);
  const Sink<E> sink = B::lds_sink(s);
  // this wave's C tiles of S^T: rows d = 16 (TDP part + t) + 4g + i, column e0 + c
  f32x4 St[TDP];
  {
    const float* Sin = a.state_in ? a.state_in + ((size_t)bh * DV + e0 + cc) * DK + 4 * gq : nullptr;
#pragma unroll
    for (int t = 0; t < TDP; ++t) St[t] = Sin ? *reinterpret_cast<const f32x4*>(Sin + 16 * (TDP * part + t)) : zero4();
  }
  // this wave's S operand fragments into the exchange buffer of parity p
  auto share = [&](int p) {
    if constexpr (PARTS > 1) {
#pragma unroll
      for (int q = 0; q < NFP; ++q) xc[((p * NW + slice) * NF + NFP * part + q) * 64 + lane] = MM::from_c(St, q);
    }
  };
  __syncthreads();                                   // the LDS clear is complete
  share(0);
  for (int e = tid; e < DV; e += NT) s.M[e] = a.mean_in ? a.mean_in[(size_t)bh * DV + e] : 0.f;
  __syncthreads();

  // The content projection of this head stays in registers for the whole
  // sequence (the bias is recomputed at every chunk boundary, on the serial
  // chain, so it must not wait for memory). The chunk mean reaches it as the
  // column sums of each wave's own output tiles, so no wave waits for the
  // whole mean before it forms its share of y = U_down m:
  //   y_r: lane (g, c) holds U_down[h][r][e0 + 4g + i] (i < 4) for the rows
  //       r = c + 16 k of its value slice's channels (ud(k)); it multiplies
  //       them with its row group's channel sums, the four row groups are
  //       added with lane swaps, and the wave's partial sum of y_r goes to
  //       Yp[r][wave]; whoever forms z adds the partials of every wave;
  //   z_d = sum_r U_up[h][d][r] y_r: TPD = NT / DK lanes per key channel
  //       (d = tid / TPD), lane q = tid % TPD holds r = q + TPD i: uu(i).
  // Values stay in the input type, two per register for U_up; the sums over
  // a key channel's lanes are DPP moves inside quads and rows.
  constexpr int NWV = NT / 64, RKG = kMaxRank / 16;
  constexpr int TPD = NT / DK, RPT = kMaxRank / TPD;
  static_assert((TPD == 4 || TPD == 8) && RPT % 2 == 0 && NWV % 4 == 0, "lanes per key channel");
  typedef E e2 __attribute__((ext_vector_type(2)));
  const int zd = tid / TPD, zq = tid % TPD;
  float* Yp = reinterpret_cast<float*>(smem + LY::oYp);     // [kMaxRank][NWV]
  typename B::e4 ud[RKG];
  e2 uu[RPT / 2];
#pragma unroll
  for (int k = 0; k < RKG; ++k) {
    const int r = cc + 16 * k;
    ud[k] = r < rank ? *reinterpret_cast<const typename B::e4*>(Ud + ((size_t)h * rank + r) * DV + e0 + 4 * gq)
                     : typename B::e4{};
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = zq + TPD * i;
    uu[i / 2][i % 2] = r < rank ? Uu[((size_t)h * DK + zd) * rank + r] : from_f32<E>(0.f);
  }
  // z = U_up (U_down m) into s.Z with m = scale * (the sum over waves of tot),
  // tot: this wave's sums for channels e0 + 4g + i. With `mean` and several
  // waves per value slice, s.M = scale * (the parts' sums in Mp) as well.
  // All threads call; two barriers.
  auto content_bias = [&](const f32x4& tot, float scale, bool bias, bool mean) {
    if (bias && rank > 0) {
#pragma unroll
      for (int k = 0; k < RKG; ++k) {
        if (16 * k < rank) {                         // uniform
          float p = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) p += to_f32(ud[k][i]) * tot[i];
          p = sum_halves(sum_row_pairs(p));          // the four row groups: all 16 channels of the slice
          if (gq == 0) Yp[(16 * k + cc) * NWV + wave] = p;
        }
      }
    }
    __syncthreads();
    if (bias && rank > 0) {
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = zq + TPD * i;
        if (r < rank) {
          float y = 0.f;
#pragma unroll
          for (int w = 0; w < NWV; w += 4) {
            const f32x4 yv = *reinterpret_cast<const f32x4*>(Yp + r * NWV + w);
            y += (yv[0] + yv[1]) + (yv[2] + yv[3]);
          }
          z += to_f32(uu[i / 2][i % 2]) * y;
        }
      }
      z = quad_sum(z);
      if constexpr (TPD == 8) z += dpp_mov<0x114>(z);  // lanes 4..7 of an eight: the total
      if (zq == TPD - 1) s.Z[zd] = z * scale;
    }
    if constexpr (PARTS > 1) {
      if (mean)
        for (int e = tid; e < DV; e += NT) {
          float m = 0.f;
#pragma unroll
          for (int p = 0; p < PARTS; ++p) m += Mp[p * DV + e];
          s.M[e] = m * scale;
        }
    }
    __syncthreads();
  };
  {
    // the bias of the first chunk, from mean_in (part 0 of each slice holds it)
    f32x4 m0 = zero4();
    if (a.mean_in && part == 0) m0 = *reinterpret_cast<const f32x4*>(a.mean_in + (size_t)bh * DV + e0 + 4 * gq);
    content_bias(m0, 1.0f, true, false);
  }

  f32x4 m_part = zero4();               // running sums of O over tokens, channels e0 + 4g + i
  const int nblk = (T + BL - 1) / BL;
  using Unit = typename B::Unit;
  const Unit* mtu = sink.Mt;
  const Unit* qeu = sink.Qe;
  // Where the raw inputs of a block are fetched: with d_k = 64 or 16-token
  // blocks, those of block blk + 1 as soon as the gate pass has consumed
  // those of block blk. Wider heads with longer blocks have no registers to
  // spare during the Grams and the solve: with 64-token blocks the fetch of
  // block blk + 1 waits until the affine maps of block blk are formed (the
  // output, the chunk mean and the content bias still hide its latency);
  // 32-token blocks fetch their own inputs just before their gate pass
  // (measured faster than after the affine maps).
  constexpr int kFetch = DK == 64 || BL == 16 ? 0 : BL == 64 ? 1 : 2;   // after the gate pass, after affine, in place
  typename B::Raw raw;
  if (kFetch < 2 && nblk > 0) raw.template load<kNorm>(src, 0, min(BL, T));
  auto fetch_next = [&](int blk) {
    const int nb = min(blk + 1, nblk - 1);           // unconditional: keeps the load waits simple
    raw.template load<kNorm>(src, nb * BL, min(BL, T - nb * BL));
  };
  // the final mean in the order of the chunk-parallel state pass (see below)
  const bool lean_mean_out = LY::kLean && L == BL && a.mean_out != nullptr;
  for (int blk = 0; blk < nblk; ++blk) {
    const int t0 = blk * BL;
    const int nvalid = min(BL, T - t0);
    E qd[16];
    f32x4 Pt[B::TPW];
    if constexpr (kCkpt) {
      if (t0 % L == 0) {
        const int c = t0 / L;
        float* base = a.ckpt + (size_t)bh * a.ckpt_bh;
        float* S = base + (size_t)c * DV * DK + (size_t)(e0 + cc) * DK + 4 * gq;
#pragma unroll
        for (int t = 0; t < TDP; ++t) *reinterpret_cast<f32x4*>(S + 16 * (TDP * part + t)) = St[t];
        for (int e = tid; e < DK; e += NT) base[a.ckpt_z + (size_t)c * DK + e] = s.Z[e];
        for (int e = tid; e < DV; e += NT) base[a.ckpt_m + (size_t)c * DV + e] = s.M[e];
      }
    }
    if (kFetch == 2) raw.template load<kNorm>(src, t0, nvalid);
    const bool fallback = B::template gate_pass<true, kLogits, kNorm>(s, raw, nvalid, qd);
    if (kFetch == 0) fetch_next(blk);
    f32x4 CtR[TDP], OltR[NBP], Ot[NBP];
    // lean blocks (uniform: the flag is read after the gate pass's barrier)
    if (LY::kLean && !fallback) {
      if constexpr (LY::kLean) {
        const auto ln = B::lean(smem);
        B::lean_qd(ln, qd);
        B::grams_lean(s, ln);                        // ends with a barrier
        B::solve_affine_lean(s, ln, CtR, OltR);      // ends with a barrier (then part 0 reads Cx)
      }
    } else {
      B::template grams<kLogits, kNorm>(s, src, t0, nvalid, fallback, Pt);
      B::inverse_diag(s);
      B::solve(s, qd, Pt);
      B::affine(s, sink, CtR, OltR);                 // ends with a barrier
    }
    if (kFetch == 1) fetch_next(blk);
    // S operand fragments of the state at the block start: this wave's from
    // its registers, the other parts' from the exchange buffer
    Frag sf[NF];
#pragma unroll
    for (int p = 0; p < NF; ++p) {
      if (PARTS == 1 || p / NFP == part) sf[p] = MM::from_c(St, p % NFP);
      else sf[p] = xc[(((blk & 1) * NW + slice) * NF + p) * 64 + lane];
    }
    // O^T = S Qe^T + Ol^T and S^T <- Mt S^T + Ct for this wave's tiles
    // (reduction steps outermost)
#pragma unroll
    for (int j = 0; j < NBP; ++j) Ot[j] = OltR[j];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < SPU; ++i) {
#pragma unroll
        for (int j = 0; j < NBP; ++j)
          Ot[j] = MM::mma(sf[u * SPU + i], MM::step(qeu[((NBP * part + j) * NU + u) * 64 + lane], i), Ot[j]);
#pragma unroll
        for (int t = 0; t < TDP; ++t)
          CtR[t] = MM::mma(MM::step(mtu[((TDP * part + t) * NU + u) * 64 + lane], i), sf[u * SPU + i], CtR[t]);
      }
#pragma unroll
    for (int t = 0; t < TDP; ++t) St[t] = CtR[t];
    share((blk + 1) & 1);
#pragma unroll
    for (int j = 0; j < NBP; ++j) m_part += Ot[j];   // tokens past nvalid are exactly 0
    // O^T tile NBP part + j: lane (g, c) writes token t0 + 16 (NBP part + j) + c,
    // channels e0 + 4g .. e0 + 4g + 3
#pragma unroll
    for (int j = 0; j < NBP; ++j) {
      const int r = 16 * (NBP * part + j) + cc;
      if (r < nvalid)
        *reinterpret_cast<typename B::e4*>(O + src.row(t0 + r) * DV + e0 + 4 * gq) =
            typename B::e4{from_f32<E>(Ot[j][0]), from_f32<E>(Ot[j][1]), from_f32<E>(Ot[j][2]), from_f32<E>(Ot[j][3])};
    }
    // No barrier here: the next block's gate pass writes only LDS that this
    // block's output stage does not read (the S fragments and the Mt/Qe
    // units have their own areas), and at a chunk end the bias below holds
    // two barriers of its own.
    const bool chunk_end = ((t0 + BL) % L == 0) || (t0 + BL >= T);
    if (chunk_end) {
      const int chunk = t0 / L;
      const int count = min(L, T - chunk * L);
      // this wave's output sums over its tokens of the chunk, channels e0 + 4g + i
      f32x4 tot;
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[i] = sum_row16(m_part[i]);
      const float scale = 1.0f / (float)count;
      if constexpr (PARTS == 1) {
        if (cc == 0) *reinterpret_cast<f32x4*>(s.M + e0 + 4 * gq) = tot * scale;
      } else {
        if (cc == 0) *reinterpret_cast<f32x4*>(Mp + part * DV + e0 + 4 * gq) = tot;
      }
      // Lean blocks with one block per chunk: the final mean is summed in
      // the order of the chunk-parallel state pass (the four token tiles of
      // the last block in turn, then the columns by xor swaps), so that with
      // a zero projection this kernel's mean_out equals that of the pair
      // without one bit for bit, as its o and state do: part 0 hands its
      // running tile sum to part 1, which adds its own tiles after the
      // bias's first barrier.
      const bool lean_mean = lean_mean_out && t0 + BL >= T;   // uniform
      f32x4* xm = reinterpret_cast<f32x4*>(smem + LY::oLXm) + slice * 64 + lane;
      if (lean_mean && part == 0) *xm = m_part;
      m_part = zero4();
      content_bias(tot, scale, t0 + BL < T, true);
      if (lean_mean && part == 1) {
        f32x4 fin = *xm;
#pragma unroll
        for (int j = 0; j < NBP; ++j) fin += Ot[j];
        fin = sum_cols(fin);
        if (cc == 0) {
          float* mo = a.mean_out + (size_t)bh * DV + e0 + 4 * gq;
#pragma unroll
          for (int i = 0; i < 4; ++i) mo[i] = fin[i] * scale;
        }
      }
    }
  }
  if (a.state_out) {
    float* So = a.state_out + ((size_t)bh * DV + e0 + cc) * DK + 4 * gq;
#pragma unroll
    for (int t = 0; t < TDP; ++t) *reinterpret_cast<f32x4*>(So + 16 * (TDP * part + t)) = St[t];
  }
  // (the lean blocks' part-1 waves have written mean_out already)
  if (a.mean_out && !(lean_mean_out && T > 0))
    for (int e = tid; e < DV; e += NT) a.mean_out[(size_t)bh * DV + e] = s.M[e];
}

// Waves of an intra-kernel workgroup: eight, whatever the head width, so the
// stages of one block split over more waves and each block finishes sooner.
constexpr int kIntraWaves = 8;

// One workgroup per (batch, head, block): everything that does not depend on
// the state. Writes the block's state-pass operand image to the workspace.
// kLogits and kNorm as for the chunk-serial kernel.
template <typename E, int DK, int DV, int BL, bool kLogits, bool kNorm>
__global__ void __launch_bounds__((BlockLayout<E, DK, DV, BL, kIntraWaves>::NT))
carve_intra_kernel(FwdArgs a) {
  using B = Block<E, DK, DV, BL, kIntraWaves>;
  using LY = typename B::LY;
  constexpr int NT = LY::NT;
  static_assert(BL >= 32, "the image has no padding columns to clear");
  extern __shared__ __align__(16) unsigned char smem[];
  const auto s = B::carve(smem);

  const int nblk = (a.T + BL - 1) / BL;
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const Rows<E> src{static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v),
                    static_cast<const E*>(a.g), static_cast<const E*>(a.bx), static_cast<const E*>(a.w),
                    a.T, a.H, bh / a.H, bh % a.H};
  const int t0 = blk * BL;
  const int nvalid = min(BL, a.T - t0);
  unsigned char* img = static_cast<unsigned char*>(a.ws) + (size_t)blockIdx.x * LY::wBytes;

  typename B::Raw raw;
  raw.template load<kNorm>(src, t0, nvalid);
  // no content projection: the gate pass takes z = 0 without reading s.Z; the
  // zeros here serve only the pairwise fallback, several barriers later
  for (int d = threadIdx.x; d < DK; d += NT) s.Z[d] = 0.f;
  E qd[16];
  f32x4 Pt[B::TPW];
  const bool fallback = B::template gate_pass<false, kLogits, kNorm>(s, raw, nvalid, qd);
  B::template grams<kLogits, kNorm>(s, src, t0, nvalid, fallback, Pt);
  B::inverse_diag(s);
  B::template solve<true>(s, qd, Pt, img);           // also writes the block's image
}

// Output waves of a state-pass workgroup, next to its one chain wave.
constexpr int kOutWaves = 2;
constexpr int kStateThreads = 64 * (1 + kOutWaves);

// Placement of the state pass: one workgroup per (batch, head, 16-channel
// value slice). Workgroups are dealt to the XCDs round-robin, so the NW
// slices of one (batch, head) are given ids that are equal modulo 8: they
// then share one L2 for the block images they all read and for the output
// rows they write together.
__host__ __device__ inline int state_grid(int BH, int NW) { return (BH + 7) / 8 * 8 * NW; }
__device__ inline bool state_place(int id, int BH, int NW, int& bh, int& ws) {
  const int r = id / 8;
  ws = r % NW;
  bh = id % 8 + 8 * (r / NW);
  return bh < BH;
}

// Bounded waits between the waves of a state-pass workgroup: polls of an
// LDS counter (each sleeps about 64 cycles), far beyond any real wait.
constexpr int kRingSpins = 1 << 22;

// The serial state pass and the output of one (batch, head, value slice),
// split over the waves of a workgroup. Every wave is bound by the latency of
// its image loads, so the work is spread to keep more blocks in flight:
//   wave 0 (chain):     S^T <- M^T S^T + C^T through all blocks; before each
//                       block it publishes the S operand fragments (the
//                       state at the block start) in an LDS ring;
//   waves 1..K (output): wave 1 + o takes blocks o, o + K, o + 2K, ...:
//                       O^T = S Q_eff^T + O_loc^T from the ring, the output
//                       stores and its share of the last chunk's mean.
// Each wave loads its part of a block image into registers several of its
// blocks ahead (register sets rotated by unrolling its block loop); the
// loads of the last sets are clamped into range so that every set always
// has one load group in flight and the waits before a block cover only its
// own loads.
// kCkpt: the chain also stores the state entering every (1 << ckpt_shift)-th
// block at a.ckpt (a variant of its own, so the plain pass carries no check).
template <typename E, int DK, int DV, int BL, bool kCkpt = false>
__global__ void __launch_bounds__(kStateThreads)
carve_state_kernel(FwdArgs a) {
  using B = Block<E, DK, DV, BL>;
  using LY = typename B::LY;
  using Unit = typename B::Unit;
  using Frag = typename B::Frag;
  using e8 = typename B::e8;
  constexpr int NB = LY::NB, TD = LY::TD, NU = LY::NU, NW = LY::NW, NF = DK / Mma<E>::KS;
  constexpr int K = kOutWaves;
  // register sets of the chain wave (six with the checkpoint stores: eight
  // spilled there, 636 bytes per lane)
  constexpr int NSC = DK == 64 ? (kCkpt ? 6 : 8) : 2;
  constexpr int NSO = DK == 64 ? 4 : 2;                // register sets of an output wave
  constexpr int R = 8;                                 // ring slots
  __shared__ Frag ring[R][NF][64];
  __shared__ int produced, consumed[K];
  __shared__ __align__(16) float mtot[K][16];

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int gq = lane >> 4, cc = lane & 15;
  const int T = a.T, H = a.H, L = a.L;
  int bh, ws;
  if (!state_place(blockIdx.x, a.B * H, NW, bh, ws)) return;   // uniform per workgroup
  const int e0 = 16 * ws;
  const int nblk = (T + BL - 1) / BL;
  if (threadIdx.x == 0) produced = 0;
  if (threadIdx.x < K) consumed[threadIdx.x] = 0;
  __syncthreads();
  const unsigned char* imgs = static_cast<const unsigned char*>(a.ws) + (size_t)bh * nblk * LY::wBytes;
  auto img = [&](int blk) { return imgs + (size_t)min(blk, nblk - 1) * LY::wBytes; };
  bool lost = false;                                   // a wait ran out
  auto wait_for = [&](auto ready) {
    for (int spin = 0; spin < kRingSpins && !lost; ++spin) {
      if (ready()) return;
      __builtin_amdgcn_s_sleep(1);
    }
    lost = true;
  };
  auto load_acq = [](int* p) { return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); };
  auto store_rel = [](int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); };
  auto unpair = [](e8 x, f32x4& lo, f32x4& hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { lo[i] = to_f32(x[i]); hi[i] = to_f32(x[4 + i]); }
  };
  const uint32_t lo16 = 16u * lane;
  const int mstart = T > 0 ? ((T - 1) / L) * L : 0;   // first token of the last chunk

  if (wave == 0) {
    // ------------------------------------------------------------ chain
    struct Set { Unit mt[TD][NU]; e8 ct[TD / 2]; };
    auto fetch = [&](Set& r, int blk) {
      const unsigned char* p = img(blk);
#pragma unroll
      for (int t = 0; t < TD; ++t)
#pragma unroll
        for (int u = 0; u < NU; ++u)
          r.mt[t][u] = *reinterpret_cast<const Unit*>(p + LY::wMt + (t * NU + u) * 1024 + lo16);
#pragma unroll
      for (int t = 0; t < TD / 2; ++t)
        r.ct[t] = *reinterpret_cast<const e8*>(p + LY::wCt + (ws * (TD / 2) + t) * 1024 + lo16);
    };
    f32x4 St[TD];
    B::load_state(a.state_in, bh, ws, St);
    // the initial state lands before any image load is issued; otherwise the
    // waits in the block loop cannot tell its loads from the prefetches
    __builtin_amdgcn_s_waitcnt(0);
    Set set[NSC];
    int done = 0;                                     // every block below it has been read from the ring
    auto step = [&](int blk, Set& r, bool refill) {
      Frag sf[NF];
      B::state_frags(St, sf);
      if constexpr (kCkpt) {
        if ((blk & ((1 << a.ckpt_shift) - 1)) == 0) {   // the state entering the block
          float* S = a.ckpt + (size_t)bh * a.ckpt_bh + (size_t)(blk >> a.ckpt_shift) * (DV * DK);
#pragma unroll
          for (int dt = 0; dt < TD; ++dt)
            *reinterpret_cast<f32x4*>(S + (size_t)(e0 + cc) * DK + 16 * dt + 4 * gq) = St[dt];
        }
      }
      // Publish the previous block (its ring writes finished long ago, so the
      // release costs nothing), then make sure slot blk % R is free: block
      // blk - R must have been read by its output wave.
      store_rel(&produced, blk);
      if (blk - done >= R)
        wait_for([&] {
          int m = load_acq(&consumed[0]);
#pragma unroll
          for (int o = 1; o < K; ++o) m = min(m, load_acq(&consumed[o]));
          done = m;
          return blk - done < R;
        });
#pragma unroll
      for (int p = 0; p < NF; ++p) ring[blk % R][p][lane] = sf[p];
      f32x4 Ct[TD];
#pragma unroll
      for (int t = 0; t < TD / 2; ++t) unpair(r.ct[t], Ct[2 * t], Ct[2 * t + 1]);
      B::state_chain([&](int dt, int u) { return r.mt[dt][u]; }, Ct, sf, St);
      if (refill) fetch(r, blk + NSC);
    };
    if (nblk > 0) {
#pragma unroll
      for (int j = 0; j < NSC; ++j) fetch(set[j], j);
    }
    int blk = 0;
    for (; blk + NSC <= nblk; blk += NSC) {
#pragma unroll
      for (int j = 0; j < NSC; ++j) step(blk + j, set[j], true);
    }
#pragma unroll
    for (int j = 0; j < NSC - 1; ++j)
      if (blk + j < nblk) step(blk + j, set[j], false);
    store_rel(&produced, nblk);
    if (lost) {
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int t = 0; t < TD; ++t) St[t] = f32x4{nan, nan, nan, nan};
    }
    if (a.state_out) B::store_state(a.state_out, bh, ws, St);
  } else {
    // ------------------------------------------------------------ output
    const int o = wave - 1;
    struct Set { Unit qe[NB][NU]; e8 ol[NB / 2]; };
    auto fetch = [&](Set& r, int blk) {
      const unsigned char* p = img(blk);
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int u = 0; u < NU; ++u)
          r.qe[t][u] = *reinterpret_cast<const Unit*>(p + LY::wQe + (t * NU + u) * 1024 + lo16);
#pragma unroll
      for (int t = 0; t < NB / 2; ++t)
        r.ol[t] = *reinterpret_cast<const e8*>(p + LY::wOl + (ws * (NB / 2) + t) * 1024 + lo16);
    };
    E* __restrict__ O = static_cast<E*>(a.o);
    const int bidx = bh / H, h = bh % H;
    const uint32_t olane = (uint32_t)(((size_t)cc * H * DV + (size_t)h * DV + e0 + 4 * gq) * sizeof(E));
    f32x4 m_part = zero4();
    Set set[NSO];
    int seen = 0;                                     // last value of `produced` read
    auto step = [&](int blk, Set& r, bool refill) {
      // release the slots of this wave's earlier blocks (their ring reads are
      // done), then wait until this block's fragments are published
      store_rel(&consumed[o], blk);
      if (seen <= blk) wait_for([&] { seen = load_acq(&produced); return seen > blk; });
      Frag sf[NF];
#pragma unroll
      for (int p = 0; p < NF; ++p) sf[p] = ring[blk % R][p][lane];
      f32x4 Olt[NB], Ot[NB];
#pragma unroll
      for (int t = 0; t < NB / 2; ++t) unpair(r.ol[t], Olt[2 * t], Olt[2 * t + 1]);
      B::state_out([&](int rt, int u) { return r.qe[rt][u]; }, Olt, sf, Ot);
      if (lost) {                                     // the ring slot may be stale: poison o too
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) Ot[rt] = f32x4{nan, nan, nan, nan};
      }
      if (refill) fetch(r, blk + NSO * K);
      const int t0 = blk * BL;
      if (t0 + BL > mstart) {                         // the block reaches into the last chunk
#pragma unroll
        for (int rt = 0; rt < NB; ++rt)
          if (t0 + 16 * rt + cc >= mstart) m_part += Ot[rt];   // tokens past T are exactly 0
      }
      // O^T tile rt: lane (g, c) writes token t0 + 16 rt + c, channels e0 + 4g .. e0 + 4g + 3
      E* ob = O + ((size_t)bidx * T + t0) * H * DV;     // uniform
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const typename B::e4 v{from_f32<E>(Ot[rt][0]), from_f32<E>(Ot[rt][1]), from_f32<E>(Ot[rt][2]),
                               from_f32<E>(Ot[rt][3])};
        if (t0 + 16 * rt + 16 <= T || t0 + 16 * rt + cc < T)
          *reinterpret_cast<typename B::e4*>(reinterpret_cast<unsigned char*>(ob + (size_t)16 * rt * H * DV) + olane) = v;
      }
    };
    // this wave's blocks: o + K i for i < mine
    const int mine = nblk > o ? (nblk - o + K - 1) / K : 0;
#pragma unroll
    for (int j = 0; j < NSO; ++j)
      if (mine > 0) fetch(set[j], o + K * j);
    int i = 0;
    for (; i + NSO <= mine; i += NSO) {
#pragma unroll
      for (int j = 0; j < NSO; ++j) step(o + K * (i + j), set[j], true);
    }
#pragma unroll
    for (int j = 0; j < NSO - 1; ++j)
      if (i + j < mine) step(o + K * (i + j), set[j], false);
    store_rel(&consumed[o], nblk);
    if (lost) m_part = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    const f32x4 tot = sum_cols(m_part);
    if (cc == 0) *reinterpret_cast<f32x4*>(&mtot[o][4 * gq]) = tot;
  }
  __syncthreads();
  // the mean of the last chunk's outputs, from the output waves' shares
  if (a.mean_out && wave == 1 && lane < 16) {
    float* mo = a.mean_out + (size_t)bh * DV + e0 + lane;
    if (T == 0) {
      *mo = a.mean_in ? a.mean_in[(size_t)bh * DV + e0 + lane] : 0.f;
    } else {
      float tot = 0.f;
#pragma unroll
      for (int o = 0; o < K; ++o) tot += mtot[o][lane];
      *mo = tot * (1.0f / (float)(T - mstart));
    }
  }
}

}  // namespace carve
