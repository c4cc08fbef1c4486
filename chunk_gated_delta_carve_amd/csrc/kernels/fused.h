// One-pass chunk-parallel forward for d_k = d_v = 64, bf16, no content
// projection: a single launch in which
//   * one workgroup per (batch, head, 64-token block) runs the gate pass,
//     the gated Grams, the triangular inverse and the WY solve (the same
//     per-block operations as the chunk-serial kernel, block.h), forms the
//     block's affine map S <- S M + C and publishes only M^T and C^T (16 KiB)
//     through the L2; it keeps Q_eff = Qd - P W in LDS and O_loc = P U in
//     registers, waits for the state at its block start, and writes its own
//     output O = Q_eff S^T + O_loc (and the final chunk mean);
//   * one chain workgroup per (batch, head) stages the published maps in an
//     LDS ring (direct global-to-LDS loads by a loader wave) and carries the
//     state through the blocks on four waves, one per 16-channel value slice,
//     publishing the bf16 operand fragments of every block-start state.
// The per-block algebra and the readout o_t = S_{t-1} q_t are those of the
// gist.science technical summary (§2 and §2.1; one triangular system per
// block because every gate acts on the key axis, Theorem 11 of §3).
//
// Exchange through the L2. Workgroups are dealt to the XCDs round-robin by
// workgroup index, so a head's chain workgroup and all its block workgroups
// are given indices equal modulo 8: they share one L2, and plain stores,
// completed (s_waitcnt) before a flag is raised, are visible to a reader on
// that XCD that loads after seeing the flag. Every flag carries the writer's
// XCC id; a reader on another XCC flags an error (sticky word at the start of
// the workspace) and poisons its results with NaN instead of using data that
// might be stale. Every wait is bounded; a wait that runs out does the same.
//
// Deadlock freedom: chain workgroups have the lowest indices and never wait
// for anything but published maps; a block workgroup publishes its map before
// it waits, and blocks are numbered block-major, so the workgroups that a
// resident workgroup waits for have lower indices and were dispatched first.
//
// Flags are cleared by their single reader, so every call leaves the flag
// area zero; the workspace must be zero-filled before its first use.
#pragma once
#include "kernels.h"

namespace carve {

// Workspace of the one-pass schedule (byte offsets), for BH (batch, head)
// pairs of nblk 64-token blocks.
struct FusedWs {
  static constexpr int DK = 64, DV = 64, BL = 64, NW = DV / 16;
  static constexpr int MC_BYTES = 16384;   // M^T units (8 KiB) then C^T pairs (8 KiB)
  static constexpr int SF_BYTES = 2048;    // bf16 S operand fragments of one value slice
  int64_t err, fmc, fs, fmean, mpart, mc, sf, total;
  __host__ __device__ FusedWs(int64_t BH, int64_t nblk) {
    err = 0;                                 // int: bit 0 a wait ran out, bit 1 an XCC mismatch
    fmc = 256;                               // int [BH][nblk]: map of block published (XCC + 1)
    fs = fmc + BH * nblk * 4;                // int [BH][nblk][NW]: block-start state published
    fmean = fs + BH * nblk * NW * 4;         // int [BH][NW]: partial chunk sums published
    mpart = fmean + BH * NW * 4;             // f32 [BH][DV]: partial chunk sums
    mc = (mpart + BH * DV * 4 + 255) / 256 * 256;
    sf = mc + BH * nblk * MC_BYTES;          // [BH][nblk][NW][2][64 lanes][16 B]
    total = sf + BH * nblk * NW * SF_BYTES;
  }
};

// Chain workgroups come first; their count is rounded up to a multiple of 8 so
// that block workgroup i sits on XCD i mod 8 as well.
__host__ __device__ inline int fused_chains(int BH) { return (BH + 7) / 8 * 8; }
__host__ __device__ inline int64_t fused_grid(int BH, int nblk) {
  return fused_chains(BH) + (int64_t)8 * ((BH + 7) / 8) * nblk;
}

constexpr int kFusedRing = 3;               // LDS slots of the chain workgroup's map ring
constexpr int kFusedLag = 3;                // blocks between a state's fragment stores and its flag
constexpr int kFusedSpins = 1 << 22;        // bounded waits: polls of about 64+ cycles each

__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg(6164) & 15u; }   // HW_REG_XCC_ID[3:0]
__device__ __forceinline__ int ld_flag(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every vector memory operation of this wave (in particular its stores) has completed
__device__ __forceinline__ void drain_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <bool kLogits, bool kNorm>
__global__ void __launch_bounds__(64 * kIntraWaves)
carve_fused_kernel(FwdArgs a) {
  using E = bf16;
  constexpr int DK = 64, DV = 64, BL = 64;
  using B = Block<E, DK, DV, BL, kIntraWaves>;
  using LY = typename B::LY;
  using Unit = typename B::Unit;
  using Frag = typename B::Frag;
  using e4 = typename B::e4;
  using e8 = typename B::e8;
  using M16 = Mma16<E>;
  constexpr int NT = LY::NT, NB = LY::NB, TD = LY::TD, NU = LY::NU, NW = LY::NW, LK = LY::LK, LD = LY::LD;
  constexpr int NF = DK / Mma<E>::KS;
  constexpr int R = kFusedRing;
  static_assert(NT == 512 && NB == 4 && TD == 4 && NU == 2 && NW == 4 && NF == 2, "d = 64, 64-token blocks");
  static_assert(R * FusedWs::MC_BYTES + 64 <= LY::intra_bytes, "chain ring fits the intra LDS size");
  extern __shared__ __align__(16) unsigned char smem[];

  const int BH = a.B * a.H, T = a.T, H = a.H;
  const int nblk = (T + BL - 1) / BL;
  const FusedWs W(BH, nblk);
  unsigned char* ws = static_cast<unsigned char*>(a.ws);
  int* err = reinterpret_cast<int*>(ws + W.err);
  int* fmc = reinterpret_cast<int*>(ws + W.fmc);
  int* fs = reinterpret_cast<int*>(ws + W.fs);
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int gq = lane >> 4, cc = lane & 15;
  const int NC = fused_chains(BH);
  const int me = (int)xcc_id() + 1;         // flag value: this workgroup's XCC, plus one
  const uint32_t lo16 = 16u * lane;

  if ((int)blockIdx.x < NC) {
    // ================================================================ chain workgroup
    const int bh = blockIdx.x;
    if (bh >= BH) return;
    int* ready = reinterpret_cast<int*>(smem + R * FusedWs::MC_BYTES);   // blocks staged in the ring
    int* consumed = ready + 1;                                            // [NW] blocks done per slice
    int* lostp = ready + 1 + NW;                                          // a wait of this workgroup ran out
    if (threadIdx.x <= NW + 1) ready[threadIdx.x] = 0;
    __syncthreads();
    auto lds_ld = [](int* p) { return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); };
    auto lds_st = [](int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); };
    if (T == 0) {
      // nothing to carry: the outputs are the inputs
      if (wave < NW) {
        f32x4 St[TD];
        B::load_state(a.state_in, bh, wave, St);
        if (a.state_out) B::store_state(a.state_out, bh, wave, St);
      } else if (wave == NW && a.mean_out && lane < DV) {
        a.mean_out[(size_t)bh * DV + lane] = a.mean_in ? a.mean_in[(size_t)bh * DV + lane] : 0.f;
      }
      return;
    }
    const unsigned char* mc = ws + W.mc + (size_t)bh * nblk * FusedWs::MC_BYTES;
    unsigned char* sfb = ws + W.sf + (size_t)bh * nblk * NW * FusedWs::SF_BYTES;
    if (wave < NW) {
      // ---------------------------------------------------------- chain wave, value slice `wave`
      const int ws_ = wave;
      f32x4 St[TD];
      B::load_state(a.state_in, bh, ws_, St);
      Frag sf[NF];
      B::state_frags(St, sf);
      auto publish_frags = [&](int c) {
        unsigned char* p = sfb + ((size_t)c * NW + ws_) * FusedWs::SF_BYTES + lo16;
#pragma unroll
        for (int q = 0; q < NF; ++q) *reinterpret_cast<Frag*>(p + q * 1024) = sf[q];
      };
      publish_frags(0);
      // Block j's flag is raised K blocks later, once its fragment stores
      // have completed: vector memory operations of a wave complete in issue
      // order, and by then this wave has issued at least 2 K more (two
      // fragment stores per block, plus one flag per block from block K - 1
      // on: 2 K + j for j < K, 3 K after), so vmcnt(2 K) covers block j's
      // stores without waiting for the newest ones.
      constexpr int K = kFusedLag;
      int flagged = 0;
      bool lost = false;
      for (int c = 0; c < nblk; ++c) {
        // the map of block c is staged once `ready` passes c
        int spin = 0;
        while (!lost && lds_ld(ready) <= c) {
          if (++spin > kFusedSpins || lds_ld(lostp)) lost = true;
          else __builtin_amdgcn_s_sleep(1);
        }
        const unsigned char* slot = smem + (c % R) * FusedWs::MC_BYTES;
        f32x4 Ct[TD];
#pragma unroll
        for (int t = 0; t < TD / 2; ++t) {
          const e8 x = *reinterpret_cast<const e8*>(slot + 8192 + (ws_ * (TD / 2) + t) * 1024 + lo16);
#pragma unroll
          for (int i = 0; i < 4; ++i) { Ct[2 * t][i] = to_f32(x[i]); Ct[2 * t + 1][i] = to_f32(x[4 + i]); }
        }
        B::state_chain([&](int dt, int u) { return *reinterpret_cast<const Unit*>(slot + (dt * NU + u) * 1024 + lo16); },
                       Ct, sf, St);
        lds_st(&consumed[ws_], c + 1);              // the slot's reads are done (their values are in use)
        if (lost) {
          const float nan = __builtin_nanf("");
#pragma unroll
          for (int t = 0; t < TD; ++t) St[t] = f32x4{nan, nan, nan, nan};
        }
        if (c + 1 < nblk) {
          B::state_frags(St, sf);
          publish_frags(c + 1);
          if (c + 1 >= K) {
            static_assert(2 * kFusedLag <= 63, "vmcnt range");
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * K) : "memory");
            st_flag(fs + ((size_t)bh * nblk + flagged) * NW + ws_, me);
            ++flagged;
          }
        }
      }
      drain_vm();                                   // the last blocks' fragments
      for (; flagged < nblk; ++flagged) st_flag(fs + ((size_t)bh * nblk + flagged) * NW + ws_, me);
      if (lost && lane == 0) atomicOr(err, 1);
      if (a.state_out) B::store_state(a.state_out, bh, ws_, St);
    } else if (wave == NW) {
      // ---------------------------------------------------------- loader wave
      // Stages the maps of ready blocks into free ring slots in batches:
      // poll, copy (direct global-to-LDS, 16 units of 1 KiB per block), wait,
      // then publish the batch.
      // Each round trip copies the blocks found ready in the previous one
      // (as far as ring slots are free) and polls the flags of the next
      // candidates; one wait covers both.
      int staged = 0, known = 0;                     // blocks published in the ring / seen ready
      bool lost = false;
      int spin = 0;
      while (staged < nblk && !lost) {
        int done = lds_ld(&consumed[0]);
#pragma unroll
        for (int s2 = 1; s2 < NW; ++s2) done = min(done, lds_ld(&consumed[s2]));
        const int ncopy = min(known, done + R) - staged;   // ready blocks with a free slot
        for (int j = 0; j < ncopy; ++j) {
          const int c = staged + j;
          unsigned char* slot = smem + (c % R) * FusedWs::MC_BYTES;
          const unsigned char* src = mc + (size_t)c * FusedWs::MC_BYTES + lo16;
#pragma unroll
          for (int q = 0; q < 16; ++q)
            __builtin_amdgcn_global_load_lds(src + q * 1024, (__attribute__((address_space(3))) void*)(slot + q * 1024),
                                             16, 0, 0);
        }
        const int cand = known + lane;               // lane l polls block known + l
        int* f = fmc + (size_t)bh * nblk + cand;
        const int v = (lane < R && cand < nblk) ? ld_flag(f) : 0;
        const unsigned long long got = __ballot(v != 0);
        const int nnew = __builtin_ctzll(~got);      // ready blocks from `known` on
        if (lane < nnew) {
          if (v != me) atomicOr(err, 2);             // the map was written on another XCD
          st_flag(f, 0);
        }
        drain_vm();                                  // the copies have landed in LDS
        if (ncopy > 0) {
          staged += ncopy;
          lds_st(ready, staged);
        }
        known += nnew;
        if (ncopy > 0 || nnew > 0) {
          spin = 0;
        } else if (++spin > kFusedSpins) {
          lost = true;
        } else {
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (lost) {
        lds_st(lostp, 1);
        if (lane == 0) atomicOr(err, 1);
      }
    }
    return;
  }

  // ================================================================== block workgroup
  const int i = blockIdx.x - NC, x = i & 7, k = i >> 3, NHX = (BH + 7) / 8;
  const int blk = k / NHX, bh = x + 8 * (k % NHX);
  if (bh >= BH || blk >= nblk) return;               // uniform per workgroup
  const auto s = B::carve(smem);
  const Rows<E> src{static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v),
                    static_cast<const E*>(a.g), static_cast<const E*>(a.bx), static_cast<const E*>(a.w),
                    T, H, bh / H, bh % H};
  const int t0 = blk * BL;
  const int nvalid = min(BL, T - t0);
  unsigned char* mc = ws + W.mc + ((size_t)bh * nblk + blk) * FusedWs::MC_BYTES;
  unsigned char* qe = s.base + LY::oR1;              // Q_eff units [NB][NU][64 lanes][16 B]

  typename B::Raw raw;
  raw.template load<kNorm>(src, t0, nvalid);
  for (int d = threadIdx.x; d < DK; d += NT) s.Z[d] = 0.f;
  E qd[16];
  f32x4 Pt[B::TPW];
  const bool fallback = B::template gate_pass<false, kLogits, kNorm>(s, raw, nvalid, qd);
  B::template grams<kLogits, kNorm>(s, src, t0, nvalid, fallback, Pt);
  B::inverse_diag(s);
  // Affine map from the [W | U] tiles of this wave (as image_from_x in
  // block.h): W waves publish M^T half-units and keep Q_eff half-units in
  // LDS; U waves publish C^T and keep O_loc^T in registers.
  f32x4 Ol[NB];
  B::template solve_then<true>(s, qd, Pt, [&](const e4 (&X)[NB][B::CTW], bool isW, int x0) {
    static_assert(B::CTW == 1, "one [W | U] column tile per wave");
    auto rd = [&](const E* base, int pitch, int row, int I) {
      return *reinterpret_cast<const e4*>(base + row * pitch + 16 * I + 4 * gq);
    };
    if (isW) {
      const int kt = x0 / 16, u = kt / 2, half = kt % 2;
#pragma unroll
      for (int D = 0; D < TD; ++D) {
        f32x4 acc = zero4();
#pragma unroll
        for (int I = 0; I < NB; ++I) acc = M16::mma(X[I][0], rd(s.KdT, LK, 16 * D + cc, I), acc);
        const float eg = s.Egl[16 * D + cc];
        e4 v;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          v[ii] = from_f32<E>((16 * kt + 4 * gq + ii == 16 * D + cc ? eg : 0.f) - acc[ii]);
        *reinterpret_cast<e4*>(mc + ((D * NU + u) * 64 + lane) * 16 + half * 8) = v;
      }
#pragma unroll
      for (int Rr = 0; Rr < NB; ++Rr) {
        f32x4 acc = zero4();
#pragma unroll
        for (int I = 0; I <= Rr; ++I) acc = M16::mma(X[I][0], rd(s.P, LK, 16 * Rr + cc, I), acc);
        const e4 q = *reinterpret_cast<const e4*>(s.Qd + (16 * Rr + cc) * LD + 16 * kt + 4 * gq);
        e4 v;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v[ii] = from_f32<E>(to_f32(q[ii]) - acc[ii]);
        *reinterpret_cast<e4*>(qe + ((Rr * NU + u) * 64 + lane) * 16 + half * 8) = v;
      }
    } else {
      const int slice = x0 / 16;
      f32x4 Ct[TD];
#pragma unroll
      for (int D = 0; D < TD; ++D) {
        Ct[D] = zero4();
#pragma unroll
        for (int I = 0; I < NB; ++I) Ct[D] = M16::mma(rd(s.KdT, LK, 16 * D + cc, I), X[I][0], Ct[D]);
      }
#pragma unroll
      for (int Rr = 0; Rr < NB; ++Rr) {
        f32x4 acc = zero4();
#pragma unroll
        for (int I = 0; I <= Rr; ++I) acc = M16::mma(X[I][0], rd(s.P, LK, 16 * Rr + cc, I), acc);
        // O_loc^T in operand precision, as the image of the two-pass schedule holds it
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[ii] = to_f32(from_f32<E>(acc[ii]));
        Ol[Rr] = acc;
      }
      e8* ct = reinterpret_cast<e8*>(mc + 8192) + slice * (TD / 2) * 64 + lane;
#pragma unroll
      for (int aa = 0; aa < TD / 2; ++aa) ct[aa * 64] = B::pair(Ct[2 * aa], Ct[2 * aa + 1]);
    }
  });
  drain_vm();                                        // this wave's M^T / C^T stores have reached the L2
  __syncthreads();                                   // ... every wave's; Q_eff is complete in LDS
  if (threadIdx.x == 0) st_flag(fmc + (size_t)bh * nblk + blk, me);
  if (wave < kIntraWaves - NW) return;               // the W waves are done
  // ------------------------------------------------------------ output (U waves)
  const int slice = wave - (kIntraWaves - NW), e0 = 16 * slice;
  bool lost = false;
  {
    int* f = fs + ((size_t)bh * nblk + blk) * NW + slice;
    int v = 0, spin = 0;
    while ((v = ld_flag(f)) == 0) {
      if (++spin > kFusedSpins) { lost = true; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!lost) {
      if (v != me) lost = true;                      // written on another XCD: do not trust the data
      st_flag(f, 0);
    }
    if (lost && lane == 0) atomicOr(err, v == 0 ? 1 : 2);
  }
  asm volatile("" ::: "memory");                     // the fragments are read after the flag was seen
  Frag sf[NF];
  {
    const unsigned char* p = ws + W.sf + (((size_t)bh * nblk + blk) * NW + slice) * FusedWs::SF_BYTES + lo16;
#pragma unroll
    for (int q = 0; q < NF; ++q) sf[q] = *reinterpret_cast<const Frag*>(p + q * 1024);
  }
  f32x4 Ot[NB];
  B::state_out([&](int rt, int u) { return *reinterpret_cast<const Unit*>(qe + (rt * NU + u) * 1024 + lo16); },
               Ol, sf, Ot);
  if (lost) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) Ot[rt] = f32x4{nan, nan, nan, nan};
  }
  E* __restrict__ O = static_cast<E*>(a.o);
  const int bidx = bh / H, h = bh % H;
  const uint32_t olane = (uint32_t)(((size_t)cc * H * DV + (size_t)h * DV + e0 + 4 * gq) * sizeof(E));
  E* ob = O + ((size_t)bidx * T + t0) * H * DV;
#pragma unroll
  for (int rt = 0; rt < NB; ++rt) {
    const e4 v{from_f32<E>(Ot[rt][0]), from_f32<E>(Ot[rt][1]), from_f32<E>(Ot[rt][2]), from_f32<E>(Ot[rt][3])};
    if (16 * rt + 16 <= nvalid || 16 * rt + cc < nvalid)   // written once: streaming stores
      __builtin_nontemporal_store(v, reinterpret_cast<e4*>(reinterpret_cast<unsigned char*>(ob + (size_t)16 * rt * H * DV) + olane));
  }
  // The mean of the last chunk's outputs (the carried content state; it is
  // only returned, as nothing reads it without a projection). It lies in
  // this block, or (64 < L) in this block and the previous one, whose sums
  // come through the workspace.
  if (a.mean_out) {
    const int L = a.L;
    const int mstart = ((T - 1) / L) * L;
    const int first = mstart / BL;
    if (blk >= first) {
      f32x4 m_part = zero4();
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
        if (t0 + 16 * rt + cc >= mstart) m_part += Ot[rt];   // tokens past T are exactly 0
      const f32x4 tot = sum_cols(m_part);
      float* mp = reinterpret_cast<float*>(ws + W.mpart) + (size_t)bh * DV + e0 + 4 * gq;
      int* fm = reinterpret_cast<int*>(ws + W.fmean) + (size_t)bh * NW + slice;
      if (blk < nblk - 1) {
        // the previous block of a two-block last chunk: hand over the sums
        if (cc == 0) *reinterpret_cast<f32x4*>(mp) = tot;
        drain_vm();
        st_flag(fm, me);
      } else {
        f32x4 prev = zero4();
        if (first < blk) {
          int v = 0, spin = 0;
          bool lost2 = false;
          while ((v = ld_flag(fm)) == 0) {
            if (++spin > kFusedSpins) { lost2 = true; break; }
            __builtin_amdgcn_s_sleep(1);
          }
          if (!lost2) {
            st_flag(fm, 0);
            if (v != me) lost2 = true;
          }
          asm volatile("" ::: "memory");
          if (lost2) {
            if (lane == 0) atomicOr(err, v == 0 ? 1 : 2);
            const float nan = __builtin_nanf("");
            prev = f32x4{nan, nan, nan, nan};
          } else if (cc == 0) {
            prev = *reinterpret_cast<const f32x4*>(mp);
          }
        }
        if (cc == 0)
          *reinterpret_cast<f32x4*>(a.mean_out + (size_t)bh * DV + e0 + 4 * gq) =
              (prev + tot) * (1.0f / (float)(T - mstart));
      }
    }
  }
}

}  // namespace carve
