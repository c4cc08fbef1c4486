// One token of the CARVE recurrence for every (batch, head): the decode step.
//
// Per token (gist.science technical summaries of arXiv 2606.27229, §2.1 for
// the readout, the chunk mean and the one-chunk-stale erase gate, §2.2 for the
// scalar write gate, §2.3 for the key-axis decay; readings: b scales the
// retrieval key, decay precedes erase):
//   b = sigmoid(bx + U_up (U_down m_prev)),  o = S q,
//   S <- S diag(exp(g)),  S <- S + (w v - S (b * k)) k^T.
// The caller carries S, m_prev (the previous chunk's mean) and the running sum
// of this chunk's outputs; at the chunk's last position the chunk's mean
// replaces m_prev and the sum restarts from zero.
//
// One workgroup per (batch, head), four lanes per state row e: lane quarter
// p holds columns [p D/4, (p + 1) D/4) of row e in registers. The state is
// fp32 and all arithmetic is fp32, whatever the input type. The kernel is
// bound by streaming the state (read and written once per token).
#pragma once

#include "common.h"

namespace carve {

struct StepArgs {
  const void* q; const void* k; const void* v; const void* g; const void* bx; const void* w;
  const void* ub_down; const void* ub_up;
  float* state; float* mean_prev; float* chunk_acc;
  void* o;
  int B, H, L, rank, pos;
  int logits;   // nonzero: g holds raw decay logits a, and exp(g) = sigmoid(-a)
  int norm;     // nonzero: q and k are divided by their L2 norms (max(|x|, 1e-12))
};

template <typename E, int D>
__global__ void __launch_bounds__(4 * D)
carve_step_kernel(StepArgs a) {
  constexpr int NT = 4 * D, CW = D / 4;                // threads, columns per lane
  static_assert(CW % 4 == 0, "whole float4 column groups");
  __shared__ __align__(16) float qs[D], ks[D], dec[D], bk[D], vs[D], ms[D], bxs[D];
  __shared__ float ys[64], wsc, nrm[4];
  // this head's U_down [rank][D] and U_up [D][rank] (dynamic LDS, sized by the rank)
  extern __shared__ __align__(16) unsigned char dyn[];
  E* uds = reinterpret_cast<E*>(dyn);
  E* uus = uds + a.rank * D;
  const int tid = threadIdx.x, bh = blockIdx.x, h = bh % a.H;
  const size_t tok = (size_t)bh * D;                   // [B, 1, H, D]: row b H + h
  const E* q = static_cast<const E*>(a.q);
  const E* k = static_cast<const E*>(a.k);
  const E* v = static_cast<const E*>(a.v);
  const E* g = static_cast<const E*>(a.g);
  const E* bx = static_cast<const E*>(a.bx);
  // the state row segment first: its loads need nothing else, so their
  // latency overlaps the staging and the gate below
  const int e = tid >> 2, c0 = (tid & 3) * CW;
  float* srow = a.state + (tok + e) * D + c0;
  f32x4 s[CW / 4];
#pragma unroll
  for (int j = 0; j < CW / 4; ++j) s[j] = reinterpret_cast<const f32x4*>(srow)[j];
  if (tid < D) {
    qs[tid] = to_f32(q[tok + tid]);
    ks[tid] = to_f32(k[tok + tid]);
    const float gx = to_f32(g[tok + tid]);
    dec[tid] = a.logits ? sigmoid_f(-gx) : fast_exp2(gx * kLog2e);
    bxs[tid] = to_f32(bx[tok + tid]);
    vs[tid] = to_f32(v[tok + tid]);
    ms[tid] = a.mean_prev[tok + tid];
  }
  if (tid == 0) wsc = to_f32(static_cast<const E*>(a.w)[bh]);
  if (a.rank > 0) {
    const E* ud = static_cast<const E*>(a.ub_down) + (size_t)h * a.rank * D;
    const E* uu = static_cast<const E*>(a.ub_up) + (size_t)h * D * a.rank;
    for (int i = tid; i < a.rank * D; i += NT) {
      uds[i] = ud[i];
      uus[i] = uu[i];
    }
  }
  __syncthreads();
  if (a.norm) {                                        // q, k over their L2 norms (uniform branch)
    if (tid < D) {
      const float sq = wave_sum(qs[tid] * qs[tid]), sk = wave_sum(ks[tid] * ks[tid]);
      if ((tid & 63) == 0) {
        nrm[2 * (tid >> 6)] = sq;
        nrm[2 * (tid >> 6) + 1] = sk;
      }
    }
    __syncthreads();
    if (tid < D) {
      float sq = nrm[0], sk = nrm[1];
      if (D == 128) {
        sq += nrm[2];
        sk += nrm[3];
      }
      qs[tid] *= inv_norm(sq);
      ks[tid] *= inv_norm(sk);
    }
    __syncthreads();
  }
  // erase gate of this chunk: z = U_up (U_down m_prev), b = sigmoid(bx + z)
  if (a.rank > 0) {
    const int r = tid >> 2, sub = tid & 3;             // four lanes per rank row
    if (r < a.rank) {                                  // uniform across each quad
      const E* ud = uds + r * D;
      float p = 0.f;
      for (int e = sub; e < D; e += 4) p += to_f32(ud[e]) * ms[e];
      p = quad_sum(p);
      if (sub == 0) ys[r] = p;
    }
    __syncthreads();
    if (tid < D) {
      const E* uu = uus + tid * a.rank;
      float z = 0.f;
      for (int i = 0; i < a.rank; ++i) z += to_f32(uu[i]) * ys[i];
      bk[tid] = sigmoid_f(bxs[tid] + z) * ks[tid];
    }
  } else if (tid < D) {
    bk[tid] = sigmoid_f(bxs[tid]) * ks[tid];
  }
  __syncthreads();

  // readout before the update: o_e = S[e] . q
  float po = 0.f;
#pragma unroll
  for (int j = 0; j < CW / 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) po += s[j][i] * qs[c0 + 4 * j + i];
  const float o = quad_sum(po);
  // decay, then the erase-weighted retrieval of the decayed row
  float pr = 0.f;
#pragma unroll
  for (int j = 0; j < CW / 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[j][i] *= dec[c0 + 4 * j + i];
      pr += s[j][i] * bk[c0 + 4 * j + i];
    }
  const float delta = wsc * vs[e] - quad_sum(pr);
#pragma unroll
  for (int j = 0; j < CW / 4; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[j][i] += delta * ks[c0 + 4 * j + i];
    reinterpret_cast<f32x4*>(srow)[j] = s[j];
  }
  if ((tid & 3) == 0) {
    static_cast<E*>(a.o)[tok + e] = from_f32<E>(o);
    const float acc = a.chunk_acc[tok + e] + o;
    if (a.pos == a.L - 1) {                            // the chunk ends with this token
      a.mean_prev[tok + e] = acc * (1.0f / (float)a.L);
      a.chunk_acc[tok + e] = 0.f;
    } else {
      a.chunk_acc[tok + e] = acc;
    }
  }
}

}  // namespace carve
