// Backward pass of the CARVE layer: gradients of every input of the forward
// pass from the gradients of its outputs (o, the final state and the last
// chunk's mean). The layer is trained in the pages (gist.science technical
// summaries, §2 and the gradient-flow theorem of §3) but no backward pass is
// given; these are the exact derivatives of the forward pass as the header of
// carve.h defines it, through every path: the stale chunk mean passes
// gradient to the previous chunk's outputs and to mean_in, and the projection
// factors receive theirs through the erase gate (§2.1).
//
// Per token, with S' = S diag(e^g), r = S' (b*k), delta = w v - r and
// S_t = S' + delta k^T, the adjoint of S_t (dS) and the token's total output
// gradient dout give
//   d delta = dS k,  dr = -d delta,  dv = w d delta,  dw = <d delta, v>
//   dk = dS^T delta + (S'^T dr) * b,  db = (S'^T dr) * k,  dbx = db b (1 - b)
//   dS' = dS + dr (b*k)^T,  dg = column sums of dS' * S'
//   dq = S^T dout,  dS <- dS' diag(e^g) + dout q^T
// and dout of a token in chunk c adds dm_c / n_c (n_c tokens in the chunk),
// where dm_c is what chunk c + 1's gate z = U_up (U_down m_c) sends back.
//
// Schedule: one workgroup per (batch, head), four lanes per state row e, lane
// quarter p holding columns [p D/4, (p + 1) D/4) of S and of dS in registers.
//   1. A forward sweep stores the state at every chunk start, and each
//      chunk's gate bias z, gate mean m_{c-1} and U_down m_{c-1}.
//   2. For each chunk from the last: the chunk's states before each token are
//      recomputed from its checkpoint into the workspace, then the tokens are
//      walked backwards with dS in registers. Row sums (r, d delta) are quad
//      reductions; the column sums behind dk, db, dg and dq are reduced over
//      the rows of each wave with DPP row rotations and over the waves through
//      LDS, one barrier per token. At the chunk's start the gate's gradient
//      gives dU_up, dU_down (per (batch, head) partial sums) and dm_{c-1}.
// A second kernel sums the projection factors' partial gradients over the
// batch, in a fixed order.
#pragma once

#include "common.h"

namespace carve {

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* g; const void* bx; const void* w;
  const void* ub_down; const void* ub_up;
  const float* state_in; const float* mean_in;
  const void* d_o; const float* d_state_out; const float* d_mean_out;
  void* dq; void* dk; void* dv; void* dg; void* dbx; void* dw;
  float* d_state_in; float* d_mean_in;
  float* d_ub_down; float* d_ub_up;
  float* ws;
  int B, H, T, L, rank;
};

// Workspace of one (batch, head), in floats: the chunk checkpoints and the
// recomputed states of one chunk first (16-byte aligned), then the per-chunk
// gate vectors and the projection factors' partial gradients.
struct BwdWs {
  size_t ckpt, sbuf, z, m, y, dud, duu, total;
  __host__ __device__ BwdWs(int D, int T, int L, int rank) {
    const size_t nc = (size_t)(T + L - 1) / L, DD = (size_t)D * D;
    ckpt = 0;
    sbuf = ckpt + nc * DD;
    z = sbuf + (size_t)L * DD;
    m = z + nc * D;
    y = m + nc * D;
    dud = y + nc * rank;
    duu = dud + (size_t)rank * D;
    total = (duu + (size_t)D * rank + 3) & ~(size_t)3;
  }
};

// Sum over the four rows of a 16-lane DPP row that share this lane's column
// quarter (lanes i, i + 4, i + 8, i + 12 of the row), in every lane.
__device__ __forceinline__ float sum_row_quads(float x) {
  x += dpp_mov<0x128>(x);   // row_ror:8
  return x + dpp_mov<0x124>(x);   // row_ror:4
}
// Sum of the two 16-lane rows of each pair (rows 0 and 1, rows 2 and 3).
__device__ __forceinline__ float sum_row_pairs(float x) {
  const unsigned u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sum of the two halves of the wave.
__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D>
struct BwdLayout {
  static constexpr int NT = 4 * D, NW = NT / 64, CW = D / 4;
  // column partials per token: after the in-wave steps each wave leaves
  // PPW partial rows (4 with two DPP steps, 2 with the extra pair step)
  static constexpr int PPW = D == 64 ? 4 : 2;
  static constexpr int NP = NW * PPW;
  static constexpr int TOKF = 6 * D + 4;              // q, k, dec, b, v, dout, w (+pad)
  static constexpr int oTok = 0;                      // 3 token buffers
  static constexpr int oPart = oTok + 3 * TOKF;       // 2 x [NP][4][D]
  static constexpr int oWp = oPart + 2 * NP * 4 * D;  // 2 x [16] dw partials
  static constexpr int oZ = oWp + 32;                 // gate bias z of the chunk
  static constexpr int oM = oZ + D;                   // gate mean m_{c-1} of the chunk
  static constexpr int oDm = oM + D;                  // dm from the next chunk's gate
  static constexpr int oDmc = oDm + D;                // dm_c / n_c, added to dout
  static constexpr int oDz = oDmc + D;                // dz of the chunk
  static constexpr int oY = oDz + D;                  // U_down m_{c-1}
  static constexpr int oDy = oY + 64;                 // dy
  static constexpr int floats = oDy + 64;
  static constexpr int bytes = floats * 4;
  static_assert(TOKF % 4 == 0 && oPart % 4 == 0, "16-byte aligned LDS arrays");
};

template <typename E, int D, bool kLogits>
__global__ void __launch_bounds__(4 * D)
carve_bwd_kernel(BwdArgs a) {
  using LY = BwdLayout<D>;
  constexpr int NT = LY::NT, CW = LY::CW, NP = LY::NP, TOKF = LY::TOKF;
  constexpr size_t DD = (size_t)D * D;
  extern __shared__ __align__(16) float lds[];
  float* part0 = lds + LY::oPart;
  float* wp0 = lds + LY::oWp;
  float* zs = lds + LY::oZ;
  float* ms = lds + LY::oM;
  float* dms = lds + LY::oDm;
  float* dmcs = lds + LY::oDmc;
  float* dzs = lds + LY::oDz;
  float* ys = lds + LY::oY;
  float* dys = lds + LY::oDy;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = tid >> 2, seg = tid & 3, c0 = seg * CW;
  const int bh = blockIdx.x, bi = bh / a.H, h = bh % a.H;
  const int T = a.T, L = a.L, H = a.H, rank = a.rank;
  const int nc = (T + L - 1) / L;
  const bool content = rank > 0;
  const BwdWs lay(D, T, L, rank);
  float* ws = a.ws + (size_t)bh * lay.total;
  const E* Q = static_cast<const E*>(a.q);
  const E* K = static_cast<const E*>(a.k);
  const E* V = static_cast<const E*>(a.v);
  const E* G = static_cast<const E*>(a.g);
  const E* BX = static_cast<const E*>(a.bx);
  const E* W = static_cast<const E*>(a.w);
  const E* DO = static_cast<const E*>(a.d_o);
  const E* Ud = static_cast<const E*>(a.ub_down) + (size_t)h * rank * D;   // [rank][D]
  const E* Uu = static_cast<const E*>(a.ub_up) + (size_t)h * D * rank;     // [D][rank]
  auto tok_at = [&](int t) { return ((size_t)bi * T + t) * H + h; };      // row of [B, T, H, .]
  auto tokbuf = [&](int i) { return lds + LY::oTok + (i % 3) * TOKF; };

  // the token's vectors into an LDS buffer (threads d < D): q, k, the decay
  // factor, the erase gate b (with this chunk's z), v, and with `grad` the
  // total output gradient dout = do + dm_c / n_c
  auto stage = [&](float* tb, int t, bool grad) {
    if (tid < D) {
      const size_t off = tok_at(t) * D + tid;
      tb[tid] = to_f32(Q[off]);
      tb[D + tid] = to_f32(K[off]);
      tb[2 * D + tid] = fast_exp2(decay_log2<kLogits>(to_f32(G[off])));
      tb[3 * D + tid] = sigmoid_f(to_f32(BX[off]) + zs[tid]);
      tb[4 * D + tid] = to_f32(V[off]);
      if (grad) tb[5 * D + tid] = to_f32(DO[off]) + dmcs[tid];
    }
    if (tid == 0) tb[6 * D] = to_f32(W[tok_at(t)]);
  };

  // the content gate of a chunk from the mean in ms: ys = U_down m, zs = U_up ys
  auto gate = [&]() {
    const int r = tid >> 2, sub = tid & 3;
    if (r < rank) {                                  // uniform across each quad
      float p = 0.f;
      for (int j = sub; j < D; j += 4) p += to_f32(Ud[(size_t)r * D + j]) * ms[j];
      p = quad_sum(p);
      if (sub == 0) ys[r] = p;
    }
    __syncthreads();
    if (tid < D) {
      float z = 0.f;
      for (int i = 0; i < rank; ++i) z += to_f32(Uu[(size_t)tid * rank + i]) * ys[i];
      zs[tid] = z;
    }
  };

  // one token of the forward recurrence on this lane's row segment
  auto advance = [&](f32x4 (&s)[CW / 4], const float* tb) {
    const float* tq = tb;
    const float* tk = tb + D;
    const float* td = tb + 2 * D;
    const float* tbb = tb + 3 * D;
    float pr = 0.f;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + 4 * j + i;
        s[j][i] *= td[c];
        pr += s[j][i] * (tbb[c] * tk[c]);
      }
    (void)tq;
    const float delta = tb[6 * D] * tb[4 * D + e] - quad_sum(pr);
#pragma unroll
    for (int j = 0; j < CW / 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[j][i] += delta * tk[c0 + 4 * j + i];
  };

  // ---------------------------------------------------------------- forward sweep
  f32x4 s[CW / 4];
  {
    const float* sin = a.state_in ? a.state_in + (size_t)bh * DD + (size_t)e * D + c0 : nullptr;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) s[j] = sin ? reinterpret_cast<const f32x4*>(sin)[j] : zero4();
  }
  if (tid < D) {
    ms[tid] = a.mean_in ? a.mean_in[(size_t)bh * D + tid] : 0.f;
    zs[tid] = 0.f;
  }
  // the projection factors' partial gradients of this (batch, head) start at
  // zero; each element is cleared and later updated by the same thread
  for (int idx = tid; idx < rank * D; idx += NT) {
    ws[lay.dud + idx] = 0.f;
    ws[lay.duu + idx] = 0.f;
  }
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const int t0 = c * L, t1 = min(T, t0 + L);
    float* ck = ws + lay.ckpt + (size_t)c * DD + (size_t)e * D + c0;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) reinterpret_cast<f32x4*>(ck)[j] = s[j];
    if (content) {
      gate();
      if (tid < D) {
        ws[lay.z + (size_t)c * D + tid] = zs[tid];
        ws[lay.m + (size_t)c * D + tid] = ms[tid];
      }
      if (tid < rank) ws[lay.y + (size_t)c * rank + tid] = ys[tid];
      __syncthreads();
    }
    stage(tokbuf(0), t0, false);
    __syncthreads();
    float acc = 0.f;
    for (int t = t0; t < t1; ++t) {
      const float* tb = tokbuf(t - t0);
      if (t + 1 < t1) stage(tokbuf(t - t0 + 1), t + 1, false);
      if (content) {                                 // o_t = S_{t-1} q_t feeds the chunk mean
        float po = 0.f;
#pragma unroll
        for (int j = 0; j < CW / 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) po += s[j][i] * tb[c0 + 4 * j + i];
        acc += quad_sum(po);
      }
      advance(s, tb);
      __syncthreads();
    }
    if (content && seg == 0) ms[e] = acc / (float)(t1 - t0);
    __syncthreads();
  }

  // ---------------------------------------------------------------- reverse sweep
  f32x4 ds[CW / 4];
  {
    const float* dso = a.d_state_out ? a.d_state_out + (size_t)bh * DD + (size_t)e * D + c0 : nullptr;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) ds[j] = dso ? reinterpret_cast<const f32x4*>(dso)[j] : zero4();
  }
  if (tid < D) dms[tid] = 0.f;
  __syncthreads();
  const int ro = tid / D, rcol = tid % D;            // this thread's output: dk, dbx, dg or dq of column rcol
  float* sbuf = ws + lay.sbuf + (size_t)e * D + c0;
  for (int c = nc - 1; c >= 0; --c) {
    const int t0 = c * L, t1 = min(T, t0 + L), n = t1 - t0;
    if (tid < D) {
      float dm = dms[tid];
      if (c == nc - 1 && a.d_mean_out) dm += a.d_mean_out[(size_t)bh * D + tid];
      dmcs[tid] = dm / (float)n;
      zs[tid] = content ? ws[lay.z + (size_t)c * D + tid] : 0.f;
      if (content) ms[tid] = ws[lay.m + (size_t)c * D + tid];
    }
    if (tid < rank) ys[tid] = ws[lay.y + (size_t)c * rank + tid];
    __syncthreads();

    // states before each token of the chunk, from its checkpoint
    {
      const float* ck = ws + lay.ckpt + (size_t)c * DD + (size_t)e * D + c0;
#pragma unroll
      for (int j = 0; j < CW / 4; ++j) s[j] = reinterpret_cast<const f32x4*>(ck)[j];
    }
    stage(tokbuf(0), t0, false);
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
      float* sb = sbuf + (size_t)(t - t0) * DD;
#pragma unroll
      for (int j = 0; j < CW / 4; ++j) reinterpret_cast<f32x4*>(sb)[j] = s[j];
      const float* tb = tokbuf(t - t0);
      if (t + 1 < t1) stage(tokbuf(t - t0 + 1), t + 1, false);
      advance(s, tb);
      __syncthreads();
    }

    // backward through the chunk's tokens
    stage(tokbuf(0), t1 - 1, true);
    f32x4 sp[CW / 4];
    {
      const float* sb = sbuf + (size_t)(n - 1) * DD;
#pragma unroll
      for (int j = 0; j < CW / 4; ++j) sp[j] = reinterpret_cast<const f32x4*>(sb)[j];
    }
    __syncthreads();
    float dz = 0.f;
    for (int i = 0; i < n; ++i) {
      const int t = t1 - 1 - i;
      const float* tb = tokbuf(i);
      float* pb = part0 + (i & 1) * NP * 4 * D;
      float* wpb = wp0 + (i & 1) * 16;
      f32x4 spn[CW / 4];
      if (i + 1 < n) {
        const float* sb = sbuf + (size_t)(n - 2 - i) * DD;
#pragma unroll
        for (int j = 0; j < CW / 4; ++j) spn[j] = reinterpret_cast<const f32x4*>(sb)[j];
        stage(tokbuf(i + 1), t - 1, true);
      }
      const float* tq = tb;
      const float* tk = tb + D;
      const float* td = tb + 2 * D;
      const float* tbb = tb + 3 * D;
      const float wt = tb[6 * D], dout = tb[5 * D + e];
      float pr = 0.f, pdd = 0.f;
#pragma unroll
      for (int j = 0; j < CW / 4; ++j)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int cc = c0 + 4 * j + ii;
          pr += sp[j][ii] * td[cc] * (tbb[cc] * tk[cc]);
          pdd += ds[j][ii] * tk[cc];
        }
      const float delta = wt * tb[4 * D + e] - quad_sum(pr);
      const float ddelta = quad_sum(pdd);
      const float dr = -ddelta;
      if (seg == 0) static_cast<E*>(a.dv)[tok_at(t) * D + e] = from_f32<E>(wt * ddelta);
      // dw: sum over the rows of d delta * v
      {
        float pw = seg == 0 ? ddelta * tb[4 * D + e] : 0.f;
        pw = sum_halves(sum_row_pairs(sum_row_quads(pw)));
        if (lane == 0) wpb[wave] = pw;
      }
      // column partials of dS^T delta, S'^T dr, dS' * S' and S^T dout, four
      // columns at a time, summed over this wave's rows
#pragma unroll
      for (int j = 0; j < CW / 4; ++j) {
        f32x4 p1, p2, p3, p4;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int cc = c0 + 4 * j + ii;
          const float dec = td[cc];
          const float sd = sp[j][ii] * dec;
          const float dsd = ds[j][ii] + dr * (tbb[cc] * tk[cc]);
          p1[ii] = ds[j][ii] * delta;
          p2[ii] = sd * dr;
          p3[ii] = dsd * sd;
          p4[ii] = sp[j][ii] * dout;
          ds[j][ii] = dsd * dec + dout * tq[cc];
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          p1[ii] = sum_row_quads(p1[ii]);
          p2[ii] = sum_row_quads(p2[ii]);
          p3[ii] = sum_row_quads(p3[ii]);
          p4[ii] = sum_row_quads(p4[ii]);
          if constexpr (LY::PPW == 2) {
            p1[ii] = sum_row_pairs(p1[ii]);
            p2[ii] = sum_row_pairs(p2[ii]);
            p3[ii] = sum_row_pairs(p3[ii]);
            p4[ii] = sum_row_pairs(p4[ii]);
          }
        }
        // writers: the first quad of each DPP row (of each row pair)
        const bool writer = LY::PPW == 4 ? (lane & 12) == 0 : (lane & 28) == 0;
        if (writer) {
          const int p = wave * LY::PPW + (LY::PPW == 4 ? (lane >> 4) : (lane >> 5));
          float* dst = pb + (size_t)p * 4 * D + c0 + 4 * j;
          *reinterpret_cast<f32x4*>(dst) = p1;
          *reinterpret_cast<f32x4*>(dst + D) = p2;
          *reinterpret_cast<f32x4*>(dst + 2 * D) = p3;
          *reinterpret_cast<f32x4*>(dst + 3 * D) = p4;
        }
      }
      __syncthreads();
      // finish the column sums: thread (ro, rcol) forms one output element
      {
        float P = 0.f, P2 = 0.f;
        const int qsel = ro == 0 ? 0 : ro == 1 ? 1 : ro;   // dk: P1 (+ P2), dbx: P2, dg: P3, dq: P4
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          P += pb[(size_t)p * 4 * D + qsel * D + rcol];
          if (ro == 0) P2 += pb[(size_t)p * 4 * D + D + rcol];
        }
        const size_t off = tok_at(t) * D + rcol;
        const float b = tbb[rcol], kk = tk[rcol];
        if (ro == 0) {
          static_cast<E*>(a.dk)[off] = from_f32<E>(P + P2 * b);
        } else if (ro == 1) {
          const float dbx = P * kk * b * (1.f - b);
          static_cast<E*>(a.dbx)[off] = from_f32<E>(dbx);
          dz += dbx;
        } else if (ro == 2) {
          // dg, or with raw logits a (g = -softplus(a)) da = dg (e^g - 1)
          const float dg = kLogits ? P * (td[rcol] - 1.f) : P;
          static_cast<E*>(a.dg)[off] = from_f32<E>(dg);
        } else {
          static_cast<E*>(a.dq)[off] = from_f32<E>(P);
        }
        if (tid == 0) {
          float dw = 0.f;
#pragma unroll
          for (int ww = 0; ww < LY::NW; ++ww) dw += wpb[ww];
          static_cast<E*>(a.dw)[tok_at(t)] = from_f32<E>(dw);
        }
      }
      if (i + 1 < n) {
#pragma unroll
        for (int j = 0; j < CW / 4; ++j) sp[j] = spn[j];
      }
    }

    // the chunk's gate: z = U_up y, y = U_down m_{c-1}
    if (content) {
      if (ro == 1) dzs[rcol] = dz;
      __syncthreads();
      const int r = tid >> 2, sub = tid & 3;
      if (r < rank) {
        float p = 0.f;
        for (int d = sub; d < D; d += 4) p += to_f32(Uu[(size_t)d * rank + r]) * dzs[d];
        p = quad_sum(p);
        if (sub == 0) dys[r] = p;
      }
      for (int idx = tid; idx < D * rank; idx += NT)       // dU_up[d][i] += dz_d y_i
        ws[lay.duu + idx] += dzs[idx / rank] * ys[idx % rank];
      __syncthreads();
      for (int idx = tid; idx < rank * D; idx += NT)       // dU_down[i][e] += dy_i m_e
        ws[lay.dud + idx] += dys[idx / D] * ms[idx % D];
      if (tid < D) {
        float dm = 0.f;
        for (int r2 = 0; r2 < rank; ++r2) dm += to_f32(Ud[(size_t)r2 * D + tid]) * dys[r2];
        dms[tid] = dm;
      }
      __syncthreads();
    }
  }

  // gradients of the incoming state and mean
  if (a.d_state_in) {
    float* dsi = a.d_state_in + (size_t)bh * DD + (size_t)e * D + c0;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) reinterpret_cast<f32x4*>(dsi)[j] = ds[j];
  }
  if (a.d_mean_in && tid < D) {
    float dm;
    if (nc == 0) dm = a.d_mean_out ? a.d_mean_out[(size_t)bh * D + tid] : 0.f;
    else dm = content ? dms[tid] : 0.f;
    a.d_mean_in[(size_t)bh * D + tid] = dm;
  }
}

// dU_down [H][rank][D] and dU_up [H][D][rank]: sums of the per-(batch, head)
// partials over the batch, in batch order.
template <int D>
__global__ void carve_bwd_ub_kernel(const float* ws, size_t ws_per_bh, size_t dud_off, int B, int H, int rank,
                                    float* d_ub_down, float* d_ub_up) {
  const size_t per = (size_t)rank * D;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= 2 * per * H) return;
  const int which = (int)(idx / (per * H));
  const size_t rem = idx % (per * H);
  const int h = (int)(rem / per);
  const size_t i = rem % per;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += ws[((size_t)b * H + h) * ws_per_bh + dud_off + which * per + i];
  (which == 0 ? d_ub_down : d_ub_up)[(size_t)h * per + i] = s;
}

}  // namespace carve
