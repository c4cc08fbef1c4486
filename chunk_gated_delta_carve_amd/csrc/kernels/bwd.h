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
// Both schedules below share the plan:
//   1. A forward sweep stores the state at every chunk start (and, with a
//      projection, each chunk's gate bias z, gate mean m_{c-1} and
//      U_down m_{c-1}). Without a projection, in bf16 with L a multiple of
//      64, the forward's chunk-parallel pair has already written those
//      states (pre_ckpt) and the sweep is skipped.
//   2. For each chunk from the last: the chunk's states before each token are
//      recomputed from its checkpoint into the workspace, then the tokens are
//      walked backwards with dS in registers. Token inputs are staged into
//      LDS a block of tokens at a time.
// With a content projection (carve_bwd_kernel): one workgroup per (batch,
// head), four lanes per state row e, lane quarter p holding columns
// [p D/4, (p + 1) D/4) of S and dS. Row sums (r, d delta) are quad
// reductions; the column sums behind dk, db, dg and dq are reduced over the
// rows of each wave with DPP row rotations and over the waves through LDS,
// one barrier per token. At each chunk's start the gate's gradient gives
// dU_up, dU_down (per (batch, head) partial sums) and dm_{c-1}; a second
// kernel sums the partials over the batch in a fixed order.
// Without a projection the rows are independent and a head is split over
// several workgroups (carve_bwd_split_kernel and carve_bwd_finish_kernel,
// further down).
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
  int norm;   // nonzero: q, k are used over their L2 norms (inverse norms in the workspace)
  int detach; // nonzero: the gate's chunk means are constants (no dm from the gate)
  int pre_ckpt; // nonzero: the chunk-start states are already in the workspace (no forward sweep);
                // 2: in the layout of the chunk-parallel schedule (carve_bwd_chunk_kernel)
};

// Chunk groups of the row-lane schedule without a projection when the
// chunk-start states come from the forward pair (pre_ckpt): the state
// gradient at every chunk end is first carried back over all tokens alone
// (the dS sweep: its recurrence needs the inputs, not the forward states),
// and then up to kBwdGroups workgroups per row slice walk disjoint runs of
// chunks at once (16: measured 2% faster than 8, no slower than 32). Otherwise one workgroup walks all chunks.
constexpr int kBwdGroups = 16;
// Tokens per sub-block of the row-lane reverse walk: the walk keeps a
// sub-block's recomputed states in registers and stores only the state at
// each sub-block start.
constexpr int kBwdSub = 8;
__host__ __device__ inline int bwd_groups(int T, int L, int rank, bool pre_ckpt) {
  const int nc = L > 0 ? (T + L - 1) / L : 0;
  return pre_ckpt && rank == 0 && nc > 1 ? (nc < kBwdGroups ? nc : kBwdGroups) : 1;
}

// Workspace of one (batch, head), in floats: the chunk checkpoints and the
// recomputed states of one chunk per chunk group first (16-byte aligned),
// then, with several groups, the state gradient at every chunk end, then the
// per-chunk gate vectors and the projection factors' partial gradients.
// Row slices of the row-lane schedule (below): D / 16 without a projection;
// one slice of all D rows with a projection at D = 64; none otherwise (the
// per-head schedule).
__host__ __device__ constexpr int bwd_slices(int D, int rank) { return rank == 0 ? D / 16 : (D == 64 ? 1 : 0); }

// The row-lane schedule also keeps, per token and row slice, the slice's
// column sums (4 D floats) and its share of dw, for the kernel that adds up
// the slices and forms dk, dbx, dg and dq.
// With q, k normalisation it also keeps every token's inverse norms of q
// and k and the fp32 gradients of the normalised q and k, which a last
// kernel takes through the normalisation.
//
// The chunk-parallel schedule (carve_bwd_chunk_kernel, `chunked`) keeps only
// the state at every 64-token block start, the state gradient at every block
// end and each row's share of d_mean_out over the last chunk's tokens; with a
// projection (carve_bwd_chunk_serial_kernel) the states, gate biases and
// gate means of every chunk, one carried state gradient and the factor
// gradients' partial sums.
struct BwdWs {
  size_t ckpt, sbuf, sbuf_group, dsck, dmo, z, m, y, dud, duu, part, wpart, nrm, dqh, dkh, total;
  int groups;
  __host__ __device__ BwdWs(int D, int T, int L, int rank, bool norm, bool pre_ckpt, bool chunked = false) {
    const size_t nc = (size_t)(T + L - 1) / L, DD = (size_t)D * D;
    if (chunked) {                                     // per 64-token block, whatever L is
      const size_t nb = (size_t)(T + 63) / 64;
      groups = 1;
      ckpt = 0;
      sbuf = sbuf_group = 0;
      if (rank > 0) {
        // the per-head chunk walk of the content schedule (L = 64): the
        // carried state gradient, each chunk's gate bias and gate mean, and
        // the factor gradients' partial sums
        dsck = nb * DD;
        z = dsck + DD;
        m = z + nb * D;
        y = dud = m + nb * D;
        duu = dud + (size_t)rank * D;
        dmo = duu + (size_t)D * rank;
      } else {
        dsck = nb * DD;
        dmo = 2 * nb * DD;
        z = m = y = dud = duu = dmo + D;
      }
      // with q, k normalisation: every token's inverse norms and the fp32
      // gradients of the normalised q and k
      part = wpart = dmo + D;
      nrm = (dmo + D + 3) & ~(size_t)3;
      const size_t tn = norm ? (size_t)T : 0;
      dqh = nrm + 2 * tn;
      dkh = dqh + tn * D;
      total = (dkh + tn * D + 3) & ~(size_t)3;
      return;
    }
    groups = bwd_groups(T, L, rank, pre_ckpt);
    ckpt = 0;
    sbuf = ckpt + nc * DD;
    // recomputed states of one chunk per group: every token's for the
    // one-workgroup-per-head kernel (d = 128 with a projection), every
    // sub-block start for the row-lane kernel
    sbuf_group = (rank > 0 && D == 128 ? (size_t)L : (size_t)(L + kBwdSub - 1) / kBwdSub) * DD;
    dsck = sbuf + (size_t)groups * sbuf_group;
    dmo = z = dsck + (groups > 1 ? nc * DD : 0);
    m = z + nc * D;
    y = m + nc * D;
    dud = y + nc * rank;
    duu = dud + (size_t)rank * D;
    part = (duu + (size_t)D * rank + 3) & ~(size_t)3;
    const size_t slices = (size_t)bwd_slices(D, rank);
    wpart = part + (size_t)T * slices * 4 * D;
    nrm = (wpart + (size_t)T * slices + 3) & ~(size_t)3;
    const size_t tn = norm ? (size_t)T : 0;
    dqh = nrm + 2 * tn;
    dkh = dqh + tn * D;
    total = (dkh + tn * D + 3) & ~(size_t)3;
  }
};

// Sum over the four rows of a 16-lane DPP row that share this lane's column
// quarter (lanes i, i + 4, i + 8, i + 12 of the row), in every lane.
__device__ __forceinline__ float sum_row_quads(float x) {
  x += dpp_mov<0x128>(x);   // row_ror:8
  return x + dpp_mov<0x124>(x);   // row_ror:4
}

// Workgroup barrier that orders LDS only: this wave's LDS operations complete
// and become visible to the workgroup, while its global loads (prefetches)
// and stores stay in flight. No thread here passes global data to another
// thread of its workgroup (each reads back only what it wrote itself), so
// the kernel's barriers need no more than this.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D>
struct BwdLayout {
  static constexpr int NT = 4 * D, NW = NT / 64, CW = D / 4;
  // column partials per token: after the in-wave steps each wave leaves
  // PPW partial rows (4 with two DPP steps, 2 with the extra pair step)
  static constexpr int PPW = D == 64 ? 4 : 2;
  static constexpr int NP = NW * PPW;
  // tokens staged per LDS block (a divisor of every chunk length), and the
  // (token, channel) elements each thread stages
  static constexpr int NB = D == 64 ? 16 : 8;
  static constexpr int EPT = NB * D / NT;
  // tokens ahead that the states before a token are loaded (register ring
  // of PD + 1 sets; two ahead where the registers allow it)
  static constexpr int PD = D == 64 ? 2 : 1;
  static constexpr int TOKF = 6 * D + 4;              // q, k, dec, b, v, dout, w (+pad)
  static constexpr int oBlk = 0;                      // 2 x [NB][TOKF] token blocks
  static constexpr int oPart = oBlk + 2 * NB * TOKF;  // 2 x [NP][4][D]
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
  static_assert(EPT * NT == NB * D && NB <= 16, "whole staging shares");
};

template <typename E, int D, bool kLogits, bool kNorm>
__global__ void __launch_bounds__(4 * D)
carve_bwd_kernel(BwdArgs a) {
  using LY = BwdLayout<D>;
  constexpr int NT = LY::NT, CW = LY::CW, NP = LY::NP, TOKF = LY::TOKF, NB = LY::NB, EPT = LY::EPT;
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
  const BwdWs lay(D, T, L, rank, kNorm, a.pre_ckpt != 0);
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
  auto blockbuf = [&](int i) { return lds + LY::oBlk + (i & 1) * NB * TOKF; };

  // Token blocks: nb <= NB consecutive tokens from tb0, staged into LDS as
  // [token][q | k | dec | b | v | dout | w]. Loading (raw values into
  // registers, in the inputs' type, the token index clamped into the block so
  // no load sits under a branch) is split from storing (values converted,
  // decay factor and erase gate formed, the chunk's dm_c / n_c added to do)
  // so the next block's loads stay in flight during the current block's
  // work. Element r of a thread is (token, channel) = divmod(tid + r NT, D).
  struct Staged { E q[EPT], k[EPT], g[EPT], bx[EPT], v[EPT], dout[EPT], w; float nq[kNorm ? EPT : 1], nk[kNorm ? EPT : 1]; };
  auto load_block = [&](Staged& st, int tb0, int nb, bool grad) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int idx = tid + r * NT, j = min(idx / D, nb - 1), d = idx % D;
      const size_t off = tok_at(tb0 + j) * D + d;
      st.q[r] = Q[off];
      st.k[r] = K[off];
      if constexpr (kNorm) {                          // the tokens' inverse norms of q and k
        st.nq[r] = ws[lay.nrm + 2 * (size_t)(tb0 + j)];
        st.nk[r] = ws[lay.nrm + 2 * (size_t)(tb0 + j) + 1];
      }
      st.g[r] = G[off];
      st.bx[r] = BX[off];
      st.v[r] = V[off];
      st.dout[r] = grad ? DO[off] : from_f32<E>(0.f);
    }
    st.w = W[tok_at(tb0 + min(tid, nb - 1))];
  };
  auto store_block = [&](float* buf, const Staged& st, int nb) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int idx = tid + r * NT, j = idx / D, d = idx % D;
      if (j < nb) {
        float* tb = buf + j * TOKF;
        float qv = to_f32(st.q[r]), kv = to_f32(st.k[r]);
        if constexpr (kNorm) {                        // q, k over their norms
          qv *= st.nq[r];
          kv *= st.nk[r];
        }
        tb[d] = qv;
        tb[D + d] = kv;
        tb[2 * D + d] = fast_exp2(decay_log2<kLogits>(to_f32(st.g[r])));
        tb[3 * D + d] = sigmoid_f(to_f32(st.bx[r]) + zs[d]);
        tb[4 * D + d] = to_f32(st.v[r]);
        tb[5 * D + d] = to_f32(st.dout[r]) + dmcs[d];
      }
    }
    if (tid < nb) buf[tid * TOKF + 6 * D] = to_f32(st.w);
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
    const float* tk = tb + D;
    const float* td = tb + 2 * D;
    const float* tbb = tb + 3 * D;
    f32x4 pr = zero4();                              // four independent partial sums
#pragma unroll
    for (int j = 0; j < CW / 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + 4 * j + i;
        s[j][i] *= td[c];
        pr[i] += s[j][i] * (tbb[c] * tk[c]);
      }
    const float delta = tb[6 * D] * tb[4 * D + e] - quad_sum((pr[0] + pr[1]) + (pr[2] + pr[3]));
#pragma unroll
    for (int j = 0; j < CW / 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[j][i] += delta * tk[c0 + 4 * j + i];
  };

  // Forward over the tokens [t0, t1) of one chunk from the state in s, block
  // by block; `per_token(t, tb)` runs before each token's update.
  Staged st;
  auto sweep = [&](f32x4 (&s)[CW / 4], int t0, int t1, auto per_token) {
    const int nblk = (t1 - t0 + NB - 1) / NB;
    load_block(st, t0, min(NB, t1 - t0), false);
    store_block(blockbuf(0), st, min(NB, t1 - t0));
    lds_barrier();
    for (int jb = 0; jb < nblk; ++jb) {
      const int tb0 = t0 + jb * NB, nb = min(NB, t1 - tb0);
      const float* buf = blockbuf(jb);
      if (jb + 1 < nblk) load_block(st, tb0 + NB, min(NB, t1 - tb0 - NB), false);
      for (int j = 0; j < nb; ++j) {
        per_token(tb0 + j, buf + j * TOKF);
        advance(s, buf + j * TOKF);
      }
      if (jb + 1 < nblk) store_block(blockbuf(jb + 1), st, min(NB, t1 - tb0 - NB));
      lds_barrier();
    }
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
    dmcs[tid] = 0.f;
  }
  // the projection factors' partial gradients of this (batch, head) start at
  // zero; each element is cleared and later updated by the same thread
  for (int idx = tid; idx < rank * D; idx += NT) {
    ws[lay.dud + idx] = 0.f;
    ws[lay.duu + idx] = 0.f;
  }
  lds_barrier();
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
      lds_barrier();
    }
    float acc = 0.f;
    sweep(s, t0, t1, [&](int, const float* tb) {
      if (content) {                                 // o_t = S_{t-1} q_t feeds the chunk mean
        float po = 0.f;
#pragma unroll
        for (int j = 0; j < CW / 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) po += s[j][i] * tb[c0 + 4 * j + i];
        acc += quad_sum(po);
      }
    });
    if (content && seg == 0) ms[e] = acc / (float)(t1 - t0);
    lds_barrier();
  }

  // ---------------------------------------------------------------- reverse sweep
  f32x4 ds[CW / 4];
  {
    const float* dso = a.d_state_out ? a.d_state_out + (size_t)bh * DD + (size_t)e * D + c0 : nullptr;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) ds[j] = dso ? reinterpret_cast<const f32x4*>(dso)[j] : zero4();
  }
  if (tid < D) dms[tid] = 0.f;
  lds_barrier();
  const int ro = tid / D, rcol = tid % D;            // this thread's output: dk, dbx, dg or dq of column rcol
  float* sbuf = ws + lay.sbuf + (size_t)e * D + c0;
  for (int c = nc - 1; c >= 0; --c) {
    const int t0 = c * L, t1 = min(T, t0 + L), n = t1 - t0;
    if (tid < D) {
      zs[tid] = content ? ws[lay.z + (size_t)c * D + tid] : 0.f;
      if (content) ms[tid] = ws[lay.m + (size_t)c * D + tid];
      dmcs[tid] = 0.f;                                // the recompute stages no output gradient
    }
    if (tid < rank) ys[tid] = ws[lay.y + (size_t)c * rank + tid];
    lds_barrier();

    // states before each token of the chunk, from its checkpoint
    {
      const float* ck = ws + lay.ckpt + (size_t)c * DD + (size_t)e * D + c0;
#pragma unroll
      for (int j = 0; j < CW / 4; ++j) s[j] = reinterpret_cast<const f32x4*>(ck)[j];
    }
    sweep(s, t0, t1, [&](int t, const float*) {
      float* sb = sbuf + (size_t)(t - t0) * DD;
#pragma unroll
      for (int j = 0; j < CW / 4; ++j) reinterpret_cast<f32x4*>(sb)[j] = s[j];
    });
    if (tid < D) {
      float dm = dms[tid];
      if (c == nc - 1 && a.d_mean_out) dm += a.d_mean_out[(size_t)bh * D + tid];
      dmcs[tid] = dm / (float)n;
    }
    lds_barrier();

    // backward through the chunk's tokens: blocks of NB from the last, each
    // from its last token. The states before the tokens come from the
    // workspace through a ring of PD + 1 register sets, each load issued PD
    // tokens before its use; the loop is unrolled over the ring so every set
    // keeps a fixed register name while its load is in flight.
    const int nblk = (n + NB - 1) / NB;
    {
      const int tb0 = t0 + (nblk - 1) * NB, nb = t1 - tb0;
      load_block(st, tb0, nb, true);
      store_block(blockbuf(0), st, nb);
    }
    constexpr int PD = LY::PD, RING = PD + 1;
    f32x4 ring[RING][CW / 4];
    auto load_state = [&](f32x4 (&dst)[CW / 4], int t) {
      const float* sb = sbuf + (size_t)(t - t0) * DD;
#pragma unroll
      for (int jj = 0; jj < CW / 4; ++jj) dst[jj] = reinterpret_cast<const f32x4*>(sb)[jj];
    };
#pragma unroll
    for (int k = 0; k < PD; ++k)
      if (k < n) load_state(ring[k], t1 - 1 - k);
    lds_barrier();
    float dz = 0.f;

    auto step = [&](int i, const f32x4 (&sp)[CW / 4], f32x4 (&nxt)[CW / 4]) {
      const int t = t1 - 1 - i;
      const int jb = (t - t0) / NB, tb0 = t0 + jb * NB, j = t - tb0, kb = nblk - 1 - jb;
      if (t - PD >= t0) load_state(nxt, t - PD);
      if (t == min(tb0 + NB, t1) - 1 && jb > 0) load_block(st, tb0 - NB, NB, true);
      const float* tb = blockbuf(kb) + j * TOKF;
      float* pb = part0 + (i & 1) * NP * 4 * D;
      float* wpb = wp0 + (i & 1) * 16;
      const float* tq = tb;
      const float* tk = tb + D;
      const float* td = tb + 2 * D;
      const float* tbb = tb + 3 * D;
      const float wt = tb[6 * D], dout = tb[5 * D + e];
      f32x4 pr4 = zero4(), pdd4 = zero4();           // four independent partial sums each
#pragma unroll
      for (int jj = 0; jj < CW / 4; ++jj)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int cc = c0 + 4 * jj + ii;
          pr4[ii] += sp[jj][ii] * td[cc] * (tbb[cc] * tk[cc]);
          pdd4[ii] += ds[jj][ii] * tk[cc];
        }
      const float delta = wt * tb[4 * D + e] - quad_sum((pr4[0] + pr4[1]) + (pr4[2] + pr4[3]));
      const float ddelta = quad_sum((pdd4[0] + pdd4[1]) + (pdd4[2] + pdd4[3]));
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
      for (int jj = 0; jj < CW / 4; ++jj) {
        f32x4 p1, p2, p3, p4;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int cc = c0 + 4 * jj + ii;
          const float dec = td[cc];
          const float sd = sp[jj][ii] * dec;
          const float dsd = ds[jj][ii] + dr * (tbb[cc] * tk[cc]);
          p1[ii] = ds[jj][ii] * delta;
          p2[ii] = sd * dr;
          p3[ii] = dsd * sd;
          p4[ii] = sp[jj][ii] * dout;
          ds[jj][ii] = dsd * dec + dout * tq[cc];
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
          float* dst = pb + (size_t)p * 4 * D + c0 + 4 * jj;
          *reinterpret_cast<f32x4*>(dst) = p1;
          *reinterpret_cast<f32x4*>(dst + D) = p2;
          *reinterpret_cast<f32x4*>(dst + 2 * D) = p3;
          *reinterpret_cast<f32x4*>(dst + 3 * D) = p4;
        }
      }
      lds_barrier();
      // finish the column sums: thread (ro, rcol) forms one output element
      {
        f32x4 P = zero4(), P2 = zero4();
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          P[p & 3] += pb[(size_t)p * 4 * D + ro * D + rcol];
          if (ro == 0) P2[p & 3] += pb[(size_t)p * 4 * D + D + rcol];
        }
        const float Ps = (P[0] + P[1]) + (P[2] + P[3]);
        const size_t off = tok_at(t) * D + rcol;
        const float b = tbb[rcol], kk = tk[rcol];
        if (ro == 0) {                                 // dk = dS^T delta + (S'^T dr) b
          const float dkv = Ps + ((P2[0] + P2[1]) + (P2[2] + P2[3])) * b;
          if constexpr (kNorm) ws[lay.dkh + (size_t)t * D + rcol] = dkv;   // gradient of the normalised k
          else static_cast<E*>(a.dk)[off] = from_f32<E>(dkv);
        } else if (ro == 1) {                          // dbx = (S'^T dr) k b (1 - b)
          const float dbx = Ps * kk * b * (1.f - b);
          static_cast<E*>(a.dbx)[off] = from_f32<E>(dbx);
          dz += dbx;
        } else if (ro == 2) {
          // dg, or with raw logits a (g = -softplus(a)) da = dg (e^g - 1)
          const float dg = kLogits ? Ps * (td[rcol] - 1.f) : Ps;
          static_cast<E*>(a.dg)[off] = from_f32<E>(dg);
        } else {                                       // dq = S^T dout
          if constexpr (kNorm) ws[lay.dqh + (size_t)t * D + rcol] = Ps;
          else static_cast<E*>(a.dq)[off] = from_f32<E>(Ps);
        }
        if (tid == 0) {
          float dw = 0.f;
#pragma unroll
          for (int ww = 0; ww < LY::NW; ++ww) dw += wpb[ww];
          static_cast<E*>(a.dw)[tok_at(t)] = from_f32<E>(dw);
        }
      }
      if (j == 0 && jb > 0) {                          // the block's last token: stage the next block
        store_block(blockbuf(kb + 1), st, NB);
        lds_barrier();
      }
    };
    for (int i = 0; i < n; i += RING) {
      step(i, ring[0], ring[PD % RING]);
      if (i + 1 < n) step(i + 1, ring[1 % RING], ring[(1 + PD) % RING]);
      if constexpr (RING > 2) {
        if (i + 2 < n) step(i + 2, ring[2 % RING], ring[(2 + PD) % RING]);
      }
    }

    // the chunk's gate: z = U_up y, y = U_down m_{c-1}
    if (content) {
      if (ro == 1) dzs[rcol] = dz;
      lds_barrier();
      const int r = tid >> 2, sub = tid & 3;
      if (r < rank) {
        float p = 0.f;
        for (int d = sub; d < D; d += 4) p += to_f32(Uu[(size_t)d * rank + r]) * dzs[d];
        p = quad_sum(p);
        if (sub == 0) dys[r] = p;
      }
      for (int idx = tid; idx < D * rank; idx += NT)       // dU_up[d][i] += dz_d y_i
        ws[lay.duu + idx] += dzs[idx / rank] * ys[idx % rank];
      lds_barrier();
      for (int idx = tid; idx < rank * D; idx += NT)       // dU_down[i][e] += dy_i m_e
        ws[lay.dud + idx] += dys[idx / D] * ms[idx % D];
      if (tid < D) {
        float dm = 0.f;
        for (int r2 = 0; r2 < rank; ++r2) dm += to_f32(Ud[(size_t)r2 * D + tid]) * dys[r2];
        dms[tid] = a.detach ? 0.f : dm;
      }
      lds_barrier();
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

// ---------------------------------------------------------------------------
// Row-lane schedule: sixteen lanes per state row, each lane holding CW = D/16
// consecutive columns of S and dS; waves of four rows. Row sums are four DPP
// rotations inside a 16-lane row; the column sums over a wave's four rows
// are two lane swaps, over the workgroup's waves an LDS pass, and over the
// workgroups of a head a second kernel (carve_bwd_finish_kernel) that also
// forms dk, dbx, dg and dq from them.
//   Without a projection (kContent false) the gates do not depend on the
//   outputs, so the rows of S evolve independently: a head's rows are split
//   into D / 16 slices of four waves, one workgroup each, spreading a head
//   over several compute units.
//   With a projection (kContent true, D = 64) chunk c's gate reads the mean
//   of chunk c-1's outputs over every row, so one workgroup of D / 4 waves
//   holds all rows of a head (four waves per SIMD, hiding each other's
//   latency). It forms the chunk means and gates in the forward sweep, and in
//   the reverse sweep dz = sum of dbx over each chunk (from the per-token
//   column sums), then dm_{c-1} (fed into the previous chunk's output
//   gradients) and the per-(batch, head) partial sums of dU_up and dU_down.
template <int D, bool kContent>
struct SplitLayout {
  static constexpr int ROWS = kContent ? D : 16, NW = ROWS / 4, NT = 64 * NW;
  static constexpr int S = D / ROWS, CW = D / 16;
  static_assert(S == bwd_slices(D, kContent ? 1 : 0), "slices of the workspace layout");
  // tokens per staged block (blocks never cross a chunk boundary; a chunk
  // shorter than NB makes short blocks): 16, so that three workgroups fit a
  // CU's LDS and hide each other's latency (32 tokens took 83 KiB, one
  // workgroup per CU)
  static constexpr int NB = 16;
  static constexpr int TOKF = 4 * D + 2 * ROWS + 4;   // q, k, dec, b | v, dout of the rows | w
  static constexpr int EPT = NB * D / NT;             // (token, channel) elements staged per thread
  static constexpr int RPT = NB * ROWS / NT;          // (token, row) pairs of v and do per thread
  static constexpr int oBlk = 0;                      // 2 x [NB][TOKF]
  static constexpr int oPart = oBlk + 2 * NB * TOKF;  // 2 x [NW waves][4][D]
  static constexpr int oWp = oPart + 2 * NW * 4 * D;  // 2 x [NW] dw partials
  static constexpr int oVec = oWp + 2 * NW;           // per-chunk vectors (projection only)
  static constexpr int oZ = oVec, oM = oZ + D, oDm = oM + D, oDmc = oDm + D, oDz = oDmc + D, oY = oDz + D,
                       oDy = oY + 64;
  static constexpr int floats = oDy + 64;
  static constexpr int bytes = floats * 4;
  static_assert(TOKF % 4 == 0 && oPart % 4 == 0 && EPT * NT == NB * D && RPT * NT == NB * ROWS && NB <= NT &&
                NT <= 1024 && (!kContent || 4 * D <= NT), "layout");
};

// kDsSweep: the dS sweep of the chunk groups (no projection): the state
// gradient carried back over every token from d_state_out, stored at each
// chunk end; nothing else is written.
template <typename E, int D, bool kLogits, bool kContent, bool kNorm, bool kDsSweep = false>
__global__ void __launch_bounds__((SplitLayout<D, kContent>::NT))
carve_bwd_split_kernel(BwdArgs a) {
  static_assert(!(kDsSweep && kContent), "the dS sweep runs without a projection only");
  using LY = SplitLayout<D, kContent>;
  constexpr int NT = LY::NT, NW = LY::NW, CW = LY::CW, NB = LY::NB, TOKF = LY::TOKF, EPT = LY::EPT;
  constexpr int S = LY::S, ROWS = LY::ROWS, RPT = LY::RPT, SB = kBwdSub;
  static_assert(NB % SB == 0, "a sub-block lies inside one staged block");
  constexpr size_t DD = (size_t)D * D;
  extern __shared__ __align__(16) float lds[];
  float* part0 = lds + LY::oPart;
  float* wp0 = lds + LY::oWp;
  float* zs = lds + LY::oZ;       // chunk's gate bias z (zero without a projection)
  float* ms = lds + LY::oM;       // chunk's gate mean m_{c-1}
  float* dms = lds + LY::oDm;     // dm of the chunk's outputs from the next chunk's gate
  float* dmcs = lds + LY::oDmc;   // per row: dm_c / n_c, added to each output gradient
  float* dzs = lds + LY::oDz;
  float* ys = lds + LY::oY;
  float* dys = lds + LY::oDy;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, L = a.L, H = a.H, rank = kContent ? a.rank : 0;
  const int nc = (T + L - 1) / L;
  const BwdWs lay(D, T, L, rank, kNorm, a.pre_ckpt != 0);
  // workgroup: (batch, head), chunk group (the dS sweep has one), row slice
  const int NG = kDsSweep ? 1 : lay.groups;
  const int slice = blockIdx.x % S, grp = (blockIdx.x / S) % NG, bh = blockIdx.x / S / NG;
  const int bi = bh / a.H, h = bh % a.H;
  const int cpg = (nc + lay.groups - 1) / lay.groups;  // chunks per group
  const int c_lo = kDsSweep ? 0 : grp * cpg, c_hi = kDsSweep ? nc : min(nc, c_lo + cpg);
  if (c_lo >= c_hi && grp > 0) return;                 // an empty group (uniform per workgroup)
  const int rl = wave * 4 + (lane >> 4);              // row within the slice
  const int e = slice * ROWS + rl, cl = lane & 15, c0 = cl * CW;
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
  auto tok_at = [&](int t) { return ((size_t)bi * T + t) * H + h; };
  auto blockbuf = [&](int i) { return lds + LY::oBlk + (i & 1) * NB * TOKF; };

  // token blocks: [token][q | k | dec | b | v, dout of the rows | w]; b uses
  // the chunk's z, and dout adds the row's dm_c / n_c. The loads of a block
  // keep the inputs' own type and are converted only when the block is
  // staged into LDS, so they stay in flight while the previous block is
  // worked on; the token index is clamped into the block (rows past nb are
  // loaded again and never staged), so no load sits under a branch.
  struct Staged { E q[EPT], k[EPT], g[EPT], bx[EPT], v[RPT], dout[RPT], w; float nq[kNorm ? EPT : 1], nk[kNorm ? EPT : 1]; };
  auto load_block = [&](Staged& st, int tb0, int nb, bool grad) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int idx = tid + r * NT, j = min(idx / D, nb - 1), d = idx % D;
      const size_t off = tok_at(tb0 + j) * D + d;
      st.q[r] = Q[off];
      st.k[r] = K[off];
      st.g[r] = G[off];
      st.bx[r] = BX[off];
      if constexpr (kNorm) {                          // the tokens' inverse norms of q and k
        st.nq[r] = ws[lay.nrm + 2 * (size_t)(tb0 + j)];
        st.nk[r] = ws[lay.nrm + 2 * (size_t)(tb0 + j) + 1];
      }
    }
#pragma unroll
    for (int r2 = 0; r2 < RPT; ++r2) {
      const int idx = tid + r2 * NT, j = min(idx / ROWS, nb - 1), r = idx % ROWS;
      const size_t off = tok_at(tb0 + j) * D + slice * ROWS + r;
      st.v[r2] = V[off];
      st.dout[r2] = grad ? DO[off] : from_f32<E>(0.f);
    }
    st.w = W[tok_at(tb0 + min(tid, nb - 1))];
  };
  auto store_block = [&](float* buf, const Staged& st, int nb) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int idx = tid + r * NT, j = idx / D, d = idx % D;
      if (j < nb) {
        float* tb = buf + j * TOKF;
        float qv = to_f32(st.q[r]), kv = to_f32(st.k[r]);
        if constexpr (kNorm) {                        // q, k over their norms
          qv *= st.nq[r];
          kv *= st.nk[r];
        }
        tb[d] = qv;
        tb[D + d] = kv;
        tb[2 * D + d] = fast_exp2(decay_log2<kLogits>(to_f32(st.g[r])));
        tb[3 * D + d] = sigmoid_f(to_f32(st.bx[r]) + zs[d]);
      }
    }
#pragma unroll
    for (int r2 = 0; r2 < RPT; ++r2) {
      const int idx = tid + r2 * NT, j = idx / ROWS, r = idx % ROWS;
      if (j < nb) {
        buf[j * TOKF + 4 * D + r] = to_f32(st.v[r2]);
        buf[j * TOKF + 4 * D + ROWS + r] = to_f32(st.dout[r2]) + dmcs[r];
      }
    }
    if (tid < nb) buf[tid * TOKF + 4 * D + 2 * ROWS] = to_f32(st.w);
  };
  auto advance = [&](float (&s)[CW], const float* tb) {
    const float* tk = tb + D;
    const float* td = tb + 2 * D;
    const float* tbb = tb + 3 * D;
    float pr = 0.f;
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      s[j] *= td[c0 + j];
      pr += s[j] * (tbb[c0 + j] * tk[c0 + j]);
    }
    const float delta = tb[4 * D + 2 * ROWS] * tb[4 * D + rl] - sum_row16(pr);
#pragma unroll
    for (int j = 0; j < CW; ++j) s[j] += delta * tk[c0 + j];
  };
  Staged st;
  // forward over the tokens [t0, t1) of one chunk from the state in s;
  // per_token(t, tb) runs before each token's update
  auto sweep = [&](float (&s)[CW], int t0, int t1, auto per_token) {
    const int nblk = (t1 - t0 + NB - 1) / NB;
    load_block(st, t0, min(NB, t1 - t0), false);
    store_block(blockbuf(0), st, min(NB, t1 - t0));
    lds_barrier();
    for (int jb = 0; jb < nblk; ++jb) {
      const int tb0 = t0 + jb * NB, nb = min(NB, t1 - tb0);
      const float* buf = blockbuf(jb);
      if (jb + 1 < nblk) load_block(st, tb0 + NB, min(NB, t1 - tb0 - NB), false);
      for (int j = 0; j < nb; ++j) {
        per_token(tb0 + j, buf + j * TOKF);
        advance(s, buf + j * TOKF);
      }
      if (jb + 1 < nblk) store_block(blockbuf(jb + 1), st, min(NB, t1 - tb0 - NB));
      lds_barrier();
    }
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
  const size_t rowoff = (size_t)e * D + c0;
  auto ld = [&](float (&dst)[CW], const float* src) {
#pragma unroll
    for (int j = 0; j < CW; j += 4) *reinterpret_cast<f32x4*>(dst + j) = *reinterpret_cast<const f32x4*>(src + j);
  };
  auto st4 = [&](float* dst, const float (&src)[CW]) {
#pragma unroll
    for (int j = 0; j < CW; j += 4) *reinterpret_cast<f32x4*>(dst + j) = *reinterpret_cast<const f32x4*>(src + j);
  };

  // ---------------------------------------------------------------- forward sweep
  float s[CW];
  if (a.state_in) ld(s, a.state_in + (size_t)bh * DD + rowoff);
  else
#pragma unroll
    for (int j = 0; j < CW; ++j) s[j] = 0.f;
  if (tid < D) {
    zs[tid] = 0.f;
    dmcs[tid] = 0.f;
    dms[tid] = 0.f;
    if (kContent) ms[tid] = a.mean_in ? a.mean_in[(size_t)bh * D + tid] : 0.f;
  }
  if constexpr (kContent) {
    // this (batch, head)'s partial projection gradients start at zero; each
    // element is cleared and later updated by the same thread
    for (int idx = tid; idx < rank * D; idx += NT) {
      ws[lay.dud + idx] = 0.f;
      ws[lay.duu + idx] = 0.f;
    }
  }
  __syncthreads();
  const int nsweep = kContent || !a.pre_ckpt ? nc : 0;
  for (int c = 0; c < nsweep; ++c) {
    const int t0 = c * L, t1 = min(T, t0 + L);
    st4(ws + lay.ckpt + (size_t)c * DD + rowoff, s);
    if constexpr (kContent) {
      gate();
      if (tid < D) {
        ws[lay.z + (size_t)c * D + tid] = zs[tid];
        ws[lay.m + (size_t)c * D + tid] = ms[tid];
      }
      if (tid < rank) ws[lay.y + (size_t)c * rank + tid] = ys[tid];
      __syncthreads();
      float acc = 0.f;                                 // this row's outputs over the chunk
      sweep(s, t0, t1, [&](int, const float* tb) {
        float po = 0.f;
#pragma unroll
        for (int j = 0; j < CW; ++j) po += s[j] * tb[c0 + j];
        acc += sum_row16(po);
      });
      if (cl == 0) ms[e] = acc / (float)(t1 - t0);
      __syncthreads();
    } else {
      sweep(s, t0, t1, [](int, const float*) {});
    }
  }

  if constexpr (kDsSweep) {
    // -------------------------------------------------------------- dS sweep
    // The reverse walk's recurrence of the state gradient alone: per token,
    // with d delta = dS k,
    //   dS <- (dS - d delta (b k)^T) diag(e^g) + dout q^T,
    // which needs the inputs but not the forward states. dsck[c] receives the
    // dS that enters the reverse walk of chunk c (its value at the chunk's
    // end); chunk 0 is walked by its group only. The tokens of chunks nc - 1
    // .. 1 are one stream of NB-token blocks from the end (L is a multiple of
    // NB here, so no block crosses a chunk boundary), their loads issued two
    // blocks ahead through three register sets.
    float ds[CW];
    if (a.d_state_out) ld(ds, a.d_state_out + (size_t)bh * DD + rowoff);
    else
#pragma unroll
      for (int j = 0; j < CW; ++j) ds[j] = 0.f;
    float* dsck = ws + lay.dsck + rowoff;
    const int tl0 = (nc - 1) * L;                        // first token of the last chunk
    // this row's share of d_mean_out, added to each output gradient of the last chunk
    const float dml = a.d_mean_out ? a.d_mean_out[(size_t)bh * D + e] / (float)(T - tl0) : 0.f;
    const int nbt = (T + NB - 1) / NB, nwalk = nbt - L / NB;   // blocks of chunks nc - 1 .. 1
    auto tb0_of = [&](int kb) { return (nbt - 1 - kb) * NB; };
    auto nb_of = [&](int kb) { return min(NB, T - tb0_of(kb)); };
    Staged sets[3];
    load_block(sets[0], tb0_of(0), nb_of(0), true);
    if (1 < nwalk) load_block(sets[1], tb0_of(1), nb_of(1), true);
    store_block(blockbuf(0), sets[0], nb_of(0));
    lds_barrier();
    auto block = [&](int kb, Staged& next2, Staged& next1) {
      const int tb0 = tb0_of(kb), nb = nb_of(kb), c = tb0 / L;
      if (kb + 2 < nwalk) load_block(next2, tb0_of(kb + 2), nb_of(kb + 2), true);
      if (tb0 + nb == min(T, (c + 1) * L)) st4(dsck + (size_t)c * DD, ds);   // entering chunk c
      const float dm = tb0 >= tl0 ? dml : 0.f;
      const float* buf = blockbuf(kb);
#pragma unroll 4
      for (int j = nb - 1; j >= 0; --j) {
        const float* tb = buf + j * TOKF;
        float pdd = 0.f;
#pragma unroll
        for (int jj = 0; jj < CW; ++jj) pdd += ds[jj] * tb[D + c0 + jj];
        const float ddelta = sum_row16(pdd);
        const float dout = tb[4 * D + ROWS + rl] + dm;
#pragma unroll
        for (int jj = 0; jj < CW; ++jj) {
          const int cc = c0 + jj;
          ds[jj] = (ds[jj] - ddelta * (tb[3 * D + cc] * tb[D + cc])) * tb[2 * D + cc] + dout * tb[cc];
        }
      }
      if (kb + 1 < nwalk) store_block(blockbuf(kb + 1), next1, nb_of(kb + 1));
      lds_barrier();
    };
    for (int kb = 0; kb < nwalk; kb += 3) {
      block(kb, sets[2], sets[1]);
      if (kb + 1 < nwalk) block(kb + 1, sets[0], sets[2]);
      if (kb + 2 < nwalk) block(kb + 2, sets[1], sets[0]);
    }
    st4(dsck, ds);                                       // entering chunk 0
    return;
  }

  // ---------------------------------------------------------------- reverse sweep
  // this group's chunks [c_lo, c_hi), from the dS at the end of its last one
  float ds[CW];
  if (lay.groups > 1) ld(ds, ws + lay.dsck + (size_t)(c_hi - 1) * DD + rowoff);
  else if (a.d_state_out) ld(ds, a.d_state_out + (size_t)bh * DD + rowoff);
  else
#pragma unroll
    for (int j = 0; j < CW; ++j) ds[j] = 0.f;
  float* sbuf = ws + lay.sbuf + (size_t)grp * lay.sbuf_group + rowoff;
  float* gpart = ws + lay.part;                       // [T][S][4][D]
  float* gw = ws + lay.wpart;                         // [T][S]
  for (int c = c_hi - 1; c >= c_lo; --c) {
    const int t0 = c * L, t1 = min(T, t0 + L), n = t1 - t0;
    if (tid < D) {
      if (kContent) {
        zs[tid] = ws[lay.z + (size_t)c * D + tid];
        ms[tid] = ws[lay.m + (size_t)c * D + tid];
      }
      dmcs[tid] = 0.f;                                // the recompute stages no output gradient
    }
    if (kContent && tid < rank) ys[tid] = ws[lay.y + (size_t)c * rank + tid];
    __syncthreads();
    ld(s, ws + lay.ckpt + (size_t)c * DD + rowoff);
    // the state before every sub-block (every SB tokens from the chunk start)
    sweep(s, t0, t1, [&](int t, const float*) {
      if ((t - t0) % SB == 0) st4(sbuf + (size_t)((t - t0) / SB) * DD, s);
    });
    // each output gradient of the chunk gains dm_c / n: dm_c from the next
    // chunk's gate (with a projection) and, for the last chunk, d_mean_out
    if (tid < ROWS) {
      const int row = slice * ROWS + tid;
      float dm = kContent ? dms[row] : 0.f;
      if (c == nc - 1 && a.d_mean_out) dm += a.d_mean_out[(size_t)bh * D + row];
      dmcs[tid] = dm / (float)n;
    }
    __syncthreads();
    const int nblk = (n + NB - 1) / NB;
    {
      const int tb0 = t0 + (nblk - 1) * NB, nb = t1 - tb0;
      load_block(st, tb0, nb, true);
      store_block(blockbuf(0), st, nb);
    }
    lds_barrier();
    float dz = 0.f;                                    // this thread's column of dz (projection)
    // the staged inputs of token t (its block is in LDS while the walk is in it)
    auto tokbuf = [&](int t) {
      const int jb = (t - t0) / NB;
      return blockbuf(nblk - 1 - jb) + (t - t0 - jb * NB) * TOKF;
    };

    // token t's adjoint step, sp the state before the token
    auto step = [&](int t, const float (&sp)[CW]) {
      const int i = t1 - 1 - t;
      const int jb = (t - t0) / NB, tb0 = t0 + jb * NB, j = t - tb0, kb = nblk - 1 - jb;
      if (t == min(tb0 + NB, t1) - 1 && jb > 0) load_block(st, tb0 - NB, NB, true);
      const float* tb = blockbuf(kb) + j * TOKF;
      float* pb = part0 + (i & 1) * NW * 4 * D;
      float* wpb = wp0 + (i & 1) * NW;
      const float* tq = tb;
      const float* tk = tb + D;
      const float* td = tb + 2 * D;
      const float* tbb = tb + 3 * D;
      const float wt = tb[4 * D + 2 * ROWS], ve = tb[4 * D + rl], dout = tb[4 * D + ROWS + rl];
      float pr = 0.f, pdd = 0.f;
#pragma unroll
      for (int jj = 0; jj < CW; ++jj) {
        pr += sp[jj] * td[c0 + jj] * (tbb[c0 + jj] * tk[c0 + jj]);
        pdd += ds[jj] * tk[c0 + jj];
      }
      const float delta = wt * ve - sum_row16(pr);
      const float ddelta = sum_row16(pdd);
      const float dr = -ddelta;
      if (cl == 0) static_cast<E*>(a.dv)[tok_at(t) * D + e] = from_f32<E>(wt * ddelta);
      {                                                // dw share of this wave's four rows
        float pw = cl == 0 ? ddelta * ve : 0.f;
        pw = sum_halves(sum_row_pairs(pw));
        if (lane == 0) wpb[wave] = pw;
      }
      float p1[CW], p2[CW], p3[CW], p4[CW];
#pragma unroll
      for (int jj = 0; jj < CW; ++jj) {
        const int cc = c0 + jj;
        const float dec = td[cc];
        const float sd = sp[jj] * dec;
        const float dsd = ds[jj] + dr * (tbb[cc] * tk[cc]);
        p1[jj] = sum_halves(sum_row_pairs(ds[jj] * delta));
        p2[jj] = sum_halves(sum_row_pairs(sd * dr));
        p3[jj] = sum_halves(sum_row_pairs(dsd * sd));
        p4[jj] = sum_halves(sum_row_pairs(sp[jj] * dout));
        ds[jj] = dsd * dec + dout * tq[cc];
      }
      if (lane < 16) {                                 // one row of lanes writes the wave's sums
        float* dst = pb + wave * 4 * D + c0;
#pragma unroll
        for (int jj = 0; jj < CW; jj += 4) {
          *reinterpret_cast<f32x4*>(dst + jj) = f32x4{p1[jj], p1[jj + 1], p1[jj + 2], p1[jj + 3]};
          *reinterpret_cast<f32x4*>(dst + D + jj) = f32x4{p2[jj], p2[jj + 1], p2[jj + 2], p2[jj + 3]};
          *reinterpret_cast<f32x4*>(dst + 2 * D + jj) = f32x4{p3[jj], p3[jj + 1], p3[jj + 2], p3[jj + 3]};
          *reinterpret_cast<f32x4*>(dst + 3 * D + jj) = f32x4{p4[jj], p4[jj + 1], p4[jj + 2], p4[jj + 3]};
        }
      }
      lds_barrier();
      // the workgroup's column sums (over its waves) to the partial buffer,
      // output o = quantity * D + column; with a projection 4 D <= NT and
      // thread o keeps its column of dz (dbx summed over the chunk)
#pragma unroll
      for (int o = tid; o < 4 * D; o += NT) {
        f32x4 acc = zero4();
#pragma unroll
        for (int w = 0; w < NW; ++w) acc[w & 3] += pb[w * 4 * D + o];
        const float P = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        gpart[((size_t)t * S + slice) * 4 * D + o] = P;
        if (kContent && o >= D && o < 2 * D) {
          const float b = tbb[o - D];
          dz += P * tk[o - D] * b * (1.f - b);
        }
      }
      if (tid == 0) {
        float dw = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) dw += wpb[w];
        gw[(size_t)t * S + slice] = dw;
      }
      if (j == 0 && jb > 0) {                          // the block's last token: stage the next block
        store_block(blockbuf(kb + 1), st, NB);
        lds_barrier();
      }
    };
    // sub-blocks from the chunk's end: their states recomputed into registers
    // from the stored sub-block start (a sub-block lies inside one staged
    // block), then walked backwards
    const int nsb = (n + SB - 1) / SB;
    for (int q = nsb - 1; q >= 0; --q) {
      const int s0 = t0 + q * SB, s1 = min(t1, s0 + SB);
      float sts[SB][CW];
      ld(sts[0], sbuf + (size_t)q * DD);
#pragma unroll
      for (int u = 1; u < SB; ++u) {
        if (s0 + u < s1) {
#pragma unroll
          for (int jj = 0; jj < CW; ++jj) sts[u][jj] = sts[u - 1][jj];
          advance(sts[u], tokbuf(s0 + u - 1));
        }
      }
#pragma unroll
      for (int u = SB - 1; u >= 0; --u)
        if (s0 + u < s1) step(s0 + u, sts[u]);
    }

    // the chunk's gate: z = U_up y, y = U_down m_{c-1}
    if constexpr (kContent) {
      if (tid >= D && tid < 2 * D) dzs[tid - D] = dz;
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
        dms[tid] = a.detach ? 0.f : dm;
      }
      __syncthreads();
    }
  }
  if (grp > 0) return;                                // the incoming gradients belong to group 0
  if (a.d_state_in) st4(a.d_state_in + (size_t)bh * DD + rowoff, ds);
  if (a.d_mean_in && cl == 0) {
    // the incoming mean gates chunk 0 (with a projection); with T = 0 it
    // passes straight through to mean_out
    float dm;
    if (nc == 0) dm = a.d_mean_out ? a.d_mean_out[(size_t)bh * D + e] : 0.f;
    else dm = kContent ? dms[e] : 0.f;
    a.d_mean_in[(size_t)bh * D + e] = dm;
  }
}

// Sums the row slices' column sums of every (batch, token, head) and forms
// dk = P1 + P2 b, dbx = P2 k b (1 - b), dg = P3 (da = P3 (e^g - 1) with raw
// logits) and dq = P4, with b (using the chunk's z with a projection), k and
// the decay recomputed from the inputs; and dw from the slices' shares. One
// thread per (token row, channel).
template <typename E, int D, bool kLogits, bool kContent, bool kNorm>
__global__ void __launch_bounds__(256)
carve_bwd_finish_kernel(BwdArgs a) {
  constexpr int S = SplitLayout<D, kContent>::S;
  const size_t rows = (size_t)a.B * a.T * a.H;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * D) return;
  const size_t row = idx / D;                          // (b, t, h) in [B, T, H] order
  const int d = (int)(idx % D);
  const int h = (int)(row % a.H);
  const size_t bt = row / a.H;
  const int t = (int)(bt % a.T), bi = (int)(bt / a.T);
  const BwdWs lay(D, a.T, a.L, kContent ? a.rank : 0, kNorm, a.pre_ckpt != 0);
  float* ws = a.ws + ((size_t)bi * a.H + h) * lay.total;
  const float* gp = ws + lay.part + (size_t)t * S * 4 * D + d;
  float P[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sl = 0; sl < S; ++sl)
#pragma unroll
    for (int q = 0; q < 4; ++q) P[q] += gp[(sl * 4 + q) * D];
  const size_t off = row * D + d;
  float kk = to_f32(static_cast<const E*>(a.k)[off]);
  if constexpr (kNorm) kk *= ws[lay.nrm + 2 * (size_t)t + 1];
  const float z = kContent ? ws[lay.z + (size_t)(t / a.L) * D + d] : 0.f;
  const float b = sigmoid_f(to_f32(static_cast<const E*>(a.bx)[off]) + z);
  const float dec = fast_exp2(decay_log2<kLogits>(to_f32(static_cast<const E*>(a.g)[off])));
  static_cast<E*>(a.dbx)[off] = from_f32<E>(P[1] * kk * b * (1.f - b));
  static_cast<E*>(a.dg)[off] = from_f32<E>(kLogits ? P[2] * (dec - 1.f) : P[2]);
  if constexpr (kNorm) {                               // gradients of the normalised q, k
    ws[lay.dkh + (size_t)t * D + d] = P[0] + P[1] * b;
    ws[lay.dqh + (size_t)t * D + d] = P[3];
  } else {
    static_cast<E*>(a.dk)[off] = from_f32<E>(P[0] + P[1] * b);
    static_cast<E*>(a.dq)[off] = from_f32<E>(P[3]);
  }
  if (d == 0) {
    float dw = 0.f;
#pragma unroll
    for (int sl = 0; sl < S; ++sl) dw += ws[lay.wpart + (size_t)t * S + sl];
    static_cast<E*>(a.dw)[row] = from_f32<E>(dw);
  }
}

// q, k normalisation around the backward pass: one wave per (batch, token,
// head) row, D / 64 channels per lane.
//   carve_bwd_norms_kernel: the inverse norms 1 / max(|x|, 1e-12) of the row's
//   q and k, into the workspace of its (batch, head).
//   carve_bwd_unnorm_kernel: from the gradients g of the normalised q and k,
//   the gradients of the raw ones, (g - xh <xh, g>) / max(|x|, 1e-12) with
//   xh = x / max(|x|, 1e-12) (g / 1e-12 for a row of norm at most 1e-12).
template <typename E, int D, bool kNorms>
__global__ void __launch_bounds__(256)
carve_bwd_norm_kernel(BwdArgs a) {
  constexpr int CPL = D / 64;
  const size_t row = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;   // (b, t, h)
  const int lane = threadIdx.x & 63;
  if (row >= (size_t)a.B * a.T * a.H) return;          // whole waves leave together
  const int h = (int)(row % a.H);
  const size_t bt = row / a.H;
  const int t = (int)(bt % a.T), bi = (int)(bt / a.T);
  const BwdWs lay(D, a.T, a.L, a.rank, true, a.pre_ckpt != 0, a.pre_ckpt >= 2);
  float* ws = a.ws + ((size_t)bi * a.H + h) * lay.total;
  const E* Q = static_cast<const E*>(a.q) + row * D;
  const E* K = static_cast<const E*>(a.k) + row * D;
  float q[CPL], k[CPL], sq = 0.f, sk = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    q[c] = to_f32(Q[lane + 64 * c]);
    k[c] = to_f32(K[lane + 64 * c]);
    sq += q[c] * q[c];
    sk += k[c] * k[c];
  }
  const float iq = inv_norm(wave_sum(sq)), ik = inv_norm(wave_sum(sk));
  if constexpr (kNorms) {
    if (lane == 0) {
      ws[lay.nrm + 2 * (size_t)t] = iq;
      ws[lay.nrm + 2 * (size_t)t + 1] = ik;
    }
  } else {
    const float* gq = ws + lay.dqh + (size_t)t * D;
    const float* gk = ws + lay.dkh + (size_t)t * D;
    float dq = 0.f, dk = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      dq += q[c] * iq * gq[lane + 64 * c];
      dk += k[c] * ik * gk[lane + 64 * c];
    }
    dq = wave_sum(dq);
    dk = wave_sum(dk);
    E* DQ = static_cast<E*>(a.dq) + row * D;
    E* DK = static_cast<E*>(a.dk) + row * D;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int d = lane + 64 * c;
      const float vq = iq >= 1e12f ? gq[d] * iq : (gq[d] - q[c] * iq * dq) * iq;
      const float vk = ik >= 1e12f ? gk[d] * ik : (gk[d] - k[c] * ik * dk) * ik;
      DQ[d] = from_f32<E>(vq);
      DK[d] = from_f32<E>(vk);
    }
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
