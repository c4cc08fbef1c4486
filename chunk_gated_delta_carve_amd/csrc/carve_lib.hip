// Host side of the CARVE C ABI: validation, shape contract, dispatch.
// Every check runs before the first HIP call so argument errors are reported
// (and unit-testable) on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>

#include "carve.h"
#include "kernels/kernels.h"
#include "kernels/bwd.h"
#include "kernels/bwd_chunk.h"
#include "kernels/step.h"

namespace {

thread_local char g_hip_msg[256] = "no HIP error recorded";

size_t elem_bytes(int dtype) { return dtype == CARVE_F32 ? 4 : 2; }

bool valid_width(int d) { return d == 64 || d == 128; }
bool valid_chunk(int L) { return L == 16 || L == 32 || L == 64 || L == 128; }

int check_config(const carve_config* c) {
  if (!c) return CARVE_EINVAL;
  if (c->B < 0 || c->H < 0 || c->T < 0 || c->rank < 0) return CARVE_EINVAL;
  if (c->dtype != CARVE_F32 && c->dtype != CARVE_BF16) return CARVE_EINVAL;
  if (!valid_width(c->dk) || !valid_width(c->dv) || c->dk != c->dv) return CARVE_EUNSUPPORTED;
  if (!valid_chunk(c->L)) return CARVE_EUNSUPPORTED;
  if (c->rank > 64) return CARVE_EUNSUPPORTED;
  if (c->flags & ~(CARVE_DECAY_LOGITS | CARVE_QK_L2NORM | CARVE_DETACH_MEAN)) return CARVE_EINVAL;
  // offsets are computed in 64-bit, grids in 32-bit (the state pass launches
  // 8 (B H / 8 rounded up) (d_v / 16) workgroups)
  if ((int64_t)c->B * c->H > 0x7fffffffLL / 8 - 8) return CARVE_EUNSUPPORTED;
  // (batch, head, block) items of the chunk-parallel kernels are counted in int
  if ((int64_t)c->B * c->H * ((c->T + 63) / 64) > 0x7fffffffLL) return CARVE_EUNSUPPORTED;
  // per-lane output offsets inside 16 token rows are 32-bit, and so are the
  // per-lane input offsets inside one block of up to 64 token rows
  if ((int64_t)16 * c->H * c->dv * elem_bytes(c->dtype) > 0x7fffffffLL) return CARVE_EUNSUPPORTED;
  if ((int64_t)64 * c->H * (c->dk > c->dv ? c->dk : c->dv) * elem_bytes(c->dtype) > 0xffffffffLL)
    return CARVE_EUNSUPPORTED;
  return CARVE_OK;
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// block length used by the chunk-serial kernel: divides L, fits LDS
int serial_block(const carve_config* c) {
  int bl = c->L < 64 ? c->L : 64;
  if (c->dtype == CARVE_F32 && c->dk == 128) bl = 16;
  return bl;
}

// Without a content projection the gates do not depend on earlier outputs and
// the chunk-parallel schedule (intra + state kernels, block length 64) is used.
bool chunk_parallel(const carve_config* c) { return c->rank == 0 && c->dtype == CARVE_BF16; }
constexpr int kParallelBlock = 64;

int64_t parallel_workspace_bytes(const carve_config* c) {
  const int64_t nblk = (c->T + kParallelBlock - 1) / kParallelBlock;
  const int64_t img = c->dk == 64 ? carve::BlockLayout<carve::bf16, 64, 64, kParallelBlock>::wBytes
                                  : carve::BlockLayout<carve::bf16, 128, 128, kParallelBlock>::wBytes;
  return (int64_t)c->B * c->H * nblk * img;
}

// Without a projection in bf16, when L is a whole number of the forward's
// 64-token blocks, the backward takes its chunk-start states from the forward
// pair's state pass (tens of microseconds) instead of a serial sweep over all
// tokens. The pair's block images and an output it does not need follow the
// backward's own workspace.
bool bwd_from_forward(const carve_config* c) { return chunk_parallel(c) && c->L % kParallelBlock == 0; }

// The chunk-parallel backward (one workgroup per (batch, head, 64-token
// block), dense products on the matrix cores) covers bf16 without a
// projection at d = 64, any L; every other shape walks the tokens.
bool bwd_chunked(const carve_config* c) { return chunk_parallel(c) && c->dk == 64 && c->T > 0; }
// With a projection in bf16 at d = 64 and 64-token chunks the chunks are
// differentiated one after another by one workgroup per head with the same
// dense per-chunk products, after a checkpointing chunk-serial forward.
bool bwd_content_chunked(const carve_config* c) {
  return c->rank > 0 && c->dtype == CARVE_BF16 && c->dk == 64 && c->L == kParallelBlock && c->T > 0 &&
         !(c->flags & CARVE_QK_L2NORM);
}

struct BwdBytes {
  int64_t img, o, total;   // byte offsets of the forward's images and output, and the size
};
BwdBytes bwd_bytes(const carve_config* c) {
  const int64_t B = c->B, H = c->H, T = c->T;
  const int64_t own = B * H * 4 * (int64_t)carve::BwdWs(c->dk, c->T, c->L, c->rank, (c->flags & CARVE_QK_L2NORM) != 0,
                                                       bwd_from_forward(c) && c->T > 0,
                                                       bwd_chunked(c) || bwd_content_chunked(c)).total;
  if (bwd_content_chunked(c)) {                      // the forward's output goes to a scratch buffer
    const int64_t o = (own + 255) & ~(int64_t)255;
    return {o, o, o + B * T * H * c->dv * (int64_t)sizeof(carve::bf16)};
  }
  if (!bwd_from_forward(c) && !bwd_chunked(c)) return {0, 0, own};
  const int64_t img = (own + 255) & ~(int64_t)255;
  const int64_t o = img + parallel_workspace_bytes(c);
  return {img, o, o + B * T * H * c->dv * (int64_t)sizeof(carve::bf16)};
}

// Raises kernel Kern's dynamic-LDS limit to `bytes`. The attribute only ever
// needs raising, so the largest value set so far is kept per kernel (one
// instantiation of this function per kernel) and device, and the driver is
// called only to go beyond it: later calls (and launches inside a graph
// capture) make no attribute call at all.
constexpr int kMaxDevices = 64;
template <auto Kern>
hipError_t set_lds(int bytes) {
  static std::atomic<int> set_bytes[kMaxDevices];
  auto raise = [&] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(Kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  };
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return raise();
  int cur = set_bytes[dev].load(std::memory_order_acquire);
  if (cur >= bytes) return hipSuccess;
  const hipError_t e = raise();
  if (e != hipSuccess) return e;
  while (cur < bytes && !set_bytes[dev].compare_exchange_weak(cur, bytes, std::memory_order_acq_rel)) {
  }
  return hipSuccess;
}

template <typename E, int D, int BL, bool LG, bool NRM>
hipError_t launch_serial(const carve::FwdArgs& a, hipStream_t s) {
  using LY = carve::BlockLayout<E, D, D, BL, carve::serial_waves<D, BL>()>;
  constexpr auto kern = carve::carve_chunk_serial_kernel<E, D, D, BL, LG, NRM>;
  hipError_t e = set_lds<kern>(LY::serial_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(LY::NT), LY::serial_bytes, s, a);
  return hipGetLastError();
}

template <int D, bool LG, bool NRM, bool CKPT = false>
hipError_t launch_parallel(const carve::FwdArgs& a, hipStream_t s) {
  using E = carve::bf16;
  constexpr int BL = kParallelBlock;
  using LY = carve::BlockLayout<E, D, D, BL>;                        // state pass, images
  using LI = carve::BlockLayout<E, D, D, BL, carve::kIntraWaves>;    // intra kernel
  const int nblk = (a.T + BL - 1) / BL;
  constexpr auto intra = carve::carve_intra_kernel<E, D, D, BL, LG, NRM>;
  auto state = carve::carve_state_kernel<E, D, D, BL, CKPT>;
  hipError_t e = set_lds<intra>(LI::intra_bytes);
  if (e != hipSuccess) return e;
  if (nblk > 0) {
    hipLaunchKernelGGL(intra, dim3(a.B * a.H * nblk), dim3(LI::NT), LI::intra_bytes, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(state, dim3(carve::state_grid(a.B * a.H, LY::NW)), dim3(carve::kStateThreads), 0, s, a);
  return hipGetLastError();
}

template <typename E, int D, bool LG, bool NRM>
hipError_t dispatch_block(const carve::FwdArgs& a, int bl, hipStream_t s) {
  switch (bl) {
    case 16: return launch_serial<E, D, 16, LG, NRM>(a, s);
    case 32:
      if constexpr (sizeof(E) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_serial<E, D, 32, LG, NRM>(a, s);
    default:
      if constexpr (sizeof(E) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_serial<E, D, 64, LG, NRM>(a, s);
  }
}

// dtype, width and schedule dispatch of the forward pass for one input mode
// (raw decay logits or not, q and k normalised or not)
template <bool LG, bool NRM>
hipError_t dispatch_fwd(const carve_config* cfg, const carve::FwdArgs& a, hipStream_t s) {
  const int bl = serial_block(cfg);
  if (chunk_parallel(cfg))
    return cfg->dk == 64 ? launch_parallel<64, LG, NRM>(a, s) : launch_parallel<128, LG, NRM>(a, s);
  if (cfg->dtype == CARVE_BF16)
    return cfg->dk == 64 ? dispatch_block<carve::bf16, 64, LG, NRM>(a, bl, s)
                         : dispatch_block<carve::bf16, 128, LG, NRM>(a, bl, s);
  return cfg->dk == 64 ? dispatch_block<float, 64, LG, NRM>(a, bl, s) : dispatch_block<float, 128, LG, NRM>(a, bl, s);
}

hipError_t dispatch_fwd_flags(const carve_config* cfg, const carve::FwdArgs& a, hipStream_t s) {
  const bool lg = (cfg->flags & CARVE_DECAY_LOGITS) != 0, nrm = (cfg->flags & CARVE_QK_L2NORM) != 0;
  return lg ? (nrm ? dispatch_fwd<true, true>(cfg, a, s) : dispatch_fwd<true, false>(cfg, a, s))
            : (nrm ? dispatch_fwd<false, true>(cfg, a, s) : dispatch_fwd<false, false>(cfg, a, s));
}

// the chunk-parallel pair with the checkpointing state pass (the backward's
// chunk-start states; bf16 without a projection only)
template <bool LG, bool NRM>
hipError_t dispatch_fwd_ckpt(const carve_config* cfg, const carve::FwdArgs& a, hipStream_t s) {
  return cfg->dk == 64 ? launch_parallel<64, LG, NRM, true>(a, s) : launch_parallel<128, LG, NRM, true>(a, s);
}

hipError_t dispatch_fwd_ckpt_flags(const carve_config* cfg, const carve::FwdArgs& a, hipStream_t s) {
  const bool lg = (cfg->flags & CARVE_DECAY_LOGITS) != 0, nrm = (cfg->flags & CARVE_QK_L2NORM) != 0;
  return lg ? (nrm ? dispatch_fwd_ckpt<true, true>(cfg, a, s) : dispatch_fwd_ckpt<true, false>(cfg, a, s))
            : (nrm ? dispatch_fwd_ckpt<false, true>(cfg, a, s) : dispatch_fwd_ckpt<false, false>(cfg, a, s));
}

// Row-lane schedule (all widths without a projection; d = 64 with one): the
// sliced kernel, then the sum over its slices that forms dk, dbx, dg, dq, dw.
template <typename E, int D, bool LG, bool CONTENT, bool NRM>
hipError_t launch_row_lane(const carve::BwdArgs& a, hipStream_t s) {
  using SL = carve::SplitLayout<D, CONTENT>;
  constexpr auto split = carve::carve_bwd_split_kernel<E, D, LG, CONTENT, NRM>;
  hipError_t e = set_lds<split>(SL::bytes);
  if (e != hipSuccess) return e;
  // chunk groups (no projection, chunk-start states from the forward pair):
  // the dS sweep first, then every group's workgroups at once
  const int groups = carve::bwd_groups(a.T, a.L, CONTENT ? a.rank : 0, a.pre_ckpt != 0);
  if constexpr (!CONTENT) {
    if (groups > 1 && (int64_t)a.B * a.H > 0) {
      constexpr auto sweep = carve::carve_bwd_split_kernel<E, D, LG, false, NRM, true>;
      e = set_lds<sweep>(SL::bytes);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(sweep, dim3(a.B * a.H * SL::S), dim3(SL::NT), SL::bytes, s, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if ((int64_t)a.B * a.H > 0) {
    hipLaunchKernelGGL(split, dim3(a.B * a.H * SL::S * groups), dim3(SL::NT), SL::bytes, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t n = (size_t)a.B * a.T * a.H * D;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((carve::carve_bwd_finish_kernel<E, D, LG, CONTENT, NRM>), dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

// the projection factors' gradients, summed over the batch (zeros for B = 0)
template <int D>
hipError_t launch_ub_sum(const carve::BwdArgs& a, hipStream_t s) {
  if (a.H == 0) return hipSuccess;
  const carve::BwdWs lay(D, a.T, a.L, a.rank, a.norm != 0, a.pre_ckpt != 0, a.pre_ckpt == 3);
  const size_t n = 2 * (size_t)a.rank * D * a.H;
  hipLaunchKernelGGL(carve::carve_bwd_ub_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     a.ws, lay.total, lay.dud, a.B, a.H, a.rank, a.d_ub_down, a.d_ub_up);
  return hipGetLastError();
}

// q, k normalisation around the backward: inverse norms before it, the
// chain rule through the normalisation after it (one wave per token row)
template <typename E, int D, bool NORMS>
hipError_t launch_norm(const carve::BwdArgs& a, hipStream_t s) {
  const size_t rows = (size_t)a.B * a.T * a.H;
  if (!a.norm || rows == 0) return hipSuccess;
  hipLaunchKernelGGL((carve::carve_bwd_norm_kernel<E, D, NORMS>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

// Chunk-parallel schedule (after the forward pair has written the chunk-start
// states and its block images): the images become the backward chain's, the
// checkpointing state pass walks that chain from the last chunk and stores
// the state gradient at every chunk end, then one workgroup per (batch,
// head, chunk) forms the gradients.
template <bool LG, bool NRM>
hipError_t launch_chunked(const carve::BwdArgs& a, unsigned char* imgs, void* o_scratch, hipStream_t s) {
  using CL = carve::ChunkBwdLayout<64>;
  using LY = carve::BlockLayout<carve::bf16, 64, 64, kParallelBlock>;
  constexpr auto image = carve::carve_bwd_image_kernel<64>;
  constexpr auto chain = carve::carve_state_kernel<carve::bf16, 64, 64, kParallelBlock, true>;
  constexpr auto chunk = carve::carve_bwd_chunk_kernel<64, LG, NRM>;
  hipError_t e = set_lds<chunk>(CL::bytes);
  if (e != hipSuccess) return e;
  const int64_t nc = (a.T + kParallelBlock - 1) / kParallelBlock, BH = (int64_t)a.B * a.H;
  hipLaunchKernelGGL(image, dim3((unsigned)(BH * ((nc + 1) / 2))), dim3(256), 0, s, a, imgs);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const carve::BwdWs lay(64, a.T, kParallelBlock, 0, NRM, true, true);
  carve::FwdArgs f{};
  f.ws = imgs;
  f.state_in = a.d_state_out;
  f.o = o_scratch;
  f.ckpt = a.ws + lay.dsck;
  f.ckpt_bh = lay.total;
  f.ckpt_shift = 0;
  f.B = a.B; f.H = a.H; f.T = a.T; f.L = kParallelBlock; f.rank = 0;
  hipLaunchKernelGGL(chain, dim3(carve::state_grid(a.B * a.H, LY::NW)), dim3(carve::kStateThreads), 0, s, f);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (NRM) {                               // every token's inverse norms of q and k
    e = launch_norm<carve::bf16, 64, true>(a, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(chunk, dim3((unsigned)(BH * nc)), dim3(CL::NT), CL::bytes, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (NRM) return launch_norm<carve::bf16, 64, false>(a, s);   // through the normalisation
  return hipSuccess;
}

template <typename E, int D, bool LG, bool NRM>
hipError_t launch_bwd_core(const carve::BwdArgs& a, hipStream_t s) {
  if (a.rank == 0) return launch_row_lane<E, D, LG, false, NRM>(a, s);
  hipError_t e;
  if constexpr (D == 64) {
    e = launch_row_lane<E, D, LG, true, NRM>(a, s);
  } else {
    // one workgroup per (batch, head), four lanes per row: a row-lane
    // workgroup holding all 128 rows would need 32 waves
    using LY = carve::BwdLayout<D>;
    constexpr auto kern = carve::carve_bwd_kernel<E, D, LG, NRM>;
    e = set_lds<kern>(LY::bytes);
    if (e != hipSuccess) return e;
    if ((int64_t)a.B * a.H > 0) {
      hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(LY::NT), LY::bytes, s, a);
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess) return e;
  return launch_ub_sum<D>(a, s);
}

template <typename E, int D, bool LG>
hipError_t launch_bwd(const carve::BwdArgs& a, hipStream_t s) {
  hipError_t e = launch_norm<E, D, true>(a, s);
  if (e != hipSuccess) return e;
  e = a.norm ? launch_bwd_core<E, D, LG, true>(a, s) : launch_bwd_core<E, D, LG, false>(a, s);
  if (e != hipSuccess) return e;
  return launch_norm<E, D, false>(a, s);
}

template <typename E, bool LG>
hipError_t dispatch_bwd_width(const carve_config* cfg, const carve::BwdArgs& a, hipStream_t s) {
  return cfg->dk == 64 ? launch_bwd<E, 64, LG>(a, s) : launch_bwd<E, 128, LG>(a, s);
}

// Content schedule at d = 64 (after the checkpointing chunk-serial forward):
// the per-head chunk walk, then the factor gradients summed over the batch.
template <bool LG>
hipError_t launch_content_chunked(const carve::BwdArgs& a, hipStream_t s) {
  using CL = carve::ChunkBwdLayout<64>;
  constexpr auto kern = carve::carve_bwd_chunk_serial_kernel<64, LG>;
  hipError_t e = set_lds<kern>(CL::bytes);
  if (e != hipSuccess) return e;
  if ((int64_t)a.B * a.H > 0) {
    hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(CL::NT), CL::bytes, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_ub_sum<64>(a, s);
}

// the checkpointing chunk-serial forward of the content schedule
template <bool LG>
hipError_t launch_serial_ckpt(const carve::FwdArgs& a, hipStream_t s) {
  using E = carve::bf16;
  using LY = carve::BlockLayout<E, 64, 64, kParallelBlock, carve::serial_waves<64, kParallelBlock>()>;
  constexpr auto kern = carve::carve_chunk_serial_kernel<E, 64, 64, kParallelBlock, LG, false, true>;
  hipError_t e = set_lds<kern>(LY::serial_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(LY::NT), LY::serial_bytes, s, a);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_step(const carve::StepArgs& a, hipStream_t s) {
  constexpr auto kern = carve::carve_step_kernel<E, D>;
  const int lds = 2 * a.rank * D * (int)sizeof(E);   // the head's U_down and U_up
  hipError_t e = set_lds<kern>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(4 * D), lds, s, a);
  return hipGetLastError();
}

}  // namespace

extern "C" int carve_recurrent_ref_shapes(const carve_config* cfg, carve_shapes* out) {
  const int st = check_config(cfg);
  if (st != CARVE_OK) return st;
  if (!out) return CARVE_EINVAL;
  const int64_t B = cfg->B, H = cfg->H, T = cfg->T, dk = cfg->dk, dv = cfg->dv, r = cfg->rank;
  out->q = out->k = out->g = out->bx = B * T * H * dk;
  out->v = out->o = B * T * H * dv;
  out->w = B * T * H;
  out->ub_down = H * r * dv;
  out->ub_up = H * dk * r;
  out->state = B * H * dv * dk;
  out->mean = B * H * dv;
  out->workspace_bytes = chunk_parallel(cfg) ? parallel_workspace_bytes(cfg) : 0;
  out->bwd_workspace_bytes = bwd_bytes(cfg).total;
  return CARVE_OK;
}

namespace {

// Argument checks of the forward entry points (no HIP call): fills `sh` and
// returns CARVE_OK when the call may go ahead.
int fwd_check(const carve_config* cfg, const void* q, const void* k, const void* v, const void* g, const void* bx,
              const void* w, const void* ub_down, const void* ub_up, const float* state_in, const float* mean_in,
              const void* o, const float* state_out, const float* mean_out, const void* workspace,
              size_t workspace_bytes, carve_shapes* sh) {
  int st = carve_recurrent_ref_shapes(cfg, sh);
  if (st != CARVE_OK) return st;
  const bool tokens = sh->q > 0;
  if (tokens && (!q || !k || !v || !g || !bx || !w || !o)) return CARVE_EINVAL;
  const bool content = cfg->rank > 0;
  if (content && (int64_t)cfg->B * cfg->H > 0 && (!ub_down || !ub_up)) return CARVE_EINVAL;
  const void* ptrs[] = {q, k, v, g, bx, w, content ? ub_down : nullptr, content ? ub_up : nullptr,
                        state_in, mean_in, o, state_out, mean_out, workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return CARVE_EALIGN;
  if (workspace_bytes < (size_t)sh->workspace_bytes) return CARVE_EWORKSPACE;
  const size_t es = elem_bytes(cfg->dtype);
  const size_t ob = (size_t)sh->o * es;
  const struct { const void* p; size_t n; } ins[] = {
      {q, (size_t)sh->q * es}, {k, (size_t)sh->k * es}, {v, (size_t)sh->v * es},
      {g, (size_t)sh->g * es}, {bx, (size_t)sh->bx * es}, {w, (size_t)sh->w * es},
      {state_in, (size_t)sh->state * 4}, {mean_in, (size_t)sh->mean * 4}};
  for (const auto& in : ins)
    if (overlaps(o, ob, in.p, in.n)) return CARVE_EINVAL;
  return CARVE_OK;
}

// Whether a checked forward call has any work to queue.
bool fwd_has_work(const carve_config* cfg, const carve_shapes& sh, const float* state_out, const float* mean_out) {
  if ((int64_t)cfg->B * cfg->H == 0) return false;
  return sh.q > 0 || state_out || mean_out;
}

int fwd_launch(const carve_config* cfg, const void* q, const void* k, const void* v, const void* g, const void* bx,
               const void* w, const void* ub_down, const void* ub_up, const float* state_in, const float* mean_in,
               void* o, float* state_out, float* mean_out, void* workspace, void* stream) {
  carve::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.bx = bx; a.w = w;
  a.ub_down = ub_down; a.ub_up = ub_up;
  a.state_in = state_in; a.mean_in = mean_in;
  a.o = o; a.state_out = state_out; a.mean_out = mean_out;
  a.ws = workspace;
  a.B = cfg->B; a.H = cfg->H; a.T = cfg->T; a.L = cfg->L; a.rank = cfg->rank;
  a.ckpt = nullptr; a.ckpt_bh = 0; a.ckpt_shift = 0;

  const hipError_t e = dispatch_fwd_flags(cfg, a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    std::snprintf(g_hip_msg, sizeof(g_hip_msg), "%s", hipGetErrorString(e));
    return CARVE_EHIP;
  }
  return CARVE_OK;
}

// Scratch of carve_chunk_fwd_noalloc: the two-launch schedule's block images
// (the only workspace any forward schedule uses), in a fixed device array
// that every GPU the library runs on holds until the process ends. In host
// code `scratch` names a host-side stand-in, never device memory: its device
// address on the current device comes from hipGetSymbolAddress, looked up
// once per device and kept in noalloc_scratch.
constexpr size_t kNoAllocScratch = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];
std::atomic<void*> noalloc_scratch[kMaxDevices];

hipError_t noalloc_scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = noalloc_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current: its copy of the array
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    noalloc_scratch[dev].store(p, std::memory_order_release);   // racing first calls store the same address
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" int carve_chunk_fwd(const carve_config* cfg,
                               const void* q, const void* k, const void* v,
                               const void* g, const void* bx, const void* w,
                               const void* ub_down, const void* ub_up,
                               const float* state_in, const float* mean_in,
                               void* o, float* state_out, float* mean_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  carve_shapes sh;
  const int st = fwd_check(cfg, q, k, v, g, bx, w, ub_down, ub_up, state_in, mean_in, o, state_out, mean_out,
                           workspace, workspace_bytes, &sh);
  if (st != CARVE_OK) return st;
  if (!fwd_has_work(cfg, sh, state_out, mean_out)) return CARVE_OK;
  return fwd_launch(cfg, q, k, v, g, bx, w, ub_down, ub_up, state_in, mean_in, o, state_out, mean_out, workspace,
                    stream);
}

extern "C" int carve_chunk_fwd_noalloc(const carve_config* cfg,
                                       const void* q, const void* k, const void* v,
                                       const void* g, const void* bx, const void* w,
                                       const void* ub_down, const void* ub_up,
                                       const float* state_in, const float* mean_in,
                                       void* o, float* state_out, float* mean_out, void* stream) {
  carve_shapes sh;
  // the fixed scratch stands in for the workspace: a problem that needs more
  // is CARVE_EWORKSPACE
  const int st = fwd_check(cfg, q, k, v, g, bx, w, ub_down, ub_up, state_in, mean_in, o, state_out, mean_out,
                           nullptr, kNoAllocScratch, &sh);
  if (st != CARVE_OK) return st;
  if (!fwd_has_work(cfg, sh, state_out, mean_out)) return CARVE_OK;
  void* ws = nullptr;
  if (sh.workspace_bytes > 0) {
    const hipError_t e = noalloc_scratch_ptr(&ws);
    if (e != hipSuccess) {
      std::snprintf(g_hip_msg, sizeof(g_hip_msg), "%s", hipGetErrorString(e));
      return CARVE_EHIP;
    }
  }
  return fwd_launch(cfg, q, k, v, g, bx, w, ub_down, ub_up, state_in, mean_in, o, state_out, mean_out, ws, stream);
}

extern "C" int carve_chunk_bwd(const carve_config* cfg,
                               const void* q, const void* k, const void* v,
                               const void* g, const void* bx, const void* w,
                               const void* ub_down, const void* ub_up,
                               const float* state_in, const float* mean_in,
                               const void* d_o, const float* d_state_out, const float* d_mean_out,
                               void* dq, void* dk, void* dv, void* dg, void* dbx, void* dw,
                               float* d_ub_down, float* d_ub_up, float* d_state_in, float* d_mean_in,
                               void* workspace, size_t workspace_bytes, void* stream) {
  carve_shapes sh;
  int st = carve_recurrent_ref_shapes(cfg, &sh);
  if (st != CARVE_OK) return st;
  const bool tokens = sh.q > 0;
  if (tokens && (!q || !k || !v || !g || !bx || !w || !d_o || !dq || !dk || !dv || !dg || !dbx || !dw))
    return CARVE_EINVAL;
  const bool content = cfg->rank > 0;
  if (content && cfg->H > 0 && (!d_ub_down || !d_ub_up)) return CARVE_EINVAL;
  if (content && (int64_t)cfg->B * cfg->H > 0 && (!ub_down || !ub_up)) return CARVE_EINVAL;
  const void* ptrs[] = {q, k, v, g, bx, w, content ? ub_down : nullptr, content ? ub_up : nullptr,
                        state_in, mean_in, d_o, d_state_out, d_mean_out, dq, dk, dv, dg, dbx, dw,
                        content ? d_ub_down : nullptr, content ? d_ub_up : nullptr, d_state_in, d_mean_in,
                        workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return CARVE_EALIGN;
  // one-dimensional grids of the slice-sum (one thread per gradient element)
  // and batch-sum kernels, 256 threads per block
  if ((int64_t)cfg->B * cfg->T * cfg->H * cfg->dk / 256 >= 0x7fffffffLL ||
      2 * (int64_t)cfg->rank * cfg->dk * cfg->H / 256 >= 0x7fffffffLL ||
      (int64_t)cfg->B * cfg->H * (cfg->dk / 16) * carve::kBwdGroups >= 0x7fffffffLL)   // row slices x chunk groups
    return CARVE_EUNSUPPORTED;
  if (workspace_bytes < (size_t)sh.bwd_workspace_bytes) return CARVE_EWORKSPACE;
  if (sh.bwd_workspace_bytes > 0 && (int64_t)cfg->B * cfg->H > 0 && !workspace) return CARVE_EINVAL;
  const size_t es = elem_bytes(cfg->dtype);
  struct Span { const void* p; size_t n; };
  const Span ins[] = {
      {q, (size_t)sh.q * es}, {k, (size_t)sh.k * es}, {v, (size_t)sh.v * es},
      {g, (size_t)sh.g * es}, {bx, (size_t)sh.bx * es}, {w, (size_t)sh.w * es},
      {content ? ub_down : nullptr, (size_t)sh.ub_down * es}, {content ? ub_up : nullptr, (size_t)sh.ub_up * es},
      {state_in, (size_t)sh.state * 4}, {mean_in, (size_t)sh.mean * 4}, {d_o, (size_t)sh.o * es}};
  // d_state_out and d_mean_out may be the very buffers that receive
  // d_state_in and d_mean_in (each element is read before it is written, by
  // the same thread); any other overlap is an error
  const Span grads_out[] = {{d_state_out, (size_t)sh.state * 4}, {d_mean_out, (size_t)sh.mean * 4}};
  const Span outs[] = {
      {dq, (size_t)sh.q * es}, {dk, (size_t)sh.k * es}, {dv, (size_t)sh.v * es}, {dg, (size_t)sh.g * es},
      {dbx, (size_t)sh.bx * es}, {dw, (size_t)sh.w * es},
      {content ? d_ub_down : nullptr, (size_t)sh.ub_down * 4}, {content ? d_ub_up : nullptr, (size_t)sh.ub_up * 4},
      {d_state_in, (size_t)sh.state * 4}, {d_mean_in, (size_t)sh.mean * 4},
      {workspace, (size_t)sh.bwd_workspace_bytes}};
  constexpr size_t NO = sizeof(outs) / sizeof(outs[0]);
  for (size_t i = 0; i < NO; ++i) {
    for (const auto& in : ins)
      if (overlaps(outs[i].p, outs[i].n, in.p, in.n)) return CARVE_EINVAL;
    for (size_t j = 0; j < 2; ++j) {
      const bool allowed = (i == 8 && j == 0 && outs[i].p == grads_out[j].p) ||
                           (i == 9 && j == 1 && outs[i].p == grads_out[j].p);
      if (!allowed && overlaps(outs[i].p, outs[i].n, grads_out[j].p, grads_out[j].n)) return CARVE_EINVAL;
    }
    for (size_t j = i + 1; j < NO; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return CARVE_EINVAL;
  }
  if ((int64_t)cfg->B * cfg->H == 0 && !(content && cfg->H > 0)) return CARVE_OK;

  carve::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.bx = bx; a.w = w;
  a.ub_down = ub_down; a.ub_up = ub_up;
  a.state_in = state_in; a.mean_in = mean_in;
  a.d_o = d_o; a.d_state_out = d_state_out; a.d_mean_out = d_mean_out;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbx = dbx; a.dw = dw;
  a.d_state_in = d_state_in; a.d_mean_in = d_mean_in;
  a.d_ub_down = d_ub_down; a.d_ub_up = d_ub_up;
  a.ws = static_cast<float*>(workspace);
  a.B = cfg->B; a.H = cfg->H; a.T = cfg->T; a.L = cfg->L; a.rank = cfg->rank;
  a.norm = (cfg->flags & CARVE_QK_L2NORM) != 0;
  a.detach = (cfg->flags & CARVE_DETACH_MEAN) != 0;
  a.pre_ckpt = bwd_content_chunked(cfg) ? 3 : bwd_chunked(cfg) ? 2 : bwd_from_forward(cfg) && cfg->T > 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool lg = (cfg->flags & CARVE_DECAY_LOGITS) != 0;
  hipError_t e = hipSuccess;
  if (a.pre_ckpt == 3 && (int64_t)cfg->B * cfg->H > 0) {
    // the chunk-serial forward stores the state, gate bias and gate mean at
    // every chunk start; its output goes to a scratch buffer
    const BwdBytes bb = bwd_bytes(cfg);
    const carve::BwdWs lay(64, cfg->T, cfg->L, cfg->rank, false, true, true);
    carve::FwdArgs f{};
    f.q = q; f.k = k; f.v = v; f.g = g; f.bx = bx; f.w = w;
    f.ub_down = ub_down; f.ub_up = ub_up;
    f.state_in = state_in; f.mean_in = mean_in;
    f.o = static_cast<unsigned char*>(workspace) + bb.o;
    f.B = cfg->B; f.H = cfg->H; f.T = cfg->T; f.L = cfg->L; f.rank = cfg->rank;
    f.ckpt = static_cast<float*>(workspace);
    f.ckpt_bh = lay.total;
    f.ckpt_z = lay.z;
    f.ckpt_m = lay.m;
    e = lg ? launch_serial_ckpt<true>(f, s) : launch_serial_ckpt<false>(f, s);
    if (e == hipSuccess) e = lg ? launch_content_chunked<true>(a, s) : launch_content_chunked<false>(a, s);
  } else if (a.pre_ckpt == 3) {
    e = launch_ub_sum<64>(a, s);                      // no (batch, head): zero factor gradients
  } else if (a.pre_ckpt) {
    // the forward pair writes the state at every chunk start into the
    // backward's checkpoints (chunk c starts at block c L / 64)
    const BwdBytes bb = bwd_bytes(cfg);
    unsigned char* wsb = static_cast<unsigned char*>(workspace);
    carve::FwdArgs f;
    f.q = q; f.k = k; f.v = v; f.g = g; f.bx = bx; f.w = w;
    f.ub_down = nullptr; f.ub_up = nullptr;
    f.state_in = state_in; f.mean_in = mean_in;
    f.o = wsb + bb.o; f.state_out = nullptr; f.mean_out = nullptr;
    f.ws = wsb + bb.img;
    f.B = cfg->B; f.H = cfg->H; f.T = cfg->T; f.L = cfg->L; f.rank = 0;
    f.ckpt = static_cast<float*>(workspace);
    f.ckpt_bh = carve::BwdWs(cfg->dk, cfg->T, cfg->L, 0, a.norm != 0, true, a.pre_ckpt == 2).total;
    f.ckpt_shift = a.pre_ckpt != 2 && cfg->L == 2 * kParallelBlock ? 1 : 0;
    e = dispatch_fwd_ckpt_flags(cfg, f, s);
  }
  if (e == hipSuccess && a.pre_ckpt == 2) {
    const BwdBytes bb = bwd_bytes(cfg);
    unsigned char* wsb = static_cast<unsigned char*>(workspace);
    unsigned char* img = wsb + bb.img;
    void* o = wsb + bb.o;
    e = a.norm ? (lg ? launch_chunked<true, true>(a, img, o, s) : launch_chunked<false, true>(a, img, o, s))
               : (lg ? launch_chunked<true, false>(a, img, o, s) : launch_chunked<false, false>(a, img, o, s));
  }
  else if (e == hipSuccess && a.pre_ckpt != 3)
    e = cfg->dtype == CARVE_BF16
            ? (lg ? dispatch_bwd_width<carve::bf16, true>(cfg, a, s) : dispatch_bwd_width<carve::bf16, false>(cfg, a, s))
            : (lg ? dispatch_bwd_width<float, true>(cfg, a, s) : dispatch_bwd_width<float, false>(cfg, a, s));
  if (e != hipSuccess) {
    std::snprintf(g_hip_msg, sizeof(g_hip_msg), "%s", hipGetErrorString(e));
    return CARVE_EHIP;
  }
  return CARVE_OK;
}

extern "C" int carve_recurrent_step(const carve_config* cfg, int32_t pos,
                                    const void* q, const void* k, const void* v,
                                    const void* g, const void* bx, const void* w,
                                    const void* ub_down, const void* ub_up,
                                    float* state, float* mean_prev, float* chunk_acc,
                                    void* o, void* stream) {
  carve_shapes sh;
  int st = carve_recurrent_ref_shapes(cfg, &sh);
  if (st != CARVE_OK) return st;
  if (cfg->T != 1 || pos < 0 || pos >= cfg->L) return CARVE_EINVAL;
  const bool heads = (int64_t)cfg->B * cfg->H > 0;
  if (heads && (!q || !k || !v || !g || !bx || !w || !o || !state || !mean_prev || !chunk_acc))
    return CARVE_EINVAL;
  const bool content = cfg->rank > 0;
  if (content && heads && (!ub_down || !ub_up)) return CARVE_EINVAL;
  const void* ptrs[] = {q, k, v, g, bx, w, content ? ub_down : nullptr, content ? ub_up : nullptr,
                        state, mean_prev, chunk_acc, o};
  for (const void* p : ptrs)
    if (misaligned(p)) return CARVE_EALIGN;
  const size_t es = elem_bytes(cfg->dtype);
  const struct { const void* p; size_t n; } ins[] = {
      {q, (size_t)sh.q * es}, {k, (size_t)sh.k * es}, {v, (size_t)sh.v * es},
      {g, (size_t)sh.g * es}, {bx, (size_t)sh.bx * es}, {w, (size_t)sh.w * es},
      {content ? ub_down : nullptr, (size_t)sh.ub_down * es}, {content ? ub_up : nullptr, (size_t)sh.ub_up * es}};
  const struct { const void* p; size_t n; } outs[] = {
      {o, (size_t)sh.o * es}, {state, (size_t)sh.state * 4}, {mean_prev, (size_t)sh.mean * 4},
      {chunk_acc, (size_t)sh.mean * 4}};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const auto& in : ins)
      if (overlaps(outs[i].p, outs[i].n, in.p, in.n)) return CARVE_EINVAL;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return CARVE_EINVAL;
  }
  if (!heads) return CARVE_OK;

  carve::StepArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.bx = bx; a.w = w;
  a.ub_down = ub_down; a.ub_up = ub_up;
  a.state = state; a.mean_prev = mean_prev; a.chunk_acc = chunk_acc; a.o = o;
  a.B = cfg->B; a.H = cfg->H; a.L = cfg->L; a.rank = cfg->rank; a.pos = pos;
  a.logits = (cfg->flags & CARVE_DECAY_LOGITS) != 0;
  a.norm = (cfg->flags & CARVE_QK_L2NORM) != 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (cfg->dtype == CARVE_BF16)
    e = cfg->dk == 64 ? launch_step<carve::bf16, 64>(a, s) : launch_step<carve::bf16, 128>(a, s);
  else
    e = cfg->dk == 64 ? launch_step<float, 64>(a, s) : launch_step<float, 128>(a, s);
  if (e != hipSuccess) {
    std::snprintf(g_hip_msg, sizeof(g_hip_msg), "%s", hipGetErrorString(e));
    return CARVE_EHIP;
  }
  return CARVE_OK;
}

extern "C" const char* carve_error_string(int code) {
  switch (code) {
    case CARVE_OK: return "ok";
    case CARVE_EINVAL: return "invalid argument (NULL required pointer, negative size, unknown flag or overlapping output)";
    case CARVE_EUNSUPPORTED: return "unsupported configuration (dk/dv in {64,128} with dk == dv, L in {16,32,64,128}, rank <= 64, sizes within 32-bit indexing)";
    case CARVE_EALIGN: return "a tensor pointer is not 16-byte aligned";
    case CARVE_EWORKSPACE: return "workspace smaller than carve_recurrent_ref_shapes() requires (for carve_chunk_fwd_noalloc: the problem needs more workspace than its fixed 64 MiB scratch)";
    case CARVE_EHIP: return g_hip_msg;
    default: return "unknown status code";
  }
}
