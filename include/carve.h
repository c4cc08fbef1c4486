/*
 * carve.h: C ABI of the CARVE chunk-parallel forward pass on MI355X (gfx950).
 *
 * The operation is the forward pass of the CARVE recurrent layer (arXiv
 * 2606.27229, "CARVE: Content-Aware Recurrent with Value Efficiency for
 * Chunk-Parallel Linear Attention"), as described in the gist.science
 * technical summaries:
 *   section 1 (problem statement)   per head a state S of shape d_v x d_k;
 *   section 2 (method)              every gate acts on the key axis only;
 *   section 2.1 (output reuse)      o_t = S_{t-1} q_t, chunk mean
 *                                   m_c = (1/L) sum o_t, erase gate
 *                                   b = sigmoid(b_x + U_b m), one chunk stale;
 *   section 2.2 (scalar write)      one write gate w per head and token,
 *                                   broadcast over the value channels;
 *   section 2.3 (key-axis decay)    exponential decay exp(g) on the key axis;
 *                                   the activation that turns the decay
 *                                   logits into g may run inside the kernel
 *                                   ("gate-in-kernel", CARVE_DECAY_LOGITS).
 * Per token (readings: b scales the retrieval key; decay precedes erase):
 *   o_t = S q_t;  S <- S diag(exp(g_t)) (I - (b_t * k_t) k_t^T) + w_t v_t k_t^T
 * with b_t = sigmoid(bx_t + U_up (U_down m_{c-1})) for every token of chunk c,
 * m_{-1} = mean_in (zero when absent), and m_c the mean of chunk c's outputs
 * over the tokens it holds (a last chunk may be partial).
 * The library computes this with the WY-form chunk solver (Theorem 11 in
 * section 3 of the same summaries: key-axis-only erase leaves one triangular
 * system per chunk).
 *
 * Conventions for every entry point:
 *   - No HIP types cross this header; `stream` is a hipStream_t passed as
 *     void* (NULL = the null stream).
 *   - All tensor pointers are device pointers owned by the caller. The library
 *     never allocates, frees or synchronises; work is queued on `stream` and
 *     the call returns before it finishes.
 *   - Tensors are dense, row-major, 16-byte aligned, no strides.
 *   - Every argument check runs before the first HIP call, so invalid
 *     arguments are reported (and testable) without a GPU.
 *   - The library keeps no state beyond a per-device record of the kernels'
 *     LDS limits it has raised; concurrent calls need distinct outputs.
 *   - Errors are returned as a carve_status code; nothing is thrown.
 */
#ifndef CARVE_H
#define CARVE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CARVE_OK = 0,
  CARVE_EINVAL = 1,        /* NULL required pointer, negative size, unknown flag bit */
  CARVE_EUNSUPPORTED = 2,  /* d_k/d_v not in {64,128}, L not in {16,32,64,128}, d_k != d_v,
                              rank > 64, or a size past the kernels' 32-bit index range */
  CARVE_EALIGN = 3,        /* a pointer is not 16-byte aligned */
  CARVE_EWORKSPACE = 4,    /* workspace smaller than carve_recurrent_ref_shapes() asks */
  CARVE_EHIP = 5           /* a HIP launch failed; carve_error_string(CARVE_EHIP) has the text */
} carve_status;

typedef enum { CARVE_F32 = 0, CARVE_BF16 = 1 } carve_dtype;

/* Bits of carve_config.flags.
 *   CARVE_DECAY_LOGITS  the g tensor holds raw decay logits a instead of the
 *                       log-decay, and the kernels form g = -softplus(a)
 *                       = -log(1 + e^a) themselves (the decay activation of
 *                       section 2.3 applied in-kernel), so the caller never
 *                       materialises the activated tensor. Any real a is
 *                       valid; exp(g) = sigmoid(-a) lies in (0, 1).
 *   CARVE_QK_L2NORM     q and k are raw: the kernels divide each token's q
 *                       and k by their L2 norms over dk (x / max(|x|, 1e-12))
 *                       before using them, so the caller need not normalise
 *                       them in a separate pass.
 *   CARVE_DETACH_MEAN   backward only (the forward and the step ignore it):
 *                       the chunk means that feed the content gate are taken
 *                       as constants, as when a training loop detaches them.
 *                       U_down and U_up still get their gradients through the
 *                       gate; no gradient reaches earlier outputs or mean_in
 *                       through it (d_mean_out still reaches the last chunk's
 *                       outputs). Without the bit the gradients are the exact
 *                       ones, through every stale mean. */
enum { CARVE_DECAY_LOGITS = 1, CARVE_QK_L2NORM = 2, CARVE_DETACH_MEAN = 4 };

/* Problem description. B batch, H heads, T tokens, dk key width, dv value
 * width, L chunk length of the content signal, rank of U_b (0 = no content
 * projection), dtype of every activation tensor and of U_down/U_up, flags a
 * bitwise OR of the bits above (0 for none; an unknown bit is CARVE_EINVAL). */
typedef struct {
  int32_t B, H, T, dk, dv, L, rank;
  int32_t dtype; /* carve_dtype */
  int32_t flags; /* a bitwise OR of the CARVE_* bits above, or 0 */
} carve_config;

/* Element counts of every tensor (not bytes), and the workspace size in bytes. */
typedef struct {
  int64_t q, k, v, g, bx, w;   /* inputs */
  int64_t ub_down, ub_up;      /* content projection factors (0 when rank == 0) */
  int64_t o;                   /* output */
  int64_t state, mean;         /* optional fp32 state_in/out and mean_in/out */
  int64_t workspace_bytes;     /* device scratch carve_chunk_fwd needs */
  int64_t bwd_workspace_bytes; /* device scratch carve_chunk_bwd needs */
} carve_shapes;

/* Validates `cfg` and fills `out` with the shape contract of the recurrence:
 *   q, k, g, bx : [B, T, H, dk]      v, o : [B, T, H, dv]      w : [B, T, H]
 *   ub_down     : [H, rank, dv]      ub_up : [H, dk, rank]
 *   state       : [B, H, dv, dk] fp32   mean : [B, H, dv] fp32
 * Returns CARVE_OK, CARVE_EINVAL or CARVE_EUNSUPPORTED. Makes no HIP call. */
int carve_recurrent_ref_shapes(const carve_config* cfg, carve_shapes* out);

/* Forward pass of the CARVE layer (see the header comment for the math).
 *   q, k       [B,T,H,dk] dtype   query and key (used as given: no scaling)
 *   v          [B,T,H,dv] dtype   value
 *   g          [B,T,H,dk] dtype   log-decay, expected <= 0; with
 *                                 CARVE_DECAY_LOGITS the raw decay logits
 *   bx         [B,T,H,dk] dtype   erase logit
 *   w          [B,T,H]    dtype   scalar write gate
 *   ub_down    [H,rank,dv] dtype, ub_up [H,dk,rank] dtype: U_b = ub_up @ ub_down
 *              per head. Ignored when rank == 0; required when rank > 0.
 *   state_in   [B,H,dv,dk] fp32 or NULL (zeros)
 *   mean_in    [B,H,dv] fp32 or NULL (zeros): the mean that gates chunk 0
 *   o          [B,T,H,dv] dtype   output; must not overlap any input
 *   state_out  [B,H,dv,dk] fp32 or NULL (not written); may equal state_in
 *   mean_out   [B,H,dv] fp32 or NULL (not written); may equal mean_in. It
 *              receives the mean of the last (possibly partial) chunk, or
 *              mean_in when T == 0.
 *   workspace  device scratch of at least shapes.workspace_bytes (may be NULL
 *              when that is 0)
 *   stream     hipStream_t as void*
 * B, H or T may be 0 (nothing to compute; with T == 0 the state and mean pass
 * through). T need not be a multiple of L.
 * The chunk-parallel state pass hands block states between the waves of a
 * workgroup through LDS with bounded waits. A wait that runs out (none has
 * ever been observed; it would take a hardware fault) writes NaN to the
 * affected output tiles, state and mean instead of hanging; the call still
 * returns CARVE_OK, since the kernels run after it returns. */
int carve_chunk_fwd(const carve_config* cfg,
                    const void* q, const void* k, const void* v,
                    const void* g, const void* bx, const void* w,
                    const void* ub_down, const void* ub_up,
                    const float* state_in, const float* mean_in,
                    void* o, float* state_out, float* mean_out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* carve_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code recorded under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. Arguments and results are
 * those of carve_chunk_fwd (bit for bit: the same kernels run). The library
 * allocates nothing for the call: where a schedule needs workspace (bf16 with
 * no content projection: the two-launch pair's block images), it uses a fixed
 * 64 MiB device array that every GPU the library runs on holds until the
 * process ends. A problem that needs more (shapes.workspace_bytes > 64 MiB,
 * e.g. more than 2048 (batch, head, 64-token block) triples at dk = dv = 64)
 * is CARVE_EWORKSPACE, before any HIP call. All calls on one GPU share that
 * array, so calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. */
int carve_chunk_fwd_noalloc(const carve_config* cfg,
                            const void* q, const void* k, const void* v,
                            const void* g, const void* bx, const void* w,
                            const void* ub_down, const void* ub_up,
                            const float* state_in, const float* mean_in,
                            void* o, float* state_out, float* mean_out, void* stream);

/* Backward pass: gradients of a scalar loss with respect to every input of
 * carve_chunk_fwd, from its gradients with respect to the outputs. The pages
 * train the layer but give no backward pass; these are the exact derivatives
 * of the recurrence in the header comment through every path it has: the
 * stale chunk mean m_{c-1} that gates chunk c passes gradient back to chunk
 * c-1's outputs (and to mean_in for chunk 0), and U_down, U_up receive
 * theirs through the erase gate.
 *   cfg, q .. mean_in   exactly as given to carve_chunk_fwd (the forward pass
 *                       is recomputed; nothing from it is kept)
 *   d_o         [B,T,H,dv] dtype   gradient of o (required when B T H > 0)
 *   d_state_out [B,H,dv,dk] fp32 or NULL (zeros)
 *   d_mean_out  [B,H,dv] fp32 or NULL (zeros)
 *   dq, dk, dg, dbx [B,T,H,dk], dv [B,T,H,dv], dw [B,T,H]: dtype, written.
 *               With CARVE_DECAY_LOGITS, dg is the gradient of the raw logit.
 *   d_ub_down [H,rank,dv], d_ub_up [H,dk,rank]: fp32, written (summed over
 *               the batch); required when rank > 0 and H > 0
 *   d_state_in [B,H,dv,dk], d_mean_in [B,H,dv]: fp32 or NULL (not written).
 *               They may be the same buffers as d_state_out and d_mean_out.
 *   workspace   at least shapes.bwd_workspace_bytes of device scratch: the
 *               state at every chunk start and one chunk's recomputed states,
 *               4 (nc + L) dk dv bytes per (batch, head) at dk = 128 with a
 *               projection, 4 (nc + ceil(L / 8)) dk dv otherwise, plus small
 *               vectors;
 *               with rank == 0 also every token's per-slice column sums,
 *               4 T (dk / 16) (4 dk + 1) bytes per (batch, head); in bf16
 *               with rank == 0 and L a multiple of 64, also the forward
 *               pair's block images and an output, since the chunk-start
 *               states then come from the forward's chunk-parallel state pass;
 *               the chunks are then walked in up to 16 groups at once, which
 *               takes one chunk's recomputed states per group and the state
 *               gradient at every chunk end, 4 (G ceil(L / 8) + nc) dk dv
 *               bytes per (batch, head) in place of 4 ceil(L / 8) dk dv (the
 *               row-lane schedules keep the state at every 8-token sub-block
 *               start rather than at every token; 4 L dk dv at dk = 128 with
 *               a projection). In bf16 with rank == 0, dk = 64 and without
 *               CARVE_QK_L2NORM (any L), every 64-token block is
 *               differentiated at once from its start state and its
 *               end-of-block state gradient (dense products per block); the
 *               workspace then holds only those two per block and a row share
 *               of d_mean_out, 4 (2 nb dk dv + dv) bytes per (batch, head)
 *               with nb = ceil(T / 64), besides the forward pair's images and
 *               output
 * No output may overlap an input, another output or the workspace, except
 * for the two aliases above. Results are deterministic (no atomics).
 * Returns the status codes of carve_chunk_fwd. */
int carve_chunk_bwd(const carve_config* cfg,
                    const void* q, const void* k, const void* v,
                    const void* g, const void* bx, const void* w,
                    const void* ub_down, const void* ub_up,
                    const float* state_in, const float* mean_in,
                    const void* d_o, const float* d_state_out, const float* d_mean_out,
                    void* dq, void* dk, void* dv, void* dg, void* dbx, void* dw,
                    float* d_ub_down, float* d_ub_up, float* d_state_in, float* d_mean_in,
                    void* workspace, size_t workspace_bytes, void* stream);

/* One decode step: the token recurrence of the header comment for a single
 * token of every (batch, head), for serving loops that produce one token at a
 * time. The caller carries three fp32 tensors from step to step:
 *   state      [B,H,dv,dk]  S before this token; updated in place
 *   mean_prev  [B,H,dv]     the mean of the previous chunk's outputs, which
 *                           gates this token (section 2.1: one chunk stale);
 *                           replaced by this chunk's mean at its last position
 *   chunk_acc  [B,H,dv]     sum of this chunk's outputs before this token; the
 *                           token's output is added, and it restarts from zero
 *                           after the chunk's last position
 * and `pos`, the token's position within its chunk (0 <= pos < L). Stepping
 * tokens t = 0, 1, ... with pos = t mod L from (state_in, mean_in, zeros)
 * gives carve_chunk_fwd's outputs and final state; after a whole chunk,
 * mean_prev holds its mean (for a partial last chunk, carve_chunk_fwd's
 * mean_out is chunk_acc divided by the tokens it holds).
 *   cfg        B, H, dk, dv, L, rank, dtype as for carve_chunk_fwd; T must be 1
 *   q, k, g, bx [B,H,dk] dtype; v [B,H,dv] dtype; w [B,H] dtype: this token
 *              ([B,1,H,.] in the layout of carve_chunk_fwd)
 *   ub_down, ub_up as for carve_chunk_fwd
 *   o          [B,H,dv] dtype: this token's output
 * state, mean_prev and chunk_acc are required (when B H > 0); none of o,
 * state, mean_prev and chunk_acc may overlap each other or an input. Returns
 * CARVE_EINVAL for T != 1, pos outside [0, L), a missing pointer or an
 * overlap, and the status codes of carve_chunk_fwd otherwise. Needs no
 * workspace. */
int carve_recurrent_step(const carve_config* cfg, int32_t pos,
                         const void* q, const void* k, const void* v,
                         const void* g, const void* bx, const void* w,
                         const void* ub_down, const void* ub_up,
                         float* state, float* mean_prev, float* chunk_acc,
                         void* o, void* stream);

/* Static text for a status code. For CARVE_EHIP it returns the HIP error text
 * of the most recent failure on the calling thread. */
const char* carve_error_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* CARVE_H */
