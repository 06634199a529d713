/*
 * hc.h -- C ABI of libhc, the Hyper-Connections (HC) residual glue for
 * AMD Instinct MI355X (gfx950).
 *
 * In a Hyper-Connections block the residual is hc parallel copies ("streams")
 * of width d.  Around every sublayer the glue
 *   - derives (2+hc)*hc mix numbers per token from the streams (hc_mixes;
 *     24 at hc = 4),
 *   - turns them into reading weights pre, writing weights post and a
 *     Sinkhorn-normalised hc x hc combination comb (hc_split_sinkhorn),
 *   - reads the streams into one sublayer input (hc_pre),
 *   - writes the sublayer output back into the streams (hc_post).
 * Sources: the model-atlas pages "Source layer, pairs pooled" (Block code
 * panel: hc_mixes, hc_pre, hc_post, forward), "Reading weights" (reading-weight
 * equation; split/Sinkhorn kernel panel), "Write the streams" (stream-update
 * equation) and "Final RMSNorm" (RMSNorm equation and class).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major and
 *     contiguous.  The library keeps no pointer after a call returns and
 *     allocates no memory in any compute entry point.
 *   - bf16 tensors are passed as raw bit patterns (hc_bf16) and must be 16-byte
 *     aligned; float tensors must be 16-byte aligned.
 *   - n = number of tokens (batch x positions, flattened).  hc is 2, 4 or 8;
 *     hc = 4 (the pages' setting) runs the fused kernels, hc = 2 and 8 a
 *     plainer schedule of separate launches (the write, the projection, the
 *     split, the read; at hc = 2 a boundary with a write and a fresh pre does
 *     the write and the projection in one pass), with the same arithmetic.  d must be a positive
 *     multiple of 64 and at most 32768 (at most 10240 where the read row is
 *     RMS-normalised).
 *   - stream is a hipStream_t (NULL = the null stream).  Calls enqueue work on
 *     it and return without synchronising; the current HIP device of the
 *     calling thread is used.  Calls on distinct streams may run concurrently
 *     from different threads.
 *   - Arguments are validated before any HIP call: a bad argument returns
 *     HC_EINVAL or HC_ENOTSUP and enqueues nothing.  n == 0 returns HC_OK and
 *     enqueues nothing.  A failed launch returns HC_EHIP; hc_last_error() then
 *     names the HIP error.  Faults inside a kernel surface, as with any
 *     asynchronous HIP work, at the caller's next synchronisation.
 *   - Inputs and outputs must not overlap unless an entry point says so.
 *   - No NaN/Inf checks are made; non-finite inputs propagate.
 */
#ifndef HC_H
#define HC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t hc_bf16; /* raw bf16 bit pattern */

enum hc_status {
  HC_OK = 0,
  HC_EINVAL = -1,  /* NULL or misaligned pointer, negative size, iters < 1, ... */
  HC_ENOTSUP = -2, /* hc not 2/4/8, d not a multiple of 64, or d too large    */
  HC_EHIP = -3,    /* a HIP call or kernel launch failed                        */
  HC_ENODEV = -4   /* no HIP device is visible                                  */
};

/* Library version as 10000*major + 100*minor + patch. */
int hc_version(void);

/* Static description of a status code (never NULL). */
const char* hc_strerror(int status);

/* Detail of the last failure on the calling thread ("" if none).  The string
 * stays valid until the next call on this thread. */
const char* hc_last_error(void);

/* ---------------------------------------------------------------------------
 * Projection weight packing.
 * The projection weight hc_fn is [(2+hc)*hc, hc*d] float32 in the out x in
 * layout of a linear layer ("Source layer, pairs pooled": Block constructor).
 * The compute entry points take it pre-packed: each fp32 weight is split into
 * three bf16 terms hi + mid + lo (each the nearest bf16 to what the previous
 * terms leave), which together hold the fp32 value to about 2^-26 relative,
 * laid out in the tile order of the matrix-core kernels (one order for hc =
 * 4, another for hc = 2 and 8).  Pack once per parameter set.
 * ------------------------------------------------------------------------- */

/* Bytes of the packed weight for (hc, d); 0 if (hc, d) is not supported. */
size_t hc_fn_packed_bytes(int hc, int d);

/* hc_fn [(2+hc)*hc, hc*d] float32 -> fn_packed (hc_fn_packed_bytes(hc, d)
 * bytes, 16-byte aligned): each fp32 weight split exactly into three bf16
 * terms, laid out as the matrix cores' operand tiles; at hc = 4 followed by the
 * same tiles of the weight summed over the four stream blocks (the projection
 * of four identical streams, used by the block entry from the expanded
 * embedding).  Pack once per parameter set. */
int hc_fn_pack(const float* hc_fn, int hc, int d, void* fn_packed, void* stream);

/* ---------------------------------------------------------------------------
 * Workspace.  The entry points that derive mixes (hc_mixes, hc_boundary with
 * fn_packed) split the feature range of each token over several workgroups,
 * which leave per-token partial sums in a caller-owned device workspace of
 * hc_workspace_bytes(n, hc, d) bytes (0 for n == 0), 16-byte aligned, for a
 * later kernel, or the last workgroup to finish, to sum.  The workspace must
 * be zero before its first use; the calls keep it valid for the next call (a
 * workspace of the size asked for some (n, d) serves every call that needs no
 * more).  Calls that may run concurrently (different streams) need different
 * workspaces; calls on one stream can share one, also when captured in a
 * graph and replayed.  For hc = 2 and 8 the per-slice sums are placed after
 * the regions an hc = 4 call of the same d keeps, so one workspace may serve
 * calls of every hc.
 *
 * Few token tiles (hc = 4: decode, short prefill).  hc_mixes for n <= 2048,
 * and hc_boundary with a given pre_in (the pages' data flow; with or without
 * gamma), for up to 32 tiles of 64 tokens (2048 tokens at d = 5120), with d a
 * multiple of 64 from 256 to 8192, run as one launch: each workgroup streams a
 * (64-token tile, slice of 1 to 10 chunks of 64 features) item and adds its
 * per-token partial sums to the workspace as tagged words; the owner slice of
 * each token sums the token's words over the slices, derives its mixes,
 * pre/post and comb ("Reading weights") and, with gamma, publishes the
 * token's RMS factor for the other slices, which then write their part of z.
 * All of the launch's workgroups (at most 256) must be resident at once.  A
 * word a workgroup waits for that never becomes visible sets bit 0 of the
 * workspace's error mask (see hc_workspace_status); the call then finishes
 * with wrong results instead of hanging.  The workspace holds a control block
 * (the error mask and the exchanges' call counters) and the exchanges' words
 * at the same place whatever (n, hc, d), then the per-slice sums of the
 * two-launch schedule (or of hc = 2, 8).
 * ------------------------------------------------------------------------- */
size_t hc_workspace_bytes(int64_t n, int hc, int d);

/* The workspace's regions for a call of shape (n, hc, d), as byte offsets and
 * sizes in regions[0..5]: the control block, the exchanges' tagged words
 * (these two at the same place and size for every shape, so that no call
 * writes another call's persistent words), then the per-slice sums of this
 * shape.  Their end is hc_workspace_bytes (for n > 0).  HC_EINVAL /
 * HC_ENOTSUP as hc_workspace_bytes would return 0. */
int hc_workspace_layout(int64_t n, int hc, int d, size_t regions[6]);

/* Reads a workspace's sticky error mask into *mask (host memory), after the
 * work already enqueued on stream has finished (the call synchronises the
 * stream): bit 0 set means that some earlier call on this workspace waited for
 * another workgroup's words until its bound and then finished with wrong
 * values.  With clear != 0 the mask is then reset to zero by work enqueued on
 * stream.  HC_EINVAL for a NULL or misaligned workspace, fewer than 8192 bytes,
 * or a NULL mask; HC_EHIP if the copy fails. */
int hc_workspace_status(void* workspace, size_t workspace_bytes, int clear, uint32_t* mask, void* stream);

/* ---------------------------------------------------------------------------
 * hc_mixes -- "Source layer, pairs pooled", Block.hc_mixes.
 *   r[t]        = 1 / sqrt(mean_c x[t,c]^2 + norm_eps), c over the flattened
 *                 hc*d row (index j*d + i)
 *   mixes[t,q]  = r[t] * sum_c hc_fn[q,c] * x[t,c]
 * x      [n, hc, d] bf16;  fn_packed from hc_fn_pack.
 * mixes  [n, (2+hc)*hc] float32 output, or NULL.
 * If pre, post and comb are all non-NULL the split/Sinkhorn step of
 * hc_split_sinkhorn also runs (with hc_scale, hc_base, iters, hc_eps) and
 * writes them, as Block.hc_mixes returns them; otherwise hc_scale/hc_base/
 * iters/hc_eps are ignored.  At least one of mixes or (pre, post, comb) must
 * be given.  workspace: see hc_workspace_bytes.
 * ------------------------------------------------------------------------- */
int hc_mixes(const hc_bf16* x, const void* fn_packed, int64_t n, int hc, int d, float norm_eps,
             float* mixes, const float* hc_scale, const float* hc_base, int iters, float hc_eps,
             float* pre, float* post, float* comb, void* workspace, size_t workspace_bytes,
             void* stream);

/* ---------------------------------------------------------------------------
 * hc_split_sinkhorn -- "Reading weights": reading-weight equation and the
 * split/Sinkhorn kernel panel.  With m = mixes[t], s = hc_scale, b = hc_base:
 *   pre[t,j]  = sigmoid(s[0]*m[j] + b[j]) + hc_eps                 j < hc
 *   post[t,j] = 2 * sigmoid(s[1]*m[hc+j] + b[hc+j])                j < hc
 *   L[j][k]   = s[2]*m[2hc + j*hc + k] + b[2hc + j*hc + k]
 *   comb      = row softmax of L, + hc_eps; each column divided by (its sum +
 *               hc_eps); then iters-1 rounds of: each row divided by (its sum
 *               + hc_eps), each column divided by (its sum + hc_eps).
 * mixes [n, (2+hc)*hc], hc_scale [3], hc_base [(2+hc)*hc] float32 inputs;
 * pre, post [n, hc] and comb [n, hc, hc] float32 outputs, comb[t][j][k] with
 * j the source stream (row) and k the destination stream (column).
 * iters >= 1.  Arithmetic is fp32.
 * ------------------------------------------------------------------------- */
int hc_split_sinkhorn(const float* mixes, const float* hc_scale, const float* hc_base, int64_t n,
                      int hc, int iters, float hc_eps, float* pre, float* post, float* comb,
                      void* stream);

/* ---------------------------------------------------------------------------
 * hc_pre -- "Source layer, pairs pooled", Block.hc_pre.
 *   y[t,i] = bf16( sum_j pre_mix[t,j] * x[t,j,i] )
 * computed in fp32 with one rounding per product and per partial sum, j
 * ascending (bit-identical to that sequence of fp32 operations).
 * x [n, hc, d] bf16, pre_mix [n, hc] float32 -> y [n, d] bf16.
 * ------------------------------------------------------------------------- */
int hc_pre(const hc_bf16* x, const float* pre_mix, int64_t n, int hc, int d, hc_bf16* y,
           void* stream);

/* ---------------------------------------------------------------------------
 * hc_post -- "Write the streams" stream-update equation; "Source layer, pairs
 * pooled", Block.hc_post (argument order as there: sublayer output first).
 *   x_out[t,k,i] = bf16( post[t,k]*delta[t,i] + sum_j comb[t,j,k]*x[t,j,i] )
 * in fp32 with one rounding per product and per sum: the comb terms summed
 * j ascending, then added to the post term (bit-identical to that sequence).
 * delta [n, d] bf16, x [n, hc, d] bf16, post [n, hc], comb [n, hc, hc]
 * float32 -> x_out [n, hc, d] bf16 (must not overlap x or delta).
 * ------------------------------------------------------------------------- */
int hc_post(const hc_bf16* delta, const hc_bf16* x, const float* post, const float* comb,
            int64_t n, int hc, int d, hc_bf16* x_out, void* stream);

/* ---------------------------------------------------------------------------
 * hc_boundary -- one sublayer boundary in one pass over the streams, read off
 * "Source layer, pairs pooled", Block.forward:
 *   X'              = hc_post(delta, x, post_in, comb_in)       (skipped if delta == NULL: X' = x)
 *   pre/post/comb   = hc_split_sinkhorn(hc_mixes(X'))           (skipped if fn_packed == NULL)
 *   y               = hc_pre(X', pre_in)                        (pre_in == NULL: the pre just derived)
 *   y_out           = gamma ? RMSNorm_gamma(y, rms_eps) : y
 * RMSNorm ("Final RMSNorm"): y_out[t,i] = bf16(gamma[i] * (y[t,i] * r)),
 * r = 1/sqrt(mean_i y[t,i]^2 + rms_eps), on the bf16 y.  With pre_in == NULL
 * the mean square is instead formed as p^T G p from the 4x4 Gram matrix G of
 * the X' streams, i.e. of the y before its bf16 rounding, so that the row
 * need not wait for its own mean square; the two differ by a relative 2^-8 at
 * most (from the rounding of y), which moves z by at most half a bf16 ulp.
 * (hc = 2 and 8 take the mean square of the bf16 y in every case, running the
 * write, the projection, the split and the read as separate launches: begin
 * enqueues the write, and the read when pre_in is given; end the rest.  At
 * hc = 2 with delta and a fresh pre, begin enqueues the write and the
 * projection as one pass, end the split and the read.)
 * With pre_in given the call follows the pages' data flow: the streams are
 * read with the reading mix of the previous boundary and the call returns the
 * (pre, post, comb) of this boundary for the next one.  Use delta == NULL at a
 * block entry and fn_packed == NULL at the stack exit.
 * x_out must not overlap x; y_out must not overlap x, x_out or delta.
 * workspace/workspace_bytes: required when fn_packed != NULL, see
 * hc_workspace_bytes (hc_boundary_workspace_bytes returns the same size).
 * flags: 0, or HC_BOUNDARY_* bits (below); a caller built against a header
 * without this field passes the shorter struct_size and gets 0.
 *
 * Schedules (hc = 4).  With a given pre_in (or at a block entry without a
 * read) and few token tiles (see hc_workspace_bytes: up to 2048 tokens at d =
 * 5120), the call is one launch, the few-tile exchange.  With a given pre_in
 * and gamma beyond that, when the feature slices of a token tile are 640 or
 * 1280 features wide and a tile has 4 to 8 of them (d = 5120 up to 4096
 * tokens, or in general d / S for the slice count S the call picks), the call
 * is one launch as well: each slice keeps its read row on chip, the slices of
 * a tile exchange their per-token sums through the workspace as tagged words,
 * and the RMSNorm is applied without writing y first; beyond 4096 tokens
 * (when 4096 tokens take that form) the call runs as consecutive such calls
 * of 4096 tokens and a last one for the rest (so does a call with a fresh pre
 * from 16384 tokens on).  In every other case two launches: a streaming pass (X', the read row of
 * a given pre, per-slice sums) and a finish (mixes, pre/post/comb, and the read
 * row where it depends on them or on its RMSNorm).  A wait for another
 * workgroup's words that times out sets bit 0 of the workspace's error mask
 * (hc_workspace_status) and the call finishes with wrong values instead of
 * hanging; one call at a time per workspace.
 * ------------------------------------------------------------------------- */
/* x is [n, d] and every one of the hc streams is that row: the stack entry
 * ("Final RMSNorm", the model driver copies the embedding into hc streams)
 * without materialising the copies.  With delta the call writes the real
 * streams to x_out; without, it derives the mixes of the copies and reads
 * them. */
#define HC_BOUNDARY_X_EXPANDED 4u
/* Always the two-launch schedule (the one hc_boundary_begin / _end run):
 * never one of the one-launch exchanges. */
#define HC_BOUNDARY_TWO_LAUNCH 16u

typedef struct hc_boundary_args {
  uint32_t struct_size; /* = sizeof(hc_boundary_args) */
  int32_t hc, d, iters;
  int64_t n;
  float hc_eps, norm_eps, rms_eps;
  const hc_bf16* delta;    /* [n, d] or NULL (block entry)                      */
  const hc_bf16* x;        /* [n, hc, d]                                         */
  const float* post_in;    /* [n, hc]      required iff delta != NULL            */
  const float* comb_in;    /* [n, hc, hc]  required iff delta != NULL            */
  const float* pre_in;     /* [n, hc] or NULL (read with the pre just derived)   */
  const void* fn_packed;   /* packed weight, or NULL (stack exit: no mixes)      */
  const float* hc_base;    /* [(2+hc)*hc]  required iff fn_packed != NULL        */
  const float* hc_scale;   /* [3]          required iff fn_packed != NULL        */
  const float* gamma;      /* [d] RMSNorm gain, or NULL (no RMSNorm)             */
  hc_bf16* x_out;          /* [n, hc, d]   required iff delta != NULL            */
  hc_bf16* y_out;          /* [n, d]       required                              */
  float* mixes_out;        /* [n, (2+hc)*hc] or NULL                             */
  float* pre_out;          /* [n, hc]      required iff fn_packed != NULL        */
  float* post_out;         /* [n, hc]      required iff fn_packed != NULL        */
  float* comb_out;         /* [n, hc, hc]  required iff fn_packed != NULL        */
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;          /* 0, or HC_BOUNDARY_* bits (above)                    */
  /* [n, d] bf16 or NULL: the mean over the hc streams of the new streams (x_out,
   * or x at a block entry), the MTP head's tap of a block's input ("Final
   * RMSNorm", the model driver); the streams summed in fp32 in stream order
   * (((X'_0 + X'_1) + X'_2) + X'_3 at hc = 4), times 1/hc, rounded to bf16.
   * A caller built against a header
   * without this field passes the shorter struct_size. */
  hc_bf16* x_mean_out;
} hc_boundary_args;

int hc_boundary(const hc_boundary_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * hc_boundary_static -- hc_boundary for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same call, but args->workspace and workspace_bytes
 * are ignored and the library's own static device workspace is used instead
 * (16 MiB on each GPU the library runs on, held until the process ends; zero
 * when the library is loaded).  It allocates nothing.  Shapes whose workspace
 * (hc_workspace_bytes) exceeds 16 MiB return HC_ENOTSUP -- hc = 4 fits up to
 * 92 736 tokens at d = 5120.  Every call on one GPU shares that GPU's
 * static workspace, which keeps the last call's contents: calls that may
 * overlap on one GPU (different streams, different threads) race and must be
 * serialised by the caller.  Same status codes as hc_boundary.
 * ------------------------------------------------------------------------- */
int hc_boundary_static(const hc_boundary_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * hc_boundary_begin / hc_boundary_end -- hc_boundary in two halves, for a
 * caller that places other work between them or times them apart.  With
 * fn_packed, begin enqueues the streaming pass (x_out; with pre_in, y; the
 * per-slice partial sums into the workspace) and end the finish (mixes,
 * pre/post/comb, and the read row where it depends on them).  Without
 * fn_packed, begin does the whole call and end does nothing.  Call end with
 * the same arguments, on the same stream or ordered after begin; nothing may
 * touch the workspace or the outputs in between.  Both validate as
 * hc_boundary and return its status codes; begin followed by end computes
 * exactly what hc_boundary does.
 * ------------------------------------------------------------------------- */
int hc_boundary_begin(const hc_boundary_args* args, void* stream);
int hc_boundary_end(const hc_boundary_args* args, void* stream);

/* Workspace bytes hc_boundary needs for n tokens (= hc_workspace_bytes). */
size_t hc_boundary_workspace_bytes(int64_t n, int hc, int d);

#ifdef __cplusplus
}
#endif

#endif /* HC_H */
