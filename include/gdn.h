/*
 * gdn.h — C ABI of the MI355X (gfx950) chunked gated-delta-rule training kernel.
 *
 * The operation (Gated DeltaNet training, forward and backward, on packed variable-length
 * sequences; flashinfer PR #8172 "non-deterministic context-parallel Cake GDN chunked
 * autograd backend", PR description) is, per document n and value head h, with q/k head
 * j = h / (HV / H):
 *
 *     qh, kh = l2norm(q_t), l2norm(k_t)        (only when l2norm_qk; l2norm(x) = x / sqrt(x.x + 1e-6))
 *     S_t    = exp(g_t) S_{t-1} + beta_t kh (v_t - exp(g_t) S_{t-1}^T kh)^T
 *     o_t    = S_t^T qh
 *
 * with S_0 = h0[n,h] (or 0) a d x d FP32 state (row = key index) and ht[n,h] = S_last.
 * g is the log decay and beta the write strength, both used as given. Documents never share
 * state. The argument set (q, k, v, g, beta, cu_seqlens, optional h0, optional in-kernel
 * q/k L2 norm, light/full saved set) follows the pages' problem statement (flashinfer PR #8542
 * description and README saved-set table quoted in its review).
 *
 * Layouts (row-major, token-major, all pointers 16-byte aligned device pointers):
 *   q, k        [T, H,  d]   io dtype (bf16 or f32)
 *   v, o        [T, HV, d]   io dtype
 *   dO, dv      [T, HV, d]   io dtype
 *   dq, dk      [T, H,  d]   io dtype
 *   g, beta     [T, HV]      f32;  dg, dbeta [T, HV] f32
 *   h0, ht      [N, HV, d, d] f32 (key index, value index); dht, dh0 the same
 *   cu_seqlens  [N + 1]      int32, cu_seqlens[0] = 0, nondecreasing, cu_seqlens[N] = T
 *
 * Ownership: the caller allocates every buffer (outputs, the saved set, the workspace) and
 * owns every stream. The library never allocates or frees device memory, never creates a
 * stream and never synchronises the host (gdn_status, a query, is the one call that waits).
 * Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and, when the
 * problem names one, on the caller's auxiliary stream problem->aux_stream: all of it runs
 * after the work enqueued on `stream` before the call and before the work enqueued there
 * after it (the auxiliary stream is forked from and joined back into `stream` with events).
 * With aux_stream = NULL every launch goes to `stream`. Inputs are not modified. Calls are
 * reentrant; calls that share a workspace or a saved buffer must not overlap. Concurrent calls
 * may name the same auxiliary stream: their auxiliary work then runs there one call after the
 * other.
 *
 * Errors: every entry returns GDN_OK or an error code; gdn_last_error() gives a message for
 * the calling thread. Host validation (shapes, cu_seqlens, sizes, pointers, alignment) runs
 * before the first launch, so a call it rejects writes nothing. A launch failure returns
 * GDN_EHIP. Two conditions can only be seen on the device, by the first kernel of a call:
 * a device cu_seqlens that disagrees with the host copy in the problem, and (gdn_bwd) a saved
 * buffer whose 256-byte tag does not name this problem, save mode and ABI version. Then every
 * kernel of the call skips its work, the call's floating-point outputs are filled with NaN,
 * and gdn_status() reports GDN_EINVAL or GDN_ESAVED. Faults inside kernels surface at the
 * caller's next synchronisation.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

/* return codes */
#define GDN_OK 0
#define GDN_EINVAL 1       /* bad shape, cu_seqlens, null required pointer, misalignment */
#define GDN_EUNSUPPORTED 2 /* d not 64 or 128, or an unsupported dtype */
#define GDN_ESAVED 3       /* saved buffer not written by gdn_fwd/gdn_fwd_recompute for this problem */
#define GDN_EWORKSPACE 4   /* workspace smaller than gdn_workspace_bytes() */
#define GDN_EHIP 5         /* a HIP launch or runtime call failed */

/* io dtypes (q, k, v, o, dO, dq, dk, dv) */
#define GDN_DTYPE_BF16 0
#define GDN_DTYPE_F32 1

/* Saved-set forms (README saved-set table quoted in the review of flashinfer PR #8542; the
 * kept-tape form follows the `reuse_recompute_tapes` row of the option table quoted in the
 * review of flashinfer PR #8172).
 * LIGHT keeps Akk (the inverse of I + L per chunk, bf16 [T, HV, 64]), gcum (f32 [HV, T]) and
 * gamma (f32 [NT, HV]); the backward replays the state tape. FULL also keeps the state tape
 * (bf16 [NT, HV, d, d]), v_new (bf16 [T, HV, d]), w and u (bf16 [T, HV, d]) and Aqk
 * (bf16 [T, HV, 64]). TAPE keeps LIGHT plus the state tape only: a checkpointed step runs
 * gdn_fwd in LIGHT form, then gdn_fwd_recompute and gdn_bwd in TAPE form, so the backward binds
 * the tape that the recompute's walk wrote instead of replaying it. FULL and TAPE backwards
 * skip the replay walk. All forms give bitwise identical outputs and gradients. */
#define GDN_SAVE_LIGHT 0
#define GDN_SAVE_FULL 1
#define GDN_SAVE_TAPE 2

/* operations, for gdn_workspace_bytes and gdn_status */
#define GDN_OP_FWD 0
#define GDN_OP_RECOMPUTE 1
#define GDN_OP_BWD 2

typedef struct gdn_problem {
  int32_t n_seqs;                 /* N >= 1 documents (zero-length documents allowed) */
  int32_t h_qk;                   /* H q/k heads */
  int32_t h_v;                    /* HV value heads, a multiple of H */
  int32_t d;                      /* head dim, d_k = d_v = 64 or 128 */
  int64_t n_tokens;               /* T = cu_seqlens[N] */
  int32_t dtype;                  /* GDN_DTYPE_* of the io tensors */
  int32_t l2norm_qk;              /* 1: L2-normalise q and k rows inside the kernel */
  int32_t has_h0;                 /* 1: h0 is given (and gdn_bwd writes dh0) */
  int32_t want_ht;                /* 1: gdn_fwd writes ht */
  int32_t save_mode;              /* GDN_SAVE_LIGHT, GDN_SAVE_FULL or GDN_SAVE_TAPE */
  int32_t deterministic;          /* 1: fixed-order dq/dk reduction over the HV/H value heads
                                     of each q/k head (bitwise reproducible); 0: FP32 atomics */
  const int32_t* cu_seqlens_host; /* host copy of cu_seqlens, read during each call only */
  void* aux_stream;               /* optional second stream (hipStream_t) of the caller on the
                                     device of `stream`; NULL: every launch on `stream` */
  int32_t segments;               /* walk segments per document (the PR #8172 README option
                                     table's `segments` / `walk_seg` and its plan policy):
                                     1 = each document's state walk is one serial chain;
                                     P >= 2 = documents of at least 16 chunks are walked as up to
                                     P segments (transfer walks, a carry merge, then the
                                     segments' walks side by side); 0 = the library's count,
                                     from the shape and the device's CU count (segments only
                                     when the chains fill at most half of the CUs). At P > 1
                                     the saved set ends with the segments' start states */
  int32_t reserved0;              /* must be 0 */
} gdn_problem;

/* Bytes of the saved buffer for this problem and save_mode: a 256-byte tag plus the saved
 * tensors, each 256-byte aligned (per-token figures of the README saved-set table quoted in
 * the review of flashinfer PR #8542: light 6,339 B/token and full +67,584 B/token at
 * HV = 48, d = 128, all chunks full). 0 if the problem is invalid (see gdn_last_error). */
size_t gdn_saved_bytes(const gdn_problem* p);

/* Bytes of device workspace one call of `op` needs: chunk tables, the status word, inverse q/k
 * norms, the per-value-head decayed q.k tiles, the replayed state tape, the end-state-gradient
 * tape and the chunk-gradient work-queue counters (backward), FP32 dq/dk accumulators (atomic
 * reduction), the segment carry states. The
 * pages' byte queries (flashinfer PR #8172 description: saved, workspace and communication
 * byte-accounting APIs) are the model. 0 if the problem is invalid. */
size_t gdn_workspace_bytes(const gdn_problem* p, int op);

/* Forward (flashinfer PR #8172 description: the chunked training kernel's forward call; the
 * chunk programs it runs are those the commit messages of flashinfer PR #7097 name: prep,
 * intra, WY and the state walk). Writes o [T, HV, d], ht [N, HV, d, d] (if want_ht) and the
 * saved set. h0 may be NULL iff has_h0 = 0; ht may be NULL iff want_ht = 0. */
int gdn_fwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
            void* saved, void* workspace, size_t workspace_bytes, void* stream);

/* Checkpoint re-run of the forward (flashinfer PR #8172 description: the checkpointed call;
 * README option table: `recompute_output`, the re-run that launches no output program).
 * Writes the saved set only (no o, no ht), bitwise equal to the saved set gdn_fwd writes for
 * the same inputs and save_mode. */
int gdn_fwd_recompute(const gdn_problem* p, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const int32_t* cu_seqlens,
                      const float* h0, void* saved, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Backward (flashinfer PR #8172 description: the backward call, with its gradient-state
 * traversal and gradient programs; the deterministic and float-atomic dq/dk reductions are
 * the pages' deterministic and non-deterministic packages). Reads the saved set of the
 * matching forward or recompute (same problem and save_mode), dO and optional dht (NULL = 0),
 * and writes dq, dk, dv, dg, dbeta and (if has_h0) dh0. */
int gdn_bwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const int32_t* cu_seqlens, const float* h0, const void* saved,
            const void* dO, const float* dht, void* dq, void* dk, void* dv, float* dg,
            float* dbeta, float* dh0, void* workspace, size_t workspace_bytes, void* stream);

/* Device-side status of the last call of `op` that used this workspace (the refusals of
 * flashinfer PR #8542's description: a saved set that does not match is refused). Enqueues a
 * copy of the status word on `stream` and waits for `stream`: this query synchronises the
 * host. Returns GDN_OK, GDN_EINVAL (the device cu_seqlens disagreed with the host copy) or
 * GDN_ESAVED (gdn_bwd was given a saved buffer whose tag does not name this problem, save
 * mode and ABI version); a copy failure returns GDN_EHIP. */
int gdn_status(const gdn_problem* p, int op, const void* workspace, void* stream);

/* Size of the fixed device scratch array behind gdn_fwd_noalloc (64 MiB per device). */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* gdn_fwd for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same forward, with its workspace in a
 * fixed device array of GDN_NOALLOC_SCRATCH_BYTES that the library holds on each device until
 * the process ends, instead of a caller's buffer. Every launch goes to `stream` (aux_stream is
 * ignored); no device memory is allocated or freed and no event is created. A problem whose
 * forward workspace (gdn_workspace_bytes(p, GDN_OP_FWD)) exceeds the array is refused with
 * GDN_EWORKSPACE. Calls on one device share the array: calls that overlap there (two streams,
 * two threads) race and must not be issued. */
int gdn_fwd_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
                    void* saved, void* stream);

/* ---- Short causal conv1d + SiLU front-end ------------------------------------------------
 * The depthwise causal convolution that the pages run over the packed q/k/v channels together
 * with the gated delta rule (flashinfer PR #8542 "Conventions": shape B23 runs the short causal
 * convolution over the 10,240 packed q/k/v channels on every timed call; flashinfer PR #7117: the
 * causal conv1d + SiLU training backend of the same kernel family; the README saved-set table
 * keeps at most 3 history rows, a window of 4 taps). Per document (cu_seqlens as above), channel
 * c and token t:
 *
 *     pre[t, c] = bias[c] + sum_{i<W} weight[c, i] x[t - (W-1) + i, c]   (x = 0 before the document)
 *     y[t, c]   = SiLU(pre[t, c]) = pre / (1 + exp(-pre))                 (pre when silu = 0)
 *
 * x is [T, C] in the io dtype; weight f32 [C, W] (tap W-1 multiplies the current token); bias f32
 * [C] or NULL. The output channels are written split into n_groups tensors y[g] of
 * [T, group_channels[g]] (e.g. q, k, v: 2048, 2048, 6144 channels), so the gated delta rule reads
 * them without a copy; the backward takes the upstream gradients split the same way and writes dx
 * [T, C], dweight f32 [C, W] and dbias f32 [C] (if non-NULL). The weight and bias gradients are
 * summed in a fixed order (bitwise reproducible). Ownership, streams and errors as above; these
 * calls use `stream` only. */
typedef struct gdn_conv_problem {
  int32_t n_seqs;                 /* N >= 1 documents */
  int32_t channels;               /* C = sum of group_channels, a multiple of 8 */
  int64_t n_tokens;               /* T = cu_seqlens[N] */
  int32_t width;                  /* W taps, 1..4 */
  int32_t dtype;                  /* GDN_DTYPE_* of x, y, dy, dx */
  int32_t silu;                   /* 1: y = SiLU(pre); 0: y = pre */
  int32_t n_groups;               /* 1..4 output tensors */
  int32_t group_channels[4];      /* channels of each output tensor, multiples of 8 */
  const int32_t* cu_seqlens_host; /* host copy of cu_seqlens, read during each call only */
} gdn_conv_problem;

/* Bytes of device workspace gdn_conv_bwd needs (the per-workgroup partial sums of dweight and
 * dbias). 0 if the problem is invalid. */
size_t gdn_conv_workspace_bytes(const gdn_conv_problem* p);

/* Forward: y[g] for every group. */
int gdn_conv_fwd(const gdn_conv_problem* p, const void* x, const float* weight, const float* bias,
                 const int32_t* cu_seqlens, void* const* y, void* stream);

/* Backward: dx, dweight and (if non-NULL) dbias from x and the split upstream gradients dy[g]. */
int gdn_conv_bwd(const gdn_conv_problem* p, const void* x, const float* weight, const float* bias,
                 const int32_t* cu_seqlens, const void* const* dy, void* dx, float* dweight, float* dbias,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Message of the calling thread's last error ("" if none). */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

/* Kernel timing, for benchmarks. While enabled (on = 1), every kernel launch of the library is
 * bracketed by two hipEvents recorded on the stream it is launched on (no synchronisation at
 * launch). gdn_timing_collect waits for all recorded events, adds their elapsed times to
 * per-kernel totals and returns the number of distinct kernels; for the first `max` (in name
 * order) it fills names (valid until the next collect on this thread), total_ms and launch
 * counts (any array may be NULL). gdn_timing_launches (call it before gdn_timing_collect, which
 * drops the pending events) waits for them as well and fills, for up to `max` launches in
 * launch order, the kernel name and the start and end times in ms after the earliest start;
 * it returns the number of pending launches. gdn_timing_reset drops totals and pending events. */
void gdn_timing_enable(int on);
int gdn_timing_collect(int max, const char** names, double* total_ms, int* launches);
int gdn_timing_launches(int max, const char** names, double* start_ms, double* end_ms);
void gdn_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
