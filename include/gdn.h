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
 * Ownership: the caller allocates every buffer (outputs, the saved set, the workspace). The
 * library never allocates or frees device memory and never synchronises the host. Work is
 * enqueued on the stream it is given (a hipStream_t; NULL = the default stream): all of it runs
 * after the work enqueued there before the call and before the work enqueued there after it.
 * When one document is much longer than the others, gdn_fwd, gdn_fwd_recompute (full mode) and
 * gdn_bwd fork part of their launches onto a second stream the library creates once per device
 * (default priority, kept until the process ends) and join it back with events, so this
 * ordering holds as for one stream. Inputs are not modified. Calls are reentrant; calls that
 * share a workspace or saved buffer must not overlap.
 *
 * Errors: every entry returns GDN_OK or an error code; gdn_last_error() gives a message for
 * the calling thread. All validation (shapes, cu_seqlens, sizes, pointers, alignment, the
 * saved-set tag) happens on the host before the first launch, so a rejected call writes
 * nothing. A launch failure returns GDN_EHIP. Faults inside kernels surface at the caller's
 * next synchronisation. The device copy of cu_seqlens must equal the host copy given in the
 * problem; if the device tables built from it disagree with the host's chunk count, every
 * kernel of the call skips all work (outputs are left unwritten) rather than read out of range.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

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

/* saved-set forms (README saved-set table quoted in flashinfer PR #8542):
 * LIGHT keeps Akk (the inverse of I + L per chunk, bf16 [T, HV, 64]), gcum (f32 [HV, T]) and
 * gamma (f32 [NT, HV]); the backward replays the state tape. FULL also keeps the state tape
 * (bf16 [NT, HV, d, d]), v_new (bf16 [T, HV, d]), w and u (bf16 [T, HV, d]) and Aqk
 * (bf16 [T, HV, 64]); the backward then skips the replay walk. Both forms give bitwise
 * identical gradients. */
#define GDN_SAVE_LIGHT 0
#define GDN_SAVE_FULL 1

/* operations, for gdn_workspace_bytes */
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
  int32_t save_mode;              /* GDN_SAVE_LIGHT or GDN_SAVE_FULL */
  int32_t deterministic;          /* 1: fixed-order dq/dk reduction over the HV/H value heads
                                     of each q/k head (bitwise reproducible); 0: FP32 atomics */
  const int32_t* cu_seqlens_host; /* host copy of cu_seqlens, read during each call only */
} gdn_problem;

/* Bytes of the saved buffer for this problem and save_mode (a 256-byte tag plus the saved
 * tensors, each 256-byte aligned). 0 if the problem is invalid (see gdn_last_error). */
size_t gdn_saved_bytes(const gdn_problem* p);

/* Bytes of device workspace one call of `op` needs (chunk tables, norms, q.k products, tapes,
 * FP32 accumulators). 0 if the problem is invalid. */
size_t gdn_workspace_bytes(const gdn_problem* p, int op);

/* Forward. Writes o, ht (if want_ht) and the saved set. h0 may be NULL iff has_h0 = 0; ht may
 * be NULL iff want_ht = 0. */
int gdn_fwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const int32_t* cu_seqlens, const float* h0, void* o, float* ht,
            void* saved, void* workspace, size_t workspace_bytes, void* stream);

/* Checkpoint re-run of the forward: writes the saved set only (no o, no ht), bitwise equal to
 * the saved set gdn_fwd writes for the same inputs (activation checkpointing = forward,
 * recompute, backward). */
int gdn_fwd_recompute(const gdn_problem* p, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const int32_t* cu_seqlens,
                      const float* h0, void* saved, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Backward. Reads the saved set of the matching forward, dO and optional dht (NULL = 0), and
 * writes dq, dk, dv, dg, dbeta and (if has_h0) dh0. */
int gdn_bwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const int32_t* cu_seqlens, const float* h0, const void* saved,
            const void* dO, const float* dht, void* dq, void* dk, void* dv, float* dg,
            float* dbeta, float* dh0, void* workspace, size_t workspace_bytes, void* stream);

/* Message of the calling thread's last error ("" if none). */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

/* Kernel timing, for benchmarks. While enabled (on = 1), every kernel launch of the library is
 * bracketed by two hipEvents recorded on the call's stream (no synchronisation at launch).
 * gdn_timing_collect waits for all recorded events, adds their elapsed times to per-kernel
 * totals and returns the number of distinct kernels; for the first `max` (in name order) it
 * fills names (valid until the next collect on this thread), total_ms and launch counts (any
 * array may be NULL). gdn_timing_reset drops totals and pending events. */
void gdn_timing_enable(int on);
int gdn_timing_collect(int max, const char** names, double* total_ms, int* launches);
void gdn_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
