// Internal (host + device) description of one call: sizes and every device pointer the
// kernels touch. Passed to kernels by value.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct Args {
  // sizes
  int N, H, HV, G, D, NT;
  int64_t T;
  int dtype; // 0 bf16, 1 f32 (io tensors)
  int l2norm, has_h0, want_ht, full;
  // inputs
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu;
  const float* h0;
  const void* dO;
  const float* dht;
  // outputs
  void* o;
  float* ht;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dh0;
  // saved set
  uint16_t* akk;   // bf16 [T, HV, 64]: row i of the chunk's (I + L)^-1 at the token of row i
  float* gcum;     // f32  [HV, T]: in-chunk inclusive cumulative log decay (head-major, so that
                   // a chunk's 64 tokens of one head are one 256-byte run)
  float* gamma;    // f32  [NT, HV]: exp(gcum of the chunk's last token)
  uint16_t* htape; // bf16 [NT, HV, d(value), d(key)]: state at each chunk start, transposed
  uint16_t* vnew;  // bf16 [T, HV, d]: R = U - W S (full form only)
  uint16_t* w;     // bf16 [T, HV, d] (full form only)
  uint16_t* u;     // bf16 [T, HV, d] (full form only)
  uint16_t* aqk;   // bf16 [T, HV, 64]: decayed, masked q.k (full form only)
  // workspace
  int* seq_c0;     // [N + 1] first chunk of each document
  int* c_t0;       // [NT] first token of each chunk
  int* c_len;      // [NT] valid tokens of each chunk (1..64)
  int* seq_order;  // [N] documents, longest first
  int* status;     // [1] 0 ok; 1 the device tables disagree with the host's chunk count;
                   // 2 (backward) the saved set's tag does not name this problem
  float* rk;       // [H, T] inverse L2 norms of k rows (1 when the norm is off), head-major
  float* rq;       // [H, T] inverse L2 norms of q rows, head-major
  uint16_t* qk;    // bf16 [NT, HV, 64, 64] P = exp(G_q - G_k) qh.kh masked to q >= k, per value head
                   // (row-major P for the forward, P^T for the backward)
  uint16_t* dstape;// bf16 [NT, HV, d(value), d(key)]: gradient of each chunk's end state, transposed
  float* dqacc;    // f32 [T, H, d] (atomic reduction only)
  float* dkacc;    // f32 [T, H, d] (atomic reduction only)
  // (Fields are appended here: moving the offsets of the fields above has cost the walks several
  // per cent, for reasons the generated loop code does not show.)
  int* pair_order; // [2 (ceil(N H / 8) + 1)] super-groups of the paired walk launches, longest
                   // first (bit 30: reverse walk, else tape walk; low bits: super-group)
  // Part of the problem covered by one launch (the longest document's work and the others' run
  // on two streams). Chain launches cover the (document rank, q/k head) groups [grp_off, grp_end)
  // and read their paired-walk order from pair_order + pair_off. Chunk launches cover c_count
  // chunks: launch index x is chunk c_base + x, plus c_skip from x = c_skip_at on (the other
  // part's chunks form one contiguous range, which is skipped).
  int grp_off, grp_end, pair_off;
  int c_base, c_skip_at, c_skip, c_count;
  int grp_split; // k_tables: paired-walk orders of the groups [grp_split, N H), then [0, grp_split)
  // Forward and tape walks over a piece of each document: its chunks [piece_lo, piece_hi) counted
  // from the document's first. state_in (if set) replaces h0 as the starting state and state_out
  // (if set) receives the final state, both f32 [HV, d, d]: a launch that uses them covers one
  // document, and consecutive pieces hand the state over through them.
  int piece_lo, piece_hi;
  const float* state_in;
  float* state_out;
  // Segmented walks: f32 [slots][HV, d, d] transfer matrices and zero-start end states of the
  // middle segments (workspace), and the segments' start states (the saved set's carry plane).
  float* carry;
  float* splane;
  // k_chunk_grad's work queue: the number of items claimed beyond the grid's first (zeroed once
  // per call, after the tables kernel; a launch that runs beside another has its own counter)
  int* gq;
};

// Segmented walks of long documents (problem->segments >= 2). A document of P segments is walked
// as: its segment 0 from its true start (h0 or 0), and for each middle segment 1..P-2 a transfer
// walk from the identity with v = 0 (the segment's linear map M) and one from zero (its affine
// part B), side by side; then a carry merge S_in(i+1) = M(i) S_in(i) + B(i); then segments 1..P-1
// from their true start states, side by side. Each unit below is one (document, chunk range)
// walked for every value head of the document.
constexpr int MAX_SEG_UNITS = 80;
struct SegUnit {
  int doc;       // document index
  int lo, hi;    // chunks [lo, hi) counted from the document's first
  int kind;      // 0: true walk; 1: transfer walk from the identity with v = 0; 2: walk from zero
  int in_slot;   // carry-plane slot of the start state (-1: h0 or zero)
  int out_slot;  // slot for the end state (-1: none)
  int out_plane; // 1: out_slot is a carry-plane slot (a start state); 0: a workspace slot (M or B)
  int write_ht;  // 1: the document's last segment, writes ht (when the problem wants it)
};
struct SegPlan {
  int n_units;
  SegUnit u[MAX_SEG_UNITS];
};
// Carry merge of one document: S_in(i + 1) = M(i) S_in(i) + B(i), i = 1 .. n_mid, with S_in(i) in
// carry-plane slot s_base + i - 1, M(i) in workspace slot m_base + i - 1, B(i) in b_base + i - 1.
constexpr int MAX_MERGE_DOCS = 32;
struct MergeDoc {
  int s_base, m_base, b_base, n_mid;
};
struct MergePlan {
  int n_docs;
  MergeDoc d[MAX_MERGE_DOCS];
};

int chain_blocks(const Args& a, int ntile);

// Whole-problem launch ranges (every group, every chunk, no split of the paired-walk order).
void whole_range(Args& a);

// Launchers (defined in the .hip translation units). Each returns a hipError_t as int.
// tag / tag_words: the saved set's 256-byte tag and the four words it must hold (backward calls
// only; NULL otherwise). A mismatch sets status 2, a cu_seqlens disagreement status 1.
int launch_tables(const Args& a, const uint64_t* tag, const uint64_t* tag_words, void* stream);
int launch_intra(const Args& a, int bwd_prep, void* stream);
// write_tape: the chunk-start state tape; write_vnew: v_new (the full saved set)
int launch_walk_fwd(const Args& a, int write_o, int write_tape, int write_vnew, void* stream);
// The units of a segment plan: true walks (transfer = 0) or transfer walks (transfer = 1, which
// write nothing but their end states).
int launch_walk_seg(const Args& a, const SegPlan& plan, int write_o, int write_tape, int write_vnew, int transfer,
                    void* stream);
int launch_seg_merge(const Args& a, const MergePlan& plan, void* stream);
int launch_walk_pair(const Args& a, void* stream); // tape walk and reverse walk in one launch
int launch_wy_full(const Args& a, void* stream);
int launch_walk_bwd(const Args& a, void* stream);
int launch_chunk_grad(const Args& a, int deterministic, void* stream);
int launch_fill_zero(float* p, size_t n, void* stream);
int launch_finalize_qk(const Args& a, void* stream);
// The saved set's tag (zeros when the call's status is nonzero, so that it is refused later).
int launch_write_tag(void* dst, const uint64_t* words, const int* status, void* stream);
// When the call's status is nonzero: its floating-point outputs (op GDN_OP_FWD: o, ht;
// GDN_OP_BWD: dq, dk, dv, dg, dbeta, dh0) are filled with NaN. Otherwise it does nothing.
int launch_poison(const Args& a, int op, void* stream);

// Short causal conv1d + SiLU front-end (gdn_conv.hip): sizes and pointers of one call.
struct ConvArgs {
  int64_t T;
  int C, W, N, silu, n_groups;
  int goff[5]; // channel offset of each output group (goff[n_groups] = C)
  const void* x;
  const float* w;
  const float* b;
  const int32_t* cu;
  void* y[4];
  const void* dy[4];
  void* dx;
  float* dw;
  float* db;
  float* part; // [blocks][C][W + 1] partial sums of dweight and dbias
};

// Workgroups along the tokens (each covers 1024 tokens); the backward's partial sums are
// [conv_blocks(T)][C][W + 1] f32.
int conv_blocks(int64_t T);
int launch_conv_fwd(const ConvArgs& a, int dtype, void* stream);
int launch_conv_bwd(const ConvArgs& a, int dtype, void* stream);

} // namespace gdn
