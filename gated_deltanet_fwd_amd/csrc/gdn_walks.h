// State walks of the chunked gated delta rule on gfx950 (bodies shared by the forward, tape,
// reverse and paired launches).
#pragma once
#include "gdn_device.h"

namespace gdn {

__device__ __forceinline__ bf16x8 scale8(bf16x8 v, float s) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)(s * (float)v[e]);
  return v;
}

// ---------------------------------------------------------------------------------------
// State walk, one workgroup per (document, value head); chunks in order.
// WRITE_O: write o (and ht). WRITE_TAPE: write the chunk-start state tape (bf16, transposed).
// FULL: also write v_new = R.
//
// D / 16 waves; wave w owns value columns [16 w, 16 w + 16) of the state and keeps them, and
// every per-chunk intermediate (K S, X, R, the output), in registers. Results of one MFMA become
// operands of the next by packing alone (k-permuted fragments; A and P are staged with their
// columns permuted to match, so every row fragment is one 16-byte read), and the state, in
// natural key order, is the B operand of K S and the A operand of (Q S)^T. The output is formed transposed, so a lane holds four
// consecutive values of one token's row. The waves never exchange data; LDS holds only the
// chunk's shared inputs (K, Q, V, A, P and per-token factors), double-buffered, so the next chunk
// is staged while this one computes, with one barrier per chunk.
// 16-column value tiles per wave. Every K, Q, A, P and K^T fragment a wave reads from LDS feeds
// one MFMA per tile, so two tiles would halve a chunk step's LDS traffic, but at one wave per
// SIMD the step's dependent chain (K S, X, R, the state update) is no longer hidden by a second
// wave: measured on the packed 262k-token workload, the forward took 7.5 ms with two tiles
// against 6.05 ms with one.
constexpr int WALK_CT = 1;

template <int D>
constexpr int walk_threads() {
  return 64 * (D / (16 * WALK_CT));
}

template <int D, bool WRITE_O>
struct WalkSmem {
  static constexpr int SK = D + 16; // token rows of K, Q, V
  static constexpr int SA = CH + 16; // token rows of A and P, columns k-permuted
  static constexpr int NQ = WRITE_O ? 2 : 1;
  static constexpr int LQ = WRITE_O ? CH * SK : 8;
  static constexpr int LP = WRITE_O ? CH * SA : 8;
  bf16 sK[2][CH * SK];
  bf16 sV[2][CH * SK];
  bf16 sA[2][CH * SA];
  bf16 sQ[NQ][LQ];
  bf16 sP[NQ][LP];
  // per token: exp(G) rk, beta, exp(G_last - G) rk, exp(G) rq (zero past the chunk's end);
  // gamma = exp(G_last)
  float sc[2][4][CH];
  float sgam[2];
};

// One chain of a segmented walk (see SegPlan): the unit's document, chunk range and carry slots,
// and the value head.
struct SegChain {
  int n, j, gi;       // document, q/k head, value head within the group
  int lo, hi;         // chunks [lo, hi) counted from the document's first
  int kind;           // SegUnit::kind
  const float* s_in;  // start states [HV, d, d] (NULL: h0 or zero)
  float* s_out;       // end states [HV, d, d] (NULL: none)
  int write_ht;
};

// SEG = 0: a chain of a whole-document launch (decode_chain, pieces); SEG = 1: a true walk of a
// segment; SEG = 2: a walk that writes only its end state (kind 0: from the true start state;
// kind 1: from the identity with v = 0; kind 2: from zero).
template <int D, typename TI, bool WRITE_O, bool WRITE_TAPE, bool FULL, int SEG = 0>
__device__ __forceinline__ void walk_fwd_body(const Args& a, int blk, WalkSmem<D, WRITE_O>& sm,
                                              const SegChain& sc = SegChain{}) {
  if (a.status[0]) return;
  int n, j, h, c_begin, c_end, piece_lo;
  if constexpr (SEG == 0) {
    const ChainMap cm = decode_chain(blk, a, 1);
    if (!cm.valid) return;
    // chain constants are uniform: held in scalar registers (the chunk's buffer resources below
    // are built from them)
    n = __builtin_amdgcn_readfirstlane(a.seq_order[cm.rank]);
    j = cm.j;
    h = j * a.G + cm.gi;
    // this launch's piece of the document: chunks [piece_lo, piece_hi) from its first
    const int c_doc = __builtin_amdgcn_readfirstlane(a.seq_c0[n]);
    piece_lo = a.piece_lo;
    c_begin = c_doc + a.piece_lo;
    c_end = c_doc + min(__builtin_amdgcn_readfirstlane(a.seq_c0[n + 1]) - c_doc, a.piece_hi);
  } else {
    n = sc.n;
    j = sc.j;
    h = j * a.G + sc.gi;
    const int c_doc = __builtin_amdgcn_readfirstlane(a.seq_c0[n]);
    piece_lo = sc.lo;
    c_begin = c_doc + sc.lo;
    c_end = c_doc + sc.hi;
  }
  // transfer walk from the identity: v contributes nothing
  const bool zero_v = SEG == 2 && sc.kind == 1;
  constexpr int NT = walk_threads<D>();
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int NRT = D / 16;       // state row tiles (key dim)
  constexpr int KD = D / 32;        // k-steps over the key dim
  constexpr int RP = D / 8;         // 16-byte pieces per token row of K, Q, V
  constexpr int PPT = CH * RP / NT; // pieces per thread of a 64 x D token tile (2)
  constexpr int APT = CH * 8 / NT;  // pieces per thread of a 64 x 64 tile
  using SM = WalkSmem<D, WRITE_O>;
  constexpr int SK = SM::SK, SA = SM::SA;
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;
  const TI* vp = (const TI*)a.v;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  const bf16* pm = reinterpret_cast<const bf16*>(a.qk);
  constexpr int CT = WALK_CT;
  const int v0 = 16 * CT * w; // tile ct holds value columns v0 + 16 ct ..
  // chunk c of the piece starts at token doc_t0 + 64 (c - c_begin)
  const int doc_t0 = __builtin_amdgcn_readfirstlane(a.cu[n]) + piece_lo * CH;
  const int doc_t1 = __builtin_amdgcn_readfirstlane(a.cu[n + 1]);

  // ---- staging: global -> registers (issued before a chunk's compute) -> LDS (after it).
  // The token tiles are read through buffer resources bounded at the chunk's last row, at
  // per-lane offsets fixed for the whole walk: rows past the chunk's end read as zeros, whose
  // contributions vanish (beta and the row factors are zero there and P is masked).
  int oK[PPT], oV[PPT], oA[APT], oP[APT]; // element offsets of this thread's pieces
#pragma unroll
  for (int it = 0; it < PPT; ++it) {
    const int p = tid + NT * it, row = p / RP, pc = p % RP;
    oK[it] = row * a.H * D + pc * 8;
    oV[it] = row * a.HV * D + pc * 8;
  }
#pragma unroll
  for (int it = 0; it < APT; ++it) {
    const int p = tid + NT * it, row = p >> 3, pc = p & 7;
    oA[it] = row * a.HV * CH + pc * 8;
    oP[it] = row * CH + pc * 8;
  }
  bf16x8 rK[PPT], rV[PPT], rQ[PPT], rA[APT], rP[APT];
  float sg = 0.f, sglast = 0.f, sbeta = 0.f, srk = 0.f, srq = 0.f;
  auto load_chunk = [&](int c) {
    const int t0 = doc_t0 + (c - c_begin) * CH;
    const int last = min(CH, doc_t1 - t0) - 1;
    const int kq_bytes = (last * a.H * D + D) * (int)sizeof(TI), v_bytes = (last * a.HV * D + D) * (int)sizeof(TI);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp + ((size_t)t0 * a.H + j) * D, kq_bytes);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qp + ((size_t)t0 * a.H + j) * D, kq_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp + ((size_t)t0 * a.HV + h) * D, v_bytes);
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      rK[it] = IO<TI>::bload8(kr, oK[it]);
      rV[it] = IO<TI>::bload8(vr, oV[it]);
      if (WRITE_O) rQ[it] = IO<TI>::bload8(qr, oK[it]);
    }
    if (SEG == 2) {
#pragma unroll
      for (int it = 0; it < PPT; ++it) rV[it] = keep8(rV[it], !zero_v);
    }
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(akk + ((size_t)t0 * a.HV + h) * CH, (last * a.HV * CH + CH) * 2);
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(pm + ((size_t)c * a.HV + h) * CH * CH, CH * CH * 2);
#pragma unroll
    for (int it = 0; it < APT; ++it) {
      rA[it] = IO<bf16>::bload8(ar, oA[it]);
      if (WRITE_O) rP[it] = IO<bf16>::bload8(pr, oP[it]);
    }
    {
      // per-token scalars of row `lane`, staged by wave 0; the other waves load one row (the
      // loads stay unconditional, and touch one cache line instead of 64)
      const size_t rl = (size_t)(t0 + last), rv = w == 0 ? (size_t)(t0 + min(lane, last)) : rl;
      sg = a.gcum[(size_t)h * a.T + rv];
      sglast = a.gcum[(size_t)h * a.T + rl];
      sbeta = a.beta[rv * a.HV + h];
      srk = a.rk[(size_t)j * a.T + rv];
      if (WRITE_O) srq = a.rq[(size_t)j * a.T + rv];
    }
  };
  auto store_chunk = [&](int b, int c) {
    const int t0 = doc_t0 + (c - c_begin) * CH;
    const int len = min(CH, doc_t1 - t0);
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int p = tid + NT * it, row = p / RP, pc = p % RP;
      *reinterpret_cast<bf16x8*>(&sm.sK[b][row * SK + pc * 8]) = rK[it];
      *reinterpret_cast<bf16x8*>(&sm.sV[b][row * SK + pc * 8]) = rV[it];
      if (WRITE_O) *reinterpret_cast<bf16x8*>(&sm.sQ[b][row * SK + pc * 8]) = rQ[it];
    }
#pragma unroll
    for (int it = 0; it < APT; ++it) {
      const int p = tid + NT * it, row = p >> 3, pc = p & 7;
      lds_store_kp8(sm.sA[b], SA, row, pc, rA[it]);
      if (WRITE_O) lds_store_kp8(sm.sP[b], SA, row, pc, rP[it]);
    }
    if (w == 0) {
      const bool ok = lane < len;
      const float eb = __expf(sg);
      sm.sc[b][0][lane] = ok ? eb * srk : 0.f;
      sm.sc[b][1][lane] = ok ? sbeta : 0.f;
      sm.sc[b][2][lane] = ok ? __expf(sglast - sg) * srk : 0.f;
      if (WRITE_O) sm.sc[b][3][lane] = ok ? eb * srq : 0.f;
      if (lane == 0) sm.sgam[b] = __expf(sglast);
    }
  };

  // ---- state: rows 16 rt + 4 lg + i (key), column v0 + 16 ct + lr (value)
  f32x4 S[CT][NRT];
  const float* s_in = SEG ? sc.s_in : a.state_in;
  // segment walks: h0 only for a document's first segment (true walk from no slot)
  const bool use_h0 = a.has_h0 && (SEG == 0 || sc.kind == 0);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * rt + 4 * lg + i, v = v0 + 16 * ct + lr;
        if (SEG == 2 && sc.kind == 1) S[ct][rt][i] = d == v ? 1.f : 0.f;
        else if (SEG == 2 && sc.kind == 2) S[ct][rt][i] = 0.f;
        else
          S[ct][rt][i] = s_in ? s_in[((size_t)h * D + d) * D + v]
                         : use_h0 ? a.h0[(((size_t)n * a.HV + h) * D + d) * D + v]
                                  : 0.f;
      }

  auto step = [&](int b, int c) {
    const bf16* Kt = sm.sK[b];
    const bf16* Vt = sm.sV[b];
    const bf16* At = sm.sA[b];
    const bf16* Qt = sm.sQ[WRITE_O ? b : 0];
    const bf16* Pt = sm.sP[WRITE_O ? b : 0];
    const float* BKs = sm.sc[b][0];
    const float* Bs = sm.sc[b][1];
    const float* DKs = sm.sc[b][2];
    const float* BQs = sm.sc[b][3];
    const int t0 = doc_t0 + (c - c_begin) * CH;
    const int len = min(CH, doc_t1 - t0);
    const float gam = sm.sgam[b];

    // the state as operands in natural key order (k = key dim)
    bf16x8 sb[CT][KD];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) sb[ct][kd] = c_to_b(S[ct][2 * kd], S[ct][2 * kd + 1]);
    if (WRITE_TAPE) {
      // tape[v][k]: this lane's column, key rows 32 kd + 8 lg .. +7
      const __amdgpu_buffer_rsrc_t tr = make_rsrc(reinterpret_cast<bf16*>(a.htape) + ((size_t)c * a.HV + h) * D * D, D * D * 2);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int kd = 0; kd < KD; ++kd)
          buf_store16(sb[ct][kd], tr, ((v0 + 16 * ct + lr) * D + 8 * lg + 32 * kd) * 2);
    }
    // K S (64 tokens x 16 columns) and (Q S)^T (16 columns x 64 tokens) of every tile
    f32x4 ks[CT][4], qsT[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) ks[ct][mt] = qsT[ct][mt] = zero4();
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 kf = lds8(Kt, SK, 16 * mt + lr, 32 * kd + 8 * lg);
        bf16x8 qf;
        if (WRITE_O) qf = lds8(Qt, SK, 16 * mt + lr, 32 * kd + 8 * lg);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          ks[ct][mt] = mfma(kf, sb[ct][kd], ks[ct][mt]);
          if (WRITE_O) qsT[ct][mt] = mfma(sb[ct][kd], qf, qsT[ct][mt]);
        }
      }
    // X = diag(beta) (V - diag(b rk) K S)
    bf16x8 xb[CT][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 X[CT][2];
#pragma unroll
      for (int hm = 0; hm < 2; ++hm) {
        const int mt = 2 * kt + hm, r0 = 16 * mt + 4 * lg;
        const float4 bk4 = *reinterpret_cast<const float4*>(BKs + r0);
        const float4 be4 = *reinterpret_cast<const float4*>(Bs + r0);
        const float bk[4] = {bk4.x, bk4.y, bk4.z, bk4.w}, be[4] = {be4.x, be4.y, be4.z, be4.w};
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const bf16x4 vv = lds_tr4c(Vt, SK, 16 * mt, v0 + 16 * ct);
#pragma unroll
          for (int i = 0; i < 4; ++i) X[ct][hm][i] = be[i] * __builtin_fmaf(-bk[i], ks[ct][mt][i], (float)vv[i]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) xb[ct][kt] = pack_kp(X[ct][0], X[ct][1]);
    }
    // R = A X. The full saved set's v_new = R is formed a second time transposed, R^T = X^T A^T
    // (the same two fragments with their roles swapped), so that a lane holds 4 consecutive
    // values of one token's row: one 8-byte store, dropped past the chunk's end
    f32x4 R[CT][4];
    __amdgpu_buffer_rsrc_t vr;
    if (FULL)
      vr = make_rsrc(reinterpret_cast<bf16*>(a.vnew) + ((size_t)t0 * a.HV + h) * D, ((len - 1) * a.HV * D + D) * 2);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 RT[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) R[ct][mt] = RT[ct] = zero4();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 af = lds8(At, SA, 16 * mt + lr, 32 * kt + 8 * lg);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          R[ct][mt] = mfma(af, xb[ct][kt], R[ct][mt]);
          if (FULL) RT[ct] = mfma(xb[ct][kt], af, RT[ct]);
        }
      }
      if (FULL) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const float x4[4] = {RT[ct][0], RT[ct][1], RT[ct][2], RT[ct][3]};
          IO<bf16>::bstore4(vr, (16 * mt + lr) * a.HV * D + v0 + 16 * ct + 4 * lg, x4);
        }
      }
    }
    // operands of R (for (P R)^T) and of diag(exp(G_last - G) rk) R (for the state update)
    bf16x8 rb[CT][2], rdb[CT][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float4 dk4[2];
#pragma unroll
      for (int hm = 0; hm < 2; ++hm) dk4[hm] = *reinterpret_cast<const float4*>(DKs + 16 * (2 * kt + hm) + 4 * lg);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if (WRITE_O) rb[ct][kt] = pack_kp(R[ct][2 * kt], R[ct][2 * kt + 1]);
        f32x4 d[2];
#pragma unroll
        for (int hm = 0; hm < 2; ++hm) {
          d[hm][0] = dk4[hm].x * R[ct][2 * kt + hm][0];
          d[hm][1] = dk4[hm].y * R[ct][2 * kt + hm][1];
          d[hm][2] = dk4[hm].z * R[ct][2 * kt + hm][2];
          d[hm][3] = dk4[hm].w * R[ct][2 * kt + hm][3];
        }
        rdb[ct][kt] = pack_kp(d[0], d[1]);
      }
    }
    // O^T = diag-column(b rq) (Q S)^T + (P R)^T; lane holds O[t][v0 + 16 ct + 4 lg .. +3],
    // t = 16 mt + lr
    if (WRITE_O) {
      // rows of the chunk only: stores past the resource's end (tokens >= len) are dropped
      const __amdgpu_buffer_rsrc_t orr = make_rsrc((TI*)a.o + ((size_t)t0 * a.HV + h) * D,
                                                   ((len - 1) * a.HV * D + D) * (int)sizeof(TI));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] = zero4();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 pf = lds8(Pt, SA, 16 * mt + lr, 32 * kt + 8 * lg);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma(rb[ct][kt], pf, acc[ct]);
        }
        const int t = 16 * mt + lr;
        const float sq = BQs[t];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          float ov[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = __builtin_fmaf(sq, qsT[ct][mt][i], acc[ct][i]);
          IO<TI>::bstore4(orr, t * a.HV * D + v0 + 16 * ct + 4 * lg, ov);
        }
      }
    }
    // S <- gamma S + K^T diag(exp(G_last - G) rk) R
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x4 acc[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct] = S[ct][rt] * gam;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kT = lds_tr_kp(Kt, SK, 32 * kt, 16 * rt);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma(kT, rdb[ct][kt], acc[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) S[ct][rt] = acc[ct];
    }
  };

  if (c_begin < c_end) {
    load_chunk(c_begin);
    store_chunk(0, c_begin);
  }
  __syncthreads();
  for (int c = c_begin; c < c_end; ++c) {
    const int b = (c - c_begin) & 1;
    // the next chunk (the last one again at the end: staged into the idle buffer, never read);
    // unconditional, so the loads stay in flight across the whole step
    const int cn = min(c + 1, c_end - 1);
    load_chunk(cn);
    __builtin_amdgcn_sched_barrier(0); // keep every prefetch load ahead of the chunk's compute
    step(b, c);
    store_chunk(b ^ 1, cn);
    __syncthreads();
  }
  float* s_out = SEG ? sc.s_out : a.state_out;
  if (s_out) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_out[((size_t)h * D + 16 * rt + 4 * lg + i) * D + v0 + 16 * ct + lr] = S[ct][rt][i];
  }
  if (WRITE_O && a.want_ht && (SEG == 0 || sc.write_ht)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 16 * rt + 4 * lg + i;
          a.ht[(((size_t)n * a.HV + h) * D + d) * D + v0 + 16 * ct + lr] = S[ct][rt][i];
        }
  }
}

// ---------------------------------------------------------------------------------------
// Reverse walk, one workgroup per (document, value head), chunks in reverse. Writes the
// end-state gradient of every chunk (bf16, transposed) and dh0. Same organisation as the forward
// walk: D / 16 waves, wave w keeps columns [16 w, 16 w + 16) of dS and every per-chunk
// intermediate in registers, chaining MFMA results into operands by packing alone (k-permuted
// fragments, with P^T staged column-permuted to match); LDS holds the double-buffered chunk inputs (K, Q pre-scaled by exp(G) rq, dO, A,
// P^T and per-token factors), one barrier per chunk.
template <int D>
constexpr int bwalk_threads() {
  return 64 * (D / (16 * WALK_CT));
}

template <int D>
struct BWalkSmem {
  static constexpr int SK = D + 16;
  static constexpr int SA = CH + 16;
  bf16 sK[2][CH * SK];
  bf16 sQ[2][CH * SK];
  bf16 sdO[2][CH * SK];
  bf16 sA[2][CH * SA];
  bf16 sPT[2][CH * SA]; // columns k-permuted
  // per token: exp(G_last - G) rk, -beta exp(G) rk (zero past the chunk's end); gamma = exp(G_last)
  float sc[2][2][CH];
  float sgam[2];
};

template <int D, typename TI>
__device__ __forceinline__ void walk_bwd_body(const Args& a, int blk, BWalkSmem<D>& sm) {
  if (a.status[0]) return;
  const ChainMap cm = decode_chain(blk, a, 1);
  if (!cm.valid) return;
  const int n = __builtin_amdgcn_readfirstlane(a.seq_order[cm.rank]); // uniform (scalar registers)
  const int j = cm.j, h = j * a.G + cm.gi;
  const int c_begin = __builtin_amdgcn_readfirstlane(a.seq_c0[n]);
  const int c_end = __builtin_amdgcn_readfirstlane(a.seq_c0[n + 1]);
  constexpr int NT = bwalk_threads<D>();
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int NRT = D / 16, KD = D / 32, RP = D / 8;
  constexpr int PPT = CH * RP / NT, APT = CH * 8 / NT;
  using SM = BWalkSmem<D>;
  constexpr int SK = SM::SK, SA = SM::SA;
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;
  const TI* dop = (const TI*)a.dO;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  const bf16* pm = reinterpret_cast<const bf16*>(a.qk);
  constexpr int CT = WALK_CT;
  const int v0 = 16 * CT * w; // tile ct holds value columns v0 + 16 ct ..
  const int doc_t0 = __builtin_amdgcn_readfirstlane(a.cu[n]), doc_t1 = __builtin_amdgcn_readfirstlane(a.cu[n + 1]);

  // staging through buffer resources bounded at the chunk's last row, at per-lane offsets fixed
  // for the whole walk (rows past the chunk's end read as zeros; the row factors and the q scale
  // are zero there and P^T is masked, so they contribute nothing)
  int oK[PPT], oV[PPT], oR[PPT], oA[APT], oP[APT]; // element offsets of this thread's pieces
#pragma unroll
  for (int it = 0; it < PPT; ++it) {
    const int p = tid + NT * it, row = p / RP, pc = p % RP;
    oK[it] = row * a.H * D + pc * 8;
    oV[it] = row * a.HV * D + pc * 8;
    oR[it] = row;
  }
#pragma unroll
  for (int it = 0; it < APT; ++it) {
    const int p = tid + NT * it, row = p >> 3, pc = p & 7;
    oA[it] = row * a.HV * CH + pc * 8;
    oP[it] = row * CH + pc * 8;
  }
  bf16x8 rK[PPT], rQ[PPT], rD[PPT], rA[APT], rP[APT];
  float rgq[PPT], rrq[PPT];
  float sg = 0.f, sglast = 0.f, sbeta = 0.f, srk = 0.f;
  auto load_chunk = [&](int c) {
    const int t0 = doc_t0 + (c - c_begin) * CH;
    const int last = min(CH, doc_t1 - t0) - 1;
    const int kq_bytes = (last * a.H * D + D) * (int)sizeof(TI), v_bytes = (last * a.HV * D + D) * (int)sizeof(TI);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp + ((size_t)t0 * a.H + j) * D, kq_bytes);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qp + ((size_t)t0 * a.H + j) * D, kq_bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dop + ((size_t)t0 * a.HV + h) * D, v_bytes);
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.gcum + (size_t)h * a.T + t0, (last + 1) * 4);
    const __amdgpu_buffer_rsrc_t rqr = make_rsrc(a.rq + (size_t)j * a.T + t0, (last + 1) * 4);
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      rK[it] = IO<TI>::bload8(kr, oK[it]);
      rQ[it] = IO<TI>::bload8(qr, oK[it]);
      rD[it] = IO<TI>::bload8(dr, oV[it]);
      // Q rows are staged scaled by exp(G) rq (zero past the end; formed in store_chunk, so no
      // load result is used before the chunk's compute)
      rgq[it] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gr, oR[it] * 4, 0, 0));
      rrq[it] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rqr, oR[it] * 4, 0, 0));
    }
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(akk + ((size_t)t0 * a.HV + h) * CH, (last * a.HV * CH + CH) * 2);
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(pm + ((size_t)c * a.HV + h) * CH * CH, CH * CH * 2);
#pragma unroll
    for (int it = 0; it < APT; ++it) {
      rA[it] = IO<bf16>::bload8(ar, oA[it]);
      rP[it] = IO<bf16>::bload8(pr, oP[it]);
    }
    {
      // per-token scalars of row `lane`, staged by wave 0; the other waves load one row (the
      // loads stay unconditional, and touch one cache line instead of 64)
      const size_t rl = (size_t)(t0 + last), rv = w == 0 ? (size_t)(t0 + min(lane, last)) : rl;
      sg = a.gcum[(size_t)h * a.T + rv];
      sglast = a.gcum[(size_t)h * a.T + rl];
      sbeta = a.beta[rv * a.HV + h];
      srk = a.rk[(size_t)j * a.T + rv];
    }
  };
  auto store_chunk = [&](int b, int c) {
    const int t0 = doc_t0 + (c - c_begin) * CH;
    const int len = min(CH, doc_t1 - t0);
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int p = tid + NT * it, row = p / RP, pc = p % RP;
      *reinterpret_cast<bf16x8*>(&sm.sK[b][row * SK + pc * 8]) = rK[it];
      *reinterpret_cast<bf16x8*>(&sm.sQ[b][row * SK + pc * 8]) = scale8(rQ[it], row < len ? __expf(rgq[it]) * rrq[it] : 0.f);
      *reinterpret_cast<bf16x8*>(&sm.sdO[b][row * SK + pc * 8]) = rD[it];
    }
#pragma unroll
    for (int it = 0; it < APT; ++it) {
      const int p = tid + NT * it, row = p >> 3, pc = p & 7;
      *reinterpret_cast<bf16x8*>(&sm.sA[b][row * SA + pc * 8]) = rA[it];
      lds_store_kp8(sm.sPT[b], SA, row, pc, rP[it]);
    }
    if (w == 0) {
      const bool ok = lane < len;
      sm.sc[b][0][lane] = ok ? __expf(sglast - sg) * srk : 0.f;
      sm.sc[b][1][lane] = ok ? -sbeta * __expf(sg) * srk : 0.f;
      if (lane == 0) sm.sgam[b] = __expf(sglast);
    }
  };

  f32x4 dS[CT][NRT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * rt + 4 * lg + i;
        dS[ct][rt][i] = a.dht ? a.dht[(((size_t)n * a.HV + h) * D + d) * D + v0 + 16 * ct + lr] : 0.f;
      }

  auto step = [&](int b, int c) {
    const bf16* Kt = sm.sK[b];
    const bf16* Qt = sm.sQ[b];
    const bf16* Dt = sm.sdO[b];
    const bf16* At = sm.sA[b];
    const bf16* PTt = sm.sPT[b];
    const float* DKs = sm.sc[b][0];
    const float* YKs = sm.sc[b][1];
    const float gam = sm.sgam[b];

    bf16x8 sb[CT][KD];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) sb[ct][kd] = c_to_b(dS[ct][2 * kd], dS[ct][2 * kd + 1]);
    {
      // tape[v][k]: this lane's column, key rows 32 kd + 8 lg .. +7
      const __amdgpu_buffer_rsrc_t tr = make_rsrc(reinterpret_cast<bf16*>(a.dstape) + ((size_t)c * a.HV + h) * D * D, D * D * 2);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int kd = 0; kd < KD; ++kd)
          buf_store16(sb[ct][kd], tr, ((v0 + 16 * ct + lr) * D + 8 * lg + 32 * kd) * 2);
    }
    // dO as operands (k = tokens), shared by P^T dO and (Q')^T dO
    bf16x8 db[CT][2];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) db[ct][kt] = lds_tr_kp(Dt, SK, 32 * kt, v0 + 16 * ct);
    // dR = P^T dO + diag(exp(G_last - G) rk) K dS
    bf16x8 drb[CT][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 dR[CT][2];
#pragma unroll
      for (int hm = 0; hm < 2; ++hm) {
        const int mt = 2 * kt + hm;
        f32x4 kd_[CT], pd[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) kd_[ct] = pd[ct] = zero4();
#pragma unroll
        for (int kd = 0; kd < KD; ++kd) {
          const bf16x8 kf = lds8(Kt, SK, 16 * mt + lr, 32 * kd + 8 * lg);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) kd_[ct] = mfma(kf, sb[ct][kd], kd_[ct]);
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const bf16x8 pf = lds8(PTt, SA, 16 * mt + lr, 32 * k2 + 8 * lg);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) pd[ct] = mfma(pf, db[ct][k2], pd[ct]);
        }
        const float4 dk4 = *reinterpret_cast<const float4*>(DKs + 16 * mt + 4 * lg);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          dR[ct][hm][0] = __builtin_fmaf(dk4.x, kd_[ct][0], pd[ct][0]);
          dR[ct][hm][1] = __builtin_fmaf(dk4.y, kd_[ct][1], pd[ct][1]);
          dR[ct][hm][2] = __builtin_fmaf(dk4.z, kd_[ct][2], pd[ct][2]);
          dR[ct][hm][3] = __builtin_fmaf(dk4.w, kd_[ct][3], pd[ct][3]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) drb[ct][kt] = pack_kp(dR[ct][0], dR[ct][1]);
    }
    // -Y' = -diag(beta b rk) A^T dR
    bf16x8 yb[CT][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 Y[CT][2];
#pragma unroll
      for (int hm = 0; hm < 2; ++hm) {
        const int mt = 2 * kt + hm;
        f32x4 acc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const bf16x8 aT = lds_tr_kp(At, SA, 32 * k2, 16 * mt);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) acc[ct] = mfma(aT, drb[ct][k2], acc[ct]);
        }
        const float4 y4 = *reinterpret_cast<const float4*>(YKs + 16 * mt + 4 * lg);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          Y[ct][hm][0] = y4.x * acc[ct][0];
          Y[ct][hm][1] = y4.y * acc[ct][1];
          Y[ct][hm][2] = y4.z * acc[ct][2];
          Y[ct][hm][3] = y4.w * acc[ct][3];
        }
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) yb[ct][kt] = pack_kp(Y[ct][0], Y[ct][1]);
    }
    // dS <- gamma dS + (Q')^T dO - K^T Y'
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x4 acc[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct] = dS[ct][rt] * gam;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 qT = lds_tr_kp(Qt, SK, 32 * kt, 16 * rt);
        const bf16x8 kT = lds_tr_kp(Kt, SK, 32 * kt, 16 * rt);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          acc[ct] = mfma(qT, db[ct][kt], acc[ct]);
          acc[ct] = mfma(kT, yb[ct][kt], acc[ct]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) dS[ct][rt] = acc[ct];
    }
  };

  if (c_begin < c_end) {
    load_chunk(c_end - 1);
    store_chunk(0, c_end - 1);
  }
  __syncthreads();
  for (int c = c_end - 1; c >= c_begin; --c) {
    const int b = (c_end - 1 - c) & 1;
    // the next chunk in reverse (the first one again at the end, staged into the idle buffer)
    const int cn = max(c - 1, c_begin);
    load_chunk(cn);
    __builtin_amdgcn_sched_barrier(0); // keep every prefetch load ahead of the chunk's compute
    step(b, c);
    store_chunk(b ^ 1, cn);
    __syncthreads();
  }
  if (a.dh0) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 16 * rt + 4 * lg + i;
          a.dh0[(((size_t)n * a.HV + h) * D + d) * D + v0 + 16 * ct + lr] = dS[ct][rt][i];
        }
  }
}

} // namespace gdn
