// Forward kernels of the chunked gated delta rule on gfx950.
//
// The chunked form (64-token chunks per document; the chunk factors gamma, gcum, Akk and the
// h tape / v_new / w / u / Aqk rows of the README saved-set table quoted in flashinfer
// PR #8542) with start state S, per value head:
//   G_i = sum_{s<=i} g_s, b_i = exp(G_i), gamma = b_last
//   L_ij = beta_i exp(G_i - G_j) kh_i.kh_j (i > j), A = (I + L)^-1               [k_intra]
//   X = diag(beta) (V - diag(b) Kh S),  R = A X  (= U - W S)                         [k_walk_fwd]
//   O = diag(b) Qh S + P R,  P_ij = exp(G_i - G_j) qh_i.kh_j (i >= j)
//   S <- gamma S + Kh^T diag(exp(G_last - G)) R
// k_intra runs one workgroup per (chunk, q/k head) and is fully parallel; k_walk_fwd runs one
// workgroup per (document, value head, value-column tile) and walks that document's chunks in
// order, keeping its FP32 state tile in registers. Every contraction is a bf16 MFMA with FP32
// accumulation; the state is rounded to bf16 only as an MFMA operand.
#include "gdn_device.h"

namespace gdn {

// ---------------------------------------------------------------------------------------
// Chunk tables from the device copy of cu_seqlens (one workgroup of 1024 threads).
__global__ __launch_bounds__(1024) void k_tables(const int32_t* __restrict__ cu, int N, int NT, int64_t T,
                                                 int* __restrict__ seq_c0, int* __restrict__ c_t0,
                                                 int* __restrict__ c_len, int* __restrict__ seq_order,
                                                 int* __restrict__ status) {
  __shared__ int s_scan[1024];
  __shared__ int s_carry, s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_carry = 0;
    s_bad = 0;
  }
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    int cnt = 0;
    if (n < N) {
      const int lo = cu[n], hi = cu[n + 1];
      if (hi < lo || lo < 0 || (int64_t)hi > T) s_bad = 1;
      else cnt = (hi - lo + CH - 1) / CH;
    }
    s_scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int x = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += x;
      __syncthreads();
    }
    if (n < N) seq_c0[n] = s_carry + s_scan[tid] - cnt;
    __syncthreads();
    if (tid == 1023) s_carry += s_scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    if (cu[0] != 0 || (int64_t)cu[N] != T || s_carry != NT) s_bad = 1;
    seq_c0[N] = s_carry;
    status[0] = s_bad;
  }
  __syncthreads();
  const int bad = s_bad;
  for (int c = tid; c < NT; c += 1024) {
    if (bad) {
      c_len[c] = 0;
      c_t0[c] = 0;
      continue;
    }
    int lo = 0, hi = N; // seq_c0[lo] <= c < seq_c0[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seq_c0[mid] <= c) lo = mid;
      else hi = mid;
    }
    const int t0 = cu[lo] + (c - seq_c0[lo]) * CH;
    c_t0[c] = t0;
    c_len[c] = min(CH, cu[lo + 1] - t0);
  }
  // documents, longest first (ties: lower index first); identity order for very many documents
  for (int n = tid; n < N; n += 1024) {
    if (bad || N > 8192) {
      seq_order[n] = n;
      continue;
    }
    const int Ln = cu[n + 1] - cu[n];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const int Lm = cu[m + 1] - cu[m];
      rank += (Lm > Ln) || (Lm == Ln && m < n);
    }
    seq_order[rank] = n;
  }
}

// ---------------------------------------------------------------------------------------
// Per (chunk, q/k head): inverse norms rk, rq; normalised q.k (bf16, workspace; row-major for the
// forward, transposed for the backward); and, unless BWD, per value head of the group: gcum,
// gamma and Akk = (I + L)^-1 (saved).
//
// K K^T and the q.k products run on MFMA; each wave keeps 16 rows of K K^T in registers. The
// inverse runs one value head per wave: every lane owns one column c of A and forward-substitutes
// it, x_i = -sum_{m<i} L_im x_m (x_c = 1), reading rows of L from LDS as broadcasts.
template <int D, typename TI, bool BWD>
__global__ __launch_bounds__(NTHREADS) void k_intra(Args a) {
  if (a.status[0]) return;
  const int c = blockIdx.x, j = blockIdx.y;
  const int len = a.c_len[c];
  if (len <= 0) return;
  const int t0 = a.c_t0[c];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int SK = D + PAD;
  constexpr int SL = CH + 4; // fp32 row stride of L: 16-byte aligned rows
  constexpr int KS = D / 32;
  constexpr int NB = 4;      // value heads per batch, one wave each
  struct KQ {
    bf16 k[CH * SK];
    bf16 q[CH * SK];
  };
  union Smem {
    KQ kq;
    float L[NB][CH][SL];
  };
  __shared__ __attribute__((aligned(16))) Smem u;
  __shared__ float srk[CH], srq[CH];
  __shared__ float sG[NB][CH], sB[NB][CH];
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;

  // this wave's 16 rows of K and Q (MFMA A fragments), their squared norms
  const int ar = 16 * w + lr;
  const bool ok = ar < len;
  bf16x8 fk[KS], fq[KS];
  float ssk = 0.f, ssq = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float kf[8], qf[8];
    if (ok) {
      IO<TI>::load8f(kp + ((size_t)(t0 + ar) * a.H + j) * D + ks * 32 + lg * 8, kf);
      IO<TI>::load8f(qp + ((size_t)(t0 + ar) * a.H + j) * D + ks * 32 + lg * 8, qf);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = qf[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ssk += kf[e] * kf[e];
      ssq += qf[e] * qf[e];
      fk[ks][e] = (bf16)kf[e];
      fq[ks][e] = (bf16)qf[e];
    }
    *reinterpret_cast<bf16x8*>(u.kq.k + ar * SK + ks * 32 + lg * 8) = fk[ks];
    *reinterpret_cast<bf16x8*>(u.kq.q + ar * SK + ks * 32 + lg * 8) = fq[ks];
  }
  ssk += __shfl_xor(ssk, 16);
  ssk += __shfl_xor(ssk, 32);
  ssq += __shfl_xor(ssq, 16);
  ssq += __shfl_xor(ssq, 32);
  if (lg == 0) {
    const float rkv = a.l2norm ? 1.f / sqrtf(ssk + 1e-6f) : 1.f;
    const float rqv = a.l2norm ? 1.f / sqrtf(ssq + 1e-6f) : 1.f;
    srk[ar] = ok ? rkv : 0.f;
    srq[ar] = ok ? rqv : 0.f;
    if (ok) {
      a.rk[(size_t)(t0 + ar) * a.H + j] = rkv;
      a.rq[(size_t)(t0 + ar) * a.H + j] = rqv;
    }
  }
  __syncthreads();

  // K K^T (rows k, cols k) and, for the q.k tile, Q K^T (backward: rows q) or K Q^T (forward:
  // rows k), so that the stored layout is written 4 contiguous elements per lane.
  f32x4 kk[4], qk[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) kk[ct] = qk[ct] = zero4();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 bk = lds8(u.kq.k, SK, 16 * ct + lr, ks * 32 + lg * 8);
      kk[ct] = mfma(fk[ks], bk, kk[ct]);
      if (BWD) qk[ct] = mfma(fq[ks], bk, qk[ct]);
      else qk[ct] = mfma(fk[ks], lds8(u.kq.q, SK, 16 * ct + lr, ks * 32 + lg * 8), qk[ct]);
    }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
      kk[ct][i] *= srk[r] * srk[cc];
      // backward: C[q = r][k = cc]; forward: C[k = r][q = cc]
      qk[ct][i] *= BWD ? srq[r] * srk[cc] : srk[r] * srq[cc];
    }

  bf16* aout = reinterpret_cast<bf16*>(a.akk);
  for (int hb = 0; hb < a.G; hb += NB) {
    const int nb = min(NB, a.G - hb);
    if (w < nb) {
      const int h = j * a.G + hb + w, r = lane;
      float x;
      if (BWD) {
        x = r < len ? a.gcum[(size_t)(t0 + r) * a.HV + h] : 0.f;
      } else {
        const float gv = r < len ? a.g[(size_t)(t0 + r) * a.HV + h] : 0.f;
        const float bv = r < len ? a.beta[(size_t)(t0 + r) * a.HV + h] : 0.f;
        x = gv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        sB[w][r] = bv;
        if (r < len) a.gcum[(size_t)(t0 + r) * a.HV + h] = x;
        if (r == len - 1) a.gamma[(size_t)c * a.HV + h] = __expf(x);
      }
      sG[w][r] = x;
    }
    __syncthreads();
    // P_qk = exp(G_q - G_k) qh.kh for q >= k, per value head: the forward stores P[q][k], the
    // backward P^T[k][q]; both are [cc][r..r+3] of this wave's tile
    for (int b = 0; b < nb; ++b) {
      const int h = j * a.G + hb + b;
      bf16* pout = reinterpret_cast<bf16*>(a.qk) + ((size_t)c * a.HV + h) * CH * CH;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int cc = 16 * ct + lr;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i;
          const int qi = BWD ? r : cc, ki = BWD ? cc : r;
          const float e = __expf(fminf(sG[b][qi] - sG[b][ki], 0.f));
          v[i] = qi >= ki ? e * qk[ct][i] : 0.f;
        }
        lds_store4_t(pout, CH, cc, 16 * w + lg * 4, v[0], v[1], v[2], v[3]);
      }
    }
    if (BWD) {
      __syncthreads();
      continue;
    }
    for (int b = 0; b < nb; ++b)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
          u.L[b][r][cc] = r > cc ? sB[b][r] * __expf(sG[b][r] - sG[b][cc]) * kk[ct][i] : 0.f;
        }
    __syncthreads();
    if (w < nb) {
      const int h = j * a.G + hb + w, col = lane;
      float x[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
        for (int m = 0; m + 4 <= i; m += 4) {
          const float4 l4 = *reinterpret_cast<const float4*>(&u.L[w][i][m]);
          s0 = __builtin_fmaf(l4.x, x[m], s0);
          s1 = __builtin_fmaf(l4.y, x[m + 1], s1);
          s2 = __builtin_fmaf(l4.z, x[m + 2], s2);
          s3 = __builtin_fmaf(l4.w, x[m + 3], s3);
        }
#pragma unroll
        for (int m = (i / 4) * 4; m < i; ++m) s0 = __builtin_fmaf(u.L[w][i][m], x[m], s0);
        x[i] = i < col ? 0.f : (i == col ? 1.f : -((s0 + s1) + (s2 + s3)));
      }
      // stage the inverse (bf16) in this wave's own L area, row-major
      bf16* stage = reinterpret_cast<bf16*>(&u.L[w][0][0]);
#pragma unroll
      for (int i = 0; i < CH; ++i) stage[i * (CH + PAD) + col] = (bf16)x[i];
    }
    __syncthreads();
    if (w < nb) {
      const int h = j * a.G + hb + w;
      const bf16* stage = reinterpret_cast<const bf16*>(&u.L[w][0][0]);
#pragma unroll
      for (int it = 0; it < CH / 8; ++it) {
        const int r = it * 8 + (lane >> 3), pc = lane & 7;
        if (r < len)
          *reinterpret_cast<bf16x8*>(aout + ((size_t)(t0 + r) * a.HV + h) * CH + pc * 8) =
              lds8(stage, CH + PAD, r, pc * 8);
      }
    }
    __syncthreads();
  }
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
template <int D>
constexpr int walk_threads() {
  return 64 * (D / 16);
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

template <int D, typename TI, bool WRITE_O, bool WRITE_TAPE, bool FULL>
__global__ __launch_bounds__(walk_threads<D>(), 1) void k_walk_fwd(Args a) {
  if (a.status[0]) return;
  const ChainMap cm = decode_chain(blockIdx.x, a.N, a.H, a.G, 1);
  if (!cm.valid) return;
  const int n = a.seq_order[cm.rank];
  const int j = cm.j, h = j * a.G + cm.gi;
  const int c_begin = a.seq_c0[n], c_end = a.seq_c0[n + 1];
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
  __shared__ __attribute__((aligned(16))) SM sm;
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;
  const TI* vp = (const TI*)a.v;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  const bf16* pm = reinterpret_cast<const bf16*>(a.qk);
  const int v0 = 16 * w;
  // chunk c of the document starts at token cu[n] + 64 (c - c_begin)
  const int doc_t0 = a.cu[n], doc_t1 = a.cu[n + 1];

  // ---- staging: global -> registers (issued before a chunk's compute) -> LDS (after it).
  // Rows past the chunk's end re-read its last row: finite values whose contributions vanish
  // because beta and the row factors are zero there and P is masked.
  bf16x8 rK[PPT], rV[PPT], rQ[PPT], rA[APT], rP[APT];
  float sg = 0.f, sglast = 0.f, sbeta = 0.f, srk = 0.f, srq = 0.f;
  auto load_chunk = [&](int c) {
    const int t0 = doc_t0 + (c - c_begin) * CH;
    const int last = min(CH, doc_t1 - t0) - 1;
    const TI* kc = kp + ((size_t)t0 * a.H + j) * D;
    const TI* qc = qp + ((size_t)t0 * a.H + j) * D;
    const TI* vc = vp + ((size_t)t0 * a.HV + h) * D;
#pragma unroll
    for (int it = 0; it < PPT; ++it) {
      const int p = tid + NT * it, row = min(p / RP, last), pc = p % RP;
      rK[it] = IO<TI>::load8(kc + row * a.H * D + pc * 8);
      rV[it] = IO<TI>::load8(vc + row * a.HV * D + pc * 8);
      if (WRITE_O) rQ[it] = IO<TI>::load8(qc + row * a.H * D + pc * 8);
    }
    const bf16* ac = akk + ((size_t)t0 * a.HV + h) * CH;
    const bf16* pc_ = pm + ((size_t)c * a.HV + h) * CH * CH;
#pragma unroll
    for (int it = 0; it < APT; ++it) {
      const int p = tid + NT * it, row = p >> 3, pc = p & 7;
      rA[it] = *reinterpret_cast<const bf16x8*>(ac + min(row, last) * a.HV * CH + pc * 8);
      if (WRITE_O) rP[it] = *reinterpret_cast<const bf16x8*>(pc_ + row * CH + pc * 8);
    }
    {
      // per-token scalars of row `lane` (every wave loads them; wave 0 stages them)
      const size_t rv = (size_t)(t0 + min(lane, last)), rl = (size_t)(t0 + last);
      sg = a.gcum[rv * a.HV + h];
      sglast = a.gcum[rl * a.HV + h];
      sbeta = a.beta[rv * a.HV + h];
      srk = a.rk[rv * a.H + j];
      if (WRITE_O) srq = a.rq[rv * a.H + j];
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

  // ---- state: rows 16 rt + 4 lg + i (key), column v0 + lr (value)
  f32x4 S[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * rt + 4 * lg + i;
      S[rt][i] = a.has_h0 ? a.h0[(((size_t)n * a.HV + h) * D + d) * D + v0 + lr] : 0.f;
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
    bf16x8 sb[KD];
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) sb[kd] = c_to_b(S[2 * kd], S[2 * kd + 1]);
    if (WRITE_TAPE) {
      // tape[v][k]: this lane's column, key rows 32 kd + 8 lg .. +7
      bf16* tp = reinterpret_cast<bf16*>(a.htape) + ((size_t)c * a.HV + h) * D * D + (size_t)(v0 + lr) * D + 8 * lg;
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) *reinterpret_cast<bf16x8*>(tp + 32 * kd) = sb[kd];
    }
    // K S (64 tokens x 16 columns) and (Q S)^T (16 columns x 64 tokens)
    f32x4 ks[4], qsT[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ks[mt] = qsT[mt] = zero4();
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        ks[mt] = mfma(lds8(Kt, SK, 16 * mt + lr, 32 * kd + 8 * lg), sb[kd], ks[mt]);
        if (WRITE_O) qsT[mt] = mfma(sb[kd], lds8(Qt, SK, 16 * mt + lr, 32 * kd + 8 * lg), qsT[mt]);
      }
    // X = diag(beta) (V - diag(b rk) K S)
    bf16x8 xb[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 X[2];
#pragma unroll
      for (int hm = 0; hm < 2; ++hm) {
        const int mt = 2 * kt + hm, r0 = 16 * mt + 4 * lg;
        const float4 bk4 = *reinterpret_cast<const float4*>(BKs + r0);
        const float4 be4 = *reinterpret_cast<const float4*>(Bs + r0);
        const float bk[4] = {bk4.x, bk4.y, bk4.z, bk4.w}, be[4] = {be4.x, be4.y, be4.z, be4.w};
        const bf16x4 vv = lds_tr4c(Vt, SK, 16 * mt, v0);
#pragma unroll
        for (int i = 0; i < 4; ++i) X[hm][i] = be[i] * __builtin_fmaf(-bk[i], ks[mt][i], (float)vv[i]);
      }
      xb[kt] = pack_kp(X[0], X[1]);
    }
    // R = A X
    f32x4 R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      R[mt] = zero4();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) R[mt] = mfma(lds8(At, SA, 16 * mt + lr, 32 * kt + 8 * lg), xb[kt], R[mt]);
    }
    if (FULL) {
      // rows past the chunk's end go to the discard area (no branch around the stores)
      bf16* vn = reinterpret_cast<bf16*>(a.vnew) + ((size_t)t0 * a.HV + h) * D + v0 + lr;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * lg + i;
          bf16* dst = r < len ? vn + (size_t)r * a.HV * D : reinterpret_cast<bf16*>(a.discard) + lane;
          *dst = (bf16)R[mt][i];
        }
    }
    // operands of R (for (P R)^T) and of diag(exp(G_last - G) rk) R (for the state update)
    bf16x8 rb[2], rdb[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (WRITE_O) rb[kt] = pack_kp(R[2 * kt], R[2 * kt + 1]);
      f32x4 d[2];
#pragma unroll
      for (int hm = 0; hm < 2; ++hm) {
        const float4 dk4 = *reinterpret_cast<const float4*>(DKs + 16 * (2 * kt + hm) + 4 * lg);
        d[hm][0] = dk4.x * R[2 * kt + hm][0];
        d[hm][1] = dk4.y * R[2 * kt + hm][1];
        d[hm][2] = dk4.z * R[2 * kt + hm][2];
        d[hm][3] = dk4.w * R[2 * kt + hm][3];
      }
      rdb[kt] = pack_kp(d[0], d[1]);
    }
    // O^T = diag-column(b rq) (Q S)^T + (P R)^T; lane holds O[t][v0 + 4 lg .. +3], t = 16 mt + lr
    if (WRITE_O) {
      TI* op = (TI*)a.o + ((size_t)t0 * a.HV + h) * D + v0 + 4 * lg;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) acc = mfma(rb[kt], lds8(Pt, SA, 16 * mt + lr, 32 * kt + 8 * lg), acc);
        const int t = 16 * mt + lr;
        const float sq = BQs[t];
        float ov[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = __builtin_fmaf(sq, qsT[mt][i], acc[i]);
        // tokens past the chunk's end go to the discard area: every lane stores, so no branch
        // hides the number of outstanding stores from the wait counts
        IO<TI>::store4(t < len ? op + (size_t)t * a.HV * D : reinterpret_cast<TI*>(a.discard) + 4 * lane, ov);
      }
    }
    // S <- gamma S + K^T diag(exp(G_last - G) rk) R
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x4 acc = S[rt] * gam;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc = mfma(lds_tr_kp(Kt, SK, 32 * kt, 16 * rt), rdb[kt], acc);
      S[rt] = acc;
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
  if (WRITE_O && a.want_ht) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * rt + 4 * lg + i;
        a.ht[(((size_t)n * a.HV + h) * D + d) * D + v0 + lr] = S[rt][i];
      }
  }
}

// ---------------------------------------------------------------------------------------
// launchers

static inline hipStream_t S_(void* s) { return reinterpret_cast<hipStream_t>(s); }

int launch_tables(const Args& a, void* stream) {
  hipLaunchKernelGGL(k_tables, dim3(1), dim3(1024), 0, S_(stream), a.cu, a.N, a.NT, a.T, a.seq_c0, a.c_t0,
                     a.c_len, a.seq_order, a.status);
  return (int)hipGetLastError();
}

template <int D, typename TI>
static int intra_t(const Args& a, int bwd, hipStream_t s) {
  if (a.NT == 0) return 0;
  const dim3 grid(a.NT, a.H);
  if (bwd) hipLaunchKernelGGL((k_intra<D, TI, true>), grid, dim3(NTHREADS), 0, s, a);
  else hipLaunchKernelGGL((k_intra<D, TI, false>), grid, dim3(NTHREADS), 0, s, a);
  return (int)hipGetLastError();
}

int launch_intra(const Args& a, int bwd_prep, void* stream) {
  const hipStream_t s = S_(stream);
  if (a.D == 128) return a.dtype == 0 ? intra_t<128, bf16>(a, bwd_prep, s) : intra_t<128, float>(a, bwd_prep, s);
  return a.dtype == 0 ? intra_t<64, bf16>(a, bwd_prep, s) : intra_t<64, float>(a, bwd_prep, s);
}

// Number of workgroups of a chain launch: (document, q/k head) groups padded to a multiple of 8
// (one per XCD), times the G value heads and the value tiles of each group.
int chain_blocks(const Args& a, int ntile) { return ((a.N * a.H + 7) / 8) * 8 * a.G * ntile; }

template <int D, typename TI>
static int walk_t(const Args& a, int write_o, int write_tape, hipStream_t s) {
  const dim3 grid(chain_blocks(a, 1)), blk(walk_threads<D>());
  if (write_o && !write_tape) hipLaunchKernelGGL((k_walk_fwd<D, TI, true, false, false>), grid, blk, 0, s, a);
  else if (write_o) hipLaunchKernelGGL((k_walk_fwd<D, TI, true, true, true>), grid, blk, 0, s, a);
  else if (a.full) hipLaunchKernelGGL((k_walk_fwd<D, TI, false, true, true>), grid, blk, 0, s, a);
  else hipLaunchKernelGGL((k_walk_fwd<D, TI, false, true, false>), grid, blk, 0, s, a);
  return (int)hipGetLastError();
}

int launch_walk_fwd(const Args& a, int write_o, int write_tape, void* stream) {
  const hipStream_t s = S_(stream);
  if (a.D == 128)
    return a.dtype == 0 ? walk_t<128, bf16>(a, write_o, write_tape, s) : walk_t<128, float>(a, write_o, write_tape, s);
  return a.dtype == 0 ? walk_t<64, bf16>(a, write_o, write_tape, s) : walk_t<64, float>(a, write_o, write_tape, s);
}

} // namespace gdn
