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
// State walk, one workgroup per (document, value head, value tile of DVT columns).
// WRITE_O: write o (and ht). WRITE_TAPE: write the chunk-start state tape (bf16, transposed).
// FULL: also write v_new = R.
//
// The next chunk's inputs are loaded into registers while the current chunk computes, so the
// serial chain per chunk is LDS + MFMA only. K is staged row-major in LDS; its transpose for the
// state update comes from transpose-reads.
template <int D, int DVT>
struct WalkSmem {
  static constexpr int SK = D + 16;   // row stride of K (conflict-free transpose-reads)
  static constexpr int SST = D + PAD; // row stride of S^T
  static constexpr int STK = CH + PAD;
  static constexpr int SV = DVT + PAD;
  bf16 sK[CH * SK];
  bf16 sST[DVT * SST];
  bf16 sXT[DVT * STK];
  bf16 sRT[DVT * STK];
  bf16 sRdT[DVT * STK];
  bf16 sV[CH * SV];
  float sG[CH], sB[CH], srk[CH], srq[CH];
};

// Inputs of one chunk, loaded into registers one chunk ahead of use.
template <int KS>
struct WalkPrefetch {
  bf16x8 k[KS], q[KS], a[2], p[2], v;
  float g, b, rk, rq, gam;
  int len, t0;
};

template <int D, int DVT, typename TI, bool WRITE_O, bool WRITE_TAPE, bool FULL>
__global__ __launch_bounds__(NTHREADS) void k_walk_fwd(Args a) {
  if (a.status[0]) return;
  constexpr int NTILE = D / DVT;
  const ChainMap cm = decode_chain(blockIdx.x, a.N, a.H, a.G, NTILE);
  if (!cm.valid) return;
  const int n = a.seq_order[cm.rank];
  const int j = cm.j, h = j * a.G + cm.gi, col0 = cm.tile * DVT;
  const int c_begin = a.seq_c0[n], c_end = a.seq_c0[n + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int NCT = DVT / 16; // value-column tiles
  constexpr int NRT = D / 64;   // state row tiles per wave
  constexpr int KS = D / 32;    // k-steps over the key dim
  using SM = WalkSmem<D, DVT>;
  constexpr int SK = SM::SK, SST = SM::SST, STK = SM::STK, SV = SM::SV;
  constexpr int VPR = DVT / 8; // 16-byte pieces per row of the value tile
  __shared__ __attribute__((aligned(16))) SM sm;
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;
  const TI* vp = (const TI*)a.v;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  const bf16* qkp = reinterpret_cast<const bf16*>(a.qk);
  const int ar = 16 * w + lr; // this lane's A-fragment row (token in the chunk)
  // chunk c of the document starts at token cu[n] + 64 (c - c_begin): no table lookup on the
  // serial path
  const int doc_t0 = a.cu[n], doc_t1 = a.cu[n + 1];
  using PF = WalkPrefetch<KS>;

  // Unconditional loads from rows clamped into the chunk; rows past its end are zeroed when the
  // data is consumed, so nothing waits on a load before its use one chunk later.
  auto prefetch = [&](PF& P, int c) {
    P.t0 = doc_t0 + (c - c_begin) * CH;
    P.len = min(CH, doc_t1 - P.t0);
    const int rr = min(ar, P.len - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      P.k[ks] = IO<TI>::load8(kp + ((size_t)(P.t0 + rr) * a.H + j) * D + ks * 32 + lg * 8);
      if (WRITE_O) P.q[ks] = IO<TI>::load8(qp + ((size_t)(P.t0 + rr) * a.H + j) * D + ks * 32 + lg * 8);
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      P.a[k2] = *reinterpret_cast<const bf16x8*>(akk + ((size_t)(P.t0 + rr) * a.HV + h) * CH + k2 * 32 + lg * 8);
      if (WRITE_O)
        P.p[k2] = *reinterpret_cast<const bf16x8*>(qkp + ((size_t)c * a.HV + h) * CH * CH + ar * CH + k2 * 32 + lg * 8);
    }
    // every thread loads (threads past the tile re-read a valid row), so no load sits in a
    // divergent branch and the wait counts before each use stay exact
    {
      const int r = min((tid / VPR) % CH, P.len - 1), pc = tid % VPR;
      P.v = IO<TI>::load8(vp + ((size_t)(P.t0 + r) * a.HV + h) * D + col0 + pc * 8);
    }
    {
      const int r = min(tid % CH, P.len - 1);
      P.g = a.gcum[(size_t)(P.t0 + r) * a.HV + h];
      P.b = a.beta[(size_t)(P.t0 + r) * a.HV + h];
      P.rk = a.rk[(size_t)(P.t0 + r) * a.H + j];
      P.rq = a.rq[(size_t)(P.t0 + r) * a.H + j];
    }
    P.gam = a.gamma[(size_t)c * a.HV + h];
  };

  f32x4 S[NRT][NCT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * (w * NRT + rt) + lg * 4 + i, cc = col0 + 16 * ct + lr;
        S[rt][ct][i] = a.has_h0 ? a.h0[(((size_t)n * a.HV + h) * D + d) * D + cc] : 0.f;
      }
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      lds_store4_t(sm.sST, SST, 16 * ct + lr, 16 * (w * NRT + rt) + lg * 4, S[rt][ct][0], S[rt][ct][1],
                   S[rt][ct][2], S[rt][ct][3]);

  // one chunk: stage P into LDS, start loading chunk `cn` into Q, then the chunk's products and
  // the state update
  auto step = [&](const PF& P, int c, PF& Q, int cn) {
    const int len = P.len, t0 = P.t0;
    const float gam = P.gam;
    // K, Q, A and V rows past the chunk's end hold copies of its last row: they stay finite and
    // their contributions vanish because beta and rk are zero there and P is masked
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<bf16x8*>(sm.sK + ar * SK + ks * 32 + lg * 8) = P.k[ks];
    if (tid < CH * VPR) *reinterpret_cast<bf16x8*>(sm.sV + (tid / VPR) * SV + (tid % VPR) * 8) = P.v;
    if (tid < CH) {
      const bool rok = tid < len;
      sm.sG[tid] = rok ? P.g : 0.f;
      sm.sB[tid] = rok ? P.b : 0.f;
      sm.srk[tid] = rok ? P.rk : 0.f;
      sm.srq[tid] = rok ? P.rq : 0.f;
    }
    if (cn < c_end) prefetch(Q, cn);
    __syncthreads();

    if (WRITE_TAPE) {
      bf16* tp = reinterpret_cast<bf16*>(a.htape) + ((size_t)c * a.HV + h) * D * D + (size_t)col0 * D;
      for (int idx = tid; idx < DVT * (D / 8); idx += NTHREADS) {
        const int cc = idx / (D / 8), pc = idx % (D / 8);
        *reinterpret_cast<bf16x8*>(tp + (size_t)cc * D + pc * 8) = lds8(sm.sST, SST, cc, pc * 8);
      }
    }
    f32x4 ksv[NCT], qsv[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) ksv[ct] = qsv[ct] = zero4();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bf16x8 bS = lds8(sm.sST, SST, 16 * ct + lr, kk * 32 + lg * 8);
        ksv[ct] = mfma(P.k[kk], bS, ksv[ct]);
        if (WRITE_O) qsv[ct] = mfma(P.q[kk], bS, qsv[ct]);
      }
    const int r0 = 16 * w + lg * 4;
    const float4 g4 = *reinterpret_cast<const float4*>(&sm.sG[r0]);
    const float4 b4 = *reinterpret_cast<const float4*>(&sm.sB[r0]);
    const float4 k4 = *reinterpret_cast<const float4*>(&sm.srk[r0]);
    const float4 q4 = *reinterpret_cast<const float4*>(&sm.srq[r0]);
    const float grow[4] = {g4.x, g4.y, g4.z, g4.w}, brw[4] = {b4.x, b4.y, b4.z, b4.w};
    const float rkw[4] = {k4.x, k4.y, k4.z, k4.w}, rqw[4] = {q4.x, q4.y, q4.z, q4.w};
    float brow[4], krow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      brow[i] = __expf(grow[i]);
      krow[i] = brow[i] * rkw[i];
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float vv = (float)sm.sV[(r0 + i) * SV + 16 * ct + lr];
        x[i] = brw[i] * (vv - krow[i] * ksv[ct][i]);
      }
      lds_store4_t(sm.sXT, STK, 16 * ct + lr, r0, x[0], x[1], x[2], x[3]);
    }
    __syncthreads();

    const float glast = sm.sG[len - 1];
    float dec[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dec[i] = __expf(glast - grow[i]) * rkw[i];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 R = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) R = mfma(P.a[k2], lds8(sm.sXT, STK, 16 * ct + lr, k2 * 32 + lg * 8), R);
      if (FULL) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0 + i < len)
            reinterpret_cast<bf16*>(a.vnew)[((size_t)(t0 + r0 + i) * a.HV + h) * D + col0 + 16 * ct + lr] = (bf16)R[i];
      }
      lds_store4_t(sm.sRT, STK, 16 * ct + lr, r0, R[0], R[1], R[2], R[3]);
      lds_store4_t(sm.sRdT, STK, 16 * ct + lr, r0, dec[0] * R[0], dec[1] * R[1], dec[2] * R[2], dec[3] * R[3]);
    }
    __syncthreads();

    if (WRITE_O) {
      TI* op = (TI*)a.o;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) acc = mfma(P.p[k2], lds8(sm.sRT, STK, 16 * ct + lr, k2 * 32 + lg * 8), acc);
        float ov[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = brow[i] * rqw[i] * qsv[ct][i] + acc[i];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0 + i < len) IO<TI>::store1(op + ((size_t)(t0 + r0 + i) * a.HV + h) * D + col0 + 16 * ct + lr, ov[i]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          acc = mfma(lds_tr8(sm.sK, SK, k2 * 32, 16 * (w * NRT + rt)),
                     lds8(sm.sRdT, STK, 16 * ct + lr, k2 * 32 + lg * 8), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[rt][ct][i] = __builtin_fmaf(gam, S[rt][ct][i], acc[i]);
      }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        lds_store4_t(sm.sST, SST, 16 * ct + lr, 16 * (w * NRT + rt) + lg * 4, S[rt][ct][0], S[rt][ct][1],
                     S[rt][ct][2], S[rt][ct][3]);
  };

  // two register sets, alternating: the loads for chunk c+1 fly while chunk c computes
  PF pa, pb;
  if (c_begin < c_end) prefetch(pa, c_begin);
  for (int c = c_begin; c < c_end; c += 2) {
    step(pa, c, pb, c + 1);
    if (c + 1 >= c_end) break;
    step(pb, c + 1, pa, c + 2);
  }
  if (WRITE_O && a.want_ht) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 16 * (w * NRT + rt) + lg * 4 + i, cc = col0 + 16 * ct + lr;
          a.ht[(((size_t)n * a.HV + h) * D + d) * D + cc] = S[rt][ct][i];
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

template <int D, int DVT, typename TI>
static int walk_t(const Args& a, int write_o, int write_tape, hipStream_t s) {
  const dim3 grid(chain_blocks(a, D / DVT)), blk(NTHREADS);
  if (write_o && !write_tape) hipLaunchKernelGGL((k_walk_fwd<D, DVT, TI, true, false, false>), grid, blk, 0, s, a);
  else if (write_o) hipLaunchKernelGGL((k_walk_fwd<D, DVT, TI, true, true, true>), grid, blk, 0, s, a);
  else if (a.full) hipLaunchKernelGGL((k_walk_fwd<D, DVT, TI, false, true, true>), grid, blk, 0, s, a);
  else hipLaunchKernelGGL((k_walk_fwd<D, DVT, TI, false, true, false>), grid, blk, 0, s, a);
  return (int)hipGetLastError();
}

int launch_walk_fwd(const Args& a, int write_o, int write_tape, void* stream) {
  const hipStream_t s = S_(stream);
  if (a.D == 128)
    return a.dtype == 0 ? walk_t<128, WALK_DVT, bf16>(a, write_o, write_tape, s)
                        : walk_t<128, WALK_DVT, float>(a, write_o, write_tape, s);
  return a.dtype == 0 ? walk_t<64, WALK_DVT, bf16>(a, write_o, write_tape, s)
                      : walk_t<64, WALK_DVT, float>(a, write_o, write_tape, s);
}

} // namespace gdn
