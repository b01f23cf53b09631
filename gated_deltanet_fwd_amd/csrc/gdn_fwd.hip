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
// (I + L)^-1 of a 64x64 unit lower-triangular matrix (strict lower part in Lm), FP32 in LDS.
// Diagonal 16x16 blocks by forward substitution (one lane per column), then block rows in
// order: A_ij = -A_ii * sum_{m=j}^{i-1} L_im A_mj. Ends with a barrier.
__device__ void invert64(float (*Lm)[CH + 1], float (*A)[CH + 1], float (*Tm)[16][17], int tid) {
  const int w = tid >> 6, lane = tid & 63;
  if (lane < 16) {
    const int b0 = 16 * w, col = lane;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == col) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= Lm[b0 + i][b0 + m] * x[m];
      x[i] = (i < col) ? 0.f : s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) A[b0 + i][b0 + col] = x[i];
  }
  __syncthreads();
  for (int bi = 1; bi < 4; ++bi) {
    for (int e = tid; e < bi * 256; e += 256) {
      const int bj = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      float s = 0.f;
      for (int m = bj; m < bi; ++m) {
#pragma unroll
        for (int x = 0; x < 16; ++x) s += Lm[16 * bi + r][16 * m + x] * A[16 * m + x][16 * bj + cc];
      }
      Tm[bj][r][cc] = s;
    }
    __syncthreads();
    for (int e = tid; e < bi * 256; e += 256) {
      const int bj = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      float s = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) s += A[16 * bi + r][16 * bi + x] * Tm[bj][x][cc];
      A[16 * bi + r][16 * bj + cc] = -s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// Per (chunk, q/k head): inverse norms rk, rq; normalised q.k (bf16, workspace; transposed for
// the backward); and, unless BWD, per value head of the group: gcum, gamma and Akk (saved).
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
  constexpr int PPR = D / 8;
  __shared__ __attribute__((aligned(16))) bf16 sK[CH * SK];
  __shared__ __attribute__((aligned(16))) bf16 sQ[CH * SK];
  __shared__ float srk[CH], srq[CH], sG[CH], sB[CH];
  __shared__ float sKK[CH][CH + 1];
  __shared__ float sL[CH][CH + 1];
  __shared__ float sA[CH][CH + 1];
  __shared__ float sT[3][16][17];
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;

  for (int idx = tid; idx < CH * PPR; idx += NTHREADS) {
    const int r = idx / PPR, pc = idx % PPR;
    float kf[8], qf[8];
    if (r < len) {
      IO<TI>::load8f(kp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8, kf);
      IO<TI>::load8f(qp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8, qf);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = qf[e] = 0.f;
    }
    float ssk = 0.f, ssq = 0.f;
    bf16x8 kb, qb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ssk += kf[e] * kf[e];
      ssq += qf[e] * qf[e];
      kb[e] = (bf16)kf[e];
      qb[e] = (bf16)qf[e];
    }
    *reinterpret_cast<bf16x8*>(sK + r * SK + pc * 8) = kb;
    *reinterpret_cast<bf16x8*>(sQ + r * SK + pc * 8) = qb;
#pragma unroll
    for (int off = PPR / 2; off >= 1; off >>= 1) {
      ssk += __shfl_xor(ssk, off);
      ssq += __shfl_xor(ssq, off);
    }
    if (pc == 0) {
      const float rkv = a.l2norm ? 1.f / sqrtf(ssk + 1e-6f) : 1.f;
      const float rqv = a.l2norm ? 1.f / sqrtf(ssq + 1e-6f) : 1.f;
      srk[r] = r < len ? rkv : 0.f;
      srq[r] = r < len ? rqv : 0.f;
      if (r < len) {
        a.rk[(size_t)(t0 + r) * a.H + j] = rkv;
        a.rq[(size_t)(t0 + r) * a.H + j] = rqv;
      }
    }
  }
  __syncthreads();

  // K K^T and Q K^T: wave w owns rows 16w..16w+15
  f32x4 kk[4], qk[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) kk[ct] = qk[ct] = zero4();
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const bf16x8 ak = lds8(sK, SK, 16 * w + lr, ks * 32 + lg * 8);
    const bf16x8 aq = lds8(sQ, SK, 16 * w + lr, ks * 32 + lg * 8);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 bk = lds8(sK, SK, 16 * ct + lr, ks * 32 + lg * 8);
      kk[ct] = mfma(ak, bk, kk[ct]);
      qk[ct] = mfma(aq, bk, qk[ct]);
    }
  }
  bf16* qkout = reinterpret_cast<bf16*>(a.qk) + ((size_t)c * a.H + j) * CH * CH;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
      sKK[r][cc] = kk[ct][i] * srk[r] * srk[cc];
      const bf16 qv = (bf16)(r >= cc ? qk[ct][i] * srq[r] * srk[cc] : 0.f);
      if (BWD) qkout[cc * CH + r] = qv;
      else qkout[r * CH + cc] = qv;
    }
  }
  if (BWD) return;
  __syncthreads();

  bf16* aout = reinterpret_cast<bf16*>(a.akk);
  for (int gi = 0; gi < a.G; ++gi) {
    const int h = j * a.G + gi;
    if (tid < CH) {
      const int r = tid;
      const float gv = r < len ? a.g[(size_t)(t0 + r) * a.HV + h] : 0.f;
      const float bv = r < len ? a.beta[(size_t)(t0 + r) * a.HV + h] : 0.f;
      float x = gv;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      sG[r] = x;
      sB[r] = bv;
      if (r < len) a.gcum[(size_t)(t0 + r) * a.HV + h] = x;
      if (r == len - 1) a.gamma[(size_t)c * a.HV + h] = expf(x);
    }
    __syncthreads();
    for (int idx = tid; idx < CH * CH; idx += NTHREADS) {
      const int r = idx >> 6, cc = idx & 63;
      sL[r][cc] = r > cc ? sB[r] * expf(sG[r] - sG[cc]) * sKK[r][cc] : 0.f;
    }
    __syncthreads();
    invert64(sL, sA, sT, tid);
    for (int idx = tid; idx < len * CH; idx += NTHREADS) {
      const int r = idx >> 6, cc = idx & 63;
      aout[((size_t)(t0 + r) * a.HV + h) * CH + cc] = (bf16)(cc <= r ? sA[r][cc] : 0.f);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// State walk, one workgroup per (document, value head, value tile of DVT columns).
// WRITE_O: write o (and ht). WRITE_TAPE: write the chunk-start state tape (bf16, transposed).
// FULL: also write v_new = R.
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
  constexpr int STK = CH + PAD; // stride of token-indexed transposed tiles
  constexpr int SST = D + PAD;
  __shared__ __attribute__((aligned(16))) bf16 sKT[D * STK];
  __shared__ __attribute__((aligned(16))) bf16 sST[DVT * SST];
  __shared__ __attribute__((aligned(16))) bf16 sXT[DVT * STK];
  __shared__ __attribute__((aligned(16))) bf16 sRT[DVT * STK];
  __shared__ __attribute__((aligned(16))) bf16 sRdT[DVT * STK];
  __shared__ float sG[CH], sB[CH], srk[CH], srq[CH];
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;
  const TI* vp = (const TI*)a.v;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  const bf16* qkp = reinterpret_cast<const bf16*>(a.qk);

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
      lds_store4_t(sST, SST, 16 * ct + lr, 16 * (w * NRT + rt) + lg * 4, S[rt][ct][0], S[rt][ct][1], S[rt][ct][2],
                   S[rt][ct][3]);
  __syncthreads();

  for (int c = c_begin; c < c_end; ++c) {
    const int len = a.c_len[c], t0 = a.c_t0[c];
    if (tid < CH) {
      const int r = tid;
      const bool ok = r < len;
      sG[r] = ok ? a.gcum[(size_t)(t0 + r) * a.HV + h] : 0.f;
      sB[r] = ok ? a.beta[(size_t)(t0 + r) * a.HV + h] : 0.f;
      srk[r] = ok ? a.rk[(size_t)(t0 + r) * a.H + j] : 0.f;
      srq[r] = ok ? a.rq[(size_t)(t0 + r) * a.H + j] : 0.f;
    }
    for (int idx = tid; idx < CH * (D / 8); idx += NTHREADS) {
      const int r = idx & 63, pc = idx >> 6;
      const bf16x8 kv = r < len ? IO<TI>::load8(kp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8) : zero8();
#pragma unroll
      for (int e = 0; e < 8; ++e) sKT[(pc * 8 + e) * STK + r] = kv[e];
    }
    const int ar = 16 * w + lr;
    const bool arok = ar < len;
    bf16x8 fk[KS], fq[KS], fa[2], fp[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fk[ks] = arok ? IO<TI>::load8(kp + ((size_t)(t0 + ar) * a.H + j) * D + ks * 32 + lg * 8) : zero8();
      if (WRITE_O) fq[ks] = arok ? IO<TI>::load8(qp + ((size_t)(t0 + ar) * a.H + j) * D + ks * 32 + lg * 8) : zero8();
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      fa[k2] = arok ? *reinterpret_cast<const bf16x8*>(akk + ((size_t)(t0 + ar) * a.HV + h) * CH + k2 * 32 + lg * 8)
                    : zero8();
      if (WRITE_O)
        fp[k2] = *reinterpret_cast<const bf16x8*>(qkp + ((size_t)c * a.H + j) * CH * CH + ar * CH + k2 * 32 + lg * 8);
    }
    float vv[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i;
        vv[ct][i] = r < len ? IO<TI>::load1(vp + ((size_t)(t0 + r) * a.HV + h) * D + col0 + 16 * ct + lr) : 0.f;
      }
    const float gam = a.gamma[(size_t)c * a.HV + h];
    __syncthreads();

    if (WRITE_TAPE) {
      bf16* tp = reinterpret_cast<bf16*>(a.htape) + ((size_t)c * a.HV + h) * D * D + (size_t)col0 * D;
      for (int idx = tid; idx < DVT * (D / 8); idx += NTHREADS) {
        const int cc = idx / (D / 8), pc = idx % (D / 8);
        *reinterpret_cast<bf16x8*>(tp + (size_t)cc * D + pc * 8) = lds8(sST, SST, cc, pc * 8);
      }
    }
    if (WRITE_O) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = k2 * 32 + lg * 8 + e;
          fp[k2][e] = (jj <= ar) ? (bf16)(expf(sG[ar] - sG[jj]) * (float)fp[k2][e]) : (bf16)0.f;
        }
    }
    f32x4 ksv[NCT], qsv[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) ksv[ct] = qsv[ct] = zero4();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bf16x8 bS = lds8(sST, SST, 16 * ct + lr, kk * 32 + lg * 8);
        ksv[ct] = mfma(fk[kk], bS, ksv[ct]);
        if (WRITE_O) qsv[ct] = mfma(fq[kk], bS, qsv[ct]);
      }
    float brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) brow[i] = expf(sG[16 * w + lg * 4 + i]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i;
        x[i] = sB[r] * (vv[ct][i] - brow[i] * srk[r] * ksv[ct][i]);
      }
      lds_store4_t(sXT, STK, 16 * ct + lr, 16 * w + lg * 4, x[0], x[1], x[2], x[3]);
    }
    __syncthreads();

    const float glast = sG[len - 1];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 R = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) R = mfma(fa[k2], lds8(sXT, STK, 16 * ct + lr, k2 * 32 + lg * 8), R);
      float rd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i;
        rd[i] = expf(glast - sG[r]) * srk[r] * R[i];
        if (FULL && r < len)
          reinterpret_cast<bf16*>(a.vnew)[((size_t)(t0 + r) * a.HV + h) * D + col0 + 16 * ct + lr] = (bf16)R[i];
      }
      lds_store4_t(sRT, STK, 16 * ct + lr, 16 * w + lg * 4, R[0], R[1], R[2], R[3]);
      lds_store4_t(sRdT, STK, 16 * ct + lr, 16 * w + lg * 4, rd[0], rd[1], rd[2], rd[3]);
    }
    __syncthreads();

    if (WRITE_O) {
      TI* op = (TI*)a.o;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) acc = mfma(fp[k2], lds8(sRT, STK, 16 * ct + lr, k2 * 32 + lg * 8), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i;
          if (r < len)
            IO<TI>::store1(op + ((size_t)(t0 + r) * a.HV + h) * D + col0 + 16 * ct + lr,
                           brow[i] * srq[r] * qsv[ct][i] + acc[i]);
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          acc = mfma(lds8(sKT, STK, 16 * (w * NRT + rt) + lr, k2 * 32 + lg * 8),
                     lds8(sRdT, STK, 16 * ct + lr, k2 * 32 + lg * 8), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[rt][ct][i] = __builtin_fmaf(gam, S[rt][ct][i], acc[i]);
      }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        lds_store4_t(sST, SST, 16 * ct + lr, 16 * (w * NRT + rt) + lg * 4, S[rt][ct][0], S[rt][ct][1],
                     S[rt][ct][2], S[rt][ct][3]);
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
