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
#include <type_traits>

#include "gdn_walks.h"

namespace gdn {

// ---------------------------------------------------------------------------------------
// Chunk tables from the device copy of cu_seqlens (one workgroup of 1024 threads).
// A backward call also compares the saved set's tag (tag[0..3]) with the words of its own problem
// (w0..w3); on a mismatch the status is 2 and every later kernel of the call skips its work.
__global__ __launch_bounds__(1024) void k_tables(const int32_t* __restrict__ cu, int N, int H, int NT, int64_t T,
                                                 int* __restrict__ seq_c0, int* __restrict__ c_t0,
                                                 int* __restrict__ c_len, int* __restrict__ seq_order,
                                                 int* __restrict__ pair_order, int* __restrict__ status,
                                                 int grp_split, const uint64_t* __restrict__ tag, uint64_t w0,
                                                 uint64_t w1, uint64_t w2, uint64_t w3) {
  __shared__ int s_scan[1024];
  __shared__ int s_carry, s_bad, s_tag_bad;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_carry = 0;
    s_bad = 0;
    s_tag_bad = tag && (tag[0] != w0 || tag[1] != w1 || tag[2] != w2 || tag[3] != w3);
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
    status[0] = s_bad ? 1 : s_tag_bad ? 2 : 0;
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
  // Launch order of the paired walks: the reverse-walk and tape-walk super-groups (8 (document,
  // q/k head) groups each, documents longest first) merged by estimated run time, chunks times
  // 5 for a reverse-walk step and 4 for a tape-walk step, longest first, so that the workgroups
  // left waiting for a free CU are the shortest. Each item's place is its index in its own list
  // plus the number of items of the other list that precede it (both lists are sorted).
  // Without the longest-first document order, the kinds simply alternate. Two orders are built,
  // one per launch: the groups [grp_split, N H), then the groups [0, grp_split) after it.
  __syncthreads();
  int out0 = 0;
  for (int part = 0; part < 2; ++part) {
    const int g_lo = part == 0 ? grp_split : 0, g_hi = part == 0 ? N * H : grp_split;
    const int nsg = (g_hi - g_lo + 7) / 8;
    auto steps = [&](int s) {
      const int n = seq_order[min((g_lo + 8 * s) / H, N - 1)];
      return seq_c0[n + 1] - seq_c0[n];
    };
    for (int i = tid; i < 2 * nsg; i += 1024) {
      const int kind = i / nsg, s = i - kind * nsg; // kind 1: reverse walk
      int pos;
      if (bad || N > 8192) {
        pos = 2 * s + kind;
      } else {
        const long w = (long)steps(s) * (kind ? 5 : 4);
        int lo = 0, hi = nsg; // items of the other list that precede this one: a prefix [0, lo)
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          const long wo = (long)steps(mid) * (kind ? 4 : 5);
          if (kind ? wo > w : wo >= w) lo = mid + 1; // ties: the reverse walk first
          else hi = mid;
        }
        pos = s + lo;
      }
      pair_order[out0 + pos] = s | (kind << 30);
    }
    out0 += 2 * nsg;
  }
}

// ---------------------------------------------------------------------------------------
// Per (chunk, q/k head): inverse norms rk, rq; normalised q.k (bf16, workspace; row-major for the
// forward, transposed for the backward); and, unless BWD, per value head of the group: gcum,
// gamma and Akk = (I + L)^-1 (saved).
//
// K K^T and the q.k products run on MFMA; each wave keeps 16 rows of K K^T in registers. The
// inverse runs one value head per wave, by 16 x 16 blocks: forward substitution for the four
// diagonal blocks (one column of one block per lane), fp32 MFMA for the six blocks below them.
template <int D, typename TI, bool BWD>
__global__ __launch_bounds__(NTHREADS, 3) void k_intra(Args a) {
  if (a.status[0]) return;
  const int c = launch_chunk(a, blockIdx.x), j = blockIdx.y;
  const int len = a.c_len[c];
  if (len <= 0) return;
  const int t0 = a.c_t0[c];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int SK = D + PAD;
  constexpr int SL = CH + 4; // fp32 row stride of L: 16-byte aligned rows
  constexpr int KS = D / 32;
  // value heads per batch, one wave each; three keep the LDS footprint within a third of the CU,
  // so three workgroups share one
  constexpr int NB = 3;
  struct KQ {
    bf16 k[CH * SK];
    bf16 q[CH * SK];
  };
  union Smem { // the backward pass builds no L: its smaller footprint lets more workgroups share a CU
    KQ kq;
    float L[BWD ? 1 : NB][CH][SL];
  };
  __shared__ __attribute__((aligned(16))) Smem u;
  __shared__ float srk[CH], srq[CH];
  __shared__ float sG[NB][CH], sB[NB][CH];
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;

  // the first batch's per-token g and beta (backward: gcum) of this wave's value head, loaded
  // together with K and Q so that their latencies overlap
  const int h_pre = j * a.G + min(w, a.G - 1), r_pre = t0 + (w < a.G ? min(lane, len - 1) : 0); // waves past G: one line
  const float pre_g = BWD ? a.gcum[(size_t)h_pre * a.T + r_pre] : a.g[(size_t)r_pre * a.HV + h_pre];
  const float pre_b = BWD ? 0.f : a.beta[(size_t)r_pre * a.HV + h_pre];

  // this wave's 16 rows of K and Q (MFMA A fragments), their squared norms. The loads are
  // unconditional (rows past the chunk's end re-read its last row and are zeroed through a mask
  // the compiler cannot see through), so all of them are in flight together.
  const int ar = 16 * w + lr;
  const bool ok = ar < len;
  const size_t roff = ((size_t)(t0 + min(ar, len - 1)) * a.H + j) * D + lg * 8;
  unsigned okm = ok ? ~0u : 0u;
  asm volatile("" : "+v"(okm));
  bf16x8 fk[KS], fq[KS];
  float ssk = 0.f, ssq = 0.f;
  if constexpr (std::is_same<TI, bf16>::value) {
    // bf16 rows stay packed: masked as 32-bit words, and the squared norms summed from exact
    // products of bf16 pairs, two per instruction (v_dot2_f32_bf16)
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    struct Pairs { bf16x2_t p[4]; };
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fk[ks] = IO<TI>::load8(kp + roff + ks * 32);
      fq[ks] = IO<TI>::load8(qp + roff + ks * 32);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fk[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, fk[ks]) & okm);
      fq[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, fq[ks]) & okm);
      const Pairs pk = __builtin_bit_cast(Pairs, fk[ks]), pq = __builtin_bit_cast(Pairs, fq[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ssk = __builtin_amdgcn_fdot2_f32_bf16(pk.p[e], pk.p[e], ssk, false);
        ssq = __builtin_amdgcn_fdot2_f32_bf16(pq.p[e], pq.p[e], ssq, false);
      }
      *reinterpret_cast<bf16x8*>(u.kq.k + ar * SK + ks * 32 + lg * 8) = fk[ks];
      *reinterpret_cast<bf16x8*>(u.kq.q + ar * SK + ks * 32 + lg * 8) = fq[ks];
    }
  } else {
    float kf[KS][8], qf[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      IO<TI>::load8f(kp + roff + ks * 32, kf[ks]);
      IO<TI>::load8f(qp + roff + ks * 32, qf[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kv = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, kf[ks][e]) & okm);
        const float qv = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, qf[ks][e]) & okm);
        ssk += kv * kv;
        ssq += qv * qv;
        fk[ks][e] = (bf16)kv;
        fq[ks][e] = (bf16)qv;
      }
      *reinterpret_cast<bf16x8*>(u.kq.k + ar * SK + ks * 32 + lg * 8) = fk[ks];
      *reinterpret_cast<bf16x8*>(u.kq.q + ar * SK + ks * 32 + lg * 8) = fq[ks];
    }
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
      const size_t rr = (size_t)(t0 + min(r, len - 1)) * a.HV + h;
      if (BWD) {
        x = r < len ? (hb == 0 ? pre_g : a.gcum[(size_t)h * a.T + t0 + min(r, len - 1)]) : 0.f;
      } else {
        const float gv = r < len ? (hb == 0 ? pre_g : a.g[rr]) : 0.f;
        const float bv = r < len ? (hb == 0 ? pre_b : a.beta[rr]) : 0.f;
        x = wave_prefix_sum(gv);
        sB[w][r] = bv;
        if (r < len) a.gcum[(size_t)h * a.T + t0 + r] = x;
        if (r == len - 1) a.gamma[(size_t)c * a.HV + h] = __expf(x);
      }
      sG[w][r] = x;
    }
    __syncthreads();
    // P_qk = exp(G_q - G_k) qh.kh for q >= k, per value head: the forward stores P[q][k], the
    // backward P^T[k][q]; both are [cc][r..r+3] of this wave's tile
    // Every element's exponential is computed and then masked through an opaque mask (keepf): with
    // a select the compiler branches around each one, and every branch waits for its own LDS reads.
    // G of this lane's rows (16 w + 4 lg + i) and columns (16 ct + lr) are read once per head.
    for (int b = 0; b < nb; ++b) {
      const int h = j * a.G + hb + b;
      bf16* pout = reinterpret_cast<bf16*>(a.qk) + ((size_t)c * a.HV + h) * CH * CH;
      const float4 gr4 = *reinterpret_cast<const float4*>(&sG[b][16 * w + lg * 4]);
      const float gr[4] = {gr4.x, gr4.y, gr4.z, gr4.w};
      float gc[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) gc[ct] = sG[b][16 * ct + lr];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int cc = 16 * ct + lr;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i;
          const int qi = BWD ? r : cc, ki = BWD ? cc : r;
          const float gq = BWD ? gr[i] : gc[ct], gk = BWD ? gc[ct] : gr[i];
          const float e = __expf(fminf(gq - gk, 0.f));
          v[i] = keepf(e * qk[ct][i], qi >= ki);
        }
        lds_store4_t(pout, CH, cc, 16 * w + lg * 4, v[0], v[1], v[2], v[3]);
      }
    }
    if (BWD) {
      __syncthreads();
      continue;
    }
    for (int b = 0; b < nb; ++b) {
      const float4 gr4 = *reinterpret_cast<const float4*>(&sG[b][16 * w + lg * 4]);
      const float4 br4 = *reinterpret_cast<const float4*>(&sB[b][16 * w + lg * 4]);
      const float gr[4] = {gr4.x, gr4.y, gr4.z, gr4.w}, br[4] = {br4.x, br4.y, br4.z, br4.w};
      float gc[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) gc[ct] = sG[b][16 * ct + lr];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
          u.L[b][r][cc] = keepf(br[i] * __expf(gr[i] - gc[ct]) * kk[ct][i], r > cc);
        }
    }
    __syncthreads();
    if (w < nb) {
      // (I + L)^-1 by 16 x 16 blocks. D_b = (I + L_bb)^-1 by forward substitution, lane (b, col)
      // forming column col of D_b; then the blocks below the diagonal, one block diagonal at a
      // time, A_ij = -D_i sum_{k=j}^{i-1} L_ik A_kj (A_jj = D_j), on fp32 MFMA 16x16x4 with the k
      // index permuted (at k-step e, lane l supplies k = 4 (l / 16) + e) so that a product's
      // result is the next product's B operand as it stands.
      float (*Lw)[SL] = u.L[w];
      const int blk = lane >> 4, col = lane & 15, r16 = lane & 15, g4 = 4 * (lane >> 4);
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float* Lrow = &Lw[16 * blk + i][16 * blk];
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int m = 0; m + 4 <= i; m += 4) {
          const float4 l4 = *reinterpret_cast<const float4*>(Lrow + m);
          s0 = __builtin_fmaf(l4.x, x[m], s0);
          s1 = __builtin_fmaf(l4.y, x[m + 1], s1);
          s0 = __builtin_fmaf(l4.z, x[m + 2], s0);
          s1 = __builtin_fmaf(l4.w, x[m + 3], s1);
        }
#pragma unroll
        for (int m = (i / 4) * 4; m < i; ++m) s0 = __builtin_fmaf(Lrow[m], x[m], s0);
        x[i] = i < col ? 0.f : (i == col ? 1.f : -(s0 + s1));
      }
      // D_b row-major over the diagonal block of L (read above), D_b^T over the zero block to its
      // right (b < 3: only D_0..D_2 are right operands)
#pragma unroll
      for (int i = 0; i < 16; ++i) Lw[16 * blk + i][16 * blk + col] = x[i];
      if (blk < 3) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(&Lw[16 * blk + col][16 * (blk + 1) + 4 * q]) =
              make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
      }
      // left operand X (rows R.., columns C.. of the area): X[l % 16][4 (l / 16) + e] for k-step e;
      // a right operand read from its stored transpose has the same form
      auto frag = [&](int R, int C) {
        const float4 v = *reinterpret_cast<const float4*>(&Lw[R + r16][C + g4]);
        return f32x4{v.x, v.y, v.z, v.w};
      };
      auto mm = [](f32x4 x4, f32x4 y4, f32x4 acc) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x4[0], y4[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x4[1], y4[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x4[2], y4[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x4[3], y4[3], acc, 0, 0, 0);
        return acc;
      };
      const f32x4 D0t = frag(0, 16), D1t = frag(16, 32), D2t = frag(32, 48);
      const f32x4 D1 = frag(16, 16), D2 = frag(32, 32), D3 = frag(48, 48);
      const f32x4 L10 = frag(16, 0), L21 = frag(32, 16), L32 = frag(48, 32);
      const f32x4 L20 = frag(32, 0), L31 = frag(48, 16), L30 = frag(48, 0);
      const f32x4 z = zero4();
      const f32x4 A10 = -mm(D1, mm(L10, D0t, z), z);
      const f32x4 A21 = -mm(D2, mm(L21, D1t, z), z);
      const f32x4 A32 = -mm(D3, mm(L32, D2t, z), z);
      const f32x4 A20 = -mm(D2, mm(L21, A10, mm(L20, D0t, z)), z);
      const f32x4 A31 = -mm(D3, mm(L32, A21, mm(L31, D1t, z)), z);
      const f32x4 A30 = -mm(D3, mm(L32, A20, mm(L31, A10, mm(L30, D0t, z))), z);
      // stage the inverse (bf16) over the same area, row-major; every fp32 read above comes first
      asm volatile("" ::: "memory");
      bf16* stage = reinterpret_cast<bf16*>(&Lw[0][0]);
      constexpr int SS = CH + PAD;
#pragma unroll
      for (int i = 0; i < 16; ++i) stage[(16 * blk + i) * SS + 16 * blk + col] = (bf16)x[i];
      auto put = [&](int bi, int bj, f32x4 v) { // result layout: rows 4 (l / 16) + e, column l % 16
#pragma unroll
        for (int e = 0; e < 4; ++e) stage[(16 * bi + g4 + e) * SS + 16 * bj + r16] = (bf16)v[e];
      };
      put(1, 0, A10);
      put(2, 1, A21);
      put(3, 2, A32);
      put(2, 0, A20);
      put(3, 1, A31);
      put(3, 0, A30);
      for (int cc = 16 * (lane / 16 + 1); cc < CH; cc += 8) // zeros right of the diagonal blocks
        *reinterpret_cast<bf16x8*>(stage + lane * SS + cc) = zero8();
    }
    __syncthreads();
    if (w < nb) {
      const int h = j * a.G + hb + w;
      const bf16* stage = reinterpret_cast<const bf16*>(&u.L[w][0][0]);
      // rows of the chunk only: stores past the buffer's end (rows >= len) are dropped
      const __amdgpu_buffer_rsrc_t ar_ = make_rsrc(aout + (size_t)t0 * a.HV * CH, len * a.HV * CH * (int)sizeof(bf16));
#pragma unroll
      for (int it = 0; it < CH / 8; ++it) {
        const int r = it * 8 + (lane >> 3), pc = lane & 7;
        buf_store16(lds8(stage, CH + PAD, r, pc * 8), ar_, ((r * a.HV + h) * CH + pc * 8) * (int)sizeof(bf16));
      }
    }
    __syncthreads();
  }
  // the norms go out last: a store issued earlier would be waited for at the first wait on a
  // later load (memory operations complete in order)
  if (tid < len) {
    a.rk[(size_t)j * a.T + t0 + tid] = srk[tid];
    a.rq[(size_t)j * a.T + t0 + tid] = srq[tid];
  }
}

// ---------------------------------------------------------------------------------------
// Forward and tape walks (bodies in gdn_walks.h).
template <int D, typename TI, bool WRITE_O, bool WRITE_TAPE, bool FULL>
__global__ __launch_bounds__(walk_threads<D>(), 1) void k_walk_fwd(Args a) {
  __shared__ __attribute__((aligned(16))) WalkSmem<D, WRITE_O> sm;
  walk_fwd_body<D, TI, WRITE_O, WRITE_TAPE, FULL>(a, blockIdx.x, sm);
}

// ---------------------------------------------------------------------------------------
// Segmented walks. Workgroup b walks unit u of the plan for one value head: the (unit, q/k head)
// groups are dealt 8 at a time to the 8 XCDs (as decode_chain does), so the value heads that share
// a q/k head run on one XCD.
template <int D, typename TI, bool WRITE_O, bool WRITE_TAPE, bool FULL, int SEG>
__global__ __launch_bounds__(walk_threads<D>(), 1) void k_walk_seg(Args a, SegPlan plan) {
  __shared__ __attribute__((aligned(16))) WalkSmem<D, WRITE_O> sm;
  const int b = blockIdx.x, GS = a.G;
  const int sg = b / (8 * GS), rem = b - sg * 8 * GS, x = rem & 7, gi = rem >> 3;
  const int grp = sg * 8 + x; // (unit, q/k head), unit-major
  if (grp >= plan.n_units * a.H) return;
  const int u = grp / a.H;
  const SegUnit su = plan.u[u];
  SegChain sc;
  sc.n = su.doc;
  sc.j = grp - u * a.H;
  sc.gi = gi;
  sc.lo = su.lo;
  sc.hi = su.hi;
  sc.kind = su.kind;
  const size_t slot = (size_t)a.HV * D * D;
  sc.s_in = su.in_slot >= 0 ? a.splane + su.in_slot * slot : nullptr;
  sc.s_out = su.out_slot >= 0 ? (su.out_plane ? a.splane : a.carry) + su.out_slot * slot : nullptr;
  sc.write_ht = su.write_ht;
  walk_fwd_body<D, TI, WRITE_O, WRITE_TAPE, FULL, SEG>(a, b, sm, sc);
}

// Carry merge: S_in(i + 1) = M(i) S_in(i) + B(i) for i = 1 .. n_mid of one document, in FP32.
// Workgroup (document, value head, 16-column tile): the columns of S are independent, so the
// tile's chain of products runs alone. M(i) is staged in LDS (rows padded to 132 floats, read as
// float4 along k) and the current S tile beside it; thread (row group, column) forms D/16 rows of
// one column.
__global__ __launch_bounds__(256) void k_seg_merge(Args a, MergePlan plan, int D) {
  if (a.status[0]) return;
  constexpr int SM_ = 132;
  const int ntile = D / 16;
  const int b = blockIdx.x;
  const int doc = b / (a.HV * ntile), rem = b - doc * a.HV * ntile, h = rem / ntile, tile = rem - h * ntile;
  if (doc >= plan.n_docs) return;
  const MergeDoc md = plan.d[doc];
  __shared__ __attribute__((aligned(16))) float sM[128 * SM_];
  __shared__ float sS[128][17];
  const int tid = threadIdx.x, col = tid & 15, nr = D / 16, r0 = (tid >> 4) * nr;
  const size_t slot = (size_t)a.HV * D * D, head = (size_t)h * D * D;
  const int c = 16 * tile + col;
  for (int r = tid >> 4; r < D; r += 16) sS[r][col] = a.splane[(md.s_base) * slot + head + (size_t)r * D + c];
  for (int i = 1; i <= md.n_mid; ++i) {
    const float* M = a.carry + (md.m_base + i - 1) * slot + head;
    const float* B = a.carry + (md.b_base + i - 1) * slot + head;
    // stage M(i): D rows of D floats, 16-byte pieces
    for (int pc = tid; pc < D * D / 4; pc += 256) {
      const int r = pc / (D / 4), k4 = pc - r * (D / 4);
      *reinterpret_cast<float4*>(&sM[r * SM_ + 4 * k4]) = reinterpret_cast<const float4*>(M)[pc];
    }
    float bv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) bv[q] = q < nr ? B[(size_t)(r0 + q) * D + c] : 0.f;
    __syncthreads(); // M(i) and the current S tile are staged
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = bv[q];
    for (int k = 0; k < D; k += 4) {
      const float s0 = sS[k][col], s1 = sS[k + 1][col], s2 = sS[k + 2][col], s3 = sS[k + 3][col];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < nr) {
          const float4 m = *reinterpret_cast<const float4*>(&sM[(r0 + q) * SM_ + k]);
          acc[q] = __builtin_fmaf(m.x, s0, acc[q]);
          acc[q] = __builtin_fmaf(m.y, s1, acc[q]);
          acc[q] = __builtin_fmaf(m.z, s2, acc[q]);
          acc[q] = __builtin_fmaf(m.w, s3, acc[q]);
        }
    }
    __syncthreads(); // every read of M(i) and the current S tile is done
    float* out = a.splane + (md.s_base + i) * slot + head;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < nr) {
        sS[r0 + q][col] = acc[q];
        out[(size_t)(r0 + q) * D + c] = acc[q];
      }
  }
}

// ---------------------------------------------------------------------------------------
// launchers

static inline hipStream_t S_(void* s) { return reinterpret_cast<hipStream_t>(s); }

int launch_tables(const Args& a, const uint64_t* tag, const uint64_t* w, void* stream) {
  const uint64_t z[4] = {0, 0, 0, 0};
  if (!w) w = z;
  hipLaunchKernelGGL(k_tables, dim3(1), dim3(1024), 0, S_(stream), a.cu, a.N, a.H, a.NT, a.T, a.seq_c0, a.c_t0,
                     a.c_len, a.seq_order, a.pair_order, a.status, a.grp_split, tag, w[0], w[1], w[2], w[3]);
  return (int)hipGetLastError();
}

template <int D, typename TI>
static int intra_t(const Args& a, int bwd, hipStream_t s) {
  if (a.c_count == 0) return 0;
  const dim3 grid(a.c_count, a.H);
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
int chain_blocks(const Args& a, int ntile) { return ((a.grp_end - a.grp_off + 7) / 8) * 8 * a.G * ntile; }

void whole_range(Args& a) {
  a.grp_off = 0;
  a.grp_end = a.N * a.H;
  a.pair_off = 0;
  a.c_base = 0;
  a.c_skip_at = 0x7fffffff;
  a.c_skip = 0;
  a.c_count = a.NT;
  a.grp_split = 0;
  a.piece_lo = 0;
  a.piece_hi = 0x7fffffff;
  a.state_in = nullptr;
  a.state_out = nullptr;
}

template <int D, typename TI>
static int walk_t(const Args& a, int write_o, int write_tape, int write_vnew, hipStream_t s) {
  const dim3 grid(chain_blocks(a, 1)), blk(walk_threads<D>());
  if (!write_tape) write_vnew = 0;
  if (write_o && !write_tape) hipLaunchKernelGGL((k_walk_fwd<D, TI, true, false, false>), grid, blk, 0, s, a);
  else if (write_o && write_vnew) hipLaunchKernelGGL((k_walk_fwd<D, TI, true, true, true>), grid, blk, 0, s, a);
  else if (write_o) hipLaunchKernelGGL((k_walk_fwd<D, TI, true, true, false>), grid, blk, 0, s, a);
  else if (write_vnew) hipLaunchKernelGGL((k_walk_fwd<D, TI, false, true, true>), grid, blk, 0, s, a);
  else if (write_tape) hipLaunchKernelGGL((k_walk_fwd<D, TI, false, true, false>), grid, blk, 0, s, a);
  else return (int)hipErrorInvalidValue; // a walk that writes nothing
  return (int)hipGetLastError();
}

int launch_walk_fwd(const Args& a, int write_o, int write_tape, int write_vnew, void* stream) {
  const hipStream_t s = S_(stream);
  if (a.D == 128)
    return a.dtype == 0 ? walk_t<128, bf16>(a, write_o, write_tape, write_vnew, s)
                        : walk_t<128, float>(a, write_o, write_tape, write_vnew, s);
  return a.dtype == 0 ? walk_t<64, bf16>(a, write_o, write_tape, write_vnew, s)
                      : walk_t<64, float>(a, write_o, write_tape, write_vnew, s);
}

} // namespace gdn

namespace gdn {

template <int D, typename TI>
static int walk_seg_t(const Args& a, const SegPlan& plan, int write_o, int write_tape, int write_vnew, int transfer,
                      hipStream_t s) {
  if (plan.n_units == 0) return 0;
  const dim3 grid(((plan.n_units * a.H + 7) / 8) * 8 * a.G), blk(walk_threads<D>());
  if (!write_tape) write_vnew = 0;
  if (transfer) hipLaunchKernelGGL((k_walk_seg<D, TI, false, false, false, 2>), grid, blk, 0, s, a, plan);
  else if (write_o && !write_tape) hipLaunchKernelGGL((k_walk_seg<D, TI, true, false, false, 1>), grid, blk, 0, s, a, plan);
  else if (write_o && write_vnew) hipLaunchKernelGGL((k_walk_seg<D, TI, true, true, true, 1>), grid, blk, 0, s, a, plan);
  else if (write_o) hipLaunchKernelGGL((k_walk_seg<D, TI, true, true, false, 1>), grid, blk, 0, s, a, plan);
  else if (write_vnew) hipLaunchKernelGGL((k_walk_seg<D, TI, false, true, true, 1>), grid, blk, 0, s, a, plan);
  else if (write_tape) hipLaunchKernelGGL((k_walk_seg<D, TI, false, true, false, 1>), grid, blk, 0, s, a, plan);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_walk_seg(const Args& a, const SegPlan& plan, int write_o, int write_tape, int write_vnew, int transfer,
                    void* stream) {
  const hipStream_t s = S_(stream);
  if (a.D == 128)
    return a.dtype == 0 ? walk_seg_t<128, bf16>(a, plan, write_o, write_tape, write_vnew, transfer, s)
                        : walk_seg_t<128, float>(a, plan, write_o, write_tape, write_vnew, transfer, s);
  return a.dtype == 0 ? walk_seg_t<64, bf16>(a, plan, write_o, write_tape, write_vnew, transfer, s)
                      : walk_seg_t<64, float>(a, plan, write_o, write_tape, write_vnew, transfer, s);
}

int launch_seg_merge(const Args& a, const MergePlan& plan, void* stream) {
  if (plan.n_docs == 0) return 0;
  const dim3 grid(plan.n_docs * a.HV * (a.D / 16));
  hipLaunchKernelGGL(k_seg_merge, grid, dim3(256), 0, S_(stream), a, plan, a.D);
  return (int)hipGetLastError();
}

} // namespace gdn
