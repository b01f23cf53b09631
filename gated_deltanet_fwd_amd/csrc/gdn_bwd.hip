// Backward kernels of the chunked gated delta rule on gfx950, plus small utility kernels.
//
// For one chunk and value head with start state S and end-state gradient dSn (notation of the
// forward file; Kh = diag(rk) K, Qh = diag(rq) Q, b = exp(G), Gam_ij = exp(G_i - G_j)):
//   dR  = P^T dO + diag(exp(G_last - G)) Kh dSn
//   dS  = gamma dSn + (diag(b) Qh)^T dO - Kh^T diag(beta b) A^T dR        [k_walk_bwd, serial]
// and, chunk-parallel [k_chunk_grad], with X = diag(beta) Xu, Xu = V - diag(b) Kh S, R = A X,
// dX = A^T dR:
//   dQh += diag(b) dO S^T + (dP o Gam) Kh,   dP = mask_{i>=j}(dO R^T)
//   dKh += diag(exp(G_last - G)) R dSn^T - diag(beta b) dX S^T + (dP o Gam)^T Qh + (dKk + dKk^T) Kh
//   dV   = diag(beta) dX,   dbeta_i = Xu_i . dX_i + sum_j dL_ij Gam_ij Kk_ij
//   dA   = dR X^T,  dL = mask_{i>j}(-A^T dA A^T),  dKk = dL o (beta Gam)
//   dG_i = sum_j dGam_ij Gam_ij - sum_j dGam_ji Gam_ji + b_i db_i - Z_i exp(G_last - G_i)
//          (+ gamma <dSn, S> + sum_k Z_k exp(G_last - G_k) on the last row),
//   with dGam = mask(dP o Qk) + dL o (beta Kk), db_i = qh_i.(dO S^T)_i - beta_i (Kh S)_i.dX_i,
//   Z_i = (Kh dSn)_i . R_i; dg is the in-chunk reverse cumulative sum of dG. dq, dk are the
//   L2-norm backward of the sums of dQh, dKh over the value heads that share the q/k head.
#include "gdn_device.h"

namespace gdn {

static inline hipStream_t S_(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------------------
// utilities

__global__ void k_write_tag(uint64_t* dst, uint64_t w0, uint64_t w1, uint64_t w2, uint64_t w3) {
  if (threadIdx.x == 0) {
    dst[0] = w0;
    dst[1] = w1;
    dst[2] = w2;
    dst[3] = w3;
  }
}

int launch_write_tag(void* dst, const uint64_t* w, void* stream) {
  hipLaunchKernelGGL(k_write_tag, dim3(1), dim3(64), 0, S_(stream), (uint64_t*)dst, w[0], w[1], w[2], w[3]);
  return (int)hipGetLastError();
}

__global__ void k_fill_zero(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

int launch_fill_zero(float* p, size_t n, void* stream) {
  if (n == 0) return 0;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, S_(stream), p, n);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Full saved set extras, per (chunk, value head): w = A diag(beta b) Kh, u = A diag(beta) V,
// Aqk = P (decayed, masked normalised q.k), all bf16 token rows.
template <int D, typename TI>
__global__ __launch_bounds__(NTHREADS) void k_wy_full(Args a) {
  if (a.status[0]) return;
  const int c = blockIdx.x, h = blockIdx.y, j = h / a.G;
  const int len = a.c_len[c];
  if (len <= 0) return;
  const int t0 = a.c_t0[c];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int STK = CH + PAD;
  __shared__ __attribute__((aligned(16))) bf16 sKsT[D * STK];
  __shared__ __attribute__((aligned(16))) bf16 sVsT[D * STK];
  __shared__ float sG[CH], sB[CH], srk[CH];
  const TI* kp = (const TI*)a.k;
  const TI* vp = (const TI*)a.v;
  if (tid < CH) {
    const bool ok = tid < len;
    sG[tid] = ok ? a.gcum[(size_t)(t0 + tid) * a.HV + h] : 0.f;
    sB[tid] = ok ? a.beta[(size_t)(t0 + tid) * a.HV + h] : 0.f;
    srk[tid] = ok ? a.rk[(size_t)(t0 + tid) * a.H + j] : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < CH * (D / 8); idx += NTHREADS) {
    const int r = idx & 63, pc = idx >> 6;
    float kf[8], vf[8];
    if (r < len) {
      IO<TI>::load8f(kp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8, kf);
      IO<TI>::load8f(vp + ((size_t)(t0 + r) * a.HV + h) * D + pc * 8, vf);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = vf[e] = 0.f;
    }
    const float sk = sB[r] * expf(sG[r]) * srk[r], sv = sB[r];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sKsT[(pc * 8 + e) * STK + r] = (bf16)(kf[e] * sk);
      sVsT[(pc * 8 + e) * STK + r] = (bf16)(vf[e] * sv);
    }
  }
  const int ar = 16 * w + lr;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  bf16x8 fa[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
    fa[k2] = ar < len ? *reinterpret_cast<const bf16x8*>(akk + ((size_t)(t0 + ar) * a.HV + h) * CH + k2 * 32 + lg * 8)
                      : zero8();
  __syncthreads();
  bf16* wo = reinterpret_cast<bf16*>(a.w);
  bf16* uo = reinterpret_cast<bf16*>(a.u);
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) {
    f32x4 accw = zero4(), accu = zero4();
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      accw = mfma(fa[k2], lds8(sKsT, STK, 16 * ct + lr, k2 * 32 + lg * 8), accw);
      accu = mfma(fa[k2], lds8(sVsT, STK, 16 * ct + lr, k2 * 32 + lg * 8), accu);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + lg * 4 + i;
      if (r < len) {
        wo[((size_t)(t0 + r) * a.HV + h) * D + 16 * ct + lr] = (bf16)accw[i];
        uo[((size_t)(t0 + r) * a.HV + h) * D + 16 * ct + lr] = (bf16)accu[i];
      }
    }
  }
  const bf16* qkp = reinterpret_cast<const bf16*>(a.qk) + ((size_t)c * a.H + j) * CH * CH;
  bf16* aq = reinterpret_cast<bf16*>(a.aqk);
  for (int idx = tid; idx < len * CH; idx += NTHREADS) {
    const int r = idx >> 6, cc = idx & 63;
    const float p = cc <= r ? expf(sG[r] - sG[cc]) * (float)qkp[r * CH + cc] : 0.f;
    aq[((size_t)(t0 + r) * a.HV + h) * CH + cc] = (bf16)p;
  }
}

int launch_wy_full(const Args& a, void* stream) {
  if (a.NT == 0) return 0;
  const dim3 grid(a.NT, a.HV);
  const hipStream_t s = S_(stream);
  if (a.D == 128) {
    if (a.dtype == 0) hipLaunchKernelGGL((k_wy_full<128, bf16>), grid, dim3(NTHREADS), 0, s, a);
    else hipLaunchKernelGGL((k_wy_full<128, float>), grid, dim3(NTHREADS), 0, s, a);
  } else {
    if (a.dtype == 0) hipLaunchKernelGGL((k_wy_full<64, bf16>), grid, dim3(NTHREADS), 0, s, a);
    else hipLaunchKernelGGL((k_wy_full<64, float>), grid, dim3(NTHREADS), 0, s, a);
  }
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Reverse walk, one workgroup per (document, value head, value tile), chunks in reverse.
// Writes the end-state gradient of every chunk (bf16, transposed) and dh0.
template <int D, int DVT, typename TI>
__global__ __launch_bounds__(NTHREADS) void k_walk_bwd(Args a) {
  if (a.status[0]) return;
  constexpr int NTILE = D / DVT;
  const ChainMap cm = decode_chain(blockIdx.x, a.N, a.H, a.G, NTILE);
  if (!cm.valid) return;
  const int n = a.seq_order[cm.rank];
  const int j = cm.j, h = j * a.G + cm.gi, col0 = cm.tile * DVT;
  const int c_begin = a.seq_c0[n], c_end = a.seq_c0[n + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int NCT = DVT / 16;
  constexpr int NRT = D / 64;
  constexpr int KS = D / 32;
  constexpr int STK = CH + PAD;
  constexpr int SST = D + PAD;
  __shared__ __attribute__((aligned(16))) bf16 sKT[D * STK];
  __shared__ __attribute__((aligned(16))) bf16 sQT[D * STK];
  __shared__ __attribute__((aligned(16))) bf16 sAT[CH * STK];
  __shared__ __attribute__((aligned(16))) bf16 sdST[DVT * SST];
  __shared__ __attribute__((aligned(16))) bf16 sdOT[DVT * STK];
  __shared__ __attribute__((aligned(16))) bf16 sdOpT[DVT * STK];
  __shared__ __attribute__((aligned(16))) bf16 sdRT[DVT * STK];
  __shared__ __attribute__((aligned(16))) bf16 sYT[DVT * STK];
  __shared__ float sG[CH], sB[CH], srk[CH], srq[CH];
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;
  const TI* dop = (const TI*)a.dO;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  const bf16* qkt = reinterpret_cast<const bf16*>(a.qk);

  f32x4 dS[NRT][NCT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * (w * NRT + rt) + lg * 4 + i, cc = col0 + 16 * ct + lr;
        dS[rt][ct][i] = a.dht ? a.dht[(((size_t)n * a.HV + h) * D + d) * D + cc] : 0.f;
      }
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      lds_store4_t(sdST, SST, 16 * ct + lr, 16 * (w * NRT + rt) + lg * 4, dS[rt][ct][0], dS[rt][ct][1],
                   dS[rt][ct][2], dS[rt][ct][3]);
  __syncthreads();

  for (int c = c_end - 1; c >= c_begin; --c) {
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
      bf16x8 kv = zero8(), qv = zero8();
      if (r < len) {
        kv = IO<TI>::load8(kp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8);
        qv = IO<TI>::load8(qp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sKT[(pc * 8 + e) * STK + r] = kv[e];
        sQT[(pc * 8 + e) * STK + r] = qv[e];
      }
    }
    for (int idx = tid; idx < CH * (CH / 8); idx += NTHREADS) {
      const int r = idx & 63, pc = idx >> 6;
      const bf16x8 av =
          r < len ? *reinterpret_cast<const bf16x8*>(akk + ((size_t)(t0 + r) * a.HV + h) * CH + pc * 8) : zero8();
#pragma unroll
      for (int e = 0; e < 8; ++e) sAT[(pc * 8 + e) * STK + r] = av[e];
    }
    const int ar = 16 * w + lr;
    const bool arok = ar < len;
    bf16x8 fk[KS], fpt[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      fk[ks] = arok ? IO<TI>::load8(kp + ((size_t)(t0 + ar) * a.H + j) * D + ks * 32 + lg * 8) : zero8();
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
      fpt[k2] = *reinterpret_cast<const bf16x8*>(qkt + ((size_t)c * a.H + j) * CH * CH + ar * CH + k2 * 32 + lg * 8);
    float dov[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i;
        dov[ct][i] = r < len ? IO<TI>::load1(dop + ((size_t)(t0 + r) * a.HV + h) * D + col0 + 16 * ct + lr) : 0.f;
      }
    const float gam = a.gamma[(size_t)c * a.HV + h];
    __syncthreads();

    {
      bf16* tp = reinterpret_cast<bf16*>(a.dstape) + ((size_t)c * a.HV + h) * D * D + (size_t)col0 * D;
      for (int idx = tid; idx < DVT * (D / 8); idx += NTHREADS) {
        const int cc = idx / (D / 8), pc = idx % (D / 8);
        *reinterpret_cast<bf16x8*>(tp + (size_t)cc * D + pc * 8) = lds8(sdST, SST, cc, pc * 8);
      }
    }
    float brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) brow[i] = expf(sG[16 * w + lg * 4 + i]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      lds_store4_t(sdOT, STK, 16 * ct + lr, 16 * w + lg * 4, dov[ct][0], dov[ct][1], dov[ct][2], dov[ct][3]);
      float t[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = brow[i] * srq[16 * w + lg * 4 + i] * dov[ct][i];
      lds_store4_t(sdOpT, STK, 16 * ct + lr, 16 * w + lg * 4, t[0], t[1], t[2], t[3]);
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ii = k2 * 32 + lg * 8 + e;
        fpt[k2][e] = (ii >= ar) ? (bf16)(expf(sG[ii] - sG[ar]) * (float)fpt[k2][e]) : (bf16)0.f;
      }
    __syncthreads();

    const float glast = sG[len - 1];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 kd = zero4(), pd = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kd = mfma(fk[ks], lds8(sdST, SST, 16 * ct + lr, ks * 32 + lg * 8), kd);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) pd = mfma(fpt[k2], lds8(sdOT, STK, 16 * ct + lr, k2 * 32 + lg * 8), pd);
      float dr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i;
        dr[i] = pd[i] + expf(glast - sG[r]) * srk[r] * kd[i];
      }
      lds_store4_t(sdRT, STK, 16 * ct + lr, 16 * w + lg * 4, dr[0], dr[1], dr[2], dr[3]);
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 y = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        y = mfma(lds8(sAT, STK, 16 * w + lr, k2 * 32 + lg * 8), lds8(sdRT, STK, 16 * ct + lr, k2 * 32 + lg * 8), y);
      float t[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i;
        t[i] = sB[r] * brow[i] * srk[r] * y[i];
      }
      lds_store4_t(sYT, STK, 16 * ct + lr, 16 * w + lg * 4, t[0], t[1], t[2], t[3]);
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          a1 = mfma(lds8(sQT, STK, 16 * (w * NRT + rt) + lr, k2 * 32 + lg * 8),
                    lds8(sdOpT, STK, 16 * ct + lr, k2 * 32 + lg * 8), a1);
          a2 = mfma(lds8(sKT, STK, 16 * (w * NRT + rt) + lr, k2 * 32 + lg * 8),
                    lds8(sYT, STK, 16 * ct + lr, k2 * 32 + lg * 8), a2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[rt][ct][i] = __builtin_fmaf(gam, dS[rt][ct][i], a1[i] - a2[i]);
      }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        lds_store4_t(sdST, SST, 16 * ct + lr, 16 * (w * NRT + rt) + lg * 4, dS[rt][ct][0], dS[rt][ct][1],
                     dS[rt][ct][2], dS[rt][ct][3]);
  }
  if (a.dh0) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 16 * (w * NRT + rt) + lg * 4 + i, cc = col0 + 16 * ct + lr;
          a.dh0[(((size_t)n * a.HV + h) * D + d) * D + cc] = dS[rt][ct][i];
        }
  }
}

template <int D, typename TI>
static int walk_bwd_t(const Args& a, hipStream_t s) {
  const dim3 grid(chain_blocks(a, D / BWALK_DVT));
  hipLaunchKernelGGL((k_walk_bwd<D, BWALK_DVT, TI>), grid, dim3(NTHREADS), 0, s, a);
  return (int)hipGetLastError();
}

int launch_walk_bwd(const Args& a, void* stream) {
  const hipStream_t s = S_(stream);
  if (a.D == 128) return a.dtype == 0 ? walk_bwd_t<128, bf16>(a, s) : walk_bwd_t<128, float>(a, s);
  return a.dtype == 0 ? walk_bwd_t<64, bf16>(a, s) : walk_bwd_t<64, float>(a, s);
}

// ---------------------------------------------------------------------------------------
// Chunk gradients. DET: one workgroup per (chunk, q/k head) looping over its G value heads,
// summing dQh/dKh in registers in a fixed order, then the L2-norm backward. Otherwise one
// workgroup per (chunk, value head) adding dQh/dKh into FP32 accumulators with atomics.
template <int D>
struct GradSmem {
  static constexpr int SK = D + PAD, STK = CH + PAD, DC = 32, SDC = DC + PAD;
  // persistent
  bf16 sK[CH * SK];
  bf16 sKT[D * STK];
  bf16 sQT[D * STK];
  bf16 sA[CH * STK];
  bf16 sAT[CH * STK];
  bf16 sPT[CH * STK];
  float srk[CH], srq[CH], sG[CH], sB[CH];
  float sZ[CH], sDb[CH], sDbeta[CH];
  float sred[8];
  // per value-column slice, reused for the per-head tail
  union U {
    struct B {
      bf16 sS_tr[DC * SK];
      bf16 sdS_tr[DC * SK];
      bf16 sS_rm[D * SDC];
      bf16 sdS_rm[D * SDC];
      bf16 sdO_rm[CH * SDC];
      bf16 sdO_tr[DC * STK];
      bf16 sX_tr[DC * STK];
      bf16 sX_rm[CH * SDC];
      bf16 sR_rm[CH * SDC];
      bf16 sdR_tr[DC * STK];
      bf16 sdR_rm[CH * SDC];
      bf16 sdX_rm[CH * SDC];
    } b;
    struct C {
      float sM[CH][CH + 1];
      bf16 sT1[CH * STK];
      bf16 sT2[CH * STK];
      bf16 sT3[CH * STK];
    } t;
  } u;
};

template <int D, typename TI, bool DET>
__global__ __launch_bounds__(NTHREADS) void k_chunk_grad(Args a) {
  if (a.status[0]) return;
  const int c = blockIdx.x;
  const int len = a.c_len[c];
  if (len <= 0) return;
  const int t0 = a.c_t0[c];
  const int j = DET ? (int)blockIdx.y : (int)blockIdx.y / a.G;
  const int h_first = DET ? j * a.G : (int)blockIdx.y;
  const int h_count = DET ? a.G : 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  using SM = GradSmem<D>;
  constexpr int SK = SM::SK, STK = SM::STK, DC = SM::DC, SDC = SM::SDC;
  constexpr int KS = D / 32, NDT = D / 16, NDC = D / DC;
  __shared__ __attribute__((aligned(16))) SM sm;
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;
  const TI* vp = (const TI*)a.v;
  const TI* dop = (const TI*)a.dO;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  const bf16* htape = reinterpret_cast<const bf16*>(a.htape);
  const bf16* dstape = reinterpret_cast<const bf16*>(a.dstape);

  // ---- q/k tiles, norms, Kk = Kh Kh^T and Qk = Qh Kh^T (C layout, rows 16w..)
  if (tid < CH) {
    const bool ok = tid < len;
    sm.srk[tid] = ok ? a.rk[(size_t)(t0 + tid) * a.H + j] : 0.f;
    sm.srq[tid] = ok ? a.rq[(size_t)(t0 + tid) * a.H + j] : 0.f;
  }
  for (int idx = tid; idx < CH * (D / 8); idx += NTHREADS) {
    const int r = idx & 63, pc = idx >> 6;
    bf16x8 kv = zero8(), qv = zero8();
    if (r < len) {
      kv = IO<TI>::load8(kp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8);
      qv = IO<TI>::load8(qp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8);
    }
    *reinterpret_cast<bf16x8*>(sm.sK + r * SK + pc * 8) = kv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sm.sKT[(pc * 8 + e) * STK + r] = kv[e];
      sm.sQT[(pc * 8 + e) * STK + r] = qv[e];
    }
  }
  __syncthreads();
  f32x4 Kk[4], Qk[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) Kk[ct] = Qk[ct] = zero4();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 ak = lds8(sm.sK, SK, 16 * w + lr, ks * 32 + lg * 8);
    // Q rows as an A fragment: Q[r][d..d+7] = Q^T[d..d+7][r], gathered from the transposed tile
    bf16x8 aq;
#pragma unroll
    for (int e = 0; e < 8; ++e) aq[e] = sm.sQT[(ks * 32 + lg * 8 + e) * STK + 16 * w + lr];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 bk = lds8(sm.sK, SK, 16 * ct + lr, ks * 32 + lg * 8);
      Kk[ct] = mfma(ak, bk, Kk[ct]);
      Qk[ct] = mfma(aq, bk, Qk[ct]);
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
      Kk[ct][i] *= sm.srk[r] * sm.srk[cc];
      Qk[ct][i] *= sm.srq[r] * sm.srk[cc];
    }

  f32x4 dQacc[NDT], dKacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) dQacc[t] = dKacc[t] = zero4();

  for (int hh = 0; hh < h_count; ++hh) {
    const int h = h_first + hh;
    __syncthreads(); // previous head's tail is done with the shared buffers
    if (tid < CH) {
      const bool ok = tid < len;
      sm.sG[tid] = ok ? a.gcum[(size_t)(t0 + tid) * a.HV + h] : 0.f;
      sm.sB[tid] = ok ? a.beta[(size_t)(t0 + tid) * a.HV + h] : 0.f;
    }
    for (int idx = tid; idx < CH * (CH / 8); idx += NTHREADS) {
      const int r = idx & 63, pc = idx >> 6;
      const bf16x8 av =
          r < len ? *reinterpret_cast<const bf16x8*>(akk + ((size_t)(t0 + r) * a.HV + h) * CH + pc * 8) : zero8();
      *reinterpret_cast<bf16x8*>(sm.sA + r * STK + pc * 8) = av;
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.sAT[(pc * 8 + e) * STK + r] = av[e];
    }
    const float gam = a.gamma[(size_t)c * a.HV + h];
    __syncthreads();
    const float glast = sm.sG[len - 1];
    float brow[4], beta_r[4], rk_r[4], rq_r[4], dec_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + lg * 4 + i;
      brow[i] = expf(sm.sG[r]);
      beta_r[i] = sm.sB[r];
      rk_r[i] = sm.srk[r];
      rq_r[i] = sm.srq[r];
      dec_r[i] = expf(glast - sm.sG[r]);
    }
    // P^T (transposed, decayed, masked) from the fp32 Qk tile
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      float t[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
        t[i] = r >= cc ? expf(sm.sG[r] - sm.sG[cc]) * Qk[ct][i] : 0.f;
      }
      lds_store4_t(sm.sPT, STK, 16 * ct + lr, 16 * w + lg * 4, t[0], t[1], t[2], t[3]);
    }

    f32x4 dOS[NDT], RdS[NDT], dXS[NDT], dP[4], dA[4];
#pragma unroll
    for (int t = 0; t < NDT; ++t) dOS[t] = RdS[t] = dXS[t] = zero4();
#pragma unroll
    for (int t = 0; t < 4; ++t) dP[t] = dA[t] = zero4();
    float zpart[4] = {0.f, 0.f, 0.f, 0.f}, dbx[4] = {0.f, 0.f, 0.f, 0.f}, dbr[4] = {0.f, 0.f, 0.f, 0.f};
    float sdot = 0.f;

    for (int cv = 0; cv < NDC; ++cv) {
      auto& B = sm.u.b;
      __syncthreads(); // previous slice's readers are done
      // state slice S[:, cv*DC + dvl] and dSn slice, both from transposed bf16 tapes
      for (int idx = tid; idx < DC * (D / 8); idx += NTHREADS) {
        const int dvl = idx & (DC - 1), pc = idx / DC;
        const size_t off = ((size_t)c * a.HV + h) * D * D + (size_t)(cv * DC + dvl) * D + pc * 8;
        const bf16x8 sv = *reinterpret_cast<const bf16x8*>(htape + off);
        const bf16x8 dv = *reinterpret_cast<const bf16x8*>(dstape + off);
        *reinterpret_cast<bf16x8*>(B.sS_tr + dvl * SK + pc * 8) = sv;
        *reinterpret_cast<bf16x8*>(B.sdS_tr + dvl * SK + pc * 8) = dv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          B.sS_rm[(pc * 8 + e) * SDC + dvl] = sv[e];
          B.sdS_rm[(pc * 8 + e) * SDC + dvl] = dv[e];
          sdot += (float)sv[e] * (float)dv[e];
        }
      }
      for (int idx = tid; idx < CH * (DC / 8); idx += NTHREADS) {
        const int r = idx & 63, pc = idx >> 6;
        const bf16x8 ov =
            r < len ? IO<TI>::load8(dop + ((size_t)(t0 + r) * a.HV + h) * D + cv * DC + pc * 8) : zero8();
        *reinterpret_cast<bf16x8*>(B.sdO_rm + r * SDC + pc * 8) = ov;
#pragma unroll
        for (int e = 0; e < 8; ++e) B.sdO_tr[(pc * 8 + e) * STK + r] = ov[e];
      }
      float vv[2][4];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i;
          vv[ct][i] = r < len ? IO<TI>::load1(vp + ((size_t)(t0 + r) * a.HV + h) * D + cv * DC + 16 * ct + lr) : 0.f;
        }
      __syncthreads();

      f32x4 ksv[2], kdv[2], pdv[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        ksv[ct] = kdv[ct] = pdv[ct] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ak = lds8(sm.sK, SK, 16 * w + lr, ks * 32 + lg * 8);
          ksv[ct] = mfma(ak, lds8(B.sS_tr, SK, 16 * ct + lr, ks * 32 + lg * 8), ksv[ct]);
          kdv[ct] = mfma(ak, lds8(B.sdS_tr, SK, 16 * ct + lr, ks * 32 + lg * 8), kdv[ct]);
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          pdv[ct] = mfma(lds8(sm.sPT, STK, 16 * w + lr, k2 * 32 + lg * 8),
                         lds8(B.sdO_tr, STK, 16 * ct + lr, k2 * 32 + lg * 8), pdv[ct]);
      }
      float xu[2][4];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float x[4], dr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
          xu[ct][i] = vv[ct][i] - brow[i] * rk_r[i] * ksv[ct][i];
          x[i] = beta_r[i] * xu[ct][i];
          dr[i] = pdv[ct][i] + dec_r[i] * rk_r[i] * kdv[ct][i];
          B.sX_rm[r * SDC + cc] = (bf16)x[i];
          B.sdR_rm[r * SDC + cc] = (bf16)dr[i];
        }
        lds_store4_t(B.sX_tr, STK, 16 * ct + lr, 16 * w + lg * 4, x[0], x[1], x[2], x[3]);
        lds_store4_t(B.sdR_tr, STK, 16 * ct + lr, 16 * w + lg * 4, dr[0], dr[1], dr[2], dr[3]);
      }
      __syncthreads();

      TI* dvp = (TI*)a.dv;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 R = zero4(), dX = zero4();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          R = mfma(lds8(sm.sA, STK, 16 * w + lr, k2 * 32 + lg * 8), lds8(B.sX_tr, STK, 16 * ct + lr, k2 * 32 + lg * 8),
                   R);
          dX = mfma(lds8(sm.sAT, STK, 16 * w + lr, k2 * 32 + lg * 8),
                    lds8(B.sdR_tr, STK, 16 * ct + lr, k2 * 32 + lg * 8), dX);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
          B.sR_rm[r * SDC + cc] = (bf16)R[i];
          B.sdX_rm[r * SDC + cc] = (bf16)dX[i];
          zpart[i] += rk_r[i] * kdv[ct][i] * R[i];
          dbx[i] += xu[ct][i] * dX[i];
          dbr[i] -= beta_r[i] * rk_r[i] * ksv[ct][i] * dX[i];
          if (r < len) IO<TI>::store1(dvp + ((size_t)(t0 + r) * a.HV + h) * D + cv * DC + cc, beta_r[i] * dX[i]);
        }
      }
      __syncthreads();

#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const bf16x8 bS = lds8(B.sS_rm, SDC, 16 * t + lr, lg * 8);
        dOS[t] = mfma(lds8(B.sdO_rm, SDC, 16 * w + lr, lg * 8), bS, dOS[t]);
        dXS[t] = mfma(lds8(B.sdX_rm, SDC, 16 * w + lr, lg * 8), bS, dXS[t]);
        RdS[t] = mfma(lds8(B.sR_rm, SDC, 16 * w + lr, lg * 8), lds8(B.sdS_rm, SDC, 16 * t + lr, lg * 8), RdS[t]);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        dP[t] = mfma(lds8(B.sdO_rm, SDC, 16 * w + lr, lg * 8), lds8(B.sR_rm, SDC, 16 * t + lr, lg * 8), dP[t]);
        dA[t] = mfma(lds8(B.sdR_rm, SDC, 16 * w + lr, lg * 8), lds8(B.sX_rm, SDC, 16 * t + lr, lg * 8), dA[t]);
      }
    }

    // ---- per-head tail
    auto& Tt = sm.u.t;
    // row sums over the 16 lanes of a row group; block sum of <dSn, S>
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      zpart[i] = sum16(zpart[i]);
      dbx[i] = sum16(dbx[i]);
      dbr[i] = sum16(dbr[i]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sdot += __shfl_xor(sdot, off);
    __syncthreads(); // all slice readers done: the union switches to the tail layout
    if (lane == 0) sm.sred[w] = sdot;
    // dQk (masked dP o Gam) scaled two ways, dGam from dP, and dA
    float dgam[4][4], gmat[4][4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      float tq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
        const bool lo = r >= cc;
        const float gm = lo ? expf(sm.sG[r] - sm.sG[cc]) : 0.f;
        gmat[ct][i] = gm;
        const float dqk = lo ? dP[ct][i] * gm : 0.f;
        dgam[ct][i] = lo ? dP[ct][i] * Qk[ct][i] : 0.f;
        Tt.sT1[r * STK + cc] = (bf16)(dqk * sm.srk[cc]);
        tq[i] = dqk * rq_r[i];
        Tt.sT3[r * STK + cc] = (bf16)dA[ct][i];
      }
      lds_store4_t(Tt.sT2, STK, 16 * ct + lr, 16 * w + lg * 4, tq[0], tq[1], tq[2], tq[3]);
    }
    __syncthreads();
    // M1 = dA A^T
    f32x4 m1[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      m1[ct] = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        m1[ct] = mfma(lds8(Tt.sT3, STK, 16 * w + lr, k2 * 32 + lg * 8), lds8(sm.sA, STK, 16 * ct + lr, k2 * 32 + lg * 8),
                      m1[ct]);
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      lds_store4_t(Tt.sT3, STK, 16 * ct + lr, 16 * w + lg * 4, m1[ct][0], m1[ct][1], m1[ct][2], m1[ct][3]);
    __syncthreads();
    // dL = -A^T M1 (strictly lower)
    float dbl[4] = {0.f, 0.f, 0.f, 0.f};
    float dkk[4][4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      f32x4 acc = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        acc = mfma(lds8(sm.sAT, STK, 16 * w + lr, k2 * 32 + lg * 8), lds8(Tt.sT3, STK, 16 * ct + lr, k2 * 32 + lg * 8),
                   acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
        const float dl = r > cc ? -acc[i] : 0.f;
        dbl[i] += dl * gmat[ct][i] * Kk[ct][i];
        dkk[ct][i] = dl * beta_r[i] * gmat[ct][i];
        dgam[ct][i] += dl * beta_r[i] * Kk[ct][i];
        Tt.sM[r][cc] = dgam[ct][i] * gmat[ct][i];
      }
    }
    __syncthreads(); // done reading sT3 (M1^T)
    // dKs = dKk + dKk^T (symmetric, zero diagonal), columns scaled by rk
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i, cc = 16 * ct + lr;
        if (r > cc) {
          Tt.sT3[r * STK + cc] = (bf16)(dkk[ct][i] * sm.srk[cc]);
          Tt.sT3[cc * STK + r] = (bf16)(dkk[ct][i] * sm.srk[r]);
        } else if (r == cc) {
          Tt.sT3[r * STK + r] = (bf16)0.f;
        }
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) dbl[i] = sum16(dbl[i]);
    __syncthreads();

    // dQh = diag(b) dOS + (dQk rk) K ; dKh = dec R dSn^T - beta b dXS + (dQk rq)^T Q + (dKs rk) K
    float dbo[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      f32x4 a1 = zero4(), a2 = zero4(), a3 = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8 bK = lds8(sm.sKT, STK, 16 * t + lr, k2 * 32 + lg * 8);
        a1 = mfma(lds8(Tt.sT1, STK, 16 * w + lr, k2 * 32 + lg * 8), bK, a1);
        a2 = mfma(lds8(Tt.sT2, STK, 16 * w + lr, k2 * 32 + lg * 8), lds8(sm.sQT, STK, 16 * t + lr, k2 * 32 + lg * 8),
                  a2);
        a3 = mfma(lds8(Tt.sT3, STK, 16 * w + lr, k2 * 32 + lg * 8), bK, a3);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i, dk = 16 * t + lr;
        const float qv = (float)sm.sQT[dk * STK + r];
        dbo[i] += rq_r[i] * qv * dOS[t][i];
        const float dq = brow[i] * dOS[t][i] + a1[i];
        const float dkv = dec_r[i] * RdS[t][i] - beta_r[i] * brow[i] * dXS[t][i] + a2[i] + a3[i];
        if (DET) {
          dQacc[t][i] += dq;
          dKacc[t][i] += dkv;
        } else if (r < len) {
          atomicAdd(a.dqacc + ((size_t)(t0 + r) * a.H + j) * D + dk, dq);
          atomicAdd(a.dkacc + ((size_t)(t0 + r) * a.H + j) * D + dk, dkv);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dbo[i] = sum16(dbo[i]);
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i;
        sm.sZ[r] = zpart[i];
        sm.sDb[r] = dbo[i] + dbr[i];
        sm.sDbeta[r] = dbx[i] + dbl[i];
      }
    }
    __syncthreads();
    if (w == 0) {
      const int r = lane;
      float rows = 0.f, cols = 0.f;
      for (int x = 0; x < CH; ++x) {
        rows += Tt.sM[r][x];
        cols += Tt.sM[x][r];
      }
      const bool ok = r < len;
      const float dec = ok ? expf(glast - sm.sG[r]) : 0.f;
      const float zd = ok ? sm.sZ[r] * dec : 0.f;
      float zsum = zd;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) zsum += __shfl_xor(zsum, off);
      float dG = ok ? rows - cols + expf(sm.sG[r]) * sm.sDb[r] - zd : 0.f;
      if (r == len - 1) dG += gam * (sm.sred[0] + sm.sred[1] + sm.sred[2] + sm.sred[3]) + zsum;
      float x = dG;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_down(x, off);
        if (lane + off < 64) x += y;
      }
      if (ok) {
        a.dg[(size_t)(t0 + r) * a.HV + h] = x;
        a.dbeta[(size_t)(t0 + r) * a.HV + h] = sm.sDbeta[r];
      }
    }
  }

  if (DET) {
    // L2-norm backward of the group sums: dx = r (dxh - xh (xh . dxh)), xh = r x
    TI* dqp = (TI*)a.dq;
    TI* dkp = (TI*)a.dk;
    float qd[4] = {0.f, 0.f, 0.f, 0.f}, kd[4] = {0.f, 0.f, 0.f, 0.f};
    float rq_r[4], rk_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rq_r[i] = sm.srq[16 * w + lg * 4 + i];
      rk_r[i] = sm.srk[16 * w + lg * 4 + i];
    }
    if (a.l2norm) {
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + lg * 4 + i, dk = 16 * t + lr;
          qd[i] += rq_r[i] * (float)sm.sQT[dk * STK + r] * dQacc[t][i];
          kd[i] += rk_r[i] * (float)sm.sKT[dk * STK + r] * dKacc[t][i];
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qd[i] = sum16(qd[i]);
        kd[i] = sum16(kd[i]);
      }
    }
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + lg * 4 + i, dk = 16 * t + lr;
        if (r >= len) continue;
        float dqv = dQacc[t][i], dkv = dKacc[t][i];
        if (a.l2norm) {
          dqv = rq_r[i] * (dqv - rq_r[i] * (float)IO<TI>::load1(qp + ((size_t)(t0 + r) * a.H + j) * D + dk) * qd[i]);
          dkv = rk_r[i] * (dkv - rk_r[i] * (float)IO<TI>::load1(kp + ((size_t)(t0 + r) * a.H + j) * D + dk) * kd[i]);
        }
        IO<TI>::store1(dqp + ((size_t)(t0 + r) * a.H + j) * D + dk, dqv);
        IO<TI>::store1(dkp + ((size_t)(t0 + r) * a.H + j) * D + dk, dkv);
      }
  }
}

template <int D, typename TI>
static int chunk_grad_t(const Args& a, int det, hipStream_t s) {
  if (a.NT == 0) return 0;
  if (det) hipLaunchKernelGGL((k_chunk_grad<D, TI, true>), dim3(a.NT, a.H), dim3(NTHREADS), 0, s, a);
  else hipLaunchKernelGGL((k_chunk_grad<D, TI, false>), dim3(a.NT, a.HV), dim3(NTHREADS), 0, s, a);
  return (int)hipGetLastError();
}

int launch_chunk_grad(const Args& a, int det, void* stream) {
  const hipStream_t s = S_(stream);
  if (a.D == 128) return a.dtype == 0 ? chunk_grad_t<128, bf16>(a, det, s) : chunk_grad_t<128, float>(a, det, s);
  return a.dtype == 0 ? chunk_grad_t<64, bf16>(a, det, s) : chunk_grad_t<64, float>(a, det, s);
}

// ---------------------------------------------------------------------------------------
// Atomic reduction epilogue: L2-norm backward of the FP32 dq/dk sums and the cast to the io
// dtype, one wave per (token, q/k head) row.
template <int D, typename TI>
__global__ __launch_bounds__(NTHREADS) void k_finalize_qk(Args a) {
  const int64_t rows = a.T * a.H;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  constexpr int PER = D / 64;
  const TI* xs[2] = {(const TI*)a.q, (const TI*)a.k};
  const float* acc[2] = {a.dqacc, a.dkacc};
  TI* out[2] = {(TI*)a.dq, (TI*)a.dk};
  const float* rn[2] = {a.rq, a.rk};
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    float x[PER], g[PER];
    float dot = 0.f;
    const float r = rn[which][row];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = lane + 64 * e;
      x[e] = IO<TI>::load1(xs[which] + row * D + d);
      g[e] = acc[which][row * D + d];
      dot += r * x[e] * g[e];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float v = a.l2norm ? r * (g[e] - r * x[e] * dot) : g[e];
      IO<TI>::store1(out[which] + row * D + lane + 64 * e, v);
    }
  }
}

int launch_finalize_qk(const Args& a, void* stream) {
  const int64_t rows = a.T * a.H;
  if (rows == 0) return 0;
  const dim3 grid((unsigned)((rows + 3) / 4));
  const hipStream_t s = S_(stream);
  if (a.D == 128) {
    if (a.dtype == 0) hipLaunchKernelGGL((k_finalize_qk<128, bf16>), grid, dim3(NTHREADS), 0, s, a);
    else hipLaunchKernelGGL((k_finalize_qk<128, float>), grid, dim3(NTHREADS), 0, s, a);
  } else {
    if (a.dtype == 0) hipLaunchKernelGGL((k_finalize_qk<64, bf16>), grid, dim3(NTHREADS), 0, s, a);
    else hipLaunchKernelGGL((k_finalize_qk<64, float>), grid, dim3(NTHREADS), 0, s, a);
  }
  return (int)hipGetLastError();
}

} // namespace gdn
