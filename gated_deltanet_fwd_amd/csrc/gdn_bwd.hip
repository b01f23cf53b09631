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
#include <atomic>

#include "gdn_walks.h"

namespace gdn {

static inline hipStream_t S_(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------------------
// utilities

// The saved set's tag; zeros when the call failed on the device (status nonzero), so that a
// backward refuses the buffer.
__global__ void k_write_tag(uint64_t* dst, const int* status, uint64_t w0, uint64_t w1, uint64_t w2, uint64_t w3) {
  if (threadIdx.x == 0) {
    const bool ok = status[0] == 0;
    dst[0] = ok ? w0 : 0;
    dst[1] = ok ? w1 : 0;
    dst[2] = ok ? w2 : 0;
    dst[3] = ok ? w3 : 0;
  }
}

int launch_write_tag(void* dst, const uint64_t* w, const int* status, void* stream) {
  hipLaunchKernelGGL(k_write_tag, dim3(1), dim3(64), 0, S_(stream), (uint64_t*)dst, status, w[0], w[1], w[2],
                     w[3]);
  return (int)hipGetLastError();
}

// After a call whose status is nonzero (every kernel skipped its work): its floating-point
// outputs are filled with NaN, so that no stale buffer content passes for a result.
template <typename TI>
__device__ void nan_fill(void* p, size_t n) {
  if (!p) return;
  const TI nanv = (TI)__builtin_nanf("");
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    ((TI*)p)[i] = nanv;
}

template <typename TI>
__global__ __launch_bounds__(NTHREADS) void k_poison(Args a, int bwd) {
  if (a.status[0] == 0) return;
  const size_t T = (size_t)a.T, d = (size_t)a.D, states = (size_t)a.N * a.HV * d * d;
  if (!bwd) {
    nan_fill<TI>(a.o, T * a.HV * d);
    if (a.want_ht) nan_fill<float>(a.ht, states);
    return;
  }
  nan_fill<TI>(a.dq, T * a.H * d);
  nan_fill<TI>(a.dk, T * a.H * d);
  nan_fill<TI>(a.dv, T * a.HV * d);
  nan_fill<float>(a.dg, T * a.HV);
  nan_fill<float>(a.dbeta, T * a.HV);
  nan_fill<float>(a.dh0, states);
}

int launch_poison(const Args& a, int op, void* stream) {
  const int bwd = op == 2; // GDN_OP_BWD
  if (a.dtype == 0) hipLaunchKernelGGL(k_poison<bf16>, dim3(512), dim3(NTHREADS), 0, S_(stream), a, bwd);
  else hipLaunchKernelGGL(k_poison<float>, dim3(512), dim3(NTHREADS), 0, S_(stream), a, bwd);
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
//
// The row-scaled K and V rows are staged in LDS as they are stored (16-byte rows) and read back
// transposed; the products are formed transposed (w^T = (diag(beta b) Kh)^T A^T, the A rows as the
// B operand straight from memory), so each lane holds 4 consecutive d of one token and writes
// them with one 8-byte store.
template <int D, typename TI>
__global__ __launch_bounds__(NTHREADS) void k_wy_full(Args a) {
  if (a.status[0]) return;
  const int c = blockIdx.x, h = blockIdx.y, j = h / a.G;
  const int len = a.c_len[c];
  if (len <= 0) return;
  const int t0 = a.c_t0[c];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int SK = D + 16; // rows of 32 mod 64 bytes
  __shared__ __attribute__((aligned(16))) bf16 sKs[CH * SK];
  __shared__ __attribute__((aligned(16))) bf16 sVs[CH * SK];
  __shared__ float sSk[CH], sSv[CH];
  const TI* kp = (const TI*)a.k;
  const TI* vp = (const TI*)a.v;
  // every load first (rows past the chunk's end clamped, zeroed through the row factors or a
  // mask), so that they are in flight together
  constexpr int IT = CH * (D / 8) / NTHREADS;
  float kf[IT][8], vf[IT][8];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * NTHREADS, rr = min(idx / (D / 8), len - 1), pc = idx % (D / 8);
    IO<TI>::load8f(kp + ((size_t)(t0 + rr) * a.H + j) * D + pc * 8, kf[it]);
    IO<TI>::load8f(vp + ((size_t)(t0 + rr) * a.HV + h) * D + pc * 8, vf[it]);
  }
  // this wave's A rows (tokens 16 w + lr) as MFMA B operands: B[k = token'][n = token]
  const int ar = 16 * w + lr;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  bf16x8 fa[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
    fa[k2] = *reinterpret_cast<const bf16x8*>(akk + ((size_t)(t0 + min(ar, len - 1)) * a.HV + h) * CH + k2 * 32 +
                                              lg * 8);
  // the P rows to copy: thread tid takes 16-byte pieces tid and tid + 256 of the 64 x 64 tile
  const bf16* pp = reinterpret_cast<const bf16*>(a.qk) + ((size_t)c * a.HV + h) * CH * CH;
  const bf16x8 pv0 = *reinterpret_cast<const bf16x8*>(pp + tid * 8);
  const bf16x8 pv1 = *reinterpret_cast<const bf16x8*>(pp + (tid + NTHREADS) * 8);
  if (tid < CH) {
    // row factors: beta exp(G) rk for K, beta for V; zero past the chunk's end
    const int r = min(tid, len - 1);
    const float bt = a.beta[(size_t)(t0 + r) * a.HV + h];
    const float sk = bt * __expf(a.gcum[(size_t)h * a.T + t0 + r]) * a.rk[(size_t)j * a.T + t0 + r];
    sSk[tid] = keepf(sk, tid < len);
    sSv[tid] = keepf(bt, tid < len);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * NTHREADS, r = idx / (D / 8), pc = idx % (D / 8);
    const float sk = sSk[r], sv = sSv[r];
    bf16x8 kb, vb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kb[e] = (bf16)(kf[it][e] * sk);
      vb[e] = (bf16)(vf[it][e] * sv);
    }
    *reinterpret_cast<bf16x8*>(sKs + r * SK + pc * 8) = kb;
    *reinterpret_cast<bf16x8*>(sVs + r * SK + pc * 8) = vb;
  }
  fa[0] = keep8(fa[0], ar < len);
  fa[1] = keep8(fa[1], ar < len);
  __syncthreads();
  bf16* wo = reinterpret_cast<bf16*>(a.w) + ((size_t)(t0 + ar) * a.HV + h) * D;
  bf16* uo = reinterpret_cast<bf16*>(a.u) + ((size_t)(t0 + ar) * a.HV + h) * D;
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) {
    f32x4 accw = zero4(), accu = zero4();
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      accw = mfma(lds_tr8(sKs, SK, k2 * 32, 16 * ct), fa[k2], accw);
      accu = mfma(lds_tr8(sVs, SK, k2 * 32, 16 * ct), fa[k2], accu);
    }
    // lane: d = 16 ct + 4 lg + i of token ar
    if (ar < len) {
      const float xw[4] = {accw[0], accw[1], accw[2], accw[3]}, xu[4] = {accu[0], accu[1], accu[2], accu[3]};
      IO<bf16>::store4(wo + 16 * ct + 4 * lg, xw);
      IO<bf16>::store4(uo + 16 * ct + 4 * lg, xu);
    }
  }
  // Aqk: the rows of P within the chunk
  bf16* aq = reinterpret_cast<bf16*>(a.aqk) + ((size_t)t0 * a.HV + h) * CH;
  if ((tid >> 3) < len) *reinterpret_cast<bf16x8*>(aq + (size_t)(tid >> 3) * a.HV * CH + (tid & 7) * 8) = pv0;
  if (((tid + NTHREADS) >> 3) < len)
    *reinterpret_cast<bf16x8*>(aq + (size_t)((tid + NTHREADS) >> 3) * a.HV * CH + (tid & 7) * 8) = pv1;
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
// Reverse walk (body in gdn_walks.h).
template <int D, typename TI>
__global__ __launch_bounds__(bwalk_threads<D>(), 1) void k_walk_bwd(Args a) {
  __shared__ __attribute__((aligned(16))) BWalkSmem<D> sm;
  walk_bwd_body<D, TI>(a, blockIdx.x, sm);
}

// Tape walk and reverse walk in one launch. They are independent (the reverse walk never reads
// the state tape), and each alone leaves CUs idle once the shorter documents' chains finish.
// Workgroups come in segments of one super-group (8 (document, q/k head) groups times G value
// heads, the G heads of a group on one XCD) of one kind, in the order the chunk tables computed:
// longest estimated run time first.
template <int D, typename TI>
__global__ __launch_bounds__(bwalk_threads<D>(), 1) void k_walk_pair(Args a) {
  static_assert(walk_threads<D>() == bwalk_threads<D>(), "the two walks use the same workgroup size");
  __shared__ __attribute__((aligned(16))) union U {
    WalkSmem<D, false> f;
    BWalkSmem<D> r;
  } sm;
  const int SG = 8 * a.G; // workgroups of one super-group of one kind
  const int b = blockIdx.x, seg = b / SG;
  const int code = a.pair_order[a.pair_off + seg];
  const int blk = (code & 0x3fffffff) * SG + (b - seg * SG);
  if ((code >> 30) == 0) walk_fwd_body<D, TI, false, true, false>(a, blk, sm.f);
  else walk_bwd_body<D, TI>(a, blk, sm.r);
}

template <int D, typename TI>
static int walk_pair_t(const Args& a, hipStream_t s) {
  const dim3 grid(2 * chain_blocks(a, 1));
  hipLaunchKernelGGL((k_walk_pair<D, TI>), grid, dim3(bwalk_threads<D>()), 0, s, a);
  return (int)hipGetLastError();
}

int launch_walk_pair(const Args& a, void* stream) {
  const hipStream_t s = S_(stream);
  if (a.D == 128) return a.dtype == 0 ? walk_pair_t<128, bf16>(a, s) : walk_pair_t<128, float>(a, s);
  return a.dtype == 0 ? walk_pair_t<64, bf16>(a, s) : walk_pair_t<64, float>(a, s);
}

template <int D, typename TI>
static int walk_bwd_t(const Args& a, hipStream_t s) {
  const dim3 grid(chain_blocks(a, 1));
  hipLaunchKernelGGL((k_walk_bwd<D, TI>), grid, dim3(bwalk_threads<D>()), 0, s, a);
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
//
// 8 waves: wave w owns rows 16*(w%4).. of every 64-row product and half w/4 of its columns.
// The state and adjoint tapes stream through LDS in 32-column value slices (the next slice is
// prefetched into registers); every tile is stored once and read in the other orientation with
// transpose-reads. Products that have a transpose-read operand take both operands in the
// k-permuted order (lds_tr_kp, lds_kp, or a tile whose columns are stored permuted): its
// transpose-reads touch 8 consecutive rows per 32 lanes, which the padded row strides spread over
// all LDS banks, where the plain order's rows r and r + 8 share banks. The value-dimension contractions feed dQh and dKh directly through row-scaled
// A fragments: diag(b) dO S^T, diag(exp(G_last - G)) R dSn^T and -diag(beta b) dX S^T.
constexpr int GRAD_THREADS = 512;
constexpr int GRAD_MAXG = 8; // value heads per q/k head whose dg, dbeta wait in LDS (more: stored per head)

template <int D>
struct GradSmem {
  static constexpr int SK = D + 16;  // K, Q rows; S^T, dSn^T slice rows
  static constexpr int SA = CH + 16; // A rows and token-indexed transposed tiles
  static constexpr int DC = 32;      // value columns per slice
  static constexpr int SDO = DC + 16;
  static constexpr int SV = DC + PAD;
  bf16 sK[CH * SK];
  bf16 sQ[CH * SK];
  bf16 sA[CH * SA];
  bf16 sP[CH * SA];
  float sG[CH], sB[CH], srk[CH], srq[CH];
  float sRow[2][4][CH];
  float sRowM[2][CH]; // per column half: row sums of dGam o Gam
  float sCol[4][CH];  // per row tile: column sums of dGam o Gam
  float sred[8];
  f32x4 sKQ[2][8][2][64]; // Kk, Qk: each wave's own C tiles, parked for the per-head tails
  float sDGB[GRAD_MAXG][2][CH]; // dg, dbeta of each head, written out after the last head
  union U {
    struct Sl {
      bf16 sS[DC * SK];
      bf16 sdS[DC * SK];
      bf16 sdO[CH * SDO];
      bf16 sV[CH * SV];
      bf16 sXT[DC * SA];
      bf16 sdRT[DC * SA];
      bf16 sRT[DC * SA];
      bf16 sRTd[DC * SA]; // R^T with the rows of R scaled by exp(G_last - G)
      bf16 sdXT[DC * SA]; // dX^T with the rows of dX scaled by -beta exp(G)
    } b;
    struct Tl {
      bf16 sT1t[CH * SA];
      bf16 sT2[CH * SA];
      bf16 sT3[CH * SA];  // dA^T, then M1^T
      bf16 sE1t[CH * SA]; // (dKk diag(rk))^T
      bf16 sE2[CH * SA];  // dKk^T diag(rk), row-major
    } t;
  } u;
  int next_item; // the item claimed from the work queue, published by thread 0 (last: the tiles
                 // above keep their 16-byte alignment)
};


static_assert(offsetof(GradSmem<128>, u) % 16 == 0 && offsetof(GradSmem<64>, u) % 16 == 0,
              "the slice and tail tiles start 16-byte aligned");

template <int D, typename TI, bool DET>
__global__ __launch_bounds__(GRAD_THREADS) void k_chunk_grad(Args a) {
  if (a.status[0]) return;
  // Persistent: workgroup b takes item b, then items claimed from the launch's work queue
  // (a.gq: gridDim.x + the counter's old value), until the queue runs past the last item (item =
  // chunk x per-chunk index y; y is the q/k head, or the value head in atomic mode). Workgroups
  // that start late, behind another launch's, take fewer items. The next item is claimed at the
  // start of the current one and its first loads are issued during the current item's last head
  // and before its epilogue, so they are in flight while it finishes.
  const int nj = DET ? a.H : a.HV;
  const int n_items = a.c_count * nj;
  int item = blockIdx.x;
  if (item >= n_items) return;
  int c, j, h_first, len, t0;
  auto decode = [&](int it, int& ci, int& ji, int& hi, int& li, int& ti) {
    const int x = it / nj, y = it - x * nj;
    ci = launch_chunk(a, x);
    ji = DET ? y : y / a.G;
    hi = DET ? y * a.G : y;
    li = __builtin_amdgcn_readfirstlane(a.c_len[ci]); // uniform: kept in scalar registers
    ti = __builtin_amdgcn_readfirstlane(a.c_t0[ci]);
  };
  decode(item, c, j, h_first, len, t0);
  const int h_count = DET ? a.G : 1;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w & 3, half = w >> 2;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = 16 * rt;      // rows of this wave's product tiles
  const int arow = row0 + lr;    // row of this lane's A fragments
  using SM = GradSmem<D>;
  constexpr int SK = SM::SK, SA = SM::SA, DC = SM::DC, SDO = SM::SDO, SV = SM::SV;
  constexpr int KS = D / 32, NDC = D / DC;
  constexpr int NT2 = D / 32;    // 16-wide key-dim column tiles per wave (half of D/16)
  __shared__ __attribute__((aligned(16))) SM sm;
  const TI* kp = (const TI*)a.k;
  const TI* qp = (const TI*)a.q;
  const TI* vp = (const TI*)a.v;
  const TI* dop = (const TI*)a.dO;
  const bf16* akk = reinterpret_cast<const bf16*>(a.akk);
  const bf16* htape = reinterpret_cast<const bf16*>(a.htape);
  const bf16* dstape = reinterpret_cast<const bf16*>(a.dstape);
  const bf16* qkt = reinterpret_cast<const bf16*>(a.qk);

  // Prefetch registers. Every load is unconditional (rows clamped to the chunk, rows past its end
  // zeroed when staged), so the loads of one batch are in flight together and waited for once.
  bf16x8 nS, ndS, nx; // slice: S^T / dSn^T piece; dO piece (threads < 256) or V piece (threads >= 256)
  bf16x8 nA, nP;      // head: A and P row pieces
  float nGB;          // head: G (wave 0) or beta (other waves) of row tid % 64
  auto prefetch = [&](int c, int t0, int len, int h, int cv, int tid) {
    const int dvl = min(tid / (D / 8), DC - 1), pc = tid % (D / 8); // 32 rows x D/8 pieces
    const size_t off = ((size_t)c * a.HV + h) * D * D + (size_t)(cv * DC + dvl) * D + pc * 8;
    nS = *reinterpret_cast<const bf16x8*>(htape + off);
    ndS = *reinterpret_cast<const bf16x8*>(dstape + off);
    const int u = tid & 255, r = min(u >> 2, len - 1), pv = u & 3;
    const TI* src = tid < 256 ? dop : vp;
    nx = IO<TI>::load8(src + ((size_t)(t0 + r) * a.HV + h) * D + cv * DC + pv * 8);
  };
  auto store_head = [&](int len, int tid) {
    const int r = tid >> 3, pc = tid & 7;
    *reinterpret_cast<bf16x8*>(sm.sA + r * SA + pc * 8) = keep8(nA, r < len);
    lds_store_kp8(sm.sP, SA, r, pc, keep8(nP, r < len)); // k-permuted columns: lds8 reads P . dO operands
    if (tid < 2 * CH) (tid < CH ? sm.sG : sm.sB)[tid & 63] = keepf(nGB, (tid & 63) < len);
  };
  auto prefetch_head = [&](int c, int t0, int len, int h, int tid) {
    const int r = min(tid >> 3, len - 1), pc = tid & 7;
    nA = *reinterpret_cast<const bf16x8*>(akk + ((size_t)(t0 + r) * a.HV + h) * CH + pc * 8);
    // waves 0 and 1 gather 64 rows; the others read one row (one cache line, no branch)
    const int rr = tid < 2 * CH ? min(tid & 63, len - 1) : 0;
    nGB = *((tid >> 6) == 0 ? a.gcum + (size_t)h * a.T + t0 + rr : a.beta + (size_t)(t0 + rr) * a.HV + h);
    nP = *reinterpret_cast<const bf16x8*>(qkt + ((size_t)c * a.HV + h) * CH * CH + r * CH + pc * 8);
  };

  // K, Q rows and their norms of an item
  constexpr int KQ_IT = CH * (D / 8) / GRAD_THREADS;
  static_assert(KQ_IT * GRAD_THREADS == CH * (D / 8), "K/Q staging covers the tile");
  bf16x8 kv[KQ_IT], qv[KQ_IT];
  float rkv, rqv;
  auto load_kq = [&](int t0, int len, int j, int tid) {
#pragma unroll
    for (int it = 0; it < KQ_IT; ++it) {
      const int idx = tid + it * GRAD_THREADS, r = min(idx / (D / 8), len - 1), pc = idx % (D / 8);
      kv[it] = IO<TI>::load8(kp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8);
      qv[it] = IO<TI>::load8(qp + ((size_t)(t0 + r) * a.H + j) * D + pc * 8);
    }
    const int rr0 = tid < CH ? min(tid & 63, len - 1) : 0; // only wave 0 stages the norms
    rkv = a.rk[(size_t)j * a.T + t0 + rr0];
    rqv = a.rq[(size_t)j * a.T + t0 + rr0];
  };
  load_kq(t0, len, j, tid);
  prefetch_head(c, t0, len, h_first, tid);
  prefetch(c, t0, len, h_first, 0, tid);

  for (;;) {
  // lane indices re-derived from an opaque thread id per item, as in the head loop below (else
  // lane-dependent addresses are hoisted out of the item loop and held in registers throughout)
  int tid_i = threadIdx.x;
  asm volatile("" : "+v"(tid_i));
  const int tid = tid_i, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w & 3, half = w >> 2, lr = lane & 15, lg = lane >> 4, row0 = 16 * rt, arow = row0 + lr;
  // claim the next item; every thread reads it after the staging barrier below (and thread 0
  // writes the slot again only in the next item, after several more barriers)
  if (tid == 0) sm.next_item = (int)gridDim.x + atomicAdd(a.gq, 1);

  // ---- stage K, Q and the norms; Kk = Kh Kh^T, Qk = Qh Kh^T on this wave's tiles
#pragma unroll
  for (int it = 0; it < KQ_IT; ++it) {
    const int idx = tid + it * GRAD_THREADS, r = idx / (D / 8), pc = idx % (D / 8);
    *reinterpret_cast<bf16x8*>(sm.sK + r * SK + pc * 8) = keep8(kv[it], r < len);
    *reinterpret_cast<bf16x8*>(sm.sQ + r * SK + pc * 8) = keep8(qv[it], r < len);
  }
  if (tid < CH) {
    sm.srk[tid] = keepf(rkv, tid < len);
    sm.srq[tid] = keepf(rqv, tid < len);
  }
  __syncthreads();
  // the next item (this one again after the last: its loads then repeat this item's, unused)
  const int item_n = __builtin_amdgcn_readfirstlane(sm.next_item);
  const bool has_next = item_n < n_items;
  int c_n, j_n, hf_n, len_n, t0_n;
  decode(has_next ? item_n : item, c_n, j_n, hf_n, len_n, t0_n);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    f32x4 Kk = zero4(), Qk = zero4();
    const int ct = 2 * half + c2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 bk = lds8(sm.sK, SK, 16 * ct + lr, ks * 32 + lg * 8);
      Kk = mfma(lds8(sm.sK, SK, arow, ks * 32 + lg * 8), bk, Kk);
      Qk = mfma(lds8(sm.sQ, SK, arow, ks * 32 + lg * 8), bk, Qk);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + lg * 4 + i, cc = 16 * ct + lr;
      Kk[i] *= sm.srk[r] * sm.srk[cc];
      Qk[i] *= sm.srq[r] * sm.srk[cc];
    }
    sm.sKQ[0][w][c2][lane] = Kk;
    sm.sKQ[1][w][c2][lane] = Qk;
  }
  store_head(len, tid); // the first head's tiles (not read above)
  // norms of this lane's C rows, re-read from LDS where used
  auto rk4 = [&]() { return *reinterpret_cast<const f32x4*>(sm.srk + row0 + lg * 4); };
  auto rq4 = [&]() { return *reinterpret_cast<const f32x4*>(sm.srq + row0 + lg * 4); };

  f32x4 dQacc[NT2], dKacc[NT2];
#pragma unroll
  for (int t = 0; t < NT2; ++t) dQacc[t] = dKacc[t] = zero4();
  // qh . dQacc on this lane's C rows, over this lane's columns
  auto qdot_acc = [&](int row0, int lg, int half, int lr) {
    f32x4 acc = zero4();
#pragma unroll
    for (int t = 0; t < NT2; ++t) {
      const bf16x4 qv = lds_tr4c(sm.sQ, SK, row0, 16 * (half * NT2 + t)); // this lane's C rows
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += (float)qv[i] * dQacc[t][i];
    }
    const f32x4 rq_r = *reinterpret_cast<const f32x4*>(sm.srq + row0 + lg * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= rq_r[i];
    return acc;
  };
  f32x4 qprev = zero4(); // qdot_acc() after the previous head

  for (int hh = 0; hh < h_count; ++hh) {
    const int h = h_first + hh;
    // Lane indices re-derived from an opaque copy of the thread id in every head: otherwise the
    // compiler hoists dozens of lane-dependent addresses out of the head loop and spills.
    int tid_o = threadIdx.x;
    if (DET) asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), rt = w & 3, half = w >> 2, row0 = 16 * rt, arow = row0 + lr;
    // column of this lane's 4 C rows in a tile whose columns are kept k-permuted (lds_store_kp8's
    // order), so that lds8 row reads of it pair with k-permuted transpose reads
    const int kpcol = 32 * (rt >> 1) + 8 * lg + 4 * (rt & 1);
    __syncthreads(); // this head's A, P, G and beta are staged
    const float glast = sm.sG[len - 1];
    // per-row factors: this lane's C rows (r) and A-fragment row (arow)
    float brow[4], beta_r[4], dec_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + lg * 4 + i;
      brow[i] = __expf(sm.sG[r]);
      beta_r[i] = sm.sB[r];
      dec_r[i] = __expf(glast - sm.sG[r]);
    }
    const float a_b = __expf(sm.sG[arow]);

    float zp[4] = {0.f, 0.f, 0.f, 0.f}, dbx[4] = {0.f, 0.f, 0.f, 0.f}, dbr[4] = {0.f, 0.f, 0.f, 0.f};
    float sdot = 0.f;
    f32x4 dP[2], dA[2];
    dP[0] = dP[1] = dA[0] = dA[1] = zero4();

    for (int cv = 0; cv < NDC; ++cv) {
      auto& B = sm.u.b;
      __syncthreads(); // readers of the previous slice are done
      {
        const int dvl = tid / (D / 8), pc = tid % (D / 8);
        if (dvl < DC) {
          *reinterpret_cast<bf16x8*>(B.sS + dvl * SK + pc * 8) = nS;
          *reinterpret_cast<bf16x8*>(B.sdS + dvl * SK + pc * 8) = ndS;
          // <dSn, S> of this piece: bf16 pair products (exact in f32) summed two at a time
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          struct Pairs { bf16x2_t p[4]; };
          const Pairs ps = __builtin_bit_cast(Pairs, nS), pd = __builtin_bit_cast(Pairs, ndS);
#pragma unroll
          for (int e = 0; e < 4; ++e) sdot = __builtin_amdgcn_fdot2_f32_bf16(ps.p[e], pd.p[e], sdot, false);
        }
        const int u = tid & 255, r = u >> 2, pv = u & 3;
        const bf16x8 xv = r < len ? nx : zero8();
        if (tid < 256) *reinterpret_cast<bf16x8*>(B.sdO + r * SDO + pv * 8) = xv;
        else *reinterpret_cast<bf16x8*>(B.sV + r * SV + pv * 8) = xv;
      }
      // the next slice, the next head's first, or after the last head the next item's first:
      // always a load, so no branch leaves the wait counts unsure which registers are loading
      {
        const bool nslice = cv + 1 < NDC, nitem = !nslice && hh + 1 == h_count;
        prefetch(nitem ? c_n : c, nitem ? t0_n : t0, nitem ? len_n : len, nslice ? h : nitem ? hf_n : h + 1,
                 nslice ? cv + 1 : 0, tid);
      }
      __syncthreads();

      // this wave's 16 x 16 tile of the slice: rows row0.., slice columns 16*half..
      const int cs = 16 * half;
      f32x4 ksv = zero4(), kdv = zero4(), pdv = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 fk = lds8(sm.sK, SK, arow, ks * 32 + lg * 8);
        ksv = mfma(fk, lds8(B.sS, SK, cs + lr, ks * 32 + lg * 8), ksv);
        kdv = mfma(fk, lds8(B.sdS, SK, cs + lr, ks * 32 + lg * 8), kdv);
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) pdv = mfma(lds8(sm.sP, SA, arow, k2 * 32 + lg * 8), lds_tr_kp(B.sdO, SDO, k2 * 32, cs), pdv);
      float xu[4], x[4], dr[4];
      const f32x4 rk_r = rk4();
      const bf16x4 vv = lds_tr4c(B.sV, SV, row0, cs);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xu[i] = (float)vv[i] - brow[i] * rk_r[i] * ksv[i];
        x[i] = beta_r[i] * xu[i];
        dr[i] = pdv[i] + dec_r[i] * rk_r[i] * kdv[i];
      }
      lds_store4_t(B.sXT, SA, cs + lr, row0 + lg * 4, x[0], x[1], x[2], x[3]);
      lds_store4_t(B.sdRT, SA, cs + lr, row0 + lg * 4, dr[0], dr[1], dr[2], dr[3]);
      __syncthreads();

      f32x4 R = zero4(), dX = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        R = mfma(lds8(sm.sA, SA, arow, k2 * 32 + lg * 8), lds8(B.sXT, SA, cs + lr, k2 * 32 + lg * 8), R);
        dX = mfma(lds_tr8(sm.sA, SA, k2 * 32, row0), lds8(B.sdRT, SA, cs + lr, k2 * 32 + lg * 8), dX);
      }
      TI* dvp = (TI*)a.dv;
      const f32x4 rk_r2 = rk4();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + lg * 4 + i, cc = cs + lr;
        zp[i] += rk_r2[i] * kdv[i] * R[i];
        dbx[i] += xu[i] * dX[i];
        dbr[i] -= beta_r[i] * rk_r2[i] * ksv[i] * dX[i];
        if (r < len) IO<TI>::store1(dvp + ((size_t)(t0 + r) * a.HV + h) * D + cv * DC + cc, beta_r[i] * dX[i]);
      }
      // R and dX are stored transposed (the A operands below), also with their row factors applied
      // here, on the fp32 values (one rounding to bf16 instead of two)
      lds_store4_t(B.sRT, SA, cs + lr, row0 + lg * 4, R[0], R[1], R[2], R[3]);
      lds_store4_t(B.sRTd, SA, cs + lr, row0 + lg * 4, R[0] * dec_r[0], R[1] * dec_r[1], R[2] * dec_r[2],
                   R[3] * dec_r[3]);
      lds_store4_t(B.sdXT, SA, cs + lr, row0 + lg * 4, dX[0] * (-beta_r[0] * brow[0]), dX[1] * (-beta_r[1] * brow[1]),
                   dX[2] * (-beta_r[2] * brow[2]), dX[3] * (-beta_r[3] * brow[3]));
      __syncthreads();

      // value-dimension contractions over this slice (32 = one MFMA k-step)
      const bf16x8 aO = lds_kp(B.sdO, SDO, arow, 0);
      const bf16x8 aOb = scale8(aO, a_b);
      const bf16x8 aR = lds_tr_kp(B.sRTd, SA, 0, row0);
      const bf16x8 aX = lds_tr_kp(B.sdXT, SA, 0, row0);
#pragma unroll
      for (int t = 0; t < NT2; ++t) {
        const int dcol = 16 * (half * NT2 + t);
        const bf16x8 bS = lds_tr_kp(B.sS, SK, 0, dcol);
        dQacc[t] = mfma(aOb, bS, dQacc[t]);
        dKacc[t] = mfma(aX, bS, dKacc[t]);
        dKacc[t] = mfma(aR, lds_tr_kp(B.sdS, SK, 0, dcol), dKacc[t]);
      }
      const bf16x8 adR = lds_tr_kp(B.sdRT, SA, 0, row0);
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int ct = 2 * half + c2;
        dP[c2] = mfma(aO, lds_tr_kp(B.sRT, SA, 0, 16 * ct), dP[c2]);
        dA[c2] = mfma(adR, lds_tr_kp(B.sXT, SA, 0, 16 * ct), dA[c2]);
      }
    }

    // ---- per-head tail; the next head's (or the next item's first head's) tiles load meanwhile
    {
      const bool nitem = hh + 1 == h_count;
      prefetch_head(nitem ? c_n : c, nitem ? t0_n : t0, nitem ? len_n : len, nitem ? hf_n : h + 1, tid);
    }
    auto& T = sm.u.t;
    // b_i (Qh S dO^T)_ii: the slices added diag(b) dO S^T of this head to dQacc, so it is the
    // growth of qh_i . dQacc_i over the slice loop
    float dbo[4];
    {
      const f32x4 qn = qdot_acc(row0, lg, half, lr);
#pragma unroll
      for (int i = 0; i < 4; ++i) dbo[i] = qn[i] - qprev[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      zp[i] = row_sum16(zp[i]);
      dbx[i] = row_sum16(dbx[i]);
      dbr[i] = row_sum16(dbr[i]);
      dbo[i] = row_sum16(dbo[i]);
    }
    sdot = col_sum4(row_sum16(sdot));
    __syncthreads(); // slice tiles are dead: the union switches to the tail layout
    if (lane == 0) sm.sred[w] = sdot;
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + lg * 4 + i;
        sm.sRow[half][0][r] = zp[i];
        sm.sRow[half][1][r] = dbo[i] + brow[i] * dbr[i];
        sm.sRow[half][2][r] = dbx[i];
      }
    }
    // Gam = exp(G_r - G_c) on and below the diagonal: computed for every element and masked
    // (keepf), since a select makes the compiler branch around each exponential and wait for its
    // LDS reads inside every branch
    float gm[2][4], dgam[2][4];
    const f32x4 rq_r = rq4();
    const f32x4 g_r = *reinterpret_cast<const f32x4*>(sm.sG + row0 + lg * 4);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int ct = 2 * half + c2, cc = 16 * ct + lr;
      const f32x4 Qk = sm.sKQ[1][w][c2][lane];
      const float g_c = sm.sG[cc];
      float t1[4], t2[4], t3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + lg * 4 + i;
        // rows past the chunk's end are masked too: their G is staged as 0, so exp(G_r - G_c) may
        // overflow there, and an infinite factor would turn their zero dP into NaN
        const bool lo = r >= cc && r < len;
        gm[c2][i] = keepf(__expf(g_r[i] - g_c), lo);
        const float dqk = lo ? dP[c2][i] * gm[c2][i] : 0.f;
        dgam[c2][i] = lo ? dP[c2][i] * Qk[i] : 0.f;
        t1[i] = dqk * sm.srk[cc];
        t2[i] = dqk * rq_r[i];
        t3[i] = dA[c2][i];
      }
      lds_store4_t(T.sT1t, SA, cc, row0 + lg * 4, t1[0], t1[1], t1[2], t1[3]); // (dQk rk)^T
      lds_store4_t(T.sT2, SA, cc, kpcol, t2[0], t2[1], t2[2], t2[3]);          // (dQk rq)^T
      lds_store4_t(T.sT3, SA, cc, row0 + lg * 4, t3[0], t3[1], t3[2], t3[3]);  // dA^T
    }
    __syncthreads();
    // M1 = dA A^T
    f32x4 m1[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int ct = 2 * half + c2;
      m1[c2] = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        m1[c2] = mfma(lds_tr8(T.sT3, SA, k2 * 32, row0), lds8(sm.sA, SA, 16 * ct + lr, k2 * 32 + lg * 8), m1[c2]);
    }
    __syncthreads();
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int ct = 2 * half + c2;
      lds_store4_t(T.sT3, SA, 16 * ct + lr, kpcol, m1[c2][0], m1[c2][1], m1[c2][2], m1[c2][3]); // M1^T
    }
    __syncthreads();
    // dL = -A^T M1 (strictly lower); dKk = dL o (beta Gam) goes to two tiles, one per term of
    // (dKk + dKk^T) diag(rk); row and column sums of dGam o Gam are reduced per wave (DPP rows,
    // lane-group columns) into per-half and per-row-tile partials
    float dbl[4] = {0.f, 0.f, 0.f, 0.f}, rsum[4] = {0.f, 0.f, 0.f, 0.f};
    const f32x4 rk_r = rk4();
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int ct = 2 * half + c2, cc = 16 * ct + lr;
      const float rkc = sm.srk[cc];
      const f32x4 Kk = sm.sKQ[0][w][c2][lane];
      f32x4 acc = zero4();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        acc = mfma(lds_tr_kp(sm.sA, SA, k2 * 32, row0), lds8(T.sT3, SA, 16 * ct + lr, k2 * 32 + lg * 8), acc);
      float e1[4], e2[4], csum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + lg * 4 + i;
        const float dl = r > cc ? -acc[i] : 0.f;
        dbl[i] += dl * gm[c2][i] * Kk[i];
        const float dkk = dl * beta_r[i] * gm[c2][i];
        dgam[c2][i] += dl * beta_r[i] * Kk[i];
        const float mm = dgam[c2][i] * gm[c2][i];
        rsum[i] += mm;
        csum += mm;
        e1[i] = dkk * rkc;     // (dKk diag(rk))[r][cc], stored transposed
        e2[i] = dkk * rk_r[i]; // (dKk^T diag(rk))[cc][r]
      }
      csum = col_sum4(csum);
      if (lg == 0) sm.sCol[rt][cc] = csum;
      lds_store4_t(T.sE1t, SA, cc, row0 + lg * 4, e1[0], e1[1], e1[2], e1[3]);
      lds_store4_t(T.sE2, SA, cc, kpcol, e2[0], e2[1], e2[2], e2[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dbl[i] = row_sum16(dbl[i]);
      rsum[i] = row_sum16(rsum[i]);
    }
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sm.sRow[half][3][row0 + lg * 4 + i] = dbl[i];
        sm.sRowM[half][row0 + lg * 4 + i] = rsum[i];
      }
    }
    __syncthreads();
    // dQh += (dQk rk) K ; dKh += (dQk rq)^T Q + (dKs rk) K
    {
      const bf16x8 a1[2] = {lds_tr_kp(T.sT1t, SA, 0, row0), lds_tr_kp(T.sT1t, SA, 32, row0)};
      const bf16x8 a2[2] = {lds8(T.sT2, SA, arow, lg * 8), lds8(T.sT2, SA, arow, 32 + lg * 8)};
      const bf16x8 e1[2] = {lds_tr_kp(T.sE1t, SA, 0, row0), lds_tr_kp(T.sE1t, SA, 32, row0)};
      const bf16x8 e2[2] = {lds8(T.sE2, SA, arow, lg * 8), lds8(T.sE2, SA, arow, 32 + lg * 8)};
#pragma unroll
      for (int t = 0; t < NT2; ++t) {
        const int dcol = 16 * (half * NT2 + t);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const bf16x8 bK = lds_tr_kp(sm.sK, SK, k2 * 32, dcol);
          dQacc[t] = mfma(a1[k2], bK, dQacc[t]);
          dKacc[t] = mfma(a2[k2], lds_tr_kp(sm.sQ, SK, k2 * 32, dcol), dKacc[t]);
          dKacc[t] = mfma(e1[k2], bK, dKacc[t]);
          dKacc[t] = mfma(e2[k2], bK, dKacc[t]);
        }
      }
    }
    qprev = qdot_acc(row0, lg, half, lr); // dQacc is complete for this head
    if (w == 0) {
      // lane l takes row 63 - l, so the in-chunk reverse cumulative sum is a prefix sum over lanes
      const int r = 63 - lane;
      const float rows = sm.sRowM[0][r] + sm.sRowM[1][r];
      const float cols = sm.sCol[0][r] + sm.sCol[1][r] + sm.sCol[2][r] + sm.sCol[3][r];
      const bool ok = r < len;
      const float g_r1 = sm.sG[r];
      const float dec = keepf(__expf(glast - g_r1), ok);
      const float z = sm.sRow[0][0][r] + sm.sRow[1][0][r];
      const float db = sm.sRow[0][1][r] + sm.sRow[1][1][r];
      const float dbeta = sm.sRow[0][2][r] + sm.sRow[1][2][r] + sm.sRow[0][3][r] + sm.sRow[1][3][r];
      const float zd = ok ? z * dec : 0.f;
      const float zsum = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_prefix_sum(zd)), 63));
      float dG = keepf(rows - cols + db - zd, ok); // db carries its factor exp(G)
      float sd = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) sd += sm.sred[q];
      if (r == len - 1) dG += __expf(glast) * sd + zsum; // gamma = exp(G_last)
      const float xs = wave_prefix_sum(dG);
      if (hh < GRAD_MAXG) {
        sm.sDGB[hh][0][r] = xs;
        sm.sDGB[hh][1][r] = dbeta;
      } else if (ok) {
        a.dg[(size_t)(t0 + r) * a.HV + h] = xs;
        a.dbeta[(size_t)(t0 + r) * a.HV + h] = dbeta;
      }
    }
    if (!DET) {
#pragma unroll
      for (int t = 0; t < NT2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = row0 + lg * 4 + i, dk = 16 * (half * NT2 + t) + lr;
          if (r < len) {
            atomicAdd(a.dqacc + ((size_t)(t0 + r) * a.H + j) * D + dk, dQacc[t][i]);
            atomicAdd(a.dkacc + ((size_t)(t0 + r) * a.H + j) * D + dk, dKacc[t][i]);
          }
        }
    }
    if (hh + 1 < h_count) {
      __syncthreads(); // this head's tail is done with the shared tiles
      store_head(len, tid);
    }
  }
  load_kq(t0_n, len_n, j_n, tid); // the next item's K, Q rows and norms, in flight during the epilogue

  // dg, dbeta of the heads held in LDS (the last head's are visible after one more barrier)
  __syncthreads();
  for (int idx = tid; idx < min(h_count, GRAD_MAXG) * 2 * CH; idx += GRAD_THREADS) {
    const int hh = idx / (2 * CH), k = (idx / CH) & 1, r = idx % CH;
    if (r < len) (k ? a.dbeta : a.dg)[(size_t)(t0 + r) * a.HV + h_first + hh] = sm.sDGB[hh][k][r];
  }
  if (DET) {
    // L2-norm backward of the group sums: dx = r (dxh - xh (xh . dxh)), xh = r x
    TI* dqp = (TI*)a.dq;
    TI* dkp = (TI*)a.dk;
    float qd[4] = {0.f, 0.f, 0.f, 0.f}, kd[4] = {0.f, 0.f, 0.f, 0.f};
    const f32x4 rk_r = rk4(), rq_r = rq4();
    if (a.l2norm) {
#pragma unroll
      for (int t = 0; t < NT2; ++t) {
        const bf16x4 qv = lds_tr4c(sm.sQ, SK, row0, 16 * (half * NT2 + t));
        const bf16x4 kv4 = lds_tr4c(sm.sK, SK, row0, 16 * (half * NT2 + t));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qd[i] += rq_r[i] * (float)qv[i] * dQacc[t][i];
          kd[i] += rk_r[i] * (float)kv4[i] * dKacc[t][i];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qd[i] = row_sum16(qd[i]);
        kd[i] = row_sum16(kd[i]);
      }
      __syncthreads();
      if (lr == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm.sRow[half][0][row0 + lg * 4 + i] = qd[i];
          sm.sRow[half][1][row0 + lg * 4 + i] = kd[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + lg * 4 + i;
        qd[i] = sm.sRow[0][0][r] + sm.sRow[1][0][r];
        kd[i] = sm.sRow[0][1][r] + sm.sRow[1][1][r];
      }
    }
#pragma unroll
    for (int t = 0; t < NT2; ++t) {
      const int dk = 16 * (half * NT2 + t) + lr;
      const bf16x4 qv = lds_tr4c(sm.sQ, SK, row0, 16 * (half * NT2 + t));
      const bf16x4 kv4 = lds_tr4c(sm.sK, SK, row0, 16 * (half * NT2 + t));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + lg * 4 + i;
        float dqv = dQacc[t][i], dkv = dKacc[t][i];
        if (a.l2norm) { // (rows past the chunk's end hold zeros in LDS and are not stored)
          dqv = rq_r[i] * (dqv - rq_r[i] * (float)qv[i] * qd[i]);
          dkv = rk_r[i] * (dkv - rk_r[i] * (float)kv4[i] * kd[i]);
        }
        if (r >= len) continue;
        IO<TI>::store1(dqp + ((size_t)(t0 + r) * a.H + j) * D + dk, dqv);
        IO<TI>::store1(dkp + ((size_t)(t0 + r) * a.H + j) * D + dk, dkv);
      }
    }
  }
  if (!has_next) break;
  __syncthreads(); // the epilogue's reads of K, Q, the norms and the row sums are done
  item = item_n;
  c = c_n;
  j = j_n;
  h_first = hf_n;
  len = len_n;
  t0 = t0_n;
  }
}

template <int D, typename TI>
static int chunk_grad_t(const Args& a, int det, hipStream_t s) {
  if (a.c_count == 0) return 0;
  // One persistent workgroup per resident slot (CUs x workgroups per CU), found once per kernel
  // instance (this template's D and io type, the reduction mode) and device.
  constexpr int kMaxDev = 64;
  static std::atomic<int> slots[2][kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return (int)hipErrorInvalidDevice;
  int n = dev < kMaxDev ? slots[det][dev].load(std::memory_order_relaxed) : 0;
  if (n == 0) {
    int ncu = 0, per = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return (int)hipErrorInvalidDevice;
    const hipError_t e = det ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_chunk_grad<D, TI, true>, GRAD_THREADS, 0)
                             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_chunk_grad<D, TI, false>, GRAD_THREADS, 0);
    if (e != hipSuccess) return (int)e;
    n = ncu * (per > 0 ? per : 1);
    if (dev < kMaxDev) slots[det][dev].store(n, std::memory_order_relaxed);
  }
  const long items = (long)a.c_count * (det ? a.H : a.HV);
  const dim3 grid((unsigned)(items < n ? items : n));
  if (det) hipLaunchKernelGGL((k_chunk_grad<D, TI, true>), grid, dim3(GRAD_THREADS), 0, s, a);
  else hipLaunchKernelGGL((k_chunk_grad<D, TI, false>), grid, dim3(GRAD_THREADS), 0, s, a);
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
    const float r = rn[which][(row % a.H) * a.T + row / a.H]; // norms are head-major
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
