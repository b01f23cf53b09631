// Short causal conv1d + SiLU front-end on gfx950: the depthwise causal convolution of each
// channel within each document, plus bias, then SiLU, over the packed q/k/v channels (the pages
// run it with the gated delta rule on every call of their shape B23: flashinfer PR #8542
// "Conventions"; the conv1d + SiLU training backend of flashinfer PR #7117):
//
//   pre[t, c] = bias[c] + sum_{i<W} weight[c, i] x[t - (W-1) + i, c]   (x = 0 before t's document)
//   y[t, c]   = SiLU(pre[t, c])
//
// and its backward (dpre = dy SiLU'(pre); dx[t] = sum_i weight[i] dpre[t + (W-1) - i] within the
// document; dweight[c, i] = sum_t dpre[t, c] x[t - (W-1) + i, c]; dbias[c] = sum_t dpre[t, c]).
//
// x and y (and dy, dx) are streamed once. A lane owns CONV_CPL consecutive channels (an 8-byte
// bf16 row piece), a wave 64 * CONV_CPL channels and a run of CONV_TB tokens, which it walks in
// order keeping the window's last W - 1 inputs (and, backward, the last W values of dpre) in a
// register buffer indexed at compile time; a document boundary inside the run is the same token for
// every lane (uniform branch). With a full-precision division in SiLU and a history shifted token
// by token the kernels were bound by VALU issue (FP32 runs unpacked here), so the sigmoid uses the
// hardware reciprocal and the window only moves once per CONV_U tokens. The output channels are
// split into up to 4 tensors (q, k, v) as they are written, so the gated delta rule reads them
// without a copy. The weight and bias gradients are summed per wave in registers, over the 4 waves
// of a workgroup in LDS, and over the workgroups in a fixed order by a second kernel: the result
// is deterministic.
#include "gdn_device.h"

namespace gdn {

constexpr int CONV_TB = 128;      // tokens per wave
constexpr int CONV_WAVES = 4;     // waves per workgroup (consecutive token runs, same channels)
constexpr int CONV_U = 8;         // tokens whose loads are issued together
constexpr int CONV_CPL = 4;       // consecutive channels per lane (a wave covers 64 * CONV_CPL)


// N consecutive channels of one token row, as floats (N = 4 or 8; 8- or 16-byte aligned pieces).
template <typename TI, int N>
__device__ __forceinline__ void loadrow(const TI* p, float v[N]) {
  if constexpr (N == 8) {
    IO<TI>::load8f(p, v);
  } else if constexpr (sizeof(TI) == 2) {
    const bf16x4 r = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (float)r[e];
  } else {
    const float4 r = *reinterpret_cast<const float4*>(p);
    v[0] = r.x, v[1] = r.y, v[2] = r.z, v[3] = r.w;
  }
}

template <typename TI, int N>
__device__ __forceinline__ void storerow(TI* p, const float v[N]) {
  if constexpr (sizeof(TI) == 2) {
    typedef __bf16 vec_t __attribute__((ext_vector_type(N)));
    vec_t r;
#pragma unroll
    for (int e = 0; e < N; ++e) r[e] = (bf16)v[e];
    *reinterpret_cast<vec_t*>(p) = r;
  } else {
#pragma unroll
    for (int q = 0; q < N / 4; ++q)
      reinterpret_cast<float4*>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
}

// SiLU and its derivative with the hardware reciprocal (about 1 ulp) in place of a full-precision
// division: the outputs are rounded to the input type (or compared at 1e-2) afterwards.
__device__ __forceinline__ float sigmoid_f(float p) { return __builtin_amdgcn_rcpf(1.f + __expf(-p)); }
__device__ __forceinline__ float silu_f(float p) { return p * sigmoid_f(p); }
__device__ __forceinline__ float silu_grad(float p) {
  const float s = sigmoid_f(p);
  return s * (1.f + p * (1.f - s));
}

// Document of token t: the largest n with cu[n] <= t (empty documents are skipped over).
__device__ __forceinline__ int doc_of(const int32_t* cu, int N, int64_t t) {
  int lo = 0, hi = N; // cu[lo] <= t < cu[hi] (t < T = cu[N])
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The window slides over a register buffer indexed by compile-time positions: for a step of
// CONV_U tokens starting at t, xb[j] holds x[t - (W-1) + j], so token t + u reads xb[u .. u+W-1]
// and only the last W - 1 rows move at the end of the step.
template <typename TI, int W, bool SILU>
__global__ __launch_bounds__(64 * CONV_WAVES) void k_conv_fwd(ConvArgs a) {
  constexpr int H = W - 1, NB = H + CONV_U;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c0 = blockIdx.x * (64 * CONV_CPL) + CONV_CPL * lane;
  const int64_t t_begin = ((int64_t)blockIdx.y * CONV_WAVES + wv) * CONV_TB;
  if (c0 >= a.C || t_begin >= a.T) return;
  const int64_t t_end = min(t_begin + CONV_TB, a.T);
  const TI* x = (const TI*)a.x + c0;
  // output group of this lane's channels
  int g = 0;
#pragma unroll
  for (int k = 1; k < 4; ++k) g += (k < a.n_groups && c0 >= a.goff[k]) ? 1 : 0;
  const int Cg = a.goff[g + 1] - a.goff[g];
  TI* y = (TI*)a.y[g] + (c0 - a.goff[g]);
  float wt[CONV_CPL][W], bs[CONV_CPL];
#pragma unroll
  for (int e = 0; e < CONV_CPL; ++e) {
#pragma unroll
    for (int i = 0; i < W; ++i) wt[e][i] = a.w[(size_t)(c0 + e) * W + i];
    bs[e] = a.b ? a.b[c0 + e] : 0.f;
  }
  int n = doc_of(a.cu, a.N, t_begin);
  int64_t d_next = a.cu[n + 1];
  const int64_t d_start = a.cu[n];
  float xb[NB][CONV_CPL];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int64_t tt = t_begin - H + j;
    if (tt >= d_start) loadrow<TI, CONV_CPL>(x + tt * a.C, xb[j]);
    else {
#pragma unroll
      for (int e = 0; e < CONV_CPL; ++e) xb[j][e] = 0.f;
    }
  }
  for (int64_t t = t_begin; t < t_end; t += CONV_U) {
#pragma unroll
    for (int u = 0; u < CONV_U; ++u) loadrow<TI, CONV_CPL>(x + min(t + u, t_end - 1) * a.C, xb[H + u]);
#pragma unroll
    for (int u = 0; u < CONV_U; ++u) {
      const int64_t tu = t + u;
      if (tu >= t_end) break;
      if (tu == d_next) { // a new document starts here (uniform): its window starts empty
        while (a.cu[n + 1] <= tu) ++n;
        d_next = a.cu[n + 1];
#pragma unroll
        for (int j = 0; j < H; ++j)
#pragma unroll
          for (int e = 0; e < CONV_CPL; ++e) xb[u + j][e] = 0.f;
      }
      float out[CONV_CPL];
#pragma unroll
      for (int e = 0; e < CONV_CPL; ++e) {
        float p = bs[e];
#pragma unroll
        for (int i = 0; i < W; ++i) p = __builtin_fmaf(wt[e][i], xb[u + i][e], p);
        out[e] = SILU ? silu_f(p) : p;
      }
      storerow<TI, CONV_CPL>(y + tu * Cg, out);
    }
#pragma unroll
    for (int j = 0; j < H; ++j)
#pragma unroll
      for (int e = 0; e < CONV_CPL; ++e) xb[j][e] = xb[CONV_U + j][e];
  }
}

// Backward over positions [t_begin, t_end + W - 1): the last W - 1 are the halo whose dpre the
// run's last tokens need (zero past the document's end); dx[p - (W-1)] is final once dpre[p] is
// in. As forward, xb[j] = x[t - (W-1) + j] and db[j] = dpre[t - (W-1) + j] for the step at t.
template <typename TI, int W, bool SILU>
__global__ __launch_bounds__(64 * CONV_WAVES) void k_conv_bwd(ConvArgs a) {
  constexpr int NP = W + 1; // dweight taps and dbias per channel
  constexpr int H = W - 1, NB = H + CONV_U;
  __shared__ float sred[CONV_WAVES][64][CONV_CPL * NP + 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c0 = blockIdx.x * (64 * CONV_CPL) + CONV_CPL * lane;
  const int64_t t_begin = ((int64_t)blockIdx.y * CONV_WAVES + wv) * CONV_TB;
  const bool active = c0 < a.C && t_begin < a.T;
  float acc[CONV_CPL][NP];
#pragma unroll
  for (int e = 0; e < CONV_CPL; ++e)
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[e][i] = 0.f;
  if (active) {
    const int64_t t_end = min(t_begin + CONV_TB, a.T);
    const TI* x = (const TI*)a.x + c0;
    TI* dx = (TI*)a.dx + c0;
    int g = 0;
#pragma unroll
    for (int k = 1; k < 4; ++k) g += (k < a.n_groups && c0 >= a.goff[k]) ? 1 : 0;
    const int Cg = a.goff[g + 1] - a.goff[g];
    const TI* dy = (const TI*)a.dy[g] + (c0 - a.goff[g]);
    float wt[CONV_CPL][W], bs[CONV_CPL];
#pragma unroll
    for (int e = 0; e < CONV_CPL; ++e) {
#pragma unroll
      for (int i = 0; i < W; ++i) wt[e][i] = a.w[(size_t)(c0 + e) * W + i];
      bs[e] = a.b ? a.b[c0 + e] : 0.f;
    }
    int n = doc_of(a.cu, a.N, t_begin);
    int64_t d_start = a.cu[n], d_next = a.cu[n + 1];
    float xb[NB][CONV_CPL], db[NB][CONV_CPL];
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int64_t tt = t_begin - H + j;
      if (tt >= d_start) loadrow<TI, CONV_CPL>(x + tt * a.C, xb[j]);
      else {
#pragma unroll
        for (int e = 0; e < CONV_CPL; ++e) xb[j][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < CONV_CPL; ++e) db[j][e] = 0.f;
    }
    const int64_t u_end = t_end + H;
    for (int64_t t = t_begin; t < u_end; t += CONV_U) {
      float gr[CONV_U][CONV_CPL];
#pragma unroll
      for (int u = 0; u < CONV_U; ++u) {
        const int64_t tl = min(t + u, a.T - 1);
        loadrow<TI, CONV_CPL>(x + tl * a.C, xb[H + u]);
        loadrow<TI, CONV_CPL>(dy + tl * Cg, gr[u]);
      }
#pragma unroll
      for (int u = 0; u < CONV_U; ++u) {
        const int64_t tu = t + u;
        if (tu >= u_end) break;
        if (tu == d_next && tu < t_end) {
          // a new document starts at tu (uniform): finish the previous document's last W - 1
          // positions with that document's dpre only, then start empty
#pragma unroll
          for (int j = 1; j < W; ++j) {
            const int64_t tp = tu - j;
            if (tp >= t_begin && tp >= d_start) {
              float o[CONV_CPL];
#pragma unroll
              for (int e = 0; e < CONV_CPL; ++e) {
                float s = 0.f;
#pragma unroll
                for (int i = W - j; i < W; ++i) s = __builtin_fmaf(wt[e][i], db[u + 2 * H - i - j][e], s);
                o[e] = s;
              }
              storerow<TI, CONV_CPL>(dx + tp * a.C, o);
            }
          }
          while (a.cu[n + 1] <= tu) ++n;
          d_start = tu;
          d_next = a.cu[n + 1];
#pragma unroll
          for (int j = 0; j < H; ++j)
#pragma unroll
            for (int e = 0; e < CONV_CPL; ++e) {
              xb[u + j][e] = 0.f;
              db[u + j][e] = 0.f;
            }
        }
        // dpre at tu: zero in the halo past the document's end (or the problem's)
        const bool live = tu < d_next;
        float dp[CONV_CPL];
#pragma unroll
        for (int e = 0; e < CONV_CPL; ++e) {
          if (!live) xb[u + H][e] = 0.f;
          float p = bs[e];
#pragma unroll
          for (int i = 0; i < W; ++i) p = __builtin_fmaf(wt[e][i], xb[u + i][e], p);
          const float d = SILU ? gr[u][e] * silu_grad(p) : gr[u][e];
          dp[e] = live ? d : 0.f;
          db[u + H][e] = dp[e];
        }
        if (tu < t_end) {
#pragma unroll
          for (int e = 0; e < CONV_CPL; ++e) {
#pragma unroll
            for (int i = 0; i < W; ++i) acc[e][i] = __builtin_fmaf(dp[e], xb[u + i][e], acc[e][i]);
            acc[e][W] += dp[e];
          }
        }
        const int64_t tf = tu - H; // position whose dx is now complete
        if (tf >= t_begin && tf >= d_start && tf < t_end) {
          float o[CONV_CPL];
#pragma unroll
          for (int e = 0; e < CONV_CPL; ++e) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < W; ++i) s = __builtin_fmaf(wt[e][i], db[u + H - i][e], s);
            o[e] = s;
          }
          storerow<TI, CONV_CPL>(dx + tf * a.C, o);
        }
      }
#pragma unroll
      for (int j = 0; j < H; ++j)
#pragma unroll
        for (int e = 0; e < CONV_CPL; ++e) {
          xb[j][e] = xb[CONV_U + j][e];
          db[j][e] = db[CONV_U + j][e];
        }
    }
  }
  // weight and bias gradients: the 4 waves' sums in LDS, added in wave order by wave 0
#pragma unroll
  for (int e = 0; e < CONV_CPL; ++e)
#pragma unroll
    for (int i = 0; i < NP; ++i) sred[wv][lane][e * NP + i] = acc[e][i];
  __syncthreads();
  if (wv == 0 && c0 < a.C) {
    float* dst = a.part + ((size_t)blockIdx.y * a.C + c0) * NP;
#pragma unroll
    for (int k = 0; k < CONV_CPL * NP; ++k) {
      float s = sred[0][lane][k];
#pragma unroll
      for (int q = 1; q < CONV_WAVES; ++q) s += sred[q][lane][k];
      dst[k] = s;
    }
  }
}

// dweight[c][i] and dbias[c]: the workgroups' partial sums, added in workgroup order.
__global__ __launch_bounds__(256) void k_conv_reduce(ConvArgs a, int blocks) {
  const int NP = a.W + 1;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.C * NP) return;
  float s = 0.f;
  for (int b = 0; b < blocks; ++b) s += a.part[(size_t)b * a.C * NP + idx];
  const int c = idx / NP, i = idx - c * NP;
  if (i < a.W) a.dw[(size_t)c * a.W + i] = s;
  else if (a.db) a.db[c] = s;
}

int conv_blocks(int64_t T) { return (int)((T + (int64_t)CONV_TB * CONV_WAVES - 1) / ((int64_t)CONV_TB * CONV_WAVES)); }

template <typename TI>
static int conv_fwd_t(const ConvArgs& a, hipStream_t s) {
  const dim3 grid((a.C + 64 * CONV_CPL - 1) / (64 * CONV_CPL), conv_blocks(a.T)), blk(64 * CONV_WAVES);
  switch (a.W * 2 + (a.silu ? 1 : 0)) {
    case 2: hipLaunchKernelGGL((k_conv_fwd<TI, 1, false>), grid, blk, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_conv_fwd<TI, 1, true>), grid, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_conv_fwd<TI, 2, false>), grid, blk, 0, s, a); break;
    case 5: hipLaunchKernelGGL((k_conv_fwd<TI, 2, true>), grid, blk, 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_conv_fwd<TI, 3, false>), grid, blk, 0, s, a); break;
    case 7: hipLaunchKernelGGL((k_conv_fwd<TI, 3, true>), grid, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_conv_fwd<TI, 4, false>), grid, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k_conv_fwd<TI, 4, true>), grid, blk, 0, s, a); break;
  }
  return (int)hipGetLastError();
}

template <typename TI>
static int conv_bwd_t(const ConvArgs& a, hipStream_t s) {
  const int blocks = conv_blocks(a.T);
  const dim3 grid((a.C + 64 * CONV_CPL - 1) / (64 * CONV_CPL), blocks), blk(64 * CONV_WAVES);
  switch (a.W * 2 + (a.silu ? 1 : 0)) {
    case 2: hipLaunchKernelGGL((k_conv_bwd<TI, 1, false>), grid, blk, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_conv_bwd<TI, 1, true>), grid, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_conv_bwd<TI, 2, false>), grid, blk, 0, s, a); break;
    case 5: hipLaunchKernelGGL((k_conv_bwd<TI, 2, true>), grid, blk, 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_conv_bwd<TI, 3, false>), grid, blk, 0, s, a); break;
    case 7: hipLaunchKernelGGL((k_conv_bwd<TI, 3, true>), grid, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_conv_bwd<TI, 4, false>), grid, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k_conv_bwd<TI, 4, true>), grid, blk, 0, s, a); break;
  }
  int e = (int)hipGetLastError();
  if (e) return e;
  const int n = a.C * (a.W + 1);
  hipLaunchKernelGGL(k_conv_reduce, dim3((n + 255) / 256), dim3(256), 0, s, a, blocks);
  return (int)hipGetLastError();
}

int launch_conv_fwd(const ConvArgs& a, int dtype, void* stream) {
  if (a.T == 0) return 0;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return dtype == 0 ? conv_fwd_t<bf16>(a, s) : conv_fwd_t<float>(a, s);
}

int launch_conv_bwd(const ConvArgs& a, int dtype, void* stream) {
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.T == 0) { // no tokens: the weight and bias gradients are zero
    const int n = a.C * (a.W + 1);
    ConvArgs z = a;
    hipLaunchKernelGGL(k_conv_reduce, dim3((n + 255) / 256), dim3(256), 0, s, z, 0);
    return (int)hipGetLastError();
  }
  return dtype == 0 ? conv_bwd_t<bf16>(a, s) : conv_bwd_t<float>(a, s);
}

} // namespace gdn
