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
// HBM-bound: x and y (and dy, dx) are streamed once. A lane owns 8 consecutive channels (one
// 16-byte row piece), a wave 512 channels and a run of CONV_TB tokens, which it walks in order
// keeping the window's last W - 1 inputs (and, backward, the last W values of dpre) in registers;
// a document boundary inside the run is the same token for every lane (uniform branch). The
// output channels are split into up to 4 tensors (q, k, v) as they are written, so the gated
// delta rule reads them without a copy. The weight and bias gradients are summed per wave in
// registers, over the 4 waves of a workgroup in LDS, and over the workgroups in a fixed order by
// a second kernel: the result is deterministic.
#include "gdn_device.h"

namespace gdn {

constexpr int CONV_TB = 256;      // tokens per wave
constexpr int CONV_WAVES = 4;     // waves per workgroup (consecutive token runs, same channels)
constexpr int CONV_U = 4;         // tokens whose loads are issued together


template <typename TI>
__device__ __forceinline__ void load8row(const TI* p, float v[8]) {
  IO<TI>::load8f(p, v);
}

template <typename TI>
__device__ __forceinline__ void store8row(TI* p, const float v[8]);
template <>
__device__ __forceinline__ void store8row<bf16>(bf16* p, const float v[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  *reinterpret_cast<bf16x8*>(p) = r;
}
template <>
__device__ __forceinline__ void store8row<float>(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ float silu_f(float p) { return p / (1.f + __expf(-p)); }
__device__ __forceinline__ float silu_grad(float p) {
  const float s = 1.f / (1.f + __expf(-p));
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

template <typename TI, int W>
__global__ __launch_bounds__(64 * CONV_WAVES) void k_conv_fwd(ConvArgs a) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 512 + 8 * lane;
  const int64_t t_begin = ((int64_t)blockIdx.y * CONV_WAVES + wv) * CONV_TB;
  if (c0 >= a.C || t_begin >= a.T) return;
  const int64_t t_end = min(t_begin + CONV_TB, a.T);
  const TI* x = (const TI*)a.x;
  // output group of this lane's channels
  int g = 0;
#pragma unroll
  for (int k = 1; k < 4; ++k) g += (k < a.n_groups && c0 >= a.goff[k]) ? 1 : 0;
  const int Cg = a.goff[g + 1] - a.goff[g];
  TI* y = (TI*)a.y[g] + (c0 - a.goff[g]);
  float wt[8][W], bs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int i = 0; i < W; ++i) wt[e][i] = a.w[(size_t)(c0 + e) * W + i];
    bs[e] = a.b ? a.b[c0 + e] : 0.f;
  }
  // document and window history (hist[j] = x[t - 1 - j])
  int n = doc_of(a.cu, a.N, t_begin);
  int64_t d_start = a.cu[n], d_next = a.cu[n + 1];
  float hist[W > 1 ? W - 1 : 1][8];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int64_t tt = t_begin - 1 - j;
    if (tt >= d_start) load8row<TI>(x + tt * a.C + c0, hist[j]);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hist[j][e] = 0.f;
    }
  }
  for (int64_t t = t_begin; t < t_end; t += CONV_U) {
    float xr[CONV_U][8];
#pragma unroll
    for (int u = 0; u < CONV_U; ++u) load8row<TI>(x + min(t + u, t_end - 1) * a.C + c0, xr[u]);
#pragma unroll
    for (int u = 0; u < CONV_U; ++u) {
      const int64_t tu = t + u;
      if (tu >= t_end) break;
      if (tu == d_next) { // a new document starts here (uniform): empty window history
        while (a.cu[n + 1] <= tu) ++n;
        d_start = tu;
        d_next = a.cu[n + 1];
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) hist[j][e] = 0.f;
      }
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float p = bs[e] + wt[e][W - 1] * xr[u][e];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) p = __builtin_fmaf(wt[e][W - 2 - j], hist[j][e], p);
        out[e] = a.silu ? silu_f(p) : p;
      }
      store8row<TI>(y + tu * Cg, out);
#pragma unroll
      for (int j = W - 2; j > 0; --j)
#pragma unroll
        for (int e = 0; e < 8; ++e) hist[j][e] = hist[j - 1][e];
      if (W > 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) hist[0][e] = xr[u][e];
      }
    }
  }
}

template <typename TI, int W>
__global__ __launch_bounds__(64 * CONV_WAVES) void k_conv_bwd(ConvArgs a) {
  constexpr int NP = W + 1; // dweight taps and dbias per channel
  __shared__ float sred[CONV_WAVES][64][8 * NP + 1];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 512 + 8 * lane;
  const int64_t t_begin = ((int64_t)blockIdx.y * CONV_WAVES + wv) * CONV_TB;
  const bool active = c0 < a.C && t_begin < a.T;
  float acc[8][NP];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[e][i] = 0.f;
  if (active) {
    const int64_t t_end = min(t_begin + CONV_TB, a.T);
    const TI* x = (const TI*)a.x;
    TI* dx = (TI*)a.dx;
    int g = 0;
#pragma unroll
    for (int k = 1; k < 4; ++k) g += (k < a.n_groups && c0 >= a.goff[k]) ? 1 : 0;
    const int Cg = a.goff[g + 1] - a.goff[g];
    const TI* dy = (const TI*)a.dy[g] + (c0 - a.goff[g]);
    float wt[8][W], bs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int i = 0; i < W; ++i) wt[e][i] = a.w[(size_t)(c0 + e) * W + i];
      bs[e] = a.b ? a.b[c0 + e] : 0.f;
    }
    int n = doc_of(a.cu, a.N, t_begin);
    int64_t d_start = a.cu[n], d_next = a.cu[n + 1];
    // hist[j] = x[u - 1 - j]; ring[k] = dpre[u - k] (after position u is pushed)
    float hist[W > 1 ? W - 1 : 1][8], ring[W][8];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int64_t tt = t_begin - 1 - j;
      if (tt >= d_start) load8row<TI>(x + tt * a.C + c0, hist[j]);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) hist[j][e] = 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) ring[k][e] = 0.f;
    // Positions u in [t_begin, t_end + W - 1): the last W - 1 are the halo whose dpre the run's
    // last tokens need (zero past the document's end); dx[u - (W - 1)] is final once dpre[u] is in.
    const int64_t u_end = t_end + (W - 1);
    for (int64_t t = t_begin; t < u_end; t += CONV_U) {
      float xr[CONV_U][8], gr[CONV_U][8];
#pragma unroll
      for (int u = 0; u < CONV_U; ++u) {
        const int64_t tl = min(t + u, a.T - 1);
        load8row<TI>(x + tl * a.C + c0, xr[u]);
        load8row<TI>(dy + tl * Cg, gr[u]);
      }
#pragma unroll
      for (int u = 0; u < CONV_U; ++u) {
        const int64_t tu = t + u;
        if (tu >= u_end) break;
        if (tu == d_next && tu < t_end) {
          // a new document starts at tu (uniform): finish the previous document's last W - 1
          // positions with the dpre of that document only, then start empty
#pragma unroll
          for (int j = 1; j < W; ++j) {
            const int64_t tp = tu - j;
            if (tp >= t_begin && tp >= d_start) {
              float o[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                float s = 0.f;
#pragma unroll
                for (int i = W - j; i < W; ++i) s = __builtin_fmaf(wt[e][i], ring[i - (W - j)][e], s);
                o[e] = s;
              }
              store8row<TI>(dx + tp * a.C + c0, o);
            }
          }
          while (a.cu[n + 1] <= tu) ++n;
          d_start = tu;
          d_next = a.cu[n + 1];
#pragma unroll
          for (int j = 0; j < W - 1; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) hist[j][e] = 0.f;
#pragma unroll
          for (int k = 0; k < W; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) ring[k][e] = 0.f;
        }
        // dpre at tu: zero in the halo past the document's end (or the problem's)
        const bool live = tu < d_next;
        const bool own = tu < t_end;
        float dp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float p = bs[e] + wt[e][W - 1] * xr[u][e];
#pragma unroll
          for (int j = 0; j < W - 1; ++j) p = __builtin_fmaf(wt[e][W - 2 - j], hist[j][e], p);
          const float d = a.silu ? gr[u][e] * silu_grad(p) : gr[u][e];
          dp[e] = live ? d : 0.f;
        }
        if (own) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            acc[e][W - 1] = __builtin_fmaf(dp[e], xr[u][e], acc[e][W - 1]);
#pragma unroll
            for (int j = 0; j < W - 1; ++j) acc[e][W - 2 - j] = __builtin_fmaf(dp[e], hist[j][e], acc[e][W - 2 - j]);
            acc[e][W] += dp[e];
          }
        }
#pragma unroll
        for (int k = W - 1; k > 0; --k)
#pragma unroll
          for (int e = 0; e < 8; ++e) ring[k][e] = ring[k - 1][e];
#pragma unroll
        for (int e = 0; e < 8; ++e) ring[0][e] = dp[e];
#pragma unroll
        for (int j = W - 2; j > 0; --j)
#pragma unroll
          for (int e = 0; e < 8; ++e) hist[j][e] = hist[j - 1][e];
        if (W > 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) hist[0][e] = live ? xr[u][e] : 0.f;
        }
        const int64_t tf = tu - (W - 1); // position whose dx is now complete
        if (tf >= t_begin && tf >= d_start && tf < t_end) {
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < W; ++i) s = __builtin_fmaf(wt[e][i], ring[i][e], s);
            o[e] = s;
          }
          store8row<TI>(dx + tf * a.C + c0, o);
        }
      }
    }
  }
  // weight and bias gradients: the 4 waves' sums in LDS, added in wave order by wave 0
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int i = 0; i < NP; ++i) sred[wv][lane][e * NP + i] = acc[e][i];
  __syncthreads();
  if (wv == 0 && c0 < a.C) {
    float* dst = a.part + ((size_t)blockIdx.y * a.C + c0) * NP;
#pragma unroll
    for (int k = 0; k < 8 * NP; ++k) {
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
  const dim3 grid((a.C + 511) / 512, conv_blocks(a.T)), blk(64 * CONV_WAVES);
  switch (a.W) {
    case 1: hipLaunchKernelGGL((k_conv_fwd<TI, 1>), grid, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_conv_fwd<TI, 2>), grid, blk, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_conv_fwd<TI, 3>), grid, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k_conv_fwd<TI, 4>), grid, blk, 0, s, a); break;
  }
  return (int)hipGetLastError();
}

template <typename TI>
static int conv_bwd_t(const ConvArgs& a, hipStream_t s) {
  const int blocks = conv_blocks(a.T);
  const dim3 grid((a.C + 511) / 512, blocks), blk(64 * CONV_WAVES);
  switch (a.W) {
    case 1: hipLaunchKernelGGL((k_conv_bwd<TI, 1>), grid, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_conv_bwd<TI, 2>), grid, blk, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_conv_bwd<TI, 3>), grid, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k_conv_bwd<TI, 4>), grid, blk, 0, s, a); break;
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
