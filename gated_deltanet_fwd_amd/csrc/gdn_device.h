// Device-side building blocks for the gfx950 (CDNA4) kernels: bf16 MFMA tiles, io loads,
// wave shuffles. Wave size is 64; every kernel runs 256 threads = 4 waves.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;        // chunk length (tokens)
constexpr int NTHREADS = 256; // threads per workgroup
constexpr int PAD = 8;        // bf16 elements of row padding in LDS tiles (keeps 16-byte rows aligned)

// v_mfma_f32_16x16x32_bf16: C[16x16] += A[16x32] B[32x16].
// Lane l holds A[l % 16][(l / 16) * 8 + e] and B[(l / 16) * 8 + e][l % 16] for e = 0..7, and
// C[(l / 16) * 4 + i][l % 16] for i = 0..3 (layout checked on gfx950 by a lane probe).
__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
  return z;
}

// v if keep, else zeros; f if keep, else 0. The mask is opaque to the compiler, so a value that
// was just loaded stays an unconditional load (a select on it lets the compiler move the load
// into a branch, and the branch's join then waits for every outstanding load).
__device__ __forceinline__ bf16x8 keep8(bf16x8 v, bool keep) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  unsigned m = keep ? ~0u : 0u;
  asm volatile("" : "+v"(m));
  return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) & m);
}
__device__ __forceinline__ float keepf(float f, bool keep) {
  unsigned m = keep ? ~0u : 0u;
  asm volatile("" : "+v"(m));
  return __builtin_bit_cast(float, __builtin_bit_cast(unsigned, f) & m);
}

// Fragment read from an LDS tile stored row-major with `stride` elements per row:
// 8 consecutive elements of row `row` starting at column `col` (16-byte aligned).
__device__ __forceinline__ bf16x8 lds8(const bf16* base, int stride, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(base + row * stride + col);
}

// Transposed fragment read from an LDS tile stored row-major as tile[k][m] (m contiguous,
// `stride` elements per row, rows 8-byte aligned): lane l receives tile[k0 + (l/16)*8 + e][m0 + l%16]
// for e = 0..7, i.e. an MFMA A (or B) fragment of the transposed tile. Uses ds_read_b64_tr_b16,
// which hands lane i of each 16-lane group element i%4 of the 8-byte blocks addressed by lanes
// i/4, i/4+4, i/4+8, i/4+12 of that group (layout checked on gfx950 by a lane probe).
__device__ __forceinline__ bf16x8 lds_tr8(const bf16* tile, int stride, int k0, int m0) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, j = l & 15;
  const bf16* p0 = tile + (k0 + g * 8 + (j >> 2)) * stride + m0 + 4 * (j & 3);
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 4 * stride));
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// C-layout read of a 16x16 block of a row-major LDS tile: lane l receives
// tile[r0 + (l/16)*4 + i][c0 + l%16] for i = 0..3 (the layout of an MFMA result tile), with one
// transpose-read per lane.
__device__ __forceinline__ bf16x4 lds_tr4c(const bf16* tile, int stride, int r0, int c0) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, j = l & 15;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(tile + (r0 + 4 * g + (j >> 2)) * stride + c0 + 4 * (j & 3)));
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, v);
}

// MFMA B operand (32 rows of k, 16 columns) from the two 16x16 result tiles that hold rows
// [0, 16) and [16, 32) of that k range, without LDS. A result tile gives lane l rows
// (l/16)*4 .. +3; the B operand wants rows (l/16)*8 .. +7. With the four 16-lane groups of t0 and
// t1 written G0..G3, permlane32_swap(t0, t1) yields (t0.G0 t0.G1 t1.G0 t1.G1 | t0.G2 t0.G3 t1.G2
// t1.G3) and permlane16_swap of those yields (t0.G0 t0.G2 t1.G0 t1.G2 | t0.G1 t0.G3 t1.G1 t1.G3):
// the low and high 4-row halves of every group's 8 rows (swap semantics checked on gfx950 by a
// lane probe).
__device__ __forceinline__ bf16x8 c_to_b(const f32x4& t0, const f32x4& t1) {
  const unsigned a0 = pack_bf16x2(t0[0], t0[1]), a1 = pack_bf16x2(t0[2], t0[3]);
  const unsigned b0 = pack_bf16x2(t1[0], t1[1]), b1 = pack_bf16x2(t1[2], t1[3]);
  const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  const auto u0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
  const auto u1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r;
  r[0] = u0[0];
  r[1] = u1[0];
  r[2] = u0[1];
  r[3] = u1[1];
  return __builtin_bit_cast(bf16x8, r);
}

// ---------------------------------------------------------------------------------------
// k-permuted fragments. An MFMA sums over its 32 k values in any order, as long as the A and B
// operands agree on it. The fragments below give lane group g (= lane / 16) the k values
// 4g .. 4g+3 and 16+4g .. 16+4g+3 of a 32-wide k block, in that order. With that order the two
// 16x16 result tiles holding k rows [0, 16) and [16, 32) become a B (or A) operand by packing
// alone: a result tile gives lane group g rows 4g .. 4g+3.

// B (or A) operand from two result tiles, t0 = k rows [0, 16), t1 = k rows [16, 32).
__device__ __forceinline__ bf16x8 pack_kp(const f32x4& t0, const f32x4& t1) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r;
  r[0] = pack_bf16x2(t0[0], t0[1]);
  r[1] = pack_bf16x2(t0[2], t0[3]);
  r[2] = pack_bf16x2(t1[0], t1[1]);
  r[3] = pack_bf16x2(t1[2], t1[3]);
  return __builtin_bit_cast(bf16x8, r);
}

// Staging store of 8 consecutive columns [8 q, 8 q + 8) of a row (q = piece index within the row)
// into a tile kept column-permuted within each 32-column block, so that lds8 at column 32 b + 8 g
// returns the k-permuted fragment of block b. Column c of a block sits at position
// 8 ((c % 16) / 4) + 4 (c / 16) + c % 4; a piece splits into two 8-byte writes.
__device__ __forceinline__ void lds_store_kp8(bf16* tile, int stride, int row, int q, const bf16x8& v) {
  const int qq = q & 3;
  bf16* p = tile + row * stride + 32 * (q >> 2) + 16 * (qq & 1) + 4 * (qq >> 1);
  *reinterpret_cast<bf16x4*>(p) = bf16x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<bf16x4*>(p + 8) = bf16x4{v[4], v[5], v[6], v[7]};
}

// Operand whose rows are m (lane % 16) and whose k runs along a row-major LDS tile's row:
// tile[row][k0 + k] in k-permuted order (two 8-byte reads).
__device__ __forceinline__ bf16x8 lds_kp(const bf16* tile, int stride, int row, int k0) {
  const int g = (threadIdx.x & 63) >> 4;
  const bf16* p = tile + row * stride + k0 + 4 * g;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Operand whose k runs down a row-major LDS tile's columns: lane receives tile[k0 + k][m0 + lane % 16]
// in k-permuted order (two transpose-reads; see lds_tr8 for the instruction's lane mapping).
__device__ __forceinline__ bf16x8 lds_tr_kp(const bf16* tile, int stride, int k0, int m0) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, j = l & 15;
  const bf16* p0 = tile + (k0 + 4 * g + (j >> 2)) * stride + m0 + 4 * (j & 3);
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 16 * stride));
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Store 4 values of one column, rows r..r+3, into an LDS tile stored transposed
// (tile[col][row]): one 8-byte write.
__device__ __forceinline__ void lds_store4_t(bf16* base, int stride, int col, int row, float a, float b, float c,
                                             float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(base + col * stride + row) = v;
}

// Raw buffer resource over [base, base + bytes) (gfx9 word 3). A buffer store whose offset lies
// past the end is dropped by the hardware, so lanes past a chunk's end store without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
// 16-byte buffer load at a byte offset; bytes past the resource's end read as zero.
__device__ __forceinline__ i32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, int off_bytes) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off_bytes, 0, 0);
}
__device__ __forceinline__ void buf_store16(const bf16x8& v, __amdgpu_buffer_rsrc_t r, int off_bytes) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off_bytes, 0, 0);
}

// ---------------------------------------------------------------------------------------
// io dtype access (bf16 or f32)

template <typename T>
struct IO;

template <>
struct IO<bf16> {
  static __device__ __forceinline__ void load8f(const bf16* p, float out[8]) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
  }
  static __device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  // 8 consecutive values through a buffer resource (zeros past its end); off in elements
  static __device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(bf16x8, buf_load16(r, off * 2));
  }
  // 4 consecutive values through a buffer resource (dropped past its end); off in elements
  static __device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, int off, const float x[4]) {
    i32x2_t v;
    v[0] = (int)pack_bf16x2(x[0], x[1]);
    v[1] = (int)pack_bf16x2(x[2], x[3]);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off * 2, 0, 0);
  }
  static __device__ __forceinline__ float load1(const bf16* p) { return (float)*p; }
  static __device__ __forceinline__ void store1(bf16* p, float x) { *p = (bf16)x; }
  // 4 consecutive values (8-byte aligned)
  static __device__ __forceinline__ void store4(bf16* p, const float x[4]) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  }
};

template <>
struct IO<float> {
  static __device__ __forceinline__ void load8f(const float* p, float out[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
  static __device__ __forceinline__ bf16x8 load8(const float* p) {
    float f[8];
    load8f(p, f);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)f[e];
    return r;
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, int off) {
    const float4 a = __builtin_bit_cast(float4, buf_load16(r, off * 4));
    const float4 b = __builtin_bit_cast(float4, buf_load16(r, off * 4 + 16));
    bf16x8 v;
    v[0] = (bf16)a.x; v[1] = (bf16)a.y; v[2] = (bf16)a.z; v[3] = (bf16)a.w;
    v[4] = (bf16)b.x; v[5] = (bf16)b.y; v[6] = (bf16)b.z; v[7] = (bf16)b.w;
    return v;
  }
  static __device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, int off, const float x[4]) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, make_float4(x[0], x[1], x[2], x[3])), r,
                                           off * 4, 0, 0);
  }
  static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
  // 4 consecutive values (16-byte aligned)
  static __device__ __forceinline__ void store4(float* p, const float x[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

// Sum over the 16 lanes that share l / 16 (the lanes of one MFMA output row group).
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

// Sum over the 16 lanes of each row (lanes with equal l / 16), in every lane: DPP row rotations,
// no LDS traffic.
__device__ __forceinline__ float row_sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave (lane l gets the sum over lanes 0..l):
// Hillis-Steele shifts within 16-lane rows, then DPP broadcasts of lane 15 into rows 1 and 3 and
// of lane 31 into rows 2 and 3. Lanes whose DPP source is absent add the zero "old" operand.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
  return x;
}

// Sum over the four 16-lane rows (lanes with equal l % 16), in every lane. (The lane-swap
// instructions are not used here: with one value as both operands the compiler folds them away.)
__device__ __forceinline__ float col_sum4(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Chain index -> (document rank, q/k head, v head within the group, value tile), with
// workgroups that read the same q/k tiles placed on the same XCD. Workgroups are dealt to
// the 8 XCDs round-robin by workgroup id, so a group of GS chains (one q/k head of one
// document: its G value heads times the value tiles) gets ids that agree mod 8; groups are
// taken 8 at a time in longest-document-first order.
struct ChainMap {
  int rank, j, gi, tile;
  bool valid;
};
__device__ __forceinline__ ChainMap decode_chain(int b, const Args& a, int ntile) {
  const int H = a.H, GS = a.G * ntile;
  const int sg = b / (8 * GS);
  const int rem = b - sg * 8 * GS;
  const int x = rem & 7;
  const int s = rem >> 3;
  const long group = (long)a.grp_off + (long)sg * 8 + x; // (rank, j) in rank-major order
  ChainMap m;
  m.valid = group < (long)a.grp_end;
  const int grp = (int)group;
  m.rank = grp / H;
  m.j = grp - m.rank * H;
  m.gi = s / ntile;
  m.tile = s - m.gi * ntile;
  return m;
}

// Chunk processed by workgroup x of a chunk-parallel launch (see Args::c_base).
__device__ __forceinline__ int launch_chunk(const Args& a, int x) {
  return a.c_base + x + (x >= a.c_skip_at ? a.c_skip : 0);
}

} // namespace gdn
