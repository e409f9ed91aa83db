// Device-side building blocks shared by the CARVE kernels (gfx950 / CDNA4).
//
// Matrix products run on the 16x16 MFMA tiles of CDNA4:
//   * bf16 operands: v_mfma_f32_16x16x32_bf16 (one instruction per 32-deep k block)
//   * fp32 operands: v_mfma_f32_16x16x4_f32   (eight instructions per 32-deep k block)
// Both consume a per-lane "fragment" of 8 consecutive k values:
//   A operand (16 x 32):  lane l holds A[l % 16][8 * (l / 16) + j], j = 0..7
//   B operand (32 x 16):  lane l holds B[8 * (l / 16) + j][l % 16]
// and produce the same accumulator layout:
//   C (16 x 16):          lane l holds C[4 * (l / 16) + i][l % 16], i = 0..3
// For the fp32 instruction the eight values of a fragment are fed as eight
// k=4 steps; because A and B fragments use the same k permutation the sum is
// unchanged.  These layouts were checked on gfx950 with a lane-layout probe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace carve {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // four wave64 waves per workgroup
constexpr int kWaves = 4;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Sum over the 16 lanes of each row of the wave (lanes 16 m .. 16 m + 15) by DPP
// row rotations; every lane of the row receives the row's sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return x;
}

// Calls fn(f) for f = wave, wave + NW, ... < F.  When NW divides F every wave runs the
// same iterations with no branch, so memory operations inside stay unconditional (the
// compiler's per-wave memory counters are then exact across loop iterations).
template <int F, int NW, typename Fn>
__device__ __forceinline__ void for_wave_items(int wave, Fn&& fn) {
  if constexpr (F % NW == 0) {
#pragma unroll
    for (int u = 0; u < F / NW; ++u) fn(wave + NW * u);
  } else {
#pragma unroll
    for (int u = 0; u < (F + NW - 1) / NW; ++u)
      if (wave + NW * u < F) fn(wave + NW * u);
  }
}

// Hardware exponential and logarithm (v_exp_f32 / v_log_f32, base 2, about 1 ulp): no
// range reduction or denormal fix-up around them.  Results below float range flush to 0,
// log of 0 (or of a flushed denormal) is -inf; the callers' range logic expects exactly that.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float flog(float x) { return __builtin_amdgcn_logf(x) * 0.6931471805599453f; }

// ------------------------------------------------------------------ fragments
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

// 8 consecutive elements starting at p (16-byte aligned for bf16, 32 for f32)
__device__ __forceinline__ Frag<bf16> load_frag(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> load_frag(const float* p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}
// 8 elements with a stride (used for operands stored with k along rows)
__device__ __forceinline__ Frag<bf16> load_frag_strided(const bf16* p, int stride) {
  Frag<bf16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = p[j * stride];
  return f;
}
__device__ __forceinline__ Frag<float> load_frag_strided(const float* p, int stride) {
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) { f.lo[j] = p[j * stride]; f.hi[j] = p[(j + 4) * stride]; }
  return f;
}

// Fragment of a bf16 matrix M in LDS (row stride ld elements, ld a multiple of 4,
// M 8-byte aligned) whose 8 k values run down 8 consecutive rows:
//   lane l receives M[k0 + 8 (l / 16) + j][c0 + l % 16], j = 0..7.
// Two LDS transpose reads (ds_read_b64_tr_b16) replace eight 2-byte reads.  Within
// each 16-lane group the instruction returns to lane 4a + e the element e of the
// 4-element rows addressed by lanes a, a + 4, a + 8, a + 12 (value i from lane a + 4i);
// so lane s of the group points at row k0 + 8 g + 4 h + s / 4, columns c0 + 4 (s % 4)
// (h = 0 for values 0..3, h = 1 for values 4..7).  Layout checked on gfx950 with a
// lane-layout probe.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ Frag<bf16> lds_frag_tr(const bf16* m, int ld, int c0, int k0) {
  const int lane = lane_id(), s = lane & 15, g = lane >> 4;
  bf16* p = const_cast<bf16*>(m) + (k0 + 8 * g + (s >> 2)) * ld + c0 + 4 * (s & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * ld));
  const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, both);
  return f;
}
// The same fragment for either operand type (fp32: eight strided LDS reads).
__device__ __forceinline__ Frag<bf16> lds_frag_cols(const bf16* m, int ld, int c0, int k0) {
  return lds_frag_tr(m, ld, c0, k0);
}
__device__ __forceinline__ Frag<float> lds_frag_cols(const float* m, int ld, int c0, int k0) {
  const int lane = lane_id();
  return load_frag_strided(m + (k0 + 8 * (lane >> 4)) * ld + c0 + (lane & 15), ld);
}
// element e (0..7) of a fragment
__device__ __forceinline__ bf16 frag_elem(const Frag<bf16>& f, int e) { return f.v[e]; }
__device__ __forceinline__ float frag_elem(const Frag<float>& f, int e) { return e < 4 ? f.lo[e] : f.hi[e - 4]; }
__device__ __forceinline__ Frag<bf16> zero_frag(bf16) {
  Frag<bf16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = (bf16)0.0f;
  return f;
}
__device__ __forceinline__ Frag<float> zero_frag(float) {
  Frag<float> f;
  f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
  f.hi = f.lo;
  return f;
}

__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], c, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], c, 0, 0, 0);
}

// 16 x 16 bf16 tile transposed by one v_mfma_f32_16x16x16_bf16 against the identity.
// That instruction takes A[r][4 g + i] from lane r + 16 g and returns C[4 g + i][c]
// to lane c + 16 g (i = 0..3), so with B = I lane c + 16 g receives X[4 g + i][c] of
// the tile X whose row r, columns 4 g .. 4 g + 3 lane r + 16 g passed in: four rows
// of one column, exactly (products with 1 and 0).
__device__ __forceinline__ bf16x4 transpose_tile16(bf16x4 x_row4) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  i16x4 eye;
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = (4 * g + i == c) ? (short)0x3F80 : (short)0;   // bf16 1.0
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, x_row4), eye, z, 0, 0, 0);
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (bf16)t[i];
  return r;
}

// X[r0 + 4 g + i][c0 + c] (i = 0..3) for lane c + 16 g, of a row-major bf16 matrix in
// LDS (row stride ld, a multiple of 4): the accumulator layout of the tile at (r0, c0),
// from one 8-byte read of row r0 + c, columns c0 + 4 g .. + 3, and a product with the
// identity as above (exact), in place of four 2-byte column reads.
__device__ __forceinline__ f32x4 lds_acc_tile(const bf16* m, int ld, int r0, int c0) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(m + (r0 + c) * ld + c0 + 4 * g);
  i16x4 eye;
#pragma unroll
  for (int i = 0; i < 4; ++i) eye[i] = (4 * g + i == c) ? (short)0x3F80 : (short)0;   // bf16 1.0
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, x), eye, z, 0, 0, 0);
}
__device__ __forceinline__ f32x4 lds_acc_tile(const float* m, int ld, int r0, int c0) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  f32x4 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = m[(r0 + 4 * g + i) * ld + c0 + c];
  return x;
}

// The reverse: the lane's accumulator-layout values v[i] = X[r0 + 4 g + i][c0 + c] stored
// into a row-major matrix in LDS.  bf16: rounded, turned into the row piece X[r0 + c][c0 +
// 4 g .. + 3] by transpose_tile16 (which, given a tile's accumulator layout, returns its
// row pieces), and written with one 8-byte store instead of four 2-byte ones.
__device__ __forceinline__ void lds_store_acc_tile(bf16* m, int ld, int r0, int c0, f32x4 v) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  bf16x4 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (bf16)v[i];
  *reinterpret_cast<bf16x4*>(m + (r0 + c) * ld + c0 + 4 * g) = transpose_tile16(x);
}
__device__ __forceinline__ void lds_store_acc_tile(float* m, int ld, int r0, int c0, f32x4 v) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) m[(r0 + 4 * g + i) * ld + c0 + c] = v[i];
}
// A 16 x 16 tile of zeros at (r0, c0): every lane writes one row piece.
__device__ __forceinline__ void lds_zero_tile(bf16* m, int ld, int r0, int c0) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  *reinterpret_cast<i16x4*>(m + (r0 + c) * ld + c0 + 4 * g) = i16x4{0, 0, 0, 0};
}
__device__ __forceinline__ void lds_zero_tile(float* m, int ld, int r0, int c0) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  *reinterpret_cast<f32x4*>(m + (r0 + c) * ld + c0 + 4 * g) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// fragment values e = 0..7 multiplied by (g0, g1)[e] (rounded once to the operand type)
__device__ __forceinline__ Frag<bf16> scale_frag(const Frag<bf16>& f, f32x4 g0, f32x4 g1) {
  Frag<bf16> r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.v[e] = (bf16)((float)f.v[e] * g0[e]);
    r.v[e + 4] = (bf16)((float)f.v[e + 4] * g1[e]);
  }
  return r;
}
__device__ __forceinline__ Frag<float> scale_frag(const Frag<float>& f, f32x4 g0, f32x4 g1) {
  Frag<float> r;
  r.lo = f.lo * g0;
  r.hi = f.hi * g1;
  return r;
}

// single fp32 MFMA step (k = 4): lane l supplies A[l%16][l/16] and B[l/16][l%16]
__device__ __forceinline__ void mma_k4(f32x4& c, float a, float b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------- conversions
template <typename T> __device__ __forceinline__ T to(float x);
template <> __device__ __forceinline__ float to<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 to<bf16>(float x) { return (bf16)x; }
__device__ __forceinline__ float tof(float x) { return x; }
__device__ __forceinline__ float tof(bf16 x) { return (float)x; }

// 4 accumulator values written as 4 consecutive elements
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = b;
}
__device__ __forceinline__ f32x4 load4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4f(const bf16* p) {
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

// ------------------------------------------------------------------ 16-deep products
// One 16-token block of a contraction: v_mfma_f32_16x16x16_bf16 (bf16) or four
// v_mfma_f32_16x16x4_f32 steps (fp32).  Operand layouts:
//   bf16  A: lane l holds A[l % 16][4 (l / 16) + j]        B: B[4 (l / 16) + j][l % 16], j = 0..3
//   fp32  A: lane l holds A[l % 16][4 s + l / 16] (step s) B: B[4 s + l / 16][l % 16]
// (A and B share the k permutation, so the sum is unchanged); C as the 32-deep form.
template <typename T> struct Frag16;
template <> struct Frag16<bf16> { bf16x4 v; };
template <> struct Frag16<float> { f32x4 v; };

__device__ __forceinline__ void mma16(f32x4& c, const Frag16<bf16>& a, const Frag16<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a.v), __builtin_bit_cast(i16x4, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& c, const Frag16<float>& a, const Frag16<float>& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}
// Fragment whose 16 rows are rows r0.. of a row-major LDS matrix M (stride ld) and whose
// 16-deep k block starts at column k0 (the A operand of a matrix stored [row][k]).
__device__ __forceinline__ Frag16<bf16> lds_frag16_rows(const bf16* m, int ld, int r0, int k0) {
  const int lane = lane_id();
  Frag16<bf16> f;
  f.v = *reinterpret_cast<const bf16x4*>(m + (r0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4));
  return f;
}
__device__ __forceinline__ Frag16<float> lds_frag16_rows(const float* m, int ld, int r0, int k0) {
  const int lane = lane_id();
  Frag16<float> f;
#pragma unroll
  for (int s = 0; s < 4; ++s) f.v[s] = m[(r0 + (lane & 15)) * ld + k0 + 4 * s + (lane >> 4)];
  return f;
}
// Fragment whose 16 rows are columns c0.. of a row-major LDS matrix M and whose k block
// is rows k0 .. k0 + 15 (the B operand of a matrix stored [k][column], or the A operand
// of one stored transposed).  bf16: one LDS transpose read, lane s of each 16-lane group
// g pointing at row k0 + 4 g + s / 4, columns c0 + 4 (s % 4) (see lds_frag_tr).
__device__ __forceinline__ Frag16<bf16> lds_frag16_cols(const bf16* m, int ld, int c0, int k0) {
  const int lane = lane_id(), s = lane & 15, g = lane >> 4;
  bf16* p = const_cast<bf16*>(m) + (k0 + 4 * g + (s >> 2)) * ld + c0 + 4 * (s & 3);
  Frag16<bf16> f;
  f.v = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
  return f;
}
__device__ __forceinline__ Frag16<float> lds_frag16_cols(const float* m, int ld, int c0, int k0) {
  const int lane = lane_id();
  Frag16<float> f;
#pragma unroll
  for (int s = 0; s < 4; ++s) f.v[s] = m[(k0 + 4 * s + (lane >> 4)) * ld + c0 + (lane & 15)];
  return f;
}

// padded leading dimensions for LDS tiles: rows shifted by 16 bytes to spread banks
template <typename T> struct Pad;
template <> struct Pad<bf16> { static constexpr int v = 8; };
template <> struct Pad<float> { static constexpr int v = 4; };

}  // namespace carve
