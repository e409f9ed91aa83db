// Recurrent decode step of the CARVE key-axis gated delta rule on gfx950: one new
// token per (batch, head), the state updated in place.
//
// The token recurrence (CARVE notes, sections 2.1 and 2.2):
//   a = exp(log g) * b,  P = S Diag(a),  e = v - P k,  S' = P + w e k^T,  o = S' q.
// Every value row v of the state is independent:
//   P_v = S_v .* a,   e_v = v_v - P_v . k,   S'_v = P_v + w e_v k,
//   o_v = S'_v . q = P_v . q + w e_v (k . q),
// so one pass over S reads each element once and writes it once; the cost is the
// state's HBM traffic (2 * 4 * Dv * Dk bytes per head and token, the O(d_v d_k)
// per-token inference cost of the comparison table in section 3 of the notes).
//
// Content-aware erase (section 2.2): b = sigmoid(b_x + U2 (U1 m)) with m the mean
// output of the previous complete chunk; the running sum of the current chunk's
// outputs is carried between calls and turned into the next m at the chunk's end.
#include "carve_device.h"
#include "carve_internal.h"

namespace carve {

// CPL consecutive elements (4 or 8) at p, as floats, with 16-byte (float) or 8/16-byte (bf16) loads
template <int CPL>
__device__ __forceinline__ void load_cols(const float* p, float (&x)[CPL]) {
#pragma unroll
  for (int u = 0; u < CPL / 4; ++u) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p + 4 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * u + e] = t[e];
  }
}
template <int CPL>
__device__ __forceinline__ void load_cols(const bf16* p, float (&x)[CPL]) {
#pragma unroll
  for (int u = 0; u < CPL / 4; ++u) {
    const bf16x4 t = *reinterpret_cast<const bf16x4*>(p + 4 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * u + e] = (float)t[e];
  }
}
__device__ __forceinline__ float load_el(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_el(const bf16* p, size_t i) { return (float)p[i]; }

// One workgroup of 256 threads handles 16 * RPT value rows of one head: the 16 lanes
// of a DPP row own RPT state rows (16 apart), CPL = Dk / 16 consecutive key columns
// of each.
constexpr int kDecodeRows = 2;   // state rows per thread
template <typename T, int DK, bool CONTENT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int CPL = DK / 16, RPT = kDecodeRows, WR = 16 * RPT;
  static_assert(CPL == 4 || CPL == 8, "key width 64 or 128");
  __shared__ float rS[64];               // U1 m (content path; rank <= 64)
  const int tid = threadIdx.x, c16 = tid & 15;
  const int nvb = a.Dv / WR;
  const int bh = blockIdx.x / nvb, vb = blockIdx.x % nvb;
  const int h = bh % a.H;
  const int row0 = WR * vb + (tid >> 4);  // rows row0 + 16 i
  const int c0 = CPL * c16;
  float* S = a.S + ((size_t)bh * a.Dv + row0) * DK + c0;

  // state row pieces first: they are the bulk of the traffic
  f32x4 s[RPT][CPL / 4];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
#pragma unroll
    for (int u = 0; u < CPL / 4; ++u) s[i][u] = *reinterpret_cast<const f32x4*>(S + (size_t)16 * i * DK + 4 * u);

  float kc[CPL], qc[CPL], ac[CPL];
  load_cols<CPL>(reinterpret_cast<const T*>(a.k) + (size_t)bh * DK + c0, kc);
  load_cols<CPL>(reinterpret_cast<const T*>(a.q) + (size_t)bh * DK + c0, qc);
  load_cols<CPL>(a.log_g + (size_t)bh * DK + c0, ac);

  // erase gate at the lane's key columns
  float bc[CPL];
  if constexpr (CONTENT) {
    // z = U2 (U1 m) for this head (every workgroup of the head forms it; R x (Dv + Dk) MACs)
    const bool proj = a.U1 != nullptr && a.m_in != nullptr;
    if (proj) {
      const float* U1 = a.U1 + (size_t)h * a.R * a.Dv;
      const float* m = a.m_in + (size_t)bh * a.Dv;
      const int per = a.Dv / 16;
      for (int idx = tid; idx < 16 * a.R; idx += 256) {    // 16 lanes per rank index
        const int r = idx >> 4, part = idx & 15;
        float acc = 0.f;
        for (int j = 0; j < per; ++j) acc += U1[(size_t)r * a.Dv + part * per + j] * m[part * per + j];
        acc = row16_sum(acc);
        if (part == 0) rS[r] = acc;
      }
    }
    __syncthreads();
    load_cols<CPL>(a.b_x + (size_t)bh * DK + c0, bc);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float z = 0.f;
      if (proj) {
        const float* U2 = a.U2 + ((size_t)h * DK + c0 + j) * a.R;
        for (int r = 0; r < a.R; ++r) z += U2[r] * rS[r];
      }
      bc[j] = 1.f / (1.f + __expf(-(bc[j] + z)));
    }
  } else if (a.b) {
    load_cols<CPL>(a.b + (size_t)bh * DK + c0, bc);
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) bc[j] = 1.f;
  }

  float kq = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    ac[j] = __expf(ac[j]) * bc[j];                       // a = exp(log g) * b
    kq += kc[j] * qc[j];
  }
  kq = row16_sum(kq);
  const float w = a.w[bh];
  const T* v = reinterpret_cast<const T*>(a.v) + (size_t)bh * a.Dv;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = row0 + 16 * i;
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const float p = s[i][j / 4][j % 4] * ac[j];        // P = S Diag(a)
      s[i][j / 4][j % 4] = p;
      pk += p * kc[j];
      pq += p * qc[j];
    }
    pk = row16_sum(pk);
    pq = row16_sum(pq);
    const float e = load_el(v, row) - pk;                // prediction error of this value row
    const float we = w * e;
#pragma unroll
    for (int j = 0; j < CPL; ++j) s[i][j / 4][j % 4] += we * kc[j];
#pragma unroll
    for (int u = 0; u < CPL / 4; ++u) *reinterpret_cast<f32x4*>(S + (size_t)16 * i * DK + 4 * u) = s[i][u];

    if (c16 == 0) {
      const float o = pq + we * kq;                      // S' q
      reinterpret_cast<T*>(a.o)[(size_t)bh * a.Dv + row] = to<T>(o);
      if constexpr (CONTENT) {
        const size_t idx = (size_t)bh * a.Dv + row;
        const float cs = (a.pos == 0 ? 0.f : a.csum[idx]) + o;
        if (a.pos == a.L - 1) {
          a.m_out[idx] = cs / (float)a.L;                // this chunk is complete
          a.csum[idx] = 0.f;
        } else {
          a.m_out[idx] = a.m_in ? a.m_in[idx] : 0.f;
          a.csum[idx] = cs;
        }
      }
    }
  }
}

template <typename T, int DK>
static hipError_t decode_launch_dk(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.B * a.H * (a.Dv / (16 * kDecodeRows)));
  if (a.b_x) hipLaunchKernelGGL((decode_kernel<T, DK, true>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((decode_kernel<T, DK, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t st) {
  if (a.Dk == 128) return dtype ? decode_launch_dk<bf16, 128>(a, st) : decode_launch_dk<float, 128>(a, st);
  if (a.Dk == 64) return dtype ? decode_launch_dk<bf16, 64>(a, st) : decode_launch_dk<float, 64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace carve
