// Gate backward of one content period (CARVE notes, section 2.2), shared by the
// per-period gate kernel and the chunk-gradient kernel's tail: with one token tile per
// content period the chunk-gradient workgroup of a head runs it right after its stores.
#pragma once
#include "carve_chunk.h"

namespace carve {

// LDS floats content_gate_body needs (rank R <= 64)
__host__ __device__ constexpr size_t content_gate_lds_floats(int D, int NT, int R) {
  return (size_t)NT + 3 * D + 2 * 64 + 2 * (size_t)R * D;
}

// Gate backward of period p for head bh, run by the NT threads of one workgroup: the sum
// of the period's d/db_x (written by the chunk-gradient kernel) per key channel, then the
// projection's gradients and the output-gradient term g of period p-1, which is added at
// once to that period's dO (into dOp; period 0's dm goes to m0).  Nothing it loads depends
// on what it computes, so every load is issued at the start (d/db_x of the first 64
// tokens, U1 and U2 for LDS, m_{p-1}, the running dU sums, the first 64 tokens of period
// p-1's dO): one round trip to memory instead of one per phase.  The rank contractions run
// 16 lanes per rank index with DPP row sums.  lds: content_gate_lds_floats(D, NT, R)
// floats; every thread of the workgroup must call it (it holds barriers).
template <typename T, int D, int NT>
__device__ __forceinline__ void content_gate_body(const ContentBwdArgs& a, int bh, const T* dO, T* dOp, float* lds) {
  constexpr int NPART = NT / D, TPT = 64 / NPART;               // tokens per thread in a 64-token batch
  constexpr int RMAX = 64, UPT = RMAX * D / NT;                // projection elements per thread, at most
  constexpr int OP = 64 * D / 4 / NT;                          // 4-element dO pieces per thread, 64 tokens
  static_assert(NT % D == 0 && 64 % NPART == 0, "threads must split into whole key columns");
  float* dzp = lds;                                            // [NT]
  float* dz = dzp + NT;                                        // [D]
  float* gS = dz + D;                                          // [D]
  float* mS = gS + D;                                          // [D]
  float* rS = mS + D;                                          // [RMAX]
  float* drS = rS + RMAX;                                      // [RMAX]
  float* Us = drS + RMAX;                                      // U1 [R][D], then U2 [D][R]
  const int h = bh % a.H, tid = threadIdx.x;
  const int t0 = a.p * a.L, t1 = min(t0 + a.L, a.T);
  const int k = tid % D, part = tid / D;
  const bool proj = a.U1 != nullptr;
  const int R = proj ? a.R : 0, RD = R * D;
  const float* m = a.m_all + ((size_t)bh * a.NP + a.p) * D;    // m_{p-1}
  float* dU1p = a.dU1p + (size_t)bh * RD;                      // [R][D]
  float* dU2p = a.dU2p + (size_t)bh * RD;                      // [D][R]
  float* U1s = Us;
  float* U2s = Us + RD;

  // ---- every load
  float gv[TPT];
  auto load_batch = [&](int tb) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int t = min(tb + part + NPART * j, t1 - 1);
      gv[j] = a.dbx[((size_t)bh * a.T + t) * D + k];
    }
  };
  load_batch(t0);
  // Unconditional loads from clamped indices (without a projection, from b: any valid
  // address; the values past RD are never used).  A branch around a load makes the
  // compiler copy its result at the join, which waits for every load issued before it.
  float u1[UPT], u2[UPT], du1[UPT], du2[UPT];
  const float* U1g = proj ? a.U1 + (size_t)h * RD : a.bmat;
  const float* U2g = proj ? a.U2 + (size_t)h * RD : a.bmat;
  const float* dU1g = proj ? dU1p : a.bmat;
  const float* dU2g = proj ? dU2p : a.bmat;
  const int ilast = max(RD - 1, 0);
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int i = min(tid + NT * j, ilast);
    u1[j] = U1g[i];
    u2[j] = U2g[i];
    du1[j] = dU1g[i];
    du2[j] = dU2g[i];
  }
  const float mv = m[min(tid, D - 1)];
  const bool addg = a.p > 0;
  // period p-1 (whole) when there is one; period 0's tokens are loaded in vain otherwise
  const size_t obase = ((size_t)bh * a.T + (size_t)(addg ? a.p - 1 : 0) * a.L) * D;
  const int n4 = a.L * D / 4, nl4 = addg ? n4 : (t1 - t0) * D / 4;   // pieces that exist
  f32x4 ov[OP];
#pragma unroll
  for (int j = 0; j < OP; ++j) ov[j] = load4f(dO + obase + 4 * min(tid + NT * j, nl4 - 1));
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int i = tid + NT * j;
    if (i < RD) {
      U1s[i] = u1[j];
      U2s[i] = u2[j];
    }
  }
  if (tid < D) mS[tid] = mv;

  // ---- dx = d/db_x (the chunk-gradient kernel already wrote dlog a (1 - b)), summed over
  // the period's tokens per key column (each thread in token order)
  float acc = 0.f;
  for (int tb = t0;;) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int t = tb + part + NPART * j;
      if (t < t1) acc += gv[j];
    }
    tb += 64;
    if (tb >= t1) break;
    load_batch(tb);
  }
  dzp[tid] = acc;
  __syncthreads();
  if (tid < D) {
    float sum = 0.f;
#pragma unroll
    for (int pp = 0; pp < NPART; ++pp) sum += dzp[pp * D + tid];
    dz[tid] = sum;
  }
  __syncthreads();
  if (proj) {
    // r = U1 m and dr = U2^T dz: lanes 16 r' .. 16 r' + 15 of a row share rank index r'
    constexpr int PER = D / 16;
    for (int idx = tid; idx < 16 * R; idx += NT) {
      const int r = idx >> 4, c = (idx & 15) * PER;
      float x = 0.f, y = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        x += U1s[r * D + c + j] * mS[c + j];
        y += U2s[(c + j) * R + r] * dz[c + j];
      }
      x = row16_sum(x);
      y = row16_sum(y);
      if ((idx & 15) == 0) {
        rS[r] = x;
        drS[r] = y;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int i = tid + NT * j;
      if (i < RD) {
        dU2p[i] = du2[j] + dz[i / R] * rS[i % R];
        dU1p[i] = du1[j] + drS[i / D] * mS[i % D];
      }
    }
  }
  if (tid < D) {
    float dm = 0.f;
    for (int r = 0; r < R; ++r) dm += U1s[r * D + tid] * drS[r];
    if (addg) gS[tid] = dm / (float)a.L;
    else if (a.dm0) a.dm0[(size_t)bh * D + tid] = dm;
  }
  if (!addg) return;
  __syncthreads();
  // dO + g for the tokens of period p-1
#pragma unroll
  for (int j = 0; j < OP; ++j) {
    const int i = tid + NT * j;
    if (i < n4) {
      const int col = (4 * i) % D;
      store4(dOp + obase + 4 * i, ov[j] + f32x4{gS[col], gS[col + 1], gS[col + 2], gS[col + 3]});
    }
  }
  for (int i = tid + NT * OP; i < n4; i += NT) {              // periods longer than 64 tokens
    const int col = (4 * i) % D;
    store4(dOp + obase + 4 * i, load4f(dO + obase + 4 * i) + f32x4{gS[col], gS[col + 1], gS[col + 2], gS[col + 3]});
  }
}

}  // namespace carve
