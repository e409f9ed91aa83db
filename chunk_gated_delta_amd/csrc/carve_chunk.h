// Per-chunk factor preparation shared by the forward and backward kernels.
//
// Chunk algebra (rows = tokens of one chunk, S = state entering the chunk,
// Gamma_r = prod_{i<=r} a_i per key channel, Gamma_L its value at the chunk end):
//   K+ = K .* Gamma, K- = K ./ Gamma, Q+ = Q .* Gamma, K-> = K .* Gamma_L ./ Gamma
//   A  = strict_tril(diag(w) K+ K-^T)       shared by every value channel
//   T  = (I + A)^-1                          (one triangular solve per chunk)
//   U  = T diag(w) V - T diag(w) K+ S^T = Ubar - W S^T
//   O  = Q+ S^T + tril(Q+ K-^T) U = (P Ubar) + Q~ S^T
//   S' = S Diag(Gamma_L) + U^T K->
// This is the token recurrence of the CARVE notes (sections 2.1-2.3) unrolled
// over one chunk: the shared coupling is what the notes call the single WY-form
// triangular solve that key-axis-only gating keeps valid.
#pragma once
#include "carve_device.h"
#include "carve_internal.h"

namespace carve {

// ------------------------------------------------------------------ helpers
template <typename T, int LC, int D, int NT = kThreads>
struct PrepLayout {
  static constexpr int LDD = D + Pad<T>::v;      // [LC][D] row stride (elements)
  static constexpr int LDL = LC + Pad<T>::v;     // [D][LC] and [LC][LC] row stride
  static constexpr int LDF = LC + 4;             // fp32 [LC][LC] row stride
  static constexpr int P = NT / D;               // token parts per key channel (one channel a thread)
  static constexpr size_t szLD = sizeof(T) * LC * LDD;
  static constexpr size_t szDL = sizeof(T) * D * LDL;
  static constexpr size_t szLLf = sizeof(float) * LC * LDF;
  static constexpr size_t szLL = sizeof(T) * LC * LDL;
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t x) { return (x + 255) & ~size_t(255); }
  // region 1: K+ and K- (gate pass .. coupling), then T (fp32) and Tb (dtype)
  static constexpr size_t R1 = 0;
  static constexpr size_t R1sz = al(cmax(2 * szLD, szLLf + szLL));
  static constexpr size_t R2 = R1 + R1sz;                 // Q+           (gate pass .. Q~)
  static constexpr size_t R3 = R2 + al(szLD);             // Kw^T, Vw^T   (gate pass .. WY factors)
  static constexpr size_t R4 = R3 + al(2 * szDL);         // A (fp32), then (-W)^T
  static constexpr size_t R5 = R4 + al(cmax(szLLf, szDL)); // P (dtype)
  static constexpr size_t R6 = R5 + al(szLL);             // raw V, then the diagonal-tile K operand, then Ubar^T
  static constexpr size_t R7 = R6 + al(szDL);             // w [LC], part sums of log a [<= 2P][D]
  // R8: per-chunk gate tables: flags [16] int (1 = block needs the exact diagonal
  // tiles) and exp of the log-retention at each block start [NB][D]
  static constexpr int NB = LC / 16;
  static constexpr int NFAR = (NB - 1) * (NB - 2) / 2;
  static constexpr size_t R8 = R7 + al(sizeof(float) * (LC + 2 * P * D));   // up to 2P parts
  // R9: column operands of the far coupling tiles (blocks I >= J + 2), [NFAR][16][LDD]:
  // K^-_J times the retention between the end of block J and the start of block I
  static constexpr size_t R9 = R8 + al(sizeof(int) * 16 + sizeof(float) * NB * D);
  static constexpr size_t bytes = R9 + al(sizeof(T) * NFAR * 16 * LDD);
};

// Range of the gate algebra.  The per-token log-retention la = log g + log b is taken
// in [kLaFloor, 0] (a retention below e^kLaFloor is zero in float32; NaN passes
// through).  Inside a 16-token block the diagonal coupling tiles use one operand scaled
// by exp(-(decay since the block start)); that is finite while the block's decay stays
// below kSafeLog in every key channel.  Blocks beyond that take the exact elementwise
// tiles (running products of the retention).
constexpr float kLaFloor = -1.0e4f;
constexpr float kSafeLog = 64.f;
// A chunk whose log-retention stays above -kChunkSafe in every key channel takes the
// fast path: operands referred to the chunk start, K- = k / Gamma at most e^kChunkSafe.
constexpr float kChunkSafe = 80.f;
constexpr float kMinOwn = 1.6038109e-28f;   // exp(-64)
__device__ __forceinline__ float clamp_la(float la) {
  la = la > 0.f ? 0.f : la;
  return la < kLaFloor ? kLaFloor : la;
}
// blocks I >= J + 2 of a chunk -> index into the far-pair table
__device__ __forceinline__ constexpr int far_index(int I, int J) { return (I - 2) * (I - 1) / 2 + J; }

// ------------------------------------------------------------------ global layouts
// MFMA fragment order of a [rows][C] matrix M (C = contraction length): fragment
// (rt, kb) holds, for lane l, M[16 rt + l%16][32 kb + 8 (l/16) + j], j = 0..7, at
// ((rt * C/32 + kb) * 64 + l) * 8, so one fragment is one contiguous 16-byte
// (bf16) load per lane and 1 KB per wave.
template <int C>
__device__ __forceinline__ size_t frag_offset(int rt, int kb, int lane) {
  return ((size_t)(rt * (C / 32) + kb) * 64 + lane) * 8;
}
// Accumulator order of a [rows][W] matrix (an MFMA output): tile (rt, ct) holds, for
// lane l, M[16 rt + 4 (l/16) + i][16 ct + l%16], i = 0..3, at ((rt * W/16 + ct) * 64 + l) * 4.
template <int W>
__device__ __forceinline__ size_t acc_offset(int rt, int ct, int lane) {
  return ((size_t)(rt * (W / 16) + ct) * 64 + lane) * 4;
}

// CPT (1 or 2) adjacent elements of a row in LDS, as floats (loads) or rounded to T
// (stores; st_row with a column index stores x[c][i]).
template <typename T, int CPT>
__device__ __forceinline__ void ld_row(const T* p, float (&x)[CPT]) {
  if constexpr (CPT == 2) {
    if constexpr (sizeof(T) == 2) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
      x[0] = (float)v[0];
      x[1] = (float)v[1];
    } else {
      const f32x2 v = *reinterpret_cast<const f32x2*>(p);
      x[0] = v[0];
      x[1] = v[1];
    }
  } else {
    x[0] = tof(p[0]);
  }
}
template <typename T, int CPT>
__device__ __forceinline__ void st_row(T* p, const float (&x)[CPT]) {
  if constexpr (CPT == 2) {
    if constexpr (sizeof(T) == 2) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<bf16x2*>(p) = bf16x2{to<bf16>(x[0]), to<bf16>(x[1])};
    } else {
      *reinterpret_cast<f32x2*>(p) = f32x2{x[0], x[1]};
    }
  } else {
    p[0] = to<T>(x[0]);
  }
}
template <typename T, int CPT, int N>
__device__ __forceinline__ void st_row(T* p, const float (&x)[CPT][N], int i) {
  float y[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) y[c] = x[c][i];
  st_row<T, CPT>(p, y);
}

// lower-triangular block index -> (i, j), j <= i
__device__ __forceinline__ void tri_index(int t, int& i, int& j) {
  i = 0;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  j = t - i * (i + 1) / 2;
}

// T = (I + A)^-1 for strictly lower-triangular A (fp32 in LDS), LC = 16 * NB.
// Diagonal 16x16 blocks by column-parallel forward substitution, then the
// off-diagonal blocks by block forward substitution on fp32 MFMA:
//   T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj = -sum_{m=j}^{i-1} (T_ii A_im) T_mj,
// with the scaled blocks T_ii A_im formed first (all in parallel) and the T_ij
// by increasing distance i - j.  The strictly lower blocks of A are overwritten;
// the blocks of T above the diagonal are not written.
// LDS-typed pointers, so that every access is an LDS instruction.  triangular_inverse
// is the out-of-line copy (used where inlining would add its registers to those of the
// chunk prefetched in the persistent loop, or to the content-aware kernel's, and spill);
// an out-of-line function starts by waiting for all of its caller's outstanding memory
// operations, so callers issue prefetches after the call.
typedef __attribute__((address_space(3))) float lds_float;
template <int LC, int LDF, int NT = kThreads>
__device__ __forceinline__ void triangular_inverse_inl(lds_float* Af, lds_float* Tf) {
  constexpr int NB = LC / 16;
  static_assert(NT / 64 >= NB - 1, "one wave per off-diagonal block of a distance");
  static_assert(LDF % 4 == 0, "rows of A are read as 16-byte pieces");
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  if (tid < 16 * NB) {
    // lane (block, column j) solves (I + A_bb) x = e_j row by row: x[r] = e_j[r] -
    // sum_{m<r} A[r][m] x[m], accumulated in the order m = 0, 1, ...; the rows of A
    // are read as 4-float pieces (every lane of a block reads the same addresses), all
    // independent of x, so only the final subtraction of each row waits on x[r-1]
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    const int base = 16 * (tid / 16), j = tid % 16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float xr = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int c4 = 0; 4 * c4 < r; ++c4) {
        const f32x4 av = *reinterpret_cast<const lds_f32x4*>(Af + (base + r) * LDF + base + 4 * c4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * c4 + e < r) xr -= av[e] * x[4 * c4 + e];
      }
      x[r] = xr;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tf[(base + r) * LDF + base + j] = x[r];
  }
  __syncthreads();   // blocks above the diagonal are never written: readers treat them as 0
  const int lr = lane & 15, lg = lane >> 4;
  // scaled coupling blocks Ahat_im = T_ii A_im (i > m), written over A_im (one wave
  // per block; a wave reads only its own block of A before writing it)
  constexpr int NPAIR = NB * (NB - 1) / 2;
  lds_float* Ah = Af;
  for (int t = wave; t < NPAIR; t += NT / 64) {
    int i = 1, m = t;
    while (m >= i) { m -= i; ++i; }           // t -> (i, m), 0 <= m < i
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      mma_k4(y, Tf[(16 * i + lr) * LDF + 16 * i + 4 * s4 + lg], Af[(16 * i + 4 * s4 + lg) * LDF + 16 * m + lr]);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) Ah[(16 * i + 4 * lg + ii) * LDF + 16 * m + lr] = y[ii];
  }
  __syncthreads();
  // off-diagonal blocks by increasing distance: T_ij = -sum_{m=j}^{i-1} Ahat_im T_mj
  for (int d = 1; d < NB; ++d) {
    if (wave < NB - d) {
      const int j = wave, i = wave + d;
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      for (int m = j; m < i; ++m) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          mma_k4(y, Ah[(16 * i + lr) * LDF + 16 * m + 4 * s4 + lg], Tf[(16 * m + 4 * s4 + lg) * LDF + 16 * j + lr]);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Tf[(16 * i + 4 * lg + ii) * LDF + 16 * j + lr] = -y[ii];
    }
    __syncthreads();
  }
}
template <int LC, int LDF, int NT = kThreads>
__device__ __attribute__((noinline)) void triangular_inverse(lds_float* Af, lds_float* Tf) {
  triangular_inverse_inl<LC, LDF, NT>(Af, Tf);
}

// ------------------------------------------------------------------ gate sources
// Erase gate of one element, split into a raw load (issued early, branch-free) and the
// log-retention it contributes: token-only with b given, token-only with b = 1, or
// content-aware b = sigmoid(b_x + z) with the chunk's content signal z (per key channel,
// in LDS).  la(lg, x, ch, A, tau) is the per-token log-retention log g + log b of key
// channel ch from the staged decay input lg and erase input x (A, tau: the channel's
// amplitude and bias when the gates come as pre-activations).
// Every source also maps the staged write input to w (wact: the identity unless the
// gates come as pre-activations; kLogits marks that case, whose staged decay input is
// the logit f).
// (hardware exp / log / reciprocal: softplus(y) = max(y, 0) + log(1 + exp(-|y|)),
// log sigmoid(y) = -softplus(-y))
__device__ __forceinline__ float softplusf(float y) { return fmaxf(y, 0.f) + flog(1.f + fexp(-fabsf(y))); }
__device__ __forceinline__ float sigmoidf(float y) { return __builtin_amdgcn_rcpf(1.f + fexp(-y)); }
struct TokenGatesB {
  static constexpr bool kLogits = false;
  const float* b;
  __device__ __forceinline__ Frag<float> load8(size_t idx) const { return load_frag(b + idx); }
  __device__ __forceinline__ float la(float lg, float x, int, float, float) const { return clamp_la(lg + flog(x)); }
  __device__ __forceinline__ float wact(float x) const { return x; }
};
struct TokenGates1 {
  static constexpr bool kLogits = false;
  __device__ __forceinline__ Frag<float> load8(size_t) const {
    Frag<float> f;
    f.lo = f32x4{1.f, 1.f, 1.f, 1.f};
    f.hi = f.lo;
    return f;
  }
  __device__ __forceinline__ float la(float lg, float, int, float, float) const { return clamp_la(lg); }
  __device__ __forceinline__ float wact(float x) const { return x; }
};
struct ContentGates {
  static constexpr bool kLogits = false;
  const float* b_x;
  const float* z;
  __device__ __forceinline__ Frag<float> load8(size_t idx) const { return load_frag(b_x + idx); }
  __device__ __forceinline__ float la(float lg, float x, int ch, float, float) const {
    return clamp_la(lg - softplusf(-(x + z[ch])));
  }
  __device__ __forceinline__ float wact(float x) const { return x; }
};

// Gates given as pre-activations (the fused gate of the notes, section 2.3):
// log g = -A softplus(f + tau) with A, tau per head and key channel, b = sigmoid(b_x)
// (HAS_BX; else b = 1), w = sigmoid(w_hat).  The staged decay input is f, the staged
// erase input b_x, the staged write input w_hat.
template <int D, bool HAS_BX>
struct LogitGates {
  static constexpr bool kLogits = true;
  const float* b_x;
  const float* A;     // [H][D]
  const float* tau;   // [H][D]
  __device__ __forceinline__ Frag<float> load8(size_t idx) const {
    if constexpr (HAS_BX) return load_frag(b_x + idx);
    return TokenGates1{}.load8(idx);
  }
  // log g from the decay logit x and the channel's amplitude and bias
  __device__ __forceinline__ float logdecay_p(float x, float a, float t) const { return -a * softplusf(x + t); }
  __device__ __forceinline__ float la(float lg, float x, int, float a, float t) const {
    const float l = logdecay_p(lg, a, t);
    return clamp_la(HAS_BX ? l - softplusf(-x) : l);
  }
  __device__ __forceinline__ float wact(float x) const { return sigmoidf(x); }
};

// ------------------------------------------------------------------ per-chunk prep
// Computes the factors of chunk c of head bh and writes them to slot `ci` of
// the factor arrays.  Uses PrepLayout<T, LC, D>::bytes of LDS at `smem`.
// MODE bit 1 writes the factor only the forward output uses (P Ubar); bit 2 writes
// the inverse T the chunk-gradient pass needs.  -W, Q~, K->^T, Ubar^T and Gamma_L
// are always written.
constexpr int kPrepFwd = 1, kPrepBwd = 2;

// Raw inputs of one chunk as 16-byte pieces (8 consecutive channels of one token),
// piece tid + NT u of thread tid.  Loaded from clamped rows (branch-free), then
// staged in LDS: k, q, v raw in the K+, Q+ and Ubar^T regions, the per-element
// log-retention la = log g + log b (clamped, see clamp_la) in the Kw^T region
// (fp32 [LC][D]); rows past the end become k = q = v = 0, la = 0.
template <typename T, int LC, int D, int NT>
struct PrepStage {
  static constexpr int PR = D / 8, NP = LC * PR, NST = (NP + NT - 1) / NT;
  Frag<T> k[NST], q[NST], v[NST];
  Frag<float> lg[NST], g[NST];
  float w;
  int h;                // head of the staged chunk
};

// PART 1: log g, the erase input and w; PART 2: k, q, v; PART 0: all of them.
template <typename T, int LC, int D, typename Gates, int NT, int PART = 0>
__device__ __forceinline__ void prep_stage_load(const FwdArgs& a, const Gates& gates, int bh, int c,
                                                PrepStage<T, LC, D, NT>& st) {
  using St = PrepStage<T, LC, D, NT>;
  const int tid = threadIdx.x;
  const int n = min(LC, a.T - c * LC);
  const size_t row0 = (size_t)bh * a.T + (size_t)c * LC;
  const T* kb = reinterpret_cast<const T*>(a.k) + row0 * D;
  const T* qb = reinterpret_cast<const T*>(a.q) + row0 * D;
  const T* vb = reinterpret_cast<const T*>(a.v) + row0 * D;
  const float* lb = a.log_g + row0 * D;
  if (PART != 2) {
    st.w = a.w[row0 + min(tid, n - 1)];
    st.h = bh % a.H;
  }
  // (the gate pieces, the larger half, are the ones issued early by the persistent loop)
#pragma unroll
  for (int u = 0; u < St::NST; ++u) {
    const int idx = min(tid + NT * u, St::NP - 1), r = idx / St::PR, g = idx % St::PR;
    const unsigned e = (unsigned)(min(r, n - 1) * D + 8 * g);
    if (PART != 1) {
      st.k[u] = load_frag(kb + e);
      st.q[u] = load_frag(qb + e);
      st.v[u] = load_frag(vb + e);
    }
    if (PART != 2) {
      st.lg[u] = load_frag(lb + e);
      st.g[u] = gates.load8(row0 * D + e);
    }
  }
}

template <typename T, int LC, int D, typename Gates, int NT>
__device__ __forceinline__ void prep_stage_write(const FwdArgs& a, const Gates& gates, int c,
                                                 const PrepStage<T, LC, D, NT>& st, unsigned char* smem) {
  using Lay = PrepLayout<T, LC, D, NT>;
  using St = PrepStage<T, LC, D, NT>;
  constexpr int LDD = Lay::LDD;
  static_assert(sizeof(float) * LC * D <= 2 * Lay::szDL, "retention staging exceeds the Kw^T region");
  static_assert(Lay::szLD <= Lay::szDL, "raw v staging exceeds the Ubar^T region");
  T* Kp = reinterpret_cast<T*>(smem + Lay::R1);
  T* Qp = reinterpret_cast<T*>(smem + Lay::R2);
  float* aS = reinterpret_cast<float*>(smem + Lay::R3);
  T* Vr = reinterpret_cast<T*>(smem + Lay::R6);
  float* wL = reinterpret_cast<float*>(smem + Lay::R7);
  const int tid = threadIdx.x;
  const int n = min(LC, a.T - c * LC);
  // gates as pre-activations: amplitude and bias of the thread's 8 channels (every piece
  // of a thread covers the same channels, as NT is a multiple of D / 8); [H][D] arrays
  // small enough to stay cached, read here rather than held through the prefetch
  Frag<float> pA, pT;
  if constexpr (Gates::kLogits) {
    static_assert(NT % St::PR == 0, "pieces of a thread must share their channels");
    pA = load_frag(gates.A + st.h * D + 8 * (tid % St::PR));
    pT = load_frag(gates.tau + st.h * D + 8 * (tid % St::PR));
  }
  if (tid < LC) wL[tid] = (tid < n) ? gates.wact(st.w) : 0.f;
  if (tid < 16) reinterpret_cast<int*>(smem + Lay::R8)[tid] = 0;   // exact-diagonal flags of the chunk
#pragma unroll
  for (int u = 0; u < St::NST; ++u) {
    const int idx = tid + NT * u;
    if (St::NP % NT == 0 || idx < St::NP) {
      const int r = idx / St::PR, g = idx % St::PR;
      const bool valid = r < n;
      *reinterpret_cast<Frag<T>*>(Kp + r * LDD + 8 * g) = valid ? st.k[u] : zero_frag(T());
      *reinterpret_cast<Frag<T>*>(Qp + r * LDD + 8 * g) = valid ? st.q[u] : zero_frag(T());
      *reinterpret_cast<Frag<T>*>(Vr + r * LDD + 8 * g) = valid ? st.v[u] : zero_frag(T());
      f32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float alo = 0.f, tlo = 0.f, ahi = 0.f, thi = 0.f;
        if constexpr (Gates::kLogits) {
          alo = pA.lo[e];
          tlo = pT.lo[e];
          ahi = pA.hi[e];
          thi = pT.hi[e];
        }
        lo[e] = valid ? gates.la(st.lg[u].lo[e], st.g[u].lo[e], 8 * g + e, alo, tlo) : 0.f;
        hi[e] = valid ? gates.la(st.lg[u].hi[e], st.g[u].hi[e], 8 * g + 4 + e, ahi, thi) : 0.f;
      }
      *reinterpret_cast<f32x4*>(aS + r * D + 8 * g) = lo;
      *reinterpret_cast<f32x4*>(aS + r * D + 8 * g + 4) = hi;
    }
  }
}

// Sum over the G lanes g = 0..G-1 of a lane group (G a power of two, the groups aligned);
// every lane of the group receives the sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// Exact diagonal coupling tiles of a 16-token block I whose log-retention falls below
// -kSafeLog in some key channel (the fast tiles would need factors beyond float range):
// for r >= s inside the block
//   B_rs = sum_ch k_r k_s R_rs,   P_rs = sum_ch q_r k_s R_rs,   R_rs = prod_{t=s+1..r} a_t,
// the retention ratio as a running product of a = e^la (no exponent range issue; a
// product that underflows is one whose true value is below float range).  The block's
// raw k, q and la are read again from global memory (the same gate arithmetic as the
// staging) into the scratch region R1, which is free after the coupling phase.  Thread
// (s, channel group g of 8 channels) runs r = 0..15, contributing for r >= s, and the
// groups of one s are summed with shuffles.  Overwrites the block's diagonal tiles of A
// (= w_r B_rs for s < r, fp32) and P, and with gB (backward modes) stores B in the
// accumulator order of the coupling phase.  Starts and ends with a barrier-separated
// phase (callers reach it from a workgroup-uniform branch).  Inlined: as an out-of-line
// call it would make the whole kernel address memory through generic pointers.
template <typename T, int LC, int D, typename Gates, int NT>
__device__ __forceinline__ void prep_diag_exact(const FwdArgs& a, const Gates& gates, int bh, int c, int I,
                                                          unsigned char* smem, float* Af, T* Pb, T* gB) {
  using Lay = PrepLayout<T, LC, D, NT>;
  constexpr int LDF = Lay::LDF, LDL = Lay::LDL, LDD = Lay::LDD, LDA = D + 4;
  constexpr int PR = D / 8, G = D / 8;
  static_assert(16 * G <= NT && (16 * G) % 64 == 0, "one thread per (column, channel group), whole waves");
  static_assert(sizeof(float) * 16 * LDA + 2 * sizeof(T) * 16 * LDD <= Lay::R1sz, "exact-tile scratch exceeds R1");
  float* aS = reinterpret_cast<float*>(smem + Lay::R1);                         // [16][LDA] a
  T* kS = reinterpret_cast<T*>(smem + Lay::R1 + sizeof(float) * 16 * LDA);      // [16][LDD] raw k
  T* qS = kS + 16 * LDD;                                                         // [16][LDD] raw q
  const float* wL = reinterpret_cast<const float*>(smem + Lay::R7);
  const int tid = threadIdx.x, lane = lane_id();
  const int n = min(LC, a.T - c * LC);
  const size_t row0 = (size_t)bh * a.T + (size_t)c * LC;
  const T* kg = reinterpret_cast<const T*>(a.k);
  const T* qg = reinterpret_cast<const T*>(a.q);
  for (int idx = tid; idx < 16 * PR; idx += NT) {
    const int rr = idx / PR, g = idx % PR, r = 16 * I + rr;
    const bool valid = r < n;
    const size_t e = (row0 + (size_t)min(r, n - 1)) * D + 8 * g;
    const Frag<T> kf = load_frag(kg + e), qf = load_frag(qg + e);
    const Frag<float> lf = load_frag(a.log_g + e), gf = gates.load8(e);
    Frag<float> pA = zero_frag(0.f), pT = zero_frag(0.f);
    if constexpr (Gates::kLogits) {
      pA = load_frag(gates.A + (bh % a.H) * D + 8 * g);
      pT = load_frag(gates.tau + (bh % a.H) * D + 8 * g);
    }
    f32x4 lo, hi;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      lo[e4] = valid ? fexp(gates.la(lf.lo[e4], gf.lo[e4], 8 * g + e4, pA.lo[e4], pT.lo[e4])) : 1.f;
      hi[e4] = valid ? fexp(gates.la(lf.hi[e4], gf.hi[e4], 8 * g + 4 + e4, pA.hi[e4], pT.hi[e4])) : 1.f;
    }
    *reinterpret_cast<f32x4*>(aS + rr * LDA + 8 * g) = lo;
    *reinterpret_cast<f32x4*>(aS + rr * LDA + 8 * g + 4) = hi;
    *reinterpret_cast<Frag<T>*>(kS + rr * LDD + 8 * g) = valid ? kf : zero_frag(T());
    *reinterpret_cast<Frag<T>*>(qS + rr * LDD + 8 * g) = valid ? qf : zero_frag(T());
  }
  __syncthreads();
  if (tid < 16 * G) {
    const int s = tid / G, g = tid % G;
    float ks[8], rho[8];
    {
      const Frag<T> f = load_frag(kS + s * LDD + 8 * g);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ks[j] = tof(frag_elem(f, j));
        rho[j] = 1.f;
      }
    }
    const int t = I * (I + 1) / 2 + I;             // tri index of the diagonal tile
#pragma unroll 1
    for (int r = 0; r < 16; ++r) {
      const Frag<T> kr = load_frag(kS + r * LDD + 8 * g), qr = load_frag(qS + r * LDD + 8 * g);
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(aS + r * LDA + 8 * g);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(aS + r * LDA + 8 * g + 4);
      float sb = 0.f, sp = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ar = j < 4 ? a0[j] : a1[j - 4];
        rho[j] = r > s ? rho[j] * ar : rho[j];
        const float x = ks[j] * rho[j];
        sb += tof(frag_elem(kr, j)) * x;
        sp += tof(frag_elem(qr, j)) * x;
      }
      sb = group_sum<G>(r >= s ? sb : 0.f);
      sp = group_sum<G>(r >= s ? sp : 0.f);
      if (g == 0) {
        const int row = 16 * I + r, col = 16 * I + s;
        const float bv = s < r ? sb : 0.f;
        Af[row * LDF + col] = wL[row] * bv;
        Pb[row * LDL + col] = to<T>(s <= r ? sp : 0.f);
        if (gB) gB[((size_t)t * 64 + s + 16 * (r / 4)) * 4 + r % 4] = to<T>(bv);
      }
    }
  }
  (void)lane;
  __syncthreads();
}

// The chunk's factors from its staged inputs (LDS, after a barrier).
struct NoPrefetch {
  __device__ __forceinline__ void operator()() const {}
};
// `after_solve` runs right after the triangular inverse (the persistent loop issues the
// next chunk's loads there, past the out-of-line call's wait for outstanding loads).
template <typename T, int LC, int D, typename Gates, int MODE = kPrepFwd, int NT = kThreads,
          typename AfterSolve = NoPrefetch>
__device__ __forceinline__ void prep_compute(const FwdArgs& a, const Gates& gates, int bh, int c, size_t ci,
                             unsigned char* smem, const AfterSolve& after_solve = AfterSolve{}) {
  using Lay = PrepLayout<T, LC, D, NT>;
  constexpr int NW = NT / 64;
  constexpr int NB = LC / 16, NCT = D / 16;
  constexpr int LDD = Lay::LDD, LDL = Lay::LDL, LDF = Lay::LDF, P = Lay::P;
  T* Kp = reinterpret_cast<T*>(smem + Lay::R1);
  T* Km = Kp + LC * LDD;
  float* Tf = reinterpret_cast<float*>(smem + Lay::R1);
  T* Tb = reinterpret_cast<T*>(smem + Lay::R1 + Lay::szLLf);
  T* Qp = reinterpret_cast<T*>(smem + Lay::R2);
  T* KwT = reinterpret_cast<T*>(smem + Lay::R3);
  T* VwT = KwT + D * LDL;
  float* Af = reinterpret_cast<float*>(smem + Lay::R4);
  T* WnT = reinterpret_cast<T*>(smem + Lay::R4);
  T* QtTs = KwT;                                    // Q~^T once the WY factors are done
  T* Pb = reinterpret_cast<T*>(smem + Lay::R5);
  T* UbTs = reinterpret_cast<T*>(smem + Lay::R6);
  float* wL = reinterpret_cast<float*>(smem + Lay::R7);
  float* part = wL + LC;

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int t0 = c * LC;
  const int n = min(LC, a.T - t0);
  const size_t row0 = (size_t)bh * a.T + t0;   // global token row of the chunk's first token
  constexpr bool FWD = (MODE & kPrepFwd) != 0, BWD = (MODE & kPrepBwd) != 0;
  T* gWn = reinterpret_cast<T*>(a.f.Wn) + ci * LC * D;
  T* gQt = reinterpret_cast<T*>(a.f.Qt) + ci * LC * D;
  T* gKfT = reinterpret_cast<T*>(a.f.KfT) + ci * D * LC;
  T* gUbT = reinterpret_cast<T*>(a.f.UbT) + ci * D * LC;
  T* gOiT = FWD ? reinterpret_cast<T*>(a.f.OiT) + ci * D * LC : nullptr;

  // ---- gate pass, in log space.  G_r = sum_{t<=r} la_t inside the chunk (la <= 0).  A
  // chunk whose G_L stays above -kChunkSafe in every key channel refers its operands to
  // the chunk start (fast path below).  Otherwise (range-safe path): Gb[I] is G at
  // the start of 16-token block I (Gb[0] = 0) and btot_I = Gb[I+1] - Gb[I] <= 0 the
  // block's log-retention.  Per element, with loc = G_r - Gb[I(r)] in [btot, 0]:
  //   K^+ = k e^loc, Q^+ = q e^loc        row operands of the coupling tiles (<= |k|, |q|)
  //   K^- = k e^(btot - loc)              column operand, referred to the block end (<= |k|)
  //   K^d = k e^-loc                      column operand of the diagonal tiles (>= |k|,
  //                                       finite while -btot <= kSafeLog)
  //   Kw = w k e^(Gb + loc), K-> = k e^(G_L - Gb[I+1]) e^(btot - loc)   (chunk references)
  // so a tile (I, J) of the coupling is K^+_I D_IJ K^-_J^T with D_IJ = 1 for J = I - 1,
  // the retention between the end of block J and the start of block I (<= 1) for
  // J <= I - 2, and K^+_I K^d_I^T on the diagonal: every retention ratio Gamma_r/Gamma_s
  // is a product of factors <= 1, except inside a diagonal block, which the exact path
  // below takes over when its decay leaves the safe range.  Raw k, q, v are read from
  // their slots; with at least four tokens per part a thread takes two adjacent key
  // channels so that every row-major LDS access moves both.
  const float* laS = reinterpret_cast<const float*>(smem + Lay::R3);
  const T* Vraw = reinterpret_cast<const T*>(smem + Lay::R6);
  T* Kd = reinterpret_cast<T*>(smem + Lay::R6);       // diagonal-tile operand, written over raw v
  int* flags = reinterpret_cast<int*>(smem + Lay::R8);
  float* gbeT = reinterpret_cast<float*>(smem + Lay::R8 + 16 * sizeof(int));   // [NB][D] e^Gb
  T* Kfar = reinterpret_cast<T*>(smem + Lay::R9);                                // [NFAR][16][LDD]
  constexpr int CPT = (LC * D / (2 * NT)) % 4 == 0 && LC * D / (2 * NT) >= 4 ? 2 : 1;
  constexpr int PG = CPT * NT / D, RG = LC / PG;   // token parts, tokens per part
  static_assert(RG % 4 == 0 && PG * D <= 2 * P * D, "token parts must hold whole groups of 4");
  static_assert(RG <= 16 && 16 % RG == 0, "a token part must lie inside one 16-token block");
  constexpr int PB = 16 / RG;                      // parts per block
  const int ch = CPT * (tid % (D / CPT)), pid = tid / (D / CPT), r0 = pid * RG;
  const int blk = pid / PB, pf = blk * PB;         // the part's block and that block's first part
  float gl[CPT][RG];                               // inclusive sums of la inside the part
  {
    float run[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) run[c] = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const float* ar = laS + (r0 + i) * D + ch;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        run[c] += ar[c];
        gl[c][i] = run[c];
      }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) part[pid * D + ch + c] = run[c];
  }
  __syncthreads();
  // per channel: the parts before the block (gst = Gb), the block's parts before this
  // one (bpre), the whole block (btot) and the parts after it (gaf = G_L - Gb[I+1])
  float bpre[CPT], btot[CPT], gst[CPT], gaf[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) bpre[c] = btot[c] = gst[c] = gaf[c] = 0.f;
#pragma unroll
  for (int pp = 0; pp < PG; ++pp) {
    const bool before = pp < pf, inblk = !before && pp < pf + PB, mine = inblk && pp < pid;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const float pt = part[pp * D + ch + c];
      gst[c] += before ? pt : 0.f;
      btot[c] += inblk ? pt : 0.f;
      bpre[c] += mine ? pt : 0.f;
      gaf[c] += (!before && !inblk) ? pt : 0.f;
    }
  }
  // the chunk's path: a key channel whose log-retention over the whole chunk falls
  // below -kChunkSafe sends the chunk down the range-safe path (flag word 15)
  if (pid == 0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (-(btot[c] + gaf[c]) > kChunkSafe) flags[15] = 1;
  }
  __syncthreads();
  const bool wide = flags[15] != 0;
  if (BWD && tid == 0) a.f.cflag[ci] = wide ? 1 : 0;
  if (!wide) {
    // ---- fast path: the retention referred to the chunk start, Gamma_r = e^G_r >= e^-kChunkSafe,
    //   K+ = k Gamma, K- = k / Gamma, Q+ = q Gamma, K-> = k Gamma_L / Gamma
    // (every coupling tile is K+_I K-_J^T, each product of a ratio Gamma_r / Gamma_s <= 1
    // formed from two factors inside float range)
    float egl[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) egl[c] = fexp(gst[c] + btot[c] + gaf[c]);
    float kf[CPT][RG], kw[CPT][RG], vw[CPT][RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int r = r0 + i;
      float kv[CPT], qv[CPT], vv[CPT], kp[CPT], km[CPT], qp[CPT];
      ld_row<T, CPT>(Kp + r * LDD + ch, kv);       // staged raw, 0 past the end
      ld_row<T, CPT>(Qp + r * LDD + ch, qv);
      ld_row<T, CPT>(Vraw + r * LDD + ch, vv);
      const float wr = wL[r];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const float gam = fexp(gst[c] + bpre[c] + gl[c][i]);
        const float inv = __builtin_amdgcn_rcpf(gam);
        kp[c] = kv[c] * gam;
        km[c] = kv[c] * inv;
        qp[c] = qv[c] * gam;
        kw[c][i] = wr * kp[c];
        vw[c][i] = wr * vv[c];
        kf[c][i] = kv[c] * (egl[c] * inv);
      }
      st_row<T, CPT>(Kp + r * LDD + ch, kp);
      st_row<T, CPT>(Km + r * LDD + ch, km);
      st_row<T, CPT>(Qp + r * LDD + ch, qp);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
#pragma unroll
      for (int t = 0; t < RG / 4; ++t) {
        store4(KwT + (ch + c) * LDL + r0 + 4 * t, f32x4{kw[c][4 * t], kw[c][4 * t + 1], kw[c][4 * t + 2], kw[c][4 * t + 3]});
        store4(VwT + (ch + c) * LDL + r0 + 4 * t, f32x4{vw[c][4 * t], vw[c][4 * t + 1], vw[c][4 * t + 2], vw[c][4 * t + 3]});
      }
      const int cc = ch + c;
#pragma unroll
      for (int t = 0; t < RG / 4; ++t) {
        const int r = r0 + 4 * t;
        T* dst = gKfT + frag_offset<LC>(cc / 16, r / 32, cc % 16 + 16 * ((r % 32) / 8)) + r % 8;
        store4(dst, f32x4{kf[c][4 * t], kf[c][4 * t + 1], kf[c][4 * t + 2], kf[c][4 * t + 3]});
      }
      if (pid == 0) a.f.gL[ci * D + cc] = egl[c];
    }
  } else {
  // ---- range-safe path
  if (pid == pf) {
    // one part per block: the block's flag and its start retention e^Gb
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      if (-btot[c] > kSafeLog) flags[blk] = 1;
      gbeT[blk * D + ch + c] = fexp(gst[c]);
    }
  }
  // far-pair factors of this block as column block J: the retention from its end to the
  // start of block I = J + 2 + d
  constexpr int NFD = NB > 2 ? NB - 2 : 1;
  float dfar[CPT][NFD];
#pragma unroll
  for (int d = 0; d < NFD; ++d)
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float sm = 0.f;
#pragma unroll
      for (int pp = 0; pp < PG; ++pp) sm += (pp >= pf + PB && pp < (blk + 2 + d) * PB) ? part[pp * D + ch + c] : 0.f;
      dfar[c][d] = fexp(sm);
    }
  {
    float egs[CPT], ega[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      egs[c] = fexp(gst[c]);
      ega[c] = fexp(gaf[c]);
    }
    float kf[CPT][RG], kw[CPT][RG], vw[CPT][RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int r = r0 + i;
      float kv[CPT], qv[CPT], vv[CPT], kp[CPT], km[CPT], kd[CPT], qp[CPT];
      ld_row<T, CPT>(Kp + r * LDD + ch, kv);       // staged raw, 0 past the end
      ld_row<T, CPT>(Qp + r * LDD + ch, qv);
      ld_row<T, CPT>(Vraw + r * LDD + ch, vv);
      const float wr = wL[r];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const float loc = bpre[c] + gl[c][i];
        const float eo = fexp(loc), ee = fexp(btot[c] - loc);
        const float ed = __builtin_amdgcn_rcpf(fmaxf(eo, kMinOwn));
        kp[c] = kv[c] * eo;
        qp[c] = qv[c] * eo;
        km[c] = kv[c] * ee;
        kd[c] = kv[c] * ed;
        kw[c][i] = wr * kv[c] * (eo * egs[c]);
        vw[c][i] = wr * vv[c];
        kf[c][i] = kv[c] * (ee * ega[c]);
      }
      st_row<T, CPT>(Kp + r * LDD + ch, kp);
      st_row<T, CPT>(Km + r * LDD + ch, km);
      st_row<T, CPT>(Qp + r * LDD + ch, qp);
      st_row<T, CPT>(Kd + r * LDD + ch, kd);       // over the raw v this thread just read
#pragma unroll
      for (int d = 0; d < NB - 2; ++d) {
        if (blk + 2 + d < NB) {                    // far tile (blk + 2 + d, blk)
          float kx[CPT];
#pragma unroll
          for (int c = 0; c < CPT; ++c) kx[c] = km[c] * dfar[c][d];
          st_row<T, CPT>(Kfar + (far_index(blk + 2 + d, blk) * 16 + r % 16) * LDD + ch, kx);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      // Kw^T and Vw^T rows (key channel ch + c) take this thread's RG consecutive tokens
#pragma unroll
      for (int t = 0; t < RG / 4; ++t) {
        store4(KwT + (ch + c) * LDL + r0 + 4 * t, f32x4{kw[c][4 * t], kw[c][4 * t + 1], kw[c][4 * t + 2], kw[c][4 * t + 3]});
        store4(VwT + (ch + c) * LDL + r0 + 4 * t, f32x4{vw[c][4 * t], vw[c][4 * t + 1], vw[c][4 * t + 2], vw[c][4 * t + 3]});
      }
      // K->^T in fragment order, 4 tokens at a time (rounded to the operand type)
      const int cc = ch + c;
#pragma unroll
      for (int t = 0; t < RG / 4; ++t) {
        const int r = r0 + 4 * t;
        T* dst = gKfT + frag_offset<LC>(cc / 16, r / 32, cc % 16 + 16 * ((r % 32) / 8)) + r % 8;
        store4(dst, f32x4{kf[c][4 * t], kf[c][4 * t + 1], kf[c][4 * t + 2], kf[c][4 * t + 3]});
      }
      if (pid == 0) a.f.gL[ci * D + cc] = fexp(btot[c] + gaf[c]);   // Gamma_L = e^(G_L)
    }
  }
  }   // range-safe path
  __syncthreads();

  // ---- coupling A = strict_tril(diag(w) B), B_rs = sum_ch k_r k_s Gamma_r/Gamma_s (fp32),
  // and P = tril(sum_ch q_r k_s Gamma_r/Gamma_s), tile (I, J) from K^+_I (A) or Q^+_I (P)
  // against K^d_I (J = I), K^-_J (J = I - 1) or K^-_J scaled by the far-pair factor.
  // Wave w takes tiles w, w + NW, ... (A tiles first, then P); all of its operand
  // fragments are loaded before its first product (a wave past the last tile reloads
  // that tile and skips the product).  The backward modes also keep B (acc order).
  constexpr int NTRI = NB * (NB + 1) / 2, NTILE = 2 * NTRI, TPW = (NTILE + NW - 1) / NW, KD = D / 32;
  T* gB = BWD ? reinterpret_cast<T*>(a.f.Bt) + ci * LC * LC : nullptr;
  {
    Frag<T> fa[TPW][KD], fb[TPW][KD];
    int ti[TPW], tj[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = min(wave + NW * m, NTILE - 1);
      tri_index(t < NTRI ? t : t - NTRI, ti[m], tj[m]);
      const T* Ar = (t < NTRI ? Kp : Qp) + 16 * ti[m] * LDD;
      const T* Br = !wide || ti[m] == tj[m] + 1 ? Km + 16 * tj[m] * LDD
                  : ti[m] == tj[m] ? Kd + 16 * tj[m] * LDD
                  : Kfar + far_index(ti[m], tj[m]) * 16 * LDD;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        fa[m][kk] = load_frag(Ar + lr * LDD + 32 * kk + 8 * lg);
        fb[m][kk] = load_frag(Br + lr * LDD + 32 * kk + 8 * lg);
      }
    }
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = wave + NW * m;
      if (t >= NTILE) continue;
      const bool isA = t < NTRI;
      const int i = ti[m], j = tj[m];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) mma(acc, fa[m][kk], fb[m][kk]);
      const int s = 16 * j + lr;
      if (isA) {
        f32x4 bm;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * i + 4 * lg + ii;
          bm[ii] = (s < r) ? acc[ii] : 0.f;
          Af[r * LDF + s] = wL[r] * bm[ii];
        }
        if (BWD && wide && !(i == j && flags[i])) store4(gB + ((size_t)t * 64 + lane) * 4, bm);
      } else {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[ii] = (s <= 16 * i + 4 * lg + ii) ? acc[ii] : 0.f;
        lds_store_acc_tile(Pb, LDL, 16 * i, 16 * j, acc);
        // the products with P run over 32-token blocks: block (i, i+1) of an even row
        // tile i is read by them and must be zero
        if (j == i && i % 2 == 0 && i + 1 < NB) lds_zero_tile(Pb, LDL, 16 * i, 16 * (i + 1));
      }
    }
  }
  __syncthreads();
  // exact diagonal tiles of the blocks beyond the fast tiles' range (range-safe path only)
  if (wide) {
#pragma unroll
    for (int I = 0; I < NB; ++I)
      if (flags[I]) prep_diag_exact<T, LC, D, Gates, NT>(a, gates, bh, c, I, smem, Af, Pb, gB);
  }

  // ---- T = (I + A)^-1 (fp32), then a dtype copy for the WY products; the backward
  // modes also keep that copy and P of the chunk (row-major [LC][LC]).  The solve is an
  // out-of-line call in every mode (inlined, its registers add to the persistent loop's
  // prefetch and spill)
  triangular_inverse<LC, LDF, NT>((lds_float*)Af, (lds_float*)Tf);
  after_solve();
  for (int idx = tid; idx < LC * LC / 4; idx += NT) {
    const int r = idx / (LC / 4), s = 4 * (idx % (LC / 4));
    const f32x4 t4 = ((s >> 4) > (r >> 4)) ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(Tf + r * LDF + s);
    store4(Tb + r * LDL + s, t4);
    if (BWD) {
      store4(reinterpret_cast<T*>(a.f.Tt) + (ci * LC + r) * LC + s, t4);
      if (wide) {   // the range-safe backward takes P from here
        const f32x4 p4 = ((s >> 4) > (r >> 4)) ? f32x4{0.f, 0.f, 0.f, 0.f} : load4f(Pb + r * LDL + s);
        store4(reinterpret_cast<T*>(a.f.Pt) + (ci * LC + r) * LC + s, p4);
      }
    }
  }
  __syncthreads();

  // ---- WY factors: W = T Kw, Ubar = T Vw  (Kw = diag(w) K+, Vw = diag(w) V)
  if constexpr (NW == NCT) {
    // one wave per key/value column tile: its columns of Kw and Vw are loaded once and
    // every operand of the phase is in flight before the first product
    constexpr int KL = LC / 32;
    const int ct = wave, col = 16 * ct + lr;
    Frag<T> bw[KL], bu[KL], ta[NB][KL];
#pragma unroll
    for (int kb = 0; kb < KL; ++kb) {
      bw[kb] = load_frag(KwT + col * LDL + 32 * kb + 8 * lg);
      bu[kb] = load_frag(VwT + col * LDL + 32 * kb + 8 * lg);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int kb = 0; kb <= i / 2; ++kb) ta[i][kb] = load_frag(Tb + (16 * i + lr) * LDL + 32 * kb + 8 * lg);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      f32x4 aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= i / 2; ++kb) {
        mma(aw, ta[i][kb], bw[kb]);
        mma(au, ta[i][kb], bu[kb]);
      }
      const int r = 16 * i + 4 * lg;
      store4(WnT + col * LDL + r, -aw);
      store4(UbTs + col * LDL + r, au);
      store4(gUbT + acc_offset<D>(i, ct, lane), au);
    }
  } else
  for (int t = wave; t < 2 * NB * NCT; t += NW) {
    const bool isW = t < NB * NCT;
    const int tt = isW ? t : t - NB * NCT;
    const int i = tt / NCT, ct = tt % NCT;
    const T* Bs = isW ? KwT : VwT;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < 16 * (i + 1); kk += 32) {
      const Frag<T> fa = load_frag(Tb + (16 * i + lr) * LDL + kk + 8 * lg);
      const Frag<T> fb = load_frag(Bs + (16 * ct + lr) * LDL + kk + 8 * lg);
      mma(acc, fa, fb);
    }
    const int col = 16 * ct + lr, r = 16 * i + 4 * lg;
    if (isW) {
      store4(WnT + col * LDL + r, -acc);
    } else {
      store4(UbTs + col * LDL + r, acc);
      store4(gUbT + acc_offset<D>(i, ct, lane), acc);
    }
  }
  __syncthreads();
  // -W out of LDS in fragment order, rows = tokens
  for_wave_items<NB * (D / 32), NW>(wave, [&](int f) {
    const int rt = f / (D / 32), kb = f % (D / 32);
    *reinterpret_cast<Frag<T>*>(gWn + frag_offset<D>(rt, kb, lane)) = lds_frag_cols(WnT, LDL, 16 * rt, 32 * kb);
  });

  // ---- intra-chunk output P Ubar and Q~ = Q+ - P W
  if constexpr (NW == NCT) {
    // one wave per column tile, as above: P's row blocks serve both products
    constexpr int KL = LC / 32;
    const int ct = wave, col = 16 * ct + lr;
    Frag<T> bo[KL], bq[KL], pa[NB][KL];
#pragma unroll
    for (int kb = 0; kb < KL; ++kb) {
      if (FWD) bo[kb] = load_frag(UbTs + col * LDL + 32 * kb + 8 * lg);
      bq[kb] = load_frag(WnT + col * LDL + 32 * kb + 8 * lg);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int kb = 0; kb <= i / 2; ++kb) pa[i][kb] = load_frag(Pb + (16 * i + lr) * LDL + 32 * kb + 8 * lg);
    f32x4 aq[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      aq[i] = lds_acc_tile(Qp, LDD, 16 * i, 16 * ct);
      if (wide) aq[i] *= gbeT[i * D + col];   // Q+ = Q^+ e^Gb
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      f32x4 ao = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= i / 2; ++kb) {
        if (FWD) mma(ao, pa[i][kb], bo[kb]);
        mma(aq[i], pa[i][kb], bq[kb]);
      }
      if (FWD) store4(gOiT + acc_offset<D>(i, ct, lane), ao);
      store4(QtTs + col * LDL + 16 * i + 4 * lg, aq[i]);
    }
  } else
  for (int t = FWD ? wave : wave + NB * NCT; t < 2 * NB * NCT; t += NW) {
    const bool isO = t < NB * NCT;
    const int tt = isO ? t : t - NB * NCT;
    const int i = tt / NCT, ct = tt % NCT;
    const int col = 16 * ct + lr, r = 16 * i + 4 * lg;
    f32x4 acc;
    if (isO) {
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      acc = lds_acc_tile(Qp, LDD, 16 * i, 16 * ct);
      if (wide) acc *= gbeT[i * D + col];   // Q+ = Q^+ e^Gb
    }
    const T* Bs = isO ? UbTs : WnT;
    for (int kk = 0; kk < 16 * (i + 1); kk += 32) {
      const Frag<T> fa = load_frag(Pb + (16 * i + lr) * LDL + kk + 8 * lg);
      const Frag<T> fb = load_frag(Bs + (16 * ct + lr) * LDL + kk + 8 * lg);
      mma(acc, fa, fb);
    }
    if (isO) store4(gOiT + acc_offset<D>(i, ct, lane), acc);
    else store4(QtTs + col * LDL + r, acc);
  }
  __syncthreads();
  // Q~ out of LDS in fragment order, rows = tokens
  for_wave_items<NB * (D / 32), NW>(wave, [&](int f) {
    const int rt = f / (D / 32), kb = f % (D / 32);
    *reinterpret_cast<Frag<T>*>(gQt + frag_offset<D>(rt, kb, lane)) = lds_frag_cols(QtTs, LDL, 16 * rt, 32 * kb);
  });
}


// Workgroups are dispatched round-robin over the 8 XCDs (block id mod 8), each
// with its own L2.  The value slices of one (batch, head) read the same chunk
// factors, so they are mapped to one XCD: block b -> XCD x = b % 8, i = b / 8,
// head bh = (i / nslices) * 8 + x, slice = i % nslices (when B*H is a multiple of 8).
__device__ __forceinline__ void xcd_slice_map(int nslices, int BH, int& bh, int& slice) {
  const int b = blockIdx.x;
  if (BH % 8 == 0) {
    const int x = b % 8, i = b / 8;
    bh = (i / nslices) * 8 + x;
    slice = i % nslices;
  } else {
    bh = b / nslices;
    slice = b % nslices;
  }
}

// State tiles of a workgroup holding VS value rows of a D x D state: lane l of
// tile (ct, vt) holds S[16 vt + l%16][16 ct + 4 (l/16) + i], i = 0..3
// (accumulator layout of S^T); wave w owns tiles w*SPW .. w*SPW+SPW-1.
template <int D, int VS, int NW = kWaves>
struct StateTiles {
  static constexpr int NVT = VS / 16, NCT = D / 16;
  static constexpr int SPW = NCT * NVT / NW;       // state tiles per wave
  static_assert(NCT * NVT % NW == 0, "state tiles must split evenly over waves");
  static_assert(SPW % NVT == 0 || NVT % SPW == 0, "a wave's tiles must cover whole key tiles or part of one");
  static constexpr int SCT = SPW >= NVT ? SPW / NVT : 1;   // key tiles a wave touches
  // key tile of the wave's tile j, relative to the wave's first key tile
  static constexpr int jc(int j) { return SPW >= NVT ? j / NVT : 0; }
};

// The D x D state matrices handed to the chunk-gradient kernel, M[v][k], use the
// fragment order of frag_offset with rows v and contraction k ("vk").

// Scatter one accumulator group (lane (lr, lg) of state tile (vt, ct): the four
// values M[16 vt + lr][16 ct + 4 lg + i]) into the "vk" fragment order.
template <typename T, int D>
__device__ __forceinline__ void store_vk_group(T* vk, int vt, int ct, f32x4 x_vk) {
  const int lane = lane_id(), lr = lane & 15, lg = lane >> 4;
  store4(vk + frag_offset<D>(vt, ct >> 1, lr + 16 * (2 * (ct & 1) + (lg >> 1))) + 4 * (lg & 1), x_vk);
}

// Value slices of 32 or more rows copy whole fragments (and outputs) out of their
// LDS copies with 16-byte stores (a fragment spans 32 rows of the slice).
template <int VS> constexpr bool kWideSlice = VS >= 32;

// Operand of a contraction over v from the "vk" fragment order: the fragment for
// rows k = 16 kc .. 16 kc + 15 and v block kb, lane c + 16 g receiving
// M[32 kb + 8 g + e][16 kc + c], e = 0..7.  It is loaded as raw pieces (issued early)
// and finished where it is used.
//   bf16: two identity transposes (transpose_tile16), t = 0, 1; for transpose t, input
//   row r carries M[32 kb + 8 (r / 4) + 4 t + r % 4][16 kc + 4 g ..], an 8-byte piece of
//   stored lane (row % 16) + 16 (2 (kc % 2) + g / 2) at element 4 (g % 2), so that
//   output value i of lane c + 16 g is M[32 kb + 8 g + 4 t + i][16 kc + c].
//   fp32: eight element reads per lane, already in place.
template <typename T> struct KmajorPieces;
template <> struct KmajorPieces<bf16> { bf16x4 h[2]; };
template <> struct KmajorPieces<float> { Frag<float> f; };

template <int D>
__device__ __forceinline__ KmajorPieces<bf16> load_kmajor_pieces(const bf16* vk, int kc, int kb) {
  const int lane = lane_id(), r = lane & 15, g = lane >> 4;
  KmajorPieces<bf16> p;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int v = 8 * (r >> 2) + 4 * t + (r & 3);          // row inside the 32-row block
    p.h[t] = *reinterpret_cast<const bf16x4*>(
        vk + frag_offset<D>(2 * kb + (v >> 4), kc >> 1, (v & 15) + 16 * (2 * (kc & 1) + (g >> 1))) + 4 * (g & 1));
  }
  return p;
}
template <int D>
__device__ __forceinline__ KmajorPieces<float> load_kmajor_pieces(const float* vk, int kc, int kb) {
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  const int cc = 16 * (kc & 1) + c;      // column inside the 32-wide k block
  KmajorPieces<float> p;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int v = 8 * g + e;
    const float x = vk[frag_offset<D>(2 * kb + (v >> 4), kc >> 1, (v & 15) + 16 * (cc >> 3)) + (cc & 7)];
    if (e < 4) p.f.lo[e] = x;
    else p.f.hi[e - 4] = x;
  }
  return p;
}
__device__ __forceinline__ Frag<bf16> kmajor_frag(const KmajorPieces<bf16>& p) {
  const bf16x4 lo = transpose_tile16(p.h[0]), hi = transpose_tile16(p.h[1]);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> kmajor_frag(const KmajorPieces<float>& p) { return p.f; }

}  // namespace carve
