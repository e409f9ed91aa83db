// Backward kernels of the CARVE key-axis gated delta rule on gfx950.
//
// The backward of the token-only forward runs as
//   1. fwd_prep (backward layouts)          chunk factors, all chunks in parallel
//   2. fwd_state without output             S_c, the state entering every chunk
//   3. bwd_state (this file)                reverse pass over chunks:
//        dS_c = dS_{c+1} Diag(Gamma_L) - (dS_{c+1} K->^T) W + dO_c^T Q~
//      which stores dS_{c+1} (gradient w.r.t. the state leaving chunk c)
//   4. bwd_chunk (this file)                all chunks in parallel: with S_c and
//      dS_{c+1} known, the chunk's gradients follow from the chunk algebra of
//      carve_chunk.h by reverse-mode differentiation (dU, dP, dW, dT, dA = -T^T dT T^T,
//      the coupling's dB, then the key-axis retention through a reverse cumulative
//      sum of dlog a inside the chunk).
// Gradients are w.r.t. log g, the erase probability b and the write strength w.
#include "carve_chunk.h"

namespace carve {

// ------------------------------------------------------------------ fragments
// Fragment of rows row0..row0+15 of a logical [rows][K] matrix X at k block k0:
// TR = false: X stored row-major (X[r][k] at base[r*ld + k]);
// TR = true : X stored transposed (X[r][k] at base[k*ld + r]).
template <bool TR, typename T>
__device__ __forceinline__ Frag<T> frag(const T* base, int ld, int row0, int k0) {
  const int lane = lane_id(), lr = lane & 15, lg = lane >> 4;
  if (!TR) return load_frag(base + (size_t)(row0 + lr) * ld + k0 + 8 * lg);
  return load_frag_strided(base + (size_t)(k0 + 8 * lg) * ld + row0 + lr, ld);
}

// Same from an fp32 matrix in global memory, converted to the operand type,
// optionally scaled per k by kscale[k].
template <bool TR, typename T>
__device__ __forceinline__ Frag<T> frag32(const float* base, int ld, int row0, int k0, const float* kscale) {
  const int lane = lane_id(), lr = lane & 15, lg = lane >> 4;
  float x[8];
  if (!TR) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(base + (size_t)(row0 + lr) * ld + k0 + 8 * lg);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(base + (size_t)(row0 + lr) * ld + k0 + 8 * lg + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = lo[j]; x[j + 4] = hi[j]; }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = base[(size_t)(k0 + 8 * lg + j) * ld + row0 + lr];
  }
  if (kscale) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= kscale[k0 + 8 * lg + j];
  }
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = (bf16)x[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) { f.lo[j] = x[j]; f.hi[j] = x[j + 4]; }
  }
  return f;
}

__device__ __forceinline__ bf16 frag_elem(const Frag<bf16>& f, int e) { return f.v[e]; }
__device__ __forceinline__ float frag_elem(const Frag<float>& f, int e) { return e < 4 ? f.lo[e] : f.hi[e - 4]; }

// ------------------------------------------------------------------ reverse state pass
template <typename T, int LC, int D, int VS>
struct RevLayout {
  static constexpr int LDS_ = D + Pad<T>::v;
  static constexpr int LDU = LC + Pad<T>::v;
  static constexpr size_t bytes = sizeof(T) * (VS * LDS_ + 2 * VS * LDU);
};

// Global operands of one chunk for one wave (loaded one chunk ahead):
//   X^T tiles [s][v] = K-> dS^T: wave w owns tiles tix = w*XPW + u (one row tile of s)
//   dS^T tiles [k][v]: wave w owns key tiles ct = w*SCT + j
//   the chunk's dO slice (LC x VS), spread over all threads
template <typename T, int LC, int D, int VS>
struct RevOps {
  static constexpr int NVT = VS / 16, NB = LC / 16, NCT = D / 16;
  static constexpr int NX = NB * NVT;
  static constexpr int XPW = (NX + kWaves - 1) / kWaves;
  static constexpr int SCT = NCT / kWaves;
  static constexpr int KD = D / 32, KL = LC / 32;
  static constexpr int VEC = 8;                                   // elements per fragment-sized piece
  static constexpr int NDO = (LC * VS / VEC + kThreads - 1) / kThreads;
  static_assert(NVT % XPW == 0, "a wave's X tiles must share one row tile");
  Frag<T> kf[KD];
  Frag<T> wt[SCT][KL];
  Frag<T> qt[SCT][KL];
  f32x4 gl[SCT];
  Frag<T> dov[NDO];   // raw 16-byte pieces of dO: VEC consecutive value columns of one token

  __device__ __forceinline__ void load(const BwdArgs& a, int bh, int c, int v0) {
    const FwdArgs& f = a.fwd;
    const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
    const size_t ci = (size_t)bh * f.NC + c;
    const T* Kf = reinterpret_cast<const T*>(f.f.Kf);
    const T* WnT = reinterpret_cast<const T*>(f.f.WnT);
    const T* QtT = reinterpret_cast<const T*>(f.f.QtT);
    const int t0 = wave * XPW;
    if (t0 < NX) {
      const int rt = t0 / NVT;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) kf[kk] = load_frag(Kf + (ci * LC + 16 * rt + lr) * D + 32 * kk + 8 * lg);
    }
#pragma unroll
    for (int j = 0; j < SCT; ++j) {
      const int ct = wave * SCT + j;
      gl[j] = load4f(f.f.gL + ci * D + 16 * ct + 4 * lg);
#pragma unroll
      for (int kk = 0; kk < KL; ++kk) {
        wt[j][kk] = load_frag(WnT + (ci * D + 16 * ct + lr) * LC + 32 * kk + 8 * lg);
        qt[j][kk] = load_frag(QtT + (ci * D + 16 * ct + lr) * LC + 32 * kk + 8 * lg);
      }
    }
    const T* dO = reinterpret_cast<const T*>(a.dO);
    const int n = min(LC, f.T - c * LC);
#pragma unroll
    for (int u = 0; u < NDO; ++u) {
      const int idx = threadIdx.x + kThreads * u;            // piece index: token r, column group g
      const int r = idx / (VS / VEC), g = idx % (VS / VEC);
      if (idx < LC * VS / VEC) {
        const int rr = min(r, n - 1);
        dov[u] = load_frag(dO + ((size_t)bh * f.T + c * LC + rr) * D + v0 + VEC * g);
        if (r >= n) dov[u] = zero_frag(T());
      }
    }
  }
};

template <typename T, int LC, int D, int VS>
__global__ __launch_bounds__(kThreads) void bwd_state_kernel(BwdArgs a) {
  using Lay = RevLayout<T, LC, D, VS>;
  using Op = RevOps<T, LC, D, VS>;
  using ST = StateTiles<D, VS>;
  constexpr int NVT = ST::NVT, SPW = ST::SPW, LDS_ = Lay::LDS_, LDU = Lay::LDU;
  constexpr int VEC = Op::VEC;
  extern __shared__ __align__(16) unsigned char smem[];
  T* dSb = reinterpret_cast<T*>(smem);
  T* XT = dSb + VS * LDS_;
  T* dOT = XT + VS * LDU;
  const FwdArgs& f = a.fwd;
  const int slice = blockIdx.x, bh = blockIdx.y;
  const int v0 = slice * VS;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;

  f32x4 dS[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int st = wave * SPW + j, ct = st / NVT, vt = st % NVT;
    const int vl = 16 * vt + lr, kc = 16 * ct + 4 * lg;
    if (a.dS_T) dS[j] = load4f(a.dS_T + ((size_t)bh * D + v0 + vl) * D + kc);
    else dS[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    store4(dSb + vl * LDS_ + kc, dS[j]);
  }
  Op cur, nxt;
  cur.load(a, bh, f.NC - 1, v0);
  __syncthreads();
  for (int c = f.NC - 1; c >= 0; --c) {
    const size_t ci = (size_t)bh * f.NC + c;
    if (c > 0) nxt.load(a, bh, c - 1, v0);
    // gradient w.r.t. the state leaving chunk c
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int st = wave * SPW + j, ct = st / NVT, vt = st % NVT;
      store4(a.dS_chunk + (ci * D + v0 + 16 * vt + lr) * D + 16 * ct + 4 * lg, dS[j]);
    }
    // dO^T slice into LDS
#pragma unroll
    for (int u = 0; u < Op::NDO; ++u) {
      const int idx = threadIdx.x + kThreads * u;
      if (idx < LC * VS / VEC) {
        const int r = idx / (VS / VEC), g = idx % (VS / VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) dOT[(VEC * g + e) * LDU + r] = frag_elem(cur.dov[u], e);
      }
    }
    // X^T = K-> dS^T  (tiles [s][v])
    {
      const int t0 = wave * Op::XPW;
      if (t0 < Op::NX) {
        const int rt = t0 / NVT;
#pragma unroll
        for (int u = 0; u < Op::XPW; ++u) {
          const int vt = (t0 + u) % NVT;
          const int vl = 16 * vt + lr;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < Op::KD; ++kk) mma(acc, cur.kf[kk], load_frag(dSb + vl * LDS_ + 32 * kk + 8 * lg));
          store4(XT + vl * LDU + 16 * rt + 4 * lg, acc);
        }
      }
    }
    __syncthreads();
    // dS^T <- Diag(Gamma_L) dS^T + (-W)^T X^T + Q~^T dO
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      // wave*SPW is a multiple of NVT, so the key tile index within the wave is j / NVT
      const int jc = j / NVT, ct = wave * Op::SCT + jc, vt = j % NVT;
      const int kc = 16 * ct + 4 * lg, vl = 16 * vt + lr;
      dS[j] *= cur.gl[jc];
#pragma unroll
      for (int kk = 0; kk < Op::KL; ++kk) {
        mma(dS[j], cur.wt[jc][kk], load_frag(XT + vl * LDU + 32 * kk + 8 * lg));
        mma(dS[j], cur.qt[jc][kk], load_frag(dOT + vl * LDU + 32 * kk + 8 * lg));
      }
      store4(dSb + vl * LDS_ + kc, dS[j]);
    }
    __syncthreads();
    cur = nxt;
  }
  if (a.dS0) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int st = wave * SPW + j, ct = st / NVT, vt = st % NVT;
      store4(a.dS0 + ((size_t)bh * D + v0 + 16 * vt + lr) * D + 16 * ct + 4 * lg, dS[j]);
    }
  }
}

// ------------------------------------------------------------------ chunk gradients
// LDS slots (reused as the computation proceeds; "row-major" = [token][width]):
//   s0 K+            s1 K-            s2 Q+ -> dW        s3 V (raw)
//   s4 A (fp32) -> -W -> dO             s5 T (fp32) -> U    s6 T-solve scratch -> dU
//   p0 P -> dT        p1 T (dtype)     p2 Tw = T diag(w)  p3 dP -> Z -> dA
// Tiles of [token][key] and [token][value] results are owned by column: wave w
// computes every token tile of key/value tiles ct = w*CPW .. w*CPW+CPW-1, so the
// cumulative retention Gamma of those columns stays in that wave's registers
// (accumulator layout) for the elementwise tail and the reverse cumulative sum.
template <typename T, int LC, int D>
struct GradLayout {
  static constexpr int LDD = D + Pad<T>::v;
  static constexpr int LDL = LC + Pad<T>::v;
  static constexpr int LDF = LC + 4;
  static constexpr int NB = LC / 16;
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t x) { return (x + 255) & ~size_t(255); }
  static constexpr size_t S1 = al(cmax(cmax(sizeof(T) * LC * LDD, sizeof(float) * LC * LDF),
                                      sizeof(float) * kWaves * 16 * 20));   // also holds the T-solve scratch
  static constexpr size_t S2 = al(sizeof(T) * LC * LDL);
  static constexpr size_t slot(int i) { return S1 * i; }
  static constexpr size_t pslot(int i) { return 7 * S1 + S2 * i; }
  static constexpr size_t small = 7 * S1 + 4 * S2;                  // w, Gamma_L, dw partials, G_L term
  static constexpr size_t bytes = small + sizeof(float) * (LC + D + 2 * NB * LC + D);
};

template <typename T, int LC, int D, bool HAS_B>
__global__ __launch_bounds__(kThreads) void bwd_chunk_kernel(BwdArgs a) {
  using Lay = GradLayout<T, LC, D>;
  constexpr int NB = LC / 16, NCT = D / 16, CPW = NCT / kWaves;
  constexpr int LDD = Lay::LDD, LDL = Lay::LDL, LDF = Lay::LDF;
  constexpr int NTRI = NB * (NB + 1) / 2;
  static_assert(NCT % kWaves == 0, "key tiles must split evenly over waves");
  extern __shared__ __align__(16) unsigned char smem[];
  T* Kp = reinterpret_cast<T*>(smem + Lay::slot(0));
  T* Km = reinterpret_cast<T*>(smem + Lay::slot(1));
  T* Qp = reinterpret_cast<T*>(smem + Lay::slot(2));
  T* dWr = Qp;
  T* Vr = reinterpret_cast<T*>(smem + Lay::slot(3));
  float* Af = reinterpret_cast<float*>(smem + Lay::slot(4));
  T* Wn = reinterpret_cast<T*>(smem + Lay::slot(4));
  T* dOr = Wn;
  float* Tf = reinterpret_cast<float*>(smem + Lay::slot(5));
  T* Ur = reinterpret_cast<T*>(smem + Lay::slot(5));
  float* scratch = reinterpret_cast<float*>(smem + Lay::slot(6));
  T* dUr = reinterpret_cast<T*>(smem + Lay::slot(6));
  T* Pb = reinterpret_cast<T*>(smem + Lay::pslot(0));
  T* dTb = Pb;
  T* Tb = reinterpret_cast<T*>(smem + Lay::pslot(1));
  T* Twb = reinterpret_cast<T*>(smem + Lay::pslot(2));
  T* dPb = reinterpret_cast<T*>(smem + Lay::pslot(3));
  T* Zb = dPb;
  T* dAb = dPb;
  float* wL = reinterpret_cast<float*>(smem + Lay::small);
  float* gLs = wL + LC;
  float* dwp = gLs + D;            // [NB][LC] column sums of T .* dT' per token-tile row
  float* dwq = dwp + NB * LC;      // [NB][LC] row sums of B .* dA per token-tile column
  float* glt = dwq + NB * LC;      // [D] G_L term per key column

  const FwdArgs& f = a.fwd;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
  const int n = min(LC, f.T - c * LC);
  const size_t ci = (size_t)bh * f.NC + c;
  const size_t row0 = (size_t)bh * f.T + (size_t)c * LC;
  const T* q = reinterpret_cast<const T*>(f.q);
  const T* k = reinterpret_cast<const T*>(f.k);
  const T* v = reinterpret_cast<const T*>(f.v);
  const T* dO = reinterpret_cast<const T*>(a.dO);
  const float* S = f.S_chunk + ci * D * D;        // state entering the chunk  [v][k]
  const float* dS = a.dS_chunk + ci * D * D;      // gradient w.r.t. the state leaving it [v][k]

  auto zero4 = []() { return f32x4{0.f, 0.f, 0.f, 0.f}; };

  // ---- gate pass in accumulator layout: lane holds rows 16 rt + 4 lg + i of column 16 ct + lr
  if (tid < LC) wL[tid] = (tid < n) ? f.w[row0 + min(tid, n - 1)] : 0.f;
  f32x4 gam[NB][CPW];     // cumulative retention Gamma inside the chunk
  float gLc[CPW];         // Gamma_L of the lane's columns
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int col = 16 * (wave * CPW + j) + lr;
    float run = 1.f;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        const size_t idx = (row0 + min(r, n - 1)) * D + col;
        const float lgv = f.log_g[idx];
        const float bv = HAS_B ? f.b[idx] : 1.f;
        av[i] = (r < n) ? __expf(lgv) * bv : 1.f;
      }
      float loc[4];
      loc[0] = av[0];
      loc[1] = loc[0] * av[1];
      loc[2] = loc[1] * av[2];
      loc[3] = loc[2] * av[3];
      // product of the 4-row groups of this row tile held by lanes with smaller lg
      float pre = run;
      float tile = 1.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float tg = __shfl(loc[3], lr + 16 * g);
        if (g < lg) pre *= tg;
        tile *= tg;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) gam[rt][j][i] = pre * loc[i];
      run *= tile;
    }
    gLc[j] = run;
    if (lg == 0) gLs[col] = run;
  }
  // operand matrices K+, K-, Q+ and raw V in LDS
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int col = 16 * (wave * CPW + j) + lr;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        const size_t idx = (row0 + min(r, n - 1)) * D + col;
        const bool valid = r < n;
        const float kv = valid ? tof(k[idx]) : 0.f;
        const float qv = valid ? tof(q[idx]) : 0.f;
        const float vv = valid ? tof(v[idx]) : 0.f;
        const float g = gam[rt][j][i];
        Kp[r * LDD + col] = to<T>(kv * g);
        Km[r * LDD + col] = to<T>(kv / g);
        Qp[r * LDD + col] = to<T>(qv * g);
        Vr[r * LDD + col] = to<T>(vv);
      }
    }
  }
  __syncthreads();

  // ---- A = strict_tril(diag(w) K+ K-^T) (fp32), P = tril(Q+ K-^T)
  for (int t = wave; t < 2 * NTRI; t += kWaves) {
    const bool isA = t < NTRI;
    int i, j;
    tri_index(isA ? t : t - NTRI, i, j);
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < D; kk += 32)
      mma(acc, frag<false>(isA ? Kp : Qp, LDD, 16 * i, kk), frag<false>(Km, LDD, 16 * j, kk));
    const int s = 16 * j + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 16 * i + 4 * lg + ii;
      if (isA) Af[r * LDF + s] = (s < r) ? wL[r] * acc[ii] : 0.f;
      else Pb[r * LDL + s] = to<T>((s <= r) ? acc[ii] : 0.f);
    }
  }
  for (int idx = tid; idx < LC * LC; idx += kThreads) {
    const int r = idx / LC, s = idx % LC;
    if ((s >> 4) > (r >> 4)) {
      Pb[r * LDL + s] = to<T>(0.f);
      dPb[r * LDL + s] = to<T>(0.f);
    }
  }
  __syncthreads();

  // ---- T = (I + A)^-1; dtype copies T and Tw = T diag(w)
  triangular_inverse<LC, LDF>(Af, Tf, scratch);
  for (int idx = tid; idx < LC * LC; idx += kThreads) {
    const int r = idx / LC, s = idx % LC;
    const float tv = Tf[r * LDF + s];
    Tb[r * LDL + s] = to<T>(tv);
    Twb[r * LDL + s] = to<T>(tv * wL[s]);
  }
  __syncthreads();

  // ---- W = Tw K+ (stored negated), Ubar = Tw V (kept in registers as U's accumulator)
  f32x4 acc2[NB][CPW];
#pragma unroll
  for (int kk = 0; kk < LC; kk += 32) {
    Frag<T> bk[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) bk[j] = frag<true>(Kp, LDD, 16 * (wave * CPW + j), kk);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const Frag<T> at = frag<false>(Twb, LDL, 16 * rt, kk);
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        if (kk == 0) acc2[rt][j] = zero4();
        mma(acc2[rt][j], at, bk[j]);
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < NB; ++rt)
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        Wn[(16 * rt + 4 * lg + ii) * LDD + 16 * (wave * CPW + j) + lr] = to<T>(-acc2[rt][j][ii]);
  f32x4 accU[NB][CPW];
#pragma unroll
  for (int kk = 0; kk < LC; kk += 32) {
    Frag<T> bv[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) bv[j] = frag<true>(Vr, LDD, 16 * (wave * CPW + j), kk);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const Frag<T> at = frag<false>(Twb, LDL, 16 * rt, kk);
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        if (kk == 0) accU[rt][j] = zero4();
        mma(accU[rt][j], at, bv[j]);
      }
    }
  }
  __syncthreads();

  // ---- U = Ubar + (-W) S^T  -> row-major U
#pragma unroll
  for (int kk = 0; kk < D; kk += 32) {
    Frag<T> bs[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) bs[j] = frag32<false, T>(S, D, 16 * (wave * CPW + j), kk, nullptr);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const Frag<T> at = frag<false>(Wn, LDD, 16 * rt, kk);
#pragma unroll
      for (int j = 0; j < CPW; ++j) mma(accU[rt][j], at, bs[j]);
    }
  }
#pragma unroll
  for (int rt = 0; rt < NB; ++rt)
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        Ur[(16 * rt + 4 * lg + ii) * LDD + 16 * (wave * CPW + j) + lr] = to<T>(accU[rt][j][ii]);
  __syncthreads();   // -W no longer needed: its slot takes dO

  // ---- dO into LDS (row-major, zero for tokens past the end)
  for (int idx = tid; idx < LC * D / 8; idx += kThreads) {
    const int r = idx / (D / 8), g = idx % (D / 8);
    Frag<T> x = (r < n) ? load_frag(dO + (row0 + r) * D + 8 * g) : zero_frag(T());
    *reinterpret_cast<Frag<T>*>(dOr + r * LDD + 8 * g) = x;
  }
  __syncthreads();

  // ---- dU = P^T dO + K- (dS' Diag(Gamma_L))^T  -> row-major dU
  {
    f32x4 acc[NB][CPW];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) acc[rt][j] = zero4();
#pragma unroll
    for (int kk = 0; kk < LC; kk += 32) {
      Frag<T> bo[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j) bo[j] = frag<true>(dOr, LDD, 16 * (wave * CPW + j), kk);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const Frag<T> at = frag<true>(Pb, LDL, 16 * rt, kk);
#pragma unroll
        for (int j = 0; j < CPW; ++j) mma(acc[rt][j], at, bo[j]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) {
      Frag<T> bs[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j) bs[j] = frag32<false, T>(dS, D, 16 * (wave * CPW + j), kk, gLs);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const Frag<T> at = frag<false>(Km, LDD, 16 * rt, kk);
#pragma unroll
        for (int j = 0; j < CPW; ++j) mma(acc[rt][j], at, bs[j]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          dUr[(16 * rt + 4 * lg + ii) * LDD + 16 * (wave * CPW + j) + lr] = to<T>(acc[rt][j][ii]);
  }
  // ---- dP = tril(dO U^T)
  for (int t = wave; t < NTRI; t += kWaves) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) mma(acc, frag<false>(dOr, LDD, 16 * i, kk), frag<false>(Ur, LDD, 16 * j, kk));
    const int s = 16 * j + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 16 * i + 4 * lg + ii;
      dPb[r * LDL + s] = to<T>((s <= r) ? acc[ii] : 0.f);
    }
  }
  __syncthreads();

  // ---- token x key gradients owned by this wave's columns
  f32x4 dKacc[NB][CPW];   // dk accumulated: Gamma dK+ + dK- / Gamma + (Gamma_L / Gamma) dK->
  f32x4 dGacc[NB][CPW];   // d G (gradient w.r.t. the cumulative log retention), per element
  f32x4 dKm[NB][CPW];     // dK- partial
  float gsum[CPW];        // sum over tokens of K-> .* dK-> per column (part of the G_L term)
  // dQ+ = dO S + dP K-  -> dq = Gamma dQ+, dG += q dq
  {
    f32x4 acc[NB][CPW];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) acc[rt][j] = zero4();
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) {
      Frag<T> bs[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j) bs[j] = frag32<true, T>(S, D, 16 * (wave * CPW + j), kk, nullptr);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const Frag<T> at = frag<false>(dOr, LDD, 16 * rt, kk);
#pragma unroll
        for (int j = 0; j < CPW; ++j) mma(acc[rt][j], at, bs[j]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < LC; kk += 32) {
      Frag<T> bk[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j) bk[j] = frag<true>(Km, LDD, 16 * (wave * CPW + j), kk);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const Frag<T> at = frag<false>(dPb, LDL, 16 * rt, kk);
#pragma unroll
        for (int j = 0; j < CPW; ++j) mma(acc[rt][j], at, bk[j]);
      }
    }
    T* dq = reinterpret_cast<T*>(a.dq);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int col = 16 * (wave * CPW + j) + lr;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          const float dqv = gam[rt][j][ii] * acc[rt][j][ii];
          const float qv = (r < n) ? tof(q[(row0 + min(r, n - 1)) * D + col]) : 0.f;
          dGacc[rt][j][ii] = qv * dqv;
          if (r < n) dq[(row0 + r) * D + col] = to<T>(dqv);
        }
    }
  }
  // dK-> = U dS'  -> dk += (Gamma_L / Gamma) dK->, dG -= k (Gamma_L / Gamma) dK->
  {
    f32x4 acc[NB][CPW];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) acc[rt][j] = zero4();
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) {
      Frag<T> bs[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j) bs[j] = frag32<true, T>(dS, D, 16 * (wave * CPW + j), kk, nullptr);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const Frag<T> at = frag<false>(Ur, LDD, 16 * rt, kk);
#pragma unroll
        for (int j = 0; j < CPW; ++j) mma(acc[rt][j], at, bs[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int col = 16 * (wave * CPW + j) + lr;
      float cs = 0.f;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          const float e3 = gLc[j] / gam[rt][j][ii] * acc[rt][j][ii];
          const float kv = (r < n) ? tof(k[(row0 + min(r, n - 1)) * D + col]) : 0.f;
          dKacc[rt][j][ii] = e3;
          dGacc[rt][j][ii] -= kv * e3;
          cs += kv * e3;
        }
      gsum[j] = cs;
    }
  }
  // dK- (first part) = dP^T Q+
  {
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) dKm[rt][j] = zero4();
#pragma unroll
    for (int kk = 0; kk < LC; kk += 32) {
      Frag<T> bq[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j) bq[j] = frag<true>(Qp, LDD, 16 * (wave * CPW + j), kk);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const Frag<T> at = frag<true>(dPb, LDL, 16 * rt, kk);
#pragma unroll
        for (int j = 0; j < CPW; ++j) mma(dKm[rt][j], at, bq[j]);
      }
    }
  }
  __syncthreads();   // Q+ is dead: its slot takes dW

  // ---- dW = -dU S  -> row-major dW
  {
    f32x4 acc[NB][CPW];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) acc[rt][j] = zero4();
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) {
      Frag<T> bs[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j) bs[j] = frag32<true, T>(S, D, 16 * (wave * CPW + j), kk, nullptr);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const Frag<T> at = frag<false>(dUr, LDD, 16 * rt, kk);
#pragma unroll
        for (int j = 0; j < CPW; ++j) mma(acc[rt][j], at, bs[j]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          dWr[(16 * rt + 4 * lg + ii) * LDD + 16 * (wave * CPW + j) + lr] = to<T>(-acc[rt][j][ii]);
  }
  __syncthreads();

  // ---- dT' = dW K+^T + dU V^T (lower tiles); dT = dT' diag(w); dw term sum_i T[i][r] dT'[i][r]
  for (int t = wave; t < NTRI; t += kWaves) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) {
      mma(acc, frag<false>(dWr, LDD, 16 * i, kk), frag<false>(Kp, LDD, 16 * j, kk));
      mma(acc, frag<false>(dUr, LDD, 16 * i, kk), frag<false>(Vr, LDD, 16 * j, kk));
    }
    const int s = 16 * j + lr;
    float cs = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 16 * i + 4 * lg + ii;
      dTb[r * LDL + s] = to<T>(acc[ii] * wL[s]);
      cs += tof(Tb[r * LDL + s]) * acc[ii];
    }
    cs += __shfl_xor(cs, 16);
    cs += __shfl_xor(cs, 32);
    if (lg == 0) dwp[i * LC + s] = cs;
  }
  for (int idx = tid; idx < LC * LC; idx += kThreads) {
    const int r = idx / LC, s = idx % LC;
    const int it = r >> 4, jt = s >> 4;
    if (jt > it) dTb[r * LDL + s] = to<T>(0.f);
    if (jt > it) dwp[it * LC + s] = 0.f;      // tiles above the diagonal contribute nothing
  }
  // ---- dV = Tw^T dU (write dv) and dK+ (first part) = Tw^T dW
  f32x4 dKp[NB][CPW];
  {
    f32x4 acc[NB][CPW];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) { acc[rt][j] = zero4(); dKp[rt][j] = zero4(); }
#pragma unroll
    for (int kk = 0; kk < LC; kk += 32) {
      Frag<T> bu[CPW], bw[CPW];
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        bu[j] = frag<true>(dUr, LDD, 16 * (wave * CPW + j), kk);
        bw[j] = frag<true>(dWr, LDD, 16 * (wave * CPW + j), kk);
      }
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const Frag<T> at = frag<true>(Twb, LDL, 16 * rt, kk);
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
          mma(acc[rt][j], at, bu[j]);
          mma(dKp[rt][j], at, bw[j]);
        }
      }
    }
    T* dv = reinterpret_cast<T*>(a.dv);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int col = 16 * (wave * CPW + j) + lr;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          if (r < n) dv[(row0 + r) * D + col] = to<T>(acc[rt][j][ii]);
        }
    }
  }
  __syncthreads();   // dT complete; dP no longer needed (its slot takes Z)

  // ---- Z = dT T^T (lower tiles)
  for (int t = wave; t < NTRI; t += kWaves) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < LC; kk += 32) mma(acc, frag<false>(dTb, LDL, 16 * i, kk), frag<false>(Tb, LDL, 16 * j, kk));
    const int s = 16 * j + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) Zb[(16 * i + 4 * lg + ii) * LDL + s] = to<T>(acc[ii]);
  }
  __syncthreads();
  // ---- dA = -T^T Z (strictly lower), dB = diag(w) dA; dw term sum_s B_rs dA_rs
  {
    constexpr int MAXT = (NTRI + kWaves - 1) / kWaves;
    f32x4 dA[MAXT];
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int t = wave + kWaves * u;
      dA[u] = zero4();
      if (t < NTRI) {
        int i, j;
        tri_index(t, i, j);
#pragma unroll
        for (int kk = 0; kk < LC; kk += 32) mma(dA[u], frag<true>(Tb, LDL, 16 * i, kk), frag<true>(Zb, LDL, 16 * j, kk));
        f32x4 bacc = zero4();
#pragma unroll
        for (int kk = 0; kk < D; kk += 32) mma(bacc, frag<false>(Kp, LDD, 16 * i, kk), frag<false>(Km, LDD, 16 * j, kk));
        const int s = 16 * j + lr;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * i + 4 * lg + ii;
          const float da = (s < r) ? -dA[u][ii] : 0.f;
          dA[u][ii] = da;
          float rs = bacc[ii] * da;
          rs += __shfl_xor(rs, 1);
          rs += __shfl_xor(rs, 2);
          rs += __shfl_xor(rs, 4);
          rs += __shfl_xor(rs, 8);
          if (lr == 0) dwq[j * LC + r] = rs;
        }
      }
    }
    __syncthreads();   // every read of Z is done
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int t = wave + kWaves * u;
      if (t < NTRI) {
        int i, j;
        tri_index(t, i, j);
        const int s = 16 * j + lr;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * i + 4 * lg + ii;
          dAb[r * LDL + s] = to<T>(wL[r] * dA[u][ii]);
        }
      }
    }
    for (int idx = tid; idx < LC * LC; idx += kThreads) {
      const int r = idx / LC, s = idx % LC;
      const int it = r >> 4, jt = s >> 4;
      if (jt > it) {
        dAb[r * LDL + s] = to<T>(0.f);
        dwq[jt * LC + r] = 0.f;
      }
    }
  }
  __syncthreads();

  // ---- dK+ += dB K-, dK- += dB^T K+; combine everything per element
#pragma unroll
  for (int kk = 0; kk < LC; kk += 32) {
    Frag<T> bm[CPW], bp[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      bm[j] = frag<true>(Km, LDD, 16 * (wave * CPW + j), kk);
      bp[j] = frag<true>(Kp, LDD, 16 * (wave * CPW + j), kk);
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const Frag<T> ab = frag<false>(dAb, LDL, 16 * rt, kk);
      const Frag<T> abt = frag<true>(dAb, LDL, 16 * rt, kk);
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        mma(dKp[rt][j], ab, bm[j]);
        mma(dKm[rt][j], abt, bp[j]);
      }
    }
  }
  // G_L term of each column: sum_s K->_s dK->_s + Gamma_L sum_v S[v][k] dS'[v][k]
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int col = 16 * (wave * CPW + j) + lr;
    float sd = 0.f;
    for (int vv = lg; vv < D; vv += 4) sd += S[(size_t)vv * D + col] * dS[(size_t)vv * D + col];
    float tot = gsum[j] + gLc[j] * sd;
    tot += __shfl_xor(tot, 16);
    tot += __shfl_xor(tot, 32);
    if (lg == 0) glt[col] = tot;
  }
  {
    T* dk = reinterpret_cast<T*>(a.dk);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int col = 16 * (wave * CPW + j) + lr;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          const float g = gam[rt][j][ii];
          const float e1 = g * dKp[rt][j][ii];
          const float e2 = dKm[rt][j][ii] / g;
          const float kv = (r < n) ? tof(k[(row0 + min(r, n - 1)) * D + col]) : 0.f;
          const float dkv = dKacc[rt][j][ii] + e1 + e2;
          dGacc[rt][j][ii] += kv * (e1 - e2);
          if (r < n) dk[(row0 + r) * D + col] = to<T>(dkv);
        }
    }
  }
  __syncthreads();   // glt, dwp, dwq complete

  // ---- dlog a = reverse cumulative sum of dG over the chunk's tokens + G_L term
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int col = 16 * (wave * CPW + j) + lr;
    float run = glt[col];
#pragma unroll
    for (int rt = NB - 1; rt >= 0; --rt) {
      float loc[4];
      loc[3] = dGacc[rt][j][3];
      loc[2] = loc[3] + dGacc[rt][j][2];
      loc[1] = loc[2] + dGacc[rt][j][1];
      loc[0] = loc[1] + dGacc[rt][j][0];
      float post = run, tile = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float tg = __shfl(loc[0], lr + 16 * g);
        if (g > lg) post += tg;
        tile += tg;
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * rt + 4 * lg + ii;
        if (r < n) {
          const size_t idx = (row0 + r) * D + col;
          const float dla = post + loc[ii];
          a.dlog_g[idx] = dla;
          if (HAS_B) a.db[idx] = dla / f.b[idx];
        }
      }
      run += tile;
    }
  }
  // ---- dw_r = sum_s B_rs dA_rs + sum_i T[i][r] dT'[i][r]
  if (tid < LC && tid < n) {
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < NB; ++t) s += dwq[t * LC + tid] + dwp[t * LC + tid];
    a.dw[row0 + tid] = s;
  }
}

// ------------------------------------------------------------------ launchers
template <typename T, int LC, int D, int VS>
static hipError_t rev_launch(const BwdArgs& a, hipStream_t st) {
  using Lay = RevLayout<T, LC, D, VS>;
  static_assert(Lay::bytes <= 64 * 1024, "reverse-state LDS exceeds 64 KB");
  dim3 grid(D / VS, a.fwd.B * a.fwd.H);
  hipLaunchKernelGGL((bwd_state_kernel<T, LC, D, VS>), grid, dim3(kThreads), Lay::bytes, st, a);
  return hipGetLastError();
}

template <typename T, int LC, int D>
static hipError_t rev_launch_vs(const BwdArgs& a, hipStream_t st) {
  switch (a.fwd.VS) {
    case 16: return rev_launch<T, LC, D, 16>(a, st);
    case 32: return rev_launch<T, LC, D, 32>(a, st);
    case 64: return rev_launch<T, LC, D, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int LC, int D>
static hipError_t grad_launch(const BwdArgs& a, hipStream_t st) {
  using Lay = GradLayout<T, LC, D>;
  static_assert(Lay::bytes <= 160 * 1024, "chunk-gradient LDS exceeds 160 KB");
  auto kern = a.fwd.b ? bwd_chunk_kernel<T, LC, D, true> : bwd_chunk_kernel<T, LC, D, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
  if (e != hipSuccess) return e;
  dim3 grid(a.fwd.NC, a.fwd.B * a.fwd.H);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), Lay::bytes, st, a);
  return hipGetLastError();
}

// bf16: 64- or 32-token tiles; float32: 32-token tiles only
#define CARVE_BWD_DISPATCH(FN, A, ST)                                           \
  do {                                                                          \
    const FwdArgs& f_ = (A).fwd;                                                \
    if (f_.dtype == 1) {                                                        \
      if (f_.D == 128) return f_.LC == 64 ? FN<bf16, 64, 128>(A, ST) : FN<bf16, 32, 128>(A, ST); \
      return f_.LC == 64 ? FN<bf16, 64, 64>(A, ST) : FN<bf16, 32, 64>(A, ST);   \
    }                                                                           \
    if (f_.LC != 32) return hipErrorInvalidValue;                               \
    return f_.D == 128 ? FN<float, 32, 128>(A, ST) : FN<float, 32, 64>(A, ST);  \
  } while (0)

hipError_t launch_bwd_state(const BwdArgs& a, hipStream_t st) { CARVE_BWD_DISPATCH(rev_launch_vs, a, st); }
hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t st) { CARVE_BWD_DISPATCH(grad_launch, a, st); }

}  // namespace carve
