// Forward kernels of the CARVE key-axis gated delta rule on gfx950.
//
//   fwd_prep   one workgroup per chunk (all chunks in parallel): key-axis
//              cumulative retention, coupling A, T = (I + A)^-1, the WY factors
//              W = T diag(w) K+ and Ubar = T diag(w) V, the intra-chunk output
//              P Ubar and Q~ = Q+ - P W, and K-> for the state update.
//   fwd_state  one workgroup per (batch*head, slice of value rows): carries the
//              fp32 state across chunks in registers and writes o.
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
#include "carve_device.h"
#include "carve_internal.h"

namespace carve {

// ------------------------------------------------------------------ helpers
template <typename T, int LC, int D>
struct PrepLayout {
  static constexpr int LDD = D + Pad<T>::v;      // [LC][D] row stride (elements)
  static constexpr int LDL = LC + Pad<T>::v;     // [D][LC] and [LC][LC] row stride
  static constexpr int LDF = LC + 4;             // fp32 [LC][LC] row stride
  static constexpr int P = kThreads / D;         // token parts per key channel in the gate pass
  static constexpr int RP = LC / P;              // tokens per part
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
  static constexpr size_t R6 = R5 + al(szLL);             // Ubar^T
  static constexpr size_t R7 = R6 + al(szDL);             // w [LC], part products [P][D], T-solve scratch
  static constexpr size_t bytes = R7 + al(sizeof(float) * (LC + P * D + kWaves * 16 * 20));
};

// lower-triangular block index -> (i, j), j <= i
__device__ __forceinline__ void tri_index(int t, int& i, int& j) {
  i = 0;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  j = t - i * (i + 1) / 2;
}

// T = (I + A)^-1 for strictly lower-triangular A (fp32 in LDS), LC = 16 * NB.
// Diagonal 16x16 blocks by column-parallel forward substitution, then the
// off-diagonal blocks by block forward substitution on fp32 MFMA:
//   T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj,   processed by increasing i - j.
template <int LC, int LDF>
__device__ void triangular_inverse(const float* Af, float* Tf, float* scratch) {
  constexpr int NB = LC / 16;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  if (tid < 16 * NB) {
    const int base = 16 * (tid / 16), j = tid % 16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s -= Af[(base + r) * LDF + base + m] * x[m];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tf[(base + r) * LDF + base + j] = x[r];
  }
  for (int idx = tid; idx < LC * LC; idx += kThreads) {
    const int r = idx / LC, s = idx % LC;
    if ((s >> 4) > (r >> 4)) Tf[r * LDF + s] = 0.f;
  }
  __syncthreads();
  for (int d = 1; d < NB; ++d) {
    if (wave < NB - d) {
      const int j = wave, i = wave + d;
      const int lr = lane & 15, lg = lane >> 4;
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      for (int m = j; m < i; ++m) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const float a = Af[(16 * i + lr) * LDF + 16 * m + 4 * s4 + lg];
          const float b = Tf[(16 * m + 4 * s4 + lg) * LDF + 16 * j + lr];
          mma_k4(y, a, b);
        }
      }
      float* Y = scratch + wave * 16 * 20;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Y[(4 * lg + ii) * 20 + lr] = y[ii];
      wave_lds_sync();
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float a = Tf[(16 * i + lr) * LDF + 16 * i + 4 * s4 + lg];
        const float b = Y[(4 * s4 + lg) * 20 + lr];
        mma_k4(x, a, b);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Tf[(16 * i + 4 * lg + ii) * LDF + 16 * j + lr] = -x[ii];
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ gate sources
// Erase gate of one element: token-only (b given or 1) or content-aware
// b = sigmoid(b_x + z) with the chunk's content signal z (per key channel, in LDS).
struct TokenGates {
  const float* b;
  __device__ __forceinline__ float operator()(size_t idx, int) const { return b ? b[idx] : 1.f; }
};
struct ContentGates {
  const float* b_x;
  const float* z;
  __device__ __forceinline__ float operator()(size_t idx, int ch) const {
    return 1.f / (1.f + __expf(-(b_x[idx] + z[ch])));
  }
};

// ------------------------------------------------------------------ per-chunk prep
// Computes the factors of chunk c of head bh and writes them to slot `ci` of
// the factor arrays.  Uses PrepLayout<T, LC, D>::bytes of LDS at `smem`.
template <typename T, int LC, int D, typename Gates>
__device__ void prep_chunk(const FwdArgs& a, const Gates& gates, int bh, int c, size_t ci,
                           unsigned char* smem) {
  using Lay = PrepLayout<T, LC, D>;
  constexpr int NB = LC / 16, NCT = D / 16;
  constexpr int LDD = Lay::LDD, LDL = Lay::LDL, LDF = Lay::LDF, P = Lay::P, RP = Lay::RP;
  T* Kp = reinterpret_cast<T*>(smem + Lay::R1);
  T* Km = Kp + LC * LDD;
  float* Tf = reinterpret_cast<float*>(smem + Lay::R1);
  T* Tb = reinterpret_cast<T*>(smem + Lay::R1 + Lay::szLLf);
  T* Qp = reinterpret_cast<T*>(smem + Lay::R2);
  T* KwT = reinterpret_cast<T*>(smem + Lay::R3);
  T* VwT = KwT + D * LDL;
  float* Af = reinterpret_cast<float*>(smem + Lay::R4);
  T* WnT = reinterpret_cast<T*>(smem + Lay::R4);
  T* Pb = reinterpret_cast<T*>(smem + Lay::R5);
  T* UbTs = reinterpret_cast<T*>(smem + Lay::R6);
  float* wL = reinterpret_cast<float*>(smem + Lay::R7);
  float* part = wL + LC;
  float* scratch = part + P * D;

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int t0 = c * LC;
  const int n = min(LC, a.T - t0);
  const size_t row0 = (size_t)bh * a.T + t0;   // global token row of the chunk's first token
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  T* gWn = reinterpret_cast<T*>(a.f.Wn) + ci * LC * D;
  T* gQt = reinterpret_cast<T*>(a.f.Qt) + ci * LC * D;
  T* gKfT = reinterpret_cast<T*>(a.f.KfT) + ci * D * LC;
  T* gUbT = reinterpret_cast<T*>(a.f.UbT) + ci * D * LC;
  T* gOiT = reinterpret_cast<T*>(a.f.OiT) + ci * D * LC;

  // ---- gate pass: cumulative key-axis retention Gamma (thread = key channel x token part)
  const int ch = tid % D, pid = tid / D, r0 = pid * RP;
  if (tid < LC) wL[tid] = (tid < n) ? a.w[row0 + tid] : 0.f;
  float G[RP];
  {
    float run = 1.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const int r = r0 + i;
      float av = 1.f;
      if (r < n) {
        const size_t idx = (row0 + r) * D + ch;
        av = __expf(a.log_g[idx]) * gates(idx, ch);
      }
      run *= av;
      G[i] = run;
    }
    part[pid * D + ch] = run;
  }
  __syncthreads();
  float pre = 1.f, tot = 1.f;
#pragma unroll
  for (int pp = 0; pp < P; ++pp) {
    const float pt = part[pp * D + ch];
    if (pp < pid) pre *= pt;
    tot *= pt;
  }
  {
    T kf[RP];
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const int r = r0 + i;
      const float gam = pre * G[i];
      const float inv = 1.f / gam;
      float kv = 0.f, qv = 0.f, vv = 0.f;
      if (r < n) {
        const size_t idx = (row0 + r) * D + ch;
        kv = tof(k[idx]);
        qv = tof(q[idx]);
        vv = tof(v[idx]);
      }
      const float wr = wL[r];
      Kp[r * LDD + ch] = to<T>(kv * gam);
      Km[r * LDD + ch] = to<T>(kv * inv);
      Qp[r * LDD + ch] = to<T>(qv * gam);
      KwT[ch * LDL + r] = to<T>(wr * (kv * gam));
      VwT[ch * LDL + r] = to<T>(wr * vv);
      kf[i] = to<T>(kv * (tot * inv));
    }
#pragma unroll
    for (int i = 0; i < RP; ++i) gKfT[ch * LC + r0 + i] = kf[i];
    if (pid == 0) a.f.gL[ci * D + ch] = tot;
  }
  __syncthreads();

  // ---- coupling A = strict_tril(diag(w) K+ K-^T) (fp32) and P = tril(Q+ K-^T)
  constexpr int NTRI = NB * (NB + 1) / 2;
  for (int t = wave; t < 2 * NTRI; t += kWaves) {
    const bool isA = t < NTRI;
    int i, j;
    tri_index(isA ? t : t - NTRI, i, j);
    const T* Ar = isA ? Kp : Qp;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) {
      const Frag<T> fa = load_frag(Ar + (16 * i + lr) * LDD + kk + 8 * lg);
      const Frag<T> fb = load_frag(Km + (16 * j + lr) * LDD + kk + 8 * lg);
      mma(acc, fa, fb);
    }
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
    if ((s >> 4) > (r >> 4)) Pb[r * LDL + s] = to<T>(0.f);
  }
  __syncthreads();

  // ---- T = (I + A)^-1 (fp32), then a dtype copy for the WY products
  triangular_inverse<LC, LDF>(Af, Tf, scratch);
  for (int idx = tid; idx < LC * LC; idx += kThreads) {
    const int r = idx / LC, s = idx % LC;
    Tb[r * LDL + s] = to<T>(Tf[r * LDF + s]);
  }
  __syncthreads();

  // ---- WY factors: W = T Kw, Ubar = T Vw  (Kw = diag(w) K+, Vw = diag(w) V)
  for (int t = wave; t < 2 * NB * NCT; t += kWaves) {
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
      const f32x4 neg = -acc;
      store4(WnT + col * LDL + r, neg);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) gWn[(r + ii) * D + col] = to<T>(neg[ii]);
    } else {
      store4(UbTs + col * LDL + r, acc);
      store4(gUbT + col * LC + r, acc);
    }
  }
  __syncthreads();

  // ---- intra-chunk output P Ubar and Q~ = Q+ - P W
  for (int t = wave; t < 2 * NB * NCT; t += kWaves) {
    const bool isO = t < NB * NCT;
    const int tt = isO ? t : t - NB * NCT;
    const int i = tt / NCT, ct = tt % NCT;
    const int col = 16 * ct + lr, r = 16 * i + 4 * lg;
    f32x4 acc;
    if (isO) {
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) acc[ii] = tof(Qp[(r + ii) * LDD + col]);
    }
    const T* Bs = isO ? UbTs : WnT;
    for (int kk = 0; kk < 16 * (i + 1); kk += 32) {
      const Frag<T> fa = load_frag(Pb + (16 * i + lr) * LDL + kk + 8 * lg);
      const Frag<T> fb = load_frag(Bs + (16 * ct + lr) * LDL + kk + 8 * lg);
      mma(acc, fa, fb);
    }
    if (isO) {
      store4(gOiT + col * LC + r, acc);
    } else {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) gQt[(r + ii) * D + col] = to<T>(acc[ii]);
    }
  }
}

template <typename T, int LC, int D>
__global__ __launch_bounds__(kThreads) void fwd_prep_kernel(FwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int c = blockIdx.x, bh = blockIdx.y;
  prep_chunk<T, LC, D>(a, TokenGates{a.b}, bh, c, (size_t)bh * a.NC + c, smem);
}

// ------------------------------------------------------------------ state step
// Workgroup = (slice of VS value rows, batch*head).  The state slice lives in
// MFMA accumulators as S^T tiles: lane l of tile (ct, vt) holds
// S[16 vt + l%16][16 ct + 4 (l/16) + i], i = 0..3.  A dtype copy of the slice
// in LDS (row-major [v][key]) is the B operand of W S^T and Q~ S^T.
template <typename T, int LC, int D, int VS>
struct StateLayout {
  static constexpr int LDS_ = D + Pad<T>::v;
  static constexpr int LDU = LC + Pad<T>::v;
  static constexpr int NB = LC / 16, NVT = VS / 16;
  static constexpr size_t bytes = sizeof(T) * (VS * LDS_ + VS * LDU) + sizeof(float) * NB * VS;
};

template <int D, int VS>
struct StateTiles {
  static constexpr int NVT = VS / 16, NCT = D / 16;
  static constexpr int SPW = NCT * NVT / kWaves;   // state tiles per wave
  static_assert(NCT * NVT % kWaves == 0, "state tiles must split evenly over waves");
};

// Load the state slice (S0 or zero) into registers and its dtype copy into LDS.
template <typename T, int D, int VS>
__device__ void state_init(const FwdArgs& a, int bh, int v0, f32x4 (&S)[StateTiles<D, VS>::SPW], T* Sb) {
  using ST = StateTiles<D, VS>;
  constexpr int LDS_ = D + Pad<T>::v;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int j = 0; j < ST::SPW; ++j) {
    const int st = wave * ST::SPW + j, ct = st / ST::NVT, vt = st % ST::NVT;
    const int vl = 16 * vt + lr, kc = 16 * ct + 4 * lg;
    if (a.S0) S[j] = load4f(a.S0 + ((size_t)bh * D + v0 + vl) * D + kc);
    else S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    store4(Sb + vl * LDS_ + kc, S[j]);
  }
}

// One chunk of the state recurrence for a slice of VS value rows:
//   U = Ubar + (-W) S^T,  O = (P Ubar) + Q~ S^T  (o written when a.o is set),
//   S^T <- Diag(Gamma_L) S^T + K->^T U.
// Factors are read from slot ci.  On entry Sb holds the dtype copy of S; on exit
// S and Sb hold the updated state.  If colsum is given, the per-row-tile column
// sums of the fp32 outputs (valid tokens only) are written to colsum[NB][VS].
template <typename T, int LC, int D, int VS>
__device__ void state_chunk(const FwdArgs& a, int bh, int c, size_t ci, int v0,
                            f32x4 (&S)[StateTiles<D, VS>::SPW], unsigned char* smem, float* colsum) {
  using Lay = StateLayout<T, LC, D, VS>;
  using ST = StateTiles<D, VS>;
  constexpr int NVT = ST::NVT, NB = LC / 16, SPW = ST::SPW;
  constexpr int NUO = NB * NVT;
  constexpr int UPW = (NUO + kWaves - 1) / kWaves;
  constexpr int LDS_ = Lay::LDS_, LDU = Lay::LDU;
  T* Sb = reinterpret_cast<T*>(smem);
  T* UT = Sb + VS * LDS_;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
  const T* Wn = reinterpret_cast<const T*>(a.f.Wn);
  const T* Qt = reinterpret_cast<const T*>(a.f.Qt);
  const T* KfT = reinterpret_cast<const T*>(a.f.KfT);
  const T* UbT = reinterpret_cast<const T*>(a.f.UbT);
  const T* OiT = reinterpret_cast<const T*>(a.f.OiT);
  T* o = reinterpret_cast<T*>(a.o);

#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    const int tix = wave + kWaves * u;
    if (tix < NUO) {
      const int rt = tix / NVT, vt = tix % NVT;
      const int r = 16 * rt + 4 * lg, vl = 16 * vt + lr, vg = v0 + vl;
      f32x4 accU = load4f(UbT + (ci * D + vg) * LC + r);
      f32x4 accO = {0.f, 0.f, 0.f, 0.f};
      if (a.o) accO = load4f(OiT + (ci * D + vg) * LC + r);
#pragma unroll
      for (int kk = 0; kk < D; kk += 32) {
        const Frag<T> fs = load_frag(Sb + vl * LDS_ + kk + 8 * lg);
        const Frag<T> fw = load_frag(Wn + (ci * LC + 16 * rt + lr) * D + kk + 8 * lg);
        mma(accU, fw, fs);
        if (a.o) {
          const Frag<T> fq = load_frag(Qt + (ci * LC + 16 * rt + lr) * D + kk + 8 * lg);
          mma(accO, fq, fs);
        }
      }
      if (a.o) {
        float csum = 0.f;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int t = c * LC + r + ii;
          if (t < a.T) {
            o[((size_t)bh * a.T + t) * D + vg] = to<T>(accO[ii]);
            csum += accO[ii];
          }
        }
        if (colsum) {
          csum += __shfl_xor(csum, 16);
          csum += __shfl_xor(csum, 32);
          if (lg == 0) colsum[rt * VS + vl] = csum;
        }
      }
      store4(UT + vl * LDU + r, accU);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int st = wave * SPW + j, ct = st / NVT, vt = st % NVT;
    const int kc = 16 * ct + 4 * lg, vl = 16 * vt + lr;
    const f32x4 gl = load4f(a.f.gL + ci * D + kc);
    S[j] *= gl;
#pragma unroll
    for (int kk = 0; kk < LC; kk += 32) {
      const Frag<T> fk = load_frag(KfT + (ci * D + 16 * ct + lr) * LC + kk + 8 * lg);
      const Frag<T> fu = load_frag(UT + vl * LDU + kk + 8 * lg);
      mma(S[j], fk, fu);
    }
    store4(Sb + vl * LDS_ + kc, S[j]);
  }
  __syncthreads();
}

template <typename T, int D, int VS>
__device__ void state_store(const FwdArgs& a, int bh, int v0, const f32x4 (&S)[StateTiles<D, VS>::SPW], float* dst) {
  using ST = StateTiles<D, VS>;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int j = 0; j < ST::SPW; ++j) {
    const int st = wave * ST::SPW + j, ct = st / ST::NVT, vt = st % ST::NVT;
    store4(dst + ((size_t)bh * D + v0 + 16 * vt + lr) * D + 16 * ct + 4 * lg, S[j]);
  }
}

template <typename T, int LC, int D, int VS>
__global__ __launch_bounds__(kThreads) void fwd_state_kernel(FwdArgs a) {
  using ST = StateTiles<D, VS>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int slice = blockIdx.x, bh = blockIdx.y;
  const int v0 = slice * VS;
  f32x4 S[ST::SPW];
  state_init<T, D, VS>(a, bh, v0, S, reinterpret_cast<T*>(smem));
  __syncthreads();
  for (int c = 0; c < a.NC; ++c) {
    const size_t ci = (size_t)bh * a.NC + c;
    if (a.S_chunk) state_store<T, D, VS>(a, (int)ci, v0, S, a.S_chunk);
    state_chunk<T, LC, D, VS>(a, bh, c, ci, v0, S, smem, nullptr);
  }
  if (a.S_T) state_store<T, D, VS>(a, bh, v0, S, a.S_T);
}

// ------------------------------------------------------------------ content-aware forward
// One workgroup per (batch*head) runs every chunk in order, because the erase
// gate of chunk c depends on the outputs of chunk c-1 (notes section 2.2): at
// the start of each content period (L tokens) the signal z = U2 (U1 m) of the
// previous period's mean output m is formed, the chunk's factors are prepared
// with b = sigmoid(b_x + z) into this head's factor slot (one chunk, L2
// resident), and the state step consumes them with all Dv rows in the
// workgroup.  The mean is accumulated from the fp32 outputs before rounding,
// in a fixed order (deterministic).
template <typename T, int LC, int D>
struct ContentLayout {
  static constexpr size_t prep = PrepLayout<T, LC, D>::bytes;
  static constexpr size_t step = StateLayout<T, LC, D, D>::bytes;
  static constexpr size_t body = (prep > step ? prep : step);
  static constexpr size_t bytes = body + sizeof(float) * (4 * D + 64);   // z, msum, m, r
};

template <typename T, int LC, int D>
__global__ __launch_bounds__(kThreads) void fwd_content_kernel(FwdArgs a, ContentArgs cg) {
  using Lay = ContentLayout<T, LC, D>;
  using ST = StateTiles<D, D>;
  constexpr int NB = LC / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  float* zL = reinterpret_cast<float*>(smem + Lay::body);
  float* msum = zL + D;
  float* mL = msum + D;
  float* rL = mL + D;           // [64] low-rank intermediate U1 m
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int h = bh % a.H;
  const int per = cg.period / LC;   // chunks per content period

  if (tid < D) {
    mL[tid] = cg.m0 ? cg.m0[(size_t)bh * D + tid] : 0.f;
    msum[tid] = 0.f;
  }
  f32x4 S[ST::SPW];
  __syncthreads();
  int count = 0;
  for (int c = 0; c < a.NC; ++c) {
    if (c % per == 0) {
      // content signal of this period from the previous period's mean output
      if (cg.U1) {
        if (tid < cg.R) {
          const float* u1 = cg.U1 + ((size_t)h * cg.R + tid) * D;
          float acc = 0.f;
          for (int vv = 0; vv < D; ++vv) acc += u1[vv] * mL[vv];
          rL[tid] = acc;
        }
        __syncthreads();
        if (tid < D) {
          const float* u2 = cg.U2 + ((size_t)h * D + tid) * cg.R;
          float acc = 0.f;
          for (int j = 0; j < cg.R; ++j) acc += u2[j] * rL[j];
          zL[tid] = acc;
        }
      } else if (tid < D) {
        zL[tid] = 0.f;
      }
      if (tid < D) msum[tid] = 0.f;
      count = 0;
      __syncthreads();
    }
    // prepare this chunk's factors into the head's slot
    prep_chunk<T, LC, D>(a, ContentGates{cg.b_x, zL}, bh, c, (size_t)bh, smem);
    __syncthreads();
    if (c == 0) {
      state_init<T, D, D>(a, bh, 0, S, reinterpret_cast<T*>(smem));
      __syncthreads();
    } else {
      // rebuild the LDS copy of the state (the prep pass reused that memory)
      constexpr int LDS_ = D + Pad<T>::v;
      const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
      T* Sb = reinterpret_cast<T*>(smem);
#pragma unroll
      for (int j = 0; j < ST::SPW; ++j) {
        const int st = wave * ST::SPW + j, ct = st / ST::NVT, vt = st % ST::NVT;
        store4(Sb + (16 * vt + lr) * LDS_ + 16 * ct + 4 * lg, S[j]);
      }
      __syncthreads();
    }
    float* cs = reinterpret_cast<float*>(smem + StateLayout<T, LC, D, D>::bytes - sizeof(float) * NB * D);
    state_chunk<T, LC, D, D>(a, bh, c, (size_t)bh, 0, S, smem, cs);
    // fold this chunk's column sums into the period sum (fixed order over row tiles)
    const int nvalid = min(LC, a.T - c * LC);
    if (tid < D) {
      float sacc = msum[tid];
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) sacc += cs[rt * D + tid];
      msum[tid] = sacc;
    }
    count += nvalid;
    if ((c + 1) % per == 0 || c == a.NC - 1) {
      if (tid < D) mL[tid] = msum[tid] / (float)count;
    }
    __syncthreads();
  }
  if (a.S_T) state_store<T, D, D>(a, bh, 0, S, a.S_T);
  if (cg.m_out && tid < D) cg.m_out[(size_t)bh * D + tid] = mL[tid];
}

// ------------------------------------------------------------------ small helpers
// dst[i] = src ? src[i] : 0 (used for empty inputs: S_T = S0, m_out = m0).
__global__ void copy_or_zero_kernel(float* dst, const float* src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers
size_t factors_bytes(int dtype, int BH, int NC, int LC, int D) {
  const size_t es = dtype ? 2 : 4;
  const size_t nchunk = (size_t)BH * NC;
  return nchunk * (5 * (size_t)LC * D * es + (size_t)D * 4) + 5 * 256;
}

ChunkFactors carve_factors(void* ws, int dtype, int BH, int NC, int LC, int D) {
  const size_t es = dtype ? 2 : 4;
  const size_t nchunk = (size_t)BH * NC;
  const size_t blk = (nchunk * LC * D * es + 255) & ~size_t(255);
  char* p = static_cast<char*>(ws);
  ChunkFactors f;
  f.Wn = p;
  f.Qt = p + blk;
  f.KfT = p + 2 * blk;
  f.UbT = p + 3 * blk;
  f.OiT = p + 4 * blk;
  f.gL = reinterpret_cast<float*>(p + 5 * blk);
  return f;
}

template <typename T, int LC, int D>
static hipError_t prep_launch(const FwdArgs& a, hipStream_t st) {
  using Lay = PrepLayout<T, LC, D>;
  static_assert(Lay::bytes <= 160 * 1024, "prep LDS exceeds 160 KB");
  auto kern = fwd_prep_kernel<T, LC, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
  if (e != hipSuccess) return e;
  dim3 grid(a.NC, a.B * a.H);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), Lay::bytes, st, a);
  return hipGetLastError();
}

template <typename T, int LC, int D, int VS>
static hipError_t state_launch(const FwdArgs& a, hipStream_t st) {
  using Lay = StateLayout<T, LC, D, VS>;
  static_assert(Lay::bytes <= 64 * 1024, "state LDS exceeds 64 KB");
  auto kern = fwd_state_kernel<T, LC, D, VS>;
  dim3 grid(D / VS, a.B * a.H);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), Lay::bytes, st, a);
  return hipGetLastError();
}

template <typename T, int LC, int D>
static hipError_t state_launch_vs(const FwdArgs& a, hipStream_t st) {
  switch (a.VS) {
    case 16: return state_launch<T, LC, D, 16>(a, st);
    case 32: return state_launch<T, LC, D, 32>(a, st);
    case 64: return state_launch<T, LC, D, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// Instantiated (dtype, token tile, width) combinations.  fp32 at width 128 only
// uses the 32-token tile (the 64-token tile would not fit in 160 KB of LDS).
#define CARVE_DISPATCH(FN, A, ST)                                              \
  do {                                                                         \
    if ((A).dtype == 1) {                                                      \
      if ((A).D == 128) return (A).LC == 64 ? FN<bf16, 64, 128>(A, ST) : FN<bf16, 32, 128>(A, ST); \
      return (A).LC == 64 ? FN<bf16, 64, 64>(A, ST) : FN<bf16, 32, 64>(A, ST); \
    }                                                                          \
    if ((A).D == 128) return (A).LC == 32 ? FN<float, 32, 128>(A, ST) : hipErrorInvalidValue; \
    return (A).LC == 64 ? FN<float, 64, 64>(A, ST) : FN<float, 32, 64>(A, ST); \
  } while (0)

template <typename T, int LC, int D>
static hipError_t content_launch(const FwdArgs& a, const ContentArgs& cg, hipStream_t st) {
  using Lay = ContentLayout<T, LC, D>;
  static_assert(Lay::bytes <= 160 * 1024, "content LDS exceeds 160 KB");
  auto kern = fwd_content_kernel<T, LC, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(kThreads), Lay::bytes, st, a, cg);
  return hipGetLastError();
}

hipError_t launch_fwd_content(const FwdArgs& a, const ContentArgs& cg, hipStream_t st) {
  if (a.dtype == 1) {
    if (a.D == 128) return a.LC == 64 ? content_launch<bf16, 64, 128>(a, cg, st) : content_launch<bf16, 32, 128>(a, cg, st);
    return a.LC == 64 ? content_launch<bf16, 64, 64>(a, cg, st) : content_launch<bf16, 32, 64>(a, cg, st);
  }
  if (a.D == 128) return a.LC == 32 ? content_launch<float, 32, 128>(a, cg, st) : hipErrorInvalidValue;
  return a.LC == 64 ? content_launch<float, 64, 64>(a, cg, st) : content_launch<float, 32, 64>(a, cg, st);
}

hipError_t launch_fwd_prep(const FwdArgs& a, hipStream_t st) { CARVE_DISPATCH(prep_launch, a, st); }
hipError_t launch_fwd_state(const FwdArgs& a, hipStream_t st) { CARVE_DISPATCH(state_launch_vs, a, st); }

}  // namespace carve
