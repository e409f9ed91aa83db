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
#include <algorithm>
#include <type_traits>

#include "carve_chunk.h"
#include "content_gate.h"

namespace carve {

// ------------------------------------------------------------------ fragments
// Fragment of rows row0..row0+15 of a logical [rows][K] matrix X at k block k0:
// TR = false: X stored row-major (X[r][k] at base[r*ld + k]);
// TR = true : X stored transposed (X[r][k] at base[k*ld + r]); base must point into
//             LDS (bf16 uses the LDS transpose read).
template <bool TR, typename T>
__device__ __forceinline__ Frag<T> frag(const T* base, int ld, int row0, int k0) {
  const int lane = lane_id(), lr = lane & 15, lg = lane >> 4;
  if constexpr (!TR) return load_frag(base + (size_t)(row0 + lr) * ld + k0 + 8 * lg);
  else return lds_frag_cols(base, ld, row0, k0);
}


// ------------------------------------------------------------------ reverse state pass
// LDS: the dtype copy of the dS^T slice [VS][D], X^T [VS][LC], the chunk's dO slice
// (row-major [LC][VS]) and the chunk's factors in their forward layouts, row-major:
// -W and Q~ [LC][D] (rows = tokens), K->^T [D][LC] (rows = keys).  The products read
// the factors and dO as transposed fragments.
template <typename T, int LC, int D, int VS>
struct RevLayout {
  static constexpr int LDS_ = D + Pad<T>::v;
  static constexpr int LDU = LC + Pad<T>::v;
  static constexpr int LDV = VS + Pad<T>::v;
  static constexpr size_t state = sizeof(T) * (VS * LDS_ + VS * LDU + LC * LDV);
  static constexpr size_t Wl = state, Ql = Wl + sizeof(T) * LC * LDS_, Kl = Ql + sizeof(T) * LC * LDS_;
  static constexpr size_t bytes = Kl + sizeof(T) * D * LDU;
};

// Global operands of one chunk (loaded two chunks ahead, chunks running last to first):
//   the chunk's -W, Q~ and K->^T blocks as they are stored (fragment order), piece
//   tid + kThreads u of each block, staged in LDS one chunk step ahead of their use
//   Gamma_L of the wave's key tiles
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
  static constexpr int NPT = LC * D / VEC / kThreads;             // pieces of each factor block per thread
  static_assert(NVT % XPW == 0, "a wave's X tiles must share one row tile");
  static_assert(NPT * kThreads * VEC == LC * D, "factor blocks must split evenly over the threads");
  static constexpr bool kAllWaves = XPW * (kWaves - 1) < NX;          // every wave owns X tiles
  static constexpr bool kFullDO = (LC * VS / VEC) % kThreads == 0;    // every thread loads NDO pieces
  Frag<T> wn[NPT], qt[NPT], kt[NPT];
  f32x4 gl[SCT];
  Frag<T> dov[NDO];   // raw 16-byte pieces of dO: VEC consecutive value columns of one token

  // with_do = false: the output term is left out (dO read as zero; the rows of the linear
  // part of a segment's reverse map)
  __device__ __forceinline__ void load(const BwdArgs& a, int bh, int c, int v0, bool with_do = true) {
    const FwdArgs& f = a.fwd;
    const int lg = lane_id() >> 4, wave = wave_id();
    const size_t ci = (size_t)bh * f.NC + c;
    const T* Wn = reinterpret_cast<const T*>(f.f.Wn) + ci * LC * D;
    const T* Qt = reinterpret_cast<const T*>(f.f.Qt) + ci * LC * D;
    const T* KfT = reinterpret_cast<const T*>(f.f.KfT) + ci * D * LC;
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int pc = threadIdx.x + kThreads * u;
      wn[u] = load_frag(Wn + VEC * pc);
      qt[u] = load_frag(Qt + VEC * pc);
      kt[u] = load_frag(KfT + VEC * pc);
    }
#pragma unroll
    for (int j = 0; j < SCT; ++j) gl[j] = load4f(f.f.gL + ci * D + 16 * (wave * SCT + j) + 4 * lg);
    const T* dO = reinterpret_cast<const T*>(a.dO);
    const int n = min(LC, f.T - c * LC);
#pragma unroll
    for (int u = 0; u < NDO; ++u) {
      const int idx = threadIdx.x + kThreads * u;            // piece index: token r, column group g
      const int r = idx / (VS / VEC), g = idx % (VS / VEC);
      if (kFullDO || idx < LC * VS / VEC) {
        const int rr = min(r, n - 1);   // rows past the sequence end meet zero columns of Q~^T
        dov[u] = with_do ? load_frag(dO + ((size_t)bh * f.T + c * LC + rr) * D + v0 + VEC * g) : zero_frag(T());
      }
    }
  }

  // The factor pieces into LDS, row-major: piece p of a block with C columns holds row
  // 16 (b / (C/32)) + l % 16, columns 32 (b % (C/32)) + 8 (l / 16) .. + 7 (b = p / 64,
  // l = p % 64; the fragment order of the prep pass).
  __device__ __forceinline__ void stage(T* Wl, T* Ql, T* Kl) const {
    constexpr int LDS_ = D + Pad<T>::v, LDU = LC + Pad<T>::v;
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int pc = threadIdx.x + kThreads * u, l = pc % 64, b = pc / 64;
      const int rowd = 16 * (b / (D / 32)) + l % 16, cold = 32 * (b % (D / 32)) + 8 * (l / 16);
      const int rowl = 16 * (b / (LC / 32)) + l % 16, coll = 32 * (b % (LC / 32)) + 8 * (l / 16);
      *reinterpret_cast<Frag<T>*>(Wl + rowd * LDS_ + cold) = wn[u];
      *reinterpret_cast<Frag<T>*>(Ql + rowd * LDS_ + cold) = qt[u];
      *reinterpret_cast<Frag<T>*>(Kl + rowl * LDU + coll) = kt[u];
    }
  }
};

// Reverse state pass.  A slice of VS rows of the state gradient is held as accumulator
// tiles of dS^T (lane of tile (ct, vt) holds dS[v0 + 16 vt + lr][16 ct + 4 lg + i]) and
// stepped over chunks chi down to clo:
//   dS^T <- Diag(Gamma_L) dS^T + (-W)^T (K-> dS^T) + Q~^T dO.
// AFF = false: workgroup = (slice of VS value rows, batch*head[, segment]).  Unsegmented:
// chunks c_lo .. (all by default) from dS_T, ending in dS0.  Segmented (fwd.nseg > 1):
// segment s runs its chunks from dS_seg[s], the gradient w.r.t. the state leaving it, and
// the first segment ends in dS0.  The gradient w.r.t. the state leaving every chunk goes
// to dS_vk (fragment order).
// AFF = true: the segments' reverse maps (see the segmented reverse pass below):
// workgroup = (VS rows of [C; Pi], batch*head, segment s >= 1); C rows start from zero
// with the output term, Pi rows from the identity rows without it; nothing is stored
// per chunk, and the rows end in raff.
template <typename T, int LC, int D, int VS, bool AFF>
__global__ __launch_bounds__(kThreads) void bwd_state_kernel(BwdArgs a) {
  using Lay = RevLayout<T, LC, D, VS>;
  using Op = RevOps<T, LC, D, VS>;
  using ST = StateTiles<D, VS>;
  constexpr int NVT = ST::NVT, SPW = ST::SPW, LDS_ = Lay::LDS_, LDU = Lay::LDU, LDV = Lay::LDV;
  constexpr int VEC = Op::VEC;
  extern __shared__ __align__(16) unsigned char smem[];
  T* dSb = reinterpret_cast<T*>(smem);
  T* XT = dSb + VS * LDS_;
  T* dOr = XT + VS * LDU;
  T* Wl = reinterpret_cast<T*>(smem + Lay::Wl);
  T* Ql = reinterpret_cast<T*>(smem + Lay::Ql);
  T* Kl = reinterpret_cast<T*>(smem + Lay::Kl);
  const FwdArgs& f = a.fwd;
  const int nseg = f.nseg > 1 ? f.nseg : 1;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
  int u, slice, bh, seg, v0, eye_row = -1;
  bool with_do = true;
  const float* init = nullptr;
  if constexpr (AFF) {
    const int nsa = nseg - 1;                  // segments with a reverse map: all but the first
    xcd_slice_map(2 * D / VS, f.B * f.H * nsa, u, slice);
    bh = u / nsa;
    seg = 1 + u % nsa;
    const int r0 = slice * VS;                 // first row of [C; Pi]
    v0 = r0 < D ? r0 : 0;                      // value rows of C (Pi rows read no dO)
    if (r0 >= D) {
      eye_row = r0 - D;
      with_do = false;
    }
  } else {
    xcd_slice_map(D / VS, f.B * f.H * nseg, u, slice);
    bh = u / nseg;
    seg = u % nseg;
    v0 = slice * VS;
    init = nseg > 1 ? a.dS_seg + (size_t)u * D * D : (a.dS_T ? a.dS_T + (size_t)bh * D * D : nullptr);
  }

  f32x4 dS[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int st = wave * SPW + j, ct = st / NVT, vt = st % NVT;
    const int vl = 16 * vt + lr, kc = 16 * ct + 4 * lg;
    if (AFF && eye_row >= 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[j][i] = (eye_row + vl == kc + i) ? 1.f : 0.f;
    } else if (init) {
      dS[j] = load4f(init + (size_t)(v0 + vl) * D + kc);
    } else {
      dS[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    store4(dSb + vl * LDS_ + kc, dS[j]);
  }
  // three operand buffers, loaded two chunks ahead (chunks run last to first); a
  // chunk's factors are staged in LDS during the step before its own.  Chunks below
  // the last one run in a main loop with clamped prefetch.
  constexpr int PF = 3;
  // chunk range: the segment's chunks, or (unsegmented) c_lo .. (all by default)
  const int clo = nseg > 1 ? seg * f.seg_len : a.c_lo;
  const int chi = nseg > 1 ? min(f.NC, clo + f.seg_len) - 1 : (a.c_count ? a.c_lo + a.c_count - 1 : f.NC - 1);
  const int nch = chi - clo + 1;
  Op buf[PF];
#pragma unroll
  for (int j = 0; j < PF - 1; ++j) buf[j].load(a, bh, max(chi - j, clo), v0, with_do);
  buf[0].stage(Wl, Ql, Kl);
  __syncthreads();
  auto step = [&](int c, const Op& cur, const Op& nxt) {
    const size_t ci = (size_t)bh * f.NC + c;
    if constexpr (!AFF) {
      // gradient w.r.t. the state leaving chunk c, in fragment order rows v
      T* vk = reinterpret_cast<T*>(a.dS_vk) + ci * D * D;
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int jc = j / NVT, ct = wave * Op::SCT + jc, vt = j % NVT;
        store_vk_group<T, D>(vk, v0 / 16 + vt, ct, dS[j]);
      }
    }
    // dO slice into LDS as whole pieces (no per-element work on the loaded data, so none
    // of it can be scheduled ahead of the step that owns the chunk).  Rows past the
    // sequence end hold the clamped copy of the last row; they only meet columns of
    // Q~^T that are exactly zero (q is zero past the end, so Q+, P and Q~ vanish there).
#pragma unroll
    for (int u2 = 0; u2 < Op::NDO; ++u2) {
      const int idx = threadIdx.x + kThreads * u2;
      if (Op::kFullDO || idx < LC * VS / VEC) {
        const int r = idx / (VS / VEC), g = idx % (VS / VEC);
        *reinterpret_cast<Frag<T>*>(dOr + r * LDV + VEC * g) = cur.dov[u2];
      }
    }
    // this chunk's factor fragments, transposed out of the staged blocks: K-> rows of
    // the wave's X row tile (contraction over keys), (-W)^T and Q~^T rows of its key
    // tiles (contraction over tokens); all are read before the barrier below, after
    // which the next chunk's factors take the staging slots
    Frag<T> kf[Op::KD], wt[Op::SCT][Op::KL], qt[Op::SCT][Op::KL];
    const int t0 = wave * Op::XPW, rt = t0 / NVT;
    if (Op::kAllWaves || t0 < Op::NX) {
#pragma unroll
      for (int kk = 0; kk < Op::KD; ++kk) kf[kk] = lds_frag_cols(Kl, LDU, 16 * rt, 32 * kk);
    }
#pragma unroll
    for (int jc = 0; jc < Op::SCT; ++jc)
#pragma unroll
      for (int kk = 0; kk < Op::KL; ++kk) {
        wt[jc][kk] = lds_frag_cols(Wl, LDS_, 16 * (wave * Op::SCT + jc), 32 * kk);
        qt[jc][kk] = lds_frag_cols(Ql, LDS_, 16 * (wave * Op::SCT + jc), 32 * kk);
      }
    // X^T = K-> dS^T  (tiles [s][v])
    if (Op::kAllWaves || t0 < Op::NX) {
#pragma unroll
      for (int x = 0; x < Op::XPW; ++x) {
        const int vt = (t0 + x) % NVT;
        const int vl = 16 * vt + lr;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Op::KD; ++kk) mma(acc, kf[kk], load_frag(dSb + vl * LDS_ + 32 * kk + 8 * lg));
        store4(XT + vl * LDU + 16 * rt + 4 * lg, acc);
      }
    }
    __syncthreads();
    if (c > clo) nxt.stage(Wl, Ql, Kl);   // (the last chunk has no successor to stage)
    // dS^T <- Diag(Gamma_L) dS^T + (-W)^T X^T + Q~^T dO
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      // wave*SPW is a multiple of NVT, so the key tile index within the wave is j / NVT
      const int jc = j / NVT, ct = wave * Op::SCT + jc, vt = j % NVT;
      const int kc = 16 * ct + 4 * lg, vl = 16 * vt + lr;
      dS[j] *= cur.gl[jc];
#pragma unroll
      for (int kk = 0; kk < Op::KL; ++kk) {
        mma(dS[j], wt[jc][kk], load_frag(XT + vl * LDU + 32 * kk + 8 * lg));
        mma(dS[j], qt[jc][kk], lds_frag_cols(dOr, LDV, 16 * vt, 32 * kk));
      }
      store4(dSb + vl * LDS_ + kc, dS[j]);
    }
    __syncthreads();
  };
  const int nmain = nch - (nch % PF);       // chunks chi .. chi-nmain+1 in groups of PF
  for (int g = 0; g < nmain; g += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int c = chi - (g + j);
      buf[(j + PF - 1) % PF].load(a, bh, max(c - (PF - 1), clo), v0, with_do);
      step(c, buf[j], buf[(j + 1) % PF]);
    }
  }
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int c = chi - (nmain + j);
    if (c >= clo) {
      if (c - (PF - 1) >= clo) buf[(j + PF - 1) % PF].load(a, bh, c - (PF - 1), v0, with_do);
      step(c, buf[j], buf[(j + 1) % PF]);
    }
  }
  // AFF: the rows of [C; Pi]; otherwise dS0 from the first segment
  float* dst = AFF ? a.raff + (size_t)(bh * f.nseg + seg) * 2 * D * D + (size_t)(slice * VS) * D
                   : (a.dS0 && seg == 0 ? a.dS0 + ((size_t)bh * D + v0) * D : nullptr);
  if (dst) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int st = wave * SPW + j, ct = st / NVT, vt = st % NVT;
      store4(dst + (size_t)(16 * vt + lr) * D + 16 * ct + 4 * lg, dS[j]);
    }
  }
}

// ------------------------------------------------------------------ segmented reverse pass
// The reverse step is affine in dS, so a segment maps the gradient w.r.t. the state
// leaving it to the gradient w.r.t. the state entering it as dS_in = dS_out Pi + C: C is
// the segment's reverse pass from dS_out = 0, and Pi, the product of the transposed
// chunk maps, is the pass with no output term started from the identity (its rows are
// indexed by key).  bwd_state_kernel<AFF = true> computes [C; Pi] as 2D rows per (head,
// segment) for every segment but the first; the reverse scan of seg_scan chains them from
// dS_T down (dS_out(s - 1) = dS_out(s) Pi_s + C_s); then every segment runs its reverse
// pass from its dS_out, storing the chunk-level gradients.  The reverse side of the
// chunk-level scan of affine state maps behind the logarithmic parallel depth the notes
// list for CARVE (complexity table), taken as two levels like the forward.

// ------------------------------------------------------------------ chunk gradients
// LDS slots (reused as the computation proceeds; "row-major" = [token][width]):
//   s0 K^+           s1 K^-           s2 Q^+ -> dW       s3 V (raw)
//   s4 -W -> dO      s5 U             s6 dU
//   (s4..s5 first stage the fp32 log-retention la of the chunk, then the block-local G)
//   p0 P -> dT       p1 T (dtype)     p2 Tw = T diag(w) -> e^(G_L - Gb[J+1]) -> e^Gb
//   p3 block log-retention table -> dP -> Z -> dA
// T = (I + A)^-1, P and the coupling B come from the prep pass.  The gate algebra is
// the prep pass's (carve_chunk.h): G is the cumulative log-retention inside the chunk,
// Gb[I] its value at the start of 16-token block I, btot_I the block's log-retention,
// loc = G - Gb[I] <= 0, and the operands
//   K^+ = k e^loc, Q^+ = q e^loc, K^- = k e^(btot - loc)
// (row operands referred to their block start, column operands to their block end).
// A ratio-weighted product over the tokens s of blocks J <= I, such as
//   X_r = sum_s dB_rs k_s Gamma_r/Gamma_s = e^loc_r sum_J D_IJ (dB_IJ K^-_J)_r,
// runs one 16-token block J at a time, with the per-key-channel factor
// D_IJ = e^(Gb[I] - Gb[J+1]) (1 for J = I - 1, <= 1 for J < I - 1, e^-btot_I on the
// diagonal) applied to the fp32 result: every operand is rounded once.  A diagonal block
// whose log-retention falls below -kSafeLog in some channel leaves out its 16-deep
// product; the kernel stores that block's diagonal tiles of dP and dB, and the fix-up
// pass (bwd_diag_fix_kernel) adds the exact elementwise terms.
// Tiles of [token][key] and [token][value] results are owned by column: wave w
// computes every token tile of key/value tiles ct = w*CPW .. w*CPW+CPW-1, so the
// block-local log-retention of those columns stays in that wave's registers
// (accumulator layout) for the elementwise tail and the reverse cumulative sum.
template <typename T, int LC, int D>
struct GradLayout {
  static constexpr int LDD = D + Pad<T>::v;
  static constexpr int LDL = LC + Pad<T>::v;
  static constexpr int LDF = LC + 4;
  static constexpr int NB = LC / 16;
  static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t al(size_t x) { return (x + 255) & ~size_t(255); }
  static constexpr size_t S1 = al(sizeof(T) * LC * LDD);
  static constexpr size_t S2 = al(sizeof(T) * LC * LDL);
  static constexpr size_t slot(int i) { return S1 * i; }
  static constexpr size_t pslot(int i) { return 7 * S1 + S2 * i; }
  static constexpr size_t small = 7 * S1 + 4 * S2;   // w, Gamma_L, dw partials, G_L term, block flags
  static constexpr size_t bytes = small + sizeof(float) * (LC + D + 2 * NB * LC + D) + 16 * sizeof(int);
};

// Operand sources for the column-owned products below: a fragment of rows
// row0..row0+15 at k block k0 of a logical [rows][K] matrix.
template <typename T, bool TR>
struct LdsSrc {
  const T* p;
  int ld;
  __device__ __forceinline__ Frag<T> operator()(int row0, int k0) const { return frag<TR>(p, ld, row0, k0); }
};

// acc[rt][j] += A[16 rt .. ][:] * B^T[16 (ct0 + j) .. ][:]  over K (multiple of 32),
// with B fragments taken from bpre[k block][j] (already in registers).
template <typename T, int NB, int CPW, int KB, typename ASrc>
__device__ __forceinline__ void owned_mma(f32x4 (&acc)[NB][CPW], const ASrc& A, const Frag<T> (&bpre)[KB][CPW]) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const Frag<T> af = A(16 * rt, 32 * kb);
#pragma unroll
      for (int j = 0; j < CPW; ++j) mma(acc[rt][j], af, bpre[kb][j]);
    }
  }
}
template <typename T, int NB, int CPW, int KB, typename ASrc, typename BSrc>
__device__ __forceinline__ void owned_mma(f32x4 (&acc)[NB][CPW], const ASrc& A, const BSrc& B, int ct0) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    Frag<T> bf[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) bf[j] = B(16 * (ct0 + j), 32 * kb);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const Frag<T> af = A(16 * rt, 32 * kb);
#pragma unroll
      for (int j = 0; j < CPW; ++j) mma(acc[rt][j], af, bf[j]);
    }
  }
}
// fragments of a "vk"-ordered D x D matrix M[v][k] for the wave's row tiles ct0 + j:
// rows v, contraction over k
template <typename T, int D, int CPW>
__device__ __forceinline__ void load_state_frags(Frag<T> (&dst)[D / 32][CPW], const T* base, int ct0) {
  const int lane = lane_id();
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
    for (int j = 0; j < CPW; ++j) dst[kb][j] = load_frag(base + frag_offset<D>(ct0 + j, kb, lane));
}
// the same matrix with rows k for the wave's key tiles ct0 + j (contraction over v):
// raw pieces, then the fragments
template <typename T, int D, int CPW>
__device__ __forceinline__ void load_state_kmajor(KmajorPieces<T> (&dst)[D / 32][CPW], const T* base, int ct0) {
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
    for (int j = 0; j < CPW; ++j) dst[kb][j] = load_kmajor_pieces<D>(base, ct0 + j, kb);
}
template <typename T, int KB, int CPW>
__device__ __forceinline__ void finish_kmajor(Frag<T> (&dst)[KB][CPW], const KmajorPieces<T> (&src)[KB][CPW]) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < CPW; ++j) dst[kb][j] = kmajor_frag(src[kb][j]);
}
template <int NB, int CPW>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[NB][CPW]) {
#pragma unroll
  for (int rt = 0; rt < NB; ++rt)
#pragma unroll
    for (int j = 0; j < CPW; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Block-wise column-owned products, one 16-token contraction block at a time with the
// lane's factor applied to the fp32 result (see the layout notes above):
//   LOWER: acc[I][j] += sc(I, J, j) * (A_{I,J} B_{J,col})   for J <= I   (output rows I)
//   UPPER: acc[J][j] += sc(I, J, j) * (A_{J,I} B_{I,col})   for I >= J   (output rows J)
// A16(output block, contraction block) and B16(contraction block, column tile) give
// 16-deep fragments; sc(I, J, j) is the lane's factor for its column of tile ct0 + j.
template <typename T, int NB, int CPW, bool LOWER, typename ASrc, typename BSrc, typename Sc>
__device__ __forceinline__ void owned_mma_blk(f32x4 (&acc)[NB][CPW], const ASrc& A16, const BSrc& B16, int ct0,
                                              const Sc& sc) {
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    Frag16<T> bf[CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) bf[j] = B16(kb, ct0 + j);
#pragma unroll
    for (int ob = 0; ob < NB; ++ob) {
      if (LOWER ? kb > ob : kb < ob) continue;
      const Frag16<T> af = A16(ob, kb);
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        mma16(t, af, bf[j]);
        acc[ob][j] += (LOWER ? sc(ob, kb, j) : sc(kb, ob, j)) * t;
      }
    }
  }
}

// ------------------------------------------------------------------ within-block terms
// Exact within-block terms for the 16-token blocks (bits of mask) of a range-safe chunk
// whose log-retention left the fast tiles' range (the chunk's 16-deep products left them
// out and stored the blocks' diagonal tiles of dP and dB = diag(w) dA).  For block I, key
// column ch and r, s in the block, with R_rs = prod_{t=s+1..r} a_t formed as running
// products of the retention:
//   x2_r = sum_{s<=r} dP_rs k_s R_rs,   x1_r = sum_{s<r} dB_rs k_s R_rs,
//   x3_s = sum_{r>=s} (dP_rs q_r + dB_rs k_r) R_rs,
// dq_r += x2_r and dk_r += x1_r + x3_r; the gradient w.r.t. the cumulative
// log-retention gains q_r x2_r + k_r x1_r - k_r x3_r, whose reverse cumulative sum over
// the chunk's tokens is added to dlog g (and, through the erase factor, to db).  k, q and
// the retention come from global memory with the staging's gate arithmetic; the chunk's
// own gradients are read back (same workgroup, after a barrier).  Every thread of the
// workgroup (NT) takes part in the barriers and the staging; threads 0 .. D-1 take one
// key column each.  tl: 2 x 16 x 17 + 3 x 16 x (D + 1) floats of free LDS.
template <typename T, int LC, int D, bool HAS_B, bool LG, int NT>
__device__ __forceinline__ void diag_fix_chunk(const BwdArgs& a, int bh, int c, int mask, float* tl) {
  constexpr int NB = LC / 16, LDC = D + 1;
  static_assert(NT >= D, "one thread per key column");
  const FwdArgs& f = a.fwd;
  const int ch = threadIdx.x;
  const bool col = ch < D;
  const size_t ci = (size_t)bh * f.NC + c;
  const T* kg = reinterpret_cast<const T*>(f.k);
  const T* qg = reinterpret_cast<const T*>(f.q);
  T* dq = reinterpret_cast<T*>(a.dq);
  T* dk = reinterpret_cast<T*>(a.dk);
  float* aS = tl + 2 * 16 * 17;     // [16][LDC] retention a of the block, per column
  float* kS = aS + 16 * LDC;        // [16][LDC] k
  float* qS = kS + 16 * LDC;        // [16][LDC] q
  const int n = min(LC, f.T - c * LC);
  const size_t row0 = (size_t)bh * f.T + (size_t)c * LC;
  const int chc = min(ch, D - 1);
  float gA = 0.f, gt = 0.f;
  if constexpr (LG) {
    gA = f.gA[(bh % f.H) * D + chc];
    gt = f.gtau[(bh % f.H) * D + chc];
  }
  // the erase factor of dlog g in the erase gradient at token r (as in the chunk kernels)
  auto efac = [&](size_t idx) -> float {
    if constexpr (!HAS_B) return 0.f;
    const float bvv = f.b[idx];
    return LG ? sigmoidf(-bvv) : (a.db_mode ? 1.f - bvv : __builtin_amdgcn_rcpf(bvv));
  };
  float carry = 0.f;   // sum of the corrections of the later tokens
  for (int I = NB - 1; I >= 0; --I) {
    if (mask & (1 << I)) {
      // the block's tiles, row-major [2][16][17], and a, k, q of every column
      for (int e = threadIdx.x; e < 2 * 256; e += NT) {
        const int which = e / 256, l = (e % 256) / 4, ii = e % 4;
        tl[(which * 16 + 4 * (l / 16) + ii) * 17 + l % 16] =
            tof(reinterpret_cast<const T*>(a.diag)[((ci * NB + I) * 2 + which) * 256 + e % 256]);
      }
      for (int e = threadIdx.x; e < 16 * D; e += NT) {
        const int t = e / D, cc = e % D, r = 16 * I + t;
        const bool valid = r < n;
        const size_t idx = (row0 + (size_t)min(r, n - 1)) * D + cc;
        const float lgv = f.log_g[idx];
        float la = lgv;
        if constexpr (LG) la = -f.gA[(bh % f.H) * D + cc] * softplusf(lgv + f.gtau[(bh % f.H) * D + cc]);
        if constexpr (HAS_B) la += LG ? -softplusf(-f.b[idx]) : flog(f.b[idx]);
        aS[t * LDC + cc] = valid ? fexp(clamp_la(la)) : 1.f;
        kS[t * LDC + cc] = valid ? tof(kg[idx]) : 0.f;
        qS[t * LDC + cc] = valid ? tof(qg[idx]) : 0.f;
      }
      __syncthreads();
      if (col) {
#pragma unroll 1
        for (int r = 15; r >= 0; --r) {
          // row role of row r (s <= r, running product downwards) and column role of
          // column r (rows r' >= r, running product upwards)
          float rho = 1.f, x1 = 0.f, x2 = 0.f;
#pragma unroll 1
          for (int s = r; s >= 0; --s) {
            const float ks = kS[s * LDC + ch];
            x2 += tl[r * 17 + s] * ks * rho;
            x1 += tl[(16 + r) * 17 + s] * ks * rho;
            rho *= aS[s * LDC + ch];
          }
          float x3 = 0.f;
          rho = 1.f;
#pragma unroll 1
          for (int rr = r; rr < 16; ++rr) {
            if (rr > r) rho *= aS[rr * LDC + ch];
            x3 += (tl[rr * 17 + r] * qS[rr * LDC + ch] + tl[(16 + rr) * 17 + r] * kS[rr * LDC + ch]) * rho;
          }
          const float kr = kS[r * LDC + ch];
          carry += qS[r * LDC + ch] * x2 + kr * (x1 - x3);
          const int tok = 16 * I + r;
          if (tok < n) {
            const size_t idx = row0 * D + (size_t)tok * D + ch;
            dq[idx] = to<T>(tof(dq[idx]) + x2);
            dk[idx] = to<T>(tof(dk[idx]) + x1 + x3);
            a.dlog_g[idx] += carry;
            if (HAS_B) a.db[idx] += carry * efac(idx);
          }
        }
      }
      __syncthreads();   // every read of this block's staging is done
    } else if (col && carry != 0.f) {
      for (int r = 15; r >= 0; --r) {
        const int tok = 16 * I + r;
        if (tok < n) {
          const size_t idx = row0 * D + (size_t)tok * D + ch;
          a.dlog_g[idx] += carry;
          if (HAS_B) a.db[idx] += carry * efac(idx);
        }
      }
    }
  }
  (void)gA;
  (void)gt;
}

// Fast path of the chunk gradients (chunks whose log-retention stays within the fast
// range, -kChunkSafe, in every key channel): the retention referred to the chunk start,
// Gamma = running product of a inside the chunk, K+ = K Gamma, K- = K / Gamma, Q+ = Q Gamma.
template <typename T, int LC, int D, bool HAS_B, bool LG>
__device__ __forceinline__ void bwd_chunk_fast(const BwdArgs& a, unsigned char* smem) {
  using Lay = GradLayout<T, LC, D>;
  // one wave per 16-column tile of the key/value width: NW = D/16 waves
  constexpr int NW = D / 16, NT = 64 * NW;
  constexpr int NB = LC / 16, NCT = D / 16, CPW = NCT / NW, KD = D / 32, KL = LC / 32;
  constexpr int LDD = Lay::LDD, LDL = Lay::LDL;
  constexpr int NTRI = NB * (NB + 1) / 2;
  static_assert(NCT % NW == 0, "key tiles must split evenly over waves");
  T* Kp = reinterpret_cast<T*>(smem + Lay::slot(0));
  T* Km = reinterpret_cast<T*>(smem + Lay::slot(1));
  T* Qp = reinterpret_cast<T*>(smem + Lay::slot(2));
  T* dWr = Qp;
  T* Vr = reinterpret_cast<T*>(smem + Lay::slot(3));
  T* Wn = reinterpret_cast<T*>(smem + Lay::slot(4));
  T* dOr = Wn;
  T* Ur = reinterpret_cast<T*>(smem + Lay::slot(5));
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
  const int c = a.c_lo + blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
  const int ct0 = wave * CPW;      // first key/value tile owned by this wave
  const int n = min(LC, f.T - c * LC);
  const size_t ci = (size_t)bh * f.NC + c;
  const size_t row0 = (size_t)bh * f.T + (size_t)c * LC;
  const T* q = reinterpret_cast<const T*>(f.q);
  const T* k = reinterpret_cast<const T*>(f.k);
  const T* v = reinterpret_cast<const T*>(f.v);
  const T* dO = reinterpret_cast<const T*>(a.dO);
  const T* Svk = reinterpret_cast<const T*>(f.S_vk) + ci * D * D;     // state entering the chunk
  const T* dSvk = reinterpret_cast<const T*>(a.dS_vk) + ci * D * D;   // gradient w.r.t. the state leaving it

  // ---- stage the chunk's raw inputs in LDS with coalesced 16-byte loads:
  // k, q, v (dtype) in the K+, Q+, V slots; log g in slots 4-5 and b from slot 6 on
  // (fp32, row stride D+4).  Tokens past the end read as k = q = v = 0, log g = 0, b = 1.
  constexpr int LDG = D + 4;
  float* lgS = reinterpret_cast<float*>(smem + Lay::slot(4));
  float* bS = reinterpret_cast<float*>(smem + Lay::slot(6));
  static_assert(sizeof(float) * LC * LDG <= 2 * Lay::S1, "log g staging exceeds two slots");
  static_assert(6 * Lay::S1 + sizeof(float) * LC * LDG <= Lay::small, "b staging exceeds the slots");
  // All of the chunk's global loads are issued here, from clamped rows (n >= 1), before
  // anything waits on them: the staged inputs, dO (written to LDS once its slot is
  // free), the chunk's inverse T = (I + A)^-1 from the prep pass (dtype), and w.
  constexpr int PR = D / 8;                      // 8-element pieces per token row
  constexpr int NST = LC * PR / NT;              // pieces per thread
  static_assert(NST * NT == LC * PR, "pieces must split evenly over the threads");
  const float wv = f.w[row0 + min(tid, n - 1)];
  Frag<T> kx[NST], qx[NST], vx[NST], dOx[NST];
  Frag<float> lx[NST], bx[NST];
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int idx = tid + NT * u, r = idx / PR, g = idx % PR;
    const size_t src = row0 * D + (unsigned)(min(r, n - 1) * D + 8 * g);
    kx[u] = load_frag(k + src);
    qx[u] = load_frag(q + src);
    vx[u] = load_frag(v + src);
    lx[u] = load_frag(f.log_g + src);
    if (HAS_B) bx[u] = load_frag(f.b + src);
    dOx[u] = load_frag(dO + src);
  }
  // gates as pre-activations: amplitude and bias of the thread's 8 channels (the same
  // for all of its pieces, as NT is a multiple of D / 8)
  Frag<float> pA, pT;
  if constexpr (LG) {
    static_assert(NT % PR == 0, "pieces of a thread must share their channels");
    pA = load_frag(f.gA + (bh % f.H) * D + 8 * (tid % PR));
    pT = load_frag(f.gtau + (bh % f.H) * D + 8 * (tid % PR));
  }
  constexpr int TP = LC * LC / 4, NTP = (TP + NT - 1) / NT;   // 4 consecutive columns per piece
  f32x4 tpre[NTP];
#pragma unroll
  for (int u = 0; u < NTP; ++u)
    tpre[u] = load4f(reinterpret_cast<const T*>(f.f.Tt) + ci * LC * LC + 4 * min(tid + NT * u, TP - 1));
  // k, q, v (dtype) into the K+, Q+, V slots; log g into slots 4-5 and b from slot 6 on
  // (fp32, row stride D+4).  Tokens past the end read as k = q = v = 0, log g = 0, b = 1.
  if (tid < LC) wL[tid] = (tid < n) ? (LG ? sigmoidf(wv) : wv) : 0.f;
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int idx = tid + NT * u, r = idx / PR, g = idx % PR;
    const bool valid = r < n;
    *reinterpret_cast<Frag<T>*>(Kp + r * LDD + 8 * g) = valid ? kx[u] : zero_frag(T());
    *reinterpret_cast<Frag<T>*>(Qp + r * LDD + 8 * g) = valid ? qx[u] : zero_frag(T());
    *reinterpret_cast<Frag<T>*>(Vr + r * LDD + 8 * g) = valid ? vx[u] : zero_frag(T());
    if constexpr (LG) {
      const LogitGates<D, HAS_B> gate{nullptr, f.gA, f.gtau};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lx[u].lo[e] = gate.logdecay_p(lx[u].lo[e], pA.lo[e], pT.lo[e]);
        lx[u].hi[e] = gate.logdecay_p(lx[u].hi[e], pA.hi[e], pT.hi[e]);
        if (HAS_B) {
          bx[u].lo[e] = sigmoidf(bx[u].lo[e]);
          bx[u].hi[e] = sigmoidf(bx[u].hi[e]);
        }
      }
    }
    Frag<float> lw = lx[u];
    lw.lo = valid ? lw.lo : f32x4{0.f, 0.f, 0.f, 0.f};
    lw.hi = valid ? lw.hi : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<Frag<float>*>(lgS + r * LDG + 8 * g) = lw;
    if (HAS_B) {
      Frag<float> bw = bx[u];
      bw.lo = valid ? bw.lo : f32x4{1.f, 1.f, 1.f, 1.f};
      bw.hi = valid ? bw.hi : f32x4{1.f, 1.f, 1.f, 1.f};
      *reinterpret_cast<Frag<float>*>(bS + r * LDG + 8 * g) = bw;
    }
  }
  __syncthreads();
  // ---- gate pass in accumulator layout: lane holds rows 16 rt + 4 lg + i of column 16 (ct0 + j) + lr
  f32x4 gam[NB][CPW];     // cumulative retention Gamma inside the chunk
  float gLc[CPW];         // Gamma_L of the lane's columns
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int col = 16 * (ct0 + j) + lr;
    float run = 1.f;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      float loc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        const float av = fexp(lgS[r * LDG + col]) * (HAS_B ? bS[r * LDG + col] : 1.f);
        loc[i] = (i == 0) ? av : loc[i - 1] * av;
      }
      // product of the 4-row groups of this row tile held by lanes with smaller lg
      float pre = run, tile = 1.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float tg = __shfl(loc[3], lr + 16 * g);
        if (g < lg) pre *= tg;
        tile *= tg;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gam[rt][j][i] = pre * loc[i];
        lgS[(16 * rt + 4 * lg + i) * LDG + col] = gam[rt][j][i];   // only this lane reads it
      }
      run *= tile;
    }
    gLc[j] = run;
    if (lg == 0) gLs[col] = run;
  }
  __syncthreads();
  // operand matrices K+ (in place), K-, Q+ (in place) in the staging pieces, with Gamma
  // read back from the log g slots; V stays raw
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int idx = tid + NT * u, r = idx / PR, g = idx % PR;
    const Frag<float> gm = load_frag(lgS + r * LDG + 8 * g);
    f32x4 ri0, ri1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ri0[e] = rcp(gm.lo[e]);
      ri1[e] = rcp(gm.hi[e]);
    }
    const Frag<T> kf = load_frag(Kp + r * LDD + 8 * g), qf = load_frag(Qp + r * LDD + 8 * g);
    *reinterpret_cast<Frag<T>*>(Kp + r * LDD + 8 * g) = scale_frag(kf, gm.lo, gm.hi);
    *reinterpret_cast<Frag<T>*>(Km + r * LDD + 8 * g) = scale_frag(kf, ri0, ri1);
    *reinterpret_cast<Frag<T>*>(Qp + r * LDD + 8 * g) = scale_frag(qf, gm.lo, gm.hi);
  }
  __syncthreads();

  // ---- P = tril(Q+ K-^T)
  for (int t = wave; t < NTRI; t += NW) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) mma(acc, frag<false>(Qp, LDD, 16 * i, kk), frag<false>(Km, LDD, 16 * j, kk));
    const int s = 16 * j + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) acc[ii] = (s <= 16 * i + 4 * lg + ii) ? acc[ii] : 0.f;
    lds_store_acc_tile(Pb, LDL, 16 * i, 16 * j, acc);
    if (j < i) {
      // the mirrored tile above the diagonal is zero in P and in dP (written later)
      lds_zero_tile(Pb, LDL, 16 * j, 16 * i);
      lds_zero_tile(dPb, LDL, 16 * j, 16 * i);
    }
  }
  // state fragments for U = Ubar - W S^T
  Frag<T> fS[KD][CPW];
  load_state_frags<T, D, CPW>(fS, Svk, ct0);
  // dtype copies of T and Tw = T diag(w)
#pragma unroll
  for (int u = 0; u < NTP; ++u) {
    const int idx = tid + NT * u;
    if (idx < TP) {
      const int r = idx / (LC / 4), s = 4 * (idx % (LC / 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Tb[r * LDL + s + e] = to<T>(tpre[u][e]);
        Twb[r * LDL + s + e] = to<T>(tpre[u][e] * wL[s + e]);
      }
    }
  }
  __syncthreads();

  // ---- W = Tw K+ (stored negated), Ubar = Tw V (kept as U's accumulator)
  {
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KL>(acc, LdsSrc<T, false>{Twb, LDL}, LdsSrc<T, true>{Kp, LDD}, ct0);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) lds_store_acc_tile(Wn, LDD, 16 * rt, 16 * (ct0 + j), -acc[rt][j]);
  }
  f32x4 accU[NB][CPW];
  zero_acc(accU);
  owned_mma<T, NB, CPW, KL>(accU, LdsSrc<T, false>{Twb, LDL}, LdsSrc<T, true>{Vr, LDD}, ct0);
  __syncthreads();

  // ---- U = Ubar + (-W) S^T  -> row-major U
  owned_mma<T, NB, CPW, KD>(accU, LdsSrc<T, false>{Wn, LDD}, fS);
#pragma unroll
  for (int rt = 0; rt < NB; ++rt)
#pragma unroll
    for (int j = 0; j < CPW; ++j) lds_store_acc_tile(Ur, LDD, 16 * rt, 16 * (ct0 + j), accU[rt][j]);
  Frag<T> fG[KD][CPW];                       // dS' fragments, scaled to dS' Diag(Gamma_L) for dU
  load_state_frags<T, D, CPW>(fG, dSvk, ct0);
  __syncthreads();   // -W no longer needed: its slot takes dO

  // ---- dO into LDS (row-major, zero for tokens past the end)
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int idx = tid + NT * u, r = idx / PR, g = idx % PR;
    *reinterpret_cast<Frag<T>*>(dOr + r * LDD + 8 * g) = (r < n) ? dOx[u] : zero_frag(T());
  }
  __syncthreads();

  // ---- dU = P^T dO + K- (dS' Diag(Gamma_L))^T  -> row-major dU
  {
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KL>(acc, LdsSrc<T, true>{Pb, LDL}, LdsSrc<T, true>{dOr, LDD}, ct0);
    // column scaling by Gamma_L: the lane's values of block kb sit at k = 32 kb + 8 lg + e
#pragma unroll
    for (int kb = 0; kb < KD; ++kb) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gLs + 32 * kb + 8 * lg);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gLs + 32 * kb + 8 * lg + 4);
#pragma unroll
      for (int j = 0; j < CPW; ++j) fG[kb][j] = scale_frag(fG[kb][j], g0, g1);
    }
    owned_mma<T, NB, CPW, KD>(acc, LdsSrc<T, false>{Km, LDD}, fG);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) lds_store_acc_tile(dUr, LDD, 16 * rt, 16 * (ct0 + j), acc[rt][j]);
  }
  KmajorPieces<T> pSk[KD][CPW], pDk[KD][CPW];   // S and dS' with rows k, for the key-owned products
  load_state_kmajor<T, D, CPW>(pSk, Svk, ct0);
  load_state_kmajor<T, D, CPW>(pDk, dSvk, ct0);
  // ---- dP = tril(dO U^T)
  for (int t = wave; t < NTRI; t += NW) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) mma(acc, frag<false>(dOr, LDD, 16 * i, kk), frag<false>(Ur, LDD, 16 * j, kk));
    const int s = 16 * j + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) acc[ii] = (s <= 16 * i + 4 * lg + ii) ? acc[ii] : 0.f;
    lds_store_acc_tile(dPb, LDL, 16 * i, 16 * j, acc);
  }
  __syncthreads();

  // ---- token x key gradients of this wave's columns, folded as they are produced into
  //   dK = Gamma dK+ + dK- / Gamma + (Gamma_L / Gamma) dK->        (gradient w.r.t. k)
  //   dG = K+ dK+ - K- dK- + Q+ dQ+ - K-> dK->                        (gradient w.r.t. the
  //        cumulative log-retention, elementwise; K-> = K- Gamma_L)
  Frag<T> fSk[KD][CPW], fDk[KD][CPW];
  f32x4 dK[NB][CPW], dG[NB][CPW];
  float gsum[CPW];        // sum over tokens of K-> .* dK-> per column (part of the G_L term)
  // M[16 rt + 4 lg + i][16 (ct0 + j) + lr], i = 0..3: the lane's accumulator-layout
  // elements of an operand matrix in LDS
  auto lds_tile = [&](const T* m, int rt, int j) { return lds_acc_tile(m, LDD, 16 * rt, 16 * (ct0 + j)); };
  {
    // dQ+ = dO S + dP K-  -> dq = Gamma dQ+, dG = Q+ dQ+
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KL>(acc, LdsSrc<T, false>{dPb, LDL}, LdsSrc<T, true>{Km, LDD}, ct0);
    finish_kmajor(fSk, pSk);
    owned_mma<T, NB, CPW, KD>(acc, LdsSrc<T, false>{dOr, LDD}, fSk);
    finish_kmajor(fDk, pDk);
    T* dq = reinterpret_cast<T*>(a.dq);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 qv = lds_tile(Qp, rt, j);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          dG[rt][j][ii] = qv[ii] * acc[rt][j][ii];
          if (r < n) dq[row0 * D + (unsigned)(r * D + 16 * (ct0 + j) + lr)] = to<T>(gam[rt][j][ii] * acc[rt][j][ii]);
        }
      }
  }
  {
    // dK-> = U dS'  -> dK = (Gamma_L / Gamma) dK->, dG -= K-> dK->
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KD>(acc, LdsSrc<T, false>{Ur, LDD}, fDk);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      float cs = 0.f;
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 kmv = lds_tile(Km, rt, j);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float kf = kmv[ii] * gLc[j];       // K->
          dK[rt][j][ii] = gLc[j] * rcp(gam[rt][j][ii]) * acc[rt][j][ii];
          dG[rt][j][ii] -= kf * acc[rt][j][ii];
          cs += kf * acc[rt][j][ii];
        }
      }
      gsum[j] = cs;
    }
    // G_L term of each column: sum_s K->_s dK->_s + Gamma_L sum_v S[v][k] dS'[v][k]
    // (the lane's fragments hold S and dS' at v = 32 kb + 8 lg + e of column 16 (ct0 + j) + lr)
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      float sd = 0.f;
#pragma unroll
      for (int kb = 0; kb < KD; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) sd += tof(frag_elem(fSk[kb][j], e)) * tof(frag_elem(fDk[kb][j], e));
      float tot = gLc[j] * sd;
      tot += __shfl_xor(tot, 16);
      tot += __shfl_xor(tot, 32);
      float gs = gsum[j];
      gs += __shfl_xor(gs, 16);
      gs += __shfl_xor(gs, 32);
      if (lg == 0) glt[16 * (ct0 + j) + lr] = tot + gs;
    }
  }
  {
    // dK- (first part) = dP^T Q+  -> dK += dK- / Gamma, dG -= K- dK-
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KL>(acc, LdsSrc<T, true>{dPb, LDL}, LdsSrc<T, true>{Qp, LDD}, ct0);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 kmv = lds_tile(Km, rt, j);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          dK[rt][j][ii] += rcp(gam[rt][j][ii]) * acc[rt][j][ii];
          dG[rt][j][ii] -= kmv[ii] * acc[rt][j][ii];
        }
      }
  }
  __syncthreads();   // Q+ is dead: its slot takes dW

  // ---- dW = -dU S  -> row-major dW
  {
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KD>(acc, LdsSrc<T, false>{dUr, LDD}, fSk);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) lds_store_acc_tile(dWr, LDD, 16 * rt, 16 * (ct0 + j), -acc[rt][j]);
  }
  __syncthreads();

  // ---- dT' = dW K+^T + dU V^T (lower tiles); dT = dT' diag(w); dw term sum_i T[i][r] dT'[i][r]
  for (int t = wave; t < NTRI; t += NW) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) {
      mma(acc, frag<false>(dWr, LDD, 16 * i, kk), frag<false>(Kp, LDD, 16 * j, kk));
      mma(acc, frag<false>(dUr, LDD, 16 * i, kk), frag<false>(Vr, LDD, 16 * j, kk));
    }
    const int s = 16 * j + lr;
    float cs = 0.f;
    const f32x4 tv = lds_acc_tile(Tb, LDL, 16 * i, 16 * j);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) cs += tv[ii] * acc[ii];
    lds_store_acc_tile(dTb, LDL, 16 * i, 16 * j, acc * wL[s]);
    if (j < i) lds_zero_tile(dTb, LDL, 16 * j, 16 * i);   // mirrored tile: zero
    cs += __shfl_xor(cs, 16);
    cs += __shfl_xor(cs, 32);
    if (lg == 0) {
      dwp[i * LC + s] = cs;
      if (j < i) dwp[j * LC + 16 * i + lr] = 0.f;      // tiles above the diagonal contribute nothing
    }
  }
  // ---- dV = Tw^T dU (write dv); dK+ (first part) = Tw^T dW -> dK += Gamma dK+, dG += K+ dK+
  {
    f32x4 acc[NB][CPW], acc2[NB][CPW];
    zero_acc(acc);
    zero_acc(acc2);
    owned_mma<T, NB, CPW, KL>(acc, LdsSrc<T, true>{Twb, LDL}, LdsSrc<T, true>{dUr, LDD}, ct0);
    owned_mma<T, NB, CPW, KL>(acc2, LdsSrc<T, true>{Twb, LDL}, LdsSrc<T, true>{dWr, LDD}, ct0);
    T* dv = reinterpret_cast<T*>(a.dv);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 kpv = lds_tile(Kp, rt, j);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          if (r < n) dv[row0 * D + (unsigned)(r * D + 16 * (ct0 + j) + lr)] = to<T>(acc[rt][j][ii]);
          dK[rt][j][ii] += gam[rt][j][ii] * acc2[rt][j][ii];
          dG[rt][j][ii] += kpv[ii] * acc2[rt][j][ii];
        }
      }
  }
  __syncthreads();   // dT complete; dP no longer needed (its slot takes Z)

  // ---- Z = dT T^T (lower tiles)
  for (int t = wave; t < NTRI; t += NW) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < LC; kk += 32) mma(acc, frag<false>(dTb, LDL, 16 * i, kk), frag<false>(Tb, LDL, 16 * j, kk));
    lds_store_acc_tile(Zb, LDL, 16 * i, 16 * j, acc);
  }
  __syncthreads();
  // b at the lane's gradient positions, for db = dlog a / b; loaded here so that the
  // loads are consumed before the chunk's gradient stores are issued
  float binv[CPW][NB][4];
  if (HAS_B) {
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          binv[j][rt][ii] = f.b[row0 * D + (unsigned)(min(16 * rt + 4 * lg + ii, n - 1) * D + 16 * (ct0 + j) + lr)];
  }
  // ---- dA = -T^T Z (strictly lower), dB = diag(w) dA; dw term sum_s B_rs dA_rs
  {
    constexpr int MAXT = (NTRI + NW - 1) / NW;
    f32x4 dA[MAXT];
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int t = wave + NW * u;
      dA[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < NTRI) {
        int i, j;
        tri_index(t, i, j);
#pragma unroll
        for (int kk = 0; kk < LC; kk += 32) mma(dA[u], frag<true>(Tb, LDL, 16 * i, kk), frag<true>(Zb, LDL, 16 * j, kk));
        f32x4 bacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D; kk += 32) mma(bacc, frag<false>(Kp, LDD, 16 * i, kk), frag<false>(Km, LDD, 16 * j, kk));
        const int s = 16 * j + lr;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * i + 4 * lg + ii;
          const float da = (s < r) ? -dA[u][ii] : 0.f;
          dA[u][ii] = da;
          const float rs = row16_sum(bacc[ii] * da);
          if (lr == 0) dwq[j * LC + r] = rs;
        }
      }
    }
    __syncthreads();   // every read of Z is done
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int t = wave + NW * u;
      if (t < NTRI) {
        int i, j;
        tri_index(t, i, j);
        f32x4 v;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v[ii] = wL[16 * i + 4 * lg + ii] * dA[u][ii];
        lds_store_acc_tile(dAb, LDL, 16 * i, 16 * j, v);
        if (j < i) {
          // mirrored tile above the diagonal: zero, and no row-sum contribution
          lds_zero_tile(dAb, LDL, 16 * j, 16 * i);
          if (lr == 0) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) dwq[i * LC + 16 * j + 4 * lg + ii] = 0.f;
          }
        }
      }
    }
  }
  __syncthreads();

  if (HAS_B) {
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          // d/db = dlog a / b; with pre-activations d/db_x = d/db * b (1 - b) = dlog a * sigmoid(-b_x);
          // for b = sigmoid(x) given as b (db_mode 1), d/dx = dlog a (1 - b)
          binv[j][rt][ii] = LG ? sigmoidf(-binv[j][rt][ii]) : (a.db_mode ? 1.f - binv[j][rt][ii] : rcp(binv[j][rt][ii]));
  }
  // ---- dK+ += dB K-, dK- += dB^T K+
  {
    f32x4 accp[NB][CPW], accm[NB][CPW];
    zero_acc(accp);
    zero_acc(accm);
    owned_mma<T, NB, CPW, KL>(accp, LdsSrc<T, false>{dAb, LDL}, LdsSrc<T, true>{Km, LDD}, ct0);
    owned_mma<T, NB, CPW, KL>(accm, LdsSrc<T, true>{dAb, LDL}, LdsSrc<T, true>{Kp, LDD}, ct0);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 kpv = lds_tile(Kp, rt, j), kmv = lds_tile(Km, rt, j);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float g = gam[rt][j][ii];
          dK[rt][j][ii] += g * accp[rt][j][ii] + rcp(g) * accm[rt][j][ii];
          dG[rt][j][ii] += kpv[ii] * accp[rt][j][ii] - kmv[ii] * accm[rt][j][ii];
        }
      }
  }
  __syncthreads();   // glt, dwp, dwq complete

  // ---- dlog a = reverse cumulative sum of dG over the chunk's tokens + G_L term
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int col = 16 * (ct0 + j) + lr;
    float run = glt[col];
#pragma unroll
    for (int rt = NB - 1; rt >= 0; --rt) {
      float loc[4];
      loc[3] = dG[rt][j][3];
      loc[2] = loc[3] + dG[rt][j][2];
      loc[1] = loc[2] + dG[rt][j][1];
      loc[0] = loc[1] + dG[rt][j][0];
      float post = run, tile = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float tg = __shfl(loc[0], lr + 16 * g);
        if (g > lg) post += tg;
        tile += tg;
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) dG[rt][j][ii] = post + loc[ii];    // dlog a
      run += tile;
    }
  }
  // gradient stores; a full chunk stores without per-element token checks
  auto store_grads = [&](auto full) {
    T* dk = reinterpret_cast<T*>(a.dk);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          if (decltype(full)::value || r < n) {
            const size_t idx = row0 * D + (unsigned)(r * D + 16 * (ct0 + j) + lr);
            a.dlog_g[idx] = dG[rt][j][ii];
            if (HAS_B) a.db[idx] = dG[rt][j][ii] * binv[j][rt][ii];
            dk[idx] = to<T>(dK[rt][j][ii]);
          }
        }
  };
  if (n == LC) store_grads(std::true_type{});
  else store_grads(std::false_type{});
  // ---- dw_r = sum_s B_rs dA_rs + sum_i T[i][r] dT'[i][r]
  if (tid < LC && tid < n) {
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < NB; ++t) s += dwq[t * LC + tid] + dwp[t * LC + tid];
    a.dw[row0 + tid] = LG ? s * wL[tid] * (1.f - wL[tid]) : s;     // d/dw_hat = d/dw * w (1 - w)
  }
}

// Range-safe path of the chunk gradients (chunks whose log-retention over the chunk
// falls below -kChunkSafe in some key channel): operands referred to their 16-token
// blocks, as described with the layout above.
template <typename T, int LC, int D, bool HAS_B, bool LG>
__device__ __forceinline__ void bwd_chunk_range(const BwdArgs& a, unsigned char* smem) {
  using Lay = GradLayout<T, LC, D>;
  // one wave per 16-column tile of the key/value width: NW = D/16 waves
  constexpr int NW = D / 16, NT = 64 * NW;
  constexpr int NB = LC / 16, NCT = D / 16, CPW = NCT / NW, KD = D / 32, KL = LC / 32;
  constexpr int LDD = Lay::LDD, LDL = Lay::LDL;
  constexpr int NTRI = NB * (NB + 1) / 2;
  static_assert(NCT % NW == 0, "key tiles must split evenly over waves");
  T* Kp = reinterpret_cast<T*>(smem + Lay::slot(0));
  T* Km = reinterpret_cast<T*>(smem + Lay::slot(1));
  T* Qp = reinterpret_cast<T*>(smem + Lay::slot(2));
  T* dWr = Qp;
  T* Vr = reinterpret_cast<T*>(smem + Lay::slot(3));
  T* Wn = reinterpret_cast<T*>(smem + Lay::slot(4));
  T* dOr = Wn;
  T* Ur = reinterpret_cast<T*>(smem + Lay::slot(5));
  T* dUr = reinterpret_cast<T*>(smem + Lay::slot(6));
  T* Pb = reinterpret_cast<T*>(smem + Lay::pslot(0));
  T* dTb = Pb;
  T* Tb = reinterpret_cast<T*>(smem + Lay::pslot(1));
  T* Twb = reinterpret_cast<T*>(smem + Lay::pslot(2));
  float* cKT = reinterpret_cast<float*>(smem + Lay::pslot(2));   // [NB][D] e^(G_L - Gb[J+1]) once Tw is done
  float* gbeT = cKT;                                               // [NB][D] e^Gb[J] for dT'
  T* dPb = reinterpret_cast<T*>(smem + Lay::pslot(3));
  float* btT = reinterpret_cast<float*>(smem + Lay::pslot(3));   // [NB][D] block log-retention (gate pass)
  T* Zb = dPb;
  T* dAb = dPb;
  float* wL = reinterpret_cast<float*>(smem + Lay::small);
  float* gLs = wL + LC;
  float* dwp = gLs + D;            // [NB][LC] column sums of T .* dT' per token-tile row
  float* dwq = dwp + NB * LC;      // [NB][LC] row sums of B .* dA per token-tile column
  float* glt = dwq + NB * LC;      // [D] G_L term per key column
  int* flags = reinterpret_cast<int*>(glt + D);   // [NB] block needs the exact within-block terms
  static_assert(sizeof(float) * NB * D * 2 <= Lay::S2, "gate tables exceed a tile slot");

  const FwdArgs& f = a.fwd;
  const int c = a.c_lo + blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
  const int ct0 = wave * CPW;      // first key/value tile owned by this wave
  const int n = min(LC, f.T - c * LC);
  const size_t ci = (size_t)bh * f.NC + c;
  const size_t row0 = (size_t)bh * f.T + (size_t)c * LC;
  const T* q = reinterpret_cast<const T*>(f.q);
  const T* k = reinterpret_cast<const T*>(f.k);
  const T* v = reinterpret_cast<const T*>(f.v);
  const T* dO = reinterpret_cast<const T*>(a.dO);
  const T* Svk = reinterpret_cast<const T*>(f.S_vk) + ci * D * D;     // state entering the chunk
  const T* dSvk = reinterpret_cast<const T*>(a.dS_vk) + ci * D * D;   // gradient w.r.t. the state leaving it

  // ---- stage the chunk's raw inputs in LDS with coalesced 16-byte loads: k, q, v (dtype)
  // in the K^+, Q^+, V slots; the per-token log-retention la = log g + log b (clamped as
  // in the prep pass) in slots 4-5 (fp32, row stride D+4); P from the prep pass.  Tokens
  // past the end read as k = q = v = 0, la = 0.
  constexpr int LDG = D + 4;
  float* lgS = reinterpret_cast<float*>(smem + Lay::slot(4));
  static_assert(sizeof(float) * LC * LDG <= 2 * Lay::S1, "log-retention staging exceeds two slots");
  // All of the chunk's global loads are issued here, from clamped rows (n >= 1), before
  // anything waits on them: the staged inputs, dO (written to LDS once its slot is
  // free), the chunk's inverse T = (I + A)^-1 and P from the prep pass (dtype), and w.
  constexpr int PR = D / 8;                      // 8-element pieces per token row
  constexpr int NST = LC * PR / NT;              // pieces per thread
  static_assert(NST * NT == LC * PR, "pieces must split evenly over the threads");
  const float wv = f.w[row0 + min(tid, n - 1)];
  Frag<T> kx[NST], qx[NST], vx[NST], dOx[NST];
  Frag<float> lx[NST], bx[NST];
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int idx = tid + NT * u, r = idx / PR, g = idx % PR;
    const size_t src = row0 * D + (unsigned)(min(r, n - 1) * D + 8 * g);
    kx[u] = load_frag(k + src);
    qx[u] = load_frag(q + src);
    vx[u] = load_frag(v + src);
    lx[u] = load_frag(f.log_g + src);
    if (HAS_B) bx[u] = load_frag(f.b + src);
    dOx[u] = load_frag(dO + src);
  }
  // gates as pre-activations: amplitude and bias of the thread's 8 channels (the same
  // for all of its pieces, as NT is a multiple of D / 8)
  Frag<float> pA, pT;
  if constexpr (LG) {
    static_assert(NT % PR == 0, "pieces of a thread must share their channels");
    pA = load_frag(f.gA + (bh % f.H) * D + 8 * (tid % PR));
    pT = load_frag(f.gtau + (bh % f.H) * D + 8 * (tid % PR));
  }
  constexpr int TP = LC * LC / 4, NTP = (TP + NT - 1) / NT;   // 4 consecutive columns per piece
  f32x4 tpre[NTP], ppre[NTP];
#pragma unroll
  for (int u = 0; u < NTP; ++u) {
    const size_t o = ci * LC * LC + 4 * min(tid + NT * u, TP - 1);
    tpre[u] = load4f(reinterpret_cast<const T*>(f.f.Tt) + o);
    ppre[u] = load4f(reinterpret_cast<const T*>(f.f.Pt) + o);
  }
  if (tid < LC) wL[tid] = (tid < n) ? (LG ? sigmoidf(wv) : wv) : 0.f;
  if (tid < 16) flags[tid] = 0;
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int idx = tid + NT * u, r = idx / PR, g = idx % PR;
    const bool valid = r < n;
    *reinterpret_cast<Frag<T>*>(Kp + r * LDD + 8 * g) = valid ? kx[u] : zero_frag(T());
    *reinterpret_cast<Frag<T>*>(Qp + r * LDD + 8 * g) = valid ? qx[u] : zero_frag(T());
    *reinterpret_cast<Frag<T>*>(Vr + r * LDD + 8 * g) = valid ? vx[u] : zero_frag(T());
    Frag<float> lw;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float la = frag_elem(lx[u], e);
      if constexpr (LG) la = -(e < 4 ? pA.lo[e] : pA.hi[e - 4]) * softplusf(la + (e < 4 ? pT.lo[e] : pT.hi[e - 4]));
      if constexpr (HAS_B) la += LG ? -softplusf(-frag_elem(bx[u], e)) : flog(frag_elem(bx[u], e));
      la = valid ? clamp_la(la) : 0.f;
      if (e < 4) lw.lo[e] = la;
      else lw.hi[e - 4] = la;
    }
    *reinterpret_cast<Frag<float>*>(lgS + r * LDG + 8 * g) = lw;
  }
#pragma unroll
  for (int u = 0; u < NTP; ++u) {
    const int idx = tid + NT * u;
    if (idx < TP) store4(Pb + (idx / (LC / 4)) * LDL + 4 * (idx % (LC / 4)), ppre[u]);
  }
  __syncthreads();
  // ---- gate pass in accumulator layout: lane holds rows 16 rt + 4 lg + i of column
  // 16 (ct0 + j) + lr.  Inclusive sums of la inside each 16-token block (loc = G - Gb),
  // the block log-retention btot and the block starts Gb; loc goes back over the staged
  // la (each lane overwrites only what it read)
  f32x4 loc[NB][CPW];
  float gbs[NB][CPW], bto[NB][CPW], GLs[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int col = 16 * (ct0 + j) + lr;
    float run = 0.f;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      float cs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cs[i] = (i == 0 ? 0.f : cs[i - 1]) + lgS[(16 * rt + 4 * lg + i) * LDG + col];
      // sum of the 4-row groups of this block held by lanes with smaller lg
      float pre = 0.f, tile = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float tg = __shfl(cs[3], lr + 16 * g);
        if (g < lg) pre += tg;
        tile += tg;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        loc[rt][j][i] = pre + cs[i];
        lgS[(16 * rt + 4 * lg + i) * LDG + col] = loc[rt][j][i];
      }
      gbs[rt][j] = run;
      bto[rt][j] = tile;
      run += tile;
    }
    GLs[j] = run;
    if (lg == 0) {
      gLs[col] = fexp(run);
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        btT[rt * D + col] = bto[rt][j];
        if (-bto[rt][j] > kSafeLog) flags[rt] = 1;
      }
    }
  }
  __syncthreads();
  bool unsafe[NB];
  int mask = 0;
#pragma unroll
  for (int I = 0; I < NB; ++I) {
    unsafe[I] = flags[I] != 0;
    mask |= unsafe[I] ? 1 << I : 0;
  }

  // the lane's factor of block pair (I, J), J <= I: e^(Gb[I] - Gb[J+1]); on the diagonal
  // e^-btot_I, or 0 where the exact terms replace the block's product
  auto dfac = [&](int I, int J, int j) -> float {
    if (I == J) return unsafe[I] ? 0.f : fexp(-bto[I][j]);
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < NB; ++m)
      if (m > J && m < I) s += bto[m][j];
    return I == J + 1 ? 1.f : fexp(s);
  };
  // operand matrices K^+ (in place), K^-, Q^+ (in place) in the staging pieces, with loc
  // read back from the staging slots and btot from the table; V stays raw
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int idx = tid + NT * u, r = idx / PR, g = idx % PR;
    const Frag<float> lc = load_frag(lgS + r * LDG + 8 * g);
    const Frag<float> bt = load_frag(btT + (r / 16) * D + 8 * g);
    f32x4 eo0, eo1, ee0, ee1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      eo0[e] = fexp(lc.lo[e]);
      eo1[e] = fexp(lc.hi[e]);
      ee0[e] = fexp(bt.lo[e] - lc.lo[e]);
      ee1[e] = fexp(bt.hi[e] - lc.hi[e]);
    }
    const Frag<T> kf = load_frag(Kp + r * LDD + 8 * g), qf = load_frag(Qp + r * LDD + 8 * g);
    *reinterpret_cast<Frag<T>*>(Kp + r * LDD + 8 * g) = scale_frag(kf, eo0, eo1);
    *reinterpret_cast<Frag<T>*>(Km + r * LDD + 8 * g) = scale_frag(kf, ee0, ee1);
    *reinterpret_cast<Frag<T>*>(Qp + r * LDD + 8 * g) = scale_frag(qf, eo0, eo1);
  }
  // state fragments for U = Ubar - W S^T
  Frag<T> fS[KD][CPW];
  load_state_frags<T, D, CPW>(fS, Svk, ct0);
  // dtype copies of T and Tw = T diag(w)
#pragma unroll
  for (int u = 0; u < NTP; ++u) {
    const int idx = tid + NT * u;
    if (idx < TP) {
      const int r = idx / (LC / 4), s = 4 * (idx % (LC / 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Tb[r * LDL + s + e] = to<T>(tpre[u][e]);
        Twb[r * LDL + s + e] = to<T>(tpre[u][e] * wL[s + e]);
      }
    }
  }
  __syncthreads();

  // ---- W = Tw K+ with K+ = K^+ e^Gb (chunk reference: block J's factor on the lane's
  // column), stored negated; Ubar = Tw V (kept as U's accumulator)
  {
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma_blk<T, NB, CPW, true>(
        acc, [&](int ob, int kb) { return lds_frag16_rows(Twb, LDL, 16 * ob, 16 * kb); },
        [&](int kb, int ct) { return lds_frag16_cols(Kp, LDD, 16 * ct, 16 * kb); }, ct0,
        [&](int, int J, int j) { return fexp(gbs[J][j]); });
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) lds_store_acc_tile(Wn, LDD, 16 * rt, 16 * (ct0 + j), -acc[rt][j]);
  }
  f32x4 accU[NB][CPW];
  zero_acc(accU);
  owned_mma<T, NB, CPW, KL>(accU, LdsSrc<T, false>{Twb, LDL}, LdsSrc<T, true>{Vr, LDD}, ct0);
  __syncthreads();

  // ---- U = Ubar + (-W) S^T  -> row-major U
  owned_mma<T, NB, CPW, KD>(accU, LdsSrc<T, false>{Wn, LDD}, fS);
#pragma unroll
  for (int rt = 0; rt < NB; ++rt)
#pragma unroll
    for (int j = 0; j < CPW; ++j) lds_store_acc_tile(Ur, LDD, 16 * rt, 16 * (ct0 + j), accU[rt][j]);
  Frag<T> fG[KD][CPW];                       // dS' fragments
  load_state_frags<T, D, CPW>(fG, dSvk, ct0);
  __syncthreads();   // -W and Tw no longer needed: their slots take dO and the K-> factors

  // ---- dO into LDS (row-major, zero for tokens past the end); e^(G_L - Gb[J+1]) of the
  // lane's column (the suffix of the block log-retentions) into the table
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int idx = tid + NT * u, r = idx / PR, g = idx % PR;
    *reinterpret_cast<Frag<T>*>(dOr + r * LDD + 8 * g) = (r < n) ? dOx[u] : zero_frag(T());
  }
  if (lg == 0) {
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      float sfx = 0.f;
#pragma unroll
      for (int rt = NB - 1; rt >= 0; --rt) {
        cKT[rt * D + 16 * (ct0 + j) + lr] = fexp(sfx);
        sfx += bto[rt][j];
      }
    }
  }
  __syncthreads();

  // ---- dU = P^T dO + K-> dS'^T, K->_s = K^-_s e^(G_L - Gb[J+1]) for s in block J (the
  // factor of the contraction's key channels, applied to the dS' fragment per row block)
  {
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KL>(acc, LdsSrc<T, true>{Pb, LDL}, LdsSrc<T, true>{dOr, LDD}, ct0);
#pragma unroll
    for (int kb = 0; kb < KD; ++kb) {
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(cKT + rt * D + 32 * kb + 8 * lg);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(cKT + rt * D + 32 * kb + 8 * lg + 4);
        const Frag<T> af = frag<false>(Km, LDD, 16 * rt, 32 * kb);
#pragma unroll
        for (int j = 0; j < CPW; ++j) mma(acc[rt][j], af, scale_frag(fG[kb][j], g0, g1));
      }
    }
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) lds_store_acc_tile(dUr, LDD, 16 * rt, 16 * (ct0 + j), acc[rt][j]);
  }
  KmajorPieces<T> pSk[KD][CPW], pDk[KD][CPW];   // S and dS' with rows k, for the key-owned products
  load_state_kmajor<T, D, CPW>(pSk, Svk, ct0);
  load_state_kmajor<T, D, CPW>(pDk, dSvk, ct0);
  // ---- dP = tril(dO U^T) (the mirrored tiles above the diagonal are zero)
  for (int t = wave; t < NTRI; t += NW) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) mma(acc, frag<false>(dOr, LDD, 16 * i, kk), frag<false>(Ur, LDD, 16 * j, kk));
    const int s = 16 * j + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) acc[ii] = (s <= 16 * i + 4 * lg + ii) ? acc[ii] : 0.f;
    lds_store_acc_tile(dPb, LDL, 16 * i, 16 * j, acc);
    if (j < i) lds_zero_tile(dPb, LDL, 16 * j, 16 * i);
    if (i == j && unsafe[i]) store4(reinterpret_cast<T*>(a.diag) + ((ci * NB + i) * 2 * 64 + lane) * 4, acc);
  }
  __syncthreads();

  // ---- token x key gradients of this wave's columns, folded as they are produced into
  //   dk (gradient w.r.t. k) and dG (gradient w.r.t. the cumulative log-retention G,
  //   elementwise): per term, the row role of a ratio-weighted product adds
  //   e^loc X to dk and K^+ X to dG, the column role e^(btot - loc) X to dk and -K^- X
  //   to dG (X before the element's own factor)
  Frag<T> fSk[KD][CPW], fDk[KD][CPW];
  f32x4 dK[NB][CPW], dG[NB][CPW];
  zero_acc(dK);
  float gsum[CPW];        // sum over tokens of K-> .* dK-> per column (part of the G_L term)
  // M[16 rt + 4 lg + i][16 (ct0 + j) + lr], i = 0..3: the lane's accumulator-layout
  // elements of an operand matrix in LDS
  auto lds_tile = [&](const T* m, int rt, int j) { return lds_acc_tile(m, LDD, 16 * rt, 16 * (ct0 + j)); };
  {
    // dQ+ = (dO S) e^Gb + X2 with X2 = sum_J D_IJ (dP_IJ K^-_J): dq = e^loc dQ+, dG = Q^+ dQ+
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    finish_kmajor(fSk, pSk);
    owned_mma<T, NB, CPW, KD>(acc, LdsSrc<T, false>{dOr, LDD}, fSk);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) acc[rt][j] *= fexp(gbs[rt][j]);
    owned_mma_blk<T, NB, CPW, true>(
        acc, [&](int ob, int kb) { return lds_frag16_rows(dPb, LDL, 16 * ob, 16 * kb); },
        [&](int kb, int ct) { return lds_frag16_cols(Km, LDD, 16 * ct, 16 * kb); }, ct0, dfac);
    finish_kmajor(fDk, pDk);
    T* dq = reinterpret_cast<T*>(a.dq);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 qv = lds_tile(Qp, rt, j);
        f32x4 dqv;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float y = acc[rt][j][ii];
          dG[rt][j][ii] = qv[ii] * y;
          dqv[ii] = fexp(loc[rt][j][ii]) * y;
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          if (r < n) dq[row0 * D + (unsigned)(r * D + 16 * (ct0 + j) + lr)] = to<T>(dqv[ii]);
        }
      }
  }
  {
    // dK-> = U dS'  -> dk += e^(G_L - G) dK->, dG -= K-> dK->
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KD>(acc, LdsSrc<T, false>{Ur, LDD}, fDk);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      float cs = 0.f, tail = 0.f;
#pragma unroll
      for (int rt = NB - 1; rt >= 0; --rt) {
        const float eK = fexp(tail);             // e^(G_L - Gb[rt+1])
        const f32x4 kmv = lds_tile(Km, rt, j);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float kf = kmv[ii] * eK;           // K->
          dK[rt][j][ii] += fexp(bto[rt][j] - loc[rt][j][ii]) * eK * acc[rt][j][ii];
          dG[rt][j][ii] -= kf * acc[rt][j][ii];
          cs += kf * acc[rt][j][ii];
        }
        tail += bto[rt][j];
      }
      gsum[j] = cs;
    }
    // G_L term of each column: sum_s K->_s dK->_s + Gamma_L sum_v S[v][k] dS'[v][k]
    // (the lane's fragments hold S and dS' at v = 32 kb + 8 lg + e of column 16 (ct0 + j) + lr)
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      float sd = 0.f;
#pragma unroll
      for (int kb = 0; kb < KD; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) sd += tof(frag_elem(fSk[kb][j], e)) * tof(frag_elem(fDk[kb][j], e));
      float tot = fexp(GLs[j]) * sd;
      tot += __shfl_xor(tot, 16);
      tot += __shfl_xor(tot, 32);
      float gs = gsum[j];
      gs += __shfl_xor(gs, 16);
      gs += __shfl_xor(gs, 32);
      if (lg == 0) glt[16 * (ct0 + j) + lr] = tot + gs;
    }
  }
  {
    // column role of the dP product: X3 = sum_I D_IJ (dP_IJ^T Q^+_I)
    //   -> dk += e^(btot - loc) X3, dG -= K^- X3
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma_blk<T, NB, CPW, false>(
        acc, [&](int ob, int kb) { return lds_frag16_cols(dPb, LDL, 16 * ob, 16 * kb); },
        [&](int kb, int ct) { return lds_frag16_cols(Qp, LDD, 16 * ct, 16 * kb); }, ct0, dfac);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 kmv = lds_tile(Km, rt, j);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          dK[rt][j][ii] += fexp(bto[rt][j] - loc[rt][j][ii]) * acc[rt][j][ii];
          dG[rt][j][ii] -= kmv[ii] * acc[rt][j][ii];
        }
      }
  }
  __syncthreads();   // Q^+ is dead: its slot takes dW; the K-> table's slot takes e^Gb

  // ---- dW = -dU S  -> row-major dW; e^Gb of the lane's column into the table for dT'
  {
    f32x4 acc[NB][CPW];
    zero_acc(acc);
    owned_mma<T, NB, CPW, KD>(acc, LdsSrc<T, false>{dUr, LDD}, fSk);
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
      for (int j = 0; j < CPW; ++j) lds_store_acc_tile(dWr, LDD, 16 * rt, 16 * (ct0 + j), -acc[rt][j]);
    if (lg == 0) {
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) gbeT[rt * D + 16 * (ct0 + j) + lr] = fexp(gbs[rt][j]);
    }
  }
  __syncthreads();

  // ---- dT' = dW K+^T + dU V^T (lower tiles; K+ = K^+ e^Gb, the factor of the key channels
  // of block j applied to the fragment); dT = dT' diag(w); dw term sum_i T[i][r] dT'[i][r]
  for (int t = wave; t < NTRI; t += NW) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D; kk += 32) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gbeT + j * D + kk + 8 * lg);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gbeT + j * D + kk + 8 * lg + 4);
      mma(acc, frag<false>(dWr, LDD, 16 * i, kk), scale_frag(frag<false>(Kp, LDD, 16 * j, kk), g0, g1));
      mma(acc, frag<false>(dUr, LDD, 16 * i, kk), frag<false>(Vr, LDD, 16 * j, kk));
    }
    const int s = 16 * j + lr;
    float cs = 0.f;
    const f32x4 tv = lds_acc_tile(Tb, LDL, 16 * i, 16 * j);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) cs += tv[ii] * acc[ii];
    lds_store_acc_tile(dTb, LDL, 16 * i, 16 * j, acc * wL[s]);
    if (j < i) lds_zero_tile(dTb, LDL, 16 * j, 16 * i);   // mirrored tile: zero
    cs += __shfl_xor(cs, 16);
    cs += __shfl_xor(cs, 32);
    if (lg == 0) {
      dwp[i * LC + s] = cs;
      if (j < i) dwp[j * LC + 16 * i + lr] = 0.f;      // tiles above the diagonal contribute nothing
    }
  }
  // ---- dV = Tw^T dU = diag(w) T^T dU (write dv); dK+ (first part) = diag(w) T^T dW
  //   -> dk += Gamma dK+, dG += K+ dK+ (Gamma = e^(Gb + loc), K+ = K^+ e^Gb)
  {
    f32x4 acc[NB][CPW], acc2[NB][CPW];
    zero_acc(acc);
    zero_acc(acc2);
    owned_mma<T, NB, CPW, KL>(acc, LdsSrc<T, true>{Tb, LDL}, LdsSrc<T, true>{dUr, LDD}, ct0);
    owned_mma<T, NB, CPW, KL>(acc2, LdsSrc<T, true>{Tb, LDL}, LdsSrc<T, true>{dWr, LDD}, ct0);
    T* dv = reinterpret_cast<T*>(a.dv);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 kpv = lds_tile(Kp, rt, j);
        const float egb = fexp(gbs[rt][j]);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          const float wr = wL[r];
          if (r < n) dv[row0 * D + (unsigned)(r * D + 16 * (ct0 + j) + lr)] = to<T>(wr * acc[rt][j][ii]);
          const float x = egb * wr * acc2[rt][j][ii];
          dK[rt][j][ii] += fexp(loc[rt][j][ii]) * x;
          dG[rt][j][ii] += kpv[ii] * x;
        }
      }
  }
  __syncthreads();   // dT complete; dP no longer needed (its slot takes Z)

  // ---- Z = dT T^T (lower tiles)
  for (int t = wave; t < NTRI; t += NW) {
    int i, j;
    tri_index(t, i, j);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < LC; kk += 32) mma(acc, frag<false>(dTb, LDL, 16 * i, kk), frag<false>(Tb, LDL, 16 * j, kk));
    lds_store_acc_tile(Zb, LDL, 16 * i, 16 * j, acc);
  }
  __syncthreads();
  // b (or b_x) at the lane's gradient positions, for the erase gradient; loaded here so
  // that the loads are consumed before the chunk's gradient stores are issued
  float binv[CPW][NB][4];
  if (HAS_B) {
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          binv[j][rt][ii] = f.b[row0 * D + (unsigned)(min(16 * rt + 4 * lg + ii, n - 1) * D + 16 * (ct0 + j) + lr)];
  }
  // ---- dA = -T^T Z (strictly lower), dB = diag(w) dA; dw term sum_s B_rs dA_rs with B
  // (the coupling before the row scaling by w) from the prep pass
  {
    constexpr int MAXT = (NTRI + NW - 1) / NW;
    f32x4 dA[MAXT];
    const T* gB = reinterpret_cast<const T*>(f.f.Bt) + ci * LC * LC;
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int t = wave + NW * u;
      dA[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < NTRI) {
        int i, j;
        tri_index(t, i, j);
        const f32x4 bacc = load4f(gB + ((size_t)t * 64 + lane) * 4);
#pragma unroll
        for (int kk = 0; kk < LC; kk += 32) mma(dA[u], frag<true>(Tb, LDL, 16 * i, kk), frag<true>(Zb, LDL, 16 * j, kk));
        const int s = 16 * j + lr;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * i + 4 * lg + ii;
          const float da = (s < r) ? -dA[u][ii] : 0.f;
          dA[u][ii] = da;
          const float rs = row16_sum(bacc[ii] * da);
          if (lr == 0) dwq[j * LC + r] = rs;
        }
      }
    }
    __syncthreads();   // every read of Z is done
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
      const int t = wave + NW * u;
      if (t < NTRI) {
        int i, j;
        tri_index(t, i, j);
        f32x4 v;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v[ii] = wL[16 * i + 4 * lg + ii] * dA[u][ii];
        lds_store_acc_tile(dAb, LDL, 16 * i, 16 * j, v);
        if (i == j && unsafe[i]) store4(reinterpret_cast<T*>(a.diag) + (((ci * NB + i) * 2 + 1) * 64 + lane) * 4, v);
        if (j < i) {
          // mirrored tile above the diagonal: zero, and no row-sum contribution
          lds_zero_tile(dAb, LDL, 16 * j, 16 * i);
          if (lr == 0) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) dwq[i * LC + 16 * j + 4 * lg + ii] = 0.f;
          }
        }
      }
    }
  }
  __syncthreads();

  if (HAS_B) {
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          // the erase gradient from d log a: d/db = dlog a / b; with pre-activations
          // d/db_x = dlog a * sigmoid(-b_x); for b = sigmoid(x) given as b (db_mode 1)
          // d/dx = dlog a * (1 - b)
          const float bvv = binv[j][rt][ii];
          binv[j][rt][ii] = LG ? sigmoidf(-bvv) : (a.db_mode ? 1.f - bvv : rcp(bvv));
        }
  }
  // ---- the coupling's row and column roles: X1 = sum_J D_IJ (dB_IJ K^-_J) and
  // X3 = sum_I D_IJ (dB_IJ^T K^+_I)
  {
    f32x4 accp[NB][CPW], accm[NB][CPW];
    zero_acc(accp);
    zero_acc(accm);
    owned_mma_blk<T, NB, CPW, true>(
        accp, [&](int ob, int kb) { return lds_frag16_rows(dAb, LDL, 16 * ob, 16 * kb); },
        [&](int kb, int ct) { return lds_frag16_cols(Km, LDD, 16 * ct, 16 * kb); }, ct0, dfac);
    owned_mma_blk<T, NB, CPW, false>(
        accm, [&](int ob, int kb) { return lds_frag16_cols(dAb, LDL, 16 * ob, 16 * kb); },
        [&](int kb, int ct) { return lds_frag16_cols(Kp, LDD, 16 * ct, 16 * kb); }, ct0, dfac);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt) {
        const f32x4 kpv = lds_tile(Kp, rt, j), kmv = lds_tile(Km, rt, j);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float lo = loc[rt][j][ii];
          dK[rt][j][ii] += fexp(lo) * accp[rt][j][ii] + fexp(bto[rt][j] - lo) * accm[rt][j][ii];
          dG[rt][j][ii] += kpv[ii] * accp[rt][j][ii] - kmv[ii] * accm[rt][j][ii];
        }
      }
  }
  __syncthreads();   // glt, dwp, dwq complete

  // ---- dlog a = reverse cumulative sum of dG over the chunk's tokens + G_L term
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int col = 16 * (ct0 + j) + lr;
    float run = glt[col];
#pragma unroll
    for (int rt = NB - 1; rt >= 0; --rt) {
      float l4[4];
      l4[3] = dG[rt][j][3];
      l4[2] = l4[3] + dG[rt][j][2];
      l4[1] = l4[2] + dG[rt][j][1];
      l4[0] = l4[1] + dG[rt][j][0];
      float post = run, tile = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float tg = __shfl(l4[0], lr + 16 * g);
        if (g > lg) post += tg;
        tile += tg;
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) dG[rt][j][ii] = post + l4[ii];    // dlog a
      run += tile;
    }
  }
  // gradient stores; a full chunk stores without per-element token checks
  auto store_grads = [&](auto full) {
    T* dk = reinterpret_cast<T*>(a.dk);
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
      for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 16 * rt + 4 * lg + ii;
          if (decltype(full)::value || r < n) {
            const size_t idx = row0 * D + (unsigned)(r * D + 16 * (ct0 + j) + lr);
            a.dlog_g[idx] = dG[rt][j][ii];
            if (HAS_B) a.db[idx] = dG[rt][j][ii] * binv[j][rt][ii];
            dk[idx] = to<T>(dK[rt][j][ii]);
          }
        }
  };
  if (n == LC) store_grads(std::true_type{});
  else store_grads(std::false_type{});
  // ---- dw_r = sum_s B_rs dA_rs + sum_i T[i][r] dT'[i][r]
  if (tid < LC && tid < n) {
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < NB; ++t) s += dwq[t * LC + tid] + dwp[t * LC + tid];
    a.dw[row0 + tid] = LG ? s * wL[tid] * (1.f - wL[tid]) : s;     // d/dw_hat = d/dw * w (1 - w)
  }
  // ---- exact within-block terms of the blocks beyond the fast tiles' range, by this
  // workgroup once its gradient stores are done
  if (mask) {
    __syncthreads();
    diag_fix_chunk<T, LC, D, HAS_B, LG, NT>(a, bh, c, mask, reinterpret_cast<float*>(smem));
  }
}

template <typename T, int LC, int D, bool HAS_B, bool LG>
__global__ __launch_bounds__(D * 4) void bwd_chunk_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const size_t ci = (size_t)blockIdx.y * a.fwd.NC + a.c_lo + blockIdx.x;
  if (a.fwd.f.cflag[ci]) bwd_chunk_range<T, LC, D, HAS_B, LG>(a, smem);
  else bwd_chunk_fast<T, LC, D, HAS_B, LG>(a, smem);
  if (a.cg_on) {
    // the chunk's d/db_x stores are visible to the whole workgroup and every LDS read of
    // the gradient phases is done: the gate backward of the chunk's period follows
    __syncthreads();
    content_gate_body<T, D, D * 4>(a.cg, (int)blockIdx.y, reinterpret_cast<const T*>(a.cg_dO),
                                   reinterpret_cast<T*>(const_cast<void*>(a.dO)), reinterpret_cast<float*>(smem));
  }
}

size_t diag_fix_bytes(int dtype, int BH, int NC, int LC) {
  return ((size_t)BH * NC * (LC / 16) * 512 * (dtype ? 2 : 4) + 255) & ~size_t(255);
}

// ------------------------------------------------------------------ launchers
template <typename T, int LC, int D, int VS>
static hipError_t rev_affine_launch(const BwdArgs& a, hipStream_t st) {
  using Lay = RevLayout<T, LC, D, VS>;
  static_assert(Lay::bytes <= 80 * 1024, "reverse-state LDS exceeds half a compute unit's 160 KB");
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_state_kernel<T, LC, D, VS, true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
  if (e != hipSuccess) return e;
  dim3 grid((2 * D / VS) * a.fwd.B * a.fwd.H * (a.fwd.nseg - 1));
  hipLaunchKernelGGL((bwd_state_kernel<T, LC, D, VS, true>), grid, dim3(kThreads), Lay::bytes, st, a);
  return hipGetLastError();
}

template <typename T, int LC, int D, int VS>
static hipError_t rev_launch(const BwdArgs& a, hipStream_t st) {
  using Lay = RevLayout<T, LC, D, VS>;
  static_assert(Lay::bytes <= 80 * 1024, "reverse-state LDS exceeds half a compute unit's 160 KB");
  const FwdArgs& f = a.fwd;
  const int nseg = f.nseg > 1 ? f.nseg : 1;
  if (nseg > 1) {
    // every segment but the last holds seg_len whole chunks; the last is non-empty
    if (f.seg_len < 1 || (long long)(nseg - 1) * f.seg_len > f.NC - 1 || !a.raff || !a.dS_seg || a.c_count)
      return hipErrorInvalidValue;
    hipError_t e = f.aff_vs == 16 ? rev_affine_launch<T, LC, D, 16>(a, st) : rev_affine_launch<T, LC, D, 32>(a, st);
    if (e != hipSuccess) return e;
    e = launch_seg_scan(ScanArgs{a.dS_T, a.dS_seg, a.raff, nseg}, D, f.B * f.H, true, st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_state_kernel<T, LC, D, VS, false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
  if (e != hipSuccess) return e;
  dim3 grid((D / VS) * f.B * f.H * nseg);
  hipLaunchKernelGGL((bwd_state_kernel<T, LC, D, VS, false>), grid, dim3(kThreads), Lay::bytes, st, a);
  return hipGetLastError();
}

// The reverse pass takes at most 32 value rows per workgroup: with the staged factor
// blocks a 64-row slice would need more than half of a compute unit's LDS, so two of
// its workgroups could not share one (the forward pass's 64-row plans get twice as
// many 32-row workgroups here).
template <typename T, int LC, int D>
static hipError_t rev_launch_vs(const BwdArgs& a, hipStream_t st) {
  switch (a.fwd.VS) {
    case 16: return rev_launch<T, LC, D, 16>(a, st);
    case 32:
    case 64: return rev_launch<T, LC, D, 32>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int LC, int D>
static hipError_t grad_launch(const BwdArgs& a, hipStream_t st) {
  using Lay = GradLayout<T, LC, D>;
  static_assert(Lay::bytes <= 160 * 1024, "chunk-gradient LDS exceeds 160 KB");
  auto kern = a.fwd.logits ? (a.fwd.b ? bwd_chunk_kernel<T, LC, D, true, true> : bwd_chunk_kernel<T, LC, D, false, true>)
                           : (a.fwd.b ? bwd_chunk_kernel<T, LC, D, true, false> : bwd_chunk_kernel<T, LC, D, false, false>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
  if (e != hipSuccess) return e;
  dim3 grid(a.c_count ? a.c_count : a.fwd.NC, a.fwd.B * a.fwd.H);
  hipLaunchKernelGGL(kern, grid, dim3(D * 4), Lay::bytes, st, a);
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
