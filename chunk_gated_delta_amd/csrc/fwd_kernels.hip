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
#include <algorithm>

#include "carve_chunk.h"

namespace carve {

// threads of the chunk-prep kernel: one wave per 16 columns of the width
template <int D> constexpr int prep_threads() { return 4 * D; }

// Persistent over chunks: workgroup g prepares chunks g, g + G, g + 2G, ... (G = grid
// size, chunk index ci = bh * NC + c).  Once a chunk's raw inputs are staged in LDS
// the registers take the next chunk's loads, which land while this chunk computes:
// the gate pieces right away, k, q, v right after the chunk's triangular inverse (an
// out-of-line call, which starts by waiting for every outstanding load; issuing only
// part of the prefetch before it keeps that wait short and the live registers fewer).
template <typename T, int LC, int D, int MODE, typename Gates>
__device__ __forceinline__ void prep_loop(const FwdArgs& a, const Gates& gates, unsigned char* smem) {
  constexpr int NT = prep_threads<D>();
  const int total = a.B * a.H * a.NC;
  PrepStage<T, LC, D, NT> st;
  int ci = blockIdx.x;
  prep_stage_load<T, LC, D, Gates, NT>(a, gates, ci / a.NC, ci % a.NC, st);
  for (; ci < total; ci += gridDim.x) {
    const int bh = ci / a.NC, c = ci % a.NC;
    prep_stage_write<T, LC, D, Gates, NT>(a, gates, c, st, smem);
    __syncthreads();
    const int cn = min(ci + (int)gridDim.x, total - 1);      // clamped: the last pass reloads a valid chunk
    prep_stage_load<T, LC, D, Gates, NT, 1>(a, gates, cn / a.NC, cn % a.NC, st);
    prep_compute<T, LC, D, Gates, MODE, NT>(a, gates, bh, c, ci, smem, [&]() {
      prep_stage_load<T, LC, D, Gates, NT, 2>(a, gates, cn / a.NC, cn % a.NC, st);
    });
    __syncthreads();                                         // LDS is restaged by the next chunk
  }
}

template <typename T, int LC, int D, int MODE, bool LOGITS>
__global__ __launch_bounds__(4 * D) void fwd_prep_kernel(FwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  if constexpr (LOGITS) {
    if (a.b) prep_loop<T, LC, D, MODE>(a, LogitGates<D, true>{a.b, a.gA, a.gtau}, smem);
    else prep_loop<T, LC, D, MODE>(a, LogitGates<D, false>{nullptr, a.gA, a.gtau}, smem);
  } else {
    if (a.b) prep_loop<T, LC, D, MODE>(a, TokenGatesB{a.b}, smem);
    else prep_loop<T, LC, D, MODE>(a, TokenGates1{}, smem);
  }
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
  // Sb [VS][LDS_] dtype state, UT [VS][LDU] U^T, OT [VS][LDU] O^T, colsum [NB][VS]
  static constexpr size_t bytes = sizeof(T) * (VS * LDS_ + 2 * VS * LDU) + sizeof(float) * NB * VS;
};


template <typename T> struct Raw4;
template <> struct Raw4<bf16> { bf16x4 v; };
template <> struct Raw4<float> { f32x4 v; };
__device__ __forceinline__ Raw4<bf16> load_raw4(const bf16* p) { return Raw4<bf16>{*reinterpret_cast<const bf16x4*>(p)}; }
__device__ __forceinline__ Raw4<float> load_raw4(const float* p) { return Raw4<float>{*reinterpret_cast<const f32x4*>(p)}; }
__device__ __forceinline__ f32x4 widen(const Raw4<bf16>& r) {
  return f32x4{(float)r.v[0], (float)r.v[1], (float)r.v[2], (float)r.v[3]};
}
__device__ __forceinline__ f32x4 widen(const Raw4<float>& r) { return r.v; }

// The global operands one wave needs for one chunk.  Wave w (of NW) owns the U/O
// tiles tix = w*UPW + u (all in one row tile of the chunk) and the state tiles
// st = w*SPW + j (key tile st / NVT, value tile st % NVT).
template <typename T, int LC, int D, int VS, bool HAS_O, int NW = kWaves>
struct ChunkOps {
  using ST = StateTiles<D, VS, NW>;
  static constexpr int NVT = VS / 16, NB = LC / 16, NCT = D / 16;
  static constexpr int NUO = NB * NVT;
  static constexpr int UPW = (NUO + NW - 1) / NW;
  static constexpr int SCT = ST::SCT;
  static constexpr int KD = D / 32, KL = LC / 32;
  static_assert(NVT % UPW == 0, "a wave's U/O tiles must share one row tile");
  static constexpr bool kAllWaves = UPW * (NW - 1) < NUO;   // every wave owns U/O tiles
  Frag<T> w[KD];
  Frag<T> q[HAS_O ? KD : 1];
  Raw4<T> ub[UPW];
  Raw4<T> oi[HAS_O ? UPW : 1];
  Frag<T> kf[SCT][KL];
  f32x4 gl[SCT];

  // no_ub: the slice has no write term (Ubar = 0; the Pi rows of an affine map)
  __device__ __forceinline__ void load(const FwdArgs& a, size_t ci, int v0, bool no_ub = false) {
    const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
    const T* Wn = reinterpret_cast<const T*>(a.f.Wn);
    const T* Qt = reinterpret_cast<const T*>(a.f.Qt);
    const T* KfT = reinterpret_cast<const T*>(a.f.KfT);
    const T* UbT = reinterpret_cast<const T*>(a.f.UbT);
    const T* OiT = reinterpret_cast<const T*>(a.f.OiT);
    const int t0 = wave * UPW;
    if (kAllWaves || t0 < NUO) {
      const int rt = t0 / NVT;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        w[kk] = load_frag(Wn + ci * LC * D + frag_offset<D>(rt, kk, lane));
        if (HAS_O) q[kk] = load_frag(Qt + ci * LC * D + frag_offset<D>(rt, kk, lane));
      }
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        const int vt = (t0 + u) % NVT;
        if (no_ub) ub[u] = Raw4<T>{};
        else ub[u] = load_raw4(UbT + ci * LC * D + acc_offset<D>(rt, v0 / 16 + vt, lane));
        if (HAS_O) oi[u] = load_raw4(OiT + ci * LC * D + acc_offset<D>(rt, v0 / 16 + vt, lane));
      }
    }
#pragma unroll
    for (int j = 0; j < SCT; ++j) {
      const int ct = (wave * ST::SPW) / NVT + j;
      gl[j] = load4f(a.f.gL + ci * D + 16 * ct + 4 * lg);
#pragma unroll
      for (int kk = 0; kk < KL; ++kk) kf[j][kk] = load_frag(KfT + ci * D * LC + frag_offset<LC>(ct, kk, lane));
    }
  }
};

// Load the state slice (rows v0 .. v0+VS-1 of the D x D matrix init, or zero when
// init is null) into registers and its dtype copy into LDS.
template <typename T, int D, int VS, int NW = kWaves>
__device__ __forceinline__ void state_init_from(const float* init, int v0, f32x4 (&S)[StateTiles<D, VS, NW>::SPW], T* Sb) {
  using ST = StateTiles<D, VS, NW>;
  constexpr int LDS_ = D + Pad<T>::v;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int j = 0; j < ST::SPW; ++j) {
    const int st = wave * ST::SPW + j, ct = st / ST::NVT, vt = st % ST::NVT;
    const int vl = 16 * vt + lr, kc = 16 * ct + 4 * lg;
    if (init) S[j] = load4f(init + (size_t)(v0 + vl) * D + kc);
    else S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    store4(Sb + vl * LDS_ + kc, S[j]);
  }
}

// The state slice from S0 (or zero).
template <typename T, int D, int VS, int NW = kWaves>
__device__ __forceinline__ void state_init(const FwdArgs& a, int bh, int v0, f32x4 (&S)[StateTiles<D, VS, NW>::SPW], T* Sb) {
  state_init_from<T, D, VS, NW>(a.S0 ? a.S0 + (size_t)bh * D * D : nullptr, v0, S, Sb);
}

// One chunk of the state recurrence for a slice of VS value rows:
//   U = Ubar + (-W) S^T,  O = (P Ubar) + Q~ S^T  (written when HAS_O),
//   S^T <- Diag(Gamma_L) S^T + K->^T U.
// Operands come from `op` (this chunk's factors).  On entry Sb holds the dtype
// copy of S; on exit S and Sb hold the updated state.  If colsum is given, the
// per-row-tile column sums of the fp32 outputs (valid tokens only) are written
// to colsum[NB][VS].
template <typename T, int LC, int D, int VS, bool HAS_O, bool FULL = false, int NW = kWaves>
__device__ __forceinline__ void state_chunk(const FwdArgs& a, int bh, int c, int v0, const ChunkOps<T, LC, D, VS, HAS_O, NW>& op,
                            f32x4 (&S)[StateTiles<D, VS, NW>::SPW], unsigned char* smem, float* colsum) {
  using Lay = StateLayout<T, LC, D, VS>;
  using Op = ChunkOps<T, LC, D, VS, HAS_O, NW>;
  using ST = StateTiles<D, VS, NW>;
  constexpr int NVT = ST::NVT, SPW = ST::SPW, UPW = Op::UPW, NUO = Op::NUO;
  constexpr int LDS_ = Lay::LDS_, LDU = Lay::LDU;
  T* Sb = reinterpret_cast<T*>(smem);
  T* UT = Sb + VS * LDS_;
  T* OT = UT + VS * LDU;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
  T* o = reinterpret_cast<T*>(a.o);
  constexpr bool WIDE = kWideSlice<VS>;

  const int t0 = wave * UPW;
  if (Op::kAllWaves || t0 < NUO) {
    const int rt = t0 / NVT;
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int vt = (t0 + u) % NVT;
      const int r = 16 * rt + 4 * lg, vl = 16 * vt + lr, vg = v0 + vl;
      f32x4 accU = widen(op.ub[u]);
      f32x4 accO = HAS_O ? widen(op.oi[u]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < Op::KD; ++kk) {
        const Frag<T> fs = load_frag(Sb + vl * LDS_ + 32 * kk + 8 * lg);
        mma(accU, op.w[kk], fs);
        if (HAS_O) mma(accO, op.q[kk], fs);
      }
      if (HAS_O) {
        float csum = 0.f;
        if (WIDE) store4(OT + vl * LDU + r, accO);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int t = c * LC + r + ii;
          if (FULL || t < a.T) {          // FULL: every token of the chunk exists
            if (!WIDE) o[((size_t)bh * a.T + t) * D + vg] = to<T>(accO[ii]);
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
  if (HAS_O && WIDE) {
    // O^T fragments: lane (lr, lg) gets 8 consecutive value rows of token 16 tt + lr
    for_wave_items<(LC / 16) * (VS / 32), NW>(wave, [&](int f) {
      const int tt = f / (VS / 32), vb = f % (VS / 32);
      const Frag<T> x = lds_frag_cols(OT, LDU, 16 * tt, 32 * vb);
      const int t = c * LC + 16 * tt + lr;
      if (FULL || t < a.T)
        *reinterpret_cast<Frag<T>*>(o + ((size_t)bh * a.T + t) * D + v0 + 32 * vb + 8 * lg) = x;
    });
  }
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int st = wave * SPW + j, jc = ST::jc(j), ct = st / NVT, vt = st % NVT;
    const int kc = 16 * ct + 4 * lg, vl = 16 * vt + lr;
    S[j] *= op.gl[jc];
#pragma unroll
    for (int kk = 0; kk < Op::KL; ++kk) {
      const Frag<T> fu = load_frag(UT + vl * LDU + 32 * kk + 8 * lg);
      mma(S[j], op.kf[jc][kk], fu);
    }
    store4(Sb + vl * LDS_ + kc, S[j]);
  }
  __syncthreads();
}

template <typename T, int D, int VS, int NW = kWaves>
__device__ __forceinline__ void state_store(const FwdArgs& a, int bh, int v0, const f32x4 (&S)[StateTiles<D, VS, NW>::SPW], float* dst) {
  using ST = StateTiles<D, VS, NW>;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int j = 0; j < ST::SPW; ++j) {
    const int st = wave * ST::SPW + j, ct = st / ST::NVT, vt = st % ST::NVT;
    store4(dst + ((size_t)bh * D + v0 + 16 * vt + lr) * D + 16 * ct + 4 * lg, S[j]);
  }
}

// Store the state entering chunk ci in the fragment order of the backward ("vk":
// 8 consecutive k of one row v per lane).  Wide slices copy whole fragments out of
// the dtype copy Sb (rows v0.., in LDS) with one 16-byte store per lane; narrow
// slices scatter the registers' accumulator groups.
template <typename T, int D, int VS>
__device__ __forceinline__ void save_state(const FwdArgs& a, size_t ci, int v0, const f32x4 (&S)[StateTiles<D, VS>::SPW],
                                           const T* Sb) {
  using ST = StateTiles<D, VS>;
  T* vk = reinterpret_cast<T*>(a.S_vk) + ci * D * D;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
  if constexpr (kWideSlice<VS>) {
    constexpr int LDS_ = D + Pad<T>::v;
    for_wave_items<(VS / 16) * (D / 32), kWaves>(wave, [&](int f) {
      const int vt = f / (D / 32), kb = f % (D / 32);
      const Frag<T> x = load_frag(Sb + (16 * vt + lr) * LDS_ + 32 * kb + 8 * lg);
      *reinterpret_cast<Frag<T>*>(vk + frag_offset<D>(v0 / 16 + vt, kb, lane)) = x;
    });
  } else {
#pragma unroll
    for (int jj = 0; jj < ST::SPW; ++jj) {
      const int st = wave * ST::SPW + jj, ct = st / ST::NVT, vt = st % ST::NVT;
      store_vk_group<T, D>(vk, v0 / 16 + vt, ct, S[jj]);
    }
  }
}

// The chunk loop keeps three operand buffers: chunk c is consumed from buffer c % 3,
// which then takes the loads of chunk c + 3, so every chunk's factors are in flight
// for two whole chunk steps and a step never waits on loads issued in the same step.
// Full chunks run in a branch-free main loop (prefetch indices are clamped, no token
// checks); the last chunks run in a checked tail.  With a segmented pass (nseg > 1)
// the workgroup runs the chunks of one segment from that segment's entering state.
template <typename T, int LC, int D, int VS, bool HAS_O, bool SAVE>
__global__ __launch_bounds__(kThreads) void fwd_state_kernel(FwdArgs a) {
  using ST = StateTiles<D, VS>;
  using Op = ChunkOps<T, LC, D, VS, HAS_O>;
  constexpr int PF = 3;
  extern __shared__ __align__(16) unsigned char smem[];
  const int nseg = a.nseg > 1 ? a.nseg : 1;
  int u, slice;
  xcd_slice_map(D / VS, a.B * a.H * nseg, u, slice);
  const int bh = u / nseg, seg = u % nseg;
  const int v0 = slice * VS;
  const int cs = nseg > 1 ? seg * a.seg_len : 0;
  const int ce = nseg > 1 ? min(a.NC, cs + a.seg_len) : a.NC;
  const size_t c0i = (size_t)bh * a.NC;
  const float* init = nseg > 1 ? a.S_seg + (size_t)u * D * D : (a.S0 ? a.S0 + (size_t)bh * D * D : nullptr);
  f32x4 S[ST::SPW];
  Op buf[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) buf[j].load(a, c0i + min(cs + j, ce - 1), v0);
  state_init_from<T, D, VS>(init, v0, S, reinterpret_cast<T*>(smem));
  __syncthreads();
  const int nfull = min(ce, (a.T % LC == 0) ? a.NC : a.NC - 1) - cs;   // full chunks of the range
  const int nmain = nfull - nfull % PF;
  for (int l0 = 0; l0 < nmain; l0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int c = cs + l0 + j;
      if (SAVE) save_state<T, D, VS>(a, c0i + c, v0, S, reinterpret_cast<const T*>(smem));
      state_chunk<T, LC, D, VS, HAS_O, true>(a, bh, c, v0, buf[j], S, smem, nullptr);
      buf[j].load(a, c0i + min(c + PF, ce - 1), v0);
    }
  }
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int c = cs + nmain + j;
    if (c < ce) {
      if (SAVE) save_state<T, D, VS>(a, c0i + c, v0, S, reinterpret_cast<const T*>(smem));
      state_chunk<T, LC, D, VS, HAS_O, false>(a, bh, c, v0, buf[j], S, smem, nullptr);
    }
  }
  if (a.S_T && seg == nseg - 1) state_store<T, D, VS>(a, bh, v0, S, a.S_T);
}

// ------------------------------------------------------------------ segmented state pass
// For long sequences with few heads the chunk chain of a head is cut into segments.
// The state step is affine in S, so a segment maps its entering state to
// S_out = S_in Pi + C: C is the pass over the segment from S_in = 0, and Pi, the
// product of the chunk maps M_c = Diag(Gamma_L) - W^T K->, is the same pass with no
// write term (Ubar = 0) started from the identity (its rows are indexed by key).
// fwd_affine runs both at once as 2D state rows [C; Pi] per (head, segment) for every
// segment but the last; seg_scan chains the maps (S_in(s+1) = S_in(s) Pi_s + C_s,
// fp32); the state pass then runs every segment from its S_in, writing o.  This is
// the chunk-level scan of the affine state maps behind the logarithmic parallel depth
// the notes list for CARVE (complexity table), taken as two levels.
template <typename T, int LC, int D, int VS>
__global__ __launch_bounds__(kThreads) void fwd_affine_kernel(FwdArgs a) {
  using ST = StateTiles<D, VS>;
  using Op = ChunkOps<T, LC, D, VS, false>;
  constexpr int PF = 3, LDS_ = D + Pad<T>::v;
  extern __shared__ __align__(16) unsigned char smem[];
  const int nsa = a.nseg - 1;                  // segments with a map: all but the last
  int u, slice;
  xcd_slice_map(2 * D / VS, a.B * a.H * nsa, u, slice);
  const int bh = u / nsa, seg = u % nsa;
  const int r0 = slice * VS;                   // first row of [C; Pi]
  const bool pi = r0 >= D;
  const int v0 = pi ? 0 : r0;                  // value rows of C (Pi rows load no Ubar)
  const int cs = seg * a.seg_len, ce = cs + a.seg_len;   // whole chunks (only the last segment is ragged)
  const size_t c0i = (size_t)bh * a.NC;
  const int lane = lane_id(), wave = wave_id(), lr = lane & 15, lg = lane >> 4;
  f32x4 S[ST::SPW];
  Op buf[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) buf[j].load(a, c0i + min(cs + j, ce - 1), v0, pi);
  T* Sb = reinterpret_cast<T*>(smem);
#pragma unroll
  for (int j = 0; j < ST::SPW; ++j) {
    const int st = wave * ST::SPW + j, ct = st / ST::NVT, vt = st % ST::NVT;
    const int row = r0 - D + 16 * vt + lr, kc = 16 * ct + 4 * lg;   // Pi row index (key) when pi
#pragma unroll
    for (int i = 0; i < 4; ++i) S[j][i] = (pi && kc + i == row) ? 1.f : 0.f;
    store4(Sb + (16 * vt + lr) * LDS_ + kc, S[j]);
  }
  __syncthreads();
  const int n = ce - cs, nmain = n - n % PF;
  for (int l0 = 0; l0 < nmain; l0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int c = cs + l0 + j;
      state_chunk<T, LC, D, VS, false, true>(a, bh, c, v0, buf[j], S, smem, nullptr);
      buf[j].load(a, c0i + min(c + PF, ce - 1), v0, pi);
    }
  }
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int c = cs + nmain + j;
    if (c < ce) state_chunk<T, LC, D, VS, false, true>(a, bh, c, v0, buf[j], S, smem, nullptr);
  }
  float* dst = a.aff + ((size_t)(bh * a.nseg + seg) * 2 * D + r0) * D;
#pragma unroll
  for (int j = 0; j < ST::SPW; ++j) {
    const int st = wave * ST::SPW + j, ct = st / ST::NVT, vt = st % ST::NVT;
    store4(dst + (size_t)(16 * vt + lr) * D + 16 * ct + 4 * lg, S[j]);
  }
}

// Forward: S_in(0) = S0 (or 0), S_in(s+1) = S_in(s) Pi_s + C_s for s = 0 .. nseg-2.
// Reverse (REV): the gradient w.r.t. the state leaving segment nseg-1 is dS_T (or 0), and
// dS_out(s-1) = dS_out(s) Pi_s + C_s for s = nseg-1 .. 1.  Both in fp32 with a fixed
// summation order.  Workgroup (16 rows, head): its rows depend only on themselves, so they
// stay in LDS across the segments (transposed, [key][row]).  Pi_s is staged whole in
// LDS; the next map's Pi and C rows are loaded into registers while the current product
// runs.  Wave q owns rows 4q .. 4q+3, lane l the columns CW l .. CW l + CW - 1 (CW = D / 64).
template <int D>
struct ScanLayout {
  static constexpr size_t bytes = sizeof(float) * (D * D + D * 16);
};

template <int D, bool REV>
__global__ __launch_bounds__(256) void seg_scan_kernel(ScanArgs a) {
  constexpr int CW = D / 64, NL = D * D / 4 / 256;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Pi = reinterpret_cast<float*>(smem);
  float* SrT = Pi + D * D;
  const int bh = blockIdx.y, r0 = 16 * blockIdx.x;
  const int tid = threadIdx.x, rq = tid / 64, c0 = CW * (tid % 64);
  // step k (k = 0 .. nseg-2) reads the rows of segment slot(k) and map slot(k) and
  // writes slot(k + 1)
  auto slot = [&](int k) { return REV ? a.nseg - 1 - k : k; };
  float acc[4][CW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + 4 * rq + i;
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const float x = a.init ? a.init[((size_t)bh * D + row) * D + c0 + c] : 0.f;
      acc[i][c] = x;
      a.seg[(((size_t)bh * a.nseg + slot(0)) * D + row) * D + c0 + c] = x;
      SrT[(c0 + c) * 16 + 4 * rq + i] = x;
    }
  }
  f32x4 pre[NL];
  float cpre[4][CW];
  auto fetch = [&](int k) {
    const float* map = a.aff + (size_t)(bh * a.nseg + slot(k)) * 2 * D * D;
#pragma unroll
    for (int l = 0; l < NL; ++l) pre[l] = load4f(map + (size_t)D * D + 4 * (tid + 256 * l));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < CW; ++c) cpre[i][c] = map[(size_t)(r0 + 4 * rq + i) * D + c0 + c];
  };
  if (a.nseg > 1) fetch(0);
  for (int k = 0; k + 1 < a.nseg; ++k) {
    // every read of the previous Pi and SrT finished before the barrier that ended the last step
#pragma unroll
    for (int l = 0; l < NL; ++l) store4(Pi + 4 * (tid + 256 * l), pre[l]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < CW; ++c) acc[i][c] = cpre[i][c];
    __syncthreads();
    if (k + 2 < a.nseg) fetch(k + 1);
#pragma unroll 4
    for (int j = 0; j < D; ++j) {
      const f32x4 sv = load4f(SrT + j * 16 + 4 * rq);
      float pv[CW];
      if constexpr (CW == 2) {
        const float2 p2 = *reinterpret_cast<const float2*>(Pi + j * D + c0);
        pv[0] = p2.x;
        pv[1] = p2.y;
      } else {
        pv[0] = Pi[j * D + c0];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[i][c] = fmaf(sv[i], pv[c], acc[i][c]);
    }
    __syncthreads();                            // every read of Pi_s and SrT(s) done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 4 * rq + i;
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        a.seg[(((size_t)bh * a.nseg + slot(k + 1)) * D + row) * D + c0 + c] = acc[i][c];
        SrT[(c0 + c) * 16 + 4 * rq + i] = acc[i][c];
      }
    }
  }
}

template <int D, bool REV>
static hipError_t scan_launch(const ScanArgs& a, int BH, hipStream_t st) {
  auto scan = seg_scan_kernel<D, REV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(scan), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)ScanLayout<D>::bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan, dim3(D / 16, BH), dim3(256), ScanLayout<D>::bytes, st, a);
  return hipGetLastError();
}

hipError_t launch_seg_scan(const ScanArgs& a, int D, int BH, bool rev, hipStream_t st) {
  if (a.nseg < 2 || !a.aff || !a.seg) return hipErrorInvalidValue;
  if (D == 128) return rev ? scan_launch<128, true>(a, BH, st) : scan_launch<128, false>(a, BH, st);
  if (D == 64) return rev ? scan_launch<64, true>(a, BH, st) : scan_launch<64, false>(a, BH, st);
  return hipErrorInvalidValue;
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
// eight waves per workgroup: the per-chunk work of one head is spread over the CU
constexpr int kContentWaves = 8;

template <typename T, int LC, int D>
struct ContentLayout {
  static constexpr size_t prep = PrepLayout<T, LC, D, 64 * kContentWaves>::bytes;
  static constexpr size_t step = StateLayout<T, LC, D, D>::bytes;
  static constexpr size_t body = (prep > step ? prep : step);
  static constexpr size_t bytes = body + sizeof(float) * (4 * D + 64);   // z, msum, m, r
};

template <typename T, int LC, int D>
__global__ __launch_bounds__(64 * kContentWaves) void fwd_content_kernel(FwdArgs a, ContentArgs cg) {
  constexpr int NW = kContentWaves, NT = 64 * NW;
  using Lay = ContentLayout<T, LC, D>;
  using ST = StateTiles<D, D, NW>;
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
  // the raw inputs of the next chunk are loaded (into registers) as soon as a chunk's state
  // step is done, so they arrive while the period's mean and signal are formed
  const ContentGates gates{cg.b_x, zL};
  PrepStage<T, LC, D, NT> st;
  prep_stage_load<T, LC, D, ContentGates, NT>(a, gates, bh, 0, st);
  int count = 0;
  for (int c = 0; c < a.NC; ++c) {
    if (c % per == 0) {
      // content signal of this period from the previous period's mean output, with every
      // thread: r = U1 m (each row of U1 over 32 lanes), then z = U2 r (each row over 4 lanes)
      if (cg.U1) {
        for (int j0 = 0; j0 < cg.R; j0 += NT / 32) {
          const int j = j0 + tid / 32, part = tid % 32;
          float acc = 0.f;
          if (j < cg.R) {
            const float* u1 = cg.U1 + ((size_t)h * cg.R + j) * D;
#pragma unroll
            for (int vv = part; vv < D; vv += 32) acc += u1[vv] * mL[vv];
          }
#pragma unroll
          for (int o = 16; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
          if (j < cg.R && part == 0) rL[j] = acc;
        }
        __syncthreads();
        static_assert(NT >= 4 * D, "four lanes per key channel for z = U2 r");
        {
          const int kk = tid / 4, part = tid % 4;
          float acc = 0.f;
          if (kk < D) {
            const float* u2 = cg.U2 + ((size_t)h * D + kk) * cg.R;
            for (int j = part; j < cg.R; j += 4) acc += u2[j] * rL[j];
          }
          acc += __shfl_xor(acc, 2);
          acc += __shfl_xor(acc, 1);
          if (kk < D && part == 0) zL[kk] = acc;
        }
      } else if (tid < D) {
        zL[tid] = 0.f;
      }
      __syncthreads();   // z is written by other threads than the ones recording it
      if (tid < D) {
        msum[tid] = 0.f;
        if (cg.z_all) {
          // per-period record for the backward: z and the mean it was formed from
          const size_t pi = (size_t)bh * ((a.NC + per - 1) / per) + c / per;
          cg.z_all[pi * D + tid] = zL[tid];
          cg.m_all[pi * D + tid] = mL[tid];
        }
      }
      count = 0;
      __syncthreads();
    }
    // prepare this chunk's factors into the head's slot (its raw inputs are in registers)
    prep_stage_write<T, LC, D, ContentGates, NT>(a, gates, c, st, smem);
    __syncthreads();
    prep_compute<T, LC, D, ContentGates, kPrepFwd, NT>(a, gates, bh, c, (size_t)bh, smem);
    __syncthreads();
    // the chunk's factors (just written by this workgroup) are loaded before the state's
    // LDS copy is rebuilt, so that their round trip overlaps it
    ChunkOps<T, LC, D, D, true, NW> op;
    op.load(a, (size_t)bh, 0);
    if (c == 0) {
      state_init<T, D, D, NW>(a, bh, 0, S, reinterpret_cast<T*>(smem));
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
    state_chunk<T, LC, D, D, true, false, NW>(a, bh, c, 0, op, S, smem, cs);
    prep_stage_load<T, LC, D, ContentGates, NT>(a, gates, bh, min(c + 1, a.NC - 1), st);   // (the last reloads itself)
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
  if (a.S_T) state_store<T, D, D, NW>(a, bh, 0, S, a.S_T);
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
// Workgroups of a persistent launch: one per compute unit of the current device
// (the prep's LDS footprint allows one resident workgroup per unit).
static int persistent_blocks() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static size_t factor_block(int dtype, int BH, int NC, int LC, int D) {  // one [chunk][LC][D] block
  const size_t es = dtype ? 2 : 4;
  return ((size_t)BH * NC * LC * D * es + 255) & ~size_t(255);
}

// Factor blocks in the workspace: -W, K->^T, Ubar^T, Q~ always; P Ubar with the
// forward mode; then Gamma_L, and with the backward mode the inverse T, the intra-chunk
// weights P and the coupling B of every chunk (LC x LC each, dtype; P and B written for
// range-safe chunks only) and the chunks' path flags.
static int factor_blocks(int mode) { return 4 + ((mode & 1) ? 1 : 0); }
static size_t gl_block(int BH, int NC, int D) { return ((size_t)BH * NC * D * sizeof(float) + 255) & ~size_t(255); }

static size_t tile_block(int dtype, int BH, int NC, int LC) {   // one [chunk][LC][LC] block
  return ((size_t)BH * NC * LC * LC * (dtype ? 2 : 4) + 255) & ~size_t(255);
}

static size_t flag_block(int BH, int NC) { return ((size_t)BH * NC * sizeof(int) + 255) & ~size_t(255); }

size_t factors_bytes(int dtype, int BH, int NC, int LC, int D, int mode) {
  return factor_blocks(mode) * factor_block(dtype, BH, NC, LC, D) + gl_block(BH, NC, D) +
         ((mode & 2) ? 3 * tile_block(dtype, BH, NC, LC) + flag_block(BH, NC) : 0);
}

ChunkFactors carve_factors(void* ws, int dtype, int BH, int NC, int LC, int D, int mode) {
  const size_t blk = factor_block(dtype, BH, NC, LC, D);
  char* p = static_cast<char*>(ws);
  ChunkFactors f;
  int i = 0;
  f.Wn = p + blk * i++;
  f.KfT = p + blk * i++;
  f.UbT = p + blk * i++;
  f.Qt = p + blk * i++;
  f.OiT = (mode & 1) ? p + blk * i++ : nullptr;
  f.gL = reinterpret_cast<float*>(p + blk * i);
  char* tiles = p + blk * i + gl_block(BH, NC, D);
  const size_t tb = tile_block(dtype, BH, NC, LC);
  f.Tt = (mode & 2) ? tiles : nullptr;
  f.Pt = (mode & 2) ? tiles + tb : nullptr;
  f.Bt = (mode & 2) ? tiles + 2 * tb : nullptr;
  f.cflag = (mode & 2) ? reinterpret_cast<int*>(tiles + 3 * tb) : nullptr;
  return f;
}

template <typename T, int LC, int D>
static hipError_t prep_launch(const FwdArgs& a, hipStream_t st) {
  using Lay = PrepLayout<T, LC, D, prep_threads<D>()>;
  static_assert(Lay::bytes <= 160 * 1024, "prep LDS exceeds 160 KB");
  auto kern = a.logits ? (a.mode == 3 ? fwd_prep_kernel<T, LC, D, 3, true>
                                      : (a.mode == 2 ? fwd_prep_kernel<T, LC, D, 2, true> : fwd_prep_kernel<T, LC, D, 1, true>))
                       : (a.mode == 3 ? fwd_prep_kernel<T, LC, D, 3, false>
                                      : (a.mode == 2 ? fwd_prep_kernel<T, LC, D, 2, false> : fwd_prep_kernel<T, LC, D, 1, false>));
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::bytes);
  if (e != hipSuccess) return e;
  const int total = a.NC * a.B * a.H;
  hipLaunchKernelGGL(kern, dim3(std::min(total, persistent_blocks())), dim3(prep_threads<D>()), Lay::bytes, st, a);
  return hipGetLastError();
}

template <typename T, int LC, int D, int VS>
static hipError_t affine_launch(const FwdArgs& a, hipStream_t st) {
  using Lay = StateLayout<T, LC, D, VS>;
  static_assert(Lay::bytes <= 64 * 1024, "state LDS exceeds 64 KB");
  hipLaunchKernelGGL((fwd_affine_kernel<T, LC, D, VS>), dim3((2 * D / VS) * a.B * a.H * (a.nseg - 1)),
                     dim3(kThreads), Lay::bytes, st, a);
  return hipGetLastError();
}

template <typename T, int LC, int D, int VS>
static hipError_t state_launch(const FwdArgs& a, hipStream_t st) {
  using Lay = StateLayout<T, LC, D, VS>;
  static_assert(Lay::bytes <= 64 * 1024, "state LDS exceeds 64 KB");
  const int nseg = a.nseg > 1 ? a.nseg : 1;
  if (nseg > 1) {
    // every segment but the last holds seg_len whole chunks; the last is non-empty
    if (a.seg_len < 1 || (long long)(nseg - 1) * a.seg_len > a.NC - 1 || !a.aff || !a.S_seg)
      return hipErrorInvalidValue;
    hipError_t e = hipSuccess;
    switch (a.aff_vs) {
      case 16: e = affine_launch<T, LC, D, 16>(a, st); break;
      case 32: e = affine_launch<T, LC, D, 32>(a, st); break;
      case 64: e = affine_launch<T, LC, D, 64>(a, st); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    e = launch_seg_scan(ScanArgs{a.S0, a.S_seg, a.aff, nseg}, D, a.B * a.H, false, st);
    if (e != hipSuccess) return e;
  }
  dim3 grid((D / VS) * a.B * a.H * nseg);
  if (a.o && a.S_vk) hipLaunchKernelGGL((fwd_state_kernel<T, LC, D, VS, true, true>), grid, dim3(kThreads), Lay::bytes, st, a);
  else if (a.o) hipLaunchKernelGGL((fwd_state_kernel<T, LC, D, VS, true, false>), grid, dim3(kThreads), Lay::bytes, st, a);
  else if (a.S_vk) hipLaunchKernelGGL((fwd_state_kernel<T, LC, D, VS, false, true>), grid, dim3(kThreads), Lay::bytes, st, a);
  else hipLaunchKernelGGL((fwd_state_kernel<T, LC, D, VS, false, false>), grid, dim3(kThreads), Lay::bytes, st, a);
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
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(64 * kContentWaves), Lay::bytes, st, a, cg);
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
