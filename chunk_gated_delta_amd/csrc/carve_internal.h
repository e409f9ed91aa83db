// Internal launch interface between the C ABI (carve_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace carve {

// Per-chunk factors produced by the chunk-parallel prep kernel and consumed by
// the sequential state kernels.  Chunk index ci = (b*H + h) * NC + c; every block
// holds LC*D elements per chunk, in the order the state kernels load them
// ("frag <C>": MFMA fragment order with contraction length C, frag_offset;
// "acc": accumulator order, acc_offset):
//   Wn  -W [LC][D], frag<D>     with W = T diag(w) (K .* Gamma)       (dtype)
//   Qt  Q~ [LC][D], frag<D>     Q~ = (Q .* Gamma) - P W               (dtype)
//   KfT K->^T [D][LC], frag<LC> K-> = K .* Gamma_L / Gamma            (dtype)
//   UbT Ubar [LC][D], acc       Ubar = T diag(w) V                    (dtype)
//   OiT P Ubar [LC][D], acc     the intra-chunk output                (dtype)
//   gL  [ci][D]                 Gamma_L, the chunk's total retention  (float)
// where Gamma is the inclusive cumulative product of a inside the chunk,
// T = (I + A)^-1, A = strict_tril(diag(w) (K.*Gamma)(K./Gamma)^T) and
// P = tril((Q.*Gamma)(K./Gamma)^T).
// The reverse state pass reads Wn, Qt and KfT too (transposed on chip); the backward
// modes also write
//   Tt  [ci][LC][LC] row-major, T = (I + A)^-1 (dtype)
//   cflag [ci] the chunk's path (1: range-safe, whose log-retention over the chunk
//       fell below the fast path's range in some key channel), and for those chunks
//   Pt  [ci][LC][LC] row-major, P (dtype)
//   Bt  [ci][NTRI][64][4], B = A before the row scaling by w (strictly lower
//       coupling), the lower 16x16 tiles (tri index) in accumulator order (dtype)
// Prep modes: 1 = forward only, 2 = backward only (no OiT), 3 = both.
struct ChunkFactors {
  void* Wn;
  void* Qt;
  void* KfT;
  void* UbT;
  void* OiT;
  float* gL;
  void* Tt;               // [ci][LC][LC] T = (I + A)^-1 in the operand type (backward modes)
  void* Pt;               // [ci][LC][LC] P (backward modes, range-safe chunks)
  void* Bt;               // [ci][LC*LC] B tiles in accumulator order (backward modes, range-safe chunks)
  int* cflag;             // [ci] 1 = the chunk took the range-safe path (backward modes)
};

struct FwdArgs {
  int B, H, T, D, LC, NC, VS;
  int mode;               // prep mode: 1 forward, 2 backward, 3 both
  int dtype;              // 0 f32, 1 bf16
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const float* b;         // may be null (= 1)
  const float* w;
  const float* S0;        // may be null
  void* o;                // may be null (state-only pass)
  float* S_T;             // may be null
  void* S_vk;             // may be null: state entering every chunk, [ci][D*D] dtype, fragment order rows v
  ChunkFactors f;
  // gates as pre-activations (logits != 0): log_g then holds the decay logits f, b the
  // erase pre-activation b_x (or null), w the write pre-activation w_hat, and
  // log g = -gA softplus(f + gtau) (gA, gtau [H][D]), b = sigmoid(b_x), w = sigmoid(w_hat)
  int logits;
  const float* gA;
  const float* gtau;
  // Segmented state pass (long sequences with few heads; nseg <= 1: one pass from S0).
  // The NC chunks of every head run as nseg segments of seg_len chunks.  The state
  // step is affine in S, so segment s maps its entering state to S_in Pi_s + C_s;
  // aff receives those maps for s = 0 .. nseg-2 as [(bh*nseg + s)][2D][D] fp32
  // (rows 0..D-1 C_s, rows D..2D-1 Pi_s), S_seg the entering state of every
  // segment as [(bh*nseg + s)][D][D] fp32 (S_in(0) = S0).
  int nseg, seg_len;
  int aff_vs;             // rows of [C; Pi] per workgroup of the affine-map pass (16, 32 or 64)
  float* aff;
  float* S_seg;
};

struct ContentArgs {
  const float* b_x;
  const float* U1;        // may be null
  const float* U2;        // may be null
  int R;
  const float* m0;        // may be null
  float* m_out;           // may be null
  int period;             // content period in tokens (the chunk length L), multiple of LC
  float* z_all;           // may be null: [B*H][periods][Dk] content signal z of every period
  float* m_all;           // may be null: [B*H][periods][Dv] the mean output each period's z was formed from
};

// Per-period pieces of the backward through the content-aware erase.
struct ContentBwdArgs {
  int B, H, T, D, L, NP, R;   // L = content period in tokens, NP = number of periods
  int p;                      // the period a launch works on
  const float* z_all;         // [B*H][NP][D] content signal of every period
  const float* m_all;         // [B*H][NP][D] mean output each period's signal was formed from
  const float* bmat;          // [B,H,T,D] the gate b of every token
  float* dbx;                 // [B,H,T,D] in: d/db of period p; out: d/db_x
  const float* U1;            // [H,R,D] or null (no projection)
  const float* U2;            // [H,D,R]
  float* dU1p;                // [B*H][R][D] per-sequence accumulators
  float* dU2p;                // [B*H][D][R]
  float* g;                   // [B*H][D] output-gradient term of the last period (before the sweep)
  float* dm0;                 // [B*H][D] or null
};

struct BwdArgs {
  FwdArgs fwd;            // forward inputs, factors and S_vk (all required)
  const void* dO;
  const float* dS_T;      // may be null
  void* dS_vk;            // [ci][D*D] dtype: dS_{c+1}, fragment order rows v
  void* dq;
  void* dk;
  void* dv;
  float* dlog_g;
  float* db;              // may be null (iff b is null)
  int db_mode;            // what db receives: 0 d/db; 1 d/dx for b = sigmoid(x) given as b, i.e. dlog a (1 - b)
  float* dw;
  float* dS0;             // may be null
  // chunk range of the backward kernels: chunks c_lo .. c_lo + c_count - 1 of every
  // head (c_count = 0: all chunks).  The reverse state pass starts from dS_T and
  // ends in dS0 for that range.
  int c_lo, c_count;
  // Segmented reverse pass (fwd.nseg > 1, the forward's segments of fwd.seg_len chunks):
  // raff receives the reverse maps of segments s = 1 .. nseg-1 as [(bh*nseg + s)][2D][D]
  // fp32 (rows 0..D-1 C_s, the segment's pass from a zero gradient; rows D..2D-1 Pi_s,
  // the pass with no output term from the identity), dS_seg the gradient w.r.t. the
  // state leaving every segment as [(bh*nseg + s)][D][D] fp32 (segment nseg-1: dS_T).
  float* raff;
  float* dS_seg;
  // Content-aware backward with one token tile per content period (cg_on != 0): the
  // chunk-gradient workgroup of each head runs the gate backward of its period
  // (content_gate_body) after its stores; cg holds the period's arguments, cg_dO the raw
  // output gradient, and dO (above) receives dO + g for the period before.
  int cg_on;
  ContentBwdArgs cg;
  const void* cg_dO;
  // Range-safe chunks: diag [ci][NB][2][64][4] (dtype) receives the diagonal tiles of
  // dP and dB of the blocks whose log-retention leaves the fast tiles' range (accumulator
  // order); the same workgroup reads them back for those blocks' exact terms.
  void* diag;
};
size_t diag_fix_bytes(int dtype, int BH, int NC, int LC);

// One recurrent decode step (one token per batch and head), state updated in place.
struct DecodeArgs {
  int B, H, Dk, Dv;
  const void* q;          // [B,H,Dk] dtype
  const void* k;          // [B,H,Dk] dtype
  const void* v;          // [B,H,Dv] dtype
  const float* log_g;     // [B,H,Dk]
  const float* b;         // [B,H,Dk] or null (= 1); null on the content path
  const float* w;         // [B,H]
  float* S;               // [B,H,Dv,Dk] read and overwritten
  void* o;                // [B,H,Dv] dtype
  // content-aware erase (b_x null: token-only gates)
  const float* b_x;       // [B,H,Dk]
  const float* U1;        // [H,R,Dv] or null (with U2)
  const float* U2;        // [H,Dk,R] or null
  int R;
  const float* m_in;      // [B,H,Dv] or null (= 0)
  float* m_out;           // [B,H,Dv]
  float* csum;            // [B,H,Dv] running sum of the current chunk's outputs
  int L, pos;             // content period and the token's position inside it
};


// Logit-space epilogue of the backward for gates given as pre-activations.
struct LogitGradArgs {
  int B, H, T, D;
  const float* f;             // [B,H,T,D] decay logits
  const float* A;             // [H,D]
  const float* tau;           // [H,D]
  float* df;                  // [B,H,T,D] in: d/dlog g; out: d/df
  float* partA;               // [B*H][token blocks][D] partial sums
  float* partT;
};
size_t logit_partials_bytes(int B, int H, int T, int D);

size_t factors_bytes(int dtype, int BH, int NC, int LC, int D, int mode);
ChunkFactors carve_factors(void* ws, int dtype, int BH, int NC, int LC, int D, int mode);

// Chain of the segments' affine maps (seg_scan_kernel): init [B*H][D][D] (null: zero),
// seg [(bh*nseg + s)][D][D] the chained rows, aff [(bh*nseg + s)][2D][D] the maps [C; Pi].
struct ScanArgs {
  const float* init;
  float* seg;
  const float* aff;
  int nseg;
};
hipError_t launch_seg_scan(const ScanArgs& a, int D, int BH, bool rev, hipStream_t st);
hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t st);
hipError_t launch_fwd_prep(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_state(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_content(const FwdArgs& a, const ContentArgs& c, hipStream_t st);
hipError_t launch_bwd_state(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t st);
hipError_t launch_content_gates(const ContentBwdArgs& a, const float* b_x, float* bmat, hipStream_t st);
hipError_t launch_add_grad_mean(const ContentBwdArgs& a, int dtype, const void* dO, void* dOp, hipStream_t st);
hipError_t launch_content_gate_bwd(const ContentBwdArgs& a, int dtype, const void* dO, void* dOp, hipStream_t st);
hipError_t launch_init_grad_mean(const ContentBwdArgs& a, const float* dm_out, hipStream_t st);
hipError_t launch_sum_over_batch(const float* part, float* out, int B, int H, int n, hipStream_t st);
hipError_t launch_logit_grads(const LogitGradArgs& a, float* dA, float* dtau, hipStream_t st);
// n16 16-byte vectors; cus = compute units of the current device (sizes the grid)
hipError_t launch_stream_copy(void* dst, const void* src, size_t n16, int cus, hipStream_t st);
// dst[r][c] = c < w_in ? src[r][c] : fill for r < rows, c < w_out; elements of 2 or 4
// bytes, fill given as the element's bit pattern (unequal key and value widths)
hipError_t launch_resize_rows(void* dst, const void* src, size_t rows, size_t w_in, size_t w_out, int elem_bytes,
                              unsigned fill_bits, hipStream_t st);

}  // namespace carve
