// C ABI of the CARVE key-axis gated delta rule: argument checks, workspace
// sizing and kernel dispatch.  Checks run on the host before any launch, so a
// rejected call touches nothing.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/carve.h"
#include "carve_internal.h"

namespace {

struct Plan {
  int BH;      // B * H
  int D;       // Dk == Dv
  int LC;      // token tile of the chunk kernels (32 or 64)
  int NC;      // number of token tiles, ceil(T / LC)
  int VS;      // value rows per state workgroup
  bool empty;  // no token to process
  int nseg;    // segments of the forward state pass (1: one sequential pass per head)
  int seg_len; // chunks per segment
  int aff_vs;  // rows per workgroup of the segments' affine-map pass
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// largest rank of the content projection U_b = U2 U1 (the content kernels hold U1 m in a
// 64-float buffer); padded copies of U1 and U2 are sized for it
constexpr int kMaxRank = 64;

// token tile of the chunk kernels: 32 for short chunks and for float32 inputs
// (LDS budget of the backward chunk kernel), else 64
int tile_for(int L, int dtype, int D) {
  (void)D;
  return (L <= 32 || dtype == CARVE_F32) ? 32 : 64;
}

// value rows per state workgroup: enough workgroups to cover the 256 compute units
int value_slice(int BH, int D) {
  for (int vs : {64, 32, 16}) {
    if (vs <= D && (long long)BH * (D / vs) >= 256) return vs;
  }
  return 16;
}

// Segmented forward state pass: when even 16-row value slices leave compute units
// idle (few heads) and the sequence is long, every head's chunk chain is cut into
// segments whose affine maps are chained by a short scan, so about kSegUnits
// (head, segment) pairs of state workgroups run at once.  Segments keep at least
// kSegMinLen chunks.
#ifndef CARVE_SEG_UNITS
#define CARVE_SEG_UNITS 64
#endif
#ifndef CARVE_AFF_ROWS
#define CARVE_AFF_ROWS 32
#endif
constexpr int kSegUnits = CARVE_SEG_UNITS;
constexpr int kAffRows = CARVE_AFF_ROWS;   // rows of [C; Pi] per affine-pass workgroup
constexpr int kSegMinLen = 16;

void seg_plan(Plan* p) {
  p->nseg = 1;
  p->seg_len = p->NC;
  if (p->empty || (long long)p->BH * (p->D / 16) >= 256 || p->NC < 2 * kSegMinLen) return;
  int want = (kSegUnits + p->BH - 1) / p->BH;
  want = std::min(want, p->NC / kSegMinLen);
  if (want < 2) return;
  const int len = (p->NC + want - 1) / want;
  const int nseg = (p->NC + len - 1) / len;
  if (nseg < 2 || (long long)(nseg - 1) * len > p->NC - 1) return;
  p->nseg = nseg;
  p->seg_len = len;
  p->VS = value_slice(p->BH * nseg, p->D);
  p->aff_vs = std::min(kAffRows, p->D);
}

// fp32 affine maps [C; Pi] and entering states of the segments
size_t seg_bytes(const Plan& p) {
  if (p.nseg <= 1) return 0;
  return (size_t)p.BH * p.nseg * 3 * p.D * p.D * sizeof(float) + 512;
}

carve_status check_shape(const carve_shape* s, Plan* p) {
  if (!s) return CARVE_ERR_INVALID_ARG;
  if (s->B < 0 || s->H < 0 || s->T < 0 || s->L < 1) return CARVE_ERR_INVALID_ARG;
  if (s->dtype != CARVE_F32 && s->dtype != CARVE_BF16) return CARVE_ERR_INVALID_ARG;
  if (s->Dk != s->Dv) return CARVE_ERR_UNSUPPORTED;
  if (s->Dk != 64 && s->Dk != 128) return CARVE_ERR_UNSUPPORTED;
  if ((long long)s->B * s->H > 65535 || s->T > (1 << 30)) return CARVE_ERR_UNSUPPORTED;  // grid y = B*H
  p->BH = s->B * s->H;
  p->D = s->Dk;
  p->LC = tile_for(s->L, s->dtype, s->Dk);
  p->NC = (s->T + p->LC - 1) / p->LC;
  p->VS = value_slice(p->BH, p->D);
  p->empty = (p->BH == 0 || s->T == 0);
  p->nseg = 1;
  p->seg_len = p->NC;
  return CARVE_OK;
}

carve_status check_content(const carve_shape* s, const Plan& p, const carve_content* c, const float* b) {
  if (!c) return CARVE_OK;
  if (b) return CARVE_ERR_INVALID_ARG;                       // erase comes from the content gate
  if ((c->U1 == nullptr) != (c->U2 == nullptr)) return CARVE_ERR_INVALID_ARG;
  if (c->U1 && (c->R < 1 || c->R > kMaxRank)) return CARVE_ERR_INVALID_ARG;
  if (s->L % p.LC != 0) return CARVE_ERR_UNSUPPORTED;        // content period must be whole tiles
  if (!p.empty && !c->b_x) return CARVE_ERR_INVALID_ARG;
  if ((c->z_rec == nullptr) != (c->m_rec == nullptr)) return CARVE_ERR_INVALID_ARG;   // records come in pairs
  for (const void* q : {(const void*)c->b_x, (const void*)c->U1, (const void*)c->U2, (const void*)c->m0,
                        (const void*)c->m_out, (const void*)c->z_rec, (const void*)c->m_rec})
    if (q && !aligned16(q)) return CARVE_ERR_INVALID_ARG;
  return CARVE_OK;
}

size_t fwd_ws(const carve_shape* s, const Plan& p, const carve_content* c) {
  if (p.empty) return 0;
  if (c) return carve::factors_bytes(s->dtype == CARVE_BF16, p.BH, 1, p.LC, p.D, 1);  // one slot per head
  Plan ps = p;
  seg_plan(&ps);
  return carve::factors_bytes(s->dtype == CARVE_BF16, p.BH, p.NC, p.LC, p.D, 1) + seg_bytes(ps);
}

// carve the segment buffers (segmented pass only) from `base` (seg_bytes of space)
void set_segments(carve::FwdArgs* a, const Plan& p, void* base) {
  if (p.nseg <= 1) return;
  char* al = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(base) + 255) & ~uintptr_t(255));
  a->nseg = p.nseg;
  a->seg_len = p.seg_len;
  a->aff_vs = p.aff_vs;
  a->VS = p.VS;
  a->aff = reinterpret_cast<float*>(al);
  a->S_seg = a->aff + (size_t)p.BH * p.nseg * 2 * p.D * p.D;
}
void* after_factors(void* workspace, const carve_shape* s, const Plan& p, int mode) {
  return static_cast<char*>(workspace) + carve::factors_bytes(s->dtype == CARVE_BF16, p.BH, p.NC, p.LC, p.D, mode);
}
// the plan with the segmented state passes (long sequences, few heads)
Plan seg_planned(const Plan& p) {
  Plan ps = p;
  seg_plan(&ps);
  return ps;
}

// one fragment-order copy of the D x D state for every chunk, in the operand type
size_t states_bytes(const carve_shape* s, const Plan& p) {
  return (size_t)p.BH * p.NC * p.D * p.D * (s->dtype == CARVE_BF16 ? 2 : 4);
}

// saved buffer of carve_fwd_save: factors (forward + backward layouts) and the
// state entering every chunk (one fragment-order copy)
size_t saved_bytes(const carve_shape* s, const Plan& p) {
  if (p.empty) return 0;
  // (+ the segmented forward pass's maps and entering states, when it is segmented)
  return carve::factors_bytes(s->dtype == CARVE_BF16, p.BH, p.NC, p.LC, p.D, 3) + (states_bytes(s, p) + 256) + 256 +
         seg_bytes(seg_planned(p));
}

// diagonal tiles of the blocks whose exact within-block terms the range-safe chunk
// gradients add
size_t diag_bytes(const carve_shape* s, const Plan& p) {
  return carve::diag_fix_bytes(s->dtype == CARVE_BF16, p.BH, p.NC, p.LC) + 256;
}
void set_diag(carve::BwdArgs* a, const carve_shape* s, const Plan& p, void* base) {
  a->diag = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(base) + 255) & ~uintptr_t(255));
  (void)s;
  (void)p;
}

// workspace of carve_bwd_saved: the state gradients (one fragment-order copy), then the
// fix-up flags and tiles
size_t bwd_saved_ws(const carve_shape* s, const Plan& p) {
  if (p.empty) return 0;
  // (+ the segmented reverse pass's maps and segment gradients, when it is segmented)
  return (states_bytes(s, p) + 256) + 256 + diag_bytes(s, p) + seg_bytes(seg_planned(p));
}

size_t bwd_ws(const carve_shape* s, const Plan& p) {
  if (p.empty) return 0;
  // S and dS per chunk, one fragment-order copy each, in the operand type; the fix-up
  // flags and tiles
  // (+ the segment maps, used by the forward pass and then by the reverse pass)
  return carve::factors_bytes(s->dtype == CARVE_BF16, p.BH, p.NC, p.LC, p.D, 2) + 2 * (states_bytes(s, p) + 256) + 256 +
         diag_bytes(s, p) + seg_bytes(seg_planned(p));
}

carve::FwdArgs fwd_args(const carve_shape* s, const Plan& p, const void* q, const void* k, const void* v,
                        const float* log_g, const float* b, const float* w, const float* S0, void* o,
                        float* S_T) {
  carve::FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.B = s->B;
  a.H = s->H;
  a.T = s->T;
  a.D = p.D;
  a.LC = p.LC;
  a.NC = p.NC;
  a.VS = p.VS;
  a.dtype = s->dtype == CARVE_BF16 ? 1 : 0;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_g = log_g;
  a.b = b;
  a.w = w;
  a.S0 = S0;
  a.o = o;
  a.S_T = S_T;
  return a;
}

void mark(const carve_profile* prof, int i, hipStream_t st) {
  if (prof && i >= 0 && i < prof->n_events && i <= CARVE_MAX_STAGES && prof->events[i])
    (void)hipEventRecord(reinterpret_cast<hipEvent_t>(prof->events[i]), st);
}

char* align_up(void* p) {
  return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(p) + 255) & ~uintptr_t(255));
}

// Library-owned scratch of carve_fwd_noalloc: one copy of this array on every device the
// library runs on (held until the process ends).  Its name is a host-side stand-in;
// the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[CARVE_NOALLOC_SCRATCH_BYTES];

void* scratch_address(carve_status* st) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *st = CARVE_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *st = CARVE_ERR_HIP;
      return nullptr;
    }
    addr[dev] = ptr;
  }
  *st = CARVE_OK;
  return addr[dev];
}

// ------------------------------------------------------------ unequal key and value widths
// The state is d_v x d_k with independent widths (CARVE notes, section 1).  A call with
// Dk != Dv (each 64 or 128) runs the equal-width path at D = max(Dk, Dv) on padded copies
// of its operands.  Padded key channels get k = q = 0, log g = 0 and b = 1 (retention 1):
// the state columns they own stay zero and add nothing to S k or S q.  Padded value rows
// get v = 0 and dO = 0: the state rows they own stay zero and change no other row.  Every
// padded term is therefore an exact zero, and the outputs restricted to the true widths
// are the result of the unequal-width recurrence.  The padded copies sit in front of the
// workspace (for the training pair, the padded inputs sit in front of the saved buffer,
// where the backward finds them again).
bool width_ok(int d) { return d == 64 || d == 128; }
bool unequal_widths(const carve_shape* s) {
  return s && s->Dk != s->Dv && width_ok(s->Dk) && width_ok(s->Dv);
}
carve_shape widened(const carve_shape* s) {
  carve_shape w = *s;
  w.Dk = w.Dv = std::max(s->Dk, s->Dv);
  return w;
}

enum class PadUse { Fwd, FwdContent, Bwd, BwdContent, Saved, BwdSaved };
constexpr size_t kNone = ~size_t(0);

// Byte offsets of the padded operands of one call (kNone: not used), each 256-byte aligned.
struct PadLayout {
  size_t q = kNone, k = kNone, v = kNone, lg = kNone, b = kNone;           // inputs
  size_t S0 = kNone, S_T = kNone, o = kNone;                               // forward
  size_t dO = kNone, dS_T = kNone, dq = kNone, dk = kNone, dv = kNone;     // backward
  size_t dlg = kNone, db = kNone, dS0 = kNone;
  size_t bx = kNone, U1 = kNone, U2 = kNone, m0 = kNone, m_out = kNone, z_rec = kNone, m_rec = kNone;  // content
  size_t gA = kNone, gtau = kNone, dgA = kNone, dgtau = kNone;   // gate pre-activations: A, tau and their gradients
  size_t dm_out = kNone, dU1 = kNone, dU2 = kNone, dm0 = kNone;   // content backward
  size_t total = 0;
};

PadLayout pad_layout(const carve_shape* s, PadUse use) {
  PadLayout L;
  const size_t D = std::max(s->Dk, s->Dv), BH = (size_t)s->B * s->H, T = (size_t)s->T;
  const size_t es = s->dtype == CARVE_BF16 ? 2 : 4;
  const size_t tok = BH * T * D, st = BH * D * D * sizeof(float);
  const bool kn = s->Dk < s->Dv;   // the key axis is the narrow one
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += (bytes + 255) & ~size_t(255); return at; };
  // inputs of the forward first: for the training pair they persist in the saved buffer
  if (use != PadUse::BwdSaved) {
    if (kn) {
      L.q = take(tok * es);
      L.k = take(tok * es);
      L.lg = take(tok * 4);   // log g, or the decay logits f
      L.b = take(tok * 4);    // b, or the erase pre-activation b_x
      L.gA = take((size_t)s->H * D * 4);
      L.gtau = take((size_t)s->H * D * 4);
    } else {
      L.v = take(tok * es);
    }
  }
  if (use == PadUse::Fwd || use == PadUse::FwdContent || use == PadUse::Saved) {
    L.S0 = take(st);
    L.S_T = take(st);
    if (!kn) L.o = take(tok * es);
  }
  if (use == PadUse::FwdContent || use == PadUse::BwdContent) {
    // the content gate's operands on the narrow axis: b_x, U2 and z (key), or U1 and m (value)
    const size_t per = ((size_t)s->T + s->L - 1) / s->L;   // content periods
    if (kn) {
      L.bx = take(tok * 4);
      L.U2 = take((size_t)s->H * D * kMaxRank * 4);
      L.z_rec = take(BH * per * D * 4);
    } else {
      L.U1 = take((size_t)s->H * kMaxRank * D * 4);
      L.m0 = take(BH * D * 4);
      L.m_out = take(BH * D * 4);
      L.m_rec = take(BH * per * D * 4);
    }
  }
  if (use == PadUse::BwdContent) {
    if (kn) {
      L.dU2 = take((size_t)s->H * D * kMaxRank * 4);
    } else {
      L.dm_out = take(BH * D * 4);
      L.dU1 = take((size_t)s->H * kMaxRank * D * 4);
      L.dm0 = take(BH * D * 4);
    }
  }
  if (use == PadUse::Bwd || use == PadUse::BwdContent) L.S0 = take(st);
  if (use == PadUse::Bwd || use == PadUse::BwdContent || use == PadUse::BwdSaved) {
    L.dS_T = take(st);
    L.dS0 = take(st);
    if (kn) {
      L.dq = take(tok * es);
      L.dk = take(tok * es);
      L.dlg = take(tok * 4);
      L.db = take(tok * 4);
      L.dgA = take((size_t)s->H * D * 4);
      L.dgtau = take((size_t)s->H * D * 4);
    } else {
      L.dO = take(tok * es);
      L.dv = take(tok * es);
    }
  }
  L.total = off;
  return L;
}

// Moves operands between the caller's widths and the padded width D.
struct Widen {
  const carve_shape* s;
  size_t D, BH, T, es;
  bool kn;
  char* base;
  hipStream_t st;
  hipError_t e = hipSuccess;
  Widen(const carve_shape* s_, char* base_, hipStream_t st_)
      : s(s_), D(std::max(s_->Dk, s_->Dv)), BH((size_t)s_->B * s_->H), T((size_t)s_->T),
        es(s_->dtype == CARVE_BF16 ? 2 : 4), kn(s_->Dk < s_->Dv), base(base_), st(st_) {}
  void* at(size_t off) const { return off == kNone ? nullptr : base + off; }
  // [BH*T][narrow] <-> [BH*T][D] of the narrow axis (elements of `eb` bytes)
  void* pad_tok(size_t off, const void* src, size_t eb, unsigned fill) {
    if (!src || off == kNone) return nullptr;
    const size_t nw = kn ? s->Dk : s->Dv;
    if (e == hipSuccess) e = carve::launch_resize_rows(at(off), src, BH * T, nw, D, (int)eb, fill, st);
    return at(off);
  }
  void unpad_tok(void* dst, size_t off, size_t eb) {
    if (!dst || off == kNone) return;
    const size_t nw = kn ? s->Dk : s->Dv;
    if (e == hipSuccess) e = carve::launch_resize_rows(dst, at(off), BH * T, D, nw, (int)eb, 0u, st);
  }
  // state [BH][Dv][Dk] <-> [BH][D][D]: padded key columns, or padded value rows
  float* pad_state(size_t off, const float* src) {
    if (!src || off == kNone) return nullptr;
    if (e == hipSuccess)
      e = kn ? carve::launch_resize_rows(at(off), src, BH * D, s->Dk, D, 4, 0u, st)
             : carve::launch_resize_rows(at(off), src, BH, (size_t)s->Dv * D, D * D, 4, 0u, st);
    return static_cast<float*>(at(off));
  }
  // per head and key channel [H][Dk] <-> [H][D] (narrow key axis only)
  const float* pad_head(size_t off, const float* src) {
    if (!src || off == kNone) return src;
    if (e == hipSuccess) e = carve::launch_resize_rows(at(off), src, s->H, s->Dk, D, 4, 0u, st);
    return static_cast<const float*>(at(off));
  }
  void unpad_head(float* dst, size_t off) {
    if (!dst || off == kNone) return;
    if (e == hipSuccess) e = carve::launch_resize_rows(dst, at(off), s->H, D, s->Dk, 4, 0u, st);
  }
  void unpad_state(float* dst, size_t off) {
    if (!dst || off == kNone) return;
    if (e == hipSuccess)
      e = kn ? carve::launch_resize_rows(dst, at(off), BH * D, D, s->Dk, 4, 0u, st)
             : carve::launch_resize_rows(dst, at(off), BH, D * D, (size_t)s->Dv * D, 4, 0u, st);
  }
};
constexpr unsigned kOneBits = 0x3f800000u;   // 1.0f
// erase pre-activation of a padded key channel: sigmoid(1e30 + z) = 1 and its
// log-sigmoid is exactly 0 in float32, with no infinity in the arithmetic
constexpr unsigned kBigBits = 0x7149f2cau;   // 1.0e30f

bool all_aligned(std::initializer_list<const void*> ptrs) {
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return false;
  return true;
}
size_t unequal_need(const Plan& p, const PadLayout& L, size_t inner) { return p.empty ? 0 : L.total + inner + 512; }

// The content gate's operands padded for the wider width (b_x = 1e30 with zero rows of U2
// on a narrow key axis; zero columns of U1 and zero means on a narrow value axis); the
// records, when given, are read (backward) or written (forward) through padded buffers.
carve_content pad_content(Widen& W, const PadLayout& L, const carve_content* c, bool records_in) {
  carve_content cp = *c;
  const int R = c->U1 ? c->R : 0;
  const size_t H = (size_t)W.s->H, per = ((size_t)W.s->T + W.s->L - 1) / W.s->L;
  hipStream_t hs = W.st;
  if (W.kn) {
    cp.b_x = static_cast<const float*>(W.pad_tok(L.bx, c->b_x, 4, kBigBits));
    if (c->U2 && W.e == hipSuccess)
      W.e = carve::launch_resize_rows(W.at(L.U2), c->U2, H, (size_t)W.s->Dk * R, W.D * R, 4, 0u, hs);
    if (c->U2) cp.U2 = static_cast<const float*>(W.at(L.U2));
    if (c->z_rec) {
      if (records_in && W.e == hipSuccess)
        W.e = carve::launch_resize_rows(W.at(L.z_rec), c->z_rec, W.BH * per, W.s->Dk, W.D, 4, 0u, hs);
      cp.z_rec = static_cast<float*>(W.at(L.z_rec));
    }
  } else {
    if (c->U1 && W.e == hipSuccess)
      W.e = carve::launch_resize_rows(W.at(L.U1), c->U1, H * R, W.s->Dv, W.D, 4, 0u, hs);
    if (c->U1) cp.U1 = static_cast<const float*>(W.at(L.U1));
    if (c->m0 && W.e == hipSuccess)
      W.e = carve::launch_resize_rows(W.at(L.m0), c->m0, W.BH, W.s->Dv, W.D, 4, 0u, hs);
    if (c->m0) cp.m0 = static_cast<const float*>(W.at(L.m0));
    if (c->m_out) cp.m_out = static_cast<float*>(W.at(L.m_out));
    if (c->m_rec) {
      if (records_in && W.e == hipSuccess)
        W.e = carve::launch_resize_rows(W.at(L.m_rec), c->m_rec, W.BH * per, W.s->Dv, W.D, 4, 0u, hs);
      cp.m_rec = static_cast<float*>(W.at(L.m_rec));
    }
  }
  return cp;
}

carve_status fwd_unequal(const carve_shape* s, const void* q, const void* k, const void* v, const float* log_g,
                         const float* b, const float* w, const float* S0, const carve_content* content, void* o,
                         float* S_T, void* workspace, size_t workspace_bytes, void* stream,
                         const carve_profile* prof) {
  const carve_shape ws = widened(s);
  Plan p;
  carve_status st = check_shape(&ws, &p);
  if (st != CARVE_OK) return st;
  st = check_content(&ws, p, content, b);
  if (st != CARVE_OK) return st;
  if (!p.empty && (!q || !k || !v || !log_g || !w || !o)) return CARVE_ERR_INVALID_ARG;
  if (!all_aligned({q, k, v, log_g, b, w, S0, o, S_T})) return CARVE_ERR_INVALID_ARG;
  const PadLayout L = pad_layout(s, content ? PadUse::FwdContent : PadUse::Fwd);
  const size_t need = unequal_need(p, L, fwd_ws(&ws, p, content));
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = S_T ? carve::launch_copy_or_zero(S_T, S0, (size_t)p.BH * s->Dv * s->Dk, hs) : hipSuccess;
    if (e == hipSuccess && content && content->m_out)
      e = carve::launch_copy_or_zero(content->m_out, content->m0, (size_t)p.BH * s->Dv, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  Widen W(s, align_up(workspace), hs);
  carve_content cp{};
  if (content) cp = pad_content(W, L, content, false);
  const void* qp = W.kn ? W.pad_tok(L.q, q, W.es, 0u) : q;
  const void* kp = W.kn ? W.pad_tok(L.k, k, W.es, 0u) : k;
  const float* lgp = W.kn ? static_cast<const float*>(W.pad_tok(L.lg, log_g, 4, 0u)) : log_g;
  const float* bp = W.kn ? static_cast<const float*>(W.pad_tok(L.b, b, 4, kOneBits)) : b;
  const void* vp = W.kn ? v : W.pad_tok(L.v, v, W.es, 0u);
  const float* S0p = W.pad_state(L.S0, S0);
  void* op = W.kn ? o : W.at(L.o);
  float* STp = S_T ? static_cast<float*>(W.at(L.S_T)) : nullptr;
  if (W.e != hipSuccess) return CARVE_ERR_HIP;
  char* inner = align_up(W.base + L.total);
  st = carve_fwd_ex(&ws, qp, kp, vp, lgp, bp, w, S0p, content ? &cp : nullptr, op, STp, inner,
                    workspace_bytes - (size_t)(inner - static_cast<char*>(workspace)), stream, prof);
  if (st != CARVE_OK) return st;
  if (!W.kn) W.unpad_tok(o, L.o, W.es);
  W.unpad_state(S_T, L.S_T);
  if (content && W.e == hipSuccess) {
    const size_t per = ((size_t)s->T + s->L - 1) / s->L;
    if (W.kn && content->z_rec)
      W.e = carve::launch_resize_rows(content->z_rec, W.at(L.z_rec), W.BH * per, W.D, s->Dk, 4, 0u, hs);
    if (!W.kn && content->m_out && W.e == hipSuccess)
      W.e = carve::launch_resize_rows(content->m_out, W.at(L.m_out), W.BH, W.D, s->Dv, 4, 0u, hs);
    if (!W.kn && content->m_rec && W.e == hipSuccess)
      W.e = carve::launch_resize_rows(content->m_rec, W.at(L.m_rec), W.BH * per, W.D, s->Dv, 4, 0u, hs);
  }
  return W.e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

// outputs of a backward at the padded width: the narrow axis's gradients go to padded
// buffers and come back cut to the caller's width
struct BwdOut {
  void *dq, *dk, *dv;
  float *dlog_g, *db, *dS0;
};
BwdOut bwd_outputs(Widen& W, const PadLayout& L, void* dq, void* dk, void* dv, float* dlog_g, float* db,
                   float* dS0) {
  BwdOut r{dq, dk, dv, dlog_g, db, dS0 ? static_cast<float*>(W.at(L.dS0)) : nullptr};
  if (W.kn) {
    r.dq = W.at(L.dq);
    r.dk = W.at(L.dk);
    r.dlog_g = static_cast<float*>(W.at(L.dlg));
    r.db = db ? static_cast<float*>(W.at(L.db)) : nullptr;
  } else {
    r.dv = W.at(L.dv);
  }
  return r;
}
void bwd_unpad(Widen& W, const PadLayout& L, void* dq, void* dk, void* dv, float* dlog_g, float* db, float* dS0) {
  if (W.kn) {
    W.unpad_tok(dq, L.dq, W.es);
    W.unpad_tok(dk, L.dk, W.es);
    W.unpad_tok(dlog_g, L.dlg, 4);
    W.unpad_tok(db, L.db, 4);
  } else {
    W.unpad_tok(dv, L.dv, W.es);
  }
  W.unpad_state(dS0, L.dS0);
}

carve_status bwd_unequal(const carve_shape* s, const void* q, const void* k, const void* v, const float* log_g,
                         const float* b, const float* w, const float* S0, const void* dO, const float* dS_T,
                         void* dq, void* dk, void* dv, float* dlog_g, float* db, float* dw, float* dS0,
                         void* workspace, size_t workspace_bytes, void* stream, const carve_profile* prof) {
  const carve_shape ws = widened(s);
  Plan p;
  carve_status st = check_shape(&ws, &p);
  if (st != CARVE_OK) return st;
  if ((b == nullptr) != (db == nullptr)) return CARVE_ERR_INVALID_ARG;
  if (!p.empty && (!q || !k || !v || !log_g || !w || !dO || !dq || !dk || !dv || !dlog_g || !dw))
    return CARVE_ERR_INVALID_ARG;
  if (!all_aligned({q, k, v, log_g, b, w, S0, dO, dS_T, dq, dk, dv, dlog_g, db, dw, dS0}))
    return CARVE_ERR_INVALID_ARG;
  const PadLayout L = pad_layout(s, PadUse::Bwd);
  const size_t need = unequal_need(p, L, bwd_ws(&ws, p));
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = dS0 ? carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * s->Dv * s->Dk, hs) : hipSuccess;
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  Widen W(s, align_up(workspace), hs);
  const void* qp = W.kn ? W.pad_tok(L.q, q, W.es, 0u) : q;
  const void* kp = W.kn ? W.pad_tok(L.k, k, W.es, 0u) : k;
  const float* lgp = W.kn ? static_cast<const float*>(W.pad_tok(L.lg, log_g, 4, 0u)) : log_g;
  const float* bp = W.kn ? static_cast<const float*>(W.pad_tok(L.b, b, 4, kOneBits)) : b;
  const void* vp = W.kn ? v : W.pad_tok(L.v, v, W.es, 0u);
  const void* dOp = W.kn ? dO : W.pad_tok(L.dO, dO, W.es, 0u);
  const float* S0p = W.pad_state(L.S0, S0);
  const float* dSTp = W.pad_state(L.dS_T, dS_T);
  const BwdOut r = bwd_outputs(W, L, dq, dk, dv, dlog_g, db, dS0);
  if (W.e != hipSuccess) return CARVE_ERR_HIP;
  char* inner = align_up(W.base + L.total);
  st = carve_bwd_ex(&ws, qp, kp, vp, lgp, bp, w, S0p, dOp, dSTp, r.dq, r.dk, r.dv, r.dlog_g, r.db, dw, r.dS0,
                    inner, workspace_bytes - (size_t)(inner - static_cast<char*>(workspace)), stream, prof);
  if (st != CARVE_OK) return st;
  bwd_unpad(W, L, dq, dk, dv, dlog_g, db, dS0);
  return W.e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

size_t saved_unequal_bytes(const carve_shape* s) {
  const carve_shape ws = widened(s);
  Plan p;
  if (check_shape(&ws, &p) != CARVE_OK) return 0;
  return unequal_need(p, pad_layout(s, PadUse::Saved), saved_bytes(&ws, p));
}
size_t bwd_saved_unequal_ws(const carve_shape* s) {
  const carve_shape ws = widened(s);
  Plan p;
  if (check_shape(&ws, &p) != CARVE_OK) return 0;
  return unequal_need(p, pad_layout(s, PadUse::BwdSaved), bwd_saved_ws(&ws, p));
}

carve_status fwd_save_unequal(const carve_shape* s, const void* q, const void* k, const void* v,
                              const float* log_g, const float* b, const float* w, const float* S0, void* o,
                              float* S_T, void* saved, size_t saved_bytes_given, void* stream,
                              const carve_profile* prof) {
  const carve_shape ws = widened(s);
  Plan p;
  carve_status st = check_shape(&ws, &p);
  if (st != CARVE_OK) return st;
  if (!p.empty && (!q || !k || !v || !log_g || !w || !o)) return CARVE_ERR_INVALID_ARG;
  if (!all_aligned({q, k, v, log_g, b, w, S0, o, S_T, saved})) return CARVE_ERR_INVALID_ARG;
  const PadLayout L = pad_layout(s, PadUse::Saved);
  const size_t need = unequal_need(p, L, saved_bytes(&ws, p));
  if (saved_bytes_given < need || (need > 0 && !saved)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = S_T ? carve::launch_copy_or_zero(S_T, S0, (size_t)p.BH * s->Dv * s->Dk, hs) : hipSuccess;
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  // the padded inputs stay in the saved buffer for carve_bwd_saved
  Widen W(s, align_up(saved), hs);
  const void* qp = W.kn ? W.pad_tok(L.q, q, W.es, 0u) : q;
  const void* kp = W.kn ? W.pad_tok(L.k, k, W.es, 0u) : k;
  const float* lgp = W.kn ? static_cast<const float*>(W.pad_tok(L.lg, log_g, 4, 0u)) : log_g;
  const float* bp = W.kn ? static_cast<const float*>(W.pad_tok(L.b, b, 4, kOneBits)) : b;
  const void* vp = W.kn ? v : W.pad_tok(L.v, v, W.es, 0u);
  const float* S0p = W.pad_state(L.S0, S0);
  void* op = W.kn ? o : W.at(L.o);
  float* STp = S_T ? static_cast<float*>(W.at(L.S_T)) : nullptr;
  if (W.e != hipSuccess) return CARVE_ERR_HIP;
  char* inner = align_up(W.base + L.total);
  st = carve_fwd_save(&ws, qp, kp, vp, lgp, bp, w, S0p, op, STp, inner,
                      saved_bytes_given - (size_t)(inner - static_cast<char*>(saved)), stream, prof);
  if (st != CARVE_OK) return st;
  if (!W.kn) W.unpad_tok(o, L.o, W.es);
  W.unpad_state(S_T, L.S_T);
  return W.e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

carve_status bwd_saved_unequal(const carve_shape* s, const void* q, const void* k, const void* v,
                               const float* log_g, const float* b, const float* w, const void* dO,
                               const float* dS_T, const void* saved, size_t saved_bytes_given, void* dq, void* dk,
                               void* dv, float* dlog_g, float* db, float* dw, float* dS0, void* workspace,
                               size_t workspace_bytes, void* stream, const carve_profile* prof) {
  const carve_shape ws = widened(s);
  Plan p;
  carve_status st = check_shape(&ws, &p);
  if (st != CARVE_OK) return st;
  if ((b == nullptr) != (db == nullptr)) return CARVE_ERR_INVALID_ARG;
  if (!p.empty && (!q || !k || !v || !log_g || !w || !dO || !dq || !dk || !dv || !dlog_g || !dw))
    return CARVE_ERR_INVALID_ARG;
  if (!all_aligned({q, k, v, log_g, b, w, dO, dS_T, saved, dq, dk, dv, dlog_g, db, dw, dS0}))
    return CARVE_ERR_INVALID_ARG;
  const PadLayout Ls = pad_layout(s, PadUse::Saved);
  const size_t need_saved = unequal_need(p, Ls, saved_bytes(&ws, p));
  if (saved_bytes_given < need_saved || (need_saved > 0 && !saved)) return CARVE_ERR_WORKSPACE;
  const PadLayout L = pad_layout(s, PadUse::BwdSaved);
  const size_t need = unequal_need(p, L, bwd_saved_ws(&ws, p));
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = dS0 ? carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * s->Dv * s->Dk, hs) : hipSuccess;
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  // the forward's padded inputs, from the saved buffer (same layout as carve_fwd_save wrote)
  Widen Ws(s, align_up(const_cast<void*>(saved)), hs);
  const void* qp = Ws.kn ? Ws.at(Ls.q) : q;
  const void* kp = Ws.kn ? Ws.at(Ls.k) : k;
  const float* lgp = Ws.kn ? static_cast<const float*>(Ws.at(Ls.lg)) : log_g;
  const float* bp = Ws.kn ? (b ? static_cast<const float*>(Ws.at(Ls.b)) : nullptr) : b;
  const void* vp = Ws.kn ? v : Ws.at(Ls.v);
  char* inner_saved = align_up(Ws.base + Ls.total);
  Widen W(s, align_up(workspace), hs);
  const void* dOp = W.kn ? dO : W.pad_tok(L.dO, dO, W.es, 0u);
  const float* dSTp = W.pad_state(L.dS_T, dS_T);
  const BwdOut r = bwd_outputs(W, L, dq, dk, dv, dlog_g, db, dS0);
  if (W.e != hipSuccess) return CARVE_ERR_HIP;
  char* inner = align_up(W.base + L.total);
  st = carve_bwd_saved(&ws, qp, kp, vp, lgp, bp, w, dOp, dSTp, inner_saved,
                       saved_bytes_given - (size_t)(inner_saved - static_cast<const char*>(saved)), r.dq, r.dk, r.dv,
                       r.dlog_g, r.db, dw, r.dS0, inner,
                       workspace_bytes - (size_t)(inner - static_cast<char*>(workspace)), stream, prof);
  if (st != CARVE_OK) return st;
  bwd_unpad(W, L, dq, dk, dv, dlog_g, db, dS0);
  return W.e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

carve_status bwd_content_unequal(const carve_shape* s, const void* q, const void* k, const void* v,
                                 const float* log_g, const float* w, const float* S0, const carve_content* content,
                                 const void* dO, const float* dS_T, const float* dm_out, void* dq, void* dk, void* dv,
                                 float* dlog_g, float* db_x, float* dw, float* dU1, float* dU2, float* dm0,
                                 float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  const carve_shape ws = widened(s);
  Plan p;
  carve_status st = check_shape(&ws, &p);
  if (st != CARVE_OK) return st;
  if (!content) return CARVE_ERR_INVALID_ARG;
  st = check_content(&ws, p, content, nullptr);
  if (st != CARVE_OK) return st;
  const bool proj = content->U1 != nullptr;
  if ((dU1 == nullptr) != !proj || (dU2 == nullptr) != !proj) return CARVE_ERR_INVALID_ARG;
  if (!p.empty && (!q || !k || !v || !log_g || !w || !dO || !dq || !dk || !dv || !dlog_g || !db_x || !dw))
    return CARVE_ERR_INVALID_ARG;
  if (!all_aligned({q, k, v, log_g, w, S0, dO, dS_T, dm_out, dq, dk, dv, dlog_g, db_x, dw, dU1, dU2, dm0, dS0}))
    return CARVE_ERR_INVALID_ARG;
  const PadLayout L = pad_layout(s, PadUse::BwdContent);
  const size_t need = unequal_need(p, L, carve_bwd_content_workspace_size(&ws, content));
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int R = proj ? content->R : 0;
  if (p.empty) {
    hipError_t e = dS0 ? carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * s->Dv * s->Dk, hs) : hipSuccess;
    if (e == hipSuccess && dm0) e = carve::launch_copy_or_zero(dm0, dm_out, (size_t)p.BH * s->Dv, hs);
    if (e == hipSuccess && proj) e = carve::launch_copy_or_zero(dU1, nullptr, (size_t)s->H * R * s->Dv, hs);
    if (e == hipSuccess && proj) e = carve::launch_copy_or_zero(dU2, nullptr, (size_t)s->H * s->Dk * R, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  Widen W(s, align_up(workspace), hs);
  const void* qp = W.kn ? W.pad_tok(L.q, q, W.es, 0u) : q;
  const void* kp = W.kn ? W.pad_tok(L.k, k, W.es, 0u) : k;
  const float* lgp = W.kn ? static_cast<const float*>(W.pad_tok(L.lg, log_g, 4, 0u)) : log_g;
  const void* vp = W.kn ? v : W.pad_tok(L.v, v, W.es, 0u);
  const void* dOp = W.kn ? dO : W.pad_tok(L.dO, dO, W.es, 0u);
  const carve_content cp = pad_content(W, L, content, true);
  const float* S0p = W.pad_state(L.S0, S0);
  const float* dSTp = W.pad_state(L.dS_T, dS_T);
  const float* dmop = dm_out;
  if (!W.kn && dm_out && W.e == hipSuccess)
    W.e = carve::launch_resize_rows(W.at(L.dm_out), dm_out, W.BH, s->Dv, W.D, 4, 0u, hs);
  if (!W.kn && dm_out) dmop = static_cast<const float*>(W.at(L.dm_out));
  const BwdOut r = bwd_outputs(W, L, dq, dk, dv, dlog_g, db_x, dS0);
  float* dU1p = (!W.kn && dU1) ? static_cast<float*>(W.at(L.dU1)) : dU1;
  float* dU2p = (W.kn && dU2) ? static_cast<float*>(W.at(L.dU2)) : dU2;
  float* dm0p = (!W.kn && dm0) ? static_cast<float*>(W.at(L.dm0)) : dm0;
  if (W.e != hipSuccess) return CARVE_ERR_HIP;
  char* inner = align_up(W.base + L.total);
  st = carve_bwd_content(&ws, qp, kp, vp, lgp, w, S0p, &cp, dOp, dSTp, dmop, r.dq, r.dk, r.dv, r.dlog_g, r.db, dw,
                         dU1p, dU2p, dm0p, r.dS0, inner, workspace_bytes - (size_t)(inner - static_cast<char*>(workspace)),
                         stream);
  if (st != CARVE_OK) return st;
  bwd_unpad(W, L, dq, dk, dv, dlog_g, db_x, dS0);
  if (W.e == hipSuccess && !W.kn && dU1)
    W.e = carve::launch_resize_rows(dU1, dU1p, (size_t)s->H * R, W.D, s->Dv, 4, 0u, hs);
  if (W.e == hipSuccess && W.kn && dU2)
    W.e = carve::launch_resize_rows(dU2, dU2p, (size_t)s->H, W.D * R, (size_t)s->Dk * R, 4, 0u, hs);
  if (W.e == hipSuccess && !W.kn && dm0)
    W.e = carve::launch_resize_rows(dm0, dm0p, W.BH, W.D, s->Dv, 4, 0u, hs);
  return W.e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

// gate pre-activations on a narrow key axis: f, A and tau padded with 0 (log g = -0 * softplus
// = 0), b_x with 1e30 (b = 1); w_hat is per token and needs nothing
carve_gate_logits pad_logits(Widen& W, const PadLayout& L, const carve_gate_logits* g) {
  carve_gate_logits r = *g;
  if (!W.kn) return r;
  r.f = static_cast<const float*>(W.pad_tok(L.lg, g->f, 4, 0u));
  r.b_x = static_cast<const float*>(W.pad_tok(L.b, g->b_x, 4, kBigBits));
  r.A = W.pad_head(L.gA, g->A);
  r.tau = W.pad_head(L.gtau, g->tau);
  return r;
}
// the same padded gates, as carve_fwd_logits_save left them in the saved buffer
carve_gate_logits saved_logits(const Widen& W, const PadLayout& L, const carve_gate_logits* g) {
  carve_gate_logits r = *g;
  if (!W.kn) return r;
  r.f = static_cast<const float*>(W.at(L.lg));
  r.b_x = g->b_x ? static_cast<const float*>(W.at(L.b)) : nullptr;
  r.A = static_cast<const float*>(W.at(L.gA));
  r.tau = static_cast<const float*>(W.at(L.gtau));
  return r;
}
carve_status check_logits(const carve_shape* s, const Plan& p, const carve_gate_logits* g) {
  if (!g) return CARVE_ERR_INVALID_ARG;
  if (!p.empty && (!g->f || !g->A || !g->tau || !g->w_hat)) return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {(const void*)g->f, (const void*)g->b_x, (const void*)g->w_hat})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  return CARVE_OK;
}

carve_status fwd_logits_unequal(const carve_shape* s, const void* q, const void* k, const void* v,
                                const carve_gate_logits* gates, const float* S0, void* o, float* S_T,
                                void* saved_or_ws, size_t bytes, void* stream, const carve_profile* prof,
                                bool save) {
  const carve_shape ws = widened(s);
  Plan p;
  carve_status st = check_shape(&ws, &p);
  if (st != CARVE_OK) return st;
  st = check_logits(&ws, p, gates);
  if (st != CARVE_OK) return st;
  if (!p.empty && (!q || !k || !v || !o)) return CARVE_ERR_INVALID_ARG;
  if (!all_aligned({q, k, v, S0, o, S_T, save ? saved_or_ws : nullptr})) return CARVE_ERR_INVALID_ARG;
  const PadLayout L = pad_layout(s, save ? PadUse::Saved : PadUse::Fwd);
  const size_t need = unequal_need(p, L, save ? saved_bytes(&ws, p) : fwd_ws(&ws, p, nullptr));
  if (bytes < need || (need > 0 && !saved_or_ws)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = S_T ? carve::launch_copy_or_zero(S_T, S0, (size_t)p.BH * s->Dv * s->Dk, hs) : hipSuccess;
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  // for the training pair the padded inputs stay in the saved buffer for the backward
  Widen W(s, align_up(saved_or_ws), hs);
  const void* qp = W.kn ? W.pad_tok(L.q, q, W.es, 0u) : q;
  const void* kp = W.kn ? W.pad_tok(L.k, k, W.es, 0u) : k;
  const void* vp = W.kn ? v : W.pad_tok(L.v, v, W.es, 0u);
  const carve_gate_logits gp = pad_logits(W, L, gates);
  const float* S0p = W.pad_state(L.S0, S0);
  void* op = W.kn ? o : W.at(L.o);
  float* STp = S_T ? static_cast<float*>(W.at(L.S_T)) : nullptr;
  if (W.e != hipSuccess) return CARVE_ERR_HIP;
  char* inner = align_up(W.base + L.total);
  const size_t left = bytes - (size_t)(inner - static_cast<char*>(saved_or_ws));
  st = save ? carve_fwd_logits_save(&ws, qp, kp, vp, &gp, S0p, op, STp, inner, left, stream, prof)
            : carve_fwd_logits(&ws, qp, kp, vp, &gp, S0p, op, STp, inner, left, stream);
  if (st != CARVE_OK) return st;
  if (!W.kn) W.unpad_tok(o, L.o, W.es);
  W.unpad_state(S_T, L.S_T);
  return W.e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

// the recomputing backward (saved == nullptr) or the saved one
carve_status bwd_logits_unequal(const carve_shape* s, const void* q, const void* k, const void* v,
                                const carve_gate_logits* gates, const float* S0, const void* dO, const float* dS_T,
                                const void* saved, size_t saved_bytes_given, void* dq, void* dk, void* dv,
                                float* df, float* dA, float* dtau, float* db_x, float* dw_hat, float* dS0,
                                void* workspace, size_t workspace_bytes, void* stream, const carve_profile* prof,
                                bool use_saved) {
  const carve_shape ws = widened(s);
  Plan p;
  carve_status st = check_shape(&ws, &p);
  if (st != CARVE_OK) return st;
  st = check_logits(&ws, p, gates);
  if (st != CARVE_OK) return st;
  if ((gates->b_x == nullptr) != (db_x == nullptr)) return CARVE_ERR_INVALID_ARG;
  if (!p.empty && (!q || !k || !v || !dO || !dq || !dk || !dv || !df || !dA || !dtau || !dw_hat))
    return CARVE_ERR_INVALID_ARG;
  if (!all_aligned({q, k, v, S0, dO, dS_T, use_saved ? saved : nullptr, dq, dk, dv, df, db_x, dw_hat, dS0}))
    return CARVE_ERR_INVALID_ARG;
  const PadLayout Ls = pad_layout(s, PadUse::Saved);
  if (use_saved) {
    const size_t need_saved = unequal_need(p, Ls, saved_bytes(&ws, p));
    if (saved_bytes_given < need_saved || (need_saved > 0 && !saved)) return CARVE_ERR_WORKSPACE;
  }
  const PadLayout L = pad_layout(s, use_saved ? PadUse::BwdSaved : PadUse::Bwd);
  const size_t inner_need = use_saved ? carve_bwd_logits_saved_workspace_size(&ws) : carve_bwd_logits_workspace_size(&ws);
  const size_t need = unequal_need(p, L, inner_need);
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = dS0 ? carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * s->Dv * s->Dk, hs) : hipSuccess;
    if (e == hipSuccess && dA && s->H > 0) e = carve::launch_copy_or_zero(dA, nullptr, (size_t)s->H * s->Dk, hs);
    if (e == hipSuccess && dtau && s->H > 0) e = carve::launch_copy_or_zero(dtau, nullptr, (size_t)s->H * s->Dk, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  Widen W(s, align_up(workspace), hs);
  const void *qp, *kp, *vp;
  carve_gate_logits gp;
  char* inner_saved = nullptr;
  if (use_saved) {
    // the forward's padded inputs, from the saved buffer (same layout as carve_fwd_logits_save wrote)
    Widen Ws(s, align_up(const_cast<void*>(saved)), hs);
    qp = Ws.kn ? Ws.at(Ls.q) : q;
    kp = Ws.kn ? Ws.at(Ls.k) : k;
    vp = Ws.kn ? v : Ws.at(Ls.v);
    gp = saved_logits(Ws, Ls, gates);
    inner_saved = align_up(Ws.base + Ls.total);
  } else {
    qp = W.kn ? W.pad_tok(L.q, q, W.es, 0u) : q;
    kp = W.kn ? W.pad_tok(L.k, k, W.es, 0u) : k;
    vp = W.kn ? v : W.pad_tok(L.v, v, W.es, 0u);
    gp = pad_logits(W, L, gates);
  }
  const void* dOp = W.kn ? dO : W.pad_tok(L.dO, dO, W.es, 0u);
  const float* S0p = use_saved ? nullptr : W.pad_state(L.S0, S0);
  const float* dSTp = W.pad_state(L.dS_T, dS_T);
  const BwdOut r = bwd_outputs(W, L, dq, dk, dv, df, db_x, dS0);
  float* dAp = W.kn ? static_cast<float*>(W.at(L.dgA)) : dA;
  float* dtaup = W.kn ? static_cast<float*>(W.at(L.dgtau)) : dtau;
  if (W.e != hipSuccess) return CARVE_ERR_HIP;
  char* inner = align_up(W.base + L.total);
  const size_t left = workspace_bytes - (size_t)(inner - static_cast<char*>(workspace));
  st = use_saved
           ? carve_bwd_logits_saved(&ws, qp, kp, vp, &gp, dOp, dSTp, inner_saved,
                                    saved_bytes_given - (size_t)(inner_saved - static_cast<const char*>(saved)), r.dq,
                                    r.dk, r.dv, r.dlog_g, dAp, dtaup, r.db, dw_hat, r.dS0, inner, left, stream, prof)
           : carve_bwd_logits(&ws, qp, kp, vp, &gp, S0p, dOp, dSTp, r.dq, r.dk, r.dv, r.dlog_g, dAp, dtaup, r.db,
                              dw_hat, r.dS0, inner, left, stream);
  if (st != CARVE_OK) return st;
  bwd_unpad(W, L, dq, dk, dv, df, db_x, dS0);
  if (W.kn) {
    W.unpad_head(dA, L.dgA);
    W.unpad_head(dtau, L.dgtau);
  }
  return W.e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

}  // namespace

extern "C" {

size_t carve_fwd_workspace_size(const carve_shape* s, const carve_content* content) {
  if (unequal_widths(s)) {
    const carve_shape ws = widened(s);
    Plan p;
    if (check_shape(&ws, &p) != CARVE_OK) return 0;
    return unequal_need(p, pad_layout(s, content ? PadUse::FwdContent : PadUse::Fwd), fwd_ws(&ws, p, content));
  }
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return fwd_ws(s, p, content);
}

size_t carve_bwd_workspace_size(const carve_shape* s) {
  if (unequal_widths(s)) {
    const carve_shape ws = widened(s);
    Plan p;
    if (check_shape(&ws, &p) != CARVE_OK) return 0;
    return unequal_need(p, pad_layout(s, PadUse::Bwd), bwd_ws(&ws, p));
  }
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return bwd_ws(s, p);
}

carve_status carve_fwd(const carve_shape* s, const void* q, const void* k, const void* v, const float* log_g,
                       const float* b, const float* w, const float* S0, const carve_content* content, void* o,
                       float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
  return carve_fwd_ex(s, q, k, v, log_g, b, w, S0, content, o, S_T, workspace, workspace_bytes, stream, nullptr);
}

carve_status carve_fwd_ex(const carve_shape* s, const void* q, const void* k, const void* v, const float* log_g,
                          const float* b, const float* w, const float* S0, const carve_content* content, void* o,
                          float* S_T, void* workspace, size_t workspace_bytes, void* stream,
                          const carve_profile* prof) {
  if (unequal_widths(s))
    return fwd_unequal(s, q, k, v, log_g, b, w, S0, content, o, S_T, workspace, workspace_bytes, stream, prof);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  st = check_content(s, p, content, b);
  if (st != CARVE_OK) return st;
  if (!p.empty) {
    if (!q || !k || !v || !log_g || !w || !o) return CARVE_ERR_INVALID_ARG;
  }
  for (const void* ptr : {q, k, v, (const void*)log_g, (const void*)b, (const void*)w, (const void*)S0,
                          (const void*)o, (const void*)S_T})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const size_t need = fwd_ws(s, p, content);
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = hipSuccess;
    if (S_T) e = carve::launch_copy_or_zero(S_T, S0, (size_t)p.BH * p.D * p.D, hs);
    if (e == hipSuccess && content && content->m_out)
      e = carve::launch_copy_or_zero(content->m_out, content->m0, (size_t)p.BH * p.D, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  carve::FwdArgs a = fwd_args(s, p, q, k, v, log_g, b, w, S0, o, S_T);
  a.mode = 1;
  hipError_t e;
  if (content) {
    a.f = carve::carve_factors(workspace, a.dtype, p.BH, 1, p.LC, p.D, 1);
    carve::ContentArgs cg = {};
    cg.b_x = content->b_x;
    cg.U1 = content->U1;
    cg.U2 = content->U2;
    cg.R = content->U1 ? content->R : 0;
    cg.m0 = content->m0;
    cg.m_out = content->m_out;
    cg.period = s->L;
    cg.z_all = content->z_rec;      // per-period records (may be null)
    cg.m_all = content->m_rec;
    mark(prof, 0, hs);
    e = carve::launch_fwd_content(a, cg, hs);
    mark(prof, 1, hs);
  } else {
    a.f = carve::carve_factors(workspace, a.dtype, p.BH, p.NC, p.LC, p.D, 1);
    set_segments(&a, seg_planned(p), after_factors(workspace, s, p, 1));
    mark(prof, 0, hs);
    e = carve::launch_fwd_prep(a, hs);
    mark(prof, 1, hs);
    if (e == hipSuccess) e = carve::launch_fwd_state(a, hs);
    mark(prof, 2, hs);
  }
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

carve_status carve_fwd_noalloc(const carve_shape* s, const void* q, const void* k, const void* v,
                               const float* log_g, const float* b, const float* w, const float* S0,
                               const carve_content* content, void* o, float* S_T, void* stream) {
  carve_status st;
  if (unequal_widths(s)) {
    const carve_shape wide = widened(s);
    Plan p;
    st = check_shape(&wide, &p);
    if (st != CARVE_OK) return st;
    st = check_content(&wide, p, content, b);
    if (st != CARVE_OK) return st;
    if (carve_fwd_workspace_size(s, content) > CARVE_NOALLOC_SCRATCH_BYTES) return CARVE_ERR_WORKSPACE;
    void* ws = scratch_address(&st);
    if (st != CARVE_OK) return st;
    return carve_fwd_ex(s, q, k, v, log_g, b, w, S0, content, o, S_T, ws, CARVE_NOALLOC_SCRATCH_BYTES, stream,
                        nullptr);
  }
  Plan p;
  st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  st = check_content(s, p, content, b);
  if (st != CARVE_OK) return st;
  if (fwd_ws(s, p, content) > CARVE_NOALLOC_SCRATCH_BYTES) return CARVE_ERR_WORKSPACE;
  void* ws = scratch_address(&st);
  if (st != CARVE_OK) return st;
  return carve_fwd_ex(s, q, k, v, log_g, b, w, S0, content, o, S_T, ws, CARVE_NOALLOC_SCRATCH_BYTES, stream,
                      nullptr);
}

carve_status carve_bwd(const carve_shape* s, const void* q, const void* k, const void* v, const float* log_g,
                       const float* b, const float* w, const float* S0, const void* dO, const float* dS_T,
                       void* dq, void* dk, void* dv, float* dlog_g, float* db, float* dw, float* dS0,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return carve_bwd_ex(s, q, k, v, log_g, b, w, S0, dO, dS_T, dq, dk, dv, dlog_g, db, dw, dS0, workspace,
                      workspace_bytes, stream, nullptr);
}

carve_status carve_bwd_ex(const carve_shape* s, const void* q, const void* k, const void* v, const float* log_g,
                          const float* b, const float* w, const float* S0, const void* dO, const float* dS_T,
                          void* dq, void* dk, void* dv, float* dlog_g, float* db, float* dw, float* dS0,
                          void* workspace, size_t workspace_bytes, void* stream, const carve_profile* prof) {
  if (unequal_widths(s))
    return bwd_unequal(s, q, k, v, log_g, b, w, S0, dO, dS_T, dq, dk, dv, dlog_g, db, dw, dS0, workspace,
                       workspace_bytes, stream, prof);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  if ((b == nullptr) != (db == nullptr)) return CARVE_ERR_INVALID_ARG;
  if (!p.empty) {
    if (!q || !k || !v || !log_g || !w || !dO || !dq || !dk || !dv || !dlog_g || !dw)
      return CARVE_ERR_INVALID_ARG;
  }
  for (const void* ptr : {q, k, v, (const void*)log_g, (const void*)b, (const void*)w, (const void*)S0, dO,
                          (const void*)dS_T, (const void*)dq, (const void*)dk, (const void*)dv,
                          (const void*)dlog_g, (const void*)db, (const void*)dw, (const void*)dS0})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const size_t need = bwd_ws(s, p);
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = hipSuccess;
    if (dS0) e = carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * p.D * p.D, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  carve::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.fwd = fwd_args(s, p, q, k, v, log_g, b, w, S0, nullptr, nullptr);
  a.fwd.mode = 2;
  a.fwd.f = carve::carve_factors(workspace, a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 2);
  char* base = align_up(static_cast<char*>(workspace) +
                        carve::factors_bytes(a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 2));
  const size_t states = states_bytes(s, p);
  a.fwd.S_vk = base;
  a.dS_vk = align_up(base + states);
  set_diag(&a, s, p, static_cast<char*>(a.dS_vk) + states);
  // segmented state passes: the forward's maps, then (the same memory) the reverse maps
  set_segments(&a.fwd, seg_planned(p),
               static_cast<char*>(a.diag) + carve::diag_fix_bytes(a.fwd.dtype, p.BH, p.NC, p.LC));
  a.raff = a.fwd.aff;
  a.dS_seg = a.fwd.S_seg;
  a.dO = dO;
  a.dS_T = dS_T;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_g = dlog_g;
  a.db = db;
  a.dw = dw;
  a.dS0 = dS0;
  mark(prof, 0, hs);
  hipError_t e = carve::launch_fwd_prep(a.fwd, hs);
  mark(prof, 1, hs);
  if (e == hipSuccess) e = carve::launch_fwd_state(a.fwd, hs);
  mark(prof, 2, hs);
  if (e == hipSuccess) e = carve::launch_bwd_state(a, hs);
  mark(prof, 3, hs);
  if (e == hipSuccess) e = carve::launch_bwd_chunk(a, hs);
  mark(prof, 4, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

size_t carve_saved_size(const carve_shape* s) {
  if (unequal_widths(s)) return saved_unequal_bytes(s);
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return saved_bytes(s, p);
}

size_t carve_bwd_saved_workspace_size(const carve_shape* s) {
  if (unequal_widths(s)) return bwd_saved_unequal_ws(s);
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return bwd_saved_ws(s, p);
}

carve_status carve_fwd_save(const carve_shape* s, const void* q, const void* k, const void* v, const float* log_g,
                            const float* b, const float* w, const float* S0, void* o, float* S_T, void* saved,
                            size_t saved_bytes_given, void* stream, const carve_profile* prof) {
  if (unequal_widths(s))
    return fwd_save_unequal(s, q, k, v, log_g, b, w, S0, o, S_T, saved, saved_bytes_given, stream, prof);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  if (!p.empty && (!q || !k || !v || !log_g || !w || !o)) return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, (const void*)log_g, (const void*)b, (const void*)w, (const void*)S0,
                          (const void*)o, (const void*)S_T, (const void*)saved})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const size_t need = saved_bytes(s, p);
  if (saved_bytes_given < need || (need > 0 && !saved)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = hipSuccess;
    if (S_T) e = carve::launch_copy_or_zero(S_T, S0, (size_t)p.BH * p.D * p.D, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  carve::FwdArgs a = fwd_args(s, p, q, k, v, log_g, b, w, S0, o, S_T);
  a.mode = 3;
  a.f = carve::carve_factors(saved, a.dtype, p.BH, p.NC, p.LC, p.D, 3);
  char* base = align_up(static_cast<char*>(saved) + carve::factors_bytes(a.dtype, p.BH, p.NC, p.LC, p.D, 3));
  a.S_vk = base;
  set_segments(&a, seg_planned(p), base + states_bytes(s, p) + 256);
  mark(prof, 0, hs);
  hipError_t e = carve::launch_fwd_prep(a, hs);
  mark(prof, 1, hs);
  if (e == hipSuccess) e = carve::launch_fwd_state(a, hs);
  mark(prof, 2, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

carve_status carve_bwd_saved(const carve_shape* s, const void* q, const void* k, const void* v,
                             const float* log_g, const float* b, const float* w, const void* dO,
                             const float* dS_T, const void* saved, size_t saved_bytes_given, void* dq, void* dk,
                             void* dv, float* dlog_g, float* db, float* dw, float* dS0, void* workspace,
                             size_t workspace_bytes, void* stream, const carve_profile* prof) {
  if (unequal_widths(s))
    return bwd_saved_unequal(s, q, k, v, log_g, b, w, dO, dS_T, saved, saved_bytes_given, dq, dk, dv, dlog_g, db,
                             dw, dS0, workspace, workspace_bytes, stream, prof);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  if ((b == nullptr) != (db == nullptr)) return CARVE_ERR_INVALID_ARG;
  if (!p.empty) {
    if (!q || !k || !v || !log_g || !w || !dO || !dq || !dk || !dv || !dlog_g || !dw) return CARVE_ERR_INVALID_ARG;
  }
  for (const void* ptr : {q, k, v, (const void*)log_g, (const void*)b, (const void*)w, dO, (const void*)dS_T,
                          saved, (const void*)dq, (const void*)dk, (const void*)dv, (const void*)dlog_g,
                          (const void*)db, (const void*)dw, (const void*)dS0})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const size_t need_saved = saved_bytes(s, p);
  if (saved_bytes_given < need_saved || (need_saved > 0 && !saved)) return CARVE_ERR_WORKSPACE;
  const size_t need = bwd_saved_ws(s, p);
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = hipSuccess;
    if (dS0) e = carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * p.D * p.D, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  carve::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.fwd = fwd_args(s, p, q, k, v, log_g, b, w, nullptr, nullptr, nullptr);
  a.fwd.mode = 3;
  void* sv = const_cast<void*>(saved);
  a.fwd.f = carve::carve_factors(sv, a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 3);
  char* base = align_up(static_cast<char*>(sv) + carve::factors_bytes(a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 3));
  const size_t states = states_bytes(s, p);
  a.fwd.S_vk = base;
  a.dS_vk = align_up(workspace);
  set_diag(&a, s, p, static_cast<char*>(a.dS_vk) + states);
  // segmented reverse pass: the reverse maps and segment gradients
  set_segments(&a.fwd, seg_planned(p),
               static_cast<char*>(a.diag) + carve::diag_fix_bytes(a.fwd.dtype, p.BH, p.NC, p.LC));
  a.raff = a.fwd.aff;
  a.dS_seg = a.fwd.S_seg;
  a.dO = dO;
  a.dS_T = dS_T;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_g = dlog_g;
  a.db = db;
  a.dw = dw;
  a.dS0 = dS0;
  mark(prof, 0, hs);
  hipError_t e = carve::launch_bwd_state(a, hs);
  mark(prof, 1, hs);
  if (e == hipSuccess) e = carve::launch_bwd_chunk(a, hs);
  mark(prof, 2, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

// ------------------------------------------------------------ gate pre-activations

// arguments of the logit-space epilogue (df in place, dA and dtau from per-block partial sums)
carve::LogitGradArgs logit_grad_args(const carve_shape* s, const Plan& p, const carve_gate_logits* gates, float* df,
                                     float* partA) {
  carve::LogitGradArgs lg = {};
  lg.B = s->B;
  lg.H = s->H;
  lg.T = s->T;
  lg.D = p.D;
  lg.f = gates->f;
  lg.A = gates->A;
  lg.tau = gates->tau;
  lg.df = df;
  lg.partA = partA;
  lg.partT = partA + carve::logit_partials_bytes(s->B, s->H, s->T, p.D) / (2 * sizeof(float));
  return lg;
}

carve_status carve_fwd_logits(const carve_shape* s, const void* q, const void* k, const void* v,
                              const carve_gate_logits* gates, const float* S0, void* o, float* S_T,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (unequal_widths(s))
    return fwd_logits_unequal(s, q, k, v, gates, S0, o, S_T, workspace, workspace_bytes, stream, nullptr, false);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  st = check_logits(s, p, gates);
  if (st != CARVE_OK) return st;
  if (!p.empty && (!q || !k || !v || !o)) return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, (const void*)S0, (const void*)o, (const void*)S_T})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const size_t need = fwd_ws(s, p, nullptr);
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = S_T ? carve::launch_copy_or_zero(S_T, S0, (size_t)p.BH * p.D * p.D, hs) : hipSuccess;
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  carve::FwdArgs a = fwd_args(s, p, q, k, v, gates->f, gates->b_x, gates->w_hat, S0, o, S_T);
  a.logits = 1;
  a.gA = gates->A;
  a.gtau = gates->tau;
  a.mode = 1;
  a.f = carve::carve_factors(workspace, a.dtype, p.BH, p.NC, p.LC, p.D, 1);
  set_segments(&a, seg_planned(p), after_factors(workspace, s, p, 1));
  hipError_t e = carve::launch_fwd_prep(a, hs);
  if (e == hipSuccess) e = carve::launch_fwd_state(a, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

size_t carve_bwd_logits_workspace_size(const carve_shape* s) {
  if (unequal_widths(s)) {
    const carve_shape ws = widened(s);
    Plan p;
    if (check_shape(&ws, &p) != CARVE_OK) return 0;
    return unequal_need(p, pad_layout(s, PadUse::Bwd), carve_bwd_logits_workspace_size(&ws));
  }
  Plan p;
  if (check_shape(s, &p) != CARVE_OK || p.empty) return 0;
  return bwd_ws(s, p) + carve::logit_partials_bytes(s->B, s->H, s->T, p.D) + 1024;
}

carve_status carve_bwd_logits(const carve_shape* s, const void* q, const void* k, const void* v,
                              const carve_gate_logits* gates, const float* S0, const void* dO, const float* dS_T,
                              void* dq, void* dk, void* dv, float* df, float* dA, float* dtau, float* db_x,
                              float* dw_hat, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  if (unequal_widths(s))
    return bwd_logits_unequal(s, q, k, v, gates, S0, dO, dS_T, nullptr, 0, dq, dk, dv, df, dA, dtau, db_x, dw_hat,
                              dS0, workspace, workspace_bytes, stream, nullptr, false);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  st = check_logits(s, p, gates);
  if (st != CARVE_OK) return st;
  if ((gates->b_x == nullptr) != (db_x == nullptr)) return CARVE_ERR_INVALID_ARG;
  if (!p.empty && (!q || !k || !v || !dO || !dq || !dk || !dv || !df || !dA || !dtau || !dw_hat))
    return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, (const void*)S0, dO, (const void*)dS_T, (const void*)dq, (const void*)dk,
                          (const void*)dv, (const void*)df, (const void*)db_x, (const void*)dw_hat, (const void*)dS0})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const size_t need = carve_bwd_logits_workspace_size(s);
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = dS0 ? carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * p.D * p.D, hs) : hipSuccess;
    if (e == hipSuccess && dA && s->H > 0) e = carve::launch_copy_or_zero(dA, nullptr, (size_t)s->H * p.D, hs);
    if (e == hipSuccess && dtau && s->H > 0) e = carve::launch_copy_or_zero(dtau, nullptr, (size_t)s->H * p.D, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  carve::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.fwd = fwd_args(s, p, q, k, v, gates->f, gates->b_x, gates->w_hat, S0, nullptr, nullptr);
  a.fwd.logits = 1;
  a.fwd.gA = gates->A;
  a.fwd.gtau = gates->tau;
  a.fwd.mode = 2;
  char* ws = align_up(workspace);
  a.fwd.f = carve::carve_factors(ws, a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 2);
  char* base = align_up(ws + carve::factors_bytes(a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 2));
  const size_t states = states_bytes(s, p);
  a.fwd.S_vk = base;
  a.dS_vk = align_up(base + states);
  set_diag(&a, s, p, static_cast<char*>(a.dS_vk) + states);
  float* partA = reinterpret_cast<float*>(align_up(static_cast<char*>(a.dS_vk) + states + 256 + diag_bytes(s, p)));
  a.dO = dO;
  a.dS_T = dS_T;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_g = df;        // d/dlog g, turned into d/df by the logit pass
  a.db = db_x;          // the chunk kernel returns d/db_x directly
  a.dw = dw_hat;        // ... and d/dw_hat
  a.dS0 = dS0;
  hipError_t e = carve::launch_fwd_prep(a.fwd, hs);
  if (e == hipSuccess) e = carve::launch_fwd_state(a.fwd, hs);
  if (e == hipSuccess) e = carve::launch_bwd_state(a, hs);
  if (e == hipSuccess) e = carve::launch_bwd_chunk(a, hs);
  if (e == hipSuccess) e = carve::launch_logit_grads(logit_grad_args(s, p, gates, df, partA), dA, dtau, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

// ------------------------------------------------------------ training pair, gates as pre-activations
size_t bwd_logits_saved_ws(const carve_shape* s, const Plan& p) {
  if (p.empty) return 0;
  return bwd_saved_ws(s, p) + carve::logit_partials_bytes(s->B, s->H, s->T, p.D) + 512;
}

size_t carve_bwd_logits_saved_workspace_size(const carve_shape* s) {
  if (unequal_widths(s)) {
    const carve_shape ws = widened(s);
    Plan p;
    if (check_shape(&ws, &p) != CARVE_OK) return 0;
    return unequal_need(p, pad_layout(s, PadUse::BwdSaved), carve_bwd_logits_saved_workspace_size(&ws));
  }
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return bwd_logits_saved_ws(s, p);
}

carve_status carve_fwd_logits_save(const carve_shape* s, const void* q, const void* k, const void* v,
                                   const carve_gate_logits* gates, const float* S0, void* o, float* S_T,
                                   void* saved, size_t saved_bytes_given, void* stream, const carve_profile* prof) {
  if (unequal_widths(s))
    return fwd_logits_unequal(s, q, k, v, gates, S0, o, S_T, saved, saved_bytes_given, stream, prof, true);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  st = check_logits(s, p, gates);
  if (st != CARVE_OK) return st;
  if (!p.empty && (!q || !k || !v || !o)) return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, (const void*)S0, (const void*)o, (const void*)S_T, (const void*)saved})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const size_t need = saved_bytes(s, p);
  if (saved_bytes_given < need || (need > 0 && !saved)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = S_T ? carve::launch_copy_or_zero(S_T, S0, (size_t)p.BH * p.D * p.D, hs) : hipSuccess;
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  carve::FwdArgs a = fwd_args(s, p, q, k, v, gates->f, gates->b_x, gates->w_hat, S0, o, S_T);
  a.logits = 1;
  a.gA = gates->A;
  a.gtau = gates->tau;
  a.mode = 3;
  a.f = carve::carve_factors(saved, a.dtype, p.BH, p.NC, p.LC, p.D, 3);
  char* base = align_up(static_cast<char*>(saved) + carve::factors_bytes(a.dtype, p.BH, p.NC, p.LC, p.D, 3));
  a.S_vk = base;
  set_segments(&a, seg_planned(p), base + states_bytes(s, p) + 256);
  mark(prof, 0, hs);
  hipError_t e = carve::launch_fwd_prep(a, hs);
  mark(prof, 1, hs);
  if (e == hipSuccess) e = carve::launch_fwd_state(a, hs);
  mark(prof, 2, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

carve_status carve_bwd_logits_saved(const carve_shape* s, const void* q, const void* k, const void* v,
                                    const carve_gate_logits* gates, const void* dO, const float* dS_T,
                                    const void* saved, size_t saved_bytes_given, void* dq, void* dk, void* dv,
                                    float* df, float* dA, float* dtau, float* db_x, float* dw_hat, float* dS0,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    const carve_profile* prof) {
  if (unequal_widths(s))
    return bwd_logits_unequal(s, q, k, v, gates, nullptr, dO, dS_T, saved, saved_bytes_given, dq, dk, dv, df, dA, dtau,
                              db_x, dw_hat, dS0, workspace, workspace_bytes, stream, prof, true);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  st = check_logits(s, p, gates);
  if (st != CARVE_OK) return st;
  if ((gates->b_x == nullptr) != (db_x == nullptr)) return CARVE_ERR_INVALID_ARG;
  if (!p.empty && (!q || !k || !v || !dO || !dq || !dk || !dv || !df || !dA || !dtau || !dw_hat))
    return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, dO, (const void*)dS_T, saved, (const void*)dq, (const void*)dk, (const void*)dv,
                          (const void*)df, (const void*)db_x, (const void*)dw_hat, (const void*)dS0})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const size_t need_saved = saved_bytes(s, p);
  if (saved_bytes_given < need_saved || (need_saved > 0 && !saved)) return CARVE_ERR_WORKSPACE;
  const size_t need = bwd_logits_saved_ws(s, p);
  if (workspace_bytes < need || (need > 0 && !workspace)) return CARVE_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (p.empty) {
    hipError_t e = dS0 ? carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * p.D * p.D, hs) : hipSuccess;
    if (e == hipSuccess && dA && s->H > 0) e = carve::launch_copy_or_zero(dA, nullptr, (size_t)s->H * p.D, hs);
    if (e == hipSuccess && dtau && s->H > 0) e = carve::launch_copy_or_zero(dtau, nullptr, (size_t)s->H * p.D, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  carve::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.fwd = fwd_args(s, p, q, k, v, gates->f, gates->b_x, gates->w_hat, nullptr, nullptr, nullptr);
  a.fwd.logits = 1;
  a.fwd.gA = gates->A;
  a.fwd.gtau = gates->tau;
  a.fwd.mode = 3;
  void* sv = const_cast<void*>(saved);
  a.fwd.f = carve::carve_factors(sv, a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 3);
  char* base = align_up(static_cast<char*>(sv) + carve::factors_bytes(a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 3));
  const size_t states = states_bytes(s, p);
  a.fwd.S_vk = base;
  a.dS_vk = align_up(workspace);
  set_diag(&a, s, p, static_cast<char*>(a.dS_vk) + states);
  set_segments(&a.fwd, seg_planned(p),
               static_cast<char*>(a.diag) + carve::diag_fix_bytes(a.fwd.dtype, p.BH, p.NC, p.LC));
  a.raff = a.fwd.aff;
  a.dS_seg = a.fwd.S_seg;
  // the logit epilogue's partial sums after everything the saved backward uses
  float* partA = reinterpret_cast<float*>(align_up(static_cast<char*>(workspace) + bwd_saved_ws(s, p)));
  a.dO = dO;
  a.dS_T = dS_T;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_g = df;        // d/dlog g, turned into d/df by the logit pass
  a.db = db_x;          // the chunk kernel returns d/db_x directly
  a.dw = dw_hat;        // ... and d/dw_hat
  a.dS0 = dS0;
  mark(prof, 0, hs);
  hipError_t e = carve::launch_bwd_state(a, hs);
  mark(prof, 1, hs);
  if (e == hipSuccess) e = carve::launch_bwd_chunk(a, hs);
  mark(prof, 2, hs);
  if (e == hipSuccess) e = carve::launch_logit_grads(logit_grad_args(s, p, gates, df, partA), dA, dtau, hs);
  mark(prof, 3, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

// Workspace of carve_bwd_content, in order: the content forward's factor slot, its
// output (scratch), z and m of every period, the gates b, the token-only backward's
// workspace (factors, S and dS per chunk), dO with the mean-output term, the dS carry,
// the period's output-gradient term g, and per-sequence dU1 / dU2 accumulators.
struct ContentBwdLayout {
  size_t fwd, o, z, m, bmat, bwd, dOp, carry, g, du1, du2, total;
};
ContentBwdLayout content_bwd_layout(const carve_shape* s, const Plan& p, const carve_content* c) {
  const size_t es = s->dtype == CARVE_BF16 ? 2 : 4;
  const size_t NP = ((size_t)s->T + s->L - 1) / s->L;
  const size_t R = c && c->U1 ? (size_t)c->R : 0;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  ContentBwdLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += al(bytes); return at; };
  // with the forward's records the content-aware forward is not re-run: no room for it
  const bool rec = c && c->z_rec && c->m_rec;
  L.fwd = take(rec ? 0 : fwd_ws(s, p, c));
  L.o = take(rec ? 0 : (size_t)p.BH * s->T * s->Dv * es);
  L.z = take(rec ? 0 : (size_t)p.BH * NP * p.D * 4);
  L.m = take(rec ? 0 : (size_t)p.BH * NP * p.D * 4);
  L.bmat = take((size_t)p.BH * s->T * p.D * 4);
  L.bwd = take(bwd_ws(s, p));
  L.dOp = take((size_t)p.BH * s->T * s->Dv * es);
  L.carry = take((size_t)p.BH * p.D * p.D * 4);
  L.g = take((size_t)p.BH * p.D * 4);
  L.du1 = take((size_t)p.BH * R * p.D * 4);
  L.du2 = take((size_t)p.BH * p.D * R * 4);
  L.total = p.empty ? 0 : off + 256;
  return L;
}

size_t carve_bwd_content_workspace_size(const carve_shape* s, const carve_content* content) {
  if (unequal_widths(s)) {
    const carve_shape ws = widened(s);
    Plan p;
    if (check_shape(&ws, &p) != CARVE_OK) return 0;
    return unequal_need(p, pad_layout(s, PadUse::BwdContent), carve_bwd_content_workspace_size(&ws, content));
  }
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return content_bwd_layout(s, p, content).total;
}

carve_status carve_bwd_content(const carve_shape* s, const void* q, const void* k, const void* v,
                               const float* log_g, const float* w, const float* S0, const carve_content* content,
                               const void* dO, const float* dS_T, const float* dm_out, void* dq, void* dk,
                               void* dv, float* dlog_g, float* db_x, float* dw, float* dU1, float* dU2,
                               float* dm0, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  if (unequal_widths(s))
    return bwd_content_unequal(s, q, k, v, log_g, w, S0, content, dO, dS_T, dm_out, dq, dk, dv, dlog_g, db_x, dw, dU1,
                               dU2, dm0, dS0, workspace, workspace_bytes, stream);
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  if (!content) return CARVE_ERR_INVALID_ARG;
  st = check_content(s, p, content, nullptr);
  if (st != CARVE_OK) return st;
  const bool proj = content->U1 != nullptr;
  if ((dU1 == nullptr) != !proj || (dU2 == nullptr) != !proj) return CARVE_ERR_INVALID_ARG;
  if (!p.empty) {
    if (!q || !k || !v || !log_g || !w || !dO || !dq || !dk || !dv || !dlog_g || !db_x || !dw)
      return CARVE_ERR_INVALID_ARG;
  }
  for (const void* ptr : {q, k, v, (const void*)log_g, (const void*)w, (const void*)S0, dO, (const void*)dS_T,
                          (const void*)dm_out, (const void*)dq, (const void*)dk, (const void*)dv,
                          (const void*)dlog_g, (const void*)db_x, (const void*)dw, (const void*)dU1,
                          (const void*)dU2, (const void*)dm0, (const void*)dS0})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const ContentBwdLayout Lw = content_bwd_layout(s, p, content);
  if (workspace_bytes < Lw.total || (Lw.total > 0 && !workspace)) return CARVE_ERR_WORKSPACE;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int R = proj ? content->R : 0;
  if (p.empty) {
    // no tokens: S_T = S0 and m_out = m0, so their gradients pass straight through
    hipError_t e = hipSuccess;
    if (dS0) e = carve::launch_copy_or_zero(dS0, dS_T, (size_t)p.BH * p.D * p.D, hs);
    if (e == hipSuccess && dm0) e = carve::launch_copy_or_zero(dm0, dm_out, (size_t)p.BH * p.D, hs);
    if (e == hipSuccess && proj) e = carve::launch_copy_or_zero(dU1, nullptr, (size_t)s->H * R * p.D, hs);
    if (e == hipSuccess && proj) e = carve::launch_copy_or_zero(dU2, nullptr, (size_t)s->H * p.D * R, hs);
    return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
  }
  char* ws = align_up(workspace);
  const bool rec = content->z_rec && content->m_rec;
  const float* z_all = rec ? content->z_rec : reinterpret_cast<float*>(ws + Lw.z);
  const float* m_all = rec ? content->m_rec : reinterpret_cast<float*>(ws + Lw.m);
  float* bmat = reinterpret_cast<float*>(ws + Lw.bmat);

  // 1. each period's z and the mean it was formed from: the forward's records, or the
  //    content-aware forward run again to record them
  hipError_t e = hipSuccess;
  if (!rec) {
    carve::FwdArgs fa = fwd_args(s, p, q, k, v, log_g, nullptr, w, S0, ws + Lw.o, nullptr);
    fa.mode = 1;
    fa.f = carve::carve_factors(ws + Lw.fwd, fa.dtype, p.BH, 1, p.LC, p.D, 1);
    carve::ContentArgs cg = {};
    cg.b_x = content->b_x;
    cg.U1 = content->U1;
    cg.U2 = content->U2;
    cg.R = R;
    cg.m0 = content->m0;
    cg.period = s->L;
    cg.z_all = reinterpret_cast<float*>(ws + Lw.z);
    cg.m_all = reinterpret_cast<float*>(ws + Lw.m);
    e = carve::launch_fwd_content(fa, cg, hs);
  }

  carve::ContentBwdArgs ca = {};
  ca.B = s->B;
  ca.H = s->H;
  ca.T = s->T;
  ca.D = p.D;
  ca.L = s->L;
  ca.NP = (s->T + s->L - 1) / s->L;
  ca.R = R;
  ca.z_all = z_all;
  ca.m_all = m_all;
  ca.bmat = bmat;
  ca.dbx = db_x;
  ca.U1 = content->U1;
  ca.U2 = content->U2;
  ca.dU1p = reinterpret_cast<float*>(ws + Lw.du1);
  ca.dU2p = reinterpret_cast<float*>(ws + Lw.du2);
  ca.g = reinterpret_cast<float*>(ws + Lw.g);
  ca.dm0 = dm0;
  // 2. the gates of every token
  if (e == hipSuccess) e = carve::launch_content_gates(ca, content->b_x, bmat, hs);

  // 3. the token-only backward machinery with those gates: factors and chunk states
  carve::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.fwd = fwd_args(s, p, q, k, v, log_g, bmat, w, S0, nullptr, nullptr);
  a.fwd.mode = 2;
  char* wb = ws + Lw.bwd;
  a.fwd.f = carve::carve_factors(wb, a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 2);
  char* base = align_up(wb + carve::factors_bytes(a.fwd.dtype, p.BH, p.NC, p.LC, p.D, 2));
  a.fwd.S_vk = base;
  a.dS_vk = align_up(base + states_bytes(s, p));
  set_diag(&a, s, p, static_cast<char*>(a.dS_vk) + states_bytes(s, p));
  float* carry = reinterpret_cast<float*>(ws + Lw.carry);
  a.dO = ws + Lw.dOp;
  a.dS_T = carry;
  a.dS0 = carry;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_g = dlog_g;
  a.db = db_x;          // d/db_x for b = sigmoid(b_x + z) directly (dlog a (1 - b))
  a.db_mode = 1;
  a.dw = dw;
  if (e == hipSuccess) e = carve::launch_fwd_prep(a.fwd, hs);
  if (e == hipSuccess) e = carve::launch_fwd_state(a.fwd, hs);

  // 4. the periods in reverse
  if (e == hipSuccess) e = carve::launch_copy_or_zero(carry, dS_T, (size_t)p.BH * p.D * p.D, hs);
  if (e == hipSuccess) e = carve::launch_init_grad_mean(ca, dm_out, hs);
  if (e == hipSuccess && proj) e = carve::launch_copy_or_zero(ca.dU1p, nullptr, (size_t)p.BH * R * p.D, hs);
  if (e == hipSuccess && proj) e = carve::launch_copy_or_zero(ca.dU2p, nullptr, (size_t)p.BH * p.D * R, hs);
  const int per = s->L / p.LC;     // tiles per period
  // the last period's dO + dm_out / n; every other period's dO + g is written by the
  // gate kernel of the period after it
  ca.p = ca.NP - 1;
  if (e == hipSuccess) e = carve::launch_add_grad_mean(ca, a.fwd.dtype, dO, ws + Lw.dOp, hs);
  // with one token tile per period the chunk-gradient workgroup of each head runs its
  // period's gate backward itself; otherwise a gate kernel per period follows
  const bool fused_gate = per == 1;
  a.cg_on = fused_gate ? 1 : 0;
  a.cg_dO = dO;
  for (int pp = ca.NP - 1; pp >= 0 && e == hipSuccess; --pp) {
    ca.p = pp;
    a.c_lo = pp * per;
    a.c_count = std::min(per, p.NC - a.c_lo);
    a.cg = ca;
    e = carve::launch_bwd_state(a, hs);
    if (e == hipSuccess) e = carve::launch_bwd_chunk(a, hs);
    if (e == hipSuccess && !fused_gate) e = carve::launch_content_gate_bwd(ca, a.fwd.dtype, dO, ws + Lw.dOp, hs);
  }
  if (e == hipSuccess && dS0) e = carve::launch_copy_or_zero(dS0, carry, (size_t)p.BH * p.D * p.D, hs);
  if (e == hipSuccess && proj) e = carve::launch_sum_over_batch(ca.dU1p, dU1, s->B, s->H, R * p.D, hs);
  if (e == hipSuccess && proj) e = carve::launch_sum_over_batch(ca.dU2p, dU2, s->B, s->H, p.D * R, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

carve_status carve_decode_step(const carve_shape* s, const void* q, const void* k, const void* v,
                               const float* log_g, const float* b, const float* w, float* S,
                               const carve_decode_content* content, void* o, void* stream) {
  if (!s || s->T != 1) return CARVE_ERR_INVALID_ARG;
  // the decode kernel takes the key and value widths separately
  const carve_shape sc = unequal_widths(s) ? widened(s) : *s;
  Plan p;
  carve_status st = check_shape(&sc, &p);
  if (st != CARVE_OK) return st;
  if (p.BH == 0) return CARVE_OK;
  if (!q || !k || !v || !log_g || !w || !S || !o) return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {(const void*)q, k, (const void*)log_g, (const void*)b, (const void*)S})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const carve_decode_content* c = content;
  if (c) {
    if (b || !c->b_x || !c->m_out || !c->csum) return CARVE_ERR_INVALID_ARG;
    if ((c->U1 == nullptr) != (c->U2 == nullptr)) return CARVE_ERR_INVALID_ARG;
    if (c->U1 && (c->R < 1 || c->R > kMaxRank)) return CARVE_ERR_INVALID_ARG;
    if (c->pos < 0 || c->pos >= s->L) return CARVE_ERR_INVALID_ARG;
    if (c->m_in && c->m_in == c->m_out) return CARVE_ERR_INVALID_ARG;
    if (!aligned16(c->b_x)) return CARVE_ERR_INVALID_ARG;
  }
  carve::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.B = s->B;
  a.H = s->H;
  a.Dk = s->Dk;
  a.Dv = s->Dv;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_g = log_g;
  a.b = b;
  a.w = w;
  a.S = S;
  a.o = o;
  if (c) {
    a.b_x = c->b_x;
    a.U1 = c->U1;
    a.U2 = c->U2;
    a.R = c->U1 ? c->R : 0;
    a.m_in = c->m_in;
    a.m_out = c->m_out;
    a.csum = c->csum;
    a.L = s->L;
    a.pos = c->pos;
  }
  hipError_t e = carve::launch_decode(a, s->dtype == CARVE_BF16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

carve_status carve_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0) return CARVE_OK;
  if (!dst || !src || bytes % 16 || ((uintptr_t)dst | (uintptr_t)src) % 16) return CARVE_ERR_INVALID_ARG;
  const uintptr_t d0 = (uintptr_t)dst, s0 = (uintptr_t)src;
  if (d0 < s0 + bytes && s0 < d0 + bytes) return CARVE_ERR_INVALID_ARG;      // overlapping ranges
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return CARVE_ERR_HIP;
  return carve::launch_stream_copy(dst, src, bytes / 16, cus, (hipStream_t)stream) == hipSuccess ? CARVE_OK
                                                                                                  : CARVE_ERR_HIP;
}

const char* carve_status_string(carve_status st) {
  switch (st) {
    case CARVE_OK: return "CARVE_OK";
    case CARVE_ERR_INVALID_ARG: return "CARVE_ERR_INVALID_ARG: invalid argument";
    case CARVE_ERR_UNSUPPORTED: return "CARVE_ERR_UNSUPPORTED: shape or option not supported";
    case CARVE_ERR_WORKSPACE: return "CARVE_ERR_WORKSPACE: workspace too small";
    case CARVE_ERR_HIP: return "CARVE_ERR_HIP: kernel launch failed";
  }
  return "CARVE_ERR_UNKNOWN";
}

int carve_abi_version(void) { return CARVE_ABI_VERSION; }

}  // extern "C"
