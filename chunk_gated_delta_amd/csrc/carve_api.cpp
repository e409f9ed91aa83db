// C ABI of the CARVE key-axis gated delta rule: argument checks, workspace
// sizing and kernel dispatch.  Checks run on the host before any launch, so a
// rejected call touches nothing.
#include <stdint.h>
#include <string.h>

#include <algorithm>

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
  if (c->U1 && (c->R < 1 || c->R > 64)) return CARVE_ERR_INVALID_ARG;
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

// carve the segment buffers after the forward factors (segmented pass only)
void set_segments(carve::FwdArgs* a, const carve_shape* s, const Plan& p, void* workspace) {
  if (p.nseg <= 1) return;
  char* base = static_cast<char*>(workspace) + carve::factors_bytes(s->dtype == CARVE_BF16, p.BH, p.NC, p.LC, p.D, 1);
  char* al = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(base) + 255) & ~uintptr_t(255));
  a->nseg = p.nseg;
  a->seg_len = p.seg_len;
  a->aff_vs = p.aff_vs;
  a->VS = p.VS;
  a->aff = reinterpret_cast<float*>(al);
  a->S_seg = a->aff + (size_t)p.BH * p.nseg * 2 * p.D * p.D;
}

// one fragment-order copy of the D x D state for every chunk, in the operand type
size_t states_bytes(const carve_shape* s, const Plan& p) {
  return (size_t)p.BH * p.NC * p.D * p.D * (s->dtype == CARVE_BF16 ? 2 : 4);
}

// saved buffer of carve_fwd_save: factors (forward + backward layouts) and the
// state entering every chunk (one fragment-order copy)
size_t saved_bytes(const carve_shape* s, const Plan& p) {
  if (p.empty) return 0;
  return carve::factors_bytes(s->dtype == CARVE_BF16, p.BH, p.NC, p.LC, p.D, 3) + (states_bytes(s, p) + 256) + 256;
}

// workspace of carve_bwd_saved: the state gradients (one fragment-order copy)
size_t bwd_saved_ws(const carve_shape* s, const Plan& p) {
  if (p.empty) return 0;
  return (states_bytes(s, p) + 256) + 256;
}

size_t bwd_ws(const carve_shape* s, const Plan& p) {
  if (p.empty) return 0;
  // S and dS per chunk, one fragment-order copy each, in the operand type
  return carve::factors_bytes(s->dtype == CARVE_BF16, p.BH, p.NC, p.LC, p.D, 2) + 2 * (states_bytes(s, p) + 256) + 256;
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

}  // namespace

extern "C" {

size_t carve_fwd_workspace_size(const carve_shape* s, const carve_content* content) {
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return fwd_ws(s, p, content);
}

size_t carve_bwd_workspace_size(const carve_shape* s) {
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
    Plan ps = p;
    seg_plan(&ps);
    set_segments(&a, s, ps, workspace);
    mark(prof, 0, hs);
    e = carve::launch_fwd_prep(a, hs);
    mark(prof, 1, hs);
    if (e == hipSuccess) e = carve::launch_fwd_state(a, hs);
    mark(prof, 2, hs);
  }
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
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
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return saved_bytes(s, p);
}

size_t carve_bwd_saved_workspace_size(const carve_shape* s) {
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return bwd_saved_ws(s, p);
}

carve_status carve_fwd_save(const carve_shape* s, const void* q, const void* k, const void* v, const float* log_g,
                            const float* b, const float* w, const float* S0, void* o, float* S_T, void* saved,
                            size_t saved_bytes_given, void* stream, const carve_profile* prof) {
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
carve_status check_logits(const carve_shape* s, const Plan& p, const carve_gate_logits* g) {
  if (!g) return CARVE_ERR_INVALID_ARG;
  if (!p.empty && (!g->f || !g->A || !g->tau || !g->w_hat)) return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {(const void*)g->f, (const void*)g->b_x, (const void*)g->w_hat})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  return CARVE_OK;
}

carve_status carve_fwd_logits(const carve_shape* s, const void* q, const void* k, const void* v,
                              const carve_gate_logits* gates, const float* S0, void* o, float* S_T,
                              void* workspace, size_t workspace_bytes, void* stream) {
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
  Plan ps = p;
  seg_plan(&ps);
  set_segments(&a, s, ps, workspace);
  hipError_t e = carve::launch_fwd_prep(a, hs);
  if (e == hipSuccess) e = carve::launch_fwd_state(a, hs);
  return e == hipSuccess ? CARVE_OK : CARVE_ERR_HIP;
}

size_t carve_bwd_logits_workspace_size(const carve_shape* s) {
  Plan p;
  if (check_shape(s, &p) != CARVE_OK || p.empty) return 0;
  return bwd_ws(s, p) + carve::logit_partials_bytes(s->B, s->H, s->T, p.D) + 512;
}

carve_status carve_bwd_logits(const carve_shape* s, const void* q, const void* k, const void* v,
                              const carve_gate_logits* gates, const float* S0, const void* dO, const float* dS_T,
                              void* dq, void* dk, void* dv, float* df, float* dA, float* dtau, float* db_x,
                              float* dw_hat, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
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
  float* partA = reinterpret_cast<float*>(align_up(static_cast<char*>(a.dS_vk) + states));
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
  if (e == hipSuccess) e = carve::launch_logit_grads(lg, dA, dtau, hs);
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
  Plan p;
  if (check_shape(s, &p) != CARVE_OK) return 0;
  return content_bwd_layout(s, p, content).total;
}

carve_status carve_bwd_content(const carve_shape* s, const void* q, const void* k, const void* v,
                               const float* log_g, const float* w, const float* S0, const carve_content* content,
                               const void* dO, const float* dS_T, const float* dm_out, void* dq, void* dk,
                               void* dv, float* dlog_g, float* db_x, float* dw, float* dU1, float* dU2,
                               float* dm0, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
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
  float* carry = reinterpret_cast<float*>(ws + Lw.carry);
  a.dO = ws + Lw.dOp;
  a.dS_T = carry;
  a.dS0 = carry;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_g = dlog_g;
  a.db = db_x;          // d/db first; the gate kernel turns it into d/db_x
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
  for (int pp = ca.NP - 1; pp >= 0 && e == hipSuccess; --pp) {
    ca.p = pp;
    a.c_lo = pp * per;
    a.c_count = std::min(per, p.NC - a.c_lo);
    e = carve::launch_bwd_state(a, hs);
    if (e == hipSuccess) e = carve::launch_bwd_chunk(a, hs);
    if (e == hipSuccess) e = carve::launch_content_gate_bwd(ca, a.fwd.dtype, dO, ws + Lw.dOp, hs);
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
  Plan p;
  carve_status st = check_shape(s, &p);
  if (st != CARVE_OK) return st;
  if (p.BH == 0) return CARVE_OK;
  if (!q || !k || !v || !log_g || !w || !S || !o) return CARVE_ERR_INVALID_ARG;
  for (const void* ptr : {(const void*)q, k, (const void*)log_g, (const void*)b, (const void*)S})
    if (ptr && !aligned16(ptr)) return CARVE_ERR_INVALID_ARG;
  const carve_decode_content* c = content;
  if (c) {
    if (b || !c->b_x || !c->m_out || !c->csum) return CARVE_ERR_INVALID_ARG;
    if ((c->U1 == nullptr) != (c->U2 == nullptr)) return CARVE_ERR_INVALID_ARG;
    if (c->U1 && (c->R < 1 || c->R > 64)) return CARVE_ERR_INVALID_ARG;
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
