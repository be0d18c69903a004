// C ABI of the block-sparse attention library: argument checks, buffer sizes,
// workspace / saved-state carving and the launch sequence of vsa_fwd / vsa_bwd.
// Declarations and argument contracts: include/vsa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"

namespace vsa {
int coarse_rows_per_block(int KVb);
size_t coarse_bwd_lds(int KVb);
}

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return VSA_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(VSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// ---- opt-in kernel timing: event pairs around each launch --------------------
struct ProfRec {
  int kid;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<hipEvent_t> g_prof_pool;
std::vector<ProfRec> g_prof_recs;
size_t g_prof_next = 0;
constexpr size_t kProfMax = 65536;

// Records events around one launch when profiling is on.
struct Prof {
  ProfRec* r = nullptr;
  hipStream_t st;
  Prof(int kid, hipStream_t s) : st(s) {
    if (!g_prof_on || kid < 0) return;  // kid < 0: a launch that records nothing
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_recs.size() >= kProfMax) return;
    while (g_prof_pool.size() < 2 * (g_prof_recs.size() + 1)) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return;
      g_prof_pool.push_back(e);
    }
    ProfRec rec{kid, g_prof_pool[2 * g_prof_recs.size()], g_prof_pool[2 * g_prof_recs.size() + 1]};
    g_prof_recs.push_back(rec);
    r = &g_prof_recs.back();
    (void)hipEventRecord(r->a, st);
  }
  ~Prof() {
    if (r) (void)hipEventRecord(r->b, st);
  }
};

// Sub-buffers of one caller buffer, each 256-byte aligned. With base == nullptr
// it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(long long count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += (size_t)count * sizeof(T);
    return p;
  }
};

bool is_video(const vsa_problem* p) { return p->topk > 0 || p->gate_mode != VSA_GATE_NONE; }

long long nnz_cap(const vsa_problem* p) {
  const long long per = p->topk > 0 ? std::min<long long>(p->topk, p->KVb) : p->KVb;
  return (long long)p->B * p->Hq * p->Qb * per;
}

long long q_elems(const vsa_problem* p) {
  return p->layout == VSA_TND ? (long long)p->Sq * p->Hq * p->D
                              : (long long)p->B * p->Sq * p->Hq * p->D;
}

long long rows_total(const vsa_problem* p) {
  return p->layout == VSA_TND ? (long long)p->Hq * p->Sq : (long long)p->B * p->Hq * p->Sq;
}

// Pieces of the saved state (training forward -> backward).
struct Saved {
  int32_t* q_rp;
  int32_t* q_col;
  int32_t* kv_rp;
  int32_t* kv_col;
  float* qc;
  float* kc;
  float* vc;
  float* oc;
  float* lse_c;
  uint16_t* osel;
};

Saved carve_saved(const vsa_problem* p, void* base, size_t* bytes) {
  Carver c(base);
  Saved s{};
  const long long cap = nnz_cap(p);
  s.q_rp = c.take<int32_t>((long long)p->B * p->Hq * p->Qb + 1);
  s.q_col = c.take<int32_t>(std::max(cap, 1LL));
  s.kv_rp = c.take<int32_t>((long long)p->B * p->Hq * p->KVb + 1);
  s.kv_col = c.take<int32_t>(std::max(cap, 1LL));
  if (p->gate_mode != VSA_GATE_NONE) {
    s.qc = c.take<float>((long long)p->B * p->Hq * p->Qb * p->D);
    s.kc = c.take<float>((long long)p->B * p->Hkv * p->KVb * p->D);
    s.vc = c.take<float>((long long)p->B * p->Hkv * p->KVb * p->D);
    s.oc = c.take<float>((long long)p->B * p->Hq * p->Qb * p->D);
    s.lse_c = c.take<float>((long long)p->B * p->Hq * p->Qb);
    s.osel = c.take<uint16_t>(q_elems(p));
  }
  if (bytes) *bytes = c.off;
  return s;
}

// Forward workspace: the inference-mode index and coarse state, the pooled
// tiles and the selection map of the top-k path.
int compute_units(hipStream_t st, int* out);

struct FwdWs {
  int32_t* q_rp;
  int32_t* q_col;
  float* qc;
  float* kc;
  float* vc;
  float* oc;
  float* lse_c;
  uint8_t* map;
};

FwdWs carve_fwd(const vsa_problem* p, void* base, size_t* bytes) {
  Carver c(base);
  FwdWs w{};
  const long long cap = nnz_cap(p);
  w.q_rp = c.take<int32_t>((long long)p->B * p->Hq * p->Qb + 1);
  w.q_col = c.take<int32_t>(std::max(cap, 1LL));
  if (is_video(p)) {
    w.qc = c.take<float>((long long)p->B * p->Hq * p->Qb * p->D);
    w.kc = c.take<float>((long long)p->B * p->Hkv * p->KVb * p->D);
    w.vc = c.take<float>((long long)p->B * p->Hkv * p->KVb * p->D);
  }
  if (p->gate_mode != VSA_GATE_NONE) {
    w.oc = c.take<float>((long long)p->B * p->Hq * p->Qb * p->D);
    w.lse_c = c.take<float>((long long)p->B * p->Hq * p->Qb);
  }
  if (p->topk > 0) w.map = c.take<uint8_t>((long long)p->B * p->Hq * p->Qb * p->KVb);
  if (bytes) *bytes = c.off;
  return w;
}

vsa::Geom make_geom(const vsa_problem* p);

struct BwdWs {
  float* dr;
  float* lse2;
  int32_t* qlive;
  float* dqacc;  // VSA_FLAG_ATOMIC_DQ: dS K summed over KV blocks, laid out like q
  int32_t* lpt_hist;   // VSA_FLAG_PERSISTENT: sort histogram, then the item counter
  int32_t* lpt_order;  // VSA_FLAG_PERSISTENT: the dK/dV spans, longest first
  float* doc;
  float* dqc;
  float* dkc;
  float* dvc;
  float* ps;
  float* dss;
  float* csum;
  float* dlogit;  // VSA_GATE_PROJECTED: dL/dz per row, laid out like lse
  float* dwp;     // VSA_GATE_PROJECTED: per-Q-block partial sums of dL/dz q
  float* dbp;     // VSA_GATE_PROJECTED: per-Q-block partial sums of dL/dz
};

BwdWs carve_bwd(const vsa_problem* p, void* base, size_t* bytes) {
  Carver c(base);
  BwdWs w{};
  w.dr = c.take<float>(std::max(rows_total(p), 1LL));
  w.lse2 = c.take<float>(std::max(rows_total(p), 1LL));
  w.qlive = c.take<int32_t>(std::max((long long)p->B * p->Hq * p->Qb, 1LL));
  if (p->flags & VSA_FLAG_ATOMIC_DQ) w.dqacc = c.take<float>(std::max(q_elems(p), 1LL));
  if (!(p->flags & VSA_FLAG_NO_PERSISTENT)) {  // the persistent grid may be used
    const vsa::Geom g = make_geom(p);
    w.lpt_hist = c.take<int32_t>(vsa::lpt_hist_entries(g));
    w.lpt_order = c.take<int32_t>(std::max(vsa::dkdv_items(g, vsa::DKDV_SPAN_MIN), 1LL));
  }
  if (p->gate_mode != VSA_GATE_NONE) {
    w.doc = c.take<float>((long long)p->B * p->Hq * p->Qb * p->D);
    w.dqc = c.take<float>((long long)p->B * p->Hq * p->Qb * p->D);
    w.dkc = c.take<float>((long long)p->B * p->Hkv * p->KVb * p->D);
    w.dvc = c.take<float>((long long)p->B * p->Hkv * p->KVb * p->D);
    w.ps = c.take<float>((long long)p->B * p->Hq * p->Qb * p->KVb);
    w.dss = c.take<float>((long long)p->B * p->Hq * p->Qb * p->KVb);
    w.csum = c.take<float>((long long)p->B * p->Hq * p->Qb);
  }
  if (p->gate_mode == VSA_GATE_PROJECTED) {
    w.dlogit = c.take<float>(std::max(rows_total(p), 1LL));
    w.dwp = c.take<float>((long long)p->B * p->Hq * p->Qb * p->D);
    w.dbp = c.take<float>((long long)p->B * p->Hq * p->Qb);
  }
  if (bytes) *bytes = c.off;
  return w;
}

vsa::Geom make_geom(const vsa_problem* p) {
  vsa::Geom g;
  g.layout = p->layout;
  g.B = p->B;
  g.Hq = p->Hq;
  g.Hkv = p->Hkv;
  g.Sq = p->Sq;
  g.Skv = p->Skv;
  g.q_block = p->q_block;
  g.kv_block = p->kv_block;
  g.Qb = p->Qb;
  g.KVb = p->KVb;
  g.group = p->Hq / p->Hkv;
  g.q_valid = p->q_valid;
  g.kv_valid = p->kv_valid;
  g.qv_bs = p->q_valid_batch_stride;
  g.kvv_bs = p->kv_valid_batch_stride;
  g.cu_q = p->cu_seqlens_q;
  g.cu_kv = p->cu_seqlens_kv;
  g.scale = p->scale;
  g.map_bstride = p->map_batch_stride;
  return g;
}

int validate(const vsa_problem* p) {
  if (!p) return fail(VSA_ERR_INVALID_ARG, "problem is NULL");
  if (p->abi_version != VSA_ABI_VERSION)
    return fail(VSA_ERR_INVALID_ARG, "abi_version %d, library has %d", p->abi_version,
                VSA_ABI_VERSION);
  if (p->dtype != VSA_BF16 && p->dtype != VSA_FP16)
    return fail(VSA_ERR_INVALID_ARG, "dtype must be VSA_BF16 or VSA_FP16");
  if (p->layout != VSA_BHSD && p->layout != VSA_BSHD && p->layout != VSA_TND)
    return fail(VSA_ERR_INVALID_ARG, "layout must be BHSD, BSHD or TND");
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1)
    return fail(VSA_ERR_INVALID_ARG, "B, Hq and Hkv must be positive (B=%d Hq=%d Hkv=%d)", p->B,
                p->Hq, p->Hkv);
  if (p->Hq % p->Hkv != 0)
    return fail(VSA_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->D < 1) return fail(VSA_ERR_INVALID_ARG, "D must be positive");
  if (p->D > vsa::HD)
    return fail(VSA_ERR_UNSUPPORTED, "head dimension %d: the kernels take D <= 128", p->D);
  if (p->q_block < 1 || p->kv_block < 1)
    return fail(VSA_ERR_INVALID_ARG, "q_block and kv_block must be positive");
  if ((p->q_block % 32 != 0 && p->q_block != 8 && p->q_block != 16) || p->kv_block % 64 != 0)
    return fail(VSA_ERR_UNSUPPORTED,
                "q_block must be 8, 16 or a multiple of 32 and kv_block a multiple of 64 (got %d, %d)",
                p->q_block, p->kv_block);
  if (p->Sq < 0 || p->Skv < 0) return fail(VSA_ERR_INVALID_ARG, "Sq and Skv must be >= 0");
  if (!(p->scale > 0.f) || !std::isfinite(p->scale))
    return fail(VSA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (p->topk < 0) return fail(VSA_ERR_INVALID_ARG, "topk must be >= 0");
  if (p->gate_mode < VSA_GATE_NONE || p->gate_mode > VSA_GATE_PROJECTED)
    return fail(VSA_ERR_INVALID_ARG, "gate_mode must be NONE, PER_TOKEN, PER_ELEMENT or PROJECTED");
  if (p->gate_mode == VSA_GATE_PROJECTED && !p->gate_proj)
    return fail(VSA_ERR_INVALID_ARG, "gate_proj must be given with VSA_GATE_PROJECTED");
  if (p->gate_mode != VSA_GATE_PROJECTED && p->gate_proj)
    return fail(VSA_ERR_INVALID_ARG, "gate_proj is only read with VSA_GATE_PROJECTED (set it to NULL)");
  if (p->gate_proj && ((uintptr_t)p->gate_proj & 15u))
    return fail(VSA_ERR_INVALID_ARG, "gate_proj must be 16-byte aligned");
  if (p->map_batch_stride < 0) return fail(VSA_ERR_INVALID_ARG, "map_batch_stride must be >= 0");
  if (p->q_valid_batch_stride < 0 || p->kv_valid_batch_stride < 0)
    return fail(VSA_ERR_INVALID_ARG, "q_valid_batch_stride / kv_valid_batch_stride must be >= 0");
  if ((p->q_valid_batch_stride && !p->q_valid) || (p->kv_valid_batch_stride && !p->kv_valid))
    return fail(VSA_ERR_INVALID_ARG, "a valid-count batch stride needs the counts it strides");
  if ((p->q_valid_batch_stride && p->q_valid_batch_stride < p->Qb) ||
      (p->kv_valid_batch_stride && p->kv_valid_batch_stride < p->KVb))
    return fail(VSA_ERR_INVALID_ARG,
                "a valid-count batch stride must be 0 or at least Qb / KVb (got %lld / %lld)",
                (long long)p->q_valid_batch_stride, (long long)p->kv_valid_batch_stride);
  constexpr int kFlags = VSA_FLAG_ATOMIC_DQ | VSA_FLAG_PERSISTENT | VSA_FLAG_NO_PERSISTENT;
  if (p->flags & ~kFlags)
    return fail(VSA_ERR_INVALID_ARG, "flags: unknown bits 0x%x", p->flags & ~kFlags);
  if ((p->flags & VSA_FLAG_PERSISTENT) && (p->flags & VSA_FLAG_NO_PERSISTENT))
    return fail(VSA_ERR_INVALID_ARG, "flags: VSA_FLAG_PERSISTENT and VSA_FLAG_NO_PERSISTENT exclude each other");
  if (p->layout == VSA_TND) {
    if (!p->cu_seqlens_q) return fail(VSA_ERR_INVALID_ARG, "actual_seq_lengths must be specified");
    if (!p->cu_seqlens_kv)
      return fail(VSA_ERR_INVALID_ARG, "actual_seq_lengths_kv must be specified");
    if (p->max_seqlen_q < 0 || p->max_seqlen_kv < 0)
      return fail(VSA_ERR_INVALID_ARG, "max_seqlen_q / max_seqlen_kv must be >= 0");
    if (p->Qb != ceil_div(p->max_seqlen_q, p->q_block) || p->KVb != ceil_div(p->max_seqlen_kv, p->kv_block))
      return fail(VSA_ERR_INVALID_ARG,
                  "Qb/KVb must be ceil(max_seqlen/block): got %d/%d, want %lld/%lld", p->Qb, p->KVb,
                  ceil_div(p->max_seqlen_q, p->q_block), ceil_div(p->max_seqlen_kv, p->kv_block));
    if (p->topk > 0 || p->gate_mode != VSA_GATE_NONE)
      return fail(VSA_ERR_UNSUPPORTED, "top-k selection and the compression gate need BHSD or BSHD");
    if (p->q_valid || p->kv_valid)
      return fail(VSA_ERR_INVALID_ARG, "TND derives valid counts from the sequence lengths");
  } else {
    if (p->Qb != ceil_div(p->Sq, p->q_block) || p->KVb != ceil_div(p->Skv, p->kv_block))
      return fail(VSA_ERR_INVALID_ARG, "Qb/KVb must be ceil(S/block): got %d/%d, want %lld/%lld",
                  p->Qb, p->KVb, ceil_div(p->Sq, p->q_block), ceil_div(p->Skv, p->kv_block));
  }
  // tiles are staged with 24-bit row offsets: a row stride (heads x 256 B in the
  // token-major layouts) must stay below 2^24 bytes
  if (p->layout != VSA_BHSD && (p->Hq >= 65536 || p->Hkv >= 65536))
    return fail(VSA_ERR_UNSUPPORTED, "BSHD and TND need fewer than 65536 heads (Hq=%d Hkv=%d)",
                p->Hq, p->Hkv);
  if ((long long)p->B * p->Hq * p->Qb * std::max(p->KVb, 1) >= (1LL << 31))
    return fail(VSA_ERR_UNSUPPORTED, "B*Hq*Qb*KVb must stay below 2^31");
  if (rows_total(p) >= (1LL << 31)) return fail(VSA_ERR_UNSUPPORTED, "B*Hq*Sq must stay below 2^31");
  if (is_video(p) && vsa::coarse_rows_per_block(p->KVb) < 1)
    return fail(VSA_ERR_UNSUPPORTED, "KVb %d too large for the coarse kernels", p->KVb);
  if (p->gate_mode != VSA_GATE_NONE && vsa::coarse_bwd_lds(p->KVb) > 160 * 1024)
    return fail(VSA_ERR_UNSUPPORTED, "KVb %d too large for the compression backward", p->KVb);
  return VSA_OK;
}

// A pointer a kernel may dereference: device or managed memory, or pinned host
// memory with a device mapping. A plain host pointer (which would fault the
// GPU) is rejected here, before any launch.
bool device_accessible(const void* ptr) {
  hipPointerAttribute_t a{};
  const hipError_t e = hipPointerGetAttributes(&a, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // an unregistered pointer is an answer, not a pending error
    return false;
  }
  return a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged ||
         (a.type == hipMemoryTypeHost && a.devicePointer != nullptr);
}

struct Arg {
  const void* ptr;
  const char* name;
};

// every non-NULL pointer of a compute call, the problem's own ones included
int check_device(const vsa_problem* p, std::initializer_list<Arg> args) {
  const Arg own[] = {{p->q_valid, "q_valid"},
                     {p->kv_valid, "kv_valid"},
                     {p->cu_seqlens_q, "cu_seqlens_q"},
                     {p->cu_seqlens_kv, "cu_seqlens_kv"},
                     {p->gate_proj, "gate_proj"}};
  for (const Arg& a : own)
    if (a.ptr && !device_accessible(a.ptr))
      return fail(VSA_ERR_INVALID_ARG, "%s must be a device tensor", a.name);
  for (const Arg& a : args)
    if (a.ptr && !device_accessible(a.ptr))
      return fail(VSA_ERR_INVALID_ARG, "%s must be a device tensor", a.name);
  return VSA_OK;
}

// ---- head dimensions below HD -------------------------------------------------
// The kernels are built for D = HD. A problem with a smaller D runs them on
// copies whose rows are widened with zero columns: a zero column adds nothing
// to any score, pooled tile or coarse score, and the extra output columns are
// dropped, so every result equals that of the D-column problem (the softmax
// scale is an explicit parameter). The copies sit at the front of the caller's
// workspace, ahead of the widened problem's own workspace; the saved state is
// the widened problem's.
bool narrow(const vsa_problem* p) { return p->D < vsa::HD; }

vsa_problem widened(const vsa_problem* p) {
  vsa_problem w = *p;
  w.D = vsa::HD;
  w.gate_proj = nullptr;  // set to the widened copy by the caller
  return w;
}

long long rows_q(const vsa_problem* p) { return q_elems(p) / p->D; }
long long rows_kv(const vsa_problem* p) {
  return p->layout == VSA_TND ? (long long)p->Skv * p->Hkv : (long long)p->B * p->Skv * p->Hkv;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

struct PadBufs {
  uint16_t *q, *k, *v, *dout, *out, *gate, *dq, *dk, *dv, *dgate;
  float *theta, *dtheta;
};

// Widened copies: the forward needs q, k, v, out and a q-shaped gate or the
// projection; the backward also dout, out (O_sel without a gate), dq, dk, dv
// and dgate.
PadBufs carve_pad(const vsa_problem* p, bool bwd, void* base, size_t* bytes) {
  Carver c(base);
  PadBufs b{};
  const long long qn = rows_q(p) * vsa::HD, kn = rows_kv(p) * vsa::HD;
  const long long tn = (long long)p->Hq * vsa::HD + p->Hq;
  b.q = c.take<uint16_t>(qn);
  b.k = c.take<uint16_t>(kn);
  b.v = c.take<uint16_t>(kn);
  b.out = c.take<uint16_t>(qn);
  if (p->gate_mode == VSA_GATE_PER_ELEMENT) b.gate = c.take<uint16_t>(qn);
  if (p->gate_mode == VSA_GATE_PROJECTED) b.theta = c.take<float>(tn);
  if (bwd) {
    b.dout = c.take<uint16_t>(qn);
    b.dq = c.take<uint16_t>(qn);
    b.dk = c.take<uint16_t>(kn);
    b.dv = c.take<uint16_t>(kn);
    if (p->gate_mode == VSA_GATE_PER_ELEMENT) b.dgate = c.take<uint16_t>(qn);
    if (p->gate_mode == VSA_GATE_PROJECTED) b.dtheta = c.take<float>(tn);
  }
  if (bytes) *bytes = round256(c.off);
  return b;
}

size_t ws_fwd_bytes(const vsa_problem* p) {
  size_t inner = 0, pad = 0;
  if (!narrow(p)) {
    carve_fwd(p, nullptr, &inner);
    return inner;
  }
  const vsa_problem w = widened(p);
  carve_fwd(&w, nullptr, &inner);
  carve_pad(p, false, nullptr, &pad);
  return pad + inner;
}

size_t ws_bwd_bytes(const vsa_problem* p) {
  size_t inner = 0, pad = 0;
  if (!narrow(p)) {
    carve_bwd(p, nullptr, &inner);
    return inner;
  }
  const vsa_problem w = widened(p);
  carve_bwd(&w, nullptr, &inner);
  carve_pad(p, true, nullptr, &pad);
  return pad + inner;
}

size_t saved_bytes_of(const vsa_problem* p) {
  size_t s = 0;
  if (narrow(p)) {
    const vsa_problem w = widened(p);
    carve_saved(&w, nullptr, &s);
  } else {
    carve_saved(p, nullptr, &s);
  }
  return s;
}

// widen the projection [w (Hq x D) | b (Hq)] to [w (Hq x HD) | b]
hipError_t widen_theta(const vsa_problem* p, const float* src, float* dst, hipStream_t st) {
  hipError_t e = vsa::launch_widen_rows(src, dst, p->Hq, p->D, 4, st);
  if (e == hipSuccess) e = vsa::launch_copy_words(src + (long long)p->Hq * p->D, dst + (long long)p->Hq * vsa::HD, p->Hq, st);
  return e;
}

hipError_t narrow_theta(const vsa_problem* p, const float* src, float* dst, hipStream_t st) {
  hipError_t e = vsa::launch_narrow_rows(src, dst, p->Hq, p->D, 4, st);
  if (e == hipSuccess) e = vsa::launch_copy_words(src + (long long)p->Hq * vsa::HD, dst + (long long)p->Hq * p->D, p->Hq, st);
  return e;
}

int fwd_impl(const vsa_problem* p, const void* q, const void* k, const void* v, uint8_t* block_map,
             const void* gate, void* out, float* lse, void* saved, size_t saved_bytes, void* ws,
             size_t ws_bytes, void* stream, bool ws_scratch);

// The forward of a D < HD problem: widen, run the HD forward, narrow out.
int fwd_narrow(const vsa_problem* p, const void* q, const void* k, const void* v,
               uint8_t* block_map, const void* gate, void* out, float* lse, void* saved,
               size_t saved_bytes, void* ws, size_t ws_bytes, void* stream, bool ws_scratch) {
  const size_t need = ws_fwd_bytes(p);
  if (ws_bytes < need || !ws)
    return fail(VSA_ERR_WORKSPACE, "forward workspace: %zu bytes needed, %zu given", need, ws_bytes);
  if (int c = check_device(p, {{q, "q"}, {k, "k"}, {v, "v"}, {block_map, "block_map"}, {gate, "gate"},
                               {out, "out"}, {lse, "lse"}, {saved, "saved"},
                               {ws_scratch ? nullptr : ws, "ws"}}))
    return c;
  hipStream_t st = (hipStream_t)stream;
  size_t pad = 0;
  const PadBufs b = carve_pad(p, false, ws, &pad);
  const bool proj = p->gate_mode == VSA_GATE_PROJECTED;
  const bool elem = p->gate_mode == VSA_GATE_PER_ELEMENT;
  hipError_t e;
  {
    Prof pr(ws_scratch ? -1 : VSA_KERNEL_PAD, st);
    e = vsa::launch_widen_rows(q, b.q, rows_q(p), p->D, 2, st);
    if (e == hipSuccess) e = vsa::launch_widen_rows(k, b.k, rows_kv(p), p->D, 2, st);
    if (e == hipSuccess) e = vsa::launch_widen_rows(v, b.v, rows_kv(p), p->D, 2, st);
    if (e == hipSuccess && elem) e = vsa::launch_widen_rows(gate, b.gate, rows_q(p), p->D, 2, st);
    if (e == hipSuccess && proj) e = widen_theta(p, p->gate_proj, b.theta, st);
  }
  if (e != hipSuccess) return hip_fail(e, "widening the inputs");
  vsa_problem w = widened(p);
  w.gate_proj = b.theta;
  const int rc = fwd_impl(&w, b.q, b.k, b.v, block_map, elem ? b.gate : gate, b.out, lse, saved,
                          saved_bytes, (char*)ws + pad, ws_bytes - pad, stream, ws_scratch);
  if (rc != VSA_OK) return rc;
  {
    Prof pr(ws_scratch ? -1 : VSA_KERNEL_PAD, st);
    e = vsa::launch_narrow_rows(b.out, out, rows_q(p), p->D, 2, st);
  }
  if (e != hipSuccess) return hip_fail(e, "narrowing out");
  return ok();
}

// The forward launch sequence. ws_scratch: ws is the library's own scratch
// (the no-alloc entry point): it is not checked as a caller pointer, and no
// profiler events are recorded.
int fwd_impl(const vsa_problem* p, const void* q, const void* k, const void* v, uint8_t* block_map,
             const void* gate, void* out, float* lse, void* saved, size_t saved_bytes, void* ws,
             size_t ws_bytes, void* stream, bool ws_scratch) {
  int rc = validate(p);
  if (rc != VSA_OK) return rc;
  if (!q || !k || !v || !out || !lse)
    return fail(VSA_ERR_INVALID_ARG, "q, k, v, out and lse must be device buffers");
  if (p->topk == 0 && !block_map)
    return fail(VSA_ERR_INVALID_ARG, "block_map must be given when topk == 0");
  if (p->topk > 0 && block_map && p->map_batch_stride != (long long)p->Hq * p->Qb * p->KVb &&
      !(p->map_batch_stride == 0 && p->B == 1))
    return fail(VSA_ERR_INVALID_ARG, "an output block_map must be a dense [B,Hq,Qb,KVb] buffer");
  const bool proj = p->gate_mode == VSA_GATE_PROJECTED;
  if (p->gate_mode != VSA_GATE_NONE && !proj && !gate)
    return fail(VSA_ERR_INVALID_ARG, "gate must be given with a PER_TOKEN or PER_ELEMENT gate");
  if (narrow(p))
    return fwd_narrow(p, q, k, v, block_map, gate, out, lse, saved, saved_bytes, ws, ws_bytes, stream,
                      ws_scratch);
  size_t need_ws = 0, need_saved = 0;
  carve_fwd(p, nullptr, &need_ws);
  carve_saved(p, nullptr, &need_saved);
  if (ws_bytes < need_ws || (!ws && need_ws))
    return fail(VSA_ERR_WORKSPACE, "forward workspace: %zu bytes needed, %zu given", need_ws, ws_bytes);
  if (saved && saved_bytes < need_saved)
    return fail(VSA_ERR_WORKSPACE, "saved state: %zu bytes needed, %zu given", need_saved,
                saved_bytes);
  if (int c = check_device(p, {{q, "q"}, {k, "k"}, {v, "v"}, {block_map, "block_map"}, {gate, "gate"},
                               {out, "out"}, {lse, "lse"}, {saved, "saved"},
                               {ws_scratch ? nullptr : ws, "ws"}}))
    return c;
  hipStream_t st = (hipStream_t)stream;
  const FwdWs w = carve_fwd(p, ws, nullptr);
  const Saved s = saved ? carve_saved(p, saved, nullptr) : Saved{};
  vsa::Geom g = make_geom(p);
  hipError_t e = hipSuccess;
  const long long cap = nnz_cap(p);

  // pooled tiles, top-k selection and the coarse attention
  const bool gated = p->gate_mode != VSA_GATE_NONE;
  float* qc = (gated && saved) ? s.qc : w.qc;
  float* kc = (gated && saved) ? s.kc : w.kc;
  float* vc = (gated && saved) ? s.vc : w.vc;
  float* oc = (gated && saved) ? s.oc : w.oc;
  float* lse_c = (gated && saved) ? s.lse_c : w.lse_c;
  const uint8_t* sel_map = block_map;
  if (is_video(p)) {
    {
      Prof pr(ws_scratch ? -1 : VSA_KERNEL_POOL, st);
      e = vsa::launch_pool(g, p->dtype, q, k, v, qc, kc, vc, st);
    }
    if (e != hipSuccess) return hip_fail(e, "pool");
    vsa::CoarseArgs ca{};
    ca.g = g;
    ca.qc = qc;
    ca.kc = kc;
    ca.vc = vc;
    ca.topk = p->topk;
    ca.map = p->topk > 0 ? (block_map ? block_map : w.map) : nullptr;
    ca.oc = oc;
    ca.lse_c = lse_c;
    {
      Prof pr(ws_scratch ? -1 : VSA_KERNEL_COARSE_FWD, st);
      e = vsa::launch_coarse_fwd(ca, p->topk > 0, gated, st);
    }
    if (e != hipSuccess) return hip_fail(e, "coarse forward");
    if (p->topk > 0) {
      sel_map = ca.map;
      g.map_bstride = (long long)p->Hq * p->Qb * p->KVb;
    }
  }
  // index: Q-owned always, KV-owned only when a backward follows
  int32_t* q_rp = saved ? s.q_rp : w.q_rp;
  int32_t* q_col = saved ? s.q_col : w.q_col;
  {
    Prof pr(ws_scratch ? -1 : VSA_KERNEL_INDEX, st);
    e = saved ? vsa::launch_index_both(g, sel_map, q_rp, q_col, s.kv_rp, s.kv_col, cap, st)
              : vsa::launch_index(g, sel_map, 0, q_rp, q_col, cap, st);
  }
  if (e != hipSuccess) return hip_fail(e, "index");
  vsa::FwdArgs fa{};
  fa.g = g;
  fa.q = (const uint16_t*)q;
  fa.k = (const uint16_t*)k;
  fa.v = (const uint16_t*)v;
  fa.gate = proj ? nullptr : (const uint16_t*)gate;
  fa.oc = oc;
  fa.gate_mode = p->gate_mode;
  fa.gproj = p->gate_proj;
  fa.gate_out = proj ? (uint16_t*)const_cast<void*>(gate) : nullptr;
  fa.out = (uint16_t*)out;
  fa.osel = (gated && saved) ? s.osel : nullptr;
  fa.lse = lse;
  fa.row_ptr = q_rp;
  fa.col = q_col;
  {
    Prof pr(ws_scratch ? -1 : VSA_KERNEL_SPARSE_FWD, st);
    e = vsa::launch_sparse_fwd(fa, p->dtype, st);
  }
  if (e != hipSuccess) return hip_fail(e, "sparse forward");
  return ok();
}

// Compute units of the device that owns `st` (cached per device).
std::mutex g_cu_mu;
int g_cu_count[64] = {};
int compute_units(hipStream_t st, int* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (st) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(st, &sd);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    dev = (int)sd;
  }
  if (dev < 0 || dev >= 64) return fail(VSA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_cu_mu);
  if (!g_cu_count[dev]) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n < 1) return hip_fail(e, "compute unit count");
    g_cu_count[dev] = n;
  }
  *out = g_cu_count[dev];
  return VSA_OK;
}

// ---- scratch of the entry point that allocates nothing ----------------------
// A static device array (each GPU holds its own copy while the library is
// loaded). Its name is a host-side stand-in in host code: kernels get the
// device address looked up once per device with hipGetSymbolAddress.
constexpr size_t kScratchBytes = VSA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that owns `st` (which must be the current
// device: the launches go to `st`, the lookup to the current device).
int scratch_of_stream(hipStream_t st, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "vsa_fwd_noalloc: hipGetDevice");
  if (st) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(st, &sd);
    if (e != hipSuccess) return hip_fail(e, "vsa_fwd_noalloc: hipStreamGetDevice");
    if (sd != dev)
      return fail(VSA_ERR_INVALID_ARG, "vsa_fwd_noalloc: the stream belongs to device %d, the "
                  "current device is %d", (int)sd, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VSA_ERR_UNSUPPORTED, "vsa_fwd_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "vsa_fwd_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return VSA_OK;
}

}  // namespace

extern "C" {

const char* vsa_last_error(void) { return g_err.c_str(); }

int vsa_abi_version(void) { return VSA_ABI_VERSION; }

int vsa_validate(const vsa_problem* p) {
  const int rc = validate(p);
  return rc == VSA_OK ? ok() : rc;
}

int vsa_sizes(const vsa_problem* p, size_t* ws_fwd, size_t* ws_bwd, size_t* saved_bytes,
              int64_t* nnz_capacity) {
  const int rc = validate(p);
  if (rc != VSA_OK) return rc;
  const size_t f = ws_fwd_bytes(p), b = ws_bwd_bytes(p), s = saved_bytes_of(p);
  if (ws_fwd) *ws_fwd = f;
  if (ws_bwd) *ws_bwd = b;
  if (saved_bytes) *saved_bytes = s;
  if (nnz_capacity) *nnz_capacity = nnz_cap(p);
  return ok();
}

int block_map_to_index(const vsa_problem* p, const uint8_t* block_map, int kv_owned,
                       int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, void* ws,
                       size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  const int rc = validate(p);
  if (rc != VSA_OK) return rc;
  if (!block_map) return fail(VSA_ERR_INVALID_ARG, "block_map must be a device tensor (got NULL)");
  if (!row_ptr || (!col_idx && col_capacity > 0))
    return fail(VSA_ERR_INVALID_ARG, "row_ptr / col_idx must be device buffers");
  if (col_capacity < 0) return fail(VSA_ERR_INVALID_ARG, "col_capacity must be >= 0");
  if (int c = check_device(p, {{block_map, "block_map"}, {row_ptr, "row_ptr"}, {col_idx, "col_idx"}}))
    return c;
  const vsa::Geom g = make_geom(p);
  hipError_t e;
  {
    Prof pr(VSA_KERNEL_INDEX, (hipStream_t)stream);
    e = vsa::launch_index(g, block_map, kv_owned ? 1 : 0, row_ptr, col_idx, col_capacity,
                          (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "block_map_to_index");
  return ok();
}

int vsa_fwd(const vsa_problem* p, const void* q, const void* k, const void* v, uint8_t* block_map,
            const void* gate, void* out, float* lse, void* saved, size_t saved_bytes, void* ws,
            size_t ws_bytes, void* stream) {
  return fwd_impl(p, q, k, v, block_map, gate, out, lse, saved, saved_bytes, ws, ws_bytes, stream,
                  false);
}

int vsa_fwd_noalloc(const vsa_problem* p, const void* q, const void* k, const void* v,
                    uint8_t* block_map, const void* gate, void* out, float* lse, void* saved,
                    size_t saved_bytes, void* stream) {
  int rc = validate(p);
  if (rc != VSA_OK) return rc;
  const size_t need = ws_fwd_bytes(p);
  if (need > kScratchBytes)
    return fail(VSA_ERR_WORKSPACE,
                "vsa_fwd_noalloc: the forward workspace needs %zu bytes, more than its %zu-byte "
                "scratch (use vsa_fwd with a caller workspace)",
                need, kScratchBytes);
  if (!q || !k || !v || !out || !lse)
    return fail(VSA_ERR_INVALID_ARG, "q, k, v, out and lse must be device buffers");
  void* ws = nullptr;
  rc = scratch_of_stream((hipStream_t)stream, &ws);
  if (rc != VSA_OK) return rc;
  return fwd_impl(p, q, k, v, block_map, gate, out, lse, saved, saved_bytes, ws, kScratchBytes,
                  stream, true);
}

int vsa_bwd(const vsa_problem* p, const void* q, const void* k, const void* v, const void* gate,
            const void* dout, const void* out, const float* lse, const void* saved,
            size_t saved_bytes, void* dq, void* dk, void* dv, void* dgate, void* ws,
            size_t ws_bytes, void* stream) {
  int rc = validate(p);
  if (rc != VSA_OK) return rc;
  if (!q || !k || !v || !lse || !dq || !dk || !dv)
    return fail(VSA_ERR_INVALID_ARG, "q, k, v, lse, dq, dk and dv must be device buffers");
  if (!saved) return fail(VSA_ERR_INVALID_ARG, "saved must be the state of a training vsa_fwd");
  const bool gated = p->gate_mode != VSA_GATE_NONE;
  const bool proj = p->gate_mode == VSA_GATE_PROJECTED;
  if (gated && !proj && !gate)
    return fail(VSA_ERR_INVALID_ARG, "gate must be given with a PER_TOKEN or PER_ELEMENT gate");
  if (proj) gate = nullptr;  // the library recomputes it from q and gate_proj
  if (!gated && !out && dout) return fail(VSA_ERR_INVALID_ARG, "out must be given");
  if (narrow(p)) {  // D < HD: widen, run the HD backward, narrow the gradients
    const size_t need = ws_bwd_bytes(p), need_sv = saved_bytes_of(p);
    if (saved_bytes < need_sv)
      return fail(VSA_ERR_WORKSPACE, "saved state: %zu bytes needed, %zu given", need_sv, saved_bytes);
    if (ws_bytes < need || !ws)
      return fail(VSA_ERR_WORKSPACE, "backward workspace: %zu bytes needed, %zu given", need, ws_bytes);
    if (int c = check_device(p, {{q, "q"}, {k, "k"}, {v, "v"}, {gate, "gate"}, {dout, "dout"},
                                 {out, "out"}, {lse, "lse"}, {saved, "saved"}, {dq, "dq"},
                                 {dk, "dk"}, {dv, "dv"}, {dgate, "dgate"}, {ws, "ws"}}))
      return c;
    hipStream_t st = (hipStream_t)stream;
    size_t pad = 0;
    const PadBufs b = carve_pad(p, true, ws, &pad);
    const bool elem = p->gate_mode == VSA_GATE_PER_ELEMENT;
    const bool with_out = !gated && out;  // the row term reads O_sel = out
    hipError_t e;
    {
      Prof pr(VSA_KERNEL_PAD, st);
      e = vsa::launch_widen_rows(q, b.q, rows_q(p), p->D, 2, st);
      if (e == hipSuccess) e = vsa::launch_widen_rows(k, b.k, rows_kv(p), p->D, 2, st);
      if (e == hipSuccess) e = vsa::launch_widen_rows(v, b.v, rows_kv(p), p->D, 2, st);
      if (e == hipSuccess && dout) e = vsa::launch_widen_rows(dout, b.dout, rows_q(p), p->D, 2, st);
      if (e == hipSuccess && with_out) e = vsa::launch_widen_rows(out, b.out, rows_q(p), p->D, 2, st);
      if (e == hipSuccess && elem) e = vsa::launch_widen_rows(gate, b.gate, rows_q(p), p->D, 2, st);
      if (e == hipSuccess && proj) e = widen_theta(p, p->gate_proj, b.theta, st);
    }
    if (e != hipSuccess) return hip_fail(e, "widening the inputs");
    vsa_problem w = widened(p);
    w.gate_proj = b.theta;
    void* wdg = elem ? (dgate ? (void*)b.dgate : nullptr)
                     : proj ? (dgate ? (void*)b.dtheta : nullptr) : dgate;  // per-token: as is
    rc = vsa_bwd(&w, b.q, b.k, b.v, elem ? b.gate : gate, dout ? b.dout : nullptr,
                 with_out ? b.out : nullptr, lse, saved, saved_bytes, b.dq, b.dk, b.dv, wdg,
                 (char*)ws + pad, ws_bytes - pad, stream);
    if (rc != VSA_OK) return rc;
    {
      Prof pr(VSA_KERNEL_PAD, st);
      e = vsa::launch_narrow_rows(b.dq, dq, rows_q(p), p->D, 2, st);
      if (e == hipSuccess) e = vsa::launch_narrow_rows(b.dk, dk, rows_kv(p), p->D, 2, st);
      if (e == hipSuccess) e = vsa::launch_narrow_rows(b.dv, dv, rows_kv(p), p->D, 2, st);
      if (e == hipSuccess && elem && dgate)
        e = vsa::launch_narrow_rows(b.dgate, dgate, rows_q(p), p->D, 2, st);
      if (e == hipSuccess && proj && dgate) e = narrow_theta(p, b.dtheta, (float*)dgate, st);
    }
    if (e != hipSuccess) return hip_fail(e, "narrowing the gradients");
    return ok();
  }
  size_t need_ws = 0, need_saved = 0;
  carve_bwd(p, nullptr, &need_ws);
  carve_saved(p, nullptr, &need_saved);
  if (saved_bytes < need_saved)
    return fail(VSA_ERR_WORKSPACE, "saved state: %zu bytes needed, %zu given", need_saved, saved_bytes);
  if (ws_bytes < need_ws || (!ws && need_ws))
    return fail(VSA_ERR_WORKSPACE, "backward workspace: %zu bytes needed, %zu given", need_ws, ws_bytes);
  if (int c = check_device(p, {{q, "q"}, {k, "k"}, {v, "v"}, {gate, "gate"}, {dout, "dout"},
                               {out, "out"}, {lse, "lse"}, {saved, "saved"}, {dq, "dq"}, {dk, "dk"},
                               {dv, "dv"}, {dgate, "dgate"}, {ws, "ws"}}))
    return c;
  hipStream_t st = (hipStream_t)stream;
  const long long qn = q_elems(p);
  const long long kn = p->layout == VSA_TND ? (long long)p->Skv * p->Hkv * p->D
                                            : (long long)p->B * p->Skv * p->Hkv * p->D;
  hipError_t e = hipSuccess;
  if (!dout) {  // no upstream gradient: every gradient is zero
    e = vsa::launch_zero(dq, (size_t)qn * 2, st);
    if (e == hipSuccess) e = vsa::launch_zero(dk, (size_t)kn * 2, st);
    if (e == hipSuccess) e = vsa::launch_zero(dv, (size_t)kn * 2, st);
    if (e == hipSuccess && gated && dgate)
      e = vsa::launch_zero(dgate,
                           proj ? (size_t)((long long)p->Hq * p->D + p->Hq) * sizeof(float)
                                : (size_t)(p->gate_mode == VSA_GATE_PER_TOKEN ? qn / p->D : qn) * 2,
                           st);
    if (e != hipSuccess) return hip_fail(e, "zero gradients");
    return ok();
  }
  const Saved s = carve_saved(p, const_cast<void*>(saved), nullptr);
  const BwdWs w = carve_bwd(p, ws, nullptr);
  const vsa::Geom g = make_geom(p);

  vsa::PreArgs pa{};
  pa.g = g;
  pa.q = (const uint16_t*)q;
  pa.dout = (const uint16_t*)dout;
  pa.osel = gated ? s.osel : (const uint16_t*)out;
  pa.gate = (const uint16_t*)gate;
  pa.oc = s.oc;
  pa.gate_mode = p->gate_mode;
  pa.lse = lse;
  pa.dr = w.dr;
  pa.lse2 = w.lse2;
  pa.doc = w.doc;
  pa.dgate = proj ? nullptr : (uint16_t*)dgate;
  pa.qlive = w.qlive;
  pa.gproj = p->gate_proj;
  pa.dlogit = w.dlogit;
  pa.dwp = w.dwp;
  pa.dbp = w.dbp;
  {
    Prof pr(VSA_KERNEL_BWD_PRE, st);
    e = vsa::launch_bwd_pre(pa, p->dtype, st);
    if (e == hipSuccess && proj && dgate)
      e = vsa::launch_gate_proj_grad(g, w.dwp, w.dbp, (float*)dgate, st);
  }
  if (e != hipSuccess) return hip_fail(e, "backward preprocess");

  if (gated) {
    vsa::CoarseArgs ca{};
    ca.g = g;
    ca.qc = s.qc;
    ca.kc = s.kc;
    ca.vc = s.vc;
    ca.lse_c = s.lse_c;
    ca.doc = w.doc;
    ca.ps = w.ps;
    ca.dss = w.dss;
    ca.csum = w.csum;
    ca.dqc = w.dqc;
    ca.dkc = w.dkc;
    ca.dvc = w.dvc;
    {
      Prof pr(VSA_KERNEL_COARSE_BWD, st);
      e = vsa::launch_coarse_bwd(ca, st);
    }
    if (e != hipSuccess) return hip_fail(e, "coarse backward");
  }

  vsa::BwdArgs ba{};
  ba.g = g;
  ba.q = (const uint16_t*)q;
  ba.k = (const uint16_t*)k;
  ba.v = (const uint16_t*)v;
  ba.dout = (const uint16_t*)dout;
  ba.lse2 = w.lse2;
  ba.dr = w.dr;
  ba.qlive = w.qlive;
  ba.dqc = gated ? w.dqc : nullptr;
  ba.dkc = gated ? w.dkc : nullptr;
  ba.dvc = gated ? w.dvc : nullptr;
  ba.gproj = p->gate_proj;
  ba.dlogit = w.dlogit;
  ba.dq = (uint16_t*)dq;
  ba.dk = (uint16_t*)dk;
  ba.dv = (uint16_t*)dv;
  ba.row_ptr = s.kv_rp;
  ba.col = s.kv_col;
  const bool atomic_dq = (p->flags & VSA_FLAG_ATOMIC_DQ) != 0;
  ba.dqacc = atomic_dq ? w.dqacc : nullptr;
  int cus = 0;
  rc = compute_units((hipStream_t)stream, &cus);
  if (rc != VSA_OK) return rc;
  // work items of 256 keys; of 64 when even those fit on the compute units at
  // once (one work-group per CU): a small problem's dK/dV time is then the
  // length of one item's walk, which is shorter for fewer keys
  ba.span = (g.kv_block > vsa::DKDV_SPAN_MIN && vsa::dkdv_items(g, vsa::DKDV_SPAN_MIN) <= cus)
                ? vsa::DKDV_SPAN_MIN : vsa::DKDV_SPAN;
  const bool persistent =
      !(p->flags & VSA_FLAG_NO_PERSISTENT) &&
      ((p->flags & VSA_FLAG_PERSISTENT) ||
       vsa::dkdv_items(g, ba.span) >= (long long)VSA_PERSISTENT_MIN_SPANS_PER_CU * cus);
  if (persistent) {  // longest-first list of the dK/dV spans
    ba.n_items = (int)vsa::dkdv_items(g, ba.span);
    ba.persist_grid = cus;
    const long long nh = vsa::lpt_hist_entries(g);
    Prof pr(VSA_KERNEL_DKDV_ORDER, st);
    ba.lpt_counter = w.lpt_hist + (nh - 1);
    if (!vsa::lpt_order_small(g, ba.span))  // the one-launch order clears the counter itself
      e = vsa::launch_zero(w.lpt_hist, (size_t)nh * sizeof(int32_t), st);
    if (e == hipSuccess) e = vsa::launch_lpt_order(ba, w.lpt_hist, w.lpt_order, st);
    if (e != hipSuccess) return hip_fail(e, "dK/dV order");
    ba.lpt_order = w.lpt_order;
  }
  if (atomic_dq) {  // the accumulator starts at zero (a fill kernel: safe under graph capture)
    Prof pr(VSA_KERNEL_DQ_ATOMIC, st);
    e = vsa::launch_zero(w.dqacc, (size_t)qn * sizeof(float), st);
    if (e != hipSuccess) return hip_fail(e, "dQ accumulator clear");
  }
  {
    Prof pr(VSA_KERNEL_SPARSE_DKDV, st);
    e = vsa::launch_sparse_dkdv(ba, p->dtype, st);
  }
  if (e != hipSuccess) return hip_fail(e, "dK/dV");
  if (atomic_dq) {
    Prof pr(VSA_KERNEL_DQ_ATOMIC, st);
    e = vsa::launch_dq_cast(ba, p->dtype, st);
    if (e != hipSuccess) return hip_fail(e, "dQ cast");
    return ok();
  }
  ba.row_ptr = s.q_rp;
  ba.col = s.q_col;
  {
    Prof pr(VSA_KERNEL_SPARSE_DQ, st);
    e = vsa::launch_sparse_dq(ba, p->dtype, st);
  }
  if (e != hipSuccess) return hip_fail(e, "dQ");
  return ok();
}

int vsa_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_recs.clear();
  g_prof_recs.reserve(kProfMax);
  g_prof_on = true;
  return ok();
}

int vsa_profile_end(double* ms_total, int64_t* launches, int n) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = false;
  for (int k = 0; k < n; ++k) {
    if (ms_total) ms_total[k] = 0.0;
    if (launches) launches[k] = 0;
  }
  for (const ProfRec& r : g_prof_recs) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "vsa_profile_end");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "vsa_profile_end");
    if (r.kid < n) {
      if (ms_total) ms_total[r.kid] += ms;
      if (launches) launches[r.kid] += 1;
    }
  }
  g_prof_recs.clear();
  return ok();
}

}  // extern "C"
