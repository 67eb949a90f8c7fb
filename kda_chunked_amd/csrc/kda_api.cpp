// Host side of the C ABI declared in include/kda.h: argument validation,
// buffer sizing, workspace carving and the stream-ordered launch sequence.
// Nothing here reads device memory or synchronises with the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "kda.h"
#include "kda_state.h"
#include "kda_internal.h"

namespace {
// Message of the calling thread's last failed call (plain storage: no
// dynamic initialisation or destructor in the thread-local block).
thread_local char g_last_error[512];
}  // namespace

namespace kda {
kda_status fail(kda_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}
}  // namespace kda

namespace {
using kda::fail;

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sequential carving of a byte buffer into aligned regions.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += up(count * sizeof(T));
    return p;
  }
};

struct Sizes {
  int64_t T, H, N, NC;
  int64_t L, NS;    // segment length (chunks; 0: whole documents), segment upper bound
};

// Segment length of the segment-parallel scans, from sizes the host knows
// (document lengths stay on the device). With few chains (documents x heads x
// 4 column tiles well below the 256 compute units) and documents that average
// at least two segments, each document is cut into segments of L chunks,
// about 64 chains over the heads, at least 16 chunks long; otherwise 0 (one
// chain per document: the summaries and walks would cost more than they save).
int64_t seg_len(int64_t T, int64_t H, int64_t N) {
  const int64_t NC = T / 64 + N;
  if (N * H * 4 >= 192) return 0;
  int64_t L = (NC * H + 63) / 64;
  if (L < 16) L = 16;
  return 2 * L * N > NC ? 0 : L;
}

Sizes sizes_of(const kda_problem* p) {
  Sizes s;
  s.T = p->T;
  s.H = p->H;
  s.N = p->num_seqs;
  s.NC = p->T / 64 + p->num_seqs;
  s.L = seg_len(s.T, s.H, s.N);
  // document d has ceil(n_d / L) <= n_d / L + 1 segments
  s.NS = s.L > 0 ? s.NC / s.L + s.N : s.N;
  return s;
}

kda::ChunkTable carve_table(Carver& c, const Sizes& s) {
  kda::ChunkTable ct;
  ct.doc_c0 = c.take<int32_t>(s.N + 1);
  ct.tok = c.take<int32_t>(s.NC);
  ct.len = c.take<int32_t>(s.NC);
  ct.seg_doc0 = c.take<int32_t>(s.N + 1);
  ct.seg_doc = c.take<int32_t>(s.NS);
  return ct;
}

// One fp32 128 x 128 matrix per (segment, head).
float* take_seg(Carver& c, const Sizes& s) { return c.take<float>((size_t)s.NS * s.H * 128 * 128); }

// The saved forward set: per-chunk matrices, L2 scalars, states and panels.
kda::SavedSet carve_saved(Carver& c, const Sizes& s) {
  kda::SavedSet sv{};
  const size_t mat = (size_t)s.NC * s.H * 64 * 64;
  sv.Tm = c.take<float>(mat);
  sv.Akk = c.take<float>(mat);
  sv.rq = c.take<float>((size_t)s.T * s.H);
  sv.rk = c.take<float>((size_t)s.T * s.H);
  sv.S_in = c.take<float>((size_t)s.NC * s.H * 128 * 128);
  sv.R = c.take<float>((size_t)s.NC * s.H * 64 * 128);
  sv.U = c.take<float>((size_t)s.NC * s.H * 64 * 128);
  sv.panels = c.take<uint16_t>((size_t)s.NC * s.H * kda::fwd_panel::ELEMS);
  sv.Mseg = s.L > 0 ? take_seg(c, s) : nullptr;
  return sv;
}

// What the prep writes (the state summaries store nothing per chunk beyond it).
kda::SavedSet carve_prep(Carver& c, const Sizes& s) {
  kda::SavedSet sv{};
  const size_t mat = (size_t)s.NC * s.H * 64 * 64;
  sv.Tm = c.take<float>(mat);
  sv.Akk = c.take<float>(mat);
  sv.rq = c.take<float>((size_t)s.T * s.H);
  sv.rk = c.take<float>((size_t)s.T * s.H);
  sv.panels = c.take<uint16_t>((size_t)s.NC * s.H * kda::fwd_panel::ELEMS);
  return sv;
}

kda::BwdWork carve_bwd(Carver& c, const Sizes& s) {
  kda::BwdWork bw;
  bw.dS = c.take<float>((size_t)s.NC * s.H * 128 * 128);
  bw.dU = c.take<float>((size_t)s.NC * s.H * 64 * 128);
  bw.part_A = c.take<float>((size_t)s.NC * s.H);
  bw.part_dt = c.take<float>((size_t)s.NC * s.H * 128);
  return bw;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

kda_status check_problem(const kda_problem* p) {
  if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "T = %lld is negative", (long long)p->T);
  if (p->T > (int64_t)1 << 30)
    return fail(KDA_ERR_INVALID_ARGUMENT, "T = %lld exceeds 2^30 tokens", (long long)p->T);
  if (p->H < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "H = %d: need at least one head", p->H);
  if (p->num_seqs < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs = %d: need at least one document",
                p->num_seqs);
  if (p->num_seqs > (1 << 24))
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs = %d is too large", p->num_seqs);
  if (p->H > 65535)
    return fail(KDA_ERR_UNSUPPORTED, "H = %d exceeds 65535 heads (a launch grid dimension)",
                p->H);
  {
    // the scans launch one workgroup per (document, head, column tile), with
    // the pairs rounded up to a multiple of 8: 4 * ceil8(N * H) must fit an int
    const int64_t pairs = (int64_t)p->num_seqs * p->H;
    if (4 * ((pairs + 7) / 8 * 8) >= ((int64_t)1 << 31))
      return fail(KDA_ERR_UNSUPPORTED, "num_seqs * H = %lld (document, head) pairs exceeds 2^29",
                  (long long)pairs);
  }
  {
    // the per-chunk backward launches one workgroup per (chunk, head)
    const int64_t chunk_heads = (p->T / 64 + p->num_seqs) * (int64_t)p->H;
    if (chunk_heads >= ((int64_t)1 << 31))
      return fail(KDA_ERR_UNSUPPORTED, "%lld (chunk, head) pairs exceed 2^31 workgroups",
                  (long long)chunk_heads);
  }
  if (p->dk != 128 || p->dv != 128)
    return fail(KDA_ERR_UNSUPPORTED, "dk = %d, dv = %d: this build serves 128, 128", p->dk,
                p->dv);
  if (p->gate != KDA_GATE_G && p->gate != KDA_GATE_RAW)
    return fail(KDA_ERR_INVALID_ARGUMENT, "unknown gate form %d", p->gate);
  if (p->l2norm != 0 && p->l2norm != 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "l2norm must be 0 or 1, got %d", p->l2norm);
  if (!std::isfinite(p->scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (!std::isfinite(p->l2_eps) || p->l2_eps < 0.f)
    return fail(KDA_ERR_INVALID_ARGUMENT, "l2_eps must be finite and >= 0");
  return KDA_OK;
}

#define REQUIRE_PTR(ptr, name)                                                         \
  do {                                                                                 \
    if (!(ptr)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", name);             \
    if (!aligned(ptr)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
  } while (0)

kda::Dims dims_of(const kda_problem* p) {
  kda::Dims d;
  d.T = p->T;
  d.H = p->H;
  d.N = p->num_seqs;
  d.NC = (int)(p->T / 64 + p->num_seqs);
  const Sizes s = sizes_of(p);
  d.L = (int)s.L;
  d.NS = (int)s.NS;
  d.raw = p->gate == KDA_GATE_RAW;
  d.l2norm = p->l2norm;
  d.scale = p->scale;
  d.l2_eps = p->l2_eps;
  return d;
}

// Segment summaries and walk results. The forward takes B and S0 (M lives in
// the saved set); the backward B' and D0, which a replay also lends to its
// forward as B and S0 (the forward is done with them before the backward's
// summary pass writes B').
kda::SegWork carve_seg_fwd(Carver& c, const Sizes& s, const kda::SavedSet& sv) {
  kda::SegWork sg{};
  if (s.L > 0) {
    sg.M = sv.Mseg;
    sg.B = take_seg(c, s);
    sg.S0 = take_seg(c, s);
  }
  return sg;
}
kda::SegWork carve_seg_bwd(Carver& c, const Sizes& s, const kda::SavedSet& sv) {
  kda::SegWork sg{};
  if (s.L > 0) {
    sg.M = sv.Mseg;
    sg.Brev = take_seg(c, s);
    sg.D0 = take_seg(c, s);
    sg.B = sg.Brev;
    sg.S0 = sg.D0;
  }
  return sg;
}

// A forward that saves nothing keeps its per-chunk set in the workspace.
size_t fwd_ws_bytes(const Sizes& s, int nosave) {
  Carver c(nullptr);
  carve_table(c, s);
  kda::SavedSet sv{};
  if (nosave) sv = carve_saved(c, s);
  carve_seg_fwd(c, s, sv);
  return c.off;
}

size_t bwd_ws_bytes(const Sizes& s, int replay) {
  Carver c(nullptr);
  carve_table(c, s);
  carve_bwd(c, s);
  kda::SavedSet sv{};
  if (replay) sv = carve_saved(c, s);
  carve_seg_bwd(c, s, sv);
  return c.off;
}

kda_launch_hook g_hook = nullptr;
void* g_hook_user = nullptr;

#define LAUNCH(name, call)                                                              \
  do {                                                                                  \
    if (g_hook) g_hook(g_hook_user, name, 0, hs);                                       \
    hipError_t e_ = (call);                                                             \
    if (g_hook) g_hook(g_hook_user, name, 1, hs);                                       \
    if (e_ != hipSuccess)                                                               \
      return fail(KDA_ERR_DEVICE, "%s failed: %s", #call, hipGetErrorString(e_));       \
  } while (0)

}  // namespace

extern "C" {

size_t kda_saved_bytes(const kda_problem* p) {
  if (check_problem(p) != KDA_OK) return 0;
  Carver c(nullptr);
  carve_saved(c, sizes_of(p));
  return c.off;
}

size_t kda_workspace_bytes(const kda_problem* p, int backward, int replay) {
  if (check_problem(p) != KDA_OK) return 0;
  const Sizes s = sizes_of(p);
  return backward ? bwd_ws_bytes(s, replay != 0) : fwd_ws_bytes(s, replay != 0);
}

}  // extern "C"

namespace {

#define OPT_PTR(ptr, name)                                                               \
  do {                                                                                   \
    if ((ptr) && !aligned(ptr))                                                          \
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);          \
  } while (0)

// kda_fwd and kda_fwd_state: s_init, s_final as in kda_fwd_state (nullable).
kda_status fwd_impl(const kda_problem* p, const void* q, const void* k, const void* v,
                    const void* beta, const void* g_or_a, const float* A_log,
                    const float* dt_bias, const int32_t* cu_seqlens, const float* s_init,
                    void* o, float* s_final, void* saved, int flags, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  OPT_PTR(s_init, "s_init");
  OPT_PTR(s_final, "s_final");
  if (flags & ~KDA_FWD_PREP_DONE) return fail(KDA_ERR_INVALID_ARGUMENT, "unknown flags %d", flags);
  const bool prep_done = (flags & KDA_FWD_PREP_DONE) != 0;
  if (prep_done && !saved)
    return fail(KDA_ERR_INVALID_ARGUMENT, "KDA_FWD_PREP_DONE needs the saved set");
  if (p->T == 0) {
    // no tokens: the last document is empty; it is document 0 (entering
    // with s_init) only when there is one document
    if (s_final) {
      hipStream_t hs = static_cast<hipStream_t>(stream);
      LAUNCH("fill_states", kda::launch_fill_states(p->H, s_final, s_init,
                                                    p->num_seqs == 1 ? kda::FILL_COPY
                                                                     : kda::FILL_ZERO, hs));
    }
    return KDA_OK;
  }
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(beta, "beta");
  REQUIRE_PTR(g_or_a, "g_or_a");
  REQUIRE_PTR(cu_seqlens, "cu_seqlens");
  REQUIRE_PTR(o, "o");
  if (p->gate == KDA_GATE_RAW) {
    REQUIRE_PTR(A_log, "A_log");
    REQUIRE_PTR(dt_bias, "dt_bias");
  }
  if (saved && !aligned(saved)) return fail(KDA_ERR_INVALID_ARGUMENT, "saved is not 16-byte aligned");
  REQUIRE_PTR(workspace, "workspace");
  const Sizes s = sizes_of(p);
  const size_t need = fwd_ws_bytes(s, saved == nullptr);
  if (workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                workspace_bytes, need);

  const kda::Dims d = dims_of(p);
  const kda::Inputs in{q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens};
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carver wc(workspace);
  const kda::ChunkTable ct = carve_table(wc, s);
  kda::SavedSet sv;
  if (saved) {
    Carver sc(saved);
    sv = carve_saved(sc, s);
  } else {
    sv = carve_saved(wc, s);   // private per-chunk set in the workspace
  }
  kda::SegWork sg = carve_seg_fwd(wc, s, sv);
  sg.s_init = s_init;
  sg.s_final = s_final;
  LAUNCH("chunk_map", kda::launch_chunk_map(d, cu_seqlens, ct, hs));
  LAUNCH("seg_map", kda::launch_seg_map(d, ct, hs));
  if (!prep_done) LAUNCH("fwd_prep", kda::launch_fwd_prep(d, in, ct, sv, saved != nullptr, hs));
  // an empty last document has no chain when documents are cut into
  // segments: its leaving state is the zero it starts from
  if (s_final) LAUNCH("fill_states", kda::launch_fill_states(p->H, s_final, nullptr, kda::FILL_ZERO, hs));
  if (d.L > 0) {
    LAUNCH("fwd_scan_summary", kda::launch_fwd_scan(d, in, ct, sv, sv.panels, 0, sg,
                                                    kda::SCAN_SUMMARY, hs));
    LAUNCH("walk", kda::launch_walk(d, ct, sg, 0, hs));
  }
  LAUNCH("fwd_scan", kda::launch_fwd_scan(d, in, ct, sv, sv.panels, saved != nullptr, sg,
                                          kda::SCAN_FINISH, hs));
  LAUNCH("fwd_out", kda::launch_fwd_out(d, ct, sv, sv.panels, o, hs));
  return KDA_OK;
}

// kda_bwd and kda_bwd_state: s_init, ds_final, ds_init as in kda_bwd_state.
kda_status bwd_impl(const kda_problem* p, const void* q, const void* k, const void* v,
                    const void* beta, const void* g_or_a, const float* A_log,
                    const float* dt_bias, const int32_t* cu_seqlens, const float* s_init,
                    const void* dO, const float* ds_final, const void* saved, void* dq,
                    void* dk, void* dv, void* dbeta, void* dg_or_da, float* dA_log,
                    float* ddt_bias, float* ds_init, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_last_error[0] = 0;
  kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  OPT_PTR(s_init, "s_init");
  OPT_PTR(ds_final, "ds_final");
  OPT_PTR(ds_init, "ds_init");
  if (p->T == 0) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // no tokens: the raw form's parameter gradients are sums over nothing
    if (p->gate == KDA_GATE_RAW) {
      REQUIRE_PTR(dA_log, "dA_log");
      REQUIRE_PTR(ddt_bias, "ddt_bias");
      const kda::Dims d = dims_of(p);
      LAUNCH("zero_params", kda::launch_zero_params(d, dA_log, ddt_bias, hs));
    }
    // the state passes through an empty document 0 only when it is the last
    if (ds_init)
      LAUNCH("fill_states", kda::launch_fill_states(p->H, ds_init, ds_final,
                                                    p->num_seqs == 1 ? kda::FILL_COPY
                                                                     : kda::FILL_ZERO, hs));
    return KDA_OK;
  }
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(beta, "beta");
  REQUIRE_PTR(g_or_a, "g_or_a");
  REQUIRE_PTR(cu_seqlens, "cu_seqlens");
  REQUIRE_PTR(dO, "dO");
  REQUIRE_PTR(dq, "dq");
  REQUIRE_PTR(dk, "dk");
  REQUIRE_PTR(dv, "dv");
  REQUIRE_PTR(dbeta, "dbeta");
  REQUIRE_PTR(dg_or_da, "dg_or_da");
  if (p->gate == KDA_GATE_RAW) {
    REQUIRE_PTR(A_log, "A_log");
    REQUIRE_PTR(dt_bias, "dt_bias");
    REQUIRE_PTR(dA_log, "dA_log");
    REQUIRE_PTR(ddt_bias, "ddt_bias");
  }
  if (saved && !aligned(saved)) return fail(KDA_ERR_INVALID_ARGUMENT, "saved is not 16-byte aligned");
  REQUIRE_PTR(workspace, "workspace");
  const Sizes s = sizes_of(p);
  const int replay = saved == nullptr;
  const size_t need = bwd_ws_bytes(s, replay);
  if (workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                workspace_bytes, need);

  const kda::Dims d = dims_of(p);
  const kda::Inputs in{q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens};
  hipStream_t hs = static_cast<hipStream_t>(stream);
  Carver wc(workspace);
  const kda::ChunkTable ct = carve_table(wc, s);
  const kda::BwdWork bw = carve_bwd(wc, s);
  kda::SavedSet sv;
  if (replay) {
    sv = carve_saved(wc, s);
  } else {
    Carver sc(const_cast<void*>(saved));
    sv = carve_saved(sc, s);
  }
  const kda::BwdOut out{dq, dk, dv, dbeta, dg_or_da, dA_log, ddt_bias};
  kda::SegWork sg = carve_seg_bwd(wc, s, sv);
  sg.s_init = s_init;
  sg.ds_final = ds_final;
  sg.ds_init = ds_init;
  LAUNCH("chunk_map", kda::launch_chunk_map(d, cu_seqlens, ct, hs));
  LAUNCH("seg_map", kda::launch_seg_map(d, ct, hs));
  // an empty document 0 has no chain when documents are cut into segments
  if (ds_init) LAUNCH("fill_states", kda::launch_fill_states(p->H, ds_init, nullptr, kda::FILL_ZERO, hs));
  if (replay) {
    LAUNCH("fwd_prep", kda::launch_fwd_prep(d, in, ct, sv, 1, hs));
    if (d.L > 0) {
      LAUNCH("fwd_scan_summary", kda::launch_fwd_scan(d, in, ct, sv, sv.panels, 0, sg,
                                                      kda::SCAN_SUMMARY, hs));
      LAUNCH("walk", kda::launch_walk(d, ct, sg, 0, hs));
    }
    LAUNCH("fwd_scan", kda::launch_fwd_scan(d, in, ct, sv, sv.panels, 1, sg, kda::SCAN_FINISH,
                                            hs));
  }
  if (d.L > 0) {
    LAUNCH("bwd_scan_summary", kda::launch_bwd_scan(d, in, ct, sv, dO, dv, bw, sg,
                                                    kda::SCAN_SUMMARY, hs));
    LAUNCH("walk_rev", kda::launch_walk(d, ct, sg, 1, hs));
  }
  LAUNCH("bwd_scan", kda::launch_bwd_scan(d, in, ct, sv, dO, dv, bw, sg, kda::SCAN_FINISH, hs));
  LAUNCH("bwd_intra", kda::launch_bwd_intra(d, in, ct, sv, dO, out, bw, hs));
  if (p->gate == KDA_GATE_RAW) LAUNCH("finalize", kda::launch_finalize(d, ct, out, bw, hs));
  return KDA_OK;
}

// The state summaries' workspace: their own chunk table and the prep's
// outputs, with the documents never cut into segments.
Sizes map_sizes(const kda_problem* p) {
  Sizes s = sizes_of(p);
  s.L = 0;
  s.NS = s.N;
  return s;
}

size_t table_bytes(const Sizes& s) {
  Carver c(nullptr);
  carve_table(c, s);
  return c.off;
}

size_t map_ws_bytes(const Sizes& s) {
  Carver c(nullptr);
  carve_table(c, s);
  carve_prep(c, s);
  return c.off;
}

kda::Dims map_dims(const kda_problem* p) {
  kda::Dims d = dims_of(p);
  d.L = 0;
  d.NS = d.N;
  return d;
}

}  // namespace

extern "C" {

kda_status kda_fwd(const kda_problem* p, const void* q, const void* k, const void* v,
                   const void* beta, const void* g_or_a, const float* A_log,
                   const float* dt_bias, const int32_t* cu_seqlens, void* o, void* saved,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, nullptr, o, nullptr,
                  saved, 0, workspace, workspace_bytes, stream);
}

kda_status kda_fwd_state(const kda_problem* p, const void* q, const void* k, const void* v,
                         const void* beta, const void* g_or_a, const float* A_log,
                         const float* dt_bias, const int32_t* cu_seqlens, const float* s_init,
                         void* o, float* s_final, void* saved, int flags, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return fwd_impl(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, s_init, o, s_final,
                  saved, flags, workspace, workspace_bytes, stream);
}

kda_status kda_bwd(const kda_problem* p, const void* q, const void* k, const void* v,
                   const void* beta, const void* g_or_a, const float* A_log,
                   const float* dt_bias, const int32_t* cu_seqlens, const void* dO,
                   const void* saved, void* dq, void* dk, void* dv, void* dbeta,
                   void* dg_or_da, float* dA_log, float* ddt_bias, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return bwd_impl(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, nullptr, dO, nullptr,
                  saved, dq, dk, dv, dbeta, dg_or_da, dA_log, ddt_bias, nullptr, workspace,
                  workspace_bytes, stream);
}

kda_status kda_bwd_state(const kda_problem* p, const void* q, const void* k, const void* v,
                         const void* beta, const void* g_or_a, const float* A_log,
                         const float* dt_bias, const int32_t* cu_seqlens, const float* s_init,
                         const void* dO, const float* ds_final, const void* saved, void* dq,
                         void* dk, void* dv, void* dbeta, void* dg_or_da, float* dA_log,
                         float* ddt_bias, float* ds_init, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return bwd_impl(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, s_init, dO, ds_final,
                  saved, dq, dk, dv, dbeta, dg_or_da, dA_log, ddt_bias, ds_init, workspace,
                  workspace_bytes, stream);
}

size_t kda_state_summary_workspace_bytes(const kda_problem* p) {
  if (check_problem(p) != KDA_OK) return 0;
  return map_ws_bytes(map_sizes(p));
}

kda_status kda_state_summary(const kda_problem* p, const void* q, const void* k, const void* v,
                             const void* beta, const void* g_or_a, const float* A_log,
                             const float* dt_bias, const int32_t* cu_seqlens, float* M, float* B,
                             void* saved, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_last_error[0] = 0;
  kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  OPT_PTR(M, "M");
  OPT_PTR(B, "B");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // more than one document: the last one starts inside the sequence from
  // zero and does not see the entering state (M = 0); no tokens: the state
  // passes through one document unchanged (M = I) and nothing is added
  const int fill_M = p->num_seqs > 1 ? kda::FILL_ZERO : kda::FILL_IDENTITY;
  if (p->T == 0) {
    if (M) LAUNCH("fill_states", kda::launch_fill_states(p->H, M, nullptr, fill_M, hs));
    if (B) LAUNCH("fill_states", kda::launch_fill_states(p->H, B, nullptr, kda::FILL_ZERO, hs));
    return KDA_OK;
  }
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(beta, "beta");
  REQUIRE_PTR(g_or_a, "g_or_a");
  REQUIRE_PTR(cu_seqlens, "cu_seqlens");
  if (p->gate == KDA_GATE_RAW) {
    REQUIRE_PTR(A_log, "A_log");
    REQUIRE_PTR(dt_bias, "dt_bias");
  }
  if (saved && !aligned(saved)) return fail(KDA_ERR_INVALID_ARGUMENT, "saved is not 16-byte aligned");
  REQUIRE_PTR(workspace, "workspace");
  const Sizes s = map_sizes(p);
  const size_t need = saved ? table_bytes(s) : map_ws_bytes(s);
  if (workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                workspace_bytes, need);
  if (M && p->num_seqs > 1)
    LAUNCH("fill_states", kda::launch_fill_states(p->H, M, nullptr, fill_M, hs));
  if (!(M && p->num_seqs == 1) && !B && !saved) return KDA_OK;
  const kda::Dims d = map_dims(p);
  const kda::Inputs in{q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens};
  Carver wc(workspace);
  const kda::ChunkTable ct = carve_table(wc, s);
  kda::SavedSet sv;
  if (saved) {
    // the prep goes into the caller's saved set (with the backward's panels),
    // in the layout of kda_fwd, for a kda_fwd_state with KDA_FWD_PREP_DONE
    Carver sc(saved);
    sv = carve_saved(sc, sizes_of(p));
  } else {
    sv = carve_prep(wc, s);
  }
  kda::SegWork sg{};
  sg.map_M = p->num_seqs == 1 ? M : nullptr;
  sg.map_B = B;
  LAUNCH("chunk_map", kda::launch_chunk_map(d, cu_seqlens, ct, hs));
  LAUNCH("seg_map", kda::launch_seg_map(d, ct, hs));
  LAUNCH("fwd_prep", kda::launch_fwd_prep(d, in, ct, sv, saved != nullptr, hs));
  if (!(M && p->num_seqs == 1) && !B) return KDA_OK;
  LAUNCH("fwd_scan_map", kda::launch_fwd_scan(d, in, ct, sv, sv.panels, 0, sg, kda::SCAN_MAP, hs));
  return KDA_OK;
}

kda_status kda_state_grad_summary(const kda_problem* p, const void* q, const void* k,
                                  const void* v, const void* beta, const void* g_or_a,
                                  const float* A_log, const float* dt_bias,
                                  const int32_t* cu_seqlens, const void* dO, const void* saved,
                                  float* dB, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  g_last_error[0] = 0;
  kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  REQUIRE_PTR(dB, "dB");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // no tokens: no dO reaches the entering state
  if (p->T == 0) {
    LAUNCH("fill_states", kda::launch_fill_states(p->H, dB, nullptr, kda::FILL_ZERO, hs));
    return KDA_OK;
  }
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(beta, "beta");
  REQUIRE_PTR(g_or_a, "g_or_a");
  REQUIRE_PTR(cu_seqlens, "cu_seqlens");
  REQUIRE_PTR(dO, "dO");
  if (p->gate == KDA_GATE_RAW) {
    REQUIRE_PTR(A_log, "A_log");
    REQUIRE_PTR(dt_bias, "dt_bias");
  }
  if (saved && !aligned(saved)) return fail(KDA_ERR_INVALID_ARGUMENT, "saved is not 16-byte aligned");
  REQUIRE_PTR(workspace, "workspace");
  const Sizes s = map_sizes(p);
  const size_t need = saved ? table_bytes(s) : map_ws_bytes(s);
  if (workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                workspace_bytes, need);
  const kda::Dims d = map_dims(p);
  const kda::Inputs in{q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens};
  Carver wc(workspace);
  const kda::ChunkTable ct = carve_table(wc, s);
  kda::SavedSet sv;
  if (saved) {
    // the saving forward's set, in its own layout
    Carver sc(const_cast<void*>(saved));
    sv = carve_saved(sc, sizes_of(p));
  } else {
    sv = carve_prep(wc, s);
  }
  kda::SegWork sg{};
  sg.ds_init = dB;
  LAUNCH("chunk_map", kda::launch_chunk_map(d, cu_seqlens, ct, hs));
  LAUNCH("seg_map", kda::launch_seg_map(d, ct, hs));
  if (!saved) LAUNCH("fwd_prep", kda::launch_fwd_prep(d, in, ct, sv, 1, hs));
  LAUNCH("bwd_scan_map", kda::launch_bwd_scan(d, in, ct, sv, dO, nullptr, kda::BwdWork{}, sg,
                                              kda::SCAN_MAP, hs));
  return KDA_OK;
}

kda_status kda_state_apply(int32_t H, const float* M, int transpose, const float* B,
                           const float* x, float* y, void* stream) {
  g_last_error[0] = 0;
  if (H < 1 || H > 65535) return fail(KDA_ERR_INVALID_ARGUMENT, "H = %d outside [1, 65535]", H);
  if (transpose != 0 && transpose != 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "transpose must be 0 or 1");
  REQUIRE_PTR(M, "M");
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(y, "y");
  OPT_PTR(B, "B");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  LAUNCH("state_apply", kda::launch_state_apply(H, M, transpose, B, x, y, hs));
  return KDA_OK;
}

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KDA_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* kda_last_error(void) { return g_last_error; }

void kda_set_launch_hook(kda_launch_hook hook, void* user) {
  g_hook = hook;
  g_hook_user = user;
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
