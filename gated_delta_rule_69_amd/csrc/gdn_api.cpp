// C ABI entry points: argument validation, workspace sizing and dispatch.
// This translation unit makes no HIP call itself; launches live in the .hip files.
#include <cstdint>
#include <cstring>

#include "gdn_internal.h"

namespace gdn {
namespace {

bool head_dim_ok(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }
bool opt_ptr_ok(const void* p) { return p == nullptr || aligned16(p); }

}  // namespace

int validate(const gdn_args* a, Entry e, Problem* out) {
  if (a == nullptr) return GDN_ERR_ARG;
  if (a->variant < GDN_VARIANT_FG2 || a->variant > GDN_VARIANT_ASYM) return GDN_ERR_ARG;
  if (a->dtype != GDN_DTYPE_F32 && a->dtype != GDN_DTYPE_BF16) return GDN_ERR_ARG;
  if (a->B < 1 || a->H < 1 || a->T < 0) return GDN_ERR_ARG;
  // Keep every element offset far inside int64 and every grid dimension valid.
  if (a->B > (1 << 20) || a->H > (1 << 16) || a->B * a->H > (1 << 24) ||
      a->T > (int64_t(1) << 31))
    return GDN_ERR_UNSUPPORTED;
  if (!head_dim_ok(a->dk) || !head_dim_ok(a->dv)) return GDN_ERR_UNSUPPORTED;
  const bool dp = a->variant == GDN_VARIANT_DELTAPRODUCT;
  if (dp) {
    if (a->n_h < 1) return GDN_ERR_ARG;
    if (a->n_h > 8) return GDN_ERR_UNSUPPORTED;
  } else if (a->n_h != 1) {
    return GDN_ERR_ARG;
  }
  const bool chunked = e != Entry::Recurrent && e != Entry::Stabilize;
  int chunk = a->chunk;
  // DeltaProduct is laid out in chunks with a power-of-two number of steps a token
  // (three Householder steps as four, five to seven as eight), the extra ones
  // identity steps, so that a chunk holds whole tokens
  const int n_step = !chunked ? a->n_h : a->n_h == 3 ? 4 : a->n_h >= 5 ? 8 : a->n_h;
  if (chunked) {
    if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERR_UNSUPPORTED;
    // fp32 tiles of a 64-step chunk with 128 key channels exceed the 160 KB of LDS of
    // the scan's double-buffered record image: such calls run with 32-step chunks,
    // the same recurrence up to rounding
    if (a->dtype == GDN_DTYPE_F32 && a->dk == 128 && chunk == 64) chunk = 32;
    if (chunk % n_step != 0) return GDN_ERR_UNSUPPORTED;
    // output rows a chunk: 8 (one half-filled 16-row tile) or a multiple of 16
    if (chunk / n_step < 8) return GDN_ERR_UNSUPPORTED;
  }
  if (a->variant == GDN_VARIANT_FG2 && a->beta_v == nullptr && a->dk != a->dv)
    return GDN_ERR_ARG;  // one beta vector scales both key and value channels
  if (a->variant != GDN_VARIANT_FG2 && a->beta_v != nullptr) return GDN_ERR_ARG;
  if (e != Entry::Stabilize) {  // the standalone stabiliser takes its mode as an argument
    if (a->stabilize < 0 || a->stabilize > GDN_STABILIZE_PROJECT_J) return GDN_ERR_ARG;
    if (a->stabilize != 0 && a->variant != GDN_VARIANT_ASYM) return GDN_ERR_ARG;
  }

  if (e == Entry::Stabilize) {
    // Only k, j, alpha (= D) and eta are read; with T == 0 they may be NULL.
    if (a->variant != GDN_VARIANT_ASYM) return GDN_ERR_ARG;
    auto need = [&](const void* p) { return a->T == 0 ? opt_ptr_ok(p) : ptr_ok(p); };
    if (!need(a->k) || !need(a->j) || !need(a->alpha) || !need(a->eta)) return GDN_ERR_ARG;
  } else if (e != Entry::Shapes) {
    // With T == 0 the per-token arrays are empty and may be NULL.
    auto need = [&](const void* p) { return a->T == 0 ? opt_ptr_ok(p) : ptr_ok(p); };
    if (!need(a->k) || !need(a->v) || !need(a->alpha)) return GDN_ERR_ARG;
    if (a->variant == GDN_VARIANT_ASYM) {
      if (!need(a->j) || !need(a->eta)) return GDN_ERR_ARG;
      if (!opt_ptr_ok(a->beta)) return GDN_ERR_ARG;
    } else {
      if (!need(a->beta)) return GDN_ERR_ARG;
      if (a->j != nullptr || a->eta != nullptr) return GDN_ERR_ARG;
    }
    if (!opt_ptr_ok(a->beta_v)) return GDN_ERR_ARG;
    if (e != Entry::FinalState) {
      if (!need(a->q) || !need(a->o)) return GDN_ERR_ARG;
    } else {
      if (!opt_ptr_ok(a->q) || !opt_ptr_ok(a->o)) return GDN_ERR_ARG;
      if (a->s_final == nullptr) return GDN_ERR_ARG;
    }
    if (!opt_ptr_ok(a->s0) || !opt_ptr_ok(a->s_final)) return GDN_ERR_ARG;
  }

  if (chunked) {
    const int64_t nchunks = (a->T * n_step + chunk - 1) / chunk;
    if (nchunks * a->B * a->H >= (int64_t(1) << 31)) return GDN_ERR_UNSUPPORTED;  // grid size
  }

  if (out) {
    Problem& p = *out;
    p.variant = a->variant;
    p.dtype = a->dtype;
    p.B = a->B;
    p.T = a->T;
    p.H = a->H;
    p.dk = a->dk;
    p.dv = a->dv;
    p.chunk = chunk;
    p.n_h = a->n_h;
    p.n_step = n_step;
    p.stabilize = e == Entry::Stabilize ? 0 : a->stabilize;
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.alpha = a->alpha;
    p.beta = a->beta;
    p.beta_v = a->beta_v;
    p.j = a->j;
    p.eta = a->eta;
    p.s0 = a->s0;
    p.s_final = a->s_final;
    p.o = a->o;
    p.steps = a->T * n_step;
    p.c0 = 0;
    if (chunked) {
      p.nchunks = (p.steps + chunk - 1) / chunk;
      p.rows_out = chunk / n_step;
    } else {
      p.nchunks = 0;
      p.rows_out = 0;
    }
  }
  return GDN_OK;
}

ChunkLayout chunk_layout(const Problem& p) {
  return make_chunk_layout(p.dtype == GDN_DTYPE_BF16 ? 2 : 4, size_t(p.dk), size_t(p.dv),
                           size_t(p.chunk));
}

}  // namespace gdn

using gdn::Entry;
using gdn::Problem;

extern "C" {

size_t gdn_workspace_bytes(const gdn_args* args) {
  Problem p;
  if (gdn::validate(args, Entry::Shapes, &p) != GDN_OK) return 0;
  if (p.nchunks == 0) return 256;
  return gdn::workspace_bytes(p, gdn::chunk_layout(p));
}

enum class Stage { Both, Prepare, Scan };

static int run_chunked(const gdn_args* args, void* ws, size_t ws_bytes, void* stream,
                       Entry e, Stage stage) {
  Problem p;
  int st = gdn::validate(args, e, &p);
  if (st != GDN_OK) return st;
  if (p.T == 0) {
    if (p.s_final == nullptr || stage == Stage::Prepare) return GDN_OK;
    return gdn::launch_state_copy(p, stream) == 0 ? GDN_OK : GDN_ERR_HIP;
  }
  const size_t need = gdn_workspace_bytes(args);
  if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return GDN_ERR_WORKSPACE;
  const bool want_out = e == Entry::ChunkFwd;
  int rc = 0;
  switch (stage) {
    case Stage::Both: rc = gdn::launch_chunk(p, ws, want_out, stream); break;
    case Stage::Prepare: rc = gdn::launch_prep(p, ws, want_out, stream); break;
    case Stage::Scan: rc = gdn::launch_scan(p, ws, want_out, stream); break;
  }
  return rc == 0 ? GDN_OK : GDN_ERR_HIP;
}

int gdn_chunk_fwd(const gdn_args* args, void* ws, size_t ws_bytes, void* stream) {
  return run_chunked(args, ws, ws_bytes, stream, Entry::ChunkFwd, Stage::Both);
}

int gdn_final_state(const gdn_args* args, void* ws, size_t ws_bytes, void* stream) {
  return run_chunked(args, ws, ws_bytes, stream, Entry::FinalState, Stage::Both);
}

static Entry stage_entry(const gdn_args* args) {
  return (args != nullptr && args->o == nullptr) ? Entry::FinalState : Entry::ChunkFwd;
}

int gdn_chunk_prepare(const gdn_args* args, void* ws, size_t ws_bytes, void* stream) {
  return run_chunked(args, ws, ws_bytes, stream, stage_entry(args), Stage::Prepare);
}

int gdn_chunk_scan(const gdn_args* args, void* ws, size_t ws_bytes, void* stream) {
  return run_chunked(args, ws, ws_bytes, stream, stage_entry(args), Stage::Scan);
}

int gdn_recurrent_step(const gdn_args* args, float* state_inout, void* stream) {
  Problem p;
  int st = gdn::validate(args, Entry::Recurrent, &p);
  if (st != GDN_OK) return st;
  if (state_inout == nullptr || (reinterpret_cast<uintptr_t>(state_inout) & 15u) != 0)
    return GDN_ERR_ARG;
  if (p.T == 0) return GDN_OK;
  return gdn::launch_recurrent(p, state_inout, stream) == 0 ? GDN_OK : GDN_ERR_HIP;
}

static int bwd_problem(const gdn_args* args, Problem* p) {
  if (args == nullptr) return GDN_ERR_ARG;
  gdn_args a = *args;
  if (a.o == nullptr) a.o = const_cast<void*>(a.q);  // not written by the backward pass
  int st = gdn::validate(&a, Entry::Recurrent, p);
  if (st != GDN_OK) return st;
  if (p->stabilize != 0) return GDN_ERR_UNSUPPORTED;
  if (p->B * p->H * p->steps > (int64_t(1) << 33)) return GDN_ERR_UNSUPPORTED;  // keeps every grid in 32 bits
  return GDN_OK;
}

size_t gdn_bwd_workspace_bytes(const gdn_args* args) {
  Problem p;
  if (args == nullptr) return 0;
  gdn_args a = *args;  // shapes only: the pointer checks belong to the call itself
  if (a.T > 0) a.q = a.k = a.v = a.alpha = a.o = reinterpret_cast<void*>(uintptr_t(1) << 20);
  if (a.T > 0 && a.variant == GDN_VARIANT_ASYM) a.j = a.eta = a.k;
  if (a.T > 0 && a.variant != GDN_VARIANT_ASYM) a.beta = a.k;
  if (bwd_problem(&a, &p) != GDN_OK) return 0;
  return gdn::bwd_workspace_bytes(p);
}

int gdn_recurrent_bwd(const gdn_args* args, const void* d_o, const float* d_s_final,
                      const gdn_grads* grads, void* ws, size_t ws_bytes, void* stream) {
  Problem p;
  int st = bwd_problem(args, &p);
  if (st != GDN_OK) return st;
  if (grads == nullptr) return GDN_ERR_ARG;
  auto a16 = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; };
  auto need = [&](const void* x) { return p.T == 0 ? a16(x) : (x != nullptr && a16(x)); };
  auto none = [](const void* x) { return x == nullptr; };
  const bool asym = p.variant == GDN_VARIANT_ASYM;
  const bool plus = p.variant == GDN_VARIANT_FG2 && p.beta_v != nullptr;
  if (!need(d_o) || !need(grads->dq) || !need(grads->dk) || !need(grads->dv) || !need(grads->dalpha))
    return GDN_ERR_ARG;
  if (asym ? !(need(grads->dj) && need(grads->deta) && none(grads->dbeta))
           : !(need(grads->dbeta) && none(grads->dj) && none(grads->deta)))
    return GDN_ERR_ARG;
  if (plus ? !need(grads->dbeta_v) : !none(grads->dbeta_v)) return GDN_ERR_ARG;
  if (!a16(grads->ds0) || !a16(d_s_final)) return GDN_ERR_ARG;
  const size_t need_ws = gdn::bwd_workspace_bytes(p);
  if (ws == nullptr || ws_bytes < need_ws || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return GDN_ERR_WORKSPACE;
  const gdn::GradPtrs g{grads->dq, grads->dk, grads->dv, grads->dalpha, grads->dbeta,
                        grads->dbeta_v, grads->dj, grads->deta, grads->ds0};
  return gdn::launch_recurrent_bwd(p, d_o, d_s_final, g, ws, stream) == 0 ? GDN_OK : GDN_ERR_HIP;
}

int gdn_asym_stabilize(const gdn_args* args, int mode, void* out, void* stream) {
  Problem p;
  int st = gdn::validate(args, Entry::Stabilize, &p);
  if (st != GDN_OK) return st;
  if (mode != GDN_STABILIZE_CLIP_DECAY && mode != GDN_STABILIZE_PROJECT_J) return GDN_ERR_ARG;
  if (p.T == 0) return GDN_OK;
  if (out == nullptr || (reinterpret_cast<uintptr_t>(out) & 15u) != 0) return GDN_ERR_ARG;
  return gdn::launch_stabilize(p, mode, out, stream) == 0 ? GDN_OK : GDN_ERR_HIP;
}

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_ARG: return "invalid argument (null or misaligned pointer, or bad shape)";
    case GDN_ERR_UNSUPPORTED: return "unsupported size, chunk length or step count";
    case GDN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case GDN_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
