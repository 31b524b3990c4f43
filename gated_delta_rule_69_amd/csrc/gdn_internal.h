// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <cstddef>
#include <cstdint>

#include "gdn.h"

namespace gdn {

// Shape and pointer bundle after validation (all sizes as int64).
struct Problem {
  int variant;
  int dtype;
  int64_t B, T, H, dk, dv;
  int chunk;
  int n_h;
  int n_step;     // steps a token takes in a chunk: n_h, or 4 for n_h = 3 (the fourth
                  // an identity step: beta = 0 writes and erases nothing)
  int stabilize;  // ASYM: 0, or the gdn_stabilize_mode applied to each token's inputs
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* beta;
  const void* beta_v;
  const void* j;
  const void* eta;
  const float* s0;
  float* s_final;
  void* o;
  // chunk geometry (chunked entry points)
  int64_t steps;     // virtual steps: T * n_step (chunked), T * n_h (recurrent)
  int64_t nchunks;   // chunks of one launch: ceil(steps / chunk) for the whole sequence
  int64_t c0;        // first chunk of the launch (0 for the whole sequence); the
                     // workspace holds the records of chunks c0 .. c0 + nchunks - 1,
                     // s0 is the state before chunk c0 and s_final the state after
                     // the launch's last chunk
  int rows_out;      // output rows per chunk: chunk / n_h
};

// Shapes: the chunked shape checks only (no pointer checks), for workspace sizing.
enum class Entry { ChunkFwd, FinalState, Recurrent, Stabilize, Shapes };

// Pure argument checks; no HIP call. Returns GDN_OK or a negative status.
int validate(const gdn_args* a, Entry e, Problem* out);

// Per-chunk workspace record. Elements are fp16 (bf16 inputs) or fp32 (fp32
// inputs). Two formats:
//
// Image format (every configuration except the one below): the first part is
// byte-for-byte the LDS image the image scan stages (padded rows), so staging is
// a flat copy:
//   W     [C][dk+4]   A^^T [dk][C+4]   gamma [dk] f32   1/ws [4] f32     (state image)
//   Q+    [C][dk+4]   P    [C][C+4]    1/qs  [C] f32                      (output part)
// followed by U~^T [dv][C] (read straight into registers).
//
// Fragment format (fp16 operands, dk = 128, C = 64): every operand is stored in
// the order the row-split scan's lanes read it, 16 bytes per lane per MFMA
// fragment, so one wave-wide load moves 1 KB of contiguous memory:
//   W, Q+  [row tile][k-block of 32 channels][lane][8]   lane = row % 16 + 16 * (k % 32 / 8)
//   A^^T   [channel tile][k-block of 32 steps][lane][8]
//   P      [row tile][k-block of 32 steps][lane][8]
//   U~     [step tile][value-column tile][lane][4]        lane = column % 16 + 16 * (step % 16 / 4)
//   gamma [dk] f32, 1/qs [C] f32, 1/ws [4] f32.
struct ChunkLayout {
  size_t elem, ldk, ldc;
  size_t off_W, off_AT, off_gamma, off_winv, state_bytes;
  size_t off_Q, off_P, off_qinv, image_bytes;
  size_t off_UT, bytes;
  bool frag;
};

constexpr size_t round_up_c(size_t x, size_t m) { return (x + m - 1) / m * m; }

// The fragment format (and the row-split scan) covers fp16 operands with dk = 128
// and chunk 64.
constexpr bool frag_layout(size_t es, size_t dk, size_t C) { return es == 2 && dk == 128 && C == 64; }

constexpr ChunkLayout make_chunk_layout(size_t es, size_t dk, size_t dv, size_t C) {
  ChunkLayout L{};
  L.elem = es;
  L.frag = frag_layout(es, dk, C);
  if (L.frag) {
    L.ldk = dk;
    L.ldc = C;
    L.off_W = 0;
    L.off_Q = L.off_W + C * dk * es;
    L.off_AT = L.off_Q + C * dk * es;
    L.off_P = L.off_AT + dk * C * es;
    L.off_UT = L.off_P + C * C * es;
    L.off_gamma = L.off_UT + dv * C * es;
    L.off_qinv = L.off_gamma + dk * 4;
    L.off_winv = L.off_qinv + C * 4;
    L.state_bytes = L.image_bytes = 0;
    L.bytes = round_up_c(L.off_winv + 16, 256);
    return L;
  }
  L.ldk = dk + 4;
  L.ldc = C + 4;
  L.off_W = 0;
  L.off_AT = L.off_W + C * L.ldk * es;
  L.off_gamma = L.off_AT + dk * L.ldc * es;
  L.off_winv = L.off_gamma + dk * 4;
  L.state_bytes = L.off_winv + 16;
  L.off_Q = L.state_bytes;
  L.off_P = L.off_Q + C * L.ldk * es;
  L.off_qinv = L.off_P + C * L.ldc * es;
  L.image_bytes = L.off_qinv + C * 4;
  L.off_UT = round_up_c(L.image_bytes, 256);
  L.bytes = round_up_c(L.off_UT + dv * C * es, 256);
  return L;
}

ChunkLayout chunk_layout(const Problem& p);

// Workspace of a chunked launch: the records of its B * H * nchunks items, then one
// flag byte per item (set by the prepare pass for chunks it leaves to its second
// pass), rounded to 256 bytes.
inline size_t record_bytes(const Problem& p, const ChunkLayout& L) {
  return size_t(p.B) * size_t(p.H) * size_t(p.nchunks) * L.bytes;
}
inline size_t workspace_bytes(const Problem& p, const ChunkLayout& L) {
  return record_bytes(p, L) + round_up_c(size_t(p.B) * size_t(p.H) * size_t(p.nchunks), 256);
}

// Kernel launchers (defined in the .hip translation units). Return hipError_t as int.
int launch_recurrent(const Problem& p, float* state, void* stream);
int launch_chunk(const Problem& p, void* ws, bool want_output, void* stream);
int launch_prep(const Problem& p, void* ws, bool want_output, void* stream);
int launch_scan(const Problem& p, void* ws, bool want_output, void* stream);
// Preparation launchers, one translation unit per variant (gdn_prep_*.hip).
int launch_prep_fg2(const Problem& p, void* ws, bool want_output, void* stream);
int launch_prep_kda(const Problem& p, void* ws, bool want_output, void* stream);
int launch_prep_gdn(const Problem& p, void* ws, bool want_output, void* stream);
int launch_prep_dp(const Problem& p, void* ws, bool want_output, void* stream);
int launch_prep_asym(const Problem& p, void* ws, bool want_output, void* stream);
int launch_state_copy(const Problem& p, void* stream);
// Gradient outputs of the backward pass (float32; see gdn_grads).
struct GradPtrs {
  float *dq, *dk, *dv, *dalpha, *dbeta, *dbeta_v, *dj, *deta, *ds0;
};
// Backward pass of the token recurrence (gdn_backward.hip).
size_t bwd_workspace_bytes(const Problem& p);
int launch_recurrent_bwd(const Problem& p, const void* d_o, const float* dsf, const GradPtrs& g,
                         void* ws, void* stream);
// ASYM stabilisers (gdn_stabilize.hip); mode as in gdn_asym_stabilize.
int launch_stabilize(const Problem& p, int mode, void* out, void* stream);

}  // namespace gdn
