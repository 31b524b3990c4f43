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
  int64_t steps;     // virtual steps: T * n_h
  int64_t nchunks;   // ceil(steps / chunk)
  int rows_out;      // output rows per chunk: chunk / n_h
};

// Shapes: the chunked shape checks only (no pointer checks), for workspace sizing.
enum class Entry { ChunkFwd, FinalState, Recurrent, Shapes };

// Pure argument checks; no HIP call. Returns GDN_OK or a negative status.
int validate(const gdn_args* a, Entry e, Problem* out);

// Per-chunk workspace record (bytes) and the offsets of its parts.
struct ChunkLayout {
  size_t elem;        // 2 (fp16 operands) or 4 (fp32 operands)
  size_t off_W;       // W      [C][dk]
  size_t off_UT;      // U~^T   [dv][C]
  size_t off_AT;      // A^^T   [dk][C]
  size_t off_Q;       // Q+     [R][dk]
  size_t off_P;       // P      [R][C]
  size_t off_gamma;   // gamma  [dk] float
  size_t off_qinv;    // per-output-row inverse q scale [R] float
  size_t off_winv;    // per-chunk inverse w scale      [4] float
  size_t bytes;       // record size (multiple of 256)
};
ChunkLayout chunk_layout(const Problem& p);

// Kernel launchers (defined in the .hip translation units). Return hipError_t as int.
int launch_recurrent(const Problem& p, float* state, void* stream);
int launch_chunk(const Problem& p, void* ws, bool want_output, void* stream);
int launch_prep(const Problem& p, void* ws, bool want_output, void* stream);
int launch_scan(const Problem& p, void* ws, bool want_output, void* stream);
int launch_state_copy(const Problem& p, void* stream);

}  // namespace gdn
