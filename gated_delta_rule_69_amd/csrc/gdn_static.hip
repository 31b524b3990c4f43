// gdn_chunk_fwd_static: the chunked forward pass without a caller workspace, for
// callers that cannot allocate device memory. The chunk records live in a buffer
// of GDN_STATIC_SCRATCH_BYTES inside the library (one per device, held until the
// process ends); the sequence runs in blocks of as many chunks as that buffer
// holds for every (batch, head), each block a prepare launch and a scan launch
// that starts from the state the previous block left. The per-chunk records and
// the float32 state carried between blocks are the same values gdn_chunk_fwd
// computes, so the results are bitwise equal to it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "gdn_internal.h"

namespace gdn {
namespace {

// The record buffer. In host code `scratch` names a host-side stand-in, not the
// device array: its device address on each device comes from hipGetSymbolAddress
// and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[GDN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up yet)

// Device address of the buffer on the current device, looked up once per device.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return GDN_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return GDN_OK;
}

}  // namespace
}  // namespace gdn

extern "C" int gdn_chunk_fwd_static(const gdn_args* args, void* stream) {
  using namespace gdn;
  Problem p;
  int st = validate(args, Entry::ChunkFwd, &p);
  if (st != GDN_OK) return st;
  if (p.T == 0) {
    if (p.s_final == nullptr) return GDN_OK;
    return launch_state_copy(p, stream) == 0 ? GDN_OK : GDN_ERR_HIP;
  }
  const ChunkLayout L = chunk_layout(p);
  const size_t bh = size_t(p.B) * size_t(p.H);
  // without s_final the state between blocks is kept at the start of the buffer
  const size_t carry = p.s_final ? 0 : round_up_c(bh * size_t(p.dk) * size_t(p.dv) * sizeof(float), 256);
  const size_t cap = GDN_STATIC_SCRATCH_BYTES;
  // records and flag bytes of a block of n chunks
  auto block_bytes = [&](int64_t n) {
    Problem q = p;
    q.nchunks = n;
    return workspace_bytes(q, L);
  };
  if (carry + block_bytes(1) > cap) return GDN_ERR_UNSUPPORTED;  // one chunk of every sequence must fit
  int64_t per_block = int64_t((cap - carry) / (bh * (L.bytes + 1)));
  while (per_block > 1 && carry + block_bytes(per_block) > cap) --per_block;
  void* base = nullptr;
  st = scratch_address(&base);
  if (st != GDN_OK) return st;
  float* state = p.s_final ? p.s_final : static_cast<float*>(base);
  unsigned char* rec = static_cast<unsigned char*>(base) + carry;
  const int64_t NC = p.nchunks;
  for (int64_t c = 0; c < NC; c += per_block) {
    Problem q = p;
    q.c0 = c;
    q.nchunks = std::min<int64_t>(per_block, NC - c);
    q.s0 = c == 0 ? p.s0 : state;
    q.s_final = c + q.nchunks == NC ? p.s_final : state;
    if (launch_prep(q, rec, true, stream) != 0) return GDN_ERR_HIP;
    if (launch_scan(q, rec, true, stream) != 0) return GDN_ERR_HIP;
  }
  return GDN_OK;
}
