/* Compiled as C99 against include/gdn.h and linked with libgdn.so: the header is
 * valid C, every entry point links, and the host-side checks answer without a GPU
 * (every call below fails validation or the workspace check before any launch). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"

#define FAKE ((void*)(uintptr_t)(1u << 20)) /* aligned, never dereferenced */

static int failures = 0;
static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main(void) {
  gdn_args a;
  memset(&a, 0, sizeof a);
  a.variant = GDN_VARIANT_FG2;
  a.dtype = GDN_DTYPE_BF16;
  a.B = 2;
  a.T = 100;
  a.H = 4;
  a.dk = a.dv = 128;
  a.chunk = 64;
  a.n_h = 1;
  a.q = a.k = a.v = a.alpha = a.beta = FAKE;
  a.o = FAKE;

  expect("abi version", gdn_abi_version(), GDN_ABI_VERSION);
  const size_t need = gdn_workspace_bytes(&a);
  expect("workspace > 0", need > 0, 1);
  expect("no workspace", gdn_chunk_fwd(&a, NULL, 0, NULL), GDN_ERR_WORKSPACE);
  expect("small workspace", gdn_chunk_fwd(&a, FAKE, need - 1, NULL), GDN_ERR_WORKSPACE);
  expect("prepare, no workspace", gdn_chunk_prepare(&a, NULL, 0, NULL), GDN_ERR_WORKSPACE);
  expect("scan, no workspace", gdn_chunk_scan(&a, NULL, 0, NULL), GDN_ERR_WORKSPACE);
  expect("null args", gdn_chunk_fwd(NULL, FAKE, need, NULL), GDN_ERR_ARG);
  expect("recurrent, null state", gdn_recurrent_step(&a, NULL, NULL), GDN_ERR_ARG);

  gdn_args f = a;
  f.s_final = NULL;
  expect("final state needs s_final", gdn_final_state(&f, FAKE, need, NULL), GDN_ERR_ARG);

  gdn_args bad = a;
  bad.dk = 48;
  expect("unsupported dk", gdn_chunk_fwd(&bad, FAKE, need, NULL), GDN_ERR_UNSUPPORTED);
  expect("no workspace size for bad args", (int)gdn_workspace_bytes(&bad), 0);

  gdn_args st = a;
  st.variant = GDN_VARIANT_ASYM;
  st.beta = NULL;
  st.j = st.eta = FAKE;
  expect("stabilize mode", gdn_asym_stabilize(&st, 0, FAKE, NULL), GDN_ERR_ARG);
  expect("stabilize out", gdn_asym_stabilize(&st, GDN_STABILIZE_CLIP_DECAY, NULL, NULL), GDN_ERR_ARG);
  st.stabilize = 3;
  expect("fused stabilizer mode", gdn_chunk_fwd(&st, FAKE, need, NULL), GDN_ERR_ARG);

  expect("status text", strcmp(gdn_status_str(GDN_OK), "ok"), 0);
  if (failures == 0) printf("abi_check ok\n");
  return failures == 0 ? 0 : 1;
}
