/* Controls of the CPU stand-in for the HIP runtime and the kernel launchers
 * (i4s_hip_stub.cpp), used by the sanitized host-layer driver.  Test
 * infrastructure only. */
#ifndef I4S_HIP_STUB_H
#define I4S_HIP_STUB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct i4s_stub_launch {
  int kind;          /* 0 none, 1 pack analyze, 2 pack emit, 3 gemv, 4 gemv with workspace, 5 fused */
  int rows, cols, n_keep, group_size, batch, layers;
  int adaptive;
  const void *workspace;
} i4s_stub_launch;

/* The architecture name the device reports ("gfx950" by default). */
void i4s_stub_set_arch(const char *arch);
/* What the pack analysis leaves in the workspace: the flag word and the three
 * 128-bit SSE totals (lo, hi for G = 64, 128, 256). */
void i4s_stub_set_pack_result(uint32_t flag, const uint64_t totals_lo_hi[6]);
/* Number of launches so far, and the last one. */
int i4s_stub_launches(void);
i4s_stub_launch i4s_stub_last_launch(void);
/* The address the no-allocation entry point receives as its scratch. */
const void *i4s_stub_scratch(void);

#ifdef __cplusplus
}
#endif

#endif
