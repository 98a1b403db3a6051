/* The C ABI from a C99 program (no Python, no GPU): the header compiles as C,
 * the library links, and host-side validation returns the documented codes
 * before any device call.  Exit status 0 when every check holds; each failed
 * check prints one line. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fp8q.h"

static int failures = 0;

static void expect(const char* what, fp8q_status got, fp8q_status want) {
  if (got != want) {
    printf("FAIL %s: %s, expected %s\n", what, fp8q_status_string(got), fp8q_status_string(want));
    ++failures;
  }
}

int main(void) {
  /* fake, suitably aligned pointers: every call below must return before
     dereferencing them */
  uint8_t* const P = (uint8_t*)(uintptr_t)0x100000;
  float* const F = (float*)(uintptr_t)0x200000;
  int32_t* const I = (int32_t*)(uintptr_t)0x300000;
  uint8_t* const U = (uint8_t*)(uintptr_t)0x100001;   /* not 16-byte aligned */

  if (fp8q_abi_version() != FP8Q_ABI_VERSION) {
    printf("FAIL abi version %d, header %d\n", fp8q_abi_version(), FP8Q_ABI_VERSION);
    ++failures;
  }
  if (strncmp(fp8q_status_string(FP8Q_ERR_SHAPE), "FP8Q_ERR_SHAPE", 14) != 0) {
    printf("FAIL status string\n");
    ++failures;
  }

  /* empty inputs are no-ops */
  expect("quantize_act M=0", fp8q_quantize_act(NULL, 0, 128, NULL, NULL, FP8Q_SCALE_F32, NULL), FP8Q_OK);
  expect("gemm M=0", fp8q_gemm(NULL, NULL, NULL, NULL, 0, 128, 128, NULL, FP8Q_OUT_F32, NULL), FP8Q_OK);
  expect("gemm_precise N=0", fp8q_gemm_precise(NULL, NULL, NULL, NULL, 4, 0, 128, NULL, FP8Q_OUT_F32, NULL), FP8Q_OK);
  expect("grouped M_total=0", fp8q_grouped_gemm(NULL, NULL, 0, I, 2, NULL, NULL, 128, 128, NULL, FP8Q_OUT_BF16, NULL), FP8Q_OK);

  /* NULL, shape, alignment and enum errors, in the documented order */
  expect("quantize_act NULL", fp8q_quantize_act(NULL, 4, 128, P, F, FP8Q_SCALE_F32, NULL), FP8Q_ERR_NULL);
  expect("quantize_act K%128", fp8q_quantize_act(P, 4, 100, P, F, FP8Q_SCALE_F32, NULL), FP8Q_ERR_SHAPE);
  expect("quantize_act align", fp8q_quantize_act(U, 4, 128, P, F, FP8Q_SCALE_F32, NULL), FP8Q_ERR_ALIGN);
  expect("quantize_act mode", fp8q_quantize_act(P, 4, 128, P, F, (fp8q_scale_mode)7, NULL), FP8Q_ERR_ENUM);
  expect("quantize_weight N%128", fp8q_quantize_weight(P, 100, 128, P, F, FP8Q_SCALE_POW2, NULL), FP8Q_ERR_SHAPE);
  expect("gemm NULL c", fp8q_gemm(P, F, P, F, 4, 128, 128, NULL, FP8Q_OUT_F32, NULL), FP8Q_ERR_NULL);
  expect("gemm N%128", fp8q_gemm(P, F, P, F, 4, 100, 128, P, FP8Q_OUT_F32, NULL), FP8Q_ERR_SHAPE);
  expect("gemm out enum", fp8q_gemm(P, F, P, F, 4, 128, 128, P, (fp8q_out_dtype)5, NULL), FP8Q_ERR_ENUM);
  expect("gemm K=0", fp8q_gemm(P, F, P, F, 4, 128, 0, P, FP8Q_OUT_F32, NULL), FP8Q_ERR_UNSUPPORTED);
  expect("gemm_mfma_scaled align", fp8q_gemm_mfma_scaled(U, F, P, F, 4, 128, 128, P, FP8Q_OUT_F32, NULL), FP8Q_ERR_ALIGN);
  expect("grouped G=0", fp8q_grouped_gemm(P, F, 8, I, 0, P, F, 128, 128, P, FP8Q_OUT_F32, NULL), FP8Q_ERR_SHAPE);
  expect("grouped_precise NULL off", fp8q_grouped_gemm_precise(P, F, 8, NULL, 2, P, F, 128, 128, P, FP8Q_OUT_F32, NULL), FP8Q_ERR_NULL);
  expect("rowscaled K%128", fp8q_gemm_rowscaled(P, F, P, F, 4, 128, 100, P, FP8Q_OUT_F32, NULL), FP8Q_ERR_SHAPE);
  expect("gemm_bf16 N%128", fp8q_gemm_bf16(P, P, 4, 100, 128, P, FP8Q_OUT_F32, NULL), FP8Q_ERR_SHAPE);
  expect("gemm_fused mode", fp8q_gemm_fused(P, P, F, 4, 128, 128, P, FP8Q_OUT_F32, (fp8q_scale_mode)9, NULL), FP8Q_ERR_ENUM);

  if (failures == 0) printf("c abi ok\n");
  return failures == 0 ? 0 : 1;
}
