/*
 * liblora benchmark instrumentation -- NOT part of the production library.
 *
 * Exported only by liblora_timed.so, a second build of the same sources in
 * which the host dispatch file is compiled with LORA_TIMING_HOOKS: its GPU
 * kernels are the same object files as liblora.so's; the host code
 * additionally records two caller-supplied hipEvents around one GEMM
 * launch.  A benchmark loads liblora_timed.so in place of liblora.so (every
 * entry point of liblora.h is exported by both) to time one GEMM class
 * inside a whole step on the step's own stream.
 *
 * lora_debug_time_next: record the hipEvents `start` and `stop` (hipEvent_t
 * handles) on the launch stream immediately before and after the next
 * launch of GEMM class `which` made BY THE CALLING HOST THREAD.  One-shot per
 * class; the armed events are per host thread (other threads' calls are not
 * timed); NULL events clear the slot.  Returns LORA_OK, or
 * LORA_ERR_BAD_SHAPE for an unknown class.
 */
#ifndef LIBLORA_TIMING_H
#define LIBLORA_TIMING_H

#include "liblora.h"

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_KC_GATEUP_FWD  0   /* gate/up GEMM with the SwiGLU epilogue   */
#define LORA_KC_DOWN_FWD    1   /* down-projection forward GEMM            */
#define LORA_KC_DOWN_BWD    2   /* dY Wd GEMM with the SwiGLU' epilogue    */
#define LORA_KC_GATEUP_BWD  3   /* [de|dg] [Wg;Wu] GEMM (MLP dX)           */
#define LORA_KC_LINEAR_FWD  4   /* lora_linear_fwd GEMM                    */
#define LORA_KC_LINEAR_DX   5   /* lora_linear_bwd dX GEMM                 */
#define LORA_KC_QKV_FWD     6   /* lora_qkv_fwd fused GEMM                 */
#define LORA_KC_QKV_DX      7   /* lora_qkv_bwd fused dX GEMM              */
#define LORA_KC_COUNT       8

int lora_debug_time_next(int which, void *start, void *stop);

#ifdef __cplusplus
}
#endif
#endif /* LIBLORA_TIMING_H */
