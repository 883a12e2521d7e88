// Attention launchers of the recurrent block.
#pragma once

#include "common.h"

// Any head widths (dq, dv <= 128), fp32 or bf16 storage.
void launch_attn_generic(int dtype_bf16, const void* q, const void* k, const void* vt, void* o, int B, int H,
                         int G, int Tq, int cap, int dq, int dv, int kbase, float scale, hipStream_t s);
// bf16, head width 128, MFMA flash kernel (prefill).  `cap` must be a
// multiple of 8.
void launch_attn_flash_bf16(const void* q, const void* k, const void* vt, void* o, int B, int H, int G, int Tq,
                            int cap, int kbase, float scale, hipStream_t s);
