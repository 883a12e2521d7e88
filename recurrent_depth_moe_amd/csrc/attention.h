// Attention launchers of the recurrent block.
#pragma once

#include "common.h"

// Generic kernel's LDS: the query row (dq floats, rounded up to 4) then one
// score per visible key.  The runtime refuses configurations whose longest
// call would need more than RDT_GENERIC_LDS_MAX bytes.
constexpr size_t RDT_GENERIC_LDS_MAX = 64 * 1024;
__host__ __device__ inline int attn_generic_qslots(int dq) { return (dq + 3) & ~3; }
inline size_t attn_generic_lds_bytes(int dq, int nk) {
  return ((size_t)attn_generic_qslots(dq) + (size_t)nk) * sizeof(float);
}
// Any query width dq (the query row and the scores share the dynamic LDS,
// see above), fp32 or bf16 storage.
// `live` (nullable): skip the launch when it points to 0 (every position
// halted in the previous loop).
void launch_attn_generic(int dtype_bf16, const void* q, const void* k, const void* vt, void* o, int B, int H,
                         int G, int Tq, int cap, int dq, int dv, int kbase, float scale, hipStream_t s,
                         const int32_t* live = nullptr);
// bf16, head width 128, MFMA flash kernel (prefill).  `cap` must be a
// multiple of 8.  lse2 (nullable, fp32 [B][H][Tq]) receives each query row's
// log2 softmax normaliser: p = exp2(score * scale * log2(e) - lse2).
void launch_attn_flash_bf16(const void* q, const void* k, const void* vt, void* o, int B, int H, int G, int Tq,
                            int cap, int kbase, float scale, hipStream_t s, const int32_t* live = nullptr,
                            float* lse2 = nullptr);
// bf16, head width 128, one query per sequence against the cache (decode
// step), H / G <= 16, cap >= 4.  Keys are split over blocks of 512; `part`
// is fp32 scratch of attn_decode_part_floats(B, H, nk) floats.
int attn_decode_blocks(int nk);
inline size_t attn_decode_part_floats(int B, int H, int nk) {
  return (size_t)B * H * attn_decode_blocks(nk) * (128 + 2);
}
void launch_attn_decode_bf16(const void* q, const void* k, const void* vt, void* o, float* part, int B, int H, int G,
                             int cap, int nk, float scale, hipStream_t s);
