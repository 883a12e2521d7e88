// AdamW update of the recurrent block's trained tensors over fp32 master
// weights and moments kept in the gradient buffer's layout.
#pragma once

#include "common.h"

// AdamW over the gradient layout (fp32 master weights, first and second
// moments, each a buffer in that layout).  Segment i is one tensor:
// elements [off, off + numel) of the layout, whose weight lives at dst
// (bf16 when bf16 is set, else fp32); the segments' blocks of
// RDT_ADAMW_BLOCK elements are numbered from first_block.
#define RDT_ADAMW_MAX_SEGS 32
#define RDT_ADAMW_BLOCK 4096
struct AdamwSeg {
  int64_t off, numel;
  void* dst;
  int bf16;
  int first_block;
};
struct AdamwArgs {
  AdamwSeg seg[RDT_ADAMW_MAX_SEGS];
  int nseg, nblocks;
  const float* grad;
  float *master, *m, *v;
  float lr, beta1, beta2, eps, weight_decay;
  float bc1, bc2;  // 1 - beta1^step, 1 - beta2^step
};
// m = beta1 m + (1 - beta1) g, v = beta2 v + (1 - beta2) g^2,
// master -= lr (m / bc1 / (sqrt(v / bc2) + eps) + weight_decay master),
// weight = master (bf16: nearest even)
void launch_adamw_step(const AdamwArgs& a, hipStream_t s);
// master = weight (bf16 widened), m = v = 0, over the segments
void launch_adamw_init(const AdamwArgs& a, hipStream_t s);
