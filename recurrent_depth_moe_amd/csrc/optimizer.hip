// AdamW update (decoupled weight decay, bias-corrected moments) over the
// gradient layout: one HBM-bound elementwise pass that also writes the
// block's weights.
#include "optimizer.h"

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// segment of block blockIdx.x (the table holds at most RDT_ADAMW_MAX_SEGS
// entries; kernel arguments are uniform, so the scan runs on the scalar unit)
__device__ __forceinline__ int adamw_seg(const AdamwArgs& a) {
  int s = 0;
  for (int i = 1; i < a.nseg; ++i)
    if ((int)blockIdx.x >= a.seg[i].first_block) s = i;
  return s;
}

__device__ __forceinline__ void adamw_one(const AdamwArgs& a, float g, float& p, float& m, float& v) {
  m = a.beta1 * m + (1.f - a.beta1) * g;
  v = a.beta2 * v + (1.f - a.beta2) * (g * g);
  const float u = (m / a.bc1) / (sqrtf(v / a.bc2) + a.eps) + a.weight_decay * p;
  p = p - a.lr * u;
}

// 256 threads; block b covers RDT_ADAMW_BLOCK consecutive elements of its
// segment, four at a time per thread when the run of four is whole and
// 16-byte aligned in the layout (the weight then 8- or 16-byte aligned).
__global__ __launch_bounds__(256) void adamw_step_kernel(const AdamwArgs a) {
  const int si = adamw_seg(a);
  const AdamwSeg sg = a.seg[si];
  const int64_t base = (int64_t)(blockIdx.x - sg.first_block) * RDT_ADAMW_BLOCK;
  const bool vec_ok = (sg.off & 3) == 0 && ((uintptr_t)sg.dst & (sg.bf16 ? 7 : 15)) == 0;
  if (vec_ok && base + RDT_ADAMW_BLOCK <= sg.numel) {
    // a whole block: every load of the thread's 16 elements is issued
    // before the arithmetic; each value is read and written once, so the
    // accesses are marked non-temporal
    constexpr int IT = RDT_ADAMW_BLOCK / 1024;
    f32x4_t g[IT], p[IT], m[IT], v[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int64_t o = sg.off + base + it * 1024 + threadIdx.x * 4;
      g[it] = __builtin_nontemporal_load((const f32x4_t*)(a.grad + o));
      p[it] = __builtin_nontemporal_load((const f32x4_t*)(a.master + o));
      m[it] = __builtin_nontemporal_load((const f32x4_t*)(a.m + o));
      v[it] = __builtin_nontemporal_load((const f32x4_t*)(a.v + o));
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int64_t e0 = base + it * 1024 + threadIdx.x * 4;
      const int64_t o = sg.off + e0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float pj = p[it][j], mj = m[it][j], vj = v[it][j];
        adamw_one(a, g[it][j], pj, mj, vj);
        p[it][j] = pj;
        m[it][j] = mj;
        v[it][j] = vj;
      }
      __builtin_nontemporal_store(p[it], (f32x4_t*)(a.master + o));
      __builtin_nontemporal_store(m[it], (f32x4_t*)(a.m + o));
      __builtin_nontemporal_store(v[it], (f32x4_t*)(a.v + o));
      if (sg.bf16) {
        u32x2_t w;
        w[0] = pack_bf16x2(p[it][0], p[it][1]);
        w[1] = pack_bf16x2(p[it][2], p[it][3]);
        __builtin_nontemporal_store(w, (u32x2_t*)((bf16_t*)sg.dst + e0));
      } else {
        __builtin_nontemporal_store(p[it], (f32x4_t*)((float*)sg.dst + e0));
      }
    }
    return;
  }
  for (int it = 0; it < RDT_ADAMW_BLOCK / 1024; ++it) {
    const int64_t e0 = base + it * 1024 + threadIdx.x * 4;
    if (e0 >= sg.numel) break;
    const int64_t o = sg.off + e0;
    if (vec_ok && e0 + 4 <= sg.numel) {
      const float4 g = *(const float4*)(a.grad + o);
      float4 p = *(const float4*)(a.master + o);
      float4 m = *(const float4*)(a.m + o);
      float4 v = *(const float4*)(a.v + o);
      adamw_one(a, g.x, p.x, m.x, v.x);
      adamw_one(a, g.y, p.y, m.y, v.y);
      adamw_one(a, g.z, p.z, m.z, v.z);
      adamw_one(a, g.w, p.w, m.w, v.w);
      *(float4*)(a.master + o) = p;
      *(float4*)(a.m + o) = m;
      *(float4*)(a.v + o) = v;
      if (sg.bf16) {
        uint2 w;
        w.x = pack_bf16x2(p.x, p.y);
        w.y = pack_bf16x2(p.z, p.w);
        *(uint2*)((bf16_t*)sg.dst + e0) = w;
      } else {
        *(float4*)((float*)sg.dst + e0) = p;
      }
    } else {
      for (int j = 0; j < 4 && e0 + j < sg.numel; ++j) {
        float p = a.master[o + j], m = a.m[o + j], v = a.v[o + j];
        adamw_one(a, a.grad[o + j], p, m, v);
        a.master[o + j] = p;
        a.m[o + j] = m;
        a.v[o + j] = v;
        if (sg.bf16)
          ((bf16_t*)sg.dst)[e0 + j] = f2bf(p);
        else
          ((float*)sg.dst)[e0 + j] = p;
      }
    }
  }
}

__global__ __launch_bounds__(256) void adamw_init_kernel(const AdamwArgs a) {
  const int si = adamw_seg(a);
  const AdamwSeg sg = a.seg[si];
  const int64_t base = (int64_t)(blockIdx.x - sg.first_block) * RDT_ADAMW_BLOCK;
  for (int it = 0; it < RDT_ADAMW_BLOCK / 256; ++it) {
    const int64_t e = base + it * 256 + threadIdx.x;
    if (e >= sg.numel) break;
    const int64_t o = sg.off + e;
    a.master[o] = sg.bf16 ? bf2f(((const bf16_t*)sg.dst)[e]) : ((const float*)sg.dst)[e];
    a.m[o] = 0.f;
    a.v[o] = 0.f;
  }
}

}  // namespace

void launch_adamw_step(const AdamwArgs& a, hipStream_t s) {
  if (a.nblocks > 0) adamw_step_kernel<<<a.nblocks, 256, 0, s>>>(a);
}

void launch_adamw_init(const AdamwArgs& a, hipStream_t s) {
  if (a.nblocks > 0) adamw_init_kernel<<<a.nblocks, 256, 0, s>>>(a);
}
