// Causal attention of the recurrent block (GQA; MLA after its K/V rebuild).
//
// Layouts (per loop): q [B][H][Tq][dq]; K [B][G][cap][dq]; V transposed
// [B][G][dv][cap]; output o [B][Tq][H][dv] (= [N][H*dv], the O-projection
// input).  Query i sits at buffer index kbase + i and sees buffer keys
// [0, kbase + i]; query head h reads KV head h / (H / G).
#include "attention.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

// ------------------------------------------------------------ generic
// One wave per (query, head): scores to LDS, exact softmax, then P.V.
// Used by the fp32 configs (small head widths, MLA) and by decode steps.
template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ vt, T* __restrict__ o,
                                                          int H, int G, int Tq, int cap, int dq, int dv,
                                                          int kbase, float scale) {
  extern __shared__ float sm[];
  float* qs = sm;          // [dq]
  float* sc = sm + 128;    // [nk]
  const int i = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H, g = h / (H / G);
  const int lane = threadIdx.x;
  const int nk = kbase + i + 1;
  const T* qr = q + ((int64_t)(b * H + h) * Tq + i) * dq;
  const T* kb = k + (int64_t)(b * G + g) * cap * dq;
  const T* vb = vt + (int64_t)(b * G + g) * dv * cap;
  for (int d = lane; d < dq; d += 64) qs[d] = St<T>::ld(qr + d);
  __syncthreads();
  float mx = -INFINITY;
  for (int j = lane; j < nk; j += 64) {
    const T* kr = kb + (int64_t)j * dq;
    float s = 0.f;
    for (int d = 0; d < dq; ++d) s = fmaf(qs[d], St<T>::ld(kr + d), s);
    s *= scale;
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int j = lane; j < nk; j += 64) {
    const float p = expf(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  __syncthreads();
  const float inv = 1.0f / sum;
  T* orow = o + ((int64_t)(b * Tq + i) * H + h) * dv;
  for (int d = lane; d < dv; d += 64) {
    const T* vr = vb + (int64_t)d * cap;
    float acc = 0.f;
    for (int j = 0; j < nk; ++j) acc = fmaf(sc[j], St<T>::ld(vr + j), acc);
    St<T>::st(orow + d, acc * inv);
  }
}

// ------------------------------------------------------------ flash, bf16, d=128
// Block = 4 wave64s = 128 queries of one (b, h); each wave owns 32 queries.
// Per 64-key tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on the
// row axis, queries on the column axis, so lane l keeps query l % 32 for the
// whole kernel and the softmax statistics never leave the lane pair l,
// l ^ 32), online softmax in fp32, then O^T += V^T P^T with P packed from the
// S^T accumulators straight into the B operand.  A 32x32 accumulator holds,
// in lane l and element e, row 8*(e/4) + 4*(l/32) + e%4 and column l%32, so
// elements 0..7 of a 32-key block cover keys {4g..4g+3, 8+4g..8+4g+3}
// (g = l/32) -- together with the other lane half, keys 0..15 -- and the
// V^T fragment is read with the same key order.
constexpr int FD = 128, FBQ = 128, FBK = 64;

__global__ __launch_bounds__(256, 2) void attn_flash_bf16_kernel(const bf16_t* __restrict__ q,
                                                                  const bf16_t* __restrict__ k,
                                                                  const bf16_t* __restrict__ vt,
                                                                  bf16_t* __restrict__ o, int H, int G, int Tq,
                                                                  int cap, int kbase, float scale_log2) {
  __shared__ uint4 sK[2][FBK * 16];   // [key][16 chunks of 8 d], chunk ^ (key & 15)
  __shared__ uint4 sV[2][FD * 8];     // [d][8 chunks of 8 keys], chunk ^ ((d >> 1) & 7)
  const int nqt = (Tq + FBQ - 1) / FBQ;
  const int qt = nqt - 1 - blockIdx.x;   // longest tiles first
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5;            // which 4-row group of each 8 the lane holds
  const int myq = qt * FBQ + w * 32 + (lane & 31);

  // Q as the B operand: lane holds Q[myq][16 ds + 8 half .. +7], ds = 0..7
  bf16x8_t qf[8];
  {
    const bf16_t* qr = q + ((int64_t)(b * H + h) * Tq + min(myq, Tq - 1)) * FD;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      uint4 v = *(const uint4*)(qr + ds * 16 + half * 8);
      if (myq >= Tq) v = uint4{0u, 0u, 0u, 0u};
      qf[ds] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const bf16_t* kb = k + (int64_t)(b * G + g) * cap * FD;
  const bf16_t* vb = vt + (int64_t)(b * G + g) * FD * cap;
  const int kv_valid = kbase + Tq;
  const int kend = min(kbase + min(qt * FBQ + FBQ, Tq), kv_valid);   // last visible key + 1
  const int ntiles = (kend + FBK - 1) / FBK;

  floatx16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Direct-to-LDS tile loads: lane i of each load fills 16-byte slot i of
  // a 1 KB window, so the swizzles are applied by choosing the source chunk.
  // Every tile read stays inside the buffers (their capacity is a multiple
  // of 64 keys); keys past kv_valid are masked (S) or zeroed (V) below.
  auto issue = [&](int buf, int t) {
    const int k0 = t * FBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = (j * 4 + w) * 64 + lane;            // K slot: row sl/16, position sl%16
      const int kr = sl >> 4, kc = (sl & 15) ^ (kr & 15);
      __builtin_amdgcn_global_load_lds((const void*)(kb + (int64_t)(k0 + kr) * FD + kc * 8),
                                       (lds_void_t*)&sK[buf][(j * 4 + w) * 64], 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = (j * 4 + w) * 64 + lane;            // V^T slot: row sl/8, position sl%8
      const int vd = sl >> 3, vc = (sl & 7) ^ ((vd >> 1) & 7);
      __builtin_amdgcn_global_load_lds((const void*)(vb + (int64_t)vd * cap + k0 + vc * 8),
                                       (lds_void_t*)&sV[buf][(j * 4 + w) * 64], 16, 0, 0);
    }
  };

  if (ntiles > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int qlim = kbase + myq;      // last visible key of this lane's query
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) issue(buf ^ 1, t + 1);
    // S^T for two key blocks of 32: 8 chained k-steps of 16 d each
    floatx16_t s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb2][e] = 0.f;
    // K fragments in two batches of 8 reads, each batch in flight before
    // its MFMAs
#pragma unroll
    for (int dh2 = 0; dh2 < 2; ++dh2) {
      bf16x8_t kf[4][2];
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int kr = kb2 * 32 + (lane & 31);
          const int ch = (dh2 * 4 + dd) * 2 + half;
          kf[dd][kb2] = __builtin_bit_cast(bf16x8_t, sK[buf][kr * 16 + (ch ^ (kr & 15))]);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dd][kb2], qf[dh2 * 4 + dd], s[kb2], 0, 0, 0);
    }
    // mask + online softmax
    const int k0 = t * FBK;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + kb2 * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        float v = s[kb2][e] * scale_log2;
        if (key > qlim || key >= kv_valid) v = -INFINITY;
        s[kb2][e] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    // masked scores are -inf: with a finite reference they give exp2 = 0;
    // a row with nothing visible yet uses reference 0 so no NaN appears
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
    bf16x8_t pf[4];   // key steps of 16: (kb2, elements 0..7) and (kb2, 8..15)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          p[x] = __builtin_amdgcn_exp2f(s[kb2][hh * 8 + x] - m_use);
          psum += p[x];
        }
        const uint4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
        pf[kb2 * 2 + hh] = __builtin_bit_cast(bf16x8_t, pk);
      }
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; key step ks covers keys
    // 16 ks .. 16 ks + 15 in the slot order of pf
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + (lane & 31);
        const int key_a = ks * 16 + 4 * half;        // slots 0..3
        const int key_b = ks * 16 + 8 + 4 * half;    // slots 4..7
        const uint2* row = (const uint2*)&sV[buf][d * 8];
        const int sw = (d >> 1) & 7;
        uint2 va = row[(((key_a >> 3) ^ sw) << 1) + ((key_a >> 2) & 1)];
        uint2 vb2 = row[(((key_b >> 3) ^ sw) << 1) + ((key_b >> 2) & 1)];
        if (k0 + FBK > kv_valid) {   // zero V past the buffer's valid keys
          const int ka = k0 + key_a, kb_ = k0 + key_b;
          va.x = (ka + 1 < kv_valid) ? va.x : (ka < kv_valid ? (va.x & 0xffffu) : 0u);
          va.y = (ka + 3 < kv_valid) ? va.y : (ka + 2 < kv_valid ? (va.y & 0xffffu) : 0u);
          vb2.x = (kb_ + 1 < kv_valid) ? vb2.x : (kb_ < kv_valid ? (vb2.x & 0xffffu) : 0u);
          vb2.y = (kb_ + 3 < kv_valid) ? vb2.y : (kb_ + 2 < kv_valid ? (vb2.y & 0xffffu) : 0u);
        }
        const uint4 vv = {va.x, va.y, vb2.x, vb2.y};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pf[ks], oacc[db], 0, 0, 0);
      }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (myq < Tq) {
    const float inv = 1.0f / l_run;
    bf16_t* orow = o + ((int64_t)(b * Tq + myq) * H + h) * FD;
    // lane holds d = 32 db + 8 (e/4) + 4 half + e%4
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const uint2 ov = {pack_bf16x2(oacc[db][e4 * 4] * inv, oacc[db][e4 * 4 + 1] * inv),
                          pack_bf16x2(oacc[db][e4 * 4 + 2] * inv, oacc[db][e4 * 4 + 3] * inv)};
        *(uint2*)(orow + db * 32 + 8 * e4 + 4 * half) = ov;
      }
  }
}

}  // namespace

void launch_attn_generic(int dtype_bf16, const void* q, const void* k, const void* vt, void* o, int B, int H,
                         int G, int Tq, int cap, int dq, int dv, int kbase, float scale, hipStream_t s) {
  const dim3 grid(Tq, B * H), block(64);
  const size_t shm = (128 + (size_t)(kbase + Tq)) * sizeof(float);
  if (dtype_bf16)
    attn_generic_kernel<bf16_t><<<grid, block, shm, s>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)vt,
                                                         (bf16_t*)o, H, G, Tq, cap, dq, dv, kbase, scale);
  else
    attn_generic_kernel<float><<<grid, block, shm, s>>>((const float*)q, (const float*)k, (const float*)vt,
                                                        (float*)o, H, G, Tq, cap, dq, dv, kbase, scale);
}

void launch_attn_flash_bf16(const void* q, const void* k, const void* vt, void* o, int B, int H, int G, int Tq,
                            int cap, int kbase, float scale, hipStream_t s) {
  const dim3 grid((Tq + FBQ - 1) / FBQ, B * H), block(256);
  const float scale_log2 = scale * 1.4426950408889634f;
  attn_flash_bf16_kernel<<<grid, block, 0, s>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)vt, (bf16_t*)o,
                                                H, G, Tq, cap, kbase, scale_log2);
}
