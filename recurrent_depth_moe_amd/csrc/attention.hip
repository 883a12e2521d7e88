// Causal attention of the recurrent block (GQA; MLA after its K/V rebuild).
//
// Layouts (per loop): q [B][H][Tq][dq]; K [B][G][cap][dq]; V transposed
// [B][G][dv][cap]; output o [B][Tq][H][dv] (= [N][H*dv], the O-projection
// input).  Query i sits at buffer index kbase + i and sees buffer keys
// [0, kbase + i]; query head h reads KV head h / (H / G).
#include "attention.h"

namespace {

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
// Block = 4 wave64s = 64 queries of one (b, h); each wave owns 16 queries.
// Per 64-key tile: S^T = K Q^T (keys on the MFMA row axis, queries on the
// column axis, so each lane keeps one query for the whole kernel), online
// softmax in fp32, then O^T += V^T P^T with P packed from the S^T
// accumulators straight into the B operand (no LDS round trip).
constexpr int FD = 128, FBQ = 64, FBK = 64;

__global__ __launch_bounds__(256, 2) void attn_flash_bf16_kernel(const bf16_t* __restrict__ q,
                                                                  const bf16_t* __restrict__ k,
                                                                  const bf16_t* __restrict__ vt,
                                                                  bf16_t* __restrict__ o, int H, int G, int Tq,
                                                                  int cap, int kbase, float scale_log2) {
  __shared__ uint4 sK[2][FBK * 16];   // [key][16 chunks of 8 d], chunk ^ (key & 15)
  __shared__ uint4 sV[2][FD * 8];     // [d][8 chunks of 8 keys], chunk ^ (d & 7)
  const int nqt = (Tq + FBQ - 1) / FBQ;
  const int qt = nqt - 1 - blockIdx.x;   // longest tiles first
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qi0 = qt * FBQ + w * 16;     // first query of this wave
  const int myq = qi0 + (lane & 15);     // this lane's query (column of S^T)
  const int grp = lane >> 4;

  // Q fragments as the B operand: lane holds Q[myq][32c + 8grp .. +7]
  bf16x8_t qf[4];
  {
    const bf16_t* qr = q + ((int64_t)(b * H + h) * Tq + min(myq, Tq - 1)) * FD;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = *(const uint4*)(qr + c * 32 + grp * 8);
      if (myq >= Tq) v = uint4{0u, 0u, 0u, 0u};
      qf[c] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const bf16_t* kb = k + (int64_t)(b * G + g) * cap * FD;
  const bf16_t* vb = vt + (int64_t)(b * G + g) * FD * cap;
  const int kv_valid = kbase + Tq;                               // keys in the buffer
  const int kend = min(kbase + min(qt * FBQ + FBQ, Tq), kv_valid); // last visible key + 1
  const int ntiles = (kend + FBK - 1) / FBK;

  floatx4_t oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  uint4 rk[4], rv[4];
  auto gload = [&](int t) {
    const int k0 = t * FBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + j * 256;
      const int kr = idx >> 4, kc = idx & 15;          // K: 64 rows x 16 chunks
      rk[j] = (k0 + kr < kv_valid) ? *(const uint4*)(kb + (int64_t)(k0 + kr) * FD + kc * 8) : uint4{0u, 0u, 0u, 0u};
      const int vd = idx >> 3, vc = idx & 7;           // V^T: 128 rows x 8 chunks
      const int key = k0 + vc * 8;
      if (key + 8 <= kv_valid) {
        rv[j] = *(const uint4*)(vb + (int64_t)vd * cap + key);
      } else {
        bf16_t tmp[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) tmp[x] = (key + x < kv_valid) ? vb[(int64_t)vd * cap + key + x] : (bf16_t)0;
        rv[j] = *(const uint4*)tmp;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + j * 256;
      const int kr = idx >> 4, kc = idx & 15;
      sK[buf][kr * 16 + (kc ^ (kr & 15))] = rk[j];
      const int vd = idx >> 3, vc = idx & 7;
      sV[buf][vd * 8 + (vc ^ (vd & 7))] = rv[j];
    }
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    // S^T for 4 key blocks of 16
    floatx4_t s[4];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      s[kb4] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      const int kr = kb4 * 16 + (lane & 15);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ch = c * 4 + grp;
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, sK[buf][kr * 16 + (ch ^ (kr & 15))]);
        s[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], s[kb4], 0, 0, 0);
      }
    }
    // mask + online softmax (lane's query = myq; keys 4*grp + r of each block)
    const int k0 = t * FBK;
    const int qlim = kbase + myq;      // last visible key of this query
    float tmax = -INFINITY;
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + kb4 * 16 + grp * 4 + r;
        float v = s[kb4][r] * scale_log2;
        if (key > qlim || key >= kv_valid) v = -INFINITY;
        s[kb4][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8_t pf[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16_t pv[8];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = (m_new == -INFINITY) ? 0.f : exp2f(s[kc * 2 + half][r] - m_new);
          psum += p;
          pv[half * 4 + r] = f2bf(p);
        }
      pf[kc] = __builtin_bit_cast(bf16x8_t, *(const uint4*)pv);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 8; ++i) oacc[i] *= alpha;
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; key slots match pf's packing
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = db * 16 + (lane & 15);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int key_a = kc * 32 + grp * 4;        // first 4 keys
        const int key_b = kc * 32 + 16 + grp * 4;   // second 4 keys
        const uint2* row = (const uint2*)&sV[buf][d * 8];
        const int ca = key_a >> 3, cb = key_b >> 3;
        const uint2 va = row[((ca ^ (d & 7)) << 1) + ((key_a >> 2) & 1)];
        const uint2 vb2 = row[((cb ^ (d & 7)) << 1) + ((key_b >> 2) & 1)];
        const uint4 vv = {va.x, va.y, vb2.x, vb2.y};
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv), pf[kc], oacc[db], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }
  if (myq < Tq) {
    const float inv = 1.0f / l_run;
    bf16_t* orow = o + ((int64_t)(b * Tq + myq) * H + h) * FD;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      bf16_t ov[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ov[r] = f2bf(oacc[db][r] * inv);
      *(uint2*)(orow + db * 16 + grp * 4) = *(const uint2*)ov;
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
