// Causal attention of the recurrent block (GQA; MLA after its K/V rebuild).
//
// Layouts (per loop): q [B][H][Tq][dq]; K [B][G][cap][dq]; V transposed
// [B][G][dv][cap]; output o [B][Tq][H][dv] (= [N][H*dv], the O-projection
// input).  Query i sits at buffer index kbase + i and sees buffer keys
// [0, kbase + i]; query head h reads KV head h / (H / G).
#include "attention.h"

#include <type_traits>

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

// global -> LDS copy of 16 bytes per lane into the 1 KB window at lds (lane
// i fills bytes 16 i .. 16 i + 15), written as asm so the compiler does not
// add its own vmcnt wait before every later LDS read: the caller waits
// explicitly before reading the window.
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m) : "memory", "m0");
}

// ------------------------------------------------------------ generic
// One wave per (query, head): scores to LDS, exact softmax, then P.V.
// Used by the fp32 configs (small head widths, MLA) and by decode steps.
template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ vt, T* __restrict__ o,
                                                          int H, int G, int Tq, int cap, int dq, int dv,
                                                          int kbase, float scale, const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  extern __shared__ float sm[];
  float* qs = sm;                     // [dq]
  float* sc = sm + attn_generic_qslots(dq);   // [nk]
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
// in lane l and element e, row 8*(e/4) + 4*(l/32) + e%4 and column l%32;
// the K rows are fed to the MFMA in the order that maps those rows of lane
// half g to the keys 16g .. 16g+15 of each 32-key block, so the V^T
// fragment of a P V key step is one 16-byte LDS read per lane.
constexpr int FD = 128, FBQ = 128, FBK = 64;

// K tile row kr keeps its 16-byte chunk c at position c ^ kswz(kr).  The
// 16 lanes of a quarter-wave read rows {r..r+3, r+16..r+19, r+4..r+7,
// r+20..r+23} (r a multiple of 8, see kperm), which kswz sends to 16
// distinct positions: one 256-byte bank sweep, no conflicts.
__device__ __forceinline__ int kswz(int kr) { return (kr & 7) | (((kr >> 4) & 1) << 3); }

__global__ __launch_bounds__(256, 2) void attn_flash_bf16_kernel(const bf16_t* __restrict__ q,
                                                                  const bf16_t* __restrict__ k,
                                                                  const bf16_t* __restrict__ vt,
                                                                  bf16_t* __restrict__ o, int H, int G, int Tq,
                                                                  int cap, int kbase, float scale_log2,
                                                                  const int32_t* live, float* __restrict__ lse2) {
  RDT_SKIP_IF_ALL_HALTED(live);
  __shared__ uint4 sK[2][FBK * 16];   // [key][16 chunks of 8 d], chunk ^ (key & 15)
  __shared__ uint4 sV[2][FD * 8];     // [d][8 chunks of 8 keys], chunk ^ ((d >> 1) & 7)
  // Block order: longest query tiles first.  When the (b, kv head) groups
  // split evenly over the XCDs, each XCD takes its own groups (blocks go to
  // XCDs round-robin by linear index), so the K / V tiles its blocks stream
  // stay in that XCD's L2.
  const int nqt = (Tq + FBQ - 1) / FBQ, rep = H / G;
  int qt, b, h;
  {
    const int L = blockIdx.x, BG = gridDim.x / (nqt * rep);
    if (BG % RDT_NUM_XCD == 0) {
      const int ppc = BG / RDT_NUM_XCD, xcd = L % RDT_NUM_XCD, j = L / RDT_NUM_XCD;
      const int rank = j / (ppc * rep), rest = j - rank * (ppc * rep);
      const int bg = xcd * ppc + rest / rep;
      qt = nqt - 1 - rank;
      b = bg / G;
      h = (bg - b * G) * rep + (rest % rep);
    } else {
      const int rank = L / (BG * rep), bh = L - rank * (BG * rep);
      qt = nqt - 1 - rank;
      b = bh / H;
      h = bh - b * H;
    }
  }
  const int g = h / rep;
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
  float l_run = 0.f;

  // Direct-to-LDS tile loads: lane i of each load fills 16-byte slot i of
  // a 1 KB window, so the swizzles are applied by choosing the source chunk.
  // Every tile read stays inside the buffers (their capacity is a multiple
  // of 64 keys); keys past kv_valid are masked (S) or zeroed (V) below.
  auto issue = [&](int buf, int t) {
    const int k0 = t * FBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = (j * 4 + w) * 64 + lane;            // K slot: row sl/16, position sl%16
      const int kr = sl >> 4, kc = (sl & 15) ^ kswz(kr);
      dma16(kb + (int64_t)(k0 + kr) * FD + kc * 8, &sK[buf][(j * 4 + w) * 64]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = (j * 4 + w) * 64 + lane;            // V^T slot: row sl/8, position sl%8
      const int vd = sl >> 3, vc = (sl & 7) ^ ((vd >> 1) & 7);
      dma16(vb + (int64_t)vd * cap + k0 + vc * 8, &sV[buf][(j * 4 + w) * 64]);
    }
  };

  // The tile holding the end of the keys gets its V^T entries past kv_valid
  // zeroed in LDS once (the buffers past the last position hold whatever
  // the caller or an earlier call left there), so the P V reads need no
  // per-element masking; the scores of those keys are masked to -inf.
  auto zero_v_tail = [&](int buf, int k0) {
    const int nvalid = kv_valid - k0;
    unsigned short* sv = (unsigned short*)&sV[buf][0];
    for (int idx = tid; idx < FD * FBK; idx += 256) {
      const int d = idx >> 6, key = idx & (FBK - 1);
      if (key >= nvalid) sv[(d * 8 + ((key >> 3) ^ ((d >> 1) & 7))) * 8 + (key & 7)] = 0;
    }
  };
  if (ntiles > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (ntiles > 0 && FBK > kv_valid) {
    zero_v_tail(0, 0);
    __syncthreads();
  }
  const int qlim = kbase + myq;      // last visible key of this lane's query
  // K row this lane feeds into S^T: accumulator row r holds key
  // 16 ((r >> 2) & 1) + 4 (r >> 3) + r % 4 of each 32-key block, so lane
  // half g ends up with the 16 consecutive keys 16 g .. 16 g + 15 (element
  // e = key 16 g + e) and each P V key step reads whole V^T chunks
  const int kperm = 16 * (((lane & 31) >> 2) & 1) + 4 * ((lane & 31) >> 3) + (lane & 3);
  const int wfirst = kbase + qt * FBQ + w * 32;   // last key every query of this wave sees
  const int wlast = wfirst + 31;                  // last key any query of this wave sees
  // Softmax reference: m_ref trails the running maximum and is moved (with
  // O and l rescaled) only when some query of the wave would otherwise get
  // p above 2^8; O / l does not depend on the reference, and p <= 256 is
  // exact enough in bf16 and far from overflow in the fp32 sums.
  float m_ref = -INFINITY;
  const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  auto tile = [&](auto masked, int t, int buf) {
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
          const int kr = kb2 * 32 + kperm;
          const int ch = (dh2 * 4 + dd) * 2 + half;
          kf[dd][kb2] = __builtin_bit_cast(bf16x8_t, sK[buf][kr * 16 + (ch ^ kswz(kr))]);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dd][kb2], qf[dh2 * 4 + dd], s[kb2], 0, 0, 0);
    }
    const int k0 = t * FBK;
    if constexpr (decltype(masked)::value) {
      // a tile that crosses this wave's diagonal or the key end
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb2 * 32 + 16 * half + e;
          if (key > qlim || key >= kv_valid) s[kb2][e] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[kb2][e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_ref, tmax);
    if (__any((m_new - m_ref) * scale_log2 > 8.f)) {
      // (kept a real branch: the rescale is rare and 64 multiplies long)
      asm volatile("" ::: "memory");
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * scale_log2);
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
      l_run *= alpha;
      m_ref = m_new;
    }
    // masked scores are -inf: with a finite reference they give exp2 = 0;
    // a row with nothing visible yet uses reference 0 so no NaN appears
    const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * scale_log2;
    float psum = 0.f;
    bf16x8_t pf[4];   // key steps of 16: (kb2, elements 0..7) and (kb2, 8..15)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) p[x] = __builtin_amdgcn_exp2f(fmaf(s[kb2][hh * 8 + x], scale_log2, -mc));
        const uint4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
        // l sums the bf16 values the P V product uses
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk.x), ones2, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk.y), ones2, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk.z), ones2, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk.w), ones2, psum, false);
        pf[kb2 * 2 + hh] = __builtin_bit_cast(bf16x8_t, pk);
      }
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;
    // O^T[d][q] += V^T[d][keys] P^T[keys][q]; key step ks = 2 kb2 + hh
    // takes, from lane half g, keys 32 kb2 + 16 g + 8 hh .. +7: one
    // 16-byte chunk of the V^T row
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + (lane & 31);
        const int ch = 4 * (ks >> 1) + 2 * half + (ks & 1);
        const uint4 vv = sV[buf][d * 8 + (ch ^ ((d >> 1) & 7))];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pf[ks], oacc[db], 0, 0, 0);
      }
  };
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) issue(buf ^ 1, t + 1);
    if (t * FBK <= wlast) {   // else every key of the tile is past this wave's queries
      const int k0 = t * FBK;
      if (k0 + FBK - 1 > wfirst || k0 + FBK > kv_valid) tile(std::true_type{}, t, buf);
      else tile(std::false_type{}, t, buf);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles && (t + 2) * FBK > kv_valid) {
      zero_v_tail(buf ^ 1, (t + 1) * FBK);
      __syncthreads();
    }
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
    // log2 of the row's softmax normaliser in the exp2 domain of the scores
    // (p = exp2(s * scale_log2 - lse2)), kept for the backward pass
    if (lse2 != nullptr && half == 0) {
      const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * scale_log2;
      lse2[(int64_t)(b * H + h) * Tq + myq] = mc + __log2f(l_run);
    }
  }
}


// ------------------------------------------------------------ split-KV decode, bf16, d=128
// One query per sequence (a decode step against the cache).  The visible
// keys of each (b, kv head) are cut into blocks of DEC_BLK; a block is four
// wave64s, each owning DEC_U consecutive keys and ALL query heads of the kv
// group at once (up to 16), so every cached K / V byte is read from HBM
// exactly once.  Both products run on v_mfma_f32_16x16x32_bf16 with the K
// and V^T fragments loaded straight from global memory (each fragment is
// used once; LDS staging would only add a copy):
//   S^T = K Q^T : A = 16 keys x 32 dims, B = Q^T (heads on the column axis),
//                 lane l gets keys 4*(l/16)+i of the 16-key group for head l%16;
//   O   = P V   : A = P with lane l holding head l%16 at the eight keys it
//                 already scored in two adjacent groups (the key slots are
//                 ordered so those eight are consecutive), B = V read from
//                 V^T in that same key order (one 16-byte piece per lane).
// Each wave takes an exact softmax over its keys (scores stay in registers),
// the four waves merge through LDS, and the block leaves one partial
// (max, sum, unnormalised o) per head; a second kernel merges the partials
// of a row in block order, so the result does not depend on timing.
constexpr int DEC_U = 128, DEC_BLK = 4 * DEC_U, DEC_D = 128, DEC_MAXREP = 16;

__device__ __forceinline__ uint32_t keep_keys(uint32_t pair, int key, int nk) {
  // zero the bf16 halves of keys >= nk (the cache past the last position
  // holds whatever the caller left there)
  const uint32_t lo = key < nk ? 0xffffu : 0u, hi = key + 1 < nk ? 0xffff0000u : 0u;
  return pair & (lo | hi);
}

__global__ __launch_bounds__(256) void attn_decode_split_kernel(const bf16_t* __restrict__ q,
                                                                 const bf16_t* __restrict__ k,
                                                                 const bf16_t* __restrict__ vt,
                                                                 float* __restrict__ part_o,
                                                                 float* __restrict__ part_ml, int H, int G,
                                                                 int cap, int nk, float scale_log2) {
  __shared__ float sO[4][DEC_MAXREP][DEC_D + 4];
  __shared__ float sM[4][DEC_MAXREP], sL[4][DEC_MAXREP];
  const int nblk = gridDim.x, blk = blockIdx.x, bg = blockIdx.y;
  const int b = bg / G, g = bg - b * G, rep = H / G;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, qd = lane >> 4, c16 = lane & 15;
  const int j0 = blk * DEC_BLK + w * DEC_U;
  const bf16_t* kb = k + (int64_t)bg * cap * DEC_D;
  const bf16_t* vb = vt + (int64_t)bg * DEC_D * cap;

  // Q^T as the B operand: lane l holds head c16 of this group, dims 32 ds + 8 qd .. +7
  bf16x8_t qf[4];
  {
    const bool hv = c16 < rep;
    const bf16_t* qr = q + (int64_t)(b * H + g * rep + (hv ? c16 : 0)) * DEC_D + 8 * qd;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      uint4 v = *(const uint4*)(qr + 32 * ds);
      if (!hv) v = uint4{0u, 0u, 0u, 0u};
      qf[ds] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Scores of 8 groups of 16 key slots.  Slot s of group gi = 2 c + h is key
  // j0 + 32 c + 8 (s / 4) + 4 h + s % 4, so accumulator element i of lane
  // (qd, c16) in groups 2c and 2c+1 holds keys j0 + 32 c + 8 qd + i and
  // + 4 + i: eight consecutive keys, which is the k order P takes into the
  // P V product and lets each lane read V^T in 16-byte pieces.  All K loads
  // are issued before the first product, the V^T loads right after the
  // products (they do not depend on the scores), so the waits come once.
  uint4 kv4[8][4];
#pragma unroll
  for (int gi = 0; gi < 8; ++gi) {
    const int key = min(j0 + 32 * (gi >> 1) + 8 * (c16 >> 2) + 4 * (gi & 1) + (c16 & 3), cap - 1);
    const bf16_t* kr = kb + (int64_t)key * DEC_D + 8 * qd;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) kv4[gi][ds] = *(const uint4*)(kr + 32 * ds);
  }
  __builtin_amdgcn_sched_barrier(0);
  floatx4_t sc[8];
#pragma unroll
  for (int gi = 0; gi < 8; ++gi) {
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv4[gi][ds]), qf[ds], acc, 0, 0, 0);
    sc[gi] = acc;
  }
  // V^T: dim 16 db + c16, keys j0 + 32 c + 8 qd .. + 7 (cap is a multiple of
  // 64, so the clamped start stays 16-byte aligned; a clamped piece lies
  // wholly past the last key and is zeroed below)
  uint4 vv[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ka = min(j0 + 32 * c + 8 * qd, cap - 8);
#pragma unroll
    for (int db = 0; db < 8; ++db) vv[c][db] = *(const uint4*)(vb + (int64_t)(16 * db + c16) * cap + ka);
  }
  __builtin_amdgcn_sched_barrier(0);
  float m = -INFINITY;
#pragma unroll
  for (int gi = 0; gi < 8; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = j0 + 32 * (gi >> 1) + 8 * qd + 4 * (gi & 1) + i;
      const float v = key < nk ? sc[gi][i] * scale_log2 : -INFINITY;
      sc[gi][i] = v;
      m = fmaxf(m, v);
    }
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  const float mu = m == -INFINITY ? 0.f : m;   // a wave past the last key keeps p = 0
  float l = 0.f;
  bf16x8_t pf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float pv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(sc[2 * c][i] - mu);
      pv[4 + i] = __builtin_amdgcn_exp2f(sc[2 * c + 1][i] - mu);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) l += pv[i];
    uint4 u;
    u.x = pack_bf16x2(pv[0], pv[1]);
    u.y = pack_bf16x2(pv[2], pv[3]);
    u.z = pack_bf16x2(pv[4], pv[5]);
    u.w = pack_bf16x2(pv[6], pv[7]);
    pf[c] = __builtin_bit_cast(bf16x8_t, u);
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);

  // O = P V over 4 blocks of 32 keys x 8 blocks of 16 dims
  floatx4_t o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int k0 = j0 + 32 * c + 8 * qd;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint4 u;
      u.x = keep_keys(vv[c][db].x, k0, nk);
      u.y = keep_keys(vv[c][db].y, k0 + 2, nk);
      u.z = keep_keys(vv[c][db].z, k0 + 4, nk);
      u.w = keep_keys(vv[c][db].w, k0 + 6, nk);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[c], __builtin_bit_cast(bf16x8_t, u), o[db], 0, 0, 0);
    }
  }

  // merge the four waves: o[db][i] is head 4 qd + i, dim 16 db + c16
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) sO[w][4 * qd + i][16 * db + c16] = o[db][i];
  if (qd == 0) {
    sM[w][c16] = m;
    sL[w][c16] = l;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rep * DEC_D; idx += 256) {
    const int hh = idx / DEC_D, d = idx - hh * DEC_D;
    float M = sM[0][hh];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, sM[ww][hh]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = sM[ww][hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sM[ww][hh] - M);
      L += f * sL[ww][hh];
      acc += f * sO[ww][hh][d];
    }
    const int64_t row = (int64_t)(b * H + g * rep + hh) * nblk + blk;
    part_o[row * DEC_D + d] = acc;
    if (d == 0) {
      part_ml[row * 2] = M;
      part_ml[row * 2 + 1] = L;
    }
  }
}

// merge the per-block partials of one (b, head) in block order
__global__ __launch_bounds__(DEC_D) void attn_decode_merge_kernel(const float* __restrict__ part_o,
                                                                   const float* __restrict__ part_ml,
                                                                   bf16_t* __restrict__ o, int nblk) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* ml = part_ml + (int64_t)bh * nblk * 2;
  float M = -INFINITY;
  for (int j = 0; j < nblk; ++j) M = fmaxf(M, ml[2 * j]);
  float L = 0.f, acc = 0.f;
  for (int j = 0; j < nblk; ++j) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * j] - M);
    L += f * ml[2 * j + 1];
    acc += f * part_o[((int64_t)bh * nblk + j) * DEC_D + d];
  }
  o[(int64_t)bh * DEC_D + d] = f2bf(acc / L);
}

}  // namespace

void launch_attn_generic(int dtype_bf16, const void* q, const void* k, const void* vt, void* o, int B, int H,
                         int G, int Tq, int cap, int dq, int dv, int kbase, float scale, hipStream_t s,
                         const int32_t* live) {
  const dim3 grid(Tq, B * H), block(64);
  const size_t shm = attn_generic_lds_bytes(dq, kbase + Tq);
  if (dtype_bf16)
    attn_generic_kernel<bf16_t><<<grid, block, shm, s>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)vt,
                                                         (bf16_t*)o, H, G, Tq, cap, dq, dv, kbase, scale, live);
  else
    attn_generic_kernel<float><<<grid, block, shm, s>>>((const float*)q, (const float*)k, (const float*)vt,
                                                        (float*)o, H, G, Tq, cap, dq, dv, kbase, scale, live);
}

void launch_attn_flash_bf16(const void* q, const void* k, const void* vt, void* o, int B, int H, int G, int Tq,
                            int cap, int kbase, float scale, hipStream_t s, const int32_t* live, float* lse2) {
  const dim3 grid((Tq + FBQ - 1) / FBQ * B * H), block(256);
  const float scale_log2 = scale * 1.4426950408889634f;
  attn_flash_bf16_kernel<<<grid, block, 0, s>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)vt, (bf16_t*)o,
                                                H, G, Tq, cap, kbase, scale_log2, live, lse2);
}

int attn_decode_blocks(int nk) { return (nk + DEC_BLK - 1) / DEC_BLK; }

void launch_attn_decode_bf16(const void* q, const void* k, const void* vt, void* o, float* part, int B, int H, int G,
                             int cap, int nk, float scale, hipStream_t s) {
  const int nblk = attn_decode_blocks(nk);
  float* part_o = part;
  float* part_ml = part + (size_t)B * H * nblk * DEC_D;
  const float scale_log2 = scale * 1.4426950408889634f;
  attn_decode_split_kernel<<<dim3(nblk, B * G), 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)vt,
                                                              part_o, part_ml, H, G, cap, nk, scale_log2);
  attn_decode_merge_kernel<<<B * H, DEC_D, 0, s>>>(part_o, part_ml, (bf16_t*)o, nblk);
}
