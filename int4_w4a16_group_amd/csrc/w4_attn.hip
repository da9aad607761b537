// Slot-indexed GQA decode attention on gfx950.
//
// KV arena of one layer: per (slot, kv head) a run of 64-position chunks; a
// chunk holds its K block (64 x D) and, in a separate array, its V block, each
// stored in MFMA operand order so that every operand load of a wave is one
// contiguous 1 KB (64 lanes x 16 bytes, with each 4-lane group reading 64
// contiguous bytes, the rate at which the vector memory unit takes 16-byte
// loads):
//   K: (pos, d) at [pt = pos/16][ks = d/32][quad = d%32/8][col = pos%16][d%8],
//      the B operand of S = Q K^T for position tile pt and k-step ks;
//   V: (pos, d) at [dt = d/16][ks = pos/32][quad = pos%32/8][col = d%16][pos%8],
//      the B operand of O = P V for d tile dt and k-step ks.
// A stream reads and writes only its own slot ("Per-stream KV-slot isolation
// ...", section 1: a stable per-stream slot, never wiped when the batch
// changes).
//
// Split-KV: work-group (chunk c, kv head g, stream b) handles positions
// 64c .. 64c+63 of that stream for the n_q/n_kv query heads of head g:
//   S = Q K^T (MFMA, fp32), z = S log2(e) / sqrt(D) (log2 units), masked beyond
//   the stream's p; m_c = max z, P = 2^(z - m_c) (v_exp_f32), l_c = sum P;
//   O_c = P V (MFMA on P split into fp16 hi + lo parts, fp32 accumulate).
// The reduce kernel combines chunks in chunk order:
//   M = max m_c, L = sum l_c 2^(m_c - M), o = sum O_c 2^(m_c - M) / L.
// The chunk count is a function of the stream's own position only, so a
// stream's result is the same in any batch.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

// cos/sin of p * theta^(-2i/D) for p < cap, i < D/2, computed in fp64 and
// rounded to fp32 (table[p][i] = (cos, sin)).
__global__ void k_rope_table(int cap, int D, double theta, float2* table) {
  const int half = D / 2;
  const int n = cap * half;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += gridDim.x * blockDim.x) {
    const int p = idx / half, i = idx - p * half;
    const double ang = (double)p * pow(theta, -2.0 * (double)i / (double)D);
    table[idx] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

hipError_t launch_rope_table(int cap, int D, double theta, float2* table, hipStream_t st) {
  const int n = cap * (D / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((n + 255) / 256), dim3(256), 0, st, cap, D, theta, table);
  return hipGetLastError();
}

// Value of lane (lane's DPP source) within a 16-lane row.
template <int CTRL>
static __device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Max / sum over the 16 lanes of a row: swap neighbours, swap pairs, mirror
// within 8, mirror within 16.  Each step combines two values that the paired
// lane combines in the other order, so every lane ends with the same result.
static __device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  return v;
}
static __device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_f<0xB1>(v);
  v = v + dpp_f<0x4E>(v);
  v = v + dpp_f<0x141>(v);
  v = v + dpp_f<0x140>(v);
  return v;
}

static __device__ __forceinline__ size_t kv_base(const KV& kv, int layer, int slot, int g) {
  return (((size_t)layer * kv.S + slot) * kv.Hkv + g) * (size_t)kv.cap * kv.D;
}
// Offsets of K[p][d] and V[p][d] within a (layer, slot, head) block.
static __device__ __forceinline__ size_t k_off(int D, int p, int d) {
  const int q = p & 63;
  return (size_t)(p >> 6) * 64 * D +
         (size_t)(((((q >> 4) * (D >> 5) + (d >> 5)) * 4 + ((d & 31) >> 3)) * 16 + (q & 15)) * 8 + (d & 7));
}
static __device__ __forceinline__ size_t v_off(int D, int p, int d) {
  const int q = p & 63;
  return (size_t)(p >> 6) * 64 * D + (size_t)(((((d >> 4) * 2 + (q >> 5)) * 4 + ((q & 31) >> 3)) * 16 + (d & 15)) * 8 + (q & 7));
}

// Rotary on the q and k heads of qkv[b] (rotate-half pairs (i, i+D/2)), then
// append k (rotated) and v at position pos[b] of slot[b]; rotated q -> q_out.
__global__ void k_rope_append(int layer, int Hq, KV kv, const int32_t* __restrict__ slot,
                              const int32_t* __restrict__ pos, const uint16_t* __restrict__ qkv, int ldqkv,
                              const float2* __restrict__ table, uint16_t* __restrict__ q_out) {
  const int b = blockIdx.x;
  const int D = kv.D, half = D / 2, Hkv = kv.Hkv;
  const int p = pos[b], s = slot[b];
  const uint16_t* src = qkv + (size_t)b * ldqkv;
  const int npairs = (Hq + Hkv) * half;
  for (int idx = threadIdx.x; idx < npairs; idx += blockDim.x) {
    const int h = idx / half, i = idx - h * half;
    const float2 cs = table[(size_t)p * half + i];
    const float a = h2f(src[h * D + i]), bb = h2f(src[h * D + i + half]);
    const uint16_t o0 = f2h(a * cs.x - bb * cs.y);
    const uint16_t o1 = f2h(a * cs.y + bb * cs.x);
    if (h < Hq) {
      q_out[((size_t)b * Hq + h) * D + i] = o0;
      q_out[((size_t)b * Hq + h) * D + i + half] = o1;
    } else {
      uint16_t* kb = kv.K + kv_base(kv, layer, s, h - Hq);
      kb[k_off(D, p, i)] = o0;
      kb[k_off(D, p, i + half)] = o1;
    }
  }
  const uint16_t* vsrc = src + (Hq + Hkv) * D;
  for (int idx = threadIdx.x; idx < Hkv * D; idx += blockDim.x) {
    const int g = idx / D, d = idx - g * D;
    kv.VT[kv_base(kv, layer, s, g) + v_off(D, p, d)] = vsrc[idx];
  }
}

hipError_t launch_rope_append(int B, int layer, int Hq, const KV& kv, const int32_t* slot, const int32_t* pos,
                              const uint16_t* qkv, int ldqkv, const float2* table, uint16_t* q_out,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_rope_append, dim3(B), dim3(256), 0, st, layer, Hq, kv, slot, pos, qkv, ldqkv, table, q_out);
  return hipGetLastError();
}

__global__ void k_append(int layer, KV kv, const int32_t* __restrict__ slot, const int32_t* __restrict__ pos,
                         const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new) {
  const int b = blockIdx.x;
  const int p = pos[b], s = slot[b], D = kv.D;
  for (int idx = threadIdx.x; idx < kv.Hkv * D; idx += blockDim.x) {
    const int g = idx / D, d = idx - g * D;
    const size_t base = kv_base(kv, layer, s, g);
    kv.K[base + k_off(D, p, d)] = k_new[(size_t)b * kv.Hkv * D + idx];
    kv.VT[base + v_off(D, p, d)] = v_new[(size_t)b * kv.Hkv * D + idx];
  }
}

hipError_t launch_append(int B, int layer, const KV& kv, const int32_t* slot, const int32_t* pos,
                         const uint16_t* k_new, const uint16_t* v_new, hipStream_t st) {
  hipLaunchKernelGGL(k_append, dim3(B), dim3(256), 0, st, layer, kv, slot, pos, k_new, v_new);
  return hipGetLastError();
}

// Seed a slot from canonical k, v [L][P][Hkv][D].  Block (pos chunk of 64, layer*Hkv + g).
__global__ void k_seed(int P, int slot, KV kv, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v) {
  const int p0 = blockIdx.x * 64;
  const int l = blockIdx.y / kv.Hkv, g = blockIdx.y - l * kv.Hkv;
  const int D = kv.D;
  const size_t base = kv_base(kv, l, slot, g);
  const int np = min(64, P - p0);
  for (int idx = threadIdx.x; idx < np * D; idx += blockDim.x) {
    const int pp = idx / D, d = idx - pp * D;
    const size_t src = (((size_t)l * P + p0 + pp) * kv.Hkv + g) * D + d;
    kv.K[base + k_off(D, p0 + pp, d)] = k[src];
    kv.VT[base + v_off(D, p0 + pp, d)] = v[src];
  }
}

hipError_t launch_seed(int L, int P, int slot, const KV& kv, const uint16_t* k, const uint16_t* v, hipStream_t st) {
  if (P <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_seed, dim3((P + 63) / 64, L * kv.Hkv), dim3(256), 0, st, P, slot, kv, k, v);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention
struct AttnArgs {
  KV kv;
  int layer, Hq, nchmax;
  const int32_t* slot;
  const int32_t* pos;
  const uint16_t* q;  // [B][Hq][D]
  float* part_o;      // [B][Hq][nchmax][D]
  float* part_ml;     // [B][Hq][nchmax][2]  (row max in log2 units, row sum)
  float scale;        // log2(e) / sqrt(D): scores are kept in log2 units, p = 2^(z - max)
};

template <int D>
__global__ void __launch_bounds__(64) k_attn(AttnArgs a) {
  constexpr int KSQ = D / 32;  // k-steps of q.K
  constexpr int NDT = D / 16;  // output d-tiles
  __shared__ float Pl[16][65];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int p = a.pos[b];
  if (c * 64 > p) return;
  const int lane = threadIdx.x;
  const int G = a.Hq / a.kv.Hkv;
  const int s = a.slot[b];
  const size_t base = kv_base(a.kv, a.layer, s, g);
  const uint16_t* Kb = a.kv.K + base;
  const uint16_t* Vb = a.kv.VT + base;
  const int c0 = c * 64;
  const int col = lane & 15, quad = lane >> 4;
  const bool last = (c0 + 63 > p);

  // K operands first (the scores need them first), then V, all in flight
  // together; each load is 1 KB contiguous across the wave.
  const uint16_t* Kc = Kb + (size_t)c * 64 * D + lane * 8;
  const uint16_t* Vc = Vb + (size_t)c * 64 * D + lane * 8;
  h8 kb[4][KSQ];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) kb[pt][ks] = ld_h8(Kc + (pt * KSQ + ks) * 512);
  h8 vop[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vop[dt][ks] = ld_h8(Vc + (dt * 2 + ks) * 512);
  // Q operand: rows = the G query heads of kv head g (rows >= G are zero).
  h8 qa[KSQ];
  {
    const uint16_t* qp = a.q + ((size_t)b * a.Hq + g * G + col) * D + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) qa[ks] = col < G ? ld_h8(qp + 32 * ks) : h8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  // scores: lane holds S[head 4*quad + r][pos c0 + 16*pt + col]
  f4 S[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) acc = mfma16x16x32(qa[ks], kb[pt][ks], acc);
    S[pt] = acc;
  }
  float mrow[4], lrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float m = -INFINITY;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int pp = c0 + pt * 16 + col;
      const float z = S[pt][r] * a.scale;
      S[pt][r] = pp > p ? -INFINITY : z;
      m = fmaxf(m, S[pt][r]);
    }
    m = row16_max(m);
    float l = 0.f;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const float e = __builtin_amdgcn_exp2f(S[pt][r] - m);
      S[pt][r] = e;
      l = l + e;
    }
    l = row16_sum(l);
    mrow[r] = m;
    lrow[r] = l;
  }
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int r = 0; r < 4; ++r) Pl[4 * quad + r][pt * 16 + col] = S[pt][r];
  __syncthreads();
  // P as the A operand (row = head col, k = positions 32ks + 8quad + j), hi + lo fp16.
  h8 phi[2], plo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pv = Pl[col][32 * ks + 8 * quad + j];
      const _Float16 hi = (_Float16)pv;
      phi[ks][j] = hi;
      plo[ks][j] = (_Float16)(pv - (float)hi);
    }
  if (last) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (c0 + 32 * ks + 8 * quad + j > p) vop[dt][ks][j] = (_Float16)0.0f;
  }
  float* po = a.part_o + (((size_t)b * a.Hq + g * G) * a.nchmax + c) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    f4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      o = mfma16x16x32(phi[ks], vop[dt][ks], o);
      o = mfma16x16x32(plo[ks], vop[dt][ks], o);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * quad + r;
      if (h < G) po[(size_t)h * a.nchmax * D + dt * 16 + col] = o[r];
    }
  }
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * quad + r;
      if (h < G) {
        float* ml = a.part_ml + (((size_t)b * a.Hq + g * G + h) * a.nchmax + c) * 2;
        ml[0] = mrow[r];
        ml[1] = lrow[r];
      }
    }
  }
}

// One wave per (head, stream): combine the stream's chunks.  Output o is
// [B][Hq*D], row-major (rows == 0) or an activation panel with that many rows.  Lane c holds
// chunk c (c + 64, ... beyond 64 chunks); M and L are wave reductions with a
// fixed tree, then every lane sums its columns over the chunks in order.
// nchmax <= 256 (ctx_cap <= 16384, checked at context creation).
__global__ void __launch_bounds__(64) k_attn_reduce(int Hq, int D, int nchmax, const int32_t* __restrict__ pos,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml, uint16_t* __restrict__ o,
                                                    int rows) {
  __shared__ float wgt[256];
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int nch = (pos[b] + 1 + 63) / 64;
  const float* ml = part_ml + ((size_t)b * Hq + h) * nchmax * 2;
  float mv[4], lv[4];
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = lane + 64 * j;
    mv[j] = c < nch ? ml[2 * c] : -INFINITY;
    lv[j] = c < nch ? ml[2 * c + 1] : 0.f;
    M = fmaxf(M, mv[j]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float L = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = lane + 64 * j;
    const float e = c < nch ? __builtin_amdgcn_exp2f(mv[j] - M) : 0.f;
    if (c < nch) wgt[c] = e;
    L = L + lv[j] * e;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L = L + __shfl_xor(L, off, 64);
  __syncthreads();
  const float* po = part_o + ((size_t)b * Hq + h) * nchmax * D;
  for (int d = lane; d < D; d += 64) {
    float acc = 0.f;
    for (int c = 0; c < nch; ++c) acc = acc + po[(size_t)c * D + d] * wgt[c];
    const int kk = h * D + d;  // column of the [B][Hq*D] output
    const size_t off = rows ? ((size_t)(kk >> 3) * rows + b) * 8 + (kk & 7) : (size_t)b * Hq * D + kk;
    o[off] = f2h(acc / L);
  }
}

hipError_t launch_attention(int B, int layer, int Hq, const KV& kv, const int32_t* slot, const int32_t* pos,
                            int max_pos, const uint16_t* q, float* part_o, float* part_ml, uint16_t* o,
                            hipStream_t st, void* prof, int o_rows) {
  AttnArgs a;
  a.kv = kv;
  a.layer = layer;
  a.Hq = Hq;
  a.nchmax = kv.cap / 64;
  a.slot = slot;
  a.pos = pos;
  a.q = q;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.scale = (float)(1.4426950408889634 / sqrt((double)kv.D));
  const int nch = (max_pos + 1 + 63) / 64;
  dim3 grid(nch, kv.Hkv, B);
  if (prof) prof_mark(prof, st);
  if (kv.D == 128)
    hipLaunchKernelGGL(k_attn<128>, grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(k_attn<64>, grid, dim3(64), 0, st, a);
  if (prof) prof_mark(prof, st);
  hipLaunchKernelGGL(k_attn_reduce, dim3(Hq, B), dim3(64), 0, st, Hq, kv.D, a.nchmax, pos, part_o, part_ml, o,
                     o_rows);
  return hipGetLastError();
}

}  // namespace w4
