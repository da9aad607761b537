// Per-stream glue of the decode step on gfx950: embedding gather, RMSNorm,
// top-k softmax routing with (stream, expert) bucketing, expert combine with
// the residual, and greedy argmax.  Each stream's row is handled by its own
// work-group with a fixed reduction order, so a row's result never depends on
// the other rows (the batched design of "Batched-concurrent 4-bit serving on
// Apple Silicon", section 3, keeps each stream's own steps on its own data).
#include <algorithm>

#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

static constexpr int kNormThreads = 256;

// Offset of element (row b, column k) of a [.][H] activation: row-major when
// rows == 0, else the panel layout of the dense products (w4_internal.h).
__device__ __forceinline__ size_t act_off(int b, int k, int H, int rows) {
  return rows ? ((size_t)(k >> 3) * rows + b) * 8 + (k & 7) : (size_t)b * H + k;
}

// Block-wide sum with a fixed order (wave shuffles, then waves in order).
__device__ __forceinline__ float block_sum(float v, float* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = v + __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float t = sh[0];
  for (int i = 1; i < nw; ++i) t = t + sh[i];
  return t;
}

// out = x * (1/sqrt(mean(x^2) + eps)) * gamma, row held in registers (H <= 16*256).
template <int PER>
__device__ __forceinline__ void norm_row(const float (&v)[PER], int H, const uint16_t* __restrict__ gamma, float eps,
                                         uint16_t* __restrict__ out, int b, int rows, float* sh) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * kNormThreads;
    if (i < H) ss = ss + v[j] * v[j];
  }
  ss = block_sum(ss, sh);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * kNormThreads;
    if (i < H) out[act_off(b, i, H, rows)] = f2h((v[j] * r) * h2f(gamma[i]));
  }
}

constexpr int kPer = 16;  // hidden <= 4096

__global__ void __launch_bounds__(kNormThreads) k_rmsnorm(int H, const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ gamma, float eps,
                                                          uint16_t* __restrict__ out, int rows) {
  __shared__ float sh[16];
  const int b = blockIdx.x;
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = threadIdx.x + j * kNormThreads;
    v[j] = i < H ? h2f(x[(size_t)b * H + i]) : 0.f;
  }
  norm_row<kPer>(v, H, gamma, eps, out, b, rows, sh);
}

hipError_t launch_rmsnorm(int B, int H, const uint16_t* x, const uint16_t* gamma, float eps, uint16_t* out,
                          hipStream_t st, int out_rows) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(kNormThreads), 0, st, H, x, gamma, eps, out, out_rows);
  return hipGetLastError();
}

// h[b] = fp16(code * scale) of the token's embedding row; xn[b] =
// RMSNorm(h[b]).  bad[b] = 1 when the token id is outside [0, V) (the row is
// then all zeros and the host reports the step as invalid), else 0.  Each
// thread owns runs of eight columns: one 4-byte load of their codes, one scale
// (g is a multiple of 8), 16-byte stores.
__global__ void __launch_bounds__(kNormThreads) k_embed(int H, int V, int g, const int32_t* __restrict__ tokens,
                                                        const uint8_t* __restrict__ emb_p,
                                                        const uint16_t* __restrict__ emb_s, uint16_t* __restrict__ h,
                                                        const uint16_t* __restrict__ gamma, float eps,
                                                        uint16_t* __restrict__ xn, int rows, int32_t* __restrict__ bad) {
  __shared__ float sh[16];
  const int b = blockIdx.x;
  int t = tokens[b];
  const bool invalid = t < 0 || t >= V;
  if (threadIdx.x == 0) bad[b] = invalid ? 1 : 0;
  if (invalid) t = 0;  // in bounds; every value below is replaced by zero
  const uint8_t* row = emb_p + (size_t)t * (H / 2);
  const uint16_t* srow = emb_s + (size_t)t * (H / g);
  constexpr int PER = 2;  // H <= 4096 = 8 columns x 2 x 256 threads
  // the norm's gain is requested with the codes, not after the sum
  uint4 gv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = 8 * (threadIdx.x + j * kNormThreads);
    gv[j] = i < H ? *reinterpret_cast<const uint4*>(gamma + i) : make_uint4(0u, 0u, 0u, 0u);
  }
  float v[8 * PER];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = 8 * (threadIdx.x + j * kNormThreads);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * j + e] = 0.f;
    if (i < H) {
      const uint32_t pk = invalid ? 0u : *reinterpret_cast<const uint32_t*>(row + i / 2);  // element i+e in nibble e
      const float sc = invalid ? 0.f : h2f(srow[i / g]);
      uint32_t out[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint16_t hv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const unsigned nib = (pk >> (4 * (e + u))) & 15u;
          const int q = (int)nib - ((nib & 8u) ? 16 : 0);
          hv[u] = f2h((float)q * sc);
          v[8 * j + e + u] = h2f(hv[u]);
        }
        out[e / 2] = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
      }
      *reinterpret_cast<uint4*>(h + (size_t)b * H + i) = make_uint4(out[0], out[1], out[2], out[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = ss + v[8 * j + e] * v[8 * j + e];
    }
  }
  ss = block_sum(ss, sh);
  const float rr = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = 8 * (threadIdx.x + j * kNormThreads);
    if (i < H) {
      const uint32_t gw[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
      uint32_t out[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint16_t o0 = f2h((v[8 * j + e] * rr) * h2f((uint16_t)(gw[e / 2] & 0xFFFFu)));
        const uint16_t o1 = f2h((v[8 * j + e + 1] * rr) * h2f((uint16_t)(gw[e / 2] >> 16)));
        out[e / 2] = (uint32_t)o0 | ((uint32_t)o1 << 16);
      }
      *reinterpret_cast<uint4*>(xn + act_off(b, i, H, rows)) = make_uint4(out[0], out[1], out[2], out[3]);
    }
  }
}

hipError_t launch_embed(int B, int H, int V, int g, const int32_t* tokens, const uint8_t* emb_p,
                        const uint16_t* emb_s, uint16_t* h, const uint16_t* gamma, float eps, uint16_t* xn,
                        int32_t* bad, hipStream_t st, int xn_rows) {
  hipLaunchKernelGGL(k_embed, dim3(B), dim3(kNormThreads), 0, st, H, V, g, tokens, emb_p, emb_s, h, gamma, eps, xn,
                     xn_rows, bad);
  return hipGetLastError();
}

// moe = fp16(sum_r w_r * y_r) in rank order; resid: h = fp16(h + moe), else h = moe.
// Then (gamma != null) xn = RMSNorm(h) * gamma.  One work-group per row; each
// thread owns runs of eight columns, so every load and store is 16 bytes (few
// memory instructions per compute unit: this launch is latency-bound).
constexpr int kCombThreads = 256;

template <bool DIRECT>
__global__ void __launch_bounds__(kCombThreads) k_combine(int H, int k, const float* __restrict__ w,
                                                          const int32_t* __restrict__ inv,
                                                          const uint16_t* __restrict__ y, uint16_t* __restrict__ h,
                                                          int resid, const uint16_t* __restrict__ gamma, float eps,
                                                          uint16_t* __restrict__ xn, int rows) {
  __shared__ float sh[16];
  __shared__ int s_inv[16];
  __shared__ float s_w[16];
  const int b = blockIdx.x;
  constexpr int PER = 2;  // H <= 4096 = 8 columns x 2 x 256 threads
  auto half_of = [](const uint4& q, int e) -> float {
    const uint32_t u = e < 2 ? q.x : e < 4 ? q.y : e < 6 ? q.z : q.w;
    return h2f((uint16_t)(u >> (16 * (e & 1))));
  };
  // the residual row and the norm's gain do not depend on the routing:
  // requested first, so the gain is not a memory round trip after the sum
  uint4 hres[PER], gv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = 8 * (threadIdx.x + j * kCombThreads);
    hres[j] = make_uint4(0u, 0u, 0u, 0u);
    gv[j] = make_uint4(0u, 0u, 0u, 0u);
    if (resid && i < H) hres[j] = *reinterpret_cast<const uint4*>(h + (size_t)b * H + i);
    if (gamma && i < H) gv[j] = *reinterpret_cast<const uint4*>(gamma + i);
  }
  // DIRECT (y in (stream, rank) order): the rows of the first column run are
  // requested with the weights (their places do not depend on the routing)
  uint4 yd[16];
  if (DIRECT) {
    const int i = 8 * threadIdx.x;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      yd[r] = (r < k && i < H) ? *reinterpret_cast<const uint4*>(y + ((size_t)b * k + r) * H + i)
                               : make_uint4(0u, 0u, 0u, 0u);
  }
  if (threadIdx.x < k) {
    if (!DIRECT) s_inv[threadIdx.x] = inv[b * k + threadIdx.x];
    s_w[threadIdx.x] = w[b * k + threadIdx.x];
  }
  __syncthreads();
  float v[8 * PER];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = 8 * (threadIdx.x + j * kCombThreads);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * j + e] = 0.f;
    if (i < H) {
      uint4 yr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r < k)
          yr[r] = DIRECT ? (j == 0 ? yd[r] : *reinterpret_cast<const uint4*>(y + ((size_t)b * k + r) * H + i))
                         : *reinterpret_cast<const uint4*>(y + (size_t)s_inv[r] * H + i);
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r < k) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = acc[e] + s_w[r] * half_of(yr[r], e);
        }
      uint32_t out[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint16_t m0 = f2h(acc[e]), m1 = f2h(acc[e + 1]);
        if (resid) {
          m0 = f2h(half_of(hres[j], e) + h2f(m0));
          m1 = f2h(half_of(hres[j], e + 1) + h2f(m1));
        }
        out[e / 2] = (uint32_t)m0 | ((uint32_t)m1 << 16);
        v[8 * j + e] = h2f(m0);
        v[8 * j + e + 1] = h2f(m1);
      }
      *reinterpret_cast<uint4*>(h + (size_t)b * H + i) = make_uint4(out[0], out[1], out[2], out[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = ss + v[8 * j + e] * v[8 * j + e];
    }
  }
  if (!gamma) return;
  ss = block_sum(ss, sh);
  const float rr = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = 8 * (threadIdx.x + j * kCombThreads);
    if (i < H) {
      uint32_t out[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint16_t o0 = f2h((v[8 * j + e] * rr) * half_of(gv[j], e));
        const uint16_t o1 = f2h((v[8 * j + e + 1] * rr) * half_of(gv[j], e + 1));
        out[e / 2] = (uint32_t)o0 | ((uint32_t)o1 << 16);
      }
      *reinterpret_cast<uint4*>(xn + act_off(b, i, H, rows)) = make_uint4(out[0], out[1], out[2], out[3]);
    }
  }
}

hipError_t launch_combine(int B, int H, int k, const float* w, const int32_t* inv, const uint16_t* y, uint16_t* h,
                          bool resid, const uint16_t* gamma, float eps, uint16_t* xn, hipStream_t st, int xn_rows,
                          bool direct) {
  if (direct)
    hipLaunchKernelGGL(k_combine<true>, dim3(B), dim3(kCombThreads), 0, st, H, k, w, inv, y, h, resid ? 1 : 0, gamma,
                       eps, xn, xn_rows);
  else
    hipLaunchKernelGGL(k_combine<false>, dim3(B), dim3(kCombThreads), 0, st, H, k, w, inv, y, h, resid ? 1 : 0, gamma,
                       eps, xn, xn_rows);
  return hipGetLastError();
}

// ------------------------------------------------------------------ routing
// Top-k softmax routing and the (stream, expert) bucketing with the 16-row
// work units of the grouped GEMMs, shared by the routing primitive (k_route,
// from given logits) and the decode router (k_router).  All of it is per-row
// arithmetic with fixed orders, so a row's routing never depends on the
// other rows.

// Order-preserving key of a logit: larger float -> larger unsigned; NaN
// ranks as -inf and -0 as +0 (they compare equal as floats).
__device__ __forceinline__ uint32_t sort_key(float v) {
  if (v != v) v = -INFINITY;
  if (v == 0.0f) v = 0.0f;
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Top-k of one row held by one wave (lane owns experts lane + 64j): ranks by
// logit descending, ties to the lower id; w_r = exp(l_r - l_0) / sum, summed in
// rank order.  Radix select of the k-th largest key over wave ballots, then
// each selected expert's rank among the selected.  sel(e, rank, w) records one
// selected expert (called by the lane that owns it).
template <int EPL, class Sel>
__device__ __forceinline__ void topk_row(const float* lg, int E, int k, int lane, Sel sel) {
  uint32_t key[EPL];
  float val[EPL];  // the row's logits, read once
  bool valid[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    valid[j] = e < E;
    val[j] = valid[j] ? lg[e] : 0.f;
    key[j] = valid[j] ? sort_key(val[j]) : 0u;
  }
  uint32_t prefix = 0;
  int need = k;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t want = (prefix | (1u << bit)) >> bit;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) cnt += __popcll(__ballot(valid[j] && (key[j] >> bit) == want));
    if (cnt >= need)
      prefix |= 1u << bit;
    else
      need -= cnt;
  }
  // selected: key > T, plus the `need` lowest-index experts with key == T
  bool sl[EPL];
  int before = 0;  // equal keys at lower indices in earlier slots
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const bool eq = valid[j] && key[j] == prefix;
    const unsigned long long m = __ballot(eq);
    const int below = before + __popcll(m & ((1ull << lane) - 1ull));
    sl[j] = valid[j] && (key[j] > prefix || (eq && below < need));
    before += __popcll(m);
  }
  // rank of each selected expert among the selected
  int rank[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) rank[j] = 0;
#pragma unroll
  for (int j2 = 0; j2 < EPL; ++j2) {
    unsigned long long m = __ballot(sl[j2]);
    while (m) {
      const int L = __ffsll((long long)m) - 1;
      m &= m - 1;
      const uint32_t k2 = __shfl(key[j2], L, 64);
      const int e2 = L + 64 * j2;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        rank[j] += (sl[j] && (k2 > key[j] || (k2 == key[j] && e2 < e))) ? 1 : 0;
      }
    }
  }
  // softmax over the selected, summed in rank order
  float l0 = 0.f, sum = 0.f;
  for (int r = 0; r < k; ++r) {
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const unsigned long long m = __ballot(sl[j] && rank[j] == r);
      if (m) v = __shfl(val[j], __ffsll((long long)m) - 1, 64);
    }
    if (v != v) v = -INFINITY;
    if (r == 0) l0 = v;
    sum = sum + expf(v - l0);
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (sl[j]) {
      const int e = lane + 64 * j;
      float v = val[j];
      if (v != v) v = -INFINITY;
      sel(e, rank[j], expf(v - l0) / sum);
    }
}

// Exclusive prefix sum over the wave of small non-negative values (< 2^BITS),
// and the wave total, from one ballot per bit.
template <int BITS>
__device__ __forceinline__ int wave_excl_sum(int v, int lane, int* total) {
  const unsigned long long lt = (1ull << lane) - 1ull;
  int ex = 0, tot = 0;
#pragma unroll
  for (int bit = 0; bit < BITS; ++bit) {
    const unsigned long long m = __ballot((v >> bit) & 1);
    ex += __popcll(m & lt) << bit;
    tot += __popcll(m) << bit;
  }
  *total = tot;
  return ex;
}

// Bucketing of B rows whose expert ids are in s_ids [B*k] and stream masks
// in s_mask [E] (bit b set when row b chose the expert): exclusive scans over
// experts (wave bit-sliced prefix sums, waves in order; needs >= 4 waves),
// the pairs ordered by (expert, stream), and the 16-row work units of the
// grouped products: units[u] = (expert, first pair, rows), unit_rows[u][i] =
// the stream of the unit's row i (rows past the unit's count repeat row 0),
// and, when unit_rows8 is given, the same streams as bytes.
struct BucketLds {
  unsigned* mask;  // [E]
  int* off;        // [E] first pair of the expert
  int* ubase;      // [E] first unit of the expert
  int* tot;        // [12]
  int* urows;      // [(E + B*k/16 + 1) * 16]
};
__device__ void bucket_core(int E, int k, int B, const int* s_ids, const BucketLds& L, const RouteOut& o) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int P = B * k;
  int c = 0, u = 0, nu = 0, ec = 0, eu = 0, en = 0;
  const int e = tid;
  if (w < 4) {  // experts 64w .. 64w+63
    c = e < E ? __popc(L.mask[e]) : 0;
    u = c > 0;
    nu = (c + 15) >> 4;
    int tc, tu, tn;
    ec = wave_excl_sum<6>(c, lane, &tc);
    eu = wave_excl_sum<1>(u, lane, &tu);
    en = wave_excl_sum<2>(nu, lane, &tn);
    if (lane == 0) {
      L.tot[3 * w] = tc;
      L.tot[3 * w + 1] = tu;
      L.tot[3 * w + 2] = tn;
    }
  }
  __syncthreads();
  if (w < 4) {
    for (int ww = 0; ww < w; ++ww) {
      ec += L.tot[3 * ww];
      eu += L.tot[3 * ww + 1];
      en += L.tot[3 * ww + 2];
    }
    if (e < E) {
      L.off[e] = ec;
      L.ubase[e] = en;
      if (o.counts) o.counts[e] = c;
      if (o.offsets) o.offsets[e] = ec;
      if (u) o.used[eu] = e;
      for (int j = 0; j < nu; ++j) {
        o.units[en + j] = make_int4(e, ec + 16 * j, min(16, c - 16 * j), 0);
        if (o.done) o.done[(size_t)(en + j) * kDoneStride] = 0u;
      }
    }
    if (e == E - 1) {
      if (o.offsets) o.offsets[E] = ec + c;
      *o.n_used = eu + u;
      *o.n_units = en + nu;
    }
  }
  __syncthreads();
  for (int i = tid; i < P; i += blockDim.x) {
    const int b = i / k, ex = s_ids[i];
    const int r = __popc(L.mask[ex] & ((1u << b) - 1u));  // row of the pair within its expert
    const int pos = L.off[ex] + r;
    if (o.pair_stream) o.pair_stream[pos] = b;
    if (o.pair_rank) o.pair_rank[pos] = i - b * k;
    if (o.pair_flat) o.pair_flat[pos] = i;
    o.inv[i] = pos;
    L.urows[(L.ubase[ex] + (r >> 4)) * 16 + (r & 15)] = b;
  }
  __syncthreads();
  if (e < E && w < 4 && c > 0) {  // pad the expert's last unit with its first row
    const int ul = en + nu - 1, ml = c - 16 * (nu - 1);
    for (int i = ml; i < 16; ++i) L.urows[ul * 16 + i] = L.urows[ul * 16];
  }
  __syncthreads();
  const int nun = L.tot[2] + L.tot[5] + L.tot[8] + L.tot[11];  // units of all experts
  if (o.unit_rows)
    for (int i = tid; i < nun * 16; i += blockDim.x) o.unit_rows[i] = L.urows[i];
  if (o.unit_rows8) {  // the same rows as bytes (streams < 32), four per word
    uint32_t* r8 = reinterpret_cast<uint32_t*>(o.unit_rows8);
    for (int i = tid; i < nun * 4; i += blockDim.x)
      r8[i] = (uint32_t)L.urows[4 * i] | ((uint32_t)L.urows[4 * i + 1] << 8) | ((uint32_t)L.urows[4 * i + 2] << 16) |
              ((uint32_t)L.urows[4 * i + 3] << 24);
  }
}

// bucket_core's outputs for one row whose k distinct experts (in rank order)
// are te[0..k): each selected expert's position in ascending expert order is
// the number of selected experts with a smaller id; it gets one unit of one
// row (stream 0, the other unit rows repeating it).  One pass, no barrier.
__device__ void bucket_single(int E, int k, const int* te, const RouteOut& o) {
  const int tid = threadIdx.x;
  if (tid < E) {
    int below = 0;
    bool sel = false;
    for (int r = 0; r < k; ++r) {
      below += te[r] < tid ? 1 : 0;
      sel = sel || te[r] == tid;
    }
    if (o.counts) o.counts[tid] = sel ? 1 : 0;
    if (o.offsets) o.offsets[tid] = below;
    if (sel) {
      o.used[below] = tid;
      o.units[below] = make_int4(tid, below, 1, 0);
      if (o.done) o.done[(size_t)below * kDoneStride] = 0u;
    }
  }
  if (tid < k) {
    const int e = te[tid];
    int pos = 0;
    for (int r = 0; r < k; ++r) pos += te[r] < e ? 1 : 0;
    if (o.pair_stream) o.pair_stream[pos] = 0;
    if (o.pair_rank) o.pair_rank[pos] = tid;
    if (o.pair_flat) o.pair_flat[pos] = tid;
    o.inv[tid] = pos;
  }
  if (tid == 0) {
    if (o.offsets) o.offsets[E] = k;
    *o.n_used = k;
    *o.n_units = k;
  }
  for (int i = tid; i < k * 16; i += blockDim.x) o.unit_rows[i] = 0;
  if (o.unit_rows8) {
    uint32_t* r8 = reinterpret_cast<uint32_t*>(o.unit_rows8);
    for (int i = tid; i < k * 4; i += blockDim.x) r8[i] = 0u;
  }
}

// One work-group of 1024 threads: top-k softmax of every row (one wave per
// row), then the (stream, expert) bucketing and the 16-row work units of the
// grouped GEMMs.
__global__ void __launch_bounds__(1024) k_route(const float* __restrict__ logits, int B, int E, int k, RouteOut o) {
  __shared__ float s_lg[32 * kRouteMaxE];  // [B][E] fp32 logits
  __shared__ int s_ids[32 * 16];
  __shared__ unsigned s_mask[kRouteMaxE];
  __shared__ int s_off[kRouteMaxE];
  __shared__ int s_ub[kRouteMaxE];
  __shared__ int s_tot[12];
  __shared__ int s_ur[kMaxUnits * 16];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_mask[e] = 0u;
  for (int i = threadIdx.x; i < B * E; i += blockDim.x) s_lg[i] = logits[i];
  __syncthreads();
  // top-k per row, one wave per row
  for (int b = w; b < B; b += 16) {
    auto sel = [&](int e, int r, float wt) {
      o.ids[b * k + r] = e;
      o.w[b * k + r] = wt;
      s_ids[b * k + r] = e;
      atomicOr(&s_mask[e], 1u << b);
    };
    if (E <= 64)
      topk_row<1>(s_lg + b * E, E, k, lane, sel);
    else if (E <= 128)
      topk_row<2>(s_lg + b * E, E, k, lane, sel);
    else
      topk_row<4>(s_lg + b * E, E, k, lane, sel);
  }
  __syncthreads();
  bucket_core(E, k, B, s_ids, BucketLds{s_mask, s_off, s_ub, s_tot, s_ur}, o);
}

hipError_t launch_route(const float* logits, int B, int E, int k, const RouteOut& o, hipStream_t st) {
  hipLaunchKernelGGL(k_route, dim3(1), dim3(1024), 0, st, logits, B, E, k, o);
  return hipGetLastError();
}

// Routing of the P rows of a prefill, into the same outputs as k_route, in
// two launches.  k_topk_rows: one wave per row, the top-k softmax of k_route
// (same arithmetic); it records the ids, the weights, each (row, rank)'s
// expert as one byte, and sets bit b of expert e's row mask (global, zero
// before).  k_bucket_prefill: the pairs ordered by (expert, row) -- a pair's
// place within its expert is the number of lower rows in the expert's mask,
// a prefix popcount -- and the work units of o.unit_n rows (and, when
// o.units2 is given, the records of a second list of 64-row units over the
// same pair order, each the run of two consecutive 32-row units of the first:
// its fourth field is the first of them).  Its work-groups share the pairs'
// stores (pair i in work-group (i / 1024) mod gridDim.x) and the unit records
// (one wave per expert); each one computes the masks' prefix counts and the
// scans itself, and work-group 0 alone writes the per-expert counts.  The masks are left as they are;
// the launch clears mask_next, the next call's masks, which nothing reads
// meanwhile.
__global__ void __launch_bounds__(1024) k_topk_rows(const float* __restrict__ logits, int P, int E, int k,
                                                    RouteOut o, uint32_t* __restrict__ mask,
                                                    uint8_t* __restrict__ e8) {
  const int W = (P + 31) / 32;
  const int b = blockIdx.x * 16 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= P) return;
  auto sel = [&](int e, int r, float wt) {
    o.ids[b * k + r] = e;
    o.w[b * k + r] = wt;
    e8[b * k + r] = (uint8_t)e;
    atomicOr(&mask[e * W + (b >> 5)], 1u << (b & 31));
  };
  const float* lg = logits + (size_t)b * E;
  if (E <= 64)
    topk_row<1>(lg, E, k, lane, sel);
  else if (E <= 128)
    topk_row<2>(lg, E, k, lane, sel);
  else
    topk_row<4>(lg, E, k, lane, sel);
}

__global__ void __launch_bounds__(1024) k_bucket_prefill(int P, int E, int k, RouteOut o,
                                                         const uint32_t* __restrict__ mask,
                                                         uint32_t* __restrict__ mask_next,
                                                         const uint8_t* __restrict__ e8) {
  // [E][W] row masks, then [E][W] 16-bit counts of the set bits in the words
  // before each word (a pair's place within its expert is one lookup)
  extern __shared__ uint32_t s_pm[];
  __shared__ int s_cnt[kRouteMaxE], s_off[kRouteMaxE], s_ub[kRouteMaxE], s_ub2[kRouteMaxE];
  const int W = (P + 31) / 32;
  const int US = o.unit_n;  // rows per unit
  const bool two = o.units2 != nullptr;
  const int US2 = two ? o.unit_n2 : US;  // rows per unit of the second list
  uint16_t* s_pre = reinterpret_cast<uint16_t*>(s_pm + (size_t)E * W);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int NB = gridDim.x, bx = blockIdx.x;
  const bool lead = bx == 0;  // writes the per-expert outputs
  // this thread's pairs tid + 1024 (bx + NB q) (at most kPrefillMaxPairs /
  // 1024 = 16): their experts requested first, so the pair loop below waits
  // for nothing
  const int PK = P * k;
  static_assert(kPrefillMaxPairs <= 16 * 1024, "16 pairs per thread");
  uint8_t ev[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = tid + 1024 * (bx + NB * q);
    ev[q] = i < PK ? e8[i] : (uint8_t)0;
  }
  // the masks into LDS, every load requested before the first store (E W <=
  // 10240 words: the launch's LDS bound)
  constexpr int kMW = 10;
  uint32_t mv[kMW];
#pragma unroll
  for (int q = 0; q < kMW; ++q) mv[q] = tid + 1024 * q < E * W ? mask[tid + 1024 * q] : 0u;
#pragma unroll
  for (int q = 0; q < kMW; ++q)
    if (tid + 1024 * q < E * W) s_pm[tid + 1024 * q] = mv[q];
  for (int i = bx * 1024 + tid; i < E * W; i += NB * 1024) mask_next[i] = 0u;
  __syncthreads();
  // prefix counts of each expert's words: wave w takes experts w, w + 16, ..,
  // its lanes 64 consecutive words at a time
  for (int e = w; e < E; e += 16) {
    int c = 0;
    for (int j0 = 0; j0 < W; j0 += 64) {
      const int j = j0 + lane;
      const int pc = j < W ? __popc(s_pm[e * W + j]) : 0;
      int t;
      const int ex = wave_excl_sum<6>(pc, lane, &t);
      if (j < W) s_pre[e * W + j] = (uint16_t)(c + ex);
      c += t;
    }
    if (lane == 0) s_cnt[e] = c;
  }
  __syncthreads();
  // exclusive scans over the experts, in expert order: wave w takes experts
  // 64w .. 64w+63 (ballot bit-sliced prefix sums), then the waves in order
  __shared__ int s_tot[16];
  int xc = 0, xu = 0, xn = 0, xn2 = 0, ec = 0, eu = 0, en = 0, en2 = 0;
  if (w < 4) {
    const int e = tid;
    xc = e < E ? s_cnt[e] : 0;
    xu = xc > 0;
    xn = (xc + US - 1) / US;
    xn2 = (xc + US2 - 1) / US2;
    int tc, tu, tn, tn2;
    ec = wave_excl_sum<15>(xc, lane, &tc);  // c <= P <= 16384
    eu = wave_excl_sum<1>(xu, lane, &tu);
    en = wave_excl_sum<11>(xn, lane, &tn);
    en2 = wave_excl_sum<11>(xn2, lane, &tn2);
    if (lane == 0) {
      s_tot[4 * w] = tc;
      s_tot[4 * w + 1] = tu;
      s_tot[4 * w + 2] = tn;
      s_tot[4 * w + 3] = tn2;
    }
  }
  __syncthreads();
  if (w < 4) {
    const int e = tid;
    for (int ww = 0; ww < w; ++ww) {
      ec += s_tot[4 * ww];
      eu += s_tot[4 * ww + 1];
      en += s_tot[4 * ww + 2];
      en2 += s_tot[4 * ww + 3];
    }
    if (e < E) {
      s_off[e] = ec;
      s_ub[e] = en;
      s_ub2[e] = en2;
      if (lead) {
        if (o.counts) o.counts[e] = xc;
        if (o.offsets) o.offsets[e] = ec;
        if (xu) o.used[eu] = e;
      }
    }
    if (lead && e == E - 1) {
      if (o.offsets) o.offsets[E] = ec + xc;
      *o.n_used = eu + xu;
      *o.n_units = en + xn;
      if (two) *o.n_units2 = en2 + xn2;
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = tid + 1024 * (bx + NB * q);
    if (i >= PK) continue;
    const int b = i / k, e = ev[q];
    const int r = s_pre[e * W + (b >> 5)] + __popc(s_pm[e * W + (b >> 5)] & ((1u << (b & 31)) - 1u));
    const int pos = s_off[e] + r;
    if (o.pair_stream) o.pair_stream[pos] = b;
    if (o.pair_rank) o.pair_rank[pos] = i - b * k;
    if (o.pair_flat) o.pair_flat[pos] = i;
    o.inv[i] = pos;
    o.unit_rows[(s_ub[e] + r / US) * US + r % US] = b;
  }
  // unit records, spread over the work-groups: wave w of work-group bx takes
  // experts bx * 16 + w + 16 NB t, its lanes the expert's units.  Rows past a
  // unit's count repeat its first row: the row of rank want = US (nu - 1)
  // within the expert, in the last word whose prefix count is <= want.
  for (int e = bx * 16 + w; e < E; e += 16 * NB) {
    const int c = s_cnt[e];
    const int nu = (c + US - 1) / US;
    for (int j = lane; j < nu; j += 64) {
      o.units[s_ub[e] + j] = make_int4(e, s_off[e] + US * j, min(US, c - US * j), 0);
      if (o.done) o.done[(size_t)(s_ub[e] + j) * kDoneStride] = 0u;
    }
    if (c > 0 && (c % US)) {
      const int want = US * (nu - 1);
      int lo = 0, hi = W - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[e * W + mid] <= want)
          lo = mid;
        else
          hi = mid - 1;
      }
      uint32_t mm = s_pm[e * W + lo];
      for (int q = 0; q < want - s_pre[e * W + lo]; ++q) mm &= mm - 1;  // drop the lower set bits
      const int first = 32 * lo + __ffs(mm) - 1;
      for (int i = c - US * (nu - 1) + lane; i < US; i += 64) o.unit_rows[(s_ub[e] + nu - 1) * US + i] = first;
    }
    if (two)
      for (int j = lane; j < (c + US2 - 1) / US2; j += 64)
        o.units2[s_ub2[e] + j] = make_int4(e, s_off[e] + US2 * j, min(US2, c - US2 * j), s_ub[e] + j * (US2 / US));
  }
}

hipError_t launch_route_prefill(const float* logits, int P, int E, int k, const RouteOut& o, uint32_t* mask,
                                uint32_t* mask_next, uint8_t* e8, hipStream_t st) {
  const size_t lds = route_prefill_lds(P, E, k);
  if (P < 1 || E > kRouteMaxE || (size_t)P * k > (size_t)kPrefillMaxPairs || lds > 61440 || !mask || !mask_next || mask == mask_next || !e8 ||
      (o.unit_n != 16 && o.unit_n != 32) ||
      (o.units2 && (o.unit_n2 != 64 || o.unit_n != 32 || !o.n_units2)))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_topk_rows, dim3((P + 15) / 16), dim3(1024), 0, st, logits, P, E, k, o, mask, e8);
  const int nb = std::min(kBucketPrefillGroups, (P * k + 1023) / 1024);
  hipLaunchKernelGGL(k_bucket_prefill, dim3(nb), dim3(1024), lds, st, P, E, k, o, mask, mask_next, e8);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router
// The whole MoE front end of a decode layer in one launch.  Work-group
// (b, t) (1024 threads) owns stream row b and the 16 experts of tile t:
//   xn = RMSNorm(h[b]) * gamma (fp16; every tile's work-group computes it,
//     tile 0's writes it out for the expert GEMMs);
//   logits[e] = sum over 128-column chunks c, in chunk order, of
//     P[e][c] = sum over the chunk's groups of fma(scale, MFMA chain, .) from 0,
//     published with device-scope stores;
// the last of the row's work-groups to take the row's ticket reads the row's
// logits back and takes its top-k softmax (ranked by logit, ties to the lower
// id).  Then each row's last work-group takes the launch ticket; the last one
// buckets all rows.  Every order above depends on the geometry only, never
// on B or on the other rows.
//
// One work-group per (row, tile) rather than per row: a compute unit keeps
// only so many misses in flight, so one work-group streaming the whole 128 KB
// bank took about 9 us; a 16 KB tile arrives in a fraction of that, and the
// exchange of the logits costs less than it saves.
constexpr int kRouterMaxChunks = 32;  // H <= 4096

struct RouterArgs {
  const uint16_t* h;       // [B][H] residual rows
  const uint16_t* gamma;   // [H]
  float eps;
  uint16_t* xn;            // [B][H] out
  const uint4* tiles;      // router bank tiles [Ep/16][H/128][64] x 16 B
  const uint16_t* scales;  // [Ep][H/g]
  int H, E, k, B;
  RouteOut o;
  unsigned* ticket;        // zero between launches
  float* lg;               // [B][E] logits, exchanged between a row's work-groups
  unsigned* rticket;       // [B] row tickets, zero between launches
  const uint8_t* pf;       // work-groups B*NT .. B*NT+npf-1 touch this span (touch_lines)
  size_t pf_lines;
  int npf;
  // and the live KV chunks of layer kvl for the rows (slot, pos as in the
  // attention), when kv.K is not null
  KV kv;
  int kvl;
  const int32_t* slot;
  const int32_t* pos;
};

// Spare work-group j of the router launch: the live 64-position chunks of
// every (row, kv head) of layer a.kvl, K and V, npf / (2 B Hkv) work-groups
// per span, one 4-byte load per 128-byte line.
__device__ __forceinline__ void touch_kv(const RouterArgs& a, int j) {
  const int ns = 2 * a.B * a.kv.Hkv, wps = a.npf / ns;
  if (j >= ns * wps) return;
  const int s = j / wps, q = j - s * wps;
  const int bg = s >> 1, b = bg / a.kv.Hkv, g = bg - b * a.kv.Hkv;
  const size_t base = (((size_t)a.kvl * a.kv.S + a.slot[b]) * a.kv.Hkv + g) * (size_t)a.kv.cap * a.kv.D;
  const uint8_t* span = reinterpret_cast<const uint8_t*>(((s & 1) ? a.kv.VT : a.kv.K) + base);
  const size_t lines = (size_t)(a.pos[b] / 64 + 1) * 64 * a.kv.D * 2 / 128;
  for (size_t li = (size_t)q * blockDim.x + threadIdx.x; li < lines; li += (size_t)wps * blockDim.x) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(span + (li << 7));
    asm volatile("" ::"v"(v));
  }
}

template <int G>
__global__ void __launch_bounds__(1024) k_router(RouterArgs a) {
  constexpr int SPG = G / 32;   // k-steps per group
  constexpr int NGC = 128 / G;  // groups per 128-column chunk
  __shared__ __align__(16) uint16_t s_x[4096];
  __shared__ float s_part[kRouterMaxChunks * 16];
  __shared__ float s_lg[kRouteMaxE];
  __shared__ float sh[16];
  __shared__ __align__(16) uint32_t s_key[kRouteMaxE];
  __shared__ int s_rank[kRouteMaxE];
  __shared__ int s_te[16];
  __shared__ float s_tl[16], s_ex[16];
  __shared__ unsigned s_mask[kRouteMaxE];
  __shared__ int s_off[kRouteMaxE];
  __shared__ int s_tot[12];
  __shared__ int s_ids[32 * 16];
  __shared__ int s_ub[kRouteMaxE];
  __shared__ int s_ur[kMaxUnits * 16];
  __shared__ int s_last;
  const int H = a.H, E = a.E, k = a.k;
  const int NC = H >> 7, NT = (E + 15) >> 4;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if ((int)blockIdx.x >= a.B * NT) {
    touch_lines(a.pf, a.pf_lines, blockIdx.x - a.B * NT, a.npf);
    if (a.kv.K) touch_kv(a, blockIdx.x - a.B * NT);
    return;
  }
  const int b = blockIdx.x / NT, t = blockIdx.x - b * NT;

  // The row and gain are requested first (their wait comes first); then the
  // weights and scales of this wave's first chunk (wave w takes chunks w,
  // w + 16, ...), whose latency overlaps the norm.
  const int i0 = 4 * tid;
  uint2 hraw = make_uint2(0u, 0u), graw = make_uint2(0u, 0u);
  if (i0 < H) {
    hraw = *reinterpret_cast<const uint2*>(a.h + (size_t)b * H + i0);
    graw = *reinterpret_cast<const uint2*>(a.gamma + i0);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these two loads ahead of the weight loads
  uint4 wv;
  uint16_t sr[NGC];
  const uint16_t* srow = a.scales + (size_t)(16 * t + (lane & 15)) * (H / G);
  auto load_chunk = [&](int c) {
    wv = a.tiles[((size_t)t * NC + c) * 64 + lane];
#pragma unroll
    for (int j = 0; j < NGC; ++j) sr[j] = srow[c * NGC + j];
  };
  // Unconditional (chunk clamped): a load under a branch would make every
  // later wait on the row count the weight loads too.
  load_chunk(min(w, NC - 1));
  __builtin_amdgcn_sched_barrier(0);

  // 1. RMSNorm of the row: 4 columns per thread, fixed-order block sum.
  {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    if (i0 < H) {
      v[0] = h2f((uint16_t)(hraw.x & 0xFFFFu));
      v[1] = h2f((uint16_t)(hraw.x >> 16));
      v[2] = h2f((uint16_t)(hraw.y & 0xFFFFu));
      v[3] = h2f((uint16_t)(hraw.y >> 16));
      ss = v[0] * v[0];
      ss = ss + v[1] * v[1];
      ss = ss + v[2] * v[2];
      ss = ss + v[3] * v[3];
    }
    ss = block_sum(ss, sh);
    const float rs = 1.0f / sqrtf(ss / (float)H + a.eps);
    if (i0 < H) {
      const uint16_t o0 = f2h((v[0] * rs) * h2f((uint16_t)(graw.x & 0xFFFFu)));
      const uint16_t o1 = f2h((v[1] * rs) * h2f((uint16_t)(graw.x >> 16)));
      const uint16_t o2 = f2h((v[2] * rs) * h2f((uint16_t)(graw.y & 0xFFFFu)));
      const uint16_t o3 = f2h((v[3] * rs) * h2f((uint16_t)(graw.y >> 16)));
      const uint2 packed = make_uint2((uint32_t)o0 | ((uint32_t)o1 << 16), (uint32_t)o2 | ((uint32_t)o3 << 16));
      *reinterpret_cast<uint2*>(s_x + i0) = packed;
      if (t == 0) *reinterpret_cast<uint2*>(a.xn + (size_t)b * H + i0) = packed;
    }
  }
  __syncthreads();

  // 2. Chunk partials P[c] of the tile's 16 experts.  Every A-operand row is
  // the normalised row, so D row 0 (lanes 0..15, element 0) is the result;
  // the A operand of a chunk is read from LDS (a broadcast read).
  const DqConst dk;
  for (int c = w; c < NC; c += 16) {
    if (c != w) load_chunk(c);
    h8 xa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xa[s] = *reinterpret_cast<const h8*>(s_x + 128 * c + 32 * s + 8 * (lane >> 4));
    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
    f4 acc = {0.f, 0.f, 0.f, 0.f}, part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s % SPG == 0) part = f4{0.f, 0.f, 0.f, 0.f};
      part = mfma16x16x32(xa[s], dq8(wd[s], dk), part);
      if ((s + 1) % SPG == 0) {
        const float sc = h2f(sr[s / SPG]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = fmaf(sc, part[q], acc[q]);
      }
    }
    // All four rows are equal; keeping every element of the MFMA results
    // live stops the compiler from reusing a destination register of an
    // MFMA still in flight for the next operand.
    asm volatile("" ::"v"(acc));
    if (lane < 16) s_part[c * 16 + lane] = acc[0];
  }
  __syncthreads();

  // 3. The tile's logits to memory; the row's last work-group reads all back.
  if (tid < 16 && 16 * t + tid < E) {
    float l = s_part[tid];
    for (int c = 1; c < NC; ++c) l = l + s_part[c * 16 + tid];
    __hip_atomic_store(reinterpret_cast<uint32_t*>(a.lg) + (size_t)b * E + 16 * t + tid, __float_as_uint(l),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the stores complete before the row ticket
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(a.rticket + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(NT - 1);
  __syncthreads();
  if (!s_last) return;
  if (tid < E)
    s_lg[tid] = __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(a.lg) + (size_t)b * E + tid,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (tid == 0) __hip_atomic_store(a.rticket + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();

  // 4. Top-k of the row by rank counting: rank(e) = #{e' : key e' > key e, or
  // equal keys and e' < e} (NaN ranks as -inf); thread (e, part) counts over
  // one part of the experts, integer LDS adds combine the parts.  The experts
  // of rank < k are the top-k in rank order.
  {
    const int NE = E <= 128 ? 128 : 256, parts = 1024 / NE, per = NE / parts;
    const int e = tid & (NE - 1), p = tid / NE;
    if (tid < NE) {
      s_key[tid] = tid < E ? sort_key(s_lg[tid]) : 0u;  // padding ranks below every expert
      s_rank[tid] = 0;
    }
    __syncthreads();
    const uint32_t ke = s_key[e];
    int cnt = 0;
    for (int j = p * per; j < (p + 1) * per; j += 4) {
      const uint4 kk = *reinterpret_cast<const uint4*>(s_key + j);
      cnt += (kk.x > ke || (kk.x == ke && j < e)) ? 1 : 0;
      cnt += (kk.y > ke || (kk.y == ke && j + 1 < e)) ? 1 : 0;
      cnt += (kk.z > ke || (kk.z == ke && j + 2 < e)) ? 1 : 0;
      cnt += (kk.w > ke || (kk.w == ke && j + 3 < e)) ? 1 : 0;
    }
    if (cnt) atomicAdd(&s_rank[e], cnt);
    __syncthreads();
    if (tid < E && s_rank[tid] < k) {
      float v = s_lg[tid];
      if (v != v) v = -INFINITY;
      s_te[s_rank[tid]] = tid;
      s_tl[s_rank[tid]] = v;
    }
  }
  __syncthreads();
  if (tid < k) s_ex[tid] = expf(s_tl[tid] - s_tl[0]);
  __syncthreads();
  if (tid < k) {
    float sum = 0.f;
    for (int r = 0; r < k; ++r) sum = sum + s_ex[r];
    // ids are read by the last row within this launch: device-scope
    // atomic stores, complete (vmcnt 0) before the ticket is taken.  The
    // other outputs are read by later launches only.
    __hip_atomic_store(&a.o.ids[b * k + tid], s_te[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.o.w[b * k + tid] = s_ex[tid] / sum;
  }
  // 5. Launch ticket: the last row to arrive buckets every row.  With one
  // row, its last work-group writes the buckets of the row's ids straight
  // from LDS, with no launch ticket and no round trip through memory (the
  // ticket stays zero): 1.9 us of bucket_core against a single pass.
  if (a.B == 1) {
    bucket_single(E, k, s_te, a.o);
    return;
  } else {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (unsigned)(a.B - 1);
    __syncthreads();
    if (!s_last) return;
    if (tid < E) s_mask[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < a.B * k; i += blockDim.x) {
      const int ex = __hip_atomic_load(&a.o.ids[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_ids[i] = ex;
      atomicOr(&s_mask[ex], 1u << (i / k));
    }
    __syncthreads();
  }
  bucket_core(E, k, a.B, s_ids, BucketLds{s_mask, s_off, s_ub, s_tot, s_ur}, a.o);
  if (tid == 0) __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int touch_groups(size_t bytes, int threads) {
  const size_t lines = bytes / 128;
  return (int)std::min(lines, std::max<size_t>(256, (lines + threads - 1) / threads));
}

hipError_t launch_router(int B, int H, int E, int k, int g, const uint16_t* h, const uint16_t* gamma, float eps,
                         uint16_t* xn, const uint4* tiles, const uint16_t* scales, const RouteOut& o,
                         unsigned* ticket, float* lg, unsigned* rticket, hipStream_t st, const void* pf,
                         size_t pf_bytes, const KV* kv_next, int kv_layer, const int32_t* slot, const int32_t* pos) {
  if (H % 128 != 0 || H / 128 > kRouterMaxChunks || E > kRouteMaxE || !lg || !rticket) return hipErrorInvalidValue;
  const int npf = pf ? touch_groups(pf_bytes, 1024) : 0;
  RouterArgs a{h, gamma, eps, xn, tiles, scales, H, E, k, B, o, ticket, lg, rticket,
               static_cast<const uint8_t*>(pf), pf_bytes / 128, npf};
  a.kv = KV{};
  if (kv_next && npf > 0 && slot && pos) {
    a.kv = *kv_next;
    a.kvl = kv_layer;
    a.slot = slot;
    a.pos = pos;
  }
  const dim3 grid(B * ((E + 15) / 16) + npf);
  switch (g) {
    case 32: w4_launch(k_router<32>, grid, dim3(1024), 0, st, a); break;
    case 64: w4_launch(k_router<64>, grid, dim3(1024), 0, st, a); break;
    default: w4_launch(k_router<128>, grid, dim3(1024), 0, st, a); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ argmax
// Largest fp16 logit per row, ties to the lower id (NaN never wins).
// Greedy next token: argmax of each logits row (larger value first, then
// the lower index; NaN never wins; a row of NaN gives 0).  Work-group
// (split s, row b) scans V/8 consecutive entries with 16-byte loads (four in
// flight per thread) and publishes its best with device-scope stores; the
// last of a row's eight work-groups (per-row ticket, zero before and after)
// combines them.  The result is the same as one scan of the row.
constexpr int kArgmaxSplits = 8;
__device__ __forceinline__ bool am_better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

template <bool VEC>
__global__ void __launch_bounds__(256) k_argmax(int V, const uint16_t* __restrict__ logits, int32_t* __restrict__ next,
                                                float* part_v, int32_t* part_i, unsigned* ticket) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int s_last;
  const int sp = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const uint16_t* row = logits + (size_t)b * V;
  const int per = ((V + kArgmaxSplits - 1) / kArgmaxSplits + 7) & ~7;
  const int lo = sp * per, hi = min(V, lo + per);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (VEC) {  // V % 8 == 0: rows and slices are 16-byte aligned
    for (int base = lo + 8 * tid; base < hi; base += 4 * 8 * 256) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const uint4*>(row + min(base + u * 8 * 256, hi - 8));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i0 = base + u * 8 * 256;
        if (i0 < hi) {
          const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = h2f((uint16_t)(wd[j >> 1] >> (16 * (j & 1))));
            if (am_better(x, i0 + j, bv, bi)) {
              bv = x;
              bi = i0 + j;
            }
          }
        }
      }
    }
  } else {
    for (int i = lo + tid; i < hi; i += 256) {
      const float x = h2f(row[i]);
      if (am_better(x, i, bv, bi)) {
        bv = x;
        bi = i;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (am_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int j = 1; j < 4; ++j)
      if (am_better(sv[j], si[j], bv, bi)) {
        bv = sv[j];
        bi = si[j];
      }
    __hip_atomic_store(part_v + b * kArgmaxSplits + sp, bv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(part_i + b * kArgmaxSplits + sp, bi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // partial stored before the ticket
    s_last = __hip_atomic_fetch_add(ticket + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(kArgmaxSplits - 1);
  }
  __syncthreads();
  if (!s_last || tid != 0) return;
  float pv[kArgmaxSplits];
  int pi[kArgmaxSplits];
#pragma unroll
  for (int j = 0; j < kArgmaxSplits; ++j) {
    pv[j] = __hip_atomic_load(part_v + b * kArgmaxSplits + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pi[j] = __hip_atomic_load(part_i + b * kArgmaxSplits + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  bv = pv[0];
  bi = pi[0];
#pragma unroll
  for (int j = 1; j < kArgmaxSplits; ++j)
    if (am_better(pv[j], pi[j], bv, bi)) {
      bv = pv[j];
      bi = pi[j];
    }
  next[b] = bi == 0x7fffffff ? 0 : bi;
  __hip_atomic_store(ticket + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_argmax(int B, int V, const uint16_t* logits, int32_t* next, float* part_v, int32_t* part_i,
                         unsigned* ticket, hipStream_t st) {
  const dim3 grid(kArgmaxSplits, B);
  if (V % 8 == 0)
    hipLaunchKernelGGL(k_argmax<true>, grid, dim3(256), 0, st, V, logits, next, part_v, part_i, ticket);
  else
    hipLaunchKernelGGL(k_argmax<false>, grid, dim3(256), 0, st, V, logits, next, part_v, part_i, ticket);
  return hipGetLastError();
}

// ------------------------------------------------------------------ sampling
// Next token of each row by temperature / top-k / top-p sampling with a
// counter-based draw, one 1024-thread work-group per row.  Steps (the same as
// the CPU reference's):
//   1. rank ids by (logit descending, id ascending), NaN as -inf, -0 as +0, and
//      keep the first k = min(top_k, V): the k-th largest 16-bit ordered key is
//      found by two 256-bin histogram passes (high byte, then the low byte
//      within the bin that holds it); every id with a larger key is kept, and
//      of the ids with that key the lowest ones (a block scan over contiguous
//      id ranges, in id order) fill the remaining places;
//   2. temperature 0 or k = 1: the first rank (greedy);
//   3. e_r = exp((l_r - l_0) * (1/T)), c_r = e_0 + ... + e_r in rank order;
//   4. nucleus: the shortest prefix 0..m with c_m >= top_p * c_{k-1};
//   5. u = (z >> 40) * 2^-24 with z the output number pos of SplitMix64
//      started at the row's seed; the first rank r <= m with u * c_m < c_r.
// The draw depends on the stream's seed and position only, so a stream's
// samples are the same in any batch.
constexpr int kSampleThreads = 1024;

__device__ __forceinline__ uint32_t sample_key(uint16_t h) {
  if ((h & 0x7C00u) == 0x7C00u && (h & 0x03FFu)) h = 0xFC00u;  // NaN -> -inf
  if (h == 0x8000u) h = 0;                                      // -0 -> +0
  return (h & 0x8000u) ? (~(uint32_t)h & 0xFFFFu) : ((uint32_t)h | 0x8000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  const uint16_t h = (key & 0x8000u) ? (uint16_t)(key & 0x7FFFu) : (uint16_t)(~key & 0xFFFFu);
  return h2f(h);
}
// SplitMix64 (Steele, Lea and Flood 2014; Vigna's splitmix64.c): output
// number pos of the generator started at seed.
__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t pos) {
  uint64_t z = seed + (pos + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Exclusive scan over the work-group (1024 threads) of a small count.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    base += i < w ? sh[i] : 0;
    tot += sh[i];
  }
  *total = tot;
  return base + incl - v;
}

__global__ void __launch_bounds__(kSampleThreads) k_sample(int V, const uint16_t* __restrict__ logits,
                                                           const int32_t* __restrict__ params,
                                                           const int32_t* __restrict__ pos,
                                                           int32_t* __restrict__ next) {
  __shared__ int hist[256];
  __shared__ int s_scan[16];
  __shared__ uint32_t c_key[kSampleMaxK];
  __shared__ int c_id[kSampleMaxK];
  __shared__ float r_val[kSampleMaxK];
  __shared__ int r_id[kSampleMaxK];
  __shared__ int s_b1, s_above, s_thr, s_cgt;
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint16_t* row = logits + (size_t)b * V;
  const int32_t* pr = params + (size_t)b * kSampleParams;
  const float temp = __int_as_float(pr[0]), top_p = __int_as_float(pr[2]);
  const int k = min(max(pr[1], 1), V);
  const uint64_t seed = (uint64_t)(uint32_t)pr[3] | ((uint64_t)(uint32_t)pr[4] << 32);

  // 1a. high-byte histogram, then the bin holding the k-th largest key
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  for (int i = tid; i < V; i += kSampleThreads) atomicAdd(&hist[sample_key(row[i]) >> 8], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = 0, bin = 255;
    for (; bin > 0 && acc + hist[bin] < k; --bin) acc += hist[bin];
    s_b1 = bin;
    s_above = acc;
  }
  __syncthreads();
  const int b1 = s_b1;
  // 1b. low-byte histogram within that bin: the k-th largest key itself
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  for (int i = tid; i < V; i += kSampleThreads) {
    const uint32_t key = sample_key(row[i]);
    if ((int)(key >> 8) == b1) atomicAdd(&hist[key & 255u], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = s_above, bin = 255;
    for (; bin > 0 && acc + hist[bin] < k; --bin) acc += hist[bin];
    s_thr = (b1 << 8) | bin;
    s_cgt = acc;  // keys above the threshold key (< k)
  }
  __syncthreads();
  const uint32_t thr = (uint32_t)s_thr;
  const int cgt = s_cgt, need = k - cgt;
  // 1c. candidates in id order: wave w owns the contiguous ids
  // [w*per, (w+1)*per), its lanes reading consecutive ids (coalesced); in-wave
  // order from ballots, across waves from a scan of the per-wave counts
  const int lane = tid & 63, wv = tid >> 6;
  const int per = (V + 15) / 16;
  const int lo = min(wv * per, V), hi = min(lo + per, V);
  int ngt = 0, neq = 0;
  for (int i = lo + lane; i < hi; i += 64) {
    const uint32_t key = sample_key(row[i]);
    ngt += key > thr;
    neq += key == thr;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    ngt += __shfl_xor(ngt, o, 64);
    neq += __shfl_xor(neq, o, 64);
  }
  int tg = 0, te = 0;
  // per-wave totals in lane 0 of each wave; the other lanes add zero
  const int og = block_excl_scan(lane == 0 ? ngt : 0, s_scan, &tg);
  const int oe = block_excl_scan(lane == 0 ? neq : 0, s_scan, &te);
  int g = __shfl(og, 0, 64), e = __shfl(oe, 0, 64);
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int i0 = lo; i0 < hi; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t key = i < hi ? sample_key(row[i]) : 0u;
    const bool isg = i < hi && key > thr, ise = i < hi && key == thr;
    const unsigned long long mg = __ballot(isg), me = __ballot(ise);
    if (isg) {
      const int at = g + __popcll(mg & below);
      c_key[at] = key;
      c_id[at] = i;
    }
    if (ise) {
      const int r = e + __popcll(me & below);
      if (r < need) {
        c_key[cgt + r] = key;
        c_id[cgt + r] = i;
      }
    }
    g += __popcll(mg);
    e += __popcll(me);
  }
  __syncthreads();
  // rank of each candidate: (key descending, id ascending)
  if (tid < k) {
    const uint32_t kk = c_key[tid];
    const int ii = c_id[tid];
    int r = 0;
    for (int j = 0; j < k; ++j) r += (c_key[j] > kk || (c_key[j] == kk && c_id[j] < ii)) ? 1 : 0;
    r_val[r] = key_value(kk);
    r_id[r] = ii;
  }
  __syncthreads();
  if (tid != 0) return;
  int out = r_id[0];
  if (temp > 0.0f && k > 1) {
    const float inv_t = 1.0f / temp;
    float c[kSampleMaxK];
    float run = 0.0f;
    const float l0 = r_val[0];
    for (int r = 0; r < k; ++r) {
      run = run + expf((r_val[r] - l0) * inv_t);
      c[r] = run;
    }
    const float want = top_p * c[k - 1];
    int m = 0;
    while (m < k - 1 && c[m] < want) ++m;
    const float u = (float)(uint32_t)(splitmix64_at(seed, (uint64_t)pos[b]) >> 40) * 0x1p-24f;
    const float t = u * c[m];
    int r = 0;
    while (r < m && !(t < c[r])) ++r;
    out = r_id[r];
  }
  next[b] = out;
}

hipError_t launch_sample(int B, int V, const uint16_t* logits, const int32_t* params, const int32_t* pos,
                         int32_t* next, hipStream_t st) {
  hipLaunchKernelGGL(k_sample, dim3(B), dim3(kSampleThreads), 0, st, V, logits, params, pos, next);
  return hipGetLastError();
}

// Streaming-read probe: every 16-byte chunk of src is loaded once (four
// loads in flight per thread, consecutive lanes on consecutive chunks), the
// words are folded into one value per thread, and a work-group stores it only
// if it equals a constant no real data hits, so the loads stay and almost no
// bytes are written.  Measures the HBM read ceiling with the load width the
// weight kernels use, plain or non-temporal (NT).
template <bool NT>
__global__ void __launch_bounds__(256) k_read_probe(const uint4* __restrict__ src, size_t n16,
                                                    uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  auto ld = [&](size_t j) { return NT ? ld_nt(src + j) : src[j]; };
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = ld(i), b = ld(i + stride), c = ld(i + 2 * stride), d = ld(i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) + (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, bool nt, hipStream_t st) {
  if (nt)
    hipLaunchKernelGGL(k_read_probe<true>, dim3(grid), dim3(256), 0, st, static_cast<const uint4*>(src), bytes / 16,
                       sink);
  else
    hipLaunchKernelGGL(k_read_probe<false>, dim3(grid), dim3(256), 0, st, static_cast<const uint4*>(src), bytes / 16,
                       sink);
  return hipGetLastError();
}

// Device-wide barrier probe (diagnostic, not part of the step): n barriers
// among `grid` co-resident 512-thread work-groups in one launch.  Two-level
// counters: a work-group adds to its group's counter (8 groups by index, 256
// bytes apart), the last arrival of a group adds to the top counter, and
// every work-group polls the top counter with device-scope loads.  Each wait
// is bounded; one that runs out sets ctr[1] and the launch goes on.
// ctr: [kSyncProbeWords], zero at launch.
constexpr int kSyncGroups = 8;
__global__ void __launch_bounds__(512) k_barrier_probe(uint32_t* ctr, int n) {
  const int g = blockIdx.x % kSyncGroups;
  const unsigned per = (gridDim.x - g + kSyncGroups - 1) / kSyncGroups;
  uint32_t* gc = ctr + 64 * (1 + g);
  for (int i = 1; i <= n; ++i) {
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned old = __hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == (unsigned)i * per - 1) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned target = (unsigned)i * kSyncGroups;
      for (int spin = 0; __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++spin) {
        if (spin > (1 << 16)) {
          __hip_atomic_store(ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
  }
}

// The reference for the probe above: a launch of the same shape that does nothing.
__global__ void __launch_bounds__(512) k_empty_probe(uint32_t* ctr) {
  if (threadIdx.x == 0 && blockIdx.x == 0x7fffffff) ctr[2] = 1u;
}

int sync_probe_max_grid() {
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_barrier_probe), 512, 0) !=
          hipSuccess ||
      per_cu < 1)
    return 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 0;
  return per_cu * cus;
}

hipError_t launch_sync_probe(int mode, int grid, int n, uint32_t* ctr, hipStream_t st) {
  if (mode == 0) {
    hipError_t e = launch_fill_u32(ctr, 0u, kSyncProbeWords, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_barrier_probe, dim3(grid), dim3(512), 0, st, ctr, n);
  } else {
    for (int i = 0; i < n; ++i) hipLaunchKernelGGL(k_empty_probe, dim3(grid), dim3(512), 0, st, ctr);
  }
  return hipGetLastError();
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t st) {
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_fill_u32, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

}  // namespace w4
