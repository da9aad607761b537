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

// Prefill of one layer: block (position i, kv head g); the key pair (t, t + D/2)
// rotated at i with the same arithmetic as the decode step's append.
__global__ void k_prefill_kv(int layer, int slot, KV kv, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                             int ld, const float2* __restrict__ table) {
  const int i = blockIdx.x, g = blockIdx.y, D = kv.D, t = threadIdx.x;
  if (t >= D / 2) return;
  const size_t base = kv_base(kv, layer, slot, g);
  const uint16_t* kp = k + (size_t)i * ld + g * D;
  const uint16_t* vp = v + (size_t)i * ld + g * D;
  const float x0 = h2f(kp[t]), x1 = h2f(kp[t + D / 2]);
  const float2 cs = table[(size_t)i * (D / 2) + t];
  kv.K[base + k_off(D, i, t)] = f2h(x0 * cs.x - x1 * cs.y);
  kv.K[base + k_off(D, i, t + D / 2)] = f2h(x0 * cs.y + x1 * cs.x);
  kv.VT[base + v_off(D, i, t)] = vp[t];
  kv.VT[base + v_off(D, i, t + D / 2)] = vp[t + D / 2];
}

hipError_t launch_prefill_kv(int P, int layer, int slot, const KV& kv, const uint16_t* k, const uint16_t* v, int ld,
                             const float2* table, hipStream_t st) {
  if (P <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_prefill_kv, dim3(P, kv.Hkv), dim3(64), 0, st, layer, slot, kv, k, v, ld, table);
  return hipGetLastError();
}

// The inverse of k_seed: positions 0..P-1 of a slot -> canonical k, v [L][P][Hkv][D].
__global__ void k_read_kv(int P, int slot, KV kv, uint16_t* __restrict__ k, uint16_t* __restrict__ v) {
  const int p0 = blockIdx.x * 64;
  const int l = blockIdx.y / kv.Hkv, g = blockIdx.y - l * kv.Hkv;
  const int D = kv.D;
  const size_t base = kv_base(kv, l, slot, g);
  const int np = min(64, P - p0);
  for (int idx = threadIdx.x; idx < np * D; idx += blockDim.x) {
    const int pp = idx / D, d = idx - pp * D;
    const size_t dst = (((size_t)l * P + p0 + pp) * kv.Hkv + g) * D + d;
    k[dst] = kv.K[base + k_off(D, p0 + pp, d)];
    v[dst] = kv.VT[base + v_off(D, p0 + pp, d)];
  }
}

hipError_t launch_read_kv(int L, int P, int slot, const KV& kv, uint16_t* k, uint16_t* v, hipStream_t st) {
  if (P <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_read_kv, dim3((P + 63) / 64, L * kv.Hkv), dim3(256), 0, st, P, slot, kv, k, v);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention
// Work-group (split sp, kv head g, stream b) of four waves: wave w takes the
// 64-position chunk c = 4 sp + w of stream b (positions 64c .. 64c+63, masked
// beyond the stream's position p).  A stream has nch = p/64 + 1 chunks and
// ns = ceil(nch/4) splits, functions of its own position only, so its result
// is the same in any batch.  With z in log2 units (z = S log2(e) / sqrt(D)):
//   chunk (one wave): S = Q K^T (MFMA); m_c = max z; P = 2^(z - m_c);
//     l_c = sum P; O_c = P V (MFMA, P as fp16 hi + lo parts, fp32 accumulate);
//   split (the work-group, chunks in order): M_s = max m_c, a_c = 2^(m_c - M_s),
//     L_s = sum l_c a_c, O_s = sum O_c a_c;
//   stream and head (the last work-group of (b, g) to finish, splits in
//     order): M = max M_s, b_s = 2^(M_s - M), L = sum L_s b_s,
//     o = sum O_s b_s / L.
// Split partials are published with device-scope stores and counted with a
// device-scope ticket per (b, g); the last work-group reads them back with
// device-scope loads (no cache-wide fence is needed).
struct AttnArgs {
  KV kv;
  int layer, Hq, nsmax;
  // this step's q, k, v of stream b: q at q + b*ldq ([Hq][D]), k and v at
  // knew/vnew + b*ldkv ([Hkv][D]); rotated at the stream's position through
  // table (cos, sin of p * theta^(-2i/D), [cap][D/2]) when table is not null
  const uint16_t* q;
  const uint16_t* knew;
  const uint16_t* vnew;
  int ldq, ldkv;
  const float2* table;
  float* part_o;      // [B][Hq][nsmax][D]  split partials (unnormalised)
  float* part_ml;     // [B][Hq][nsmax][2]  (M_s in log2 units, L_s)
  unsigned* ticket;   // [B][Hkv], zero between launches
  // work-group x -> 8-byte entry (stream b << 16 | split << 8 | kv head,
  // slot << 16 | position): every split of every stream for every kv head,
  // no idle groups
  const int32_t* splits;
  uint16_t* o;        // [B][Hq*D]: row-major (o_rows == 0) or an activation panel with o_rows rows
  int o_rows;
  float scale;        // log2(e) / sqrt(D)
};

// A float pair through one 8-byte device-scope access (partials written and
// read by different work-groups of the same launch).
__device__ __forceinline__ float2 ld_pair(const float* p) {
  const uint64_t u =
      __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
__device__ __forceinline__ void st_pair(float* p, float x, float y) {
  const uint64_t u = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Final combine over a stream's splits, in split order: thread -> (head h,
// four consecutive d).  The partials of NB splits are requested at a time
// (indices clamped within the last batch) before any is used; they are read
// with device-scope loads because other work-groups wrote them in this launch.
template <int D, int NB>
__device__ void combine_splits(const AttnArgs& a, int b, int g, int G, int ns, int tid) {
  for (int i = tid; i < G * D / 4; i += 256) {
    const int h = i / (D / 4), d0 = (i - h * (D / 4)) * 4;
    const size_t row = (size_t)b * a.Hq + g * G + h;
    const float* ml = a.part_ml + row * a.nsmax * 2;
    const float* po = a.part_o + row * a.nsmax * D + d0;
    // M over every split first; when all splits fit one batch (ns <= NB) the
    // batch loaded below gives it, with no separate pass.
    float M = -INFINITY;
    if (ns > NB) {
      for (int s0 = 0; s0 < ns; s0 += NB) {
        float mv[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
          mv[j] = __hip_atomic_load(ml + 2 * min(s0 + j, ns - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < NB; ++j) M = fmaxf(M, mv[j]);  // clamped duplicates do not change a max
      }
    }
    float L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ns; s0 += NB) {
      float mv[NB], lv[NB], ov[NB][4];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int s2 = min(s0 + j, ns - 1);
        const float2 m_l = ld_pair(ml + 2 * s2);
        mv[j] = m_l.x;
        lv[j] = m_l.y;
        const float2 o01 = ld_pair(po + (size_t)s2 * D), o23 = ld_pair(po + (size_t)s2 * D + 2);
        ov[j][0] = o01.x;
        ov[j][1] = o01.y;
        ov[j][2] = o23.x;
        ov[j][3] = o23.y;
      }
      if (ns <= NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) M = fmaxf(M, mv[j]);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (s0 + j < ns) {
          const float bs = __builtin_amdgcn_exp2f(mv[j] - M);
          L = L + lv[j] * bs;
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[k] = acc[k] + ov[j][k] * bs;
        }
    }
    // columns kk .. kk+3 of the [B][Hq*D] output (kk % 4 == 0): consecutive in
    // the row and within one 8-column block of a panel, so one 8-byte store
    const int kk = (g * G + h) * D + d0;
    const size_t off = a.o_rows ? ((size_t)(kk >> 3) * a.o_rows + b) * 8 + (kk & 7) : (size_t)b * a.Hq * D + kk;
    uint16_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = f2h(acc[k] / L);
    *reinterpret_cast<uint2*>(a.o + off) =
        make_uint2((uint32_t)r[0] | ((uint32_t)r[1] << 16), (uint32_t)r[2] | ((uint32_t)r[3] << 16));
  }
}

// VE: the V operands are requested together with K (one memory round trip
// less; about 226 registers, for a work list that fits one work-group per
// compute unit); otherwise after the scores, into the registers K held.
// NT: the K/V chunks with non-temporal loads (each is read once per step).
template <int D, bool VE, bool NT>
__global__ void __launch_bounds__(256, VE ? 1 : 3) k_attn(AttnArgs a) {
  constexpr int KSQ = D / 32;  // k-steps of q.K
  constexpr int NDT = D / 16;  // output d-tiles
  __shared__ float Pl[4][16][65];
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ float s_a[4][16];
  __shared__ __align__(16) uint16_t s_k[4][D];
  __shared__ int s_last;
  extern __shared__ float Ob[];  // [4 waves][G][D]
  const int2 ent = reinterpret_cast<const int2*>(a.splits)[blockIdx.x];
  const int b = ent.x >> 16, sp = (ent.x >> 8) & 0xFF, g = ent.x & 0xFF;
  const int p = ent.y & 0xFFFF, slot_b = ent.y >> 16;
  const int nch = p / 64 + 1, ns = attn_splits(p);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int Hkv = a.kv.Hkv, G = a.Hq / Hkv;
  const int c = kAttnSplitChunks * sp + w;
  static_assert(kAttnSplitChunks == 4, "one wave per chunk in a four-wave work-group");
  const bool live = c < nch;  // this wave's chunk holds positions <= p
  const int col = lane & 15, quad = lane >> 4;
  float mrow[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, lrow[4] = {0.f, 0.f, 0.f, 0.f};
  f4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f4{0.f, 0.f, 0.f, 0.f};
  if (live) {
    const size_t base = kv_base(a.kv, a.layer, slot_b, g);
    const int c0 = c * 64;
    const bool last = (c0 + 63 > p);
    // K operands now; V once the scores are issued, into the registers K
    // held (this keeps the wave under 168 registers: three work-groups per
    // compute unit, so a whole decode batch fits one round of work-groups).
    // Each load is 1 KB contiguous across the wave.
    const uint16_t* Kc = a.kv.K + base + (size_t)c * 64 * D + lane * 8;
    const uint16_t* Vc = a.kv.VT + base + (size_t)c * 64 * D + lane * 8;
    h8 kb[4][KSQ];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks)
        kb[pt][ks] = NT ? ld_h8_nt(Kc + (pt * KSQ + ks) * 512) : ld_h8(Kc + (pt * KSQ + ks) * 512);
    h8 vop[NDT][2];
    auto load_v = [&]() {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          vop[dt][ks] = NT ? ld_h8_nt(Vc + (dt * 2 + ks) * 512) : ld_h8(Vc + (dt * 2 + ks) * 512);
    };
    if (VE) load_v();
    // this wave's chunk holds position p and the launch appends (knew given);
    // a launch without knew appends nothing: every position's K/V is in the arena
    const bool own = a.knew && c == (p >> 6);
    // The wave whose chunk holds position p: this step's k (rotated) and v go
    // into the arena at p and replace what the loads above read there.
    if (own) {
      uint16_t* Ka = a.kv.K + base;
      uint16_t* Va = a.kv.VT + base;
      const uint16_t* kp = a.knew + (size_t)b * a.ldkv + g * D;
      const uint16_t* vp = a.vnew + (size_t)b * a.ldkv + g * D;
      if (lane < D / 2) {
        const float x0 = h2f(kp[lane]), x1 = h2f(kp[lane + D / 2]);
        uint16_t k0 = kp[lane], k1 = kp[lane + D / 2];
        if (a.table) {
          const float2 cs = a.table[(size_t)p * (D / 2) + lane];
          k0 = f2h(x0 * cs.x - x1 * cs.y);
          k1 = f2h(x0 * cs.y + x1 * cs.x);
        }
        s_k[w][lane] = k0;
        s_k[w][lane + D / 2] = k1;
        Ka[k_off(D, p, lane)] = k0;
        Ka[k_off(D, p, lane + D / 2)] = k1;
      }
      for (int d = lane; d < D; d += 64) Va[v_off(D, p, d)] = vp[d];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): s_k written
      __builtin_amdgcn_wave_barrier();
      // K operand: position p is column p%16 of position tile (p%64)/16
      const int ptp = (p & 63) >> 4, colp = p & 15;
      h8 kf[KSQ];
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) kf[ks] = *reinterpret_cast<const h8*>(&s_k[w][32 * ks + 8 * quad]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks)
          if (pt == ptp && col == colp) kb[pt][ks] = kf[ks];
    }
    // Q operand: rows = the G query heads of kv head g (rows >= G are zero),
    // rotated pairs (i, i + D/2) = k-steps (ks, ks + KSQ/2) of the same lane.
    h8 qa[KSQ];
    {
      const uint16_t* qp = a.q + (size_t)b * a.ldq + (g * G + col) * D + 8 * quad;
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) qa[ks] = col < G ? ld_h8(qp + 32 * ks) : h8{0, 0, 0, 0, 0, 0, 0, 0};
      if (a.table && col < G) {
        // 16-byte loads (two (cos, sin) pairs each): the row is 16-byte aligned
        const float4* tr = reinterpret_cast<const float4*>(a.table + (size_t)p * (D / 2) + 8 * quad);
#pragma unroll
        for (int ks = 0; ks < KSQ / 2; ++ks) {
          float4 t4[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) t4[jj] = tr[16 * ks + jj];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float2 cs = (j & 1) ? make_float2(t4[j / 2].z, t4[j / 2].w) : make_float2(t4[j / 2].x, t4[j / 2].y);
            const float x0 = (float)qa[ks][j], x1 = (float)qa[ks + KSQ / 2][j];
            qa[ks][j] = (_Float16)(x0 * cs.x - x1 * cs.y);
            qa[ks + KSQ / 2][j] = (_Float16)(x0 * cs.y + x1 * cs.x);
          }
        }
      }
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
    if (!VE) load_v();
    if (own) {
      // V operand: position p is element p%8 of k-step (p%64)/32 in lane quad
      // (p%32)/8 (the arena already holds it; the loads above may not see it)
      const uint16_t* vp = a.vnew + (size_t)b * a.ldkv + g * D;
      const int ksp = (p & 63) >> 5, qdp = (p & 31) >> 3, jp = p & 7;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const _Float16 vf = __builtin_bit_cast(_Float16, vp[16 * dt + col]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (ks == ksp && quad == qdp && j == jp) vop[dt][ks][j] = vf;
      }
    }
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
      for (int r = 0; r < 4; ++r) Pl[w][4 * quad + r][pt * 16 + col] = S[pt][r];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's P is in LDS
    __builtin_amdgcn_wave_barrier();
    // P as the A operand (row = head col, k = positions 32ks + 8quad + j), hi + lo fp16.
    h8 phi[2], plo[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = Pl[w][col][32 * ks + 8 * quad + j];
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
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        o = mfma16x16x32(phi[ks], vop[dt][ks], o);
        o = mfma16x16x32(plo[ks], vop[dt][ks], o);
      }
      oacc[dt] = o;
    }
  }
  // chunk results to LDS: heads h < G of this wave
  float* ob = Ob + (size_t)w * G * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * quad + r;
      if (h < G) ob[h * D + dt * 16 + col] = oacc[dt][r];
    }
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s_m[w][4 * quad + r] = mrow[r];
      s_l[w][4 * quad + r] = lrow[r];
    }
  }
  __syncthreads();
  // split combine, chunks (waves) in order
  if (tid < G) {
    float M = s_m[0][tid];
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, s_m[ww][tid]);
    float L = 0.f;
    for (int ww = 0; ww < 4; ++ww) {
      const float al = s_m[ww][tid] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[ww][tid] - M);
      s_a[ww][tid] = al;
      L = L + s_l[ww][tid] * al;
    }
    float* ml = a.part_ml + (((size_t)b * a.Hq + g * G + tid) * a.nsmax + sp) * 2;
    st_pair(ml, M, L);
  }
  __syncthreads();
  for (int i = 2 * tid; i < G * D; i += 512) {  // column pairs (d, d + 1)
    const int h = i / D, d = i - h * D;
    float v0 = Ob[(size_t)h * D + d] * s_a[0][h], v1 = Ob[(size_t)h * D + d + 1] * s_a[0][h];
    for (int ww = 1; ww < 4; ++ww) {
      v0 = v0 + Ob[((size_t)ww * G + h) * D + d] * s_a[ww][h];
      v1 = v1 + Ob[((size_t)ww * G + h) * D + d + 1] * s_a[ww][h];
    }
    st_pair(a.part_o + (((size_t)b * a.Hq + g * G + h) * a.nsmax + sp) * D + d, v0, v1);
  }
  __builtin_amdgcn_s_waitcnt(0);  // every partial store complete before the ticket
  __syncthreads();
  unsigned* tk = a.ticket + (size_t)b * Hkv + g;
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(ns - 1);
  __syncthreads();
  if (!s_last) return;
  if (ns <= 2)
    combine_splits<D, 2>(a, b, g, G, ns, tid);
  else if (ns <= 4)
    combine_splits<D, 4>(a, b, g, G, ns, tid);
  else if (ns <= 8)
    combine_splits<D, 8>(a, b, g, G, ns, tid);
  else
    combine_splits<D, 16>(a, b, g, G, ns, tid);
  if (tid == 0) __hip_atomic_store(tk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ prefill attention
// Causal attention of a prompt's P rows over its own K/V in the slot (rows
// 0..P-1 written by k_prefill_kv), one pass over the keys per query block:
// work-group (query block qb of 64 rows, query head h) of four waves; wave w
// takes rows 64 qb + 16 w .. +15 of head h, rotated at their positions
// through table.  The products run transposed, keys (or head dimensions) as
// the MFMA rows and the wave's 16 queries as its columns, so that lane l
// holds query l & 15 throughout.  For each 64-key chunk c = 0 .. qb in order:
//   S^T = K Q^T (MFMA, fp32) as four 16-key tiles, z = S log2(e) / sqrt(D),
//   keys past the row's position masked (the chunk c = qb only);
//   m' = max(m, max_c z) (the lane's 16 keys, then over the four lanes of
//   the query); a = 2^(m - m'); P = 2^(z - m'); l = l a + sum P (per lane,
//   summed over the query's four lanes at the end); O^T = O^T a + V^T P^T
//   (MFMA on P split into fp16 hi + lo parts).
// The tiles' rows are the keys in the order that puts each lane's P values
// where the P^T operand wants them: tile (ks, e), row 4 q + r is key
// 32 ks + 8 q + 4 e + r of the chunk, read from the stored K blocks by a
// per-lane address.  No pass through LDS.
// Then o = O / l, row-major fp16 [P][Hq * D].  Each row attends to keys
// 0 .. its position, the causal definition of the prompt's attention.
struct PfAttnArgs {
  KV kv;
  int layer, slot, P, Hq;
  const uint16_t* qkv;  // q of row i, head h at qkv + i * ldq + h * D
  int ldq;
  const float2* table;  // rotary (cos, sin) [cap][D / 2]
  uint16_t* o;          // [P][ldo], head h at columns h * D ..
  int ldo;
  float scale;          // log2(e) / sqrt(D)
};

typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 hf2 __attribute__((ext_vector_type(2)));

template <int D>
__global__ void __launch_bounds__(256, 3) k_prefill_attn(PfAttnArgs a) {
  constexpr int KSQ = D / 32;  // k-steps of q.K
  constexpr int NDT = D / 16;  // output d-tiles
  // work-groups go out in linear order, x fastest: every head's block of one
  // length before any shorter block (the longest first), and x -> head so
  // that work-groups on one XCD (dispatched round-robin over 8) hold
  // neighbouring heads, which share their kv heads
  const int nqb = (a.P + 63) >> 6;
  const int qb = nqb - 1 - (int)blockIdx.y;
  const int hx = blockIdx.x;
  const int h = (a.Hq & 7) ? hx : (hx & 7) * (a.Hq >> 3) + (hx >> 3), G = a.Hq / a.kv.Hkv, g = h / G;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int r0 = 64 * qb + 16 * w;  // this wave's first row
  // Q^T operand: query col of the wave's 16, rotated pairs (i, i + D/2) =
  // k-steps (ks, ks + KSQ/2) of the same lane
  h8 qa[KSQ];
  {
    const int qp = min(r0 + col, a.P - 1);
    const uint16_t* qrow = a.qkv + (size_t)qp * a.ldq + (size_t)h * D + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) qa[ks] = ld_h8(qrow + 32 * ks);
    const float4* tr = reinterpret_cast<const float4*>(a.table + (size_t)qp * (D / 2) + 8 * quad);
#pragma unroll
    for (int ks = 0; ks < KSQ / 2; ++ks) {
      float4 t4[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) t4[jj] = tr[16 * ks + jj];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 cs = (j & 1) ? make_float2(t4[j / 2].z, t4[j / 2].w) : make_float2(t4[j / 2].x, t4[j / 2].y);
        const float x0 = (float)qa[ks][j], x1 = (float)qa[ks + KSQ / 2][j];
        qa[ks][j] = (_Float16)(x0 * cs.x - x1 * cs.y);
        qa[ks + KSQ / 2][j] = (_Float16)(x0 * cs.y + x1 * cs.x);
      }
    }
  }
  const int qp = r0 + col;  // this lane's query
  float m = -INFINITY, lp = 0.f;
  f4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f4{0.f, 0.f, 0.f, 0.f};
  const size_t base = kv_base(a.kv, a.layer, a.slot, g);
  // K operand of tile (ks, e): row col is key kr = 32 ks + 8 (col >> 2) + 4 e +
  // (col & 3), stored in block kr >> 4 at lane 16 quad + (kr & 15)
  int koff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kr = 32 * (t >> 1) + 8 * (col >> 2) + 4 * (t & 1) + (col & 3);
    koff[t] = (kr >> 4) * KSQ * 512 + (16 * quad + (kr & 15)) * 8;
  }
  for (int c = 0; c <= qb; ++c) {
    const int c0 = 64 * c;
    const uint16_t* Kc = a.kv.K + base + (size_t)c * 64 * D;
    const uint16_t* Vc = a.kv.VT + base + (size_t)c * 64 * D + lane * 8;
    h8 kb[4][KSQ];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) kb[t][ks] = ld_h8(Kc + koff[t] + ks * 512);
    // lane holds S[query col][key c0 + 32 (t >> 1) + 8 quad + 4 (t & 1) + r]
    f4 S[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) acc = mfma16x16x32(kb[t][ks], qa[ks], acc);
      S[t] = acc;
    }
    h8 vop[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) vop[dt][ks] = ld_h8(Vc + (dt * 2 + ks) * 512);
    if (c == qb) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c0 + 32 * (t >> 1) + 8 * quad + 4 * (t & 1) + r > qp) S[t][r] = -INFINITY;
    }
    float mc = S[0][0];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t | r) mc = fmaxf(mc, S[t][r]);
    mc = fmaxf(mc, __shfl_xor(mc, 16, 64));
    mc = fmaxf(mc, __shfl_xor(mc, 32, 64));
    // the scale is positive: the max of the scaled scores is the scaled max
    const float mn = fmaxf(m, mc * a.scale);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float ls = 0.f;
    h8 phi[2], plo[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const f2 e = {__builtin_amdgcn_exp2f(fmaf(S[t][r], a.scale, -mn)),
                      __builtin_amdgcn_exp2f(fmaf(S[t][r + 1], a.scale, -mn))};
        ls = ls + e.x;
        ls = ls + e.y;
        const hf2 hi = __builtin_convertvector(e, hf2);
        const f2 hb = __builtin_convertvector(hi, f2);
        const hf2 lo = __builtin_convertvector((f2{e.x - hb.x, e.y - hb.y}), hf2);
        phi[t >> 1][4 * (t & 1) + r] = hi.x;
        phi[t >> 1][4 * (t & 1) + r + 1] = hi.y;
        plo[t >> 1][4 * (t & 1) + r] = lo.x;
        plo[t >> 1][4 * (t & 1) + r + 1] = lo.y;
      }
    lp = lp * alpha + ls;
    if (c0 + 63 >= a.P) {
      // keys past the prompt hold no data of this stream: zero their V
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c0 + 32 * ks + 8 * quad + j >= a.P) vop[dt][ks][j] = (_Float16)0.0f;
    }
    // O a only where some query of the wave has a new max (a = 1 exactly
    // otherwise, and O 1 = O)
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[dt][r] = oacc[dt][r] * alpha;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f4 o = oacc[dt];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        o = mfma16x16x32(vop[dt][ks], phi[ks], o);
        o = mfma16x16x32(vop[dt][ks], plo[ks], o);
      }
      oacc[dt] = o;
    }
  }
  // l over the query's four lanes; o = O / l for queries below P (lane holds
  // O^T[16 dt + 4 quad + r][query col])
  lp = lp + __shfl_xor(lp, 16, 64);
  lp = lp + __shfl_xor(lp, 32, 64);
  if (qp < a.P) {
    uint16_t* orow = a.o + (size_t)qp * a.ldo + (size_t)h * D + 4 * quad;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 pk;
      pk.x = (uint32_t)f2h(oacc[dt][0] / lp) | ((uint32_t)f2h(oacc[dt][1] / lp) << 16);
      pk.y = (uint32_t)f2h(oacc[dt][2] / lp) | ((uint32_t)f2h(oacc[dt][3] / lp) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * dt) = pk;
    }
  }
}

hipError_t launch_prefill_attention(int P, int layer, int slot, int Hq, const KV& kv, const uint16_t* qkv, int ldq,
                                    const float2* table, uint16_t* o, int ldo, hipStream_t st) {
  if (P < 1 || P > kv.cap || Hq % kv.Hkv || (kv.D != 64 && kv.D != 128)) return hipErrorInvalidValue;
  if (ldo % 4 || reinterpret_cast<uintptr_t>(o) % 8) return hipErrorInvalidValue;  // 8-byte row pieces
  PfAttnArgs a{kv, layer, slot, P, Hq, qkv, ldq, table, o, ldo, (float)(1.4426950408889634 / sqrt((double)kv.D))};
  const dim3 grid(Hq, (P + 63) / 64);
  if (kv.D == 128)
    hipLaunchKernelGGL(k_prefill_attn<128>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_prefill_attn<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(int B, int layer, int Hq, const KV& kv, const int32_t* splits, int nsplits, const uint16_t* q, int ldq, const uint16_t* knew,
                            const uint16_t* vnew, int ldkv, const float2* table, float* part_o, float* part_ml,
                            unsigned* ticket, uint16_t* o, hipStream_t st, void* prof, int o_rows) {
  (void)B;
  AttnArgs a;
  a.kv = kv;
  a.layer = layer;
  a.Hq = Hq;
  a.nsmax = attn_splits(kv.cap - 1);
  a.q = q;
  a.knew = knew;
  a.vnew = vnew;
  a.ldq = ldq;
  a.ldkv = ldkv;
  a.table = table;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.ticket = ticket;
  a.splits = splits;
  a.o = o;
  a.o_rows = o_rows;
  a.scale = (float)(1.4426950408889634 / sqrt((double)kv.D));
  dim3 grid(nsplits);
  const size_t shm = (size_t)4 * (Hq / kv.Hkv) * kv.D * sizeof(float);
  if (prof) prof_arm(prof);
  // measured on the 48-layer model: V with K is faster while the work list
  // fits one work-group per compute unit; beyond that the smaller register
  // footprint (three work-groups per unit) wins
  const bool ve = nsplits <= 128;
  // non-temporal K/V loads for a long decode list (measured: 22.5 against
  // 23.9 us at B = 32, 17.3 against 17.8 at B = 16, slower at B = 8)
  const bool nt = nsplits >= 256;
  if (kv.D == 128) {
    if (ve)
      w4_launch(k_attn<128, true, false>, grid, dim3(256), shm, st, a);
    else if (nt)
      w4_launch(k_attn<128, false, true>, grid, dim3(256), shm, st, a);
    else
      w4_launch(k_attn<128, false, false>, grid, dim3(256), shm, st, a);
  } else {
    if (ve)
      w4_launch(k_attn<64, true, false>, grid, dim3(256), shm, st, a);
    else if (nt)
      w4_launch(k_attn<64, false, true>, grid, dim3(256), shm, st, a);
    else
      w4_launch(k_attn<64, false, false>, grid, dim3(256), shm, st, a);
  }
  return hipGetLastError();
}

}  // namespace w4
