// W4A16 products on gfx950 MFMA: bank repack, the dense M-row GEMM (one
// weight read for all B rows), and the grouped expert GEMMs (gate/up with a
// SwiGLU epilogue, down) over the (expert, stream) buckets.
//
// Operation: y[b][n] = sum_k x[b][k] * q[n][k] * s[n][k/g] with fp32
// accumulation (dense projections applied to all B rows at once and the
// selected experts run as one grouped operation: "Batched-concurrent 4-bit
// serving on Apple Silicon", section 1).
//
// Arithmetic of one output, identical for every batch size B, every row
// position and every tile schedule:
//   * K is cut into slices of KS = 256 columns (128 when K % 256 != 0);
//     wave w of a work-group owns slice w.  KS depends on K only.
//   * within a slice, for each group of g columns: part = MFMA chain
//     (v_mfma_f32_16x16x32_f16, x rows as the A operand, int4 codes converted
//     exactly to fp16 as the B operand) started from zero; then
//     acc = fma(scale, part, acc).
//   * the work-group sums the slices' acc in slice order through LDS.
// MFMA computes each output element from its own A row and B column only, so
// a row's bits do not depend on which other rows share its 16-row tile.
#include "w4_device.h"
#include "w4_internal.h"
#include "w4_tile.h"

namespace w4 {

// ------------------------------------------------------------------ repack
// One thread per 16-byte lane chunk of the destination.
__global__ void k_repack(const uint8_t* __restrict__ src, int N, int K, int Np, int count,
                         uint4* __restrict__ dst) {
  const size_t per = (size_t)Np / 16 * (K / 128) * 64;
  const size_t total = per * count;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t e = idx / per;
    size_t r = idx - e * per;
    const int lane = (int)(r & 63);
    r >>= 6;
    const int kc = (int)(r % (K / 128));
    const int t = (int)(r / (K / 128));
    const int n = t * 16 + (lane & 15);
    const int q = lane >> 4;
    uint32_t out[4];
    for (int s = 0; s < 4; ++s) {
      uint32_t d = 0x88888888u;  // code 0 in offset binary
      if (n < N) {
        const uint8_t* row = src + (e * (size_t)N + n) * (size_t)(K / 2) + kc * 64 + 16 * s + 4 * q;
        uint32_t c = (uint32_t)row[0] | ((uint32_t)row[1] << 8) | ((uint32_t)row[2] << 16) |
                     ((uint32_t)row[3] << 24);
        c ^= 0x88888888u;  // two's complement -> offset binary, per nibble
        d = 0;
        for (int j = 0; j < 4; ++j) {
          d |= ((c >> (8 * j)) & 0xFu) << (4 * j);            // element 2j  -> nibble j
          d |= ((c >> (8 * j + 4)) & 0xFu) << (4 * (j + 4));  // element 2j+1 -> nibble j+4
        }
      }
      out[s] = d;
    }
    dst[idx] = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

__global__ void k_copy_scales(const uint16_t* __restrict__ src, int N, int Np, int G, int count,
                              uint16_t* __restrict__ dst) {
  const size_t total = (size_t)count * Np * G;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t e = i / ((size_t)Np * G);
    const size_t r = i - e * (size_t)Np * G;
    const int n = (int)(r / G), j = (int)(r % G);
    dst[i] = n < N ? src[(e * N + n) * (size_t)G + j] : (uint16_t)0;
  }
}

hipError_t launch_repack(const uint8_t* src_packed, const uint16_t* src_scales, int count, int N, int K, int g,
                         uint4* dst_tiles, uint16_t* dst_scales, hipStream_t st) {
  const int Np = (N + 15) / 16 * 16;
  const size_t total = (size_t)Np / 16 * (K / 128) * 64 * count;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(k_repack, dim3(blocks), dim3(256), 0, st, src_packed, N, K, Np, count, dst_tiles);
  const size_t ts = (size_t)count * Np * (K / g);
  const int b2 = (int)std::min<size_t>((ts + 255) / 256, 65536);
  hipLaunchKernelGGL(k_copy_scales, dim3(b2), dim3(256), 0, st, src_scales, N, Np, K / g, count, dst_scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dense
struct DenseArgs {
  const uint4* tiles;
  const uint16_t* scales;
  int N, K, ntiles;
  const uint16_t* x;
  int ldx, B;
  void* y;
  int ldy;
  int xrows;  // XP kernels: x is a panel with this many rows (see load_x_panel)
};

// Row blocks: work-group row blockIdx.y takes rows 16*MT*blockIdx.y .. +16*MT-1
// of a row-major x (a panel has one block); an output row depends on its own
// input row only, so the blocking never changes a result.
template <int MT, int NCH, int G, int EPI, int LB, bool XP, bool NT = false>
__global__ void __launch_bounds__(LB) k_gemm_dense(DenseArgs a) {
  extern __shared__ float red[];  // two buffers of [NW][MT][64][4]
  constexpr int NS = NCH * 128 / G;
  const int NW = blockDim.x >> 6;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kbase = w * NCH * 128;
  const int G0 = gridDim.x;
  if ((int)blockIdx.x >= a.ntiles) return;
  const int rb = XP ? 0 : (int)blockIdx.y * MT * 16;
  a.B = min(a.B - rb, MT * 16);  // rows of this block
  if (!XP) {
    a.x += (size_t)rb * a.ldx;
    if (EPI == EPI_F32)
      a.y = reinterpret_cast<float*>(a.y) + (size_t)rb * a.ldy;
    else
      a.y = reinterpret_cast<uint16_t*>(a.y) + (size_t)rb * a.ldy;
  }
  XRegs<MT, NCH * 4> x;
  if (XP)
    load_x_panel<MT, NCH>(x, a.x, a.xrows, a.B, kbase, lane);
  else
    load_x<MT, NCH>(x, [&](int row) -> const uint16_t* { return row < a.B ? a.x + (size_t)row * a.ldx : nullptr; },
                    kbase, lane);
  const DqConst dk;
  int buf = 0;
  uint16_t hpre = 0;  // see the single-tile case below
  bool pre = false;
  auto run = [&](const Stage<NCH, G, NT>& st, int t, bool valid) {
    float sv[NS];
    st.scales_f32(sv);
    f4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f4{0.f, 0.f, 0.f, 0.f};
    tile_mac<MT, NCH, G>(x, st.w, sv, acc, dk);
    float* rb = red + buf * NW * MT * 256;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) reinterpret_cast<f4*>(rb)[(w * MT + mt) * 64 + lane] = acc[mt];
    __syncthreads();  // partials of this tile visible; the other buffer's readers are done
    reduce_tile<MT, LB / 64>(rb, NW, [&](int row, int j, float v) {
      const int n = t * 16 + j;
      if (valid && row < a.B && n < a.N) {
        if (EPI == EPI_F32) {
          reinterpret_cast<float*>(a.y)[(size_t)row * a.ldy + n] = v;
        } else if (EPI == EPI_F16) {
          reinterpret_cast<uint16_t*>(a.y)[(size_t)row * a.ldy + n] = f2h(v);
        } else {
          uint16_t* h = reinterpret_cast<uint16_t*>(a.y) + (size_t)row * a.ldy + n;
          const uint16_t hold = pre ? hpre : *h;
          *h = f2h(h2f(hold) + h2f(f2h(v)));
        }
      }
    });
    buf ^= 1;
  };
  // this work-group's tiles: blockIdx.x + i*G0, i < n; processed in pairs,
  // with every load issued unconditionally (indices clamped to the last tile)
  const int n = (a.ntiles - (int)blockIdx.x + G0 - 1) / G0;
  const int last = blockIdx.x + (n - 1) * G0;
  Stage<NCH, G, NT> sa, sb;
  sa.load(a.tiles, a.scales, a.K, blockIdx.x, w, lane);
  if (n == 1) {
    // Residual epilogue of a single tile with one output per thread: the
    // thread's h value is requested now, with the operands, instead of after
    // the reduction (the thread that reads an element is its only writer).
    if (EPI == EPI_RESID && (int)blockDim.x >= MT * 256) {
      const int o = threadIdx.x;
      const int row = (o >> 8) * 16 + ((o >> 4) & 15), col = (int)blockIdx.x * 16 + (o & 15);
      if (o < MT * 256 && row < a.B && col < a.N)
        hpre = reinterpret_cast<const uint16_t*>(a.y)[(size_t)row * a.ldy + col];
      pre = true;
    }
    run(sa, blockIdx.x, true);
    return;
  }
  for (int i = 0; i < n; i += 2) {
    const int ta = blockIdx.x + i * G0, tb = ta + G0;
    sb.load(a.tiles, a.scales, a.K, min(tb, last), w, lane);
    run(sa, ta, true);
    sa.load(a.tiles, a.scales, a.K, min(tb + G0, last), w, lane);
    run(sb, tb, i + 1 < n);
  }
}

// The residual product with K = 16 slices of 256 (the output projection at
// K = 4096) over two 8-wave work-groups per 16-column tile, so that 2x as many
// compute units share the activation panel reads.  Work-group 2t + u takes
// slices 8u .. 8u+7 of tile t and sums its waves' partials in slice order
// (run u); both publish their run sums with device-scope stores and take the
// tile's ticket, and the one that arrives second adds run 0 + run 1 and
// applies the residual epilogue: the order of the one-work-group form
// (reduce_tile), bit for bit.  Neither work-group waits for the other.
// part: [ntiles][2][MT * 256] fp32; ticket [ntiles], zero before and after.
template <int MT, int G, bool NT = false>
__global__ void __launch_bounds__(512) k_gemm_resid_split(DenseArgs a, float* part, unsigned* ticket) {
  extern __shared__ float red[];  // [8 waves][MT][64][4]
  __shared__ int s_last;
  constexpr int NCH = 2, NS = NCH * 128 / G;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x >> 1, half = blockIdx.x & 1;
  if (t >= a.ntiles) return;
  const int ws = half * 8 + w;  // this wave's K slice
  XRegs<MT, NCH * 4> x;
  load_x_panel<MT, NCH>(x, a.x, a.xrows, a.B, ws * NCH * 128, lane);
  Stage<NCH, G, NT> st;
  st.load(a.tiles, a.scales, a.K, t, ws, lane);
  float sv[NS];
  st.scales_f32(sv);
  f4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f4{0.f, 0.f, 0.f, 0.f};
  const DqConst dk;
  tile_mac<MT, NCH, G>(x, st.w, sv, acc, dk);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) reinterpret_cast<f4*>(red)[(w * MT + mt) * 64 + lane] = acc[mt];
  __syncthreads();
  // one output per thread (MT * 256 <= 512 threads): this half's run sum
  const int o = threadIdx.x;
  const bool has = o < MT * 256;
  float run = 0.f;
  uint32_t* mine = reinterpret_cast<uint32_t*>(part) + ((size_t)t * 2 + half) * MT * 256;
  if (has) {
    const int idx = tile_out_idx(o);
    float p[8];
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) p[ww] = red[ww * MT * 256 + idx];
    run = run_sum(p, 8);
    __hip_atomic_store(mine + o, __float_as_uint(run), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the run sums stored before the ticket
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ticket + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1u;
  __syncthreads();
  if (!s_last) return;
  if (has) {
    const uint32_t* other = reinterpret_cast<const uint32_t*>(part) + ((size_t)t * 2 + (half ^ 1)) * MT * 256;
    const float r2 = __uint_as_float(__hip_atomic_load(other + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const float v = half == 0 ? run + r2 : r2 + run;  // run 0 + run 1
    const int row = ((o >> 8) << 4) + ((o >> 4) & 15), n = t * 16 + (o & 15);
    if (row < a.B && n < a.N) {
      uint16_t* h = reinterpret_cast<uint16_t*>(a.y) + (size_t)row * a.ldy + n;
      *h = f2h(h2f(*h) + h2f(f2h(v)));
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(ticket + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef void (*DenseKernel)(DenseArgs);

// LB: launch bound; 512 threads (<= 8 waves) leaves up to 256 VGPRs per lane.
template <int MT, int NCH, int G, int LB, bool XP, bool NT>
static DenseKernel pick_epi(int epi) {
  switch (epi) {
    case EPI_F16: return k_gemm_dense<MT, NCH, G, EPI_F16, LB, XP, NT>;
    case EPI_F32: return k_gemm_dense<MT, NCH, G, EPI_F32, LB, XP, NT>;
    default: return k_gemm_dense<MT, NCH, G, EPI_RESID, LB, XP, NT>;
  }
}
template <int MT, int NCH, int LB, bool XP, bool NT>
static DenseKernel pick_g_lb(int g, int epi) {
  switch (g) {
    case 32: return pick_epi<MT, NCH, 32, LB, XP, NT>(epi);
    case 64: return pick_epi<MT, NCH, 64, LB, XP, NT>(epi);
    default: return pick_epi<MT, NCH, 128, LB, XP, NT>(epi);
  }
}
// non-temporal weight loads only for the decode step's panel products with
// up to 8 waves per tile
template <int MT, int NCH, bool XP>
static DenseKernel pick_g(int g, int epi, int nw, bool nt) {
  if (nw <= 8) {
    if (XP && nt) return pick_g_lb<MT, NCH, 512, XP, true>(g, epi);
    return pick_g_lb<MT, NCH, 512, XP, false>(g, epi);
  }
  return pick_g_lb<MT, NCH, 1024, XP, false>(g, epi);
}
template <bool XP>
static DenseKernel pick(int MT, int nch, int g, int epi, int nw, bool nt) {
  if (MT == 1) return nch == 2 ? pick_g<1, 2, XP>(g, epi, nw, nt) : pick_g<1, 1, XP>(g, epi, nw, nt);
  return nch == 2 ? pick_g<2, 2, XP>(g, epi, nw, nt) : pick_g<2, 1, XP>(g, epi, nw, nt);
}

// Slice width: 256 columns, or 128 when K is not a multiple of 256.
static inline int nch_for(int K) { return (K % 256 == 0) ? 2 : 1; }

hipError_t launch_gemm(const Mat& w, int B, const uint16_t* x, int ldx, void* y, int ldy, int epi, hipStream_t st,
                       int xrows, bool nt) {
  const int nch = nch_for(w.K);
  const int NW = w.K / (nch * 128);
  const int MT = B > 16 ? 2 : 1;
  if (xrows > 0 && B > 32) return hipErrorInvalidValue;  // a panel holds at most 32 rows
  const DenseKernel k = xrows > 0 ? pick<true>(MT, nch, w.g, epi, NW, nt) : pick<false>(MT, nch, w.g, epi, NW, false);
  const int ntiles = w.ntiles();
  const int row_blocks = xrows > 0 ? 1 : (B + 31) / 32;  // 32-row blocks of a longer row-major x
  // enough work-groups to fill 256 CUs at ~16 waves each, each looping over
  // tiles; a mid-size product with at most 8 waves per tile takes two tiles
  // per work-group (the x slices in registers serve both: measured 6.2 us
  // against 7.4 us for 320 tiles at K = 2048, B = 32)
  const int target = std::max(1, 4096 / NW);
  int grid = std::min(ntiles, target);
  if (NW <= 8 && ntiles >= 256 && ntiles <= 1024) grid = (ntiles + 1) / 2;
  // many row blocks (a prompt): about 8 column tiles per work-group, so the x
  // rows in registers serve 8 weight tiles instead of being re-read for each
  if (row_blocks > 1) grid = std::max(1, (ntiles + 7) / 8);
  DenseArgs a{w.tiles, w.scales, w.N, w.K, ntiles, x, ldx, B, y, ldy, xrows};
  w4_launch(k, dim3(grid, row_blocks), dim3(NW * 64), 2 * NW * MT * 1024, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ large-M products (prompt rows)
// y[M][N] for a prompt's M rows.  Work-group (row block of 128 rows, column
// block of 8 tiles) of four waves in a 2 x 2 grid; wave (wm, wn) computes rows
// 64 wm .. +63 by tiles 4 wn .. +3 (16 MFMA tiles).  K streams in 128-column
// chunks through two LDS stages filled by direct-to-LDS loads (16 bytes per
// lane, no registers): the block's x rows in A operand order ([row tile]
// [k-step][lane]) and the 8 tiles' codes as stored.  The next chunk is
// requested right after the barrier that publishes the current one, so it
// arrives while the current one is multiplied; each wave converts its four
// tiles' codes per k-step.  Per output: acc = fma(scale, MFMA chain of the
// group from zero, acc) over the groups in K order, fp32 (the M-row decode
// product adds per-slice sums instead: the same terms, rounded differently).
struct LmArgs {
  const uint4* tiles;
  const uint16_t* scales;
  int N, K, ntiles;
  const uint16_t* x;
  int ldx, M;
  void* y;
  int ldy;
};

template <int G, int EPI>
__global__ void __launch_bounds__(256, 2) k_gemm_lm(LmArgs a) {
  constexpr int NGC = 128 / G, SPG = G / 32;
  constexpr int AW = 8 * 4 * 64;  // 16-byte words of a stage's A part; then 8 x 64 words of codes
  __shared__ __align__(16) v4u lds[2][AW + 8 * 64];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, i16 = lane & 15, quad = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.x * 128, t0 = blockIdx.y * 8;
  const int NK = a.K / 128, KG = a.K / G;
  // this wave's loads of a chunk: row tiles 2w, 2w+1 (rows past M read row
  // M-1) and the codes of tiles 2w, 2w+1 (tiles past N read tile 0; neither
  // is stored)
  const uint16_t* xr0 = a.x + (size_t)min(m0 + 32 * w + i16, a.M - 1) * a.ldx + 8 * quad;
  const uint16_t* xr1 = a.x + (size_t)min(m0 + 32 * w + 16 + i16, a.M - 1) * a.ldx + 8 * quad;
  const int tc0 = t0 + 2 * w < a.ntiles ? t0 + 2 * w : 0, tc1 = t0 + 2 * w + 1 < a.ntiles ? t0 + 2 * w + 1 : 0;
  const uint4* bp0 = a.tiles + (size_t)tc0 * NK * 64 + lane;
  const uint4* bp1 = a.tiles + (size_t)tc1 * NK * 64 + lane;
  const uint16_t* sp[4];  // scales of this lane's column in the wave's four tiles
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = t0 + 4 * wn + c;
    sp[c] = a.scales + (size_t)((t < a.ntiles ? t : 0) * 16 + i16) * KG;
  }
  uint16_t scn[4][NGC];
  auto issue = [&](int kc, int st) {
    v4u* L = lds[st];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      __builtin_amdgcn_global_load_lds(xr0 + kc * 128 + 32 * ks, L + ((2 * w) * 4 + ks) * 64, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(xr1 + kc * 128 + 32 * ks, L + ((2 * w + 1) * 4 + ks) * 64, 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(bp0 + kc * 64, L + AW + (2 * w) * 64, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(bp1 + kc * 64, L + AW + (2 * w + 1) * 64, 16, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int gq = 0; gq < NGC; ++gq) scn[c][gq] = sp[c][kc * NGC + gq];
  };
  const DqConst dk;
  f4 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = f4{0.f, 0.f, 0.f, 0.f};
  issue(0, 0);
  for (int kc = 0; kc < NK; ++kc) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk kc are in LDS (and its scales in registers)
    float sc[4][NGC];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int gq = 0; gq < NGC; ++gq) sc[c][gq] = h2f(scn[c][gq]);
    __syncthreads();  // every wave's chunk kc is in LDS; every wave is done with chunk kc-1's stage
    if (kc + 1 < NK) issue(kc + 1, (kc + 1) & 1);
    const v4u* L = lds[kc & 1];
    v4u braw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) braw[c] = L[AW + (4 * wn + c) * 64 + lane];
#pragma unroll
    for (int gq = 0; gq < NGC; ++gq) {
      f4 part[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) part[r][c] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = gq * SPG; s2 < (gq + 1) * SPG; ++s2) {
        h8 av[4], bv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = __builtin_bit_cast(h8, L[((4 * wm + r) * 4 + s2) * 64 + lane]);
#pragma unroll
        for (int c = 0; c < 4; ++c) bv[c] = dq8(braw[c][s2], dk);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < 4; ++c) part[r][c] = mfma16x16x32(av[r], bv[c], part[r][c]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[r][c][e] = fmaf(sc[c][gq], part[r][c][e], acc[r][c][e]);
    }
  }
  // lane holds rows 4 quad + e of each row tile, column i16 of each tile
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = t0 + 4 * wn + c, n = t * 16 + i16;
    if (t >= a.ntiles || n >= a.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 64 * wm + 16 * r + 4 * quad + e;
        if (row >= a.M) continue;
        const float v = acc[r][c][e];
        const size_t o = (size_t)row * a.ldy + n;
        if (EPI == EPI_F32) {
          reinterpret_cast<float*>(a.y)[o] = v;
        } else if (EPI == EPI_F16) {
          reinterpret_cast<uint16_t*>(a.y)[o] = f2h(v);
        } else {
          uint16_t* h = reinterpret_cast<uint16_t*>(a.y) + o;
          *h = f2h(h2f(*h) + h2f(f2h(v)));
        }
      }
  }
}

template <int EPI>
static void (*lm_pick(int g))(LmArgs) {
  switch (g) {
    case 32: return k_gemm_lm<32, EPI>;
    case 64: return k_gemm_lm<64, EPI>;
    default: return k_gemm_lm<128, EPI>;
  }
}

bool lm_ok(const Mat& w, int ldx) {
  return w.K % 128 == 0 && (w.g == 32 || w.g == 64 || w.g == 128) && ldx % 8 == 0 && ldx >= w.K;
}

hipError_t launch_gemm_lm(const Mat& w, int M, const uint16_t* x, int ldx, void* y, int ldy, int epi,
                          hipStream_t st) {
  if (!lm_ok(w, ldx) || M < 1 || (reinterpret_cast<uintptr_t>(x) & 15)) return hipErrorInvalidValue;
  LmArgs a{w.tiles, w.scales, w.N, w.K, w.ntiles(), x, ldx, M, y, ldy};
  void (*k)(LmArgs) = epi == EPI_F32 ? lm_pick<EPI_F32>(w.g) : epi == EPI_F16 ? lm_pick<EPI_F16>(w.g)
                                                                               : lm_pick<EPI_RESID>(w.g);
  w4_launch(k, dim3((M + 127) / 128, (a.ntiles + 7) / 8), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ grouped experts
struct MoeArgs {
  const uint4* t0;        // gate (or down) tiles of expert 0; experts consecutive
  const uint4* t1;        // up tiles (gate/up only)
  const uint16_t* s0;
  const uint16_t* s1;
  int N, K, ntiles;       // per expert
  size_t tile_stride;     // uint4 per expert
  size_t scale_stride;    // halves per expert
  const uint16_t* x;      // gate/up: rows by stream; down: rows by pair
  int ldx;
  const int4* units;      // (expert, first pair, rows, 0) of every 16-row unit, experts ascending
  const int32_t* unit_rows;  // [unit][16] stream of each row (gate/up input rows)
  const uint4* rows8;        // [unit] the same as 16 bytes when rows8_ok, else any readable [units_cap] array
  int rows8_ok;
  const int32_t* n_units;
  int units_cap;          // records allocated in units, at most 2 per thread
  uint16_t* out;          // [pairs][N]
  const int32_t* dst_rows;  // down: output row of each pair (null: the pair's own row)
  int ncu;                // compute units
  int dshare;             // range weight skew in 1/1000 (see k_moe)
};

// s_setprio takes an immediate: level 0..3.
__device__ __forceinline__ void set_prio_level(int l) {
  if (l >= 3)
    __builtin_amdgcn_s_setprio(3);
  else if (l == 2)
    __builtin_amdgcn_s_setprio(2);
  else if (l == 1)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Persistent grouped GEMM.  The work is the flattened list of (unit, column
// tile) items, unit = 16 rows of one used expert (the routing kernel builds
// the unit list on the device); work-group i takes items
// [i*total/grid, (i+1)*total/grid), so every work-group gets the same share
// whatever the routing.  Its NW waves own the K slices (as in the dense
// product); the x slice of the current unit stays in registers.  Items go
// through two register stages in pairs, the next item's loads in flight
// while the current one is multiplied and reduced; the prefetch runs across
// unit boundaries (the x slice of a new unit is loaded after the last
// multiply of the previous one, with its first tiles already in flight).
// The arithmetic of an output does not depend on which work-group computes
// it.
// ONE (gate/up of a single stream): every unit's rows are row 0 of x, so the
// x slice is requested at the start with the unit records, not after them.
// MT = 2 (a prompt's products): units of 32 rows, two 16-row MFMA tiles per
// item sharing each converted weight operand; MFMA computes each output row
// from its own A row, so the results are the same as with 16-row units.
template <int NCH, int G, bool GATEUP, int LB, bool NT = false, bool ONE = false, int MT = 1>
__global__ void __launch_bounds__(LB) k_moe(MoeArgs a) {
  static_assert(MT == 1 || (!NT && !ONE), "32-row units: plain loads, several streams");
  constexpr int US = 16 * MT;  // rows per unit
  // dynamic LDS: two buffers of [GATEUP ? 2 : 1][NW][MT][64][4] partials, then
  // the unit records (max(units_cap, kMaxUnits)), then for the non-temporal
  // gate/up the unit rows as bytes (kMaxUnits x 16)
  extern __shared__ float red[];
  constexpr int NS = NCH * 128 / G;
  const int NW = blockDim.x >> 6;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = a.ntiles;
  // Every allocated unit record is requested together with the unit count
  // (records past the count are stale and never used), so the work range and
  // its records arrive in one round trip.
  const int tid = threadIdx.x, nth = blockDim.x;
  const int4 rec0 = a.units[min(tid, a.units_cap - 1)], rec1 = a.units[min(tid + nth, a.units_cap - 1)];
  // gate/up of more than 8 streams in a decode step (the non-temporal
  // variant): the unit rows (input row of each unit row, one byte each) come
  // in the same round trip, so a unit's x rows are requested without waiting
  // for its row list first (B = 32: 6288 against 6232 tok/s; at B = 4 and 8
  // with plain loads it was measured 0.8% slower, so those keep the row list
  // loads)
  constexpr bool ROWS = GATEUP && !ONE && NT;
  const bool rl = ROWS && a.rows8_ok;
  uint4 rr0 = {0u, 0u, 0u, 0u}, rr1 = {0u, 0u, 0u, 0u};
  if constexpr (ROWS) {
    rr0 = a.rows8[min(tid, a.units_cap - 1)];
    rr1 = a.rows8[min(tid + nth, a.units_cap - 1)];
  }
  const int nu = *a.n_units;
  const long long total = (long long)nu * T;
  XRegs<MT, NCH * 4> x;
  if constexpr (ONE) {
    const uint16_t* xr = a.x + w * NCH * 128 + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < NCH * 4; ++ks) x.a[0][ks] = ld_h8(xr + ks * 32);
  }
  // Ranges by weight: the first work-group dispatched to each compute unit
  // (blockIdx < ncu) takes 1 + d shares, the other 1 - d (d = dshare/1000):
  // with equal shares the second ones were measured to finish 2-3 us later.
  // (gate/up only; the down product keeps equal shares)
  int f_begin, f_end;
  if (GATEUP) {
    const long long C = min((long long)a.ncu, (long long)gridDim.x), dq = a.dshare;
    const long long W = C * (1000 + dq) + ((long long)gridDim.x - C) * (1000 - dq);
    auto cum = [&](long long i) {
      return i <= C ? i * (1000 + dq) : C * (1000 + dq) + (i - C) * (1000 - dq);
    };
    f_begin = (int)(cum(blockIdx.x) * total / W);
    f_end = (int)(cum(blockIdx.x + 1) * total / W);
  } else {
    f_begin = (int)(blockIdx.x * total / gridDim.x);
    f_end = (int)((blockIdx.x + 1) * total / gridDim.x);
  }
  if (f_begin >= f_end) return;
  const int last = f_end - 1;
  const int kbase = w * NCH * 128;
  const int bufsz = (GATEUP ? 2 : 1) * NW * MT * 256;
  const int i16 = lane & 15;
  const DqConst dk;
  // Unit records are read from LDS inside the loop: a record loaded from
  // global memory there is a vector load (the kernel's stores might alias
  // it), and a wait for it would also wait for the tile loads in flight.
  int4* lrec = reinterpret_cast<int4*>(red + 2 * bufsz);
  if (tid < a.units_cap) lrec[tid] = rec0;
  if (tid + nth < a.units_cap) lrec[tid + nth] = rec1;
  for (int i = tid + 2 * nth; i < a.units_cap; i += nth) lrec[i] = a.units[i];  // prefill: more records
  uint4* lrow8 = reinterpret_cast<uint4*>(lrec + max(a.units_cap, kMaxUnits));
  const uint8_t* lrow = reinterpret_cast<const uint8_t*>(lrow8);
  if (rl) {
    if (tid < a.units_cap) lrow8[tid] = rr0;
    if (tid + nth < a.units_cap) lrow8[tid + nth] = rr1;
    for (int i = tid + 2 * nth; i < a.units_cap; i += nth) lrow8[i] = a.rows8[i];
  }
  __syncthreads();

  // item f's tile into a stage.  Past the range: with plain loads the WG's
  // last tile again (a cache hit); with non-temporal loads, which do not keep
  // that tile in the cache, every lane of a wave reads the first 16-byte word
  // of the wave's slice of expert 0's tile (blockIdx mod tiles) instead: one
  // line per load, spread over the cache channels, whose results are never
  // stored.  Either way the loads are issued on every trip, so the waits in
  // the loop stay the same (B = 32 gate/up: 180.0 against 213.4 MB fetched per
  // launch, 1.5% more tok/s).
  auto stage_load = [&](Stage<NCH, G, NT>& g0, Stage<NCH, G, NT>& g1, int f) {
    const bool ok = !NT || f <= last;
    const int fc = min(f, last), u = __builtin_amdgcn_readfirstlane(fc / T);
    const int t = ok ? fc - u * T : (int)(blockIdx.x % T), ln = ok ? lane : 0;
    const int e = ok ? lrec[u].x : 0;
    g0.load(a.t0 + a.tile_stride * e, a.s0 + a.scale_stride * e, a.K, t, w, ln);
    if (GATEUP) g1.load(a.t1 + a.tile_stride * e, a.s1 + a.scale_stride * e, a.K, t, w, ln);
  };
  // x slice of unit u (rows past the unit's count repeat row 0; their
  // outputs are not stored)
  // (gate/up: the next unit's row index is loaded a unit ahead, so a switch
  // does not wait for it)
  int xu = -1, nrow[MT] = {};
  // stream of row i of unit u (rows past the unit's count: any of its rows);
  // 64-row units (a prompt's gate/up) are runs of two 32-row units whose rows
  // are listed from the first of them (record field w)
  auto unit_row = [&](int u, int i) -> int {
    if constexpr (MT == 4) {
      const int4 un = lrec[u];
      return a.unit_rows[un.w * 32 + min(i, un.z - 1)];
    }
    return a.unit_rows[u * US + i];
  };
  // down with dst_rows: output rows of the unit being loaded, written to
  // s_dst[unit & 1] by the unit's first multiply (a load in flight is not
  // waited for before the next tile loads are issued); a unit's rows are
  // read after a barrier that every wave passes after the previous unit's
  // last reduction
  __shared__ int s_dst[2][16];
  int dreg = 0;
  bool dpend = false;
  auto load_x = [&](int uv, const int (&grow)[MT]) {
    const int u = __builtin_amdgcn_readfirstlane(uv);
    if constexpr (ONE) {
      xu = u;
      return;
    }
    const int4 un = lrec[u];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row =
          GATEUP ? (rl ? lrow[u * 16 + i16] : grow[mt]) : un.y + min(mt * 16 + i16, un.z - 1);
      const uint16_t* xr = a.x + (size_t)row * a.ldx + kbase + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < NCH * 4; ++ks) x.a[mt][ks] = ld_h8(xr + ks * 32);
    }
    xu = u;
    if (GATEUP && !ONE && !rl) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) nrow[mt] = unit_row(min(u + 1, nu - 1), mt * 16 + i16);
    }
    if (!GATEUP && a.dst_rows) {
      dreg = a.dst_rows[un.y + min(i16, un.z - 1)];
      dpend = true;
    }
  };

  int buf = 0;
  auto run = [&](const Stage<NCH, G, NT>& g0, const Stage<NCH, G, NT>& g1, int f, bool valid) {
    const int u = __builtin_amdgcn_readfirstlane(min(f, last) / T), t = min(f, last) - u * T;
    const int4 un = lrec[u];
    const int off = un.y, m = un.z;
    float sv0[NS], sv1[NS];
    g0.scales_f32(sv0);
    f4 acc0[MT], acc1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc0[mt] = f4{0.f, 0.f, 0.f, 0.f};
      acc1[mt] = f4{0.f, 0.f, 0.f, 0.f};
    }
    tile_mac<MT, NCH, G>(x, g0.w, sv0, acc0, dk);
    if (GATEUP) {
      g1.scales_f32(sv1);
      tile_mac<MT, NCH, G>(x, g1.w, sv1, acc1, dk);
    }
    float* rb = red + buf * bufsz;
    f4* r4 = reinterpret_cast<f4*>(rb);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      r4[(w * MT + mt) * 64 + lane] = acc0[mt];
      if (GATEUP) r4[((NW + w) * MT + mt) * 64 + lane] = acc1[mt];
    }
    if (!GATEUP && dpend) {
      if (tid < 16) s_dst[u & 1][tid] = dreg;
      dpend = false;
    }
    __syncthreads();  // this tile's partials visible; the other buffer's readers are done
    if (GATEUP) {
      // lanes l and l^32 of a wave sum the gate and the up partials of one
      // output (slices in order, every read issued before the adds)
      constexpr int NB = LB / 64;  // >= NW
      for (int ob = 0; ob < MT * 256; ob += NW * 32) {  // uniform trip count
        const int o = ob + w * 32 + (lane & 31), pp = lane >> 5;
        const int oc = min(o, MT * 256 - 1);
        const int i = ((oc >> 8) << 4) + ((oc >> 4) & 15), j = oc & 15;  // unit row, column
        const float* p = rb + pp * NW * MT * 256 + tile_out_idx(oc);
        float r[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) r[k] = p[min(k, NW - 1) * MT * 256];
        float v = r[0];
#pragma unroll
        for (int k = 1; k < NB; ++k) v = k < NW ? v + r[k] : v;
        const float vu = __shfl_xor(v, 32, 64);
        const int n = t * 16 + j;
        if (pp == 0 && o < MT * 256 && valid && i < m && n < a.N) {
          const float gt = h2f(f2h(v)), up = h2f(f2h(vu));
          const float silu = gt / (1.0f + expf(-gt));
          a.out[(size_t)(off + i) * a.N + n] = f2h(silu * up);
        }
      }
    } else {
      reduce_tile<MT, LB / 64>(rb, NW, [&](int i, int j, float v) {
        const int n = t * 16 + j;
        if (valid && i < m && n < a.N) {
          const int orow = a.dst_rows ? s_dst[u & 1][i] : off + i;
          a.out[(size_t)orow * a.N + n] = f2h(v);
        }
      });
    }
    buf ^= 1;
  };

  // Items in pairs through stages a and b.  A new unit's x is loaded after
  // the previous multiply and before the next prefetch: the multiply that
  // needs it waits for its own stage, issued earlier, in any case.
  Stage<NCH, G, NT> a0, a1, b0, b1;
  stage_load(a0, a1, f_begin);
  {
    int r0[MT] = {};
    if (GATEUP && !ONE && !rl) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) r0[mt] = unit_row(f_begin / T, mt * 16 + i16);
    }
    load_x(f_begin / T, r0);
  }
  stage_load(b0, b1, f_begin + 1);
  // Whole pairs in the loop; an odd range's last item after it, from the
  // stage the loop's last trip loaded (no multiply of a stage that holds no
  // item of the range; the loop body and its waits are the same as with the
  // odd item inside it).
  const int f_pairs = f_begin + ((f_end - f_begin) & ~1);
  for (int f = f_begin; f < f_pairs; f += 2) {
    // Issue priority by remaining work: the waves of the work-group with
    // more tiles left win the compute unit's arbitration, so a work-group
    // that falls behind the one sharing its compute unit catches up.
    set_prio_level((4 * (f_end - f)) / (f_end - f_begin + 1));
    run(a0, a1, f, true);
    if ((f + 1) / T != xu) load_x((f + 1) / T, nrow);
    stage_load(a0, a1, f + 2);
    run(b0, b1, f + 1, true);
    if (f + 2 < f_end && (f + 2) / T != xu) load_x((f + 2) / T, nrow);
    stage_load(b0, b1, f + 3);
  }
  if (f_pairs < f_end) {
    set_prio_level(0);
    run(a0, a1, f_pairs, true);
  }
}

// ------------------------------------------------------------------ fused expert products
// The grouped gate/up (+ SwiGLU) and down products in one launch, with the
// arithmetic of k_moe for both, bit for bit.  Work-group i:
//   1. runs its range of gate/up items, the range and the item loop of the
//      gate/up launch (8 waves own the K slices), but stores the activations
//      with device-scope stores;
//   2. once its range is done (every store complete), adds the number of
//      items it finished of each unit to that unit's counter done[u] (zeroed
//      by the bucketing that built the units); the work-group whose add
//      completes a unit writes the launch's epoch into the unit's ready
//      word, in eight copies;
//   3. requests the weights of its first down items, then one thread waits
//      until every unit its down range touches is ready (polling the copy
//      blockIdx % 8, so few work-groups poll one line), and the work-group
//      runs the range in S = NW / NWd sub-groups of NWd waves (the down
//      product's slices), sub-group s a contiguous part of the range, reading
//      the activations through the caches after an acquire (the waiting
//      thread invalidates this compute unit's and this XCD's stale lines).
// Counters and ready copies sit 256 bytes apart.  The down product's tiles
// therefore start on compute units whose gate/up share is done while others
// still finish theirs.  Gate/up items never wait and the grid is the number
// of work-groups the device keeps resident, so every wait ends; one that
// exceeds its bound sets *err (a host-visible word) and goes on.
struct MoeFusedArgs {
  MoeArgs gu, dn;
  uint32_t* done;   // [units_cap] x kDoneStride words: zero for the units of this launch
  uint32_t* ready;  // [units_cap][8] x kDoneStride words: never equal to a later epoch
  uint32_t epoch;   // this launch's value, larger than any earlier one on these words
  int32_t* err;     // host-mapped word
};

constexpr int kWaitSpins = 1 << 18;

template <int NCH, int NCHD, int G, int LB>
__global__ void __launch_bounds__(LB) k_moe_fused(MoeFusedArgs fa) {
  extern __shared__ float red[];
  const MoeArgs& a = fa.gu;
  constexpr int NS = NCH * 128 / G;
  const int NW = blockDim.x >> 6;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = a.ntiles;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int4 rec0 = a.units[min(tid, a.units_cap - 1)], rec1 = a.units[min(tid + nth, a.units_cap - 1)];
  const int nu = *a.n_units;
  const long long total = (long long)nu * T;
  int f_begin, f_end;
  {
    const long long C = min((long long)a.ncu, (long long)gridDim.x), dq = a.dshare;
    const long long W = C * (1000 + dq) + ((long long)gridDim.x - C) * (1000 - dq);
    auto cum = [&](long long i) {
      return i <= C ? i * (1000 + dq) : C * (1000 + dq) + (i - C) * (1000 - dq);
    };
    f_begin = (int)(cum(blockIdx.x) * total / W);
    f_end = (int)(cum(blockIdx.x + 1) * total / W);
  }
  const int bufsz = 2 * NW * 256;
  const int i16 = lane & 15;
  const DqConst dk;
  int4* lrec = reinterpret_cast<int4*>(red + 2 * bufsz);
  if (tid < a.units_cap) lrec[tid] = rec0;
  if (tid + nth < a.units_cap) lrec[tid + nth] = rec1;
  for (int i = tid + 2 * nth; i < a.units_cap; i += nth) lrec[i] = a.units[i];
  __syncthreads();

  // ---- 1. gate/up items [f_begin, f_end)
  if (f_begin < f_end) {
    const int last = f_end - 1;
    const int kbase = w * NCH * 128;
    auto stage_load = [&](Stage<NCH, G>& g0, Stage<NCH, G>& g1, int f) {
      const int fc = min(f, last), u = __builtin_amdgcn_readfirstlane(fc / T), t = fc - u * T;
      const int e = lrec[u].x;
      g0.load(a.t0 + a.tile_stride * e, a.s0 + a.scale_stride * e, a.K, t, w, lane);
      g1.load(a.t1 + a.tile_stride * e, a.s1 + a.scale_stride * e, a.K, t, w, lane);
    };
    XRegs<1, NCH * 4> x;
    int xu = -1, nrow = 0;
    auto load_x = [&](int uv, int grow) {
      const int u = __builtin_amdgcn_readfirstlane(uv);
      const uint16_t* xr = a.x + (size_t)grow * a.ldx + kbase + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < NCH * 4; ++ks) x.a[0][ks] = ld_h8(xr + ks * 32);
      xu = u;
      nrow = a.unit_rows[min(u + 1, nu - 1) * 16 + i16];
    };
    int buf = 0;
    auto run = [&](const Stage<NCH, G>& g0, const Stage<NCH, G>& g1, int f, bool valid) {
      const int u = __builtin_amdgcn_readfirstlane(min(f, last) / T), t = min(f, last) - u * T;
      const int4 un = lrec[u];
      const int off = un.y, m = un.z;
      float sv0[NS], sv1[NS];
      g0.scales_f32(sv0);
      f4 acc0[1] = {f4{0.f, 0.f, 0.f, 0.f}}, acc1[1] = {f4{0.f, 0.f, 0.f, 0.f}};
      tile_mac<1, NCH, G>(x, g0.w, sv0, acc0, dk);
      g1.scales_f32(sv1);
      tile_mac<1, NCH, G>(x, g1.w, sv1, acc1, dk);
      float* rb = red + buf * bufsz;
      f4* r4 = reinterpret_cast<f4*>(rb);
      r4[w * 64 + lane] = acc0[0];
      r4[(NW + w) * 64 + lane] = acc1[0];
      __syncthreads();
      constexpr int NB = LB / 64;
      for (int ob = 0; ob < 256; ob += NW * 32) {
        const int o = ob + w * 32 + (lane & 31), pp = lane >> 5;
        const int oc = min(o, 255);
        const int i = oc >> 4, j = oc & 15;
        const float* p = rb + pp * NW * 256 + ((i >> 2) * 16 + j) * 4 + (i & 3);
        float r[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) r[k] = p[min(k, NW - 1) * 256];
        float v = r[0];
#pragma unroll
        for (int k = 1; k < NB; ++k) v = k < NW ? v + r[k] : v;
        const float vu = __shfl_xor(v, 32, 64);
        const int n = t * 16 + j;
        if (pp == 0 && o < 256 && valid && i < m && n < a.N) {
          const float gt = h2f(f2h(v)), up = h2f(f2h(vu));
          const float silu = gt / (1.0f + expf(-gt));
          __hip_atomic_store(a.out + (size_t)(off + i) * a.N + n, f2h(silu * up), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      buf ^= 1;
    };
    Stage<NCH, G> a0, a1, b0, b1;
    stage_load(a0, a1, f_begin);
    load_x(f_begin / T, a.unit_rows[(f_begin / T) * 16 + i16]);
    stage_load(b0, b1, f_begin + 1);
    for (int f = f_begin; f < f_end; f += 2) {
      set_prio_level((4 * (f_end - f)) / (f_end - f_begin + 1));
      run(a0, a1, f, true);
      if (f + 1 < f_end && (f + 1) / T != xu) load_x((f + 1) / T, nrow);
      stage_load(a0, a1, f + 2);
      run(b0, b1, f + 1, f + 1 < f_end);
      if (f + 2 < f_end && (f + 2) / T != xu) load_x((f + 2) / T, nrow);
      stage_load(b0, b1, f + 3);
    }
    set_prio_level(0);
  }
  // ---- 2. this range's items are stored: count them per unit
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (f_begin < f_end) {
    const int u0 = f_begin / T, u1 = (f_end - 1) / T;
    for (int u = u0 + tid; u <= u1; u += nth) {
      const uint32_t n = (uint32_t)(min(f_end, (u + 1) * T) - max(f_begin, u * T));
      const uint32_t old = __hip_atomic_fetch_add(fa.done + (size_t)u * kDoneStride, n, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      if (old + n == (uint32_t)T)
        for (int c = 0; c < 8; ++c)
          __hip_atomic_store(fa.ready + ((size_t)u * 8 + c) * kDoneStride, fa.epoch, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- 3. down items of this work-group, in sub-groups of NWd waves
  const MoeArgs& d = fa.dn;
  constexpr int NSD = NCHD * 128 / G;
  const int NWd = d.K / (NCHD * 128);
  const int S = NW / NWd;
  const int sg = w / NWd, ws = w - sg * NWd;
  const bool act = sg < S;
  const int Td = d.ntiles;
  const long long dtotal = (long long)nu * Td;
  const int d0 = (int)(blockIdx.x * dtotal / gridDim.x), d1 = (int)((blockIdx.x + 1) * dtotal / gridDim.x);
  const int len = d1 - d0, n_iter = (len + S - 1) / S;
  const int sb = act ? d0 + (int)((long long)sg * len / S) : d0;
  const int se = act ? d0 + (int)((long long)(sg + 1) * len / S) : d0;
  const int cnt = se - sb;
  const bool any = act && cnt > 0;
  const int dlast = any ? se - 1 : 0;
  const int kb = ws * NCHD * 128;
  float* dred = red + (act ? sg : 0) * 2 * NWd * 256;
  auto dstage = [&](Stage<NCHD, G>& g, int i) {
    const int f = min(sb + i, dlast), u = __builtin_amdgcn_readfirstlane(f / Td), t = f - u * Td;
    const int e = lrec[u].x;
    g.load(d.t0 + d.tile_stride * e, d.s0 + d.scale_stride * e, d.K, t, ws, lane);
  };
  XRegs<1, NCHD * 4> xd;
  int xdu = -1;
  auto dload_x = [&](int uv) {
    const int u = __builtin_amdgcn_readfirstlane(uv);
    const int4 un = lrec[u];
    const int row = un.y + min(i16, un.z - 1);
    const uint16_t* xr = d.x + (size_t)row * d.ldx + kb + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < NCHD * 4; ++ks) xd.a[0][ks] = ld_h8(xr + ks * 32);
    xdu = u;
  };
  int dbuf = 0;
  auto drun = [&](const Stage<NCHD, G>& g, int i) {
    const bool valid = any && i < cnt;
    const int f = min(sb + i, dlast);
    const int u = __builtin_amdgcn_readfirstlane(f / Td), t = f - u * Td;
    const int4 un = lrec[u];
    const int off = un.y, m = un.z;
    float* rb = dred + dbuf * NWd * 256;
    if (any) {
      float sv[NSD];
      g.scales_f32(sv);
      f4 acc[1] = {f4{0.f, 0.f, 0.f, 0.f}};
      tile_mac<1, NCHD, G>(xd, g.w, sv, acc, dk);
      reinterpret_cast<f4*>(rb)[ws * 64 + lane] = acc[0];
    }
    __syncthreads();
    if (any)
      reduce_tile_sub<1, LB / 64>(rb, NWd, tid - sg * NWd * 64, NWd * 64, [&](int i_, int j, float v) {
        const int n = t * 16 + j;
        if (valid && i_ < m && n < d.N) d.out[(size_t)(off + i_) * d.N + n] = f2h(v);
      });
    dbuf ^= 1;
  };
  // three stages per sub-group: with NWd of the NW waves busy, as many tile
  // loads in flight per compute unit as the down launch's two stages over
  // its six three-wave work-groups
  Stage<NCHD, G> da, db, dc;
  if (any) {
    dstage(da, 0);
    dstage(db, 1);
    dstage(dc, 2);
  }
  // every unit of the range ready (one thread waits; the barrier passes it on)
  if (tid == 0 && d0 < d1) {
    const uint32_t* rw = fa.ready + (size_t)(blockIdx.x & 7) * kDoneStride;
    for (int u = d0 / Td; u <= (d1 - 1) / Td; ++u)
      for (int spin = 0; __hip_atomic_load(rw + (size_t)u * 8 * kDoneStride, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) != fa.epoch;
           ++spin) {
        if (spin > kWaitSpins) {
          __hip_atomic_store(fa.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    // acquire: this compute unit's and this XCD's caches hold no line of the
    // activations from before (they were written through to memory with
    // device-scope stores), so the plain loads below read them fresh
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (any) dload_x(sb / Td);
  for (int i = 0; i < n_iter; i += 3) {
    drun(da, i);
    if (any) {
      if (i + 1 < cnt && (sb + i + 1) / Td != xdu) dload_x((sb + i + 1) / Td);
      dstage(da, i + 3);
    }
    drun(db, i + 1);
    if (any) {
      if (i + 2 < cnt && (sb + i + 2) / Td != xdu) dload_x((sb + i + 2) / Td);
      dstage(db, i + 4);
    }
    drun(dc, i + 2);
    if (any) {
      if (i + 3 < cnt && (sb + i + 3) / Td != xdu) dload_x((sb + i + 3) / Td);
      dstage(dc, i + 5);
    }
  }
}

typedef void (*MoeKernel)(MoeArgs);

template <bool GU, int NCH, int LB, bool NT, bool ONE = false>
static MoeKernel moe_pick_g(int g) {
  switch (g) {
    case 32: return k_moe<NCH, 32, GU, LB, NT, ONE>;
    case 64: return k_moe<NCH, 64, GU, LB, NT, ONE>;
    default: return k_moe<NCH, 128, GU, LB, NT, ONE>;
  }
}
// nt: non-temporal weight loads; one: gate/up of a single stream (both for up
// to 8 waves per tile only)
template <bool GU>
static MoeKernel moe_pick(int nch, int g, int nw, bool nt, bool one) {
  if (nw <= 8) {
    if (nt) return nch == 2 ? moe_pick_g<GU, 2, 512, true>(g) : moe_pick_g<GU, 1, 512, true>(g);
    if (GU && one) return nch == 2 ? moe_pick_g<GU, 2, 512, false, GU>(g) : moe_pick_g<GU, 1, 512, false, GU>(g);
    return nch == 2 ? moe_pick_g<GU, 2, 512, false>(g) : moe_pick_g<GU, 1, 512, false>(g);
  }
  return nch == 2 ? moe_pick_g<GU, 2, 1024, false>(g) : moe_pick_g<GU, 1, 1024, false>(g);
}

// 32-row units (a prompt's products): plain loads, up to 8 waves per tile
template <bool GU, int NCH>
static MoeKernel moe_pick_mt2_g(int g) {
  switch (g) {
    case 32: return k_moe<NCH, 32, GU, 512, false, false, 2>;
    case 64: return k_moe<NCH, 64, GU, 512, false, false, 2>;
    default: return k_moe<NCH, 128, GU, 512, false, false, 2>;
  }
}
template <bool GU>
static MoeKernel moe_pick_mt2(int nch, int g) {
  return nch == 2 ? moe_pick_mt2_g<GU, 2>(g) : moe_pick_mt2_g<GU, 1>(g);
}
// 64-row units (gate/up of a long prompt)
template <bool GU, int NCH>
static MoeKernel moe_pick_mt4_g(int g) {
  switch (g) {
    case 32: return k_moe<NCH, 32, GU, 512, false, false, 4>;
    case 64: return k_moe<NCH, 64, GU, 512, false, false, 4>;
    default: return k_moe<NCH, 128, GU, 512, false, false, 4>;
  }
}
template <bool GU>
static MoeKernel moe_pick_mt4(int nch, int g) {
  return nch == 2 ? moe_pick_mt4_g<GU, 2>(g) : moe_pick_mt4_g<GU, 1>(g);
}

static int cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, c = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 256;
    cus = c;
  }
  return cus;
}

// Grid = the number of work-groups the device keeps resident at once
// (occupancy query, cached per kernel), so the persistent loop covers the
// whole chip in one round.
static int resident_grid(const void* k, int threads, size_t shm) {
  struct Entry {
    const void* k;
    int threads;
    size_t shm;
    int grid;
  };
  static Entry cache[64];
  static int n = 0;
  for (int i = 0; i < n; ++i)
    if (cache[i].k == k && cache[i].threads == threads && cache[i].shm == shm) return cache[i].grid;
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, shm) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  // at most 18 waves per compute unit: more, smaller work-groups were
  // measured slower (down product: 8 three-wave groups per unit 26.6 us,
  // 6 groups 22.2 us)
  per_cu = std::max(1, std::min(per_cu, 18 / (threads / 64)));
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  const int grid = per_cu * cus;
  if (n < 64) cache[n++] = Entry{k, threads, shm, grid};
  return grid;
}

static MoeArgs moe_args(bool gateup, const Mat& m0, const Mat* m1, const uint16_t* x, int ldx, const RouteOut& r,
                        uint16_t* out);

static hipError_t launch_moe_common(bool gateup, const Mat& m0, const Mat* m1, const uint16_t* x, int ldx,
                                    const RouteOut& r, uint16_t* out, bool nt, bool one, hipStream_t st,
                                    bool direct = false) {
  const int nch = nch_for(m0.K);
  const int NW = m0.K / (nch * 128);
  MoeArgs a = moe_args(gateup, m0, m1, x, ldx, r, out);
  if (direct) {
    if (gateup || !r.pair_flat) return hipErrorInvalidValue;
    a.dst_rows = r.pair_flat;
  }
  const int MT = r.unit_n / 16;
  if (r.unit_n != 16 && ((r.unit_n != 32 && !(r.unit_n == 64 && gateup)) || nt || one || direct || NW > 8))
    return hipErrorInvalidValue;
  // 64-row units list their rows through the first list's (and only they do)
  if ((r.unit_n == 64) != (r.rows_via_rec != 0)) return hipErrorInvalidValue;
  // the unit rows: as bytes (non-temporal gate/up) or as words (the other forms)
  if (gateup && !one && !(nt && a.rows8_ok) && !r.unit_rows) return hipErrorInvalidValue;
  MoeKernel k = MT == 4   ? moe_pick_mt4<true>(nch, m0.g)
                : MT == 2 ? (gateup ? moe_pick_mt2<true>(nch, m0.g) : moe_pick_mt2<false>(nch, m0.g))
                : gateup ? moe_pick<true>(nch, m0.g, NW, nt, one)
                         : moe_pick<false>(nch, m0.g, NW, nt, false);
  if (r.units_cap < 1 || r.units_cap > kMaxUnitsPrefill) return hipErrorInvalidValue;
  // the records of every unit in LDS (at most kMaxUnits in a decode step, whose
  // launch shape is kept; a prefill can have more)
  // (non-temporal gate/up: then the unit rows as bytes)
  const size_t shm = 2 * (size_t)(gateup ? 2 : 1) * NW * MT * 1024 + (size_t)std::max(r.units_cap, kMaxUnits) * 16 +
                     (gateup && nt ? (size_t)kMaxUnits * 16 : 0);
  const int grid = resident_grid(reinterpret_cast<const void*>(k), NW * 64, shm);
  w4_launch(k, dim3(grid), dim3(NW * 64), (uint32_t)shm, st, a);
  return hipGetLastError();
}

static MoeArgs moe_args(bool gateup, const Mat& m0, const Mat* m1, const uint16_t* x, int ldx, const RouteOut& r,
                        uint16_t* out) {
  MoeArgs a;
  a.t0 = m0.tiles;
  a.t1 = m1 ? m1->tiles : nullptr;
  a.s0 = m0.scales;
  a.s1 = m1 ? m1->scales : nullptr;
  a.N = m0.N;
  a.K = m0.K;
  a.ntiles = m0.ntiles();
  a.tile_stride = (size_t)m0.Np() / 16 * (m0.K / 128) * 64;
  a.scale_stride = (size_t)m0.Np() * (m0.K / m0.g);
  a.x = x;
  a.ldx = ldx;
  a.units = r.units;
  a.unit_rows = r.unit_rows;
  // the byte rows fit the LDS area of a decode step's unit count only
  a.rows8_ok = r.unit_rows8 != nullptr && r.units_cap <= kMaxUnits;
  a.rows8 = a.rows8_ok ? r.unit_rows8 : reinterpret_cast<const uint4*>(r.unit_rows);
  a.n_units = r.n_units;
  a.units_cap = r.units_cap;
  a.out = out;
  a.dst_rows = nullptr;
  a.ncu = cu_count();
  // measured (gate/up share, with an odd range's last item run alone):
  // 40 against 0, 75 and 110: +0.3% tok/s at B = 4, 8 and 32; gate/up 120
  // with the down product at 60 (its first work-group per compute unit also
  // ends earlier): about 1% fewer
  a.dshare = gateup ? 40 : 0;
  return a;
}

typedef void (*MoeFusedKernel)(MoeFusedArgs);
template <int NCH, int NCHD>
static MoeFusedKernel fused_pick_g(int g) {
  switch (g) {
    case 32: return k_moe_fused<NCH, NCHD, 32, 512>;
    case 64: return k_moe_fused<NCH, NCHD, 64, 512>;
    default: return k_moe_fused<NCH, NCHD, 128, 512>;
  }
}

bool moe_fused_ok(const Mat& gate0, const Mat& down0) {
  const int nch = nch_for(gate0.K), NW = gate0.K / (nch * 128);
  const int nchd = nch_for(down0.K), NWd = down0.K / (nchd * 128);
  return NW <= 8 && NWd <= NW && gate0.g == down0.g;
}

hipError_t launch_moe_fused(const Mat& gate0, const Mat& up0, const Mat& down0, const uint16_t* x, int ldx,
                            const RouteOut& r, uint16_t* act, uint16_t* y, uint32_t* ready, uint32_t epoch,
                            int32_t* err, hipStream_t st) {
  if (!moe_fused_ok(gate0, down0) || !r.done || !ready || !err || epoch == 0 || r.unit_n != 16)
    return hipErrorInvalidValue;
  if (r.units_cap < 1 || r.units_cap > kMaxUnitsPrefill) return hipErrorInvalidValue;
  const int nch = nch_for(gate0.K), NW = gate0.K / (nch * 128);
  const int nchd = nch_for(down0.K);
  MoeFusedArgs fa;
  fa.gu = moe_args(true, gate0, &up0, x, ldx, r, act);
  fa.dn = moe_args(false, down0, nullptr, act, down0.K, r, y);
  fa.done = r.done;
  fa.ready = ready;
  fa.epoch = epoch;
  fa.err = err;
  MoeFusedKernel k = nch == 2 ? (nchd == 2 ? fused_pick_g<2, 2>(gate0.g) : fused_pick_g<2, 1>(gate0.g))
                              : (nchd == 2 ? fused_pick_g<1, 2>(gate0.g) : fused_pick_g<1, 1>(gate0.g));
  const size_t shm = 2 * (size_t)2 * NW * 1024 + (size_t)std::max(r.units_cap, kMaxUnits) * 16;
  const int grid = resident_grid(reinterpret_cast<const void*>(k), NW * 64, shm);
  w4_launch(k, dim3(grid), dim3(NW * 64), (uint32_t)shm, st, fa);
  return hipGetLastError();
}

template <bool NTV>
static void launch_resid_split_nt(const Mat& w, int MT, const DenseArgs& a, float* part, unsigned* ticket,
                                  hipStream_t st) {
  const dim3 grid(2 * w.ntiles());
  const uint32_t shm = 8 * MT * 1024;
  switch (w.g) {
    case 32:
      MT == 2 ? w4_launch(k_gemm_resid_split<2, 32, NTV>, grid, dim3(512), shm, st, a, part, ticket)
              : w4_launch(k_gemm_resid_split<1, 32, NTV>, grid, dim3(512), shm, st, a, part, ticket);
      break;
    case 64:
      MT == 2 ? w4_launch(k_gemm_resid_split<2, 64, NTV>, grid, dim3(512), shm, st, a, part, ticket)
              : w4_launch(k_gemm_resid_split<1, 64, NTV>, grid, dim3(512), shm, st, a, part, ticket);
      break;
    default:
      MT == 2 ? w4_launch(k_gemm_resid_split<2, 128, NTV>, grid, dim3(512), shm, st, a, part, ticket)
              : w4_launch(k_gemm_resid_split<1, 128, NTV>, grid, dim3(512), shm, st, a, part, ticket);
      break;
  }
}

hipError_t launch_gemm_resid_split(const Mat& w, int B, const uint16_t* xp, int xrows, uint16_t* h, int ldh,
                                  float* part, unsigned* ticket, hipStream_t st, bool nt) {
  if (w.K != 16 * 256 || w.ntiles() > kSplitMaxTiles || xrows < 1 || !part || !ticket) return hipErrorInvalidValue;
  const int MT = B > 16 ? 2 : 1;
  DenseArgs a{w.tiles, w.scales, w.N, w.K, w.ntiles(), xp, 0, B, h, ldh, xrows};
  if (nt)
    launch_resid_split_nt<true>(w, MT, a, part, ticket, st);
  else
    launch_resid_split_nt<false>(w, MT, a, part, ticket, st);
  return hipGetLastError();
}

hipError_t launch_moe_gateup(const Mat& gate0, const Mat& up0, const uint16_t* x, int ldx, const RouteOut& r,
                             uint16_t* act, hipStream_t st, bool nt, bool one) {
  return launch_moe_common(true, gate0, &up0, x, ldx, r, act, nt, one, st);
}

hipError_t launch_moe_down(const Mat& down0, const uint16_t* act, const RouteOut& r, uint16_t* y, hipStream_t st,
                           bool nt, bool direct) {
  return launch_moe_common(false, down0, nullptr, act, down0.K, r, y, nt, false, st, direct);
}

}  // namespace w4
