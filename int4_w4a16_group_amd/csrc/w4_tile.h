// Device building blocks of the W4A16 products on gfx950 MFMA, shared by the
// dense and grouped-expert kernels (w4_gemm.hip) and the fused output
// projection + router launch (w4_glue.hip): per-wave activation slices,
// weight stages, the tile multiply-accumulate and the in-order slice sum.
#pragma once

#include "w4_device.h"

namespace w4 {

// ------------------------------------------------------------------ core
// x slice of one wave in registers: xa[mt][ks] is the A operand of k-step ks
// for rows 16mt + lane%16.
template <int MT, int NKS>
struct XRegs {
  h8 a[MT][NKS];
};

// Multiply-accumulate one 16-column tile over the wave's slice.
// wv: the slice's repacked chunks; sv: its scales (one per group, column
// n = 16t + lane%16); acc[mt] += over groups fma(scale, MFMA chain).
template <int MT, int NCH, int G>
__device__ __forceinline__ void tile_mac(const XRegs<MT, NCH * 4>& x, const uint4 (&wv)[NCH],
                                         const float (&sv)[NCH * 128 / G], f4 (&acc)[MT], const DqConst& dk) {
  constexpr int SPG = G / 32;
  f4 part[MT];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t wd[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ks = c * 4 + s;
      const h8 b = dq8(wd[s], dk);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (ks % SPG == 0) part[mt] = f4{0.f, 0.f, 0.f, 0.f};
        part[mt] = mfma16x16x32(x.a[mt][ks], b, part[mt]);
      }
      if ((ks + 1) % SPG == 0) {
        const float sc = sv[ks / SPG];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][0] = fmaf(sc, part[mt][0], acc[mt][0]);
          acc[mt][1] = fmaf(sc, part[mt][1], acc[mt][1]);
          acc[mt][2] = fmaf(sc, part[mt][2], acc[mt][2]);
          acc[mt][3] = fmaf(sc, part[mt][3], acc[mt][3]);
        }
      }
    }
  }
}

// NT: non-temporal loads (faster for a bandwidth-bound stream read once,
// slower for a latency-bound launch; the data are the same either way).
template <int NCH, bool NT = false>
__device__ __forceinline__ void load_tile(const uint4* __restrict__ tiles, int K, int t, int w, int lane,
                                          uint4 (&wv)[NCH]) {
  const uint4* p = tiles + ((size_t)t * (K / 128) + (size_t)w * NCH) * 64 + lane;
#pragma unroll
  for (int c = 0; c < NCH; ++c) wv[c] = NT ? ld_nt(p + c * 64) : p[c * 64];
}

template <int NCH, int G>
__device__ __forceinline__ void load_scales(const uint16_t* __restrict__ scales, int K, int t, int w, int lane,
                                            float (&sv)[NCH * 128 / G]) {
  const uint16_t* p = scales + (size_t)(t * 16 + (lane & 15)) * (K / G) + (size_t)w * (NCH * 128 / G);
#pragma unroll
  for (int i = 0; i < NCH * 128 / G; ++i) sv[i] = h2f(p[i]);
}

// One pipeline stage: a tile's weight chunks and raw scale bits for this wave's
// K slice (scales kept as the loaded dwords, two fp16 per dword, and only
// unpacked when the stage is used), so the loads stay in flight while the
// other stage is computed.
template <int NCH, int G, bool NT = false>
struct Stage {
  static constexpr int NS = NCH * 128 / G;       // scales per lane per tile
  static constexpr int ND = NS >= 2 ? NS / 2 : 1;  // dwords holding them
  uint4 w[NCH];
  uint32_t s[ND];
  __device__ __forceinline__ void load(const uint4* __restrict__ tiles, const uint16_t* __restrict__ scales, int K,
                                       int t, int wv, int lane) {
    load_tile<NCH, NT>(tiles, K, t, wv, lane, w);
    const uint16_t* p = scales + (size_t)(t * 16 + (lane & 15)) * (K / G) + (size_t)wv * NS;
    if (NS >= 2) {
#pragma unroll
      for (int i = 0; i < ND; ++i)
        s[i] = NT ? ld_u32_nt(reinterpret_cast<const uint32_t*>(p) + i) : reinterpret_cast<const uint32_t*>(p)[i];
    } else {
      s[0] = NT ? ld_u16_nt(p) : p[0];
    }
  }
  __device__ __forceinline__ void scales_f32(float (&sv)[NS]) const {
#pragma unroll
    for (int i = 0; i < NS; ++i) sv[i] = h2f((uint16_t)(s[i / 2] >> (16 * (i & 1))));
  }
};

// A-operand rows: row i of the tile reads rowptr(i) (nullptr = zero row).
template <int MT, int NCH, class RowPtr>
__device__ __forceinline__ void load_x(XRegs<MT, NCH * 4>& x, RowPtr rowptr, int kbase, int lane) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint16_t* p = rowptr(mt * 16 + (lane & 15));
#pragma unroll
    for (int ks = 0; ks < NCH * 4; ++ks)
      x.a[mt][ks] = p ? ld_h8(p + kbase + ks * 32 + 8 * (lane >> 4)) : h8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// A-operand rows from an activation panel: element (row b, column k) of a
// [rows][K] activation at ((k / 8) * rows + b) * 8 + k % 8, so the 4-lane
// groups of every operand load read 64 contiguous bytes (rows is a multiple
// of 16).  Tile rows past the batch read row B-1 again: lanes that share an
// address cost the load unit one access, and those rows only reach output
// rows that are never stored (an MFMA output row depends on its own A row).
template <int MT, int NCH>
__device__ __forceinline__ void load_x_panel(XRegs<MT, NCH * 4>& x, const uint16_t* __restrict__ xp, int rows,
                                             int B, int kbase, int lane) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = min(16 * mt + (lane & 15), B - 1);
#pragma unroll
    for (int ks = 0; ks < NCH * 4; ++ks)
      x.a[mt][ks] = ld_h8(xp + ((size_t)((kbase >> 3) + 4 * ks + (lane >> 4)) * rows + row) * 8);
  }
}

// Index in a [.][MT][64 lanes][4] partial tile of output o = (mt, row i,
// column j) of the tile (the MFMA result layout: lane (i/4)*16 + j, element i%4).
__device__ __forceinline__ int tile_out_idx(int o) {
  const int mt = o >> 8, i = (o >> 4) & 15, j = o & 15;
  return mt * 256 + ((i >> 2) * 16 + j) * 4 + (i & 3);
}

// Sum of the K-slice partials w0 .. w1-1 (< w0 + 8) of one output, in slice
// order; p: the partials of slices w0 .. w0+7 (entries past w1 not added).
__device__ __forceinline__ float run_sum(const float (&p)[8], int n) {
  float v = p[0];
#pragma unroll
  for (int w = 1; w < 8; ++w) v = w < n ? v + p[w] : v;
  return v;
}

// Sum the waves' partial tiles (red: [NW][MT][64 lanes][4], NW <= NWMAX <=
// 16) and hand each output (row, col-in-tile, value) to epi.  Order of the
// sum, a function of the slice count only: slices in order in runs of eight,
// then the run sums in order -- ((p0 + ... + p7) + (p8 + ... + p15)) for 16
// slices, one plain in-order chain for up to 8.  (The split output projection
// computes each run in its own work-group and adds the two run sums the same
// way.)  Consecutive threads take consecutive columns.  All NWMAX reads are
// issued before the sums; slots w >= NW re-read the last slice and are not
// added (selects, no branch, so the reads are never held back).
// reduce_tile_sub: the same sums by the nt threads tid = 0 .. nt-1 of a
// sub-group of the work-group.
template <int MT, int NWMAX, class EpiF>
__device__ __forceinline__ void reduce_tile_sub(const float* red, int NW, int tid, int nt, EpiF epi) {
  static_assert(NWMAX >= 1 && NWMAX <= 16, "at most 16 slices");
  for (int o = tid; o < MT * 256; o += nt) {
    const int idx = tile_out_idx(o);
    float p[NWMAX];
#pragma unroll
    for (int w = 0; w < NWMAX; ++w) p[w] = red[min(w, NW - 1) * MT * 256 + idx];
    float v = p[0];
#pragma unroll
    for (int w = 1; w < (NWMAX < 8 ? NWMAX : 8); ++w) v = w < NW ? v + p[w] : v;
    if constexpr (NWMAX > 8) {
      float u = p[8];
#pragma unroll
      for (int w = 9; w < NWMAX; ++w) u = w < NW ? u + p[w] : u;
      v = NW > 8 ? v + u : v;
    }
    epi(((o >> 8) << 4) + ((o >> 4) & 15), o & 15, v);
  }
}
template <int MT, int NWMAX, class EpiF>
__device__ __forceinline__ void reduce_tile(const float* red, int NW, EpiF epi) {
  reduce_tile_sub<MT, NWMAX>(red, NW, (int)threadIdx.x, (int)blockDim.x, epi);
}

}  // namespace w4
