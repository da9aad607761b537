// Internal declarations shared by the gfx950 kernels and the host side of
// the w4moe library.  Nothing here is part of the public C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "w4moe.h"

namespace w4 {

// ---------------------------------------------------------------------------
// Repacked bank layout of one int4 tensor W[N][K] (N padded to Np = 16*ceil(N/16)).
//
// tiles: [Np/16][K/128][64 lanes][16 bytes].  Lane L of tile (t, c) holds, for
// MFMA k-steps s = 0..3, one dword with the 8 codes of row n = 16t + L%16,
// columns k = 128c + 32s + 8(L/16) + j, j = 0..7, as offset-binary nibbles
// (code + 8): nibble j holds element 2j and nibble j+4 holds element 2j+1, so
// ((w >> 4j) & 0x000F000F) | 0x64006400 is the fp16 pair (1024 + u_2j, 1024 +
// u_2j+1).  Pad rows hold code 0.  A wave reads a (16 x 128) block as one
// fully coalesced 1 KiB load.
// scales: [Np][K/g] fp16, pad rows zero.
// ---------------------------------------------------------------------------
struct Mat {
  const uint4* tiles;
  const uint16_t* scales;
  int N, K, g;
  int Np() const { return (N + 15) / 16 * 16; }
  int ntiles() const { return (N + 15) / 16; }
};

enum Epi { EPI_F16 = 0, EPI_F32 = 1, EPI_RESID = 2 };

// Activation panel: element (row b, column k) of a [rows][K] fp16 activation
// at ((k / 8) * rows + b) * 8 + k % 8, rows = max streams rounded up to 16.
// The dense products read their input from a panel in the decode step (every
// MFMA operand load then reads 64 contiguous bytes per 4-lane group); the
// per-stage entry points keep row-major activations (rows = 0 below).
inline int panel_rows(int max_streams) { return (max_streams + 15) / 16 * 16; }

// ---- launchers (kernels in *.hip); all return hipGetLastError() ----
hipError_t launch_repack(const uint8_t* src_packed, const uint16_t* src_scales, int count, int N, int K,
                         int g, uint4* dst_tiles, uint16_t* dst_scales, hipStream_t st);
// xrows > 0: x is a panel with xrows rows (ldx unused); else row-major with stride ldx.
// nt (panel products only): non-temporal weight loads (same results).
hipError_t launch_gemm(const Mat& w, int B, const uint16_t* x, int ldx, void* y, int ldy, int epi,
                       hipStream_t st, int xrows = 0, bool nt = false);

// Routing limits: experts, and 16-row units of the grouped products (used
// experts + B*k/16 with B <= 32, k <= 16).
constexpr int kRouteMaxE = 256;
constexpr int kMaxUnits = kRouteMaxE + 32 * 16 / 16 + 1;
// Prefill: at most kPrefillMaxPairs (prompt tokens x top_k) routed pairs.
constexpr int kPrefillMaxPairs = 16384;
constexpr int kMaxUnitsPrefill = kRouteMaxE + kPrefillMaxPairs / 16 + 1;

struct RouteOut {
  int32_t* ids;          // [B][k]
  float* w;              // [B][k]
  int32_t* counts;       // [E]
  int32_t* offsets;      // [E+1]
  int32_t* pair_stream;  // [B*k]
  int32_t* pair_rank;    // [B*k]
  int32_t* inv;          // [B][k] position of pair (b, r) in expert order
  int32_t* used;         // [E] used experts, ascending
  int32_t* n_used;       // [1]
  int4* units;           // [E + B*k/16 + 1] per 16-row unit of each used expert: (expert, first pair, rows, 0)
  int32_t* unit_rows;    // [same][16] stream of each unit row (rows past the count repeat row 0), or null
  int32_t* n_units;      // [1]
  int units_cap;         // records allocated in units (>= any n_units)
  int unit_n = 16;       // rows per unit: 16, or 32 for a prompt's products (prompt routing only)
  // prompt routing only: a second unit list of unit_n2 (64) rows per unit over the same pair order, for
  // the gate/up product, each unit the run of two consecutive 32-row units of the first list (record
  // field w: the first of them); null: none
  int4* units2 = nullptr;
  int32_t* n_units2 = nullptr;
  int unit_n2 = 0;
  int units_cap2 = 0;
  // the units' row streams are unit_rows[units[u].w * 32 + i] (the first list's, 32 rows per unit)
  // instead of unit_rows[u * unit_n + i]
  int rows_via_rec = 0;
  uint4* unit_rows8 = nullptr;  // [units_cap] or null: byte i of record u = unit_rows[u][i] (B <= 32)
  int32_t* pair_flat = nullptr;  // [B*k] or null: b*k + r of each pair, in expert order (the inverse of inv)
  uint32_t* done = nullptr;  // [units_cap] x kDoneStride words or null: zeroed for every unit written
                             // (fused expert products)
};
// Routing in one work-group: top-k softmax of fp32 logits [B][E], bucketing and 16-row units.  B <= 32.
hipError_t launch_route(const float* logits, int B, int E, int k, const RouteOut& o, hipStream_t st);

// Spare work-groups for touching a span of that many bytes with threads-wide
// work-groups: about one per compute unit, each touching at most one line
// per thread.
int touch_groups(size_t bytes, int threads);

// h += x * W^T (fp16 residual epilogue) for K = 4096 with the K slices split
// over two work-groups per tile (bit-identical to launch_gemm's EPI_RESID);
// xp an activation panel with xrows rows; part [ntiles][2][512] fp32 and
// ticket [ntiles] (zero before and after) are scratch.  ntiles <= kSplitMaxTiles.
constexpr int kSplitMaxTiles = 256;
hipError_t launch_gemm_resid_split(const Mat& w, int B, const uint16_t* xp, int xrows, uint16_t* h, int ldh,
                                  float* part, unsigned* ticket, hipStream_t st, bool nt = false);

// Grouped expert GEMMs over the bucketed pairs (persistent, work list from
// route).  nt: non-temporal weight loads (same results; measured faster for a
// decode batch above 8 rows, slower below it and in a prefill, which reads
// each expert's tiles once per 16-row unit).
// one: x holds a single stream's row (every unit's rows are row 0).
hipError_t launch_moe_gateup(const Mat& gate0, const Mat& up0, const uint16_t* x, int ldx, const RouteOut& r,
                             uint16_t* act, hipStream_t st, bool nt = false, bool one = false);
// direct: output row of pair p at y[r.pair_flat[p]] (the (stream, rank) order
// the combine reads without an index), else at y[p].
hipError_t launch_moe_down(const Mat& down0, const uint16_t* act, const RouteOut& r, uint16_t* y, hipStream_t st,
                           bool nt = false, bool direct = false);
// The large-M product of a prompt's rows (k_gemm_lm: 128 x 128 blocks, both
// operands streamed through LDS by direct-to-LDS loads): x row-major [M][ldx]
// (16-byte aligned, ldx a multiple of 8), epilogues as launch_gemm.  fp32 sums
// of the same terms as launch_gemm, in group order over K (launch_gemm adds
// per-slice sums), so the rounding may differ from it.  lm_ok: the
// geometries it takes.
bool lm_ok(const Mat& w, int ldx);
hipError_t launch_gemm_lm(const Mat& w, int M, const uint16_t* x, int ldx, void* y, int ldy, int epi,
                          hipStream_t st);
// Both grouped products in one launch (same results bit for bit); needs
// r.done, the ready words ([units_cap][8] x kDoneStride, zeroed once, then
// only written with epochs), a nonzero epoch larger than any earlier one on
// them, and a host-visible error word.  moe_fused_ok: the geometries it takes.
constexpr int kDoneStride = 64;  // words between counters (256 bytes)
bool moe_fused_ok(const Mat& gate0, const Mat& down0);
hipError_t launch_moe_fused(const Mat& gate0, const Mat& up0, const Mat& down0, const uint16_t* x, int ldx,
                            const RouteOut& r, uint16_t* act, uint16_t* y, uint32_t* ready, uint32_t epoch,
                            int32_t* err, hipStream_t st);
// h[b] = fp16(h[b] + fp16(sum_r w[b][r] * y[inv[b][r]]))  (resid), or out = fp16(sum ...) (no resid);
// then optionally xn[b] = RMSNorm(h[b]) * gamma.  direct: y is in (stream, rank)
// order, y[b*k + r] (inv unused).  Same results either way.
// Normalised outputs (xn, out) go to a panel with that many rows when
// xn_rows > 0, else row-major [B][H].
hipError_t launch_combine(int B, int H, int k, const float* w, const int32_t* inv, const uint16_t* y,
                          uint16_t* h, bool resid, const uint16_t* gamma, float eps, uint16_t* xn,
                          hipStream_t st, int xn_rows = 0, bool direct = false);
hipError_t launch_rmsnorm(int B, int H, const uint16_t* x, const uint16_t* gamma, float eps, uint16_t* out,
                          hipStream_t st, int out_rows = 0);
// bad [B]: 1 where the token id is outside [0, V) (that row is zero), else 0.
hipError_t launch_embed(int B, int H, int V, int g, const int32_t* tokens, const uint8_t* emb_p,
                        const uint16_t* emb_s, uint16_t* h, const uint16_t* gamma, float eps, uint16_t* xn,
                        int32_t* bad, hipStream_t st, int xn_rows = 0);
// next[b] = argmax of logits row b (ties to the lower index); part_v/part_i
// [B][8] hold the split partials, ticket [B] is zero before and after.
hipError_t launch_argmax(int B, int V, const uint16_t* logits, int32_t* next, float* part_v, int32_t* part_i,
                         unsigned* ticket, hipStream_t st);
// Next token by temperature / top-k / top-p sampling (w4_glue.hip): params
// [B][kSampleParams] = (temperature bits, top_k, top_p bits, seed low, seed
// high) per row, pos [B] the row's position (the draw's counter).
constexpr int kSampleMaxK = 64;
constexpr int kSampleParams = 5;
hipError_t launch_sample(int B, int V, const uint16_t* logits, const int32_t* params, const int32_t* pos,
                         int32_t* next, hipStream_t st);

struct KV {
  uint16_t* K;   // [L][S][Hkv][cap/64][64*D], MFMA operand order (w4_attn.hip)
  uint16_t* VT;  // [L][S][Hkv][cap/64][64*D], MFMA operand order (w4_attn.hip)
  int S, Hkv, cap, D;
};
// MoE front end of a decode layer in one launch (one work-group per row and
// 16-expert tile, B <= 32): xn = RMSNorm(h) * gamma, the router product, top-k
// softmax and the bucketing.  lg [B][E]: the logits exchanged between a row's
// work-groups; rticket [B] and ticket: counters, zero before and after.
// pf, pf_bytes: a span of the bank touched by spare work-groups of the launch
// (touch_lines below); null for none.  kv_next (with slot, pos as in the
// attention): that KV's live chunks of layer kv_layer are touched too.
hipError_t launch_router(int B, int H, int E, int k, int g, const uint16_t* h, const uint16_t* gamma, float eps,
                         uint16_t* xn, const uint4* tiles, const uint16_t* scales, const RouteOut& o,
                         unsigned* ticket, float* lg, unsigned* rticket, hipStream_t st, const void* pf = nullptr,
                         size_t pf_bytes = 0, const KV* kv_next = nullptr, int kv_layer = 0,
                         const int32_t* slot = nullptr, const int32_t* pos = nullptr);
hipError_t launch_rope_table(int cap, int D, double theta, float2* table, hipStream_t st);
hipError_t launch_seed(int L, int P, int slot, const KV& kv, const uint16_t* k, const uint16_t* v,
                       hipStream_t st);
// Prefill of one layer's K/V: row i of k, v (row stride ld, [Hkv][D]) is the
// prompt's position i; keys rotated at i through table (as the decode step's
// append), both written at (layer, slot, i) for i < P.
hipError_t launch_prefill_kv(int P, int layer, int slot, const KV& kv, const uint16_t* k, const uint16_t* v, int ld,
                             const float2* table, hipStream_t st);
// Routing of P prefill rows (P * k <= kPrefillMaxPairs, E <= kRouteMaxE), two
// launches: top-k softmax per row (one wave each) and the (row, expert)
// bucketing into the same outputs as launch_route (units_cap = E + P*k/16 + 1).
// mask [E][ceil(P/32)] words (zero before, left set) and e8 [P*k] bytes are
// scratch; mask_next, a second buffer of that size (the next call's mask), is
// zeroed by the call.
hipError_t launch_route_prefill(const float* logits, int P, int E, int k, const RouteOut& o, uint32_t* mask,
                                uint32_t* mask_next, uint8_t* e8, hipStream_t st);
// Work-groups of the prefill bucketing (sharing the pairs' stores).
constexpr int kBucketPrefillGroups = 16;
// Dynamic LDS bytes of the prefill bucketing (row masks and their prefix
// counts; at most 60 KiB is allowed, beside its static arrays).
inline size_t route_prefill_lds(int P, int E, int k) {
  (void)k;
  return (size_t)E * ((P + 31) / 32) * 6;
}
// Causal attention of a prompt's P rows (q of row i, head h at qkv + i * ldq
// + h * D, rotated here through table) over positions 0..P-1 of the slot's
// K/V of the layer (already written), one pass over the keys per 64-row
// query block; o row-major [P][ldo].
hipError_t launch_prefill_attention(int P, int layer, int slot, int Hq, const KV& kv, const uint16_t* qkv, int ldq,
                                    const float2* table, uint16_t* o, int ldo, hipStream_t st);
// positions 0..P-1 of a slot -> canonical k, v [L][P][Hkv][D]
hipError_t launch_read_kv(int L, int P, int slot, const KV& kv, uint16_t* k, uint16_t* v, hipStream_t st);
// Split-KV decode attention in one launch.  A stream at position p has
// attn_splits(p) splits of 256 positions; splits [2 * nsplits] lists one
// 8-byte entry (b << 16 | split << 8 | kv head, slot << 16 | p) for every
// split of every row and kv head (built on the host with the rows, 8-byte
// aligned), one work-group each.  part_o [B][Hq][nsmax][D] f32, part_ml
// [B][Hq][nsmax][2]; prof: when non-null, the launch is timed (prof_arm).
// A list of 256 or more entries streams the K/V with non-temporal loads
// (each chunk is read once per step).  The
// last work-group of each (stream, kv head) combines the splits; ticket
// [B][Hkv] is zero before and after.  This step's q (row stride ldq) and k,
// v (row stride ldkv) are rotated at each stream's position through table
// when it is not null; k and v are appended to the arena at the position.
// o: [B][Hq*D] row-major, or an activation panel with o_rows rows.
constexpr int kAttnSplitChunks = 4;  // 64-position chunks per split = waves per attention work-group
__host__ __device__ inline int attn_splits(int pos) {
  return (pos / 64 + kAttnSplitChunks) / kAttnSplitChunks;
}
hipError_t launch_attention(int B, int layer, int Hq, const KV& kv, const int32_t* splits, int nsplits, const uint16_t* q, int ldq, const uint16_t* knew,
                            const uint16_t* vnew, int ldkv, const float2* table, float* part_o, float* part_ml,
                            unsigned* ticket, uint16_t* o, hipStream_t st, void* prof = nullptr, int o_rows = 0);
// Kernel timing: the host arms a (start, stop) event pair for the next
// launch of the profiled kernel family (prof_arm, from the context's pool);
// that launch records them with its own dispatch (hipExtLaunchKernelGGL), so
// the elapsed time is the kernel's alone, without the gap before it.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_ev;
void prof_arm(void* ctx);
template <typename F, typename... Args>
inline void w4_launch(F kernel, const dim3& grid, const dim3& block, uint32_t shm, hipStream_t st, Args... args) {
  if (g_launch_ev.start) {
    const LaunchEvents e = g_launch_ev;
    g_launch_ev = LaunchEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, shm, st, e.start, e.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shm, st, args...);
  }
}

// Touch line j + nj*t (128 bytes each) of a span, t = the thread, so that the
// memory-side cache holds the span for a launch that reads it soon after.
// Run by spare work-groups of a launch that leaves most compute units idle:
// one compute unit fetches only a small share of the chip's bandwidth, so
// the span is spread over many work-groups.
__device__ __forceinline__ void touch_lines(const uint8_t* span, size_t lines, size_t j, size_t nj) {
  const size_t li = j + nj * threadIdx.x;
  if (li < lines) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(span + (li << 7));
    asm volatile("" ::"v"(v));
  }
}
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t st);
// Device-wide barrier probe and its empty-launch reference (diagnostic).
constexpr size_t kSyncProbeWords = 64 * 9;
int sync_probe_max_grid();
hipError_t launch_sync_probe(int mode, int grid, int n, uint32_t* ctr, hipStream_t st);
// Message of the last failed context-free entry point on this thread.
extern thread_local std::string g_free_err;
// Streaming-read probe (diagnostic): src[bytes] read once with 16-byte loads; sink [grid] words.
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, bool nt, hipStream_t st);

}  // namespace w4
