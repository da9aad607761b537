// Host side of the w4moe C ABI: geometry checks, bank and workspace layout,
// the slot table (stable per-stream KV slots with seed-once / logical-reset
// lifecycle, admission against the context cap), and the enqueue order of
// one decode step.  The library owns host state only; all device memory is
// the caller's.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "w4_internal.h"

using namespace w4;

namespace {

constexpr size_t kAlign = 256;
constexpr int kRing = 8;
constexpr int kMaxStreams = 32;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Loc {  // one int4 tensor in the bank (expert 0 for expert tensors)
  size_t tiles = 0, scales = 0;
  int N = 0, K = 0;
  size_t tile_bytes() const { return (size_t)((N + 15) / 16 * 16) * K / 2; }
};

struct LayerLoc {
  size_t attn_norm = 0, moe_norm = 0;
  Loc qkv, o, router, gate, up, down;
};

struct BankPlan {
  std::vector<LayerLoc> layers;
  size_t emb_p = 0, emb_s = 0, final_norm = 0;
  Loc lm;
  size_t total = 0;
};

struct WsPlan {
  size_t h, xn, xp, qkv, attn_o, part_o, part_ml, aticket, amax_v, amax_i, amax_ticket, rlogits, ticket, rlg, rticket, spart, sticket, ids, w, counts, offsets, pair_stream, pair_rank, inv,
      used, n_used, units, unit_rows, unit_rows8, pair_flat, n_units, done, ready, act, y, logits, next, rows,
      table, total;
};

bool geometry_ok(const w4_model_desc* d, std::string* why) {
  auto bad = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (!d) return bad("null model description");
  if (d->n_layers < 1) return bad("n_layers must be >= 1");
  if (d->hidden < 128 || d->hidden % 128 || d->hidden > 4096) return bad("hidden must be a multiple of 128 in [128, 4096]");
  if (d->head_dim != 64 && d->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (d->n_kv_heads < 1 || d->n_q_heads < 1 || d->n_q_heads % d->n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
  if (d->n_q_heads / d->n_kv_heads > 16) return bad("at most 16 query heads per kv head");
  const int qd = d->n_q_heads * d->head_dim;
  if (qd % 128 || qd > 4096) return bad("n_q_heads*head_dim must be a multiple of 128, at most 4096");
  if (d->moe_inter < 128 || d->moe_inter % 128 || d->moe_inter > 4096) return bad("moe_inter must be a multiple of 128 in [128, 4096]");
  // every product's K is cut into at most 16 slices of 256 (128 when K % 256 != 0)
  for (int K : {d->hidden, qd, d->moe_inter})
    if (K % 256 != 0 && K > 2048) return bad("a reduction length that is not a multiple of 256 must be at most 2048");
  if (d->top_k < 1 || d->top_k > 16) return bad("top_k must be in [1, 16]");
  if (d->n_experts < d->top_k || d->n_experts > 256) return bad("n_experts must be in [top_k, 256]");
  if (d->group != 32 && d->group != 64 && d->group != 128) return bad("group must be 32, 64 or 128");
  if (d->vocab < 1) return bad("vocab must be >= 1");
  if (!(d->rms_eps >= 0.f) || !(d->rope_theta > 0.f)) return bad("rms_eps >= 0 and rope_theta > 0 required");
  return true;
}

bool sizes_ok(int32_t max_streams, int32_t cap, std::string* why) {
  if (max_streams < 1 || max_streams > kMaxStreams) {
    if (why) *why = "max_streams must be in [1, 32]";
    return false;
  }
  if (cap < 64 || cap % 64 || cap > 16384) {
    if (why) *why = "ctx_cap must be a multiple of 64 in [64, 16384]";
    return false;
  }
  return true;
}

BankPlan plan_bank(const w4_model_desc& d) {
  BankPlan p;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  auto tensor = [&](int N, int K, int count) {
    Loc l;
    l.N = N;
    l.K = K;
    const size_t Np = (size_t)(N + 15) / 16 * 16;
    l.tiles = take(Np * K / 2 * count);
    l.scales = take(Np * (K / d.group) * 2 * count);
    return l;
  };
  const int H = d.hidden, E = d.n_experts, I = d.moe_inter;
  const int nqkv = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim, qd = d.n_q_heads * d.head_dim;
  p.layers.resize(d.n_layers);
  for (auto& L : p.layers) {
    L.attn_norm = take((size_t)H * 2);
    L.moe_norm = take((size_t)H * 2);
    L.qkv = tensor(nqkv, H, 1);
    L.o = tensor(H, qd, 1);
    L.router = tensor(E, H, 1);
    L.gate = tensor(I, H, E);
    L.up = tensor(I, H, E);
    L.down = tensor(H, I, E);
  }
  p.emb_p = take((size_t)d.vocab * H / 2);
  p.emb_s = take((size_t)d.vocab * (H / d.group) * 2);
  p.final_norm = take((size_t)H * 2);
  p.lm = tensor(d.vocab, H, 1);
  p.total = cur;
  return p;
}

// Words uploaded with each step's rows: slot [Bm], position [Bm], sampling
// parameters [Bm][kSampleParams], then the attention work list (two words
// per entry, at an even word offset so its 8-byte entries align).
size_t split_words_off(int Bm) { return ((2 + (size_t)kSampleParams) * Bm + 1) / 2 * 2; }

size_t row_list_words(const w4_model_desc& d, int Bm, int cap) {
  return split_words_off(Bm) + 2 * (size_t)Bm * attn_splits(cap - 1) * d.n_kv_heads;
}

WsPlan plan_ws(const w4_model_desc& d, int Bm, int cap) {
  WsPlan w;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  const size_t H = d.hidden, E = d.n_experts, k = d.top_k, I = d.moe_inter, Hq = d.n_q_heads, D = d.head_dim;
  const size_t nqkv = (d.n_q_heads + 2 * d.n_kv_heads) * D, nch = cap / 64;
  w.h = take(Bm * H * 2);
  w.xn = take(Bm * H * 2);
  const size_t R = panel_rows(Bm);
  w.xp = take(R * H * 2);
  w.qkv = take(Bm * nqkv * 2);
  w.attn_o = take(R * Hq * D * 2);
  w.part_o = take(Bm * Hq * nch * D * 4);
  w.part_ml = take(Bm * Hq * nch * 2 * 4);
  w.aticket = take(Bm * d.n_kv_heads * 4);
  w.amax_v = take(Bm * 8 * 4);
  w.amax_i = take(Bm * 8 * 4);
  w.amax_ticket = take(Bm * 4);
  w.rlogits = take(Bm * E * 4);
  w.ticket = take(64);
  w.rlg = take(Bm * E * 4);
  w.rticket = take(Bm * 4);
  w.spart = take((size_t)kSplitMaxTiles * 2 * 512 * 4);
  w.sticket = take((size_t)kSplitMaxTiles * 4);
  w.ids = take(Bm * k * 4);
  w.w = take(Bm * k * 4);
  w.counts = take(E * 4);
  w.offsets = take((E + 1) * 4);
  w.pair_stream = take(Bm * k * 4);
  w.pair_rank = take(Bm * k * 4);
  w.inv = take(Bm * k * 4);
  w.used = take(E * 4);
  w.n_used = take(4);
  w.units = take((E + Bm * k / 16 + 1) * 16);
  w.unit_rows = take((E + Bm * k / 16 + 1) * 16 * 4);
  w.unit_rows8 = take((E + Bm * k / 16 + 1) * 16);
  w.pair_flat = take(Bm * k * 4);
  w.n_units = take(4);
  w.done = take((E + Bm * k / 16 + 1) * kDoneStride * 4);
  w.ready = take((E + Bm * k / 16 + 1) * 8 * kDoneStride * 4);
  w.act = take(Bm * k * I * 2);
  w.y = take(Bm * k * H * 2);
  w.logits = take((size_t)Bm * d.vocab * 2);
  w.next = take(Bm * 4);
  // slot ids, positions, sampling parameters, attention work list (every split
  // of every row, per kv head): row_list_words
  w.rows = take(row_list_words(d, Bm, cap) * 4);
  w.table = take((size_t)cap * (D / 2) * 8);
  w.total = cur;
  return w;
}

// Prefill workspace (caller-owned, from w4_prefill_workspace_bytes): the
// prompt's rows through every layer.
struct PfPlan {
  size_t h, xn, qkv, attn_o, lg, ids, w, counts, offsets, inv, used, n_used, units, unit_rows, n_units, units2,
      n_units2, done, ready, act, y, rows, logits, rmask, re8, total;
  size_t row_cap;  // int32 words of the rows region
};

// Words of the prefill upload: slot [P], position [P], sampling parameters.
size_t pf_row_words(const w4_model_desc& d, int P) {
  (void)d;
  return 2 * (size_t)P + kSampleParams;
}

PfPlan plan_prefill(const w4_model_desc& d, int P, int cap) {
  PfPlan w{};
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  const size_t H = d.hidden, E = d.n_experts, k = d.top_k, I = d.moe_inter, Hq = d.n_q_heads, D = d.head_dim;
  const size_t nqkv = (d.n_q_heads + 2 * d.n_kv_heads) * D, pairs = (size_t)P * k;
  const size_t ucap = E + pairs / 16 + 1;
  w.h = take(P * H * 2);
  w.xn = take(P * H * 2);
  w.qkv = take(P * nqkv * 2);
  w.attn_o = take(P * Hq * D * 2);
  w.lg = take(P * E * 4);
  w.ids = take(pairs * 4);
  w.w = take(pairs * 4);
  w.counts = take(E * 4);
  w.offsets = take((E + 1) * 4);
  w.inv = take(pairs * 4);
  w.used = take(E * 4);
  w.n_used = take(4);
  w.units = take(ucap * 16);
  w.unit_rows = take(ucap * 32 * 4);  // 16-row units, or half as many of 32 rows
  w.n_units = take(4);
  // the gate/up product's 64-row units over the same pair order
  w.units2 = take((E + pairs / 64 + 1) * 16);
  w.n_units2 = take(4);
  w.done = take(ucap * kDoneStride * 4);
  w.ready = take(ucap * 8 * kDoneStride * 4);
  w.act = take(pairs * I * 2);
  w.y = take(pairs * H * 2);
  w.row_cap = pf_row_words(d, P);
  w.rows = take(w.row_cap * 4);
  w.logits = take((size_t)d.vocab * 2);
  w.rmask = take(2 * E * (((size_t)P + 31) / 32) * 4);  // two buffers, layers alternating
  w.re8 = take(pairs);
  w.total = cur;
  return w;
}

}  // namespace

struct Sampling {  // per slot; temperature 0 = greedy
  uint64_t seed = 0;
  float temperature = 0.f, top_p = 1.f;
  int32_t top_k = 1;
};

struct w4_ctx {
  w4_model_desc d{};
  int Bm = 0, cap = 0;
  char* arena = nullptr;
  char* bank = nullptr;
  char* ws = nullptr;
  BankPlan bp;
  WsPlan wp{};
  std::vector<int32_t> pos, prompt;
  std::vector<uint8_t> live, need_seed;
  std::vector<Sampling> smp;
  bool any_sampled = false;  // a row of the last upload samples
  bool dev_ready = false, table_ready = false;
  int device = -1;
  int32_t* pinned = nullptr;
  // per ring entry, the step's invalid-token flags [Bm]: host-mapped, coherent
  // memory that the embedding kernel writes through flags_dev (no copy)
  int32_t* flags = nullptr;
  int32_t* flags_dev = nullptr;
  // a device-side wait that ran out of its bound (fused expert products):
  // host-mapped word, nonzero once one did
  int32_t* werr = nullptr;
  int32_t* werr_dev = nullptr;
  bool fused_moe = false;  // W4_OPT_FUSED_MOE
  uint32_t moe_epoch = 0;  // last epoch of a fused expert launch on this context's ready words
  int nsplits = 0;  // attention splits of the rows last uploaded
  // uploaded with each step's rows: slot [Bm], position [Bm], sampling
  // parameters [Bm][kSampleParams], then the attention work list
  size_t split_off() const { return split_words_off(Bm); }
  size_t row_words() const { return row_list_words(d, Bm, cap); }
  const int32_t* dev_rows() { return reinterpret_cast<const int32_t*>(ws + wp.rows); }
  const int32_t* dev_splits() { return dev_rows() + split_off(); }
  hipEvent_t ev[kRing] = {};      // the entry's upload has been read
  hipEvent_t ev_err[kRing] = {};  // the entry's invalid-token flags have arrived
  bool ev_used[kRing] = {};
  bool err_pending[kRing] = {};
  int err_rows[kRing] = {};
  int ring = 0, cur = 0;  // next entry; entry of the last upload
  std::string sticky;     // an invalid token seen in an earlier step, not yet reported
  // prefill uploads: pinned staging (grown on demand), free again once ev_pf has passed
  int32_t* pf_pinned = nullptr;
  size_t pf_words = 0;
  hipEvent_t ev_pf = nullptr;
  bool pf_used = false;
  // the last prefill's invalid-token flags [pf_flag_rows] (host-mapped, written
  // by its embedding kernel), read once ev_pf_done has passed
  int32_t* pf_flags = nullptr;
  int32_t* pf_flags_dev = nullptr;
  int pf_flag_cap = 0, pf_flag_rows = 0;
  hipEvent_t ev_pf_done = nullptr;
  bool pf_pending = false;
  std::string err;
  int launches = 0, syncs = 0;
  int last_launches = 0, last_syncs = 0;
  // kernel timing (w4_profile_begin/end)
  int prof_kernel = 0;
  std::vector<hipEvent_t> prof_ev;  // pool, used in (start, stop) pairs
  size_t prof_used = 0;
  // arm the next launch with the pool's next (start, stop) pair
  void prof_arm() {
    while (prof_ev.size() < prof_used + 2) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return;
      prof_ev.push_back(e);
    }
    g_launch_ev.start = prof_ev[prof_used];
    g_launch_ev.stop = prof_ev[prof_used + 1];
    prof_used += 2;
  }

  template <class T>
  T* W(size_t off) { return reinterpret_cast<T*>(ws + off); }
  template <class T>
  T* Bk(size_t off) { return reinterpret_cast<T*>(bank + off); }
  Mat mat(const Loc& l, int expert = 0) {
    const size_t Np = (size_t)(l.N + 15) / 16 * 16;
    Mat m;
    m.tiles = reinterpret_cast<const uint4*>(bank + l.tiles + (size_t)expert * Np * l.K / 2);
    m.scales = reinterpret_cast<const uint16_t*>(bank + l.scales + (size_t)expert * Np * (l.K / d.group) * 2);
    m.N = l.N;
    m.K = l.K;
    m.g = d.group;
    return m;
  }
  KV kv() {
    KV k;
    const size_t half = (size_t)d.n_layers * Bm * d.n_kv_heads * cap * d.head_dim;
    k.K = reinterpret_cast<uint16_t*>(arena);
    k.VT = reinterpret_cast<uint16_t*>(arena) + half;
    k.S = Bm;
    k.Hkv = d.n_kv_heads;
    k.cap = cap;
    k.D = d.head_dim;
    return k;
  }
  RouteOut route_out(int32_t* ids_user = nullptr) {
    RouteOut r;
    r.ids = ids_user ? ids_user : W<int32_t>(wp.ids);
    r.w = W<float>(wp.w);
    r.counts = W<int32_t>(wp.counts);
    r.offsets = W<int32_t>(wp.offsets);
    r.pair_stream = W<int32_t>(wp.pair_stream);
    r.pair_rank = W<int32_t>(wp.pair_rank);
    r.inv = W<int32_t>(wp.inv);
    r.used = W<int32_t>(wp.used);
    r.n_used = W<int32_t>(wp.n_used);
    r.units = W<int4>(wp.units);
    r.unit_rows = W<int32_t>(wp.unit_rows);
    r.unit_rows8 = W<uint4>(wp.unit_rows8);
    r.pair_flat = W<int32_t>(wp.pair_flat);
    r.n_units = W<int32_t>(wp.n_units);
    r.units_cap = d.n_experts + Bm * d.top_k / 16 + 1;
    r.done = W<uint32_t>(wp.done);
    return r;
  }
};

namespace {

int fail(w4_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  return code;
}

#define HIPCHK(ctx, expr)                                                                           \
  do {                                                                                              \
    hipError_t e_ = (expr);                                                                         \
    if (e_ != hipSuccess) return fail(ctx, W4_E_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

int ensure_device(w4_ctx* c, hipStream_t st) {
  if (!c->dev_ready) {
    int dev = -1;
    HIPCHK(c, hipGetDevice(&dev));
    hipDeviceProp_t prop;
    HIPCHK(c, hipGetDeviceProperties(&prop, dev));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(c, W4_E_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", library built for gfx950");
    HIPCHK(c, hipHostMalloc((void**)&c->pinned, sizeof(int32_t) * c->row_words() * kRing, hipHostMallocDefault));
    HIPCHK(c, hipHostMalloc((void**)&c->flags, sizeof(int32_t) * c->Bm * kRing,
                            hipHostMallocMapped | hipHostMallocCoherent));
    HIPCHK(c, hipHostGetDevicePointer((void**)&c->flags_dev, c->flags, 0));
    HIPCHK(c, hipHostMalloc((void**)&c->werr, 64, hipHostMallocMapped | hipHostMallocCoherent));
    HIPCHK(c, hipHostGetDevicePointer((void**)&c->werr_dev, c->werr, 0));
    *c->werr = 0;
    for (int i = 0; i < kRing; ++i) {
      HIPCHK(c, hipEventCreateWithFlags(&c->ev[i], hipEventDisableTiming));
      HIPCHK(c, hipEventCreateWithFlags(&c->ev_err[i], hipEventDisableTiming));
    }
    c->device = dev;
    c->dev_ready = true;
  }
  if (!c->table_ready) {
    HIPCHK(c, launch_rope_table(c->cap, c->d.head_dim, (double)c->d.rope_theta, c->W<float2>(c->wp.table), st));
    HIPCHK(c, launch_fill_u32(c->W<uint32_t>(c->wp.ticket), 0u, 16, st));
    HIPCHK(c, launch_fill_u32(c->W<uint32_t>(c->wp.aticket), 0u, (size_t)c->Bm * c->d.n_kv_heads, st));
    HIPCHK(c, launch_fill_u32(c->W<uint32_t>(c->wp.amax_ticket), 0u, (size_t)c->Bm, st));
    HIPCHK(c, launch_fill_u32(c->W<uint32_t>(c->wp.rticket), 0u, (size_t)c->Bm, st));
    HIPCHK(c, launch_fill_u32(c->W<uint32_t>(c->wp.sticket), 0u, (size_t)kSplitMaxTiles, st));
    HIPCHK(c, launch_fill_u32(c->W<uint32_t>(c->wp.ready), 0u, (c->wp.act - c->wp.ready) / 4, st));
    c->launches += 7;
    c->table_ready = true;
  }
  return W4_OK;
}

// All-or-nothing check of a row list: distinct, live, seeded, below the cap.
int check_rows(w4_ctx* c, int32_t B, const int32_t* slots) {
  if (B < 1 || B > c->Bm) return fail(c, W4_E_INVALID, "B must be in [1, max_streams]");
  if (!slots) return fail(c, W4_E_INVALID, "null slot list");
  std::vector<uint8_t> seen(c->Bm, 0);
  for (int b = 0; b < B; ++b) {
    const int s = slots[b];
    if (s < 0 || s >= c->Bm || !c->live[s]) return fail(c, W4_E_BAD_SLOT, "slot " + std::to_string(s) + " is not live");
    if (seen[s]) return fail(c, W4_E_BAD_SLOT, "slot " + std::to_string(s) + " listed twice");
    seen[s] = 1;
    if (c->need_seed[s]) return fail(c, W4_E_NOT_READY, "slot " + std::to_string(s) + " has an unseeded prompt");
    if (c->pos[s] >= c->cap) return fail(c, W4_E_CONTEXT_CAP, "slot " + std::to_string(s) + " is at the context cap");
  }
  return W4_OK;
}

// Invalid-token flags of ring entry i (a finished step) -> the sticky report.
void take_flags(w4_ctx* c, int i) {
  const int32_t* f = c->flags + (size_t)i * c->Bm;
  for (int b = 0; b < c->err_rows[i]; ++b)
    if (f[b] && c->sticky.empty())
      c->sticky = "a token id outside [0, vocab) was given to row " + std::to_string(b) +
                  " of an earlier decode step (its embedding row was taken as zero)";
  c->err_pending[i] = false;
}

// Collect the flags of every step that has finished (wait: every enqueued
// step), then report and clear an invalid token seen since the last report.
int poll_errors(w4_ctx* c, bool wait) {
  for (int i = 0; i < kRing; ++i) {
    if (!c->err_pending[i]) continue;
    const hipError_t q = hipEventQuery(c->ev_err[i]);
    if (q == hipErrorNotReady && !wait) continue;
    if (q == hipErrorNotReady) {
      HIPCHK(c, hipEventSynchronize(c->ev_err[i]));
      c->syncs++;
    } else if (q != hipSuccess) {
      return fail(c, W4_E_HIP, std::string("hipEventQuery: ") + hipGetErrorString(q));
    }
    take_flags(c, i);
  }
  if (c->pf_pending) {
    const hipError_t q = hipEventQuery(c->ev_pf_done);
    if (q == hipSuccess || wait) {
      if (q != hipSuccess) {
        HIPCHK(c, hipEventSynchronize(c->ev_pf_done));
        c->syncs++;
      }
      for (int b = 0; b < c->pf_flag_rows; ++b)
        if (c->pf_flags[b] && c->sticky.empty())
          c->sticky = "a token id outside [0, vocab) was given at prompt position " + std::to_string(b) +
                      " of an earlier prefill (its embedding row was taken as zero)";
      c->pf_pending = false;
    }
  }
  if (c->werr && __atomic_load_n(c->werr, __ATOMIC_ACQUIRE)) {
    __atomic_store_n(c->werr, 0, __ATOMIC_RELEASE);
    return fail(c, W4_E_HIP,
                "a device-side wait of the fused expert products ran out of its bound in an earlier call (another "
                "launch holding compute units?); that call's results are not valid");
  }
  if (c->sticky.empty()) return W4_OK;
  const std::string m = c->sticky;
  c->sticky.clear();
  return fail(c, W4_E_INVALID, m);
}

// Slot ids and positions of the rows -> workspace, through a pinned ring.
int upload_rows(w4_ctx* c, int32_t B, const int32_t* slots, hipStream_t st, int* max_pos) {
  const int i = c->ring;
  c->ring = (c->ring + 1) % kRing;
  if (c->ev_used[i] && hipEventQuery(c->ev[i]) == hipErrorNotReady) {
    HIPCHK(c, hipEventSynchronize(c->ev[i]));
    c->syncs++;
  }
  if (c->err_pending[i]) {  // the entry's flags are overwritten by this step: collect them first
    if (hipEventQuery(c->ev_err[i]) == hipErrorNotReady) {
      HIPCHK(c, hipEventSynchronize(c->ev_err[i]));
      c->syncs++;
    }
    take_flags(c, i);
  }
  c->cur = i;
  int32_t* p = c->pinned + (size_t)i * c->row_words();
  int32_t* split = p + c->split_off();
  int32_t* prm = p + 2 * c->Bm;
  bool sampled = false;
  int mp = 0, n = 0;
  for (int b = 0; b < B; ++b) {
    const int pos = c->pos[slots[b]];
    p[b] = slots[b];
    p[c->Bm + b] = pos;
    const Sampling& sp = c->smp[slots[b]];
    int32_t* q = prm + (size_t)b * kSampleParams;
    std::memcpy(&q[0], &sp.temperature, 4);
    q[1] = sp.top_k;
    std::memcpy(&q[2], &sp.top_p, 4);
    q[3] = (int32_t)(uint32_t)(sp.seed & 0xFFFFFFFFu);
    q[4] = (int32_t)(uint32_t)(sp.seed >> 32);
    sampled = sampled || sp.temperature > 0.f;
    mp = std::max(mp, pos);
  }
  // Attention work list, one entry (stream b << 16 | split << 8 | kv head,
  // slot << 16 | position) per work-group, the splits with the most
  // 64-position chunks first: work-groups are dispatched in list order, so the
  // short tail splits are the ones that double up on a compute unit.  The
  // order does not change any result.
  const int W = kAttnSplitChunks;
  for (int cnt = W; cnt >= 1; --cnt)
    for (int b = 0; b < B; ++b) {
      const int pb = c->pos[slots[b]];
      const int nch = pb / 64 + 1, ns = attn_splits(pb);
      for (int sp = 0; sp < ns; ++sp)
        if (std::min(W, nch - W * sp) == cnt)
          for (int g = 0; g < c->d.n_kv_heads; ++g) {
            split[2 * n] = (b << 16) | (sp << 8) | g;
            split[2 * n + 1] = (slots[b] << 16) | pb;
            ++n;
          }
    }
  if (c->split_off() + 2 * n > c->row_words()) return fail(c, W4_E_INVALID, "row list exceeds its workspace region");
  HIPCHK(c, hipMemcpyAsync(c->W<int32_t>(c->wp.rows), p, sizeof(int32_t) * (c->split_off() + 2 * n),
                           hipMemcpyHostToDevice, st));
  c->any_sampled = sampled;
  HIPCHK(c, hipEventRecord(c->ev[i], st));
  c->ev_used[i] = true;
  c->nsplits = n;
  if (max_pos) *max_pos = mp;
  return W4_OK;
}

// Times the one launch in its scope when it belongs to the profiled kernel
// family (events recorded with that launch's dispatch, see w4_launch).
struct ProfScope {
  ProfScope(w4_ctx* c, int kernel, hipStream_t) {
    if (c->prof_kernel == kernel) c->prof_arm();
  }
  ~ProfScope() { g_launch_ev = LaunchEvents{}; }
};

#define LCHK(ctx, n, expr)                                                                      \
  do {                                                                                          \
    hipError_t e_ = (expr);                                                                     \
    (ctx)->launches += (n);                                                                     \
    if (e_ != hipSuccess) return fail(ctx, W4_E_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

// Decode batches above this many rows read the weights (expert, dense and
// output projection) with non-temporal loads; same results.  Measured: expert
// gate/up 37.9 against 39.2 us and down 22.2 against 23.4 us at B = 32, but
// 13.5 against 12.5 and 8.5 against 7.9 us at B = 1.
constexpr int kNtMinRows = 8;

// A prompt of at least this many rows runs its expert products over 32-row
// units, and from the second size on its gate/up product over 64-row units
// (about 64 rows per expert at top-8 of 128 experts, so little padding; the
// down product keeps 32-row units: its 64-row form holds two work-groups per
// compute unit instead of five and was measured slower, 180 against 135 us).
constexpr int kPromptUnitRows32 = 64, kPromptUnitRows64 = 1024;

// Dense product of a prompt's rows: the large-M form (128 x 128 blocks) for a
// prompt of at least 128 rows and an output of at least 64 tiles (enough
// blocks to fill the chip), else the row-block form.
hipError_t pf_gemm(const Mat& w, int P, const uint16_t* x, int ldx, void* y, int ldy, int epi, hipStream_t st) {
  if (P >= 128 && w.ntiles() >= 64 && lm_ok(w, ldx)) return launch_gemm_lm(w, P, x, ldx, y, ldy, epi, st);
  return launch_gemm(w, P, x, ldx, y, ldy, epi, st);
}

// The grouped expert products of one layer: one fused launch (gate/up +
// SwiGLU, then down; see k_moe_fused) where the geometry allows and the
// option is on, else the two launches.  Same results bit for bit.  *direct:
// y is in (stream, rank) order (the two launches with non-temporal loads,
// when r has pair_flat: the combine then reads it without the permutation,
// B = 32: 6316 against 6285 tok/s; at B = 1 and 8 it measured 0.3-0.5%
// slower), else in pair order.
int launch_experts(w4_ctx* c, const LayerLoc& L, const uint16_t* xn, int ldx, const RouteOut& r, uint16_t* act,
                   uint16_t* y, uint32_t* ready, bool nt, bool one, hipStream_t st, bool* direct) {
  const Mat gate = c->mat(L.gate), up = c->mat(L.up), down = c->mat(L.down);
  *direct = false;
  if (c->fused_moe && moe_fused_ok(gate, down)) {
    if (c->moe_epoch == 0xFFFFFFFFu) return fail(c, W4_E_UNSUPPORTED, "fused expert launch epochs exhausted");
    ProfScope ps(c, W4_K_MOE, st);
    LCHK(c, 1, launch_moe_fused(gate, up, down, xn, ldx, r, act, y, ready, ++c->moe_epoch, c->werr_dev, st));
    return W4_OK;
  }
  {
    ProfScope ps(c, W4_K_MOE_GATEUP, st);
    RouteOut rg = r;  // the gate/up product over the second unit list when there is one
    if (r.units2) {
      rg.units = r.units2;
      rg.rows_via_rec = 1;
      rg.n_units = r.n_units2;
      rg.unit_n = r.unit_n2;
      rg.units_cap = r.units_cap2;
      rg.unit_rows8 = nullptr;
    }
    LCHK(c, 1, launch_moe_gateup(gate, up, xn, ldx, rg, act, st, nt, one));
  }
  {
    ProfScope ps(c, W4_K_MOE_DOWN, st);
    LCHK(c, 1, launch_moe_down(down, act, r, y, st, nt, nt && r.pair_flat != nullptr));
  }
  *direct = nt && r.pair_flat != nullptr;
  return W4_OK;
}

// One decoder layer on rows whose slot/pos vectors are uploaded.  Input: h
// (residual, row-major) and xp = RMSNorm_attn(h) as an activation panel.
// Output: h updated; if next_gamma, xp = RMSNorm(h) * next_gamma (panel).
int layer_body(w4_ctx* c, int l, int B, int max_pos, uint16_t* h, uint16_t* xp, int32_t* ids_out,
               const uint16_t* next_gamma, hipStream_t st) {
  const w4_model_desc& d = c->d;
  const LayerLoc& L = c->bp.layers[l];
  const int H = d.hidden, nqkv = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim, qd = d.n_q_heads * d.head_dim;
  const int R = panel_rows(c->Bm);
  const int32_t* slot = c->W<int32_t>(c->wp.rows);
  const int32_t* pos = slot + c->Bm;
  KV kv = c->kv();
  uint16_t* qkv = c->W<uint16_t>(c->wp.qkv);
  uint16_t* xn = c->W<uint16_t>(c->wp.xn);  // MoE input, row-major (gathered by stream)
  uint16_t* o = c->W<uint16_t>(c->wp.attn_o);
  {
    ProfScope ps(c, W4_K_DENSE, st);
    LCHK(c, 1, launch_gemm(c->mat(L.qkv), B, xp, H, qkv, nqkv, EPI_F16, st, R, B > kNtMinRows));
  }
  // Spare work-groups of the router launch touch the next layer's norms and
  // q/k/v, o and router weights (contiguous in the bank), so that those
  // latency-bound launches find them in the memory-side cache.  Measured on
  // the 48-layer model: q/k/v and o 0.5 us faster each at B <= 8; at B = 32
  // the expert and KV traffic in between evicts the span again.  With one
  // row they also touch that row's live KV chunks of the next layer: its
  // attention 11.2 -> 10.4 us, +2% tok/s; with 2..8 rows the larger touch
  // lengthened the router launch by about as much as the attention gained
  // (B = 2: -0.8%, 3: +1.3%, 4: -0.4%, 8: -1.7%).
  const uint8_t* next_span = nullptr;
  size_t next_bytes = 0;
  if (l + 1 < d.n_layers && B <= 8) {
    const LayerLoc& Ln = c->bp.layers[l + 1];
    next_span = c->Bk<uint8_t>(Ln.attn_norm);
    next_bytes = Ln.gate.tiles - Ln.attn_norm;
  }
  LCHK(c, 1, launch_attention(B, l, d.n_q_heads, kv, c->dev_splits(), c->nsplits, qkv, nqkv,
                              qkv + (size_t)d.n_q_heads * d.head_dim, qkv + (size_t)(d.n_q_heads + d.n_kv_heads) * d.head_dim,
                              nqkv, c->W<float2>(c->wp.table), c->W<float>(c->wp.part_o), c->W<float>(c->wp.part_ml),
                              c->W<unsigned>(c->wp.aticket), o, st, c->prof_kernel == W4_K_ATTENTION ? c : nullptr, R));
  // Above 16 rows (a 32-row tile) the output projection at K = 4096 runs as
  // two work-groups per tile (same sums, bit for bit; see
  // launch_gemm_resid_split).  Measured on the 48-layer model with the earlier
  // flag-wait form: +0.4% tok/s at B = 32, -1..2% at B <= 8.
  {
    ProfScope ps(c, W4_K_DENSE, st);
    const Mat Om = c->mat(L.o);
    if (B > 16 && Om.K == 16 * 256 && Om.ntiles() <= kSplitMaxTiles)
      LCHK(c, 1, launch_gemm_resid_split(Om, B, o, R, h, H, c->W<float>(c->wp.spart), c->W<unsigned>(c->wp.sticket), st,
                                         B > kNtMinRows));
    else
      LCHK(c, 1, launch_gemm(Om, B, o, qd, h, H, EPI_RESID, st, R, B > kNtMinRows));
  }
  RouteOut r = c->route_out(ids_out);
  // outputs that no kernel of the step reads are not written (B = 32: +0.15%
  // tok/s); the non-temporal gate/up (more than kNtMinRows streams) reads its
  // unit rows as bytes, the fused expert launch as words
  r.counts = nullptr;
  r.offsets = nullptr;
  r.pair_stream = nullptr;
  r.pair_rank = nullptr;
  if (B > kNtMinRows && !c->fused_moe) r.unit_rows = nullptr;
  {
    ProfScope ps(c, W4_K_ROUTER, st);
    const Mat Rm = c->mat(L.router);
    LCHK(c, 1, launch_router(B, H, d.n_experts, d.top_k, d.group, h, c->Bk<uint16_t>(L.moe_norm), d.rms_eps, xn,
                             Rm.tiles, Rm.scales, r, c->W<unsigned>(c->wp.ticket), c->W<float>(c->wp.rlg),
                             c->W<unsigned>(c->wp.rticket), st, next_span, next_bytes,
                             next_span && B == 1 ? &kv : nullptr, l + 1, slot, pos));
  }
  bool direct = false;
  {
    int rc = launch_experts(c, L, xn, H, r, c->W<uint16_t>(c->wp.act), c->W<uint16_t>(c->wp.y),
                            c->W<uint32_t>(c->wp.ready), B > kNtMinRows, B == 1, st, &direct);
    if (rc) return rc;
  }
  LCHK(c, 1, launch_combine(B, H, d.top_k, r.w, r.inv, c->W<uint16_t>(c->wp.y), h, true, next_gamma, d.rms_eps,
                            xp, st, R, direct));
  return W4_OK;
}

}  // namespace

namespace w4 {
thread_local LaunchEvents g_launch_ev;
void prof_arm(void* ctx) { static_cast<w4_ctx*>(ctx)->prof_arm(); }
}  // namespace w4

// =========================================================================== C ABI
extern "C" {

size_t w4_arena_bytes(const w4_model_desc* d, int32_t max_streams, int32_t cap) {
  if (!geometry_ok(d, nullptr) || !sizes_ok(max_streams, cap, nullptr)) return 0;
  return 2 * (size_t)d->n_layers * max_streams * d->n_kv_heads * (size_t)cap * d->head_dim * 2;
}

size_t w4_bank_bytes(const w4_model_desc* d) {
  if (!geometry_ok(d, nullptr)) return 0;
  return plan_bank(*d).total;
}

size_t w4_workspace_bytes(const w4_model_desc* d, int32_t max_streams, int32_t cap) {
  if (!geometry_ok(d, nullptr) || !sizes_ok(max_streams, cap, nullptr)) return 0;
  return plan_ws(*d, max_streams, cap).total;
}

int w4_create(const w4_model_desc* d, int32_t max_streams, int32_t cap, void* arena_dev, void* bank_dev,
              void* ws_dev, w4_ctx** out) {
  std::string why;
  if (!out) return W4_E_INVALID;
  *out = nullptr;
  if (!geometry_ok(d, &why) || !sizes_ok(max_streams, cap, &why)) {
    std::fprintf(stderr, "w4_create: %s\n", why.c_str());
    return W4_E_INVALID;
  }
  // The grouped expert products keep every 16-row unit record of a launch in
  // two records per thread: E + max_streams * top_k / 16 + 1 records must fit
  // in 2 * 64 * (waves of the product), for K = hidden (gate/up) and
  // K = moe_inter (down), waves = K / 256 (K / 128 when K % 256 != 0).
  for (int K : {d->hidden, d->moe_inter}) {
    const int nw = K / ((K % 256 == 0) ? 256 : 128);
    const int units_cap = d->n_experts + max_streams * d->top_k / 16 + 1;
    if (units_cap > 2 * 64 * nw || units_cap > kMaxUnits) {
      std::fprintf(stderr, "w4_create: %d experts with max_streams %d and top_k %d need %d expert work units, more "
                   "than the %d that a product over K = %d holds\n", d->n_experts, max_streams, d->top_k, units_cap,
                   2 * 64 * nw, K);
      return W4_E_UNSUPPORTED;
    }
  }
  if (!arena_dev || !bank_dev || !ws_dev) return W4_E_INVALID;
  if (((uintptr_t)arena_dev | (uintptr_t)bank_dev | (uintptr_t)ws_dev) % kAlign) return W4_E_INVALID;
  w4_ctx* c = new w4_ctx;
  c->d = *d;
  c->Bm = max_streams;
  c->cap = cap;
  c->arena = static_cast<char*>(arena_dev);
  c->bank = static_cast<char*>(bank_dev);
  c->ws = static_cast<char*>(ws_dev);
  c->bp = plan_bank(*d);
  c->wp = plan_ws(*d, max_streams, cap);
  c->pos.assign(max_streams, 0);
  c->prompt.assign(max_streams, 0);
  c->live.assign(max_streams, 0);
  c->need_seed.assign(max_streams, 0);
  c->smp.assign(max_streams, Sampling{});
  *out = c;
  return W4_OK;
}

void w4_destroy(w4_ctx* c) {
  if (!c) return;
  for (hipEvent_t e : c->prof_ev) (void)hipEventDestroy(e);
  if (c->dev_ready) {
    for (int i = 0; i < kRing; ++i) {
      if (c->ev[i]) (void)hipEventSynchronize(c->ev[i]), (void)hipEventDestroy(c->ev[i]);
      if (c->ev_err[i]) (void)hipEventSynchronize(c->ev_err[i]), (void)hipEventDestroy(c->ev_err[i]);
    }
    if (c->pinned) (void)hipHostFree(c->pinned);
    if (c->flags) (void)hipHostFree(c->flags);
    if (c->werr) (void)hipHostFree(c->werr);
    if (c->ev_pf) (void)hipEventSynchronize(c->ev_pf), (void)hipEventDestroy(c->ev_pf);
    if (c->ev_pf_done) (void)hipEventSynchronize(c->ev_pf_done), (void)hipEventDestroy(c->ev_pf_done);
    if (c->pf_pinned) (void)hipHostFree(c->pf_pinned);
    if (c->pf_flags) (void)hipHostFree(c->pf_flags);
  }
  delete c;
}

int w4_bank_load(w4_ctx* c, int32_t layer, int32_t tensor, int32_t expert, const void* packed, const void* scales,
                 void* stream) {
  if (!c) return W4_E_INVALID;
  const w4_model_desc& d = c->d;
  const bool global = tensor == W4_T_EMBED || tensor == W4_T_LM_HEAD || tensor == W4_T_FINAL_NORM;
  if (!global && (layer < 0 || layer >= d.n_layers)) return fail(c, W4_E_INVALID, "layer out of range");
  if (!packed) return fail(c, W4_E_INVALID, "null source");
  const bool is_norm = tensor == W4_T_ATTN_NORM || tensor == W4_T_MOE_NORM || tensor == W4_T_FINAL_NORM;
  if (!is_norm && !scales) return fail(c, W4_E_INVALID, "null scales");
  const bool is_expert = tensor == W4_T_GATE || tensor == W4_T_UP || tensor == W4_T_DOWN;
  if (is_expert && (expert < -1 || expert >= d.n_experts)) return fail(c, W4_E_INVALID, "expert out of range");
  hipStream_t st = (hipStream_t)stream;
  int rc = ensure_device(c, st);
  if (rc) return rc;
  const LayerLoc* L = global ? nullptr : &c->bp.layers[layer];
  const size_t H2 = (size_t)d.hidden * 2;
  auto copy = [&](size_t off, const void* src, size_t bytes) -> int {
    HIPCHK(c, hipMemcpyAsync(c->bank + off, src, bytes, hipMemcpyDeviceToDevice, st));
    return W4_OK;
  };
  switch (tensor) {
    case W4_T_ATTN_NORM: return copy(L->attn_norm, packed, H2);
    case W4_T_MOE_NORM: return copy(L->moe_norm, packed, H2);
    case W4_T_FINAL_NORM: return copy(c->bp.final_norm, packed, H2);
    case W4_T_EMBED:
      rc = copy(c->bp.emb_p, packed, (size_t)d.vocab * d.hidden / 2);
      if (rc) return rc;
      return copy(c->bp.emb_s, scales, (size_t)d.vocab * (d.hidden / d.group) * 2);
    default: break;
  }
  const Loc* loc = nullptr;
  switch (tensor) {
    case W4_T_QKV: loc = &L->qkv; break;
    case W4_T_O: loc = &L->o; break;
    case W4_T_ROUTER: loc = &L->router; break;
    case W4_T_GATE: loc = &L->gate; break;
    case W4_T_UP: loc = &L->up; break;
    case W4_T_DOWN: loc = &L->down; break;
    case W4_T_LM_HEAD: loc = &c->bp.lm; break;
    default: return fail(c, W4_E_INVALID, "unknown tensor id");
  }
  const int count = (is_expert && expert < 0) ? d.n_experts : 1;
  const int first = (is_expert && expert >= 0) ? expert : 0;
  Mat m = c->mat(*loc, first);
  LCHK(c, 2, launch_repack(static_cast<const uint8_t*>(packed), static_cast<const uint16_t*>(scales), count, loc->N,
                           loc->K, d.group, const_cast<uint4*>(m.tiles), const_cast<uint16_t*>(m.scales), st));
  return W4_OK;
}

int w4_slot_alloc(w4_ctx* c, int32_t prompt_len, int32_t max_new, int32_t* slot_out) {
  if (!c || !slot_out) return W4_E_INVALID;
  if (prompt_len < 0 || max_new < 0) return fail(c, W4_E_INVALID, "negative length");
  if ((int64_t)prompt_len + max_new > c->cap)
    return fail(c, W4_E_CONTEXT_CAP, "prompt_len + max_new_tokens exceeds the context cap");
  for (int s = 0; s < c->Bm; ++s)
    if (!c->live[s]) {
      c->live[s] = 1;
      c->pos[s] = 0;
      c->prompt[s] = prompt_len;
      c->need_seed[s] = prompt_len > 0;
      c->smp[s] = Sampling{};  // greedy until set
      *slot_out = s;
      return W4_OK;
    }
  return fail(c, W4_E_NO_SLOT, "every slot is live");
}

int w4_slot_seed(w4_ctx* c, int32_t slot, const void* k, const void* v, void* stream) {
  if (!c) return W4_E_INVALID;
  if (slot < 0 || slot >= c->Bm || !c->live[slot]) return fail(c, W4_E_BAD_SLOT, "slot is not live");
  if (!c->need_seed[slot]) return fail(c, W4_E_BAD_SLOT, "slot has no unseeded prompt (seed once per join)");
  if (!k || !v) return fail(c, W4_E_INVALID, "null K/V");
  hipStream_t st = (hipStream_t)stream;
  int rc = ensure_device(c, st);
  if (rc) return rc;
  LCHK(c, 1, launch_seed(c->d.n_layers, c->prompt[slot], slot, c->kv(), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), st));
  c->need_seed[slot] = 0;
  c->pos[slot] = c->prompt[slot];
  return W4_OK;
}

int w4_slot_set_sampling(w4_ctx* c, int32_t slot, uint64_t seed, float temperature, int32_t top_k, float top_p) {
  if (!c) return W4_E_INVALID;
  if (slot < 0 || slot >= c->Bm || !c->live[slot]) return fail(c, W4_E_BAD_SLOT, "slot is not live");
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(c, W4_E_INVALID, "temperature must be finite and >= 0");
  if (top_k < 1 || top_k > kSampleMaxK) return fail(c, W4_E_INVALID, "top_k must be in [1, 64]");
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(c, W4_E_INVALID, "top_p must be in (0, 1]");
  c->smp[slot] = Sampling{seed, temperature, top_p, top_k};
  return W4_OK;
}

int w4_slot_read_kv(w4_ctx* c, int32_t slot, void* k, void* v, void* stream) {
  if (!c) return W4_E_INVALID;
  if (slot < 0 || slot >= c->Bm || !c->live[slot]) return fail(c, W4_E_BAD_SLOT, "slot is not live");
  if (c->need_seed[slot]) return fail(c, W4_E_NOT_READY, "slot has an unseeded prompt");
  if (!k || !v) return fail(c, W4_E_INVALID, "null K/V");
  hipStream_t st = (hipStream_t)stream;
  int rc = ensure_device(c, st);
  if (rc) return rc;
  LCHK(c, 1, launch_read_kv(c->d.n_layers, c->pos[slot], slot, c->kv(), static_cast<uint16_t*>(k),
                            static_cast<uint16_t*>(v), st));
  return W4_OK;
}

int w4_slot_release(w4_ctx* c, int32_t slot) {
  if (!c) return W4_E_INVALID;
  if (slot < 0 || slot >= c->Bm || !c->live[slot]) return fail(c, W4_E_BAD_SLOT, "slot is not live");
  c->live[slot] = 0;
  c->need_seed[slot] = 0;
  c->pos[slot] = 0;
  return W4_OK;
}

int w4_slot_position(const w4_ctx* c, int32_t slot, int32_t* pos_out) {
  if (!c || !pos_out) return W4_E_INVALID;
  if (slot < 0 || slot >= c->Bm || !c->live[slot]) return W4_E_BAD_SLOT;
  *pos_out = c->pos[slot];
  return W4_OK;
}

int w4_slots_advance(w4_ctx* c, int32_t n, const int32_t* slots) {
  if (!c) return W4_E_INVALID;
  int rc = check_rows(c, n, slots);
  if (rc) return rc;
  for (int b = 0; b < n; ++b) c->pos[slots[b]]++;
  return W4_OK;
}

int w4_decode_step(w4_ctx* c, int32_t B, const int32_t* slots, const int32_t* tokens, void* logits, int32_t* next,
                   int32_t* route_ids, void* stream) {
  if (!c) return W4_E_INVALID;
  int rc = check_rows(c, B, slots);
  if (rc) return rc;
  if (!tokens || !next) return fail(c, W4_E_INVALID, "null tokens or next");
  hipStream_t st = (hipStream_t)stream;
  rc = ensure_device(c, st);
  if (rc) return rc;
  rc = poll_errors(c, false);
  if (rc) return rc;
  const int l0 = c->launches, s0 = c->syncs;
  const w4_model_desc& d = c->d;
  int max_pos = 0;
  rc = upload_rows(c, B, slots, st, &max_pos);
  if (rc) return rc;
  uint16_t* h = c->W<uint16_t>(c->wp.h);
  uint16_t* xp = c->W<uint16_t>(c->wp.xp);
  const int R = panel_rows(c->Bm);
  LCHK(c, 1, launch_embed(B, d.hidden, d.vocab, d.group, tokens, c->Bk<uint8_t>(c->bp.emb_p),
                          c->Bk<uint16_t>(c->bp.emb_s), h, c->Bk<uint16_t>(c->bp.layers[0].attn_norm), d.rms_eps, xp,
                          c->flags_dev + (size_t)c->cur * c->Bm, st, R));
  for (int l = 0; l < d.n_layers; ++l) {
    const uint16_t* ng = l + 1 < d.n_layers ? c->Bk<uint16_t>(c->bp.layers[l + 1].attn_norm)
                                            : c->Bk<uint16_t>(c->bp.final_norm);
    rc = layer_body(c, l, B, max_pos, h, xp, route_ids ? route_ids + (size_t)l * B * d.top_k : nullptr, ng, st);
    if (rc) return rc;
  }
  uint16_t* lg = logits ? static_cast<uint16_t*>(logits) : c->W<uint16_t>(c->wp.logits);
  {
    ProfScope ps(c, W4_K_DENSE, st);
    LCHK(c, 1, launch_gemm(c->mat(c->bp.lm), B, xp, d.hidden, lg, d.vocab, EPI_F16, st, R, B > kNtMinRows));
  }
  // greedy rows only: the split argmax; any sampled row: the sampler for every
  // row (a greedy row's id is the same either way: the first rank)
  if (c->any_sampled) {
    const int32_t* rows = c->dev_rows();
    LCHK(c, 1, launch_sample(B, d.vocab, lg, rows + 2 * c->Bm, rows + c->Bm, next, st));
  } else {
    LCHK(c, 1, launch_argmax(B, d.vocab, lg, next, c->W<float>(c->wp.amax_v), c->W<int32_t>(c->wp.amax_i),
                              c->W<unsigned>(c->wp.amax_ticket), st));
  }
  // the embedding wrote the step's invalid-token flags into its ring entry;
  // a later call reads them once this event has passed (see poll_errors)
  {
    const int i = c->cur;
    HIPCHK(c, hipEventRecord(c->ev_err[i], st));
    c->err_pending[i] = true;
    c->err_rows[i] = B;
  }
  for (int b = 0; b < B; ++b) c->pos[slots[b]]++;
  c->last_launches = c->launches - l0;
  c->last_syncs = c->syncs - s0;
  return W4_OK;
}

size_t w4_prefill_workspace_bytes(const w4_model_desc* d, int32_t max_prompt, int32_t cap) {
  if (!geometry_ok(d, nullptr) || !sizes_ok(1, cap, nullptr) || max_prompt < 1 || max_prompt > cap) return 0;
  if ((size_t)max_prompt * d->top_k > (size_t)kPrefillMaxPairs) return 0;
  if (route_prefill_lds(max_prompt, d->n_experts, d->top_k) > 61440) return 0;
  return plan_prefill(*d, max_prompt, cap).total;
}

int w4_slot_prefill(w4_ctx* c, int32_t slot, const int32_t* tokens, void* ws_dev, size_t ws_bytes, void* logits,
                    int32_t* next, int32_t* route_ids, void* stream) {
  if (!c) return W4_E_INVALID;
  const w4_model_desc& d = c->d;
  if (slot < 0 || slot >= c->Bm || !c->live[slot]) return fail(c, W4_E_BAD_SLOT, "slot is not live");
  if (!c->need_seed[slot]) return fail(c, W4_E_BAD_SLOT, "slot has no prompt waiting (prefill once per join)");
  const int P = c->prompt[slot];
  if (!tokens || !ws_dev) return fail(c, W4_E_INVALID, "null tokens or workspace");
  if ((uintptr_t)ws_dev % kAlign) return fail(c, W4_E_INVALID, "prefill workspace must be 256-byte aligned");
  if ((size_t)P * d.top_k > (size_t)kPrefillMaxPairs || route_prefill_lds(P, d.n_experts, d.top_k) > 61440)
    return fail(c, W4_E_UNSUPPORTED, "prompt too long for the prefill routing (prompt * top_k <= 16384, and "
                                     "n_experts * ceil(prompt / 32) * 6 <= 61440)");
  const PfPlan pp = plan_prefill(d, P, c->cap);
  if (ws_bytes < pp.total) return fail(c, W4_E_INVALID, "prefill workspace smaller than w4_prefill_workspace_bytes");
  hipStream_t st = (hipStream_t)stream;
  int rc = ensure_device(c, st);
  if (rc) return rc;
  rc = poll_errors(c, false);
  if (rc) return rc;
  const int l0 = c->launches;
  char* ws = static_cast<char*>(ws_dev);
  auto PW = [&](size_t off) { return ws + off; };
  // upload: slot and position of every prompt row, the slot's sampling
  // parameters, and each chunk's attention work list (rows relative to the chunk)
  const size_t words = pp.row_cap;
  if (c->pf_used && hipEventQuery(c->ev_pf) == hipErrorNotReady) {
    HIPCHK(c, hipEventSynchronize(c->ev_pf));
    c->syncs++;
  }
  if (c->pf_pending) {  // the flag buffer is reused below: collect the last prefill's flags first
    rc = poll_errors(c, true);
    if (rc) return rc;
  }
  if (P > c->pf_flag_cap) {
    if (c->pf_flags) HIPCHK(c, hipHostFree(c->pf_flags));
    c->pf_flags = nullptr;
    HIPCHK(c, hipHostMalloc((void**)&c->pf_flags, sizeof(int32_t) * P, hipHostMallocMapped | hipHostMallocCoherent));
    HIPCHK(c, hipHostGetDevicePointer((void**)&c->pf_flags_dev, c->pf_flags, 0));
    c->pf_flag_cap = P;
  }
  if (!c->ev_pf_done) HIPCHK(c, hipEventCreateWithFlags(&c->ev_pf_done, hipEventDisableTiming));
  if (words > c->pf_words) {
    if (c->pf_pinned) HIPCHK(c, hipHostFree(c->pf_pinned));
    c->pf_pinned = nullptr;
    HIPCHK(c, hipHostMalloc((void**)&c->pf_pinned, words * 4, hipHostMallocDefault));
    c->pf_words = words;
  }
  if (!c->ev_pf) HIPCHK(c, hipEventCreateWithFlags(&c->ev_pf, hipEventDisableTiming));
  int32_t* hp = c->pf_pinned;
  for (int i = 0; i < P; ++i) {
    hp[i] = slot;
    hp[P + i] = i;
  }
  {
    const Sampling& sp = c->smp[slot];
    int32_t* q = hp + 2 * P;
    std::memcpy(&q[0], &sp.temperature, 4);
    q[1] = sp.top_k;
    std::memcpy(&q[2], &sp.top_p, 4);
    q[3] = (int32_t)(uint32_t)(sp.seed & 0xFFFFFFFFu);
    q[4] = (int32_t)(uint32_t)(sp.seed >> 32);
  }
  const size_t n = 2 * (size_t)P + kSampleParams;
  if (n > words) return fail(c, W4_E_INVALID, "prefill row list exceeds its workspace region");
  int32_t* drows = reinterpret_cast<int32_t*>(PW(pp.rows));
  HIPCHK(c, hipMemcpyAsync(drows, hp, n * 4, hipMemcpyHostToDevice, st));
  HIPCHK(c, hipEventRecord(c->ev_pf, st));
  c->pf_used = true;
  HIPCHK(c, launch_fill_u32(reinterpret_cast<uint32_t*>(PW(pp.rmask)), 0u,
                            2 * (size_t)d.n_experts * ((P + 31) / 32), st));
  c->launches += 1;

  const int H = d.hidden, E = d.n_experts, k = d.top_k, Hq = d.n_q_heads, D = d.head_dim;
  const int nqkv = (d.n_q_heads + 2 * d.n_kv_heads) * D, qd = Hq * D;
  uint16_t* h = reinterpret_cast<uint16_t*>(PW(pp.h));
  uint16_t* xn = reinterpret_cast<uint16_t*>(PW(pp.xn));
  uint16_t* qkv = reinterpret_cast<uint16_t*>(PW(pp.qkv));
  uint16_t* ao = reinterpret_cast<uint16_t*>(PW(pp.attn_o));
  KV kv = c->kv();
  RouteOut r;
  r.w = reinterpret_cast<float*>(PW(pp.w));
  r.counts = reinterpret_cast<int32_t*>(PW(pp.counts));
  r.offsets = reinterpret_cast<int32_t*>(PW(pp.offsets));
  r.pair_stream = nullptr;
  r.pair_rank = nullptr;
  r.inv = reinterpret_cast<int32_t*>(PW(pp.inv));
  r.used = reinterpret_cast<int32_t*>(PW(pp.used));
  r.n_used = reinterpret_cast<int32_t*>(PW(pp.n_used));
  r.units = reinterpret_cast<int4*>(PW(pp.units));
  r.unit_rows = reinterpret_cast<int32_t*>(PW(pp.unit_rows));
  r.n_units = reinterpret_cast<int32_t*>(PW(pp.n_units));
  // a long prompt's expert products take 32-row units (each converted weight
  // operand serves two 16-row MFMA tiles; same results)
  r.unit_n = P >= kPromptUnitRows32 && !c->fused_moe ? 32 : 16;
  r.units_cap = E + P * k / r.unit_n + 1;
  if (r.unit_n == 32 && P >= kPromptUnitRows64) {
    r.units2 = reinterpret_cast<int4*>(PW(pp.units2));
    r.n_units2 = reinterpret_cast<int32_t*>(PW(pp.n_units2));
    r.unit_n2 = 64;
    r.units_cap2 = E + P * k / 64 + 1;
  }
  r.done = reinterpret_cast<uint32_t*>(PW(pp.done));
  // the fused expert launches' ready words: zero once per call (the caller's
  // buffer may hold anything), then written with this context's epochs only
  uint32_t* ready = reinterpret_cast<uint32_t*>(PW(pp.ready));
  LCHK(c, 1, launch_fill_u32(ready, 0u, (pp.act - pp.ready) / 4, st));
  LCHK(c, 1, launch_embed(P, H, d.vocab, d.group, tokens, c->Bk<uint8_t>(c->bp.emb_p), c->Bk<uint16_t>(c->bp.emb_s), h,
                          c->Bk<uint16_t>(c->bp.layers[0].attn_norm), d.rms_eps, xn, c->pf_flags_dev, st, 0));
  for (int l = 0; l < d.n_layers; ++l) {
    const LayerLoc& Ly = c->bp.layers[l];
    LCHK(c, 1, pf_gemm(c->mat(Ly.qkv), P, xn, H, qkv, nqkv, EPI_F16, st));
    LCHK(c, 1, launch_prefill_kv(P, l, slot, kv, qkv + qd, qkv + qd + d.n_kv_heads * D, nqkv,
                                 c->W<float2>(c->wp.table), st));
    LCHK(c, 1, launch_prefill_attention(P, l, slot, Hq, kv, qkv, nqkv, c->W<float2>(c->wp.table), ao, qd, st));
    LCHK(c, 1, pf_gemm(c->mat(Ly.o), P, ao, qd, h, H, EPI_RESID, st));
    LCHK(c, 1, launch_rmsnorm(P, H, h, c->Bk<uint16_t>(Ly.moe_norm), d.rms_eps, xn, st, 0));
    float* lg = reinterpret_cast<float*>(PW(pp.lg));
    LCHK(c, 1, launch_gemm(c->mat(Ly.router), P, xn, H, lg, E, EPI_F32, st));
    r.ids = route_ids ? route_ids + (size_t)l * P * k : reinterpret_cast<int32_t*>(PW(pp.ids));
    uint32_t* rmask = reinterpret_cast<uint32_t*>(PW(pp.rmask));
    const size_t mwords = (size_t)E * ((P + 31) / 32);
    LCHK(c, 2, launch_route_prefill(lg, P, E, k, r, rmask + (l & 1) * mwords, rmask + ((l + 1) & 1) * mwords,
                                    reinterpret_cast<uint8_t*>(PW(pp.re8)), st));
    uint16_t* act = reinterpret_cast<uint16_t*>(PW(pp.act));
    uint16_t* y = reinterpret_cast<uint16_t*>(PW(pp.y));
    bool direct = false;
    rc = launch_experts(c, Ly, xn, H, r, act, y, ready, false, P == 1, st, &direct);
    if (rc) return rc;
    const uint16_t* ng = l + 1 < d.n_layers ? c->Bk<uint16_t>(c->bp.layers[l + 1].attn_norm)
                                            : c->Bk<uint16_t>(c->bp.final_norm);
    LCHK(c, 1, launch_combine(P, H, k, r.w, r.inv, y, h, true, ng, d.rms_eps, xn, st, 0, direct));
  }
  // the last prompt token: output projection and its next token (the slot's
  // sampling at draw counter P - 1, the last prompt position)
  uint16_t* lgo = logits ? static_cast<uint16_t*>(logits) : reinterpret_cast<uint16_t*>(PW(pp.logits));
  int32_t* nx = next ? next : c->W<int32_t>(c->wp.next);
  LCHK(c, 1, launch_gemm(c->mat(c->bp.lm), 1, xn + (size_t)(P - 1) * H, H, lgo, d.vocab, EPI_F16, st));
  if (c->smp[slot].temperature > 0.f)
    LCHK(c, 1, launch_sample(1, d.vocab, lgo, drows + 2 * P, drows + P + (P - 1), nx, st));
  else
    LCHK(c, 1, launch_argmax(1, d.vocab, lgo, nx, c->W<float>(c->wp.amax_v), c->W<int32_t>(c->wp.amax_i),
                              c->W<unsigned>(c->wp.amax_ticket), st));
  HIPCHK(c, hipEventRecord(c->ev_pf_done, st));
  c->pf_pending = true;
  c->pf_flag_rows = P;
  c->need_seed[slot] = 0;
  c->pos[slot] = P;
  c->last_launches = c->launches - l0;
  return W4_OK;
}

int w4_gemm(w4_ctx* c, int32_t layer, int32_t tensor, int32_t expert, int32_t B, const void* x, void* y,
            void* stream) {
  if (!c) return W4_E_INVALID;
  const w4_model_desc& d = c->d;
  if (B < 1 || B > c->Bm) return fail(c, W4_E_INVALID, "B must be in [1, max_streams]");
  if (!x || !y) return fail(c, W4_E_INVALID, "null x or y");
  const bool global = tensor == W4_T_LM_HEAD;
  if (!global && (layer < 0 || layer >= d.n_layers)) return fail(c, W4_E_INVALID, "layer out of range");
  const LayerLoc* L = global ? nullptr : &c->bp.layers[layer];
  const Loc* loc = nullptr;
  int e = 0;
  switch (tensor) {
    case W4_T_QKV: loc = &L->qkv; break;
    case W4_T_O: loc = &L->o; break;
    case W4_T_ROUTER: loc = &L->router; break;
    case W4_T_GATE: loc = &L->gate; e = expert; break;
    case W4_T_UP: loc = &L->up; e = expert; break;
    case W4_T_DOWN: loc = &L->down; e = expert; break;
    case W4_T_LM_HEAD: loc = &c->bp.lm; break;
    default: return fail(c, W4_E_INVALID, "tensor has no product");
  }
  if (e < 0 || e >= d.n_experts) return fail(c, W4_E_INVALID, "expert out of range");
  hipStream_t st = (hipStream_t)stream;
  int rc = ensure_device(c, st);
  if (rc) return rc;
  const int epi = tensor == W4_T_ROUTER ? EPI_F32 : EPI_F16;
  ProfScope ps(c, W4_K_DENSE, st);
  LCHK(c, 1, launch_gemm(c->mat(*loc, e), B, static_cast<const uint16_t*>(x), loc->K, y, loc->N, epi, st));
  return W4_OK;
}

int w4_route(w4_ctx* c, int32_t B, const float* logits, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
             int32_t* pair_stream, int32_t* pair_rank, void* stream) {
  if (!c) return W4_E_INVALID;
  if (B < 1 || B > c->Bm) return fail(c, W4_E_INVALID, "B must be in [1, max_streams]");
  if (!logits || !ids || !w) return fail(c, W4_E_INVALID, "null logits, ids or w");
  hipStream_t st = (hipStream_t)stream;
  int rc = ensure_device(c, st);
  if (rc) return rc;
  RouteOut r = c->route_out();
  r.ids = ids;
  r.w = w;
  r.counts = counts;
  r.offsets = offsets;
  r.pair_stream = pair_stream;
  r.pair_rank = pair_rank;
  LCHK(c, 1, launch_route(logits, B, c->d.n_experts, c->d.top_k, r, st));
  return W4_OK;
}

int w4_moe(w4_ctx* c, int32_t layer, int32_t B, const void* x, const float* router_logits, void* y,
           int32_t* route_ids, void* stream) {
  if (!c) return W4_E_INVALID;
  const w4_model_desc& d = c->d;
  if (layer < 0 || layer >= d.n_layers) return fail(c, W4_E_INVALID, "layer out of range");
  if (B < 1 || B > c->Bm) return fail(c, W4_E_INVALID, "B must be in [1, max_streams]");
  if (!x || !y) return fail(c, W4_E_INVALID, "null x or y");
  hipStream_t st = (hipStream_t)stream;
  int rc = ensure_device(c, st);
  if (rc) return rc;
  const LayerLoc& L = c->bp.layers[layer];
  const uint16_t* xh = static_cast<const uint16_t*>(x);
  const float* lg = router_logits;
  if (!lg) {
    LCHK(c, 1, launch_gemm(c->mat(L.router), B, xh, d.hidden, c->W<float>(c->wp.rlogits), d.n_experts, EPI_F32, st));
    lg = c->W<float>(c->wp.rlogits);
  }
  RouteOut r = c->route_out(route_ids);
  LCHK(c, 1, launch_route(lg, B, d.n_experts, d.top_k, r, st));
  bool direct = false;
  rc = launch_experts(c, L, xh, d.hidden, r, c->W<uint16_t>(c->wp.act), c->W<uint16_t>(c->wp.y),
                      c->W<uint32_t>(c->wp.ready), B > kNtMinRows, B == 1, st, &direct);
  if (rc) return rc;
  LCHK(c, 1, launch_combine(B, d.hidden, d.top_k, r.w, r.inv, c->W<uint16_t>(c->wp.y), static_cast<uint16_t*>(y),
                            false, nullptr, d.rms_eps, nullptr, st, 0, direct));
  return W4_OK;
}

int w4_attn_decode(w4_ctx* c, int32_t layer, int32_t B, const int32_t* slots, const void* q, const void* k_new,
                   const void* v_new, void* o, void* stream) {
  if (!c) return W4_E_INVALID;
  if (layer < 0 || layer >= c->d.n_layers) return fail(c, W4_E_INVALID, "layer out of range");
  int rc = check_rows(c, B, slots);
  if (rc) return rc;
  if (!q || !k_new || !v_new || !o) return fail(c, W4_E_INVALID, "null q, k_new, v_new or o");
  hipStream_t st = (hipStream_t)stream;
  rc = ensure_device(c, st);
  if (rc) return rc;
  rc = poll_errors(c, false);
  if (rc) return rc;
  int max_pos = 0;
  rc = upload_rows(c, B, slots, st, &max_pos);
  if (rc) return rc;
  KV kv = c->kv();
  const int Hq = c->d.n_q_heads, Hkv = c->d.n_kv_heads, D = c->d.head_dim;
  LCHK(c, 1, launch_attention(B, layer, Hq, kv, c->dev_splits(), c->nsplits, static_cast<const uint16_t*>(q),
                              Hq * D, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), Hkv * D,
                              nullptr, c->W<float>(c->wp.part_o), c->W<float>(c->wp.part_ml),
                              c->W<unsigned>(c->wp.aticket), static_cast<uint16_t*>(o), st,
                              c->prof_kernel == W4_K_ATTENTION ? c : nullptr));
  return W4_OK;
}

int w4_layer_step(w4_ctx* c, int32_t layer, int32_t B, const int32_t* slots, void* h, int32_t* route_ids,
                  void* stream) {
  if (!c) return W4_E_INVALID;
  if (layer < 0 || layer >= c->d.n_layers) return fail(c, W4_E_INVALID, "layer out of range");
  int rc = check_rows(c, B, slots);
  if (rc) return rc;
  if (!h) return fail(c, W4_E_INVALID, "null h");
  hipStream_t st = (hipStream_t)stream;
  rc = ensure_device(c, st);
  if (rc) return rc;
  rc = poll_errors(c, false);
  if (rc) return rc;
  int max_pos = 0;
  rc = upload_rows(c, B, slots, st, &max_pos);
  if (rc) return rc;
  uint16_t* hh = static_cast<uint16_t*>(h);
  uint16_t* xp = c->W<uint16_t>(c->wp.xp);
  LCHK(c, 1, launch_rmsnorm(B, c->d.hidden, hh, c->Bk<uint16_t>(c->bp.layers[layer].attn_norm), c->d.rms_eps, xp, st,
                            panel_rows(c->Bm)));
  return layer_body(c, layer, B, max_pos, hh, xp, route_ids, nullptr, st);
}

const char* w4_status_string(int32_t s) {
  switch (s) {
    case W4_OK: return "ok";
    case W4_E_INVALID: return "invalid argument";
    case W4_E_NO_SLOT: return "no free slot";
    case W4_E_CONTEXT_CAP: return "context cap exceeded";
    case W4_E_BAD_SLOT: return "bad slot";
    case W4_E_NOT_READY: return "slot not seeded";
    case W4_E_HIP: return "HIP runtime error";
    case W4_E_UNSUPPORTED: return "unsupported device or size";
    default: return "unknown status";
  }
}

const char* w4_last_error(const w4_ctx* c) { return c ? c->err.c_str() : w4::g_free_err.c_str(); }

int w4_profile_begin(w4_ctx* c, int32_t kernel) {
  if (!c) return W4_E_INVALID;
  if (kernel < W4_K_DENSE || kernel > W4_K_MOE) return fail(c, W4_E_INVALID, "unknown kernel family");
  c->prof_kernel = kernel;
  c->prof_used = 0;
  return W4_OK;
}

int w4_profile_end(w4_ctx* c, double* total_ms, int32_t* launches) {
  if (!c) return W4_E_INVALID;
  double ms = 0;
  const size_t n = c->prof_used / 2;
  if (n) HIPCHK(c, hipEventSynchronize(c->prof_ev[2 * n - 1]));
  for (size_t i = 0; i < n; ++i) {
    float t = 0.f;
    HIPCHK(c, hipEventElapsedTime(&t, c->prof_ev[2 * i], c->prof_ev[2 * i + 1]));
    ms += t;
  }
  c->prof_kernel = 0;
  c->prof_used = 0;
  if (total_ms) *total_ms = ms;
  if (launches) *launches = (int32_t)n;
  return W4_OK;
}

int w4_read_probe(const void* src, size_t bytes, void* sink, int32_t grid, int32_t nontemporal, void* stream) {
  if (!src || !sink || grid < 1 || grid > (1 << 20) || bytes == 0 || bytes % 16 ||
      ((uintptr_t)src % 16) != 0 || (nontemporal != 0 && nontemporal != 1))
    return W4_E_INVALID;
  hipError_t e = launch_read_probe(src, bytes, static_cast<uint32_t*>(sink), grid, nontemporal != 0,
                                   (hipStream_t)stream);
  return e == hipSuccess ? W4_OK : W4_E_HIP;
}

int w4_sync_probe(int32_t mode, int32_t grid, int32_t n, void* scratch, size_t bytes, void* stream) {
  if ((mode != 0 && mode != 1) || !scratch || bytes < kSyncProbeWords * 4 || n < 1 || n > 100000 || grid < 1)
    return W4_E_INVALID;
  if (mode == 0 && grid > sync_probe_max_grid()) return W4_E_INVALID;  // every work-group must be resident
  if (mode == 1 && grid > (1 << 20)) return W4_E_INVALID;
  hipError_t e = launch_sync_probe(mode, grid, n, static_cast<uint32_t*>(scratch), (hipStream_t)stream);
  return e == hipSuccess ? W4_OK : W4_E_HIP;
}

int w4_set_option(w4_ctx* c, int32_t option, int32_t value) {
  if (!c) return W4_E_INVALID;
  switch (option) {
    case W4_OPT_FUSED_MOE:
      if (value != 0 && value != 1) return fail(c, W4_E_INVALID, "W4_OPT_FUSED_MOE takes 0 or 1");
      c->fused_moe = value != 0;
      return W4_OK;
    default:
      return fail(c, W4_E_INVALID, "unknown option");
  }
}

int w4_check_errors(w4_ctx* c) {
  if (!c) return W4_E_INVALID;
  if (!c->dev_ready) return W4_OK;
  return poll_errors(c, true);
}

int w4_last_step_counts(const w4_ctx* c, int32_t* launches, int32_t* syncs) {
  if (!c) return W4_E_INVALID;
  if (launches) *launches = c->last_launches;
  if (syncs) *syncs = c->last_syncs;
  return W4_OK;
}

}  // extern "C"
