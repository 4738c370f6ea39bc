// C ABI of the sink + rolling-KV chunk-attention library: validation, cache layout, host
// bookkeeping (slot table, RoPE base, step protocol) and kernel launches.  See include/sdv2.h.
#include "sdv2.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

using namespace sdv2;

static_assert(SDV2_F32 == kKvF32 && SDV2_BF16 == kKvBF16 && SDV2_BF16_KV_FP8 == kKvFP8,
              "the config dtype codes are the kernels' cache types");

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return SDV2_OK;
}

// Fault injection (sdv2_debug_fail_hip_call): calls left before the one that fails, -1 = off.
std::atomic<int> g_fail_hip{-1};

bool injected_failure() {
  int v = g_fail_hip.load();
  while (v >= 0)
    if (g_fail_hip.compare_exchange_weak(v, v - 1)) return v == 0;
  return false;
}

#define SDV2_HIP(call)                                                                         \
  do {                                                                                         \
    if (injected_failure()) return fail(SDV2_EHIP, "%s: injected failure", #call);            \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess) return fail(SDV2_EHIP, "%s: %s", #call, hipGetErrorString(e_));      \
  } while (0)

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool tau_on(const sdv2_config& c) {
  return !std::isnan(c.sink_threshold) && c.sink_threshold != -INFINITY;
}

// Key scaling: k = -floor(log2(key_scale * log2 e) + 1/2); the bf16 cache stores keys times
// key_scale * log2 e, the e4m3 cache times key_scale * log2 e * 2^k (O(1), keeping e4m3's
// range), with the queries staged times 2^-k.
int key_exponent(double key_scale) {
  return -(int)std::floor(std::log2(key_scale * 1.4426950408889634) + 0.5);
}

float key_factor(const sdv2_config& c) {
  const double ks = c.key_scale * 1.4426950408889634;
  return (float)(c.dtype == SDV2_BF16_KV_FP8 ? std::ldexp(ks, key_exponent(c.key_scale)) : ks);
}

int validate(const sdv2_config* c) {
  if (!c) return fail(SDV2_EINVAL, "config is NULL");
  if (c->num_layers < 1) return fail(SDV2_EINVAL, "num_layers must be >= 1");
  if (c->num_heads < 1) return fail(SDV2_EINVAL, "num_heads must be >= 1");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(SDV2_EINVAL, "head_dim must be 64 or 128");
  if (c->grid_h < 1 || c->grid_w < 1) return fail(SDV2_EINVAL, "grid_h and grid_w must be >= 1");
  if ((int64_t)c->grid_h * c->grid_w > (1 << 20)) return fail(SDV2_EINVAL, "too many tokens per frame");
  if (c->sink_frames < 0 || c->sink_frames > kMaxSinks)
    return fail(SDV2_EINVAL, "sink_frames must be in [0, %d]", kMaxSinks);
  if (c->window_frames < 1) return fail(SDV2_EINVAL, "window_frames must be >= 1");
  if (c->chunk_frames < 1) return fail(SDV2_EINVAL, "chunk_frames must be >= 1");
  if (c->sink_frames + c->window_frames + c->chunk_frames > kMaxShared)
    return fail(SDV2_EINVAL, "sink_frames + window_frames + chunk_frames must be <= %d", kMaxShared);
  if (c->stream_batch < 1 || c->stream_batch > kMaxBatch)
    return fail(SDV2_EINVAL, "stream_batch must be in [1, %d]", kMaxBatch);
  if ((int64_t)c->stream_batch * c->chunk_frames > kMaxBatch)
    return fail(SDV2_EINVAL, "stream_batch * chunk_frames must be <= %d", kMaxBatch);
  if (c->rope_dim_t < 0 || c->rope_dim_h < 0 || c->rope_dim_w < 0 || (c->rope_dim_t & 1) ||
      (c->rope_dim_h & 1) || (c->rope_dim_w & 1))
    return fail(SDV2_EINVAL, "rope dims must be even and >= 0");
  if (c->rope_dim_t + c->rope_dim_h + c->rope_dim_w != c->head_dim)
    return fail(SDV2_EINVAL, "rope dims must sum to head_dim");
  if (c->rope_dim_t / 2 > kMaxTPairs) return fail(SDV2_EINVAL, "rope_dim_t must be <= %d", 2 * kMaxTPairs);
  if (!(c->rope_theta > 1.0) || !std::isfinite(c->rope_theta))
    return fail(SDV2_EINVAL, "rope_theta must be finite and > 1");
  if (c->rope_refresh_period < 0) return fail(SDV2_EINVAL, "rope_refresh_period must be >= 0");
  if (c->dtype != SDV2_F32 && c->dtype != SDV2_BF16 && c->dtype != SDV2_BF16_KV_FP8)
    return fail(SDV2_EINVAL, "dtype must be F32, BF16 or BF16_KV_FP8");
  if (c->dtype == SDV2_BF16_KV_FP8 && c->head_dim != 128)
    return fail(SDV2_EINVAL, "the e4m3 cache needs head_dim 128");
  if (c->embed_dim < 0) return fail(SDV2_EINVAL, "embed_dim must be >= 0");
  if (c->rope_pin_sinks != 0 && c->rope_pin_sinks != 1) return fail(SDV2_EINVAL, "rope_pin_sinks must be 0 or 1");
  if (tau_on(*c) && (c->embed_dim < 1 || c->sink_frames < 1))
    return fail(SDV2_EINVAL, "sink refresh needs embed_dim >= 1 and sink_frames >= 1");
  if (!(c->key_scale >= 0.0) || !std::isfinite(c->key_scale))
    return fail(SDV2_EINVAL, "key_scale must be finite and >= 0");
  if (c->key_scale > 0.0 && (c->dtype == SDV2_F32 || c->head_dim != 128))
    return fail(SDV2_EINVAL, "key_scale > 0 needs a bf16 or e4m3 cache with head_dim 128");
  if (c->dtype == SDV2_BF16_KV_FP8 && !(c->key_scale > 0.0))
    return fail(SDV2_EINVAL, "the e4m3 cache needs key_scale > 0");
  // The attention tile loop forms a tile's byte offset inside a layer's K (or V) block as
  // slot * slot_bytes + tile offset in 32-bit scalar arithmetic, with slot_bytes a signed int.
  const int64_t N = (int64_t)c->grid_h * c->grid_w;
  const int64_t eb = c->dtype == SDV2_F32 ? 4 : c->dtype == SDV2_BF16 ? 2 : 1;
  const int64_t slot_bytes = (int64_t)c->num_heads * ((N + kTileKeys - 1) / kTileKeys * kTileKeys) * c->head_dim * eb;
  const int64_t slots = c->sink_frames + c->window_frames + (int64_t)c->stream_batch * c->chunk_frames;
  if (slot_bytes >= (int64_t)1 << 31)
    return fail(SDV2_EINVAL, "one cache slot (%lld bytes) must be under 2 GiB", (long long)slot_bytes);
  if (slots * slot_bytes >= (int64_t)1 << 32)
    return fail(SDV2_EINVAL, "a layer's K block (%lld slots x %lld bytes) must be under 4 GiB",
                (long long)slots, (long long)slot_bytes);
  return SDV2_OK;
}

sdv2_layout make_layout(const sdv2_config& c) {
  sdv2_layout l;
  const int64_t N = (int64_t)c.grid_h * c.grid_w;
  l.slots = c.sink_frames + c.window_frames + (int64_t)c.stream_batch * c.chunk_frames;
  l.tokens_padded = align_up(N, kTileKeys);
  l.elem_bytes = c.dtype == SDV2_F32 ? 4 : c.dtype == SDV2_BF16 ? 2 : 1;
  l.head_stride = l.tokens_padded * c.head_dim;
  l.slot_stride = c.num_heads * l.head_stride;
  l.layer_stride = 2 * l.slots * l.slot_stride;
  l.kv_elems = c.num_layers * l.layer_stride;
  return l;
}

// Split-KV work plan (WorkPlan in common.h) for nbatch elements.  Each XCD runs its items on its
// 32 CUs, one workgroup per CU at a time, the whole items first.  A plan (whole items per XCD in
// full rounds of 32, the rest split into k key ranges) costs, on the slowest XCD, its rounds x
// (tiles per workgroup x one 64-key tile step + the workgroup's prologue and epilogue), plus
// the bf16 partial results the tail items write and the combine reads back.  The constants are
// measured on MI355X with the 64-row kernel: about 1.5 us per tile step of a 256-row workgroup
// with every CU busy, 8 us of prologue/epilogue per round and ~5 TB/s for the partial traffic.
// A round that leaves CUs idle runs at a higher clock (the chip is power-bound): its tile step
// is shorter by kClockGain x the idle fraction (1.26 us measured at 3/4 occupancy).
constexpr int kCuPerXcd = 32;
constexpr int kMaxSplit = 16;
constexpr double kTileUs = 1.51, kRoundUs = 8.0, kClockGain = 0.66;
constexpr double kPartialBytesPerUs = 5.0e6, kCombineUs = 6.0;

// Rounds of n workgroups of `tiles` tiles each on one XCD.
double xcd_rounds_us(int64_t n, double tiles) {
  const int64_t full = n / kCuPerXcd, part = n % kCuPerXcd;
  double us = (double)full * (tiles * kTileUs + kRoundUs);
  if (part) us += tiles * kTileUs * (1.0 - kClockGain * (1.0 - (double)part / kCuPerXcd)) + kRoundUs;
  return us;
}

// total_tiles: key tiles of the longest query tile; min_tiles: of the shortest (block-causal
// chunks end the walk at a query tile's last own frame), which bounds the split count so that
// every split has at least one tile.  SDV2_NSPLIT=n (tests, tuning) splits every item n ways.
WorkPlan make_plan(const sdv2_config& c, int nbatch, int total_tiles, int min_tiles) {
  const int64_t R = (int64_t)c.chunk_frames * c.grid_h * c.grid_w;   // query rows per element
  const int qtiles = (int)((R + kQTile - 1) / kQTile);
  const int items = nbatch * c.num_heads * qtiles;
  int ix[kNumXcd];
  WorkPlan p{};
  for (int x = 0; x <= kNumXcd; ++x) p.first[x] = (int)((int64_t)x * items / kNumXcd);
  for (int x = 0; x < kNumXcd; ++x) ix[x] = p.first[x + 1] - p.first[x];
  int best_k = 1, best_rounds = 0;
  const char* forced = std::getenv("SDV2_NSPLIT");
  if (c.dtype != SDV2_F32 && forced && std::atoi(forced) > 0) {
    best_k = std::max(1, std::min({std::atoi(forced), kMaxSplit, min_tiles}));
  } else if (c.dtype != SDV2_F32) {
    double best = 1e300;
    // k = 1: every item whole; else whole rounds r (the first r x 32 items of each XCD) and the
    // rest split k ways
    for (int k = 1; k <= kMaxSplit && k <= min_tiles; ++k)
      for (int r = 0; r * kCuPerXcd <= items; ++r) {
        if (k == 1 && r > 0) break;
        double slowest = 0.0;
        int64_t tail_items = 0;
        for (int x = 0; x < kNumXcd; ++x) {
          const int whole = k == 1 ? ix[x] : std::min(ix[x], r * kCuPerXcd);
          const int tail = ix[x] - whole;
          tail_items += tail;
          double us = 0.0;
          if (k == 1) {
            us = xcd_rounds_us(whole, total_tiles);
          } else {
            us = (double)(whole / kCuPerXcd) * (total_tiles * kTileUs + kRoundUs);
            if (whole % kCuPerXcd) us += total_tiles * kTileUs + kRoundUs;   // (r caps whole at full rounds)
            us += xcd_rounds_us((int64_t)tail * k, (double)total_tiles / k);
          }
          slowest = std::max(slowest, us);
        }
        if (k > 1 && tail_items == 0) continue;
        double cost = slowest;
        if (k > 1)
          cost += (double)k * tail_items * kQTile * (2.0 * (c.head_dim * 2 + 8)) / kPartialBytesPerUs + kCombineUs;
        if (cost < best * 0.98) {   // prefer fewer splits unless clearly cheaper
          best = cost;
          best_k = k;
          best_rounds = r;
        }
      }
  }
  p.nsplit = best_k;
  int tail_total = 0;
  for (int x = 0; x < kNumXcd; ++x) {
    p.whole[x] = best_k == 1 ? ix[x] : std::min(ix[x], best_rounds * kCuPerXcd);
    p.tail_first[x] = tail_total;
    tail_total += ix[x] - p.whole[x];
  }
  p.tail_first[kNumXcd] = tail_total;
  if (tail_total == 0) p.nsplit = 1;
  p.wg_per_xcd = 0;
  for (int x = 0; x < kNumXcd; ++x)
    p.wg_per_xcd = std::max(p.wg_per_xcd, p.whole[x] + (ix[x] - p.whole[x]) * p.nsplit);
  return p;
}

// Bytes of the split-KV partials of a plan.
int64_t plan_partial_bytes(const WorkPlan& p, int head_dim, int64_t* o_bytes) {
  const int64_t rows = (int64_t)p.nsplit * p.tail_first[kNumXcd] * kQTile;
  const int64_t ob = align_up(rows * head_dim * 2, 256);
  if (o_bytes) *o_bytes = ob;
  return p.tail_first[kNumXcd] ? ob + align_up(rows * 8, 256) : 0;
}

struct MetaLayout {
  int64_t tab_h, tab_w, embeds, decision, alpha, stats_part, total;
};

MetaLayout meta_layout(const sdv2_config& c) {
  MetaLayout m;
  int64_t off = 0;
  m.tab_h = off;
  off = align_up(off + (int64_t)c.grid_h * (c.rope_dim_h / 2) * 8, kAlign);
  m.tab_w = off;
  off = align_up(off + (int64_t)c.grid_w * (c.rope_dim_w / 2) * 8, kAlign);
  m.embeds = off;
  off = align_up(off + (int64_t)c.sink_frames * c.embed_dim * 4, kAlign);
  m.decision = off;
  off = align_up(off + 16, kAlign);
  m.alpha = off;
  off = align_up(off + 16, kAlign);
  m.stats_part = off;                  // partial sums of the fused chunk-statistics pass
  off = align_up(off + (int64_t)kStatsMaxBlocks * kStatsQ * 8, kAlign);
  m.total = off;
  return m;
}

int64_t workspace_bytes(const sdv2_config& c) {
  const int64_t N = (int64_t)c.grid_h * c.grid_w;
  const int tpf = (int)(align_up(N, kTileKeys) / kTileKeys);
  int64_t best = 0;
  // every (nbatch, shared frames present) the stream can reach, warm-up included
  for (int nb = 1; nb <= c.stream_batch; ++nb)
    for (int shared = 0; shared <= c.sink_frames + c.window_frames; ++shared) {
      const WorkPlan p = make_plan(c, nb, (shared + c.chunk_frames) * tpf, (shared + 1) * tpf);
      best = std::max(best, plan_partial_bytes(p, c.head_dim, nullptr));
    }
  return best;
}

// omega_i = theta^(-2i / dim_axis)
double omega(double theta, int i, int dim_axis) { return std::pow(theta, -2.0 * i / dim_axis); }

enum State { kIdle = 0, kStep = 1, kCommitted = 2 };

}  // namespace

struct sdv2_cache {
  sdv2_config cfg;
  sdv2_layout lay;
  MetaLayout meta;
  char* kv;
  char* meta_base;
  char* ws;
  int64_t ws_bytes;
  int64_t N;
  // bookkeeping
  int64_t base = 0;            // RoPE base b0
  int64_t committed = 0;       // chunks committed
  int64_t refreshes = 0;
  std::vector<int64_t> slot_frame;   // per slot; -1 empty, -2 unknown
  std::vector<int64_t> slot_label;
  std::vector<uint8_t> slot_written; // slot holds a committed frame (shared slots only)
  bool sinks_unknown = false;
  // step protocol
  int state = kIdle;
  bool started = false;
  int64_t newest = -1;
  int64_t step_first = -1;
  int32_t step_nbatch = 0;
  std::vector<uint8_t> appended;
  int64_t last_commit_frame = -1;
};

namespace {

int check_cache(const sdv2_cache* c) {
  if (!c) return fail(SDV2_EINVAL, "cache is NULL");
  return SDV2_OK;
}

// Slot of frame f once committed: sink slot f for f < S, else one of W + T' ring slots.  The
// ring holds T' slots more than the window: the slots of the chunk being finished hold frames
// that already left the window, so the append writes element 0 to its final slots and the
// commit moves no data.
int home_slot(const sdv2_config& c, int64_t f) {
  return f < c.sink_frames ? (int)f
                           : c.sink_frames + (int)(f % (c.window_frames + c.chunk_frames));
}

// Sinks and ring slots; the staging slots of elements 1..B-1 follow.
int shared_region(const sdv2_config& c) {
  return c.sink_frames + c.window_frames + c.chunk_frames;
}

// Slot of frame t of element b's chunk at a step whose element 0 holds chunk `first`.
int chunk_slot(const sdv2_config& c, int64_t first, int b, int t) {
  return b == 0 ? home_slot(c, first * c.chunk_frames + t)
                : c.sink_frames + c.window_frames + b * c.chunk_frames + t;
}

// Present shared slots in attention order: sinks by slot index, then the ring by slot index.
int shared_slots(const sdv2_cache* c, int* out) {
  int n = 0;
  const int R = shared_region(c->cfg);
  for (int s = 0; s < R; ++s)
    if (c->slot_written[s]) out[n++] = s;
  return n;
}

// One attention call; split-KV partial results go to ws (ws_bytes long).
int attention_call(sdv2_cache* c, int32_t layer, int32_t nbatch, const void* d_q_rot, void* d_out,
                   float scale, void* stream, char* ws, int64_t ws_bytes, const char* ws_name) {
  const sdv2_config& cfg = c->cfg;
  if (c->state != kStep) return fail(SDV2_ESTATE, "attention outside a step or after the commit");
  if (layer < 0 || layer >= cfg.num_layers) return fail(SDV2_EINVAL, "layer %d out of range", layer);
  if (!c->appended[layer]) return fail(SDV2_ESTATE, "layer %d not appended this step", layer);
  if (nbatch != c->step_nbatch) return fail(SDV2_EINVAL, "nbatch %d differs from the append's %d", nbatch, c->step_nbatch);
  if (!d_q_rot || !d_out) return fail(SDV2_EINVAL, "q_rot and out must not be NULL");
  if (((uintptr_t)d_q_rot | (uintptr_t)d_out) & 15) return fail(SDV2_EINVAL, "q_rot and out must be 16-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SDV2_EINVAL, "scale must be finite and > 0");
  if (cfg.key_scale > 0.0 && scale != (float)cfg.key_scale)
    return fail(SDV2_EINVAL, "scale %g differs from the cache's key_scale %g", (double)scale, cfg.key_scale);

  AttnArgs a{};
  a.q = d_q_rot;
  a.out = d_out;
  a.kv = c->kv;
  a.k_layer_off = layer * c->lay.layer_stride;
  a.v_layer_off = a.k_layer_off + c->lay.slots * c->lay.slot_stride;
  a.slot_stride = c->lay.slot_stride;
  a.head_stride = c->lay.head_stride;
  a.N = (int)c->N;
  a.Npad = (int)c->lay.tokens_padded;
  a.H = cfg.num_heads;
  a.nbatch = nbatch;
  a.nshared = shared_slots(c, a.slots);
  const int Tc = cfg.chunk_frames;
  a.T = Tc;
  for (int b = 0; b < nbatch; ++b)
    for (int t = 0; t < Tc; ++t) a.own_slot[b * Tc + t] = chunk_slot(cfg, c->step_first, b, t);
  a.tiles_per_frame = (int)(c->lay.tokens_padded / kTileKeys);
  a.total_tiles = (a.nshared + Tc) * a.tiles_per_frame;
  a.plan = make_plan(cfg, nbatch, a.total_tiles, (a.nshared + 1) * a.tiles_per_frame);
  a.qtiles = (int)((Tc * c->N + kQTile - 1) / kQTile);
  a.scale = scale;
  // keys cached times scale * log2(e) (e4m3: times 2^k more, queries staged times 2^-k): the
  // scores are the exponent already
  a.scaled_keys = cfg.key_scale > 0.0;
  a.qmul = cfg.dtype == SDV2_BF16_KV_FP8 ? std::ldexp(1.0f, -key_exponent(cfg.key_scale)) : 1.0f;
  a.scale_log2 = a.scaled_keys ? 1.0f : (float)((double)scale * 1.4426950408889634);
  a.scale_log2_inv = 1.0f / a.scale_log2;
  a.neg_bias = -8.0f / a.scale_log2;
  if (cfg.dtype != SDV2_F32 && a.plan.nsplit > 1) {
    int64_t ob = 0;
    const int64_t need = plan_partial_bytes(a.plan, cfg.head_dim, &ob);
    if (need > ws_bytes)
      return fail(SDV2_ENOSPC, "%s of %lld bytes is too small for %d splits of %d query tiles (%lld bytes)",
                  ws_name, (long long)ws_bytes, a.plan.nsplit, a.plan.tail_first[kNumXcd], (long long)need);
    a.part_o = (uint16_t*)ws;
    a.part_ml = (float2*)(ws + ob);
  }
  SDV2_HIP(launch_attention(a, cfg.head_dim, cfg.dtype, (hipStream_t)stream));
  if (cfg.dtype != SDV2_F32 && a.plan.nsplit > 1) {
    CombineArgs m{a.part_o, a.part_ml, d_out, (int)(Tc * c->N), a.H, nbatch, a.qtiles, a.plan};
    SDV2_HIP(launch_combine(m, cfg.head_dim, (hipStream_t)stream));
  }
  return ok();
}

// Split-KV partials of sdv2_chunk_attention_static: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never uses the array's name as an address: its
// device address is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept.
constexpr int64_t kStaticScratchBytes = SDV2_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
std::vector<char*> g_scratch_ptr;   // per device ordinal; nullptr until looked up

int static_scratch(char** out) {
  int dev = 0;
  SDV2_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    SDV2_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return SDV2_OK;
}

}  // namespace

extern "C" {

int sdv2_config_validate(const sdv2_config* cfg) {
  const int rc = validate(cfg);
  return rc ? rc : ok();
}

int sdv2_cache_layout(const sdv2_config* cfg, sdv2_layout* out) {
  if (int rc = validate(cfg)) return rc;
  if (!out) return fail(SDV2_EINVAL, "out is NULL");
  *out = make_layout(*cfg);
  return ok();
}

int sdv2_cache_size(const sdv2_config* cfg, size_t* kv_bytes, size_t* meta_bytes,
                    size_t* workspace) {
  if (int rc = validate(cfg)) return rc;
  const sdv2_layout l = make_layout(*cfg);
  if (kv_bytes) *kv_bytes = (size_t)(l.kv_elems * l.elem_bytes);
  if (meta_bytes) *meta_bytes = (size_t)meta_layout(*cfg).total;
  if (workspace) *workspace = (size_t)workspace_bytes(*cfg);
  return ok();
}

int sdv2_cache_create(const sdv2_config* cfg, void* d_kv, size_t kv_bytes, void* d_meta,
                      size_t meta_bytes, void* d_workspace, size_t ws_bytes, void* stream,
                      sdv2_cache** out) {
  if (int rc = validate(cfg)) return rc;
  if (!out) return fail(SDV2_EINVAL, "out is NULL");
  size_t need_kv, need_meta, need_ws;
  sdv2_cache_size(cfg, &need_kv, &need_meta, &need_ws);
  if (!d_kv || !d_meta) return fail(SDV2_EINVAL, "d_kv and d_meta must not be NULL");
  if (need_ws && !d_workspace) return fail(SDV2_EINVAL, "d_workspace must not be NULL");
  if (((uintptr_t)d_kv | (uintptr_t)d_meta | (uintptr_t)d_workspace) % kAlign)
    return fail(SDV2_EINVAL, "device buffers must be 256-byte aligned");
  if (kv_bytes < need_kv) return fail(SDV2_ENOSPC, "kv buffer %zu < %zu bytes", kv_bytes, need_kv);
  if (meta_bytes < need_meta) return fail(SDV2_ENOSPC, "meta buffer %zu < %zu bytes", meta_bytes, need_meta);
  if (ws_bytes < need_ws) return fail(SDV2_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, need_ws);

  const sdv2_config& c = *cfg;
  const MetaLayout ml = meta_layout(c);
  // h / w RoPE tables: (cos, sin) of pos * omega, computed in double, stored as fp32
  std::vector<char> host(ml.total, 0);
  float2* th = (float2*)(host.data() + ml.tab_h);
  float2* tw = (float2*)(host.data() + ml.tab_w);
  const int ph = c.rope_dim_h / 2, pw = c.rope_dim_w / 2;
  for (int h = 0; h < c.grid_h; ++h)
    for (int i = 0; i < ph; ++i) {
      const double ang = h * omega(c.rope_theta, i, c.rope_dim_h);
      th[h * ph + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  for (int w = 0; w < c.grid_w; ++w)
    for (int i = 0; i < pw; ++i) {
      const double ang = w * omega(c.rope_theta, i, c.rope_dim_w);
      tw[w * pw + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  *(int32_t*)(host.data() + ml.decision) = -1;

  hipStream_t s = (hipStream_t)stream;
  SDV2_HIP(hipMemsetAsync(d_kv, 0, need_kv, s));
  SDV2_HIP(hipMemcpyAsync(d_meta, host.data(), ml.total, hipMemcpyHostToDevice, s));
  SDV2_HIP(hipStreamSynchronize(s));

  sdv2_cache* cache = new sdv2_cache();
  cache->cfg = c;
  cache->lay = make_layout(c);
  cache->meta = ml;
  cache->kv = (char*)d_kv;
  cache->meta_base = (char*)d_meta;
  cache->ws = (char*)d_workspace;
  cache->ws_bytes = (int64_t)ws_bytes;
  cache->N = (int64_t)c.grid_h * c.grid_w;
  cache->slot_frame.assign(cache->lay.slots, -1);
  cache->slot_label.assign(cache->lay.slots, 0);
  cache->slot_written.assign(cache->lay.slots, 0);
  cache->appended.assign(c.num_layers, 0);
  *out = cache;
  return ok();
}

int sdv2_cache_destroy(sdv2_cache* cache) {
  delete cache;
  return ok();
}

int sdv2_rope_refresh(sdv2_cache* c, int64_t newest_frame, int32_t* applied, void* stream) {
  if (int rc = check_cache(c)) return rc;
  if (newest_frame < 0) return fail(SDV2_EINVAL, "newest_frame must be >= 0");
  if (c->started && newest_frame < c->newest)
    return fail(SDV2_ESTATE, "newest_frame %lld is older than the previous step's %lld",
                (long long)newest_frame, (long long)c->newest);
  if (newest_frame < c->committed * c->cfg.chunk_frames)
    return fail(SDV2_ESTATE, "newest_frame %lld is already committed", (long long)newest_frame);
  const sdv2_config& cfg = c->cfg;
  const int64_t T = cfg.rope_refresh_period;
  int64_t count = 0;
  if (T > 0 && newest_frame - c->base >= T) count = (newest_frame - c->base) / T;
  if (count > 0) {
    // every attended slot, or only the window when the sinks are pinned
    int all[kMaxShared], slots[kMaxShared], ns = 0;
    const int na = shared_slots(c, all);
    for (int i = 0; i < na; ++i)
      if (!cfg.rope_pin_sinks || all[i] >= cfg.sink_frames) slots[ns++] = all[i];
    if (ns > 0 && cfg.rope_dim_t > 0) {
      RebaseArgs a{};
      a.kv = c->kv;
      a.layer_stride = c->lay.layer_stride;
      a.slot_stride = c->lay.slot_stride;
      a.head_stride = c->lay.head_stride;
      a.L = cfg.num_layers;
      a.H = cfg.num_heads;
      a.N = (int)c->N;
      a.pt = cfg.rope_dim_t / 2;
      a.nslots = ns;
      // 16-byte chunks of a key row that hold the temporal dims 0 .. 2 pt - 1 (e4m3: at their
      // permuted byte positions)
      const int per_chunk = 16 / (int)c->lay.elem_bytes;
      int last = 2 * a.pt - 1;
      if (cfg.dtype == SDV2_BF16_KV_FP8)
        for (int d = 0; d < 2 * a.pt; ++d) last = std::max(last, fp8_pos(d));
      a.cpr = last / per_chunk + 1;
      // whole 128-byte lines of the row (the chunks past the temporal dims are written back
      // unchanged): a write of part of a line makes the memory read the rest of it
      a.cpr = std::min(cfg.head_dim * (int)c->lay.elem_bytes / 16, (a.cpr + 7) / 8 * 8);
      for (int i = 0; i < ns; ++i) a.slots[i] = slots[i];
      const double delta = (double)(count * T);
      for (int i = 0; i < a.pt; ++i) {
        const double ang = -delta * omega(cfg.rope_theta, i, cfg.rope_dim_t);
        a.cs[i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
      }
      SDV2_HIP(launch_rebase(a, cfg.head_dim, cfg.dtype, (hipStream_t)stream));
    }
    c->base += count * T;
    c->refreshes += count;
    for (int s = cfg.rope_pin_sinks ? cfg.sink_frames : 0; s < shared_region(cfg); ++s)
      if (c->slot_written[s]) c->slot_label[s] -= count * T;
  }
  c->started = true;
  c->newest = newest_frame;
  c->state = kStep;
  c->step_first = -1;
  c->step_nbatch = 0;
  std::fill(c->appended.begin(), c->appended.end(), 0);
  // staging slots hold nothing committed-visible until the appends of this step
  for (int64_t s = shared_region(cfg); s < c->lay.slots; ++s) c->slot_frame[s] = -1;
  if (applied) *applied = (int32_t)count;
  return ok();
}

int sdv2_cache_append(sdv2_cache* c, int32_t layer, int64_t first_chunk, int32_t nbatch,
                      void* d_q, const void* d_k, const void* d_v, void* stream) {
  if (int rc = check_cache(c)) return rc;
  const sdv2_config& cfg = c->cfg;
  if (c->state != kStep) return fail(SDV2_ESTATE, "append outside a step (call sdv2_rope_refresh first)");
  if (layer < 0 || layer >= cfg.num_layers) return fail(SDV2_EINVAL, "layer %d out of range", layer);
  if (nbatch < 1 || nbatch > cfg.stream_batch)
    return fail(SDV2_EINVAL, "nbatch must be in [1, %d]", cfg.stream_batch);
  if (!d_q || !d_k || !d_v) return fail(SDV2_EINVAL, "q, k and v must not be NULL");
  if (((uintptr_t)d_q | (uintptr_t)d_k | (uintptr_t)d_v) & 15)
    return fail(SDV2_EINVAL, "q, k and v must be 16-byte aligned");
  if (first_chunk != c->committed)
    return fail(SDV2_ESTATE, "first_chunk %lld must equal the committed count %lld",
                (long long)first_chunk, (long long)c->committed);
  const int Tc = cfg.chunk_frames;
  if ((first_chunk + nbatch) * Tc - 1 != c->newest)
    return fail(SDV2_ESTATE, "newest chunk's last frame %lld differs from the step's newest frame %lld",
                (long long)((first_chunk + nbatch) * Tc - 1), (long long)c->newest);
  if (c->step_nbatch != 0 && (c->step_nbatch != nbatch || c->step_first != first_chunk))
    return fail(SDV2_ESTATE, "nbatch/first_chunk differ between layers of one step");
  if (c->appended[layer]) return fail(SDV2_ESTATE, "layer %d already appended this step", layer);

  AppendArgs a{};
  a.q = d_q;
  a.k = d_k;
  a.v = d_v;
  a.kv = c->kv;
  a.k_layer_off = layer * c->lay.layer_stride;
  a.v_layer_off = a.k_layer_off + c->lay.slots * c->lay.slot_stride;
  a.slot_stride = c->lay.slot_stride;
  a.head_stride = c->lay.head_stride;
  a.tab_h = (const float2*)(c->meta_base + c->meta.tab_h);
  a.tab_w = (const float2*)(c->meta_base + c->meta.tab_w);
  a.N = (int)c->N;
  a.Npad = (int)c->lay.tokens_padded;
  a.H = cfg.num_heads;
  a.grid_w = cfg.grid_w;
  a.nbatch = nbatch;
  a.T = Tc;
  // element 0 goes to the slots its frames keep once committed, the others to staging slots
  for (int b = 0; b < nbatch; ++b)
    for (int t = 0; t < Tc; ++t) a.dst_slot[b * Tc + t] = chunk_slot(cfg, first_chunk, b, t);
  for (int t = 0; t < Tc; ++t)
    if (c->slot_written[a.dst_slot[t]])
      return fail(SDV2_ESTATE, "internal: slot %d of chunk %lld is still attended", a.dst_slot[t],
                  (long long)first_chunk);
  a.pt = cfg.rope_dim_t / 2;
  a.ph = cfg.rope_dim_h / 2;
  a.pw = cfg.rope_dim_w / 2;
  a.kmul = cfg.key_scale > 0.0 ? key_factor(cfg) : 1.0f;
  for (int b = 0; b < nbatch; ++b)
    for (int t = 0; t < Tc; ++t) {
      const double p = (double)((first_chunk + b) * Tc + t - c->base);   // position f - b0
      for (int i = 0; i < a.pt; ++i) {
        const double ang = p * omega(cfg.rope_theta, i, cfg.rope_dim_t);
        a.tcs[b * Tc + t][i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
      }
    }
  SDV2_HIP(launch_rope_append(a, cfg.head_dim, cfg.dtype, (hipStream_t)stream));
  c->appended[layer] = 1;
  c->step_first = first_chunk;
  c->step_nbatch = nbatch;
  for (int b = 0; b < nbatch; ++b)
    for (int t = 0; t < Tc; ++t) {
      const int64_t f = (first_chunk + b) * Tc + t;
      c->slot_frame[a.dst_slot[b * Tc + t]] = f;
      c->slot_label[a.dst_slot[b * Tc + t]] = f - c->base;
    }
  return ok();
}

int sdv2_chunk_attention(sdv2_cache* c, int32_t layer, int32_t nbatch, const void* d_q_rot,
                         void* d_out, float scale, void* stream) {
  if (int rc = check_cache(c)) return rc;
  return attention_call(c, layer, nbatch, d_q_rot, d_out, scale, stream, c->ws, c->ws_bytes, "workspace");
}

int sdv2_chunk_attention_static(sdv2_cache* c, int32_t layer, int32_t nbatch, const void* d_q_rot,
                                void* d_out, float scale, void* stream) {
  if (int rc = check_cache(c)) return rc;
  char* ptr = nullptr;
  if (int rc = static_scratch(&ptr)) return rc;
  return attention_call(c, layer, nbatch, d_q_rot, d_out, scale, stream, ptr, kStaticScratchBytes,
                        "static scratch");
}

int sdv2_cache_commit(sdv2_cache* c, int64_t chunk, void* stream) {
  if (int rc = check_cache(c)) return rc;
  const sdv2_config& cfg = c->cfg;
  if (c->state != kStep) return fail(SDV2_ESTATE, "commit outside a step or twice in one step");
  for (int l = 0; l < cfg.num_layers; ++l)
    if (!c->appended[l]) return fail(SDV2_ESTATE, "layer %d not appended this step", l);
  if (chunk != c->step_first) return fail(SDV2_ESTATE, "only element 0 (chunk %lld) can be committed", (long long)c->step_first);
  (void)stream;              // the appends already wrote the frames to their slots
  const int S = cfg.sink_frames, W = cfg.window_frames, Tc = cfg.chunk_frames;
  for (int t = 0; t < Tc; ++t) {
    const int64_t f = chunk * Tc + t;
    if (f - W >= S) {        // frame f - W leaves the window
      const int old = home_slot(cfg, f - W);
      c->slot_written[old] = 0;
      c->slot_frame[old] = -1;
    }
    const int dst = home_slot(cfg, f);
    c->slot_frame[dst] = f;
    c->slot_label[dst] = f - c->base;
    c->slot_written[dst] = 1;
  }
  c->committed = chunk + 1;
  c->last_commit_frame = (chunk + 1) * Tc - 1;
  c->state = kCommitted;
  return ok();
}

int sdv2_sink_replace(sdv2_cache* c, int64_t frame, const float* d_embed, const float* d_prev_latent,
                      const float* d_cur_latent, int64_t latent_elems, double* d_stats, int32_t* h_slot,
                      double* h_alpha, void* stream) {
  if (int rc = check_cache(c)) return rc;
  const sdv2_config& cfg = c->cfg;
  if (c->state != kCommitted) return fail(SDV2_ESTATE, "sink_replace must follow a commit");
  if (frame != c->last_commit_frame) return fail(SDV2_ESTATE, "frame %lld is not the committed frame %lld",
                                                  (long long)frame, (long long)c->last_commit_frame);
  if (cfg.embed_dim < 1 && d_embed) return fail(SDV2_EINVAL, "the cache has no chunk embeddings (embed_dim 0)");
  if (cfg.embed_dim >= 1 && !d_embed) return fail(SDV2_EINVAL, "d_embed must not be NULL (embed_dim %d)", cfg.embed_dim);
  if ((d_prev_latent == nullptr) != (d_cur_latent == nullptr))
    return fail(SDV2_EINVAL, "give both latent frames or neither");
  const bool motion = d_cur_latent != nullptr;
  if (motion && latent_elems < 1) return fail(SDV2_EINVAL, "latent_elems must be >= 1");
  if (motion && latent_elems > ((int64_t)1 << 40)) return fail(SDV2_EINVAL, "latent_elems too large");
  if (motion && (((uintptr_t)d_prev_latent | (uintptr_t)d_cur_latent) & 3))
    return fail(SDV2_EINVAL, "latent frames must be 4-byte aligned");
  if ((uintptr_t)d_embed & 3) return fail(SDV2_EINVAL, "d_embed must be 4-byte aligned");
  if ((uintptr_t)d_stats & 7) return fail(SDV2_EINVAL, "d_stats must be 8-byte aligned");
  const int S = cfg.sink_frames, D = d_embed ? cfg.embed_dim : 0;
  const int64_t n_lat = motion ? latent_elems : 0;
  // the chunk's frames below S became sinks: h is their embedding
  const int64_t first = frame - cfg.chunk_frames + 1;
  const int store_lo = (int)std::min<int64_t>(first, S), store_hi = (int)std::min<int64_t>(frame + 1, S);
  const bool decide = frame >= S && tau_on(cfg);
  hipStream_t s = (hipStream_t)stream;
  int32_t* decision = (int32_t*)(c->meta_base + c->meta.decision);
  double* alpha_dev = (double*)(c->meta_base + c->meta.alpha);
  if (D > 0 || motion || d_stats) {
    // pass 1: enough blocks for both reductions, each block at least 8192 latent or 1024
    // embedding elements (a fixed split for a given size, so results repeat bit for bit)
    int64_t blocks = std::max<int64_t>({1, (n_lat + kStatsLatPerBlock - 1) / kStatsLatPerBlock,
                                        ((int64_t)D + kStatsEmbPerBlock - 1) / kStatsEmbPerBlock});
    blocks = std::min<int64_t>(blocks, kStatsMaxBlocks);
    StatsArgs st{};
    st.prev = d_prev_latent;
    st.cur = d_cur_latent;
    st.n_lat = n_lat;
    st.lat_per_block = align_up((n_lat + blocks - 1) / blocks, 4);
    st.h = d_embed;
    st.embeds = (const float*)(c->meta_base + c->meta.embeds);
    st.S = D > 0 ? S : 0;
    st.D = D;
    st.emb_per_block = (int)((D + blocks - 1) / blocks);
    st.part = (double*)(c->meta_base + c->meta.stats_part);
    SDV2_HIP(launch_chunk_stats(st, (int)blocks, s));
    // pass 2: statistics, decision, embedding stores
    SinkArgs a{};
    a.part = st.part;
    a.blocks = (int)blocks;
    a.n_lat = n_lat;
    a.h = d_embed;
    a.embeds = (float*)(c->meta_base + c->meta.embeds);
    a.S = S;                           // the statistics hold 4 + 2S values
    a.D = D;
    a.store_lo = D > 0 ? store_lo : 0;
    a.store_hi = D > 0 ? store_hi : 0;
    a.decide = decide ? 1 : 0;
    a.tau = cfg.sink_threshold;
    a.decision = decision;
    a.alpha = alpha_dev;
    a.stats = d_stats;
    SDV2_HIP(launch_sink_decide(a, s));
  }
  if (decide) {
    CopyArgs cp{};
    cp.kv = c->kv;
    cp.layer_stride_bytes = c->lay.layer_stride * c->lay.elem_bytes;
    cp.v_block_bytes = c->lay.slots * c->lay.slot_stride * c->lay.elem_bytes;
    cp.slot_bytes = c->lay.slot_stride * c->lay.elem_bytes;
    cp.src_slot = home_slot(cfg, frame);
    cp.dst_slot = -1;
    cp.dst_from = decision;
    cp.L = cfg.num_layers;
    SDV2_HIP(launch_copy_slots(cp, s));
  }
  int32_t slot = -1;
  double alpha = 1.0;
  if (decide && h_slot) {
    SDV2_HIP(hipMemcpyAsync(&slot, decision, sizeof(slot), hipMemcpyDeviceToHost, s));
    SDV2_HIP(hipMemcpyAsync(&alpha, alpha_dev, sizeof(alpha), hipMemcpyDeviceToHost, s));
    SDV2_HIP(hipStreamSynchronize(s));
    if (slot >= 0) {
      c->slot_frame[slot] = frame;
      c->slot_label[slot] = c->slot_label[home_slot(cfg, frame)];
    }
  } else if (decide) {
    c->sinks_unknown = true;
  }
  if (h_slot) *h_slot = slot;
  if (h_alpha) *h_alpha = alpha;
  c->state = kIdle;
  return ok();
}

int sdv2_motion_workspace_size(int32_t nframes, int64_t elems_per_frame, size_t* bytes) {
  if (nframes < 2) return fail(SDV2_EINVAL, "nframes must be >= 2");
  if (elems_per_frame < 1) return fail(SDV2_EINVAL, "elems_per_frame must be >= 1");
  if (!bytes) return fail(SDV2_EINVAL, "bytes is NULL");
  *bytes = (size_t)(nframes - 1) * motion_parts(elems_per_frame) * sizeof(double);
  return ok();
}

int sdv2_motion_l2(const float* d_frames, int32_t nframes, int64_t elems_per_frame, double* d_dist,
                   void* d_workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  if (int rc = sdv2_motion_workspace_size(nframes, elems_per_frame, &need)) return rc;
  if (!d_frames || !d_dist || !d_workspace) return fail(SDV2_EINVAL, "frames, dist and workspace must not be NULL");
  if (workspace_bytes < need) return fail(SDV2_ENOSPC, "motion workspace %zu < %zu bytes", workspace_bytes, need);
  if (nframes - 1 > 65535) return fail(SDV2_EINVAL, "at most 65536 frames per call");
  if (((uintptr_t)d_dist | (uintptr_t)d_workspace) & 7) return fail(SDV2_EINVAL, "dist and workspace must be 8-byte aligned");
  if ((uintptr_t)d_frames & 3) return fail(SDV2_EINVAL, "frames must be 4-byte aligned");
  SDV2_HIP(launch_motion(d_frames, nframes, elems_per_frame, d_dist, (double*)d_workspace,
                         motion_parts(elems_per_frame), (hipStream_t)stream));
  return ok();
}

int sdv2_noise_schedule(const double* h_dist, int32_t n, double sigma, int32_t k, double lambda,
                        double s_min, double s_max, double s0, double* h_rate) {
  if (n < 0 || (n > 0 && (!h_dist || !h_rate))) return fail(SDV2_EINVAL, "bad distance/rate arrays");
  if (!(sigma > 0.0) || k < 1) return fail(SDV2_EINVAL, "sigma must be > 0 and k >= 1");
  if (!(lambda > 0.0 && lambda <= 1.0)) return fail(SDV2_EINVAL, "lambda must be in (0, 1]");
  double s = s0;
  for (int32_t t = 0; t < n; ++t) {
    double m = 0.0;
    for (int32_t i = (t - k + 1 > 0 ? t - k + 1 : 0); i <= t; ++i) m = h_dist[i] > m ? h_dist[i] : m;
    const double dhat = m / sigma < 1.0 ? m / sigma : 1.0;
    const double target = s_max - (s_max - s_min) * dhat;
    s = lambda * target + (1.0 - lambda) * s;
    h_rate[t] = s;
  }
  return ok();
}

int sdv2_latency_fit(const int32_t* h_frames, const double* h_latency_s, int32_t n, double* c0,
                     double* c1) {
  if (n < 2 || !h_frames || !h_latency_s || !c0 || !c1)
    return fail(SDV2_EINVAL, "need n >= 2 measurements and non-NULL arrays");
  double mx = 0.0, my = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    mx += h_frames[i];
    my += h_latency_s[i];
  }
  mx /= n;
  my /= n;
  double sxx = 0.0, sxy = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    const double dx = h_frames[i] - mx;
    sxx += dx * dx;
    sxy += dx * (h_latency_s[i] - my);
  }
  if (!(sxx > 0.0)) return fail(SDV2_EINVAL, "the measurements need at least two distinct frame counts");
  *c1 = sxy / sxx;
  *c0 = my - *c1 * mx;
  return ok();
}

int sdv2_slo_select(double c0, double c1, double target_fps, double deadline_s, int32_t frames_ready,
                    int32_t max_batch, int32_t max_chunk, int32_t* B, int32_t* T, double* fps,
                    double* latency_s, int32_t* feasible) {
  if (!B || !T) return fail(SDV2_EINVAL, "B and T must not be NULL");
  if (!(target_fps > 0.0)) return fail(SDV2_EINVAL, "target_fps must be > 0");
  const int32_t cap = frames_ready < kMaxBatch ? frames_ready : kMaxBatch;
  struct Cand { int b, t; double f, lat; };
  Cand best{0, 0, 0.0, 0.0}, best_any{0, 0, 0.0, 0.0};
  bool have = false, have_any = false;
  auto better = [](const Cand& c, const Cand& ref) {
    if (c.f > ref.f * (1.0 + 1e-12)) return true;
    if (c.f < ref.f * (1.0 - 1e-12)) return false;
    return c.lat < ref.lat || (c.lat == ref.lat && c.b < ref.b);
  };
  for (int b = 1; b <= max_batch; ++b)
    for (int t = 1; t <= max_chunk; ++t) {
      if (b * t > cap) continue;
      const double L = c0 + c1 * b * t;
      if (!(L > 0.0)) return fail(SDV2_EINVAL, "latency model gives L <= 0 at B*T' = %d", b * t);
      const Cand c{b, t, b * t / L, b * L + (t - 1) / target_fps};
      if (!have_any || better(c, best_any)) best_any = c, have_any = true;
      if (c.f >= target_fps && c.lat <= deadline_s && (!have || better(c, best))) best = c, have = true;
    }
  if (!have_any) return fail(SDV2_EINVAL, "no (B, T') candidate: check frames_ready, max_batch, max_chunk");
  const Cand& r = have ? best : best_any;
  *B = r.b;
  *T = r.t;
  if (fps) *fps = r.f;
  if (latency_s) *latency_s = r.lat;
  if (feasible) *feasible = have ? 1 : 0;
  return ok();
}

int sdv2_cache_slot_info(const sdv2_cache* c, int32_t slot, int64_t* frame, int32_t* tpos) {
  if (int rc = check_cache(c)) return rc;
  if (slot < 0 || slot >= c->lay.slots) return fail(SDV2_EINVAL, "slot %d out of range", slot);
  int64_t f = c->slot_frame[slot];
  int64_t p = c->slot_label[slot];
  if (c->sinks_unknown && slot < c->cfg.sink_frames && f >= 0) f = -2;
  if (frame) *frame = f;
  if (tpos) *tpos = (int32_t)p;
  return ok();
}

int sdv2_cache_state(const sdv2_cache* c, int64_t* rope_base, int64_t* committed, int64_t* refreshes) {
  if (int rc = check_cache(c)) return rc;
  if (rope_base) *rope_base = c->base;
  if (committed) *committed = c->committed;
  if (refreshes) *refreshes = c->refreshes;
  return ok();
}

int sdv2_plan_step(const sdv2_config* cfg, int64_t num_chunks, int64_t step, int64_t* first_chunk,
                   int32_t* nbatch, int64_t* commit_chunk, int64_t* newest_frame) {
  if (int rc = validate(cfg)) return rc;
  if (num_chunks < 1 || step < 0) return fail(SDV2_EINVAL, "num_chunks must be >= 1 and step >= 0");
  const int64_t B = cfg->stream_batch;
  const int64_t lo = step - B + 1 > 0 ? step - B + 1 : 0;
  const int64_t hi = step < num_chunks - 1 ? step : num_chunks - 1;
  const int64_t nb = hi >= lo ? hi - lo + 1 : 0;
  const int64_t c0 = step - B + 1;
  if (first_chunk) *first_chunk = nb > 0 ? lo : -1;
  if (nbatch) *nbatch = (int32_t)nb;
  if (commit_chunk) *commit_chunk = (c0 >= 0 && c0 < num_chunks) ? c0 : -1;
  if (newest_frame) *newest_frame = nb > 0 ? (hi + 1) * cfg->chunk_frames - 1 : -1;
  return ok();
}

int sdv2_debug_check_plan(const sdv2_config* cfg, int32_t nbatch, int32_t nshared, int32_t* nsplit,
                          int32_t* tail_items, int32_t* workgroups) {
  if (int rc = validate(cfg)) return rc;
  const sdv2_config& c = *cfg;
  if (nbatch < 1 || nbatch > c.stream_batch) return fail(SDV2_EINVAL, "nbatch out of range");
  if (nshared < 0 || nshared > c.sink_frames + c.window_frames) return fail(SDV2_EINVAL, "nshared out of range");
  const int64_t N = (int64_t)c.grid_h * c.grid_w, R = c.chunk_frames * N;
  const int tpf = (int)(align_up(N, kTileKeys) / kTileKeys);
  const WorkPlan p = make_plan(c, nbatch, (nshared + c.chunk_frames) * tpf, (nshared + 1) * tpf);
  const int qtiles = (int)((R + kQTile - 1) / kQTile), items = nbatch * c.num_heads * qtiles;
  const int ntail = p.tail_first[kNumXcd];
  if (p.first[0] != 0 || p.first[kNumXcd] != items) return fail(SDV2_EINVAL, "plan: items not partitioned");
  if (ntail > 0 && p.nsplit < 2) return fail(SDV2_EINVAL, "plan: tail items with one split");
  // every key tile of every item covered once; whole items by one workgroup; partial rows in range
  std::vector<std::vector<int>> cover(items);
  std::vector<int> tail_seen(ntail, 0);
  int wg = 0;
  for (int b = 0; b < kNumXcd * p.wg_per_xcd; ++b) {
    WorkItem w;
    if (!plan_item(p, qtiles, nbatch, b, w)) continue;
    ++wg;
    if (w.head < 0 || w.head >= c.num_heads || w.elem < 0 || w.elem >= nbatch || w.qtile < 0 || w.qtile >= qtiles)
      return fail(SDV2_EINVAL, "plan: workgroup %d decodes out of range", b);
    const int item = (w.head * nbatch + w.elem) * qtiles + w.qtile;
    const int x = b % kNumXcd;
    if (item < p.first[x] || item >= p.first[x + 1]) return fail(SDV2_EINVAL, "plan: item %d off its XCD", item);
    if ((w.tail < 0) != (w.nsplit == 1) || w.split < 0 || w.split >= w.nsplit)
      return fail(SDV2_EINVAL, "plan: workgroup %d split %d of %d tail %d", b, w.split, w.nsplit, w.tail);
    if (w.tail >= 0) {
      if (w.tail >= ntail) return fail(SDV2_EINVAL, "plan: tail index %d of %d", w.tail, ntail);
      int h2, e2, q2;
      plan_tail(p, qtiles, nbatch, w.tail, h2, e2, q2);
      if (h2 != w.head || e2 != w.elem || q2 != w.qtile) return fail(SDV2_EINVAL, "plan: tail %d maps back wrong", w.tail);
      ++tail_seen[w.tail];
    }
    // the kernels' split of the item's walk (block-causal: it ends at the last own frame the
    // query tile sees)
    const int tq_hi = (int)std::min<int64_t>(c.chunk_frames - 1, ((int64_t)w.qtile * kQTile + kQTile - 1) / N);
    const int tiles_q = (nshared + tq_hi + 1) * tpf;
    const int t0 = (int)((int64_t)w.split * tiles_q / w.nsplit), t1 = (int)((int64_t)(w.split + 1) * tiles_q / w.nsplit);
    if (t1 <= t0) return fail(SDV2_EINVAL, "plan: workgroup %d has no key tile", b);
    for (int t = t0; t < t1; ++t) cover[item].push_back(t);
  }
  for (int i = 0; i < items; ++i) {
    std::vector<int>& v = cover[i];
    std::sort(v.begin(), v.end());
    const int q = i % qtiles;
    const int tq_hi = (int)std::min<int64_t>(c.chunk_frames - 1, ((int64_t)q * kQTile + kQTile - 1) / N);
    const int tiles_q = (nshared + tq_hi + 1) * tpf;
    if ((int)v.size() != tiles_q) return fail(SDV2_EINVAL, "plan: item %d covered %zu of %d tiles", i, v.size(), tiles_q);
    for (int t = 0; t < tiles_q; ++t)
      if (v[t] != t) return fail(SDV2_EINVAL, "plan: item %d tile %d not covered exactly once", i, t);
  }
  for (int t = 0; t < ntail; ++t)
    if (tail_seen[t] != p.nsplit) return fail(SDV2_EINVAL, "plan: tail item %d has %d of %d splits", t, tail_seen[t], p.nsplit);
  // the partial results fit the workspace sdv2_cache_size asks for
  if (plan_partial_bytes(p, c.head_dim, nullptr) > workspace_bytes(c))
    return fail(SDV2_EINVAL, "plan: partials exceed the workspace");
  if (nsplit) *nsplit = p.nsplit;
  if (tail_items) *tail_items = ntail;
  if (workgroups) *workgroups = wg;
  return ok();
}

int sdv2_debug_fail_hip_call(int32_t nth) {
  g_fail_hip.store(nth < 0 ? -1 : nth);
  return ok();
}

const char* sdv2_last_error(void) { return g_error.c_str(); }

}  // extern "C"
