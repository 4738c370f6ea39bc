// Host-only exercise of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer: config
// validation, layout and sizes, the step schedule, the noise schedule, the latency fit and SLO
// choice, motion workspace sizes, and the error paths that return before any HIP call (short
// or misaligned buffers at create, NULL handles).  The kernel launchers are stubs: no entry
// point called here reaches them.  Built and run by tests/test_host_sanitizers.py.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.h"
#include "sdv2.h"

namespace sdv2 {
hipError_t launch_rope_append(const AppendArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention(const AttnArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention_w64(const AttnArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_combine(const CombineArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_rebase(const RebaseArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_copy_slots(const CopyArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_chunk_stats(const StatsArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_sink_decide(const SinkArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_motion(const float*, int, int64_t, double*, double*, int, hipStream_t) {
  return hipErrorNotSupported;
}
int motion_parts(int64_t elems) { return (int)((elems + 16383) / 16384); }
}  // namespace sdv2

static int failures = 0;
#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

static sdv2_config wan14b() {
  sdv2_config c{};
  c.num_layers = 40; c.num_heads = 40; c.head_dim = 128; c.grid_h = 32; c.grid_w = 32;
  c.sink_frames = 1; c.window_frames = 8; c.chunk_frames = 1; c.stream_batch = 4;
  c.rope_dim_t = 44; c.rope_dim_h = 42; c.rope_dim_w = 42; c.rope_theta = 10000.0;
  c.rope_refresh_period = 0; c.dtype = SDV2_BF16; c.embed_dim = 5120; c.rope_pin_sinks = 0;
  c.sink_threshold = 0.95;
  return c;
}

static sdv2_config tiny() {
  sdv2_config c{};
  c.num_layers = 1; c.num_heads = 2; c.head_dim = 64; c.grid_h = 4; c.grid_w = 4;
  c.sink_frames = 1; c.window_frames = 4; c.chunk_frames = 1; c.stream_batch = 1;
  c.rope_dim_t = 24; c.rope_dim_h = 20; c.rope_dim_w = 20; c.rope_theta = 10000.0;
  c.rope_refresh_period = 8; c.dtype = SDV2_F32; c.embed_dim = 64; c.rope_pin_sinks = 0;
  c.sink_threshold = 0.9;
  return c;
}

int main() {
  const sdv2_config base[] = {wan14b(), tiny()};
  for (const sdv2_config& c0 : base) {
    CHECK(sdv2_config_validate(&c0) == SDV2_OK);
    sdv2_layout l{};
    CHECK(sdv2_cache_layout(&c0, &l) == SDV2_OK);
    size_t kv = 0, meta = 0, ws = 0;
    CHECK(sdv2_cache_size(&c0, &kv, &meta, &ws) == SDV2_OK);
    CHECK((int64_t)kv == l.kv_elems * l.elem_bytes);
    CHECK(sdv2_cache_size(&c0, nullptr, nullptr, nullptr) == SDV2_OK);
    // every field pushed through a range of values, valid or not
    for (int field = 0; field < 19; ++field)
      for (int v = -3; v <= 300; v += 7) {
        sdv2_config c = c0;
        int32_t* i32[] = {&c.num_layers, &c.num_heads, &c.head_dim, &c.grid_h, &c.grid_w,
                          &c.sink_frames, &c.window_frames, &c.chunk_frames, &c.stream_batch,
                          &c.rope_dim_t, &c.rope_dim_h, &c.rope_dim_w, &c.rope_refresh_period,
                          &c.dtype, &c.embed_dim, &c.rope_pin_sinks};
        if (field < 16) *i32[field] = v;
        else if (field == 16) c.rope_theta = v * 100.0;
        else if (field == 17) c.sink_threshold = v / 100.0;
        else c.sink_threshold = std::nan("");
        const int rc = sdv2_config_validate(&c);
        CHECK(rc == SDV2_OK || rc == SDV2_EINVAL);
        if (rc == SDV2_OK) {
          CHECK(sdv2_cache_size(&c, &kv, &meta, &ws) == SDV2_OK);
          for (int64_t step = 0; step < 40; ++step) {
            int64_t first, commit, newest;
            int32_t nb;
            CHECK(sdv2_plan_step(&c, 17, step, &first, &nb, &commit, &newest) == SDV2_OK);
            CHECK(nb >= 0 && nb <= c.stream_batch);
          }
        } else {
          CHECK(std::strlen(sdv2_last_error()) > 0);
        }
      }
    // create: short or misaligned buffers fail before any device work
    const uintptr_t fake = 1u << 20;
    sdv2_cache* h = nullptr;
    CHECK(sdv2_cache_size(&c0, &kv, &meta, &ws) == SDV2_OK);
    if (kv > 0)
      CHECK(sdv2_cache_create(&c0, (void*)fake, kv - 1, (void*)fake, meta, (void*)fake, ws, nullptr, &h) == SDV2_ENOSPC);
    CHECK(sdv2_cache_create(&c0, (void*)fake, kv, (void*)fake, meta - 1, (void*)fake, ws, nullptr, &h) == SDV2_ENOSPC);
    CHECK(sdv2_cache_create(&c0, (void*)(fake + 8), kv, (void*)fake, meta, (void*)fake, ws, nullptr, &h) == SDV2_EINVAL);
    CHECK(sdv2_cache_create(&c0, nullptr, kv, (void*)fake, meta, (void*)fake, ws, nullptr, &h) == SDV2_EINVAL);
    CHECK(sdv2_cache_create(&c0, (void*)fake, kv, (void*)fake, meta, (void*)fake, ws, nullptr, nullptr) == SDV2_EINVAL);
    CHECK(h == nullptr);
  }
  CHECK(sdv2_config_validate(nullptr) == SDV2_EINVAL);
  // NULL handles
  int64_t a = 0, b = 0, c = 0;
  int32_t t = 0;
  CHECK(sdv2_cache_state(nullptr, &a, &b, &c) == SDV2_EINVAL);
  CHECK(sdv2_cache_slot_info(nullptr, 0, &a, &t) == SDV2_EINVAL);
  CHECK(sdv2_rope_refresh(nullptr, 0, &t, nullptr) == SDV2_EINVAL);
  CHECK(sdv2_cache_append(nullptr, 0, 0, 1, nullptr, nullptr, nullptr, nullptr) == SDV2_EINVAL);
  CHECK(sdv2_chunk_attention(nullptr, 0, 1, nullptr, nullptr, 1.f, nullptr) == SDV2_EINVAL);
  CHECK(sdv2_chunk_attention_static(nullptr, 0, 1, nullptr, nullptr, 1.f, nullptr) == SDV2_EINVAL);
  CHECK(sdv2_cache_commit(nullptr, 0, nullptr) == SDV2_EINVAL);
  CHECK(sdv2_sink_replace(nullptr, 0, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr) == SDV2_EINVAL);
  CHECK(sdv2_cache_destroy(nullptr) == SDV2_OK);
  // noise schedule over random distances, windows 1..6
  std::vector<double> d(257), r(257);
  unsigned s = 12345;
  for (double& x : d) { s = s * 1103515245u + 12345u; x = (s >> 8) / double(1 << 24) * 2.0; }
  for (int k = 1; k <= 6; ++k) {
    CHECK(sdv2_noise_schedule(d.data(), (int32_t)d.size(), 1.0, k, 0.9, 0.25, 1.0, 1.0, r.data()) == SDV2_OK);
    for (double x : r) CHECK(x >= 0.25 - 1e-12 && x <= 1.0 + 1e-12);
  }
  CHECK(sdv2_noise_schedule(d.data(), 0, 1.0, 4, 0.9, 0.25, 1.0, 1.0, r.data()) == SDV2_OK);
  CHECK(sdv2_noise_schedule(nullptr, 3, 1.0, 4, 0.9, 0.25, 1.0, 1.0, r.data()) == SDV2_EINVAL);
  CHECK(sdv2_noise_schedule(d.data(), 3, 0.0, 4, 0.9, 0.25, 1.0, 1.0, r.data()) == SDV2_EINVAL);
  // latency fit and SLO choice
  const int32_t frames[] = {1, 2, 4, 8, 2, 4};
  const double lat[] = {0.003, 0.005, 0.009, 0.017, 0.0052, 0.0091};
  double c0 = 0, c1 = 0;
  CHECK(sdv2_latency_fit(frames, lat, 6, &c0, &c1) == SDV2_OK);
  CHECK(c1 > 0.0);
  CHECK(sdv2_latency_fit(frames, lat, 1, &c0, &c1) == SDV2_EINVAL);
  const int32_t same[] = {2, 2};
  CHECK(sdv2_latency_fit(same, lat, 2, &c0, &c1) == SDV2_EINVAL);
  for (int ready = 0; ready <= 10; ++ready)
    for (int mb = 0; mb <= 9; ++mb) {
      int32_t B = 0, T = 0, feas = 0;
      double fps = 0, l = 0;
      const int rc = sdv2_slo_select(0.001, 0.002, 30.0, 0.1, ready, mb, 8, &B, &T, &fps, &l, &feas);
      CHECK(rc == SDV2_OK || rc == SDV2_EINVAL);
      if (rc == SDV2_OK) CHECK(B >= 1 && T >= 1 && B * T <= ready);
    }
  size_t bytes = 0;
  CHECK(sdv2_motion_workspace_size(129, 16 * 60 * 104, &bytes) == SDV2_OK && bytes > 0);
  CHECK(sdv2_motion_workspace_size(1, 10, &bytes) == SDV2_EINVAL);
  CHECK(sdv2_debug_fail_hip_call(2) == SDV2_OK && sdv2_debug_fail_hip_call(-1) == SDV2_OK);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host entry points clean under ASan + UBSan\n");
  return 0;
}
