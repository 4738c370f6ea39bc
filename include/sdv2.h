/*
 * sdv2.h - C ABI of the sink + rolling-KV chunk-attention library for AMD MI355X (gfx950).
 *
 * The operation: a causal video DiT streams latent frames in chunks of T' frames; a stream batch
 * of B chunks at different noise levels runs in one call and the oldest one finishes each call.
 * Every chunk attends over a KV cache made of S pinned "sink" frames, a rolling window of the W
 * most recently finished frames, and its own chunk.  Keys carry a 3-axis (t, h, w) rotary
 * position embedding whose temporal phase is periodically rebased ("RoPE refresh"); the sinks
 * are refreshed when a new chunk embedding is too dissimilar to all of them; a per-frame motion
 * estimate drives the noise-rate EMA.
 *
 * Pages this interface follows (title, section):
 *  [WT]   "直播革命來了！StreamDiffusionV2" paper walkthrough (qq8o.cn), section "方法" (Method):
 *         "SLO感知的批處理調度器" (SLO-aware batching scheduler: chunk size T, stream batch B,
 *         B*T must not exceed the frames collected), "自適應的sink和RoPE刷新" (adaptive sink and
 *         RoPE refresh), "運動感知的噪聲調度器" (motion-aware noise scheduler).
 *  [NEWS] admirer.cn article on StreamDiffusionV2 (MLSys 2026), section "方法" (Method),
 *         algorithm items 1 (sink tokens + rolling KV cache) and 2 (motion-aware noise),
 *         system item 1 (pipelined batch denoising: one finished frame per DiT call).
 *  [REPO] agentlenshq page "chenfengxu714/StreamDiffusionV2", section "核心组件" (core
 *         components: ring-buffer KV cache with sliding-window attention) and "快速 Python 示例"
 *         (quick example: encode -> denoise, which yields nothing while the pipeline fills).
 *
 * Conventions (all entry points):
 *  - Return 0 (SDV2_OK) or a negative error code.  A failing call changes no host state and
 *    launches nothing, except SDV2_EHIP from a launch, after which the cache must be destroyed.
 *    The message of the last error on the calling thread: sdv2_last_error().
 *  - Device pointers are caller-owned (the library never allocates or frees device memory);
 *    they must stay valid while work that uses them is in flight.  The cache handle is
 *    library-owned host memory, freed by sdv2_cache_destroy.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued asynchronously
 *    on it; no call synchronises unless its comment says so.
 *  - q, k, v and attention outputs are contiguous [nbatch][T'*N][H][head_dim] in the cache dtype
 *    (fp32, or bf16 bit patterns rounded to nearest even), N = grid_h * grid_w tokens per frame,
 *    token n at row n / grid_w, column n % grid_w.  Embeddings and latent frames are fp32.
 *  - Step protocol (per stream step):
 *        sdv2_rope_refresh  ->  for each layer: sdv2_cache_append, sdv2_chunk_attention
 *        -> [sdv2_cache_commit -> [sdv2_sink_replace]]
 *    Calls out of this order return SDV2_ESTATE and change nothing.
 */
#ifndef SDV2_H
#define SDV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SDV2_OK = 0,
  SDV2_EINVAL = -1, /* bad argument or configuration */
  SDV2_ESTATE = -2, /* call out of the step protocol */
  SDV2_EHIP = -3,   /* a HIP runtime call or kernel launch failed */
  SDV2_ENOSPC = -4  /* a caller buffer is smaller than sdv2_cache_size() asks for */
};

enum {
  SDV2_F32 = 0,          /* fp32 activations and cache */
  SDV2_BF16 = 1,         /* bf16 activations and cache */
  SDV2_BF16_KV_FP8 = 2   /* bf16 activations, OCP e4m3 cache (head_dim 128): K_rot and V are
                            rounded to nearest even, saturated at +-448; fp32 accumulation */
};

/* Library limits (validated by sdv2_config_validate).  Besides these: one slot of the cache
 * (slot_stride * elem_bytes) must be under 2 GiB and one layer's K block (slots * slot_stride *
 * elem_bytes) under 4 GiB, since the attention kernel forms offsets inside a block in 32 bits;
 * and N = grid_h * grid_w <= 2^20. */
enum {
  SDV2_MAX_SLOTS_SHARED = 64, /* S + W + T' */
  SDV2_MAX_BATCH = 8,         /* B, and B * T' */
  SDV2_MAX_SINKS = 16,        /* S */
  SDV2_MAX_TPAIRS = 32        /* rope_dim_t / 2 */
};

typedef struct sdv2_config {
  int32_t num_layers;
  int32_t num_heads;     /* H */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t grid_h;        /* latent tokens per frame: N = grid_h * grid_w */
  int32_t grid_w;
  int32_t sink_frames;   /* S >= 0 */
  int32_t window_frames; /* W >= 1 */
  int32_t chunk_frames;  /* T' >= 1 frames per chunk, B * T' <= SDV2_MAX_BATCH */
  int32_t stream_batch;  /* B in [1, SDV2_MAX_BATCH] */
  int32_t rope_dim_t;    /* even; rope_dim_t + rope_dim_h + rope_dim_w == head_dim */
  int32_t rope_dim_h;
  int32_t rope_dim_w;
  double rope_theta;     /* > 1 */
  int32_t rope_refresh_period; /* T_reset >= 0; 0 = never */
  int32_t dtype;         /* SDV2_F32 | SDV2_BF16 | SDV2_BF16_KV_FP8 */
  int32_t embed_dim;     /* D >= 0: chunk-embedding length; 0 = no sink refresh */
  int32_t rope_pin_sinks; /* 0: a RoPE refresh rebases every cached key; 1: sinks keep their
                             labels (pinned anchors), only the window is rebased */
  double sink_threshold; /* tau; NaN or -INFINITY = sink refresh off */
  double key_scale;      /* 0: K is cached as rotated (SDV2_BF16, SDV2_F32).  > 0 (head_dim 128;
                            required for SDV2_BF16_KV_FP8): K is cached as rotated x g, rounded
                            once from fp32, g = key_scale x log2(e) for the bf16 cache and
                            key_scale x log2(e) x 2^k for the e4m3 one, k = -floor(log2(
                            key_scale x log2(e)) + 1/2) (keys keep their range; queries are
                            then scaled by 2^-k inside the attention, exactly), so the
                            attention's exponent needs no per-score product; every
                            sdv2_chunk_attention on the cache must pass scale == key_scale. */
} sdv2_config;

/* Device layout of the KV cache (element offsets from d_kv, element = 4, 2 or 1 bytes).
 * Slots [0,S) are sinks, [S,S+W+T') the ring (frame f >= S lives in slot S + f mod (W+T');
 * W of these slots hold the window, the T' spare ones receive the chunk being finished), and
 * [S+W+T', S+W+B*T') the staging slots of stream-batch elements 1..B-1 (frame t of element b
 * in S+W+b*T'+t).
 *   K of (layer, slot, head, token n, dim i): k_offset(layer) + slot*slot_stride
 *        + head*head_stride + n*head_dim + i                      (rows of head_dim)
 *   V of (layer, slot, head, token n, dim i): v_offset(layer) + slot*slot_stride
 *        + head*head_stride + i*tokens_padded + n                 (stored transposed)
 * with k_offset(l) = l*layer_stride, v_offset(l) = l*layer_stride + slot_stride*slots.
 * e4m3 cache: within each group of 32 dims of a K row, and of 32 tokens of a V^T row inside a
 * 64-token tile, element 32p + 16h + 8g + e is stored at 32p + 16g + 8h + e.
 * Tokens n in [N, tokens_padded) are zero padding. */
typedef struct sdv2_layout {
  int64_t slots;          /* S + (W + T') + (B - 1) T' */
  int64_t tokens_padded;  /* N rounded up to 64 */
  int64_t elem_bytes;     /* 4 (fp32), 2 (bf16) or 1 (e4m3) */
  int64_t head_stride;    /* tokens_padded * head_dim */
  int64_t slot_stride;    /* num_heads * head_stride */
  int64_t layer_stride;   /* 2 * slots * slot_stride (K block then V block) */
  int64_t kv_elems;       /* num_layers * layer_stride */
} sdv2_layout;

typedef struct sdv2_cache sdv2_cache;

/* Check a configuration against the library limits.  Host only. */
int sdv2_config_validate(const sdv2_config* cfg);

/* Fill *out with the cache layout of cfg.  Host only. */
int sdv2_cache_layout(const sdv2_config* cfg, sdv2_layout* out);

/* Bytes the caller must allocate on the device: the KV cache (layout above), the metadata
 * block (RoPE h/w tables, sink embeddings, the last sink decision) and the workspace
 * (split-KV partial results).  Host only.  Any pointer may be NULL. */
int sdv2_cache_size(const sdv2_config* cfg, size_t* kv_bytes, size_t* meta_bytes,
                    size_t* workspace_bytes);

/* Create a cache over caller-owned device buffers (sizes from sdv2_cache_size; 256-byte
 * aligned).  Zero-fills d_kv and writes the h/w RoPE tables into d_meta on `stream`, then
 * synchronises `stream` once.  On success *out owns host bookkeeping only. */
int sdv2_cache_create(const sdv2_config* cfg, void* d_kv, size_t kv_bytes, void* d_meta,
                      size_t meta_bytes, void* d_workspace, size_t workspace_bytes,
                      void* stream, sdv2_cache** out);

/* Free the handle (not the device buffers).  NULL is accepted. */
int sdv2_cache_destroy(sdv2_cache* cache);

/* Start a stream step ([WT] adaptive sink and RoPE refresh: the RoPE phase is reset when the
 * frame index passes a threshold).  `newest_frame` is the last frame of the newest chunk in
 * flight this step (non-decreasing over calls).  While newest_frame - b0 >= T_reset, the RoPE
 * base b0 grows by T_reset and every cached key (sinks and window) is re-rotated in place by
 * -T_reset on the temporal pairs, so scores are unchanged (e4m3 cache: up to the rounding of
 * the re-rotated keys, which are widened, turned in fp32 and rounded again).  With
 * rope_pin_sinks the sinks are
 * left as they are: their labels stay, so the query-to-sink distance drops by T_reset (the
 * anchors are reset with the phase).  *applied (may be NULL) receives
 * the number of rebases.  Must open every step, also when T_reset == 0. */
int sdv2_rope_refresh(sdv2_cache* cache, int64_t newest_frame, int32_t* applied, void* stream);

/* RoPE + append for one layer ([NEWS] algorithm item 1; [REPO] ring-buffer KV cache).
 * Elements b = 0..nbatch-1 hold chunks first_chunk+b (b = 0 oldest) of T' frames each, frame
 * f = chunk*T' + t in rows [t*N, (t+1)*N); first_chunk must equal the number of chunks
 * committed so far and (first_chunk + nbatch)*T' - 1 the newest frame given to
 * sdv2_rope_refresh.  d_q is rotated in place at temporal position f - b0 (row h, col w); k is
 * rotated likewise (in fp32, then rounded once; with key_scale > 0 multiplied by
 * key_scale * log2(e) before the rounding) and written with v: element 0's frames
 * into the slots they keep once
 * committed (sink slot f, or ring slot S + f mod (W+T'), which hold no attended frame), the
 * others into their staging slots.  Buffers:
 * [nbatch][T'N][H][d] each; d_q read-write, d_k and d_v read-only.  Once per layer per step. */
int sdv2_cache_append(sdv2_cache* cache, int32_t layer, int64_t first_chunk, int32_t nbatch,
                      void* d_q, const void* d_k, const void* d_v, void* stream);

/* Chunk attention for one layer (after its append this step).  For each element b and head:
 * out = softmax(scale * Q_rot K^T) V over the keys [present sinks | window | own chunk], with
 * Q_rot = d_q_rot as rotated by sdv2_cache_append; inside the own chunk a query of frame t sees
 * the keys of frames 0..t (block-causal).  d_out: [nbatch][T'N][H][d], written.  The
 * workspace given at create time is used for split-KV partial results (calls on one cache
 * must not overlap in time).  On a cache with key_scale > 0, scale must equal key_scale
 * (SDV2_EINVAL otherwise, nothing launched).  The split-KV
 * count follows a cost model; SDV2_NSPLIT=n (read at create and at each call; clamped to
 * [1, 16] and to the shortest walk) forces it, for tests and tuning: the cache must be created
 * with the variable set, so that the workspace covers the forced count. */
int sdv2_chunk_attention(sdv2_cache* cache, int32_t layer, int32_t nbatch, const void* d_q_rot,
                         void* d_out, float scale, void* stream);

/* Chunk attention for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): the operation, arguments and
 * kernels of sdv2_chunk_attention, with the split-KV partial results kept in a static device
 * array of the library (SDV2_STATIC_SCRATCH_BYTES per GPU, held until the process ends) instead
 * of the workspace given at create time.  Allocates nothing.  The split count is the one
 * sdv2_chunk_attention uses; if its partial results exceed the array the call returns
 * SDV2_ENOSPC and launches nothing.  The array's device address is looked up on the first call
 * on each device.  Every call on one GPU shares that GPU's array (nothing in it needs to start
 * at zero): calls that overlap in time on one GPU race, whatever cache they use. */
enum { SDV2_STATIC_SCRATCH_BYTES = 96 << 20 };
int sdv2_chunk_attention_static(sdv2_cache* cache, int32_t layer, int32_t nbatch,
                                const void* d_q_rot, void* d_out, float scale, void* stream);

/* Commit the finished chunk (element 0, which must be `chunk`) for all layers: from the next
 * step on, its T' frames' K and V (already in sink slot f if f < S, else in ring slot
 * S + f mod (W+T')) are attended, and for each of them the frame W older leaves the window.
 * Requires every layer appended this step.  Host bookkeeping only: no device work is queued on
 * `stream`. */
int sdv2_cache_commit(sdv2_cache* cache, int64_t chunk, void* stream);

/* Chunk statistics and adaptive sink refresh after a commit, one fused statistics launch
 * ([WT] adaptive sink and RoPE refresh; [WT] motion-aware noise scheduler and [NEWS] algorithm
 * item 2: the distance between consecutive latent frames drives the noise rate).  `frame` is the
 * last frame of the committed chunk.
 *  - d_embed: fp32 [embed_dim] chunk embedding h (device); required when embed_dim >= 1, NULL
 *    otherwise.  Every frame of the chunk below S became a sink and gets h as its embedding.
 *  - d_prev_latent, d_cur_latent: fp32 [latent_elems] latent frames x_{t-1}, x_t (device), both
 *    or neither (NULL: no motion term).
 *  - One launch reduces, in fp64 and a fixed order, sum_i (x_t[i] - x_{t-1}[i])^2 and h.h,
 *    e_j.e_j, h.e_j for the S sinks; a one-block launch then forms the statistics and the
 *    decision: if frame >= S and tau is on, alpha_j = cos(h, e_j) (0 if a norm is 0), j* = argmin
 *    (lowest j on ties), and if alpha_j* < tau frame `frame`'s K/V are copied into sink j* for
 *    all layers and e_j* = h.  A sink stored by this call has e_j = h in the decision.
 *  - d_stats (device, may be NULL): fp64 [4 + 2S] = { sum (dx)^2, sqrt(sum (dx)^2 /
 *    latent_elems), h.h, e_0.e_0 .. e_{S-1}.e_{S-1}, h.e_0 .. h.e_{S-1}, alpha_j* }, NaN for a
 *    term not computed (no latents, no embedding, no decision).  8-byte aligned.
 * The decision stays on the device.  If h_slot is non-NULL and a decision is taken the call
 * synchronises `stream` and returns j* if replaced, else -1 (h_alpha, may be NULL: alpha_j*);
 * with h_slot NULL nothing synchronises and sdv2_cache_slot_info reports the sink slots as
 * unknown (-2) from then on.  With no embedding, no latents and d_stats NULL nothing is launched
 * (the call only closes the step). */
int sdv2_sink_replace(sdv2_cache* cache, int64_t frame, const float* d_embed,
                      const float* d_prev_latent, const float* d_cur_latent, int64_t latent_elems,
                      double* d_stats, int32_t* h_slot, double* h_alpha, void* stream);

/* Batched motion estimate over a stored series ([NEWS] algorithm item 2; [WT] motion-aware
 * noise scheduler; the per-step form is the motion term of sdv2_sink_replace): for t = 1 ..
 * nframes-1, d_dist[t-1] = sqrt(sum_i (x_t[i] - x_{t-1}[i])^2 / elems_per_frame), summed in fp64
 * in a fixed order.  d_frames: fp32 [nframes][elems_per_frame], 4-byte aligned (16-byte
 * aligned with elems_per_frame % 4 == 0 takes 16-byte loads); d_dist: fp64 [nframes-1];
 * d_workspace: at least sdv2_motion_workspace_size() bytes (per-part partial sums, contents
 * unspecified on return); both 8-byte aligned.  Stateless; results are run-to-run identical.
 * Errors: SDV2_EINVAL for nframes < 2, elems_per_frame < 1, more than 65536 frames, a NULL or
 * misaligned pointer; SDV2_ENOSPC for a short workspace; nothing is launched then. */
int sdv2_motion_workspace_size(int32_t nframes, int64_t elems_per_frame, size_t* bytes);
int sdv2_motion_l2(const float* d_frames, int32_t nframes, int64_t elems_per_frame,
                   double* d_dist, void* d_workspace, size_t workspace_bytes, void* stream);

/* Motion-aware noise rate ([WT] motion-aware noise scheduler), host scalars: dhat_t =
 * min(1, max of the last k distances / sigma), target = s_max - (s_max - s_min) * dhat,
 * s_t = lambda * target + (1 - lambda) * s_{t-1}, from s_0 = s0.  h_dist: [n] distances
 * d_1..d_n; h_rate: [n] rates s_1..s_n.  Host only. */
int sdv2_noise_schedule(const double* h_dist, int32_t n, double sigma, int32_t k, double lambda,
                        double s_min, double s_max, double s0, double* h_rate);

/* SLO-aware choice of stream batch B and chunk size T' ([WT] SLO-aware batching scheduler: the
 * step latency L(T', B) is parameter plus activation traffic over an effective bandwidth, the
 * activations growing linearly in B*T'; f = B*T'/L; B*T' must not exceed the frames collected).
 * Host only.
 * sdv2_latency_fit: least-squares L = c0 + c1 * frames from n >= 2 measured steps (frames =
 *   B*T' of each, at least two distinct values; latency in seconds).
 * sdv2_slo_select: over 1 <= B <= max_batch, 1 <= T' <= max_chunk with B*T' <= frames_ready and
 *   B*T' <= SDV2_MAX_BATCH: L = c0 + c1*B*T', f = B*T'/L, a frame's latency = B*L (its chunk is in
 *   flight for B steps) + (T'-1)/target_fps (waiting for its chunk's frames).  Feasible: f >=
 *   target_fps and latency <= deadline_s.  Returns the feasible candidate of highest f (f within a
 *   relative 1e-12 counts as equal; ties: lower latency, then smaller B) with *feasible = 1, else
 *   the highest-f candidate with *feasible = 0.  Outputs may be NULL except B and T.  Errors:
 *   SDV2_EINVAL if a candidate's L <= 0, target_fps <= 0 or no candidate exists. */
int sdv2_latency_fit(const int32_t* h_frames, const double* h_latency_s, int32_t n, double* c0,
                     double* c1);
int sdv2_slo_select(double c0, double c1, double target_fps, double deadline_s, int32_t frames_ready,
                    int32_t max_batch, int32_t max_chunk, int32_t* B, int32_t* T, double* fps,
                    double* latency_s, int32_t* feasible);

/* Host bookkeeping of one slot: committed frame (-1 empty, -2 unknown after an unsynchronised
 * sink decision) and its temporal RoPE position label = frame - b0 at commit, shifted by every
 * later rebase.  A slot written by an append and not (yet) committed reports the chunk staged
 * there (staging slots, and element 0's sink or ring slot before its commit).  Never
 * synchronises. */
int sdv2_cache_slot_info(const sdv2_cache* cache, int32_t slot, int64_t* frame, int32_t* tpos);

/* RoPE base b0, chunks committed so far and rebases applied so far.  Any pointer may be NULL. */
int sdv2_cache_state(const sdv2_cache* cache, int64_t* rope_base, int64_t* committed,
                     int64_t* refreshes);

/* Stream-batch schedule of step `step` for a stream of num_chunks chunks ([NEWS] system item 1;
 * [REPO] quick example): in-flight chunks [first_chunk, first_chunk + nbatch), the chunk
 * finished and committed at its end (-1 while the pipeline fills) and the newest in-flight
 * frame, the last frame of the newest chunk (-1 past the end).  Host only. */
int sdv2_plan_step(const sdv2_config* cfg, int64_t num_chunks, int64_t step, int64_t* first_chunk,
                   int32_t* nbatch, int64_t* commit_chunk, int64_t* newest_frame);

/* Fault injection for tests of the error paths: the nth HIP runtime call or kernel launch the
 * library makes from now on (0 = the next one) is not issued and its entry point returns
 * SDV2_EHIP, as a failing launch would; nth < 0 disarms.  Process-wide; fires once.  An entry
 * point whose first launch fails this way has launched nothing and changed no state. */
int sdv2_debug_fail_hip_call(int32_t nth);

/* Check of the split-KV work plan sdv2_chunk_attention uses for nbatch elements with nshared
 * cached frames present, for tests: every workgroup of the grid decodes (as the kernels decode
 * it) to a query tile of its XCD; every key tile of every query tile is covered by exactly one
 * workgroup; split query tiles have all their splits and partial-result indices inside the
 * workspace sdv2_cache_size asks for.  Outputs (may be NULL): the split count of the split
 * query tiles, their number and the workgroups that do work.  SDV2_EINVAL names the first
 * violation.  Host only. */
int sdv2_debug_check_plan(const sdv2_config* cfg, int32_t nbatch, int32_t nshared, int32_t* nsplit,
                          int32_t* tail_items, int32_t* workgroups);

/* Message of the last failing call on this thread ("" if none). */
const char* sdv2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SDV2_H */
