"""Thin Python binding of libsdv2.so (ctypes): argument marshalling only.

Every entry point of include/sdv2.h is exposed under the same name.  Device buffers are torch
tensors (PyTorch supplies device memory and streams); every step of the path runs in the HIP
kernels of the library.  There is no fallback: if libsdv2.so is missing or fails to load, every
call raises.
"""
from __future__ import annotations

import ctypes
import pathlib
from typing import Optional

_LIB_PATH = pathlib.Path(__file__).resolve().parent / "libsdv2.so"

SDV2_OK, SDV2_EINVAL, SDV2_ESTATE, SDV2_EHIP, SDV2_ENOSPC = 0, -1, -2, -3, -4
SDV2_F32, SDV2_BF16, SDV2_BF16_KV_FP8 = 0, 1, 2
SDV2_STATIC_SCRATCH_BYTES = 96 << 20
ERROR_NAMES = {SDV2_EINVAL: "EINVAL", SDV2_ESTATE: "ESTATE", SDV2_EHIP: "EHIP", SDV2_ENOSPC: "ENOSPC"}


class Config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("sink_frames", ctypes.c_int32), ("window_frames", ctypes.c_int32),
                ("chunk_frames", ctypes.c_int32), ("stream_batch", ctypes.c_int32),
                ("rope_dim_t", ctypes.c_int32), ("rope_dim_h", ctypes.c_int32),
                ("rope_dim_w", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("rope_refresh_period", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("embed_dim", ctypes.c_int32), ("rope_pin_sinks", ctypes.c_int32),
                ("sink_threshold", ctypes.c_double), ("key_scale", ctypes.c_double)]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("slots", "tokens_padded", "elem_bytes", "head_stride",
                                              "slot_stride", "layer_stride", "kv_elems")]


class SDV2Error(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn}: {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None

_P, _I32, _I64, _SZ, _D, _F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                              ctypes.c_double, ctypes.c_float)
_PROTOS = {
    "sdv2_config_validate": [ctypes.POINTER(Config)],
    "sdv2_cache_layout": [ctypes.POINTER(Config), ctypes.POINTER(Layout)],
    "sdv2_cache_size": [ctypes.POINTER(Config), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
    "sdv2_cache_create": [ctypes.POINTER(Config), _P, _SZ, _P, _SZ, _P, _SZ, _P, ctypes.POINTER(_P)],
    "sdv2_cache_destroy": [_P],
    "sdv2_rope_refresh": [_P, _I64, ctypes.POINTER(_I32), _P],
    "sdv2_cache_append": [_P, _I32, _I64, _I32, _P, _P, _P, _P],
    "sdv2_chunk_attention": [_P, _I32, _I32, _P, _P, _F, _P],
    "sdv2_chunk_attention_static": [_P, _I32, _I32, _P, _P, _F, _P],
    "sdv2_cache_commit": [_P, _I64, _P],
    "sdv2_sink_replace": [_P, _I64, _P, _P, _P, _I64, _P, ctypes.POINTER(_I32), ctypes.POINTER(_D), _P],
    "sdv2_motion_workspace_size": [_I32, _I64, ctypes.POINTER(_SZ)],
    "sdv2_motion_l2": [_P, _I32, _I64, _P, _P, _SZ, _P],
    "sdv2_noise_schedule": [_P, _I32, _D, _I32, _D, _D, _D, _D, _P],
    "sdv2_latency_fit": [_P, _P, _I32, _P, _P],
    "sdv2_slo_select": [_D, _D, _D, _D, _I32, _I32, _I32, _P, _P, _P, _P, _P],
    "sdv2_cache_slot_info": [_P, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I32)],
    "sdv2_cache_state": [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I64)],
    "sdv2_debug_fail_hip_call": [_I32],
    "sdv2_debug_check_plan": [ctypes.POINTER(Config), _I32, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                              ctypes.POINTER(_I32)],
    "sdv2_plan_step": [ctypes.POINTER(Config), _I64, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I32),
                       ctypes.POINTER(_I64), ctypes.POINTER(_I64)],
}


def lib() -> ctypes.CDLL:
    """Load libsdv2.so (built in-tree by rolling_kv_causal_amd.build); raises if it is missing."""
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m rolling_kv_causal_amd.build` (there is no fallback path)")
        L = ctypes.CDLL(str(_LIB_PATH))
        for name, args in _PROTOS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.sdv2_last_error.argtypes = []
        L.sdv2_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def library_path() -> pathlib.Path:
    return _LIB_PATH


def _call(name: str, *args) -> None:
    rc = getattr(lib(), name)(*args)
    if rc != SDV2_OK:
        raise SDV2Error(rc, name, lib().sdv2_last_error().decode())


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


def make_config(*, num_layers, num_heads, head_dim, grid_h, grid_w, sink_frames, window_frames,
                chunk_frames=1, stream_batch=1, rope_dim_t, rope_dim_h, rope_dim_w,
                rope_theta=10000.0, rope_refresh_period=0, dtype="bf16", embed_dim=0,
                rope_pin_sinks=False, sink_threshold=None, kv_fp8=False, key_scale=0.0, **_ignored) -> Config:
    """Build the C config; dtype "bf16"/"fp32" (activations); kv_fp8 with bf16: e4m3 cache;
    sink_threshold None = sink refresh off; key_scale > 0: keys cached times it (bf16, d 128)."""
    code = SDV2_F32 if dtype != "bf16" else (SDV2_BF16_KV_FP8 if kv_fp8 else SDV2_BF16)
    return Config(num_layers, num_heads, head_dim, grid_h, grid_w, sink_frames, window_frames,
                  chunk_frames, stream_batch, rope_dim_t, rope_dim_h, rope_dim_w, float(rope_theta),
                  rope_refresh_period, code, embed_dim,
                  int(bool(rope_pin_sinks)), float("nan") if sink_threshold is None else float(sink_threshold),
                  float(key_scale))


def config_of(obj) -> Config:
    """C config from any object carrying the config's field names as attributes."""
    names = [f[0] for f in Config._fields_]
    kw = {n: getattr(obj, n) for n in names}
    return make_config(kv_fp8=getattr(obj, "kv_fp8", False), **kw)


# ---- entry points (same names as the C ABI) ----------------------------------------------------
def sdv2_config_validate(cfg: Config) -> None:
    _call("sdv2_config_validate", ctypes.byref(cfg))


def sdv2_cache_layout(cfg: Config) -> Layout:
    out = Layout()
    _call("sdv2_cache_layout", ctypes.byref(cfg), ctypes.byref(out))
    return out


def sdv2_cache_size(cfg: Config) -> tuple[int, int, int]:
    kv, meta, ws = _SZ(), _SZ(), _SZ()
    _call("sdv2_cache_size", ctypes.byref(cfg), ctypes.byref(kv), ctypes.byref(meta), ctypes.byref(ws))
    return kv.value, meta.value, ws.value


def sdv2_cache_create(cfg: Config, kv, meta, workspace, stream=None) -> int:
    h = _P()
    _call("sdv2_cache_create", ctypes.byref(cfg), _ptr(kv), kv.numel() * kv.element_size(),
          _ptr(meta), meta.numel() * meta.element_size(), _ptr(workspace),
          0 if workspace is None else workspace.numel() * workspace.element_size(),
          _stream(stream), ctypes.byref(h))
    return h.value


def sdv2_cache_destroy(handle) -> None:
    _call("sdv2_cache_destroy", handle)


def sdv2_rope_refresh(handle, newest_frame: int, stream=None) -> int:
    applied = _I32()
    _call("sdv2_rope_refresh", handle, newest_frame, ctypes.byref(applied), _stream(stream))
    return applied.value


def sdv2_cache_append(handle, layer: int, first_chunk: int, nbatch: int, q, k, v, stream=None) -> None:
    _call("sdv2_cache_append", handle, layer, first_chunk, nbatch, _ptr(q), _ptr(k), _ptr(v), _stream(stream))


def sdv2_chunk_attention(handle, layer: int, nbatch: int, q_rot, out, scale: float, stream=None) -> None:
    _call("sdv2_chunk_attention", handle, layer, nbatch, _ptr(q_rot), _ptr(out), scale, _stream(stream))


def sdv2_chunk_attention_static(handle, layer: int, nbatch: int, q_rot, out, scale: float, stream=None) -> None:
    _call("sdv2_chunk_attention_static", handle, layer, nbatch, _ptr(q_rot), _ptr(out), scale, _stream(stream))


def sdv2_cache_commit(handle, chunk: int, stream=None) -> None:
    _call("sdv2_cache_commit", handle, chunk, _stream(stream))


def sdv2_sink_replace(handle, frame: int, embed=None, prev_latent=None, cur_latent=None, stats=None,
                      sync: bool = True, stream=None):
    """Fused chunk statistics + sink refresh.  Returns (slot or -1, alpha) when sync, else None
    (the decision stays on the device).  stats: fp64 device tensor of 4 + 2S values, or None."""
    slot, alpha = _I32(), _D()
    n = 0 if cur_latent is None else cur_latent.numel()
    _call("sdv2_sink_replace", handle, frame, _ptr(embed), _ptr(prev_latent), _ptr(cur_latent), n,
          _ptr(stats), ctypes.byref(slot) if sync else None, ctypes.byref(alpha) if sync else None,
          _stream(stream))
    return (slot.value, alpha.value) if sync else None


def sdv2_motion_workspace_size(nframes: int, elems_per_frame: int) -> int:
    out = _SZ()
    _call("sdv2_motion_workspace_size", nframes, elems_per_frame, ctypes.byref(out))
    return out.value


def sdv2_motion_l2(frames, nframes: int, elems_per_frame: int, dist, workspace, stream=None) -> None:
    _call("sdv2_motion_l2", _ptr(frames), nframes, elems_per_frame, _ptr(dist), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream))


def sdv2_latency_fit(frames, latency_s) -> tuple[float, float]:
    n = len(frames)
    f = (ctypes.c_int32 * max(n, 1))(*frames)
    y = (ctypes.c_double * max(n, 1))(*latency_s)
    c0, c1 = _D(), _D()
    _call("sdv2_latency_fit", ctypes.cast(f, _P), ctypes.cast(y, _P), n, ctypes.addressof(c0), ctypes.addressof(c1))
    return c0.value, c1.value


def sdv2_slo_select(c0, c1, target_fps, deadline_s, frames_ready, max_batch, max_chunk) -> dict:
    B, T, feas = _I32(), _I32(), _I32()
    fps, lat = _D(), _D()
    _call("sdv2_slo_select", c0, c1, target_fps, deadline_s, frames_ready, max_batch, max_chunk,
          ctypes.addressof(B), ctypes.addressof(T), ctypes.addressof(fps), ctypes.addressof(lat),
          ctypes.addressof(feas))
    return {"B": B.value, "T": T.value, "fps": fps.value, "latency": lat.value, "feasible": bool(feas.value)}


def sdv2_noise_schedule(dist, sigma: float, k: int, lam: float, s_min: float, s_max: float, s0: float):
    n = len(dist)
    d = (ctypes.c_double * max(n, 1))(*dist)
    out = (ctypes.c_double * max(n, 1))()
    _call("sdv2_noise_schedule", ctypes.cast(d, _P), n, sigma, k, lam, s_min, s_max, s0, ctypes.cast(out, _P))
    return [out[i] for i in range(n)]


def sdv2_cache_slot_info(handle, slot: int) -> tuple[int, int]:
    f, p = _I64(), _I32()
    _call("sdv2_cache_slot_info", handle, slot, ctypes.byref(f), ctypes.byref(p))
    return f.value, p.value


def sdv2_cache_state(handle) -> tuple[int, int, int]:
    b, c, r = _I64(), _I64(), _I64()
    _call("sdv2_cache_state", handle, ctypes.byref(b), ctypes.byref(c), ctypes.byref(r))
    return b.value, c.value, r.value


def sdv2_plan_step(cfg: Config, num_chunks: int, step: int) -> tuple[int, int, int, int]:
    f, n, c, nf = _I64(), _I32(), _I64(), _I64()
    _call("sdv2_plan_step", ctypes.byref(cfg), num_chunks, step, ctypes.byref(f), ctypes.byref(n),
          ctypes.byref(c), ctypes.byref(nf))
    return f.value, n.value, c.value, nf.value


def sdv2_debug_fail_hip_call(nth: int) -> None:
    _call("sdv2_debug_fail_hip_call", nth)


def sdv2_debug_check_plan(cfg: Config, nbatch: int, nshared: int) -> tuple[int, int, int]:
    """(split count, split query tiles, working workgroups) of the checked plan."""
    ns, nt, wg = _I32(), _I32(), _I32()
    _call("sdv2_debug_check_plan", ctypes.byref(cfg), nbatch, nshared, ctypes.byref(ns), ctypes.byref(nt),
          ctypes.byref(wg))
    return ns.value, nt.value, wg.value


def sdv2_last_error() -> str:
    return lib().sdv2_last_error().decode()


# ---- convenience owner of the device buffers -------------------------------------------------
class Cache:
    """Allocates the cache's device buffers with torch and owns the C handle."""

    def __init__(self, cfg: Config, device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.layout = sdv2_cache_layout(cfg)
        kv_b, meta_b, ws_b = sdv2_cache_size(cfg)
        self.kv = torch.empty(kv_b, dtype=torch.uint8, device=device)
        self.meta = torch.empty(meta_b, dtype=torch.uint8, device=device)
        self.ws = torch.empty(max(ws_b, 256), dtype=torch.uint8, device=device)
        self.handle = sdv2_cache_create(cfg, self.kv, self.meta, self.ws, stream)
        # cache element type: fp32, bf16, or e4m3 bytes
        self.torch_dtype = {SDV2_F32: torch.float32, SDV2_BF16: torch.bfloat16}.get(cfg.dtype, torch.uint8)

    def close(self):
        if self.handle:
            sdv2_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # views of the device cache per the documented layout
    def _typed(self):
        return self.kv.view(self.torch_dtype)

    def k_view(self, layer: int):
        """K of one layer: [slots][H][tokens_padded][head_dim]."""
        L, c = self.layout, self.cfg
        base = layer * L.layer_stride
        return self._typed()[base:base + L.slots * L.slot_stride].view(
            L.slots, c.num_heads, L.tokens_padded, c.head_dim)

    def v_view(self, layer: int):
        """V of one layer, stored transposed: [slots][H][head_dim][tokens_padded]."""
        L, c = self.layout, self.cfg
        base = layer * L.layer_stride + L.slots * L.slot_stride
        return self._typed()[base:base + L.slots * L.slot_stride].view(
            L.slots, c.num_heads, c.head_dim, L.tokens_padded)

    def refresh(self, newest_frame, stream=None):
        return sdv2_rope_refresh(self.handle, newest_frame, stream)

    def append(self, layer, first_chunk, nbatch, q, k, v, stream=None):
        sdv2_cache_append(self.handle, layer, first_chunk, nbatch, q, k, v, stream)

    def attention(self, layer, nbatch, q_rot, out, scale, stream=None):
        sdv2_chunk_attention(self.handle, layer, nbatch, q_rot, out, scale, stream)

    def commit(self, chunk, stream=None):
        sdv2_cache_commit(self.handle, chunk, stream)

    def sink_replace(self, frame, embed=None, prev_latent=None, cur_latent=None, stats=None, sync=True,
                     stream=None):
        return sdv2_sink_replace(self.handle, frame, embed, prev_latent, cur_latent, stats, sync, stream)

    def slot_info(self, slot):
        return sdv2_cache_slot_info(self.handle, slot)

    def state(self):
        return sdv2_cache_state(self.handle)
