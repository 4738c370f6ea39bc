"""Drive the HIP path and the oracle side by side on the same seeded inputs (GPU tests only)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

from oracle import fp8 as ofp8
from oracle import motion as omotion
from oracle import rope as orope
from oracle import stream as ost
from rolling_kv_causal_amd import sdv2
from rolling_kv_causal_amd.stream import StreamRunner
from synth import inputs

BF16_MAX_ABS, BF16_MEAN_ABS, FP32_MAX_ABS = 2e-2, 2e-3, 1e-5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(cfg, arr):
    if cfg.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bits_of(x64: np.ndarray) -> np.ndarray:
    """bf16-exact float64 values -> their bit patterns."""
    return (np.asarray(x64, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def fp8_pos(i):
    """Byte position of element i in an e4m3 row of the cache (sdv2.h: bits 3 and 4 of i swap;
    the map is its own inverse, so it also gives the element at position i)."""
    i = np.asarray(i)
    return (i & ~24) | ((i & 8) << 1) | ((i & 16) >> 1)


def check_fp8_keys(got, want, refreshes, what):
    """Rotated e4m3 keys [.., d]: almost all bytes equal; where the kernel's fp32 rotation and the
    oracle's float64 one round to neighbouring codes (near-midpoint values, compounded by the
    re-rounding of each refresh), each pair stays within an e4m3 ulp per rounding."""
    same = np.mean(got == want)
    assert same >= 1 - 1e-3, f"{what}: only {same:.5f} of the key bytes agree"
    err = np.hypot(got[..., 0::2] - want[..., 0::2], got[..., 1::2] - want[..., 1::2])
    norm = np.hypot(want[..., 0::2], want[..., 1::2])
    assert np.all(err <= (refreshes + 1) * (2.0 ** -3 * norm + 2.0 ** -8)), f"{what}: key pair off by {err.max():.3g}"


def assert_close(cfg, got, want, what, scale=1.0):
    err = np.abs(np.asarray(got, np.float64) - want)
    if cfg.dtype == "fp32":
        assert err.max() <= FP32_MAX_ABS * scale, f"{what}: max-abs {err.max():.3g}"
    else:
        assert err.max() <= BF16_MAX_ABS * scale, f"{what}: max-abs {err.max():.3g}"
        assert err.mean() <= BF16_MEAN_ABS * scale, f"{what}: mean-abs {err.mean():.3g}"
    return float(err.max())


class Harness:
    """GPU stream + oracle stream.  Layers in `layers` get seeded numpy inputs for element 0 at
    every step (so the oracle knows every cached frame) and for all elements at checked steps;
    other (layer, element) pairs get device-side random inputs."""

    def __init__(self, cfg, layers, num_chunks=None, seed=1234, motion_cfg=None, sink_sync=True):
        self.cfg = cfg
        # sink_sync False: sdv2_sink_replace with h_slot NULL, the decision stays on the device
        # and the host's slot table reports the sink slots as unknown after the first decision
        self.sink_sync = sink_sync
        self.sinks_unknown = False
        self.kmul = float(np.float32(cfg.key_scale * np.log2(np.e))) if cfg.key_scale > 0 else 1.0
        self.layers = list(layers)
        self.M = cfg.num_chunks if num_chunks is None else num_chunks
        self.ccfg = sdv2.config_of(cfg)
        self.run = StreamRunner(self.ccfg, cfg.num_chunks, cfg.softmax_scale)
        self.st = ost.OracleStream(cfg, layers=self.layers)
        self.gen = torch.Generator(device="cuda")
        self.gen.manual_seed(seed)
        self.np_inputs = {}
        self.refresh_applied = {}
        self.decisions = {}
        self.step_no = -1
        # fused chunk statistics: fp64 [4 + 2S] per commit; the motion term from the workload's
        # latent series (frame f against f - 1) where it has one
        self.stats = torch.full((4 + 2 * cfg.sink_frames,), float("nan"), dtype=torch.float64, device="cuda")
        self.frames = None
        if (motion_cfg or cfg).motion is not None:
            self.frames_np = inputs.motion_frames(motion_cfg or cfg)
            self.frames = torch.from_numpy(self.frames_np).cuda()
        self.stats_checked = 0

    def _random(self, nb):
        shape = (nb, self.cfg.chunk_rows, self.cfg.num_heads, self.cfg.head_dim)
        x = torch.randn(shape, generator=self.gen, device="cuda")
        return x.to(self.run.dtype)

    def step(self, s, full=False):
        """Advance both sides one step; full = numpy inputs for every element of the layers."""
        cfg = self.cfg
        plan = self.st.begin_step(s)
        nb = len(plan["chunks"])
        self.np_inputs = {}
        for layer in self.layers:
            for b in (range(nb) if full else [0]):
                self.np_inputs[(layer, b)] = inputs.qkv(cfg, s, layer, b)

        def qkv(s_, layer, nb_):
            out = []
            for j in range(3):
                t = self._random(nb_)
                for b in range(nb_):
                    if (layer, b) in self.np_inputs:
                        t[b] = dev(cfg, self.np_inputs[(layer, b)][j])
                out.append(t)
            return tuple(out)

        emb = None
        if cfg.embed_dim > 0:
            emb = lambda c: dev(cfg, inputs.chunk_embedding(cfg, c))
        lat = None
        if self.frames is not None:
            lat = lambda f: ((self.frames[f - 1], self.frames[f]) if 1 <= f < len(self.frames) else None)
        self.stats.fill_(float("nan"))
        info = self.run.step(s, qkv, embed=emb, latents=lat, stats=self.stats, sink_sync=self.sink_sync)
        self.refresh_applied[s] = info["refreshed"]
        commit_kv = {layer: self.np_inputs[(layer, 0)][1:] for layer in self.layers}
        h = inputs.chunk_embedding(cfg, plan["commit"]) if (cfg.embed_dim > 0 and plan["commit"] is not None) else None
        self._pending = (plan, info, commit_kv, h)
        self.step_no = s
        return plan, info

    def finish_step(self):
        plan, info, commit_kv, h = self._pending
        dec = self.st.end_step(commit_kv, h)
        if dec is not None:
            self.decisions[plan["commit"]] = (dec, info["sink"])
            if self.sink_sync:
                want = dec["slot"] if dec["replaced"] else -1
                assert info["sink"][0] == want, f"sink decision chunk {plan['commit']}: gpu {info['sink']} oracle {dec}"
                assert abs(info["sink"][1] - dec["alpha"]) <= 1e-9, (info["sink"], dec)
            else:                          # decided on the device; alpha is checked in the stats
                assert info["sink"] is None
                self.sinks_unknown = True
        if plan["commit"] is not None:
            self._check_stats(plan, dec)
        # refresh events must match the oracle's
        n_ref = sum(1 for (s_, _) in self.st.refresh_log if s_ == self.step_no)
        assert self.refresh_applied[self.step_no] == n_ref, (self.step_no, self.refresh_applied[self.step_no], n_ref)
        return dec

    def _check_stats(self, plan, dec):
        """The fused statistics of this commit against oracle.motion (the newest latent frame's
        distance) and oracle.sink (h.h, e.e, h.e, alpha of the decision), rtol 1e-12."""
        cfg, S = self.cfg, self.cfg.sink_frames
        st = self.stats.cpu().numpy()
        f = (plan["commit"] + 1) * cfg.chunk_frames - 1
        if self.frames is not None and 1 <= f < len(self.frames_np):
            d = omotion.frame_distances(self.frames_np[f - 1:f + 1])[0]
            n = self.frames_np[f].size
            np.testing.assert_allclose(st[1], d, rtol=1e-12, atol=0)
            np.testing.assert_allclose(st[0], d * d * n, rtol=1e-12, atol=0)
            self.stats_checked += 1
        else:
            assert np.isnan(st[0]) and np.isnan(st[1])
        if dec is not None:
            t = dec["terms"]
            np.testing.assert_allclose(st[2], t["hh"], rtol=1e-12, atol=0)
            np.testing.assert_allclose(st[3:3 + S], t["ee"], rtol=1e-12, atol=0)
            # h.e may cancel to near zero: its bar scales with |h| |e_j|
            he_bar = 1e-12 * (np.abs(t["he"]) + np.sqrt(t["hh"] * np.array(t["ee"])))
            assert np.all(np.abs(st[3 + S:3 + 2 * S] - t["he"]) <= he_bar), (st[3 + S:3 + 2 * S], t["he"])
            assert abs(st[3 + 2 * S] - dec["alpha"]) <= 1e-12
            self.stats_checked += 1
        elif cfg.embed_dim == 0:
            assert np.all(np.isnan(st[2:]))

    def check_outputs(self, rows=None, heads=None, rotated="exact"):
        """Compare the current step's outputs of every element on the checked layers."""
        cfg = self.cfg
        plan = self.st.plan
        worst = 0.0
        for layer in self.layers:
            for b in range(len(plan["chunks"])):
                q, k, v = self.np_inputs[(layer, b)]
                ref = self.st.attend(layer, b, q, k, v, rows=rows, heads=heads, rotated=rotated)
                got = self.run.out[layer, b]
                if rows is not None:
                    got = got[torch.as_tensor(rows, device="cuda")]
                if heads is not None:
                    got = got[:, torch.as_tensor(heads, device="cuda")]
                worst = max(worst, assert_close(cfg, host64(got), ref, f"out step {self.step_no} layer {layer} elem {b}"))
                if rows is None and cfg.tokens >= 1024:
                    log(f"  {cfg.name} step {self.step_no} layer {layer} elem {b}: all rows ok, worst {worst:.3g}")
        return worst

    def check_cache(self, layers=None):
        """Slot table bit-exact (frame and label per slot, each window frame in the slot the
        oracle's ring_slot() gives it), V bytes bit-exact, K_rot within tolerance."""
        cfg = self.cfg
        N = cfg.tokens
        r = len(self.st.refresh_log)
        cache = self.run.cache
        base, committed, refreshes = cache.state()
        assert base == self.st.base and refreshes == r
        entries = [(j, e) for j, e in enumerate(self.st.sinks) if e is not None]
        entries += [(ost.ring_slot(cfg, e.frame), e) for e in self.st.window]
        # every other sink / ring slot is empty, or holds a frame of the staged (not yet
        # committed) chunk written there by this step's append
        held = {slot for slot, _ in entries}
        T = cfg.chunk_frames
        for slot in range(cfg.sink_frames + cfg.window_frames + T):
            if slot not in held:
                f = cache.slot_info(slot)[0]
                assert f == -1 or (committed * T <= f < (committed + 1) * T and slot == ost.ring_slot(cfg, f)), \
                    (slot, f, committed)
        if self.st.kv_fp8:
            return self._check_cache_fp8(entries, r, layers)
        for layer in (self.layers if layers is None else layers):
            Kg, Vg = cache.k_view(layer), cache.v_view(layer)
            for slot, e in entries:
                self._check_slot_info(slot, e)
                k_ref = orope.rope_frame(cfg, e.kv[layer][0], e.label)
                # a cache with a key scale holds K times the fp32 value of key_scale * log2(e)
                k_got = host64(Kg[slot, :, :N, :].permute(1, 0, 2)) / self.kmul
                assert_close(cfg, k_got, k_ref, f"K slot {slot} frame {e.frame}", scale=1 + r)
                v_got = Vg[slot, :, :, :N].permute(2, 0, 1).contiguous()
                if cfg.dtype == "bf16":
                    got_bits = v_got.view(torch.int16).cpu().numpy().view(np.uint16)
                    assert np.array_equal(got_bits, bf16_bits_of(e.kv[layer][1])), f"V bytes slot {slot}"
                else:
                    assert np.array_equal(v_got.cpu().numpy(), np.asarray(e.kv[layer][1], np.float32)), f"V slot {slot}"
            # zero padding of the token axis stays zero
            if cache.layout.tokens_padded > N:
                assert torch.count_nonzero(Kg[:, :, N:, :]) == 0 and torch.count_nonzero(Vg[:, :, :, N:]) == 0


    def _check_slot_info(self, slot, e):
        """Frame and label of a slot against the oracle's entry.  After a sink decision taken
        on the device only (sink_sync False), the library reports its sink slots as unknown
        (frame -2): the bytes checked after this must still be the oracle's sink."""
        info = self.run.cache.slot_info(slot)
        if self.sinks_unknown and slot < self.cfg.sink_frames:
            assert info[0] == -2, (slot, info)
        else:
            assert info == (e.frame, e.label), (slot, info, e.frame, e.label)

    def _check_cache_fp8(self, entries, r, layers):
        """e4m3 cache: V bytes bit-exact against the oracle's encoding, K per check_fp8_keys,
        padding tokens zero; rows read back through the documented byte permutation."""
        cfg, cache = self.cfg, self.run.cache
        N, D, Npad = cfg.tokens, cfg.head_dim, cache.layout.tokens_padded
        dperm = torch.as_tensor(fp8_pos(np.arange(D)), device="cuda")
        tperm = torch.as_tensor(fp8_pos(np.arange(Npad)), device="cuda")
        for layer in (self.layers if layers is None else layers):
            Kg = cache.k_view(layer)[..., dperm]                     # [slot][H][Npad][d], d in order
            Vg = cache.v_view(layer)[..., tperm]                     # [slot][H][d][Npad], tokens in order
            for slot, e in entries:
                self._check_slot_info(slot, e)
                k_codes = Kg[slot, :, :N, :].permute(1, 0, 2).cpu().numpy()
                check_fp8_keys(ofp8.decode(k_codes), e.kv[layer][0], r, f"K slot {slot} frame {e.frame}")
                v_codes = Vg[slot, :, :, :N].permute(2, 0, 1).cpu().numpy()
                assert np.array_equal(v_codes, ofp8.encode(e.kv[layer][1])), f"V bytes slot {slot}"
            if Npad > N:
                assert torch.count_nonzero(Kg[:, :, N:, :]) == 0 and torch.count_nonzero(Vg[:, :, :, N:]) == 0


def sample_rows(N, n=40, seed=0):
    g = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, N // 2, N - 2, N - 1]
    return np.array(sorted(set([x for x in fixed if 0 <= x < N] + list(g.choice(N, min(n, N), replace=False)))))
