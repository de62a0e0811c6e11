"""Shared pieces of the GPU parity tests: seeded cases, the oracle reference, comparisons.

Inputs come from the seeded generator; expected values come from the fp64 oracle only."""
import functools
import json
import os

import numpy as np
import torch

import moe_speculative_decode_amd as mdl
from moe_speculative_decode_amd import device as dev
from moe_speculative_decode_amd import synth
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# max-abs(y_gpu - y_oracle) / rms(y_oracle) bars: bf16 and MXFP4 from the layer's accuracy target;
# FP8 weights take the bf16 bar (the oracle dequantises the same codes exactly, so only the bf16
# rounding of the SwiGLU rows and of y remains, as for bf16 weights); fp32 derived from fp32
# accumulation over K <= 4096 terms (relative error well below 1e-5)
TOL = {synth.F32: 1e-4, synth.BF16: 2e-2, synth.MXFP4: 5e-2, synth.FP8: 2e-2}
W_TOL = 1e-5  # routing weights, absolute


SUMMARY = []  # every logged line, repeated in the run's terminal summary (conftest)


def log(*a):
    line = " ".join(str(x) for x in a)
    SUMMARY.append(line)
    print("[gpu-test]", line, flush=True)


def _layer_key(cfg):
    """Everything the layer's weights depend on (not the token workload)."""
    return (cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter, cfg.shared_inter, cfg.act_fmt, cfg.weight_fmt,
            cfg.layer_seed, cfg.router_norm, cfg.router_bias)


@functools.lru_cache(maxsize=4)
def _host_layer(key):
    H, E, k, I, Is, af, wf, seed, rn, rb = key
    return synth.Layer(synth.LayerConfig("layer", H, E, k, I, Is, af, wf, (1,), "iid", seed, router_norm=rn,
                                         router_bias=rb))


@functools.lru_cache(maxsize=2)
def _device_layer(key):
    return dev.DeviceLayer(_host_layer(key))


def host_layer(cfg):
    return _host_layer(_layer_key(cfg))


def device_layer(cfg):
    return _device_layer(_layer_key(cfg))


def seeds():
    return json.load(open(os.path.join(GOLDEN, "seeds.json")))


def accepted_hidden(cfg, layer, min_gap=1e-3, start=0):
    d = O.layer_desc(cfg)
    for s in range(start, start + 500):
        x = synth.make_hidden(cfg, s)
        if O.route(d, x, layer.router, **O.router_aux(layer))[3].min() >= min_gap:
            return x, s
    raise RuntimeError("no accepted hidden seed")


class Case:
    """One seeded workload on the device plus the oracle's answer."""

    def __init__(self, cfg, x_host=None, hidden_seed=None, layer_cfg=None, oracle_threads=0):
        self.cfg = cfg
        lcfg = layer_cfg or cfg
        self.layer = host_layer(lcfg)
        self.dl = device_layer(lcfg)
        if x_host is None:
            if hidden_seed is None:
                x_host, hidden_seed = accepted_hidden(cfg, self.layer)
            else:
                x_host = synth.make_hidden(cfg, hidden_seed)
        self.x_host = np.ascontiguousarray(x_host)
        self.M = self.x_host.shape[0]
        self.desc = dev.desc_of(cfg, max_tokens=max(self.M, cfg.M), layer=self.dl)
        self.x = dev.to_device(self.x_host)
        self.ws = dev.workspace(self.desc)
        d = O.layer_desc(cfg)
        self.y_ref, self.ids_ref, self.w_ref, self.gap = O.forward(d, O.layer_weights(self.layer), self.x_host,
                                                                   self.layer.router, threads=oracle_threads,
                                                                   **O.router_aux(self.layer))
        self.comp_ref = O.compact(self.ids_ref, self.w_ref, cfg.num_experts)

    def run(self, req_offsets=None, disp=None, stream=None, x=None):
        M, H, k = self.M, self.cfg.hidden, self.cfg.top_k
        y = torch.empty((M, H), dtype=dev.act_dtype(self.cfg), device="cuda")
        ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((M, k), -1.0, dtype=torch.float32, device="cuda")
        off = None if req_offsets is None else torch.tensor(req_offsets, dtype=torch.int32, device="cuda")
        R = 0 if req_offsets is None else len(req_offsets) - 1
        mdl.moe_decode_forward(self.desc, M, self.x if x is None else x, self.dl.router, self.dl.weights(), y,
                               self.ws, req_offsets=off, R=R, topk_ids=ids, topk_w=w,
                               disp=None if disp is None else disp.struct(), stream=stream)
        return y, ids, w


def y_error(y_gpu: torch.Tensor, y_ref: np.ndarray):
    yg = y_gpu.float().cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    return float(np.max(np.abs(yg - y_ref)) / rms), rms


def check_routing(ids_gpu, w_gpu, ids_ref, w_ref):
    ids_g = ids_gpu.cpu().numpy()
    w_g = w_gpu.cpu().numpy().astype(np.float64)
    for m in range(ids_ref.shape[0]):
        assert set(ids_g[m].tolist()) == set(ids_ref[m].tolist()), (m, ids_g[m], ids_ref[m])
        ref = dict(zip(ids_ref[m].tolist(), w_ref[m].tolist()))
        for e, wv in zip(ids_g[m].tolist(), w_g[m].tolist()):
            assert abs(wv - ref[e]) <= W_TOL, (m, e, wv, ref[e])
        assert np.all(np.diff(w_g[m]) <= 1e-7), "weights not in descending order"


def check_dispatch(d: dev.DispatchOut, comp_ref, ids_gpu, ids_ref, w_ref, M, k, has_shared=True):
    """Units, offsets and row tokens are unique and compared exactly; a row's slot refers to the
    GPU's own top-k order (which may legitimately differ from the oracle's on sub-1e-5 near-ties
    inside the top-k), so it is checked to point at the row's expert, and its weight against the
    oracle's weight of that (token, expert)."""
    U = comp_ref["U"]
    nu = U + (1 if has_shared else 0)
    assert int(d.unit_count.item()) == U
    ue = d.unit_expert.cpu().numpy()
    uo = d.unit_off.cpu().numpy()
    assert ue[:nu].tolist() == comp_ref["unit_expert"][:nu].tolist()
    assert uo[:nu + 1].tolist() == comp_ref["unit_off"][:nu + 1].tolist()
    n = M * k + (M if has_shared else 0)
    rt = d.row_token.cpu().numpy()[:n]
    rs = d.row_slot.cpu().numpy()[:n]
    rw = d.row_weight.cpu().numpy()[:n].astype(np.float64)
    assert rt.tolist() == comp_ref["row_token"][:n].tolist()
    ids_g = ids_gpu.cpu().numpy()
    for u in range(nu):
        for r in range(uo[u], uo[u + 1]):
            m = rt[r]
            if u < U:
                assert ids_g[m, rs[r]] == ue[u]
                wref = w_ref[m][list(ids_ref[m]).index(ue[u])]
                assert abs(rw[r] - wref) <= W_TOL
            else:
                assert rs[r] == k and rw[r] == 1.0
