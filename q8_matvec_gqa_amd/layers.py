"""Device-side decode layers and MoE blocks built from host (numpy) arrays:
uploads with torch, fills the lq_layer_desc / lq_moe_desc descriptors and
owns the workspace.  Marshalling only; every computation runs in liblq."""
import numpy as np

from . import (LQ_FMT_Q4_0, LQ_FMT_Q6_K, lq_decode_layer, lq_decode_layer_workspace_size, lq_layer_desc,
               lq_layer_taps, lq_moe_block, lq_moe_block_workspace_size, lq_moe_desc, lq_moe_taps, lq_q4_0_pack_ggml,
               lq_q6_k_pack_ggml, lq_q8_weight, lq_rope_table, lq_rope_table_freqs, q4_0_weight, q6_k_weight,
               q8_weight)

PROJECTIONS = ("qkv", "o", "gu", "dn")     # lq_layer_desc.w_format order


def ggml_device_weight(fmt, blocks, rows, cols, torch):
    """GGML blocks (host, AoS) -> the library's SoA device arrays (packed by
    its host helper) and the matching weight descriptor."""
    if fmt == "q4_0":
        qs = np.zeros((rows, cols // 2), np.uint8)
        d = np.zeros((rows, cols // 32), np.uint16)
        lq_q4_0_pack_ggml(blocks, rows, cols, qs, d)
        return q4_0_weight(_dev(qs, torch), _dev(d, torch), rows, cols)
    ql = np.zeros((rows, cols // 2), np.uint8)
    qh = np.zeros((rows, cols // 4), np.uint8)
    sc = np.zeros((rows, cols // 16), np.int8)
    d = np.zeros((rows, cols // 256), np.uint16)
    lq_q6_k_pack_ggml(blocks, rows, cols, ql, qh, sc, d)
    return q6_k_weight(_dev(ql, torch), _dev(qh, torch), _dev(sc, torch), _dev(d, torch), rows, cols)


def _dev(a, torch):
    if isinstance(a, torch.Tensor):
        return a
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


class DeviceLayer:
    """Device buffers + lq_layer_desc for one decode layer (inputs `w`: numpy
    arrays, uploaded here, or device tensors, used as they are)."""

    def __init__(self, cfg, w, torch):
        self.cfg, self.torch = cfg, torch
        H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
        self.t = {k: _dev(v, torch) for k, v in w.items()
                  if k != "x" and not k.endswith(("_fmt", "_blocks", "_dev"))}
        c = np.zeros((cfg["max_ctx"], hd // 2), np.float32)
        s = np.zeros((cfg["max_ctx"], hd // 2), np.float32)
        if cfg.get("rope_freqs") is not None:
            lq_rope_table_freqs(cfg["max_ctx"], hd, cfg["theta"], np.ascontiguousarray(cfg["rope_freqs"], np.float32),
                                c, s)
        else:
            lq_rope_table(cfg["max_ctx"], hd, cfg["theta"], c, s)
        self.t["rope_cos"], self.t["rope_sin"] = _dev(c, torch), _dev(s, torch)
        t = self.t
        empty_w = lq_q8_weight(None, None, 0, 32)
        W = lambda name: q8_weight(t[name + "_qs"], t[name + "_d"]) if name + "_qs" in t else empty_w
        self.desc = lq_layer_desc(
            hidden=H, n_q=nq, n_kv=nkv, head_dim=hd, ffn=I, max_ctx=cfg["max_ctx"],
            window=cfg["window"], eps=cfg["eps"], attn_scale=cfg["attn_scale"], kind=cfg["kind"],
            kv_dtype=cfg["kv_dtype"], qk_norm=cfg["qk_norm"], v_unit_norm=cfg["v_unit_norm"],
            w_qkv=W("qkv"), w_o=W("o"),
            w_gate_up=W("gu") if I else empty_w, w_down=W("dn") if I else empty_w,
            g_in=t["g_in"].data_ptr(), g_q=t["g_q"].data_ptr(), g_k=t["g_k"].data_ptr(),
            g_post=t["g_post"].data_ptr(), k_cache=t["k_cache"].data_ptr(),
            v_cache=t["v_cache"].data_ptr(), rope_cos=t["rope_cos"].data_ptr(),
            rope_sin=t["rope_sin"].data_ptr(), ffn_act=cfg.get("ffn_act", 0),
            attn_softcap=cfg.get("attn_softcap", 0.0))
        # projections in GGML formats
        shapes = {"qkv": (nq * hd + 2 * nkv * hd, H), "o": (H, nq * hd), "gu": (2 * I, H), "dn": (H, I)}
        self.ggml = []
        for i, key in enumerate(PROJECTIONS):
            f = w.get(key + "_fmt")
            if f is None:
                continue
            # host GGML blocks (packed here), or a device weight built by the caller
            gw = w[key + "_dev"] if key + "_dev" in w else ggml_device_weight(f, w[key + "_blocks"], *shapes[key], torch)
            self.ggml.append(gw)                      # keeps the device arrays alive
            self.desc.w_format[i] = LQ_FMT_Q4_0 if f == "q4_0" else LQ_FMT_Q6_K
            if f == "q4_0":
                self.desc.w_q4_0[i] = gw
            else:
                self.desc.w_q6_k[i] = gw
        self.ws_bytes = lq_decode_layer_workspace_size(self.desc)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")

    def make_taps(self):
        torch, cfg = self.torch, self.cfg
        H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
        qd = nq * hd
        e = lambda n, dt: torch.empty(n, dtype=dt, device="cuda")
        bufs = dict(xq=e(H, torch.int8), xd=e(H // 32, torch.int16), qkv=e(qd + 2 * nkv * hd, torch.float32),
                    qkv_post=e(qd + 2 * nkv * hd, torch.float32),
                    attn=e(qd, torch.float32), aq=e(qd, torch.int8), ad=e(qd // 32, torch.int16),
                    x1=e(H, torch.float32))
        if I:
            bufs.update(nq=e(H, torch.int8), nd=e(H // 32, torch.int16), h=e(I, torch.float32),
                        hq=e(I, torch.int8), hd=e(I // 32, torch.int16))
        taps = lq_layer_taps(**{k: v.data_ptr() for k, v in bufs.items()})
        return taps, bufs

    def run(self, x, pos, taps=None, stream=None):
        lq_decode_layer(self.desc, x, pos, taps, self.ws, self.ws_bytes, stream=stream)


class DeviceMoe:
    def __init__(self, cfg, w, torch):
        self.cfg, self.torch = cfg, torch
        H, I, E, k = cfg["hidden"], cfg["ffn"], cfg["n_experts"], cfg["top_k"]
        self.t = {n: _dev(w[n], torch) for n in ("gu_qs", "gu_d", "dn_qs", "dn_d", "expert_scale") if n in w}
        t = self.t
        self.desc = lq_moe_desc(H, I, E, k,
                                   lq_q8_weight(t["gu_qs"].data_ptr(), t["gu_d"].data_ptr(), 2 * I, H),
                                   lq_q8_weight(t["dn_qs"].data_ptr(), t["dn_d"].data_ptr(), H, I),
                                   expert_scale=None if t.get("expert_scale") is None else t["expert_scale"].data_ptr())
        self.ws_bytes = lq_moe_block_workspace_size(self.desc, cfg["tokens"])
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")

    def make_taps(self):
        torch, c = self.torch, self.cfg
        T, H, I, k = c["tokens"], c["hidden"], c["ffn"], c["top_k"]
        e = lambda n, dt: torch.empty(n, dtype=dt, device="cuda")
        bufs = dict(ids=e(T * k, torch.int32), w=e(T * k, torch.float32), xq=e(T * H, torch.int8),
                    xd=e(T * H // 32, torch.int16), y1=e(T * k * 2 * I, torch.float32),
                    hq=e(T * k * I, torch.int8), hd=e(T * k * I // 32, torch.int16),
                    y2=e(T * k * H, torch.float32))
        return lq_moe_taps(**{n: v.data_ptr() for n, v in bufs.items()}), bufs

    def run(self, x, logits, out, taps=None, stream=None):
        lq_moe_block(self.desc, x, logits, self.cfg["tokens"], out, taps, self.ws, self.ws_bytes,
                        stream=stream)
