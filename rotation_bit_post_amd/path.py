"""One decoder layer's linear path on the device, built from the C-ABI entry points.

Per layer (two correction sites, one at the attention input and one at the
FFN input, as each of the MHSA and FFN blocks carries its own rotations,
zh 2.2):

  site A: rsq_correct_quant  h -> h_A, codes, scales      (correction + RMSNorm + quant)
          rsq_qgemm          -> y_qkv                     (fused q|k|v weights)
          rsq_quant_act      o_proj input -> codes
          rsq_qgemm          -> y_o
  site B: rsq_correct_quant  h_A -> h_B, codes, scales
          rsq_qgemm          -> y_gate_up                 (fused gate|up weights)
          rsq_quant_act      down_proj input -> codes
          rsq_qgemm          -> y_down

The attention core and SiLU * up are outside this path: the o_proj and
down_proj inputs are fixed stand-ins. The residual adds are taken in with
``stages(chain=True)``: the o_proj and down_proj outputs are added to the
corrected residual in the GEMM epilogue (rsq_qgemm_residual) and site B reads
the sum. With ``correction=False``
each site runs RMSNorm + quantisation only (rsq_quant_act), the cost of a
single global rotation (T = I), for the overhead comparison.

Weights are quantised on the device with rsq_quant_act (per output channel,
no norm); the sites come from ``offline.convert_site`` and rsq_site_prepare.

3-bit codes at prefill sizes (more than 64 tokens) run on the fp4 matrix
cores: the weights are converted once (rsq_codes_to_fp4), the sites and the
stand-in quantisations write their codes in the fp4 layout (bits = 3 |
RSQ_FP4) and the GEMMs are rsq_qgemm_fp4 / its residual form; the results
are the same bits as with int3 codes.
"""
from __future__ import annotations

import time

from dataclasses import dataclass, field

import numpy as np
import torch

from . import _binding as B
from . import offline
from synth import Workload, layer_linears, workload
from synth import generators as G


def _dev_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 array of bf16-exact values -> bf16 device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(torch.bfloat16)


def _dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return t if dtype is None else t.to(dtype)


@dataclass
class Site:
    r: int
    U: torch.Tensor
    M: torch.Tensor
    buf: torch.Tensor


@dataclass
class QLinear:
    name: str
    N: int
    K: int
    codes: torch.Tensor
    scales: torch.Tensor
    source: str = ""
    fp4: torch.Tensor | None = None   # the 3-bit codes as fp4 rows, when the fp4 GEMM is used


def make_site(U: np.ndarray, M: np.ndarray) -> Site:
    d, r = U.shape
    buf = torch.empty(B.rsq_site_bytes(d, r), dtype=torch.uint8, device="cuda")
    Ud, Md = _dev(U.astype(np.float32)), _dev(M.astype(np.float32))
    B.rsq_site_prepare(Ud, Md, buf)
    return Site(r, Ud, Md, buf)


def quantize_weight_on_device(w: np.ndarray, bits: int, name: str = "") -> QLinear:
    """Per-output-channel quantisation of a float32 weight with the library's kernel."""
    N, K = w.shape
    wd = _dev(w.astype(np.float32))
    codes = torch.empty((N, B.rsq_packed_row_bytes(K, bits)), dtype=torch.uint8, device="cuda")
    scales = torch.empty(N, dtype=torch.float32, device="cuda")
    B.rsq_quant_act(wd, codes, scales, bits, rmsnorm=False)
    del wd
    return QLinear(name, N, K, codes, scales)


def synthetic_mismatch(cfg: Workload, which: str) -> np.ndarray:
    """T (float64) of a synthetic site: rotations H C(eps A) from the seeded skew generators."""
    r_in = offline.synthetic_rotation(G.skew_generator(cfg, which, "in"), cfg.eps_rot)
    r_out = offline.synthetic_rotation(G.skew_generator(cfg, which, "out"), cfg.eps_rot)
    return offline.mismatch(r_in, r_out)


def synthetic_site(cfg: Workload, which: str, r: int):
    """(U_r, M) of a synthetic site."""
    return offline.convert_mismatch(synthetic_mismatch(cfg, which), r)


@dataclass
class LayerPath:
    cfg: Workload
    n: int
    r: int
    gqa: bool = True
    eps: float = 1e-5
    sites: dict = field(default_factory=dict)
    linears: dict = field(default_factory=dict)
    bufs: dict = field(default_factory=dict)
    mismatch: dict = field(default_factory=dict)   # site -> T (float32), kept on request
    prep_info: dict = field(default_factory=dict)  # site -> how its (U_r, M) was prepared
    fp4: bool = False                              # 3-bit GEMMs on fp4 codes

    @classmethod
    def build(cls, wl, n: int | None = None, r: int | None = None, gqa: bool = True,
              sites=None, weights=None, keep_mismatch: bool = False, prep: str = "host",
              fp4: bool | None = None) -> "LayerPath":
        """Device-resident inputs and outputs of one layer path.

        wl: the workload (a name from synth.WORKLOADS, its position there, or
        the Workload itself). sites: optional {"A": (U, M), "B": (U, M)}; weights: optional
        {linear name: float32 (N, K)} - both default to the seeded synthetic ones.
        keep_mismatch: also keep each synthetic site's dense T (for comparisons).
        prep: "host" (float64 eigensolver on the CPU) or "device" (float64
        block subspace iteration on the GPU) for the synthetic sites.
        fp4: run the 3-bit GEMMs on fp4 codes; default: for 3-bit codes and
        more than 64 tokens (the decode-size batches keep the int8 kernels).
        """
        cfg = workload(wl)
        self = cls(cfg, n or cfg.n, r or cfg.r, gqa)
        self.fp4 = (cfg.bits == 3 and self.n > 64) if fp4 is None else bool(fp4)
        if self.fp4 and cfg.bits != 3:
            raise ValueError("fp4 holds 3-bit codes only")
        lins = layer_linears(cfg, gqa)
        names = sorted({l.source for l in lins if l.source.startswith("site")})
        for src in names:
            which = src[-1]
            if sites is not None:
                U, M = sites[which]
            elif prep == "device":
                from . import offline_device as OD
                t0 = time.perf_counter()
                r_in = OD.synthetic_rotation_device(G.skew_generator(cfg, which, "in"), cfg.eps_rot)
                r_out = OD.synthetic_rotation_device(G.skew_generator(cfg, which, "out"), cfg.eps_rot)
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                U, M, iters, res = OD.convert_site_device(r_in, r_out, self.r)
                t2 = time.perf_counter()
                if keep_mismatch:
                    self.mismatch[which] = (r_out.T @ r_in).to(torch.float32).cpu().numpy()
                self.prep_info[which] = {"where": "device", "rotations_s": round(t1 - t0, 3),
                                         "subspace_s": round(t2 - t1, 3), "iterations": iters, "residual": res}
                del r_in, r_out
            else:
                t0 = time.perf_counter()
                t = synthetic_mismatch(cfg, which)
                t1 = time.perf_counter()
                U, M = offline.convert_mismatch(t, self.r)
                self.prep_info[which] = {"where": "host", "rotations_s": round(t1 - t0, 3),
                                         "subspace_s": round(time.perf_counter() - t1, 3)}
                if keep_mismatch:
                    self.mismatch[which] = t.astype(np.float32)
                del t
            self.sites[which] = make_site(U, M)
        for lin in lins:
            if weights is not None:
                w = weights[lin.name]
            else:
                w = np.concatenate([G.weight(cfg, part, rows, lin.K) for part, rows in lin.parts], axis=0)
            q = quantize_weight_on_device(w, cfg.bits, lin.name)
            q.source = lin.source
            if self.fp4:
                q.fp4 = torch.empty((q.N, q.K // 2), dtype=torch.uint8, device="cuda")
                B.rsq_codes_to_fp4(q.codes, q.N, q.K, q.fp4)
            self.linears[lin.name] = q
            del w
        self._alloc()
        return self

    def clone(self) -> "LayerPath":
        """An independent copy of every device buffer (same values)."""
        other = LayerPath(self.cfg, self.n, self.r, self.gqa, self.eps, fp4=self.fp4)
        other.sites = {k: Site(v.r, v.U.clone(), v.M.clone(), v.buf.clone()) for k, v in self.sites.items()}
        other.linears = {k: QLinear(v.name, v.N, v.K, v.codes.clone(), v.scales.clone(), v.source,
                                    None if v.fp4 is None else v.fp4.clone())
                         for k, v in self.linears.items()}
        other.bufs = {k: v.clone() for k, v in self.bufs.items()}
        return other

    @property
    def code_bits(self) -> int:
        """The `bits` argument of the quantising entry points: the code format written."""
        return (3 | B.RSQ_FP4) if self.fp4 else self.cfg.bits

    def _alloc(self):
        cfg, n, bits = self.cfg, self.n, self.code_bits
        hdt = torch.bfloat16 if cfg.h_dtype == "bf16" else torch.float32
        ydt = torch.bfloat16 if cfg.y_dtype == "bf16" else torch.float32
        h = G.residual(cfg, n)
        self.bufs["h"] = _dev_bf16(h) if hdt == torch.bfloat16 else _dev(h)
        for which in self.sites:
            self.bufs[f"h_{which}"] = torch.empty_like(self.bufs["h"])
        if "B" in self.sites:   # residual stream after the attention and after the FFN block
            self.bufs["h2"] = torch.empty_like(self.bufs["h"])
            self.bufs["h3"] = torch.empty_like(self.bufs["h"])
        for which in self.sites:
            self.bufs[f"codes_{which}"] = torch.empty((n, B.rsq_packed_row_bytes(cfg.D, bits)), dtype=torch.uint8, device="cuda")
            self.bufs[f"scales_{which}"] = torch.empty(n, dtype=torch.float32, device="cuda")
        # one workspace for every stage (they run one after another on one stream)
        need = [B.rsq_correct_workspace_bytes(n, cfg.D)]
        need += [B.rsq_qgemm_workspace_bytes(n, lin.N, lin.K, bits) for lin in self.linears.values()]
        self.bufs["workspace"] = B.rsq_workspace(max(need))
        for name, lin in self.linears.items():
            self.bufs[f"y_{name}"] = torch.empty((n, lin.N), dtype=ydt, device="cuda")
            if lin.source in ("o_in", "down_in"):
                x = G.linear_input(cfg, lin.source, n, lin.K)
                self.bufs[lin.source] = _dev_bf16(x) if hdt == torch.bfloat16 else _dev(x)
                self.bufs[f"codes_{lin.source}"] = torch.empty((n, B.rsq_packed_row_bytes(lin.K, bits)), dtype=torch.uint8, device="cuda")
                self.bufs[f"scales_{lin.source}"] = torch.empty(n, dtype=torch.float32, device="cuda")

    # ------------------------------------------------------------------ run
    def stages(self, correction: bool = True, chain: bool = False):
        """The path as a list of (stage name, kind, callable); kind is "site", "quant" or "gemm".

        chain: carry the residual stream through the layer - the o_proj output
        is added to site A's corrected residual (giving h2, site B's input) and
        the down_proj output to site B's (giving h3, the next layer's input),
        both inside the GEMM epilogue. Without it, site B reads site A's output
        and the o / down outputs are separate tensors.
        """
        cfg, bits, b = self.cfg, self.code_bits, self.bufs
        ws = b["workspace"]
        if chain and "B" not in self.sites:
            raise ValueError("a chained layer needs both sites")
        out = []
        h_cur = b["h"]
        order = ["A", "B"] if "B" in self.sites else ["A"]
        for which in order:
            site = self.sites[which]
            h_in, h_out = h_cur, b[f"h_{which}"]
            codes, scales = b[f"codes_{which}"], b[f"scales_{which}"]
            if correction:
                fn = (lambda h_in=h_in, h_out=h_out, site=site, codes=codes, scales=scales:
                      B.rsq_correct_quant(h_in, h_out, site.buf, site.r, codes, scales, bits, eps=self.eps,
                                          workspace=ws))
            else:
                fn = (lambda h_in=h_in, codes=codes, scales=scales:
                      B.rsq_quant_act(h_in, codes, scales, bits, rmsnorm=True, eps=self.eps))
            out.append((f"site{which}", "site" if correction else "quant", fn))
            for lin in self.linears.values():
                if lin.source == f"site{which}":
                    out.append(self._gemm(lin, codes, scales))
                    break
            h_cur = h_out if correction else h_in
            stand_in = "o_in" if which == "A" else "down_in"
            for lin in self.linears.values():
                if lin.source == stand_in:
                    x, c, s = b[stand_in], b[f"codes_{stand_in}"], b[f"scales_{stand_in}"]
                    out.append((f"quant_{stand_in}", "quant",
                                lambda x=x, c=c, s=s: B.rsq_quant_act(x, c, s, bits, rmsnorm=False)))
                    if chain:
                        dst = b["h2"] if which == "A" else b["h3"]
                        out.append(self._gemm(lin, c, s, residual=h_cur, dst=dst))
                        h_cur = dst
                    else:
                        out.append(self._gemm(lin, c, s))
        return out

    def _gemm(self, lin: QLinear, codes, scales, residual=None, dst=None):
        """The stage of one linear; with a residual the result goes to dst (added in the epilogue)."""
        n, bits, ws = self.n, self.cfg.bits, self.bufs["workspace"]
        name = f"gemm_{lin.name}" + ("_res" if residual is not None else "")
        y = dst if residual is not None else self.bufs[f"y_{lin.name}"]
        if self.fp4:
            return (name, "gemm", lambda: B.rsq_qgemm_fp4(codes, scales, n, lin.fp4, lin.scales, lin.N, lin.K, y,
                                                         residual=residual, workspace=ws))
        if residual is not None:
            return (name, "gemm", lambda: B.rsq_qgemm_residual(codes, scales, n, lin.codes, lin.scales, lin.N, lin.K,
                                                                bits, residual, y, workspace=ws))
        return (name, "gemm", lambda: B.rsq_qgemm(codes, scales, n, lin.codes, lin.scales, lin.N, lin.K, bits, y,
                                                   workspace=ws))

    def step(self, correction: bool = True, chain: bool = False):
        for _, _, fn in self.stages(correction, chain):
            fn()

    def outputs(self, chain: bool = False):
        """Every tensor a step writes (for comparing two ways of running it)."""
        keys = [k for k in self.bufs if k.startswith(("h_", "codes_", "scales_", "y_")) or k in ("h2", "h3")]
        if chain:   # the o / down results land on the residual stream instead
            keys = [k for k in keys if k not in ("y_o", "y_down")]
        else:
            keys = [k for k in keys if k not in ("h2", "h3")]
        return {k: self.bufs[k] for k in sorted(keys)}

    def capture(self, correction: bool = True, chain: bool = False):
        """One step recorded as a HIP graph (launches only: the step allocates
        nothing and sets no memory), replayed with ``graph.replay()``."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step(correction, chain)      # first launches of every kernel outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step(correction, chain)
        return graph

    # -------------------------------------------------- algorithmic work
    def stage_work(self, name: str):
        """(algorithmic bytes, algorithmic integer ops) of one stage launch."""
        cfg, n = self.cfg, self.n
        cb = 4 if self.fp4 else cfg.bits   # bits per stored code (fp4 codes take a nibble)
        hs = 2 if cfg.h_dtype == "bf16" else 4
        ys = 2 if cfg.y_dtype == "bf16" else 4
        if name.startswith("site"):
            r = self.r
            return (n * (2 * cfg.D * hs + cfg.D * cb // 8 + 4) + 4 * cfg.D * r + 4 * r * r, 0)
        if name.startswith("quant_"):
            k = self.linears["o"].K if name == "quant_o_in" else self.linears["down"].K
            return (n * (k * hs + k * cb // 8 + 4), 0)
        res = name.endswith("_res")
        lin = self.linears[name[len("gemm_"):len(name) - (4 if res else 0)]]
        byts = lin.N * lin.K * cb // 8 + 4 * lin.N + n * (lin.K * cb // 8 + 4) + n * lin.N * ys
        if res:
            byts += n * lin.N * hs   # the residual read beside the output write
        return (byts, 2 * n * lin.N * lin.K)
