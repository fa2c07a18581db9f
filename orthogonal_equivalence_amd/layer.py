"""POET-X linear layers on top of the libpoetx binding.

PoetxLinear holds the device buffers of one layer (theta, orthogonal blocks,
workspaces) allocated with torch and drives the three library calls;
PoetxLinearSet puts several layers' generators and blocks into shared buffers
so that one build call rebuilds all of them. Both allocate and call; every
step of the computation runs in libpoetx's kernels.
"""
from __future__ import annotations

import torch

from . import poetx as P

_DT = {"f32": (torch.float32, P.POETX_F32), "bf16": (torch.bfloat16, P.POETX_BF16)}


class PoetxLinear:
    """y = R W0 P x for token-major x [tokens, d_in]; W0 [d_out, d_in] frozen.

    theta_R [nb_out, b_out(b_out-1)/2] and theta_P [nb_in, b_in(b_in-1)/2]
    are float32 views into one buffer, so that both block sets are built by a
    single poetx_build_orthogonal call when b_in == b_out and b divides both
    d_in and d_out.

    recompute_z=True is the memory-saving variant: the forward keeps no
    Z = W0 P x for the backward, which recomputes it (POETX_RECOMPUTE_Z).
    saved_y=True keeps nothing beside y: the backward takes y in place of Z
    (POETX_SAVED_Y; per block Z = Y R for orthogonal R), for callers that
    keep y anyway. forward() returns (y, saved), saved being what backward()
    takes as z: Z, y itself with saved_y, None with recompute_z.
    map="cnp" builds the blocks by the truncated Cayley-Neumann series
    (poetx_build_cnp) and keeps the skew blocks Q for its VJP
    (POETX_CAYLEY_NEUMANN); map="cayley" (default) is the exact map.
    perm_out / perm_in (both or neither): block-mixing index maps of R and P;
    W0 is folded with them once here (poetx_fold_weight) and the calls then
    gather and scatter the activations' columns.
    int8=True stores the frozen weight as INT8 codes with per-row scales
    (poetx_quantize_weight, after any folding); the act-type copy is dropped.
    """

    def __init__(self, W0: torch.Tensor, b_in: int, b_out: int, act: str, device="cuda",
                 recompute_z: bool = False, map: str = "cayley", perm_out=None, perm_in=None,
                 int8: bool = False, saved_y: bool = False):
        if map not in ("cayley", "cnp"):
            raise ValueError(f"unknown orthogonal map {map!r}")
        self.torch_dtype, self.act = _DT[act]
        self.map = map
        self.flags = (P.POETX_RECOMPUTE_Z if recompute_z else 0) | \
            (P.POETX_CAYLEY_NEUMANN if map == "cnp" else 0) | \
            (P.POETX_SAVED_Y if saved_y else 0)
        self.device = torch.device(device)
        self.W0 = W0.to(self.device, self.torch_dtype).contiguous()
        self.d_out, self.d_in = self.W0.shape
        if (perm_out is None) != (perm_in is None):
            raise ValueError("give both permutations or neither")
        self.perm_out = self.perm_in = None
        if perm_out is not None:
            i32 = dict(device=self.device, dtype=torch.int32)
            self.perm_out = torch.as_tensor(perm_out).to(**i32).contiguous()
            self.perm_in = torch.as_tensor(perm_in).to(**i32).contiguous()
            folded = torch.empty_like(self.W0)
            P.poetx_fold_weight(self.W0, self.d_out, self.d_in, self.perm_out, self.perm_in,
                                self.act, folded)
            self.W0 = folded
        self.w_scale = None
        if int8:
            q = torch.empty(self.d_out, self.d_in, device=self.device, dtype=torch.int8)
            self.w_scale = torch.empty(self.d_out, device=self.device, dtype=torch.float32)
            P.poetx_quantize_weight(self.W0, self.d_out, self.d_in, self.act, q, self.w_scale)
            self.W0 = q
        self.b_in, self.b_out = b_in, b_out
        self.nb_in = P.poetx_num_blocks(self.d_in, b_in)
        self.nb_out = P.poetx_num_blocks(self.d_out, b_out)
        tri_in, tri_out = b_in * (b_in - 1) // 2, b_out * (b_out - 1) // 2
        n_tR, n_tP = self.nb_out * tri_out, self.nb_in * tri_in
        f32 = dict(device=self.device, dtype=torch.float32)
        self._theta = torch.zeros(max(n_tR + n_tP, 1), **f32)
        self.theta_R = self._theta[:n_tR].view(self.nb_out, tri_out)
        self.theta_P = self._theta[n_tR:n_tR + n_tP].view(self.nb_in, tri_in)
        self.combined = (b_in == b_out and self.d_in % b_in == 0 and self.d_out % b_out == 0)
        nR, nP = self.nb_out * b_out * b_out, self.nb_in * b_in * b_in
        self._blocks_f32 = torch.empty(nR + nP, **f32)
        self._blocks_act = torch.empty(nR + nP, device=self.device, dtype=self.torch_dtype)
        self.R_f32 = self._blocks_f32[:nR].view(self.nb_out, b_out, b_out)
        self.P_f32 = self._blocks_f32[nR:].view(self.nb_in, b_in, b_in)
        self.R_act = self._blocks_act[:nR].view(self.nb_out, b_out, b_out)
        self.P_act = self._blocks_act[nR:].view(self.nb_in, b_in, b_in)
        if map == "cnp":
            self._q = torch.empty(nR + nP, **f32)
            self.Q_R = self._q[:nR].view(self.nb_out, b_out, b_out)
            self.Q_P = self._q[nR:].view(self.nb_in, b_in, b_in)
        wsz = P.poetx_build_cnp_workspace_size if map == "cnp" else P.poetx_build_workspace_size
        if self.combined:
            ws = wsz(self.d_out + self.d_in, b_out)
        else:
            ws = max(wsz(self.d_out, b_out), wsz(self.d_in, b_in))
        self._build_ws = torch.empty(max(ws, 1), device=self.device, dtype=torch.uint8)
        self._fwd_ws = {}
        self._bwd_ws = {}

    # -- parameters ---------------------------------------------------------
    def set_theta(self, theta_R, theta_P):
        self.theta_R.copy_(torch.as_tensor(theta_R, dtype=torch.float32))
        self.theta_P.copy_(torch.as_tensor(theta_P, dtype=torch.float32))

    def desc(self, tokens: int, events=None):
        return P.make_desc(tokens, self.d_in, self.d_out, self.b_in, self.b_out, self.act, events,
                           self.flags, self.perm_in, self.perm_out, self.w_scale)

    def _ws(self, cache, size_fn, tokens):
        if tokens not in cache:
            n = size_fn(self.desc(tokens))
            cache[tokens] = torch.empty(max(n, 1), device=self.device, dtype=torch.uint8)
        return cache[tokens]

    # -- the three calls ----------------------------------------------------
    def build(self, stream=None):
        """Build of the R and P blocks (one call when the sets combine)."""
        act_R = self.R_act if self.act == P.POETX_BF16 else None
        act_P = self.P_act if self.act == P.POETX_BF16 else None
        if self.map == "cnp":
            act_all = self._blocks_act if self.act == P.POETX_BF16 else None
            if self.combined:
                P.poetx_build_cnp(self._theta, self.d_out + self.d_in, self.b_out, self._q,
                                  self._blocks_f32, act_all, self.act, self._build_ws, stream)
            else:
                P.poetx_build_cnp(self.theta_R, self.d_out, self.b_out, self.Q_R, self.R_f32,
                                  act_R, self.act, self._build_ws, stream)
                P.poetx_build_cnp(self.theta_P, self.d_in, self.b_in, self.Q_P, self.P_f32,
                                  act_P, self.act, self._build_ws, stream)
            return
        if self.combined:
            P.poetx_build_orthogonal(self._theta, self.d_out + self.d_in, self.b_out,
                                     self._blocks_f32,
                                     self._blocks_act if self.act == P.POETX_BF16 else None,
                                     self.act, self._build_ws, stream)
        else:
            P.poetx_build_orthogonal(self.theta_R, self.d_out, self.b_out, self.R_f32, act_R,
                                     self.act, self._build_ws, stream)
            P.poetx_build_orthogonal(self.theta_P, self.d_in, self.b_in, self.P_f32, act_P,
                                     self.act, self._build_ws, stream)

    def blocks_for_act(self):
        if self.act == P.POETX_BF16:
            return self.R_act, self.P_act
        return self.R_f32, self.P_f32

    def forward(self, x, y=None, z=None, stream=None, events=None):
        N = x.shape[0]
        y = torch.empty(N, self.d_out, device=self.device, dtype=self.torch_dtype) if y is None else y
        if self.flags & (P.POETX_RECOMPUTE_Z | P.POETX_SAVED_Y):
            z = None
        elif z is None:
            z = torch.empty(N, self.d_out, device=self.device, dtype=self.torch_dtype)
        R, Pb = self.blocks_for_act()
        ws = self._ws(self._fwd_ws, P.poetx_fwd_workspace_size, N)
        P.poetx_linear_fwd(self.desc(N, events), x, self.W0, R, Pb, y, z, ws, stream)
        return y, (y if self.flags & P.POETX_SAVED_Y else z)

    def backward(self, g_y, x, z=None, g_x=None, g_theta_R=None, g_theta_P=None, stream=None,
                 events=None):
        N = x.shape[0]
        g_x = torch.empty(N, self.d_in, device=self.device, dtype=self.torch_dtype) if g_x is None else g_x
        if g_theta_R is None:
            g_theta_R = torch.empty_like(self.theta_R)
        if g_theta_P is None:
            g_theta_P = torch.empty_like(self.theta_P)
        R, Pb = self.blocks_for_act()
        ws = self._ws(self._bwd_ws, P.poetx_bwd_workspace_size, N)
        vR, vP = (self.Q_R, self.Q_P) if self.map == "cnp" else (self.R_f32, self.P_f32)
        P.poetx_linear_bwd(self.desc(N, events), g_y, x, self.W0, vR, vP, R, Pb, z,
                           g_x, g_theta_R if g_theta_R.numel() else None,
                           g_theta_P if g_theta_P.numel() else None, ws, stream)
        return g_x, g_theta_R, g_theta_P


class PoetxLinearSet:
    """Several POET-X layers with one block size b whose generators and
    orthogonal blocks live in shared buffers, layer after layer (each layer's
    R blocks, then its P blocks), so that one build call rebuilds every
    layer's R and P: the blocks are independent, so this is the same work as
    one call per layer, batched over all of them. Every layer must combine its
    two sets (b_in == b_out == b, b dividing d_in and d_out), and all must
    share the activation type and the orthogonal map. Each layer keeps working
    on its own views; its own build() still builds just that layer."""

    def __init__(self, layers):
        if not layers:
            raise ValueError("no layers")
        first = layers[0]
        self.layers = list(layers)
        self.b, self.act, self.map = first.b_out, first.act, first.map
        self.device, self.torch_dtype = first.device, first.torch_dtype
        for lay in self.layers:
            if not lay.combined or lay.b_in != self.b or lay.b_out != self.b:
                raise ValueError("every layer must have b_in == b_out == b dividing its sizes")
            if lay.act != self.act or lay.map != self.map or lay.device != self.device:
                raise ValueError("the layers must share the activation type, map and device")
        f32 = dict(device=self.device, dtype=torch.float32)
        n_theta = sum(lay.theta_R.numel() + lay.theta_P.numel() for lay in self.layers)
        n_blk = sum(lay._blocks_f32.numel() for lay in self.layers)
        self._theta = torch.empty(n_theta, **f32)
        self._blocks_f32 = torch.empty(n_blk, **f32)
        self._blocks_act = torch.empty(n_blk, device=self.device, dtype=self.torch_dtype)
        self._q = torch.empty(n_blk, **f32) if self.map == "cnp" else None
        ot = ob = 0
        for lay in self.layers:
            b = self.b
            n_tR, n_tP = lay.theta_R.numel(), lay.theta_P.numel()
            nR, nP = lay.nb_out * b * b, lay.nb_in * b * b
            th = self._theta[ot:ot + n_tR + n_tP]
            th.copy_(lay._theta[:n_tR + n_tP])
            lay._theta = th
            lay.theta_R = th[:n_tR].view(lay.nb_out, -1)
            lay.theta_P = th[n_tR:].view(lay.nb_in, -1)
            bf, ba = self._blocks_f32[ob:ob + nR + nP], self._blocks_act[ob:ob + nR + nP]
            lay._blocks_f32, lay._blocks_act = bf, ba
            lay.R_f32, lay.P_f32 = bf[:nR].view(lay.nb_out, b, b), bf[nR:].view(lay.nb_in, b, b)
            lay.R_act, lay.P_act = ba[:nR].view(lay.nb_out, b, b), ba[nR:].view(lay.nb_in, b, b)
            if self._q is not None:
                q = self._q[ob:ob + nR + nP]
                lay._q = q
                lay.Q_R, lay.Q_P = q[:nR].view(lay.nb_out, b, b), q[nR:].view(lay.nb_in, b, b)
            ot += n_tR + n_tP
            ob += nR + nP
        self.d_total = sum(lay.d_out + lay.d_in for lay in self.layers)
        wsz = P.poetx_build_cnp_workspace_size if self.map == "cnp" else P.poetx_build_workspace_size
        self._build_ws = torch.empty(max(wsz(self.d_total, self.b), 1), device=self.device,
                                     dtype=torch.uint8)

    def build(self, stream=None):
        """One call: the R and P blocks of every layer."""
        act_all = self._blocks_act if self.act == P.POETX_BF16 else None
        if self.map == "cnp":
            P.poetx_build_cnp(self._theta, self.d_total, self.b, self._q, self._blocks_f32,
                              act_all, self.act, self._build_ws, stream)
        else:
            P.poetx_build_orthogonal(self._theta, self.d_total, self.b, self._blocks_f32, act_all,
                                     self.act, self._build_ws, stream)
