"""A GPT2 training step written from Python through the generic task
interface (tt_submit), the way a user of the library would express any
layer: tiled tensors, then every layer of the forward, the loss, the
backward and the update as tasks over a few tiles, in program order. No
grouping beyond what an op needs (one task per tile product, per LayerNorm
row block, per attention tile pair), so the task graph is the plainest one.

Used by the dry-run tests (access modes, edges, races) and by the GPU test
that checks the step against the oracle."""
from __future__ import annotations

import ctypes as C
import math

import numpy as np

import synth
from tile_task_transformer_amd import _lib as L


class SubmitGPT2:
    def __init__(self, ctx, s: synth.GPT2Shape, t: synth.Tiles, fused_head: bool = False):
        """fused_head: the head's last embd tile as one batched task over all
        vocab tiles with the cross-entropy statistics in its epilogue
        (TT_EPI_XSTATS), merged by 64-column groups; else every product its
        own task and a separate statistics pass."""
        self.ctx, self.s, self.t, self.fused_head = ctx, s, t, fused_head
        d, I, H, V, T, B = s.n_embd, s.n_inner, s.n_head, s.vocab, s.seq, s.batch
        hd = d // H
        et, it, ht, vt, st, bt = min(t.embd, d), min(t.inner, I), t.head, min(t.vocab, V), t.seq, t.batch
        self.hd, self.et, self.it, self.ht, self.vt, self.st, self.bt = hd, et, it, ht, vt, st, bt
        self.NE, self.NI, self.NH, self.NV = -(-d // et), -(-I // it), H // ht, -(-V // vt)
        self.nb, self.ns = B // bt, T // st
        self.rows = bt * st
        mk = ctx.tensor
        # parameters, gradients and moments in the order of synth.param_specs
        self.specs = synth.param_specs(s)
        layouts = {"wte": ((V, d), (vt, et), 1), "wpe": ((T, d), (st, et), 1),
                   "ln1_g": ((d,), (et,), 0), "ln1_b": ((d,), (et,), 0),
                   "w_qkv": ((d, 3, H, hd), (et, 1, ht, hd), 1), "b_qkv": ((3, H, hd), (1, ht, hd), 0),
                   "w_o": ((H, hd, d), (ht, hd, et), 2), "b_o": ((d,), (et,), 0),
                   "ln2_g": ((d,), (et,), 0), "ln2_b": ((d,), (et,), 0),
                   "w_fc": ((d, I), (et, it), 1), "b_fc": ((I,), (it,), 0),
                   "w_p": ((I, d), (it, et), 1), "b_p": ((d,), (et,), 0),
                   "lnf_g": ((d,), (et,), 0), "lnf_b": ((d,), (et,), 0)}
        self.P, self.G, self.M, self.Vm = {}, {}, {}, {}
        for name, _, _ in self.specs:
            shp, tl, split = layouts[name.split(".")[-1]]
            for store in (self.P, self.G, self.M, self.Vm):
                store[name] = mk(shp, tl).set_matrix_split(split)

        def act(shape, tile, split=2, dtype=L.TT_F32):
            return mk(shape, tile, dtype).set_matrix_split(split)

        self.tokens = act((B, T + 1), (B, T + 1), 1, L.TT_I32)
        self.ids, self.labels, self.sorted, self.perm = (act((B, T), (bt, st), 1, L.TT_I32) for _ in range(4))
        nq = bt * st * ht
        self.blk = []
        h = act((B, T, d), (bt, st, et))
        for _ in range(s.n_layer):
            b = dict(h_in=h, ln1=act((B, T, 2), (bt, st, 2)), n1=act((B, T, d), (bt, st, et)),
                     q=act((B, T, H, hd), (bt, st, ht, hd)), k=act((B, T, H, hd), (bt, st, ht, hd)),
                     v=act((B, T, H, hd), (bt, st, ht, hd)), o=act((B, T, H, hd), (bt, st, ht, hd)),
                     lse=act((B // bt, T // st, H // ht, nq), (1, 1, 1, nq), 3),
                     h_mid=act((B, T, d), (bt, st, et)), ln2=act((B, T, 2), (bt, st, 2)),
                     n2=act((B, T, d), (bt, st, et)), u=act((B, T, I), (bt, st, it)), g=act((B, T, I), (bt, st, it)))
            h = act((B, T, d), (bt, st, et))
            b["h_out"] = h
            self.blk.append(b)
        self.h_last = h
        ntok = self.nb * self.ns
        self.lnf, self.nf = act((B, T, 2), (bt, st, 2)), act((B, T, d), (bt, st, et))
        self.z = act((B, T, V), (bt, st, vt))
        self.ml = act((B // bt, T // st, H // ht, 2 * nq), (1, 1, 1, 2 * nq), 3)
        groups = -(-vt // 64) if fused_head else 1
        self.ce_parts = act((self.NV, ntok, groups * self.rows * 3), (1, 1, groups * self.rows * 3))
        self.ce_lse, self.row_loss = act((ntok, self.rows), (1, self.rows), 1), act((ntok, self.rows), (1, self.rows), 1)
        self.loss = act((1,), (1,), 0)
        self.dnf, self.dh, self.dn = (act((B, T, d), (bt, st, et)) for _ in range(3))
        self.dgu = act((B, T, I), (bt, st, it))
        self.dO, self.dq, self.dk, self.dv = (act((B, T, H, hd), (bt, st, ht, hd)) for _ in range(4))
        self.Dv = act((B // bt, T // st, H // ht, nq), (1, 1, 1, nq), 3)
        self.step_ctr = act((1,), (1,), 0, L.TT_I32)
        self.bc = act((2,), (2,), 0)
        self.tasks = 0

    # ---------------------------------------------------------------- helpers
    def sub(self, op, tiles, sc=None):
        self.ctx.submit(op, tiles, sc)
        self.tasks += 1

    def gemm(self, A, ia, B, ib, Cc, ic, ta=0, tb=0, beta=0.0, epi=0, bias=None, res=None, aux=None, split=1):
        tl = [(A, ia), (B, ib), (Cc, ic)] + [x for x in (bias, res, aux) if x is not None]
        self.sub(L.TT_OP_GEMM, tl, L.tt_op_gemm(ta, tb, epi, 1.0, beta, split))

    # ------------------------------------------------------------------- step
    def submit_step(self, tokens_ptr, lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.1):
        s = self
        sh = s.s
        NE, NI, NH, NV, nb, ns, st = s.NE, s.NI, s.NH, s.NV, s.nb, s.ns, s.st
        scale = 1.0 / math.sqrt(s.hd)
        inv_n = 1.0 / (sh.batch * sh.seq)
        P, G = s.P, s.G
        s.sub(L.TT_OP_COPY_IN, [(s.tokens, (0, 0))], L.tt_op_copy(tokens_ptr))
        for bi in range(nb):
            for si in range(ns):
                s.sub(L.TT_OP_SPLIT_TOKENS, [(s.tokens, (0, 0)), (s.ids, (bi, si)), (s.labels, (bi, si))])
                s.sub(L.TT_OP_EMBEDDING_INDEX, [(s.ids, (bi, si)), (s.sorted, (bi, si)), (s.perm, (bi, si))])
        h0 = s.blk[0]["h_in"] if s.blk else s.h_last
        for bi in range(nb):
            for si in range(ns):
                for e in range(NE):
                    s.sub(L.TT_OP_EMBEDDING_FWD, [(s.ids, (bi, si)), (P["wpe"], (si, e)), (h0, (bi, si, e))] +
                          [(P["wte"], (v, e)) for v in range(NV)], L.tt_op_embedding(st))

        def ln_fwd(x, g_, b_, stats, y, bi, si):
            s.sub(L.TT_OP_LAYERNORM_FWD, [(x, (bi, si, e)) for e in range(NE)] + [(g_, (e,)) for e in range(NE)] +
                  [(b_, (e,)) for e in range(NE)] + [(stats, (bi, si, 0))] + [(y, (bi, si, e)) for e in range(NE)],
                  L.tt_op_layernorm(1e-5, 0))

        def ln_bwd(dy, x, g_, stats, dx, dx_acc, dg, db, bi, si):
            s.sub(L.TT_OP_LAYERNORM_BWD, [(dy, (bi, si, e)) for e in range(NE)] + [(x, (bi, si, e)) for e in range(NE)]
                  + [(g_, (e,)) for e in range(NE)] + [(stats, (bi, si, 0))] + [(dx, (bi, si, e)) for e in range(NE)]
                  + [(dg, (e,)) for e in range(NE)] + [(db, (e,)) for e in range(NE)], L.tt_op_layernorm(1e-5, dx_acc))

        for l, b in enumerate(s.blk):
            p = f"h{l}."
            for bi in range(nb):
                for si in range(ns):
                    ln_fwd(b["h_in"], P[p + "ln1_g"], P[p + "ln1_b"], b["ln1"], b["n1"], bi, si)
                    for cq, dst in enumerate((b["q"], b["k"], b["v"])):
                        for hj in range(NH):
                            for ek in range(NE):
                                last = ek == NE - 1
                                s.gemm(b["n1"], (bi, si, ek), P[p + "w_qkv"], (ek, cq, hj, 0), dst, (bi, si, hj, 0),
                                       beta=float(ek > 0), epi=L.TT_EPI_BIAS if last else 0,
                                       bias=(P[p + "b_qkv"], (cq, hj, 0)) if last else None)
            for bi in range(nb):
                for hj in range(NH):
                    for qi in range(ns):
                        for ki in range(qi + 1):
                            s.sub(L.TT_OP_ATTENTION_FWD, [(b["q"], (bi, qi, hj, 0)), (b["k"], (bi, ki, hj, 0)),
                                                          (b["v"], (bi, ki, hj, 0)), (b["o"], (bi, qi, hj, 0)),
                                                          (s.ml, (bi, qi, hj, 0)), (b["lse"], (bi, qi, hj, 0))],
                                  L.tt_op_attention(qi * st, ki * st, int(ki == 0), int(ki == qi), 0, 0, scale))
            for bi in range(nb):
                for si in range(ns):
                    for ej in range(NE):
                        for hk in range(NH):
                            epi = (L.TT_EPI_RES if hk == 0 else 0) | (L.TT_EPI_BIAS if hk == NH - 1 else 0)
                            s.gemm(b["o"], (bi, si, hk, 0), P[p + "w_o"], (hk, 0, ej), b["h_mid"], (bi, si, ej),
                                   beta=float(hk > 0), epi=epi,
                                   bias=(P[p + "b_o"], (ej,)) if hk == NH - 1 else None,
                                   res=(b["h_in"], (bi, si, ej)) if hk == 0 else None)
                    ln_fwd(b["h_mid"], P[p + "ln2_g"], P[p + "ln2_b"], b["ln2"], b["n2"], bi, si)
                    for ij in range(NI):
                        for ek in range(NE):
                            last = ek == NE - 1
                            s.gemm(b["n2"], (bi, si, ek), P[p + "w_fc"], (ek, ij), b["g"] if last else b["u"],
                                   (bi, si, ij), beta=float(ek > 0),
                                   epi=(L.TT_EPI_GELU | L.TT_EPI_BIAS) if last else 0,
                                   bias=(P[p + "b_fc"], (ij,)) if last else None,
                                   aux=(b["u"], (bi, si, ij)) if last else None)
                    for ej in range(NE):
                        for ik in range(NI):
                            epi = (L.TT_EPI_RES if ik == 0 else 0) | (L.TT_EPI_BIAS if ik == NI - 1 else 0)
                            s.gemm(b["g"], (bi, si, ik), P[p + "w_p"], (ik, ej), b["h_out"], (bi, si, ej),
                                   beta=float(ik > 0), epi=epi,
                                   bias=(P[p + "b_p"], (ej,)) if ik == NI - 1 else None,
                                   res=(b["h_mid"], (bi, si, ej)) if ik == 0 else None)
        # final LayerNorm, tied head, loss
        for bi in range(nb):
            for si in range(ns):
                ti = bi + nb * si
                ln_fwd(s.h_last, P["lnf_g"], P["lnf_b"], s.lnf, s.nf, bi, si)
                if s.fused_head:
                    for vj in range(NV):
                        for ek in range(NE - 1):
                            s.gemm(s.nf, (bi, si, ek), P["wte"], (vj, ek), s.z, (bi, si, vj), tb=1,
                                   beta=float(ek > 0))
                    last = NE - 1
                    tl = [x for vj in range(NV) for x in ((s.nf, (bi, si, last)), (P["wte"], (vj, last)),
                                                          (s.z, (bi, si, vj)))]
                    tl += [(s.labels, (bi, si))] + [(s.ce_parts, (v, ti, 0)) for v in range(NV)]
                    s.sub(L.TT_OP_GEMM_BATCH, tl, L.tt_op_gemm(0, 1, L.TT_EPI_XSTATS, 1.0, float(last > 0), 0))
                    s.sub(L.TT_OP_XENTROPY_MERGE, [(s.ce_lse, (ti, 0)), (s.row_loss, (ti, 0))] +
                          [(s.ce_parts, (v, ti, 0)) for v in range(NV)], L.tt_op_xe_groups(sh.vocab, s.vt, 64))
                else:
                    for vj in range(NV):
                        for ek in range(NE):
                            s.gemm(s.nf, (bi, si, ek), P["wte"], (vj, ek), s.z, (bi, si, vj), tb=1,
                                   beta=float(ek > 0))
                    s.sub(L.TT_OP_XENTROPY_STATS, [(s.labels, (bi, si))] + [(s.z, (bi, si, v)) for v in range(NV)] +
                          [(s.ce_parts, (v, ti, 0)) for v in range(NV)])
                    s.sub(L.TT_OP_XENTROPY_MERGE, [(s.ce_lse, (ti, 0)), (s.row_loss, (ti, 0))] +
                          [(s.ce_parts, (v, ti, 0)) for v in range(NV)])
                s.sub(L.TT_OP_XENTROPY_LOSS, [(s.row_loss, (ti, 0)), (s.loss, (0,))],
                      L.tt_op_xentropy(int(ti > 0), inv_n))
                s.sub(L.TT_OP_XENTROPY_GRAD, [(s.labels, (bi, si)), (s.ce_lse, (ti, 0))] +
                      [(s.z, (bi, si, v)) for v in range(NV)], L.tt_op_xentropy(0, inv_n))
        opt = L.tt_op_optim(lr, beta1, beta2, eps, wd)
        s.sub(L.TT_OP_ADAMW_ADVANCE, [(s.step_ctr, (0,)), (s.bc, (0,))], opt)

        def adamw(names):
            for name in names:
                grid, _ = s.P[name].grid()
                for idx in np.ndindex(*grid):
                    s.sub(L.TT_OP_ADAMW, [(s.bc, (0,)), (s.P[name], idx), (s.G[name], idx), (s.M[name], idx),
                                          (s.Vm[name], idx)], opt)

        # backward: head
        for bi in range(nb):
            for si in range(ns):
                ti = bi + nb * si
                for vj in range(NV):
                    for ek in range(NE):
                        s.gemm(s.z, (bi, si, vj), s.nf, (bi, si, ek), G["wte"], (vj, ek), ta=1, beta=float(ti > 0))
                for ek in range(NE):
                    s.sub(L.TT_OP_GEMM_KSUM, [(s.dnf, (bi, si, ek))] +
                          [x for v in range(NV) for x in ((s.z, (bi, si, v)), (P["wte"], (v, ek)))],
                          L.tt_op_gemm(0, 0, 0, 1.0, 0.0, 0))
        zero = [(G[n], (e,)) for n, _, _ in s.specs if n.split(".")[-1] in ("ln1_g", "ln1_b", "ln2_g", "ln2_b",
                                                                            "lnf_g", "lnf_b") for e in range(NE)]
        grid, _ = G["wpe"].grid()
        zero += [(G["wpe"], idx) for idx in np.ndindex(*grid)]
        for z0 in range(0, len(zero), 16):
            s.sub(L.TT_OP_FILL, zero[z0:z0 + 16], L.tt_op_fill(0.0))
        for bi in range(nb):
            for si in range(ns):
                ln_bwd(s.dnf, s.h_last, P["lnf_g"], s.lnf, s.dh, 0, G["lnf_g"], G["lnf_b"], bi, si)
        adamw(["lnf_g", "lnf_b"])
        for l in reversed(range(sh.n_layer)):
            b, p = s.blk[l], f"h{l}."
            for si in range(ns):
                for bi in range(nb):
                    ti = bi + nb * si
                    acc = float(ti > 0)
                    for ej in range(NE):
                        for ik in range(NI):
                            s.gemm(b["g"], (bi, si, ik), s.dh, (bi, si, ej), G[p + "w_p"], (ik, ej), ta=1, beta=acc)
                    s.sub(L.TT_OP_REDUCE_ROWS, [x for ej in range(NE) for x in ((s.dh, (bi, si, ej)),
                                                                                 (G[p + "b_p"], (ej,)))],
                          L.tt_op_reduce(int(ti > 0)))
                    for ik in range(NI):
                        for ej in range(NE):
                            last = ej == NE - 1
                            s.gemm(s.dh, (bi, si, ej), P[p + "w_p"], (ik, ej), s.dgu, (bi, si, ik), tb=1,
                                   beta=float(ej > 0), epi=L.TT_EPI_GELU_BWD if last else 0,
                                   aux=(b["u"], (bi, si, ik)) if last else None)
                    for ik in range(NI):
                        for ek in range(NE):
                            s.gemm(b["n2"], (bi, si, ek), s.dgu, (bi, si, ik), G[p + "w_fc"], (ek, ik), ta=1,
                                   beta=acc)
                    s.sub(L.TT_OP_REDUCE_ROWS, [x for ik in range(NI) for x in ((s.dgu, (bi, si, ik)),
                                                                                 (G[p + "b_fc"], (ik,)))],
                          L.tt_op_reduce(int(ti > 0)))
                    for ek in range(NE):
                        for ik in range(NI):
                            s.gemm(s.dgu, (bi, si, ik), P[p + "w_fc"], (ek, ik), s.dn, (bi, si, ek), tb=1,
                                   beta=float(ik > 0))
                    ln_bwd(s.dn, b["h_mid"], P[p + "ln2_g"], b["ln2"], s.dh, 1, G[p + "ln2_g"], G[p + "ln2_b"], bi, si)
                    for ej in range(NE):
                        for hk in range(NH):
                            s.gemm(b["o"], (bi, si, hk, 0), s.dh, (bi, si, ej), G[p + "w_o"], (hk, 0, ej), ta=1,
                                   beta=acc)
                    s.sub(L.TT_OP_REDUCE_ROWS, [x for ej in range(NE) for x in ((s.dh, (bi, si, ej)),
                                                                                 (G[p + "b_o"], (ej,)))],
                          L.tt_op_reduce(int(ti > 0)))
                    for hk in range(NH):
                        for ej in range(NE):
                            s.gemm(s.dh, (bi, si, ej), P[p + "w_o"], (hk, 0, ej), s.dO, (bi, si, hk, 0), tb=1,
                                   beta=float(ej > 0))
            for bi in range(nb):
                for hj in range(NH):
                    for qi in range(ns):
                        s.sub(L.TT_OP_ATTENTION_PREP, [(b["o"], (bi, qi, hj, 0)), (s.dO, (bi, qi, hj, 0)),
                                                       (s.Dv, (bi, qi, hj, 0))],
                              L.tt_op_attention(0, 0, 0, 0, 0, 0, scale))
                    for qi in range(ns):
                        for ki in range(qi + 1):
                            s.sub(L.TT_OP_ATTENTION_BWD,
                                  [(b["q"], (bi, qi, hj, 0)), (b["k"], (bi, ki, hj, 0)), (b["v"], (bi, ki, hj, 0)),
                                   (s.dO, (bi, qi, hj, 0)), (b["lse"], (bi, qi, hj, 0)), (s.Dv, (bi, qi, hj, 0)),
                                   (s.dq, (bi, qi, hj, 0)), (s.dk, (bi, ki, hj, 0)), (s.dv, (bi, ki, hj, 0))],
                                  L.tt_op_attention(qi * st, ki * st, 0, 0, int(ki > 0), int(qi > ki), scale))
            for si in range(ns):
                for bi in range(nb):
                    ti = bi + nb * si
                    for cq, dsrc in enumerate((s.dq, s.dk, s.dv)):
                        for hj in range(NH):
                            for ek in range(NE):
                                s.gemm(b["n1"], (bi, si, ek), dsrc, (bi, si, hj, 0), G[p + "w_qkv"], (ek, cq, hj, 0),
                                       ta=1, beta=float(ti > 0))
                            s.sub(L.TT_OP_REDUCE_ROWS, [(dsrc, (bi, si, hj, 0)), (G[p + "b_qkv"], (cq, hj, 0))],
                                  L.tt_op_reduce(int(ti > 0)))
                    for ek in range(NE):
                        s.sub(L.TT_OP_GEMM_KSUM, [(s.dn, (bi, si, ek))] +
                              [x for cq, dsrc in enumerate((s.dq, s.dk, s.dv)) for hj in range(NH)
                               for x in ((dsrc, (bi, si, hj, 0)), (P[p + "w_qkv"], (ek, cq, hj, 0)))],
                              L.tt_op_gemm(0, 1, 0, 1.0, 0.0, 0))
                    ln_bwd(s.dn, b["h_in"], P[p + "ln1_g"], b["ln1"], s.dh, 1, G[p + "ln1_g"], G[p + "ln1_b"], bi, si)
            adamw([p + n for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b", "w_fc", "b_fc",
                                   "w_p", "b_p")])
        # embedding backward, then the embeddings' update
        for ek in range(NE):
            for si in range(ns):
                for bi in range(nb):
                    s.sub(L.TT_OP_EMBEDDING_BWD, [(s.dh, (bi, si, ek)), (s.sorted, (bi, si)), (s.perm, (bi, si))] +
                          [(G["wte"], (v, ek)) for v in range(NV)], L.tt_op_embedding(st))
        for si in range(ns):
            for ek in range(NE):
                for bi in range(nb):
                    s.sub(L.TT_OP_EMBEDDING_POS_BWD, [(s.dh, (bi, si, ek)), (G["wpe"], (si, ek))],
                          L.tt_op_embedding(st))
        adamw(["wpe", "wte"])

    # ------------------------------------------------------------- host I/O
    def set_params(self, params):
        for name, shp, _ in self.specs:
            self.P[name].copy_in(np.asarray(params[name], np.float32).reshape(self.P[name].shape))
            for store in (self.M, self.Vm):
                store[name].copy_in(np.zeros(self.P[name].shape, np.float32))
        self.step_ctr.copy_in(np.zeros(1, np.int32))

    def get(self, store):
        return {name: store[name].copy_out().reshape(shp) for name, shp, _ in self.specs}

    def loss_value(self) -> float:
        return float(self.loss.copy_out()[0])


def tile_ptr(x) -> int:
    return x.data_ptr() if hasattr(x, "data_ptr") else int(x)


__all__ = ["SubmitGPT2", "tile_ptr", "C"]
