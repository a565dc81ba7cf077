"""One Focus-dLLM denoising step over a stack of attention layers, through the C ABI.

Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Method
steps": a block-entry step refreshes densely (every row attends to every key
in every layer); any other step runs (1) PCGI, (2) windows, (3) dense layers
1..l_dense on the active rows with sinks taken from layer l_dense, then (4)
block top-C and (5) sparse attention in every deeper layer, reusing the sinks.

StepRunner only sequences the library's entry points with buffers allocated
once, so a whole step can be captured in a HIP graph and replayed; it performs
no arithmetic of its own.  The block means of step (4) depend on the prompt keys
only; with overlap_means a sparse step computes them on a second stream while the
caller's stream runs the layers before them, and each layer's scoring waits for its
own means.  The attention kernels hold every CU while they run, so the means run in
the gaps between them: with means_ahead = a, the means of layer l are issued once the
attention of layer l - a has finished (the first a sparse layers' means once PCGI
has), and fill the CUs that the split merge and the next layer's scoring leave idle.
means_ahead None (the default) issues every layer's means at the start of the step: on
the 32K stack that is the faster order (5.59 ms a step against 5.71 ms with a = 2 to 4,
and 5.93 ms with a = 1), since means that run alone stream at full rate while means
squeezed between attention launches delay them.  Without it,
each layer computes its means right before scoring them.

Variants (Summary, "Independent weaknesses" and "Reproducibility"): dense_tail keeps the
last layers of the stack dense on the active rows (Dream-like models need their last 4
layers kept); per_head gives every KV head its own top-C blocks; aggregator "max" scores
a block by its strongest query instead of the summed relevance.

cached_step is the same step over an approximate KV cache ("Prerequisites",
approximate KV cache): every layer first writes the recomputed keys and values
of U(t) = I_active into its cache, then recomputes only the block means those
rows touch (the means of the other blocks are kept from the previous step), so
the per-layer scan of the prompt keys is skipped.
"""
from __future__ import annotations

import torch

from . import fdl as F


class StepRunner:
    def __init__(self, *, B, L, P, Hq, Hkv, d, dtype, n_t, rho, w, bs, C, n_sinks, layers, l_dense,
                 scale=0.0, device="cuda", overlap_means=True, dense_tail=0, per_head=False, aggregator="sum",
                 means_ahead=None):
        self.B, self.L, self.P, self.Hq, self.Hkv, self.d = B, L, P, Hq, Hkv, d
        self.n_t, self.rho, self.w, self.bs, self.C, self.n_sinks = n_t, rho, w, bs, C, n_sinks
        self.layers, self.l_dense, self.scale = layers, l_dense, scale
        self.dense_tail, self.per_head, self.aggregator = dense_tail, per_head, aggregator
        self.k = F.focus_count(n_t, rho)
        self.nq_max = max(min(self.k * w, L), 1)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.focus = torch.empty((B, max(self.k, 1)), **i32)
        self.n_focus = torch.empty((B,), **i32)
        self.active = torch.empty((B, self.nq_max), **i32)
        self.n_active = torch.empty((B,), **i32)
        self.sinks = torch.empty((B, max(n_sinks, 1)), **i32)
        lead = (B, Hkv) if per_head else (B,)
        self.blocks = [torch.empty(lead + (max(C, 1),), **i32) for _ in range(layers)]
        self.nb = -(-P // bs)
        sparse_layers = range(l_dense, layers - dense_tail) if C else range(0)
        self.kbar = {l: torch.empty((B, Hkv, self.nb, d), dtype=torch.float32, device=dev) for l in sparse_layers}
        self.overlap_means = overlap_means
        self.side = torch.cuda.Stream(device=dev) if dev.type == "cuda" and overlap_means else None
        self.means_done = {l: torch.cuda.Event() for l in sparse_layers}
        if means_ahead is not None and means_ahead < 1:
            raise ValueError("means_ahead must be >= 1 or None")
        self.means_ahead = means_ahead
        self.pcgi_done = torch.cuda.Event()
        self.attn_done = {l: torch.cuda.Event() for l in sparse_layers}
        self.out = [torch.empty((B, Hq, self.nq_max, d), dtype=dtype, device=dev) for _ in range(layers)]
        self.lse = torch.empty((B, Hq, self.nq_max), dtype=torch.float32, device=dev)
        self.workspace = F.Workspace(dev)
        # size the shared workspace once, so a captured step never allocates
        dt = F.FDL_BF16 if dtype == torch.bfloat16 else F.FDL_F32
        lib = F.lib()
        need = max(
            lib.fdl_dense_attention_workspace_bytes(dt, B, Hq, Hkv, L, d, self.nq_max),
            lib.fdl_sink_identify_workspace_bytes(dt, B, Hq, Hkv, L, d, self.nq_max),
            lib.fdl_block_score_topc_workspace_bytes(dt, B, Hq, Hkv, P, d, bs, self.nq_max),
            lib.fdl_sparse_attention_ex_workspace_bytes(dt, B, Hq, Hkv, L, P, d, self.nq_max, n_sinks, C, bs,
                                                        int(per_head)),
        )
        self.workspace.get(need)

    def _rows(self):
        return dict(q_idx=self.active, n_q=self.n_active, nq_max=self.nq_max, scale=self.scale,
                    workspace=self.workspace)

    def is_dense(self, l):
        """Layers 1..l_dense and the dense tail attend densely on the active rows."""
        return l < self.l_dense or l >= self.layers - self.dense_tail

    def pcgi(self, conf, mask):
        F.pcgi_select(conf, mask, self.n_t, self.rho, self.w, k_cap=self.focus.shape[1], nq_max=self.nq_max,
                      out=(self.focus, self.n_focus, self.active, self.n_active))

    def dense_layer(self, l, q, k, v, vt=None):
        F.dense_attention(q, k, v, vt=vt, out=self.out[l], lse=self.lse, **self._rows())

    def sinks_at(self, q, k):
        if self.n_sinks:
            F.sink_identify(q, k, self.lse, self.n_sinks, out=self.sinks, **self._rows())

    def score_blocks(self, l, q):
        """Block top-C of one sparse layer from its block means (already in self.kbar[l])."""
        F.block_score_topc(q, None, self.P, self.bs, self.C, kbar=self.kbar[l], L=self.L, out=self.blocks[l],
                           per_head=self.per_head, aggregator=self.aggregator, **self._rows())

    def attend(self, l, q, k, v, vt=None):
        """Sparse attention of one layer over the step's sinks and the layer's selected blocks."""
        sinks = self.sinks[:, : self.n_sinks] if self.n_sinks else None
        blocks = self.blocks[l][..., : self.C] if self.C else None
        F.sparse_attention(q, k, v, self.P, sinks, blocks, self.bs, vt=vt, out=self.out[l], **self._rows())

    def sparse_step(self, conf, mask, qs, ks, vs, hooks=None, vts=None):
        """A non-block-entry step; qs/ks/vs are per-layer [B, H, L, d] tensors, vts None or
        per-layer V^T copies (F.transpose_v) that the attention reads for runs of keys.

        `hooks` (optional) maps a stage name ("pcgi", "dense", "sinks", "means",
        "blocks", "sparse") to a (before, after) pair of callables run around each
        call of that stage on the stream it runs on, e.g. to record events."""
        def run(name, fn):
            h = hooks.get(name) if hooks else None
            if h:
                h[0]()
            fn()
            if h:
                h[1]()
        main = torch.cuda.current_stream()
        overlap = bool(self.kbar) and self.overlap_means
        order = sorted(self.kbar)
        ahead = self.means_ahead

        def issue_means(ls, after):
            # block means of the layers ls on the second stream, once `after` has been reached
            self.side.wait_event(after) if after is not None else self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                for ml in ls:
                    run("means", lambda: F.block_means(ks[ml], self.P, self.bs, out=self.kbar[ml]))
                    self.means_done[ml].record(self.side)

        if overlap and ahead is None:
            issue_means(order, None)
        run("pcgi", lambda: self.pcgi(conf, mask))
        if overlap and ahead is not None:
            self.pcgi_done.record(main)
            issue_means(order[:ahead], self.pcgi_done)
        for l in range(self.layers):
            q, k, v = qs[l], ks[l], vs[l]
            vt = vts[l] if vts is not None else None
            if self.is_dense(l):
                run("dense", lambda: self.dense_layer(l, q, k, v, vt))
                if l == self.l_dense - 1:
                    run("sinks", lambda: self.sinks_at(q, k))
            else:
                if self.C:
                    if overlap:
                        main.wait_event(self.means_done[l])
                    else:
                        run("means", lambda: F.block_means(k, self.P, self.bs, out=self.kbar[l]))
                    run("blocks", lambda: self.score_blocks(l, q))
                run("sparse", lambda: self.attend(l, q, k, v, vt))
                if overlap and ahead is not None and l in self.kbar:
                    i = order.index(l)
                    if i + ahead < len(order):
                        self.attn_done[l].record(main)
                        issue_means([order[i + ahead]], self.attn_done[l])
        if overlap:
            main.wait_stream(self.side)

    def init_means(self, ks):
        """Block means of every sparse layer from its whole cache (after a block-entry step),
        the state cached_step keeps up to date."""
        for l, kb in self.kbar.items():
            F.block_means(ks[l], self.P, self.bs, out=kb)

    def cached_step(self, conf, mask, qs, ks, vs, k_new, v_new, hooks=None, vts=None):
        """A non-block-entry step over an approximate KV cache.

        k_new[l], v_new[l] ([B, Hkv, nq_max, d]) hold layer l's recomputed keys and values of
        the active rows, row i for active_idx[b, i].  Layer l's new rows come from layer l's
        own forward pass, which follows layer l-1's attention, so each layer refreshes its cache
        (and V^T, when kept), and a sparse layer its touched block means, on the caller's
        stream right before it attends.  self.kbar must hold the means of the cache as it was
        before the step (init_means, or the previous cached step).  Stage names for `hooks`:
        "pcgi", "refresh", "dense", "sinks", "blocks", "sparse"."""
        def run(name, fn):
            h = hooks.get(name) if hooks else None
            if h:
                h[0]()
            fn()
            if h:
                h[1]()
        run("pcgi", lambda: self.pcgi(conf, mask))
        for l in range(self.layers):
            q, k, v = qs[l], ks[l], vs[l]
            vt = vts[l] if vts is not None else None

            def refresh():
                # a sparse layer refreshes its cache rows and its touched means in one launch
                if l in self.kbar:
                    F.kv_refresh_means(self.active, k_new[l], v_new[l], k, v, self.P, self.bs, self.kbar[l],
                                       n_rows=self.n_active, vt=vt)
                else:
                    F.kv_refresh(self.active, k_new[l], v_new[l], k, v, n_rows=self.n_active, vt=vt)
            run("refresh", refresh)
            if self.is_dense(l):
                run("dense", lambda: self.dense_layer(l, q, k, v, vt))
                if l == self.l_dense - 1:
                    run("sinks", lambda: self.sinks_at(q, k))
            else:
                if self.C:
                    run("blocks", lambda: self.score_blocks(l, q))
                run("sparse", lambda: self.attend(l, q, k, v, vt))

    def dense_refresh(self, qs, ks, vs, outs, vts=None):
        """A block-entry step: every query row of every layer attends to all L keys."""
        for l in range(self.layers):
            F.dense_attention(qs[l], ks[l], vs[l], vt=vts[l] if vts is not None else None, out=outs[l],
                              want_lse=False, scale=self.scale, workspace=self.workspace)
