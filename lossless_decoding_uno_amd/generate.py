"""End-to-end generation over the decode step: prompt prefill in chunks, then
continuous Psi-Spec steps with natural (or forced) acceptance, KV pages handed
out on demand from one pool.

The four library calls do all the device work; this module only orders them,
keeps the page table and reads back the committed tokens.  Tokens per forward
pass (TPF) follow the pages' definition: output tokens per forward pass, where
one step runs two passes (draft and verify) and commits a + 1 tokens, so
1 <= TPF <= (K + 1) / 2 (paperglide reader, "The Uno Framework"); AL is the mean
number of tokens a step commits.  With n draft passes per step (multi-pass
drafting) a step runs n + 1 passes; ``stats`` reports TPF over all of them.
With ``tree=(topk, n_keep)`` each step uses the tree sampler instead of the
linear one: the last draft pass's logits give the prefix tree of the best
n_keep candidates, one tree-masked verify pass scores every node, and the walk
commits the longest accepted path plus one token.
"""
import numpy as np
import torch

from . import (PagedKV, TreeBuffers, alloc_workspace, draft_passes, kv_commit, spec_accept,
               spec_accept_workspace_bytes, tree_accept, tree_build, tree_commit, verify_block,
               verify_tree, workspace_bytes)


class PagePool:
    """Host-side allocator of the KV pages of one PagedKV pool.

    Sequence b owns the pages listed in row b of the page table, in position
    order; ``ensure(b, n)`` appends free pages until the sequence can hold n
    positions, ``release(b)`` returns them.  ``sync()`` copies the rows that
    changed to the device table (call it before a pass that reads them)."""

    def __init__(self, kv):
        self.kv = kv
        self.ps = kv.page_size
        self.free = list(range(kv.n_pages - 1, -1, -1))    # pop() hands out 0, 1, ...
        self.owned = [[] for _ in range(kv.batch)]
        self.table = np.zeros((kv.batch, kv.max_pages), dtype=np.int32)
        self.dirty = False

    def ensure(self, b, n_positions):
        need = (n_positions + self.ps - 1) // self.ps
        if need > self.kv.max_pages:
            raise RuntimeError("sequence %d needs %d pages, the table holds %d"
                               % (b, need, self.kv.max_pages))
        while len(self.owned[b]) < need:
            if not self.free:
                raise RuntimeError("KV page pool exhausted")
            p = self.free.pop()
            self.table[b, len(self.owned[b])] = p
            self.owned[b].append(p)
            self.dirty = True

    def release(self, b):
        self.free.extend(reversed(self.owned[b]))
        self.owned[b] = []
        self.table[b, :] = 0
        self.dirty = True

    def pages_in_use(self):
        return sum(len(o) for o in self.owned)

    def sync(self):
        if self.dirty:
            self.kv.page_table.copy_(torch.from_numpy(self.table))
            self.dirty = False


class Generator:
    """Batch of B sequences with equal-length prompts.

        g = Generator(model, B, K, max_ctx, n_pages)
        g.prefill(prompts)            # int array [B, P]
        tokens = g.generate(n_new)    # list of B token lists
    """

    def __init__(self, model, batch, K, max_ctx, n_pages=None, inv_temp=1.0, seed=0,
                 prefill_chunk=512, page_size=16, device="cuda", n_passes=1, tree=None,
                 kappa=1.0):
        self.model, self.B, self.K = model, batch, K
        self.n_passes = int(n_passes)      # draft passes per step (multi-pass drafting)
        self.kappa = kappa                  # corrector strength between draft passes
        self.cfg = model.cfg
        self.inv_temp, self.seed = float(inv_temp), int(seed)
        self.chunk = int(prefill_chunk)
        self.max_ctx = int(max_ctx)
        max_pages = (self.max_ctx + page_size - 1) // page_size
        self.kv = PagedKV(self.cfg, batch, self.max_ctx, page_size=page_size, device=device,
                          n_pages=n_pages or batch * max_pages)
        self.pool = PagePool(self.kv)
        V = self.cfg["vocab"]
        self.tb = TreeBuffers(batch, K, tree[0], tree[1], V, device) if tree else None
        self.n_rows = self.tb.N if tree else K          # verify rows per sequence
        rows = max(self.n_rows, self.chunk)
        self.ws = alloc_workspace(max(workspace_bytes(model, batch, K, self.max_ctx),
                                      workspace_bytes(model, batch, rows, self.max_ctx)))
        self.aws = alloc_workspace(spec_accept_workspace_bytes(batch, K))
        self.zq = torch.empty((batch, K, V), dtype=torch.float32, device=device)
        self.zp = torch.empty((batch, self.n_rows, V), dtype=torch.float32, device=device)
        self.d = torch.empty((batch, K), dtype=torch.int32, device=device)
        # row maxima of the draft and verify logits (the LM head writes them,
        # the sampler then streams every row once)
        self.qmax = torch.empty((batch, K), dtype=torch.float32, device=device)
        self.pmax = torch.empty((batch, K), dtype=torch.float32, device=device)
        self.a = torch.empty(batch, dtype=torch.int32, device=device)
        self.c = torch.empty((batch, K + 1), dtype=torch.int32, device=device)
        self.e = torch.empty(batch, dtype=torch.int32, device=device)
        self.step_ctr = torch.zeros(batch, dtype=torch.uint64).to(device)
        self.status = torch.zeros(batch, dtype=torch.int32, device=device)
        self.kv_len = np.zeros(batch, dtype=np.int64)          # host mirror
        self.out = [[] for _ in range(batch)]
        self.steps = 0
        self.committed_per_step = []

    # -- prefill: verify passes over the prompt (AR weights, causal), in chunks
    def prefill(self, prompts):
        prompts = np.asarray(prompts, dtype=np.int32)
        assert prompts.shape[0] == self.B and prompts.shape[1] >= 2
        body = prompts[:, :-1]                  # the last prompt token is the first anchor
        dev = self.kv.kv_len.device
        for s in range(0, body.shape[1], self.chunk):
            rows = body[:, s: s + self.chunk]
            n = rows.shape[1]
            for b in range(self.B):
                self.pool.ensure(b, int(self.kv_len[b]) + n)
            self.pool.sync()
            verify_block(self.model, self.kv, torch.from_numpy(np.ascontiguousarray(rows)).to(dev),
                         self.max_ctx, 0, None, self.ws, self.status)
            kv_commit(self.kv, torch.full((self.B,), n - 1, dtype=torch.int32, device=dev), n)
            self.kv_len += n
        self.e.copy_(torch.from_numpy(prompts[:, -1].copy()))
        self._check_status()

    # -- one Psi-Spec step (natural acceptance unless `forced` [B] is given)
    def step(self, forced=None):
        K = self.K
        for b in range(self.B):
            # draft writes kv_len .. kv_len+K-1, verify kv_len+1 .. kv_len+rows
            self.pool.ensure(b, int(self.kv_len[b]) + self.n_rows + 1)
        self.pool.sync()
        draft_passes(self.model, self.kv, self.e, K, self.max_ctx, self.inv_temp, self.seed,
                     self.step_ctr, self.n_passes, self.zq, self.d, self.ws, self.status,
                     kappa=self.kappa, row_max=self.qmax)
        if self.tb is not None:
            if forced is not None:
                raise ValueError("forced accept lengths apply to the linear sampler only")
            tree_build(self.zq, self.d, self.tb, self.status)
            verify_tree(self.model, self.kv, self.tb, self.max_ctx, self.zp, self.ws, self.status)
            tree_accept(self.zp, self.tb, self.inv_temp, self.seed, self.step_ctr, self.a, self.c,
                        self.e, self.status)
            tree_commit(self.model, self.kv, self.tb, self.a, self.step_ctr, self.status)
        else:
            verify_block(self.model, self.kv, self.d, self.max_ctx, 1, self.zp, self.ws,
                         self.status, row_max=self.pmax)
            spec_accept(self.zq, self.zp, self.d, self.inv_temp, self.seed, self.step_ctr,
                        self.a, self.c, self.e, self.aws, status=self.status,
                        forced_accept=forced, draft_row_max=self.qmax,
                        verify_row_max=self.pmax)
            kv_commit(self.kv, self.a, K, self.step_ctr, self.status)
        a = self.a.cpu().numpy().astype(np.int64)
        c = self.c.cpu().numpy()
        for b in range(self.B):
            self.out[b].extend(int(t) for t in c[b, : a[b] + 1])
        self.kv_len += a + 1
        self.steps += 1
        self.committed_per_step.append(a + 1)
        return a

    def generate(self, n_new, forced=None, on_step=None):
        """Step until every sequence has n_new tokens.  A sequence that is done
        while others are not keeps stepping with the batch, but its cache is
        put back to the length it finished at after every step (its later
        tokens are dropped and its steps leave the statistics), so the page
        table never needs more than prompt + n_new + two blocks per sequence.
        ``on_step()`` is called after every step."""
        held = np.full(self.B, -1, dtype=np.int64)
        while min(len(o) for o in self.out) < n_new:
            self.step(None if forced is None else forced[self.steps])
            back = [b for b in range(self.B) if held[b] >= 0]
            for b in back:
                self.kv_len[b] = held[b]
                self.committed_per_step[-1][b] = 0
            for b in range(self.B):
                if held[b] < 0 and len(self.out[b]) >= n_new:
                    held[b] = self.kv_len[b]
            if back:
                self.kv.kv_len.copy_(torch.from_numpy(self.kv_len.astype(np.int32)))
            if on_step is not None:
                on_step()
        self._check_status()
        return [o[:n_new] for o in self.out]

    def stats(self):
        per = np.array(self.committed_per_step, dtype=np.float64)   # [steps, B]
        live = per[per > 0]            # steps of sequences not yet done
        return {"steps": self.steps,
                "AL": float(live.mean()) if live.size else 0.0,
                "TPF": float(live.mean() / (self.n_passes + 1)) if live.size else 0.0,
                "pages_in_use": self.pool.pages_in_use()}

    def _check_status(self):
        st = self.status.cpu().numpy()
        if np.any(st):
            raise RuntimeError("device status flags %s" % st.tolist())
