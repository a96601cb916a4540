"""One pass of the hot path with buffers allocated once.

``HotPath.step`` enqueues, on the current stream and without allocating or
synchronising:

  1. wa_build_block_index   mask -> CSR + CSC                  (WaveAlign §II-B)
  2. wa_reorder_rows        per-head permutation              (WaveAlign §IV)
  3. wa_sparse_attn_fwd     attention in the permuted order   (WaveAlign §II-C, §V)
                            + Phase-1 block LSE G             (GSRS §5.3)
  4. wa_block_importance    block weights W                   (GSRS §5.3 Phase 2)
  5. wa_topp_select         next block mask                   (GSRS Algorithm 3)

Steps 4-5 run only when ``gsrs_p`` is set; step 2 is replaced by the identity
order when ``reorder`` is None.  ``GsrsSearch`` chains three such passes into the
GSRS search step (full pass, Top-p candidates, restricted second selection).
"""

from __future__ import annotations

import ctypes

import torch

from . import (WA_SCHED_AUTO, WA_SCHED_DEFAULT, WA_SCHED_XCD_SLICED, WA_SKIP_ADAPTIVE,
               BlockIndex, ReorderParams, _check, _ptr, _stream, load_library, reorder_needs_csc,
               sparse_attn_workspace_size)


class HotPath:
    def __init__(self, heads: int, seq_len: int, head_dim: int, block: int, device,
                 capacity: int | None = None, reorder: ReorderParams | None = None,
                 schedule: int = WA_SCHED_XCD_SLICED, gsrs_p: float | None = 0.9,
                 head_capacity: int | None = None):
        # capacity: CSR entries the buffers hold (all heads); head_capacity: an upper
        # bound on the selected blocks of any one head, if the caller knows one (from
        # how its masks are made).  Both only bound the adaptive skip's size and work
        # rules on the host; a head above head_capacity is still attended correctly,
        # it may just keep its original order.
        self.lib = load_library()
        self.H, self.L, self.d, self.b = heads, seq_len, head_dim, block
        self.mb = -(-seq_len // block)
        self.lp = self.mb * block
        self.device = torch.device(device)
        self.cap = heads * self.mb * self.mb if capacity is None else int(capacity)
        self.head_cap = None if head_capacity is None else int(head_capacity)
        self.reorder = reorder
        if schedule == WA_SCHED_AUTO and reorder is None:
            raise ValueError("WA_SCHED_AUTO follows the reorder's skip flags; give a reorder")
        self.schedule = schedule
        self.gsrs_p = gsrs_p
        dev = self.device
        i32 = dict(dtype=torch.int32, device=dev)
        H, mb = heads, self.mb
        self.row_ptr = torch.empty(H * mb + 1, **i32)
        self.row_nnz = torch.empty(H * mb, **i32)
        self.col_idx = torch.empty(max(self.cap, 1), **i32)
        # The transposed lists are built only when the reorder cannot hold the mask
        # as bitmasks in LDS.
        self.with_csc = reorder is not None and reorder_needs_csc(mb, mb)
        self.csc_ptr = torch.empty(H * mb + 1, **i32) if self.with_csc else None
        self.csc_idx = torch.empty(max(self.cap, 1), **i32) if self.with_csc else None
        self.perm = torch.empty(H, mb, **i32)
        self.inv_perm = torch.empty(H, mb, **i32)
        self.skipped = torch.empty(H, dtype=torch.uint8, device=dev)
        self.angles = torch.empty(H, mb, dtype=torch.float64, device=dev)
        self.stats = torch.empty(H, 5, dtype=torch.float64, device=dev)
        self.o = torch.empty(H, self.lp, head_dim, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(H, self.lp, dtype=torch.float32, device=dev)
        self.g = (torch.empty(max(self.cap, 1), block, dtype=torch.float32, device=dev)
                  if gsrs_p is not None else None)
        self.w = (torch.empty(max(self.cap, 1), dtype=torch.float32, device=dev)
                  if gsrs_p is not None else None)
        self.next_mask = (torch.empty(H, mb, mb, dtype=torch.uint8, device=dev)
                          if gsrs_p is not None else None)
        self.ws_bytes = sparse_attn_workspace_size(heads, seq_len, head_dim, block)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.entropy = None   # [H, L_pad] row attention entropy, when diagnostics are on
        self.distance = None  # [H, L_pad] mean attention distance (tokens)
        self._params = (reorder or ReorderParams())._c()
        self.host_skip = False
        self._decide_on_host()

    def _decide_on_host(self) -> None:
        # The adaptive skip's size and work rules (WaveAlign §IV-E) bounded on the host:
        # when even a full mask (MB x NB selected blocks, or the capacity or the
        # per-head capacity if smaller) could not pass them, every head keeps its order
        # whatever the mask, so the
        # reorder is not launched and the attention runs the default path
        # (WA_SCHED_DEFAULT, what WA_SCHED_AUTO would choose), at no cost over not
        # reordering.
        r = self.reorder
        self.host_skip = False
        if r is None or r.skip_mode != WA_SKIP_ADAPTIVE:
            return
        ws = float(self.mb * self.b * self.d * 4)
        pairs = min(self.mb * self.mb, self.cap)
        if self.head_cap is not None:
            pairs = min(pairs, self.head_cap)
        fmax = 4.0 * self.b * self.b * self.d * pairs
        if not (ws > r.ws_min_bytes and fmax >= r.flops_min):
            self.host_skip = True
            H, mb = self.H, self.mb
            ident = torch.arange(mb, dtype=torch.int32, device=self.device).repeat(H, 1)
            self.perm.copy_(ident)
            self.inv_perm.copy_(ident)
            self.skipped.fill_(1)

    def enable_diagnostics(self) -> None:
        """Every later attention pass also writes the row entropy and mean attention
        distance (wa_sparse_attn_fwd_diag, GSRS §4)."""
        if self.entropy is None:
            self.entropy = torch.empty(self.H, self.lp, dtype=torch.float32, device=self.device)
            self.distance = torch.empty_like(self.entropy)

    def set_reorder_params(self, reorder: ReorderParams) -> None:
        """New reorder parameters for a path built with reordering."""
        if self.reorder is None:
            raise ValueError("this path was built without reordering")
        self.reorder = reorder
        self._params = reorder._c()
        self._decide_on_host()

    def index(self) -> BlockIndex:
        return BlockIndex(self.row_ptr, self.col_idx, self.row_nnz, self.csc_ptr, self.csc_idx,
                          self.H, self.mb, self.mb)

    # Individual stages (each enqueues its launches on the current stream).
    def build_index(self, mask: torch.Tensor, transposed: bool = True) -> None:
        """CSR of the mask, and the transposed lists when the reorder needs them
        (``transposed=False`` skips those: the index of the unreordered path)."""
        lib, s = self.lib, _stream(self.device)
        csc = transposed and self.with_csc
        _check(lib.wa_build_block_index(_ptr(mask), self.H, self.mb, self.mb, _ptr(self.row_ptr),
                                        _ptr(self.col_idx), self.cap, _ptr(self.row_nnz),
                                        _ptr(self.csc_ptr if csc else None),
                                        _ptr(self.csc_idx if csc else None),
                                        self.cap if csc else 0, s),
               "wa_build_block_index")

    def reorder_rows(self, x0: torch.Tensor) -> None:
        if self.host_skip:
            return
        lib, s = self.lib, _stream(self.device)
        _check(lib.wa_reorder_rows(_ptr(self.row_ptr), _ptr(self.col_idx), _ptr(self.csc_ptr),
                                   _ptr(self.csc_idx), self.cap, _ptr(x0), self.H, self.mb, self.mb,
                                   self.b, self.d, ctypes.byref(self._params), _ptr(self.perm),
                                   _ptr(self.inv_perm), _ptr(self.skipped), _ptr(self.angles),
                                   _ptr(self.stats), s), "wa_reorder_rows")
        if self.schedule == WA_SCHED_AUTO:
            # all heads skipped: the attention falls back to the default path
            # (WA_SCHED_DEFAULT), chosen on the device (WaveAlign §VI-F)
            _check(lib.wa_attn_schedule_select(_ptr(self.skipped), self.H, _ptr(self.workspace),
                                               self.ws_bytes, s), "wa_attn_schedule_select")

    def attention(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  permuted: bool = True) -> None:
        """The attention pass in the reordered order, or with ``permuted=False`` in the
        original order (the unreordered path, on the same buffers)."""
        lib, s = self.lib, _stream(self.device)
        use_perm = permuted and self.reorder is not None and not self.host_skip
        perm = self.perm if use_perm else None
        schedule = self.schedule
        if not use_perm and schedule == WA_SCHED_AUTO:
            schedule = WA_SCHED_DEFAULT
        g = self.g if self.gsrs_p is not None else None
        slices = self.reorder.n_slices if perm is not None else 0
        args = (_ptr(q), _ptr(k), _ptr(v), self.H, self.L, self.d, self.b, _ptr(self.row_ptr),
                _ptr(self.col_idx), self.cap, _ptr(perm), slices, schedule, self.d ** -0.5,
                _ptr(self.o), _ptr(self.lse), _ptr(g))
        if self.entropy is not None:
            _check(lib.wa_sparse_attn_fwd_diag(*args, _ptr(self.entropy), _ptr(self.distance),
                                               _ptr(self.workspace), self.ws_bytes, s),
                   "wa_sparse_attn_fwd_diag")
        else:
            _check(lib.wa_sparse_attn_fwd(*args, _ptr(self.workspace), self.ws_bytes, s),
                   "wa_sparse_attn_fwd")

    def attention_plain(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
        """The attention pass without the block LSE, whatever ``gsrs_p`` is."""
        saved, self.gsrs_p = self.gsrs_p, None
        try:
            self.attention(q, k, v)
        finally:
            self.gsrs_p = saved

    def importance(self) -> None:
        """Block weights W of the last attention pass (it must have emitted G)."""
        lib, s = self.lib, _stream(self.device)
        _check(lib.wa_block_importance(_ptr(self.g), _ptr(self.lse), _ptr(self.row_ptr), self.cap,
                                       self.H, self.mb, self.L, self.b, _ptr(self.w), s),
               "wa_block_importance")

    def select(self) -> None:
        lib, s = self.lib, _stream(self.device)
        _check(lib.wa_block_importance(_ptr(self.g), _ptr(self.lse), _ptr(self.row_ptr), self.cap,
                                       self.H,
                                       self.mb, self.L, self.b, _ptr(self.w), s),
               "wa_block_importance")
        _check(lib.wa_topp_select(_ptr(self.w), _ptr(self.row_ptr), _ptr(self.col_idx), self.cap,
                                  self.H,
                                  self.mb, self.mb, float(self.gsrs_p), _ptr(self.next_mask), s),
               "wa_topp_select")

    def step(self, q, k, v, mask, x0) -> None:
        self.build_index(mask)
        if self.reorder is not None:
            self.reorder_rows(x0)
        self.attention(q, k, v)
        if self.gsrs_p is not None:
            self.select()


class GsrsSearch:
    """The GSRS search step around WaveAlign, with buffers allocated once.

    ``step`` enqueues on the current stream:

      1. a full (all blocks) pass that also emits the Phase-1 block LSE G
         (GSRS §5.3 Phase 1) and the row LSE;
      2. the Phase-2 block importance W (§5.3 Phase 2);
      3. Top-p at ``p1`` over all blocks, giving the candidate set S1 (Algorithm 3);
      4. the WaveAlign reorder and the sparse pass over S1, again with G;
      5. W and Top-p at ``p2`` restricted to S1, giving S2 (a subset of S1, the mask
         of a later denoising step), and the reordered sparse pass over S2.

    Every pass has the full capacity H*MB*MB, so no selected set can overflow.
    """

    def __init__(self, heads: int, seq_len: int, head_dim: int, block: int, device,
                 reorder: ReorderParams | None, p1: float = 0.9, p2: float = 0.8,
                 schedule: int = WA_SCHED_XCD_SLICED):
        self.dense = HotPath(heads, seq_len, head_dim, block, device, reorder=None,
                             schedule=schedule, gsrs_p=p1)
        self.s1 = HotPath(heads, seq_len, head_dim, block, device, reorder=reorder,
                          schedule=schedule, gsrs_p=p2)
        self.s2 = HotPath(heads, seq_len, head_dim, block, device, reorder=reorder,
                          schedule=schedule, gsrs_p=None)
        self.ones = torch.ones(heads, self.dense.mb, self.dense.mb, dtype=torch.uint8,
                               device=self.dense.device)

    @property
    def mask1(self) -> torch.Tensor:
        return self.dense.next_mask

    @property
    def mask2(self) -> torch.Tensor:
        return self.s1.next_mask

    def step(self, q, k, v, x0) -> None:
        self.dense.step(q, k, v, self.ones, x0)      # steps 1-3
        self.s1.step(q, k, v, self.mask1, x0)        # steps 4-5 (W and Top-p over S1)
        self.s2.step(q, k, v, self.mask2, x0)        # the pass over S2

    def selected_pairs(self) -> tuple[int, int, int]:
        """Block pairs of the dense pass, S1 and S2 (reads back three counts)."""
        return tuple(int(hp.row_ptr[-1].item()) for hp in (self.dense, self.s1, self.s2))


class GsrsSchedule:
    """The GSRS inference schedule over denoising steps, around WaveAlign.

    The GSRS page describes its pipeline (warmup, fused evaluation, growing sparsity,
    reduced search, mask reuse; §4-5 and Algorithm 4, whose listing the text only
    summarises).  Read plainly, step t of ``steps`` runs:

      * t < T[0] (warmup): full attention;
      * t = T[0] (first search): full attention with the block LSE, then block
        importance and Top-p at p[0]; the kept set is the candidate set S1 and the
        current mask;
      * t = T[k], k >= 1 (reduced search): attention over S1 with the block LSE,
        importance normalised over S1, Top-p at p[k]; the kept set (inside S1) is the
        current mask;
      * any other t > T[0]: attention under the current mask (mask reuse).

    Every sparse pass runs in the WaveAlign order of its mask; a mask's index and
    reorder are built once, when the mask is chosen, and reused until it changes.
    ``inputs(t)`` returns the (q, k, v, x0) of step t.
    """

    def __init__(self, heads: int, seq_len: int, head_dim: int, block: int, device,
                 reorder: ReorderParams | None, steps: int = 50,
                 search_steps=(10, 20, 30, 40), thresholds=(0.95, 0.9, 0.85, 0.8),
                 schedule: int = WA_SCHED_XCD_SLICED, diagnostics: bool = False):
        if len(search_steps) != len(thresholds) or not search_steps:
            raise ValueError("one threshold per search step")
        if list(search_steps) != sorted(search_steps) or search_steps[-1] >= steps:
            raise ValueError("search steps must be increasing and below the step count")
        self.steps, self.T, self.p = steps, tuple(search_steps), tuple(thresholds)
        self.full = HotPath(heads, seq_len, head_dim, block, device, reorder=None,
                            schedule=schedule, gsrs_p=thresholds[0])
        self.search = HotPath(heads, seq_len, head_dim, block, device, reorder=reorder,
                              schedule=schedule, gsrs_p=thresholds[-1])
        self.sparse = HotPath(heads, seq_len, head_dim, block, device, reorder=reorder,
                              schedule=schedule, gsrs_p=None)
        mb = self.full.mb
        self.ones = torch.ones(heads, mb, mb, dtype=torch.uint8, device=self.full.device)
        self.s1 = torch.zeros_like(self.ones)     # candidate set of the first search
        self.mask = torch.zeros_like(self.ones)   # current mask
        self.kinds: list[str] = []                # what each step ran
        # With diagnostics, per step the mean row entropy and mean attention distance
        # over the valid rows (device scalars; GSRS §4, Fig. 1 tracks both over steps).
        self.diagnostics = diagnostics
        self.trace: list[tuple] = []
        if diagnostics:
            for path in (self.full, self.search, self.sparse):
                path.enable_diagnostics()

    def run(self, inputs, on_step=None) -> None:
        """Enqueue the whole schedule; ``on_step(t, kind)`` is called after each step."""
        self.kinds = []
        self.full.build_index(self.ones)
        for t in range(self.steps):
            q, k, v, x0 = inputs(t)
            if t < self.T[0]:
                kind = "warmup"
                self.full.attention_plain(q, k, v)
            elif t == self.T[0]:
                kind = "search"
                self.full.attention(q, k, v)
                self.full.select()
                self.s1.copy_(self.full.next_mask)
                self.mask.copy_(self.s1)
                self.search.build_index(self.s1)
                if self.search.reorder is not None:
                    self.search.reorder_rows(x0)
                self._choose_mask(x0)
            elif t in self.T:
                kind = "search"
                self.search.gsrs_p = self.p[self.T.index(t)]
                self.search.attention(q, k, v)
                self.search.select()
                self.mask.copy_(self.search.next_mask)
                self._choose_mask(x0)
            else:
                kind = "reuse"
                self.sparse.attention(q, k, v)
            self.kinds.append(kind)
            if self.diagnostics:
                path = (self.full if (t < self.T[0] or t == self.T[0]) else
                        self.search if t in self.T else self.sparse)
                L = path.L
                self.trace.append((t, kind, path.entropy[:, :L].mean(),
                                   path.distance[:, :L].mean()))
            if on_step is not None:
                on_step(t, kind)

    def _choose_mask(self, x0) -> None:
        self.sparse.build_index(self.mask)
        if self.sparse.reorder is not None:
            self.sparse.reorder_rows(x0)
