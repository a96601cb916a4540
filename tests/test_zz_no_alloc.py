"""wa_sparse_attn_fwd_noalloc (the entry point for callers that cannot allocate:
its AUTO schedule word lives in a static device array) against the existing
entry point with a caller workspace, through the C ABI: bitwise the same O, LSE
and G on two calls in a row, the second smaller and with the other schedule
choice, so a stale schedule word from the first call would show."""

import ctypes

import pytest
import torch

import cache_aware_query_amd as caq
import synth
from helpers import banner, gpu

pytestmark = pytest.mark.gpu


def _inputs(seed, heads, seq_len, skip_mode):
    dev = gpu()
    w = synth.random_tiny_case(seed, heads=heads, seq_len=seq_len, head_dim=128, block=128,
                               density=0.4, empty_rows=(1,))
    q, k, v, mask, x0 = (t.to(dev) for t in (w.q, w.k, w.v, w.mask, w.x0))
    idx = caq.build_block_index(mask)
    n_xcd = caq.schedule_info(0, 128)[0]
    ro = caq.reorder_rows(idx, x0, 128, 128, caq.ReorderParams(wave=8, n_slices=n_xcd,
                                                               skip_mode=skip_mode))
    return w, q, k, v, idx, ro


def _outputs(q, seq_len, nnz):
    H, lp, d = q.shape
    return (torch.full_like(q, 7.0), torch.full((H, lp), 7.0, device=q.device),
            torch.full((max(nnz, 1), 128), 7.0, device=q.device))


def _call_noalloc(lib, w, q, k, v, idx, ro, schedule):
    o, lse, g = _outputs(q, w.seq_len, int(idx.row_ptr[-1].item()))
    st = caq._check(lib.wa_sparse_attn_fwd_noalloc(
        caq._ptr(q), caq._ptr(k), caq._ptr(v), q.shape[0], w.seq_len, 128, 128,
        caq._ptr(idx.row_ptr), caq._ptr(idx.col_idx), idx.col_idx.numel(), caq._ptr(ro.perm),
        ro.n_slices, schedule, caq._ptr(ro.skipped), w.scale, caq._ptr(o), caq._ptr(lse),
        caq._ptr(g), caq._stream(q.device)), "wa_sparse_attn_fwd_noalloc")
    return o, lse, g


def _call_workspace(lib, w, q, k, v, idx, ro, schedule):
    o, lse, g = _outputs(q, w.seq_len, int(idx.row_ptr[-1].item()))
    n = caq.sparse_attn_workspace_size(q.shape[0], w.seq_len, 128, 128)
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device=q.device)
    if schedule == caq.WA_SCHED_AUTO:
        caq._check(lib.wa_attn_schedule_select(caq._ptr(ro.skipped), q.shape[0], caq._ptr(ws), n,
                                               caq._stream(q.device)), "wa_attn_schedule_select")
    caq._check(lib.wa_sparse_attn_fwd(
        caq._ptr(q), caq._ptr(k), caq._ptr(v), q.shape[0], w.seq_len, 128, 128,
        caq._ptr(idx.row_ptr), caq._ptr(idx.col_idx), idx.col_idx.numel(), caq._ptr(ro.perm),
        ro.n_slices, schedule, w.scale, caq._ptr(o), caq._ptr(lse), caq._ptr(g), caq._ptr(ws), n,
        caq._stream(q.device)), "wa_sparse_attn_fwd")
    return o, lse, g


def _same(a, b, nnz):
    (o1, l1, g1), (o2, l2, g2) = a, b
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)
    assert torch.equal(g1[:nnz], g2[:nnz])


def test_noalloc_equals_the_workspace_entry_point_on_two_calls():
    lib = caq.load_library()
    # first call: every head kept its order -> the default path; second call, fewer
    # heads and tokens: heads reordered -> XCD-sliced, read from the same static word
    cases = [(41, 4, 2000, caq.WA_SKIP_ALWAYS), (42, 2, 900, caq.WA_SKIP_NEVER)]
    for seed, heads, seq_len, skip_mode in cases:
        banner(f"noalloc AUTO H={heads} L={seq_len} skip_mode={skip_mode}")
        w, q, k, v, idx, ro = _inputs(seed, heads, seq_len, skip_mode)
        nnz = int(idx.row_ptr[-1].item())
        a = _call_noalloc(lib, w, q, k, v, idx, ro, caq.WA_SCHED_AUTO)
        b = _call_workspace(lib, w, q, k, v, idx, ro, caq.WA_SCHED_AUTO)
        torch.cuda.synchronize()
        _same(a, b, nnz)
        # and a schedule that takes no scratch at all
        c = _call_noalloc(lib, w, q, k, v, idx, ro, caq.WA_SCHED_NATURAL)
        d = _call_workspace(lib, w, q, k, v, idx, ro, caq.WA_SCHED_NATURAL)
        torch.cuda.synchronize()
        _same(c, d, nnz)
        _same(a, c, nnz)  # the schedule changes the order of work, not its result


def test_noalloc_checks_its_arguments_first():
    lib = caq.load_library()
    gpu()
    fake = ctypes.c_void_p(16)
    # AUTO without skip flags, bad schedule: refused on the host, nothing enqueued
    assert lib.wa_sparse_attn_fwd_noalloc(fake, fake, fake, 1, 128, 128, 128, fake, fake, 1,
                                          None, 0, caq.WA_SCHED_AUTO, None, 0.1, fake, fake, None,
                                          None) == -1
    assert lib.wa_sparse_attn_fwd_noalloc(fake, fake, fake, 1, 128, 128, 128, fake, fake, 1,
                                          None, 0, 7, None, 0.1, fake, fake, None, None) == -1
