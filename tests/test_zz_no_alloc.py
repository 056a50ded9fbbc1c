"""csa2_sparse_attn_noalloc (the attention call without a workspace: split partials and
arrival counters in the library's static per-device scratch) against csa2_sparse_attn with
a workspace of its own: two calls in a row, the second with a smaller batch, each
bit-identical to the workspace call (same kernels and split plan) and within 2e-3 of the
oracle."""
import numpy as np
import pytest
import torch

import kv_cache_decode_csa2_amd as k
import oracle
import synth_inputs as si
from gpu_harness import GpuState, attn_close
from harness import OracleState, make_table

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def test_noalloc_attention_matches_workspace_call():
    wl = si.small("noal", 401, [5000, 700, 3000, 4000, 64, 2500, 1000, 6000], H_I=4, d_I=64,
                  K_blk=64, k=450, H_q=32, W=100)
    table, nblk = make_table(wl.ctx, seed=wl.seed)
    o = OracleState(wl, table, nblk)
    g = GpuState(wl, table, nblk)
    _, _, tg, tlg = g.index_full(*g.layer_q(0))
    _, _, to, tlo = oracle.index_full(o.cfg, *o.layer_q(0), o.idx, o.table, o.ctx)
    assert np.array_equal(_np(tg), to)
    swg, swo = g.layer_swa(0), o.layer_swa(0)
    qa = si.layer_attn_q(wl, 0)
    for rows in (list(range(8)), [5]):  # the second call is smaller
        sel = torch.tensor(rows, device="cuda")
        args = (g.cfg, torch.from_numpy(qa[rows].view(np.int16)).cuda(), g.kv, g.n_blocks,
                g.table[sel].contiguous(), swg[sel].contiguous(), g.C, g.ctx[sel].contiguous(),
                tg[sel].contiguous(), tlg[sel].contiguous())
        B = len(rows)
        res = []
        for noalloc in (False, True):
            out = torch.full((B, wl.H_q, wl.D), float("nan"), device="cuda")
            lse = torch.full((B, wl.H_q), float("nan"), device="cuda")
            if noalloc:
                k.csa2_sparse_attn_noalloc(*args, out, lse)
            else:
                ws = torch.zeros(k.csa2_workspace_bytes(g.cfg, k.CSA2_OP_SPARSE_ATTN, B,
                                                        table.shape[1]),
                                 dtype=torch.uint8, device="cuda")
                k.csa2_sparse_attn(*args, out, lse, ws)
            torch.cuda.synchronize()
            res.append((_np(out), _np(lse)))
        (oa, la), (ob, lb) = res
        assert np.array_equal(oa.view(np.uint32), ob.view(np.uint32)), rows
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), rows
        ro, rl = oracle.sparse_attn(o.cfg, qa[rows], o.kv, o.table[rows], swo[rows], o.C,
                                    o.ctx[rows], to[rows], tlo[rows])
        ok, rel, lerr = attn_close(ob, lb, ro, rl)
        assert ok, (rows, rel, lerr)
