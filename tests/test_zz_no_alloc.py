"""lsa_forward_noalloc (the library's own device array as the workspace) against
lsa_forward with a workspace of its own: the same index lists, counts, outputs and
LSE bit for bit, on calls in a row whose later ones are smaller (the array then holds
the earlier call's contents), and on a prefill chunk that the array's size splits into
more chunks than lsa_forward's workspace does."""
from __future__ import annotations

import pytest
import torch

import synthetic
from tests.gpu_util import dev

pytestmark = [pytest.mark.gpu]


@pytest.fixture(scope="module")
def lsa():
    import learned_top_sparse_amd as m
    m.lib()
    return m


def _same(a: dict, b: dict, tag: str):
    for name in ("idx", "count", "out", "lse"):
        assert torch.equal(a[name], b[name]), f"{tag}: {name} differs"


def _case(lsa, wl, tag):
    print(f"[noalloc {tag}: B={wl.B} n_q={wl.n_q} L={wl.L}]", flush=True)
    inp = synthetic.make_inputs(wl, dev())
    want = lsa.lsa_forward(inp, k_top=wl.k)
    got = lsa.lsa_forward_noalloc(inp, k_top=wl.k)
    torch.cuda.synchronize()
    _same(got, want, tag)
    return inp, got


def test_noalloc_calls_in_a_row(lsa):
    """Decode over 64 sequences, then a smaller decode, then a short prefill chunk."""
    base = synthetic.WORKLOADS["decode_128k"]
    _case(lsa, base.replace(L=60001, q_pos0=60000), "decode 64 x 60001")
    _case(lsa, base.replace(B=5, L=7001, q_pos0=7000), "decode 5 x 7001")
    _case(lsa, synthetic.WORKLOADS["tiny_prefill_1k"].replace(n_q=300, L=700, q_pos0=400), "prefill 300")


def test_noalloc_prefill_in_more_chunks(lsa):
    """2048 queries over 20000 keys: lsa_forward's workspace takes them in one chunk, the
    device array in several; the results agree bit for bit."""
    wl = synthetic.WORKLOADS["chunk_256k"].replace(n_q=2048, L=20000, q_pos0=20000 - 2048)
    inp, got = _case(lsa, wl, "prefill 2048 x 20000")
    rows_own, _ = lsa.lsa_forward_plan(inp, wl.k, lsa.lsa_forward_workspace_size(inp, wl.k))
    rows_arr, _ = lsa.lsa_forward_plan(inp, wl.k, lsa.NOALLOC_SCRATCH_BYTES)
    assert rows_own == 2048 and rows_arr < 2048, (rows_own, rows_arr)


def test_noalloc_rejects_oversized_chunks(lsa):
    """A requested chunk that does not fit the array is refused before any launch."""
    wl = synthetic.WORKLOADS["chunk_256k"].replace(n_q=1024, L=65536, q_pos0=65536 - 1024)
    inp = synthetic.make_inputs(wl, dev())
    # chunks of 128 rows (330 KB each: score row, sampled scores, candidate list) fit
    # the 128 MiB array; chunks of 256 do not
    out = lsa.lsa_forward_noalloc(inp, k_top=wl.k, chunk_rows=128)
    torch.cuda.synchronize()
    before = {name: v.clone() for name, v in out.items()}
    with pytest.raises(lsa.LsaError) as e:
        lsa.lsa_forward_noalloc(inp, k_top=wl.k, chunk_rows=256, out=out)
    assert e.value.status == -3
    torch.cuda.synchronize()
    _same(out, before, "outputs untouched by the refused call")
    # the same chunks through lsa_forward (chunks of 128 rows split the attention in two,
    # so a different chunking would round the outputs differently)
    want = lsa.lsa_forward(inp, k_top=wl.k, chunk_rows=128)
    torch.cuda.synchronize()
    _same(out, want, "chunks of 128")
