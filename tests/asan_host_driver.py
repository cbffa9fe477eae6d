"""Drives the host side of liblsa (argument validation, workspace sizing, chunk planning,
stage listing) through the C ABI without a GPU; run by test_host_asan.py in a process
that has the AddressSanitizer runtime preloaded, against the library built with its host
code instrumented.  Device pointers are fake, aligned addresses that the host code only
checks and passes on: every call here must return before any launch.

Usage: python asan_host_driver.py LIB
"""
from __future__ import annotations

import ctypes as C
import itertools
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from learned_top_sparse_amd.abi import SZ, ForwardArgs, SemanticPages, SemanticParams, declare  # noqa: E402

FAKE = 1 << 20   # an aligned stand-in for device memory: never dereferenced on the host

_libc = C.CDLL(None)
_libc.malloc.restype = C.c_void_p
_libc.malloc.argtypes = [C.c_size_t]
_libc.free.argtypes = [C.c_void_p]
_held: list[int] = []


def heap(ctype, n: int = 1, init=None):
    """An exact-size block from the C allocator (which the sanitizer watches, unlike
    Python's own small-object arenas), holding n values of ctype or a copy of init."""
    size = C.sizeof(ctype) * n
    addr = _libc.malloc(size)
    assert addr
    _held.append(addr)
    C.memset(addr, 0, size)
    if init is not None:
        C.memmove(addr, C.addressof(init), size)
    return C.cast(addr, C.POINTER(ctype))


def release() -> None:
    while _held:
        _libc.free(_held.pop())


def forward_args(B, n_q, L, H_I=64, d_I=128, H_q=16, k=2048, two=0, bs=128, nk=64, page=0, select=0, chunk=0):
    a = ForwardArgs()
    a.mode = 1 if (n_q == 1 and B > 1) else 0
    a.two_stage = two
    a.q_idx = a.k_idx = a.w = a.q_pos = a.q = a.k = a.v = FAKE
    a.B, a.n_q, a.L_max, a.H_I, a.d_I, a.H_q, a.d, a.k_top = B, n_q, L, H_I, d_I, H_q, 128, k
    a.block_size, a.n_keep = bs, nk
    a.scale = 0.088
    a.chunk_rows = chunk
    a.idx = a.out = a.count = FAKE
    a.select_mode = select
    if page:
        max_pages = -(-L // page)
        a.L_max = max_pages * page
        a.page_table = FAKE
        a.page_size = page
        a.max_pages = max_pages
        a.n_slots = (B * max_pages + 7) * page
    return a


def main(path: str) -> int:
    L = C.CDLL(path)
    declare(L)
    n = 0
    for s in range(-6, 2):
        assert L.lsa_status_string(s)
    assert L.lsa_version() >= 10000
    # every forward configuration the path has, sized, planned and listed
    shapes = [(1, 1024, 1024, 4, 64, 8, 64), (1, 32768, 32768, 64, 128, 16, 2048), (64, 1, 131073, 64, 128, 16, 2048),
              (1, 16384, 262144, 64, 128, 16, 2048), (3, 1, 5000, 20, 64, 16, 300), (2, 40, 3000, 64, 128, 16, 256)]
    for (B, n_q, Lk, H_I, d_I, H_q, k), two, page, select in itertools.product(
            shapes, (0, 1, 2), (0, 64, 256), (0, 1, 2, 3)):
        bs, nk = (4, k // 4) if two == 2 else (128, 64)
        if two == 2 and nk > 4096:
            continue
        a = forward_args(B, n_q, Lk, H_I, d_I, H_q, k, two, bs, nk, page, select)
        ha = heap(ForwardArgs, init=a)
        ws = heap(SZ)
        st = L.lsa_forward_workspace_size(ha, ws)
        if st != 0:
            release()
            continue
        for budget in (ws[0], ws[0] // 3 + 16, 1 << 20):
            rows, split = heap(C.c_int64), heap(C.c_int32)
            if L.lsa_forward_plan(ha, budget, rows, split) != 0:
                continue
            cnt = heap(C.c_int32)
            assert L.lsa_forward_stages(ha, budget, None, 0, cnt) == 0
            n_codes = cnt[0]
            codes = heap(C.c_int32, max(n_codes, 1))
            assert L.lsa_forward_stages(ha, budget, codes, n_codes, cnt) == 0 and cnt[0] == n_codes
            n += 1
        release()
    # invalid forward arguments return before any launch
    for bad in (forward_args(1, 4, 0), forward_args(1, 4, 100, d_I=96), forward_args(1, 4, 100, H_I=65),
                forward_args(2, 2, 100, two=9), forward_args(1, 4, 100, k=5000), forward_args(1, 4, 100, page=32),
                forward_args(1, 4, 100, two=2, bs=4, nk=10, k=64)):
        hb = heap(ForwardArgs, init=bad)
        assert L.lsa_forward(hb, FAKE, 1 << 20, None) < 0
        assert L.lsa_forward_noalloc(hb, None) < 0
        n += 1
    release()
    # a chunk larger than the allocation-free entry point's device array is refused first
    big = forward_args(1, 1024, 65536, chunk=1024)
    assert L.lsa_forward_noalloc(heap(ForwardArgs, init=big), None) == -3
    # the separate calls' sizes and checks
    for B, n_q, Lk, k in ((1, 4096, 4096, 2048), (64, 1, 131073, 2048), (2, 7, 9000, 64)):
        ws = heap(SZ)
        assert L.lsa_topk_workspace_size(B, n_q, Lk, k, ws) == 0
        assert L.lsa_sparse_attn_workspace_size(B, n_q, 16, 128, k, 0, ws) == 0
        assert L.lsa_block_prefilter_workspace_size(B, n_q, Lk // 128, 128, ws) == 0
        n += 3
    assert L.lsa_topk(None, 10, None, None, 0, 0, 1, 1, 10, 5000, None, None, None, 0, None) == -2
    assert L.lsa_block_cache_paged(None, 64, None, 32, 4, 1, 128, 4, 8, 0, 8, None, None) == -1
    assert L.lsa_block_cache_paged(FAKE, 640, FAKE, 64, 4, 1, 128, 4, 64, 0, 65, FAKE, None) == -1
    # semantic search: parameters, sizes, paging checks
    for prm in ((512, 4, 8, 32), (512, 4, 16, 64), (256, 2, 4, 16), (512, 4, 8, 128), (512, 3, 8, 32)):
        p = heap(SemanticParams, init=SemanticParams(*prm))
        for nb in (0, 1, 256, 513, 4097):
            ws = heap(SZ)
            L.lsa_semantic_select_workspace_size(64, 1, nb, p, ws)
            n += 1
    pg = heap(SemanticPages, init=SemanticPages(FAKE, 3, FAKE, 48, 10, 480))
    p = heap(SemanticParams, init=SemanticParams(512, 4, 8, 32))
    assert L.lsa_semantic_select_paged(FAKE, FAKE, 1, 1, 64, p, pg, 480, 1, FAKE, FAKE, FAKE,
                                       64, 16, 4, 512, FAKE, FAKE, FAKE, 1 << 20, None) < 0
    # the ceilings' microbenchmarks refuse bad arguments on the host
    assert L.lsa_peak_mfma(7, 1, 1, FAKE, None) == -1
    assert L.lsa_peak_read(FAKE, 17, 1, FAKE, None) == -1
    assert L.lsa_peak_gather(None, 1, FAKE, 1, 1, FAKE, None) == -1
    release()
    print(f"host-side calls exercised: {n}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
