"""llmk_argmax_noalloc (the allocation-free argmax) against llmk_argmax, through the C ABI (MI355X only).

Two calls in a row on the same GPU share the library's fixed scratch: the first at the largest size it
takes (256 rows of a 128,256-wide vocabulary, planted exact ties), the second smaller (3 rows of 1,000),
so stale partials or tickets of the first call would show in the second. Tokens must be bit-exact with
llmk_argmax and with the oracle; the maximum logits equal.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _rows(rows, n, seed):
    x = synth.normal((rows, n), 40 + seed, 0, 3.0)
    # planted exact ties of each row's maximum at two indices (adjacent, far apart, at the ends)
    for r in range(rows):
        m = float(x[r].max()) + 0.25
        a = (r * 7919) % n
        b = (a + 1 + (r % 3) * (n // 2)) % n
        x[r, a] = x[r, b] = m
    x[0, :] = -np.inf                                   # a row of equal values: index 0
    if rows > 2:
        x[2, 5] = np.nan                                # the first NaN wins
    return x


def _both(x):
    rows, n = x.shape
    lg = dev(x.ravel())
    tok_a = torch.full((rows,), -5, dtype=torch.int32, device="cuda")
    val_a = torch.zeros(rows, dtype=torch.float32, device="cuda")
    ws = llmk.workspace(llmk.argmax_workspace_bytes(rows, n))
    assert llmk.argmax(lg, rows, n, tok_a, val_a, ws) == llmk.OK
    tok_b = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    val_b = torch.zeros(rows, dtype=torch.float32, device="cuda")
    st = llmk.lib.llmk_argmax_noalloc(lg.data_ptr(), lg.numel(), rows, n, tok_b.data_ptr(), val_b.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == llmk.OK, llmk.status_name(st)
    torch.cuda.synchronize()
    return host(tok_a), host(val_a), host(tok_b), host(val_b)


def test_noalloc_argmax_equals_workspace_argmax_twice():
    for rows, n, seed in ((256, 128256, 0), (3, 1000, 1)):
        say(f"argmax_noalloc rows={rows} n={n}")
        x = _rows(rows, n, seed)
        ta, va, tb, vb = _both(x)
        ref = [oracle.argmax(x[r])[0] for r in range(rows)]
        assert tb.tolist() == ta.tolist() == ref
        assert np.array_equal(va.view(np.uint32), vb.view(np.uint32))


def test_noalloc_argmax_refuses_beyond_its_scratch():
    lg = torch.zeros(257 * 10, dtype=torch.float32, device="cuda")
    tok = torch.zeros(257, dtype=torch.int32, device="cuda")
    st = llmk.lib.llmk_argmax_noalloc(lg.data_ptr(), lg.numel(), 257, 10, tok.data_ptr(), None, None)
    assert st == 564
    assert llmk.lib.llmk_argmax_noalloc(lg.data_ptr(), 11, 1, 10, tok.data_ptr(), None, None) == 568
