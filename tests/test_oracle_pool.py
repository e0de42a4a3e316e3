"""Host logic of the tests' oracle thread pools (CPU only): the row spans
that split a head among workers, and the BLAS limit held meanwhile."""
import pytest

from gpu_common import oracle_threads, row_spans, spans_per_head


@pytest.mark.parametrize("n,causal,parts", [(65536, True, 4), (16384, True, 1), (2048, False, 3), (1000, True, 5),
                                            (256, False, 8), (300, True, 2), (1, False, 4)])
def test_row_spans_cover_every_row_once_on_aligned_cuts(n, causal, parts):
    spans = row_spans(n, causal, parts)
    assert spans[0][0] == 0 and spans[-1][1] == n and 1 <= len(spans) <= parts
    for (a0, a1), (b0, b1) in zip(spans[:-1], spans[1:]):
        assert a1 == b0 and a0 < a1 and b0 % 256 == 0


def test_causal_spans_balance_the_quadratic_work():
    spans = row_spans(65536, True, 4)
    work = [r1 * r1 - r0 * r0 for r0, r1 in spans]
    assert len(spans) == 4 and max(work) <= 1.05 * min(work)


def test_spans_per_head_gives_each_worker_about_two_tasks():
    assert spans_per_head(8, 65536, 16) == 4
    assert spans_per_head(512, 2048, 16) == 1
    assert spans_per_head(1, 300, 16) == 1
    assert spans_per_head(2, 256 * 40, 8) == 8


def test_oracle_pool_holds_blas_to_one_thread_and_restores_it():
    threadpoolctl = pytest.importorskip("threadpoolctl")
    before = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i["user_api"] == "blas"]
    with oracle_threads() as workers:
        assert 1 <= workers <= 16
        inside = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i["user_api"] == "blas"]
        assert all(t == 1 for t in inside)
    after = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i["user_api"] == "blas"]
    assert after == before
