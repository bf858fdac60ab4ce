"""The oracle against the worked examples the pages print (tests/golden/*.json,
each file names the page and section it comes from)."""
import numpy as np
import pytest

from oracle import ccsim as cs


def _rs3_inputs(golden, dtype):
    g = golden("reduce_scatter_3rank.json")
    xs = []
    for r in range(g["nranks"]):
        chunks = [np.array([r + 1, 2 * (r + 1)], dtype=np.int64) ** (j + 1) for j in range(g["nranks"])]
        xs.append(np.concatenate(chunks))
    if dtype == "int32":
        xs = [x.astype(np.int32) for x in xs]
    elif dtype == "f32":
        xs = [x.astype(np.float32) for x in xs]
    else:
        xs = [cs.f32_to_bf16_bits(x.astype(np.float32)) for x in xs]
    return xs, g["expected"]


@pytest.mark.parametrize("dtype", ["int32", "f32", "bf16"])
def test_reduce_scatter_3rank_example(golden, dtype):
    xs, expected = _rs3_inputs(golden, dtype)
    out = cs.ring_reduce_scatter(xs, "sum", dtype)
    for r in range(3):
        got = out[r] if dtype != "bf16" else cs.bf16_bits_to_f32(out[r])
        assert np.array_equal(np.asarray(got, dtype=np.float64), np.asarray(expected[r], dtype=np.float64)), (r, got)


def test_reduce_scatter_example_via_all_reduce_chunks(golden):
    """The same example through AllReduce: chunk r of every rank's output is the
    expected reduced chunk r (AllReduce = ReduceScatter + AllGather)."""
    xs, expected = _rs3_inputs(golden, "int32")
    out = cs.ring_all_reduce(xs, "sum", "int32")
    for r in range(3):
        for c in range(3):
            assert list(out[r][2 * c:2 * c + 2]) == expected[c]


@pytest.mark.parametrize("dtype", ["int32", "f32", "bf16"])
def test_all_reduce_ranks_123(golden, dtype):
    g = golden("allreduce_ranks_123.json")
    xs = [np.array(v, dtype=np.int32) for v in g["inputs"]]
    if dtype == "f32":
        xs = [x.astype(np.float32) for x in xs]
    elif dtype == "bf16":
        xs = [cs.f32_to_bf16_bits(x.astype(np.float32)) for x in xs]
    out = cs.ring_all_reduce(xs, "sum", dtype)
    for r in range(3):
        got = out[r] if dtype != "bf16" else cs.bf16_bits_to_f32(out[r])
        assert np.array_equal(np.asarray(got, dtype=np.float64), np.array(g["all_reduce"][r], dtype=np.float64))
    # Reduce to rank 0: the plain result on rank 0, the others untouched
    red0 = cs.plain_reduce([np.array(v, dtype=np.int32) for v in g["inputs"]], "sum", "int32")
    assert list(red0) == g["reduce_dst0"][0]


@pytest.mark.parametrize("schedule", ["ring", "binomial"])
def test_broadcast_examples(golden, schedule):
    for case in golden("broadcast_examples.json")["cases"]:
        xs = [np.array(v, dtype=np.float32) for v in case["inputs"]]
        out = cs.broadcast(xs, case["root"], schedule)
        for r in range(len(xs)):
            assert list(out[r]) == case["expected"][r]


def test_all_gather_3rank(golden):
    g = golden("allgather_3rank.json")
    shards = [np.array(v, dtype=np.int32) for v in g["inputs"]]
    for fn in (cs.ring_all_gather,):
        out = fn(shards, "int32")
        for r in range(3):
            assert list(out[r]) == g["expected_each_rank"]


@pytest.mark.parametrize("algo", ["ring", "hd", "butterfly"])
def test_example_1_1_four_gpus(golden, algo):
    g = golden("ring_trace_4gpu.json")
    fn = {"ring": cs.ring_all_reduce, "hd": cs.hd_all_reduce, "butterfly": cs.butterfly_all_reduce}[algo]
    for dtype in ("int32", "f32"):
        xs = [np.array(v, dtype=np.int32 if dtype == "int32" else np.float32) for v in g["inputs"]]
        out = fn(xs, "sum", dtype)
        for r in range(4):
            assert list(out[r]) == g["expected"]


@pytest.mark.parametrize("algo", ["ring", "hd", "butterfly"])
def test_figure5_all_reduce_one_element(golden, algo):
    """M=1 < N=4: three of the four ring chunks are empty."""
    g = golden("figure5_primitives.json")["all_reduce"]
    fn = {"ring": cs.ring_all_reduce, "hd": cs.hd_all_reduce, "butterfly": cs.butterfly_all_reduce}[algo]
    xs = [np.array(v, dtype=np.int32) for v in g["inputs"]]
    out = fn(xs, "sum", "int32")
    for r in range(4):
        assert list(out[r]) == g["expected"]


def test_figure5_reduce_scatter_and_all_gather_symbolic():
    """Figure 5's symbolic panels: G_i holds [a_i, b_i, c_i, d_i]; after
    ReduceScatter G0 holds sum a, G1 sum b ...; AllGather of a, b, c, d gives
    [a, b, c, d] everywhere.  Symbols are encoded as distinct powers of two."""
    N = 4
    xs = [np.array([1 << (4 * c + i) for c in range(N)], dtype=np.int64).astype(np.int32) for i in range(N)]
    out = cs.ring_reduce_scatter(xs, "sum", "int32")
    for c in range(N):
        assert int(out[c][0]) == sum(1 << (4 * c + i) for i in range(N))
    shards = [np.array([10 + i], dtype=np.int32) for i in range(N)]
    ag = cs.ring_all_gather(shards, "int32")
    for r in range(N):
        assert list(ag[r]) == [10, 11, 12, 13]
