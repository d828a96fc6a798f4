"""Shape checks of the Python binding (no GPU needed).

The C library sees plain pointers, not allocation sizes, so the binding is
what stops a call from writing past a caller's tensors: a state holding fewer
sequences than the call carries, tables whose sequence counts disagree, or a
caller-supplied output of the wrong size must be refused before any launch.
"""

import pytest

from sparse_weight_memory_amd.memory import Config, check_rows, state_strides

CFG = Config(sqrt_slots=8, dim_qk=16, dim_v=12, topk=2, chunk_size=4, num_heads=3, max_batch=8)
H, n, dh, N, dv = 3, 8, 8, 64, 12


def shapes(bk1, bk2, bv):
    return ((bk1, H, n, dh), (bk2, H, n, dh), (bv, H, N, dv))


def test_per_sequence_strides():
    assert state_strides(shapes(8, 8, 8), CFG, 8) == (H * n * dh, H * N * dv)
    assert state_strides(shapes(9, 9, 9), CFG, 8) == (H * n * dh, H * N * dv)   # spare sequences


def test_shared_state_has_zero_strides():
    assert state_strides(((H, n, dh), (H, n, dh), (H, N, dv)), CFG, 8) == (0, 0)


def test_fewer_sequences_than_the_batch_is_refused():
    # [1, H, n, dh] with B = 8: the old check passed it and the library would
    # have read and written seven sequences past the end
    with pytest.raises(ValueError, match="hold 1 sequence"):
        state_strides(shapes(1, 1, 1), CFG, 8)


@pytest.mark.parametrize("counts", [(8, 8, 4), (8, 4, 8), (4, 8, 8), (8, 9, 8)])
def test_sequence_counts_must_agree(counts):
    with pytest.raises(ValueError, match="different numbers of sequences"):
        state_strides(shapes(*counts), CFG, 4)


@pytest.mark.parametrize("bad", [
    ((8, H, n, dh), (8, H, n, dh), (8, H, N, dv + 4)),      # wrong d_v
    ((8, H, n + 1, dh), (8, H, n + 1, dh), (8, H, N, dv)),  # wrong n
    ((8, 1, n, dh), (8, 1, n, dh), (8, 1, N, dv)),          # wrong head count
    ((8 * H, n, dh), (8 * H, n, dh), (8 * H, N, dv)),       # flattened units are not a shared state
    ((H, n, dh), (H, n, dh), (8, H, N, dv)),                # mixed ranks
])
def test_table_shapes_must_match_the_configuration(bad):
    with pytest.raises(ValueError):
        state_strides(bad, CFG, 8)


def test_output_rows_are_checked():
    check_rows("retrieved", (8, 4, H, dv), 8, 4, H, dv)
    check_rows("retrieved", (8, 4, dv), 8, 4, 1, dv)              # [B, T, d_v] when H == 1
    for bad in [(8, 4, H, dv - 4), (7, 4, H, dv), (8, 3, H, dv), (8, 4 * H * dv)]:
        with pytest.raises(ValueError, match="retrieved must be"):
            check_rows("retrieved", bad, 8, 4, H, dv)
    with pytest.raises(ValueError):
        check_rows("retrieved", (8, 4, dv), 8, 4, H, dv)          # 3-D only when H == 1
