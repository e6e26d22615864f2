"""The Python binding's host-array marshalling (no GPU): int32 position / sequence arrays
go to the library as (array, data pointer), with the pointers of recently passed small
arrays remembered."""
import gc

import numpy as np

import kv_cache_causal_amd as kvc


def test_int32_arrays_pass_as_is_and_keep_their_pointer():
    a = np.arange(5, dtype=np.int32)
    arr, ptr = kvc._host_i32(a)
    assert arr is a and ptr == a.ctypes.data
    a[:] = 9                                  # contents change, the buffer does not
    arr2, ptr2 = kvc._host_i32(a)
    assert arr2 is a and ptr2 == ptr == a.ctypes.data


def test_other_inputs_are_converted():
    for x in ([3, 1, 2], np.array([3, 1, 2], np.int64), np.array([[3, 1, 2]], np.int32),
              np.array([3, 9, 1, 9, 2], np.int32)[::2], (3, 1, 2)):
        arr, ptr = kvc._host_i32(x)
        assert arr.dtype == np.int32 and arr.ndim == 1 and arr.flags.c_contiguous
        assert arr.tolist() == [3, 1, 2] and ptr == arr.ctypes.data


def test_a_remembered_array_cannot_move_and_large_arrays_are_not_kept():
    a = np.zeros(8, np.int32)
    kvc._host_i32(a)
    try:                                      # the remembered reference blocks a resize
        a.resize(100)
        moved = True
    except ValueError:
        moved = False
    assert not moved
    big = np.zeros(kvc._PTRS_MAX_SIZE + 1, np.int32)
    kvc._host_i32(big)
    assert id(big) not in kvc._PTRS
    # The table stays bounded however many arrays pass through it.
    for _ in range(3 * kvc._PTRS_MAX):
        kvc._host_i32(np.zeros(2, np.int32))
    gc.collect()
    assert len(kvc._PTRS) <= kvc._PTRS_MAX
