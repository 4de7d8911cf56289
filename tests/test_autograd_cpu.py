"""Host logic of the autograd wrappers: the stale-layout check.  No GPU is
used: the check reads only the handle's generation counter."""
import types

import pytest

from combine_moe_layout_04_amd import autograd as A


def test_a_relaid_handle_is_refused_and_the_same_one_passes():
    handle = types.SimpleNamespace(generation=3)
    ctx = types.SimpleNamespace(handle=handle, generation=3)
    A._same_layout(ctx, "combine")          # the layout the forward used
    handle.generation = 4                   # moe_layout ran again on the handle
    with pytest.raises(A.StaleLayoutError, match="layout 4.*layout 3"):
        A._same_layout(ctx, "combine")
