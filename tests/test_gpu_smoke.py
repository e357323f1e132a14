"""The smoke check (__graft_entry__.smoke) also runs as a GPU test, so that a
break in it shows up with the other GPU tests."""
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def test_smoke():
    import __graft_entry__
    __graft_entry__.smoke()
