import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.hookimpl(trylast=True)
def pytest_collection_modifyitems(items):
    """Run the full-size tests one config after the other (each config's
    inputs are generated and its GPU path run once, by a module-scoped
    fixture): stable-sort those items by config, in their own slots."""
    slots = [i for i, it in enumerate(items)
             if getattr(it, "callspec", None) is not None and "fullsize" in it.callspec.params]
    ordered = sorted((items[i] for i in slots), key=lambda it: it.callspec.params["fullsize"])
    for i, it in zip(slots, ordered):
        items[i] = it
