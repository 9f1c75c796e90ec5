import os
import sys

_TESTS = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_TESTS)
for p in (_ROOT, _TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


def _reload_tuning():
    import grouped_query_kv_decode_amd as gqa
    if os.path.exists(gqa.library_path()):
        gqa.tuning_reload()


@pytest.fixture(autouse=True)
def _tuning_follows_env(monkeypatch):
    """The library reads its GQA_* launch-plan overrides when it loads and on
    gqa_tuning_reload(), never during a call.  Tests set them with
    monkeypatch.setenv / delenv; here each of those is followed by a reload,
    and after the test the environment is restored and read once more."""
    set_env, del_env = monkeypatch.setenv, monkeypatch.delenv

    def setenv(name, value, prepend=None):
        set_env(name, value, prepend)
        _reload_tuning()

    def delenv(name, raising=True):
        del_env(name, raising)
        _reload_tuning()

    monkeypatch.setenv, monkeypatch.delenv = setenv, delenv
    yield
    monkeypatch.undo()
    _reload_tuning()


@pytest.fixture(autouse=True)
def _counters_zero_between_calls(request):
    """After every GPU test: each workspace the binding cached still holds
    zeroed arrival counters in its first 256 KiB, the state every call must
    leave behind for the next call on that workspace."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch
    import grouped_query_kv_decode_amd as gqa
    torch.cuda.synchronize()
    for key, ws in gqa._ws_cache.items():
        head = ws[:min(ws.numel(), 256 * 1024) // 4 * 4].cpu().view(torch.int32)
        nz = head.nonzero().flatten()[:8].tolist()
        assert not nz, "workspace %s: counters left non-zero at int32 index %s" % (key, nz)
