"""Progress lines that reach the terminal while pytest captures test output.

The full-size GPU tests spend minutes in the fp64 oracle; their stage lines go through
pytest's capture manager so that a run shows it is alive (captured output appears only when
a test ends).  Not a test module.
"""
import sys

_config = None


def set_config(config):
    global _config
    _config = config


def progress(msg):
    capman = _config.pluginmanager.getplugin("capturemanager") if _config is not None else None
    if capman is None:
        print(msg, file=sys.stderr, flush=True)
        return
    with capman.global_and_fixture_disabled():
        print(msg, file=sys.stderr, flush=True)
