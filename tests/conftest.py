import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmoda")


def pytest_sessionfinish(session, exitstatus):
    """With MODA_PARITY_REPORT set, write every parity check's margins to that file."""
    path = os.environ.get("MODA_PARITY_REPORT")
    if not path:
        return
    try:
        from parity import MARGINS
    except Exception:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        f.write("# check\telement-bound-used\trel-bound-used\n")
        for name, used, rel in MARGINS:
            f.write(f"{name}\t{used:.4f}\t{rel:.4f}\n")
