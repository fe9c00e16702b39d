import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Table of every layer comparison the GPU tests made (cosine, max-abs
    over RMS, and max-abs beyond bf16 rounding over RMS against its bar), and
    a copy in the file MOE_FP4_PARITY_OUT names, if set."""
    mod = sys.modules.get("gpu_util") or sys.modules.get("tests.gpu_util")
    recs = getattr(mod, "RECORDS", None) if mod else None
    if not recs:
        return
    lines = ["| test | case | values | cos | max-abs / RMS | beyond bf16 rounding / RMS | bar |",
             "|---|---|---|---|---|---|---|"]
    for r in recs:
        lines.append(f"| {r['test'].split('::')[-1]} | {r['label'].strip()} | {r['n']} | {r['cos']:.8f} | "
                     f"{r['maxabs_rel']:.3e} | {r['excess_rel']:.3e} | {r['bar']} |")
    worst = max(recs, key=lambda r: r["excess_rel"] / r["bar"])
    lines.append("")
    lines.append(f"{len(recs)} comparisons; lowest cos {min(r['cos'] for r in recs):.8f}; largest "
                 f"beyond-rounding/RMS relative to its bar: {worst['excess_rel']:.3e} (bar {worst['bar']}) "
                 f"in {worst['test'].split('::')[-1]} / {worst['label'].strip()}")
    terminalreporter.write_sep("-", "layer parity against the oracle")
    for l in lines:
        terminalreporter.write_line(l)
    out = os.environ.get("MOE_FP4_PARITY_OUT")
    if out:
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
