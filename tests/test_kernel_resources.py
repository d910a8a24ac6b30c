"""The compiler's resource report for every kernel of the HIP library: no register
spills and no scratch memory (a spill turns into per-lane memory traffic inside the
hot loops).  The report is written by the library build; the check builds the
library when no report is there."""
import os
import re

import pytest

from hybrid_sparse_linear_la_amd import _build

OBJDIR = os.path.join(_build.PKG, "_build")


def _reports():
    paths = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".resources.txt") for s in _build.SOURCES]
    if not all(os.path.exists(p) for p in paths):
        _build.build()
    return {p: open(p).read() for p in paths}


def _kernels(text):
    """(kernel name, {field: value}) for each kernel in one compiler report."""
    out = []
    for block in text.split("Function Name: ")[1:]:
        name = block.split()[0]
        fields = dict((k.strip(), int(v)) for k, v in re.findall(r"remark:\s+([A-Za-z ]+?(?:\[[^\]]*\])?):\s+(\d+)", block))
        out.append((name, fields))
    return out


def test_every_kernel_is_reported():
    kernels = [k for text in _reports().values() for k in _kernels(text)]
    names = " ".join(n for n, _ in kernels)
    for kernel in ("la_chunk_output_kernel", "la_chunk_state_kernel", "la_decode_kernel", "la_linear_ring_kernel",
                   "la_backward_chunk_kernel", "la_sparse_attn_kernel"):
        assert kernel in names, kernel


@pytest.mark.parametrize("src", _build.SOURCES)
def test_no_spills_and_no_scratch(src):
    path = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".resources.txt")
    text = _reports()[path]
    kernels = _kernels(text)
    if src != "la_api.hip":  # the boundary's host code holds no kernel
        assert kernels, f"no kernel in the report of {src}"
    for name, f in kernels:
        assert f.get("VGPRs Spill", 0) == 0, f"{src}: {name} spills {f['VGPRs Spill']} VGPRs"
        assert f.get("ScratchSize [bytes/lane]", 0) == 0, f"{src}: {name} uses scratch"
