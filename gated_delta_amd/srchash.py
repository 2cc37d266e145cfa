"""Hash of the device code (the HIP kernels and the headers they include),
comments and whitespace removed, so that the HBM counter summary under
profiles/ stays attached to the code it was measured on and no longer
matches once any kernel changes."""
import glob
import hashlib
import os
import re

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def _code_only(text: str) -> str:
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(_CSRC, "*"))):
        if os.path.basename(f) == "rda_api.hip":   # host-side launch code only
            continue
        h.update(os.path.basename(f).encode())
        h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]
