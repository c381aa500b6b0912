"""Writes stubs.cpp: a no-op definition of every kernel launcher that
moe_internal.h declares (hipError_t launch_*), each counting its calls, so
that the host code of the C ABI links and runs without a GPU."""
import re
import sys


def stubs(header_text: str) -> str:
    decls = re.findall(r"hipError_t\s+(launch_\w+)\s*\(([^;]*?)\)\s*;", header_text, flags=re.S)
    out = ['#include "moe_internal.h"', "int g_launches = 0;", "namespace moe {"]
    for name, params in decls:
        params = re.sub(r"\s*=\s*[^,)]+", "", params)     # drop default arguments
        out.append(f"hipError_t {name}({params}) {{ ++g_launches; return hipSuccess; }}")
    out.append("}  // namespace moe")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    header, target = sys.argv[1], sys.argv[2]
    with open(target, "w") as f:
        f.write(stubs(open(header).read()))
