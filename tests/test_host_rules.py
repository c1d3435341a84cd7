"""Host-side checks of the planning rules the kernels and the C-ABI share (no GPU).

The attention grid is sized from the longest reach in a batch, and each workgroup
takes one (chunk, kv head, stream) item, returning at once past its stream's own
chunks. That is correct only if a stream's chunk count never decreases as its reach
grows and no chunk exceeds the 64 pages whose ids the kernel holds one per lane. The
rule lives in a header shared by the host plan and the kernels; this test compiles it
for the host and checks both properties, and that the chunks cover the reach, over
every reach up to 20,000 pages. (The last chunks of a rounded-up split may be empty;
the kernel gives them no pages.)
"""
import os
import subprocess

import pytest

from block_diffusion_drafter_dflash_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_drafter_dflash_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include "kernels.h"
int main() {
  for (int cls = 0; cls < 3; ++cls) {
    int prev = 0;
    for (int pages = 0; pages <= 20000; ++pages) {
      const int n = dfl::attention_chunks(pages, cls), cp = dfl::attention_chunk_pages(pages, cls);
      if (n < 1 || n < prev || (long)cp * n < pages || cp > 64) {
        std::printf("FAIL cls %d pages %d chunks %d (previous %d) of %d pages\n", cls, pages, n, prev, cp);
        return 1;
      }
      prev = n;
    }
    std::printf("cls %d: 2048 pages -> %d chunks, 4096 -> %d, 8192 -> %d\n", cls, dfl::attention_chunks(2048, cls),
                dfl::attention_chunks(4096, cls), dfl::attention_chunks(8192, cls));
  }
  return 0;
}
"""


def test_attention_chunking_is_monotone_and_bounded(tmp_path):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available")
    src = tmp_path / "rules.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "rules"
    subprocess.run([cc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    lines = out.stdout.strip().splitlines()
    assert len(lines) == 3, out.stdout
    # a single long stream in a narrow or mid batch: 64 chunks of 32 pages at 2048 pages
    assert lines[0].startswith("cls 0: 2048 pages -> 64 chunks") and lines[1].startswith("cls 1: 2048 pages -> 64 chunks")
