"""Host-side rule of the shared workspaces (CPU tensors; no GPU): a decoder
that captured graphs holds the workspaces those graphs point into, so a later,
larger call that replaces the shared workspace of a tag cannot free them."""
import torch

from block_diffusion_decoding_amd import ops
from block_diffusion_decoding_amd.decoder import BlockDecoder


class _Holder:
    device = torch.device("cpu")


def test_held_workspaces_survive_growth_of_the_shared_ones():
    need = {"host-test-attn": 1000, "host-test-lm": 5000}
    d = _Holder()
    BlockDecoder.hold_workspaces(d, need)
    ptr = {tag: t.data_ptr() for tag, t in d._held_ws.items()}
    assert all(d._held_ws[tag].numel() >= n for tag, n in need.items())
    for tag in need:
        assert ops.workspace(0, "cpu", tag).data_ptr() == ptr[tag]      # shared until something grows it
        grown = ops.workspace(need[tag] * 4, "cpu", tag)
        assert grown.data_ptr() != ptr[tag] and grown.numel() >= need[tag] * 4
    for tag, t in d._held_ws.items():                                     # still alive, still the same buffers
        assert t.data_ptr() == ptr[tag] and t.numel() >= need[tag]
        t.fill_(1)
