"""Host-side checks of the Python binding's stream handling (no GPU needed:
torch's stream classes are replaced by recorders)."""
import contextlib

import pytest


def test_wrappers_allocate_on_the_launch_stream(monkeypatch):
    """With a stream given, the allocating wrappers run inside
    torch.cuda.stream(<that stream>), so their outputs and workspace belong
    to the launch stream in torch's caching allocator; without one nothing
    changes (torch's current stream is the launch stream)."""
    import torch
    from megatron_tensor_transformer_04_amd import _binding
    seen = []

    class FakeStream:
        def __init__(self, handle):
            self.cuda_stream = handle

    @contextlib.contextmanager
    def fake_stream_ctx(s):
        seen.append(s.cuda_stream)
        yield

    monkeypatch.setattr(torch.cuda, "Stream", FakeStream, raising=False)
    monkeypatch.setattr(torch.cuda, "ExternalStream", FakeStream, raising=False)
    monkeypatch.setattr(torch.cuda, "stream", fake_stream_ctx, raising=False)
    with _binding._on_stream(None):
        pass
    assert seen == []
    with _binding._on_stream(0x1234):
        pass
    assert seen == [0x1234]
    with _binding._on_stream(FakeStream(0x99)):
        pass
    assert seen == [0x1234, 0x99]
    assert _binding._stream(FakeStream(0x77)) == 0x77 and _binding._stream(0x55) == 0x55


@pytest.mark.parametrize("name", ["fwd", "bwd", "bwd_recompute", "db2", "attn_fwd", "attn_bwd"])
def test_every_allocating_wrapper_uses_the_stream_context(name):
    """Each wrapper that allocates with torch does so inside _on_stream."""
    import inspect
    from megatron_tensor_transformer_04_amd import _binding
    src = inspect.getsource(getattr(_binding, name))
    body = src[src.index("with _on_stream(stream):"):]
    assert "torch.empty" in body and "torch.empty" not in src[:src.index("with _on_stream(stream):")]
