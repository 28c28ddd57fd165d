"""A decode step of a stack of LLaMA decoder layers, captured once as a HIP
graph and replayed per generated token.

Every kernel of the step is the library's (`w4a16_decode_layer` per layer);
this module only owns the step's device buffers and the graph.  The
position of every sequence advances on the device inside the graph, so
replays need no host work.
"""

import torch

from . import binding as B


class DecodeGraph:
    """Decode steps over `layers` (dicts as `binding.decode_layer` takes
    them) for B sequences whose next positions are `pos0` (int32, one per
    sequence).  A step starts from `embed` (fp16 [B, H D], the new tokens'
    embeddings, written by the caller before the step): the residual stream
    is set to it and x to zero, the layers run, and the positions advance by
    one.  After a step the last hidden state is residual + x (`hidden()`),
    and the layers' KV caches hold the new tokens.  The first `step()` runs
    eagerly (it also loads the kernels); the second captures the step as a
    graph and replays it; later ones replay."""

    def __init__(self, layers, pos0, max_len=None, eps=1e-6, rope_base=10000.0):
        kc = layers[0]["k_cache"]
        self.B, self.H, self.S, self.D = kc.shape
        self.I = layers[0]["gate_up"][0].shape[0] // 2
        self.layers = layers
        self.max_len = self.S if max_len is None else max_len
        self.eps, self.rope_base = eps, rope_base
        dev = kc.device
        hd = self.H * self.D
        self.embed = torch.zeros((self.B, hd), dtype=torch.float16, device=dev)
        self.residual = torch.zeros((self.B, hd), dtype=torch.float16, device=dev)
        self.x = torch.zeros((self.B, hd), dtype=torch.float16, device=dev)
        self.pos = torch.as_tensor(pos0, dtype=torch.int32).to(dev).contiguous()
        nbytes = B.decode_layer_workspace_size(self.B, self.H, self.D, self.I, self.S, self.max_len)
        if nbytes == 0:
            raise ValueError("unsupported decode shape")
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.graph = None
        self.steps = 0
        self.stream = torch.cuda.Stream(device=dev)

    def _enqueue(self):
        self.residual.copy_(self.embed)
        self.x.zero_()   # a fill kernel (no memset node in the graph)
        for layer in self.layers:
            B.decode_layer(layer, self.pos, self.residual, self.x, self.workspace, max_len=self.max_len,
                           eps=self.eps, rope_base=self.rope_base)
        self.pos.add_(1)

    def eager_step(self):
        """One step without the graph (on the current stream)."""
        self._enqueue()
        self.steps += 1

    def step(self):
        if self.steps == 0:
            self.eager_step()
            return
        if self.graph is None:
            torch.cuda.synchronize()
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph, stream=self.stream):
                self._enqueue()
        self.graph.replay()
        self.steps += 1

    def hidden(self):
        """The last layer's output added to the stream (fp32 on the device)."""
        return self.residual.float() + self.x.float()
