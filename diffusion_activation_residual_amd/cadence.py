"""The codec at model cadence: one grouped compress and one grouped decode per layer (its K and
V, which the sender has together once the layer's QKV projection is done), with the layers
spread round-robin over several streams so that one layer's launches overlap another's.

Patch parallelism exchanges each layer's K and V once per denoising step (paper: reproducibility
table, "Pseudocode", Algorithm 1: project QKV, all-gather K and V, attention).  Layer l's codec
work touches only layer l's states and payload buffers, so its compress and decode keep their
order on one stream while other layers' launches run beside them on other streams; each
launch's ramp-up and drain then overlap another launch's streaming.

Host logic only: every launch is a call of the C ABI through the binding."""
from . import cfz


def enqueue_layer_step(layers, senders, receivers, x, codes, scales, streams, xhat=None):
    """Enqueue one step: for layer l (a list of tensor indices, e.g. [2l, 2l + 1]) one grouped
    compress of x[i] for i in layers[l], then one grouped decode of the codes it wrote, both on
    streams[l % len(streams)].  The other streams first wait for streams[0] and streams[0]
    finally waits for all of them, so the whole step is ordered after work queued before it on
    streams[0] and before work queued after it.  Works eagerly and under torch.cuda.graph
    capture (streams[0] is then the capture stream).

    senders / receivers: cfz handles per tensor; x, codes, scales (and xhat, or None): device
    tensors per tensor index.  The tensors of different layers must not share buffers."""
    if not streams:
        raise ValueError("at least one stream")
    s0 = streams[0]
    for s in streams[1:]:
        s.wait_stream(s0)
    for l, c in enumerate(layers):
        st = streams[l % len(streams)]
        cfz.cfz_compress_group([senders[i] for i in c], [x[i] for i in c], [codes[i] for i in c],
                               [scales[i] for i in c], stream=st)
        cfz.cfz_decompress_group([receivers[i] for i in c], [codes[i] for i in c],
                                 [scales[i] for i in c],
                                 None if xhat is None else [xhat[i] for i in c], stream=st)
    for s in streams[1:]:
        s0.wait_stream(s)
