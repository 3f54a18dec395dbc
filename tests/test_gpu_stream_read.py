"""The streaming-read ceiling kernel (kvq_stream_read) reads every byte."""
import numpy as np
import pytest

from gpu_helpers import announce, dev, host

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")

MAGIC = 0x9E3779B9  # the fold value that makes the kernel write its sink


@pytest.mark.parametrize("nbytes,at", [(16, 0), (4096, 4080), (1 << 20, 777 * 16),
                                       (41943040, 41943040 - 16)])
def test_stream_read_touches_every_word(nbytes, at):
    """A buffer whose only non-zero 16-byte word folds to the magic value:
    the sink is written only if that word (anywhere in the buffer, the last
    one included) was read."""
    announce(f"stream_read bytes={nbytes} word={at}")
    words = np.zeros(nbytes // 4, np.uint32)
    words[at // 4] = MAGIC
    buf = dev(words.view(np.uint8))
    sink = kvq.stream_read(buf)
    assert int(host(sink)[0]) & 0xFFFFFFFF == MAGIC
    zero = dev(np.zeros(nbytes, np.uint8))
    assert int(host(kvq.stream_read(zero))[0]) == 0
