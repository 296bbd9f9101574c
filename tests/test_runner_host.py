"""Host-side logic of the timed configuration (runner.py), on the CPU: how
many layers the steps cycle over, and the layer order inside the captured
graphs, which must bring every layer's double-buffered counts back to the
buffer the next replay reads."""
import collections

from long_context_decode_attn_amd import runner as R


def test_layers_cover_twice_the_infinity_cache():
    """At least 12 layers, enough that their steps' bytes are twice the
    256 MB Infinity Cache, and no more than that needs."""
    cache = 256 * 2 ** 20
    for step_bytes in (45_191_936, 18_450_000, 36_640_000, 118_660_000, 892_270_000, 1_000):
        L = R.layers_for(step_bytes)
        assert L >= 12 and L * step_bytes >= 2 * cache
        assert L == 12 or (L - 1) * step_bytes < 2 * cache
    assert R.layers_for(18_450_000) == 30 and R.layers_for(45_191_936) == 12


class _Orders(R.LayeredDecoder):
    """The order logic alone (no device state)."""
    def __init__(self, L):
        self.L, self.G = L, 2 * L


def test_graph_orders_step_every_layer_an_even_number_of_times():
    for L in (1, 2, 12, 29):
        d = _Orders(L)
        full = d.order(d.G)
        assert full == [g % L for g in range(2 * L)]
        assert all(c == 2 for c in collections.Counter(full).values())
        for n in range(1, 2 * L):
            tail = d.order(n)
            c = collections.Counter(tail)
            # each layer twice in a row; only the last one of an odd tail once
            assert all(tail[i] == i // 2 for i in range(n))
            odd = [layer for layer, k in c.items() if k % 2]
            assert odd == ([tail[-1]] if n % 2 else [])
