"""The Python binding's cross-tensor checks (CPU only).  The C ABI receives
bare pointers, so shapes, dtypes and devices that disagree are caught here,
before the library is reached: every case below raises ValueError while
`binding.lib` is replaced by a function that fails the test if called."""
import pytest
import torch

from gqa_flash_attention_prefill_amd import binding


@pytest.fixture(autouse=True)
def _no_library(monkeypatch):
    def fail():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(binding, "lib", fail)


F16, BF16, F32 = torch.float16, torch.bfloat16, torch.float32


def _t(*shape, dtype=F16):
    return torch.zeros(*shape, dtype=dtype)


def _dense(tokens=16, h_q=8, h_kv=2, d=64, batch=1, s_cap=64, dtype=F16):
    return dict(q=_t(tokens, h_q, d, dtype=dtype), k=_t(batch, h_kv, s_cap, d, dtype=dtype),
                v=_t(batch, h_kv, s_cap, d, dtype=dtype), out=_t(tokens, h_q, d, dtype=dtype),
                sink=_t(h_q, dtype=F32))


def _prefill(a, **kw):
    a = {**a, **kw}
    return binding.attn_prefill(a["q"], a["k"], a["v"], 0, -1, a["sink"], 0.125, a["out"])


def _varlen(a, cu=(0, 16), past=(0,), **kw):
    a = {**a, **kw}
    return binding.attn_prefill_varlen(a["q"], a["k"], a["v"], list(cu), list(past), -1,
                                       a["sink"], 0.125, a["out"], tile_log=a.get("log"))


def _split(a, cu=(0, 16), past=(0,), **kw):
    a = {**a, **kw}
    return binding.attn_prefill_split(a["q"], a["k"], a["v"], list(cu), list(past), -1,
                                      a["sink"], 0.125, a["out"], lse=a.get("lse"),
                                      n_split=2, workspace=a.get("ws"))


def _match(exc, text):
    assert text in str(exc.value), str(exc.value)


@pytest.mark.parametrize("change,text", [
    (dict(out=_t(16, 8, 32)), "q's shape"),
    (dict(out=_t(16, 8, 64, dtype=BF16)), "out dtype"),
    (dict(k=_t(1, 2, 64, 64, dtype=BF16)), "k / v dtypes"),
    (dict(v=_t(1, 2, 64, 64, dtype=BF16)), "k / v dtypes"),
    (dict(v=_t(1, 2, 32, 64)), "v ("),
    (dict(k=_t(1, 2, 64, 128), v=_t(1, 2, 64, 128)), "head dim"),
    (dict(k=_t(0, 2, 64, 64), v=_t(0, 2, 64, 64)), "sequence slots"),
    (dict(sink=_t(4, dtype=F32)), "head_sink has"),
    (dict(sink=_t(8, dtype=F16)), "float32"),
])
def test_attn_prefill_cross_checks(change, text):
    with pytest.raises(ValueError) as e:
        _prefill(_dense(), **change)
    _match(e, text)


def test_host_tensors_are_refused():
    with pytest.raises(ValueError) as e:
        _prefill(_dense())
    _match(e, "GPU tensor")
    with pytest.raises(ValueError) as e:
        _varlen(_dense())
    _match(e, "GPU tensor")


def test_varlen_cross_checks():
    a = _dense(tokens=30, batch=2)
    with pytest.raises(ValueError) as e:          # q rows vs cu_seqlens
        _varlen(a, cu=(0, 10, 20), past=(0, 0))
    _match(e, "cu_seqlens_q ends")
    with pytest.raises(ValueError) as e:          # three sequences, two cache slots
        _varlen(a, cu=(0, 10, 20, 30), past=(0, 0, 0))
    _match(e, "sequence slots")
    with pytest.raises(ValueError) as e:
        _varlen(a, cu=(0, 30), past=(0, 0))
    _match(e, "len(past_len) + 1")
    with pytest.raises(ValueError) as e:          # old record width
        _varlen(a, cu=(0, 10, 30), past=(0, 0), log=torch.zeros(8, 8, dtype=torch.int32))
    _match(e, "tile_log")


def test_split_cross_checks():
    a = _dense()
    with pytest.raises(ValueError) as e:
        _split(a, lse=_t(16, 4, dtype=F32))
    _match(e, "lse")
    with pytest.raises(ValueError) as e:
        _split(a, ws=_t(4, 16, dtype=F32)[:, ::2])
    _match(e, "workspace")
    with pytest.raises(ValueError) as e:          # host workspace
        _split(a, ws=_t(64, dtype=F32))
    _match(e, "GPU tensor")


def test_paged_cross_checks():
    q, out = _t(16, 8, 64), _t(16, 8, 64)
    kp, vp = _t(100, 2, 64), _t(100, 2, 64)
    idx = torch.zeros(40, dtype=torch.int32)

    def call(**kw):
        a = dict(q=q, k=kp, v=vp, idx=idx, indptr=[0, 50], out=out, sink=None)
        a.update(kw)
        return binding.attn_prefill_paged(a["q"], a["k"], a["v"], a["idx"], a["indptr"], [0, 16],
                                          [0], -1, a["sink"], 0.125, a["out"])
    with pytest.raises(ValueError) as e:          # 40 indices, indptr ends at 50
        call()
    _match(e, "kv_indices has")
    with pytest.raises(ValueError) as e:
        call(indptr=[0, 40], v=_t(100, 2, 32))
    _match(e, "v (")
    with pytest.raises(ValueError) as e:
        call(indptr=[0, 40], idx=torch.zeros(40, dtype=torch.int64))
    _match(e, "int32")
    with pytest.raises(ValueError) as e:
        call(indptr=[0, 40])
    _match(e, "GPU tensor")
