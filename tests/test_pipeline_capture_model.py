"""Host-side model of recording the two-stream pipeline into a graph (no GPU).

Recording ``stream.Pipeline.run`` into a HIP graph crashed the runtime inside
end-capture, so the library refuses it.  This test looks for a cause in our
own code: it replays the stream and event operations ``Pipeline.run`` issues
(with stand-ins for torch's streams, events and tensors) against the rules of
stream capture as CUDA documents them and HIP follows them:

* a stream joins a capture by waiting on an event recorded in it (a fork);
* work enqueued on a stream that has not joined would run eagerly, outside the
  graph;
* a capturing stream must not wait on an event recorded outside the capture;
* before the capture ends, the origin stream must wait on every joined
  stream's last captured work (a join), or end-capture fails as unjoined;
* no stream or event of the capture may be synchronised or queried.

The model records the operations only; nothing runs.  The pipeline's stage
calls are stand-ins that log the stream they are enqueued on.
"""
import contextlib

import pytest
import torch

from video_vae_causal_amd import stream


class Event:
    def __init__(self, *a, **k):
        self.captured = None      # (stream, op index) of the last record made inside the capture
        self.recorded_outside = False
        self.records_in_capture = 0

    def record(self, s=None):
        s = s if s is not None else Model.current
        Model.op(s, "record")
        if s.capturing:
            self.captured = (s, len(s.ops) - 1)
            self.records_in_capture += 1
        else:
            self.captured = None
            self.recorded_outside = True

    def query(self):
        Model.violation("event queried")

    def synchronize(self):
        Model.violation("event synchronised")


class Stream:
    def __init__(self, *a, **k):
        self.capturing = False
        self.ops = []
        self.joined_waits = []    # (event source stream, op index of the record) this stream waited on
        Model.streams.append(self)

    def wait_event(self, ev):
        if ev.captured is not None:
            src, idx = ev.captured
            if not self.capturing:
                self.capturing = True            # a fork: this stream joins the capture
                Model.joined.append(self)
            self.joined_waits.append((src, idx))
        elif self.capturing:
            Model.violation("a capturing stream waits on an event recorded outside the capture")
        Model.op(self, "wait")

    def wait_stream(self, other):
        Model.violation("wait_stream records a temporary event")

    def synchronize(self):
        Model.violation("stream synchronised")

    @property
    def cuda_stream(self):
        return id(self)


class Model:
    streams = []
    joined = []
    violations = []
    current = None

    @classmethod
    def reset(cls):
        cls.streams, cls.joined, cls.violations = [], [], []
        cls.current = Stream()
        cls.origin = cls.current

    @classmethod
    def op(cls, s, what):
        s.ops.append(what)

    @classmethod
    def violation(cls, what):
        cls.violations.append(what)

    @classmethod
    def kernel(cls, tag):
        s = cls.current
        if cls.origin.capturing and not s.capturing:
            cls.violation(f"{tag} enqueued on a stream outside the capture")
        cls.op(s, "kernel")


class Tensor:
    """Stand-in for a chunk tensor: record_stream is allocator bookkeeping."""

    def __init__(self):
        self.streams = set()

    def record_stream(self, s):
        self.streams.add(s)


class Stack:
    """Stand-in for a stack: ``n`` stages, each one enqueued call."""
    PIPELINE_SPLIT = 2

    def __init__(self, n):
        self.n = n

    def stages(self, x, y, buf):
        return [(lambda k=k: Model.kernel(f"stage {k}")) for k in range(self.n)]


@pytest.fixture
def model(monkeypatch):
    Model.reset()

    @contextlib.contextmanager
    def use(s):
        prev, Model.current = Model.current, s
        try:
            yield
        finally:
            Model.current = prev

    monkeypatch.setattr(torch.cuda, "Stream", Stream)
    monkeypatch.setattr(torch.cuda, "Event", Event)
    monkeypatch.setattr(torch.cuda, "stream", use)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda *a, **k: Model.current)
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    # Pipeline.run refuses to be recorded; the model looks past that refusal
    # to the operations it would record.
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: False)
    return Model


def joined_back(origin, s):
    """Whether the origin waited on an event recorded on s after s's last
    captured operation other than that record itself."""
    last_work = max(i for i, o in enumerate(s.ops) if o != "record")
    return any(src is s and idx > last_work for src, idx in origin.joined_waits)


@pytest.mark.parametrize("chunks,slots,stages,split", [(5, 3, 4, 2), (21, 3, 10, 5), (2, 3, 3, 1),
                                                       (7, 2, 11, 6)])
def test_pipeline_run_follows_the_capture_rules(model, chunks, slots, stages, split):
    stack = Stack(stages)
    pipe = stream.Pipeline(stack, split=split, slots=slots, device="cpu")
    xs, ys = [Tensor() for _ in range(chunks)], [Tensor() for _ in range(chunks)]
    pipe.run(xs, ys)                      # an eager pass first, as stream.capture requires
    assert not model.violations

    origin = Stream()                     # the stream stream.capture records on
    origin.capturing = True
    model.origin = origin
    for s in model.streams:
        if s is not origin:
            s.capturing = False
        s.ops.clear()
        s.joined_waits.clear()
    model.joined.clear()
    model.current = origin
    pipe.run(xs, ys)

    assert not model.violations, model.violations
    sa, sb = pipe.streams
    assert set(model.joined) == {sa, sb}                   # both streams forked from the origin
    for s in (sa, sb):
        assert joined_back(origin, s), "a forked stream is not joined back before end-capture"
    assert sa.ops.count("kernel") == chunks * split
    assert sb.ops.count("kernel") == chunks * (stages - split)
    # the per-chunk events are recorded once per chunk of their slot, so more
    # than once in one capture when chunks > slots (legal: a wait names the
    # event's latest record, and every wait above found one made inside the
    # capture)
    for k in range(slots):
        n_k = len(range(k, chunks, slots))
        assert pipe._ev_a[k].records_in_capture == n_k
        assert pipe._ev_b[k].records_in_capture == n_k


def _run_with(old, new):
    """Pipeline.run with one line changed (a planted mistake, host only)."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(stream.Pipeline.run))
    assert old in src
    ns = {}
    exec(src.replace(old, new), stream.__dict__, ns)
    return ns["run"]


@pytest.mark.parametrize("old,new", [
    # stream B is never joined back into the origin
    ("for ev, st in zip(self._ev_join, (sa, sb)):", "for ev, st in zip(self._ev_join[:1], (sa,)):"),
    # A waits on B's per-chunk event before B has recorded it in this capture
    ("if i >= self.slots:", "if i >= 0:"),
])
def test_the_model_catches_planted_mistakes(model, monkeypatch, old, new):
    """The model is not vacuous: a pipeline with either mistake fails it."""
    monkeypatch.setattr(stream.Pipeline, "run", _run_with(old, new))
    pipe = stream.Pipeline(Stack(4), split=2, slots=3, device="cpu")
    xs, ys = [Tensor() for _ in range(5)], [Tensor() for _ in range(5)]
    origin = Stream()
    origin.capturing = True
    model.origin = model.current = origin
    pipe.run(xs, ys)
    sa, sb = pipe.streams
    assert model.violations or not all(joined_back(origin, s) for s in (sa, sb))
