"""The build's kernel resource report: the compiler's per-kernel remarks are
parsed into (kernel, fields), and a kernel with scratch fails the build."""

from kv_cache_vector_04_amd import build as B


def _remark(loc, body):
    return "%s: remark: %s [%s]" % (loc, body, B.REMARK)


def test_resource_remarks_parse_per_kernel():
    stderr = "\n".join([
        _remark("x.hip:1:1", "Function Name: _Z1kv"),
        "    1 | __global__ void k() {",
        "      | ^",
        _remark("x.hip:1:1", "    VGPRs: 100"),
        _remark("x.hip:1:1", "    ScratchSize [bytes/lane]: 0"),
        "x.hip:9:3: warning: something else",
        _remark("x.hip:2:1", "Function Name: _Z1jv"),
        _remark("x.hip:2:1", "    ScratchSize [bytes/lane]: 12"),
        _remark("x.hip:2:1", "    Occupancy [waves/SIMD]: 2"),
    ])
    res = B._resources(stderr)
    assert res == [("_Z1kv", {"VGPRs": "100", "ScratchSize [bytes/lane]": "0"}),
                   ("_Z1jv", {"ScratchSize [bytes/lane]": "12", "Occupancy [waves/SIMD]": "2"})]
    scratch = [n for n, r in res if r.get("ScratchSize [bytes/lane]", "0") != "0"]
    assert scratch == ["_Z1jv"]


def test_no_remarks_no_kernels():
    assert B._resources("plain warning text\nmore text") == []
