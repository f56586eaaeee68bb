"""Host logic of the profile summaries: the kernel hash that ties counter
readings to the code they were taken on."""
from lsh_eviction_amd import profiling


def test_code_only_drops_comments_and_whitespace():
    src = 'int a = 1;   // note\n/* block\n comment */ const char* s = "x // y /* z */";\nchar c = \'/\';  int b;'
    assert profiling._code_only(src) == 'int a = 1; const char* s = "x // y /* z */"; char c = \'/\'; int b;'
    # a comment edit leaves the code text as it was; a code edit does not
    assert profiling._code_only(src.replace("note", "other words")) == profiling._code_only(src)
    assert profiling._code_only(src.replace("int b;", "int b = 2;")) != profiling._code_only(src)


def test_escaped_quotes_stay_inside_strings():
    src = 'const char* s = "a \\" // not a comment"; int x;  // a comment'
    assert profiling._code_only(src) == 'const char* s = "a \\" // not a comment"; int x;'


def test_kernel_hash_is_stable():
    h = profiling.kernel_source_hash()
    assert len(h) == 16 and h == profiling.kernel_source_hash()
