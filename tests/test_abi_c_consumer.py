"""The C ABI from a plain C99 program, on a machine without a GPU.

The header is meant for C callers, so this compiles a small C program against
include/llama_mi355x.h with gcc (-std=c99 -Wall -Wextra -Werror), with AddressSanitizer
and UndefinedBehaviorSanitizer on that host program, links it to the built library and
runs the calls that need no device: size queries, argument and shape validation at
init, the error message, and llama_free(NULL).
"""
import os
import shutil
import subprocess

import pytest

from llama_decoder_forward_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

C_SOURCE = r"""
#include <stdio.h>
#include <string.h>
#include "llama_mi355x.h"

static int failures = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); ++failures; } } while (0)

static llama_config tiny(void) {
    llama_config c;
    memset(&c, 0, sizeof c);
    c.dim = 64; c.n_layers = 2; c.n_heads = 4; c.n_kv_heads = 2; c.head_dim = 16;
    c.ffn_hidden = 192; c.vocab_size = 256; c.norm_eps = 1e-5f; c.rope_theta = 500000.0f;
    c.max_batch = 2; c.max_seq = 32; c.max_tokens = 64; c.dtype = LLAMA_F32;
    return c;
}

int main(void) {
    llama_config c = tiny();
    const size_t kv = llama_kv_cache_bytes(&c), ws = llama_workspace_bytes(&c);
    /* K and V: layers x batch x KV heads x positions (64-aligned) x head_dim x fp32 */
    EXPECT(kv == (size_t)2 * 2 * 2 * 2 * 64 * 16 * 4);
    EXPECT(ws > 0);
    EXPECT(llama_kv_cache_bytes(NULL) == 0);

    llama_config bad = tiny();
    bad.n_heads = 3;
    EXPECT(llama_workspace_bytes(&bad) == 0);
    bad = tiny();
    bad.dtype = (llama_dtype)7;
    EXPECT(llama_kv_cache_bytes(&bad) == 0);

    llama_model *m = (llama_model *)&c;  /* must be reset to NULL on failure */
    EXPECT(llama_init_weights(&c, NULL, NULL, 0, NULL, 0, &m) == LLAMA_ERR_INVALID_ARG);
    EXPECT(m == NULL);
    EXPECT(strlen(llama_last_error()) > 0);
    EXPECT(llama_init_weights(&c, NULL, NULL, 0, NULL, 0, NULL) == LLAMA_ERR_INVALID_ARG);

    /* a weights struct whose layer table has a NULL matrix */
    static char dummy[256] __attribute__((aligned(256)));
    llama_layer_weights layers[2];
    for (int l = 0; l < 2; ++l) {
        layers[l].attention_norm = dummy; layers[l].wq = dummy; layers[l].wk = dummy;
        layers[l].wv = dummy; layers[l].wo = dummy; layers[l].ffn_norm = dummy;
        layers[l].w1 = dummy; layers[l].w3 = dummy; layers[l].w2 = dummy;
    }
    layers[1].w2 = NULL;
    llama_weights w;
    w.tok_embeddings = dummy; w.layers = layers; w.norm = dummy; w.output = dummy;
    m = NULL;
    EXPECT(llama_init_weights(&c, &w, dummy, kv, dummy, ws, &m) == LLAMA_ERR_INVALID_ARG);
    EXPECT(m == NULL);
    EXPECT(strstr(llama_last_error(), "layer 1") != NULL);

    /* complete weights, but the cache and workspace sizes are one byte short */
    layers[1].w2 = dummy;
    EXPECT(llama_init_weights(&c, &w, dummy, kv - 1, dummy, ws, &m) == LLAMA_ERR_CAPACITY);
    EXPECT(llama_init_weights(&c, &w, dummy, kv, dummy, ws - 1, &m) == LLAMA_ERR_CAPACITY);
    EXPECT(m == NULL);

    bad = tiny();
    bad.head_dim = 15;
    EXPECT(llama_init_weights(&bad, &w, dummy, kv, dummy, ws, &m) == LLAMA_ERR_SHAPE);

    llama_free(NULL);
    printf("%s\n", failures ? "C consumer: failures" : "C consumer: ok");
    return failures != 0;
}
"""


def test_header_compiles_as_c99_and_validation_runs_from_c(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    if not os.path.exists(bd.LIB_PATH):
        from llama_decoder_forward_amd import build
        build.build()
    src = tmp_path / "consumer.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(bd.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-g",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-lllama_mi355x", f"-Wl,-rpath,{libdir}",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C consumer: ok" in r.stdout
