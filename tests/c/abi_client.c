/* A plain C99 caller of the library: it includes the public header as a C
 * translation unit and links libchipmunk.so, then exercises the parts of the
 * boundary that need no GPU: the version, source digest, kernel names and
 * workspace sizes, and the argument checks that return an error before any HIP
 * call.  Prints "ok" and exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "chipmunk.h"

static int failures = 0;

static void check(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAILED: %s (last error: %s)\n", what, chipmunk_last_error());
    ++failures;
  }
}

int main(int argc, char** argv) {
  const char* want_digest = argc > 1 ? argv[1] : NULL;
  check(chipmunk_abi_version() == CHIPMUNK_ABI_VERSION, "ABI version matches the header");
  const char* dig = chipmunk_source_digest();
  check(dig != NULL && strlen(dig) == 16, "source digest is 16 hex digits");
  if (want_digest) check(dig != NULL && strcmp(dig, want_digest) == 0, "source digest matches the sources");
  check(chipmunk_kernel_count() > 0, "the library names its kernels");
  for (int i = 0; i < chipmunk_kernel_count(); ++i)
    check(chipmunk_kernel_name(i) != NULL && chipmunk_kernel_name(i)[0] != '\0', "kernel name");

  /* A sparse MLP delta at the FLUX.1-dev shape needs a workspace; a dense one
   * of a bf16 layer does not. */
  check(chipmunk_workspace_bytes(CHIPMUNK_OP_SPARSE_MLP, 4352, 3072, 12288, 3686) > 0, "sparse MLP workspace");

  /* Argument checks: every one returns before any HIP call. */
  int32_t idx[4] = {0, 1, 2, 3};
  check(chipmunk_identify_topk(NULL, 1, 8, 2, idx, NULL, 0, NULL) == CHIPMUNK_E_NULLPTR, "top-k without scores");
  check(strlen(chipmunk_last_error()) > 0, "an error leaves a message");

  chipmunk_mlp mlp;
  memset(&mlp, 0, sizeof mlp);
  mlp.n = 256;
  mlp.d = 128;
  mlp.h = 512;
  check(chipmunk_sparse_mlp_delta(&mlp, NULL, NULL, 128, NULL, NULL, NULL, 0, NULL) == CHIPMUNK_E_NULLPTR,
        "sparse MLP delta on a layer without weights");
  check(chipmunk_sparse_mlp_delta(NULL, NULL, NULL, 0, NULL, NULL, NULL, 0, NULL) == CHIPMUNK_E_NULLPTR,
        "sparse MLP delta without a layer");

  chipmunk_attn att;
  memset(&att, 0, sizeof att);
  att.n = 300;
  att.heads = 2;
  att.head_dim = 64;
  att.scale = 0.125f;
  check(chipmunk_dense_step(CHIPMUNK_ATTN, &att, NULL, NULL, NULL, NULL, NULL, 0, NULL) != CHIPMUNK_OK,
        "dense attention step without buffers");

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
