/* Plain-C use of the library's boundary (include/lynx.h), host-side calls only:
 * size queries and argument validation, which return before any launch.  Built and run
 * by tests/test_c_abi.py; prints "ok" and returns 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>

#include "lynx.h"

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      return 1;                                                            \
    }                                                                      \
  } while (0)

int main(void) {
  size_t a = 0, r = 0;
  CHECK(lynx_stream_sizes(256, 8, 128, 64, &a, &r) == LYNX_OK);
  CHECK(r == 256 * 8 * 128 / 2);
  CHECK(a == r + 4 * 8 * 128 * (2 + 2 * 4));
  CHECK(lynx_stream_sizes(256, 8, 128, 48, &a, &r) == LYNX_EINVAL);
  CHECK(lynx_strerror(LYNX_EALIGN)[0] != '\0');

  /* an aligned dummy address: never dereferenced, every call below fails validation first */
  void* dummy = (void*)(uintptr_t)0x10000;
  CHECK(lynx_encode(dummy, 4, 256, 8, 64, 64, 255.0f, LYNX_SEL_ANCHOR, dummy, dummy, NULL) == LYNX_EUNSUPPORTED);
  CHECK(lynx_encode(dummy, 4, 256, 8, 128, 64, 0.0f, LYNX_SEL_ANCHOR, dummy, dummy, NULL) == LYNX_EINVAL);
  CHECK(lynx_encode((void*)(uintptr_t)0x10008, 4, 256, 8, 128, 64, 255.0f, LYNX_SEL_ANCHOR, dummy, dummy, NULL) ==
        LYNX_EALIGN);
  CHECK(lynx_decode_full(dummy, dummy, 4, 256, 8, 128, 64, 255.0f, 7, dummy, NULL) == LYNX_EINVAL);

  size_t ws = lynx_attn_workspace_bytes(16, 32768, 64, 8, 128, 256, 64);
  CHECK(ws > 0);
  CHECK(lynx_attn_anchor(dummy, dummy, dummy, 16, 32768, 64, 8, 128, 256, 64, 255.0f, 0.0f, dummy, ws - 1,
                         LYNX_OUT_F32, dummy, NULL) == LYNX_ENOSPACE);
  size_t wv = lynx_attn_verify_workspace_bytes(16, 64, 32768, 64, 8, 128, 256, 64);
  CHECK(wv > 0);
  CHECK(lynx_attn_verify(dummy, dummy, dummy, dummy, dummy, 16, 64, 32768, 64, 8, 128, 256, 64, 255.0f, 0.0f, dummy,
                         wv - 1, LYNX_OUT_BF16, dummy, NULL, NULL) == LYNX_ENOSPACE);
  const int32_t* no_table = NULL;
  CHECK(lynx_attn_anchor_paged(dummy, dummy, dummy, 8, no_table, no_table, 2, 4, 16, 2, 128, 256, 64, 255.0f, 0.0f,
                               dummy, 0, LYNX_OUT_F32, dummy, NULL) == LYNX_EALIGN);
  CHECK(lynx_encode_to_host_staging_bytes(256, 256, 8, 128, 64) == 2 * 256 * (a + r));
  printf("ok\n");
  return 0;
}
