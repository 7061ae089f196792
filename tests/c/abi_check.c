/* The C ABI used from plain C99, with nothing but the public headers: sizes,
 * layouts, status strings and the host-side validation of every entry point
 * (each call below fails validation before anything is enqueued, so no GPU is
 * needed).  Prints one line per failed check; exit status = number of
 * failures. */
#include <stdio.h>
#include <string.h>

#include "moe_mi355x.h"
#include "moe_probe.h"
#include "moe_shared.h"

static int failures = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);         \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static moe_shape shape(int T, int H, int E, int k, int Im, int mu, moe_dtype dt) {
  moe_shape s;
  memset(&s, 0, sizeof s);
  s.T = T; s.H = H; s.E = E; s.k = k; s.Im = Im; s.micro_count = mu; s.dtype = dt; s.renormalize = 1;
  return s;
}

int main(void) {
  /* placeholder device pointers: never dereferenced, validation fails first */
  void* P = (void*)(size_t)4096;
  const moe_shape den = shape(4096, 4096, 64, 8, 1536, 1, MOE_BF16);
  const size_t R = (size_t)4096 * 8;

  /* workspace: layout in order, 256-byte aligned, y sized by MOE_Y_BYTES */
  moe_workspace_layout L;
  CHECK(moe_get_workspace_layout(&den, &L) == MOE_OK);
  CHECK(L.total == moe_workspace_size(&den));
  CHECK(L.logits < L.topk_ids && L.topk_ids < L.topk_w && L.topk_w < L.counts && L.counts < L.offsets);
  CHECK(L.offsets < L.perm && L.perm < L.inv && L.inv < L.h && L.h < L.y);
  CHECK(L.y % 256 == 0 && L.h % 256 == 0);
  CHECK(L.y - L.h >= R * 1536 * 2);
  CHECK(L.total - L.y >= MOE_Y_BYTES(MOE_BF16, R, 4096));
  CHECK(MOE_Y_BYTES(MOE_BF16, 3, 320) == 3u * 320 * 2 + 3u * 2); /* a partial last block */
  CHECK(MOE_Y_BYTES(MOE_F32, 3, 320) == 3u * 320 * 4);
  /* the micro split does not change the size; fp32 intermediates are wider */
  {
    const moe_shape two = shape(4096, 4096, 64, 8, 768, 2, MOE_BF16);
    const moe_shape f32 = shape(64, 256, 8, 2, 128, 1, MOE_F32), b16 = shape(64, 256, 8, 2, 128, 1, MOE_BF16);
    CHECK(moe_workspace_size(&two) == L.total);
    CHECK(moe_workspace_size(&f32) > moe_workspace_size(&b16));
  }

  /* status strings */
  CHECK(strncmp(moe_status_string(MOE_OK), "MOE_OK", 6) == 0);
  CHECK(strncmp(moe_status_string(MOE_ERR_INVALID_ARG), "MOE_ERR_INVALID_ARG", 19) == 0);
  CHECK(strncmp(moe_status_string(MOE_ERR_UNSUPPORTED), "MOE_ERR_UNSUPPORTED", 19) == 0);
  CHECK(strncmp(moe_status_string(MOE_ERR_WORKSPACE), "MOE_ERR_WORKSPACE", 17) == 0);
  CHECK(strncmp(moe_status_string(MOE_ERR_HIP), "MOE_ERR_HIP", 11) == 0);

  /* shape validation, through every entry point */
  {
    const moe_shape bad_k = shape(64, 256, 8, 9, 128, 1, MOE_BF16);   /* k > E */
    const moe_shape bad_h = shape(64, 200, 8, 2, 128, 1, MOE_BF16);   /* H % 64 != 0 */
    const moe_shape bad_e = shape(64, 256, 65, 2, 128, 1, MOE_BF16);  /* E > 64 */
    moe_shape bad_r = shape(64, 256, 8, 2, 128, 1, MOE_BF16);
    bad_r.renormalize = 2;
    CHECK(moe_workspace_size(&bad_k) == 0 && moe_workspace_size(&bad_h) == 0);
    CHECK(moe_route(&bad_k, P, P, NULL, P, P, P, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_route(&bad_r, P, P, NULL, P, P, P, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_permute(&bad_h, P, P, P, P, P, NULL, NULL, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_grouped_gemm_w13_swiglu(&bad_e, P, P, P, P, P, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_grouped_gemm_down(&bad_h, P, P, P, P, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_finalize(&bad_k, P, P, P, P, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_forward(&bad_h, P, P, NULL, P, P, P, P, (size_t)1 << 40, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_forward(NULL, P, P, NULL, P, P, P, P, (size_t)1 << 40, NULL) == MOE_ERR_INVALID_ARG);
  }
  /* pointers: null and misaligned inputs; a workspace that is too small */
  {
    const moe_shape s = shape(64, 256, 8, 2, 128, 1, MOE_BF16);
    void* mis = (void*)(size_t)(4096 + 4);
    const size_t need = moe_workspace_size(&s);
    CHECK(need > 0);
    CHECK(moe_forward(&s, NULL, P, NULL, P, P, P, P, need, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_forward(&s, mis, P, NULL, P, P, P, P, need, NULL) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_forward(&s, P, P, NULL, P, P, P, P, need - 1, NULL) == MOE_ERR_WORKSPACE);
    CHECK(moe_forward_noalloc(&den, P, P, NULL, P, P, P, NULL) == MOE_ERR_WORKSPACE); /* > the static scratch */
  }
  /* the shared expert's width */
  {
    const moe_shape s = shape(64, 4096, 8, 2, 128, 1, MOE_BF16);
    moe_shared_layout Ls;
    CHECK(moe_shared_workspace_size(&s, 48) == 0);                 /* Is % 32 != 0 */
    CHECK(moe_shared_workspace_size(&s, 96) > moe_workspace_size(&s));
    CHECK(moe_get_shared_workspace_layout(&s, 1536, &Ls) == MOE_OK);
    CHECK(Ls.hs == moe_workspace_size(&s) && Ls.ys > Ls.hs && Ls.total == moe_shared_workspace_size(&s, 1536));
    CHECK(moe_shared_ffn(&s, 0, P, P, P, P, P, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_forward_shared(&s, 48, P, P, NULL, P, P, P, P, P, P, (size_t)1 << 40, NULL) == MOE_ERR_UNSUPPORTED);
  }
  /* probes: the FLOP count is a host formula; a misaligned buffer is refused */
  CHECK(moe_probe_mfma_flops(1) == 256.0 * 8 * 8 * 32768);
  CHECK(moe_probe_read((void*)(size_t)(4096 + 4), 1024, P, NULL) == MOE_ERR_UNSUPPORTED);

  printf("%s: %d failed\n", failures ? "abi_check FAILED" : "abi_check ok", failures);
  return failures;
}
