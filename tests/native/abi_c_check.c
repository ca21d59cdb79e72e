/* The C ABI used from plain C (no C++, no HIP headers): include/moe.h must
 * compile as C11, and the host-only entry points and the argument checks
 * (which reject bad calls before any HIP call) must work from C.
 * Prints "ok" and exits 0 on success; the first failure is printed. */
#include <stdio.h>
#include <string.h>

#include <stdint.h>

#include "moe.h"

static int fail(const char* what) {
  printf("FAIL: %s (last error: %s)\n", what, moe_last_error());
  return 1;
}

int main(void) {
  /* the 4K-context layer of one rank: 8192 tokens, 6144 -> 3072 latent, 384
     experts over 64 ranks, top-8, 3 waves, expert hidden 1536, 2 shared
     experts of hidden 1536, factors 1.10 and 1.15, the scratch of every wave
     held at once (live_waves 0) */
  moe_dims d = {8192, 6144, 3072, 384, 8, 64, 3, 1536, 2, 1536, 0, MOE_ACT_BF16, 110, 100, 115, 100, 0, 0};
  int64_t send_cap = 0, recv_cap = 0, stride = 0;
  if (moe_capacity(&d, &send_cap, &recv_cap, &stride) != MOE_OK) return fail("moe_capacity");
  /* ceil(1.10 * 8192 * 8 / 64) = 1127; ceil(1.15 * 64 * 8192 * 8 / 384) = 12562;
     a row is 6144 bytes of bf16 and the 4-byte id, padded to 128 bytes */
  if (send_cap != 1127 || recv_cap != 12562 || stride != 6272) return fail("capacities");
  size_t ws = 0;
  if (moe_workspace_size(&d, &ws) != MOE_OK || ws == 0 || ws % 256) return fail("moe_workspace_size");

  /* one live wave: one block of SwiGLU hidden rows (2 x 12562 x 1536 bf16)
     and one of partial tiles (256 tiles of 256 x 256 fp32) fewer per wave */
  moe_dims one = d;
  one.live_waves = 1;
  size_t ws1 = 0;
  if (moe_workspace_size(&one, &ws1) != MOE_OK) return fail("moe_workspace_size, one live wave");
  if (ws - ws1 != 2 * ((size_t)2 * 12562 * 1536 * 2 + (size_t)256 * 256 * 256 * 4))
    return fail("workspace of one live wave");
  one.live_waves = 4;
  if (moe_workspace_size(&one, &ws1) != MOE_EINVAL) return fail("live_waves > waves accepted");
  /* a ragged hidden-row bank of 20000 rows per wave instead of 2 x 12562 */
  moe_dims rag = d;
  rag.wave_rows = 20000;
  size_t ws2 = 0;
  if (moe_workspace_size(&rag, &ws2) != MOE_OK) return fail("moe_workspace_size, ragged banks");
  if (ws - ws2 != 3 * (size_t)(2 * 12562 - 20000) * 1536 * 2) return fail("workspace of ragged banks");
  rag.wave_rows = -1;
  if (moe_workspace_size(&rag, &ws2) != MOE_EINVAL) return fail("negative wave_rows accepted");
  /* the allocation-free packing refuses a batch over its scratch before any launch */
  moe_dims big = d;
  big.tokens = 600000;
  if (moe_pack_pools_noalloc(&big, NULL, NULL, NULL, 0, NULL, NULL, NULL) != MOE_EINVAL ||
      strstr(moe_last_error(), "scratch") == NULL)
    return fail("oversized allocation-free packing accepted");

  moe_dims bad = d;
  bad.n_experts = 385; /* not a multiple of the rank count */
  if (moe_capacity(&bad, NULL, NULL, NULL) != MOE_EINVAL || strlen(moe_last_error()) == 0)
    return fail("bad dims accepted");
  bad = d;
  bad.act_dtype = 7;
  if (moe_workspace_size(&bad, &ws) != MOE_EDTYPE) return fail("bad act_dtype accepted");
  /* a NULL input is refused before any launch */
  if (moe_route(&d, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL) != MOE_EINVAL)
    return fail("NULL input accepted");
  if (strstr(moe_last_error(), "NULL") == NULL) return fail("error message");

  /* dims fuzz: 1-3 fields of the layer above set to arbitrary int32 values
     (extremes included) from a fixed linear congruential sequence; the host
     code must answer with a documented code every time (and, under the
     sanitizers, without undefined behaviour such as a signed overflow) */
  {
    static const int32_t special[] = {INT32_MIN, -1, 0, 1, 2, 3, 7, 63, 64, 100, 1000, 4096, 65536,
                                      1 << 24, 1 << 30, INT32_MAX};
    const int nspecial = (int)(sizeof(special) / sizeof(special[0]));
    uint64_t lcg = 0x9e3779b97f4a7c15ull;
    int accepted = 0;
    for (int it = 0; it < 20000; ++it) {
      moe_dims f = d;
      int32_t* fields = (int32_t*)&f;
      const int nfields = (int)(sizeof(moe_dims) / sizeof(int32_t));
      lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
      const int nedit = 1 + (int)((lcg >> 60) % 3);
      for (int e = 0; e < nedit; ++e) {
        lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
        const int field = (int)((lcg >> 33) % (uint64_t)nfields);
        const int32_t v = (lcg >> 62) ? special[(lcg >> 40) % (uint64_t)nspecial] : (int32_t)((lcg >> 20) % 70000) - 3;
        fields[field] = v;
      }
      int64_t s = 0, r = 0, p = 0;
      size_t b = 0;
      const int rc = moe_capacity(&f, &s, &r, &p), rc2 = moe_workspace_size(&f, &b);
      if (rc != MOE_OK && rc != MOE_EINVAL && rc != MOE_EDTYPE) return fail("fuzz: moe_capacity code");
      if (rc2 != MOE_OK && rc2 != MOE_EINVAL && rc2 != MOE_EDTYPE) return fail("fuzz: moe_workspace_size code");
      if (rc == MOE_OK && (s <= 0 || r <= 0 || p <= 0 || p % 16)) {
        if (!(s == 0 && f.tokens == 0)) return fail("fuzz: accepted dims gave bad capacities");
      }
      /* no wrapped size: the workspace holds at least the 4-byte send rank of every assignment */
      if (rc2 == MOE_OK && b < (size_t)f.tokens * (size_t)f.top_k * 4u) return fail("fuzz: workspace size wrapped");
      if (rc == MOE_OK && rc2 == MOE_OK) ++accepted;
    }
    if (accepted == 0) return fail("fuzz: nothing accepted");
  }
  printf("ok send_cap=%lld recv_cap=%lld stride=%lld workspace=%zu\n", (long long)send_cap, (long long)recv_cap,
         (long long)stride, ws);
  return 0;
}
