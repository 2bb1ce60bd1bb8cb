// Host-side entry points of the C ABI, for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer: configuration checks, the weight table and its
// digest, position ids and RoPE tables, row layouts, the flow-match
// schedule, safetensors validation of the files named on the command line,
// and the no-GPU error path.  Prints one line per check; exits non-zero on
// the first failed expectation (the sanitizers abort on their own findings).
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "zimg_dit.h"
#include "zimg_ops.h"

static int fails = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "FAILED: %s (line %d)\n", #cond, __LINE__);  \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

int main(int argc, char** argv) {
  zimg_dit_config c;
  zimg_dit_default_config(&c);
  EXPECT(zimg_dit_check_config(&c) == ZIMG_OK);
  EXPECT(zimg_dit_check_config(nullptr) == ZIMG_EINVAL);
  zimg_dit_config bad = c;
  bad.hidden = 3712;
  EXPECT(zimg_dit_check_config(&bad) != ZIMG_OK && std::strlen(zimg_last_error()) > 0);
  bad = c;
  bad.token_pad = 16;
  EXPECT(zimg_dit_check_config(&bad) == ZIMG_EUNSUPPORTED);

  int32_t n = 0;
  EXPECT(zimg_dit_manifest_size(&c, &n) == ZIMG_OK && n == 521);
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    const char* name = nullptr;
    int32_t nd = 0;
    int64_t shape[4];
    EXPECT(zimg_dit_manifest_entry(&c, i, &name, &nd, shape) == ZIMG_OK && name && nd >= 1 && nd <= 4);
    int64_t e = 1;
    for (int d = 0; d < nd; ++d) e *= shape[d];
    total += e;
  }
  EXPECT(total == 6154908736LL);
  EXPECT(zimg_dit_manifest_entry(&c, n, nullptr, nullptr, nullptr) != ZIMG_OK);
  char hex[65];
  EXPECT(zimg_dit_manifest_digest(&c, hex) == ZIMG_OK);
  EXPECT(std::string(hex) == "3a9216f208c1873b2cf06394411a53e1e95e10fae3b01dca0f7223556e47c354");
  std::printf("config, weight table, digest: ok\n");

  std::vector<int32_t> cap(512 * 3), img(64 * 64 * 3);
  EXPECT(zimg_position_ids(512, 64, 64, cap.data(), img.data()) == ZIMG_OK);
  EXPECT(cap[3 * 511] == 512 && img[0] == 513 && img[3 * (64 * 64 - 1) + 2] == 63);
  std::vector<int32_t> ids(img);
  ids.insert(ids.end(), cap.begin(), cap.end());
  const int64_t S = (int64_t)ids.size() / 3;
  std::vector<float> cs(S * 64), sn(S * 64);
  EXPECT(zimg_rope_tables(&c, ids.data(), S, cs.data(), sn.data()) == ZIMG_OK);
  for (int64_t i = 0; i < S * 64; ++i) EXPECT(std::fabs(cs[i] * cs[i] + sn[i] * sn[i] - 1.0f) < 1e-6f);
  std::printf("position ids, RoPE tables: ok\n");

  int32_t lens[3] = {1, 77, 33}, io[3], co[3], St = 0;
  EXPECT(zimg_row_layout(3, 600, lens, io, co, &St) == ZIMG_OK && io[1] == 608 && St == 3 * 608 + 16 + 80 + 48);
  int32_t nimg[3] = {120, 6, 17};
  EXPECT(zimg_row_layout_varsize(3, nimg, lens, io, co, &St) == ZIMG_OK && io[2] == 144);
  int32_t zero[1] = {0};
  EXPECT(zimg_row_layout(1, 16, zero, io, co, &St) == ZIMG_EINVAL);
  std::printf("row layouts: ok\n");

  for (int steps : {1, 2, 8, 28, 50}) {
    std::vector<double> sig(steps + 1), t(steps);
    EXPECT(zimg_flowmatch_schedule(steps, 3.0, sig.data(), t.data()) == ZIMG_OK);
    EXPECT(sig[0] == 1.0 && sig[steps] == 0.0 && t[0] == 0.0);
    for (int k = 0; k < steps; ++k) EXPECT(sig[k + 1] < sig[k]);
  }
  EXPECT(zimg_flowmatch_schedule(0, 3.0, nullptr, nullptr) == ZIMG_EINVAL);
  std::printf("flow-match schedule: ok\n");

  // safetensors files: argv[1] = the config kind ("tiny"), then pairs of
  // (expected code, path)
  if (argc > 1 && std::string(argv[1]) == "tiny") {
    zimg_dit_config t;
    zimg_dit_default_config(&t);
    t.hidden = 512;
    t.n_heads = 4;
    t.ffn = 1536;
    t.n_layers = 1;
    t.n_noise_refiner = 0;
    t.n_context_refiner = 0;
    t.max_image_tokens = 256;
    t.max_caption_tokens = 32;
    for (int i = 2; i + 1 < argc; i += 2) {
      const int want = std::atoi(argv[i]);
      const char* path = argv[i + 1];
      int32_t cnt = -1;
      const int rc = zimg_safetensors_check(&t, &path, 1, &cnt);
      if (rc != want) std::fprintf(stderr, "%s: code %d, expected %d (%s)\n", path, rc, want, zimg_last_error());
      EXPECT(rc == want);
    }
    std::printf("safetensors files: ok\n");
  }

  zimg_dit* h = nullptr;
  const int rc = zimg_dit_alloc(&c, nullptr, &h);
  EXPECT(h == nullptr || rc == ZIMG_OK);
  if (h) zimg_dit_destroy(h);
  std::printf("allocation path: rc %d\n", rc);
  std::printf(fails ? "host checks: %d FAILED\n" : "host checks: all passed\n", fails);
  return fails ? 1 : 0;
}
