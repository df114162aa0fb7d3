// Host-side argument checks of every C-ABI entry point, for a build whose host
// code carries AddressSanitizer and UndefinedBehaviorSanitizer
// (test_abi_sanitizers.py compiles it together with the library's sources).
// Every call here is refused on the host before anything is launched, so no
// GPU is needed; the pointers are never dereferenced.  Prints one line per
// failed expectation and exits with their count.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "smcsd.h"

namespace {

int failures = 0;

void expect(int32_t got, int32_t want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d, want %d\n", what, got, want);
    failures++;
  }
}

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t)0x10000 + off); }
template <typename T>
T* fk(uintptr_t off = 0) {
  return static_cast<T*>(fake(off));
}

const float kNaN = std::numeric_limits<float>::quiet_NaN();
const float kInf = std::numeric_limits<float>::infinity();

struct Sd {
  int32_t dtype = SMCSD_BF16, B = 4, K = 2, V = 1000;
  float T = 1.0f;
  const void *tgt = fake(), *drf = fake();
  const int32_t *tok = fk<int32_t>(), *off = nullptr;
  const float* u = fk<float>();
  int64_t rows_d = 8;
  int32_t *na = fk<int32_t>(), *ft = fk<int32_t>();
  void* ws = fake();
  size_t wsb = size_t(1) << 30;
  int32_t call() const {
    return sd_verify(dtype, B, K, V, T, tgt, drf, tok, u, off, rows_d, na, ft, nullptr, ws, wsb, nullptr);
  }
};

struct Smc {
  int32_t dtype = SMCSD_BF16, P = 2, N = 8, K = 2, V = 1000, L = 0;
  float T = 1.0f, ess = 0.5f, beta = 1.0f;
  const void *tgt = fake(), *drf = fake();
  const int32_t* tok = fk<int32_t>();
  const float *ub = fk<float>(), *ur = fk<float>();
  float* lw = fk<float>();
  const int32_t* pti = nullptr;
  int32_t* pto = nullptr;
  void* ws = fake();
  size_t wsb = size_t(1) << 30;
  int32_t call() const {
    return smc_reweight_resample(dtype, P, N, K, V, T, ess, tgt, drf, tok, ub, ur, lw, pti, pto, L, fk<int32_t>(),
                                 fk<int32_t>(), fk<float>(), fk<int32_t>(), nullptr, ws, wsb, nullptr);
  }
  int32_t power() const {
    return smc_reweight_resample_power(dtype, P, N, K, V, T, beta, ess, tgt, drf, tok, ub, ur, lw, pti, pto, L,
                                       fk<int32_t>(), fk<int32_t>(), fk<float>(), fk<int32_t>(), nullptr, ws, wsb,
                                       nullptr);
  }
  int32_t noalloc() const {
    return smc_reweight_resample_noalloc(dtype, P, N, K, V, T, ess, tgt, drf, tok, ub, ur, lw, pti, pto, L,
                                         fk<int32_t>(), fk<int32_t>(), fk<float>(), fk<int32_t>(), nullptr, nullptr);
  }
};

struct Tree {
  int32_t dtype = SMCSD_BF16, B = 4, V = 1000;
  float T = 1.0f;
  const int32_t *noff = fk<int32_t>(), *par = fk<int32_t>(), *tok = fk<int32_t>(), *doff = fk<int32_t>();
  int64_t nodes = 28, rows_d = 12;
  const void *tgt = fake(), *drf = fake();
  const float* u = fk<float>();
  int32_t* ln = fk<int32_t>();
  void* ws = fake();
  size_t wsb = size_t(1) << 30;
  int32_t call() const {
    return tree_verify(dtype, B, V, T, noff, par, tok, nodes, tgt, doff, rows_d, drf, u, fk<int32_t>(), ln,
                       fk<int32_t>(), nullptr, ws, wsb, nullptr);
  }
};

#define CASE(type, field, value, want)  \
  do {                                  \
    type c;                             \
    c.field = value;                    \
    expect(c.call(), want, #type " " #field "=" #value); \
  } while (0)

void sd_cases() {
  CASE(Sd, dtype, 2, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, V, 1 << 20, SMCSD_ERR_UNSUPPORTED);
  CASE(Sd, V, 0, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, T, 0.0f, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, T, -1.0f, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, T, kNaN, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, T, kInf, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, B, -1, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, K, -1, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, rows_d, 7, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, rows_d, 9, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, tgt, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, u, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, drf, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, na, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Sd, ws, nullptr, SMCSD_ERR_WORKSPACE);
  CASE(Sd, wsb, 16, SMCSD_ERR_WORKSPACE);
  CASE(Sd, ws, fake(8), SMCSD_ERR_WORKSPACE);
  {
    Sd c;
    c.K = 300;
    c.rows_d = 1200;
    expect(c.call(), SMCSD_ERR_UNSUPPORTED, "Sd K above the largest");
  }
  {
    Sd c;
    c.off = fk<int32_t>();
    c.rows_d = 9;
    expect(c.call(), SMCSD_ERR_INVALID_ARG, "Sd CSR with more rows than B*K allows");
  }
  {
    Sd c;
    c.B = 0;
    c.rows_d = 0;
    c.tgt = c.drf = nullptr;
    expect(c.call(), SMCSD_OK, "Sd empty call");
  }
}

void smc_cases() {
  CASE(Smc, dtype, 5, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, N, 0, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, P, -1, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, T, 0.0f, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, ess, -0.1f, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, ess, kNaN, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, N, 2000, SMCSD_ERR_UNSUPPORTED);
  CASE(Smc, K, 257, SMCSD_ERR_UNSUPPORTED);
  CASE(Smc, lw, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, ur, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, L, -1, SMCSD_ERR_INVALID_ARG);
  CASE(Smc, ws, nullptr, SMCSD_ERR_WORKSPACE);
  CASE(Smc, wsb, 100, SMCSD_ERR_WORKSPACE);
  {
    Smc c;
    c.pti = fk<int32_t>();
    c.pto = fk<int32_t>(64);
    c.L = 4;
    expect(c.call(), SMCSD_ERR_INVALID_ARG, "Smc overlapping page tables");
    c.pto = nullptr;
    expect(c.call(), SMCSD_ERR_INVALID_ARG, "Smc page table without an output");
  }
  {
    Smc c;
    c.P = 0;
    c.tgt = nullptr;
    expect(c.call(), SMCSD_OK, "Smc empty call");
  }
  {
    Smc c;
    c.beta = 0.0f;
    expect(c.power(), SMCSD_ERR_INVALID_ARG, "Smc power beta 0");
    c.beta = kNaN;
    expect(c.power(), SMCSD_ERR_INVALID_ARG, "Smc power beta NaN");
    c.beta = 2.0f;
    c.ws = nullptr;
    expect(c.power(), SMCSD_ERR_WORKSPACE, "Smc power without workspace");
  }
  {
    Smc c;
    c.dtype = 5;
    expect(c.noalloc(), SMCSD_ERR_INVALID_ARG, "noalloc dtype");
    c.dtype = SMCSD_BF16;
    c.T = 0.0f;
    expect(c.noalloc(), SMCSD_ERR_INVALID_ARG, "noalloc temperature");
    c.T = 1.0f;
    c.P = 0;
    expect(c.noalloc(), SMCSD_OK, "noalloc empty call");
  }
}

void tree_cases() {
  CASE(Tree, dtype, 3, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, V, 1 << 20, SMCSD_ERR_UNSUPPORTED);
  CASE(Tree, V, 0, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, T, 0.0f, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, T, kNaN, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, B, -1, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, nodes, 3, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, nodes, 4 * 256 + 1, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, rows_d, -1, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, rows_d, 25, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, noff, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, par, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, tok, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, doff, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, u, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, ln, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, drf, nullptr, SMCSD_ERR_INVALID_ARG);
  CASE(Tree, ws, nullptr, SMCSD_ERR_WORKSPACE);
  CASE(Tree, wsb, 1000, SMCSD_ERR_WORKSPACE);
  CASE(Tree, ws, fake(4), SMCSD_ERR_WORKSPACE);
  {
    Tree c;
    c.B = 0;
    c.nodes = c.rows_d = 0;
    c.tgt = c.drf = nullptr;
    expect(c.call(), SMCSD_OK, "Tree empty call");
  }
}

void draft_and_pages_cases() {
  const auto draw = [](int32_t dtype, int32_t R, int32_t V, float T, void* ws, size_t wsb) {
    return draft_sample(dtype, R, V, T, fake(), fk<float>(), fk<int32_t>(), nullptr, ws, wsb, nullptr);
  };
  expect(draw(7, 4, 100, 1.0f, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "draft dtype");
  expect(draw(SMCSD_BF16, -1, 100, 1.0f, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "draft R");
  expect(draw(SMCSD_BF16, 4, 100, kInf, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "draft T");
  expect(draw(SMCSD_BF16, 4, 1 << 20, 1.0f, fake(), 1 << 30), SMCSD_ERR_UNSUPPORTED, "draft V");
  expect(draw(SMCSD_BF16, 4, 100, 1.0f, nullptr, 0), SMCSD_ERR_WORKSPACE, "draft workspace");
  expect(draw(SMCSD_BF16, 0, 100, 1.0f, nullptr, 0), SMCSD_OK, "draft empty call");

  const auto pacer = [](int32_t B, int32_t block, int32_t maxb, double t0, double rho, int32_t* offsets) {
    return pacer_lengths(B, block, maxb, t0, rho, fk<float>(), fk<int32_t>(), offsets, nullptr);
  };
  expect(pacer(-1, 4, 4, 0.5, 1.1, fk<int32_t>()), SMCSD_ERR_INVALID_ARG, "pacer B");
  expect(pacer(4, 0, 4, 0.5, 1.1, fk<int32_t>()), SMCSD_ERR_INVALID_ARG, "pacer block");
  expect(pacer(4, 4, 0, 0.5, 1.1, fk<int32_t>()), SMCSD_ERR_INVALID_ARG, "pacer max_blocks");
  expect(pacer(4, 4, 4, std::nan(""), 1.1, fk<int32_t>()), SMCSD_ERR_INVALID_ARG, "pacer t0");
  expect(pacer(4, 4, 4, 0.5, INFINITY, fk<int32_t>()), SMCSD_ERR_INVALID_ARG, "pacer rho");
  expect(pacer(1 << 20, 1 << 10, 1 << 10, 0.5, 1.1, fk<int32_t>()), SMCSD_ERR_INVALID_ARG, "pacer lengths overflow");
  expect(pacer(4, 4, 4, 0.5, 1.1, nullptr), SMCSD_ERR_INVALID_ARG, "pacer offsets");

  int32_t* I = fk<int32_t>();
  const auto append = [&](int32_t P, int32_t N, int32_t L, int32_t S, int32_t A, int64_t M, void* ws, size_t wsb) {
    return smc_pages_append(P, N, L, S, A, M, I, I, I, I, I, I, I, I, nullptr, ws, wsb, nullptr);
  };
  expect(append(-1, 4, 8, 16, 5, 1024, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "append P");
  expect(append(2, 0, 8, 16, 5, 1024, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "append N");
  expect(append(2, 4, 0, 16, 5, 1024, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "append L");
  expect(append(2, 4, 8, 0, 5, 1024, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "append page size");
  expect(append(2, 4, 8, 16, -1, 1024, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "append tokens");
  expect(append(2, 4, 8, 16, 5, int64_t(1) << 33, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "append pool size");
  expect(append(2, 4, 1 << 30, 1 << 10, 5, 1024, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "append row bytes");
  expect(append(2, 4, 8, 16, 5, 1024, nullptr, 0), SMCSD_ERR_WORKSPACE, "append workspace");
  expect(append(0, 4, 8, 16, 5, 1024, nullptr, 0), SMCSD_OK, "append empty call");
  const auto resample = [&](int32_t P, int32_t N, int32_t* len_in, int32_t* len_out, void* ws, size_t wsb) {
    return smc_pages_resample(P, N, 8, 16, 1024, I, I, len_in, len_out, I, I, I, nullptr, ws, wsb, nullptr);
  };
  expect(resample(2, 0, I, fk<int32_t>(4096), fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "resample N");
  expect(resample(2, 4, I, fk<int32_t>(4), fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "resample aliased lengths");
  expect(resample(2, 4, I, nullptr, fake(), 1 << 30), SMCSD_ERR_INVALID_ARG, "resample lengths out");
  expect(resample(2, 4, I, fk<int32_t>(4096), nullptr, 0), SMCSD_ERR_WORKSPACE, "resample workspace");
}

void size_and_misc_cases() {
  // workspace sizes: 0 for empty or invalid shapes, aligned and growing otherwise
  expect(sd_verify_workspace_bytes(SMCSD_BF16, 0, 4, 32768, 0) == 0, 1, "sd size empty");
  const size_t a = sd_verify_workspace_bytes(SMCSD_BF16, 64, 4, 32768, 256);
  const size_t b = sd_verify_workspace_bytes(SMCSD_BF16, 64, 4, SMCSD_MAX_V, 256);
  expect(a > 0 && b > a && a % SMCSD_WORKSPACE_ALIGN == 0, 1, "sd sizes");
  expect(smc_workspace_bytes(SMCSD_BF16, 0, 16, 4, 100) == 0, 1, "smc size empty");
  const size_t c = smc_workspace_bytes(SMCSD_BF16, 32, 64, 8, 151936);
  expect(c > 0 && c % SMCSD_WORKSPACE_ALIGN == 0, 1, "smc size");
  expect(smc_workspace_bytes(SMCSD_BF16, 1 << 20, SMCSD_MAX_N, SMCSD_MAX_K, SMCSD_MAX_V) > c, 1, "smc size large");
  expect(tree_verify_workspace_bytes(SMCSD_BF16, 0, 100, 0, 0) == 0, 1, "tree size empty");
  expect(tree_verify_workspace_bytes(SMCSD_BF16, 64, 32768, 64 * 15, 64 * 7) % SMCSD_WORKSPACE_ALIGN == 0, 1,
         "tree size");
  expect(draft_sample_workspace_bytes(SMCSD_BF16, 4096, SMCSD_MAX_V) > 0, 1, "draft size");
  expect(smc_pages_workspace_bytes(32, 64, 512, 1 << 20) > 0, 1, "pages size");
  expect(smc_pages_workspace_bytes(0, 0, 0, 0) == 0, 1, "pages size invalid");

  // measurement aids
  uint32_t* sink = fk<uint32_t>();
  expect(smcsd_read_ceiling(nullptr, 64, nullptr, 0, sink, nullptr, nullptr, nullptr), SMCSD_ERR_INVALID_ARG,
         "read ceiling NULL buffer");
  expect(smcsd_read_ceiling(fake(), 63, nullptr, 0, sink, nullptr, nullptr, nullptr), SMCSD_ERR_INVALID_ARG,
         "read ceiling odd size");
  expect(smcsd_read_ceiling(fake(8), 64, nullptr, 0, sink, nullptr, nullptr, nullptr), SMCSD_ERR_INVALID_ARG,
         "read ceiling alignment");
  uint64_t stamps[4] = {7, 7, 7, 7};
  expect(smcsd_phase_stamps(stamps, sizeof(stamps), 1), SMCSD_ERR_UNSUPPORTED, "phase stamps");
  expect(stamps[0] == 7 && stamps[3] == 7, 1, "phase stamps untouched");
  smcsd_time_next_call(nullptr, nullptr, nullptr, nullptr);

  // status strings and version
  expect(smcsd_abi_version(), SMCSD_ABI_VERSION, "abi version");
  for (int32_t s = -1; s <= 8; s++) expect(smcsd_status_string(s) != nullptr, 1, "status string");
  expect(std::strcmp(smcsd_status_string(SMCSD_OK), "SMCSD_OK"), 0, "status OK");
}

}  // namespace

int main() {
  sd_cases();
  smc_cases();
  tree_cases();
  draft_and_pages_cases();
  size_and_misc_cases();
  std::printf("host checks done, %d failed\n", failures);
  return failures;
}
