// Sanitizer harness of the C ABI's host code (include/vsa.h): every
// validation error of vsa_plan, valid plans of each mask policy with their
// info and workspace regions, and the argument checks of the execution and
// getter entry points that end before any device access.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (see
// tests/test_abi_sanitized.py); exit status 0 when every expectation holds.
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/vsa.h"

static int g_fails = 0;

#define EXPECT(cond, ...)                      \
  do {                                         \
    if (!(cond)) {                             \
      std::fprintf(stderr, "FAIL: " __VA_ARGS__); \
      std::fprintf(stderr, "\n");              \
      ++g_fails;                               \
    }                                          \
  } while (0)

static vsa_problem problem() {
  vsa_problem p;
  std::memset(&p, 0, sizeof p);
  p.B = 1; p.H = 2; p.d = 128;
  p.grid[0] = 12; p.grid[1] = 16; p.grid[2] = 24;
  p.tile[0] = 6; p.tile[1] = 8; p.tile[2] = 8;
  p.n_cand = 2;
  const int c[2][3] = {{1, 16, 16}, {6, 4, 4}};
  for (int i = 0; i < 2; ++i)
    for (int a = 0; a < 3; ++a) p.cand_tile[i][a] = c[i][a];
  p.dtype = VSA_BF16;
  return p;
}

static vsa_mask_policy policy() {
  vsa_mask_policy m;
  std::memset(&m, 0, sizeof m);
  m.flags = VSA_WINDOW;
  m.win[0] = 3; m.win[1] = 3; m.win[2] = 5;
  m.win_mode = VSA_WIN_TRUNCATE;
  return m;
}

typedef void (*Mutate)(vsa_problem*, vsa_mask_policy*);

struct Case {
  const char* name;
  Mutate mutate;
  int want;
};

static const Case kCases[] = {
    {"B = 0", [](vsa_problem* p, vsa_mask_policy*) { p->B = 0; }, VSA_ERR_INVALID_ARG},
    {"H < 0", [](vsa_problem* p, vsa_mask_policy*) { p->H = -1; }, VSA_ERR_INVALID_ARG},
    {"grid 0", [](vsa_problem* p, vsa_mask_policy*) { p->grid[1] = 0; }, VSA_ERR_INVALID_ARG},
    {"dtype", [](vsa_problem* p, vsa_mask_policy*) { p->dtype = 7; }, VSA_ERR_UNSUPPORTED},
    {"d = 96", [](vsa_problem* p, vsa_mask_policy*) { p->d = 96; }, VSA_ERR_UNSUPPORTED},
    {"too many tokens", [](vsa_problem* p, vsa_mask_policy*) { p->grid[0] = p->grid[1] = p->grid[2] = 2048; },
     VSA_ERR_UNSUPPORTED},
    {"B*H > 65535", [](vsa_problem* p, vsa_mask_policy*) { p->B = 300; p->H = 300; }, VSA_ERR_UNSUPPORTED},
    {"unknown flag", [](vsa_problem*, vsa_mask_policy* m) { m->flags |= 0x1000u; }, VSA_ERR_INVALID_ARG},
    {"no flags", [](vsa_problem*, vsa_mask_policy* m) { m->flags = 0; }, VSA_ERR_INVALID_ARG},
    {"fine with window", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_FINE | VSA_WINDOW; },
     VSA_ERR_INVALID_ARG},
    {"topk and topk_frac", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_TOPK | VSA_TOPK_FRAC; },
     VSA_ERR_INVALID_ARG},
    {"sics alone", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_SICS_SELECT; }, VSA_ERR_INVALID_ARG},
    {"sics and profile",
     [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_WINDOW | VSA_SICS_SELECT | VSA_PROFILE_SELECT; },
     VSA_ERR_INVALID_ARG},
    {"profile without static mask", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_PROFILE_SELECT | VSA_TOPK; m->topk = 2; },
     VSA_ERR_INVALID_ARG},
    {"profile with top-p",
     [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_PROFILE_SELECT | VSA_WINDOW | VSA_TOPP; m->topp = 0.5; },
     VSA_ERR_UNSUPPORTED},
    {"profile_frac > 1", [](vsa_problem*, vsa_mask_policy* m) { m->profile_frac = 1.5; }, VSA_ERR_INVALID_ARG},
    {"negative scale", [](vsa_problem*, vsa_mask_policy* m) { m->scale = -1.0; }, VSA_ERR_INVALID_ARG},
    {"summarizer", [](vsa_problem*, vsa_mask_policy* m) { m->summarizer = 9; }, VSA_ERR_INVALID_ARG},
    {"negative sink", [](vsa_problem*, vsa_mask_policy* m) { m->sink = -2; }, VSA_ERR_INVALID_ARG},
    {"compute mode", [](vsa_problem*, vsa_mask_policy* m) { m->compute = 5; }, VSA_ERR_INVALID_ARG},
    {"fp8 with fine",
     [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_FINE; m->fine_group = 64; m->fine_keep = 0.1; m->compute = VSA_COMPUTE_FP8; },
     VSA_ERR_UNSUPPORTED},
    {"fine group 20", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_FINE; m->fine_group = 20; m->fine_keep = 0.1; },
     VSA_ERR_INVALID_ARG},
    {"fine keep 0", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_FINE; m->fine_group = 64; m->fine_keep = 0.0; },
     VSA_ERR_INVALID_ARG},
    {"fine sink", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_FINE; m->fine_group = 64; m->fine_keep = 0.1; m->sink = 1; },
     VSA_ERR_INVALID_ARG},
    {"fine groups*N", [](vsa_problem* p, vsa_mask_policy* m) { p->grid[0] = 64; p->grid[1] = 256; p->grid[2] = 256; m->flags = VSA_FINE; m->fine_group = 16; m->fine_keep = 0.1; },
     VSA_ERR_UNSUPPORTED},
    {"n_cand 0", [](vsa_problem* p, vsa_mask_policy* m) { p->n_cand = 0; m->flags = VSA_WINDOW | VSA_SICS_SELECT; },
     VSA_ERR_INVALID_ARG},
    {"n_cand 5", [](vsa_problem* p, vsa_mask_policy* m) { p->n_cand = 5; m->flags = VSA_WINDOW | VSA_SICS_SELECT; },
     VSA_ERR_INVALID_ARG},
    {"tile 0", [](vsa_problem* p, vsa_mask_policy*) { p->tile[2] = 0; }, VSA_ERR_INVALID_ARG},
    {"tile beyond grid", [](vsa_problem* p, vsa_mask_policy*) { p->tile[2] = 25; }, VSA_ERR_UNSUPPORTED},
    {"tile beyond 4096 tokens", [](vsa_problem* p, vsa_mask_policy*) { p->grid[0] = 64; p->tile[0] = 64; p->grid[1] = p->tile[1] = 16; p->grid[2] = 24; p->tile[2] = 8; },
     VSA_ERR_UNSUPPORTED},
    {"more than 4096 tiles", [](vsa_problem* p, vsa_mask_policy*) { p->grid[0] = 64; p->grid[1] = 64; p->grid[2] = 64; p->tile[0] = p->tile[1] = 1; p->tile[2] = 2; },
     VSA_ERR_UNSUPPORTED},
    {"topk 0", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_TOPK; m->topk = 0; }, VSA_ERR_INVALID_ARG},
    {"topk_frac 0", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_TOPK_FRAC; m->topk_frac = 0.0; },
     VSA_ERR_INVALID_ARG},
    {"topp > 1", [](vsa_problem*, vsa_mask_policy* m) { m->flags = VSA_TOPP; m->topp = 1.5; }, VSA_ERR_INVALID_ARG},
    {"win_mode", [](vsa_problem*, vsa_mask_policy* m) { m->win_mode = 4; }, VSA_ERR_INVALID_ARG},
    {"even window", [](vsa_problem*, vsa_mask_policy* m) { m->win[1] = 2; }, VSA_ERR_INVALID_ARG},
    {"zero window", [](vsa_problem*, vsa_mask_policy* m) { m->win[0] = 0; }, VSA_ERR_INVALID_ARG},
};

static void check_valid(const char* name, const vsa_problem& p, const vsa_mask_policy& m) {
  vsa_plan_t* plan = nullptr;
  const int st = vsa_plan(&p, &m, &plan);
  EXPECT(st == VSA_OK && plan, "%s: status %d (%s)", name, st, vsa_last_error());
  if (!plan) return;
  vsa_plan_info info;
  EXPECT(vsa_plan_get_info(plan, &info) == VSA_OK, "%s: info", name);
  size_t ws = 0;
  EXPECT(vsa_workspace_bytes(plan, &ws) == VSA_OK && ws > 0, "%s: workspace bytes", name);
  size_t end = 0;
  for (int r = 0; r < VSA_WS_NREGIONS; ++r) {
    size_t off = 0, n = 0;
    EXPECT(vsa_workspace_region(plan, r, &off, &n) == VSA_OK, "%s: region %d", name, r);
    EXPECT(off % 256 == 0, "%s: region %d offset %zu not 256-aligned", name, r, off);
    if (n) end = off + n > end ? off + n : end;
  }
  EXPECT(end <= ws, "%s: regions end at %zu beyond the workspace %zu", name, end, ws);
  size_t off, n;
  EXPECT(vsa_workspace_region(plan, VSA_WS_NREGIONS, &off, &n) == VSA_ERR_INVALID_ARG, "%s: bad region", name);
  EXPECT(vsa_workspace_region(plan, -1, &off, &n) == VSA_ERR_INVALID_ARG, "%s: negative region", name);

  // execution entry points: argument errors are reported before any device access
  alignas(256) static unsigned char buf[4096];
  void* a = buf;
  void* mis = buf + 8;
  EXPECT(vsa_forward(plan, a, a, a, a, nullptr, ws, nullptr) == VSA_ERR_INVALID_ARG, "%s: NULL workspace", name);
  EXPECT(vsa_forward(plan, a, a, a, a, mis, ws, nullptr) == VSA_ERR_INVALID_ARG, "%s: misaligned workspace", name);
  EXPECT(vsa_forward(plan, a, a, a, a, a, ws - 1, nullptr) == VSA_ERR_WORKSPACE_TOO_SMALL, "%s: small workspace", name);
  EXPECT(vsa_forward(plan, nullptr, a, a, a, a, ws, nullptr) == VSA_ERR_INVALID_ARG, "%s: NULL q", name);
  EXPECT(vsa_forward(plan, a, a, mis, a, a, ws, nullptr) == VSA_ERR_INVALID_ARG, "%s: misaligned v", name);
  EXPECT(vsa_forward_cached(plan, a, a, a, nullptr, a, ws, nullptr) == VSA_ERR_INVALID_ARG, "%s: cached NULL o", name);
  EXPECT(vsa_attend(plan, a, a, a, nullptr, a, ws, nullptr) == VSA_ERR_INVALID_ARG, "%s: attend NULL o", name);
  if (m.compute == VSA_COMPUTE_BF16 && !(m.flags & VSA_FINE))
    EXPECT(vsa_attend(plan, nullptr, a, a, a, a, ws, nullptr) == VSA_ERR_INVALID_ARG,
           "%s: bf16 attend without q (read in raster order)", name);
  EXPECT(vsa_untile(plan, 0, a, ws, a, nullptr) == VSA_ERR_UNSUPPORTED, "%s: untile of Q", name);
  EXPECT(vsa_layout(plan, a, nullptr, a, a, ws, nullptr) == VSA_ERR_INVALID_ARG, "%s: layout NULL k", name);
  EXPECT(vsa_untile(plan, 2, a, ws, a, nullptr) != VSA_OK, "%s: untile which = 2", name);
  int64_t kept = 0;
  EXPECT(vsa_read_selection(plan, a, ws, nullptr, nullptr, 0, &kept, nullptr, nullptr) != VSA_OK,
         "%s: read_selection NULL row_ptr", name);
  int64_t pairs = 0;
  EXPECT(vsa_retained_work(plan, a, ws, &pairs, nullptr, nullptr) == VSA_ERR_INVALID_ARG,
         "%s: retained_work NULL flops", name);
  if (ws > VSA_NOALLOC_BYTES)
    EXPECT(vsa_forward_noalloc(plan, a, a, a, a, nullptr) == VSA_ERR_UNSUPPORTED, "%s: noalloc refusal", name);
  vsa_plan_destroy(plan);
}

int main() {
  // every validation error
  for (const Case& c : kCases) {
    vsa_problem p = problem();
    vsa_mask_policy m = policy();
    c.mutate(&p, &m);
    vsa_plan_t* plan = reinterpret_cast<vsa_plan_t*>(0x1);
    const int st = vsa_plan(&p, &m, &plan);
    EXPECT(st == c.want, "%s: status %d, want %d (%s)", c.name, st, c.want, vsa_last_error());
    EXPECT(plan == nullptr, "%s: plan not cleared", c.name);
    EXPECT(std::strlen(vsa_last_error()) > 0, "%s: no error message", c.name);
    EXPECT(std::strcmp(vsa_status_string(st), "VSA_ERR_UNKNOWN") != 0, "%s: status string", c.name);
  }
  // NULL arguments
  vsa_problem p = problem();
  vsa_mask_policy m = policy();
  vsa_plan_t* plan = nullptr;
  EXPECT(vsa_plan(nullptr, &m, &plan) == VSA_ERR_INVALID_ARG, "NULL problem");
  EXPECT(vsa_plan(&p, nullptr, &plan) == VSA_ERR_INVALID_ARG, "NULL policy");
  EXPECT(vsa_plan(&p, &m, nullptr) == VSA_ERR_INVALID_ARG, "NULL out");
  EXPECT(vsa_plan_get_info(nullptr, nullptr) == VSA_ERR_INVALID_ARG, "NULL info");
  EXPECT(vsa_workspace_bytes(nullptr, nullptr) == VSA_ERR_INVALID_ARG, "NULL bytes");
  EXPECT(vsa_forward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == VSA_ERR_INVALID_ARG,
         "NULL plan");
  EXPECT(vsa_forward_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == VSA_ERR_INVALID_ARG,
         "noalloc NULL plan");
  vsa_plan_destroy(nullptr);
  EXPECT(std::strcmp(vsa_status_string(1234), "VSA_ERR_UNKNOWN") == 0, "unknown status string");

  // valid plans of every mask policy
  check_valid("window", p, m);
  m.win_mode = VSA_WIN_CLAMP;
  check_valid("clamp window", p, m);
  m = policy();
  m.flags = VSA_TOPK | VSA_WINDOW; m.topk = 3; m.summarizer = VSA_SUMM_MINMAX; m.sink = 2;
  check_valid("topk minmax sink", p, m);
  m = policy();
  m.flags = VSA_TOPP | VSA_WINDOW; m.topp = 0.9; m.compute = VSA_COMPUTE_FP8;
  check_valid("topp fp8", p, m);
  m = policy();
  m.flags = VSA_TOPK_FRAC | VSA_SICS_SELECT; m.topk_frac = 0.2;
  check_valid("sics", p, m);
  m = policy();
  m.flags = VSA_WINDOW | VSA_PROFILE_SELECT; m.win[0] = m.win[1] = m.win[2] = 1;
  check_valid("profile", p, m);
  m = policy();
  m.flags = VSA_DENSE;
  check_valid("dense", p, m);
  m = policy();
  m.flags = VSA_FINE; m.fine_group = 64; m.fine_keep = 0.15;
  check_valid("fine", p, m);
  vsa_problem big = problem();
  big.H = 24; big.grid[0] = 30; big.grid[1] = 48; big.grid[2] = 80;
  m = policy();
  check_valid("hunyuan window (beyond the no-alloc scratch)", big, m);

  std::printf("%d failures\n", g_fails);
  return g_fails != 0;
}
