/* A plain C client of libzshard: device memory from the HIP runtime's C API,
 * the step through include/zshard.h, and the CPU oracle (liboracle, its C
 * entry points) as the reference.  No Python and no PyTorch are involved.
 *
 * Cases (each compared bit for bit with the oracle):
 *   1. flat shard, n = 100,003, N = 3, step 7, weight decay 0.1, arrays
 *      starting 5 elements past an allocation (a peeled head);
 *   2. a list plan over three tensors (1, 5,000 and 70,001 parameters, each
 *      in its own allocations), run at steps 1 and 2;
 *   3. the one-shot list call on the same tensors at step 3;
 *   4. argument errors (N = 0, a NULL array) return their statuses before
 *      anything is enqueued; the write-window setting and its query;
 *   5. the two-pass form with global-norm clipping active (70,001 parameters,
 *      a peeled head): the mean gradient, the norm (to 1e-12 relative, as
 *      the order of the double sum is the kernel's) and the clipped step;
 *   6. the device loss scaler over a sequence of finite, Inf and NaN norms;
 *   7. the optimizer-offload step (fp32 state in host memory, 13 chunks).
 * Prints "zs_c_client ok" and exits 0 on success, 1 on any mismatch or error.
 * Test code: the inputs come from a small generator of its own. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zshard.h"

/* the oracle's C entry points (oracle/oracle.cpp) */
typedef struct oracle_hp {
  double lr, beta1, beta2, eps, weight_decay;
} oracle_hp;
int oracle_reduce_adam(const uint16_t* const* G, int32_t N, int64_t n, float* P, float* M, float* V, uint16_t* B,
                       const oracle_hp* hp, int64_t t, int32_t threads);
int oracle_reduce_unscale(const uint16_t* const* G, int32_t N, int64_t n, int32_t fmt, double loss_scale, float* gbar,
                          int32_t threads);
double oracle_sqnorm(const float* gbar, int64_t n);
int oracle_adam_from_gbar(const float* gbar, int64_t n, float* P, float* M, float* V, uint16_t* B, int32_t out_fmt,
                          const oracle_hp* hp, int64_t t, double total_sq, double max_norm, int32_t skip_nonfinite,
                          int32_t threads);
typedef struct oracle_scaler {
  double scale, min_scale;
  int64_t window, hysteresis, overflows, clean;
} oracle_scaler;
int oracle_scaler_update(oracle_scaler* s, int32_t overflow);

#define CHECK_HIP(x)                                                              \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

#define CHECK_ZS(x)                                                                               \
  do {                                                                                            \
    zs_status s_ = (x);                                                                           \
    if (s_ != ZS_OK) {                                                                            \
      fprintf(stderr, "%s:%d: %s: %s (%s)\n", __FILE__, __LINE__, #x, zs_status_string(s_), zs_last_error()); \
      exit(1);                                                                                    \
    }                                                                                             \
  } while (0)

/* input generator: SplitMix64 -> uniform in [-1, 1) */
static uint64_t g_state = 0x5EEDull;
static double uniform(void) {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static uint16_t bf16_bits(float x) { /* input preparation: the upper half of the fp32 bits */
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

/* One shard's host inputs and its device copies. */
typedef struct {
  int64_t n;
  int32_t N;
  uint16_t** hg;   /* N host gradient arrays */
  float *hp, *hm, *hv;
  uint16_t** dg;   /* N device gradient pointers (into allocations with `pad` leading elements) */
  float *dp, *dm, *dv;
  uint16_t* db;
  void* allocs[32];
  int nalloc;
} shard;

static void* dalloc(shard* s, size_t bytes) {
  void* p = NULL;
  CHECK_HIP(hipMalloc(&p, bytes));
  s->allocs[s->nalloc++] = p;
  return p;
}

static void shard_init(shard* s, int64_t n, int32_t N, int64_t pad) {
  memset(s, 0, sizeof *s);
  s->n = n;
  s->N = N;
  s->hg = (uint16_t**)calloc((size_t)N, sizeof(uint16_t*));
  s->dg = (uint16_t**)calloc((size_t)N, sizeof(uint16_t*));
  s->hp = (float*)malloc((size_t)n * 4);
  s->hm = (float*)malloc((size_t)n * 4);
  s->hv = (float*)malloc((size_t)n * 4);
  for (int32_t r = 0; r < N; ++r) {
    s->hg[r] = (uint16_t*)malloc((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i) s->hg[r][i] = bf16_bits((float)(uniform() * 2e-3));
  }
  for (int64_t i = 0; i < n; ++i) {
    s->hp[i] = (float)(uniform() * 0.04);
    s->hm[i] = (float)(uniform() * 1e-4);
    s->hv[i] = (float)((uniform() + 1.0) * 1e-6);
  }
  for (int32_t r = 0; r < N; ++r) {
    s->dg[r] = (uint16_t*)dalloc(s, (size_t)(n + pad) * 2) + pad;
    CHECK_HIP(hipMemcpy(s->dg[r], s->hg[r], (size_t)n * 2, hipMemcpyHostToDevice));
  }
  s->dp = (float*)dalloc(s, (size_t)(n + pad) * 4) + pad;
  s->dm = (float*)dalloc(s, (size_t)(n + pad) * 4) + pad;
  s->dv = (float*)dalloc(s, (size_t)(n + pad) * 4) + pad;
  s->db = (uint16_t*)dalloc(s, (size_t)(n + pad) * 2) + pad;
  CHECK_HIP(hipMemcpy(s->dp, s->hp, (size_t)n * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(s->dm, s->hm, (size_t)n * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(s->dv, s->hv, (size_t)n * 4, hipMemcpyHostToDevice));
}

static void shard_free(shard* s) {
  for (int k = 0; k < s->nalloc; ++k) CHECK_HIP(hipFree(s->allocs[k]));
  for (int32_t r = 0; r < s->N; ++r) free(s->hg[r]);
  free(s->hg);
  free(s->dg);
  free(s->hp);
  free(s->hm);
  free(s->hv);
}

/* Advances the host copy with the oracle at step t and compares the device state with it, bit for bit. */
static int oracle_compare(shard* s, const zs_adam_hp* hp, int64_t t, const char* what) {
  const int64_t n = s->n;
  uint16_t* hb = (uint16_t*)malloc((size_t)n * 2);
  oracle_hp oh = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  if (oracle_reduce_adam((const uint16_t* const*)s->hg, s->N, n, s->hp, s->hm, s->hv, hb, &oh, t, 4) != 0) {
    fprintf(stderr, "%s: oracle rejected its arguments\n", what);
    return 1;
  }
  float* gp = (float*)malloc((size_t)n * 4);
  float* gm = (float*)malloc((size_t)n * 4);
  float* gv = (float*)malloc((size_t)n * 4);
  uint16_t* gb = (uint16_t*)malloc((size_t)n * 2);
  CHECK_HIP(hipMemcpy(gp, s->dp, (size_t)n * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(gm, s->dm, (size_t)n * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(gv, s->dv, (size_t)n * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(gb, s->db, (size_t)n * 2, hipMemcpyDeviceToHost));
  int bad = memcmp(gp, s->hp, (size_t)n * 4) || memcmp(gm, s->hm, (size_t)n * 4) ||
            memcmp(gv, s->hv, (size_t)n * 4) || memcmp(gb, hb, (size_t)n * 2);
  if (bad) fprintf(stderr, "%s: device state differs from the oracle\n", what);
  free(gp);
  free(gm);
  free(gv);
  free(gb);
  free(hb);
  return bad;
}

int main(void) {
  int bad = 0;
  if (zs_abi_version() != ZS_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", zs_abi_version(), ZS_ABI_VERSION);
    return 1;
  }
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  zs_adam_hp hp = {1e-3, 0.9, 0.999, 1e-8, 0.1};

  /* 1. flat shard with a peeled head */
  shard f;
  shard_init(&f, 100003, 3, 5);
  CHECK_ZS(zs_reduce_adam_flat((const uint16_t* const*)f.dg, f.N, f.n, f.dp, f.dm, f.dv, f.db, &hp, 7, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  bad |= oracle_compare(&f, &hp, 7, "flat");

  /* 1b. a flat shard in consecutive launches of one tile each, then the default limit again */
  {
    shard g;
    shard_init(&g, 20011, 5, 3);
    CHECK_ZS(zs_set_launch_bytes(1));
    CHECK_ZS(zs_reduce_adam_flat((const uint16_t* const*)g.dg, g.N, g.n, g.dp, g.dm, g.dv, g.db, &hp, 4, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    bad |= oracle_compare(&g, &hp, 4, "flat, one tile per launch");
    CHECK_ZS(zs_set_launch_bytes(0));
    if (zs_launch_bytes() != 3000000000LL || zs_set_launch_bytes(-1) != ZS_ERR_RANGE) {
      fprintf(stderr, "launch byte limit: default %lld, or a negative limit accepted\n", (long long)zs_launch_bytes());
      bad = 1;
    }
    shard_free(&g);
  }

  /* 4. argument errors, before anything is enqueued */
  if (zs_reduce_adam_flat((const uint16_t* const*)f.dg, 0, f.n, f.dp, f.dm, f.dv, f.db, &hp, 8, stream) !=
      ZS_ERR_RANGE) {
    fprintf(stderr, "N = 0 was not rejected\n");
    bad = 1;
  }
  if (zs_reduce_adam_flat((const uint16_t* const*)f.dg, f.N, f.n, NULL, f.dm, f.dv, f.db, &hp, 8, stream) !=
      ZS_ERR_NULL) {
    fprintf(stderr, "a NULL master was not rejected\n");
    bad = 1;
  }
  shard_free(&f);

  /* 4b. the write-window and schedule settings and their queries, from C (no GPU work) */
  {
    int32_t per = -1, open = -1, sched = -1;
    CHECK_ZS(zs_write_window(ZS_WINDOW_LIST_PLAN, 64, (int64_t)1 << 30, &per, &open));
    if (per != 0 || open != 0) {
      fprintf(stderr, "list plans of N = 64 take the phased schedule, but the query gives %d / %d\n", per, open);
      bad = 1;
    }
    CHECK_ZS(zs_flat_schedule(64, (int64_t)1 << 30, &sched));
    if (sched != ZS_SCHEDULE_PHASED) {
      fprintf(stderr, "default flat schedule for N = 64 on 2^30 parameters: %d\n", sched);
      bad = 1;
    }
    {
      /* 64 tensors of 2^24 parameters in arenas on 2 MiB boundaries: addresses that only stand for their
         alignment (the query reads none of them) */
      enum { LT = 64, LN = 32 };
      const uintptr_t base = (uintptr_t)1 << 40, span = (uintptr_t)1 << 32;
      static const uint16_t* lg[LT][LN];
      static zs_tensor lt[LT];
      for (int t = 0; t < LT; ++t) {
        const uintptr_t o = (uintptr_t)t << 24;
        for (int r = 0; r < LN; ++r) lg[t][r] = (const uint16_t*)(base + (4 + (uintptr_t)r) * span + 2 * o);
        lt[t].n = (int64_t)1 << 24;
        lt[t].master = (float*)(base + 4 * o);
        lt[t].m = (float*)(base + span + 4 * o);
        lt[t].v = (float*)(base + 2 * span + 4 * o);
        lt[t].param_bf16 = (uint16_t*)(base + 3 * span + 2 * o);
        lt[t].grad_chunks = lg[t];
      }
      CHECK_ZS(zs_list_schedule(lt, LT, 24, &sched));
      if (sched != ZS_SCHEDULE_STREAM) {
        fprintf(stderr, "default list schedule for N = 24 on 2^30 parameters: %d\n", sched);
        bad = 1;
      }
      CHECK_ZS(zs_list_schedule(lt, LT, 32, &sched));
      if (sched != ZS_SCHEDULE_PHASED) {
        fprintf(stderr, "default list schedule for N = 32 on 2^30 parameters: %d\n", sched);
        bad = 1;
      }
    }
    CHECK_ZS(zs_set_flat_schedule(ZS_SCHEDULE_WINDOWED));
    CHECK_ZS(zs_write_window(ZS_WINDOW_FLAT_STEP, 64, (int64_t)1 << 30, &per, &open));
    if (per != 4096 || open != 512) {
      fprintf(stderr, "flat window on the windowed schedule for N = 64: %d / %d\n", per, open);
      bad = 1;
    }
    CHECK_ZS(zs_write_window(ZS_WINDOW_LIST_PLAN, 64, (int64_t)1 << 30, &per, &open));
    if (per != 4096 || open != 512) {
      fprintf(stderr, "list-plan window on the windowed schedule for N = 64: %d / %d\n", per, open);
      bad = 1;
    }
    CHECK_ZS(zs_set_flat_schedule(ZS_SCHEDULE_AUTO));
    if (zs_set_flat_schedule(7) != ZS_ERR_RANGE) {
      fprintf(stderr, "an unknown schedule was not rejected\n");
      bad = 1;
    }
    CHECK_ZS(zs_set_write_window(1, 0));
    CHECK_ZS(zs_write_window(ZS_WINDOW_REDUCE_PASS, 64, (int64_t)1 << 30, &per, &open));
    if (per != 0 || open != 0) {
      fprintf(stderr, "windows switched off, but the query gives %d / %d\n", per, open);
      bad = 1;
    }
    if (zs_set_write_window(100, 10) != ZS_ERR_RANGE) {
      fprintf(stderr, "a period that is not a power of two was not rejected\n");
      bad = 1;
    }
    CHECK_ZS(zs_set_write_window(0, 0));
  }

  /* 2. and 3. a ragged list */
  const int64_t sizes[3] = {1, 5000, 70001};
  shard ts[3];
  zs_tensor tab[3];
  for (int k = 0; k < 3; ++k) {
    shard_init(&ts[k], sizes[k], 3, 0);
    tab[k].n = ts[k].n;
    tab[k].master = ts[k].dp;
    tab[k].m = ts[k].dm;
    tab[k].v = ts[k].dv;
    tab[k].param_bf16 = ts[k].db;
    tab[k].grad_chunks = (const uint16_t* const*)ts[k].dg;
  }
  zs_list_plan_t plan = NULL;
  CHECK_ZS(zs_list_plan_create(tab, 3, 3, stream, &plan));
  for (int64_t t = 1; t <= 2; ++t) {
    CHECK_ZS(zs_reduce_adam_list_plan(plan, &hp, t, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    for (int k = 0; k < 3; ++k) bad |= oracle_compare(&ts[k], &hp, t, "list plan");
  }
  zs_list_plan_destroy(plan);
  CHECK_ZS(zs_reduce_adam_list(tab, 3, 3, &hp, 3, stream));
  for (int k = 0; k < 3; ++k) bad |= oracle_compare(&ts[k], &hp, 3, "one-shot list");
  for (int k = 0; k < 3; ++k) shard_free(&ts[k]);

  /* 5. two-pass form with clipping */
  {
    shard s;
    shard_init(&s, 70001, 3, 3);
    const int64_t n = s.n;
    const size_t wsb = zs_two_pass_workspace_bytes(n);
    void* ws = dalloc(&s, wsb);
    double* dsq = (double*)dalloc(&s, 8);
    CHECK_ZS(zs_reduce_grads_flat((const uint16_t* const*)s.dg, s.N, n, ZS_FORMAT_BF16, 1.0, ws, wsb, dsq, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    double sq = 0;
    CHECK_HIP(hipMemcpy(&sq, dsq, 8, hipMemcpyDeviceToHost));
    float* gref = (float*)malloc((size_t)n * 4);
    float* gdev = (float*)malloc((size_t)n * 4);
    oracle_reduce_unscale((const uint16_t* const*)s.hg, s.N, n, 0, 1.0, gref, 4);
    const uintptr_t g0 = ((uintptr_t)ws + 255) & ~(uintptr_t)255;  /* the mean gradient's place in the workspace */
    CHECK_HIP(hipMemcpy(gdev, (void*)g0, (size_t)n * 4, hipMemcpyDeviceToHost));
    if (memcmp(gdev, gref, (size_t)n * 4)) { fprintf(stderr, "two-pass: mean gradient differs\n"); bad = 1; }
    const double sref = oracle_sqnorm(gref, n);
    if (!(sq == sq) || (sq > sref ? sq - sref : sref - sq) > 1e-12 * sref) {
      fprintf(stderr, "two-pass: norm %.17g against %.17g\n", sq, sref);
      bad = 1;
    }
    const double max_norm = 0.5 * __builtin_sqrt(sref);  /* clipping active: coefficient about 1/2 */
    CHECK_ZS(zs_adam_from_grads_flat(ws, wsb, n, s.dp, s.dm, s.dv, s.db, ZS_FORMAT_BF16, &hp, 11, dsq, max_norm, 1,
                                     stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    uint16_t* hb = (uint16_t*)malloc((size_t)n * 2);
    oracle_hp oh = {hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay};
    if (oracle_adam_from_gbar(gref, n, s.hp, s.hm, s.hv, hb, 0, &oh, 11, sq, max_norm, 1, 4) != 0) {
      fprintf(stderr, "two-pass: the oracle skipped or rejected the step\n");
      bad = 1;
    }
    float* gp = (float*)malloc((size_t)n * 4);
    uint16_t* gb = (uint16_t*)malloc((size_t)n * 2);
    CHECK_HIP(hipMemcpy(gp, s.dp, (size_t)n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gb, s.db, (size_t)n * 2, hipMemcpyDeviceToHost));
    if (memcmp(gp, s.hp, (size_t)n * 4) || memcmp(gb, hb, (size_t)n * 2)) {
      fprintf(stderr, "two-pass: clipped step differs from the oracle\n");
      bad = 1;
    }
    free(gref); free(gdev); free(hb); free(gp); free(gb);
    shard_free(&s);
  }

  /* 6. device loss scaler */
  {
    zs_loss_scaler host;
    CHECK_ZS(zs_loss_scaler_init(&host, 65536.0, 1.0, 3, 2));
    oracle_scaler ref = {65536.0, 1.0, 3, 2, 0, 0};
    zs_loss_scaler* dstate = NULL;
    double* dsq = NULL;
    int32_t* dtaken = NULL;
    CHECK_HIP(hipMalloc((void**)&dstate, sizeof host));
    CHECK_HIP(hipMalloc((void**)&dsq, 8));
    CHECK_HIP(hipMalloc((void**)&dtaken, 4));
    CHECK_HIP(hipMemcpy(dstate, &host, sizeof host, hipMemcpyHostToDevice));
    const double inf = __builtin_inf(), nan = __builtin_nan("");
    const double norms[12] = {1.0, inf, 2.0, nan, inf, 0.5, 0.25, 3.0, 4.0, inf, inf, 1.0};
    for (int k = 0; k < 12; ++k) {
      CHECK_HIP(hipMemcpy(dsq, &norms[k], 8, hipMemcpyHostToDevice));
      CHECK_ZS(zs_loss_scaler_update_device(dstate, dsq, dtaken, stream));
      CHECK_HIP(hipStreamSynchronize(stream));
      const int32_t want = oracle_scaler_update(&ref, !(norms[k] - norms[k] == 0.0));
      zs_loss_scaler got;
      int32_t taken = -1;
      CHECK_HIP(hipMemcpy(&got, dstate, sizeof got, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(&taken, dtaken, 4, hipMemcpyDeviceToHost));
      if (memcmp(&got, &ref, sizeof got) || taken != want) {
        fprintf(stderr, "device scaler differs from the oracle at step %d\n", k);
        bad = 1;
      }
    }
    CHECK_HIP(hipFree(dstate));
    CHECK_HIP(hipFree(dsq));
    CHECK_HIP(hipFree(dtaken));
  }

  /* 7. optimizer offload */
  {
    shard s;
    shard_init(&s, 50000, 4, 0);
    const int64_t n = s.n;
    float* P = (float*)malloc((size_t)n * 4);
    float* M = (float*)malloc((size_t)n * 4);
    float* V = (float*)malloc((size_t)n * 4);
    memcpy(P, s.hp, (size_t)n * 4);
    memcpy(M, s.hm, (size_t)n * 4);
    memcpy(V, s.hv, (size_t)n * 4);
    zs_offload_t off = NULL;
    CHECK_ZS(zs_offload_create(4096, 3, &off));
    CHECK_ZS(zs_offload_step_flat(off, (const uint16_t* const*)s.dg, s.N, n, P, M, V, s.db, &hp, 13, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    zs_offload_destroy(off);
    uint16_t* hb = (uint16_t*)malloc((size_t)n * 2);
    uint16_t* gb = (uint16_t*)malloc((size_t)n * 2);
    oracle_hp oh = {hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay};
    oracle_reduce_adam((const uint16_t* const*)s.hg, s.N, n, s.hp, s.hm, s.hv, hb, &oh, 13, 4);
    CHECK_HIP(hipMemcpy(gb, s.db, (size_t)n * 2, hipMemcpyDeviceToHost));
    if (memcmp(P, s.hp, (size_t)n * 4) || memcmp(M, s.hm, (size_t)n * 4) || memcmp(V, s.hv, (size_t)n * 4) ||
        memcmp(gb, hb, (size_t)n * 2)) {
      fprintf(stderr, "offload step differs from the oracle\n");
      bad = 1;
    }
    free(P); free(M); free(V); free(hb); free(gb);
    shard_free(&s);
  }

  CHECK_HIP(hipStreamDestroy(stream));
  if (bad) return 1;
  printf("zs_c_client ok\n");
  return 0;
}
