/*
 * Host side of the seeded input generator (see synth_core.h for the
 * definition).  Fills host buffers with pthreads.
 *
 * Layout helper: a tensor is generated in LOGICAL row-major order
 * [batch][rows][cols] (counter = offset + (b*rows + r)*cols + c) and written
 * to PHYSICAL address out[b*ld_b + r*ld_r + c*ld_c].  This lets the same
 * logical values land in padded or transposed buffers.
 */
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#include "synth_core.h"

uint64_t synth_stream_id(const char *name) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (const unsigned char *p = (const unsigned char *)name; *p; ++p) {
    h ^= (uint64_t)(*p);
    h *= 0x100000001B3ull;
  }
  return h;
}

typedef struct {
  int kind; /* 0 = normal bf16, 1 = uniform int32 */
  uint64_t key, offset;
  int64_t batch, rows, cols, ld_b, ld_r, ld_c;
  float mean, stdv;
  int32_t lo, hi;
  void *out;
  int64_t begin, end; /* range over batch*rows */
} job_t;

static void *worker(void *arg) {
  job_t *j = (job_t *)arg;
  for (int64_t br = j->begin; br < j->end; ++br) {
    int64_t b = br / j->rows, r = br % j->rows;
    uint64_t cnt = j->offset + (uint64_t)br * (uint64_t)j->cols;
    int64_t base = b * j->ld_b + r * j->ld_r;
    if (j->kind == 0) {
      uint16_t *o = (uint16_t *)j->out;
      for (int64_t c = 0; c < j->cols; ++c)
        o[base + c * j->ld_c] = synth_normal_bf16_at(j->key, cnt + (uint64_t)c, j->mean, j->stdv);
    } else {
      int32_t *o = (int32_t *)j->out;
      for (int64_t c = 0; c < j->cols; ++c)
        o[base + c * j->ld_c] = synth_uniform_at(j->key, cnt + (uint64_t)c, j->lo, j->hi);
    }
  }
  return 0;
}

static void run(job_t proto, int nthreads) {
  int64_t total = proto.batch * proto.rows;
  if (total <= 0 || proto.cols <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > total) nthreads = (int)total;
  pthread_t th[256];
  job_t jobs[256];
  int64_t per = (total + nthreads - 1) / nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].begin = t * per;
    jobs[t].end = jobs[t].begin + per < total ? jobs[t].begin + per : total;
    if (jobs[t].begin >= jobs[t].end) break;
    if (t == 0) continue;
    pthread_create(&th[t], 0, worker, &jobs[t]);
    started = t;
  }
  worker(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], 0);
}

void synth_normal_bf16_3d(uint64_t seed, uint64_t stream, uint64_t offset, int64_t batch,
                          int64_t rows, int64_t cols, float mean, float stdv, uint16_t *out,
                          int64_t ld_b, int64_t ld_r, int64_t ld_c, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof j);
  j.kind = 0;
  j.key = synth_key(seed, stream);
  j.offset = offset;
  j.batch = batch; j.rows = rows; j.cols = cols;
  j.ld_b = ld_b; j.ld_r = ld_r; j.ld_c = ld_c;
  j.mean = mean; j.stdv = stdv;
  j.out = out;
  run(j, nthreads);
}

void synth_uniform_i32_3d(uint64_t seed, uint64_t stream, uint64_t offset, int64_t batch,
                          int64_t rows, int64_t cols, int32_t lo, int32_t hi, int32_t *out,
                          int64_t ld_b, int64_t ld_r, int64_t ld_c, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof j);
  j.kind = 1;
  j.key = synth_key(seed, stream);
  j.offset = offset;
  j.batch = batch; j.rows = rows; j.cols = cols;
  j.ld_b = ld_b; j.ld_r = ld_r; j.ld_c = ld_c;
  j.lo = lo; j.hi = hi;
  j.out = out;
  run(j, nthreads);
}
