/*
 * Plain fp64 CPU oracle for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the reference the HIP library is
 * checked against; it shares no code, header or constant with the library.
 * Only tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it. It is deliberately slow and obvious: every (sequence, head) first
 * gathers its cached K/V through the block table into a contiguous fp64
 * buffer, then runs textbook softmax attention on that buffer.
 *
 * What is computed follows the pages:
 *  - the KV cache is cut into fixed-size blocks of block_size tokens that
 *    may live anywhere in a pool; a per-sequence block table maps logical
 *    block i to a physical block (devpress.csdn.net page, section
 *    "分页式KV缓存：让显存利用接近理论极限"; aidocs.cortexgrid.cn page, FAQ
 *    answer on the block table; betteryeah.com page, section 2.2).
 *  - at attention time the kernel follows the table and attends across the
 *    scattered blocks as if they were one stream (devpress page, same
 *    section; betteryeah page, section 2.4).
 *  - sequences that share a prefix point at the same physical blocks
 *    (devpress page, "实际收益远超预期"; aidocs page, FAQ on parallel
 *    sampling): the gather simply reads aliased ids twice.
 * The attention formula itself is not written on the pages; the plain
 * reading used here is scaled dot-product softmax attention per (sequence,
 * head): x_t = scale * <q, K_t>, w_t = exp(x_t - max x), out = sum w_t V_t /
 * sum w_t, over the sequence's first ctx tokens (decode: all ctx tokens, the
 * new one included; causal prefill chunk of L queries: query j sits at
 * position ctx - L + j and sees tokens 0..ctx-L+j).
 *
 * Layouts (shared with the library's ABI, a property of the interface, not
 * of the method): caches [num_blocks][H][block_size][d]; q/out rows [.][H][d];
 * block tables int32 [S][max_blocks]; slot = block * block_size + offset.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ODT_F32 = 0, ODT_F16 = 1, ODT_BF16 = 2 };
enum {
  O_OK = 0,
  O_BAD_ARG = -1,
  O_BAD_SLOT = -2,
  O_DUP_SLOT = -3,
  O_BAD_BLOCK = -4,
  O_BAD_CTX = -5,
  O_NOMEM = -6
};

/* ---- exact widening of storage elements to double ---------------------- */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h) {
  int sign = h >> 15;
  int ex = (h >> 10) & 0x1f;
  int fr = h & 0x3ff;
  double mag;
  if (ex == 0)
    mag = ldexp((double)fr, -24); /* subnormal: fr * 2^-24 */
  else if (ex == 31)
    mag = fr ? NAN : INFINITY;
  else
    mag = ldexp((double)(fr | 0x400), ex - 25); /* 1.fr * 2^(ex-15) */
  return sign ? -mag : mag;
}

/* bfloat16 is the top half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case ODT_F32: return (double)((const float*)base)[i];
    case ODT_F16: return half_bits_to_double(((const uint16_t*)base)[i]);
    default: return bf16_bits_to_double(((const uint16_t*)base)[i]);
  }
}

static int elt_bytes(int dtype) { return dtype == ODT_F32 ? 4 : 2; }

/* Exported so the conversion itself can be pinned against a library. */
int oracle_widen(double* out, const void* src, int64_t n, int dtype) {
  if (!out || !src || n < 0 || dtype < 0 || dtype > 2) return O_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = elem(src, dtype, i);
  return O_OK;
}

/* ---- writing new tokens into their slots -------------------------------- */

/* For every new token n with slot_mapping[n] >= 0, copy its K and V rows (all
 * heads) bit for bit into block slot/bs, offset slot%bs. Negative slots are
 * padding and skipped. Out-of-range or repeated slots are rejected before
 * anything is written. */
int oracle_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int32_t* slot_mapping, int num_tokens, int H, int d, int bs,
                             int num_blocks, int dtype) {
  if (num_tokens < 0 || H <= 0 || d <= 0 || bs <= 0 || num_blocks <= 0) return O_BAD_ARG;
  if (num_tokens > 0 && (!k || !v || !k_cache || !v_cache || !slot_mapping)) return O_BAD_ARG;
  const int64_t nslots = (int64_t)num_blocks * bs;
  unsigned char* seen = calloc((size_t)nslots, 1);
  if (!seen) return O_NOMEM;
  for (int n = 0; n < num_tokens; ++n) {
    int32_t s = slot_mapping[n];
    if (s < 0) continue;
    if (s >= nslots) { free(seen); return O_BAD_SLOT; }
    if (seen[s]) { free(seen); return O_DUP_SLOT; }
    seen[s] = 1;
  }
  free(seen);
  const size_t eb = (size_t)elt_bytes(dtype);
  const size_t row = (size_t)d * eb;
  for (int n = 0; n < num_tokens; ++n) {
    int32_t s = slot_mapping[n];
    if (s < 0) continue;
    int64_t blk = s / bs, off = s % bs;
    for (int h = 0; h < H; ++h) {
      size_t src = (((size_t)n * H) + h) * row;
      size_t dst = ((((size_t)blk * H) + h) * bs + off) * row;
      memcpy((char*)k_cache + dst, (const char*)k + src, row);
      memcpy((char*)v_cache + dst, (const char*)v + src, row);
    }
  }
  return O_OK;
}

/* ---- copy-on-write of whole blocks -------------------------------------- */

/* Parallel sampling shares the prompt's blocks; before a sharer writes into a
 * shared block, that block is copied to a fresh one (aidocs.cortexgrid.cn
 * page, FAQ answer on parallel sampling: per-block reference counts and
 * copy-on-write). For each pair i, block pairs[2i+1] of both caches becomes a
 * bit copy of block pairs[2i] (all heads, all offsets). Ids out of range, a
 * destination named twice, or a destination that is also a source (the
 * result would depend on the order) are rejected before anything is copied. */
int oracle_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int npairs, int H, int d,
                       int bs, int num_blocks, int dtype) {
  if (npairs < 0 || H <= 0 || d <= 0 || bs <= 0 || num_blocks <= 0 || dtype < 0 || dtype > 2)
    return O_BAD_ARG;
  if (npairs > 0 && (!k_cache || !v_cache || !pairs)) return O_BAD_ARG;
  unsigned char* role = calloc((size_t)num_blocks, 1); /* bit 0: source, bit 1: destination */
  if (!role) return O_NOMEM;
  for (int i = 0; i < npairs; ++i) {
    int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) { free(role); return O_BAD_BLOCK; }
    if (role[dst] & 2) { free(role); return O_BAD_ARG; }
    role[src] |= 1;
    role[dst] |= 2;
  }
  for (int b = 0; b < num_blocks; ++b)
    if (role[b] == 3) { free(role); return O_BAD_ARG; }
  free(role);
  const size_t block_bytes = (size_t)H * bs * d * (size_t)elt_bytes(dtype);
  for (int i = 0; i < npairs; ++i) {
    size_t src = (size_t)pairs[2 * i] * block_bytes, dst = (size_t)pairs[2 * i + 1] * block_bytes;
    memcpy((char*)k_cache + dst, (const char*)k_cache + src, block_bytes);
    memcpy((char*)v_cache + dst, (const char*)v_cache + src, block_bytes);
  }
  return O_OK;
}

/* ---- block-table translation -------------------------------------------- */

static int check_tables(const int32_t* bt, const int32_t* ctx, int S, int bs, int num_blocks,
                        int max_blocks) {
  for (int s = 0; s < S; ++s) {
    if (ctx[s] < 0 || (int64_t)ctx[s] > (int64_t)max_blocks * bs) return O_BAD_CTX;
    int nblk = (ctx[s] + bs - 1) / bs;
    for (int i = 0; i < nblk; ++i) {
      int32_t b = bt[(int64_t)s * max_blocks + i];
      if (b < 0 || b >= num_blocks) return O_BAD_BLOCK;
    }
  }
  return O_OK;
}

/* Element index of (logical token t, head h, dim 0) of sequence row bt_row. */
static int64_t cache_index(const int32_t* bt_row, int t, int h, int H, int d, int bs) {
  int64_t blk = bt_row[t / bs];
  int64_t off = t % bs;
  return ((blk * H + h) * bs + off) * d;
}

/* Raw copy of the logical K/V of every sequence, rows [cu[s] + t][H][d]. */
int oracle_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                     const int32_t* bt, const int32_t* ctx, int S, int H, int d, int bs,
                     int num_blocks, int max_blocks, int dtype) {
  if (S < 0 || H <= 0 || d <= 0 || bs <= 0 || num_blocks <= 0 || max_blocks <= 0) return O_BAD_ARG;
  int rc = check_tables(bt, ctx, S, bs, num_blocks, max_blocks);
  if (rc) return rc;
  const size_t eb = (size_t)elt_bytes(dtype), row = (size_t)d * eb;
  int64_t base = 0;
  for (int s = 0; s < S; ++s) {
    const int32_t* bt_row = bt + (int64_t)s * max_blocks;
    for (int t = 0; t < ctx[s]; ++t)
      for (int h = 0; h < H; ++h) {
        size_t src = (size_t)cache_index(bt_row, t, h, H, d, bs) * eb;
        size_t dst = (((size_t)(base + t)) * H + h) * row;
        memcpy((char*)k_out + dst, (const char*)k_cache + src, row);
        memcpy((char*)v_out + dst, (const char*)v_cache + src, row);
      }
    base += ctx[s];
  }
  return O_OK;
}

/* Gather tokens 0..n-1 of one (sequence, head) into contiguous fp64 rows. */
static void gather_head(double* K, double* V, const void* k_cache, const void* v_cache,
                        const int32_t* bt_row, int n, int h, int H, int d, int bs, int dtype) {
  for (int t = 0; t < n; ++t) {
    int64_t base = cache_index(bt_row, t, h, H, d, bs);
    for (int e = 0; e < d; ++e) {
      K[(int64_t)t * d + e] = elem(k_cache, dtype, base + e);
      V[(int64_t)t * d + e] = elem(v_cache, dtype, base + e);
    }
  }
}

/* Softmax attention of one query over n contiguous fp64 K/V rows. */
static void attend(double* out, const double* q, const double* K, const double* V, int n, int d,
                   double scale, double* x) {
  if (n == 0) {
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    return;
  }
  double m = -INFINITY;
  for (int t = 0; t < n; ++t) {
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += q[e] * K[(int64_t)t * d + e];
    x[t] = scale * dot;
    if (x[t] > m) m = x[t];
  }
  double sum = 0.0;
  for (int t = 0; t < n; ++t) {
    x[t] = exp(x[t] - m);
    sum += x[t];
  }
  for (int e = 0; e < d; ++e) {
    double acc = 0.0;
    for (int t = 0; t < n; ++t) acc += x[t] * V[(int64_t)t * d + e];
    out[e] = acc / sum;
  }
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Decode: one query per sequence, attending to all ctx[s] cached tokens.
 * pairs = npairs (s, h) pairs; out = [npairs][d] fp64. */
int oracle_decode(double* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* bt, const int32_t* ctx, int S, int H, int d, int bs,
                  int num_blocks, int max_blocks, double scale, int dtype, const int32_t* pairs,
                  int npairs, int nthreads) {
  if (S < 0 || H <= 0 || d <= 0 || bs <= 0 || num_blocks <= 0 || max_blocks <= 0 || npairs < 0 ||
      dtype < 0 || dtype > 2)
    return O_BAD_ARG;
  for (int i = 0; i < npairs; ++i)
    if (pairs[2 * i] < 0 || pairs[2 * i] >= S || pairs[2 * i + 1] < 0 || pairs[2 * i + 1] >= H)
      return O_BAD_ARG;
  int rc = check_tables(bt, ctx, S, bs, num_blocks, max_blocks);
  if (rc) return rc;
  int64_t maxctx = 0;
  for (int s = 0; s < S; ++s) maxctx = ctx[s] > maxctx ? ctx[s] : maxctx;
  set_threads(nthreads);
  int fail = 0;
#pragma omp parallel
  {
    double* K = malloc(sizeof(double) * (size_t)(maxctx + 1) * d);
    double* V = malloc(sizeof(double) * (size_t)(maxctx + 1) * d);
    double* x = malloc(sizeof(double) * (size_t)(maxctx + 1));
    double* qd = malloc(sizeof(double) * (size_t)d);
    const int ok = K && V && x && qd;
    if (!ok) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < npairs; ++i) {
      if (ok) {
        int s = pairs[2 * i], h = pairs[2 * i + 1];
        for (int e = 0; e < d; ++e) qd[e] = elem(q, dtype, ((int64_t)s * H + h) * d + e);
        gather_head(K, V, k_cache, v_cache, bt + (int64_t)s * max_blocks, ctx[s], h, H, d, bs,
                    dtype);
        attend(out + (int64_t)i * d, qd, K, V, ctx[s], d, scale, x);
      }
    }
    free(K); free(V); free(x); free(qd);
  }
  return fail ? O_NOMEM : O_OK;
}

/* Causal prefill of query chunks. Sequence s owns query rows
 * qsl[s]..qsl[s+1]-1 (L_s of them); its context ctx[s] includes the chunk, so
 * row qsl[s]+j is at position ctx[s]-L_s+j and sees tokens 0..ctx[s]-L_s+j.
 * rows = nrows (row, h) pairs; out = [nrows][d] fp64. Rows are grouped by
 * (sequence, head) so each group gathers its K/V once. */
typedef struct { int64_t key; int idx; } row_ref;

static int cmp_row_ref(const void* a, const void* b) {
  const row_ref* x = a;
  const row_ref* y = b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  return x->idx - y->idx;
}

static int seq_of_row(const int32_t* qsl, int S, int r) {
  int lo = 0, hi = S - 1; /* largest s with qsl[s] <= r */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (qsl[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

int oracle_prefill(double* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* bt, const int32_t* ctx, const int32_t* qsl, int S, int H, int d,
                   int bs, int num_blocks, int max_blocks, double scale, int dtype,
                   const int32_t* rows, int nrows, int nthreads) {
  if (S <= 0 || H <= 0 || d <= 0 || bs <= 0 || num_blocks <= 0 || max_blocks <= 0 || nrows < 0 ||
      dtype < 0 || dtype > 2 || qsl[0] != 0)
    return O_BAD_ARG;
  for (int s = 0; s < S; ++s) {
    int L = qsl[s + 1] - qsl[s];
    if (L < 0 || L > ctx[s]) return O_BAD_CTX;
  }
  const int total_q = qsl[S];
  int rc = check_tables(bt, ctx, S, bs, num_blocks, max_blocks);
  if (rc) return rc;
  row_ref* refs = malloc(sizeof(row_ref) * (size_t)(nrows > 0 ? nrows : 1));
  if (!refs) return O_NOMEM;
  for (int i = 0; i < nrows; ++i) {
    int r = rows[2 * i], h = rows[2 * i + 1];
    if (r < 0 || r >= total_q || h < 0 || h >= H) { free(refs); return O_BAD_ARG; }
    refs[i].key = (int64_t)seq_of_row(qsl, S, r) * H + h;
    refs[i].idx = i;
  }
  qsort(refs, (size_t)nrows, sizeof(row_ref), cmp_row_ref);
  /* group starts */
  int* starts = malloc(sizeof(int) * (size_t)(nrows + 1));
  if (!starts) { free(refs); return O_NOMEM; }
  int ngroups = 0;
  for (int i = 0; i < nrows; ++i)
    if (i == 0 || refs[i].key != refs[i - 1].key) starts[ngroups++] = i;
  starts[ngroups] = nrows;
  int64_t maxctx = 0;
  for (int s = 0; s < S; ++s) maxctx = ctx[s] > maxctx ? ctx[s] : maxctx;
  set_threads(nthreads);
  int fail = 0;
#pragma omp parallel
  {
    double* K = malloc(sizeof(double) * (size_t)(maxctx + 1) * d);
    double* V = malloc(sizeof(double) * (size_t)(maxctx + 1) * d);
    double* x = malloc(sizeof(double) * (size_t)(maxctx + 1));
    double* qd = malloc(sizeof(double) * (size_t)d);
    const int ok = K && V && x && qd;
    if (!ok) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int g = 0; g < ngroups; ++g) {
      if (ok) {
        int s = (int)(refs[starts[g]].key / H), h = (int)(refs[starts[g]].key % H);
        int L = qsl[s + 1] - qsl[s];
        gather_head(K, V, k_cache, v_cache, bt + (int64_t)s * max_blocks, ctx[s], h, H, d, bs,
                    dtype);
        for (int i = starts[g]; i < starts[g + 1]; ++i) {
          int idx = refs[i].idx;
          int r = rows[2 * idx];
          int j = r - qsl[s];
          int visible = ctx[s] - L + j + 1;
          for (int e = 0; e < d; ++e) qd[e] = elem(q, dtype, ((int64_t)r * H + h) * d + e);
          attend(out + (int64_t)idx * d, qd, K, V, visible, d, scale, x);
        }
      }
    }
    free(K); free(V); free(x); free(qd);
  }
  free(starts);
  free(refs);
  return fail ? O_NOMEM : O_OK;
}
