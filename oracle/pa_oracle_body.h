/*
 * pa_oracle_body.h -- precision-generic body of the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY (see pa_oracle.h).  Included twice by pa_oracle.c
 * with REAL = double / float, EXPR / LOGR the matching libm routines and
 * NAME(x) appending the precision suffix.  Every loop runs in ascending index
 * order, one (sequence, q head) pair at a time, with no blocking or fusion.
 */

/* Key range [lo, n) a query attends to.  Window reading: with a window W > 0
 * the newest W keys are kept (t >= n - W), else every key; the pages only
 * name a windowed instantiation of the decode kernel [vllm.cpp PR #425,
 * LIMITATIONS: the HasWindow instantiation] and the sliding-window workload
 * masks keys older than ctx - W. */
static int32_t NAME(window_lo)(int32_t n, int32_t window) {
  if (window <= 0) return 0;
  int32_t lo = n - window;
#if ORACLE_MUTATION == 1
  lo += 1; /* planted: window one key short */
#endif
  return lo > 0 ? lo : 0;
}

/* Address of row (token t, KV head g) in a pool: page = bt[t / ps],
 * slot = t % ps.  Returns NULL when the page id is out of range. */
static const uint16_t* NAME(gather_row)(const uint16_t* base,
                                        const oracle_pool* pool,
                                        const int32_t* bt_row, int32_t t,
                                        int32_t g) {
  int32_t page = bt_row[t / pool->page_size];
  int32_t slot = t % pool->page_size;
#if ORACLE_MUTATION == 3
  slot = pool->page_size - 1 - slot; /* planted: slot mirrored in the page */
#endif
  if (page < 0 || page >= pool->num_pages) return 0;
  return base + (int64_t)page * pool->page_stride +
         (int64_t)g * pool->head_stride + (int64_t)slot * pool->token_stride;
}

/* Softmax attention of one query row over keys [t_begin, t_end) of one
 * sequence, two-pass:
 *   s_t = scale * sum_d q_d k_{t,d}
 *   m   = max_t s_t,  l = sum_t exp(s_t - m),
 *   o   = (sum_t exp(s_t - m) v_t) / l.
 * Writes m, l and o[D].  An empty range gives m = -inf, l = 0, o = 0. */
static int NAME(attend_range)(const uint16_t* q_row, const uint16_t* k_pool,
                              const uint16_t* v_pool, const oracle_pool* pool,
                              const int32_t* bt_row, int32_t g, int32_t t_begin,
                              int32_t t_end, REAL scale, REAL* m_out,
                              REAL* l_out, REAL* o) {
  const int32_t D = pool->head_dim;
  for (int32_t d = 0; d < D; ++d) o[d] = 0;
  if (t_end <= t_begin) {
    *m_out = -(REAL)INFINITY;
    *l_out = 0;
    return ORACLE_OK;
  }
  const int32_t n = t_end - t_begin;
  REAL* s = (REAL*)malloc(sizeof(REAL) * (size_t)n);
  if (!s) return ORACLE_ERR_ARGS;
  /* pass 1: scores and their maximum */
  REAL m = -(REAL)INFINITY;
  for (int32_t i = 0; i < n; ++i) {
    const uint16_t* k = NAME(gather_row)(k_pool, pool, bt_row, t_begin + i, g);
    if (!k) { free(s); return ORACLE_ERR_PAGE; }
    REAL dot = 0;
    for (int32_t d = 0; d < D; ++d) dot += BF(q_row[d]) * BF(k[d]);
#if ORACLE_MUTATION == 7
    s[i] = dot; /* planted: scale dropped */
#else
    s[i] = scale * dot;
#endif
    if (s[i] > m) m = s[i];
  }
  /* pass 2: denominator and weighted value sum */
  REAL l = 0;
  for (int32_t i = 0; i < n; ++i) {
    const uint16_t* v = NAME(gather_row)(v_pool, pool, bt_row, t_begin + i, g);
    if (!v) { free(s); return ORACLE_ERR_PAGE; }
    REAL e = EXPR(s[i] - m);
    l += e;
    for (int32_t d = 0; d < D; ++d) o[d] += e * BF(v[d]);
  }
  for (int32_t d = 0; d < D; ++d) o[d] = o[d] / l;
  free(s);
  *m_out = m;
  *l_out = l;
  return ORACLE_OK;
}

static int NAME(check_pool)(const oracle_pool* pool) {
  return pool && pool->num_pages > 0 && pool->page_size > 0 &&
         pool->num_kv_heads > 0 && pool->head_dim > 0;
}

static int32_t NAME(kv_head_of)(int32_t h, int32_t num_q_heads, int32_t num_kv_heads) {
#if ORACLE_MUTATION == 2
  (void)num_q_heads;
  return h % num_kv_heads; /* planted: interleaved instead of contiguous groups */
#else
  return h / (num_q_heads / num_kv_heads);
#endif
}

int NAME(oracle_pa_decode)(const uint16_t* q, const uint16_t* k_pool,
                           const uint16_t* v_pool, const oracle_pool* pool,
                           const int32_t* block_table, int32_t bt_stride,
                           const int32_t* context_lens, int32_t batch,
                           int32_t num_q_heads, double scale, int32_t window,
                           double* out, double* lse) {
  if (!q || !k_pool || !v_pool || !NAME(check_pool)(pool) || !block_table ||
      !context_lens || !out || !lse || batch < 0 || num_q_heads <= 0 ||
      num_q_heads % pool->num_kv_heads != 0)
    return ORACLE_ERR_ARGS;
  const int32_t D = pool->head_dim;
  int err = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t h = 0; h < num_q_heads; ++h) {
      const int32_t n = context_lens[b];
      const int32_t lo = NAME(window_lo)(n, window);
      const int32_t g = NAME(kv_head_of)(h, num_q_heads, pool->num_kv_heads);
      REAL* o = (REAL*)malloc(sizeof(REAL) * (size_t)D);
      REAL m = 0, l = 0;
      int rc = o ? NAME(attend_range)(q + ((int64_t)b * num_q_heads + h) * D,
                                      k_pool, v_pool, pool,
                                      block_table + (int64_t)b * bt_stride, g,
                                      lo, n, (REAL)scale, &m, &l, o)
                 : ORACLE_ERR_ARGS;
      if (rc != ORACLE_OK) {
#pragma omp atomic write
        err = rc;
      } else {
        double* dst = out + ((int64_t)b * num_q_heads + h) * D;
        for (int32_t d = 0; d < D; ++d) dst[d] = (double)o[d];
#if ORACLE_MUTATION == 5
        lse[(int64_t)b * num_q_heads + h] = (l > 0) ? (double)LOGR(l) : -INFINITY; /* planted */
#else
        lse[(int64_t)b * num_q_heads + h] = (l > 0) ? (double)(m + LOGR(l)) : -INFINITY;
#endif
      }
      free(o);
    }
  }
  return err;
}

/* Multi-query decode (the verify step of speculative decoding): sequence b
 * carries S query tokens at the last S positions of its context, q laid out
 * [b][s][h][d].  Query s sees keys up to its own position n - S + s when
 * causal, or the whole context otherwise; a window counts back from the last
 * key it sees [pegainfer PR #938, commit message: the b=8 and b=16 verify
 * steps; vllm.cpp kernel matrix, row KERNEL-ATTN-DFLASH-PAGED-BLOCK: the
 * (1+k) block queries attend over the paged context that holds their own
 * block, with an in-block mask that is either causal or not].  A query with
 * no key gives out = 0, lse = -inf. */
int NAME(oracle_pa_decode_multi)(const uint16_t* q, const uint16_t* k_pool,
                                 const uint16_t* v_pool, const oracle_pool* pool,
                                 const int32_t* block_table, int32_t bt_stride,
                                 const int32_t* context_lens, int32_t batch,
                                 int32_t num_q_heads, int32_t num_queries, int32_t causal,
                                 double scale, int32_t window, double* out, double* lse) {
  if (!q || !k_pool || !v_pool || !NAME(check_pool)(pool) || !block_table ||
      !context_lens || !out || !lse || batch < 0 || num_q_heads <= 0 || num_queries <= 0 ||
      num_q_heads % pool->num_kv_heads != 0)
    return ORACLE_ERR_ARGS;
  const int32_t D = pool->head_dim;
  const int32_t S = num_queries;
  int err = ORACLE_OK;
#pragma omp parallel for collapse(3) schedule(dynamic)
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t sq = 0; sq < S; ++sq) {
      for (int32_t h = 0; h < num_q_heads; ++h) {
        const int32_t n = context_lens[b];
#if ORACLE_MUTATION == 13
        const int32_t last = causal ? n - S + sq + 1 : n - 1; /* planted: one key too far */
#else
        const int32_t last = causal ? n - S + sq : n - 1;
#endif
        const int32_t hi = last + 1 < n ? last + 1 : n;
        const int32_t lo = window > 0 ? (hi - window > 0 ? hi - window : 0) : 0;
        const int64_t row = ((int64_t)b * S + sq) * num_q_heads + h;
        const int32_t g = NAME(kv_head_of)(h, num_q_heads, pool->num_kv_heads);
        REAL* o = (REAL*)malloc(sizeof(REAL) * (size_t)D);
        REAL m = 0, l = 0;
        int rc = !o ? ORACLE_ERR_ARGS
                    : NAME(attend_range)(q + row * D, k_pool, v_pool, pool,
                                         block_table + (int64_t)b * bt_stride, g,
                                         lo > 0 ? lo : 0, hi > 0 ? hi : 0, (REAL)scale, &m, &l, o);
        if (rc != ORACLE_OK) {
#pragma omp atomic write
          err = rc;
        } else {
          for (int32_t d = 0; d < D; ++d) out[row * D + d] = (double)o[d];
          lse[row] = (l > 0) ? (double)(m + LOGR(l)) : -INFINITY;
        }
        free(o);
      }
    }
  }
  return err;
}

int NAME(oracle_pa_partials)(const uint16_t* q, const uint16_t* k_pool,
                             const uint16_t* v_pool, const oracle_pool* pool,
                             const int32_t* block_table, int32_t bt_stride,
                             const int32_t* context_lens, int32_t batch,
                             int32_t num_q_heads, double scale, int32_t window,
                             int32_t partition_size, int32_t max_parts,
                             double* part_out, double* part_max,
                             double* part_sum) {
  if (!q || !k_pool || !v_pool || !NAME(check_pool)(pool) || !block_table ||
      !context_lens || !part_out || !part_max || !part_sum || batch < 0 ||
      num_q_heads <= 0 || num_q_heads % pool->num_kv_heads != 0 ||
      partition_size <= 0 || max_parts <= 0)
    return ORACLE_ERR_ARGS;
  const int32_t D = pool->head_dim;
  int err = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t h = 0; h < num_q_heads; ++h) {
      const int32_t n = context_lens[b];
      const int32_t lo = NAME(window_lo)(n, window);
      const int32_t g = NAME(kv_head_of)(h, num_q_heads, pool->num_kv_heads);
      REAL* o = (REAL*)malloc(sizeof(REAL) * (size_t)D);
      for (int32_t j = 0; j < max_parts && o; ++j) {
        /* Partitions count from the first attended key (reading of the
         * pages: they do not say where splits start under a window). */
#if ORACLE_MUTATION == 10
        int64_t begin = (int64_t)j * partition_size; /* planted: absolute */
#else
        int64_t begin = (int64_t)lo + (int64_t)j * partition_size;
#endif
        int64_t end = begin + partition_size;
        if (begin < lo) begin = lo;
        if (end > n) end = n;
        if (begin > end) begin = end;
        REAL m = 0, l = 0;
        int rc = NAME(attend_range)(q + ((int64_t)b * num_q_heads + h) * D,
                                    k_pool, v_pool, pool,
                                    block_table + (int64_t)b * bt_stride, g,
                                    (int32_t)begin, (int32_t)end, (REAL)scale,
                                    &m, &l, o);
        if (rc != ORACLE_OK) {
#pragma omp atomic write
          err = rc;
          break;
        }
        const int64_t idx = ((int64_t)b * num_q_heads + h) * max_parts + j;
        part_max[idx] = (double)m;
        part_sum[idx] = (double)l;
        for (int32_t d = 0; d < D; ++d) part_out[idx * D + d] = (double)o[d];
      }
      if (!o) {
#pragma omp atomic write
        err = ORACLE_ERR_ARGS;
      }
      free(o);
    }
  }
  return err;
}

/* Merge of split partials:
 *   M = max_j m_j,  w_j = l_j exp(m_j - M),  W = sum_j w_j,
 *   o = sum_j (w_j / W) o_j,  lse = M + log(W),
 * over the live partitions j < ceil((ctx - lo) / P) in ascending j (the same
 * value as sum_j w_j o_j / W; normalising the weights first makes a single
 * live partition reproduce its partial exactly).  No live partition, or
 * every live one empty (M = -inf): o = 0, lse = -inf. */
int NAME(oracle_pa_merge)(const double* part_out, const double* part_max,
                          const double* part_sum, const int32_t* context_lens,
                          int32_t batch, int32_t num_q_heads, int32_t head_dim,
                          int32_t partition_size, int32_t max_parts,
                          int32_t window, double* out, double* lse) {
  if (!part_out || !part_max || !part_sum || !context_lens || !out || !lse ||
      batch < 0 || num_q_heads <= 0 || head_dim <= 0 || partition_size <= 0 ||
      max_parts <= 0)
    return ORACLE_ERR_ARGS;
  int err = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t h = 0; h < num_q_heads; ++h) {
      const int32_t n = context_lens[b];
      const int32_t lo = NAME(window_lo)(n, window);
      int64_t live = ((int64_t)n - lo + partition_size - 1) / partition_size;
      if (live > max_parts) {
#pragma omp atomic write
        err = ORACLE_ERR_ARGS;
        continue;
      }
      const int64_t row = (int64_t)b * num_q_heads + h;
      double* dst = out + row * head_dim;
      for (int32_t d = 0; d < head_dim; ++d) dst[d] = 0.0;
      REAL M = -(REAL)INFINITY;
      for (int64_t j = 0; j < live; ++j) {
        REAL mj = (REAL)part_max[row * max_parts + j];
        if (mj > M) M = mj;
      }
      if (live == 0 || M == -(REAL)INFINITY) {
        lse[row] = -INFINITY;
        continue;
      }
      /* pass 1: weights and their total */
      REAL W = 0;
      for (int64_t j = 0; j < live; ++j) {
        const int64_t idx = row * max_parts + j;
        REAL mj = (REAL)part_max[idx];
        REAL lj = (REAL)part_sum[idx];
        if (mj == -(REAL)INFINITY || lj == 0) continue; /* empty partition */
#if ORACLE_MUTATION == 6
        W += EXPR(mj - M); /* planted: partition weight without its sum */
#else
        W += lj * EXPR(mj - M);
#endif
      }
      /* pass 2: weighted sum of the normalised partial outputs */
      REAL* acc = (REAL*)calloc((size_t)head_dim, sizeof(REAL));
      if (!acc) {
#pragma omp atomic write
        err = ORACLE_ERR_ARGS;
        continue;
      }
      for (int64_t j = 0; j < live; ++j) {
        const int64_t idx = row * max_parts + j;
        REAL mj = (REAL)part_max[idx];
        REAL lj = (REAL)part_sum[idx];
        if (mj == -(REAL)INFINITY || lj == 0) continue;
#if ORACLE_MUTATION == 6
        REAL w = EXPR(mj - M) / W;
#else
        REAL w = lj * EXPR(mj - M) / W;
#endif
        for (int32_t d = 0; d < head_dim; ++d)
          acc[d] += w * (REAL)part_out[idx * head_dim + d];
      }
      for (int32_t d = 0; d < head_dim; ++d) dst[d] = (double)acc[d];
      lse[row] = (double)(M + LOGR(W));
      free(acc);
    }
  }
  return err;
}

/* Absorbed MLA decode for one (sequence, head), following the order of the
 * kernel schedule quoted in pegainfer PR #938 (steps 1-7), every intermediate
 * kept at REAL precision (no bf16 landing):
 *   1. q_abs[j] = sum_d q_nope[d] W_UK[h][d][j]
 *   2. s_t = scale * (sum_j q_abs[j] c_t[j] + sum_r q_rope[r] c_t[d_lat + r])
 *   3. m = max s_t, l = sum exp(s_t - m)
 *   4. o_lat[j] = sum_t exp(s_t - m) c_t[j] / l     (V = the latent)
 *   5. out[dv] = sum_j W_UV[h][dv][j] o_lat[j]                              */
int NAME(oracle_mla_decode)(const uint16_t* q_nope, const uint16_t* q_rope,
                            const uint16_t* cache, const oracle_pool* pool,
                            const uint16_t* w_uk, const uint16_t* w_uv,
                            const int32_t* block_table, int32_t bt_stride,
                            const int32_t* context_lens, int32_t batch,
                            int32_t num_heads, int32_t d_nope, int32_t d_rope,
                            int32_t d_lat, int32_t d_v, double scale,
                            double* out, double* q_abs_out, double* lse) {
  if (!q_nope || !q_rope || !cache || !NAME(check_pool)(pool) || !w_uk ||
      !w_uv || !block_table || !context_lens || !out || batch < 0 ||
      num_heads <= 0 || d_nope <= 0 || d_rope < 0 || d_lat <= 0 || d_v <= 0 ||
      pool->num_kv_heads != 1 || pool->head_dim != d_lat + d_rope)
    return ORACLE_ERR_ARGS;
  int err = ORACLE_OK;
  const REAL sc = (REAL)scale;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t h = 0; h < num_heads; ++h) {
      const int64_t row = (int64_t)b * num_heads + h;
      const int32_t n = context_lens[b];
      const int32_t* bt_row = block_table + (int64_t)b * bt_stride;
      const uint16_t* qn = q_nope + row * d_nope;
      const uint16_t* qr = q_rope + row * d_rope;
      REAL* q_abs = (REAL*)malloc(sizeof(REAL) * (size_t)d_lat);
      REAL* o_lat = (REAL*)calloc((size_t)d_lat, sizeof(REAL));
      REAL* s = (REAL*)malloc(sizeof(REAL) * (size_t)(n > 0 ? n : 1));
      if (!q_abs || !o_lat || !s) {
#pragma omp atomic write
        err = ORACLE_ERR_ARGS;
        free(q_abs); free(o_lat); free(s);
        continue;
      }
      /* step 1: absorb W_UK into the query */
      for (int32_t j = 0; j < d_lat; ++j) {
        REAL acc = 0;
        for (int32_t d = 0; d < d_nope; ++d) {
#if ORACLE_MUTATION == 4
          const int64_t wi = ((int64_t)h * d_lat + j) * d_nope + d; /* planted: [j][d] */
#else
          const int64_t wi = ((int64_t)h * d_nope + d) * d_lat + j;
#endif
          acc += BF(qn[d]) * BF(w_uk[wi]);
        }
        q_abs[j] = acc;
      }
      if (q_abs_out)
        for (int32_t j = 0; j < d_lat; ++j) q_abs_out[row * d_lat + j] = (double)q_abs[j];
      /* steps 2-3: scores over the 576-wide rows, then max and sum */
      REAL m = -(REAL)INFINITY;
      int bad = 0;
      for (int32_t t = 0; t < n && !bad; ++t) {
        const uint16_t* c = NAME(gather_row)(cache, pool, bt_row, t, 0);
        if (!c) { bad = 1; break; }
        REAL dot = 0;
        for (int32_t j = 0; j < d_lat; ++j) dot += q_abs[j] * BF(c[j]);
#if ORACLE_MUTATION == 9
        (void)qr; /* planted: rope term dropped */
#else
        for (int32_t r = 0; r < d_rope; ++r)
          dot += BF(qr[r]) * BF(c[d_lat + r]);
#endif
        s[t] = sc * dot;
        if (s[t] > m) m = s[t];
      }
      REAL l = 0;
      for (int32_t t = 0; t < n && !bad; ++t) {
        const uint16_t* c = NAME(gather_row)(cache, pool, bt_row, t, 0);
        REAL e = EXPR(s[t] - m);
        l += e;
#if ORACLE_MUTATION == 8
        const uint16_t* vrow = c + d_rope; /* planted: value row shifted */
#else
        const uint16_t* vrow = c;
#endif
        for (int32_t j = 0; j < d_lat; ++j) o_lat[j] += e * BF(vrow[j]);
      }
      if (bad) {
#pragma omp atomic write
        err = ORACLE_ERR_PAGE;
      } else {
        /* step 4: normalise; an empty context gives o_lat = 0 */
        for (int32_t j = 0; j < d_lat; ++j) o_lat[j] = (n > 0) ? o_lat[j] / l : 0;
        /* step 5: up-project through W_UV */
        for (int32_t dv = 0; dv < d_v; ++dv) {
          REAL acc = 0;
          for (int32_t j = 0; j < d_lat; ++j)
            acc += BF(w_uv[((int64_t)h * d_v + dv) * d_lat + j]) * o_lat[j];
          out[row * d_v + dv] = (double)acc;
        }
        if (lse) lse[row] = (n > 0) ? (double)(m + LOGR(l)) : -INFINITY;
      }
      free(q_abs); free(o_lat); free(s);
    }
  }
  return err;
}
