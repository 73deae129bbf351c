/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the swizzled
 * tiled GEMM.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product library never
 * does, and this file shares no code, header, table or helper with it.
 *
 * What it computes, and where the pages define it:
 *   - the block -> tile map of GemmIdentityBlockSwizzle: loop counts
 *     ("Block Scheduler Code Explained", s4.1 Constructor, s4.3
 *     GetCoreLoops), the batch index (s4.4 GetBatchIdx), the Zn window
 *     order with snake reversal (s4.5 GetBlockCoord, s5.1, s5.2), the Nz
 *     order (s4.5, whose body the page elides: read here as the Zn rule with
 *     the roles of M and N exchanged, as the page's prose on the Nz
 *     direction says), and the tail-tile shapes (s4.6 GetActualBlockShape,
 *     s5.3);
 *   - a RASTER order (row-major over tiles, no windows, no snake) that the
 *     pages do not define; it is the row-major baseline of the comparison;
 *   - the grouped slice-M decomposition: groups concatenated in order, each
 *     re-targeted with Update (s4.2) to its own M;
 *   - the grouped slice-K product: K cut into consecutive groups, one output
 *     matrix per group, the groups' tasks numbered like batches (s4.4);
 *   - C = A.B in fp64 (int64 for int8), element by element, one task at a
 *     time in map order, each output element written exactly once; and the
 *     per-token / per-channel dequant out = acc * s_row[i] * s_col[g][j].
 *
 * Parity pins (tests/test_oracle_*.py): generative brute force of the window
 * order, bijection and tail sums, closed forms (identity, rank-1, all-ones),
 * brute force in exact integer arithmetic on tiny shapes, numpy fp64 / int64
 * matmul on medium shapes, exhaustive decoder tables against torch casts.
 * The choice of the Nz mirror reading is "parity unpinned" by the pages
 * (only its self-consistency is pinned).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes (the oracle's own; the product header has its own enum) */
enum { ORC_F16 = 1, ORC_BF16 = 2, ORC_E4M3 = 3, ORC_MXE4M3 = 4, ORC_I8 = 5 };

/* ---------------------------------------------------------------- map --- */

/* CeilDiv ("Block Scheduler Code Explained", s4.1). */
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

/*
 * Block coordinate of task `inner` inside one problem of loopsM x loopsN
 * tiles (s4.5 GetBlockCoord, runtime offset and direction as in s6
 * DynamicGemmIdentityBlockSwizzle).  dir 0 = Zn, 1 = Nz, 2 = RASTER.
 * Returns 0 on success, -1 on an undefined parameter.
 */
static int block_coord(int64_t loopsM, int64_t loopsN, int64_t off, int dir,
                       int64_t inner, int64_t *mIdx, int64_t *nIdx) {
  if (off <= 0) return -1;
  if (dir == 0) {
    /* Zn: windows of `off` tile-rows; inside a window the M index runs
     * fastest; the last window holds the remaining rows; odd windows walk
     * the N index backwards (snake). */
    int64_t tileBlockLoop = cdiv(loopsM, off);
    int64_t tileBlockIdx = inner / (off * loopsN);
    int64_t inTileBlockIdx = inner % (off * loopsN);
    int64_t nRow = off;
    if (tileBlockIdx == tileBlockLoop - 1) nRow = loopsM - off * tileBlockIdx;
    *mIdx = tileBlockIdx * off + inTileBlockIdx % nRow;
    *nIdx = inTileBlockIdx / nRow;
    if (tileBlockIdx % 2 == 1) *nIdx = loopsN - *nIdx - 1;
    return 0;
  }
  if (dir == 1) {
    /* Nz: the same rule with M and N exchanged: windows of `off`
     * tile-columns, N index fastest inside a window, odd windows walk the
     * M index backwards. */
    int64_t tileBlockLoop = cdiv(loopsN, off);
    int64_t tileBlockIdx = inner / (off * loopsM);
    int64_t inTileBlockIdx = inner % (off * loopsM);
    int64_t nCol = off;
    if (tileBlockIdx == tileBlockLoop - 1) nCol = loopsN - off * tileBlockIdx;
    *nIdx = tileBlockIdx * off + inTileBlockIdx % nCol;
    *mIdx = inTileBlockIdx / nCol;
    if (tileBlockIdx % 2 == 1) *mIdx = loopsM - *mIdx - 1;
    return 0;
  }
  if (dir == 2) {
    /* RASTER: row-major over the tile grid (not on the pages). */
    *mIdx = inner / loopsN;
    *nIdx = inner % loopsN;
    return 0;
  }
  return -1;
}

/*
 * Batched map.  out[t*5 + {0..4}] = {batch, m, n, mActual, nActual} for
 * t in [0, batch*loopsM*loopsN).  Returns the task count, or -1 on bad
 * arguments, or -2 if max_tasks is too small.
 */
int64_t orc_tile_map(int64_t batch, int64_t M, int64_t N, int64_t tm, int64_t tn,
                     int64_t off, int dir, uint32_t *out, int64_t max_tasks) {
  if (batch < 0 || M < 0 || N < 0 || tm <= 0 || tn <= 0 || off <= 0) return -1;
  if (dir < 0 || dir > 2) return -1;
  int64_t loopsM = cdiv(M, tm), loopsN = cdiv(N, tn);       /* s4.1 */
  int64_t core = loopsM * loopsN;                             /* s4.3 */
  int64_t T = batch * core;
  if (T > max_tasks) return -2;
  for (int64_t t = 0; t < T; ++t) {
    int64_t b = t / core;                                     /* s4.4 */
    int64_t inner = t % core;                                 /* s4.5 */
    int64_t m, n;
    if (block_coord(loopsM, loopsN, off, dir, inner, &m, &n)) return -1;
    /* s4.6 GetActualBlockShape */
    int64_t mAct = (m == loopsM - 1) ? (M - m * tm) : tm;
    int64_t nAct = (n == loopsN - 1) ? (N - n * tn) : tn;
    uint32_t *o = out + 5 * t;
    o[0] = (uint32_t)b; o[1] = (uint32_t)m; o[2] = (uint32_t)n;
    o[3] = (uint32_t)mAct; o[4] = (uint32_t)nAct;
  }
  return T;
}

/*
 * Grouped slice-M map.  Group g has M = group_m[g] rows (rows of all groups
 * are stacked in order) and shares N.  Tasks are the groups' task ranges
 * concatenated in group order; inside a group the scheduler is re-targeted
 * to (group_m[g], N) (s4.2 Update) and maps the local index.
 * out[t*6 + {0..5}] = {g, m, n, mActual, nActual, first row of the tile in
 * the stacked A / C}.  Returns the task count, -1 on bad arguments, -2 if
 * max_tasks is too small.
 */
int64_t orc_grouped_tile_map(int32_t G, const int32_t *group_m, int64_t N, int64_t tm,
                             int64_t tn, int64_t off, int dir, uint32_t *out,
                             int64_t max_tasks) {
  if (G < 0 || N < 0 || tm <= 0 || tn <= 0 || off <= 0 || dir < 0 || dir > 2) return -1;
  int64_t t = 0, row0 = 0;
  for (int32_t g = 0; g < G; ++g) {
    int64_t Mg = group_m[g];
    if (Mg < 0) return -1;
    int64_t loopsM = cdiv(Mg, tm), loopsN = cdiv(N, tn);
    int64_t core = loopsM * loopsN;
    for (int64_t inner = 0; inner < core; ++inner, ++t) {
      if (t >= max_tasks) return -2;
      int64_t m, n;
      if (block_coord(loopsM, loopsN, off, dir, inner, &m, &n)) return -1;
      int64_t mAct = (m == loopsM - 1) ? (Mg - m * tm) : tm;
      int64_t nAct = (n == loopsN - 1) ? (N - n * tn) : tn;
      uint32_t *o = out + 6 * t;
      o[0] = (uint32_t)g; o[1] = (uint32_t)m; o[2] = (uint32_t)n;
      o[3] = (uint32_t)mAct; o[4] = (uint32_t)nAct;
      o[5] = (uint32_t)(row0 + m * tm);
    }
    row0 += Mg;
  }
  return t;
}

/* ----------------------------------------------------------- decoders --- */
/* Each decoder takes the raw bit pattern and returns its exact value.  The
 * formats: IEEE binary16; bfloat16 (the top half of a binary32); OCP FP8
 * E4M3 "fn" (bias 7, no infinities, S.1111.111 is NaN, max 448, subnormals
 * m * 2^-9); OCP E8M0 scale (2^(e-127), 0xFF is NaN). */

static double dec_f16(uint32_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 0x400), e - 25);
  return s ? -v : v;
}

static double dec_bf16(uint32_t h) {
  int s = (h >> 15) & 1, e = (h >> 7) & 0xff, m = h & 0x7f;
  double v;
  if (e == 0) v = ldexp((double)m, -133);
  else if (e == 255) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 0x80), e - 134);
  return s ? -v : v;
}

static double dec_e4m3(uint32_t b) {
  int s = (b >> 7) & 1, e = (b >> 3) & 0xf, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp((double)(m | 8), e - 10);
  return s ? -v : v;
}

static double dec_e8m0(uint32_t b) {
  if (b == 255) return NAN;
  return ldexp(1.0, (int)b - 127);
}

/* kind: 1 f16, 2 bf16, 3 e4m3fn, 5 int8, 6 int32, 7 f32, 8 e8m0 */
int orc_decode(int kind, const void *src, int64_t n, double *dst) {
  for (int64_t i = 0; i < n; ++i) {
    switch (kind) {
      case 1: dst[i] = dec_f16(((const uint16_t *)src)[i]); break;
      case 2: dst[i] = dec_bf16(((const uint16_t *)src)[i]); break;
      case 3: dst[i] = dec_e4m3(((const uint8_t *)src)[i]); break;
      case 5: dst[i] = (double)((const int8_t *)src)[i]; break;
      case 6: dst[i] = (double)((const int32_t *)src)[i]; break;
      case 7: dst[i] = (double)((const float *)src)[i]; break;
      case 8: dst[i] = dec_e8m0(((const uint8_t *)src)[i]); break;
      default: return -1;
    }
  }
  return 0;
}

/* ------------------------------------------------------------- GEMM ----- */

static double elem(int ab, const void *p, int64_t idx) {
  switch (ab) {
    case ORC_F16: return dec_f16(((const uint16_t *)p)[idx]);
    case ORC_BF16: return dec_bf16(((const uint16_t *)p)[idx]);
    case ORC_E4M3:
    case ORC_MXE4M3: return dec_e4m3(((const uint8_t *)p)[idx]);
    case ORC_I8: return (double)((const int8_t *)p)[idx];
  }
  return NAN;
}

/*
 * Row selection: rows[] lists the wanted rows of the stacked (batch*M) row
 * space; NULL means all rows in order.  pos[r] is the output row of stacked
 * row r, or -1.  Returns NULL on a bad list.
 */
static int64_t *row_positions(int64_t total_rows, const int64_t *rows, int64_t nrows) {
  int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)(total_rows > 0 ? total_rows : 1));
  if (!pos) return NULL;
  if (!rows) {
    for (int64_t r = 0; r < total_rows; ++r) pos[r] = r;
    return pos;
  }
  for (int64_t r = 0; r < total_rows; ++r) pos[r] = -1;
  for (int64_t i = 0; i < nrows; ++i) {
    if (rows[i] < 0 || rows[i] >= total_rows || pos[rows[i]] != -1) { free(pos); return NULL; }
    pos[rows[i]] = i;
  }
  return pos;
}

/*
 * Batched dense GEMM oracle: for b in [0,batch): C_b = A_b . B_b with
 * A_b = A + b*strideA (row-major [M][lda]), B_b = B + b*strideB (row-major
 * [K][ldb]).  For ORC_MXE4M3, sa is [M][ldsa] e8m0 (one scale per row and
 * 32-element K block) and sb is [K/32][ldsb] e8m0 (one per K block and
 * column); they are shared by all batches.
 *
 * ref[p][j] = sum over k of a_ik * b_kj in fp64 (for MX: the sum of each
 * 32-element block, times 2^(sa-127) * 2^(sb-127), summed over blocks), and
 * den[p][j] = the same sum over |a_ik * b_kj| (times the scales), for each
 * selected stacked row b*M+i at output row p.  acc (optional, int8 only)
 * receives the exact int64 sums.
 *
 * The tasks are visited in the order of the block map (tm, tn, off, dir);
 * each output element is written by exactly one task, which the function
 * checks.  Returns 0, -1 on bad arguments, -3 if an element was written
 * other than once.
 */
int orc_gemm(int ab, int64_t batch, int64_t M, int64_t N, int64_t K,
             const void *A, int64_t lda, int64_t strideA,
             const void *B, int64_t ldb, int64_t strideB,
             const uint8_t *sa, int64_t ldsa, const uint8_t *sb, int64_t ldsb,
             int64_t tm, int64_t tn, int64_t off, int dir,
             const int64_t *rows, int64_t nrows,
             double *ref, double *den, int64_t *acc) {
  if (batch < 0 || M < 0 || N < 0 || K < 0 || tm <= 0 || tn <= 0) return -1;
  if (ab == ORC_MXE4M3 && (K % 32 != 0 || !sa || !sb)) return -1;
  int64_t loopsM = cdiv(M, tm), loopsN = cdiv(N, tn), core = loopsM * loopsN;
  int64_t T = batch * core;
  int64_t total_rows = batch * M;
  if (!rows) nrows = total_rows;
  int64_t *pos = row_positions(total_rows, rows, nrows);
  if (!pos) return -1;
  uint8_t *count = (uint8_t *)calloc((size_t)(nrows * N > 0 ? nrows * N : 1), 1);
  if (!count) { free(pos); return -1; }
  int bad = 0;

  #pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
  for (int64_t t = 0; t < T; ++t) {
    int64_t b = t / core, inner = t % core, m, n;
    if (block_coord(loopsM, loopsN, off, dir, inner, &m, &n)) { bad |= 1; continue; }
    int64_t mAct = (m == loopsM - 1) ? (M - m * tm) : tm;
    int64_t nAct = (n == loopsN - 1) ? (N - n * tn) : tn;
    const char *Ab = (const char *)A;
    const char *Bb = (const char *)B;
    int64_t esz = (ab == ORC_F16 || ab == ORC_BF16) ? 2 : 1;
    Ab += b * strideA * esz;
    Bb += b * strideB * esz;
    for (int64_t i = m * tm; i < m * tm + mAct; ++i) {
      int64_t p = pos[b * M + i];
      if (p < 0) continue;
      for (int64_t j = n * tn; j < n * tn + nAct; ++j) {
        double s = 0.0, d = 0.0;
        int64_t si = 0, di = 0;
        if (ab == ORC_MXE4M3) {
          for (int64_t kb = 0; kb < K / 32; ++kb) {
            double bs = 0.0, bd = 0.0;
            for (int64_t k = kb * 32; k < kb * 32 + 32; ++k) {
              double x = elem(ab, Ab, i * lda + k) * elem(ab, Bb, k * ldb + j);
              bs += x; bd += fabs(x);
            }
            double scale = dec_e8m0(sa[i * ldsa + kb]) * dec_e8m0(sb[kb * ldsb + j]);
            s += scale * bs; d += scale * bd;
          }
        } else if (ab == ORC_I8) {
          for (int64_t k = 0; k < K; ++k) {
            int64_t x = (int64_t)((const int8_t *)Ab)[i * lda + k] *
                        (int64_t)((const int8_t *)Bb)[k * ldb + j];
            si += x; di += x < 0 ? -x : x;
          }
          s = (double)si; d = (double)di;
        } else {
          for (int64_t k = 0; k < K; ++k) {
            double x = elem(ab, Ab, i * lda + k) * elem(ab, Bb, k * ldb + j);
            s += x; d += fabs(x);
          }
        }
        ref[p * N + j] = s;
        den[p * N + j] = d;
        if (acc) acc[p * N + j] = si;
        #pragma omp atomic
        count[p * N + j] += 1;
      }
    }
  }
  int rc = bad ? -1 : 0;
  for (int64_t e = 0; rc == 0 && e < nrows * N; ++e)
    if (count[e] != 1) rc = -3;
  free(count); free(pos);
  return rc;
}

/*
 * Grouped slice-M int8 GEMM with optional per-token / per-channel dequant.
 * A is the stacked int8 [total_m][lda] (group g owns rows
 * [sum_{h<g} group_m[h], + group_m[g])), B_g = B + g*strideB is int8
 * [K][ldb].  acc[p][j] = exact int64 sum; if row_scale and col_scale are
 * given, ref[p][j] = acc * row_scale[r] * col_scale[g*N + j] in fp64 and
 * den = sum |a*b| * |row_scale * col_scale|; otherwise ref = acc and
 * den = sum |a*b|.  Rows are the stacked rows (rows[] as in orc_gemm).
 * Tasks follow the grouped map; each element is written exactly once.
 */
int orc_grouped_gemm(int32_t G, const int32_t *group_m, int64_t total_m, int64_t N, int64_t K,
                     const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb, int64_t strideB,
                     const float *row_scale, const float *col_scale,
                     int64_t tm, int64_t tn, int64_t off, int dir,
                     const int64_t *rows, int64_t nrows,
                     double *ref, double *den, int64_t *acc) {
  if (G < 0 || N < 0 || K < 0 || tm <= 0 || tn <= 0 || off <= 0) return -1;
  int64_t sumM = 0;
  for (int32_t g = 0; g < G; ++g) { if (group_m[g] < 0) return -1; sumM += group_m[g]; }
  if (sumM > total_m) return -1;
  int64_t T = 0;
  for (int32_t g = 0; g < G; ++g) T += cdiv(group_m[g], tm) * cdiv(N, tn);
  uint32_t *map = (uint32_t *)malloc(sizeof(uint32_t) * 6 * (size_t)(T > 0 ? T : 1));
  if (!map) return -1;
  if (orc_grouped_tile_map(G, group_m, N, tm, tn, off, dir, map, T) != T) { free(map); return -1; }
  if (!rows) nrows = sumM;
  int64_t *pos = row_positions(sumM, rows, nrows);
  if (!pos) { free(map); return -1; }
  uint8_t *count = (uint8_t *)calloc((size_t)(nrows * N > 0 ? nrows * N : 1), 1);
  if (!count) { free(map); free(pos); return -1; }

  #pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t) {
    const uint32_t *o = map + 6 * t;
    int64_t g = o[0], n = o[2], mAct = o[3], nAct = o[4], r0 = o[5];
    const int8_t *Bg = B + g * strideB;
    for (int64_t r = r0; r < r0 + mAct; ++r) {
      int64_t p = pos[r];
      if (p < 0) continue;
      for (int64_t j = n * tn; j < n * tn + nAct; ++j) {
        int64_t s = 0, d = 0;
        for (int64_t k = 0; k < K; ++k) {
          int64_t x = (int64_t)A[r * lda + k] * (int64_t)Bg[k * ldb + j];
          s += x; d += x < 0 ? -x : x;
        }
        if (acc) acc[p * N + j] = s;
        if (row_scale && col_scale) {
          double rs = (double)row_scale[r], cs = (double)col_scale[g * N + j];
          ref[p * N + j] = (double)s * rs * cs;
          den[p * N + j] = (double)d * fabs(rs * cs);
        } else {
          ref[p * N + j] = (double)s;
          den[p * N + j] = (double)d;
        }
        #pragma omp atomic
        count[p * N + j] += 1;
      }
    }
  }
  int rc = 0;
  for (int64_t e = 0; rc == 0 && e < nrows * N; ++e)
    if (count[e] != 1) rc = -3;
  free(count); free(pos); free(map);
  return rc;
}

/* ------------------------------------------------ grouped slice-K ----- */

/*
 * Grouped slice-K GEMM, with optional per-token / per-channel dequant
 * ("Block Dispatch Policies" names a grouped-matmul-slice-K example and its
 * per-token-dequant variant under the PreloadAsync policies; reading: the K
 * dimension is cut into G consecutive groups and each group is its own
 * product with its own output matrix).
 *
 * Group g owns K indices [Q_g, Q_g + group_k[g]) with Q_g the sum of the
 * earlier groups' sizes: columns of A (row-major [M][lda], total_k columns
 * allocated) and rows of B (row-major [total_k][ldb]).  Its output is
 * C_g = A[:, Q_g : Q_g + k_g] . B[Q_g : Q_g + k_g, :], an M x N matrix; the
 * outputs are stacked as rows g*M + i.  An empty group (k_g = 0) has an
 * all-zero output.  Every group shares M and N, so the tasks are those of
 * a batched problem with G batches: task t belongs to group t / core and
 * maps its local index with the block map (s4.3, s4.4, s4.5, s4.6).
 *
 * acc (int8 only) receives the exact int64 sums.  ref / den as in orc_gemm:
 * ref = the exact sum (fp64; int8: the int64 sum), den = the sum of
 * |products|; with row_scale ([G][M]: per group and token row) and
 * col_scale ([G][N]: per group and channel), int8 only, ref = acc *
 * row_scale[g*M + i] * col_scale[g*N + j] and den is scaled by
 * |row_scale * col_scale|.  Rows select stacked rows g*M + i as in orc_gemm.
 * Returns 0, -1 on bad arguments (negative group size, sizes summing past
 * total_k, scales with non-int8 operands), -3 if an element was written
 * other than once.
 */
int orc_grouped_gemm_slice_k(int ab, int32_t G, const int32_t *group_k, int64_t total_k,
                             int64_t M, int64_t N, const void *A, int64_t lda,
                             const void *B, int64_t ldb,
                             const float *row_scale, const float *col_scale,
                             int64_t tm, int64_t tn, int64_t off, int dir,
                             const int64_t *rows, int64_t nrows,
                             double *ref, double *den, int64_t *acc) {
  if (G < 0 || M < 0 || N < 0 || total_k < 0 || tm <= 0 || tn <= 0 || off <= 0) return -1;
  if (ab != ORC_F16 && ab != ORC_BF16 && ab != ORC_I8) return -1;
  if ((row_scale || col_scale) && (ab != ORC_I8 || !row_scale || !col_scale)) return -1;
  int64_t *q = (int64_t *)malloc(sizeof(int64_t) * (size_t)(G + 1));
  if (!q) return -1;
  q[0] = 0;
  for (int32_t g = 0; g < G; ++g) {
    if (group_k[g] < 0) { free(q); return -1; }
    q[g + 1] = q[g] + group_k[g];
  }
  if (q[G] > total_k) { free(q); return -1; }
  int64_t loopsM = cdiv(M, tm), loopsN = cdiv(N, tn), core = loopsM * loopsN;
  int64_t T = (int64_t)G * core;
  int64_t total_rows = (int64_t)G * M;
  if (!rows) nrows = total_rows;
  int64_t *pos = row_positions(total_rows, rows, nrows);
  if (!pos) { free(q); return -1; }
  uint8_t *count = (uint8_t *)calloc((size_t)(nrows * N > 0 ? nrows * N : 1), 1);
  if (!count) { free(q); free(pos); return -1; }
  int bad = 0;

  #pragma omp parallel for schedule(dynamic, 1) reduction(|: bad)
  for (int64_t t = 0; t < T; ++t) {
    int64_t g = t / core, inner = t % core, m, n;       /* the group, like s4.4 */
    if (block_coord(loopsM, loopsN, off, dir, inner, &m, &n)) { bad |= 1; continue; }
    int64_t mAct = (m == loopsM - 1) ? (M - m * tm) : tm;
    int64_t nAct = (n == loopsN - 1) ? (N - n * tn) : tn;
    for (int64_t i = m * tm; i < m * tm + mAct; ++i) {
      int64_t p = pos[g * M + i];
      if (p < 0) continue;
      for (int64_t j = n * tn; j < n * tn + nAct; ++j) {
        double s = 0.0, d = 0.0;
        int64_t si = 0, di = 0;
        for (int64_t k = q[g]; k < q[g + 1]; ++k) {
          if (ab == ORC_I8) {
            int64_t x = (int64_t)((const int8_t *)A)[i * lda + k] *
                        (int64_t)((const int8_t *)B)[k * ldb + j];
            si += x; di += x < 0 ? -x : x;
          } else {
            double x = elem(ab, A, i * lda + k) * elem(ab, B, k * ldb + j);
            s += x; d += fabs(x);
          }
        }
        if (ab == ORC_I8) { s = (double)si; d = (double)di; }
        if (row_scale) {
          double rs = (double)row_scale[g * M + i], cs = (double)col_scale[g * N + j];
          ref[p * N + j] = s * rs * cs;
          den[p * N + j] = d * fabs(rs * cs);
        } else {
          ref[p * N + j] = s;
          den[p * N + j] = d;
        }
        if (acc) acc[p * N + j] = si;
        #pragma omp atomic
        count[p * N + j] += 1;
      }
    }
  }
  int rc = bad ? -1 : 0;
  for (int64_t e = 0; rc == 0 && e < nrows * N; ++e)
    if (count[e] != 1) rc = -3;
  free(count); free(pos); free(q);
  return rc;
}

/* -------------------------------------------------------- matmul-add ---- */

/*
 * matmul-add ("Block Dispatch Policies" lists a matmul-add example under its
 * ping-pong policy; reading: C = A.B + X with X of C's shape and type).
 * Given the exact A.B in ref and its error scale sum |a*b| in den (from
 * orc_gemm), adds the addend's exact values x to ref and |x| to den, so that
 * the compare criterion |got - ref| / den stays a relative error of the
 * whole sum.  n elements, all arrays float64.
 */
int orc_add_addend(int64_t n, const double *x, double *ref, double *den) {
  if (n < 0 || (n > 0 && (!x || !ref || !den))) return -1;
  for (int64_t i = 0; i < n; ++i) {
    ref[i] += x[i];
    den[i] += fabs(x[i]);
  }
  return 0;
}

/* ----------------------------------------------------------- threads ---- */

/* Thread count of the OpenMP loops above: n > 0 sets it, n <= 0 only asks.
 * Returns the count the next parallel loop will use (no arithmetic here;
 * the CPU-baseline timing reports it as its core count). */
#ifdef _OPENMP
#include <omp.h>
#endif
int orc_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ---------------------------------------------------------- compare ----- */

/*
 * Normalised error: e = max |got - ref| / den over n elements.  Where
 * den == 0 the element must be exactly zero (else e = +inf); a NaN or Inf
 * in got gives e = +inf.  *argmax receives the worst element (or -1).
 */
double orc_compare(int64_t n, const double *got, const double *ref, const double *den,
                   int64_t *argmax) {
  double worst = 0.0;
  int64_t at = -1;
  for (int64_t i = 0; i < n; ++i) {
    double e;
    if (!isfinite(got[i])) e = INFINITY;
    else if (den[i] == 0.0) e = (got[i] == 0.0) ? 0.0 : INFINITY;
    else e = fabs(got[i] - ref[i]) / den[i];
    if (e > worst) { worst = e; at = i; }
  }
  if (argmax) *argmax = at;
  return worst;
}
