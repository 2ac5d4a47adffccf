/* tess_oracle.c -- plain fp64 CPU oracle for the Tessera hot path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the benchmark's CPU
 * baseline leg, never by the GPU library. It is written for clarity: one loop per step of
 * the method, fp64 throughout, OpenMP only across independent atoms. Build with
 * -ffp-contract=off so every multiply and add rounds on its own (the wrap, key and
 * neighbour decisions below are specified operation by operation).
 *
 * Source of the method: "Ab Initio Accuracy Beyond the Cutoff: Distributed Message-Passing
 * Equivariant Attention at Tens-of-Millions-of-Atom Scale" (Tessera), abstract. The
 * abstract names the parts (space-filling-curve sort, three-level neighbour search with a
 * conservative skin, an equivariant message-passing Transformer, force back-propagation,
 * velocity-Verlet-style MD); it gives no equations. Each function below states the
 * concrete reading it implements. The backward pass follows the vector-Jacobian-product
 * formulation reviewed for REANN-MPI (pith.science verdict on arXiv 2505.06711,
 * key_machinery field): gradients flow back through each layer's neighbour sums.
 */
#include "tess_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define PI 3.14159265358979323846

int32_t tor_abi_version(void) { return 1; }

/* Threads the oracle's parallel loops use (OpenMP's current maximum). */
int32_t tor_num_threads(void) { return (int32_t)omp_get_max_threads(); }

/* ------------------------------------------------------------------------------------
 * Step 1 -- wrap (Tessera abstract: fixed shapes between rebuilds; periodic box).
 * Reading: t = x/L, f = floor(t), x_w = x - f*L with each operation rounded separately in
 * fp64, then rounded to fp32. The result lies in [0, L].
 * ---------------------------------------------------------------------------------- */
float tor_wrap1(float x, double L) {
  double t = (double)x / L;
  double f = floor(t);
  double p = f * L;
  double xw = (double)x - p;
  return (float)xw;
}

/* ------------------------------------------------------------------------------------
 * Step 2 -- Hilbert key (Tessera abstract: atoms sorted along a space-filling curve,
 * contrasted with Morton order). Reading: Skilling's transpose form of the Hilbert index
 * (J. Skilling, "Programming the Hilbert curve", AIP Conf. Proc. 707, 381 (2004)),
 * n = 3 axes, `bits` bits per axis, key bits read level by level with axis 0 first.
 * ---------------------------------------------------------------------------------- */
uint32_t tor_hilbert_key3(uint32_t x, uint32_t y, uint32_t z, int32_t bits) {
  uint32_t X[3] = {x, y, z};
  uint32_t top = 1u << (bits - 1);
  /* undo the excess work of the inverse transform, from the top level down */
  for (uint32_t Q = top; Q > 1; Q >>= 1) {
    uint32_t P = Q - 1;
    for (int i = 0; i < 3; i++) {
      if (X[i] & Q) {
        X[0] ^= P;
      } else {
        uint32_t t = (X[0] ^ X[i]) & P;
        X[0] ^= t;
        X[i] ^= t;
      }
    }
  }
  /* Gray encode */
  for (int i = 1; i < 3; i++) X[i] ^= X[i - 1];
  uint32_t t = 0;
  for (uint32_t Q = top; Q > 1; Q >>= 1)
    if (X[2] & Q) t ^= Q - 1;
  for (int i = 0; i < 3; i++) X[i] ^= t;
  /* read the transposed index out, most significant level first */
  uint32_t key = 0;
  for (int lev = bits - 1; lev >= 0; lev--)
    for (int i = 0; i < 3; i++) key = (key << 1) | ((X[i] >> lev) & 1u);
  return key;
}

/* Quantisation reading: S = 2^10 / L (IEEE division), q = clamp(floor(x_w * S), 0, 1023),
 * computed from the stored fp32 wrapped coordinate. */
static uint32_t quantise10(float xw, double L) {
  double S = (double)(1 << 10) / L;
  double v = floor((double)xw * S);
  if (v < 0.0) v = 0.0;
  if (v > 1023.0) v = 1023.0;
  return (uint32_t)v;
}

void tor_wrap_keys(int32_t n, const float box[3], const float* pos_in, float* pos_out,
                   uint32_t* keys) {
  for (int32_t i = 0; i < n; i++) {
    uint32_t q[3];
    for (int a = 0; a < 3; a++) {
      float w = tor_wrap1(pos_in[3 * i + a], (double)box[a]);
      pos_out[3 * i + a] = w;
      q[a] = quantise10(w, (double)box[a]);
    }
    keys[i] = tor_hilbert_key3(q[0], q[1], q[2], 10);
  }
}

/* Step 3a -- stable ascending sort of the keys (reading: ties keep pre-call index order).
 * Plain top-down merge sort on indices. */
static void merge_sort_idx(int32_t* a, int32_t* tmp, int32_t lo, int32_t hi, const uint32_t* k) {
  if (hi - lo < 2) return;
  int32_t mid = lo + (hi - lo) / 2;
  merge_sort_idx(a, tmp, lo, mid, k);
  merge_sort_idx(a, tmp, mid, hi, k);
  int32_t i = lo, j = mid, o = lo;
  while (i < mid && j < hi) tmp[o++] = (k[a[j]] < k[a[i]]) ? a[j++] : a[i++];
  while (i < mid) tmp[o++] = a[i++];
  while (j < hi) tmp[o++] = a[j++];
  memcpy(a + lo, tmp + lo, sizeof(int32_t) * (size_t)(hi - lo));
}

void tor_stable_argsort_u32(int32_t n, const uint32_t* keys, int32_t* perm) {
  int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  for (int32_t i = 0; i < n; i++) perm[i] = i;
  merge_sort_idx(perm, tmp, 0, n, keys);
  free(tmp);
}

/* ------------------------------------------------------------------------------------
 * Step 3b -- candidate pairs at r_cut + skin (Tessera abstract: a conservative neighbour
 * skin keeps the topology fixed between rebuilds). Reading: for sorted atoms i != j,
 * d = x_j - x_i in fp64 from the stored fp32 coordinates; minimum-image shift
 * s_a = -1 if d_a > L_a/2, +1 if d_a < -L_a/2, else 0; r = d + s*L; keep the pair iff
 * r.r < (r_cut+skin)^2 (strict), with r.r = (rx*rx + ry*ry) + rz*rz.
 * ---------------------------------------------------------------------------------- */
static int pair_test(const float* xi, const float* xj, const double L[3], double rcs2,
                     int* code, double* r2out) {
  int s[3];
  double r[3];
  for (int a = 0; a < 3; a++) {
    double d = (double)xj[a] - (double)xi[a];
    s[a] = (d > 0.5 * L[a]) ? -1 : ((d < -0.5 * L[a]) ? 1 : 0);
    r[a] = d + (double)s[a] * L[a];
  }
  double r2 = r[0] * r[0] + r[1] * r[1];
  r2 = r2 + r[2] * r[2];
  *code = 9 * (s[0] + 1) + 3 * (s[1] + 1) + (s[2] + 1);
  *r2out = r2;
  return r2 < rcs2;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Candidate j indices for atom i: all atoms (method 0) or those in the 27 cells around
 * i's cell (method 1), as a sorted, duplicate-free list. Cells are an enumeration aid
 * only; the decision is always pair_test. Cell width is kept >= (r_cut+skin)(1+1e-6). */
typedef struct {
  int nc[3];
  int32_t* start;
  int32_t* atoms;
} cells_t;

static void cells_build(cells_t* c, int32_t n, const float* pos, const double L[3], double rcs) {
  for (int a = 0; a < 3; a++) {
    int k = (int)floor(L[a] / (rcs * (1.0 + 1e-6)));
    c->nc[a] = k < 1 ? 1 : k;
  }
  int64_t ncell = (int64_t)c->nc[0] * c->nc[1] * c->nc[2];
  c->start = (int32_t*)calloc((size_t)ncell + 1, sizeof(int32_t));
  c->atoms = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t* cid = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  for (int32_t i = 0; i < n; i++) {
    int q[3];
    for (int a = 0; a < 3; a++) {
      int v = (int)floor((double)pos[3 * i + a] * (double)c->nc[a] / L[a]);
      q[a] = v < 0 ? 0 : (v >= c->nc[a] ? c->nc[a] - 1 : v);
    }
    cid[i] = (q[0] * c->nc[1] + q[1]) * c->nc[2] + q[2];
    c->start[cid[i] + 1]++;
  }
  for (int64_t k = 0; k < ncell; k++) c->start[k + 1] += c->start[k];
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)(ncell + 1));
  memcpy(fill, c->start, sizeof(int32_t) * (size_t)(ncell + 1));
  for (int32_t i = 0; i < n; i++) c->atoms[fill[cid[i]]++] = i;
  free(fill);
  free(cid);
}

static int32_t cells_candidates(const cells_t* c, const float* pos, const double L[3],
                                int32_t i, int32_t* out) {
  int q[3];
  for (int a = 0; a < 3; a++) {
    int v = (int)floor((double)pos[3 * i + a] * (double)c->nc[a] / L[a]);
    q[a] = v < 0 ? 0 : (v >= c->nc[a] ? c->nc[a] - 1 : v);
  }
  int32_t cnt = 0;
  int seen[27];
  int nseen = 0;
  for (int dx = -1; dx <= 1; dx++)
    for (int dy = -1; dy <= 1; dy++)
      for (int dz = -1; dz <= 1; dz++) {
        int cx = ((q[0] + dx) % c->nc[0] + c->nc[0]) % c->nc[0];
        int cy = ((q[1] + dy) % c->nc[1] + c->nc[1]) % c->nc[1];
        int cz = ((q[2] + dz) % c->nc[2] + c->nc[2]) % c->nc[2];
        int cell = (cx * c->nc[1] + cy) * c->nc[2] + cz;
        int dup = 0;
        for (int s = 0; s < nseen; s++) dup |= (seen[s] == cell);
        if (dup) continue;
        seen[nseen++] = cell;
        for (int32_t k = c->start[cell]; k < c->start[cell + 1]; k++) out[cnt++] = c->atoms[k];
      }
  qsort(out, (size_t)cnt, sizeof(int32_t), cmp_i32);
  return cnt;
}

int32_t tor_neighbors(int32_t n, const float box[3], const float* pos, float r_cut,
                      float skin, int32_t method, int64_t cap, int32_t* row_ptr,
                      uint32_t* col_shift, int64_t* n_edges) {
  double L[3] = {(double)box[0], (double)box[1], (double)box[2]};
  double rcs = (double)r_cut + (double)skin;
  double rcs2 = rcs * rcs;
  for (int a = 0; a < 3; a++)
    if (!(L[a] > 2.0 * rcs)) return TOR_ERR_BOX;
  cells_t cells = {{0, 0, 0}, NULL, NULL};
  int use_cells = (method == 1);
  if (use_cells) cells_build(&cells, n, pos, L, rcs);
  int32_t* counts = (int32_t*)calloc((size_t)n + 1, sizeof(int32_t));
  /* pass 1: count */
#pragma omp parallel
  {
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
#pragma omp for schedule(dynamic, 64)
    for (int32_t i = 0; i < n; i++) {
      int32_t nc = 0;
      if (use_cells) {
        nc = cells_candidates(&cells, pos, L, i, cand);
      } else {
        for (int32_t j = 0; j < n; j++) cand[nc++] = j;
      }
      int32_t cnt = 0;
      for (int32_t k = 0; k < nc; k++) {
        int32_t j = cand[k];
        if (j == i) continue;
        int code;
        double r2;
        cnt += pair_test(&pos[3 * i], &pos[3 * j], L, rcs2, &code, &r2);
      }
      counts[i] = cnt;
    }
    free(cand);
  }
  row_ptr[0] = 0;
  int64_t tot = 0;
  for (int32_t i = 0; i < n; i++) {
    tot += counts[i];
    row_ptr[i + 1] = (int32_t)(tot < 2147483647 ? tot : 2147483647);
  }
  *n_edges = tot;
  if (tot > cap || col_shift == NULL) {
    free(counts);
    if (use_cells) { free(cells.start); free(cells.atoms); }
    return tot > cap ? TOR_ERR_CAPACITY : TOR_OK;
  }
  /* pass 2: fill, rows ascending in j */
#pragma omp parallel
  {
    int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
#pragma omp for schedule(dynamic, 64)
    for (int32_t i = 0; i < n; i++) {
      int32_t nc = 0;
      if (use_cells) {
        nc = cells_candidates(&cells, pos, L, i, cand);
      } else {
        for (int32_t j = 0; j < n; j++) cand[nc++] = j;
      }
      int64_t o = row_ptr[i];
      for (int32_t k = 0; k < nc; k++) {
        int32_t j = cand[k];
        if (j == i) continue;
        int code;
        double r2;
        if (pair_test(&pos[3 * i], &pos[3 * j], L, rcs2, &code, &r2))
          col_shift[o++] = (uint32_t)j | ((uint32_t)code << 27);
      }
    }
    free(cand);
  }
  free(counts);
  if (use_cells) { free(cells.start); free(cells.atoms); }
  return TOR_OK;
}

int64_t tor_flagged_pairs(int32_t n, const float box[3], const float* pos, float r_cut,
                          float skin, double band, int64_t cap, int32_t* fi, int32_t* fj) {
  double L[3] = {(double)box[0], (double)box[1], (double)box[2]};
  double rcs = (double)r_cut + (double)skin;
  cells_t cells = {{0, 0, 0}, NULL, NULL};
  /* cells sized for rcs + band so that no pair inside the band is missed */
  cells_build(&cells, n, pos, L, rcs + 2.0 * band);
  int64_t cnt = 0;
  int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  for (int32_t i = 0; i < n; i++) {
    int32_t nc = cells_candidates(&cells, pos, L, i, cand);
    for (int32_t k = 0; k < nc; k++) {
      int32_t j = cand[k];
      if (j <= i) continue;
      int code;
      double r2;
      pair_test(&pos[3 * i], &pos[3 * j], L, 0.0, &code, &r2);
      if (fabs(sqrt(r2) - rcs) < band) {
        if (cnt < cap) { fi[cnt] = i; fj[cnt] = j; }
        cnt++;
      }
    }
  }
  free(cand);
  free(cells.start);
  free(cells.atoms);
  return cnt;
}

int32_t tor_build_neighbors(int32_t n, const float box[3], float r_cut, float skin,
                            float* pos, int32_t* species, double* vel, int32_t* perm,
                            uint32_t* keys_sorted, int64_t cap, int32_t* row_ptr,
                            uint32_t* col_shift, int64_t* n_edges) {
  double rcs = (double)r_cut + (double)skin;
  for (int a = 0; a < 3; a++)
    if (!((double)box[a] > 2.0 * rcs)) return TOR_ERR_BOX;
  float* w = (float*)malloc(sizeof(float) * 3 * (size_t)(n > 0 ? n : 1));
  uint32_t* keys = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(n > 0 ? n : 1));
  tor_wrap_keys(n, box, pos, w, keys);
  tor_stable_argsort_u32(n, keys, perm);
  int32_t* sp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  double* v = vel ? (double*)malloc(sizeof(double) * 3 * (size_t)(n > 0 ? n : 1)) : NULL;
  for (int32_t k = 0; k < n; k++) {
    int32_t o = perm[k];
    for (int a = 0; a < 3; a++) pos[3 * k + a] = w[3 * o + a];
    sp[k] = species[o];
    if (keys_sorted) keys_sorted[k] = keys[o];
    if (v)
      for (int a = 0; a < 3; a++) v[3 * k + a] = vel[3 * o + a];
  }
  memcpy(species, sp, sizeof(int32_t) * (size_t)n);
  if (v) { memcpy(vel, v, sizeof(double) * 3 * (size_t)n); free(v); }
  free(sp);
  free(w);
  free(keys);
  return tor_neighbors(n, box, pos, r_cut, skin, n > 5000 ? 1 : 0, cap, row_ptr, col_shift,
                       n_edges);
}

/* ------------------------------------------------------------------------------------
 * Step 6 -- real spherical harmonics on a unit vector, component normalisation
 * (sum_m Y_lm^2 = 2l+1). Reading (the pages only say "equivariant"):
 *   Y0 = 1;  Y1 = sqrt3 (x, y, z);
 *   Y2 = (sqrt15 xy, sqrt15 yz, sqrt5/2 (3z^2-1), sqrt15 xz, sqrt15/2 (x^2-y^2)).
 * Component order within the feature axis: offset l^2 + m.
 * ---------------------------------------------------------------------------------- */
void tor_sph(int32_t l_max, const double nv[3], double* Y) {
  double x = nv[0], y = nv[1], z = nv[2];
  Y[0] = 1.0;
  if (l_max >= 1) {
    double s3 = sqrt(3.0);
    Y[1] = s3 * x; Y[2] = s3 * y; Y[3] = s3 * z;
  }
  if (l_max >= 2) {
    double s15 = sqrt(15.0), s5 = sqrt(5.0);
    Y[4] = s15 * x * y;
    Y[5] = s15 * y * z;
    Y[6] = 0.5 * s5 * (3.0 * z * z - 1.0);
    Y[7] = s15 * x * z;
    Y[8] = 0.5 * s15 * (x * x - y * y);
  }
}

/* Jacobian dY_d/dn_a of the polynomial forms above, J[d][a]. */
static void sph_jac(int l_max, const double nv[3], double J[9][3]) {
  double x = nv[0], y = nv[1], z = nv[2];
  memset(J, 0, sizeof(double) * 27);
  if (l_max >= 1) {
    double s3 = sqrt(3.0);
    J[1][0] = s3; J[2][1] = s3; J[3][2] = s3;
  }
  if (l_max >= 2) {
    double s15 = sqrt(15.0), s5 = sqrt(5.0);
    J[4][0] = s15 * y; J[4][1] = s15 * x;
    J[5][1] = s15 * z; J[5][2] = s15 * y;
    J[6][2] = 3.0 * s5 * z;
    J[7][0] = s15 * z; J[7][2] = s15 * x;
    J[8][0] = s15 * x; J[8][1] = -s15 * y;
  }
}

/* ------------------------------------------------------------------------------------
 * Step 7 -- coupling paths and tensors. Reading: paths (l1, l2, l3) with every l <= l_max,
 * |l1-l2| <= l3 <= l1+l2 and l1+l2+l3 even, in lexicographic order; l1 is the sender
 * feature degree, l2 the harmonic degree, l3 the output degree. The coupling tensor is the
 * real Gaunt integral G[m1][m2][m3] = (1/4pi) * integral of Y_l1m1 Y_l2m2 Y_l3m3 over the
 * sphere, scaled to Frobenius norm sqrt(2 l3 + 1).
 * ---------------------------------------------------------------------------------- */
int32_t tor_n_paths(int32_t l_max) {
  int32_t p = 0;
  for (int l1 = 0; l1 <= l_max; l1++)
    for (int l2 = 0; l2 <= l_max; l2++)
      for (int l3 = 0; l3 <= l_max; l3++)
        if (l3 >= abs(l1 - l2) && l3 <= l1 + l2 && ((l1 + l2 + l3) % 2 == 0)) p++;
  return p;
}

void tor_paths(int32_t l_max, int32_t* o1, int32_t* o2, int32_t* o3) {
  int32_t p = 0;
  for (int l1 = 0; l1 <= l_max; l1++)
    for (int l2 = 0; l2 <= l_max; l2++)
      for (int l3 = 0; l3 <= l_max; l3++)
        if (l3 >= abs(l1 - l2) && l3 <= l1 + l2 && ((l1 + l2 + l3) % 2 == 0)) {
          o1[p] = l1; o2[p] = l2; o3[p] = l3;
          p++;
        }
}

/* Gauss-Legendre nodes/weights on [-1,1] by Newton iteration on P_n. */
static void gauss_legendre(int n, double* xs, double* ws) {
  for (int i = 0; i < n; i++) {
    double x = cos(PI * (i + 0.75) / (n + 0.5));
    for (int it = 0; it < 100; it++) {
      double p0 = 1.0, p1 = x;
      for (int k = 2; k <= n; k++) {
        double p2 = ((2.0 * k - 1.0) * x * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      double dp = n * (x * p1 - p0) / (x * x - 1.0);
      double dx = p1 / dp;
      x -= dx;
      if (fabs(dx) < 1e-16) break;
    }
    double p0 = 1.0, p1 = x;
    for (int k = 2; k <= n; k++) {
      double p2 = ((2.0 * k - 1.0) * x * p1 - (k - 1.0) * p0) / k;
      p0 = p1;
      p1 = p2;
    }
    double dp = n * (x * p1 - p0) / (x * x - 1.0);
    xs[i] = x;
    ws[i] = 2.0 / ((1.0 - x * x) * dp * dp);
  }
}

/* cg[p][m1][m2][m3] with each index padded to 5. The quadrature (8 Gauss-Legendre nodes in
 * cos(theta) times 16 equally spaced phi) is exact for the degree-6 integrands here. */
void tor_coupling(int32_t l_max, double* cg) {
  int32_t P = tor_n_paths(l_max);
  int32_t l1s[16], l2s[16], l3s[16];
  tor_paths(l_max, l1s, l2s, l3s);
  memset(cg, 0, sizeof(double) * (size_t)P * 125);
  double xs[8], ws[8];
  gauss_legendre(8, xs, ws);
  for (int it = 0; it < 8; it++) {
    for (int ip = 0; ip < 16; ip++) {
      double ct = xs[it], st = sqrt(1.0 - ct * ct), ph = 2.0 * PI * ip / 16.0;
      double nv[3] = {st * cos(ph), st * sin(ph), ct};
      double Y[9];
      tor_sph(2, nv, Y);
      double wq = ws[it] * (2.0 * PI / 16.0) / (4.0 * PI);
      for (int p = 0; p < P; p++) {
        int a = l1s[p], b = l2s[p], c = l3s[p];
        for (int m1 = 0; m1 < 2 * a + 1; m1++)
          for (int m2 = 0; m2 < 2 * b + 1; m2++)
            for (int m3 = 0; m3 < 2 * c + 1; m3++)
              cg[((p * 5 + m1) * 5 + m2) * 5 + m3] +=
                  wq * Y[a * a + m1] * Y[b * b + m2] * Y[c * c + m3];
      }
    }
  }
  for (int p = 0; p < P; p++) {
    double f = 0.0;
    for (int k = 0; k < 125; k++) f += cg[p * 125 + k] * cg[p * 125 + k];
    double sc = sqrt(2.0 * l3s[p] + 1.0) / sqrt(f);
    for (int k = 0; k < 125; k++) cg[p * 125 + k] *= sc;
  }
}

/* ------------------------------------------------------------------------------------
 * Step 14 -- weights: one fp32 blob, row-major [out][in] (y = W x):
 *   Emb[S][C]; per layer W_q[C][C], W_k[C][C], W1[R][K], W2[P][R], W_lin0[C(1+Lmax)][C],
 *   W_lin^l[C][C] for l = 1..Lmax; then w_E[C].
 * ---------------------------------------------------------------------------------- */
typedef struct {
  const double *Wq, *Wk, *W1, *W2, *W0, *Wl[3];
} layer_w;

typedef struct {
  int S, T, C, Lm, H, K, R, P, D, dh;
  double rc;
  double* blob;
  const double* emb;
  layer_w lw[16];
  const double* wE;
  double cg[16 * 125];
  int l1[16], l2[16], l3[16];
} model_t;

int64_t tor_weights_count(const tor_model* m) {
  int64_t C = m->channels, R = m->radial_hidden, K = m->n_rbf, Lm = m->l_max;
  int64_t P = tor_n_paths(m->l_max);
  int64_t per = 2 * C * C + R * K + P * R + C * (1 + Lm) * C + Lm * C * C;
  return (int64_t)m->n_species * C + m->n_layers * per + C;
}

static int model_init(model_t* M, const tor_model* m, const float* weights) {
  if (m->l_max < 0 || m->l_max > 2 || m->n_layers < 1 || m->n_layers > 16 || m->channels < 1 ||
      m->n_heads < 1 || m->channels % m->n_heads || m->n_rbf < 1 || m->radial_hidden < 1 ||
      m->n_species < 1 || !(m->r_cut > 0.0f) || m->channels > 256 || m->n_heads > 64 ||
      m->n_rbf > 64 || m->radial_hidden > 256)
    return TOR_ERR_ARG;
  M->S = m->n_species; M->T = m->n_layers; M->C = m->channels; M->Lm = m->l_max;
  M->H = m->n_heads; M->K = m->n_rbf; M->R = m->radial_hidden;
  M->P = tor_n_paths(m->l_max);
  M->D = (m->l_max + 1) * (m->l_max + 1);
  M->dh = M->C / M->H;
  M->rc = (double)m->r_cut;
  int64_t nw = tor_weights_count(m);
  M->blob = (double*)malloc(sizeof(double) * (size_t)nw);
  for (int64_t k = 0; k < nw; k++) M->blob[k] = (double)weights[k];
  const double* p = M->blob;
  int C = M->C;
  M->emb = p; p += (size_t)M->S * C;
  for (int t = 0; t < M->T; t++) {
    layer_w* L = &M->lw[t];
    L->Wq = p; p += C * C;
    L->Wk = p; p += C * C;
    L->W1 = p; p += M->R * M->K;
    L->W2 = p; p += M->P * M->R;
    L->W0 = p; p += C * (1 + M->Lm) * C;
    for (int l = 1; l <= M->Lm; l++) { L->Wl[l] = p; p += C * C; }
  }
  M->wE = p;
  tor_coupling(M->Lm, M->cg);
  tor_paths(M->Lm, M->l1, M->l2, M->l3);
  return TOR_OK;
}

static double sigm(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu(double z) { return z * sigm(z); }
static double silu_d(double z) { double s = sigm(z); return s * (1.0 + z * (1.0 - s)); }

/* Step 6 -- radial functions. Reading: cosine envelope u(r) = (cos(pi r/rc)+1)/2 for
 * r < rc (0 beyond), Bessel basis b_k(r) = u(r) sqrt(2/rc) sin(k pi r/rc)/r, k = 1..K;
 * derivatives returned alongside. */
static void radial(const model_t* M, double r, double* u, double* du, double* b, double* db) {
  double rc = M->rc;
  if (r >= rc) {
    *u = 0.0; *du = 0.0;
    for (int k = 0; k < M->K; k++) { b[k] = 0.0; db[k] = 0.0; }
    return;
  }
  *u = 0.5 * (cos(PI * r / rc) + 1.0);
  *du = -0.5 * (PI / rc) * sin(PI * r / rc);
  double pref = sqrt(2.0 / rc);
  for (int k = 0; k < M->K; k++) {
    double a = (k + 1) * PI / rc;
    double B = pref * sin(a * r) / r;
    double dB = pref * (a * cos(a * r) / r - sin(a * r) / (r * r));
    b[k] = (*u) * B;
    db[k] = (*du) * B + (*u) * dB;
  }
}

/* K^p[(l3,m3)][(l1,m1)] = sum_m2 C^p[m1][m2][m3] Y_(l2,m2); A = sum_p w_p K^p (D x D). */
static void coupling_matrix(const model_t* M, const double* w, const double* Y, double* A) {
  int D = M->D;
  memset(A, 0, sizeof(double) * (size_t)D * D);
  for (int p = 0; p < M->P; p++) {
    int a = M->l1[p], b = M->l2[p], c = M->l3[p];
    for (int m3 = 0; m3 < 2 * c + 1; m3++)
      for (int m1 = 0; m1 < 2 * a + 1; m1++) {
        double k = 0.0;
        for (int m2 = 0; m2 < 2 * b + 1; m2++)
          k += M->cg[((p * 5 + m1) * 5 + m2) * 5 + m3] * Y[b * b + m2];
        A[(c * c + m3) * D + (a * a + m1)] += w[p] * k;
      }
  }
}

/* Per-layer state kept from the forward pass for the backward pass. */
typedef struct {
  double *h;      /* input features h^t [N][C][D] */
  double *q, *k;  /* [N][C] */
  double *Mx, *Z; /* softmax max and normaliser [N][H] */
  double *m;      /* aggregated messages [N][C][D] */
  double *y0;     /* [N][C] */
  double *gate;   /* [N][Lm][C] */
  double *yl;     /* W_lin^l m^l for l>=1: [N][C][D] (l=0 slot unused) */
} layer_state;

/* Geometry of edge (dest i <- source j, shift code): r = x_j - x_i + s*L. */
static void edge_vec(const double* pos, const double L[3], int32_t i, int32_t j, int code,
                     double rv[3]) {
  int s[3] = {code / 9 - 1, (code / 3) % 3 - 1, code % 3 - 1};
  for (int a = 0; a < 3; a++) rv[a] = pos[3 * j + a] - pos[3 * i + a] + (double)s[a] * L[a];
}

/* Step 8 -- radial MLP (reading: one weight per path, shared by all channels and heads,
 * no biases): z = W1 b, a = SiLU(z), w = W2 a. */
static void radial_mlp(const model_t* M, const layer_w* Lw, const double* b, double* z,
                       double* w) {
  for (int r = 0; r < M->R; r++) {
    double s = 0.0;
    for (int k = 0; k < M->K; k++) s += Lw->W1[r * M->K + k] * b[k];
    z[r] = s;
  }
  for (int p = 0; p < M->P; p++) {
    double s = 0.0;
    for (int r = 0; r < M->R; r++) s += Lw->W2[p * M->R + r] * silu(z[r]);
    w[p] = s;
  }
}

/* ------------------------------------------------------------------------------------
 * One layer, forward (Tessera title: message-passing equivariant attention).
 * Reading of the layer:
 *   q_i = W_q h_i^0, k_j = W_k h_j^0; heads split channels into contiguous groups of
 *   d = C/H; logit s_e^h = (1/sqrt d) sum_{c in h} q_ic k_jc.
 *   Per destination i over edges with r < rc: M^h = max s, w_e^h = u(r) exp(s - M),
 *   Z^h = sum w, alpha = w/Z (0 when Z = 0); the envelope inside the weight keeps E
 *   continuous as pairs cross rc. The softmax is local to each row (no global
 *   normalisation, which would break a halo decomposition -- REANN-MPI verdict,
 *   falsifier field).
 *   m_ic = sum_e alpha_e^h(c) A_e h_jc  (A_e from the coupling tensors and harmonics).
 *   Update: y0 = W_lin0[0:C] m^0, gates g^l = W_lin0[lC:(l+1)C] m^0,
 *   h^0 += SiLU(y0), h^(l,m) += sigmoid(g^l) * (W_lin^l m^(l,m)).
 * ---------------------------------------------------------------------------------- */
static void layer_forward(const model_t* M, int t, int32_t n, const double L[3],
                          const double* pos, const int32_t* row_ptr, const uint32_t* col,
                          layer_state* st, double* hout) {
  const layer_w* Lw = &M->lw[t];
  int C = M->C, D = M->D, H = M->H, dh = M->dh;
  double isd = 1.0 / sqrt((double)dh);
  const double* h = st->h;
#pragma omp parallel for schedule(static)
  for (int32_t i = 0; i < n; i++) {
    for (int c = 0; c < C; c++) {
      double sq = 0.0, sk = 0.0;
      for (int k = 0; k < C; k++) {
        sq += Lw->Wq[c * C + k] * h[((size_t)i * C + k) * D];
        sk += Lw->Wk[c * C + k] * h[((size_t)i * C + k) * D];
      }
      st->q[(size_t)i * C + c] = sq;
      st->k[(size_t)i * C + c] = sk;
    }
  }
#pragma omp parallel
  {
    double b[64], db[64], z[256], w[16], Y[9], A[81], rv[3], nv[3];
#pragma omp for schedule(dynamic, 32)
    for (int32_t i = 0; i < n; i++) {
      double Mx[64], Z[64];
      for (int hh = 0; hh < H; hh++) { Mx[hh] = -INFINITY; Z[hh] = 0.0; }
      double* mi = &st->m[(size_t)i * C * D];
      memset(mi, 0, sizeof(double) * (size_t)C * D);
      /* pass over the row: maxima of the logits over edges inside rc */
      for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; e++) {
        int32_t j = (int32_t)(col[e] & 0x7FFFFFFu);
        int code = (int)(col[e] >> 27);
        edge_vec(pos, L, i, j, code, rv);
        double r = sqrt(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]);
        if (r >= M->rc) continue;
        for (int hh = 0; hh < H; hh++) {
          double s = 0.0;
          for (int c = hh * dh; c < (hh + 1) * dh; c++)
            s += st->q[(size_t)i * C + c] * st->k[(size_t)j * C + c];
          s *= isd;
          if (s > Mx[hh]) Mx[hh] = s;
        }
      }
      /* normaliser */
      for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; e++) {
        int32_t j = (int32_t)(col[e] & 0x7FFFFFFu);
        int code = (int)(col[e] >> 27);
        edge_vec(pos, L, i, j, code, rv);
        double r = sqrt(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]);
        if (r >= M->rc) continue;
        double u, du;
        radial(M, r, &u, &du, b, db);
        for (int hh = 0; hh < H; hh++) {
          double s = 0.0;
          for (int c = hh * dh; c < (hh + 1) * dh; c++)
            s += st->q[(size_t)i * C + c] * st->k[(size_t)j * C + c];
          s *= isd;
          Z[hh] += u * exp(s - Mx[hh]);
        }
      }
      /* aggregation */
      for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; e++) {
        int32_t j = (int32_t)(col[e] & 0x7FFFFFFu);
        int code = (int)(col[e] >> 27);
        edge_vec(pos, L, i, j, code, rv);
        double r = sqrt(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]);
        if (r >= M->rc) continue;
        double u, du;
        radial(M, r, &u, &du, b, db);
        for (int a = 0; a < 3; a++) nv[a] = rv[a] / r;
        tor_sph(M->Lm, nv, Y);
        radial_mlp(M, Lw, b, z, w);
        coupling_matrix(M, w, Y, A);
        for (int hh = 0; hh < H; hh++) {
          double s = 0.0;
          for (int c = hh * dh; c < (hh + 1) * dh; c++)
            s += st->q[(size_t)i * C + c] * st->k[(size_t)j * C + c];
          s *= isd;
          double alpha = Z[hh] > 0.0 ? u * exp(s - Mx[hh]) / Z[hh] : 0.0;
          for (int c = hh * dh; c < (hh + 1) * dh; c++) {
            const double* hj = &h[((size_t)j * C + c) * D];
            for (int d3 = 0; d3 < D; d3++) {
              double v = 0.0;
              for (int d1 = 0; d1 < D; d1++) v += A[d3 * D + d1] * hj[d1];
              mi[c * D + d3] += alpha * v;
            }
          }
        }
      }
      for (int hh = 0; hh < H; hh++) {
        st->Mx[(size_t)i * H + hh] = Mx[hh];
        st->Z[(size_t)i * H + hh] = Z[hh];
      }
    }
  }
  /* node update */
#pragma omp parallel for schedule(static)
  for (int32_t i = 0; i < n; i++) {
    const double* mi = &st->m[(size_t)i * C * D];
    const double* hi = &h[(size_t)i * C * D];
    double* ho = &hout[(size_t)i * C * D];
    for (int c = 0; c < C; c++) {
      double y = 0.0;
      for (int k = 0; k < C; k++) y += Lw->W0[c * C + k] * mi[k * D];
      st->y0[(size_t)i * C + c] = y;
      ho[c * D] = hi[c * D] + silu(y);
    }
    for (int l = 1; l <= M->Lm; l++) {
      for (int c = 0; c < C; c++) {
        double g = 0.0;
        for (int k = 0; k < C; k++) g += Lw->W0[(l * C + c) * C + k] * mi[k * D];
        st->gate[((size_t)i * M->Lm + (l - 1)) * C + c] = g;
        for (int mm = 0; mm < 2 * l + 1; mm++) {
          int d = l * l + mm;
          double y = 0.0;
          for (int k = 0; k < C; k++) y += Lw->Wl[l][c * C + k] * mi[k * D + d];
          st->yl[((size_t)i * C + c) * D + d] = y;
          ho[c * D + d] = hi[c * D + d] + sigm(g) * y;
        }
      }
    }
  }
}

/* ------------------------------------------------------------------------------------
 * One edge, backward. Given the destination adjoint mbar_i (dE/dm_i), returns the
 * logit adjoint sbar^h, the position-gradient g = dE/d(r_e) (r_e = x_j - x_i + sL), and,
 * if hbar_c is non-NULL, the contribution A^T (alpha mbar_ic) to dE/dh_jc for every c.
 * Chain (step 12 of the reading):
 *   v_c = A h_jc; abar^h = sum_{c in h} <mbar_ic, v_c>; D_i^h = <mbar_i^h, m_i^h>;
 *   sbar^h = alpha^h (abar^h - D^h); ubar = sum_h p^h (abar^h - D^h), p = exp(s-M)/Z;
 *   Abar = sum_c alpha^h(c) mbar_ic (x) h_jc; wbar_p = <Abar, K^p>;
 *   Ybar_m2 = sum_p w_p sum_{m1,m3} C^p[m1][m2][m3] Abar[(l3m3),(l1m1)];
 *   zbar = (W2^T wbar) * SiLU'(z); bbar = W1^T zbar;
 *   dE/dr = sum_k bbar_k b_k'(r) + ubar u'(r);
 *   g = dE/dr n + (I - n n^T)/r J_Y(n)^T Ybar.
 * ---------------------------------------------------------------------------------- */
static int edge_backward(const model_t* M, int t, const layer_state* st, const double* mbar,
                         const double* Dst, const double* pos, const double L[3], int32_t i,
                         int32_t j, int code, double* sbar, double g[3], double* hbar_c) {
  const layer_w* Lw = &M->lw[t];
  int C = M->C, D = M->D, H = M->H, dh = M->dh, P = M->P;
  double isd = 1.0 / sqrt((double)dh);
  double rv[3], nv[3], b[64], db[64], z[256], w[16], Y[9], A[81], Ab[81];
  edge_vec(pos, L, i, j, code, rv);
  double r = sqrt(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]);
  if (r >= M->rc) return 0;
  double u, du;
  radial(M, r, &u, &du, b, db);
  for (int a = 0; a < 3; a++) nv[a] = rv[a] / r;
  tor_sph(M->Lm, nv, Y);
  radial_mlp(M, Lw, b, z, w);
  coupling_matrix(M, w, Y, A);
  const double* h = st->h;
  const double* mb = &mbar[(size_t)i * C * D];
  memset(Ab, 0, sizeof(Ab));
  double ubar = 0.0;
  for (int hh = 0; hh < H; hh++) {
    double s = 0.0;
    for (int c = hh * dh; c < (hh + 1) * dh; c++)
      s += st->q[(size_t)i * C + c] * st->k[(size_t)j * C + c];
    s *= isd;
    double Zi = st->Z[(size_t)i * H + hh];
    double p = Zi > 0.0 ? exp(s - st->Mx[(size_t)i * H + hh]) / Zi : 0.0;
    double alpha = u * p;
    double abar = 0.0;
    for (int c = hh * dh; c < (hh + 1) * dh; c++) {
      const double* hj = &h[((size_t)j * C + c) * D];
      for (int d3 = 0; d3 < D; d3++) {
        double v = 0.0;
        for (int d1 = 0; d1 < D; d1++) v += A[d3 * D + d1] * hj[d1];
        abar += mb[c * D + d3] * v;
      }
      for (int d3 = 0; d3 < D; d3++)
        for (int d1 = 0; d1 < D; d1++) Ab[d3 * D + d1] += alpha * mb[c * D + d3] * hj[d1];
      if (hbar_c) {
        for (int d1 = 0; d1 < D; d1++) {
          double v = 0.0;
          for (int d3 = 0; d3 < D; d3++) v += A[d3 * D + d1] * alpha * mb[c * D + d3];
          hbar_c[c * D + d1] = v;
        }
      }
    }
    double diff = abar - Dst[(size_t)i * H + hh];
    sbar[hh] = alpha * diff;
    ubar += p * diff;
  }
  /* coupling adjoints */
  double wbar[16], Ybar[9];
  memset(wbar, 0, sizeof(wbar));
  memset(Ybar, 0, sizeof(Ybar));
  for (int p = 0; p < P; p++) {
    int a = M->l1[p], bb = M->l2[p], c = M->l3[p];
    for (int m3 = 0; m3 < 2 * c + 1; m3++)
      for (int m1 = 0; m1 < 2 * a + 1; m1++) {
        double abar = Ab[(c * c + m3) * D + (a * a + m1)];
        for (int m2 = 0; m2 < 2 * bb + 1; m2++) {
          double cg = M->cg[((p * 5 + m1) * 5 + m2) * 5 + m3];
          wbar[p] += abar * cg * Y[bb * bb + m2];
          Ybar[bb * bb + m2] += w[p] * cg * abar;
        }
      }
  }
  /* radial MLP adjoint */
  double bbar[64];
  for (int k = 0; k < M->K; k++) bbar[k] = 0.0;
  for (int rr = 0; rr < M->R; rr++) {
    double abar = 0.0;
    for (int p = 0; p < P; p++) abar += Lw->W2[p * M->R + rr] * wbar[p];
    double zbar = abar * silu_d(z[rr]);
    for (int k = 0; k < M->K; k++) bbar[k] += Lw->W1[rr * M->K + k] * zbar;
  }
  double dEdr = ubar * du;
  for (int k = 0; k < M->K; k++) dEdr += bbar[k] * db[k];
  double J[9][3];
  sph_jac(M->Lm, nv, J);
  double gy[3] = {0.0, 0.0, 0.0};
  for (int d = 0; d < D; d++)
    for (int a = 0; a < 3; a++) gy[a] += J[d][a] * Ybar[d];
  double ng = nv[0] * gy[0] + nv[1] * gy[1] + nv[2] * gy[2];
  for (int a = 0; a < 3; a++) g[a] = dEdr * nv[a] + (gy[a] - ng * nv[a]) / r;
  return 1;
}

/* Backward of one layer. gbar = dE/dh^(t+1) in, hbar = dE/dh^t out; dEdx accumulates. */
static void layer_backward(const model_t* M, int t, int32_t n, const double L[3],
                           const double* pos, const int32_t* row_ptr, const uint32_t* col,
                           const layer_state* st, const double* gbar, double* hbar,
                           double* dEdx) {
  const layer_w* Lw = &M->lw[t];
  int C = M->C, D = M->D, H = M->H, dh = M->dh, Lm = M->Lm;
  double isd = 1.0 / sqrt((double)dh);
  double* mbar = (double*)calloc((size_t)n * C * D, sizeof(double));
  double* Dst = (double*)calloc((size_t)n * H, sizeof(double));
  double* qbar = (double*)calloc((size_t)n * C, sizeof(double));
  double* kbar = (double*)calloc((size_t)n * C, sizeof(double));
  /* update adjoint; the residual passes gbar straight to hbar */
#pragma omp parallel for schedule(static)
  for (int32_t i = 0; i < n; i++) {
    const double* gb = &gbar[(size_t)i * C * D];
    double* hb = &hbar[(size_t)i * C * D];
    double* mb = &mbar[(size_t)i * C * D];
    memcpy(hb, gb, sizeof(double) * (size_t)C * D);
    double ybar0[256], gateb[3][256];
    for (int c = 0; c < C; c++) ybar0[c] = gb[c * D] * silu_d(st->y0[(size_t)i * C + c]);
    for (int l = 1; l <= Lm; l++)
      for (int c = 0; c < C; c++) {
        double g = st->gate[((size_t)i * Lm + (l - 1)) * C + c];
        double sg = sigm(g), acc = 0.0;
        for (int mm = 0; mm < 2 * l + 1; mm++) {
          int d = l * l + mm;
          acc += gb[c * D + d] * st->yl[((size_t)i * C + c) * D + d];
        }
        gateb[l - 1][c] = acc * sg * (1.0 - sg);
      }
    for (int k = 0; k < C; k++) {
      double s = 0.0;
      for (int c = 0; c < C; c++) s += Lw->W0[c * C + k] * ybar0[c];
      for (int l = 1; l <= Lm; l++)
        for (int c = 0; c < C; c++) s += Lw->W0[(l * C + c) * C + k] * gateb[l - 1][c];
      mb[k * D] = s;
      for (int l = 1; l <= Lm; l++)
        for (int mm = 0; mm < 2 * l + 1; mm++) {
          int d = l * l + mm;
          double s2 = 0.0;
          for (int c = 0; c < C; c++) {
            double sg = sigm(st->gate[((size_t)i * Lm + (l - 1)) * C + c]);
            s2 += Lw->Wl[l][c * C + k] * gb[c * D + d] * sg;
          }
          mb[k * D + d] = s2;
        }
    }
    for (int hh = 0; hh < H; hh++) {
      double s = 0.0;
      for (int c = hh * dh; c < (hh + 1) * dh; c++)
        for (int d = 0; d < D; d++) s += mb[c * D + d] * st->m[((size_t)i * C + c) * D + d];
      Dst[(size_t)i * H + hh] = s;
    }
  }
  /* destination side of every edge: q adjoint and -g on x_i */
#pragma omp parallel for schedule(dynamic, 32)
  for (int32_t i = 0; i < n; i++) {
    double sbar[64], g[3];
    for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; e++) {
      int32_t j = (int32_t)(col[e] & 0x7FFFFFFu);
      int code = (int)(col[e] >> 27);
      if (!edge_backward(M, t, st, mbar, Dst, pos, L, i, j, code, sbar, g, NULL)) continue;
      for (int hh = 0; hh < H; hh++)
        for (int c = hh * dh; c < (hh + 1) * dh; c++)
          qbar[(size_t)i * C + c] += sbar[hh] * st->k[(size_t)j * C + c] * isd;
      for (int a = 0; a < 3; a++) dEdx[3 * i + a] -= g[a];
    }
  }
  /* source side: every edge (i <- j, s) appears in row j as (j <- i, -s); sum over them
   * the value adjoint, the k adjoint and +g on x_j. */
#pragma omp parallel
  {
    double* hb_c = (double*)malloc(sizeof(double) * (size_t)C * D);
#pragma omp for schedule(dynamic, 32)
    for (int32_t jj = 0; jj < n; jj++) {
      double sbar[64], g[3];
      for (int32_t e = row_ptr[jj]; e < row_ptr[jj + 1]; e++) {
        int32_t i = (int32_t)(col[e] & 0x7FFFFFFu);
        int code = 26 - (int)(col[e] >> 27); /* shift of the forward edge (i <- jj) */
        if (!edge_backward(M, t, st, mbar, Dst, pos, L, i, jj, code, sbar, g, hb_c)) continue;
        for (int k = 0; k < C * D; k++) hbar[(size_t)jj * C * D + k] += hb_c[k];
        for (int hh = 0; hh < H; hh++)
          for (int c = hh * dh; c < (hh + 1) * dh; c++)
            kbar[(size_t)jj * C + c] += sbar[hh] * st->q[(size_t)i * C + c] * isd;
        for (int a = 0; a < 3; a++) dEdx[3 * jj + a] += g[a];
      }
    }
    free(hb_c);
  }
  /* logit projections back to the scalar features */
#pragma omp parallel for schedule(static)
  for (int32_t i = 0; i < n; i++) {
    for (int k = 0; k < C; k++) {
      double s = 0.0;
      for (int c = 0; c < C; c++)
        s += Lw->Wq[c * C + k] * qbar[(size_t)i * C + c] + Lw->Wk[c * C + k] * kbar[(size_t)i * C + c];
      hbar[((size_t)i * C + k) * D] += s;
    }
  }
  free(mbar);
  free(Dst);
  free(qbar);
  free(kbar);
}

/* ------------------------------------------------------------------------------------
 * Energy and forces. Steps 5 (embedding: h^0,l=0 = Emb[z_i], higher l zero), the T layers,
 * step 11 (E_i = w_E . h_i^(T,0), E = sum_i E_i) and step 12 (F = -dE/dx by the VJP chain).
 * ---------------------------------------------------------------------------------- */
int32_t tor_energy_forces(const tor_model* mdesc, const float* weights, int32_t n,
                          const float box[3], const double* pos, const int32_t* species,
                          const int32_t* row_ptr, const uint32_t* col, double* energy,
                          double* e_atom, double* forces, double* feats) {
  model_t* M = (model_t*)calloc(1, sizeof(model_t));
  int rc = model_init(M, mdesc, weights);
  if (rc != TOR_OK) { free(M); return rc; }
  for (int32_t i = 0; i < n; i++)
    if (species[i] < 0 || species[i] >= M->S) { free(M->blob); free(M); return TOR_ERR_SPECIES; }
  double L[3] = {(double)box[0], (double)box[1], (double)box[2]};
  int C = M->C, D = M->D, H = M->H, T = M->T, Lm = M->Lm;
  size_t nf = (size_t)n * C * D;
  layer_state* st = (layer_state*)calloc((size_t)T, sizeof(layer_state));
  double** hs = (double**)calloc((size_t)T + 1, sizeof(double*));
  for (int t = 0; t <= T; t++) hs[t] = (double*)calloc(nf > 0 ? nf : 1, sizeof(double));
  for (int32_t i = 0; i < n; i++)
    for (int c = 0; c < C; c++) hs[0][((size_t)i * C + c) * D] = M->emb[species[i] * C + c];
  for (int t = 0; t < T; t++) {
    st[t].h = hs[t];
    st[t].q = (double*)calloc((size_t)n * C + 1, sizeof(double));
    st[t].k = (double*)calloc((size_t)n * C + 1, sizeof(double));
    st[t].Mx = (double*)calloc((size_t)n * H + 1, sizeof(double));
    st[t].Z = (double*)calloc((size_t)n * H + 1, sizeof(double));
    st[t].m = (double*)calloc(nf + 1, sizeof(double));
    st[t].y0 = (double*)calloc((size_t)n * C + 1, sizeof(double));
    st[t].gate = (double*)calloc((size_t)n * C * (Lm > 0 ? Lm : 1) + 1, sizeof(double));
    st[t].yl = (double*)calloc(nf + 1, sizeof(double));
    layer_forward(M, t, n, L, pos, row_ptr, col, &st[t], hs[t + 1]);
  }
  double E = 0.0;
  for (int32_t i = 0; i < n; i++) {
    double ei = 0.0;
    for (int c = 0; c < C; c++) ei += M->wE[c] * hs[T][((size_t)i * C + c) * D];
    if (e_atom) e_atom[i] = ei;
    E += ei;
  }
  *energy = E;
  if (feats) memcpy(feats, hs[T], sizeof(double) * nf);
  if (forces) {
    double* gbar = (double*)calloc(nf + 1, sizeof(double));
    double* hbar = (double*)calloc(nf + 1, sizeof(double));
    double* dEdx = (double*)calloc((size_t)n * 3 + 1, sizeof(double));
    for (int32_t i = 0; i < n; i++)
      for (int c = 0; c < C; c++) gbar[((size_t)i * C + c) * D] = M->wE[c];
    for (int t = T - 1; t >= 0; t--) {
      layer_backward(M, t, n, L, pos, row_ptr, col, &st[t], gbar, hbar, dEdx);
      double* tmp = gbar; gbar = hbar; hbar = tmp;
    }
    for (int32_t k = 0; k < 3 * n; k++) forces[k] = -dEdx[k];
    free(gbar); free(hbar); free(dEdx);
  }
  for (int t = 0; t < T; t++) {
    free(st[t].q); free(st[t].k); free(st[t].Mx); free(st[t].Z); free(st[t].m);
    free(st[t].y0); free(st[t].gate); free(st[t].yl);
  }
  for (int t = 0; t <= T; t++) free(hs[t]);
  free(hs); free(st); free(M->blob); free(M);
  return TOR_OK;
}

/* ------------------------------------------------------------------------------------
 * Step 13 -- MD between rebuilds (Tessera abstract: each rebuild interval replays with a
 * fixed neighbour topology; NVE runs). Reading: velocity-Verlet with a = F/m * 9.648533e-3
 * (eV/A/amu to A/fs^2). Loop, for s = 0..n_steps-1:
 *   if s % rebuild_every == 0: rebuild (positions wrapped and rounded to their stored fp32
 *     values, sorted; velocities, forces, species and perm_accum permuted along; the
 *     reference positions for the skin check reset); if s == 0 and forces are not valid,
 *     compute them;
 *   v += dt/2 a; x += dt v (not re-wrapped); flag if any |x - x_ref| > skin/2;
 *   F = -dE/dx (epot_trace[s] = E); v += dt/2 a;
 *   with thermostat 1, v *= lambda (Berendsen coupling, below);
 *   ke_trace[s] = kinetic energy; rmin_trace[s] = shortest pair distance below r_cut.
 * After an interval whose flag is set the call stops and returns TOR_ERR_SKIN.
 *
 * NVT and monitors (Tessera abstract: NVT runs of the capsid with no anomalously close
 * pairs; the pages name no thermostat). Reading: the weak-coupling thermostat of
 * Berendsen et al. (J. Chem. Phys. 81, 3684, 1984) on the instantaneous kinetic temperature
 * T = 2 KE / (3 N k_B), 3N degrees of freedom, KE = sum m v^2 / 2 (amu A^2/fs^2 converted to
 * eV by 1/9.648533e-3): after the second half-kick each velocity is multiplied by
 * lambda = sqrt(1 + (dt/tau)(t_target/T - 1)) (lambda = 1 when T = 0; tau >= dt keeps the
 * radicand >= 0). The shortest pair distance is taken over the pairs of the current list
 * with r < r_cut at the positions where the forces were evaluated (+inf when none).
 * ---------------------------------------------------------------------------------- */
#define KB_EV_PER_K 8.617333262e-5

static double kinetic_energy(int32_t n, const double* vel, const int32_t* species,
                             const double* mass_by_species, double conv) {
  double s = 0.0;
  for (int32_t k = 0; k < n; k++) {
    double v2 = 0.0;
    for (int a = 0; a < 3; a++) v2 += vel[3 * k + a] * vel[3 * k + a];
    s += mass_by_species[species[k]] * v2;
  }
  return 0.5 * s / conv;
}

static double min_pair_distance(int32_t n, const double* pos, const double L[3],
                                const int32_t* row_ptr, const uint32_t* col, double rc) {
  double best = INFINITY;
  for (int32_t i = 0; i < n; i++)
    for (int32_t e = row_ptr[i]; e < row_ptr[i + 1]; e++) {
      double rv[3];
      edge_vec(pos, L, i, (int32_t)(col[e] & 0x7FFFFFFu), (int)(col[e] >> 27), rv);
      double r = sqrt((rv[0] * rv[0] + rv[1] * rv[1]) + rv[2] * rv[2]);
      if (r < rc && r < best) best = r;
    }
  return best;
}

int32_t tor_md_steps(const tor_model* m, const float* weights, int32_t n, const float box[3],
                     float r_cut, float skin, double* pos, double* vel, int32_t* species,
                     const double* mass_by_species, double dt_fs, int32_t n_steps,
                     int32_t rebuild_every, int32_t* perm_accum, double* forces,
                     int32_t forces_valid, double* epot_trace, int64_t cap, int32_t thermostat,
                     double t_target_K, double tau_fs, double* ke_trace, double* rmin_trace) {
  const double conv = 9.648533e-3;
  const double L[3] = {(double)box[0], (double)box[1], (double)box[2]};
  if (thermostat != 0 && (thermostat != 1 || !(tau_fs >= dt_fs) || !(t_target_K >= 0.0)))
    return TOR_ERR_ARG;
  int32_t* row_ptr = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
  uint32_t* col = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(cap > 0 ? cap : 1));
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  float* pf = (float*)malloc(sizeof(float) * 3 * (size_t)(n > 0 ? n : 1));
  double* ref = (double*)malloc(sizeof(double) * 3 * (size_t)(n > 0 ? n : 1));
  double* tmp = (double*)malloc(sizeof(double) * 3 * (size_t)(n > 0 ? n : 1));
  int32_t* itmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t status = TOR_OK;
  int flag = 0;
  double half_skin2 = 0.25 * (double)skin * (double)skin;
  for (int32_t s = 0; s < n_steps && status == TOR_OK; s++) {
    if (s % rebuild_every == 0) {
      if (flag) { status = TOR_ERR_SKIN; break; }
      for (int32_t k = 0; k < 3 * n; k++) pf[k] = (float)pos[k];
      int64_t ne = 0;
      int32_t rc = tor_build_neighbors(n, box, r_cut, skin, pf, species, vel, perm, NULL, cap,
                                       row_ptr, col, &ne);
      if (rc != TOR_OK) { status = rc; break; }
      for (int32_t k = 0; k < 3 * n; k++) pos[k] = (double)pf[k];
      for (int32_t k = 0; k < n; k++) itmp[k] = perm_accum[perm[k]];
      memcpy(perm_accum, itmp, sizeof(int32_t) * (size_t)n);
      if (forces_valid || s > 0) {
        for (int32_t k = 0; k < n; k++)
          for (int a = 0; a < 3; a++) tmp[3 * k + a] = forces[3 * perm[k] + a];
        memcpy(forces, tmp, sizeof(double) * 3 * (size_t)n);
      } else {
        double E;
        rc = tor_energy_forces(m, weights, n, box, pos, species, row_ptr, col, &E, NULL, forces,
                               NULL);
        if (rc != TOR_OK) { status = rc; break; }
      }
      memcpy(ref, pos, sizeof(double) * 3 * (size_t)n);
    }
    for (int32_t k = 0; k < n; k++) {
      double im = conv / mass_by_species[species[k]];
      double d2 = 0.0;
      for (int a = 0; a < 3; a++) {
        vel[3 * k + a] += 0.5 * dt_fs * forces[3 * k + a] * im;
        pos[3 * k + a] += dt_fs * vel[3 * k + a];
        double d = pos[3 * k + a] - ref[3 * k + a];
        d2 += d * d;
      }
      if (d2 > half_skin2) flag = 1;
    }
    double E;
    int32_t rc = tor_energy_forces(m, weights, n, box, pos, species, row_ptr, col, &E, NULL,
                                   forces, NULL);
    if (rc != TOR_OK) { status = rc; break; }
    if (epot_trace) epot_trace[s] = E;
    for (int32_t k = 0; k < n; k++) {
      double im = conv / mass_by_species[species[k]];
      for (int a = 0; a < 3; a++) vel[3 * k + a] += 0.5 * dt_fs * forces[3 * k + a] * im;
    }
    if (thermostat == 1) {
      double T = 2.0 * kinetic_energy(n, vel, species, mass_by_species, conv) /
                 (3.0 * (double)n * KB_EV_PER_K);
      double lam = T > 0.0 ? sqrt(1.0 + (dt_fs / tau_fs) * (t_target_K / T - 1.0)) : 1.0;
      for (int32_t k = 0; k < 3 * n; k++) vel[k] *= lam;
    }
    if (ke_trace) ke_trace[s] = kinetic_energy(n, vel, species, mass_by_species, conv);
    if (rmin_trace) rmin_trace[s] = min_pair_distance(n, pos, L, row_ptr, col, (double)r_cut);
  }
  if (status == TOR_OK && flag) status = TOR_ERR_SKIN;
  free(row_ptr); free(col); free(perm); free(pf); free(ref); free(tmp); free(itmp);
  return status;
}
