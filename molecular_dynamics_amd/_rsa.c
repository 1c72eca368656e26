/* Random sequential addition (RSA) for the seeded synthetic boxes.
 *
 * Input generator only: it holds none of the potential's arithmetic.  The
 * caller (inputs.py) draws every random number with numpy and passes a pool of
 * candidate molecules; this routine walks the pool in order and accepts a
 * candidate iff every one of its atoms is at least `min_sep` (minimum image in
 * a cubic periodic box of side L) from every atom already accepted.  Atoms of
 * one molecule are not tested against each other.  Returns the number of
 * candidates consumed; stops once `n_target` molecules are accepted.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

typedef struct {
  double L, cs, min_sep2;
  int ng, maxc;
  int32_t* cell;   /* [ng^3][maxc], -1 = empty */
  double* pos;     /* accepted atoms [cap][3] */
  int64_t n_atoms, cap;
} rsa_grid;

static int cell_of(const rsa_grid* g, double x) {
  int c = (int)floor(x / g->cs);
  if (c < 0) c += g->ng;
  if (c >= g->ng) c -= g->ng;
  if (c < 0 || c >= g->ng) c = 0;
  return c;
}

static double wrap(double x, double L) {
  x = x - L * floor(x / L);
  if (x >= L) x -= L;
  if (x < 0) x += L;
  return x;
}

static int conflicts(const rsa_grid* g, const double* p) {
  int cx = cell_of(g, p[0]), cy = cell_of(g, p[1]), cz = cell_of(g, p[2]);
  for (int dx = -1; dx <= 1; ++dx)
    for (int dy = -1; dy <= 1; ++dy)
      for (int dz = -1; dz <= 1; ++dz) {
        int ix = (cx + dx + g->ng) % g->ng, iy = (cy + dy + g->ng) % g->ng, iz = (cz + dz + g->ng) % g->ng;
        const int32_t* c = g->cell + ((int64_t)(ix * g->ng + iy) * g->ng + iz) * g->maxc;
        for (int s = 0; s < g->maxc; ++s) {
          if (c[s] < 0) break;
          const double* q = g->pos + 3 * (int64_t)c[s];
          double d2 = 0;
          for (int a = 0; a < 3; ++a) {
            double d = q[a] - p[a];
            d -= g->L * nearbyint(d / g->L);
            d2 += d * d;
          }
          if (d2 < g->min_sep2) return 1;
        }
      }
  return 0;
}

static int insert(rsa_grid* g, const double* p) {
  int cx = cell_of(g, p[0]), cy = cell_of(g, p[1]), cz = cell_of(g, p[2]);
  int32_t* c = g->cell + ((int64_t)(cx * g->ng + cy) * g->ng + cz) * g->maxc;
  for (int s = 0; s < g->maxc; ++s)
    if (c[s] < 0) {
      c[s] = (int32_t)g->n_atoms;
      for (int a = 0; a < 3; ++a) g->pos[3 * g->n_atoms + a] = p[a];
      g->n_atoms++;
      return 0;
    }
  return -1;
}

void* rsa_create(double L, double min_sep, int64_t cap) {
  rsa_grid* g = (rsa_grid*)calloc(1, sizeof(rsa_grid));
  g->L = L;
  g->ng = (int)floor(L / min_sep);
  if (g->ng < 3) g->ng = 3;
  g->cs = L / g->ng;
  g->min_sep2 = min_sep * min_sep;
  g->maxc = 16;
  int64_t ncell = (int64_t)g->ng * g->ng * g->ng;
  g->cell = (int32_t*)malloc(sizeof(int32_t) * ncell * g->maxc);
  for (int64_t i = 0; i < ncell * g->maxc; ++i) g->cell[i] = -1;
  g->pos = (double*)malloc(sizeof(double) * 3 * cap);
  g->cap = cap;
  g->n_atoms = 0;
  return g;
}

void rsa_destroy(void* h) {
  rsa_grid* g = (rsa_grid*)h;
  free(g->cell);
  free(g->pos);
  free(g);
}

/* cand: [n_cand][atoms_per][3]; accepted molecules are appended to `out`
 * ([.][atoms_per][3], wrapped into [0,L)).  Returns candidates consumed. */
int64_t rsa_add(void* h, const double* cand, int64_t n_cand, int atoms_per, int64_t n_target,
                double* out, int64_t* n_accepted) {
  rsa_grid* g = (rsa_grid*)h;
  int64_t k = 0;
  double p[64 * 3];
  for (; k < n_cand && *n_accepted < n_target; ++k) {
    int bad = 0;
    for (int a = 0; a < atoms_per && !bad; ++a) {
      for (int d = 0; d < 3; ++d) p[3 * a + d] = wrap(cand[(k * atoms_per + a) * 3 + d], g->L);
      bad = conflicts(g, p + 3 * a);
    }
    if (bad) continue;
    if (g->n_atoms + atoms_per > g->cap) return -1;
    for (int a = 0; a < atoms_per; ++a)
      if (insert(g, p + 3 * a) != 0) return -2;
    for (int a = 0; a < 3 * atoms_per; ++a) out[*n_accepted * 3 * atoms_per + a] = p[a];
    (*n_accepted)++;
  }
  return k;
}
