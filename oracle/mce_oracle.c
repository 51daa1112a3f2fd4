/*
 * Oracle for maximal clique enumeration: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU reference that the GPU engine is checked
 * against. Only the tests, the smoke check and the bench's CPU-baseline leg may
 * load it; the product path never does. It shares no code, header or table with
 * the GPU library.
 *
 * What it computes follows "Parallelizing Maximal Clique Enumeration on GPUs"
 * (arxiv 2212.01473v2):
 *   - section 2.1: G is simple and undirected; a clique C is maximal when no
 *     vertex outside C is adjacent to all of C; the answer is all such cliques;
 *   - section 2.3, Algorithm 2: Bron-Kerbosch with pivoting, with Tomita's rule
 *     (pivot = vertex of P u X with the most neighbours in P);
 *   - section 2.4, Algorithm 3: one independent first-level subtree per vertex
 *     v_i, P = later neighbours, X = earlier neighbours, under a degeneracy order;
 *   - section 3.2, Algorithm 4 (oracle_mce_l2): one independent second-level
 *     subtree per edge {v_i, v_j}, P = common neighbours after both, X = common
 *     neighbours before the later one; vertices of degree 0 are cliques of
 *     their own (the pages' loop over edges does not meet them);
 *   - section 2.4 "Induced Subgraphs": each subtree only needs the edges between
 *     P u X and P, so sets are bitsets over the root's neighbourhood.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - ordering: round-synchronous k-core peel. At level k every alive vertex of
 *     current degree <= k is removed in one round; k rises to the smallest alive
 *     degree when a round finds none. Vertex v is "earlier" than u iff
 *     (round(v), v) < (round(u), u). Any degeneracy order gives the same cliques.
 *   - pivot ties: smallest vertex id. Branch order: ascending vertex id.
 *   - result: count, histogram by clique size, and the order-free set hash
 *       h(c)        = mix64(c + G)
 *       hash(C)     = mix64(sum_{c in C} h(c) + |C| * G)        (mod 2^64)
 *       set hash    = sum over maximal cliques C of hash(C)     (mod 2^64)
 *     with G = 0x9E3779B97F4A7C15 and mix64 the SplitMix64 finaliser
 *     (Steele, Lea and Flood, OOPSLA 2014).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

/* error classes reported by oracle_validate */
#define OV_ROWPTR 1   /* row_ptr[0] != 0, row_ptr[n] != nnz, or a row that runs backwards */
#define OV_RANGE 2    /* a column id outside [0, n) */
#define OV_LOOP 4     /* an edge (v, v) */
#define OV_ORDER 8    /* a row that is not strictly ascending (unsorted or duplicate) */
#define OV_ASYM 16    /* u in N(v) but v not in N(u) */

uint64_t oracle_mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

/* hash of one clique given as a list of vertex ids (any order) */
uint64_t oracle_clique_hash(int k, const int32_t *ids) {
  uint64_t s = 0;
  for (int i = 0; i < k; i++) s += oracle_mix64((uint64_t)(int64_t)ids[i] + GOLDEN);
  return oracle_mix64(s + (uint64_t)k * GOLDEN);
}

/* does the sorted row ci[lo..hi) contain key? plain binary search */
static int row_has(const int32_t *ci, int64_t lo, int64_t hi, int32_t key) {
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (ci[mid] == key) return 1;
    if (ci[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  return 0;
}

static int adjacent(const int32_t *rp, const int32_t *ci, int32_t u, int32_t v) {
  return row_has(ci, rp[u], rp[u + 1], v);
}

/* Checks that (rp, ci) is a simple undirected graph in CSR form. Returns 0 or a
   bitmask of the OV_* classes found. */
int oracle_validate(int32_t n, int64_t nnz, const int32_t *rp, const int32_t *ci) {
  int err = 0;
  if (n < 0 || nnz < 0) return OV_ROWPTR;
  if (rp[0] != 0 || (int64_t)rp[n] != nnz) err |= OV_ROWPTR;
  for (int32_t v = 0; v < n; v++)
    if (rp[v] > rp[v + 1] || rp[v] < 0 || (int64_t)rp[v + 1] > nnz) err |= OV_ROWPTR;
  if (err) return err;
  for (int32_t v = 0; v < n; v++) {
    for (int64_t e = rp[v]; e < rp[v + 1]; e++) {
      int32_t u = ci[e];
      if (u < 0 || u >= n) { err |= OV_RANGE; continue; }
      if (u == v) err |= OV_LOOP;
      if (e + 1 < rp[v + 1] && ci[e + 1] <= u) err |= OV_ORDER;
    }
  }
  if (err & (OV_RANGE | OV_ORDER)) return err;   /* binary search needs sorted, in-range rows */
  for (int32_t v = 0; v < n; v++)
    for (int64_t e = rp[v]; e < rp[v + 1]; e++)
      if (!adjacent(rp, ci, ci[e], v)) err |= OV_ASYM;
  return err;
}

/* Round-synchronous k-core peel (the ordering reading above).
   core[v] = k at v's removal (the core number), rnd[v] = round index.
   Returns d = max core number (0 for n == 0), or -1 on allocation failure. */
int32_t oracle_peel(int32_t n, const int32_t *rp, const int32_t *ci, int32_t *core, int32_t *rnd) {
  if (n == 0) return 0;
  int32_t *deg = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  int32_t *alive = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  int32_t *front = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
  char *gone = (char *)calloc((size_t)n, 1);
  if (!deg || !alive || !front || !gone) { free(deg); free(alive); free(front); free(gone); return -1; }
  int32_t na = n, k = 0, round = 0, d = 0;
  for (int32_t v = 0; v < n; v++) { deg[v] = rp[v + 1] - rp[v]; alive[v] = v; }
  while (na > 0) {
    int32_t nf = 0;
    for (int32_t i = 0; i < na; i++)
      if (deg[alive[i]] <= k) front[nf++] = alive[i];
    if (nf == 0) {             /* nothing at this level: raise k to the smallest alive degree */
      int32_t mn = deg[alive[0]];
      for (int32_t i = 1; i < na; i++) if (deg[alive[i]] < mn) mn = deg[alive[i]];
      k = mn;
      continue;
    }
    for (int32_t i = 0; i < nf; i++) {
      int32_t v = front[i];
      gone[v] = 1; core[v] = k; rnd[v] = round;
    }
    if (k > d) d = k;
    for (int32_t i = 0; i < nf; i++) {
      int32_t v = front[i];
      for (int64_t e = rp[v]; e < rp[v + 1]; e++)
        if (!gone[ci[e]]) deg[ci[e]]--;
    }
    round++;
    int32_t w = 0;
    for (int32_t i = 0; i < na; i++) if (!gone[alive[i]]) alive[w++] = alive[i];
    na = w;
  }
  free(deg); free(alive); free(front); free(gone);
  return d;
}

/* ------------------------------------------------------------------ search */
typedef struct {
  /* graph */
  const int32_t *rp, *ci;
  const int32_t *rnd;
  /* current root: L = P_root (ascending id) followed by X_root (ascending id) */
  int32_t root, p, nl;
  int32_t *L;
  int wp, wl;          /* words in a P-bitset and in an L-bitset */
  uint64_t *adjP;      /* nl rows of wp words: bit b of row a iff L[a] ~ L[b], b < p */
  uint64_t *colL;      /* p rows of wl words:  bit a of row b iff L[a] ~ L[b] */
  uint64_t *arena;     /* per-level P and X copies */
  int32_t *R;          /* clique under construction (global ids, R[0] = root) */
  int32_t *tmp;
  /* output */
  uint64_t count, hash;
  uint64_t *hist;
  int32_t hist_cap, hist_len;
  int64_t nodes, budget;
  int over_budget, hist_overflow;
} search;

static int later(const int32_t *rnd, int32_t u, int32_t v) {  /* is u after v in the order? */
  return rnd[u] > rnd[v] || (rnd[u] == rnd[v] && u > v);
}

static int popc(uint64_t x) { return __builtin_popcountll(x); }

static void report(search *s, int k) {
  s->count++;
  s->hash += oracle_clique_hash(k, s->R);
  if (k < s->hist_cap) s->hist[k]++;
  else s->hist_overflow = 1;
  if (k + 1 > s->hist_len) s->hist_len = k + 1;
}

/* Algorithm 2 with Tomita's pivot. P is a p-bit set of P_root members; X is an
   nl-bit set over L (its low p bits are X members from P_root, the rest from
   X_root). depth = |R| - 1. Level `depth` owns arena record depth: P, X, cand. */
static void bkt(search *s, int depth) {
  if (s->over_budget) return;
  s->nodes++;
  if (s->budget > 0 && s->nodes > s->budget) { s->over_budget = 1; return; }
  int wp = s->wp, wl = s->wl;
  uint64_t *P = s->arena + (size_t)depth * (2 * wp + wl);
  uint64_t *X = P + wp;
  uint64_t *cand = X + wl;
  int pe = 1, xe = 1;
  for (int w = 0; w < wp; w++) if (P[w]) { pe = 0; break; }
  for (int w = 0; w < wl; w++) if (X[w]) { xe = 0; break; }
  if (pe) {
    if (xe) report(s, depth + 1);     /* Algorithm 2, lines 2-3 */
    return;                           /* P empty: no branch can follow */
  }
  /* pivot: u in P u X maximising |P n N(u)|, ties to the smallest vertex id */
  int32_t best = -1, bestc = -1;
  for (int w = 0; w < wl; w++) {
    uint64_t bits = X[w] | (w < wp ? P[w] : 0);
    while (bits) {
      int32_t u = w * 64 + __builtin_ctzll(bits);
      bits &= bits - 1;
      const uint64_t *row = s->adjP + (size_t)u * wp;
      int c = 0;
      for (int i = 0; i < wp; i++) c += popc(P[i] & row[i]);
      if (c > bestc || (c == bestc && s->L[u] < s->L[best])) { best = u; bestc = c; }
    }
  }
  /* branches: v in P - N(pivot), ascending id */
  const uint64_t *prow = s->adjP + (size_t)best * wp;
  for (int w = 0; w < wp; w++) cand[w] = P[w] & ~prow[w];
  uint64_t *Pn = s->arena + (size_t)(depth + 1) * (2 * wp + wl);
  uint64_t *Xn = Pn + wp;
  for (int w = 0; w < wp; w++) {
    while (cand[w]) {
      int b = __builtin_ctzll(cand[w]);
      cand[w] &= cand[w] - 1;
      int32_t v = w * 64 + b;
      const uint64_t *vrow = s->adjP + (size_t)v * wp;
      const uint64_t *vcol = s->colL + (size_t)v * wl;
      for (int i = 0; i < wp; i++) Pn[i] = P[i] & vrow[i];      /* P n N(v) */
      for (int i = 0; i < wl; i++) Xn[i] = X[i] & vcol[i];      /* X n N(v) */
      s->R[depth + 1] = s->L[v];
      bkt(s, depth + 1);
      P[w] &= ~(1ULL << b);          /* P = P - {v} */
      X[w] |= (1ULL << b);           /* X = X u {v} */
      if (s->over_budget) return;
    }
  }
}

/* Builds the root's neighbourhood bitsets and runs Algorithm 2 from ({root}, P, X). */
static int run_root(search *s, int32_t root, int32_t *loc) {
  const int32_t *rp = s->rp, *ci = s->ci;
  int64_t lo = rp[root], hi = rp[root + 1];
  int32_t deg = (int32_t)(hi - lo);
  int32_t p = 0;
  for (int64_t e = lo; e < hi; e++) if (later(s->rnd, ci[e], root)) s->L[p++] = ci[e];
  int32_t nx = p;
  for (int64_t e = lo; e < hi; e++) if (!later(s->rnd, ci[e], root)) s->L[nx++] = ci[e];
  s->root = root; s->p = p; s->nl = deg;
  int wp = (p + 63) / 64; if (wp == 0) wp = 1;
  int wl = (deg + 63) / 64; if (wl == 0) wl = 1;
  s->wp = wp; s->wl = wl;
  s->adjP = (uint64_t *)calloc((size_t)(deg > 0 ? deg : 1) * wp, sizeof(uint64_t));
  s->colL = (uint64_t *)calloc((size_t)(p > 0 ? p : 1) * wl, sizeof(uint64_t));
  s->arena = (uint64_t *)calloc((size_t)(p + 2) * (2 * wp + wl), sizeof(uint64_t));
  if (!s->adjP || !s->colL || !s->arena) { free(s->adjP); free(s->colL); free(s->arena); return -1; }
  for (int32_t a = 0; a < deg; a++) loc[s->L[a]] = a;
  /* adjP[a] bit b  <=>  L[b] in N(L[a]) with b < p */
  for (int32_t a = 0; a < deg; a++) {
    int32_t x = s->L[a];
    for (int64_t e = rp[x]; e < rp[x + 1]; e++) {
      int32_t b = loc[ci[e]];
      if (b >= 0 && b < p) s->adjP[(size_t)a * wp + (b >> 6)] |= 1ULL << (b & 63);
    }
  }
  for (int32_t a = 0; a < deg; a++)
    for (int32_t b = 0; b < p; b++)
      if ((s->adjP[(size_t)a * wp + (b >> 6)] >> (b & 63)) & 1)
        s->colL[(size_t)b * wl + (a >> 6)] |= 1ULL << (a & 63);
  for (int32_t a = 0; a < deg; a++) loc[s->L[a]] = -1;
  uint64_t *P = s->arena, *X = s->arena + wp;
  for (int32_t b = 0; b < p; b++) P[b >> 6] |= 1ULL << (b & 63);
  for (int32_t a = p; a < deg; a++) X[a >> 6] |= 1ULL << (a & 63);
  s->R[0] = root;
  bkt(s, 0);
  free(s->adjP); free(s->colL); free(s->arena);
  s->adjP = s->colL = s->arena = NULL;
  return 0;
}

/* Enumerates the maximal cliques whose earliest vertex (in the peel order) is in
   roots[0..nroots) (roots == NULL: every vertex, i.e. the whole graph).
   node_budget > 0 stops after that many search-tree nodes and returns 1.
   hist must hold hist_cap entries; hist_len receives max clique size + 1 (0 if none).
   Returns 0 on success, 1 over budget, 2 hist_cap too small, -1 on allocation failure,
   -2 for a root id out of range. */
int oracle_mce(int32_t n, const int32_t *rp, const int32_t *ci, const int32_t *rnd,
               const int32_t *roots, int32_t nroots, int64_t node_budget,
               uint64_t *count, uint64_t *hash, uint64_t *hist, int32_t hist_cap,
               int32_t *hist_len, int64_t *nodes) {
  search s;
  memset(&s, 0, sizeof(s));
  s.rp = rp; s.ci = ci; s.rnd = rnd;
  s.hist = hist; s.hist_cap = hist_cap; s.budget = node_budget;
  for (int32_t i = 0; i < hist_cap; i++) hist[i] = 0;
  int32_t maxdeg = 0;
  for (int32_t v = 0; v < n; v++) if (rp[v + 1] - rp[v] > maxdeg) maxdeg = rp[v + 1] - rp[v];
  s.L = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxdeg + 1));
  s.R = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxdeg + 2));
  int32_t *loc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!s.L || !s.R || !loc) { free(s.L); free(s.R); free(loc); return -1; }
  for (int32_t v = 0; v < n; v++) loc[v] = -1;
  int rc = 0;
  int32_t cnt = roots ? nroots : n;
  for (int32_t i = 0; i < cnt && !s.over_budget; i++) {
    int32_t r = roots ? roots[i] : i;
    if (r < 0 || r >= n) { rc = -2; break; }
    if (run_root(&s, r, loc) != 0) { rc = -1; break; }
  }
  free(s.L); free(s.R); free(loc);
  *count = s.count; *hash = s.hash; *hist_len = s.hist_len;
  if (nodes) *nodes = s.nodes;
  if (rc) return rc;
  if (s.over_budget) return 1;
  if (s.hist_overflow) return 2;
  return 0;
}

/* Algorithm 2 from (R0, P, X) for explicit id lists: P (ascending id) and X
   (ascending id) become L = P then X, bitsets as in run_root. R0 holds k0 ids. */
static int run_sub(search *s, const int32_t *R0, int k0, int32_t p, int32_t x, int32_t *loc) {
  const int32_t *rp = s->rp, *ci = s->ci;
  int32_t nl = p + x;
  s->p = p; s->nl = nl;
  int wp = (p + 63) / 64; if (wp == 0) wp = 1;
  int wl = (nl + 63) / 64; if (wl == 0) wl = 1;
  s->wp = wp; s->wl = wl;
  s->adjP = (uint64_t *)calloc((size_t)(nl > 0 ? nl : 1) * wp, sizeof(uint64_t));
  s->colL = (uint64_t *)calloc((size_t)(p > 0 ? p : 1) * wl, sizeof(uint64_t));
  s->arena = (uint64_t *)calloc((size_t)(p + k0 + 1) * (2 * wp + wl), sizeof(uint64_t));
  if (!s->adjP || !s->colL || !s->arena) { free(s->adjP); free(s->colL); free(s->arena); return -1; }
  for (int32_t a = 0; a < nl; a++) loc[s->L[a]] = a;
  for (int32_t a = 0; a < nl; a++) {
    int32_t v = s->L[a];
    for (int64_t e = rp[v]; e < rp[v + 1]; e++) {
      int32_t b = loc[ci[e]];
      if (b >= 0 && b < p) s->adjP[(size_t)a * wp + (b >> 6)] |= 1ULL << (b & 63);
    }
  }
  for (int32_t a = 0; a < nl; a++)
    for (int32_t b = 0; b < p; b++)
      if ((s->adjP[(size_t)a * wp + (b >> 6)] >> (b & 63)) & 1)
        s->colL[(size_t)b * wl + (a >> 6)] |= 1ULL << (a & 63);
  for (int32_t a = 0; a < nl; a++) loc[s->L[a]] = -1;
  uint64_t *P = s->arena + (size_t)(k0 - 1) * (2 * wp + wl), *X = P + wp;
  for (int32_t b = 0; b < p; b++) P[b >> 6] |= 1ULL << (b & 63);
  for (int32_t a = p; a < nl; a++) X[a >> 6] |= 1ULL << (a & 63);
  for (int i = 0; i < k0; i++) s->R[i] = R0[i];
  bkt(s, k0 - 1);
  free(s->adjP); free(s->colL); free(s->arena);
  s->adjP = s->colL = s->arena = NULL;
  return 0;
}

/* The same cliques as oracle_mce (those whose earliest vertex is a listed root,
   or all), found through independent second-level subtrees (Algorithm 4): a root
   of degree 0 is a clique of its own; every edge {r, w} with w after r starts
   Algorithm 2 from R = {r, w}, P = the common neighbours after w and X = the
   common neighbours before w. Same arguments and return codes as oracle_mce. */
int oracle_mce_l2(int32_t n, const int32_t *rp, const int32_t *ci, const int32_t *rnd,
                  const int32_t *roots, int32_t nroots, int64_t node_budget,
                  uint64_t *count, uint64_t *hash, uint64_t *hist, int32_t hist_cap,
                  int32_t *hist_len, int64_t *nodes) {
  search s;
  memset(&s, 0, sizeof(s));
  s.rp = rp; s.ci = ci; s.rnd = rnd;
  s.hist = hist; s.hist_cap = hist_cap; s.budget = node_budget;
  for (int32_t i = 0; i < hist_cap; i++) hist[i] = 0;
  int32_t maxdeg = 0;
  for (int32_t v = 0; v < n; v++) if (rp[v + 1] - rp[v] > maxdeg) maxdeg = rp[v + 1] - rp[v];
  s.L = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxdeg + 1));
  s.R = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxdeg + 3));
  int32_t *loc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t *Xtmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxdeg + 1));
  if (!s.L || !s.R || !loc || !Xtmp) { free(s.L); free(s.R); free(loc); free(Xtmp); return -1; }
  for (int32_t v = 0; v < n; v++) loc[v] = -1;
  int rc = 0;
  int32_t cnt = roots ? nroots : n;
  for (int32_t i = 0; i < cnt && !s.over_budget; i++) {
    int32_t r = roots ? roots[i] : i;
    if (r < 0 || r >= n) { rc = -2; break; }
    if (rp[r + 1] == rp[r]) {   /* an isolated vertex */
      s.R[0] = r;
      report(&s, 1);
      continue;
    }
    for (int64_t e = rp[r]; e < rp[r + 1] && !s.over_budget; e++) {
      int32_t w = ci[e];
      if (!later(rnd, w, r)) continue;
      /* common neighbours of r and w, split at w */
      int32_t p = 0, x = 0;
      for (int64_t f = rp[r]; f < rp[r + 1]; f++) {
        int32_t c = ci[f];
        if (c == w || !row_has(ci, rp[w], rp[w + 1], c)) continue;
        if (later(rnd, c, w)) s.L[p++] = c;
        else Xtmp[x++] = c;
      }
      for (int32_t j = 0; j < x; j++) s.L[p + j] = Xtmp[j];
      const int32_t R0[2] = {r, w};
      if (run_sub(&s, R0, 2, p, x, loc) != 0) { rc = -1; break; }
    }
    if (rc) break;
  }
  free(s.L); free(s.R); free(loc); free(Xtmp);
  *count = s.count; *hash = s.hash; *hist_len = s.hist_len;
  if (nodes) *nodes = s.nodes;
  if (rc) return rc;
  if (s.over_budget) return 1;
  if (s.hist_overflow) return 2;
  return 0;
}

/* Like oracle_mce over roots[0..nroots), but each root's first-level subtree
   gets its own budget of root_budget search-tree nodes (0: none): for root i,
   nodes[i] = nodes searched, count[i] and hash[i] = its maximal cliques and
   their hash sum, done[i] = 1 if the subtree was searched to the end (else its
   count and hash are partial and must not be used). Returns 0, -1 on
   allocation failure, -2 for a root out of range. */
int oracle_mce_each(int32_t n, const int32_t *rp, const int32_t *ci, const int32_t *rnd,
                    const int32_t *roots, int32_t nroots, int64_t root_budget,
                    int64_t *nodes, uint64_t *count, uint64_t *hash, uint8_t *done) {
  search s;
  memset(&s, 0, sizeof(s));
  s.rp = rp; s.ci = ci; s.rnd = rnd;
  int32_t maxdeg = 0;
  for (int32_t v = 0; v < n; v++) if (rp[v + 1] - rp[v] > maxdeg) maxdeg = rp[v + 1] - rp[v];
  s.hist_cap = maxdeg + 3;
  s.hist = (uint64_t *)calloc((size_t)s.hist_cap, sizeof(uint64_t));
  s.L = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxdeg + 1));
  s.R = (int32_t *)malloc(sizeof(int32_t) * (size_t)(maxdeg + 2));
  int32_t *loc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!s.hist || !s.L || !s.R || !loc) { free(s.hist); free(s.L); free(s.R); free(loc); return -1; }
  for (int32_t v = 0; v < n; v++) loc[v] = -1;
  int rc = 0;
  for (int32_t i = 0; i < nroots; i++) {
    int32_t r = roots[i];
    if (r < 0 || r >= n) { rc = -2; break; }
    s.count = 0; s.hash = 0; s.nodes = 0; s.over_budget = 0;
    s.budget = root_budget;
    if (run_root(&s, r, loc) != 0) { rc = -1; break; }
    nodes[i] = s.nodes;
    count[i] = s.count;
    hash[i] = s.hash;
    done[i] = s.over_budget ? 0 : 1;
  }
  free(s.hist); free(s.L); free(s.R); free(loc);
  return rc;
}

/* ------------------------------------------------------------------ subtree size estimate
   Knuth's random-probe estimate of a backtrack tree (D. E. Knuth, "Estimating
   the efficiency of backtrack programs", Mathematics of Computation 29, 1975),
   applied to the first-level subtree of one root (Algorithm 3 with Algorithm
   2). A walk starts at the root node and, at every node whose P is not empty,
   takes one of its branches uniformly at random: branch j (v_j, the j-th
   vertex of P - N(pivot) in ascending id, pivot by Tomita's rule as in bkt) is
   the child (P_j n N(v_j), X_j n N(v_j)), where P_j and X_j are P and X after
   the branches before it moved v_1 .. v_{j-1} from P to X. With c_t the branch
   count met at depth t, the walk estimates the node count (calls of bkt) as
   1 + c_0 + c_0 c_1 + ..., and the maximal cliques as c_0 c_1 ... c_{t-1} when
   it ends at a node with P and X empty (else 0). Both estimates are unbiased.
   A test-side tool: it sizes workloads, it is never compared with the engine. */
static uint64_t knuth_next(uint64_t *state) {   /* SplitMix64 sequence */
  *state += GOLDEN;
  return oracle_mix64(*state);
}

static void knuth_walk(search *s, uint64_t *rng, double *est_nodes, double *est_cliques, int *depth_out) {
  int wp = s->wp, wl = s->wl;
  double w = 1.0, nodes = 1.0;
  int depth = 0;
  for (;;) {
    uint64_t *P = s->arena + (size_t)depth * (2 * wp + wl);
    uint64_t *X = P + wp;
    uint64_t *cand = X + wl;
    int pe = 1, xe = 1;
    for (int i = 0; i < wp; i++) if (P[i]) { pe = 0; break; }
    for (int i = 0; i < wl; i++) if (X[i]) { xe = 0; break; }
    if (pe) {
      *est_cliques = xe ? w : 0.0;
      break;
    }
    int32_t best = -1, bestc = -1;
    for (int i = 0; i < wl; i++) {
      uint64_t bits = X[i] | (i < wp ? P[i] : 0);
      while (bits) {
        int32_t u = i * 64 + __builtin_ctzll(bits);
        bits &= bits - 1;
        const uint64_t *row = s->adjP + (size_t)u * wp;
        int c = 0;
        for (int t = 0; t < wp; t++) c += popc(P[t] & row[t]);
        if (c > bestc || (c == bestc && s->L[u] < s->L[best])) { best = u; bestc = c; }
      }
    }
    const uint64_t *prow = s->adjP + (size_t)best * wp;
    int64_t nc = 0;
    for (int i = 0; i < wp; i++) { cand[i] = P[i] & ~prow[i]; nc += popc(cand[i]); }
    if (nc == 0) {                 /* an X vertex adjacent to all of P: no branch */
      *est_cliques = 0.0;
      break;
    }
    const uint64_t pick = (uint64_t)(((unsigned __int128)knuth_next(rng) * (uint64_t)nc) >> 64);
    /* the branches before the picked one move from P to X */
    uint64_t left = pick;
    int32_t v = -1;
    for (int i = 0; i < wp && v < 0; i++) {
      uint64_t bits = cand[i];
      while (bits) {
        const int b = __builtin_ctzll(bits);
        bits &= bits - 1;
        if (left == 0) { v = i * 64 + b; break; }
        P[i] &= ~(1ULL << b);
        X[i] |= 1ULL << b;
        left--;
      }
    }
    const uint64_t *vrow = s->adjP + (size_t)v * wp;
    const uint64_t *vcol = s->colL + (size_t)v * wl;
    uint64_t *Pn = s->arena + (size_t)(depth + 1) * (2 * wp + wl);
    uint64_t *Xn = Pn + wp;
    for (int i = 0; i < wp; i++) Pn[i] = P[i] & vrow[i];
    for (int i = 0; i < wl; i++) Xn[i] = X[i] & vcol[i];
    w *= (double)nc;
    nodes += w;
    depth++;
  }
  *est_nodes = nodes;
  *depth_out = depth;
}

/* `walks` probes of root's first-level subtree (bitsets as in run_root).
   Returns, over the walks, the sums of the node and clique estimates and of
   their squares, and the deepest walk (its leaf is a clique of depth + 1
   vertices when maximal). 0 on success, -1 on allocation failure, -2 for a
   root out of range. */
int oracle_knuth(int32_t n, const int32_t *rp, const int32_t *ci, const int32_t *rnd, int32_t root,
                 int64_t walks, uint64_t seed, double *sums, int32_t *max_depth) {
  if (root < 0 || root >= n) return -2;
  search s;
  memset(&s, 0, sizeof(s));
  s.rp = rp; s.ci = ci; s.rnd = rnd;
  int32_t deg = rp[root + 1] - rp[root];
  s.L = (int32_t *)malloc(sizeof(int32_t) * (size_t)(deg + 1));
  int32_t *loc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!s.L || !loc) { free(s.L); free(loc); return -1; }
  for (int32_t v = 0; v < n; v++) loc[v] = -1;
  int32_t p = 0;
  for (int64_t e = rp[root]; e < rp[root + 1]; e++) if (later(rnd, ci[e], root)) s.L[p++] = ci[e];
  int32_t nx = p;
  for (int64_t e = rp[root]; e < rp[root + 1]; e++) if (!later(rnd, ci[e], root)) s.L[nx++] = ci[e];
  int wp = (p + 63) / 64; if (wp == 0) wp = 1;
  int wl = (deg + 63) / 64; if (wl == 0) wl = 1;
  s.p = p; s.nl = deg; s.wp = wp; s.wl = wl;
  const size_t rec = (size_t)(2 * wp + wl);
  s.adjP = (uint64_t *)calloc((size_t)(deg > 0 ? deg : 1) * wp, sizeof(uint64_t));
  s.colL = (uint64_t *)calloc((size_t)(p > 0 ? p : 1) * wl, sizeof(uint64_t));
  s.arena = (uint64_t *)calloc((size_t)(p + 2) * rec, sizeof(uint64_t));
  uint64_t *root_rec = (uint64_t *)calloc(rec, sizeof(uint64_t));
  if (!s.adjP || !s.colL || !s.arena || !root_rec) {
    free(s.adjP); free(s.colL); free(s.arena); free(root_rec); free(s.L); free(loc);
    return -1;
  }
  for (int32_t a = 0; a < deg; a++) loc[s.L[a]] = a;
  for (int32_t a = 0; a < deg; a++) {
    int32_t x = s.L[a];
    for (int64_t e = rp[x]; e < rp[x + 1]; e++) {
      int32_t b = loc[ci[e]];
      if (b >= 0 && b < p) s.adjP[(size_t)a * wp + (b >> 6)] |= 1ULL << (b & 63);
    }
  }
  for (int32_t a = 0; a < deg; a++)
    for (int32_t b = 0; b < p; b++)
      if ((s.adjP[(size_t)a * wp + (b >> 6)] >> (b & 63)) & 1)
        s.colL[(size_t)b * wl + (a >> 6)] |= 1ULL << (a & 63);
  for (int32_t b = 0; b < p; b++) root_rec[b >> 6] |= 1ULL << (b & 63);
  for (int32_t a = p; a < deg; a++) root_rec[wp + (a >> 6)] |= 1ULL << (a & 63);
  uint64_t rng = seed;
  double sn = 0, sn2 = 0, sc = 0, sc2 = 0;
  int32_t dmax = 0;
  for (int64_t t = 0; t < walks; t++) {
    memcpy(s.arena, root_rec, rec * sizeof(uint64_t));   /* the walk changes the root's P and X */
    double en, ec;
    int d;
    knuth_walk(&s, &rng, &en, &ec, &d);
    sn += en; sn2 += en * en; sc += ec; sc2 += ec * ec;
    if (d > dmax) dmax = d;
  }
  sums[0] = sn; sums[1] = sn2; sums[2] = sc; sums[3] = sc2;
  *max_depth = dmax;
  free(s.adjP); free(s.colL); free(s.arena); free(root_rec); free(s.L); free(loc);
  return 0;
}

/* Small graphs only: like oracle_mce over every root, but writes each maximal
   clique (its ids, sorted ascending) into out, cliques separated by -1.
   Returns the number of int32 written, or -1 if out_cap is too small. */
typedef struct { int32_t *out; int64_t cap, len; int overflow; } lister;
static lister *g_list;

static void list_clique(const int32_t *R, int k) {
  if (!g_list || g_list->overflow) return;
  if (g_list->len + k + 1 > g_list->cap) { g_list->overflow = 1; return; }
  int32_t *dst = g_list->out + g_list->len;
  for (int i = 0; i < k; i++) dst[i] = R[i];
  for (int i = 1; i < k; i++) {          /* insertion sort */
    int32_t x = dst[i]; int j = i - 1;
    while (j >= 0 && dst[j] > x) { dst[j + 1] = dst[j]; j--; }
    dst[j + 1] = x;
  }
  dst[k] = -1;
  g_list->len += k + 1;
}

/* plain Bron-Kerbosch with Tomita pivot over explicit sorted vertex lists (no
   bitsets), used only to list cliques of small graphs */
static void bk_list(const int32_t *rp, const int32_t *ci, int32_t *R, int k,
                    const int32_t *P, int np, const int32_t *X, int nx) {
  if (np == 0) {
    if (nx == 0) list_clique(R, k);
    return;
  }
  int32_t best = -1; int bestc = -1;
  for (int i = 0; i < np + nx; i++) {
    int32_t u = i < np ? P[i] : X[i - np];
    int c = 0;
    for (int j = 0; j < np; j++) c += adjacent(rp, ci, u, P[j]);
    if (c > bestc || (c == bestc && u < best)) { best = u; bestc = c; }
  }
  int32_t *Pc = (int32_t *)malloc(sizeof(int32_t) * (np + 1));
  int32_t *Xc = (int32_t *)malloc(sizeof(int32_t) * (np + nx + 1));
  int32_t *Pn = (int32_t *)malloc(sizeof(int32_t) * (np + 1));
  int32_t *Xn = (int32_t *)malloc(sizeof(int32_t) * (np + nx + 1));
  int32_t *br = (int32_t *)malloc(sizeof(int32_t) * (np + 1));
  int ncp = np, ncx = nx, nb = 0;
  memcpy(Pc, P, sizeof(int32_t) * np);
  memcpy(Xc, X, sizeof(int32_t) * nx);
  for (int j = 0; j < np; j++) if (!adjacent(rp, ci, best, P[j])) br[nb++] = P[j];
  for (int t = 0; t < nb; t++) {
    int32_t v = br[t];
    int a = 0, b = 0;
    for (int j = 0; j < ncp; j++) if (adjacent(rp, ci, v, Pc[j])) Pn[a++] = Pc[j];
    for (int j = 0; j < ncx; j++) if (adjacent(rp, ci, v, Xc[j])) Xn[b++] = Xc[j];
    R[k] = v;
    bk_list(rp, ci, R, k + 1, Pn, a, Xn, b);
    int w = 0;
    for (int j = 0; j < ncp; j++) if (Pc[j] != v) Pc[w++] = Pc[j];
    ncp = w;
    Xc[ncx++] = v;
  }
  free(Pc); free(Xc); free(Pn); free(Xn); free(br);
}

int64_t oracle_list(int32_t n, const int32_t *rp, const int32_t *ci, const int32_t *rnd,
                    int32_t *out, int64_t out_cap) {
  lister l = {out, out_cap, 0, 0};
  g_list = &l;
  int32_t maxdeg = 0;
  for (int32_t v = 0; v < n; v++) if (rp[v + 1] - rp[v] > maxdeg) maxdeg = rp[v + 1] - rp[v];
  int32_t *P = (int32_t *)malloc(sizeof(int32_t) * (maxdeg + 1));
  int32_t *X = (int32_t *)malloc(sizeof(int32_t) * (maxdeg + 1));
  int32_t *R = (int32_t *)malloc(sizeof(int32_t) * (maxdeg + 2));
  for (int32_t v = 0; v < n; v++) {
    int np = 0, nx = 0;
    for (int64_t e = rp[v]; e < rp[v + 1]; e++) {
      if (later(rnd, ci[e], v)) P[np++] = ci[e];
      else X[nx++] = ci[e];
    }
    R[0] = v;
    bk_list(rp, ci, R, 1, P, np, X, nx);
  }
  free(P); free(X); free(R);
  g_list = NULL;
  return l.overflow ? -1 : l.len;
}

/* ------------------------------------------------------------------------
 * One root's bit-encoded induced subgraph (section 2.4 "Induced Subgraphs",
 * section 3.4), written in the word layout the GPU engine's inspection call
 * documents, so that the engine's build can be compared with it word by word:
 *   [0] |P| | |X| << 32   [1] root | 1 << 32   [2] h(root)
 *   rows: for each member of P, then (full) of X, in id order within each,
 *         W words; bit b set iff the member is adjacent to the b-th member of P
 *   (micro) for each member of P, the bitset of its neighbours in X
 *   the hash terms h(u) of P's members, then the ids of P and of X as int32,
 *   two a word (the last word's high half is left 0 when |P| + |X| is odd).
 * P = the root's later neighbours, X = its earlier ones (Algorithm 3), each
 * in ascending id order as the CSR row holds them. Adjacency is looked up
 * pair by pair in the CSR (a binary search per pair). Returns the number of
 * words, or -1 if cap is too small or W cannot hold P. */
int64_t oracle_root_table(int32_t n, const int32_t *rp, const int32_t *ci, const int32_t *rnd, int32_t root,
                          int32_t W, int32_t micro, int32_t full, uint64_t *out, int64_t cap) {
  if (root < 0 || root >= n || W < 1) return -1;
  int32_t deg = rp[root + 1] - rp[root];
  int32_t *L = (int32_t *)malloc(sizeof(int32_t) * (size_t)(deg > 0 ? deg : 1));
  if (!L) return -1;
  int32_t p = 0, x = 0;
  for (int64_t e = rp[root]; e < rp[root + 1]; e++)
    if (later(rnd, ci[e], root)) L[p++] = ci[e];
  for (int64_t e = rp[root]; e < rp[root + 1]; e++)
    if (!later(rnd, ci[e], root)) L[p + x++] = ci[e];
  const int64_t rows = full ? (int64_t)p + x : p;
  const int64_t need = 3 + rows * W + (micro ? p : 0) + p + ((int64_t)p + x + 1) / 2;
  if (p > 64 * W || need > cap) {
    free(L);
    return -1;
  }
  memset(out, 0, sizeof(uint64_t) * (size_t)need);
  out[0] = (uint64_t)(uint32_t)p | ((uint64_t)(uint32_t)x << 32);
  out[1] = (uint64_t)(uint32_t)root | (1ULL << 32);
  out[2] = oracle_mix64((uint64_t)(int64_t)root + GOLDEN);
  int64_t w = 3;
  for (int64_t a = 0; a < rows; a++, w += W)
    for (int32_t b = 0; b < p; b++)
      if (adjacent(rp, ci, L[a], L[b])) out[w + b / 64] |= 1ULL << (b % 64);
  if (micro) {
    for (int32_t j = 0; j < p; j++, w++)
      for (int32_t a = 0; a < x; a++)
        if (adjacent(rp, ci, L[j], L[p + a])) out[w] |= 1ULL << a;
  }
  for (int32_t j = 0; j < p; j++) out[w++] = oracle_mix64((uint64_t)(int64_t)L[j] + GOLDEN);
  for (int32_t j = 0; j < p + x; j++) out[w + j / 2] |= (uint64_t)(uint32_t)L[j] << (32 * (j % 2));
  free(L);
  return need;
}
