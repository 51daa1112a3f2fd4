// The search: Bron-Kerbosch with pivoting over independent first-level subtrees,
// one wavefront per subtree, as one persistent launch per sub-class (bitset width
// and staging place).
//
// "Parallelizing Maximal Clique Enumeration on GPUs" (arxiv 2212.01473v2):
//  - section 2.3, Algorithm 2: branch on P - N(pivot); after a branch on v,
//    P = P - {v} and X = X u {v}; R is maximal when P and X are both empty;
//    Tomita's rule: the pivot is the vertex of P u X with most neighbours in P;
//  - section 2.4, Algorithm 3: subtree of v_i starts from ({v_i}, later
//    neighbours, earlier neighbours) under a degeneracy order;
//  - section 3.1: a block walks its subtree depth-first, its threads sharing the
//    set operations and the pivot search;
//  - section 3.3: persistent blocks take subtrees from a shared counter; then
//    idle blocks wait in a worker list (a multi-producer multi-consumer circular
//    buffer of block ids) and sleep on a flag with exponential back-off, and a
//    busy block donates a new branch when |P| of the branch is at least a
//    threshold and unexplored branches remain at this level and a shallower one;
//  - section 3.4: the induced subgraph of a subtree, bit-encoded: full (rows for
//    P u X over P) or partial (rows for P over P; P-X edges looked up in the CSR);
//  - section 3.5: X split into X_P (bitset, one copy per level) and X_X (one
//    array for all levels, partitioned in place, with an end index lpX per
//    level); with the partial subgraph the pivot comes from X_P u P only.
//
// MI355X mapping: the "block" is one 64-lane wavefront. A bitset over P of W
// 64-bit words lives in lanes 0..W-1 (registers) for the current level; the
// pivot scores one candidate row per lane (AND + popcount over W words) and
// takes a DPP max-reduction of a packed (count, index) key; child sets are
// W-lane ANDs; X_X is filtered by a ballot/mbcnt stable partition over 64
// entries at a time. The induced subgraph of every root is built once into a
// shared HBM heap before the launch, so a donation hands over a reference to it
// plus the branch's own sets (P, X_P, X_X, R's size and hash sum).
#include "mce_device.h"
#include "mce_internal.h"

#define REC_WORDS(W) (3 * (W) + 2)   // per level: P[W], X_P[W], C[W], s, lpX
// mailbox (agent-scope atomic words): table offset, (k | lpX << 32), s; then
// P[W], X_P[W], then the X_X entries as int32
#define MAIL_HDR 3

#include "worklist.h"

// ------------------------------------------------------------------ X_X membership
// Is entry a of X_X adjacent to the branch vertex v (P-local index)?
//  full subgraph: a is a local row index; bit v of row a.
//  partial subgraph: a is a vertex id; a binary search in the CSR.
template <int W, bool IPX>
struct XxTest {
  const u64* rows;
  const int* rp;
  const int* ci;
  int v;                 // P-local index of the branch vertex
  int vg, va, vb;        // its id and CSR row (partial only)
  __device__ void init(const u64* rows_, const int* rp_, const int* ci_, int v_, const int* pid, bool used) {
    rows = rows_;
    rp = rp_;
    ci = ci_;
    v = v_;
    vg = va = vb = 0;
    if constexpr (!IPX) {
      if (!used) return;
      vg = pid[v_];
      va = rp[vg];
      vb = rp[vg + 1];
    }
  }
  __device__ bool adj(int a) const {
    if constexpr (IPX) {
      return (rows[(size_t)a * W + (v >> 6)] >> (v & 63)) & 1ull;
    } else {
      const int xa = rp[a], xb = rp[a + 1];
      return (xb - xa <= vb - va) ? csr_range_has(ci, xa, xb, vg) : csr_range_has(ci, va, vb, a);
    }
  }
};

// The X_X passes below read XX_GROUP chunks of 64 entries, and issue their row
// loads, before acting on the first: with the rows in HBM, each chunk's loads
// were one dependent round trip. A chunk's writes stay below its own end, so
// reading the later chunks of the group early sees the values they would have.
#define XX_GROUP 4

// Stable in-place partition of xx[0, L): entries adjacent to v move to the front
// in their order, the others after them (section 3.5, Figure 2). Returns the
// number kept. Each 64-entry chunk is read whole before any of it is written:
// kept entries go to [wk, wk+kc); removed entries that sat there move, with the
// chunk's removed entries, behind the kept ones (all below the chunk's end).
template <class T>
__device__ int xx_partition(int* xx, int L, const T& test) {
  const int lane = lane_id();
  int wk = 0;
  for (int c0 = 0; c0 < L; c0 += XX_GROUP * MCE_WAVE) {
    int xg[XX_GROUP];
    bool kg[XX_GROUP];
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) {
      const int i = c0 + z * MCE_WAVE + lane;
      xg[z] = i < L ? xx[i] : 0;
    }
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) kg[z] = c0 + z * MCE_WAVE + lane < L && test.adj(xg[z]);
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) {
      const int c = c0 + z * MCE_WAVE;
      if (c >= L) break;
      const int x = xg[z];
      const bool valid = c + lane < L;
      const int kc_bound = min(MCE_WAVE, c - wk);
      const int dval = lane < kc_bound ? xx[wk + lane] : 0;
      const bool keep = kg[z];
      const u64 km = ballot(keep);
      const u64 vm = ballot(valid);
      const int kc = __popcll(km);
      const int D = min(kc, c - wk);
      const int base = max(c, wk + kc);
      __syncthreads();   // every lane holds its values before anything is written
      if (keep) xx[wk + mbcnt(km)] = x;
      if (lane < D) xx[base + lane] = dval;
      if (valid && !keep) xx[base + D + mbcnt(vm & ~km)] = x;
      wk += kc;
      __syncthreads();
    }
  }
  return wk;
}

// The X_X part of Tomita's pivot with the full subgraph: the key of every
// entry a of xx[0, L) (|N(a) n P| << 20, ties to the smallest local index) goes
// into `best`, and, in the same pass over 64-entry chunks, the entries with no
// neighbour in P move behind the others in a stable in-place partition
// (xx_partition's steps). Such an entry can hold no clique of this subtree back
// from being maximal: R is reported only where P is empty, and the X of every
// node below is X n N(v) for branch vertices v taken from this P, which it
// misses; and it cannot be the pivot of a node below (its key there is that of
// a neighbour count of 0 and a local index after every P member's). So the node
// and its subtree keep only the others: the return value is their number. The
// scan ends early when an X vertex adjacent to all of P turns up (pc = |P|: the
// node has no branch, and L is returned unchanged). Only the order of xx[0, L)
// changes, so every enclosing level's X_X, a prefix xx[0, L') with L' >= L,
// still holds the same set.
template <class Score>
__device__ int xx_pivot_prune(int* xx, int L, u32 pc, u32& best, const Score& score) {
  const int lane = lane_id();
  int wk = 0;
  for (int c0 = 0; c0 < L; c0 += XX_GROUP * MCE_WAVE) {
    int xg[XX_GROUP];
    u32 ng[XX_GROUP];
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) {
      const int i = c0 + z * MCE_WAVE + lane;
      xg[z] = i < L ? xx[i] : 0;
    }
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) ng[z] = c0 + z * MCE_WAVE + lane < L ? score(xg[z]) : 0u;
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) {
      const int c = c0 + z * MCE_WAVE;
      if (c >= L) break;
      const int x = xg[z];
      const bool valid = c + lane < L;
      const int kc_bound = min(MCE_WAVE, c - wk);
      const int dval = lane < kc_bound ? xx[wk + lane] : 0;
      const u32 nb = ng[z];
      if (valid) {
        const u32 key = (nb << 20) | (u32)(MCE_MAX_LOCAL - x);
        best = best > key ? best : key;
      }
      const bool keep = valid && nb != 0u;
      const u64 km = ballot(keep);
      const u64 vm = ballot(valid);
      const int kc = __popcll(km);
      const int D = min(kc, c - wk);
      const int base = max(c, wk + kc);
      __syncthreads();   // every lane holds its values before anything is written
      if (keep) xx[wk + mbcnt(km)] = x;
      if (lane < D) xx[base + lane] = dval;
      if (valid && !keep) xx[base + D + mbcnt(vm & ~km)] = x;
      wk += kc;
      __syncthreads();
      if (c + MCE_WAVE < L && (wave_max_u32(best) >> 20) == pc) return L;
    }
  }
  return wk;
}

// Is any entry of xx[0, L) adjacent to v? (X_X n N(v) emptiness at a leaf.)
template <class T>
__device__ bool xx_any(const int* xx, int L, const T& test) {
  const int lane = lane_id();
  for (int c0 = 0; c0 < L; c0 += XX_GROUP * MCE_WAVE) {
    bool hit = false;
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) {
      const int i = c0 + z * MCE_WAVE + lane;
      hit |= i < L && test.adj(xx[i]);
    }
    if (ballot(hit)) return true;
  }
  return false;
}

// Copy the entries of xx[0, L) adjacent to v to a mailbox, in order, with
// atomic stores; returns how many.
template <class T>
__device__ int xx_filter_copy(const int* xx, int L, const T& test, int* dst) {
  const int lane = lane_id();
  int n = 0;
  for (int c0 = 0; c0 < L; c0 += XX_GROUP * MCE_WAVE) {
    int ag[XX_GROUP];
    bool kg[XX_GROUP];
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) {
      const int i = c0 + z * MCE_WAVE + lane;
      ag[z] = i < L ? xx[i] : 0;
    }
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) kg[z] = c0 + z * MCE_WAVE + lane < L && test.adj(ag[z]);
#pragma unroll
    for (int z = 0; z < XX_GROUP; z++) {
      const u64 m = ballot(kg[z]);
      if (kg[z]) st_relaxed_i(&dst[n + mbcnt(m)], ag[z]);
      n += __popcll(m);
    }
  }
  return n;
}

// ------------------------------------------------------------------ the kernel
// STG: where the root's table is read from. 0: HBM; 1: the P rows staged in
// LDS (the rows every node reads: pivot candidates of P u X_P, the branch
// vertex's row), the X rows read from HBM by the X_X passes; 2: every row and
// the X_X array in LDS.
template <int W, bool IPX, int STG, bool SSTACK, bool ACT>
__global__ __launch_bounds__(64) void k_search(SearchParams prm) {
  constexpr int REC = REC_WORDS(W);
  extern __shared__ u64 lds[];

  const int lane = lane_id();
  const int wid = blockIdx.x;
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ ci = prm.ci;
  MceWl* wl = prm.wl;
  const u64 t_start = wall_clock64();
  ActClock<ACT> act;   // per-activity cycles (counting instance)
  act.start();
  const u64 deadline = ld_relaxed64(prm.t_run) + prm.budget;

  char* slot = prm.slots + (size_t)wid * prm.slot_bytes;
  u64* mail = (u64*)(slot + prm.s_mail);
  u64* s_hist = lds + prm.l_hist;
  u64* hv = lds + prm.l_hv;
  int* pid = (int*)(lds + prm.l_pid);   // partial subgraph: ids of the P members
  u64* stk = SSTACK ? lds + prm.l_stack : (u64*)(slot + prm.s_stack);
  int* xx = STG == 2 ? (int*)(lds + prm.l_xx) : (int*)(slot + prm.s_xx);
  u64* lrows = lds + prm.l_rows;

  // a failed build leaves some tables unwritten, and a run past its time limit
  // goes no further: search nothing
  if (ld_relaxed(prm.status) & MCE_E_STOP) {
    if (wid == 0 && lane == 0 && prm.taken) st_relaxed(prm.taken, min(ld_relaxed(&wl->root_ctr), (u32)prm.nroots));
    return;
  }
  const u64 hwloc = wave_hw_location();
  for (int i = lane; i < prm.hcap; i += MCE_WAVE) s_hist[i] = 0;
  __syncthreads();
  // this wave is active until phase 1 finds the roots exhausted (wl_idle gives
  // the share back)
  wl_join(wl);

  u64 hacc = 0;
  u64 st_nodes = 0, st_leaves = 0, st_don = 0, st_prow = 0, st_xx = 0, st_roots = 0, st_recv = 0, st_br = 0;
  u64 idle_ticks = 0;
  u64 t_first = 0, t_last = 0;
  bool phase2 = false;
  bool req_closed = true;   // the request word starts closed and is closed again by wl_idle
  bool abort = false;
  u32 rng = 0x9E3779B9u ^ ((u32)wid * 0x85EBCA6Bu) ^ (u32)prm.nroots;
  if (rng == 0) rng = 1;
  RootCursor rc{0u, 0u};

  for (;;) {
    // ---------------------------------------------------------- get a task
    int k0 = 1, lpx = 0;
    u64 toff = 0, s = 0, pj = 0, xj = 0;
    if (!phase2) {
      const u32 idx = take_root(wl, rc, (u32)prm.nroots, (u32)prm.nworkers, 16u);
      act.mark(ACT_WL);
      if (idx >= (u32)prm.nroots) {
        phase2 = true;
        continue;
      }
      toff = uni(prm.tab_off[idx]) - uni(prm.tab_off[0]);
    } else {
      if (!prm.worker_list) break;
      const u64 t0 = wall_clock64();
      const int got = wl_idle(wl, wid, prm.nworkers, deadline, prm.status, rng);
      act.mark(ACT_IDLE);
      req_closed = true;
      idle_ticks += wall_clock64() - t0;
      if (!got) break;
      toff = uni(ld_relaxed64(&mail[0]));
      const u64 m1 = uni(ld_relaxed64(&mail[1]));
      k0 = (int)(u32)m1;
      lpx = (int)(m1 >> 32);
      s = uni(ld_relaxed64(&mail[2]));
      if (lane < W) {
        pj = ld_relaxed64(&mail[MAIL_HDR + lane]);
        xj = ld_relaxed64(&mail[MAIL_HDR + W + lane]);
      }
    }

    // ---------------------------------------------------------- the root's induced subgraph
    const u64* T = prm.heap + toff;
    const u64 hdr = T[0];
    const int p = (int)(u32)hdr;
    const int x = (int)(hdr >> 32);
    const int nrows = IPX ? p + x : p;
    const u64* grow = T + 3;
    const u64* ghv = grow + (size_t)nrows * W;
    const int* gids = (const int*)(ghv + p);
    const u64* rows;   // every row
    const u64* prow;   // the P rows (local index < p)
    if constexpr (STG == 2) {
      for (int i = lane; i < nrows * W; i += MCE_WAVE) lrows[i] = grow[i];
      rows = prow = lrows;
    } else if constexpr (STG == 1) {
      for (int i = lane; i < p * W; i += MCE_WAVE) lrows[i] = grow[i];
      rows = grow;
      prow = lrows;
    } else {
      rows = prow = grow;
    }
    for (int i = lane; i < p; i += MCE_WAVE) hv[i] = ghv[i];
    if constexpr (!IPX) {
      for (int i = lane; i < p; i += MCE_WAVE) pid[i] = gids[i];
    }
    if (!phase2) {
      // a subtree root: R = the root's vertices (|R| and their hash terms summed in
      // the table), P = P_root, X_P = {}, X_X = X_root
      k0 = (int)(T[1] >> 32);
      s = T[2];
      lpx = x;
      if (lane < W) {
        const int cnt = p - lane * 64;
        pj = cnt <= 0 ? 0ull : (cnt >= 64 ? ~0ull : ((1ull << cnt) - 1));
      }
      for (int i = lane; i < x; i += MCE_WAVE) xx[i] = IPX ? p + i : gids[p + i];
      st_roots++;
    } else {
      const u32* mx = (const u32*)(mail + MAIL_HDR + 2 * W);
      for (int i = lane; i < lpx; i += MCE_WAVE) xx[i] = (int)ld_relaxed(&mx[i]);
      st_recv++;
    }
    __syncthreads();
    u64 myrow = 0;   // W == 1: P row `lane` kept in a register
    if constexpr (W == 1) {
      if (lane < p) myrow = rows[lane];
    }
    if (prm.worker_list && req_closed) {
      wl_open(wl, wid);
      req_closed = false;
    }
    if (t_first == 0) t_first = wall_clock64();
    u32 rq_next = 0;   // request word, read at one node and acted on at the next
    act.mark(ACT_STAGE);

    // ---------------------------------------------------------- depth-first search
    // Current level in registers: P, X_P, C (lane w < W holds word w), s = sum of
    // the hash terms of R, lpX.
    u64 cj = 0;
    int l = 0;
    bool need_pivot = true;
    for (;;) {
      if (need_pivot) {
        need_pivot = false;
        st_nodes++;
        if ((st_nodes & 1023u) == 0) {
          int stop = 0;
          if (lane == 0) {
            if (ld_relaxed(&wl->done)) {
              stop = 1;
            } else if (past_deadline(deadline)) {
              atomicOr(prm.status, MCE_E_TIMEOUT);
              st_relaxed(&wl->done, 1u);
              stop = 1;
            }
          }
          if (read_lane(stop, 0)) {
            abort = true;
            break;
          }
        }
        // Tomita pivot: most neighbours in P among P u X_P (and X_X with the full
        // subgraph); ties go to the largest key, i.e. the smallest local index.
        u32 best = 0;
        if constexpr (W >= 2 && W <= 4) {
          // every word's candidate rows are loaded before any is scored, so
          // their reads overlap (one round trip where the words took W); a lane
          // without a candidate reads row 0, which every table has
          u64 pw[W], cwv[W], rw[W][W];
#pragma unroll
          for (int w = 0; w < W; w++) {
            pw[w] = read_lane(pj, w);
            cwv[w] = read_lane(pj | xj, w);
          }
#pragma unroll
          for (int wb = 0; wb < W; wb++) {
            const bool on = (cwv[wb] >> lane) & 1ull;
            const u64* row = prow + (size_t)(on ? wb * 64 + lane : 0) * W;
#pragma unroll
            for (int w = 0; w < W; w++) rw[wb][w] = row[w];
          }
#pragma unroll
          for (int wb = 0; wb < W; wb++) {
            if (cwv[wb] == 0) continue;
            st_prow += (u64)__popcll(cwv[wb]);
            if ((cwv[wb] >> lane) & 1ull) {
              u32 c = 0;
#pragma unroll
              for (int w = 0; w < W; w++) c += (u32)__popcll(pw[w] & rw[wb][w]);
              const u32 key = (c << 20) | (u32)(MCE_MAX_LOCAL - (wb * 64 + lane));
              best = best > key ? best : key;
            }
          }
        } else {
#pragma unroll
          for (int wb = 0; wb < W; wb++) {
            const u64 cw = read_lane(pj | xj, wb);
            if (cw == 0) continue;
            st_prow += (u64)__popcll(cw);
            const int i = wb * 64 + lane;
            if ((cw >> lane) & 1ull) {
              u32 c = 0;
              if constexpr (W == 1) {
                if (lane < p) {
                  c = (u32)__popcll(read_lane(pj, 0) & myrow);
                } else {
                  c = (u32)__popcll(read_lane(pj, 0) & rows[i]);
                }
              } else {
                const u64* row = prow + (size_t)i * W;
#pragma unroll
                for (int w = 0; w < W; w++) c += (u32)__popcll(read_lane(pj, w) & row[w]);
              }
              const u32 key = (c << 20) | (u32)(MCE_MAX_LOCAL - i);
              best = best > key ? best : key;
            }
          }
        }
        if constexpr (IPX) {
          if (lpx > 0) {
            u32 pc;
            if constexpr (W == 1) pc = (u32)__popcll(read_lane(pj, 0));
            else pc = wave_sum_u32(lane < W ? (u32)__popcll(pj) : 0u);
            st_prow += (u64)lpx;
            u64 pw[W];
#pragma unroll
            for (int w = 0; w < W; w++) pw[w] = read_lane(pj, w);
            // (an X vertex adjacent to all of P makes every branch fruitless)
            lpx = xx_pivot_prune(xx, lpx, pc, best, [&](int a) {
              const u64* row = rows + (size_t)a * W;
              u32 c = 0;
#pragma unroll
              for (int w = 0; w < W; w++) c += (u32)__popcll(pw[w] & row[w]);
              return c;
            });
          }
        }
        best = wave_max_u32(best);
        const int u = MCE_MAX_LOCAL - (int)(best & (u32)MCE_MAX_LOCAL);
        cj = 0;
        if constexpr (W == 1) {
          const u64 ru = (u < p) ? read_lane(myrow, u) : rows[u];
          if (lane == 0) cj = pj & ~ru;
        } else {
          if (lane < W) cj = pj & ~(u < p ? prow : rows)[(size_t)u * W + lane];
        }
        act.mark(ACT_PIVOT);

        // Branch requests (section 3.3; the idle wave asks, see wl_idle): the
        // request word read at the previous node is acted on now. The branch
        // handed over is the first unexplored one of the shallowest level that
        // has any; the current level qualifies only with another branch left.
        if (prm.worker_list) {
          const u32 rq = rq_next;
          if (rq != 0u && rq != MCE_REQ_CLOSED) {
            const int rcv = (int)rq - 1;
            bool given = false;
            int dl = -1;
            for (int q = 0; q < l && dl < 0; q++) {
              const u64 cq = lane < W ? stk[(size_t)q * REC + 2 * W + lane] : 0ull;
              if (ballot(cq != 0)) dl = q;
            }
            if (dl < 0 && wave_sum_u32(lane < W ? (u32)__popcll(cj) : 0u) >= 2u) dl = l;
            if (dl >= 0) {
              u64* Rd = stk + (size_t)dl * REC;
              u64 dP = pj, dX = xj, dC = cj, ds = s;
              int dlpx = lpx;
              if (dl < l) {
                dP = lane < W ? Rd[lane] : 0ull;
                dX = lane < W ? Rd[W + lane] : 0ull;
                dC = lane < W ? Rd[2 * W + lane] : 0ull;
                u64 sv = 0, mv = 0;
                if (lane == 0) {   // written by lane 0, read back by lane 0
                  sv = Rd[3 * W];
                  mv = Rd[3 * W + 1];
                }
                ds = read_lane(sv, 0);
                dlpx = (int)(u32)read_lane(mv, 0);
              }
              const u64 dnz = ballot(lane < W && dC != 0);
              const int j0 = __builtin_ctzll(dnz);
              const u64 cw = read_lane(dC, j0);
              const int v = j0 * 64 + __builtin_ctzll(cw);
              const u64 vbit = cw & (~cw + 1);
              const u64 rv = lane < W ? prow[(size_t)v * W + lane] : 0ull;
              const u64 pn = dP & rv;
              const u64 xn = dX & rv;
              if ((int)wave_sum_u32(lane < W ? (u32)__popcll(pn) : 0u) >= prm.donate_min_p) {
                char* dslot = prm.slots + (size_t)rcv * prm.slot_bytes;
                u64* dm = (u64*)(dslot + prm.s_mail);
                int* dx = (int*)(dm + MAIL_HDR + 2 * W);
                int lpxc = 0;
                if (dlpx > 0) {
                  XxTest<W, IPX> dtest;
                  dtest.init(rows, rp, ci, v, pid, true);
                  lpxc = xx_filter_copy(xx, dlpx, dtest, dx);
                }
                if (lane < W) {
                  st_relaxed64(&dm[MAIL_HDR + lane], pn);
                  st_relaxed64(&dm[MAIL_HDR + W + lane], xn);
                }
                const u64 s_don = ds + hv[v];
                if (lane == 0) {
                  st_relaxed64(&dm[0], toff);
                  st_relaxed64(&dm[1], (u64)(u32)(k0 + dl + 1) | ((u64)(u32)lpxc << 32));
                  st_relaxed64(&dm[2], s_don);
                }
                wl_give(wl, wid, rcv);
                // the donor's level dl moves on past v: C -= {v}, P -= {v}, X_P += {v}
                if (lane == j0) {
                  if (dl < l) {
                    Rd[2 * W + j0] = dC & ~vbit;
                    Rd[j0] = dP & ~vbit;
                    Rd[W + j0] = dX | vbit;
                  } else {
                    cj &= ~vbit;
                    pj &= ~vbit;
                    xj |= vbit;
                  }
                }
                st_don++;
                given = true;
              }
            }
            if (!given) wl_refuse(wl, wid, rcv);
          }
          rq_next = wl_poll(wl, wid);
        }
        act.mark(ACT_WL);
      }

      // next branch of this level: the lowest vertex of C = P - N(pivot)
      const u64 nz = ballot(lane < W && cj != 0);
      if (nz == 0) {
        if (l == 0) break;
        l--;
        const u64* R = stk + (size_t)l * REC;
        if (lane < W) {
          pj = R[lane];
          xj = R[W + lane];
          cj = R[2 * W + lane];
        }
        u64 sv = 0, mv = 0;
        if (lane == 0) {   // written by lane 0, read back by lane 0
          sv = R[3 * W];
          mv = R[3 * W + 1];
        }
        s = read_lane(sv, 0);
        mv = read_lane(mv, 0);
        lpx = (int)(u32)mv;
        act.mark(ACT_STACK);
        continue;
      }
      const int j0 = __builtin_ctzll(nz);
      const u64 cw = read_lane(cj, j0);
      const int v = j0 * 64 + __builtin_ctzll(cw);
      const u64 vbit = cw & (~cw + 1);
      st_br++;
      u64 rv;
      if constexpr (W == 1) rv = read_lane(myrow, v);
      else rv = lane < W ? prow[(size_t)v * W + lane] : 0;
      const u64 pn = pj & rv;   // P n N(v)
      const u64 xn = xj & rv;   // X_P n N(v)
      if (lane == j0) {         // C -= {v}; P -= {v}; X_P += {v} (Algorithm 2)
        cj &= ~vbit;
        pj &= ~vbit;
        xj |= vbit;
      }
      const u64 s_child = s + hv[v];
      const int k_child = k0 + l + 1;
      XxTest<W, IPX> test;
      test.init(rows, rp, ci, v, pid, lpx > 0);
      if (ballot(lane < W && pn != 0) == 0) {
        // P n N(v) is empty: R u {v} is maximal iff X n N(v) is empty too
        if (ballot(lane < W && xn != 0) == 0) {
          st_xx += (u64)lpx;
          const bool maximal = !xx_any(xx, lpx, test);
          act.mark(ACT_SETOPS);
          if (maximal) {
            hacc += mce_clique_term(s_child, k_child);
            if (lane == 0) s_hist[k_child] += 1;
            st_leaves++;
            act.mark(ACT_EMIT);
          }
        }
        act.mark(ACT_SETOPS);
        continue;
      }
      // X_X n N(v): stable partition, the child's part is xx[0, lpx_child)
      st_xx += (u64)lpx;
      const int lpx_child = lpx > 0 ? xx_partition(xx, lpx, test) : 0;
      act.mark(ACT_SETOPS);

      // descend: save this level, the child becomes the current level
      u64* R = stk + (size_t)l * REC;
      if (lane < W) {
        R[lane] = pj;
        R[W + lane] = xj;
        R[2 * W + lane] = cj;
      }
      if (lane == 0) {
        R[3 * W] = s;
        R[3 * W + 1] = (u64)(u32)lpx;
      }
      l++;
      pj = pn;
      xj = xn;
      s = s_child;
      lpx = lpx_child;
      need_pivot = true;
      act.mark(ACT_STACK);
    }
    t_last = wall_clock64();
    if (abort) break;
  }

  // ---------------------------------------------------------- flush
  // (also after a stop at the time limit: the cliques found so far)
  const u64 t_end = wall_clock64();
  __syncthreads();
  for (int i = lane; i < prm.hcap; i += MCE_WAVE) {
    const u64 h = s_hist[i];
    if (h) atomicAdd(&prm.g_hist[i], h);
  }
  if (lane == 0 && hacc) atomicAdd(prm.g_hash, hacc);
  if (wid == 0 && lane == 0) record_taken(prm.taken, wl, (u32)prm.nroots);
  act.mark(ACT_EMIT);
  if (lane == 0) {
    u64* st = prm.stats + (size_t)wid * MCE_NSTAT;
    st[ST_HWID] = hwloc;
    st[ST_NODES] = st_nodes;
    st[ST_LEAVES] = st_leaves;
    st[ST_DONATIONS] = st_don;
    st[ST_PIVOT_ROWS] = st_prow;
    st[ST_PIVOT_WORDS] = st_prow * (u64)W;
    st[ST_XX_TESTS] = st_xx;
    st[ST_BRANCHES] = st_br;
    st[ST_BUSY_TICKS] = (t_end - t_start) - idle_ticks;
    st[ST_ROOTS] = st_roots;
    st[ST_RECEIVED] = st_recv;
    st[ST_TOTAL_TICKS] = t_end - t_start;
    st[ST_START_ABS] = t_start;
    st[ST_FIRST_ABS] = t_first;
    st[ST_LAST_ABS] = t_last;
    act.store(st);
  }
}

// ------------------------------------------------------------------ width 1 (|P_root| <= 64)
// The hot case: every set over P fits one 64-bit word, so the current level's
// P, X_P, C, hash sum and lpX are wave-uniform scalars (SALU work,
// scalar branches), and lane i holds row i of P, the hash term and the id of P
// member i, read by v_readlane. The level stack lives in VGPRs, level l in lane
// l (depth <= |P_root| - 2 < 64), and clique sizes below 64 are counted in
// lane k of a per-lane histogram. Few values stay live in scalar registers:
// timing and rare counters sit in LDS; CNT adds the work counters (pivot rows
// scored, X_X entries tested) for measurement runs.
template <bool IPX, bool SROWS, bool CNT>
__global__ __launch_bounds__(64) void k_search_w1(SearchParams prm) {
  extern __shared__ u64 lds[];

  const int lane = lane_id();
  const int wid = blockIdx.x;
  MceWl* wl = prm.wl;

  char* slot = prm.slots + (size_t)wid * prm.slot_bytes;
  u64* mail = (u64*)(slot + prm.s_mail);
  u64* s_hist = lds + prm.l_hist;   // clique sizes >= 64
  // [0] start tick, [1] deadline, [2] idle ticks, [3] nodes, [4] donate ticks,
  // [5] setup ticks, [6] first-task tick, [7] ticks of successful donations
  u64* s_misc = lds + prm.l_misc;
  int* xx = SROWS ? (int*)(lds + prm.l_xx) : (int*)(slot + prm.s_xx);
  u64* lrows = lds + prm.l_rows;

  if (ld_relaxed(prm.status) & MCE_E_STOP) {
    if (wid == 0 && lane == 0 && prm.taken) st_relaxed(prm.taken, min(ld_relaxed(&wl->root_ctr), (u32)prm.nroots));
    return;
  }
  const u64 hwloc = wave_hw_location();
  ActClock<CNT> act;   // per-activity cycles (counting instance)
  act.start();
  for (int i = lane; i < prm.hcap; i += MCE_WAVE) s_hist[i] = 0;
  if (lane == 0) {
    const u64 t0 = wall_clock64();
    s_misc[0] = t0;
    s_misc[1] = ld_relaxed64(prm.t_run) + prm.budget;
    s_misc[2] = 0;
    s_misc[3] = 0;
    s_misc[4] = 0;
    s_misc[5] = 0;
    s_misc[6] = 0;
    s_misc[7] = 0;
  }
  wl_join(wl);
  __syncthreads();

  u64 hist_lane = 0;   // lane k: maximal cliques of size k (k < 64)
  u64 hacc = 0;
  u32 nodes = 0;       // since the last fold into s_misc[3]
  u32 st_don = 0, st_roots = 0, st_recv = 0, st_checks = 0;
  u64 st_prow = 0, st_xx = 0, st_br = 0;   // CNT only
  u64 t_last = 0;
  bool phase2 = false;
  bool req_closed = true;   // the request word starts closed and is closed again by wl_idle
  bool abort = false;
  u32 rng = 0x9E3779B9u ^ ((u32)wid * 0x85EBCA6Bu) ^ (u32)prm.nroots;
  if (rng == 0) rng = 1;
  RootCursor rc{0u, 0u};

  for (;;) {
    // ---------------------------------------------------------- get a task
    int k0 = 1, lpx = 0;
    u64 toff = 0, s = 0, P = 0, XP = 0;
    if (!phase2) {
      const u32 idx = take_root(wl, rc, (u32)prm.nroots, (u32)prm.nworkers, 16u);
      act.mark(ACT_WL);
      if (idx >= (u32)prm.nroots) {
        phase2 = true;
        continue;
      }
      toff = uni(prm.tab_off[idx]) - uni(prm.tab_off[0]);
    } else {
      if (!prm.worker_list) break;
      const u64 t0 = wall_clock64();
      const int got = wl_idle(wl, wid, prm.nworkers, uni(s_misc[1]), prm.status, rng);
      act.mark(ACT_IDLE);
      req_closed = true;
      if (lane == 0) {
        const u64 t1 = wall_clock64();
        s_misc[2] += t1 - t0;
        s_misc[5] -= t1;   // plus the search start below
      }
      if (!got) {
        if (lane == 0) s_misc[5] += wall_clock64();
        break;
      }
      toff = uni(ld_relaxed64(&mail[0]));
      const u64 m1 = uni(ld_relaxed64(&mail[1]));
      k0 = (int)(u32)m1;
      lpx = (int)(m1 >> 32);
      s = uni(ld_relaxed64(&mail[2]));
      P = uni(ld_relaxed64(&mail[MAIL_HDR]));
      XP = uni(ld_relaxed64(&mail[MAIL_HDR + 1]));
    }

    // ---------------------------------------------------------- the root's induced subgraph
    const u64* T = prm.heap + toff;
    const u64 hdr = uni(T[0]);
    const int p = (int)(u32)hdr;
    const int x = (int)(hdr >> 32);
    const int nrows = IPX ? p + x : p;
    const u64* grow = T + 3;
    const u64* ghv = grow + nrows;
    const int* gids = (const int*)(ghv + p);
    const u64* rows;
    if constexpr (SROWS) {
      if (IPX) {
        for (int i = p + lane; i < nrows; i += MCE_WAVE) lrows[i] = grow[i];   // X rows
      }
      rows = lrows;
    } else {
      rows = grow;
    }
    const u64 myrow = lane < p ? grow[lane] : 0ull;
    const u64 myhv = lane < p ? ghv[lane] : 0ull;
    const int mypid = (!IPX && lane < p) ? gids[lane] : 0;
    if (!phase2) {
      k0 = (int)uni((u32)(T[1] >> 32));
      s = uni(T[2]);
      lpx = x;
      P = p >= 64 ? ~0ull : ((1ull << p) - 1);
      for (int i = lane; i < x; i += MCE_WAVE) xx[i] = IPX ? p + i : gids[p + i];
      st_roots++;
    } else {
      const u32* mx = (const u32*)(mail + MAIL_HDR + 2);
      for (int i = lane; i < lpx; i += MCE_WAVE) xx[i] = (int)ld_relaxed(&mx[i]);
      st_recv++;
    }
    __syncthreads();
    if (lane == 0) {
      const u64 t1 = wall_clock64();
      if (phase2) s_misc[5] += t1;
      if (s_misc[6] == 0) s_misc[6] = t1;
    }
    if (prm.worker_list && req_closed) {
      wl_open(wl, wid);
      req_closed = false;
    }
    u32 rq_next = 0;   // request word, read at one node and acted on at the next
    act.mark(ACT_STAGE);

    // ---------------------------------------------------------- depth-first search
    u64 stP = 0, stX = 0, stC = 0, stS = 0, stL = 0;   // level stack, level l in lane l
    u64 C = 0;
    int l = 0;
    bool need_pivot = true;
    for (;;) {
      if (need_pivot) {
        need_pivot = false;
        if ((++nodes & 1023u) == 0) {
          int stop = 0;
          if (lane == 0) {
            s_misc[3] += nodes;
            nodes = 0;
            if (ld_relaxed(&wl->done)) {
              stop = 1;
            } else if (past_deadline(s_misc[1])) {
              atomicOr(prm.status, MCE_E_TIMEOUT);
              st_relaxed(&wl->done, 1u);
              stop = 1;
            }
          }
          nodes = (u32)read_lane((int)nodes, 0);
          if (read_lane(stop, 0)) {
            abort = true;
            break;
          }
        }
        // Tomita pivot over P u X_P (lane i scores P member i), then X_X with the
        // full subgraph; ties to the smallest local index
        const u64 cand = P | XP;
        if constexpr (CNT) st_prow += (u64)__popcll(cand);
        u32 best = 0;
        if ((cand >> lane) & 1ull) best = ((u32)__popcll(P & myrow) << 20) | (u32)(MCE_MAX_LOCAL - lane);
        if constexpr (IPX) {
          if (lpx > 0) {
            const u32 pc = (u32)__popcll(P);
            if constexpr (CNT) st_prow += (u64)lpx;
            lpx = xx_pivot_prune(xx, lpx, pc, best, [&](int a) { return (u32)__popcll(P & rows[a]); });
          }
        }
        best = wave_max_u32(best);
        const int u = MCE_MAX_LOCAL - (int)(best & (u32)MCE_MAX_LOCAL);
        const u64 ru = u < p ? read_lane(myrow, u) : uni(rows[u]);
        C = P & ~ru;
        act.mark(ACT_PIVOT);

        // Branch requests (section 3.3; here the idle wave asks, see wl_idle):
        // the request word read at the previous node is acted on now, and read
        // again for the next one, so its latency hides behind this node. The
        // branch handed over is the first unexplored one of the shallowest
        // level that has any (the largest piece of work this wave holds); the
        // current level qualifies only with another branch left. Taking a
        // sibling out of order is sound: the receiver's X holds every sibling
        // taken before it, and the donor's later siblings see it in X.
        if (prm.worker_list) {
          const u32 rq = rq_next;
          if (rq != 0u && rq != MCE_REQ_CLOSED) {
            const int rcv = (int)rq - 1;
            const u64 td = wall_clock64();
            st_checks++;
            bool given = false;
            const u64 sm = ballot(lane < l && stC != 0);
            int dl = -1;
            if (sm) dl = __builtin_ctzll(sm);
            else if (__popcll(C) >= 2) dl = l;
            if (dl >= 0) {
              u64 dP = P, dX = XP, dC = C, ds = s;
              int dlpx = lpx;
              if (dl < l) {
                dP = read_lane(stP, dl);
                dX = read_lane(stX, dl);
                dC = read_lane(stC, dl);
                ds = read_lane(stS, dl);
                dlpx = (int)(u32)read_lane(stL, dl);
              }
              const int v = __builtin_ctzll(dC);
              const u64 vbit = 1ull << v;
              const u64 rv = read_lane(myrow, v);
              const u64 pn = dP & rv;
              const u64 xn = dX & rv;
              if (__popcll(pn) >= prm.donate_min_p) {
                char* dslot = prm.slots + (size_t)rcv * prm.slot_bytes;
                u64* dm = (u64*)(dslot + prm.s_mail);
                int* dx = (int*)(dm + MAIL_HDR + 2);
                int lpxc = 0;
                if (dlpx > 0) {
                  XxTest<1, IPX> test;
                  test.rows = rows;
                  test.rp = prm.rp;
                  test.ci = prm.ci;
                  test.v = v;
                  if constexpr (!IPX) {
                    test.vg = read_lane(mypid, v);
                    test.va = prm.rp[test.vg];
                    test.vb = prm.rp[test.vg + 1];
                  }
                  lpxc = xx_filter_copy(xx, dlpx, test, dx);
                }
                const u64 s_don = ds + read_lane(myhv, v);
                if (lane == 0) {
                  st_relaxed64(&dm[0], toff);
                  st_relaxed64(&dm[1], (u64)(u32)(k0 + dl + 1) | ((u64)(u32)lpxc << 32));
                  st_relaxed64(&dm[2], s_don);
                  st_relaxed64(&dm[MAIL_HDR], pn);
                  st_relaxed64(&dm[MAIL_HDR + 1], xn);
                }
                wl_give(wl, wid, rcv);
                // the donor's level dl moves on past v: C -= {v}, P -= {v}, X_P += {v}
                if (dl < l) {
                  if (lane == dl) {
                    stC = dC ^ vbit;
                    stP = dP ^ vbit;
                    stX = dX | vbit;
                  }
                } else {
                  C ^= vbit;
                  P ^= vbit;
                  XP |= vbit;
                }
                st_don++;
                given = true;
                if (lane == 0) s_misc[7] += wall_clock64() - td;
              }
            }
            if (!given) wl_refuse(wl, wid, rcv);
            if (lane == 0) s_misc[4] += wall_clock64() - td;
          }
          rq_next = wl_poll(wl, wid);
        }
        act.mark(ACT_WL);
      }

      // next branch of this level: the lowest vertex of C = P - N(pivot)
      if (C == 0) {
        if (l == 0) break;
        l--;
        P = read_lane(stP, l);
        XP = read_lane(stX, l);
        C = read_lane(stC, l);
        s = read_lane(stS, l);
        lpx = (int)(u32)read_lane(stL, l);
        act.mark(ACT_STACK);
        continue;
      }
      const int v = __builtin_ctzll(C);
      const u64 vbit = 1ull << v;
      if constexpr (CNT) st_br++;
      C ^= vbit;   // C -= {v}; P -= {v}; X_P += {v} (Algorithm 2)
      P ^= vbit;
      XP |= vbit;
      const u64 rv = read_lane(myrow, v);
      const u64 pn = P & rv;   // P n N(v)
      const u64 xn = XP & rv;  // X_P n N(v)
      if (pn == 0) {
        // P n N(v) is empty: R u {v} is maximal iff X n N(v) is empty too
        if (xn == 0) {
          bool maximal = true;
          if (lpx > 0) {
            if constexpr (CNT) st_xx += (u64)lpx;
            XxTest<1, IPX> test;
            test.rows = rows;
            test.rp = prm.rp;
            test.ci = prm.ci;
            test.v = v;
            if constexpr (!IPX) {
              test.vg = read_lane(mypid, v);
              test.va = prm.rp[test.vg];
              test.vb = prm.rp[test.vg + 1];
            }
            maximal = !xx_any(xx, lpx, test);
          }
          act.mark(ACT_SETOPS);
          if (maximal) {
            const int k = k0 + l + 1;
            hacc += mce_clique_term(s + read_lane(myhv, v), k);
            if (k < 64) {
              hist_lane += lane == k ? 1ull : 0ull;
            } else if (lane == 0) {
              s_hist[k] += 1;
            }
            act.mark(ACT_EMIT);
          }
        }
        act.mark(ACT_SETOPS);
        continue;
      }
      // X_X n N(v): stable partition, the child's part is xx[0, lpx_child)
      int lpx_child = 0;
      if (lpx > 0) {
        if constexpr (CNT) st_xx += (u64)lpx;
        XxTest<1, IPX> test;
        test.rows = rows;
        test.rp = prm.rp;
        test.ci = prm.ci;
        test.v = v;
        if constexpr (!IPX) {
          test.vg = read_lane(mypid, v);
          test.va = prm.rp[test.vg];
          test.vb = prm.rp[test.vg + 1];
        }
        lpx_child = xx_partition(xx, lpx, test);
      }
      act.mark(ACT_SETOPS);
      // descend: save this level in lane l, the child becomes the current level
      if (lane == l) {
        stP = P;
        stX = XP;
        stC = C;
        stS = s;
        stL = (u64)(u32)lpx;
      }
      l++;
      s += read_lane(myhv, v);
      P = pn;
      XP = xn;
      lpx = lpx_child;
      need_pivot = true;
      act.mark(ACT_STACK);
    }
    t_last = wall_clock64();
    if (abort) break;
  }

  // ---------------------------------------------------------- flush
  // (also after a stop at the time limit: the cliques found so far)
  const u64 t_end = wall_clock64();
  u64 leaves = wave_sum_u64(hist_lane);
  __syncthreads();
  if (hist_lane) atomicAdd(&prm.g_hist[lane], hist_lane);
  for (int i = 64 + lane; i < prm.hcap; i += MCE_WAVE) {
    const u64 h = s_hist[i];
    if (h) atomicAdd(&prm.g_hist[i], h);
  }
  if (lane == 0 && hacc) atomicAdd(prm.g_hash, hacc);
  if (wid == 0 && lane == 0) record_taken(prm.taken, wl, (u32)prm.nroots);
  act.mark(ACT_EMIT);
  for (int i = 64; i < prm.hcap; i++) leaves += s_hist[i];
  if (lane == 0) {
    u64* st = prm.stats + (size_t)wid * MCE_NSTAT;
    const u64 total = t_end - s_misc[0];
    st[ST_NODES] = s_misc[3] + nodes;
    st[ST_LEAVES] = leaves;
    st[ST_DONATIONS] = st_don;
    st[ST_PIVOT_ROWS] = st_prow;
    st[ST_PIVOT_WORDS] = st_prow;
    st[ST_XX_TESTS] = st_xx;
    st[ST_BRANCHES] = st_br;
    st[ST_BUSY_TICKS] = total - s_misc[2];
    st[ST_ROOTS] = st_roots;
    st[ST_RECEIVED] = st_recv;
    st[ST_TOTAL_TICKS] = total;
    st[ST_DONATE_TICKS] = s_misc[4];
    st[ST_SETUP_TICKS] = s_misc[5];
    st[ST_FIRST_TICKS] = s_misc[6] ? s_misc[6] - s_misc[0] : total;
    st[ST_START_ABS] = s_misc[0];
    st[ST_FIRST_ABS] = s_misc[6];
    st[ST_LAST_ABS] = t_last;
    st[ST_CHECKS] = st_checks;
    st[ST_DONATE_OK_TICKS] = s_misc[7];
    st[ST_HWID] = hwloc;
    act.store(st);
  }
}

// Worker-list reset before a launch: counters zero, wake flags zero, request
// words closed (a wave opens its own when it starts a task).
// Worker-list words and the launch's per-wave counter rows start at zero
// (request words closed).
__global__ void k_wl_init(MceWl* wl, int nworkers, u64* stats) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int nt = gridDim.x * blockDim.x;
  u32* head = (u32*)wl;
  const int nhead = (int)(offsetof(MceWl, line) / 4);
  for (int i = tid; i < nhead; i += nt) head[i] = 0u;
  for (int i = tid; i < nworkers; i += nt) {
    wl->line[(size_t)i * MCE_LINE_WORDS] = 0u;
    for (int k = 0; k < MCE_REQ_SLOTS; k++) wl->line[(size_t)i * MCE_LINE_WORDS + MCE_REQ_WORD + k] = MCE_REQ_CLOSED;
  }
  for (long long i = tid; i < (long long)nworkers * MCE_NSTAT; i += nt) stats[i] = 0ull;
}

// ------------------------------------------------------------------ host side
hipError_t mce_launch_wl_init(MceWl* wl, int nworkers, u64* stats, hipStream_t s) {
  hipLaunchKernelGGL(k_wl_init, dim3(std::max(1, std::min(64, (nworkers + 255) / 256))), dim3(256), 0, s, wl,
                     nworkers, stats);
  return hipGetLastError();
}

template <int W, bool IPX, int STG, bool SS>
static const void* fn(bool act) {
  return act ? (const void*)k_search<W, IPX, STG, SS, true> : (const void*)k_search<W, IPX, STG, SS, false>;
}

template <int W, bool IPX>
static const void* pick_w(int stg, bool sstack, bool act) {
  switch (stg) {
    case 0: return sstack ? fn<W, IPX, 0, true>(act) : fn<W, IPX, 0, false>(act);
    case 1: return sstack ? fn<W, IPX, 1, true>(act) : fn<W, IPX, 1, false>(act);
    case 2: return sstack ? fn<W, IPX, 2, true>(act) : fn<W, IPX, 2, false>(act);
  }
  return nullptr;
}

// Variants (width 1 has its own kernel): widths 2 and 4 stage rows (all of a
// light sub-class's, or the P rows) and the stack in LDS as the layout allows;
// wider classes keep both in HBM.
template <bool IPX>
static const void* pick(int wclass, int stg, bool sstack, bool act) {
  switch (wclass) {
    case 1: return pick_w<2, IPX>(stg, sstack, act);
    case 2: return pick_w<4, IPX>(stg, sstack, act);
    case 3: return fn<8, IPX, 0, false>(act);
    case 4: return fn<16, IPX, 0, false>(act);
    case 5: return fn<32, IPX, 0, false>(act);
  }
  return nullptr;
}

static const void* search_kernel(const SearchLayout& L) {
  if (L.wclass == 0) {
    const bool ipx = L.mode == MCE_MODE_IPX;
    if (L.counters)
      return ipx ? (L.srows ? (const void*)k_search_w1<true, true, true> : (const void*)k_search_w1<true, false, true>)
                 : (L.srows ? (const void*)k_search_w1<false, true, true>
                            : (const void*)k_search_w1<false, false, true>);
    return ipx ? (L.srows ? (const void*)k_search_w1<true, true, false> : (const void*)k_search_w1<true, false, false>)
               : (L.srows ? (const void*)k_search_w1<false, true, false> : (const void*)k_search_w1<false, false, false>);
  }
  if (L.wclass >= 3 && (L.srows || L.sprows || L.sstack)) return nullptr;
  const int stg = L.srows ? 2 : L.sprows ? 1 : 0;
  return L.mode == MCE_MODE_IPX ? pick<true>(L.wclass, stg, L.sstack, L.counters)
                                : pick<false>(L.wclass, stg, L.sstack, L.counters);
}

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// LDS words: histogram, hash terms, P ids (partial only), then the stack and the
// staged rows and X_X array when they are placed in LDS.
// Heavy sub-classes (tables over MCE_LIGHT_BYTES) stage their rows in LDS too
// when the launch has few roots (at most two per CU) and its largest table and
// X_X array fit in this many bytes: a node's row reads then cost an LDS round
// trip, not an L2 one, and a launch of few roots needs no more waves than the
// LDS leaves (R-MAT's heaviest width-4 sample: 6.3 -> 3.6 ms). A launch of
// thousands of heavy roots keeps them in HBM and its wavefronts (the 500k
// Chung-Lu graph's width-2 launch ran slower with its rows in LDS).
#define HEAVY_STAGE_BYTES (24 * 1024)
// Otherwise a width-2 or width-4 launch stages the P rows alone when they take
// at most this many bytes: the rows that every node reads (pivot candidates of
// P u X_P, the branch vertex's row) then cost an LDS round trip, while the X
// rows, read only by the X_X passes, stay in HBM.
#define PROWS_STAGE_BYTES 2048

SearchLayout mce_search_layout(int sub, int mode, int pcap, int xcap, int rcap, int nroots, int num_cu,
                               bool force_hbm, bool counters) {
  SearchLayout L{};
  L.counters = counters;
  L.sub = sub;
  L.wclass = sub >> 1;
  L.mode = mode;
  const int W = 1 << L.wclass;
  const bool light = (sub & 1) == 0;
  L.pcap = std::max(pcap, 1);
  L.xcap = std::max(xcap, 0);
  L.rcap = std::max(rcap, 1);
  L.levels = L.pcap;
  L.hcap = L.pcap + 3;   // clique sizes up to |R at the root| + |P| <= 2 + pcap
  const size_t rec = (size_t)REC_WORDS(W);
  const size_t stage = (size_t)L.rcap * W * 8 + (size_t)L.xcap * 4;
  L.srows = !force_hbm && L.wclass <= 2 &&
            (light || (nroots <= 2 * num_cu && stage <= (size_t)HEAVY_STAGE_BYTES));
  L.sprows = !force_hbm && !L.srows && L.wclass >= 1 && L.wclass <= 2 &&
             (size_t)L.pcap * W * 8 <= (size_t)PROWS_STAGE_BYTES;
  const size_t stack_words = (size_t)L.levels * rec;
  // width 1 keeps its level stack in VGPRs
  L.sstack = L.wclass > 0 && !force_hbm && L.wclass <= 2 && stack_words * 8 <= 12288;
  size_t o = 0;
  L.l_misc = (int)o;
  o += 8;   // width-1 kernel: timing and rare counters
  L.l_hist = (int)o;
  o += (size_t)L.hcap;
  L.l_hv = (int)o;
  if (L.wclass > 0) o += (size_t)L.pcap;   // width 1 keeps hash terms and ids in VGPRs
  L.l_pid = (int)o;
  if (L.wclass > 0 && mode == MCE_MODE_IP) o += ((size_t)L.pcap + 1) / 2;
  L.l_stack = (int)o;
  if (L.sstack) o += stack_words;
  L.l_rows = (int)o;
  if (L.srows) o += (size_t)L.rcap * W;
  else if (L.sprows) o += (size_t)L.pcap * W;
  L.l_xx = (int)o;
  if (L.srows) o += ((size_t)L.xcap + 1) / 2;
  L.lds_bytes = o * 8;
  size_t b = 0;
  L.s_stack = b;
  if (!L.sstack) b = a256(b + stack_words * 8);
  L.s_xx = b;
  if (!L.srows) b = a256(b + (size_t)std::max(L.xcap, 1) * 4);
  L.s_mail = b;
  b = a256(b + (size_t)(MAIL_HDR + 2 * W) * 8 + (size_t)std::max(L.xcap, 1) * 4);
  L.slot_bytes = b;
  return L;
}

int mce_search_max_workers(const SearchLayout& L, int num_cu) {
  const void* f = search_kernel(L);
  if (!f) return 0;
  if (L.lds_bytes > 64 * 1024) {
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.lds_bytes) != hipSuccess)
      return 0;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, 64, L.lds_bytes) != hipSuccess) return 0;
  long long total = (long long)per_cu * num_cu;
  if (total > MCE_MAX_WORKERS) total = MCE_MAX_WORKERS;
  return (int)total;
}

hipError_t mce_launch_search(const SearchLayout& L, const SearchParams& prm, hipStream_t s) {
  const void* f = search_kernel(L);
  if (!f) return hipErrorInvalidValue;
  SearchParams p = prm;
  void* args[] = {&p};
  // an ordinary launch: the worker list does not need every wave resident
  return hipLaunchKernel(f, dim3(prm.nworkers), dim3(64), args, (unsigned)L.lds_bytes, s);
}
