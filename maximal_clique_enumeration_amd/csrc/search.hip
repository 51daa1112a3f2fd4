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

#define REC_WORDS(W) (3 * (W) + 2)   // per level: P[W], X_P[W], C[W], s, (lpX | open << 32)
#define MAIL_HDR 3                   // mailbox: (root list index | k << 32), lpX, s; then P, X_P, X_X

// ------------------------------------------------------------------ worker list
// 64-bit ring slot: sequence number (high half) and wave id + 1 (low half).
// Producer of ring index t waits for sequence t (the previous lap's consumer is
// done with the slot) and publishes sequence t + 1; the consumer of index h
// waits for sequence h + 1 and hands the slot to lap h + nworkers.
__device__ __forceinline__ u64 ld_acquire64(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release64(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

#define WL_SPIN_LIMIT (1u << 22)

// Receiver side (section 3.3). Gives up this wave's share of n_active; the wave
// that brings it to zero (no task held anywhere; only active waves donate, so
// none can appear) writes MCE_FLAG_EXIT into every wake flag. Any other wave
// enqueues its id and spins on its flag with exponential back-off. Returns 1
// with a task in the mailbox (the donor counted this wave active again), 0 to
// exit. The flag is cleared before the share is given up, so the exit broadcast
// (ordered after every share release) cannot be overwritten.
__device__ int wl_wait(MceWl* wl, int wid, int nworkers, u64 deadline, u32* status) {
  int res = 0, bcast = 0;
  if (lane_id() == 0) {
    u32* my = &wl->flag[(size_t)wid * MCE_LINE_WORDS];
    st_relaxed(my, 0u);
    const int left =
        __hip_atomic_fetch_add(&wl->n_active, -1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) - 1;
    if (left <= 0) {
      if (left < 0) atomicOr(status, MCE_E_PROTO);
      bcast = 1;
    } else {
      const u32 t = __hip_atomic_fetch_add(&wl->tail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      u64* slot = &wl->ring[t % (u32)nworkers];
      u32 spins = 0;
      while ((u32)(ld_acquire64(slot) >> 32) != t) {
        if (++spins > WL_SPIN_LIMIT) {
          atomicOr(status, MCE_E_PROTO);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      st_release64(slot, ((u64)(t + 1u) << 32) | (u64)(u32)(wid + 1));
      __hip_atomic_fetch_add(&wl->avail, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      int backoff = 1;
      u32 it = 0;
      for (;;) {
        const u32 f = ld_relaxed(my);
        if (f) {
          res = f == MCE_FLAG_TASK;
          break;
        }
        if ((++it & 7u) == 0 && past_deadline(deadline)) {
          atomicOr(status, MCE_E_TIMEOUT);
          st_release(&wl->done, 1u);
          break;
        }
        for (int i = 0; i < backoff; i++) __builtin_amdgcn_s_sleep(2);
        if (backoff < 32) backoff <<= 1;
      }
    }
  }
  res = read_lane(res, 0);
  if (read_lane(bcast, 0)) {
    for (int i = lane_id(); i < nworkers; i += MCE_WAVE)
      st_relaxed(&wl->flag[(size_t)i * MCE_LINE_WORDS], MCE_FLAG_EXIT);
  }
  fence_acquire_agent();
  return res;
}

// Donor side: take one idle wave out of the ring, or -1. The claimed wave is
// counted active before the donor can ever give up its own share, so n_active
// cannot reach zero while the donated branch is in flight.
__device__ int wl_claim(MceWl* wl, int nworkers, u32* status) {
  int r = -1;
  if (lane_id() == 0) {
    if (ld_relaxed(&wl->avail) > 0) {
      const int old = __hip_atomic_fetch_add(&wl->avail, -1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      if (old > 0) {
        const u32 h = __hip_atomic_fetch_add(&wl->head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        u64* slot = &wl->ring[h % (u32)nworkers];
        u64 val = 0;
        u32 spins = 0;
        while ((u32)((val = ld_acquire64(slot)) >> 32) != h + 1u) {
          if (++spins > WL_SPIN_LIMIT) {
            atomicOr(status, MCE_E_PROTO);
            st_release(&wl->done, 1u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if ((u32)(val >> 32) == h + 1u) {
          r = (int)(u32)val - 1;
          st_release64(slot, (u64)(h + (u32)nworkers) << 32);
          __hip_atomic_fetch_add(&wl->n_active, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        __hip_atomic_fetch_add(&wl->avail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  return read_lane(r, 0);
}

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

// Stable in-place partition of xx[0, L): entries adjacent to v move to the front
// in their order, the others after them (section 3.5, Figure 2). Returns the
// number kept. Each 64-entry chunk is read whole before any of it is written:
// kept entries go to [wk, wk+kc); removed entries that sat there move, with the
// chunk's removed entries, behind the kept ones.
template <class T>
__device__ int xx_partition(int* xx, int L, const T& test) {
  const int lane = lane_id();
  int wk = 0;
  for (int c = 0; c < L; c += MCE_WAVE) {
    const int i = c + lane;
    const bool valid = i < L;
    const int x = valid ? xx[i] : 0;
    const int kc_bound = min(MCE_WAVE, c - wk);
    const int dval = lane < kc_bound ? xx[wk + lane] : 0;
    const bool keep = valid && test.adj(x);
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
  return wk;
}

// Is any entry of xx[0, L) adjacent to v? (X_X n N(v) emptiness at a leaf.)
template <class T>
__device__ bool xx_any(const int* xx, int L, const T& test) {
  const int lane = lane_id();
  for (int c = 0; c < L; c += MCE_WAVE) {
    const int i = c + lane;
    const bool hit = i < L && test.adj(xx[i]);
    if (ballot(hit)) return true;
  }
  return false;
}

// ------------------------------------------------------------------ the kernel
template <int W, bool IPX, bool SROWS, bool SSTACK>
__global__ __launch_bounds__(64) void k_search(SearchParams prm) {
  constexpr int REC = REC_WORDS(W);
  extern __shared__ u64 lds[];

  const int lane = lane_id();
  const int wid = blockIdx.x;
  const int* __restrict__ rp = prm.rp;
  const int* __restrict__ ci = prm.ci;
  MceWl* wl = prm.wl;
  const u64 t_start = wall_clock64();
  const u64 deadline = t_start + prm.budget;

  char* slot = prm.slots + (size_t)wid * prm.slot_bytes;
  u64* mail = (u64*)(slot + prm.s_mail);
  u64* s_hist = lds + prm.l_hist;
  u64* hv = lds + prm.l_hv;
  int* pid = (int*)(lds + prm.l_pid);   // partial subgraph: ids of the P members
  u64* stk = SSTACK ? lds + prm.l_stack : (u64*)(slot + prm.s_stack);
  int* xx = SROWS ? (int*)(lds + prm.l_xx) : (int*)(slot + prm.s_xx);
  u64* lrows = lds + prm.l_rows;

  // a failed build leaves some tables unwritten: search nothing
  if (ld_relaxed(prm.status) & (MCE_E_HEAP | MCE_E_LIMIT)) return;
  for (int i = lane; i < prm.hcap; i += MCE_WAVE) s_hist[i] = 0;
  __syncthreads();
  // this wave is active until phase 1 finds the roots exhausted (wl_wait gives
  // the share back)
  if (lane == 0) __hip_atomic_fetch_add(&wl->n_active, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  u64 hacc = 0;
  u64 st_nodes = 0, st_leaves = 0, st_don = 0, st_prow = 0, st_xx = 0, st_roots = 0, st_recv = 0;
  u64 idle_ticks = 0;
  bool phase2 = false;
  bool abort = false;
  int wl_countdown = 0, wl_gap = 1;

  for (;;) {
    // ---------------------------------------------------------- get a task
    int tidx = 0, k0 = 1, lpx = 0;
    u64 s = 0, pj = 0, xj = 0;
    if (!phase2) {
      u32 idx = 0;
      if (lane == 0) idx = atomicAdd(&wl->root_ctr, 1u);
      idx = (u32)read_lane((int)idx, 0);
      if (idx >= (u32)prm.nroots) {
        phase2 = true;
        continue;
      }
      tidx = (int)idx;
    } else {
      if (!prm.worker_list) break;
      const u64 t0 = wall_clock64();
      const int got = wl_wait(wl, wid, prm.nworkers, deadline, prm.status);
      idle_ticks += wall_clock64() - t0;
      if (!got) break;
      const u64 h0 = mail[0];
      tidx = (int)(u32)h0;
      k0 = (int)(h0 >> 32);
      lpx = (int)(u32)mail[1];
      s = mail[2];
      if (lane < W) {
        pj = mail[MAIL_HDR + lane];
        xj = mail[MAIL_HDR + W + lane];
      }
    }

    // ---------------------------------------------------------- the root's induced subgraph
    const u64* T = prm.heap + prm.tab_off[tidx];
    const u64 hdr = T[0];
    const int p = (int)(u32)hdr;
    const int x = (int)(hdr >> 32);
    const int nrows = IPX ? p + x : p;
    const u64* grow = T + 3;
    const u64* ghv = grow + (size_t)nrows * W;
    const int* gids = (const int*)(ghv + p);
    const u64* rows;
    if constexpr (SROWS) {
      for (int i = lane; i < nrows * W; i += MCE_WAVE) lrows[i] = grow[i];
      rows = lrows;
    } else {
      rows = grow;
    }
    for (int i = lane; i < p; i += MCE_WAVE) hv[i] = ghv[i];
    if constexpr (!IPX) {
      for (int i = lane; i < p; i += MCE_WAVE) pid[i] = gids[i];
    }
    if (!phase2) {
      // a first-level subtree: R = {root}, P = P_root, X_P = {}, X_X = X_root
      s = T[2];
      lpx = x;
      if (lane < W) {
        const int cnt = p - lane * 64;
        pj = cnt <= 0 ? 0ull : (cnt >= 64 ? ~0ull : ((1ull << cnt) - 1));
      }
      for (int i = lane; i < x; i += MCE_WAVE) xx[i] = IPX ? p + i : gids[p + i];
      st_roots++;
    } else {
      const int* mx = (const int*)(mail + MAIL_HDR + 2 * W);
      for (int i = lane; i < lpx; i += MCE_WAVE) xx[i] = mx[i];
      st_recv++;
    }
    __syncthreads();
    u64 myrow = 0;   // W == 1: P row `lane` kept in a register
    if constexpr (W == 1) {
      if (lane < p) myrow = rows[lane];
    }

    // ---------------------------------------------------------- depth-first search
    // Current level in registers: P, X_P, C (lane w < W holds word w), s = sum of
    // the hash terms of R, lpX, open = shallower levels with branches left.
    u64 cj = 0;
    int open = 0;
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
              st_release(&wl->done, 1u);
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
              const u64* row = rows + (size_t)i * W;
#pragma unroll
              for (int w = 0; w < W; w++) c += (u32)__popcll(read_lane(pj, w) & row[w]);
            }
            const u32 key = (c << 20) | (u32)(MCE_MAX_LOCAL - i);
            best = best > key ? best : key;
          }
        }
        if constexpr (IPX) {
          if (lpx > 0) {
            u32 pc;
            if constexpr (W == 1) pc = (u32)__popcll(read_lane(pj, 0));
            else pc = wave_sum_u32(lane < W ? (u32)__popcll(pj) : 0u);
            st_prow += (u64)lpx;
            for (int c0 = 0; c0 < lpx; c0 += MCE_WAVE) {
              const int i = c0 + lane;
              if (i < lpx) {
                const int a = xx[i];
                const u64* row = rows + (size_t)a * W;
                u32 c = 0;
#pragma unroll
                for (int w = 0; w < W; w++) c += (u32)__popcll(read_lane(pj, w) & row[w]);
                const u32 key = (c << 20) | (u32)(MCE_MAX_LOCAL - a);
                best = best > key ? best : key;
              }
              // an X vertex adjacent to all of P: every branch is fruitless
              if (c0 + MCE_WAVE < lpx && (wave_max_u32(best) >> 20) == pc) break;
            }
          }
        }
        best = wave_max_u32(best);
        const int u = MCE_MAX_LOCAL - (int)(best & (u32)MCE_MAX_LOCAL);
        cj = 0;
        if constexpr (W == 1) {
          const u64 ru = (u < p) ? read_lane(myrow, u) : rows[u];
          if (lane == 0) cj = pj & ~ru;
        } else {
          if (lane < W) cj = pj & ~rows[(size_t)u * W + lane];
        }
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
        open = (int)(mv >> 32);
        continue;
      }
      const int j0 = __builtin_ctzll(nz);
      const u64 cw = read_lane(cj, j0);
      const int v = j0 * 64 + __builtin_ctzll(cw);
      const u64 vbit = cw & (~cw + 1);
      const bool more_here = (nz & ~(1ull << j0)) != 0 || (cw & (cw - 1)) != 0;
      u64 rv;
      if constexpr (W == 1) rv = read_lane(myrow, v);
      else rv = lane < W ? rows[(size_t)v * W + lane] : 0;
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
          if (!xx_any(xx, lpx, test)) {
            hacc += mce_clique_term(s_child, k_child);
            if (lane == 0) s_hist[k_child] += 1;
            st_leaves++;
          }
        }
        continue;
      }
      // X_X n N(v): stable partition, the child's part is xx[0, lpx_child)
      st_xx += (u64)lpx;
      const int lpx_child = lpx > 0 ? xx_partition(xx, lpx, test) : 0;

      // donate this branch to an idle wave? (section 3.3 conditions)
      if (prm.worker_list && more_here && open > 0) {
        if (wl_countdown > 0) {
          wl_countdown--;
        } else {
          u32 pc;
          if constexpr (W == 1) pc = (u32)__popcll(read_lane(pn, 0));
          else pc = wave_sum_u32(lane < W ? (u32)__popcll(pn) : 0u);
          if ((int)pc >= prm.donate_min_p) {
            const int rcv = wl_claim(wl, prm.nworkers, prm.status);
            if (rcv >= 0) {
              char* dslot = prm.slots + (size_t)rcv * prm.slot_bytes;
              u64* dm = (u64*)(dslot + prm.s_mail);
              int* dx = (int*)(dm + MAIL_HDR + 2 * W);
              if (lane < W) {
                dm[MAIL_HDR + lane] = pn;
                dm[MAIL_HDR + W + lane] = xn;
              }
              for (int i = lane; i < lpx_child; i += MCE_WAVE) dx[i] = xx[i];
              if (lane == 0) {
                dm[0] = (u64)(u32)tidx | ((u64)(u32)k_child << 32);
                dm[1] = (u64)(u32)lpx_child;
                dm[2] = s_child;
              }
              fence_release_agent();
              if (lane == 0) st_release(&wl->flag[(size_t)rcv * MCE_LINE_WORDS], MCE_FLAG_TASK);
              st_don++;
              wl_gap = 1;
              continue;
            }
            // nobody idle: look again after a growing number of branches
            wl_countdown = wl_gap;
            wl_gap = wl_gap < 64 ? 2 * wl_gap : 64;
          }
        }
      }
      // descend: save this level, the child becomes the current level
      u64* R = stk + (size_t)l * REC;
      if (lane < W) {
        R[lane] = pj;
        R[W + lane] = xj;
        R[2 * W + lane] = cj;
      }
      if (lane == 0) {
        R[3 * W] = s;
        R[3 * W + 1] = (u64)(u32)lpx | ((u64)(u32)open << 32);
      }
      open += more_here ? 1 : 0;
      l++;
      pj = pn;
      xj = xn;
      s = s_child;
      lpx = lpx_child;
      need_pivot = true;
    }
    if (abort) break;
  }

  // ---------------------------------------------------------- flush
  const u64 t_end = wall_clock64();
  if (!abort) {
    __syncthreads();
    for (int i = lane; i < prm.hcap; i += MCE_WAVE) {
      const u64 h = s_hist[i];
      if (h) atomicAdd(&prm.g_hist[i], h);
    }
    if (lane == 0 && hacc) atomicAdd(prm.g_hash, hacc);
  }
  if (lane == 0) {
    u64* st = prm.stats + (size_t)wid * MCE_NSTAT;
    st[ST_NODES] = st_nodes;
    st[ST_LEAVES] = st_leaves;
    st[ST_DONATIONS] = st_don;
    st[ST_PIVOT_ROWS] = st_prow;
    st[ST_PIVOT_WORDS] = st_prow * (u64)W;
    st[ST_XX_TESTS] = st_xx;
    st[ST_IP_ROWS] = 0;
    st[ST_BUSY_TICKS] = (t_end - t_start) - idle_ticks;
    st[ST_ROOTS] = st_roots;
    st[ST_RECEIVED] = st_recv;
    st[ST_TOTAL_TICKS] = t_end - t_start;
  }
}

// Worker-list reset before a launch: counters zero, ring slot i at sequence i,
// wake flags of the launch's waves zero.
__global__ void k_wl_init(MceWl* wl, int nworkers) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int nt = gridDim.x * blockDim.x;
  u32* head = (u32*)wl;
  const int nhead = (int)(offsetof(MceWl, ring) / 4);
  for (int i = tid; i < nhead; i += nt) head[i] = 0;
  for (int i = tid; i < nworkers; i += nt) {
    wl->ring[i] = (u64)(u32)i << 32;
    wl->flag[(size_t)i * MCE_LINE_WORDS] = 0;
  }
}

// ------------------------------------------------------------------ host side
hipError_t mce_launch_wl_init(MceWl* wl, int nworkers, hipStream_t s) {
  hipLaunchKernelGGL(k_wl_init, dim3(std::max(1, std::min(64, (nworkers + 255) / 256))), dim3(256), 0, s, wl,
                     nworkers);
  return hipGetLastError();
}

template <int W, bool IPX, bool SR, bool SS>
static const void* fn() {
  return (const void*)k_search<W, IPX, SR, SS>;
}

// Variants: widths 1, 2, 4 stage rows (light sub-classes) and stack in LDS as
// the layout allows; wider classes keep both in HBM.
template <bool IPX>
static const void* pick(int wclass, bool srows, bool sstack) {
  switch (wclass) {
    case 0:
      return srows ? (sstack ? fn<1, IPX, true, true>() : fn<1, IPX, true, false>())
                   : (sstack ? fn<1, IPX, false, true>() : fn<1, IPX, false, false>());
    case 1:
      return srows ? (sstack ? fn<2, IPX, true, true>() : fn<2, IPX, true, false>())
                   : (sstack ? fn<2, IPX, false, true>() : fn<2, IPX, false, false>());
    case 2:
      return srows ? (sstack ? fn<4, IPX, true, true>() : fn<4, IPX, true, false>())
                   : (sstack ? fn<4, IPX, false, true>() : fn<4, IPX, false, false>());
    case 3: return fn<8, IPX, false, false>();
    case 4: return fn<16, IPX, false, false>();
    case 5: return fn<32, IPX, false, false>();
  }
  return nullptr;
}

static const void* search_kernel(const SearchLayout& L) {
  if (L.wclass >= 3 && (L.srows || L.sstack)) return nullptr;
  return L.mode == MCE_MODE_IPX ? pick<true>(L.wclass, L.srows, L.sstack) : pick<false>(L.wclass, L.srows, L.sstack);
}

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// LDS words: histogram, hash terms, P ids (partial only), then the stack and the
// staged rows and X_X array when they are placed in LDS.
SearchLayout mce_search_layout(int sub, int mode, int pcap, int xcap, int rcap, bool force_hbm) {
  SearchLayout L{};
  L.sub = sub;
  L.wclass = sub >> 1;
  L.mode = mode;
  const int W = 1 << L.wclass;
  const bool light = (sub & 1) == 0;
  L.pcap = std::max(pcap, 1);
  L.xcap = std::max(xcap, 0);
  L.rcap = std::max(rcap, 1);
  L.levels = L.pcap;
  L.hcap = L.pcap + 2;
  const size_t rec = (size_t)REC_WORDS(W);
  L.srows = !force_hbm && light && L.wclass <= 2;
  const size_t stack_words = (size_t)L.levels * rec;
  L.sstack = !force_hbm && L.wclass <= 2 && stack_words * 8 <= 12288;
  size_t o = 0;
  L.l_hist = (int)o;
  o += (size_t)L.hcap;
  L.l_hv = (int)o;
  o += (size_t)L.pcap;
  L.l_pid = (int)o;
  if (mode == MCE_MODE_IP) o += ((size_t)L.pcap + 1) / 2;
  L.l_stack = (int)o;
  if (L.sstack) o += stack_words;
  L.l_rows = (int)o;
  if (L.srows) o += (size_t)L.rcap * W;
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
